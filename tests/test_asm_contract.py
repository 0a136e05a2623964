"""Static checks of the inline-asm statements in the decode kernels.

The compiler sees each statement as one instruction with the operands and
clobbers it declares, so a statement must (a) declare every register it names
literally, (b) declare as an output every operand it writes, (c) leave no LDS
read in flight when it ends (a late return would overwrite a register the
compiler has since reused), (d) declare SCC / VCC when it writes them and
(e) give M0 back the value it found.  These checks read the generated
statements and the call sites in the kernel source; no GPU is needed.
"""

import os
import re

import pytest

CSRC = os.path.join(os.path.dirname(__file__), "..", "mla_latent_kv_absorbed_amd", "csrc")


def _defines():
    text = open(os.path.join(CSRC, "tile_asm.inc")).read()
    defs, cur = {}, None
    for line in text.splitlines():
        m = re.match(r"#define (\w+)", line)
        if m:
            cur = m.group(1)
            defs[cur] = line[m.end():] + "\n"
        elif cur:
            defs[cur] += line + "\n"
    return defs


DEFS = _defines()
STATEMENTS = sorted(n for n in DEFS if n.endswith("_ASM"))


def _instrs(name):
    return [x.strip() for x in re.findall(r'"([^"]*)\\n\\t"', DEFS[name])]


def _clobbers(name):
    return DEFS.get(name[: -len("_ASM")] + "_CLOBBERS", "")


def _call_sites(name):
    src = open(os.path.join(CSRC, "mla_kernels.hip")).read()
    sites = []
    for m in re.finditer(r"asm volatile\(" + name + r"\b", src):
        depth, i = 1, m.end()
        while depth:
            depth += {"(": 1, ")": -1}.get(src[i], 0)
            i += 1
        sites.append(src[m.end():i - 1])
    return src, sites


def _expand(src, text):
    # Expand the operand-list macros used at call sites.
    for mac in re.findall(r"\bMLA_\w+_OPERANDS\w*", text):
        m = re.search(r"#define " + mac + r"\b(.*?)(?<!\\)\n", src, re.S)
        if m:
            text = text.replace(mac, m.group(1).replace("\\\n", " "))
    return text


def _split_top(text):
    # Split an asm argument list at the colons that separate its sections
    # (not those inside quotes or brackets, as in "+{a[0:15]}").
    parts, depth, quote, cur = [], 0, False, ""
    for ch in text:
        if ch == '"':
            quote = not quote
        elif not quote and ch in "([{":
            depth += 1
        elif not quote and ch in ")]}":
            depth -= 1
        if ch == ":" and not quote and depth == 0:
            parts.append(cur)
            cur = ""
        else:
            cur += ch
    parts.append(cur)
    return parts


def _literal_vgprs(text):
    regs = set()
    for m in re.finditer(r"(?<![%\w])v\[(\d+):(\d+)\]", text):
        regs.update(range(int(m.group(1)), int(m.group(2)) + 1))
    for m in re.finditer(r"(?<![%\w\[])v(\d+)(?![\d:])", text):
        regs.add(int(m.group(1)))
    return regs


NO_DST = ("ds_write", "global_load_lds", "s_cmp", "s_cbranch", "s_waitcnt", "s_nop",
          "v_cmp", "s_barrier")


def _written_operands(name):
    out = set()
    for ins in _instrs(name):
        if not ins or ins.endswith(":") or ins.startswith(NO_DST):
            continue
        parts = ins.split(None, 1)
        if len(parts) == 2:
            m = re.match(r"%\[(\w+)\]", parts[1].split(",")[0].strip())
            if m:
                out.add(m.group(1))
    return out


def test_statements_found():
    assert "MLA_STEP_FP8_ASM" in STATEMENTS and "MLA_FUSED_BF16_ASM" in STATEMENTS


def _literal_sgprs(text):
    regs = set()
    for m in re.finditer(r"(?<![%\w])s\[(\d+):(\d+)\]", text):
        regs.update(range(int(m.group(1)), int(m.group(2)) + 1))
    for m in re.finditer(r"(?<![%\w\[])s(\d+)(?![\d:])", text):
        regs.add(int(m.group(1)))
    return regs


@pytest.mark.parametrize("name", STATEMENTS)
def test_literal_registers_are_clobbered(name):
    text = " ".join(_instrs(name))
    declared = set(int(x) for x in re.findall(r'"v(\d+)"', _clobbers(name)))
    assert _literal_vgprs(text) <= declared
    declared_s = set(int(x) for x in re.findall(r'"s(\d+)"', _clobbers(name)))
    assert _literal_sgprs(text) <= declared_s, "a literal SGPR that is not declared clobbered"


@pytest.mark.parametrize("name", STATEMENTS)
def test_lds_reads_drained(name):
    pending = []  # LDS operations complete in issue order
    for ins in _instrs(name):
        op = ins.split(None, 1)[0] if ins else ""
        if op.startswith(("ds_read", "ds_bpermute")):
            pending.append(True)
        elif op.startswith("ds_write"):
            pending.append(False)
        elif op == "s_waitcnt":
            m = re.search(r"lgkmcnt\((\d+)\)", ins)
            if m:
                pending = pending[len(pending) - int(m.group(1)):] if int(m.group(1)) < len(pending) else pending
    assert not any(pending), "an LDS read is still in flight when the statement ends"


@pytest.mark.parametrize("name", STATEMENTS)
def test_m0_restored(name):
    ins = _instrs(name)
    touch = [k for k, i in enumerate(ins) if re.search(r"\bm0\b", i)]
    writes = [k for k in touch if re.match(r"s_\w+ m0\b", ins[k])]
    if not writes:
        assert not any(i.startswith("global_load_lds") for i in ins)
        return
    # Saved before M0 is first touched (in %[m0s], or in a literal SGPR the
    # statement declares clobbered), restored from it by the last write, and
    # no DMA (which reads M0) after the restore.
    m = re.fullmatch(r"s_mov_b32 (%\[m0s\]|s\d+), m0", ins[touch[0]])
    assert m, ins[touch[0]]
    save = m.group(1)
    if save.startswith("s"):
        assert f'"{save}"' in _clobbers(name)
    assert ins[writes[-1]] == f"s_mov_b32 m0, {save}"
    assert not any(i.startswith("global_load_lds") for i in ins[writes[-1]:])


@pytest.mark.parametrize("name", STATEMENTS)
def test_call_sites_declare_outputs_and_flags(name):
    src, sites = _call_sites(name)
    if name == "MLA_QK_BF16_ASM" or name == "MLA_QK_FP8_ASM":
        assert sites
    ins = _instrs(name)
    writes_scc = any(re.match(r"s_(add|sub|cmp|and|or|xor|lshl|lshr)", i) for i in ins)
    writes_vcc = any(re.match(r"v_cmp\w* vcc", i) for i in ins)
    for site in sites:
        site = _expand(src, site)
        sections = _split_top(site)
        outputs = sections[1]
        clob = sections[3] if len(sections) > 3 else ""
        declared_out = set(re.findall(r"\[(\w+)\]\s*\"[=+]", outputs))
        missing = _written_operands(name) - declared_out
        assert not missing, f"operands written but not declared as outputs: {sorted(missing)}"
        if _clobbers(name):
            assert name[: -len("_ASM")] + "_CLOBBERS" in clob
        # SCC / VCC declared at the call site or in the statement's clobber macro.
        flags = clob + _clobbers(name)
        if writes_scc:
            assert '"scc"' in flags
        if writes_vcc:
            assert '"vcc"' in flags
        # Outputs written before the last input is read must be early-clobber
        # (or tied read-write) so that no input shares their register.
        for op, cons in re.findall(r"\[(\w+)\]\s*\"([=+][^\"]*)\"", outputs):
            assert cons.startswith("+") or "&" in cons, f"{op} is not early-clobber"


# ---------------------------------------------------------------- compiled loops

def _compiled_asm(tmp_path_factory):
    import shutil
    import subprocess
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "k.s"
    inc = os.path.join(os.path.dirname(__file__), "..", "include")
    subprocess.run([hipcc, "--offload-arch=gfx950", "-O3", "-std=c++17", "-I", inc,
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    "--cuda-device-only", "-S", os.path.join(CSRC, "mla_kernels.hip"),
                    "-o", str(out)], check=True, capture_output=True)
    return out.read_text()


@pytest.fixture(scope="module")
def compiled(tmp_path_factory):
    return _compiled_asm(tmp_path_factory)


LABEL = re.compile(r"^(\.LBB\w+|; %bb\.\d+):")


def _blocks_with_depth(body):
    # Split a function's assembly into basic blocks, each with the loop depth
    # the compiler annotates on its label line and the comment lines right
    # after it (0 outside loops).
    blocks = []
    for line in body:
        if LABEL.match(line):
            blocks.append({"depth": 0, "lines": [], "head": True})
        if not blocks:
            continue
        blk = blocks[-1]
        if blk["head"] and (LABEL.match(line) or line.strip().startswith(";")):
            blk["depth"] = max([blk["depth"]] + [int(x) for x in re.findall(r"Depth=(\d+)", line)])
        else:
            blk["head"] = False
        blk["lines"].append(line)
    return blocks


# decode_kernel<kKv, kPaged>: kKv 0 BF16, 1 FP8, 2 FP4, 3 MXFP8.
@pytest.mark.parametrize("variant", ["ILi1ELb1E", "ILi1ELb0E", "ILi0ELb1E", "ILi0ELb0E",
                                     "ILi2ELb1E", "ILi2ELb0E", "ILi3ELb1E", "ILi3ELb0E"])
def test_tile_loops_do_not_spill(compiled, variant):
    # A scratch reload inside a tile loop is a VMEM load: waiting for it also
    # waits for every global->LDS DMA issued before it, which serialises the
    # prefetch pipeline.  Every block of the tile loops (loop depth 2 and
    # deeper: inside the loop over work units) must be free of scratch
    # accesses.
    sym = f"_ZN3mla13decode_kernel{variant}EEvNS_10DecodeArgsE:"
    start = compiled.index(sym)
    body = compiled[start:compiled.index(".Lfunc_end", start)].splitlines()
    blocks = _blocks_with_depth(body)
    deep = [b["lines"] for b in blocks if b["depth"] >= 2]
    assert deep, "no tile loop found"
    for lines in deep:
        assert not any("scratch_" in l for l in lines), f"spill in loop block {lines[0].split()[0]}"


def test_block_depths_parsed():
    body = [".LBB0_1:  ; %bb.0", "\tv_mov_b32 v0, 0", ".LBB0_2:  ; Parent Loop BB0_1 Depth=1",
            "  ; =>  This Inner Loop Header: Depth=2", "\tscratch_load_dword v1, off, s0",
            "; %bb.3:  ; in Loop: Header=BB0_2 Depth=2", "\ts_nop 0", ".LBB0_4:",
            "\ts_endpgm"]
    got = [(b["lines"][0].split(":")[0], b["depth"]) for b in _blocks_with_depth(body)]
    assert got == [(".LBB0_1", 0), (".LBB0_2", 2), ("; %bb.3", 2), (".LBB0_4", 0)]


# ------------------------------------------------------------ launch shapes

def _hip_sources():
    return {f: open(os.path.join(CSRC, f)).read()
            for f in sorted(os.listdir(CSRC)) if f.endswith(".hip")}


def test_every_kernel_is_launched_within_its_launch_bounds():
    """Every __global__ kernel declares __launch_bounds__, and every launch
    of it uses a block no larger than that bound: the register budget the
    compiler gives a kernel (the decode kernel: 512 registers, one wave per
    SIMD) only holds for the block size it was told."""
    bounds = {}
    for f, text in _hip_sources().items():
        for m in re.finditer(r"__global__\s+(__launch_bounds__\((\d+)(?:,\s*\d+)?\)\s+)?void\s+(\w+)",
                             text):
            assert m.group(1), f"{f}: kernel {m.group(3)} has no __launch_bounds__"
            bounds[m.group(3)] = int(m.group(2))
    assert {"decode_kernel", "merge_split_kernel", "merge_split_wave_kernel",
            "lse_combine_kernel", "prepare_kernel", "combine_project_kernel"} <= set(bounds)
    launches = 0
    for f, text in _hip_sources().items():
        for m in re.finditer(r"hipLaunchKernelGGL\(\s*(\w+)\s*,[^,]*,\s*dim3\((\d+)\)", text):
            kernel, block = m.group(1), int(m.group(2))
            # decode_kernel is launched through a pointer to one of its
            # instantiations (`kernel`).
            name = "decode_kernel" if kernel == "kernel" else kernel
            assert name in bounds, f"{f}: launch of unknown kernel {kernel}"
            assert block <= bounds[name], f"{f}: {kernel} launched with {block} > {bounds[name]}"
            launches += 1
    assert launches >= 7
    # ... and `go`, the lambda that launches `kernel`, is only ever handed
    # instantiations of decode_kernel.
    text = _hip_sources()["mla_kernels.hip"]
    handed = re.findall(r"\bgo\((\w+)<", text)
    assert handed and set(handed) == {"decode_kernel"}, handed
