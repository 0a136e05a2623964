"""CPU check of the generated FP4 / MXFP8 dequantization programs.

gen_tile_asm.dq_program and dq_program_mx emit the instructions that, spread
over a tile statement's MFMAs, turn one raw tile into the BF16 tile layout.
This test interprets those instructions for every wave and lane (address
arithmetic, LDS reads and writes, and which code byte and scale byte each
conversion takes) and checks that:

* every byte of the BF16 tile's chunks is written exactly once per tile;
* each written BF16 pair comes from the right code byte(s) of the same token
  under the scale byte of the right block;
* every raw read stays inside the raw tile.

Layouts (16-byte chunk c of token t): raw at 512 c + 16 t; BF16 at 512 c +
16 (t ^ 4 (c & 3)).  FP4 rows: code byte i holds elements 2 i, 2 i + 1;
block b's scale is row byte 288 + b.  MXFP8 rows: code byte i is element i;
block b's scale is row byte 576 + b.
"""

import importlib.util
import os
import re

import pytest

CSRC = os.path.join(os.path.dirname(__file__), "..", "mla_latent_kv_absorbed_amd", "csrc")


def _gen():
    spec = importlib.util.spec_from_file_location("gen_tile_asm",
                                                  os.path.join(CSRC, "gen_tile_asm.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


RAW, BF = 1 << 20, 1 << 22          # distinct symbolic bases of the two tiles


def _scalars(fmt, w):
    if fmt == "fp4":
        return {"dqa": RAW + 1024 * w, "dqb": RAW + 4 * w, "dqc": BF + 4096 * w,
                "dqd": RAW + (w >> 1), "dqe": 64 * w, "dqf": BF + 512 * w}
    return {"dqa": RAW + 1024 * w, "dqb": RAW + w, "dqc": BF + 2048 * w, "dqd": RAW + 512 * w,
            "dqe": RAW + (w >> 1), "dqf": BF + 1024 * w, "dqg": 128 * (w & 1)}


def _run(prog, lane, sc):
    """Interpret a program for one lane: returns (raw reads, writes)."""
    reg = {}
    reads, writes = [], []

    def val(op):
        op = op.strip()
        m = re.fullmatch(r"%\[(\w+)\]", op)
        if m:
            return sc[m.group(1)]
        if op.startswith("v"):
            return reg[int(op[1:])]
        return int(op, 0)

    for kind, text, *_ in prog:
        if kind == "wait":
            continue
        m = re.match(r"(\S+)\s+(.*)", text)
        ins, args = m.group(1), m.group(2)
        sel = re.search(r"op_sel:\[(\d),(\d),0\]", args)
        args = re.sub(r"\s*op_sel:\[.*\]", "", args)
        off = re.search(r"offset:(\d+)", args)
        off = int(off.group(1)) if off else 0
        args = re.sub(r"\s*offset:\d+", "", args)
        a = [x.strip() for x in args.split(",")]
        rng = re.fullmatch(r"v\[(\d+):(\d+)\]", a[0])
        d = int(a[0][1:]) if a[0].startswith("v") and not rng else None
        if ins == "v_mbcnt_lo_u32_b32":
            reg[d] = min(lane, 32)
        elif ins == "v_mbcnt_hi_u32_b32":
            reg[d] = max(lane - 32, 0) + val(a[2])
        elif ins == "v_and_b32":
            reg[d] = val(a[1]) & val(a[2])
        elif ins == "v_xor_b32":
            reg[d] = val(a[1]) ^ val(a[2])
        elif ins == "v_lshlrev_b32":
            x = reg[int(a[2][1:])]
            reg[d] = ("scale", x[1]) if isinstance(x, tuple) else x << val(a[1])
        elif ins == "v_lshrrev_b32":
            reg[d] = val(a[2]) >> val(a[1])
        elif ins == "v_lshl_add_u32":
            reg[d] = (val(a[1]) << val(a[2])) + val(a[3])
        elif ins == "v_add_u32":
            reg[d] = val(a[1]) + val(a[2])
        elif ins == "v_add3_u32":
            reg[d] = val(a[1]) + val(a[2]) + val(a[3])
        elif ins.startswith("ds_read"):
            addr = val(a[1]) + off
            n = {"ds_read_b64": 8, "ds_read_b32": 4, "ds_read_u8": 1}[ins]
            reads.append((addr, n))
            if rng:
                for i in range(int(rng.group(1)), int(rng.group(2)) + 1):
                    reg[i] = ("code", addr + 4 * (i - int(rng.group(1))))
            else:
                reg[d] = ("scale", addr) if n == 1 else ("code", addr)
        elif ins.startswith("v_cvt_scalef32_pk_bf16_fp"):
            src, scl = reg[int(a[1][1:])], reg[int(a[2][1:])]
            b = (int(sel.group(1)) + 2 * int(sel.group(2))) if sel else 0
            reg[d] = ("cvt", src[1], b, scl[1])
        elif ins == "ds_write_b64":
            r = re.fullmatch(r"v\[(\d+):(\d+)\]", a[1])
            writes.append((val(a[0]) + off, [reg[int(r.group(1))], reg[int(r.group(2))]]))
        else:
            raise AssertionError(f"unexpected instruction {text}")
    return reads, writes


@pytest.mark.parametrize("fmt", ["fp4", "mxfp8"])
def test_dq_program_covers_the_tile_from_the_right_codes(fmt):
    g = _gen()
    make = g.dq_program if fmt == "fp4" else g.dq_program_mx
    raw_tile = 22 * 512 if fmt == "fp4" else 38 * 512
    for p in (make(203), make(202)):        # both register-base parities
        written = {}
        for w in range(4):
            for lane in range(64):
                reads, writes = _run(p, lane, _scalars(fmt, w))
                for addr, n in reads:
                    assert RAW <= addr and addr + n <= RAW + raw_tile, (w, lane, addr - RAW)
                for addr, parts in writes:
                    a = addr - BF
                    cc, rem = divmod(a, 512)
                    tsw, half = divmod(rem, 16)
                    t = tsw ^ (4 * (cc & 3))
                    assert half in (0, 8) and 0 <= cc < 72
                    for k, (tag, src, b, scl) in enumerate(parts):
                        assert tag == "cvt"
                        s_rel = src - RAW
                        sc_chunk, s_rem = divmod(s_rel, 512)
                        s_t, s_byte = divmod(s_rem, 16)
                        assert s_t == t, (fmt, w, lane, cc)
                        elem = 8 * cc + half // 2 + 2 * k          # first of the BF16 pair
                        if fmt == "fp4":
                            code_byte = 16 * sc_chunk + s_byte + b   # element pair 2 byte, + 1
                            assert code_byte == elem // 2 and elem % 2 == 0
                            block = elem // 16
                            scale_byte = 288 + block
                        else:
                            code_byte = 16 * sc_chunk + s_byte + 2 * b
                            assert code_byte == elem
                            block = elem // 32
                            scale_byte = 576 + block
                        q_rel = scl - RAW
                        q_chunk, q_rem = divmod(q_rel, 512)
                        q_t, q_byte = divmod(q_rem, 16)
                        assert q_t == t and 16 * q_chunk + q_byte == scale_byte, (fmt, cc, k)
                    key = (cc, t, half)
                    written[key] = written.get(key, 0) + 1
        want = {(cc, t, h) for cc in range(72) for t in range(32) for h in (0, 8)}
        assert set(written) == want
        assert all(v == 1 for v in written.values())
