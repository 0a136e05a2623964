"""The C-ABI library: loads, exports every declared symbol, validates arguments.

CPU only: nothing here launches a kernel (plans are made with an explicit
compute-unit count, so no device is queried).
"""

import ctypes
import os
import re

import numpy as np
import pytest

import mla_latent_kv_absorbed_amd as mla
from mla_latent_kv_absorbed_amd._binding import DecodeDesc, MlaError

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    inc = os.path.join(ROOT, "include")
    for fn in os.listdir(inc):
        if fn.endswith(".h"):
            text = open(os.path.join(inc, fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(mla_\w+)\s*\(", text))
    return names


def test_library_exports_every_declared_symbol():
    lib = mla.load_library()
    names = declared_functions()
    assert {"mla_decode_plan", "mla_decode", "mla_decode_attend", "mla_decode_merge",
            "mla_lse_combine"} <= names
    for n in sorted(names):
        assert hasattr(lib, n), f"{n} declared in include/ but not exported"


def test_status_strings():
    for code, text in [(0, "ok"), (-1, "invalid argument"), (-2, "unsupported shape"),
                       (-3, "workspace or plan buffer too small"), (-4, "HIP runtime error")]:
        assert mla.status_string(code) == text


def _desc(**kw):
    base = dict(batch=2, q_len=5, num_heads=96, kv_dtype="fp8", page_size=64, num_cus=256)
    base.update(kw)
    return mla.make_desc(**base)


@pytest.mark.parametrize("bad", [dict(batch=0), dict(q_len=0), dict(q_len=9), dict(num_heads=0),
                                 dict(page_size=0), dict(dcp_size=0), dict(dcp_rank=8, dcp_size=8),
                                 dict(dcp_rank=-1), dict(kv_dtype=7), dict(kv_dtype=4),
                                 dict(kv_dtype=-1), dict(num_cus=-1),
                                 dict(force_splits=-2)])
def test_plan_rejects_invalid_descriptions(bad):
    d = _desc(**bad)
    assert mla.plan_max_bytes(d) == 0
    with pytest.raises(MlaError):
        mla.make_plan(d, [100] * max(1, d.batch))


def test_plan_accepts_every_pool_format():
    # BF16, FP8 and FP4 pools plan alike (the work is in tokens, not bytes).
    plans = [mla.make_plan(_desc(kv_dtype=kv), [3000, 40])
             for kv in ("bf16", "fp8", "fp4", "mxfp8")]
    for p, code in zip(plans, (0, 1, 2, 3)):
        assert p.header["kv_dtype"] == code
    assert len({p.header["num_units"] for p in plans}) == 1
    assert np.array_equal(plans[0].units(), plans[2].units())


def test_fp4_format_constants_match_the_header():
    text = open(os.path.join(ROOT, "include", "mla.h")).read()
    assert re.search(r"MLA_KV_FP4_E2M1\s*=\s*2", text)
    assert re.search(r"MLA_KV_MXFP8_E4M3\s*=\s*3", text)
    assert "336" in text and mla._binding.FP4_ROW_BYTES == 336
    assert "608" in text and mla._binding.MXFP8_ROW_BYTES == 608


def test_plan_rejects_unsupported_dims():
    d = DecodeDesc(1, 1, 16, 256, 64, 64, 0, 1, 0, 256, 0)
    lib = mla.load_library()
    buf = np.zeros(4096, np.uint8)
    n, ws = ctypes.c_size_t(), ctypes.c_size_t()
    lens = np.array([100], np.int32)
    st = lib.mla_decode_plan(ctypes.byref(d), lens.ctypes.data, buf.ctypes.data, buf.size,
                             ctypes.byref(n), ctypes.byref(ws))
    assert st == -2


def test_plan_rejects_short_lengths_and_small_buffers():
    d = _desc()
    with pytest.raises(MlaError, match="invalid"):
        mla.make_plan(d, [4, 100])  # seq_len < q_len
    lib = mla.load_library()
    buf = np.zeros(64, np.uint8)
    n, ws = ctypes.c_size_t(), ctypes.c_size_t()
    lens = np.array([100, 100], np.int32)
    st = lib.mla_decode_plan(ctypes.byref(d), lens.ctypes.data, buf.ctypes.data, 64,
                             ctypes.byref(n), ctypes.byref(ws))
    assert st == -3


def test_decode_and_combine_reject_bad_arguments_on_host():
    lib = mla.load_library()
    p = mla.make_plan(_desc(), [100, 200])
    # null pointers
    st = lib.mla_decode(p.host.ctypes.data, None, None, None, None, None, 1, None, 1, None,
                        ctypes.c_float(0.1), None, 0, None, None, None)
    assert st == -1
    # corrupted plan magic
    bad = p.host.copy()
    bad[:4] = 0
    fake = 1 << 20  # never dereferenced: validation fails first
    st = lib.mla_decode(bad.ctypes.data, fake, fake, fake, fake, fake, 10, fake, 1024, fake,
                        ctypes.c_float(0.1), fake, 1 << 30, fake, fake, None)
    assert st == -1
    # misaligned pointer
    st = lib.mla_decode(p.host.ctypes.data, fake + 4, fake, fake, fake, fake, 10, fake, 1024,
                        fake, ctypes.c_float(0.1), fake, 1 << 30, fake, fake, None)
    assert st == -1
    # table stride smaller than the longest local length
    st = lib.mla_decode(p.host.ctypes.data, fake, fake, fake, fake, fake, 10, fake, 100, fake,
                        ctypes.c_float(0.1), fake, 1 << 30, fake, fake, None)
    assert st == -1
    # workspace too small (a plan that splits requests needs one)
    ps = mla.make_plan(_desc(force_splits=2), [100, 200])
    assert ps.workspace_bytes > 0
    st = lib.mla_decode(ps.host.ctypes.data, fake, fake, fake, fake, fake, 10, fake, 1024, fake,
                        ctypes.c_float(0.1), fake, ps.workspace_bytes - 256, fake, fake, None)
    assert st == -3
    # pools of 2^31 slots or more are rejected (32-bit slot arithmetic)
    st = lib.mla_decode(p.host.ctypes.data, fake, fake, fake, fake, fake, 1 << 31, fake, 1024,
                        fake, ctypes.c_float(0.1), fake, 1 << 30, fake, fake, None)
    assert st == -1
    # FP8 without scales
    st = lib.mla_decode(p.host.ctypes.data, fake, fake, fake, fake, None, 10, fake, 1024, fake,
                        ctypes.c_float(0.1), fake, 1 << 30, fake, fake, None)
    assert st == -1
    # non-finite scale
    st = lib.mla_decode(p.host.ctypes.data, fake, fake, fake, fake, fake, 10, fake, 1024, fake,
                        ctypes.c_float(float("nan")), fake, 1 << 30, fake, fake, None)
    assert st == -1
    # the two halves check the same way
    st = lib.mla_decode_attend(p.host.ctypes.data, fake, fake, fake, fake, None, 10, fake, 1024,
                               fake, ctypes.c_float(0.1), fake, 1 << 30, fake, fake, None)
    assert st == -1
    st = lib.mla_decode_merge(ps.host.ctypes.data, fake, fake, ps.workspace_bytes - 256, fake,
                              fake, None)
    assert st == -3
    st = lib.mla_decode_merge(ps.host.ctypes.data, fake, None, ps.workspace_bytes, fake, fake,
                              None)
    assert st == -1
    assert lib.mla_decode_merge(p.host.ctypes.data, fake, None, 0, fake, fake, None) == 0
    assert lib.mla_decode_merge(bad.ctypes.data, fake, None, 0, fake, fake, None) == -1
    assert lib.mla_lse_combine(None, None, 0, 10, None, None, None) == -1
    assert lib.mla_lse_combine(fake, fake, 2, 0, fake, fake, None) == 0  # nothing to do
    assert lib.mla_lse_combine(fake + 4, fake, 2, 5, fake, fake, None) == -1


def test_plan_header_fields():
    p = mla.make_plan(_desc(batch=3, dcp_size=8, dcp_rank=5), [100000, 8, 6])
    h = p.header
    assert h["magic"] == 0x504C414D and h["version"] == 3
    assert h["rows"] == 480 and h["row_groups"] == 4
    assert h["max_local"] == 12500 and h["dcp_size"] == 8 and h["dcp_rank"] == 5
    assert h["plan_bytes"] == len(p.host) and h["page_size"] == 64
    # Workspace of the split partials: O in fp16 [parts, M, 512], then the
    # LSE and the row factors in fp32 [parts, M], each 256-byte aligned.
    parts, M = h["num_parts"], h["rows"]
    assert parts > 0

    def up(x):
        return -(-x // 256) * 256
    assert h["ws_lse_offset"] == up(parts * M * 512 * 2)
    assert h["ws_sc_offset"] == up(h["ws_lse_offset"] + parts * M * 4)
    assert h["workspace_bytes"] == up(h["ws_sc_offset"] + parts * M * 4) == p.workspace_bytes


def test_prepare_rejects_bad_arguments_on_host():
    lib = mla.load_library()
    f = 1 << 20  # never dereferenced: validation fails first (or T = 0 enqueues nothing)
    g = f + 4096

    def call(T=4, H=2, kv=1, ptrs=None, max_pos=8, nslots=16, scale=f):
        p = ptrs or [f] * 5
        return lib.mla_prepare(T, H, kv, p[0], p[1], p[2], p[3], p[4], f, f, max_pos, f, f, g,
                               f, scale, nslots, None)
    assert call(T=0) == 0
    assert call(T=0, kv=0, scale=None) == 0
    assert call(T=-1) == -1
    assert call(H=0) == -1
    assert call(kv=4) == -1                          # not a pool format (3 is MXFP8)
    assert call(kv=-1) == -1
    assert call(max_pos=0) == -1
    assert call(nslots=0) == -1
    assert call(ptrs=[None, f, f, f, f]) == -1
    assert call(ptrs=[f, f, f + 8, f, f]) == -1     # misaligned w_kc_t
    assert call(scale=None) == -1                    # FP8 pool without scales
    assert call(scale=f + 2) == -1                   # misaligned scales
    # q_rope_out aliasing q_rope_in
    assert lib.mla_prepare(4, 2, 0, f, g, f, f, f, f, f, 8, f, f, g, f, None, 16, None) == -1


def test_combine_project_rejects_bad_arguments_on_host():
    lib = mla.load_library()
    f = 1 << 20
    assert lib.mla_lse_combine_project(f, f, 2, 0, 4, f, f, f, None) == 0     # T = 0
    assert lib.mla_lse_combine_project(f, f, 0, 4, 4, f, f, f, None) == -1    # no parts
    assert lib.mla_lse_combine_project(f, f, 2, -1, 4, f, f, f, None) == -1
    assert lib.mla_lse_combine_project(f, f, 2, 4, 0, f, f, f, None) == -1
    assert lib.mla_lse_combine_project(None, f, 2, 4, 4, f, f, f, None) == -1
    assert lib.mla_lse_combine_project(f, f, 2, 4, 4, f + 8, f, f, None) == -1
    assert lib.mla_lse_combine_project(f, f, 2, 4, 4, f, f, f + 2, None) == -1
