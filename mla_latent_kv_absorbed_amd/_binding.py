"""ctypes binding of libmla (the C ABI declared in include/mla.h).

Argument marshalling only: every step of the decode runs in the HIP kernels
of libmla.  PyTorch provides device memory and the current HIP stream.  There
is no fallback: if the library is not built, every call raises.
"""

from __future__ import annotations

import ctypes
import os
import struct
from dataclasses import dataclass

import numpy as np

KV_BF16 = 0
KV_FP8 = 1
KV_FP4 = 2
KV_MXFP8 = 3
_KV_CODES = {"bf16": KV_BF16, "fp8": KV_FP8, "fp4": KV_FP4, "mxfp8": KV_MXFP8}
FP4_ROW_BYTES = 336
MXFP8_ROW_BYTES = 608
_BLOCK_ROW_BYTES = {KV_FP4: FP4_ROW_BYTES, KV_MXFP8: MXFP8_ROW_BYTES}

MLA_OK = 0
_STATUS = {0: "ok", -1: "invalid argument", -2: "unsupported shape",
           -3: "workspace or plan buffer too small", -4: "HIP runtime error"}


class MlaError(RuntimeError):
    def __init__(self, what: str, status: int | None = None):
        super().__init__(what if status is None else f"{what}: {_STATUS.get(status, status)}")
        self.status = status


class DecodeDesc(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int32) for name in (
        "batch", "q_len", "num_heads", "kv_lora_rank", "rope_dim", "page_size", "kv_dtype",
        "dcp_size", "dcp_rank", "num_cus", "force_splits")]


_LIB = None


def library_path() -> str:
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmla.so")


def load_library():
    """Load libmla.so from the package directory (raises if it is not built)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise MlaError(f"{path} is not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    vp, sz, i32, i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64
    lib.mla_plan_max_bytes.argtypes = [ctypes.POINTER(DecodeDesc)]
    lib.mla_plan_max_bytes.restype = sz
    lib.mla_decode_plan.argtypes = [ctypes.POINTER(DecodeDesc), vp, vp, sz,
                                    ctypes.POINTER(sz), ctypes.POINTER(sz)]
    lib.mla_decode_plan.restype = i32
    lib.mla_check_table.argtypes = [ctypes.POINTER(DecodeDesc), vp, vp, i64, i64,
                                    ctypes.POINTER(i64), ctypes.POINTER(i64)]
    lib.mla_check_table.restype = i32
    lib.mla_decode.argtypes = [vp, vp, vp, vp, vp, vp, i64, vp, i64, vp, ctypes.c_float,
                               vp, sz, vp, vp, vp]
    lib.mla_decode.restype = i32
    lib.mla_decode_attend.argtypes = lib.mla_decode.argtypes
    lib.mla_decode_attend.restype = i32
    lib.mla_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i64, vp, i64, vp,
                                       ctypes.c_float, vp, vp, vp]
    lib.mla_decode_noalloc.restype = i32
    lib.mla_decode_merge.argtypes = [vp, vp, vp, sz, vp, vp, vp]
    lib.mla_decode_merge.restype = i32
    lib.mla_lse_combine.argtypes = [vp, vp, i32, i64, vp, vp, vp]
    lib.mla_lse_combine.restype = i32
    lib.mla_prepare.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp,
                                vp, i64, vp]
    lib.mla_prepare.restype = i32
    lib.mla_lse_combine_project.argtypes = [vp, vp, i32, i32, i32, vp, vp, vp, vp]
    lib.mla_lse_combine_project.restype = i32
    lib.mla_status_string.argtypes = [i32]
    lib.mla_status_string.restype = ctypes.c_char_p
    _LIB = lib
    return lib


def status_string(status: int) -> str:
    return load_library().mla_status_string(status).decode()


# Plan header fields, in the order of mla::PlanHeader (csrc/plan_layout.h).
_HEADER = struct.Struct("<2I18i4q")
_HEADER_NAMES = ("magic", "version", "batch", "q_len", "num_heads", "rows", "row_groups",
                 "num_wgs", "num_units", "num_parts", "num_split_reqs", "kv_dtype", "dcp_size",
                 "dcp_rank", "off_wg", "off_units", "off_reqs", "off_split", "max_local",
                 "page_size", "plan_bytes", "workspace_bytes", "ws_lse_offset", "ws_sc_offset")


def _aligned_bytes(n: int) -> np.ndarray:
    raw = np.zeros(n + 64, dtype=np.uint8)
    off = (-raw.ctypes.data) % 64
    return raw[off:off + n]


@dataclass
class Plan:
    """A decode plan: the host blob, its header fields and (optionally) a device copy."""
    desc: DecodeDesc
    host: np.ndarray  # uint8, exactly plan_bytes long, 64-byte aligned
    header: dict
    device: object = None  # torch uint8 tensor on the GPU

    @property
    def workspace_bytes(self) -> int:
        return self.header["workspace_bytes"]

    def wg_begin(self) -> np.ndarray:
        h = self.header
        return self.host[h["off_wg"]:h["off_wg"] + 4 * (h["num_wgs"] + 1)].view(np.int32)

    def units(self) -> np.ndarray:
        """int32 [num_units, 8]: b, g, j0, j1, part, pad, pad, pad."""
        h = self.header
        return self.host[h["off_units"]:h["off_units"] + 32 * h["num_units"]].view(
            np.int32).reshape(-1, 8)

    def req_parts(self) -> np.ndarray:
        h = self.header
        return self.host[h["off_reqs"]:h["off_reqs"] + 8 * h["batch"]].view(
            np.int32).reshape(-1, 2)

    def split_reqs(self) -> np.ndarray:
        """int32 [num_split_reqs, 4]: b, first_part, num_parts, pad."""
        h = self.header
        return self.host[h["off_split"]:h["off_split"] + 16 * h["num_split_reqs"]].view(
            np.int32).reshape(-1, 4)

    def to_device(self, device="cuda"):
        import torch
        self.device = torch.from_numpy(self.host.copy()).to(device)
        return self


def make_desc(batch: int, q_len: int, num_heads: int, kv_dtype="bf16", page_size: int = 64,
              dcp_size: int = 1, dcp_rank: int = 0, num_cus: int = 0,
              force_splits: int = 0) -> DecodeDesc:
    kv = _KV_CODES[kv_dtype] if isinstance(kv_dtype, str) else int(kv_dtype)
    return DecodeDesc(batch, q_len, num_heads, 512, 64, page_size, kv, dcp_size, dcp_rank,
                      num_cus, force_splits)


def plan_max_bytes(desc: DecodeDesc) -> int:
    return int(load_library().mla_plan_max_bytes(ctypes.byref(desc)))


def make_plan(desc: DecodeDesc, seq_lens, device=None) -> Plan:
    """Run the host planner (mla_decode_plan) for global lengths seq_lens."""
    lib = load_library()
    lens = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    if lens.shape != (desc.batch,):
        raise MlaError(f"seq_lens must have {desc.batch} entries")
    cap = plan_max_bytes(desc)
    if cap == 0:
        raise MlaError("invalid decode description")
    buf = _aligned_bytes(cap)
    nbytes, ws = ctypes.c_size_t(0), ctypes.c_size_t(0)
    st = lib.mla_decode_plan(ctypes.byref(desc), lens.ctypes.data, buf.ctypes.data, cap,
                             ctypes.byref(nbytes), ctypes.byref(ws))
    if st != MLA_OK:
        raise MlaError("mla_decode_plan failed", st)
    host = buf[:nbytes.value]
    header = dict(zip(_HEADER_NAMES, _HEADER.unpack_from(host.tobytes(), 0)))
    p = Plan(desc=desc, host=host, header=header)
    if device is not None:
        p.to_device(device)
    return p


def check_table(desc: DecodeDesc, seq_lens, req_to_token, num_slots: int) -> None:
    """mla_check_table on a host copy of the table: raises MlaError naming the
    first entry that is out of the pool or breaks the 32-slot runs a paged
    plan relies on."""
    lens = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    if lens.shape != (desc.batch,):
        raise MlaError(f"seq_lens must have {desc.batch} entries")
    if hasattr(req_to_token, "cpu"):
        req_to_token = req_to_token.cpu().numpy()
    table = np.ascontiguousarray(np.asarray(req_to_token, dtype=np.int32))
    if table.ndim != 2 or table.shape[0] != desc.batch:
        raise MlaError("req_to_token must be [batch, stride]")
    bad_b, bad_j = ctypes.c_int64(0), ctypes.c_int64(0)
    st = load_library().mla_check_table(ctypes.byref(desc), lens.ctypes.data,
                                        table.ctypes.data, int(table.shape[1]), int(num_slots),
                                        ctypes.byref(bad_b), ctypes.byref(bad_j))
    if st != MLA_OK:
        where = "" if bad_b.value < 0 else f" at request {bad_b.value}, index {bad_j.value}"
        raise MlaError(f"req_to_token breaks the table contract{where}", st)


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _stream(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def decode(plan: Plan, q_nope, q_rope, kv_pool, kv_scale, req_to_token, seq_lens,
           softmax_scale: float, workspace=None, out=None, lse=None, stream=None,
           phase: str = "both", verify_table: bool = False):
    """mla_decode on torch device tensors; allocates out / lse / workspace if not given.

    phase "attend" runs only mla_decode_attend, "merge" only mla_decode_merge
    (same arguments; the workspace must then be the one the attend call used).
    verify_table copies req_to_token and seq_lens to the host first and runs
    mla_check_table on them (a synchronizing debug check).
    """
    if phase not in ("both", "attend", "merge"):
        raise MlaError(f"unknown phase {phase!r}")
    import torch
    h = plan.header
    if plan.device is None:
        raise MlaError("plan has no device copy (call plan.to_device())")
    B, M = h["batch"], h["rows"]
    dev = q_nope.device
    for name, t in (("q_nope", q_nope), ("q_rope", q_rope), ("kv_pool", kv_pool),
                    ("req_to_token", req_to_token), ("seq_lens", seq_lens)):
        if t.device != dev or not t.is_contiguous():
            raise MlaError(f"{name} must be a contiguous tensor on {dev}")
    if q_nope.dtype != torch.bfloat16 or q_rope.dtype != torch.bfloat16:
        raise MlaError("q_nope / q_rope must be bfloat16")
    if tuple(q_nope.shape) != (B, h["q_len"], h["num_heads"], 512) or \
            tuple(q_rope.shape) != (B, h["q_len"], h["num_heads"], 64):
        raise MlaError("query shapes do not match the plan")
    fp8 = h["kv_dtype"] == KV_FP8
    if h["kv_dtype"] in _BLOCK_ROW_BYTES:
        rb = _BLOCK_ROW_BYTES[h["kv_dtype"]]
        if kv_pool.dtype != torch.uint8 or kv_pool.dim() != 2 or kv_pool.shape[1] != rb:
            raise MlaError(f"this plan's pools must be uint8 [num_slots, {rb}]")
    else:
        want_pool = torch.uint8 if fp8 else torch.bfloat16
        if kv_pool.dtype not in ((want_pool, torch.float8_e4m3fn) if fp8 else (want_pool,)) or \
                kv_pool.dim() != 2 or kv_pool.shape[1] != 576:
            raise MlaError("kv_pool must be [num_slots, 576] of the plan's dtype")
    if fp8 and (kv_scale is None or kv_scale.dtype != torch.float32 or
                kv_scale.numel() < kv_pool.shape[0] or kv_scale.device != dev):
        raise MlaError("FP8 pools need an fp32 kv_scale per slot on the same device")
    if req_to_token.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise MlaError("req_to_token and seq_lens must be int32")
    if req_to_token.dim() != 2 or req_to_token.shape[0] != B:
        raise MlaError("req_to_token must be [batch, stride]")
    if seq_lens.dim() != 1 or seq_lens.numel() != B:
        raise MlaError(f"seq_lens must hold {B} entries")
    o_shape = (B, h["q_len"], h["num_heads"], 512)
    if out is None:
        out = torch.empty(o_shape, dtype=torch.float32, device=dev)
    elif out.dtype != torch.float32 or tuple(out.shape) != o_shape or out.device != dev or \
            not out.is_contiguous():
        raise MlaError(f"out must be a contiguous float32 {list(o_shape)} tensor on {dev}")
    if lse is None:
        lse = torch.empty(o_shape[:3], dtype=torch.float32, device=dev)
    elif lse.dtype != torch.float32 or tuple(lse.shape) != o_shape[:3] or lse.device != dev or \
            not lse.is_contiguous():
        raise MlaError(f"lse must be a contiguous float32 {list(o_shape[:3])} tensor on {dev}")
    ws_bytes = h["workspace_bytes"]
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    elif workspace is not None and (workspace.dtype != torch.uint8 or workspace.device != dev or
                                    not workspace.is_contiguous()):
        raise MlaError(f"workspace must be a contiguous uint8 tensor on {dev}")
    if verify_table:
        check_table(plan.desc, seq_lens.cpu().numpy(), req_to_token.cpu().numpy(),
                    int(kv_pool.shape[0]))
    ws_given = 0 if workspace is None else int(workspace.numel() * workspace.element_size())
    lib = load_library()
    if phase == "merge":
        st = lib.mla_decode_merge(plan.host.ctypes.data, _ptr(plan.device), _ptr(workspace),
                                  ws_given, _ptr(out), _ptr(lse), _stream(stream))
    else:
        fn = lib.mla_decode if phase == "both" else lib.mla_decode_attend
        st = fn(plan.host.ctypes.data, _ptr(plan.device), _ptr(q_nope), _ptr(q_rope),
                _ptr(kv_pool), _ptr(kv_scale if fp8 else None), int(kv_pool.shape[0]),
                _ptr(req_to_token), int(req_to_token.shape[1]), _ptr(seq_lens),
                float(softmax_scale), _ptr(workspace), ws_given, _ptr(out), _ptr(lse),
                _stream(stream))
    if st != MLA_OK:
        raise MlaError(f"mla_decode ({phase}) failed", st)
    return out, lse


def decode_noalloc(plan: Plan, q_nope, q_rope, kv_pool, kv_scale, req_to_token, seq_lens,
                   softmax_scale: float, out, lse, stream=None):
    """mla_decode_noalloc: mla_decode with the split partials in the library's
    per-GPU scratch array.  out / lse must be given (nothing is allocated)."""
    import torch
    h = plan.header
    o_shape = (h["batch"], h["q_len"], h["num_heads"], 512)
    for name, t, shape in (("out", out, o_shape), ("lse", lse, o_shape[:3])):
        if t is None or t.dtype != torch.float32 or tuple(t.shape) != shape or \
                t.device != q_nope.device or not t.is_contiguous():
            raise MlaError(f"{name} must be a contiguous float32 {list(shape)} tensor on "
                           f"{q_nope.device}")
    if plan.device is None:
        raise MlaError("plan has no device copy (call plan.to_device())")
    fp8 = h["kv_dtype"] == KV_FP8
    if seq_lens.numel() != h["batch"] or seq_lens.dtype != torch.int32:
        raise MlaError(f"seq_lens must be int32 with {h['batch']} entries")
    if req_to_token.dim() != 2 or req_to_token.shape[0] != h["batch"] or \
            req_to_token.dtype != torch.int32:
        raise MlaError("req_to_token must be int32 [batch, stride]")
    st = load_library().mla_decode_noalloc(
        plan.host.ctypes.data, _ptr(plan.device), _ptr(q_nope), _ptr(q_rope), _ptr(kv_pool),
        _ptr(kv_scale if fp8 else None), int(kv_pool.shape[0]), _ptr(req_to_token),
        int(req_to_token.shape[1]), _ptr(seq_lens), float(softmax_scale), _ptr(out), _ptr(lse),
        _stream(stream))
    if st != MLA_OK:
        raise MlaError("mla_decode_noalloc failed", st)
    return out, lse


def lse_combine(part_o, part_lse, out=None, lse=None, stream=None):
    """mla_lse_combine: merge [P, ..., 512] / [P, ...] partials into [..., 512] / [...]."""
    import torch
    P = part_o.shape[0]
    rows = int(np.prod(part_o.shape[1:-1])) if part_o.dim() > 2 else part_o.shape[1]
    if part_o.shape[-1] != 512 or tuple(part_lse.shape) != tuple(part_o.shape[:-1]):
        raise MlaError("part_o must be [P, ..., 512] and part_lse [P, ...]")
    if not (part_o.is_contiguous() and part_lse.is_contiguous()):
        raise MlaError("partials must be contiguous")
    if part_o.dtype != torch.float32 or part_lse.dtype != torch.float32:
        raise MlaError("partials must be float32")
    if out is None:
        out = torch.empty(part_o.shape[1:], dtype=torch.float32, device=part_o.device)
    if lse is None:
        lse = torch.empty(part_lse.shape[1:], dtype=torch.float32, device=part_o.device)
    st = load_library().mla_lse_combine(_ptr(part_o), _ptr(part_lse), int(P), int(rows),
                                        _ptr(out), _ptr(lse), _stream(stream))
    if st != MLA_OK:
        raise MlaError("mla_lse_combine failed", st)
    return out, lse


def prepare(q_nope, q_rope_in, w_kc_t, c_kv_new, k_rope_new, positions, cos_sin, slots,
            kv_pool, kv_scale=None, q_nope_absorbed=None, q_rope_out=None, stream=None):
    """mla_prepare on torch device tensors.

    Shapes: q_nope [T, H, 128], q_rope_in [T, H, 64], w_kc_t [H, 512, 128],
    c_kv_new [T, 512], k_rope_new [T, 64] (bf16); positions, slots int32 [T];
    cos_sin fp32 [max_pos, 64]; kv_pool [num_slots, 576] (bf16, or uint8 /
    float8_e4m3fn with an fp32 kv_scale [num_slots]), or uint8 [num_slots,
    336] for FP4 rows, [num_slots, 608] for MXFP8 rows.  Returns
    (q_nope_absorbed [T, H, 512], q_rope_out [T, H, 64]); the pool rows at
    `slots` (and their scales) are written in place.
    """
    import torch
    T, H = int(q_nope.shape[0]), int(q_nope.shape[1])
    dev = q_nope.device
    bf = torch.bfloat16
    checks = (("q_nope", q_nope, (T, H, 128), bf), ("q_rope_in", q_rope_in, (T, H, 64), bf),
              ("w_kc_t", w_kc_t, (H, 512, 128), bf), ("c_kv_new", c_kv_new, (T, 512), bf),
              ("k_rope_new", k_rope_new, (T, 64), bf), ("positions", positions, (T,), torch.int32),
              ("slots", slots, (T,), torch.int32))
    for name, t, shape, dt in checks:
        if tuple(t.shape) != shape or t.dtype != dt or t.device != dev or not t.is_contiguous():
            raise MlaError(f"{name} must be a contiguous {dt} tensor of shape {shape} on {dev}")
    if cos_sin.dtype != torch.float32 or cos_sin.dim() != 2 or cos_sin.shape[1] != 64 or \
            not cos_sin.is_contiguous():
        raise MlaError("cos_sin must be a contiguous float32 [max_pos, 64] tensor")
    block = None
    if kv_pool.dtype == torch.uint8 and kv_pool.dim() == 2:
        block = {FP4_ROW_BYTES: KV_FP4, MXFP8_ROW_BYTES: KV_MXFP8}.get(int(kv_pool.shape[1]))
    fp8 = block is None and kv_pool.dtype in (torch.uint8, torch.float8_e4m3fn)
    if kv_pool.dim() != 2 or not (block is not None or (kv_pool.shape[1] == 576 and
                                                        (fp8 or kv_pool.dtype == bf))):
        raise MlaError("kv_pool must be [num_slots, 576] of bf16 or e4m3fn bytes, or "
                       f"uint8 [num_slots, {FP4_ROW_BYTES}] FP4 / [num_slots, "
                       f"{MXFP8_ROW_BYTES}] MXFP8 rows")
    if fp8 and (kv_scale is None or kv_scale.dtype != torch.float32):
        raise MlaError("FP8 pools need an fp32 kv_scale per slot")
    if q_nope_absorbed is None:
        q_nope_absorbed = torch.empty((T, H, 512), dtype=bf, device=dev)
    if q_rope_out is None:
        q_rope_out = torch.empty((T, H, 64), dtype=bf, device=dev)
    st = load_library().mla_prepare(
        T, H, block if block is not None else (KV_FP8 if fp8 else KV_BF16), _ptr(q_nope), _ptr(q_rope_in), _ptr(w_kc_t),
        _ptr(c_kv_new), _ptr(k_rope_new), _ptr(positions), _ptr(cos_sin), int(cos_sin.shape[0]),
        _ptr(slots), _ptr(q_nope_absorbed), _ptr(q_rope_out), _ptr(kv_pool),
        _ptr(kv_scale if fp8 else None), int(kv_pool.shape[0]), _stream(stream))
    if st != MLA_OK:
        raise MlaError("mla_prepare failed", st)
    return q_nope_absorbed, q_rope_out


def lse_combine_project(part_o, part_lse, w_vc_t, out_v=None, lse=None, stream=None):
    """mla_lse_combine_project: merge [P, T, H, 512] / [P, T, H] partials by LSE
    and project the merged rows with w_vc_t [H, 128, 512] (bf16).  Returns
    (out_v bf16 [T, H, 128], lse fp32 [T, H])."""
    import torch
    if part_o.dim() != 4 or part_o.shape[-1] != 512 or part_o.dtype != torch.float32 or \
            tuple(part_lse.shape) != tuple(part_o.shape[:3]) or part_lse.dtype != torch.float32:
        raise MlaError("part_o must be fp32 [P, T, H, 512] and part_lse fp32 [P, T, H]")
    P, T, H = (int(v) for v in part_o.shape[:3])
    if tuple(w_vc_t.shape) != (H, 128, 512) or w_vc_t.dtype != torch.bfloat16:
        raise MlaError("w_vc_t must be bf16 [H, 128, 512]")
    for name, t in (("part_o", part_o), ("part_lse", part_lse), ("w_vc_t", w_vc_t)):
        if not t.is_contiguous() or t.device != part_o.device:
            raise MlaError(f"{name} must be contiguous on {part_o.device}")
    if out_v is None:
        out_v = torch.empty((T, H, 128), dtype=torch.bfloat16, device=part_o.device)
    if lse is None:
        lse = torch.empty((T, H), dtype=torch.float32, device=part_o.device)
    st = load_library().mla_lse_combine_project(_ptr(part_o), _ptr(part_lse), P, T, H,
                                                _ptr(w_vc_t), _ptr(out_v), _ptr(lse),
                                                _stream(stream))
    if st != MLA_OK:
        raise MlaError("mla_lse_combine_project failed", st)
    return out_v, lse
