"""Generates tile_asm.inc: the tile work of the decode loop as inline-asm
statements in which LDS reads, the softmax, the FP4 dequantization,
global->LDS DMA and MFMAs are software-pipelined by hand.

Building blocks of a statement (any combination):

  QK    S^T = K . Q^T of one tile: BF16 36 MFMAs 32x32x16; FP8 16 scaled
        MFMAs 32x32x64 on the stored codes against two e4m3 terms of Q, plus
        the RoPE part on 4 BF16 MFMAs (its codes widened in registers)
  PV    O^T += V^T . P^T of one tile: BF16 32 MFMAs; FP8 16 scaled MFMAs
        (the codes against two e4m3 terms of P)
  SM    the online softmax of one tile, given its scores: scale, max, the
        lazy rescale decision, exponentials, row sum and P packed to BF16
  DMA   the global->LDS copy of a later tile (row instructions)

Statements (T = BF16 or FP8):

  MLA_QK_T_ASM       QK (first tile of a unit)
  MLA_FUSED_BF16_ASM QK of tile t+1 and PV of tile t, plus DMA
  MLA_FUSED_BF16_DQ_ASM  the same without the DMA, plus the dequantization
                     of a raw FP4 tile (FP4 pools: their DMA is issued outside)
  MLA_DQ_FP4_ASM     that dequantization alone (a wave with no rows)
  MLA_FUSED_BF16_DQMX_ASM, MLA_DQ_MX_ASM  the same two for a raw MXFP8 tile
  MLA_PV_T_ASM       PV (last tile of a unit)
  FP8, pipelined one tile deeper so that the softmax runs in the MFMA shadow:
  MLA_QKSM_FP8_ASM   QK of tile t+1 and SM of tile t, plus DMA (first step)
  MLA_STEP_FP8_ASM   QK of tile t+1, SM of tile t and PV of tile t-1, plus DMA
  MLA_SMPV_FP8_ASM   SM of tile t and PV of tile t-1 (last step)
  MLA_SM_FP8_ASM     SM alone (one-tile units)
  MLA_LOOP_FP8_ASM   the whole tile loop of a paged FP8 unit of two or more
                     tiles (a wave with rows): the steps above unrolled by
                     the 8-buffer ring, each with its workgroup barrier, the
                     DMA of tile t+6 and the table walk (fp8_loop)
  MLA_RESCALE_ASM    O *= alpha over all 256 accumulators

QK and PV MFMAs alternate one for one, so the dependent S chain never stalls
the matrix pipe while PV MFMAs remain, and the VALU and LDS work (widening,
softmax, dequantization) issues between MFMAs, in the shadow of the one that
is running.  A
small list scheduler (below) assigns scratch registers in rings, issues each
LDS read as early as its ring slot allows, waits for it with the exact lgkmcnt
(LDS operations complete in issue order), keeps every VALU result two
instructions away from an MFMA that reads it and every transcendental result
one instruction away from its first reader.

Operand names:
  %[q0]..%[q35]  Q^T operands (bf16x8) of k-steps 0..35
  %[s], %[s1]    S^T accumulator chains of the tile being scored (written);
                 statements with PV put k-steps 33 and 35 in s1, QK-only
                 statements the odd k-steps
  %[a0]..%[a15]  O^T accumulators (AGPR f32x16, read-write), pinned by the
                 caller to a[16 d : 16 d + 15]; MLA_RESCALE_ASM (O *= %[al])
                 names them a0..a255
  %[p0], %[p1]   P^T operands (bf16x8) of the two 16-token halves of the tile
                 whose PV runs
  %[ke], %[ko]   BF16 K lane addresses (even / odd k-steps); %[kb] FP8
  %[va], %[vb]   V^T lane addresses of the two token-row sets
  %[x0]..%[x15]  SM: the 16 scores of this lane (read-write); on return
                 %[x0]..%[x7] hold P as 8 packed BF16 pairs
  %[mref], %[lsum]  SM: running max (raw units) and row-sum share (read-write)
  %[alpha]       SM: factor the O accumulators must be multiplied by (written)
  %[c2], %[nfm]  SM scalars: softmax_scale * log2(e) and -FLT_MAX
  %[bpa]         SM: byte address of lane ^ 32 for ds_bpermute_b32
  %[mon], %[limh], %[ninf]  SM mask: nonzero (scalar) if some token of the
                 tile lies past a row's last visible index; the last visible
                 token minus 4 hk (per lane); -inf (scalar)
  %[sc]          SM, FP8: LDS address of this lane's first 4 token scales
  %[m0b], %[m0s] DMA: LDS base of this wave's share; scratch SGPR that keeps
                 M0, which the statement restores; the address operands
                 appear in the MLA_GLD(offset) macro
Each statement clobbers its scratch registers (<NAME>_CLOBBERS, the top of the
VGPR file), VCC and SCC.

K operands.  BF16: k-step ks reads chunk 2 ks + hk (8 features) of the lane's
token with one ds_read_b128.  FP8: one ds_read_b128 per k-step pair a fetches
chunk 2 a + hk (16 codes) of the lane's token; k-step 2 a + h uses codes
8 h .. 8 h + 7, so k-step 2 a + h, half hk covers features 16 (2 a + hk) +
8 h .. + 8, and the Q operands are loaded in that order.

V^T operand of block db (features 32 db .. +32), token half e.  BF16: two
ds_read_b64_tr_b16 at %[va] / %[vb] + 2048 db + 256 e.  FP8: one
ds_read_b64_tr_b8 at (e ? %[vb] : %[va]) + 1024 db, widened in registers.

SM, per lane (16 scores x_i of one query row; token of x_i is
8 (i / 4) + 4 hk + i % 4): FP8 x_i *= scale_i; m_t = max over the row (the
other half of the row sits in lane ^ 32); if (m_t - mref) c2 > 8 the running
max moves to m_t and alpha = 2^((mref - m_t) c2), else alpha = 1; lsum *= alpha;
e_i = 2^(x_i c2 - m c2) (with m c2 floored at -FLT_MAX, so a row with nothing
visible yet gives e = 0); lsum += sum e_i; P_i = e_i, packed to BF16 with
round-to-nearest-even (FP8: P_i = e_i * scale_i as two e4m3 terms, hi and the
rounded remainder lo, in units of 2^(E-8) where 2^E bounds the row's P in the
tile; the E8M0 code of 2^(E-8) goes to %[psco] for the P.V MFMAs).

DMA.  Row instruction k (k = 0..3 FP8, 0..8 BF16) moves 16 bytes per lane from
the lane's row address + 128 k to LDS %[m0b] + 4096 k + 16 lane (the
immediate offset applies to both addresses, so M0 advances by 4096 - 128).

Run `python gen_tile_asm.py` after editing; the output is committed.
"""

from __future__ import annotations

import math
import os
import re

SCRATCH_HI = 255   # rings are allocated downwards from here


def fp8_v_order():
    """FP8 PV ops: feature blocks, each MFMA covering the whole tile."""
    return list(range(16))


def v_order():
    """PV ops (db, e): feature blocks in pairs so that the two MFMAs into
    one accumulator are never adjacent."""
    seq = []
    for p in range(8):
        for e in (0, 1):
            for db in (2 * p, 2 * p + 1):
                seq.append((db, e))
    return seq


class Read:
    def __init__(self, rid, ring, instrs, widen_inplace=False, dup_half=False):
        self.rid = rid
        self.ring = ring
        self.instrs = instrs    # templates; {r} .. {r7} = ring slot registers
        self.widen_inplace = widen_inplace  # 16 codes in r4..r7 -> 16 BF16 in r0..r7
        self.dup_half = dup_half            # r4..r7 = copy of r0..r3
        self.users = []         # stream positions of its consumers
        self.need = None        # first position that needs the data


class Op:
    def __init__(self, kind, mfma, read, acc=None, xoff=0):
        self.kind = kind        # "K" or "V"
        self.xoff = xoff        # first register of the A operand within the read's slot
        self.acc = acc
        self.mfma = mfma        # template: {acc} {x} {x3} {c}
        self.read = read        # rid feeding the A operand


class Stream:
    def __init__(self, rings):
        self.lines = []
        self.lgkm = []          # LDS op tags in issue order
        self.done = -1          # index of the last LDS op known complete
        self.last_valu = {}     # register -> len(lines) after it was written
        self.trans_at = {}      # operand text -> len(lines) after a TRANS op wrote it
        self.base = {}
        self.rings = rings
        r = SCRATCH_HI + 1
        for name, (n, w) in rings.items():
            r -= n * w
            self.base[name] = r
        self.lowest = r

    def reg(self, ring, slot):
        n, w = self.rings[ring]
        return self.base[ring] + (slot % n) * w

    def emit(self, line):
        self.lines.append(line)

    def lds(self, line, tag):
        self.emit(line)
        self.lgkm.append(tag)

    def outstanding(self):
        return len(self.lgkm) - 1 - self.done

    def wait_index(self, last):
        if last <= self.done:
            return
        n = len(self.lgkm) - 1 - last
        self.emit(f"s_waitcnt lgkmcnt({min(n, 15)})")
        self.done = last if n <= 15 else len(self.lgkm) - 16

    def wait(self, tag):
        self.wait_index(max(i for i, t in enumerate(self.lgkm) if t == tag))


def sm_program(fp8: bool, sk: int, tmp: int):
    """The softmax of one tile as a list of (kind, text, reads, writes, tag).

    kind: "valu", "trans" (v_exp_f32), "lds" (an LDS read; tag names it),
    "wait" (wait for the LDS read `tag`).  reads / writes are operand texts,
    for the transcendental-result spacing.  sk: base of a 4-register scale
    slot; tmp: base of 4 temporaries."""
    x = [f"%[x{i}]" for i in range(16)]
    t = [f"v{tmp + i}" for i in range(4)]
    prog = []
    n_scale_reads = [0]

    def valu(text, reads, writes, kind="valu"):
        prog.append((kind, text, reads, writes, None))

    def scale_read(c):
        tag = ("SC", n_scale_reads[0])
        n_scale_reads[0] += 1
        prog.append(("lds", f"ds_read_b128 v[{sk}:{sk + 3}], %[sc] offset:{32 * c}", [], [], tag))
        return sk, tag

    def scale_pass():
        # x_i *= scale_i, four tokens per 16-byte read (one slot: the stream
        # scheduler defers the wait, so other work covers the latency).
        for c in range(4):
            slot, tag = scale_read(c)
            prog.append(("wait", "", [], [], tag))
            for j in range(4):
                i = 4 * c + j
                valu(f"v_mul_f32 {x[i]}, {x[i]}, v{slot + j}", [x[i]], [x[i]])

    if fp8:
        scale_pass()
    # Causal / range mask (only tiles that need it, %[mon] != 0): token
    # 8 (i / 4) + 4 hk + i % 4 is visible iff 8 (i / 4) + i % 4 <= %[limh].
    # One block, so that nothing else lands between the branch and its label.
    # (-inf goes through a VGPR: v_cndmask reads VCC over the constant bus.)
    block = ["s_cmp_eq_u32 %[mon], 0", "s_cbranch_scc1 88f", f"v_mov_b32 {t[3]}, %[ninf]"]
    for i in range(16):
        block.append(f"v_cmp_le_i32 vcc, {8 * (i >> 2) + (i & 3)}, %[limh]")
        block.append("s_nop 1")  # VALU-written VCC read as a lane mask
        block.append(f"v_cndmask_b32 {x[i]}, {t[3]}, {x[i]}, vcc")
    block.append("88:")
    prog.append(("block", block, list(x), list(x) + ["vcc"], None))
    # Row max of this lane's 16 scores.
    valu(f"v_max3_f32 {t[0]}, {x[0]}, {x[1]}, {x[2]}", x[0:3], [t[0]])
    valu(f"v_max3_f32 {t[1]}, {x[3]}, {x[4]}, {x[5]}", x[3:6], [t[1]])
    valu(f"v_max3_f32 {t[0]}, {t[0]}, {t[1]}, {x[6]}", [t[0], t[1], x[6]], [t[0]])
    valu(f"v_max3_f32 {t[1]}, {x[7]}, {x[8]}, {x[9]}", x[7:10], [t[1]])
    valu(f"v_max3_f32 {t[0]}, {t[0]}, {t[1]}, {x[10]}", [t[0], t[1], x[10]], [t[0]])
    valu(f"v_max3_f32 {t[1]}, {x[11]}, {x[12]}, {x[13]}", x[11:14], [t[1]])
    valu(f"v_max3_f32 {t[0]}, {t[0]}, {t[1]}, {x[14]}", [t[0], t[1], x[14]], [t[0]])
    valu(f"v_max_f32 {t[0]}, {t[0]}, {x[15]}", [t[0], x[15]], [t[0]])
    # ... and of the other half of the row (lane ^ 32).
    prog.append(("lds", f"ds_bpermute_b32 {t[1]}, %[bpa], {t[0]}", [t[0]], [], ("BP",)))
    prog.append(("wait", "", [], [], ("BP",)))
    valu(f"v_max_f32 {t[0]}, {t[0]}, {t[1]}", [t[0], t[1]], [t[0]])
    # Lazy rescale: the running max moves only when the tile max exceeds it
    # by more than 8 in the exponent, (m_t - mref) c2 > 8 (a row with no
    # visible token yet has mref = -inf and moves as soon as m_t is finite).
    # One block: when no lane's max moves (the usual case) the new max is the
    # old one and alpha = 1, and the branch skips the update; the two moves
    # also keep the VALU-written VCC three instructions from its first use
    # as a lane mask, and the move after the exponential keeps its result
    # one instruction from its reader.
    valu(f"v_sub_f32 {t[1]}, {t[0]}, %[mref]", [t[0], "%[mref]"], [t[1]])
    valu(f"v_mul_f32 {t[1]}, %[c2], {t[1]}", [t[1]], [t[1]])
    valu(f"v_cmp_lt_f32 vcc, 8.0, {t[1]}", [t[1]], ["vcc"])
    lazy = [f"v_mov_b32 {t[2]}, %[mref]",
            "v_mov_b32 %[alpha], 1.0",
            "s_cbranch_vccz 89f",
            f"v_cndmask_b32 {t[2]}, %[mref], {t[0]}, vcc",
            f"v_sub_f32 {t[3]}, %[mref], {t[2]}",
            f"v_mul_f32 {t[3]}, %[c2], {t[3]}",
            f"v_exp_f32 {t[3]}, {t[3]}",
            f"v_mov_b32 %[mref], {t[2]}",
            f"v_cndmask_b32 %[alpha], 1.0, {t[3]}, vcc",
            "v_mul_f32 %[lsum], %[lsum], %[alpha]",
            "89:"]
    prog.append(("block", lazy, [t[0], "%[mref]", "%[lsum]", "vcc"],
                 [t[2], t[3], "%[alpha]", "%[mref]", "%[lsum]"], None))
    # m c2, floored so that an all-masked row (m = -inf) gives e = 0.
    valu(f"v_mul_f32 {t[3]}, %[c2], {t[2]}", [t[2]], [t[3]])
    valu(f"v_max_f32 {t[3]}, %[nfm], {t[3]}", [t[3]], [t[3]])
    for i in range(16):
        valu(f"v_fma_f32 {x[i]}, {x[i]}, %[c2], -{t[3]}", [x[i], t[3]], [x[i]])
    for i in range(16):
        valu(f"v_exp_f32 {x[i]}, {x[i]}", [x[i]], [x[i]], kind="trans")
    # Row-sum share: pairwise tree, then into lsum.
    valu(f"v_add_f32 {t[0]}, {x[0]}, {x[1]}", x[0:2], [t[0]])
    valu(f"v_add_f32 {t[1]}, {x[2]}, {x[3]}", x[2:4], [t[1]])
    valu(f"v_add_f32 {t[2]}, {x[4]}, {x[5]}", x[4:6], [t[2]])
    valu(f"v_add_f32 {t[3]}, {x[6]}, {x[7]}", x[6:8], [t[3]])
    valu(f"v_add_f32 {t[0]}, {t[0]}, {t[1]}", [t[0], t[1]], [t[0]])
    valu(f"v_add_f32 {t[2]}, {t[2]}, {t[3]}", [t[2], t[3]], [t[2]])
    valu(f"v_add_f32 {t[1]}, {x[8]}, {x[9]}", x[8:10], [t[1]])
    valu(f"v_add_f32 {t[3]}, {x[10]}, {x[11]}", x[10:12], [t[3]])
    valu(f"v_add_f32 {t[0]}, {t[0]}, {t[2]}", [t[0], t[2]], [t[0]])
    valu(f"v_add_f32 {t[1]}, {t[1]}, {t[3]}", [t[1], t[3]], [t[1]])
    valu(f"v_add_f32 {t[2]}, {x[12]}, {x[13]}", x[12:14], [t[2]])
    valu(f"v_add_f32 {t[3]}, {x[14]}, {x[15]}", x[14:16], [t[3]])
    valu(f"v_add_f32 {t[0]}, {t[0]}, {t[1]}", [t[0], t[1]], [t[0]])
    valu(f"v_add_f32 {t[2]}, {t[2]}, {t[3]}", [t[2], t[3]], [t[2]])
    valu(f"v_add_f32 {t[0]}, {t[0]}, {t[2]}", [t[0], t[2]], [t[0]])
    valu(f"v_add_f32 %[lsum], %[lsum], {t[0]}", ["%[lsum]", t[0]], ["%[lsum]"])
    if not fp8:
        for j in range(8):
            valu(f"v_cvt_pk_bf16_f32 {x[j]}, {x[2 * j]}, {x[2 * j + 1]}",
                 [x[2 * j], x[2 * j + 1]], [x[j]])
        return prog
    scale_pass()   # P_i = e_i * scale_i (the value scale of token i)
    # P as two e4m3 terms for the FP8 P.V product, in units of 2^(E - 8)
    # where 2^E bounds the row's P in this tile (both lanes of the row agree
    # on E, clamped so that the block-scale code stays in 1..254):
    # hi_i = rne(P_i / 2^(E-8)), lo_i = rne((P_i - hi_i 2^(E-8)) / 2^(E-8)).
    # The hi codes of x_{4d..4d+3} end in dword x_d, the lo codes in x_{4+d};
    # %[psco] = 119 + E, the E8M0 code of 2^(E-8) (the MFMA block scale of
    # both terms).
    # Four more temporaries: the scale slot, free after the last scale pass.
    t4, t5, t6, t7 = (f"v{sk + i}" for i in range(4))
    valu(f"v_max3_f32 {t[0]}, {x[0]}, {x[1]}, {x[2]}", x[0:3], [t[0]])
    valu(f"v_max3_f32 {t[1]}, {x[3]}, {x[4]}, {x[5]}", x[3:6], [t[1]])
    valu(f"v_max3_f32 {t[0]}, {t[0]}, {t[1]}, {x[6]}", [t[0], t[1], x[6]], [t[0]])
    valu(f"v_max3_f32 {t[1]}, {x[7]}, {x[8]}, {x[9]}", x[7:10], [t[1]])
    valu(f"v_max3_f32 {t[0]}, {t[0]}, {t[1]}, {x[10]}", [t[0], t[1], x[10]], [t[0]])
    valu(f"v_max3_f32 {t[1]}, {x[11]}, {x[12]}, {x[13]}", x[11:14], [t[1]])
    valu(f"v_max3_f32 {t[0]}, {t[0]}, {t[1]}, {x[14]}", [t[0], t[1], x[14]], [t[0]])
    valu(f"v_max_f32 {t[0]}, {t[0]}, {x[15]}", [t[0], x[15]], [t[0]])
    prog.append(("lds", f"ds_bpermute_b32 {t[1]}, %[bpa], {t[0]}", [t[0]], [], ("BP2",)))
    prog.append(("wait", "", [], [], ("BP2",)))
    valu(f"v_max_f32 {t[0]}, {t[0]}, {t[1]}", [t[0], t[1]], [t[0]])
    valu(f"v_frexp_exp_i32_f32 {t[1]}, {t[0]}", [t[0]], [t[1]])
    valu(f"v_max_i32 {t[1]}, 0xffffff8a, {t[1]}", [t[1]], [t[1]])   # E >= -118
    valu(f"v_min_i32 {t[1]}, 0x87, {t[1]}", [t[1]], [t[1]])         # E <= 135
    valu(f"v_add_u32 {t[3]}, -8, {t[1]}", [t[1]], [t[3]])
    valu(f"v_ldexp_f32 {t7}, 1.0, {t[3]}", [t[3]], [t7])
    valu(f"v_add_u32 %[psco], 0x77, {t[1]}", [t[1]], ["%[psco]"])
    for d in range(4):
        a, b, c, e = x[4 * d:4 * d + 4]
        hi = t4 if d == 0 else x[d]          # x_1..x_3 are free once group 0 is done
        lo = t5 if d == 0 else x[4 + d]      # x_5..x_7 are free once group 1 is read
        valu(f"v_cvt_scalef32_pk_fp8_f32 {hi}, {a}, {b}, {t7}", [a, b, t7], [hi])
        valu(f"v_cvt_scalef32_pk_fp8_f32 {hi}, {c}, {e}, {t7} op_sel:[0,0,0,1]", [c, e, t7], [hi])
        valu(f"v_cvt_scalef32_pk_f32_fp8 v[{tmp}:{tmp + 1}], {hi}, {t7}", [hi, t7], [t[0], t[1]])
        valu(f"v_cvt_scalef32_pk_f32_fp8 v[{tmp + 2}:{tmp + 3}], {hi}, {t7} op_sel:[1,0,0]",
             [hi, t7], [t[2], t[3]])
        valu(f"v_sub_f32 {a}, {a}, {t[0]}", [a, t[0]], [a])
        valu(f"v_sub_f32 {b}, {b}, {t[1]}", [b, t[1]], [b])
        valu(f"v_sub_f32 {c}, {c}, {t[2]}", [c, t[2]], [c])
        valu(f"v_sub_f32 {e}, {e}, {t[3]}", [e, t[3]], [e])
        valu(f"v_cvt_scalef32_pk_fp8_f32 {lo}, {a}, {b}, {t7}", [a, b, t7], [lo])
        valu(f"v_cvt_scalef32_pk_fp8_f32 {lo}, {c}, {e}, {t7} op_sel:[0,0,0,1]", [c, e, t7], [lo])
        if d == 0:
            valu(f"v_mov_b32 {x[0]}, {t4}", [t4], [x[0]])
        if d == 1:
            valu(f"v_mov_b32 {x[4]}, {t5}", [t5], [x[4]])
    return prog


FP4_SEL = ("", " op_sel:[1,0,0]", " op_sel:[0,1,0]", " op_sel:[1,1,0]")  # byte 0..3


def dq_program(base: int):
    """Dequantization of one raw FP4 tile into the BF16 tile layout, as a list
    of (kind, text, reads, writes, tag) like the softmax program, for the
    statement to spread over its MFMA slots.

    Raw tile: code chunk c (16 bytes: blocks 2 c and 2 c + 1) of token t at
    512 c + 16 t; the scale byte of block b of token t at 512 (18 + b / 16) +
    16 t + b % 16.  BF16 tile: chunk cc of token t at 512 cc + 16 (t ^ 4 (cc
    & 3)).  Lane (t, h) = (lane % 32, lane / 32) of wave w converts the code
    chunks c = 2 w + h and 2 w + h + 8 whole (blocks in halves of 8 bytes),
    and one dword (chunk w) of code chunk 16 + h: every wave 2.25 chunks.
    The lane terms (16 t, and 32 h from which 512 h, 2 h and 2048 h follow)
    are computed here from the lane id; the wave terms come in scalars:
    %[dqa] = raw + 1024 w, %[dqb] = raw + 4 w, %[dqc] = bf16 tile + 4096 w,
    %[dqd] = raw + w / 2, %[dqe] = 64 w, %[dqf] = bf16 tile + 512 w.
    Scratch: codes (2), one BF16 pair (2), scale, two addresses, 16 t, 32 h.
    """
    # nine registers; the two pairs start on even registers (as the ISA
    # requires), wherever the ring begins
    if base % 2:
        SC, C, O, T, T2, TT, HH = base, base + 1, base + 3, base + 5, base + 6, base + 7, base + 8
    else:
        C, O, SC, T, T2, TT, HH = base, base + 2, base + 4, base + 5, base + 6, base + 7, base + 8
    prog = []

    def valu(text):
        prog.append(("valu", text, [], [], None))

    def lds(text, tag):
        prog.append(("lds", text, [], [], tag))

    def wait(tag):
        prog.append(("wait", "", [], [], tag))

    def convert_dword(src, write_addr, off):
        # 8 codes of one dword -> one 16-byte BF16 chunk, written in halves
        for q2 in (0, 1):
            for b in (0, 1):
                valu(f"v_cvt_scalef32_pk_bf16_fp4 v{O + b}, v{src}, v{SC}{FP4_SEL[2 * q2 + b]}")
            lds(f"ds_write_b64 {write_addr}, v[{O}:{O + 1}] offset:{off + 8 * q2}", ("DQW",))

    valu(f"v_mbcnt_lo_u32_b32 v{TT}, -1, 0")
    valu(f"v_mbcnt_hi_u32_b32 v{TT}, -1, v{TT}")
    valu(f"v_and_b32 v{HH}, 32, v{TT}")                 # 32 h
    valu(f"v_and_b32 v{TT}, 31, v{TT}")
    valu(f"v_lshlrev_b32 v{TT}, 4, v{TT}")              # 16 t
    for k in (0, 1):
        for hh in (0, 1):
            tag = ("DQ", k, hh)
            valu(f"v_lshl_add_u32 v{T}, v{HH}, 4, v{TT}")           # 16 t + 512 h
            valu(f"v_add_u32 v{T}, %[dqa], v{T}")
            lds(f"ds_read_b64 v[{C}:{C + 1}], v{T} offset:{4096 * k + 8 * hh}", tag + ("c",))
            valu(f"v_lshrrev_b32 v{T}, 4, v{HH}")                   # 2 h
            valu(f"v_add3_u32 v{T}, %[dqb], v{T}, v{TT}")
            lds(f"ds_read_u8 v{SC}, v{T} offset:{9216 + 512 * k + hh}", tag + ("s",))
            wait(tag + ("s",))
            valu(f"v_lshlrev_b32 v{SC}, 23, v{SC}")
            wait(tag + ("c",))
            for jj in (0, 1):
                j = 2 * hh + jj
                valu(f"v_xor_b32 v{T2}, {64 * j}, v{TT}")
                valu(f"v_lshl_add_u32 v{T2}, v{HH}, 6, v{T2}")        # + 2048 h
                valu(f"v_add_u32 v{T2}, %[dqc], v{T2}")
                convert_dword(C + jj, f"v{T2}", 16384 * k + 512 * j)
    # The 64 units of code chunks 16, 17: wave w takes their dword w.
    tag = ("DQ", 2)
    valu(f"v_lshl_add_u32 v{T}, v{HH}, 4, v{TT}")
    valu(f"v_add_u32 v{T}, %[dqb], v{T}")
    lds(f"ds_read_b32 v{C}, v{T} offset:8192", tag + ("c",))
    valu(f"v_lshrrev_b32 v{T}, 4, v{HH}")
    valu(f"v_add3_u32 v{T}, %[dqd], v{T}, v{TT}")
    lds(f"ds_read_u8 v{SC}, v{T} offset:10240", tag + ("s",))
    wait(tag + ("s",))
    valu(f"v_lshlrev_b32 v{SC}, 23, v{SC}")
    wait(tag + ("c",))
    valu(f"v_xor_b32 v{T2}, %[dqe], v{TT}")
    valu(f"v_lshl_add_u32 v{T2}, v{HH}, 6, v{T2}")
    valu(f"v_add_u32 v{T2}, %[dqf], v{T2}")
    convert_dword(C, f"v{T2}", 32768)
    return prog


def dq_program_mx(base: int):
    """Dequantization of one raw MXFP8 tile into the BF16 tile layout (the
    MXFP8 counterpart of dq_program).

    Raw tile: code chunk c (16 e4m3fn codes, elements 16 c .. + 16, block
    c / 2) of token t at 512 c + 16 t; the scale byte of block b at 512 (36 +
    b / 16) + 16 t + b % 16.  Code chunk c becomes BF16 chunks 2 c and 2 c +
    1.  Lane (t, h) of wave w converts code chunks 2 w + h + 8 k (k = 0..3)
    whole, in halves of 8 bytes (one BF16 chunk each), and half h of code
    chunk 32 + w: every lane 4.5 chunks.  Scalars: %[dqa] = raw + 1024 w,
    %[dqb] = raw + w, %[dqc] = bf16 tile + 2048 w, %[dqd] = raw + 512 w,
    %[dqe] = raw + w / 2, %[dqf] = bf16 tile + 1024 w, %[dqg] = 128 (w % 2).
    Scratch as in dq_program.
    """
    if base % 2:
        SC, C, O, T, T2, TT, HH = base, base + 1, base + 3, base + 5, base + 6, base + 7, base + 8
    else:
        C, O, SC, T, T2, TT, HH = base, base + 2, base + 4, base + 5, base + 6, base + 7, base + 8
    prog = []

    def valu(text):
        prog.append(("valu", text, [], [], None))

    def lds(text, tag):
        prog.append(("lds", text, [], [], tag))

    def wait(tag):
        prog.append(("wait", "", [], [], tag))

    def convert_half(write_addr, off):
        # 8 codes (two dwords) -> one 16-byte BF16 chunk, written in halves
        for d in (0, 1):
            for hi in (0, 1):
                sel = " op_sel:[1,0,0]" if hi else ""
                valu(f"v_cvt_scalef32_pk_bf16_fp8 v{O + hi}, v{C + d}, v{SC}{sel}")
            lds(f"ds_write_b64 {write_addr}, v[{O}:{O + 1}] offset:{off + 8 * d}", ("DQW",))

    valu(f"v_mbcnt_lo_u32_b32 v{TT}, -1, 0")
    valu(f"v_mbcnt_hi_u32_b32 v{TT}, -1, v{TT}")
    valu(f"v_and_b32 v{HH}, 32, v{TT}")                 # 32 h
    valu(f"v_and_b32 v{TT}, 31, v{TT}")
    valu(f"v_lshlrev_b32 v{TT}, 4, v{TT}")              # 16 t
    for k in range(4):
        # code chunk c = 2 w + h + 8 k, block w + 4 k
        tag = ("DQM", k)
        valu(f"v_add_u32 v{T}, %[dqb], v{TT}")
        lds(f"ds_read_u8 v{SC}, v{T} offset:{512 * 36 + 4 * k}", tag + ("s",))
        for q in (0, 1):
            valu(f"v_lshl_add_u32 v{T}, v{HH}, 4, v{TT}")               # 16 t + 512 h
            valu(f"v_add_u32 v{T}, %[dqa], v{T}")
            lds(f"ds_read_b64 v[{C}:{C + 1}], v{T} offset:{4096 * k + 8 * q}", tag + ("c", q))
            if q == 0:
                wait(tag + ("s",))
                valu(f"v_lshlrev_b32 v{SC}, 23, v{SC}")
            wait(tag + ("c", q))
            # BF16 chunk 4 w + 2 h + 16 k + q; its index & 3 is 2 h + q
            valu(f"v_lshlrev_b32 v{T2}, 2, v{HH}")                     # 128 h
            valu(f"v_xor_b32 v{T2}, v{T2}, v{TT}")
            if q:
                valu(f"v_xor_b32 v{T2}, 64, v{T2}")
            valu(f"v_lshl_add_u32 v{T2}, v{HH}, 5, v{T2}")            # + 1024 * 2 h
            valu(f"v_add_u32 v{T2}, %[dqc], v{T2}")
            convert_half(f"v{T2}", 8192 * k + 512 * q)
    # half h of code chunk 32 + w (block 16 + w / 2): BF16 chunk 64 + 2 w + h
    tag = ("DQM", 4)
    valu(f"v_add_u32 v{T}, %[dqe], v{TT}")
    lds(f"ds_read_u8 v{SC}, v{T} offset:{512 * 37}", tag + ("s",))
    valu(f"v_lshrrev_b32 v{T}, 2, v{HH}")                           # 8 h
    valu(f"v_add3_u32 v{T}, %[dqd], v{T}, v{TT}")
    lds(f"ds_read_b64 v[{C}:{C + 1}], v{T} offset:16384", tag + ("c",))
    wait(tag + ("s",))
    valu(f"v_lshlrev_b32 v{SC}, 23, v{SC}")
    wait(tag + ("c",))
    valu(f"v_lshlrev_b32 v{T2}, 1, v{HH}")                          # 64 h
    valu(f"v_xor_b32 v{T2}, v{T2}, v{TT}")
    valu(f"v_xor_b32 v{T2}, %[dqg], v{T2}")
    valu(f"v_lshl_add_u32 v{T2}, v{HH}, 4, v{T2}")                  # + 512 h
    valu(f"v_add_u32 v{T2}, %[dqf], v{T2}")
    convert_half(f"v{T2}", 32768)
    return prog


def statement(fp8: bool, qk: bool, pv: bool, sm: bool = False, n_dma: int = 0,
              tail_chains: int = 2, dq: bool = False, dqmx: bool = False,
              one_chain: bool = False, lead_pv: int = 0, gate=None, subst=None,
              gld_fmt=None, tail: bool = True, keep_m0: bool = False, addr=None,
              early_prep: bool = False):
    """One statement (see the module docstring).  The keyword arguments after
    dqmx serve the FP8 unit loop (fp8_loop): one_chain puts every QK MFMA
    on the chain %[s]; lead_pv schedules that many PV MFMAs before the first
    QK MFMA; gate = (pos, lines) emits `lines` (the loop's barrier and DMA
    set-up) before the MFMA at position pos and holds every K read back
    until then; subst maps operand texts to literal registers; gld_fmt
    formats the DMA rows in place of the MLA_GLD macro; tail False leaves
    out the closing waits for the MFMA results; keep_m0 leaves M0 to the
    caller; addr maps the LDS address operands (%[kb], %[va], %[vb], %[sc])
    to (register, byte delta) so that a buffer's reads become constant
    offsets from a base register; early_prep waits for the next MFMA's
    operand read and widens or duplicates it in the middle of the current
    slot, so that the MFMA needs no s_nop."""
    reads = {}
    kops, vops = [], []
    if qk:
        mf = "v_mfma_f32_32x32x16_bf16 {acc}, v[{x}:{x3}], %[qKS], {c}"
        if fp8:
            # FP8 MFMAs on the stored codes: per 64-feature block kb, lane
            # half h holds features 64 kb + 16 h + (0..15) in bytes 0..15 and
            # 64 kb + 32 + 16 h + (0..15) in bytes 16..31 (chunks 4 kb + h and
            # 4 kb + 2 + h of its token), against the hi and lo e4m3 terms
            # of Q (%[qhKB], %[qlKB]) with the row's block scale %[qsc].
            mq = ("v_mfma_scale_f32_32x32x64_f8f6f4 {acc}, v[{x}:{x7}], %[qTKB], {c}, "
                  "%[s127], %[qsc] op_sel_hi:[0,0,0]")
            for kb in range(8):
                reads[("K", kb)] = Read(("K", kb), "KR", [
                    f"ds_read_b128 v[{{r}}:{{r3}}], %[kb] offset:{2048 * kb}",
                    f"ds_read_b128 v[{{r4}}:{{r7}}], %[kb] offset:{2048 * kb + 1024}"])
                for term in ("h", "l"):
                    kops.append(Op("K", mq.replace("T", term).replace("KB", str(kb)), ("K", kb)))
            # The RoPE features (512..575) stay on BF16 MFMAs, exact for any
            # magnitude: read a = 16, 17 fetches chunk 2 a + hk (16 codes,
            # features 16 (2 a + hk) + 0..15), widened in its own slot;
            # k-step 2 a + h uses the BF16 features 8 h .. 8 h + 7 of it
            # against %[qr(2 a + h)].
            for a in (16, 17):
                reads[("K", a)] = Read(("K", a), "KR", [
                    f"ds_read_b128 v[{{r4}}:{{r7}}], %[kb] offset:{1024 * a}"], widen_inplace=True)
                for h in (0, 1):
                    ks = 2 * a + h
                    kops.append(Op("K", mf.replace("%[qKS]", f"%[qr{ks - 32}]"), ("K", a),
                                   xoff=4 * h))
        else:
            for ks in range(36):
                base = "%[ke]" if ks % 2 == 0 else "%[ko]"
                reads[("K", ks)] = Read(("K", ks), "KR",
                                        [f"ds_read_b128 v[{{r}}:{{r3}}], {base} offset:{1024 * ks}"])
                kops.append(Op("K", mf.replace("KS", str(ks)), ("K", ks)))
    if pv:
        if fp8:
            # One FP8 MFMA per feature block: K = 64 = the tile's 32 tokens
            # twice, P_hi against the first copy of V^T and P_lo against the
            # second (bytes 0..15 / 16..31 of every lane).
            for db in fp8_v_order():
                mfma = (f"v_mfma_scale_f32_32x32x64_f8f6f4 %[a{db}], v[{{x}}:{{x7}}], %[pp], "
                        f"%[a{db}], %[s127], %[pscv] op_sel_hi:[0,0,0]")
                # V^T of the 32 tokens is read once (r0..r3) and copied to
                # r4..r7 by VALU, which halves the LDS traffic of P.V.
                reads[("V", db)] = Read(("V", db), "VR", [
                    f"ds_read_b64_tr_b8 v[{{r}}:{{r1}}], %[va] offset:{1024 * db}",
                    f"ds_read_b64_tr_b8 v[{{r2}}:{{r3}}], %[vb] offset:{1024 * db}"],
                    dup_half=True)
                vops.append(Op("V", mfma, ("V", db), acc=f"a{db}"))
        for j, (db, e) in enumerate(v_order() if not fp8 else []):
            mfma = f"v_mfma_f32_32x32x16_bf16 %[a{db}], v[{{x}}:{{x3}}], %[p{e}], %[a{db}]"
            if True:
                off = 2048 * db + 256 * e
                reads[("V", j)] = Read(("V", j), "VR", [
                    f"ds_read_b64_tr_b16 v[{{r}}:{{r1}}], %[va] offset:{off}",
                    f"ds_read_b64_tr_b16 v[{{r2}}:{{r3}}], %[vb] offset:{off}"])
                vops.append(Op("V", mfma, ("V", j), acc=f"a{db}"))
    # S chains: QK-only statements alternate two chains; with PV one chain
    # while PV MFMAs separate its steps, and two for the tail.
    for i, op in enumerate(kops):
        if one_chain:
            op.acc = "s"
        elif not pv:
            op.acc = "s" if i % 2 == 0 else "s1"
        else:
            tail = i - len(vops)
            op.acc = "s1" if tail_chains == 2 and tail >= 0 and tail % 2 == 1 else "s"
    # Spread the PV MFMAs evenly between the QK MFMAs (one for one when the
    # counts match), so the dependent S chain is broken up along the whole
    # statement.
    ops = list(vops[:lead_pv])
    vops = vops[lead_pv:]
    j = 0
    for i, kop in enumerate(kops):
        ops.append(kop)
        while j < len(vops) and (j + 1) * len(kops) <= (i + 1) * len(vops) + len(kops) // 2:
            ops.append(vops[j])
            j += 1
    ops.extend(vops[j:])
    n = len(ops)
    for p, op in enumerate(ops):
        rd = reads[op.read]
        rd.users.append(p)
        rd.need = p if rd.need is None else min(rd.need, p)

    dma_at = {}
    for k in range(n_dma):
        dma_at.setdefault((2 * k + 1) * n // (2 * n_dma), []).append(k)

    rings = {}
    if qk:
        rings["KR"] = (2, 8) if fp8 else (5, 4)
    if pv:
        rings["VR"] = (2, 8) if fp8 else ((6, 4) if qk else (4, 4))
    if sm:
        rings["SK"] = (1, 4)
        rings["ST"] = (1, 4)
    if dq or dqmx:
        rings["DQ"] = (1, 9)
    st = Stream(rings)
    st.emit("s_nop 2")  # operands may have just been written by VALU instructions
    if n_dma and not keep_m0:
        st.emit("s_mov_b32 %[m0s], m0")  # M0 is handed back unchanged
    gate_open = [gate is None]

    smp = sm_program(fp8, st.base["SK"], st.base["ST"]) if sm else []
    if dq:
        smp = smp + dq_program(st.base["DQ"])
    if dqmx:
        smp = smp + dq_program_mx(st.base["DQ"])
    sm_next = [0]

    queue = {}
    for rid, rd in sorted(reads.items(), key=lambda kv: kv[1].need):
        queue.setdefault(rd.ring, []).append(rid)
    slot_of = {rid: k for q in queue.values() for k, rid in enumerate(q)}
    nxt = {ring: 0 for ring in queue}
    issued, freed = set(), set()
    state = {"pos": -1}  # last issued MFMA

    def slot_free(ring):
        if ring == "KR" and not gate_open[0]:
            return False
        q, k = queue[ring], nxt[ring]
        size = rings[ring][0]
        return k < len(q) and (k < size or q[k - size] in freed)

    def budget_ok(ring):
        return st.outstanding() + len(reads[queue[ring][nxt[ring]]].instrs) <= 13

    def issue(ring):
        rid = queue[ring][nxt[ring]]
        nxt[ring] += 1
        r = st.reg(ring, slot_of[rid])
        for tmpl in reads[rid].instrs:
            st.lds(tmpl.format(r=r, r1=r + 1, r2=r + 2, r3=r + 3, r4=r + 4, r5=r + 5,
                               r6=r + 6, r7=r + 7), rid)
        issued.add(rid)

    def fill():
        while True:
            cands = [g for g in queue if slot_free(g) and budget_ok(g)]
            if not cands:
                return
            cands.sort(key=lambda g: reads[queue[g][nxt[g]]].need)
            issue(cands[0])

    widened_inplace = set()

    def ensure(rid):
        ring = reads[rid].ring
        while rid not in issued:
            assert slot_free(ring), f"{rid}: ring {ring} has no free slot"
            if not budget_ok(ring):
                st.wait_index(st.done + 1)  # retire the oldest LDS op
                continue
            issue(ring)
        st.wait(rid)
        if reads[rid].dup_half and rid not in widened_inplace:
            r = st.reg(ring, slot_of[rid])
            st.emit(f"v_mov_b64 v[{r + 4}:{r + 5}], v[{r}:{r + 1}]")
            st.emit(f"v_mov_b64 v[{r + 6}:{r + 7}], v[{r + 2}:{r + 3}]")
            st.last_valu[r] = len(st.lines)
            widened_inplace.add(rid)
        if reads[rid].widen_inplace and rid not in widened_inplace:
            # codes in r4..r7 -> BF16 in r0..r7, each source dword read
            # before the pair that overwrites it
            r = st.reg(ring, slot_of[rid])
            for d in range(4):
                src = r + 4 + d
                st.emit(f"v_cvt_scalef32_pk_bf16_fp8 v{r + 2 * d}, v{src}, 1.0")
                st.emit(f"v_cvt_scalef32_pk_bf16_fp8 v{r + 2 * d + 1}, v{src}, 1.0 op_sel:[1,0,0]")
            st.last_valu[r] = len(st.lines)
            st.last_valu[r + 4] = len(st.lines)
            widened_inplace.add(rid)

    def release_direct(rid):
        # A read's ring slot is free once every MFMA that reads it has issued.
        if all(u <= state["pos"] - 1 for u in reads[rid].users):
            freed.add(rid)

    sm_lds_slot = {}

    def sm_emit(count, slot=None):
        """Emit up to `count` softmax instructions (waits do not count).  A
        wait for a softmax LDS read issued less than two MFMA slots ago is
        deferred to a later slot, so the wave does not stall on it."""
        done = 0
        while sm_next[0] < len(smp) and done < count:
            kind, text, rds, wrs, tag = smp[sm_next[0]]
            if kind == "wait":
                if slot is not None and sm_lds_slot.get(tag, -9) > slot - 2:
                    return
                sm_next[0] += 1
                st.wait(tag)
                continue
            sm_next[0] += 1
            # A transcendental result needs one instruction before its reader.
            for r in rds:
                at = st.trans_at.get(r)
                if at is not None and len(st.lines) - at < 1:
                    st.emit("s_nop 0")
            if kind == "lds":
                if st.outstanding() >= 13:
                    st.wait_index(st.done + 1)
                st.lds(text, tag)
                sm_lds_slot[tag] = slot if slot is not None else -9
            elif kind == "block":
                for line in text:
                    st.emit(line)
            else:
                st.emit(text)
            for w in wrs:
                if kind == "trans":
                    st.trans_at[w] = len(st.lines)
                else:
                    st.trans_at.pop(w, None)
            done += 1

    n_sm = sum(1 for p in smp if p[0] != "wait")
    per_slot = math.ceil(n_sm / max(1, n - 2)) if n else n_sm

    started = set()
    fill()
    for i, op in enumerate(ops):
        if gate is not None and i == gate[0]:
            for line in gate[1]:
                st.emit(line)
            gate_open[0] = True
            fill()
        ensure(op.read)
        x = st.reg(reads[op.read].ring, slot_of[op.read]) + op.xoff
        gap = len(st.lines) - st.last_valu[x] if x in st.last_valu else 2
        if gap < 2:
            st.emit(f"s_nop {1 - gap}")
        if op.kind == "K":
            c = f"%[{op.acc}]" if op.acc in started else "0"
            started.add(op.acc)
            st.emit(op.mfma.format(acc=f"%[{op.acc}]", x=x, x3=x + 3, x7=x + 7, c=c))
        else:
            st.emit(op.mfma.format(x=x, x3=x + 3, x7=x + 7))
        state["pos"] = i
        if i >= 1:
            release_direct(ops[i - 1].read)
        for k in dma_at.get(i, []):
            assert gate_open[0], "a DMA row before the gate"
            st.emit("s_mov_b32 m0, %[m0b]" if k == 0 else "s_add_u32 m0, m0, 3968")
            st.emit("s_nop 0")
            st.emit(gld_fmt.format(off=128 * k) if gld_fmt else f"@GLD({128 * k})")
        if i >= 1:
            if early_prep and i + 1 < n:
                nr = reads[ops[i + 1].read]
                half = per_slot // 2
                sm_emit(half, i)
                if (nr.dup_half or nr.widen_inplace) and ops[i + 1].read in issued:
                    ensure(ops[i + 1].read)
                sm_emit(per_slot - half, i)
            else:
                sm_emit(per_slot, i)
        fill()
    sm_emit(len(smp))
    for rid in reads:
        assert rid in issued, f"read {rid} never issued"
    if sm:
        st.emit("s_waitcnt lgkmcnt(0)")
    if n_dma and not keep_m0:
        st.emit("s_mov_b32 m0, %[m0s]")
    if tail:
        if ops:
            # S chains are read by VALU code next; O accumulators may be read by
            # v_accvgpr_read next: wait out the MFMA write latency.
            st.emit("s_nop 7")
            st.emit("s_nop 7")
            st.emit("s_nop 7")
        elif sm:
            st.emit("s_nop 1")  # the last results are packed by VALU just above
    lines = st.lines
    if addr:
        def reloc(m):
            reg, delta = addr[m.group(1)]
            off = int(m.group(2)) + delta
            assert 0 <= off < 65536, off
            return f"{reg} offset:{off}"
        pat_a = re.compile(r"(%\[(?:kb|va|vb|sc)\]) offset:(\d+)")
        lines = [pat_a.sub(reloc, l) for l in lines]
    if subst:
        keys = sorted(subst, key=len, reverse=True)
        pat = re.compile("|".join(re.escape(k) for k in keys))
        lines = [pat.sub(lambda m: subst[m.group(0)], l) for l in lines]
    return lines, st.lowest


# ---------------------------------------------------------------- FP8 unit loop

# Literal registers of MLA_LOOP_FP8_ASM below the statement scratch rings
# (v216..v255).
LOOP_SA, LOOP_SB, LOOP_PB = 168, 184, 200    # score sets A, B; P of the next P.V
LOOP_PSCP, LOOP_PSCC, LOOP_ALPHA = 208, 209, 210
LOOP_KB = (160, 161, 162)   # tiles + K lane offset (+ 3, 6 tile buffers)
LOOP_VB = (163, 164, 165)   # tiles + V^T lane offset (+ 3, 6 tile buffers)
LOOP_SC0 = 166              # scale ring + the lane's scale offset
LOOP_BPA = 167              # byte address of lane ^ 32
LOOP_VOFF, LOOP_SOFF, LOOP_TOK, LOOP_CHOFF, LOOP_DYN = 211, 212, 213, 214, 215
LOOP_VLOW = 160
# s36 it, s37 jlast - (j0 + 32 (it + lead)), s38 table entry of tile it +
# lead, s39 lim_min, s40 mask flag, s41..s44 temporaries, s45 row DMA M0,
# s[46:47] pool row base, s[48:49] scale base, s[50:51] saved EXEC, s52 saved
# M0, s53 ntiles - 1, s54 the rescale's return site, s55 table byte offset of
# the next entry load, s56 its largest value, s57 tiles + 1024 w, s58 ns - 1,
# s59 the row size 576.
LOOP_SGPRS = (36, 59)
FP8_RING = 8             # tile buffers (the unit loop is unrolled by the ring size)
FP8_LEAD = FP8_RING - 2  # tiles the DMA runs ahead
FP8_TILE_BYTES = 36 * 512
LOOP_LEAD_PV = 3         # P.V MFMAs at the head of a step (one before the barrier)


def fp8_loop():
    """The whole tile loop of one FP8 unit (paged tables, a wave with rows, at
    least two tiles) as one statement, from S^T of tile 0 to the last P.V.

    Iteration it (tile it in ring buffer it % 8): the statement of the steady
    state (S^T of tile it+1, the softmax of tile it, O^T += V^T . P^T of tile
    it-1), with the DMA of tile it+lead issued after the workgroup barrier.
    The loop is unrolled by the ring size, so every LDS operand address is a
    constant offset from a base register set up once per unit.  The barrier
    and the DMA set-up come after the first P.V MFMA (P.V needs no barrier:
    V of tile it-1 and P are in place), so the wait overlaps a running MFMA;
    the K reads of tile it+1 are held back until after it and land while the
    next P.V MFMAs run.  The two score sets swap roles from one iteration to
    the next, so that nothing is copied but the 8 registers of P.

    Operands (besides the Q operands, the accumulators and the softmax
    scalars of the other statements): %[tiles], %[scb] LDS bases of the tile
    ring and of the scale ring; %[ke], %[vao], %[scl], %[bpa] the lane parts of
    the K, V^T and scale addresses and the lane ^ 32 address; %[tok],
    %[choff] the lane's DMA token and chunk offset; %[pool_lo/hi],
    %[kvs_lo/hi], %[trow] the pool, the scales and this request's table row;
    %[j0], %[jlast], %[ntiles], %[ns], %[w] the unit's first and last local
    index, its tile count, the pool's slot count and the wave index;
    %[raw0] the table entry of tile lead; %[limmin] the unit's lim_min;
    %[mref], %[lsum], %[limh] (read-write) as in the softmax.
    """
    A, B, PB = LOOP_SA, LOOP_SB, LOOP_PB
    R, lead, T = FP8_RING, FP8_LEAD, FP8_TILE_BYTES

    def kaddr(buf):
        return (f"v{LOOP_KB[buf // 3]}", (buf % 3) * T)

    def vaddr(buf):
        return (f"v{LOOP_VB[buf // 3]}", (buf % 3) * T)

    def addr_static(buf):
        # K of tile it+1, V^T of tile it-1, the scales of tile it.
        kr, kd = kaddr((buf + 1) % R)
        vr, vd = vaddr((buf - 1) % R)
        return {"%[kb]": (kr, kd), "%[va]": (vr, vd), "%[vb]": (vr, vd + 256),
                "%[sc]": (f"v{LOOP_SC0}", 128 * buf)}

    def subst(cur, nxt):
        d = {f"%[x{i}]": f"v{cur + i}" for i in range(16)}
        d.update({"%[s]": f"v[{nxt}:{nxt + 15}]", "%[pp]": f"v[{PB}:{PB + 7}]",
                  "%[pscv]": f"v{LOOP_PSCP}", "%[psco]": f"v{LOOP_PSCC}",
                  "%[alpha]": f"v{LOOP_ALPHA}", "%[mon]": "s40", "%[m0b]": "s45",
                  "%[bpa]": f"v{LOOP_BPA}"})
        return d

    gld = f"global_load_lds_dwordx4 v{LOOP_VOFF}, s[46:47] offset:{{off}}"

    def mask_flag():
        return ["s_cmp_lt_i32 s39, 31", "s_cselect_b32 s40, 1, 0"]

    def gate(buf):
        # After the barrier: DMA of tile it+lead (a clamped copy of the
        # unit's last token past its end) into buffer it-2, whose last
        # reader (P.V of tile it-2) every wave has passed.  s38, the table
        # entry of tile it+lead, was loaded during the previous statement,
        # whose final lgkmcnt(0) it has passed; the entry of tile it+1+lead
        # is loaded here and waited for by this statement's final lgkmcnt(0).
        bd = (buf - 2) % R
        return [
            f"s_waitcnt vmcnt({5 * (lead - 2)})",             # own share of tile it+1
            "s_barrier",
            "s_max_i32 s41, s38, 0",
            "s_min_i32 s41, s41, s58",                       # raw_c
            "s_load_dword s38, %[trow], s55",                # entry of tile it+1+lead
            "s_add_u32 s55, s55, 0x80",
            "s_min_u32 s55, s55, s56",
            "s_sub_i32 s42, s58, s41",                       # ns - 1 - raw_c
            "s_max_i32 s43, s37, 0",
            "s_min_i32 s43, s43, s42",
            "s_min_i32 s43, s43, 31",                        # lim of the tile
            f"v_min_i32 v{LOOP_VOFF}, s43, v{LOOP_TOK}",      # token of this lane
            f"v_lshlrev_b32 v{LOOP_SOFF}, 2, v{LOOP_VOFF}",
            f"v_mad_u32_u24 v{LOOP_VOFF}, v{LOOP_VOFF}, s59, v{LOOP_CHOFF}",
            "s_mul_i32 s46, s41, 0x240",
            "s_mul_hi_u32 s47, s41, 0x240",
            "s_add_u32 s46, s46, %[pool_lo]",
            "s_addc_u32 s47, s47, %[pool_hi]",               # pool row of raw_c
            "s_lshl_b32 s48, s41, 2",
            "s_lshr_b32 s49, s41, 30",
            "s_add_u32 s48, s48, %[kvs_lo]",
            "s_addc_u32 s49, s49, %[kvs_hi]",                # its scale
            f"s_add_u32 s45, s57, {bd * T}",                 # M0 of the row DMA
            # waves 0, 1: row instruction 4; waves 2, 3 (lanes 0..31): the scales
            "s_cmp_lt_u32 %[w], 2",
            "s_cbranch_scc0 61f",
            "s_add_u32 m0, s45, 0x3e00",
            "s_nop 0",
            f"global_load_lds_dwordx4 v{LOOP_VOFF}, s[46:47] offset:512",
            "s_branch 62f",
            "61:",
            f"s_add_u32 m0, %[scb], {128 * bd}",
            "s_mov_b64 s[50:51], exec",
            "s_mov_b32 exec_hi, 0",
            "s_nop 0",
            f"global_load_lds_dword v{LOOP_SOFF}, s[48:49] offset:0",
            "s_mov_b64 exec, s[50:51]",
            "62:",
        ]

    # O *= alpha when some row's running max moved: one out-of-line block
    # (label 80) shared by every site; s54 says where to return.
    sites = []

    def rescale():
        k = len(sites)
        sites.append(70 + k)
        return [f"v_cmp_neq_f32 vcc, 1.0, v{LOOP_ALPHA}", f"s_mov_b32 s54, {k}",
                "s_cbranch_vccnz 80f", f"{70 + k}:"]

    def take_p(cur):
        return [f"v_mov_b64 v[{PB + 2 * k}:{PB + 2 * k + 1}], v[{cur + 2 * k}:{cur + 2 * k + 1}]"
                for k in range(4)] + [f"v_mov_b32 v{LOOP_PSCP}, v{LOOP_PSCC}"]

    def advance():
        # it += 1; the mask limits and the DMA's tile limit move by one tile.
        return ["s_add_u32 s36, s36, 1", "v_add_u32 %[limh], -32, %[limh]",
                "s_add_i32 s39, s39, -32", "s_add_i32 s37, s37, -32"]

    def step(cur, nxt, buf, first):
        body, _ = statement(fp8=True, qk=True, pv=not first, sm=True, n_dma=4, tail_chains=1,
                            one_chain=True, lead_pv=0 if first else LOOP_LEAD_PV,
                            gate=(0 if first else 1, gate(buf)), subst=subst(cur, nxt),
                            gld_fmt=gld, keep_m0=True, tail=False, addr=addr_static(buf),
                            early_prep=True)
        return body

    def exit_to(nxt, buf_next):
        # The next tile (it, in buffer buf_next, scores in set nxt) is the last.
        return [f"s_mov_b32 s44, {buf_next}", "s_cmp_eq_u32 s36, s53",
                f"s_cbranch_scc1 {65 if nxt == A else 66}f"]

    out = ["s_mov_b32 s52, m0", "s_mov_b32 s36, 0", "s_mov_b32 s38, %[raw0]",
           "s_mov_b32 s39, %[limmin]", "s_add_i32 s53, %[ntiles], -1",
           "s_sub_i32 s37, %[jlast], %[j0]", f"s_add_i32 s37, s37, {-32 * lead}",
           "s_lshl_b32 s56, s53, 5", "s_add_u32 s56, s56, %[j0]", "s_lshl_b32 s56, s56, 2",
           f"s_add_u32 s55, %[j0], {32 * (lead + 1)}", "s_lshl_b32 s55, s55, 2",
           "s_min_u32 s55, s55, s56",
           "s_lshl_b32 s57, %[w], 10", "s_add_u32 s57, s57, %[tiles]",
           "s_add_i32 s58, %[ns], -1", "s_movk_i32 s59, 0x240",
           f"v_add_u32 v{LOOP_KB[0]}, %[tiles], %[ke]",
           f"v_add_u32 v{LOOP_KB[1]}, {3 * T}, v{LOOP_KB[0]}",
           f"v_add_u32 v{LOOP_KB[2]}, {6 * T}, v{LOOP_KB[0]}",
           f"v_add_u32 v{LOOP_VB[0]}, %[tiles], %[vao]",
           f"v_add_u32 v{LOOP_VB[1]}, {3 * T}, v{LOOP_VB[0]}",
           f"v_add_u32 v{LOOP_VB[2]}, {6 * T}, v{LOOP_VB[0]}",
           f"v_add_u32 v{LOOP_SC0}, %[scb], %[scl]",
           f"v_mov_b32 v{LOOP_BPA}, %[bpa]", f"v_mov_b32 v{LOOP_TOK}, %[tok]",
           f"v_mov_b32 v{LOOP_CHOFF}, %[choff]"]
    # S^T of tile 0 (buffer 0) into A (two chains, A and B, summed).
    qk0, _ = statement(fp8=True, qk=True, pv=False,
                       subst={"%[s]": f"v[{A}:{A + 15}]", "%[s1]": f"v[{B}:{B + 15}]"},
                       addr={"%[kb]": kaddr(0)})
    out += qk0
    out += [f"v_add_f32 v{A + i}, v{A + i}, v{B + i}" for i in range(16)]
    # it = 0: S^T of tile 1 into B, softmax of tile 0 (no P.V yet).
    out += mask_flag() + step(A, B, 0, True) + take_p(A) + advance() + exit_to(B, 1)
    # Steady state, unrolled by the ring size: iteration it sits at position
    # it % 8, its buffer; odd it: softmax on B, S^T into A.
    out += ["63:"]
    for k in range(R):
        buf = (1 + k) % R
        cur, nxt = (B, A) if buf % 2 else (A, B)
        out += mask_flag() + step(cur, nxt, buf, False) + rescale() + take_p(cur) + advance()
        if k < R - 1:
            out += exit_to(nxt, (buf + 1) % R)
        else:
            out += [f"s_mov_b32 s44, {(buf + 1) % R}", "s_cmp_eq_u32 s36, s53",
                    f"s_cbranch_scc0 63b", f"s_branch {65 if nxt == A else 66}f"]

    def last(cur):
        # The last tile, in buffer s44 (scores in set cur): its softmax with
        # P.V of the tile before, then its own P.V; addresses from s44.
        dyn = {"%[va]": (f"v{LOOP_DYN}", 0), "%[vb]": (f"v{LOOP_DYN}", 256),
               "%[sc]": (f"v{LOOP_TOK}", 0)}
        smpv, _ = statement(fp8=True, qk=False, pv=True, sm=True, subst=subst(cur, cur),
                            addr=dyn)
        pv, _ = statement(fp8=True, qk=False, pv=True, subst=subst(cur, cur), addr=dyn)
        pre = ["s_add_u32 s41, s44, 7", "s_and_b32 s41, s41, 7",
               f"s_mul_i32 s41, s41, {T}",
               f"v_add_u32 v{LOOP_DYN}, s41, v{LOOP_VB[0]}",      # V^T of tile it-1
               "s_lshl_b32 s42, s44, 7",
               f"v_add_u32 v{LOOP_TOK}, s42, v{LOOP_SC0}"]       # scales of tile it
        own = [f"s_mul_i32 s41, s44, {T}",
               f"v_add_u32 v{LOOP_DYN}, s41, v{LOOP_VB[0]}"]     # V^T of tile it
        return pre + mask_flag() + smpv + rescale() + take_p(cur) + own + pv

    out += ["65:"] + last(A) + ["s_branch 67f"]
    out += ["66:"] + last(B)
    out += ["67:", "s_mov_b32 m0, s52", "s_branch 69f"]
    lines, _ = rescale_statement()
    out += ["80:"] + [l.replace("%[al]", f"v{LOOP_ALPHA}") for l in lines]
    for k, lab in enumerate(sites):
        out += [f"s_cmp_eq_u32 s54, {k}", f"s_cbranch_scc1 {lab}b"]
    out += ["69:"]
    return out


def rescale_statement():
    """O *= alpha: every accumulator register (a0..a255, pinned by the
    caller's operand constraints) through VGPR temporaries, eight in flight,
    so that each value is two or more instructions old before it is read."""
    tmp = list(range(SCRATCH_HI - 7, SCRATCH_HI + 1))
    lines = ["s_nop 7", "s_nop 7", "s_nop 7"]  # accumulators may just have been written by MFMAs
    for base in range(0, 256, 8):
        for k in range(8):
            lines.append(f"v_accvgpr_read_b32 v{tmp[k]}, a{base + k}")
        for k in range(8):
            lines.append(f"v_mul_f32 v{tmp[k]}, %[al], v{tmp[k]}")
        for k in range(8):
            lines.append(f"v_accvgpr_write_b32 a{base + k}, v{tmp[k]}")
    lines.append("s_nop 2")  # accumulators written by VALU, read by MFMAs next
    return lines, tmp[0]


def emit_macro(name: str, lines: list[str]) -> str:
    parts = []
    for l in lines:
        if l.startswith("@GLD("):
            parts.append(f"    MLA_GLD({l[5:-1]})\n")
        else:
            parts.append(f'    "{l}\\n\\t"\n')
    body = "".join(parts)
    return f"#define {name} \\\n" + body.rstrip("\n").replace("\n", " \\\n") + "\n"


STATEMENTS = (
    ("MLA_QK_BF16_ASM", dict(fp8=False, qk=True, pv=False)),
    ("MLA_FUSED_BF16_ASM", dict(fp8=False, qk=True, pv=True, n_dma=9)),
    ("MLA_PV_BF16_ASM", dict(fp8=False, qk=False, pv=True)),
    ("MLA_QK_FP8_ASM", dict(fp8=True, qk=True, pv=False)),
    ("MLA_QKSM_FP8_ASM", dict(fp8=True, qk=True, pv=False, sm=True, n_dma=4)),
    ("MLA_STEP_FP8_ASM", dict(fp8=True, qk=True, pv=True, sm=True, n_dma=4, tail_chains=1)),
    ("MLA_SMPV_FP8_ASM", dict(fp8=True, qk=False, pv=True, sm=True)),
    ("MLA_SM_FP8_ASM", dict(fp8=True, qk=False, pv=False, sm=True)),
    ("MLA_PV_FP8_ASM", dict(fp8=True, qk=False, pv=True)),
    # FP4 pools: the BF16 tiles are dequantized in LDS, and the FP4 DMA is
    # issued outside the statement; the steady state dequantizes the tile
    # after next inside the statement.
    ("MLA_FUSED_BF16_DQ_ASM", dict(fp8=False, qk=True, pv=True, dq=True)),
    # The dequantization alone: the share of a wave with no rows to compute.
    ("MLA_DQ_FP4_ASM", dict(fp8=False, qk=False, pv=False, dq=True)),
    # The same for a raw MXFP8 tile.
    ("MLA_FUSED_BF16_DQMX_ASM", dict(fp8=False, qk=True, pv=True, dqmx=True)),
    ("MLA_DQ_MX_ASM", dict(fp8=False, qk=False, pv=False, dqmx=True)),
)


def generate() -> str:
    """The text of tile_asm.inc."""
    out = ["// Generated by gen_tile_asm.py -- do not edit.\n"]
    lines, low = rescale_statement()
    out.append(emit_macro("MLA_RESCALE_ASM", lines))
    regs = ", ".join(f'"v{r}"' for r in range(low, SCRATCH_HI + 1))
    out.append(f"// Scratch registers of MLA_RESCALE_ASM.\n#define MLA_RESCALE_CLOBBERS {regs}\n")
    for name, kw in STATEMENTS:
        lines, low = statement(**kw)
        out.append(emit_macro(name, lines))
        regs = ", ".join(f'"v{r}"' for r in range(low, SCRATCH_HI + 1))
        out.append(f"// Scratch registers of {name}.\n#define {name[:-4]}_CLOBBERS {regs}, \"memory\"\n")
    out.append(emit_macro("MLA_LOOP_FP8_ASM", fp8_loop()))
    regs = ", ".join(f'"v{r}"' for r in range(LOOP_VLOW, SCRATCH_HI + 1))
    sregs = ", ".join(f'"s{r}"' for r in range(LOOP_SGPRS[0], LOOP_SGPRS[1] + 1))
    out.append("// Scratch registers of MLA_LOOP_FP8_ASM.\n#define MLA_LOOP_FP8_CLOBBERS "
               f"{regs}, {sregs}, \"vcc\", \"scc\", \"memory\"\n")
    return "\n".join(out)


def main() -> None:
    here = os.path.dirname(os.path.abspath(__file__))
    with open(os.path.join(here, "tile_asm.inc"), "w") as f:
        f.write(generate())


if __name__ == "__main__":
    main()
