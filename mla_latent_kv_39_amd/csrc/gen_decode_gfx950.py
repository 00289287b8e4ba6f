#!/usr/bin/env python3
"""Emit the gfx950 assembly of the bf16 split-KV MLA decode kernel.

The kernel is written here as a program that prints GCN assembly, so that the
register file can be laid out by hand: one wave per SIMD holds its 32 heads of
Q (144 VGPRs) and its 32 x 512 fp32 output accumulator (all 256 AGPRs) for a
whole sequence segment, which a compiler's register allocator does not manage
without spilling.  Everything else (page walk, tile ring, softmax, epilogue)
is spelled out below with the same structure as the description in
include/mla.h:

  * work partition: units of 64 rows (one cache page), sequence after
    sequence; partition p of P (a power of two) owns units
    [(pU) >> log2 P, ((p+1)U) >> log2 P);
  * tile ring: two LDS slots of one page each (72 KB), filled one unit ahead
    with direct-to-LDS loads; chunk-column-major layout (chunk k of the 64
    rows at k*1024, row r at slot r ^ 12(k&1), so that both the 16-row score
    reads and the 4-row x 2-chunk transposed reads hit distinct banks);
  * per 32-row sub-step: scores S^T = C Q^T (72 MFMA 16x16x32 bf16),
    softmax against a per-segment reference m_ref (first max + 30, log2
    units), output O += P C (64 MFMAs, B operand read with ds_read_b64_tr_b16);
  * a max that passes m_ref + 64 raises the reference and restarts the
    segment (LDS flag, all waves together).

Score/softmax/output follow DeepSeek-V3 architecture notes (deepseek.csdn.net)
§2.1.1-§2.1.3: one shared latent row per token serves as key (with the
decoupled RoPE part) and, its first 512 values, as value; scores are scaled by
1/sqrt(d_h + d_h^R).

Usage: gen_decode_gfx950.py OUT.s
"""
from __future__ import annotations

import sys

KNAME = "mla_decode_bf16_gfx950"
SLOT_BYTES = 64 * 1152          # one page of bf16 rows
FLAG_ADDR = 2 * SLOT_BYTES      # restart flag (LDS)
LDS_BYTES = FLAG_ADDR + 16
NEG_INF = "0xff800000"
LN2 = "0x3f317218"

# ---------------------------------------------------------------- registers
# VGPRs
V_TID, V_LANE, V_G, V_R16, V_QKOFF, V_PVOFF, V_ROWE, V_ROWO = 0, 1, 2, 3, 4, 5, 6, 7
V_MREF = (8, 9)
V_LRUN = (10, 11)
V_T = 12                 # v12..v15 temporaries
V_S = 16                 # S[tb][h] at 16 + (2*tb + h)*4, 16 regs
V_A = 32                 # QK A-operand ring: NA buffers of 4
NA = 6
V_B = 56                 # PV B-operand ring: NB buffers of 4
NB = 6
V_P = 80                 # P fragments: P[h] at 80 + 4h
V_QK, V_QK2, V_PV = 88, 89, 90   # per-unit operand bases (set at the top of every unit)
V_X = 91                 # v91..v107 temporaries of the softmax and the epilogue
V_X_END = 108
V_G4, V_FLAG, V_NEGINF = 109, 110, 111   # set once in the prologue
V_Q = 112                # Q[ks][h] at 112 + (2*ks + h)*4, 144 regs
PERSISTENT = {V_LANE, V_G, V_R16, V_QKOFF, V_PVOFF, *V_MREF, *V_LRUN, V_G4, V_FLAG, V_NEGINF}


def temps(*regs):
    """Check that scratch registers stay inside the scratch range."""
    for r in regs:
        assert V_X <= r < V_X_END and r not in PERSISTENT, f"v{r} is not a scratch register"
    return regs
# AGPRs: O[cb][h] at (2*cb + h)*4

# SGPRs (s0:1 kernarg, s2 workgroup id)
S_QA, S_QR, S_ROWS, S_TABLE, S_LENS, S_POUT, S_PLSE, S_OUT = 4, 6, 8, 10, 12, 14, 16, 18
S_LSE, S_SCALE, S_MAXB, S_BATCH, S_NPART, S_SQ, S_HB = 20, 22, 23, 24, 25, 26, 27
S_NHB, S_LOG2P = 28, 29
S_WAVE, S_PART, S_HBLK, S_U, S_UA, S_UB, S_STOK, S_HEAD0 = 30, 31, 32, 33, 34, 35, 36, 37
S_LSEQ, S_LPRE, S_LUNITS, S_LLEN = 38, 39, 40, 41
S_CSEQ, S_CPRE, S_CUNITS, S_CLEN, S_NVIS = 42, 43, 44, 45, 46
S_UCUR, S_SEGEND, S_ROW0, S_SLOT = 47, 48, 49, 50
S_PAGE = 52              # s52:53
S_QBASE, S_RBASE = 54, 56  # s54:55, s56:57
S_EXEC = 58              # s58:59
S_TMP = 60               # s60..s79 scratch
S_MAX = 96


def vreg(i):
    return f"v{i}"


def vr(i, n):
    return f"v[{i}:{i + n - 1}]"


def ar(i, n):
    return f"a[{i}:{i + n - 1}]"


def s(i):
    return f"s{i}"


def sp(i):
    return f"s[{i}:{i + 1}]"


class Asm:
    def __init__(self):
        self.lines = []
        self.nlabel = 0

    def __call__(self, *lines):
        for line in lines:
            self.lines.append("\t" + line)

    def label(self, name):
        self.lines.append(f"{name}:")

    def new_label(self, stem):
        self.nlabel += 1
        return f".L{stem}_{self.nlabel}"

    def comment(self, text):
        self.lines.append(f"\t; {text}")

    def text(self):
        return "\n".join(self.lines) + "\n"


def s_waitcnt_vm(n):
    return f"s_waitcnt vmcnt({n})"


def s_waitcnt_lgkm(n):
    return f"s_waitcnt lgkmcnt({n})"


# --------------------------------------------------------------- helpers
def load_len(a, dst, idx):
    """dst = seq_lens[idx] (scalar load)."""
    a(f"s_lshl_b32 s{S_TMP + 18}, {s(idx)}, 2",
      f"s_load_dword {s(dst)}, {sp(S_LENS)}, s{S_TMP + 18}",
      s_waitcnt_lgkm(0))


def units_of(a, dst, length):
    """dst = max(1, (len + 63) >> 6)."""
    a(f"s_add_i32 {s(dst)}, {s(length)}, 63",
      f"s_ashr_i32 {s(dst)}, {s(dst)}, 6",
      f"s_max_i32 {s(dst)}, {s(dst)}, 1")


def wave_incl_scan(a, dst, src):
    """Inclusive prefix sum of src over the 64 lanes into dst (DPP)."""
    a(f"v_add_u32_dpp {vreg(dst)}, {vreg(src)}, {vreg(src)} row_shr:1 row_mask:0xf bank_mask:0xf bound_ctrl:1",
      "s_nop 1",
      f"v_add_u32_dpp {vreg(dst)}, {vreg(src)}, {vreg(dst)} row_shr:2 row_mask:0xf bank_mask:0xf bound_ctrl:1",
      "s_nop 1",
      f"v_add_u32_dpp {vreg(dst)}, {vreg(src)}, {vreg(dst)} row_shr:3 row_mask:0xf bank_mask:0xf bound_ctrl:1",
      "s_nop 1",
      f"v_add_u32_dpp {vreg(dst)}, {vreg(dst)}, {vreg(dst)} row_shr:4 row_mask:0xf bank_mask:0xe",
      "s_nop 1",
      f"v_add_u32_dpp {vreg(dst)}, {vreg(dst)}, {vreg(dst)} row_shr:8 row_mask:0xf bank_mask:0xc",
      "s_nop 1",
      f"v_add_u32_dpp {vreg(dst)}, {vreg(dst)}, {vreg(dst)} row_bcast:15 row_mask:0xa bank_mask:0xf",
      "s_nop 1",
      f"v_add_u32_dpp {vreg(dst)}, {vreg(dst)}, {vreg(dst)} row_bcast:31 row_mask:0xc bank_mask:0xf",
      "s_nop 1")


def xor_reduce(a, v, op, t0, t1):
    """v <- op(v, v^16) then op(v, v^32) with permlane swaps (gfx950)."""
    for swap in ("v_permlane16_swap_b32", "v_permlane32_swap_b32"):
        a(f"v_mov_b32 {vreg(t0)}, {vreg(v)}",
          f"v_mov_b32 {vreg(t1)}, {vreg(v)}",
          "s_nop 1",
          f"{swap} {vreg(t0)}, {vreg(t1)}",
          "s_nop 1",
          f"{op} {vreg(v)}, {vreg(t0)}, {vreg(t1)}")


def seq_units_pass(a, find_first):
    """Walk seq_lens in chunks of 64 lanes.  Without find_first: S_U = total
    units.  With find_first: S_CSEQ/S_CPRE = the sequence holding unit S_UA and
    its first unit."""
    t = V_T
    loop, found = a.new_label("seqpass"), a.new_label("seqfound")
    a(f"s_mov_b32 s{S_TMP}, 0",          # b0
      f"s_mov_b32 s{S_TMP + 1}, 0")      # carry
    a.label(loop)
    a(f"v_add_u32 {vreg(t)}, s{S_TMP}, {vreg(V_LANE)}",
      f"v_mov_b32 {vreg(t + 1)}, 0",
      f"v_cmp_gt_i32 vcc, {s(S_BATCH)}, {vreg(t)}",
      f"s_and_saveexec_b64 {sp(S_EXEC)}, vcc",
      f"v_lshlrev_b32 {vreg(t + 2)}, 2, {vreg(t)}",
      f"global_load_dword {vreg(t + 3)}, {vreg(t + 2)}, {sp(S_LENS)}",
      s_waitcnt_vm(0),
      f"v_add_u32 {vreg(t + 3)}, 63, {vreg(t + 3)}",
      f"v_ashrrev_i32 {vreg(t + 3)}, 6, {vreg(t + 3)}",
      f"v_max_i32 {vreg(t + 1)}, 1, {vreg(t + 3)}",
      f"s_mov_b64 exec, {sp(S_EXEC)}",
      "s_nop 1")
    wave_incl_scan(a, t + 2, t + 1)
    a(f"v_add_u32 {vreg(t + 2)}, s{S_TMP + 1}, {vreg(t + 2)}", "s_nop 1")
    if find_first:
        a(f"v_cmp_lt_u32 vcc, {s(S_UA)}, {vreg(t + 2)}",
          f"s_ff1_i32_b64 s{S_TMP + 2}, vcc",
          f"s_cmp_lt_i32 s{S_TMP + 2}, 0",
          f"s_cbranch_scc0 {found}")
    a(f"v_readlane_b32 s{S_TMP + 1}, {vreg(t + 2)}, 63",
      f"s_add_u32 s{S_TMP}, s{S_TMP}, 64",
      f"s_cmp_lt_u32 s{S_TMP}, {s(S_BATCH)}",
      f"s_cbranch_scc1 {loop}")
    if find_first:
        a(f"s_branch .Lkernel_end")   # cannot happen when ua < U
        a.label(found)
        a(f"s_add_u32 {s(S_CSEQ)}, s{S_TMP}, s{S_TMP + 2}",
          f"v_sub_u32 {vreg(t + 3)}, {vreg(t + 2)}, {vreg(t + 1)}",
          "s_nop 4",
          f"v_readlane_b32 {s(S_CPRE)}, {vreg(t + 3)}, s{S_TMP + 2}")
    else:
        a(f"s_mov_b32 {s(S_U)}, s{S_TMP + 1}")


def issue_unit(a, u_sgpr, slot_sgpr):
    """Direct-to-LDS copy of unit u into the slot: advance the loader cursor,
    find the page, 18 x 16 B per lane (wave w fills chunk columns 18w..18w+17;
    lane L loads row L of even columns and row L ^ 12 of odd ones)."""
    adv, adv_done, haspage, contig, pagedone = (a.new_label(x) for x in
                                                ("adv", "advdone", "haspage", "contig", "pagedone"))
    T = S_TMP
    a.label(adv)
    a(f"s_add_u32 s{T}, {s(S_LPRE)}, {s(S_LUNITS)}",
      f"s_cmp_lt_u32 {s(u_sgpr)}, s{T}",
      f"s_cbranch_scc1 {adv_done}",
      f"s_mov_b32 {s(S_LPRE)}, s{T}",
      f"s_add_u32 {s(S_LSEQ)}, {s(S_LSEQ)}, 1")
    load_len(a, S_LLEN, S_LSEQ)
    units_of(a, S_LUNITS, S_LLEN)
    a(f"s_branch {adv}")
    a.label(adv_done)
    a(f"s_sub_u32 s{T + 1}, {s(u_sgpr)}, {s(S_LPRE)}",        # j
      f"s_lshl_b32 s{T + 2}, s{T + 1}, 6",
      f"s_sub_i32 s{T + 3}, {s(S_LLEN)}, s{T + 2}",           # valid = len - 64 j
      f"s_min_i32 s{T + 3}, s{T + 3}, 64",
      f"s_cmp_gt_i32 s{T + 3}, 0",
      f"s_cbranch_scc1 {haspage}",
      f"s_mov_b64 {sp(S_PAGE)}, {sp(S_ROWS)}",                # nothing visible: page 0 row 0
      f"s_branch {pagedone}")
    a.label(haspage)
    a(f"s_mul_i32 s{T + 4}, {s(S_LSEQ)}, {s(S_MAXB)}",
      f"s_add_u32 s{T + 4}, s{T + 4}, s{T + 1}",
      f"s_cmp_eq_u64 {sp(S_TABLE)}, 0",
      f"s_cbranch_scc1 {contig}",
      f"s_lshl_b32 s{T + 5}, s{T + 4}, 2",
      f"s_load_dword s{T + 4}, {sp(S_TABLE)}, s{T + 5}",
      s_waitcnt_lgkm(0))
    a.label(contig)
    a(f"s_mul_i32 s{T + 5}, s{T + 4}, {SLOT_BYTES}",
      f"s_mul_hi_u32 s{T + 6}, s{T + 4}, {SLOT_BYTES}",
      f"s_add_u32 s{S_PAGE}, {s(S_ROWS)}, s{T + 5}",
      f"s_addc_u32 s{S_PAGE + 1}, s{S_ROWS + 1}, s{T + 6}")
    a.label(pagedone)
    # per-lane source rows: lane (even columns) and lane ^ 12 (odd columns), clamped to row 0
    a(f"v_cmp_gt_i32 vcc, s{T + 3}, {vreg(V_LANE)}",
      f"v_xor_b32 {vreg(V_T)}, 12, {vreg(V_LANE)}",
      "s_nop 1",
      f"v_cndmask_b32 {vreg(V_ROWE)}, 0, {vreg(V_LANE)}, vcc",
      f"v_cmp_gt_i32 vcc, s{T + 3}, {vreg(V_T)}",
      f"v_mul_u32_u24 {vreg(V_ROWE)}, 0x480, {vreg(V_ROWE)}",
      "s_nop 1",
      f"v_cndmask_b32 {vreg(V_ROWO)}, 0, {vreg(V_T)}, vcc",
      f"v_mul_u32_u24 {vreg(V_ROWO)}, 0x480, {vreg(V_ROWO)}",
      f"s_mul_i32 s{T + 4}, {s(slot_sgpr)}, {SLOT_BYTES}",
      f"s_mul_i32 s{T + 5}, {s(S_WAVE)}, {18 * 1024}",
      f"s_add_u32 s{T + 4}, s{T + 4}, s{T + 5}",             # LDS base of this wave's columns
      f"s_mul_i32 s{T + 5}, {s(S_WAVE)}, {18 * 16}")          # global byte offset of column 18w
    for i in range(18):
        src = V_ROWO if (i & 1) else V_ROWE
        tmp = V_T + 1 + (i & 1)
        a(f"s_add_u32 s{T + 6}, s{T + 5}, {16 * i}",
          f"v_add_u32 {vreg(tmp)}, s{T + 6}, {vreg(src)}",
          f"s_add_u32 m0, s{T + 4}, {1024 * i}",
          "s_nop 0",
          f"global_load_lds_dwordx4 {vreg(tmp)}, {sp(S_PAGE)}")


def qk_read(a, i, ss):
    ks, tb = divmod(i, 2)
    buf = V_A + 4 * (i % NA)
    if ks < 16:
        base, off = V_QK, ks * 4096 + ss * 512 + tb * 256
    else:
        base, off = V_QK2, (ks - 16) * 4096 + ss * 512 + tb * 256
    a(f"ds_read_b128 {vr(buf, 4)}, {vreg(base)} offset:{off}")


def pv_read(a, cb, ss):
    buf = V_B + 4 * (cb % NB)
    off = cb * 2048 + ss * 512
    a(f"ds_read_b64_tr_b16 {vr(buf, 2)}, {vreg(V_PV)} offset:{off}",
      f"ds_read_b64_tr_b16 {vr(buf + 2, 2)}, {vreg(V_PV)} offset:{off + 256}")


def substep(a, ss, masked_label_stem):
    """QK, softmax, PV for rows 32ss..32ss+31 of the current unit."""
    NQK = 36
    # ---- scores
    for i in range(min(NA, NQK)):
        qk_read(a, i, ss)
    for i in range(NQK):
        ks, tb = divmod(i, 2)
        ahead = min(NA - 1, NQK - 1 - i)
        a(s_waitcnt_lgkm(ahead))
        buf = V_A + 4 * (i % NA)
        for h in range(2):
            sreg = V_S + (2 * tb + h) * 4
            qreg = V_Q + (2 * ks + h) * 4
            c = "0" if ks == 0 else vr(sreg, 4)
            a(f"v_mfma_f32_16x16x32_bf16 {vr(sreg, 4)}, {vr(buf, 4)}, {vr(qreg, 4)}, {c}")
        if i + NA < NQK:
            qk_read(a, i + NA, ss)
    # prefetch the first output-operand fragments while the softmax runs
    for cb in range(NB):
        pv_read(a, cb, ss)
    a("s_nop 7", "s_nop 7", "s_nop 3")   # MFMA results -> VALU
    # ---- softmax (log2 domain)
    for r in range(16):
        a(f"v_mul_f32 {vreg(V_S + r)}, {s(S_SCALE)}, {vreg(V_S + r)}")
    skip = a.new_label(masked_label_stem)
    T = S_TMP
    a(f"s_add_u32 s{T}, {s(S_ROW0)}, {32 * ss + 32}",
      f"s_cmp_ge_i32 {s(S_NVIS)}, s{T}",
      f"s_cbranch_scc1 {skip}")
    # rows at or past nvis get -inf: pos = row0 + 32ss + 16tb + 4g + i < nvis
    for tb in range(2):
        for i in range(4):
            a(f"s_sub_i32 s{T}, {s(S_NVIS)}, {s(S_ROW0)}",
              f"s_sub_i32 s{T}, s{T}, {32 * ss + 16 * tb + i}",
              f"v_cmp_gt_i32 vcc, s{T}, {vreg(V_G4)}",
              "s_nop 1")
            for h in range(2):
                r = V_S + (2 * tb + h) * 4 + i
                a(f"v_cndmask_b32 {vreg(r)}, {vreg(V_NEGINF)}, {vreg(r)}, vcc")
    a.label(skip)
    flag_skip = a.new_label("noflag")
    a(f"s_mov_b64 s[{T + 2}:{T + 3}], 0")
    for h in range(2):
        regs = [V_S + (2 * tb + h) * 4 + i for tb in range(2) for i in range(4)]
        m, t0, t1, ref = temps(V_X, V_X + 1, V_X + 2, V_X + 3)
        a(f"v_max3_f32 {vreg(m)}, {vreg(regs[0])}, {vreg(regs[1])}, {vreg(regs[2])}",
          f"v_max3_f32 {vreg(m)}, {vreg(m)}, {vreg(regs[3])}, {vreg(regs[4])}",
          f"v_max3_f32 {vreg(m)}, {vreg(m)}, {vreg(regs[5])}, {vreg(regs[6])}",
          f"v_max_f32 {vreg(m)}, {vreg(m)}, {vreg(regs[7])}")
        xor_reduce(a, m, "v_max_f32", t0, t1)
        mref = V_MREF[h]
        # first visible rows of the segment: m_ref = max + 30 (stays -inf while all masked)
        a(f"v_add_f32 {vreg(t0)}, 0x41f00000, {vreg(m)}",        # +30.0
          f"v_cmp_eq_f32 vcc, {NEG_INF}, {vreg(mref)}",
          "s_nop 1",
          f"v_cndmask_b32 {vreg(mref)}, {vreg(mref)}, {vreg(t0)}, vcc",
          # overflow guard: max - m_ref > 64 -> raise m_ref, ask for a restart
          f"v_sub_f32 {vreg(t1)}, {vreg(m)}, {vreg(mref)}",
          f"v_cmp_lt_f32 vcc, 0x42800000, {vreg(t1)}",             # 64.0 < max - m_ref
          "s_nop 1",
          f"v_cndmask_b32 {vreg(mref)}, {vreg(mref)}, {vreg(t0)}, vcc",
          f"s_or_b64 s[{T + 2}:{T + 3}], s[{T + 2}:{T + 3}], vcc",
          # reference used for P: 0 while nothing is visible yet
          f"v_cmp_eq_f32 vcc, {NEG_INF}, {vreg(mref)}",
          "s_nop 1",
          f"v_cndmask_b32 {vreg(ref)}, {vreg(mref)}, 0, vcc")
        for r in regs:
            a(f"v_sub_f32 {vreg(r)}, {vreg(r)}, {vreg(ref)}")
        for r in regs:
            a(f"v_exp_f32 {vreg(r)}, {vreg(r)}")
        a("s_nop 0",
          f"v_add_f32 {vreg(t0)}, {vreg(regs[0])}, {vreg(regs[1])}",
          f"v_add_f32 {vreg(t1)}, {vreg(regs[2])}, {vreg(regs[3])}",
          f"v_add_f32 {vreg(t0)}, {vreg(t0)}, {vreg(regs[4])}",
          f"v_add_f32 {vreg(t1)}, {vreg(t1)}, {vreg(regs[5])}",
          f"v_add_f32 {vreg(t0)}, {vreg(t0)}, {vreg(regs[6])}",
          f"v_add_f32 {vreg(t1)}, {vreg(t1)}, {vreg(regs[7])}",
          f"v_add_f32 {vreg(t0)}, {vreg(t0)}, {vreg(t1)}",
          f"v_add_f32 {vreg(V_LRUN[h])}, {vreg(V_LRUN[h])}, {vreg(t0)}")
        p = V_P + 4 * h
        a(f"v_cvt_pk_bf16_f32 {vreg(p)}, {vreg(regs[0])}, {vreg(regs[1])}",
          f"v_cvt_pk_bf16_f32 {vreg(p + 1)}, {vreg(regs[2])}, {vreg(regs[3])}",
          f"v_cvt_pk_bf16_f32 {vreg(p + 2)}, {vreg(regs[4])}, {vreg(regs[5])}",
          f"v_cvt_pk_bf16_f32 {vreg(p + 3)}, {vreg(regs[6])}, {vreg(regs[7])}")
    a(f"s_cmp_eq_u64 s[{T + 2}:{T + 3}], 0",
      f"s_cbranch_scc1 {flag_skip}",
      f"v_mov_b32 {vreg(V_T)}, 1",
      f"ds_write_b32 {vreg(V_FLAG)}, {vreg(V_T)}")
    a.label(flag_skip)
    a("s_nop 4")   # VALU writes of P -> MFMA reads
    # ---- output: O[h] += P[h] C[:, 16cb .. 16cb+15]
    NPV = 32
    for cb in range(NPV):
        ahead = min(NB - 1, NPV - 1 - cb)
        a(s_waitcnt_lgkm(2 * ahead))
        buf = V_B + 4 * (cb % NB)
        for h in range(2):
            o = (2 * cb + h) * 4
            a(f"v_mfma_f32_16x16x32_bf16 {ar(o, 4)}, {vr(V_P + 4 * h, 4)}, {vr(buf, 4)}, {ar(o, 4)}")
        if cb + NB < NPV:
            pv_read(a, cb + NB, ss)


def zero_o(a):
    for i in range(256):
        a(f"v_accvgpr_write_b32 a{i}, 0")


def epilogue(a):
    """Normalise O by l and store it with lse: the final result for a sequence
    wholly inside this partition, else partial slot 0 (the sequence the
    partition starts in) or 1 (the one it ends in)."""
    T = S_TMP
    whole_no, pslot1, addr_done = a.new_label("notwhole"), a.new_label("pslot1"), a.new_label("addrdone")
    a("s_nop 7", "s_nop 7", "s_nop 3")   # last MFMAs -> accvgpr reads
    # row_base and destination pointers
    a(f"s_cmp_lt_u32 {s(S_CPRE)}, {s(S_UA)}",
      f"s_cbranch_scc1 {whole_no}",
      f"s_add_u32 s{T}, {s(S_CPRE)}, {s(S_CUNITS)}",
      f"s_cmp_gt_u32 s{T}, {s(S_UB)}",
      f"s_cbranch_scc1 {whole_no}",
      # whole: row_base = (c_seq * s_q + s_tok) * 128
      f"s_mul_i32 s{T + 1}, {s(S_CSEQ)}, {s(S_SQ)}",
      f"s_add_u32 s{T + 1}, s{T + 1}, {s(S_STOK)}",
      f"s_lshl_b32 s{T + 1}, s{T + 1}, 7",
      f"s_mov_b64 s[{T + 4}:{T + 5}], {sp(S_OUT)}",
      f"s_mov_b64 s[{T + 6}:{T + 7}], {sp(S_LSE)}",
      f"s_branch {addr_done}")
    a.label(whole_no)
    a(f"s_mov_b32 s{T + 2}, 0",
      f"s_cmp_le_u32 {s(S_CPRE)}, {s(S_UA)}",
      f"s_cbranch_scc1 {pslot1}",
      f"s_mov_b32 s{T + 2}, 1")
    a.label(pslot1)
    a(f"s_lshl_b32 s{T + 1}, {s(S_PART)}, 1",
      f"s_add_u32 s{T + 1}, s{T + 1}, s{T + 2}",
      f"s_mul_i32 s{T + 1}, s{T + 1}, {s(S_SQ)}",
      f"s_add_u32 s{T + 1}, s{T + 1}, {s(S_STOK)}",
      f"s_lshl_b32 s{T + 1}, s{T + 1}, 7",
      f"s_mov_b64 s[{T + 4}:{T + 5}], {sp(S_POUT)}",
      f"s_mov_b64 s[{T + 6}:{T + 7}], {sp(S_PLSE)}")
    a.label(addr_done)
    a(f"s_add_u32 s{T + 1}, s{T + 1}, {s(S_HEAD0)}")   # first row of this wave's heads
    x = V_X
    for h in range(2):
        lt, inv, lse, t0, t1 = temps(x, x + 1, x + 2, x + 3, x + 4)
        a(f"v_mov_b32 {vreg(lt)}, {vreg(V_LRUN[h])}")
        xor_reduce(a, lt, "v_add_f32", t0, t1)
        a(f"v_rcp_f32 {vreg(inv)}, {vreg(lt)}",
          f"v_log_f32 {vreg(lse)}, {vreg(lt)}",
          "s_nop 1",
          f"v_cmp_lt_f32 vcc, 0, {vreg(lt)}",
          f"v_add_f32 {vreg(lse)}, {vreg(V_MREF[h])}, {vreg(lse)}",
          f"v_mul_f32 {vreg(lse)}, {LN2}, {vreg(lse)}",
          "s_nop 1",
          f"v_cndmask_b32 {vreg(inv)}, 0, {vreg(inv)}, vcc",
          f"v_cndmask_b32 {vreg(lse)}, {vreg(V_NEGINF)}, {vreg(lse)}, vcc")
        # lse of head r16 from lanes with g == 0: address (row + 16h + r16) * 4
        a(f"s_add_u32 s{T + 8}, s{T + 1}, {16 * h}",
          f"s_lshl_b32 s{T + 8}, s{T + 8}, 2",
          f"s_add_u32 s{T + 10}, s{T + 6}, s{T + 8}",
          f"s_addc_u32 s{T + 11}, s{T + 7}, 0",
          f"v_cmp_eq_u32 vcc, 0, {vreg(V_G)}",
          f"s_and_saveexec_b64 {sp(S_EXEC)}, vcc",
          f"v_lshlrev_b32 {vreg(t0)}, 2, {vreg(V_R16)}",
          f"global_store_dword {vreg(t0)}, {vreg(lse)}, s[{T + 10}:{T + 11}]",
          f"s_mov_b64 exec, {sp(S_EXEC)}")
        # 1/l of head 4g+i, from lane 4g+i
        invs = list(temps(*[x + 5 + i for i in range(4)]))
        for i in range(4):
            a(f"v_lshlrev_b32 {vreg(t0)}, 2, {vreg(V_G)}",
              f"v_add_u32 {vreg(t0)}, {i}, {vreg(t0)}",
              f"v_lshlrev_b32 {vreg(t0)}, 2, {vreg(t0)}",
              f"ds_bpermute_b32 {vreg(invs[i])}, {vreg(t0)}, {vreg(inv)}")
        a(s_waitcnt_lgkm(0))
        # out rows: base + (row + 16h) * 2048 B; lane offset (4g+i)*2048 + r16*4; column block cb at 64 cb
        a(f"s_add_u32 s{T + 8}, s{T + 1}, {16 * h}",
          f"s_mul_i32 s{T + 9}, s{T + 8}, 2048",
          f"s_mul_hi_u32 s{T + 12}, s{T + 8}, 2048",
          f"s_add_u32 s{T + 10}, s{T + 4}, s{T + 9}",
          f"s_addc_u32 s{T + 11}, s{T + 5}, s{T + 12}")
        offs = list(temps(*[x + 9 + i for i in range(4)]))
        for i in range(4):
            a(f"v_lshlrev_b32 {vreg(t0)}, 2, {vreg(V_G)}",
              f"v_add_u32 {vreg(t0)}, {i}, {vreg(t0)}",
              f"v_lshlrev_b32 {vreg(t0)}, 11, {vreg(t0)}",
              f"v_lshl_add_u32 {vreg(offs[i])}, {vreg(V_R16)}, 2, {vreg(t0)}")
        vv = list(temps(*[x + 13 + i for i in range(4)]))
        for cb in range(32):
            o = (2 * cb + h) * 4
            for i in range(4):
                a(f"v_accvgpr_read_b32 {vreg(vv[i])}, a{o + i}")
            a("s_nop 1")
            for i in range(4):
                a(f"v_mul_f32 {vreg(vv[i])}, {vreg(vv[i])}, {vreg(invs[i])}")
            for i in range(4):
                a(f"global_store_dword {vreg(offs[i])}, {vreg(vv[i])}, s[{T + 10}:{T + 11}] offset:{64 * cb}")


def kernel():
    a = Asm()
    a.lines += [
        '\t.amdgcn_target "amdgcn-amd-amdhsa--gfx950"',
        "\t.amdhsa_code_object_version 6",
        "\t.text",
        f"\t.globl {KNAME}",
        "\t.p2align 8",
        f"\t.type {KNAME},@function",
        f"{KNAME}:",
    ]
    T = S_TMP
    # ------------------------------------------------------------ prologue
    a(f"s_load_dwordx16 s[{S_QA}:{S_QA + 15}], s[0:1], 0x0",
      f"s_load_dwordx8 s[{S_LSE}:{S_LSE + 7}], s[0:1], 0x40",
      f"s_load_dwordx2 s[{S_NHB}:{S_NHB + 1}], s[0:1], 0x60",
      f"v_and_b32 {vreg(V_LANE)}, 63, {vreg(V_TID)}",
      f"v_lshrrev_b32 {vreg(V_G)}, 4, {vreg(V_LANE)}",
      f"v_and_b32 {vreg(V_R16)}, 15, {vreg(V_LANE)}",
      f"v_lshrrev_b32 {vreg(V_T)}, 6, {vreg(V_TID)}",
      "s_nop 1",
      f"v_readfirstlane_b32 {s(S_WAVE)}, {vreg(V_T)}",
      s_waitcnt_lgkm(0))
    # ------------------------------------------------ workgroup -> (partition, head block)
    plain, mapped = a.new_label("mapplain"), a.new_label("mapdone")
    a(f"s_sub_u32 s{T}, {s(S_NHB)}, 1",
      f"s_and_b32 s{T + 1}, {s(S_NPART)}, 7",
      f"s_cmp_eq_u32 s{T + 1}, 0",
      f"s_cbranch_scc0 {plain}",
      # consecutive partitions on one XCD: xcd = wg & 7 owns partitions xcd*P/8 ..
      f"s_lshr_b32 s{T + 1}, s2, 3",
      f"s_and_b32 s{T + 2}, s2, 7",
      f"s_lshr_b32 s{T + 3}, {s(S_NPART)}, 3",
      f"s_mul_i32 s{T + 2}, s{T + 2}, s{T + 3}",
      f"s_lshr_b32 {s(S_PART)}, s{T + 1}, s{T}",
      f"s_add_u32 {s(S_PART)}, {s(S_PART)}, s{T + 2}",
      f"s_and_b32 {s(S_HBLK)}, s{T + 1}, s{T}",
      f"s_branch {mapped}")
    a.label(plain)
    a(f"s_lshr_b32 {s(S_PART)}, s2, s{T}",
      f"s_and_b32 {s(S_HBLK)}, s2, s{T}")
    a.label(mapped)
    # ------------------------------------------------ partition map
    seq_units_pass(a, find_first=False)
    a(f"s_mul_i32 s{T}, {s(S_PART)}, {s(S_U)}",
      f"s_mul_hi_u32 s{T + 1}, {s(S_PART)}, {s(S_U)}",
      f"s_lshr_b64 s[{T}:{T + 1}], s[{T}:{T + 1}], {s(S_LOG2P)}",
      f"s_mov_b32 {s(S_UA)}, s{T}",
      f"s_add_u32 s{T + 2}, {s(S_PART)}, 1",
      f"s_mul_i32 s{T}, s{T + 2}, {s(S_U)}",
      f"s_mul_hi_u32 s{T + 1}, s{T + 2}, {s(S_U)}",
      f"s_lshr_b64 s[{T}:{T + 1}], s[{T}:{T + 1}], {s(S_LOG2P)}",
      f"s_mov_b32 {s(S_UB)}, s{T}",
      f"s_cmp_ge_u32 {s(S_UA)}, {s(S_UB)}",
      "s_cbranch_scc1 .Lkernel_end")
    seq_units_pass(a, find_first=True)
    # ------------------------------------------------ this wave's query rows
    a(f"s_lshl_b32 s{T}, {s(S_WAVE)}, 5",
      f"s_sub_u32 s{T + 1}, {s(S_HB)}, 1",
      f"s_and_b32 s{T + 2}, s{T}, s{T + 1}",
      f"s_mul_i32 s{T + 3}, {s(S_HBLK)}, {s(S_HB)}",
      f"s_add_u32 {s(S_HEAD0)}, s{T + 2}, s{T + 3}",
      f"s_ff1_i32_b32 s{T + 1}, {s(S_HB)}",
      f"s_lshr_b32 {s(S_STOK)}, s{T}, s{T + 1}")
    # ------------------------------------------------ lane-constant LDS offsets
    t = V_T
    a(f"v_and_b32 {vreg(t)}, 1, {vreg(V_G)}",
      f"v_mul_u32_u24 {vreg(t)}, 12, {vreg(t)}",
      f"v_xor_b32 {vreg(t)}, {vreg(V_R16)}, {vreg(t)}",
      f"v_lshlrev_b32 {vreg(t)}, 4, {vreg(t)}",
      f"v_lshlrev_b32 {vreg(t + 1)}, 10, {vreg(V_G)}",
      f"v_add_u32 {vreg(V_QKOFF)}, {vreg(t)}, {vreg(t + 1)}",
      f"v_lshrrev_b32 {vreg(t)}, 1, {vreg(V_R16)}",
      f"v_and_b32 {vreg(t)}, 1, {vreg(t)}",
      f"v_lshlrev_b32 {vreg(t + 1)}, 2, {vreg(V_G)}",
      f"v_lshrrev_b32 {vreg(t + 2)}, 2, {vreg(V_R16)}",
      f"v_add_u32 {vreg(t + 1)}, {vreg(t + 1)}, {vreg(t + 2)}",
      f"v_mul_u32_u24 {vreg(t + 2)}, 12, {vreg(t)}",
      f"v_xor_b32 {vreg(t + 1)}, {vreg(t + 1)}, {vreg(t + 2)}",
      f"v_lshlrev_b32 {vreg(t + 1)}, 4, {vreg(t + 1)}",
      f"v_lshlrev_b32 {vreg(t + 2)}, 10, {vreg(t)}",
      f"v_add_u32 {vreg(t + 1)}, {vreg(t + 1)}, {vreg(t + 2)}",
      f"v_and_b32 {vreg(t + 2)}, 1, {vreg(V_R16)}",
      f"v_lshlrev_b32 {vreg(t + 2)}, 3, {vreg(t + 2)}",
      f"v_add_u32 {vreg(V_PVOFF)}, {vreg(t + 1)}, {vreg(t + 2)}",
      f"v_lshlrev_b32 {vreg(V_G4)}, 2, {vreg(V_G)}",
      f"v_mov_b32 {vreg(V_FLAG)}, {FLAG_ADDR}",
      f"v_mov_b32 {vreg(V_NEGINF)}, {NEG_INF}")
    # restart flag = 0
    nowrite = a.new_label("flaginit")
    a(f"s_cmp_eq_u32 {s(S_WAVE)}, 0",
      f"s_cbranch_scc0 {nowrite}",
      f"v_mov_b32 {vreg(t)}, 0",
      f"ds_write_b32 {vreg(V_FLAG)}, {vreg(t)}")
    a.label(nowrite)
    a(s_waitcnt_lgkm(0), "s_barrier")
    # ------------------------------------------------ loader cursor, first unit
    a(f"s_mov_b32 {s(S_LSEQ)}, {s(S_CSEQ)}",
      f"s_mov_b32 {s(S_LPRE)}, {s(S_CPRE)}")
    load_len(a, S_LLEN, S_LSEQ)
    units_of(a, S_LUNITS, S_LLEN)
    a(f"s_mov_b32 {s(S_UCUR)}, {s(S_UA)}",
      f"s_mov_b32 {s(S_SLOT)}, 0")
    issue_unit(a, S_UCUR, S_SLOT)
    # ------------------------------------------------ segments
    a.label(".Lseg")
    load_len(a, S_CLEN, S_CSEQ)
    units_of(a, S_CUNITS, S_CLEN)
    a(f"s_add_u32 {s(S_SEGEND)}, {s(S_CPRE)}, {s(S_CUNITS)}",
      f"s_min_u32 {s(S_SEGEND)}, {s(S_SEGEND)}, {s(S_UB)}",
      f"s_sub_i32 {s(S_NVIS)}, {s(S_CLEN)}, {s(S_SQ)}",
      f"s_add_i32 {s(S_NVIS)}, {s(S_NVIS)}, {s(S_STOK)}",
      f"s_add_i32 {s(S_NVIS)}, {s(S_NVIS)}, 1",
      # Q row index (c_seq * s_q + s_tok) * 128 + head0
      f"s_mul_i32 s{T}, {s(S_CSEQ)}, {s(S_SQ)}",
      f"s_add_u32 s{T}, s{T}, {s(S_STOK)}",
      f"s_lshl_b32 s{T}, s{T}, 7",
      f"s_add_u32 s{T}, s{T}, {s(S_HEAD0)}",
      f"s_mov_b32 s{T + 1}, 0",
      f"s_lshl_b64 s[{T + 2}:{T + 3}], s[{T}:{T + 1}], 10",
      f"s_add_u32 s{S_QBASE}, {s(S_QA)}, s{T + 2}",
      f"s_addc_u32 s{S_QBASE + 1}, s{S_QA + 1}, s{T + 3}",
      f"s_lshl_b64 s[{T + 2}:{T + 3}], s[{T}:{T + 1}], 7",
      f"s_add_u32 s{S_RBASE}, {s(S_QR)}, s{T + 2}",
      f"s_addc_u32 s{S_RBASE + 1}, s{S_QR + 1}, s{T + 3}",
      # lane offsets: latent (16h + r16)*1024 + 16g ; rope (16h + r16)*128 + 16g
      f"v_lshlrev_b32 {vreg(t)}, 10, {vreg(V_R16)}",
      f"v_lshlrev_b32 {vreg(t + 1)}, 4, {vreg(V_G)}",
      f"v_add_u32 {vreg(t)}, {vreg(t)}, {vreg(t + 1)}",
      f"v_add_u32 {vreg(t + 2)}, 0x4000, {vreg(t)}",
      f"v_lshlrev_b32 {vreg(t + 3)}, 7, {vreg(V_R16)}",
      f"v_add_u32 {vreg(t + 3)}, {vreg(t + 3)}, {vreg(t + 1)}",
      f"v_add_u32 {vreg(t + 1)}, 0x800, {vreg(t + 3)}")
    for h in range(2):
        off = vreg(t) if h == 0 else vreg(t + 2)
        for ks in range(16):
            q = V_Q + (2 * ks + h) * 4
            a(f"global_load_dwordx4 {vr(q, 4)}, {off}, s[{S_QBASE}:{S_QBASE + 1}] offset:{64 * ks}")
    for h in range(2):
        off = vreg(t + 3) if h == 0 else vreg(t + 1)
        for ks in range(2):
            q = V_Q + (2 * (16 + ks) + h) * 4
            a(f"global_load_dwordx4 {vr(q, 4)}, {off}, s[{S_RBASE}:{S_RBASE + 1}] offset:{64 * ks}")
    a(f"v_mov_b32 {vreg(V_MREF[0])}, {NEG_INF}",
      f"v_mov_b32 {vreg(V_MREF[1])}, {NEG_INF}",
      f"v_mov_b32 {vreg(V_LRUN[0])}, 0",
      f"v_mov_b32 {vreg(V_LRUN[1])}, 0")
    zero_o(a)
    # ------------------------------------------------ units of the segment
    a.label(".Lunit")
    a(f"s_sub_u32 {s(S_SLOT)}, {s(S_UCUR)}, {s(S_UA)}",
      f"s_and_b32 {s(S_SLOT)}, {s(S_SLOT)}, 1",
      f"s_add_u32 s{T + 20}, {s(S_UCUR)}, 1",
      f"s_cmp_lt_u32 s{T + 20}, {s(S_UB)}",
      "s_cbranch_scc0 .Lnomore",
      f"s_xor_b32 s{T + 21}, {s(S_SLOT)}, 1")
    issue_unit(a, T + 20, T + 21)
    a(s_waitcnt_vm(18), "s_branch .Lwaited")
    a.label(".Lnomore")
    a(s_waitcnt_vm(0))
    a.label(".Lwaited")
    a("s_barrier")
    a(f"s_sub_u32 {s(S_ROW0)}, {s(S_UCUR)}, {s(S_CPRE)}",
      f"s_lshl_b32 {s(S_ROW0)}, {s(S_ROW0)}, 6",
      f"s_mul_i32 s{T}, {s(S_SLOT)}, {SLOT_BYTES}",
      f"v_add_u32 {vreg(V_QK)}, s{T}, {vreg(V_QKOFF)}",
      f"v_add_u32 {vreg(V_PV)}, s{T}, {vreg(V_PVOFF)}",
      f"v_add_u32 {vreg(V_QK2)}, 0x10000, {vreg(V_QK)}")
    for ss in range(2):
        skip = a.new_label(f"skipss{ss}")
        a(f"s_add_u32 s{T}, {s(S_ROW0)}, {32 * ss}",
          f"s_cmp_gt_i32 {s(S_NVIS)}, s{T}",
          f"s_cbranch_scc0 {skip}")
        substep(a, ss, f"nomask{ss}")
        a.label(skip)
    a(s_waitcnt_lgkm(0), "s_barrier")
    # restart requested?
    a(f"ds_read_b32 {vreg(t)}, {vreg(V_FLAG)}",
      s_waitcnt_lgkm(0),
      "s_nop 1",
      f"v_readfirstlane_b32 s{T}, {vreg(t)}",
      f"s_cmp_eq_u32 s{T}, 0",
      "s_cbranch_scc0 .Lrestart",
      f"s_add_u32 {s(S_UCUR)}, {s(S_UCUR)}, 1",
      f"s_cmp_lt_u32 {s(S_UCUR)}, {s(S_SEGEND)}",
      "s_cbranch_scc1 .Lunit")
    epilogue(a)
    a(f"s_add_u32 {s(S_CPRE)}, {s(S_CPRE)}, {s(S_CUNITS)}",
      f"s_add_u32 {s(S_CSEQ)}, {s(S_CSEQ)}, 1",
      f"s_cmp_lt_u32 {s(S_UCUR)}, {s(S_UB)}",
      "s_cbranch_scc1 .Lseg",
      "s_branch .Lkernel_end")
    # ------------------------------------------------ restart of the segment
    a.label(".Lrestart")
    a(s_waitcnt_vm(0), "s_barrier")
    noclear = a.new_label("noclear")
    a(f"s_cmp_eq_u32 {s(S_WAVE)}, 0",
      f"s_cbranch_scc0 {noclear}",
      f"v_mov_b32 {vreg(t)}, 0",
      f"ds_write_b32 {vreg(V_FLAG)}, {vreg(t)}")
    a.label(noclear)
    a(f"s_max_u32 {s(S_UCUR)}, {s(S_UA)}, {s(S_CPRE)}",
      f"s_mov_b32 {s(S_LSEQ)}, {s(S_CSEQ)}",
      f"s_mov_b32 {s(S_LPRE)}, {s(S_CPRE)}",
      f"s_mov_b32 {s(S_LUNITS)}, {s(S_CUNITS)}",
      f"s_mov_b32 {s(S_LLEN)}, {s(S_CLEN)}",
      f"v_mov_b32 {vreg(V_LRUN[0])}, 0",
      f"v_mov_b32 {vreg(V_LRUN[1])}, 0")
    zero_o(a)
    a(f"s_sub_u32 {s(S_SLOT)}, {s(S_UCUR)}, {s(S_UA)}",
      f"s_and_b32 {s(S_SLOT)}, {s(S_SLOT)}, 1")
    issue_unit(a, S_UCUR, S_SLOT)
    a(s_waitcnt_lgkm(0), "s_barrier", "s_branch .Lunit")
    a.label(".Lkernel_end")
    a("s_endpgm")
    a.lines += [f".L{KNAME}_end:", f"\t.size {KNAME}, .L{KNAME}_end-{KNAME}", ""]
    a.lines += descriptor()
    return a.text()


def descriptor():
    return f"""	.rodata
	.p2align 6
	.amdhsa_kernel {KNAME}
		.amdhsa_group_segment_fixed_size {LDS_BYTES}
		.amdhsa_private_segment_fixed_size 0
		.amdhsa_kernarg_size 104
		.amdhsa_user_sgpr_count 2
		.amdhsa_user_sgpr_kernarg_segment_ptr 1
		.amdhsa_system_sgpr_workgroup_id_x 1
		.amdhsa_system_vgpr_workitem_id 0
		.amdhsa_next_free_vgpr 512
		.amdhsa_next_free_sgpr {S_MAX}
		.amdhsa_accum_offset 256
		.amdhsa_reserve_vcc 1
		.amdhsa_float_denorm_mode_32 3
		.amdhsa_float_denorm_mode_16_64 3
		.amdhsa_ieee_mode 1
		.amdhsa_dx10_clamp 1
	.end_amdhsa_kernel

	.amdgpu_metadata
---
amdhsa.kernels:
  - .agpr_count:     256
    .args:
      - {{ .address_space: global, .offset: 0, .size: 8, .value_kind: global_buffer }}
      - {{ .address_space: global, .offset: 8, .size: 8, .value_kind: global_buffer }}
      - {{ .address_space: global, .offset: 16, .size: 8, .value_kind: global_buffer }}
      - {{ .address_space: global, .offset: 24, .size: 8, .value_kind: global_buffer }}
      - {{ .address_space: global, .offset: 32, .size: 8, .value_kind: global_buffer }}
      - {{ .address_space: global, .offset: 40, .size: 8, .value_kind: global_buffer }}
      - {{ .address_space: global, .offset: 48, .size: 8, .value_kind: global_buffer }}
      - {{ .address_space: global, .offset: 56, .size: 8, .value_kind: global_buffer }}
      - {{ .address_space: global, .offset: 64, .size: 8, .value_kind: global_buffer }}
      - {{ .offset: 72, .size: 4, .value_kind: by_value }}
      - {{ .offset: 76, .size: 4, .value_kind: by_value }}
      - {{ .offset: 80, .size: 4, .value_kind: by_value }}
      - {{ .offset: 84, .size: 4, .value_kind: by_value }}
      - {{ .offset: 88, .size: 4, .value_kind: by_value }}
      - {{ .offset: 92, .size: 4, .value_kind: by_value }}
      - {{ .offset: 96, .size: 4, .value_kind: by_value }}
      - {{ .offset: 100, .size: 4, .value_kind: by_value }}
    .group_segment_fixed_size: {LDS_BYTES}
    .kernarg_segment_align: 8
    .kernarg_segment_size: 104
    .max_flat_workgroup_size: 256
    .name:           {KNAME}
    .private_segment_fixed_size: 0
    .sgpr_count:     {S_MAX + 6}
    .symbol:         {KNAME}.kd
    .vgpr_count:     512
    .wavefront_size: 64
amdhsa.target:   amdgcn-amd-amdhsa--gfx950
amdhsa.version:
  - 1
  - 2
...
	.end_amdgpu_metadata
""".splitlines()


if __name__ == "__main__":
    out = sys.argv[1] if len(sys.argv) > 1 else "mla_decode_gfx950.s"
    with open(out, "w") as f:
        f.write(kernel())
