#!/usr/bin/env python3
"""Emit the gfx950 assembly of the split-KV MLA decode kernels (bf16 and
e4m3 latent caches).

The kernels are written here as a program that prints GCN assembly, so that
the register file can be laid out by hand: one wave per SIMD holds 32 query
rows of Q (144 VGPRs) and a 128 x 128 (bf16) or 32 x 512 (e4m3) fp32 block of
the output accumulator (all 256 AGPRs) for a whole sequence segment, which a
compiler's register allocator does not manage without spilling.  Everything
else is spelled out below:

  * work partition: units of 64 rows (one cache page), sequence after
    sequence; every sequence also weighs SEG_WEIGHT units (its fixed cost),
    so unit j of sequence b sits at position u0_b + SEG_WEIGHT (b + 1) + j,
    and partition p of P (a power of two) takes the units whose positions lie
    in [(pW) >> log2 P, ((p+1)W) >> log2 P), W the total weight;
  * bf16 kernel, steps of 32 rows (half a page): four LDS tiles of a half
    page filled two steps ahead with direct-to-LDS loads (one load moves
    eight whole 128-byte lines; an XOR swizzle keeps the 16-row score reads
    and the transposed output reads free of bank conflicts); in step t the
    score MFMAs of step t (S^T = C Q^T) run interleaved with the output MFMAs
    of step t - 1 (O += P C, B operand read with ds_read_b64_tr_b16), the
    softmax of step t beside the last of them, one barrier per step;
  * e4m3 kernel, units of 64 rows: raw pages (codes, 1x128 scales, bf16 k^R)
    staged one unit ahead, widened exactly to bf16 in LDS, scores per 128-wide
    block scaled in fp32 after the block's MFMAs, P * scale rounded to bf16
    for the output;
  * softmax against a per-segment reference m_ref (first max + 30, log2
    units) instead of a running max; sums that overflow, or a max far past
    the reference, restart the segment with an exact reference; the bf16
    kernel normalises the output by the sum of the bf16-rounded
    probabilities its MFMAs use and takes lse from the exact fp32 sum;
  * epilogue: final rows in fp32 for a sequence wholly inside the partition,
    else an fp16 partial with one power-of-two descale per (column quarter,
    head) and its lse (the partial_out layout of include/mla.h).

Score/softmax/output follow DeepSeek-V3 architecture notes (deepseek.csdn.net)
§2.1.1-§2.1.3: one shared latent row per token serves as key (with the
decoupled RoPE part) and, its first 512 values, as value; scores are scaled by
1/sqrt(d_h + d_h^R).  The e4m3 cache and its 1x128 scales follow DeepSeek-V3
详解 (yudonglee.me) §4.2.

Usage: gen_decode_gfx950.py OUT.s
"""
from __future__ import annotations

import sys

SLOT_BYTES = 64 * 1152          # one page of bf16 rows = one LDS tile
KARG_BYTES = 128                # kernel argument block (both kernels)

# bf16 kernel: two tile slots, then the probability exchange buffer (16 KB):
# the bf16 probabilities of all 128 query rows for the two 32-row sub-steps of
# a unit, as MFMA B-operand fragments: (sub-step ss, 16-row block hb) at
# P_BASE + 1024 (8 ss + hb), lane L's 16 bytes at + 16 L.  The whole 160 KB of
# a compute unit's LDS.
KNAME = "mla_decode_bf16_gfx950"
FP8 = False
P_BASE = 2 * SLOT_BYTES
P_BYTES = 2 * 8 * 1024
FLAG_ADDR = None                # the fp8 kernel's restart flag
LDS_BYTES = P_BASE + P_BYTES
PAGE_BYTES = SLOT_BYTES         # global bytes of one page of the row array

# fp8 kernel: one bf16 tile, two staging slots of raw pages (e4m3 codes, bf16
# rope, fp32 scales), the current unit's scales as [block][row], their
# reciprocals as bf16 (hi, lo) pairs, the flag
F8_CODES, F8_ROPE, F8_SCALES = 64 * 512, 64 * 128, 64 * 16
F8_RAW = F8_CODES + F8_ROPE + F8_SCALES          # 41984
F8_RAW0 = SLOT_BYTES
F8_SCL = F8_RAW0 + 2 * F8_RAW                    # 157696
# 1/scale of the unit's rows as MFMA operands, one 16 x 32 bf16 fragment per
# sub-step ss (rows of the fragment x the sub-step's 32 cache rows, in the
# order the probabilities hold them: lane group g has rows 4g .. 4g + 3, then
# 16 + 4g .. 16 + 4g + 3): fragment row 4q holds bf16(1/s) of latent block q,
# row 4q + 1 the remainder bf16(1/s - bf16(1/s)), rows 4q + 2, 4q + 3 zero.
# Cache row t of the unit (u = t % 32), block q, part h (hi 0, lo 1) sits at
# F8_RF + 1024 (t / 32) + 64 (4q + h) + 16 ((u % 16) / 4) + 8 (u / 16) + 2 (u % 4).
F8_RF = F8_SCL + 1024
F8_FLAG = F8_RF + 2048


def configure(fp8):
    """Select the kernel the generator functions emit."""
    global KNAME, FP8, FLAG_ADDR, LDS_BYTES, PAGE_BYTES
    FP8 = fp8
    if fp8:
        KNAME, FLAG_ADDR, PAGE_BYTES = "mla_decode_fp8_gfx950", F8_FLAG, F8_CODES
        LDS_BYTES = F8_FLAG + 16
    else:
        KNAME, FLAG_ADDR, PAGE_BYTES = "mla_decode_bf16_gfx950", None, SLOT_BYTES
        LDS_BYTES = P_BASE + P_BYTES
NEG_INF = "0xff800000"
LN2 = "0x3f317218"
OVF_SUM = "0x5f800000"   # 2^64

# ---------------------------------------------------------------- registers
# VGPRs
V_TID, V_LANE, V_G, V_R16 = 0, 1, 2, 3
V_QKE, V_QKO, V_PV0, V_LDROW = 4, 5, 6, 7   # lane constants of the tile layout
V_MREF = (8, 9)
V_LRUN = (10, 11)
V_T = 12                 # v12..v15 temporaries
V_S = (16, 32)           # scores of sub-step ss: S[ss][tb][h] at V_S[ss] + (2*tb + h)*4
V_A = 48                 # score-operand ring: NA buffers of 4
NA = 4
V_B = 64                 # output-operand ring: NB buffers of 4
NB = 4
V_P = (80, 88)           # probabilities of sub-step ss: P[ss][h] at V_P[ss] + 4h
V_UQ = 96                # per-unit score-read bases: [even, odd chunk group] x [+0, +64 KB]
V_UP = 100               # per-unit output-read bases, one per 32-byte column phase
V_LDA, V_LDB, V_LCA, V_LCB = 104, 105, 106, 107   # loader lane constants
V_LIM = 15               # visible-row limit of the current sub-step (mask; a temporary outside the phases)
V_ENT = 108              # block-table entry of the unit after next (vector load, one unit ahead)
V_NEGINF = 109
V_PEAK = (110, 111)      # e4m3: largest 8-row probability sum seen per lane in this segment (lean
                         # softmax); bf16: the lane's exact fp32 probability sum, for lse
V_Q = 112                # Q[ks][h] at 112 + (2*ks + h)*4, 144 regs
V_LBLK = (0, 7)          # e4m3: lane (g, r16): running sum over the segment of the rounded
                         # weights of latent block g, bf16(P s_g) / s_g, head 16h + r16 (v0 and v7
                         # serve only the prologue and the bf16 loader)
# source offsets of the next unit's loads (row groups 2w, 2w+1): live through the phases
V_DMA = (V_T + 1, V_T + 2)
# softmax scratch: sub-step 0 borrows P[1], sub-step 1 borrows S[0] (both free at that time)
V_SMT = (tuple(range(V_P[1], V_P[1] + 4)), tuple(range(V_S[0], V_S[0] + 4)))
EPI_TEMPS = list(range(16, 48))   # the epilogue runs between units
# bf16 kernel (output columns split over the waves):
V_PX = 0                 # P_BASE + 16 lane (after the prologue)
V_PXW = V_T              # P_BASE + 16 lane + 2048 w: this wave's fragments (set per unit)
P_OWN = (80, 48)         # this wave's packed probabilities of sub-step ss: + 4h for heads 16h..
SMT_SPLIT = ((88, 89, 90, 91), (56, 57, 58, 59))   # softmax scratch per sub-step
# probability fragments of all 128 query rows read back for the output MFMAs
PF = ((16, 20, 24, 28, 80, 84, 88, 92), tuple(range(32, 64, 4)))
PERSISTENT = {V_LANE, V_G, V_R16, V_QKE, V_QKO, V_PV0, V_LDROW, *V_MREF, *V_LRUN,
              V_LDA, V_LDB, V_LCA, V_LCB, V_NEGINF, *V_PEAK}
# AGPRs: O[cb][h] at (2*cb + h)*4, lane (g, r16) holds columns 16cb + 4g .. +3 of head 16h + r16

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
S_TMP = 60               # s60..s81 scratch
S_OVF = 82               # s82:83 lanes whose max passed the reference in this unit
S_ENTRY, S_NVALID, S_DMALDS, S_SMT = 84, 85, 86, 87
S_FSC, S_FRO = 92, 94    # fp8 scales / rope arrays (s92:93, s94:95)
S_CURVALID = 96          # fp8: valid rows of the unit being dequantized
S_EXACT = 88             # 1 after a restart: the rest of the segment keeps the max-based softmax
S_NV2, S_ENT2 = 89, 90   # prefetched valid rows / page of the unit after next (-1: page in V_ENT)
S_DPAGE = 80             # s80:81 page address + chunk-group offset of one load (S_TMP + 20, + 21)
S_NVLO, S_NVHI = 91, 97  # bf16: rows visible to the workgroup's first / last query token
S_MODE = S_TMP + 13      # bf16: kind of the current unit (0 none, 1 half, 2 classic, 3 lean)
S_PFOFF = S_TMP + 14     # bf16: block-table byte offset of the page prefetch to issue
# loads of the next unit issued in phases 1, 2, 3 of a full unit
DMA_SPLIT = (8, 6, 4)
S_ONES = 98              # bf16 pair (1.0, 1.0): sums of packed probabilities by v_dot2
# query tokens are launched in groups of 1, 2 or 4: S_SQ is the group's size,
# S_STRIDE the tokens per sequence in the query, output and partial arrays,
# S_TOK0 the group's first token
S_STRIDE, S_TOK0 = 100, 101
S_MAX = 102


def temps(*regs, pool):
    """Check that scratch registers come from the given scratch pool."""
    for r in regs:
        assert r in pool and r not in PERSISTENT, f"v{r} is not a scratch register"
    return regs


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


_LABELS = [0]


class Asm:
    def __init__(self):
        self.lines = []

    def __call__(self, *lines):
        for line in lines:
            self.lines.append("\t" + line)

    def label(self, name):
        self.lines.append(f"{name}:")

    def new_label(self, stem):
        _LABELS[0] += 1
        return f".L{stem}_{_LABELS[0]}"

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


SEG_WEIGHT = 3    # the fixed cost of one sequence in a partition, in units (must equal kSegWeight)


def pages_before_pass(a, x_sgpr, dst_sgpr):
    """s[dst] = number of units (pages) whose weighted position lies below
    s[x_sgpr]: the sum over sequences b of clamp(x - (u0_b + (b + 1) W), 0,
    n_b), n_b the units of b, u0_b those before it, W = SEG_WEIGHT."""
    t = V_T
    T = S_TMP
    loop = a.new_label("pbpass")
    a(f"s_mov_b32 s{T}, 0",            # b0
      f"s_mov_b32 s{T + 1}, 0",        # units before the chunk
      f"s_mov_b32 s{dst_sgpr}, 0")
    a.label(loop)
    a(f"v_add_u32 {vreg(t)}, s{T}, {vreg(V_LANE)}",
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
    a(f"v_add_u32 {vreg(t + 2)}, s{T + 1}, {vreg(t + 2)}",          # u0 + n (with the carry)
      f"v_sub_u32 {vreg(t + 3)}, {vreg(t + 2)}, {vreg(t + 1)}",     # u0
      f"v_mad_u32_u24 {vreg(t + 3)}, {vreg(t)}, {SEG_WEIGHT}, {vreg(t + 3)}",
      f"v_add_u32 {vreg(t + 3)}, {SEG_WEIGHT}, {vreg(t + 3)}",     # weighted position of page 0
      f"v_sub_u32 {vreg(t + 3)}, s{x_sgpr}, {vreg(t + 3)}",
      f"v_max_i32 {vreg(t + 3)}, 0, {vreg(t + 3)}",
      f"v_min_i32 {vreg(t + 3)}, {vreg(t + 1)}, {vreg(t + 3)}",
      "s_nop 1")
    wave_incl_scan(a, t, t + 3)
    a(f"v_readlane_b32 s{T + 2}, {vreg(t)}, 63",
      f"v_readlane_b32 s{T + 1}, {vreg(t + 2)}, 63",
      f"s_add_u32 s{dst_sgpr}, s{dst_sgpr}, s{T + 2}",
      f"s_add_u32 s{T}, s{T}, 64",
      f"s_cmp_lt_u32 s{T}, {s(S_BATCH)}",
      f"s_cbranch_scc1 {loop}")


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


FAST_LENS = 4     # chunks of 64 sequence lengths the prologue keeps in registers
V_LENS = 52       # v52..v55: seq_lens[64 c + lane] (free until the first step)


def load_lens_fast(a):
    """v[V_LENS + c] = seq_lens[min(64 c + lane, batch - 1)], c < FAST_LENS:
    every length the partition map needs in one memory round trip."""
    t = V_T
    a(f"s_sub_u32 s{S_TMP}, {s(S_BATCH)}, 1")
    for c in range(FAST_LENS):
        a(f"v_add_u32 {vreg(t + c)}, {64 * c}, {vreg(V_LANE)}",
          f"v_min_u32 {vreg(t + c)}, s{S_TMP}, {vreg(t + c)}",
          f"v_lshlrev_b32 {vreg(t + c)}, 2, {vreg(t + c)}",
          f"global_load_dword {vreg(V_LENS + c)}, {vreg(t + c)}, {sp(S_LENS)}")
    a(s_waitcnt_vm(0))


def units_fast(a, c):
    """v[t+1] = units of sequence 64 c + lane (0 past the batch), v[t] = 64 c + lane."""
    t = V_T
    a(f"v_add_u32 {vreg(t)}, {64 * c}, {vreg(V_LANE)}",
      f"v_cmp_gt_i32 vcc, {s(S_BATCH)}, {vreg(t)}",
      f"v_add_u32 {vreg(t + 3)}, 63, {vreg(V_LENS + c)}",
      f"v_ashrrev_i32 {vreg(t + 3)}, 6, {vreg(t + 3)}",
      f"v_max_i32 {vreg(t + 3)}, 1, {vreg(t + 3)}",
      f"v_cndmask_b32 {vreg(t + 1)}, 0, {vreg(t + 3)}, vcc",
      "s_nop 1")


def pages_before_fast(a, x_sgpr, dst_sgpr):
    """pages_before_pass over the lengths in registers (batch <= 64 FAST_LENS)."""
    t = V_T
    T = S_TMP
    done = a.new_label("pbfdone")
    a(f"s_mov_b32 s{T + 1}, 0",
      f"s_mov_b32 s{dst_sgpr}, 0")
    for c in range(FAST_LENS):
        if c:
            a(f"s_cmp_le_u32 {s(S_BATCH)}, {64 * c}",
              f"s_cbranch_scc1 {done}")
        units_fast(a, c)
        wave_incl_scan(a, t + 2, t + 1)
        a(f"v_add_u32 {vreg(t + 2)}, s{T + 1}, {vreg(t + 2)}",
          f"v_sub_u32 {vreg(t + 3)}, {vreg(t + 2)}, {vreg(t + 1)}",
          f"v_mad_u32_u24 {vreg(t + 3)}, {vreg(t)}, {SEG_WEIGHT}, {vreg(t + 3)}",
          f"v_add_u32 {vreg(t + 3)}, {SEG_WEIGHT}, {vreg(t + 3)}",
          f"v_sub_u32 {vreg(t + 3)}, s{x_sgpr}, {vreg(t + 3)}",
          f"v_max_i32 {vreg(t + 3)}, 0, {vreg(t + 3)}",
          f"v_min_i32 {vreg(t + 3)}, {vreg(t + 1)}, {vreg(t + 3)}",
          "s_nop 1")
        wave_incl_scan(a, t, t + 3)
        a(f"v_readlane_b32 s{T + 2}, {vreg(t)}, 63",
          f"v_readlane_b32 s{T + 1}, {vreg(t + 2)}, 63",
          f"s_add_u32 s{dst_sgpr}, s{dst_sgpr}, s{T + 2}")
    a.label(done)


def seq_units_fast(a, find_first):
    """seq_units_pass over the lengths in registers; with find_first also
    S_LLEN = the length of the sequence found."""
    t = V_T
    T = S_TMP
    done = a.new_label("suf")
    a(f"s_mov_b32 s{T + 1}, 0")
    founds = []
    for c in range(FAST_LENS):
        if c:
            a(f"s_cmp_le_u32 {s(S_BATCH)}, {64 * c}",
              f"s_cbranch_scc1 {done}")
        units_fast(a, c)
        wave_incl_scan(a, t + 2, t + 1)
        a(f"v_add_u32 {vreg(t + 2)}, s{T + 1}, {vreg(t + 2)}", "s_nop 1")
        if find_first:
            founds.append(a.new_label("suffound"))
            a(f"v_cmp_lt_u32 vcc, {s(S_UA)}, {vreg(t + 2)}",
              f"s_ff1_i32_b64 s{T + 2}, vcc",
              f"s_cmp_lt_i32 s{T + 2}, 0",
              f"s_cbranch_scc0 {founds[-1]}")
        a(f"v_readlane_b32 s{T + 1}, {vreg(t + 2)}, 63")
    a.label(done)
    if not find_first:
        a(f"s_mov_b32 {s(S_U)}, s{T + 1}")
        return
    a("s_branch .Lkernel_end")   # cannot happen when ua < U
    out = a.new_label("sufout")
    for c, f in enumerate(founds):
        a.label(f)
        a(f"s_add_u32 {s(S_CSEQ)}, s{T + 2}, {64 * c}",
          f"v_sub_u32 {vreg(t + 3)}, {vreg(t + 2)}, {vreg(t + 1)}",
          "s_nop 4",
          f"v_readlane_b32 {s(S_CPRE)}, {vreg(t + 3)}, s{T + 2}",
          f"v_readlane_b32 {s(S_LLEN)}, {vreg(V_LENS + c)}, s{T + 2}",
          f"s_branch {out}")
    a.label(out)


def partition_map(a, fast):
    """S_U, then this partition's units [S_UA, S_UB) (ends the kernel when
    empty), the sequence S_CSEQ holding S_UA with its first unit S_CPRE and
    length S_LLEN: every sequence weighs its units + SEG_WEIGHT; partition p of
    P takes the weighted positions [(p W) >> log2 P, ((p + 1) W) >> log2 P), W
    the total, i.e. the units whose positions fall there."""
    T = S_TMP
    (seq_units_fast(a, False) if fast else seq_units_pass(a, find_first=False))
    a(f"s_mul_i32 s{T + 3}, {s(S_BATCH)}, {SEG_WEIGHT}",
      f"s_add_u32 s{T + 3}, s{T + 3}, {s(S_U)}",
      f"s_mul_i32 s{T}, {s(S_PART)}, s{T + 3}",
      f"s_mul_hi_u32 s{T + 1}, {s(S_PART)}, s{T + 3}",
      f"s_lshr_b64 s[{T}:{T + 1}], s[{T}:{T + 1}], {s(S_LOG2P)}",
      f"s_mov_b32 s{T + 10}, s{T}",
      f"s_add_u32 s{T + 2}, {s(S_PART)}, 1",
      f"s_mul_i32 s{T}, s{T + 2}, s{T + 3}",
      f"s_mul_hi_u32 s{T + 1}, s{T + 2}, s{T + 3}",
      f"s_lshr_b64 s[{T}:{T + 1}], s[{T}:{T + 1}], {s(S_LOG2P)}",
      f"s_mov_b32 s{T + 11}, s{T}")
    pb = pages_before_fast if fast else pages_before_pass
    pb(a, T + 10, S_UA)
    pb(a, T + 11, S_UB)
    a(f"s_cmp_ge_u32 {s(S_UA)}, {s(S_UB)}",
      "s_cbranch_scc1 .Lkernel_end")
    if fast:
        seq_units_fast(a, True)
    else:
        seq_units_pass(a, find_first=True)
        load_len(a, S_LLEN, S_CSEQ)


def loader_advance(a, u_sgpr):
    """Move the loader cursor (LSEQ, LPRE, LUNITS, LLEN) forward to the sequence
    that holds unit u."""
    adv, adv_done = a.new_label("adv"), a.new_label("advdone")
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


def loader_lookup(a, u_sgpr, wait):
    """S_NVALID = rows of unit u that hold data (<= 0: none); S_ENTRY = its page
    (block table load left in flight unless wait)."""
    T = S_TMP
    done, contig = a.new_label("lkdone"), a.new_label("contig")
    a(f"s_sub_u32 s{T + 1}, {s(u_sgpr)}, {s(S_LPRE)}",        # j
      f"s_lshl_b32 s{T + 2}, s{T + 1}, 6",
      f"s_sub_i32 {s(S_NVALID)}, {s(S_LLEN)}, s{T + 2}",     # len - 64 j
      f"s_min_i32 {s(S_NVALID)}, {s(S_NVALID)}, 64",
      f"s_cmp_gt_i32 {s(S_NVALID)}, 0",
      f"s_cbranch_scc0 {done}",
      f"s_mul_i32 s{T + 4}, {s(S_LSEQ)}, {s(S_MAXB)}",
      f"s_add_u32 s{T + 4}, s{T + 4}, s{T + 1}",
      f"s_mov_b32 {s(S_ENTRY)}, s{T + 4}",
      f"s_cmp_eq_u64 {sp(S_TABLE)}, 0",
      f"s_cbranch_scc1 {done}",
      f"s_lshl_b32 s{T + 5}, s{T + 4}, 2",
      f"s_load_dword {s(S_ENTRY)}, {sp(S_TABLE)}, s{T + 5}")
    if wait:
        a(s_waitcnt_lgkm(0))
    a.label(done)


def loader_prefetch(a, u_sgpr, issue=True):
    """Look up unit u one unit before its loads are issued: S_NV2 = its valid
    rows (<= 0: none), S_ENT2 = its page for a contiguous cache, or -1 with the
    page on its way into V_ENT (a vector load, so that the LDS waits of the
    phases never wait on it; it lands before the next unit's barrier).  With
    issue=False the load is left to the caller (issue_prefetch): its table
    offset is in S_PFOFF."""
    T = S_TMP
    done = a.new_label("pfdone")
    a(f"s_mov_b32 {s(S_ENT2)}, 0",
      f"s_sub_u32 s{T + 1}, {s(u_sgpr)}, {s(S_LPRE)}",        # j
      f"s_lshl_b32 s{T + 2}, s{T + 1}, 6",
      f"s_sub_i32 {s(S_NV2)}, {s(S_LLEN)}, s{T + 2}",
      f"s_min_i32 {s(S_NV2)}, {s(S_NV2)}, 64",
      f"s_cmp_gt_i32 {s(S_NV2)}, 0",
      f"s_cbranch_scc0 {done}",
      f"s_mul_i32 s{T + 4}, {s(S_LSEQ)}, {s(S_MAXB)}",
      f"s_add_u32 {s(S_ENT2)}, s{T + 4}, s{T + 1}",
      f"s_cmp_eq_u64 {sp(S_TABLE)}, 0",
      f"s_cbranch_scc1 {done}",
      f"s_lshl_b32 s{T + 5}, {s(S_ENT2)}, 2")
    if issue:
        a(f"v_mov_b32 {vreg(V_T + 3)}, s{T + 5}",       # v13/v14 hold the next unit's load offsets
          f"global_load_dword {vreg(V_ENT)}, {vreg(V_T + 3)}, {sp(S_TABLE)}")
    else:
        a(f"s_mov_b32 {s(S_PFOFF)}, s{T + 5}")
    a(f"s_mov_b32 {s(S_ENT2)}, -1")
    a.label(done)


def prefetch_next(a, u_sgpr, issue=True):
    """Prefetch the page of unit u + 1 if the partition has it (else none)."""
    T = S_TMP
    nonext, done = a.new_label("pfnone"), a.new_label("pfend")
    a(f"s_add_u32 s{T + 20}, {s(u_sgpr)}, 1",
      f"s_cmp_lt_u32 s{T + 20}, {s(S_UB)}",
      f"s_cbranch_scc0 {nonext}")
    loader_advance(a, T + 20)
    loader_prefetch(a, T + 20, issue)
    a(f"s_branch {done}")
    a.label(nonext)
    a(f"s_mov_b32 {s(S_NV2)}, 0", f"s_mov_b32 {s(S_ENT2)}, 0")
    a.label(done)


def take_prefetched(a):
    """S_NVALID / S_ENTRY of the next unit from the prefetch (vector loads done)."""
    fromtab, done = a.new_label("fromtab"), a.new_label("takedone")
    a(f"s_mov_b32 {s(S_NVALID)}, {s(S_NV2)}",
      f"s_mov_b32 {s(S_ENTRY)}, {s(S_ENT2)}",
      f"s_cmp_eq_i32 {s(S_ENT2)}, -1",
      f"s_cbranch_scc0 {done}",
      f"v_readfirstlane_b32 {s(S_ENTRY)}, {vreg(V_ENT)}")
    a.label(done)


def loader_page(a):
    """S_PAGE = address of page S_ENTRY, or of the pool's first page when the
    unit holds no rows (its loads are then never used)."""
    T = S_TMP
    done = a.new_label("pgdone")
    a(f"s_mov_b64 {sp(S_PAGE)}, {sp(S_ROWS)}",
      f"s_cmp_gt_i32 {s(S_NVALID)}, 0",
      f"s_cbranch_scc0 {done}",
      f"s_mul_i32 s{T + 5}, {s(S_ENTRY)}, {PAGE_BYTES}",
      f"s_mul_hi_u32 s{T + 6}, {s(S_ENTRY)}, {PAGE_BYTES}",
      f"s_add_u32 s{S_PAGE}, {s(S_ROWS)}, s{T + 5}",
      f"s_addc_u32 s{S_PAGE + 1}, s{S_ROWS + 1}, s{T + 6}")
    a.label(done)


def qk_read(ss, i):
    """A fragment of rows 32ss + 16tb + r16, chunk 4ks + g (i = 2ks + tb)."""
    ks, tb = divmod(i, 2)
    hi = ks >= 16
    base = V_UQ + (ks & 1) + (2 if hi else 0)
    off = 8192 * ((ks >> 1) - (8 if hi else 0)) + 4096 * ss + 2048 * tb
    return [f"\tds_read_b128 {{buf}}, {vreg(base)} offset:{off}"]


def pv_read(ss, cb):
    """Operand of output columns 16cb..16cb+15: rows 32ss + 4g + r, then
    32ss + 16 + 4g + r, r < 4 (the row order of the probabilities)."""
    base = V_UP + (cb & 3)
    off = 8192 * (cb >> 2) + 4096 * ss
    return [f"\tds_read_b64_tr_b16 {{lo}}, {vreg(base)} offset:{off}",
            f"\tds_read_b64_tr_b16 {{hi}}, {vreg(base)} offset:{off + 2048}"]


class Frag:
    """One LDS operand fragment (read into a ring buffer) and the MFMAs that
    consume it."""

    def __init__(self, ring, ring_base, nring, idx, reads, mfmas, deps=None):
        self.ring, self.idx, self.nring = ring, idx, nring
        buf = ring_base + 4 * (idx % nring)
        self.reads = [r.format(buf=vr(buf, 4), lo=vr(buf, 2), hi=vr(buf + 2, 2)) for r in reads]
        self.mfmas = [m.format(buf=vr(buf, 4)) for m in mfmas]
        self.deps = deps or [()] * len(mfmas)   # per MFMA: keys of other LDS reads it waits for
        self.read_ids = []


def pv_frags(ss):
    """O^T[cols, heads] += C^T P^T: lane (g, r16) accumulates columns 16cb + 4g + i of head r16."""
    out = []
    for cb in range(32):
        mf = []
        for h in range(2):
            o = (2 * cb + h) * 4
            mf.append(f"\tv_mfma_f32_16x16x32_bf16 {ar(o, 4)}, {{buf}}, {vr(V_P[ss] + 4 * h, 4)}, {ar(o, 4)}")
        out.append(Frag("B", V_B, NB, 32 * ss + cb, pv_read(ss, cb), mf))
    return out


class LdsOrder:
    """LDS reads in issue order, for exact lgkmcnt waits (LDS ops complete in order)."""

    def __init__(self):
        self.n = 0
        self.done = 0

    def issue(self):
        self.n += 1
        return self.n - 1

    def wait(self, rid):
        if rid < self.done:
            return []
        k = min(self.n - 1 - rid, 15)
        self.done = self.n - k
        return [f"\ts_waitcnt lgkmcnt({k})"]


def softmax_code(ss, S=None, P=None, tmp=None):
    """Softmax of sub-step ss (log2 domain) as a plain instruction list:
    mask rows at or past the visible count, running reference m_ref (first
    max + 30; a max more than 64 above it raises it and flags a restart),
    P = 2^(scale S - m_ref), row sums, bf16 pack into P (kept in S as fp32
    when P is None)."""
    if S is None:
        S, P, tmp = V_S[ss], V_P[ss], V_SMT[ss]
    m, t0, t1, ref = tmp
    x = Asm()
    T = S_SMT
    # lane (g, r16) holds rows 16tb + 4g + i: visible iff 16tb + i < nvis - row0 - 32ss - 4g
    x(f"s_sub_i32 s{T}, {s(S_NVIS)}, {s(S_ROW0)}",
      f"s_sub_i32 s{T}, s{T}, {32 * ss}",
      f"v_mad_i32_i24 {vreg(V_LIM)}, {vreg(V_G)}, -4, s{T}")
    for tb in range(2):
        for i in range(4):
            x(f"v_cmp_lt_i32 vcc, {16 * tb + i}, {vreg(V_LIM)}",
              "s_nop 1")
            for h in range(2):
                r = S + (2 * tb + h) * 4 + i
                x(f"v_cndmask_b32 {vreg(r)}, {vreg(V_NEGINF)}, {vreg(r)}, vcc")
    for h in range(2):
        regs = [S + (2 * tb + h) * 4 + i for tb in range(2) for i in range(4)]
        x(f"v_max3_f32 {vreg(m)}, {vreg(regs[0])}, {vreg(regs[1])}, {vreg(regs[2])}",
          f"v_max3_f32 {vreg(m)}, {vreg(m)}, {vreg(regs[3])}, {vreg(regs[4])}",
          f"v_max3_f32 {vreg(m)}, {vreg(m)}, {vreg(regs[5])}, {vreg(regs[6])}",
          f"v_max_f32 {vreg(m)}, {vreg(m)}, {vreg(regs[7])}")
        xor_reduce(x, m, "v_max_f32", t0, t1)
        mref = V_MREF[h]
        x(f"v_mul_f32 {vreg(m)}, {s(S_SCALE)}, {vreg(m)}",
          # first visible rows of the segment: m_ref = max + 30 (stays -inf while all masked)
          f"v_add_f32 {vreg(t0)}, 0x41f00000, {vreg(m)}",
          f"v_cmp_eq_f32 vcc, {NEG_INF}, {vreg(mref)}",
          "s_nop 1",
          f"v_cndmask_b32 {vreg(mref)}, {vreg(mref)}, {vreg(t0)}, vcc",
          # overflow guard: max - m_ref > 64 -> raise m_ref, ask for a restart
          f"v_sub_f32 {vreg(t1)}, {vreg(m)}, {vreg(mref)}",
          f"v_cmp_lt_f32 vcc, 0x42800000, {vreg(t1)}",
          "s_nop 1",
          f"v_cndmask_b32 {vreg(mref)}, {vreg(mref)}, {vreg(t0)}, vcc",
          f"s_or_b64 {sp(S_OVF)}, {sp(S_OVF)}, vcc",
          # reference used for P: 0 while nothing is visible yet
          f"v_cmp_eq_f32 vcc, {NEG_INF}, {vreg(mref)}",
          "s_nop 1",
          f"v_cndmask_b32 {vreg(ref)}, {vreg(mref)}, 0, vcc")
        for r in regs:
            x(f"v_fma_f32 {vreg(r)}, {vreg(r)}, {s(S_SCALE)}, -{vreg(ref)}")
        for r in regs:
            x(f"v_exp_f32 {vreg(r)}, {vreg(r)}")
        x("s_nop 0", *exact_sum(regs, t0, t1))
        if P is not None:
            # bf16: the exact sum goes to lse (V_PEAK), the sum of the rounded
            # probabilities to the normalisation (V_LRUN)
            x(f"v_add_f32 {vreg(V_PEAK[h])}, {vreg(V_PEAK[h])}, {vreg(t0)}",
              *pack_and_sum(regs, P + 4 * h, t1),
              f"v_add_f32 {vreg(V_LRUN[h])}, {vreg(V_LRUN[h])}, {vreg(t1)}")
        else:
            x(f"v_add_f32 {vreg(V_LRUN[h])}, {vreg(V_LRUN[h])}, {vreg(t0)}")
    return x.lines


def exact_sum(regs, t0, t1):
    """t0 = the fp32 sum of the eight probabilities regs (t1 scratch)."""
    return [f"v_add_f32 {vreg(t0)}, {vreg(regs[0])}, {vreg(regs[1])}",
            f"v_add_f32 {vreg(t1)}, {vreg(regs[2])}, {vreg(regs[3])}",
            f"v_add_f32 {vreg(t0)}, {vreg(t0)}, {vreg(regs[4])}",
            f"v_add_f32 {vreg(t1)}, {vreg(t1)}, {vreg(regs[5])}",
            f"v_add_f32 {vreg(t0)}, {vreg(t0)}, {vreg(regs[6])}",
            f"v_add_f32 {vreg(t1)}, {vreg(t1)}, {vreg(regs[7])}",
            f"v_add_f32 {vreg(t0)}, {vreg(t0)}, {vreg(t1)}"]


def pack_and_sum(regs, p, t):
    """The eight fp32 probabilities regs -> four bf16 pairs at p .. p + 3 (the
    output MFMAs' operand), and t = the sum of the rounded values (v_dot2
    against (1.0, 1.0): exact products, fp32 accumulation; a DOT result read
    by another VALU instruction needs three wait states).  Normalising the
    output by this sum makes it an exact convex combination of the rows with
    the rounded weights: when one row takes nearly all of a softmax its weight
    rounds to nearly 1 and the output to nearly that row."""
    return [f"v_cvt_pk_bf16_f32 {vreg(p)}, {vreg(regs[0])}, {vreg(regs[1])}",
            f"v_cvt_pk_bf16_f32 {vreg(p + 1)}, {vreg(regs[2])}, {vreg(regs[3])}",
            f"v_cvt_pk_bf16_f32 {vreg(p + 2)}, {vreg(regs[4])}, {vreg(regs[5])}",
            f"v_cvt_pk_bf16_f32 {vreg(p + 3)}, {vreg(regs[6])}, {vreg(regs[7])}",
            f"v_dot2_f32_bf16 {vreg(t)}, {vreg(p)}, {s(S_ONES)}, 0",
            f"v_dot2_f32_bf16 {vreg(t)}, {vreg(p + 1)}, {s(S_ONES)}, {vreg(t)}",
            f"v_dot2_f32_bf16 {vreg(t)}, {vreg(p + 2)}, {s(S_ONES)}, {vreg(t)}",
            f"v_dot2_f32_bf16 {vreg(t)}, {vreg(p + 3)}, {s(S_ONES)}, {vreg(t)}",
            "s_nop 2"]


def softmax_lean(ss, S=None, P=None, tmp=None):
    """Softmax of a fully visible sub-step once the segment's reference is
    set: P = 2^(scale S - m_ref), row sums, bf16 pack.  No max: a lane whose
    8-row sum passes 2^64 (the largest score more than ~64 above m_ref) flags a
    restart.  V_PEAK: in the e4m3 kernel the largest such sum, so that the
    restart can raise m_ref past it; in the bf16 kernel the exact running sum
    (for lse), and at a restart every head whose running sum has passed 2^64
    starts over from its first maximum.  That includes a head whose sum got
    there without any one 8-row sum passing 2^64 (only when another head
    overflowed): it costs that head a recomputation, not accuracy, since the
    restarted segment is exact either way.

    The two row halves are interleaved so that no two exponentials (quarter
    rate) sit next to each other: spread between MFMAs, each MFMA then hides
    at most one of them."""
    if S is None:
        S, P, tmp = V_S[ss], V_P[ss], V_SMT[ss]
    t0, t1 = tmp[0], tmp[1]
    fma, exp, tail = [], [], []
    for h in range(2):
        regs = [S + (2 * tb + h) * 4 + i for tb in range(2) for i in range(4)]
        mref = V_MREF[h]
        fma.append([f"\tv_fma_f32 {vreg(r)}, {vreg(r)}, {s(S_SCALE)}, -{vreg(mref)}" for r in regs])
        exp.append([f"\tv_exp_f32 {vreg(r)}, {vreg(r)}" for r in regs])
        x = Asm()
        x(*exact_sum(regs, t0, t1),
          f"v_cmp_lt_f32 vcc, {OVF_SUM}, {vreg(t0)}")
        if P is not None:
            # bf16: exact sum for lse, rounded sum for the normalisation (softmax_code)
            x(f"v_add_f32 {vreg(V_PEAK[h])}, {vreg(V_PEAK[h])}, {vreg(t0)}",
              f"s_or_b64 {sp(S_OVF)}, {sp(S_OVF)}, vcc",
              *pack_and_sum(regs, P + 4 * h, t1),
              f"v_add_f32 {vreg(V_LRUN[h])}, {vreg(V_LRUN[h])}, {vreg(t1)}")
        else:
            x(f"v_add_f32 {vreg(V_LRUN[h])}, {vreg(V_LRUN[h])}, {vreg(t0)}",
              f"v_max_f32 {vreg(V_PEAK[h])}, {vreg(V_PEAK[h])}, {vreg(t0)}",
              f"s_or_b64 {sp(S_OVF)}, {sp(S_OVF)}, vcc")
        tail.append(x.lines)
    # half 0's sums read its exponentials long after they issue, half 1's sums
    # follow seven other instructions (a transcendental result needs one)
    out = list(fma[0])
    for i in range(8):
        out += [exp[0][i], fma[1][i]]
    for i in range(8):
        out += [exp[1][i], tail[0][i]]
    out += tail[0][8:] + tail[1]
    return out


def merge_filler(ins, groups):
    """Spread the load groups evenly through an instruction list (order kept)."""
    if not groups:
        return list(ins)
    out, step = [], len(ins) / len(groups)
    gi = 0
    for k, x in enumerate(ins):
        while gi < len(groups) and k >= gi * step:
            out.append(list(groups[gi]))
            gi += 1
        out.append(x)
    for g in groups[gi:]:
        out.append(list(g))
    return out


# ======================================================= bf16: split output
# In the bf16 kernel each wave scores its own 32 query rows against all 64 rows
# of a unit (Q stays in its registers), publishes its bf16 probabilities in the
# exchange buffer, and then accumulates the output of its own 128 latent
# columns for all 128 query rows: O^T[cols, rows] += C^T P^T with one
# transposed tile read per 16 columns feeding eight MFMAs.  Each tile byte is
# then read once per wave for the scores and once per workgroup for the
# output, instead of four times for both.
def emit_stream(a, frags, lead, fillers, events=None, marks=None):
    """Emit the MFMA stream `frags` with its LDS reads, filler and events.

    Ring reads as in emit_phases.  fillers: (first, last, instructions),
    spread evenly over the MFMAs of fragments first..last (no LDS operations
    inside).  events: {p: items} emitted after the MFMAs (and ring reads) of
    fragment p (-1: before the stream); an item is an instruction, ("lds",
    instruction, key) for an LDS operation whose completion others wait on,
    or ("wait", key).  An MFMA with dependency keys waits for those
    operations first (LDS operations complete in issue order)."""
    lds = LdsOrder()
    keys = {}
    nring = {f.ring: f.nring for f in frags}
    by_ring = {}
    for f in frags:
        by_ring.setdefault(f.ring, []).append(f)
    pending = {}
    pos_of = {id(f): p for p, f in enumerate(frags)}
    for ring, lst in by_ring.items():
        for j, f in enumerate(lst):
            at = lead[ring] if j < nring[ring] else pos_of[id(lst[j - nring[ring]])]
            pending.setdefault(at, []).append(f)
    slots = {}
    for item in fillers:
        if item[0] == "slots":           # precomputed {(fragment, MFMA): instructions}
            for sl, ins in item[1].items():
                slots.setdefault(sl, []).extend(ins)
            continue
        first, last, ins = item
        mslots = [(p, m) for p in range(first, last + 1) for m in range(len(frags[p].mfmas))]
        n = len(mslots)
        per = [len(ins) * (k + 1) // n - len(ins) * k // n for k in range(n)]
        it = iter(ins)
        for k, sl in enumerate(mslots):
            for _ in range(per[k]):
                item = next(it)     # a list is an atomic group: emitted together
                slots.setdefault(sl, []).extend(item if isinstance(item, list) else [item])

    def issue_reads(f):
        for r in f.reads:
            f.read_ids.append(lds.issue())
            a.lines.append(r)

    def run_events(p):
        for item in (events or {}).get(p, []):
            if isinstance(item, str):
                a.lines.append(item)
            elif item[0] == "lds":
                keys[item[2]] = lds.issue()
                a.lines.append(item[1])
            else:
                a.lines += lds.wait(keys[item[1]])

    for f in pending.get(-1, []):
        issue_reads(f)
    run_events(-1)
    for p, f in enumerate(frags):
        a.lines += lds.wait(max(f.read_ids))
        for m, mf in enumerate(f.mfmas):
            if f.deps[m]:
                a.lines += lds.wait(max(keys[k] for k in f.deps[m]))
            a.lines.append(mf)
            a.lines += slots.get((p, m), [])
        for g in pending.get(p, []):
            issue_reads(g)
        run_events(p)
        if marks and p in marks:
            a.comment(f"phase {marks[p]} issued")


# ============================================================== fp8 cache
# The fp8 kernel keeps one bf16 tile (same layout as above) and two staging
# slots of raw pages.  Per unit: the raw pages of the next unit are loaded
# into the free staging slot; the current unit's e4m3 codes are widened to
# bf16 (exact) into the tile, with the rows past the sequence zeroed, and its
# scales are stored as [block][row] fp32.  Scores then take the four 128-wide
# latent blocks one at a time: T = C8_blk Q_blk by MFMA, S += T * s_blk in
# fp32, so that z = scale * (sum_blk s_blk (q_blk . c8_blk) + q^R . k^R) holds
# with the e4m3 values exact; the output takes P * s_blk (rounded to bf16 like
# P in the bf16 kernel) against the widened codes, block by block.
# (DeepSeek-V3 详解, yudonglee.me, §4.2: 1x128 fine-grained scaling, E4M3.)
F8_S = V_S[0]           # scores, then probabilities (fp32) of the current sub-step
F8_T = V_S[1]           # block accumulator; scale values and products in the output phase
F8_P = V_P              # P * s_blk (bf16) of even / odd blocks
V_DWE0, V_L16, V_CSRC, V_SCLB = V_LDA, V_LDB, V_LCA, V_LCB   # fp8 lane constants
S_RPAGE, S_SPAGE = S_TMP + 8, S_TMP + 10                       # rope / scale pages of the next unit


def lane_constants_fp8(a):
    """fp8 lane constants (after the shared ones).
    V_DWE0: tile offset of (row-in-block L>>3, chunk slot of L&7) for an even
    row group (the odd one is V_DWE0 ^ 32); V_L16 = 16 L; V_CSRC: byte offset
    in a page of e4m3 codes read by lane L of a staging load (rows (L&31)>>2,
    8-byte chunks 2 (L&3) and +1 of chunk group L>>5); V_SCLB: LDS address of
    the scales of rows 4g .. 4g+3 (block 0)."""
    t0, t1 = V_T, V_T + 1
    a(f"v_lshrrev_b32 {vreg(t0)}, 3, {vreg(V_LANE)}",
      f"v_lshl_add_u32 {vreg(V_DWE0)}, {vreg(t0)}, 7, {vreg(V_LCA)}",     # uses LCA before it is replaced
      f"v_lshlrev_b32 {vreg(V_L16)}, 4, {vreg(V_LANE)}",
      f"v_bfe_u32 {vreg(t0)}, {vreg(V_LANE)}, 2, 3",                     # rb = (L & 31) >> 2
      f"v_lshlrev_b32 {vreg(t0)}, 9, {vreg(t0)}",
      f"v_lshrrev_b32 {vreg(t1)}, 5, {vreg(V_LANE)}",                     # Ksel
      f"v_lshl_add_u32 {vreg(t0)}, {vreg(t1)}, 6, {vreg(t0)}",
      f"v_and_b32 {vreg(t1)}, 3, {vreg(V_LANE)}",
      f"v_lshl_add_u32 {vreg(V_CSRC)}, {vreg(t1)}, 4, {vreg(t0)}",        # + 16 (L & 3)
      f"v_lshlrev_b32 {vreg(V_SCLB)}, 4, {vreg(V_G)}",
      f"v_add_u32 {vreg(V_SCLB)}, {F8_SCL}, {vreg(V_SCLB)}")


def loader_page_fp8(a):
    """S_PAGE / S_RPAGE / S_SPAGE = the code, rope and scale pages of S_ENTRY
    (page 0 of each array when the unit holds no rows)."""
    T = S_TMP
    done = a.new_label("pgdone")
    a(f"s_mov_b64 {sp(S_PAGE)}, {sp(S_ROWS)}",
      f"s_mov_b64 {sp(S_RPAGE)}, {sp(S_FRO)}",
      f"s_mov_b64 {sp(S_SPAGE)}, {sp(S_FSC)}",
      f"s_cmp_gt_i32 {s(S_NVALID)}, 0",
      f"s_cbranch_scc0 {done}")
    for dst, base, nbytes in ((S_PAGE, S_ROWS, F8_CODES), (S_RPAGE, S_FRO, F8_ROPE), (S_SPAGE, S_FSC, F8_SCALES)):
        a(f"s_mul_i32 s{T + 5}, {s(S_ENTRY)}, {nbytes}",
          f"s_mul_hi_u32 s{T + 6}, {s(S_ENTRY)}, {nbytes}",
          f"s_add_u32 s{dst}, s{base}, s{T + 5}",
          f"s_addc_u32 s{dst + 1}, s{base + 1}, s{T + 6}")
    a.label(done)


def dma_fp8(a, slot_sgpr):
    """Copy the rows 16w .. 16w+15 of the next unit's raw pages into staging
    slot `slot`: 8 loads of codes (8 rows x 128 B each), 2 of rope, 1 of
    scales (16 lanes)."""
    T = S_TMP
    m0c, m0r, m0s = T + 12, T + 13, T + 14
    a(f"s_mul_i32 s{m0c}, {s(slot_sgpr)}, {F8_RAW}",
      f"s_add_u32 s{m0c}, s{m0c}, {F8_RAW0}",
      f"s_lshl_b32 s{T + 15}, {s(S_WAVE)}, 11",                 # 2048 w
      f"s_add_u32 s{m0r}, s{m0c}, {F8_CODES}",
      f"s_add_u32 s{m0r}, s{m0r}, s{T + 15}",
      f"s_add_u32 s{S_RPAGE}, s{S_RPAGE}, s{T + 15}",
      f"s_addc_u32 s{S_RPAGE + 1}, s{S_RPAGE + 1}, 0",
      f"s_lshl_b32 s{T + 15}, {s(S_WAVE)}, 13",                 # 8192 w
      f"s_add_u32 s{m0c}, s{m0c}, s{T + 15}",
      f"s_add_u32 s{S_PAGE}, s{S_PAGE}, s{T + 15}",
      f"s_addc_u32 s{S_PAGE + 1}, s{S_PAGE + 1}, 0",
      f"s_lshl_b32 s{T + 15}, {s(S_WAVE)}, 8",                  # 256 w
      f"s_add_u32 s{S_SPAGE}, s{S_SPAGE}, s{T + 15}",
      f"s_addc_u32 s{S_SPAGE + 1}, s{S_SPAGE + 1}, 0",
      f"s_mul_i32 s{m0s}, {s(slot_sgpr)}, {F8_RAW}",
      f"s_add_u32 s{m0s}, s{m0s}, {F8_RAW0 + F8_CODES + F8_ROPE}",
      f"s_add_u32 s{m0s}, s{m0s}, s{T + 15}")
    for j in range(8):
        a(f"s_add_u32 s{S_DPAGE}, s{S_PAGE}, {(j >> 2) * 4096 + (j & 3) * 128}",
          f"s_addc_u32 s{S_DPAGE + 1}, s{S_PAGE + 1}, 0",
          f"s_add_u32 m0, s{m0c}, {1024 * j}",
          "s_nop 0",
          f"global_load_lds_dwordx4 {vreg(V_CSRC)}, {sp(S_DPAGE)}")
    for i in range(2):
        a(f"s_add_u32 s{S_DPAGE}, s{S_RPAGE}, {1024 * i}",
          f"s_addc_u32 s{S_DPAGE + 1}, s{S_RPAGE + 1}, 0",
          f"s_add_u32 m0, s{m0r}, {1024 * i}",
          "s_nop 0",
          f"global_load_lds_dwordx4 {vreg(V_L16)}, {sp(S_DPAGE)}")
    a(f"s_mov_b64 exec, 0xffff",
      f"s_mov_b32 m0, s{m0s}",
      "s_nop 0",
      f"global_load_lds_dwordx4 {vreg(V_L16)}, {sp(S_SPAGE)}",
      "s_mov_b64 exec, -1")


def issue_unit_fp8(a, u_sgpr, slot_sgpr):
    """Stand-alone staging copy of unit u (prologue and restart)."""
    loader_advance(a, u_sgpr)
    loader_lookup(a, u_sgpr, wait=True)
    loader_page_fp8(a)
    dma_fp8(a, slot_sgpr)


def dequant_fp8(a, masked=True):
    """Rows 16w .. 16w+15 of the current unit: staging slot S_SLOT -> bf16
    tile (codes widened exactly, rows at or past S_CURVALID zeroed), rope
    copied, scales transposed to [block][row].  Ends with the LDS writes in
    flight.  masked=False: every row holds data (S_CURVALID >= 64), no
    zeroing."""
    T = S_TMP
    lds = LdsOrder()
    lds.issue()                                 # the restart-flag read issued before
    raw = T + 12
    mk = (T + 16, T + 18)                       # row masks of the two row groups (SGPR pairs)
    rdb, w0, w1, t0 = V_B, V_B + 1, V_B + 2, V_B + 3      # output-ring registers are free here
    a(f"s_mul_i32 s{raw}, {s(S_SLOT)}, {F8_RAW}",
      f"s_add_u32 s{raw}, s{raw}, {F8_RAW0}",
      f"s_lshl_b32 s{T + 13}, {s(S_WAVE)}, 13",
      f"s_add_u32 s{T + 13}, s{raw}, s{T + 13}",             # raw + 8192 w
      f"v_lshlrev_b32 {vreg(rdb)}, 3, {vreg(V_LANE)}",
      f"v_add_u32 {vreg(rdb)}, s{T + 13}, {vreg(rdb)}",
      f"s_lshl_b32 s{T + 14}, {s(S_WAVE)}, 11",              # 2048 w
      f"v_add_u32 {vreg(w0)}, s{T + 14}, {vreg(V_DWE0)}",
      f"v_xor_b32 {vreg(w1)}, 32, {vreg(V_DWE0)}",
      f"s_add_u32 s{T + 15}, s{T + 14}, 1024",
      f"v_add_u32 {vreg(w1)}, s{T + 15}, {vreg(w1)}",
      # row 16w + 8 Rsel + (L >> 3) < valid
      f"v_lshrrev_b32 {vreg(t0)}, 3, {vreg(V_LANE)}",
      f"s_lshl_b32 s{T + 15}, {s(S_WAVE)}, 4",
      f"v_add_u32 {vreg(t0)}, s{T + 15}, {vreg(t0)}",
      f"v_cmp_gt_i32 s[{mk[0]}:{mk[0] + 1}], {s(S_CURVALID)}, {vreg(t0)}",
      f"v_add_u32 {vreg(t0)}, 8, {vreg(t0)}",
      f"v_cmp_gt_i32 s[{mk[1]}:{mk[1] + 1}], {s(S_CURVALID)}, {vreg(t0)}")
    # codes: 16 reads of 8 bytes per lane up front (v16..v47), 4 output sets (v48..v63)
    rid = []
    for n in range(16):
        rsel, kk = divmod(n, 8)
        d = 16 + 2 * n
        a(f"ds_read_b64 {vr(d, 2)}, {vreg(rdb)} offset:{(rsel * 4 + kk // 2) * 1024 + (kk & 1) * 512}")
        rid.append(lds.issue())
    for n in range(16):
        rsel, kk = divmod(n, 8)
        d, o = 16 + 2 * n, 48 + 4 * (n % 4)
        m = f"s[{mk[rsel]}:{mk[rsel] + 1}]"
        a.lines += lds.wait(rid[n])
        if masked:
            a(f"v_cndmask_b32 {vreg(d)}, 0, {vreg(d)}, {m}",
              f"v_cndmask_b32 {vreg(d + 1)}, 0, {vreg(d + 1)}, {m}")
        a(f"v_cvt_scalef32_pk_bf16_fp8 {vreg(o)}, {vreg(d)}, 1.0",
          f"v_cvt_scalef32_pk_bf16_fp8 {vreg(o + 1)}, {vreg(d)}, 1.0 op_sel:[1,0,0]",
          f"v_cvt_scalef32_pk_bf16_fp8 {vreg(o + 2)}, {vreg(d + 1)}, 1.0",
          f"v_cvt_scalef32_pk_bf16_fp8 {vreg(o + 3)}, {vreg(d + 1)}, 1.0 op_sel:[1,0,0]",
          "s_nop 1",
          f"ds_write_b128 {vreg(w1 if rsel else w0)}, {vr(o, 4)} offset:{8192 * kk}")
        lds.issue()
    # rope: rows 16w + 8 Rsel + (L >> 3), chunk 64 + (L & 7)
    rrb = V_B + 4
    a(f"s_add_u32 s{T + 13}, s{raw}, {F8_CODES}",
      f"s_lshl_b32 s{T + 14}, {s(S_WAVE)}, 11",
      f"s_add_u32 s{T + 13}, s{T + 13}, s{T + 14}",
      f"v_add_u32 {vreg(rrb)}, s{T + 13}, {vreg(V_L16)}")
    rr = []
    for rsel in range(2):
        d = 64 + 8 + 4 * rsel
        a(f"ds_read_b128 {vr(d, 4)}, {vreg(rrb)} offset:{1024 * rsel}")
        rr.append(lds.issue())
    for rsel in range(2):
        d = 64 + 8 + 4 * rsel
        m = f"s[{mk[rsel]}:{mk[rsel] + 1}]"
        a.lines += lds.wait(rr[rsel])
        for q in range(4 if masked else 0):
            a(f"v_cndmask_b32 {vreg(d + q)}, 0, {vreg(d + q)}, {m}")
        a(f"v_add_u32 {vreg(t0)}, 0x10000, {vreg(w1 if rsel else w0)}",
          "s_nop 1",
          f"ds_write_b128 {vreg(t0)}, {vr(d, 4)}")
        lds.issue()
        if rsel == 0:
            t0 = V_B + 5
    # scales of rows 16w + L (lanes 0..15) -> [block][row]
    sc, sa, st = 80, V_B + 6, V_B + 7
    a(f"s_add_u32 s{T + 13}, s{raw}, {F8_CODES + F8_ROPE}",
      f"s_lshl_b32 s{T + 14}, {s(S_WAVE)}, 8",
      f"s_add_u32 s{T + 13}, s{T + 13}, s{T + 14}",
      "s_mov_b64 exec, 0xffff",
      f"v_add_u32 {vreg(st)}, s{T + 13}, {vreg(V_L16)}",
      f"ds_read_b128 {vr(sc, 4)}, {vreg(st)}")
    r = lds.issue()
    a(f"s_lshl_b32 s{T + 15}, {s(S_WAVE)}, 4",
      f"v_add_u32 {vreg(st)}, s{T + 15}, {vreg(V_LANE)}",       # row 16w + L
      f"v_cmp_gt_i32 vcc, {s(S_CURVALID)}, {vreg(st)}",
      f"v_lshlrev_b32 {vreg(sa)}, 2, {vreg(st)}",
      f"v_add_u32 {vreg(sa)}, {F8_SCL}, {vreg(sa)}")
    a.lines += lds.wait(r)
    for q in range(4 if masked else 0):
        a(f"v_cndmask_b32 {vreg(sc + q)}, 0, {vreg(sc + q)}, vcc")
    a("s_nop 1")
    for q in range(4):
        a(f"ds_write_b32 {vreg(sa)}, {vreg(sc + q)} offset:{256 * q}")
    # reciprocal scales, for the per-block normalisation of the output: lane
    # L < 32 takes rows 16w + 2p, + 1 (p = L & 7) of block q = L >> 3, and
    # writes 1/s as bf16 hi + lo pairs (0 for a row past the sequence or a
    # scale that is not positive)
    ia, r0, r1, i0, i1, t, hi, lo, pp, qq = range(16, 26)      # the code reads are consumed (hi even)
    mk0, mk1 = T + 16, T + 18
    a("s_mov_b64 exec, 0xffffffff",
      f"v_and_b32 {vreg(pp)}, 7, {vreg(V_LANE)}",
      f"v_lshrrev_b32 {vreg(qq)}, 3, {vreg(V_LANE)}",
      f"v_lshlrev_b32 {vreg(ia)}, 5, {vreg(pp)}",
      f"v_lshl_add_u32 {vreg(ia)}, {vreg(qq)}, 2, {vreg(ia)}",
      f"v_add_u32 {vreg(ia)}, s{T + 13}, {vreg(ia)}",           # staged scales: 16 B per row
      f"ds_read_b32 {vreg(r0)}, {vreg(ia)}",
      f"ds_read_b32 {vreg(r1)}, {vreg(ia)} offset:16")
    rr = lds.issue(), lds.issue()
    a(f"s_lshl_b32 s{T + 15}, {s(S_WAVE)}, 4",
      f"v_lshl_add_u32 {vreg(t)}, {vreg(pp)}, 1, s{T + 15}",   # row 16w + 2p
      f"v_cmp_gt_i32 s[{mk0}:{mk0 + 1}], {s(S_CURVALID)}, {vreg(t)}",
      f"v_add_u32 {vreg(t)}, 1, {vreg(t)}",
      f"v_cmp_gt_i32 s[{mk1}:{mk1 + 1}], {s(S_CURVALID)}, {vreg(t)}",
      # rows t0 = 16 (w & 1) + 2p, t0 + 1 of sub-step w >> 1, in the token order
      # of the probabilities: F8_RF + 1024 (w >> 1) + 64 (4q) + 8 (w & 1)
      # + 16 (p >> 1) + 4 (p & 1) for the hi pair, the lo pair 64 B on
      f"s_lshr_b32 s{T + 15}, {s(S_WAVE)}, 1",
      f"s_lshl_b32 s{T + 15}, s{T + 15}, 10",
      f"s_and_b32 s{T + 14}, {s(S_WAVE)}, 1",
      f"s_lshl_b32 s{T + 14}, s{T + 14}, 3",
      f"s_add_u32 s{T + 15}, s{T + 15}, s{T + 14}",
      f"s_add_u32 s{T + 15}, s{T + 15}, {F8_RF}",
      f"v_and_b32 {vreg(t)}, 6, {vreg(pp)}",
      f"v_lshlrev_b32 {vreg(t)}, 3, {vreg(t)}",
      f"v_and_b32 {vreg(lo)}, 1, {vreg(pp)}",
      f"v_lshl_add_u32 {vreg(t)}, {vreg(lo)}, 2, {vreg(t)}",
      f"v_lshl_add_u32 {vreg(t)}, {vreg(qq)}, 8, {vreg(t)}",
      f"v_add_u32 {vreg(ia)}, s{T + 15}, {vreg(t)}")
    a.lines += lds.wait(rr[1])
    if masked:
        a(f"v_cndmask_b32 {vreg(r0)}, 0, {vreg(r0)}, s[{mk0}:{mk0 + 1}]",
          f"v_cndmask_b32 {vreg(r1)}, 0, {vreg(r1)}, s[{mk1}:{mk1 + 1}]")
    a(f"v_rcp_f32 {vreg(i0)}, {vreg(r0)}",
      f"v_rcp_f32 {vreg(i1)}, {vreg(r1)}",
      f"v_cmp_lt_f32 vcc, 0, {vreg(r0)}",
      "s_nop 1",
      f"v_cndmask_b32 {vreg(i0)}, 0, {vreg(i0)}, vcc",
      f"v_cmp_lt_f32 vcc, 0, {vreg(r1)}",
      "s_nop 1",
      f"v_cndmask_b32 {vreg(i1)}, 0, {vreg(i1)}, vcc",
      f"v_cvt_pk_bf16_f32 {vreg(hi)}, {vreg(i0)}, {vreg(i1)}",
      f"v_lshlrev_b32 {vreg(t)}, 16, {vreg(hi)}",
      f"v_sub_f32 {vreg(t)}, {vreg(i0)}, {vreg(t)}",              # exact: 1/s - hi
      f"v_and_b32 {vreg(lo)}, 0xffff0000, {vreg(hi)}",
      f"v_sub_f32 {vreg(lo)}, {vreg(i1)}, {vreg(lo)}",
      f"v_cvt_pk_bf16_f32 {vreg(lo)}, {vreg(t)}, {vreg(lo)}",
      f"ds_write_b32 {vreg(ia)}, {vreg(hi)}",
      f"ds_write_b32 {vreg(ia)}, {vreg(lo)} offset:64")
    lds.issue()
    lds.issue()
    a("s_mov_b64 exec, -1")


def f8_scale_reads(ss, blk, dst):
    """Scales of rows 32ss + 16tb + 4g .. +3, block blk -> dst + 4tb (tb = 0, 1)."""
    return [f"\tds_read_b128 {vr(dst + 4 * tb, 4)}, {vreg(V_SCLB)} offset:{blk * 256 + (32 * ss + 16 * tb) * 4}"
            for tb in range(2)]


def qk_fp8(a, ss):
    """Scores of sub-step ss: k^R part into S, then per latent block
    T = C8_blk Q_blk (MFMA) and S += T * s_blk (fp32).  Blocks alternate
    between two accumulators (F8_T and the output-operand ring, which the
    scores leave free) so that the fp32 update of block k runs between the
    MFMAs of block k + 1; only the last block's update is exposed."""
    TB = (F8_T, V_B)                 # block accumulators of even / odd blocks
    SCB = (F8_P[0], F8_P[1])         # their scales (rows 4g .. of both row halves)
    order = [(16, tb) for tb in range(2)] + [(17, tb) for tb in range(2)]
    order += [(ks, tb) for ks in range(16) for tb in range(2)]
    frags = []
    for n, (ks, tb) in enumerate(order):
        acc = F8_S if ks >= 16 else TB[(ks // 4) % 2]
        first = ks == 16 or (ks < 16 and ks % 4 == 0)
        mf = []
        for h in range(2):
            d = acc + (2 * tb + h) * 4
            qreg = V_Q + (2 * ks + h) * 4
            c = "0" if first else vr(d, 4)
            mf.append(f"\tv_mfma_f32_16x16x32_bf16 {vr(d, 4)}, {{buf}}, {vr(qreg, 4)}, {c}")
        frags.append(Frag("A", V_A, NA, n, qk_read(ss, 2 * ks + tb), mf))

    def update(blk):
        """S += T_blk * s_blk, 16 fp32 FMAs."""
        out = []
        for tb in range(2):
            for h in range(2):
                for i in range(4):
                    r = (2 * tb + h) * 4 + i
                    out.append(f"\tv_fma_f32 {vreg(F8_S + r)}, {vreg(TB[blk % 2] + r)}, "
                               f"{vreg(SCB[blk % 2] + 4 * tb + i)}, {vreg(F8_S + r)}")
        return out

    lds = LdsOrder()
    for f in frags[:NA]:
        for r in f.reads:
            f.read_ids.append(lds.issue())
            a.lines.append(r)
    sc_ids = {}
    pending = []                      # the previous block's update, spread over this block's fragments
    for p, f in enumerate(frags):
        ks, tb = order[p]
        if ks < 16 and ks % 4 == 0 and tb == 0:      # block start: its scales
            blk = ks // 4
            for r in f8_scale_reads(ss, blk, SCB[blk % 2]):
                a.lines.append(r)
            sc_ids[blk] = (lds.issue(), lds.issue())
            if blk > 0:
                pending = update(blk - 1)
                a.lines += lds.wait(sc_ids[blk - 1][1])
        a.lines += lds.wait(max(f.read_ids))
        a.lines += f.mfmas
        if p + NA < len(frags):
            g = frags[p + NA]
            for r in g.reads:
                g.read_ids.append(lds.issue())
                a.lines.append(r)
        # the update starts two fragments (four MFMAs) into the next block, past the
        # last MFMA of its block by more than the MFMA-to-VALU latency
        if ks < 16 and pending and (ks % 4) * 2 + tb >= 2:
            a.lines += pending[:3]
            pending = pending[3:]
    a.lines += pending
    a("s_nop 7", "s_nop 7", "s_nop 3")   # last block's MFMAs -> its update
    a.lines += lds.wait(sc_ids[3][1])
    a.lines += update(3)


PV_ACC = 48     # e4m3 output phase: rounded-weight sums, head half h at 48 + 4h (rows 4g.. of lane g)
PV_RF = 56      # the sub-step's reciprocal-scale fragment (4 VGPRs)
PV_RA = 60      # the fragment with the rows of other blocks cleared: one block's operand


F8_RM = S_TMP   # s60..s67: lane masks r16 >> 2 == blk of the four blocks (output phase only)


def f8_rf_read(ss):
    """The sub-step's fragment: lane (g, r16) reads fragment row r16, cache
    rows 32ss + 8g .. +7 of the unit (F8_RF + 64 r16 + 16 g, from V_SCLB =
    F8_SCL + 16 g); and the four block masks."""
    ad, sh = PV_RA, PV_RA + 1
    out = [f"\tv_lshl_add_u32 {vreg(ad)}, {vreg(V_R16)}, 6, {vreg(V_SCLB)}",
           f"\tds_read_b128 {vr(PV_RF, 4)}, {vreg(ad)} offset:{F8_RF - F8_SCL + 1024 * ss}",
           f"\tv_lshrrev_b32 {vreg(sh)}, 2, {vreg(V_R16)}"]
    out += [f"\tv_cmp_eq_u32 s[{F8_RM + 2 * b}:{F8_RM + 2 * b + 1}], {b}, {vreg(sh)}" for b in range(4)]
    return out


def block_weight_operand(blk):
    """PV_RA <- the fragment with every row outside 4blk .. 4blk + 3 zero
    (lanes r16 >> 2 != blk), under the lane mask s[F8_RM + 2 blk]."""
    return [f"\tv_cndmask_b32 {vreg(PV_RA + k)}, 0, {vreg(PV_RF + k)}, s[{F8_RM + 2 * blk}:{F8_RM + 2 * blk + 1}]"
            for k in range(4)]


def block_weight_mfmas(blk):
    """PV_ACC[h] += (1/s fragment of block blk) x (rounded weights of block
    blk): row 4blk of the result is the sum over the sub-step's rows of
    bf16(P s) * bf16(1/s), row 4blk + 1 that of bf16(P s) * lo(1/s); the
    products are exact and the sums fp32."""
    pb = F8_P[blk & 1]
    out = []
    for h in range(2):
        c = "0" if blk == 0 else vr(PV_ACC + 4 * h, 4)
        out.append(f"\tv_mfma_f32_16x16x32_bf16 {vr(PV_ACC + 4 * h, 4)}, {vr(PV_RA, 4)}, {vr(pb + 4 * h, 4)}, {c}")
    return out


def block_sums_add():
    """Lane (g, r16) adds block g's sums (rows 4g, 4g + 1 of PV_ACC) for
    head 16h + r16 to its running V_LBLK[h]."""
    out = ["\ts_nop 7", "\ts_nop 7", "\ts_nop 3"]      # MFMA results -> VALU
    for h in range(2):
        out += [f"\tv_add_f32 {vreg(V_LBLK[h])}, {vreg(V_LBLK[h])}, {vreg(PV_ACC + 4 * h)}",
                f"\tv_add_f32 {vreg(V_LBLK[h])}, {vreg(V_LBLK[h])}, {vreg(PV_ACC + 4 * h + 1)}"]
    return out


def pv_fp8(a, ss):
    """O^T += C8^T (P * s_blk)^T block by block (8 column blocks of 16 per
    latent block).  The scaled probabilities of block blk + 1 are formed between
    the MFMAs of block blk (the two bf16 buffers alternate).  Each block's
    rounded weights are also summed divided by their scales, so that the
    epilogue can normalise block blk by the weights its MFMAs actually used."""
    frags = pv_frags(ss)
    lds = LdsOrder()
    for f in frags[:NB]:
        for r in f.reads:
            f.read_ids.append(lds.issue())
            a.lines.append(r)

    def scaled(blk):
        """P * s_blk -> bf16 buffer F8_P[blk & 1] (24 VALU instructions)."""
        pb = F8_P[blk & 1]
        out = []
        for h in range(2):
            regs = [F8_S + (2 * tb + h) * 4 + i for tb in range(2) for i in range(4)]
            prod = [F8_T + 8 + j for j in range(8)]
            for j, r in enumerate(regs):
                out.append(f"\tv_mul_f32 {vreg(prod[j])}, {vreg(r)}, {vreg(F8_T + j)}")
            q = pb + 4 * h
            out += [f"\tv_cvt_pk_bf16_f32 {vreg(q)}, {vreg(prod[0])}, {vreg(prod[1])}",
                    f"\tv_cvt_pk_bf16_f32 {vreg(q + 1)}, {vreg(prod[2])}, {vreg(prod[3])}",
                    f"\tv_cvt_pk_bf16_f32 {vreg(q + 2)}, {vreg(prod[4])}, {vreg(prod[5])}",
                    f"\tv_cvt_pk_bf16_f32 {vreg(q + 3)}, {vreg(prod[6])}, {vreg(prod[7])}"]
        return out

    for r in f8_scale_reads(ss, 0, F8_T):
        a.lines.append(r)
    sid = lds.issue(), lds.issue()
    rf = f8_rf_read(ss)
    a.lines += rf[:2]
    rfid = lds.issue()
    a.lines += rf[2:]
    a.lines += lds.wait(sid[1])
    a.lines += scaled(0)
    a("s_nop 4")   # VALU writes of P -> MFMA reads
    for blk in range(4):
        pb = F8_P[blk & 1]
        nxt = []
        if blk < 3:
            # scale values of the next block into F8_T (free: this block's products are packed)
            for r in f8_scale_reads(ss, blk + 1, F8_T):
                a.lines.append(r)
            sid = lds.issue(), lds.issue()
            nxt = scaled(blk + 1)
        # this block's weight-sum operand: the fragment with other blocks' rows cleared
        sums = block_weight_operand(blk)
        for j, cb in enumerate(range(8 * blk, 8 * blk + 8)):
            f = frags[cb]
            a.lines += lds.wait(max(f.read_ids))
            for h in range(2):
                o = (2 * cb + h) * 4
                buf = V_B + 4 * (f.idx % NB)
                a(f"v_mfma_f32_16x16x32_bf16 {ar(o, 4)}, {vr(buf, 4)}, {vr(pb + 4 * h, 4)}, {ar(o, 4)}")
            if cb + NB < len(frags):
                g = frags[cb + NB]
                for r in g.reads:
                    g.read_ids.append(lds.issue())
                    a.lines.append(r)
            # the next block's products over fragments 1 .. 4 (done three fragments,
            # six MFMAs, before its first MFMA reads them)
            if nxt and 1 <= j <= 4:
                if j == 1:
                    a.lines += lds.wait(sid[1])
                k = 6 if j < 4 else len(nxt)
                a.lines += nxt[:k]
                nxt = nxt[k:]
            # the block's weight-sum operand over fragments 5, 6; its MFMAs after the
            # block's last output MFMAs (more than five wait states after the operand)
            if j == 5:
                a.lines += lds.wait(rfid)
            if j in (5, 6):
                a.lines += sums[:2]
                sums = sums[2:]
            if j == 7:
                a.lines += block_weight_mfmas(blk)
    a.lines += block_sums_add()


def substep_fp8(a, ss, lean):
    qk_fp8(a, ss)
    if lean:
        a.lines += softmax_lean(ss, S=F8_S, P=None, tmp=(F8_T, F8_T + 1))
    else:
        a.lines += softmax_code(ss, S=F8_S, P=None, tmp=(F8_T, F8_T + 1, F8_T + 2, F8_T + 3))
    pv_fp8(a, ss)


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
      # whole: row_base = (c_seq * stride + tok0 + s_tok) * 128
      f"s_mul_i32 s{T + 1}, {s(S_CSEQ)}, {s(S_STRIDE)}",
      f"s_add_u32 s{T + 1}, s{T + 1}, {s(S_TOK0)}",
      f"s_add_u32 s{T + 1}, s{T + 1}, {s(S_STOK)}",
      f"s_lshl_b32 s{T + 1}, s{T + 1}, 7",
      f"s_mov_b64 s[{T + 4}:{T + 5}], {sp(S_OUT)}",
      f"s_mov_b64 s[{T + 6}:{T + 7}], {sp(S_LSE)}",
      f"s_mov_b32 s{T + 3}, 0",
      f"s_branch {addr_done}")
    a.label(whole_no)
    a(f"s_mov_b32 s{T + 2}, 0",
      f"s_cmp_le_u32 {s(S_CPRE)}, {s(S_UA)}",
      f"s_cbranch_scc1 {pslot1}",
      f"s_mov_b32 s{T + 2}, 1")
    a.label(pslot1)
    a(f"s_lshl_b32 s{T + 1}, {s(S_PART)}, 1",
      f"s_add_u32 s{T + 1}, s{T + 1}, s{T + 2}",
      f"s_mul_i32 s{T + 1}, s{T + 1}, {s(S_STRIDE)}",
      f"s_add_u32 s{T + 1}, s{T + 1}, {s(S_TOK0)}",
      f"s_add_u32 s{T + 1}, s{T + 1}, {s(S_STOK)}",
      f"s_lshl_b32 s{T + 1}, s{T + 1}, 7",
      f"s_mov_b64 s[{T + 4}:{T + 5}], {sp(S_POUT)}",
      f"s_mov_b64 s[{T + 6}:{T + 7}], {sp(S_PLSE)}",
      f"s_mov_b32 s{T + 3}, 1")
    a.label(addr_done)
    a(f"s_add_u32 s{T + 1}, s{T + 1}, {s(S_HEAD0)}",   # first row of this wave's heads
      # lse row pointer and out row pointer (row * 2048 B)
      f"s_lshl_b32 s{T + 8}, s{T + 1}, 2",
      f"s_add_u32 s{T + 10}, s{T + 6}, s{T + 8}",
      f"s_addc_u32 s{T + 11}, s{T + 7}, 0",
      f"s_mul_i32 s{T + 9}, s{T + 1}, 2048",
      f"s_mul_hi_u32 s{T + 12}, s{T + 1}, 2048",
      f"s_add_u32 s{T + 12 + 2}, s{T + 4}, s{T + 9}",
      f"s_addc_u32 s{T + 12 + 3}, s{T + 5}, s{T + 12}")
    obase = sp(T + 14)
    # lse from the exact fp32 sums; the output is normalised per latent block
    # by the sums of the rounded weights (block_inverses)
    for h in range(2):
        lt, lse, t0, t1 = 18, 19, 20, 21
        a(f"v_mov_b32 {vreg(lt)}, {vreg(V_LRUN[h])}")
        xor_reduce(a, lt, "v_add_f32", t0, t1)
        a(f"v_log_f32 {vreg(lse)}, {vreg(lt)}",
          "s_nop 1",
          f"v_cmp_lt_f32 vcc, 0, {vreg(lt)}",
          f"v_add_f32 {vreg(lse)}, {vreg(V_MREF[h])}, {vreg(lse)}",
          f"v_mul_f32 {vreg(lse)}, {LN2}, {vreg(lse)}",
          "s_nop 1",
          f"v_cndmask_b32 {vreg(lse)}, {vreg(V_NEGINF)}, {vreg(lse)}, vcc")
        # lse of head 16h + r16 from the lanes with g == 0
        a(f"v_cmp_eq_u32 vcc, 0, {vreg(V_G)}",
          f"s_and_saveexec_b64 {sp(S_EXEC)}, vcc",
          f"v_lshlrev_b32 {vreg(t0)}, 2, {vreg(V_R16)}",
          f"global_store_dword {vreg(t0)}, {vreg(lse)}, s[{T + 10}:{T + 11}] offset:{64 * h}",
          f"s_mov_b64 exec, {sp(S_EXEC)}")
    inv = block_inverses(a)
    rowwise, stored = a.new_label("rowwise"), a.new_label("stored")
    a(f"s_cmp_eq_u32 s{T + 3}, 0",
      f"s_cbranch_scc1 {rowwise}")
    epi_partial_f16_fp8(a, inv)
    a(f"s_branch {stored}")
    # final result: row layout, lane (g, r16) -> (16h + r16) * 2048 + 16g + 64cb
    a.label(rowwise)
    x = EPI_TEMPS
    bufs = [x[8:12], x[12:16], x[16:20], x[20:24]]
    off, t0 = 18, 19
    for h in range(2):
        a(f"v_lshlrev_b32 {vreg(t0)}, 4, {vreg(V_G)}",
          f"v_lshl_add_u32 {vreg(off)}, {vreg(V_R16)}, 11, {vreg(t0)}")
        if h:
            a(f"v_add_u32 {vreg(off)}, {16 * 2048}, {vreg(off)}")
        for cb in range(32):
            epi_store(a, h, cb, bufs[cb % 4], inv[h][cb // 8], f"{vreg(off)}, {{v}}, {obase} offset:{64 * cb}")
    a.label(stored)


def block_inverses(a):
    """e4m3 epilogue: 1 / (sum of block k's rounded weights) of both heads of
    this lane, for k = 0..3, in v96 + 4h + k (the unit's read bases, free
    between units); 0 where the sum is not positive.  Lane (g, r16) holds
    block g's sum (V_LBLK); permlane swaps spread all four to every lane."""
    t = 27
    inv = [[96 + 4 * h + k for k in range(4)] for h in range(2)]
    for h in range(2):
        r = inv[h]
        a(f"v_mov_b32 {vreg(r[0])}, {vreg(V_LBLK[h])}",
          f"v_mov_b32 {vreg(r[1])}, {vreg(V_LBLK[h])}",
          "s_nop 1",
          f"v_permlane16_swap_b32 {vreg(r[0])}, {vreg(r[1])}",     # rows: L0 L0 L2 L2 / L1 L1 L3 L3
          "s_nop 1",
          f"v_mov_b32 {vreg(r[2])}, {vreg(r[0])}",
          f"v_mov_b32 {vreg(r[3])}, {vreg(r[1])}",
          "s_nop 1",
          f"v_permlane32_swap_b32 {vreg(r[0])}, {vreg(r[2])}",
          f"v_permlane32_swap_b32 {vreg(r[1])}, {vreg(r[3])}",
          "s_nop 1")
        for k in range(4):
            a(f"v_rcp_f32 {vreg(t)}, {vreg(r[k])}",
              f"v_cmp_lt_f32 vcc, 0, {vreg(r[k])}",
              "s_nop 1",
              f"v_cndmask_b32 {vreg(r[k])}, 0, {vreg(t)}, vcc")
    return inv


def epi_partial_f16_fp8(a, inv):
    """e4m3 kernel: this wave's 32 query rows (row index s[T+1]) over all 512
    columns, normalised, as fp16 partials with their descales (the layout of
    the bf16 kernel's partials: chunk (column block c, lane) holds heads
    16a + r16, a < 2, columns 16c + 4g .. +3, at 1 KB c + 16 lane).  Per
    column quarter the 64 accumulator values of each lane are read, the
    per-row largest |value| taken (the four lanes g of a row), the descales
    stored, and the values scaled, packed and stored."""
    T = S_TMP
    vals = list(range(32, 96))           # (cb - 8q, a, i) at 32 + 8 (cb - 8q) + 4 a + i
    invq, m0, m1, t, t0, t1, off, offt = (18, 19), 20, 21, 22, 23, 24, 25, 26
    a(f"s_mul_i32 s{T + 8}, {s(S_NPART)}, {s(S_STRIDE)}",
      f"s_lshr_b32 s{T + 7}, s{T + 8}, 14",
      f"s_lshl_b32 s{T + 6}, s{T + 8}, 18",
      f"s_add_u32 s{T + 6}, s{T + 6}, s{T + 4}",
      f"s_addc_u32 s{T + 7}, s{T + 7}, s{T + 5}",
      # values: out + 1024 row; descales: table + 16 row - 12 (row & 127)
      f"s_lshl_b32 s{T + 16}, s{T + 1}, 10",
      f"s_lshr_b32 s{T + 17}, s{T + 1}, 22",
      f"s_add_u32 s{T + 16}, s{T + 16}, s{T + 4}",
      f"s_addc_u32 s{T + 17}, s{T + 17}, s{T + 5}",
      f"s_and_b32 s{T + 8}, s{T + 1}, 127",
      f"s_mul_i32 s{T + 8}, s{T + 8}, 12",
      f"s_lshl_b32 s{T + 9}, s{T + 1}, 4",
      f"s_sub_u32 s{T + 9}, s{T + 9}, s{T + 8}",
      f"s_add_u32 s{T + 18}, s{T + 6}, s{T + 9}",
      f"s_addc_u32 s{T + 19}, s{T + 7}, 0",
      f"v_lshlrev_b32 {vreg(off)}, 4, {vreg(V_LANE)}",
      f"v_lshlrev_b32 {vreg(offt)}, 3, {vreg(V_R16)}")
    for q in range(4):
        for cl in range(8):
            for h in range(2):
                for i in range(4):
                    a(f"v_accvgpr_read_b32 {vreg(vals[8 * cl + 4 * h + i])}, a{(2 * (8 * q + cl) + h) * 4 + i}")
        for h, m in ((0, m0), (1, m1)):
            lane_abs_max(a, m, [vals[8 * cl + 4 * h + i] for cl in range(8) for i in range(4)])
            xor_reduce(a, m, "v_max_f32", t0, t1)
            a(f"v_mov_b32 {vreg(invq[h])}, {vreg(inv[h][q])}")
            f16_scale(a, m, invq[h], t)
        a(f"v_cmp_eq_u32 vcc, 0, {vreg(V_G)}",
          f"s_and_saveexec_b64 {sp(S_EXEC)}, vcc",
          f"global_store_dwordx2 {vreg(offt)}, {vr(m0, 2)}, s[{T + 18}:{T + 19}] offset:{512 * q} sc0 sc1",
          f"s_mov_b64 exec, {sp(S_EXEC)}")
        for cl in range(8):
            for h in range(2):
                for i in range(4):
                    r = vals[8 * cl + 4 * h + i]
                    a(f"v_mul_f32 {vreg(r)}, {vreg(r)}, {vreg(invq[h])}")
        for cl in range(8):
            v0 = vals[8 * cl]
            for k in range(4):
                a(f"v_cvt_pk_f16_f32 {vreg(v0 + k)}, {vreg(v0 + 2 * k)}, {vreg(v0 + 2 * k + 1)}")
            cb = 8 * q + cl
            if cb and cb % 4 == 0:
                a(f"s_add_u32 s{T + 16}, s{T + 16}, 4096", f"s_addc_u32 s{T + 17}, s{T + 17}, 0")
            a(f"global_store_dwordx4 {vreg(off)}, {vr(v0, 4)}, s[{T + 16}:{T + 17}] offset:{1024 * (cb % 4)} sc0 sc1")


def epilogue_split(a):
    """bf16 kernel, end of a segment (after a barrier that every wave reaches
    past its last output MFMA): publish this wave's row sums and its restart
    request; restart the segment if any wave asks; else normalise this wave's
    128 output columns of all 128 query rows by their row sums and store them
    (final result, or partial slot 0 / 1 of the partition), with the lse of
    the wave's own rows."""
    T = S_TMP
    L, t0, t1 = (16, 17), 18, 19
    LX = (32, 33)                         # exact sums of this wave's rows, for lse
    for h in range(2):
        a(f"v_mov_b32 {vreg(L[h])}, {vreg(V_LRUN[h])}",
          f"v_mov_b32 {vreg(LX[h])}, {vreg(V_PEAK[h])}")
        xor_reduce(a, L[h], "v_add_f32", t0, t1)
        xor_reduce(a, LX[h], "v_add_f32", t0, t1)
    # row sum of query row 32w + 16h + r16 at P_BASE + 4 (32w + 16h + r16); request at P_BASE + 512 + 4w
    a(f"s_lshl_b32 s{T}, {s(S_WAVE)}, 7",
      f"v_lshlrev_b32 {vreg(t0)}, 2, {vreg(V_R16)}",
      f"v_add_u32 {vreg(t0)}, s{T}, {vreg(t0)}",
      f"v_add_u32 {vreg(t0)}, {P_BASE}, {vreg(t0)}",
      f"v_cmp_eq_u32 vcc, 0, {vreg(V_G)}",
      f"s_and_saveexec_b64 {sp(S_EXEC)}, vcc",
      f"ds_write_b32 {vreg(t0)}, {vreg(L[0])}",
      f"ds_write_b32 {vreg(t0)}, {vreg(L[1])} offset:64",
      f"s_mov_b64 exec, {sp(S_EXEC)}",
      f"s_cmp_lg_u64 {sp(S_OVF)}, 0",
      f"s_cselect_b32 s{T + 1}, 1, 0",
      f"s_lshl_b32 s{T}, {s(S_WAVE)}, 2",
      f"s_add_u32 s{T}, s{T}, {P_BASE + 512}",
      f"v_mov_b32 {vreg(t0)}, s{T}",
      f"v_mov_b32 {vreg(t1)}, s{T + 1}",
      f"ds_write_b32 {vreg(t0)}, {vreg(t1)}",
      s_waitcnt_lgkm(0),
      "s_barrier",
      f"v_mov_b32 {vreg(t0)}, {P_BASE + 512}",
      f"ds_read_b128 {vr(20, 4)}, {vreg(t0)}",
      s_waitcnt_lgkm(0),
      "v_or3_b32 v20, v20, v21, v22",
      "v_or_b32 v20, v20, v23",
      "s_nop 1",
      f"v_readfirstlane_b32 s{T}, v20",
      f"s_cmp_eq_u32 s{T}, 0",
      "s_cbranch_scc0 .Lrestart")
    # row sums of all 128 query rows -> 1 / l (0 for a row that saw nothing): lane (g, r16), block hb
    inv = list(range(24, 32))
    a(f"v_lshlrev_b32 {vreg(t0)}, 2, {vreg(V_R16)}",
      f"v_add_u32 {vreg(t0)}, {P_BASE}, {vreg(t0)}")
    for hb in range(8):
        a(f"ds_read_b32 {vreg(inv[hb])}, {vreg(t0)} offset:{64 * hb}")
    # destination: R = first token row of the (sequence | partition slot), flag s[T+3] = partial
    whole_no, pslot1, addr_done = a.new_label("notwhole"), a.new_label("pslot1"), a.new_label("addrdone")
    a(f"s_cmp_lt_u32 {s(S_CPRE)}, {s(S_UA)}",
      f"s_cbranch_scc1 {whole_no}",
      f"s_add_u32 s{T}, {s(S_CPRE)}, {s(S_CUNITS)}",
      f"s_cmp_gt_u32 s{T}, {s(S_UB)}",
      f"s_cbranch_scc1 {whole_no}",
      f"s_mul_i32 s{T + 1}, {s(S_CSEQ)}, {s(S_STRIDE)}",
      f"s_add_u32 s{T + 1}, s{T + 1}, {s(S_TOK0)}",
      f"s_mov_b64 s[{T + 4}:{T + 5}], {sp(S_OUT)}",
      f"s_mov_b64 s[{T + 6}:{T + 7}], {sp(S_LSE)}",
      f"s_mov_b32 s{T + 3}, 0",
      f"s_branch {addr_done}")
    a.label(whole_no)
    a(f"s_mov_b32 s{T + 2}, 0",
      f"s_cmp_le_u32 {s(S_CPRE)}, {s(S_UA)}",
      f"s_cbranch_scc1 {pslot1}",
      f"s_mov_b32 s{T + 2}, 1")
    a.label(pslot1)
    a(f"s_lshl_b32 s{T + 1}, {s(S_PART)}, 1",
      f"s_add_u32 s{T + 1}, s{T + 1}, s{T + 2}",
      f"s_mul_i32 s{T + 1}, s{T + 1}, {s(S_STRIDE)}",
      f"s_add_u32 s{T + 1}, s{T + 1}, {s(S_TOK0)}",
      f"s_mov_b64 s[{T + 4}:{T + 5}], {sp(S_POUT)}",
      f"s_mov_b64 s[{T + 6}:{T + 7}], {sp(S_PLSE)}",
      f"s_mov_b32 s{T + 3}, 1")
    a.label(addr_done)
    # lse of this wave's rows (lanes g == 0): row (R + stok) * 128 + head0 + 16h + r16
    a(f"s_add_u32 s{T + 8}, s{T + 1}, {s(S_STOK)}",
      f"s_lshl_b32 s{T + 8}, s{T + 8}, 7",
      f"s_add_u32 s{T + 8}, s{T + 8}, {s(S_HEAD0)}",
      f"s_lshl_b32 s{T + 8}, s{T + 8}, 2",
      f"s_add_u32 s{T + 10}, s{T + 6}, s{T + 8}",
      f"s_addc_u32 s{T + 11}, s{T + 7}, 0")
    for h in range(2):
        lse = t1
        a(f"v_log_f32 {vreg(lse)}, {vreg(LX[h])}",
          "s_nop 1",
          f"v_cmp_lt_f32 vcc, 0, {vreg(LX[h])}",
          f"v_add_f32 {vreg(lse)}, {vreg(V_MREF[h])}, {vreg(lse)}",
          f"v_mul_f32 {vreg(lse)}, {LN2}, {vreg(lse)}",
          "s_nop 1",
          f"v_cndmask_b32 {vreg(lse)}, {vreg(V_NEGINF)}, {vreg(lse)}, vcc",
          f"v_cmp_eq_u32 vcc, 0, {vreg(V_G)}",
          f"s_and_saveexec_b64 {sp(S_EXEC)}, vcc",
          f"v_lshlrev_b32 {vreg(t0)}, 2, {vreg(V_R16)}",
          f"global_store_dword {vreg(t0)}, {vreg(lse)}, s[{T + 10}:{T + 11}] offset:{64 * h}",
          f"s_mov_b64 exec, {sp(S_EXEC)}")
    a(s_waitcnt_lgkm(0))
    for hb in range(8):
        a(f"v_rcp_f32 {vreg(t1)}, {vreg(inv[hb])}",
          f"v_cmp_lt_f32 vcc, 0, {vreg(inv[hb])}",
          "s_nop 1",
          f"v_cndmask_b32 {vreg(inv[hb])}, 0, {vreg(t1)}, vcc")
    a("s_nop 7", "s_nop 7", "s_nop 3")   # last MFMAs -> accvgpr reads
    # per owner group j (query rows 32j ..): token (32j) >> log2(heads per block), head
    # (32j & (heads per block - 1)) + head block * heads per block; its row index
    # (128 rows per (slot | sequence, token) + head) in s[T+12+j]
    a(f"s_ff1_i32_b32 s{T + 9}, {s(S_HB)}",
      f"s_sub_u32 s{T + 10}, {s(S_HB)}, 1",
      f"s_mul_i32 s{T + 11}, {s(S_HBLK)}, {s(S_HB)}")
    for j in range(4):
        b = T + 12 + j
        a(f"s_lshr_b32 s{b}, {32 * j}, s{T + 9}",
          f"s_add_u32 s{b}, s{b}, s{T + 1}",
          f"s_lshl_b32 s{b}, s{b}, 7",
          f"s_and_b32 s{T + 16}, {32 * j}, s{T + 10}",
          f"s_add_u32 s{b}, s{b}, s{T + 16}",
          f"s_add_u32 s{b}, s{b}, s{T + 11}")
    rowwise, stored = a.new_label("rowwise"), a.new_label("stored")
    a(f"s_cmp_eq_u32 s{T + 3}, 0",
      f"s_cbranch_scc1 {rowwise}")
    # S_EPI tells the next segment's first step how many stores follow its Q
    # loads (the two lse stores above, then this branch's)
    n0 = len(a.lines)
    epi_partial_f16(a, inv)
    assert 2 + sum(ln.strip().startswith("global_store") for ln in a.lines[n0:]) == EPI_STORES_PARTIAL
    a(f"s_mov_b32 {s(S_EPI)}, 2",
      f"s_branch {stored}")
    # final result: row layout, lane (g, r16) of block (hb, cb) -> row head + 16h + r16,
    # columns 128w + 16cb + 4g ..
    bufs = [list(range(32 + 4 * k, 36 + 4 * k)) for k in range(4)]
    off = 48
    a.label(rowwise)
    a(f"v_lshlrev_b32 {vreg(t0)}, 4, {vreg(V_G)}",
      f"v_lshl_add_u32 {vreg(off)}, {vreg(V_R16)}, 11, {vreg(t0)}",
      f"s_lshl_b32 s{T + 8}, {s(S_WAVE)}, 9")
    n = 0
    n0 = len(a.lines)
    for j in range(4):
        b = T + 12 + j
        for h in range(2):
            # s[T+6:T+7] = out + 2048 row + 512 w (+ 16 rows for the second half)
            a(f"s_lshl_b32 s{T + 6}, s{b}, 11",
              f"s_lshr_b32 s{T + 7}, s{b}, 21",
              f"s_add_u32 s{T + 6}, s{T + 6}, s{T + 8}",
              f"s_addc_u32 s{T + 7}, s{T + 7}, 0",
              f"s_add_u32 s{T + 6}, s{T + 6}, s{T + 4}",
              f"s_addc_u32 s{T + 7}, s{T + 7}, s{T + 5}")
            if h:
                a(f"s_add_u32 s{T + 6}, s{T + 6}, 0x8000",
                  f"s_addc_u32 s{T + 7}, s{T + 7}, 0")
            for cb in range(8):
                epi_store_split(a, 2 * j + h, cb, bufs[n % 4], inv[2 * j + h],
                                f"{vreg(off)}, {{v}}, s[{T + 6}:{T + 7}] offset:{64 * cb}")
                n += 1
    assert 2 + sum(ln.strip().startswith("global_store") for ln in a.lines[n0:]) == EPI_STORES_ROWS
    a(f"s_mov_b32 {s(S_EPI)}, 1")
    a.label(stored)


# Partial outputs are written as fp16 with a power-of-two descale per (block,
# column quarter, head): d = 2^(e - 15) for the largest |value| m of the quarter
# (m in [2^(e-1), 2^e)), so that |value / d| < 2^15 stays inside fp16 and keeps
# 11 significant bits; d is clamped to 2^-90 for rows that are (nearly) zero.
F16_DESC_FIELD_MIN = 51    # clamp of the exponent field: scale <= 2^90


def f16_scale(a, m, inv, t):
    """m = this lane's largest |O| of a row (one column quarter), inv its 1/l:
    inv <- inv * 2^k with (m inv) 2^k in [2^14, 2^15), m <- the descale 2^-k
    (fp32 bits built from the exponent field of m inv)."""
    a(f"v_mul_f32 {vreg(m)}, {vreg(m)}, {vreg(inv)}",
      f"v_bfe_u32 {vreg(m)}, {vreg(m)}, 23, 8",
      f"v_max_i32 {vreg(m)}, {F16_DESC_FIELD_MIN}, {vreg(m)}",
      f"v_sub_u32 {vreg(t)}, 268, {vreg(m)}",
      f"v_lshlrev_b32 {vreg(t)}, 23, {vreg(t)}",
      f"v_mul_f32 {vreg(inv)}, {vreg(inv)}, {vreg(t)}",
      f"v_subrev_u32 {vreg(m)}, 14, {vreg(m)}",
      f"v_lshlrev_b32 {vreg(m)}, 23, {vreg(m)}")


def lane_abs_max(a, dst, regs):
    """dst = max |regs| (v_max3 chain)."""
    a(f"v_max3_f32 {vreg(dst)}, |{vreg(regs[0])}|, |{vreg(regs[1])}|, |{vreg(regs[2])}|")
    rest = regs[3:]
    for k in range(0, len(rest), 2):
        if k + 1 < len(rest):
            a(f"v_max3_f32 {vreg(dst)}, {vreg(dst)}, |{vreg(rest[k])}|, |{vreg(rest[k + 1])}|")
        else:
            a(f"v_max_f32 {vreg(dst)}, {vreg(dst)}, |{vreg(rest[k])}|")


def epi_partial_f16(a, inv):
    """bf16 kernel: this wave's 128 columns (quarter w) of all 128 query rows,
    normalised, as fp16 partials with their descales.  Owner group j holds
    query rows 32j .. (row index s[T+12+j]); per j the 64 accumulator values of
    each lane are read (and cleared for the next segment), the per-row largest
    |value| taken over the wave's columns (the four lanes g of a row), the
    descales stored, and the values scaled, packed and stored: chunk
    (column block c = 8w + cb, lane) = 16 bytes at 1 KB c + 16 lane of the
    group's 32 KB."""
    T = S_TMP
    vals = list(range(32, 96))           # (cb, a, i) at 32 + 8 cb + 4 a + i
    off, offt, m0, m1, t, t0, t1 = 20, 21, 22, 23, 18, 16, 17
    # table of descales after the num_splits * 2 * s_q value blocks of 128 KB
    a(f"s_mul_i32 s{T + 8}, {s(S_NPART)}, {s(S_STRIDE)}",
      f"s_lshr_b32 s{T + 7}, s{T + 8}, 14",
      f"s_lshl_b32 s{T + 6}, s{T + 8}, 18",
      f"s_add_u32 s{T + 6}, s{T + 6}, s{T + 4}",
      f"s_addc_u32 s{T + 7}, s{T + 7}, s{T + 5}",
      f"s_lshl_b32 s{T + 8}, {s(S_WAVE)}, 13",          # 8 KB w: the wave's column blocks
      f"s_lshl_b32 s{T + 9}, {s(S_WAVE)}, 9",           # 512 B w: the wave's quarter of the table
      f"v_lshlrev_b32 {vreg(off)}, 4, {vreg(V_LANE)}",
      f"v_lshlrev_b32 {vreg(offt)}, 3, {vreg(V_R16)}")
    for j in range(4):
        b = T + 12 + j
        # values: out + 1024 row + 8 KB w; descales: table + 16 row - 12 (row & 127) + 512 w
        a(f"s_lshl_b32 s{T + 16}, s{b}, 10",
          f"s_lshr_b32 s{T + 17}, s{b}, 22",
          f"s_add_u32 s{T + 16}, s{T + 16}, s{T + 8}",
          f"s_addc_u32 s{T + 17}, s{T + 17}, 0",
          f"s_add_u32 s{T + 16}, s{T + 16}, s{T + 4}",
          f"s_addc_u32 s{T + 17}, s{T + 17}, s{T + 5}",
          f"s_and_b32 s{T + 10}, s{b}, 127",
          f"s_mul_i32 s{T + 10}, s{T + 10}, 12",
          f"s_lshl_b32 s{T + 11}, s{b}, 4",
          f"s_sub_u32 s{T + 11}, s{T + 11}, s{T + 10}",
          f"s_add_u32 s{T + 11}, s{T + 11}, s{T + 9}",
          f"s_add_u32 s{T + 18}, s{T + 6}, s{T + 11}",
          f"s_addc_u32 s{T + 19}, s{T + 7}, 0")
        for cb in range(8):
            for h in range(2):
                o = (8 * cb + 2 * j + h) * 4
                for i in range(4):
                    a(f"v_accvgpr_read_b32 {vreg(vals[8 * cb + 4 * h + i])}, a{o + i}")
        for cb in range(8):
            for h in range(2):
                o = (8 * cb + 2 * j + h) * 4
                for i in range(4):
                    a(f"v_accvgpr_write_b32 a{o + i}, 0")
        for h, m in ((0, m0), (1, m1)):
            lane_abs_max(a, m, [vals[8 * cb + 4 * h + i] for cb in range(8) for i in range(4)])
            xor_reduce(a, m, "v_max_f32", t0, t1)
            f16_scale(a, m, inv[2 * j + h], t)
        # descales of rows 32j + r16 (a = 0) and + 16 (a = 1), lanes g == 0
        a(f"v_cmp_eq_u32 vcc, 0, {vreg(V_G)}",
          f"s_and_saveexec_b64 {sp(S_EXEC)}, vcc",
          f"global_store_dwordx2 {vreg(offt)}, {vr(m0, 2)}, s[{T + 18}:{T + 19}] sc0 sc1",
          f"s_mov_b64 exec, {sp(S_EXEC)}")
        for cb in range(8):
            for h in range(2):
                for i in range(4):
                    r = vals[8 * cb + 4 * h + i]
                    a(f"v_mul_f32 {vreg(r)}, {vreg(r)}, {vreg(inv[2 * j + h])}")
        for cb in range(8):
            v0 = vals[8 * cb]
            for k in range(4):
                a(f"v_cvt_pk_f16_f32 {vreg(v0 + k)}, {vreg(v0 + 2 * k)}, {vreg(v0 + 2 * k + 1)}")
            if cb == 4:
                a(f"s_add_u32 s{T + 16}, s{T + 16}, 4096", f"s_addc_u32 s{T + 17}, s{T + 17}, 0")
            a(f"global_store_dwordx4 {vreg(off)}, {vr(v0, 4)}, s[{T + 16}:{T + 17}] offset:{1024 * (cb % 4)} sc0 sc1")


def epi_store_split(a, hb, cb, vv, inv, operands):
    """O[cb][hb] / l -> one 16-byte store per lane; the accumulators are
    cleared for the next segment as they are read (under the store issue)."""
    o = (8 * cb + hb) * 4
    for i in range(4):
        a(f"v_accvgpr_read_b32 {vreg(vv[i])}, a{o + i}")
    for i in range(4):
        a(f"v_accvgpr_write_b32 a{o + i}, 0")
    for i in range(4):
        a(f"v_mul_f32 {vreg(vv[i])}, {vreg(vv[i])}, {vreg(inv)}")
    # system scope: written through the L2, which then holds no dirty output
    # lines for the end of the kernel to write back (the merge reads them next)
    a("global_store_dwordx4 " + operands.format(v=vr(vv[0], 4)) + " sc0 sc1")


def epi_store(a, h, cb, vv, inv, operands):
    """O[cb][h] * inv -> one 16-byte store per lane."""
    o = (2 * cb + h) * 4
    for i in range(4):
        a(f"v_accvgpr_read_b32 {vreg(vv[i])}, a{o + i}")
    a("s_nop 1")
    for i in range(4):
        a(f"v_mul_f32 {vreg(vv[i])}, {vreg(vv[i])}, {vreg(inv)}")
    a("global_store_dwordx4 " + operands.format(v=vr(vv[0], 4)))


def emit_t(a, dst, q, tmp):
    """dst = t(q) = 2 (q & 3) + (q >> 2) for 0 <= q < 8: the chunk swizzle of a
    row within its 8-row block."""
    a(f"v_and_b32 {vreg(tmp)}, 3, {vreg(q)}",
      f"v_lshrrev_b32 {vreg(dst)}, 2, {vreg(q)}",
      f"v_lshl_or_b32 {vreg(dst)}, {vreg(tmp)}, 1, {vreg(dst)}")


def lane_constants(a):
    """Per-lane offsets of the tile layout.  A page tile is 9 x 8 blocks of
    1 KB: block (K, R) at (8K + R) KB holds rows 8R..8R+7, chunks 8K..8K+7
    (chunk = 8 bf16); row r sits at 128 (r % 8) in its block and chunk c at
    16 ((c % 8) ^ tp(r)), tp(r) = t(r % 8) ^ 2 ((r / 8) % 2).  The swizzle puts
    the 16 rows of a score read and the 4 rows x 2 chunks of a transposed read
    on distinct bank groups."""
    g, j = V_G, V_R16
    t0, t1, t2, t3 = V_T, V_T + 1, V_T + 2, V_T + 3
    u0, u1, u2, u3 = V_S[0], V_S[0] + 1, V_S[0] + 2, V_S[0] + 3
    # score reads: lane (g, j) reads row j, chunk g of a 16-row tile -> j*128 + 16 (g ^ tp(j))
    a(f"v_and_b32 {vreg(t0)}, 7, {vreg(j)}")
    emit_t(a, t1, t0, t2)
    a(f"v_lshrrev_b32 {vreg(t2)}, 2, {vreg(j)}",
      f"v_and_b32 {vreg(t2)}, 2, {vreg(t2)}",
      f"v_xor_b32 {vreg(t1)}, {vreg(t1)}, {vreg(t2)}",
      f"v_xor_b32 {vreg(t1)}, {vreg(g)}, {vreg(t1)}",
      f"v_lshlrev_b32 {vreg(t1)}, 4, {vreg(t1)}",
      f"v_lshl_add_u32 {vreg(V_QKE)}, {vreg(j)}, 7, {vreg(t1)}",
      f"v_xor_b32 {vreg(V_QKO)}, 64, {vreg(V_QKE)}")
    # transposed reads: source lane j of group g supplies row 4g + (j >> 2) (+16 for the
    # second read), columns 4 (j & 3) .. +3 of a 16-column block:
    #   r8 = 4 (g & 1) + (j >> 2), tpp = t(r8) ^ (g & 2), e = (j >> 1) & 1
    #   pv0 = 1024 (g >> 1) + 128 r8 + 16 (e ^ tpp) + 8 (j & 1)
    a(f"v_and_b32 {vreg(t0)}, 1, {vreg(g)}",
      f"v_lshrrev_b32 {vreg(t1)}, 2, {vreg(j)}",
      f"v_lshl_or_b32 {vreg(t0)}, {vreg(t0)}, 2, {vreg(t1)}")      # r8
    emit_t(a, t1, t0, t2)
    a(f"v_and_b32 {vreg(t2)}, 2, {vreg(g)}",
      f"v_xor_b32 {vreg(t1)}, {vreg(t1)}, {vreg(t2)}",              # tpp
      f"v_bfe_u32 {vreg(t2)}, {vreg(j)}, 1, 1",                      # e
      f"v_xor_b32 {vreg(t1)}, {vreg(t1)}, {vreg(t2)}",
      f"v_lshlrev_b32 {vreg(t1)}, 4, {vreg(t1)}",
      f"v_lshl_add_u32 {vreg(t1)}, {vreg(t0)}, 7, {vreg(t1)}",
      f"v_and_b32 {vreg(t2)}, 1, {vreg(j)}",
      f"v_lshl_add_u32 {vreg(t1)}, {vreg(t2)}, 3, {vreg(t1)}",
      f"v_lshrrev_b32 {vreg(t2)}, 1, {vreg(g)}",
      f"v_lshl_add_u32 {vreg(V_PV0)}, {vreg(t2)}, 10, {vreg(t1)}")
    # loader: lane L of a block load writes row-in-block lr = L >> 3 and slot lx = L & 7,
    # i.e. chunk lx ^ t(lr) (even row groups) or that ^ 2 (odd ones)
    T = S_TMP
    a(f"v_lshrrev_b32 {vreg(u0)}, 3, {vreg(V_LANE)}",                # lr
      f"v_and_b32 {vreg(u1)}, 7, {vreg(V_LANE)}")                    # lx
    emit_t(a, u2, u0, u3)
    a(f"v_xor_b32 {vreg(u2)}, {vreg(u1)}, {vreg(u2)}",
      f"v_lshlrev_b32 {vreg(V_LCA)}, 4, {vreg(u2)}",
      f"v_xor_b32 {vreg(V_LCB)}, 32, {vreg(V_LCA)}",
      f"s_mul_i32 s{T}, {s(S_WAVE)}, {16 * 1152}",
      f"v_mul_u32_u24 {vreg(u3)}, {1152}, {vreg(u0)}",
      f"v_add_u32 {vreg(u3)}, s{T}, {vreg(u3)}",                      # row term of row 16w + lr
      f"v_add_u32 {vreg(V_LDA)}, {vreg(u3)}, {vreg(V_LCA)}",
      f"v_add_u32 {vreg(V_LDB)}, {vreg(u3)}, {vreg(V_LCB)}",
      f"v_add_u32 {vreg(V_LDB)}, {8 * 1152}, {vreg(V_LDB)}",
      f"s_lshl_b32 s{T}, {s(S_WAVE)}, 4",
      f"v_add_u32 {vreg(V_LDROW)}, s{T}, {vreg(u0)}")


def flag_write(a, value, all_waves=False):
    """Write the restart flag (wave 0 only unless all_waves)."""
    skip = a.new_label("flagw")
    if not all_waves:
        a(f"s_cmp_eq_u32 {s(S_WAVE)}, 0",
          f"s_cbranch_scc0 {skip}")
    a(f"v_mov_b32 {vreg(V_T)}, {value}",
      f"v_mov_b32 {vreg(V_T + 1)}, {FLAG_ADDR}",
      f"ds_write_b32 {vreg(V_T + 1)}, {vreg(V_T)}")
    a.label(skip)


def flag_check(a):
    """After a barrier: restart the segment if any wave raised the flag."""
    a(f"v_mov_b32 {vreg(V_T)}, {FLAG_ADDR}",
      f"ds_read_b32 {vreg(V_T)}, {vreg(V_T)}",
      s_waitcnt_lgkm(0),
      "s_nop 1",
      f"v_readfirstlane_b32 s{S_TMP}, {vreg(V_T)}",
      f"s_cmp_eq_u32 s{S_TMP}, 0",
      "s_cbranch_scc0 .Lrestart")


def unit_body_fp8(a):
    """One unit of the fp8 kernel up to the unit-end label (returned)."""
    T = S_TMP
    a.label(".Lunit")
    a(f"s_mov_b64 {sp(S_OVF)}, 0",
      f"s_sub_u32 {s(S_SLOT)}, {s(S_UCUR)}, {s(S_UA)}",
      f"s_and_b32 {s(S_SLOT)}, {s(S_SLOT)}, 1")
    # this unit's raw pages have landed (own loads), the table prefetch too,
    # and every wave is past the previous unit (the tile is free)
    a(s_waitcnt_vm(0), s_waitcnt_lgkm(0), "s_barrier")
    a(f"v_mov_b32 {vreg(V_T)}, {FLAG_ADDR}",
      f"ds_read_b32 {vreg(V_T)}, {vreg(V_T)}",         # restart flag, checked below
      f"s_mov_b32 {s(S_CURVALID)}, {s(S_NVALID)}")
    take_prefetched(a)
    loader_page_fp8(a)
    a(f"s_add_u32 s{T + 19}, {s(S_UCUR)}, 1")
    prefetch_next(a, T + 19)
    dqfull, dqdone = a.new_label("dqfull"), a.new_label("dqdone")
    a(f"s_cmp_ge_i32 {s(S_CURVALID)}, 64",
      f"s_cbranch_scc1 {dqfull}")
    dequant_fp8(a, masked=True)
    a(f"s_branch {dqdone}")
    a.label(dqfull)
    dequant_fp8(a, masked=False)
    a.label(dqdone)
    # the next unit's raw pages: issued after the widening, whose LDS work
    # then never waits behind these loads at issue (2-3% on the long-context
    # workload)
    a(f"s_xor_b32 s{T + 21}, {s(S_SLOT)}, 1")
    dma_fp8(a, T + 21)
    a(s_waitcnt_lgkm(0), "s_barrier",
      "s_nop 1",
      f"v_readfirstlane_b32 s{T}, {vreg(V_T)}",
      f"s_cmp_eq_u32 s{T}, 0",
      "s_cbranch_scc0 .Lrestart")
    a(f"s_sub_u32 {s(S_ROW0)}, {s(S_UCUR)}, {s(S_CPRE)}",
      f"s_lshl_b32 {s(S_ROW0)}, {s(S_ROW0)}, 6",
      f"v_mov_b32 {vreg(V_UQ)}, {vreg(V_QKE)}",
      f"v_mov_b32 {vreg(V_UQ + 1)}, {vreg(V_QKO)}",
      f"v_add_u32 {vreg(V_UQ + 2)}, 0x10000, {vreg(V_QKE)}",
      f"v_add_u32 {vreg(V_UQ + 3)}, 0x10000, {vreg(V_QKO)}",
      f"v_mov_b32 {vreg(V_UP)}, {vreg(V_PV0)}")
    for m in range(1, 4):
        a(f"v_xor_b32 {vreg(V_UP + m)}, {32 * m}, {vreg(V_PV0)}")
    half, uend, classic = (a.new_label(x) for x in ("half", "uend", "classic"))
    a(f"s_sub_i32 s{T}, {s(S_NVIS)}, {s(S_ROW0)}",
      f"s_cmp_le_i32 s{T}, 0",
      f"s_cbranch_scc1 {uend}",
      f"s_cmp_le_i32 s{T}, 32",
      f"s_cbranch_scc1 {half}",
      f"s_cmp_lt_i32 s{T}, 64",
      f"s_cbranch_scc1 {classic}",
      f"s_max_u32 s{T + 1}, {s(S_UA)}, {s(S_CPRE)}",
      f"s_cmp_eq_u32 {s(S_UCUR)}, s{T + 1}",
      f"s_cbranch_scc1 {classic}",
      f"s_cmp_eq_u32 {s(S_EXACT)}, 0",
      f"s_cbranch_scc0 {classic}")
    for ss in range(2):
        substep_fp8(a, ss, lean=True)
    a(f"s_branch {uend}")
    a.label(classic)
    for ss in range(2):
        substep_fp8(a, ss, lean=False)
    a(f"s_branch {uend}")
    a.label(half)
    substep_fp8(a, 0, lean=False)
    return uend


# ======================================================= bf16: half-page steps
# The bf16 kernel works in steps of 32 rows (half a page).  LDS holds four
# half-page tiles (9 x 4 blocks of 1 KB: block (K, R) at (4K + R) KB holds rows
# 8R..8R+7, chunks 8K..8K+7, swizzled as in the page tile) and two 8 KB
# probability buffers.  Step t reads tile t % 4 for its scores, tile
# (t - 1) % 4 for the output of step t - 1, publishes its probabilities in
# buffer t % 2 and issues the loads of step t + 2 into tile (t + 2) % 4, which
# step t - 2 (output done during step t - 1) has freed.  One barrier per step.
HS_BYTES = 32 * 1152
PB_BYTES = 8192
H_S = 16                          # S[tb][h] at 16 + (2tb + h) * 4; packed P at 16 + 4h after the softmax
H_SMT = (32, 33, 34, 35)          # softmax scratch
H_A, H_NA = 36, 4                 # score-operand ring (v36..v51)
H_PF = tuple(range(52, 84, 4))    # probability fragments of the previous step, one per 16-row block
H_B, H_NB = 84, 3                 # output-operand ring (v84..v95)
V_PXR = 106                       # P_BASE + 16 lane + 8192 ((t - 1) % 2): the previous step's fragments
V_LDZ = 105                       # source offset of a load lane whose row holds no data (row 0 of the half)
V_DMAS = V_T + 1                  # source offsets of this wave's loads of the next step (masked)
S_T, S_TL, S_PH, S_NSTEP = 92, 93, 94, 96   # step of the partition, of the segment; half-page address; steps
S_PNONE = 51                      # 1: the previous step had no visible row (its output is skipped:
                                  # the rows of its tile may lie past the sequence's data)
V_PVM = (V_PV0, 98, 99, 107)      # output-read lane offsets of the four 16-column phases of a chunk group
# values of the next step, computed during the current one (scalar temporaries the
# steps leave alone; the epilogue does not, so a segment start recomputes them)
N_PH, N_STEP, N_NVH, N_ROW0, N_MODE, N_DMALDS = 70, 72, 74, 75, 76, 77
S_LKUP = 3                        # page to look up (the loader items' own; s3 holds nothing else)
S_EPI = 50                        # 1 / 2: the segment follows an epilogue of final rows / of a
                                  # partial (its Q loads went out before that epilogue's stores)
EPI_STORES_ROWS, EPI_STORES_PARTIAL = 66, 38
# The cache rows are read once per launch: their direct-to-LDS loads are
# nontemporal (streaming), which measured 2-5% faster than the default policy.
ROW_LOAD_POLICY = " nt"
DMA_EARLY = 9                     # > 0: the loads of step t + 2 go out over fragments 0..DMA_EARLY
PV_INTERLEAVE = 3                 # output fragments of step t - 1 placed among the score fragments of step t
P_GATHER_AT = (1, 1, 2, 2, 3, 3, 4, 4)   # score fragments after which the 8 probability reads go out
PV_READ_LEAD = 6                  # score fragment after which the first output-operand reads go out


def lane_constants_hp(a):
    """bf16 step constants (after lane_constants): wave w loads row group w
    of a half page (rows 8w + lr, lr = lane >> 3), V_LDA its source offset
    in the half page, V_LDZ that of row 0 (rows past the data); the wave's
    output columns 128w .. in V_PV0 (8 KB per 128 columns of a half tile);
    the exchange-buffer lane address V_PX."""
    T = S_TMP
    u0, u3 = V_S[0], V_S[0] + 3
    a(f"v_lshrrev_b32 {vreg(u0)}, 3, {vreg(V_LANE)}",
      f"s_and_b32 s{T}, {s(S_WAVE)}, 1",
      f"s_lshl_b32 s{T}, s{T}, 5",
      f"v_xor_b32 {vreg(V_LDZ)}, s{T}, {vreg(V_LCA)}",
      f"s_lshl_b32 s{T}, {s(S_WAVE)}, 3",
      f"v_add_u32 {vreg(V_LDROW)}, s{T}, {vreg(u0)}",
      f"v_mul_u32_u24 {vreg(u3)}, 1152, {vreg(V_LDROW)}",
      f"v_add_u32 {vreg(V_LDA)}, {vreg(u3)}, {vreg(V_LDZ)}",
      f"v_lshlrev_b32 {vreg(V_PX)}, 4, {vreg(V_LANE)}",
      f"v_add_u32 {vreg(V_PX)}, {P_BASE}, {vreg(V_PX)}",
      f"s_lshl_b32 s{T}, {s(S_WAVE)}, 13",
      f"v_add_u32 {vreg(V_PV0)}, s{T}, {vreg(V_PV0)}")
    for m in range(1, 4):
        a(f"v_xor_b32 {vreg(V_PVM[m])}, {32 * m}, {vreg(V_PV0)}")


def qk_read_hp(i):
    """A fragment (ks, tb) = divmod(i, 2): rows 16tb + r16 of the half tile, chunk 4ks + g."""
    ks, tb = divmod(i, 2)
    return [f"\tds_read_b128 {{buf}}, {vreg(V_UQ + (ks & 1))} offset:{4096 * (ks >> 1) + 2048 * tb}"]


def pv_read_hp(cb):
    """V^T operand of this wave's column block cb: rows 4g + r, then 16 + 4g + r."""
    off = 4096 * (cb >> 2)
    base = V_UP + (cb & 3)
    return [f"\tds_read_b64_tr_b16 {{lo}}, {vreg(base)} offset:{off}",
            f"\tds_read_b64_tr_b16 {{hi}}, {vreg(base)} offset:{off + 2048}"]


def qk_frags_hp():
    out = []
    for i in range(36):
        ks, tb = divmod(i, 2)
        mf = []
        for h in range(2):
            sreg = H_S + (2 * tb + h) * 4
            qreg = V_Q + (2 * ks + h) * 4
            c = "0" if ks == 0 else vr(sreg, 4)
            mf.append(f"\tv_mfma_f32_16x16x32_bf16 {vr(sreg, 4)}, {{buf}}, {vr(qreg, 4)}, {c}")
        out.append(Frag("A", H_A, H_NA, i, qk_read_hp(i), mf))
    return out


def pv_frags_hp():
    """Output of the previous step: fragment cb (this wave's columns 16cb ..)
    times the probability fragment of every 16-row block hb of query rows."""
    out = []
    for cb in range(8):
        mf, deps = [], []
        for hb in range(8):
            o = (8 * cb + hb) * 4
            mf.append(f"\tv_mfma_f32_16x16x32_bf16 {ar(o, 4)}, {{buf}}, {vr(H_PF[hb], 4)}, {ar(o, 4)}")
            deps.append((("pf", hb),))
        out.append(Frag("B", H_B, H_NB, cb, pv_read_hp(cb), mf, deps))
    return out


def p_gather_hp():
    """Events: the previous step's probability fragments of all query rows."""
    return [("lds", f"\tds_read_b128 {vr(H_PF[hb], 4)}, {vreg(V_PXR)} offset:{1024 * hb}", ("pf", hb))
            for hb in range(8)]


def p_publish_hp():
    """This wave's packed probabilities (fragments 2w, 2w + 1 of its buffer)."""
    return [f"\tds_write_b128 {vreg(V_PXW)}, {vr(H_S + 4 * h, 4)} offset:{1024 * h}" for h in range(2)]


def dma_groups_hp():
    """The 9 direct-to-LDS loads of this wave for one half page: row group
    w, chunk groups K = 0..8 (one 8-row x 8-chunk block each)."""
    groups = []
    for k in range(9):
        groups.append([f"\ts_add_u32 s{S_DPAGE}, s{S_PH}, {128 * k}",
                       f"\ts_addc_u32 s{S_DPAGE + 1}, s{S_PH + 1}, 0",
                       f"\ts_add_u32 m0, {s(S_DMALDS)}, {4096 * k}",
                       "\ts_nop 0",
                       f"\tglobal_load_lds_dwordx4 {vreg(V_DMAS)}, {sp(S_DPAGE)}{ROW_LOAD_POLICY}"])
    return groups


def dma_setup_hp(a, half, step_sgpr):
    """Loads of half `half` of page S_PAGE (S_NVALID rows hold data) into the
    tile of step s[step_sgpr]: lane source offsets (row 0 of the half for rows
    past the data), LDS base, half-page address."""
    T = S_TMP
    a(f"s_sub_i32 s{T + 6}, {s(S_NVALID)}, {32 * half}",
      f"v_cmp_gt_i32 vcc, s{T + 6}, {vreg(V_LDROW)}",
      f"s_and_b32 s{T + 7}, s{step_sgpr}, 3",
      f"s_mul_i32 {s(S_DMALDS)}, s{T + 7}, {HS_BYTES}",
      f"s_lshl_b32 s{T + 7}, {s(S_WAVE)}, 10",
      f"s_add_u32 {s(S_DMALDS)}, {s(S_DMALDS)}, s{T + 7}",
      f"v_cndmask_b32 {vreg(V_DMAS)}, {vreg(V_LDZ)}, {vreg(V_LDA)}, vcc",
      f"s_add_u32 s{S_PH}, s{S_PAGE}, {HS_BYTES * half}",
      f"s_addc_u32 s{S_PH + 1}, s{S_PAGE + 1}, 0")


def _atomic(lines):
    """Instruction lines (an Asm's) -> one filler item kept together."""
    return [list(lines)]


def take_items(n_sgpr):
    """Filler items, loader side of step n (= s[n_sgpr]): the loads issued in
    step n are those of step n + 2, page UA + ((n + 2) >> 1), half n & 1.  For
    even n that page is new: take its prefetched rows / entry and address."""
    T = S_TMP
    return [["\ts_bitcmp1_b32 s%d, 0" % n_sgpr,
             f"\ts_cselect_b32 {s(S_NVALID)}, {s(S_NVALID)}, {s(S_NV2)}",
             f"\ts_cselect_b32 {s(S_ENTRY)}, {s(S_ENTRY)}, {s(S_ENT2)}"],
            f"\ts_mul_i32 s{T + 4}, {s(S_ENTRY)}, {PAGE_BYTES}",
            f"\ts_mul_hi_u32 s{T + 5}, {s(S_ENTRY)}, {PAGE_BYTES}",
            [f"\ts_add_u32 s{T + 4}, {s(S_ROWS)}, s{T + 4}",
             f"\ts_addc_u32 s{T + 5}, {s(S_ROWS + 1)}, s{T + 5}"],
            [f"\ts_cmp_gt_i32 {s(S_NVALID)}, 0",
             f"\ts_cselect_b64 {sp(S_PAGE)}, s[{T + 4}:{T + 5}], {sp(S_ROWS)}"]]


def lookup_items(u_sgpr):
    """Filler items: look up page u (= s[u_sgpr], may lie past the partition):
    S_NV2 = its rows holding data (0 past the partition), S_ENT2 = its page
    (for a paged cache a scalar load left in flight: read only after a later
    lgkmcnt(0)).  The loader cursor moves to the sequence of min(u, UB - 1)."""
    T = S_TMP
    items = [f"\ts_sub_u32 s{T + 3}, {s(S_UB)}, 1",
             f"\ts_min_u32 s{T + 19}, s{u_sgpr}, s{T + 3}"]
    a2 = Asm()
    loader_advance(a2, T + 19)
    items += _atomic(a2.lines)
    skip = Asm().new_label("pfskip")
    items += [f"\ts_sub_u32 s{T + 1}, s{T + 19}, {s(S_LPRE)}",
              f"\ts_lshl_b32 s{T + 2}, s{T + 1}, 6",
              f"\ts_sub_i32 {s(S_NV2)}, {s(S_LLEN)}, s{T + 2}",
              f"\ts_min_i32 {s(S_NV2)}, {s(S_NV2)}, 64",
              f"\ts_mul_i32 s{T + 4}, {s(S_LSEQ)}, {s(S_MAXB)}",
              f"\ts_add_u32 {s(S_ENT2)}, s{T + 4}, s{T + 1}",
              [f"\ts_cmp_lt_u32 s{u_sgpr}, {s(S_UB)}",
               f"\ts_cselect_b32 {s(S_NV2)}, {s(S_NV2)}, 0"],
              [f"\ts_cmp_gt_i32 {s(S_NV2)}, 0",
               f"\ts_cbranch_scc0 {skip}",
               f"\ts_cmp_eq_u64 {sp(S_TABLE)}, 0",
               f"\ts_cbranch_scc1 {skip}",
               f"\ts_lshl_b32 s{T + 5}, {s(S_ENT2)}, 2",
               f"\ts_load_dword {s(S_ENT2)}, {sp(S_TABLE)}, s{T + 5}",
               f"{skip}:"]]
    return items


def loader_items(n_sgpr):
    """take_items(n), then the lookup of the page after the loads' page
    (every step; an odd step repeats the even one's)."""
    T = S_TMP
    return (take_items(n_sgpr) +
            [f"\ts_lshr_b32 s{S_LKUP}, s{n_sgpr}, 1",
             f"\ts_add_u32 s{S_LKUP}, s{S_LKUP}, {s(S_UA)}",
             f"\ts_add_u32 s{S_LKUP}, s{S_LKUP}, 2"] + lookup_items(S_LKUP))


def next_items(n_sgpr, tl_first):
    """Filler items: the values step n (= s[n_sgpr]) starts from (N_*): its
    loads (half page, LDS base, rows holding data), its first row in the
    sequence and its kind (tl_first: n is a segment's first step)."""
    T = S_TMP
    n = n_sgpr
    items = [f"\ts_and_b32 s{T + 6}, s{n}, 1",                       # half of the loads / buffer parity
             f"\ts_mul_i32 s{T + 7}, s{T + 6}, {HS_BYTES}",
             [f"\ts_add_u32 s{N_PH}, s{S_PAGE}, s{T + 7}",
              f"\ts_addc_u32 s{N_PH + 1}, s{S_PAGE + 1}, 0"],
             f"\ts_lshl_b32 s{T + 7}, s{T + 6}, 5",
             f"\ts_sub_i32 s{N_NVH}, {s(S_NVALID)}, s{T + 7}",
             f"\ts_add_u32 s{T + 7}, s{n}, 2",
             f"\ts_and_b32 s{T + 7}, s{T + 7}, 3",
             f"\ts_mul_i32 s{N_DMALDS}, s{T + 7}, {HS_BYTES}",
             f"\ts_lshl_b32 s{T + 7}, {s(S_WAVE)}, 10",
             f"\ts_add_u32 s{N_DMALDS}, s{N_DMALDS}, s{T + 7}",
             # first row of the step in its sequence: 64 (page - first page of the sequence) + 32 half
             f"\ts_lshr_b32 s{N_ROW0}, s{n}, 1",
             f"\ts_add_u32 s{N_ROW0}, s{N_ROW0}, {s(S_UA)}",
             f"\ts_sub_u32 s{N_ROW0}, s{N_ROW0}, {s(S_CPRE)}",
             f"\ts_lshl_b32 s{N_ROW0}, s{N_ROW0}, 1",
             f"\ts_add_u32 s{N_ROW0}, s{N_ROW0}, s{T + 6}",
             f"\ts_lshl_b32 s{N_ROW0}, s{N_ROW0}, 5",
             # kind: 0 none (no query token of the workgroup sees a row of it),
             # 3 lean (every token sees all 32 rows, not a segment's first step,
             # no restart), else 2 classic
             f"\ts_sub_i32 s{T + 8}, {s(S_NVHI)}, s{N_ROW0}",
             f"\ts_sub_i32 s{T + 9}, {s(S_NVLO)}, s{N_ROW0}",
             f"\ts_mov_b32 s{N_MODE}, {2 if tl_first else 3}",
             [f"\ts_cmp_lt_i32 s{T + 9}, 32",
              f"\ts_cselect_b32 s{N_MODE}, 2, s{N_MODE}"],
             [f"\ts_cmp_lg_u32 {s(S_EXACT)}, 0",
              f"\ts_cselect_b32 s{N_MODE}, 2, s{N_MODE}"],
             [f"\ts_cmp_le_i32 s{T + 8}, 0",
              f"\ts_cselect_b32 s{N_MODE}, 0, s{N_MODE}"]]
    return items


def pre_step_items():
    """Filler items of a step: everything the next step starts from."""
    return ([f"\ts_add_u32 s{N_STEP}, {s(S_T)}, 1"] + loader_items(N_STEP) + next_items(N_STEP, False))


def flatten(items):
    out = []
    for x in items:
        out += x if isinstance(x, list) else [x]
    return out


def step_body_hp(a, kind, with_pv):
    """kind: 'lean' | 'classic' | 'none'.  Scores and softmax of this step
    (none: P = 0), the output of the previous step (with_pv), the loads of
    step t + 2, the values the next step starts from, the publication of this
    step's probabilities."""
    qk = qk_frags_hp() if kind != "none" else []
    pv = pv_frags_hp() if with_pv else []
    groups = [list(g) for g in dma_groups_hp()]
    pre = pre_step_items()
    if kind == "none":
        a(*[f"v_mov_b32 {vreg(H_S + i)}, 0" for i in range(8)])
    if qk and pv:
        # scores interleaved with the first PV_INTERLEAVE output fragments
        # (balances the LDS traffic), the other output fragments carry the softmax
        k = PV_INTERLEAVE
        cut = [36 * j // (k + 1) for j in range(k + 2)]
        order = []
        for j in range(k + 1):
            order += qk[cut[j]:cut[j + 1]] + ([pv[j]] if j < k else [])
        order += pv[k:]
        tail = order.index(pv[k])
        sm = (softmax_lean if kind == "lean" else softmax_code)(0, S=H_S, P=H_S, tmp=H_SMT)
        # the softmax starts one fragment after the last score MFMA (MFMA
        # results -> VALU); the load groups stay whole (their carry chains)
        if DMA_EARLY:
            fillers = [(0, DMA_EARLY, groups), (0, tail - 1, pre),
                       (tail + 1, len(order) - 1, merge_filler(sm, []))]
        else:
            fillers = [(0, tail - 1, pre),
                       (tail, tail, groups[:2]),
                       (tail + 1, len(order) - 1, merge_filler(sm, groups[2:]))]
        # the previous step's probabilities and the first output operands are read
        # a few score fragments in, behind the first score operands: LDS reads
        # complete in order, and read at the step's top they would hold up the
        # score MFMAs (2-3% on the MTP workload)
        assert max(P_GATHER_AT) < PV_READ_LEAD < order.index(pv[0])
        events = {len(order) - 1: p_publish_hp()}
        for pos, item in zip(P_GATHER_AT, p_gather_hp()):
            events.setdefault(pos, []).append(item)
        emit_stream(a, order, {"A": -1, "B": PV_READ_LEAD}, fillers, events,
                    marks={tail - 1: 1, len(order) - 1: 2})
    elif qk:
        emit_stream(a, qk, {"A": -1}, [(0, 35, groups), (0, 35, pre)])
        a("s_nop 7", "s_nop 7", "s_nop 3")   # MFMA results -> VALU
        a.lines += (softmax_lean if kind == "lean" else softmax_code)(0, S=H_S, P=H_S, tmp=H_SMT)
        a.lines += p_publish_hp()
    elif pv:
        emit_stream(a, pv, {"B": -1}, [(0, 7, groups), (0, 7, pre)], {-1: p_gather_hp(), 7: p_publish_hp()})
    else:
        a.lines += flatten(groups) + flatten(pre)
        a.lines += p_publish_hp()


def drain_hp(a):
    """The output of a segment's last step (its probabilities published
    before the barrier), unless that step had no visible row."""
    skip = a.new_label("nodrain")
    a(f"s_cmp_lg_u32 {s(S_PNONE)}, 0",
      f"s_cbranch_scc1 {skip}",
      s_waitcnt_lgkm(0), "s_barrier")
    drain_bases_hp(a)
    pv = pv_frags_hp()
    emit_stream(a, pv, {"B": -1}, [], {-1: p_gather_hp()})
    a.label(skip)


def step_hp(a):
    """One step: take the precomputed values, wait for this step's rows and
    for every wave, run the body for the step's kind."""
    T = S_TMP
    a.label(".Lstep")
    a(f"s_mov_b32 {s(S_ROW0)}, s{N_ROW0}",
      f"s_mov_b32 {s(S_MODE)}, s{N_MODE}",
      f"s_mov_b64 {sp(S_PH)}, s[{N_PH}:{N_PH + 1}]",
      f"s_mov_b32 {s(S_DMALDS)}, s{N_DMALDS}",
      # this step's tile, the previous step's; this step's probability buffer (plus
      # the wave's fragments), the previous step's
      f"s_and_b32 s{T}, {s(S_T)}, 3",
      f"s_mul_i32 s{T}, s{T}, {HS_BYTES}",
      f"s_add_u32 s{T + 1}, {s(S_T)}, 3",
      f"s_and_b32 s{T + 1}, s{T + 1}, 3",
      f"s_mul_i32 s{T + 1}, s{T + 1}, {HS_BYTES}",
      f"s_and_b32 s{T + 2}, {s(S_T)}, 1",
      f"s_lshl_b32 s{T + 2}, s{T + 2}, 13",
      f"s_lshl_b32 s{T + 3}, {s(S_WAVE)}, 11",
      f"s_add_u32 s{T + 3}, s{T + 3}, s{T + 2}",
      f"s_xor_b32 s{T + 2}, s{T + 2}, {PB_BYTES}",
      f"v_add_u32 {vreg(V_UQ)}, s{T}, {vreg(V_QKE)}",
      f"v_add_u32 {vreg(V_UQ + 1)}, s{T}, {vreg(V_QKO)}",
      *[f"v_add_u32 {vreg(V_UP + m)}, s{T + 1}, {vreg(V_PVM[m])}" for m in range(4)],
      f"v_add_u32 {vreg(V_PXW)}, s{T + 3}, {vreg(V_PX)}",
      f"v_add_u32 {vreg(V_PXR)}, s{T + 2}, {vreg(V_PX)}",
      f"v_cmp_gt_i32 vcc, s{N_NVH}, {vreg(V_LDROW)}",
      f"v_cndmask_b32 {vreg(V_DMAS)}, {vreg(V_LDZ)}, {vreg(V_LDA)}, vcc")
    # this step's rows have landed (the next step's nine loads may still be in
    # flight; a segment's first step also waits for its Q loads)
    w0, wdone = a.new_label("w0"), a.new_label("wdone")
    a(f"s_cmp_eq_u32 {s(S_TL)}, 0",
      f"s_cbranch_scc1 {w0}",
      s_waitcnt_vm(9),
      f"s_branch {wdone}")
    a.label(w0)
    # a segment's first step: Q and this step's rows.  After an epilogue, the
    # stores that went out after the Q loads may stay outstanding (at most 63
    # of the 66 of final rows, all 38 of a partial); else nothing
    wz, wpart = a.new_label("wz"), a.new_label("wpart")
    a(f"s_cmp_eq_u32 {s(S_EPI)}, 0",
      f"s_cbranch_scc1 {wz}",
      f"s_cmp_eq_u32 {s(S_EPI)}, 2",
      f"s_cbranch_scc1 {wpart}",
      s_waitcnt_vm(min(63, EPI_STORES_ROWS)),
      f"s_branch {wdone}")
    a.label(wpart)
    a(s_waitcnt_vm(EPI_STORES_PARTIAL),
      f"s_branch {wdone}")
    a.label(wz)
    a(s_waitcnt_vm(0))
    a.label(wdone)
    a(s_waitcnt_lgkm(0), "s_barrier")
    first, notlean, nonepv, nonefirst, send = (a.new_label(x) for x in
                                               ("first", "notlean", "nonepv", "nonefirst", "send"))
    # steps without visible rows come last in a segment: after the first of
    # them (whose output of the step before it is still due) none has an output
    a(f"s_cmp_eq_u32 {s(S_TL)}, 0",
      f"s_cbranch_scc1 {first}",
      f"s_cmp_lg_u32 {s(S_PNONE)}, 0",
      f"s_cbranch_scc1 {nonefirst}",
      f"s_cmp_lt_u32 {s(S_MODE)}, 3",
      f"s_cbranch_scc1 {notlean}")
    step_body_hp(a, "lean", True)
    a(f"s_branch {send}")
    a.label(notlean)
    a(f"s_cmp_eq_u32 {s(S_MODE)}, 0",
      f"s_cbranch_scc1 {nonepv}")
    step_body_hp(a, "classic", True)
    a(f"s_branch {send}")
    a.label(nonepv)
    step_body_hp(a, "none", True)
    a(f"s_branch {send}")
    a.label(first)
    a(f"s_cmp_eq_u32 {s(S_MODE)}, 0",
      f"s_cbranch_scc1 {nonefirst}")
    step_body_hp(a, "classic", False)
    a(f"s_branch {send}")
    a.label(nonefirst)
    step_body_hp(a, "none", False)
    a.label(send)
    a(f"s_cmp_eq_u32 {s(S_MODE)}, 0",
      f"s_cselect_b32 {s(S_PNONE)}, 1, 0")


def drain_bases_hp(a):
    """Output-read bases of step S_T - 1 (the segment's last step)."""
    T = S_TMP
    a(f"s_add_u32 s{T + 1}, {s(S_T)}, 3",
      f"s_and_b32 s{T + 1}, s{T + 1}, 3",
      f"s_mul_i32 s{T + 1}, s{T + 1}, {HS_BYTES}",
      *[f"v_add_u32 {vreg(V_UP + m)}, s{T + 1}, {vreg(V_PVM[m])}" for m in range(4)],
      f"s_and_b32 s{T + 2}, {s(S_T)}, 1",
      f"s_lshl_b32 s{T + 2}, s{T + 2}, 13",
      f"s_xor_b32 s{T + 2}, s{T + 2}, {PB_BYTES}",
      f"v_add_u32 {vreg(V_PXR)}, s{T + 2}, {vreg(V_PX)}")


def start_loads_hp(a):
    """Loads of the steps S_T, S_T + 1 (page S_UCUR) and the loader state the
    step S_T starts from (kernel start, restart).  The block-table entries of
    page S_UCUR and the next one are fetched together (one wait)."""
    T = S_TMP
    loader_advance(a, S_UCUR)
    loader_lookup(a, S_UCUR, wait=False)
    a(f"s_add_u32 s{S_LKUP}, {s(S_UCUR)}, 1")
    a.lines += flatten(lookup_items(S_LKUP))
    a(s_waitcnt_lgkm(0))
    loader_page(a)
    for half in range(2):
        a(f"s_add_u32 s{T + 8}, {s(S_T)}, {half}")
        dma_setup_hp(a, half, T + 8)
        for g in dma_groups_hp():
            a.lines += g
    a.lines += flatten(loader_items(S_T))


def kernel_tail_hp(a):
    """bf16 kernel after the prologue: loader start, segments of steps,
    restart, end."""
    T = S_TMP
    lane_constants_hp(a)
    a(f"v_mov_b32 {vreg(V_ENT)}, 0")
    a(f"s_mov_b32 {s(S_UCUR)}, {s(S_UA)}",
      f"s_mov_b32 {s(S_T)}, 0",
      f"s_mov_b32 {s(S_EPI)}, 0")
    load_q(a, S_CSEQ)      # Q first: its loads overlap the block-table lookups
    start_loads_hp(a)
    zero_o(a)              # later segments find O cleared by the epilogue
    # ------------------------------------------------ segments
    a.label(".Lseg")
    segment_setup(a, with_q=False, zero=False)
    a(f"s_sub_u32 {s(S_NSTEP)}, {s(S_SEGEND)}, {s(S_UCUR)}",
      f"s_lshl_b32 {s(S_NSTEP)}, {s(S_NSTEP)}, 1",
      f"s_mov_b32 {s(S_TL)}, 0",
      f"s_mov_b32 {s(S_PNONE)}, 0")
    a.lines += flatten(next_items(S_T, True))
    step_hp(a)
    a(f"s_add_u32 {s(S_T)}, {s(S_T)}, 1",
      f"s_add_u32 {s(S_TL)}, {s(S_TL)}, 1",
      f"s_lshr_b32 s{T}, {s(S_T)}, 1",
      f"s_add_u32 {s(S_UCUR)}, {s(S_UA)}, s{T}",
      f"s_cmp_lt_u32 {s(S_TL)}, {s(S_NSTEP)}",
      "s_cbranch_scc1 .Lstep")
    # the scores are done: Q of the next segment (if the partition has one) now,
    # under the last output and the epilogue
    noq = a.new_label("noq")
    a(f"s_cmp_lt_u32 {s(S_UCUR)}, {s(S_UB)}",
      f"s_cbranch_scc0 {noq}",
      f"s_add_u32 s{S_LKUP}, {s(S_CSEQ)}, 1")
    load_q(a, S_LKUP)
    a.label(noq)
    drain_hp(a)
    # end of the segment: every wave past its output reads
    a(s_waitcnt_lgkm(0), "s_barrier")
    epilogue_split(a)
    a(f"s_add_u32 {s(S_CPRE)}, {s(S_CPRE)}, {s(S_CUNITS)}",
      f"s_add_u32 {s(S_CSEQ)}, {s(S_CSEQ)}, 1",
      f"s_cmp_lt_u32 {s(S_UCUR)}, {s(S_UB)}",
      "s_cbranch_scc1 .Lseg",
      "s_branch .Lkernel_end")
    # ------------------------------------------------ restart of the segment
    a.label(".Lrestart")
    a(s_waitcnt_vm(0), "s_barrier")   # every wave has read the requests; no loads in flight
    a(f"s_mov_b64 {sp(S_OVF)}, 0",
      f"s_mov_b32 {s(S_EXACT)}, 1")
    for h in range(2):
        pk, t0, t1 = V_T, V_T + 1, V_T + 2
        a(f"v_mov_b32 {vreg(pk)}, {vreg(V_PEAK[h])}")
        xor_reduce(a, pk, "v_max_f32", t0, t1)
        # the restart comes at the segment's end, after steps that may have
        # moved the reference since the overflow: a head whose lean sub-step
        # overflowed starts over from its first maximum (max-based from now on)
        a(f"v_cmp_lt_f32 vcc, {OVF_SUM}, {vreg(pk)}",
          "s_nop 1",
          f"v_cndmask_b32 {vreg(V_MREF[h])}, {vreg(V_MREF[h])}, {vreg(V_NEGINF)}, vcc",
          f"v_mov_b32 {vreg(V_PEAK[h])}, 0")
    a(f"s_max_u32 {s(S_UCUR)}, {s(S_UA)}, {s(S_CPRE)}",
      f"s_sub_u32 {s(S_T)}, {s(S_UCUR)}, {s(S_UA)}",
      f"s_lshl_b32 {s(S_T)}, {s(S_T)}, 1",
      f"s_mov_b32 {s(S_TL)}, 0",
      f"s_mov_b32 {s(S_LSEQ)}, {s(S_CSEQ)}",
      f"s_mov_b32 {s(S_LPRE)}, {s(S_CPRE)}",
      f"s_mov_b32 {s(S_LUNITS)}, {s(S_CUNITS)}",
      f"s_mov_b32 {s(S_LLEN)}, {s(S_CLEN)}",
      f"v_mov_b32 {vreg(V_LRUN[0])}, 0",
      f"v_mov_b32 {vreg(V_LRUN[1])}, 0")
    zero_o(a)
    start_loads_hp(a)
    load_q(a, S_CSEQ)         # Q may hold the next segment's rows by now
    a(f"s_mov_b32 {s(S_PNONE)}, 0",
      f"s_mov_b32 {s(S_EPI)}, 0")
    a.lines += flatten(next_items(S_T, True))
    a("s_branch .Lstep")
    a.label(".Lkernel_end")
    a(s_waitcnt_vm(0), "s_endpgm")   # the last loads must land before the LDS is released


def load_q(a, seq_sgpr):
    """Q of this wave's query rows of sequence s[seq_sgpr] into V_Q (36
    loads): row (seq * s_q + s_tok) * 128 + head0 .. + 31, latent then rope."""
    T = S_TMP
    t = V_T
    a(f"s_mul_i32 s{T}, s{seq_sgpr}, {s(S_STRIDE)}",
      f"s_add_u32 s{T}, s{T}, {s(S_TOK0)}",
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


def segment_setup(a, with_q=True, zero=True):
    """Start of a segment (the sequence S_CSEQ from unit S_UCUR on): its
    length, units and visible rows, the query rows of this wave (Q into
    registers unless with_q is False: then they are on their way already),
    the running softmax state, O = 0 (unless zero is False: the previous
    epilogue, or the kernel start, cleared it)."""
    T = S_TMP
    own, got = a.new_label("lenown"), a.new_label("lengot")
    a(f"s_cmp_eq_u32 {s(S_LSEQ)}, {s(S_CSEQ)}",
      f"s_cbranch_scc0 {own}",
      f"s_mov_b32 {s(S_CLEN)}, {s(S_LLEN)}",     # the loader holds this sequence's length
      f"s_branch {got}")
    a.label(own)
    load_len(a, S_CLEN, S_CSEQ)
    a.label(got)
    units_of(a, S_CUNITS, S_CLEN)
    a(f"s_add_u32 {s(S_SEGEND)}, {s(S_CPRE)}, {s(S_CUNITS)}",
      f"s_min_u32 {s(S_SEGEND)}, {s(S_SEGEND)}, {s(S_UB)}",
      f"s_sub_i32 {s(S_NVIS)}, {s(S_CLEN)}, {s(S_STRIDE)}",
      f"s_add_i32 {s(S_NVIS)}, {s(S_NVIS)}, {s(S_TOK0)}",
      f"s_add_i32 {s(S_NVLO)}, {s(S_NVIS)}, 1",
      f"s_add_i32 {s(S_NVIS)}, {s(S_NVIS)}, {s(S_STOK)}",
      f"s_add_i32 {s(S_NVIS)}, {s(S_NVIS)}, 1",
      # the workgroup's last query token: (32 * 3) >> log2(heads per block)
      f"s_ff1_i32_b32 s{T}, {s(S_HB)}",
      f"s_lshr_b32 s{T}, 96, s{T}",
      f"s_add_i32 {s(S_NVHI)}, {s(S_NVLO)}, s{T}",
      f"s_mov_b64 {sp(S_OVF)}, 0")
    if with_q:
        load_q(a, S_CSEQ)
    a(f"v_mov_b32 {vreg(V_MREF[0])}, {NEG_INF}",
      f"v_mov_b32 {vreg(V_MREF[1])}, {NEG_INF}",
      f"v_mov_b32 {vreg(V_LRUN[0])}, 0",
      f"v_mov_b32 {vreg(V_LRUN[1])}, 0",
      f"v_mov_b32 {vreg(V_PEAK[0])}, 0",
      f"v_mov_b32 {vreg(V_PEAK[1])}, 0",
      f"s_mov_b32 {s(S_EXACT)}, 0")
    if FP8:
        a(f"v_mov_b32 {vreg(V_LBLK[0])}, 0",
          f"v_mov_b32 {vreg(V_LBLK[1])}, 0")
    if zero:
        zero_o(a)


def kernel(fp8=False):
    configure(fp8)
    a = Asm()
    a.lines += [
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
      *([f"s_load_dwordx4 s[{S_FSC}:{S_FSC + 3}], s[0:1], 0x68"] if FP8 else []),
      f"s_load_dwordx2 s[{S_STRIDE}:{S_TOK0}], s[0:1], 0x78",
      f"s_mov_b32 {s(S_ONES)}, 0x3f803f80",
      f"v_and_b32 {vreg(V_LANE)}, 63, {vreg(V_TID)}",
      f"v_lshrrev_b32 {vreg(V_G)}, 4, {vreg(V_LANE)}",
      f"v_and_b32 {vreg(V_R16)}, 15, {vreg(V_LANE)}",
      f"v_lshrrev_b32 {vreg(V_T)}, 6, {vreg(V_TID)}",
      "s_nop 1",
      f"v_readfirstlane_b32 {s(S_WAVE)}, {vreg(V_T)}",
      s_waitcnt_lgkm(0))
    # ------------------------------------------------ workgroup -> (partition, head block)
    plain, mapped = a.new_label("mapplain"), a.new_label("mapdone")
    # head blocks per partition: a power of two (mask s[T], shift s[T+4])
    a(f"s_sub_u32 s{T}, {s(S_NHB)}, 1",
      f"s_ff1_i32_b32 s{T + 4}, {s(S_NHB)}",
      f"s_and_b32 s{T + 1}, {s(S_NPART)}, 7",
      f"s_cmp_eq_u32 s{T + 1}, 0",
      f"s_cbranch_scc0 {plain}",
      # consecutive partitions on one XCD: xcd = wg & 7 owns partitions xcd*P/8 ..
      f"s_lshr_b32 s{T + 1}, s2, 3",
      f"s_and_b32 s{T + 2}, s2, 7",
      f"s_lshr_b32 s{T + 3}, {s(S_NPART)}, 3",
      f"s_mul_i32 s{T + 2}, s{T + 2}, s{T + 3}",
      f"s_lshr_b32 {s(S_PART)}, s{T + 1}, s{T + 4}",
      f"s_add_u32 {s(S_PART)}, {s(S_PART)}, s{T + 2}",
      f"s_and_b32 {s(S_HBLK)}, s{T + 1}, s{T}",
      f"s_branch {mapped}")
    a.label(plain)
    a(f"s_lshr_b32 {s(S_PART)}, s2, s{T + 4}",
      f"s_and_b32 {s(S_HBLK)}, s2, s{T}")
    a.label(mapped)
    # ------------------------------------------------ partition map
    # up to 64 FAST_LENS sequences from lengths held in registers (one load),
    # larger batches in passes over memory
    slow, mapdone = a.new_label("mapslow"), a.new_label("mapfound")
    a(f"s_cmp_gt_u32 {s(S_BATCH)}, {64 * FAST_LENS}",
      f"s_cbranch_scc1 {slow}")
    load_lens_fast(a)
    partition_map(a, fast=True)
    a(f"s_branch {mapdone}")
    a.label(slow)
    partition_map(a, fast=False)
    a.label(mapdone)
    # the loader cursor starts at the partition's first sequence
    a(f"s_mov_b32 {s(S_LSEQ)}, {s(S_CSEQ)}",
      f"s_mov_b32 {s(S_LPRE)}, {s(S_CPRE)}")
    units_of(a, S_LUNITS, S_LLEN)
    # ------------------------------------------------ this wave's query rows
    a(f"s_lshl_b32 s{T}, {s(S_WAVE)}, 5",
      f"s_sub_u32 s{T + 1}, {s(S_HB)}, 1",
      f"s_and_b32 s{T + 2}, s{T}, s{T + 1}",
      f"s_mul_i32 s{T + 3}, {s(S_HBLK)}, {s(S_HB)}",
      f"s_add_u32 {s(S_HEAD0)}, s{T + 2}, s{T + 3}",
      f"s_ff1_i32_b32 s{T + 1}, {s(S_HB)}",
      f"s_lshr_b32 {s(S_STOK)}, s{T}, s{T + 1}")
    # ------------------------------------------------ lane-constant LDS offsets
    lane_constants(a)
    if FP8:
        lane_constants_fp8(a)
    t = V_T
    a(f"v_mov_b32 {vreg(V_NEGINF)}, {NEG_INF}")
    if FP8:
        flag_write(a, 0)    # restart flag = 0
        # the reciprocal fragments' zero rows (4q + 2, 4q + 3): written once
        a(f"v_lshlrev_b32 {vreg(V_T)}, 3, {vreg(V_TID)}",
          f"v_add_u32 {vreg(V_T)}, {F8_RF}, {vreg(V_T)}",
          f"v_mov_b32 {vreg(V_T + 2)}, 0",
          f"v_mov_b32 {vreg(V_T + 3)}, 0",
          f"ds_write_b64 {vreg(V_T)}, {vr(V_T + 2, 2)}")
    a(s_waitcnt_lgkm(0), "s_barrier")
    if not FP8:
        kernel_tail_hp(a)
        a.lines += [f".L{KNAME}_end:", f"\t.size {KNAME}, .L{KNAME}_end-{KNAME}", ""]
        a.lines += descriptor()
        return a.text()
    # ------------------------------------------------ first unit
    a(f"s_mov_b32 {s(S_UCUR)}, {s(S_UA)}",
      f"s_mov_b32 {s(S_SLOT)}, 0")
    (issue_unit_fp8 if FP8 else issue_unit)(a, S_UCUR, S_SLOT)
    prefetch_next(a, S_UCUR)
    # ------------------------------------------------ segments
    a.label(".Lseg")
    segment_setup(a)
    # ------------------------------------------------ units of the segment
    # On entry the loads of unit S_UCUR into its slot are in flight.
    uend = unit_body_fp8(a)
    a.label(uend)
    if FP8:
        noflag = a.new_label("noflag")
        a(f"s_cmp_eq_u64 {sp(S_OVF)}, 0",
          f"s_cbranch_scc1 {noflag}")
        flag_write(a, 1, all_waves=True)
        a.label(noflag)
    a(f"s_add_u32 {s(S_UCUR)}, {s(S_UCUR)}, 1",
      f"s_cmp_lt_u32 {s(S_UCUR)}, {s(S_SEGEND)}",
      "s_cbranch_scc1 .Lunit")
    # end of the segment: a restart request of its last unit (fp8), or of any of its units (bf16)?
    a(s_waitcnt_lgkm(0), "s_barrier")
    if FP8:
        flag_check(a)
        epilogue(a)
    else:
        epilogue_split(a)
    a(f"s_add_u32 {s(S_CPRE)}, {s(S_CPRE)}, {s(S_CUNITS)}",
      f"s_add_u32 {s(S_CSEQ)}, {s(S_CSEQ)}, 1",
      f"s_cmp_lt_u32 {s(S_UCUR)}, {s(S_UB)}",
      "s_cbranch_scc1 .Lseg",
      "s_branch .Lkernel_end")
    # ------------------------------------------------ restart of the segment
    a.label(".Lrestart")
    a(s_waitcnt_vm(0), "s_barrier")   # every wave has read the flag; no loads in flight
    if FP8:
        flag_write(a, 0)
    a(f"s_mov_b64 {sp(S_OVF)}, 0")
    # the re-run keeps the exact (max-based) reference for the whole segment, so
    # every further restart raises m_ref past an observed maximum: at most one
    # restart per sub-step whose max passes the reference
    a(f"s_mov_b32 {s(S_EXACT)}, 1")
    for h in range(2):
        pk, t0, t1, lp = V_T, V_T + 1, V_T + 2, V_T + 3
        a(f"v_mov_b32 {vreg(pk)}, {vreg(V_PEAK[h])}")
        xor_reduce(a, pk, "v_max_f32", t0, t1)
        if FP8:
            # the restart follows the unit whose lean sub-step overflowed:
            # m_ref += log2(peak sum of the head) + 27, at most 128 + 27
            a(f"v_log_f32 {vreg(lp)}, {vreg(pk)}",
              f"v_cmp_lt_f32 vcc, {OVF_SUM}, {vreg(pk)}",
              "s_nop 0",
              f"v_min_f32 {vreg(lp)}, 0x43000000, {vreg(lp)}",          # 128
              f"v_add_f32 {vreg(lp)}, 0x41d80000, {vreg(lp)}",          # + 27
              f"v_add_f32 {vreg(lp)}, {vreg(V_MREF[h])}, {vreg(lp)}",
              "s_nop 1",
              f"v_cndmask_b32 {vreg(V_MREF[h])}, {vreg(V_MREF[h])}, {vreg(lp)}, vcc")
        else:
            # the restart comes at the segment's end, after units that may have
            # moved the reference since the overflow: a head whose lean sub-step
            # overflowed starts over from its first maximum (max-based from now on)
            a(f"v_cmp_lt_f32 vcc, {OVF_SUM}, {vreg(pk)}",
              "s_nop 1",
              f"v_cndmask_b32 {vreg(V_MREF[h])}, {vreg(V_MREF[h])}, {vreg(V_NEGINF)}, vcc")
        a(f"v_mov_b32 {vreg(V_PEAK[h])}, 0")
    a(f"s_max_u32 {s(S_UCUR)}, {s(S_UA)}, {s(S_CPRE)}",
      f"s_mov_b32 {s(S_LSEQ)}, {s(S_CSEQ)}",
      f"s_mov_b32 {s(S_LPRE)}, {s(S_CPRE)}",
      f"s_mov_b32 {s(S_LUNITS)}, {s(S_CUNITS)}",
      f"s_mov_b32 {s(S_LLEN)}, {s(S_CLEN)}",
      f"v_mov_b32 {vreg(V_LRUN[0])}, 0",
      f"v_mov_b32 {vreg(V_LRUN[1])}, 0")
    if FP8:
        a(f"v_mov_b32 {vreg(V_LBLK[0])}, 0",
          f"v_mov_b32 {vreg(V_LBLK[1])}, 0")
    zero_o(a)
    a(f"s_sub_u32 {s(S_SLOT)}, {s(S_UCUR)}, {s(S_UA)}",
      f"s_and_b32 {s(S_SLOT)}, {s(S_SLOT)}, 1")
    (issue_unit_fp8 if FP8 else issue_unit)(a, S_UCUR, S_SLOT)
    prefetch_next(a, S_UCUR)
    a("s_branch .Lunit")
    a.label(".Lkernel_end")
    a(s_waitcnt_vm(0), "s_endpgm")   # the last unit's spare copy must land before the LDS is released
    a.lines += [f".L{KNAME}_end:", f"\t.size {KNAME}, .L{KNAME}_end-{KNAME}", ""]
    a.lines += descriptor()
    return a.text()


def descriptor():
    return f"""	.rodata
	.p2align 6
	.amdhsa_kernel {KNAME}
		.amdhsa_group_segment_fixed_size {LDS_BYTES}
		.amdhsa_private_segment_fixed_size 0
		.amdhsa_kernarg_size {KARG_BYTES}
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
	.text
""".splitlines()


def metadata(kernels):
    """Code-object metadata for the given (name, lds_bytes) kernels, which all
    take the same argument block: 9 pointers, 8 scalars, 2 pointers, 2 scalars."""
    lines = ["\t.amdgpu_metadata", "---", "amdhsa.kernels:"]
    for name, lds in kernels:
        lines += [f"  - .agpr_count:     256", "    .args:"]
        for k in range(9):
            lines.append(f"      - {{ .address_space: global, .offset: {8 * k}, .size: 8, .value_kind: global_buffer }}")
        for k in range(8):
            lines.append(f"      - {{ .offset: {72 + 4 * k}, .size: 4, .value_kind: by_value }}")
        for k in range(2):
            lines.append(f"      - {{ .address_space: global, .offset: {104 + 8 * k}, .size: 8, .value_kind: global_buffer }}")
        for k in range(2):
            lines.append(f"      - {{ .offset: {120 + 4 * k}, .size: 4, .value_kind: by_value }}")
        lines += [f"    .group_segment_fixed_size: {lds}",
                  "    .kernarg_segment_align: 8",
                  f"    .kernarg_segment_size: {KARG_BYTES}",
                  "    .max_flat_workgroup_size: 256",
                  f"    .name:           {name}",
                  "    .private_segment_fixed_size: 0",
                  f"    .sgpr_count:     {S_MAX + 6}",
                  f"    .symbol:         {name}.kd",
                  "    .vgpr_count:     512",
                  "    .wavefront_size: 64"]
    lines += ["amdhsa.target:   amdgcn-amd-amdhsa--gfx950", "amdhsa.version:", "  - 1", "  - 2", "...",
              "\t.end_amdgpu_metadata"]
    return lines


def code_object_source():
    """Both kernels (bf16 and fp8 cache) in one assembly file."""
    import re
    parts, kernels = ['\t.amdgcn_target "amdgcn-amd-amdhsa--gfx950"', "\t.amdhsa_code_object_version 6"], []
    for fp8 in (False, True):
        text = kernel(fp8)
        tag = "f8" if fp8 else "bf"
        code, desc = text.split("\t.rodata", 1)
        code = re.sub(r"\.L(\w+)", lambda m: f".L{tag}_{m.group(1)}", code)   # labels local to each kernel
        parts += [code, "\t.rodata" + desc]
        kernels.append((KNAME, LDS_BYTES))
    configure(False)
    return "\n".join(parts) + "\n" + "\n".join(metadata(kernels)) + "\n"


if __name__ == "__main__":
    out = sys.argv[1] if len(sys.argv) > 1 else "mla_decode_gfx950.s"
    with open(out, "w") as f:
        f.write(code_object_source())
