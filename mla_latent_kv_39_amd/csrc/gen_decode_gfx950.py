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
    with direct-to-LDS loads.  A slot is 9 x 8 blocks of 8 rows x 8 chunks
    (chunk = 16 bytes); one load instruction moves one block, eight whole
    128-byte lines of the page, and an XOR swizzle of the chunk slot inside
    a block keeps the 16-row score reads and the transposed output reads
    free of bank conflicts (lane_constants below);
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

SLOT_BYTES = 64 * 1152          # one page of bf16 rows = one LDS tile
KARG_BYTES = 120                # kernel argument block (both kernels)

# bf16 kernel: two tile slots, the restart flag after them
KNAME = "mla_decode_bf16_gfx950"
FP8 = False
FLAG_ADDR = 2 * SLOT_BYTES
LDS_BYTES = FLAG_ADDR + 16
PAGE_BYTES = SLOT_BYTES         # global bytes of one page of the row array

# fp8 kernel: one bf16 tile, two staging slots of raw pages (e4m3 codes, bf16
# rope, fp32 scales), the current unit's scales as [block][row], the flag
F8_CODES, F8_ROPE, F8_SCALES = 64 * 512, 64 * 128, 64 * 16
F8_RAW = F8_CODES + F8_ROPE + F8_SCALES          # 41984
F8_RAW0 = SLOT_BYTES
F8_SCL = F8_RAW0 + 2 * F8_RAW                    # 157696
F8_FLAG = F8_SCL + 1024


def configure(fp8):
    """Select the kernel the generator functions emit."""
    global KNAME, FP8, FLAG_ADDR, LDS_BYTES, PAGE_BYTES
    FP8 = fp8
    if fp8:
        KNAME, FLAG_ADDR, PAGE_BYTES = "mla_decode_fp8_gfx950", F8_FLAG, F8_CODES
    else:
        KNAME, FLAG_ADDR, PAGE_BYTES = "mla_decode_bf16_gfx950", 2 * SLOT_BYTES, SLOT_BYTES
    LDS_BYTES = FLAG_ADDR + 16
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
V_PEAK = (110, 111)      # largest 8-row probability sum seen per lane in this segment (lean softmax)
V_Q = 112                # Q[ks][h] at 112 + (2*ks + h)*4, 144 regs
# source offsets of the next unit's loads (row groups 2w, 2w+1): live through the phases
V_DMA = (V_T + 1, V_T + 2)
# softmax scratch: sub-step 0 borrows P[1], sub-step 1 borrows S[0] (both free at that time)
V_SMT = (tuple(range(V_P[1], V_P[1] + 4)), tuple(range(V_S[0], V_S[0] + 4)))
EPI_TEMPS = list(range(16, 48))   # the epilogue runs between units
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
# loads of the next unit issued in phases 1, 2, 3 of a full unit
DMA_SPLIT = (8, 6, 4)
S_MAX = 98


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


def loader_prefetch(a, u_sgpr):
    """Look up unit u one unit before its loads are issued: S_NV2 = its valid
    rows (<= 0: none), S_ENT2 = its page for a contiguous cache, or -1 with the
    page on its way into V_ENT (a vector load, so that the LDS waits of the
    phases never wait on it; it lands before the next unit's barrier)."""
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
      f"s_lshl_b32 s{T + 5}, {s(S_ENT2)}, 2",
      f"v_mov_b32 {vreg(V_T + 3)}, s{T + 5}",       # v13/v14 hold the next unit's load offsets
      f"global_load_dword {vreg(V_ENT)}, {vreg(V_T + 3)}, {sp(S_TABLE)}",
      f"s_mov_b32 {s(S_ENT2)}, -1")
    a.label(done)


def prefetch_next(a, u_sgpr):
    """Prefetch the page of unit u + 1 if the partition has it (else none)."""
    T = S_TMP
    nonext, done = a.new_label("pfnone"), a.new_label("pfend")
    a(f"s_add_u32 s{T + 20}, {s(u_sgpr)}, 1",
      f"s_cmp_lt_u32 s{T + 20}, {s(S_UB)}",
      f"s_cbranch_scc0 {nonext}")
    loader_advance(a, T + 20)
    loader_prefetch(a, T + 20)
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


def dma_setup(a, slot_sgpr):
    """Lane source offsets of the two row groups this wave copies (row 0 past
    the valid rows) and the LDS base of its blocks in the slot."""
    va, vb = V_DMA
    t0 = V_T + 3
    a(f"v_cmp_gt_i32 vcc, {s(S_NVALID)}, {vreg(V_LDROW)}",
      f"v_add_u32 {vreg(t0)}, 8, {vreg(V_LDROW)}",
      "s_nop 1",
      f"v_cndmask_b32 {vreg(va)}, {vreg(V_LCA)}, {vreg(V_LDA)}, vcc",
      f"v_cmp_gt_i32 vcc, {s(S_NVALID)}, {vreg(t0)}",
      f"s_mul_i32 {s(S_DMALDS)}, {s(slot_sgpr)}, {SLOT_BYTES}",
      f"s_lshl_b32 s{S_TMP + 5}, {s(S_WAVE)}, 11",
      f"s_add_u32 {s(S_DMALDS)}, {s(S_DMALDS)}, s{S_TMP + 5}",   # slot + block (0, 2w)
      "s_nop 0",
      f"v_cndmask_b32 {vreg(vb)}, {vreg(V_LCB)}, {vreg(V_LDB)}, vcc")


def dma_groups():
    """The 18 direct-to-LDS loads of one unit, as separate instruction groups.
    Wave w fills the tile blocks of rows 16w .. 16w+15 (row groups 2w, 2w+1,
    all nine chunk groups); one load moves one 8-row x 8-chunk block, i.e.
    eight 128-byte lines of the page."""
    va, vb = V_DMA
    groups = []
    for i in range(18):
        k, odd = divmod(i, 2)
        src = vb if odd else va
        groups.append([f"\ts_add_u32 s{S_DPAGE}, s{S_PAGE}, {128 * k}",
                       f"\ts_addc_u32 s{S_DPAGE + 1}, s{S_PAGE + 1}, 0",
                       f"\ts_add_u32 m0, {s(S_DMALDS)}, {1024 * (8 * k + odd)}",
                       "\ts_nop 0",
                       f"\tglobal_load_lds_dwordx4 {vreg(src)}, {sp(S_DPAGE)}"])
    return groups


def issue_unit(a, u_sgpr, slot_sgpr):
    """Stand-alone copy of unit u into the slot (prologue and restart)."""
    loader_advance(a, u_sgpr)
    loader_lookup(a, u_sgpr, wait=True)
    loader_page(a)
    dma_setup(a, slot_sgpr)
    for g in dma_groups():
        a.lines += g


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
    """One LDS operand fragment and the two MFMAs that consume it."""

    def __init__(self, ring, ring_base, nring, idx, reads, mfmas):
        self.ring, self.idx = ring, idx
        buf = ring_base + 4 * (idx % nring)
        self.reads = [r.format(buf=vr(buf, 4), lo=vr(buf, 2), hi=vr(buf + 2, 2)) for r in reads]
        self.mfmas = [m.format(buf=vr(buf, 4)) for m in mfmas]
        self.read_ids = []


def qk_frags(ss):
    out = []
    for i in range(36):
        ks, tb = divmod(i, 2)
        mf = []
        for h in range(2):
            sreg = V_S[ss] + (2 * tb + h) * 4
            qreg = V_Q + (2 * ks + h) * 4
            c = "0" if ks == 0 else vr(sreg, 4)
            mf.append(f"\tv_mfma_f32_16x16x32_bf16 {vr(sreg, 4)}, {{buf}}, {vr(qreg, 4)}, {c}")
        out.append(Frag("A", V_A, NA, 36 * ss + i, qk_read(ss, i), mf))
    return out


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


def emit_phases(a, frags, lead, fillers, marks=None):
    """Emit the MFMA stream `frags` with its LDS reads and interleaved filler.

    Reads of ring fragment f are issued right after the MFMAs of f - ring size
    (the previous user of its buffer); the first fragments of each ring are
    issued at the stream position given by `lead` {ring: index of the fragment
    after whose MFMAs they go, -1 = at the start}.  fillers: list of
    (first, last, instructions): spread evenly between the MFMAs of fragments
    first..last (no LDS operations inside)."""
    lds = LdsOrder()
    nring = {"A": NA, "B": NB}
    by_ring = {}
    for f in frags:
        by_ring.setdefault(f.ring, []).append(f)
    pending = {}   # position -> list of frags whose reads go after that position's MFMAs

    def issue_reads(f):
        for r in f.reads:
            f.read_ids.append(lds.issue())
            a.lines.append(r)

    pos_of = {id(f): p for p, f in enumerate(frags)}
    for ring, lst in by_ring.items():
        for j, f in enumerate(lst):
            if j < nring[ring]:
                at = lead[ring]
            else:
                at = pos_of[id(lst[j - nring[ring]])]
            pending.setdefault(at, []).append(f)
    # filler slots: after each of the two MFMAs of a fragment
    slots = {}
    for first, last, ins in fillers:
        n = 2 * (last - first + 1)
        per = [len(ins) * (k + 1) // n - len(ins) * k // n for k in range(n)]
        it = iter(ins)
        for k in range(n):
            slots.setdefault((first + k // 2, k % 2), []).extend(next(it) for _ in range(per[k]))
    for f in pending.get(-1, []):
        issue_reads(f)
    for p, f in enumerate(frags):
        a.lines += lds.wait(max(f.read_ids))
        for m, mf in enumerate(f.mfmas):
            a.lines.append(mf)
            a.lines += slots.get((p, m), [])
        for g in pending.get(p, []):
            issue_reads(g)
        if marks and p in marks:
            a.comment(f"phase {marks[p]} issued")


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
        x("s_nop 0",
          f"v_add_f32 {vreg(t0)}, {vreg(regs[0])}, {vreg(regs[1])}",
          f"v_add_f32 {vreg(t1)}, {vreg(regs[2])}, {vreg(regs[3])}",
          f"v_add_f32 {vreg(t0)}, {vreg(t0)}, {vreg(regs[4])}",
          f"v_add_f32 {vreg(t1)}, {vreg(t1)}, {vreg(regs[5])}",
          f"v_add_f32 {vreg(t0)}, {vreg(t0)}, {vreg(regs[6])}",
          f"v_add_f32 {vreg(t1)}, {vreg(t1)}, {vreg(regs[7])}",
          f"v_add_f32 {vreg(t0)}, {vreg(t0)}, {vreg(t1)}",
          f"v_add_f32 {vreg(V_LRUN[h])}, {vreg(V_LRUN[h])}, {vreg(t0)}")
        if P is not None:
            p = P + 4 * h
            x(f"v_cvt_pk_bf16_f32 {vreg(p)}, {vreg(regs[0])}, {vreg(regs[1])}",
              f"v_cvt_pk_bf16_f32 {vreg(p + 1)}, {vreg(regs[2])}, {vreg(regs[3])}",
              f"v_cvt_pk_bf16_f32 {vreg(p + 2)}, {vreg(regs[4])}, {vreg(regs[5])}",
              f"v_cvt_pk_bf16_f32 {vreg(p + 3)}, {vreg(regs[6])}, {vreg(regs[7])}")
    return x.lines


def softmax_lean(ss, S=None, P=None, tmp=None):
    """Softmax of a fully visible sub-step once the segment's reference is
    set: P = 2^(scale S - m_ref), row sums, bf16 pack.  No max: a lane whose
    8-row sum passes 2^64 (the largest score more than ~64 above m_ref) flags a
    restart, and V_PEAK keeps the largest such sum so that the restart can
    raise m_ref past it."""
    if S is None:
        S, P, tmp = V_S[ss], V_P[ss], V_SMT[ss]
    t0, t1 = tmp[0], tmp[1]
    x = Asm()
    for h in range(2):
        regs = [S + (2 * tb + h) * 4 + i for tb in range(2) for i in range(4)]
        mref = V_MREF[h]
        for r in regs:
            x(f"v_fma_f32 {vreg(r)}, {vreg(r)}, {s(S_SCALE)}, -{vreg(mref)}")
        for r in regs:
            x(f"v_exp_f32 {vreg(r)}, {vreg(r)}")
        x("s_nop 0",
          f"v_add_f32 {vreg(t0)}, {vreg(regs[0])}, {vreg(regs[1])}",
          f"v_add_f32 {vreg(t1)}, {vreg(regs[2])}, {vreg(regs[3])}",
          f"v_add_f32 {vreg(t0)}, {vreg(t0)}, {vreg(regs[4])}",
          f"v_add_f32 {vreg(t1)}, {vreg(t1)}, {vreg(regs[5])}",
          f"v_add_f32 {vreg(t0)}, {vreg(t0)}, {vreg(regs[6])}",
          f"v_add_f32 {vreg(t1)}, {vreg(t1)}, {vreg(regs[7])}",
          f"v_add_f32 {vreg(t0)}, {vreg(t0)}, {vreg(t1)}",
          f"v_add_f32 {vreg(V_LRUN[h])}, {vreg(V_LRUN[h])}, {vreg(t0)}",
          f"v_cmp_lt_f32 vcc, {OVF_SUM}, {vreg(t0)}",
          f"v_max_f32 {vreg(V_PEAK[h])}, {vreg(V_PEAK[h])}, {vreg(t0)}",
          f"s_or_b64 {sp(S_OVF)}, {sp(S_OVF)}, vcc")
        if P is not None:
            p = P + 4 * h
            x(f"v_cvt_pk_bf16_f32 {vreg(p)}, {vreg(regs[0])}, {vreg(regs[1])}",
              f"v_cvt_pk_bf16_f32 {vreg(p + 1)}, {vreg(regs[2])}, {vreg(regs[3])}",
              f"v_cvt_pk_bf16_f32 {vreg(p + 2)}, {vreg(regs[4])}, {vreg(regs[5])}",
              f"v_cvt_pk_bf16_f32 {vreg(p + 3)}, {vreg(regs[6])}, {vreg(regs[7])}")
    return x.lines


def unit_full(a, lean):
    """Both 32-row sub-steps.  Phases: scores of sub-step 0 (next unit's loads
    interleaved), scores of 1 with softmax of 0, output of 0 with softmax of
    1, output of 1."""
    q0, q1, p0, p1 = qk_frags(0), qk_frags(1), pv_frags(0), pv_frags(1)
    frags = q0 + q1 + p0 + p1
    groups = dma_groups()
    n1, n2, n3 = DMA_SPLIT
    assert n1 + n2 + n3 == len(groups)
    sm = softmax_lean if lean else softmax_code
    fillers = [(0, 35, [ins for g in groups[:n1] for ins in g]),
               (36 + 3, 71 - 1, merge_filler(sm(0), groups[n1:n1 + n2])),
               (72 + 3, 103 - 3, merge_filler(sm(1), groups[n1 + n2:]))]
    emit_phases(a, frags, {"A": -1, "B": 71 - NB}, fillers, marks={35: 1, 71: 2, 103: 3})


def merge_filler(ins, groups):
    """Spread the load groups evenly through an instruction list (order kept)."""
    if not groups:
        return list(ins)
    out, step = [], len(ins) / len(groups)
    gi = 0
    for k, x in enumerate(ins):
        while gi < len(groups) and k >= gi * step:
            out += groups[gi]
            gi += 1
        out.append(x)
    for g in groups[gi:]:
        out += g
    return out


def unit_half(a):
    """Only sub-step 0 has visible rows (last unit of a sequence)."""
    q0, p0 = qk_frags(0), pv_frags(0)
    dma = [ins for g in dma_groups() for ins in g]
    emit_phases(a, q0, {"A": -1}, [(0, 35, dma)])
    a("s_nop 7", "s_nop 7", "s_nop 3")   # MFMA results -> VALU
    sm = softmax_code(0)
    # output-operand reads go out first, overlapping the softmax
    emit_phases_split(a, p0, sm)


def emit_phases_split(a, p0, sm):
    lds = LdsOrder()
    for f in p0[:NB]:
        for r in f.reads:
            f.read_ids.append(lds.issue())
            a.lines.append(r)
    a.lines += sm
    a("s_nop 4")   # VALU writes of P -> MFMA reads
    for p, f in enumerate(p0):
        a.lines += lds.wait(max(f.read_ids))
        a.lines += f.mfmas
        if p + NB < len(p0):
            g = p0[p + NB]
            for r in g.reads:
                g.read_ids.append(lds.issue())
                a.lines.append(r)


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


def dequant_fp8(a):
    """Rows 16w .. 16w+15 of the current unit: staging slot S_SLOT -> bf16
    tile (codes widened exactly, rows at or past S_CURVALID zeroed), rope
    copied, scales transposed to [block][row].  Ends with the LDS writes in
    flight."""
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
        a(f"v_cndmask_b32 {vreg(d)}, 0, {vreg(d)}, {m}",
          f"v_cndmask_b32 {vreg(d + 1)}, 0, {vreg(d + 1)}, {m}",
          f"v_cvt_scalef32_pk_bf16_fp8 {vreg(o)}, {vreg(d)}, 1.0",
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
        for q in range(4):
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
    for q in range(4):
        a(f"v_cndmask_b32 {vreg(sc + q)}, 0, {vreg(sc + q)}, vcc")
    a("s_nop 1")
    for q in range(4):
        a(f"ds_write_b32 {vreg(sa)}, {vreg(sc + q)} offset:{256 * q}")
    a("s_mov_b64 exec, -1")


def f8_scale_reads(ss, blk, dst):
    """Scales of rows 32ss + 16tb + 4g .. +3, block blk -> dst + 4tb (tb = 0, 1)."""
    return [f"\tds_read_b128 {vr(dst + 4 * tb, 4)}, {vreg(V_SCLB)} offset:{blk * 256 + (32 * ss + 16 * tb) * 4}"
            for tb in range(2)]


def qk_fp8(a, ss):
    """Scores of sub-step ss: k^R part into S, then per latent block
    T = C8_blk Q_blk (MFMA) and S += T * s_blk (fp32)."""
    order = [(16, tb) for tb in range(2)] + [(17, tb) for tb in range(2)]
    order += [(ks, tb) for ks in range(16) for tb in range(2)]
    frags = []
    for n, (ks, tb) in enumerate(order):
        acc = F8_S if ks >= 16 else F8_T
        first = ks == 16 or (ks < 16 and ks % 4 == 0)
        mf = []
        for h in range(2):
            d = acc + (2 * tb + h) * 4
            qreg = V_Q + (2 * ks + h) * 4
            c = "0" if first else vr(d, 4)
            mf.append(f"\tv_mfma_f32_16x16x32_bf16 {vr(d, 4)}, {{buf}}, {vr(qreg, 4)}, {c}")
        frags.append(Frag("A", V_A, NA, n, qk_read(ss, 2 * ks + tb), mf))
    lds = LdsOrder()
    for f in frags[:NA]:
        for r in f.reads:
            f.read_ids.append(lds.issue())
            a.lines.append(r)
    sc_ids = None
    for p, f in enumerate(frags):
        ks = order[p][0]
        if ks < 16 and ks % 4 == 0 and order[p][1] == 0:      # block start: its scales
            for r in f8_scale_reads(ss, ks // 4, F8_P[0]):
                a.lines.append(r)
            sc_ids = lds.issue(), lds.issue()
        a.lines += lds.wait(max(f.read_ids))
        a.lines += f.mfmas
        if p + NA < len(frags):
            g = frags[p + NA]
            for r in g.reads:
                g.read_ids.append(lds.issue())
                a.lines.append(r)
        if ks < 16 and ks % 4 == 3 and order[p][1] == 1:      # block end: S += T * s
            a.lines += lds.wait(sc_ids[1])
            a("s_nop 7", "s_nop 7", "s_nop 3")
            for tb in range(2):
                for h in range(2):
                    for i in range(4):
                        r = (2 * tb + h) * 4 + i
                        a(f"v_fma_f32 {vreg(F8_S + r)}, {vreg(F8_T + r)}, {vreg(F8_P[0] + 4 * tb + i)}, {vreg(F8_S + r)}")
    a("s_nop 7", "s_nop 7", "s_nop 3")


def pv_fp8(a, ss):
    """O^T += C8^T (P * s_blk)^T block by block (8 column blocks of 16 per latent block)."""
    frags = pv_frags(ss)
    lds = LdsOrder()
    for f in frags[:NB]:
        for r in f.reads:
            f.read_ids.append(lds.issue())
            a.lines.append(r)
    for blk in range(4):
        pb = F8_P[blk & 1]
        for r in f8_scale_reads(ss, blk, F8_T):
            a.lines.append(r)
        sid = lds.issue(), lds.issue()
        a.lines += lds.wait(sid[1])
        for h in range(2):
            regs = [F8_S + (2 * tb + h) * 4 + i for tb in range(2) for i in range(4)]
            prod = [F8_T + 8 + j for j in range(8)]
            for j, r in enumerate(regs):
                a(f"v_mul_f32 {vreg(prod[j])}, {vreg(r)}, {vreg(F8_T + j)}")
            p = pb + 4 * h
            a(f"v_cvt_pk_bf16_f32 {vreg(p)}, {vreg(prod[0])}, {vreg(prod[1])}",
              f"v_cvt_pk_bf16_f32 {vreg(p + 1)}, {vreg(prod[2])}, {vreg(prod[3])}",
              f"v_cvt_pk_bf16_f32 {vreg(p + 2)}, {vreg(prod[4])}, {vreg(prod[5])}",
              f"v_cvt_pk_bf16_f32 {vreg(p + 3)}, {vreg(prod[6])}, {vreg(prod[7])}")
        a("s_nop 4")   # VALU writes of P -> MFMA reads
        for cb in range(8 * blk, 8 * blk + 8):
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
      # whole: row_base = (c_seq * s_q + s_tok) * 128
      f"s_mul_i32 s{T + 1}, {s(S_CSEQ)}, {s(S_SQ)}",
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
      f"s_mul_i32 s{T + 1}, s{T + 1}, {s(S_SQ)}",
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
    x = EPI_TEMPS
    obase = sp(T + 14)
    for h in range(2):
        lt, inv, lse, t0, t1, off = temps(*x[0:6], pool=x)
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
        # lse of head 16h + r16 from the lanes with g == 0
        a(f"v_cmp_eq_u32 vcc, 0, {vreg(V_G)}",
          f"s_and_saveexec_b64 {sp(S_EXEC)}, vcc",
          f"v_lshlrev_b32 {vreg(t0)}, 2, {vreg(V_R16)}",
          f"global_store_dword {vreg(t0)}, {vreg(lse)}, s[{T + 10}:{T + 11}] offset:{64 * h}",
          f"s_mov_b64 exec, {sp(S_EXEC)}")
        bufs = [x[8:12], x[12:16], x[16:20], x[20:24]]
        rowwise, stored = a.new_label("rowwise"), a.new_label("stored")
        a(f"s_cmp_eq_u32 s{T + 3}, 0",
          f"s_cbranch_scc1 {rowwise}")
        # partial: lane order, store (h, cb) of lane L at (32h + cb) KB + 16 L of the wave's 64 KB
        a(f"v_lshlrev_b32 {vreg(off)}, 4, {vreg(V_LANE)}",
          f"s_add_u32 s{T + 16}, s{T + 14}, {32 * 1024 * h}",
          f"s_addc_u32 s{T + 17}, s{T + 15}, 0")
        for cb in range(32):
            if cb and cb % 4 == 0:
                a(f"s_add_u32 s{T + 16}, s{T + 16}, 4096", f"s_addc_u32 s{T + 17}, s{T + 17}, 0")
            epi_store(a, h, cb, bufs[cb % 4], inv, f"{vreg(off)}, {{v}}, s[{T + 16}:{T + 17}] offset:{1024 * (cb % 4)}")
        a(f"s_branch {stored}")
        # final result: row layout, lane (g, r16) -> (16h + r16) * 2048 + 16g + 64cb
        a.label(rowwise)
        a(f"v_lshlrev_b32 {vreg(t0)}, 4, {vreg(V_G)}",
          f"v_lshl_add_u32 {vreg(off)}, {vreg(V_R16)}, 11, {vreg(t0)}")
        if h:
            a(f"v_add_u32 {vreg(off)}, {16 * 2048}, {vreg(off)}")
        for cb in range(32):
            epi_store(a, h, cb, bufs[cb % 4], inv, f"{vreg(off)}, {{v}}, {obase} offset:{64 * cb}")
        a.label(stored)


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


def unit_body_bf16(a):
    """One unit of the bf16 kernel up to the unit-end label (returned)."""
    T = S_TMP
    a.label(".Lunit")
    a(f"s_mov_b64 {sp(S_OVF)}, 0",
      f"s_sub_u32 {s(S_SLOT)}, {s(S_UCUR)}, {s(S_UA)}",
      f"s_and_b32 {s(S_SLOT)}, {s(S_SLOT)}, 1")
    # this unit's rows have landed (own loads), the table prefetch too, and
    # every wave is past the previous unit
    a(s_waitcnt_vm(0), s_waitcnt_lgkm(0), "s_barrier")
    a(f"v_mov_b32 {vreg(V_T)}, {FLAG_ADDR}",
      f"ds_read_b32 {vreg(V_T)}, {vreg(V_T)}")       # restart flag, checked below
    take_prefetched(a)
    loader_page(a)
    a(f"s_xor_b32 s{T + 21}, {s(S_SLOT)}, 1")
    dma_setup(a, T + 21)
    a(f"s_add_u32 s{T + 19}, {s(S_UCUR)}, 1")
    prefetch_next(a, T + 19)
    a(f"s_sub_u32 {s(S_ROW0)}, {s(S_UCUR)}, {s(S_CPRE)}",
      f"s_lshl_b32 {s(S_ROW0)}, {s(S_ROW0)}, 6",
      f"s_mul_i32 s{T}, {s(S_SLOT)}, {SLOT_BYTES}",
      f"v_add_u32 {vreg(V_UQ)}, s{T}, {vreg(V_QKE)}",
      f"v_add_u32 {vreg(V_UQ + 1)}, s{T}, {vreg(V_QKO)}",
      f"v_add_u32 {vreg(V_UQ + 2)}, 0x10000, {vreg(V_UQ)}",
      f"v_add_u32 {vreg(V_UQ + 3)}, 0x10000, {vreg(V_UQ + 1)}",
      f"v_add_u32 {vreg(V_UP)}, s{T}, {vreg(V_PV0)}")
    for m in range(1, 4):
        a(f"v_xor_b32 {vreg(V_UP + m)}, {32 * m}, {vreg(V_PV0)}",
          f"v_add_u32 {vreg(V_UP + m)}, s{T}, {vreg(V_UP + m)}")
    # rows of this unit this wave's query token sees: none, only the first 32, or more
    a(s_waitcnt_lgkm(0),
      "s_nop 1",
      f"v_readfirstlane_b32 s{T}, {vreg(V_T)}",
      f"s_cmp_eq_u32 s{T}, 0",
      "s_cbranch_scc0 .Lrestart")
    # fully visible units after the first of the segment take the lean softmax
    half, none, uend, classic = (a.new_label(x) for x in ("half", "none", "uend", "classic"))
    a(f"s_sub_i32 s{T}, {s(S_NVIS)}, {s(S_ROW0)}",
      f"s_cmp_le_i32 s{T}, 0",
      f"s_cbranch_scc1 {none}",
      f"s_cmp_le_i32 s{T}, 32",
      f"s_cbranch_scc1 {half}",
      f"s_cmp_lt_i32 s{T}, 64",
      f"s_cbranch_scc1 {classic}",
      f"s_max_u32 s{T + 1}, {s(S_UA)}, {s(S_CPRE)}",
      f"s_cmp_eq_u32 {s(S_UCUR)}, s{T + 1}",
      f"s_cbranch_scc1 {classic}",
      f"s_cmp_eq_u32 {s(S_EXACT)}, 0",
      f"s_cbranch_scc0 {classic}")
    unit_full(a, lean=True)
    a(f"s_branch {uend}")
    a.label(classic)
    unit_full(a, lean=False)
    a(f"s_branch {uend}")
    a.label(half)
    unit_half(a)
    a(f"s_branch {uend}")
    a.label(none)
    for g in dma_groups():
        a.lines += g
    return uend


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
    a(f"s_xor_b32 s{T + 21}, {s(S_SLOT)}, 1")
    dma_fp8(a, T + 21)
    a(f"s_add_u32 s{T + 19}, {s(S_UCUR)}, 1")
    prefetch_next(a, T + 19)
    dequant_fp8(a)
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
    lane_constants(a)
    if FP8:
        lane_constants_fp8(a)
    t = V_T
    a(f"v_mov_b32 {vreg(V_NEGINF)}, {NEG_INF}")
    # restart flag = 0
    flag_write(a, 0)
    a(s_waitcnt_lgkm(0), "s_barrier")
    # ------------------------------------------------ loader cursor, first unit
    a(f"s_mov_b32 {s(S_LSEQ)}, {s(S_CSEQ)}",
      f"s_mov_b32 {s(S_LPRE)}, {s(S_CPRE)}")
    load_len(a, S_LLEN, S_LSEQ)
    units_of(a, S_LUNITS, S_LLEN)
    a(f"s_mov_b32 {s(S_UCUR)}, {s(S_UA)}",
      f"s_mov_b32 {s(S_SLOT)}, 0")
    (issue_unit_fp8 if FP8 else issue_unit)(a, S_UCUR, S_SLOT)
    prefetch_next(a, S_UCUR)
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
      f"v_mov_b32 {vreg(V_LRUN[1])}, 0",
      f"v_mov_b32 {vreg(V_PEAK[0])}, 0",
      f"v_mov_b32 {vreg(V_PEAK[1])}, 0",
      f"s_mov_b32 {s(S_EXACT)}, 0")
    zero_o(a)
    # ------------------------------------------------ units of the segment
    # On entry the loads of unit S_UCUR into its slot are in flight.
    uend = (unit_body_fp8 if FP8 else unit_body_bf16)(a)
    a.label(uend)
    noflag = a.new_label("noflag")
    a(f"s_cmp_eq_u64 {sp(S_OVF)}, 0",
      f"s_cbranch_scc1 {noflag}")
    flag_write(a, 1, all_waves=True)
    a.label(noflag)
    a(f"s_add_u32 {s(S_UCUR)}, {s(S_UCUR)}, 1",
      f"s_cmp_lt_u32 {s(S_UCUR)}, {s(S_SEGEND)}",
      "s_cbranch_scc1 .Lunit")
    # end of the segment: a restart request of its last unit?
    a(s_waitcnt_lgkm(0), "s_barrier")
    flag_check(a)
    epilogue(a)
    a(f"s_add_u32 {s(S_CPRE)}, {s(S_CPRE)}, {s(S_CUNITS)}",
      f"s_add_u32 {s(S_CSEQ)}, {s(S_CSEQ)}, 1",
      f"s_cmp_lt_u32 {s(S_UCUR)}, {s(S_UB)}",
      "s_cbranch_scc1 .Lseg",
      "s_branch .Lkernel_end")
    # ------------------------------------------------ restart of the segment
    a.label(".Lrestart")
    a(s_waitcnt_vm(0), "s_barrier")   # every wave has read the flag; no loads in flight
    flag_write(a, 0)
    # the re-run keeps the exact (max-based) reference for the whole segment, so
    # every further restart raises m_ref past an observed maximum: at most one
    # restart per sub-step whose max passes the reference
    a(f"s_mov_b32 {s(S_EXACT)}, 1")
    # a lean sub-step overflowed: m_ref += log2(peak sum of the head) + 27, at most 128 + 27
    for h in range(2):
        pk, t0, t1, lp = V_T, V_T + 1, V_T + 2, V_T + 3
        a(f"v_mov_b32 {vreg(pk)}, {vreg(V_PEAK[h])}")
        xor_reduce(a, pk, "v_max_f32", t0, t1)
        a(f"v_log_f32 {vreg(lp)}, {vreg(pk)}",
          f"v_cmp_lt_f32 vcc, {OVF_SUM}, {vreg(pk)}",
          "s_nop 0",
          f"v_min_f32 {vreg(lp)}, 0x43000000, {vreg(lp)}",          # 128
          f"v_add_f32 {vreg(lp)}, 0x41d80000, {vreg(lp)}",          # + 27
          f"v_add_f32 {vreg(lp)}, {vreg(V_MREF[h])}, {vreg(lp)}",
          "s_nop 1",
          f"v_cndmask_b32 {vreg(V_MREF[h])}, {vreg(V_MREF[h])}, {vreg(lp)}, vcc",
          f"v_mov_b32 {vreg(V_PEAK[h])}, 0")
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
    take the same argument block: 11 pointers, then 8 scalars."""
    lines = ["\t.amdgpu_metadata", "---", "amdhsa.kernels:"]
    for name, lds in kernels:
        lines += [f"  - .agpr_count:     256", "    .args:"]
        for k in range(9):
            lines.append(f"      - {{ .address_space: global, .offset: {8 * k}, .size: 8, .value_kind: global_buffer }}")
        for k in range(8):
            lines.append(f"      - {{ .offset: {72 + 4 * k}, .size: 4, .value_kind: by_value }}")
        for k in range(2):
            lines.append(f"      - {{ .address_space: global, .offset: {104 + 8 * k}, .size: 8, .value_kind: global_buffer }}")
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
