"""fp64 CPU oracle for decode-step Multi-head Latent Attention over a latent cache.

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this module.  It shares no code with the HIP path
(mla_latent_kv_39_amd) and imports nothing from it.

What it computes, and where the pages define it (page titles as given):

* [P2] = DeepSeek-V3 architecture notes (deepseek.csdn.net), §2.1 MLA.
  - §2.1.1: one decode step is softmax(Q_t K_{1:t}^T) V_{1:t} over the cached
    history.
  - §2.1.2: the cached object is c^KV (width d_c); k^C = W^UK c^KV and
    v^C = W^UV c^KV are both expanded from the same latent.
  - §2.1.3(B): by associativity q^T (W^UK c) = (W^UK^T q)^T c, so the query can
    carry W^UK ("absorbed") and the scores use c^KV directly; W^UV can likewise
    move to the output side, leaving the attention output in latent space.
  - §2.1.3(D): decoupled RoPE: q = [q^C; q^R], k = [k^C; k^R] with k^R shared by
    all heads, scores divided by sqrt(d_h + d_h^R); the cache keeps c^KV and k^R,
    d_c + d_h^R values per token per layer.
* [P1] = DeepSeek-V3 详解 (yudonglee.me), §2.1: d_c = 512, d_h^R = 64, 128
  heads, 576 cached values per token per layer; §3.3: MTP speculative decoding
  feeds x_{t+1} and the draft x_{t+2} through one forward pass.
* [P1] §4.2 / [P5] 拆解DeepSeek V3 (kongchang.com), "MLA 与 FP8": E4M3 with
  fine-grained 1x128 scaling; E4M3's range is about 448.

Readings where the pages are silent (each also listed in the design notes):
  * scale = 1/sqrt(d_h + d_h^R) = 1/sqrt(192) ([P2] §2.1.3(D) with d_h = 128).
  * V is the 512-wide latent only; k^R does not enter V ([P2] §2.1.2).
  * lse is the natural-log log-sum-exp of the scaled scores.
  * With S_q query tokens per sequence (MTP), seq_len counts every cached row
    including the S_q new ones, and query token s sees rows j < seq_len - S_q + s + 1.
  * fp8 rows dequantize as e4m3(code) * scale[block], one fp32 scale per
    128-wide block of the 512 latent values; k^R stays bf16.
  * A query that sees no row gives out = 0 and lse = -inf.

Parity pins (tests/test_oracle_pins.py): uniform scores, single row,
associativity against the unabsorbed per-head form, torch's fp64 SDPA,
split/merge identity, brute-force loops, paged == contiguous, row permutation,
MTP consistency, the e4m3 decoder over all 256 codes, cache-size invariants.
"""
from __future__ import annotations

import math

import numpy as np

# Dimensions as the pages give them ([P1] §2.1; [P2] §2.1.3(D), §3).
N_H = 128          # n_h, query heads
D_C = 512          # d_c, latent width
D_H_R = 64         # d_h^R, decoupled RoPE width
D_H = 128          # d_h, per-head width of the unabsorbed path
D_ROW = D_C + D_H_R  # values cached per token per layer
FP8_BLOCK = 128


def mha_cache_values_per_token(n_h: int = N_H, d_h: int = D_H) -> int:
    """Values a standard MHA layer caches per token: K and V for every head, 2 n_h d_h ([P2] §2.1.1)."""
    return 2 * n_h * d_h


def mla_cache_values_per_token(d_c: int = D_C, d_h_r: int = D_H_R) -> int:
    """Values MLA caches per token: c^KV plus the shared k^R, d_c + d_h^R ([P2] §2.1.3(D))."""
    return d_c + d_h_r


def default_scale(d_h: int = D_H, d_h_r: int = D_H_R) -> float:
    """Score scale 1/sqrt(d_h + d_h^R) ([P2] §2.1.3(D))."""
    return 1.0 / math.sqrt(d_h + d_h_r)


# --------------------------------------------------------------------------- fp8
def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Decode OCP E4M3 (e4m3fn) bytes to fp64.

    Bit layout: sign (1) | exponent (4, bias 7) | mantissa (3).  Exponent 0 is
    subnormal, value m/8 * 2^-6; otherwise (1 + m/8) * 2^(e-7).  There is no
    infinity; exponent 15 with mantissa 7 is NaN, so the largest finite value
    is 1.75 * 2^8 = 448 ([P5] "MLA 与 FP8": E4M3's range is about 448).
    """
    c = np.asarray(codes).astype(np.int64)
    sign = np.where((c & 0x80) != 0, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((e == 15) & ((c & 0x7) == 7), np.nan, mag)
    return sign * mag


def dequantize_latent(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """c[k] = e4m3(code[k]) * scale[k // 128]  (1x128 block scaling, [P1] §4.2)."""
    vals = e4m3_decode(codes)
    rep = np.repeat(np.asarray(scales, dtype=np.float64), FP8_BLOCK, axis=-1)
    return vals * rep


# ----------------------------------------------------------------------- paging
def sequence_pages(b: int, block_table, max_blocks: int) -> list:
    """Page ids of sequence b; without a table, page b*max_blocks + u holds rows 64u..64u+63."""
    if block_table is None:
        return [b * max_blocks + u for u in range(max_blocks)]
    return [int(p) for p in block_table[b]]


# -------------------------------------------------------------------- attention
def attend_latent(q_cat: np.ndarray, rows: np.ndarray, scale: float):
    """Absorbed decode attention of every head over the cached rows.

    q_cat: [H, d_c + d_h^R] = [q_absorbed ; q^R] per head.
    rows:  [n, d_c + d_h^R] = [c^KV ; k^R] per cached token.
    Scores z = scale * q_cat . row  ([P2] §2.1.3(B) absorption, (D) concatenation
    and scale); p = softmax_j(z); out = sum_j p_j c^KV_j, the latent-space output
    that W^UV would map per head ([P2] §2.1.2); lse = log sum_j exp(z_j).
    Returns (out [H, d_c], lse [H]) in fp64.
    """
    H = q_cat.shape[0]
    n = rows.shape[0]
    if n == 0:
        return np.zeros((H, D_C)), np.full((H,), -np.inf)
    z = scale * (q_cat @ rows.T)                 # [H, n]
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    s = e.sum(axis=1, keepdims=True)
    lse = (m + np.log(s))[:, 0]
    out = (e / s) @ rows[:, :D_C]
    return out, lse


def visible_rows(seq_len: int, s_q: int, s: int) -> int:
    """Rows query token s of S_q sees: seq_len - S_q + s + 1 (MTP causal reading, [P1] §3.3)."""
    return max(0, int(seq_len) - int(s_q) + int(s) + 1)


def _to64(t) -> np.ndarray:
    """Exact upcast of a bf16/fp32 torch tensor (or array) to fp64."""
    if hasattr(t, "detach"):
        return t.detach().to("cpu").double().numpy()
    return np.asarray(t, dtype=np.float64)


def sequence_rows(inp, b: int, n: int) -> np.ndarray:
    """The first n cached rows [c^KV ; k^R] of sequence b of an MlaInputs, in fp64."""
    pages = sequence_pages(b, None if inp.block_table is None else inp.block_table.numpy(), inp.max_blocks)
    bs = inp.cache.shape[1]
    need = (n + bs - 1) // bs
    pg = pages[:need]
    if n == 0:
        return np.zeros((0, D_ROW))
    if inp.cache_dtype == "bf16":
        blocks = _to64(inp.cache[pg])                       # [need, bs, 576]
        return blocks.reshape(-1, D_ROW)[:n]
    codes = inp.cache[pg].numpy()                           # uint8 [need, bs, 512]
    scales = inp.cache_scales[pg].numpy()                   # [need, bs, 4]
    lat = dequantize_latent(codes, scales)
    rope = _to64(inp.cache_rope[pg])
    return np.concatenate([lat, rope], axis=-1).reshape(-1, D_ROW)[:n]


def decode_one(inp, b: int, s: int, heads=None):
    """Oracle result for sequence b, query token s: (out [H, 512], lse [H]) fp64."""
    n = visible_rows(int(inp.seq_lens[b]), inp.s_q, s)
    rows = sequence_rows(inp, b, n)
    qa = _to64(inp.q_absorbed[b, s])
    qr = _to64(inp.q_rope[b, s])
    if heads is not None:
        qa, qr = qa[heads], qr[heads]
    q_cat = np.concatenate([qa, qr], axis=-1)
    return attend_latent(q_cat, rows, inp.scale)


def mla_decode(inp):
    """Full oracle over a batch: out [B, S_q, 128, 512] and lse [B, S_q, 128], fp64."""
    B, S = inp.batch, inp.s_q
    out = np.zeros((B, S, N_H, D_C))
    lse = np.zeros((B, S, N_H))
    for b in range(B):
        for s in range(S):
            out[b, s], lse[b, s] = decode_one(inp, b, s)
    return out, lse


# ---------------------------------------------------------------- split / merge
def partial_over_range(q_cat: np.ndarray, rows: np.ndarray, j0: int, j1: int, scale: float):
    """Attention restricted to rows [j0, j1): the (out_s, lse_s) partial of one split."""
    return attend_latent(q_cat, rows[j0:j1], scale)


def merge_partials(outs, lses):
    """Merge split partials by log-sum-exp.

    LSE = log sum_s exp(lse_s);  out = sum_s exp(lse_s - LSE) out_s.  A split that
    saw no rows has lse_s = -inf and weight 0.  This is an exact identity of the
    softmax over the union of the splits' rows.
    outs: [S, H, D], lses: [S, H].
    """
    outs = np.asarray(outs, dtype=np.float64)
    lses = np.asarray(lses, dtype=np.float64)
    m = lses.max(axis=0)                                  # [H]
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    w = np.exp(lses - m_safe[None, :])                    # -inf -> 0
    tot = w.sum(axis=0)
    lse = np.where(finite, m_safe + np.log(np.where(tot > 0, tot, 1.0)), -np.inf)
    wn = np.where(tot[None, :] > 0, w / np.where(tot > 0, tot, 1.0)[None, :], 0.0)
    out = (wn[:, :, None] * outs).sum(axis=0)
    return out, lse


# ------------------------------------------------------- unabsorbed cross-check
def unabsorbed_attention(q_c: np.ndarray, q_r: np.ndarray, c_kv: np.ndarray, k_r: np.ndarray,
                         W_UK: np.ndarray, W_UV: np.ndarray, scale: float):
    """The explicit per-head form the absorption replaces ([P2] §2.1.2, §2.1.3(D)).

    Per head h: k^C_j = W^UK_h c^KV_j and v^C_j = W^UV_h c^KV_j (each d_h = 128
    wide); score z_j = scale * (q^C_h . k^C_j + q^R_h . k^R_j);
    o_h = sum_j softmax(z)_j v^C_j.  Returns (o [H, d_h], lse [H], z [H, n]).
    """
    H = q_c.shape[0]
    n = c_kv.shape[0]
    o = np.zeros((H, W_UV.shape[1]))
    lse = np.zeros((H,))
    zs = np.zeros((H, n))
    for h in range(H):
        k_c = c_kv @ W_UK[h].T            # [n, d_h]
        v_c = c_kv @ W_UV[h].T            # [n, d_h]
        z = scale * (k_c @ q_c[h] + k_r @ q_r[h])
        m = z.max()
        e = np.exp(z - m)
        o[h] = (e / e.sum()) @ v_c
        lse[h] = m + math.log(e.sum())
        zs[h] = z
    return o, lse, zs


def absorb_query(q_c: np.ndarray, W_UK: np.ndarray) -> np.ndarray:
    """q_absorbed_h = W^UK_h^T q^C_h ([P2] §2.1.3(B)); [H, d_h] -> [H, d_c]."""
    return np.einsum("hdc,hd->hc", W_UK, q_c)


def apply_output_absorption(out_latent: np.ndarray, W_UV: np.ndarray) -> np.ndarray:
    """o_h = W^UV_h out_latent_h: the per-head value output recovered from latent space."""
    return np.einsum("hdc,hc->hd", W_UV, out_latent)
