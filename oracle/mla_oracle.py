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


# =============================================== around the decode: the next rows
# The steps that feed the decode and consume its output in one MLA attention
# layer ([P2] §2.1.2, §2.1.3(B), (D)): the absorbed query with its rotated
# RoPE part, the latent-space output mapped back to per-head values, and the
# cache row of a new token (its projection, its RoPE key, its fp8 encoding).
#
# Readings where the pages are silent (each also listed in the design notes):
#  * RoPE ([P2] §2.1.3(A): a position-dependent rotation of q and k, LLaMA
#    style) rotates consecutive pairs (x_{2i}, x_{2i+1}) of a d-wide vector by
#    the angle pos * base^(-2i/d), base 10000, with no long-context frequency
#    scaling; both the query's q^R and the cached k^R use it.
#  * k^R of token t is RoPE(W^KR h_t, t) with W^KR of shape [d_h^R, d] and
#    c^KV_t = W^DKV h_t ([P2] §2.1.2), d = 7168 ([P2] §3).
#  * The position of query token s of sequence b is seq_len[b] - S_q + s (the
#    count of rows before it, the same reading as visible_rows).
#  * The fp8 encoding of a new row: per 128-wide block, amax = max |x|, scale =
#    amax / 448 rounded to fp32 (1 for an all-zero block), code = the e4m3
#    value nearest to x / scale (fp32 quotient), ties to the even code,
#    saturated to +-448 ([P1] §4.2; [P5] "MLA 与 FP8"); the quantizer works in
#    fp32 because that is where the kernel decides the codes.
ROPE_BASE = 10000.0


def rope(x, pos, base: float = ROPE_BASE) -> np.ndarray:
    """RoPE(x, pos): pairs (x_{2i}, x_{2i+1}) of the last dim rotated by
    pos * base^(-2i/d) ([P2] §2.1.3(A), (D)).  pos broadcasts over x's
    leading dims.  fp64."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    theta = base ** (-2.0 * np.arange(d // 2) / d)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * theta
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty(np.broadcast_shapes(x.shape, ang.shape[:-1] + (d,)))
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def token_positions(seq_lens, s_q: int) -> np.ndarray:
    """[B, S_q] positions of the query tokens: seq_len - S_q + s."""
    lens = np.asarray(seq_lens, dtype=np.int64)
    return lens[:, None] - s_q + np.arange(s_q)[None, :]


def query_side(q_c, q_r, W_UK, seq_lens, base: float = ROPE_BASE):
    """The decode's query inputs from the per-head query parts.

    q_c [B, S, H, d_h], q_r [B, S, H, d_h^R] (before rotation), W_UK [H, d_h, d_c].
    q_absorbed = W^UK_h^T q^C_h ([P2] §2.1.3(B)), q_rope = RoPE(q^R, position)
    ([P2] §2.1.3(D)).  Returns fp64 (q_absorbed [B, S, H, d_c], q_rope [B, S, H, d_h^R])."""
    q_c = np.asarray(q_c, dtype=np.float64)
    B, S = q_c.shape[:2]
    q_abs = np.einsum("hdc,bshd->bshc", np.asarray(W_UK, dtype=np.float64), q_c)
    pos = token_positions(seq_lens, S)
    q_rot = rope(q_r, pos[:, :, None])
    return q_abs, q_rot


def output_side(out_latent, W_UV) -> np.ndarray:
    """o_h = W^UV_h out_latent_h for every token ([P2] §2.1.2, §2.1.3(B)):
    out_latent [B, S, H, d_c], W_UV [H, d_h, d_c] -> [B, S, H, d_h], fp64."""
    return np.einsum("hdc,bshc->bshd", np.asarray(W_UV, dtype=np.float64), np.asarray(out_latent, dtype=np.float64))


def kv_project(h, W_DKV, W_KR) -> np.ndarray:
    """The cache row of each token before its RoPE: [c^KV ; W^KR h] with
    c^KV = W^DKV h ([P2] §2.1.2).  h [T, d], W_DKV [d_c, d], W_KR [d_h^R, d]
    -> [T, d_c + d_h^R], fp64."""
    h = np.asarray(h, dtype=np.float64)
    return np.concatenate([h @ np.asarray(W_DKV, dtype=np.float64).T, h @ np.asarray(W_KR, dtype=np.float64).T],
                          axis=-1)


_E4M3_FINITE = None


def _e4m3_table():
    """(values, codes) of the 127 non-negative finite e4m3 values, ascending."""
    global _E4M3_FINITE
    if _E4M3_FINITE is None:
        codes = np.arange(128)
        vals = e4m3_decode(codes)
        keep = np.isfinite(vals)
        _E4M3_FINITE = (vals[keep], codes[keep])
    return _E4M3_FINITE


def e4m3_nearest(v) -> np.ndarray:
    """OCP E4M3 code of the value nearest to each fp32 v (ties: the even
    code), saturated to +-448; NaN maps to 0x7F."""
    v = np.asarray(v, dtype=np.float64)
    vals, codes = _e4m3_table()
    a = np.minimum(np.abs(v), 448.0).reshape(-1, 1)
    dist = np.abs(vals[None, :] - a)                          # distance to every candidate
    best = dist == dist.min(axis=1, keepdims=True)
    # the nearest value; of two equally near ones, the one with the even code
    rank = np.where(best, np.where(codes[None, :] % 2 == 0, 0, 1), 2)
    out = codes[np.argmin(rank, axis=1)].astype(np.uint8).reshape(v.shape)
    out = np.where(np.isnan(v), np.uint8(0x7F), out)
    sign = (np.signbit(v) & ~np.isnan(v)).astype(np.uint8) << 7
    return (out | sign).astype(np.uint8)


def e4m3_quantize(x, block: int = FP8_BLOCK):
    """fp32 x [..., n] -> (codes uint8 [..., n], scales fp32 [..., n/block]):
    scale = fl32(amax / 448) (1 for an all-zero block), code =
    e4m3_nearest(fl32(x / scale)) ([P1] §4.2 1x128 scaling; [P5] range 448)."""
    x = np.asarray(x, dtype=np.float32)
    shp = x.shape
    xb = x.reshape(*shp[:-1], shp[-1] // block, block)
    amax = np.abs(xb).max(axis=-1)
    scales = np.where(amax > 0, np.float32(amax) / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    q = (xb / scales[..., None]).astype(np.float32)
    return e4m3_nearest(q).reshape(shp), scales


def to_bf16_bits(x) -> np.ndarray:
    """fp32 x -> bf16 bit patterns, round to nearest even (NaN stays NaN)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    return np.where(nan, np.uint16(0x7FC0), r)


def cache_append(kv, seq_lens, block_table, max_blocks: int, cache, base: float = ROPE_BASE):
    """Write the rows of the S_q new tokens of every sequence into the cache.

    kv [B, S_q, d_c + d_h^R] fp32: [c^KV ; W^KR h] of each new token (before
    RoPE).  Token s of sequence b is row p = seq_len - S_q + s: page
    block_table[b][p // 64] (contiguous: b * max_blocks + p // 64), slot p % 64.
    The stored row is [c^KV ; RoPE(W^KR h, p)].  cache: a dict of numpy arrays
    (modified copies are returned): {"rows": bf16 bits uint16 [NB, 64, 576]} or
    the e4m3 bundle {"rows": uint8 [NB, 64, 512], "scales": fp32 [NB, 64, 4],
    "rope": bf16 bits [NB, 64, 64]}.  bf16 values are round-to-nearest-even of
    the fp32 c^KV and of the fp64 rotated key; e4m3 rows through e4m3_quantize."""
    kv = np.asarray(kv, dtype=np.float32)
    B, S = kv.shape[:2]
    out = {k: np.array(v, copy=True) for k, v in cache.items()}
    fp8 = "scales" in out
    pos = token_positions(seq_lens, S)
    for b in range(B):
        for s in range(S):
            p = int(pos[b, s])
            if p < 0:
                continue
            page = (b * max_blocks + p // 64) if block_table is None else int(block_table[b][p // 64])
            slot = p % 64
            lat = kv[b, s, :D_C]
            k_r = rope(kv[b, s, D_C:].astype(np.float64), p).astype(np.float32)
            if fp8:
                codes, sc = e4m3_quantize(lat)
                out["rows"][page, slot] = codes
                out["scales"][page, slot] = sc
                out["rope"][page, slot] = to_bf16_bits(k_r)
            else:
                out["rows"][page, slot, :D_C] = to_bf16_bits(lat)
                out["rows"][page, slot, D_C:] = to_bf16_bits(k_r)
    return out
