/*
 * libmla: decode-step Multi-head Latent Attention over a paged latent cache,
 * for AMD Instinct MI355X (gfx950).
 *
 * The operation.  One decode step of attention over the cached history,
 * softmax(Q_t K^T) V (DeepSeek-V3 architecture notes, deepseek.csdn.net,
 * §2.1.1), in MLA's absorbed form: every cached token keeps one 576-value row,
 * the 512-wide latent c^KV followed by the 64-wide decoupled RoPE key k^R shared
 * by all heads (same page, §2.1.3(D); DeepSeek-V3 详解, yudonglee.me, §2.1).
 * W^UK is already folded into the query (§2.1.3(B): q^T W^UK c = (W^UK^T q)^T c),
 * so each of the 128 heads brings q_absorbed (512) and q_rope (64), and W^UV is
 * left for after the call (§2.1.2), so the output stays in the 512-wide latent
 * space.  For head h of query token s of sequence b:
 *
 *     z_j      = scale * ( q_absorbed . c^KV_j + q_rope . k^R_j ),   j < n
 *     lse      = log sum_j exp(z_j)                       (natural log)
 *     out      = sum_j exp(z_j - lse) c^KV_j              (512 values)
 *     n        = seq_len[b] - S_q + s + 1
 *
 * scale is normally 1/sqrt(d_h + d_h^R) = 1/sqrt(192) (§2.1.3(D)).  With
 * several query tokens (MTP speculative decoding, DeepSeek-V3 详解 §3.3)
 * seq_len counts every new row and token s does not see the rows of the
 * tokens after it.
 *
 * Conventions for every entry point:
 *   - Tensors are passed as mla_tensor descriptors (device pointer, dtype,
 *     rank, shape, strides in elements).  They must be densely packed
 *     row-major; the caller allocates and owns them.  Nothing is allocated,
 *     freed or synchronised inside the calls; all work is enqueued on `stream`.
 *   - Every descriptor is validated on the host before any launch: dtypes
 *     (MLA_ERR_DTYPE), ranks, shapes, strides, the head count 128 and the
 *     widths 512 / 64 / 576 (MLA_ERR_SHAPE), missing pointers (MLA_ERR_NULL),
 *     and data-pointer alignment (MLA_ERR_SHAPE): 16 bytes for bf16 / fp32 /
 *     e4m3 data the kernels move in 16-byte pieces (queries, cache rows and
 *     their e4m3 scales and rope, out_latent, the partials, the projection
 *     operands), 4 bytes for int32 arrays and lse.  A failed check returns its
 *     status and enqueues nothing.  The contents
 *     of device arrays (seq_lens, block_table) are the caller's contract and
 *     are not read on the host; mla_check_indices checks them on the device.
 *   - Calls on different streams may run concurrently as long as their output
 *     and workspace buffers do not overlap.
 *   - State: the library keeps, per device, the handle of its code object
 *     (loaded by mla_init or on the first call on that device, never
 *     unloaded, read-only afterwards), whether the device is a gfx950, and
 *     the address of mla_decode_noalloc's static scratch.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_NUM_HEADS 128   /* n_h */
#define MLA_LATENT_DIM 512  /* d_c */
#define MLA_ROPE_DIM 64     /* d_h^R */
#define MLA_HEAD_DIM 128    /* d_h, per-head width of the unabsorbed query and value */
#define MLA_ROW_DIM 576     /* d_c + d_h^R values cached per token */
#define MLA_BLOCK_SIZE 64   /* rows per cache page */
#define MLA_FP8_GROUP 128   /* latent values per fp8 scale */
#define MLA_MAX_SPLITS 65536
/* Most num_splits * S_q a call with partials takes (MLA_ERR_SHAPE above): the
 * kernels address a partial row's lse and descales with 32-bit offsets, which
 * hold up to 2 * 2^19 blocks of 128 rows (a partial_out of ~140 GB). */
#define MLA_MAX_SPLIT_TOKENS 524288
#define MLA_MAX_RANK 5

typedef enum mla_status {
  MLA_OK = 0,
  MLA_ERR_NULL = 1,        /* a required descriptor or its data pointer is NULL */
  MLA_ERR_DTYPE = 2,       /* a tensor has the wrong element type */
  MLA_ERR_SHAPE = 3,       /* rank, shape or strides inconsistent; H != 128; widths != 512/64/576 */
  MLA_ERR_UNSUPPORTED = 4, /* valid request this build does not implement (e.g. S_q > 64, block size 32) */
  MLA_ERR_LAUNCH = 5,      /* the HIP runtime refused a launch */
  MLA_ERR_DEVICE = 6,      /* the current device is not gfx950 or cannot be queried */
  MLA_ERR_SCRATCH = 7,     /* mla_decode_noalloc: num_splits * S_q above MLA_NOALLOC_MAX_SPLIT_TOKENS */
  /* not statuses: they make every int32 value a valid mla_status, so that
     mla_status_string may be given any number a caller holds */
  MLA_STATUS_RANGE_MIN_ = -2147483647 - 1,
  MLA_STATUS_RANGE_MAX_ = 2147483647
} mla_status;

typedef enum mla_dtype {
  MLA_DTYPE_BF16 = 0,
  MLA_DTYPE_FP32 = 1,
  MLA_DTYPE_INT32 = 2,
  MLA_DTYPE_FP8_E4M3 = 3,  /* OCP E4M3 (e4m3fn) bytes: no infinity, 0x7F / 0xFF are NaN, max 448 */
  MLA_DTYPE_UINT8 = 4      /* raw bytes (the partial_out workspace) */
} mla_dtype;

/* A device tensor: element (i0, i1, ..) sits at data + sum_k i_k * strides[k]
 * elements.  Only densely packed row-major tensors are accepted (the stride
 * of a dimension of size 1 is not checked). */
typedef struct mla_tensor {
  void* data;
  int32_t dtype;                 /* mla_dtype */
  int32_t rank;                  /* 1 .. MLA_MAX_RANK */
  int64_t shape[MLA_MAX_RANK];
  int64_t strides[MLA_MAX_RANK]; /* in elements */
} mla_tensor;

/*
 * The latent cache, in 64-row pages.  Row j of sequence b is slot (j % 64) of
 * page block_table[b][j / 64].  Without a block table the cache is
 * contiguous: page b * max_blocks + j / 64, where max_blocks = NB / B; rows
 * given as [B, L_cap, .] with L_cap a multiple of 64 are read the same way.
 *
 *   bf16 cache:  rows   bf16 [NB, 64, 576]   (c^KV then k^R), scales / rope data NULL
 *   e4m3 cache:  rows   e4m3 [NB, 64, 512]   (c^KV codes)
 *                scales fp32 [NB, 64, 4]     one per 128 latent values
 *                rope   bf16 [NB, 64, 64]    k^R
 *
 * e4m3 rows dequantize as e4m3(byte) * scale (fine-grained 1x128 scaling,
 * DeepSeek-V3 详解 §4.2; E4M3 range about 448, 拆解DeepSeek V3,
 * kongchang.com, "MLA 与 FP8"); scales must be positive normal numbers.
 * Page slots past a sequence's end are never read into the result: they may
 * hold any bits, NaN included.
 */
typedef struct mla_latent_cache {
  mla_tensor rows;
  mla_tensor scales;
  mla_tensor rope;
} mla_latent_cache;

/*
 * mla_decode: the split-KV decode kernel.
 *
 *   q_absorbed   bf16  [B, S_q, 128, 512]   W^UK^T q^C per head
 *   q_rope       bf16  [B, S_q, 128, 64]    rotated q^R per head
 *   cache        the latent cache above (host pointer to the descriptors)
 *   block_table  int32 [B, max_blocks]; NULL (or data NULL) = contiguous cache
 *   seq_lens     int32 [B]; requires 0 <= seq_len <= max_blocks * 64
 *   scale        score scale (1/sqrt(192) for DeepSeek-V3), finite
 *   out_latent   fp32  [B, S_q, 128, 512]
 *   lse          fp32  [B, S_q, 128]
 *   partial_out  uint8 [mla_partial_out_bytes(P, S_q)] (or larger), 16-byte aligned
 *   partial_lse  fp32  [P, 2, S_q, 128]
 *
 * S_q is 1 .. 64 (MLA_ERR_UNSUPPORTED above): the tokens run in groups of 4,
 * 2 and 1, one kernel launch each, and every group reads the rows again (the
 * decode of a few draft tokens, not a long prefill chunk).  The split count P is the
 * leading dimension of partial_lse (P = 1 when partial_lse is NULL): a power
 * of two, 1 .. MLA_MAX_SPLITS with P * S_q <= MLA_MAX_SPLIT_TOKENS, the number
 * of work partitions the rows of the
 * whole batch are cut into.  The rows of all sequences, in 64-row pages
 * (units; a sequence owns max(1, ceil(seq_len / 64)) of them), are dealt out
 * in order, so one partition can cover the tail of one sequence, whole
 * sequences and the head of another.  The shares are equal in cost rather
 * than in units: every sequence also weighs 3 units (its fixed cost), placed
 * before its pages, so unit j of sequence b sits at position
 * u0(b) + 3 (b + 1) + j (u0(b): the units of the sequences before it), and
 * partition p takes the units whose positions lie in [floor(p W / P),
 * floor((p + 1) W / P)), W = total units + 3 B.  mla_num_splits_hint() gives
 * a P for the device and the cache size.
 *
 * partial_out layout (a workspace: fp16 halves the bytes of fp32 partials
 * at a rounding of 2^-11 of the largest value, under the 2^-8 of the bf16
 * probabilities).  First P * 2 * S_q blocks (split, slot, token) of 128 x 512
 * fp16 values (131,072 bytes each), then, for the same blocks in the same
 * order, 512 fp32 descales each (2,048 bytes).  A block is four groups of 32
 * heads, 16384 values each, in the order the kernels' lanes hold them: the
 * value of head 32 j + 16 a + r (a < 2, r < 16) and latent column
 * 16 c + 4 g + i (c < 32, g < 4, i < 4) sits at index
 * 16384 j + 8 (64 c + 16 g + r) + 4 a + i of its block, and its descale d at
 * index 128 (c / 8) + 32 j + 2 r + a of the block's descales.  The partial
 * output is the fp16 value times d; d is a power of two chosen per (block,
 * column quarter c / 8, head) so that the largest |value| lies in
 * [2^14, 2^15) (d no smaller than 2^-90): 11 significant bits for every
 * element that matters.  partial_lse is plain [split, slot, token, head].
 *
 * A sequence whose rows all fall into one partition gets its final out_latent
 * and lse here.  A sequence cut across partitions leaves one normalised partial
 * (out_s, lse_s) per partition it touches; mla_combine then writes its final
 * result.  Always call mla_combine with the same partials after mla_decode.
 * A query that sees no row (seq_len < S_q) gets out = 0 and lse = -inf.
 */
mla_status mla_decode(const mla_tensor* q_absorbed, const mla_tensor* q_rope, const mla_latent_cache* cache,
                      const mla_tensor* block_table, const mla_tensor* seq_lens, float scale,
                      const mla_tensor* out_latent, const mla_tensor* lse, const mla_tensor* partial_out,
                      const mla_tensor* partial_lse, hipStream_t stream);

/*
 * mla_combine: merge the per-partition partials of every sequence that
 * mla_decode cut across partitions, by log-sum-exp:
 *     LSE = log sum_s exp(lse_s),   out = sum_s exp(lse_s - LSE) out_s,
 * an exact identity of the softmax over the union of the partitions' rows.
 * A partial with lse_s = -inf has weight 0.  Sequences that mla_decode already
 * finished are left untouched.  The split count is partial_lse's leading
 * dimension; seq_lens and the partials must be those of the preceding
 * mla_decode (they rebuild the same partition map).  With P = 1 there is
 * nothing to merge: no launch, partials may be NULL.
 */
mla_status mla_combine(const mla_tensor* partial_out, const mla_tensor* partial_lse, const mla_tensor* seq_lens,
                       const mla_tensor* out_latent, const mla_tensor* lse, hipStream_t stream);

/*
 * mla_decode_noalloc: mla_decode followed by mla_combine, with the split
 * partials in the library's own static device scratch instead of a caller's
 * workspace.  For callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * call allocates and frees nothing.  Arguments as mla_decode, except the
 * split count, given as num_splits (a power of two) with
 * num_splits * S_q <= MLA_NOALLOC_MAX_SPLIT_TOKENS (MLA_ERR_SCRATCH above):
 * the scratch holds MLA_NOALLOC_SCRATCH_BYTES (65.25 MiB) per device, taken
 * once by the device's code object and held until the process ends.  Its
 * address is looked up by mla_init (or by the first call on the device, which
 * then also loads the code object: call mla_init at set-up to keep that out
 * of the call).  Every call on a device shares that device's scratch and it
 * keeps the last call's partials (each call writes every partial it reads, so
 * nothing needs clearing): calls that overlap in time on one device, on any
 * streams, race and must be serialised by the caller.
 */
#define MLA_NOALLOC_MAX_SPLIT_TOKENS 256
#define MLA_NOALLOC_SCRATCH_BYTES 68419584  /* 256 x 2 x (131,072 + 2,048 + 512) */
mla_status mla_decode_noalloc(const mla_tensor* q_absorbed, const mla_tensor* q_rope, const mla_latent_cache* cache,
                              const mla_tensor* block_table, const mla_tensor* seq_lens, float scale,
                              const mla_tensor* out_latent, const mla_tensor* lse, int32_t num_splits,
                              hipStream_t stream);

/*
 * A split count P for mla_decode (0 on error): one work partition per compute
 * unit of `device` (per two with s_q = 2 or 3, per four with s_q >= 4), halved while
 * the cache capacity the block table allows, batch * max_blocks_per_seq pages
 * plus 3 units per sequence of fixed cost, would leave fewer than 4 units per
 * partition: short contexts then stay in few partitions and need little or no
 * merging.  max_blocks_per_seq <= 0 means unknown (no cap).
 */
int32_t mla_num_splits_hint(int32_t device, int32_t batch, int32_t s_q, int32_t max_blocks_per_seq);

/* Bytes of partial_out and partial_lse needed for (split count, s_q). */
size_t mla_partial_out_bytes(int32_t num_splits, int32_t s_q);
size_t mla_partial_lse_bytes(int32_t num_splits, int32_t s_q);

/*
 * The steps around the decode in one MLA attention layer.  RoPE (DeepSeek-V3
 * architecture notes §2.1.3(A), (D); the pages give no formula: this library
 * rotates consecutive pairs (x_{2i}, x_{2i+1}) of a 64-wide vector by the
 * angle pos * rope_base^(-2i/64), computed in fp64) acts on q^R and on the
 * cached k^R.  The position of query token s of sequence b, and of the cache
 * row it appends, is seq_len[b] - S_q + s.
 */

/*
 * mla_absorb_query: the decode's query inputs (§2.1.3(B): q^T W^UK c =
 * (W^UK^T q)^T c; §2.1.3(D)).
 *   q_c         bf16 [B, S_q, 128, 128]   q^C per head
 *   q_r         bf16 [B, S_q, 128, 64]    q^R per head, before RoPE
 *   w_uk_t      bf16 [128, 512, 128]      W^UK_h^T per head (W^UK_h is d_h x d_c; stored transposed,
 *                                          so each output feature's 128 weights are contiguous)
 *   seq_lens    int32 [B]                 positions seq_len - S_q + s
 *   rope_base   the RoPE base (10000), finite and positive
 *   q_absorbed  bf16 [B, S_q, 128, 512]   = W^UK_h^T q^C_h (fp32 accumulation, rounded once)
 *   q_rope      bf16 [B, S_q, 128, 64]    = RoPE(q^R, position); may be q_r itself (in place)
 * bf16 MFMA GEMM per head with the RoPE in the same launch; any S_q >= 1.  Data pointers
 * of q_c, q_r, w_uk_t, q_absorbed and q_rope 16-byte aligned.
 */
mla_status mla_absorb_query(const mla_tensor* q_c, const mla_tensor* q_r, const mla_tensor* w_uk_t,
                            const mla_tensor* seq_lens, float rope_base, const mla_tensor* q_absorbed,
                            const mla_tensor* q_rope, hipStream_t stream);

/*
 * mla_absorb_output: per-head values from the decode's latent-space output
 * (§2.1.2: v^C = W^UV c^KV, moved past the softmax by associativity,
 * §2.1.3(B)).
 *   out_latent  fp32 [B, S_q, 128, 512]   mla_decode's output
 *   w_uv        bf16 [128, 128, 512]      W^UV_h per head (d_h x d_c)
 *   out_values  fp32 [B, S_q, 128, 128]   = W^UV_h out_latent_h
 * bf16 MFMA GEMM per head (out_latent rounded to bf16 on load, fp32
 * accumulation).  Data pointers of out_latent, w_uv and out_values 16-byte
 * aligned.
 */
mla_status mla_absorb_output(const mla_tensor* out_latent, const mla_tensor* w_uv, const mla_tensor* out_values,
                             hipStream_t stream);

/*
 * mla_kv_project: the cache row of each new token before its RoPE (§2.1.2:
 * c^KV = W^DKV h; the decoupled key k = W^KR h of §2.1.3(D)).
 *   hidden  bf16 [T, d]     d a multiple of 128 (7168 for DeepSeek-V3, §3)
 *   w_kv    bf16 [576, d]   rows 0..511 W^DKV, rows 512..575 W^KR
 *   kv      fp32 [T, 576]   = [W^DKV h ; W^KR h]
 * bf16 MFMA GEMM with fp32 accumulation, K split over four waves.  hidden,
 * w_kv and kv 16-byte aligned.
 */
mla_status mla_kv_project(const mla_tensor* hidden, const mla_tensor* w_kv, const mla_tensor* kv,
                          hipStream_t stream);

/*
 * mla_kv_project_split: mla_kv_project with the d-deep contraction cut into S
 * slices over workgroups, for steps with few tokens (a few hundred tokens and
 * d = 7168 leave a 32 x 32 tiling with under a workgroup per compute unit).
 * Same arguments, plus
 *   workspace  fp32 [S, T, 576]   caller-owned partial sums, overwritten; S >= 1
 *                                 divides d / 128 (mla_kv_project_splits); must not
 *                                 overlap kv or the inputs
 * Slice s sums K values [s d / S, (s + 1) d / S) of every output on bf16
 * MFMA in fp32; a second kernel adds the S partials of each output in slice
 * order, so the result is the same on every run (it may differ from
 * mla_kv_project's in the last bits: another summation order).  S = 1 writes
 * kv directly.  hidden, w_kv, kv and workspace 16-byte aligned;
 * MLA_ERR_SHAPE for an S that does not divide d / 128.
 */
mla_status mla_kv_project_split(const mla_tensor* hidden, const mla_tensor* w_kv, const mla_tensor* kv,
                                const mla_tensor* workspace, hipStream_t stream);

/*
 * mla_kv_project_splits: the S for mla_kv_project_split that fills the GPU:
 * the largest divisor of d / 128 with (64-feature x 128-token tiles) x S at
 * most 256 (14 for 256 tokens and d = 7168).  0 for T < 1 or a d that
 * mla_kv_project does not take.  Host only.
 */
int32_t mla_kv_project_splits(int64_t tokens, int64_t d);

/*
 * mla_cache_append: write each new token's row into its page slot, the rows
 * mla_decode then reads (DeepSeek-V3 详解 §2.1: 576 values per token; §4.2:
 * fine-grained 1x128 fp8 scaling).
 *   kv           fp32 [B, S_q, 576]   [c^KV ; k] of the S_q new tokens (mla_kv_project)
 *   seq_lens     int32 [B]            lengths that already count the new tokens
 *   block_table  int32 [B, max_blocks], or NULL for a contiguous cache
 *   cache        the latent cache (bf16 or e4m3 bundle), written in place
 *   rope_base    the RoPE base (10000)
 * Row p = seq_len - S_q + s of sequence b gets [c^KV ; RoPE(k, p)]: bf16
 * (round to nearest even), or for an e4m3 cache, per 128-wide block,
 * scale = amax / 448 in fp32 (1 for an all-zero block), code = the e4m3 value
 * nearest to x / scale (fp32 quotient, ties to the even code, saturated at
 * +-448), and k^R in bf16.  A row whose position falls outside the block
 * table or whose page lies outside the cache is not written.  kv and the
 * cache rows 16-byte aligned.
 */
mla_status mla_cache_append(const mla_tensor* kv, const mla_tensor* seq_lens, const mla_tensor* block_table,
                            const mla_latent_cache* cache, float rope_base, hipStream_t stream);

/*
 * mla_check_indices: the device-side contract of mla_decode, checked on the
 * device (the host never reads seq_lens or block_table).  Enqueues one small
 * kernel on `stream` that writes into counts (int32 [2], device):
 *   counts[0] = sequences with seq_len < 0 or seq_len > max_blocks * 64,
 *   counts[1] = block-table entries of pages a sequence uses (j < ceil(seq_len/64))
 *               that are not in [0, NB).
 * Both zero means mla_decode reads only inside the cache.  Same descriptors
 * as mla_decode (only their shapes are used, plus the table and lengths).
 */
mla_status mla_check_indices(const mla_latent_cache* cache, const mla_tensor* block_table,
                             const mla_tensor* seq_lens, const mla_tensor* counts, hipStream_t stream);

/*
 * mla_init: load the library's code object on `device` now (otherwise the
 * first call on the device does it).  Idempotent and thread-safe.  A caller
 * that must not see the load inside a later call (graph capture, a serving
 * loop) calls it once at set-up.
 */
mla_status mla_init(int32_t device);

/* Static text for a status code. */
const char* mla_status_string(mla_status status);

/* Library version: major * 10000 + minor * 100 + patch. */
int32_t mla_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MLA_H_ */
