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
 * scale is normally 1/sqrt(d_h + d_h^R) = 1/sqrt(192) (§2.1.3(D)).  With two
 * query tokens (MTP speculative decoding, DeepSeek-V3 详解 §3.3) seq_len counts
 * both new rows and token 0 does not see token 1's row.
 *
 * Conventions for every entry point:
 *   - Tensor arguments are device pointers to densely packed row-major arrays;
 *     the caller allocates and owns them.  Nothing is allocated, freed or
 *     synchronised inside the library; all work is enqueued on `stream`.
 *   - Arguments are validated on the host before any launch; a failed check
 *     returns an error status and enqueues nothing.  The contents of device
 *     arrays (seq_lens, block_table) are the caller's contract and are not
 *     read on the host.
 *   - Calls on different streams may run concurrently as long as their output
 *     and partial buffers do not overlap.
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
#define MLA_ROW_DIM 576     /* d_c + d_h^R values cached per token */
#define MLA_BLOCK_SIZE 64   /* rows per cache page */
#define MLA_FP8_GROUP 128   /* latent values per fp8 scale */
#define MLA_MAX_SPLITS 65536

typedef enum mla_status {
  MLA_OK = 0,
  MLA_ERR_NULL = 1,        /* a required pointer is NULL */
  MLA_ERR_DTYPE = 2,       /* unsupported cache dtype */
  MLA_ERR_SHAPE = 3,       /* inconsistent or out-of-range sizes */
  MLA_ERR_UNSUPPORTED = 4, /* valid request this build does not implement (e.g. S_q > 2) */
  MLA_ERR_LAUNCH = 5,      /* the HIP runtime refused a launch */
  MLA_ERR_DEVICE = 6       /* the current device is not gfx950 or cannot be queried */
} mla_status;

typedef enum mla_cache_dtype {
  MLA_CACHE_BF16 = 0,     /* rows: bf16 [num_blocks, 64, 576]                        */
  MLA_CACHE_FP8_E4M3 = 1  /* rows: OCP e4m3 bytes [num_blocks, 64, 512];
                             scales: fp32 [num_blocks, 64, 4], one per 128 latent values;
                             rope: bf16 [num_blocks, 64, 64]                            */
} mla_cache_dtype;

/*
 * The latent cache.  Row j of sequence b is slot (j % 64) of page
 * block_table[b * max_blocks_per_seq + j / 64].  Without a block table the cache
 * is contiguous: [batch, max_blocks_per_seq * 64, .], i.e. page b *
 * max_blocks_per_seq + j / 64.  fp8 rows dequantize as e4m3(byte) * scale
 * (fine-grained 1x128 scaling, DeepSeek-V3 详解 §4.2; E4M3 range about 448,
 * 拆解DeepSeek V3, kongchang.com, "MLA 与 FP8").  Page slots past a sequence's
 * end are never read into the result: they may hold any bits, NaN included.
 */
typedef struct mla_latent_cache {
  int32_t dtype;        /* mla_cache_dtype */
  int32_t block_size;   /* must be MLA_BLOCK_SIZE */
  int64_t num_blocks;   /* pages in the pool (for bounds on the host side) */
  const void* rows;     /* see mla_cache_dtype */
  const float* scales;  /* fp8 only, else NULL */
  const void* rope;     /* fp8 only, else NULL */
} mla_latent_cache;

/*
 * mla_decode: the split-KV decode kernel.
 *
 *   q_absorbed   bf16  [batch, s_q, 128, 512]   W^UK^T q^C per head
 *   q_rope       bf16  [batch, s_q, 128, 64]    rotated q^R per head
 *   cache        host pointer to the cache descriptor above
 *   block_table  int32 [batch, max_blocks_per_seq], device; NULL = contiguous
 *   seq_lens     int32 [batch], device; requires s_q <= seq_len <= max_blocks_per_seq*64
 *   scale        score scale (1/sqrt(192) for DeepSeek-V3)
 *   num_splits   number of work partitions the rows of the whole batch are cut
 *                into: a power of two P, 1 .. MLA_MAX_SPLITS.  The rows of all
 *                sequences, in 64-row pages (units; a sequence owns
 *                max(1, ceil(seq_len / 64)) of them), are dealt out in order,
 *                so one partition can cover the tail of one sequence, whole
 *                sequences and the head of another.  The shares are equal in
 *                cost rather than in units: every sequence also weighs 3
 *                units (its fixed cost), placed before its pages, so unit j of
 *                sequence b sits at position u0(b) + 3 (b + 1) + j (u0(b): the
 *                units of the sequences before it), and partition p takes the
 *                units whose positions lie in [floor(p W / P),
 *                floor((p + 1) W / P)), W = total units + 3 batch.
 *                mla_num_splits_hint() gives one for the device and the cache size.
 *   partial_out  workspace of mla_partial_out_bytes(num_splits, s_q) bytes,
 *                16-byte aligned; may be NULL if num_splits == 1 (layout below)
 *   partial_lse  fp32 [num_splits, 2, s_q, 128]        may be NULL if num_splits == 1
 *   out_latent   fp32 [batch, s_q, 128, 512]
 *   lse          fp32 [batch, s_q, 128]
 *
 * partial_out layout.  First num_splits * 2 * s_q blocks (split, slot, token)
 * of 128 x 512 fp16 values (131,072 bytes each), then, for the same blocks in
 * the same order, 512 fp32 descales each (2,048 bytes).  A block is four
 * groups of 32 heads, 16384 values each, in the order the kernels' lanes hold
 * them: the value of head 32 j + 16 a + r (a < 2, r < 16) and latent column
 * 16 c + 4 g + i (c < 32, g < 4, i < 4) sits at index
 * 16384 j + 8 (64 c + 16 g + r) + 4 a + i of its block, and its descale d at
 * index 128 (c / 8) + 32 j + 2 r + a of the block's descales.  The partial
 * output is the fp16 value times d; d is a power of two chosen per (block,
 * column quarter c / 8, head) so that the largest |value| lies in
 * [2^14, 2^15) (d no smaller than 2^-90): 11 significant bits for every
 * element that matters.
 * partial_lse is plain [.., head] fp32.
 *
 * A sequence whose rows all fall into one partition gets its final out_latent
 * and lse here.  A sequence cut across partitions leaves one normalised partial
 * (out_s, lse_s) per partition it touches; mla_combine then writes its final
 * result.  Always call mla_combine with the same arguments after mla_decode.
 * A query that sees no row (seq_len < s_q) gets out = 0 and lse = -inf.
 */
mla_status mla_decode(const void* q_absorbed, const void* q_rope, const mla_latent_cache* cache,
                      const int32_t* block_table, int32_t max_blocks_per_seq, const int32_t* seq_lens,
                      int32_t batch, int32_t s_q, float scale, int32_t num_splits, void* partial_out,
                      float* partial_lse, float* out_latent, float* lse, hipStream_t stream);

/*
 * mla_combine: merge the per-partition partials of every sequence that
 * mla_decode cut across partitions, by log-sum-exp:
 *     LSE = log sum_s exp(lse_s),   out = sum_s exp(lse_s - LSE) out_s,
 * an exact identity of the softmax over the union of the partitions' rows.
 * A partial with lse_s = -inf has weight 0.  Sequences that mla_decode already
 * finished are left untouched.  seq_lens, batch, s_q and num_splits must equal
 * those of the preceding mla_decode (they rebuild the same partition map).
 */
mla_status mla_combine(const void* partial_out, const float* partial_lse, const int32_t* seq_lens,
                       int32_t batch, int32_t s_q, int32_t num_splits, float* out_latent, float* lse,
                       hipStream_t stream);

/*
 * A num_splits for mla_decode (0 on error): one work partition per compute
 * unit of `device` (per two with s_q = 2), halved while the cache capacity
 * the block table allows, batch * max_blocks_per_seq pages plus 3 units per
 * sequence of fixed cost, would leave fewer than 4 units per partition: short
 * contexts then stay in few partitions and need little or no merging.
 * max_blocks_per_seq <= 0 means unknown (no cap).
 */
int32_t mla_num_splits_hint(int32_t device, int32_t batch, int32_t s_q, int32_t max_blocks_per_seq);

/* Bytes of partial_out and partial_lse needed for (num_splits, s_q). */
size_t mla_partial_out_bytes(int32_t num_splits, int32_t s_q);
size_t mla_partial_lse_bytes(int32_t num_splits, int32_t s_q);

/* Static text for a status code. */
const char* mla_status_string(mla_status status);

/* Library version: major * 10000 + minor * 100 + patch. */
int32_t mla_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MLA_H_ */
