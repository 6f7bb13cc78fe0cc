/*
 * fa_bwd.h -- C ABI of libfa_bwd.so: the FlashAttention backward pass on
 * AMD MI355X (gfx950), hand-written HIP kernels.
 *
 * The operations are the ones stated on these pages (cited by page title and
 * the section of the page that states them):
 *   [metal-dq]  rustytorch, flash_attention_backward_dq.metal -- header
 *               comment and kernel body (dQ = scale * dS K, with
 *               dS = P * (dO V^T - D) and D = rowsum(dO * O); L is an input).
 *   [wgsl-fa2]  ferrotensor-backend 0.2.0, flash_attention_v2_backward.wgsl
 *               -- header comment (two atomic-free passes; dV_j =
 *               sum_i P_ij M_ij dO_i, dK_j = scale * sum_i dS_ij Q_i summed
 *               over the query heads sharing a KV head, dS_ij = P_ij *
 *               (M_ij dO_i.V_j - Delta_i)), the FlashBwdParams struct,
 *               fab2_visible, fab2_mask_at, fab2_q_off / fab2_kv_off.
 *   [wgsl-dec]  rullama 0.2.0, attention_backward_dq.wgsl -- header comment
 *               and phases A-C (decode-step backward: d_scores and d_q).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *   allocates nothing, keeps no pointer after returning, never synchronises,
 *   and only enqueues kernels on `stream` (a hipStream_t; NULL = the default
 *   stream).  Outputs are fully overwritten (never accumulated into): rows or
 *   keys that no element reaches receive exact zeros.
 * - Every argument check runs on the host before any HIP call, so a call that
 *   returns an error has launched nothing.  After launching, the library
 *   reports hipGetLastError() as FA_ERR_HIP.  Nothing throws across the ABI.
 * - NaN / Inf in inputs propagate.  A row whose every element is excluded
 *   (fully masked) has L = +inf; it contributes nothing and gets dQ = 0.
 */
#ifndef FA_BWD_H
#define FA_BWD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fa_status {
  FA_OK = 0,
  FA_ERR_NULL = -1,        /* a required pointer is NULL */
  FA_ERR_SHAPE = -2,       /* a size <= 0, or num_heads % num_kv_heads != 0 */
  FA_ERR_UNSUPPORTED = -3, /* head_dim (prefill: not a multiple of 8 up to 128), dtype, history length or
                              row stride outside the built kernels,
                              or seq_q, seq_k, causal_offset or window above 2^29,
                              or batch * num_heads * ceil(max(seq_q, seq_k) / 32) >= 2^31 */
  FA_ERR_ALIGN = -4,       /* base or row stride not a multiple of 16 bytes, or D not unit-stride */
  FA_ERR_ARG = -5,         /* dropout_p not in [0,1), causal_offset < 0, window < 0, bad stride,
                              scale zero or not finite */
  FA_ERR_HIP = -6,         /* the HIP runtime reported an error at launch */
  FA_ERR_SCRATCH = -7      /* the problem needs more dS workspace than the library-owned buffer holds */
} fa_status;

typedef enum fa_dtype {
  FA_DTYPE_F32 = 0,  /* fp32 storage, fp32 MFMA (v_mfma_f32_32x32x2_f32) */
  FA_DTYPE_BF16 = 1  /* bf16 storage, bf16 MFMA with fp32 accumulation */
} fa_dtype;

/* A hipStream_t, passed as an opaque pointer so this header needs no HIP header. */
typedef void* fa_stream_t;

/*
 * Parameters of one prefill backward problem ([wgsl-fa2] FlashBwdParams,
 * [metal-dq] FlashBackwardParams).
 *
 * Tensor layout: Q, O, dO, dQ are [batch, seq_q, num_heads, head_dim] and
 * K, V, dK, dV are [batch, seq_k, num_kv_heads, head_dim] in the sense of
 * *element strides*: element (b, s, h, d) of a query-side tensor sits at
 * b*q_stride_b + s*q_stride_s + h*q_stride_h + d (likewise kv_stride_* for
 * key-side tensors), so both [B,S,H,D] and [B,H,S,D] storage are expressed
 * by choosing the strides.  head_dim is unit-stride.  The four query-side
 * tensors share one stride set; the four key-side tensors share the other.
 * Since the outputs are written through them, each set must map distinct
 * (b, s, h, d) to distinct elements (FA_ERR_ARG otherwise; checked as:
 * taken by increasing stride, each dimension of extent > 1 steps past the
 * whole span of the smaller ones, head_dim first), so no stride of such a
 * dimension is 0.
 * The sequence strides q_stride_s and kv_stride_s may not exceed 2^24
 * elements (FA_ERR_UNSUPPORTED): tile copies use 32-bit row offsets.  For
 * bf16 with a mask, mask_stride_q and mask_stride_k must be below 2^22
 * elements and one (b, h) slice of the mask, ((seq_q-1)*mask_stride_q +
 * (seq_k-1)*mask_stride_k + 1)*4 bytes, must fit in 32 bits
 * (FA_ERR_UNSUPPORTED).
 * L (natural-log log-sum-exp from the forward) and Delta are fp32,
 * contiguous [batch, num_heads, seq_q].
 *
 * GQA: query head h reads KV head h / (num_heads / num_kv_heads)
 * (contiguous groups, [wgsl-fa2] flash_bwd_dq); dK/dV sum over the group.
 *
 * Visibility ([wgsl-fa2] fab2_visible), with qa = i + causal_offset:
 *   i < seq_q, j < seq_k, (!causal || j <= qa), (window == 0 || |j - qa| < window).
 * Mask ([wgsl-fa2] fab2_mask_at): if mask != NULL, the fp32 value at
 *   b*mask_stride_b + h*mask_stride_h + i*mask_stride_q + j*mask_stride_k
 * is added to the scaled score; an entry <= -1e30f excludes the element.
 * Strides may be 0 (broadcast).  Scores: S = scale * Q.K + mask.
 * Dropout: M_ij = keep(seed, b*num_heads + h, i, j) / (1 - dropout_p) with
 *   row = (b*num_heads + h)*seq_q + i            (mod 2^32)
 *   r   = fmix32(row + fmix32(seed))              (mod 2^32)
 *   keep iff fmix32(r ^ (j * 0x9E3779B9)) >= floor(dropout_p * 2^32)
 * where fmix32 is MurmurHash3's 32-bit finaliser; dropout_p == 0 means M == 1.
 */
typedef struct fa_bwd_params {
  int32_t dtype; /* fa_dtype of Q, K, V, O, dO, dQ, dK, dV */
  int32_t batch;
  int32_t num_heads;    /* Hq */
  int32_t num_kv_heads; /* Hkv, divides Hq */
  int32_t seq_q;
  int32_t seq_k;
  int32_t head_dim;     /* any multiple of 8 up to 128 (tiles are 64 or 128 wide, the tail zero-padded) */
  int64_t q_stride_b, q_stride_s, q_stride_h;    /* elements; Q, O, dO, dQ */
  int64_t kv_stride_b, kv_stride_s, kv_stride_h; /* elements; K, V, dK, dV */
  float scale;           /* softmax scale; finite, nonzero, with a finite fp32 reciprocal (else FA_ERR_ARG) */
  int32_t causal;        /* 0 or 1 */
  int32_t causal_offset; /* >= 0: query i sits at key position i + causal_offset */
  int32_t window;        /* 0 = no window */
  float dropout_p;       /* probability of dropping, in [0, 1) */
  uint32_t seed;
  const float* mask;     /* device pointer or NULL */
  int64_t mask_stride_b, mask_stride_h, mask_stride_q, mask_stride_k; /* elements, >= 0 */
} fa_bwd_params;

/*
 * Forward pass with the same conventions (bf16 or fp32): the O and L the
 * backward takes ([wgsl-fa2] header: the forward whose outputs the two passes
 * read, its online log-sum-exp sweep; [metal-dq] L as an input).  With S_ij =
 * scale * Q_i.K_j + mask_ij on counted (visible, unmasked) elements:
 *   L_i = ln sum_j exp(S_ij)  (+inf when no element of row i counts),
 *   O_i = sum_j exp(S_ij - L_i) M_ij V_j  (M the dropout multiplier; 0 rows
 *   when nothing counts).
 * Q, K, V, O as in fa_bwd_params (O shares Q's strides); L fp32, contiguous
 * [batch, num_heads, seq_q].  Errors as fa_bwd_dq.
 */
fa_status fa_fwd(const fa_bwd_params* p, const void* Q, const void* K, const void* V, void* O, float* L,
                 fa_stream_t stream);

/*
 * L alone, for a caller whose forward did not keep it ([wgsl-fa2] the dQ
 * pass's first sweep: the online log-sum-exp of the scores): the L of fa_fwd
 * (dropout does not enter it), without reading V or writing O.  bf16 or
 * fp32; errors as fa_fwd.
 */
fa_status fa_bwd_lse(const fa_bwd_params* p, const void* Q, const void* K, float* L, fa_stream_t stream);

/*
 * Delta_i = sum_d dO_id * O_id per (b, h, i), fp32 accumulation
 * ([metal-dq] D = rowsum(dO * O); [wgsl-fa2] pass-1 Delta).
 * O, dO: query-side tensors (dtype); delta: fp32 [batch, num_heads, seq_q].
 * Must run before fa_bwd_dkdv and fa_bwd_dq, which read delta.
 */
fa_status fa_bwd_preprocess(const fa_bwd_params* p, const void* O, const void* dO, float* delta,
                            fa_stream_t stream);

/*
 * Key-block-outer pass ([wgsl-fa2] flash_bwd_dk_dv): for each key j of each
 * KV head, summed over the query heads of its group and all queries i,
 *   dV_j = sum_i P_ij M_ij dO_i,   dK_j = scale * sum_i dS_ij Q_i,
 * with P_ij = exp(S_ij - L_i) on visible, unmasked elements (0 elsewhere) and
 * dS_ij = P_ij (M_ij dO_i.V_j - Delta_i).  No atomics; independent of fa_bwd_dq.
 * Q, dO: query-side; K, V, dK, dV: key-side; L, delta: fp32 [batch, num_heads, seq_q].
 */
fa_status fa_bwd_dkdv(const fa_bwd_params* p, const void* Q, const void* K, const void* V,
                      const void* dO, const float* L, const float* delta, void* dK, void* dV,
                      fa_stream_t stream);

/*
 * Query-block-outer pass ([metal-dq] kernel; [wgsl-fa2] flash_bwd_dq second
 * sweep, with L supplied): dQ_i = scale * sum_j dS_ij K_j.  No atomics.
 */
fa_status fa_bwd_dq(const fa_bwd_params* p, const void* Q, const void* K, const void* V,
                    const void* dO, const float* L, const float* delta, void* dQ,
                    fa_stream_t stream);

/*
 * The same two passes sharing dS through a caller-owned workspace (bf16 only):
 * fa_bwd_dkdv_ds computes exactly what fa_bwd_dkdv does and also stores every
 * visible tile's dS_ij ([wgsl-fa2] flash_bwd_dk_dv: the dS it forms for dK),
 * rounded to bf16 as its dK contraction uses it; fa_bwd_dq_ds then computes
 * dQ_i = scale * sum_j dS_ij K_j ([wgsl-fa2] flash_bwd_dq; [metal-dq] dQ sum)
 * from the stored dS instead of recomputing S, P, dP and dS.  Run
 * fa_bwd_dkdv_ds, then fa_bwd_dq_ds, on one stream (or order them); the
 * workspace's contents between the two calls are opaque.
 *
 * fa_bwd_ds_workspace_size: bytes of workspace the two calls need for *p:
 * batch * num_heads * T * 16384, T = the 64-row x 128-key tiles any element
 * of which is visible (about seq_q * seq_k / 8192 for a full matrix, half of
 * that when causal).  ds_ws: device memory, 16-byte aligned, at least that
 * many bytes (ws_bytes); the library keeps no pointer to it.
 * Errors as fa_bwd_dkdv, plus: FA_ERR_NULL (ds_ws or bytes NULL),
 * FA_ERR_UNSUPPORTED (dtype fp32), FA_ERR_ARG (ws_bytes too small),
 * FA_ERR_ALIGN (ds_ws not 16-byte aligned).  fa_bwd_dq_ds reads K and the
 * workspace only; it writes every element of dQ.
 */
fa_status fa_bwd_ds_workspace_size(const fa_bwd_params* p, uint64_t* bytes);
fa_status fa_bwd_dkdv_ds(const fa_bwd_params* p, const void* Q, const void* K, const void* V,
                         const void* dO, const float* L, const float* delta, void* dK, void* dV,
                         void* ds_ws, uint64_t ws_bytes, fa_stream_t stream);
fa_status fa_bwd_dq_ds(const fa_bwd_params* p, const void* K, const void* ds_ws, uint64_t ws_bytes,
                       void* dQ, fa_stream_t stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): both
 * passes of the shared-dS pair, fa_bwd_dkdv_ds then fa_bwd_dq_ds, in one
 * call, with the dS workspace in a buffer the library owns instead of a
 * caller-given one.  Writes dK, dV and dQ exactly as that pair does (the
 * same kernels, bitwise the same results).  The buffer is a static device
 * array of FA_BWD_NOALLOC_SCRATCH_BYTES on every GPU the library runs on,
 * held from the first launch on that GPU until the process ends; the call
 * itself allocates nothing.  Its contents are opaque and stay from one call
 * to the next; calls that overlap on one GPU (unordered streams) race on it,
 * so order them.  The stream must belong to the current device.
 * Errors as fa_bwd_dkdv_ds, plus FA_ERR_SCRATCH when
 * fa_bwd_ds_workspace_size(p) exceeds FA_BWD_NOALLOC_SCRATCH_BYTES (checked
 * before any launch).
 */
#define FA_BWD_NOALLOC_SCRATCH_BYTES (128u << 20)
fa_status fa_bwd_dkdv_dq_noalloc(const fa_bwd_params* p, const void* Q, const void* K, const void* V,
                                 const void* dO, const float* L, const float* delta, void* dQ, void* dK,
                                 void* dV, fa_stream_t stream);

/*
 * Decode-step backward, pass 1 ([wgsl-dec]): one query per head, unscaled
 * scores, probs supplied.  For each sequence n and head h (KV head
 * h / heads_per_kv):
 *   dp_j = d_out_h . V_j;  sum_pd = sum_j probs_hj dp_j;
 *   d_scores_hj = probs_hj (dp_j - sum_pd);  d_q_h = sum_j d_scores_hj K_j.
 * All tensors fp32, contiguous: k_hist, v_hist [num_seqs, history_len,
 * n_kv_heads, head_dim]; probs, d_scores [num_seqs, n_heads, history_len];
 * d_out, d_q [num_seqs, n_heads, head_dim].
 * head_dim in {64, 128, 256}; n_heads / n_kv_heads in {1, 2, 4, 8};
 * history_len <= fa_bwd_decode_max_history(p) (the LDS-resident limit).
 */
typedef struct fa_decode_params {
  int32_t num_seqs;
  int32_t n_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t history_len;
} fa_decode_params;

fa_status fa_bwd_decode(const fa_decode_params* p, const float* k_hist, const float* v_hist,
                        const float* probs, const float* d_out, float* d_scores, float* d_q,
                        fa_stream_t stream);

/*
 * Decode-step backward, pass 2 ([wgsl-dec] header: the pass after the one
 * producing d_scores, named there, its code not on the page): the history
 * gradients, summed over the query heads h of each KV head kv = h / heads_per_kv,
 *   dk_hist[n, j, kv] = sum_h d_scores[n, h, j] q[n, h],
 *   dv_hist[n, j, kv] = sum_h probs[n, h, j] d_out[n, h]
 * (scores are the unscaled q . K_j of fa_bwd_decode).  fp32, contiguous:
 * q, d_out [num_seqs, n_heads, head_dim]; probs, d_scores [num_seqs, n_heads,
 * history_len] (d_scores as fa_bwd_decode writes it); dk_hist, dv_hist
 * [num_seqs, history_len, n_kv_heads, head_dim], every element written.
 * head_dim in {64, 128, 256}; n_heads / n_kv_heads in {1, 2, 4, 8}; no limit on
 * history_len beyond 32-bit grid sizes.  Errors: FA_ERR_NULL, FA_ERR_SHAPE,
 * FA_ERR_UNSUPPORTED, FA_ERR_ALIGN (q, d_out, dk_hist, dv_hist not 16-byte
 * aligned; probs or d_scores not 4-byte aligned), FA_ERR_HIP.
 */
fa_status fa_bwd_decode_dkdv(const fa_decode_params* p, const float* q, const float* d_out,
                             const float* probs, const float* d_scores, float* dk_hist,
                             float* dv_hist, fa_stream_t stream);

/* Longest history fa_bwd_decode accepts for p's head grouping (0 if the grouping is unsupported). */
int32_t fa_bwd_decode_max_history(const fa_decode_params* p);

/* Static, human-readable name of a status code. */
const char* fa_bwd_status_string(fa_status s);

/*
 * Test hooks.  Both run the very device predicate / hash the kernels use.
 * out: device uint8 [batch, num_heads, seq_q, seq_k], fully written.
 *   fa_bwd_debug_visibility: 1 iff element (b,h,i,j) enters the softmax
 *     (visible and, with a mask, mask value > -1e30f), else 0.
 *   fa_bwd_debug_dropout_keep: the keep bit of every element (ignores
 *     visibility); all 1 when dropout_p == 0.
 */
fa_status fa_bwd_debug_visibility(const fa_bwd_params* p, uint8_t* out, fa_stream_t stream);
fa_status fa_bwd_debug_dropout_keep(const fa_bwd_params* p, uint8_t* out, fa_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FA_BWD_H */
