// C ABI of libfa_bwd.so (declared in include/fa_bwd.h).
//
// Every check runs here, on the host, before any HIP call; the launchers
// behind it assume validated arguments.  The library allocates nothing and
// only enqueues work on the caller's stream.
#include <math.h>

#include "fa_bwd.h"
#include "fa_bwd_calib.h"
#include "fa_internal.h"

namespace {

using fa::PrefillArgs;

int elem_bytes(int dtype) { return dtype == FA_DTYPE_BF16 ? 2 : 4; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int64_t kMaxSeq = int64_t(1) << 29;  // sequence lengths, causal offset, window
constexpr int64_t kMaxRowStride = int64_t(1) << 24;  // elements between consecutive rows
constexpr int64_t kMaxMaskStride = int64_t(1) << 22;  // mask row / column stride, elements (bf16 path)

// The outputs share the inputs' strides (dQ and O Q's, dK and dV K's), so a
// stride set must map distinct (b, s, h, d) to distinct elements, or blocks
// would write the same memory.  Sufficient: taken by increasing stride, every
// dimension of extent > 1 steps past the whole span of the smaller ones (the
// head_dim elements of a row first).
bool non_overlapping(int64_t head_dim, const int64_t (&st)[3], const int64_t (&ext)[3]) {
  int order[3] = {0, 1, 2};
  for (int i = 0; i < 3; ++i)
    for (int j = i + 1; j < 3; ++j)
      if (st[order[j]] < st[order[i]]) {
        const int t = order[i];
        order[i] = order[j];
        order[j] = t;
      }
  int64_t span = head_dim;  // elements from a row's first to one past the last seen so far
  for (int i = 0; i < 3; ++i) {
    const int k = order[i];
    if (ext[k] <= 1) continue;
    if (st[k] < span) return false;
    span += st[k] * (ext[k] - 1);
  }
  return true;
}

fa_status check_prefill(const fa_bwd_params* p, PrefillArgs* a) {
  if (p == nullptr) return FA_ERR_NULL;
  if (p->dtype != FA_DTYPE_F32 && p->dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED;
  if (p->batch <= 0 || p->num_heads <= 0 || p->num_kv_heads <= 0 || p->seq_q <= 0 || p->seq_k <= 0 ||
      p->head_dim <= 0)
    return FA_ERR_SHAPE;
  if (p->num_heads % p->num_kv_heads != 0) return FA_ERR_SHAPE;
  // any multiple of 8 up to 128: tiles are 64 or 128 wide, the tail zero-padded
  if (p->head_dim > 128 || p->head_dim % 8 != 0) return FA_ERR_UNSUPPORTED;
  if (p->seq_q > kMaxSeq || p->seq_k > kMaxSeq || p->causal_offset > kMaxSeq || p->window > kMaxSeq)
    return FA_ERR_UNSUPPORTED;
  // Grids count their blocks (a (b, head) pair times tiles of 32 or more rows
  // or keys) and kernels index (b, head) pairs in 32 bits.
  const int64_t heads = (int64_t)p->batch * p->num_heads;
  if (heads * ((p->seq_q + 31) / 32) >= (int64_t(1) << 31) || heads * ((p->seq_k + 31) / 32) >= (int64_t(1) << 31))
    return FA_ERR_UNSUPPORTED;
  if (p->causal != 0 && p->causal != 1) return FA_ERR_ARG;
  if (p->causal_offset < 0 || p->window < 0) return FA_ERR_ARG;
  if (!(p->dropout_p >= 0.0f && p->dropout_p < 1.0f)) return FA_ERR_ARG;  // also rejects NaN
  // The tile kernels seed the score chains with -L / scale: scale finite, nonzero, with a finite reciprocal.
  if (!isfinite(p->scale) || p->scale == 0.0f || !isfinite(1.0 / (double)p->scale) ||
      !isfinite((float)(1.0 / (double)p->scale)))
    return FA_ERR_ARG;
  const int64_t qs[3] = {p->q_stride_b, p->q_stride_s, p->q_stride_h};
  const int64_t ks[3] = {p->kv_stride_b, p->kv_stride_s, p->kv_stride_h};
  const int64_t per16 = 16 / elem_bytes(p->dtype);
  for (int i = 0; i < 3; ++i) {
    if (qs[i] < 0 || ks[i] < 0) return FA_ERR_ARG;
    if (qs[i] % per16 != 0 || ks[i] % per16 != 0) return FA_ERR_ALIGN;
  }
  const int64_t qe[3] = {p->batch, p->seq_q, p->num_heads};
  const int64_t ke[3] = {p->batch, p->seq_k, p->num_kv_heads};
  if (!non_overlapping(p->head_dim, qs, qe) || !non_overlapping(p->head_dim, ks, ke)) return FA_ERR_ARG;
  // Tile copies address rows by 32-bit byte offsets from a tile's first row.
  if (p->q_stride_s > kMaxRowStride || p->kv_stride_s > kMaxRowStride) return FA_ERR_UNSUPPORTED;
  int64_t mask_rec = 0;
  if (p->mask != nullptr) {
    if (p->mask_stride_b < 0 || p->mask_stride_h < 0 || p->mask_stride_q < 0 || p->mask_stride_k < 0)
      return FA_ERR_ARG;
    if ((reinterpret_cast<uintptr_t>(p->mask) & 3u) != 0) return FA_ERR_ALIGN;
    // The bf16 tile kernels read the mask of one (b, h) through a 32-bit byte
    // range with 24-bit row and column strides.
    if (p->mask_stride_q >= kMaxMaskStride || p->mask_stride_k >= kMaxMaskStride) {
      if (p->dtype == FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED;
    } else {
      mask_rec = ((int64_t)(p->seq_q - 1) * p->mask_stride_q + (int64_t)(p->seq_k - 1) * p->mask_stride_k + 1) * 4;
      if (mask_rec > (int64_t)UINT32_MAX && p->dtype == FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED;
    }
  }
  // Grid sizes (the kernels index blocks with 32-bit integers; the smallest
  // blocks, of the fp32 passes, hold 32 rows or 32 keys).
  const int64_t nq = (p->seq_q + 31) / 32;
  const int64_t nk = (p->seq_k + 31) / 32;
  if (nq * p->batch * p->num_heads >= (int64_t(1) << 31) || nk * p->batch * p->num_kv_heads >= (int64_t(1) << 31))
    return FA_ERR_UNSUPPORTED;

  a->B = p->batch;
  a->Hq = p->num_heads;
  a->Hkv = p->num_kv_heads;
  a->Sq = p->seq_q;
  a->Sk = p->seq_k;
  a->D = p->head_dim;
  a->group = p->num_heads / p->num_kv_heads;
  a->qsb = p->q_stride_b;
  a->qss = p->q_stride_s;
  a->qsh = p->q_stride_h;
  a->ksb = p->kv_stride_b;
  a->kss = p->kv_stride_s;
  a->ksh = p->kv_stride_h;
  a->scale = p->scale;
  a->scale_log2 = (float)((double)p->scale * 1.4426950408889634);
  a->inv_scale = (float)(1.0 / (double)p->scale);
  a->causal = p->causal;
  a->offset = p->causal_offset;
  a->window = p->window;
  const double pf = (double)p->dropout_p;  // the fp32 value, exactly
  a->drop = pf > 0.0 ? 1 : 0;
  a->drop_thr = (uint32_t)floor(pf * 4294967296.0);  // exact: an fp32 times 2^32
  a->drop_inv = (float)(1.0 / (1.0 - pf));
  a->seed_mix = fa::fmix32(p->seed);
  a->mask = p->mask;
  a->msb = p->mask_stride_b;
  a->msh = p->mask_stride_h;
  a->msq = p->mask_stride_q;
  a->msk = p->mask_stride_k;
  a->mask_rec = (uint32_t)(mask_rec > (int64_t)UINT32_MAX ? UINT32_MAX : mask_rec);
  return FA_OK;
}

fa_status hip_status(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

// dS workspace of the workspace entry points: bf16 only; fills in the tiles
// per (b, h) and the bytes needed (layout in fa_common.h).
fa_status check_ws(const fa_bwd_params* p, PrefillArgs* a, uint64_t* bytes) {
  fa_status s = check_prefill(p, a);
  if (s != FA_OK) return s;
  if (p->dtype != FA_DTYPE_BF16) return FA_ERR_UNSUPPORTED;
  const int nkb = (p->seq_k + fa::kWsKeys - 1) / fa::kWsKeys;
  const int64_t nqt = (p->seq_q + fa::kWsRows - 1) / fa::kWsRows;
  if (nqt * ((a->group + 3) / 4) * p->batch * p->num_kv_heads >= (int64_t(1) << 31)) return FA_ERR_UNSUPPORTED;
  int64_t tiles = 0;
  for (int kb = 0; kb < nkb; ++kb) {
    int ql, n;
    fa::ws_run(*a, kb, ql, n);
    tiles += n;
  }
  a->ws_tiles = tiles;
  *bytes = (uint64_t)tiles * (uint64_t)p->batch * (uint64_t)p->num_heads * (uint64_t)fa::kWsTileBytes;
  return FA_OK;
}

hipStream_t as_stream(fa_stream_t s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

fa_status fa_bwd_preprocess(const fa_bwd_params* p, const void* O, const void* dO, float* delta,
                            fa_stream_t stream) {
  PrefillArgs a;
  if (p == nullptr || O == nullptr || dO == nullptr || delta == nullptr) return FA_ERR_NULL;
  fa_status s = check_prefill(p, &a);
  if (s != FA_OK) return s;
  if (!aligned16(O) || !aligned16(dO) || (reinterpret_cast<uintptr_t>(delta) & 3u)) return FA_ERR_ALIGN;
  return hip_status(fa::launch_preprocess(a, p->dtype, p->head_dim, O, dO, delta, as_stream(stream)));
}

fa_status fa_bwd_dkdv(const fa_bwd_params* p, const void* Q, const void* K, const void* V,
                      const void* dO, const float* L, const float* delta, void* dK, void* dV,
                      fa_stream_t stream) {
  PrefillArgs a;
  if (p == nullptr || Q == nullptr || K == nullptr || V == nullptr || dO == nullptr || L == nullptr ||
      delta == nullptr || dK == nullptr || dV == nullptr)
    return FA_ERR_NULL;
  fa_status s = check_prefill(p, &a);
  if (s != FA_OK) return s;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(dO) || !aligned16(dK) || !aligned16(dV) ||
      (reinterpret_cast<uintptr_t>(L) & 3u) || (reinterpret_cast<uintptr_t>(delta) & 3u))
    return FA_ERR_ALIGN;
  return hip_status(fa::launch_dkdv(a, p->dtype, p->head_dim, Q, K, V, dO, L, delta, dK, dV, as_stream(stream)));
}

fa_status fa_bwd_dq(const fa_bwd_params* p, const void* Q, const void* K, const void* V,
                    const void* dO, const float* L, const float* delta, void* dQ,
                    fa_stream_t stream) {
  PrefillArgs a;
  if (p == nullptr || Q == nullptr || K == nullptr || V == nullptr || dO == nullptr || L == nullptr ||
      delta == nullptr || dQ == nullptr)
    return FA_ERR_NULL;
  fa_status s = check_prefill(p, &a);
  if (s != FA_OK) return s;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(dO) || !aligned16(dQ) ||
      (reinterpret_cast<uintptr_t>(L) & 3u) || (reinterpret_cast<uintptr_t>(delta) & 3u))
    return FA_ERR_ALIGN;
  return hip_status(fa::launch_dq(a, p->dtype, p->head_dim, Q, K, V, dO, L, delta, dQ, as_stream(stream)));
}

fa_status fa_bwd_ds_workspace_size(const fa_bwd_params* p, uint64_t* bytes) {
  PrefillArgs a;
  if (p == nullptr || bytes == nullptr) return FA_ERR_NULL;
  return check_ws(p, &a, bytes);
}

fa_status fa_bwd_dkdv_ds(const fa_bwd_params* p, const void* Q, const void* K, const void* V, const void* dO,
                         const float* L, const float* delta, void* dK, void* dV, void* ds_ws, uint64_t ws_bytes,
                         fa_stream_t stream) {
  PrefillArgs a;
  uint64_t need = 0;
  if (p == nullptr || Q == nullptr || K == nullptr || V == nullptr || dO == nullptr || L == nullptr ||
      delta == nullptr || dK == nullptr || dV == nullptr || ds_ws == nullptr)
    return FA_ERR_NULL;
  fa_status s = check_ws(p, &a, &need);
  if (s != FA_OK) return s;
  if (ws_bytes < need) return FA_ERR_ARG;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(dO) || !aligned16(dK) || !aligned16(dV) ||
      !aligned16(ds_ws) || (reinterpret_cast<uintptr_t>(L) & 3u) || (reinterpret_cast<uintptr_t>(delta) & 3u))
    return FA_ERR_ALIGN;
  return hip_status(
      fa::launch_dkdv_bf16_ws(a, p->head_dim, Q, K, V, dO, L, delta, dK, dV, ds_ws, as_stream(stream)));
}

fa_status fa_bwd_dq_ds(const fa_bwd_params* p, const void* K, const void* ds_ws, uint64_t ws_bytes, void* dQ,
                       fa_stream_t stream) {
  PrefillArgs a;
  uint64_t need = 0;
  if (p == nullptr || K == nullptr || ds_ws == nullptr || dQ == nullptr) return FA_ERR_NULL;
  fa_status s = check_ws(p, &a, &need);
  if (s != FA_OK) return s;
  if (ws_bytes < need) return FA_ERR_ARG;
  if (!aligned16(K) || !aligned16(ds_ws) || !aligned16(dQ)) return FA_ERR_ALIGN;
  return hip_status(fa::launch_dqs_bf16(a, p->head_dim, K, ds_ws, dQ, as_stream(stream)));
}

fa_status fa_bwd_dkdv_dq_noalloc(const fa_bwd_params* p, const void* Q, const void* K, const void* V,
                                 const void* dO, const float* L, const float* delta, void* dQ, void* dK, void* dV,
                                 fa_stream_t stream) {
  PrefillArgs a;
  uint64_t need = 0;
  if (p == nullptr || Q == nullptr || K == nullptr || V == nullptr || dO == nullptr || L == nullptr ||
      delta == nullptr || dQ == nullptr || dK == nullptr || dV == nullptr)
    return FA_ERR_NULL;
  fa_status s = check_ws(p, &a, &need);
  if (s != FA_OK) return s;
  if (need > (uint64_t)FA_BWD_NOALLOC_SCRATCH_BYTES) return FA_ERR_SCRATCH;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(dO) || !aligned16(dQ) || !aligned16(dK) ||
      !aligned16(dV) || (reinterpret_cast<uintptr_t>(L) & 3u) || (reinterpret_cast<uintptr_t>(delta) & 3u))
    return FA_ERR_ALIGN;
  void* ws = nullptr;
  if (fa::noalloc_scratch(&ws) != hipSuccess) return FA_ERR_HIP;
  const hipStream_t st = as_stream(stream);
  s = hip_status(fa::launch_dkdv_bf16_ws(a, p->head_dim, Q, K, V, dO, L, delta, dK, dV, ws, st));
  if (s != FA_OK) return s;
  return hip_status(fa::launch_dqs_bf16(a, p->head_dim, K, ws, dQ, st));
}

fa_status fa_fwd(const fa_bwd_params* p, const void* Q, const void* K, const void* V, void* O, float* L,
                 fa_stream_t stream) {
  PrefillArgs a;
  if (p == nullptr || Q == nullptr || K == nullptr || V == nullptr || O == nullptr || L == nullptr) return FA_ERR_NULL;
  fa_status s = check_prefill(p, &a);
  if (s != FA_OK) return s;
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || (reinterpret_cast<uintptr_t>(L) & 3u))
    return FA_ERR_ALIGN;
  return hip_status(fa::launch_fwd(a, p->dtype, p->head_dim, Q, K, V, O, L, as_stream(stream)));
}

fa_status fa_bwd_lse(const fa_bwd_params* p, const void* Q, const void* K, float* L, fa_stream_t stream) {
  PrefillArgs a;
  if (p == nullptr || Q == nullptr || K == nullptr || L == nullptr) return FA_ERR_NULL;
  fa_status s = check_prefill(p, &a);
  if (s != FA_OK) return s;
  if (!aligned16(Q) || !aligned16(K) || (reinterpret_cast<uintptr_t>(L) & 3u)) return FA_ERR_ALIGN;
  return hip_status(fa::launch_fwd(a, p->dtype, p->head_dim, Q, K, nullptr, nullptr, L, as_stream(stream)));
}

int32_t fa_bwd_decode_max_history(const fa_decode_params* p) {
  if (p == nullptr || p->n_kv_heads <= 0 || p->n_heads <= 0 || p->n_heads % p->n_kv_heads != 0) return 0;
  return fa::decode_max_history(p->n_heads / p->n_kv_heads);
}

fa_status fa_bwd_decode(const fa_decode_params* p, const float* k_hist, const float* v_hist,
                        const float* probs, const float* d_out, float* d_scores, float* d_q,
                        fa_stream_t stream) {
  if (p == nullptr || k_hist == nullptr || v_hist == nullptr || probs == nullptr || d_out == nullptr ||
      d_scores == nullptr || d_q == nullptr)
    return FA_ERR_NULL;
  if (p->num_seqs <= 0 || p->n_heads <= 0 || p->n_kv_heads <= 0 || p->head_dim <= 0 || p->history_len <= 0)
    return FA_ERR_SHAPE;
  if (p->n_heads % p->n_kv_heads != 0) return FA_ERR_SHAPE;
  const int g = p->n_heads / p->n_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8) return FA_ERR_UNSUPPORTED;
  if (p->head_dim != 64 && p->head_dim != 128 && p->head_dim != 256) return FA_ERR_UNSUPPORTED;
  if (p->history_len > fa::decode_max_history(g)) return FA_ERR_UNSUPPORTED;
  if ((int64_t)p->num_seqs * p->n_kv_heads >= (int64_t(1) << 31)) return FA_ERR_UNSUPPORTED;
  if (!aligned16(k_hist) || !aligned16(v_hist) || !aligned16(d_out) || !aligned16(d_q) ||
      (reinterpret_cast<uintptr_t>(probs) & 3u) || (reinterpret_cast<uintptr_t>(d_scores) & 3u))
    return FA_ERR_ALIGN;
  fa::DecodeArgs a{p->num_seqs, p->n_heads, p->n_kv_heads, p->head_dim, p->history_len, g};
  return hip_status(fa::launch_decode(a, k_hist, v_hist, probs, d_out, d_scores, d_q, as_stream(stream)));
}

fa_status fa_bwd_decode_dkdv(const fa_decode_params* p, const float* q, const float* d_out, const float* probs,
                             const float* d_scores, float* dk_hist, float* dv_hist, fa_stream_t stream) {
  if (p == nullptr || q == nullptr || d_out == nullptr || probs == nullptr || d_scores == nullptr ||
      dk_hist == nullptr || dv_hist == nullptr)
    return FA_ERR_NULL;
  if (p->num_seqs <= 0 || p->n_heads <= 0 || p->n_kv_heads <= 0 || p->head_dim <= 0 || p->history_len <= 0)
    return FA_ERR_SHAPE;
  if (p->n_heads % p->n_kv_heads != 0) return FA_ERR_SHAPE;
  const int g = p->n_heads / p->n_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8) return FA_ERR_UNSUPPORTED;
  if (p->head_dim != 64 && p->head_dim != 128 && p->head_dim != 256) return FA_ERR_UNSUPPORTED;
  const int64_t nblk = (p->history_len + fa::decode_kv_rows_per_block() - 1) / fa::decode_kv_rows_per_block();
  if ((int64_t)p->num_seqs * p->n_kv_heads * nblk >= (int64_t(1) << 31)) return FA_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(d_out) || !aligned16(dk_hist) || !aligned16(dv_hist) ||
      (reinterpret_cast<uintptr_t>(probs) & 3u) || (reinterpret_cast<uintptr_t>(d_scores) & 3u))
    return FA_ERR_ALIGN;
  fa::DecodeArgs a{p->num_seqs, p->n_heads, p->n_kv_heads, p->head_dim, p->history_len, g};
  return hip_status(fa::launch_decode_kv(a, q, d_out, probs, d_scores, dk_hist, dv_hist, as_stream(stream)));
}

const char* fa_bwd_status_string(fa_status s) {
  switch (s) {
    case FA_OK: return "FA_OK";
    case FA_ERR_NULL: return "FA_ERR_NULL: a required pointer is NULL";
    case FA_ERR_SHAPE: return "FA_ERR_SHAPE: a size is <= 0 or num_heads is not a multiple of num_kv_heads";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: head_dim, dtype, grouping or length outside the built kernels";
    case FA_ERR_ALIGN: return "FA_ERR_ALIGN: a base pointer or row stride is not 16-byte aligned";
    case FA_ERR_ARG: return "FA_ERR_ARG: invalid scalar argument (dropout_p, causal, offset, window, stride or scale)";
    case FA_ERR_HIP: return "FA_ERR_HIP: the HIP runtime reported an error";
    case FA_ERR_SCRATCH: return "FA_ERR_SCRATCH: the problem needs more dS workspace than the library-owned buffer holds";
  }
  return "unknown fa_status";
}

fa_status fa_bwd_debug_visibility(const fa_bwd_params* p, uint8_t* out, fa_stream_t stream) {
  PrefillArgs a;
  if (p == nullptr || out == nullptr) return FA_ERR_NULL;
  fa_status s = check_prefill(p, &a);
  if (s != FA_OK) return s;
  return hip_status(fa::launch_debug_visibility(a, out, as_stream(stream)));
}

fa_status fa_bwd_debug_dropout_keep(const fa_bwd_params* p, uint8_t* out, fa_stream_t stream) {
  PrefillArgs a;
  if (p == nullptr || out == nullptr) return FA_ERR_NULL;
  fa_status s = check_prefill(p, &a);
  if (s != FA_OK) return s;
  return hip_status(fa::launch_debug_dropout(a, out, as_stream(stream)));
}

fa_status fa_bwd_calib_mfma_bf16(const void* operands, float* sink, int32_t blocks, int32_t iters,
                                 fa_stream_t stream) {
  if (operands == nullptr || sink == nullptr) return FA_ERR_NULL;
  if (blocks <= 0 || iters <= 0) return FA_ERR_ARG;
  if ((reinterpret_cast<uintptr_t>(operands) & 15u) != 0) return FA_ERR_ALIGN;
  return hip_status(fa::launch_calib_mfma(operands, sink, blocks, iters, as_stream(stream)));
}

}  // extern "C"
