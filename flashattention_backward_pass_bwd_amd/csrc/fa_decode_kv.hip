// Decode-step backward, pass 2: the history gradients (rullama
// attention_backward_dq.wgsl, header comment: the pass after the one that
// produces d_scores; its code is not on the page).  For sequence n, KV head kv
// and history row j, summed over the G query heads h of the group:
//   dK_j = sum_h d_scores_hj q_h,   dV_j = sum_h probs_hj d_out_h
// (scores are the unscaled q_h . K_j, so no scale appears).
//
// gfx950 design: HBM-bound on the dK and dV writes (2 * len * Hkv * D floats
// per sequence against G * len * 2 floats read).  Block (256 threads) =
// (sequence, KV head, 64 history rows): the G heads' q and d_out rows sit in
// registers (lane l of a row's D/4 lanes owns d = 4l .. 4l+3), d_scores and
// probs of the block's rows are staged in LDS, and each row is written by D/4
// lanes as 16-byte streaming stores (whole rows, consecutive rows of a wave
// adjacent in memory).
#include "fa_internal.h"

namespace fa {

constexpr int kDkvRows = 64;  // history rows per block

template <int D, int G>
__global__ __launch_bounds__(256) void decode_kv_kernel(DecodeArgs a, const float* __restrict__ q,
                                                        const float* __restrict__ dout,
                                                        const float* __restrict__ probs,
                                                        const float* __restrict__ dscores,
                                                        float* __restrict__ dk, float* __restrict__ dv) {
  constexpr int LPR = D / 4;     // lanes per row
  constexpr int RPW = 64 / LPR;  // rows per wave and pass
  constexpr int RPP = 4 * RPW;   // rows per block and pass
  __shared__ float sds[G][kDkvRows];
  __shared__ float spr[G][kDkvRows];

  const int nblk = (a.len + kDkvRows - 1) / kDkvRows;
  const int blk = blockIdx.x % nblk;
  const int rest = blockIdx.x / nblk;
  const int kvh = rest % a.Hkv;
  const int n = rest / a.Hkv;
  const int j0 = blk * kDkvRows;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int lr = lane % LPR;
  const int rs = (tid >> 6) * RPW + lane / LPR;  // row of a pass
  const int h0 = kvh * G;

  for (int i = tid; i < G * kDkvRows; i += 256) {
    const int g = i / kDkvRows, r = i % kDkvRows, j = j0 + r;
    const int64_t o = ((int64_t)n * a.H + h0 + g) * a.len + j;
    sds[g][r] = j < a.len ? dscores[o] : 0.f;
    spr[g][r] = j < a.len ? probs[o] : 0.f;
  }
  f32x4 qv[G], ov[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const int64_t o = ((int64_t)n * a.H + h0 + g) * D + 4 * lr;
    qv[g] = *reinterpret_cast<const f32x4*>(q + o);
    ov[g] = *reinterpret_cast<const f32x4*>(dout + o);
  }
  __syncthreads();

#pragma unroll 4
  for (int r = rs; r < kDkvRows; r += RPP) {
    const int j = j0 + r;
    if (j >= a.len) break;
    f32x4 k4 = {0.f, 0.f, 0.f, 0.f}, v4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float s = sds[g][r], p = spr[g][r];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        k4[e] = __builtin_fmaf(s, qv[g][e], k4[e]);
        v4[e] = __builtin_fmaf(p, ov[g][e], v4[e]);
      }
    }
    const int64_t o = (((int64_t)n * a.len + j) * a.Hkv + kvh) * D + 4 * lr;
    __builtin_nontemporal_store(k4, reinterpret_cast<f32x4*>(dk + o));
    __builtin_nontemporal_store(v4, reinterpret_cast<f32x4*>(dv + o));
  }
}

template <int D, int G>
static hipError_t launch_t(const DecodeArgs& a, const float* q, const float* dout, const float* probs,
                           const float* dscores, float* dk, float* dv, hipStream_t st) {
  const int nblk = (a.len + kDkvRows - 1) / kDkvRows;
  const unsigned grid = (unsigned)((int64_t)a.N * a.Hkv * nblk);
  hipLaunchKernelGGL((decode_kv_kernel<D, G>), dim3(grid), dim3(256), 0, st, a, q, dout, probs, dscores, dk, dv);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_d(const DecodeArgs& a, const float* q, const float* dout, const float* probs,
                           const float* dscores, float* dk, float* dv, hipStream_t st) {
  switch (a.g) {
    case 1: return launch_t<D, 1>(a, q, dout, probs, dscores, dk, dv, st);
    case 2: return launch_t<D, 2>(a, q, dout, probs, dscores, dk, dv, st);
    case 4: return launch_t<D, 4>(a, q, dout, probs, dscores, dk, dv, st);
    default: return launch_t<D, 8>(a, q, dout, probs, dscores, dk, dv, st);
  }
}

hipError_t launch_decode_kv(const DecodeArgs& a, const float* q, const float* dout, const float* probs,
                            const float* dscores, float* dk, float* dv, hipStream_t st) {
  if (a.D == 64) return launch_d<64>(a, q, dout, probs, dscores, dk, dv, st);
  if (a.D == 128) return launch_d<128>(a, q, dout, probs, dscores, dk, dv, st);
  return launch_d<256>(a, q, dout, probs, dscores, dk, dv, st);
}

int decode_kv_rows_per_block() { return kDkvRows; }

}  // namespace fa
