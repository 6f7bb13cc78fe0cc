// Decode-step backward, pass 1 (rullama attention_backward_dq.wgsl, header
// comment and phases A-C): one query per head, unscaled scores, probs given.
//   A: dp_j = d_out_h . V_j        B: sum_pd = sum_j probs_hj dp_j
//      d_scores_hj = probs_hj (dp_j - sum_pd)
//   C: d_q_h = sum_j d_scores_hj K_j
//
// gfx950 design: HBM-bound (K and V dominate the bytes), so one 512-thread
// block owns one (sequence, KV head) and serves all G query heads of the group
// from a single pass over V (phase A) and a single pass over K (phase C); every
// history row is read exactly once, with the streaming (nt) cache policy.  A
// row is read by D/8 lanes (8 floats each, as two float4 loads that each cover
// a contiguous segment of the row), so a wave reads 512/D rows at a time and
// loads are unrolled two deep.  dp, then d_scores, stay in LDS as [len][G]
// (64 KB at G = 4 and 4096 rows), so two blocks share a CU and one streams
// while the other sits in a barrier or the short phase B.  Row dot products reduce across the
// row's lanes with butterfly shuffles; the final d_q reduces across the rows of
// a wave through shuffles and then over the 16 waves through LDS.
#include "fa_internal.h"

namespace fa {

constexpr int kDecThreads = 512;
constexpr int kDecWaves = kDecThreads / 64;
constexpr int kDecLdsBytes = 160 * 1024;

// 16-byte load with the streaming cache policy (each history row is read once).
__device__ __forceinline__ f32x4 ldnt4(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
}

template <int D, int G>
__global__ __launch_bounds__(kDecThreads, 2) void decode_kernel(DecodeArgs a, const float* __restrict__ Kh,
                                                                 const float* __restrict__ Vh,
                                                                 const float* __restrict__ probs,
                                                                 const float* __restrict__ dout,
                                                                 float* __restrict__ dscores,
                                                                 float* __restrict__ dq) {
  constexpr int LPR = D / 8;              // lanes per history row
  constexpr int NV4 = 2;                  // float4 per lane per row
  constexpr int RPI = kDecThreads / LPR;  // rows per block sweep
  constexpr int kDecUnroll = G >= 8 ? 1 : 2;  // rows in flight per lane group
  extern __shared__ float smem[];         // [len][G] dp -> d_scores; later [waves][G][D] partial d_q
  __shared__ float red[kDecWaves][G];
  __shared__ float sum_pd[G];

  const int n = blockIdx.x / a.Hkv;
  const int kvh = blockIdx.x % a.Hkv;
  const int tid = threadIdx.x;
  const int wave = tid / 64;
  const int lane = tid % 64;
  const int lr = lane % LPR;
  const int rsub = tid / LPR;  // which row of a sweep this lane group reads
  const int len = a.len;
  const int64_t rowstride = (int64_t)a.Hkv * D;
  const float* Kb = Kh + ((int64_t)n * len * a.Hkv + kvh) * D + 4 * lr;
  const float* Vb = Vh + ((int64_t)n * len * a.Hkv + kvh) * D + 4 * lr;
  const int h0 = kvh * G;
  const float* pr = probs + ((int64_t)n * a.H + h0) * len;
  float* dsg = dscores + ((int64_t)n * a.H + h0) * len;

  // d_out of the G heads, this lane's slice: d = 4*LPR*c + 4*lr + (0..3).
  f32x4 go[G][NV4];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int c = 0; c < NV4; ++c)
      go[g][c] = *reinterpret_cast<const f32x4*>(dout + ((int64_t)n * a.H + h0 + g) * D + 4 * LPR * c + 4 * lr);

  // Phase A: dp_j for the G heads -> smem[j*G + g].
  for (int j0 = rsub; j0 < len; j0 += RPI * kDecUnroll) {
    f32x4 v[kDecUnroll][NV4];
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) {
      const int j = j0 + u * RPI;
#pragma unroll
      for (int c = 0; c < NV4; ++c)
        v[u][c] = j < len ? ldnt4(Vb + (int64_t)j * rowstride + 4 * LPR * c) : f32x4{};
    }
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) {
      const int j = j0 + u * RPI;
      float acc[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float s = 0.f;
#pragma unroll
        for (int c = 0; c < NV4; ++c)
          s += go[g][c][0] * v[u][c][0] + go[g][c][1] * v[u][c][1] + go[g][c][2] * v[u][c][2] +
               go[g][c][3] * v[u][c][3];
        acc[g] = s;
      }
#pragma unroll
      for (int g = 0; g < G; ++g)
        acc[g] = group_sum<LPR>(acc[g]);
      if (j < len && lr < G) {
        float val = acc[0];
#pragma unroll
        for (int g = 1; g < G; ++g) val = lr == g ? acc[g] : val;
        smem[j * G + lr] = val;
      }
    }
  }
  __syncthreads();

  // sum_pd[g] = sum_j probs_gj dp_gj.
  float part[G];
#pragma unroll
  for (int g = 0; g < G; ++g) part[g] = 0.f;
  for (int j = tid; j < len; j += kDecThreads)
#pragma unroll
    for (int g = 0; g < G; ++g) part[g] += pr[(int64_t)g * len + j] * smem[j * G + g];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    part[g] = group_sum<64>(part[g]);
  }
  if (lane == 0)
#pragma unroll
    for (int g = 0; g < G; ++g) red[wave][g] = part[g];
  __syncthreads();
  if (tid < G) {
    float s = 0.f;
    for (int w = 0; w < kDecWaves; ++w) s += red[w][tid];
    sum_pd[tid] = s;
  }
  __syncthreads();

  // Phase B: d_scores = probs (dp - sum_pd), to LDS and to HBM.
  for (int j = tid; j < len; j += kDecThreads)
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float ds = pr[(int64_t)g * len + j] * (smem[j * G + g] - sum_pd[g]);
      smem[j * G + g] = ds;
      dsg[(int64_t)g * len + j] = ds;
    }
  __syncthreads();

  // Phase C: d_q_g = sum_j d_scores_gj K_j, this lane's d-slice and rows.
  f32x4 acc[G][NV4];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int c = 0; c < NV4; ++c) acc[g][c] = f32x4{};
  for (int j0 = rsub; j0 < len; j0 += RPI * kDecUnroll) {
    f32x4 kk[kDecUnroll][NV4];
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) {
      const int j = j0 + u * RPI;
#pragma unroll
      for (int c = 0; c < NV4; ++c)
        kk[u][c] = j < len ? ldnt4(Kb + (int64_t)j * rowstride + 4 * LPR * c) : f32x4{};
    }
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) {
      const int j = j0 + u * RPI;
      if (j < len) {
        float ds[G];
#pragma unroll
        for (int g = 0; g < G; ++g) ds[g] = smem[j * G + g];
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int c = 0; c < NV4; ++c) acc[g][c] += ds[g] * kk[u][c];
      }
    }
  }
  // Reduce over the row groups of a wave (lanes lr, lr+LPR, ...) ...
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int c = 0; c < NV4; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[g][c][e] = strided_sum<LPR>(acc[g][c][e]);
      }
  __syncthreads();  // every wave is done reading d_scores from smem
  // ... then over the 16 waves through LDS: smem[wave][g][d].
  if (lane < LPR) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int c = 0; c < NV4; ++c)
        *reinterpret_cast<f32x4*>(&smem[(wave * G + g) * D + 4 * LPR * c + 4 * lr]) = acc[g][c];
  }
  __syncthreads();
  for (int o = tid; o < G * D; o += kDecThreads) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) s += smem[w * G * D + o];
    const int g = o / D;
    const int d = o % D;
    dq[((int64_t)n * a.H + h0 + g) * D + d] = s;
  }
}

static size_t decode_lds_floats(int len, int g, int D) {
  const size_t a = (size_t)len * g;
  const size_t b = (size_t)kDecWaves * g * D;
  return a > b ? a : b;
}

int decode_max_history(int g) {
  if (g != 1 && g != 2 && g != 4 && g != 8) return 0;
  const int reserve = 2048;  // static LDS of the kernel (reduction scratch) plus slack
  return (kDecLdsBytes - reserve) / (4 * g);
}

template <int D, int G>
static hipError_t launch_g(const DecodeArgs& a, const float* k, const float* v, const float* probs,
                           const float* d_out, float* d_scores, float* d_q, hipStream_t st) {
  const size_t lds = decode_lds_floats(a.len, G, D) * sizeof(float);
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_kernel<D, G>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_kernel<D, G>), dim3(a.N * a.Hkv), dim3(kDecThreads), lds, st, a, k, v,
                     probs, d_out, d_scores, d_q);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_dd(const DecodeArgs& a, const float* k, const float* v, const float* probs,
                            const float* d_out, float* d_scores, float* d_q, hipStream_t st) {
  switch (a.g) {
    case 1: return launch_g<D, 1>(a, k, v, probs, d_out, d_scores, d_q, st);
    case 2: return launch_g<D, 2>(a, k, v, probs, d_out, d_scores, d_q, st);
    case 4: return launch_g<D, 4>(a, k, v, probs, d_out, d_scores, d_q, st);
    default: return launch_g<D, 8>(a, k, v, probs, d_out, d_scores, d_q, st);
  }
}

hipError_t launch_decode(const DecodeArgs& a, const float* k, const float* v, const float* probs,
                         const float* d_out, float* d_scores, float* d_q, hipStream_t st) {
  if (a.D == 64) return launch_dd<64>(a, k, v, probs, d_out, d_scores, d_q, st);
  if (a.D == 128) return launch_dd<128>(a, k, v, probs, d_out, d_scores, d_q, st);
  return launch_dd<256>(a, k, v, probs, d_out, d_scores, d_q, st);
}

}  // namespace fa
