// Delta_i = sum_d dO_id * O_id for every (b, h, i) row (rustytorch
// flash_attention_backward_dq.metal, header: D = rowsum(dO * O);
// ferrotensor-backend flash_attention_v2_backward.wgsl, pass-1 Delta).
//
// HBM-bound: each row is read once as 16-byte chunks by a group of lanes (with
// the streaming cache policy: nothing here is read again), multiplied in fp32
// and reduced across the group with DPP lane moves; a lane group takes several
// rows, their loads in flight together.
#include "fa_internal.h"

namespace fa {

// Each group of LPR lanes reduces RPG rows (RPG loads of O and of dO in flight
// per lane before the first sum), so a block covers RPG * 256 / LPR rows.
constexpr int kPreRowsPerGroup = 4;

template <typename T>
__device__ __forceinline__ typename Mma<T>::chunk ld16_nt(const T* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const typename Mma<T>::chunk*>(p));
}

template <typename T, int D>
__global__ __launch_bounds__(256) void preprocess_kernel(PrefillArgs a, const T* __restrict__ O,
                                                         const T* __restrict__ dO,
                                                         float* __restrict__ delta) {
  constexpr int CH = Mma<T>::CH;          // elements per 16-byte chunk
  constexpr int LPR = D / CH;             // lanes per row
  constexpr int GPB = 256 / LPR;          // lane groups per block
  constexpr int RPG = kPreRowsPerGroup;   // rows per lane group
  const int lane_in_row = threadIdx.x % LPR;
  const int64_t rows = (int64_t)a.B * a.Hq * a.Sq;
  // group g of block k takes rows (k * RPG + u) * GPB + g, u = 0 .. RPG-1
  const int64_t row0 = (int64_t)blockIdx.x * RPG * GPB + threadIdx.x / LPR;
  const bool lane_in = lane_in_row * CH < a.D;  // lanes past the head dimension add nothing
  typename Mma<T>::chunk o[RPG], g[RPG];
#pragma unroll
  for (int u = 0; u < RPG; ++u) {
    const int64_t row = row0 + (int64_t)u * GPB;
    o[u] = typename Mma<T>::chunk{};
    g[u] = typename Mma<T>::chunk{};
    if (row < rows && lane_in) {
      const int i = (int)(row % a.Sq);
      const int64_t bh = row / a.Sq;
      const int h = (int)(bh % a.Hq);
      const int b = (int)(bh / a.Hq);
      const int64_t off = (int64_t)b * a.qsb + (int64_t)i * a.qss + (int64_t)h * a.qsh + lane_in_row * CH;
      o[u] = ld16_nt<T>(O + off);
      g[u] = ld16_nt<T>(dO + off);
    }
  }
#pragma unroll
  for (int u = 0; u < RPG; ++u) {
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < CH; ++e) acc += to_f32(g[u][e]) * to_f32(o[u][e]);
    acc = group_sum<LPR>(acc);
    const int64_t row = row0 + (int64_t)u * GPB;
    if (row < rows && lane_in_row == 0) delta[row] = acc;
  }
}

template <typename T, int D>
static hipError_t launch(const PrefillArgs& a, const void* O, const void* dO, float* delta, hipStream_t st) {
  constexpr int LPR = D / Mma<T>::CH;
  constexpr int RPB = kPreRowsPerGroup * 256 / LPR;  // rows per block
  const int64_t rows = (int64_t)a.B * a.Hq * a.Sq;
  const unsigned grid = (unsigned)((rows + RPB - 1) / RPB);
  hipLaunchKernelGGL((preprocess_kernel<T, D>), dim3(grid), dim3(256), 0, st, a,
                     static_cast<const T*>(O), static_cast<const T*>(dO), delta);
  return hipGetLastError();
}

hipError_t launch_preprocess(const PrefillArgs& a, int dtype, int D, const void* O, const void* dO,
                             float* delta, hipStream_t st) {
  if (dtype == kBF16) return D <= 64 ? launch<__bf16, 64>(a, O, dO, delta, st) : launch<__bf16, 128>(a, O, dO, delta, st);
  return D <= 64 ? launch<float, 64>(a, O, dO, delta, st) : launch<float, 128>(a, O, dO, delta, st);
}

}  // namespace fa
