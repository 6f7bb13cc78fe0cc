// Test hooks: materialise, for every (b, h, i, j), the counted-element
// predicate and the dropout keep bit, using the same device functions the
// backward kernels evaluate (visible, mask_at, drop_row_key, drop_keep).
// And a calibration kernel for the MFMA roofline: the bf16 MFMA rate the chip
// sustains on given operand data with every SIMD busy.
#include "fa_internal.h"
#include "fa_tiles.h"

namespace fa {

__global__ __launch_bounds__(256) void debug_visibility_kernel(PrefillArgs a, uint8_t* __restrict__ out) {
  const int64_t total = (int64_t)a.B * a.Hq * a.Sq * a.Sk;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int j = (int)(e % a.Sk);
    const int64_t r = e / a.Sk;
    const int i = (int)(r % a.Sq);
    const int64_t bh = r / a.Sq;
    const int h = (int)(bh % a.Hq);
    const int b = (int)(bh / a.Hq);
    bool ok = visible(a, i, j);
    if (ok && a.mask != nullptr) ok = !(mask_at(a, b, h, i, j) <= kMaskedSentinel);
    out[e] = ok ? 1 : 0;
  }
}

__global__ __launch_bounds__(256) void debug_dropout_kernel(PrefillArgs a, uint8_t* __restrict__ out) {
  const int64_t total = (int64_t)a.B * a.Hq * a.Sq * a.Sk;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int j = (int)(e % a.Sk);
    const int64_t r = e / a.Sk;
    const int i = (int)(r % a.Sq);
    const int64_t bh = r / a.Sq;
    const int h = (int)(bh % a.Hq);
    const int b = (int)(bh / a.Hq);
    out[e] = (!a.drop || drop_keep(drop_row_key(a, b, h, i), j, a.drop_thr)) ? 1 : 0;
  }
}

// Back-to-back v_mfma_f32_32x32x16_bf16 only: one wave per SIMD, four
// independent accumulator chains, the A operand rotating over four VGPR blocks
// and the B operand over four AGPR blocks (as in the tile kernels, no two
// neighbouring MFMAs read the same registers), nothing else in the loop.
// Thread t reads A block i from ops[t + 256 i] and B block i from
// ops[1024 + t + 256 i] (2048 16-byte values).  A sum of the accumulators
// goes to sink[block*256 + t] so the work cannot be dropped.
__global__ __launch_bounds__(256, 1) void calib_mfma_kernel(const bf16x8* __restrict__ ops, float* __restrict__ sink,
                                                            int iters) {
  const int t = threadIdx.x;
  bf16x8 av[4], bv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    av[i] = ops[t + 256 * i];
    bv[i] = ld16_op(ops + 1024 + t + 256 * i);
  }
  wait_all_vmem();
  f32x16 acc[4] = {};
  // two wait states between the VALU zeroing of the accumulators and the first MFMA
  asm volatile("s_nop 1" : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]));
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 32; ++j)
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc[j & 3]) : "v"(av[(j >> 2) & 3]), "a"(bv[(j >> 1) & 3]));
  }
  // wait states before the accumulators are read by VALU
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]));
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  sink[blockIdx.x * 256 + t] = s;
}

hipError_t launch_calib_mfma(const void* ops, float* sink, int blocks, int iters, hipStream_t st) {
  hipLaunchKernelGGL(calib_mfma_kernel, dim3(blocks), dim3(256), 0, st, static_cast<const bf16x8*>(ops), sink, iters);
  return hipGetLastError();
}

static unsigned grid_for(const PrefillArgs& a) {
  const int64_t total = (int64_t)a.B * a.Hq * a.Sq * a.Sk;
  int64_t g = (total + 255) / 256;
  return (unsigned)(g < 65536 ? (g > 0 ? g : 1) : 65536);
}

hipError_t launch_debug_visibility(const PrefillArgs& a, uint8_t* out, hipStream_t st) {
  hipLaunchKernelGGL(debug_visibility_kernel, dim3(grid_for(a)), dim3(256), 0, st, a, out);
  return hipGetLastError();
}

hipError_t launch_debug_dropout(const PrefillArgs& a, uint8_t* out, hipStream_t st) {
  hipLaunchKernelGGL(debug_dropout_kernel, dim3(grid_for(a)), dim3(256), 0, st, a, out);
  return hipGetLastError();
}

}  // namespace fa
