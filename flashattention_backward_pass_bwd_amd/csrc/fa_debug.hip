// Test hooks: materialise, for every (b, h, i, j), the counted-element
// predicate and the dropout keep bit, using the same device functions the
// backward kernels evaluate (visible, mask_at, drop_row_key, drop_keep).
#include "fa_internal.h"

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
