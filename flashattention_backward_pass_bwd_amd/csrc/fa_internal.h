// Launchers shared between the kernel translation units and the C ABI layer.
// Every launcher assumes its arguments were validated by fa_api.cpp.
#pragma once

#include "fa_common.h"

namespace fa {

enum { kF32 = 0, kBF16 = 1 };

// Launch geometry of the prefill kernels (also used by the host for checks).
constexpr int kDkdvKeysPerWave = 32;
constexpr int kDkdvWaves = 4;
constexpr int kDkdvKeysPerBlock = kDkdvKeysPerWave * kDkdvWaves;
constexpr int kDqRowsPerWave = 32;
constexpr int kDqWaves = 4;
constexpr int kDqRowsPerBlock = kDqRowsPerWave * kDqWaves;
// The head-dimension-128 dQ kernel without window, mask or dropout: two 32-row blocks per wave.
constexpr int kDq2RowsPerWave = 64;
constexpr int kDq2RowsPerBlock = kDq2RowsPerWave * kDqWaves;

// A mask whose keys are contiguous and whose 4-key groups start on 16 bytes
// (rows, heads and batches on 16-byte strides, the base 16-byte aligned): the
// tile kernels then stage it with 16-byte copies.
inline bool mask_keys_contiguous(const PrefillArgs& a) {
  return a.mask != nullptr && a.msk == 1 && a.msq % 4 == 0 && a.msh % 4 == 0 && a.msb % 4 == 0 &&
         (reinterpret_cast<uintptr_t>(a.mask) & 15u) == 0;
}

struct DecodeArgs {
  int N, H, Hkv, D, len, g;
};

hipError_t launch_preprocess(const PrefillArgs& a, int dtype, int D, const void* O, const void* dO,
                             float* delta, hipStream_t st);
hipError_t launch_dkdv(const PrefillArgs& a, int dtype, int D, const void* Q, const void* K,
                       const void* V, const void* dO, const float* L, const float* delta, void* dK,
                       void* dV, hipStream_t st);
hipError_t launch_dkdv_bf16(const PrefillArgs& a, int D, const void* Q, const void* K, const void* V,
                            const void* dO, const float* L, const float* delta, void* dK, void* dV,
                            hipStream_t st);
hipError_t launch_dkdv_bf16_ws(const PrefillArgs& a, int D, const void* Q, const void* K, const void* V,
                               const void* dO, const float* L, const float* delta, void* dK, void* dV, void* ws,
                               hipStream_t st);
hipError_t launch_dqs_bf16(const PrefillArgs& a, int D, const void* K, const void* ws, void* dQ, hipStream_t st);
hipError_t launch_fwd_bf16(const PrefillArgs& a, int D, const void* Q, const void* K, const void* V, void* O,
                           float* L, hipStream_t st);
// The forward of either dtype (O == nullptr: L alone, V not read).
hipError_t launch_fwd(const PrefillArgs& a, int dtype, int D, const void* Q, const void* K, const void* V, void* O,
                      float* L, hipStream_t st);
hipError_t launch_dq_bf16(const PrefillArgs& a, int D, const void* Q, const void* K, const void* V,
                          const void* dO, const float* L, const float* delta, void* dQ, hipStream_t st);
hipError_t launch_dq2_bf16(const PrefillArgs& a, const void* Q, const void* K, const void* V, const void* dO,
                           const float* L, const float* delta, void* dQ, hipStream_t st);
hipError_t launch_dq(const PrefillArgs& a, int dtype, int D, const void* Q, const void* K,
                     const void* V, const void* dO, const float* L, const float* delta, void* dQ,
                     hipStream_t st);
hipError_t launch_decode(const DecodeArgs& a, const float* k_hist, const float* v_hist,
                         const float* probs, const float* d_out, float* d_scores, float* d_q,
                         hipStream_t st);
int decode_max_history(int g);
hipError_t launch_decode_kv(const DecodeArgs& a, const float* q, const float* dout, const float* probs,
                            const float* dscores, float* dk, float* dv, hipStream_t st);
int decode_kv_rows_per_block();
hipError_t launch_debug_visibility(const PrefillArgs& a, uint8_t* out, hipStream_t st);
hipError_t launch_debug_dropout(const PrefillArgs& a, uint8_t* out, hipStream_t st);
hipError_t launch_calib_mfma(const void* ops, float* sink, int blocks, int iters, hipStream_t st);
// Device address of the library-owned dS workspace on the current device (fetched once per device).
hipError_t noalloc_scratch(void** ptr);

}  // namespace fa
