// Device-side building blocks shared by the gfx950 attention-backward kernels:
// the launch-argument block, the element visibility / mask / dropout rules,
// and the 32x32 MFMA operand helpers.  Internal to libfa_bwd.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kMaskedSentinel = -1.0e30f;  // an additive mask entry <= this excludes the element

// Everything a prefill kernel needs, resolved on the host (passed by value).
struct PrefillArgs {
  int B, Hq, Hkv, Sq, Sk, group;  // group = Hq / Hkv
  int D;                          // head_dim: a multiple of 8 up to the kernel's tile width (64 or 128)
  int64_t qsb, qss, qsh;          // element strides of Q, O, dO, dQ
  int64_t ksb, kss, ksh;          // element strides of K, V, dK, dV
  float scale;                    // softmax scale (applied to dQ and dK at the end)
  float scale_log2;               // scale * log2(e): P = exp2(scale_log2 * (qk - L / scale) + mask * log2e)
  float inv_scale;                // 1 / scale (scale is finite and nonzero)
  int causal, offset, window;
  int drop;                       // dropout enabled (p > 0)
  uint32_t drop_thr;              // keep iff draw >= drop_thr
  float drop_inv;                 // 1 / (1 - p), rounded to fp32
  uint32_t seed_mix;              // fmix32(seed)
  const float* mask;
  int64_t msb, msh, msq, msk;
  uint32_t mask_rec;  // bytes of one (b, h) slice of the mask: ((Sq-1)*msq + (Sk-1)*msk + 1)*4 (bf16 path)
  int64_t ws_tiles;   // dS workspace tiles per (b, h) (workspace entry points only)
};

// MurmurHash3 32-bit finaliser (Appleby, public domain).
__host__ __device__ __forceinline__ uint32_t fmix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x85EBCA6Bu;
  x ^= x >> 13;
  x *= 0xC2B2AE35u;
  x ^= x >> 16;
  return x;
}

// fmix32's first step, x ^ (x >> 16), distributes over xor: fmix32(r ^ k) =
// fmix32_tail(xs16(r) ^ xs16(k)).  The tile kernels apply xs16 once per row key
// and once per key, and the rest per element.
__host__ __device__ __forceinline__ uint32_t xs16(uint32_t x) { return x ^ (x >> 16); }
__host__ __device__ __forceinline__ uint32_t fmix32_tail(uint32_t x) {
  x *= 0x85EBCA6Bu;
  x ^= x >> 13;
  x *= 0xC2B2AE35u;
  x ^= x >> 16;
  return x;
}

// Per-row part of the dropout draw: fmix32(((b*Hq + h)*Sq + i) + fmix32(seed)), mod 2^32.
__device__ __forceinline__ uint32_t drop_row_key(const PrefillArgs& a, int b, int h, int i) {
  uint32_t row = ((uint32_t)b * (uint32_t)a.Hq + (uint32_t)h) * (uint32_t)a.Sq + (uint32_t)i;
  return fmix32(row + a.seed_mix);
}

// Keep bit of element (row key rk, key j): fmix32(rk ^ j*0x9E3779B9) >= threshold.
__device__ __forceinline__ bool drop_keep(uint32_t rk, int j, uint32_t thr) {
  return fmix32(rk ^ ((uint32_t)j * 0x9E3779B9u)) >= thr;
}

// Cross-lane sums in registers, without LDS traffic: DPP moves within 16-lane
// rows, ds_swizzle across 16 lanes, v_permlane32_swap across 32.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float swizzle_xor16(float x) {  // lane ^ 16 within each 32-lane half
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x401F));
}
// v_permlane32_swap_b32 a, b exchanges a's lanes 32-63 with b's lanes 0-31;
// with a = b = x, a then holds x's lanes 0-31 twice and b its lanes 32-63
// twice, so a + b = x[lane] + x[lane ^ 32] in every lane.  Inline assembly:
// this compiler's builtin for it adds one of its two results to itself when
// both inputs are the same value.  Two wait states separate the VALU copies
// from the permute.
__device__ __forceinline__ float halves_sum(float x) {  // x[lane] + x[lane ^ 32]
  float a = x, b = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  return a + b;
}
__device__ __forceinline__ float halves_max(float x) {  // max(x[lane], x[lane ^ 32]), the same way
  float a = x, b = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  return fmaxf(a, b);
}
// Integer sum over the 64 lanes of a wave, in every lane.
__device__ __forceinline__ int wave_sum_i32(int x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  return x;
}

// Sum over each aligned group of N consecutive lanes (N = 1, 2, 4, ..., 64), in
// every lane of the group: quad_perm swaps lanes 1 and 2 apart, the half-row
// mirror pairs the two quads of an 8-lane half, the row mirror the two halves
// of a 16-lane row.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]
  if constexpr (N >= 4) x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]
  if constexpr (N >= 8) x += dpp_mov<0x141>(x);  // row_half_mirror
  if constexpr (N >= 16) x += dpp_mov<0x140>(x); // row_mirror
  if constexpr (N >= 32) x += swizzle_xor16(x);
  if constexpr (N >= 64) x = halves_sum(x);
  return x;
}
// Sum over the lanes congruent to this one modulo M (M = 1, 2, 4, ..., 64), in
// every such lane: row rotations by M, 2M, .., 8 within 16-lane rows, then
// across 16 and 32.
template <int M>
__device__ __forceinline__ float strided_sum(float x) {
  if constexpr (M <= 1) x += dpp_mov<0x121>(x);  // row_ror:1
  if constexpr (M <= 2) x += dpp_mov<0x122>(x);  // row_ror:2
  if constexpr (M <= 4) x += dpp_mov<0x124>(x);  // row_ror:4
  if constexpr (M <= 8) x += dpp_mov<0x128>(x);  // row_ror:8
  if constexpr (M <= 16) x += swizzle_xor16(x);
  if constexpr (M <= 32) x = halves_sum(x);
  return x;
}

// A head dimension below the tile width (64 or 128) is padded: a 16-byte
// chunk c of a row with only n real chunks is read from chunk c mod n instead
// (an address inside the row), and the operand it meets in the contraction
// over d is zero there (register-held rows are zeroed past D), so the padding
// adds exact zeros; outputs past D are not stored.
__host__ __device__ __forceinline__ int pad_chunk(int c, int n) { return c < n ? c : c % n; }

// Geometric visibility (ferrotensor-backend flash_attention_v2_backward.wgsl, fab2_visible).
__device__ __forceinline__ bool visible(const PrefillArgs& a, int i, int j) {
  if (i >= a.Sq || j >= a.Sk || i < 0 || j < 0) return false;
  const int qa = i + a.offset;
  if (a.causal && j > qa) return false;
  if (a.window > 0) {
    int d = j - qa;
    d = d < 0 ? -d : d;
    if (d >= a.window) return false;
  }
  return true;
}

// The same geometric rule as two uniform bounds on d = j - i: an in-range
// element is visible iff dlo < d < dhi (causal: d <= offset; window:
// |d - offset| < window).  Lets tile kernels test visibility branch-free.
struct DiagBounds {
  int dlo, dhi;
};

__device__ __forceinline__ DiagBounds diag_bounds(const PrefillArgs& a) {
  DiagBounds db{-(1 << 30) - 1, (1 << 30) + 1};
  if (a.causal) db.dhi = a.offset + 1;
  if (a.window > 0) {
    db.dlo = a.offset - a.window;
    if (!a.causal) db.dhi = a.offset + a.window;
  }
  return db;
}

// Declares AGPR use so the compiler selects the AGPR form of MFMA (accumulators
// and long-lived operands in the accumulation registers) instead of spilling
// VGPR-form accumulators into AGPRs.
__device__ __forceinline__ void use_agpr_form() { asm volatile("" ::: "a255"); }

__device__ __forceinline__ float mask_at(const PrefillArgs& a, int b, int h, int i, int j) {
  return a.mask[(int64_t)b * a.msb + (int64_t)h * a.msh + (int64_t)i * a.msq + (int64_t)j * a.msk];
}

// Is every element of the rectangle rows [i0, i1] x keys [j0, j1] geometrically visible?
__device__ __forceinline__ bool rect_all_visible(const PrefillArgs& a, int i0, int i1, int j0, int j1) {
  if (i1 >= a.Sq || j1 >= a.Sk) return false;
  if (a.causal && j1 > i0 + a.offset) return false;
  if (a.window > 0) {
    if ((i1 + a.offset) - j0 >= a.window) return false;
    if (j1 - (i0 + a.offset) >= a.window) return false;
  }
  return true;
}

// Is no element of the rectangle visible (so the tile can be skipped)?
__device__ __forceinline__ bool rect_none_visible(const PrefillArgs& a, int i0, int i1, int j0, int j1) {
  if (i0 >= a.Sq || j0 >= a.Sk) return true;
  if (a.causal && j0 > i1 + a.offset) return true;
  if (a.window > 0) {
    if (j0 - (i1 + a.offset) >= a.window) return true;   // every key right of every query's window
    if ((i0 + a.offset) - j1 >= a.window) return true;   // every key left of every query's window
  }
  return false;
}

// Keys [begin, end) that any query in [q0, q1] can see (tile-range version of the predicate).
__device__ __forceinline__ void key_range(const PrefillArgs& a, int q0, int q1, int& begin, int& end) {
  long e = a.Sk;
  long bg = 0;
  if (a.causal) e = min(e, (long)q1 + a.offset + 1);
  if (a.window > 0) {
    bg = max(0L, (long)q0 + a.offset - a.window + 1);
    if (!a.causal) e = min(e, (long)q1 + a.offset + a.window);
  }
  begin = (int)bg;
  end = (int)max(e, bg);
}

// Queries [begin, end) that can see any key in [k0, k1] (also used by the host
// to size the dS workspace, so written without device-only helpers).
__host__ __device__ __forceinline__ void query_range(const PrefillArgs& a, int k0, int k1, int& begin, int& end) {
  long bg = 0, e = a.Sq;
  if (a.causal) bg = (long)k0 - a.offset > 0 ? (long)k0 - a.offset : 0L;
  if (a.window > 0) {
    const long top = (long)k1 + a.window - a.offset;
    e = e < top ? e : (top > 0 ? top : 0L);
    if (!a.causal) {
      const long lo = (long)k0 - a.window - a.offset + 1;
      bg = bg > lo ? bg : lo;
    }
  }
  begin = (int)(bg < (long)a.Sq ? bg : (long)a.Sq);
  end = (int)(e > (long)begin ? e : (long)begin);
}

// The dS workspace (filled by the dK/dV pass in its workspace mode, read by
// the dQ pass over stored dS).  Its unit is a tile of 64 query rows x 128 keys
// (one key block of the dK/dV pass), 16 KB of bf16: [row half m][32-key group
// w][row group t (16 rows)][key k][row half h (8 rows)][8 rows], the rows of a
// half in the order the MFMA result registers hold them (within each 16 rows,
// quads 1 and 2 swapped); (w, t) is one 1 KB store of the dK/dV pass's wave w
// and keys 64j .. 64j+63 of a row half are 4 KB in one piece.  Per (b, h) the tiles follow
// key block by key block; key block kb stores query tiles qlo .. qlo+n-1, the
// 64-row tiles that meet the rows query_range gives for its keys.
constexpr int kWsRows = 64;
constexpr int kWsKeys = 128;
constexpr int kWsTileBytes = kWsRows * kWsKeys * 2;
__host__ __device__ __forceinline__ void ws_run(const PrefillArgs& a, int kb, int& qlo, int& n) {
  const int k0 = kb * kWsKeys;
  const int k1 = k0 + kWsKeys - 1 < a.Sk - 1 ? k0 + kWsKeys - 1 : a.Sk - 1;
  int qb, qe;
  query_range(a, k0, k1, qb, qe);
  qlo = qb / kWsRows;
  n = qe > qb ? (qe - 1) / kWsRows - qlo + 1 : 0;
}

// ----------------------------------------------------------------------------
// 32x32 MFMA operand chunks.  A "chunk" is the 16 bytes one lane supplies per
// k-block: 8 bf16 (one v_mfma_f32_32x32x16_bf16) or 4 fp32 (four
// v_mfma_f32_32x32x2_f32).  Lane l supplies row/column l%32 and the k-slice
// selected by its half h = l/32; A and B use the same (h, element) -> k map,
// so any consistent assignment of k indices to (h, element) is a valid
// contraction.  C layout: lane l holds column l%32 and rows
// 8*(r/4) + 4*h + (r%4) for r = 0..15.
// ----------------------------------------------------------------------------
template <typename T>
struct Mma;

template <>
struct Mma<__bf16> {
  static constexpr int CH = 8;  // elements per lane per chunk
  using chunk = bf16x8;
  static __device__ __forceinline__ void run(f32x16& c, const chunk& a, const chunk& b) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // Pack C registers [r0, r0+8) into a B-operand chunk (RNE to bf16).
  static __device__ __forceinline__ chunk from_acc(const f32x16& c, int r0) {
    chunk o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (__bf16)c[r0 + e];
    return o;
  }
};

template <>
struct Mma<float> {
  static constexpr int CH = 4;
  using chunk = f32x4;
  static __device__ __forceinline__ void run(f32x16& c, const chunk& a, const chunk& b) {
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[0], b[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[1], b[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[2], b[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[3], b[3], c, 0, 0, 0);
  }
  static __device__ __forceinline__ chunk from_acc(const f32x16& c, int r0) {
    chunk o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = c[r0 + e];
    return o;
  }
};

// 16-byte global / LDS loads and stores.
template <typename T>
__device__ __forceinline__ typename Mma<T>::chunk ld16(const T* p) {
  return *reinterpret_cast<const typename Mma<T>::chunk*>(p);
}

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }

template <typename T>
__device__ __forceinline__ T from_f32(float x) { return (T)x; }

}  // namespace fa
