// Forward pass producing O and L with the backward's conventions, fp32 path
// (the bf16 path is fa_fwd_bf16.hip; ferrotensor-backend
// flash_attention_v2_backward.wgsl: the forward whose O and L the backward
// takes -- its file is referenced there, not shown -- and the online
// log-sum-exp of its dQ pass's first sweep; rustytorch
// flash_attention_backward_dq.metal takes L as an input):
//   S_ij = scale * Q_i.K_j + mask_ij on visible, unmasked elements,
//   L_i = log sum_j exp(S_ij)  (natural log; +inf when no element counts),
//   O_i = sum_j exp(S_ij - L_i) M_ij V_j   (M the dropout multiplier).
//
// gfx950 design, as the fp32 dQ pass: a 256-thread block owns RG groups of 32
// query rows of one (b, h) and streams BK-key tiles of K and V through LDS
// (row-major, rows padded by 32 bytes); its four waves split the block as RG
// row groups x KSL key slices (RG * KSL = 4, BK = 32 * KSL), so a short causal
// problem still gives every CU blocks.  Each wave keeps its 32 rows of Q in
// registers as the B operand of S^T = K Q^T (v_mfma_f32_32x32x2_f32): every
// lane column is one query row, its running maximum and sum per-lane values
// (the two half-waves, which hold different keys of the same rows, agree on
// the maximum through v_permlane32_swap and add their sums at the end).  O^T
// += V^T (P.M)^T takes V^T by reading columns of the row-major V tile (one
// float per lane and k index) and (P.M)^T straight from the C registers of
// S^T.  A row's reference maximum moves only when passed by more than 2^8
// (the terms stay below 2^8; O, the sum and L share the reference).  At the
// end the KSL waves of a row group merge their (maximum, sum, O) through
// LDS: each wave rescales the partial O and sums of the group to the largest
// maximum and writes a share of the rows' outputs.  With WO false the kernel
// computes L alone (no V, no O): the log-sum-exp sweep for a caller whose
// forward did not keep L.
#include "fa_internal.h"

namespace fa {

template <int D>
struct FwdF32Shape {
  static constexpr int RG = D <= 64 ? 1 : 2;  // 32-row groups per block
  static constexpr int KSL = 4 / RG;          // key slices per tile
  static constexpr int BK = 32 * KSL;         // keys per tile
  static constexpr int ROWS = 32 * RG;        // query rows per block
};

constexpr float kF32LazyLog2 = 8.f;  // lag of a row's reference maximum before O is rescaled (log2 units)

template <int D, bool MASK, bool DROP, bool WO>
__global__ __launch_bounds__(256, 2) void fwd_f32_kernel(PrefillArgs a, const float* __restrict__ Q,
                                                         const float* __restrict__ K,
                                                         const float* __restrict__ V, float* __restrict__ O,
                                                         float* __restrict__ Lout) {
  using M = Mma<float>;
  using chunk = M::chunk;
  using Sh = FwdF32Shape<D>;
  constexpr int KSL = Sh::KSL, BK = Sh::BK;
  constexpr int CH = M::CH;           // 4 floats per lane per k-block
  constexpr int KS = D / (2 * CH);    // k-blocks of the head_dim contraction
  constexpr int PR = D + 8;           // LDS pitch (floats): +32 B per row
  constexpr int TC = 16 / CH;         // B-operand chunks per C block
  constexpr int DB = D / 32;          // 32-row blocks of O^T
  constexpr int NPART = DB * 16;      // partial-O registers per lane
  constexpr int NTILE = (WO ? 2 : 1) * BK * PR;
  constexpr int NSUM = WO ? 4 * NPART * 64 : 1;
  static_assert(Sh::RG * KSL == 4 && NPART % (4 * KSL) == 0, "block shape");

  // K (and V) rows of a tile; after the last tile, the waves' partial O^T.
  __shared__ __attribute__((aligned(16))) float sT[NTILE > NSUM ? NTILE : NSUM];
  __shared__ float sMax[4][64], sSum[4][64];
  float* const sK = sT;
  float* const sV = sT + BK * PR;

  // Query blocks: the last half descending (longest causal work first), then
  // the first half ascending, so blocks i and i + grid/2 (the two a CU holds
  // when the whole grid is resident) carry complementary causal work; the KV
  // head varies fastest, so the query heads of one KV head share an XCD.
  const int nbh = a.B * a.Hq;
  const int nqb = (a.Sq + Sh::ROWS - 1) / Sh::ROWS;
  const int ql = (int)(blockIdx.x / nbh), nqh = (nqb + 1) / 2;
  const int qbi = ql < nqh ? nqb - 1 - ql : ql - nqh;
  const int bhi = blockIdx.x % nbh;
  const int kvh = bhi % a.Hkv;
  const int rest = bhi / a.Hkv;
  const int h = kvh * a.group + rest % a.group;
  const int b = rest / a.group;

  const int tid = threadIdx.x;
  const int wave = tid / 64;
  const int lane = tid % 64;
  const int h2 = lane / 32;
  const int l32 = lane % 32;
  const int rg = wave / KSL;   // this wave's row group
  const int ksl = wave % KSL;  // and its key slice of every tile
  const int q0 = qbi * Sh::ROWS;
  const int qw0 = q0 + 32 * rg;
  const int i = qw0 + l32;  // this lane's query row (its C-layout column)

  chunk qr[KS];
  const int64_t qoff = (int64_t)b * a.qsb + (int64_t)i * a.qss + (int64_t)h * a.qsh;
#pragma unroll
  for (int s = 0; s < KS; ++s)  // zero past the head dimension
    qr[s] = i < a.Sq && 2 * CH * s + CH * h2 < a.D ? ld16<float>(Q + qoff + 2 * CH * s + CH * h2) : chunk{};
  const uint32_t rkey = (DROP && WO) ? drop_row_key(a, b, h, i) : 0u;

  f32x16 acc[WO ? DB : 1];
#pragma unroll
  for (int d = 0; d < (WO ? DB : 1); ++d) acc[d] = f32x16{};
  float m = -__builtin_inff();  // reference maximum of the exponent (log2 units), shared by both half-waves
  float l = 0.f;                // this lane's part of the running sum

  const DiagBounds vb = diag_bounds(a);
  // Row i sees the keys [jlo, jlo + span): j - i in (dlo, dhi), j < Sk (none
  // past the last row); key j is visible iff j - jlo < span (unsigned).
  const int jlo = max(i + vb.dlo + 1, 0);
  const uint32_t span = (uint32_t)max((i < a.Sq ? min(i + vb.dhi, a.Sk) : 0) - jlo, 0);

  int kb, ke;
  key_range(a, q0, min(q0 + Sh::ROWS, a.Sq) - 1, kb, ke);
  for (int kt = kb; kt < ke; kt += BK) {
    __syncthreads();  // every wave is done with the previous tile
    for (int c = tid; c < BK * (D / CH); c += 256) {
      const int r = c / (D / CH);
      const int cc = c % (D / CH);
      const int j = kt + r;
      chunk kv{}, vv{};
      if (j < a.Sk && cc * CH < a.D) {
        const int64_t off = (int64_t)b * a.ksb + (int64_t)j * a.kss + (int64_t)kvh * a.ksh + cc * CH;
        kv = ld16<float>(K + off);
        if constexpr (WO) vv = ld16<float>(V + off);
      }
      *reinterpret_cast<chunk*>(&sK[r * PR + cc * CH]) = kv;
      if constexpr (WO) *reinterpret_cast<chunk*>(&sV[r * PR + cc * CH]) = vv;
    }
    __syncthreads();
    const int kw = kt + 32 * ksl;  // this wave's 32 keys of the tile
    if (rect_none_visible(a, qw0, qw0 + 31, kw, kw + 31)) continue;

    // S^T = K Q^T (C column = query row, C row = key).
    f32x16 st{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      M::run(st, *reinterpret_cast<const chunk*>(&sK[(32 * ksl + l32) * PR + 2 * CH * ks + CH * h2]), qr[ks]);

    // Element r: key j = kw + 4*h2 + c(r), c(r) = 8*(r/4) + r%4, of row i.
    const int lb = jlo - (kw + 4 * h2);
    float tmax = -__builtin_inff();
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = kw + 8 * (r >> 2) + 4 * h2 + (r & 3);
      bool ok = (uint32_t)(8 * (r >> 2) + (r & 3) - lb) < span;
      float v = st[r] * a.scale_log2;
      if constexpr (MASK) {
        const float mv = ok ? mask_at(a, b, h, i, j) : 0.f;
        ok = ok && !(mv <= kMaskedSentinel);
        v = __builtin_fmaf(mv, kLog2e, v);
      }
      st[r] = ok ? v : -__builtin_inff();
      tmax = fmaxf(tmax, st[r]);
    }
    const float mt = halves_max(tmax);
    const bool grow = mt > m + kF32LazyLog2;  // m = -inf: any counted element
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float alpha = grow ? __builtin_amdgcn_exp2f(m - mt) : 1.f;
      m = grow ? mt : m;
      l *= alpha;
      if constexpr (WO) {
#pragma unroll
        for (int d = 0; d < DB; ++d)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[d][r] *= alpha;
      }
    }
    const float mref = m == -__builtin_inff() ? 0.f : m;  // nothing counted yet: every term is 0
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float p = __builtin_amdgcn_exp2f(st[r] - mref);
      l += p;
      if constexpr (DROP && WO) {
        const int j = kw + 8 * (r >> 2) + 4 * h2 + (r & 3);
        p = drop_keep(rkey, j, a.drop_thr) ? p * a.drop_inv : 0.f;
      }
      st[r] = p;  // P.M in the C layout of S^T: the B operand of O^T += V^T (P.M)^T
    }
    if constexpr (WO) {
#pragma unroll
      for (int t = 0; t < TC; ++t) {
        const chunk pc = M::from_acc(st, t * CH);
#pragma unroll
        for (int d = 0; d < DB; ++d) {
          // A element (lane l, k slot e of half h2) = column 32d + l%32 of key row
          // 32*ksl + 8t + 4*h2 + e: the keys C registers 4t .. 4t+3 of the lane hold.
          chunk av;
#pragma unroll
          for (int e = 0; e < CH; ++e) av[e] = sV[(32 * ksl + 8 * t + 4 * h2 + e) * PR + 32 * d + l32];
          M::run(acc[d], av, pc);
        }
      }
    }
  }

  // Merge the KSL key slices of each row group: every wave puts its maximum,
  // sum and partial O^T (register n of lane l at sPart[(wave * NPART + n) * 64
  // + l]) in LDS; then wave ksl of the group rescales the group's partials to
  // the largest maximum and writes registers ksl * NPW .. (ksl+1) * NPW - 1
  // (four consecutive head-dimension columns of the lane's row at a time).
  const float lsum = halves_sum(l);
  __syncthreads();  // every wave is done with the tiles
  float* const sPart = sT;
  sMax[wave][lane] = m;
  sSum[wave][lane] = lsum;
  if constexpr (WO) {
#pragma unroll
    for (int d = 0; d < DB; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) sPart[(wave * NPART + 16 * d + r) * 64 + lane] = acc[d][r];
  }
  __syncthreads();
  float mx = -__builtin_inff();
#pragma unroll
  for (int o = 0; o < KSL; ++o) mx = fmaxf(mx, sMax[rg * KSL + o][lane]);
  const float mxr = mx == -__builtin_inff() ? 0.f : mx;
  float f[KSL], tot = 0.f;
#pragma unroll
  for (int o = 0; o < KSL; ++o) {
    f[o] = __builtin_amdgcn_exp2f(sMax[rg * KSL + o][lane] - mxr);  // 0 for a slice that counted nothing
    tot += sSum[rg * KSL + o][lane] * f[o];
  }
  if (i < a.Sq) {
    if constexpr (WO) {
      const float inv = tot > 0.f ? 1.f / tot : 0.f;
      constexpr int NPW = NPART / KSL;
#pragma unroll
      for (int q4 = 0; q4 < NPW / 4; ++q4) {
        const int n0 = ksl * NPW + 4 * q4;  // registers n0 .. n0+3: block n0/16, rows 8*((n0%16)/4) + 4*h2 + 0..3
        const int dd = 32 * (n0 / 16) + 8 * ((n0 % 16) / 4) + 4 * h2;
        if (dd >= a.D) continue;  // past the head dimension
        f32x4 o4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int o = 0; o < KSL; ++o)
#pragma unroll
          for (int e = 0; e < 4; ++e) o4[e] += sPart[((rg * KSL + o) * NPART + n0 + e) * 64 + lane] * f[o];
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] *= inv;
        *reinterpret_cast<f32x4*>(O + qoff + dd) = o4;
      }
    }
    if (ksl == 0 && h2 == 0)
      Lout[((int64_t)b * a.Hq + h) * a.Sq + i] =
          tot > 0.f ? (mx + __builtin_log2f(tot)) * 0.6931471805599453f : __builtin_inff();
  }
}

template <int D, bool MASK, bool DROP, bool WO>
static hipError_t launch_t(const PrefillArgs& a, const void* Q, const void* K, const void* V, void* O, float* L,
                           hipStream_t st) {
  const int nqb = (a.Sq + FwdF32Shape<D>::ROWS - 1) / FwdF32Shape<D>::ROWS;
  const unsigned grid = (unsigned)((int64_t)nqb * a.B * a.Hq);
  hipLaunchKernelGGL((fwd_f32_kernel<D, MASK, DROP, WO>), dim3(grid), dim3(256), 0, st, a,
                     static_cast<const float*>(Q), static_cast<const float*>(K), static_cast<const float*>(V),
                     static_cast<float*>(O), L);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_d(const PrefillArgs& a, const void* Q, const void* K, const void* V, void* O, float* L,
                           hipStream_t st) {
  const bool mk = a.mask != nullptr, dr = a.drop != 0;
  if (O == nullptr)  // L alone: dropout does not enter it
    return mk ? launch_t<D, true, false, false>(a, Q, K, V, O, L, st) : launch_t<D, false, false, false>(a, Q, K, V, O, L, st);
  if (mk)
    return dr ? launch_t<D, true, true, true>(a, Q, K, V, O, L, st) : launch_t<D, true, false, true>(a, Q, K, V, O, L, st);
  return dr ? launch_t<D, false, true, true>(a, Q, K, V, O, L, st) : launch_t<D, false, false, true>(a, Q, K, V, O, L, st);
}

// O == nullptr: L alone (V is not read).
hipError_t launch_fwd(const PrefillArgs& a, int dtype, int D, const void* Q, const void* K, const void* V, void* O,
                      float* L, hipStream_t st) {
  if (dtype == kBF16) return launch_fwd_bf16(a, D, Q, K, V, O, L, st);
  return D <= 64 ? launch_d<64>(a, Q, K, V, O, L, st) : launch_d<128>(a, Q, K, V, O, L, st);
}

}  // namespace fa
