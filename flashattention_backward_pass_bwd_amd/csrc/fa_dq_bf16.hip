// Query-block-outer dQ pass, bf16 storage, bf16 MFMA with fp32 accumulation
// (rustytorch flash_attention_backward_dq.metal kernel; ferrotensor-backend
// flash_attention_v2_backward.wgsl, flash_bwd_dq second sweep, L supplied):
//   dQ_i = scale * sum_j dS_ij K_j,  dS_ij = P_ij (M_ij dO_i.V_j - Delta_i).
//
// Block: 4 waves own 128 consecutive query rows of one (b, h); wave w keeps
// its 32 rows of Q and dO in registers as MFMA B operands and accumulates
// dQ^T (D x 32 fp32).  K and V tiles of 64 keys live in a 3-stage LDS ring
// (swizzled, see fa_tiles.h) filled by direct global->LDS copies issued two
// tiles ahead; one fence-free barrier per tile.  S^T = K Q^T and dP^T = V dO^T read row-major
// operands; dQ^T += K^T dS^T reads K transposed through ds_read_b64_tr_b16.
// S^T has one query per lane column, so L_i and Delta_i are per-lane scalars
// (without dropout the dP^T chain starts from -Delta_i, so dP - Delta comes
// out of the MFMAs) and dS^T is already the B operand of the last contraction.  Blocks of the
// query heads sharing a KV head are dealt to one XCD; for causal attention
// without a window, block i also takes query block nqb-1-i.
#include <type_traits>

#include "fa_internal.h"
#include "fa_tiles.h"

namespace fa {

template <int D, bool MASK, bool DROP>
__global__ __launch_bounds__(256, 1) void dq_bf16_kernel(PrefillArgs a, const __bf16* __restrict__ Q,
                                                         const __bf16* __restrict__ K,
                                                         const __bf16* __restrict__ V,
                                                         const __bf16* __restrict__ dO,
                                                         const float* __restrict__ L,
                                                         const float* __restrict__ Dl,
                                                         __bf16* __restrict__ dQ, int nqb, int paired) {
  using M = Mma<__bf16>;
  constexpr int BK = 64;
  constexpr int NCH = D / 8;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int NST = 3;                    // LDS ring stages
  constexpr int RPI = 1024 / (2 * D);       // tile rows per 1 KB global->LDS copy
  constexpr int NIW = BK / RPI / 4;         // copies per wave per tile per tensor
  constexpr int TILE = BK * D;

  __shared__ __attribute__((aligned(16))) __bf16 sK[NST][TILE];
  __shared__ __attribute__((aligned(16))) __bf16 sV[NST][TILE];

  const int nbh = a.B * a.Hq;
  const int wi = blockIdx.x / nbh;
  const int bhi = blockIdx.x % nbh;
  const int kvh = bhi % a.Hkv;  // KV head varies fastest: its query heads share an XCD
  const int rest = bhi / a.Hkv;
  const int gi = rest % a.group;
  const int b = rest / a.group;
  const int h = kvh * a.group + gi;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int h2 = lane >> 5;
  const int l32 = lane & 31;
  const DiagBounds vb = diag_bounds(a);

  // Copy u of this wave fills rows (wave*NIW + u)*RPI + lane/NCH; lane l lands in
  // physical chunk l%NCH, so it fetches the logical chunk stored there.
  const int cp_row = lane / NCH;
  const int cp_pc = lane % NCH;
  int rd_off[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) rd_off[ks] = tile_off<D>(l32, 2 * ks + h2);
  int tr_lo[DB], tr_hi[DB];  // first and second 8-row halves of a transposed operand
#pragma unroll
  for (int d = 0; d < DB; ++d) {
    tr_lo[d] = tr_lane_off<D>(lane, d, 0);
    tr_hi[d] = tr_lane_off<D>(lane, d, 8);
  }

  const int npass = paired ? 2 : 1;
  for (int pass = 0; pass < npass; ++pass) {
    // Without pairing, later blocks take earlier query blocks (longest causal work first).
    const int qbi = paired ? (pass == 0 ? wi : nqb - 1 - wi) : nqb - 1 - wi;
    if (pass == 1 && qbi <= wi) break;
    const int q0 = qbi * kDqRowsPerBlock;
    const int qw0 = q0 + wave * kDqRowsPerWave;
    const int il = qw0 + l32;

    bf16x8 qr[KS], gr[KS];
    const int64_t qoff = (int64_t)b * a.qsb + (int64_t)il * a.qss + (int64_t)h * a.qsh;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      qr[s] = bf16x8{};
      gr[s] = bf16x8{};
      if (il < a.Sq) {
        qr[s] = *reinterpret_cast<const bf16x8*>(Q + qoff + 16 * s + 8 * h2);
        gr[s] = *reinterpret_cast<const bf16x8*>(dO + qoff + 16 * s + 8 * h2);
      }
    }
    const int64_t lrow = ((int64_t)b * a.Hq + h) * a.Sq + il;
    const float l2 = il < a.Sq ? L[lrow] * kLog2e : __builtin_inff();
    const float del = il < a.Sq ? Dl[lrow] : 0.f;
    uint32_t rk = 0;
    if constexpr (DROP) rk = drop_row_key(a, b, h, il);
    wait_all_vmem();  // Q, dO rows, L and Delta are in registers before the copy ring starts

    // Without dropout dP - Delta comes straight out of the MFMA chain: it starts from -Delta.
    f32x16 dp_init;
#pragma unroll
    for (int r = 0; r < 16; ++r) dp_init[r] = DROP ? 0.f : -del;
    f32x16 accq[DB];
#pragma unroll
    for (int d = 0; d < DB; ++d) accq[d] = f32x16{};

    int kb, ke;
    key_range(a, q0, min(q0 + kDqRowsPerBlock, a.Sq) - 1, kb, ke);
    const int ntiles = (ke - kb + BK - 1) / BK;

    // Copy u of this wave fills key rows (wave*NIW + u)*RPI + lane/NCH of a tile.
    // Rows past the end repeat the last key; they are never counted.  Per-lane
    // offsets are 32-bit, relative to the tile's first key (the host bounds the
    // row stride).
    auto issue_tile = [&](int it, int stage) {
      const int kt = kb + it * BK;
      const int lim = a.Sk - 1 - kt;
      const int64_t base = (int64_t)b * a.ksb + (int64_t)kt * a.kss + (int64_t)kvh * a.ksh;
#pragma unroll
      for (int u = 0; u < NIW; ++u) {
        const int blk = wave * NIW + u;
        const int r = blk * RPI + cp_row;
        const uint32_t off = 2u * ((uint32_t)min(r, lim) * (uint32_t)a.kss + 8u * (uint32_t)(cp_pc ^ swz<D>(r)));
        dma16(K + base, off, lds_addr(&sK[stage][blk * RPI * D]));
        dma16(V + base, off, lds_addr(&sV[stage][blk * RPI * D]));
      }
    };

    if (ntiles > 0) issue_tile(0, 0);
    if (ntiles > 1) {
      issue_tile(1, 1);
      wait_vmcnt<2 * NIW>();  // tile 0 landed; tile 1 may still be in flight
    } else {
      wait_vmcnt<0>();
    }
    barrier_lds();

    // One step: start the copies of tile it+2 while computing tile it.  KIND 0
    // = no element visible to this wave, 1 = boundary tile (per-element
    // predicate), 2 = interior tile; each kind runs in a loop of its own.
    auto step = [&](auto kind_c, int it) {
      constexpr int KIND = decltype(kind_c)::value;
      const int stage = it % NST;
      const bool has2 = it + 2 < ntiles;
      if (has2) issue_tile(it + 2, (it + 2) % NST);
      if constexpr (KIND != 0) {
        const int kt = kb + it * BK;
        const __bf16* tk = sK[stage];
        const __bf16* tv = sV[stage];
        // S^T (m-th 32-key half) = K Q^T and dP^T = V dO^T.
        auto mma_sdp = [&](int m, f32x16& s, f32x16& dp) {
          s = f32x16{};
          dp = dp_init;
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            M::run(s, lds_read_b128(tk + rd_off[ks] + 32 * m * D), qr[ks]);
            M::run(dp, lds_read_b128(tv + rd_off[ks] + 32 * m * D), gr[ks]);
          }
        };
        // P, dropout and dS for one half, packed into the bf16 B operands of dQ^T += K^T dS^T.
        auto elementwise = [&](int m, const f32x16& s, const f32x16& dp, bf16x8 (&dsc)[2]) {
          const int dl0 = kt - il;  // d = j - i = dl0 + row
          const int rlim = a.Sk - kt;
          const bool iin = il < a.Sq;
          const int ic = min(il, a.Sq - 1);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float x = __builtin_fmaf(s[r], a.scale_log2, -l2);
            float dpv = dp[r];
            if constexpr (KIND == 1) {
              const int row = 32 * m + 8 * (r / 4) + 4 * h2 + (r % 4);
              const int dd = dl0 + row;
              bool ok = iin && row < rlim && dd > vb.dlo && dd < vb.dhi;
              if constexpr (MASK) {
                // clamped indices keep the load in bounds; ok discards out-of-range elements
                const float mv = mask_at(a, b, h, ic, min(kt + row, a.Sk - 1));
                ok = ok && !(mv <= kMaskedSentinel);
                x = __builtin_fmaf(mv, kLog2e, x);
              }
              x = ok ? x : -__builtin_inff();
              if constexpr (DROP) dpv *= drop_keep(rk, kt + row, a.drop_thr) ? a.drop_inv : 0.f;
            }
            const float p = __builtin_amdgcn_exp2f(x);
            if constexpr (DROP) dsc[r >> 3][r & 7] = (__bf16)(p * (dpv - del));
            else dsc[r >> 3][r & 7] = (__bf16)(p * dpv);
          }
        };
        auto mma_dq = [&](int m, const bf16x8 (&dsc)[2]) {
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const int rb = (32 * m + 16 * t) * D;
#pragma unroll
            for (int d = 0; d < DB; ++d) {
              const bf16x8 ak = concat(lds_read_tr(tk + tr_lo[d] + rb), lds_read_tr(tk + tr_hi[d] + rb));
              M::run(accq[d], ak, dsc[t]);
            }
          }
        };
        f32x16 s0, dp0, s1, dp1;
        bf16x8 ds0[2], ds1[2];
        mma_sdp(0, s0, dp0);
        mma_sdp(1, s1, dp1);
        elementwise(0, s0, dp0, ds0);
        mma_dq(0, ds0);
        elementwise(1, s1, dp1, ds1);
        mma_dq(1, ds1);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (has2)
        wait_vmcnt<2 * NIW>();  // tile it+1 landed; tile it+2 may still be in flight
      else
        wait_vmcnt<0>();
      barrier_lds();
    };

    // This wave's key tiles in order: [0,v0) invisible, [v0,f0) boundary, [f0,f1)
    // interior, [f1,v1) boundary, [v1,ntiles) invisible.
    auto none = [&](int t) { return rect_none_visible(a, qw0, qw0 + kDqRowsPerWave - 1, kb + t * BK, kb + t * BK + BK - 1); };
    auto all = [&](int t) { return rect_all_visible(a, qw0, qw0 + kDqRowsPerWave - 1, kb + t * BK, kb + t * BK + BK - 1); };
    int v0 = 0;
    while (v0 < ntiles && none(v0)) ++v0;
    int v1 = v0;
    while (v1 < ntiles && !none(v1)) ++v1;
    int f0 = v1, f1 = v1;
    if constexpr (!MASK && !DROP) {
      f0 = v0;
      while (f0 < v1 && !all(f0)) ++f0;
      f1 = f0;
      while (f1 < v1 && all(f1)) ++f1;
    }
    const std::integral_constant<int, 0> kSkip;
    const std::integral_constant<int, 1> kEdge;
    const std::integral_constant<int, 2> kInner;
    int t = 0;
    for (; t < v0; ++t) step(kSkip, t);
    for (; t < f0; ++t) step(kEdge, t);
    for (; t < f1; ++t) step(kInner, t);
    for (; t < v1; ++t) step(kEdge, t);
    for (; t < ntiles; ++t) step(kSkip, t);

    if (il < a.Sq) {
#pragma unroll
      for (int d = 0; d < DB; ++d) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int dd = 32 * d + 8 * r4 + 4 * h2;
          bf16x4 o4;
#pragma unroll
          for (int e = 0; e < 4; ++e) o4[e] = (__bf16)(accq[d][4 * r4 + e] * a.scale);
          *reinterpret_cast<bf16x4*>(dQ + qoff + dd) = o4;
        }
      }
    }
  }
}

template <int D, bool MASK, bool DROP>
static hipError_t launch_t(const PrefillArgs& a, const void* Q, const void* K, const void* V, const void* dO,
                           const float* L, const float* delta, void* dQ, hipStream_t st) {
  const int nqb = (a.Sq + kDqRowsPerBlock - 1) / kDqRowsPerBlock;
  const int paired = (a.causal && a.window == 0 && nqb > 1) ? 1 : 0;
  const int nwi = paired ? (nqb + 1) / 2 : nqb;
  const unsigned grid = (unsigned)(nwi * a.B * a.Hq);
  hipLaunchKernelGGL((dq_bf16_kernel<D, MASK, DROP>), dim3(grid), dim3(256), 0, st, a,
                     static_cast<const __bf16*>(Q), static_cast<const __bf16*>(K), static_cast<const __bf16*>(V),
                     static_cast<const __bf16*>(dO), L, delta, static_cast<__bf16*>(dQ), nqb, paired);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_d(const PrefillArgs& a, const void* Q, const void* K, const void* V, const void* dO,
                           const float* L, const float* delta, void* dQ, hipStream_t st) {
  const bool mask = a.mask != nullptr;
  const bool drop = a.drop != 0;
  if (mask && drop) return launch_t<D, true, true>(a, Q, K, V, dO, L, delta, dQ, st);
  if (mask) return launch_t<D, true, false>(a, Q, K, V, dO, L, delta, dQ, st);
  if (drop) return launch_t<D, false, true>(a, Q, K, V, dO, L, delta, dQ, st);
  return launch_t<D, false, false>(a, Q, K, V, dO, L, delta, dQ, st);
}

hipError_t launch_dq_bf16(const PrefillArgs& a, int D, const void* Q, const void* K, const void* V,
                          const void* dO, const float* L, const float* delta, void* dQ, hipStream_t st) {
  return D == 64 ? launch_d<64>(a, Q, K, V, dO, L, delta, dQ, st) : launch_d<128>(a, Q, K, V, dO, L, delta, dQ, st);
}

}  // namespace fa
