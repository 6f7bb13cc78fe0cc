// Key-block-outer dK/dV pass, bf16 storage, bf16 MFMA with fp32 accumulation
// (ferrotensor-backend flash_attention_v2_backward.wgsl, flash_bwd_dk_dv and
// its header formulas):
//   dV_j = sum_h sum_i P_ij M_ij dO_i,  dK_j = scale * sum_h sum_i dS_ij Q_i,
//   P_ij = exp(S_ij - L_i) on counted elements, dS_ij = P_ij (M_ij dO_i.V_j - Delta_i).
//
// Block: 4 waves own 128 consecutive keys of one (b, kvh); wave w owns keys
// k0 + 32w .. +31 and keeps their K and V rows in registers as MFMA B operands
// (v_mfma_f32_32x32x16_bf16), accumulating dK^T and dV^T (D x 32 fp32) in
// accumulation registers.  The block walks every (query head of the group,
// 64-row query tile) pair.  Q and dO tiles live in a 3-stage LDS ring
// (swizzled, see fa_tiles.h) filled by direct global->LDS copies issued two
// tiles ahead, so their latency hides behind two tiles of MFMA work and the
// copies need no registers; L and Delta (64 floats each per tile) take the
// register path.  One fence-free barrier per tile.  S = Q K^T and dP = dO V^T read row-major
// operands; the transposed operands of dV^T += dO^T (P.M) and dK^T += Q^T dS
// come from the same tiles through ds_read_b64_tr_b16.  P and dS never leave
// registers: the C layout of S (one key per lane column) is the B layout of
// the second pair of contractions.  A tile is processed as two 32-row halves
// so that the exp/dS arithmetic of one half can overlap the MFMAs of the
// other.  For causal attention without a window, block i also takes key block
// nkb-1-i, so every block carries the same amount of work.
#include <type_traits>

#include "fa_internal.h"
#include "fa_tiles.h"

namespace fa {

template <int D, bool MASK, bool DROP>
__global__ __launch_bounds__(256, 1) void dkdv_bf16_kernel(PrefillArgs a, const __bf16* __restrict__ Q,
                                                           const __bf16* __restrict__ K,
                                                           const __bf16* __restrict__ V,
                                                           const __bf16* __restrict__ dO,
                                                           const float* __restrict__ L,
                                                           const float* __restrict__ Dl,
                                                           __bf16* __restrict__ dK, __bf16* __restrict__ dV,
                                                           int nkb, int paired) {
  using M = Mma<__bf16>;
  constexpr int BQ = 64;
  constexpr int NCH = D / 8;                // 16-byte chunks per row
  constexpr int KS = D / 16;                // k-blocks of the head_dim contraction
  constexpr int DB = D / 32;                // 32-row blocks of dK^T / dV^T
  constexpr int NST = 3;                    // LDS ring stages
  constexpr int RPI = 1024 / (2 * D);       // tile rows per 1 KB global->LDS copy (64 lanes x 16 B)
  constexpr int NIW = BQ / RPI / 4;         // copies per wave per tile per tensor
  constexpr int TILE = BQ * D;

  __shared__ __attribute__((aligned(16))) __bf16 sQ[NST][TILE];
  __shared__ __attribute__((aligned(16))) __bf16 sdO[NST][TILE];
  __shared__ __attribute__((aligned(16))) float sL[NST][BQ];
  __shared__ __attribute__((aligned(16))) float sDel[NST][BQ];
  __shared__ uint32_t sRK[NST][DROP ? BQ : 1];

  const int nbh = a.B * a.Hkv;
  const int wi = blockIdx.x / nbh;
  const int bh = blockIdx.x % nbh;  // consecutive blocks cycle over (b, kvh): one XCD per KV head
  const int b = bh / a.Hkv;
  const int kvh = bh % a.Hkv;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int h2 = lane >> 5;
  const int l32 = lane & 31;
  use_agpr_form();
  const DiagBounds vb = diag_bounds(a);

  // Copy u of this wave fills rows (wave*NIW + u)*RPI + lane/NCH; lane l lands in
  // physical chunk l%NCH, so it fetches the logical chunk stored there.
  const int cp_row = lane / NCH;
  const int cp_pc = lane % NCH;
  // Per-lane LDS offsets of the row-major operand chunks and the transposed reads.
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
    const int kb = pass == 0 ? wi : nkb - 1 - wi;
    if (pass == 1 && kb <= wi) break;
    const int k0 = kb * kDkdvKeysPerBlock;
    const int kw0 = k0 + wave * kDkdvKeysPerWave;
    const int jl = kw0 + l32;

    bf16x8 kr[KS], vr[KS];
    const int64_t koff = (int64_t)b * a.ksb + (int64_t)jl * a.kss + (int64_t)kvh * a.ksh;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      kr[s] = bf16x8{};
      vr[s] = bf16x8{};
      if (jl < a.Sk) {
        kr[s] = *reinterpret_cast<const bf16x8*>(K + koff + 16 * s + 8 * h2);
        vr[s] = *reinterpret_cast<const bf16x8*>(V + koff + 16 * s + 8 * h2);
      }
    }
    f32x16 acck[DB], accv[DB];
#pragma unroll
    for (int d = 0; d < DB; ++d) {
      acck[d] = f32x16{};
      accv[d] = f32x16{};
    }
    wait_all_vmem();  // K and V rows are in registers before the copy ring starts

    int qb, qe;
    query_range(a, k0, min(k0 + kDkdvKeysPerBlock, a.Sk) - 1, qb, qe);
    const int ntq = (qe - qb + BQ - 1) / BQ;
    const int ntiles = ntq * a.group;

    // Tiles are numbered it = g*ntq + t (query head g of the group, query tile t).
    // A scalar cursor (cg, ct) names the tile whose copies are issued next; past
    // the last tile it stays there, so the last copies repeat into a stage that
    // is no longer read and every step runs the same straight-line code.
    int cg = 0, ct = 0;
    auto advance = [&]() {
      const int tn = ct + 1;
      const bool wrap = tn == ntq;
      const int gn = cg + (wrap ? 1 : 0);
      const bool end = gn == a.group;
      ct = end ? ct : (wrap ? 0 : tn);
      cg = end ? cg : gn;
    };
    // Copies of the cursor's tile into a stage.  L (natural log) and Delta
    // (64 floats each) go first, by waves 0 and 1; then the Q and dO rows:
    // copy u of this wave fills rows (wave*NIW + u)*RPI + lane/NCH.  Rows past
    // the end repeat the last row; they are never counted.  Per-lane offsets
    // are 32-bit, relative to the tile's first row (the host bounds the row
    // stride).  Because L and Delta are issued before the 2*NIW row copies,
    // waiting until at most 2*NIW copies are in flight covers them.
    auto issue_tile = [&](int stage) {
      const int h = kvh * a.group + cg;
      const int qt = qb + ct * BQ;
      const int lim = a.Sq - 1 - qt;
      if (wave < 2) {
        const float* src = (wave == 0 ? L : Dl) + (((int64_t)b * a.Hq + h) * a.Sq + qt);
        dma4(src, 4u * (uint32_t)min(lane, lim), lds_addr(wave == 0 ? sL[stage] : sDel[stage]));
      }
      const int64_t base = (int64_t)b * a.qsb + (int64_t)h * a.qsh + (int64_t)qt * a.qss;
      const __bf16* tq = Q + base;
      const __bf16* tg = dO + base;
#pragma unroll
      for (int u = 0; u < NIW; ++u) {
        const int blk = wave * NIW + u;
        const int r = blk * RPI + cp_row;
        const uint32_t off = 2u * ((uint32_t)min(r, lim) * (uint32_t)a.qss + 8u * (uint32_t)(cp_pc ^ swz<D>(r)));
        dma16(tq, off, lds_addr(&sQ[stage][blk * RPI * D]));
        dma16(tg, off, lds_addr(&sdO[stage][blk * RPI * D]));
      }
    };
    // Dropout row keys of the cursor's tile (lanes 0-15 of each wave, 16 rows per wave).
    auto store_rk = [&](int stage) {
      if constexpr (DROP) {
        if (lane < 16) {
          const int h = kvh * a.group + cg;
          sRK[stage][16 * wave + lane] = drop_row_key(a, b, h, qb + ct * BQ + 16 * wave + lane);
        }
      }
    };
    // Wave 0 turns a landed tile's L into L*log2(e) in place (one value per lane).
    auto scale_l = [&](int stage) {
      if (wave == 0) sL[stage][lane] *= kLog2e;
    };

    if (ntiles > 0) {
      issue_tile(0);
      store_rk(0);
      advance();
      issue_tile(1);
      store_rk(1);
      advance();
      wait_vmcnt<2 * NIW>();  // tile 0 and the L/Delta of tile 1 landed
      scale_l(0);             // the first step scales tile 1's
      barrier_lds();
    }

    // One step: issue the copies of tile it+2 (the cursor) while computing tile
    // it = (g, t) from stage st.  KIND 0 = no element of the tile is visible to
    // this wave, 1 = boundary tile (per-element predicate), 2 = interior tile
    // (every element counted).  Each kind runs in a loop of its own, so no loop
    // body branches.
    int st = 0;
    auto step = [&](auto kind_c, int g, int t) {
      constexpr int KIND = decltype(kind_c)::value;
      const int stage = st;
      const int stage1 = st == NST - 1 ? 0 : st + 1;  // (st + 1) % NST
      const int stage2 = st == 0 ? 2 : st - 1;        // (st + 2) % NST
      issue_tile(stage2);
      // L of tile it+1 landed with the wait at the end of the previous step.
      scale_l(stage1);
      if constexpr (KIND != 0) {
      const int qt = qb + t * BQ;
      const int h = kvh * a.group + g;
      const __bf16* tq = sQ[stage];
      const __bf16* tg = sdO[stage];
      const float* tl = sL[stage];
      const float* td = sDel[stage];
      // S (m-th 32-row half) = Q K^T and dP = dO V^T.
      auto mma_sdp = [&](int m, f32x16& s, f32x16& dp) {
        s = f32x16{};
        dp = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          M::run(s, lds_read_b128(tq + rd_off[ks] + 32 * m * D), kr[ks]);
          M::run(dp, lds_read_b128(tg + rd_off[ks] + 32 * m * D), vr[ks]);
        }
      };
      // P, dropout and dS for one half, packed into the bf16 B operands of the next contractions.
      auto elementwise = [&](auto full_c, int m, const f32x16& s, const f32x16& dp, bf16x8 (&pmc)[2],
                             bf16x8 (&dsc)[2]) {
        constexpr bool FULL = decltype(full_c)::value;
        const int dl0 = jl - qt;  // d = j - i = dl0 - row
        const int rlim = a.Sq - qt;
        const bool jin = jl < a.Sk;
        const int jc = min(jl, a.Sk - 1);
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int row0 = 32 * m + 8 * r4 + 4 * h2;
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(tl + row0);
          const f32x4 d4 = *reinterpret_cast<const f32x4*>(td + row0);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * r4 + e;
            float x = __builtin_fmaf(s[r], a.scale_log2, -l4[e]);
            if constexpr (!FULL) {
              const int row = row0 + e;
              const int dd = dl0 - row;
              bool ok = jin && row < rlim && dd > vb.dlo && dd < vb.dhi;
              if constexpr (MASK) {
                // clamped indices keep the load in bounds; ok discards out-of-range elements
                const float mv = mask_at(a, b, h, min(qt + row, a.Sq - 1), jc);
                ok = ok && !(mv <= kMaskedSentinel);
                x = __builtin_fmaf(mv, kLog2e, x);
              }
              x = ok ? x : -__builtin_inff();
            }
            const float p = __builtin_amdgcn_exp2f(x);
            float dpv = dp[r];
            float pm = p;
            if constexpr (DROP) {
              const float mm = drop_keep(sRK[stage][row0 + e], jl, a.drop_thr) ? a.drop_inv : 0.f;
              dpv *= mm;
              pm = p * mm;
            }
            pmc[r >> 3][r & 7] = (__bf16)pm;
            dsc[r >> 3][r & 7] = (__bf16)(p * (dpv - d4[e]));
          }
        }
      };
      // dV^T += dO^T (P.M) and dK^T += Q^T dS over the m-th half's 32 queries.
      auto mma_dkdv = [&](int m, const bf16x8 (&pmc)[2], const bf16x8 (&dsc)[2]) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int rb = (32 * m + 16 * t) * D;
#pragma unroll
          for (int d = 0; d < DB; ++d) {
            const bf16x8 ao = concat(lds_read_tr(tg + tr_lo[d] + rb), lds_read_tr(tg + tr_hi[d] + rb));
            M::run(accv[d], ao, pmc[t]);
            const bf16x8 aq = concat(lds_read_tr(tq + tr_lo[d] + rb), lds_read_tr(tq + tr_hi[d] + rb));
            M::run(acck[d], aq, dsc[t]);
          }
        }
      };
      auto tile = [&](auto full_c) {
        f32x16 s0, dp0, s1, dp1;
        bf16x8 pm0[2], ds0[2], pm1[2], ds1[2];
        mma_sdp(0, s0, dp0);
        mma_sdp(1, s1, dp1);
        elementwise(full_c, 0, s0, dp0, pm0, ds0);
        mma_dkdv(0, pm0, ds0);
        elementwise(full_c, 1, s1, dp1, pm1, ds1);
        mma_dkdv(1, pm1, ds1);
      };

      tile(std::integral_constant<bool, KIND == 2>{});
      }
      __builtin_amdgcn_sched_barrier(0);
      store_rk(stage2);
      advance();
      st = stage1;
      wait_vmcnt<2 * NIW>();  // tile it+1 and the L/Delta of tile it+2 landed; its rows may still be in flight
      barrier_lds();
    };

    const std::integral_constant<int, 0> kSkip;
    const std::integral_constant<int, 1> kEdge;
    const std::integral_constant<int, 2> kInner;
    for (int g = 0; g < a.group; ++g) {
      // This wave's tiles of head g, in order: [0,v0) invisible, [v0,f0) boundary,
      // [f0,f1) interior, [f1,v1) boundary, [v1,ntq) invisible (the visible key
      // interval moves monotonically with the query row, so the classes are contiguous).
      auto none = [&](int t) { return rect_none_visible(a, qb + t * BQ, qb + t * BQ + BQ - 1, kw0, kw0 + kDkdvKeysPerWave - 1); };
      auto all = [&](int t) { return rect_all_visible(a, qb + t * BQ, qb + t * BQ + BQ - 1, kw0, kw0 + kDkdvKeysPerWave - 1); };
      int v0 = 0;
      while (v0 < ntq && none(v0)) ++v0;
      int v1 = v0;
      while (v1 < ntq && !none(v1)) ++v1;
      int f0 = v1, f1 = v1;
      if constexpr (!MASK && !DROP) {
        f0 = v0;
        while (f0 < v1 && !all(f0)) ++f0;
        f1 = f0;
        while (f1 < v1 && all(f1)) ++f1;
      }
      int t = 0;
      for (; t < v0; ++t) step(kSkip, g, t);
      for (; t < f0; ++t) step(kEdge, g, t);
      for (; t < f1; ++t) step(kInner, g, t);
      for (; t < v1; ++t) step(kEdge, g, t);
      for (; t < ntq; ++t) step(kSkip, g, t);
    }
    wait_vmcnt<0>();  // the repeated copies of the last steps have landed

    if (jl < a.Sk) {
#pragma unroll
      for (int d = 0; d < DB; ++d) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int dd = 32 * d + 8 * r4 + 4 * h2;
          bf16x4 ok4, ov4;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            ok4[e] = (__bf16)(acck[d][4 * r4 + e] * a.scale);
            ov4[e] = (__bf16)accv[d][4 * r4 + e];
          }
          *reinterpret_cast<bf16x4*>(dK + koff + dd) = ok4;
          *reinterpret_cast<bf16x4*>(dV + koff + dd) = ov4;
        }
      }
    }
  }
}

template <int D, bool MASK, bool DROP>
static hipError_t launch_t(const PrefillArgs& a, const void* Q, const void* K, const void* V, const void* dO,
                           const float* L, const float* delta, void* dK, void* dV, hipStream_t st) {
  const int nkb = (a.Sk + kDkdvKeysPerBlock - 1) / kDkdvKeysPerBlock;
  const int paired = (a.causal && a.window == 0 && nkb > 1) ? 1 : 0;
  const int nwi = paired ? (nkb + 1) / 2 : nkb;
  const unsigned grid = (unsigned)(nwi * a.B * a.Hkv);
  hipLaunchKernelGGL((dkdv_bf16_kernel<D, MASK, DROP>), dim3(grid), dim3(256), 0, st, a,
                     static_cast<const __bf16*>(Q), static_cast<const __bf16*>(K), static_cast<const __bf16*>(V),
                     static_cast<const __bf16*>(dO), L, delta, static_cast<__bf16*>(dK), static_cast<__bf16*>(dV),
                     nkb, paired);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_d(const PrefillArgs& a, const void* Q, const void* K, const void* V, const void* dO,
                           const float* L, const float* delta, void* dK, void* dV, hipStream_t st) {
  const bool mask = a.mask != nullptr;
  const bool drop = a.drop != 0;
  if (mask && drop) return launch_t<D, true, true>(a, Q, K, V, dO, L, delta, dK, dV, st);
  if (mask) return launch_t<D, true, false>(a, Q, K, V, dO, L, delta, dK, dV, st);
  if (drop) return launch_t<D, false, true>(a, Q, K, V, dO, L, delta, dK, dV, st);
  return launch_t<D, false, false>(a, Q, K, V, dO, L, delta, dK, dV, st);
}

hipError_t launch_dkdv_bf16(const PrefillArgs& a, int D, const void* Q, const void* K, const void* V,
                            const void* dO, const float* L, const float* delta, void* dK, void* dV,
                            hipStream_t st) {
  return D == 64 ? launch_d<64>(a, Q, K, V, dO, L, delta, dK, dV, st)
                 : launch_d<128>(a, Q, K, V, dO, L, delta, dK, dV, st);
}

}  // namespace fa
