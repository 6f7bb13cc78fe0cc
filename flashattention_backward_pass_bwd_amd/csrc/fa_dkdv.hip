// Key-block-outer pass, fp32 path (the bf16 path is fa_dkdv_bf16.hip): dK and dV without atomics (ferrotensor-backend
// flash_attention_v2_backward.wgsl, flash_bwd_dk_dv; formulas from its header
// comment).  For each key j of KV head kvh, summed over the query heads of the
// GQA group and over every query i that sees it:
//   dV_j = sum_i P_ij M_ij dO_i,     dK_j = scale * sum_i dS_ij Q_i,
//   P_ij = exp(S_ij - L_i) on counted elements (0 elsewhere),
//   dS_ij = P_ij (M_ij dO_i.V_j - Delta_i).
//
// gfx950 design: a 256-thread block owns KG groups of 32 keys of one (b, kvh)
// and streams RT-row tiles of Q and dO through LDS, stored row-major once: the
// A operand of S = Q K^T and dP = dO V^T is read along the rows (16 bytes per
// lane), that of dV^T += dO^T (P.M) and dK^T += Q^T dS down the columns (one
// float per lane and k index, a half-wave reading 32 consecutive floats of a
// row).  Rows are padded by 32 bytes, so the two half-waves of a column read,
// four rows apart, fall into disjoint halves of the 64 banks.  At D = 64 the
// tile area is 74 KB and two blocks share a CU, one computing while the other
// loads its next tile (at D = 128, and with both a mask and dropout, the
// registers allow one block per CU).  Its four waves split the block as KG key groups x RS
// row slices (KG * RS = 4, RT = 32 * RS): each wave keeps its 32 keys' K and V
// rows in registers as MFMA B operands (v_mfma_f32_32x32x2_f32) and
// accumulates dK^T, dV^T (D x 32, fp32) over its 32-row slice of every tile;
// the RS partial sums of a key group are added through LDS at the end.
// Splitting the rows of a key block over waves (instead of giving each wave
// keys of its own) shortens the longest chain of tiles a wave walks -- under
// causal attention the first keys see every row -- by RS and gives RS x as
// many blocks, so small problems fill the chip.  S and dP come out of the MFMA
// in the C layout whose per-lane column is a key, which is exactly the
// B-operand layout the second pair of contractions needs, so P and dS never
// leave registers.
#include "fa_internal.h"

namespace fa {

template <int D>
struct DkdvF32Shape {
  static constexpr int KG = D <= 64 ? 1 : 2;  // 32-key groups per block
  static constexpr int RS = 4 / KG;           // row slices per tile
  static constexpr int RT = 32 * RS;          // rows per tile
  static constexpr int KEYS = 32 * KG;        // keys per block
};

template <typename T, int D, bool MASK, bool DROP>
__global__ __launch_bounds__(256, D <= 64 && !(MASK && DROP) ? 2 : 1) void dkdv_kernel(PrefillArgs a, const T* __restrict__ Q,
                                                      const T* __restrict__ K,
                                                      const T* __restrict__ V,
                                                      const T* __restrict__ dO,
                                                      const float* __restrict__ L,
                                                      const float* __restrict__ Dl,
                                                      T* __restrict__ dK, T* __restrict__ dV) {
  using M = Mma<T>;
  using chunk = typename M::chunk;
  using Sh = DkdvF32Shape<D>;
  constexpr int RS = Sh::RS, RT = Sh::RT;
  constexpr int CH = M::CH;
  constexpr int KS = D / (2 * CH);             // k-blocks of the head_dim contraction
  constexpr int PR = D + 32 / (int)sizeof(T);  // LDS pitch (elements): +32 B per row
  constexpr int TC = 16 / CH;                  // B-operand chunks per 32-row C block
  constexpr int DB = D / 32;                   // 32-row blocks of dK^T / dV^T
  constexpr int NPART = 2 * DB * 16;           // partial-sum registers per lane (dK^T and dV^T)
  constexpr int NTILE = 2 * RT * PR;                                // elements of a Q, dO tile
  constexpr int NSUM = 4 * NPART * 64 * 4 / (int)sizeof(T);         // the four waves' partial sums
  static_assert(Sh::KG * RS == 4 && NPART % (4 * RS) == 0, "block shape");

  // Q, dO of a tile (row-major); after the last tile, the waves' partial dK^T, dV^T.
  __shared__ __attribute__((aligned(16))) T sTile[NTILE > NSUM ? NTILE : NSUM];
  T* const sQ = sTile;
  T* const sdO = sTile + RT * PR;
  __shared__ float sL[RT];
  __shared__ float sDel[RT];
  __shared__ uint32_t sRK[DROP ? RT : 1];

  const int nbh = a.B * a.Hkv;
  // Key blocks: the first half ascending (longest causal work first), then the
  // second half descending, so blocks i and i + grid/2 -- the two a CU holds
  // when the whole grid is resident -- take key blocks kb and nkb-1-kb, whose
  // causal work adds up to the same for every pair.
  const int nkb = (a.Sk + Sh::KEYS - 1) / Sh::KEYS;
  const int kl = blockIdx.x / nbh, nkh = (nkb + 1) / 2;
  const int kb = kl < nkh ? kl : nkb - 1 - (kl - nkh);
  const int bh = blockIdx.x % nbh;  // consecutive blocks cycle over (b, kvh) -> one XCD per KV head
  const int b = bh / a.Hkv;
  const int kvh = bh % a.Hkv;
  const int tid = threadIdx.x;
  const int wave = tid / 64;
  const int lane = tid % 64;
  const int h2 = lane / 32;
  const int l32 = lane % 32;
  const int kg = wave / RS;  // this wave's key group
  const int rs = wave % RS;  // and its row slice of every tile
  const int k0 = kb * Sh::KEYS;
  const int kw0 = k0 + 32 * kg;
  const int jl = kw0 + l32;  // this lane's key (its C-layout column)
  // Rows that see this lane's key: d = j - i in (dlo, dhi), row and key in
  // range, i.e. rows [vlo, vlo + vspan); a boundary tile tests each element
  // against that interval with one unsigned compare (no branch).
  const DiagBounds vb = diag_bounds(a);
  const int vlo = max(jl - vb.dhi + 1, 0);
  const uint32_t vspan = (uint32_t)max((jl < a.Sk ? min(jl - vb.dlo, a.Sq) : 0) - vlo, 0);

  chunk kr[KS], vr[KS];
  const int64_t koff = (int64_t)b * a.ksb + (int64_t)jl * a.kss + (int64_t)kvh * a.ksh;
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    if (jl < a.Sk && 2 * CH * s + CH * h2 < a.D) {  // zero past the head dimension
      kr[s] = ld16<T>(K + koff + 2 * CH * s + CH * h2);
      vr[s] = ld16<T>(V + koff + 2 * CH * s + CH * h2);
    } else {
      kr[s] = chunk{};
      vr[s] = chunk{};
    }
  }

  f32x16 acck[DB], accv[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d) {
    acck[d] = f32x16{};
    accv[d] = f32x16{};
  }

  int qb, qe;
  query_range(a, k0, min(k0 + Sh::KEYS, a.Sk) - 1, qb, qe);

  for (int g = 0; g < a.group; ++g) {
    const int h = kvh * a.group + g;
    const int64_t lrow = ((int64_t)b * a.Hq + h) * a.Sq;
    for (int qt = qb; qt < qe; qt += RT) {
      __syncthreads();  // the previous tile has been consumed
#pragma unroll 4
      for (int c = tid; c < RT * (D / CH); c += 256) {
        const int r = c / (D / CH);
        const int cc = c % (D / CH);
        const int i = qt + r;
        chunk qv{}, gv{};
        if (i < a.Sq && cc * CH < a.D) {
          const int64_t off = (int64_t)b * a.qsb + (int64_t)i * a.qss + (int64_t)h * a.qsh + cc * CH;
          qv = ld16<T>(Q + off);
          gv = ld16<T>(dO + off);
        }
        *reinterpret_cast<chunk*>(&sQ[r * PR + cc * CH]) = qv;
        *reinterpret_cast<chunk*>(&sdO[r * PR + cc * CH]) = gv;
      }
      for (int r = tid; r < RT; r += 256) {
        const int i = qt + r;
        const bool in = i < a.Sq;
        sL[r] = in ? L[lrow + i] * kLog2e : __builtin_inff();
        sDel[r] = in ? Dl[lrow + i] : 0.f;
        if constexpr (DROP) sRK[r] = drop_row_key(a, b, h, i);
      }
      __syncthreads();

      const int qw = qt + 32 * rs;  // this wave's 32 rows of the tile
      if (rect_none_visible(a, qw, qw + 31, kw0, kw0 + 31)) continue;
      const bool full = !MASK && !DROP && rect_all_visible(a, qw, qw + 31, kw0, kw0 + 31);

      // S = Q K^T and dP = dO V^T for this wave's rows and keys (C column = key).
      f32x16 s{}, dp{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int base = (32 * rs + l32) * PR + 2 * CH * ks + CH * h2;
        M::run(s, *reinterpret_cast<const chunk*>(&sQ[base]), kr[ks]);
        M::run(dp, *reinterpret_cast<const chunk*>(&sdO[base]), vr[ks]);
      }

      // Elementwise: P, dropout, dS.  s <- P*M, dp <- dS.  Element r sits at row
      // qt + 32*rs + 4*h2 + c(r), c(r) = 8*(r/4) + r%4, visible iff c(r) - lb < vspan.
      const int lb = vlo - (qt + 32 * rs + 4 * h2);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = 32 * rs + 8 * (r / 4) + 4 * h2 + (r % 4);
        const float l2 = sL[row];
        float p;
        if (full) {
          p = __builtin_amdgcn_exp2f(s[r] * a.scale_log2 - l2);
        } else {
          bool ok = (uint32_t)(8 * (r / 4) + (r % 4) - lb) < vspan;
          float madd = 0.f;
          if constexpr (MASK) {
            const float mv = ok ? mask_at(a, b, h, qt + row, jl) : 0.f;
            ok = ok && !(mv <= kMaskedSentinel);
            madd = mv * kLog2e;
          }
          p = __builtin_amdgcn_exp2f(ok ? s[r] * a.scale_log2 + madd - l2 : -__builtin_inff());
        }
        float dpv = dp[r];
        float pm = p;
        if constexpr (DROP) {
          const float mm = drop_keep(sRK[row], jl, a.drop_thr) ? a.drop_inv : 0.f;
          dpv *= mm;
          pm = p * mm;
        }
        dp[r] = p * (dpv - sDel[row]);
        s[r] = pm;
      }

      // dV^T += dO^T (P.M),  dK^T += Q^T dS  (contraction over the wave's rows).
#pragma unroll
      for (int t = 0; t < TC; ++t) {
        const chunk pmc = M::from_acc(s, t * CH);
        const chunk dsc = M::from_acc(dp, t * CH);
#pragma unroll
        for (int d = 0; d < DB; ++d) {
          // A element (lane l, k slot e of half h2) = column 32d + l%32 of row
          // 32*rs + 8t + 4*h2 + e: the rows C registers 4t .. 4t+3 of the lane hold.
          chunk ao, aq;
#pragma unroll
          for (int sg = 0; sg < CH / 4; ++sg) {
            const int q = 32 * rs + 8 * ((CH / 4) * t + sg) + 4 * h2;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              ao[4 * sg + e] = sdO[(q + e) * PR + 32 * d + l32];
              aq[4 * sg + e] = sQ[(q + e) * PR + 32 * d + l32];
            }
          }
          M::run(accv[d], ao, pmc);
          M::run(acck[d], aq, dsc);
        }
      }
    }
  }

  // Sum the row slices' partial dK^T, dV^T of each key group through LDS and
  // store them: every wave puts its register n (n = 32d + r: dK^T block d, n =
  // 32d + 16 + r: dV^T block d) of lane l at sPart[(wave * NPART + n) * 64 + l];
  // then the wave with row slice rs sums registers rs * NPW .. (rs+1) * NPW - 1
  // over the key group's RS waves and writes them, four registers (four
  // consecutive columns of the lane's key) at a time.
  __syncthreads();  // every wave is done with the tiles
  float* const sPart = reinterpret_cast<float*>(sTile);
#pragma unroll
  for (int d = 0; d < DB; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      sPart[(wave * NPART + 32 * d + r) * 64 + lane] = acck[d][r];
      sPart[(wave * NPART + 32 * d + 16 + r) * 64 + lane] = accv[d][r];
    }
  __syncthreads();
  if (jl >= a.Sk) return;
  constexpr int NPW = NPART / RS;
#pragma unroll
  for (int q4 = 0; q4 < NPW / 4; ++q4) {
    const int n0 = rs * NPW + 4 * q4;
    const int dd = 32 * (n0 / 32) + 8 * ((n0 % 16) / 4) + 4 * h2;
    if (dd >= a.D) continue;  // past the head dimension
    const bool is_v = (n0 / 16) & 1;
    float x[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int o = 0; o < RS; ++o)
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] += sPart[((kg * RS + o) * NPART + n0 + e) * 64 + lane];
    T* const out = is_v ? dV : dK;
    const float f = is_v ? 1.f : a.scale;
#pragma unroll
    for (int e = 0; e < 4; ++e) out[koff + dd + e] = from_f32<T>(x[e] * f);
  }
}

template <typename T, int D, bool MASK, bool DROP>
static hipError_t launch_t(const PrefillArgs& a, const void* Q, const void* K, const void* V,
                           const void* dO, const float* L, const float* delta, void* dK, void* dV,
                           hipStream_t st) {
  const int nkb = (a.Sk + DkdvF32Shape<D>::KEYS - 1) / DkdvF32Shape<D>::KEYS;
  const unsigned grid = (unsigned)((int64_t)nkb * a.B * a.Hkv);
  hipLaunchKernelGGL((dkdv_kernel<T, D, MASK, DROP>), dim3(grid), dim3(256), 0, st, a,
                     static_cast<const T*>(Q), static_cast<const T*>(K), static_cast<const T*>(V),
                     static_cast<const T*>(dO), L, delta, static_cast<T*>(dK), static_cast<T*>(dV));
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_d(const PrefillArgs& a, const void* Q, const void* K, const void* V,
                           const void* dO, const float* L, const float* delta, void* dK, void* dV,
                           hipStream_t st) {
  const bool mask = a.mask != nullptr;
  const bool drop = a.drop != 0;
  if (mask && drop) return launch_t<T, D, true, true>(a, Q, K, V, dO, L, delta, dK, dV, st);
  if (mask) return launch_t<T, D, true, false>(a, Q, K, V, dO, L, delta, dK, dV, st);
  if (drop) return launch_t<T, D, false, true>(a, Q, K, V, dO, L, delta, dK, dV, st);
  return launch_t<T, D, false, false>(a, Q, K, V, dO, L, delta, dK, dV, st);
}

hipError_t launch_dkdv(const PrefillArgs& a, int dtype, int D, const void* Q, const void* K,
                       const void* V, const void* dO, const float* L, const float* delta, void* dK,
                       void* dV, hipStream_t st) {
  if (dtype == kBF16) return launch_dkdv_bf16(a, D, Q, K, V, dO, L, delta, dK, dV, st);
  return D <= 64 ? launch_d<float, 64>(a, Q, K, V, dO, L, delta, dK, dV, st)
                 : launch_d<float, 128>(a, Q, K, V, dO, L, delta, dK, dV, st);
}

}  // namespace fa
