// Query-block-outer pass, fp32 path (the bf16 path is fa_dq_bf16.hip): dQ without atomics (rustytorch
// flash_attention_backward_dq.metal kernel; ferrotensor-backend
// flash_attention_v2_backward.wgsl, flash_bwd_dq second sweep, with L given):
//   dQ_i = scale * sum_j dS_ij K_j,  dS_ij = P_ij (M_ij dO_i.V_j - Delta_i),
//   P_ij = exp(S_ij - L_i) on counted elements, 0 elsewhere.
//
// gfx950 design: a 256-thread block owns RG groups of 32 query rows of one
// (b, h) and streams BK-key tiles of K and V through LDS, row-major: the A
// operand of S^T = K Q^T and dP^T = V dO^T is read along the rows, that of
// dQ^T += K^T dS^T down the columns of K (one float per lane and k index; rows
// padded by 32 bytes, so the two half-waves, four rows apart, use disjoint
// banks).  At D = 64 the tile area is 74 KB and two blocks share a CU.  Its
// four waves split the block as RG row groups x KSL key
// slices (RG * KSL = 4, BK = 32 * KSL): each wave keeps its 32 rows of Q and dO
// in registers as MFMA B operands (v_mfma_f32_32x32x2_f32) and accumulates
// dQ^T (D x 32, fp32) over its 32-key slice of every tile; the KSL partial
// sums of a row group are added through LDS at the end.  Splitting the keys of
// a row block over waves shortens the longest chain of tiles a wave walks --
// under causal attention the last rows see every key -- by KSL and gives KSL x
// as many blocks, so small problems fill the chip.  S^T comes out of the MFMA
// with one query per lane column, so dS^T is already the B operand of the last
// contraction and L_i, Delta_i are per-lane scalars.
#include "fa_internal.h"

namespace fa {

template <int D>
struct DqF32Shape {
  static constexpr int RG = D <= 64 ? 1 : 2;  // 32-row groups per block
  static constexpr int KSL = 4 / RG;          // key slices per tile
  static constexpr int BK = 32 * KSL;         // keys per tile
  static constexpr int ROWS = 32 * RG;        // query rows per block
};

template <typename T, int D, bool MASK, bool DROP>
__global__ __launch_bounds__(256, D <= 64 ? 2 : 1) void dq_kernel(PrefillArgs a, const T* __restrict__ Q,
                                                    const T* __restrict__ K,
                                                    const T* __restrict__ V,
                                                    const T* __restrict__ dO,
                                                    const float* __restrict__ L,
                                                    const float* __restrict__ Dl,
                                                    T* __restrict__ dQ) {
  using M = Mma<T>;
  using chunk = typename M::chunk;
  using Sh = DqF32Shape<D>;
  constexpr int KSL = Sh::KSL, BK = Sh::BK;
  constexpr int CH = M::CH;
  constexpr int KS = D / (2 * CH);
  constexpr int PR = D + 32 / (int)sizeof(T);  // LDS pitch (elements): +32 B per row
  constexpr int TC = 16 / CH;
  constexpr int DB = D / 32;
  constexpr int NPART = DB * 16;  // partial-sum registers per lane (dQ^T)
  static_assert(Sh::RG * KSL == 4 && 2 * BK * PR * (int)sizeof(T) >= Sh::RG * (KSL - 1) * NPART * 64 * 4,
                "the tile area holds the partial sums of every wave but the first of each row group");

  // K, V of a tile (row-major); after the last tile, the waves' partial dQ^T.
  __shared__ __attribute__((aligned(16))) T sTile[2 * BK * PR];
  T* const sK = sTile;
  T* const sV = sTile + BK * PR;

  const int nbh = a.B * a.Hq;
  const int nqb = (a.Sq + Sh::ROWS - 1) / Sh::ROWS;
  // Query blocks: the last half descending (longest causal work first), then
  // the first half ascending, so blocks i and i + grid/2 -- the two a CU holds
  // when the whole grid is resident -- take query blocks nqb-1-q and q.
  const int ql = (int)(blockIdx.x / nbh), nqh = (nqb + 1) / 2;
  const int qbi = ql < nqh ? nqb - 1 - ql : ql - nqh;
  // Consecutive blocks cycle over KV heads first, so the query heads of one
  // KV head land on the same XCD (blocks are dealt round-robin over XCDs).
  const int bhi = blockIdx.x % nbh;
  const int kvh = bhi % a.Hkv;
  const int rest = bhi / a.Hkv;
  const int gi = rest % a.group;
  const int b = rest / a.group;
  const int h = kvh * a.group + gi;

  const int tid = threadIdx.x;
  const int wave = tid / 64;
  const int lane = tid % 64;
  const int h2 = lane / 32;
  const int l32 = lane % 32;
  const int rg = wave / KSL;  // this wave's row group
  const int ksl = wave % KSL; // and its key slice of every tile
  const int q0 = qbi * Sh::ROWS;
  const int qw0 = q0 + 32 * rg;
  const int il = qw0 + l32;  // this lane's query row (its C-layout column)

  chunk qr[KS], gr[KS];
  const int64_t qoff = (int64_t)b * a.qsb + (int64_t)il * a.qss + (int64_t)h * a.qsh;
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    if (il < a.Sq && 2 * CH * s + CH * h2 < a.D) {  // zero past the head dimension
      qr[s] = ld16<T>(Q + qoff + 2 * CH * s + CH * h2);
      gr[s] = ld16<T>(dO + qoff + 2 * CH * s + CH * h2);
    } else {
      qr[s] = chunk{};
      gr[s] = chunk{};
    }
  }
  const int64_t lrow = ((int64_t)b * a.Hq + h) * a.Sq + il;
  const float l2 = il < a.Sq ? L[lrow] * kLog2e : __builtin_inff();
  const float del = il < a.Sq ? Dl[lrow] : 0.f;
  // Keys this lane's row sees: d = j - i in (dlo, dhi), row and key in range,
  // i.e. keys [vlo, vlo + vspan); a boundary tile tests each element against
  // that interval with one unsigned compare (no branch).
  const DiagBounds vb = diag_bounds(a);
  const int vlo = max(il + vb.dlo + 1, 0);
  const uint32_t vspan = (uint32_t)max((il < a.Sq ? min(il + vb.dhi, a.Sk) : 0) - vlo, 0);
  uint32_t rk = 0;
  if constexpr (DROP) rk = drop_row_key(a, b, h, il);

  f32x16 accq[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d) accq[d] = f32x16{};

  int kb, ke;
  key_range(a, q0, min(q0 + Sh::ROWS, a.Sq) - 1, kb, ke);

  for (int kt = kb; kt < ke; kt += BK) {
    __syncthreads();
    for (int c = tid; c < BK * (D / CH); c += 256) {
      const int r = c / (D / CH);
      const int cc = c % (D / CH);
      const int j = kt + r;
      chunk kv{}, vv{};
      if (j < a.Sk && cc * CH < a.D) {
        const int64_t off = (int64_t)b * a.ksb + (int64_t)j * a.kss + (int64_t)kvh * a.ksh + cc * CH;
        kv = ld16<T>(K + off);
        vv = ld16<T>(V + off);
      }
      *reinterpret_cast<chunk*>(&sK[r * PR + cc * CH]) = kv;
      *reinterpret_cast<chunk*>(&sV[r * PR + cc * CH]) = vv;
    }
    __syncthreads();

    const int kw = kt + 32 * ksl;  // this wave's 32 keys of the tile
    if (rect_none_visible(a, qw0, qw0 + 31, kw, kw + 31)) continue;
    const bool full = !MASK && !DROP && rect_all_visible(a, qw0, qw0 + 31, kw, kw + 31);
    // Element r is key kw + 4*h2 + c(r), c(r) = 8*(r/4) + r%4: visible iff c(r) - lb < vspan.
    const int lb = vlo - (kw + 4 * h2);

    // S^T = K Q^T, dP^T = V dO^T (C column = query).
    f32x16 st{}, dpt{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int base = (32 * ksl + l32) * PR + 2 * CH * ks + CH * h2;
      M::run(st, *reinterpret_cast<const chunk*>(&sK[base]), qr[ks]);
      M::run(dpt, *reinterpret_cast<const chunk*>(&sV[base]), gr[ks]);
    }

#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = kw + 8 * (r / 4) + 4 * h2 + (r % 4);
      float p;
      if (full) {
        p = __builtin_amdgcn_exp2f(st[r] * a.scale_log2 - l2);
      } else {
        bool ok = (uint32_t)(8 * (r / 4) + (r % 4) - lb) < vspan;
        float madd = 0.f;
        if constexpr (MASK) {
          const float mv = ok ? mask_at(a, b, h, il, j) : 0.f;
          ok = ok && !(mv <= kMaskedSentinel);
          madd = mv * kLog2e;
        }
        p = __builtin_amdgcn_exp2f(ok ? st[r] * a.scale_log2 + madd - l2 : -__builtin_inff());
      }
      float dpv = dpt[r];
      if constexpr (DROP) dpv *= drop_keep(rk, j, a.drop_thr) ? a.drop_inv : 0.f;
      dpt[r] = p * (dpv - del);
    }

    // dQ^T += K^T dS^T (contraction over the wave's keys).
#pragma unroll
    for (int t = 0; t < TC; ++t) {
      const chunk dsc = M::from_acc(dpt, t * CH);
#pragma unroll
      for (int d = 0; d < DB; ++d) {
        // A element (lane l, k slot e of half h2) = column 32d + l%32 of key row
        // 32*ksl + 8t + 4*h2 + e: the keys C registers 4t .. 4t+3 of the lane hold.
        chunk ak;
#pragma unroll
        for (int sg = 0; sg < CH / 4; ++sg) {
          const int kk = 32 * ksl + 8 * ((CH / 4) * t + sg) + 4 * h2;
#pragma unroll
          for (int e = 0; e < 4; ++e) ak[4 * sg + e] = sK[(kk + e) * PR + 32 * d + l32];
        }
        M::run(accq[d], ak, dsc);
      }
    }
  }

  // Sum the key slices' partial dQ^T of each row group through LDS: register n
  // of lane l of the wave with key slice ksl > 0 at
  // sPart[(slot * NPART + n) * 64 + l], slot = rg * (KSL - 1) + ksl - 1.
  __syncthreads();  // every wave is done with the tiles
  float* const sPart = reinterpret_cast<float*>(sTile);
  if (ksl != 0) {
    const int slot = rg * (KSL - 1) + ksl - 1;
#pragma unroll
    for (int d = 0; d < DB; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) sPart[(slot * NPART + 16 * d + r) * 64 + lane] = accq[d][r];
  }
  __syncthreads();
  if (ksl != 0) return;
#pragma unroll
  for (int o = 1; o < KSL; ++o) {
    const int slot = rg * (KSL - 1) + o - 1;
#pragma unroll
    for (int d = 0; d < DB; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) accq[d][r] += sPart[(slot * NPART + 16 * d + r) * 64 + lane];
  }

  if (il < a.Sq) {
#pragma unroll
    for (int d = 0; d < DB; ++d) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int dd = 32 * d + 8 * r4 + 4 * h2;
        if (dd >= a.D) continue;  // past the head dimension
#pragma unroll
        for (int e = 0; e < 4; ++e) dQ[qoff + dd + e] = from_f32<T>(accq[d][4 * r4 + e] * a.scale);
      }
    }
  }
}

template <typename T, int D, bool MASK, bool DROP>
static hipError_t launch_t(const PrefillArgs& a, const void* Q, const void* K, const void* V,
                           const void* dO, const float* L, const float* delta, void* dQ,
                           hipStream_t st) {
  const int nqb = (a.Sq + DqF32Shape<D>::ROWS - 1) / DqF32Shape<D>::ROWS;
  const unsigned grid = (unsigned)((int64_t)nqb * a.B * a.Hq);
  hipLaunchKernelGGL((dq_kernel<T, D, MASK, DROP>), dim3(grid), dim3(256), 0, st, a,
                     static_cast<const T*>(Q), static_cast<const T*>(K), static_cast<const T*>(V),
                     static_cast<const T*>(dO), L, delta, static_cast<T*>(dQ));
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_d(const PrefillArgs& a, const void* Q, const void* K, const void* V,
                           const void* dO, const float* L, const float* delta, void* dQ,
                           hipStream_t st) {
  const bool mask = a.mask != nullptr;
  const bool drop = a.drop != 0;
  if (mask && drop) return launch_t<T, D, true, true>(a, Q, K, V, dO, L, delta, dQ, st);
  if (mask) return launch_t<T, D, true, false>(a, Q, K, V, dO, L, delta, dQ, st);
  if (drop) return launch_t<T, D, false, true>(a, Q, K, V, dO, L, delta, dQ, st);
  return launch_t<T, D, false, false>(a, Q, K, V, dO, L, delta, dQ, st);
}

hipError_t launch_dq(const PrefillArgs& a, int dtype, int D, const void* Q, const void* K,
                     const void* V, const void* dO, const float* L, const float* delta, void* dQ,
                     hipStream_t st) {
  if (dtype == kBF16) return launch_dq_bf16(a, D, Q, K, V, dO, L, delta, dQ, st);
  return D <= 64 ? launch_d<float, 64>(a, Q, K, V, dO, L, delta, dQ, st)
                 : launch_d<float, 128>(a, Q, K, V, dO, L, delta, dQ, st);
}

}  // namespace fa
