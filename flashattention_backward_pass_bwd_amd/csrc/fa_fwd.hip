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
// gfx950 design, as the fp32 dQ pass: a 256-thread block owns 128 query rows
// of one (b, h); each wave keeps its 32 rows of Q in registers as the B
// operand of S^T = K Q^T (v_mfma_f32_32x32x2_f32), so every lane column is one
// query row and the row's running maximum and sum are per-lane values (the two
// half-waves hold different keys of the same rows: they agree on the maximum
// through v_permlane32_swap and add their sums at the end).  The block streams
// 64-key tiles through LDS: K row-major (A operand of S^T), V transposed (A
// operand of O^T += V^T (P.M)^T, whose B operand comes straight from the C
// registers of S^T).  With WO false the kernel computes L alone (no V, no O):
// the log-sum-exp sweep for a caller whose forward did not keep L.
#include "fa_internal.h"

namespace fa {

template <int D, bool MASK, bool DROP, bool WO>
__global__ __launch_bounds__(256, 1) void fwd_f32_kernel(PrefillArgs a, const float* __restrict__ Q,
                                                         const float* __restrict__ K,
                                                         const float* __restrict__ V, float* __restrict__ O,
                                                         float* __restrict__ Lout) {
  using M = Mma<float>;
  using chunk = M::chunk;
  constexpr int CH = M::CH;           // 4 floats per lane per k-block
  constexpr int KS = D / (2 * CH);    // k-blocks of the head_dim contraction
  constexpr int BK = 64;              // keys per tile
  constexpr int PR = D + 4;           // padded row of the row-major K tile
  constexpr int PT = BK + 4;          // padded row of the transposed V tile
  constexpr int MB = BK / 32;         // 32-key halves of a tile
  constexpr int TC = 16 / CH;         // B-operand chunks per C block
  constexpr int DB = D / 32;          // 32-row blocks of O^T

  __shared__ __attribute__((aligned(16))) float sK[BK * PR];
  __shared__ __attribute__((aligned(16))) float sVT[WO ? D * PT : 1];

  const int nbh = a.B * a.Hq;
  const int nqb = (a.Sq + kDqRowsPerBlock - 1) / kDqRowsPerBlock;
  const int qbi = nqb - 1 - (int)(blockIdx.x / nbh);  // last query block first: longest causal work
  const int bhi = blockIdx.x % nbh;
  const int h = bhi % a.Hq;
  const int b = bhi / a.Hq;
  const int kvh = h / a.group;

  const int tid = threadIdx.x;
  const int wave = tid / 64;
  const int lane = tid % 64;
  const int h2 = lane / 32;
  const int l32 = lane % 32;
  const int q0 = qbi * kDqRowsPerBlock;
  const int qw0 = q0 + wave * kDqRowsPerWave;
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
  float m = -__builtin_inff();  // running maximum of the exponent (log2 units), shared by both half-waves
  float l = 0.f;                // this lane's part of the running sum

  const DiagBounds vb = diag_bounds(a);
  // Row i sees the keys [jlo, jhi): j - i in (dlo, dhi), j < Sk (none past
  // the last row); key j is visible iff j - jlo < span (unsigned).
  const int jlo = max(i + vb.dlo + 1, 0);
  const int jhi = i < a.Sq ? min(i + vb.dhi, a.Sk) : 0;
  const uint32_t span = (uint32_t)max(jhi - jlo, 0);

  int kb, ke;
  key_range(a, q0, min(q0 + kDqRowsPerBlock, a.Sq) - 1, kb, ke);
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
      if constexpr (WO) {
#pragma unroll
        for (int e = 0; e < CH; ++e) sVT[(cc * CH + e) * PT + r] = vv[e];
      }
    }
    __syncthreads();
    if (rect_none_visible(a, qw0, qw0 + kDqRowsPerWave - 1, kt, kt + BK - 1)) continue;

    // S^T = K Q^T (C column = query row, C row = key).
    f32x16 st[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) st[mb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const int base = (32 * mb + l32) * PR + 2 * CH * ks + CH * h2;
        M::run(st[mb], *reinterpret_cast<const chunk*>(&sK[base]), qr[ks]);
      }
    }

#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      // Element r: key j = kt + 32*mb + 8*(r/4) + 4*h2 + r%4 of row i.
      float x[16];
      float tmax = -__builtin_inff();
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = kt + 32 * mb + 8 * (r >> 2) + 4 * h2 + (r & 3);
        bool ok = (uint32_t)(j - jlo) < span;
        float v = st[mb][r] * a.scale_log2;
        if constexpr (MASK) {
          const float mv = ok ? mask_at(a, b, h, i, j) : 0.f;
          ok = ok && !(mv <= kMaskedSentinel);
          v = __builtin_fmaf(mv, kLog2e, v);
        }
        x[r] = ok ? v : -__builtin_inff();
        tmax = fmaxf(tmax, x[r]);
      }
      const float mnew = fmaxf(m, halves_max(tmax));
      const float mref = mnew == -__builtin_inff() ? 0.f : mnew;  // nothing counted yet: every term is 0
      const float alpha = __builtin_amdgcn_exp2f(m - mref);
      l *= alpha;
      if constexpr (WO) {
#pragma unroll
        for (int d = 0; d < DB; ++d)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[d][r] *= alpha;
      }
      m = mnew;
      f32x16 pm;  // P.M in the C layout of S^T: the B operand of O^T += V^T (P.M)^T
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = __builtin_amdgcn_exp2f(x[r] - mref);
        l += p;
        if constexpr (DROP && WO) {
          const int j = kt + 32 * mb + 8 * (r >> 2) + 4 * h2 + (r & 3);
          p = drop_keep(rkey, j, a.drop_thr) ? p * a.drop_inv : 0.f;
        }
        pm[r] = p;
      }
      if constexpr (WO) {
#pragma unroll
        for (int t = 0; t < TC; ++t) {
          const chunk pc = M::from_acc(pm, t * CH);
#pragma unroll
          for (int d = 0; d < DB; ++d) {
            const int trow = (32 * d + l32) * PT;
            const int kk = 32 * mb + 8 * t + 4 * h2;  // the keys of C registers 4t .. 4t+3
            chunk av;
#pragma unroll
            for (int e = 0; e < CH; ++e) av[e] = sVT[trow + kk + e];
            M::run(acc[d], av, pc);
          }
        }
      }
    }
  }

  const float lsum = halves_sum(l);
  if (i < a.Sq) {
    if constexpr (WO) {
      const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
      for (int d = 0; d < DB; ++d) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          if (32 * d + 8 * r4 + 4 * h2 >= a.D) continue;  // past the head dimension
          f32x4 o4;
#pragma unroll
          for (int e = 0; e < 4; ++e) o4[e] = acc[d][4 * r4 + e] * inv;
          *reinterpret_cast<f32x4*>(O + qoff + 32 * d + 8 * r4 + 4 * h2) = o4;
        }
      }
    }
    if (h2 == 0)
      Lout[((int64_t)b * a.Hq + h) * a.Sq + i] =
          lsum > 0.f ? (m + __builtin_log2f(lsum)) * 0.6931471805599453f : __builtin_inff();
  }
}

template <int D, bool MASK, bool DROP, bool WO>
static hipError_t launch_t(const PrefillArgs& a, const void* Q, const void* K, const void* V, void* O, float* L,
                           hipStream_t st) {
  const int nqb = (a.Sq + kDqRowsPerBlock - 1) / kDqRowsPerBlock;
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
