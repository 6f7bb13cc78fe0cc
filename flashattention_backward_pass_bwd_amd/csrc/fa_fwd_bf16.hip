// Forward pass producing O and L with the backward's conventions, bf16 storage,
// bf16 MFMA with fp32 accumulation (ferrotensor-backend
// flash_attention_v2_backward.wgsl: the forward whose O and L the backward
// takes -- its file is referenced there, not shown -- and the online
// log-sum-exp of its dQ pass's first sweep; rustytorch
// flash_attention_backward_dq.metal takes L as an input):
//   S_ij = scale * Q_i.K_j + mask_ij on visible, unmasked elements,
//   L_i = log sum_j exp(S_ij)  (natural log; +inf when no element counts),
//   O_i = sum_j exp(S_ij - L_i) M_ij V_j   (M the dropout multiplier).
//
// Block: 4 waves own 128 consecutive query rows of one (b, h); wave w keeps its
// 32 rows of Q as the B operand of S^T = K Q^T (v_mfma_f32_32x32x16_bf16), so
// every lane column is one query row: the row's running maximum and sum are
// per-lane values (the two half-waves, which hold different keys of the same
// rows, agree on the maximum through v_permlane32_swap and add their sums at
// the end).  Per 64-key tile: K and V rows go into a 2-stage LDS ring
// (swizzled, see fa_tiles.h) by direct global->LDS copies one tile ahead;
// S^T of both 32-key halves (A operand: K rows), the exponents in fp32 (scale
// applied to the fp32 product, so L keeps fp32 accuracy), one lazy rescale
// test for the tile (a row's reference maximum moves only when passed by more
// than 2^8), and per half O^T += V^T (P.M)^T with V^T through
// ds_read_b64_tr_b16 and (P.M)^T straight from the C registers of S^T.  The
// MFMAs are compiler builtins, so the compiler keeps their wait states; two
// blocks share a CU.
// With WO false the kernel computes L alone (no V, no O): the log-sum-exp
// sweep for a caller whose forward did not keep L.
#include <type_traits>

#include "fa_internal.h"
#include "fa_tiles.h"

namespace fa {

constexpr int kFwdRowsPerBlock = 128;
constexpr float kLazyLog2 = 8.f;  // lag of a row's reference maximum before O is rescaled (log2 units)

// MV: a mask whose keys are contiguous and 16-byte aligned in groups of 4
// (mask_keys_contiguous): each lane reads its 4 consecutive keys at once.
template <int D, bool MASK, bool DROP, bool WO, bool MV>
__global__ __launch_bounds__(256, 2) void fwd_bf16_kernel(PrefillArgs a, const __bf16* __restrict__ Q,
                                                          const __bf16* __restrict__ K,
                                                          const __bf16* __restrict__ V, __bf16* __restrict__ O,
                                                          float* __restrict__ Lout) {
  constexpr int BK = 64;
  constexpr int NCH = D / 8;  // 16-byte chunks per row
  constexpr int KS = D / 16;  // k-blocks of the head_dim contraction
  constexpr int DB = D / 32;  // 32-row blocks of O^T
  constexpr int RPI = 1024 / (2 * D);  // tile rows per 1 KB copy
  constexpr int NIW = BK / RPI / 4;    // copies per wave per tile per tensor
  constexpr int NC = (WO ? 2 : 1) * NIW;
  __shared__ __attribute__((aligned(16))) __bf16 sK[2][BK * D];
  __shared__ __attribute__((aligned(16))) __bf16 sV[WO ? 2 : 1][BK * D];

  // Last query blocks first (under causal attention the longest); the KV head
  // varies fastest, then the query head of its group: blocks are dealt to the
  // XCDs round-robin, so the query heads of one KV head run on the same XCD
  // and read its K and V rows through one L2.
  const int nqb = (a.Sq + kFwdRowsPerBlock - 1) / kFwdRowsPerBlock;
  const int nkv = a.B * a.Hkv;
  const int kvi = blockIdx.x % nkv;
  const int rest = blockIdx.x / nkv;
  const int qbi = nqb - 1 - rest / a.group;
  const int kvh = kvi % a.Hkv;
  const int b = kvi / a.Hkv;
  const int h = kvh * a.group + rest % a.group;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int h2 = lane >> 5;
  const int l32 = lane & 31;
  const int q0 = qbi * kFwdRowsPerBlock;
  const int i = q0 + 32 * wave + l32;  // this lane's query row
  const int ic = min(i, a.Sq - 1);

  // Q row i as the B operand: k-block ks holds d = 16ks + 8*h2 .. +7.
  bf16x8 qr[KS];
  const __bf16* qrow = Q + (int64_t)b * a.qsb + (int64_t)ic * a.qss + (int64_t)h * a.qsh;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)  // zero past the head dimension
    qr[ks] = 2 * ks + h2 < a.D / 8 ? *reinterpret_cast<const bf16x8*>(qrow + 16 * ks + 8 * h2) : bf16x8{};

  int kb, ke;
  key_range(a, q0, min(q0 + kFwdRowsPerBlock, a.Sq) - 1, kb, ke);
  if constexpr (MV) kb -= kb % BK;  // tiles on 64-key boundaries (the keys added are invisible)
  const DiagBounds vb = diag_bounds(a);
  const uint32_t rkey = DROP ? drop_row_key(a, b, h, ic) : 0u;
  const float* mrow = MASK ? a.mask + (int64_t)b * a.msb + (int64_t)h * a.msh + (int64_t)ic * a.msq : nullptr;

  int tr_lo[DB], tr_hi[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d) {
    tr_lo[d] = tr_lane_off<D>(lane, d, 0);
    tr_hi[d] = tr_lane_off<D>(lane, d, 8);
  }

  f32x16 acc[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d) acc[d] = f32x16{};
  float m = -__builtin_inff();  // running maximum of the exponent (log2 units), shared by both half-waves
  float l = 0.f;                // this lane's part of the running sum
  const __bf16* kbase = K + (int64_t)b * a.ksb + (int64_t)kvh * a.ksh;
  const __bf16* vbase = WO ? V + (int64_t)b * a.ksb + (int64_t)kvh * a.ksh : nullptr;  // V is NULL for L alone

  // Copy u of this wave fills tile rows (wave*NIW + u)*RPI + lane/NCH, lane l
  // landing in physical chunk l%NCH (so it fetches the logical chunk stored
  // there); rows past the last key repeat it.
  uint32_t cp_off[NIW], cp_chk[NIW];
#pragma unroll
  for (int u = 0; u < NIW; ++u) {
    const int r = (wave * NIW + u) * RPI + lane / NCH;
    cp_chk[u] = 16u * (uint32_t)pad_chunk((lane % NCH) ^ swz<D>(r), a.D / 8);
    cp_off[u] = 2u * (uint32_t)r * (uint32_t)a.kss + cp_chk[u];
  }
  auto issue = [&](int kt, int st) {  // the copies of the tile at key kt into stage st
    const int kc = min(kt, a.Sk - 1);
    const uint32_t lim2 = 2u * (uint32_t)min(a.Sk - 1 - kc, BK) * (uint32_t)a.kss;
#pragma unroll
    for (int u = 0; u < NIW; ++u) {
      const uint32_t off = min(cp_off[u], lim2 + cp_chk[u]);
      dma16(kbase + (int64_t)kc * a.kss, off, lds_addr(&sK[st][(wave * NIW + u) * RPI * D]));
      if constexpr (WO) dma16(vbase + (int64_t)kc * a.kss, off, lds_addr(&sV[st][(wave * NIW + u) * RPI * D]));
    }
  };
  if (kb < ke) issue(kb, 0);
  int st = 0;
  for (int kt = kb; kt < ke; kt += BK, st ^= 1) {
    barrier_lds();  // every wave is done with the tile before, whose stage the next copies refill
    if (kt + BK < ke) {
      issue(kt + BK, st ^ 1);
      wait_vmcnt<NC>();  // this wave's copies of tile kt landed (the next tile's are in flight)
    } else {
      wait_vmcnt<0>();
    }
    barrier_lds();  // ... and every wave's
    // every element of the block's rows and the tile's keys visible, no mask:
    // no per-element test (block-uniform)
    const bool full = !MASK && rect_all_visible(a, q0, q0 + kFwdRowsPerBlock - 1, kt, kt + BK - 1);
    // Row i sees the keys [jlo, jhi): j - i in (dlo, dhi), j < Sk (none past
    // the last row); element key j is visible iff j - jlo < span (unsigned).
    const int jlo = max(i + vb.dlo + 1, 0);
    const int jhi = i < a.Sq ? min(i + vb.dhi, a.Sk) : 0;
    const uint32_t span = (uint32_t)max(jhi - jlo, 0);
    // The tile's work, with the per-element visibility test compiled out of
    // fully visible unmasked tiles.
    auto tile = [&](auto full_c) {
      constexpr bool FULL = decltype(full_c)::value;
      // S^T of both 32-key halves first (row 32*half + l32 of the tile is the A
      // operand's key): the second chain runs on the matrix cores while the
      // first half's exponents are computed; one rescale test per tile.
      f32x16 sh[2];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        sh[half] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 kr = lds_read_b128(&sK[st][tile_off<D>(32 * half + l32, 2 * ks + h2)]);
          sh[half] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr, qr[ks], sh[half], 0, 0, 0);
        }
      }
      // The exponents of both halves (in place of S^T) and their maximum.
      // Element r of half h: key j = kt + 32*h + 8*(r/4) + 4*h2 + r%4 of row i.
      float tmax = -__builtin_inff();
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        f32x4 mq[4];  // MV: the mask values of keys kt + 32*half + 8g + 4*h2 .. +3
        if constexpr (MASK && MV) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int j0 = kt + 32 * half + 8 * g + 4 * h2;
            mq[g] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (i < a.Sq && j0 + 3 - i > vb.dlo && j0 - i < vb.dhi) {
              if (j0 + 3 < a.Sk) {  // the whole group in range: one 16-byte load
                mq[g] = *reinterpret_cast<const f32x4*>(mrow + j0);
              } else {              // the last keys: one by one, none past Sk - 1
#pragma unroll
                for (int e = 0; e < 4; ++e) mq[g][e] = j0 + e < a.Sk ? mrow[j0 + e] : 0.f;
              }
            }
          }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = kt + 32 * half + 8 * (r >> 2) + 4 * h2 + (r & 3);
          bool ok = FULL || (uint32_t)(j - jlo) < span;
          float v = sh[half][r] * a.scale_log2;
          if constexpr (MASK) {
            float mv;
            if constexpr (MV) mv = mq[r >> 2][r & 3];
            else mv = ok ? mrow[(int64_t)j * a.msk] : 0.f;
            ok = ok && !(mv <= kMaskedSentinel);
            v = __builtin_fmaf(mv, kLog2e, v);
          }
          sh[half][r] = ok ? v : -__builtin_inff();
          tmax = fmaxf(tmax, sh[half][r]);
        }
      }
      // The row's reference m moves only when the tile's maximum passes it by
      // more than kLazyLog2 (then O and the sum are rescaled); otherwise the
      // terms exp2(x - m) stay at most 2^kLazyLog2, well inside fp32 and bf16
      // range, and O, the sum and L all use the same m, so the result is the same.
      const float mt = halves_max(tmax);
      const bool grow = mt > m + kLazyLog2;  // m = -inf: any counted element
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
      for (int half = 0; half < 2; ++half) {
        bf16x8 pm[2];
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          float p0 = __builtin_amdgcn_exp2f(sh[half][r] - mref), p1 = __builtin_amdgcn_exp2f(sh[half][r + 1] - mref);
          l += p0 + p1;
          if constexpr (DROP && WO) {
            const int j = kt + 32 * half + 8 * (r >> 2) + 4 * h2 + (r & 3);
            p0 = drop_keep(rkey, j, a.drop_thr) ? p0 * a.drop_inv : 0.f;
            p1 = drop_keep(rkey, j + 1, a.drop_thr) ? p1 * a.drop_inv : 0.f;
          }
          pm[r >> 3][r & 7] = (__bf16)p0;
          pm[r >> 3][(r & 7) + 1] = (__bf16)p1;
        }
        // O^T += V^T (P.M)^T: k-step t covers keys 32*half + 16t .. +15.
#pragma unroll
        for (int t = 0; t < (WO ? 2 : 0); ++t) {
#pragma unroll
          for (int d = 0; d < DB; ++d) {
            const __bf16* base = &sV[WO ? st : 0][(32 * half + 16 * t) * D];
            const bf16x8 vt = concat(lds_read_tr(base + tr_lo[d]), lds_read_tr(base + tr_hi[d]));
            acc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vt, pm[t], acc[d], 0, 0, 0);
          }
        }
      }
    };
    if (full) tile(std::true_type{});
    else tile(std::false_type{});
  }

  const float lsum = halves_sum(l);
  if (i < a.Sq) {
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    __bf16* orow = WO ? O + (int64_t)b * a.qsb + (int64_t)i * a.qss + (int64_t)h * a.qsh : nullptr;  // O is NULL for L alone
#pragma unroll
    for (int d = 0; d < (WO ? DB : 0); ++d) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        if (32 * d + 8 * r4 + 4 * h2 >= a.D) continue;  // past the head dimension
        bf16x4 o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = (__bf16)(acc[d][4 * r4 + e] * inv);
        *reinterpret_cast<bf16x4*>(orow + 32 * d + 8 * r4 + 4 * h2) = o4;
      }
    }
    if (h2 == 0)
      Lout[((int64_t)b * a.Hq + h) * a.Sq + i] =
          lsum > 0.f ? (m + __builtin_log2f(lsum)) * 0.6931471805599453f : __builtin_inff();
  }
}

template <int D, bool MASK, bool DROP, bool WO, bool MV = false>
static hipError_t launch_t(const PrefillArgs& a, const void* Q, const void* K, const void* V, void* O, float* L,
                           hipStream_t st) {
  const int nqb = (a.Sq + kFwdRowsPerBlock - 1) / kFwdRowsPerBlock;
  const unsigned grid = (unsigned)((int64_t)nqb * a.B * a.Hq);
  hipLaunchKernelGGL((fwd_bf16_kernel<D, MASK, DROP, WO, MV>), dim3(grid), dim3(256), 0, st, a,
                     static_cast<const __bf16*>(Q), static_cast<const __bf16*>(K), static_cast<const __bf16*>(V),
                     static_cast<__bf16*>(O), L);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_d(const PrefillArgs& a, const void* Q, const void* K, const void* V, void* O, float* L,
                           hipStream_t st) {
  const bool mk = a.mask != nullptr, dr = a.drop != 0;
  if (O == nullptr)  // L alone: dropout does not enter it
    return mk ? launch_t<D, true, false, false>(a, Q, K, V, O, L, st) : launch_t<D, false, false, false>(a, Q, K, V, O, L, st);
  if (mk && mask_keys_contiguous(a))
    return dr ? launch_t<D, true, true, true, true>(a, Q, K, V, O, L, st)
              : launch_t<D, true, false, true, true>(a, Q, K, V, O, L, st);
  if (mk)
    return dr ? launch_t<D, true, true, true>(a, Q, K, V, O, L, st) : launch_t<D, true, false, true>(a, Q, K, V, O, L, st);
  return dr ? launch_t<D, false, true, true>(a, Q, K, V, O, L, st) : launch_t<D, false, false, true>(a, Q, K, V, O, L, st);
}

// O == nullptr: L alone (V is not read).
hipError_t launch_fwd_bf16(const PrefillArgs& a, int D, const void* Q, const void* K, const void* V, void* O,
                           float* L, hipStream_t st) {
  return D <= 64 ? launch_d<64>(a, Q, K, V, O, L, st) : launch_d<128>(a, Q, K, V, O, L, st);
}

}  // namespace fa
