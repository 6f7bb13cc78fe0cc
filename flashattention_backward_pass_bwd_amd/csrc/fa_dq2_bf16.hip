// Query-block-outer dQ pass for head dimension 128 with two 32-row blocks per
// wave, bf16 storage, bf16 MFMA with fp32 accumulation (rustytorch
// flash_attention_backward_dq.metal kernel; ferrotensor-backend
// flash_attention_v2_backward.wgsl, flash_bwd_dq second sweep, L supplied):
//   dQ_i = scale * sum_j dS_ij K_j,  dS_ij = P_ij (dO_i.V_j - Delta_i).
//
// Block: 4 waves own 256 consecutive query rows of one (b, h); wave w keeps
// its 64 rows (row blocks rb = 0, 1 of 32 rows) of Q and dO in accumulation
// registers as MFMA B operands and accumulates dQ^T (D x 64 fp32) there too.
// Each operand read from LDS feeds two MFMAs, one per row block, so a wave
// issues half the LDS reads, copies and loop bookkeeping per MFMA of a
// 32-row wave.  Per 32-key half of a 64-key tile:
//   X: S^T = K Q^T and dP^T = V dO^T for both row blocks (32 MFMAs, chains
//      started from -L_i/scale and -Delta_i as in the 32-row kernel); the
//      exps of S^T run under the dP^T MFMAs;
//   Y: dQ^T += K^T dS^T of the previous half (16 MFMAs) with dS of this half.
// So one set of S/dP accumulators is live at a time and dQ trails S/dP by a
// half.  A step (one tile) is  barrier | X Y (second half) | X Y (first half
// of the next tile); the K/V ring and its copies work as in the 32-row
// kernel (4 stages, three tiles ahead, one barrier per tile).  Launched
// without window, mask or dropout (the 32-row kernel takes those); the
// geometric predicate (causal, offset, ragged ends) works for any window.
#include <type_traits>

#include "fa_internal.h"
#include "fa_tiles.h"

namespace fa {

__global__ __launch_bounds__(256, 1) void dq2_bf16_kernel(PrefillArgs a, const __bf16* __restrict__ Q,
                                                          const __bf16* __restrict__ K,
                                                          const __bf16* __restrict__ V,
                                                          const __bf16* __restrict__ dO,
                                                          const float* __restrict__ L,
                                                          const float* __restrict__ Dl,
                                                          __bf16* __restrict__ dQ, int nqb, int paired) {
  constexpr int D = 128;
  constexpr int BK = 64;
  constexpr int NCH = D / 8;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int NST = 4;               // K/V ring stages
  constexpr int RPI = 1024 / (2 * D);  // tile rows per 1 KB global->LDS copy
  constexpr int NIW = BK / RPI / 4;    // copies per wave per tile per tensor
  constexpr int TILE = BK * D;
  constexpr int RB = 2;                // row blocks per wave
  constexpr int NOP = 2 * KS;          // row-major operands of a half: K chunks 0..KS-1, then V chunks
  constexpr int NX = RB * NOP;         // S/dP MFMAs of a half
  constexpr int NTR = 2 * DB;          // transposed operands (two reads each) of a half's dQ
  constexpr int NY = RB * NTR;         // dQ MFMAs of a half
  constexpr int PFO = 4;               // row-major operands read ahead
  constexpr int NB = PFO + 2;          // their ring
  constexpr int PFT = 3;               // transposed operands read ahead
  constexpr int NBT = PFT + 2;
  constexpr int NC = 2 * NIW;          // copies per tile per wave
  constexpr int PER = NC / 4;          // copies per section
  // Exps of S^T row block rb run in slots kExp0 + rb .. NX - 1 of X, three
  // MFMAs after the chain's last one and behind explicit wait states; dS of row
  // block rb in slots kDs0 + rb .. NY - 1 of Y, three MFMAs after the dP^T
  // chain's last one (an MFMA result is read by other instructions only after
  // its twelve wait states).
  constexpr int kExp0 = 2 * KS + 2;
  constexpr int kDs0 = 2;
  constexpr int kPre0 = 9;             // Y slots kPre0 .. kPre0+PFO-1 read the next X's first operands
  static_assert(NC % 4 == 0 && NX % PER == 0 && NY % PER == 0, "a tile's copies spread over four sections");
  static_assert(PFT <= PFO && kPre0 + PFO <= NY, "read schedule");

  __shared__ __attribute__((aligned(16))) __bf16 sT[NST][2][TILE];

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

  const int cp_row = lane / NCH;
  const int cp_pc = lane % NCH;
  int rd_off[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) rd_off[ks] = tile_off<D>(l32, 2 * ks + h2);
  int tr_lo[DB], tr_hi[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d) {
    tr_lo[d] = tr_lane_off<D>(lane, d, 0);
    tr_hi[d] = tr_lane_off<D>(lane, d, 8);
  }

  const int npass = paired ? 2 : 1;
  for (int pass = 0; pass < npass; ++pass) {
    const int qbi = paired ? (pass == 0 ? wi : nqb - 1 - wi) : nqb - 1 - wi;
    if (pass == 1 && qbi <= wi) break;
    const int q0 = qbi * kDq2RowsPerBlock;
    const int qw0 = q0 + wave * kDq2RowsPerWave;

    // Q and dO rows of both row blocks into accumulation registers; rows past
    // the end repeat the last row and are not written.
    int il[RB];
    int64_t qoff[RB];
    bf16x8 qr[RB][KS], gr[RB][KS];
    float nl[RB], del[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      il[rb] = qw0 + 32 * rb + l32;
      qoff[rb] = (int64_t)b * a.qsb + (int64_t)il[rb] * a.qss + (int64_t)h * a.qsh;
      const int64_t qclamp = (int64_t)b * a.qsb + (int64_t)min(il[rb], a.Sq - 1) * a.qss + (int64_t)h * a.qsh;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        qr[rb][s] = ld16_op(row_chunk(Q + qclamp, 2 * s + h2, a.D / 8));  // zero past the head dimension
        gr[rb][s] = ld16_op(row_chunk(dO + qclamp, 2 * s + h2, a.D / 8));
      }
      const int64_t lrow = ((int64_t)b * a.Hq + h) * a.Sq + min(il[rb], a.Sq - 1);
      nl[rb] = il[rb] < a.Sq ? -L[lrow] * a.inv_scale : 0.f;  // rows past the end: never counted
      del[rb] = il[rb] < a.Sq ? Dl[lrow] : 0.f;
    }
    f32x16 accq[RB][DB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int d = 0; d < DB; ++d) accq[rb][d] = f32x16{};
    wait_all_vmem();

    int kb, ke;
    key_range(a, q0, min(q0 + kDq2RowsPerBlock, a.Sq) - 1, kb, ke);
    const int ntiles = (ke - kb + BK - 1) / BK;

    if (ntiles > 0) {
      // Chain seeds: every C register of a lane is query row il[rb].
      f32x16 nls[RB], dpi[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          nls[rb][r] = nl[rb];
          dpi[rb][r] = -del[rb];
        }
        pin(nls[rb]);
        pin(dpi[rb]);
      }

      // K and V rows of a tile into a ring stage, as in the 32-row kernel.
      struct Job {
        const __bf16* kp;
        const __bf16* vp;
        uint32_t lds;
        uint32_t lim2;
      };
      uint32_t cp_off[NIW], cp_chk[NIW];
#pragma unroll
      for (int i = 0; i < NIW; ++i) {
        const int r = (wave * NIW + i) * RPI + cp_row;
        cp_chk[i] = 16u * (uint32_t)pad_chunk(cp_pc ^ swz<D>(r), a.D / 8);
        cp_off[i] = 2u * (uint32_t)r * (uint32_t)a.kss + cp_chk[i];
      }
      auto job_at = [&](int kt, int64_t base, int stage) {
        const uint32_t lim = (uint32_t)min(a.Sk - 1 - kt, BK);
        return Job{K + base, V + base, lds_addr(&sT[stage][0][wave * NIW * RPI * D]), 2u * lim * (uint32_t)a.kss};
      };
      auto job_of = [&](int tt, int stage) {
        const int kt = kb + min(tt, ntiles - 1) * BK;
        return job_at(kt, (int64_t)b * a.ksb + (int64_t)kt * a.kss + (int64_t)kvh * a.ksh, stage);
      };
      int ct_kt = kb + min(3, ntiles - 1) * BK;
      int64_t ct_base = (int64_t)b * a.ksb + (int64_t)ct_kt * a.kss + (int64_t)kvh * a.ksh;
      const int kt_last = kb + (ntiles - 1) * BK;
      const int64_t inc_kt = (int64_t)BK * a.kss;
      auto issue_job = [&](const Job& j, int u) {
        const uint32_t off = min(cp_off[u >> 1], j.lim2 + cp_chk[u >> 1]);
        const uint32_t lds = j.lds + 2u * (uint32_t)((u >> 1) * RPI * D + (u & 1) * TILE);
        dma16((u & 1) ? j.vp : j.kp, off, lds);
      };
      auto copies_at = [&](const Job& j, int u0, int k, int nslots) {
        if (k % (nslots / PER) == 0) issue_job(j, u0 + k / (nslots / PER));
      };

      auto fence = []() { __builtin_amdgcn_sched_barrier(0); };
      // Row-major A operand o of a half: K chunk o (o < KS) or V chunk o - KS.
      auto rd_op = [&](int m, int stq, int o) {
        return lds_read_b128(sT[stq][o >= KS ? 1 : 0] + rd_off[o % KS] + 32 * m * D);
      };
      // Transposed A operand half j of dQ operand n = j/2 = DB*t + d of half m.
      auto rd_tr = [&](int m, int stq, int j) {
        const int n = j >> 1, t = n / DB, d = n % DB;
        return lds_read_tr(sT[stq][0] + (32 * m + 16 * t) * D + ((j & 1) ? tr_hi[d] : tr_lo[d]));
      };

      // Section X: S^T/dP^T of half m of the tile at key kt (stage stq), first
      // PFO operands in pre; exps of S^T in place (P), with the predicate on
      // edge tiles.  TRPRE: the last slots read the first PFT transposed
      // operands of the next Y's dQ (half mq, stage stqq) into trp.
      auto sec_x = [&](auto full_c, auto trpre_c, int m, int stq, int kt, f32x16 (&s)[RB], f32x16 (&dp)[RB],
                       const bf16x8 (&pre)[PFO], int mq, int stqq, bf16x4 (&trp)[PFT][2], auto&& slot_extra) {
        constexpr bool FULL = decltype(full_c)::value;
        constexpr bool TRPRE = decltype(trpre_c)::value;
        bf16x8 buf[NB];
#pragma unroll
        for (int k = 0; k < PFO; ++k) buf[k] = pre[k];
        // Visible keys of row block rb's row in the half: element r (key
        // 32*m + 4*h2 + c(r), c(r) = 8*(r/4) + r%4) counts iff c(r) - lb < span.
        int lb[RB] = {0, 0};
        uint32_t span[RB] = {0u, 0u};
        if constexpr (!FULL) {
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            const int dl0 = kt - il[rb];
            const int lo = max(vb.dlo - dl0 + 1, 0);
            const int hi = il[rb] < a.Sq ? min(vb.dhi - dl0, a.Sk - kt) : 0;
            span[rb] = (uint32_t)max(hi - lo, 0);
            lb[rb] = lo - 32 * m - 4 * h2;
          }
        }
        auto ew_exp = [&](int rb, int r) {
          float x = s[rb][r] * a.scale_log2;  // s holds Q.K - L/scale
          if constexpr (!FULL) {
            const bool ok = elem_visible(r, lb[rb], span[rb]);
            x = ok ? x : -__builtin_inff();
          }
          s[rb][r] = __builtin_amdgcn_exp2f(x);
        };
        fence();
#pragma unroll
        for (int j = 0; j < NX; ++j) {
          const int o = j >> 1, rb = j & 1;
          const bf16x8& op = buf[o % NB];
          if (o < KS) {
            if (o == 0)
              mfma_v_cseed(s[rb], op, qr[rb][0], nls[rb]);
            else
              mfma_v(s[rb], op, qr[rb][o]);
          } else {
            if (o == KS)
              mfma_v_cseed(dp[rb], op, gr[rb][0], dpi[rb]);
            else
              mfma_v(dp[rb], op, gr[rb][o - KS]);
          }
          fence();  // the slot's other work follows its MFMA
          if (rb == 0) {
            if (o + PFO < NOP) {
              buf[(o + PFO) % NB] = rd_op(m, stq, o + PFO);
            } else if constexpr (TRPRE) {
              const int q = o + PFO - NOP;
              if (q < PFT) {
                trp[q][0] = rd_tr(mq, stqq, 2 * q);
                trp[q][1] = rd_tr(mq, stqq, 2 * q + 1);
              }
            }
          }
#pragma unroll
          for (int e = 0; e < RB; ++e) {
            const int first = kExp0 + e, n = NX - first;
            if (j == first) mfma_result_wait(s[e]);
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (first + (r * n) / 16 == j) ew_exp(e, r);
          }
          slot_extra(j);
          fence();
        }
        // the seed blocks stay allocated up to here, well after the seeded MFMAs
        // that may still read them (also in the last section of the kernel)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          keep_live(nls[rb]);
          keep_live(dpi[rb]);
        }
      };

      // Section Y: dQ of half mq (stage stqq) from its dS^T dsq (MF), with the
      // first PFT transposed operands in trp; dS^T of the half just computed
      // (P in p, dP - Delta in dp) into dsn (DS); the next X's first PFO
      // operands (half mn, stage stn) into pre (PRE).
      auto sec_y = [&](auto mf_c, auto ds_c, auto pre_c, int mq, int stqq, const bf16x8 (&dsq)[RB][2],
                       const bf16x4 (&trp)[PFT][2], const f32x16 (&p)[RB], const f32x16 (&dp)[RB],
                       bf16x8 (&dsn)[RB][2], int mn, int stn, bf16x8 (&pre)[PFO], auto&& slot_extra) {
        constexpr bool MF = decltype(mf_c)::value;
        constexpr bool DS = decltype(ds_c)::value;
        constexpr bool PRE = decltype(pre_c)::value;
        bf16x4 tb[NBT][2];
#pragma unroll
        for (int q = 0; q < PFT; ++q) {
          tb[q][0] = trp[q][0];
          tb[q][1] = trp[q][1];
        }
        float dv[RB][16];
        auto ew_ds = [&](int rb, int r) {
          dv[rb][r] = p[rb][r] * dp[rb][r];
          if (r & 1) {
            const bf16x2 t = pack_here(dv[rb][r - 1], dv[rb][r]);
            dsn[rb][r >> 3][(r & 7) - 1] = t[0];
            dsn[rb][r >> 3][r & 7] = t[1];
          }
        };
        fence();
#pragma unroll
        for (int j = 0; j < NY; ++j) {
          const int n = j >> 1, rb = j & 1;
          if constexpr (MF) {
            mfma_acc(accq[rb][n % DB], concat(tb[n % NBT][0], tb[n % NBT][1]), dsq[rb][n / DB]);
            fence();
            if (rb == 0 && n + PFT < NTR) {
              tb[(n + PFT) % NBT][0] = rd_tr(mq, stqq, 2 * (n + PFT));
              tb[(n + PFT) % NBT][1] = rd_tr(mq, stqq, 2 * (n + PFT) + 1);
            }
          }
          if constexpr (PRE) {
            if (j >= kPre0 && j - kPre0 < PFO) pre[j - kPre0] = rd_op(mn, stn, j - kPre0);
          }
          if constexpr (DS) {
#pragma unroll
            for (int e = 0; e < RB; ++e) {
              const int first = kDs0 + e, nn = NY - first;
#pragma unroll
              for (int r = 0; r < 16; ++r)
                if (first + (r * nn) / 16 == j) ew_ds(e, r);
            }
          }
          slot_extra(j);
          fence();
        }
        if constexpr (DS) materialise(dsn[0], dsn[1]);
      };

      // Prologue: tiles 0, 1 and 2 copied, tile 0 landed.
#pragma unroll
      for (int u = 0; u < NC; ++u) issue_job(job_of(0, 0), u);
#pragma unroll
      for (int u = 0; u < NC; ++u) issue_job(job_of(1, 1), u);
#pragma unroll
      for (int u = 0; u < NC; ++u) issue_job(job_of(2, 2), u);
      wait_vmcnt<2 * NC>();
      barrier_lds();

      const std::false_type no;
      const std::true_type yes;
      auto none = [](int) {};
      f32x16 s[RB], dp[RB];
      bf16x8 dsa[RB][2], dsb[RB][2];
      bf16x8 pre[PFO];
      bf16x4 trp[PFT][2];
#pragma unroll
      for (int k = 0; k < PFO; ++k) pre[k] = rd_op(0, 0, k);
      // X of tile 0's first half; its dS (no dQ to overlap yet) and the
      // operands of the second half.
      sec_x(no, no, 0, 0, kb, s, dp, pre, 0, 0, trp, none);
      mfma_drain(s[0], s[1]);
      mfma_drain(dp[0], dp[1]);
      sec_y(no, yes, yes, 0, 0, dsb, trp, s, dp, dsa, 1, 0, pre, none);

      int it = 0;
      // Step of tile it (it < ntiles - 1): its second half and the next tile's first.
      auto step = [&](auto full_c) {
        const int stq = it & (NST - 1);
        const int stq1 = (it + 1) & (NST - 1);
        const int stq3 = (it + 3) & (NST - 1);
        const int kt = kb + it * BK;
        // tile it+1 landed everywhere, and every wave is done with tile it-1,
        // whose stage tile it+3 refills
        wait_vmcnt<NC>();
        barrier_only();
        const Job next = job_at(ct_kt, ct_base, stq3);
        if (ct_kt < kt_last) {
          ct_kt += BK;
          ct_base += inc_kt;
        }
        sec_x(full_c, yes, 1, stq, kt, s, dp, pre, 0, stq, trp, [&](int j) { copies_at(next, 0, j, NX); });
        sec_y(yes, yes, yes, 0, stq, dsa, trp, s, dp, dsb, 0, stq1, pre,
              [&](int j) { copies_at(next, PER, j, NY); });
        sec_x(full_c, yes, 0, stq1, kt + BK, s, dp, pre, 1, stq, trp,
              [&](int j) { copies_at(next, 2 * PER, j, NX); });
        sec_y(yes, yes, yes, 1, stq, dsb, trp, s, dp, dsa, 1, stq1, pre,
              [&](int j) { copies_at(next, 3 * PER, j, NY); });
        ++it;
      };

      // Steps whose two tiles are both wholly visible to this wave run the
      // predicate-free kind; the others the edge kind (separate loops, no
      // branches in a step).
      auto all = [&](int t) {
        return rect_all_visible(a, qw0, qw0 + kDq2RowsPerWave - 1, kb + t * BK, kb + t * BK + BK - 1);
      };
      int f0 = 0;
      while (f0 < ntiles && !all(f0)) ++f0;
      int f1 = f0;
      while (f1 < ntiles && all(f1)) ++f1;
      const int last = ntiles - 1;
      const int e0 = min(f0, last);
      const int e1 = max(e0, min(f1 - 1, last));
      while (it < e0) step(no);  // (step advances it)
      while (it < e1) step(yes);
      while (it < last) step(no);

      // Tile `last`: its second half, the dQ of its first half, then of its second.
      {
        const int stq = last & (NST - 1);
        sec_x(no, yes, 1, stq, kt_last, s, dp, pre, 0, stq, trp, none);
        sec_y(yes, yes, no, 0, stq, dsa, trp, s, dp, dsb, 0, stq, pre, none);
#pragma unroll
        for (int q = 0; q < PFT; ++q) {
          trp[q][0] = rd_tr(1, stq, 2 * q);
          trp[q][1] = rd_tr(1, stq, 2 * q + 1);
        }
        sec_y(yes, no, no, 1, stq, dsb, trp, s, dp, dsa, 0, stq, pre, none);
      }
      wait_vmcnt<0>();  // the repeated copies of the last steps have landed
      barrier_lds();    // every wave is done with the ring before the next pass refills it
    }
    mfma_drain_acc(accq[0], accq[1]);

#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      if (il[rb] < a.Sq) {
#pragma unroll
        for (int d = 0; d < DB; ++d) {
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int dd = 32 * d + 8 * r4 + 4 * h2;
            if (dd >= a.D) continue;  // past the head dimension
            bf16x4 o4;
#pragma unroll
            for (int e = 0; e < 4; ++e) o4[e] = (__bf16)(accq[rb][d][4 * r4 + e] * a.scale);
            *reinterpret_cast<bf16x4*>(dQ + qoff[rb] + dd) = o4;
          }
        }
      }
    }
  }
}

hipError_t launch_dq2_bf16(const PrefillArgs& a, const void* Q, const void* K, const void* V, const void* dO,
                           const float* L, const float* delta, void* dQ, hipStream_t st) {
  const int nqb = (a.Sq + kDq2RowsPerBlock - 1) / kDq2RowsPerBlock;
  const int paired = (a.causal && a.window == 0 && nqb > 1) ? 1 : 0;
  const int nwi = paired ? (nqb + 1) / 2 : nqb;
  const unsigned grid = (unsigned)(nwi * a.B * a.Hq);
  hipLaunchKernelGGL(dq2_bf16_kernel, dim3(grid), dim3(256), 0, st, a, static_cast<const __bf16*>(Q),
                     static_cast<const __bf16*>(K), static_cast<const __bf16*>(V), static_cast<const __bf16*>(dO),
                     L, delta, static_cast<__bf16*>(dQ), nqb, paired);
  return hipGetLastError();
}

}  // namespace fa
