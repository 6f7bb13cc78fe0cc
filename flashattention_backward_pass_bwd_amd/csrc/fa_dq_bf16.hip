// Query-block-outer dQ pass, bf16 storage, bf16 MFMA with fp32 accumulation
// (rustytorch flash_attention_backward_dq.metal kernel; ferrotensor-backend
// flash_attention_v2_backward.wgsl, flash_bwd_dq second sweep, L supplied):
//   dQ_i = scale * sum_j dS_ij K_j,  dS_ij = P_ij (M_ij dO_i.V_j - Delta_i).
//
// Block: 4 waves own 128 consecutive query rows of one (b, h); wave w keeps its
// 32 rows of Q and dO in accumulation registers as MFMA B operands
// (v_mfma_f32_32x32x16_bf16) and accumulates dQ^T (D x 32 fp32) there too.
// Per 64-key tile and wave: S^T = K Q^T and dP^T = V dO^T (row-major A
// operands from LDS), P and dS^T in registers, then dQ^T += K^T dS^T (K
// transposed through ds_read_b64_tr_b16).  S^T has one query per lane column,
// so L_i and Delta_i are per-lane scalars: the S^T chain starts from
// -L_i/scale, so P is the exp2 of the fp32 MFMA result times scale*log2(e) (Q
// enters the MFMAs as stored), and without dropout the dP^T chain starts from
// -Delta_i, so dP - Delta comes out of the MFMAs.  dS^T is already the B
// operand of the last contraction.
//
// Software pipeline, as in the dK/dV kernel: a tile is two 32-key halves and
// the step of tile it runs
//   A: S/dP of half 1 (MFMA)      with  exp/dS of half 0 (VALU)
//      -- wait for tile it+1's copies, block barrier --
//   B: dQ of half 0
//   C: S/dP of half 0 of tile it+1 with exp/dS of half 1
//   D: dQ of half 1
// with every section's first operands read by the section before it.  K and V
// tiles live in a 4-stage LDS ring (swizzled, see fa_tiles.h) filled by direct
// global->LDS copies three tiles ahead, spread over the step.  Blocks of the
// query heads sharing a KV head are dealt to one XCD; for causal attention
// without a window, block i also takes query block nqb-1-i.
#include <type_traits>

#include "fa_internal.h"
#include "fa_tiles.h"

namespace fa {

// MK: 0 no mask, 1 a mask of any strides, 2 a mask whose keys are contiguous and
// whose 4-key groups are 16-byte aligned (read four keys per lane and copy).
template <int D, int MK, bool DROP>
__global__ __launch_bounds__(256, 1) void dq_bf16_kernel(PrefillArgs a, const __bf16* __restrict__ Q,
                                                         const __bf16* __restrict__ K,
                                                         const __bf16* __restrict__ V,
                                                         const __bf16* __restrict__ dO,
                                                         const float* __restrict__ L,
                                                         const float* __restrict__ Dl,
                                                         __bf16* __restrict__ dQ, int nqb, int paired) {
  constexpr bool MASK = MK != 0;
  constexpr bool MVEC = MK == 2;
  constexpr int BK = 64;
  constexpr int NCH = D / 8;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int NST = 4;                    // K/V ring stages
  constexpr int RPI = 1024 / (2 * D);       // tile rows per 1 KB global->LDS copy
  constexpr int NIW = BK / RPI / 4;         // copies per wave per tile per tensor
  constexpr int TILE = BK * D;
  constexpr bool FOLD = !DROP;              // dP chain seeded with -Delta
  constexpr int NSD = 2 * KS;               // S/dP MFMAs per 32-key half
  constexpr int NDQ = 2 * DB;               // dQ MFMAs per 32-key half
#ifndef FA_DQ_NP
#define FA_DQ_NP 4
#endif
  constexpr int NP = FA_DQ_NP < NDQ ? FA_DQ_NP : NDQ;  // dQ MFMAs whose operands the preceding section reads
#ifndef FA_DQ_PF
#define FA_DQ_PF 6
#endif
  constexpr int PF = NDQ < FA_DQ_PF ? NDQ : FA_DQ_PF;  // S/dP operand reads in flight
  static_assert(PF < 8, "operand reads run ahead within a ring of 8");
  constexpr int NC = 2 * NIW;               // copies per tile per wave
  constexpr int PER = NC / 4;               // copies per section
  // Mask staging (MASK): element r of a half is copied into sM right after the
  // same element of the other half was used (sections A and C, the slot of
  // element r), and read MF slots before its own use two sections later.  Of
  // the copies issued after it, at least 16 - E*(MF+1) mask copies and PER - 1
  // tile copies are issued before that read (E elements per slot), so waiting
  // for at most kMaskWait accesses in flight covers it.
  constexpr int MF = 2;
  constexpr int kMaskWait = 16 - (16 / NSD) * (MF + 1) + PER - 1;
  static_assert(kMaskWait >= 0, "mask staging wait");
  // With MVEC, group g (elements 4g .. 4g+3, one 16-byte copy per lane) is copied
  // after its last element's slot and read at the start of the previous group's
  // slots (SG slots per group): at least 2 group copies and PER tile copies are
  // issued in between, so waiting for at most 1 + PER accesses in flight covers it.
  constexpr int SG = 4 / (16 / NSD);
  constexpr int kMaskWaitV = 1 + PER;
  // Mask copies of section A issued after its last tile copy (slot sl).
  constexpr int sl = (PER - 1) * (NSD / PER);
  constexpr int kMaskLateA = MVEC ? (SG - 1 >= sl) + (2 * SG - 1 >= sl) + (3 * SG - 1 >= sl) + (4 * SG - 1 >= sl)
                                  : 16 / PER;
  constexpr int kMaskPerStep = MVEC ? 8 : 32;
  static_assert(NC % 4 == 0 && NDQ % PER == 0 && NSD % PER == 0, "a tile's copies spread over four sections");
  static_assert(2 * NP <= NSD && PF <= NSD && PF <= NDQ, "prefetches fit their sections");

  // Ring stage s holds the K tile (sT[s][0]) and the V tile (sT[s][1]).
  __shared__ __attribute__((aligned(16))) __bf16 sT[NST][2][TILE];
  // Mask values of one exp/dS half per wave: element r of lane l at sM[wave][r][l].
  __shared__ __attribute__((aligned(16))) float sM[MASK ? 4 : 1][MASK ? 16 : 1][64];

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

    // Q and dO rows of this wave's queries, in registers for the whole pass
    // (rows past the end repeat the last row; their results are not written).
    bf16x8 qr[KS], gr[KS];
    const int64_t qoff = (int64_t)b * a.qsb + (int64_t)il * a.qss + (int64_t)h * a.qsh;
    const int64_t qclamp = (int64_t)b * a.qsb + (int64_t)min(il, a.Sq - 1) * a.qss + (int64_t)h * a.qsh;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      qr[s] = ld16_op(row_chunk(Q + qclamp, 2 * s + h2, a.D / 8));  // zero past the head dimension
      gr[s] = ld16_op(row_chunk(dO + qclamp, 2 * s + h2, a.D / 8));
    }
    const int64_t lrow = ((int64_t)b * a.Hq + h) * a.Sq + min(il, a.Sq - 1);
    const float nl = il < a.Sq ? -L[lrow] * a.inv_scale : 0.f;  // rows past the end: never counted
    const float del = il < a.Sq ? Dl[lrow] : 0.f;
    uint32_t rk = 0;
    if constexpr (DROP) rk = drop_row_key(a, b, h, il);
    // Mask reads: byte offset of element (row, key) in the (b, h) slice is
    // row*msq*4 + key*msk*4; lanes fix the row (clamped) and the 4-key group.
    const uint32_t msk4 = MASK ? (uint32_t)a.msk * 4u : 0u;  // 4 with MVEC
    const uint32_t m_lvo = MASK ? ((uint32_t)min(il, a.Sq - 1) * (uint32_t)a.msq + 4u * h2 * (uint32_t)a.msk) * 4u : 0u;
    f32x16 accq[DB];
#pragma unroll
    for (int d = 0; d < DB; ++d) accq[d] = f32x16{};
    wait_all_vmem();  // Q, dO rows, L and Delta are in registers before the copy ring starts

    int kb, ke;
    key_range(a, q0, min(q0 + kDqRowsPerBlock, a.Sq) - 1, kb, ke);
    const int ntiles = (ke - kb + BK - 1) / BK;

    if (ntiles > 0) {
      // The S^T chain starts from -L_i/scale and (without dropout) the dP^T
      // chain from -Delta_i: every C register of a lane is query row i.
      f32x16 nls, dpi;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        nls[r] = nl;
        dpi[r] = -del;
      }
      // kept in registers as they are, not rebuilt next to each use
      pin(nls);
      if constexpr (FOLD) pin(dpi);

      // K and V rows of tile tt (clamped to the last tile, so copies past the end
      // repeat it into stages that are never read) into a ring stage: copy u
      // (even: K, odd: V) of this wave fills rows (wave*NIW + u/2)*RPI + lane/NCH.
      // Rows past the end repeat the last key; they are never counted.
      struct Job {
        const __bf16* kp;  // first row of the tile in K and in V
        const __bf16* vp;
        uint32_t lds;      // LDS address of this wave's first K row in the stage
        uint32_t lim2;     // byte offset of the tile's last row (rows past it repeat it), at most 2*BK*kss
      };
      // Per-lane byte offsets of copy pair i's row (cp_off) and of its chunk alone
      // (cp_chk): a row r at most the last row lim is read at cp_off, else the last
      // row's chunk at lim2 + cp_chk, i.e. min(cp_off, lim2 + cp_chk).
      uint32_t cp_off[NIW], cp_chk[NIW];
#pragma unroll
      for (int i = 0; i < NIW; ++i) {
        const int r = (wave * NIW + i) * RPI + cp_row;
        cp_chk[i] = 16u * (uint32_t)pad_chunk(cp_pc ^ swz<D>(r), a.D / 8);
        cp_off[i] = 2u * (uint32_t)r * (uint32_t)a.kss + cp_chk[i];
      }
      // A job from a tile's first key and its element offset in K/V.
      auto job_at = [&](int kt, int64_t base, int stage) {
        const uint32_t lim = (uint32_t)min(a.Sk - 1 - kt, BK);
        return Job{K + base, V + base, lds_addr(&sT[stage][0][wave * NIW * RPI * D]), 2u * lim * (uint32_t)a.kss};
      };
      auto job_of = [&](int tt, int stage) {
        const int kt = kb + min(tt, ntiles - 1) * BK;
        return job_at(kt, (int64_t)b * a.ksb + (int64_t)kt * a.kss + (int64_t)kvh * a.ksh, stage);
      };
      // The copies' tile of the next step (it+3, held at the last tile), moved on
      // by one tile per step without multiplies.
      int ct_kt = kb + min(3, ntiles - 1) * BK;
      int64_t ct_base = (int64_t)b * a.ksb + (int64_t)ct_kt * a.kss + (int64_t)kvh * a.ksh;
      const int kt_last = kb + (ntiles - 1) * BK;
      const int64_t inc_kt = (int64_t)BK * a.kss;
      auto issue_job = [&](const Job& j, int u) {
        const uint32_t off = min(cp_off[u >> 1], j.lim2 + cp_chk[u >> 1]);
        const uint32_t lds = j.lds + 2u * (uint32_t)((u >> 1) * RPI * D + (u & 1) * TILE);
        dma16((u & 1) ? j.vp : j.kp, off, lds);
      };
      // Slot hook: copies u0 .. u0+PER-1 of job j, one every nslots/PER slots.
      auto copies_at = [&](const Job& j, int u0, int k, int nslots) {
        if (k % (nslots / PER) == 0) issue_job(j, u0 + k / (nslots / PER));
      };

      auto fence = []() { __builtin_amdgcn_sched_barrier(0); };
      // Row-major A operand of S/dP MFMA k (even: K chunk k/2 for S^T, odd: V chunk for dP^T).
      auto rd_op = [&](int m, int stq, int k) {
        return lds_read_b128(sT[stq][0] + rd_off[k >> 1] + (k & 1) * TILE + 32 * m * D);
      };
      // Transposed A operand half j of dQ MFMA n = j/2 = DB*t + d of half m: K^T
      // column block d over keys 32m + 16t .. +15; j even = first 8 keys, odd = last 8.
      auto rd_tr = [&](int m, int stq, int j) {
        const int n = j >> 1, t = n / DB, d = n % DB;
        return lds_read_tr(sT[stq][0] + (32 * m + 16 * t) * D + ((j & 1) ? tr_hi[d] : tr_lo[d]));
      };

      // Section "S/dP + exp/dS": S^T/dP^T of half ms from stage sts (operands of
      // its first PF MFMAs in pre), overlapped with the exp/dS of half me of key
      // tile kt (values se, dpe) and with the transposed reads of the first NP
      // MFMAs of that half's dQ (stage ste).
      auto sec_sdp_ew = [&](auto full_c, int ms, int sts, f32x16& s, f32x16& dp, const bf16x8 (&pre)[PF], int me,
                            int ste, int kt, const f32x16& se, const f32x16& dpe,
                            bf16x8 (&dsc)[2], bf16x4 (&trp)[2 * NP], auto&& slot_extra) {
        constexpr bool FULL = decltype(full_c)::value;
        bf16x8 op[8];
#pragma unroll
        for (int k = 0; k < PF; ++k) op[k] = pre[k];
        // Visible keys of this lane's row in the tile: d = j - i in (dlo, dhi), key
        // and row in range, i.e. tile keys [lo, hi).  Element r sits at key
        // 32*me + 4*h2 + c(r), c(r) = 8*(r/4) + r%4, so it is visible iff
        // c(r) - lb < span (unsigned) with lb = lo - 32*me - 4*h2.
        int lb = 0;
        uint32_t span = 0;
        if constexpr (!FULL) {
          // no overflow: |dl0| <= 2^29 + 128 and the bounds lie within +-(2^30 + 1)
          const int dl0 = kt - il;  // d = dl0 + key
          const int lo = max(vb.dlo - dl0 + 1, 0);
          const int hi = il < a.Sq ? min(vb.dhi - dl0, a.Sk - kt) : 0;
          span = (uint32_t)max(hi - lo, 0);
          lb = lo - 32 * me - 4 * h2;
        }
        // key part of the dropout draw of element r: (kt + 32*me + 4*h2 + c(r)) * 0x9E3779B9
        const uint32_t jb = DROP ? (uint32_t)(kt + 32 * me + 4 * h2) * 0x9E3779B9u : 0u;
        float pv[16], dv[16];
        float mk[16];  // mask values of the half (MASK), read ahead from sM
        // exp of element r (C-layout register r of half me); se holds
        // Q.K - L/scale, so scale*log2(e)*se is the exponent (S - L)*log2(e).
        auto ew_exp = [&](int r) {
          float x = se[r] * a.scale_log2;
          if constexpr (!FULL) {
            bool ok = elem_visible(r, lb, span);
            if constexpr (MASK) {
              const float mv = mk[r];
              ok = ok && !(mv <= kMaskedSentinel);
              x = __builtin_fmaf(mv, kLog2e, x);
            }
            x = ok ? x : -__builtin_inff();
          }
          pv[r] = __builtin_amdgcn_exp2f(x);
        };
        // dS of element r, one slot after its exp; odd r packs the pair.
        auto ew_ds = [&](int r) {
          if constexpr (DROP) {
            const uint32_t jg = jb + (uint32_t)(8 * (r >> 2) + (r & 3)) * 0x9E3779B9u;
            const float mm = fmix32(rk ^ jg) >= a.drop_thr ? a.drop_inv : 0.f;
            dv[r] = pv[r] * (dpe[r] * mm - del);
          } else {
            dv[r] = pv[r] * dpe[r];
          }
          if (r & 1) {
            const bf16x2 t = pack_here(dv[r - 1], dv[r]);
            dsc[r >> 3][(r & 7) - 1] = t[0];
            dsc[r >> 3][r & 7] = t[1];
          }
        };
        // Mask values of the half, read from this wave's LDS staging MF slots ahead
        // of their use, each once its copy (issued two sections earlier) landed.
        auto mask_rd = [&](int kk) {
          if constexpr (MVEC && !FULL) {
            // group g = kk / SG + 1 at the start of group g - 1's slots (kk < 0: group 0)
            const int g = kk < 0 ? 0 : kk / SG + 1;
            if ((kk < 0 || kk % SG == 0) && g < 4) {
              wait_vmcnt<kMaskWaitV>();
              const f32x4 v4 = *reinterpret_cast<const f32x4*>(&sM[wave][4 * g][4 * lane]);
#pragma unroll
              for (int e = 0; e < 4; ++e) mk[4 * g + e] = v4[e];
            }
          } else if constexpr (MASK && !FULL) {
            if (kk < NSD) {
              wait_vmcnt<kMaskWait>();
#pragma unroll
              for (int i = 0; i < 16 / NSD; ++i) mk[kk * (16 / NSD) + i] = sM[wave][kk * (16 / NSD) + i][lane];
            }
          }
        };
        if constexpr (MVEC) {
          mask_rd(-1);
        } else {
#pragma unroll
          for (int k = 0; k < MF; ++k) {
            if constexpr (MASK && !FULL) {
              wait_vmcnt<kMaskWait>();
#pragma unroll
              for (int i = 0; i < 16 / NSD; ++i) mk[k * (16 / NSD) + i] = sM[wave][k * (16 / NSD) + i][lane];
            }
          }
        }
        fence();
#pragma unroll
        for (int k = 0; k < NSD; ++k) {
          const bf16x8& o = op[k & 7];
          if (k & 1) {
            if (k == 1 && FOLD)
              mfma_v_seed(dp, o, gr[k >> 1], dpi);
            else if (k == 1)
              mfma_v0(dp, o, gr[k >> 1]);
            else
              mfma_v(dp, o, gr[k >> 1]);
          } else {
            if (k == 0)
              mfma_v_seed(s, o, qr[k >> 1], nls);
            else
              mfma_v(s, o, qr[k >> 1]);
          }
          if (k + PF < NSD) op[(k + PF) & 7] = rd_op(ms, sts, k + PF);
          if (k >= NSD - 2 * NP) trp[k - (NSD - 2 * NP)] = rd_tr(me, ste, k - (NSD - 2 * NP));
          // 16 exp/dS elements over the NSD slots: the exps of this slot's elements
          // and the dS of the previous slot's (no result is read right after its exp)
          constexpr int E = 16 / NSD;
#pragma unroll
          for (int i = 0; i < E; ++i) ew_exp(k * E + i);
          if (k > 0) {
#pragma unroll
            for (int i = 0; i < E; ++i) ew_ds((k - 1) * E + i);
          }
          mask_rd(MVEC ? k : k + MF);
          slot_extra(k);
          fence();
        }
#pragma unroll
        for (int i = 0; i < 16 / NSD; ++i) ew_ds(16 - 16 / NSD + i);
        // dS^T is complete here; S/dP are next read a whole section later (the
        // prologue drains them explicitly).
        materialise(dsc);
        mfma_settle(s, dp);
        fence();
      };
      // Section "dQ" of half m (stage stq): MFMAs 0 .. NP-1 take the transposed
      // operands read by the previous section; slot n reads those of MFMA n + NP.
      auto sec_dq = [&](int m, int stq, const bf16x4 (&trp)[2 * NP], const bf16x8 (&dsc)[2], auto&& slot_extra) {
        constexpr int W = NP + 1;  // operand pairs in flight
        bf16x4 buf[2 * W];
#pragma unroll
        for (int n = 0; n < NP; ++n) {
          buf[2 * n] = trp[2 * n];
          buf[2 * n + 1] = trp[2 * n + 1];
        }
#pragma unroll
        for (int n = 0; n < NDQ; ++n) {
          const int sl = n % W;
          mfma_acc(accq[n % DB], concat(buf[2 * sl], buf[2 * sl + 1]), dsc[n / DB]);
          if (n + NP < NDQ) {
            const int sn = (n + NP) % W;
            buf[2 * sn] = rd_tr(m, stq, 2 * (n + NP));
            buf[2 * sn + 1] = rd_tr(m, stq, 2 * (n + NP) + 1);
          }
          slot_extra(n);
          fence();
        }
      };

      // Mask staging: element r of half `half` of key tile tt into sM[wave][r].
      // unused (and dropped) without a mask
      const rsrc_t mrs = raw_rsrc(a.mask + (int64_t)b * a.msb + (int64_t)h * a.msh, a.mask_rec);
      auto mask_vb = [&](int tt, int half) {
        return m_lvo + (uint32_t)(kb + min(tt, ntiles - 1) * BK + 32 * half) * msk4;
      };
      auto mask_cp = [&](uint32_t vb0, int r) {
        dma_buf4(mrs, mad24(8 * (r >> 2) + (r & 3), msk4, vb0), lds_addr(&sM[wave][r][0]));
      };
      // MVEC: keys 8g + 4*h2 .. +3 of the lane's row, to sM[wave][4g .. 4g+3] (16 bytes per lane)
      auto mask_cpv = [&](uint32_t vb0, int g) { dma_buf16(mrs, vb0 + 32u * g, lds_addr(&sM[wave][4 * g][0])); };
      // Slot hook of sections A and C: the copies that refill the elements (MVEC:
      // the groups) whose last use was slot k.
      auto mask_refill = [&](uint32_t vb0, int k) {
        if constexpr (MVEC) {
          if (k % SG == SG - 1) mask_cpv(vb0, k / SG);
        } else if constexpr (MASK) {
#pragma unroll
          for (int i = 0; i < 16 / NSD; ++i) mask_cp(vb0, k * (16 / NSD) + i);
        }
      };
      if constexpr (MASK) {
        const uint32_t v0 = mask_vb(0, 0);
#pragma unroll
        for (int k = 0; k < NSD; ++k) mask_refill(v0, k);
      }

      // Prologue: K/V of tiles 0 and 1 and three quarters of tile 2's copies; all
      // landed.  A tile's copies go out over four sections from the barrier on
      // (a quarter each in B, C and D of one step and in A of the next).
#pragma unroll
      for (int u = 0; u < NC; ++u) issue_job(job_of(0, 0), u);
#pragma unroll
      for (int u = 0; u < NC; ++u) issue_job(job_of(1, 1), u);
      Job pend = job_of(2, 2);
#pragma unroll
      for (int u = 0; u < NC - PER; ++u) issue_job(pend, u);
      wait_vmcnt<0>();
      barrier_lds();

      // S/dP of half 0 of the current tile, carried between steps, and the
      // prefetched operands of the next S/dP section.
      f32x16 s0, dp0;
      bf16x8 pre[PF];
      {
        bf16x8 ds[2];
        bf16x4 trp[2 * NP];
        f32x16 z{};
#pragma unroll
        for (int k = 0; k < PF; ++k) pre[k] = rd_op(0, 0, k);
        // a section with no exp/dS work to overlap: only its S/dP result is kept
        sec_sdp_ew(std::true_type{}, 0, 0, s0, dp0, pre, 0, 0, kb, z, z, ds, trp, [](int) {});
        mfma_drain(s0, dp0);  // read by the first step's exp/dS after only a few instructions
#pragma unroll
        for (int k = 0; k < PF; ++k) pre[k] = rd_op(1, 0, k);
      }

      int it = 0;
      // One step (see the header comment).  KIND 1 = boundary tile (per-element
      // predicate), 2 = interior tile (every element counted); each kind runs in a
      // loop of its own, so no loop body branches.
      auto step = [&](auto kind_c) {
        constexpr bool FULL = decltype(kind_c)::value == 2;
        const std::integral_constant<bool, FULL> full_c;
        const int stq = it & (NST - 1);
        const int stq1 = (it + 1) & (NST - 1);
        const int stq3 = (it + 3) & (NST - 1);
        const int kt = kb + it * BK;
        bf16x8 ds[2];
        bf16x4 trp[2 * NP];
        f32x16 s1, dp1;
        // Prefetch read p of the next S/dP section goes into slot n = NDQ - PF + p.
        auto pre_at = [&](int n, int ms) {
          if (n >= NDQ - PF) pre[n - (NDQ - PF)] = rd_op(ms, stq1, n - (NDQ - PF));
        };
        // A: S/dP of half 1 with exp/dS of half 0; the last quarter of tile it+2's copies.
        // Each slot then stages the mask of half 1 of this tile in place of the
        // half-0 elements it used.
        const uint32_t mvb_a = MASK ? mask_vb(it, 1) : 0u;
        sec_sdp_ew(full_c, 1, stq, s1, dp1, pre, 0, stq, kt, s0, dp0, ds, trp, [&](int k) {
          copies_at(pend, NC - PER, k, NSD);
          mask_refill(mvb_a, k);
        });
        // tile it+1 landed everywhere once all waves pass the barrier (with a mask,
        // the mask copies of a step count too, and those of section A issued after
        // its last tile copy)
        wait_vmcnt<NC + (MASK ? kMaskPerStep + kMaskLateA : 0)>();
        barrier_only();
        const Job next = job_at(ct_kt, ct_base, stq3);
        if (ct_kt < kt_last) {
          ct_kt += BK;
          ct_base += inc_kt;
        }
        // B: dQ of half 0; prefetch for C
        sec_dq(0, stq, trp, ds, [&](int n) {
          copies_at(next, 0, n, NDQ);
          pre_at(n, 0);
        });
        // C: S/dP of half 0 of tile it+1 with exp/dS of half 1; each slot then
        // stages the mask of half 0 of tile it+1 in place of the elements it used
        const uint32_t mvb_c = MASK ? mask_vb(it + 1, 0) : 0u;
        sec_sdp_ew(full_c, 0, stq1, s0, dp0, pre, 1, stq, kt, s1, dp1, ds, trp, [&](int k) {
          copies_at(next, PER, k, NSD);
          mask_refill(mvb_c, k);
        });
        // D: dQ of half 1; prefetch for A of the next step
        sec_dq(1, stq, trp, ds, [&](int n) {
          copies_at(next, 2 * PER, n, NDQ);
          pre_at(n, 1);
        });
        pend = next;
        ++it;
      };

      // This wave's key tiles: [0,f0) boundary, [f0,f1) interior, [f1,ntiles)
      // boundary.  Boundary tiles include tiles this wave cannot see at all; the
      // predicate zeroes them.
      auto all = [&](int t) { return rect_all_visible(a, qw0, qw0 + kDqRowsPerWave - 1, kb + t * BK, kb + t * BK + BK - 1); };
      int f0 = ntiles, f1 = ntiles;
      if constexpr (!MASK) {
        f0 = 0;
        while (f0 < ntiles && !all(f0)) ++f0;
        f1 = f0;
        while (f1 < ntiles && all(f1)) ++f1;
      }
      const std::integral_constant<int, 1> kEdge;
      const std::integral_constant<int, 2> kInner;
      int t = 0;
      for (; t < f0; ++t) step(kEdge);
      for (; t < f1; ++t) step(kInner);
      for (; t < ntiles; ++t) step(kEdge);
      wait_vmcnt<0>();  // the repeated copies of the last steps have landed
      barrier_lds();    // every wave is done with the ring before the next pass refills it
    }
    mfma_drain_acc(accq);  // the accumulators' last MFMAs have finished before they are read

    if (il < a.Sq) {
#pragma unroll
      for (int d = 0; d < DB; ++d) {
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int dd = 32 * d + 8 * r4 + 4 * h2;
          if (dd >= a.D) continue;  // past the head dimension
          bf16x4 o4;
#pragma unroll
          for (int e = 0; e < 4; ++e) o4[e] = (__bf16)(accq[d][4 * r4 + e] * a.scale);
          *reinterpret_cast<bf16x4*>(dQ + qoff + dd) = o4;
        }
      }
    }
  }
}

template <int D, int MK, bool DROP>
static hipError_t launch_t(const PrefillArgs& a, const void* Q, const void* K, const void* V, const void* dO,
                           const float* L, const float* delta, void* dQ, hipStream_t st) {
  const int nqb = (a.Sq + kDqRowsPerBlock - 1) / kDqRowsPerBlock;
  const int paired = (a.causal && a.window == 0 && nqb > 1) ? 1 : 0;
  const int nwi = paired ? (nqb + 1) / 2 : nqb;
  const unsigned grid = (unsigned)(nwi * a.B * a.Hq);
  hipLaunchKernelGGL((dq_bf16_kernel<D, MK, DROP>), dim3(grid), dim3(256), 0, st, a,
                     static_cast<const __bf16*>(Q), static_cast<const __bf16*>(K), static_cast<const __bf16*>(V),
                     static_cast<const __bf16*>(dO), L, delta, static_cast<__bf16*>(dQ), nqb, paired);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_d(const PrefillArgs& a, const void* Q, const void* K, const void* V, const void* dO,
                           const float* L, const float* delta, void* dQ, hipStream_t st) {
  const bool drop = a.drop != 0;
  const int mk = a.mask == nullptr ? 0 : (mask_keys_contiguous(a) ? 2 : 1);
  if (mk == 2) return drop ? launch_t<D, 2, true>(a, Q, K, V, dO, L, delta, dQ, st)
                           : launch_t<D, 2, false>(a, Q, K, V, dO, L, delta, dQ, st);
  if (mk == 1) return drop ? launch_t<D, 1, true>(a, Q, K, V, dO, L, delta, dQ, st)
                           : launch_t<D, 1, false>(a, Q, K, V, dO, L, delta, dQ, st);
  return drop ? launch_t<D, 0, true>(a, Q, K, V, dO, L, delta, dQ, st)
              : launch_t<D, 0, false>(a, Q, K, V, dO, L, delta, dQ, st);
}

hipError_t launch_dq_bf16(const PrefillArgs& a, int D, const void* Q, const void* K, const void* V,
                          const void* dO, const float* L, const float* delta, void* dQ, hipStream_t st) {
  // Head dimension above 64 (tiles 128 wide) without window, mask or dropout:
  // two row blocks per wave (a window leaves its 256-row blocks more invisible
  // key tiles than it saves).
  if (D > 64 && a.window == 0 && a.mask == nullptr && a.drop == 0)
    return launch_dq2_bf16(a, Q, K, V, dO, L, delta, dQ, st);
  return D <= 64 ? launch_d<64>(a, Q, K, V, dO, L, delta, dQ, st) : launch_d<128>(a, Q, K, V, dO, L, delta, dQ, st);
}

}  // namespace fa
