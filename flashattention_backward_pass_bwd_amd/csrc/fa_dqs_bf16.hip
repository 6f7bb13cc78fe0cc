// dQ pass over stored dS, bf16 storage, bf16 MFMA with fp32 accumulation
// (ferrotensor-backend flash_attention_v2_backward.wgsl, flash_bwd_dq: the
// dQ sum over keys; here dS is not recomputed but read from the workspace the
// dK/dV pass filled in its workspace mode):
//   dQ_i = scale * sum_j dS_ij K_j.
//
// Block: (b, KV head, 64-row query tile, up to four query heads of the
// group); wave w takes query head 4c + w of the group and accumulates dQ^T
// (D x 64 fp32, two 32-row blocks) in accumulation registers.  The block
// walks the key blocks whose workspace tile holds its query tile, 64 keys per
// step: a 3-stage LDS ring holds the step's K rows (shared by the waves,
// swizzled, see fa_tiles.h) and each wave's dS (two row halves x 64 keys x 32
// rows, as stored), both filled by direct global->LDS copies two steps ahead.
// Per step and wave: dQ^T += K^T dS^T, both operands read with
// ds_read_b64_tr_b16 (K^T from the row-major K rows, dS^T from the key-major
// dS), 4*D/16 MFMAs.  Reading the stored dS once from HBM bounds it.
#include "fa_internal.h"
#include "fa_tiles.h"

namespace fa {

// BK keys per step (64: half a workspace tile, one block per CU; 32: a
// quarter, and a ring small enough for two blocks per CU, each hiding the
// other's barrier waits).
template <int D, int BK>
__global__ __launch_bounds__(256, BK == 32 ? 2 : 1) void dqs_bf16_kernel(PrefillArgs a, const __bf16* __restrict__ K,
                                                          const unsigned char* __restrict__ ws,
                                                          __bf16* __restrict__ dQ, int nqt, int nchunk, int nkb) {
  constexpr int NCH = D / 8;           // 16-byte chunks per K row
  constexpr int DB = D / 32;           // 32-row blocks of dQ^T
  constexpr int NST = 3;               // ring stages
  constexpr int RPI = 1024 / (2 * D);  // K rows per 1 KB copy
  constexpr int NKC = BK / RPI / 4;    // K copies per wave per step
  constexpr int NG = BK / 32;          // 32-key groups per step
  constexpr int NDC = 4 * NG;          // dS copies per wave per step (2 row halves x NG x 2 KB)
  constexpr int NC = NKC + NDC;
  constexpr int KT = BK * D;           // K elements of a stage
  constexpr int SH = BK * 32;          // dS elements of a row half of a wave's step
  constexpr int JS = kWsKeys / BK;     // steps per workspace tile
  static_assert(NKC >= 1 && (BK == 32 || BK == 64), "step width");
  // A row half of a step is 2*NG 1 KB blocks (32-key group w', 16-row group t),
  // each copied as it is; in LDS the blocks sit 1152 bytes apart, so the two
  // row groups' blocks fall into different halves of the 64 banks.
  constexpr int SBLK = 576;            // elements from one block to the next in LDS
  constexpr int SHP = 2 * NG * SBLK;   // LDS elements of a row half of a wave's stage
  static_assert(kWsRows == 64 && kWsKeys == JS * BK && kWsTileBytes == JS * 2 * SH * 2,
                "a workspace tile is JS steps of two row halves");
  constexpr int NSLOT = (BK / 16) * DB * 2;  // MFMAs per step and wave
  constexpr int CSP = 2 * NC <= NSLOT ? 2 : 1;  // MFMA slots per copy
  static_assert(NC * CSP <= NSLOT, "a step's copies fit its MFMA slots");

  __shared__ __attribute__((aligned(16))) __bf16 sK[NST][KT];
  __shared__ __attribute__((aligned(16))) __bf16 sS[NST][4][2][SHP];

  const int nbh = a.B * a.Hkv;
  const int bh = blockIdx.x % nbh;  // consecutive blocks cycle over (b, kvh): a KV head's blocks share an XCD
  const int rest = blockIdx.x / nbh;
  const int chunk = rest % nchunk;
  const int qtile = nqt - 1 - rest / nchunk;  // the longest causal rows first
  const int b = bh / a.Hkv;
  const int kvh = bh % a.Hkv;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int h2 = lane >> 5;
  const int l32 = lane & 31;
  const int gq = 4 * chunk + wave;
  const bool active = gq < a.group;  // spare waves repeat the group's last head and store nothing
  const int h = kvh * a.group + min(gq, a.group - 1);

  // Key blocks whose workspace tile holds this query tile: an interval
  // [kb0, kb1] (a key block's first and last visible rows never decrease with
  // it), and the workspace index of the first one's tile.
  // Found 64 key blocks at a time, one per lane: kb0 and kb1 are the first and
  // last lanes whose run holds the tile, tp0 the sum of the runs before kb0 (a
  // run has at most 2^23 tiles, so 64 of them sum exactly in 32 bits).
  int kb0 = -1, kb1 = -2, ql0 = 0, n0 = 0;
  int64_t tp0 = 0;
  for (int c0 = 0; c0 < nkb; c0 += 64) {
    const int k = c0 + lane;
    int ql, n;
    ws_run(a, k, ql, n);
    const bool in_range = k < nkb;
    const uint64_t holds = __ballot(in_range && qtile >= ql && qtile < ql + n);
    if (holds != 0) {
      const int f = __ffsll((unsigned long long)holds) - 1;
      if (kb0 < 0) {
        kb0 = c0 + f;
        ql0 = __builtin_amdgcn_readfirstlane(__shfl(ql, f));
        n0 = __builtin_amdgcn_readfirstlane(__shfl(n, f));
        tp0 += __builtin_amdgcn_readfirstlane(wave_sum_i32(lane < f ? n : 0));
      }
      kb1 = c0 + 63 - __clzll((unsigned long long)holds);
    } else if (kb0 < 0) {
      tp0 += __builtin_amdgcn_readfirstlane(wave_sum_i32(in_range ? n : 0));
    }
  }
  const int nsteps = kb0 >= 0 ? JS * (kb1 - kb0 + 1) : 0;

  // Copy cursor: the step whose copies go out next (held at the last step, so
  // the copies past the end repeat it into stages that are never read).
  struct Cur {
    int kb, j, ql, n, s;
    int64_t tp;
  };
  Cur cc{kb0, 0, ql0, n0, 0, tp0};
  auto advance = [&](Cur& c) {
    if (c.s + 1 >= nsteps) return;
    ++c.s;
    if (c.j + 1 < JS) {
      ++c.j;
    } else {
      c.tp += c.n;
      ++c.kb;
      c.j = 0;
      ws_run(a, c.kb, c.ql, c.n);
    }
  };

  // K copies: copy u of this wave fills rows (wave*NKC + u)*RPI + lane/NCH of
  // the stage, lane l landing in physical chunk l%NCH, so it fetches the
  // logical chunk stored there; rows past the last key repeat it (their dS
  // is zero).
  const int cp_row = lane / NCH;
  const int cp_pc = lane % NCH;
  uint32_t cp_off[NKC], cp_chk[NKC];
#pragma unroll
  for (int u = 0; u < NKC; ++u) {
    const int r = (wave * NKC + u) * RPI + cp_row;
    cp_chk[u] = 16u * (uint32_t)pad_chunk(cp_pc ^ swz<D>(r), a.D / 8);
    cp_off[u] = 2u * (uint32_t)r * (uint32_t)a.kss + cp_chk[u];
  }
  struct Job {
    const __bf16* kp;         // K row of the step's first key (clamped to the last key)
    uint32_t lim2;            // byte offset of the last row to read (rows past it repeat it)
    const unsigned char* sp;  // this wave's stored dS of the step (row half 0)
    int stage;
  };
  const int64_t ws_head = (int64_t)(b * a.Hq + h) * a.ws_tiles;
  auto job_of = [&](const Cur& c, int stage) {
    const int kt = min(c.kb * kWsKeys + c.j * BK, a.Sk - 1);
    const uint32_t lim = (uint32_t)min(a.Sk - 1 - kt, BK);
    const int64_t tile = ws_head + c.tp + (qtile - c.ql);
    return Job{K + (int64_t)b * a.ksb + (int64_t)kt * a.kss + (int64_t)kvh * a.ksh, 2u * lim * (uint32_t)a.kss,
               ws + tile * kWsTileBytes + c.j * (BK * 64), stage};
  };
  // Copy i of a job (0 .. NC-1): first the K rows, then the dS (row half
  // i'/(2*NG), 1 KB part i'%(2*NG)).
  auto issue = [&](const Job& jb, int i) {
    if (i < NKC) {
      const uint32_t off = min(cp_off[i], jb.lim2 + cp_chk[i]);
      dma16(jb.kp, off, lds_addr(&sK[jb.stage][(wave * NKC + i) * RPI * D]));
    } else {
      const int c = i - NKC, m = c / (2 * NG), part = c % (2 * NG);
      dma16_nt(jb.sp + m * 8192 + part * 1024, 16u * (uint32_t)lane,
               lds_addr(&sS[jb.stage][wave][m][part * SBLK]));
    }
  };

  // Transposed reads.  K^T (A operand of d-block d, keys 16ks .. +15): as in
  // the other tile kernels.  dS^T (B operand of row half m): a 16-lane group
  // reads a 4-key x 16-row block, lane l receiving row position l%32 of keys
  // 4*(l/32) + 0..3 (+8 for the second half of the operand), the same key
  // order as the K^T reads; each lane addresses its 4 rows (8 bytes) of one
  // key: block (w', t) = (key/32, position/16), then key%32 (32 bytes), the
  // 8-row half (16 bytes) and the 4-row quad (8 bytes).
  int tr_lo[DB], tr_hi[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d) {
    tr_lo[d] = tr_lane_off<D>(lane, d, 0);
    tr_hi[d] = tr_lane_off<D>(lane, d, 8);
  }
  const int g16 = lane >> 4, s16 = lane & 15;
  const int trs = (g16 & 1) * SBLK + (4 * (g16 >> 1) + (s16 >> 2)) * 16 + ((s16 & 3) >> 1) * 8 + (s16 & 1) * 4;

  struct Ops {
    bf16x8 ka[DB], sb[2];
  };
  auto read_ops = [&](Ops& o, int st, int ks) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const __bf16* p = &sS[st][wave][m][(ks >> 1) * 2 * SBLK + 16 * (ks & 1) * 16 + trs];
      o.sb[m] = concat(lds_read_tr(p), lds_read_tr(p + 8 * 16));
    }
#pragma unroll
    for (int d = 0; d < DB; ++d) {
      const __bf16* p = &sK[st][16 * ks * D];
      o.ka[d] = concat(lds_read_tr(p + tr_lo[d]), lds_read_tr(p + tr_hi[d]));
    }
  };

  f32x16 acc[2 * DB];  // dQ^T block d of row half m at acc[2d + m]
#pragma unroll
  for (int i = 0; i < 2 * DB; ++i) acc[i] = f32x16{};

  if (nsteps > 0) {  // (a query tile no key block sees gets zero rows)
  // Prologue: the copies of steps 0 and 1.
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const Job jb = job_of(cc, s);
#pragma unroll
    for (int i = 0; i < NC; ++i) issue(jb, i);
    advance(cc);
  }
  for (int s = 0; s < nsteps; ++s) {
    const int st = s % NST;
    wait_vmcnt<NC>();  // this wave's copies of step s landed (step s+1's are in flight) ...
    barrier_lds();     // ... and every wave's; every wave is done with stage (s+2)%3
    const Job jb = job_of(cc, (s + 2) % NST);
    advance(cc);
    Ops cur, nxt;
    read_ops(cur, st, 0);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      if (ks + 1 < BK / 16) read_ops(nxt, st, ks + 1);
#pragma unroll
      for (int d = 0; d < DB; ++d) {
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          mfma_acc(acc[2 * d + m], cur.ka[d], cur.sb[m]);
          const int slot = (ks * DB + d) * 2 + m;
          if (slot % CSP == 0 && slot / CSP < NC) issue(jb, slot / CSP);
        }
      }
      if (ks + 1 < BK / 16) cur = nxt;
    }
  }
  wait_vmcnt<0>();  // the repeated copies of the last steps have landed
  }
  mfma_drain_acc(acc);

  // dQ of the wave's rows leaves through LDS, one 32-row half at a time, so
  // that each store writes 16 bytes of a row and D/8 lanes a whole row: lane
  // (l32, h2) puts its 4-element pieces of its row into a per-wave [32][D + 8]
  // bf16 block of the dS ring (free once every wave has passed the barrier
  // below), then lane l reads chunk l % (D/8) of rows RPS*i + l / (D/8) and
  // stores it.
  constexpr int SR = D + 8;
  constexpr int CPR = D / 8;     // 16-byte chunks per row
  constexpr int RPS = 64 / CPR;  // rows per read and store
  static_assert(4 * 32 * SR <= (int)(sizeof(sS) / sizeof(__bf16)), "the staging blocks fit the dS ring");
  barrier_lds();
  __bf16* const stg = &sS[0][0][0][0] + wave * 32 * SR;
  const int c = lane % CPR;
  __bf16* const base = dQ + (int64_t)b * a.qsb + (int64_t)h * a.qsh + 8 * c;
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    // Column l%32 of row half m holds the row the dK/dV pass's lane stored
    // there: quads 1 and 2 of each 16 rows swapped.
    const int p = l32;
    const int rl = (p & 0x13) | ((p & 4) << 1) | ((p & 8) >> 1);
#pragma unroll
    for (int d = 0; d < DB; ++d) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        bf16x4 o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = (__bf16)(acc[2 * d + m][4 * r4 + e] * a.scale);
        *reinterpret_cast<bf16x4*>(stg + rl * SR + 32 * d + 8 * r4 + 4 * h2) = o4;
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's writes land before its reads
    bf16x8 v[32 / RPS];
#pragma unroll
    for (int i = 0; i < 32 / RPS; ++i) v[i] = *reinterpret_cast<const bf16x8*>(stg + (RPS * i + lane / CPR) * SR + 8 * c);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // and its reads before the next half's writes
    if (active) {
#pragma unroll
      for (int i = 0; i < 32 / RPS; ++i) {
        const int row = kWsRows * qtile + 32 * m + RPS * i + lane / CPR;
        if (row < a.Sq && 8 * c < a.D) *reinterpret_cast<bf16x8*>(base + (int64_t)row * a.qss) = v[i];
      }
    }
  }
}

#ifndef FA_DQS_BK
#define FA_DQS_BK 32
#endif
template <int D>
static hipError_t launch_t(const PrefillArgs& a, const void* K, const void* ws, void* dQ, hipStream_t st) {
  const int nqt = (a.Sq + kWsRows - 1) / kWsRows;
  const int nchunk = (a.group + 3) / 4;
  const int nkb = (a.Sk + kWsKeys - 1) / kWsKeys;
  const unsigned grid = (unsigned)(nqt * nchunk * a.B * a.Hkv);
  hipLaunchKernelGGL((dqs_bf16_kernel<D, FA_DQS_BK>), dim3(grid), dim3(256), 0, st, a, static_cast<const __bf16*>(K),
                     static_cast<const unsigned char*>(ws), static_cast<__bf16*>(dQ), nqt, nchunk, nkb);
  return hipGetLastError();
}

hipError_t launch_dqs_bf16(const PrefillArgs& a, int D, const void* K, const void* ws, void* dQ, hipStream_t st) {
  return D <= 64 ? launch_t<64>(a, K, ws, dQ, st) : launch_t<128>(a, K, ws, dQ, st);
}

}  // namespace fa
