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
// 64-row query tile) pair.  Per tile and wave: S = Q K^T and dP = dO V^T
// (row-major A operands from LDS), P and dS in registers, then dV^T += dO^T (P.M)
// and dK^T += Q^T dS (transposed A operands through ds_read_b64_tr_b16).  The
// C layout of S (one key per lane column) is the B layout of the second pair
// of contractions, so P and dS never leave registers.
//
// Software pipeline.  A tile is two 32-row halves; the step of tile it runs
//   A: S/dP of half 1 (MFMA)      with  exp/dS of half 0 (VALU)
//      -- wait for tile it+1's copies, block barrier --
//   B: copies of tile it+3 (and L/Delta of tile it+4) issued; dV/dK of half 0
//   C: S/dP of half 0 of tile it+1 with exp/dS of half 1
//   D: dV/dK of half 1
// so the exp/dS arithmetic of one half always overlaps the MFMAs of another
// (its last two elements finish in the first slots of the dV/dK section that
// follows, whose MFMAs leave issue slots free), and the next tile's first
// MFMAs follow the current tile's last without a barrier in between.  Q and dO tiles live in a 4-stage LDS ring (swizzled,
// see fa_tiles.h) filled by direct global->LDS copies three tiles ahead; one
// barrier per tile separates the last reads of a stage from its refill.  L and
// Delta (64 floats per tile) travel through an 8-stage ring four tiles ahead;
// two tiles before use, wave 0 turns L into -L/scale and wave 1 turns Delta
// into -Delta in place.  The S chain starts from the rows' -L/scale, so its
// fp32 result times scale*log2(e) is the exponent and P is one multiply and an
// exp2 (K enters the MFMAs as it is stored: no rounding of a scaled copy); without
// dropout the dP chain starts from -Delta and yields dP - Delta directly.  For
// causal attention without a window, block i also takes key block nkb-1-i, so
// every block carries the same work; it walks that second key block's tiles
// upwards, which keeps the blocks of a KV head on the same tile (see the walk
// order below).  At the end dK and dV leave through LDS as whole-row stores.
//
// Workspace mode (WS): the pass also stores every tile's dS, as the bf16 values
// its dK contraction used, into the dS workspace (layout in fa_common.h) for
// the dQ pass over stored dS.  Query tiles then start on a multiple of 64
// rows (the rows added below the first visible one are invisible), and each
// dV/dK section stores the dS of its half with two 16-byte stores per lane.
#include <type_traits>

#include "fa_internal.h"
#include "fa_tiles.h"

namespace fa {

// Vector-memory operations of slot j of an S/dP + exp/dS section of the dK/dV
// kernel below (E = 16/NSD elements per slot): the slot's tile copy (one every
// NSD/PER slots, from slot 0), then its mask copies (MVEC: one per 4-element
// group, in the slot of the group's last element; otherwise one per element).
template <int NSD, int PER, bool MVEC>
constexpr int sdp_slot_vmem(int j) {
  constexpr int E = 16 / NSD, SG = 4 / E;
  return (j % (NSD / PER) == 0 ? 1 : 0) + (MVEC ? (j % SG == SG - 1 ? 1 : 0) : E);
}

// Vector-memory operations a wave issues after the copy that stages mask
// element r and before r is read, for the reads made ahead of slot kk - MF
// (elements kk*E .. kk*E + E-1; the least of their counts): the copies after
// it in the copying section, the DKV operations of the dV/dK section in
// between, and those of the reading section's earlier slots.  vmcnt drops in
// issue order, so waiting until at most that many are in flight means r landed.
template <int NSD, int PER, bool MVEC, int MF, int DKV>
constexpr int mask_read_wait(int kk) {
  constexpr int E = 16 / NSD, SG = 4 / E;
  int least = 63;
  for (int i = 0; i < E; ++i) {
    const int r = kk * E + i;
    const int cs = MVEC ? SG * (r / 4) + SG - 1 : r / E;  // slot of r's copy
    int n = MVEC ? 0 : E - 1 - r % E;                     // copies of that slot after it
    for (int j = cs + 1; j < NSD; ++j) n += sdp_slot_vmem<NSD, PER, MVEC>(j);
    n += DKV;
    for (int j = 0; j < kk - MF; ++j) n += sdp_slot_vmem<NSD, PER, MVEC>(j);
    least = n < least ? n : least;
  }
  return least;
}

// MK: 0 no mask, 1 a mask of any strides, 2 a mask whose keys are contiguous and
// whose 4-key groups are 16-byte aligned (staged with one 16-byte copy per lane
// for 8 rows of the wave's 32 keys).
template <int D, int MK, bool DROP, bool WS>
__global__ __launch_bounds__(256, 1) void dkdv_bf16_kernel(PrefillArgs a, const __bf16* __restrict__ Q,
                                                           const __bf16* __restrict__ K,
                                                           const __bf16* __restrict__ V,
                                                           const __bf16* __restrict__ dO,
                                                           const float* __restrict__ L,
                                                           const float* __restrict__ Dl,
                                                           __bf16* __restrict__ dK, __bf16* __restrict__ dV,
                                                           unsigned char* __restrict__ ws, int nkb, int paired) {
  constexpr bool MASK = MK != 0;
  constexpr bool MVEC = MK == 2;
  constexpr int BQ = 64;
  constexpr int NCH = D / 8;                // 16-byte chunks per row
  constexpr int KS = D / 16;                // k-blocks of the head_dim contraction
  constexpr int DB = D / 32;                // 32-row blocks of dK^T / dV^T
  constexpr int NST = 4;                    // Q/dO ring stages
  constexpr int NSL = 8;                    // L/Delta/row-key ring stages
  constexpr int RPI = 1024 / (2 * D);       // tile rows per 1 KB global->LDS copy (64 lanes x 16 B)
  constexpr int NIW = BQ / RPI / 4;         // copies per wave per tile per tensor
  constexpr int TILE = BQ * D;
  constexpr bool FOLD = !DROP;              // dP chain seeded with -Delta
  constexpr int NSD = 2 * KS;               // S/dP MFMAs per 32-row half
  constexpr int NDK = 4 * DB;               // dV/dK MFMAs per 32-row half
#ifndef FA_DKDV_NP
#define FA_DKDV_NP 3
#endif
  constexpr int NP = 2 * FA_DKDV_NP <= NSD ? FA_DKDV_NP : NSD / 2;  // dV/dK MFMAs whose operands the preceding section reads
  static_assert(NSD == NDK, "the S/dP section carries one transposed read per MFMA");
  static_assert(2 * NP <= NSD, "the transposed reads of NP MFMAs fit the S/dP section's slots");
  static_assert(NSD % (NIW / 2) == 0, "a section carries a quarter of a tile's copies evenly");

  // Ring stage s holds the Q tile (sT[s][0]) and the dO tile (sT[s][1]) side by
  // side, so one per-lane address per stage serves both through immediate offsets.
  __shared__ __attribute__((aligned(16))) __bf16 sT[NST][2][TILE];
  __shared__ __attribute__((aligned(16))) float sL[NSL][BQ];
  __shared__ __attribute__((aligned(16))) float sDel[NSL][BQ];
  __shared__ __attribute__((aligned(16))) uint32_t sRK[DROP ? NSL : 1][DROP ? BQ : 1];
  // Mask values of one exp/dS half per wave: element r of lane l at sM[wave][r][l].
  __shared__ __attribute__((aligned(16))) float sM[MASK ? 4 : 1][MASK ? 16 : 1][64];
  // Landing place of the per-step writes that a wave or lane has no row for (so
  // that every wave runs the same code without branches); never read.
  __shared__ __attribute__((aligned(16))) float sDum[2][64];

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

    // K and V rows of this wave's keys in accumulation registers (keys past the
    // end repeat the last key; no element of theirs is counted).
    bf16x8 kr[KS], vr[KS];
    const int64_t kclamp = (int64_t)b * a.ksb + (int64_t)min(jl, a.Sk - 1) * a.kss + (int64_t)kvh * a.ksh;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      kr[s] = ld16_op(row_chunk(K + kclamp, 2 * s + h2, a.D / 8));  // zero past the head dimension
      vr[s] = ld16_op(row_chunk(V + kclamp, 2 * s + h2, a.D / 8));
    }
    f32x16 acck[DB], accv[DB];
#pragma unroll
    for (int d = 0; d < DB; ++d) {
      acck[d] = f32x16{};
      accv[d] = f32x16{};
    }

    // Mask reads: byte offset of element (row, key) in the (b, h) slice is
    // row*msq*4 + key*msk*4; lanes fix the key (clamped) and the 4-row group.
    const uint32_t msq4 = MASK ? (uint32_t)a.msq * 4u : 0u;
    const uint32_t m_lvo = MASK ? ((uint32_t)min(jl, a.Sk - 1) * (uint32_t)a.msk + 4u * h2 * (uint32_t)a.msq) * 4u : 0u;
    // MVEC: copy lane j fetches keys kw0 + 4*(j%8) .. +3 of row e + 4h (e = j/16,
    // h = (j/8)%2) of an 8-row group; they land at byte 256e + 128h + 16*(j%8) of
    // the group, so the reader lane (key k, half h2) finds element e at
    // 256e + 128*h2 + 4k: one row per 32 banks, no conflicts.
    const uint32_t m_lvv = MVEC ? (((uint32_t)(lane >> 4) + 4u * ((lane >> 3) & 1)) * (uint32_t)a.msq +
                                   (uint32_t)(kw0 + 4 * (lane & 7))) * 4u
                                : 0u;
    const uint32_t jg = xs16((uint32_t)jl * 0x9E3779B9u);  // key part of the dropout draw, first xorshift applied

    int qb, qe;
    query_range(a, k0, min(k0 + kDkdvKeysPerBlock, a.Sk) - 1, qb, qe);
    static_assert(!WS || (BQ == kWsRows && kDkdvKeysPerBlock == kWsKeys), "workspace tiles are the pass's tiles");
    int64_t ws_p = 0;  // WS: workspace tiles of the key blocks before this one, per (b, h)
    if constexpr (WS) {
      // Tiles start on a multiple of 64 rows; a key block no row sees keeps its
      // empty range (aligning it down would make a tile the workspace has no
      // room for: its run is empty).
      if (qe > qb) qb -= qb % BQ;
      // the key blocks before this one, one per lane (a run has at most 2^23
      // tiles, so 64 of them sum exactly in 32 bits)
      for (int c0 = 0; c0 < kb; c0 += 64) {
        int ql, n;
        ws_run(a, c0 + lane, ql, n);
        ws_p += __builtin_amdgcn_readfirstlane(wave_sum_i32(c0 + lane < kb ? n : 0));
      }
    }
    const int ntq = (qe - qb + BQ - 1) / BQ;
    const int ntiles = ntq * a.group;

    if (ntiles > 0) {
      // Steps walk the query tiles in one direction (see below), each tile for
      // every query head of the group in turn.  A cursor names the tile whose
      // copies are issued next; past the last tile of the walk it stays there, so
      // the last copies repeat into stages that are never read and every step
      // runs the same straight-line code.
      // The cursor also carries the element offsets of the tile's first row in
      // Q/dO and in L/Delta, moved on by per-pass increments (no multiplies per step).
      struct Cursor {
        int g, t, qt;
        int64_t qoff, loff;
      };
      // Order: a block's first key block walks its query tiles from the last
      // down to the first, its second one (paired causal blocks) from the first
      // up to the last.  The blocks of one KV head run side by side on one XCD
      // and start together on the last tile, so in the first pass they read the
      // same Q/dO tiles at about the same time and share them in L2.  A block's
      // second pass begins when its first one ends, on a first tile that lies
      // as many tiles higher as its first pass was shorter: walking up, every
      // block in its second pass is on the same tile at the same time as well,
      // and shares those reads too (walking down, each would re-read the top
      // tiles on its own).
      const bool up = pass == 1;
      const int tdir = up ? 1 : -1;
      const int64_t inc_qh = a.qsh;  // next head, same tile
      const int64_t inc_qt = -(int64_t)(a.group - 1) * a.qsh + (int64_t)(tdir * BQ) * a.qss;  // first head, next tile
      const int64_t inc_lt = -(int64_t)(a.group - 1) * a.Sq + tdir * BQ;
      const int tfirst = up ? 0 : ntq - 1;
      auto cursor0 = [&]() {
        const int h0 = kvh * a.group;
        const int qt = qb + tfirst * BQ;
        return Cursor{0, tfirst, qt, (int64_t)b * a.qsb + (int64_t)h0 * a.qsh + (int64_t)qt * a.qss,
                      ((int64_t)b * a.Hq + h0) * a.Sq + qt};
      };
      // Next head, else the first head of the next tile, else stay: the
      // conditions, then one field per part (parts 0..4), so that a step can
      // spread the update over several pipeline slots.
      struct Turn {
        bool ng, nt;
      };
      auto turn_of = [&](const Cursor& c) { return Turn{c.g + 1 < a.group, up ? c.t < ntq - 1 : c.t > 0}; };
      auto advance_part = [&](Cursor& c, const Turn& w, int part) {
        if (part == 0) c.qoff += w.ng ? inc_qh : (w.nt ? inc_qt : 0);
        if (part == 1) c.loff += w.ng ? (int64_t)a.Sq : (w.nt ? inc_lt : 0);
        if (part == 2) c.qt = w.ng ? c.qt : (w.nt ? c.qt + tdir * BQ : c.qt);
        if (part == 3) c.t = w.ng ? c.t : (w.nt ? c.t + tdir : c.t);
        if (part == 4) c.g = w.ng ? c.g + 1 : (w.nt ? 0 : c.g);
      };
      auto advance = [&](Cursor& c) {
        const Turn w = turn_of(c);
#pragma unroll
        for (int part = 0; part < 5; ++part) advance_part(c, w, part);
      };
      // Q and dO rows of a tile into a ring stage: copy u of this wave fills rows
      // (wave*NIW + u)*RPI + lane/NCH.  Rows past the end repeat the last row;
      // they are never counted.  Per-lane offsets are 32-bit, relative to the
      // tile's first row (the host bounds the row stride).
      // A pending set of copies: the tile's first row in Q and in dO, the LDS
      // address of this wave's first Q row in the ring stage, the last row.
      struct Job {
        const __bf16* qp;
        const __bf16* dop;
        uint32_t lds;
        uint32_t lim2;  // byte offset of the tile's last row (rows past it repeat it), at most 2*BQ*qss
      };
      // Per-lane byte offsets of copy pair i's row (cp_off) and of its chunk alone
      // (cp_chk): a row r at most the last row lim is read at cp_off, else the last
      // row's chunk at lim2 + cp_chk, i.e. min(cp_off, lim2 + cp_chk).
      uint32_t cp_off[NIW], cp_chk[NIW];
#pragma unroll
      for (int i = 0; i < NIW; ++i) {
        const int r = (wave * NIW + i) * RPI + cp_row;
        cp_chk[i] = 16u * (uint32_t)pad_chunk(cp_pc ^ swz<D>(r), a.D / 8);
        cp_off[i] = 2u * (uint32_t)r * (uint32_t)a.qss + cp_chk[i];
      }
      constexpr int NC = 2 * NIW;  // copies per tile per wave
      constexpr int PER = NC / 4;  // copies per section
      static_assert(NC % 4 == 0, "a tile's copies spread over four sections");
      // Mask staging (MASK): element r of a half is copied into sM right after the
      // same element of the other half was used (sections A and C, the slot of
      // element r; MVEC: one copy per 4-element group, after its last element's
      // slot), and read MF slots before its own use two sections later.  The
      // wait before a read lets exactly the vector-memory operations issued
      // after that copy stay in flight (mask_read_wait), so it holds up neither
      // the later tile copies nor the dS stores.
      constexpr int MF = 4;
      constexpr int SG = 4 / (16 / NSD);  // slots per group
      constexpr int sl = (PER - 1) * (NSD / PER);  // section A's last tile copy slot
      constexpr int kMaskLateA = MVEC ? (SG - 1 >= sl) + (2 * SG - 1 >= sl) + (3 * SG - 1 >= sl) + (4 * SG - 1 >= sl)
                                      : 16 / PER;
      constexpr int kMaskPerStep = MVEC ? 8 : 32;
      auto job_of = [&](const Cursor& c, int stage) {
        const uint32_t lim = (uint32_t)min(a.Sq - 1 - c.qt, BQ);
        return Job{Q + c.qoff, dO + c.qoff, lds_addr(&sT[stage][0][wave * NIW * RPI * D]), 2u * lim * (uint32_t)a.qss};
      };
      // Copy u (0 .. 2*NIW-1; even: Q, odd: dO) of a job.
      auto issue_job = [&](const Job& j, int u) {
        const uint32_t off = min(cp_off[u >> 1], j.lim2 + cp_chk[u >> 1]);
        const uint32_t lds = j.lds + 2u * (uint32_t)((u >> 1) * RPI * D + (u & 1) * TILE);
        dma16((u & 1) ? j.dop : j.qp, off, lds);
      };
      // Slot hook: copies u0 .. u0+PER-1 of job j, one every nslots/PER slots.
      auto copies_at = [&](const Job& j, int u0, int k, int nslots) {
        if (k % (nslots / PER) == 0) issue_job(j, u0 + k / (nslots / PER));
      };
      auto issue_qdo = [&](const Cursor& c, int stage) {
        const Job j = job_of(c, stage);
#pragma unroll
        for (int u = 0; u < 2 * NIW; ++u) issue_job(j, u);
      };
      // L (wave 0) and Delta (wave 1) of a tile into an L ring stage (rows past
      // the end repeat the last row; waves 2 and 3 make the same copy into sDum),
      // and the tile's dropout row keys, first xorshift applied (lanes 0-15 of each
      // wave, 16 rows per wave).
      const float* const ld_src = (wave & 1) ? Dl : L;
      const uint32_t ld_dst = lds_addr(wave == 0 ? &sL[0][0] : (wave == 1 ? &sDel[0][0] : &sDum[wave & 1][0]));
      const uint32_t ld_stride = wave < 2 ? 4u * BQ : 0u;  // bytes per ring stage
      auto issue_ld = [&](const Cursor& c, int lst) {
        dma4(ld_src + c.loff, 4u * (uint32_t)min(lane, a.Sq - 1 - c.qt), ld_dst + (uint32_t)lst * ld_stride);
        if constexpr (DROP) {
          // the row's global index ((b*Hq + h)*Sq + i) mod 2^32 (drop_row_key)
          uint32_t* rp = lane < 16 ? &sRK[lst][16 * wave + lane] : reinterpret_cast<uint32_t*>(&sDum[1][lane]);
          *rp = xs16(fmix32((uint32_t)c.loff + (uint32_t)(16 * wave + lane) + a.seed_mix));
        }
      };
      // Once a stage's L/Delta landed and a barrier passed, each wave rewrites 16
      // rows of it in place: L -> -L/scale (lanes 0-15) and, when the dP chain
      // is seeded with it, Delta -> -Delta (lanes 16-31).  The read and the write
      // go into different sections, so the LDS latency hides behind MFMAs.
      const bool fix_lane = lane < (FOLD ? 32 : 16);
      float* const fix_p = lane < 16 ? &sL[0][16 * wave + lane] : &sDel[0][16 * wave + (lane & 15)];
      const float fix_f = lane < 16 ? -a.inv_scale : -1.f;
      float fix_v = 0.f;
      auto fix_at = [&](int lst) { return fix_lane ? fix_p + lst * BQ : &sDum[0][lane]; };
      auto fix_rd = [&](int lst) { fix_v = *fix_at(lst); };
      auto fix_wr = [&](int lst) { *fix_at(lst) = fix_v * fix_f; };
      // Waits until this wave's copies issued before the previous step's have
      // landed (the tile copies and the L/Delta copy of a step; with a mask, the 32
      // mask copies of a step too, and those of section A issued after its last
      // tile copy, 16 / PER of them).
      constexpr int NMV = MASK ? kMaskPerStep + kMaskLateA : 0;
      // WS: the dS stores of the previous step's sections B and D come after
      // those copies too.
      constexpr int NWS = WS ? 4 : 0;
      auto wait_prev = [&]() { wait_vmcnt<2 * NIW + NMV + 1 + NWS>(); };
      // WS: lane l stores the dS of its key (32*wave + l%32) for rows 16t + 8*h2
      // .. +7 (register order) of half m at m*8192 + 2048*wave + 1024t + 32*(l%32)
      // + 16*h2 bytes of the tile: each store writes 1 KB in one piece.
      const uint32_t ws_lane = (uint32_t)(2048 * wave + 32 * l32 + 16 * h2);

      // Instruction order inside a step is fixed by hand: one wave per SIMD means
      // the MFMAs overlap only the VALU and LDS work placed between them, so every
      // slot below (an MFMA, the LDS reads a few MFMAs ahead, a slice of the
      // exp/dS arithmetic) is fenced off with sched_barrier.
      auto fence = []() { __builtin_amdgcn_sched_barrier(0); };
      // Row-major A operand of S/dP MFMA k (even: Q chunk k/2 for S, odd: dO chunk for dP).
      auto rd_op = [&](int m, int stq, int k) {
        return lds_read_b128(sT[stq][0] + rd_off[k >> 1] + (k & 1) * TILE + 32 * m * D);
      };
      // Transposed A operand half j (0 .. 2*NDK-1) of dV/dK MFMA j/2 of half m:
      // MFMA n = 2*DB*t + 2d + w takes dO^T (w = 0, for dV) or Q^T (w = 1, for dK)
      // rows 32m + 16t .. +15 of column block d; j even = first 8 rows, odd = last 8.
      auto rd_tr = [&](int m, int stq, int j) {
        const int n = j >> 1, t = n / (2 * DB), d = (n % (2 * DB)) >> 1, w = n & 1;
        const __bf16* base = sT[stq][0] + (w ? 0 : TILE) + (32 * m + 16 * t) * D;
        return lds_read_tr(base + ((j & 1) ? tr_hi[d] : tr_lo[d]));
      };
      auto mma_dkv = [&](int n, const bf16x4& lo, const bf16x4& hi, const bf16x8 (&pmc)[2], const bf16x8 (&dsc)[2]) {
        const int t = n / (2 * DB), d = (n % (2 * DB)) >> 1;
        if (n & 1)
          mfma_acc(acck[d], concat(lo, hi), dsc[t]);
        else
          mfma_acc(accv[d], concat(lo, hi), pmc[t]);
      };

      // What an S/dP + exp/dS section needs first, read by the section before it:
      // the A operands of its first PF MFMAs, the -L/scale rows its S chain
      // starts from, and the -Delta rows its dP chain starts from (FOLD) or the
      // Delta rows of the exp/dS half (dropout).
#ifndef FA_DKDV_PF
#define FA_DKDV_PF 6
#endif
      constexpr int PF = FA_DKDV_PF;
      static_assert(PF < 8, "operand reads run ahead within a ring of 8");
      typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
      struct SdpPre {
        bf16x8 op[PF];
        f32x16 nls, dpi;
        f32x4 dl[4];
        u32x4 rk[DROP ? 4 : 1];  // dropout row keys of the exp/dS half
      };
      constexpr int NPRE = PF + 8 + (DROP ? 4 : 0);  // LDS reads of a prefetch
      // Prefetch read p (0 .. NPRE-1) for a section computing S/dP of half ms
      // (stage sts, L ring stage lsts) and exp/dS of half me (L ring stage lste).
      // Read order: the chain seeds first (the section's first two MFMAs need
      // them), then the dropout row keys, then the A operands in MFMA order.
      auto prefetch = [&](SdpPre& pre, int p, int ms, int sts, int lsts, int me, int lste) {
        if (p < 4) {
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(&sL[lsts][32 * ms + 8 * p + 4 * h2]);
#pragma unroll
          for (int e = 0; e < 4; ++e) pre.nls[4 * p + e] = l4[e];
          return;
        }
        p -= 4;
        if (p < 4) {
          if constexpr (FOLD) {
            const f32x4 d4 = *reinterpret_cast<const f32x4*>(&sDel[lsts][32 * ms + 8 * p + 4 * h2]);
#pragma unroll
            for (int e = 0; e < 4; ++e) pre.dpi[4 * p + e] = d4[e];
          } else {
            pre.dl[p] = *reinterpret_cast<const f32x4*>(&sDel[lste][32 * me + 8 * p + 4 * h2]);
          }
          return;
        }
        p -= 4;
        if constexpr (DROP) {
          if (p < 4) {
            pre.rk[p] = *reinterpret_cast<const u32x4*>(&sRK[lste][32 * me + 8 * p + 4 * h2]);
            return;
          }
          p -= 4;
        }
        pre.op[p] = rd_op(ms, sts, p);
      };
      auto prefetch_all = [&](SdpPre& pre, int ms, int sts, int lsts, int me, int lste) {
#pragma unroll
        for (int p = 0; p < NPRE; ++p) prefetch(pre, p, ms, sts, lsts, me, lste);
      };

      // Section "S/dP + exp/dS": S/dP of half ms from stage sts (with FOLD the dP
      // chain starts from the rows' -Delta), overlapped with the exp/dS of half me
      // of tile (qt, h) (values se, dpe; L ring stage lste) and with the transposed
      // reads of the first NP MFMAs of that half's dV/dK (stage ste).  Operand
      // reads run PF MFMAs ahead; the 16 exp/dS elements are spread over the slots.
      // The last XD elements of an exp/dS half: their exponent input is formed in
      // the S/dP section (with the mask and the visibility test), their exp, P,
      // dS and packing in the first slots of the dV/dK section that follows,
      // whose MFMAs leave issue slots free (the S/dP sections have none), before
      // its MFMAs that read them (the second eight).
#ifndef FA_DKDV_XD
#define FA_DKDV_XD 2
#endif
      constexpr int XD = FA_DKDV_XD;
      static_assert(XD % 2 == 0 && XD <= 8, "deferred elements come in packed pairs of the second eight");
      struct Defer {
        float x[XD > 0 ? XD : 1], dpe[XD > 0 ? XD : 1], dl[XD > 0 ? XD : 1];
        uint32_t rk[XD > 0 ? XD : 1];
      };
      Defer df;
      auto sec_sdp_ew = [&](auto full_c, int ms, int sts, f32x16& s, f32x16& dp, const SdpPre& pre, int me,
                            int ste, int qt, const f32x16& se, const f32x16& dpe,
                            bf16x8 (&pmc)[2], bf16x8 (&dsc)[2], bf16x4 (&trp)[2 * NP], auto&& slot_extra) {
        constexpr bool FULL = decltype(full_c)::value;
        bf16x8 op[8];
#pragma unroll
        for (int k = 0; k < PF; ++k) op[k] = pre.op[k];
        // Visible rows of this lane's key in the tile: d = j - i in (dlo, dhi), row
        // in range, key in range, i.e. tile rows [lo, hi).  Element r sits at row
        // 32*me + 4*h2 + c(r), c(r) = 8*(r/4) + r%4, so it is visible iff
        // c(r) - lb < span (unsigned) with lb = lo - 32*me - 4*h2.
        int lb = 0;
        uint32_t span = 0;
        if constexpr (!FULL) {
          // no overflow: |dl0| <= 2^29 + 128 and the bounds lie within +-(2^30 + 1)
          const int dl0 = jl - qt;  // d = dl0 - row
          const int lo = max(dl0 - vb.dhi + 1, 0);
          const int hi = jl < a.Sk ? min(dl0 - vb.dlo, a.Sq - qt) : 0;
          span = (uint32_t)max(hi - lo, 0);
          lb = lo - 32 * me - 4 * h2;
        }
        float pr[16], pv[16], dv[16];
        float mk[16];  // mask values of the half (MASK), read ahead from sM
        // exp of element r (C-layout register r of half me); se holds
        // Q.K - L/scale, so scale*log2(e)*se is the exponent (S - L)*log2(e).
        // A mask value at or below the -1e30 sentinel excludes the element: added
        // in the exponent it makes exp2 exactly 0 (|S - L| is far below 1e29), so
        // it needs no compare of its own, and interior tiles with a mask take
        // the same path without the visibility test.
        auto ew_exp = [&](int r) {
          float x = se[r] * a.scale_log2;
          if constexpr (MASK) x = __builtin_fmaf(mk[r], kLog2e, x);
          if constexpr (!FULL) x = elem_visible(r, lb, span) ? x : -__builtin_inff();
          if (r >= 16 - XD) {  // finished in the next dV/dK section
            const int u = r - (16 - XD);
            df.x[u] = x;
            df.dpe[u] = dpe[r];
            if constexpr (DROP) {
              df.rk[u] = pre.rk[r >> 2][r & 3];
              df.dl[u] = pre.dl[r >> 2][r & 3];
            }
            return;
          }
          pr[r] = __builtin_amdgcn_exp2f(x);
        };
        // P and dS of element r, one slot after its exp; odd r packs the pair.
        auto ew_ds = [&](int r) {
          if (r >= 16 - XD) return;
          if constexpr (DROP) {
            const float mm = fmix32_tail(pre.rk[r >> 2][r & 3] ^ jg) >= a.drop_thr ? a.drop_inv : 0.f;
            pv[r] = pr[r] * mm;
            dv[r] = pr[r] * (dpe[r] * mm - pre.dl[r >> 2][r & 3]);
          } else {
            pv[r] = pr[r];
            dv[r] = pr[r] * dpe[r];
          }
          if (r & 1) {
            const bf16x2 tp = pack_here(pv[r - 1], pv[r]);
            const bf16x2 td = pack_here(dv[r - 1], dv[r]);
            pmc[r >> 3][(r & 7) - 1] = tp[0];
            pmc[r >> 3][r & 7] = tp[1];
            dsc[r >> 3][(r & 7) - 1] = td[0];
            dsc[r >> 3][r & 7] = td[1];
          }
        };
        // Mask values of the half, read from this wave's LDS staging MF slots ahead
        // of their use, each once its copy (issued two sections earlier) landed.
        auto mask_rd = [&](int kk) {
          if constexpr (MASK) {
            if (kk < NSD) {
              // (the dV/dK section in between: PER tile copies, the two dS stores
              // with WS, and in section B the L/Delta copy, left out: a wait for
              // one operation fewer is still sufficient)
              wait_vmcnt_n(mask_read_wait<NSD, PER, MVEC, MF, PER + (WS ? 2 : 0)>(kk));
#pragma unroll
              for (int i = 0; i < 16 / NSD; ++i) {
                const int r = kk * (16 / NSD) + i;
                if constexpr (MVEC)
                  mk[r] = (&sM[wave][0][0])[256 * (r >> 2) + 64 * (r & 3) + 32 * h2 + l32];
                else
                  mk[r] = sM[wave][r][lane];
              }
            }
          }
        };
#pragma unroll
        for (int k = 0; k < MF; ++k) mask_rd(k);
        fence();
#pragma unroll
        for (int k = 0; k < NSD; ++k) {
          const bf16x8& o = op[k & 7];
          if (k & 1) {
            if (k == 1 && FOLD)
              mfma_v_seed(dp, o, vr[k >> 1], pre.dpi);
            else if (k == 1)
              mfma_v0(dp, o, vr[k >> 1]);
            else
              mfma_v(dp, o, vr[k >> 1]);
          } else {
            if (k == 0)
              mfma_v_seed(s, o, kr[k >> 1], pre.nls);
            else
              mfma_v(s, o, kr[k >> 1]);
          }
          if (k + PF < NSD) op[(k + PF) & 7] = rd_op(ms, sts, k + PF);
          if (k >= NSD - 2 * NP) trp[k - (NSD - 2 * NP)] = rd_tr(me, ste, k - (NSD - 2 * NP));
          // 16 exp/dS elements over the NSD slots: the exps of this slot's elements
          // and the P/dS of the previous slot's (no result is read right after its exp)
          constexpr int E = 16 / NSD;
#pragma unroll
          for (int i = 0; i < E; ++i) ew_exp(k * E + i);
          if (k > 0) {
#pragma unroll
            for (int i = 0; i < E; ++i) ew_ds((k - 1) * E + i);
          }
          mask_rd(k + MF);
          slot_extra(k);
          // The seed blocks are read as accumulator inputs by the chains' first
          // MFMAs (slots 0 and 1) while those run: they stay allocated until the
          // chains' second MFMAs (which wait for the first ones' results) have
          // issued, so nothing is written into them earlier.
          if (k == 3) {
            keep_live(pre.nls);
            if constexpr (FOLD) keep_live(pre.dpi);
          }
          fence();
        }
#pragma unroll
        for (int i = 0; i < 16 / NSD; ++i) ew_ds(16 - 16 / NSD + i);
        // The packed P/dS are complete here; S/dP are next read a whole section
        // later (the prologue drains them explicitly).
        materialise(pmc, dsc);
        mfma_settle(s, dp);
        fence();
      };
      // Slots 0 and 1 of a dV/dK section: the exps of the deferred elements, then
      // their P and dS, packed into the second operand block.
      float prd[XD > 0 ? XD : 1];
      auto defer_slot = [&](int n, bf16x8 (&pmc)[2], bf16x8 (&dsc)[2]) {
        if constexpr (XD > 0) {
          if (n == 0) {
#pragma unroll
            for (int u = 0; u < XD; ++u) prd[u] = __builtin_amdgcn_exp2f(df.x[u]);
          }
          if (n == 1) {
            float pv[XD > 0 ? XD : 1], dv[XD > 0 ? XD : 1];
#pragma unroll
            for (int u = 0; u < XD; ++u) {
              if constexpr (DROP) {
                const float mm = fmix32_tail(df.rk[u] ^ jg) >= a.drop_thr ? a.drop_inv : 0.f;
                pv[u] = prd[u] * mm;
                dv[u] = prd[u] * (df.dpe[u] * mm - df.dl[u]);
              } else {
                pv[u] = prd[u];
                dv[u] = prd[u] * df.dpe[u];
              }
            }
#pragma unroll
            for (int u = 0; u < XD; u += 2) {
              const int r = 16 - XD + u;  // even: the pair r, r + 1
              const bf16x2 tp = pack_here(pv[u], pv[u + 1]);
              const bf16x2 td = pack_here(dv[u], dv[u + 1]);
              pmc[1][r & 7] = tp[0];
              pmc[1][(r & 7) + 1] = tp[1];
              dsc[1][r & 7] = td[0];
              dsc[1][(r & 7) + 1] = td[1];
            }
          }
        }
      };
      // Section "dV/dK" of half m (stage stq): MFMAs 0 .. NP-1 take the transposed
      // operands read by the previous section; slot n reads those of MFMA n + NP.
      auto sec_dkv = [&](int m, int stq, const bf16x4 (&trp)[2 * NP], const bf16x8 (&pmc)[2], const bf16x8 (&dsc)[2],
                         auto&& slot_extra) {
        constexpr int W = NP + 1;  // operand pairs in flight
        bf16x4 buf[2 * W];
#pragma unroll
        for (int n = 0; n < NP; ++n) {
          buf[2 * n] = trp[2 * n];
          buf[2 * n + 1] = trp[2 * n + 1];
        }
#pragma unroll
        for (int n = 0; n < NDK; ++n) {
          const int sl = n % W;
          mma_dkv(n, buf[2 * sl], buf[2 * sl + 1], pmc, dsc);
          if (n + NP < NDK) {
            const int sn = (n + NP) % W;
            buf[2 * sn] = rd_tr(m, stq, 2 * (n + NP));
            buf[2 * sn + 1] = rd_tr(m, stq, 2 * (n + NP) + 1);
          }
          slot_extra(n);
          fence();
        }
      };

      // Prologue: L/Delta of tiles 0-3 and Q/dO of tile 0, landed together with
      // the K and V rows; then Q/dO of tile 1 and most of tile 2's copies, which
      // stream in while the first section computes (the first step waits for
      // tile 1 itself); L/Delta of tiles 0 and 1 fixed (steps 0 and 1 fix those
      // of tiles 2 and 3).
      // Mask staging: element r of half `half` of tile (g, t) into sM[wave][r].
      auto mask_src = [&](int g) {
        return raw_rsrc(a.mask + (int64_t)b * a.msb + (int64_t)(kvh * a.group + g) * a.msh, a.mask_rec);
      };
      auto mask_vb = [&](int qt, int half) { return m_lvo + (uint32_t)(qt + 32 * half) * msq4; };
      auto mask_cp = [&](rsrc_t rs, uint32_t vb0, int r) {
        dma_buf4(rs, mad24(8 * (r >> 2) + (r & 3), msq4, vb0), lds_addr(&sM[wave][r][0]));
      };
      // MVEC: group g of a half (rows 8g .. 8g+7 from vbv, the half's first row)
      auto mask_cpv = [&](rsrc_t rs, uint32_t vbv, int g) {
        dma_buf16(rs, mad24(8 * g, msq4, vbv), lds_addr(&sM[wave][4 * g][0]));
      };
      auto mask_vbv = [&](int qt, int half) { return m_lvv + (uint32_t)(qt + 32 * half) * msq4; };
      // Slot hook of sections A and C: the copies refilling the elements (MVEC:
      // the groups) whose last use was slot k.
      auto mask_refill = [&](rsrc_t rs, int qt, int half, int k) {
        if constexpr (MVEC) {
          if (k % SG == SG - 1) mask_cpv(rs, mask_vbv(qt, half), k / SG);
        } else if constexpr (MASK) {
#pragma unroll
          for (int i = 0; i < 16 / NSD; ++i) mask_cp(rs, mask_vb(qt, half), k * (16 / NSD) + i);
        }
      };
      // The cursor cm names tile it+1, whose half 0 section C of step it stages.
      Cursor cm = cursor0();
      if constexpr (MASK) {
        const rsrc_t rs = mask_src(cm.g);  // the first step's tile
#pragma unroll
        for (int k = 0; k < NSD; ++k) mask_refill(rs, cm.qt, 0, k);
        advance(cm);
      }

      Cursor cq = cursor0(), cl = cursor0();
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        issue_ld(cl, s);
        advance(cl);
      }
      issue_qdo(cq, 0);
      advance(cq);
      wait_all_vmem();  // K, V, L/Delta and tile 0 landed (a wait the compiler sees)
      issue_qdo(cq, 1);
      advance(cq);
      // A tile's copies go out over four sections, from the barrier on (the
      // vector-memory unit takes a copy per ~16 cycles per CU, so a burst of them
      // would hold up the issuing wave): a quarter each in sections B, C and D of
      // one step and in A of the next.  Tile 2: its first three quarters now.
      Job pend = job_of(cq, 2);
#pragma unroll
      for (int u = 0; u < NC - PER; ++u) issue_job(pend, u);
      advance(cq);
      barrier_lds();
      fix_rd(0);
      fix_wr(0);
      fix_rd(1);
      fix_wr(1);
      barrier_lds();

      // S/dP of half 0 of the current tile, carried between steps, and the
      // prefetch of the next S/dP + exp/dS section.
      f32x16 s0, dp0;
      SdpPre pre;
      {
        bf16x8 pm[2], ds[2];
        bf16x4 trp[2 * NP];
        f32x16 z{};
        prefetch_all(pre, 0, 0, 0, 0, 0);
        // a section with no exp/dS work to overlap: only its S/dP result is kept
        sec_sdp_ew(std::true_type{}, 0, 0, s0, dp0, pre, 0, 0, qb, z, z, pm, ds, trp, [](int) {});
        mfma_drain(s0, dp0);  // read by the first step's exp/dS after only a few instructions
        prefetch_all(pre, 1, 0, 0, 0, 0);  // for section A of step 0
      }

      int it = 0;
      // One step (see the header comment).  KIND 1 = boundary tile (per-element
      // predicate), 2 = interior tile (every element counted); each kind runs in a
      // loop of its own, so no loop body branches.
      auto step = [&](auto kind_c, int g, int t) {
        constexpr bool FULL = decltype(kind_c)::value == 2;
        const std::integral_constant<bool, FULL> full_c;
        const int stq = it & (NST - 1);
        const int stq1 = (it + 1) & (NST - 1);
        const int stq3 = (it + 3) & (NST - 1);
        const int lst = it & (NSL - 1);
        const int lst1 = (it + 1) & (NSL - 1);
        const int lst2 = (it + 2) & (NSL - 1);
        const int lst4 = (it + 4) & (NSL - 1);
        const int qt = qb + t * BQ;
        const int h = kvh * a.group + g;
        unsigned char* wsb = nullptr;  // WS: this step's workspace tile
        if constexpr (WS) wsb = ws + ((int64_t)(b * a.Hq + h) * a.ws_tiles + ws_p + t) * kWsTileBytes;
        auto store_ds = [&](int n, int half, const bf16x8 (&d)[2]) {
          if constexpr (WS) {
            if (n == NDK - 2) st16_nt(wsb, ws_lane + 8192u * half, d[0]);
            if (n == NDK - 1) st16_nt(wsb, ws_lane + 8192u * half + 1024u, d[1]);
          }
        };
        bf16x8 pm[2], ds[2];
        bf16x4 trp[2 * NP];
        f32x16 s1, dp1;
        // Prefetch read p goes into slot pre_slot(p) of a dV/dK section (the last
        // NPRE slots, or spread over all of them when there are fewer).
        auto pre_at = [&](int n, int ms, int sts, int lsts, int me, int lste) {
#pragma unroll
          for (int p = 0; p < NPRE; ++p) {
            const int slot = NPRE <= NDK ? p : p * NDK / NPRE;
            if (slot == n) prefetch(pre, p, ms, sts, lsts, me, lste);
          }
        };
        // A: S/dP of half 1 with exp/dS of half 0; the last quarter of tile it+2's copies.
        // Each slot then stages the mask of half 1 of this tile in place of the
        // half-0 elements it used.
        const rsrc_t mrs_a = mask_src(g);
        sec_sdp_ew(full_c, 1, stq, s1, dp1, pre, 0, stq, qt, s0, dp0, pm, ds, trp, [&](int k) {
          copies_at(pend, NC / 2 + PER, k, NSD);
          mask_refill(mrs_a, qt, 1, k);
        });
        // Step 0: tile 1's copies went out in the prologue, followed only by tile
        // 2's (NC) and section A's mask copies, fewer than the steady state has.
        if (it == 0) wait_vmcnt<NC + (MASK ? kMaskPerStep / 2 : 0)>();
        wait_prev();  // tile it+1 landed everywhere once all waves pass the barrier
        barrier_only();
        const Cursor cl_now = cl;  // tile it+4: the copies' cursor of the next step
        Job next;
        Turn turn;
        // B: dV/dK of half 0; prefetch for C (S/dP of half 0 of tile it+1, exp/dS
        // of half 1).  The cursors' bookkeeping is spread over its slots (not
        // put between the barrier and its first MFMA), so its copies start one
        // slot later.
        constexpr int kLd = NDK >= 16 ? 2 : 1, kTurn = NDK >= 16 ? 3 : 1, kAdv = kTurn + 1;
        static_assert(kAdv + 4 < NDK, "the cursor update fits section B");
        sec_dkv(0, stq, trp, pm, ds, [&](int n) {
          defer_slot(n, pm, ds);
          if (n == 0) next = job_of(cq, stq3);
          if (n == kLd) issue_ld(cl, lst4);
          if (n == kTurn) turn = turn_of(cl);
          if (n >= kAdv && n < kAdv + 5) advance_part(cl, turn, n - kAdv);
          if (n >= 1) copies_at(next, 0, n - 1, NDK);
          pre_at(n, 0, stq1, lst1, 1, lst);
          if (n == NDK / 2) fix_rd(lst2);  // L/Delta of tile it+2 (its copy landed before this step's barrier)
          store_ds(n, 0, ds);
        });
        // C: S/dP of half 0 of tile it+1 with exp/dS of half 1; each slot then
        // stages the mask of half 0 of tile it+1 in place of the elements it used
        const rsrc_t mrs_c = mask_src(cm.g);
        sec_sdp_ew(full_c, 0, stq1, s0, dp0, pre, 1, stq, qt, s1, dp1, pm, ds, trp, [&](int k) {
          copies_at(next, PER, k, NSD);
          if (k == 1) fix_wr(lst2);
          mask_refill(mrs_c, cm.qt, 0, k);
        });
        // D: dV/dK of half 1; prefetch for A of the next step
        sec_dkv(1, stq, trp, pm, ds, [&](int n) {
          defer_slot(n, pm, ds);
          copies_at(next, 2 * PER, n, NDK);
          pre_at(n, 1, stq1, lst1, 0, lst1);
          store_ds(n, 1, ds);
        });
        pend = next;
        cq = cl_now;
        if constexpr (MASK) advance(cm);
        ++it;
      };

      const std::integral_constant<int, 1> kEdge;
      const std::integral_constant<int, 2> kInner;
      // This wave's tiles: [0,f0) boundary, [f0,f1) interior, [f1,ntq)
      // boundary (the visible key interval moves monotonically with the query
      // row, so the interior tiles are contiguous), walked in the pass's
      // direction, each for every query head of the group.  Boundary tiles
      // include tiles this wave cannot see at all; the predicate zeroes them.
      auto all = [&](int t) { return rect_all_visible(a, qb + t * BQ, qb + t * BQ + BQ - 1, kw0, kw0 + kDkdvKeysPerWave - 1); };
      int f0 = 0;
      while (f0 < ntq && !all(f0)) ++f0;
      int f1 = f0;
      while (f1 < ntq && all(f1)) ++f1;
      const int n_first = up ? f0 : ntq - f1, n_last = up ? ntq - f1 : f0;
      int t = tfirst;
      for (int u = 0; u < n_first; ++u, t += tdir)
        for (int g = 0; g < a.group; ++g) step(kEdge, g, t);
      for (int u = f0; u < f1; ++u, t += tdir)
        for (int g = 0; g < a.group; ++g) step(kInner, g, t);
      for (int u = 0; u < n_last; ++u, t += tdir)
        for (int g = 0; g < a.group; ++g) step(kEdge, g, t);
      wait_vmcnt<0>();  // the repeated copies of the last steps have landed
      barrier_lds();    // every wave is done with the ring before the next pass refills it
    }
    mfma_drain_acc(acck, accv);  // the accumulators' last MFMAs have finished before they are read

    // dK and dV of this wave's 32 keys leave through LDS (the ring is free: every
    // wave has passed this pass's last barrier), so that each store writes 16
    // bytes of a row and D/8 lanes a whole row: lane (l32, h2) puts its
    // 4-element pieces of key l32 into a per-wave [2][32][D + 8] bf16 block,
    // then lane l reads chunk l % (D/8) of rows RPS*i + l / (D/8) and stores it.
    {
      constexpr int SR = D + 8;                 // staging row, elements (16 bytes of padding)
      constexpr int CPR = D / 8, RPS = 64 / CPR;  // 16-byte chunks per row, rows per read and store
      static_assert(4 * 2 * 32 * SR <= NST * 2 * TILE, "the staging blocks fit the ring");
      __bf16* const stg = &sT[0][0][0] + wave * 2 * 32 * SR;
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
          *reinterpret_cast<bf16x4*>(stg + l32 * SR + dd) = ok4;
          *reinterpret_cast<bf16x4*>(stg + (32 + l32) * SR + dd) = ov4;
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave's writes land before its reads
      const int c = lane % CPR;
      const int64_t kvbase = (int64_t)b * a.ksb + (int64_t)kvh * a.ksh + 8 * c;
#pragma unroll
      for (int i = 0; i < 32 / RPS; ++i) {
        const int r = RPS * i + lane / CPR;
        const bf16x8 vk = *reinterpret_cast<const bf16x8*>(stg + r * SR + 8 * c);
        const bf16x8 vv = *reinterpret_cast<const bf16x8*>(stg + (32 + r) * SR + 8 * c);
        if (kw0 + r < a.Sk && 8 * c < a.D) {  // rows past the end, chunks past the head dimension: not written
          const int64_t off = kvbase + (int64_t)(kw0 + r) * a.kss;
          *reinterpret_cast<bf16x8*>(dK + off) = vk;
          *reinterpret_cast<bf16x8*>(dV + off) = vv;
        }
      }
      barrier_lds();  // every wave's reads are done before a next pass refills the ring
    }
  }
}

template <int D, int MK, bool DROP, bool WS>
static hipError_t launch_t(const PrefillArgs& a, const void* Q, const void* K, const void* V, const void* dO,
                           const float* L, const float* delta, void* dK, void* dV, void* ws, hipStream_t st) {
  const int nkb = (a.Sk + kDkdvKeysPerBlock - 1) / kDkdvKeysPerBlock;
  const int paired = (a.causal && a.window == 0 && nkb > 1) ? 1 : 0;
  const int nwi = paired ? (nkb + 1) / 2 : nkb;
  const unsigned grid = (unsigned)(nwi * a.B * a.Hkv);
  hipLaunchKernelGGL((dkdv_bf16_kernel<D, MK, DROP, WS>), dim3(grid), dim3(256), 0, st, a,
                     static_cast<const __bf16*>(Q), static_cast<const __bf16*>(K), static_cast<const __bf16*>(V),
                     static_cast<const __bf16*>(dO), L, delta, static_cast<__bf16*>(dK), static_cast<__bf16*>(dV),
                     static_cast<unsigned char*>(ws), nkb, paired);
  return hipGetLastError();
}

template <int D, bool WS>
static hipError_t launch_d(const PrefillArgs& a, const void* Q, const void* K, const void* V, const void* dO,
                           const float* L, const float* delta, void* dK, void* dV, void* ws, hipStream_t st) {
  const bool drop = a.drop != 0;
  const int mk = a.mask == nullptr ? 0 : (mask_keys_contiguous(a) ? 2 : 1);
  if (mk == 2) return drop ? launch_t<D, 2, true, WS>(a, Q, K, V, dO, L, delta, dK, dV, ws, st)
                           : launch_t<D, 2, false, WS>(a, Q, K, V, dO, L, delta, dK, dV, ws, st);
  if (mk == 1) return drop ? launch_t<D, 1, true, WS>(a, Q, K, V, dO, L, delta, dK, dV, ws, st)
                           : launch_t<D, 1, false, WS>(a, Q, K, V, dO, L, delta, dK, dV, ws, st);
  return drop ? launch_t<D, 0, true, WS>(a, Q, K, V, dO, L, delta, dK, dV, ws, st)
              : launch_t<D, 0, false, WS>(a, Q, K, V, dO, L, delta, dK, dV, ws, st);
}

hipError_t launch_dkdv_bf16(const PrefillArgs& a, int D, const void* Q, const void* K, const void* V,
                            const void* dO, const float* L, const float* delta, void* dK, void* dV,
                            hipStream_t st) {
  return D <= 64 ? launch_d<64, false>(a, Q, K, V, dO, L, delta, dK, dV, nullptr, st)
                 : launch_d<128, false>(a, Q, K, V, dO, L, delta, dK, dV, nullptr, st);
}

hipError_t launch_dkdv_bf16_ws(const PrefillArgs& a, int D, const void* Q, const void* K, const void* V,
                               const void* dO, const float* L, const float* delta, void* dK, void* dV, void* ws,
                               hipStream_t st) {
  return D <= 64 ? launch_d<64, true>(a, Q, K, V, dO, L, delta, dK, dV, ws, st)
                 : launch_d<128, true>(a, Q, K, V, dO, L, delta, dK, dV, ws, st);
}

}  // namespace fa
