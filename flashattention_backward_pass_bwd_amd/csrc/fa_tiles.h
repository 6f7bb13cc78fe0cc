// bf16 LDS tiles for the gfx950 MFMA kernels.
//
// A tile holds rows of D bf16 values, row-major, 2*D bytes per row with no
// padding; the 16-byte chunk c of row r is stored at chunk position
// c ^ swz(r).  Two read patterns hit the tile:
//   * row reads (ds_read_b128): lane l reads chunk c of row r0 + l%32 -- the
//     MFMA operand whose k index runs along the row;
//   * transposed reads (ds_read_b64_tr_b16): each 16-lane group reads a
//     4-row x 16-column block and every lane receives one column of 4 rows --
//     the MFMA operand whose k index runs down the rows.
// gfx950's LDS serves 256 bytes per clock (64 four-byte banks).  The swizzle
// spreads sixteen consecutive rows over sixteen distinct 16-byte bank groups
// (row reads) and four consecutive rows over four distinct 64-byte bank groups
// (transposed reads of a 32-lane half), so neither pattern has bank conflicts:
//   D = 128 (16 chunks per row): swz(r) = 4*(r%4) + (r/4)%4
//   D = 64  (8 chunks, two rows per 256 bytes): swz(r) = 4*((r/2)%2) + (r/4)%4
#pragma once

#include "fa_common.h"

namespace fa {

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// Element offset of chunk c of row r in a swizzled tile with D columns.
template <int D>
__device__ __forceinline__ int tile_off(int r, int c) {
  return r * D + ((c ^ swz<D>(r)) << 3);
}

__device__ __forceinline__ bf16x8 lds_read_b128(const __bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

__device__ __forceinline__ bf16x4 lds_read_tr(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}

__device__ __forceinline__ bf16x8 concat(const bf16x4& a, const bf16x4& b) {
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// LDS byte address of a __shared__ object: a generic pointer to LDS carries
// the LDS offset in its low 32 bits.
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)p; }

// Direct global->LDS copies (global_load_lds_dword / _dwordx4, scalar base +
// 32-bit per-lane byte offset): lane l's 4 or 16 bytes at sbase + voff land
// at LDS byte address lds + 4*l or 16*l; lds must be wave-uniform.  They are
// issued as inline assembly on purpose: the compiler then does not treat them
// as LDS writes and does not wait for every copy in flight before each later
// LDS read, which would serialise the copy ring.  Callers order them with
// wait_vmcnt (every wave waits for its own copies) and a block barrier.
// The base (and M0's value) reach the asm in SGPRs, which the compiler may
// have just written with VALU (v_readfirstlane_b32); gfx9 needs five wait
// states between such a write and a vector memory instruction reading the
// SGPR, and the compiler does not insert them in front of an asm statement, so
// every copy and store here issues them itself (s_nop 4; with the M0 write,
// six).  tests/test_asm_checks.py checks the generated assembly for it.
// M0 holds the LDS address for the copy.  It is written without being saved:
// the compiler itself never reads or writes M0 in the kernels that use these
// copies (gfx9 LDS instructions do not need it, and these kernels have no
// dynamically indexed register arrays or messages), which
// tests/test_asm_checks.py checks on the generated assembly.  One wait state
// separates the M0 write from the copy (covered by the five above).
// The base is wave-uniform by contract; it is read into SGPRs explicitly
// (readfirstlane, free when the compiler already holds it there), because an
// "s" operand the compiler happens to keep in VGPRs is not moved for the asm.
__device__ __forceinline__ uint64_t sgpr_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 4\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sgpr_ptr(sbase)), "s"(__builtin_amdgcn_readfirstlane(lds)));
}

__device__ __forceinline__ void dma4(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 4\n\tglobal_load_lds_dword %0, %1"
               :
               : "v"(voff), "s"(sgpr_ptr(sbase)), "s"(__builtin_amdgcn_readfirstlane(lds)));
}

// The same copy with the streaming cache policy (nt), for data read once.
__device__ __forceinline__ void dma16_nt(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 4\n\tglobal_load_lds_dwordx4 %0, %1 nt"
               :
               : "v"(voff), "s"(sgpr_ptr(sbase)), "s"(__builtin_amdgcn_readfirstlane(lds)));
}

// 16-byte store of a lane's register block at a wave-uniform base + 32-bit
// lane offset, with the streaming cache policy (nt: written once, read by a
// later kernel).  Inline assembly like the copies: the compiler places no
// waits for it.  Stores count in vmcnt like loads (completing in issue
// order), so callers' manual waits include the stores issued after the
// accesses they wait for.  A store of more than 8 bytes reads its data
// registers after issue: a VALU write of them needs a wait state after the
// store, which the compiler does not insert for an asm statement, so the
// statement ends with two.
#ifndef FA_WS_STORE_POLICY
#define FA_WS_STORE_POLICY " nt"
#endif
__device__ __forceinline__ void st16_nt(void* sbase, uint32_t voff, const bf16x8& v) {
  asm volatile("s_nop 4\n\tglobal_store_dwordx4 %0, %1, %2" FA_WS_STORE_POLICY "\n\ts_nop 1"
               : : "v"(voff), "v"(v), "s"(sgpr_ptr(sbase)));
}

// Buffer descriptor of a raw fp32 range of `bytes` bytes at base: a read at a
// byte offset past the range returns 0 instead of touching memory.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t raw_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Direct raw-buffer->LDS copy of one fp32 per lane: lane l's value at byte
// offset voff lands at LDS byte address lds + 4*l (a zero when voff is past the
// range).  Inline assembly like dma16, with M0 likewise; ordered after the
// reads of the LDS it overwrites.
__device__ __forceinline__ void dma_buf4(rsrc_t rsrc, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 4\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}

// The same for four consecutive fp32 per lane (16 bytes, 16-byte aligned):
// lane l's values land at lds + 16*l.
__device__ __forceinline__ void dma_buf16(rsrc_t rsrc, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}

// a*b + c with a, b < 2^24 (one full-rate VALU instruction); a must fold to
// an inline constant (0 .. 64) once loops are unrolled, b is wave-uniform.
__device__ __forceinline__ uint32_t mad24(int a, uint32_t b, uint32_t c) {
  uint32_t r;
  asm("v_mad_u32_u24 %0, %1, %2, %3" : "=v"(r) : "i"(a), "s"(b), "v"(c));
  return r;
}

// Block barrier without a memory fence: LDS writes of this wave are complete
// (lgkmcnt(0)) but outstanding global->LDS copies are not waited for, so the
// copies of later tiles stay in flight across it.  Callers wait for the copies
// they need with wait_vmcnt first.
__device__ __forceinline__ void barrier_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Block barrier that waits for nothing: for a ring step whose only LDS
// accesses still in flight are reads of stages no copy refills before the next
// barrier, and whose LDS writes are older than the operand reads that later
// waits of the wave (lgkmcnt, LDS accesses complete in order) cover before the
// readers' barrier.
__device__ __forceinline__ void barrier_only() { asm volatile("s_barrier" ::: "memory"); }

// Waits for every vector memory access of this wave, as an instruction the
// compiler sees: loads the compiler issued (register operands loaded before a
// copy ring starts) are then known complete, and it places no wait of its own
// for them inside the ring's loop, where such a wait would also stall on the
// copies in flight.
__device__ __forceinline__ void wait_all_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// wait_vmcnt for a count that becomes a constant only once the slot loops
// around the call are unrolled (the instruction takes an immediate): the chain
// of tests folds to the one wait.  A count above 63 waits for 63 (more than
// asked, still sufficient).
template <int N = 0>
__device__ __forceinline__ void wait_vmcnt_n(int n) {
  if constexpr (N >= 63) {
    wait_vmcnt<63>();
  } else {
    if (n <= N)
      wait_vmcnt<N>();
    else
      wait_vmcnt_n<N + 1>(n);
  }
}

// v_mfma_f32_32x32x16_bf16 as inline assembly, with the register file of each
// operand fixed: the accumulators of long sums (dK, dV) and the stationary B
// operands (K, V rows) live in accumulation registers (AGPRs), the short-lived
// results (S, dP) and the streamed A operands in VGPRs.  The compiler's hazard
// tracking does not see inside the asm, so callers keep these rules:
//  * a result is read by anything other than the next MFMA of its own chain
//    (same accumulator, which the hardware forwards) only after mfma_drain();
//  * a VGPR written by VALU is read as an operand only after two wait states
//    (mfma_v_init has them; B operands packed by VALU are separated from their
//    MFMAs by an mfma_drain());
//  * no VALU writes a register that an MFMA in flight reads as accumulator
//    (accumulators are written only by MFMAs).
__device__ __forceinline__ void mfma_acc(f32x16& acc, const bf16x8& a, const bf16x8& b) {  // acc (AGPR) += a b
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_v0(f32x16& c, const bf16x8& a, const bf16x8& b) {  // c = a b, b in AGPRs
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_v(f32x16& c, const bf16x8& a, const bf16x8& b) {  // c += a b, b in AGPRs
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "a"(b));
}
// The first MFMA of a chain whose starting value was just written into c.
__device__ __forceinline__ void mfma_v_init(f32x16& c, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "a"(b));
}

// c = a b + seed: the first MFMA of a chain that starts from a register block
// holding its initial value (the block itself is left as it is).  The two wait
// states cover a seed written by VALU just before.
__device__ __forceinline__ void mfma_v_seed(f32x16& c, const bf16x8& a, const bf16x8& b, const f32x16& seed) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %3" : "=&v"(c) : "v"(a), "a"(b), "v"(seed));
}

// The same with a seed block that stays unchanged for the whole kernel (no
// VALU write right before the MFMA, so no wait states).
__device__ __forceinline__ void mfma_v_cseed(f32x16& c, const bf16x8& a, const bf16x8& b, const f32x16& seed) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %3" : "=&v"(c) : "v"(a), "a"(b), "v"(seed));
}

// Two floats rounded to bf16 and packed into one register here: the asm keeps
// the conversion where it is written (its pipeline slot) instead of letting it
// sink next to the first use of the vector the pair goes into.
__device__ __forceinline__ bf16x2 pack_here(float x, float y) {
  bf16x2 t = {(__bf16)x, (__bf16)y};
  asm volatile("" : "+v"(t));
  return t;
}

// Element r of a lane's C-layout block is visible iff c(r) - lb < span
// (unsigned), c(r) = 8*(r/4) + r%4.  The difference is made opaque here, in
// the element's own slot, so the compiler does not hoist the sixteen compares
// out of the loop body as lane masks held in SGPRs (which then spill).
__device__ __forceinline__ bool elem_visible(int r, int lb, uint32_t span) {
  uint32_t d = (uint32_t)(8 * (r >> 2) + (r & 3) - lb);
  asm volatile("" : "+v"(d));
  return d < span;
}

// Sixteen zero bytes in device memory: a lane whose chunk of a register-held
// row lies past a padded head dimension loads its operand from here.
static __device__ __attribute__((aligned(16))) const uint32_t kZeroChunk[4] = {0u, 0u, 0u, 0u};

// Address of chunk c (8 bf16) of a row, or of the zero chunk when c is past the
// row's n real chunks.
__device__ __forceinline__ const void* row_chunk(const __bf16* row, int c, int n) {
  return c < n ? static_cast<const void*>(row + 8 * c) : static_cast<const void*>(kZeroChunk);
}

// 16-byte global load of a register-held MFMA operand (a row chunk of K, V, Q
// or dO that stays in registers for a whole pass).  A plain load the compiler
// sees, so it tracks the load and places the wait before the first use itself
// (kernels that issue inline-assembly copies after such loads end the
// compiler's view of them with wait_all_vmem before their copy loops).
typedef const bf16x8 __attribute__((address_space(1))) global_bf16x8;
__device__ __forceinline__ bf16x8 ld16_op(const void* p) {
  return *(global_bf16x8*)(p);
}

// Wait states after the last MFMA of a group before its results are read by
// other instructions (an XDL result read by VALU, LDS or memory instructions).
// The results pass through the asm, so no read of them can be placed before it.
__device__ __forceinline__ void mfma_drain(f32x16& x, f32x16& y) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(x), "+v"(y));
}
// End of a chain whose results are next read only after a whole section of
// other MFMAs (more wait states than an XDL result needs): it keeps the two
// wait states a VALU-written B operand needs before the next section's first
// MFMA, and passes the results through the asm so that no read of them moves
// up next to the chain.
__device__ __forceinline__ void mfma_settle(f32x16& x, f32x16& y) { asm volatile("s_nop 1" : "+v"(x), "+v"(y)); }
// Eight wait states before instructions other than MFMAs read a result whose
// chain ended a few instructions earlier: with at least four instructions
// already in between, the twelve an XDL result needs are covered.
__device__ __forceinline__ void mfma_result_wait(f32x16& x) { asm volatile("s_nop 7" : "+v"(x)); }
template <int N>
__device__ __forceinline__ void mfma_drain_acc(f32x16 (&x)[N], f32x16 (&y)[N]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+a"(x[i]), "+a"(y[i]));
}
template <int N>
__device__ __forceinline__ void mfma_drain_acc(f32x16 (&x)[N]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+a"(x[i]));
}
// Values computed by VALU are materialised here: no instruction selection may
// sink their computation past this point (next to the MFMA that reads them).
__device__ __forceinline__ void materialise(bf16x8 (&x)[2], bf16x8 (&y)[2]) {
  asm volatile("" : "+v"(x[0]), "+v"(x[1]), "+v"(y[0]), "+v"(y[1]));
}
__device__ __forceinline__ void materialise(bf16x8 (&x)[2]) { asm volatile("" : "+v"(x[0]), "+v"(x[1])); }
// Makes a register block opaque here: the compiler keeps it as it is and does
// not rebuild it next to each later use.
__device__ __forceinline__ void pin(f32x16& x) { asm volatile("" : "+v"(x)); }
// Keeps a register block allocated up to this point (a use the compiler cannot
// see through), e.g. an accumulator input that an MFMA in flight still reads.
__device__ __forceinline__ void keep_live(const f32x16& x) { asm volatile("" ::"v"(x)); }

// Instruction classes of __builtin_amdgcn_sched_group_barrier.
constexpr int kSgValu = 0x002 | 0x400;  // VALU incl. transcendental
constexpr int kSgSalu = 0x004;
constexpr int kSgMfma = 0x008;
constexpr int kSgDsRead = 0x100;
constexpr int kSgDsWrite = 0x200;

// Per-lane element offset, relative to a 16-row block, of the transposed read
// that gives lane l column 32*db + l%32 and rows rb + 4*(l/32) + 0..3 of the
// block (rb = 0 for the first half of an MFMA operand, 8 for the second).
template <int D>
__device__ __forceinline__ int tr_lane_off(int lane, int db, int rb) {
  const int g = lane >> 4;        // 16-lane group
  const int s = lane & 15;        // source slot within the group
  const int r = rb + 4 * (g >> 1) + (s >> 2);       // row within the 16-row block
  const int col = 32 * db + 16 * (g & 1) + 4 * (s & 3);
  return r * D + (((col >> 3) ^ swz<D>(r)) << 3) + (col & 7);
}

}  // namespace fa
