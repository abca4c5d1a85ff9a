// Device-side helpers shared by the gfx950 attention kernels.
//
// Matrix-core conventions (checked on the device before these kernels were
// written).  For v_mfma_f32_32x32x16_{bf16,f16}, C[32x32] += A[32x16] B[16x32]:
//   A operand, lane l: row i = l % 32, elements e = 0..7 -> k = 8 * (l / 32) + e
//   B operand, lane l: col j = l % 32, elements e = 0..7 -> k = 8 * (l / 32) + e
//   C/D, lane l, register r = 0..15: col j = l % 32,
//        row i = 8 * (r / 4) + 4 * (l / 32) + r % 4
// For v_mfma_f32_16x16x32_{bf16,f16}, C[16x16] += A[16x32] B[32x16]: A lane l
// holds row l % 16, k = 8 * (l / 16) + e; B lane l holds column l % 16, same k;
// C lane l, register r = 0..3: column l % 16, row 4 * (l / 16) + r.
// For v_mfma_f32_32x32x2_f32: A lane l holds A[l % 32][l / 32], B lane l holds
// B[l / 32][l % 32], same C layout.
// The contraction index only has to be paired the same way in A and B, so
// kernels are free to assign any k order to (l / 32, e) as long as both
// operands agree.
//
// ds_read_b64_tr_b16 (LDS transpose read), per group of 16 lanes: if lane s
// of the group points at 4 consecutive 16-bit elements, lane t of the group
// receives element (t % 4) of the rows pointed to by lanes t/4, t/4+4, t/4+8,
// t/4+12.  With lane s pointing at X[kb + s/4][nb + 4*(s%4)] of a row-major
// matrix X, lane t receives X[kb + 0..3][nb + t]: a column of four
// consecutive rows, which is the operand layout an MFMA needs when the
// contraction runs along X's rows.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <typename T> struct V8;
template <> struct V8<__bf16> { typedef bf16x8 t; typedef bf16x4 h; typedef bf16x2 p; };
template <> struct V8<_Float16> { typedef f16x8 t; typedef f16x4 h; typedef f16x2 p; };

// Round two fp32 values to one packed pair (round to nearest even).
template <typename T>
__device__ __forceinline__ unsigned pack2(float a, float b) {
  typename V8<T>::p v = {(T)a, (T)b};
  return __builtin_bit_cast(unsigned, v);
}

// acc + x.lo + x.hi for a packed pair, accumulated in fp32.
__device__ __forceinline__ float sum2_acc(unsigned x, float acc, __bf16) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x), one, acc, false);
}
__device__ __forceinline__ float sum2_acc(unsigned x, float acc, _Float16) {
  const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, x), one, acc, false);
}

// ---- LDS address helpers, direct global->LDS copies and explicit waits ----
//
// global_load_lds_dwordx4 copies 16 bytes per lane from global memory into
// LDS at (M0 + 16 * lane): each wave fills one contiguous 1 KiB block whose
// base is wave-uniform.  It is issued from inline assembly so that the
// compiler neither counts it nor inserts its own conservative waits; the
// kernels wait for it explicitly with s_waitcnt vmcnt(n) (vector-memory
// operations complete in issue order) and publish it to the other waves with
// a workgroup barrier.

// Byte address of a __shared__ object as the LDS instructions see it.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)(p);
}

__device__ __forceinline__ void dma16(const void* gsrc, uint32_t lds_wave_base) {
  // M0 is an input operand, so the compiler sets it and knows it is used.
  asm volatile("global_load_lds_dwordx4 %0, off"
               :
               : "v"(gsrc), "{m0}"(__builtin_amdgcn_readfirstlane(lds_wave_base)));
}

// Same copy with a wave-uniform 64-bit base in SGPRs and a per-lane 32-bit
// byte offset (no per-lane address arithmetic).
__device__ __forceinline__ void dma16_s(const void* sbase, uint32_t voff, uint32_t lds_wave_base) {
  asm volatile("global_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "{m0}"(__builtin_amdgcn_readfirstlane(lds_wave_base)));
}

// Streaming variants: the same copies with the non-temporal cache policy, for
// data each call reads exactly once (a decode scan over the key/value
// history).  Keeping such lines out of the way of reused data lets a
// streaming read run closer to the HBM rate than the default policy does.
__device__ __forceinline__ void dma16_stream(const void* gsrc, uint32_t lds_wave_base) {
  asm volatile("global_load_lds_dwordx4 %0, off nt"
               :
               : "v"(gsrc), "{m0}"(__builtin_amdgcn_readfirstlane(lds_wave_base)));
}
__device__ __forceinline__ void dma16_s_stream(const void* sbase, uint32_t voff,
                                               uint32_t lds_wave_base) {
  asm volatile("global_load_lds_dwordx4 %0, %1 nt"
               :
               : "v"(voff), "s"(sbase), "{m0}"(__builtin_amdgcn_readfirstlane(lds_wave_base)));
}

// 4-byte-per-lane variant: lane l's dword lands at lds_wave_base + 4 * l.
__device__ __forceinline__ void dma4(const void* gsrc, uint32_t lds_wave_base) {
  asm volatile("global_load_lds_dword %0, off"
               :
               : "v"(gsrc), "{m0}"(__builtin_amdgcn_readfirstlane(lds_wave_base)));
}

// Wait until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// Compiler-visible wait for every outstanding vector-memory load of this
// wave (vmcnt(0), other counters untouched).  Used once after the prologue's
// ordinary loads so the compiler's own wait tracking sees them complete and
// inserts no wait inside the copy-pipelined loop.
__device__ __forceinline__ void wait_all_loads() { __builtin_amdgcn_s_waitcnt(0xF70); }

// Wait until this wave's LDS reads (and other LDS/scalar-memory operations)
// have completed; no LDS access is moved across it by the compiler.  Used
// before a direct copy overwrites LDS the same wave has just read.
__device__ __forceinline__ void lds_reads_done() { asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory"); }

// Workgroup barrier without the memory fence of __syncthreads(): LDS
// accesses are not moved across it by the compiler, and no wait on
// outstanding global loads is added.
__device__ __forceinline__ void wg_barrier() {
  asm volatile("" : : : "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" : : : "memory");
}

// XOR swizzle of 16-byte chunks within an LDS row of D 16-bit elements.  For
// both the 16-byte row reads (16 lanes, 16 consecutive rows, one chunk) and
// the transpose reads (32 lanes, 4 consecutive rows x 32 columns) every lane
// of a pass hits a different bank.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 64) return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  else return ((r & 3) << 2) | ((r >> 2) & 3);
}
// Element offset of logical (row, col) in a swizzled tile with rows of D.
template <int D>
__device__ __forceinline__ int swz_off(int r, int col) {
  return r * D + 8 * ((col >> 3) ^ swz<D>(r)) + (col & 7);
}

// Instruction-scheduling hint for the straight-line block emitted just
// before it: NM matrix-core ops, the first preceded by LEAD LDS reads, each
// followed by RPM more LDS reads and VPM vector-ALU ops.  It only orders
// independent instructions (data dependences still hold), so that a wave
// issues vector work while its own matrix products are in flight.
template <int NM, int LEAD, int RPM, int VPM>
__device__ __forceinline__ void sched_interleave() {
#ifndef FA_NO_SCHED_HINTS
  if constexpr (LEAD > 0) __builtin_amdgcn_sched_group_barrier(0x100, LEAD, 0);
#pragma unroll
  for (int i = 0; i < NM; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (RPM > 0) __builtin_amdgcn_sched_group_barrier(0x100, RPM, 0);
    if constexpr (VPM > 0) __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);
  }
#endif
}

// Materialise a pair of 16-bit MFMA operands at this point: an empty
// volatile asm that reads and writes them, so the arithmetic producing them
// is not sunk past a later branch (into another scheduling region).
template <typename VT>
__device__ __forceinline__ void keep_here(VT (&x)[2]) {
  asm volatile("" : "+v"(x[0]), "+v"(x[1]));
}

// True if `pred` holds on any active lane of the wave.
__device__ __forceinline__ bool wave_any(bool pred) { return __builtin_amdgcn_ballot_w64(pred) != 0; }

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32x32x16(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x32(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32x32x2(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Transpose read of four 16-bit values (see the header comment).
__device__ __forceinline__ i16x4 lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

template <typename VT>
__device__ __forceinline__ VT cat_tr16(i16x4 lo, i16x4 hi) {
  i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(VT, v);
}

// Reductions across the two 32-lane halves of a wave: every lane gets the
// combination of its own value and the value of lane (l ^ 32).
__device__ __forceinline__ float half_swap_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// Max over all 64 lanes, in every lane: two DPP quad permutes, the half-row
// and row mirrors (max within 16 lanes), then a swap of neighbouring 16-lane
// rows and of the two 32-lane halves (no LDS traffic).
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, true)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, true)));
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  return half_swap_max(x);
}
__device__ __forceinline__ float half_swap_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- Dropout mask: Philox-4x32-10 over 4 x 4 (query, key) blocks ----
//
// Philox-4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC 2011): ten rounds of
//   (x0, x1, x2, x3) <- (hi(M1 x2) ^ x1 ^ k0, lo(M1 x2), hi(M0 x0) ^ x3 ^ k1, lo(M0 x0))
// with the key advanced by the Weyl constants between rounds.  Element
// (query i, key j) of head bh uses byte j % 4 of word i % 4 of the output at
// counter (j / 4, i / 4, bh, offset), key (seed_lo, seed_hi); it is kept iff
// that byte is >= the threshold t = round(256 p).
__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                              uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    // Three-input XORs, one v_bitop3_b32 each (truth table 0x96 = a ^ b ^ c).
    const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);
    const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
  }
  return u32x4{c0, c1, c2, c3};
}

__device__ __forceinline__ uint32_t quad_swap1(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, true);  // lanes l ^ 1
}
__device__ __forceinline__ uint32_t quad_swap2(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, true);  // lanes l ^ 2
}

// Transpose across the four lanes of a quad: lane w ends with r[t] = the
// r[w] that quad lane t held (two exchange stages, lane bits 0 and 1).
__device__ __forceinline__ void quad_transpose4(uint32_t (&r)[4], int w) {
#pragma unroll
  for (int b = 1; b <= 2; b <<= 1) {
    const bool hi = (w & b) != 0;
#pragma unroll
    for (int j0 = 0; j0 < 4; ++j0) {
      if (j0 & b) continue;
      const int j1 = j0 | b;
      // Value selects with unconditional stores keep r in registers.
      const uint32_t a = r[j0], c = r[j1];
      const uint32_t send = hi ? a : c;
      const uint32_t recv = b == 1 ? quad_swap1(send) : quad_swap2(send);
      r[j0] = hi ? recv : a;
      r[j1] = hi ? c : recv;
    }
  }
}

// In-lane transpose of the 4 x 4 byte matrix held in r (word w, byte b ->
// word b, byte w).
__device__ __forceinline__ void byte_transpose4(uint32_t (&r)[4]) {
  uint32_t o[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    o[b] = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) o[b] |= ((r[w] >> (8 * b)) & 0xFFu) << (8 * w);
  }
#pragma unroll
  for (int b = 0; b < 4; ++b) r[b] = o[b];
}

// Keep bytes for a lane that holds one query and the 16 keys
// ks + 8 t + 4 g + e (t, e = 0..3) of a 32-key unit (the S^T layout):
// word t, byte e.  Each lane of a quad computes one Philox call (the 4 x 4
// block of its quad's queries and key group t = its quad index) and the quad
// exchanges words.
__device__ __forceinline__ void drop_words_query_lane(uint32_t (&c)[4], int ks, int q0, int l32,
                                                      int g, uint32_t bh, uint32_t off,
                                                      uint32_t k0, uint32_t k1) {
  const int w = l32 & 3;
  const u32x4 r = philox4x32_10((uint32_t)(ks / 4 + 2 * w + g), (uint32_t)((q0 + l32) / 4), bh,
                                off, k0, k1);
#pragma unroll
  for (int i = 0; i < 4; ++i) c[i] = r[i];
  quad_transpose4(c, w);
}

// Keep bytes for a lane that holds one key and the 16 queries
// qb + 8 t + 4 g + e of a 32-query unit (the S layout): word t, byte e.
__device__ __forceinline__ void drop_words_key_lane(uint32_t (&c)[4], int qb, int k0w, int l32,
                                                    int g, uint32_t bh, uint32_t off,
                                                    uint32_t k0, uint32_t k1) {
  const int w = l32 & 3;
  const u32x4 r = philox4x32_10((uint32_t)((k0w + l32) / 4), (uint32_t)(qb / 4 + 2 * w + g), bh,
                                off, k0, k1);
#pragma unroll
  for (int i = 0; i < 4; ++i) c[i] = r[i];
  byte_transpose4(c);
  quad_transpose4(c, w);
}

__device__ __forceinline__ bool drop_keep(const uint32_t (&c)[4], int r, uint32_t t8) {
  return ((c[r >> 2] >> (8 * (r & 3))) & 0xFFu) >= t8;
}

// The keep decisions of the four bytes of w (byte i kept iff byte_i >= t8)
// as masks for two packed 16-bit pairs: lo = bytes 0, 1 -> halves 0xFFFF or
// 0, hi = bytes 2, 3.  Byte-parallel compare: bit 7 of byte i of
// ((w & 0x7F..) | 0x80..) - (t8 & 0x7F) * 0x01.. is (byte_i & 0x7F) >= (t8 & 0x7F)
// (no borrow crosses a byte); combined with the byte's own top bit it gives
// byte_i >= t8.  v_perm's sign selectors (8..11: bit 7 of bytes 1, 3, 5, 7
// of {S0, S1}) spread the four flags into 16-bit halves.
__device__ __forceinline__ void drop_masks16(uint32_t w, uint32_t t8, uint32_t& lo, uint32_t& hi) {
  const uint32_t d = ((w & 0x7F7F7F7Fu) | 0x80808080u) - (t8 & 0x7Fu) * 0x01010101u;
  const uint32_t ge = (t8 & 0x80u) ? (w & d) : (w | d);  // bit 8i+7: byte i kept
  const uint32_t ge8 = ge << 8;                          // bit 8i+15: byte i kept
  lo = __builtin_amdgcn_perm(ge8, ge, 0x08080A0Au);      // [b0, b0, b1, b1]
  hi = __builtin_amdgcn_perm(ge8, ge, 0x09090B0Bu);      // [b2, b2, b3, b3]
}

// The same decisions as four 32-bit masks (0xFFFFFFFF where byte i is
// kept), for selecting fp32 values with an AND: no compare, no branch.
__device__ __forceinline__ void drop_masks32(uint32_t w, uint32_t t8, uint32_t (&m)[4]) {
  const uint32_t d = ((w & 0x7F7F7F7Fu) | 0x80808080u) - (t8 & 0x7Fu) * 0x01010101u;
  const uint32_t ge = (t8 & 0x80u) ? (w & d) : (w | d);
  const uint32_t ge8 = ge << 8;
  m[0] = __builtin_amdgcn_perm(ge8, ge, 0x0A0A0A0Au);
  m[1] = __builtin_amdgcn_perm(ge8, ge, 0x08080808u);
  m[2] = __builtin_amdgcn_perm(ge8, ge, 0x0B0B0B0Bu);
  m[3] = __builtin_amdgcn_perm(ge8, ge, 0x09090909u);
}

__device__ __forceinline__ float and_bits(float x, uint32_t m) {
  return __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, x) & m);
}

// Workgroup index -> logical tile index.  The hardware hands consecutive
// workgroup ids to the 8 XCDs round robin; this mapping gives each XCD a
// contiguous range of logical ids so tiles of one head share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int total) {
  constexpr int NX = 8;
  const int x = bid % NX, r = bid / NX;
  const int per = total / NX, rem = total % NX;
  return (x < rem) ? x * (per + 1) + r : rem * (per + 1) + (x - rem) * per + r;
}

// Causal work order: workgroup id -> (head, rank), rank k being each head's
// k-th longest tile.  Ranks run longest first (a list schedule in order of
// decreasing work) and each XCD works on as few heads as an even split of
// the work allows.  The hardware deals ids to the 8 XCDs round robin, so
// XCD x runs ids 8r + x in order of r.  With P = 8 / gcd(BH, 8) ranks per
// period, the BH*P tiles of a period go to the XCDs head-major, Q = BH*P/8
// consecutive (head, rank) pairs each: whole heads when BH is a multiple of
// 8, one head and alternate ranks of a second for 12 heads, instead of
// every head on every XCD.  The ranks past the last whole period (the
// shortest tiles) take the heads round robin.
__device__ __forceinline__ void causal_tile(int bid, int BH, int n_rank, int& bh, int& rank) {
  const int low = BH & -BH;
  const int P = 8 / (low < 8 ? low : 8);  // 1, 2, 4 or 8
  const int Q = BH * P / 8;
  const int periods = n_rank / P;
  const int n_full = periods * P * BH;
  if (bid < n_full) {
    const int x = bid & 7, r = bid >> 3;
    const int period = r / Q, t = x * Q + (r - period * Q);
    bh = t / P;
    rank = period * P + (t - bh * P);
  } else {
    const int b = bid - n_full;
    bh = b % BH;
    rank = periods * P + b / BH;
  }
}

}  // namespace fa
