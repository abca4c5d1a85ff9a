// FP8 forward pass with incoherent processing on gfx950.
//
// The method (marketmaker.cc page, section "FA3 : Mécanique de la trémie",
// point 3): FP8 attention is ruined by outliers unless the vectors are first
// rotated randomly, which spreads an outlier's magnitude over every
// coordinate, and then quantised per block.  The rotation here is
// R = diag(sigma) H_d / sqrt(d) (Sylvester-Hadamard H_d, random signs sigma
// passed in by the caller); R is orthogonal, so (Q R)(K R)^T = Q K^T.  Q and
// K rows are rotated, V is not; Q is also multiplied by c = scale * log2(e),
// so that its products with K are scores in base-2 units.  Every 64-row
// block of c Q R, of K R and of V gets one block scale s, the smallest power
// of two with s * 448 >= amax (448 is the largest E4M3 value; an E8M0 scale
// as in the OCP microscaling formats), and becomes E4M3(x / s).  The
// attention itself is the online-softmax forward of the 16-bit path
// ("Método", xyznot.com reading guide) on E4M3 operands: scores
// x = s_q s_k (Q8 K8^T) accumulate in fp32 on the matrix cores, which apply
// both power-of-two block scales exactly; the softmax statistics stay fp32;
// P = 2^(x - m) is rounded to E4M3 for the P V product, whose matrix
// instruction applies the value block's scale, so that
// O = sum_j E4M3(P_ij) s_v[t(j)] V8_j / l_i.
//
// Two kernels:
//   * fp8_prep_kernel: one workgroup per (Q, K or V; batch*head; 64-row
//     block).  Four lanes hold one row; the Walsh-Hadamard transform runs as
//     in-lane butterflies plus two DPP stages across the four lanes.  Q8 and
//     K8 are written row-major (rows padded to a multiple of 64 with zeros);
//     V8 is written transposed per 64-key block, [d][64], with the keys of a
//     block permuted so that each lane's slice of a row is exactly the 32
//     keys it multiplies in the P V product.  The forward runs it on K and
//     V only: fwd8_kernel prepares each query tile's Q itself, with the same
//     arithmetic (and so the same codes).
//   * fwd8_kernel: the 16-bit forward's grid and causal / block-sparse tile
//     skipping, 64-key K and V^T tiles in a three-slot LDS ring filled by
//     direct global->LDS copies, S^T = K Q^T and O^T += V^T P^T on
//     v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 x E4M3, the block scales as the
//     instruction's E8M0 scale operands, fp32 accumulation).  The score
//     accumulators start at -m (the running reference), so the matrix core
//     also subtracts it and the exponentials take the accumulators as they
//     are.  Lane l holds query l % 32 at 16 keys of each 32-key unit, which
//     are exactly its 32 contraction slots of the P V product over the
//     tile's 64 keys: P goes from the score accumulators to the operand with
//     no shuffle.
#include <type_traits>

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr float kE4M3Max = 448.f;

template <int V>
using ic = std::integral_constant<int, V>;

// c + (2^(ea-127) A)(2^(eb-127) B): formats 0/0, both operands E4M3; ea and eb
// are E8M0 exponents (byte 0 of the scale operands), the same for every lane.
__device__ __forceinline__ f32x16 mfma_f8(i32x8 a, i32x8 b, f32x16 c, int ea, int eb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, ea, 0, eb);
}

// The smallest power of two s >= amax / 448 (so that |x| / s <= 448 for the
// block), at least 2^-126; 1 for an all-zero block.  With amax = f 2^E,
// f in [0.5, 1), and 448 = 0.875 * 2^9: 448 * 2^k >= amax holds from
// k = E - 9 when f <= 0.875 and from k = E - 8 otherwise; f <= 0.875 is the
// stored mantissa of amax <= 0.75 * 2^23.
__device__ __forceinline__ float pow2_block_scale(float amax) {
  if (!(amax > 0.f)) return 1.f;
  const uint32_t b = __float_as_uint(amax);
  const int eb = (int)(b >> 23);           // biased exponent: E = eb - 126
  int k = eb - 135 + ((b & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  if (eb == 0 || k < -126) k = -126;       // subnormal or tiny amax
  return __uint_as_float((uint32_t)(k + 127) << 23);
}

// E8M0 exponent of a power-of-two scale (its biased fp32 exponent).
__device__ __forceinline__ int e8m0_of(float s) { return (int)(__float_as_uint(s) >> 23); }

// Four fp32 values to four E4M3 bytes (a in the lowest byte).  The
// conversion rounds to nearest even; it does not saturate, so every caller
// keeps |x| <= 448.
// Each conversion replaces one 16-bit half of its `old` operand; the low half
// is written first over a's own bits, so no zeroed register is needed.
__device__ __forceinline__ int pack_e4m3(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __float_as_int(a), false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

__device__ __forceinline__ float quad_xor1(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float quad_xor2(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));
}

// XOR swizzle of 16-byte chunks in LDS tiles with rows of RB bytes, for
// reads of 16 consecutive rows at one chunk per pass.
template <int RB>
__device__ __forceinline__ int swz8(int r) {
  if constexpr (RB == 64) return (r >> 2) & 3;
  else return (r >> 1) & 7;
}

// Key (within a 64-key block) held at position p of the transposed V block:
// position 32 g + e is the e-th contraction slot of lanes g = l / 32.
__device__ __forceinline__ int vt_key(int pos) {
  const int g = pos >> 5, e = pos & 31;
  return 32 * (e >> 4) + 8 * ((e & 15) >> 2) + 4 * g + (e & 3);
}

template <typename T, int D>
__global__ __launch_bounds__(256) void fp8_prep_kernel(Fp8Params p) {
  using VT = typename V8<T>::t;
  constexpr int EPT = D / 4;        // elements per lane (four lanes per row)
  __shared__ float red[4];
  // V code tile row stride in LDS (bytes): with it the dword writes below
  // meet at most two lanes per bank and the column reads none (64 banks).
  constexpr int RSB = D + (D == 64 ? 12 : 4);
  __shared__ __attribute__((aligned(16))) uint8_t vtile[64 * RSB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int z = blockIdx.y + p.prep_z0;   // 0 = Q, 1 = K, 2 = V
  const int nt = p.n_t64;
  const int bh = blockIdx.x / nt, t = blockIdx.x - bh * nt;
  const int row = tid >> 2, qd = tid & 3;
  const int N = p.N;
  const int key = t * 64 + row;
  const T* src = (const T*)(z == 0 ? p.q : (z == 1 ? p.k : p.v));

  float x[EPT];
  if (key < N) {
    const T* rp = src + ((size_t)bh * N + key) * D + qd * EPT;
#pragma unroll
    for (int c = 0; c < EPT / 8; ++c) {
      const VT v8 = *(const VT*)(rp + 8 * c);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[8 * c + e] = (float)v8[e];
    }
  } else {
#pragma unroll
    for (int e = 0; e < EPT; ++e) x[e] = 0.f;
  }

  if (z < 2 && p.signs != nullptr) {
    // x <- (x * sigma) H_d / sqrt(d); element index = qd * EPT + e, so the
    // low bits of the index are in-lane and the two high bits are qd.
#pragma unroll
    for (int e = 0; e < EPT; ++e)
      if (p.signs[qd * EPT + e] < 0) x[e] = -x[e];
#pragma unroll
    for (int h = 1; h < EPT; h *= 2)
#pragma unroll
      for (int i = 0; i < EPT; ++i)
        if ((i & h) == 0) {
          const float a = x[i], b = x[i + h];
          x[i] = a + b;
          x[i + h] = a - b;
        }
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const float y = quad_xor1(x[e]);
      x[e] = (qd & 1) ? y - x[e] : x[e] + y;
    }
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const float y = quad_xor2(x[e]);
      x[e] = (qd & 2) ? y - x[e] : x[e] + y;
    }
    const float rs = z == 0 ? p.rsqrt_d * p.scale_log2e : p.rsqrt_d;
#pragma unroll
    for (int e = 0; e < EPT; ++e) x[e] *= rs;
  } else if (z == 0) {
#pragma unroll
    for (int e = 0; e < EPT; ++e) x[e] *= p.scale_log2e;
  }

  // Block amax over the 64 rows.
  float am = 0.f;
#pragma unroll
  for (int e = 0; e < EPT; ++e) am = fmaxf(am, fabsf(x[e]));
  am = wave_max(am);
  if (lane == 0) red[wave] = am;
  __syncthreads();
  am = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float bs = pow2_block_scale(am);
  const float inv = __uint_as_float((uint32_t)(254 - e8m0_of(bs)) << 23);   // 1 / bs, exact
  if (tid == 0) {
    float* sc = z == 0 ? p.sq : (z == 1 ? p.sk : p.sv);
    sc[(size_t)bh * nt + t] = bs;
  }

  int w[EPT / 4];
#pragma unroll
  for (int i = 0; i < EPT / 4; ++i) {
    float y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = fminf(fmaxf(x[4 * i + e] * inv, -kE4M3Max), kE4M3Max);
    w[i] = pack_e4m3(y[0], y[1], y[2], y[3]);
  }
  if (z < 2) {
    uint8_t* dst = (z == 0 ? p.q8 : p.k8) + ((size_t)bh * p.Npad + key) * D + qd * EPT;
#pragma unroll
    for (int i = 0; i < EPT / 16; ++i)
      *(i32x4*)(dst + 16 * i) = i32x4{w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]};
    return;
  }
  // V: transpose the block through LDS into [d][64 positions] (rows padded
  // to RSB bytes).
  // Each thread moves 4 x 4 byte blocks: the four keys of positions
  // 4j .. 4j+3 (consecutive keys) at columns 4dq .. 4dq+3, read as four
  // dwords and transposed with byte permutes into one dword per column.
#pragma unroll
  for (int i = 0; i < EPT / 4; ++i) *(int*)(vtile + row * RSB + qd * EPT + 4 * i) = w[i];
  __syncthreads();
  uint8_t* dst0 = p.v8t + ((size_t)bh * nt + t) * (64 * D);
#pragma unroll
  for (int kq = 0; kq < D / 64; ++kq) {
    const int P = tid + 256 * kq, j = P & 15, dq = P >> 4;
    const int k0 = vt_key(4 * j);
    uint32_t r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = *(const uint32_t*)(vtile + (k0 + i) * RSB + 4 * dq);
    // perm(S0, S1, sel): bytes 0-3 of S1, 4-7 of S0.
    const uint32_t a01l = __builtin_amdgcn_perm(r[1], r[0], 0x05010400u);  // r0b0 r1b0 r0b1 r1b1
    const uint32_t a01h = __builtin_amdgcn_perm(r[1], r[0], 0x07030602u);  // r0b2 r1b2 r0b3 r1b3
    const uint32_t a23l = __builtin_amdgcn_perm(r[3], r[2], 0x05010400u);
    const uint32_t a23h = __builtin_amdgcn_perm(r[3], r[2], 0x07030602u);
    uint8_t* o = dst0 + (size_t)(4 * dq) * 64 + 4 * j;
    *(uint32_t*)(o) = __builtin_amdgcn_perm(a23l, a01l, 0x05040100u);        // column 4dq
    *(uint32_t*)(o + 64) = __builtin_amdgcn_perm(a23l, a01l, 0x07060302u);   // 4dq + 1
    *(uint32_t*)(o + 128) = __builtin_amdgcn_perm(a23h, a01h, 0x05040100u);  // 4dq + 2
    *(uint32_t*)(o + 192) = __builtin_amdgcn_perm(a23h, a01h, 0x07060302u);  // 4dq + 3
  }
}

template <typename T, int D, bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(256, fwd8_waves(D)) void fwd8_kernel(Fp8Params p) {
  using HT = typename V8<T>::h;
  using VT = typename V8<T>::t;
  constexpr int NW = 4, BR = 128, BC = 64, NS = 3;
  constexpr int TB = BC * D;                 // bytes of a K tile (and of a V^T tile)
  constexpr int DH = D / 64;                 // score MFMAs per 32-key unit
  constexpr int DB = D / 32;                 // O^T row blocks
  constexpr int CPR = D / 16;                // 16-byte chunks per K row
  constexpr int DMA_N = TB / 16 / 256;       // copies per wave per tile
  constexpr int OPS = 2 * DMA_N + 1;         // copies per wave per tile (+ its two block scales)
  static_assert(BR == MASK_TILE, "a workgroup covers one block-mask row");
  __shared__ __attribute__((aligned(1024))) uint8_t kvs[2 * NS * TB];  // K slots, then V^T slots
  // Block scales of the tile in each slot: [0] its K scale, [1] its V scale
  // (lanes 2.. of the copy repeat them).
  __shared__ __attribute__((aligned(16))) float sc_s[NS][64];
  __shared__ float qam_s[NW];   // Q amax of each wave's 32 rows
  __shared__ uint8_t mask_s[SPARSE ? FWD_MAX_MASK_TILES : 1];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, l32 = lane & 31;
  const int N = p.N, nt = p.n_t64;
  const int n_qt = (N + BR - 1) / BR;
  int bh, qt;
  if (CAUSAL) {
    int rank;
    causal_tile(blockIdx.x, p.BH, n_qt, bh, rank);
    qt = n_qt - 1 - rank;
  } else {
    const int lid = xcd_remap(blockIdx.x, n_qt * p.BH);
    bh = lid / n_qt;
    qt = lid - bh * n_qt;
    // Block-sparse: the 16-bit forward's work order (most visible key tiles
    // first), for the same L2 reuse.
    if (SPARSE && p.qt_order != nullptr) qt = p.qt_order[qt];
  }
  const uint8_t* __restrict__ K8 = p.k8 + (size_t)bh * p.Npad * D;
  const uint8_t* __restrict__ V8 = p.v8t + (size_t)bh * nt * TB;
  const float* __restrict__ skh = p.sk + (size_t)bh * nt;
  const float* __restrict__ svh = p.sv + (size_t)bh * nt;
  const int q0w = qt * BR + wave * 32;

  if (SPARSE) {
    for (int i = tid; i < p.mask_tiles; i += 256) mask_s[i] = p.mask[(size_t)qt * p.mask_tiles + i];
    __syncthreads();
  }

  // Per-lane LDS byte offsets.  K (A operand of S^T): key 32 u + l32, bytes
  // 64 h + 32 g .. + 31.  V^T (A operand of O^T): row 32 db + l32, bytes
  // 32 g .. + 31 (positions = the lane's contraction slots).
  int koff[2][DH][2], voff[DB][2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int h = 0; h < DH; ++h)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int r = 32 * u + l32, ch = 4 * h + 2 * g + c;
        koff[u][h][c] = r * D + 16 * (ch ^ swz8<D>(r));
      }
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int r = 32 * db + l32, ch = 2 * g + c;
      voff[db][c] = TB * NS + r * 64 + 16 * (ch ^ swz8<64>(r));
    }
  // Copy schedule: copy u of this wave fills physical chunk pch of a tile.
  uint32_t kdo[DMA_N], vdo[DMA_N];
#pragma unroll
  for (int u = 0; u < DMA_N; ++u) {
    const int pch = (u * NW + wave) * 64 + lane;
    const int kr = pch / CPR, kc = (pch % CPR) ^ swz8<D>(kr);
    kdo[u] = (uint32_t)(kr * D + 16 * kc);
    const int vr = pch >> 2, vc = (pch & 3) ^ swz8<64>(vr);
    vdo[u] = (uint32_t)(vr * 64 + 16 * vc);
  }
  const uint32_t lds0 = lds_addr(kvs);

  const int n_kt = (N + BC - 1) / BC;
  int kt_end = n_kt;
  if (CAUSAL) kt_end = min(kt_end, (min(N, (qt + 1) * BR) + BC - 1) / BC);
  auto next_active = [&](int jj) {
    if (SPARSE)
      while (jj < kt_end && mask_s[(jj * BC) / MASK_TILE] == 0) ++jj;
    return jj;
  };
  const int last_key = CAUSAL ? min(N - 1, q0w + 31) : N - 1;
  const int plain_key = CAUSAL ? min(N - 1, q0w) : N - 1;

  // Copy K tile jj, V^T tile jj and their two block scales into slot `slot`
  // (rows past N are zero in both tiles: the preparation pads them).  The
  // scales travel with the tiles, so the wait that makes a tile visible
  // covers them too.
  auto issue = [&](int jj, auto slc) __attribute__((always_inline)) {
    constexpr int slot = decltype(slc)::value;
    const uint8_t* ks = K8 + (size_t)jj * TB;
    const uint8_t* vs = V8 + (size_t)jj * TB;
    const uint32_t kd = lds0 + (uint32_t)(slot * TB), vd = lds0 + (uint32_t)((NS + slot) * TB);
#pragma unroll
    for (int u = 0; u < DMA_N; ++u) dma16_s(ks, kdo[u], kd + (uint32_t)((u * NW + wave) * 1024));
#pragma unroll
    for (int u = 0; u < DMA_N; ++u) dma16_s(vs, vdo[u], vd + (uint32_t)((u * NW + wave) * 1024));
    dma4((lane & 1) ? svh + jj : skh + jj, lds_addr(&sc_s[slot][0]));
  };


  // Q^T (B operand): lane holds query q = q0w + l32, elements 64 h + 32 g
  // .. + 31 of c Q R, rotated and quantised here from the 16-bit rows with
  // the preparation kernel's arithmetic: the same sign flips, butterflies in
  // the same order of element-index bits (0-4 in the lane, 5 across the two
  // lane halves, 6 across h), the same factors and block scale (the 64-row
  // block is this wave and its neighbour), so the codes are the ones
  // fa_fp8_prepare writes for Q.
  // The rows are loaded before the first tile copies are issued, so that
  // waiting for them leaves the copies in flight.
  i32x8 qf[DH];
  int eq;
  VT qraw[DH][4];
  i32x8 sgn[DH];
  {
    const int q = q0w + l32;
    const T* qr = (const T*)p.q + ((size_t)bh * N + min(q, N - 1)) * D + 32 * g;
#pragma unroll
    for (int h = 0; h < DH; ++h)
#pragma unroll
      for (int c = 0; c < 4; ++c) qraw[h][c] = *(const VT*)(qr + 64 * h + 8 * c);
    if (p.signs != nullptr) {
#pragma unroll
      for (int h = 0; h < DH; ++h) sgn[h] = *(const i32x8*)(p.signs + 64 * h + 32 * g);
    }
  }
  int jq[NS];
  jq[0] = next_active(0);
  jq[1] = jq[0] < kt_end ? next_active(jq[0] + 1) : kt_end;
  jq[2] = jq[1] < kt_end ? next_active(jq[1] + 1) : kt_end;
  if (jq[0] < kt_end) issue(jq[0], ic<0>{});
  if (jq[1] < kt_end) issue(jq[1], ic<1>{});
  {
    const bool live = q0w + l32 < N;
    float x[DH][32];
#pragma unroll
    for (int h = 0; h < DH; ++h)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        // Packed pairs (elements 8c + 2i, 8c + 2i + 1); rows past N are zero.
        u32x4 w = __builtin_bit_cast(u32x4, qraw[h][c]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint32_t pr = live ? w[i] : 0u;
          if (p.signs != nullptr) {
            // Sign bytes of the pair (bytes 2(i%2), 2(i%2)+1 of dword (8c+2i)/4)
            // onto the pair's two sign bits: an exact negation.
            const uint32_t sw = (uint32_t)sgn[h][2 * c + i / 2];
            const uint32_t m = __builtin_amdgcn_perm(0u, sw, (i & 1) ? 0x030c020cu : 0x010c000cu);
            pr ^= m & 0x80008000u;
          }
          const uint16_t lo = (uint16_t)pr, hi = (uint16_t)(pr >> 16);
          x[h][8 * c + 2 * i] = (float)__builtin_bit_cast(T, lo);
          x[h][8 * c + 2 * i + 1] = (float)__builtin_bit_cast(T, hi);
        }
      }
    if (p.signs != nullptr) {
#pragma unroll
      for (int hs = 1; hs < 32; hs *= 2)
#pragma unroll
        for (int h = 0; h < DH; ++h)
#pragma unroll
          for (int i = 0; i < 32; ++i)
            if ((i & hs) == 0) {
              const float a = x[h][i], b = x[h][i + hs];
              x[h][i] = a + b;
              x[h][i + hs] = a - b;
            }
      // Element-index bit 5 is the lane half: the swap hands every lane the
      // low half's value (a) and the high half's (b) of its pair.
#pragma unroll
      for (int h = 0; h < DH; ++h)
#pragma unroll
        for (int e = 0; e < 32; ++e) {
          const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x[h][e]),
                                                          __float_as_uint(x[h][e]), false, false);
          const float a = __uint_as_float(r[0]), b = __uint_as_float(r[1]);
          x[h][e] = g ? a - b : a + b;
        }
      if constexpr (DH == 2) {
#pragma unroll
        for (int e = 0; e < 32; ++e) {
          const float a = x[0][e], b = x[1][e];
          x[0][e] = a + b;
          x[1][e] = a - b;
        }
      }
      const float rs = p.rsqrt_d * p.scale_log2e;
#pragma unroll
      for (int h = 0; h < DH; ++h)
#pragma unroll
        for (int e = 0; e < 32; ++e) x[h][e] *= rs;
    } else {
#pragma unroll
      for (int h = 0; h < DH; ++h)
#pragma unroll
        for (int e = 0; e < 32; ++e) x[h][e] *= p.scale_log2e;
    }
    float am = 0.f;
#pragma unroll
    for (int h = 0; h < DH; ++h)
#pragma unroll
      for (int e = 0; e < 32; ++e) am = fmaxf(am, fabsf(x[h][e]));
    am = wave_max(am);
    if (lane == 0) qam_s[wave] = am;
    lds_reads_done();   // the write above has completed
    wg_barrier();
    am = fmaxf(qam_s[wave & 2], qam_s[(wave & 2) | 1]);
    const float bs = pow2_block_scale(am);
    const float inv = __uint_as_float((uint32_t)(254 - e8m0_of(bs)) << 23);   // 1 / bs, exact
    eq = e8m0_of(bs);
#pragma unroll
    for (int h = 0; h < DH; ++h)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = fminf(fmaxf(x[h][4 * i + e] * inv, -kE4M3Max), kE4M3Max);
        qf[h][i] = pack_e4m3(y[0], y[1], y[2], y[3]);
      }
  }
  wait_all_loads();

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  // Running reference m (base-2 score units) and this lane's share of
  // sum 2^(x - m).  The score accumulators start at -m (negm), so each MFMA
  // chain ends holding x - m.  No reference exists until a query's first
  // visible key: while its sum is 0 every tile takes the reference step.
  float m_run = 0.f, l_run = 0.f;
  f32x16 negm = f32x16{};
  // Opaque to the compiler, so that it keeps the 16 registers instead of
  // rebuilding the splat before every tile.
  asm volatile("" : "+v"(negm));

  // One tile; the ring slot is a compile-time constant (the loop below is
  // unrolled over the three slots), so every LDS address folds into an
  // instruction's offset.
  auto iter = [&](auto slc) __attribute__((always_inline)) {
    constexpr int slot = decltype(slc)::value;
    const int j = jq[0];
    if (jq[1] < kt_end) wait_vmcnt<OPS>();
    else wait_vmcnt<0>();
    wg_barrier();
    if (jq[2] < kt_end) issue(jq[2], ic<(slot + NS - 1) % NS>{});
    if (j * BC <= last_key) {
      const uint8_t* kt = kvs + slot * TB;
      const uint8_t* vt = kvs + slot * TB;   // V^T offsets already include NS * TB
      const float2 sc = *(const float2*)&sc_s[slot][0];
      const int ek = e8m0_of(sc.x), ev = e8m0_of(sc.y);
      f32x16 s[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int h = 0; h < DH; ++h) {
          const i32x4 lo = *(const i32x4*)(kt + koff[u][h][0]);
          const i32x4 hi = *(const i32x4*)(kt + koff[u][h][1]);
          const i32x8 kf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          s[u] = mfma_f8(kf, qf[h], h == 0 ? negm : s[u], ek, eq);
        }
      }
      // Scores past this lane's last visible key become -inf.
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int ks = j * BC + 32 * u;
        if (ks + 31 > plain_key) {
          const int lim = min(N - 1, CAUSAL ? q0w + l32 : N - 1) - ks - 4 * g;
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (8 * (r >> 2) + (r & 3) > lim) s[u][r] = -INFINITY;
        }
      }
      i32x8 pk;
      // P = 2^(x - m), packed to E4M3; returns the lane's sum of P.
      auto exps = [&]() {
        float ls0, ls1;  // start at the first terms, not at 0
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int w4 = 0; w4 < 4; ++w4) {
            float e[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) e[b] = fast_exp2(s[u][4 * w4 + b]);
            const bool first = u == 0 && w4 == 0;
            ls0 = first ? e[0] + e[1] : ls0 + (e[0] + e[1]);
            ls1 = first ? e[2] + e[3] : ls1 + (e[2] + e[3]);
            pk[4 * u + w4] = pack_e4m3(e[0], e[1], e[2], e[3]);
            // Pinned here: otherwise the compiler sinks the packs past the
            // reference check (the rare path recomputes them) and keeps the
            // 32 fp32 values alive across it, 20 more VGPRs.
            if constexpr (FA_FP8_PIN_PACKS) asm volatile("" ::"v"(pk[4 * u + w4]));
          }
        return ls0 + ls1;
      };
      float ls = exps();
      // The reference moves only when some lane's tile sum exceeds 2^8 (so
      // every packed value stays below 448) or some query has no reference
      // yet; O, l and lse share it.  Both lanes of a query (l, l ^ 32) take
      // the same step: max over the query's scores of the tile, x - m.
      if (wave_any(!(ls <= 256.f) || l_run == 0.f)) {
        float mx = s[0][0];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[u][r]);
        mx = half_swap_max(mx);
        // A query with earlier terms only moves up; a fresh one moves to its
        // tile max (if it has a visible key here), and its O and l are 0.
        const bool fresh = half_swap_sum(l_run) == 0.f;
        const float step = fresh ? (mx > -INFINITY ? mx : 0.f) : fmaxf(mx, 0.f);
        const float alpha = fresh ? 0.f : fast_exp2(-step);
        m_run += step;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] *= alpha;
#pragma unroll
        for (int r = 0; r < 16; ++r) negm[r] = -m_run;
        asm volatile("" : "+v"(negm));
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[u][r] -= step;
        ls = exps();
      }
      l_run += ls;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const i32x4 lo = *(const i32x4*)(vt + voff[db][0]);
        const i32x4 hi = *(const i32x4*)(vt + voff[db][1]);
        o[db] = mfma_f8(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), pk, o[db], ev, 127);
      }
    }
    jq[0] = jq[1];
    jq[1] = jq[2];
    jq[2] = jq[1] < kt_end ? next_active(jq[1] + 1) : kt_end;
  };
  static_assert(NS == 3, "the loop below unrolls three slots");
  while (jq[0] < kt_end) {
    iter(ic<0>{});
    if (jq[0] >= kt_end) break;
    iter(ic<1>{});
    if (jq[0] >= kt_end) break;
    iter(ic<2>{});
  }

  // Epilogue: O = O / l, lse = (m + log2 l) * ln 2.
  const float lt = half_swap_sum(l_run);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const int q = q0w + l32;
  if (q < N) {
    T* orow = (T*)p.o + ((size_t)bh * N + q) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        HT hv;
#pragma unroll
        for (int e = 0; e < 4; ++e) hv[e] = (T)(o[db][4 * rg + e] * inv);
        *(HT*)(orow + 32 * db + 8 * rg + 4 * g) = hv;
      }
    if (g == 0)
      p.lse[(size_t)bh * N + q] = lt > 0.f ? (m_run + __log2f(lt)) * 0.69314718055994531f : -INFINITY;
  }
}

template <typename T, int D>
hipError_t launch_fp8_t(const Fp8Params& p, bool causal, bool sparse, bool prep, bool attend,
                        hipStream_t st) {
  if (prep) {
    hipLaunchKernelGGL((fp8_prep_kernel<T, D>), dim3((unsigned)(p.BH * p.n_t64), 3 - p.prep_z0),
                       dim3(256), 0, st, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || !attend) return e;
  }
  const dim3 grid((unsigned)(((p.N + 127) / 128) * p.BH)), block(256);
  if (causal && sparse) hipLaunchKernelGGL((fwd8_kernel<T, D, true, true>), grid, block, 0, st, p);
  else if (causal) hipLaunchKernelGGL((fwd8_kernel<T, D, true, false>), grid, block, 0, st, p);
  else if (sparse) hipLaunchKernelGGL((fwd8_kernel<T, D, false, true>), grid, block, 0, st, p);
  else hipLaunchKernelGGL((fwd8_kernel<T, D, false, false>), grid, block, 0, st, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fp8(Fp8Params p, int dtype, int d, bool causal, bool prep, bool attend,
                      hipStream_t st) {
  const bool sparse = p.mask != nullptr;
  if (dtype == DT_BF16)
    return d == 64 ? launch_fp8_t<__bf16, 64>(p, causal, sparse, prep, attend, st)
                   : launch_fp8_t<__bf16, 128>(p, causal, sparse, prep, attend, st);
  return d == 64 ? launch_fp8_t<_Float16, 64>(p, causal, sparse, prep, attend, st)
                 : launch_fp8_t<_Float16, 128>(p, causal, sparse, prep, attend, st);
}

}  // namespace fa
