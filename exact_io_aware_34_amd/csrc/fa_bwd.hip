// Backward pass of exact attention on gfx950 (fp16 / bf16 inputs).
//
// The pages fix the principle: the N x N probabilities are not stored; the
// backward pass recomputes S and P tile by tile from Q, K and the saved
// softmax statistic ("Passe arrière : recalculer au lieu de stocker",
// marketmaker.cc; "Recomputação no Backward Pass", xyznot.com reading guide).
// The gradient formulas are the softmax chain rule (not printed on the pages):
//   P = exp(scale*QK^T - lse),  dV = P^T dO,  dP = dO V^T,
//   D_i = sum_c dO_ic O_ic,  dS = P o (dP - D),  dQ = scale dS K,  dK = scale dS^T Q.
//
// Two kernels, no atomics, dQ first:
//   bwd_dkdv_u: one workgroup per (key tile of 128, batch*head).  Wave w owns
//     32 keys, keeps their K and V rows as MFMA operands and dK, dV in fp32
//     accumulators, and streams the 64-row query tiles that can see them
//     (causal: tiles at or after the key tile; block-sparse: set entries)
//     through an LDS ring filled by direct global->LDS copies (Q and dO tiles
//     swizzled; the tile's statistics in a separate small array).  S = Q K^T
//     and dP = dO V^T run on v_mfma_f32_32x32x16 with the key in the lane, so
//     P^T and dS^T for dV += P^T dO and dK += dS^T Q come straight from the
//     accumulators; dO and Q are read again with ds_read_b64_tr_b16.
//   bwd_dq_u: one workgroup per (query tile of 128, batch*head), the
//     forward's layout: S^T = K Q^T and dP^T = V dO^T with the query in the
//     lane (so the statistic and D are per-lane scalars), dS^T in registers,
//     and dQ^T += K^T dS^T with K read transposed; dQ is stored once.  Its
//     prologue computes each row's D = rowsum(dO o O) from the dO and O rows
//     it loads anyway, and stores -D and the log2-domain statistic
//     lse * log2(e) (+inf for rows with no visible key, so P = 0 there) into
//     the workspace for bwd_dkdv_u, launched after it.
// Recomputing S, P, dP in both kernels costs two extra products per score,
// instead of the global atomic adds a single-pass dQ would need (those
// execute at memory on this part and moved more bytes than the pass computes).
#include <type_traits>

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

template <int V>
using ic = std::integral_constant<int, V>;

// ---- unit-pipelined kernels (d = 64: 2 waves per SIMD; d = 128: 1) ----
//
// Both kernels cut their streamed dimension into 32-row units, two per
// 64-row tile, and run one block per unit in which the matrix products of
// the neighbouring units (recomputed S and dP of unit u+1, the gradient
// products of unit u-1) are issued beside the element-wise work of unit u
// (P = exp2(S c - lse2), dS = P (dP - D)).  A block has no branch, so one
// wave keeps the matrix cores and the vector ALUs busy at once.  Masked
// units (causal diagonal, rows past N, units outside a wave's range) get
// S = -inf before their element-wise work, so their P and dS are exactly 0.

// dK, dV: one workgroup per (128-key tile, batch*head); wave w owns 32 keys
// (K, V rows as MFMA operands in VGPRs, dK and dV accumulators) and streams
// 64-row Q / dO tiles plus their statistics through a 4-slot LDS ring, copies
// issued two tiles ahead.
template <typename T, int D, bool CAUSAL, bool SPARSE, bool DROP>
__global__ __launch_bounds__(256, dkdv_waves(D)) void bwd_dkdv_u_kernel(BwdParams p) {
  using VT = typename V8<T>::t;
  // Ring slots: four (copies two tiles ahead), or three (one tile ahead) when
  // three workgroups share a CU's LDS.
  constexpr int NW = 4, BC = NW * 32, QT = 64, NS = dkdv_waves(D) == 3 ? 3 : 4;
  constexpr int DS = D / 16, DB = D / 32, CPR = D / 8;
  constexpr int TILE = QT * D;                   // elements of one Q (or dO) tile
  constexpr int DMA_N = QT * CPR / 256;          // 16-byte copies per wave per tile
  constexpr int OPS = 2 * DMA_N + 1;             // copies per wave per tile (+ statistics)
  constexpr int STAGE = 2 * TILE;
  static_assert(BC == MASK_TILE, "a key tile is one block-mask column");
  static_assert(QT == 64, "statistics: one 64-lane dword copy per quantity");
  // Slot s: Q tile at [s*STAGE], dO tile at [s*STAGE + TILE] (64 KiB in all,
  // so every slot offset fits an LDS instruction's immediate), and 4 x 64
  // floats in st_s[s]: lse2 of the tile's rows, D of its rows (written by
  // waves 0 and 1; waves 2 and 3 write the same again, so every wave issues
  // the same copies).
  __shared__ __attribute__((aligned(1024))) T lds[NS * STAGE];
  __shared__ __attribute__((aligned(16))) float st_s[NS][NW * 64];
  __shared__ uint8_t mask_s[SPARSE ? FWD_MAX_MASK_TILES : 1];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, l32 = lane & 31, s16 = lane & 15, gq = lane >> 4;
  const int N = p.N;
  const int n_kt = (N + BC - 1) / BC;
  int bh, j;
  if (SPARSE) {
    // Heads in XCD-aware runs as below; within a head, key tiles with the
    // most visible query tiles first (the order of sparse_order_kernel).
    const int lid = xcd_remap(blockIdx.x, n_kt * p.BH);
    bh = lid / n_kt;
    j = p.kt_order[lid - bh * n_kt];
  } else if (CAUSAL) {
    // Key tiles with the most query tiles (small j) first, few heads per XCD.
    causal_tile(blockIdx.x, p.BH, n_kt, bh, j);
  } else {
    const int lid = xcd_remap(blockIdx.x, n_kt * p.BH);
    bh = lid / n_kt;
    j = lid - bh * n_kt;
  }
  const size_t base = (size_t)bh * N * D;
  const T* __restrict__ Q = (const T*)p.q + base;
  const T* __restrict__ K = (const T*)p.k + base;
  const T* __restrict__ V = (const T*)p.v + base;
  const T* __restrict__ dO = (const T*)p.dO + base;
  const float* __restrict__ L2 = p.lse2 + (size_t)bh * N;
  const float* __restrict__ NDEL = p.neg_delta + (size_t)bh * N;
  const int k0 = j * BC, kw0 = k0 + 32 * wave, my_k = kw0 + l32;
  const float c = p.scale_log2e;

  if (SPARSE) {
    for (int i = tid; i < p.mask_tiles; i += 256) mask_s[i] = p.mask[(size_t)i * p.mask_tiles + j];
    __syncthreads();
  }

  // Per-lane element offsets in a swizzled tile (rows = queries): A-operand
  // row reads and B-operand transpose reads; 16-row steps fold into the
  // immediate offset.
  int aoff[DS], boff[DB][2];
#pragma unroll
  for (int ds = 0; ds < DS; ++ds) aoff[ds] = swz_off<D>(l32, 16 * ds + 8 * g);
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      boff[db][h] = swz_off<D>(4 * g + (s16 >> 2) + 8 * h, 32 * db + 16 * (gq & 1) + 4 * (s16 & 3));
  uint32_t doff[DMA_N];
  int drow[DMA_N];
#pragma unroll
  for (int u = 0; u < DMA_N; ++u) {
    const int pch = (u * NW + wave) * 64 + lane;
    const int r = pch / CPR, cc = (pch % CPR) ^ swz<D>(r);
    drow[u] = r;
    doff[u] = (uint32_t)((r * D + 8 * cc) * (int)sizeof(T));
  }
  const uint32_t lds0 = lds_addr(lds);

  const int i_end = (N + QT - 1) / QT;
  const int i_beg = CAUSAL ? k0 / QT : 0;
  auto next_active = [&](int i) __attribute__((always_inline)) {
    if (SPARSE)
      while (i < i_end && mask_s[(i * QT) / MASK_TILE] == 0) ++i;
    return i;
  };
  // Copy query tile i (Q, dO, statistics) into slot `slot`.  Rows past N read
  // row N - 1; their scores are masked, so they contribute nothing.
  auto issue = [&](int i, int slot) __attribute__((always_inline)) {
    const int qa = i * QT;
    const uint32_t qd = lds0 + (uint32_t)(slot * STAGE * (int)sizeof(T));
    const uint32_t od = qd + (uint32_t)(TILE * (int)sizeof(T));
    const uint32_t sd = lds_addr(&st_s[slot][wave * 64]);
    if (qa + QT <= N) {
      const T* qb_ = Q + (size_t)qa * D;
      const T* ob_ = dO + (size_t)qa * D;
#pragma unroll
      for (int u = 0; u < DMA_N; ++u) {
        const uint32_t wo = (uint32_t)((u * NW + wave) * 64 * 16);
        dma16_s(qb_, doff[u], qd + wo);
        dma16_s(ob_, doff[u], od + wo);
      }
    } else {
#pragma unroll
      for (int u = 0; u < DMA_N; ++u) {
        const uint32_t wo = (uint32_t)((u * NW + wave) * 64 * 16);
        const size_t go = (size_t)min(qa + drow[u], N - 1) * D +
                          (doff[u] / (int)sizeof(T) - drow[u] * D);
        dma16(Q + go, qd + wo);
        dma16(dO + go, od + wo);
      }
    }
    const int qs = min(qa + lane, N - 1);
    dma4((wave & 1) ? NDEL + qs : L2 + qs, sd);
  };

  VT kf[DS], vf[DS];
  int iq[NS];  // active query tiles n .. n+NS-1 (i_end past the last one)
  iq[0] = next_active(i_beg);
#pragma unroll
  for (int t = 1; t < NS; ++t) iq[t] = iq[t - 1] < i_end ? next_active(iq[t - 1] + 1) : i_end;
#pragma unroll
  for (int t = 0; t < NS - 1; ++t)
    if (iq[t] < i_end) issue(iq[t], t);
#pragma unroll
  for (int ds = 0; ds < DS; ++ds) {
    kf[ds] = my_k < N ? *(const VT*)(K + (size_t)my_k * D + 16 * ds + 8 * g) : VT{};
    vf[ds] = my_k < N ? *(const VT*)(V + (size_t)my_k * D + 16 * ds + 8 * g) : VT{};
  }

  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }

  // S = Q K^T and dP = dO V^T of half h of the tile in slot SL: lane = key,
  // register r = query 32h + 8(r/4) + 4g + r%4 of the tile.  Without
  // dropout the dP accumulator starts at -D of its query row, so it ends
  // holding dP - D, the factor dS needs.
  auto sdp = [&](int slot, int h, f32x16& s, f32x16& dp) __attribute__((always_inline)) {
    const T* qt_ = lds + slot * STAGE + 32 * h * D;
    s = f32x16{};
    if constexpr (DROP) {
      dp = f32x16{};
    } else {
      const float* nd = &st_s[slot][QT + 32 * h];
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const float4 v4 = *(const float4*)(nd + 8 * rg + 4 * g);
        dp[4 * rg] = v4.x;
        dp[4 * rg + 1] = v4.y;
        dp[4 * rg + 2] = v4.z;
        dp[4 * rg + 3] = v4.w;
      }
    }
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      s = mfma32x32x16(*(const VT*)(qt_ + aoff[ds]), kf[ds], s);
      dp = mfma32x32x16(*(const VT*)(qt_ + TILE + aoff[ds]), vf[ds], dp);
    }
  };
  // dV += P^T dO and dK += dS^T Q for half h of the tile in slot SL.
  auto grads = [&](int slot, int h, const VT (&pa)[2], const VT (&dsa)[2]) __attribute__((always_inline)) {
    const T* qt_ = lds + slot * STAGE + 32 * h * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const VT dof = cat_tr16<VT>(lds_read_tr16(qt_ + TILE + 16 * kk * D + boff[db][0]),
                                    lds_read_tr16(qt_ + TILE + 16 * kk * D + boff[db][1]));
        dv[db] = mfma32x32x16(pa[kk], dof, dv[db]);
        const VT qfr = cat_tr16<VT>(lds_read_tr16(qt_ + 16 * kk * D + boff[db][0]),
                                    lds_read_tr16(qt_ + 16 * kk * D + boff[db][1]));
        dk[db] = mfma32x32x16(dsa[kk], qfr, dk[db]);
      }
  };
  // P and dS of half h of the tile in slot SL, rounded to 16-bit operands;
  // dp holds dP - D (see sdp).  With dropout it holds dP, and (queries
  // qb + 8t + 4g + e of the unit, this lane's key) P^T for dV keeps only the
  // kept probabilities (1 / (1 - p) is applied to dV at the end) and
  // dS = P o (Z dP / (1 - p) - D).
  auto pds = [&](int slot, int h, int qb, const f32x16& s, const f32x16& dp, VT (&pa)[2],
                 VT (&dsa)[2]) __attribute__((always_inline)) {
    const float* sf = &st_s[slot][32 * h];
    uint32_t dwk[4];
    if constexpr (DROP)
      drop_words_key_lane(dwk, qb, kw0, l32, g, (uint32_t)bh, p.drop_off, p.drop_k0, p.drop_k1);
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const float4 l4 = *(const float4*)(sf + 8 * rg + 4 * g);
      const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
      float nd[4] = {};                                    // -D (dropout only)
      if constexpr (DROP) {
        const float4 d4 = *(const float4*)(sf + QT + 8 * rg + 4 * g);
        nd[0] = d4.x;
        nd[1] = d4.y;
        nd[2] = d4.z;
        nd[3] = d4.w;
      }
      float pv[4], dsv[4];
      uint32_t km[4];  // keep masks of elements 4 rg .. 4 rg + 3 (dropout only)
      if constexpr (DROP) drop_masks32(dwk[rg], p.drop_t8, km);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pv[e] = fast_exp2(fmaf(s[4 * rg + e], c, -lv[e]));
        if constexpr (DROP) {
          // Selections as ANDs with the keep masks (a ternary here was
          // compiled to a branch per element).
          dsv[e] = pv[e] * (and_bits(dp[4 * rg + e] * p.drop_scale, km[e]) + nd[e]);
          pv[e] = and_bits(pv[e], km[e]);
        } else {
          dsv[e] = pv[e] * dp[4 * rg + e];
        }
      }
      const int kk = rg >> 1, w0 = 2 * (rg & 1);
      u32x4 pw = __builtin_bit_cast(u32x4, pa[kk]);
      u32x4 dw = __builtin_bit_cast(u32x4, dsa[kk]);
      pw[w0] = pack2<T>(pv[0], pv[1]);
      pw[w0 + 1] = pack2<T>(pv[2], pv[3]);
      dw[w0] = pack2<T>(dsv[0], dsv[1]);
      dw[w0 + 1] = pack2<T>(dsv[2], dsv[3]);
      pa[kk] = __builtin_bit_cast(VT, pw);
      dsa[kk] = __builtin_bit_cast(VT, dw);
    }
  };
  // Query q sees key my_k iff q >= my_k (causal) and q < N; S = -inf
  // elsewhere.  Units entirely before this wave's keys are masked whole.
  auto mask_unit = [&](int qa, f32x16& s) __attribute__((always_inline)) {
    if ((CAUSAL && qa <= kw0) || qa + 32 > N) {
      const int first = CAUSAL ? my_k : 0;  // first visible query
      // Visible iff first <= q < N: one unsigned compare and a select per
      // element (the two-sided test was compiled to branches).
      const unsigned span = (unsigned)(N - first);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int q = qa + 8 * (r >> 2) + 4 * g + (r & 3);
        s[r] = (unsigned)(q - first) < span ? s[r] : -INFINITY;
      }
    }
  };
  // One block: the gradient products of unit u-1 beside the element-wise
  // work of unit u, then S and dP of unit u+1 (issued last, so the scores of
  // units u and u+1 are not both live while the vector work runs).
  auto block = [&](int rslc, int gslc, int eslc, int h, int he, int qb, f32x16& s_cur,
                   f32x16& dp_cur, f32x16& s_nxt, f32x16& dp_nxt, const VT (&pa_p)[2],
                   const VT (&ds_p)[2], VT (&pa_c)[2], VT (&ds_c)[2]) __attribute__((always_inline)) {
    grads(gslc, h, pa_p, ds_p);
    pds(eslc, he, qb, s_cur, dp_cur, pa_c, ds_c);
    sdp(rslc, h, s_nxt, dp_nxt);
    keep_here(pa_c);
    keep_here(ds_c);
  };

  // Units are numbered along the active query tiles, two per tile.  Block u
  // issues S, dP of unit u+1 and the gradient products of unit u-1 beside the
  // element-wise work of unit u.  Iteration n runs blocks 2n+1 and 2n+2: it
  // reads tiles n and n+1, which must have landed; every wave has finished
  // with tile n-1, whose slot receives tile n+3.
  f32x16 s_odd, dp_odd, s_even, dp_even;
  VT pa_odd[2], ds_odd[2], pa_even[2], ds_even[2];
  if (iq[0] < i_end) {
    if (NS == 4 && iq[2] < i_end) wait_vmcnt<2 * OPS>();
    else if (iq[1] < i_end) wait_vmcnt<OPS>();
    else wait_vmcnt<0>();
    wg_barrier();
    // Block 0: S, dP of units 0 and 1, P and dS of unit 0.
    sdp(0, 0, s_even, dp_even);
    mask_unit(iq[0] * QT, s_even);
    sdp(0, 1, s_odd, dp_odd);
    pds(0, 0, iq[0] * QT, s_even, dp_even, pa_even, ds_even);
  }
  // K, V rows and the statistics were ordinary loads: drain them here, where
  // the compiler sees it, so that it places no vmcnt wait (which would also
  // wait for the copies in flight) at their first use inside the loop.
  wait_all_loads();
  // One iteration; the slot is a run-time index (four unrolled copies with
  // constant slots need more registers than the occupancy allows).  MASKED
  // iterations apply the edge masks; the others are branch-free between
  // their two blocks.
  int sl = 0;  // slot of tile n
  auto iteration = [&](auto masked_c) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_c)::value;
    const int SL = sl, SL1 = sl == NS - 1 ? 0 : sl + 1;  // slots of tiles n, n+1
    const int i = iq[0], i1 = iq[1];
    // Tile n+1 has landed once at most tile n+2's copies are in flight (four
    // slots; with three, tile n+2 is issued below).
    if (NS == 4 && iq[2] < i_end) wait_vmcnt<OPS>();
    else wait_vmcnt<0>();
    wg_barrier();
    // Tile n+NS-1 into the slot of tile n-1, which every wave has finished.
    if (iq[NS - 1] < i_end) issue(iq[NS - 1], SL == 0 ? NS - 1 : SL - 1);
    // Units 2n+1 (second half of tile n) and 2n+2 (first half of tile n+1;
    // past the last tile it is masked whole and never used).
    if constexpr (MASKED) mask_unit(i * QT + 32, s_odd);
    block(SL1, SL, SL, 0, 1, i * QT + 32, s_odd, dp_odd, s_even, dp_even, pa_even, ds_even, pa_odd,
          ds_odd);
    if constexpr (MASKED) mask_unit(i1 < i_end ? i1 * QT : N, s_even);
    block(SL1, SL, SL1, 1, 0, i1 * QT, s_even, dp_even, s_odd, dp_odd, pa_odd, ds_odd, pa_even,
          ds_even);
#pragma unroll
    for (int t = 0; t < NS - 1; ++t) iq[t] = iq[t + 1];
    iq[NS - 1] = iq[NS - 2] < i_end ? next_active(iq[NS - 2] + 1) : i_end;
    sl = SL1;
  };
  // Iterations needing no mask (units 2n+1, 2n+2 past the causal diagonal
  // and inside N) form one contiguous run: masked ones come before it
  // (causal diagonal) and after it (row tail).
  auto interior = [&]() __attribute__((always_inline)) {
    return (!CAUSAL || iq[0] * QT + 32 > kw0) && iq[1] < i_end && iq[1] * QT + 32 <= N;
  };
  while (iq[0] < i_end && !interior()) iteration(std::true_type{});
  while (iq[0] < i_end && interior()) iteration(std::false_type{});
  while (iq[0] < i_end) iteration(std::true_type{});

  // dK = scale * sum dS^T Q, dV = sum P^T dO; lane: column d, register r: key.
  float* __restrict__ dK = p.dk + base;
  float* __restrict__ dV = p.dv + base;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kw0 + 8 * (r >> 2) + 4 * g + (r & 3);
      if (key < N) {
        dK[(size_t)key * D + 32 * db + l32] = dk[db][r] * p.scale;
        dV[(size_t)key * D + 32 * db + l32] = DROP ? dv[db][r] * p.drop_scale : dv[db][r];
      }
    }
}

// dQ: one workgroup per (128-query tile, batch*head), query in the lane as in
// the forward.  64-key K and V tiles stream through two LDS rings (K: 4
// slots, V: 3), copies issued two tiles ahead.  S^T = K Q^T and
// dP^T = V dO^T take Q and dO from VGPRs; dQ^T += K^T dS^T reads K
// transposed.
template <typename T, int D, bool CAUSAL, bool SPARSE, bool DROP>
__global__ __launch_bounds__(256, bwd_u_waves(D)) void bwd_dq_u_kernel(BwdParams p) {
  using VT = typename V8<T>::t;
  constexpr int NW = 4, BR = NW * 32, BC = 64, NK = 4, NV = 3;
  constexpr int DS = D / 16, DB = D / 32, CPR = D / 8;
  constexpr int TILE = BC * D;                 // elements of one K (or V) tile
  constexpr int DMA_N = BC * CPR / 256;        // copies per wave per tile
  static_assert(BR == MASK_TILE, "a query tile is one block-mask row");
  // K slot s at [s*TILE], V slot s at [(NK+s)*TILE]; rows swizzled.
  __shared__ __attribute__((aligned(1024))) T kvs[(NK + NV) * TILE];
  __shared__ uint8_t mask_s[SPARSE ? FWD_MAX_MASK_TILES : 1];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, l32 = lane & 31, s16 = lane & 15, gq = lane >> 4;
  const int N = p.N;
  const int n_qt = (N + BR - 1) / BR;
  int bh, qt;
  if (SPARSE) {
    // Heads in XCD-aware runs; within a head, query tiles with the most
    // visible key tiles first (sparse_order_kernel).
    const int lid = xcd_remap(blockIdx.x, n_qt * p.BH);
    bh = lid / n_qt;
    qt = p.qt_order[lid - bh * n_qt];
  } else if (CAUSAL) {
    int rank;
    causal_tile(blockIdx.x, p.BH, n_qt, bh, rank);
    qt = n_qt - 1 - rank;
  } else {
    const int lid = xcd_remap(blockIdx.x, n_qt * p.BH);
    bh = lid / n_qt;
    qt = lid - bh * n_qt;
  }
  const size_t base = (size_t)bh * N * D;
  const T* __restrict__ Q = (const T*)p.q + base;
  const T* __restrict__ K = (const T*)p.k + base;
  const T* __restrict__ V = (const T*)p.v + base;
  const T* __restrict__ dO = (const T*)p.dO + base;
  const int q0 = qt * BR + wave * 32;
  const int my_q = q0 + l32;
  const float c = p.scale_log2e;

  if (SPARSE) {
    for (int i = tid; i < p.mask_tiles; i += 256) mask_s[i] = p.mask[(size_t)qt * p.mask_tiles + i];
    __syncthreads();
  }

  int koff[DS], toff[DB][2];
#pragma unroll
  for (int ds = 0; ds < DS; ++ds) koff[ds] = swz_off<D>(l32, 16 * ds + 8 * g);
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      toff[db][h] = swz_off<D>(4 * g + (s16 >> 2) + 8 * h, 32 * db + 16 * (gq & 1) + 4 * (s16 & 3));
  uint32_t doff[DMA_N];
  int drow[DMA_N];
#pragma unroll
  for (int u = 0; u < DMA_N; ++u) {
    const int pch = (u * NW + wave) * 64 + lane;
    const int r = pch / CPR, cc = (pch % CPR) ^ swz<D>(r);
    drow[u] = r;
    doff[u] = (uint32_t)((r * D + 8 * cc) * (int)sizeof(T));
  }
  const uint32_t lds0 = lds_addr(kvs);

  const int n_kt = (N + BC - 1) / BC;
  int kt_end = n_kt;
  if (CAUSAL) kt_end = min(kt_end, (min(N, (qt + 1) * BR) + BC - 1) / BC);
  auto next_active = [&](int jj) __attribute__((always_inline)) {
    if (SPARSE)
      while (jj < kt_end && mask_s[(jj * BC) / MASK_TILE] == 0) ++jj;
    return jj;
  };
  // Keys past last_key are invisible to every query of this wave.
  const int last_key = CAUSAL ? min(N - 1, q0 + 31) : N - 1;

  // Copy tile jj of K (or V) into slot `slot` of its ring.  Rows past N read
  // row N - 1; their scores are masked, so they contribute nothing.
  auto issue = [&](const T* src, int jj, uint32_t dst_slot) __attribute__((always_inline)) {
    const int k0 = jj * BC;
    const uint32_t dst = lds0 + dst_slot * (uint32_t)(TILE * (int)sizeof(T));
    if (k0 + BC <= N) {
      const T* sb = src + (size_t)k0 * D;
#pragma unroll
      for (int u = 0; u < DMA_N; ++u)
        dma16_s(sb, doff[u], dst + (uint32_t)((u * NW + wave) * 64 * 16));
    } else {
#pragma unroll
      for (int u = 0; u < DMA_N; ++u) {
        const size_t go = (size_t)min(k0 + drow[u], N - 1) * D +
                          (doff[u] / (int)sizeof(T) - drow[u] * D);
        dma16(src + go, dst + (uint32_t)((u * NW + wave) * 64 * 16));
      }
    }
  };

  int jq[NK];  // active key tiles n .. n+3 (kt_end past the last one)
  jq[0] = next_active(0);
#pragma unroll
  for (int t = 1; t < NK; ++t) jq[t] = jq[t - 1] < kt_end ? next_active(jq[t - 1] + 1) : kt_end;
  // Prologue copies K0 V0 K1 V1 K2 V2; iteration n copies K(n+3), V(n+3).
#pragma unroll
  for (int t = 0; t < 3; ++t)
    if (jq[t] < kt_end) {
      issue(K, jq[t], t);
      issue(V, jq[t], NK + t);
    }
  VT qf[DS], dof[DS];
#pragma unroll
  for (int ds = 0; ds < DS; ++ds) {
    qf[ds] = my_q < N ? *(const VT*)(Q + (size_t)my_q * D + 16 * ds + 8 * g) : VT{};
    dof[ds] = my_q < N ? *(const VT*)(dO + (size_t)my_q * D + 16 * ds + 8 * g) : VT{};
  }
  // Row statistics of this lane's query: D = sum_c dO_c O_c (this lane holds
  // half of the row, lane ^ 32 the other half) and lse * log2(e), +inf where
  // lse = -inf (no visible key) and on padding rows, so that P = 0 there.
  // Lanes 0..31 also store -D and the log2 statistic for the dK/dV kernel,
  // which runs after this one.  With dropout O is read in fp32: its kept
  // terms carry 1/(1 - p), and on a row with one visible key
  // dS = P (dP/(1 - p) - D) cancels exactly only if D does not carry O's
  // rounding to 16 bits.
  float dpart = 0.f;
  if constexpr (DROP) {
    const float* __restrict__ OA = p.o_acc + base;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
      if (my_q < N) {
        a = *(const float4*)(OA + (size_t)my_q * D + 16 * ds + 8 * g);
        b = *(const float4*)(OA + (size_t)my_q * D + 16 * ds + 8 * g + 4);
      }
      const float ov[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) dpart = fmaf(ov[e], (float)dof[ds][e], dpart);
    }
  } else {
    const T* __restrict__ O = (const T*)p.o + base;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      const VT of = my_q < N ? *(const VT*)(O + (size_t)my_q * D + 16 * ds + 8 * g) : VT{};
#pragma unroll
      for (int e = 0; e < 8; ++e) dpart = fmaf((float)of[e], (float)dof[ds][e], dpart);
    }
  }
  const float nd_row = -half_swap_sum(dpart);  // -D
  const float lse_q = my_q < N ? p.lse[(size_t)bh * N + my_q] : -INFINITY;
  const float lq = lse_q == -INFINITY ? INFINITY : lse_q * kLog2e;
  if (g == 0 && my_q < N) {
    p.neg_delta[(size_t)bh * N + my_q] = nd_row;
    p.lse2[(size_t)bh * N + my_q] = lq;
  }

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};

  // S^T = K Q^T and dP^T = V dO^T of half h of K slot KS / V slot VS: lane =
  // query, register r = key 32h + 8(r/4) + 4g + r%4 of the tile.
  auto sdp = [&](int kslot, int vslot, int h, f32x16& s, f32x16& dp) __attribute__((always_inline)) {
    const T* kt = kvs + kslot * TILE + 32 * h * D;
    const T* vt = kvs + (NK + vslot) * TILE + 32 * h * D;
    s = f32x16{};
    dp = f32x16{};
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      s = mfma32x32x16(*(const VT*)(kt + koff[ds]), qf[ds], s);
      dp = mfma32x32x16(*(const VT*)(vt + koff[ds]), dof[ds], dp);
    }
  };
  // dQ^T += K^T dS^T for half h of K slot KS (K read transposed).
  auto dqacc = [&](int kslot, int h, const VT (&dsf)[2]) __attribute__((always_inline)) {
    const T* kt = kvs + kslot * TILE + 32 * h * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const VT ktf = cat_tr16<VT>(lds_read_tr16(kt + 16 * kk * D + toff[db][0]),
                                    lds_read_tr16(kt + 16 * kk * D + toff[db][1]));
        acc[db] = mfma32x32x16(ktf, dsf[kk], acc[db]);
      }
  };
  // dS^T = P^T o (dP^T - D) with P = exp2(S c - lse2), rounded to 16 bits.
  // With dropout (keys ks + 8t + 4g + e of the unit): dS = P o (Z dP / (1 - p) - D).
  auto dscores = [&](int ks, const f32x16& s, const f32x16& dp, VT (&dsf)[2]) __attribute__((always_inline)) {
    uint32_t dwq[4];
    if constexpr (DROP)
      drop_words_query_lane(dwq, ks, q0, l32, g, (uint32_t)bh, p.drop_off, p.drop_k0, p.drop_k1);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 8 * h + 2 * e;
        const float p0 = fast_exp2(fmaf(s[r], c, -lq));
        const float p1 = fast_exp2(fmaf(s[r + 1], c, -lq));
        float d0 = dp[r], d1 = dp[r + 1];
        if constexpr (DROP) {
          d0 = drop_keep(dwq, r, p.drop_t8) ? d0 * p.drop_scale : 0.f;
          d1 = drop_keep(dwq, r + 1, p.drop_t8) ? d1 * p.drop_scale : 0.f;
        }
        w[e] = pack2<T>(p0 * (d0 + nd_row), p1 * (d1 + nd_row));
      }
      dsf[h] = __builtin_bit_cast(VT, w);
    }
  };
  // Keys past this lane's last visible key (causal diagonal, keys >= N)
  // become -inf; a unit past the wave's range is masked whole.
  auto mask_unit = [&](int ks, f32x16& s) __attribute__((always_inline)) {
    if ((CAUSAL && ks + 31 > q0) || ks + 32 > N) {
      const int lim = min(N - 1, CAUSAL ? my_q : N - 1) - ks - 4 * g;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        s[r] = 8 * (r >> 2) + (r & 3) > lim ? -INFINITY : s[r];
    }
  };
  auto block = [&](int kslc, int vslc, int gslc, int h, int ks, f32x16& s_cur, f32x16& dp_cur,
                   f32x16& s_nxt, f32x16& dp_nxt, const VT (&ds_p)[2], VT (&ds_c)[2]) __attribute__((always_inline)) {
    sdp(kslc, vslc, h, s_nxt, dp_nxt);
    dqacc(gslc, h, ds_p);
    dscores(ks, s_cur, dp_cur, ds_c);
    if constexpr (D == 64 && !DROP) sched_interleave<12, 0, 2, 6>();
    keep_here(ds_c);
  };

  // Units are numbered along the active key tiles, two per tile.  Block u
  // issues S^T, dP^T of unit u+1 and dQ += of unit u-1 beside the
  // element-wise work of unit u.  Iteration n runs blocks 2n+1 and 2n+2: it
  // reads K of tiles n and n+1 and V of tile n+1, which must have landed;
  // every wave has finished with K(n-1) and V(n), whose slots receive K(n+3)
  // and V(n+3).
  f32x16 s_odd, dp_odd, s_even, dp_even;
  VT ds_odd[2], ds_even[2];
  if (jq[0] < kt_end) {
    if (jq[2] < kt_end) wait_vmcnt<4 * DMA_N>();
    else if (jq[1] < kt_end) wait_vmcnt<2 * DMA_N>();
    else wait_vmcnt<0>();
    wg_barrier();
    // Block 0: S^T, dP^T of units 0 and 1, dS of unit 0.
    sdp(0, 0, 0, s_even, dp_even);
    mask_unit(jq[0] * BC, s_even);
    sdp(0, 0, 1, s_odd, dp_odd);
    dscores(jq[0] * BC, s_even, dp_even, ds_even);
  }
  // Q, dO rows and the row statistics were ordinary loads: drain them where
  // the compiler sees it (no vmcnt wait on the copies in flight inside the
  // loop).
  wait_all_loads();
  // One iteration; the slots are run-time indices (K: n mod 4, V: n mod 3).
  // MASKED iterations apply the edge masks; the others are branch-free
  // between their two blocks.
  int n = 0, vs0 = 0;  // vs0: V slot of tile n
  auto iteration = [&](auto masked_c) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_c)::value;
    const int KS0 = n & (NK - 1), KS1 = (n + 1) & (NK - 1);
    const int VS1 = vs0 == NV - 1 ? 0 : vs0 + 1;
    const int jj = jq[0], j1 = jq[1];
    // K(n+1), V(n+1) have landed once at most tile n+2's copies are in flight.
    if (jq[2] < kt_end) wait_vmcnt<2 * DMA_N>();
    else wait_vmcnt<0>();
    wg_barrier();
    if (jq[3] < kt_end) {
      issue(K, jq[3], (n + 3) & (NK - 1));
      issue(V, jq[3], NK + vs0);  // V(n+3) takes V(n)'s slot
    }
    if (!MASKED || jj * BC <= last_key) {
      if constexpr (MASKED) mask_unit(jj * BC + 32, s_odd);
      block(KS1, VS1, KS0, 0, jj * BC + 32, s_odd, dp_odd, s_even, dp_even, ds_even, ds_odd);
      if constexpr (MASKED) mask_unit(j1 < kt_end ? j1 * BC : N, s_even);
      block(KS1, VS1, KS0, 1, j1 * BC, s_even, dp_even, s_odd, dp_odd, ds_odd, ds_even);
    }
    vs0 = VS1;
#pragma unroll
    for (int t = 0; t < NK - 1; ++t) jq[t] = jq[t + 1];
    jq[NK - 1] = jq[NK - 2] < kt_end ? next_active(jq[NK - 2] + 1) : kt_end;
    ++n;
  };
  // Masked units (causal diagonal, keys >= N) come last in a wave's range,
  // so the mask-free iterations form a prefix.
  const int plain_key = CAUSAL ? min(N - 1, q0) : N - 1;
  while (jq[0] < kt_end && jq[1] < kt_end && jq[1] * BC + 31 <= plain_key) iteration(std::false_type{});
  while (jq[0] < kt_end) iteration(std::true_type{});

  // dQ = scale * dS K; lane: query my_q, register r: column 8*(r/4)+4*g+r%4.
  if (my_q < N) {
    float* __restrict__ row = p.dq + base + (size_t)my_q * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg)
        *(float4*)(row + 32 * db + 8 * rg + 4 * g) =
            make_float4(acc[db][4 * rg] * p.scale, acc[db][4 * rg + 1] * p.scale,
                        acc[db][4 * rg + 2] * p.scale, acc[db][4 * rg + 3] * p.scale);
  }
}

// Block-sparse work order: the mask's 128-row tiles (query tiles) and
// 128-column tiles (key tiles) sorted by how many visible tiles each holds,
// most first, ties by index (with the causal flag only tiles on or below the
// diagonal count).  The backward kernels take their tiles in this order, so
// the longest workgroups start first and the shortest fill the tail.  One
// workgroup of 16 waves; counts and ranks in LDS (n <= FWD_MAX_MASK_TILES).
__global__ __launch_bounds__(1024) void sparse_order_kernel(const uint8_t* __restrict__ mask, int n,
                                                            int causal, int* __restrict__ qt_order,
                                                            int* __restrict__ kt_order) {
  __shared__ int row_n[FWD_MAX_MASK_TILES], col_n[FWD_MAX_MASK_TILES];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < n; i += 1024) col_n[i] = 0;
  __syncthreads();
  // Tile (r, c) counts for row r and column c when it is set (and, causal,
  // c <= r).  A wave takes RB mask rows at a time (rows wave, wave + 16, ...),
  // 64 columns per step, loading the step's RB bytes per lane before using
  // any (one memory latency per step, not per row): the row count is the
  // popcount of the step ballots, the column counts LDS atomic adds.
  constexpr int RB = 8;
  for (int r0 = wave; r0 < n; r0 += 16 * RB) {
    int rc[RB] = {};
    for (int c0 = 0; c0 < n; c0 += 64) {
      const int c = c0 + lane;
      // Clamped addresses, so that the loads are unconditional and issue
      // together; the out-of-range bytes are dropped after.
      uint8_t m[RB];
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const int r = r0 + 16 * i;
        m[i] = mask[(size_t)min(r, n - 1) * n + min(c, n - 1)];
      }
#pragma unroll
      for (int i = 0; i < RB; ++i)
        if (r0 + 16 * i >= n || c >= n) m[i] = 0;
#pragma unroll
      for (int i = 0; i < RB; ++i) {
        const bool vis = m[i] != 0 && (!causal || c <= r0 + 16 * i);
        rc[i] += __popcll(__builtin_amdgcn_ballot_w64(vis));
        if (vis) atomicAdd(&col_n[c], 1);
      }
    }
#pragma unroll
    for (int i = 0; i < RB; ++i)
      if (lane == 0 && r0 + 16 * i < n) row_n[r0 + 16 * i] = rc[i];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const int ri = row_n[i], ci = col_n[i];
    int rr = 0, cr = 0;
    for (int t = 0; t < n; ++t) {
      rr += row_n[t] > ri || (row_n[t] == ri && t < i);
      cr += col_n[t] > ci || (col_n[t] == ci && t < i);
    }
    qt_order[rr] = i;
    kt_order[cr] = i;
  }
}

template <typename T, int D, bool CAUSAL, bool SPARSE, bool DROP>
hipError_t launch_bwd_t(const BwdParams& p, hipStream_t st) {
  // The dQ kernel also writes the row statistics (-D, lse * log2 e) that the
  // dK/dV kernel reads, so it runs first.
  const dim3 grid(((p.N + 127) / 128) * p.BH), block(256);
  if constexpr (SPARSE) {
    const hipError_t e = launch_sparse_order(p.mask, p.mask_tiles, CAUSAL, p.qt_order, p.kt_order, st);
    if (e != hipSuccess) return e;
  }
  bwd_dq_u_kernel<T, D, CAUSAL, SPARSE, DROP><<<grid, block, 0, st>>>(p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  bwd_dkdv_u_kernel<T, D, CAUSAL, SPARSE, DROP><<<grid, block, 0, st>>>(p);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_bwd(const BwdParams& p, bool causal, bool sparse, hipStream_t st) {
  if (p.drop) {
    if (causal && sparse) return launch_bwd_t<T, D, true, true, true>(p, st);
    if (causal) return launch_bwd_t<T, D, true, false, true>(p, st);
    if (sparse) return launch_bwd_t<T, D, false, true, true>(p, st);
    return launch_bwd_t<T, D, false, false, true>(p, st);
  }
  if (causal && sparse) return launch_bwd_t<T, D, true, true, false>(p, st);
  if (causal) return launch_bwd_t<T, D, true, false, false>(p, st);
  if (sparse) return launch_bwd_t<T, D, false, true, false>(p, st);
  return launch_bwd_t<T, D, false, false, false>(p, st);
}

}  // namespace

hipError_t launch_sparse_order(const uint8_t* mask, int n, bool causal, int* qt_order,
                               int* kt_order, hipStream_t st) {
  sparse_order_kernel<<<1, 1024, 0, st>>>(mask, n, causal ? 1 : 0, qt_order, kt_order);
  return hipGetLastError();
}

hipError_t launch_backward(BwdParams p, int dtype, int d, bool causal, hipStream_t st) {
  const bool sparse = p.mask != nullptr;
  if (dtype == DT_BF16)
    return d == 64 ? launch_bwd<__bf16, 64>(p, causal, sparse, st)
                   : launch_bwd<__bf16, 128>(p, causal, sparse, st);
  return d == 64 ? launch_bwd<_Float16, 64>(p, causal, sparse, st)
                 : launch_bwd<_Float16, 128>(p, causal, sparse, st);
}

}  // namespace fa
