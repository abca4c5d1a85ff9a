// Forward pass of exact attention on gfx950: one workgroup per (query tile,
// batch*head), streaming key/value tiles through LDS with the online-softmax
// recurrence.
//
// What is computed follows the FlashAttention pages: the query block stays
// on chip while key/value blocks stream past it, each block's scores update a
// running row max m and row sum l, the partial output is rescaled by
// exp(m_old - m_new) whenever the max grows, and only O and one statistic per
// row go back to memory ("Método", incremental softmax equations, xyznot.com
// reading guide; "La récurrence softmax en ligne", marketmaker.cc).  The
// output stays unnormalised until the last block, as in the ultralytics
// glossary's loop and the "FA2" section of the marketmaker.cc page.  The grid
// spans query tiles as well as batch and heads, and each wave owns its own
// query rows ("FA2 : parallélisme", points 2 and 3).  Tiles entirely in the
// causal future, or zero in the block mask, are never loaded ("Le masquage
// causal"; "Extensão: Block-Sparse FlashAttention").
//
// gfx950 mapping (16-bit inputs):
//   * 256 threads = 4 waves; a workgroup owns 128 query rows, a wave 32.
//   * Scores are computed transposed, S^T = K Q^T on v_mfma_f32_32x32x16, so
//     each lane holds one query's scores: the row max and row sum are
//     in-lane reductions plus one permlane32 swap, and the rescale factor
//     exp(m_old - m_new) is a per-lane scalar.
//   * Q^T stays in VGPRs for the whole key loop.  K and V tiles of 64 keys are
//     double buffered in LDS (one barrier per tile); K is read with 16-byte
//     LDS reads, V with ds_read_b64_tr_b16 so that the O^T += V^T P^T product
//     takes P^T straight from the score accumulators with no shuffle.
//   * exp is exp2 with scale*log2(e) folded into one FMA.
//   * Causal grids run longest query tiles first; workgroup ids are remapped
//     so that all tiles of one head land on one XCD (shared L2).  Given a
//     work order, block-sparse grids take a head's query tiles with the most
//     visible key tiles first.
#include <type_traits>

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

namespace {

template <int V>
using ic = std::integral_constant<int, V>;

template <typename T, int D, int NS, bool CAUSAL, bool SPARSE, bool DROP>
__global__ __launch_bounds__(256, fwd16_waves(D, NS)) void fwd16_kernel(FwdParams p) {
  using VT = typename V8<T>::t;
  using HT = typename V8<T>::h;
  constexpr int NW = 4, BR = 128;              // 4 waves x 32 query rows
  constexpr int BC = 64;                       // keys per K/V tile (two 32-key units)
  constexpr int DS = D / 16, DB = D / 32, CPR = D / 8;
  constexpr int TILE = BC * D;                 // elements of one K (or V) tile
  constexpr int DMA_N = BC * CPR / 256;        // copies per wave per tile
  static_assert(BR == MASK_TILE, "a workgroup covers one block-mask row");
  static_assert(NS == 2 || NS == 3, "ring depth");
  // K slot s at [s*TILE], V slot s at [(NS+s)*TILE]; rows swizzled.
  __shared__ __attribute__((aligned(1024))) T kvs[2 * NS * TILE];
  __shared__ uint8_t mask_s[SPARSE ? FWD_MAX_MASK_TILES : 1];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, l32 = lane & 31, s16 = lane & 15, gq = lane >> 4;
  const int N = p.N;
  const int n_qt = (N + BR - 1) / BR;
  // Split key ranges: consecutive workgroups share a query tile, one range
  // each (n_splits = 1: the whole range).
  const int n_sp = p.n_splits;
  int bid = blockIdx.x, split = 0;
  if (n_sp > 1) {
    split = bid % n_sp;
    bid /= n_sp;
  }
  int bh, qt;
  if (CAUSAL) {
    // Longest query tiles first, few heads per XCD (causal_tile).
    int rank;
    causal_tile(bid, p.BH, n_qt, bh, rank);
    qt = n_qt - 1 - rank;
  } else {
    const int lid = xcd_remap(bid, n_qt * p.BH);
    bh = lid / n_qt;
    qt = lid - bh * n_qt;
    // Block-sparse: the head's query tiles with the most visible key tiles
    // first, so that the workgroups an XCD runs at once hold rows of similar
    // length, walk the head's K/V tiles in step and find them in L2.
    if (SPARSE && p.qt_order != nullptr) qt = p.qt_order[qt];
  }
  const size_t base = (size_t)bh * N * D;
  const T* __restrict__ Q = (const T*)p.q + base;
  const T* __restrict__ K = (const T*)p.k + base;
  const T* __restrict__ V = (const T*)p.v + base;
  const int q0w = qt * BR + wave * 32;        // first query row of this wave
  const float c = p.scale_log2e;

  if (SPARSE) {
    for (int i = tid; i < p.mask_tiles; i += 256) mask_s[i] = p.mask[(size_t)qt * p.mask_tiles + i];
    __syncthreads();
  }

  // Per-lane element offsets inside one K or V tile.  The swizzle repeats
  // every 16 rows, so row offsets that are multiples of 16 (and the slot
  // base, a constant in the unrolled loop below) fold into the instruction's
  // immediate offset.
  int koff[DS], voff[DB][2];
#pragma unroll
  for (int ds = 0; ds < DS; ++ds) koff[ds] = swz_off<D>(l32, 16 * ds + 8 * g);
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      voff[db][h] = swz_off<D>(4 * g + (s16 >> 2) + 8 * h, 32 * db + 16 * (gq & 1) + 4 * (s16 & 3));
  // Copy schedule: copy u of this wave fills physical 16-byte chunk pch of a
  // tile, i.e. row r, logical chunk (pch % CPR) ^ swz(r).
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
  // This workgroup's run of key tiles: [kt_begin, kt_end).
  int kt_begin = 0;
  if (n_sp > 1) {
    const int all = kt_end;
    kt_begin = (int)((long long)all * split / n_sp);
    kt_end = (int)((long long)all * (split + 1) / n_sp);
  }
  auto next_active = [&](int jj) __attribute__((always_inline)) {
    if (SPARSE)
      while (jj < kt_end && mask_s[(jj * BC) / MASK_TILE] == 0) ++jj;
    return jj;
  };
  // Keys past last_key are invisible to every query of this wave; a unit
  // starting at ks needs masking iff ks + 31 > plain_key.
  // key_last: the last key of this workgroup's run (N - 1 without splits).
  // The unit after a run's last tile is evaluated (and must come out empty)
  // like the one past the end of the sequence.
  const int key_last = min(N, kt_end * BC) - 1;
  const int last_key = CAUSAL ? min(key_last, q0w + 31) : key_last;
  const int plain_key = CAUSAL ? min(key_last, q0w) : key_last;

  // Copy tile jj of K (or V) into slot `slot` of its ring.  Rows past N read
  // row N - 1: those keys are masked out of every score that is used, and
  // their values meet probability 0.
  auto issue = [&](const T* src, int jj, int slot, bool is_v) __attribute__((always_inline)) {
    const int k0 = jj * BC;
    const uint32_t dst = lds0 + (uint32_t)(((is_v ? NS : 0) + slot) * TILE * (int)sizeof(T));
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

  // Q^T fragments (B operand): lane holds query q0w + l32.  Loaded after the
  // first copies are issued; the first use waits for both.
  int jq[NS + 1];  // active tiles n .. n+NS (kt_end past the last one)
  jq[0] = next_active(kt_begin);
#pragma unroll
  for (int i = 1; i <= NS; ++i) jq[i] = jq[i - 1] < kt_end ? next_active(jq[i - 1] + 1) : kt_end;
  // Prologue copies, in the order K0 V0 K1 [V1 K2]: iteration n then issues
  // K(n+NS) and V(n+NS-1), each into the slot its predecessor has left.
  if (jq[0] < kt_end) {
    issue(K, jq[0], 0, false);
    issue(V, jq[0], 0, true);
  }
  if (jq[1] < kt_end) issue(K, jq[1], 1, false);
  if (NS == 3) {
    if (jq[1] < kt_end) issue(V, jq[1], 1, true);
    if (jq[2] < kt_end) issue(K, jq[2], 2, false);
  }
  VT qf[DS];
  {
    const int q = q0w + l32;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds)
      qf[ds] = q < N ? *(const VT*)(Q + (size_t)q * D + 16 * ds + 8 * g) : VT{};
  }

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  float m_run = -1e30f, l_run = 0.f;
  float mc_run = m_run * c;  // m_run * c, updated with m_run

  // ---- work on one 32-key unit ----
  // S^T[key][query] of half h of the K tile in slot SL.
  auto s_unit = [&](auto slc, int h, f32x16& s) __attribute__((always_inline)) {
    const T* kt = kvs + decltype(slc)::value * TILE + 32 * h * D;
    s = f32x16{};
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) s = mfma32x32x16(*(const VT*)(kt + koff[ds]), qf[ds], s);
  };
  // O^T += V^T P^T for half h of the V tile in slot SL (two 16-key steps).
  auto pv_unit = [&](auto slc, int h, const VT (&pu)[2]) __attribute__((always_inline)) {
    const T* vt = kvs + (NS + decltype(slc)::value) * TILE + 32 * h * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const VT vf = cat_tr16<VT>(lds_read_tr16(vt + 16 * st * D + voff[db][0]),
                                   lds_read_tr16(vt + 16 * st * D + voff[db][1]));
        o[db] = mfma32x32x16(vf, pu[st], o[db]);
      }
  };
  // Exponentials of one unit's scores against the current reference; returns
  // the lane's fp32 sum and writes the two 16-bit P^T operands.
  // With dropout the row sum takes every exponential and the P V operand
  // only the kept ones (the 1 / (1 - p) scale is applied at the end).
  auto exps = [&](const f32x16& s, VT (&pu)[2], const uint32_t (&dw)[4]) __attribute__((always_inline)) {
    const float mc = mc_run;
    // The sums start at the first terms (not at 0, which would cost an add).
    float ls0, ls1;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 8 * h + 2 * e;
        const float e0 = fast_exp2(fmaf(s[r], c, -mc));
        const float e1 = fast_exp2(fmaf(s[r + 1], c, -mc));
        ls0 = r == 0 ? e0 : ls0 + e0;
        ls1 = r == 0 ? e1 : ls1 + e1;
        w[e] = pack2<T>(e0, e1);
      }
      if constexpr (DROP) {
        // Dropped probabilities become +0 in the packed P V operand.
        uint32_t m[4];
        drop_masks16(dw[2 * h], p.drop_t8, m[0], m[1]);
        drop_masks16(dw[2 * h + 1], p.drop_t8, m[2], m[3]);
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] &= m[e];
      }
      pu[h] = __builtin_bit_cast(VT, w);
    }
    return ls0 + ls1;
  };
  // Exponentials are taken against the current reference first; the
  // reference only moves when some lane's unit sum exceeds 2^8 (so some
  // exponential may exceed 2^8, or a row had no reference yet): then the unit
  // max is taken, O and l are rescaled by exp(m_old - m_new) and the unit's
  // exponentials are recomputed.  O, l and lse share the reference, so the
  // result does not depend on it.  O already holds every earlier unit
  // (including the one whose P V was issued in the same block).
  auto settle = [&](float ls, const f32x16& s, VT (&pu)[2], const uint32_t (&dw)[4]) __attribute__((always_inline)) {
    if (wave_any(!(ls <= 256.f))) {
      float mx = s[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
      const float m_new = fmaxf(m_run, half_swap_max(mx));
      const float alpha = fast_exp2((m_run - m_new) * c);
      m_run = m_new;
      mc_run = m_new * c;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
      ls = exps(s, pu, dw);
    }
    l_run += ls;
  };
  // Scores of keys past this lane's last visible key (causal diagonal, keys
  // >= N) become -inf.  A unit past the wave's range is masked entirely, so
  // its probabilities are exactly 0 and its P V adds nothing.
  auto mask_unit = [&](int ks, f32x16& s) __attribute__((always_inline)) {
    if (ks + 31 > plain_key) {
      const int lim = min(key_last, CAUSAL ? q0w + l32 : N - 1) - ks - 4 * g;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        s[r] = 8 * (r >> 2) + (r & 3) > lim ? -INFINITY : s[r];
    }
  };
  // One block: matrix work of the neighbouring units (scores of the next,
  // P V of the previous) beside the exponentials of this one, with every LDS
  // read issued first.
  // Keep bytes of the unit starting at key ks (dropout only).
  auto drop_words = [&](int ks, uint32_t (&dw)[4]) __attribute__((always_inline)) {
    if constexpr (DROP)
      drop_words_query_lane(dw, ks, q0w, l32, g, (uint32_t)bh, p.drop_off, p.drop_k0, p.drop_k1);
  };
  auto block = [&](auto kslc, auto vslc, int h, int ks_cur, f32x16& s_cur, f32x16& s_nxt,
                   const VT (&p_prv)[2], VT (&p_cur)[2]) __attribute__((always_inline)) {
    s_unit(kslc, h, s_nxt);
    pv_unit(vslc, h, p_prv);
    uint32_t dw[4];
    drop_words(ks_cur, dw);
    const float ls = exps(s_cur, p_cur, dw);
    if constexpr (DROP) {
    } else if constexpr (D == 64) {
      sched_interleave<8, 12, 0, 7>();
    } else {
      sched_interleave<16, 12, 1, 4>();
    }
    settle(ls, s_cur, p_cur, dw);
  };

  // Units are numbered along the active tiles, two per tile.  Block u
  // evaluates the softmax of unit u, the scores of unit u+1 and P V of unit
  // u-1.  Iteration n runs blocks 2n+1 and 2n+2, so it reads only K of tile
  // n+1 and V of tile n: K(n+1) and V(n) must have landed, and every wave
  // has finished with K(n) and V(n-1), whose slots then receive K(n+NS) and
  // V(n+NS-1).  s_odd / p_even carry s(2n+1) and p(2n) between iterations.
  // Scores computed past the last tile (stale LDS) are never used.
  f32x16 s_odd, s_even;
  VT p_odd[2], p_even[2];
  // Prologue: block 0 (scores of units 0 and 1, softmax of unit 0).
  if (jq[0] < kt_end) {
    // Wait for K0, leaving the later prologue copies in flight.
    if (NS == 3) {
      if (jq[2] < kt_end) wait_vmcnt<4 * DMA_N>();
      else if (jq[1] < kt_end) wait_vmcnt<3 * DMA_N>();
      else wait_vmcnt<DMA_N>();
    } else {
      if (jq[1] < kt_end) wait_vmcnt<2 * DMA_N>();
      else wait_vmcnt<DMA_N>();
    }
    wg_barrier();
    s_unit(ic<0>{}, 0, s_even);
    mask_unit(jq[0] * BC, s_even);
    s_unit(ic<0>{}, 1, s_odd);
    uint32_t dw[4];
    drop_words(jq[0] * BC, dw);
    settle(exps(s_even, p_even, dw), s_even, p_even, dw);
  }
  // The Q^T fragments were ordinary loads: drain them where the compiler
  // sees it, so that their first use inside the loop gets no vmcnt wait
  // (which would also wait for the K/V copies in flight).
  wait_all_loads();
  auto iter = [&](auto slc) __attribute__((always_inline)) {
    constexpr int SL = decltype(slc)::value;        // n % NS
    constexpr int SL1 = (SL + 1) % NS;              // slot of tile n+1
    const int j = jq[0], j1 = jq[1];
    // K(n+1) and V(n) have landed once at most the copies issued by the
    // previous iteration (K(n+2), V(n+1)) are in flight.
    if (NS == 3 && jq[2] < kt_end) wait_vmcnt<2 * DMA_N>();
    else if (NS == 3 && j1 < kt_end) wait_vmcnt<DMA_N>();
    else wait_vmcnt<0>();
    wg_barrier();
    if (jq[NS] < kt_end) issue(K, jq[NS], SL, false);
    if (jq[NS - 1] < kt_end) issue(V, jq[NS - 1], (SL + NS - 1) % NS, true);
    // Units 2n .. 2n+2 start at keys j*BC, j*BC + 32 and j1*BC (j1 = kt_end
    // past the last tile, which masks unit 2n+2 entirely).
    if (j * BC <= last_key) {
      mask_unit(j * BC + 32, s_odd);
      block(ic<SL1>{}, ic<SL>{}, 0, j * BC + 32, s_odd, s_even, p_even, p_odd);
      mask_unit(j1 * BC, s_even);
      block(ic<SL1>{}, ic<SL>{}, 1, j1 * BC, s_even, s_odd, p_odd, p_even);
    }
#pragma unroll
    for (int i = 0; i < NS; ++i) jq[i] = jq[i + 1];
    jq[NS] = jq[NS - 1] < kt_end ? next_active(jq[NS - 1] + 1) : kt_end;
  };
  while (jq[0] < kt_end) {
    iter(ic<0>{});
    if (jq[0] >= kt_end) break;
    iter(ic<1 % NS>{});
    if constexpr (NS == 3) {
      if (jq[0] >= kt_end) break;
      iter(ic<2>{});
    }
  }

  // Epilogue: O = O / l, lse = scale * m + ln(l).
  const float lt = half_swap_sum(l_run);
  const float inv = lt > 0.f ? (DROP ? p.drop_scale : 1.0f) / lt : 0.f;
  const int q = q0w + l32;
  if (n_sp > 1) {
    // Partial result of this key range, fp32, for the merge kernel; a range
    // with no visible key leaves O = 0 and lse = -inf (weight 0 there).
    if (q < N) {
      const size_t prow = ((size_t)bh * n_sp + split) * N + q;
      float* orow = p.o_part + prow * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg)
          *(float4*)(orow + 32 * db + 8 * rg + 4 * g) =
              make_float4(o[db][4 * rg] * inv, o[db][4 * rg + 1] * inv, o[db][4 * rg + 2] * inv,
                          o[db][4 * rg + 3] * inv);
      if (g == 0) p.lse_part[prow] = lt > 0.f ? m_run * p.scale + logf(lt) : -INFINITY;
    }
    return;
  }
  if (q < N) {
    T* orow = (T*)p.o + base + (size_t)q * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        HT hv;
#pragma unroll
        for (int e = 0; e < 4; ++e) hv[e] = (T)(o[db][4 * rg + e] * inv);
        *(HT*)(orow + 32 * db + 8 * rg + 4 * g) = hv;
      }
    if constexpr (DROP) {
      // The unrounded O, for the dropout backward's D = rowsum(dO o O).
      if (p.o_acc != nullptr) {
        float* arow = p.o_acc + base + (size_t)q * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int rg = 0; rg < 4; ++rg)
            *(float4*)(arow + 32 * db + 8 * rg + 4 * g) =
                make_float4(o[db][4 * rg] * inv, o[db][4 * rg + 1] * inv,
                            o[db][4 * rg + 2] * inv, o[db][4 * rg + 3] * inv);
      }
    }
    if (g == 0) p.lse[(size_t)bh * N + q] = lt > 0.f ? m_run * p.scale + logf(lt) : -INFINITY;
  }
}

// fp32 inputs: same schedule on v_mfma_f32_32x32x2_f32, 32-key tiles.
template <int D, bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(256, 1) void fwd32_kernel(FwdParams p) {
  constexpr int BR = 128, BC = 32, RS = D + 4;
  constexpr int DB = D / 32;
  constexpr int CPR = D / 4, PT = BC * D / 4 / 256;
  __shared__ __attribute__((aligned(16))) float ks[2][BC * RS];
  __shared__ __attribute__((aligned(16))) float vs[2][BC * RS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int N = p.N;
  const int total = p.n_qtiles * p.BH;
  // Split key runs as in the 16-bit kernel: consecutive workgroups share a
  // query tile, one run of key tiles each.
  const int n_sp = p.n_splits;
  int bid = blockIdx.x, split = 0;
  if (n_sp > 1) {
    split = bid % n_sp;
    bid /= n_sp;
  }
  const int lid = xcd_remap(bid, total);
  const int bh = lid / p.n_qtiles;
  const int ir = lid - bh * p.n_qtiles;
  const int qt = CAUSAL ? (p.n_qtiles - 1 - ir) : ir;
  const size_t base = (size_t)bh * N * D;
  const float* __restrict__ Q = (const float*)p.q + base;
  const float* __restrict__ K = (const float*)p.k + base;
  const float* __restrict__ V = (const float*)p.v + base;
  const int q0 = qt * BR + wave * 32;
  const int my_q = q0 + l32;

  float qf[D / 2];
#pragma unroll
  for (int st = 0; st < D / 2; ++st) qf[st] = my_q < N ? Q[(size_t)my_q * D + 2 * st + g] : 0.f;

  int kt_end = (N + BC - 1) / BC;
  if (CAUSAL) kt_end = min(kt_end, (min(N, (qt + 1) * BR) + BC - 1) / BC);
  int kt_begin = 0;
  if (n_sp > 1) {
    const int all = kt_end;
    kt_begin = (int)((long long)all * split / n_sp);
    kt_end = (int)((long long)all * (split + 1) / n_sp);
  }
  const uint8_t* mrow = SPARSE ? p.mask + (size_t)qt * p.mask_tiles : nullptr;
  auto next_active = [&](int j) __attribute__((always_inline)) {
    if (SPARSE)
      while (j < kt_end && mrow[(j * BC) / MASK_TILE] == 0) ++j;
    return j;
  };

  float4 kreg[PT], vreg[PT];
  auto gload = [&](int j) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < PT; ++u) {
      const int c = tid + 256 * u, row = c / CPR, col = (c % CPR) * 4;
      const int key = j * BC + row;
      if (key < N) {
        kreg[u] = *(const float4*)(K + (size_t)key * D + col);
        vreg[u] = *(const float4*)(V + (size_t)key * D + col);
      } else {
        kreg[u] = make_float4(0.f, 0.f, 0.f, 0.f);
        vreg[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
  };
  auto lstore = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < PT; ++u) {
      const int c = tid + 256 * u, row = c / CPR, col = (c % CPR) * 4;
      *(float4*)(&ks[buf][row * RS + col]) = kreg[u];
      *(float4*)(&vs[buf][row * RS + col]) = vreg[u];
    }
  };

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16{};
  float m_run = -1e30f, l_run = 0.f;
  const float c = p.scale_log2e;

  int j = next_active(kt_begin);
  if (j < kt_end) {
    gload(j);
    lstore(0);
  }
  __syncthreads();
  int buf = 0;
  while (j < kt_end) {
    const int jn = next_active(j + 1);
    if (jn < kt_end) gload(jn);
    const int k0 = j * BC;
    if (!CAUSAL || k0 <= q0 + 31) {
      f32x16 s = f32x16{};
      const float* kb_ = ks[buf];
#pragma unroll
      for (int st = 0; st < D / 2; ++st) s = mfma32x32x2(kb_[l32 * RS + 2 * st + g], qf[st], s);
      if ((k0 + BC > N) || (CAUSAL && k0 + BC - 1 > q0)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 8 * (r >> 2) + 4 * g + (r & 3);
          if (key >= N || (CAUSAL && key > my_q)) s[r] = -INFINITY;
        }
      }
      float mx = m_run;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
      mx = half_swap_max(mx);
      const float alpha = fast_exp2((m_run - mx) * c);
      m_run = mx;
      const float mc = mx * c;
      float ls = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = fast_exp2(fmaf(s[r], c, -mc));
        ls += s[r];
      }
      l_run = l_run * alpha + ls;
      const float* vb = vs[buf];
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        o[db] *= alpha;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = 8 * (r >> 2) + 4 * g + (r & 3);
          o[db] = mfma32x32x2(vb[row * RS + 32 * db + l32], s[r], o[db]);
        }
      }
    }
    if (jn < kt_end) lstore(buf ^ 1);
    __syncthreads();
    buf ^= 1;
    j = jn;
  }

  const float lt = half_swap_sum(l_run);
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  if (my_q < N) {
    // With runs: this run's normalised partial output and logsumexp.
    const size_t prow = ((size_t)bh * n_sp + split) * N + my_q;
    float* orow = n_sp > 1 ? p.o_part + prow * D : (float*)p.o + base + (size_t)my_q * D;
    float* lrow = n_sp > 1 ? p.lse_part + prow : p.lse + (size_t)bh * N + my_q;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        float4 h = make_float4(o[db][4 * rg] * inv, o[db][4 * rg + 1] * inv,
                               o[db][4 * rg + 2] * inv, o[db][4 * rg + 3] * inv);
        *(float4*)(orow + 32 * db + 8 * rg + 4 * g) = h;
      }
    if (g == 0) *lrow = lt > 0.f ? m_run * p.scale + logf(lt) : -INFINITY;
  }
}

template <typename T, int D, int NS, bool DROP>
hipError_t launch16_v(const FwdParams& p, bool causal, bool sparse, dim3 grid, hipStream_t st) {
  const dim3 block(256);
  if (causal && sparse) fwd16_kernel<T, D, NS, true, true, DROP><<<grid, block, 0, st>>>(p);
  else if (causal) fwd16_kernel<T, D, NS, true, false, DROP><<<grid, block, 0, st>>>(p);
  else if (sparse) fwd16_kernel<T, D, NS, false, true, DROP><<<grid, block, 0, st>>>(p);
  else fwd16_kernel<T, D, NS, false, false, DROP><<<grid, block, 0, st>>>(p);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch16(const FwdParams& p, bool causal, bool sparse, hipStream_t st) {
  const dim3 grid(((p.N + 127) / 128) * p.BH * (p.n_splits > 1 ? p.n_splits : 1));
  constexpr int NS = D == 64 ? 3 : 2;
  if (p.drop) return launch16_v<T, D, NS, true>(p, causal, sparse, grid, st);
  if constexpr (D == 64) {
    // Grids of at least two full rounds at four workgroups per CU run the
    // two-slot form (four waves per SIMD, 128 VGPRs); smaller grids keep
    // copies two tiles ahead (three slots, three waves), which shortens
    // each workgroup.  (The dropout variant needs more than 128 VGPRs and
    // keeps three slots.)
    if (grid.x >= (unsigned)fwd16_large_grid()) return launch16_v<T, D, 2, false>(p, causal, sparse, grid, st);
  }
  return launch16_v<T, D, NS, false>(p, causal, sparse, grid, st);
}

template <int D>
hipError_t launch32(const FwdParams& p, bool causal, bool sparse, hipStream_t st) {
  dim3 grid(p.n_qtiles * p.BH * (p.n_splits > 1 ? p.n_splits : 1)), block(256);
  if (causal && sparse) fwd32_kernel<D, true, true><<<grid, block, 0, st>>>(p);
  else if (causal) fwd32_kernel<D, true, false><<<grid, block, 0, st>>>(p);
  else if (sparse) fwd32_kernel<D, false, true><<<grid, block, 0, st>>>(p);
  else fwd32_kernel<D, false, false><<<grid, block, 0, st>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_forward(FwdParams p, int dtype, int d, bool causal, hipStream_t st) {
  const bool sparse = p.mask != nullptr;
  p.n_qtiles = (p.N + FWD_BR - 1) / FWD_BR;
  if (dtype == DT_F32) {
    p.n_ktiles = (p.N + 31) / 32;
    return d == 64 ? launch32<64>(p, causal, sparse, st) : launch32<128>(p, causal, sparse, st);
  }
  p.n_ktiles = (p.N + 63) / 64;
  if (dtype == DT_BF16)
    return d == 64 ? launch16<__bf16, 64>(p, causal, sparse, st)
                   : launch16<__bf16, 128>(p, causal, sparse, st);
  return d == 64 ? launch16<_Float16, 64>(p, causal, sparse, st)
                 : launch16<_Float16, 128>(p, causal, sparse, st);
}

}  // namespace fa
