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
//     so that all tiles of one head land on one XCD (shared L2).
#include <type_traits>

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

namespace {

template <int V>
using ic = std::integral_constant<int, V>;

template <typename T, int D, bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(256, FWD16_MIN_WAVES) void fwd16_kernel(FwdParams p) {
  using VT = typename V8<T>::t;
  using HT = typename V8<T>::h;
  constexpr int NW = 4, QBL = fwd16_qblocks(D, SPARSE), QW = 32 * QBL, BR = NW * QW;
  constexpr int BC = fwd16_kcols(D), KB = BC / 32, KS = BC / 16, NST = FWD16_STAGES;
  constexpr int DS = D / 16, DB = D / 32, CPR = D / 8;
  constexpr int TILE = BC * D;                 // elements of one K (or V) tile
  constexpr int DMA_N = BC * CPR / 256;        // copies per wave per K (or V) tile
  static_assert(QBL == 1 && BR == MASK_TILE, "one 32-row query block per wave");
  // Stage st holds K at [2*st*TILE] and V at [(2*st+1)*TILE], rows swizzled.
  __shared__ __attribute__((aligned(1024))) T kvs[NST * 2 * TILE];
  __shared__ uint8_t mask_s[SPARSE ? FWD_MAX_MASK_TILES : 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31, s16 = lane & 15, gq = lane >> 4;
  const int N = p.N;
  const int n_qt = (N + BR - 1) / BR;
  int bh, qt;
  if (CAUSAL) {
    // Longest query tiles first across all heads (a list schedule in order
    // of decreasing work); with B*H a multiple of 8 the round-robin XCD
    // assignment still gives every XCD whole heads.
    bh = blockIdx.x % p.BH;
    qt = n_qt - 1 - blockIdx.x / p.BH;
  } else {
    const int lid = xcd_remap(blockIdx.x, n_qt * p.BH);
    bh = lid / n_qt;
    qt = lid - bh * n_qt;
  }
  const size_t base = (size_t)bh * N * D;
  const T* __restrict__ Q = (const T*)p.q + base;
  const T* __restrict__ K = (const T*)p.k + base;
  const T* __restrict__ V = (const T*)p.v + base;
  const int q0w = qt * BR + wave * QW;        // first query row of this wave
  const float c = p.scale_log2e;

  // Q^T fragments (B operand): lane holds query q0w + 32*qb + l32.
  VT qf[QBL][DS];
#pragma unroll
  for (int qb = 0; qb < QBL; ++qb) {
    const int q = q0w + 32 * qb + l32;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds)
      qf[qb][ds] = q < N ? *(const VT*)(Q + (size_t)q * D + 16 * ds + 8 * g) : VT{};
  }
  if (SPARSE)
    for (int i = tid; i < p.mask_tiles; i += 256) mask_s[i] = p.mask[(size_t)qt * p.mask_tiles + i];
  // Q and the mask row are in registers/LDS before any copy is in flight.
  wait_all_loads();
  __syncthreads();

  // Per-lane element offsets inside one K or V tile.  The swizzle repeats
  // every 16 rows, so row offsets that are multiples of 16 (and the stage
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
  auto next_active = [&](int jj) {
    if (SPARSE)
      while (jj < kt_end && mask_s[(jj * BC) / MASK_TILE] == 0) ++jj;
    return jj;
  };
  // Last key tile this wave needs (causal: its rows see keys <= q0w + QW - 1).
  const int wave_end = CAUSAL ? min(kt_end, (q0w + QW - 1) / BC + 1) : kt_end;

  auto issue = [&](int jj, int st) {
    const int k0 = jj * BC;
    const uint32_t kd = lds0 + (uint32_t)(2 * st * TILE * (int)sizeof(T));
    const uint32_t vd = kd + (uint32_t)(TILE * (int)sizeof(T));
    if (k0 + BC <= N) {
      const T* kb_ = K + (size_t)k0 * D;
      const T* vb_ = V + (size_t)k0 * D;
#pragma unroll
      for (int u = 0; u < DMA_N; ++u) {
        const uint32_t wo = (uint32_t)((u * NW + wave) * 64 * 16);
        dma16_s(kb_, doff[u], kd + wo);
        dma16_s(vb_, doff[u], vd + wo);
      }
    } else {
      // Tail tile: rows past N read row N - 1 (zeroed once landed).
#pragma unroll
      for (int u = 0; u < DMA_N; ++u) {
        const uint32_t wo = (uint32_t)((u * NW + wave) * 64 * 16);
        const size_t go = (size_t)min(k0 + drow[u], N - 1) * D +
                          (doff[u] / (int)sizeof(T) - drow[u] * D);
        dma16(K + go, kd + wo);
        dma16(V + go, vd + wo);
      }
    }
  };
  auto zero_tail = [&](int jj, int st) {
    const int k0 = jj * BC;
    if (k0 + BC > N) {
      for (int pch = tid; pch < BC * CPR; pch += 256)
        if (k0 + pch / CPR >= N) {
          *(VT*)(&kvs[2 * st * TILE + 8 * pch]) = VT{};
          *(VT*)(&kvs[(2 * st + 1) * TILE + 8 * pch]) = VT{};
        }
      __syncthreads();
    }
  };

  f32x16 o[QBL][DB];
#pragma unroll
  for (int qb = 0; qb < QBL; ++qb)
#pragma unroll
    for (int db = 0; db < DB; ++db) o[qb][db] = f32x16{};
  float m_run[QBL], l_run[QBL];
#pragma unroll
  for (int qb = 0; qb < QBL; ++qb) {
    m_run[qb] = -1e30f;
    l_run[qb] = 0.f;
  }

  // S^T[key][query] of one tile (the wave's 32 queries).
  auto scores1 = [&](auto stc, f32x16 (&sc)[KB]) {
    const T* kt = kvs + 2 * decltype(stc)::value * TILE;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) sc[kb] = f32x16{};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        const VT kf = *(const VT*)(kt + 32 * kb * D + koff[ds]);
        sc[kb] = mfma32x32x16(kf, qf[0][ds], sc[kb]);
      }
  };
  auto needs_mask = [&](int jj, int qb) {
    const int k0 = jj * BC;
    return (k0 + BC > N) || (CAUSAL && k0 + BC - 1 > q0w + 32 * qb);
  };
  // O^T += V^T P^T for the 32 keys of block kb (two 16-key steps).
  auto pv_half = [&](auto stc, int kb, const VT (&pq)[KS]) {
    const T* vt = kvs + (2 * decltype(stc)::value + 1) * TILE;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int kk = 2 * kb + h;
        const VT vf = cat_tr16<VT>(lds_read_tr16(vt + 16 * kk * D + voff[db][0]),
                                   lds_read_tr16(vt + 16 * kk * D + voff[db][1]));
        o[0][db] = mfma32x32x16(vf, pq[kk], o[0][db]);
      }
  };
  // Exponentials of the 32 keys of block kb against the current reference;
  // returns the lane's fp32 sum and writes the two 16-bit P^T operands.
  auto exps_half = [&](const f32x16& sq, VT (&pq)[KS], int kb) {
    const float mc = m_run[0] * c;
    float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 8 * h + 2 * e;
        const float e0 = fast_exp2(fmaf(sq[r], c, -mc));
        const float e1 = fast_exp2(fmaf(sq[r + 1], c, -mc));
        ls0 += e0;
        ls1 += e1;
        w[e] = pack2<T>(e0, e1);
      }
      pq[2 * kb + h] = __builtin_bit_cast(VT, w);
    }
    return ls0 + ls1;
  };
  // Softmax and P V of one tile, 32 keys at a time.  Exponentials are taken
  // against the current reference value first; the reference only moves when
  // some lane's block sum exceeds 2^8 (so some exponential may exceed 2^8, or
  // a row had no reference yet): then the block max is taken, O and l are
  // rescaled by exp(m_old - m_new) (O may already hold the tile's first
  // block; it is rescaled like every earlier contribution) and the block's
  // exponentials are recomputed.  O, l and lse share the reference, so the
  // result does not depend on it.
  auto softmax_pv = [&](auto stc, int jj, f32x16 (&sc)[KB]) {
    if (needs_mask(jj, 0)) {
      const int k0 = jj * BC;
      // Key offset (within the tile) of the last visible key for this lane's
      // query, less the lane's 4*g row offset in the accumulator.
      int lim = N - 1 - k0;
      if (CAUSAL) lim = min(lim, q0w + l32 - k0);
      lim -= 4 * g;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * kb + 8 * (r >> 2) + (r & 3) > lim) sc[kb][r] = -INFINITY;
    }
    VT pq[KS];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      float ls = exps_half(sc[kb], pq, kb);
      if (wave_any(!(ls <= 256.f))) {
        float mx = sc[kb][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sc[kb][r]);
        const float m_new = fmaxf(m_run[0], half_swap_max(mx));
        const float alpha = fast_exp2((m_run[0] - m_new) * c);
        m_run[0] = m_new;
        l_run[0] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[0][db] *= alpha;
        ls = exps_half(sc[kb], pq, kb);
      }
      l_run[0] += ls;
      pv_half(stc, kb, pq);
    }
  };

  // Pipeline over the active tiles t0 < t1 < ...: iteration n issues the
  // score MFMAs of tile n+1, then the softmax and P V of tile n, so the
  // exponentials overlap the matrix work still in flight.  Tile n sits in
  // stage n % NST; tiles n+2 .. n+NST-2 are in flight and tile n+NST-1 is
  // issued once every wave has left stage (n-1) % NST.
  int jq[NST];  // tiles n .. n+NST-1 (kt_end past the last one)
  jq[0] = next_active(0);
#pragma unroll
  for (int i = 1; i < NST; ++i) jq[i] = jq[i - 1] < kt_end ? next_active(jq[i - 1] + 1) : kt_end;
#pragma unroll
  for (int i = 0; i < NST - 1; ++i)
    if (jq[i] < kt_end) issue(jq[i], i);
  // Wait for tile 0, leaving the later prologue tiles in flight.
  {
    int inflight = 0;
#pragma unroll
    for (int i = 1; i < NST - 1; ++i) inflight += jq[i] < kt_end;
    if (NST == 4 && inflight == 2) wait_vmcnt<4 * DMA_N>();
    else if (inflight >= 1) wait_vmcnt<2 * DMA_N>();
    else wait_vmcnt<0>();
  }
  wg_barrier();
  f32x16 sc[KB];
  if (jq[0] < kt_end) {
    zero_tail(jq[0], 0);
    if (jq[0] < wave_end) scores1(ic<0>{}, sc);
  }
  auto iter = [&](auto stc) {
    constexpr int ST = decltype(stc)::value;
    const int j = jq[0], j1 = jq[1];
    // Tile n+1 must have landed; NST-3 later tiles may stay in flight.
    if (NST == 4 && jq[2] < kt_end) wait_vmcnt<2 * DMA_N>();
    else wait_vmcnt<0>();
    // Tile n+1 is in LDS; every wave has finished with stage (ST - 1) % NST.
    wg_barrier();
    if (jq[NST - 1] < kt_end) issue(jq[NST - 1], (ST + NST - 1) % NST);
    if (j1 < kt_end) zero_tail(j1, (ST + 1) % NST);
    f32x16 sn[KB];
    if (j1 < wave_end) scores1(ic<(ST + 1) % NST>{}, sn);
    if (j < wave_end) softmax_pv(ic<ST>{}, j, sc);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) sc[kb] = sn[kb];
#pragma unroll
    for (int i = 0; i < NST - 1; ++i) jq[i] = jq[i + 1];
    jq[NST - 1] = jq[NST - 2] < kt_end ? next_active(jq[NST - 2] + 1) : kt_end;
  };
  while (jq[0] < kt_end) {
    iter(ic<0>{});
    if (jq[0] >= kt_end) break;
    iter(ic<1>{});
    if (jq[0] >= kt_end) break;
    iter(ic<2>{});
    if constexpr (NST == 4) {
      if (jq[0] >= kt_end) break;
      iter(ic<3 % NST>{});
    }
  }

  // Epilogue: O = O / l, lse = scale * m + ln(l).
#pragma unroll
  for (int qb = 0; qb < QBL; ++qb) {
    const float lt = half_swap_sum(l_run[qb]);
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    const int q = q0w + 32 * qb + l32;
    if (q < N) {
      T* orow = (T*)p.o + base + (size_t)q * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          HT h;
#pragma unroll
          for (int e = 0; e < 4; ++e) h[e] = (T)(o[qb][db][4 * rg + e] * inv);
          *(HT*)(orow + 32 * db + 8 * rg + 4 * g) = h;
        }
      if (g == 0) p.lse[(size_t)bh * N + q] = lt > 0.f ? m_run[qb] * p.scale + logf(lt) : -INFINITY;
    }
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
  const int lid = xcd_remap(blockIdx.x, total);
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
  const uint8_t* mrow = SPARSE ? p.mask + (size_t)qt * p.mask_tiles : nullptr;
  auto next_active = [&](int j) {
    if (SPARSE)
      while (j < kt_end && mrow[(j * BC) / MASK_TILE] == 0) ++j;
    return j;
  };

  float4 kreg[PT], vreg[PT];
  auto gload = [&](int j) {
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
  auto lstore = [&](int buf) {
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

  int j = next_active(0);
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
    float* orow = (float*)p.o + base + (size_t)my_q * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        float4 h = make_float4(o[db][4 * rg] * inv, o[db][4 * rg + 1] * inv,
                               o[db][4 * rg + 2] * inv, o[db][4 * rg + 3] * inv);
        *(float4*)(orow + 32 * db + 8 * rg + 4 * g) = h;
      }
    if (g == 0) p.lse[(size_t)bh * N + my_q] = lt > 0.f ? m_run * p.scale + logf(lt) : -INFINITY;
  }
}

template <typename T, int D>
hipError_t launch16(const FwdParams& p, bool causal, bool sparse, hipStream_t st) {
  const int br = 4 * 32 * fwd16_qblocks(D, sparse);
  dim3 grid(((p.N + br - 1) / br) * p.BH), block(256);
  if (causal && sparse) fwd16_kernel<T, D, true, true><<<grid, block, 0, st>>>(p);
  else if (causal) fwd16_kernel<T, D, true, false><<<grid, block, 0, st>>>(p);
  else if (sparse) fwd16_kernel<T, D, false, true><<<grid, block, 0, st>>>(p);
  else fwd16_kernel<T, D, false, false><<<grid, block, 0, st>>>(p);
  return hipGetLastError();
}

template <int D>
hipError_t launch32(const FwdParams& p, bool causal, bool sparse, hipStream_t st) {
  dim3 grid(p.n_qtiles * p.BH), block(256);
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
