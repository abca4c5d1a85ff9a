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
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

namespace {

template <typename T, int D, bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(256, 2) void fwd16_kernel(FwdParams p) {
  using VT = typename V8<T>::t;
  using HT = typename V8<T>::h;
  constexpr int BR = 128, BC = 64, RS = D + 8;
  constexpr int DS = D / 16, DB = D / 32;
  constexpr int CPR = D / 8, PT = BC * D / 8 / 256;
  __shared__ __attribute__((aligned(16))) T ks[2][BC * RS];
  __shared__ __attribute__((aligned(16))) T vs[2][BC * RS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31, s16 = lane & 15, gq = lane >> 4;
  const int N = p.N;
  const int total = p.n_qtiles * p.BH;
  const int lid = xcd_remap(blockIdx.x, total);
  const int bh = lid / p.n_qtiles;
  const int ir = lid - bh * p.n_qtiles;
  const int qt = CAUSAL ? (p.n_qtiles - 1 - ir) : ir;
  const size_t base = (size_t)bh * N * D;
  const T* __restrict__ Q = (const T*)p.q + base;
  const T* __restrict__ K = (const T*)p.k + base;
  const T* __restrict__ V = (const T*)p.v + base;
  const int q0 = qt * BR + wave * 32;
  const int my_q = q0 + l32;

  VT qf[DS];
#pragma unroll
  for (int ds = 0; ds < DS; ++ds) {
    if (my_q < N) qf[ds] = *(const VT*)(Q + (size_t)my_q * D + 16 * ds + 8 * g);
    else qf[ds] = VT{};
  }

  int kt_end = p.n_ktiles;
  if (CAUSAL) kt_end = min(kt_end, (min(N, (qt + 1) * BR) + BC - 1) / BC);
  const uint8_t* mrow = SPARSE ? p.mask + (size_t)qt * p.mask_tiles : nullptr;
  auto next_active = [&](int j) {
    if (SPARSE)
      while (j < kt_end && mrow[(j * BC) / MASK_TILE] == 0) ++j;
    return j;
  };

  VT kreg[PT], vreg[PT];
  auto gload = [&](int j) {
#pragma unroll
    for (int u = 0; u < PT; ++u) {
      const int c = tid + 256 * u, row = c / CPR, col = (c % CPR) * 8;
      const int key = j * BC + row;
      if (key < N) {
        kreg[u] = *(const VT*)(K + (size_t)key * D + col);
        vreg[u] = *(const VT*)(V + (size_t)key * D + col);
      } else {
        kreg[u] = VT{};
        vreg[u] = VT{};
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int u = 0; u < PT; ++u) {
      const int c = tid + 256 * u, row = c / CPR, col = (c % CPR) * 8;
      *(VT*)(&ks[buf][row * RS + col]) = kreg[u];
      *(VT*)(&vs[buf][row * RS + col]) = vreg[u];
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
      // S^T[key][query] for the 64 keys of this tile, two 32-key blocks.
      f32x16 s[2] = {f32x16{}, f32x16{}};
      const T* kb_ = ks[buf];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
          const VT kf = *(const VT*)(&kb_[(32 * kb + l32) * RS + 16 * ds + 8 * g]);
          s[kb] = mfma32x32x16(kf, qf[ds], s[kb]);
        }
      const bool need_mask = (k0 + BC > N) || (CAUSAL && k0 + BC - 1 > q0);
      if (need_mask) {
        // Key offset (within the tile) of the last visible key for this
        // lane's query, less the lane's 4*g row offset in the accumulator.
        int lim = N - 1 - k0;
        if (CAUSAL) lim = min(lim, my_q - k0);
        lim -= 4 * g;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (32 * kb + 8 * (r >> 2) + (r & 3) > lim) s[kb][r] = -INFINITY;
      }
      float mx = s[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = half_swap_max(mx);
      // Lazy rescale: the running max only moves when some row's tile max
      // exceeds it by more than 8 in log2 units, so the exponentials stay
      // <= 2^8 and O, l are rescaled rarely.  Any reference value gives the
      // same O and lse as long as O, l and lse share it.
      if (wave_any(mx > m_run + p.rescale_thr)) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = fast_exp2((m_run - m_new) * c);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] *= alpha;
      }
      const float mc = m_run * c;
      // Row sums stay in fp32 on the unrounded exponentials (the saved lse
      // depends on them); only the PV operand is rounded to 16 bits.
      VT pf[4];
      float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          u32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 8 * h + 2 * e;
            const float e0 = fast_exp2(fmaf(s[kb][r], c, -mc));
            const float e1 = fast_exp2(fmaf(s[kb][r + 1], c, -mc));
            ls0 += e0;
            ls1 += e1;
            w[e] = pack2<T>(e0, e1);
          }
          pf[2 * kb + h] = __builtin_bit_cast(VT, w);
        }
      l_run += ls0 + ls1;
      const T* vb = vs[buf];
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int row = 16 * kk + 4 * g + (s16 >> 2);
          const int col = 32 * db + 16 * (gq & 1) + 4 * (s16 & 3);
          const i16x4 lo = lds_read_tr16(&vb[row * RS + col]);
          const i16x4 hi = lds_read_tr16(&vb[(row + 8) * RS + col]);
          o[db] = mfma32x32x16(cat_tr16<VT>(lo, hi), pf[kk], o[db]);
        }
    }
    if (jn < kt_end) lstore(buf ^ 1);
    __syncthreads();
    buf ^= 1;
    j = jn;
  }

  // Epilogue: O = O / l, lse = scale * m + ln(l).
  const float lt = half_swap_sum(l_run);
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  if (my_q < N) {
    T* orow = (T*)p.o + base + (size_t)my_q * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        HT h;
#pragma unroll
        for (int e = 0; e < 4; ++e) h[e] = (T)(o[db][4 * rg + e] * inv);
        *(HT*)(orow + 32 * db + 8 * rg + 4 * g) = h;
      }
    if (g == 0) p.lse[(size_t)bh * N + my_q] = lt > 0.f ? m_run * p.scale + logf(lt) : -INFINITY;
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
  dim3 grid(p.n_qtiles * p.BH), block(256);
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
