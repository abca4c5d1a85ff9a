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
// Three kernels, no atomics:
//   bwd_pre:  D = rowsum(dO o O) in fp32 (the workspace).
//   bwd_dkdv: one workgroup per (key tile of 128, batch*head).  Wave w owns 32
//     keys, keeps their K and V rows in VGPRs and dK, dV in fp32
//     accumulators, and loops over the 32-row query tiles that can see them
//     (causal: tiles at or after the key tile; block-sparse: set entries).
//     S = Q K^T and dP = dO V^T run on v_mfma_f32_32x32x16 with the key in
//     the lane, so P^T and dS^T for dV += P^T dO and dK += dS^T Q come
//     straight from the accumulators; dO and Q are read with
//     ds_read_b64_tr_b16.  Q, dO, lse and D tiles are double buffered in
//     LDS with one barrier per query tile.
//   bwd_dq: one workgroup per (query tile of 128, batch*head), the forward's
//     schedule: S^T = K Q^T and dP^T = V dO^T with the query in the lane (so
//     lse and D are per-lane scalars), dS^T in registers, and
//     dQ^T += K^T dS^T with K read by ds_read_b64_tr_b16; dQ stays in
//     registers and is stored once.
// Recomputing S, P, dP in both kernels costs two extra products per score,
// instead of the global atomic adds a single-pass dQ would need (those go to
// memory on this part and moved more bytes than the whole pass computes).
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const T* __restrict__ O, const T* __restrict__ dO,
                                                      float* __restrict__ delta, size_t rows) {
  using VT = typename V8<T>::t;
  constexpr int LPR = D / 8;  // lanes per row, 8 elements each
  const size_t gt = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t row = gt / LPR;
  const int part = (int)(gt % LPR);
  float acc = 0.f;
  if (row < rows) {
    const VT a = *(const VT*)(O + row * D + part * 8);
    const VT b = *(const VT*)(dO + row * D + part * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf((float)a[e], (float)b[e], acc);
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && part == 0) delta[row] = acc;
}

// log2-domain row statistic: +inf makes P = 0 for padding rows and for rows
// with no visible key (lse = -inf).
__device__ __forceinline__ float lse_log2(float l) { return l == -INFINITY ? INFINITY : l * kLog2e; }

template <typename T, int D, bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(256, 2) void bwd_dkdv_kernel(BwdParams p) {
  using VT = typename V8<T>::t;
  constexpr int BC = 128, QB = 32, RS = D + 8;
  constexpr int DS = D / 16, DB = D / 32;
  constexpr int CPR = D / 8, PTQ = QB * D / 8 / 256;
  __shared__ __attribute__((aligned(16))) T qs[2][QB * RS];
  __shared__ __attribute__((aligned(16))) T dos[2][QB * RS];
  __shared__ __attribute__((aligned(16))) float lsel[2][QB];
  __shared__ __attribute__((aligned(16))) float dls[2][QB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31, s16 = lane & 15, gq = lane >> 4;
  const int N = p.N;
  const int total = p.n_ktiles * p.BH;
  const int lid = xcd_remap(blockIdx.x, total);
  const int bh = lid / p.n_ktiles;
  const int j = lid - bh * p.n_ktiles;  // causal: small j has the most query tiles
  const size_t base = (size_t)bh * N * D;
  const T* __restrict__ Q = (const T*)p.q + base;
  const T* __restrict__ K = (const T*)p.k + base;
  const T* __restrict__ V = (const T*)p.v + base;
  const T* __restrict__ dO = (const T*)p.dO + base;
  const float* __restrict__ LSE = p.lse + (size_t)bh * N;
  const float* __restrict__ DEL = p.delta + (size_t)bh * N;
  const int k0 = j * BC, kw0 = k0 + 32 * wave, my_k = kw0 + l32;
  const float c = p.scale_log2e;

  VT kf[DS], vf[DS];
#pragma unroll
  for (int ds = 0; ds < DS; ++ds) {
    if (my_k < N) {
      kf[ds] = *(const VT*)(K + (size_t)my_k * D + 16 * ds + 8 * g);
      vf[ds] = *(const VT*)(V + (size_t)my_k * D + 16 * ds + 8 * g);
    } else {
      kf[ds] = VT{};
      vf[ds] = VT{};
    }
  }

  f32x16 dk[DB], dv[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }

  const int i_end = p.n_qtiles;
  const int i_beg = CAUSAL ? k0 / QB : 0;
  auto next_active = [&](int i) {
    if (SPARSE)
      while (i < i_end && p.mask[(size_t)((i * QB) / MASK_TILE) * p.mask_tiles + j] == 0) ++i;
    return i;
  };

  VT qreg[PTQ], doreg[PTQ];
  float lreg = 0.f, dreg = 0.f;
  auto gload = [&](int i) {
#pragma unroll
    for (int u = 0; u < PTQ; ++u) {
      const int cc = tid + 256 * u, row = cc / CPR, col = (cc % CPR) * 8;
      const int q = i * QB + row;
      if (q < N) {
        qreg[u] = *(const VT*)(Q + (size_t)q * D + col);
        doreg[u] = *(const VT*)(dO + (size_t)q * D + col);
      } else {
        qreg[u] = VT{};
        doreg[u] = VT{};
      }
    }
    if (tid < QB) {
      const int q = i * QB + tid;
      lreg = lse_log2(q < N ? LSE[q] : -INFINITY);
      dreg = q < N ? DEL[q] : 0.f;
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int u = 0; u < PTQ; ++u) {
      const int cc = tid + 256 * u, row = cc / CPR, col = (cc % CPR) * 8;
      *(VT*)(&qs[buf][row * RS + col]) = qreg[u];
      *(VT*)(&dos[buf][row * RS + col]) = doreg[u];
    }
    if (tid < QB) {
      lsel[buf][tid] = lreg;
      dls[buf][tid] = dreg;
    }
  };

  int i = next_active(i_beg);
  if (i < i_end) {
    gload(i);
    lstore(0);
  }
  __syncthreads();
  int buf = 0;
  while (i < i_end) {
    const int in = next_active(i + 1);
    if (in < i_end) gload(in);
    const int qa = i * QB;
    if (!CAUSAL || qa + QB - 1 >= kw0) {
      f32x16 s = f32x16{}, dp = f32x16{};
      const T* qb_ = qs[buf];
      const T* db_ = dos[buf];
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        const VT qa_ = *(const VT*)(&qb_[l32 * RS + 16 * ds + 8 * g]);
        s = mfma32x32x16(qa_, kf[ds], s);
        const VT da_ = *(const VT*)(&db_[l32 * RS + 16 * ds + 8 * g]);
        dp = mfma32x32x16(da_, vf[ds], dp);
      }
      // Lane: key my_k; register r: query qa + 8*(r/4) + 4*g + r%4.
      const bool need_mask = (kw0 + 32 > N) || (CAUSAL && qa < kw0 + 31);
      // Visible iff query offset (within the tile) >= lim (causal) and key < N.
      const int lim = (my_k >= N) ? (1 << 30) : (CAUSAL ? my_k - qa - 4 * g : -(1 << 30));
      VT pa[2] = {VT{}, VT{}}, dsa[2] = {VT{}, VT{}};
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const float4 l4 = *(const float4*)(&lsel[buf][8 * rg + 4 * g]);
        const float4 d4 = *(const float4*)(&dls[buf][8 * rg + 4 * g]);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
        const float dv4[4] = {d4.x, d4.y, d4.z, d4.w};
        float pv[4], dsv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * rg + e;
          pv[e] = fast_exp2(fmaf(s[r], c, -lv[e]));
          if (need_mask && 8 * rg + e < lim) pv[e] = 0.f;
          dsv[e] = pv[e] * (dp[r] - dv4[e]);
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
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int kk = 0; kk < QB / 16; ++kk) {
          const int row = 16 * kk + 4 * g + (s16 >> 2);
          const int col = 32 * db + 16 * (gq & 1) + 4 * (s16 & 3);
          const VT dof = cat_tr16<VT>(lds_read_tr16(&db_[row * RS + col]),
                                      lds_read_tr16(&db_[(row + 8) * RS + col]));
          dv[db] = mfma32x32x16(pa[kk], dof, dv[db]);
          const VT qf = cat_tr16<VT>(lds_read_tr16(&qb_[row * RS + col]),
                                     lds_read_tr16(&qb_[(row + 8) * RS + col]));
          dk[db] = mfma32x32x16(dsa[kk], qf, dk[db]);
        }
    }
    if (in < i_end) lstore(buf ^ 1);
    __syncthreads();
    buf ^= 1;
    i = in;
  }

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
        dV[(size_t)key * D + 32 * db + l32] = dv[db][r];
      }
    }
}

template <typename T, int D, bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(BwdParams p) {
  using VT = typename V8<T>::t;
  constexpr int BR = 128, BC = 64, RS = D + 8;
  constexpr int DS = D / 16, DB = D / 32;
  constexpr int CPR = D / 8, PT = BC * D / 8 / 256;
  __shared__ __attribute__((aligned(16))) T ks[2][BC * RS];
  __shared__ __attribute__((aligned(16))) T vs[2][BC * RS];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31, s16 = lane & 15, gq = lane >> 4;
  const int N = p.N;
  const int n_qt = (N + BR - 1) / BR;
  const int total = n_qt * p.BH;
  const int lid = xcd_remap(blockIdx.x, total);
  const int bh = lid / n_qt;
  const int ir = lid - bh * n_qt;
  const int qt = CAUSAL ? (n_qt - 1 - ir) : ir;
  const size_t base = (size_t)bh * N * D;
  const T* __restrict__ Q = (const T*)p.q + base;
  const T* __restrict__ K = (const T*)p.k + base;
  const T* __restrict__ V = (const T*)p.v + base;
  const T* __restrict__ dO = (const T*)p.dO + base;
  const int q0 = qt * BR + wave * 32;
  const int my_q = q0 + l32;
  const float c = p.scale_log2e;

  VT qf[DS], dof[DS];
  float lq = INFINITY, dq_row = 0.f;
  if (my_q < N) {
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      qf[ds] = *(const VT*)(Q + (size_t)my_q * D + 16 * ds + 8 * g);
      dof[ds] = *(const VT*)(dO + (size_t)my_q * D + 16 * ds + 8 * g);
    }
    lq = lse_log2(p.lse[(size_t)bh * N + my_q]);
    dq_row = p.delta[(size_t)bh * N + my_q];
  } else {
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      qf[ds] = VT{};
      dof[ds] = VT{};
    }
  }

  const int n_kt = (N + BC - 1) / BC;
  int kt_end = n_kt;
  if (CAUSAL) kt_end = min(kt_end, (min(N, (qt + 1) * BR) + BC - 1) / BC);
  const uint8_t* mrow = SPARSE ? p.mask + (size_t)qt * p.mask_tiles : nullptr;
  auto next_active = [&](int jj) {
    if (SPARSE)
      while (jj < kt_end && mrow[(jj * BC) / MASK_TILE] == 0) ++jj;
    return jj;
  };

  VT kreg[PT], vreg[PT];
  auto gload = [&](int jj) {
#pragma unroll
    for (int u = 0; u < PT; ++u) {
      const int cc = tid + 256 * u, row = cc / CPR, col = (cc % CPR) * 8;
      const int key = jj * BC + row;
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
      const int cc = tid + 256 * u, row = cc / CPR, col = (cc % CPR) * 8;
      *(VT*)(&ks[buf][row * RS + col]) = kreg[u];
      *(VT*)(&vs[buf][row * RS + col]) = vreg[u];
    }
  };

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};

  int jj = next_active(0);
  if (jj < kt_end) {
    gload(jj);
    lstore(0);
  }
  __syncthreads();
  int buf = 0;
  while (jj < kt_end) {
    const int jn = next_active(jj + 1);
    if (jn < kt_end) gload(jn);
    const int k0 = jj * BC;
    if (!CAUSAL || k0 <= q0 + 31) {
      f32x16 s[2] = {f32x16{}, f32x16{}}, dp[2] = {f32x16{}, f32x16{}};
      const T* kb_ = ks[buf];
      const T* vb_ = vs[buf];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
          const VT kfr = *(const VT*)(&kb_[(32 * kb + l32) * RS + 16 * ds + 8 * g]);
          s[kb] = mfma32x32x16(kfr, qf[ds], s[kb]);
          const VT vfr = *(const VT*)(&vb_[(32 * kb + l32) * RS + 16 * ds + 8 * g]);
          dp[kb] = mfma32x32x16(vfr, dof[ds], dp[kb]);
        }
      const bool need_mask = (k0 + BC > N) || (CAUSAL && k0 + BC - 1 > q0);
      int lim = N - 1 - k0;
      if (CAUSAL) lim = min(lim, my_q - k0);
      lim -= 4 * g;
      VT dsf[4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          u32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float dsv[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) {
              const int r = 8 * h + 2 * e + t;
              float pv = fast_exp2(fmaf(s[kb][r], c, -lq));
              if (need_mask && 32 * kb + 8 * (r >> 2) + (r & 3) > lim) pv = 0.f;
              dsv[t] = pv * (dp[kb][r] - dq_row);
            }
            w[e] = pack2<T>(dsv[0], dsv[1]);
          }
          dsf[2 * kb + h] = __builtin_bit_cast(VT, w);
        }
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int row = 16 * kk + 4 * g + (s16 >> 2);
          const int col = 32 * db + 16 * (gq & 1) + 4 * (s16 & 3);
          const VT kt = cat_tr16<VT>(lds_read_tr16(&kb_[row * RS + col]),
                                     lds_read_tr16(&kb_[(row + 8) * RS + col]));
          acc[db] = mfma32x32x16(kt, dsf[kk], acc[db]);
        }
    }
    if (jn < kt_end) lstore(buf ^ 1);
    __syncthreads();
    buf ^= 1;
    jj = jn;
  }

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

template <typename T, int D, bool CAUSAL, bool SPARSE>
hipError_t launch_bwd_t(const BwdParams& p, hipStream_t st) {
  const size_t rows = (size_t)p.BH * p.N;
  const size_t threads = rows * (D / 8);
  bwd_pre_kernel<T, D><<<dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st>>>(
      (const T*)p.o, (const T*)p.dO, p.delta, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  bwd_dkdv_kernel<T, D, CAUSAL, SPARSE><<<dim3(p.n_ktiles * p.BH), dim3(256), 0, st>>>(p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  bwd_dq_kernel<T, D, CAUSAL, SPARSE><<<dim3(((p.N + 127) / 128) * p.BH), dim3(256), 0, st>>>(p);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_bwd(const BwdParams& p, bool causal, bool sparse, hipStream_t st) {
  if (causal && sparse) return launch_bwd_t<T, D, true, true>(p, st);
  if (causal) return launch_bwd_t<T, D, true, false>(p, st);
  if (sparse) return launch_bwd_t<T, D, false, true>(p, st);
  return launch_bwd_t<T, D, false, false>(p, st);
}

}  // namespace

hipError_t launch_backward(BwdParams p, int dtype, int d, bool causal, hipStream_t st) {
  const bool sparse = p.mask != nullptr;
  p.n_ktiles = (p.N + 127) / 128;
  p.n_qtiles = (p.N + 31) / 32;
  if (dtype == DT_BF16)
    return d == 64 ? launch_bwd<__bf16, 64>(p, causal, sparse, st) : launch_bwd<__bf16, 128>(p, causal, sparse, st);
  return d == 64 ? launch_bwd<_Float16, 64>(p, causal, sparse, st) : launch_bwd<_Float16, 128>(p, causal, sparse, st);
}

}  // namespace fa
