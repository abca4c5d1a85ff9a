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
// Kernels:
//   bwd_pre:  D = rowsum(dO o O) in fp32 into the workspace, and dq := 0.
//   bwd_main: one workgroup per (key tile of 128, batch*head); wave w owns 32
//     keys, keeps its K and V rows in VGPRs and its dK, dV in fp32
//     accumulators, and loops over the query tiles of 32 rows that can see
//     them (causal: query tiles at or after the key tile; block-sparse: mask
//     entries that are set).  Per query tile:
//       S = Q K^T and dP = dO V^T on v_mfma_f32_32x32x16 (lane = key, so the
//       P^T and dS^T operands of dV += P^T dO and dK += dS^T Q come straight
//       from the accumulators; dO and Q are read with ds_read_b64_tr_b16),
//       dS^T of all four waves is staged in LDS, and dQ_tile += scale dS K is
//       computed on v_mfma_f32_16x16x32 split over the waves and added to the
//       fp32 dq with global atomics.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

namespace {

template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const T* __restrict__ O, const T* __restrict__ dO,
                                                      float* __restrict__ delta, float* __restrict__ dq,
                                                      size_t rows) {
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
    float4* z = (float4*)(dq + row * D + part * 8);
    z[0] = make_float4(0.f, 0.f, 0.f, 0.f);
    z[1] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && part == 0) delta[row] = acc;
}

template <typename T, int D, bool CAUSAL, bool SPARSE>
__global__ __launch_bounds__(256, 1) void bwd_main_kernel(BwdParams p) {
  using VT = typename V8<T>::t;
  using HT = typename V8<T>::h;
  constexpr int BC = 128, QB = 32, RS = D + 8, RST = QB + 8;
  constexpr int DS = D / 16, DB = D / 32;
  constexpr int CPR = D / 8, PTQ = QB * D / 8 / 256, PTK = BC * D / 8 / 256;
  constexpr int NQB16 = QB / 16, NDB16 = D / 16, DQ_PER_WAVE = NQB16 * NDB16 / 4;
  constexpr float LOG2E = 1.4426950408889634f;
  __shared__ __attribute__((aligned(16))) T qs[2][QB * RS];
  __shared__ __attribute__((aligned(16))) T dos[2][QB * RS];
  __shared__ __attribute__((aligned(16))) T kls[BC * RS];
  __shared__ __attribute__((aligned(16))) T dst[BC * RST];
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
  float* __restrict__ dQ = p.dq + base;
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
#pragma unroll
  for (int u = 0; u < PTK; ++u) {
    const int cc = tid + 256 * u, row = cc / CPR, col = (cc % CPR) * 8;
    const int key = k0 + row;
    *(VT*)(&kls[row * RS + col]) = key < N ? *(const VT*)(K + (size_t)key * D + col) : VT{};
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
      // log2-domain statistic; +inf makes P = 0 for padding rows and for
      // rows with no visible key (lse = -inf).
      const float l = q < N ? LSE[q] : -INFINITY;
      lreg = l == -INFINITY ? INFINITY : l * LOG2E;
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
    T* dsrow = &dst[(32 * wave + l32) * RST];
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
      // lane: key my_k; register r: query qa + 8*(r/4) + 4*g + r%4
      const bool need_mask = (kw0 + 32 > N) || (CAUSAL && qa < kw0 + 31);
      VT pa[2], dsa[2];
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const float4 l4 = *(const float4*)(&lsel[buf][8 * rg + 4 * g]);
        const float4 d4 = *(const float4*)(&dls[buf][8 * rg + 4 * g]);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
        const float dv4[4] = {d4.x, d4.y, d4.z, d4.w};
        HT hs;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * rg + e;
          float pv = fast_exp2(fmaf(s[r], c, -lv[e]));
          if (need_mask) {
            const int qi = qa + 8 * rg + 4 * g + e;
            if (my_k >= N || (CAUSAL && my_k > qi)) pv = 0.f;
          }
          const float dsv = pv * (dp[r] - dv4[e]);
          pa[r >> 3][r & 7] = (T)pv;
          dsa[r >> 3][r & 7] = (T)dsv;
          hs[e] = (T)dsv;
        }
        *(HT*)(dsrow + 8 * rg + 4 * g) = hs;
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
    } else {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) *(HT*)(dsrow + 8 * rg + 4 * g) = HT{};
    }
    __syncthreads();
    // dQ[qa .. qa+31][:] += scale * dS K over this tile's 128 keys.
#pragma unroll
    for (int t = 0; t < DQ_PER_WAVE; ++t) {
      const int b = wave * DQ_PER_WAVE + t;
      const int qb = b / NDB16, dbk = b % NDB16;
      f32x4 acc = f32x4{};
#pragma unroll
      for (int ks = 0; ks < BC / 32; ++ks) {
        const int kb = 32 * ks + 8 * gq + (s16 >> 2);
        const VT af = cat_tr16<VT>(lds_read_tr16(&dst[kb * RST + 16 * qb + 4 * (s16 & 3)]),
                                   lds_read_tr16(&dst[(kb + 4) * RST + 16 * qb + 4 * (s16 & 3)]));
        const VT bf = cat_tr16<VT>(lds_read_tr16(&kls[kb * RS + 16 * dbk + 4 * (s16 & 3)]),
                                   lds_read_tr16(&kls[(kb + 4) * RS + 16 * dbk + 4 * (s16 & 3)]));
        acc = mfma16x16x32(af, bf, acc);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int q = qa + 16 * qb + 4 * gq + r;
        if (q < N) unsafeAtomicAdd(&dQ[(size_t)q * D + 16 * dbk + s16], acc[r] * p.scale);
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

template <typename T, int D>
hipError_t launch_bwd(const BwdParams& p, bool causal, bool sparse, hipStream_t st) {
  const size_t rows = (size_t)p.BH * p.N;
  const size_t threads = rows * (D / 8);
  bwd_pre_kernel<T, D><<<dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st>>>(
      (const T*)p.o, (const T*)p.dO, p.delta, p.dq, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 grid(p.n_ktiles * p.BH), block(256);
  if (causal && sparse) bwd_main_kernel<T, D, true, true><<<grid, block, 0, st>>>(p);
  else if (causal) bwd_main_kernel<T, D, true, false><<<grid, block, 0, st>>>(p);
  else if (sparse) bwd_main_kernel<T, D, false, true><<<grid, block, 0, st>>>(p);
  else bwd_main_kernel<T, D, false, false><<<grid, block, 0, st>>>(p);
  return hipGetLastError();
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
