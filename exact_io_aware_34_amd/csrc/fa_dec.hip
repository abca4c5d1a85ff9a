// Decode-time attention on gfx950: a few queries (1 <= Nq <= 16) per head
// against a long key/value history, with the key range split over many
// workgroups and the per-range results merged afterwards.
//
// What is computed: the forward definition for the last Nq positions of a
// sequence of Nk cached keys and values.  Decoding has one (or a few) new
// queries and a long history, so the work is a scan over K and V that is
// parallelised along the keys ("Что это изменило на практике", sloger.press
// page).  The causal rule is the square one shifted to the end of the
// sequence: query i sits at position Nk - Nq + i ("Le masquage causal",
// marketmaker.cc page).  Each workgroup runs the online-softmax recurrence
// over its key range and returns a normalised partial output with its
// logsumexp; the partials are merged with the (m, l) identity of the
// incremental softmax ("Rastreamento Incremental do Softmax", xyznot.com
// reading guide): lse = ln sum_s exp(lse_s), o = sum_s exp(lse_s - lse) o_s.
//
// gfx950 mapping.  The scan reads 4 * d bytes per key (16-bit K and V) and
// does O(Nq * d) arithmetic on them, so it is bound by HBM bandwidth, not by
// the matrix cores; the kernel is organised to keep many bytes in flight
// with no workgroup barrier in the key loop:
//   * 256 threads = 4 waves per workgroup, one workgroup per (batch*head,
//     key range).  Waves take 32-key steps of the range round robin and keep
//     their own online-softmax state; the four states merge once at the end.
//   * Each wave owns a two-slot LDS ring; a step's K and V rows (32 x d each)
//     arrive by direct global->LDS copies issued one step ahead, so only the
//     wave's own vmcnt is waited on.  The copies use the non-temporal cache
//     policy: every K/V byte is read once per call.
//   * Scores are S^T = K Q^T on v_mfma_f32_16x16x32 with the queries padded to
//     16 columns (Q^T stays in VGPRs): lane l holds query l % 16 at 8 of the
//     32 keys, which are exactly the 8 contraction slots it supplies to
//     O^T += V^T P^T, so P needs no shuffle.  V^T comes from
//     ds_read_b64_tr_b16 transpose reads.
//   * Row max: in-lane over 8 values, then across the four 16-lane groups
//     (ds_swizzle xor 16, permlane32 swap).  exp is exp2 with scale*log2(e)
//     folded into one FMA.
#include <type_traits>

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

namespace {

constexpr int DEC_STEP = 32;   // keys per wave step
constexpr int DEC_NW = 4;      // waves per workgroup

// LDS swizzles of the decode tiles (rows of D 16-bit elements, 16-byte
// chunks; XOR keeps them involutions).  K is read 16 consecutive rows at one
// chunk per pass, so it uses the forward's swizzle.  V is read by transpose
// reads that cover 8 consecutive rows x 2 adjacent chunks per pass: shifting
// the chunk pair by the row puts every lane of a pass in its own bank.
template <int D>
__device__ __forceinline__ int dec_swz_v(int r) {
  if constexpr (D == 64) return 2 * ((r >> 1) & 3);
  else return 2 * (r & 7);
}

__device__ __forceinline__ float xor16_max(float x) {
  // ds_swizzle bit mode: and 0x1f, or 0, xor 0x10 (within 32 lanes).
  return fmaxf(x, __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F)));
}
__device__ __forceinline__ float xor16_sum(float x) {
  return x + __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F));
}

template <typename T, int D, bool CAUSAL, bool SPLIT>
__global__ __launch_bounds__(256, dec_waves(D)) void dec_kernel(DecParams p) {
  using VT = typename V8<T>::t;
  constexpr int NW = DEC_NW, BK = DEC_STEP;
  constexpr int CPR = D / 8;                 // 16-byte chunks per row
  constexpr int TILE = BK * D;               // elements of one K (or V) step tile
  constexpr int DMA_N = BK * CPR / 64;       // copies per tile (one wave)
  constexpr int DH = D / 32, DB = D / 16;    // k-chunks of the score product; O^T blocks
  constexpr int WAVE_ELEMS = 4 * TILE;       // ring: K0 V0 K1 V1
  static_assert(WAVE_ELEMS * (int)sizeof(T) >= 16 * D * (int)sizeof(float),
                "the merge reuses a wave's ring for its 16 x D fp32 partial");
  __shared__ __attribute__((aligned(1024))) T ring[NW * WAVE_ELEMS];
  __shared__ float st_m[NW][16], st_l[NW][16];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, s16 = lane & 15;
  const int S = p.n_splits;
  const int bh = blockIdx.x / S, split = blockIdx.x - bh * S;
  const int Nq = p.Nq, Nk = p.Nk;
  const T* __restrict__ K = (const T*)p.k + (size_t)bh * Nk * D;
  const T* __restrict__ V = (const T*)p.v + (size_t)bh * Nk * D;
  const int k_beg = split * p.split_len;
  const int k_end = min(Nk, k_beg + p.split_len);
  const int n_steps = (k_end - k_beg + BK - 1) / BK;
  const int n_w = n_steps > wave ? (n_steps - wave + NW - 1) / NW : 0;
  // Key j is visible to every real query iff j <= all_key; to query q iff
  // j <= all_key + q (causal), and to all of them without the causal flag.
  const int all_key = CAUSAL ? Nk - Nq : Nk - 1;
  const float c = p.scale_log2e;

  T* const wring = ring + wave * WAVE_ELEMS;
  const uint32_t wlds = lds_addr(wring);
  // Copy schedule: copy u of a tile fills physical chunk 64u + lane, i.e.
  // row r, logical chunk (pch % CPR) ^ swizzle(r).
  int drow[DMA_N], kcol[DMA_N], vcol[DMA_N];
#pragma unroll
  for (int u = 0; u < DMA_N; ++u) {
    const int pch = 64 * u + lane;
    const int r = pch / CPR, pc = pch % CPR;
    drow[u] = r;
    kcol[u] = 8 * (pc ^ swz<D>(r));
    vcol[u] = 8 * (pc ^ dec_swz_v<D>(r));
  }
  // Step i of this wave covers keys k_beg + 32 * (wave + 4 i) ...; slot i & 1.
  auto issue = [&](int i) {
    const int k0 = k_beg + BK * (wave + NW * i);
    const uint32_t kdst = wlds + (uint32_t)((2 * (i & 1)) * TILE * (int)sizeof(T));
    const uint32_t vdst = kdst + (uint32_t)(TILE * (int)sizeof(T));
    if (k0 + BK <= Nk) {
      const T* kb = K + (size_t)k0 * D;
      const T* vb = V + (size_t)k0 * D;
#pragma unroll
      for (int u = 0; u < DMA_N; ++u)
        dma16_s_stream(kb, (uint32_t)((drow[u] * D + kcol[u]) * (int)sizeof(T)), kdst + 1024u * u);
#pragma unroll
      for (int u = 0; u < DMA_N; ++u)
        dma16_s_stream(vb, (uint32_t)((drow[u] * D + vcol[u]) * (int)sizeof(T)), vdst + 1024u * u);
    } else {
      // Rows past Nk read row Nk - 1: their scores are masked to -inf and
      // their values meet probability 0.
#pragma unroll
      for (int u = 0; u < DMA_N; ++u) {
        const size_t row = (size_t)min(k0 + drow[u], Nk - 1) * D;
        dma16_stream(K + row + kcol[u], kdst + 1024u * u);
        dma16_stream(V + row + vcol[u], vdst + 1024u * u);
      }
    }
  };

  if (n_w > 0) issue(0);
  if (n_w > 1) issue(1);

  // Q^T (B operand): lane holds query s16, elements 32 h + 8 g .. + 7; the
  // padding queries are zero.
  VT qf[DH];
  {
    const T* Q = (const T*)p.q + ((size_t)bh * Nq + s16) * D;
#pragma unroll
    for (int h = 0; h < DH; ++h) qf[h] = s16 < Nq ? *(const VT*)(Q + 32 * h + 8 * g) : VT{};
  }
  // The compiler sees these loads complete here, so it adds no wait inside
  // the copy-pipelined loop (this also waits for the first two steps).
  wait_all_loads();

  // Per-lane LDS element offsets.  K (A operand of S^T): key 16 b + s16,
  // chunk 4 h + g.  V^T (A operand of O^T): transpose read of rows
  // 16 hh + 4 g + s16 / 4, columns 16 db + 4 (s16 % 4).
  int koff[2][DH], voff[DB][2];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int h = 0; h < DH; ++h) {
      const int r = 16 * b + s16, ch = 4 * h + g;
      koff[b][h] = r * D + 8 * (ch ^ swz<D>(r));
    }
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int r = 16 * hh + 4 * g + (s16 >> 2), col = 16 * db + 4 * (s16 & 3);
      voff[db][hh] = r * D + 8 * ((col >> 3) ^ dec_swz_v<D>(r)) + (col & 7);
    }

  f32x4 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x4{};
  float m_run = -INFINITY;   // running max of the raw scores of query s16
  float l_run = 0.f;         // this lane's share of the running sum

  for (int i = 0; i < n_w; ++i) {
    if (i + 1 < n_w) wait_vmcnt<2 * DMA_N>();
    else wait_vmcnt<0>();
    const T* kt = wring + 2 * (i & 1) * TILE;
    const T* vt = kt + TILE;
    const int k0 = k_beg + BK * (wave + NW * i);
    // S^T for keys k0 + 16 b + 4 g + r (r = 0..3) of query s16.
    f32x4 s[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      s[b] = f32x4{};
#pragma unroll
      for (int h = 0; h < DH; ++h) s[b] = mfma16x16x32(*(const VT*)(kt + koff[b][h]), qf[h], s[b]);
    }
    if (k0 + BK > k_end || k0 + BK - 1 > all_key) {
      const int lim = min(k_end - 1, CAUSAL ? all_key + s16 : all_key) - k0 - 4 * g;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (16 * b + r > lim) s[b][r] = -INFINITY;
    }
    float mx = fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3]));
    mx = fmaxf(mx, fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
    mx = half_swap_max(xor16_max(mx));
    const float m_new = fmaxf(m_run, mx);
    // With no visible key yet the reference is 0: every exponential is then
    // exp2(-inf) = 0 and O, l stay 0.
    const float mc = m_new == -INFINITY ? 0.f : m_new * c;
    const float alpha = fast_exp2(fmaf(m_run, c, -mc));
    m_run = m_new;
    u32x4 pw;
    float ls = 0.f;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float e0 = fast_exp2(fmaf(s[b][2 * e], c, -mc));
        const float e1 = fast_exp2(fmaf(s[b][2 * e + 1], c, -mc));
        ls += e0 + e1;
        pw[2 * b + e] = pack2<T>(e0, e1);
      }
    l_run = fmaf(l_run, alpha, ls);
    const VT pf = __builtin_bit_cast(VT, pw);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const VT vf = cat_tr16<VT>(lds_read_tr16(vt + voff[db][0]), lds_read_tr16(vt + voff[db][1]));
      o[db] = mfma16x16x32(vf, pf, o[db] * alpha);
    }
    // Every LDS read of this slot has completed before the next copy into it.
    if (i + 2 < n_w) {
      lds_reads_done();
      issue(i + 2);
    }
  }

  // Merge the four waves: reference max M, weights exp(m_w - M).
  const float lt = half_swap_sum(xor16_sum(l_run));
  if (g == 0) {
    st_m[wave][s16] = m_run;
    st_l[wave][s16] = lt;
  }
  lds_reads_done();
  float* po = (float*)wring;  // this wave's ring, now idle: [16][D] fp32
#pragma unroll
  for (int db = 0; db < DB; ++db) *(f32x4*)(po + s16 * D + 16 * db + 4 * g) = o[db];
  __syncthreads();

  const size_t row0 = SPLIT ? ((size_t)bh * S + split) * Nq : (size_t)bh * Nq;
  for (int idx = tid; idx < Nq * D; idx += 256) {
    const int q = idx / D, d = idx - q * D;
    float M = st_m[0][q];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, st_m[w][q]);
    float ov = 0.f, lse = -INFINITY;
    if (M != -INFINITY) {
      const float Mc = M * c;
      float L = 0.f, acc = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float wt = fast_exp2(fmaf(st_m[w][q], c, -Mc));
        L = fmaf(wt, st_l[w][q], L);
        acc = fmaf(wt, ((const float*)(ring + w * WAVE_ELEMS))[q * D + d], acc);
      }
      ov = acc / L;
      lse = (Mc + __log2f(L)) * 0.69314718055994531f;
    }
    if (SPLIT) {
      p.o_part[(row0 + q) * D + d] = ov;
      if (d == 0) p.lse_part[row0 + q] = lse;
    } else {
      ((T*)p.o)[(row0 + q) * D + d] = (T)ov;
      if (d == 0) p.lse[row0 + q] = lse;
    }
  }
}

// Merge of the key ranges: one thread per (row, column), D threads per row.
// The ranges are read in groups of MG, every load of a group issued before
// any is used, so a row costs two memory round trips per group (one for the
// max of the range statistics, one for the weighted sum) rather than two
// per range.
template <typename T, int D>
__global__ __launch_bounds__(256) void dec_combine_kernel(DecParams p) {
  constexpr int RPB = 256 / D, MG = 8;
  const int row = blockIdx.x * RPB + threadIdx.x / D, d = threadIdx.x % D;
  const int rows = p.BH * p.Nq;
  if (row >= rows) return;
  const int S = p.n_splits, Nq = p.Nq;
  const int bh = row / Nq, q = row - bh * Nq;
  const size_t r0 = (size_t)bh * S * Nq + q;   // partial row of range 0; stride Nq
  float M = -INFINITY;
  for (int s0 = 0; s0 < S; s0 += MG) {
    float lv[MG];
#pragma unroll
    for (int j = 0; j < MG; ++j)
      lv[j] = s0 + j < S ? p.lse_part[r0 + (size_t)(s0 + j) * Nq] : -INFINITY;
#pragma unroll
    for (int j = 0; j < MG; ++j) M = fmaxf(M, lv[j]);
  }
  float ov = 0.f, lse = -INFINITY;
  if (M != -INFINITY) {
    constexpr float kLog2e = 1.4426950408889634f;
    float W = 0.f, acc = 0.f;
    for (int s0 = 0; s0 < S; s0 += MG) {
      float lv[MG], xv[MG];
#pragma unroll
      for (int j = 0; j < MG; ++j) {
        const size_t r = r0 + (size_t)(s0 + j) * Nq;
        lv[j] = s0 + j < S ? p.lse_part[r] : -INFINITY;
        xv[j] = s0 + j < S ? p.o_part[r * D + d] : 0.f;
      }
#pragma unroll
      for (int j = 0; j < MG; ++j) {
        const float wt = fast_exp2((lv[j] - M) * kLog2e);
        W += wt;
        acc = fmaf(wt, xv[j], acc);
      }
    }
    ov = acc / W;
    lse = M + __logf(W);
  }
  ((T*)p.o)[(size_t)row * D + d] = (T)ov;
  if (d == 0) p.lse[row] = lse;
}

template <typename T, int D, bool CAUSAL>
hipError_t launch_dec_t(const DecParams& p, hipStream_t st) {
  const dim3 grid((unsigned)(p.BH * p.n_splits));
  if (p.n_splits == 1) {
    hipLaunchKernelGGL((dec_kernel<T, D, CAUSAL, false>), grid, dim3(256), 0, st, p);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((dec_kernel<T, D, CAUSAL, true>), grid, dim3(256), 0, st, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int rows = p.BH * p.Nq, rpb = 256 / D;
  hipLaunchKernelGGL((dec_combine_kernel<T, D>), dim3((unsigned)((rows + rpb - 1) / rpb)), dim3(256),
                     0, st, p);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_dec_d(const DecParams& p, bool causal, hipStream_t st) {
  return causal ? launch_dec_t<T, D, true>(p, st) : launch_dec_t<T, D, false>(p, st);
}

template <typename T>
hipError_t launch_dec_dt(const DecParams& p, int d, bool causal, hipStream_t st) {
  return d == 64 ? launch_dec_d<T, 64>(p, causal, st) : launch_dec_d<T, 128>(p, causal, st);
}

}  // namespace

hipError_t launch_split_merge(DecParams p, int dtype, int d, hipStream_t st) {
  const int rows = p.BH * p.Nq, rpb = 256 / d;
  const dim3 grid((unsigned)((rows + rpb - 1) / rpb));
  if (dtype == DT_BF16) {
    if (d == 64) hipLaunchKernelGGL((dec_combine_kernel<__bf16, 64>), grid, dim3(256), 0, st, p);
    else hipLaunchKernelGGL((dec_combine_kernel<__bf16, 128>), grid, dim3(256), 0, st, p);
  } else if (dtype == DT_F32) {
    if (d == 64) hipLaunchKernelGGL((dec_combine_kernel<float, 64>), grid, dim3(256), 0, st, p);
    else hipLaunchKernelGGL((dec_combine_kernel<float, 128>), grid, dim3(256), 0, st, p);
  } else {
    if (d == 64) hipLaunchKernelGGL((dec_combine_kernel<_Float16, 64>), grid, dim3(256), 0, st, p);
    else hipLaunchKernelGGL((dec_combine_kernel<_Float16, 128>), grid, dim3(256), 0, st, p);
  }
  return hipGetLastError();
}

hipError_t launch_decode(DecParams p, int dtype, int d, bool causal, hipStream_t st) {
  if (dtype == DT_BF16) return launch_dec_dt<__bf16>(p, d, causal, st);
  return launch_dec_dt<_Float16>(p, d, causal, st);
}

}  // namespace fa
