// Internal interface between the host API (fa_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

enum { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };
constexpr int MASK_TILE = 128;  // block-mask granularity (rows and columns)
constexpr int FWD_BR = 128;     // query rows per fp32 forward workgroup (== MASK_TILE)
// Build-time alternatives of the tile and occupancy choices below, for
// measuring them against each other (the defaults are the library's
// choices): FA_FWD16_LARGE_GRID (workgroups from which the d = 64 forward
// takes its two-slot form; 0 = always, a huge value = never),
// FA_BWD_WAVES_D64 (2 or 1), FA_BWD_WAVES_D128 (1 or 2), FA_FWD8_WAVES_D64
// (4 or 3), FA_FWD8_WAVES_D128, FA_FP8_PIN_PACKS and FA_DKDV_WAVES_D64
// (below).
#ifndef FA_FWD16_LARGE_GRID
#define FA_FWD16_LARGE_GRID 2048
#endif
#ifndef FA_BWD_WAVES_D64
#define FA_BWD_WAVES_D64 2
#endif
#ifndef FA_BWD_WAVES_D128
#define FA_BWD_WAVES_D128 1
#endif
#ifndef FA_FWD8_WAVES_D64
#define FA_FWD8_WAVES_D64 4
#endif
// FP8 forward: E4M3 packs pinned before the reference check (1) or left to
// the compiler (0: 144 VGPRs at d = 64, three waves per SIMD).
#ifndef FA_FP8_PIN_PACKS
#define FA_FP8_PIN_PACKS 1
#endif
// 16-bit forward: 64-key K/V tiles held in two LDS rings (K and V) of NS
// slots each.  d = 64: NS = 3 (48 KiB, three workgroups per CU, copies issued
// two tiles ahead) for grids below two rounds of four workgroups per CU,
// NS = 2 (32 KiB, four workgroups per CU, copies one tile ahead) from there
// on, without dropout; d = 128: NS = 2 (64 KiB, two workgroups per CU).
constexpr int fwd16_large_grid() { return FA_FWD16_LARGE_GRID; }
// Occupancy the 16-bit forward is compiled for (waves per SIMD).
constexpr int fwd16_waves(int d, int ns) { return d == 64 ? (ns == 3 ? 3 : 4) : 2; }
// Occupancy of the unit-pipelined backward kernels (waves per SIMD): at
// d = 128 one wave holds K, V rows and fp32 dK, dV accumulators (512
// registers) and its workgroup takes most of the CU's LDS.
constexpr int bwd_u_waves(int d) { return d == 64 ? FA_BWD_WAVES_D64 : FA_BWD_WAVES_D128; }
// dK/dV kernel: waves per SIMD at d = 64 may differ from the dQ kernel's
// (three needs its three-slot ring, 51 KiB of LDS per workgroup).
#ifndef FA_DKDV_WAVES_D64
#define FA_DKDV_WAVES_D64 FA_BWD_WAVES_D64
#endif
constexpr int dkdv_waves(int d) { return d == 64 ? FA_DKDV_WAVES_D64 : bwd_u_waves(d); }
// Decode: waves per SIMD (== workgroups per CU).  Each workgroup holds four
// waves' two-slot rings of 32-key K and V tiles: 64 KiB at d = 64, 128 KiB at
// d = 128.
constexpr int dec_waves(int d) { return d == 64 ? 2 : 1; }
constexpr int DEC_MAX_NQ = 16;  // queries per head the decode kernel holds (one MFMA column block)
constexpr int DEC_SPLIT_ALIGN = 128;  // key-range lengths are multiples of 4 waves x 32 keys
// FP8 forward: waves per SIMD (three-slot rings of 64-key E4M3 K and V^T
// tiles: 24 KiB at d = 64, 48 KiB at d = 128).  d = 64 fits four waves in
// 124-126 VGPRs with no spills (the E4M3 packs are pinned before the
// reference check, so the 32 fp32 exponentials die there); d = 128 fits
// three in 167-168 (147 KiB of LDS for three workgroups per CU).
#ifndef FA_FWD8_WAVES_D128
#define FA_FWD8_WAVES_D128 3
#endif
constexpr int fwd8_waves(int d) { return d == 64 ? FA_FWD8_WAVES_D64 : FA_FWD8_WAVES_D128; }
constexpr int FWD_MAX_MASK_TILES = 2048;  // block-mask columns the forward caches (N <= 262144)

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const uint8_t* mask;  // nullptr = dense
  // Block-sparse without the causal flag, 16-bit inputs: query tiles in
  // the order to take them (sparse_order_kernel's), nullptr = index order.
  const int* qt_order;
  int BH, N;
  int n_qtiles, n_ktiles, mask_tiles;
  float scale, scale_log2e;
  float rescale_thr;  // raw-score growth of the running max that forces a rescale
  // Dropout (drop_t8 = 0: none): Philox key, counter word 3, byte threshold,
  // 1 / (1 - drop_t8 / 256).
  uint32_t drop_k0, drop_k1, drop_off, drop_t8;
  float drop_scale;
  // drop != 0 runs the dropout kernels (also with drop_t8 = 0, which keeps
  // every element); they also store O in fp32 to o_acc (B*H, N, d) before its
  // rounding to the input type, when o_acc is not null.
  int drop;
  float* o_acc;
  // Split key ranges (16-bit inputs, no dropout): n_splits > 1 cuts every
  // query tile's key range into n_splits equal runs of tiles, each its own
  // workgroup, which writes its normalised partial output and logsumexp to
  // o_part (B*H, n_splits, N, d) and lse_part (B*H, n_splits, N) -- the
  // decode workspace layout with Nq = N -- for the decode merge kernel.
  int n_splits;
  float* o_part;
  float* lse_part;
};

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dO;
  const float* lse;
  float* dq;
  float* dk;
  float* dv;
  float* neg_delta;  // workspace: -D_i = -sum_c dO_ic o_ic, (B*H, N)
  float* lse2;   // workspace: lse_i * log2(e), +inf for rows with no visible key
  int* qt_order;  // workspace (block-sparse): query tiles, most visible key tiles first
  int* kt_order;  // workspace (block-sparse): key tiles, most visible query tiles first
  const uint8_t* mask;
  int BH, N;
  int n_ktiles, n_qtiles, mask_tiles;
  float scale, scale_log2e;
  uint32_t drop_k0, drop_k1, drop_off, drop_t8;  // dropout as in FwdParams
  float drop_scale;
  // drop != 0 runs the dropout kernels; D_i then comes from o_acc, the
  // forward's fp32 O (B*H, N, d), and o is not read.
  int drop;
  const float* o_acc;
};

struct DecParams {
  const void* q;   // (B*H, Nq, d)
  const void* k;   // (B*H, Nk, d)
  const void* v;
  void* o;         // (B*H, Nq, d), dtype of q
  float* lse;      // (B*H, Nq)
  float* o_part;   // workspace, n_splits > 1: (B*H, n_splits, Nq, d) normalised partial outputs
  float* lse_part; // workspace, n_splits > 1: (B*H, n_splits, Nq) partial logsumexp
  int BH, Nq, Nk;
  int n_splits, split_len;  // key range s = [s * split_len, min(Nk, (s + 1) * split_len))
  float scale_log2e;
};

struct Fp8Params {
  const void* q;  // (B*H, N, d) 16-bit inputs
  const void* k;
  const void* v;
  void* o;        // (B*H, N, d), dtype of q
  float* lse;     // (B*H, N)
  const int8_t* signs;  // d random signs of the rotation, nullptr = no rotation
  // Block-sparse without the causal flag: query tiles in the order to take
  // them (workspace, sparse_order_kernel's), nullptr = index order.
  const int* qt_order;
  // Prepared operands (workspace): Q8, K8 (B*H, Npad, d) E4M3 row-major;
  // V8^T (B*H, n_t64, d, 64) E4M3, keys of a block permuted; one fp32 scale
  // per (b*h, 64-row block) of each.
  uint8_t* q8;
  uint8_t* k8;
  uint8_t* v8t;
  float* sq;
  float* sk;
  float* sv;
  const uint8_t* mask;  // nullptr = dense
  int BH, N, Npad, n_t64, mask_tiles;
  float scale_log2e, rsqrt_d;
  // Preparation: operands prep_z0 .. 2 (0 = Q, 1 = K, 2 = V), one grid row each.
  int prep_z0;
};

struct DropMaskParams {
  uint8_t* keep;   // (B*H, N, N): 1 = kept
  int BH, N;
  uint32_t k0, k1, off, t8;
};

hipError_t launch_forward(FwdParams p, int dtype, int d, bool causal, hipStream_t st);
// Block-sparse work order (fa_bwd.hip): the mask's n row tiles and n column
// tiles ranked by visible tiles, most first (causal: on or below the
// diagonal), into qt_order[n] and kt_order[n].
hipError_t launch_sparse_order(const uint8_t* mask, int n, bool causal, int* qt_order,
                               int* kt_order, hipStream_t st);
hipError_t launch_backward(BwdParams p, int dtype, int d, bool causal, hipStream_t st);
hipError_t launch_decode(DecParams p, int dtype, int d, bool causal, hipStream_t st);
// Merge of per-range partial outputs (o_part, lse_part, n_splits, BH, Nq) into
// o and lse; the decode path's second kernel.
hipError_t launch_split_merge(DecParams p, int dtype, int d, hipStream_t st);
hipError_t launch_dropout_mask(DropMaskParams p, hipStream_t st);
hipError_t launch_fp8(Fp8Params p, int dtype, int d, bool causal, bool prep, bool attend,
                      hipStream_t st);

}  // namespace fa
