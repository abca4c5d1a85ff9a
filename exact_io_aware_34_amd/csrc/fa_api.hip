// Host side of libfa.so: argument validation and kernel dispatch for the C ABI
// declared in include/fa.h.  Every check runs before anything is enqueued; an
// unsupported request returns an error and never runs another code path.
#include <algorithm>
#include <cmath>
#include <cstdint>

#include "../../include/fa.h"
#include "fa_kernels.h"

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMaxForwardSplits = 64;  // key ranges per query tile in fa_forward_split

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_common(int B, int H, int N, int d, float scale, int dtype) {
  if (B < 1 || H < 1 || N < 1 || d < 1) return FA_ERR_INVALID_ARG;
  if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  // Grid sizes and per-head element counts must fit the kernels' int indexing.
  const long long bh = (long long)B * H;
  if (bh > (1LL << 24) || (long long)N * d > (1LL << 31) - 1) return FA_ERR_UNSUPPORTED;
  if (bh * ((N + 31) / 32) > (1LL << 31) - 1) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

int tensor_ptr_ok(const void* p) { return p != nullptr && aligned(p, 16); }

size_t delta_bytes(int B, int H, int N) {
  const size_t b = (size_t)B * H * N * sizeof(float);
  return (b + 255) / 256 * 256;
}

size_t order_bytes(int N) {
  const size_t b = 2 * (size_t)((N + 127) / 128) * sizeof(int);
  return (b + 255) / 256 * 256;
}

// Decode key ranges.  With n_splits = 0 the count aims at about 192
// (b*h, range) workgroups -- one workgroup on each of three quarters of the
// 256 CUs -- with ranges no shorter than 512 keys.  Measured on the decode
// scan: one workgroup per CU streams fastest, and a count that puts two
// workgroups on some CUs but one on others ends in a tail on the doubly
// loaded ones.  Ranges are a multiple of 128 keys long; the count actually
// used is ceil(Nk / range length).
struct DecSplit {
  int n, len;
};

DecSplit dec_split(int B, int H, int Nk, int n_splits) {
  constexpr long long kTargetWGs = 192, kMinLen = 512;
  const long long bh = (long long)B * H;
  long long want = n_splits;
  if (want <= 0) {
    want = std::max(1LL, (kTargetWGs + bh / 2) / bh);
    want = std::min(want, std::max(1LL, (Nk + kMinLen - 1) / kMinLen));
  }
  want = std::min(want, (long long)((Nk + fa::DEC_SPLIT_ALIGN - 1) / fa::DEC_SPLIT_ALIGN));
  long long len = (Nk + want - 1) / want;
  len = (len + fa::DEC_SPLIT_ALIGN - 1) / fa::DEC_SPLIT_ALIGN * fa::DEC_SPLIT_ALIGN;
  return {(int)((Nk + len - 1) / len), (int)len};
}

size_t pad256(size_t b) { return (b + 255) / 256 * 256; }

int check_decode(int B, int H, int Nq, int Nk, int d, float scale, int dtype, int n_splits) {
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || d < 1 || n_splits < 0) return FA_ERR_INVALID_ARG;
  if (Nq > Nk) return FA_ERR_INVALID_ARG;
  if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (dtype == FA_F32 || Nq > fa::DEC_MAX_NQ) return FA_ERR_UNSUPPORTED;
  const long long bh = (long long)B * H;
  if ((long long)Nk * d > (1LL << 31) - 1 || bh * Nk > (1LL << 31) - 1) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

// Dropout: byte threshold t = round(256 p) (clamped to 255) and the scale
// 1 / (1 - t / 256) of the kept values.  Returns false for p outside [0, 1).
bool dropout_args(float p, uint64_t seed, uint32_t offset, uint32_t& k0, uint32_t& k1,
                  uint32_t& off, uint32_t& t8, float& scale) {
  if (!std::isfinite(p) || p < 0.f || p >= 1.f) return false;
  t8 = (uint32_t)std::min(255.0, std::floor((double)p * 256.0 + 0.5));
  scale = (float)(256.0 / (256.0 - (double)t8));
  k0 = (uint32_t)(seed & 0xFFFFFFFFu);
  k1 = (uint32_t)(seed >> 32);
  off = offset;
  return true;
}

int forward_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                 int N, int d, float scale, int causal, const uint8_t* block_mask, int dtype,
                 bool drop, float dropout_p, uint64_t seed, uint32_t offset, float* o_acc,
                 int* order, void* stream);
int backward_impl(const void* q, const void* k, const void* v, const void* o, const void* dO,
                  const float* lse, float* dq, float* dk, float* dv, int B, int H, int N, int d,
                  float scale, int causal, const uint8_t* block_mask, int dtype, bool drop,
                  float dropout_p, uint64_t seed, uint32_t offset, const float* o_acc,
                  void* workspace, size_t workspace_bytes, void* stream);

// FP8 workspace regions, in order, each padded to 256 bytes.
struct Fp8Layout {
  size_t q8, k8, v8t, sq, sk, sv, order, total;
};

Fp8Layout fp8_layout(int B, int H, int N, int d) {
  const size_t bh = (size_t)B * H, nt = ((size_t)N + 63) / 64;
  const size_t op = pad256(bh * nt * 64 * d), sc = pad256(bh * nt * sizeof(float));
  Fp8Layout l{};
  l.q8 = 0;
  l.k8 = op;
  l.v8t = 2 * op;
  l.sq = 3 * op;
  l.sk = 3 * op + sc;
  l.sv = 3 * op + 2 * sc;
  l.order = 3 * op + 3 * sc;
  l.total = l.order + order_bytes(N);
  return l;
}

int fp8_setup(fa::Fp8Params& p, const void* q, const void* k, const void* v, int B, int H, int N,
              int d, float scale, int dtype, const int8_t* signs, void* workspace,
              size_t workspace_bytes) {
  if (!tensor_ptr_ok(q) || !tensor_ptr_ok(k) || !tensor_ptr_ok(v)) return FA_ERR_INVALID_ARG;
  if (signs != nullptr && !aligned(signs, 16)) return FA_ERR_INVALID_ARG;
  const int rc = check_common(B, H, N, d, scale, dtype);
  if (rc != FA_OK) return rc;
  if (dtype == FA_F32) return FA_ERR_UNSUPPORTED;
  const Fp8Layout l = fp8_layout(B, H, N, d);
  if (workspace == nullptr || !aligned(workspace, 256) || workspace_bytes < l.total)
    return FA_ERR_WORKSPACE;
  char* w = (char*)workspace;
  p.q = q;
  p.k = k;
  p.v = v;
  p.signs = signs;
  p.q8 = (uint8_t*)(w + l.q8);
  p.k8 = (uint8_t*)(w + l.k8);
  p.v8t = (uint8_t*)(w + l.v8t);
  p.sq = (float*)(w + l.sq);
  p.sk = (float*)(w + l.sk);
  p.sv = (float*)(w + l.sv);
  p.BH = B * H;
  p.N = N;
  p.n_t64 = (N + 63) / 64;
  p.Npad = 64 * p.n_t64;
  p.mask_tiles = (N + fa::MASK_TILE - 1) / fa::MASK_TILE;
  p.scale_log2e = scale * kLog2e;
  p.rsqrt_d = 1.0f / std::sqrt((float)d);
  return FA_OK;
}

}  // namespace

extern "C" {

int fa_abi_version(void) { return 6; }

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_INVALID_ARG: return "invalid argument (null or misaligned pointer, bad size or dtype, scale not finite and > 0)";
    case FA_ERR_UNSUPPORTED: return "unsupported request (head dim must be 64 or 128; size limits; dtype)";
    case FA_ERR_WORKSPACE: return "workspace missing or smaller than the size its *_workspace_size() call returns";
    case FA_ERR_HIP: return "HIP runtime error at kernel launch";
    default: return "unknown status";
  }
}

int fa_forward(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int N, int d, float scale, int causal,
               const uint8_t* block_mask, int dtype, void* stream) {
  return forward_impl(q, k, v, o, lse, B, H, N, d, scale, causal, block_mask, dtype, false, 0.f, 0,
                      0, nullptr, nullptr, stream);
}

int fa_forward_dropout(const void* q, const void* k, const void* v, void* o, float* lse,
                       int B, int H, int N, int d, float scale, int causal,
                       const uint8_t* block_mask, int dtype, float dropout_p, uint64_t seed,
                       uint32_t offset, float* o_acc, void* stream) {
  return forward_impl(q, k, v, o, lse, B, H, N, d, scale, causal, block_mask, dtype, true,
                      dropout_p, seed, offset, o_acc, nullptr, stream);
}

}  // extern "C"

namespace {

// The block-sparse forward without the causal flag (16-bit inputs) takes a
// head's query tiles in the backward's work order, ranked by
// sparse_order_kernel into `order` (two int32 per 128-row tile) before the
// forward kernel runs.  Other calls keep the index order.
hipError_t sparse_forward_order(fa::FwdParams& p, int causal, int dtype, int* order,
                                hipStream_t st) {
  if (p.mask == nullptr || causal != 0 || dtype == FA_F32) return hipSuccess;
  p.qt_order = order;
  return fa::launch_sparse_order(p.mask, p.mask_tiles, false, order, order + p.mask_tiles, st);
}

int forward_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                 int N, int d, float scale, int causal, const uint8_t* block_mask, int dtype,
                 bool drop, float dropout_p, uint64_t seed, uint32_t offset, float* o_acc,
                 int* order, void* stream) {
  if (!tensor_ptr_ok(q) || !tensor_ptr_ok(k) || !tensor_ptr_ok(v) || !tensor_ptr_ok(o))
    return FA_ERR_INVALID_ARG;
  if (lse == nullptr || !aligned(lse, 4)) return FA_ERR_INVALID_ARG;
  if (o_acc != nullptr && !aligned(o_acc, 16)) return FA_ERR_INVALID_ARG;
  const int rc = check_common(B, H, N, d, scale, dtype);
  if (rc != FA_OK) return rc;
  if (block_mask != nullptr && (N + fa::MASK_TILE - 1) / fa::MASK_TILE > fa::FWD_MAX_MASK_TILES)
    return FA_ERR_UNSUPPORTED;
  fa::FwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.mask = block_mask;
  p.BH = B * H;
  p.N = N;
  p.mask_tiles = (N + fa::MASK_TILE - 1) / fa::MASK_TILE;
  p.scale = scale;
  p.scale_log2e = scale * kLog2e;
  p.rescale_thr = 8.0f / p.scale_log2e;  // 2^8 headroom for the exponentials
  if (!dropout_args(dropout_p, seed, offset, p.drop_k0, p.drop_k1, p.drop_off, p.drop_t8,
                    p.drop_scale))
    return FA_ERR_INVALID_ARG;
  // The dropout kernels run when something is dropped or the fp32 O is asked
  // for; with nothing dropped and no fp32 O the plain kernel gives the same O.
  p.drop = drop && (p.drop_t8 > 0 || o_acc != nullptr);
  p.o_acc = o_acc;
  if (p.drop && dtype == FA_F32) return FA_ERR_UNSUPPORTED;
  if (order != nullptr) {
    const hipError_t e = sparse_forward_order(p, causal, dtype, order, (hipStream_t)stream);
    if (e != hipSuccess) return FA_ERR_HIP;
  }
  const hipError_t e = fa::launch_forward(p, dtype, d, causal != 0, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

// Key runs of the split forward.  n_splits = 0 picks a count for grids
// smaller than one full round of workgroups (768 at d = 64: three per CU;
// 512 at d = 128: two): enough (query tile, run) workgroups for one round,
// with runs of at least ten 64-key tiles.  In a sweep of the count (1..32)
// on five 16-bit shapes (one to four heads, N = 4096..16384, d = 64 and 128,
// causal and not) this choice was the fastest count on every one; runs
// shorter than ~10 tiles spend most of their time filling and draining the
// copy pipeline.  An fp32 tile costs the matrix cores ~16 times as long, so
// for fp32 inputs one 64-key tile per run already covers the fill and one
// workgroup per CU (256) is enough: one head at d = 64 took 89.8 us in one
// run, 21.3 in eight and 19.6 in sixteen at N = 1024, 30.4 us in two, 20.3
// in four and 19.4 in eight at N = 512, 27.3 us in one and 20 in two or
// four at N = 256, and 57.5 us in eight (its count here) against 59.8-85.7
// in 16-64 at N = 4096.  An explicit count is capped at the number of
// 64-key tiles.
int forward_split_count(int B, int H, int N, int d, int n_splits, int dtype) {
  if (B < 1 || H < 1 || N < 1 || n_splits < 0 || (d != 64 && d != 128)) return 0;
  if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return 0;
  const long long n_kt = (N + 63) / 64;
  const long long wgs = (long long)B * H * ((N + 127) / 128);
  const long long round = d == 64 ? 768 : 512;
  const long long target = dtype == FA_F32 ? 256 : round;
  const long long min_run = dtype == FA_F32 ? 1 : 10;
  long long n = n_splits;
  if (n == 0) {
    n = 1;
    if (wgs < round) n = std::min((target + wgs - 1) / wgs, std::max(1LL, n_kt / min_run));
  }
  n = std::min(n, std::min(n_kt, (long long)kMaxForwardSplits));
  return (int)std::max(1LL, n);
}

size_t forward_split_part_bytes(int B, int H, int N, int d, int n) {
  return pad256((size_t)B * H * n * N * d * sizeof(float));
}

// Both partial-result regions of a split forward with n runs (0 for one run).
size_t forward_split_parts_bytes(int B, int H, int N, int d, int n) {
  if (n <= 1) return 0;
  return forward_split_part_bytes(B, H, N, d, n) + pad256((size_t)B * H * n * N * sizeof(float));
}

}  // namespace

extern "C" {

int fa_forward_splits(int B, int H, int N, int d, int n_splits, int dtype) {
  return forward_split_count(B, H, N, d, n_splits, dtype);
}

size_t fa_forward_split_workspace_size(int B, int H, int N, int d, int n_splits, int dtype) {
  const int n = forward_split_count(B, H, N, d, n_splits, dtype);
  if (n < 1) return 0;
  return forward_split_parts_bytes(B, H, N, d, n) + order_bytes(N);
}

int fa_forward_split(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int H, int N, int d, float scale, int causal,
                     const uint8_t* block_mask, int dtype, int n_splits, void* workspace,
                     size_t workspace_bytes, void* stream) {
  if (n_splits < 0) return FA_ERR_INVALID_ARG;
  const int rc = check_common(B, H, N, d, scale, dtype);
  if (rc != FA_OK) return rc;
  const int n = forward_split_count(B, H, N, d, n_splits, dtype);
  if (n <= 1) {
    // One run: the workspace is optional (only the work order uses it).
    const bool ws_ok = workspace != nullptr && aligned(workspace, 256) &&
                       workspace_bytes >= order_bytes(N);
    return forward_impl(q, k, v, o, lse, B, H, N, d, scale, causal, block_mask, dtype, false, 0.f,
                        0, 0, nullptr, ws_ok ? (int*)workspace : nullptr, stream);
  }
  if (!tensor_ptr_ok(q) || !tensor_ptr_ok(k) || !tensor_ptr_ok(v) || !tensor_ptr_ok(o))
    return FA_ERR_INVALID_ARG;
  if (lse == nullptr || !aligned(lse, 4)) return FA_ERR_INVALID_ARG;
  if (block_mask != nullptr && (N + fa::MASK_TILE - 1) / fa::MASK_TILE > fa::FWD_MAX_MASK_TILES)
    return FA_ERR_UNSUPPORTED;
  // Partial rows and the split grid are indexed with int in the kernels.
  const long long rows = (long long)B * H * n * N;
  if (rows > (1LL << 31) - 1 || (long long)B * H * n * ((N + 127) / 128) > (1LL << 31) - 1)
    return FA_ERR_UNSUPPORTED;
  const size_t need = fa_forward_split_workspace_size(B, H, N, d, n_splits, dtype);
  if (workspace == nullptr || !aligned(workspace, 256) || workspace_bytes < need)
    return FA_ERR_WORKSPACE;
  fa::FwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.mask = block_mask;
  p.BH = B * H;
  p.N = N;
  p.mask_tiles = (N + fa::MASK_TILE - 1) / fa::MASK_TILE;
  p.scale = scale;
  p.scale_log2e = scale * kLog2e;
  p.rescale_thr = 8.0f / p.scale_log2e;
  p.n_splits = n;
  p.o_part = (float*)workspace;
  p.lse_part = (float*)((char*)workspace + forward_split_part_bytes(B, H, N, d, n));
  hipError_t e = sparse_forward_order(
      p, causal, dtype, (int*)((char*)workspace + forward_split_parts_bytes(B, H, N, d, n)),
      (hipStream_t)stream);
  if (e != hipSuccess) return FA_ERR_HIP;
  e = fa::launch_forward(p, dtype, d, causal != 0, (hipStream_t)stream);
  if (e != hipSuccess) return FA_ERR_HIP;
  fa::DecParams m{};
  m.o = o;
  m.lse = lse;
  m.o_part = p.o_part;
  m.lse_part = p.lse_part;
  m.BH = B * H;
  m.Nq = N;
  m.n_splits = n;
  e = fa::launch_split_merge(m, dtype, d, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_backward_workspace_size(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1 || d < 1) return 0;
  // -D and the log2-domain lse, one fp32 each per row; then the block-sparse
  // work order, two int32 per 128-row tile.
  return 2 * delta_bytes(B, H, N) + order_bytes(N);
}

int fa_backward(const void* q, const void* k, const void* v, const void* o,
                const void* dO, const float* lse,
                float* dq, float* dk, float* dv,
                int B, int H, int N, int d, float scale, int causal,
                const uint8_t* block_mask, int dtype,
                void* workspace, size_t workspace_bytes, void* stream) {
  return backward_impl(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, scale, causal, block_mask,
                       dtype, false, 0.f, 0, 0, nullptr, workspace, workspace_bytes, stream);
}

int fa_backward_dropout(const void* q, const void* k, const void* v, const float* o_acc,
                        const void* dO, const float* lse, float* dq, float* dk, float* dv,
                        int B, int H, int N, int d, float scale, int causal,
                        const uint8_t* block_mask, int dtype, float dropout_p, uint64_t seed,
                        uint32_t offset, void* workspace, size_t workspace_bytes, void* stream) {
  return backward_impl(q, k, v, o_acc, dO, lse, dq, dk, dv, B, H, N, d, scale, causal,
                       block_mask, dtype, true, dropout_p, seed, offset, o_acc, workspace,
                       workspace_bytes, stream);
}

int fa_dropout_mask(int B, int H, int N, float dropout_p, uint64_t seed, uint32_t offset,
                    uint8_t* keep, void* stream) {
  if (keep == nullptr || B < 1 || H < 1 || N < 1) return FA_ERR_INVALID_ARG;
  if ((long long)B * H > (1LL << 24) || N > 65536) return FA_ERR_UNSUPPORTED;
  const long long nq = (N + 3) / 4;
  if ((long long)B * H * nq * nq > (1LL << 31) * 255LL) return FA_ERR_UNSUPPORTED;  // grid size
  fa::DropMaskParams p{};
  float sc;
  if (!dropout_args(dropout_p, seed, offset, p.k0, p.k1, p.off, p.t8, sc)) return FA_ERR_INVALID_ARG;
  p.keep = keep;
  p.BH = B * H;
  p.N = N;
  const hipError_t e = fa::launch_dropout_mask(p, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // extern "C"

namespace {

int backward_impl(const void* q, const void* k, const void* v, const void* o, const void* dO,
                  const float* lse, float* dq, float* dk, float* dv, int B, int H, int N, int d,
                  float scale, int causal, const uint8_t* block_mask, int dtype, bool drop,
                  float dropout_p, uint64_t seed, uint32_t offset, const float* o_acc,
                  void* workspace, size_t workspace_bytes, void* stream) {
  if (!tensor_ptr_ok(q) || !tensor_ptr_ok(k) || !tensor_ptr_ok(v) || !tensor_ptr_ok(o) ||
      !tensor_ptr_ok(dO) || !tensor_ptr_ok(dq) || !tensor_ptr_ok(dk) || !tensor_ptr_ok(dv))
    return FA_ERR_INVALID_ARG;
  if (lse == nullptr || !aligned(lse, 4)) return FA_ERR_INVALID_ARG;
  const int rc = check_common(B, H, N, d, scale, dtype);
  if (rc != FA_OK) return rc;
  if (dtype == FA_F32) return FA_ERR_UNSUPPORTED;
  if (block_mask != nullptr && (N + fa::MASK_TILE - 1) / fa::MASK_TILE > fa::FWD_MAX_MASK_TILES)
    return FA_ERR_UNSUPPORTED;
  if (workspace == nullptr || !aligned(workspace, 16) ||
      workspace_bytes < fa_backward_workspace_size(B, H, N, d))
    return FA_ERR_WORKSPACE;
  fa::BwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.dO = dO;
  p.lse = lse;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.neg_delta = (float*)workspace;
  p.lse2 = (float*)((char*)workspace + delta_bytes(B, H, N));
  p.qt_order = (int*)((char*)workspace + 2 * delta_bytes(B, H, N));
  p.kt_order = p.qt_order + (N + 127) / 128;
  p.mask = block_mask;
  p.BH = B * H;
  p.N = N;
  p.mask_tiles = (N + fa::MASK_TILE - 1) / fa::MASK_TILE;
  p.scale = scale;
  p.scale_log2e = scale * kLog2e;
  if (!dropout_args(dropout_p, seed, offset, p.drop_k0, p.drop_k1, p.drop_off, p.drop_t8,
                    p.drop_scale))
    return FA_ERR_INVALID_ARG;
  p.drop = drop;
  p.o_acc = o_acc;
  const hipError_t e = fa::launch_backward(p, dtype, d, causal != 0, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

extern "C" {

size_t fa_forward_fp8_workspace_size(int B, int H, int N, int d) {
  if (B < 1 || H < 1 || N < 1 || d < 1) return 0;
  return fp8_layout(B, H, N, d).total;
}

int fa_fp8_prepare(const void* q, const void* k, const void* v, int B, int H, int N, int d,
                   float scale, int dtype, const int8_t* signs, void* workspace,
                   size_t workspace_bytes, void* stream) {
  fa::Fp8Params p{};
  const int rc = fp8_setup(p, q, k, v, B, H, N, d, scale, dtype, signs, workspace, workspace_bytes);
  if (rc != FA_OK) return rc;
  const hipError_t e = fa::launch_fp8(p, dtype, d, false, true, false, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_forward_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int N, int d, float scale, int causal,
                   const uint8_t* block_mask, int dtype, const int8_t* signs,
                   void* workspace, size_t workspace_bytes, void* stream) {
  if (!tensor_ptr_ok(o) || lse == nullptr || !aligned(lse, 4)) return FA_ERR_INVALID_ARG;
  fa::Fp8Params p{};
  const int rc = fp8_setup(p, q, k, v, B, H, N, d, scale, dtype, signs, workspace, workspace_bytes);
  if (rc != FA_OK) return rc;
  if (block_mask != nullptr && p.mask_tiles > fa::FWD_MAX_MASK_TILES) return FA_ERR_UNSUPPORTED;
  p.o = o;
  p.lse = lse;
  p.mask = block_mask;
  p.prep_z0 = 1;   // K and V; each query tile's Q is prepared by the attention kernel
  if (block_mask != nullptr && causal == 0) {
    // The block-sparse work order, as in the 16-bit forward.
    int* order = (int*)((char*)workspace + fp8_layout(B, H, N, d).order);
    const hipError_t e = fa::launch_sparse_order(block_mask, p.mask_tiles, false, order,
                                                 order + p.mask_tiles, (hipStream_t)stream);
    if (e != hipSuccess) return FA_ERR_HIP;
    p.qt_order = order;
  }
  const hipError_t e = fa::launch_fp8(p, dtype, d, causal != 0, true, true, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_decode_splits(int B, int H, int Nq, int Nk, int d, int n_splits) {
  if (B < 1 || H < 1 || Nq < 1 || Nk < Nq || n_splits < 0 || (d != 64 && d != 128)) return 0;
  return dec_split(B, H, Nk, n_splits).n;
}

size_t fa_decode_workspace_size(int B, int H, int Nq, int Nk, int d, int n_splits) {
  const int n = fa_decode_splits(B, H, Nq, Nk, d, n_splits);
  if (n <= 1) return 0;
  const size_t rows = (size_t)B * H * n * Nq;
  return pad256(rows * d * sizeof(float)) + pad256(rows * sizeof(float));
}

int fa_decode(const void* q, const void* k, const void* v, void* o, float* lse,
              int B, int H, int Nq, int Nk, int d, float scale, int causal,
              int n_splits, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (!tensor_ptr_ok(q) || !tensor_ptr_ok(k) || !tensor_ptr_ok(v) || !tensor_ptr_ok(o))
    return FA_ERR_INVALID_ARG;
  if (lse == nullptr || !aligned(lse, 4)) return FA_ERR_INVALID_ARG;
  const int rc = check_decode(B, H, Nq, Nk, d, scale, dtype, n_splits);
  if (rc != FA_OK) return rc;
  const DecSplit sp = dec_split(B, H, Nk, n_splits);
  const size_t need = fa_decode_workspace_size(B, H, Nq, Nk, d, n_splits);
  if (need > 0 && (workspace == nullptr || !aligned(workspace, 16) || workspace_bytes < need))
    return FA_ERR_WORKSPACE;
  fa::DecParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  if (need > 0) {
    const size_t rows = (size_t)B * H * sp.n * Nq;
    p.o_part = (float*)workspace;
    p.lse_part = (float*)((char*)workspace + pad256(rows * d * sizeof(float)));
  }
  p.BH = B * H;
  p.Nq = Nq;
  p.Nk = Nk;
  p.n_splits = sp.n;
  p.split_len = sp.len;
  p.scale_log2e = scale * kLog2e;
  const hipError_t e = fa::launch_decode(p, dtype, d, causal != 0, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // extern "C"
