/*
 * fa.h -- C ABI of libfa.so: exact attention softmax(scale * Q K^T) V on one
 * AMD Instinct MI355X (gfx950), forward and backward, with causal and
 * block-sparse masking.
 *
 * The operation is the one the FlashAttention pages define:
 *   - "FlashAttention: Fast and Memory-Efficient Exact Attention with
 *     IO-Awareness" reading guide (xyznot.com), section "Método": Q, K, V are
 *     N x d per head; the forward pass keeps a running row max m and row sum l
 *     per query (incremental softmax equations), writes O and the softmax
 *     statistics only; section "Ideias centrais", "Recomputação no Backward
 *     Pass": the backward pass recomputes S and P from Q, K and the saved
 *     statistics; section "Extensão: Block-Sparse FlashAttention": a {0,1}
 *     mask over (query tile, key tile) pairs selects the tiles evaluated.
 *   - "Attention flash et question de longueur de séquence" (marketmaker.cc),
 *     section "L'intégration est de huit lignes": tensors are laid out
 *     (batch, heads, seq, head_dim); section "Le masquage causal": the causal
 *     mask is built by the kernel, key j is visible to query i iff j <= i.
 *
 * Conventions shared by every call
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *     allocates nothing and keeps no mutable global state, so calls on
 *     different streams may run concurrently.
 *   - Tensors are contiguous, row-major (B, H, N, d) with d fastest; lse and
 *     the backward workspace's per-row terms are (B, H, N).  Pointers must be
 *     16-byte aligned.
 *   - `dtype` (fa_dtype) is the element type of q, k, v, o and dO.  lse, dq,
 *     dk, dv are always float32.  Arithmetic: products accumulate in fp32 on
 *     the matrix cores (fp32 inputs use fp32 MFMA; fp16/bf16 inputs use
 *     fp16/bf16 MFMA with fp32 accumulation); softmax statistics are fp32.
 *   - `scale` (finite, > 0) multiplies the scores (1/sqrt(d) is the usual
 *     value); gradients are with respect to the unscaled q, k, v.
 *   - `causal` != 0 excludes keys j > i.  `block_mask` (device pointer, may be
 *     NULL = dense) is uint8 [ceil(N/128)][ceil(N/128)], row-major, one entry
 *     per 128 x 128 (query tile, key tile) pair, shared by every (b, h); a zero
 *     entry excludes the whole tile.  causal and block_mask combine with AND.
 *   - A query row with no visible key gets o = 0, lse = -inf and contributes
 *     nothing to any gradient.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *     enqueue work and return without synchronising.
 *   - Arguments are validated before anything is launched; on any error
 *     nothing is enqueued and the output buffers are untouched.  There is no
 *     fallback path: an unsupported shape or dtype is an error.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FA_F32 = 0, FA_F16 = 1, FA_BF16 = 2 } fa_dtype;

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = -1, /* null/misaligned pointer, B/H/N < 1, bad dtype, scale not finite > 0 */
  FA_ERR_UNSUPPORTED = -2, /* valid request the library does not implement (e.g. d not 64/128) */
  FA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than its *_workspace_size() */
  FA_ERR_HIP = -4          /* the HIP runtime reported an error at launch */
} fa_status;

#define FA_MASK_BLOCK 128

/*
 * Forward pass.  Writes o (B,H,N,d; dtype) and lse (B,H,N; fp32), where
 *   lse_i = m_i + ln(l_i),  m_i = max_j s_ij,  l_i = sum_j exp(s_ij - m_i),
 * over the visible keys j of query i, s_ij = scale * <q_i, k_j> (natural log).
 * Supported: d in {64, 128}; dtype FA_F32, FA_F16, FA_BF16; with a block_mask,
 * N <= 262144 (2048 mask tiles).
 */
int fa_forward(const void* q, const void* k, const void* v, void* o, float* lse,
               int B, int H, int N, int d, float scale, int causal,
               const uint8_t* block_mask, int dtype, void* stream);

/*
 * Forward pass with split key ranges, for grids too small to fill the GPU
 * (few heads, few query tiles): the same o and lse as fa_forward.
 *
 * Every query tile's visible key tiles (64 keys each) are cut into n runs of
 * equal tile count, each computed by its own workgroup with the
 * online-softmax recurrence into a normalised partial output o_s and its
 * logsumexp lse_s; a second kernel merges them with the incremental-softmax
 * merge ("Rastreamento Incremental do Softmax", xyznot.com reading guide):
 * lse = ln sum_s exp(lse_s), o = sum_s exp(lse_s - lse) o_s.  A run with no
 * visible key has lse_s = -inf and weight 0.
 *
 * n_splits = 0 lets the library choose (fa_forward_splits()): one run unless
 * the plain grid (B*H*ceil(N/128) workgroups) is smaller than one round of
 * the GPU (768 workgroups at d = 64, 512 at d = 128), then enough runs for
 * one round, with at least ten 64-key tiles per run (for FA_F32 inputs, whose
 * tiles take the matrix cores far longer: enough runs for one workgroup per
 * CU, at least one tile each).  An explicit n_splits is
 * capped at ceil(N / 64) and at 64.  With one run this is fa_forward.
 * `workspace` (at least fa_forward_split_workspace_size() bytes, 256-byte
 * aligned, caller-owned, contents ignored on entry) holds, in this order,
 * each region padded to 256 bytes: o_part (B*H, n, N, d) fp32 and lse_part
 * (B*H, n, N) fp32 (both only when n > 1), then the block-sparse work order,
 * two int32 per 128-row tile.  With a block_mask, no causal flag and 16-bit
 * inputs, the forward takes each head's query tiles in the backward's work
 * order (most visible key tiles first, ties by index): workgroups that run at once then hold rows of similar
 * length, walk the head's K/V tiles in step and find them in L2; every
 * tile's arithmetic is unchanged, so o and lse are bit-identical to
 * fa_forward's.  With one run the workspace is optional: when it is null,
 * misaligned or smaller than the order, the tiles run in index order.
 * Supported: every dtype and head dimension fa_forward supports;
 * B*H*n*N < 2^31, else FA_ERR_UNSUPPORTED; n_splits < 0 -> FA_ERR_INVALID_ARG.
 */
int fa_forward_split(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int H, int N, int d, float scale, int causal,
                     const uint8_t* block_mask, int dtype, int n_splits, void* workspace,
                     size_t workspace_bytes, void* stream);

/* Number of key runs fa_forward_split uses for this shape and input dtype
 * (0 on bad input). */
int fa_forward_splits(int B, int H, int N, int d, int n_splits, int dtype);

/* Bytes of workspace fa_forward_split needs: the partial results when it uses
 * more than one run, plus the work order (0 on bad input). */
size_t fa_forward_split_workspace_size(int B, int H, int N, int d, int n_splits, int dtype);

/* Bytes of device workspace fa_backward needs for this shape (0 on bad input):
 * two fp32 values per (b, h, row), each array padded to 256 bytes, then two
 * int32 per 128-row tile (the block-sparse work order), padded to 256 bytes. */
size_t fa_backward_workspace_size(int B, int H, int N, int d);

/*
 * Backward pass of L with upstream gradient dO = dL/dO.  Inputs: q, k, v, the
 * forward's o and lse, dO (dtype).  Outputs (fp32, B,H,N,d, fully overwritten):
 *   dv = P^T dO,  dq = scale * dS K,  dk = scale * dS^T Q,
 *   P_ij = exp(s_ij - lse_i) on visible keys (else 0),
 *   dS = P o (dP - D),  dP = dO V^T,  D_i = sum_c dO_ic * o_ic.
 * `workspace` is a device buffer of at least fa_backward_workspace_size() bytes,
 * owned by the caller, scratch for the duration of the call.
 * Supported: d in {64, 128}; dtype FA_F16, FA_BF16 (FA_F32 -> FA_ERR_UNSUPPORTED);
 * with a block_mask, N <= 262144 (2048 mask tiles), else FA_ERR_UNSUPPORTED.
 */
int fa_backward(const void* q, const void* k, const void* v, const void* o,
                const void* dO, const float* lse,
                float* dq, float* dk, float* dv,
                int B, int H, int N, int d, float scale, int causal,
                const uint8_t* block_mask, int dtype,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * Dropout on the probabilities, fused into the same kernels.
 *
 * Dropout is one of the operations FlashAttention fuses into its kernel so
 * that nothing N x N reaches HBM ("FlashAttention ... IO-Awareness" reading
 * guide, xyznot.com, "Ideias centrais", "Fusão de Kernels"); the
 * marketmaker.cc page passes `dropout_p` to the fused attention call
 * ("L'intégration est de huit lignes").  With keep mask Z:
 *   O = (P o Z) V / (1 - p),  lse as without dropout (statistic of P);
 *   backward with the same Z: dV = (P o Z)^T dO / (1 - p),
 *   dS = P o (Z o dP / (1 - p) - D),  D_i = sum_c dO_ic O_ic (O with dropout).
 * Z is never stored: element (query i, key j) of head bh = b * H + h is kept
 * iff byte (j mod 4) of word (i mod 4) of Philox-4x32-10 (Salmon, Moraes,
 * Dror, Shaw, SC 2011) at counter (j div 4, i div 4, bh, offset) and key
 * (seed mod 2^32, seed div 2^32) is >= t, t = min(255, floor(256 p + 1/2));
 * kept values are scaled by 1 / (1 - t / 256).  Every kernel recomputes the
 * bytes it needs, so forward and backward apply the same mask when called
 * with the same (dropout_p, seed, offset).
 *
 * Arguments as fa_forward / fa_backward plus dropout_p (finite, 0 <= p < 1,
 * else FA_ERR_INVALID_ARG), seed and offset, and the output O in fp32:
 *   - fa_forward_dropout writes it to `o_acc` ((B,H,N,d) fp32, device,
 *     caller-owned, 16-byte aligned) when o_acc is not NULL: O before its
 *     rounding to dtype.  NULL skips it (a caller that runs no backward).
 *   - fa_backward_dropout takes that fp32 O in place of the 16-bit o
 *     (required, non-NULL, 16-byte aligned) and computes D from it.  The
 *     reason: a causal row with one visible key has dS = P (dP/(1-p) - D) = 0
 *     exactly, but D from O rounded to 16 bits leaves that rounding, times
 *     the uncancelled 1/(1-p), in dQ (measured up to 1.9e-2 at d = 128,
 *     p = 0.2 against the exact gradient).
 * With p = 0 (t = 0) nothing is dropped and the result is the plain one.
 * FA_F32 -> FA_ERR_UNSUPPORTED (also at p = 0 with o_acc, or in the
 * backward).  With a block_mask, N <= 262144 as for fa_forward / fa_backward.
 */
int fa_forward_dropout(const void* q, const void* k, const void* v, void* o, float* lse,
                       int B, int H, int N, int d, float scale, int causal,
                       const uint8_t* block_mask, int dtype, float dropout_p, uint64_t seed,
                       uint32_t offset, float* o_acc, void* stream);

int fa_backward_dropout(const void* q, const void* k, const void* v, const float* o_acc,
                        const void* dO, const float* lse, float* dq, float* dk, float* dv,
                        int B, int H, int N, int d, float scale, int causal,
                        const uint8_t* block_mask, int dtype, float dropout_p, uint64_t seed,
                        uint32_t offset, void* workspace, size_t workspace_bytes, void* stream);

/* The keep mask the two calls above apply, written out: keep (device,
 * (B, H, N, N) uint8, caller-owned) gets 1 for kept and 0 for dropped
 * elements.  N <= 65536.  For inspection and tests; the attention calls never
 * need it. */
int fa_dropout_mask(int B, int H, int N, float dropout_p, uint64_t seed, uint32_t offset,
                    uint8_t* keep, void* stream);

/*
 * Decode: a few new queries against a long cached history.
 *
 * Decoding has one (or a few) new query rows and a long history of keys and
 * values, and kernels for it parallelise the scan over that history
 * ("Почему Flash Attention быстрее", sloger.press, section "Что это изменило
 * на практике").  q (B,H,Nq,d) holds the LAST Nq positions of a sequence
 * whose keys and values k, v (B,H,Nk,d) are all cached, 1 <= Nq <= Nk:
 *   o_i = sum_j P_ij v_j,  P_ij = exp(s_ij - lse_i),  s_ij = scale * <q_i, k_j>,
 *   lse_i = ln sum_j exp(s_ij), over the visible keys j of query i;
 * without `causal` every query sees every key; with it query i, at position
 * Nk - Nq + i, sees keys j <= Nk - Nq + i (the causal rule of "Le masquage
 * causal", marketmaker.cc page, aligned to the end of the sequence; for
 * Nq = Nk it is fa_forward's rule).  Writes o (B,H,Nq,d; dtype of q) and lse
 * (B,H,Nq; fp32, natural log).
 *
 * The key range [0, Nk) is cut into n ranges of equal length L (a multiple of
 * 128 keys; the last range is shorter), each scanned by its own workgroups
 * with the online-softmax recurrence; a second kernel merges the per-range
 * (o_s, lse_s) with the incremental-softmax merge ("Rastreamento Incremental
 * do Softmax", xyznot.com reading guide): lse = ln sum_s exp(lse_s),
 * o = sum_s exp(lse_s - lse) o_s.  `n_splits` asks for a number of ranges
 * (0 = let the library fill the GPU); fa_decode_splits() returns the number
 * actually used, which may be smaller (ranges are at least 128 keys).  With
 * one range nothing is merged and no workspace is needed.
 *
 * `workspace`: device buffer of at least fa_decode_workspace_size() bytes
 * (same B, H, Nq, Nk, d, n_splits), owned by the caller, scratch for the
 * duration of the call; may be NULL when that size is 0.
 * Supported: d in {64, 128}; dtype FA_F16, FA_BF16; Nq <= 16; Nk * d and
 * B * H * Nk below 2^31.  Nq > Nk, Nq < 1, n_splits < 0 -> FA_ERR_INVALID_ARG;
 * FA_F32 or Nq > 16 -> FA_ERR_UNSUPPORTED; short workspace -> FA_ERR_WORKSPACE.
 */
int fa_decode(const void* q, const void* k, const void* v, void* o, float* lse,
              int B, int H, int Nq, int Nk, int d, float scale, int causal,
              int n_splits, int dtype, void* workspace, size_t workspace_bytes, void* stream);

/* Number of key ranges fa_decode uses for these arguments (0 on bad input). */
int fa_decode_splits(int B, int H, int Nq, int Nk, int d, int n_splits);

/* Bytes of device workspace fa_decode needs (0 with one range or bad input):
 * per range and query one fp32 partial output row and one fp32 logsumexp,
 * each array padded to 256 bytes. */
size_t fa_decode_workspace_size(int B, int H, int Nq, int Nk, int d, int n_splits);

/*
 * fa_decode for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.
 *
 * Same arguments, results and errors as fa_decode, without the workspace:
 * the key-range partials go to a device array of FA_NOALLOC_SCRATCH_BYTES
 * (16 MiB) that the library holds on every GPU it runs on until the process
 * ends.  The call allocates nothing (no hipMalloc, no library allocation);
 * the first call on a device looks the array's address up once.  When the
 * partials would need more than the array (fa_decode_workspace_size() of the
 * same arguments > FA_NOALLOC_SCRATCH_BYTES; with the automatic range count
 * that takes B * H * ranges * Nq * (d + 1) * 4 bytes, about 1.6 MB at
 * B * H = 96, Nq = 16, d = 128) it returns FA_ERR_WORKSPACE and enqueues
 * nothing.  Every call on one GPU shares that GPU's array and leaves its
 * partials there: calls that overlap on one GPU (other streams, other host
 * threads) race and must be ordered by the caller.
 */
#define FA_NOALLOC_SCRATCH_BYTES (16u << 20)

int fa_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int H, int Nq, int Nk, int d, float scale, int causal,
                      int n_splits, int dtype, void* stream);

/*
 * FP8 forward with incoherent processing.
 *
 * FP8 attention is ruined by outliers unless the vectors are first rotated
 * randomly, spreading an outlier's magnitude over every coordinate, and then
 * quantised per block ("Attention flash et question de longueur de
 * séquence", marketmaker.cc, section "FA3 : Mécanique de la trémie", point
 * 3).  Here:
 *   rotation      R = diag(signs) H_d / sqrt(d), H_d the Sylvester-Hadamard
 *                 matrix; Q and K rows are multiplied by R (Q K^T is
 *                 unchanged), V is not; Q is also multiplied by
 *                 c = scale * log2(e), so Q K^T comes out in base-2 units;
 *   quantisation  every 64-row block of c Q R, of K R and of V: scale s, the
 *                 smallest power of two with 448 s >= amax (at least 2^-126;
 *                 1 for an all-zero block: an E8M0 block scale), codes
 *                 E4M3(x / s) (OCP E4M3, round to nearest even);
 *   attention     x = s_q s_k (Q8 K8^T) with fp32 accumulation on the FP8
 *                 matrix cores (the block scales applied exactly by the
 *                 instruction), fp32 online softmax in base 2 (running
 *                 reference m, sum l of 2^(x - m)), P = 2^(x - m) rounded to
 *                 E4M3, O = sum_j E4M3(P_ij) s_v[t(j)] V8_j / l_i,
 *                 lse = (m + log2 l) ln 2.
 * The result approximates exact attention to FP8 precision (a few percent
 * of |O| on N(0, 1) inputs); it is not exact.
 *
 * q, k, v: (B,H,N,d) FA_BF16 or FA_F16; o: same shape and dtype; lse: (B,H,N)
 * fp32.  `signs`: device pointer (16-byte aligned) to d int8 values
 * (negative = -1, otherwise +1), the random signs of the rotation, drawn by
 * the caller; NULL skips the rotation (block-quantised FP8 without incoherent
 * processing).  causal and
 * block_mask as for fa_forward.  `workspace` (at least
 * fa_forward_fp8_workspace_size() bytes, 256-byte aligned, caller-owned)
 * holds the prepared operands, in this order, each region padded to 256
 * bytes, with nt = ceil(N / 64) and Npad = 64 nt (fa_forward_fp8 writes the
 * K and V regions; each query tile's c Q R is rotated and quantised inside
 * the attention kernel, with the same arithmetic and so the same codes and
 * scales fa_fp8_prepare writes to the Q regions, which fa_forward_fp8
 * leaves untouched):
 *   Q8  (B*H, Npad, d) E4M3 codes, row-major (rows >= N are zero)
 *   K8  (B*H, Npad, d) E4M3 codes
 *   V8T (B*H, nt, d, 64) E4M3 codes of each 64-key block transposed, position
 *       32 g + e holding key 32 (e / 16) + 8 ((e % 16) / 4) + 4 g + e % 4 of
 *       the block (keys >= N are zero)
 *   s_q, s_k, s_v (B*H, nt) fp32 block scales
 *   the block-sparse work order, two int32 per 128-row tile (written and
 *   used by fa_forward_fp8 with a block_mask and no causal flag: each head's
 *   query tiles run in the order fa_forward_split gives them).
 * Supported: d in {64, 128}; FA_F32 -> FA_ERR_UNSUPPORTED.
 */
int fa_forward_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int N, int d, float scale, int causal,
                   const uint8_t* block_mask, int dtype, const int8_t* signs,
                   void* workspace, size_t workspace_bytes, void* stream);

/* The rotation and quantisation step of fa_forward_fp8 alone: fills the
 * workspace regions Q8, K8, V8T, s_q, s_k, s_v described above.  `scale` is
 * the softmax scale the codes are prepared for (Q's codes hold scale * log2(e)
 * times Q R); it must be finite and > 0. */
int fa_fp8_prepare(const void* q, const void* k, const void* v, int B, int H, int N, int d,
                   float scale, int dtype, const int8_t* signs, void* workspace,
                   size_t workspace_bytes, void* stream);

/* Bytes of workspace fa_forward_fp8 and fa_fp8_prepare need (0 on bad input). */
size_t fa_forward_fp8_workspace_size(int B, int H, int N, int d);

/* Static, human-readable text for a status code. */
const char* fa_status_string(int status);

/* Library ABI version (this header: 6; 2 added fa_forward_split*, 3 the fp32
 * output o_acc of the dropout calls, 4 power-of-two FP8 block scales, the
 * scale argument of fa_fp8_prepare and the dtype argument of
 * fa_forward_splits and fa_forward_split_workspace_size, 5 fa_forward_fp8
 * no longer writing the Q regions of its workspace, and `signs` 16-byte
 * aligned, 6 the work order at the end of the fa_forward_split workspace,
 * also for one run, and of the fa_forward_fp8 workspace). */
int fa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
