/*
 * fa.h -- C ABI of the exact, IO-aware attention library (libfa.so), gfx950.
 *
 * What the library computes.  For every batch entry b and head h independently
 * (FlashAttention first principles, section 2: heads run in parallel):
 *
 *     S   = scale * Q K^T                          (N x N, never stored)
 *     S_ij = -inf where key j is masked for query i
 *     P   = softmax(S) along each row               (first principles, section 4.2)
 *     P~  = P * Z, Z = dropout keep mask / (1 - p)  (first principles, section 2
 *                                                    and section 3.2: dropout after softmax)
 *     O   = P~ V
 *     LSE_i = m_i + ln(sum_j exp(S_ij - m_i)),  m_i = max_j S_ij
 *
 * The forward streams K/V tiles through on-chip memory with a running row max
 * and row sum, rescaling the partial output for every new tile, so the N x N
 * matrix never reaches device memory (ML Canon 48 FlashAttention, "tiling and
 * online softmax").  The backward recomputes score tiles from Q, K and the saved
 * per-row normaliser instead of storing P (ML Canon 48 FlashAttention, "backward
 * without N x N"; Flash Attention hardware-aware optimisation, section 2.2).
 *
 * Masking (element-wise, first principles section 4.1): key j is allowed for query i
 * iff (causal == 0 || j <= i) && j < L_b, where L_b = key_lens[b] (clamped to
 * [0, N]) or N when key_lens is NULL.  A query row with no allowed key gets
 * O = 0, LSE = -inf and zero gradient contributions.
 *
 * Dropout (p > 0): element (b, h, i, j) is kept iff word (j & 3) of
 * Philox4x32-10(counter = (j >> 2, i, h, b), key = (seed & 0xffffffff,
 * seed >> 32)) is >= floor(p * 2^32) (p as passed, widened to double); kept
 * values are scaled by (float)(1 / (1 - p)) computed in double.  LSE is the
 * normaliser before dropout.  The backward must receive the forward's seed and p.
 *
 * Layouts.  Q, K, V, O, dO, dQ, dK, dV: [B, H, N, d] with d innermost and
 * contiguous, element type `dtype`; contiguous ([B, H, N, d] row-major) for
 * every entry point except fa_fwd_strided and fa_bwd_strided, which take
 * each tensor's batch, head and row strides (fa_strides), so that, e.g.,
 * [B, N, H, d] memory or a fused QKV projection is read in place, and the
 * packed-sequence entry points (fa_fwd_varlen, fa_bwd_varlen).  LSE:
 * contiguous fp32 [B, H, N].  key_lens: device int32 [B] or NULL.  All
 * pointers are device pointers, 16-byte aligned (LSE: 4-byte aligned).
 *
 * Ownership.  The caller allocates and owns every buffer, including the
 * backward workspace.  The library never allocates or frees device memory,
 * never synchronises, and keeps no state between calls; calls on different
 * streams may run concurrently provided their buffers do not overlap.  Outputs
 * are overwritten, never accumulated into.  Inputs and outputs must not alias.
 *
 * Streams.  Every kernel is enqueued on `stream` (NULL = the default stream)
 * and the call returns immediately; results are valid once the stream has
 * reached that point.  Inputs must stay unchanged until then.
 *
 * Errors.  Arguments are checked on the host before any HIP call; on failure
 * nothing is launched and the code says why:
 *   FA_ERR_INVALID_ARG  NULL or misaligned pointer, B/H/N <= 0, a size whose
 *                       element count overflows int64, non-finite or
 *                       non-positive scale, p outside [0, 1), workspace NULL
 *                       or smaller than fa_bwd_workspace_size(), an unknown
 *                       dtype, strides that fa_strides rules out.
 *   FA_ERR_UNSUPPORTED  d not in {32, 64, 96, 128, 256}; fp32 with dropout;
 *                       the split forward outside 16-bit d in {64, 128};
 *                       one (b, h) slice whose N + 256 rows span 2^32 bytes
 *                       or more (N >= 2^24 - 256 at d = 128, 2^25 - 256 at
 *                       d = 64, for contiguous 16-bit rows): the kernels
 *                       address a slice, including tiles fetched ahead past
 *                       its end, with 32-bit byte offsets.
 *   FA_ERR_HIP          a launch failed (hipGetLastError after launching).
 * key_lens lives in device memory and cannot be range-checked on the host; the
 * kernels clamp each L_b into [0, N].
 */
#ifndef IO_AWARE_EXACT_FA_H
#define IO_AWARE_EXACT_FA_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = 1,
  FA_ERR_UNSUPPORTED = 2,
  FA_ERR_HIP = 3,
  FA_ERR_TOO_LARGE = 4  /* fa_bwd_noalloc: sizes beyond its fixed scratch */
} fa_status;

typedef enum {
  FA_F32 = 0,   /* IEEE binary32 */
  FA_BF16 = 1,  /* bfloat16, round-to-nearest-even on output */
  FA_F16 = 2    /* IEEE binary16, round-to-nearest-even on output */
} fa_dtype;

/*
 * Element strides of one [B, H, N, d] tensor whose d elements per row are
 * contiguous: element (b, h, n, e) is at base[b * batch + h * head + n * row
 * + e] (in elements of the tensor's dtype, not bytes).  Contiguous
 * [B, H, N, d] is {H * N * d, N * d, d}; [B, N, H, d] memory viewed as
 * [B, H, N, d] is {N * H * d, d, H * d}.  Rules, checked on the host:
 *   - row >= d, batch >= 0, head >= 0 (else FA_ERR_INVALID_ARG);
 *   - batch, head and row are multiples of 16 bytes' worth of elements (8
 *     for 16-bit types, 4 for fp32), so every row starts 16-byte aligned
 *     (else FA_ERR_INVALID_ARG);
 *   - outputs (O, dQ, dK, dV) give every (b, h, n) its own row: sorted by
 *     stride, each dimension's stride is at least the span of the ones
 *     inside it (else FA_ERR_INVALID_ARG);
 *   - (N + 256) * row elements span fewer than 2^32 bytes (else
 *     FA_ERR_UNSUPPORTED).
 * Different tensors must not overlap (not checked).
 */
typedef struct {
  int64_t batch, head, row;
} fa_strides;

/*
 * Forward pass: O and LSE.
 *
 *   q, k, v   [B, H, N, d] of dtype, read only.
 *   o         [B, H, N, d] of dtype, written.
 *   lse       [B, H, N] fp32, written (natural log, scaled-score units).
 *   scale     multiplier of Q K^T (1/sqrt(d) for standard attention,
 *             ML Canon 48 FlashAttention, the PyTorch SDPA box).
 *   causal    non-zero: key j is masked for query i when j > i (top-left).
 *   key_lens  device int32 [B] or NULL (all keys valid).
 *   dropout_p probability of dropping an element, 0 <= p < 1.
 *   seed      Philox key, used only when dropout_p > 0.
 *
 * Head sizes and kernels:
 *   FA_BF16, FA_F16 at d in {64, 128}: the MFMA kernels, every mask and
 *     dropout combination.
 *   FA_BF16, FA_F16 at d in {32, 96}: the same MFMA kernels of width 64 and
 *     128, the head dimension zero-padded on chip (columns past d are read
 *     as zeros and never written), when every tensor's (b, h) slice, N + 256
 *     rows of its row stride, spans fewer than 2^31 bytes; else as below.
 *   FA_BF16, FA_F16 at d = 256, and FA_F32 at every d in
 *     {32, 64, 96, 128, 256}: generic kernels (fp32 arithmetic on the vector
 *     ALUs, 32-row tiles in LDS, eight threads per row).  FA_F32 takes no
 *     dropout (FA_ERR_UNSUPPORTED).
 */
fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int H, int N, int d, fa_dtype dtype, float scale, int causal,
                 const int32_t* key_lens, float dropout_p, uint64_t seed,
                 hipStream_t stream);

/*
 * fa_fwd on tensors laid out by strides: strides[0..3] are those of q, k, v
 * and o (see fa_strides); NULL means all four contiguous.  LSE stays
 * contiguous [B, H, N].  Same checks, kernels and results (bit for bit) as
 * fa_fwd on the same values.
 */
fa_status fa_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse,
                         const fa_strides* strides, int B, int H, int N, int d, fa_dtype dtype,
                         float scale, int causal, const int32_t* key_lens, float dropout_p,
                         uint64_t seed, hipStream_t stream);

/*
 * Split-KV forward: fa_fwd's result for small B*H, where one workgroup per
 * query block would leave most of the GPU idle.  Each query block's key tiles
 * are split num_splits ways (FlashAttention-2's better work partitioning,
 * Flash Attention hardware-aware optimisation, section 4); every split runs
 * the online softmax over its share and writes its fp32 O and LSE to the
 * workspace, then a combine pass weights the splits by exp(LSE_s - LSE).
 * Same arguments, checks and mask/dropout semantics as fa_fwd (bf16 and fp16
 * at d in {64, 128} only, else FA_ERR_UNSUPPORTED), plus
 *   num_splits       1 .. FA_MAX_SPLITS (else FA_ERR_INVALID_ARG); splits
 *                    that get no key tile are allowed and contribute nothing;
 *   workspace        device buffer of at least
 *                    fa_fwd_split_workspace_size() bytes, 16-byte aligned,
 *                    contents irrelevant on entry, garbage on exit.
 * The result equals fa_fwd's up to rounding (the softmax sums are taken in
 * another order), not bitwise.
 */
#define FA_MAX_SPLITS 64
size_t fa_fwd_split_workspace_size(int B, int H, int N, int d, fa_dtype dtype, int num_splits);
fa_status fa_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse,
                       int B, int H, int N, int d, fa_dtype dtype, float scale, int causal,
                       const int32_t* key_lens, float dropout_p, uint64_t seed, int num_splits,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Packed batches of sequences of different lengths, without padding.
 * Sequence b (0 <= b < num_seqs) is the token rows [cu_seqlens[b],
 * cu_seqlens[b + 1]) of every tensor; the tensors are [T, H, d] with
 * T = cu_seqlens[num_seqs] tokens, rows of d contiguous elements.
 *   strides     strides[t].row and strides[t].head are tensor t's token and
 *               head strides in elements (q, k, v, o here; q, k, v, o, dout,
 *               dq, dk, dv in fa_bwd_varlen); `batch` is ignored.  NULL:
 *               every tensor contiguous [T, H, d] (row = H * d, head = d).
 *               The fa_strides rules apply with B = 1 and N = T (outputs
 *               one-to-one over all tokens) and with N = the longest
 *               sequence (the 32-bit span).
 *   cu_seqlens  HOST int32 array of num_seqs + 1 offsets, cu_seqlens[0] = 0,
 *               non-decreasing (empty sequences allowed); read during the
 *               call only.
 *   lse         fp32; sequence b's LSE is the contiguous [H, len_b] block at
 *               lse + H * cu_seqlens[b].
 * Each sequence attends to its own tokens only (causal: key j <= query i,
 * positions inside the sequence); the dropout counter of fa.h uses b as the
 * batch index and positions inside the sequence as i and j.  Everything else
 * (dtype, d, scale, dropout, checks, kernels) is fa_fwd's / fa_bwd's; the
 * kernels run once per non-empty sequence, in order, on `stream`.
 * fa_bwd_varlen's workspace: fa_bwd_varlen_workspace_size() bytes (the
 * per-row terms of the longest sequence; the sequences reuse it in stream
 * order).
 */
fa_status fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                        const fa_strides* strides, const int32_t* cu_seqlens, int num_seqs,
                        int H, int d, fa_dtype dtype, float scale, int causal, float dropout_p,
                        uint64_t seed, hipStream_t stream);
size_t fa_bwd_varlen_workspace_size(const int32_t* cu_seqlens, int num_seqs, int H, int d,
                                    fa_dtype dtype);
fa_status fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv,
                        const fa_strides* strides, const int32_t* cu_seqlens, int num_seqs,
                        int H, int d, fa_dtype dtype, float scale, int causal, float dropout_p,
                        uint64_t seed, void* workspace, size_t workspace_bytes,
                        hipStream_t stream);

/*
 * Packed batches in one launch per pass: the varlen entry points above with
 * the offsets in DEVICE memory, as a training loop holds them.
 *   cu_seqlens    device int32 array of num_seqs + 1 offsets (cu_seqlens[0]
 *                 = 0, non-decreasing); read by the kernels, not checked.
 *   max_len       the longest sequence, >= every cu_seqlens[b+1] -
 *                 cu_seqlens[b] (rows past max_len of a longer sequence are
 *                 neither read nor written).
 *   total_tokens  cu_seqlens[num_seqs] (the rows the strides must cover).
 * One launch covers every sequence: workgroup (b, h, query block) reads its
 * sequence's first row and length from cu_seqlens, and blocks past the
 * length exit at once.  The MFMA kernels only: FA_BF16 / FA_F16 at d in
 * {32, 64, 96, 128} (else FA_ERR_UNSUPPORTED; the host-offset entry points
 * take every type and head size).  Everything else (strides, LSE layout,
 * masks, the dropout counter with b as the batch index) as fa_fwd_varlen /
 * fa_bwd_varlen, and the same results bit for bit.  The backward's workspace:
 * fa_bwd_varlen_device_workspace_size() bytes (the per-row terms of every
 * token and head).
 */
fa_status fa_fwd_varlen_device(const void* q, const void* k, const void* v, void* o, float* lse,
                               const fa_strides* strides, const int32_t* cu_seqlens, int num_seqs,
                               int max_len, int total_tokens, int H, int d, fa_dtype dtype,
                               float scale, int causal, float dropout_p, uint64_t seed,
                               hipStream_t stream);
size_t fa_bwd_varlen_device_workspace_size(int total_tokens, int H, int d, fa_dtype dtype);
fa_status fa_bwd_varlen_device(const void* q, const void* k, const void* v, const void* o,
                               const void* dout, const float* lse, void* dq, void* dk, void* dv,
                               const fa_strides* strides, const int32_t* cu_seqlens, int num_seqs,
                               int max_len, int total_tokens, int H, int d, fa_dtype dtype,
                               float scale, int causal, float dropout_p, uint64_t seed,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Bytes of device workspace fa_bwd needs for these sizes: two fp32 [B, H, N]
 * row arrays, D_i = sum_k dO_ik O_ik and LSE_i * log2(e), each padded to a
 * multiple of 256 bytes.
 * Returns 0 for arguments fa_bwd would reject.
 */
size_t fa_bwd_workspace_size(int B, int H, int N, int d, fa_dtype dtype);

/*
 * Backward pass: dQ, dK, dV for upstream gradient dout, recomputing the score
 * tiles from q, k and the forward's lse.
 *
 *   q, k, v, o, dout  [B, H, N, d] of dtype, read only (o and lse from fa_fwd
 *                     with the same scale, causal, key_lens, dropout_p, seed).
 *   lse               [B, H, N] fp32, read only.
 *   dq, dk, dv        [B, H, N, d] of dtype, written.
 *   workspace         device buffer of at least fa_bwd_workspace_size() bytes,
 *                     16-byte aligned; its contents on entry do not matter and
 *                     are garbage on exit.
 *
 * Every dtype and head size of fa_fwd (the MFMA kernels for 16-bit d in
 * {64, 128}, the generic kernels otherwise; fp32 without dropout).  dQ, dK
 * and dV are bitwise deterministic: each is accumulated in fp32 registers by
 * one workgroup and written once (no atomics).
 */
fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o,
                 const void* dout, const float* lse, void* dq, void* dk, void* dv,
                 int B, int H, int N, int d, fa_dtype dtype, float scale, int causal,
                 const int32_t* key_lens, float dropout_p, uint64_t seed,
                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * fa_bwd on tensors laid out by strides: strides[0..7] are those of q, k, v,
 * o, dout, dq, dk and dv (see fa_strides); NULL means all eight contiguous.
 * lse stays contiguous [B, H, N]; the workspace is sized by
 * fa_bwd_workspace_size as for fa_bwd.  Same checks, kernels and results (bit
 * for bit) as fa_bwd on the same values.
 */
fa_status fa_bwd_strided(const void* q, const void* k, const void* v, const void* o,
                         const void* dout, const float* lse, void* dq, void* dk, void* dv,
                         const fa_strides* strides, int B, int H, int N, int d, fa_dtype dtype,
                         float scale, int causal, const int32_t* key_lens, float dropout_p,
                         uint64_t seed, void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/*
 * Split backward, for shapes whose B * H leaves CUs idle (Flash Attention
 * hardware-aware optimisation, section 4: FlashAttention-2 spreads the work
 * over the sequence as well as over batch and heads).  fa_bwd launches one
 * workgroup per 128-query block for dQ and one work unit per 128-key block
 * (a causal pair of them) for dK/dV; here each of those is cut into
 * num_splits shares: dQ's workgroups take shares of a block's key tiles, and
 * dK/dV's units take shares of a block's query tiles (with a causal pair, of
 * the tiles of both blocks in turn, so the shares are equal).  Each share
 * writes fp32 partial rows to the workspace, and a combine pass sums them
 * into dq, dk and dv.
 *
 *   num_splits   1 .. FA_MAX_SPLITS (else FA_ERR_INVALID_ARG); shares
 *                without a tile are allowed and contribute zeros.
 *   workspace    device buffer of at least fa_bwd_split_workspace_size()
 *                bytes: fa_bwd's per-row terms plus three fp32
 *                [num_splits, B, H, N, d] partial arrays, each padded to a
 *                multiple of 256 bytes; 16-byte aligned, contents irrelevant
 *                on entry, garbage on exit.
 * Everything else as fa_bwd, for contiguous tensors and the MFMA kernels only
 * (FA_BF16 / FA_F16 at d in {64, 128}, else FA_ERR_UNSUPPORTED).  The result
 * is deterministic; with num_splits = 1 it equals fa_bwd's bit for bit, with
 * more shares up to rounding (the partial sums are added in another order).
 */
size_t fa_bwd_split_workspace_size(int B, int H, int N, int d, fa_dtype dtype, int num_splits);
fa_status fa_bwd_split(const void* q, const void* k, const void* v, const void* o,
                       const void* dout, const float* lse, void* dq, void* dk, void* dv,
                       int B, int H, int N, int d, fa_dtype dtype, float scale, int causal,
                       const int32_t* key_lens, float dropout_p, uint64_t seed, int num_splits,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The backward in stages.  fa_bwd enqueues fa_bwd_dq, then fa_bwd_dkdv, on its
 * stream; they are exported so that a caller can time them, or compute dK/dV
 * alone (fa_bwd_preprocess, then fa_bwd_dkdv).  Arguments have the meaning
 * and checks of fa_bwd.
 *
 * The workspace carries the backward's per-row terms, D_i = sum_k dO_ik O_ik
 * and LSE_i * log2(e), from the stage that writes them (fa_bwd_dq or
 * fa_bwd_preprocess) to fa_bwd_dkdv, which reads them: fa_bwd_dkdv must be
 * ordered after one of the two (same stream, or an event), with the same o,
 * dout and lse, and the workspace must not change while it runs.  The two
 * writers compute D with different summation orders, so dK/dV after
 * fa_bwd_preprocess can differ from fa_bwd's in the last bits.
 *
 * fa_bwd_preprocess: the per-row terms into the workspace.
 * fa_bwd_dq: dQ, plus the per-row terms into the workspace.  Each 128-query
 *   block is one workgroup that walks the key tiles, recomputing S = scale
 *   Q K^T and dP = dO V^T from Q, K, V and the saved normaliser (ML Canon 48
 *   FlashAttention, "backward without N x N"; Flash Attention hardware-aware
 *   optimisation, section 2.2).
 * fa_bwd_dkdv: dK and dV.  Each 128-key block is walked over the query tiles
 *   by one workgroup, recomputing S and dP the same way; the launch is
 *   persistent (one workgroup per CU, each taking a chain of blocks).
 */
fa_status fa_bwd_preprocess(const void* o, const void* dout, const float* lse,
                            int B, int H, int N, int d, fa_dtype dtype,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);
fa_status fa_bwd_dq(const void* q, const void* k, const void* v, const void* o,
                    const void* dout, const float* lse, void* dq,
                    int B, int H, int N, int d, fa_dtype dtype, float scale, int causal,
                    const int32_t* key_lens, float dropout_p, uint64_t seed,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);
fa_status fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout,
                      void* dk, void* dv, int B, int H, int N, int d, fa_dtype dtype,
                      float scale, int causal, const int32_t* key_lens, float dropout_p,
                      uint64_t seed, const void* workspace, size_t workspace_bytes,
                      hipStream_t stream);

/*
 * fa_bwd without a workspace argument, for callers that cannot allocate
 * device memory (code under stream capture, tight serving loops, harnesses
 * that forbid allocation).  Same arguments (minus the workspace), checks,
 * results and determinism as fa_bwd, bit for bit: the same kernels run with
 * the per-row terms kept in a fixed device array of FA_NOALLOC_SCRATCH_BYTES
 * that the library holds on every device it runs on until the process ends.
 *
 * Limit: fa_bwd_workspace_size(B, H, N, d, dtype) <= FA_NOALLOC_SCRATCH_BYTES,
 * i.e. B * H * N up to 4,194,304 query rows; larger sizes return
 * FA_ERR_TOO_LARGE before any HIP call.  The device of `stream` (the current
 * device for NULL) selects that device's array; its address is looked up
 * once per device on the first call there (no allocation).
 *
 * Concurrency: every call on one device uses that device's single array.  Calls
 * that can overlap on one device (different streams without ordering, or
 * several host threads) race on it and give wrong gradients; order them on
 * one stream or with events.
 */
#define FA_NOALLOC_SCRATCH_BYTES (32u << 20)
fa_status fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                         const void* dout, const float* lse, void* dq, void* dk, void* dv,
                         int B, int H, int N, int d, fa_dtype dtype, float scale, int causal,
                         const int32_t* key_lens, float dropout_p, uint64_t seed,
                         hipStream_t stream);

/* Static, human-readable name of a status code ("unknown status" otherwise). */
const char* fa_status_string(fa_status s);

#ifdef __cplusplus
}
#endif

#endif /* IO_AWARE_EXACT_FA_H */
