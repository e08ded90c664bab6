// C ABI of libfa.so: argument checks (all on the host, before any HIP call),
// workspace sizing, and dispatch to the gfx950 kernel launchers.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <initializer_list>
#include <mutex>

#include "fa.h"
#include "fa_internal.hpp"

namespace {

bool aligned16(const void* p) { return p != nullptr && ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return p != nullptr && ((uintptr_t)p & 3u) == 0; }

// Element count of one [B, H, N, d] tensor, or -1 when it would overflow int64
// or the per-kernel 32-bit index ranges (rows B*H*N must fit in int32).
int64_t elems(int B, int H, int N, int d) {
  if (B <= 0 || H <= 0 || N <= 0 || d <= 0) return -1;
  const int64_t rows = (int64_t)B * H * N;
  if (rows > INT32_MAX) return -1;
  const int64_t n = rows * d;
  if (n / d != rows) return -1;
  return n;
}

bool valid_dtype(fa_dtype t) { return t == FA_F32 || t == FA_BF16 || t == FA_F16; }
bool is16(fa_dtype t) { return t == FA_BF16 || t == FA_F16; }
// The MFMA kernels: 16-bit types at d = 64 and 128 (the split entry points
// take only these).  Every other supported combination runs on the generic
// kernels, except padded_path below.
bool mfma_path(fa_dtype t, int d) { return is16(t) && (d == 64 || d == 128); }
uint64_t elem_bytes(fa_dtype t) { return t == FA_F32 ? 4 : 2; }

// 16-bit d = 32 and 96 run on the MFMA kernels of width 64 and 128 with the
// columns past d zero-padded on chip.  Those kernels park the lanes of the
// padding columns at byte offset 2^31 of a slice, so every tensor's (b, h)
// slice ((N + 256) rows of its row stride) must span fewer bytes than that;
// otherwise the generic kernels run.
bool padded_path(fa_dtype t, int d, int N, std::initializer_list<int64_t> row_strides) {
  if (!is16(t) || (d != 32 && d != 96)) return false;
  for (int64_t r : row_strides)
    if (((uint64_t)N + 256) * (uint64_t)r * 2 >= (1ull << 31)) return false;
  return true;
}

// The kernels address one (b, h) slice of a tensor through a buffer resource
// whose byte range, and every tile offset inside it (rows up to 256 past the
// last, for tiles fetched ahead), is a 32-bit number: (N + 256) rows of
// `row_stride` elements must span fewer than 2^32 bytes.
bool head_bytes_fit(int N, int64_t row_stride, fa_dtype dtype) {
  return ((uint64_t)N + 256) * (uint64_t)row_stride * elem_bytes(dtype) <= (1ull << 32);
}

// The fa_strides rules of fa.h for one tensor (`output`: it is written).
// The rows are one-to-one over B x H x N (n_map, below) and one slice spans
// n_span rows (n_span = N except for packed sequences, where it is the
// longest sequence).
fa_status check_strides(const fa_strides& s, int B, int H, int N, int d, fa_dtype dtype,
                        bool output, int n_span = -1) {
  const int64_t unit = 16 / (int64_t)elem_bytes(dtype);  // elements per 16 bytes
  if (s.batch < 0 || s.head < 0 || s.row < d) return FA_ERR_INVALID_ARG;
  if (s.batch % unit != 0 || s.head % unit != 0 || s.row % unit != 0) return FA_ERR_INVALID_ARG;
  // The largest element offset, (B-1) batch + (H-1) head + (N-1) row + d - 1,
  // must fit int64: each product is kept at most 2^61, so the sum stays below
  // 2^63.
  const int64_t lim = INT64_MAX / 4;
  if (s.batch > lim / B || s.head > lim / H || s.row > lim / N) return FA_ERR_INVALID_ARG;
  if (output) {
    // Every (b, h, n) owns its own row: sorted by stride (dimensions of
    // extent 1 do not matter), each stride is at least the span of the
    // dimensions inside it, the innermost span being the d elements of a row.
    struct Dim {
      int64_t stride, extent;
    } dims[3] = {{s.batch, B}, {s.head, H}, {s.row, N}};
    std::sort(dims, dims + 3, [](const Dim& a, const Dim& b) { return a.stride < b.stride; });
    int64_t span = d;
    for (const Dim& dm : dims) {
      if (dm.extent == 1) continue;
      if (dm.stride < span) return FA_ERR_INVALID_ARG;
      span = dm.stride * (dm.extent - 1) + span;
    }
  }
  if (!head_bytes_fit(n_span < 0 ? N : n_span, s.row, dtype)) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

fa::Strides to_strides(const fa_strides* s, int H, int N, int d) {
  if (s == nullptr) return fa::contiguous_bhnd(H, N, d);
  return fa::Strides{s->batch, s->head, s->row};
}

bool valid_dropout(float p) { return isfinite(p) && p >= 0.0f && p < 1.0f; }

uint32_t drop_threshold(float p) {
  // floor(p * 2^32) in double; p < 1 keeps it below 2^32.
  return (uint32_t)floor((double)p * 4294967296.0);
}

float drop_scale(float p) { return (float)(1.0 / (1.0 - (double)p)); }

// One fp32 value per row (B * H * N of them), rounded up to 256 bytes.
size_t row_array_bytes(int B, int H, int N) {
  return (((size_t)B * H * N) * 4 + 255) & ~(size_t)255;
}

size_t pad256(size_t n) { return (n + 255) & ~(size_t)255; }

// fa_fwd (num_splits 0) and fa_fwd_split (num_splits >= 1, bf16 only, with a
// workspace of fa_fwd_split_workspace_size bytes): checks, then the launch.
// strides: q, k, v, o (NULL: contiguous).
fa_status run_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                  const fa_strides* strides, int B, int H, int N, int d, fa_dtype dtype,
                  float scale, int causal, const int32_t* key_lens, float dropout_p, uint64_t seed,
                  int num_splits, void* workspace, size_t workspace_bytes, hipStream_t stream,
                  int b0 = 0, const int32_t* cu = nullptr) {
  // cu: device offsets of packed sequences (B of them, N = the longest); the
  // caller has checked the strides by the packed-tensor rules.
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned4(lse))
    return FA_ERR_INVALID_ARG;
  if (key_lens != nullptr && ((uintptr_t)key_lens & 3u) != 0) return FA_ERR_INVALID_ARG;
  if (elems(B, H, N, d) < 0) return FA_ERR_INVALID_ARG;
  if (!isfinite(scale) || scale <= 0.0f) return FA_ERR_INVALID_ARG;
  if (!valid_dropout(dropout_p)) return FA_ERR_INVALID_ARG;
  if (!valid_dtype(dtype)) return FA_ERR_INVALID_ARG;
  if (!fa::generic_head_size(d)) return FA_ERR_UNSUPPORTED;
  if (strides != nullptr && cu == nullptr) {
    for (int t = 0; t < 4; ++t) {
      const fa_status st = check_strides(strides[t], B, H, N, d, dtype, t == 3);
      if (st != FA_OK) return st;
    }
  } else if (strides == nullptr && !head_bytes_fit(N, d, dtype)) {
    return FA_ERR_UNSUPPORTED;
  }
  if (dtype == FA_F32 && dropout_p > 0.0f) return FA_ERR_UNSUPPORTED;
  if (num_splits > 0) {
    if (!mfma_path(dtype, d)) return FA_ERR_UNSUPPORTED;
    if (!aligned16(workspace)) return FA_ERR_INVALID_ARG;
    if (workspace_bytes < fa_fwd_split_workspace_size(B, H, N, d, dtype, num_splits))
      return FA_ERR_INVALID_ARG;
  }

  fa::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.fp16 = dtype == FA_F16;
  a.sq = to_strides(strides ? &strides[0] : nullptr, H, N, d);
  a.sk = to_strides(strides ? &strides[1] : nullptr, H, N, d);
  a.sv = to_strides(strides ? &strides[2] : nullptr, H, N, d);
  a.so = to_strides(strides ? &strides[3] : nullptr, H, N, d);
  a.B = B;
  a.H = H;
  a.N = N;
  a.d = d;
  a.scale = scale;
  a.causal = causal != 0;
  a.key_lens = key_lens;
  a.dropout_p = dropout_p;
  a.drop_threshold = drop_threshold(dropout_p);
  a.drop_scale = drop_scale(dropout_p);
  a.seed = seed;
  a.b0 = b0;
  a.cu = cu;
  if (num_splits > 0) {
    const size_t rows = (size_t)B * H * N;
    a.num_splits = num_splits;
    a.opart = (float*)workspace;
    a.lsepart = (float*)((char*)workspace + pad256((size_t)num_splits * rows * d * 4));
  }
  hipError_t e;
  const bool mfma = mfma_path(dtype, d) || padded_path(dtype, d, N, {a.sq.n, a.sk.n, a.sv.n, a.so.n});
  if (cu != nullptr && !mfma) return FA_ERR_UNSUPPORTED;  // device offsets: MFMA kernels only
  if (mfma)
    e = fa::launch_fwd_16(a, stream);
  else
    e = fa::launch_fwd_generic(a, (int)dtype, stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

extern "C" {

const char* fa_status_string(fa_status s) {
  switch (s) {
    case FA_OK: return "ok";
    case FA_ERR_INVALID_ARG: return "invalid argument";
    case FA_ERR_UNSUPPORTED: return "unsupported configuration";
    case FA_ERR_HIP: return "HIP launch error";
    case FA_ERR_TOO_LARGE: return "sizes exceed the fixed scratch of this entry point";
  }
  return "unknown status";
}

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                 int N, int d, fa_dtype dtype, float scale, int causal, const int32_t* key_lens,
                 float dropout_p, uint64_t seed, hipStream_t stream) {
  return run_fwd(q, k, v, o, lse, nullptr, B, H, N, d, dtype, scale, causal, key_lens, dropout_p,
                 seed, 0, nullptr, 0, stream);
}

fa_status fa_fwd_strided(const void* q, const void* k, const void* v, void* o, float* lse,
                         const fa_strides* strides, int B, int H, int N, int d, fa_dtype dtype,
                         float scale, int causal, const int32_t* key_lens, float dropout_p,
                         uint64_t seed, hipStream_t stream) {
  return run_fwd(q, k, v, o, lse, strides, B, H, N, d, dtype, scale, causal, key_lens, dropout_p,
                 seed, 0, nullptr, 0, stream);
}

size_t fa_fwd_split_workspace_size(int B, int H, int N, int d, fa_dtype dtype, int num_splits) {
  if (elems(B, H, N, d) < 0 || !mfma_path(dtype, d) || num_splits < 1 ||
      num_splits > FA_MAX_SPLITS || !head_bytes_fit(N, d, dtype))
    return 0;
  const size_t rows = (size_t)B * H * N;
  return pad256((size_t)num_splits * rows * d * 4) + pad256((size_t)num_splits * rows * 4);
}

fa_status fa_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                       int H, int N, int d, fa_dtype dtype, float scale, int causal,
                       const int32_t* key_lens, float dropout_p, uint64_t seed, int num_splits,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (num_splits < 1 || num_splits > FA_MAX_SPLITS) return FA_ERR_INVALID_ARG;
  return run_fwd(q, k, v, o, lse, nullptr, B, H, N, d, dtype, scale, causal, key_lens, dropout_p,
                 seed, num_splits, workspace, workspace_bytes, stream);
}

size_t fa_bwd_workspace_size(int B, int H, int N, int d, fa_dtype dtype) {
  if (!valid_dtype(dtype) || !fa::generic_head_size(d)) return 0;
  if (elems(B, H, N, d) < 0 || !head_bytes_fit(N, d, dtype)) return 0;
  return 2 * row_array_bytes(B, H, N);
}

}  // extern "C"

namespace {

// Checks shared by fa_bwd and its stages; pointers that a stage does not use
// are passed as a non-null aligned placeholder by that stage.
// Stands for a tensor a stage does not read: aligned, never dereferenced.
const void* const kUnused = (const void*)(uintptr_t)16;
const float* const kNoLse = (const float*)kUnused;

// `lse` (when the stage reads it) needs 4-byte alignment only.
fa_status check_bwd(std::initializer_list<const void*> ptrs, const float* lse, int B, int H, int N,
                    int d, fa_dtype dtype, float scale, float dropout_p, const void* workspace,
                    size_t workspace_bytes, const int32_t* key_lens = nullptr) {
  for (const void* ptr : ptrs)
    if (!aligned16(ptr)) return FA_ERR_INVALID_ARG;
  if (lse != kNoLse && !aligned4(lse)) return FA_ERR_INVALID_ARG;
  if (!aligned16(workspace)) return FA_ERR_INVALID_ARG;
  if (key_lens != nullptr && ((uintptr_t)key_lens & 3u) != 0) return FA_ERR_INVALID_ARG;
  if (elems(B, H, N, d) < 0) return FA_ERR_INVALID_ARG;
  if (!isfinite(scale) || scale <= 0.0f) return FA_ERR_INVALID_ARG;
  if (!valid_dropout(dropout_p)) return FA_ERR_INVALID_ARG;
  if (!valid_dtype(dtype)) return FA_ERR_INVALID_ARG;
  if (!fa::generic_head_size(d)) return FA_ERR_UNSUPPORTED;
  if (dtype == FA_F32 && dropout_p > 0.0f) return FA_ERR_UNSUPPORTED;
  if (!head_bytes_fit(N, d, dtype)) return FA_ERR_UNSUPPORTED;
  if (workspace_bytes < fa_bwd_workspace_size(B, H, N, d, dtype)) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

// strides: q, k, v, o, dout, dq, dk, dv (NULL: contiguous).
fa_status run_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                  const float* lse, void* dq, void* dk, void* dv, const fa_strides* strides, int B,
                  int H, int N, int d, fa_dtype dtype, float scale, int causal,
                  const int32_t* key_lens, float dropout_p, uint64_t seed, void* workspace,
                  int stages, hipStream_t stream, int b0 = 0, int num_splits = 0,
                  float* dqp = nullptr, float* dkp = nullptr, float* dvp = nullptr,
                  const int32_t* cu = nullptr, int64_t cu_rows = 0) {
  // cu: device offsets of packed sequences (B of them, N = the longest) whose
  // H * cu_rows per-row terms fill the workspace; the caller has checked the
  // rest.
  fa::BwdArgs a;
  a.fp16 = dtype == FA_F16;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.B = B;
  a.H = H;
  a.N = N;
  a.d = d;
  a.scale = scale;
  a.causal = causal != 0;
  a.key_lens = key_lens;
  a.dropout_p = dropout_p;
  a.drop_threshold = drop_threshold(dropout_p);
  a.drop_scale = drop_scale(dropout_p);
  a.seed = seed;
  a.b0 = b0;
  // workspace: D, then LSE * log2(e)
  a.delta = (float*)workspace;
  a.lse2 = (float*)((char*)workspace + (cu ? pad256((size_t)H * cu_rows * 4) : row_array_bytes(B, H, N)));
  a.cu = cu;
  a.num_splits = num_splits;
  a.dqp = dqp;
  a.dkp = dkp;
  a.dvp = dvp;
  fa::Strides* dst[8] = {&a.sq, &a.sk, &a.sv, &a.so, &a.sdo, &a.sdq, &a.sdk, &a.sdv};
  for (int t = 0; t < 8; ++t) *dst[t] = to_strides(strides ? &strides[t] : nullptr, H, N, d);
  const bool mfma = mfma_path(dtype, d) ||
                    padded_path(dtype, d, N, {a.sq.n, a.sk.n, a.sv.n, a.so.n, a.sdo.n, a.sdq.n, a.sdk.n,
                                              a.sdv.n});
  if (cu != nullptr && !mfma) return FA_ERR_UNSUPPORTED;  // device offsets: MFMA kernels only
  const hipError_t e = mfma ? fa::launch_bwd_16(a, stages, stream)
                            : fa::launch_bwd_generic(a, (int)dtype, stages, stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}


}  // namespace

extern "C" {

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                 fa_dtype dtype, float scale, int causal, const int32_t* key_lens, float dropout_p,
                 uint64_t seed, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const fa_status st = check_bwd({q, k, v, o, dout, dq, dk, dv}, lse,
                                 B, H, N, d, dtype, scale, dropout_p, workspace, workspace_bytes,
                                 key_lens);
  if (st != FA_OK) return st;
  return run_bwd(q, k, v, o, dout, lse, dq, dk, dv, nullptr, B, H, N, d, dtype, scale, causal,
                 key_lens, dropout_p, seed, workspace, fa::kBwdAll, stream);
}

fa_status fa_bwd_strided(const void* q, const void* k, const void* v, const void* o,
                         const void* dout, const float* lse, void* dq, void* dk, void* dv,
                         const fa_strides* strides, int B, int H, int N, int d, fa_dtype dtype,
                         float scale, int causal, const int32_t* key_lens, float dropout_p,
                         uint64_t seed, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  // The strides first (after what they depend on), then every check of fa_bwd.
  if (elems(B, H, N, d) < 0 || !valid_dtype(dtype)) return FA_ERR_INVALID_ARG;
  if (strides != nullptr) {
    for (int t = 0; t < 8; ++t) {
      const fa_status st = check_strides(strides[t], B, H, N, d, dtype, t >= 5);
      if (st != FA_OK) return st;
    }
  }
  const fa_status st = check_bwd({q, k, v, o, dout, dq, dk, dv}, lse,
                                 B, H, N, d, dtype, scale, dropout_p, workspace, workspace_bytes,
                                 key_lens);
  if (st != FA_OK) return st;
  return run_bwd(q, k, v, o, dout, lse, dq, dk, dv, strides, B, H, N, d, dtype, scale, causal,
                 key_lens, dropout_p, seed, workspace, fa::kBwdAll, stream);
}

fa_status fa_bwd_preprocess(const void* o, const void* dout, const float* lse, int B, int H, int N,
                            int d, fa_dtype dtype, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
  const fa_status st = check_bwd({o, dout}, lse,
                                 B, H, N, d, dtype, 1.0f, 0.0f, workspace, workspace_bytes);
  if (st != FA_OK) return st;
  return run_bwd(kUnused, kUnused, kUnused, o, dout, lse, nullptr, nullptr, nullptr, nullptr, B, H,
                 N, d, dtype, 1.0f, 0, nullptr, 0.0f, 0, workspace, fa::kBwdPre, stream);
}

fa_status fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout, void* dk,
                      void* dv, int B, int H, int N, int d, fa_dtype dtype, float scale, int causal,
                      const int32_t* key_lens, float dropout_p, uint64_t seed,
                      const void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const fa_status st = check_bwd({q, k, v, dout, dk, dv}, kNoLse,
                                 B, H, N, d, dtype, scale, dropout_p, workspace, workspace_bytes,
                                 key_lens);
  if (st != FA_OK) return st;
  return run_bwd(q, k, v, kUnused, dout, kNoLse, nullptr, dk, dv, nullptr, B, H, N, d, dtype, scale,
                 causal, key_lens, dropout_p, seed, (void*)workspace, fa::kBwdKV, stream);
}

fa_status fa_bwd_dq(const void* q, const void* k, const void* v, const void* o, const void* dout,
                    const float* lse, void* dq, int B, int H, int N, int d, fa_dtype dtype,
                    float scale, int causal, const int32_t* key_lens, float dropout_p,
                    uint64_t seed, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const fa_status st = check_bwd({q, k, v, o, dout, dq}, lse,
                                 B, H, N, d, dtype, scale, dropout_p, workspace, workspace_bytes,
                                 key_lens);
  if (st != FA_OK) return st;
  return run_bwd(q, k, v, o, dout, lse, dq, nullptr, nullptr, nullptr, B, H, N, d, dtype, scale,
                 causal, key_lens, dropout_p, seed, workspace, fa::kBwdQ, stream);
}

size_t fa_bwd_split_workspace_size(int B, int H, int N, int d, fa_dtype dtype, int num_splits) {
  if (elems(B, H, N, d) < 0 || !mfma_path(dtype, d) || num_splits < 1 ||
      num_splits > FA_MAX_SPLITS || !head_bytes_fit(N, d, dtype))
    return 0;
  const size_t part = pad256((size_t)num_splits * B * H * N * d * 4);
  return fa_bwd_workspace_size(B, H, N, d, dtype) + 3 * part;
}

fa_status fa_bwd_split(const void* q, const void* k, const void* v, const void* o,
                       const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                       int H, int N, int d, fa_dtype dtype, float scale, int causal,
                       const int32_t* key_lens, float dropout_p, uint64_t seed, int num_splits,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (num_splits < 1 || num_splits > FA_MAX_SPLITS) return FA_ERR_INVALID_ARG;
  fa_status st = check_bwd({q, k, v, o, dout, dq, dk, dv}, lse, B, H, N, d, dtype, scale,
                           dropout_p, workspace, workspace_bytes, key_lens);
  if (st != FA_OK) return st;
  if (!mfma_path(dtype, d)) return FA_ERR_UNSUPPORTED;
  if (workspace_bytes < fa_bwd_split_workspace_size(B, H, N, d, dtype, num_splits))
    return FA_ERR_INVALID_ARG;
  // workspace: D, LSE * log2(e), then the partial dQ, dK and dV rows
  const size_t base = fa_bwd_workspace_size(B, H, N, d, dtype);
  const size_t part = pad256((size_t)num_splits * B * H * N * d * 4);
  char* ws = (char*)workspace;
  return run_bwd(q, k, v, o, dout, lse, dq, dk, dv, nullptr, B, H, N, d, dtype, scale, causal,
                 key_lens, dropout_p, seed, workspace, fa::kBwdAll, stream, 0, num_splits,
                 (float*)(ws + base), (float*)(ws + base + part), (float*)(ws + base + 2 * part));
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Packed sequences: the kernels once per sequence, on offset pointers.
// ---------------------------------------------------------------------------

namespace {

// cu_seqlens: starts at 0, non-decreasing.  Longest sequence and total tokens.
fa_status check_seqs(const int32_t* cu, int num_seqs, int* longest, int* total) {
  if (cu == nullptr || num_seqs < 1 || cu[0] != 0) return FA_ERR_INVALID_ARG;
  int mx = 0;
  for (int b = 0; b < num_seqs; ++b) {
    if (cu[b + 1] < cu[b]) return FA_ERR_INVALID_ARG;
    mx = std::max(mx, cu[b + 1] - cu[b]);
  }
  *longest = mx;
  *total = cu[num_seqs];
  return FA_OK;
}

// Per-sequence strides of n tensors (the first `first_output` are read,
// the rest written), checked over the whole packed tensors: rows one-to-one
// over all `total` tokens, a slice of `longest` rows within 32 bits.
fa_status packed_strides(const fa_strides* in, int n, int first_output, int H, int total,
                         int longest, int d, fa_dtype dtype, fa_strides* out) {
  for (int t = 0; t < n; ++t) {
    out[t] = in ? fa_strides{0, in[t].head, in[t].row} : fa_strides{0, d, (int64_t)H * d};
    const fa_status st =
        check_strides(out[t], 1, H, std::max(total, 1), d, dtype, t >= first_output, longest);
    if (st != FA_OK) return st;
  }
  return FA_OK;
}

template <typename P>
P at_row(P base, int64_t row, const fa_strides& s, fa_dtype dtype) {
  return (P)((const char*)base + row * s.row * (int64_t)elem_bytes(dtype));
}

}  // namespace

extern "C" {

fa_status fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                        const fa_strides* strides, const int32_t* cu_seqlens, int num_seqs,
                        int H, int d, fa_dtype dtype, float scale, int causal, float dropout_p,
                        uint64_t seed, hipStream_t stream) {
  int longest = 0, total = 0;
  fa_status st = check_seqs(cu_seqlens, num_seqs, &longest, &total);
  if (st != FA_OK) return st;
  if (H <= 0 || d <= 0 || !valid_dtype(dtype)) return FA_ERR_INVALID_ARG;
  if (!fa::generic_head_size(d)) return FA_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned4(lse))
    return FA_ERR_INVALID_ARG;
  fa_strides s[4];
  st = packed_strides(strides, 4, 3, H, total, longest, d, dtype, s);
  if (st != FA_OK) return st;
  for (int b = 0; b < num_seqs; ++b) {
    const int64_t t0 = cu_seqlens[b];
    const int len = cu_seqlens[b + 1] - cu_seqlens[b];
    if (len == 0) continue;
    st = run_fwd(at_row(q, t0, s[0], dtype), at_row(k, t0, s[1], dtype), at_row(v, t0, s[2], dtype),
                 at_row(o, t0, s[3], dtype), lse + (int64_t)H * t0, s, 1, H, len, d, dtype, scale,
                 causal, nullptr, dropout_p, seed, 0, nullptr, 0, stream, b);
    if (st != FA_OK) return st;
  }
  return FA_OK;
}

size_t fa_bwd_varlen_workspace_size(const int32_t* cu_seqlens, int num_seqs, int H, int d,
                                    fa_dtype dtype) {
  int longest = 0, total = 0;
  if (check_seqs(cu_seqlens, num_seqs, &longest, &total) != FA_OK || longest == 0) return 0;
  return fa_bwd_workspace_size(1, H, longest, d, dtype);
}

fa_status fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                        const void* dout, const float* lse, void* dq, void* dk, void* dv,
                        const fa_strides* strides, const int32_t* cu_seqlens, int num_seqs,
                        int H, int d, fa_dtype dtype, float scale, int causal, float dropout_p,
                        uint64_t seed, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
  int longest = 0, total = 0;
  fa_status st = check_seqs(cu_seqlens, num_seqs, &longest, &total);
  if (st != FA_OK) return st;
  if (H <= 0 || d <= 0 || !valid_dtype(dtype)) return FA_ERR_INVALID_ARG;
  if (!fa::generic_head_size(d)) return FA_ERR_UNSUPPORTED;
  fa_strides s[8];
  st = packed_strides(strides, 8, 5, H, total, longest, d, dtype, s);
  if (st != FA_OK) return st;
  for (int b = 0; b < num_seqs; ++b) {
    const int64_t t0 = cu_seqlens[b];
    const int len = cu_seqlens[b + 1] - cu_seqlens[b];
    if (len == 0) continue;
    const void* qb = at_row(q, t0, s[0], dtype);
    const void* kb = at_row(k, t0, s[1], dtype);
    const void* vb = at_row(v, t0, s[2], dtype);
    const void* ob = at_row(o, t0, s[3], dtype);
    const void* dob = at_row(dout, t0, s[4], dtype);
    void* dqb = at_row(dq, t0, s[5], dtype);
    void* dkb = at_row(dk, t0, s[6], dtype);
    void* dvb = at_row(dv, t0, s[7], dtype);
    const float* lb = lse + (int64_t)H * t0;
    st = check_bwd({qb, kb, vb, ob, dob, dqb, dkb, dvb}, lb, 1, H, len, d, dtype, scale, dropout_p,
                   workspace, workspace_bytes);
    if (st != FA_OK) return st;
    st = run_bwd(qb, kb, vb, ob, dob, lb, dqb, dkb, dvb, s, 1, H, len, d, dtype, scale, causal,
                 nullptr, dropout_p, seed, workspace, fa::kBwdAll, stream, b);
    if (st != FA_OK) return st;
  }
  return FA_OK;
}

}  // extern "C"

namespace {

// Arguments of the device-offset entry points: offsets on the device, counts
// and the longest length from the caller.  Strides as for the host-offset
// ones, with the longest sequence for the 32-bit span.
fa_status check_packed_dev(const int32_t* cu, int num_seqs, int max_len, int total, int H, int d,
                           fa_dtype dtype, float scale, float dropout_p) {
  if (cu == nullptr || ((uintptr_t)cu & 3u) != 0) return FA_ERR_INVALID_ARG;
  if (num_seqs < 1 || max_len < 0 || total < 0 || H <= 0 || d <= 0) return FA_ERR_INVALID_ARG;
  if (!valid_dtype(dtype)) return FA_ERR_INVALID_ARG;
  if (!isfinite(scale) || scale <= 0.0f) return FA_ERR_INVALID_ARG;
  if (!valid_dropout(dropout_p)) return FA_ERR_INVALID_ARG;
  if (!fa::generic_head_size(d)) return FA_ERR_UNSUPPORTED;
  // one launch needs the MFMA kernels (16-bit, d = 32 .. 128)
  if (!is16(dtype) || d > 128) return FA_ERR_UNSUPPORTED;
  if (max_len > 0 && elems(num_seqs, H, max_len, d) < 0) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

}  // namespace

extern "C" {

fa_status fa_fwd_varlen_device(const void* q, const void* k, const void* v, void* o, float* lse,
                               const fa_strides* strides, const int32_t* cu_seqlens, int num_seqs,
                               int max_len, int total_tokens, int H, int d, fa_dtype dtype,
                               float scale, int causal, float dropout_p, uint64_t seed,
                               hipStream_t stream) {
  fa_status st = check_packed_dev(cu_seqlens, num_seqs, max_len, total_tokens, H, d, dtype, scale,
                                  dropout_p);
  if (st != FA_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned4(lse))
    return FA_ERR_INVALID_ARG;
  fa_strides s[4];
  st = packed_strides(strides, 4, 3, H, total_tokens, max_len, d, dtype, s);
  if (st != FA_OK) return st;
  if (max_len == 0 || total_tokens == 0) return FA_OK;
  return run_fwd(q, k, v, o, lse, s, num_seqs, H, max_len, d, dtype, scale, causal, nullptr,
                 dropout_p, seed, 0, nullptr, 0, stream, 0, cu_seqlens);
}

size_t fa_bwd_varlen_device_workspace_size(int total_tokens, int H, int d, fa_dtype dtype) {
  if (total_tokens < 0 || H <= 0 || !valid_dtype(dtype) || !fa::generic_head_size(d)) return 0;
  if (elems(1, H, total_tokens, d) < 0) return 0;
  return 2 * pad256((size_t)H * total_tokens * 4);
}

fa_status fa_bwd_varlen_device(const void* q, const void* k, const void* v, const void* o,
                               const void* dout, const float* lse, void* dq, void* dk, void* dv,
                               const fa_strides* strides, const int32_t* cu_seqlens, int num_seqs,
                               int max_len, int total_tokens, int H, int d, fa_dtype dtype,
                               float scale, int causal, float dropout_p, uint64_t seed,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  fa_status st = check_packed_dev(cu_seqlens, num_seqs, max_len, total_tokens, H, d, dtype, scale,
                                  dropout_p);
  if (st != FA_OK) return st;
  for (const void* ptr : {q, k, v, o, dout, (const void*)dq, (const void*)dk, (const void*)dv})
    if (!aligned16(ptr)) return FA_ERR_INVALID_ARG;
  if (!aligned4(lse) || !aligned16(workspace)) return FA_ERR_INVALID_ARG;
  if (workspace_bytes < fa_bwd_varlen_device_workspace_size(total_tokens, H, d, dtype))
    return FA_ERR_INVALID_ARG;
  fa_strides s[8];
  st = packed_strides(strides, 8, 5, H, total_tokens, max_len, d, dtype, s);
  if (st != FA_OK) return st;
  if (max_len == 0 || total_tokens == 0) return FA_OK;
  return run_bwd(q, k, v, o, dout, lse, dq, dk, dv, s, num_seqs, H, max_len, d, dtype, scale,
                 causal, nullptr, dropout_p, seed, workspace, fa::kBwdAll, stream, 0, 0, nullptr,
                 nullptr, nullptr, cu_seqlens, total_tokens);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// fa_bwd_noalloc: fa_bwd with its per-row workspace in a fixed device array,
// for callers that cannot allocate device memory.
// ---------------------------------------------------------------------------

// The backward's per-row terms (D, then LSE * log2(e)) for every call of
// fa_bwd_noalloc on a device.  Each device holds its own copy at its own
// address, kept until the process ends.  In host code `scratch` names a
// host-side stand-in, never the device memory: only the address returned by
// hipGetSymbolAddress for a device may be handed to kernels.
static __device__ __align__(256) unsigned char scratch[FA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` per device, once resolved

// Device address of `scratch` on the device `stream` belongs to (the current
// device for the NULL stream), resolved once per device with that device
// current.
fa_status scratch_for(hipStream_t stream, void** out) {
  int dev = 0;
  if (stream != nullptr) {
    hipDevice_t d = 0;
    if (hipStreamGetDevice(stream, &d) != hipSuccess) return FA_ERR_HIP;
    dev = (int)d;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return FA_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return FA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    int cur = 0;
    if (hipGetDevice(&cur) != hipSuccess) return FA_ERR_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return FA_ERR_HIP;
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return FA_ERR_HIP;
    if (e != hipSuccess || ptr == nullptr) return FA_ERR_HIP;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return FA_OK;
}

}  // namespace

extern "C" {

fa_status fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                         const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                         int H, int N, int d, fa_dtype dtype, float scale, int causal,
                         const int32_t* key_lens, float dropout_p, uint64_t seed,
                         hipStream_t stream) {
  // Every argument check of fa_bwd, with the scratch standing in for the
  // workspace (a placeholder address here: nothing is launched before the
  // real one is known), then the size limit, all before any HIP call.
  const size_t need = fa_bwd_workspace_size(B, H, N, d, dtype);
  fa_status st = check_bwd({q, k, v, o, dout, dq, dk, dv}, lse,
                           B, H, N, d, dtype, scale, dropout_p, kUnused, need, key_lens);
  if (st != FA_OK) return st;
  if (need > (size_t)FA_NOALLOC_SCRATCH_BYTES) return FA_ERR_TOO_LARGE;
  void* ws = nullptr;
  st = scratch_for(stream, &ws);
  if (st != FA_OK) return st;
  // The dQ stage writes D and LSE * log2(e) for every row before the dK/dV
  // stage reads them (same stream), so nothing needs clearing.
  return run_bwd(q, k, v, o, dout, lse, dq, dk, dv, nullptr, B, H, N, d, dtype, scale, causal,
                 key_lens, dropout_p, seed, ws, fa::kBwdAll, stream);
}

}  // extern "C"
