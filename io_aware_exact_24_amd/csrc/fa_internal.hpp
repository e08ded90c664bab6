// Host-side argument bundles passed from the C ABI layer to the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

// Element strides (batch, head, row) of a [B, H, N, d]-indexed tensor whose
// head dimension is contiguous.
struct Strides {
  int64_t b, h, n;
};
inline Strides contiguous_bhnd(int H, int N, int d) {
  return Strides{(int64_t)H * N * d, (int64_t)N * d, (int64_t)d};
}

struct FwdArgs {
  bool fp16 = false;  // 16-bit element type: fp16 instead of bf16
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  Strides sq, sk, sv, so;
  int B, H, N, d;
  float scale;
  int causal;
  const int32_t* key_lens;  // device [B] or nullptr
  float dropout_p;          // 0 disables dropout
  uint32_t drop_threshold;  // floor(p * 2^32)
  float drop_scale;         // fp32(1 / (1 - p))
  uint64_t seed;
  int b0 = 0;  // batch index of entry 0 in the dropout counter (packed sequences)
  // Packed sequences in one launch: device offsets, entry b = rows [cu[b],
  // cu[b+1]) (batch strides 0, N = the longest); nullptr otherwise.
  const int32_t* cu = nullptr;
  // Split-KV (bf16 only): num_splits > 0 splits each query block's key tiles
  // that many ways into the fp32 workspaces opart [S][B*H][N][d] and
  // lsepart [S][B*H][N], then combines them into o and lse.  0: one pass.
  int num_splits = 0;
  float* opart = nullptr;
  float* lsepart = nullptr;
};

struct BwdArgs {
  bool fp16 = false;  // 16-bit element type: fp16 instead of bf16
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  Strides sq, sk, sv, so, sdo, sdq, sdk, sdv;
  int B, H, N, d;
  float scale;
  int causal;
  const int32_t* key_lens;
  float dropout_p;
  uint32_t drop_threshold;
  float drop_scale;
  uint64_t seed;
  int b0 = 0;  // batch index of entry 0 in the dropout counter (packed sequences)
  const int32_t* cu = nullptr;  // packed sequences in one launch (see FwdArgs)
  float* delta;   // workspace: fp32 [B, H, N], D_i = sum_k dO_ik O_ik
  float* lse2;    // workspace: fp32 [B, H, N], LSE_i * log2(e) (+inf for an empty row)
  // Split backward (16-bit, contiguous, d in {64, 128}): num_splits > 0 splits
  // dQ's key range and dK/dV's query range that many ways into the fp32
  // workspaces dqp, dkp, dvp [S][B*H][N][d], then sums them into dq, dk, dv.
  // 0: every gradient accumulated in one pass.
  int num_splits = 0;
  float* dqp = nullptr;
  float* dkp = nullptr;
  float* dvp = nullptr;
};

// Each returns hipSuccess or the launch error.
hipError_t launch_fwd_16(const FwdArgs& a, hipStream_t s);  // bf16 or fp16
// Backward stages, selected by a bit mask and launched in this order: the
// per-row preprocessing alone (D and LSE*log2e into the workspace), the dQ
// kernel (which also computes those per-row terms and writes them to the
// workspace), the dK/dV kernel (which reads them).  The full backward is
// kBwdQ | kBwdKV.
enum : int { kBwdPre = 1, kBwdKV = 2, kBwdQ = 4, kBwdAll = kBwdQ | kBwdKV };
hipError_t launch_bwd_16(const BwdArgs& a, int stages, hipStream_t s);  // bf16 or fp16

// The generic (VALU, fp32-accumulating) kernels: element type `elem` (0 fp32,
// 1 bf16, 2 fp16, the fa_dtype codes) and head size d with
// generic_head_size(d); the same stage bits as launch_bwd_16.
bool generic_head_size(int d);
hipError_t launch_fwd_generic(const FwdArgs& a, int elem, hipStream_t s);
hipError_t launch_bwd_generic(const BwdArgs& a, int elem, int stages, hipStream_t s);

}  // namespace fa
