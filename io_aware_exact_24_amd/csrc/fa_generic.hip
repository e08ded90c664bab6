// Generic attention kernels: every element type (fp32, bf16, fp16) and head
// size d in {32, 64, 96, 128, 256}, for the cases the MFMA kernels do not
// cover (the fp32 backward, and 16-bit head sizes other than 64 and 128).
//
// They compute the same quantities as the MFMA kernels (the definitions in
// include/fa.h: masks, Philox dropout, LSE before dropout; the backward's
// per-row terms D_i = sum_k dO_ik O_ik and LSE_i * log2 e in the workspace,
// written by the dQ or preprocessing kernel and read by the dK/dV kernel),
// tiled the same way (FlashAttention first principles: blocks of queries
// against blocks of keys staged in on-chip memory, running row max and sum,
// no N x N matrix in device memory; ML Canon 48 FlashAttention, "backward
// without N x N", for the recomputation), but with plain fp32 VALU
// arithmetic: correctness first, not tuned.
//
// One workgroup of 256 threads per block of 32 rows (query rows for the
// forward and dQ, key rows for dK/dV); tiles of 32 rows of the other side
// are staged in LDS as fp32 with rows padded to d + 4 floats (the 8 threads
// that read 8 different rows at one column hit 8 different bank groups).
// Thread t owns row t / 8 of its block and the columns c = t % 8 + 8 k of
// that row; its 8-thread group reduces row maxima and sums with lane
// exchanges.
#include <hip/hip_runtime.h>
#include <math.h>

#include "fa_common.hpp"
#include "fa_internal.hpp"

namespace fa {
namespace {

constexpr int GB = 32;         // rows per block, rows per staged tile
constexpr int GT = 256;        // threads per workgroup
constexpr int GS = GT / GB;    // threads per row
template <int D>
constexpr int pitch() { return D + 4; }  // floats per LDS row

struct GParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;       // forward: output; backward: the forward's O
  const void* dout;
  float* lse;          // forward output (natural log)
  const float* lse_in; // backward input
  void* dq;
  void* dk;
  void* dv;
  float* delta;        // workspace: D
  float* lse2;         // workspace: LSE * log2 e, +inf for a row with no allowed key
  Strides sq, sk, sv, so, sdo, sdq, sdk, sdv;
  const int32_t* key_lens;
  int H, N;
  int b0;  // added to the batch index in the dropout counter
  float scale;
  int causal;
  int dropout;
  uint32_t drop_threshold;
  float drop_scale;
  uint32_t seed_lo, seed_hi;
};

template <typename E>
__device__ __forceinline__ float f32_of(E x) { return (float)x; }
template <typename E>
__device__ __forceinline__ E of_f32(float x) { return (E)x; }  // round to nearest even

// Rows [r0, r0 + 32) of a slice (rows `sn` elements apart) into an LDS tile
// as fp32; rows at or past `nrows` are zero.
template <typename E, int D>
__device__ void stage(float* tile, const E* base, int64_t sn, int r0, int nrows) {
  for (int idx = threadIdx.x; idx < GB * D; idx += GT) {
    const int r = idx / D, c = idx - r * D;
    const int row = r0 + r;
    tile[r * pitch<D>() + c] = row < nrows ? f32_of(base[(int64_t)row * sn + c]) : 0.0f;
  }
}

template <int D>
__device__ __forceinline__ float dot_rows(const float* a, const float* b) {
  float s = 0.0f;
#pragma unroll 8
  for (int c = 0; c < D; c += 4) {
    const f32x4 x = *(const f32x4*)(a + c), y = *(const f32x4*)(b + c);
    s = fmaf(x[0], y[0], s);
    s = fmaf(x[1], y[1], s);
    s = fmaf(x[2], y[2], s);
    s = fmaf(x[3], y[3], s);
  }
  return s;
}

// max and sum over the 8 threads of a row (consecutive lanes of one wave)
__device__ __forceinline__ float row_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 1));
  x = fmaxf(x, __shfl_xor(x, 2));
  return fmaxf(x, __shfl_xor(x, 4));
}
__device__ __forceinline__ float row_sum(float x) {
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  return x + __shfl_xor(x, 4);
}

// Dropout factor of element (query i, key j) of head (b, h): 1/(1-p) or 0.
__device__ __forceinline__ float keep_factor(const GParams& p, int i, int j, int hi, int bi) {
  const u32x4 w = philox((uint32_t)j >> 2, (uint32_t)i, (uint32_t)hi, (uint32_t)(bi + p.b0), p.seed_lo,
                         p.seed_hi);
  return philox_word(w, j) >= p.drop_threshold ? p.drop_scale : 0.0f;
}

__device__ __forceinline__ int key_len(const GParams& p, int bi) {
  return p.key_lens ? min(max(p.key_lens[bi], 0), p.N) : p.N;
}

// ---------------------------------------------------------------------------
// Forward: O and LSE for 32 query rows, streaming 32-key tiles of K and V.
// ---------------------------------------------------------------------------
template <typename E, int D>
__global__ __launch_bounds__(GT) void fwd_generic_kernel(GParams p) {
  __shared__ __attribute__((aligned(16))) float qs[GB * pitch<D>()];
  __shared__ __attribute__((aligned(16))) float ks[GB * pitch<D>()];
  __shared__ __attribute__((aligned(16))) float vs[GB * pitch<D>()];
  __shared__ float ps[GB][GB + 1];
  const int N = p.N, nqb = (N + GB - 1) / GB;
  const int head = blockIdx.x / nqb, qb = blockIdx.x - head * nqb;
  const int bi = head / p.H, hi = head - bi * p.H;
  const int t = threadIdx.x, r = t / GS, sub = t % GS;
  const int q0 = qb * GB, qi = q0 + r;
  const int L = key_len(p, bi);
  const E* qg = (const E*)p.q + (bi * p.sq.b + hi * p.sq.h);
  const E* kg = (const E*)p.k + (bi * p.sk.b + hi * p.sk.h);
  const E* vg = (const E*)p.v + (bi * p.sv.b + hi * p.sv.h);
  E* og = (E*)p.o + (bi * p.so.b + hi * p.so.h);

  stage<E, D>(qs, qg, p.sq.n, q0, N);
  float acc[D / GS];
#pragma unroll
  for (int x = 0; x < D / GS; ++x) acc[x] = 0.0f;
  float m = -INFINITY, l = 0.0f;
  const int kend = p.causal ? min(L, q0 + GB) : L;
  for (int kt = 0; kt * GB < kend; ++kt) {
    __syncthreads();  // every thread is done with the previous tile
    stage<E, D>(ks, kg, p.sk.n, kt * GB, N);
    stage<E, D>(vs, vg, p.sv.n, kt * GB, N);
    __syncthreads();
    float s[GB / GS];
    float mt = -INFINITY;
#pragma unroll
    for (int u = 0; u < GB / GS; ++u) {
      const int j = sub + GS * u, key = kt * GB + j;
      const bool ok = key < L && (!p.causal || key <= qi);
      s[u] = ok ? p.scale * dot_rows<D>(qs + r * pitch<D>(), ks + j * pitch<D>()) : -INFINITY;
      mt = fmaxf(mt, s[u]);
    }
    const float mnew = fmaxf(m, row_max(mt));
    const float alpha = mnew == -INFINITY ? 1.0f : expf(m - mnew);
    float ls = 0.0f;
#pragma unroll
    for (int u = 0; u < GB / GS; ++u) {
      const int j = sub + GS * u;
      const float pv = s[u] == -INFINITY ? 0.0f : expf(s[u] - mnew);
      ls += pv;
      ps[r][j] = p.dropout ? pv * keep_factor(p, qi, kt * GB + j, hi, bi) : pv;
    }
    l = l * alpha + row_sum(ls);
    m = mnew;
    __syncthreads();  // the row's probabilities (written by its 8 threads) are in LDS
#pragma unroll
    for (int x = 0; x < D / GS; ++x) {
      const int c = sub + GS * x;
      float o = acc[x] * alpha;
      for (int j = 0; j < GB; ++j) o = fmaf(ps[r][j], vs[j * pitch<D>() + c], o);
      acc[x] = o;
    }
  }
  if (qi < N) {
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
    for (int x = 0; x < D / GS; ++x) og[(int64_t)qi * p.so.n + sub + GS * x] = of_f32<E>(acc[x] * inv);
    if (sub == 0) p.lse[(int64_t)head * N + qi] = l > 0.0f ? m + logf(l) : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// Backward per-row terms: D_i and LSE_i * log2 e into the workspace.
// ---------------------------------------------------------------------------
template <typename E, int D>
__global__ __launch_bounds__(GT) void bwd_generic_pre_kernel(GParams p, int64_t rows) {
  const int64_t row = (int64_t)blockIdx.x * GT + threadIdx.x;
  if (row >= rows) return;
  const int head = (int)(row / p.N), n = (int)(row - (int64_t)head * p.N);
  const int bi = head / p.H, hi = head - bi * p.H;
  const E* o = (const E*)p.o + (bi * p.so.b + hi * p.so.h + (int64_t)n * p.so.n);
  const E* d = (const E*)p.dout + (bi * p.sdo.b + hi * p.sdo.h + (int64_t)n * p.sdo.n);
  float s = 0.0f;
  for (int c = 0; c < D; ++c) s = fmaf(f32_of(d[c]), f32_of(o[c]), s);
  p.delta[row] = s;
  const float lv = p.lse_in[row];
  p.lse2[row] = lv == -INFINITY ? INFINITY : lv * kLog2e;
}

// ---------------------------------------------------------------------------
// dQ for 32 query rows, streaming 32-key tiles; writes the per-row terms.
// ---------------------------------------------------------------------------
template <typename E, int D>
__global__ __launch_bounds__(GT) void bwd_generic_dq_kernel(GParams p) {
  __shared__ __attribute__((aligned(16))) float qs[GB * pitch<D>()];
  __shared__ __attribute__((aligned(16))) float dos[GB * pitch<D>()];
  __shared__ __attribute__((aligned(16))) float ks[GB * pitch<D>()];
  __shared__ __attribute__((aligned(16))) float vs[GB * pitch<D>()];
  __shared__ float dss[GB][GB + 1];
  const int N = p.N, nqb = (N + GB - 1) / GB;
  const int head = blockIdx.x / nqb, qb = blockIdx.x - head * nqb;
  const int bi = head / p.H, hi = head - bi * p.H;
  const int t = threadIdx.x, r = t / GS, sub = t % GS;
  const int q0 = qb * GB, qi = q0 + r;
  const int L = key_len(p, bi);
  const E* qg = (const E*)p.q + (bi * p.sq.b + hi * p.sq.h);
  const E* kg = (const E*)p.k + (bi * p.sk.b + hi * p.sk.h);
  const E* vg = (const E*)p.v + (bi * p.sv.b + hi * p.sv.h);
  const E* og = (const E*)p.o + (bi * p.so.b + hi * p.so.h);
  const E* dog = (const E*)p.dout + (bi * p.sdo.b + hi * p.sdo.h);
  E* dqg = (E*)p.dq + (bi * p.sdq.b + hi * p.sdq.h);

  stage<E, D>(qs, qg, p.sq.n, q0, N);
  stage<E, D>(dos, dog, p.sdo.n, q0, N);
  __syncthreads();
  // D_i = sum_c dO_ic O_ic (this row's 8 threads split the columns) and LSE * log2 e
  float drow = 0.0f;
  if (qi < N)
    for (int c = sub; c < D; c += GS)
      drow = fmaf(dos[r * pitch<D>() + c], f32_of(og[(int64_t)qi * p.so.n + c]), drow);
  drow = row_sum(drow);
  float lrow = INFINITY;
  if (qi < N) {
    const float lv = p.lse_in[(int64_t)head * N + qi];
    lrow = lv == -INFINITY ? INFINITY : lv * kLog2e;
    if (sub == 0) {
      p.delta[(int64_t)head * N + qi] = drow;
      p.lse2[(int64_t)head * N + qi] = lrow;
    }
  }
  const float c2 = p.scale * kLog2e;
  float acc[D / GS];
#pragma unroll
  for (int x = 0; x < D / GS; ++x) acc[x] = 0.0f;
  const int kend = p.causal ? min(L, q0 + GB) : L;
  for (int kt = 0; kt * GB < kend; ++kt) {
    __syncthreads();
    stage<E, D>(ks, kg, p.sk.n, kt * GB, N);
    stage<E, D>(vs, vg, p.sv.n, kt * GB, N);
    __syncthreads();
#pragma unroll
    for (int u = 0; u < GB / GS; ++u) {
      const int j = sub + GS * u, key = kt * GB + j;
      const bool ok = key < L && (!p.causal || key <= qi);
      float ds = 0.0f;
      if (ok) {
        const float pv = exp2f(fmaf(dot_rows<D>(qs + r * pitch<D>(), ks + j * pitch<D>()), c2, -lrow));
        float dp = dot_rows<D>(dos + r * pitch<D>(), vs + j * pitch<D>());
        if (p.dropout) dp *= keep_factor(p, qi, key, hi, bi);
        ds = pv * (dp - drow);
      }
      dss[r][j] = ds;
    }
    __syncthreads();
#pragma unroll
    for (int x = 0; x < D / GS; ++x) {
      const int c = sub + GS * x;
      float a = acc[x];
      for (int j = 0; j < GB; ++j) a = fmaf(dss[r][j], ks[j * pitch<D>() + c], a);
      acc[x] = a;
    }
  }
  if (qi < N) {
#pragma unroll
    for (int x = 0; x < D / GS; ++x)
      dqg[(int64_t)qi * p.sdq.n + sub + GS * x] = of_f32<E>(acc[x] * p.scale);
  }
}

// ---------------------------------------------------------------------------
// dK and dV for 32 key rows, streaming the 32-row query tiles that can see
// them; reads the per-row terms from the workspace.
// ---------------------------------------------------------------------------
template <typename E, int D>
__global__ __launch_bounds__(GT) void bwd_generic_dkdv_kernel(GParams p) {
  __shared__ __attribute__((aligned(16))) float ks[GB * pitch<D>()];
  __shared__ __attribute__((aligned(16))) float vs[GB * pitch<D>()];
  __shared__ __attribute__((aligned(16))) float qs[GB * pitch<D>()];
  __shared__ __attribute__((aligned(16))) float dos[GB * pitch<D>()];
  __shared__ float pzs[GB][GB + 1];  // P * Z, [key][query]
  __shared__ float dss[GB][GB + 1];  // dS, [key][query]
  __shared__ float drows[GB], lrows[GB];
  const int N = p.N, nkb = (N + GB - 1) / GB;
  const int head = blockIdx.x / nkb, kb = blockIdx.x - head * nkb;
  const int bi = head / p.H, hi = head - bi * p.H;
  const int t = threadIdx.x, jr = t / GS, sub = t % GS;
  const int k0 = kb * GB, kj = k0 + jr;
  const int L = key_len(p, bi);
  const E* qg = (const E*)p.q + (bi * p.sq.b + hi * p.sq.h);
  const E* kg = (const E*)p.k + (bi * p.sk.b + hi * p.sk.h);
  const E* vg = (const E*)p.v + (bi * p.sv.b + hi * p.sv.h);
  const E* dog = (const E*)p.dout + (bi * p.sdo.b + hi * p.sdo.h);
  E* dkg = (E*)p.dk + (bi * p.sdk.b + hi * p.sdk.h);
  E* dvg = (E*)p.dv + (bi * p.sdv.b + hi * p.sdv.h);

  float adk[D / GS], adv[D / GS];
#pragma unroll
  for (int x = 0; x < D / GS; ++x) adk[x] = adv[x] = 0.0f;
  const float c2 = p.scale * kLog2e;
  if (k0 < L) {  // a block of padding keys only keeps its zero gradients
    stage<E, D>(ks, kg, p.sk.n, k0, N);
    stage<E, D>(vs, vg, p.sv.n, k0, N);
    const int it0 = p.causal ? k0 / GB : 0;
    for (int it = it0; it * GB < N; ++it) {
      __syncthreads();  // every thread is done with the previous tile
      stage<E, D>(qs, qg, p.sq.n, it * GB, N);
      stage<E, D>(dos, dog, p.sdo.n, it * GB, N);
      if (t < GB) {
        const int row = it * GB + t;
        drows[t] = row < N ? p.delta[(int64_t)head * N + row] : 0.0f;
        lrows[t] = row < N ? p.lse2[(int64_t)head * N + row] : INFINITY;
      }
      __syncthreads();
#pragma unroll
      for (int u = 0; u < GB / GS; ++u) {
        const int i = sub + GS * u, qi = it * GB + i;
        const bool ok = kj < L && qi < N && (!p.causal || kj <= qi);
        float pz = 0.0f, ds = 0.0f;
        if (ok) {
          const float pv =
              exp2f(fmaf(dot_rows<D>(qs + i * pitch<D>(), ks + jr * pitch<D>()), c2, -lrows[i]));
          const float z = p.dropout ? keep_factor(p, qi, kj, hi, bi) : 1.0f;
          const float dp = dot_rows<D>(dos + i * pitch<D>(), vs + jr * pitch<D>());
          pz = pv * z;
          ds = pv * (dp * z - drows[i]);
        }
        pzs[jr][i] = pz;
        dss[jr][i] = ds;
      }
      __syncthreads();
#pragma unroll
      for (int x = 0; x < D / GS; ++x) {
        const int c = sub + GS * x;
        float a = adv[x], b = adk[x];
        for (int i = 0; i < GB; ++i) {
          a = fmaf(pzs[jr][i], dos[i * pitch<D>() + c], a);
          b = fmaf(dss[jr][i], qs[i * pitch<D>() + c], b);
        }
        adv[x] = a;
        adk[x] = b;
      }
    }
  }
  if (kj < N) {
#pragma unroll
    for (int x = 0; x < D / GS; ++x) {
      const int c = sub + GS * x;
      dkg[(int64_t)kj * p.sdk.n + c] = of_f32<E>(adk[x] * p.scale);
      dvg[(int64_t)kj * p.sdv.n + c] = of_f32<E>(adv[x]);
    }
  }
}

GParams base_params(int H, int N, float scale, int causal, const int32_t* key_lens, float dropout_p,
                    uint32_t thr, float dscale, uint64_t seed) {
  GParams p{};
  p.H = H;
  p.N = N;
  p.scale = scale;
  p.causal = causal;
  p.key_lens = key_lens;
  p.dropout = dropout_p > 0.0f;
  p.drop_threshold = thr;
  p.drop_scale = dscale;
  p.seed_lo = (uint32_t)(seed & 0xffffffffu);
  p.seed_hi = (uint32_t)(seed >> 32);
  return p;
}

template <typename E, int D>
hipError_t fwd_e_d(const GParams& p, int heads, hipStream_t s) {
  const int grid = heads * ((p.N + GB - 1) / GB);
  hipLaunchKernelGGL((fwd_generic_kernel<E, D>), dim3(grid), dim3(GT), 0, s, p);
  return hipGetLastError();
}

template <typename E, int D>
hipError_t bwd_e_d(const GParams& p, int heads, int stages, hipStream_t s) {
  const int blocks = heads * ((p.N + GB - 1) / GB);
  if (stages & kBwdPre) {
    const int64_t rows = (int64_t)heads * p.N;
    hipLaunchKernelGGL((bwd_generic_pre_kernel<E, D>), dim3((unsigned)((rows + GT - 1) / GT)),
                       dim3(GT), 0, s, p, rows);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (stages & kBwdQ) {
    hipLaunchKernelGGL((bwd_generic_dq_kernel<E, D>), dim3(blocks), dim3(GT), 0, s, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (stages & kBwdKV) {
    hipLaunchKernelGGL((bwd_generic_dkdv_kernel<E, D>), dim3(blocks), dim3(GT), 0, s, p);
    return hipGetLastError();
  }
  return hipSuccess;
}

struct FwdCall {
  const GParams& p;
  int heads;
  hipStream_t s;
  template <typename E, int D>
  hipError_t go() const { return fwd_e_d<E, D>(p, heads, s); }
};

struct BwdCall {
  const GParams& p;
  int heads, stages;
  hipStream_t s;
  template <typename E, int D>
  hipError_t go() const { return bwd_e_d<E, D>(p, heads, stages, s); }
};

template <typename E, typename F>
hipError_t by_d(int d, const F& f) {
  switch (d) {
    case 32: return f.template go<E, 32>();
    case 64: return f.template go<E, 64>();
    case 96: return f.template go<E, 96>();
    case 128: return f.template go<E, 128>();
    case 256: return f.template go<E, 256>();
  }
  return hipErrorInvalidValue;
}

// f.go<E, D>() for the element type `elem` (0 fp32, 1 bf16, 2 fp16) and head size d.
template <typename F>
hipError_t by_type(int elem, int d, const F& f) {
  if (elem == 0) return by_d<float>(d, f);
  if (elem == 2) return by_d<f16>(d, f);
  return by_d<bf16>(d, f);
}

}  // namespace

bool generic_head_size(int d) { return d == 32 || d == 64 || d == 96 || d == 128 || d == 256; }

hipError_t launch_fwd_generic(const FwdArgs& a, int elem, hipStream_t s) {
  GParams p = base_params(a.H, a.N, a.scale, a.causal, a.key_lens, a.dropout_p, a.drop_threshold,
                          a.drop_scale, a.seed);
  p.b0 = a.b0;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.o = a.o;
  p.lse = a.lse;
  p.sq = a.sq;
  p.sk = a.sk;
  p.sv = a.sv;
  p.so = a.so;
  const int heads = a.B * a.H;
  return by_type(elem, a.d, FwdCall{p, heads, s});
}

hipError_t launch_bwd_generic(const BwdArgs& a, int elem, int stages, hipStream_t s) {
  GParams p = base_params(a.H, a.N, a.scale, a.causal, a.key_lens, a.dropout_p, a.drop_threshold,
                          a.drop_scale, a.seed);
  p.b0 = a.b0;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.o = a.o;
  p.dout = a.dout;
  p.lse_in = a.lse;
  p.dq = a.dq;
  p.dk = a.dk;
  p.dv = a.dv;
  p.delta = a.delta;
  p.lse2 = a.lse2;
  p.sq = a.sq;
  p.sk = a.sk;
  p.sv = a.sv;
  p.so = a.so;
  p.sdo = a.sdo;
  p.sdq = a.sdq;
  p.sdk = a.sdk;
  p.sdv = a.sdv;
  const int heads = a.B * a.H;
  return by_type(elem, a.d, BwdCall{p, heads, stages, s});
}

}  // namespace fa
