// Backward pass of exact attention on gfx950 (recomputation instead of a
// stored probability matrix: ML Canon 48 FlashAttention, "backward without
// N x N"; Flash Attention hardware-aware optimisation, section 2.2, keep only the softmax
// normalisation statistics and rebuild the weights blockwise).
//
// Three kernels on one stream:
//  1. bwd_pre:  D_i = sum_k dO_ik O_ik (fp32) and a zeroed fp32 dQ accumulator.
//  2. bwd_main: one workgroup per 128-key block of one head; every wave owns 32
//     keys and keeps their dK^T and dV^T in fp32 registers while the workgroup
//     walks the 64-row query tiles that can see the block.  Per tile:
//        S  = Q K^T, P = exp(scale*S - LSE)        (recomputed, masked)
//        dP = dO V^T,  dS = P * (dP*Z - D)          (Z = dropout keep/(1-p))
//        dV^T += dO^T (P*Z),  dK^T += Q^T dS
//        dQ  += dS K   (fp32 atomics; dS goes through LDS, transposed)
//     S and dP come out of the MFMA with a lane per key and 16 query rows per
//     lane, which is exactly the B-operand layout of the dV^T and dK^T products;
//     the A operands dO^T and Q^T, and both operands of dQ, come from row-major
//     LDS tiles through the transposing LDS read.
//  3. bwd_convert: dQ = scale * accumulator, rounded to bf16.
#include "fa_common.hpp"
#include "fa_internal.hpp"

namespace fa {
namespace {

struct BwdParams {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const bf16* dout;
  const float* lse;
  const float* delta;
  float* dq_acc;
  bf16* dk;
  bf16* dv;
  const int32_t* key_lens;
  int H, N, num_kblocks;
  float scale, scale_log2;
  uint32_t drop_threshold;
  float drop_scale;
  uint32_t seed_lo, seed_hi;
};

template <int D>
struct BwdCfg {
  static constexpr int NW = 4;
  static constexpr int THREADS = 64 * NW;
  static constexpr int BK = 32 * NW;  // keys per workgroup
  static constexpr int BQ = 64;       // query rows per tile
  static constexpr int KP = D + 32;   // pitch of the K block in LDS (elements)
  static constexpr int QP = D + 16;   // pitch of the Q and dO tiles
  static constexpr int SP = BQ + 8;   // pitch of dS^T (rows are keys)
  static constexpr int ROW_CHUNKS = D / 8;
  static constexpr int CPT = BQ * ROW_CHUNKS / THREADS;  // 16-byte chunks per thread per tile
  static constexpr int QTILE = BQ * QP;
  static constexpr int DQ_TILES = 2 * (D / 32) / NW;     // 32x32 dQ tiles per wave per step
  static_assert(CPT * THREADS == BQ * ROW_CHUNKS, "tile/thread mismatch");
  static_assert(DQ_TILES >= 1 && DQ_TILES * NW == 2 * (D / 32), "dQ tiles must split evenly");
};

template <int D, bool CAUSAL, bool DROPOUT>
__global__ __launch_bounds__(BwdCfg<D>::THREADS, 1) void bwd_main_kernel(BwdParams p) {
  using C = BwdCfg<D>;
  constexpr int BQ = C::BQ, KP = C::KP, QP = C::QP, SP = C::SP;
  __shared__ __attribute__((aligned(16))) bf16 k_lds[C::BK * KP];
  __shared__ __attribute__((aligned(16))) bf16 qd_lds[2][2][C::QTILE];  // [stage][Q, dO]
  __shared__ __attribute__((aligned(16))) float rl_lds[2][2][BQ];       // [stage][LSE*log2e, D]
  __shared__ __attribute__((aligned(16))) bf16 ds_lds[C::BK * SP];      // dS^T [key][row]

  const int N = p.N;
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int head = lid / p.num_kblocks;
  const int jb = lid - head * p.num_kblocks;  // low key blocks see the most rows: run first
  const int bi = head / p.H, hi = head - bi * p.H;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int li = lane & 31, hh = lane >> 5;
  const int kb = jb * C::BK;          // first key of the workgroup
  const int kw = kb + 32 * wave;      // first key of this wave
  const int key = kw + li;            // this lane's key (column of S)

  int L = N;
  if (p.key_lens) L = min(max(p.key_lens[bi], 0), N);

  const size_t head_off = (size_t)head * N * D;
  const bf16* __restrict__ qg = p.q + head_off;
  const bf16* __restrict__ kg = p.k + head_off;
  const bf16* __restrict__ vg = p.v + head_off;
  const bf16* __restrict__ dog = p.dout + head_off;
  const float* __restrict__ lseg = p.lse + (size_t)head * N;
  const float* __restrict__ dlg = p.delta + (size_t)head * N;
  float* __restrict__ dqg = p.dq_acc + head_off;

  // The epilogue layout: dV^T/dK^T tile u, register r -> dcol 32u + 8(r/4) + 4hh + r%4.
  auto store_dkdv = [&](const f32x16* dkacc, const f32x16* dvacc) {
    if (key >= N) return;
    bf16* dkrow = p.dk + head_off + (size_t)key * D;
    bf16* dvrow = p.dv + head_off + (size_t)key * D;
#pragma unroll
    for (int u = 0; u < D / 32; ++u)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 kv, vv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kv[e] = (bf16)(dkacc[u][4 * g + e] * p.scale);
          vv[e] = (bf16)dvacc[u][4 * g + e];
        }
        *(bf16x4*)(dkrow + 32 * u + 8 * g + 4 * hh) = kv;
        *(bf16x4*)(dvrow + 32 * u + 8 * g + 4 * hh) = vv;
      }
  };

  f32x16 dkacc[D / 32], dvacc[D / 32];
#pragma unroll
  for (int u = 0; u < D / 32; ++u)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dkacc[u][r] = 0.0f;
      dvacc[u][r] = 0.0f;
    }

  if (kb >= L) {  // every key of the block is padding: zero gradients
    store_dkdv(dkacc, dvacc);
    return;
  }

  // K block into LDS (for dQ = dS K), rows past N as zero.
  for (int c = tid; c < C::BK * C::ROW_CHUNKS; c += C::THREADS) {
    const int row = c / C::ROW_CHUNKS, col = (c % C::ROW_CHUNKS) * 8;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (kb + row < N) val = *(const uint4*)(kg + (size_t)(kb + row) * D + col);
    *(uint4*)(k_lds + row * KP + col) = val;
  }
  // K and V rows of this lane's key as B operands (k = head dimension).
  bf16x8 kreg[D / 16], vreg[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    if (key < N) {
      kreg[c] = *(const bf16x8*)(kg + (size_t)key * D + 16 * c + 8 * hh);
      vreg[c] = *(const bf16x8*)(vg + (size_t)key * D + 16 * c + 8 * hh);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        kreg[c][e] = (bf16)0.0f;
        vreg[c][e] = (bf16)0.0f;
      }
    }
  }

  const int it0 = CAUSAL ? kb / BQ : 0;
  const int nit = (N + BQ - 1) / BQ;

  uint4 qst[C::CPT], dost[C::CPT];
  float lse_st = 0.0f, d_st = 0.0f;
  auto load_tile = [&](int it) {
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int c = tid + i * C::THREADS;
      const int row = it * BQ + c / C::ROW_CHUNKS, col = (c % C::ROW_CHUNKS) * 8;
      if (row < N) {
        qst[i] = *(const uint4*)(qg + (size_t)row * D + col);
        dost[i] = *(const uint4*)(dog + (size_t)row * D + col);
      } else {
        qst[i] = make_uint4(0, 0, 0, 0);
        dost[i] = make_uint4(0, 0, 0, 0);
      }
    }
    if (tid < BQ) {
      const int row = it * BQ + tid;
      // Rows past N, or without any allowed key, must give P = 0: exp2(s - inf).
      float l2 = INFINITY, dd = 0.0f;
      if (row < N) {
        const float lv = lseg[row];
        l2 = lv == -INFINITY ? INFINITY : lv * kLog2e;
        dd = dlg[row];
      }
      lse_st = l2;
      d_st = dd;
    }
  };
  auto store_tile = [&](int st) {
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int c = tid + i * C::THREADS;
      const int row = c / C::ROW_CHUNKS, col = (c % C::ROW_CHUNKS) * 8;
      *(uint4*)(&qd_lds[st][0][row * QP + col]) = qst[i];
      *(uint4*)(&qd_lds[st][1][row * QP + col]) = dost[i];
    }
    if (tid < BQ) {
      rl_lds[st][0][tid] = lse_st;
      rl_lds[st][1][tid] = d_st;
    }
  };

  load_tile(it0);
  store_tile(0);
  __syncthreads();

  const float c2 = p.scale_log2;
  const int g16 = lane & 15;
  const int trow = 4 * hh + (g16 >> 2);                       // transposing-read row in a 16-row chunk
  const int tcol = 16 * ((lane >> 4) & 1) + 4 * (g16 & 3);    // and column within a 32-column block

  for (int it = it0; it < nit; ++it) {
    const int cur = (it - it0) & 1;
    if (it + 1 < nit) load_tile(it + 1);
    const int r0 = it * BQ;
    const bf16* qs = qd_lds[cur][0];
    const bf16* dos = qd_lds[cur][1];
    const float* ls = rl_lds[cur][0];
    const float* dls = rl_lds[cur][1];

    const bool active = kw < L && (!CAUSAL || kw <= r0 + BQ - 1);
    if (active) {
      f32x16 sacc[2], pacc[2];
#pragma unroll
      for (int a = 0; a < 2; ++a) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sacc[a][r] = 0.0f;
          pacc[a][r] = 0.0f;
        }
#pragma unroll
        for (int c = 0; c < D / 16; ++c) {
          const bf16x8 qa = *(const bf16x8*)(qs + (32 * a + li) * QP + 16 * c + 8 * hh);
          sacc[a] = mfma32(qa, kreg[c], sacc[a]);
          const bf16x8 da = *(const bf16x8*)(dos + (32 * a + li) * QP + 16 * c + 8 * hh);
          pacc[a] = mfma32(da, vreg[c], pacc[a]);
        }
      }

      const bool need_mask = (kw + 31 >= L) || (CAUSAL && kw + 31 > r0);
      bf16x8 pb[4], dsb[4];
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int il = 32 * a + 8 * g + 4 * hh;  // first of 4 consecutive rows
          const f32x4 l4 = *(const f32x4*)(ls + il);
          const f32x4 d4 = *(const f32x4*)(dls + il);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * g + e;
            float pv = fast_exp2(fmaf(sacc[a][r], c2, -l4[e]));
            if (need_mask) {
              const int row = r0 + il + e;
              const bool ok = key < L && (!CAUSAL || key <= row);
              pv = ok ? pv : 0.0f;
            }
            float pt = pv, dp = pacc[a][r];
            if constexpr (DROPOUT) {
              const int row = r0 + il + e;
              const u32x4 w = philox((uint32_t)key >> 2, (uint32_t)row, (uint32_t)hi, (uint32_t)bi,
                                     p.seed_lo, p.seed_hi);
              const uint32_t word = (key & 3) == 0 ? w[0] : (key & 3) == 1 ? w[1] : (key & 3) == 2 ? w[2] : w[3];
              const float z = word >= p.drop_threshold ? p.drop_scale : 0.0f;
              pt = pv * z;
              dp = dp * z;
            }
            const float ds = pv * (dp - d4[e]);
            pb[2 * a + (g >> 1)][4 * (g & 1) + e] = (bf16)pt;
            dsb[2 * a + (g >> 1)][4 * (g & 1) + e] = (bf16)ds;
          }
        }

      // dV^T += dO^T P~ and dK^T += Q^T dS (contraction over the 64 rows).
#pragma unroll
      for (int u = 0; u < D / 32; ++u)
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
          const bf16* dp_ = dos + (16 * kc + trow) * QP + 32 * u + tcol;
          const bf16x4 a0 = lds_read_tr4(dp_), a1 = lds_read_tr4(dp_ + 8 * QP);
          const bf16x8 ad = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
          dvacc[u] = mfma32(ad, pb[kc], dvacc[u]);
          const bf16* qp_ = qs + (16 * kc + trow) * QP + 32 * u + tcol;
          const bf16x4 b0 = lds_read_tr4(qp_), b1 = lds_read_tr4(qp_ + 8 * QP);
          const bf16x8 aq = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
          dkacc[u] = mfma32(aq, dsb[kc], dkacc[u]);
        }

      // dS^T rows of this wave's keys: 4 consecutive query rows per 8-byte write.
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const bf16x8& src = dsb[2 * a + (g >> 1)];
          const int o4 = 4 * (g & 1);
          const bf16x4 w4 = {src[o4], src[o4 + 1], src[o4 + 2], src[o4 + 3]};
          *(bf16x4*)(ds_lds + (32 * wave + li) * SP + 32 * a + 8 * g + 4 * hh) = w4;
        }
    } else {
      const bf16x4 z4 = {(bf16)0.0f, (bf16)0.0f, (bf16)0.0f, (bf16)0.0f};
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *(bf16x4*)(ds_lds + (32 * wave + li) * SP + 32 * a + 8 * g + 4 * hh) = z4;
    }
    __syncthreads();

    // dQ tile (rows of the query tile x 32 head dims) += dS K over the 128 keys.
#pragma unroll
    for (int t = 0; t < C::DQ_TILES; ++t) {
      const int id = wave * C::DQ_TILES + t;
      const int a = id / (D / 32), u = id % (D / 32);
      f32x16 acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
#pragma unroll
      for (int kc = 0; kc < C::BK / 16; ++kc) {
        const bf16* sp_ = ds_lds + (16 * kc + trow) * SP + 32 * a + tcol;
        const bf16x4 s0 = lds_read_tr4(sp_), s1 = lds_read_tr4(sp_ + 8 * SP);
        const bf16x8 as = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
        const bf16* kp_ = k_lds + (16 * kc + trow) * KP + 32 * u + tcol;
        const bf16x4 k0 = lds_read_tr4(kp_), k1 = lds_read_tr4(kp_ + 8 * KP);
        const bf16x8 bk = {k0[0], k0[1], k0[2], k0[3], k1[0], k1[1], k1[2], k1[3]};
        acc = mfma32(as, bk, acc);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = r0 + 32 * a + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (row < N) unsafeAtomicAdd(dqg + (size_t)row * D + 32 * u + li, acc[r]);
      }
    }

    if (it + 1 < nit) store_tile(cur ^ 1);
    __syncthreads();
  }

  store_dkdv(dkacc, dvacc);
}

// D_i = sum_k dO_ik O_ik; also clears the dQ accumulator.  D/8 lanes per row.
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const bf16* __restrict__ o,
                                                      const bf16* __restrict__ dout,
                                                      float* __restrict__ delta,
                                                      float* __restrict__ dq_acc, int64_t rows) {
  constexpr int LPR = D / 8;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = t / LPR;
  const int ch = (int)(t % LPR);
  float s = 0.0f;
  if (row < rows) {
    const bf16x8 ov = *(const bf16x8*)(o + row * D + ch * 8);
    const bf16x8 dv = *(const bf16x8*)(dout + row * D + ch * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) s = fmaf((float)ov[e], (float)dv[e], s);
    float4* z = (float4*)(dq_acc + row * D + ch * 8);
    z[0] = make_float4(0.f, 0.f, 0.f, 0.f);
    z[1] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, LPR);
  if (row < rows && ch == 0) delta[row] = s;
}

// dQ = scale * accumulator, rounded to bf16; 8 elements per thread.
__global__ __launch_bounds__(256) void bwd_convert_kernel(const float* __restrict__ acc,
                                                          bf16* __restrict__ dq, float scale,
                                                          int64_t n8) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= n8) return;
  const float4 a = ((const float4*)acc)[2 * t];
  const float4 b = ((const float4*)acc)[2 * t + 1];
  const bf16x8 r = {(bf16)(a.x * scale), (bf16)(a.y * scale), (bf16)(a.z * scale), (bf16)(a.w * scale),
                    (bf16)(b.x * scale), (bf16)(b.y * scale), (bf16)(b.z * scale), (bf16)(b.w * scale)};
  ((bf16x8*)dq)[t] = r;
}

template <int D, bool CAUSAL, bool DROPOUT>
hipError_t launch_main(const BwdParams& p, int heads, hipStream_t s) {
  hipLaunchKernelGGL((bwd_main_kernel<D, CAUSAL, DROPOUT>), dim3(heads * p.num_kblocks),
                     dim3(BwdCfg<D>::THREADS), 0, s, p);
  return hipGetLastError();
}

template <int D>
hipError_t run(const BwdArgs& a, BwdParams& p, hipStream_t s) {
  const int64_t rows = (int64_t)a.B * a.H * a.N;
  const int64_t pre_threads = rows * (D / 8);
  hipLaunchKernelGGL(bwd_pre_kernel<D>, dim3((unsigned)((pre_threads + 255) / 256)), dim3(256), 0, s,
                     (const bf16*)a.o, (const bf16*)a.dout, a.delta, a.dq_acc, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  p.num_kblocks = (a.N + BwdCfg<D>::BK - 1) / BwdCfg<D>::BK;
  const int heads = a.B * a.H;
  const bool drop = a.dropout_p > 0.0f;
  if (a.causal) {
    e = drop ? launch_main<D, true, true>(p, heads, s) : launch_main<D, true, false>(p, heads, s);
  } else {
    e = drop ? launch_main<D, false, true>(p, heads, s) : launch_main<D, false, false>(p, heads, s);
  }
  if (e != hipSuccess) return e;
  const int64_t n8 = rows * D / 8;
  hipLaunchKernelGGL(bwd_convert_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s,
                     (const float*)a.dq_acc, (bf16*)a.dq, a.scale, n8);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t s) {
  BwdParams p;
  p.q = (const bf16*)a.q;
  p.k = (const bf16*)a.k;
  p.v = (const bf16*)a.v;
  p.dout = (const bf16*)a.dout;
  p.lse = a.lse;
  p.delta = a.delta;
  p.dq_acc = a.dq_acc;
  p.dk = (bf16*)a.dk;
  p.dv = (bf16*)a.dv;
  p.key_lens = a.key_lens;
  p.H = a.H;
  p.N = a.N;
  p.scale = a.scale;
  p.scale_log2 = a.scale * kLog2e;
  p.drop_threshold = a.drop_threshold;
  p.drop_scale = a.drop_scale;
  p.seed_lo = (uint32_t)(a.seed & 0xffffffffu);
  p.seed_hi = (uint32_t)(a.seed >> 32);
  return a.d == 64 ? run<64>(a, p, s) : run<128>(a, p, s);
}

}  // namespace fa
