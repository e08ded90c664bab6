// Forward pass of exact attention on gfx950.
//
// O = softmax(mask(scale * Q K^T)) (with dropout) V and the per-row
// LSE = m + ln(l), computed tile by tile: each workgroup keeps a block of
// queries resident, streams K/V tiles through LDS, and keeps a running row max
// m and row sum l, rescaling the partial output whenever m grows (ML Canon 48
// FlashAttention, "tiling and online softmax").  The N x N scores exist only as
// one register tile at a time (FlashAttention first principles, section 4.2, explains
// why the row-wise softmax otherwise forces them into device memory).
//
// bf16 path.  Each wave owns 32 queries and computes the transposed score tile
// S^T = K Q^T with v_mfma_f32_32x32x16_bf16, so every lane holds the scores of
// ONE query against 16 keys of each 32-key block (its partner lane l^32 holds
// the other 16).  That orientation makes
//   * the row max/sum a per-lane reduction plus one permlane32 swap,
//   * the rescale factor a per-lane scalar for the transposed output O^T,
//   * the probabilities, converted to bf16, exactly the B operand of the next
//     MFMA O^T += V^T P^T with no data movement,
// while V^T is read from the row-major V tile with the LDS transposing read.
#include "fa_common.hpp"
#include "fa_internal.hpp"

namespace fa {
namespace {

struct FwdParams {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  bf16* o;
  float* lse;
  const int32_t* key_lens;
  int H, N, num_qblocks;
  float scale_log2;  // scale * log2(e): scores enter exp2 in these units
  uint32_t drop_threshold;
  float drop_scale;
  uint32_t seed_lo, seed_hi;
};

template <int D>
struct FwdCfg {
  static constexpr int NW = 8;                    // waves per workgroup
  static constexpr int THREADS = NW * 64;
  static constexpr int BM = 32 * NW;              // queries per workgroup
  static constexpr int BN = 64;                   // keys per K/V tile
  static constexpr int KP = D + 8;                // K tile row pitch (elements)
  static constexpr int VP = D + 32;               // V tile row pitch (elements)
  static constexpr int K_ELEMS = BN * KP;
  static constexpr int STAGE = BN * KP + BN * VP;  // one K tile + one V tile
  static constexpr int ROW_CHUNKS = D / 8;        // 16-byte chunks per row
  static constexpr int CPT = BN * ROW_CHUNKS / THREADS;  // chunks per thread per tile
  static_assert(CPT >= 1 && CPT * THREADS == BN * ROW_CHUNKS, "tile/thread mismatch");
};

template <int D, bool CAUSAL, bool DROPOUT>
__global__ __launch_bounds__(FwdCfg<D>::THREADS, 1) void fwd_bf16_kernel(FwdParams p) {
  using C = FwdCfg<D>;
  constexpr int BN = C::BN, KP = C::KP, VP = C::VP;
  __shared__ __attribute__((aligned(16))) bf16 smem[2 * C::STAGE];

  const int N = p.N;
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int head = lid / p.num_qblocks;                            // b * H + h
  const int qb = p.num_qblocks - 1 - (lid - head * p.num_qblocks);  // costliest blocks first
  const int bi = head / p.H, hi = head - bi * p.H;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int li = lane & 31, hh = lane >> 5;
  const int q0 = qb * C::BM;
  const int qw = q0 + wave * 32;  // first query of this wave
  const int qi = qw + li;         // this lane's query

  int L = N;
  if (p.key_lens) L = min(max(p.key_lens[bi], 0), N);
  const int kend = CAUSAL ? min(L, q0 + C::BM) : L;  // keys [0, kend) matter to the workgroup
  const int nkb = (kend + BN - 1) / BN;

  const size_t head_off = (size_t)head * N * D;
  const bf16* __restrict__ qg = p.q + head_off;
  const bf16* __restrict__ kg = p.k + head_off;
  const bf16* __restrict__ vg = p.v + head_off;

  // Q^T as the B operand of S^T = K Q^T: lane holds Q[qi][16c + 8hh .. +7].
  bf16x8 qreg[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    if (qi < N) {
      qreg[c] = *(const bf16x8*)(qg + (size_t)qi * D + 16 * c + 8 * hh);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) qreg[c][e] = (bf16)0.0f;
    }
  }

  f32x16 oacc[D / 32];
#pragma unroll
  for (int u = 0; u < D / 32; ++u)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[u][r] = 0.0f;
  float m = -INFINITY;  // running max of raw scores (q.k) for query qi
  float l = 0.0f;       // this lane's partial row sum (its 16 keys of every 32)

  const float c2 = p.scale_log2;

  // Global -> register staging of one K/V tile; rows past N read as zero.
  uint4 kreg[C::CPT], vreg[C::CPT];
  auto load_tile = [&](int jb) {
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int c = tid + i * C::THREADS;
      const int row = jb * BN + c / C::ROW_CHUNKS;
      const int col = (c % C::ROW_CHUNKS) * 8;
      if (row < N) {
        kreg[i] = *(const uint4*)(kg + (size_t)row * D + col);
        vreg[i] = *(const uint4*)(vg + (size_t)row * D + col);
      } else {
        kreg[i] = make_uint4(0, 0, 0, 0);
        vreg[i] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_tile = [&](int stage) {
    bf16* ks = smem + stage * C::STAGE;
    bf16* vs = ks + C::K_ELEMS;
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int c = tid + i * C::THREADS;
      const int row = c / C::ROW_CHUNKS;
      const int col = (c % C::ROW_CHUNKS) * 8;
      *(uint4*)(ks + row * KP + col) = kreg[i];
      *(uint4*)(vs + row * VP + col) = vreg[i];
    }
  };

  if (nkb > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int jb = 0; jb < nkb; ++jb) {
    const int cur = jb & 1;
    if (jb + 1 < nkb) load_tile(jb + 1);
    const int kb = jb * BN;
    const bool active = (!CAUSAL || kb <= qw + 31) && qw < N;
    if (active) {
      const bf16* ks = smem + cur * C::STAGE;
      const bf16* vs = ks + C::K_ELEMS;

      // S^T tile (64 keys x 32 queries) as two 32x32 MFMA tiles.
      f32x16 s[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[t][r] = 0.0f;
#pragma unroll
        for (int c = 0; c < D / 16; ++c) {
          const bf16x8 a = *(const bf16x8*)(ks + (32 * t + li) * KP + 16 * c + 8 * hh);
          s[t] = mfma32(a, qreg[c], s[t]);
        }
      }

      // Mask: padding / tail keys and, for causal, keys after the query.
      const bool need_mask = (kb + BN > L) || (CAUSAL && kb + BN - 1 > qw);
      if (need_mask) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kb + 32 * t + 8 * (r >> 2) + 4 * hh + (r & 3);
            const bool ok = key < L && (!CAUSAL || key <= qi);
            s[t][r] = ok ? s[t][r] : -INFINITY;
          }
      }

      // Online softmax update.
      float mx = s[0][0];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[t][r]);
      mx = pair_max(mx);
      const float m_new = fmaxf(m, mx);
      const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
      const float ms = m_use * c2;
      const float alpha = fast_exp2(m * c2 - ms);  // 0 while nothing was seen yet
      m = m_new;
      float psum = 0.0f;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = fast_exp2(fmaf(s[t][r], c2, -ms));
          s[t][r] = e;
          psum += e;
        }
      l = fmaf(l, alpha, psum);

      if constexpr (DROPOUT) {
        // One Philox call per 4 consecutive keys of this query row.
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const uint32_t key4 = (uint32_t)(kb + 32 * t + 8 * g + 4 * hh);
            const u32x4 w = philox(key4 >> 2, (uint32_t)qi, (uint32_t)hi, (uint32_t)bi,
                                   p.seed_lo, p.seed_hi);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              s[t][4 * g + e] = (w[e] >= p.drop_threshold) ? s[t][4 * g + e] * p.drop_scale : 0.0f;
          }
      }

      // P^T in bf16: chunk cc covers keys 16cc .. 16cc+15 (k-slots match V^T below).
      bf16x8 pb[4];
#pragma unroll
      for (int cc = 0; cc < 4; ++cc)
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[cc][e] = (bf16)s[cc >> 1][8 * (cc & 1) + e];

#pragma unroll
      for (int u = 0; u < D / 32; ++u)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[u][r] *= alpha;

      // O^T += V^T P^T.  The A operand needs V[key][dcol] for dcol = 32u + li and
      // keys 16cc + 4hh + {0..3} (slots 0-3) and 16cc + 8 + 4hh + {0..3} (slots 4-7):
      // two transposing reads of 4 x 16 blocks of the row-major V tile.
      const int g16 = lane & 15;
      const int trow = 4 * hh + (g16 >> 2);
      const int tcol = 16 * ((lane >> 4) & 1) + 4 * (g16 & 3);
#pragma unroll
      for (int u = 0; u < D / 32; ++u)
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
          const bf16* vp = vs + (16 * cc + trow) * VP + 32 * u + tcol;
          const bf16x4 lo = lds_read_tr4(vp);
          const bf16x4 hi4 = lds_read_tr4(vp + 8 * VP);
          const bf16x8 a = {lo[0], lo[1], lo[2], lo[3], hi4[0], hi4[1], hi4[2], hi4[3]};
          oacc[u] = mfma32(a, pb[cc], oacc[u]);
        }
    }
    if (jb + 1 < nkb) store_tile(cur ^ 1);
    __syncthreads();
  }

  // Epilogue: O = O^T / l, LSE = scale*m + ln(l).
  const float lt = pair_sum(l);
  if (qi < N) {
    const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
    bf16* orow = p.o + head_off + (size_t)qi * D;
#pragma unroll
    for (int u = 0; u < D / 32; ++u)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 ov;
#pragma unroll
        for (int e = 0; e < 4; ++e) ov[e] = (bf16)(oacc[u][4 * g + e] * inv);
        *(bf16x4*)(orow + 32 * u + 8 * g + 4 * hh) = ov;
      }
    if (hh == 0) {
      p.lse[(size_t)head * N + qi] = lt > 0.0f ? (m * c2 + __log2f(lt)) * kLn2 : -INFINITY;
    }
  }
}

// fp32 path: one thread per query row, K/V tiles of 64 keys staged in LDS and
// read as broadcasts; online softmax over each tile in fp32 registers.
template <int D>
__global__ __launch_bounds__(64) void fwd_f32_kernel(const float* __restrict__ q,
                                                     const float* __restrict__ k,
                                                     const float* __restrict__ v,
                                                     float* __restrict__ o, float* __restrict__ lse,
                                                     const int32_t* key_lens, int H, int N,
                                                     int causal, float scale_log2) {
  constexpr int BN = 64;
  __shared__ float ks[BN][D];
  __shared__ float vs[BN][D];
  const int nqb = (N + 63) / 64;
  const int head = blockIdx.x / nqb;
  const int qb = blockIdx.x - head * nqb;
  const int bi = head / H;
  const int qi = qb * 64 + threadIdx.x;
  int L = N;
  if (key_lens) L = min(max(key_lens[bi], 0), N);
  const int kend = causal ? min(L, qb * 64 + 64) : L;
  const size_t off = (size_t)head * N * D;

  float qr[D], acc[D];
#pragma unroll
  for (int c = 0; c < D; ++c) {
    qr[c] = qi < N ? q[off + (size_t)qi * D + c] : 0.0f;
    acc[c] = 0.0f;
  }
  float m = -INFINITY, l = 0.0f;
  for (int kb = 0; kb < kend; kb += BN) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < BN * D; idx += 64) {
      const int row = kb + idx / D;
      ks[idx / D][idx % D] = row < N ? k[off + (size_t)row * D + idx % D] : 0.0f;
      vs[idx / D][idx % D] = row < N ? v[off + (size_t)row * D + idx % D] : 0.0f;
    }
    __syncthreads();
    float s[BN];
    float mx = -INFINITY;
    for (int j = 0; j < BN; ++j) {
      float dot = 0.0f;
#pragma unroll
      for (int c = 0; c < D; ++c) dot = fmaf(qr[c], ks[j][c], dot);
      const int key = kb + j;
      const bool ok = key < L && (!causal || key <= qi);
      s[j] = ok ? dot : -INFINITY;
      mx = fmaxf(mx, s[j]);
    }
    const float m_new = fmaxf(m, mx);
    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = exp2f((m - m_use) * scale_log2);
    m = m_new;
    l *= alpha;
#pragma unroll
    for (int c = 0; c < D; ++c) acc[c] *= alpha;
    for (int j = 0; j < BN; ++j) {
      const float e = exp2f((s[j] - m_use) * scale_log2);
      l += e;
#pragma unroll
      for (int c = 0; c < D; ++c) acc[c] = fmaf(e, vs[j][c], acc[c]);
    }
  }
  if (qi < N) {
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
    for (int c = 0; c < D; ++c) o[off + (size_t)qi * D + c] = acc[c] * inv;
    lse[(size_t)head * N + qi] = l > 0.0f ? (m * scale_log2 + log2f(l)) * kLn2 : -INFINITY;
  }
}

template <int D, bool CAUSAL, bool DROPOUT>
hipError_t launch_bf16(const FwdParams& p, int heads, hipStream_t s) {
  using C = FwdCfg<D>;
  const int grid = heads * p.num_qblocks;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, DROPOUT>), dim3(grid), dim3(C::THREADS), 0, s, p);
  return hipGetLastError();
}

template <int D>
hipError_t dispatch_bf16(const FwdParams& p, int heads, bool causal, bool dropout, hipStream_t s) {
  if (causal) {
    return dropout ? launch_bf16<D, true, true>(p, heads, s) : launch_bf16<D, true, false>(p, heads, s);
  }
  return dropout ? launch_bf16<D, false, true>(p, heads, s) : launch_bf16<D, false, false>(p, heads, s);
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t s) {
  FwdParams p;
  p.q = (const bf16*)a.q;
  p.k = (const bf16*)a.k;
  p.v = (const bf16*)a.v;
  p.o = (bf16*)a.o;
  p.lse = a.lse;
  p.key_lens = a.key_lens;
  p.H = a.H;
  p.N = a.N;
  p.scale_log2 = a.scale * kLog2e;
  p.drop_threshold = a.drop_threshold;
  p.drop_scale = a.drop_scale;
  p.seed_lo = (uint32_t)(a.seed & 0xffffffffu);
  p.seed_hi = (uint32_t)(a.seed >> 32);
  const bool dropout = a.dropout_p > 0.0f;
  const int heads = a.B * a.H;
  if (a.d == 64) {
    p.num_qblocks = (a.N + FwdCfg<64>::BM - 1) / FwdCfg<64>::BM;
    return dispatch_bf16<64>(p, heads, a.causal != 0, dropout, s);
  }
  p.num_qblocks = (a.N + FwdCfg<128>::BM - 1) / FwdCfg<128>::BM;
  return dispatch_bf16<128>(p, heads, a.causal != 0, dropout, s);
}

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t s) {
  const int grid = a.B * a.H * ((a.N + 63) / 64);
  const float sl = a.scale * kLog2e;
  if (a.d == 64) {
    hipLaunchKernelGGL(fwd_f32_kernel<64>, dim3(grid), dim3(64), 0, s, (const float*)a.q,
                       (const float*)a.k, (const float*)a.v, (float*)a.o, a.lse, a.key_lens, a.H,
                       a.N, a.causal, sl);
  } else {
    hipLaunchKernelGGL(fwd_f32_kernel<128>, dim3(grid), dim3(64), 0, s, (const float*)a.q,
                       (const float*)a.k, (const float*)a.v, (float*)a.o, a.lse, a.key_lens, a.H,
                       a.N, a.causal, sl);
  }
  return hipGetLastError();
}

}  // namespace fa
