// Backward pass of exact attention on gfx950 (recomputation instead of a
// stored probability matrix: ML Canon 48 FlashAttention, "backward without
// N x N"; Flash Attention hardware-aware optimisation, section 2.2, keep only the softmax
// normalisation statistics and rebuild the weights blockwise).
//
// Three kernels on one stream:
//  1. bwd_pre:  D_i = sum_k dO_ik O_ik and LSE_i * log2(e) (fp32), and a zeroed
//     fp32 dQ accumulator.
//  2. bwd_main: one workgroup of 4 waves per 128-key block of one head; each
//     wave owns 32 keys and keeps K and V of its keys (B operands), the K
//     slice the dQ product needs, and fp32 dK^T / dV^T accumulators in
//     registers, while the workgroup walks the 64-row query tiles that can see
//     the block.  Per tile:
//        S  = Q K^T, P = exp2(S * scale*log2e - LSE_i*log2e)   (recomputed)
//        dP = dO V^T, dS = P * (dP * Z - D_i)    (Z = dropout keep / (1 - p))
//        dV^T += dO^T (P*Z), dK^T += Q^T dS
//        dQ += dS K  (dS^T exchanged through LDS; fp32 atomics into the workspace)
//     S and dP come out of the MFMA with a lane per key and 16 query rows per
//     lane, which is the B-operand layout of the dV^T and dK^T products; their
//     A operands dO^T and Q^T are transposing LDS reads of the row-major tiles.
//     Q and dO tiles (and the per-row LSE and D) are copied global -> LDS by
//     buffer loads into double-buffered, XOR-swizzled stages (conflict-free row
//     and transposing reads); a single barrier per tile both publishes the
//     dS^T exchange and hands over the next stage.
//  3. bwd_convert: dQ = scale * accumulator, rounded to bf16.
#include <type_traits>

#include "fa_common.hpp"
#include "fa_internal.hpp"

namespace fa {
namespace {

struct BwdParams {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const bf16* dout;
  const float* lse2;   // LSE * log2(e), +inf for rows without any allowed key
  const float* delta;  // D
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
  static constexpr int CHUNKS = D / 8;
  static constexpr int TILE = BQ * D;                  // elements of a Q or dO tile
  static constexpr int LOADS = BQ * CHUNKS / THREADS;  // 16-byte copies per thread per tile
  static constexpr int DQT = (D / 32) * (BQ / 32) / NW;  // 32x32 dQ tiles per wave
  static_assert(LOADS * THREADS == BQ * CHUNKS, "tile/thread mismatch");
  static_assert(DQT >= 1, "dQ tiles must cover the waves");
};

// 16-byte chunk swizzle of a row-major tile with D-element rows (see the
// forward pass): row reads of 16 consecutive rows and transposing reads of 4
// aligned rows x 64 bytes are both free of bank conflicts.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) {
    return ((r & 3) << 2) | ((r >> 2) & 3);
  } else {
    return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  }
}

template <int D, bool CAUSAL, bool DROPOUT>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void bwd_main_kernel(BwdParams p) {
  using C = BwdCfg<D>;
  constexpr int BQ = C::BQ, NW = C::NW, TILE = C::TILE, BK = C::BK;
  constexpr int KC = D / 16;  // k-steps of the S and dP products
  constexpr int DU = D / 32;  // 32-wide blocks of the head dimension
  constexpr int DST = BK * BQ;  // elements of the dS^T exchange buffer
  // Stages of the Q and dO tiles, per-row LSE*log2e and D, and the dS^T
  // exchange buffers.  Separate objects let the compiler see that a copy into
  // one stage cannot alias reads of the other.
  __shared__ __attribute__((aligned(1024))) bf16 sq0[TILE];
  __shared__ __attribute__((aligned(1024))) bf16 sq1[TILE];
  __shared__ __attribute__((aligned(1024))) bf16 so0[TILE];
  __shared__ __attribute__((aligned(1024))) bf16 so1[TILE];
  __shared__ __attribute__((aligned(256))) float sl0[BQ];
  __shared__ __attribute__((aligned(256))) float sl1[BQ];
  __shared__ __attribute__((aligned(256))) float sd0[BQ];
  __shared__ __attribute__((aligned(256))) float sd1[BQ];
  // dS^T [key][row] of the whole block, double buffered; before the loop the
  // pair holds the block's K rows (BK x D) for the dQ operand fragments.
  __shared__ __attribute__((aligned(1024))) bf16 sds[2 * DST];
  static_assert(BK * D <= 2 * DST, "K staging must fit the exchange buffers");

  const int N = p.N;
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int head = lid / p.num_kblocks;
  const int jb = lid - head * p.num_kblocks;  // low key blocks see the most rows: run first
  const int bi = head / p.H, hi = head - bi * p.H;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, hh = lane >> 5;
  const int kb = jb * BK;        // first key of the workgroup
  const int kw = kb + 32 * wave;  // first key of this wave
  const int key = kw + li;        // this lane's key (column of S)

  int L = N;
  if (p.key_lens) L = min(max(p.key_lens[bi], 0), N);

  const size_t head_off = (size_t)head * N * D;
  const bf16* __restrict__ kg = p.k + head_off;
  const bf16* __restrict__ vg = p.v + head_off;

  // Epilogue layout: dV^T / dK^T tile u, register r -> d = 32u + 8(r/4) + 4hh + r%4.
  f32x16 dkacc[DU], dvacc[DU];
#pragma unroll
  for (int u = 0; u < DU; ++u)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dkacc[u][r] = 0.0f;
      dvacc[u][r] = 0.0f;
    }
  auto store_dkdv = [&]() {
    if (key >= N) return;
    bf16* dkrow = p.dk + head_off + (size_t)key * D;
    bf16* dvrow = p.dv + head_off + (size_t)key * D;
#pragma unroll
    for (int u = 0; u < DU; ++u)
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
  if (kb >= L) {  // every key of the block is padding: zero gradients
    store_dkdv();
    return;
  }

  // ---- operands that stay in registers for the whole block
  // K and V rows of this lane's key as B operands (k = head dimension).
  bf16x8 kreg[KC], vreg[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) {
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
  // Transposing-read lane pattern (same as the forward's V^T reads): within a
  // 16-row chunk, rows trow and trow + 8; columns tcol .. tcol + 3 of a
  // 32-column block.  k-slot e of a lane <-> row 8(e/4) + 4hh + e%4 of the chunk.
  const int g16 = lane & 15;
  const int trow = 4 * hh + (g16 >> 2);
  const int tcol = 16 * ((lane >> 4) & 1) + 4 * (g16 & 3);

  // dQ tiles of this wave: (row tile dq_a[t], head-dim block dq_u[t]) for
  // t < DQT.  All of a wave's tiles share one head-dim block, so one K slice
  // serves them: d = 128 -> block = wave, both row tiles; d = 64 -> block =
  // wave % 2, row tile = wave / 2.
  int dq_a[C::DQT], dq_u[C::DQT];
#pragma unroll
  for (int t = 0; t < C::DQT; ++t) {
    dq_u[t] = wave % DU;
    dq_a[t] = t * (NW / DU) + wave / DU;
  }
  // K slice of the dQ product (B operand, k = key): stage the block's K rows
  // in LDS (swizzled like a tile) and read K^T fragments transposed.
  bf16x8 kfr[BK / 16];
  {
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(kg, (uint32_t)N * D * 2);
#pragma unroll
    for (int i = 0; i < BK * C::CHUNKS / C::THREADS; ++i) {
      const int pch = (i * NW + wave) * 64 + lane;
      const int r = pch / C::CHUNKS, pc = pch % C::CHUNKS;
      lds_dma16(krs, sds + (i * NW + wave) * 512,
                (uint32_t)((kb + r) * D + ((pc ^ swz<D>(r)) * 8)) * 2);
    }
    wait_vmem();
    __syncthreads();
    const lds_bf16* ks = to_lds(sds);
    const int u = dq_u[0];
#pragma unroll
    for (int ks16 = 0; ks16 < BK / 16; ++ks16) {
      bf16x4 lo, hi4;
      {
        const int r = 16 * ks16 + trow;
        lo = lds_read_tr4(ks + r * D + (((4 * u + (tcol >> 3)) ^ swz<D>(r)) * 8) + (tcol & 7));
      }
      {
        const int r = 16 * ks16 + trow + 8;
        hi4 = lds_read_tr4(ks + r * D + (((4 * u + (tcol >> 3)) ^ swz<D>(r)) * 8) + (tcol & 7));
      }
      kfr[ks16] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi4[0], hi4[1], hi4[2], hi4[3]};
    }
    __syncthreads();  // the staging area becomes the dS^T exchange buffers
  }

  // ---- per-tile copies: Q and dO tiles, LSE*log2e and D rows
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(p.q + head_off, (uint32_t)N * D * 2);
  const __amdgpu_buffer_rsrc_t ors = make_rsrc(p.dout + head_off, (uint32_t)N * D * 2);
  const __amdgpu_buffer_rsrc_t lrs = make_rsrc(p.lse2 + (size_t)head * N, (uint32_t)N * 4);
  const __amdgpu_buffer_rsrc_t drs = make_rsrc(p.delta + (size_t)head * N, (uint32_t)N * 4);
  uint32_t ld_off[C::LOADS];
#pragma unroll
  for (int i = 0; i < C::LOADS; ++i) {
    const int pch = (i * NW + wave) * 64 + lane;
    const int r = pch / C::CHUNKS, pc = pch % C::CHUNKS;
    ld_off[i] = (uint32_t)(r * D + ((pc ^ swz<D>(r)) * 8)) * 2;
  }
  auto issue_tile = [&](int it, auto par_t) {
    constexpr int S = decltype(par_t)::value;
    bf16* qd = S ? sq1 : sq0;
    bf16* od = S ? so1 : so0;
    const uint32_t base = (uint32_t)it * (BQ * D * 2);
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      lds_dma16(qrs, qd + (i * NW + wave) * 512, ld_off[i] + base);
      lds_dma16(ors, od + (i * NW + wave) * 512, ld_off[i] + base);
    }
    // 64 rows of 4 bytes: one wave-wide 4-byte copy each (rows past N read 0)
    if (wave == 0) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(lrs, (lds_void_t*)(S ? sl1 : sl0), 4,
                                               (uint32_t)(it * BQ + lane) * 4, 0, 0, 0);
    } else if (wave == 1) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(drs, (lds_void_t*)(S ? sd1 : sd0), 4,
                                               (uint32_t)(it * BQ + lane) * 4, 0, 0, 0);
    }
  };

  // LDS element offsets of the operand reads (relative to a tile base).
  // Row reads (A operand of S and dP): row 32a + li, logical chunk 2c + hh.
  const int rsw = swz<D>(li);
  int roff[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) roff[c] = li * D + (((2 * c + hh) ^ rsw) * 8);
  // Transposing reads (A operand of dV^T and dK^T): rows 16kc + trow (+8),
  // columns 32u + tcol.
  int toff[2][DU];
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int u = 0; u < DU; ++u) {
      const int r = trow + 8 * half;
      toff[half][u] = r * D + (((4 * u + (tcol >> 3)) ^ swz<D>(r)) * 8) + (tcol & 7);
    }
  // dS^T exchange: [key][row] with 64-row (128-byte) rows, chunk swizzle
  // swz<64>(key).  Writes: 4 consecutive rows per 8-byte store.  Reads (A
  // operand of dQ, k = key): transposing reads of keys 16ks + trow (+8), rows
  // 32a + tcol.
  int dsw[2][C::DQT];
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int t = 0; t < C::DQT; ++t) {
      const int r = trow + 8 * half;  // key within a 16-key chunk (low 4 bits of the key)
      dsw[half][t] = r * BQ + (((4 * dq_a[t] + (tcol >> 3)) ^ swz<64>(r)) * 8) + (tcol & 7);
    }
  const int wsw = swz<64>(32 * wave + li);  // this lane's dS^T row swizzle

  // dQ accumulator (fp32 workspace) addressing: tile (a, u) register r is row
  // 32a + 8(r/4) + 4hh + r%4, column 32u + li.
  const __amdgpu_buffer_rsrc_t qacc = make_rsrc(p.dq_acc + head_off, (uint32_t)N * D * 4);

  const float c2 = p.scale_log2;
  const int it0 = CAUSAL ? kb / BQ : 0;
  const int nit = (N + BQ - 1) / BQ;
  // Tiles before it_free need masking: causal diagonal tiles, or all tiles of
  // a block that reaches past the key length.
  int it_free = it0;
  if (CAUSAL) it_free = min(nit, (kb + BK - 1) / BQ + 1);
  if (kb + BK > L) it_free = nit;

  auto iter = [&](int it, auto par_t, auto masked_t) {
    constexpr int S = decltype(par_t)::value;  // stage parity = (it - it0) & 1
    constexpr bool masked = decltype(masked_t)::value;
    const bf16* qs = S ? sq1 : sq0;
    const bf16* os = S ? so1 : so0;
    const float* ls = S ? sl1 : sl0;
    const float* dls = S ? sd1 : sd0;
    bf16* dsx = sds + S * DST;
    const int r0 = it * BQ;

    // ---- S = Q K^T and dP = dO V^T: row tile a, k-step c; A from row reads.
    f32x16 sacc[2], pacc[2];
    auto rread = [&](const bf16* base, int a, int c) {
      return *(const bf16x8*)(base + roff[c] + a * 32 * D);
    };
    const f32x16 zero = {};
    constexpr int NS = 4 * KC;  // S0, S1, dP0, dP1 MFMAs
    bf16x8 ring[3];
    auto sread = [&](int i) {
      const int m = i / KC, c = i % KC;  // m: 0,1 = S row tiles, 2,3 = dP row tiles
      return rread(m < 2 ? qs : os, m & 1, c);
    };
    ring[0] = sread(0);
    ring[1] = sread(1);
    __builtin_amdgcn_sched_barrier(0);

    float lse4[2][4], dd4[2][4];  // per-row terms of the current 4-row group
    bf16x8 pb[4], dsb[4];         // P~ and dS as B operands, chunk kc = 16 rows
    // Elementwise work on S tile a (after it is complete): P (unmasked or
    // masked), packed later with dS.
    auto p_elems = [&](int a, int g) {
      // rows 32a + 8g + 4hh + e, e = 0..3
      const f32x4 l4 = *(const f32x4*)(ls + 32 * a + 8 * g + 4 * hh);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float pv = fast_exp2(fmaf(sacc[a][4 * g + e], c2, -l4[e]));
        if constexpr (masked) {
          const int row = r0 + 32 * a + 8 * g + 4 * hh + e;
          const bool ok = key < L && (!CAUSAL || key <= row);
          pv = ok ? pv : 0.0f;
        }
        sacc[a][4 * g + e] = pv;
      }
    };
    auto ds_elems = [&](int a, int g) {
      const f32x4 d4 = *(const f32x4*)(dls + 32 * a + 8 * g + 4 * hh);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * g + e;
        float pv = sacc[a][r], dp = pacc[a][r], pt = pv;
        if constexpr (DROPOUT) {
          const int row = r0 + 32 * a + 8 * g + 4 * hh + e;
          const u32x4 w = philox((uint32_t)key >> 2, (uint32_t)row, (uint32_t)hi, (uint32_t)bi,
                                 p.seed_lo, p.seed_hi);
          const uint32_t word = (key & 3) == 0 ? w[0] : (key & 3) == 1 ? w[1] : (key & 3) == 2 ? w[2] : w[3];
          const float z = word >= p.drop_threshold ? p.drop_scale : 0.0f;
          pt = pv * z;
          dp = dp * z;
        }
        const float ds = pv * (dp - d4[e]);
        // chunk kc = 2a + g/2 holds rows 16kc + 8(x/4) + 4hh + x%4 in slot x
        pb[2 * a + (g >> 1)][4 * (g & 1) + e] = (bf16)pt;
        dsb[2 * a + (g >> 1)][4 * (g & 1) + e] = (bf16)ds;
      }
    };
    // MFMA i of this phase plus its share of the elementwise work:
    //   S0 | S1 + P of tile 0 | dP0 + P of tile 1 | dP1 + dS of tile 0,
    // one 4-row group every KC/4 MFMAs.
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      if (i + 2 < NS) ring[(i + 2) % 3] = sread(i + 2);
      const int m = i / KC, c = i % KC;
      f32x16& acc = m < 2 ? sacc[m & 1] : pacc[m & 1];
      acc = mfma32(ring[i % 3], m < 2 ? kreg[c] : vreg[c], c == 0 ? zero : acc);
      if ((c * 4) % KC == 0) {
        const int g = c * 4 / KC;
        if (m == 1) p_elems(0, g);
        if (m == 2) p_elems(1, g);
        if (m == 3) ds_elems(0, g);
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- dV^T += dO^T P~ and dK^T += Q^T dS (contraction over the 64 rows);
    // the dS of row tile 1 is finished during the first dV^T MFMAs.
    const lds_bf16* qt = to_lds(qs);
    const lds_bf16* ot = to_lds(os);
    auto tread = [&](const lds_bf16* base, int u, int kc) {
      const bf16x4 lo = lds_read_tr4(base + toff[0][u] + 16 * kc * D);
      const bf16x4 h4 = lds_read_tr4(base + toff[1][u] + 16 * kc * D);
      return bf16x8{lo[0], lo[1], lo[2], lo[3], h4[0], h4[1], h4[2], h4[3]};
    };
    constexpr int NT = 8 * DU;  // dV^T then dK^T MFMAs: index = (which, kc, u)
    auto tnext = [&](int i) {
      const int which = i / (4 * DU), kc = (i / DU) % 4, u = i % DU;
      return tread(which == 0 ? ot : qt, u, kc);
    };
    ring[0] = tnext(0);
    ring[1] = tnext(1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      if (i + 2 < NT) ring[(i + 2) % 3] = tnext(i + 2);
      const int which = i / (4 * DU), kc = (i / DU) % 4, u = i % DU;
      if (which == 0) {
        dvacc[u] = mfma32(ring[i % 3], pb[kc], dvacc[u]);
      } else {
        dkacc[u] = mfma32(ring[i % 3], dsb[kc], dkacc[u]);
      }
      // dS of row tile 1 (chunks 2, 3) is needed from dK^T MFMA 2*DU on.
      if (i < 4) ds_elems(1, i);
      // dS^T rows of this wave's keys, 4 consecutive query rows per 8-byte write
      if (i >= 4 * DU && i < 4 * DU + 8) {
        const int w = i - 4 * DU, a = w >> 2, g = w & 3;
        const bf16x8& src = dsb[2 * a + (g >> 1)];
        const int o4 = 4 * (g & 1);
        const bf16x4 w4 = {src[o4], src[o4 + 1], src[o4 + 2], src[o4 + 3]};
        const int chunk = (4 * a + g) ^ wsw;
        *(bf16x4*)(dsx + (32 * wave + li) * BQ + chunk * 8 + 4 * hh) = w4;
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // The next tile's copies (issued one tile ago) must have landed before the
    // barrier that hands its stage over; the barrier also publishes dS^T.
    wait_vmem();
    __syncthreads();

    // ---- dQ tiles (rows of this tile x 32 head dims) += dS K over the block's keys.
    const lds_bf16* dt = to_lds(dsx);
    f32x16 qacc_t[C::DQT];
    auto dqread = [&](int i) {
      const int t = i / (BK / 16), ks16 = i % (BK / 16);
      const bf16x4 lo = lds_read_tr4(dt + dsw[0][t] + 16 * ks16 * BQ);
      const bf16x4 h4 = lds_read_tr4(dt + dsw[1][t] + 16 * ks16 * BQ);
      return bf16x8{lo[0], lo[1], lo[2], lo[3], h4[0], h4[1], h4[2], h4[3]};
    };
    constexpr int NQ = C::DQT * (BK / 16);
    ring[0] = dqread(0);
    ring[1] = dqread(1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      if (i + 2 < NQ) ring[(i + 2) % 3] = dqread(i + 2);
      const int t = i / (BK / 16), ks16 = i % (BK / 16);
      qacc_t[t] = mfma32(ring[i % 3], kfr[ks16], ks16 == 0 ? zero : qacc_t[t]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // fp32 atomics into the workspace; rows past N are skipped.
#pragma unroll
    for (int t = 0; t < C::DQT; ++t) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = r0 + 32 * dq_a[t] + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (row < N)
          __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(
              qacc_t[t][r], qacc, (uint32_t)(row * D + 32 * dq_u[t] + li) * 4, 0, 0);
      }
    }
    // Copies for the tile after next go into the stage this tile used.
    if (it + 2 < nit) issue_tile(it + 2, par_t);
  };
  using T = std::true_type;
  using F = std::false_type;

  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  issue_tile(it0, P0{});
  if (it0 + 1 < nit) issue_tile(it0 + 1, P1{});
  wait_vmem();
  __syncthreads();
  // Masked tiles come first; their count is even unless they run to the end.
  int it = it0;
  for (; it + 1 < it_free; it += 2) {
    iter(it, P0{}, T{});
    iter(it + 1, P1{}, T{});
  }
  if (it < it_free) {
    iter(it, P0{}, T{});
    ++it;
  }
  for (; it + 1 < nit; it += 2) {
    iter(it, P0{}, F{});
    iter(it + 1, P1{}, F{});
  }
  if (it < nit) iter(it, P0{}, F{});

  store_dkdv();
}

// D_i = sum_k dO_ik O_ik and LSE_i * log2(e) (+inf for an empty row, so that
// the recomputed probabilities exp2(s - LSE*log2e) vanish); also clears the
// dQ accumulator.  D/8 lanes per row.
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const bf16* __restrict__ o,
                                                      const bf16* __restrict__ dout,
                                                      const float* __restrict__ lse,
                                                      float* __restrict__ delta,
                                                      float* __restrict__ lse2,
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
  if (row < rows && ch == 0) {
    delta[row] = s;
    const float lv = lse[row];
    lse2[row] = lv == -INFINITY ? INFINITY : lv * kLog2e;
  }
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
                     (const bf16*)a.o, (const bf16*)a.dout, a.lse, a.delta, a.lse2, a.dq_acc, rows);
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
  p.lse2 = a.lse2;
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
