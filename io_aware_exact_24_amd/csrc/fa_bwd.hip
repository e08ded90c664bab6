// Backward pass of exact attention on gfx950 (recomputation instead of a
// stored probability matrix: ML Canon 48 FlashAttention, "backward without
// N x N"; Flash Attention hardware-aware optimisation, section 2.2, keep only the softmax
// normalisation statistics and rebuild the weights blockwise).
//
// With P = exp(scale * Q K^T - LSE) (recomputed, masked), Z the dropout
// keep mask scaled by 1/(1-p), and D_i = sum_k dO_ik O_ik:
//     dV = (P*Z)^T dO,   dP = dO V^T,   dS = P * (dP*Z - D),
//     dK = scale * dS^T Q,   dQ = scale * dS K.
//
// Three kernels on one stream:
//  1. bwd_pre:  D_i and LSE_i * log2(e) per row (fp32, in the workspace).
//  2. bwd_dkdv: one workgroup of 4 waves per 128-key block; each wave owns 32
//     keys and keeps their K and V rows (B operands) and fp32 dK^T / dV^T
//     accumulators in registers while the workgroup walks the 64-row query
//     tiles that can see the block.  S and dP come out of the MFMA with a lane
//     per key and 16 query rows per lane, which is the B-operand layout of the
//     dV^T and dK^T products; their A operands dO^T and Q^T are transposing
//     LDS reads of the row-major tiles.
//  3. bwd_dq: one workgroup of 4 waves x 32 queries per query block; each
//     wave keeps Q^T, dO^T and an fp32 dQ^T accumulator in registers and
//     streams K/V tiles, recomputing S^T and dP^T (a lane per query, so LSE
//     and D are per-lane scalars) and adding K^T dS^T.
// Splitting dQ from dK/dV costs two extra products (S and dP are computed in
// both kernels) but every gradient is accumulated in registers and written
// once: no fp32 atomics (which on this part execute at the memory side, not
// in L2), no fp32 dQ workspace and no conversion pass, and dQ is
// deterministic.
//
// Q/dO tiles (bwd_dkdv) and K/V tiles (bwd_dq) are copied global -> LDS by
// buffer loads into double-buffered, XOR-swizzled stages (conflict-free row and
// transposing reads, rows past N read as zero).
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
  bf16* dq;
  bf16* dk;
  bf16* dv;
  const int32_t* key_lens;
  int H, N, num_blocks;
  float scale, scale_log2;
  uint32_t drop_threshold;
  float drop_scale;
  uint32_t seed_lo, seed_hi;
};

using T_ = std::true_type;
using F_ = std::false_type;
using P0 = std::integral_constant<int, 0>;
using P1 = std::integral_constant<int, 1>;

// Dropout keep factor of element (row, key): 1/(1-p) or 0.
__device__ __forceinline__ float dropout_z(const BwdParams& p, int row, int key, int hi, int bi) {
  const u32x4 w = philox((uint32_t)key >> 2, (uint32_t)row, (uint32_t)hi, (uint32_t)bi, p.seed_lo,
                         p.seed_hi);
  const uint32_t word = (key & 3) == 0 ? w[0] : (key & 3) == 1 ? w[1] : (key & 3) == 2 ? w[2] : w[3];
  return word >= p.drop_threshold ? p.drop_scale : 0.0f;
}

// ----------------------------------------------------------------------------
// dK, dV
// ----------------------------------------------------------------------------
template <int D>
struct KvCfg {
  static constexpr int NW = 8;        // two waves per SIMD
  static constexpr int THREADS = 64 * NW;
  static constexpr int BK = 128;      // keys per workgroup: 4 groups of 32
  static constexpr int BQ = 64;       // query rows per tile: 2 halves of 32
  static constexpr int CHUNKS = D / 8;
  static constexpr int TILE = BQ * D;                  // elements of a Q or dO tile
  static constexpr int KTILE = BK * D;                 // elements of the K or V block
  static constexpr int LOADS = BQ * CHUNKS / THREADS;  // 16-byte copies per thread per tile
  static constexpr int KLOADS = BK * CHUNKS / THREADS;
  static_assert(LOADS * THREADS == BQ * CHUNKS, "tile/thread mismatch");
  static_assert(KLOADS * THREADS == BK * CHUNKS, "block/thread mismatch");
};

// Wave w owns key group w % 4 (32 keys) and row half w / 4 of every query
// tile, so the two waves of a key group split the contraction over rows; their
// partial dK^T / dV^T are added through LDS once at the end.  K and V of the
// block stay in LDS (B operands of S and dP), which keeps a wave within 256
// registers and lets two waves share each SIMD: one wave's exponentials and
// packing run while the other's MFMAs do.
template <int D, bool CAUSAL, bool DROPOUT>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void bwd_dkdv_kernel(BwdParams p) {
  using C = KvCfg<D>;
  constexpr int BQ = C::BQ, NW = C::NW, TILE = C::TILE, BK = C::BK, KTILE = C::KTILE;
  constexpr int KC = D / 16;  // k-steps of the S and dP products
  constexpr int DU = D / 32;  // 32-wide blocks of the head dimension
  // K and V of the block; stages of the Q and dO tiles and of the per-row
  // LSE*log2e and D.  Separate objects let the compiler see that a copy into
  // one stage cannot alias reads of the other.
  __shared__ __attribute__((aligned(1024))) bf16 sq0[TILE];
  __shared__ __attribute__((aligned(1024))) bf16 sq1[TILE];
  __shared__ __attribute__((aligned(1024))) bf16 so0[TILE];
  __shared__ __attribute__((aligned(1024))) bf16 so1[TILE];
  __shared__ __attribute__((aligned(256))) float sl0[BQ];
  __shared__ __attribute__((aligned(256))) float sl1[BQ];
  __shared__ __attribute__((aligned(256))) float sd0[BQ];
  __shared__ __attribute__((aligned(256))) float sd1[BQ];
  __shared__ __attribute__((aligned(1024))) bf16 skv[2 * KTILE];  // K block, then V block

  bf16* const sk = skv;
  bf16* const sv = skv + KTILE;

  const int N = p.N;
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int head = lid / p.num_blocks;
  const int jb = lid - head * p.num_blocks;  // low key blocks see the most rows: run first
  const int bi = head / p.H, hi = head - bi * p.H;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = wave & 3, rh = wave >> 2;  // key group, row half
  const int li = lane & 31, hh = lane >> 5;
  const int kb = jb * BK;               // first key of the workgroup
  const int key = kb + 32 * kg + li;    // this lane's key (column of S)

  int L = N;
  if (p.key_lens) L = min(max(p.key_lens[bi], 0), N);

  const size_t head_off = (size_t)head * N * D;

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
    if (rh != 0 || key >= N) return;
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

  // Copies: the K and V block once, then Q and dO tiles with LSE*log2e and D.
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(p.k + head_off, (uint32_t)N * D * 2);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(p.v + head_off, (uint32_t)N * D * 2);
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(p.q + head_off, (uint32_t)N * D * 2);
  const __amdgpu_buffer_rsrc_t ors = make_rsrc(p.dout + head_off, (uint32_t)N * D * 2);
  const __amdgpu_buffer_rsrc_t lrs = make_rsrc(p.lse2 + (size_t)head * N, (uint32_t)N * 4);
  const __amdgpu_buffer_rsrc_t drs = make_rsrc(p.delta + (size_t)head * N, (uint32_t)N * 4);
  // Byte offset within a tile of this lane's i-th 16-byte copy (the chunk
  // slot it fills is (i * NW + wave) * 64 + lane).
  auto copy_off = [&](int i) {
    const int pch = (i * NW + wave) * 64 + lane;
    const int r = pch / C::CHUNKS, pc = pch % C::CHUNKS;
    return (uint32_t)(r * D + ((pc ^ swz<D>(r)) * 8)) * 2;
  };
#pragma unroll
  for (int i = 0; i < C::KLOADS; ++i) {
    const uint32_t off = copy_off(i) + (uint32_t)kb * (D * 2);
    lds_dma16(krs, sk + (i * NW + wave) * 512, off);
    lds_dma16(vrs, sv + (i * NW + wave) * 512, off);
  }
  uint32_t ld_off[C::LOADS];
#pragma unroll
  for (int i = 0; i < C::LOADS; ++i) ld_off[i] = copy_off(i);
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

  // LDS element offsets of the operand reads; the wave's row half and key
  // group are folded in so that every stage and block base is a constant.
  // Row reads (A operand Q / dO of S and dP: row 32rh + li of a tile; B
  // operand K / V: row 32kg + li of the block), logical chunk 2c + hh.
  const int rsw = swz<D>(li);
  int roffq[KC], roffk[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    roffq[c] = (32 * rh + li) * D + (((2 * c + hh) ^ rsw) * 8);
    roffk[c] = (32 * kg + li) * D + (((2 * c + hh) ^ rsw) * 8);
  }
  // Transposing reads (A operand of dV^T and dK^T): within a 16-row chunk,
  // rows trow and trow + 8, columns tcol .. tcol + 3 of a 32-column block; the
  // k-slot e of a lane is row 8(e/4) + 4hh + e%4 of the chunk, which matches
  // the row order of P and dS in the MFMA output layout.
  const int g16 = lane & 15;
  const int trow = 4 * hh + (g16 >> 2);
  const int tcol = 16 * ((lane >> 4) & 1) + 4 * (g16 & 3);
  int toff[2][DU];
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int u = 0; u < DU; ++u) {
      const int r = trow + 8 * half;
      toff[half][u] = (32 * rh + r) * D + (((4 * u + (tcol >> 3)) ^ swz<D>(r)) * 8) + (tcol & 7);
    }
  const int rowoff = 32 * rh + 4 * hh;  // per-row terms: rows 32rh + 8g + 4hh + e of a tile

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
    constexpr bool MASKED = decltype(masked_t)::value;
    const bf16* qs = S ? sq1 : sq0;
    const bf16* os = S ? so1 : so0;
    const float* ls = S ? sl1 : sl0;
    const float* dls = S ? sd1 : sd0;
    const int r0 = it * BQ + 32 * rh;  // first row of this wave
    __syncthreads();  // tile it resident in stage S; every wave is done with tile it-1
    // copies for the next tile go into the other stage, read during tile it-1
    if (it + 1 < nit) issue_tile(it + 1, std::integral_constant<int, S ^ 1>{});

    // ---- S = Q K^T and dP = dO V^T (32 rows x 32 keys each), k-step c:
    // A from Q / dO row reads, B from K / V row reads.
    f32x16 sacc, pacc;
    const f32x16 zero = {};
    constexpr int NS = 2 * KC;  // S then dP MFMAs
    bf16x8 ra[3], rb[3];
    auto aread = [&](int i) { return *(const bf16x8*)((i < KC ? qs : os) + roffq[i % KC]); };
    auto bread = [&](int i) { return *(const bf16x8*)((i < KC ? sk : sv) + roffk[i % KC]); };
    ra[0] = aread(0);
    rb[0] = bread(0);
    ra[1] = aread(1);
    rb[1] = bread(1);
    __builtin_amdgcn_sched_barrier(0);

    bf16x8 pb[2], dsb[2];  // P~ and dS as B operands, chunk kc = 16 rows
    // P of row group g (rows 8g + 4hh + e of the wave's 32), in place.
    auto p_elems = [&](int g) {
      const f32x4 l4 = *(const f32x4*)(ls + rowoff + 8 * g);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float pv = fast_exp2(fmaf(sacc[4 * g + e], c2, -l4[e]));
        if constexpr (MASKED) {
          const int row = r0 + 8 * g + 4 * hh + e;
          const bool ok = key < L && (!CAUSAL || key <= row);
          pv = ok ? pv : 0.0f;
        }
        sacc[4 * g + e] = pv;
      }
    };
    // dS (and P~ = P*Z) of row group g, packed into the B chunks.
    auto ds_elems = [&](int g) {
      const f32x4 d4 = *(const f32x4*)(dls + rowoff + 8 * g);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * g + e;
        const float pv = sacc[r];
        float dp = pacc[r], pt = pv;
        if constexpr (DROPOUT) {
          const float z = dropout_z(p, r0 + 8 * g + 4 * hh + e, key, hi, bi);
          pt = pv * z;
          dp = dp * z;
        }
        // chunk kc = g/2 holds rows 16kc + 8(x/4) + 4hh + x%4 in slot x
        pb[g >> 1][4 * (g & 1) + e] = (bf16)pt;
        dsb[g >> 1][4 * (g & 1) + e] = (bf16)(pv * (dp - d4[e]));
      }
    };
    // MFMA i plus its share of the elementwise work: the exponentials of S
    // while dP is computed, one 4-row group every KC/4 MFMAs.
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      if (i + 2 < NS) {
        ra[(i + 2) % 3] = aread(i + 2);
        rb[(i + 2) % 3] = bread(i + 2);
      }
      const int c = i % KC;
      f32x16& acc = i < KC ? sacc : pacc;
      acc = mfma32(ra[i % 3], rb[i % 3], c == 0 ? zero : acc);
      if (i >= KC && (c * 4) % KC == 0) p_elems(c * 4 / KC);
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- dV^T += dO^T P~ and dK^T += Q^T dS (contraction over the wave's 32
    // rows); dS is finished during the first dV^T MFMAs.
    const lds_bf16* qt = to_lds(qs);
    const lds_bf16* ot = to_lds(os);
    constexpr int NT = 4 * DU;  // dV^T then dK^T MFMAs: index = (which, kc, u)
    auto tnext = [&](int i) {
      const int which = i / (2 * DU), kc = (i / DU) % 2, u = i % DU;
      const lds_bf16* base = which == 0 ? ot : qt;
      const bf16x4 lo = lds_read_tr4(base + toff[0][u] + 16 * kc * D);
      const bf16x4 h4 = lds_read_tr4(base + toff[1][u] + 16 * kc * D);
      return bf16x8{lo[0], lo[1], lo[2], lo[3], h4[0], h4[1], h4[2], h4[3]};
    };
    ra[0] = tnext(0);
    ra[1] = tnext(1);
    __builtin_amdgcn_sched_barrier(0);
    // P~ and dS groups 0, 1 form chunk 0, used from MFMA 0.
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      if (i == 0) {
        ds_elems(0);
        ds_elems(1);
      }
      if (i + 2 < NT) ra[(i + 2) % 3] = tnext(i + 2);
      const int which = i / (2 * DU), kc = (i / DU) % 2, u = i % DU;
      if (which == 0) {
        dvacc[u] = mfma32(ra[i % 3], pb[kc], dvacc[u]);
      } else {
        dkacc[u] = mfma32(ra[i % 3], dsb[kc], dkacc[u]);
      }
      // groups 2, 3 (chunk 1) are first used by MFMA DU
      if (i == 1) ds_elems(2);
      if (i == DU - 1) ds_elems(3);
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_vmem();  // next tile landed (this wave's share) before the next barrier
  };

  issue_tile(it0, P0{});
  wait_vmem();
  // Masked tiles come first; their count is even unless they run to the end.
  int it = it0;
  for (; it + 1 < it_free; it += 2) {
    iter(it, P0{}, T_{});
    iter(it + 1, P1{}, T_{});
  }
  if (it < it_free) {
    iter(it, P0{}, T_{});
    ++it;
  }
  for (; it + 1 < nit; it += 2) {
    iter(it, P0{}, F_{});
    iter(it + 1, P1{}, F_{});
  }
  if (it < nit) iter(it, P0{}, F_{});

  // Add the row-half-1 partials into the row-half-0 waves through LDS (the
  // K/V block buffer is free now), dK^T then dV^T: register r of tile u of
  // lane l at (u*16 + r)*64 + l of the key group's slot.
  float* const xs = (float*)skv;
  static_assert(4 * D / 32 * 16 * 64 * 4 <= 2 * KTILE * 2, "exchange must fit the K/V buffer");
  float* const mine = xs + kg * (DU * 16 * 64);
  auto exchange = [&](f32x16 (&acc)[DU]) {
    __syncthreads();
    if (rh == 1) {
#pragma unroll
      for (int u = 0; u < DU; ++u)
#pragma unroll
        for (int r = 0; r < 16; ++r) mine[(u * 16 + r) * 64 + lane] = acc[u][r];
    }
    __syncthreads();
    if (rh == 0) {
#pragma unroll
      for (int u = 0; u < DU; ++u)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[u][r] += mine[(u * 16 + r) * 64 + lane];
    }
  };
  exchange(dkacc);
  exchange(dvacc);
  store_dkdv();
}

// ----------------------------------------------------------------------------
// dQ
// ----------------------------------------------------------------------------
template <int D>
struct QCfg {
  static constexpr int NW = 4;
  static constexpr int THREADS = 64 * NW;
  static constexpr int BM = 32 * NW;  // queries per workgroup
  static constexpr int BN = 64;       // keys per K/V tile
  static constexpr int CHUNKS = D / 8;
  static constexpr int TILE = BN * D;
  static constexpr int LOADS = BN * CHUNKS / THREADS;
  static_assert(LOADS * THREADS == BN * CHUNKS, "tile/thread mismatch");
};

template <int D, bool CAUSAL, bool DROPOUT>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 2)))
void bwd_dq_kernel(BwdParams p) {
  using C = QCfg<D>;
  constexpr int BN = C::BN, NW = C::NW, TILE = C::TILE;
  constexpr int KC = D / 16;
  constexpr int DU = D / 32;
  __shared__ __attribute__((aligned(1024))) bf16 sk0[TILE];
  __shared__ __attribute__((aligned(1024))) bf16 sk1[TILE];
  __shared__ __attribute__((aligned(1024))) bf16 sv0[TILE];
  __shared__ __attribute__((aligned(1024))) bf16 sv1[TILE];

  const int N = p.N;
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int head = lid / p.num_blocks;
  const int qb = p.num_blocks - 1 - (lid - head * p.num_blocks);  // costliest blocks first
  const int bi = head / p.H, hi = head - bi * p.H;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, hh = lane >> 5;
  const int q0 = qb * C::BM;
  const int qi = q0 + wave * 32 + li;  // this lane's query

  int L = N;
  if (p.key_lens) L = min(max(p.key_lens[bi], 0), N);
  const int kend = CAUSAL ? min(L, q0 + C::BM) : L;
  const int nkb = (kend + BN - 1) / BN;
  // Tiles [0, nfree) are unmasked for every query of the workgroup.
  int nfree = L / BN;
  if (CAUSAL) nfree = min(nfree, q0 / BN);
  nfree = min(nfree, nkb);

  const size_t head_off = (size_t)head * N * D;
  // Q^T and dO^T as B operands (k = head dimension): lane holds row qi,
  // elements 16c + 8hh .. +7.
  bf16x8 qreg[KC], oreg[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    if (qi < N) {
      qreg[c] = *(const bf16x8*)(p.q + head_off + (size_t)qi * D + 16 * c + 8 * hh);
      oreg[c] = *(const bf16x8*)(p.dout + head_off + (size_t)qi * D + 16 * c + 8 * hh);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        qreg[c][e] = (bf16)0.0f;
        oreg[c][e] = (bf16)0.0f;
      }
    }
  }
  // Rows past N or without any allowed key: +inf makes every P vanish.
  const float lrow = qi < N ? p.lse2[(size_t)head * N + qi] : INFINITY;
  const float drow = qi < N ? p.delta[(size_t)head * N + qi] : 0.0f;

  const __amdgpu_buffer_rsrc_t krs = make_rsrc(p.k + head_off, (uint32_t)N * D * 2);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(p.v + head_off, (uint32_t)N * D * 2);
  uint32_t ld_off[C::LOADS];
#pragma unroll
  for (int i = 0; i < C::LOADS; ++i) {
    const int pch = (i * NW + wave) * 64 + lane;
    const int r = pch / C::CHUNKS, pc = pch % C::CHUNKS;
    ld_off[i] = (uint32_t)(r * D + ((pc ^ swz<D>(r)) * 8)) * 2;
  }
  auto issue = [&](int jt, auto par_t) {
    constexpr int S = decltype(par_t)::value;
    bf16* kd = S ? sk1 : sk0;
    bf16* vd = S ? sv1 : sv0;
    const uint32_t base = (uint32_t)jt * (BN * D * 2);
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      lds_dma16(krs, kd + (i * NW + wave) * 512, ld_off[i] + base);
      lds_dma16(vrs, vd + (i * NW + wave) * 512, ld_off[i] + base);
    }
  };
  // Row reads of K and V tiles (A operands of S^T and dP^T): row 32t + li,
  // logical chunk 2c + hh.  Transposing reads of the K tile (A operand of
  // dQ^T = K^T dS^T): rows 16cc + trow (+8), columns 32u + tcol.
  const int rsw = swz<D>(li);
  int roff[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) roff[c] = li * D + (((2 * c + hh) ^ rsw) * 8);
  const int g16 = lane & 15;
  const int trow = 4 * hh + (g16 >> 2);
  const int tcol = 16 * ((lane >> 4) & 1) + 4 * (g16 & 3);
  int toff[2][DU];
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int u = 0; u < DU; ++u) {
      const int r = trow + 8 * half;
      toff[half][u] = r * D + (((4 * u + (tcol >> 3)) ^ swz<D>(r)) * 8) + (tcol & 7);
    }

  f32x16 qacc[DU];  // dQ^T: tile u register r -> d = 32u + 8(r/4) + 4hh + r%4, query qi
#pragma unroll
  for (int u = 0; u < DU; ++u)
#pragma unroll
    for (int r = 0; r < 16; ++r) qacc[u][r] = 0.0f;
  const float c2 = p.scale_log2;

  auto step = [&](int j, auto par_t, auto masked_t) {
    constexpr int S = decltype(par_t)::value;  // j & 1
    constexpr bool MASKED = decltype(masked_t)::value;
    const bf16* ks = S ? sk1 : sk0;
    const bf16* vs = S ? sv1 : sv0;
    __syncthreads();  // tile j resident; every wave is done with tile j-1
    if (j + 1 < nkb) issue(j + 1, std::integral_constant<int, S ^ 1>{});

    // ---- S^T = K Q^T and dP^T = V dO^T: key tile t (32 keys), k-step c.
    f32x16 sacc[2], pacc[2];
    const f32x16 zero = {};
    constexpr int NS = 4 * KC;
    bf16x8 ring[3];
    auto sread = [&](int i) {
      const int m = i / KC, c = i % KC;
      return *(const bf16x8*)((m < 2 ? ks : vs) + roff[c] + (m & 1) * 32 * D);
    };
    ring[0] = sread(0);
    ring[1] = sread(1);
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 dsb[4];  // dS^T as B operands: chunk cc holds keys 16cc + 8(x/4) + 4hh + x%4
    // P^T of key tile t, keys 32t + 8g + 4hh + e of the tile, in place.
    auto p_elems = [&](int t, int g) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float pv = fast_exp2(fmaf(sacc[t][4 * g + e], c2, -lrow));
        if constexpr (MASKED) {
          const int key = j * BN + 32 * t + 8 * g + 4 * hh + e;
          const bool ok = key < L && (!CAUSAL || key <= qi);
          pv = ok ? pv : 0.0f;
        }
        sacc[t][4 * g + e] = pv;
      }
    };
    auto ds_elems = [&](int t, int g) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * g + e;
        float dp = pacc[t][r];
        if constexpr (DROPOUT) dp *= dropout_z(p, qi, j * BN + 32 * t + 8 * g + 4 * hh + e, hi, bi);
        dsb[2 * t + (g >> 1)][4 * (g & 1) + e] = (bf16)(sacc[t][r] * (dp - drow));
      }
    };
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      if (i + 2 < NS) ring[(i + 2) % 3] = sread(i + 2);
      const int m = i / KC, c = i % KC;
      f32x16& acc = m < 2 ? sacc[m & 1] : pacc[m & 1];
      acc = mfma32(ring[i % 3], m < 2 ? qreg[c] : oreg[c], c == 0 ? zero : acc);
      if ((c * 4) % KC == 0) {
        const int g = c * 4 / KC;
        if (m == 1) p_elems(0, g);
        if (m == 2) p_elems(1, g);
        if (m == 3) ds_elems(0, g);
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- dQ^T += K^T dS^T (contraction over the 64 keys)
    const lds_bf16* kt = to_lds(ks);
    constexpr int NQ = 4 * DU;  // index = (cc, u)
    auto tnext = [&](int i) {
      const int cc = i / DU, u = i % DU;
      const bf16x4 lo = lds_read_tr4(kt + toff[0][u] + 16 * cc * D);
      const bf16x4 h4 = lds_read_tr4(kt + toff[1][u] + 16 * cc * D);
      return bf16x8{lo[0], lo[1], lo[2], lo[3], h4[0], h4[1], h4[2], h4[3]};
    };
    ring[0] = tnext(0);
    ring[1] = tnext(1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      if (i + 2 < NQ) ring[(i + 2) % 3] = tnext(i + 2);
      const int cc = i / DU, u = i % DU;
      qacc[u] = mfma32(ring[i % 3], dsb[cc], qacc[u]);
      // chunks 2, 3 (key tile 1) are first used by MFMA 2*DU
      if (i < 4) ds_elems(1, i);
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_vmem();
  };

  if (nkb > 0) {
    issue(0, P0{});
    wait_vmem();
  }
  // Unmasked tiles first (from key 0), then the masked diagonal / tail ones.
  // Steps run in pairs from even indices so the stage parity is a compile-time
  // constant; tiles in [jm, nfree) take the masked path (harmless, it only
  // masks nothing there).
  const int jm = nfree & ~1;
  int j = 0;
  for (; j < jm; j += 2) {
    step(j, P0{}, F_{});
    step(j + 1, P1{}, F_{});
  }
  for (; j + 1 < nkb; j += 2) {
    step(j, P0{}, T_{});
    step(j + 1, P1{}, T_{});
  }
  if (j < nkb) step(j, P0{}, T_{});

  if (qi < N) {
    bf16* qrow = p.dq + head_off + (size_t)qi * D;
#pragma unroll
    for (int u = 0; u < DU; ++u)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 ov;
#pragma unroll
        for (int e = 0; e < 4; ++e) ov[e] = (bf16)(qacc[u][4 * g + e] * p.scale);
        *(bf16x4*)(qrow + 32 * u + 8 * g + 4 * hh) = ov;
      }
  }
}

// D_i = sum_k dO_ik O_ik and LSE_i * log2(e) (+inf for an empty row, so that
// the recomputed probabilities exp2(s - LSE*log2e) vanish).  D/8 lanes per row.
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const bf16* __restrict__ o,
                                                      const bf16* __restrict__ dout,
                                                      const float* __restrict__ lse,
                                                      float* __restrict__ delta,
                                                      float* __restrict__ lse2, int64_t rows) {
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
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, LPR);
  if (row < rows && ch == 0) {
    delta[row] = s;
    const float lv = lse[row];
    lse2[row] = lv == -INFINITY ? INFINITY : lv * kLog2e;
  }
}

template <int D, bool CAUSAL, bool DROPOUT>
hipError_t launch_main(BwdParams p, int heads, int stages, hipStream_t s) {
  if (stages & kBwdKV) {
    p.num_blocks = (p.N + KvCfg<D>::BK - 1) / KvCfg<D>::BK;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, DROPOUT>), dim3(heads * p.num_blocks),
                       dim3(KvCfg<D>::THREADS), 0, s, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (stages & kBwdQ) {
    p.num_blocks = (p.N + QCfg<D>::BM - 1) / QCfg<D>::BM;
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, DROPOUT>), dim3(heads * p.num_blocks),
                       dim3(QCfg<D>::THREADS), 0, s, p);
    return hipGetLastError();
  }
  return hipSuccess;
}

template <int D>
hipError_t run(const BwdArgs& a, const BwdParams& p, int stages, hipStream_t s) {
  if (stages & kBwdPre) {
    const int64_t rows = (int64_t)a.B * a.H * a.N;
    const int64_t pre_threads = rows * (D / 8);
    hipLaunchKernelGGL(bwd_pre_kernel<D>, dim3((unsigned)((pre_threads + 255) / 256)), dim3(256), 0,
                       s, (const bf16*)a.o, (const bf16*)a.dout, a.lse, a.delta, a.lse2, rows);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int heads = a.B * a.H;
  const bool drop = a.dropout_p > 0.0f;
  if (a.causal)
    return drop ? launch_main<D, true, true>(p, heads, stages, s)
                : launch_main<D, true, false>(p, heads, stages, s);
  return drop ? launch_main<D, false, true>(p, heads, stages, s)
              : launch_main<D, false, false>(p, heads, stages, s);
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs& a, int stages, hipStream_t s) {
  BwdParams p;
  p.q = (const bf16*)a.q;
  p.k = (const bf16*)a.k;
  p.v = (const bf16*)a.v;
  p.dout = (const bf16*)a.dout;
  p.lse2 = a.lse2;
  p.delta = a.delta;
  p.dq = (bf16*)a.dq;
  p.dk = (bf16*)a.dk;
  p.dv = (bf16*)a.dv;
  p.key_lens = a.key_lens;
  p.H = a.H;
  p.N = a.N;
  p.num_blocks = 0;
  p.scale = a.scale;
  p.scale_log2 = a.scale * kLog2e;
  p.drop_threshold = a.drop_threshold;
  p.drop_scale = a.drop_scale;
  p.seed_lo = (uint32_t)(a.seed & 0xffffffffu);
  p.seed_hi = (uint32_t)(a.seed >> 32);
  return a.d == 64 ? run<64>(a, p, stages, s) : run<128>(a, p, stages, s);
}

}  // namespace fa
