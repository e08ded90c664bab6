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
// Two kernels on one stream, in this order:
//  1. bwd_dq: one workgroup of 4 waves x 32 queries per query block; each
//     wave keeps Q^T, dO^T (brought in through LDS by coalesced copies) and
//     an fp32 dQ^T accumulator in registers and streams K/V tiles,
//     recomputing S^T and dP^T (a lane per query, so LSE and D are per-lane
//     scalars) and adding K^T dS^T.  Its prologue computes the per-row terms
//     D_i = sum_k dO_ik O_ik and LSE_i * log2(e) from the dO row it holds and
//     one read of the O row, and writes them to the workspace.
//  2. bwd_dkdv: persistent, one workgroup of 4 waves (one per SIMD) per CU,
//     walking a chain of 128-key blocks; each wave owns 32 keys and keeps
//     their K and V rows (B operands) and the fp32 dK^T / dV^T accumulators
//     (in AccVGPRs) in registers while the workgroup walks the 64-row query
//     tiles that can see the block, reading D and LSE * log2(e) of each
//     tile's rows from the workspace; the next block's K/V rows are fetched
//     during the current block's first tile.  S and
//     dP come out of the MFMA with a lane per key and 16 query rows per lane,
//     which is the B-operand layout of the dV^T and dK^T products; their A
//     operands dO^T and Q^T are transposing LDS reads of the row-major tiles.
//     The products of tile t are skewed against those of tile t+1 so every
//     group of MFMAs has independent elementwise work beside it.
// bwd_pre computes the same per-row terms on its own, for a caller that wants
// dK/dV without dQ.
// Splitting dQ from dK/dV costs two extra products (S and dP are computed in
// both kernels) but every gradient is accumulated in registers and written
// once: no fp32 atomics (which on this part execute at the memory side, not
// in L2), no fp32 dQ workspace and no conversion pass, and dQ is
// deterministic.
//
// Q/dO tiles (bwd_dkdv, three stages) and K/V tiles (bwd_dq, two stages) are
// copied global -> LDS by buffer loads into XOR-swizzled stages (conflict-free
// row and transposing reads, rows past N read as zero).  Gradients leave the
// registers through free LDS stages and are stored as whole rows.
#pragma once

#include <type_traits>

#include "fa_common.hpp"
#include "fa_internal.hpp"

namespace fa {

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  const void* o;       // forward output (read by the dQ kernel for D)
  const float* lse;    // forward LSE, contiguous [B, H, N] (natural log; read by the dQ kernel)
  float* lse2;         // LSE * log2(e), +inf for rows without any allowed key
  float* delta;        // D
  void* dq;
  void* dk;
  void* dv;
  // element strides (batch, head, row) of each tensor; d is contiguous
  Strides sq, sk, sv, so, sdo, sdq, sdk, sdv;
  const int32_t* key_lens;
  // Packed sequences (nullptr otherwise): batch entry b is rows [cu[b],
  // cu[b+1]) of every tensor (at most N of them; the batch strides are 0); its
  // LSE, D and LSE * log2(e) are the [H, len] blocks at H * cu[b].
  const int32_t* cu;
  int H, N, num_blocks;
  int dl;  // head size of the tensors, <= D: columns [dl, D) read as zero and are not written
  int b0;  // added to the batch index in the dropout counter
  int units;  // dK/dV work units (blocks, or causal pairs of blocks, times splits) over all heads
  int heads;  // B * H
  // Split backward: `splits` shares per query block (dQ: of its key tiles) or
  // per key-block unit (dK/dV: of its query tiles); share s writes its fp32
  // partial gradient rows to dqp / dkp / dvp + ((s * heads + head) * N + row) * d,
  // every row of its blocks (zeros where the share has no tile).
  int splits;
  float* dqp;
  float* dkp;
  float* dvp;
  float scale, scale_log2;
  uint32_t drop_threshold;
  float drop_scale;
  uint32_t seed_lo, seed_hi;
};

// Stage launchers (fa_bwd_dq.hip, fa_bwd_dkdv.hip).  contig: every tensor's
// row stride is d elements (tile offsets fold into constants).
hipError_t launch_bwd_pre(const BwdParams& p, bool fp16, int d, int64_t rows, hipStream_t s);
hipError_t launch_bwd_dq(BwdParams p, bool fp16, int d, bool causal, bool dropout, bool contig,
                         int heads, hipStream_t s);
hipError_t launch_bwd_dkdv(BwdParams p, bool fp16, int d, bool causal, bool dropout, bool contig,
                           int heads, hipStream_t s);
// Split backward (p.splits > 0, contiguous rows): the same two stages writing
// fp32 partials, then the combine pass into dq, dk, dv.
hipError_t launch_bwd_combine(const BwdParams& p, bool fp16, int d, int64_t rows, hipStream_t s);

namespace {

using T_ = std::true_type;
using F_ = std::false_type;
using P0 = std::integral_constant<int, 0>;
using P1 = std::integral_constant<int, 1>;

// Dropout keep factor of element (row, key): 1/(1-p) or 0.
__device__ __forceinline__ float dropout_z(const BwdParams& p, int row, int key, int hi, int bi) {
  const u32x4 w = philox((uint32_t)key >> 2, (uint32_t)row, (uint32_t)hi, (uint32_t)(bi + p.b0), p.seed_lo,
                         p.seed_hi);
  const uint32_t word = philox_word(w, key);
  return word >= p.drop_threshold ? p.drop_scale : 0.0f;
}

// ----------------------------------------------------------------------------
// dK, dV
// ----------------------------------------------------------------------------
template <int D>
struct KvCfg {
  static constexpr int NW = 4;        // one wave per SIMD
  static constexpr int THREADS = 64 * NW;
  static constexpr int BK = 32 * NW;  // keys per workgroup: a 32-key group per wave
  static constexpr int BQ = 64;       // query rows per tile: 2 halves of 32
  static constexpr int CHUNKS = D / 8;
  static constexpr int TILE = BQ * D;                  // elements of a Q or dO tile
  static constexpr int LOADS = BQ * CHUNKS / THREADS;  // 16-byte copies per thread per tile
  static_assert(LOADS * THREADS == BQ * CHUNKS, "tile/thread mismatch");
};

template <int S>
using Stage = std::integral_constant<int, S % 3>;

// Keep bits of rows row0 .. row0+3 at this lane's key (bit e: row row0 + e),
// for a lane whose quad (lanes 4m .. 4m+3) holds the keys 4m' .. 4m'+3 of one
// Philox counter group (key & 3 == lane & 3).  Lane q draws the counter of row
// row0 + q, whose four words are the four keys' draws at that row: one Philox
// block per lane for four elements instead of one per element.  The quad then
// transposes the 4 x 4 keep bits: lane q compares its words (bit i: key i at
// row row0 + q) into nibble q of a 16-bit word, two DPP exchanges (lanes q^1,
// then q^2) OR the four nibbles together in every lane, and lane q gathers
// bits 4e + q (key q at row row0 + e) into bit e with one multiply.
__device__ __forceinline__ uint32_t quad_keep4(const BwdParams& p, int row0, int key, int hi,
                                               int bi) {
  const int q = threadIdx.x & 3;
  const u32x4 w = philox((uint32_t)key >> 2, (uint32_t)(row0 + q), (uint32_t)hi, (uint32_t)(bi + p.b0),
                         p.seed_lo, p.seed_hi);
  uint32_t kb = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) kb |= (uint32_t)(w[i] >= p.drop_threshold) << i;
  uint32_t m = kb << (4 * q);
  constexpr int kXor1 = 1 | (0 << 2) | (3 << 4) | (2 << 6);  // lane i reads lane i ^ 1 of its quad
  constexpr int kXor2 = 2 | (3 << 2) | (0 << 4) | (1 << 6);  // lane i reads lane i ^ 2
  m |= (uint32_t)__builtin_amdgcn_mov_dpp((int)m, kXor1, 0xF, 0xF, false);
  m |= (uint32_t)__builtin_amdgcn_mov_dpp((int)m, kXor2, 0xF, 0xF, false);
  // bits 0, 4, 8, 12 of x times 1 + 2^3 + 2^6 + 2^9 land on bits 9 .. 12
  // (every other product bit falls elsewhere, without carries)
  const uint32_t x = (m >> q) & 0x1111u;
  return ((x * 0x249u) >> 9) & 0xFu;
}

// 0xFFFFFFFF if bit b of bits is set, else 0: keeps or clears a float's bits.
__device__ __forceinline__ uint32_t bit_mask(uint32_t bits, int b) {
  return (uint32_t)((int32_t)(bits << (31 - b)) >> 31);
}

// One wave per SIMD, each owning 32 keys of the block: their K and V rows
// are B operands held in registers and their dK^T / dV^T accumulators stay
// in registers for the whole walk over the 64-row query tiles.  The work of
// tile t is skewed against tile t+1 so that every group of MFMAs has
// independent elementwise work beside it:
//   phase 0: dV^T += dO_t^T P~_t      | dS_t of rows 0..31
//   phase 1: S_{t+1} = Q_{t+1} K^T    | dS_t of rows 32..63
//   phase 2: dK^T += Q_t^T dS_t       | P_{t+1} of rows 0..31
//   phase 3: dP_{t+1} = dO_{t+1} V^T  | P_{t+1} of rows 32..63
// Tiles t (transposing reads) and t+1 (row reads) are read while tile t+2 is
// copied, so Q, dO, LSE*log2e and D have three LDS stages.
template <typename E, int D, bool CAUSAL, bool DROPOUT, bool CONTIG, bool SPLIT>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void bwd_dkdv_kernel(BwdParams p) {
  using C = KvCfg<D>;
  using V8 = typename Elem<E>::v8;
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef E e2 __attribute__((ext_vector_type(2)));
  using V4 = typename Elem<E>::v4;
  constexpr int ES = 2;
  constexpr int BQ = C::BQ, NW = C::NW, TILE = C::TILE, BK = C::BK;
  constexpr int KC = D / 16;  // k-steps of the S and dP products
  constexpr int DU = D / 32;  // 32-wide blocks of the head dimension
  constexpr int NP = 2 * KC;  // MFMAs per phase (also 4 * DU)
  static_assert(NP == 4 * DU, "phase sizes");
  // Operand reads run PD MFMAs ahead through RG ring slots (RG divides every
  // body's MFMA count and covers PD reads ahead plus the three operands kept
  // live behind): six ahead at width 128 (0.7-0.9% faster there), four at 64.
  constexpr int PD = D == 128 ? 6 : 4;
  constexpr int RG = D == 128 ? 16 : 8;
  __shared__ __attribute__((aligned(1024))) E sq0[TILE];
  __shared__ __attribute__((aligned(1024))) E so0[TILE];
  __shared__ __attribute__((aligned(1024))) E sq1[TILE];
  __shared__ __attribute__((aligned(1024))) E so1[TILE];
  __shared__ __attribute__((aligned(1024))) E sq2[TILE];
  __shared__ __attribute__((aligned(1024))) E so2[TILE];
  __shared__ __attribute__((aligned(256))) float sl0[BQ];
  __shared__ __attribute__((aligned(256))) float sl1[BQ];
  __shared__ __attribute__((aligned(256))) float sl2[BQ];
  __shared__ __attribute__((aligned(256))) float sd0[BQ];
  __shared__ __attribute__((aligned(256))) float sd1[BQ];
  __shared__ __attribute__((aligned(256))) float sd2[BQ];
  // K rows of the workgroup's key block (two 64-row tiles), copied in at the
  // start of each block; its V rows go to stage 2 until the first body.
  __shared__ __attribute__((aligned(1024))) E skv[2 * TILE];
  auto qst = [&](auto s) __attribute__((always_inline)) -> E* {
    constexpr int S = decltype(s)::value;
    return S == 0 ? sq0 : S == 1 ? sq1 : sq2;
  };
  auto ost = [&](auto s) __attribute__((always_inline)) -> E* {
    constexpr int S = decltype(s)::value;
    return S == 0 ? so0 : S == 1 ? so1 : so2;
  };
  auto lst = [&](auto s) __attribute__((always_inline)) -> float* {
    constexpr int S = decltype(s)::value;
    return S == 0 ? sl0 : S == 1 ? sl1 : sl2;
  };
  auto dst = [&](auto s) __attribute__((always_inline)) -> float* {
    constexpr int S = decltype(s)::value;
    return S == 0 ? sd0 : S == 1 ? sd1 : sd2;
  };

  // Head size of the tensors: columns [dl, D) are zero-padded on chip.  The
  // kernels with compile-time strides run only at dl = D.
  const int dl = CONTIG ? D : p.dl;
  const int nb = p.num_blocks;
  // Work units: with a causal mask key block b sees nit - 2b query tiles, so a
  // unit is the pair of blocks w and nb-1-w (every unit the same work);
  // without one, a unit is one block.  The grid is persistent (one workgroup
  // per CU): each XCD takes a contiguous range of units (whole heads, whose
  // Q/dO tiles then stay in that XCD's L2), dealt round-robin to its
  // workgroups, and a workgroup walks its blocks as one chain, fetching the
  // next block's K and V rows while it works on the current one.
  // SPLIT: a unit is (block or causal pair, share s); the unit's query tiles
  // (with a pair, those of its first block followed by those of its second)
  // are divided into p.splits nearly equal shares, and share s visits each
  // block of the unit with its part of them (possibly none).
  const int per_head = CAUSAL ? (nb + 1) / 2 : nb;
  const int G = gridDim.x;
  int u, ustep, uend;
  if ((G & 7) == 0 && (p.units & 7) == 0) {
    const int x = blockIdx.x & 7, per_x = p.units >> 3;
    u = x * per_x + (blockIdx.x >> 3);
    ustep = G >> 3;
    uend = (x + 1) * per_x;
  } else {
    u = blockIdx.x;
    ustep = G;
    uend = p.units;
  }
  int sub = 0;  // which block of the unit
  auto block_of = [&](int uu, int ss, int& head_, int& jb_) {
    const int pu = SPLIT ? uu / p.splits : uu;
    head_ = pu / per_head;
    const int w = pu - head_ * per_head;
    jb_ = ss == 0 ? w : nb - 1 - w;
  };
  // Rows of batch entry b_: n_, from row r0_ on (packed sequences: its own
  // length and first row).
  auto rows_of = [&](int b_, int& n_, int64_t& r0_) {
    n_ = p.N;
    r0_ = 0;
    if (!CONTIG && p.cu) {  // packed sequences run on the run-time-stride kernels
      // wave-uniform values loaded from memory: readfirstlane keeps them in
      // scalar registers, so the buffer descriptors built from them stay
      // scalar (otherwise every buffer access becomes a loop over lanes)
      r0_ = __builtin_amdgcn_readfirstlane(p.cu[b_]);
      n_ = min(__builtin_amdgcn_readfirstlane(p.cu[b_ + 1]) - (int)r0_, p.N);
    }
  };
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, hh = lane >> 5;
  // The next block's K rows (this lane's key) land here and its V rows in skv
  // during the current block's first tile.
  V8 knext[KC];
  bool prefetched = false, started = false;
  while (u < uend) {
  if (started) __syncthreads();  // every wave is done with the previous block's LDS
  started = true;
  int head, jb;
  block_of(u, sub, head, jb);
  const int bi = head / p.H, hi = head - bi * p.H;
  int N;
  int64_t r0;
  rows_of(bi, N, r0);
  // index of row 0's LSE * log2(e) and D
  const size_t lrow0 = !CONTIG && p.cu ? (size_t)r0 * p.H + (size_t)hi * N : (size_t)head * N;
  const int nit = (N + BQ - 1) / BQ;
  // Query tiles [tlo, thi) of this visit.
  int tlo = CAUSAL ? jb * (BK / BQ) : 0, thi = nit;
  if constexpr (SPLIT) {
    const int s = u % p.splits, w = (u / p.splits) % per_head;
    if constexpr (CAUSAL) {
      const int wb = nb - 1 - w;
      const int na = nit - w * (BK / BQ), nbt = wb != w ? nit - wb * (BK / BQ) : 0;
      const int lo = (na + nbt) * s / p.splits, hi = (na + nbt) * (s + 1) / p.splits;
      if (sub == 0) {
        tlo = w * (BK / BQ) + min(lo, na);
        thi = w * (BK / BQ) + min(hi, na);
      } else {
        tlo = wb * (BK / BQ) + max(lo - na, 0);
        thi = wb * (BK / BQ) + max(hi - na, 0);
      }
    } else {
      tlo = nit * s / p.splits;
      thi = nit * (s + 1) / p.splits;
    }
  }
  const int share = SPLIT ? u % p.splits : 0;
  {
    const int w = (SPLIT ? u / p.splits : u) % per_head;
    if (CAUSAL && sub == 0 && w != nb - 1 - w) {
      sub = 1;
    } else {
      u += ustep;
      sub = 0;
    }
  }
  const bool has_next = u < uend;
  int nhead = head, njb = jb;
  if (has_next) block_of(u, sub, nhead, njb);
  const int kb = jb * BK;             // first key of the workgroup
  const int key = kb + 32 * wave + li;  // this lane's key (column of S)

  int L = N;
  if (p.key_lens) L = min(max(p.key_lens[bi], 0), N);

  // (b, h) slices through per-tensor strides
  const E* qg = (const E*)p.q + (bi * p.sq.b + hi * p.sq.h + r0 * p.sq.n);
  const E* dog = (const E*)p.dout + (bi * p.sdo.b + hi * p.sdo.h + r0 * p.sdo.n);
  E* dkg = (E*)p.dk + (bi * p.sdk.b + hi * p.sdk.h + r0 * p.sdk.n);
  E* dvg = (E*)p.dv + (bi * p.sdv.b + hi * p.sdv.h + r0 * p.sdv.n);

  // dV^T / dK^T tile u, register r -> d = 32u + 8(r/4) + 4hh + r%4; the first
  // product into each defines it.
  f32x16 dkacc[DU], dvacc[DU];
  // Keys past the key length take part in nothing: their gradients are zero.
  // Their lanes compute unmasked values (each lane's columns of S, dP, dV^T
  // and dK^T depend on its own key only), which the epilogue replaces by zeros.
  // SPLIT: partial rows of fp32 zeros also for a visit without query tiles.
  float* const dkpart = SPLIT ? p.dkp + (((size_t)share * p.heads + head) * N + key) * D : nullptr;
  float* const dvpart = SPLIT ? p.dvp + (((size_t)share * p.heads + head) * N + key) * D : nullptr;
  if (kb >= L || (SPLIT && tlo >= thi)) {  // every key of the block is padding, or no tile
    prefetched = false;  // the next block's rows are fetched at its start
    if (SPLIT && key < N) {
      const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int c = 0; c < D / 4; c += 2) {
        *(f32x4*)(dkpart + 4 * c + 4 * hh) = z;
        *(f32x4*)(dvpart + 4 * c + 4 * hh) = z;
      }
    } else if (key < N) {
      const V4 z = {(E)0.0f, (E)0.0f, (E)0.0f, (E)0.0f};
#pragma unroll
      for (int c = 0; c < D / 4; c += 2) {
        if (4 * c + 4 * hh < dl) {
          *(V4*)(dkg + (int64_t)key * (CONTIG ? D : p.sdk.n) + 4 * c + 4 * hh) = z;
          *(V4*)(dvg + (int64_t)key * (CONTIG ? D : p.sdv.n) + 4 * c + 4 * hh) = z;
        }
      }
    }
    continue;
  }

  // K and V rows of this lane's key as B operands (k = head dimension),
  // read from LDS after the block's rows have been copied in.
  V8 kreg[KC], vreg[KC];

  // Copies of Q and dO tiles with LSE*log2e and D (rows past N read as zero).
  // Row strides; CONTIG: every row is d elements after the previous one, known
  // at compile time, so tile offsets fold into constants.
  const int sqn = CONTIG ? D : (int)p.sq.n, son_ = CONTIG ? D : (int)p.sdo.n;
  const int skn = CONTIG ? D : (int)p.sk.n, svn = CONTIG ? D : (int)p.sv.n;
  const int sdkn = CONTIG ? D : (int)p.sdk.n, sdvn = CONTIG ? D : (int)p.sdv.n;
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(qg, rows_bytes(N, sqn, dl, ES));
  const __amdgpu_buffer_rsrc_t ors = make_rsrc(dog, rows_bytes(N, son_, dl, ES));
  const __amdgpu_buffer_rsrc_t lrs = make_rsrc(p.lse2 + lrow0, (uint32_t)N * 4);
  const __amdgpu_buffer_rsrc_t drs = make_rsrc(p.delta + lrow0, (uint32_t)N * 4);
  // Copy i of this lane fills chunk slot (i * NW + wave) * 64 + lane: row
  // r = i * COPY_ROWS + wave * 64 / CHUNKS + lane / CHUNKS, chunk
  // lane % CHUNKS.  The swizzle of r depends on r mod 16 only, which does not
  // change with i, so copy i is copy 0 moved by i * COPY_ROWS rows.  Per
  // tensor, the lane's part of the byte offset is ldl_*; the rest is
  // wave-uniform and is added to it.
  constexpr int COPY_ROWS = NW * 64 / C::CHUNKS;
  static_assert(COPY_ROWS % 16 == 0, "copy rows must keep their swizzle");
  const int wrow = wave * 64 / C::CHUNKS;  // wave's first row of a copy round
  uint32_t ldl_q, ldl_o;
  {
    const int r = wrow + lane / C::CHUNKS, pc = lane % C::CHUNKS;
    const int lch = (pc ^ swz<D>(r)) * 8;  // first column of the chunk this lane copies
    ldl_q = lch < dl ? (uint32_t)((lane / C::CHUNKS) * sqn + lch) * ES : kPoison;
    ldl_o = lch < dl ? (uint32_t)((lane / C::CHUNKS) * son_ + lch) * ES : kPoison;
  }
  // K rows of block (head at hoff, first key kb_) straight into registers
  // (this lane's key, rows past N read as zero), V rows into skv with the
  // tiles' coalesced copy pattern: KC + 2 * LOADS memory operations.
  constexpr int NFETCH = KC + 2 * C::LOADS;
  auto fetch_kv = [&](int head_, int kb_, V8 (&kdst)[KC]) __attribute__((always_inline)) {
    const int b_ = head_ / p.H, h_ = head_ - b_ * p.H;
    int n_;  // the rows of that block's batch entry (another one than this block's, possibly)
    int64_t r0_;
    rows_of(b_, n_, r0_);
    const __amdgpu_buffer_rsrc_t krs =
        make_rsrc((const E*)p.k + (b_ * p.sk.b + h_ * p.sk.h + r0_ * p.sk.n), rows_bytes(n_, skn, dl, ES));
    const __amdgpu_buffer_rsrc_t vrs =
        make_rsrc((const E*)p.v + (b_ * p.sv.b + h_ * p.sv.h + r0_ * p.sv.n), rows_bytes(n_, svn, dl, ES));
    const uint32_t krow = (uint32_t)(min(kb_ + 32 * wave + li, n_) * skn) * ES + (uint32_t)(16 * hh);
#pragma unroll
    for (int c = 0; c < KC; ++c)
      kdst[c] = __builtin_bit_cast(
          V8, __builtin_amdgcn_raw_buffer_load_b128(krs, 16 * c + 8 * hh < dl ? krow + 32 * c : kPoison, 0, 0));
    const int r = wrow + lane / C::CHUNKS, pc = lane % C::CHUNKS;
    const int vch = (pc ^ swz<D>(r)) * 8;
    const uint32_t vrb = (uint32_t)svn * ES;
    const uint32_t vbase = tile_offset<CONTIG>(
        vch < dl ? (uint32_t)((lane / C::CHUNKS) * svn + vch) * ES : kPoison, kb_ + wrow, vrb);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < C::LOADS; ++i)
        lds_dma16(vrs, skv + h * TILE + (i * NW + wave) * 512, vbase + (h * BQ + i * COPY_ROWS) * vrb);
  };

  // Copy piece x of tile `it` into stage s: pieces 0 .. 2*LOADS-1 are this
  // wave's Q and dO chunks, piece 2*LOADS the per-row values (waves 0-1 copy
  // LSE*log2e, waves 2-3 copy D: duplicates of the same values, no branch).
  // Tiles past the end read as zero.
  constexpr int NPIECE = 2 * C::LOADS + 1;
  // Per-lane offsets of tile it's first Q and dO copies (formed once per tile).
  const uint32_t qrb = (uint32_t)sqn * ES, orb = (uint32_t)son_ * ES;
  const uint32_t qstep = COPY_ROWS * qrb, ostep = COPY_ROWS * orb;
  struct TileAt {
    int it;
    uint32_t q, o;
  };
  auto tile_at = [&](int it) __attribute__((always_inline)) {
    return TileAt{it, tile_offset<CONTIG>(ldl_q, it * BQ + wrow, qrb),
                  tile_offset<CONTIG>(ldl_o, it * BQ + wrow, orb)};
  };
  auto issue_piece = [&](const TileAt& tl, auto s, auto x_t) __attribute__((always_inline)) {
    constexpr int x = decltype(x_t)::value;
    if constexpr (x < 2 * C::LOADS) {
      constexpr int i = x / 2;
      if constexpr (x % 2 == 0)
        lds_dma16(qrs, qst(s) + (i * NW + wave) * 512, tl.q + i * qstep);
      else
        lds_dma16(ors, ost(s) + (i * NW + wave) * 512, tl.o + i * ostep);
    } else {
      const bool dv = wave >= 2;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(dv ? drs : lrs, (lds_void_t*)(dv ? dst(s) : lst(s)), 4,
                                               (uint32_t)(tl.it * BQ + lane) * 4, 0, 0, 0);
    }
  };
  auto issue_tile = [&](int it, auto s) __attribute__((always_inline)) {
    const TileAt tl = tile_at(it);
    static_for<NPIECE>([&](auto x_t) __attribute__((always_inline)) { issue_piece(tl, s, x_t); });
  };

  // LDS element offsets of the operand reads.  Row reads (A operand of S and
  // dP): row 32a + li of a tile, logical chunk 2c + hh.  Transposing reads (A
  // operand of dV^T and dK^T): within a 16-row chunk, rows trow and trow + 8,
  // columns tcol .. tcol + 3 of a 32-column block; the k-slot x of a lane is
  // row 8(x/4) + 4hh + x%4 of the chunk, the row order of P and dS in the MFMA
  // output layout.
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
  auto row_read = [&](const E* base, int a, int c) __attribute__((always_inline)) {
    return *(const V8*)(base + roff[c] + a * 32 * D);
  };
  auto tr_read = [&](const E* base, int kc, int u) __attribute__((always_inline)) {
    const lds_bf16* b = (const lds_bf16*)base;
    const V4 lo = __builtin_bit_cast(V4, lds_read_tr4(b + toff[0][u] + 16 * kc * D));
    const V4 h4 = __builtin_bit_cast(V4, lds_read_tr4(b + toff[1][u] + 16 * kc * D));
    return V8{lo[0], lo[1], lo[2], lo[3], h4[0], h4[1], h4[2], h4[3]};
  };
  // Per-row values of group g (rows 8g + 4hh .. +3) of row half a.
  auto rows4 = [&](const float* base, int grp) __attribute__((always_inline)) {
    return *(const f32x4*)(base + 8 * grp + 4 * hh);  // grp = 4a + g
  };

  const float c2 = p.scale_log2;
  const int it0 = tlo;  // the first query tile (with a causal mask, a diagonal one unless SPLIT)

  // State carried from one tile to the next: P (fp32, masked), dP, P~ packed
  // (with dropout: P times the keep bit, the factor 1/(1-p) left to dV's
  // epilogue) as B chunks (chunk kc holds rows 16kc + 8(x/4) + 4hh + x%4 in slot x), the
  // dropout keep bits, and the operand ring.
  f32x16 sp[2], sdp[2];
  V8 spb[4];
  uint32_t zb = 0;
  V8 ring[RG];
  const f32x16 zero = {};

  // P of element pair (k, k+1) of tile `it` from its scores (in place in s),
  // packed into pb; k = 16a + r, rows 32a + 8(r/4) + 4hh + r%4.
  // Allowed iff the row offset within the tile is at least lo (and only then).
  auto exp_pair = [&](int it, f32x16 (&s)[2], V8 (&pb)[4], uint32_t& zn, int k,
                      const f32x4& l4, int lo, auto masked_t) {
    constexpr bool MASKED = decltype(masked_t)::value;
    const int a = k >> 4, r = k & 15, g = r >> 2, e = r & 3;
    float pt[2];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      float pv = fast_exp2(fmaf(s[a][r + x], c2, -l4[e + x]));
      if constexpr (MASKED) pv = (32 * a + 8 * g + e + x) >= lo ? pv : 0.0f;
      pin(pv);
      s[a][r + x] = pv;
      pt[x] = pv;
      if constexpr (DROPOUT) {
        // the keep bits of the group's four rows, drawn with the first pair
        if (e + x == 0) zn |= quad_keep4(p, it * BQ + 32 * a + 8 * g + 4 * hh, key, hi, bi) << k;
        // dropped: 0 (the factor 1/(1-p) of the kept goes to dV once, in the epilogue)
        pt[x] = __uint_as_float(__float_as_uint(pv) & bit_mask(zn, k + x));
      }
    }
    const e2 pp = __builtin_convertvector(f32x2{pt[0], pt[1]}, e2);  // one packed conversion
    pb[2 * a + (g >> 1)][4 * (g & 1) + e] = pp[0];
    pb[2 * a + (g >> 1)][4 * (g & 1) + e + 1] = pp[1];
    pin_v(pb[2 * a + (g >> 1)]);  // keep the work beside this MFMA
  };
  // Row-offset bound of the causal mask for tile `it` (see exp_pair).
  auto mask_lo = [&](int it) __attribute__((always_inline)) { return key - it * BQ - 4 * hh; };
  // dS of element pair (k, k+1) of the current tile into dsb.
  auto ds_pair = [&](V8 (&dsb)[4], int k, const f32x4& d4) {
    const int a = k >> 4, r = k & 15, g = r >> 2, e = r & 3;
    float ds[2];
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      float dp = sdp[a][r + x];
      if constexpr (DROPOUT) dp = __uint_as_float(__float_as_uint(dp * p.drop_scale) & bit_mask(zb, k + x));
      ds[x] = sp[a][r + x] * (dp - d4[e + x]);
    }
    const e2 dd = __builtin_convertvector(f32x2{ds[0], ds[1]}, e2);  // one packed conversion
    dsb[2 * a + (g >> 1)][4 * (g & 1) + e] = dd[0];
    dsb[2 * a + (g >> 1)][4 * (g & 1) + e + 1] = dd[1];
    pin_v(dsb[2 * a + (g >> 1)]);  // keep the work beside this MFMA
  };

  // ---- prologue: tiles it0 (stage 0) and it0 + 1 (stage 1); S, dP and P of
  // tile it0; the first operands of its body.
  if (prefetched) {
#pragma unroll
    for (int c = 0; c < KC; ++c) kreg[c] = knext[c];
  } else {
    fetch_kv(head, kb, kreg);
  }
  issue_tile(it0, Stage<0>{});
  issue_tile(it0 + 1, Stage<1>{});
  // Loads complete in issue order: once at most tile it0+1's pieces are
  // outstanding, the block's K/V rows and this wave's share of tile it0 have
  // landed.  Tile it0+1 is awaited after the prologue's products.
  wait_vmem_le<NPIECE>();
  __syncthreads();
  {
    // V rows 32 * wave .. +31 of the block: 64-row tile wave / 2, half wave % 2.
    const E* vt = skv + (wave >> 1) * TILE;
#pragma unroll
    for (int c = 0; c < KC; ++c) vreg[c] = row_read(vt, wave & 1, c);
  }
  {
    const E* q = qst(Stage<0>{});
    const E* o = ost(Stage<0>{});
    constexpr int NS = 2 * NP;  // S halves, then dP halves
    auto pread = [&](int i) __attribute__((always_inline)) {
      const int m = i / KC, c = i % KC;
      return row_read(m < 2 ? q : o, m & 1, c);
    };
    V8 pr[3];
    pr[0] = pread(0);
    pr[1] = pread(1);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      if (i + 2 < NS) pr[(i + 2) % 3] = pread(i + 2);
      const int m = i / KC, c = i % KC;
      f32x16& acc = m < 2 ? sp[m & 1] : sdp[m & 1];
      acc = Elem<E>::mma(pr[i % 3], m < 2 ? kreg[c] : vreg[c], c == 0 ? zero : acc);
    }
    const float* ls = lst(Stage<0>{});
    const int lo = mask_lo(it0);
#pragma unroll
    for (int k = 0; k < 32; k += 2) {
      const f32x4 l4 = rows4(ls, k >> 2);
      exp_pair(it0, sp, spb, zb, k, l4, lo, std::integral_constant<bool, CAUSAL>{});
    }
#pragma unroll
    for (int i = 0; i < PD; ++i) ring[i] = tr_read(o, i / DU, i % DU);
    wait_vmem();  // this wave's share of tile it0+1, before the first body's barrier
  }

  // ---- one tile: t in stage S, t+1 in stage S+1.  The body after the last
  // tile also computes S, dP and P of a tile t+1 = thi, from whatever its
  // stage holds; the loop ends before anything reads them.
  auto body = [&](int t, auto s_t, auto mask_next_t, auto first_t) __attribute__((always_inline)) {
    constexpr int S = decltype(s_t)::value;
    constexpr bool FIRST = decltype(first_t)::value;  // the first tile defines dK^T, dV^T
    using S1 = Stage<S + 1>;
    using S2 = Stage<S + 2>;
    constexpr int NOPS = 4 * NP;
    const E* qt = qst(s_t);
    const E* ot = ost(s_t);
    const E* qn = qst(S1{});
    const E* on = ost(S1{});
    const float* dt = dst(s_t);
    const float* ln = lst(S1{});
    __syncthreads();  // tile t+1 resident; every wave is done with tile t-1

    // A operand of MFMA i of this body; i >= NOPS: of the next body's first ones.
    auto aread = [&](auto i_t) __attribute__((always_inline)) -> V8 {
      constexpr int i = decltype(i_t)::value;
      constexpr int ph = i / NP, j = i % NP;
      if constexpr (i >= NOPS) return tr_read(on, (i - NOPS) / DU, (i - NOPS) % DU);
      else if constexpr (ph == 0) return tr_read(ot, j / DU, j % DU);
      else if constexpr (ph == 1) return row_read(qn, j / KC, j % KC);
      else if constexpr (ph == 2) return tr_read(qt, j / DU, j % DU);
      else return row_read(on, j / KC, j % KC);
    };
    f32x16 sn[2], pn[2];
    V8 dsb[4], pbn[4];
    uint32_t zn = 0;
    const int lo = mask_lo(t + 1);
    // elementwise work: dS pairs during phases 0-1, P pairs during phases 2-3,
    // 8 pairs per phase; the per-row values are read one group ahead
    f32x4 dv4[8], lv4[8];
    dv4[0] = rows4(dt, 0);
    lv4[0] = rows4(ln, 0);
    auto valu = [&](auto i_t) __attribute__((always_inline)) {
      constexpr int i = decltype(i_t)::value;
      constexpr int ph = i / NP, j = i % NP;
      constexpr int b0 = ((ph & 1) * NP + j) * 8 / NP, b1 = ((ph & 1) * NP + j + 1) * 8 / NP;
      static_for<b1 - b0>([&](auto x_t) __attribute__((always_inline)) {
        constexpr int b = b0 + decltype(x_t)::value, grp = b >> 1;
        if constexpr (ph <= 1) {
          if constexpr ((b & 1) == 0 && grp + 1 < 8) dv4[grp + 1] = rows4(dt, grp + 1);
          ds_pair(dsb, 2 * b, dv4[grp]);
        } else {
          if constexpr ((b & 1) == 0 && grp + 1 < 8) lv4[grp + 1] = rows4(ln, grp + 1);
          exp_pair(t + 1, sn, pbn, zn, 2 * b, lv4[grp], lo, mask_next_t);
        }
      });
    };
    const TileAt tn = tile_at(t + 2);  // this body's copies
    __builtin_amdgcn_sched_barrier(0);
    static_for<NOPS>([&](auto i_t) __attribute__((always_inline)) {
      constexpr int i = decltype(i_t)::value;
      constexpr int pre = i + PD;
      ring[pre % RG] = aread(std::integral_constant<int, pre>{});
      // copies of tile t+2, one piece every other MFMA (a burst of them
      // stalls the wave on the full memory queue)
      if constexpr (i % 2 == 0 && i / 2 < NPIECE)
        issue_piece(tn, S2{}, std::integral_constant<int, i / 2>{});
      constexpr int ph = i / NP, j = i % NP;
      const V8& a = ring[i % RG];
      if constexpr (ph == 0) {
        if constexpr (FIRST && j / DU == 0)
          Elem<E>::mma_acc_first(dvacc[j % DU], a, spb[j / DU]);
        else
          Elem<E>::mma_acc(dvacc[j % DU], a, spb[j / DU]);
      } else if constexpr (ph == 1) {
        sn[j / KC] = Elem<E>::mma(a, kreg[j % KC], j % KC == 0 ? zero : sn[j / KC]);
      } else if constexpr (ph == 2) {
        if constexpr (FIRST && j / DU == 0)
          Elem<E>::mma_acc_first(dkacc[j % DU], a, dsb[j / DU]);
        else
          Elem<E>::mma_acc(dkacc[j % DU], a, dsb[j / DU]);
      } else {
        pn[j / KC] = Elem<E>::mma(a, vreg[j % KC], j % KC == 0 ? zero : pn[j / KC]);
      }
      // the operands of the AccVGPR-form MFMAs of ops i-1 .. i-3 stay live
      // until here: the MFMAs of two later ops (whole groups before this one)
      // have issued since op i-3's
      static_for<3>([&](auto d_t) __attribute__((always_inline)) {
        constexpr int k = i - 1 - decltype(d_t)::value, kph = k / NP, kj = k % NP;
        if constexpr (k >= 0 && (kph == 0 || kph == 2)) {
          keep_v(ring[k % RG]);
          keep_v(kph == 0 ? spb[kj / DU] : dsb[kj / DU]);
        }
      });
      valu(i_t);
      __builtin_amdgcn_sched_barrier(0);
    });
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      sp[a] = sn[a];
      sdp[a] = pn[a];
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) spb[c] = pbn[c];
    zb = zn;
    if (FIRST && !DROPOUT && has_next) {
      // The next block's K/V rows, issued after this body's copies: they may
      // stay in flight until the end of the next body (skv is free: every
      // wave read its V rows before this body's barrier).  Not with dropout,
      // whose keep-mask state leaves no registers for them.
      fetch_kv(nhead, njb * BK, knext);
      wait_vmem_le<NFETCH>();  // tile t+2 landed (this wave's share)
    } else {
      wait_vmem();  // tile t+2 landed (this wave's share) before the next barrier
    }
  };

  // With a causal mask the block's diagonal spans its first two tiles: the
  // prologue masks the first, the first body the second.  (A split visit
  // starting past them masks nothing there.)
  using CausalT = std::integral_constant<bool, CAUSAL>;
  body(it0, Stage<0>{}, CausalT{}, T_{});
  for (int t = it0 + 1;; t += 3) {
    if (t >= thi) break;
    body(t, Stage<1>{}, F_{}, F_{});
    if (t + 1 >= thi) break;
    body(t + 1, Stage<2>{}, F_{}, F_{});
    if (t + 2 >= thi) break;
    body(t + 2, Stage<0>{}, F_{}, F_{});
  }
  // the last accumulate MFMAs complete before the VALU reads dK^T and dV^T
  settle_acc(dkacc[0]);
#pragma unroll
  for (int u = 0; u < DU; ++u) {
    if (u) tie_acc(dkacc[u]);
    tie_acc(dvacc[u]);
  }
  // dK = scale * dK^T^T and dV through LDS (stages 0 and 1 are free once every
  // wave is past the last tile), then whole rows to memory.  Keys past the key
  // length get zeros; rows past N are not written.  SPLIT: fp32 partial rows,
  // straight from the accumulators.
  if constexpr (SPLIT) {
    if (key < N) {
      acc_row_to_f32<D>(dkpart, dkacc, p.scale, key >= L, hh);
      acc_row_to_f32<D>(dvpart, dvacc, DROPOUT ? p.drop_scale : 1.0f, key >= L, hh);
    }
  } else {
    __syncthreads();
    const bool zero = key >= L;
    E* kt = ((wave >> 1) ? so0 : sq0) + (wave & 1) * 32 * D;
    E* vt = ((wave >> 1) ? so1 : sq1) + (wave & 1) * 32 * D;
    acc_rows_to_lds<D, E>(kt, dkacc, p.scale, zero, li, hh);
    acc_rows_to_lds<D, E>(vt, dvacc, DROPOUT ? p.drop_scale : 1.0f, zero, li, hh);
    const int row0 = kb + 32 * wave;
    lds_rows_to_buffer<D, E>(kt, dkg + (int64_t)row0 * sdkn, sdkn, N - row0, lane, dl);
    lds_rows_to_buffer<D, E>(vt, dvg + (int64_t)row0 * sdvn, sdvn, N - row0, lane, dl);
  }
  prefetched = !DROPOUT && has_next;
  }  // block
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

template <typename E, int D, bool CAUSAL, bool DROPOUT, bool CONTIG, bool SPLIT>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 2)))
void bwd_dq_kernel(BwdParams p) {
  using C = QCfg<D>;
  using V8 = typename Elem<E>::v8;
  using V4 = typename Elem<E>::v4;
  constexpr int ES = 2;
  constexpr int BN = C::BN, NW = C::NW, TILE = C::TILE;
  constexpr int KC = D / 16;
  constexpr int DU = D / 32;
  __shared__ __attribute__((aligned(1024))) E sk0[TILE];
  __shared__ __attribute__((aligned(1024))) E sk1[TILE];
  __shared__ __attribute__((aligned(1024))) E sv0[TILE];
  __shared__ __attribute__((aligned(1024))) E sv1[TILE];

  // Head size of the tensors: columns [dl, D) are zero-padded on chip.  The
  // kernels with compile-time strides run only at dl = D.
  const int dl = CONTIG ? D : p.dl;
  const int nqb = p.num_blocks;
  // Causal: a workgroup takes query blocks nqb-1-w and w in turn (equal work).
  // SPLIT: p.splits workgroups per such unit, workgroup s taking share s of
  // each block's key tiles and writing fp32 partial dQ rows.
  const int per_head = CAUSAL ? (nqb + 1) / 2 : nqb;
  int lid = xcd_remap(blockIdx.x, gridDim.x);
  int share = 0;
  if constexpr (SPLIT) {
    share = lid % p.splits;
    lid /= p.splits;
  }
  const int head = lid / per_head;
  const int w = lid - head * per_head;
  const int nitems = CAUSAL && w != nqb - 1 - w ? 2 : 1;
  const int bi = head / p.H, hi = head - bi * p.H;
  // Rows of this batch entry: N, from row r0 on (packed sequences: its own
  // length and first row).
  int N = p.N;
  int64_t r0 = 0;
  if (!CONTIG && p.cu) {  // packed sequences run on the run-time-stride kernels
    // wave-uniform values loaded from memory: readfirstlane keeps them in
    // scalar registers, so the buffer descriptors built from them stay
    // scalar (otherwise every buffer access becomes a loop over lanes)
    r0 = __builtin_amdgcn_readfirstlane(p.cu[bi]);
    N = min(__builtin_amdgcn_readfirstlane(p.cu[bi + 1]) - (int)r0, p.N);
  }
  // index of row 0's LSE, D and LSE * log2(e)
  const size_t lrow0 = !CONTIG && p.cu ? (size_t)r0 * p.H + (size_t)hi * N : (size_t)head * N;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, hh = lane >> 5;
  // (b, h) slices through per-tensor strides (both items of a workgroup are
  // in the same head)
  const E* qg = (const E*)p.q + (bi * p.sq.b + hi * p.sq.h + r0 * p.sq.n);
  const E* kg = (const E*)p.k + (bi * p.sk.b + hi * p.sk.h + r0 * p.sk.n);
  const E* vg = (const E*)p.v + (bi * p.sv.b + hi * p.sv.h + r0 * p.sv.n);
  const E* dog = (const E*)p.dout + (bi * p.sdo.b + hi * p.sdo.h + r0 * p.sdo.n);
  const E* og = (const E*)p.o + (bi * p.so.b + hi * p.so.h + r0 * p.so.n);
  E* dqg = (E*)p.dq + (bi * p.sdq.b + hi * p.sdq.h + r0 * p.sdq.n);
  // Row strides (CONTIG: d, known at compile time).
  const int sqn = CONTIG ? D : (int)p.sq.n, skn = CONTIG ? D : (int)p.sk.n;
  const int svn = CONTIG ? D : (int)p.sv.n, son_ = CONTIG ? D : (int)p.sdo.n;
  const int son_o = CONTIG ? D : (int)p.so.n, sdqn = CONTIG ? D : (int)p.sdq.n;
  for (int item = 0; item < nitems; ++item) {
  if (item) __syncthreads();  // every wave is done with the first block's tiles
  const int qb = CAUSAL ? (item == 0 ? nqb - 1 - w : w) : w;
  const int q0 = qb * C::BM;
  if (q0 >= N) continue;  // a packed sequence shorter than the longest
  const int qi = q0 + wave * 32 + li;  // this lane's query

  int L = N;
  if (p.key_lens) L = min(max(p.key_lens[bi], 0), N);
  const int kend = CAUSAL ? min(L, q0 + C::BM) : L;
  const int nkb = (kend + BN - 1) / BN;
  // Tiles [0, nfree) are unmasked for every query of the workgroup.
  int nfree = L / BN;
  if (CAUSAL) nfree = min(nfree, q0 / BN);
  nfree = min(nfree, nkb);

  // Q^T and dO^T as B operands (k = head dimension): lane holds row qi,
  // elements 16c + 8hh .. +7, read from LDS after the block's rows have been
  // copied in (below).
  V8 qreg[KC], oreg[KC];

  // The copies cover the tiles [0, nkb) only: copies past them (issued without
  // a branch) read zeros without touching memory.
  const int krows = min(nkb * BN, N);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kg, rows_bytes(krows, skn, dl, ES));
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vg, rows_bytes(krows, svn, dl, ES));
  // Copy i of this lane fills chunk slot (i * NW + wave) * 64 + lane, i.e.
  // row i * COPY_ROWS + wave * 64 / CHUNKS + lane / CHUNKS, chunk
  // lane % CHUNKS.  The swizzle depends on the row mod 16, which does not
  // change with i, so copy i is copy 0 moved by i * COPY_ROWS rows.  Per
  // tensor, the lane's part of the byte offset is ldl_*; the rest is
  // wave-uniform and is added to it.
  constexpr int COPY_ROWS = NW * 64 / C::CHUNKS;
  static_assert(COPY_ROWS % 16 == 0, "copy rows must keep their swizzle");
  const int wrow = wave * 64 / C::CHUNKS;
  uint32_t ldl_k, ldl_v;
  int crow, lch;  // this lane's row within a copy round and its chunk's element offset
  {
    const int r = wrow + lane / C::CHUNKS, pc = lane % C::CHUNKS;
    crow = lane / C::CHUNKS;
    lch = (pc ^ swz<D>(r)) * 8;  // first column of the chunk this lane copies
    ldl_k = lch < dl ? (uint32_t)(crow * skn + lch) * ES : kPoison;
    ldl_v = lch < dl ? (uint32_t)(crow * svn + lch) * ES : kPoison;
  }
  // Per-lane offsets of tile jt's first K and V copies (formed once per tile).
  const uint32_t krb = (uint32_t)skn * ES, vrb = (uint32_t)svn * ES;
  const uint32_t kstep = COPY_ROWS * krb, vstep = COPY_ROWS * vrb;
  struct TileAt {
    uint32_t k, v;
  };
  auto tile_at = [&](int jt) {
    return TileAt{tile_offset<CONTIG>(ldl_k, jt * BN + wrow, krb), tile_offset<CONTIG>(ldl_v, jt * BN + wrow, vrb)};
  };
  // Copy piece x of a tile (x < LOADS: K, else V) into stage S.
  auto issue_piece = [&](const TileAt& tl, auto par_t, int x) {
    constexpr int S = decltype(par_t)::value;
    const int i = x % C::LOADS;
    if (x < C::LOADS)
      lds_dma16(krs, (S ? sk1 : sk0) + (i * NW + wave) * 512, tl.k + i * kstep);
    else
      lds_dma16(vrs, (S ? sv1 : sv0) + (i * NW + wave) * 512, tl.v + i * vstep);
  };
  auto issue = [&](int jt, auto par_t) {
    const TileAt tl = tile_at(jt);
#pragma unroll
    for (int x = 0; x < 2 * C::LOADS; ++x) issue_piece(tl, par_t, x);
  };
  // Row reads of K and V tiles (A operands of S^T and dP^T): row 32t + li,
  // logical chunk 2c + hh.  Transposing reads of the K tile (A operand of
  // dQ^T = K^T dS^T): rows 16cc + trow (+8), columns 32u + tcol.
  const int rsw = swz<D>(li);
  int roff[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) roff[c] = li * D + (((2 * c + hh) ^ rsw) * 8);
  {
    // The block's Q rows go through the K stages and its dO rows through the
    // V stages (two 64-row tiles each) with the tiles' coalesced copies (rows
    // past N read as zero); every wave then reads its rows into registers.
    // Loading them straight into registers, a lane per row, cost more than
    // this whole round trip.  The stages are free again after the barrier.
    const __amdgpu_buffer_rsrc_t qrs = make_rsrc(qg, rows_bytes(N, sqn, dl, ES));
    const __amdgpu_buffer_rsrc_t ors = make_rsrc(dog, rows_bytes(N, son_, dl, ES));
    const uint32_t ldl_q = lch < dl ? (uint32_t)(crow * sqn + lch) * ES : kPoison;
    const uint32_t ldl_o = lch < dl ? (uint32_t)(crow * son_ + lch) * ES : kPoison;
    const uint32_t qrb = (uint32_t)sqn * ES, orb = (uint32_t)son_ * ES;
    const uint32_t qb = tile_offset<CONTIG>(ldl_q, q0 + wrow, qrb), ob = tile_offset<CONTIG>(ldl_o, q0 + wrow, orb);
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      lds_dma16(qrs, sk0 + (i * NW + wave) * 512, qb + (i * COPY_ROWS) * qrb);
      lds_dma16(qrs, sk1 + (i * NW + wave) * 512, qb + (i * COPY_ROWS + BN) * qrb);
      lds_dma16(ors, sv0 + (i * NW + wave) * 512, ob + (i * COPY_ROWS) * orb);
      lds_dma16(ors, sv1 + (i * NW + wave) * 512, ob + (i * COPY_ROWS + BN) * orb);
    }
    wait_vmem();
    __syncthreads();
    const E* qt = ((wave >> 1) ? sk1 : sk0) + (wave & 1) * 32 * D;
    const E* ot = ((wave >> 1) ? sv1 : sv0) + (wave & 1) * 32 * D;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      qreg[c] = *(const V8*)(qt + roff[c]);
      oreg[c] = *(const V8*)(ot + roff[c]);
    }
    __syncthreads();  // every wave has its rows before the first K/V tile lands there
  }
  // The per-row terms of this lane's query: D = sum_k dO_k O_k (each of the
  // two lanes of a row holds half of the row's dO) and LSE * log2(e).  Rows
  // past N or without any allowed key get +inf, which makes every P vanish.
  // Both go to the workspace, where the dK/dV stage reads them.
  float drow = 0.0f, lrow = INFINITY;
  if (qi < N) {
    const E* orow = og + (int64_t)qi * son_o + 8 * hh;
#pragma unroll
    for (int c = 0; c < KC; ++c)
      if (16 * c + 8 * hh < dl) drow = Elem<E>::dot8(*(const V8*)(orow + 16 * c), oreg[c], drow);
    const float lv = p.lse[lrow0 + qi];
    lrow = lv == -INFINITY ? INFINITY : lv * kLog2e;
  }
  drow = pair_sum(drow);
  if (hh == 0 && qi < N && share == 0) {
    p.delta[lrow0 + qi] = drow;
    p.lse2[lrow0 + qi] = lrow;
  }
  // Without dropout (dS = P (Z dP - D) otherwise) and where the registers
  // allow it (width 64; at 128 the block of 16 spills into the loop), the dP
  // chains start from -D: the accumulator below, every register this lane's row.
  constexpr bool NEGD = !DROPOUT && D == 64;
  f32x16 negd;
#pragma unroll
  for (int r = 0; r < 16; ++r) negd[r] = NEGD ? -drow : 0.0f;
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
    const E* ks = S ? sk1 : sk0;
    const E* vs = S ? sv1 : sv0;
    __syncthreads();  // tile j resident; every wave is done with tile j-1

    // ---- S^T = K Q^T and dP^T = V dO^T: key tile t (32 keys), k-step c.
    // NEGD: the dP chains start from -D (one row per lane), so they end at
    // dP - D and dS = P (dP - D) is one multiply.
    f32x16 sacc[2], pacc[2];
    const f32x16 zero = {};
    constexpr int NS = 4 * KC;
    V8 ring[3];
    const TileAt tn = tile_at(j + 1);  // this tile's copies of the next one
    auto sread = [&](int i) {
      const int m = i / KC, c = i % KC;
      return *(const V8*)((m < 2 ? ks : vs) + roff[c] + (m & 1) * 32 * D);
    };
    // Priority while this wave's exponentials and dS are on the critical
    // path: the other workgroup's wave on the SIMD, in its dQ products,
    // fills the gaps.
    __builtin_amdgcn_s_setprio(3);
    ring[0] = sread(0);
    ring[1] = sread(1);
    __builtin_amdgcn_sched_barrier(0);
    V8 dsb[4];  // dS^T as B operands: chunk cc holds keys 16cc + 8(x/4) + 4hh + x%4
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
        if constexpr (NEGD) {
          dsb[2 * t + (g >> 1)][4 * (g & 1) + e] = (E)(sacc[t][r] * pacc[t][r]);
        } else {
          float dp = pacc[t][r];
          if constexpr (DROPOUT) dp *= dropout_z(p, qi, j * BN + 32 * t + 8 * g + 4 * hh + e, hi, bi);
          dsb[2 * t + (g >> 1)][4 * (g & 1) + e] = (E)(sacc[t][r] * (dp - drow));
        }
      }
    };
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      // copies of tile j+1, one every other MFMA (a burst of them stalls the
      // wave on the full memory queue); a tile past the end reads as zero
      // into a stage nothing reads again
      if (i % 2 == 0 && i / 2 < 2 * C::LOADS)
        issue_piece(tn, std::integral_constant<int, S ^ 1>{}, i / 2);
      if (i + 2 < NS) ring[(i + 2) % 3] = sread(i + 2);
      const int m = i / KC, c = i % KC;
      f32x16& acc = m < 2 ? sacc[m & 1] : pacc[m & 1];
      acc = Elem<E>::mma(ring[i % 3], m < 2 ? qreg[c] : oreg[c],
                         c == 0 ? (m >= 2 && NEGD ? negd : zero) : acc);
      if ((c * 4) % KC == 0) {
        const int g = c * 4 / KC;
        if (m == 1) p_elems(0, g);
        if (m == 2) p_elems(1, g);
        if (m == 3) ds_elems(0, g);
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- dQ^T += K^T dS^T (contraction over the 64 keys)
    __builtin_amdgcn_s_setprio(0);
    const lds_bf16* kt = (const lds_bf16*)ks;
    constexpr int NQ = 4 * DU;  // index = (cc, u)
    auto tnext = [&](int i) {
      const int cc = i / DU, u = i % DU;
      const V4 lo = __builtin_bit_cast(V4, lds_read_tr4(kt + toff[0][u] + 16 * cc * D));
      const V4 h4 = __builtin_bit_cast(V4, lds_read_tr4(kt + toff[1][u] + 16 * cc * D));
      return V8{lo[0], lo[1], lo[2], lo[3], h4[0], h4[1], h4[2], h4[3]};
    };
    ring[0] = tnext(0);
    ring[1] = tnext(1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      if (i + 2 < NQ) ring[(i + 2) % 3] = tnext(i + 2);
      const int cc = i / DU, u = i % DU;
      qacc[u] = Elem<E>::mma(ring[i % 3], dsb[cc], qacc[u]);
      // chunks 2, 3 (key tile 1) are first used by MFMA 2*DU
      if (i < 4) ds_elems(1, i);
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_vmem();
  };

  // Key tiles [jlo, jhi) of this workgroup (SPLIT: its share of [0, nkb)).
  int jlo = 0, jhi = nkb;
  if constexpr (SPLIT) {
    jlo = nkb * share / p.splits;
    jhi = nkb * (share + 1) / p.splits;
  }
  if (jlo < jhi) {
    issue(jlo, P0{});
    wait_vmem();
  }
  // Unmasked tiles first (from key tile jlo), then the masked diagonal / tail
  // ones.  Steps run in pairs from jlo so the stage parity is a compile-time
  // constant; tiles in [jm, nfree) take the masked path (harmless, it only
  // masks nothing there).
  const int jm = jlo + ((min(max(nfree, jlo), jhi) - jlo) & ~1);
  int j = jlo;
  for (; j < jm; j += 2) {
    step(j, P0{}, F_{});
    step(j + 1, P1{}, F_{});
  }
  for (; j + 1 < jhi; j += 2) {
    step(j, P0{}, T_{});
    step(j + 1, P1{}, T_{});
  }
  if (j < jhi) step(j, P0{}, T_{});

  // dQ = scale * dQ^T^T, transposed through the K stages (free once every
  // wave is past the last tile) and written as whole rows.  SPLIT: fp32
  // partial rows, straight from the accumulators (zeros without a tile).
  if constexpr (SPLIT) {
    if (qi < N)
      acc_row_to_f32<D>(p.dqp + (((size_t)share * p.heads + head) * N + qi) * D, qacc, p.scale, false,
                        hh);
  } else {
    __syncthreads();
    const int qw = q0 + wave * 32;
    E* qt = ((wave >> 1) ? sk1 : sk0) + (wave & 1) * 32 * D;
    acc_rows_to_lds<D, E>(qt, qacc, p.scale, false, li, hh);
    lds_rows_to_buffer<D, E>(qt, dqg + (int64_t)qw * sdqn, sdqn, N - qw, lane, dl);
  }
  }  // item
}

// D_i = sum_k dO_ik O_ik and LSE_i * log2(e) (+inf for an empty row, so that
// the recomputed probabilities exp2(s - LSE*log2e) vanish).  D/8 lanes per row.
template <typename E, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdParams p, int64_t rows) {
  typedef E v8 __attribute__((ext_vector_type(8)));
  constexpr int LPR = D / 8;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = t / LPR;
  const int ch = (int)(t % LPR);
  float s = 0.0f;
  if (row < rows && ch * 8 < p.dl) {
    const int head = (int)(row / p.N), n = (int)(row - (int64_t)head * p.N);
    const int bi = head / p.H, hi = head - bi * p.H;
    const v8 ov = *(const v8*)((const E*)p.o + (bi * p.so.b + hi * p.so.h + (int64_t)n * p.so.n) +
                               ch * 8);
    const v8 dv = *(const v8*)((const E*)p.dout +
                               (bi * p.sdo.b + hi * p.sdo.h + (int64_t)n * p.sdo.n) + ch * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) s = fmaf((float)ov[e], (float)dv[e], s);
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, LPR);
  if (row < rows && ch == 0) {
    p.delta[row] = s;
    const float lv = p.lse[row];
    p.lse2[row] = lv == -INFINITY ? INFINITY : lv * kLog2e;
  }
}

// Split backward: dQ, dK and dV = the sums of the splits' fp32 partial rows,
// converted to the element type and written through the output strides.  One
// thread per 8 elements of a row.
template <typename E, int D>
__global__ __launch_bounds__(256) void bwd_combine_kernel(BwdParams p, int64_t rows) {
  typedef E v8 __attribute__((ext_vector_type(8)));
  constexpr int LPR = D / 8;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = t / LPR;
  if (row >= rows) return;
  const int ch = (int)(t % LPR);
  const int head = (int)(row / p.N), n = (int)(row - (int64_t)head * p.N);
  const int bi = head / p.H, hi = head - bi * p.H;
  const size_t split_stride = (size_t)rows * D;
  auto sum8 = [&](const float* part) {
    f32x4 a = {0.0f, 0.0f, 0.0f, 0.0f}, b = a;
    const float* x = part + (size_t)row * D + ch * 8;
    for (int s = 0; s < p.splits; ++s) {
      a += *(const f32x4*)(x + s * split_stride);
      b += *(const f32x4*)(x + s * split_stride + 4);
    }
    v8 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      r[e] = (E)a[e];
      r[4 + e] = (E)b[e];
    }
    return r;
  };
  if (p.dqp) *(v8*)((E*)p.dq + (bi * p.sdq.b + hi * p.sdq.h + (int64_t)n * p.sdq.n) + ch * 8) = sum8(p.dqp);
  if (p.dkp) *(v8*)((E*)p.dk + (bi * p.sdk.b + hi * p.sdk.h + (int64_t)n * p.sdk.n) + ch * 8) = sum8(p.dkp);
  if (p.dvp) *(v8*)((E*)p.dv + (bi * p.sdv.b + hi * p.sdv.h + (int64_t)n * p.sdv.n) + ch * 8) = sum8(p.dvp);
}

}  // namespace
}  // namespace fa
