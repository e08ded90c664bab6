// Forward pass of exact attention on gfx950.
//
// O = softmax(mask(scale * Q K^T)) (with dropout) V and the per-row
// LSE = m + ln(l), computed tile by tile: each workgroup keeps a block of
// queries resident, streams K/V tiles through LDS, and keeps a running row max
// m and row sum l, rescaling the partial output when m grows (ML Canon 48
// FlashAttention, "tiling and online softmax").  The N x N scores exist only as
// one register tile at a time (FlashAttention first principles, section 4.2, explains
// why the row-wise softmax otherwise forces them into device memory).
//
// bf16 path, per workgroup of 4 waves x 32 queries, two workgroups per CU:
//  * Each wave computes the transposed score tile S^T = K Q^T with
//    v_mfma_f32_32x32x16_bf16: Q^T is the B operand held in registers for the
//    whole loop, K rows the A operand read from LDS.  In that layout a lane
//    holds the scores of ONE query against 16 keys of each 32-key block (its
//    partner lane l^32 the other 16), so the row max/sum is a per-lane
//    reduction plus one permlane32 swap, and the probabilities, converted to
//    bf16, are already the B operand of O^T += V^T P^T.  V^T comes from the
//    row-major V tile through the LDS transposing read.
//  * K and V tiles (64 keys) are copied global -> LDS directly by buffer loads
//    (no register staging), double buffered, with an XOR swizzle of the
//    16-byte chunks of each row that keeps both the row reads of K and the
//    transposing reads of V free of bank conflicts.  Rows past N read as zero.
//  * Software pipeline: while the MFMAs of the next tile's scores run, the
//    VALU works on the current tile's exponentials; the next tile's row max is
//    taken while the P V products run.
//  * Lazy rescaling: the reference max used in the exponent only moves when a
//    row max exceeds it by more than 2^8 (in base-2 units), so the rescale of
//    the output accumulator is a rare, wave-uniform branch.  Numerators and
//    the denominator always use the same reference, so the result is the same
//    softmax; probabilities stay below 2^8 before normalisation.
#include <type_traits>

#include "fa_common.hpp"
#include "fa_internal.hpp"

namespace fa {
namespace {

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;  // contiguous [B, H, N]
  const int32_t* key_lens;
  // Packed sequences (nullptr otherwise): batch entry b is rows [cu[b],
  // cu[b+1]) of every tensor (at most N of them; the batch strides are 0),
  // and its LSE the [H, len] block at H * cu[b].
  const int32_t* cu;
  Strides sq, sk, sv, so;  // element strides (batch, head, row); d is contiguous
  int H, N, num_qblocks;
  int dl;  // head size of the tensors, <= D: columns [dl, D) read as zero and are not written
  int b0;  // added to the batch index in the dropout counter
  float scale_log2;  // scale * log2(e): scores enter exp2 in these units
  uint32_t drop_threshold;
  float drop_scale;
  uint32_t seed_lo, seed_hi;
  // Split-KV only: the key tiles of each query block are split num_splits
  // ways; split s writes its normalised fp32 output and its LSE to
  // opart[s][head][row][:] and lsepart[s][head][row] (head = b * H + h).
  float* opart;
  float* lsepart;
  int num_splits, heads;
};

template <int D>
struct FwdCfg {
  static constexpr int NW = 4;                  // waves per workgroup
  static constexpr int THREADS = NW * 64;
  static constexpr int BM = 32 * NW;            // queries per workgroup
  static constexpr int BN = 64;                 // keys per K/V tile
  static constexpr int CHUNKS = D / 8;          // 16-byte chunks per row
  static constexpr int TILE = BN * D;           // elements per K or V tile
  static constexpr int LOADS = BN * CHUNKS / THREADS;  // 16-byte copies per thread per tile
  static constexpr int COPY_ROWS = THREADS / CHUNKS;   // tile rows one copy round covers
  static_assert(LOADS * THREADS == BN * CHUNKS, "tile/thread mismatch");
};

// Waves per SIMD: two, or three at d = 64 without a causal mask or dropout,
// whose registers then fit 168 per lane without spills (LDS: 32 KB per
// workgroup).  The d = 64 loop has half the MFMA work of d = 128 per score
// but the same exponentials, sums and maxima, so a third wave to overlap
// them pays.
template <int D, bool CAUSAL, bool DROPOUT>
constexpr int fwd_waves() { return D == 64 && !CAUSAL && !DROPOUT ? 3 : 2; }

template <typename E, int D, bool CAUSAL, bool DROPOUT, bool SPLIT, bool CONTIG>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256),
                          amdgpu_waves_per_eu(fwd_waves<D, CAUSAL, DROPOUT>(),
                                              fwd_waves<D, CAUSAL, DROPOUT>())))
void fwd_kernel(FwdParams p) {
  using C = FwdCfg<D>;
  using V8 = typename Elem<E>::v8;
  using V4 = typename Elem<E>::v4;
  constexpr int ES = 2;  // bytes per element
  constexpr int BN = C::BN, NW = C::NW, TILE = C::TILE;
  constexpr int KC = D / 16;  // MFMA k-steps over the head dimension
  constexpr int DU = D / 32;  // 32-wide blocks of the head dimension
  // K and V tiles, two stages each.  Separate objects let the compiler see
  // that a copy into one stage cannot alias reads of another, so it does not
  // make those reads wait for the copy.
  __shared__ __attribute__((aligned(1024))) E sk0[TILE];
  __shared__ __attribute__((aligned(1024))) E sk1[TILE];
  __shared__ __attribute__((aligned(1024))) E sv0[TILE];
  __shared__ __attribute__((aligned(1024))) E sv1[TILE];
  auto kbuf = [&](int stage) -> E* { return stage ? sk1 : sk0; };
  auto vbuf = [&](int stage) -> E* { return stage ? sv1 : sv0; };

  // Head size of the tensors: columns [dl, D) are zero-padded on chip.  The
  // kernels with compile-time strides run only at dl = D.
  const int dl = CONTIG ? D : p.dl;
  const int nqb = p.num_qblocks;
  // With a causal mask query block b costs b + 1 key tiles: a workgroup takes
  // blocks nqb-1-w and w in turn, so every workgroup does the same work (no
  // stragglers at the end of the grid, half as many workgroup start-ups).
  // Split-KV: one query block per workgroup, the block's key tiles split
  // num_splits ways (consecutive workgroups), costliest blocks first.
  const int per_head = SPLIT ? nqb * p.num_splits : CAUSAL ? (nqb + 1) / 2 : nqb;
  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  const int head = lid / per_head;  // b * H + h
  const int w = lid - head * per_head;
  const int nitems = !SPLIT && CAUSAL && w != nqb - 1 - w ? 2 : 1;
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
  const size_t lse0 = !CONTIG && p.cu ? (size_t)r0 * p.H + (size_t)hi * N : (size_t)head * N;  // LSE of row 0
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31, hh = lane >> 5;
  // (b, h) slices through per-tensor strides; rows are p.s?.n elements apart
  // (both items of a workgroup are in the same head).
  const E* __restrict__ qg = (const E*)p.q + (bi * p.sq.b + hi * p.sq.h + r0 * p.sq.n);
  const E* kg = (const E*)p.k + (bi * p.sk.b + hi * p.sk.h + r0 * p.sk.n);
  const E* vg = (const E*)p.v + (bi * p.sv.b + hi * p.sv.h + r0 * p.sv.n);
  E* og = (E*)p.o + (bi * p.so.b + hi * p.so.h + r0 * p.so.n);
  // Row strides; CONTIG: every row is d elements after the previous one, known
  // at compile time, so tile offsets fold into constants.
  const int sqn = CONTIG ? D : (int)p.sq.n, skn = CONTIG ? D : (int)p.sk.n;
  const int svn = CONTIG ? D : (int)p.sv.n, son = CONTIG ? D : (int)p.so.n;
  for (int item = 0; item < nitems; ++item) {
  if (item) __syncthreads();  // every wave is done with the first block's tiles
  int qb = CAUSAL ? (item == 0 ? nqb - 1 - w : w) : w;
  if constexpr (SPLIT) qb = CAUSAL ? nqb - 1 - w / p.num_splits : w / p.num_splits;
  const int q0 = qb * C::BM;
  if (q0 >= N) continue;  // a packed sequence shorter than the longest
  const int qw = q0 + wave * 32;  // first query of this wave
  const int qi = qw + li;         // this lane's query

  int L = N;
  if (p.key_lens) L = min(max(p.key_lens[bi], 0), N);
  const int kend = CAUSAL ? min(L, q0 + C::BM) : L;  // keys [0, kend) matter to the workgroup
  int nkb = (kend + BN - 1) / BN;
  // Tiles [0, nfree) are unmasked for every query of the workgroup.
  int nfree = L / BN;
  if (CAUSAL) nfree = min(nfree, q0 / BN);
  nfree = min(nfree, nkb);
  // Key tiles [jt0, jt0 + nkb) are this workgroup's; below, tile indices are
  // relative to jt0 (0 unless the keys are split).
  int jt0 = 0, split = 0;
  if constexpr (SPLIT) {
    split = w % p.num_splits;
    const int nt = nkb;
    jt0 = split * nt / p.num_splits;
    nkb = (split + 1) * nt / p.num_splits - jt0;
    nfree = min(max(nfree - jt0, 0), nkb);
  }

  // The copies cover the tiles [0, nkb) only: copies past them (issued without
  // a branch) read zeros without touching memory.
  const int krows = min((jt0 + nkb) * BN, N);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kg, rows_bytes(krows, skn, dl, ES));
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vg, rows_bytes(krows, svn, dl, ES));

  // Q^T as the B operand of S^T = K Q^T: lane holds Q[qi][16c + 8hh .. +7].
  V8 qreg[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) {
    if (qi < N && 16 * c + 8 * hh < dl) {
      qreg[c] = *(const V8*)(qg + (int64_t)qi * sqn + 16 * c + 8 * hh);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) qreg[c][e] = (E)0.0f;
    }
  }

  // Byte offset of this lane's i-th 16-byte copy within a tile: chunk slot
  // (i * NW + wave) * 64 + lane, i.e. row i * COPY_ROWS + r0 with
  // r0 = wave * 64 / CHUNKS + lane / CHUNKS, chunk lane % CHUNKS.  The swizzle
  // depends on the row mod 16, which does not change with i, so copy i is
  // copy 0 moved by i * COPY_ROWS rows: a wave-uniform offset, added with
  // the tile's to the lane's part.
  static_assert(C::COPY_ROWS % 16 == 0, "copy rows must keep their swizzle");
  uint32_t kld0, vld0;
  {
    const int r = wave * 64 / C::CHUNKS + lane / C::CHUNKS, pc = lane % C::CHUNKS;
    const int lch = (pc ^ swz<D>(r)) * 8;  // first column of the chunk this lane copies
    kld0 = lch < dl ? (uint32_t)(r * skn + lch) * ES : kPoison;
    vld0 = lch < dl ? (uint32_t)(r * svn + lch) * ES : kPoison;
  }
  // Row strides in bytes, and the byte step between copy rounds.
  const uint32_t krb = (uint32_t)skn * ES, vrb = (uint32_t)svn * ES;
  const uint32_t kstep = C::COPY_ROWS * krb, vstep = C::COPY_ROWS * vrb;
  // Per-lane offsets of the first copy of K and V tile jt.
  auto k_base = [&](int jt) { return tile_offset<CONTIG>(kld0, (jt0 + jt) * BN, krb); };
  auto v_base = [&](int jt) { return tile_offset<CONTIG>(vld0, (jt0 + jt) * BN, vrb); };
  auto issue_k_piece = [&](uint32_t base, int stage, int i) {
    lds_dma16(krs, kbuf(stage) + (i * NW + wave) * 512, base + i * kstep);
  };
  auto issue_v_piece = [&](uint32_t base, int stage, int i) {
    lds_dma16(vrs, vbuf(stage) + (i * NW + wave) * 512, base + i * vstep);
  };
  auto issue_k = [&](int jt, int stage) {
    const uint32_t base = k_base(jt);
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) issue_k_piece(base, stage, i);
  };
  auto issue_v = [&](int jt, int stage) {
    const uint32_t base = v_base(jt);
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) issue_v_piece(base, stage, i);
  };

  // LDS element offsets of the MFMA operand reads (stage 0; stage 1 adds TILE).
  // K rows: row 32t + li, logical chunk 2c + hh.
  const int ksw = swz<D>(li);
  int koff[KC];
#pragma unroll
  for (int c = 0; c < KC; ++c) koff[c] = li * D + (((2 * c + hh) ^ ksw) * 8);
  // V^T by transposing reads: rows 16cc + trow (+8), logical columns 32u + tcol.
  const int g16 = lane & 15;
  const int trow = 4 * hh + (g16 >> 2);
  const int tcol = 16 * ((lane >> 4) & 1) + 4 * (g16 & 3);
  int voff[2][DU];
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int u = 0; u < DU; ++u) {
      const int r = trow + 8 * half;
      voff[half][u] = r * D + (((4 * u + (tcol >> 3)) ^ swz<D>(r)) * 8) + (tcol & 7);
    }

  f32x16 oacc[DU];
#pragma unroll
  for (int u = 0; u < DU; ++u)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[u][r] = 0.0f;
  const float c2 = p.scale_log2;
  float mref = -INFINITY;  // reference max of this query row, in scale*log2 units
  float l = 0.0f;          // this lane's partial row sum (its 16 keys of every 32)

  auto qk = [&](int stage, f32x16 (&s)[2]) {
    const E* ks = kbuf(stage);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[t][r] = 0.0f;
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        const V8 a = *(const V8*)(ks + koff[c] + t * 32 * D);
        s[t] = Elem<E>::mma(a, qreg[c], s[t]);
      }
    }
  };
  auto apply_mask = [&](int jt, f32x16 (&s)[2]) {
    // key = kb + key_of(t, r) with kb per lane; allowed iff key_of(t, r) < lim.
    const int kb = (jt0 + jt) * BN + 4 * hh;
    int lim = L - kb;
    if (CAUSAL) lim = min(lim, qi - kb + 1);
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kc = 32 * t + 8 * (r >> 2) + (r & 3);
        s[t][r] = kc < lim ? s[t][r] : -INFINITY;
      }
  };
  // Row max of a tile (both partner lanes get it), scaled to exp2 units, and
  // the wave-uniform decision whether the reference max must move.
  auto tile_max = [&](const f32x16 (&s)[2]) {
    float mx = s[0][0];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = (t == 0 ? 1 : 0); r < 16; ++r) mx = fmaxf(mx, s[t][r]);
    return pair_max(mx) * c2;
  };
  auto rescale_if_needed = [&](float mxc) {
    const bool grow = mxc > mref + 8.0f;
    if (__ballot(grow) != 0) {
      const float mnew = fmaxf(mref, mxc);
      const float alpha = mnew == -INFINITY ? 1.0f : fast_exp2(mref - mnew);
      mref = mnew;
      l *= alpha;
#pragma unroll
      for (int u = 0; u < DU; ++u)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[u][r] *= alpha;
    }
  };
  f32x16 sa[2], sb[2];  // score tiles of the current and the next step, alternating
  float mx_cur = -INFINITY;
  if (nkb > 0) {
    issue_k(0, 0);
    issue_v(0, 0);
    // Loads complete in issue order: with at most V_0's (and K_1's) pieces
    // outstanding, Q and this wave's share of K_0 have landed.  V_0 and K_1
    // arrive while the first scores are computed.
    if (nkb > 1) {
      issue_k(1, 1);
      wait_vmem_le<2 * C::LOADS>();
    } else {
      wait_vmem_le<C::LOADS>();
    }
    __syncthreads();
    qk(0, sa);
    if (nfree == 0) apply_mask(0, sa);
    mx_cur = tile_max(sa);
    wait_vmem();  // this wave's share of V_0 and K_1, before the first step's barrier
  }

  // One pipeline step for tile j (scores in scur, row max mx_cur).
  //   Phase A: the MFMAs of S_{j+1} = K_{j+1} Q^T, each followed by the
  //            exponentials (and bf16 packing) of EPA elements of S_j.
  //   Phase B: the MFMAs of O^T += V_j^T P_j^T, each followed by a share of
  //            the mask and row max of S_{j+1}.
  // LDS operand reads run two MFMAs ahead through a three-entry register ring;
  // a scheduling fence after every MFMA group pins that order (left alone,
  // the scheduler either hoists all reads, exhausting the registers, or
  // issues each read right before its MFMA and waits for it).  Loads of K_{j+2} and
  // V_{j+1} are issued at the start and awaited at the end of the step.
  constexpr int NA = 2 * KC;    // phase-A MFMAs
  constexpr int EPA = 32 / NA;  // exponentials per phase-A MFMA
  constexpr int NB = 4 * DU;    // phase-B MFMAs
  constexpr int MPB = 32 / NB;  // row-max elements per phase-B MFMA
  auto step = [&](int j, auto has_next_t, auto mask_next_t, auto par_t, f32x16 (&scur)[2],
                  f32x16 (&sn)[2]) {
    constexpr bool HAS_NEXT = decltype(has_next_t)::value;
    constexpr bool MASK_NEXT = decltype(mask_next_t)::value;
    constexpr int PAR = decltype(par_t)::value;  // j & 1
    __syncthreads();  // K_{j+1}, V_j resident; every wave is done with step j-1
    rescale_if_needed(mx_cur);
    const float nm = mref == -INFINITY ? 0.0f : -mref;

    // ---- phase A
    // Priority while this wave's exponentials are on the critical path: the
    // other wave on the SIMD (in phase B, MFMA-bound) fills the gaps.
    __builtin_amdgcn_s_setprio(3);
    const E* ks = kbuf(PAR ^ 1);
    auto kread = [&](int i) { return *(const V8*)(ks + koff[i % KC] + (i / KC) * 32 * D); };
    V8 pb[4];
    float ps[4];  // partial row sums, each started by its first exponential
    V8 ka[3];
    if constexpr (HAS_NEXT) {
      ka[0] = kread(0);
      ka[1] = kread(1);
    }
    const uint32_t kb2 = k_base(j + 2), vb1 = v_base(j + 1);  // this step's copies
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int t = i / KC, c = i % KC;
      // copies of K_{j+2} and V_{j+1}, one every other MFMA (a burst of them
      // stalls the wave on the full memory queue); tiles past the end read as
      // zero and land in stages nothing reads again
      if (i % 2 == 0 && i / 2 < 2 * C::LOADS) {
        const int x = i / 2;
        if (x < C::LOADS)
          issue_k_piece(kb2, PAR, x);
        else
          issue_v_piece(vb1, PAR ^ 1, x - C::LOADS);
      }
      if constexpr (HAS_NEXT) {
        if (i + 2 < NA) ka[(i + 2) % 3] = kread(i + 2);
        const f32x16 zero = {};
        sn[t] = Elem<E>::mma(ka[i % 3], qreg[c], c == 0 ? zero : sn[t]);
      }
#pragma unroll
      for (int x = 0; x < EPA; ++x) {
        const int k = i * EPA + x, tt = k >> 4, r = k & 15;
        const float e = fast_exp2(fmaf(scur[tt][r], c2, nm));
        scur[tt][r] = e;
        ps[k & 3] = k < 4 ? e : ps[k & 3] + e;
        pin(ps[k & 3]);  // keep the sum here, between this group's MFMAs
      }
      if constexpr (!DROPOUT) {
        // pack the finished pairs: element k lives in pb[k >> 3][k & 7]
#pragma unroll
        for (int x = 0; x < EPA; x += 2) {
          const int k = i * EPA + x, tt = k >> 4, r = k & 15;
          pb[k >> 3][k & 7] = (E)scur[tt][r];
          pb[k >> 3][(k & 7) + 1] = (E)scur[tt][r + 1];
        }
      }
      __builtin_amdgcn_sched_barrier(0);  // nothing crosses: keeps the ring one MFMA ahead
    }
    l += (ps[0] + ps[1]) + (ps[2] + ps[3]);
    if constexpr (DROPOUT) {
      // One Philox call per 4 consecutive keys of this query row.
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const uint32_t key4 = (uint32_t)((jt0 + j) * BN + 32 * t + 8 * g + 4 * hh);
          const u32x4 w = philox(key4 >> 2, (uint32_t)qi, (uint32_t)hi, (uint32_t)(bi + p.b0), p.seed_lo,
                                 p.seed_hi);
          // dropped keys contribute zero; the kept ones' factor 1/(1-p) is
          // applied once, to the normalised output
#pragma unroll
          for (int x = 0; x < 4; ++x)
            scur[t][4 * g + x] = (w[x] >= p.drop_threshold) ? scur[t][4 * g + x] : 0.0f;
        }
      // pairs converted together (one packed conversion each)
      typedef float f32x2 __attribute__((ext_vector_type(2)));
      typedef E e2 __attribute__((ext_vector_type(2)));
#pragma unroll
      for (int k = 0; k < 32; k += 2) {
        const e2 v = __builtin_convertvector(f32x2{scur[k >> 4][k & 15], scur[k >> 4][(k & 15) + 1]}, e2);
        pb[k >> 3][k & 7] = v[0];
        pb[k >> 3][(k & 7) + 1] = v[1];
      }
    }
    // chunk cc of pb covers keys 16cc .. 16cc+15; its k-slots match V^T below.

    // ---- phase B
    __builtin_amdgcn_s_setprio(0);
    if constexpr (HAS_NEXT && MASK_NEXT) apply_mask(j + 1, sn);
    const lds_bf16* vs = (const lds_bf16*)vbuf(PAR);
    auto vread = [&](int idx) {
      const int u = idx / 4, cc = idx % 4;
      const V4 lo = __builtin_bit_cast(V4, lds_read_tr4(vs + voff[0][u] + 16 * cc * D));
      const V4 hi4 = __builtin_bit_cast(V4, lds_read_tr4(vs + voff[1][u] + 16 * cc * D));
      const V8 a = {lo[0], lo[1], lo[2], lo[3], hi4[0], hi4[1], hi4[2], hi4[3]};
      return a;
    };
    float mp[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    V8 va[3];
    va[0] = vread(0);
    va[1] = vread(1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int idx = 0; idx < NB; ++idx) {
      if (idx + 2 < NB) va[(idx + 2) % 3] = vread(idx + 2);
      oacc[idx / 4] = Elem<E>::mma(va[idx % 3], pb[idx % 4], oacc[idx / 4]);
      if constexpr (HAS_NEXT) {
#pragma unroll
        for (int x = 0; x < MPB; x += 2) {
          const int k = idx * MPB + x, q = (k >> 1) & 3;
          max3_into(mp[q], sn[k >> 4][k & 15], sn[k >> 4][(k & 15) + 1]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (HAS_NEXT) mx_cur = pair_max(fmaxf(fmaxf(mp[0], mp[1]), fmaxf(mp[2], mp[3]))) * c2;
    wait_vmem();
  };
  using T = std::true_type;
  using F = std::false_type;
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;

  // The stage parity of every step is a compile-time constant: steps run in
  // pairs from even indices.  Steps before jm (even, at most nfree - 1) have an
  // unmasked next tile; later ones mask it (harmless where no key is masked).
  int j = 0;
  const int jm = max(nfree - 1, 0) & ~1;
  for (; j < jm; j += 2) {
    step(j, T{}, F{}, P0{}, sa, sb);
    step(j + 1, T{}, F{}, P1{}, sb, sa);
  }
  for (; j + 2 < nkb; j += 2) {
    step(j, T{}, T{}, P0{}, sa, sb);
    step(j + 1, T{}, T{}, P1{}, sb, sa);
  }
  if (j + 1 < nkb) {
    step(j, T{}, T{}, P0{}, sa, sb);
#pragma unroll
    for (int t = 0; t < 2; ++t) sa[t] = sb[t];
    ++j;
  }
  if (j < nkb) {  // the last tile: no next one
    if (j & 1)
      step(j, F{}, F{}, P1{}, sa, sb);
    else
      step(j, F{}, F{}, P0{}, sa, sb);
  }

  // Epilogue: O = O^T / l, transposed through the K stages (free once every
  // wave is past the last tile) and written as whole rows; LSE = (mref +
  // log2 l) * ln 2.  A split writes its fp32 O and LSE for the combine pass.
  const float lt = pair_sum(l);
  // 1/l, times the dropout factor 1/(1-p) of the kept keys
  const float inv = lt > 0.0f ? (DROPOUT ? p.drop_scale : 1.0f) / lt : 0.0f;
  const float lse_out = lt > 0.0f ? (mref + __log2f(lt)) * kLn2 : -INFINITY;
  if constexpr (SPLIT) {
    const size_t prow = ((size_t)split * p.heads + head) * N + qi;
    if (qi < N) {
      float* orow = p.opart + prow * D;
#pragma unroll
      for (int u = 0; u < DU; ++u)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 ov;
#pragma unroll
          for (int e = 0; e < 4; ++e) ov[e] = oacc[u][4 * g + e] * inv;
          *(f32x4*)(orow + 32 * u + 8 * g + 4 * hh) = ov;
        }
      if (hh == 0) p.lsepart[prow] = lse_out;
    }
  } else {
    __syncthreads();
    {
      E* ot = ((wave >> 1) ? sk1 : sk0) + (wave & 1) * 32 * D;
      acc_rows_to_lds<D, E>(ot, oacc, inv, false, li, hh);
      lds_rows_to_buffer<D, E>(ot, og + (int64_t)qw * son, son, N - qw, lane, dl);
    }
    if (qi < N && hh == 0) p.lse[lse0 + qi] = lse_out;
  }
  }  // item
}

// Split-KV combine: O_i = sum_s w_s O_i^(s) / sum_s w_s with w_s = exp(LSE_i^(s) - m_i),
// m_i = max_s LSE_i^(s), and LSE_i = m_i + ln sum_s w_s (each split's O is
// normalised by its own row sum l_s, and exp(LSE^(s)) = l_s e^(m_s)).  Eight
// columns per thread; a row whose splits all saw no key gets O = 0, LSE = -inf.
template <typename E, int D>
__global__ __launch_bounds__(256) void fwd_combine_kernel(FwdParams p, int64_t rows) {
  typedef E v8 __attribute__((ext_vector_type(8)));
  constexpr int LPR = D / 8;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = t / LPR;
  const int c = (int)(t % LPR);
  if (row >= rows) return;
  const int splits = p.num_splits;
  float m = -INFINITY;
  for (int s = 0; s < splits; ++s) m = fmaxf(m, p.lsepart[(int64_t)s * rows + row]);
  float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  float den = 0.0f;
  if (m != -INFINITY) {
    for (int s = 0; s < splits; ++s) {
      const float ls = p.lsepart[(int64_t)s * rows + row];
      if (ls == -INFINITY) continue;
      const float wgt = __expf(ls - m);
      den += wgt;
      const float* src = p.opart + ((int64_t)s * rows + row) * D + 8 * c;
      const f32x4 a = *(const f32x4*)src, b = *(const f32x4*)(src + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[e] = fmaf(wgt, a[e], acc[e]);
        acc[4 + e] = fmaf(wgt, b[e], acc[4 + e]);
      }
    }
  }
  const float inv = den > 0.0f ? 1.0f / den : 0.0f;
  v8 ov;
#pragma unroll
  for (int e = 0; e < 8; ++e) ov[e] = (E)(acc[e] * inv);
  const int head = (int)(row / p.N), n = (int)(row - (int64_t)head * p.N);
  const int bi = head / p.H, hi = head - bi * p.H;
  E* dst = (E*)p.o + (bi * p.so.b + hi * p.so.h + (int64_t)n * p.so.n) + 8 * c;
  *(v8*)dst = ov;
  if (c == 0) p.lse[row] = den > 0.0f ? m + __logf(den) : -INFINITY;
}

template <typename E, int D, bool CAUSAL, bool DROPOUT, bool SPLIT, bool CONTIG>
hipError_t launch(const FwdParams& p, int heads, hipStream_t s) {
  using C = FwdCfg<D>;
  const int grid = heads * (SPLIT ? p.num_qblocks * p.num_splits
                                  : CAUSAL ? (p.num_qblocks + 1) / 2 : p.num_qblocks);
  hipLaunchKernelGGL((fwd_kernel<E, D, CAUSAL, DROPOUT, SPLIT, CONTIG>), dim3(grid), dim3(C::THREADS),
                     0, s, p);
  hipError_t e = hipGetLastError();
  if (!SPLIT || e != hipSuccess) return e;
  const int64_t rows = (int64_t)heads * p.N;
  const int64_t threads = rows * (D / 8);
  hipLaunchKernelGGL((fwd_combine_kernel<E, D>), dim3((unsigned)((threads + 255) / 256)), dim3(256),
                     0, s, p, rows);
  return hipGetLastError();
}

template <typename E, int D, bool SPLIT, bool CONTIG>
hipError_t dispatch(const FwdParams& p, int heads, bool causal, bool dropout, hipStream_t s) {
  if (causal) {
    return dropout ? launch<E, D, true, true, SPLIT, CONTIG>(p, heads, s)
                   : launch<E, D, true, false, SPLIT, CONTIG>(p, heads, s);
  }
  return dropout ? launch<E, D, false, true, SPLIT, CONTIG>(p, heads, s)
                 : launch<E, D, false, false, SPLIT, CONTIG>(p, heads, s);
}

// Rows d elements apart in every tensor (the batch and head strides are free).
// Every row stride equals the kernel width, the head size fills it and the
// rows are not packed sequences (the compile-time-stride kernels neither pad
// nor read sequence offsets).
bool rows_contiguous(const FwdParams& p, int d) {
  return p.cu == nullptr && p.dl == d && p.sq.n == d && p.sk.n == d && p.sv.n == d &&
         p.so.n == d;
}

// The split path (small batch x heads) keeps run-time strides only.
template <typename E, int D>
hipError_t dispatch_s(const FwdParams& p, int heads, bool split, bool causal, bool dropout,
                      hipStream_t s) {
  if (split) return dispatch<E, D, true, false>(p, heads, causal, dropout, s);
  return rows_contiguous(p, D) ? dispatch<E, D, false, true>(p, heads, causal, dropout, s)
                               : dispatch<E, D, false, false>(p, heads, causal, dropout, s);
}

template <typename E>
hipError_t dispatch_d(FwdParams& p, const FwdArgs& a, hipStream_t s) {
  const bool dropout = a.dropout_p > 0.0f;
  const int heads = a.B * a.H;
  const bool split = a.num_splits > 0;
  const bool causal = a.causal != 0;
  // Head sizes 32 and 96 run on the kernels of width 64 and 128.
  if (a.d <= 64) {
    p.num_qblocks = (a.N + FwdCfg<64>::BM - 1) / FwdCfg<64>::BM;
    return dispatch_s<E, 64>(p, heads, split, causal, dropout, s);
  }
  p.num_qblocks = (a.N + FwdCfg<128>::BM - 1) / FwdCfg<128>::BM;
  return dispatch_s<E, 128>(p, heads, split, causal, dropout, s);
}

FwdParams make_params(const FwdArgs& a) {
  FwdParams p;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.o = a.o;
  p.lse = a.lse;
  p.key_lens = a.key_lens;
  p.cu = a.cu;
  p.sq = a.sq;
  p.sk = a.sk;
  p.sv = a.sv;
  p.so = a.so;
  p.H = a.H;
  p.N = a.N;
  p.dl = a.d;
  p.b0 = a.b0;
  p.num_qblocks = 0;
  p.scale_log2 = a.scale * kLog2e;
  p.drop_threshold = a.drop_threshold;
  p.drop_scale = a.drop_scale;
  p.seed_lo = (uint32_t)(a.seed & 0xffffffffu);
  p.seed_hi = (uint32_t)(a.seed >> 32);
  p.opart = a.opart;
  p.lsepart = a.lsepart;
  p.num_splits = a.num_splits;
  p.heads = a.B * a.H;
  return p;
}

}  // namespace

hipError_t launch_fwd_16(const FwdArgs& a, hipStream_t s) {
  FwdParams p = make_params(a);
  return a.fp16 ? dispatch_d<f16>(p, a, s) : dispatch_d<bf16>(p, a, s);
}

}  // namespace fa
