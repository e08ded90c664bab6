// Device-side building blocks shared by the gfx950 attention kernels:
// vector types, the MFMA and LDS-transpose intrinsics, lane exchange across the
// two 32-lane halves of a wave, and the Philox4x32-10 generator that draws the
// dropout keep mask.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace fa {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// D(32x32, f32) += A(32x16, bf16) * B(16x32, bf16).  Lane l supplies row/column
// (l % 32) of A/B and eight consecutive k-slots 8*(l/32) .. 8*(l/32)+7; the
// result register r of lane l is row 8*(r/4) + 4*(l/32) + r%4, column l % 32.
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// acc += A B with the accumulator pinned to AccVGPRs, for long-lived
// accumulators that only MFMAs touch (the other MFMAs and the VALU keep the
// ordinary VGPRs).  Dependent issues on the same accumulator need no wait
// states; a VALU read of acc must follow acc_settle().
__device__ __forceinline__ void mfma32_acc(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// acc = A B (the first product into an accumulator: no prior value, so the
// compiler has nothing to initialise or copy right before the MFMA reads it).
__device__ __forceinline__ void mfma32_acc_first(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=a"(acc) : "v"(a), "v"(b));
}
// The compiler does not know when an inline-asm MFMA has finished reading its
// A/B registers; keep(x) after two later MFMA issues marks x as still in use
// up to that point, so nothing overwrites it while the MFMA may read it.
__device__ __forceinline__ void keep(const bf16x8& x) { asm volatile("" ::"v"(x)); }
// Wait states covering the latency of the last mfma32_acc before its
// accumulator is read.
__device__ __forceinline__ void acc_settle() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"); }
// The same wait states, tied to the accumulators they protect: the asm claims
// to rewrite x, so every later read of x (a VALU read of the MFMA results)
// is ordered after the wait, and the MFMAs that produced x before it.  Tie
// further accumulators with tie_acc/tie_vacc right after (inline asm
// statements with side effects keep their order).
__device__ __forceinline__ void settle_acc(f32x16& x) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(x));
}
__device__ __forceinline__ void settle_vacc(f32x16& x) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(x));
}
__device__ __forceinline__ void tie_acc(f32x16& x) { asm volatile("" : "+a"(x)); }
__device__ __forceinline__ void tie_vacc(f32x16& x) { asm volatile("" : "+v"(x)); }

// LDS transposing read of four 16-bit elements.  Within each group of 16 lanes,
// lane t receives element (t % 4) of the 8-byte load issued by lane 4*e + t/4 as
// its element e.  If lane s of the group points at row (s / 4) and column
// 4*(s % 4) of a row-major 4 x 16 block, lane t therefore gets column t of the
// block: the four rows' values of that column.
__device__ __forceinline__ bf16x4 lds_read_tr4(const bf16* lds_ptr) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)((__attribute__((address_space(3))) char*)((uintptr_t)lds_ptr)));
  return __builtin_bit_cast(bf16x4, r);
}

// LDS-typed pointers: arithmetic on them stays visible to the backend, which
// folds constant displacements into the 16-bit offset field of the DS
// instruction instead of materialising one address register per access.
typedef __attribute__((address_space(3))) bf16 lds_bf16;
__device__ __forceinline__ const lds_bf16* to_lds(const bf16* p) {
  return (const lds_bf16*)p;
}
__device__ __forceinline__ bf16x4 lds_read_tr4(const lds_bf16* p) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
  return __builtin_bit_cast(bf16x4, r);
}

// Value held by lane (l ^ 32): the two halves of the wave swap.
__device__ __forceinline__ float other_half(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  // r[0]: lanes 0-31 keep their own value, lanes 32-63 get lane l-32's;
  // r[1]: lanes 0-31 get lane l+32's, lanes 32-63 keep their own.
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

// max and sum over the lane pair (l, l ^ 32); both lanes get the same bits.
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);  // lower lane's value first in both
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// acc + sum_e a[e] * b[e] over eight bf16 pairs, as four v_dot2 (the bf16
// products are exact in fp32; the sums are fp32).
__device__ __forceinline__ float dot8(const bf16x8& a, const bf16x8& b, float acc) {
#pragma unroll
  for (int e = 0; e < 8; e += 2)
    acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{a[e], a[e + 1]}, bf16x2{b[e], b[e + 1]}, acc, false);
  return acc;
}

// An empty instruction that claims to read and rewrite x: the value must be
// computed at this point of the program, which keeps a reduction step inside
// the MFMA group it was written in instead of being sunk past the loop.
__device__ __forceinline__ void pin(float& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(bf16x8& x) { asm volatile("" : "+v"(x)); }

// m = max(m, a, b) as one v_max3_f32, placed where it is written (the scores
// are never NaN, so the operand canonicalisation fmaxf would add is not needed).
__device__ __forceinline__ void max3_into(float& m, float a, float b) {
  asm volatile("v_max3_f32 %0, %0, %1, %2" : "+v"(m) : "v"(a), "v"(b));
}

// Philox4x32-10 (Salmon et al., SC'11): ten rounds of
//   (c0, c1, c2, c3) -> (hi(B*c2) ^ c1 ^ k0, lo(B*c2), hi(A*c0) ^ c3 ^ k1, lo(A*c0))
// with A = 0xD2511F53, B = 0xCD9E8D57, the key advanced by the Weyl increments
// (0x9E3779B9, 0xBB67AE85) between rounds.
__device__ __forceinline__ u32x4 philox(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                        uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    // Each product as one 32 x 32 -> 64-bit multiply: the compiler emits a
    // single v_mad_u64_u32 (and allocates its carry-out register itself)
    // instead of a v_mul_lo_u32 + v_mul_hi_u32 pair, 1.3x the Philox
    // throughput of the pair on gfx950 with the same words.
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0, p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t lo0 = (uint32_t)p0, hi0 = (uint32_t)(p0 >> 32);
    const uint32_t lo1 = (uint32_t)p1, hi1 = (uint32_t)(p1 >> 32);
    // three-input XORs as one v_bitop3_b32 each (truth table 0x96: odd
    // parity of the three inputs); the compiler leaves them as two v_xor
    const uint32_t n0 = __builtin_amdgcn_bitop3_b32(hi1, c1, k0, 0x96);
    const uint32_t n2 = __builtin_amdgcn_bitop3_b32(hi0, c3, k1, 0x96);
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  u32x4 out = {c0, c1, c2, c3};
  return out;
}

// Word i & 3 of a Philox output, where i may differ from lane to lane.  A
// dynamic vector extract lowers to selects.  A chain of comparisons against i
// is instead turned into a switch, that is, branches that diverge across the
// lanes, and the register allocator has been seen to place a whole-wave
// register copy inside one arm of such a branch, leaving it unwritten in the
// lanes that skipped that arm.
__device__ __forceinline__ uint32_t philox_word(const u32x4& w, int i) { return w[i & 3]; }

// XOR swizzle of the 16-byte chunks of a row-major bf16 tile with D-element
// rows: the physical chunk slot of logical chunk c in tile row r is c ^ swz(r).
// d = 128 (16 chunks, 256-byte rows): 16 consecutive rows get 16 distinct
// values (row reads of 16 lanes hit all 64 banks once) and 4 aligned
// consecutive rows differ in bits 2-3 (the transposing read of 4 rows x 64
// bytes hits 4 different 64-byte bank groups).  d = 64 (8 chunks, 128-byte
// rows): the same two properties with two rows per 256-byte bank cycle.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) {
    return ((r & 3) << 2) | ((r >> 2) & 3);
  } else {
    return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  }
}

// Element types of the 16-bit paths and their MFMA: D(32x32, f32) += A B with
// A 32x16 and B 16x32 of that type (same lane layout as mfma32).
template <typename E>
struct Elem;
template <>
struct Elem<bf16> {
  typedef bf16x8 v8;
  typedef bf16x4 v4;
  static __device__ __forceinline__ f32x16 mma(const v8& a, const v8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // acc += A B (acc = A B) with acc pinned to AccVGPRs (see mfma32_acc)
  static __device__ __forceinline__ void mma_acc(f32x16& acc, const v8& a, const v8& b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
  }
  static __device__ __forceinline__ void mma_acc_first(f32x16& acc, const v8& a, const v8& b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=a"(acc) : "v"(a), "v"(b));
  }
  // d = A B and d += A B with B read from AccVGPRs and d in ordinary VGPRs.
  // The compiler does not know these are MFMAs: a VALU read of d must follow
  // acc_settle() after the last of them.
  static __device__ __forceinline__ void mma_b_acc_first(f32x16& d, const v8& a, const v8& b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
  }
  static __device__ __forceinline__ void mma_b_acc(f32x16& d, const v8& a, const v8& b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
  }
  // acc + sum_e a[e] * b[e] over eight pairs (exact products, fp32 sums)
  static __device__ __forceinline__ float dot8(const v8& a, const v8& b, float acc) {
#pragma unroll
    for (int e = 0; e < 8; e += 2)
      acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{a[e], a[e + 1]}, bf16x2{b[e], b[e + 1]}, acc,
                                            false);
    return acc;
  }
};
template <>
struct Elem<f16> {
  typedef f16x8 v8;
  typedef f16x4 v4;
  static __device__ __forceinline__ f32x16 mma(const v8& a, const v8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ void mma_acc(f32x16& acc, const v8& a, const v8& b) {
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
  }
  static __device__ __forceinline__ void mma_acc_first(f32x16& acc, const v8& a, const v8& b) {
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, 0" : "=a"(acc) : "v"(a), "v"(b));
  }
  static __device__ __forceinline__ void mma_b_acc_first(f32x16& d, const v8& a, const v8& b) {
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
  }
  static __device__ __forceinline__ void mma_b_acc(f32x16& d, const v8& a, const v8& b) {
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
  }
  static __device__ __forceinline__ float dot8(const v8& a, const v8& b, float acc) {
#pragma unroll
    for (int e = 0; e < 8; e += 2)
      acc = __builtin_amdgcn_fdot2(f16x2{a[e], a[e + 1]}, f16x2{b[e], b[e + 1]}, acc, false);
    return acc;
  }
};

// Buffer resource for raw byte-addressed loads from [base, base + bytes).  A
// load whose 16-byte range lies past `bytes` returns zeros, which gives the
// ragged tail of a sequence for free.  The last word selects 32-bit raw
// buffer access on gfx9-family parts.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Bytes a buffer resource must span to cover rows [0, rows) of D elements
// each, `sn` elements apart (sn >= D): reads of any row >= rows then fall
// outside it and return zeros.
__device__ __forceinline__ uint32_t rows_bytes(int rows, int64_t sn, int D, int esize) {
  return rows <= 0 ? 0u : (uint32_t)(((int64_t)(rows - 1) * sn + D) * esize);
}

// Write a wave's 32 x D fp32 accumulator tile, held in the MFMA output layout
// with one row per lane (lane li: row li; acc[u][r]: column 32u + 8(r/4) +
// 4hh + r%4), as bf16 (acc * mul, or zeros) into a row-major 32 x D LDS tile
// whose 16-byte chunks are XOR-swizzled by swz<D>(row).
template <int D, typename E = bf16>
__device__ __forceinline__ void acc_rows_to_lds(E* tile, const f32x16 (&acc)[D / 32], float mul,
                                                bool zero, int li, int hh) {
  typedef E v4 __attribute__((ext_vector_type(4)));
  // Opaque lane indices: the addresses are computed here, where they are
  // used, rather than hoisted out of the caller's loop and kept live.
  asm volatile("" : "+v"(li), "+v"(hh));
#pragma unroll
  for (int u = 0; u < D / 32; ++u)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      v4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // The product rounded to fp32, then converted: without the pin, fp16
        // output may fuse both roundings into one mixed-precision FMA, and
        // the result would depend on which kernel variant it came from.
        float x = acc[u][4 * g + e] * mul;
        pin(x);
        v[e] = zero ? (E)0.0f : (E)x;
      }
      *(v4*)(tile + li * D + (((4 * u + g) ^ swz<D>(li)) * 8) + 4 * hh) = v;
    }
}

// Write this lane's row of such an accumulator tile (acc * mul, or zeros) as
// fp32 to row[0 .. D): 16 bytes per store, the two lanes of a row (hh = 0, 1)
// filling alternate groups of four columns.  For the split backward's
// partial gradients, which a combine pass reads once.
template <int D>
__device__ __forceinline__ void acc_row_to_f32(float* row, const f32x16 (&acc)[D / 32], float mul,
                                               bool zero, int hh) {
#pragma unroll
  for (int u = 0; u < D / 32; ++u)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      f32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = zero ? 0.0f : acc[u][4 * g + e] * mul;
      *(f32x4*)(row + 32 * u + 8 * g + 4 * hh) = v;
    }
}

// Per-lane buffer offset that no access can reach: a lane whose 16-byte chunk
// lies past a tensor's head size (the kernels of width D run head sizes
// dl < D with the columns [dl, D) zero-padded on chip) starts from it, so its
// loads read zeros and its stores are dropped by the buffer range check.
// Valid offsets stay below 2^31 (the host routes a tensor here only when its
// slice spans fewer bytes), so poison plus any tile offset neither wraps nor
// falls in range.
constexpr uint32_t kPoison = 0x80000000u;

// Copy rows [0, min(nrows, 32)) of such an LDS tile to the rows of a tensor
// slice starting at dst, rows `sn` elements apart, 16 bytes per lane: every
// store instruction writes 64 / (D/8) whole rows.  The stores go through a
// buffer resource whose byte range ends with row min(nrows, 32) - 1, so the
// range check drops the rows past it (no branch; one 32-bit per-lane offset
// plus a uniform step per row: callers keep each slice's byte span within
// 32 bits).  Columns [dl, D) are not written.
template <int D, typename E>
__device__ __forceinline__ void lds_rows_to_buffer(const E* tile, E* dst, int64_t sn, int nrows,
                                                   int lane, int dl) {
  constexpr int CH = D / 8, RPI = 64 / CH, ES = (int)sizeof(E);
  typedef E v8 __attribute__((ext_vector_type(8)));
  asm volatile("" : "+v"(lane));  // see acc_rows_to_lds
  const int c = lane % CH;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(dst, rows_bytes(min(nrows, 32), sn, dl, ES));
  const uint32_t rb = (uint32_t)sn * ES;
  const uint32_t off0 =
      c * 8 < dl ? (uint32_t)(lane / CH) * rb + (uint32_t)(c * 8 * ES) : kPoison;
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int r = i * RPI + lane / CH;
    const v8 v = *(const v8*)(tile + r * D + ((c ^ swz<D>(r)) * 8));
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs, off0 + (uint32_t)(i * RPI) * rb,
                                           0, 0);
  }
}

// Remap a linear workgroup id so that consecutive logical ids run on the same
// XCD.  The dispatcher deals workgroups round-robin to the 8 XCDs, so physical
// id p lands on XCD p % 8; logical id (p % 8) * (G / 8) + p / 8 puts each XCD's
// share in one contiguous logical range.  Only applied when G % 8 == 0.
__device__ __forceinline__ int xcd_remap(int p, int G) {
  if ((G & 7) != 0) return p;
  return (p & 7) * (G >> 3) + (p >> 3);
}



typedef __attribute__((address_space(3))) void lds_void_t;

// Direct global -> LDS copy of 16 bytes per lane: lane l's 16 bytes from
// byte offset `voff` of the buffer land at LDS byte address
// lds_wave_base + 16 * l (lds_wave_base is the same for the whole wave).
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, const void* lds_wave_base,
                                          uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds_wave_base, 16, voff, 0, 0, 0);
}

// Per-lane byte offset of a tile's first copy: voff + row0 * row_bytes for
// the wave-uniform first row row0.  Copy i of the tile then adds the
// wave-uniform i * (rows per copy round) * row_bytes.  Row offsets belong in
// the per-lane offset, never the instruction's scalar-offset field: the
// buffer range check that turns reads past the last row into zeros looks at
// the per-lane offset (plus the immediate) only, so a row offset in the
// scalar field would let tiles past the end read whatever memory follows
// the slice.  row0 is made opaque (kept in a scalar register) so that the
// base is formed once per tile where it is needed, instead of the whole sum
// being hoisted out of the loop as one register per copy.
// CONST_STRIDE: row_bytes is a compile-time constant, and the plain sum folds
// into immediates.
template <bool CONST_STRIDE = false>
__device__ __forceinline__ uint32_t tile_offset(uint32_t voff, int row0, uint32_t row_bytes) {
  if constexpr (!CONST_STRIDE) {
    row0 = __builtin_amdgcn_readfirstlane(row0);  // uniform by construction
    asm volatile("" : "+s"(row0));
  }
  return voff + (uint32_t)row0 * row_bytes;
}

// Marks x as still in use at this point (see keep).
template <typename T>
__device__ __forceinline__ void keep_v(const T& x) {
  asm volatile("" ::"v"(x));
}
template <typename T>
__device__ __forceinline__ void pin_v(T& x) {
  asm volatile("" : "+v"(x));
}
// An opaque redefinition of a per-lane offset: address arithmetic built on it
// is formed after this point, where it is used, instead of being hoisted out
// of the loop as one register per combination of offset and constant.
__device__ __forceinline__ void opaque(int& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void opaque_u(uint32_t& x) { asm volatile("" : "+v"(x)); }

// Wait until this wave's outstanding vector-memory loads (including LDS DMA)
// have completed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Wait until at most N of this wave's vector-memory operations are still
// outstanding.  They complete in issue order, so operations issued before the
// last N are done (N <= 63; the count is split over bits 3:0 and 15:14).
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// f(std::integral_constant<int, I>{}) for I = 0 .. N-1, in order: every index
// is a compile-time constant inside f.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

}  // namespace fa
