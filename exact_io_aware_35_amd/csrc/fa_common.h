// fa_common.h -- types, launch parameters and small device helpers shared by
// the forward and backward kernels of the gfx950 attention library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_params.h"

namespace fa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

__device__ __forceinline__ int key_len(const MaskParams& m, int b, int N) {
  if (m.seqlens_k == nullptr) return N;
  int L = m.seqlens_k[b];
  return L < 0 ? 0 : (L > N ? N : L);
}

// Keys visible to at least one query in [qa, qb] (inclusive): [lo, hi).
__device__ __forceinline__ void key_range(const MaskParams& m, int kl, int qa, int qb,
                                          int& lo, int& hi) {
  lo = 0;
  hi = kl;
  if (m.wl >= 0) lo = max(0, qa - m.wl);
  if (m.wr >= 0) hi = min(hi, qb + m.wr + 1);
  if (hi < lo) hi = lo;
}

// Every (i, j) with i in [qa, qb], j in [ka, kb] visible?
__device__ __forceinline__ bool block_all_visible(const MaskParams& m, int kl, int qa, int qb,
                                                  int ka, int kb) {
  if (kb >= kl) return false;
  if (m.wl >= 0 && ka < qb - m.wl) return false;
  if (m.wr >= 0 && kb > qa + m.wr) return false;
  return true;
}

// Keys visible to query i form the span [lo, hi] (empty when hi < lo).
__device__ __forceinline__ void visible_span(const MaskParams& m, int kl, int i, int& lo, int& hi) {
  lo = m.wl >= 0 ? i - m.wl : 0;
  hi = m.wr >= 0 ? min(kl - 1, i + m.wr) : kl - 1;
}

__device__ __forceinline__ bool visible(const MaskParams& m, int kl, int i, int j) {
  return j < kl && (m.wl < 0 || j >= i - m.wl) && (m.wr < 0 || j <= i + m.wr);
}

// Work-group id -> (bh, block). Workgroups are dispatched round-robin over the
// 8 XCDs (hardware id i runs on XCD i % 8), each XCD with its own L2. When the
// (b, h) count divides by 8, every XCD gets whole (b, h) groups so their K/V
// stay in one L2; within an XCD the blocks are interleaved over its heads and,
// for longest-first, ordered by decreasing block index (more keys under a
// causal mask).
// map_index takes the id explicitly (a kernel that runs two kinds of
// work-group in one grid passes each kind's own index; the XCD of index i is
// still i % 8 as long as the first kind's count divides by 8).
__device__ __forceinline__ void map_index(int i, int nbh, int nblk, int xcd_groups, int longest_first,
                                          int& bh, int& blk) {
  int rank;
  if (xcd_groups > 0) {
    const int hpx = nbh / 8;           // (b, h) per XCD
    const int xcd = i % 8, slot = i / 8;
    bh = xcd * hpx + slot % hpx;
    rank = slot / hpx;
  } else {
    bh = i % nbh;
    rank = i / nbh;
  }
  blk = longest_first ? (nblk - 1 - rank) : rank;
}
__device__ __forceinline__ void map_block(int nbh, int nblk, int xcd_groups, int longest_first,
                                          int& bh, int& blk) {
  map_index(blockIdx.x, nbh, nblk, xcd_groups, longest_first, bh, blk);
}

// ALiBi slope of (b, h) in raw score units: the bias -slope |i - j| is added
// to the scaled score c q.k, so the raw score q.k takes -(slope / c) |i - j|
// (scale_log2 = c log2 e).
__device__ __forceinline__ float alibi_raw_slope(const AlibiParams& a, int b, int h,
                                                 float scale_log2) {
  return a.slopes[b * a.bstride + h] * (1.4426950408889634f / scale_log2);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return log2f(x); }

// Max over the two 32-lane halves: permlane32_swap(x, x) yields the lower
// half's value in the first result and the upper half's in the second, in
// every lane.
__device__ __forceinline__ float half_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Round-to-nearest-even float -> bf16 bits, two at a time (gfx950 converts in
// hardware; the conversion is RNE with NaN preserved).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
  bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
  f16x2_t v = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ f32x16_t mfma_bf16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16_t mfma_f16(f16x8_t a, f16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16_t mfma_f32(float a, float b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Transposing LDS read of 4 x 16-bit values (gfx950 ds_read_b64_tr_b16). In
// each group of 16 lanes, the lanes address a 16 x 4 block (one 8-byte row
// per lane); lane i receives element (4 e + i / 4, i % 4) for e = 0..3.
__device__ __forceinline__ u32x2_t lds_read_tr16(const void* p) {
  return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)p));
}

// Raw buffer descriptor over [base, base + bytes): loads past the end return 0
// (the range check covers voffset + soffset, so a tile's first row may go in
// the scalar offset).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// 16-byte buffer load straight into LDS: lane i of the wave writes
// lds + 16 i with the 16 bytes at voffset + soffset of the buffer.
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t r, void* lds, int voffset,
                                                  int soffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                           voffset, soffset, 0, 0);
}

// 16-byte buffer load into registers (zero past the descriptor's end).
__device__ __forceinline__ u32x4_t buffer_load16(__amdgpu_buffer_rsrc_t r, int voffset, int soffset) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, voffset, soffset, 0));
}

template <typename T>
__device__ __forceinline__ T ld_global(const void* p) { return *reinterpret_cast<const T*>(p); }

// 8 bf16 (one 16-byte chunk) -> 8 fp16, rounded to nearest even (exact for
// magnitudes in fp16's normal range).
__device__ __forceinline__ u32x4_t bf16x8_to_f16x8(u32x4_t u) {
  u32x4_t r;
#pragma unroll
  for (int e = 0; e < 4; ++e) r[e] = pack_f16x2(bf16_lo(u[e]), bf16_hi(u[e]));
  return r;
}

// The two 16-bit element types of Q, K, V, O, dO and the gradients: bf16 and
// fp16 (IEEE half). Both run on the 32x32x16 MFMA with fp32 accumulation and
// round their outputs to nearest even.
template <typename T>
struct Elt16;
template <>
struct Elt16<__bf16> {
  using vec8 = bf16x8_t;
  static constexpr bool is_f16 = false;
  static __device__ __forceinline__ f32x16_t mfma(vec8 a, vec8 b, f32x16_t c) { return mfma_bf16(a, b, c); }
  static __device__ __forceinline__ uint32_t pack2(float a, float b) { return pack_bf16x2(a, b); }
  static __device__ __forceinline__ float lo(uint32_t u) { return bf16_lo(u); }
  static __device__ __forceinline__ float hi(uint32_t u) { return bf16_hi(u); }
  // 8 values -> 8 fp16 values (the backward's operand format).
  static __device__ __forceinline__ u32x4_t to_f16x8(u32x4_t u) { return bf16x8_to_f16x8(u); }
};
template <>
struct Elt16<_Float16> {
  using vec8 = f16x8_t;
  static constexpr bool is_f16 = true;
  static __device__ __forceinline__ f32x16_t mfma(vec8 a, vec8 b, f32x16_t c) { return mfma_f16(a, b, c); }
  static __device__ __forceinline__ uint32_t pack2(float a, float b) { return pack_f16x2(a, b); }
  static __device__ __forceinline__ float lo(uint32_t u) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(u & 0xffffu));
  }
  static __device__ __forceinline__ float hi(uint32_t u) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(u >> 16));
  }
  static __device__ __forceinline__ u32x4_t to_f16x8(u32x4_t u) { return u; }
};

// LDS tiles of 16-bit values, [rows][D] row-major, with the 16-byte chunks of
// each row XOR-swizzled: chunk c of row r is stored at position c ^ lds_swz(r).
// With it the two read patterns of the kernels are free of bank conflicts:
// 16 consecutive rows reading one chunk (a row-major MFMA operand) and 4
// consecutive rows x 4 consecutive chunks (a transposed read). lds_swz only
// depends on the low 4 bits of the row.
template <int D>
__device__ __forceinline__ int lds_swz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

// Byte offset of chunk c (elements 8c .. 8c+7) of row r in such a tile.
template <int D>
__device__ __forceinline__ int tile_chunk_off(int r, int c) {
  return (r * (D / 8) + (c ^ lds_swz<D>(r))) * 16;
}

// Byte offset a lane passes to lds_read_tr16 to fetch its half t (t = 0, 1)
// of a transposed 32x32x16 MFMA operand covering columns 32 db .. 32 db + 31
// and rows 0..15 of the tile: lane r of 16-lane group g addresses row
// 8 t + 4 (g / 2) + r / 4 at column 32 db + 16 (g % 2) + 4 (r % 4). Lane l
// then holds column 32 db + l % 32 at the 8 rows 8 (j / 4) + 4 (l / 32) + j % 4,
// the row order in which a 32x32 accumulator holds its rows.
template <int D>
__device__ __forceinline__ int tile_tr_off(int lane, int db, int t) {
  const int g = lane >> 4, r = lane & 15;
  const int row = 8 * t + 4 * (g >> 1) + (r >> 2);
  const int col = 32 * db + 16 * (g & 1) + 4 * (r & 3);
  return tile_chunk_off<D>(row, col >> 3) + ((col >> 2) & 1) * 8;
}

}  // namespace fa
