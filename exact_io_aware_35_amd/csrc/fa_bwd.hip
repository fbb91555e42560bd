// fa_bwd.hip -- recompute-from-LSE backward of exact attention for gfx950.
//
// The forward keeps only O and the per-row LSE; the backward rebuilds
// P = exp(c q.k - LSE) tile by tile instead of reading a stored N x N matrix
// (interview guide "FlashAttention 深入", section "反向传播：用重计算换显存";
// l189.com from-scratch article §3.3). With the softmax Jacobian
// dp_j/ds_i = p_i (delta_ij - p_j) applied over the whole row,
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  D_i = sum_j P_ij dP_ij,
//   dQ = c dS K,  dK = c dS^T Q,
// and D_i equals sum_d dO_id O_id, a row statistic computed once up front.
// (The article's code sums P * dP over one key block only; the full-row sum
// is what its own Jacobian gives, and is what is used here.)
//
// Three kernels, no atomics, so the result is deterministic (the flash_attn
// docstring's deterministic backward, claire-chang.com notes):
//   bwd_prep_kernel : per row D_i (from O and dO) and LSE log2 e; fp16 copies
//                     of Q, K and dO; per block the maxima of |Q|, |K|, |V|,
//                     |dO| (bandwidth-bound, one pass).
//   bwd_rescale_kernel : rewrites the copies of a slice whose maxima leave
//                     fp16's comfortable range (operand range, below);
//                     returns at once for every other slice.
//   bwd_kvq_kernel  : the dK/dV work-groups, then the dQ work-groups, in one
//                     grid (the two passes are independent):
//     dK/dV block   : one work-group per key block; each wave keeps K, V, dK
//                     and dV of 32 keys in registers and streams the query
//                     tiles (Q, dO and the row statistics) through LDS.
//     dQ block      : one work-group per query block; each wave keeps Q, dO
//                     and dQ of 32 queries in registers and streams the key
//                     tiles (K, V) through LDS.
// Every product with P or dS as an operand runs on fp16 MFMA: P and dS carry
// 3 more mantissa bits in fp16 than in bf16, and the bf16 inputs they meet
// (Q, K, dO) convert to fp16 exactly in fp16's normal range. The conversion is
// done once, by the pre-pass, so every tile is copied global -> LDS by the
// direct-to-LDS buffer loads (double-buffered, one barrier per tile), in the
// swizzled row-major layout of fa_common.h; the transposed operands (dO^T,
// Q^T, K^T) come from ds_read_b64_tr_b16 reads and no wave transposes data in
// registers. Accumulation is fp32 throughout.

#include <type_traits>

#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

// ---------------------------------------------------------------- pre-pass

// Operand range. The products with P or dS take fp16 operands, so Q, K and dO
// are copied to fp16 and V is converted in registers. Each of the four is
// used as it is when its largest magnitude in the (b, h) slice lies in
// [2^-6, 8]: every value then converts without overflow, values down to 2^-8
// of the largest stay normal, and |dS| <= |dP| + |D| <= 2 headdim max|dO|
// max|V| <= 2^15 fits fp16. A slice whose maximum lies outside that range
// (bf16 values above fp16's 65504, gradients of 1e-6, ...) is scaled by an
// exact power of two 2^e that brings the maximum into [4, 8) (|e| <= 40); the
// kernels fold e into the exponent's scale and the epilogues, where each
// power of two is exact, so the result is that of the scaled slice up to the
// same fp16 roundings (l189.com from-scratch article §5.2: keep every
// intermediate inside the format's range).
constexpr float kRangeLo = 0x1p-6f, kRangeHi = 8.f;

__device__ __forceinline__ int range_exp(float m) {
  if (!(m > 0.f) || !(m <= 3.4e38f) || (m >= kRangeLo && m <= kRangeHi)) return 0;
  int ex;
  (void)frexpf(m, &ex);  // m = f 2^ex, f in [0.5, 1)
  return min(40, max(-40, 3 - ex));
}

// Exponents (Q, K, dO, V) of slice bh from the pre-pass's block maxima
// (wave-uniform; every lane of the calling wave takes part).
struct SliceExp {
  int q, k, o, v;
};
__device__ __forceinline__ SliceExp slice_exp(const BwdParams& p, int bh) {
  const int lane = threadIdx.x & 63;
  f32x4_t m = f32x4_t{};
  if (lane < p.np) m = ld_global<f32x4_t>(p.part + ((size_t)bh * kMaxParts + lane) * 4);
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1)
#pragma unroll
    for (int t = 0; t < 4; ++t) m[t] = fmaxf(m[t], __shfl_xor(m[t], sh, 64));
  SliceExp e;
  e.q = __builtin_amdgcn_readfirstlane(range_exp(m[0]));
  e.k = __builtin_amdgcn_readfirstlane(range_exp(m[1]));
  e.v = __builtin_amdgcn_readfirstlane(range_exp(m[2]));
  e.o = __builtin_amdgcn_readfirstlane(range_exp(m[3]));
  return e;
}

// 8 values of type T -> 8 fp16 values of x 2^e, rounded to nearest even.
template <typename T>
__device__ __forceinline__ u32x4_t to_f16x8_scaled(u32x4_t u, int e) {
  using E = Elt16<T>;
  u32x4_t r;
#pragma unroll
  for (int j = 0; j < 4; ++j) r[j] = pack_f16x2(ldexpf(E::lo(u[j]), e), ldexpf(E::hi(u[j]), e));
  return r;
}

// One work-group per (b, h) and block of p.prows rows; one 16-byte chunk of
// one row per thread per pass: D_i = sum_d dO O (fp32), the fp16 copies of
// the Q, K and dO chunks, per row the statistics pair (LSE log2 e, or +inf for
// a row with no visible key; D_i), and per block the maxima of |Q|, |K|, |V|,
// |dO| (NaN inputs do not raise them).
template <int D, typename T>
__global__ void __launch_bounds__(256) bwd_prep_kernel(BwdParams p) {
  using E = Elt16<T>;
  constexpr int LPR = D / 8;               // lanes per row, 16 bytes each
  constexpr int RPB = 256 / LPR;           // rows per pass
  __shared__ f32x4_t red[4];
  const int tid = threadIdx.x, c = tid % LPR;
  const int bh = blockIdx.x / p.np, pb = blockIdx.x - bh * p.np;
  const int b = bh / p.H, h = bh - b * p.H;
  f32x4_t mx = f32x4_t{};
  // p.prows is a multiple of RPB: every thread runs the same passes (the
  // row sum below is a shuffle over the LPR lanes of a row).
  for (int pass = 0; pass < p.prows / RPB; ++pass) {
    const int i = pb * p.prows + pass * RPB + tid / LPR;
    float acc = 0.f;
    const bool live = i < p.N;
    if (live) {
      const size_t bi = (size_t)b * p.N + i;
      const size_t hd = (size_t)h * D + 8 * c;
      const size_t e = (bi * p.H) * D + hd;        // the fp16 copies are [B][N][H][D]
      const size_t eq = bi * p.rs_q + hd, eo = bi * p.rs_o + hd;
      const u32x4_t o = ld_global<u32x4_t>((const T*)p.o + eo);
      const u32x4_t g = ld_global<u32x4_t>((const T*)p.dout + eo);
      const u32x4_t q = ld_global<u32x4_t>((const T*)p.q + eq);
      const u32x4_t k = ld_global<u32x4_t>((const T*)p.k + eq);
      const u32x4_t v = ld_global<u32x4_t>((const T*)p.v + eq);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc += E::lo(o[j]) * E::lo(g[j]) + E::hi(o[j]) * E::hi(g[j]);
        mx[0] = fmaxf(mx[0], fmaxf(fabsf(E::lo(q[j])), fabsf(E::hi(q[j]))));
        mx[1] = fmaxf(mx[1], fmaxf(fabsf(E::lo(k[j])), fabsf(E::hi(k[j]))));
        mx[2] = fmaxf(mx[2], fmaxf(fabsf(E::lo(v[j])), fabsf(E::hi(v[j]))));
        mx[3] = fmaxf(mx[3], fmaxf(fabsf(E::lo(g[j])), fabsf(E::hi(g[j]))));
      }
      *(u32x4_t*)((_Float16*)p.do16 + e) = E::to_f16x8(g);
      *(u32x4_t*)((_Float16*)p.q16 + e) = E::to_f16x8(q);
      *(u32x4_t*)((_Float16*)p.k16 + e) = E::to_f16x8(k);
    }
#pragma unroll
    for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
    if (live && c == 0) {
      const size_t s = (size_t)bh * p.N + i;
      const float L = p.lse[s];
      *(f32x2_t*)(p.stats + 2 * s) = f32x2_t{L == -INFINITY ? INFINITY : L * 1.4426950408889634f, acc};
    }
  }
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1)
#pragma unroll
    for (int t = 0; t < 4; ++t) mx[t] = fmaxf(mx[t], __shfl_xor(mx[t], sh, 64));
  if ((tid & 63) == 0) red[tid >> 6] = mx;
  __syncthreads();
  if (tid == 0) {
    f32x4_t r = red[0];
#pragma unroll
    for (int w = 1; w < 4; ++w)
#pragma unroll
      for (int t = 0; t < 4; ++t) r[t] = fmaxf(r[t], red[w][t]);
    *(f32x4_t*)(p.part + ((size_t)bh * kMaxParts + pb) * 4) = r;
  }
}

// Rewrites the fp16 copies of a slice that needs a power-of-two scale
// (range_exp above) and scales its D_i by 2^(e_dO + e_V), the factor dP
// carries in the dK/dV pass. kRescaleGroups work-groups per (b, h); one whose
// slice needs no scale returns at once (the common case costs one small
// launch).
constexpr int kRescaleGroups = 4;
template <int D, typename T>
__global__ void __launch_bounds__(256) bwd_rescale_kernel(BwdParams p) {
  constexpr int LPR = D / 8;
  constexpr int RPB = 256 / LPR;
  const int tid = threadIdx.x, c = tid % LPR;
  const int bh = blockIdx.x / kRescaleGroups, g = blockIdx.x - bh * kRescaleGroups;
  const int b = bh / p.H, h = bh - b * p.H;
  const SliceExp ex = slice_exp(p, bh);
  if ((ex.q | ex.k | ex.o | ex.v) == 0) return;
  for (int i = g * RPB + tid / LPR; i < p.N; i += kRescaleGroups * RPB) {
    const size_t bi = (size_t)b * p.N + i;
    const size_t hd = (size_t)h * D + 8 * c;
    const size_t e = (bi * p.H) * D + hd;
    const size_t eq = bi * p.rs_q + hd, eo = bi * p.rs_o + hd;
    if (ex.o) *(u32x4_t*)((_Float16*)p.do16 + e) = to_f16x8_scaled<T>(ld_global<u32x4_t>((const T*)p.dout + eo), ex.o);
    if (ex.q) *(u32x4_t*)((_Float16*)p.q16 + e) = to_f16x8_scaled<T>(ld_global<u32x4_t>((const T*)p.q + eq), ex.q);
    if (ex.k) *(u32x4_t*)((_Float16*)p.k16 + e) = to_f16x8_scaled<T>(ld_global<u32x4_t>((const T*)p.k + eq), ex.k);
    if (c == 0 && (ex.o + ex.v) != 0) {
      float* d = p.stats + 2 * ((size_t)bh * p.N + i) + 1;
      *d = ldexpf(*d, ex.o + ex.v);
    }
  }
}

// ---------------------------------------------------------------- dK, dV

// One wave per 32 keys; used at headdim 64, where K, V, dK and dV of the
// wave's keys and the tile's working set fit in 256 VGPRs (two waves per SIMD).
template <int D>
struct KvCfg {
  static constexpr int NW = 4;                 // waves per work-group, 32 keys each
  static constexpr int BK = NW * 32;           // keys per work-group
  static constexpr int BQ = 64;                // query rows per tile
  static constexpr int CPR = D / 8;            // 16-byte chunks per row
  static constexpr int TILE = BQ * D * 2;      // bytes of the fp16 Q or dO tile
  static constexpr int LPW = TILE / 1024 / NW; // 1 KiB direct-to-LDS loads per wave per matrix
  static constexpr int BUF = 2 * TILE + 1024;  // one buffer: Q | dO | statistics
  static constexpr int DS = D / 16, DB = D / 32, QS = BQ / 32, KS = BQ / 16;
  static_assert(LPW >= 1 && TILE % (1024 * NW) == 0, "tile must split into 1 KiB loads");
  static_assert(BQ * 8 <= 1024, "one 1 KiB load covers the tile's statistics");
};

// dK and dV of a block of NW * 32 keys. Per query tile and wave (32 keys):
//   S = Q K^T and dP = dO V^T       (A: Q / dO rows from LDS, B: K / V registers;
//                                    each lane then holds one key's column),
//   P = 2^(c2 S - LSE2), dS = P (dP - D)   (LSE2 = LSE log2 e, +inf for empty rows),
//   dV^T += dO^T P and dK^T += Q^T dS     (A: transposed LDS reads, B: P / dS
//                                    packed to fp16 straight from the accumulators).
// Query rows at or past N arrive as zeros (Q, dO and both statistics), which
// makes every term they add zero.
template <int D, bool ALIBI, typename T>
__device__ __forceinline__ void dkdv_block(const BwdParams& p, int nblk, int wg, char* smem) {
  using E = Elt16<T>;
  using C = KvCfg<D>;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 31, hf = lane >> 5;
  int bh, kblk;
  map_index(wg, p.B * p.H, nblk, p.xcd_groups, 0, bh, kblk);
  const int b = bh / p.H, h = bh - b * p.H;
  const int N = p.N;
  const int kl = key_len(p.mask, b, N);
  const int rs = p.H * D;                               // the fp16 copies
  const size_t base = ((size_t)b * N * p.H + h) * D;
  const size_t vbase = (size_t)b * N * p.rs_q + (size_t)h * D;
  const size_t gbase = (size_t)b * N * p.rs_g + (size_t)h * D;
  float slope2 = 0.f;  // ALiBi slope in the log2 domain of the exponent
  if constexpr (ALIBI) slope2 = alibi_raw_slope(p.alibi, b, h, p.scale_log2) * p.scale_log2;
  // Operand exponents of the slice: scores of the fp16 copies carry
  // 2^(e_Q + e_K), dP carries 2^(e_dO + e_V) (as does D_i after the rescale
  // pass), dV^T 2^e_dO and dK^T 2^(e_Q + e_dO + e_V).
  const SliceExp ex = slice_exp(p, bh);
  const float sl2 = ldexpf(p.scale_log2, -(ex.q + ex.k));

  // This lane's key, and its K and V rows as fp16 B operands:
  // kf[s] = K[key][16 s + 8 hf .. +8). Keys past N are clamped (and masked).
  const int k0 = kblk * C::BK, wk0 = k0 + wave * 32, wk1 = wk0 + 31;
  const int key = wk0 + ln;
  f16x8_t kf[C::DS], vf[C::DS];
  {
    const int kr = min(key, N - 1);
    const size_t off = base + (size_t)kr * rs + 8 * hf;
    const size_t voff = vbase + (size_t)kr * p.rs_q + 8 * hf;
#pragma unroll
    for (int s = 0; s < C::DS; ++s) {
      kf[s] = ld_global<f16x8_t>((const _Float16*)p.k16 + off + 16 * s);
      vf[s] = __builtin_bit_cast(f16x8_t, to_f16x8_scaled<T>(ld_global<u32x4_t>((const T*)p.v + voff + 16 * s), ex.v));
    }
  }

  // Queries that see a key of the work-group / of this wave: [lo, hi).
  int qlo = 0, qhi = 0, wqlo = 0, wqhi = 0;
  {
    const int klast = min(k0 + C::BK, kl) - 1;
    if (k0 <= klast) {
      qlo = p.mask.wr >= 0 ? max(0, k0 - p.mask.wr) : 0;
      qhi = p.mask.wl >= 0 ? min(N, klast + p.mask.wl + 1) : N;
    }
    const int wklast = min(wk1, kl - 1);
    if (wk0 <= wklast) {
      wqlo = p.mask.wr >= 0 ? max(0, wk0 - p.mask.wr) : 0;
      wqhi = p.mask.wl >= 0 ? min(N, wklast + p.mask.wl + 1) : N;
    }
  }
  const int t0 = qlo / C::BQ, t1 = qhi > qlo ? (qhi + C::BQ - 1) / C::BQ : t0;
  // Rows i that see this lane's key j: vqlo <= i <= vqhi (empty for j >= kl).
  const int vqlo = key >= kl ? INT_MAX : (p.mask.wr >= 0 ? key - p.mask.wr : 0);
  const int vqhi = p.mask.wl >= 0 ? key + p.mask.wl : INT_MAX;

  // Direct-to-LDS copies: load j of this wave fills chunks
  // [(wave * LPW + j) * 64, +64) of a tile, the swizzle applied to the global
  // chunk each lane fetches; the tile's first row goes in the scalar offset.
  // Wave 0 also copies the tile's statistics (8 bytes per row).
  const int rs2 = rs * 2;
  const int nbytes = ((N - 1) * rs + D) * 2;
  const __amdgpu_buffer_rsrc_t qrsrc = make_rsrc((const _Float16*)p.q16 + base, nbytes);
  const __amdgpu_buffer_rsrc_t orsrc = make_rsrc((const _Float16*)p.do16 + base, nbytes);
  const __amdgpu_buffer_rsrc_t srsrc = make_rsrc(p.stats + ((size_t)b * p.H + h) * N * 2, N * 8);
  int loff[C::LPW];
#pragma unroll
  for (int j = 0; j < C::LPW; ++j) {
    const int u = (wave * C::LPW + j) * 64 + lane, row = u / C::CPR, pos = u % C::CPR;
    loff[j] = row * rs2 + (pos ^ lds_swz<D>(row)) * 16;
  }
  auto issue_tile = [&](int t, auto bufc) __attribute__((always_inline)) {
    constexpr int buf = decltype(bufc)::value;
    char* sb = smem + buf * C::BUF;
    const int soff = t * C::BQ * rs2;
#pragma unroll
    for (int j = 0; j < C::LPW; ++j) {
      buffer_load_lds16(qrsrc, sb + (wave * C::LPW + j) * 1024, loff[j], soff);
      buffer_load_lds16(orsrc, sb + C::TILE + (wave * C::LPW + j) * 1024, loff[j], soff);
    }
    if (wave == 0)
      buffer_load_lds16(srsrc, sb + 2 * C::TILE, lane * 16,
                        __builtin_amdgcn_readfirstlane(t * C::BQ * 8));
  };

  // Operand offsets within a tile: row operand of d-step s is row ln, chunk
  // 2 s + hf; transposed operands as tile_tr_off. Both stay valid when a
  // multiple of 16 rows is added (the swizzle only sees the low 4 row bits).
  int roff[C::DS];
#pragma unroll
  for (int s = 0; s < C::DS; ++s) roff[s] = tile_chunk_off<D>(ln, 2 * s + hf);
  int troff[C::DB][2];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int t = 0; t < 2; ++t) troff[db][t] = tile_tr_off<D>(lane, db, t);

  f32x16_t dk[C::DB], dv[C::DB];  // dK^T, dV^T (rows d, column = this lane's key)
#pragma unroll
  for (int d = 0; d < C::DB; ++d) { dk[d] = f32x16_t{}; dv[d] = f32x16_t{}; }

  // One query tile. Tiles that every key of the work-group sees in full run
  // the EDGE = false body: one straight-line block with no branch, which lets
  // the scheduler overlap one sub-block's exponentials with another's MFMAs.
  // Other tiles run the EDGE = true body, which skips a wave with nothing to
  // do and applies the per-element mask in a branch when the wave's keys
  // need it.
  auto compute = [&](int t, auto bufc, auto edgec) __attribute__((always_inline)) {
    constexpr int buf = decltype(bufc)::value;
    constexpr bool EDGE = decltype(edgec)::value;
    const int qb = t * C::BQ;
    bool masked = false;
    if constexpr (EDGE) {
      if (!(qb < wqhi && qb + C::BQ > wqlo)) return;  // wave-uniform
      masked = !block_all_visible(p.mask, kl, qb, min(qb + C::BQ, N) - 1, wk0, wk1);
    }
    const char* sq = smem + buf * C::BUF;
    const char* so = sq + C::TILE;
    const float* st = (const float*)(sq + 2 * C::TILE);
    u32x4_t pk[C::KS], dsk[C::KS];
#pragma unroll
    for (int qs = 0; qs < C::QS; ++qs) {
      f32x16_t sa = f32x16_t{}, pa = f32x16_t{};
#pragma unroll
      for (int s = 0; s < C::DS; ++s) {
        const int off = qs * 32 * C::CPR * 16 + roff[s];
        sa = mfma_f16(*(const f16x8_t*)(sq + off), kf[s], sa);
        pa = mfma_f16(*(const f16x8_t*)(so + off), vf[s], pa);
      }
      // Element i of a lane is query row 8 (i / 4) + 4 hf + i % 4 of the
      // block; st2[2 g + u] holds the statistics of rows 8 g + 4 hf + 2 u, +1.
      f32x4_t st2[8];
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int u = 0; u < 2; ++u)
          st2[2 * g + u] = *(const f32x4_t*)(st + 2 * (32 * qs + 8 * g + 4 * hf + 2 * u));
      if (EDGE && masked) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int row = qb + 32 * qs + 8 * (i >> 2) + 4 * hf + (i & 3);
          sa[i] = ((row >= vqlo) & (row <= vqhi)) ? sa[i] : -INFINITY;
        }
      }
      // ALiBi: the exponent takes -slope log2(e) |i - j| (row i, key j).
      const float di = (float)(qb + 32 * qs + 4 * hf - key);
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const f32x4_t r = st2[i >> 1];  // rows of elements i and i + 1: (L2, D, L2, D)
        float x0 = fmaf(sa[i], sl2, -r[0]);
        float x1 = fmaf(sa[i + 1], sl2, -r[2]);
        if constexpr (ALIBI) {
          x0 = fmaf(fabsf(di + (float)(8 * (i >> 2) + (i & 3))), -slope2, x0);
          x1 = fmaf(fabsf(di + (float)(8 * (i >> 2) + (i & 3) + 1)), -slope2, x1);
        }
        const float p0 = exp2_fast(x0);
        const float p1 = exp2_fast(x1);
        const float s0 = p0 * (pa[i] - r[1]);
        const float s1 = p1 * (pa[i + 1] - r[3]);
        pk[2 * qs + (i >> 3)][(i & 7) >> 1] = pack_f16x2(p0, p1);
        dsk[2 * qs + (i >> 3)][(i & 7) >> 1] = pack_f16x2(s0, s1);
      }
    }
#pragma unroll
    for (int d = 0; d < C::DB; ++d)
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const int ro = ks * 16 * C::CPR * 16;
        const u32x2_t o0 = lds_read_tr16(so + ro + troff[d][0]), o1 = lds_read_tr16(so + ro + troff[d][1]);
        const u32x2_t q0 = lds_read_tr16(sq + ro + troff[d][0]), q1 = lds_read_tr16(sq + ro + troff[d][1]);
        dv[d] = mfma_f16(__builtin_bit_cast(f16x8_t, u32x4_t{o0[0], o0[1], o1[0], o1[1]}),
                      __builtin_bit_cast(f16x8_t, pk[ks]), dv[d]);
        dk[d] = mfma_f16(__builtin_bit_cast(f16x8_t, u32x4_t{q0[0], q0[1], q1[0], q1[1]}),
                      __builtin_bit_cast(f16x8_t, dsk[ks]), dk[d]);
      }
  };

  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  // Query tiles alternate between two LDS buffers (tile t0 + i in buffer i % 2):
  // each interval issues the copy of the next tile, computes the current one,
  // then waits for the copy and meets the others at the barrier.
  auto interval = [&](int t, auto cur, auto nxt, auto edgec) __attribute__((always_inline)) {
    if (t + 1 < t1) issue_tile(t + 1, nxt);
    compute(t, cur, edgec);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };
  auto run = [&](int ta, int tb, auto edgec) __attribute__((always_inline)) {
    int t = ta;
    if (t < tb && ((t - t0) & 1)) interval(t++, B1{}, B0{}, edgec);
    for (; t < tb; t += 2) {
      interval(t, B0{}, B1{}, edgec);
      if (t + 1 < tb) interval(t + 1, B1{}, B0{}, edgec);
    }
  };
  // [ta, tb): the tiles every key of the block sees in full (a contiguous
  // range: a causal or right window bound cuts the front, a left window the
  // back, key padding inside the block removes it).
  int ta = t1, tb = t1;
  if (k0 + C::BK - 1 < kl) {
    const int kb = k0 + C::BK - 1;
    ta = p.mask.wr >= 0 ? max(t0, (max(kb - p.mask.wr, 0) + C::BQ - 1) / C::BQ) : t0;
    tb = (p.mask.wl >= 0 && k0 + p.mask.wl < N - 1) ? (k0 + p.mask.wl + 1) / C::BQ : t1;
    ta = min(ta, t1);
    tb = max(min(tb, t1), ta);
  }
  if (t0 < t1) {
    issue_tile(t0, B0{});
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    run(t0, ta, std::true_type{});
    run(ta, tb, std::false_type{});
    run(tb, t1, std::true_type{});
  }

  // Lane holds dK^T / dV^T rows (d) 32 d + 8 g + 4 hf + (0..3) of its key.
  if (key < N) {
    T* dkrow = (T*)p.dk + gbase + (size_t)key * p.rs_g;
    T* dvrow = (T*)p.dv + gbase + (size_t)key * p.rs_g;
    const int xk = -(ex.q + ex.o + ex.v), xv = -ex.o;
    auto gk = [&](float a) { return ldexpf(a * p.scale, xk); };
    auto gv = [&](float a) { return ldexpf(a, xv); };
#pragma unroll
    for (int d = 0; d < C::DB; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = 32 * d + 8 * g + 4 * hf;
        *(u32x2_t*)(dkrow + col) =
            u32x2_t{E::pack2(gk(dk[d][4 * g]), gk(dk[d][4 * g + 1])),
                    E::pack2(gk(dk[d][4 * g + 2]), gk(dk[d][4 * g + 3]))};
        *(u32x2_t*)(dvrow + col) = u32x2_t{E::pack2(gv(dv[d][4 * g]), gv(dv[d][4 * g + 1])),
                                           E::pack2(gv(dv[d][4 * g + 2]), gv(dv[d][4 * g + 3]))};
      }
  }
}

// ---------------------------------------------------------------- dK, dV (wave pairs)

// 4-byte direct-to-LDS buffer load: lane i's dword lands at lds + 4 i (zero
// past the descriptor's end).
__device__ __forceinline__ void buffer_load_lds4(__amdgpu_buffer_rsrc_t r, void* lds, int voffset,
                                                 int soffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 4,
                                           voffset, soffset, 0, 0);
}

template <int D>
struct KvPairCfg {
  static constexpr int NP = 4;                 // wave pairs per work-group, 32 keys each
  static constexpr int NW = 2 * NP;            // waves per work-group
  static constexpr int BK = NP * 32;           // keys per work-group
  static constexpr int BQ = 64;                // query rows per tile
  static constexpr int CPR = D / 8;
  static constexpr int TILE = BQ * D * 2;      // bytes of the fp16 Q or dO tile
  static constexpr int LPW = TILE / 1024 / NW; // 1 KiB direct-to-LDS loads per wave per matrix
  static constexpr int BUF = 2 * TILE + 1024;  // one buffer: Q | dO | statistics
  static constexpr int XCH = (BQ / 16) * 64 * 16;  // one pair's P: KS 16-byte operands per lane
  static constexpr int DS = D / 16, DB = D / 32, QS = BQ / 32, KS = BQ / 16;
  static_assert(LPW >= 1 && TILE % (1024 * NW) == 0, "tile must split into 1 KiB loads");
};

// dK and dV with the work of 32 keys split over a pair of waves, so that
// each wave needs few enough registers for two waves to share a SIMD (at
// headdim 128 the one-wave form above holds K, V, dK and dV of its keys in
// more than the 256 VGPRs a wave can address):
//   wave 0 of a pair: S = Q K^T, P = 2^(c2 S - LSE2) (masked), P to LDS,
//                     then dV^T += dO^T P;
//   wave 1 of a pair: dP = dO V^T, then reads P back and forms
//                     dS = P (dP - D), then dK^T += Q^T dS.
// A work-group barrier between the two phases of a tile hands P over; the
// MFMA work is the same as in the one-wave form. P crosses in fp16, the
// precision of its own MFMA operand, so dS is formed from the P that dV uses.
// Each wave needs only one of a row's two statistics (LSE2 for P, D for dS),
// so a tile's statistics sit in LDS split by kind: one 16-byte read brings
// four rows' worth of the one a wave uses.
template <int D, bool ALIBI, typename T>
__device__ __forceinline__ void dkdv_pair_block(const BwdParams& p, int nblk, int wg, char* smem) {
  using E = Elt16<T>;
  using C = KvPairCfg<D>;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = wave % C::NP, role = wave / C::NP;
  const int ln = lane & 31, hf = lane >> 5;
  int bh, kblk;
  map_index(wg, p.B * p.H, nblk, p.xcd_groups, 0, bh, kblk);
  const int b = bh / p.H, h = bh - b * p.H;
  const int N = p.N;
  const int kl = key_len(p.mask, b, N);
  const int rs = p.H * D;                               // the fp16 copies
  const size_t base = ((size_t)b * N * p.H + h) * D;
  const size_t vbase = (size_t)b * N * p.rs_q + (size_t)h * D;
  const size_t gbase = (size_t)b * N * p.rs_g + (size_t)h * D;
  // Operand exponents of the slice (see the one-wave form).
  const SliceExp ex = slice_exp(p, bh);
  const float sl2 = ldexpf(p.scale_log2, -(ex.q + ex.k));
  float slope_raw = 0.f;  // in the units of the scaled scores
  if constexpr (ALIBI) slope_raw = alibi_raw_slope(p.alibi, b, h, sl2);

  // This lane's key; the wave's B operand is its K row (role 0) or V row
  // (role 1) in fp16. Keys past N are clamped (and masked).
  const int k0 = kblk * C::BK, wk0 = k0 + pair * 32, wk1 = wk0 + 31;
  const int key = wk0 + ln;
  f16x8_t kv[C::DS];
  {
    const int kr = min(key, N - 1);
    if (role == 0) {
      const size_t off = base + (size_t)kr * rs + 8 * hf;
#pragma unroll
      for (int s = 0; s < C::DS; ++s) kv[s] = ld_global<f16x8_t>((const _Float16*)p.k16 + off + 16 * s);
    } else {
      const size_t off = vbase + (size_t)kr * p.rs_q + 8 * hf;
#pragma unroll
      for (int s = 0; s < C::DS; ++s)
        kv[s] = __builtin_bit_cast(f16x8_t, to_f16x8_scaled<T>(ld_global<u32x4_t>((const T*)p.v + off + 16 * s), ex.v));
    }
  }

  // Queries that see a key of the work-group / of this pair: [lo, hi).
  int qlo = 0, qhi = 0, wqlo = 0, wqhi = 0;
  {
    const int klast = min(k0 + C::BK, kl) - 1;
    if (k0 <= klast) {
      qlo = p.mask.wr >= 0 ? max(0, k0 - p.mask.wr) : 0;
      qhi = p.mask.wl >= 0 ? min(N, klast + p.mask.wl + 1) : N;
    }
    const int wklast = min(wk1, kl - 1);
    if (wk0 <= wklast) {
      wqlo = p.mask.wr >= 0 ? max(0, wk0 - p.mask.wr) : 0;
      wqhi = p.mask.wl >= 0 ? min(N, wklast + p.mask.wl + 1) : N;
    }
  }
  const int t0 = qlo / C::BQ, t1 = qhi > qlo ? (qhi + C::BQ - 1) / C::BQ : t0;
  const int vqlo = key >= kl ? INT_MAX : (p.mask.wr >= 0 ? key - p.mask.wr : 0);
  const int vqhi = p.mask.wl >= 0 ? key + p.mask.wl : INT_MAX;

  const int rs2 = rs * 2;
  const int nbytes = ((N - 1) * rs + D) * 2;
  const __amdgpu_buffer_rsrc_t qrsrc = make_rsrc((const _Float16*)p.q16 + base, nbytes);
  const __amdgpu_buffer_rsrc_t orsrc = make_rsrc((const _Float16*)p.do16 + base, nbytes);
  const __amdgpu_buffer_rsrc_t srsrc = make_rsrc(p.stats + ((size_t)b * p.H + h) * N * 2, N * 8);
  int loff[C::LPW];
#pragma unroll
  for (int j = 0; j < C::LPW; ++j) {
    const int u = (wave * C::LPW + j) * 64 + lane, row = u / C::CPR, pos = u % C::CPR;
    loff[j] = row * rs2 + (pos ^ lds_swz<D>(row)) * 16;
  }
  auto issue_tile = [&](int t, auto bufc) __attribute__((always_inline)) {
    constexpr int buf = decltype(bufc)::value;
    char* sb = smem + buf * C::BUF;
    const int soff = t * C::BQ * rs2;
#pragma unroll
    for (int j = 0; j < C::LPW; ++j) {
      buffer_load_lds16(qrsrc, sb + (wave * C::LPW + j) * 1024, loff[j], soff);
      buffer_load_lds16(orsrc, sb + C::TILE + (wave * C::LPW + j) * 1024, loff[j], soff);
    }
    if (wave == 0) {  // the tile's (LSE2, D) pairs, split: LSE2 of its 64 rows, then their D
      const int so = __builtin_amdgcn_readfirstlane(t * C::BQ * 8);
      buffer_load_lds4(srsrc, sb + 2 * C::TILE, lane * 8, so);
      buffer_load_lds4(srsrc, sb + 2 * C::TILE + 4 * C::BQ, lane * 8 + 4, so);
    }
  };

  int roff[C::DS];
#pragma unroll
  for (int s = 0; s < C::DS; ++s) roff[s] = tile_chunk_off<D>(ln, 2 * s + hf);
  int troff[C::DB][2];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int t = 0; t < 2; ++t) troff[db][t] = tile_tr_off<D>(lane, db, t);

  f32x16_t acc[C::DB];  // role 0: dV^T, role 1: dK^T (rows d, column = this lane's key)
#pragma unroll
  for (int d = 0; d < C::DB; ++d) acc[d] = f32x16_t{};
  char* xch = smem + 2 * C::BUF + pair * C::XCH;  // this pair's P, [ks][lane] 16 bytes

  // One query tile (EDGE as in the one-wave form). Both waves of every pair
  // reach the hand-over barrier, active or not.
  auto compute = [&](int t, auto bufc, auto edgec) __attribute__((always_inline)) {
    constexpr int buf = decltype(bufc)::value;
    constexpr bool EDGE = decltype(edgec)::value;
    const int qb = t * C::BQ;
    bool active = true, masked = false;
    if constexpr (EDGE) {
      active = qb < wqhi && qb + C::BQ > wqlo;  // wave-uniform
      masked = !block_all_visible(p.mask, kl, qb, min(qb + C::BQ, N) - 1, wk0, wk1);
    }
    const char* sq = smem + buf * C::BUF;
    const char* so = sq + C::TILE;
    const float* st = (const float*)(sq + 2 * C::TILE);
    u32x4_t pk[C::KS];    // role 0: P as fp16 B operands
    f32x16_t pa[C::QS];   // role 1: dP
    if (active) {
      if (role == 0) {
        // The sub-blocks' chains alternate (slack for each operand read); the
        // first step takes a zero accumulator as its constant operand.
        f32x16_t sall[C::QS];
#pragma unroll
        for (int s = 0; s < C::DS; ++s)
#pragma unroll
          for (int qs = 0; qs < C::QS; ++qs)
            sall[qs] = mfma_f16(*(const f16x8_t*)(sq + qs * 32 * C::CPR * 16 + roff[s]), kv[s],
                                s == 0 ? f32x16_t{} : sall[qs]);
#pragma unroll
        for (int qs = 0; qs < C::QS; ++qs) {
          f32x16_t sa = sall[qs];
          if constexpr (ALIBI) {  // row i, key j: q.k - (slope / c) |i - j|
            const float di = (float)(qb + 32 * qs + 4 * hf - key);
#pragma unroll
            for (int i = 0; i < 16; ++i)
              sa[i] = fmaf(fabsf(di + (float)(8 * (i >> 2) + (i & 3))), -slope_raw, sa[i]);
          }
          f32x4_t l4[4];  // LSE2 of rows 8 g + 4 hf + (0..3) at l4[g]
#pragma unroll
          for (int g = 0; g < 4; ++g) l4[g] = *(const f32x4_t*)(st + 32 * qs + 8 * g + 4 * hf);
          if (EDGE && masked) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int row = qb + 32 * qs + 8 * (i >> 2) + 4 * hf + (i & 3);
              sa[i] = ((row >= vqlo) & (row <= vqhi)) ? sa[i] : -INFINITY;
            }
          }
#pragma unroll
          for (int i = 0; i < 16; i += 2) {
            const float p0 = exp2_fast(fmaf(sa[i], sl2, -l4[i >> 2][i & 3]));
            const float p1 = exp2_fast(fmaf(sa[i + 1], sl2, -l4[i >> 2][(i & 3) + 1]));
            pk[2 * qs + (i >> 3)][(i & 7) >> 1] = pack_f16x2(p0, p1);
          }
        }
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) *(u32x4_t*)(xch + (ks * 64 + lane) * 16) = pk[ks];
      } else {
#pragma unroll
        for (int s = 0; s < C::DS; ++s)
#pragma unroll
          for (int qs = 0; qs < C::QS; ++qs)
            pa[qs] = mfma_f16(*(const f16x8_t*)(so + qs * 32 * C::CPR * 16 + roff[s]), kv[s],
                              s == 0 ? f32x16_t{} : pa[qs]);
      }
    }
    __syncthreads();  // P of every pair is in LDS
    if (active) {
      if (role == 0) {
#pragma unroll
        for (int d = 0; d < C::DB; ++d)
#pragma unroll
          for (int ks = 0; ks < C::KS; ++ks) {
            const int ro = ks * 16 * C::CPR * 16;
            const u32x2_t o0 = lds_read_tr16(so + ro + troff[d][0]), o1 = lds_read_tr16(so + ro + troff[d][1]);
            acc[d] = mfma_f16(__builtin_bit_cast(f16x8_t, u32x4_t{o0[0], o0[1], o1[0], o1[1]}),
                              __builtin_bit_cast(f16x8_t, pk[ks]), acc[d]);
          }
      } else {
        u32x4_t dsk[C::KS];
#pragma unroll
        for (int qs = 0; qs < C::QS; ++qs) {
          f32x4_t d4[4];  // D of rows 8 g + 4 hf + (0..3) at d4[g]
#pragma unroll
          for (int g = 0; g < 4; ++g) d4[g] = *(const f32x4_t*)(st + C::BQ + 32 * qs + 8 * g + 4 * hf);
#pragma unroll
          for (int hk = 0; hk < 2; ++hk) {
            const int ks = 2 * qs + hk;
            const u32x4_t pp = *(const u32x4_t*)(xch + (ks * 64 + lane) * 16);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int i = 8 * hk + 2 * e;  // elements i, i + 1 of this qs
              const f16x8_t ph = __builtin_bit_cast(f16x8_t, pp);
              const float s0 = (float)ph[2 * e] * (pa[qs][i] - d4[i >> 2][i & 3]);
              const float s1 = (float)ph[2 * e + 1] * (pa[qs][i + 1] - d4[i >> 2][(i & 3) + 1]);
              dsk[ks][e] = pack_f16x2(s0, s1);
            }
          }
        }
#pragma unroll
        for (int d = 0; d < C::DB; ++d)
#pragma unroll
          for (int ks = 0; ks < C::KS; ++ks) {
            const int ro = ks * 16 * C::CPR * 16;
            const u32x2_t q0 = lds_read_tr16(sq + ro + troff[d][0]), q1 = lds_read_tr16(sq + ro + troff[d][1]);
            acc[d] = mfma_f16(__builtin_bit_cast(f16x8_t, u32x4_t{q0[0], q0[1], q1[0], q1[1]}),
                              __builtin_bit_cast(f16x8_t, dsk[ks]), acc[d]);
          }
      }
    }
  };

  // Query tiles alternate between two LDS buffers (tile t0 + i in buffer
  // i % 2): each interval issues the copy of the next tile, computes the
  // current one, waits for the copy and meets the others at the barrier.
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  auto interval = [&](int t, auto cur, auto nxt, auto edgec) __attribute__((always_inline)) {
    if (t + 1 < t1) issue_tile(t + 1, nxt);
    compute(t, cur, edgec);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };
  auto run = [&](int ta, int tb, auto edgec) __attribute__((always_inline)) {
    int t = ta;
    if (t < tb && ((t - t0) & 1)) interval(t++, B1{}, B0{}, edgec);
    for (; t < tb; t += 2) {
      interval(t, B0{}, B1{}, edgec);
      if (t + 1 < tb) interval(t + 1, B1{}, B0{}, edgec);
    }
  };
  // [ta, tb): the tiles every key of the block sees in full (a contiguous
  // range: a causal or right window bound cuts the front, a left window the
  // back, key padding inside the block removes it).
  int ta = t1, tb = t1;
  if (k0 + C::BK - 1 < kl) {
    const int kb = k0 + C::BK - 1;
    ta = p.mask.wr >= 0 ? max(t0, (max(kb - p.mask.wr, 0) + C::BQ - 1) / C::BQ) : t0;
    tb = (p.mask.wl >= 0 && k0 + p.mask.wl < N - 1) ? (k0 + p.mask.wl + 1) / C::BQ : t1;
    ta = min(ta, t1);
    tb = max(min(tb, t1), ta);
  }
  if (t0 < t1) {
    issue_tile(t0, B0{});
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    run(t0, ta, std::true_type{});
    run(ta, tb, std::false_type{});
    run(tb, t1, std::true_type{});
  }

  // Lane holds dV^T (role 0) or dK^T (role 1) rows 32 d + 8 g + 4 hf + (0..3)
  // of its key.
  if (key < N) {
    const float sc = role == 0 ? 1.f : p.scale;
    const int xs = role == 0 ? -ex.o : -(ex.q + ex.o + ex.v);
    auto gs = [&](float a) { return ldexpf(a * sc, xs); };
    T* row = (T*)(role == 0 ? p.dv : p.dk) + gbase + (size_t)key * p.rs_g;
#pragma unroll
    for (int d = 0; d < C::DB; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = 32 * d + 8 * g + 4 * hf;
        *(u32x2_t*)(row + col) =
            u32x2_t{E::pack2(gs(acc[d][4 * g]), gs(acc[d][4 * g + 1])),
                    E::pack2(gs(acc[d][4 * g + 2]), gs(acc[d][4 * g + 3]))};
      }
  }
}

// ---------------------------------------------------------------- dQ

template <int D>
struct DqCfg {
  static constexpr int NW = D == 128 ? 8 : 4;  // waves per work-group, 32 queries each
  static constexpr int BM = NW * 32;           // query rows per work-group
  static constexpr int BN = 64;                // keys per tile
  static constexpr int CPR = D / 8;
  static constexpr int TILE = BN * D * 2;      // bytes of one K (fp16) or V (bf16) tile
  static constexpr int LPW = TILE / 1024 / NW; // 1 KiB direct-to-LDS loads per wave per matrix
  static constexpr int DS = D / 16, DB = D / 32, KB = BN / 32, KS = BN / 16;
  static_assert(LPW >= 1 && TILE % (1024 * NW) == 0, "tile must split into 1 KiB loads");
};

// dQ of a block of NW * 32 queries, in the forward's orientation: per key
// tile and wave,
//   S^T = K Q^T and dP^T = V dO^T      (A: K / V rows from LDS, B: Q / dO
//                                       registers; each lane holds one query),
//   P = 2^(c2 S - LSE2), dS^T = P (dP^T - D),
//   dQ^T += K^T dS^T                    (A: transposed K reads; B: dS^T packed
//                                       to fp16 from the accumulators).
// K comes from the fp16 copy (its products meet dS), V stays bf16.
template <int D, bool ALIBI, typename T>
__device__ __forceinline__ void dq_block(const BwdParams& p, int nblk, int wg, char* smem) {
  using E = Elt16<T>;
  using vec8 = typename E::vec8;
  using C = DqCfg<D>;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 31, hf = lane >> 5;
  int bh, qblk;
  map_index(wg, p.B * p.H, nblk, p.xcd_groups, p.mask.wr >= 0, bh, qblk);
  const int b = bh / p.H, h = bh - b * p.H;
  const int N = p.N;
  const int kl = key_len(p.mask, b, N);
  const int rs = p.H * D;                               // the fp16 copies
  const size_t base = ((size_t)b * N * p.H + h) * D;
  const size_t obase = (size_t)b * N * p.rs_o + (size_t)h * D;
  const size_t vbase = (size_t)b * N * p.rs_q + (size_t)h * D;
  const size_t gbase = (size_t)b * N * p.rs_g + (size_t)h * D;
  // Operand exponents of the slice: S from the fp16 copies carries
  // 2^(e_Q + e_K); dP comes from the raw V and dO, and dS is formed as
  // P 2^(e_dO + e_V) (dP - D), the scale dK/dV's dS has (and within fp16's
  // range); dQ^T = K^T dS^T then carries 2^(e_K + e_dO + e_V).
  const SliceExp ex = slice_exp(p, bh);
  const float sl2 = ldexpf(p.scale_log2, -(ex.q + ex.k));
  float slope_raw = 0.f;  // in the units of the scaled scores
  if constexpr (ALIBI) slope_raw = alibi_raw_slope(p.alibi, b, h, sl2);

  const int q0 = qblk * C::BM, wq0 = q0 + wave * 32;
  int klo, khi;
  key_range(p.mask, kl, q0, min(q0 + C::BM, N) - 1, klo, khi);
  const int t0 = klo / C::BN, t1 = (khi + C::BN - 1) / C::BN;
  const int wq1 = min(wq0 + 31, N - 1);
  int wklo = 0, wkhi = 0;
  if (wq0 <= wq1) key_range(p.mask, kl, wq0, wq1, wklo, wkhi);

  // This lane's query row: Q (fp16) and dO (bf16) as B operands, LSE2 and D.
  const int qi = wq0 + ln, qrow = min(qi, N - 1);
  f16x8_t qf[C::DS];
  vec8 of[C::DS];
  {
    const size_t off = base + (size_t)qrow * rs + 8 * hf;
    const size_t ooff = obase + (size_t)qrow * p.rs_o + 8 * hf;
#pragma unroll
    for (int s = 0; s < C::DS; ++s) {
      qf[s] = ld_global<f16x8_t>((const _Float16*)p.q16 + off + 16 * s);
      of[s] = ld_global<vec8>((const T*)p.dout + ooff + 16 * s);
    }
  }
  const f32x2_t st = ld_global<f32x2_t>(p.stats + 2 * (((size_t)b * p.H + h) * N + qrow));
  // D_i arrives scaled by 2^(e_dO + e_V) (the rescale pass); dS takes the
  // same factor as fma(dP, 2^(e_dO + e_V), -D_i): the power of two is exact,
  // so the scaled dS is the unscaled one times that power.
  const float lse2 = qi >= N ? INFINITY : st[0], dr = st[1];
  const float spv = ldexpf(1.f, ex.o + ex.v);

  // K (fp16 copy) and V (input) rows sit rs and rs_q elements apart.
  const int krs2 = rs * 2, vrs2 = p.rs_q * 2;
  const __amdgpu_buffer_rsrc_t krsrc =
      make_rsrc((const _Float16*)p.k16 + base, ((N - 1) * rs + D) * 2);
  const __amdgpu_buffer_rsrc_t vrsrc =
      make_rsrc((const T*)p.v + vbase, ((N - 1) * p.rs_q + D) * 2);
  int kloff[C::LPW], vloff[C::LPW];
#pragma unroll
  for (int j = 0; j < C::LPW; ++j) {
    const int u = (wave * C::LPW + j) * 64 + lane, row = u / C::CPR, pos = u % C::CPR;
    kloff[j] = row * krs2 + (pos ^ lds_swz<D>(row)) * 16;
    vloff[j] = row * vrs2 + (pos ^ lds_swz<D>(row)) * 16;
  }
  auto issue_tile = [&](int t, auto bufc) __attribute__((always_inline)) {
    constexpr int buf = decltype(bufc)::value;
    char* kd = smem + (2 * buf) * C::TILE + wave * C::LPW * 1024;
    char* vd = kd + C::TILE;
#pragma unroll
    for (int j = 0; j < C::LPW; ++j) {
      buffer_load_lds16(krsrc, kd + j * 1024, kloff[j], t * C::BN * krs2);
      buffer_load_lds16(vrsrc, vd + j * 1024, vloff[j], t * C::BN * vrs2);
    }
  };

  int roff[C::DS];
#pragma unroll
  for (int s = 0; s < C::DS; ++s) roff[s] = tile_chunk_off<D>(ln, 2 * s + hf);
  int troff[C::DB][2];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int t = 0; t < 2; ++t) troff[db][t] = tile_tr_off<D>(lane, db, t);

  f32x16_t dq[C::DB];
#pragma unroll
  for (int d = 0; d < C::DB; ++d) dq[d] = f32x16_t{};

  auto compute = [&](int t, auto bufc) __attribute__((always_inline)) {
    constexpr int buf = decltype(bufc)::value;
    const char* sk = smem + (2 * buf) * C::TILE;
    const char* sv = sk + C::TILE;
    const int kt = t * C::BN;
    if (!(kt < wkhi && kt + C::BN > wklo)) return;  // wave-uniform
    const bool masked = !block_all_visible(p.mask, kl, wq0, wq1, kt, kt + C::BN - 1);
    u32x4_t dsk[C::KS];
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb) {
      f32x16_t sa = f32x16_t{}, pa = f32x16_t{};
#pragma unroll
      for (int s = 0; s < C::DS; ++s) {
        const int off = kb * 32 * C::CPR * 16 + roff[s];
        sa = mfma_f16(*(const f16x8_t*)(sk + off), qf[s], sa);
        pa = E::mfma(*(const vec8*)(sv + off), of[s], pa);
      }
      if constexpr (ALIBI) {  // row i, key j: q.k - (slope / c) |i - j|
        const float di = (float)(qi - kt - 32 * kb - 4 * hf);
#pragma unroll
        for (int i = 0; i < 16; ++i)
          sa[i] = fmaf(fabsf(di - (float)(8 * (i >> 2) + (i & 3))), -slope_raw, sa[i]);
      }
      if (masked) {
        int lo, hi;
        visible_span(p.mask, kl, qi, lo, hi);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int j = kt + 32 * kb + 8 * (i >> 2) + 4 * hf + (i & 3);
          sa[i] = ((j >= lo) & (j <= hi)) ? sa[i] : -INFINITY;
        }
      }
#pragma unroll
      for (int i = 0; i < 16; i += 2) {
        const float p0 = exp2_fast(fmaf(sa[i], sl2, -lse2));
        const float p1 = exp2_fast(fmaf(sa[i + 1], sl2, -lse2));
        dsk[2 * kb + (i >> 3)][(i & 7) >> 1] =
            pack_f16x2(p0 * fmaf(pa[i], spv, -dr), p1 * fmaf(pa[i + 1], spv, -dr));
      }
    }
#pragma unroll
    for (int d = 0; d < C::DB; ++d)
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const int ro = ks * 16 * C::CPR * 16;
        const u32x2_t k0 = lds_read_tr16(sk + ro + troff[d][0]), k1 = lds_read_tr16(sk + ro + troff[d][1]);
        dq[d] = mfma_f16(__builtin_bit_cast(f16x8_t, u32x4_t{k0[0], k0[1], k1[0], k1[1]}),
                         __builtin_bit_cast(f16x8_t, dsk[ks]), dq[d]);
      }
  };

  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  auto interval = [&](int t, auto cur, auto nxt) __attribute__((always_inline)) {
    if (t + 1 < t1) issue_tile(t + 1, nxt);
    compute(t, cur);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };
  if (t0 < t1) {
    issue_tile(t0, B0{});
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    for (int t = t0; t < t1; t += 2) {
      interval(t, B0{}, B1{});
      if (t + 1 < t1) interval(t + 1, B1{}, B0{});
    }
  }

  if (qi < N) {
    T* row = (T*)p.dq + gbase + (size_t)qi * p.rs_g;
    const int xq = -(ex.k + ex.o + ex.v);
    auto gq = [&](float a) { return ldexpf(a * p.scale, xq); };
#pragma unroll
    for (int d = 0; d < C::DB; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = 32 * d + 8 * g + 4 * hf;
        *(u32x2_t*)(row + col) =
            u32x2_t{E::pack2(gq(dq[d][4 * g]), gq(dq[d][4 * g + 1])),
                    E::pack2(gq(dq[d][4 * g + 2]), gq(dq[d][4 * g + 3]))};
      }
  }
}

// ---------------------------------------------------------------- kernels

// dK/dV and dQ in one grid: the B H nblk_kv dK/dV work-groups first, then the
// B H nblk_q dQ work-groups. The two passes read the same pre-pass outputs and
// write disjoint gradients, so nothing orders them; in one grid the dQ groups
// (longest first under a causal mask) start as soon as dK/dV groups retire,
// which fills the tail that a causal mask leaves in each pass on its own
// (one launch instead of two). The groups of both kinds have the same size;
// LDS is the larger of the two layouts.
template <int D>
struct KvqShape {
  static constexpr int NW = D == 128 ? KvPairCfg<D>::NW : KvCfg<D>::NW;
  static constexpr int KV_LDS = D == 128 ? 2 * KvPairCfg<D>::BUF + KvPairCfg<D>::NP * KvPairCfg<D>::XCH
                                         : 2 * KvCfg<D>::BUF;
  static constexpr int Q_LDS = 2 * 2 * DqCfg<D>::TILE;
  static constexpr int LDS = KV_LDS > Q_LDS ? KV_LDS : Q_LDS;
  static_assert(NW == DqCfg<D>::NW, "dK/dV and dQ work-groups must have the same size");
};

template <int D, bool ALIBI, typename T>
__global__ void __launch_bounds__(KvqShape<D>::NW * 64) bwd_kvq_kernel(BwdParams p, int nblk_kv, int nblk_q) {
  __shared__ __attribute__((aligned(1024))) char smem[KvqShape<D>::LDS];
  const int nkv = p.B * p.H * nblk_kv;
  const int i = blockIdx.x;
  if (i < nkv) {
    if constexpr (D == 128) dkdv_pair_block<D, ALIBI, T>(p, nblk_kv, i, smem);
    else dkdv_block<D, ALIBI, T>(p, nblk_kv, i, smem);
  } else {
    dq_block<D, ALIBI, T>(p, nblk_q, i - nkv, smem);
  }
}

// ---------------------------------------------------------------- launcher

template <int D, bool ALIBI, typename T>
static hipError_t launch_backward_d(BwdParams p, hipStream_t stream) {
  // Pre-pass blocks: at most kMaxParts per (b, h), each a whole number of
  // 256-thread passes (256 / (D / 8) rows each).
  constexpr int rpb = 256 / (D / 8);
  const int passes = (p.N + kMaxParts * rpb - 1) / (kMaxParts * rpb);
  p.prows = passes * rpb;
  p.np = (p.N + p.prows - 1) / p.prows;
  const dim3 pgrid((unsigned)((long long)p.B * p.H * p.np));
  hipLaunchKernelGGL((bwd_prep_kernel<D, T>), pgrid, dim3(256), 0, stream, p);
  hipLaunchKernelGGL((bwd_rescale_kernel<D, T>), dim3((unsigned)((long long)p.B * p.H * kRescaleGroups)),
                     dim3(256), 0, stream, p);
  // Measured on MI355X: the one-wave dK/dV form is faster at headdim 64 (two
  // waves per SIMD either way, half the barriers); at headdim 128 only the
  // pair form keeps its state in VGPRs.
  const int nblk_kv = (p.N + (D == 128 ? KvPairCfg<D>::BK : KvCfg<D>::BK) - 1) /
                      (D == 128 ? KvPairCfg<D>::BK : KvCfg<D>::BK);
  const int nblk_q = (p.N + DqCfg<D>::BM - 1) / DqCfg<D>::BM;
  hipLaunchKernelGGL((bwd_kvq_kernel<D, ALIBI, T>), dim3((unsigned)((long long)p.B * p.H * (nblk_kv + nblk_q))),
                     dim3(KvqShape<D>::NW * 64), 0, stream, p, nblk_kv, nblk_q);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_backward_t(BwdParams p, int headdim, hipStream_t stream) {
  const bool alibi = p.alibi.slopes != nullptr;
  if (headdim == 64)
    return alibi ? launch_backward_d<64, true, T>(p, stream) : launch_backward_d<64, false, T>(p, stream);
  return alibi ? launch_backward_d<128, true, T>(p, stream) : launch_backward_d<128, false, T>(p, stream);
}

hipError_t launch_backward(BwdParams p, int headdim, ElemType et, hipStream_t stream) {
  if (et == ElemType::kF32) return hipErrorNotSupported;
  if (et == ElemType::kF16) return launch_backward_t<_Float16>(p, headdim, stream);
  return launch_backward_t<__bf16>(p, headdim, stream);
}

}  // namespace fa
