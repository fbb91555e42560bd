// fa_fwd_fp8.hip -- tiled exact-attention forward over fp8 (e4m3) inputs for gfx950.
//
// The same algorithm as the bf16 forward (interview guide "FlashAttention
// 深入", "v1 → v2 → v3 演进": FP8 is one of the v3 additions; l189.com
// from-scratch article §3.1 blocked forward with the LSE statistic, §2.2
// online softmax): one work-group per (batch, head, block of query rows), K
// and V streamed through LDS in 64-key tiles, S and O accumulated in fp32.
//
// Inputs are OCP e4m3 bytes, each tensor with one fp32 dequantisation factor
// (the value of a byte x is e4m3(x) * descale). Both products run on the
// gfx950 fp8 MFMA (32x32x64, fp32 accumulation):
//   S^T = K Q^T over raw bytes; the factor c * dq * dk is folded into the
//         exponent's scale, so the fp32 scores are exact sums of exact
//         products;
//   O^T += V^T P^T with P quantised to e4m3 (round to nearest even). The
//         library's accuracy contract (include/fa.h) lets each weight w
//         enter as e4m3(c w) / c for any factor c with c w <= 448 and
//         c w_max >= 1. Here P is taken as 2^(c2 s - M + 3) against a
//         reference M that is the exact running row max as of some earlier
//         tile, so c = 2^(3 + M_row - M) / w_max >= 2^3 / w_max: (ii) holds
//         with room to spare. A tile first uses the current M without
//         computing its own max; only if some lane's sum of P exceeds 448
//         (e4m3's largest value, so one P might) is M raised to the exact
//         running max, O and l rescaled, and the tile's P recomputed, each
//         then at most 2^3, which keeps (i). M starts at -1e30, so a row's
//         first tile with a visible key takes that path. Skipping the max on
//         the common path saves VALU work, which bounds this kernel. dv and
//         1 / l are applied in the epilogue; l sums the unrounded fp32 P, so
//         the LSE does not see the quantisation.
//
// Operand layouts (measured on gfx950): in the 32x32x64 fp8 MFMA lane l
// supplies 32 bytes of row l % 32 of A (and of column l % 32 of B), and byte
// j of lane l pairs with byte j of the lane with the same l / 32 in the other
// operand; the 16 output values per lane sit where the bf16 32x32 MFMA puts
// them. The contraction order inside one MFMA is therefore free as long as A
// and B agree: the S product takes d = 64 s + 32 (l / 32) + j, and the P V
// product takes key 32 (l / 32) + j. For the latter, row r of the 32-row
// S^T block kb is loaded from key sigma(32 kb + r), chosen so that the
// accumulator value i of block kb in lane l is key 32 (l / 32) + 16 kb + i:
// P then packs into the B operand in plain byte order. V^T is read with
// ds_read_b64_tr_b8: in each 16-lane group, lane i receives byte i % 8 of the
// 8-byte rows addressed by lanes 2 e + (i / 8) % 2, e = 0..7.

#include <type_traits>

#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

typedef __attribute__((ext_vector_type(8))) int i32x8_t;
typedef __attribute__((ext_vector_type(2))) int i32x2_t;
typedef __attribute__((address_space(3))) i32x2_t lds_i32x2_t;

template <int D, int NW_ = (D == 128 ? 8 : 4)>
struct Fp8Cfg {
  static constexpr int NW = NW_;               // waves per work-group
  static constexpr int QW = 32;                // query rows per wave
  static constexpr int BM = NW * QW;           // query rows per work-group
  static constexpr int BN = 64;                // keys per tile
  static constexpr int CPR = D / 16;           // 16-byte chunks per K/V row
  static constexpr int TILE = BN * D;          // bytes of one K or V tile
  static constexpr int DS = D / 64;            // 64-deep steps of the S product
  static constexpr int DB = D / 32;            // 32-wide d blocks of O
  static constexpr int LPW = TILE / 1024 / NW; // 1 KiB direct-to-LDS loads per wave per matrix
  static_assert(LPW >= 1 && TILE == LPW * NW * 1024, "tile must split into 1 KiB loads");
};

// LDS tiles: [64 keys][D bytes], 16-byte chunks XOR-swizzled per row. With a
// 256-byte bank window, the K swizzle keeps the 16 rows that 16 lanes read in
// one S operand read on distinct banks, and the V swizzle does the same for
// the 8 rows x 2 chunks of two 16-lane groups of a transposed read.
template <int D>
__device__ __forceinline__ int swz_k(int r) {
  if constexpr (D == 128) return ((r >> 1) & 3) | (((r >> 5) & 1) << 2);
  else return ((r >> 2) & 1) | (((r >> 5) & 1) << 1);
}
template <int D>
__device__ __forceinline__ int swz_v(int r) {
  if constexpr (D == 128) return ((r >> 1) & 3) << 1;
  else return ((r >> 2) & 1) << 1;
}

__device__ __forceinline__ f32x16_t mfma_fp8(i32x8_t a, i32x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ i32x8_t cat16(u32x4_t lo, u32x4_t hi) {
  return i32x8_t{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                 (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

__device__ __forceinline__ i32x2_t lds_read_tr8(const void* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2_t*)p);
}

// Four fp32 values -> four e4m3 bytes (round to nearest even), first value
// in the lowest byte. The two converts write the low and the high half of the
// word, so its prior contents never matter; the builtin takes them as an
// input, which costs a register clear per word, so the first convert is
// written out with a plain output operand.
__device__ __forceinline__ int pack_fp8x4(float a, float b, float c, float d) {
  int w;
  asm("v_cvt_pk_fp8_f32 %0, %1, %2" : "=v"(w) : "v"(a), "v"(b));
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

// Four waves (128 query rows) per work-group at both head dimensions, held
// to at most 168 VGPRs (three waves per SIMD, so three such work-groups fit on
// a CU). This measured faster than eight-wave groups (two waves per SIMD).
template <int D>
using Fp8Shape = Fp8Cfg<D, 4>;

template <int D>
__global__ void __launch_bounds__(Fp8Shape<D>::NW * 64) __attribute__((amdgpu_waves_per_eu(3))) fwd_fp8_kernel(FwdParams p, float v_descale) {
  using C = Fp8Shape<D>;
  __shared__ __attribute__((aligned(1024))) char smem[4 * C::TILE];  // [buf][K | V]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ln = lane & 31, hf = lane >> 5;
  int bh, qblk;
  map_block(p.B * p.H, p.nqb, p.xcd_groups, p.longest_first, bh, qblk);
  const int b = bh / p.H, h = bh - b * p.H;
  const int N = p.N;
  const int q0 = qblk * C::BM;
  const int kl = key_len(p.mask, b, N);
  const int rs = p.rs_q;                                // bytes between sequence positions
  const size_t base = (size_t)b * N * rs + (size_t)h * D;
  const char* Q = (const char*)p.q + base;
  const char* Kg = (const char*)p.k + base;
  const char* Vg = (const char*)p.v + base;
  __bf16* O = (__bf16*)p.o + (size_t)b * N * p.rs_o + (size_t)h * D;

  const int wq0 = q0 + wave * C::QW;
  int klo, khi;
  key_range(p.mask, kl, q0, min(q0 + C::BM, N) - 1, klo, khi);
  const int t0 = klo / C::BN, t1 = (khi + C::BN - 1) / C::BN;
  const int wq1 = min(wq0 + C::QW - 1, N - 1);
  int wklo = 0, wkhi = 0;
  if (wq0 <= wq1) key_range(p.mask, kl, wq0, wq1, wklo, wkhi);

  // Q as the B operand of S^T = K Q^T: qf[s] = Q[wq0 + ln][64 s + 32 hf ..+32).
  i32x8_t qf[C::DS];
  {
    const int row = min(wq0 + ln, N - 1);  // rows past N are computed, never stored
#pragma unroll
    for (int s = 0; s < C::DS; ++s) {
      const char* src = Q + (size_t)row * rs + 64 * s + 32 * hf;
      qf[s] = cat16(ld_global<u32x4_t>(src), ld_global<u32x4_t>(src + 16));
    }
  }

  // Direct-to-LDS copies: load j of a wave fills LDS chunk
  // u = 64 (LPW wave + j) + lane of a tile (row u / CPR, position u % CPR)
  // with the global chunk that the row's swizzle puts there. Rows at or past
  // N read as zero.
  const int nbytes = (N - 1) * rs + D;
  const __amdgpu_buffer_rsrc_t krsrc = make_rsrc(Kg, nbytes);
  const __amdgpu_buffer_rsrc_t vrsrc = make_rsrc(Vg, nbytes);
  int kload[C::LPW], vload[C::LPW];
#pragma unroll
  for (int j = 0; j < C::LPW; ++j) {
    const int u = (wave * C::LPW + j) * 64 + lane, row = u / C::CPR, pos = u % C::CPR;
    kload[j] = row * rs + (pos ^ swz_k<D>(row)) * 16;
    vload[j] = row * rs + (pos ^ swz_v<D>(row)) * 16;
  }
  auto issue_tile = [&](int t, auto bufc) __attribute__((always_inline)) {
    constexpr int buf = decltype(bufc)::value;
    const int soff = t * C::BN * rs;
    char* kd = smem + (2 * buf) * C::TILE + wave * C::LPW * 1024;
    char* vd = smem + (2 * buf + 1) * C::TILE + wave * C::LPW * 1024;
#pragma unroll
    for (int j = 0; j < C::LPW; ++j) {
      buffer_load_lds16(krsrc, kd + j * 1024, kload[j], soff);
      buffer_load_lds16(vrsrc, vd + j * 1024, vload[j], soff);
    }
  };

  // LDS read offsets. S operand of block kb, step s: key row
  // sigma(32 kb + ln) = 32 ((ln >> 2) & 1) + 16 kb + 4 (ln >> 3) + (ln & 3),
  // chunks 4 s + 2 hf and 4 s + 2 hf + 1. The swizzle does not depend on kb,
  // so block kb is block 0 moved by 16 rows.
  int koff[C::DS][2];
  {
    const int r = 32 * ((ln >> 2) & 1) + 4 * (ln >> 3) + (ln & 3);
#pragma unroll
    for (int s = 0; s < C::DS; ++s)
#pragma unroll
      for (int e = 0; e < 2; ++e) koff[s][e] = (r * C::CPR + ((4 * s + 2 * hf + e) ^ swz_k<D>(r))) * 16;
  }
  // V^T operand of d block db, read u (u = 0..3): lane 16 g + 2 e + o
  // addresses key row 32 (g / 2) + 8 u + e at byte 32 db + 16 (g % 2) + 8 o.
  // The swizzle does not depend on u.
  int voff[C::DB];
  {
    const int g = lane >> 4, e = (lane & 15) >> 1, o = lane & 1;
    const int r = 32 * (g >> 1) + e;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
      voff[db] = (r * C::CPR + ((2 * db + (g & 1)) ^ swz_v<D>(r))) * 16 + 8 * o;
  }

  f32x16_t oacc[C::DB];
#pragma unroll
  for (int d = 0; d < C::DB; ++d) oacc[d] = f32x16_t{};
  float m_ref = -1e30f, l_part = 0.f;
  f32x16_t sacc[2];

  // start(t): S^T = K(t) Q^T, masked on tiles that cross a mask edge. The
  // accumulator value i of block kb in lane (ln, hf) is the score of query
  // wq0 + ln and key kt + 32 hf + 16 kb + i.
  auto start = [&](int t, auto bufc) __attribute__((always_inline)) {
    constexpr int buf = decltype(bufc)::value;
    const char* sk = smem + (2 * buf) * C::TILE;
    const int kt = t * C::BN;
    sacc[0] = f32x16_t{};
    sacc[1] = f32x16_t{};
#pragma unroll
    for (int s = 0; s < C::DS; ++s)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const char* rowp = sk + kb * 16 * C::CPR * 16;
        const i32x8_t kop = cat16(*(const u32x4_t*)(rowp + koff[s][0]), *(const u32x4_t*)(rowp + koff[s][1]));
        sacc[kb] = mfma_fp8(kop, qf[s], sacc[kb]);
      }
    if (!block_all_visible(p.mask, kl, wq0, wq1, kt, kt + C::BN - 1)) {
      int lo, hi;
      visible_span(p.mask, kl, wq0 + ln, lo, hi);
      const int jb = kt + 32 * hf;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int j = jb + 16 * kb + i;
          sacc[kb][i] = ((j >= lo) & (j <= hi)) ? sacc[kb][i] : -INFINITY;
        }
    }
  };

  // finish(): online softmax of the held scores, P to e4m3, O^T += V^T P^T.
  auto finish = [&](auto bufc) __attribute__((always_inline)) {
    constexpr int buf = decltype(bufc)::value;
    const char* sv = smem + (2 * buf + 1) * C::TILE;
    // Fast path without the tile max: P' = 2^(c2 S - M + 3) against the
    // current M; if a lane's sum exceeds 448 (so possibly one P' does), redo
    // the tile with M raised to the exact running max.
    float acc = 0.f;
    i32x8_t pb;
    auto exps = [&](float mu) __attribute__((always_inline)) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; i += 4) {
          const float p0 = exp2_fast(fmaf(sacc[kb][i], p.scale_log2, -mu));
          const float p1 = exp2_fast(fmaf(sacc[kb][i + 1], p.scale_log2, -mu));
          const float p2 = exp2_fast(fmaf(sacc[kb][i + 2], p.scale_log2, -mu));
          const float p3 = exp2_fast(fmaf(sacc[kb][i + 3], p.scale_log2, -mu));
          const float g = (p0 + p1) + (p2 + p3);
          acc = (kb == 0 && i == 0) ? g : acc + g;
          pb[4 * kb + (i >> 2)] = pack_fp8x4(p0, p1, p2, p3);
        }
    };
    exps(m_ref - 3.f);
    if (__builtin_amdgcn_ballot_w64(!(acc <= 448.f)) != 0) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
      const float m_new = fmaxf(m_ref, half_max(mx) * p.scale_log2);
      const float alpha = exp2_fast(m_ref - m_new);
      l_part *= alpha;
#pragma unroll
      for (int d = 0; d < C::DB; ++d) oacc[d] *= alpha;
      m_ref = m_new;
      exps(m_ref - 3.f);
    }
    l_part += acc;
#pragma unroll
    for (int d = 0; d < C::DB; ++d) {
      const char* vb = sv + voff[d];
      const i32x2_t a0 = lds_read_tr8(vb);
      const i32x2_t a1 = lds_read_tr8(vb + 8 * C::CPR * 16);
      const i32x2_t a2 = lds_read_tr8(vb + 16 * C::CPR * 16);
      const i32x2_t a3 = lds_read_tr8(vb + 24 * C::CPR * 16);
      const i32x8_t a = i32x8_t{a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
      oacc[d] = mfma_fp8(a, pb, oacc[d]);
    }
  };

  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  auto interval = [&](int t, auto cur, auto nxt) __attribute__((always_inline)) {
    if (t + 1 < t1) issue_tile(t + 1, nxt);
    // Tiles that no query row of this wave sees are skipped whole.
    if (t * C::BN < wkhi && t * C::BN + C::BN > wklo) {
      start(t, cur);
      finish(cur);
    }
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

  const int qi = wq0 + ln;
  // The lane's half, taken afresh from the hardware lane id: keeping it live
  // across the tile loop would cost a register the cap does not leave.
  const int hfe = (int)__lane_id() >> 5;
  const float l = half_sum(l_part);
  const float inv = l > 0.f ? v_descale / l : 0.f;
  if (qi < N) {
    __bf16* orow = O + (size_t)qi * p.rs_o;
#pragma unroll
    for (int d = 0; d < C::DB; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = 32 * d + 8 * g + 4 * hfe;
        *(u32x2_t*)(orow + col) =
            u32x2_t{pack_bf16x2(oacc[d][4 * g] * inv, oacc[d][4 * g + 1] * inv),
                    pack_bf16x2(oacc[d][4 * g + 2] * inv, oacc[d][4 * g + 3] * inv)};
      }
    if (hfe == 0)
      p.lse[((size_t)b * p.H + h) * N + qi] =
          l > 0.f ? (m_ref - 3.f + log2_fast(l)) * 0.69314718055994531f : -INFINITY;
  }
}

int fwd_fp8_block_rows(int headdim) { return headdim == 64 ? Fp8Shape<64>::BM : Fp8Shape<128>::BM; }

hipError_t launch_forward_fp8(FwdParams p, float v_descale, int headdim, hipStream_t stream) {
  const dim3 grid(p.B * p.H * p.nqb);
  if (headdim == 64)
    hipLaunchKernelGGL((fwd_fp8_kernel<64>), grid, dim3(Fp8Shape<64>::NW * 64), 0, stream, p, v_descale);
  else
    hipLaunchKernelGGL((fwd_fp8_kernel<128>), grid, dim3(Fp8Shape<128>::NW * 64), 0, stream, p, v_descale);
  return hipGetLastError();
}

}  // namespace fa
