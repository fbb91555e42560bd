// fa_fwd.hip -- tiled exact-attention forward for gfx950.
//
// One work-group per (batch, head, block of BM query rows); each wave owns 32
// query rows, so the work is parallel along the sequence as well as over
// batch and heads (interview guide "FlashAttention 深入", section
// "v1 → v2 → v3 演进", the v2 row). The key/value sequence is streamed in tiles
// of BN keys through LDS (double-buffered) and never leaves the chip as an
// N x N matrix (l189.com from-scratch article, §2.1/§2.4 tiling; §3.1 loop
// over key blocks inside a query block).
//
// Per tile, a wave computes S^T = K Q^T on MFMA with fp32 accumulation, so
// that each lane holds the scores of ONE query row (lane % 32) for 16 keys per
// 32-key block; the row max is then an in-lane max plus one exchange between
// the two 32-lane halves. The online softmax (from-scratch article §2.2; the
// interview guide's "Online Softmax" section) keeps, per row, a reference max
// M (log2 domain) and the sum l of 2^(c2 s - M); the partial output and l are
// rescaled by 2^(M_old - M_new) when M changes. Rescaling is done lazily: M is
// only raised when some row's tile max exceeds it by more than 8 (log2 units),
// so P values stay <= 2^8; O and l always share the same M, so the result is
// unchanged up to rounding. O^T += V^T P^T then runs on MFMA with P packed to
// bf16 straight from the score accumulators; V is stored transposed in LDS,
// with the key order inside each 16-key group permuted to match the order in
// which the accumulator holds keys.
//
// Epilogue: O = O_acc / l rounded to the output dtype; LSE = (M + log2 l) ln 2
// (from-scratch article §3.1 LSE statistic, §5.2 fp32 statistics).

#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

// Position of key k inside a transposed V row: within every 16-key group,
// bits 2 and 3 of the index are swapped, so the 8 keys one lane feeds to a
// 32x32x16 MFMA (keys 8a + 4h + c of the group, a in {0,1}, c in 0..3, h the
// lane's half) sit at positions 8h + 4a + c, contiguous.
__device__ __forceinline__ int vt_pos(int k) {
  return (k & ~15) | ((k & 4) << 1) | ((k & 8) >> 1) | (k & 3);
}

template <int D, int NW, int BN>
struct FwdBf16Cfg {
  static constexpr int NT = NW * 64;
  static constexpr int BM = NW * 32;
  static constexpr int KSTR = D + 8;   // K row stride in LDS (elements); +16 B spreads rows over banks
  static constexpr int VSTR = BN + 8;  // transposed-V row stride (elements)
  static constexpr int KTILE = BN * KSTR;
  static constexpr int VTILE = D * VSTR;
  static constexpr int KCH = BN * D / 8 / NT;  // 16-byte K chunks per thread per tile
  static constexpr int KPT = BN * D / 8 / NT;  // keys per thread when staging V
  static constexpr int KGROUPS = BN / KPT;
  static_assert(BN % 32 == 0 && D % 32 == 0, "tile shape");
  static_assert(KPT == 2 || KPT == 4, "V staging handles 2 or 4 keys per thread");
};

template <int D, int NW, int BN>
__global__ void __launch_bounds__(NW * 64) fwd_bf16_kernel(FwdParams p) {
  using C = FwdBf16Cfg<D, NW, BN>;
  __shared__ __attribute__((aligned(16))) __bf16 sK[2][C::KTILE];
  __shared__ __attribute__((aligned(16))) __bf16 sV[2][C::VTILE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 31, hf = lane >> 5;
  int bh, qb;
  map_block(p.B * p.H, p.nqb, p.xcd_groups, p.longest_first, bh, qb);
  const int b = bh / p.H, h = bh - b * p.H;
  const int N = p.N;
  const int q0 = qb * C::BM;
  const int kl = key_len(p.mask, b, N);
  const size_t rs = (size_t)p.H * D;                    // elements between sequence positions
  const size_t base = ((size_t)b * N * p.H + h) * D;    // element (b, 0, h, 0)
  const __bf16* Q = (const __bf16*)p.q + base;
  const __bf16* K = (const __bf16*)p.k + base;
  const __bf16* V = (const __bf16*)p.v + base;
  __bf16* O = (__bf16*)p.o + base;

  const int qi = q0 + wave * 32 + ln;                   // this lane's query row
  int klo, khi;
  key_range(p.mask, kl, q0, min(q0 + C::BM, N) - 1, klo, khi);
  const int t0 = klo / BN, t1 = (khi + BN - 1) / BN;
  const int wq0 = q0 + wave * 32, wq1 = min(wq0 + 31, N - 1);
  int wklo = 0, wkhi = 0;
  if (wq0 <= wq1) key_range(p.mask, kl, wq0, wq1, wklo, wkhi);

  // Q as the B operand of S^T = K Q^T: lane holds Q[qi][16s + 8hf .. +8).
  bf16x8_t qf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    if (qi < N) qf[s] = ld_global<bf16x8_t>(Q + (size_t)qi * rs + 16 * s + 8 * hf);
    else qf[s] = bf16x8_t{};
  }

  f32x16_t oacc[D / 32];
#pragma unroll
  for (int d = 0; d < D / 32; ++d) oacc[d] = f32x16_t{};
  float m_ref = -INFINITY;  // reference max, log2 domain
  float l_part = 0.f;       // this lane's half of the row sum

  u32x4_t kreg[C::KCH];
  u32x4_t vreg[C::KPT];
  const int vkg = tid % C::KGROUPS, vdc = tid / C::KGROUPS;

  auto load_tile = [&](int t) {
    const int kt = t * BN;
#pragma unroll
    for (int r = 0; r < C::KCH; ++r) {
      const int c = tid + C::NT * r, row = c / (D / 8), col = (c % (D / 8)) * 8;
      const int key = kt + row;
      kreg[r] = key < N ? ld_global<u32x4_t>(K + (size_t)key * rs + col) : u32x4_t{};
    }
#pragma unroll
    for (int r = 0; r < C::KPT; ++r) {
      const int key = kt + vkg * C::KPT + r;
      vreg[r] = key < N ? ld_global<u32x4_t>(V + (size_t)key * rs + vdc * 8) : u32x4_t{};
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int r = 0; r < C::KCH; ++r) {
      const int c = tid + C::NT * r, row = c / (D / 8), col = (c % (D / 8)) * 8;
      *(u32x4_t*)&sK[buf][row * C::KSTR + col] = kreg[r];
    }
    const int kpos = vt_pos(vkg * C::KPT);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      __bf16* lo = &sV[buf][(vdc * 8 + 2 * e) * C::VSTR + kpos];
      __bf16* hi = lo + C::VSTR;
      if constexpr (C::KPT == 4) {
        *(u32x2_t*)lo = u32x2_t{(vreg[0][e] & 0xffffu) | (vreg[1][e] << 16),
                                (vreg[2][e] & 0xffffu) | (vreg[3][e] << 16)};
        *(u32x2_t*)hi = u32x2_t{(vreg[0][e] >> 16) | (vreg[1][e] & 0xffff0000u),
                                (vreg[2][e] >> 16) | (vreg[3][e] & 0xffff0000u)};
      } else {
        *(uint32_t*)lo = (vreg[0][e] & 0xffffu) | (vreg[1][e] << 16);
        *(uint32_t*)hi = (vreg[0][e] >> 16) | (vreg[1][e] & 0xffff0000u);
      }
    }
  };

  if (t0 < t1) {
    load_tile(t0);
    store_tile(0);
  }
  __syncthreads();

  for (int t = t0; t < t1; ++t) {
    const int buf = (t - t0) & 1;
    const bool more = t + 1 < t1;
    if (more) load_tile(t + 1);
    const int kt = t * BN;
    if (kt < wkhi && kt + BN > wklo) {
      // S^T = K Q^T. sacc[kb][i] is the score of query qi and key
      // kt + 32 kb + 8 (i / 4) + 4 hf + i % 4.
      f32x16_t sacc[BN / 32];
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb) {
        sacc[kb] = f32x16_t{};
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
          const bf16x8_t a = *(const bf16x8_t*)&sK[buf][(32 * kb + ln) * C::KSTR + 16 * s + 8 * hf];
          sacc[kb] = mfma_bf16(a, qf[s], sacc[kb]);
        }
      }
      if (!block_all_visible(p.mask, kl, wq0, wq1, kt, kt + BN - 1)) {
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int j = kt + 32 * kb + 8 * (i >> 2) + 4 * hf + (i & 3);
            if (!visible(p.mask, kl, qi, j)) sacc[kb][i] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
      const float mt = half_max(mx) * p.scale_log2;
      if (__ballot(mt > m_ref + 8.f)) {  // wave-uniform
        const float m_new = fmaxf(m_ref, mt);
        const float alpha = (m_new == -INFINITY) ? 1.f : exp2_fast(m_ref - m_new);
        l_part *= alpha;
#pragma unroll
        for (int d = 0; d < D / 32; ++d) oacc[d] *= alpha;
        m_ref = m_new;
      }
      const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
      u32x4_t pk[BN / 16];  // P in bf16, 8 keys per 16-byte operand
      float rsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          const float p0 = exp2_fast(fmaf(sacc[kb][i], p.scale_log2, -m_use));
          const float p1 = exp2_fast(fmaf(sacc[kb][i + 1], p.scale_log2, -m_use));
          rsum += p0 + p1;
          pk[2 * kb + (i >> 3)][(i & 7) >> 1] = pack_bf16x2(p0, p1);
        }
      l_part += rsum;
      // O^T += V^T P^T: A = transposed V rows (d), B = P from the accumulators.
#pragma unroll
      for (int d = 0; d < D / 32; ++d)
#pragma unroll
        for (int ks = 0; ks < BN / 16; ++ks) {
          const bf16x8_t a = *(const bf16x8_t*)&sV[buf][(32 * d + ln) * C::VSTR + 16 * ks + 8 * hf];
          oacc[d] = mfma_bf16(a, __builtin_bit_cast(bf16x8_t, pk[ks]), oacc[d]);
        }
    }
    if (more) store_tile(buf ^ 1);
    __syncthreads();
  }

  const float l = half_sum(l_part);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (qi < N) {
    __bf16* orow = O + (size_t)qi * rs;
#pragma unroll
    for (int d = 0; d < D / 32; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = 32 * d + 8 * g + 4 * hf;
        *(u32x2_t*)(orow + col) =
            u32x2_t{pack_bf16x2(oacc[d][4 * g] * inv, oacc[d][4 * g + 1] * inv),
                    pack_bf16x2(oacc[d][4 * g + 2] * inv, oacc[d][4 * g + 3] * inv)};
      }
    if (hf == 0)
      p.lse[((size_t)b * p.H + h) * N + qi] =
          l > 0.f ? (m_ref + log2_fast(l)) * 0.69314718055994531f : -INFINITY;
  }
}

// fp32 path: the same algorithm with fp32 MFMA (32x32x2) and K, V kept in
// their natural [key][d] layout in LDS (one element per lane per MFMA, so no
// transposition is needed). Rows are padded to D + 1 floats so the 32 lanes
// that read one column hit 32 different banks.
template <int D>
__global__ void __launch_bounds__(256) fwd_f32_kernel(FwdParams p) {
  constexpr int NW = 4, NT = 256, BM = 128, BN = 32, STR = D + 1;
  constexpr int CH = BN * D / 4 / NT;  // float4 chunks per thread per tile
  __shared__ float sK[2][BN * STR];
  __shared__ float sV[2][BN * STR];
  (void)NW;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 31, hf = lane >> 5;
  int bh, qb;
  map_block(p.B * p.H, p.nqb, p.xcd_groups, p.longest_first, bh, qb);
  const int b = bh / p.H, h = bh - b * p.H;
  const int N = p.N;
  const int q0 = qb * BM;
  const int kl = key_len(p.mask, b, N);
  const size_t rs = (size_t)p.H * D;
  const size_t base = ((size_t)b * N * p.H + h) * D;
  const float* Q = (const float*)p.q + base;
  const float* K = (const float*)p.k + base;
  const float* V = (const float*)p.v + base;
  float* O = (float*)p.o + base;

  const int qi = q0 + wave * 32 + ln;
  int klo, khi;
  key_range(p.mask, kl, q0, min(q0 + BM, N) - 1, klo, khi);
  const int t0 = klo / BN, t1 = (khi + BN - 1) / BN;
  const int wq0 = q0 + wave * 32, wq1 = min(wq0 + 31, N - 1);
  int wklo = 0, wkhi = 0;
  if (wq0 <= wq1) key_range(p.mask, kl, wq0, wq1, wklo, wkhi);

  float qf[D / 2];
#pragma unroll
  for (int s = 0; s < D / 2; ++s) qf[s] = qi < N ? Q[(size_t)qi * rs + 2 * s + hf] : 0.f;

  f32x16_t oacc[D / 32];
#pragma unroll
  for (int d = 0; d < D / 32; ++d) oacc[d] = f32x16_t{};
  float m_ref = -INFINITY, l_part = 0.f;
  f32x4_t kreg[CH], vreg[CH];

  auto load_tile = [&](int t) {
    const int kt = t * BN;
#pragma unroll
    for (int r = 0; r < CH; ++r) {
      const int c = tid + NT * r, row = c / (D / 4), col = (c % (D / 4)) * 4;
      const int key = kt + row;
      kreg[r] = key < N ? ld_global<f32x4_t>(K + (size_t)key * rs + col) : f32x4_t{};
      vreg[r] = key < N ? ld_global<f32x4_t>(V + (size_t)key * rs + col) : f32x4_t{};
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int r = 0; r < CH; ++r) {
      const int c = tid + NT * r, row = c / (D / 4), col = (c % (D / 4)) * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sK[buf][row * STR + col + e] = kreg[r][e];
        sV[buf][row * STR + col + e] = vreg[r][e];
      }
    }
  };

  if (t0 < t1) {
    load_tile(t0);
    store_tile(0);
  }
  __syncthreads();

  for (int t = t0; t < t1; ++t) {
    const int buf = (t - t0) & 1;
    const bool more = t + 1 < t1;
    if (more) load_tile(t + 1);
    const int kt = t * BN;
    if (kt < wkhi && kt + BN > wklo) {
      f32x16_t sacc = f32x16_t{};
#pragma unroll
      for (int s = 0; s < D / 2; ++s) sacc = mfma_f32(sK[buf][ln * STR + 2 * s + hf], qf[s], sacc);
      if (!block_all_visible(p.mask, kl, wq0, wq1, kt, kt + BN - 1)) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (!visible(p.mask, kl, qi, kt + 8 * (i >> 2) + 4 * hf + (i & 3))) sacc[i] = -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[i]);
      const float mt = half_max(mx) * p.scale_log2;
      if (__ballot(mt > m_ref + 8.f)) {
        const float m_new = fmaxf(m_ref, mt);
        const float alpha = (m_new == -INFINITY) ? 1.f : exp2_fast(m_ref - m_new);
        l_part *= alpha;
#pragma unroll
        for (int d = 0; d < D / 32; ++d) oacc[d] *= alpha;
        m_ref = m_new;
      }
      const float m_use = (m_ref == -INFINITY) ? 0.f : m_ref;
      float pv[16];
      float rsum = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        pv[i] = exp2_fast(fmaf(sacc[i], p.scale_log2, -m_use));
        rsum += pv[i];
      }
      l_part += rsum;
#pragma unroll
      for (int d = 0; d < D / 32; ++d)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = 8 * (i >> 2) + 4 * hf + (i & 3);
          oacc[d] = mfma_f32(sV[buf][key * STR + 32 * d + ln], pv[i], oacc[d]);
        }
    }
    if (more) store_tile(buf ^ 1);
    __syncthreads();
  }

  const float l = half_sum(l_part);
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (qi < N) {
    float* orow = O + (size_t)qi * rs;
#pragma unroll
    for (int d = 0; d < D / 32; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = 32 * d + 8 * g + 4 * hf;
        *(f32x4_t*)(orow + col) = f32x4_t{oacc[d][4 * g] * inv, oacc[d][4 * g + 1] * inv,
                                          oacc[d][4 * g + 2] * inv, oacc[d][4 * g + 3] * inv};
      }
    if (hf == 0)
      p.lse[((size_t)b * p.H + h) * N + qi] =
          l > 0.f ? (m_ref + log2_fast(l)) * 0.69314718055994531f : -INFINITY;
  }
}

// ---------------------------------------------------------------- launchers

static constexpr int kFwdWaves = 4;
static constexpr int kFwdBN = 64;

int fwd_block_rows(int dtype_is_f32) { return dtype_is_f32 ? 128 : kFwdWaves * 32; }

hipError_t launch_forward(FwdParams p, int headdim, int dtype_is_f32, hipStream_t stream) {
  const dim3 grid(p.B * p.H * p.nqb);
  if (dtype_is_f32) {
    if (headdim == 64) hipLaunchKernelGGL(fwd_f32_kernel<64>, grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL(fwd_f32_kernel<128>, grid, dim3(256), 0, stream, p);
  } else {
    constexpr int NT = kFwdWaves * 64;
    if (headdim == 64)
      hipLaunchKernelGGL((fwd_bf16_kernel<64, kFwdWaves, kFwdBN>), grid, dim3(NT), 0, stream, p);
    else
      hipLaunchKernelGGL((fwd_bf16_kernel<128, kFwdWaves, kFwdBN>), grid, dim3(NT), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace fa
