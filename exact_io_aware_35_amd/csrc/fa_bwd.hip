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
//   bwd_drow_kernel : D_i from O and dO (bandwidth-bound).
//   bwd_dkdv_kernel : one work-group per key block; each wave keeps dK and dV
//                     of 32 keys in registers and loops over query tiles.
//   bwd_dq_kernel   : one work-group per query block; each wave keeps dQ of
//                     32 queries in registers and loops over key tiles.
// Products whose operand is P or dS run on fp16 MFMA (P and dS in fp16 carry
// 3 more mantissa bits than bf16; bf16 inputs convert to fp16 exactly in the
// normal range); S and dP use bf16 MFMA on the bf16 inputs directly.

#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

// Same permutation as the forward's transposed V: inside each 16-row group,
// bits 2 and 3 of the row index swap, so the 8 rows one lane feeds to a
// 32x32x16 MFMA from an accumulator are contiguous.
__device__ __forceinline__ int tr_pos(int k) {
  return (k & ~15) | ((k & 4) << 1) | ((k & 8) >> 1) | (k & 3);
}

// bf16 pair (one u32) -> two fp16 in one u32.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t u) {
  return pack_f16x2(bf16_lo(u), bf16_hi(u));
}

// Write `rows` (2 or 4) staged 16-byte chunks (8 bf16 of one row each, rows
// r0..r0+rows-1, columns 8 dc .. 8 dc + 7) transposed into an fp16 LDS tile
// T[col][tr_pos(row)] with row stride TSTR.
template <int ROWS, int TSTR>
__device__ __forceinline__ void store_transposed_f16(_Float16* T, const u32x4_t* reg, int r0,
                                                     int dc) {
  const int pos = tr_pos(r0);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    _Float16* lo = T + (8 * dc + 2 * e) * TSTR + pos;
    _Float16* hi = lo + TSTR;
    if constexpr (ROWS == 4) {
      *(u32x2_t*)lo = u32x2_t{pack_f16x2(bf16_lo(reg[0][e]), bf16_lo(reg[1][e])),
                              pack_f16x2(bf16_lo(reg[2][e]), bf16_lo(reg[3][e]))};
      *(u32x2_t*)hi = u32x2_t{pack_f16x2(bf16_hi(reg[0][e]), bf16_hi(reg[1][e])),
                              pack_f16x2(bf16_hi(reg[2][e]), bf16_hi(reg[3][e]))};
    } else {
      *(uint32_t*)lo = pack_f16x2(bf16_lo(reg[0][e]), bf16_lo(reg[1][e]));
      *(uint32_t*)hi = pack_f16x2(bf16_hi(reg[0][e]), bf16_hi(reg[1][e]));
    }
  }
}

// ---------------------------------------------------------------- D_i

template <int D>
__global__ void __launch_bounds__(256) bwd_drow_kernel(BwdParams p) {
  constexpr int LPR = D / 8;               // lanes per row, 16 bytes each
  constexpr int RPB = 256 / LPR;           // rows per block
  const int tid = threadIdx.x;
  const long long r = (long long)blockIdx.x * RPB + tid / LPR;  // flattened (b, i, h)
  const int c = tid % LPR;
  const long long R = (long long)p.B * p.N * p.H;
  float acc = 0.f;
  if (r < R) {
    const u32x4_t o = ld_global<u32x4_t>((const __bf16*)p.o + r * D + 8 * c);
    const u32x4_t g = ld_global<u32x4_t>((const __bf16*)p.dout + r * D + 8 * c);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      acc += bf16_lo(o[e]) * bf16_lo(g[e]) + bf16_hi(o[e]) * bf16_hi(g[e]);
  }
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
  if (r < R && c == 0) {
    const int h = (int)(r % p.H);
    const long long bi = r / p.H;
    const int i = (int)(bi % p.N), b = (int)(bi / p.N);
    p.drow[((size_t)b * p.H + h) * p.N + i] = acc;
  }
}

// ---------------------------------------------------------------- dK, dV

template <int D, int NW, int BMQ>
__global__ void __launch_bounds__(NW * 64) bwd_dkdv_kernel(BwdParams p) {
  constexpr int NT = NW * 64, BNK = NW * 32;
  constexpr int NSTR = D + 8;             // natural [row][d] bf16 tiles
  constexpr int TSTR = BMQ + 8;           // transposed [d][row] fp16 tiles
  constexpr int QPT = BMQ * D / 8 / NT;   // query rows per thread when staging
  constexpr int QG = BMQ / QPT;
  static_assert(QPT == 2 || QPT == 4, "staging handles 2 or 4 rows per thread");
  __shared__ __attribute__((aligned(16))) __bf16 sQ[BMQ * NSTR];
  __shared__ __attribute__((aligned(16))) __bf16 sdO[BMQ * NSTR];
  __shared__ __attribute__((aligned(16))) _Float16 sQt[D * TSTR];
  __shared__ __attribute__((aligned(16))) _Float16 sdOt[D * TSTR];
  __shared__ __attribute__((aligned(16))) float sL[BMQ];   // LSE * log2(e), +inf for no row
  __shared__ __attribute__((aligned(16))) float sDr[BMQ];  // D_i

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 31, hf = lane >> 5;
  int bh, kblk;
  map_block(p.B * p.H, p.nblk, p.xcd_groups, 0, bh, kblk);
  const int b = bh / p.H, h = bh - b * p.H;
  const int N = p.N;
  const int kl = key_len(p.mask, b, N);
  const size_t rs = (size_t)p.H * D;
  const size_t base = ((size_t)b * N * p.H + h) * D;
  const __bf16* Q = (const __bf16*)p.q + base;
  const __bf16* K = (const __bf16*)p.k + base;
  const __bf16* V = (const __bf16*)p.v + base;
  const __bf16* dO = (const __bf16*)p.dout + base;
  const float* LSE = p.lse + ((size_t)b * p.H + h) * N;
  const float* DR = p.drow + ((size_t)b * p.H + h) * N;

  const int k0 = kblk * BNK;
  const int key = k0 + wave * 32 + ln;  // this lane's key
  bf16x8_t kf[D / 16], vf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    if (key < N) {
      kf[s] = ld_global<bf16x8_t>(K + (size_t)key * rs + 16 * s + 8 * hf);
      vf[s] = ld_global<bf16x8_t>(V + (size_t)key * rs + 16 * s + 8 * hf);
    } else {
      kf[s] = bf16x8_t{};
      vf[s] = bf16x8_t{};
    }
  }
  f32x16_t dk[D / 32], dv[D / 32];
#pragma unroll
  for (int d = 0; d < D / 32; ++d) { dk[d] = f32x16_t{}; dv[d] = f32x16_t{}; }

  // Queries that see at least one key of this block (keys >= kl see none).
  const int klast = min(k0 + BNK, kl) - 1;
  int qlo = 0, qhi = 0;
  if (k0 <= klast) {
    qlo = p.mask.wr >= 0 ? max(0, k0 - p.mask.wr) : 0;
    qhi = p.mask.wl >= 0 ? min(N, klast + p.mask.wl + 1) : N;
  }
  const int t0 = qlo / BMQ, t1 = qhi > qlo ? (qhi + BMQ - 1) / BMQ : t0;
  const int wk0 = k0 + wave * 32, wk1 = wk0 + 31;
  const int wklast = min(wk1, kl - 1);
  int wqlo = 0, wqhi = 0;
  if (wk0 <= wklast) {
    wqlo = p.mask.wr >= 0 ? max(0, wk0 - p.mask.wr) : 0;
    wqhi = p.mask.wl >= 0 ? min(N, wklast + p.mask.wl + 1) : N;
  }

  u32x4_t qreg[QPT], oreg[QPT];
  float lreg = INFINITY, dreg = 0.f;
  const int sg = tid % QG, sdc = tid / QG;
  auto load_tile = [&](int t) {
    const int qb = t * BMQ;
#pragma unroll
    for (int r = 0; r < QPT; ++r) {
      const int row = qb + sg * QPT + r;
      qreg[r] = row < N ? ld_global<u32x4_t>(Q + (size_t)row * rs + 8 * sdc) : u32x4_t{};
      oreg[r] = row < N ? ld_global<u32x4_t>(dO + (size_t)row * rs + 8 * sdc) : u32x4_t{};
    }
    if (tid < BMQ) {
      const int row = qb + tid;
      const float L = row < N ? LSE[row] : -INFINITY;
      lreg = L == -INFINITY ? INFINITY : L * 1.4426950408889634f;
      dreg = row < N ? DR[row] : 0.f;
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int r = 0; r < QPT; ++r) {
      *(u32x4_t*)&sQ[(sg * QPT + r) * NSTR + 8 * sdc] = qreg[r];
      *(u32x4_t*)&sdO[(sg * QPT + r) * NSTR + 8 * sdc] = oreg[r];
    }
    store_transposed_f16<QPT, TSTR>(sQt, qreg, sg * QPT, sdc);
    store_transposed_f16<QPT, TSTR>(sdOt, oreg, sg * QPT, sdc);
    if (tid < BMQ) {
      sL[tid] = lreg;
      sDr[tid] = dreg;
    }
  };

  if (t0 < t1) load_tile(t0);
  for (int t = t0; t < t1; ++t) {
    __syncthreads();  // the previous tile's readers are done
    store_tile();
    __syncthreads();
    if (t + 1 < t1) load_tile(t + 1);
    const int qb = t * BMQ;
    if (qb < wqhi && qb + BMQ > wqlo) {
      const bool full = block_all_visible(p.mask, kl, qb, min(qb + BMQ, N) - 1, wk0, wk1);
      u32x4_t ppk[BMQ / 16], dpk[BMQ / 16];  // fp16 P and dS, 8 queries per operand
#pragma unroll
      for (int qs = 0; qs < BMQ / 32; ++qs) {
        // S = Q K^T and dP = dO V^T for 32 queries x this lane's key.
        f32x16_t sa = f32x16_t{}, pa = f32x16_t{};
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
          const int off = (32 * qs + ln) * NSTR + 16 * s + 8 * hf;
          sa = mfma_bf16(*(const bf16x8_t*)&sQ[off], kf[s], sa);
          pa = mfma_bf16(*(const bf16x8_t*)&sdO[off], vf[s], pa);
        }
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          float pv[2], dsv[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int ql = 32 * qs + 8 * ((i + u) >> 2) + 4 * hf + ((i + u) & 3);
            float pp = exp2_fast(fmaf(sa[i + u], p.scale_log2, -sL[ql]));
            if (!full && !visible(p.mask, kl, qb + ql, key)) pp = 0.f;
            pv[u] = pp;
            dsv[u] = pp * (pa[i + u] - sDr[ql]);
          }
          ppk[2 * qs + (i >> 3)][(i & 7) >> 1] = pack_f16x2(pv[0], pv[1]);
          dpk[2 * qs + (i >> 3)][(i & 7) >> 1] = pack_f16x2(dsv[0], dsv[1]);
        }
      }
      // dV^T += dO^T P and dK^T += Q^T dS (fp16 operands, fp32 accumulation).
#pragma unroll
      for (int d = 0; d < D / 32; ++d)
#pragma unroll
        for (int ks = 0; ks < BMQ / 16; ++ks) {
          const int off = (32 * d + ln) * TSTR + 16 * ks + 8 * hf;
          dv[d] = mfma_f16(*(const f16x8_t*)&sdOt[off], __builtin_bit_cast(f16x8_t, ppk[ks]), dv[d]);
          dk[d] = mfma_f16(*(const f16x8_t*)&sQt[off], __builtin_bit_cast(f16x8_t, dpk[ks]), dk[d]);
        }
    }
  }

  if (key < N) {
    __bf16* dkrow = (__bf16*)p.dk + base + (size_t)key * rs;
    __bf16* dvrow = (__bf16*)p.dv + base + (size_t)key * rs;
#pragma unroll
    for (int d = 0; d < D / 32; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = 32 * d + 8 * g + 4 * hf;
        *(u32x2_t*)(dkrow + col) =
            u32x2_t{pack_bf16x2(dk[d][4 * g] * p.scale, dk[d][4 * g + 1] * p.scale),
                    pack_bf16x2(dk[d][4 * g + 2] * p.scale, dk[d][4 * g + 3] * p.scale)};
        *(u32x2_t*)(dvrow + col) = u32x2_t{pack_bf16x2(dv[d][4 * g], dv[d][4 * g + 1]),
                                           pack_bf16x2(dv[d][4 * g + 2], dv[d][4 * g + 3])};
      }
  }
}

// ---------------------------------------------------------------- dQ

template <int D, int NW, int BN>
__global__ void __launch_bounds__(NW * 64) bwd_dq_kernel(BwdParams p) {
  constexpr int NT = NW * 64, BM = NW * 32;
  constexpr int NSTR = D + 8;
  constexpr int TSTR = BN + 8;
  constexpr int KPT = BN * D / 8 / NT;
  constexpr int KG = BN / KPT;
  static_assert(KPT == 2 || KPT == 4, "staging handles 2 or 4 rows per thread");
  __shared__ __attribute__((aligned(16))) __bf16 sK[BN * NSTR];
  __shared__ __attribute__((aligned(16))) __bf16 sV[BN * NSTR];
  __shared__ __attribute__((aligned(16))) _Float16 sKt[D * TSTR];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ln = lane & 31, hf = lane >> 5;
  int bh, qblk;
  map_block(p.B * p.H, p.nblk, p.xcd_groups, p.mask.wr >= 0, bh, qblk);
  const int b = bh / p.H, h = bh - b * p.H;
  const int N = p.N;
  const int kl = key_len(p.mask, b, N);
  const size_t rs = (size_t)p.H * D;
  const size_t base = ((size_t)b * N * p.H + h) * D;
  const __bf16* Q = (const __bf16*)p.q + base;
  const __bf16* K = (const __bf16*)p.k + base;
  const __bf16* V = (const __bf16*)p.v + base;
  const __bf16* dO = (const __bf16*)p.dout + base;

  const int q0 = qblk * BM;
  const int qi = q0 + wave * 32 + ln;
  bf16x8_t qf[D / 16], of[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    if (qi < N) {
      qf[s] = ld_global<bf16x8_t>(Q + (size_t)qi * rs + 16 * s + 8 * hf);
      of[s] = ld_global<bf16x8_t>(dO + (size_t)qi * rs + 16 * s + 8 * hf);
    } else {
      qf[s] = bf16x8_t{};
      of[s] = bf16x8_t{};
    }
  }
  float lse2 = INFINITY, dr = 0.f;
  if (qi < N) {
    const float L = p.lse[((size_t)b * p.H + h) * N + qi];
    lse2 = L == -INFINITY ? INFINITY : L * 1.4426950408889634f;
    dr = p.drow[((size_t)b * p.H + h) * N + qi];
  }
  f32x16_t dq[D / 32];
#pragma unroll
  for (int d = 0; d < D / 32; ++d) dq[d] = f32x16_t{};

  int klo, khi;
  key_range(p.mask, kl, q0, min(q0 + BM, N) - 1, klo, khi);
  const int t0 = klo / BN, t1 = (khi + BN - 1) / BN;
  const int wq0 = q0 + wave * 32, wq1 = min(wq0 + 31, N - 1);
  int wklo = 0, wkhi = 0;
  if (wq0 <= wq1) key_range(p.mask, kl, wq0, wq1, wklo, wkhi);

  u32x4_t kreg[KPT], vreg[KPT];
  const int sg = tid % KG, sdc = tid / KG;
  auto load_tile = [&](int t) {
    const int kt = t * BN;
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
      const int row = kt + sg * KPT + r;
      kreg[r] = row < N ? ld_global<u32x4_t>(K + (size_t)row * rs + 8 * sdc) : u32x4_t{};
      vreg[r] = row < N ? ld_global<u32x4_t>(V + (size_t)row * rs + 8 * sdc) : u32x4_t{};
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int r = 0; r < KPT; ++r) {
      *(u32x4_t*)&sK[(sg * KPT + r) * NSTR + 8 * sdc] = kreg[r];
      *(u32x4_t*)&sV[(sg * KPT + r) * NSTR + 8 * sdc] = vreg[r];
    }
    store_transposed_f16<KPT, TSTR>(sKt, kreg, sg * KPT, sdc);
  };

  if (t0 < t1) load_tile(t0);
  for (int t = t0; t < t1; ++t) {
    __syncthreads();
    store_tile();
    __syncthreads();
    if (t + 1 < t1) load_tile(t + 1);
    const int kt = t * BN;
    if (kt < wkhi && kt + BN > wklo) {
      const bool full = block_all_visible(p.mask, kl, wq0, wq1, kt, kt + BN - 1);
      u32x4_t dsk[BN / 16];
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb) {
        // S^T = K Q^T and dP^T = V dO^T: 32 keys x this lane's query.
        f32x16_t sa = f32x16_t{}, pa = f32x16_t{};
#pragma unroll
        for (int s = 0; s < D / 16; ++s) {
          const int off = (32 * kb + ln) * NSTR + 16 * s + 8 * hf;
          sa = mfma_bf16(*(const bf16x8_t*)&sK[off], qf[s], sa);
          pa = mfma_bf16(*(const bf16x8_t*)&sV[off], of[s], pa);
        }
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          float dsv[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int j = kt + 32 * kb + 8 * ((i + u) >> 2) + 4 * hf + ((i + u) & 3);
            float pp = exp2_fast(fmaf(sa[i + u], p.scale_log2, -lse2));
            if (!full && !visible(p.mask, kl, qi, j)) pp = 0.f;
            dsv[u] = pp * (pa[i + u] - dr);
          }
          dsk[2 * kb + (i >> 3)][(i & 7) >> 1] = pack_f16x2(dsv[0], dsv[1]);
        }
      }
      // dQ^T += K^T dS^T.
#pragma unroll
      for (int d = 0; d < D / 32; ++d)
#pragma unroll
        for (int ks = 0; ks < BN / 16; ++ks) {
          const int off = (32 * d + ln) * TSTR + 16 * ks + 8 * hf;
          dq[d] = mfma_f16(*(const f16x8_t*)&sKt[off], __builtin_bit_cast(f16x8_t, dsk[ks]), dq[d]);
        }
    }
  }

  if (qi < N) {
    __bf16* row = (__bf16*)p.dq + base + (size_t)qi * rs;
#pragma unroll
    for (int d = 0; d < D / 32; ++d)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = 32 * d + 8 * g + 4 * hf;
        *(u32x2_t*)(row + col) =
            u32x2_t{pack_bf16x2(dq[d][4 * g] * p.scale, dq[d][4 * g + 1] * p.scale),
                    pack_bf16x2(dq[d][4 * g + 2] * p.scale, dq[d][4 * g + 3] * p.scale)};
      }
  }
}

// ---------------------------------------------------------------- launcher

static constexpr int kBwdWaves = 4;
static constexpr int kBwdTile = 64;

template <int D>
static hipError_t launch_backward_d(BwdParams p, hipStream_t stream) {
  constexpr int NT = kBwdWaves * 64, BLK = kBwdWaves * 32;
  const long long rows = (long long)p.B * p.N * p.H;
  const long long rpb = 256 / (D / 8);
  hipLaunchKernelGGL(bwd_drow_kernel<D>, dim3((unsigned)((rows + rpb - 1) / rpb)), dim3(256), 0,
                     stream, p);
  p.nblk = (p.N + BLK - 1) / BLK;
  const dim3 grid(p.B * p.H * p.nblk);
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, kBwdWaves, kBwdTile>), grid, dim3(NT), 0, stream, p);
  hipLaunchKernelGGL((bwd_dq_kernel<D, kBwdWaves, kBwdTile>), grid, dim3(NT), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_backward(BwdParams p, int headdim, int dtype_is_f32, hipStream_t stream) {
  if (dtype_is_f32) return hipErrorNotSupported;
  return headdim == 64 ? launch_backward_d<64>(p, stream) : launch_backward_d<128>(p, stream);
}

}  // namespace fa
