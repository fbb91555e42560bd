// fa_fwd.hip -- tiled exact-attention forward for gfx950.
//
// One work-group per (batch, head, block of query rows); the work is parallel
// along the sequence as well as over batch and heads (interview guide
// "FlashAttention 深入", section "v1 → v2 → v3 演进", the v2 row). The key/value
// sequence is streamed in tiles through LDS and never leaves the chip as an
// N x N matrix (l189.com from-scratch article, §2.1/§2.4 tiling; §3.1 loop over
// key blocks inside a query block).
//
// Per tile, a wave computes S^T = K Q^T on MFMA with fp32 accumulation, so
// that each lane holds the scores of one query row for 16 keys per 32-key
// block; the row max is then an in-lane max plus one exchange between the two
// 32-lane halves. The online softmax (from-scratch article §2.2; the interview
// guide's "Online Softmax" section) keeps, per row, a reference max M (log2
// domain) and the sum l of 2^(c2 s - M); the partial output and l are rescaled
// by 2^(M_old - M_new) when M changes. Rescaling is lazy: M is only raised when
// some row's tile max exceeds it by more than 8 (log2 units), so P values stay
// <= 2^8; O and l always share the same M, so the result is unchanged up to
// rounding. O^T += V^T P^T then runs on MFMA with P packed to the input type
// (bf16 or fp16) straight from the score accumulators, in the key order the
// accumulator holds them.
//
// Epilogue: O = O_acc / l rounded to the output dtype; LSE = (M + log2 l) ln 2
// (from-scratch article §3.1 LSE statistic, §5.2 fp32 statistics).

#include <type_traits>


#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

// Tile shape per head dimension, chosen by measurement on MI355X: at D = 128
// eight waves share each K/V tile (256 query rows per work-group); at D = 64
// two independent 4-wave work-groups per CU do better (their barriers do not
// keep the two waves of a SIMD in lockstep).
template <int D>
struct FwdShape {
  static constexpr int NW = D == 128 ? 8 : 4;
  static constexpr int BN = 64;
};

template <int D, int BN_ = FwdShape<D>::BN, int NW_ = FwdShape<D>::NW, int QW_ = 32>
struct FwdCfg {
  static constexpr int NW = NW_;               // waves per work-group
  static constexpr int QW = QW_;               // query rows per wave
  static constexpr int BM = NW * QW;           // query rows per work-group
  static constexpr int BN = BN_;               // keys per tile
  static constexpr int CPR = D / 8;            // 16-byte chunks per K/V row
  static constexpr int TILE = BN * D * 2;      // bytes of one K or V tile
  static constexpr int LPW = TILE / 1024 / NW; // 1 KiB direct-to-LDS loads per wave per matrix
  static constexpr int QB = QW / 32, KB = BN / 32, DB = D / 32, KS = BN / 16, DS = D / 16;
  static constexpr int NBUF = 2;               // K/V tile buffers in LDS
  static_assert(LPW >= 1 && TILE % (1024 * NW) == 0, "tile must split into 1 KiB loads");
};

// 16-bit (bf16 or fp16) forward. One work-group = NW waves x 32 query rows
// (FwdShape). K and V tiles are copied global -> LDS by the 16-byte
// direct-to-LDS loads (no staging
// registers), double-buffered: the copy of tile t+1 is in flight while tile t
// is computed. Rows past the end of the sequence are clamped onto the last
// row (their scores are masked to -inf, so their values never contribute).
//
// Per tile and wave: S^T = K Q^T on 32x32x16 MFMA (each lane holds the scores
// of query row ln for 16 keys per 32-key block, the other 16 in the lane of
// the other 32-lane half); online
// softmax with a lazily raised reference max; O^T += V^T P^T with the V^T
// operand read by ds_read_b64_tr_b16 (lane i of a 16-lane group receives
// element (4e + i/4, i%4) of the 16 x 4 block the group addresses, so each
// lane points at 4 values of one key row and gets 4 keys of one d column).
template <int D, bool ALIBI, typename T>
__global__ void __launch_bounds__(FwdCfg<D>::NW * 64) fwd_h16_kernel(FwdParams p) {
  using C = FwdCfg<D>;
  using E = Elt16<T>;
  using vec8 = typename E::vec8;
  __shared__ __attribute__((aligned(1024))) char smem[2 * C::NBUF * C::TILE];  // [buf][K | V]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps wave logic scalar
  const int ln = lane & 31, hf = lane >> 5;
  int bh, qblk;
  map_block(p.B * p.H, p.nqb, p.xcd_groups, p.longest_first, bh, qblk);
  const int b = bh / p.H, h = bh - b * p.H;
  const int N = p.N;
  const int q0 = qblk * C::BM;
  const int kl = key_len(p.mask, b, N);
  const int rs = p.rs_q;                                // elements between sequence positions
  const size_t base = (size_t)b * N * rs + (size_t)h * D;  // element (b, 0, h, 0)
  const T* Q = (const T*)p.q + base;
  const char* Kg = (const char*)((const T*)p.k + base);
  const char* Vg = (const char*)((const T*)p.v + base);
  T* O = (T*)p.o + (size_t)b * N * p.rs_o + (size_t)h * D;
  float slope_raw = 0.f;
  if constexpr (ALIBI) slope_raw = alibi_raw_slope(p.alibi, b, h, p.scale_log2);

  const int wq0 = q0 + wave * C::QW;                    // first query row of this wave
  int klo, khi;
  key_range(p.mask, kl, q0, min(q0 + C::BM, N) - 1, klo, khi);
  const int t0 = klo / C::BN, t1 = (khi + C::BN - 1) / C::BN;
  const int wq1 = min(wq0 + C::QW - 1, N - 1);
  int wklo = 0, wkhi = 0;
  if (wq0 <= wq1) key_range(p.mask, kl, wq0, wq1, wklo, wkhi);

  // Q as the B operand of S^T = K Q^T: qf[qb][s] = Q[wq0 + 32 qb + ln][16 s + 8 hf ..+8).
  vec8 qf[C::QB][C::DS];
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    const int row = min(wq0 + 32 * qb + ln, N - 1);     // rows past N are computed, never stored
#pragma unroll
    for (int s = 0; s < C::DS; ++s) qf[qb][s] = ld_global<vec8>(Q + (size_t)row * rs + 16 * s + 8 * hf);
  }

  // Direct-to-LDS copy through buffer loads: load j of this wave fills LDS
  // chunks [(wave * LPW + j) * 64, +64) of a tile; lane -> (row, swizzled
  // chunk). The per-lane byte offset is the same for every tile; the tile's
  // first row goes in the scalar offset. Rows at or past N lie beyond the
  // buffer's last byte and read as zero (their scores are masked anyway).
  const int rs2 = rs * 2;
  const int nbytes = ((N - 1) * rs + D) * 2;
  const __amdgpu_buffer_rsrc_t krsrc = make_rsrc(Kg, nbytes);
  const __amdgpu_buffer_rsrc_t vrsrc = make_rsrc(Vg, nbytes);
  int loff[C::LPW];
#pragma unroll
  for (int j = 0; j < C::LPW; ++j) {
    const int u = (wave * C::LPW + j) * 64 + lane;
    const int row = u / C::CPR, pos = u % C::CPR;
    loff[j] = row * rs2 + (pos ^ lds_swz<D>(row)) * 16;
  }
  auto issue_tile = [&](int t, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    const int soff = t * C::BN * rs2;
    char* kd = smem + (2 * buf) * C::TILE + wave * C::LPW * 1024;
    char* vd = smem + (2 * buf + 1) * C::TILE + wave * C::LPW * 1024;
#pragma unroll
    for (int j = 0; j < C::LPW; ++j) {
      buffer_load_lds16(krsrc, kd + j * 1024, loff[j], soff);
      buffer_load_lds16(vrsrc, vd + j * 1024, loff[j], soff);
    }
  };

  // LDS read offsets (bytes within a tile): the K operand for d-step s is
  // row ln (+32 kb), chunk 2 s + hf; the V^T operand is a transposed read.
  int koff[C::DS];
#pragma unroll
  for (int s = 0; s < C::DS; ++s) koff[s] = tile_chunk_off<D>(ln, 2 * s + hf);
  int voff[C::DB][2];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int t = 0; t < 2; ++t) voff[db][t] = tile_tr_off<D>(lane, db, t);

  f32x16_t oacc[C::DB][C::QB];
#pragma unroll
  for (int d = 0; d < C::DB; ++d)
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) oacc[d][qb] = f32x16_t{};
  float m_ref[C::QB], l_part[C::QB];
#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) { m_ref[qb] = -INFINITY; l_part[qb] = 0.f; }
  bool m_finite = false;  // wave-uniform: every row of the wave has a finite M

  // S^T of the tile a wave is working on.
  f32x16_t sacc[C::KB][C::QB];

  // start(t): S^T = K(t) Q^T on MFMA, masked on tiles that cross a mask edge.
  auto start = [&](int t, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    const char* sk = smem + (2 * buf) * C::TILE;
    const int kt = t * C::BN;
    // The 32-key blocks are independent accumulation chains whose MFMAs
    // alternate. The K operands are read PF d-steps ahead of their MFMAs; the
    // scheduling barriers keep the compiler from sinking the reads back to
    // one step ahead, where eight waves contending for LDS leave the read
    // latency exposed (measured: 1.4% of the kernel at B2 H8 N4096 D128).
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int qb = 0; qb < C::QB; ++qb) sacc[kb][qb] = f32x16_t{};
    constexpr int PF = 2;
    vec8 kr[PF + 1][C::KB];
    auto kread = [&](int s, int kb) { return *(const vec8*)(sk + kb * 32 * C::CPR * 16 + koff[s]); };
#pragma unroll
    for (int s = 0; s < PF; ++s)
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb) kr[s][kb] = kread(s, kb);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < C::DS; ++s) {
      if (s + PF < C::DS) {
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb) kr[(s + PF) % (PF + 1)][kb] = kread(s + PF, kb);
      }
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int qb = 0; qb < C::QB; ++qb)
          sacc[kb][qb] = E::mfma(kr[s % (PF + 1)][kb], qf[qb][s], sacc[kb][qb]);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (ALIBI) {  // score of row i, key j: q.k - (slope / c) |i - j|
#pragma unroll
      for (int qb = 0; qb < C::QB; ++qb) {
        const float di = (float)(wq0 + 32 * qb + ln - kt - 4 * hf);
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            sacc[kb][qb][i] = fmaf(fabsf(di - (float)(32 * kb + 8 * (i >> 2) + (i & 3))), -slope_raw,
                                   sacc[kb][qb][i]);
      }
    }
    if (!block_all_visible(p.mask, kl, wq0, wq1, kt, kt + C::BN - 1)) {
#pragma unroll
      for (int qb = 0; qb < C::QB; ++qb) {
        int lo, hi;
        visible_span(p.mask, kl, wq0 + 32 * qb + ln, lo, hi);
        const int jb = kt + 4 * hf;
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int j = jb + 32 * kb + 8 * (i >> 2) + (i & 3);
            sacc[kb][qb][i] = ((j >= lo) & (j <= hi)) ? sacc[kb][qb][i] : -INFINITY;
          }
      }
    }
  };

  // finish(): online softmax of the held scores and O^T += V^T P^T with the
  // V tile of the same key tile.
  auto finish = [&](auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    const char* sv = smem + (2 * buf + 1) * C::TILE;
    // P = 2^(c2 S - M) against the current reference M. Once a row has seen
    // a visible key, M never exceeds its true running max, so its sum l >= 1
    // and nothing underflows; the only hazard is a new score far above M.
    // The fast path therefore skips the tile max and checks the tile's row
    // sums instead: if any exceeds 2^64 (or M is still -inf for some row),
    // the tile is redone on the exact path, which raises M to the running max
    // and rescales O and l. P <= 2^64 keeps O and l far inside fp32 range;
    // with fp16 operands the bound is 2^15, so every P fits fp16 (max 65504).
    constexpr float kPmax = E::is_f16 ? 32768.f : 0x1p64f;
    u32x4_t pk[C::QB][C::KS];
    float rsum[C::QB];
    auto exps = [&](const float (&m_use)[C::QB]) {
#pragma unroll
      for (int qb = 0; qb < C::QB; ++qb) {
        float acc;
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; i += 2) {
            const float p0 = exp2_fast(fmaf(sacc[kb][qb][i], p.scale_log2, -m_use[qb]));
            const float p1 = exp2_fast(fmaf(sacc[kb][qb][i + 1], p.scale_log2, -m_use[qb]));
            // fp32 sum of the unrounded P (LSE must hold to 1e-3 on short rows)
            acc = (kb == 0 && i == 0) ? p0 + p1 : acc + (p0 + p1);
            pk[qb][2 * kb + (i >> 3)][(i & 7) >> 1] = E::pack2(p0, p1);
          }
        rsum[qb] = acc;
      }
    };
    bool slow = !m_finite;
    if (!slow) {
      exps(m_ref);
      bool big = false;
#pragma unroll
      for (int qb = 0; qb < C::QB; ++qb) big |= !(rsum[qb] <= kPmax);
      slow = __builtin_amdgcn_ballot_w64(big) != 0;
    }
    if (slow) {  // wave-uniform, rare: first visible tile, or a score far above M
      bool fin = true;
      float m_use[C::QB];
#pragma unroll
      for (int qb = 0; qb < C::QB; ++qb) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][qb][i]);
        const float m_new = fmaxf(m_ref[qb], half_max(mx) * p.scale_log2);
        const float alpha = (m_new == -INFINITY) ? 1.f : exp2_fast(m_ref[qb] - m_new);
        l_part[qb] *= alpha;
#pragma unroll
        for (int d = 0; d < C::DB; ++d) oacc[d][qb] *= alpha;
        m_ref[qb] = m_new;
        fin &= m_new != -INFINITY;
        m_use[qb] = (m_new == -INFINITY) ? 0.f : m_new;
      }
      m_finite = __builtin_amdgcn_ballot_w64(!fin) == 0;
      exps(m_use);
    }
#pragma unroll
    for (int qb = 0; qb < C::QB; ++qb) l_part[qb] += rsum[qb];
    // O^T += V^T P^T: step i covers d-block i / KS and key step i % KS. The
    // V^T operands are read VPF steps ahead, pinned like the K reads above.
    constexpr int VPF = 2, NV = C::DB * C::KS;
    auto vread = [&](int i) {
      const char* vbase = sv + (i % C::KS) * 16 * C::CPR * 16;
      const u32x2_t lo = lds_read_tr16(vbase + voff[i / C::KS][0]);
      const u32x2_t hi = lds_read_tr16(vbase + voff[i / C::KS][1]);
      return u32x4_t{lo[0], lo[1], hi[0], hi[1]};
    };
    u32x4_t vr[VPF + 1];
#pragma unroll
    for (int i = 0; i < VPF; ++i) vr[i] = vread(i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      if (i + VPF < NV) vr[(i + VPF) % (VPF + 1)] = vread(i + VPF);
      const int d = i / C::KS, ks = i % C::KS;
#pragma unroll
      for (int qb = 0; qb < C::QB; ++qb)
        oacc[d][qb] = E::mfma(__builtin_bit_cast(vec8, vr[i % (VPF + 1)]),
                              __builtin_bit_cast(vec8, pk[qb][ks]), oacc[d][qb]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  // Key tiles alternate between two LDS buffers (tile t0 + i in buffer i % 2).
  // Each interval issues the copy of the next tile into the other buffer, then
  // computes the current tile; the wait and barrier at its end make the next
  // tile visible and release the buffer just read.
  auto interval = [&](int t, auto cur, auto nxt) {
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

#pragma unroll
  for (int qb = 0; qb < C::QB; ++qb) {
    const int qi = wq0 + 32 * qb + ln;
    const float l = half_sum(l_part[qb]);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    if (qi < N) {
      T* orow = O + (size_t)qi * p.rs_o;
#pragma unroll
      for (int d = 0; d < C::DB; ++d)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = 32 * d + 8 * g + 4 * hf;
          *(u32x2_t*)(orow + col) =
              u32x2_t{E::pack2(oacc[d][qb][4 * g] * inv, oacc[d][qb][4 * g + 1] * inv),
                      E::pack2(oacc[d][qb][4 * g + 2] * inv, oacc[d][qb][4 * g + 3] * inv)};
        }
      if (hf == 0)
        p.lse[((size_t)b * p.H + h) * N + qi] =
            l > 0.f ? (m_ref[qb] + log2_fast(l)) * 0.69314718055994531f : -INFINITY;
    }
  }
}

// fp32 path: the same algorithm with fp32 MFMA (32x32x2) and K, V kept in
// their natural [key][d] layout in LDS (one element per lane per MFMA, so no
// transposition is needed). Rows are padded to D + 1 floats so the 32 lanes
// that read one column hit 32 different banks.
template <int D, bool ALIBI>
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
  const size_t rs = (size_t)p.rs_q;
  const size_t base = (size_t)b * N * rs + (size_t)h * D;
  const float* Q = (const float*)p.q + base;
  const float* K = (const float*)p.k + base;
  const float* V = (const float*)p.v + base;
  float* O = (float*)p.o + (size_t)b * N * p.rs_o + (size_t)h * D;
  float slope_raw = 0.f;
  if constexpr (ALIBI) slope_raw = alibi_raw_slope(p.alibi, b, h, p.scale_log2);

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
      if constexpr (ALIBI) {
        const float di = (float)(qi - kt - 4 * hf);
#pragma unroll
        for (int i = 0; i < 16; ++i)
          sacc[i] = fmaf(fabsf(di - (float)(8 * (i >> 2) + (i & 3))), -slope_raw, sacc[i]);
      }
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
    float* orow = O + (size_t)qi * p.rs_o;
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

int fwd_block_rows(ElemType et, int headdim) {
  if (et == ElemType::kF32) return 128;
  return headdim == 64 ? FwdCfg<64>::BM : FwdCfg<128>::BM;
}

template <bool ALIBI, typename T>
static void launch_forward_h16(const FwdParams& p, int headdim, hipStream_t stream) {
  const dim3 grid(p.B * p.H * p.nqb);
  if (headdim == 64)
    hipLaunchKernelGGL((fwd_h16_kernel<64, ALIBI, T>), grid, dim3(FwdCfg<64>::NW * 64), 0, stream, p);
  else
    hipLaunchKernelGGL((fwd_h16_kernel<128, ALIBI, T>), grid, dim3(FwdCfg<128>::NW * 64), 0, stream, p);
}

template <bool ALIBI>
static void launch_forward_a(const FwdParams& p, int headdim, ElemType et, hipStream_t stream) {
  const dim3 grid(p.B * p.H * p.nqb);
  if (et == ElemType::kF32) {
    if (headdim == 64) hipLaunchKernelGGL((fwd_f32_kernel<64, ALIBI>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((fwd_f32_kernel<128, ALIBI>), grid, dim3(256), 0, stream, p);
  } else if (et == ElemType::kF16) {
    launch_forward_h16<ALIBI, _Float16>(p, headdim, stream);
  } else {
    launch_forward_h16<ALIBI, __bf16>(p, headdim, stream);
  }
}

hipError_t launch_forward(FwdParams p, int headdim, ElemType et, hipStream_t stream) {
  if (p.alibi.slopes != nullptr) launch_forward_a<true>(p, headdim, et, stream);
  else launch_forward_a<false>(p, headdim, et, stream);
  return hipGetLastError();
}

}  // namespace fa
