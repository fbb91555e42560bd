// fa_params.h -- plain launch-parameter structs shared by the host API and
// the kernels (no device code, so host-only sources can include it).
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace fa {

// Mask description shared by all kernels. Visible(i, j) holds when
//   j < key_len(b) && (wl < 0 || j >= i - wl) && (wr < 0 || j <= i + wr);
// a causal mask is folded into wr = 0 by the host.
struct MaskParams {
  const int32_t* seqlens_k;  // [B] or null
  int wl, wr;
};

// ALiBi ([notes] docstring): the score of query i and key j gets
// -slope(b, h) * |i - j|, slope(b, h) = slopes[b * bstride + h].
struct AlibiParams {
  const float* slopes;   // null: no bias
  int bstride;           // 0 (one slope per head) or H (per batch and head)
};

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  MaskParams mask;
  AlibiParams alibi;
  int B, H, N;
  int rs_q;              // elements between sequence positions of Q, K and V
  int rs_o;              // ... of O
  int nqb;               // query blocks per (b, h)
  float scale_log2;      // softmax_scale * log2(e)
  int xcd_groups;        // >0: (b,h) count divisible by 8, remap for XCD locality
  int longest_first;     // 1: dispatch the query blocks with most keys first
};

// Blocks of rows per (batch, head) whose maxima the backward's pre-pass
// records; every backward kernel reduces them to the (b, h) maxima.
constexpr int kMaxParts = 64;

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  // Workspace, written by the pre-pass:
  float* stats;          // per row (LSE log2 e, or +inf for an empty row; D_i =
                         // sum_d dO_id O_id), [B][H][N][2] fp32
  void* q16;             // Q, K and dO in fp16, [B][N][H][D] like the inputs
  void* k16;
  void* do16;
  float* part;           // per (b, h) and block of prows rows: max |Q|, |K|, |V|, |dO|,
                         // [B * H][np][4]
  int np;                // blocks of rows per (b, h) in the pre-pass (<= kMaxParts)
  int prows;             // rows per such block
  MaskParams mask;
  AlibiParams alibi;
  int B, H, N;
  int rs_q;              // elements between sequence positions of Q, K and V
  int rs_o;              // ... of O and dO
  int rs_g;              // ... of dQ, dK and dV (the fp16 copies use H * D)
  float scale;           // softmax_scale
  float scale_log2;      // softmax_scale * log2(e)
  int xcd_groups;
};

}  // namespace fa
