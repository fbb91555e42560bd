// fa_api.cpp -- the C ABI declared in include/fa.h: argument checks, mask
// folding and dispatch to the gfx950 kernels. No allocation, no device
// synchronisation: every call only enqueues work on the caller's stream.

#include "fa.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "fa_launch.h"

namespace {

thread_local char g_msg[256] = "";

fa_status_t fail(fa_status_t s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof g_msg, fmt, ap);
  va_end(ap);
  return s;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shared size/mask/scale checks. On success fills the folded window bounds.
fa_status_t check_common(int batch, int heads, int seqlen, int headdim, float scale,
                         int causal, int wl, int wr, fa_dtype_t dtype, int* wl_eff,
                         int* wr_eff) {
  if (batch < 1 || heads < 1 || seqlen < 1)
    return fail(FA_ERR_INVALID_ARG, "batch, heads and seqlen must be >= 1 (got %d, %d, %d)",
                batch, heads, seqlen);
  if (seqlen > (1 << 24))
    return fail(FA_ERR_INVALID_ARG, "seqlen %d exceeds 2^24", seqlen);
  if ((long long)batch * heads * seqlen >= (1LL << 31))
    return fail(FA_ERR_INVALID_ARG, "batch*heads*seqlen must be < 2^31");
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F32)
    return fail(FA_ERR_UNSUPPORTED, "dtype %d is not supported", (int)dtype);
  if (headdim != 64 && headdim != 128)
    return fail(FA_ERR_UNSUPPORTED, "headdim %d is not supported (64 or 128)", headdim);
  // Kernels address one (batch, head) slice with 32-bit byte offsets (buffer
  // loads take a 32-bit offset); one key tile of slack covers the prefetch.
  const long long esize = dtype == FA_DTYPE_F32 ? 4 : 2;
  if (((long long)seqlen + 128) * heads * headdim * esize >= (1LL << 31))
    return fail(FA_ERR_UNSUPPORTED, "a (batch, head) slice of seqlen*heads*headdim elements "
                "must span less than 2^31 bytes");
  if (!std::isfinite(scale) || !(scale > 0.f))
    return fail(FA_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
  if (wl < -1 || wr < -1)
    return fail(FA_ERR_INVALID_ARG, "window bounds must be >= -1 (got %d, %d)", wl, wr);
  // A bound of seqlen or more excludes no key (0 <= i, j < seqlen), so it is
  // folded to "unbounded"; kernel index sums such as i + wr + 1 then stay
  // far below 2^31.
  *wl_eff = wl >= seqlen ? -1 : wl;
  // causal (j <= i) intersected with j <= i + wr (wr >= 0) is j <= i.
  *wr_eff = causal ? 0 : (wr >= seqlen ? -1 : wr);
  return FA_OK;
}

fa_status_t check_ptr(const void* p, const char* name) {
  if (p == nullptr) return fail(FA_ERR_INVALID_ARG, "%s is null", name);
  if (!aligned16(p)) return fail(FA_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return FA_OK;
}

size_t round256(size_t n) { return (n + 255) & ~(size_t)255; }

// Backward workspace: the row statistics (2 floats per row), then fp16
// copies of Q, K and dO; each part starts on a 256-byte boundary.
struct BwdWorkspace {
  size_t stats, q16, k16, do16, total;
};
BwdWorkspace bwd_workspace(int batch, int heads, int seqlen, int headdim) {
  const size_t rows = (size_t)batch * heads * seqlen;
  const size_t half = round256(rows * headdim * 2);
  BwdWorkspace w;
  w.stats = 0;
  w.q16 = round256(rows * 2 * sizeof(float));
  w.k16 = w.q16 + half;
  w.do16 = w.k16 + half;
  w.total = w.do16 + half;
  return w;
}

}  // namespace

extern "C" {

const char* fa_status_string(fa_status_t s) {
  switch (s) {
    case FA_OK: return "ok";
    case FA_ERR_INVALID_ARG: return "invalid argument";
    case FA_ERR_UNSUPPORTED: return "unsupported configuration";
    case FA_ERR_WORKSPACE: return "workspace missing or too small";
    case FA_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* fa_last_error_message(void) { return g_msg; }

fa_status_t fa_forward(const void* q, const void* k, const void* v, void* out, float* lse,
                       const int32_t* seqlens_k, int batch, int heads, int seqlen, int headdim,
                       float softmax_scale, int causal, int window_left, int window_right,
                       fa_dtype_t dtype, hipStream_t stream) {
  g_msg[0] = '\0';
  int wl, wr;
  fa_status_t s = check_common(batch, heads, seqlen, headdim, softmax_scale, causal,
                               window_left, window_right, dtype, &wl, &wr);
  if (s != FA_OK) return s;
  const void* ptrs[] = {q, k, v, out, lse};
  const char* names[] = {"q", "k", "v", "out", "lse"};
  for (int i = 0; i < 5; ++i)
    if ((s = check_ptr(ptrs[i], names[i])) != FA_OK) return s;
  if (seqlens_k != nullptr && (reinterpret_cast<uintptr_t>(seqlens_k) & 3u))
    return fail(FA_ERR_INVALID_ARG, "seqlens_k is not 4-byte aligned");

  const int f32 = dtype == FA_DTYPE_F32;
  fa::FwdParams p{};
  p.q = q; p.k = k; p.v = v; p.o = out; p.lse = lse;
  p.mask.seqlens_k = seqlens_k;
  p.mask.wl = wl;
  p.mask.wr = wr;
  p.B = batch; p.H = heads; p.N = seqlen;
  const int bm = fa::fwd_block_rows(f32, headdim);
  p.nqb = (seqlen + bm - 1) / bm;
  p.scale_log2 = softmax_scale * 1.4426950408889634f;
  p.xcd_groups = (batch * heads) % 8 == 0 ? 1 : 0;
  p.longest_first = wr >= 0 ? 1 : 0;
  if ((long long)batch * heads * p.nqb >= (1LL << 31))
    return fail(FA_ERR_INVALID_ARG, "grid too large");
  hipError_t e = fa::launch_forward(p, headdim, f32, stream);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "forward launch: %s", hipGetErrorString(e));
  return FA_OK;
}

size_t fa_backward_workspace_size(int batch, int heads, int seqlen, int headdim,
                                  fa_dtype_t dtype) {
  int wl, wr;
  char saved[sizeof g_msg];
  memcpy(saved, g_msg, sizeof g_msg);
  fa_status_t s = check_common(batch, heads, seqlen, headdim, 1.f, 0, -1, -1, dtype, &wl, &wr);
  memcpy(g_msg, saved, sizeof g_msg);
  if (s != FA_OK) return 0;
  return bwd_workspace(batch, heads, seqlen, headdim).total;
}

fa_status_t fa_backward(const void* q, const void* k, const void* v, const void* out,
                        const float* lse, const void* dout, void* dq, void* dk, void* dv,
                        const int32_t* seqlens_k, int batch, int heads, int seqlen, int headdim,
                        float softmax_scale, int causal, int window_left, int window_right,
                        fa_dtype_t dtype, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
  g_msg[0] = '\0';
  int wl, wr;
  fa_status_t s = check_common(batch, heads, seqlen, headdim, softmax_scale, causal,
                               window_left, window_right, dtype, &wl, &wr);
  if (s != FA_OK) return s;
  if (dtype != FA_DTYPE_BF16)
    return fail(FA_ERR_UNSUPPORTED, "the backward is built for bf16 only");
  const void* ptrs[] = {q, k, v, out, lse, dout, dq, dk, dv};
  const char* names[] = {"q", "k", "v", "out", "lse", "dout", "dq", "dk", "dv"};
  for (int i = 0; i < 9; ++i)
    if ((s = check_ptr(ptrs[i], names[i])) != FA_OK) return s;
  if (seqlens_k != nullptr && (reinterpret_cast<uintptr_t>(seqlens_k) & 3u))
    return fail(FA_ERR_INVALID_ARG, "seqlens_k is not 4-byte aligned");
  const BwdWorkspace ws = bwd_workspace(batch, heads, seqlen, headdim);
  const size_t need = ws.total;
  if (workspace == nullptr || workspace_bytes < need)
    return fail(FA_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", need,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  if (!aligned16(workspace)) return fail(FA_ERR_INVALID_ARG, "workspace is not 16-byte aligned");

  fa::BwdParams p{};
  p.q = q; p.k = k; p.v = v; p.o = out; p.dout = dout; p.lse = lse;
  p.dq = dq; p.dk = dk; p.dv = dv;
  char* wsb = static_cast<char*>(workspace);
  p.stats = reinterpret_cast<float*>(wsb + ws.stats);
  p.q16 = wsb + ws.q16;
  p.k16 = wsb + ws.k16;
  p.do16 = wsb + ws.do16;
  p.mask.seqlens_k = seqlens_k;
  p.mask.wl = wl;
  p.mask.wr = wr;
  p.B = batch; p.H = heads; p.N = seqlen;
  p.scale = softmax_scale;
  p.scale_log2 = softmax_scale * 1.4426950408889634f;
  p.xcd_groups = (batch * heads) % 8 == 0 ? 1 : 0;
  hipError_t e = fa::launch_backward(p, headdim, dtype == FA_DTYPE_F32, stream);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "backward launch: %s", hipGetErrorString(e));
  return FA_OK;
}

}  // extern "C"
