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

fa::ElemType elem_type(fa_dtype_t dtype) {
  return dtype == FA_DTYPE_F32 ? fa::ElemType::kF32
       : dtype == FA_DTYPE_F16 ? fa::ElemType::kF16 : fa::ElemType::kBF16;
}

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
                         int* wr_eff, int row_mult = 1, int elem_bytes = 0) {
  if (batch < 0 || heads < 0 || seqlen < 0)
    return fail(FA_ERR_INVALID_ARG, "batch, heads and seqlen must be >= 0 (got %d, %d, %d)",
                batch, heads, seqlen);
  if (seqlen > (1 << 24))
    return fail(FA_ERR_INVALID_ARG, "seqlen %d exceeds 2^24", seqlen);
  if ((long long)batch * heads * seqlen >= (1LL << 31))
    return fail(FA_ERR_INVALID_ARG, "batch*heads*seqlen must be < 2^31");
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F32 && dtype != FA_DTYPE_F16)
    return fail(FA_ERR_UNSUPPORTED, "dtype %d is not supported", (int)dtype);
  if (headdim != 64 && headdim != 128)
    return fail(FA_ERR_UNSUPPORTED, "headdim %d is not supported (64 or 128)", headdim);
  // Kernels address one (batch, head) slice with 32-bit byte offsets (buffer
  // loads take a 32-bit offset); one key tile of slack covers the prefetch.
  // row_mult is 3 for a packed (batch, seqlen, 3, heads, headdim) input;
  // elem_bytes, when set, overrides the element size of dtype.
  const long long esize = elem_bytes > 0 ? elem_bytes : (dtype == FA_DTYPE_F32 ? 4 : 2);
  if (((long long)seqlen + 128) * row_mult * heads * headdim * esize >= (1LL << 31))
    return fail(FA_ERR_UNSUPPORTED, "a (batch, head) slice of seqlen rows of the input must "
                "span less than 2^31 bytes");
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

// A call with no rows has nothing to compute: after its scalar arguments
// pass, it returns FA_OK without reading any pointer or launching anything.
bool empty_call(int batch, int heads, int seqlen) { return batch == 0 || heads == 0 || seqlen == 0; }

fa_status_t check_ptr(const void* p, const char* name) {
  if (p == nullptr) return fail(FA_ERR_INVALID_ARG, "%s is null", name);
  if (!aligned16(p)) return fail(FA_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return FA_OK;
}

// Three per-(q, k, v) pointers of a call and their row stride in elements:
// three tensors, or one packed (batch, seqlen, 3, heads, headdim) tensor in
// the first pointer ([notes] docstring, qkv argument) with the other two
// null. names = {packed name, first, second, third}.
fa_status_t resolve_qkv(const void* a, const void* b, const void* c, int packed, int heads,
                        int headdim, fa_dtype_t dtype, const char* const names[4],
                        void* out[3], int* rs) {
  fa_status_t s;
  if (packed) {
    if ((s = check_ptr(a, names[0])) != FA_OK) return s;
    if (b != nullptr || c != nullptr)
      return fail(FA_ERR_INVALID_ARG, "%s and %s must be null when qkv_packed is set", names[2],
                  names[3]);
    const size_t step = (size_t)heads * headdim * (dtype == FA_DTYPE_F32 ? 4 : 2);
    char* base = static_cast<char*>(const_cast<void*>(a));
    out[0] = base;
    out[1] = base + step;
    out[2] = base + 2 * step;
    *rs = 3 * heads * headdim;
    return FA_OK;
  }
  const void* ptrs[] = {a, b, c};
  for (int i = 0; i < 3; ++i) {
    if ((s = check_ptr(ptrs[i], names[i + 1])) != FA_OK) return s;
    out[i] = const_cast<void*>(ptrs[i]);
  }
  *rs = heads * headdim;
  return FA_OK;
}

const char* const kQkvNames[4] = {"qkv", "q", "k", "v"};
const char* const kGradNames[4] = {"dqkv", "dq", "dk", "dv"};

// ALiBi slopes: null, or 4-byte aligned with a batch stride of 0 or heads.
fa_status_t check_alibi(const float* slopes, int bstride, int heads) {
  if (slopes == nullptr) return FA_OK;
  if (reinterpret_cast<uintptr_t>(slopes) & 3u)
    return fail(FA_ERR_INVALID_ARG, "alibi_slopes is not 4-byte aligned");
  if (bstride != 0 && bstride != heads)
    return fail(FA_ERR_INVALID_ARG, "alibi_batch_stride must be 0 or heads (got %d)", bstride);
  return FA_OK;
}

size_t round256(size_t n) { return (n + 255) & ~(size_t)255; }

// Backward workspace: the row statistics (2 floats per row), fp16 copies
// of Q, K and dO, then the pre-pass's per-block maxima of |Q|, |K|, |V|,
// |dO| (kMaxParts blocks of 4 floats per (batch, head)); each part starts
// on a 256-byte boundary.
struct BwdWorkspace {
  size_t stats, q16, k16, do16, part, total;
};
BwdWorkspace bwd_workspace(int batch, int heads, int seqlen, int headdim) {
  const size_t rows = (size_t)batch * heads * seqlen;
  const size_t half = round256(rows * headdim * 2);
  BwdWorkspace w;
  w.stats = 0;
  w.q16 = round256(rows * 2 * sizeof(float));
  w.k16 = w.q16 + half;
  w.do16 = w.k16 + half;
  w.part = w.do16 + half;
  w.total = w.part + (rows == 0 ? 0 : round256((size_t)batch * heads * fa::kMaxParts * 4 * sizeof(float)));
  return w;
}

}  // namespace

namespace fa {

fa_status_t report(fa_status_t s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof g_msg, fmt, ap);
  va_end(ap);
  return s;
}

}  // namespace fa

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

fa_status_t fa_forward_ex(const void* q, const void* k, const void* v, int qkv_packed,
                          void* out, float* lse, const int32_t* seqlens_k,
                          const float* alibi_slopes, int alibi_batch_stride, int batch, int heads,
                          int seqlen, int headdim, float softmax_scale, int causal,
                          int window_left, int window_right, fa_dtype_t dtype,
                          hipStream_t stream) {
  g_msg[0] = '\0';
  int wl, wr;
  fa_status_t s = check_common(batch, heads, seqlen, headdim, softmax_scale, causal,
                               window_left, window_right, dtype, &wl, &wr, qkv_packed ? 3 : 1);
  if (s != FA_OK) return s;
  if (empty_call(batch, heads, seqlen)) return FA_OK;
  void* qkv[3];
  int rs_q;
  if ((s = resolve_qkv(q, k, v, qkv_packed, heads, headdim, dtype, kQkvNames, qkv, &rs_q)) !=
      FA_OK)
    return s;
  if ((s = check_ptr(out, "out")) != FA_OK) return s;
  if ((s = check_ptr(lse, "lse")) != FA_OK) return s;
  if (seqlens_k != nullptr && (reinterpret_cast<uintptr_t>(seqlens_k) & 3u))
    return fail(FA_ERR_INVALID_ARG, "seqlens_k is not 4-byte aligned");
  if ((s = check_alibi(alibi_slopes, alibi_batch_stride, heads)) != FA_OK) return s;

  const fa::ElemType et = elem_type(dtype);
  fa::FwdParams p{};
  p.q = qkv[0]; p.k = qkv[1]; p.v = qkv[2]; p.o = out; p.lse = lse;
  p.mask.seqlens_k = seqlens_k;
  p.mask.wl = wl;
  p.mask.wr = wr;
  p.alibi.slopes = alibi_slopes;
  p.alibi.bstride = alibi_batch_stride;
  p.B = batch; p.H = heads; p.N = seqlen;
  p.rs_q = rs_q;
  p.rs_o = heads * headdim;
  const int bm = fa::fwd_block_rows(et, headdim);
  p.nqb = (seqlen + bm - 1) / bm;
  p.scale_log2 = softmax_scale * 1.4426950408889634f;
  p.xcd_groups = (batch * heads) % 8 == 0 ? 1 : 0;
  p.longest_first = wr >= 0 ? 1 : 0;
  if ((long long)batch * heads * p.nqb >= (1LL << 31))
    return fail(FA_ERR_INVALID_ARG, "grid too large");
  hipError_t e = fa::launch_forward(p, headdim, et, stream);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "forward launch: %s", hipGetErrorString(e));
  return FA_OK;
}

fa_status_t fa_forward(const void* q, const void* k, const void* v, void* out, float* lse,
                       const int32_t* seqlens_k, int batch, int heads, int seqlen, int headdim,
                       float softmax_scale, int causal, int window_left, int window_right,
                       fa_dtype_t dtype, hipStream_t stream) {
  return fa_forward_ex(q, k, v, 0, out, lse, seqlens_k, nullptr, 0, batch, heads, seqlen,
                       headdim, softmax_scale, causal, window_left, window_right, dtype, stream);
}

fa_status_t fa_forward_fp8(const void* q, const void* k, const void* v, void* out, float* lse,
                           const int32_t* seqlens_k, int batch, int heads, int seqlen,
                           int headdim, float softmax_scale, float descale_q, float descale_k,
                           float descale_v, int causal, int window_left, int window_right,
                           hipStream_t stream) {
  g_msg[0] = '\0';
  int wl, wr;
  fa_status_t s = check_common(batch, heads, seqlen, headdim, softmax_scale, causal,
                               window_left, window_right, FA_DTYPE_BF16, &wl, &wr, 1, 1);
  if (s != FA_OK) return s;
  const float ds[3] = {descale_q, descale_k, descale_v};
  const char* const dnames[3] = {"descale_q", "descale_k", "descale_v"};
  for (int i = 0; i < 3; ++i)
    if (!std::isfinite(ds[i]) || !(ds[i] > 0.f))
      return fail(FA_ERR_INVALID_ARG, "%s must be finite and > 0", dnames[i]);
  const float scale_log2 = softmax_scale * descale_q * descale_k * 1.4426950408889634f;
  if (!std::isfinite(scale_log2) || !(scale_log2 > 0.f))
    return fail(FA_ERR_INVALID_ARG, "softmax_scale * descale_q * descale_k is not a finite "
                "positive fp32 value");
  // |q . k| <= 448^2 headdim over e4m3 codes; the kernel needs every scaled
  // score (log2 units) far inside fp32 range, above its -1e30 "no key yet" mark.
  if ((double)scale_log2 * 448.0 * 448.0 * headdim > 0x1p64)
    return fail(FA_ERR_INVALID_ARG, "softmax_scale * descale_q * descale_k is too large: "
                "scaled scores could exceed 2^64");
  if (empty_call(batch, heads, seqlen)) return FA_OK;
  const void* ptrs[] = {q, k, v};
  for (int i = 0; i < 3; ++i)
    if ((s = check_ptr(ptrs[i], kQkvNames[i + 1])) != FA_OK) return s;
  if ((s = check_ptr(out, "out")) != FA_OK) return s;
  if ((s = check_ptr(lse, "lse")) != FA_OK) return s;
  if (seqlens_k != nullptr && (reinterpret_cast<uintptr_t>(seqlens_k) & 3u))
    return fail(FA_ERR_INVALID_ARG, "seqlens_k is not 4-byte aligned");

  fa::FwdParams p{};
  p.q = q; p.k = k; p.v = v; p.o = out; p.lse = lse;
  p.mask.seqlens_k = seqlens_k;
  p.mask.wl = wl;
  p.mask.wr = wr;
  p.B = batch; p.H = heads; p.N = seqlen;
  p.rs_q = heads * headdim;  // bytes: one byte per element
  p.rs_o = heads * headdim;
  const int bm = fa::fwd_fp8_block_rows(headdim);
  p.nqb = (seqlen + bm - 1) / bm;
  p.scale_log2 = scale_log2;
  p.xcd_groups = (batch * heads) % 8 == 0 ? 1 : 0;
  p.longest_first = wr >= 0 ? 1 : 0;
  if ((long long)batch * heads * p.nqb >= (1LL << 31))
    return fail(FA_ERR_INVALID_ARG, "grid too large");
  hipError_t e = fa::launch_forward_fp8(p, descale_v, headdim, stream);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "fp8 forward launch: %s", hipGetErrorString(e));
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

fa_status_t fa_backward_ex(const void* q, const void* k, const void* v, int qkv_packed,
                           const void* out, const float* lse, const void* dout, void* dq,
                           void* dk, void* dv, const int32_t* seqlens_k,
                           const float* alibi_slopes, int alibi_batch_stride, int batch,
                           int heads, int seqlen, int headdim, float softmax_scale, int causal,
                           int window_left, int window_right, fa_dtype_t dtype, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  g_msg[0] = '\0';
  int wl, wr;
  fa_status_t s = check_common(batch, heads, seqlen, headdim, softmax_scale, causal,
                               window_left, window_right, dtype, &wl, &wr, qkv_packed ? 3 : 1);
  if (s != FA_OK) return s;
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F16)
    return fail(FA_ERR_UNSUPPORTED, "the backward is built for bf16 and fp16 only");
  if (empty_call(batch, heads, seqlen)) return FA_OK;
  void* qkv[3];
  int rs_q;
  if ((s = resolve_qkv(q, k, v, qkv_packed, heads, headdim, dtype, kQkvNames, qkv, &rs_q)) !=
      FA_OK)
    return s;
  // The gradients take the layout of the inputs: dq holds the packed dqkv.
  void* grads[3];
  int rs_g;
  if ((s = resolve_qkv(dq, dk, dv, qkv_packed, heads, headdim, dtype, kGradNames, grads,
                       &rs_g)) != FA_OK)
    return s;
  const void* ptrs[] = {out, lse, dout};
  const char* names[] = {"out", "lse", "dout"};
  for (int i = 0; i < 3; ++i)
    if ((s = check_ptr(ptrs[i], names[i])) != FA_OK) return s;
  if (seqlens_k != nullptr && (reinterpret_cast<uintptr_t>(seqlens_k) & 3u))
    return fail(FA_ERR_INVALID_ARG, "seqlens_k is not 4-byte aligned");
  if ((s = check_alibi(alibi_slopes, alibi_batch_stride, heads)) != FA_OK) return s;
  const BwdWorkspace ws = bwd_workspace(batch, heads, seqlen, headdim);
  const size_t need = ws.total;
  if (workspace == nullptr || workspace_bytes < need)
    return fail(FA_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", need,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  if (!aligned16(workspace)) return fail(FA_ERR_INVALID_ARG, "workspace is not 16-byte aligned");

  fa::BwdParams p{};
  p.q = qkv[0]; p.k = qkv[1]; p.v = qkv[2]; p.o = out; p.dout = dout; p.lse = lse;
  p.dq = grads[0];
  p.dk = grads[1];
  p.dv = grads[2];
  char* wsb = static_cast<char*>(workspace);
  p.stats = reinterpret_cast<float*>(wsb + ws.stats);
  p.q16 = wsb + ws.q16;
  p.k16 = wsb + ws.k16;
  p.do16 = wsb + ws.do16;
  p.part = reinterpret_cast<float*>(wsb + ws.part);
  p.mask.seqlens_k = seqlens_k;
  p.mask.wl = wl;
  p.mask.wr = wr;
  p.alibi.slopes = alibi_slopes;
  p.alibi.bstride = alibi_batch_stride;
  p.B = batch; p.H = heads; p.N = seqlen;
  p.rs_q = rs_q;
  p.rs_o = heads * headdim;
  p.rs_g = rs_g;
  p.scale = softmax_scale;
  p.scale_log2 = softmax_scale * 1.4426950408889634f;
  p.xcd_groups = (batch * heads) % 8 == 0 ? 1 : 0;
  hipError_t e = fa::launch_backward(p, headdim, elem_type(dtype), stream);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "backward launch: %s", hipGetErrorString(e));
  return FA_OK;
}

fa_status_t fa_backward(const void* q, const void* k, const void* v, const void* out,
                        const float* lse, const void* dout, void* dq, void* dk, void* dv,
                        const int32_t* seqlens_k, int batch, int heads, int seqlen, int headdim,
                        float softmax_scale, int causal, int window_left, int window_right,
                        fa_dtype_t dtype, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
  return fa_backward_ex(q, k, v, 0, out, lse, dout, dq, dk, dv, seqlens_k, nullptr, 0, batch,
                        heads, seqlen, headdim, softmax_scale, causal, window_left, window_right,
                        dtype, workspace, workspace_bytes, stream);
}

}  // extern "C"
