/*
 * fa.h -- C ABI of the MI355X (gfx950) exact-attention library (libfa_mi355x.so).
 *
 * The library computes exact attention in the tiled, IO-aware way the
 * FlashAttention pages describe: K/V tiles are streamed through on-chip memory
 * under an online softmax (running row max m, running sum l, rescaled partial
 * O), so the N x N score matrix never reaches HBM; the forward also writes the
 * per-row log-sum-exp, and the backward rebuilds the probabilities from it.
 *
 * Pages cited (title or address, and section):
 *   [interview] meko1 LLM interview guide, "FlashAttention 深入": sections
 *               "Online Softmax（增量式 softmax）" and "反向传播：用重计算换显存".
 *   [scratch]   l189.com/news/1255901 (implementing Flash Attention from scratch
 *               in PyTorch): §2.2 online softmax, §3.1 blocked forward and the
 *               LSE statistic, §3.3 backward (recompute P from LSE; softmax
 *               Jacobian), §5.2 numerical stability, §5.3 causal mask.
 *   [notes]     claire-chang.com/post/flashattention-introduction, section
 *               "flash_attn 的程式碼怎麼寫？" (flash_attn_qkvpacked_func docstring):
 *               (batch, seqlen, nheads, headdim) layout, softmax_scale default
 *               1/sqrt(headdim), causal flag, window_size (left, right) with
 *               keys [i - left, i + right] inclusive and -1 meaning unbounded,
 *               deterministic backward, the packed qkv input (batch, seqlen,
 *               3, nheads, headdim), and ALiBi slopes (fp32, per head or per
 *               batch and head; the score of query i and key j is lowered by
 *               slope times |i - j|).
 *
 * Conventions shared by every entry point:
 *   - Tensor pointers are DEVICE pointers to contiguous arrays, 16-byte
 *     aligned. Q, K, V, O, dO, dQ, dK, dV have layout [batch][seqlen][heads]
 *     [headdim] ([notes]); LSE and the backward's row statistic have layout
 *     [batch][heads][seqlen], fp32.
 *   - dtype selects the element type of Q, K, V, O, dO, dQ, dK, dV:
 *     FA_DTYPE_BF16 (bfloat16) or FA_DTYPE_F16 (IEEE half), both on MFMA with
 *     fp32 accumulation, or FA_DTYPE_F32 (forward only).
 *     LSE is always fp32 (natural log). Outputs are rounded to nearest even.
 *   - Ownership: the caller owns every buffer, the workspace included. The
 *     library allocates and frees nothing and keeps no pointer after a call.
 *   - Asynchrony: work is enqueued on `stream` and the call returns without
 *     synchronising. A null stream is the default stream.
 *   - Errors: every argument is checked before any launch. On a check failure
 *     the call returns FA_ERR_INVALID_ARG / FA_ERR_UNSUPPORTED /
 *     FA_ERR_WORKSPACE and writes nothing; fa_last_error_message() then names
 *     the argument. If a launch fails, the call returns FA_ERR_HIP and the
 *     outputs are undefined.
 *   - Masks: visible(i, j) = (!causal || j <= i)
 *                         && (window_left  < 0 || j >= i - window_left)
 *                         && (window_right < 0 || j <= i + window_right)
 *                         && j < L_b
 *     where L_b = seqlens_k[b] clamped to [0, seqlen] if seqlens_k is not NULL,
 *     else seqlen. A query row with no visible key gets O = 0, LSE = -inf and
 *     zero gradient contributions.
 *   - Supported sizes: headdim in {64, 128}; batch, heads, seqlen >= 0;
 *     batch * heads * seqlen < 2^31 and seqlen <= 2^24; one (batch, head)
 *     slice, (seqlen + 128) * heads * headdim elements, below 2^31 bytes
 *     (else FA_ERR_UNSUPPORTED); softmax_scale finite and > 0.
 *   - Empty calls: when batch, heads or seqlen is 0 and the scalar arguments
 *     are valid, a call returns FA_OK at once. It reads no pointer (they may
 *     be null), writes nothing and enqueues nothing.
 */
#ifndef FA_MI355X_H
#define FA_MI355X_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FA_DTYPE_BF16 = 0, FA_DTYPE_F32 = 1, FA_DTYPE_F16 = 2 } fa_dtype_t;

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = 1,  /* null/misaligned pointer, bad size, bad window or scale */
  FA_ERR_UNSUPPORTED = 2,  /* well-formed but not built: headdim, dtype */
  FA_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required */
  FA_ERR_HIP = 4           /* a HIP launch or runtime call failed */
} fa_status_t;

/*
 * fa_forward -- exact attention forward.
 * Computes O = softmax(softmax_scale * Q K^T + mask) V and, per query row,
 * LSE = ln sum_j exp(softmax_scale * q_i . k_j) over visible keys
 * ([scratch] §3.1 and §2.2; [interview] "Online Softmax").
 *   q, k, v   in : [batch][seqlen][heads][headdim], dtype
 *   out       out: [batch][seqlen][heads][headdim], dtype
 *   lse       out: [batch][heads][seqlen], fp32, natural log (-inf for empty rows)
 *   seqlens_k in : [batch] int32 key lengths (device), or NULL for "all seqlen"
 *   softmax_scale : scale of Q K^T; pass 1/sqrt(headdim) for the usual default
 *   causal        : nonzero keeps keys j <= i ([scratch] §5.3)
 *   window_left, window_right : sliding window, -1 = unbounded ([notes])
 * out and lse must not overlap the inputs.
 */
fa_status_t fa_forward(const void* q, const void* k, const void* v,
                       void* out, float* lse, const int32_t* seqlens_k,
                       int batch, int heads, int seqlen, int headdim,
                       float softmax_scale, int causal,
                       int window_left, int window_right,
                       fa_dtype_t dtype, hipStream_t stream);

/*
 * fa_backward_workspace_size -- bytes of device workspace fa_backward needs
 * for these sizes: per row the fp32 pair (LSE log2 e, D_i = sum_d dO_id O_id),
 * [batch][heads][seqlen][2], then fp16 copies of Q, K and dO (each
 * batch*seqlen*heads*headdim*2 bytes), then per (batch, head) 64 groups of
 * 4 fp32 maxima (|Q|, |K|, |V|, |dO| over blocks of rows), every part rounded
 * up to 256 bytes. Returns 0 for invalid sizes and for empty calls.
 */
size_t fa_backward_workspace_size(int batch, int heads, int seqlen, int headdim,
                                  fa_dtype_t dtype);

/*
 * fa_backward -- gradients of exact attention, recomputing P from the saved
 * LSE instead of storing it ([interview] "反向传播：用重计算换显存";
 * [scratch] §3.3):
 *   P = exp(softmax_scale * Q K^T - LSE) on visible pairs, 0 elsewhere
 *   dV = P^T dO;  dP = dO V^T;  D_i = sum_d dO_id O_id (= sum_j P_ij dP_ij)
 *   dS = P * (dP - D);  dQ = softmax_scale * dS K;  dK = softmax_scale * dS^T Q
 * The softmax Jacobian's row sum is taken over the whole row.
 *   q, k, v, out, dout  in : [batch][seqlen][heads][headdim], dtype; out is
 *                            the forward's output for the same arguments
 *   lse                 in : [batch][heads][seqlen] fp32 from fa_forward
 *   dq, dk, dv          out: [batch][seqlen][heads][headdim], dtype
 *   workspace           scratch of at least fa_backward_workspace_size() bytes,
 *                       16-byte aligned; its contents on entry are ignored
 * The mask arguments must match the forward call that produced out and lse.
 * The result is deterministic: dQ is produced by its own pass over the keys
 * (no atomics), dK and dV by a pass over the queries.
 * dtype is FA_DTYPE_BF16 or FA_DTYPE_F16 (FA_DTYPE_F32 returns
 * FA_ERR_UNSUPPORTED).
 * Precision: every product with P or dS as an operand takes fp16 operands
 * (fp32 accumulation), and so do the products that recompute S and dP from
 * those copies. Within each (batch, head) slice, Q, K, V and dO are used as
 * they are when their largest magnitude lies in [2^-6, 8]; a tensor whose
 * slice maximum lies outside it is scaled by an exact power of two 2^e,
 * |e| <= 40, that brings the maximum into [4, 8), and the kernels undo the
 * scale exactly ([scratch] §5.2, numerical stability). Any finite input
 * whose slice maxima lie within [2^-38, 2^42] is therefore handled with the
 * same relative precision: no fp16 overflow, and no loss to fp16's
 * subnormal range above 2^-8 of the slice maximum. The gradients must be
 * finite in the output dtype.
 */
fa_status_t fa_backward(const void* q, const void* k, const void* v,
                        const void* out, const float* lse, const void* dout,
                        void* dq, void* dk, void* dv,
                        const int32_t* seqlens_k,
                        int batch, int heads, int seqlen, int headdim,
                        float softmax_scale, int causal,
                        int window_left, int window_right,
                        fa_dtype_t dtype, void* workspace, size_t workspace_bytes,
                        hipStream_t stream);

/*
 * fa_forward_ex -- fa_forward with the two further options of the
 * flash_attn_qkvpacked_func docstring ([notes]).
 *   qkv_packed     : nonzero: q points at ONE tensor [batch][seqlen][3][heads]
 *                    [headdim] holding Q, K and V (in that order), and k and v
 *                    must be NULL (else FA_ERR_INVALID_ARG). out stays
 *                    [batch][seqlen][heads][headdim].
 *   alibi_slopes   : NULL, or a device fp32 array of slopes, 4-byte aligned;
 *                    the score of query i and key j in (b, h) becomes
 *                    softmax_scale * q_i . k_j - slope * |i - j|, with
 *                    slope = alibi_slopes[b * alibi_batch_stride + h].
 *   alibi_batch_stride : 0 for (heads,) slopes, heads for (batch, heads);
 *                    anything else is FA_ERR_INVALID_ARG. Ignored when
 *                    alibi_slopes is NULL. The slopes are read on the device.
 * Every other argument, the conventions above and the error behaviour are
 * those of fa_forward, which equals fa_forward_ex(q, k, v, 0, ..., NULL, 0, ...).
 * A packed input's (batch, head) slice spans seqlen rows of 3*heads*headdim
 * elements, which must stay below 2^31 bytes.
 */
fa_status_t fa_forward_ex(const void* q, const void* k, const void* v, int qkv_packed,
                          void* out, float* lse, const int32_t* seqlens_k,
                          const float* alibi_slopes, int alibi_batch_stride,
                          int batch, int heads, int seqlen, int headdim,
                          float softmax_scale, int causal,
                          int window_left, int window_right,
                          fa_dtype_t dtype, hipStream_t stream);

/*
 * fa_backward_ex -- fa_backward with the options of fa_forward_ex, which must
 * match the forward call that produced out and lse.
 *   qkv_packed : nonzero: q is the packed qkv input as in fa_forward_ex (k, v
 *                NULL) and dq points at ONE gradient tensor [batch][seqlen][3]
 *                [heads][headdim] receiving dQ, dK and dV in the same order
 *                (dk, dv NULL), so no concatenation of gradients is needed
 *                ([notes]). out and dout stay [batch][seqlen][heads][headdim].
 *   alibi_slopes, alibi_batch_stride : as in fa_forward_ex. The bias does not
 *                depend on Q or K, so the gradient formulas are unchanged.
 * Workspace, conventions and errors are those of fa_backward, which equals
 * fa_backward_ex(q, k, v, 0, ..., NULL, 0, ...).
 */
fa_status_t fa_backward_ex(const void* q, const void* k, const void* v, int qkv_packed,
                           const void* out, const float* lse, const void* dout,
                           void* dq, void* dk, void* dv,
                           const int32_t* seqlens_k,
                           const float* alibi_slopes, int alibi_batch_stride,
                           int batch, int heads, int seqlen, int headdim,
                           float softmax_scale, int causal,
                           int window_left, int window_right,
                           fa_dtype_t dtype, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/*
 * fa_forward_fp8 -- the forward of fa_forward over fp8 inputs. The pages list
 * an FP8 forward among the additions of FlashAttention-3 ([interview] section
 * "v1 → v2 → v3 演进", the v3 row; [wiki] section "典型例子", the paragraph on
 * the official repository); here it runs on the gfx950 fp8 matrix cores.
 *   q, k, v   in : [batch][seqlen][heads][headdim], one byte per element in
 *                  the OCP e4m3 format (bias 7, 3 mantissa bits, subnormals,
 *                  0x7f / 0xff NaN, no infinities)
 *   descale_q, descale_k, descale_v : fp32 factors, finite and > 0; element x
 *                  of Q stands for e4m3(x) * descale_q, and likewise for K, V;
 *                  softmax_scale * descale_q * descale_k * log2(e) * 448^2 *
 *                  headdim must not exceed 2^64 (every scaled score stays far
 *                  inside fp32 range), else FA_ERR_INVALID_ARG
 *   out       out: [batch][seqlen][heads][headdim], bfloat16
 *   lse       out: [batch][heads][seqlen], fp32, natural log
 * The result is the attention of fa_forward over the dequantised inputs, with
 * one further rounding, which the fp8 P V product forces: each softmax weight
 * w (an exact probability of the row) enters that product as e4m3(c w) / c,
 * rounded to nearest even, for factors c > 0 (which may differ between the
 * row's key tiles) with c w <= 448 for every weight rounded with it and
 * c w_max >= 1, w_max the row's largest weight. From the e4m3 format alone
 * (relative spacing 2^-3 above 2^-6, absolute spacing 2^-9 below), each
 * weight then moves by at most max(2^-4 w, min(w, 2^-10 w_max)), and each
 * output element by at most the sum over keys of that times |v|. The LSE is
 * computed from the unrounded probabilities.
 * Inputs must not hold NaN. seqlens_k, softmax_scale, causal, the window, the
 * conventions and the error behaviour are those of fa_forward (dtype is fixed
 * here); a (batch, head) slice of seqlen + 128 rows must span less than 2^31
 * bytes.
 */
fa_status_t fa_forward_fp8(const void* q, const void* k, const void* v,
                           void* out, float* lse, const int32_t* seqlens_k,
                           int batch, int heads, int seqlen, int headdim,
                           float softmax_scale, float descale_q, float descale_k,
                           float descale_v, int causal,
                           int window_left, int window_right, hipStream_t stream);

/*
 * fa_backward_noalloc -- fa_backward for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, and harnesses
 * that forbid hipMalloc. The workspace is not a caller buffer but a static
 * device array inside the library of FA_NOALLOC_SCRATCH_BYTES bytes; each GPU
 * the library runs on holds its own copy from the library's load until the
 * process ends. The call allocates nothing (no hipMalloc or hipFree, no
 * allocating library routine); it looks the array's address up once per
 * device, on its first call with that device current.
 * Arguments, results, conventions and errors are those of fa_backward without
 * the workspace arguments. Sizes whose fa_backward_workspace_size exceeds
 * FA_NOALLOC_SCRATCH_BYTES return FA_ERR_WORKSPACE before anything is read or
 * launched (128 MiB serves, for instance, batch 2, 8 heads, seqlen 4096,
 * headdim 128). Whatever the backward needs cleared, its kernels clear on the
 * device; the array keeps the last call's contents.
 * Every call on one GPU uses that GPU's one array: calls that overlap on a
 * GPU (on different streams, or from several host threads) race and give
 * undefined results. Serialise them.
 */
#define FA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
fa_status_t fa_backward_noalloc(const void* q, const void* k, const void* v,
                                const void* out, const float* lse, const void* dout,
                                void* dq, void* dk, void* dv,
                                const int32_t* seqlens_k,
                                int batch, int heads, int seqlen, int headdim,
                                float softmax_scale, int causal,
                                int window_left, int window_right,
                                fa_dtype_t dtype, hipStream_t stream);

/* Static English name of a status code. Never NULL. */
const char* fa_status_string(fa_status_t status);

/* Detail of the last non-OK status returned on the calling thread ("" if none).
 * The pointer stays valid until the thread's next call into the library. */
const char* fa_last_error_message(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_H */
