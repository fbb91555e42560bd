// fa_launch.h -- host-side launchers behind the C ABI (internal, C++ linkage).
#pragma once

#include <hip/hip_runtime_api.h>

#include "fa.h"
#include "fa_params.h"

namespace fa {

// Record the detail fa_last_error_message() returns for status s on this
// thread (printf-style); returns s.
fa_status_t report(fa_status_t s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// Element type of Q, K, V, O (and dO and the gradients in the backward).
enum class ElemType { kBF16, kF32, kF16 };

// Rows of the query block one forward work-group owns.
int fwd_block_rows(ElemType et, int headdim);
// Enqueue the forward on `stream`; p.nqb must equal ceil(N / fwd_block_rows()).
hipError_t launch_forward(FwdParams p, int headdim, ElemType et, hipStream_t stream);

// fp8 (e4m3) forward: p.scale_log2 already holds softmax_scale * descale_q *
// descale_k * log2(e); O is scaled by v_descale. p.nqb must equal
// ceil(N / fwd_fp8_block_rows()).
int fwd_fp8_block_rows(int headdim);
hipError_t launch_forward_fp8(FwdParams p, float v_descale, int headdim, hipStream_t stream);

// Backward: row statistic, then dK/dV (one pass over the queries per key
// block) and dQ (one pass over the keys per query block).
hipError_t launch_backward(BwdParams p, int headdim, ElemType et, hipStream_t stream);

}  // namespace fa
