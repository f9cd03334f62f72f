// Argument checks of the C ABI (HIP-free; see qlora_validate.cpp).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "qlora.h"

int qv_quantize(const float* W, int64_t N, int64_t K, const float* codebook16, int32_t blocksize, int32_t dq_group,
                const uint8_t* codes, const float* absmax, const uint8_t* absmax_q, const float* absmax_scale);
int qv_dequantize(const qlora_nf4* w, int32_t out_dtype, const void* out);
int qv_grouped(const qlora_grouped* Q);
int qv_grouped_dB(const qlora_grouped* Q, void* const* dB);
size_t qv_rmsnorm_ws(int64_t M, int64_t D);
int qv_rmsnorm_fwd(const void* X, const void* w, int64_t M, int64_t D, float eps, const void* Y, const float* rstd);
int qv_rmsnorm_bwd(const void* dY, const void* X, const void* w, const float* rstd, int64_t M, int64_t D,
                   const void* dX, const float* dw, const void* ws, size_t ws_bytes);
int qv_merge(const qlora_linear* L, int32_t out_dtype, const void* out);
int qv_linear_fwd(const qlora_linear* L, const void* X, int64_t M, const void* Y, const float* XA, const void* ws,
                  size_t ws_bytes);
// qlora_linear_fwd_static: the arguments of qlora_linear_fwd without a
// workspace; QLORA_ERR_WORKSPACE_TOO_SMALL when the pass needs more than
// scratch_bytes of scratch.
int qv_linear_fwd_static(const qlora_linear* L, const void* X, int64_t M, const void* Y, const float* XA,
                         size_t scratch_bytes);
int qv_linear_bwd(const qlora_linear* L, const void* dY, const void* X, const float* XA, int64_t M, const void* dX,
                  const void* dA, const void* dB, const void* ws, size_t ws_bytes);
int qv_mlp_fwd(const qlora_mlp* P, const void* X, int64_t M, const void* Y, const qlora_mlp_saved* S, const void* ws,
               size_t ws_bytes);
int qv_mlp_fwd_rmsnorm(const qlora_mlp* P, const void* X, const void* norm_w, float eps, int64_t M, const void* Y,
                       const qlora_mlp_saved* S, const float* rstd, const void* Xn, const void* ws, size_t ws_bytes);
int qv_mlp_bwd(const qlora_mlp* P, const void* dY, const void* X, const qlora_mlp_saved* S, int64_t M, const void* dX,
               const qlora_mlp_grads* G, const void* ws, size_t ws_bytes);
size_t qv_linear_ce_ws(int64_t T, int64_t D, int64_t V, int64_t chunk, int32_t want_dx);
int qv_linear_ce(const void* X, int64_t T, int64_t D, const void* W, int64_t V, const int32_t* targets,
                 int64_t chunk, const float* loss, const float* token_loss, const void* dX, const void* ws,
                 size_t ws_bytes);
