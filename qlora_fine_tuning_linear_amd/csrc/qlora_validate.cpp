// Argument validation and workspace sizing of the C ABI (include/qlora.h).
// This translation unit uses no HIP: every check here runs before anything
// touches the GPU, so the rejection paths can be exercised on a host without
// one.
#include <math.h>
#include <stdint.h>

#include "qlora.h"
#include "qlora_plan.h"
#include "qlora_validate.h"

namespace {

constexpr int64_t kMaxDim = ((int64_t)1 << 22) - 64;  // 4194240
// The MLP backward reads [W_g^T | W_u^T] as one bf16 copy with row stride 2I,
// and the cross-entropy's dX product its logit gradient with row stride 2V: a
// 256-row tile of either must stay below 2 GiB as well.
constexpr int64_t kMaxMlpI = (kMaxDim / 2) / 64 * 64;  // 2097088
// Tokens per call: keeps every workspace size and launch grid in range.
constexpr int64_t kMaxTokens = ((int64_t)1 << 31) - 1;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_nf4(const qlora_nf4* w) {
  if (!w || !w->codes || !w->codebook) return QLORA_ERR_INVALID_ARG;
  if (w->N < 0 || w->K < 0) return QLORA_ERR_INVALID_ARG;
  if (w->blocksize != 64) return QLORA_ERR_UNSUPPORTED_SHAPE;
  if (w->dq_group != 0 && w->dq_group != 256) return QLORA_ERR_UNSUPPORTED_SHAPE;
  if (w->dq_group == 0 && !w->absmax) return QLORA_ERR_INVALID_ARG;
  if (w->dq_group != 0 && (!w->absmax_q || !w->absmax_scale)) return QLORA_ERR_INVALID_ARG;
  if (w->N == 0 || w->K == 0) return QLORA_ERR_UNSUPPORTED_SHAPE;
  if (w->K % 64 != 0 || w->N % 64 != 0) return QLORA_ERR_UNSUPPORTED_SHAPE;
  // a 256-row tile of a bf16 row-major copy must stay below 2 GiB (32-bit
  // buffer offsets of the GEMM's direct loads)
  if (w->K > kMaxDim || w->N > kMaxDim) return QLORA_ERR_UNSUPPORTED_SHAPE;
  if (!aligned16(w->codes) || !aligned16(w->codebook)) return QLORA_ERR_MISALIGNED;
  if (w->dq_group == 0 && !aligned16(w->absmax)) return QLORA_ERR_MISALIGNED;
  if (w->dq_group != 0 && !aligned16(w->absmax_scale)) return QLORA_ERR_MISALIGNED;
  return QLORA_OK;
}

int check_linear(const qlora_linear* L) {
  if (!L) return QLORA_ERR_INVALID_ARG;
  int st = check_nf4(&L->W0);
  if (st) return st;
  if (!L->A || !L->B) return QLORA_ERR_INVALID_ARG;
  if (!isfinite(L->alpha)) return QLORA_ERR_INVALID_ARG;
  if (L->r < 1 || L->r > 128) return QLORA_ERR_UNSUPPORTED_SHAPE;
  if (!aligned16(L->A) || !aligned16(L->B)) return QLORA_ERR_MISALIGNED;
  return QLORA_OK;
}

int check_ptr(const void* p) {
  if (!p) return QLORA_ERR_INVALID_ARG;
  if (!aligned16(p)) return QLORA_ERR_MISALIGNED;
  return QLORA_OK;
}

int check_ws(const void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return QLORA_OK;
  if (ws_bytes < need) return QLORA_ERR_WORKSPACE_TOO_SMALL;
  return check_ptr(ws);
}

}  // namespace

int qv_quantize(const float* W, int64_t N, int64_t K, const float* codebook16, int32_t blocksize, int32_t dq_group,
                const uint8_t* codes, const float* absmax, const uint8_t* absmax_q, const float* absmax_scale) {
  if (N < 0 || K < 0) return QLORA_ERR_INVALID_ARG;
  if (blocksize != 64) return QLORA_ERR_UNSUPPORTED_SHAPE;
  if (dq_group != 0 && dq_group != 256) return QLORA_ERR_UNSUPPORTED_SHAPE;
  if (K % 64 != 0) return QLORA_ERR_UNSUPPORTED_SHAPE;
  if (N == 0 || K == 0) return QLORA_OK;
  if (!W || !codebook16 || !codes) return QLORA_ERR_INVALID_ARG;
  if (dq_group == 0 && !absmax) return QLORA_ERR_INVALID_ARG;
  if (dq_group != 0 && (!absmax_q || !absmax_scale)) return QLORA_ERR_INVALID_ARG;
  if (!aligned16(W) || !aligned16(codebook16) || !aligned16(codes)) return QLORA_ERR_MISALIGNED;
  if (dq_group == 0 && !aligned16(absmax)) return QLORA_ERR_MISALIGNED;
  if (dq_group != 0 && !aligned16(absmax_scale)) return QLORA_ERR_MISALIGNED;
  return QLORA_OK;
}

int qv_dequantize(const qlora_nf4* w, int32_t out_dtype, const void* out) {
  int st = check_nf4(w);
  if (st) return st;
  if (out_dtype != QLORA_DTYPE_BF16 && out_dtype != QLORA_DTYPE_F32) return QLORA_ERR_INVALID_ARG;
  return check_ptr(out);
}

int qv_grouped(const qlora_grouped* Q) {
  if (!Q) return QLORA_ERR_INVALID_ARG;
  int st = check_nf4(&Q->W0);
  if (st) return st;
  if (Q->G < 1 || Q->G > 8) return QLORA_ERR_UNSUPPORTED_SHAPE;
  if (!Q->A) return QLORA_ERR_INVALID_ARG;
  if (!aligned16(Q->A)) return QLORA_ERR_MISALIGNED;
  int64_t nsum = 0, rsum = 0;
  for (int g = 0; g < Q->G; ++g) {
    if (!Q->B[g]) return QLORA_ERR_INVALID_ARG;
    if (!aligned16(Q->B[g])) return QLORA_ERR_MISALIGNED;
    if (!isfinite(Q->alpha[g])) return QLORA_ERR_INVALID_ARG;
    if (Q->N[g] < 1 || Q->r[g] < 1) return QLORA_ERR_UNSUPPORTED_SHAPE;
    nsum += Q->N[g];
    rsum += Q->r[g];
  }
  if (nsum != Q->W0.N || rsum > 128) return QLORA_ERR_UNSUPPORTED_SHAPE;
  return QLORA_OK;
}

int qv_grouped_dB(const qlora_grouped* Q, void* const* dB) {
  if (!dB) return QLORA_ERR_INVALID_ARG;
  for (int g = 0; g < Q->G; ++g) {
    const int st = check_ptr(dB[g]);
    if (st) return st;
  }
  return QLORA_OK;
}

static int check_rms(int64_t M, int64_t D) {
  if (M < 0) return QLORA_ERR_INVALID_ARG;
  if (M > kMaxTokens) return QLORA_ERR_UNSUPPORTED_SHAPE;
  if (D < 8 || D > 8192 || D % 8 != 0) return QLORA_ERR_UNSUPPORTED_SHAPE;
  return QLORA_OK;
}

size_t qv_rmsnorm_ws(int64_t M, int64_t D) {
  if (check_rms(M, D) || M == 0) return 0;
  const int64_t g = (M + 3) / 4;
  return (size_t)(g < 256 ? g : 256) * (size_t)D * 4;
}

int qv_rmsnorm_fwd(const void* X, const void* w, int64_t M, int64_t D, float eps, const void* Y, const float* rstd) {
  int st = check_rms(M, D);
  if (st) return st;
  if (!isfinite(eps) || eps < 0.0f) return QLORA_ERR_INVALID_ARG;
  if (M == 0) return QLORA_OK;
  if ((st = check_ptr(X)) || (st = check_ptr(w)) || (st = check_ptr(Y)) || (st = check_ptr(rstd))) return st;
  return QLORA_OK;
}

int qv_rmsnorm_bwd(const void* dY, const void* X, const void* w, const float* rstd, int64_t M, int64_t D,
                   const void* dX, const float* dw, const void* ws, size_t ws_bytes) {
  int st = check_rms(M, D);
  if (st) return st;
  if (dw && (st = check_ptr(dw))) return st;
  if (M == 0) return QLORA_OK;
  if ((st = check_ptr(dY)) || (st = check_ptr(X)) || (st = check_ptr(w)) || (st = check_ptr(rstd)) ||
      (st = check_ptr(dX)))
    return st;
  return dw ? check_ws(ws, ws_bytes, qv_rmsnorm_ws(M, D)) : QLORA_OK;
}

int qv_merge(const qlora_linear* L, int32_t out_dtype, const void* out) {
  int st = check_linear(L);
  if (st) return st;
  if (out_dtype != QLORA_DTYPE_BF16 && out_dtype != QLORA_DTYPE_F16) return QLORA_ERR_INVALID_ARG;
  return check_ptr(out);
}

int qv_linear_fwd(const qlora_linear* L, const void* X, int64_t M, const void* Y, const float* XA, const void* ws,
                  size_t ws_bytes) {
  int st = check_linear(L);
  if (st) return st;
  if (M < 0) return QLORA_ERR_INVALID_ARG;
  if (M > kMaxTokens) return QLORA_ERR_UNSUPPORTED_SHAPE;
  if (M == 0) return QLORA_OK;
  if ((st = check_ptr(X)) || (st = check_ptr(Y)) || (st = check_ptr(XA))) return st;
  const qplan::LinearWs w = qplan::linear_ws(M, L->W0.N, L->W0.K, L->r);
  return check_ws(ws, ws_bytes, w.fwd_total);
}

int qv_linear_fwd_static(const qlora_linear* L, const void* X, int64_t M, const void* Y, const float* XA,
                         size_t scratch_bytes) {
  int st = check_linear(L);
  if (st) return st;
  if (M < 0) return QLORA_ERR_INVALID_ARG;
  if (M > kMaxTokens) return QLORA_ERR_UNSUPPORTED_SHAPE;
  if (M == 0) return QLORA_OK;
  if ((st = check_ptr(X)) || (st = check_ptr(Y)) || (st = check_ptr(XA))) return st;
  const qplan::LinearWs w = qplan::linear_ws(M, L->W0.N, L->W0.K, L->r);
  return w.fwd_total > scratch_bytes ? QLORA_ERR_WORKSPACE_TOO_SMALL : QLORA_OK;
}

int qv_linear_bwd(const qlora_linear* L, const void* dY, const void* X, const float* XA, int64_t M, const void* dX,
                  const void* dA, const void* dB, const void* ws, size_t ws_bytes) {
  int st = check_linear(L);
  if (st) return st;
  if (M < 0) return QLORA_ERR_INVALID_ARG;
  if (M > kMaxTokens) return QLORA_ERR_UNSUPPORTED_SHAPE;
  if ((st = check_ptr(dA)) || (st = check_ptr(dB))) return st;
  if (M == 0) return QLORA_OK;
  if ((st = check_ptr(dY)) || (st = check_ptr(X)) || (st = check_ptr(XA)) || (st = check_ptr(dX))) return st;
  const qplan::LinearWs w = qplan::linear_ws(M, L->W0.N, L->W0.K, L->r);
  return check_ws(ws, ws_bytes, w.bwd_total);
}

static int check_mlp(const qlora_mlp* P) {
  if (!P) return QLORA_ERR_INVALID_ARG;
  int st;
  if ((st = check_linear(&P->gate)) || (st = check_linear(&P->up)) || (st = check_linear(&P->down))) return st;
  const int64_t I = P->gate.W0.N, D = P->gate.W0.K;
  if (P->up.W0.N != I || P->up.W0.K != D) return QLORA_ERR_UNSUPPORTED_SHAPE;
  if (P->down.W0.N != D || P->down.W0.K != I) return QLORA_ERR_UNSUPPORTED_SHAPE;
  if (P->gate.W0.dq_group != P->up.W0.dq_group) return QLORA_ERR_UNSUPPORTED_SHAPE;
  if (I > kMaxMlpI) return QLORA_ERR_UNSUPPORTED_SHAPE;
  return QLORA_OK;
}

int qv_mlp_fwd(const qlora_mlp* P, const void* X, int64_t M, const void* Y, const qlora_mlp_saved* S, const void* ws,
               size_t ws_bytes) {
  int st = check_mlp(P);
  if (st) return st;
  if (M < 0 || !S) return QLORA_ERR_INVALID_ARG;
  if (M > kMaxTokens) return QLORA_ERR_UNSUPPORTED_SHAPE;
  if (M == 0) return QLORA_OK;
  if ((st = check_ptr(X)) || (st = check_ptr(Y)) || (st = check_ptr(S->G)) || (st = check_ptr(S->U)) ||
      (st = check_ptr(S->XA_g)) || (st = check_ptr(S->XA_u)) || (st = check_ptr(S->HA_d)))
    return st;
  const qplan::MlpWs w = qplan::mlp_ws(M, P->gate.W0.K, P->gate.W0.N, P->gate.r, P->up.r, P->down.r);
  return check_ws(ws, ws_bytes, w.fwd_total);
}

int qv_mlp_fwd_rmsnorm(const qlora_mlp* P, const void* X, const void* norm_w, float eps, int64_t M, const void* Y,
                       const qlora_mlp_saved* S, const float* rstd, const void* Xn, const void* ws, size_t ws_bytes) {
  int st = check_mlp(P);
  if (st) return st;
  if (M < 0 || !S) return QLORA_ERR_INVALID_ARG;
  if (M > kMaxTokens) return QLORA_ERR_UNSUPPORTED_SHAPE;
  if ((st = check_rms(M, P->gate.W0.K))) return st;
  if (!isfinite(eps) || eps < 0.0f) return QLORA_ERR_INVALID_ARG;
  if (M == 0) return QLORA_OK;
  if ((st = check_ptr(X)) || (st = check_ptr(norm_w)) || (st = check_ptr(Y)) || (st = check_ptr(rstd)) ||
      (st = check_ptr(S->G)) || (st = check_ptr(S->U)) || (st = check_ptr(S->XA_g)) || (st = check_ptr(S->XA_u)) ||
      (st = check_ptr(S->HA_d)))
    return st;
  if (Xn && (st = check_ptr(Xn))) return st;
  const qplan::MlpRmsWs w =
      qplan::mlp_rms_ws(M, P->gate.W0.K, P->gate.W0.N, P->gate.r, P->up.r, P->down.r);
  return check_ws(ws, ws_bytes, w.total);
}

int qv_mlp_bwd(const qlora_mlp* P, const void* dY, const void* X, const qlora_mlp_saved* S, int64_t M, const void* dX,
               const qlora_mlp_grads* G, const void* ws, size_t ws_bytes) {
  int st = check_mlp(P);
  if (st) return st;
  if (M < 0 || !S || !G) return QLORA_ERR_INVALID_ARG;
  if (M > kMaxTokens) return QLORA_ERR_UNSUPPORTED_SHAPE;
  if ((st = check_ptr(G->dA_g)) || (st = check_ptr(G->dB_g)) || (st = check_ptr(G->dA_u)) ||
      (st = check_ptr(G->dB_u)) || (st = check_ptr(G->dA_d)) || (st = check_ptr(G->dB_d)))
    return st;
  if (M == 0) return QLORA_OK;
  if ((st = check_ptr(dY)) || (st = check_ptr(X)) || (st = check_ptr(dX)) || (st = check_ptr(S->G)) ||
      (st = check_ptr(S->U)) || (st = check_ptr(S->XA_g)) || (st = check_ptr(S->XA_u)) || (st = check_ptr(S->HA_d)))
    return st;
  const qplan::MlpWs w = qplan::mlp_ws(M, P->gate.W0.K, P->gate.W0.N, P->gate.r, P->up.r, P->down.r);
  return check_ws(ws, ws_bytes, w.bwd_total);
}

extern "C" {

uint32_t qlora_abi_version(void) { return QLORA_ABI_VERSION; }

const char* qlora_strerror(int status) {
  switch (status) {
    case QLORA_OK: return "ok";
    case QLORA_ERR_INVALID_ARG: return "invalid argument";
    case QLORA_ERR_UNSUPPORTED_SHAPE: return "unsupported shape";
    case QLORA_ERR_MISALIGNED: return "tensor pointer not 16-byte aligned";
    case QLORA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case QLORA_ERR_UNSUPPORTED_DEVICE: return "unsupported device (needs gfx950)";
    case QLORA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

size_t qlora_linear_workspace_bytes(const qlora_linear* L, int64_t M) {
  if (!L || M <= 0 || M > kMaxTokens || check_linear(L)) return 0;
  return qplan::linear_ws(M, L->W0.N, L->W0.K, L->r).total;
}

size_t qlora_mlp_workspace_bytes(const qlora_mlp* P, int64_t M) {
  if (!P || M <= 0 || M > kMaxTokens || check_mlp(P)) return 0;
  return qplan::mlp_ws(M, P->gate.W0.K, P->gate.W0.N, P->gate.r, P->up.r, P->down.r).total;
}

size_t qlora_mlp_rmsnorm_workspace_bytes(const qlora_mlp* P, int64_t M) {
  if (!P || M <= 0 || M > kMaxTokens || check_mlp(P) || check_rms(M, P->gate.W0.K)) return 0;
  return qplan::mlp_rms_ws(M, P->gate.W0.K, P->gate.W0.N, P->gate.r, P->up.r, P->down.r).total;
}

}  // extern "C"

size_t qv_linear_ce_ws(int64_t T, int64_t D, int64_t V, int64_t chunk, int32_t want_dx) {
  if (T < 0 || T > kMaxTokens || D <= 0 || V <= 0 || chunk < 1 || D % 64 != 0 || V % 64 != 0) return 0;
  if (D > 65536 || V > kMaxMlpI) return 0;
  return qplan::ce_ws(T, D, V, chunk, want_dx != 0).total;
}

int qv_linear_ce(const void* X, int64_t T, int64_t D, const void* W, int64_t V, const int32_t* targets,
                 int64_t chunk, const float* loss, const float* token_loss, const void* dX, const void* ws,
                 size_t ws_bytes) {
  if (T < 0 || D <= 0 || V <= 0 || chunk < 1) return QLORA_ERR_INVALID_ARG;
  // the logit gradient is read as bf16 rows of stride 2V: a 256-row tile of
  // it stays below 2 GiB for V <= 2097088
  if (D % 64 != 0 || V % 64 != 0 || D > 65536 || V > kMaxMlpI || T > kMaxTokens) return QLORA_ERR_UNSUPPORTED_SHAPE;
  int st;
  if ((st = check_ptr(loss))) return st;
  if (token_loss && (st = check_ptr(token_loss))) return st;
  if (T == 0) return QLORA_OK;
  if ((st = check_ptr(X)) || (st = check_ptr(W)) || (st = check_ptr(targets))) return st;
  if (dX && (st = check_ptr(dX))) return st;
  return check_ws(ws, ws_bytes, qplan::ce_ws(T, D, V, chunk, dX != nullptr).total);
}
