/*
 * qlora.h - C ABI of the MI355X (gfx950) QLoRA linear / SwiGLU-MLP library.
 *
 * The layer: a frozen base weight W0 [N, K] stored as 4-bit NormalFloat
 * (NF4) codes with per-block absmax scales, plus a trainable LoRA pair
 * A [r, K], B [N, r] ("LLM Fine-Tuning in 2026: Unsloth vs QLoRA vs
 * Liger-Kernel", section 1: h = W0 x + (alpha/r) B A x; FAQ: QLoRA keeps the
 * base weight in 4-bit NormalFloat).  No dropout and no bias (section 5's
 * adapter settings), so the ABI has neither.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tokens are rows.  All matrices are row-major and contiguous.
 *   bf16 tensors are passed as pointers to 16-bit bf16 bit patterns.
 * - Every pointer argument that names a tensor is a DEVICE pointer (memory
 *   of the current HIP device), except where stated.  The caller owns all
 *   memory, including workspaces; the library never allocates, frees or
 *   synchronises.  It keeps no state between calls and is re-entrant.
 * - `stream` is a hipStream_t (NULL = the default stream).  All work is
 *   enqueued on it in order; a call returns once the work is enqueued.
 * - bf16 and fp32 tensor pointers must be 16-byte aligned.
 * - Arguments are validated before anything is enqueued; a failed check
 *   returns a negative status and enqueues nothing.  Device-side faults
 *   surface on a later synchronisation and map to QLORA_ERR_HIP when a
 *   launch itself reports an error.
 * - Gradients are written (overwritten), never accumulated.
 * - M (tokens) may be any value in [0, 2^31 - 1] (QLORA_ERR_INVALID_ARG
 *   below, QLORA_ERR_UNSUPPORTED_SHAPE above); M == 0 is a no-op that
 *   returns OK.  The *_workspace_bytes queries return 0 for arguments the
 *   matching call would reject.
 * - Shapes: K % 64 == 0 and N % 64 == 0 (whole absmax blocks, whole tiles
 *   of 64), K, N <= 4194240 (a 256-row tile of a bf16 copy stays below
 *   2 GiB), 1 <= r <= 128, blocksize == 64, dq_group in {0, 256}.
 */
#ifndef QLORA_H
#define QLORA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QLORA_ABI_VERSION 1u

/* Status codes. */
#define QLORA_OK 0
#define QLORA_ERR_INVALID_ARG (-1)         /* null pointer, negative size, bad enum, non-finite alpha */
#define QLORA_ERR_UNSUPPORTED_SHAPE (-2)   /* K or N not a multiple of 64, r out of [1,128], ... */
#define QLORA_ERR_MISALIGNED (-3)          /* a tensor pointer not 16-byte aligned */
#define QLORA_ERR_WORKSPACE_TOO_SMALL (-4) /* ws_bytes below the matching *_workspace_bytes() */
#define QLORA_ERR_UNSUPPORTED_DEVICE (-5)  /* current device is not gfx950 */
#define QLORA_ERR_HIP (-6)                 /* a HIP runtime call or launch failed */

/* Output element types of nf4_dequantize (BF16, F32) and qlora_merge (BF16, F16). */
#define QLORA_DTYPE_BF16 0
#define QLORA_DTYPE_F32 1
#define QLORA_DTYPE_F16 2

/*
 * An NF4-quantized frozen weight W0 [N, K] (QLoRA base weight; the pages name
 * the format, its parameters are fixed here).
 *
 *   codes        u8 [N*K/2]: element e = n*K + k of the row-major weight has
 *                its 4-bit code in byte e/2, bits 0-3 for even e, bits 4-7
 *                for odd e.
 *   blocksize    64: absmax block b covers elements [64b, 64b+64), i.e. 64
 *                consecutive elements of one row.
 *   dq_group 0   absmax       fp32 [N*K/64]: max |w| of each block.
 *   dq_group 256 absmax_q     u8   [N*K/64]: 8-bit linear code of each absmax,
 *                absmax_scale fp32 [ceil(N*K/64/256)]: one scale S per group
 *                of 256 consecutive blocks; absmax' = fp32(code8 * S).
 *   codebook     fp32 [16], device memory: strictly increasing, -1 and +1 at
 *                the ends, exactly one 0.0 entry.
 *
 * Element value: fp32(codebook[code] * absmax'), absmax' = absmax when
 * dq_group == 0.  Unused pointers (absmax or absmax_q/absmax_scale) may be
 * NULL.
 */
typedef struct qlora_nf4 {
  const uint8_t* codes;
  const float* absmax;
  const uint8_t* absmax_q;
  const float* absmax_scale;
  const float* codebook;
  int64_t N;
  int64_t K;
  int32_t blocksize;
  int32_t dq_group;
} qlora_nf4;

/*
 * One QLoRA linear layer: Y = X W0^T + s (X A^T) B^T with s = alpha / r
 * computed in fp32.  A bf16 [r, K], B bf16 [N, r] (orientation of B A x in
 * "LLM Fine-Tuning in 2026", section 1).  W0.N, W0.K give N and K.
 */
typedef struct qlora_linear {
  qlora_nf4 W0;
  const void* A;
  const void* B;
  int32_t r;
  float alpha;
} qlora_linear;

/*
 * SwiGLU MLP block of three QLoRA linears: gate and up map D -> I, down maps
 * I -> D.  Y = down(silu(gate(X)) * up(X)), silu(g) = g / (1 + e^-g)
 * ("MLP SwiGLU" among the hand-derived kernels, "LLM Fine-Tuning in 2026",
 * section 2).  gate and up must have the same dq_group
 * (QLORA_ERR_UNSUPPORTED_SHAPE otherwise); r, alpha and the codebook buffer
 * may differ per layer.  I <= 2097088 (the backward holds [W_g^T | W_u^T]
 * as one bf16 copy of row stride 2I; QLORA_ERR_UNSUPPORTED_SHAPE otherwise).
 */
typedef struct qlora_mlp {
  qlora_linear gate;
  qlora_linear up;
  qlora_linear down;
} qlora_mlp;

/*
 * What the MLP forward saves for the backward.  Only the gate and up
 * pre-activations are kept; sigma(G), silu(G) and H = silu(G) * U are
 * recomputed in the backward ("What is Unsloth", "Recompute instead of store").
 *   G, U   bf16 [M, I]   gate / up outputs
 *   XA_g   fp32 [M, r_g] X A_g^T      XA_u  fp32 [M, r_u] X A_u^T
 *   HA_d   fp32 [M, r_d] H A_d^T
 */
typedef struct qlora_mlp_saved {
  void* G;
  void* U;
  float* XA_g;
  float* XA_u;
  float* HA_d;
} qlora_mlp_saved;

/* LoRA gradients of the MLP, bf16, shapes of the matching A / B. */
typedef struct qlora_mlp_grads {
  void* dA_g;
  void* dB_g;
  void* dA_u;
  void* dB_u;
  void* dA_d;
  void* dB_d;
} qlora_mlp_grads;

/* ABI version of the loaded library (QLORA_ABI_VERSION it was built with). */
uint32_t qlora_abi_version(void);

/* Static message for a status code; never NULL. */
const char* qlora_strerror(int status);

/*
 * nf4_quantize: blockwise-absmax NF4 quantization of W [N, K] fp32.
 *
 * Per block of 64: a = max |w|; if a == 0 every code is the index of the
 * codebook's 0.0; otherwise q = the nearest codebook entry to the correctly
 * rounded fp32 quotient w / a, ties to the lower index.  With dq_group == 256
 * the absmax vector is then quantized in groups of 256 blocks (last group may
 * be shorter): S = fp32(max / 255), code8 = min(255, round_half_even(fp32(a/S)))
 * (0 if S == 0).  The 4-bit codes always use the exact absmax.
 *
 *   W            fp32 [N, K] device, input (finite values; others are
 *                memory-safe but give unspecified codes)
 *   codebook16   fp32 [16] device
 *   blocksize    must be 64
 *   dq_group     0 or 256
 *   codes        u8 [N*K/2] device, output
 *   absmax       fp32 [N*K/64] device, output when dq_group == 0 (else unused)
 *   absmax_q     u8 [N*K/64] device, output when dq_group == 256
 *   absmax_scale fp32 [ceil(N*K/64/256)] device, output when dq_group == 256
 * Needs no workspace.  N == 0 is a no-op.
 */
int nf4_quantize(const float* W, int64_t N, int64_t K, const float* codebook16,
                 int32_t blocksize, int32_t dq_group, uint8_t* codes, float* absmax,
                 uint8_t* absmax_q, float* absmax_scale, void* stream);

/*
 * nf4_dequantize: writes every element fp32(codebook[q] * absmax') of w as
 * out_dtype QLORA_DTYPE_BF16 (round to nearest even) or QLORA_DTYPE_F32,
 * into out [N, K] (device).  Bit-exact with the definition above.
 */
int nf4_dequantize(const qlora_nf4* w, int32_t out_dtype, void* out, void* stream);

/*
 * qlora_merge: the adapted layer as one 16-bit weight, for export after
 * training ("LLM Fine-Tuning in 2026", the listing's 16-bit merge save step;
 * the update h = W0 x + (alpha/r) B A x of section 1 folded into the weight):
 *
 *   out[n, k] = round16( fp32(codebook[q] * absmax')[n, k] + s * (B A)[n, k] ),
 *   evaluated in fp32 (the scaled product may be fused into the add):
 *   s = alpha / r in fp32, (B A)[n, k] = sum_j B[n, j] A[j, k] with exact
 *   products of the bf16 values accumulated in fp32; round16 = round to
 *   nearest even into out_dtype QLORA_DTYPE_BF16 or QLORA_DTYPE_F16 (fp16
 *   overflow gives +-inf).
 *
 *   L    the layer (W0, A, B, r, alpha as for qlora_linear_fwd)
 *   out  16-bit [N, K] device output, 16-byte aligned
 * With B == 0 the result equals nf4_dequantize(W0, QLORA_DTYPE_BF16) bit for
 * bit.  Needs no workspace; N == 0 is a no-op.  Errors as for the other entry
 * points (QLORA_ERR_INVALID_ARG for another out_dtype).
 */
int qlora_merge(const qlora_linear* L, int32_t out_dtype, void* out, void* stream);

/*
 * Several LoRA adapters over one input, packed into one layer ("Speed Up
 * Fine-Tuning 2x with Unsloth", item 3 "Memory Management": multiple LoRA
 * adapters packed into a single tensor; the q/k/v projections of attention
 * are the typical group).  Group g (g < G <= 8) is the QLoRA linear
 * Y_g = X W_g^T + s_g (X A_g^T) B_g^T with s_g = alpha[g] / r[g]; the groups
 * share X [M, K] and are stored packed:
 *
 *   W0   the NF4 weight of the row-concatenation [W_0; W_1; ...] [N_total, K]
 *        (N_total = sum N[g], a multiple of 64)
 *   A    bf16 [r_total, K], the A_g stacked (r_total = sum r[g] <= 128)
 *   B[g] bf16 [N[g], r[g]], one tensor per group
 *
 * Y, dY are [M, N_total] with group g in columns [sum_{h<g} N[h], +N[g]).
 * XA_saved is [M, r_total] fp32 (X A^T of the stacked A); dA is [r_total, K]
 * (the dA_g stacked); dB[g] is bf16 [N[g], r[g]].  Internally the groups run
 * as one layer with a block-diagonal B whose blocks are s_g B_g (rounded to
 * bf16) and s = 1, so each output is within the tolerance of the separate
 * layers (exactly them when every s_g is a power of two).
 */
typedef struct qlora_grouped {
  qlora_nf4 W0;
  const void* A;
  const void* B[8];
  int32_t N[8];
  int32_t r[8];
  float alpha[8];
  int32_t G;
} qlora_grouped;

size_t qlora_grouped_workspace_bytes(const qlora_grouped* Q, int64_t M);

/* qlora_grouped_fwd / _bwd: as qlora_linear_fwd / _bwd for the packed groups
 * (arguments as in the comment above; same errors, plus
 * QLORA_ERR_UNSUPPORTED_SHAPE for G outside [1, 8], an N[g] < 1, a sum of N
 * other than W0.N, or r_total outside [1, 128]). */
int qlora_grouped_fwd(const qlora_grouped* Q, const void* X, int64_t M, void* Y, float* XA_saved, void* ws,
                      size_t ws_bytes, void* stream);
int qlora_grouped_bwd(const qlora_grouped* Q, const void* dY, const void* X, const float* XA_saved, int64_t M,
                      void* dX, void* dA, void* const* dB, void* ws, size_t ws_bytes, void* stream);

/*
 * rmsnorm_fwd: the RMSNorm in front of the MLP block ("LLM Fine-Tuning in
 * 2026", the fused RMSNorm of section 2: the forward keeps one inverse RMS per
 * row for the backward and no full-size intermediate).  Per row m of X:
 *
 *   rstd[m] = 1 / sqrt(mean_j X[m, j]^2 + eps),  Y[m, j] = X[m, j] rstd[m] w[j]
 *
 * fp32 arithmetic, Y rounded to bf16 (nearest even).
 *   X     bf16 [M, D] input          w     bf16 [D] input
 *   Y     bf16 [M, D] output         rstd  fp32 [M] output, kept for rmsnorm_bwd
 *   D % 8 == 0 and 8 <= D <= 8192 (QLORA_ERR_UNSUPPORTED_SHAPE otherwise);
 *   eps finite and >= 0 (QLORA_ERR_INVALID_ARG otherwise; with eps == 0 an
 *   all-zero row gives non-finite values).  Needs no workspace; M == 0 is a
 *   no-op.  All pointers 16-byte aligned.
 */
int rmsnorm_fwd(const void* X, const void* w, int64_t M, int64_t D, float eps, void* Y, float* rstd,
                void* stream);

/* Workspace bytes rmsnorm_bwd needs with dw requested (0 without dw). */
size_t rmsnorm_bwd_workspace_bytes(int64_t M, int64_t D);

/*
 * rmsnorm_bwd: gradients of <Y, dY> for rmsnorm_fwd, derived by hand.  With
 * g = dY[m] * w (elementwise):
 *
 *   dX[m] = rstd[m] g - rstd[m]^3 / D (sum_j g_j X[m, j]) X[m]     (bf16 out)
 *   dw    = sum_m dY[m] X[m] rstd[m]                                (fp32 out)
 *
 * fp32 arithmetic; dw is summed in a fixed order (bitwise reproducible) and is
 * optional: dw == NULL skips it, and then ws may be NULL.
 *   dY, X bf16 [M, D]; w bf16 [D]; rstd fp32 [M] from rmsnorm_fwd; dX bf16
 *   [M, D] output; ws of ws_bytes >= rmsnorm_bwd_workspace_bytes(M, D).
 * Shapes and errors as for rmsnorm_fwd.  M == 0 writes dw = 0.
 */
int rmsnorm_bwd(const void* dY, const void* X, const void* w, const float* rstd, int64_t M, int64_t D,
                void* dX, float* dw, void* ws, size_t ws_bytes, void* stream);

/*
 * Workspace bytes qlora_linear_ce needs for T tokens, hidden size D, V classes
 * and the given chunk (0 when the shape is not supported): one chunk of
 * logits (min(chunk, T) * V fp32), T per-token fp32 losses and, with
 * want_dx != 0, the fp32 partials of the dX product (which reads the head as
 * stored: no copy of it).
 */
size_t qlora_linear_ce_workspace_bytes(int64_t T, int64_t D, int64_t V, int64_t chunk, int32_t want_dx);

/*
 * qlora_linear_ce: the output head's linear projection and the cross-entropy
 * loss in one call ("LLM Fine-Tuning in 2026", section 3, the fused
 * cross-entropy), token chunk by token chunk, so that no [T, V] logit matrix
 * is held: the only [*, V] buffer is one chunk of logits in the workspace.
 * With n the number of tokens whose target is a class index in [0, V) other
 * than ignore_index (any other value marks a token without a target):
 *
 *   z_t   = W x_t                  V logits, fp32 accumulation, kept in fp32
 *   l_t   = logsumexp(z_t) - z_t[target_t]     (fp32; 0 without a target)
 *   loss  = (1/n) sum_t l_t                     (fixed-order sum; 0 if n == 0)
 *   dX_t  = sum_v g_tv W_v,  g_tv = bf16((softmax(z_t)_v - [v == target_t]) / n)
 *           (fp32 accumulation, bf16 out; 0 rows without a target)
 *
 *   X          bf16 [T, D]  hidden states
 *   W          bf16 [V, D]  frozen head, row v = class v
 *   targets    int32 [T]    device
 *   loss       fp32 [1]     output (device)
 *   token_loss fp32 [T]     output l_t, or NULL
 *   dX         bf16 [T, D]  output, or NULL for the loss alone
 *   chunk      tokens per chunk, >= 1 (QLORA_ERR_INVALID_ARG otherwise)
 *   ws         ws_bytes >= qlora_linear_ce_workspace_bytes(T, D, V, chunk,
 *              dX != NULL); with dX the head is transposed into it once per
 *              call (V * D * 2 bytes)
 * D and V multiples of 64, D <= 65536, V <= 2097088
 * (QLORA_ERR_UNSUPPORTED_SHAPE otherwise).  T == 0 writes loss = 0 and needs
 * no workspace.  All pointers 16-byte aligned.  Results are bitwise
 * reproducible from run to run.
 */
int qlora_linear_ce(const void* X, int64_t T, int64_t D, const void* W, int64_t V, const int32_t* targets,
                    int32_t ignore_index, int64_t chunk, float* loss, float* token_loss, void* dX, void* ws,
                    size_t ws_bytes, void* stream);

/*
 * Workspace bytes the linear forward and backward need for M tokens.  From
 * M = 512 tokens on, the GEMMs expand the NF4 weight once per call into a
 * bf16 copy held in the workspace (N*K*2 bytes) instead of expanding it in
 * every 256-token tile; below that the expansion happens inside the GEMM.
 */
size_t qlora_linear_workspace_bytes(const qlora_linear* L, int64_t M);

/*
 * qlora_linear_fwd: Y = X W0^T + s XA B^T, XA = X A^T.
 *   X        bf16 [M, K] input
 *   Y        bf16 [M, N] output
 *   XA_saved fp32 [M, r] output, kept by the caller for qlora_linear_bwd
 *   ws       device workspace of ws_bytes >= qlora_linear_workspace_bytes(L, M)
 * fp32 accumulation throughout; the dequantized weight enters the matrix
 * cores as bf16(fp32(codebook[q] * absmax')).
 */
int qlora_linear_fwd(const qlora_linear* L, const void* X, int64_t M, void* Y,
                     float* XA_saved, void* ws, size_t ws_bytes, void* stream);

/*
 * qlora_linear_fwd_static: qlora_linear_fwd for callers that cannot allocate
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments and results as qlora_linear_fwd, but no
 * workspace: the pass's scratch (split partials, down-projection partials,
 * the bf16 weight copy from 512 tokens on) lives in a library-owned device
 * array of QLORA_STATIC_SCRATCH_BYTES per GPU, which that GPU holds from the
 * first call on it until the process ends.  The first call on a GPU looks up
 * the array's device address; no call allocates or frees memory.
 *   A pass that needs more scratch than that (qlora_linear_workspace_bytes
 *   larger than QLORA_STATIC_SCRATCH_BYTES for the forward's share, e.g. a
 *   bf16 copy of an 8192 x 8192 weight) returns QLORA_ERR_WORKSPACE_TOO_SMALL
 *   and enqueues nothing.
 * Every call on one GPU uses that GPU's one array and leaves the last call's
 * contents there: calls that overlap on one GPU (several streams or host
 * threads) race and must be ordered by the caller.  Nothing in the array
 * needs to start at zero.  Other errors as for qlora_linear_fwd.
 */
#define QLORA_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
int qlora_linear_fwd_static(const qlora_linear* L, const void* X, int64_t M, void* Y, float* XA_saved,
                            void* stream);

/*
 * qlora_linear_bwd: gradients of <Y, dY> ("LLM Fine-Tuning in 2026",
 * section 2: analytic gradients instead of autograd; W0 is frozen).
 *   T  = dY B                      (fp32, in the workspace)
 *   dX = dY W0 + s T A             bf16 [M, K] output
 *   dA = s T^T X                   bf16 [r, K] output
 *   dB = s dY^T XA_saved           bf16 [N, r] output
 *   dY bf16 [M, N], X bf16 [M, K], XA_saved fp32 [M, r]: inputs.
 * The reductions over M run in a fixed order, so results are bitwise
 * reproducible from run to run.  With M == 0, dA and dB are set to zero.
 */
int qlora_linear_bwd(const qlora_linear* L, const void* dY, const void* X,
                     const float* XA_saved, int64_t M, void* dX, void* dA, void* dB,
                     void* ws, size_t ws_bytes, void* stream);

/*
 * Workspace bytes the MLP forward and backward need for M tokens (with
 * M >= 512 this includes a bf16 copy of the expanded weights of one GEMM,
 * up to 2*I*D*2 bytes, as for the linear layer).
 */
size_t qlora_mlp_workspace_bytes(const qlora_mlp* P, int64_t M);

/*
 * qlora_mlp_fwd: G = gate(X), U = up(X), H = silu(G) * U (transient, in the
 * workspace), Y = down(H).
 *   X bf16 [M, D] input;  Y bf16 [M, D] output;  S: saved tensors (outputs).
 */
int qlora_mlp_fwd(const qlora_mlp* P, const void* X, int64_t M, void* Y,
                  const qlora_mlp_saved* S, void* ws, size_t ws_bytes, void* stream);

/* Workspace bytes qlora_mlp_fwd_rmsnorm needs (0 for a rejected shape). */
size_t qlora_mlp_rmsnorm_workspace_bytes(const qlora_mlp* P, int64_t M);

/*
 * qlora_mlp_fwd_rmsnorm: the RMSNorm in front of the block fused into its
 * forward ("LLM Fine-Tuning in 2026: Unsloth vs QLoRA vs Liger-Kernel",
 * section 2, the fused RMSNorm): the results of rmsnorm_fwd(X, norm_w, eps)
 * -> (Xn, rstd) followed by qlora_mlp_fwd(P, Xn, ...), without Xn between
 * them.  From 512 tokens the norm weight is folded into the expanded gate/up
 * weights (column k times norm_w[k]), the inverse RMS of each token scales
 * the gate/up product, and XA_g, XA_u are rstd * X (A w)^T; below 512 the
 * norm runs as its own pass.  Roundings differ from the two-call path only
 * inside the bf16 operands (bf16(W w) instead of bf16(X rstd w)).
 *   X      bf16 [M, D] pre-norm input     norm_w bf16 [D]    eps as rmsnorm_fwd
 *   Y, S   as qlora_mlp_fwd (S->XA_g, S->XA_u are those of the normalised input)
 *   rstd   fp32 [M] output (for rmsnorm_bwd)
 *   Xn     bf16 [M, D] output, or NULL: the normalised input is written only
 *          when Xn is given (qlora_mlp_bwd takes it as its X)
 *   ws     ws_bytes >= qlora_mlp_rmsnorm_workspace_bytes(P, M)
 * Errors: those of qlora_mlp_fwd and of rmsnorm_fwd for D = the block's
 * hidden size.  M == 0 is a no-op.
 */
int qlora_mlp_fwd_rmsnorm(const qlora_mlp* P, const void* X, const void* norm_w, float eps, int64_t M, void* Y,
                          const qlora_mlp_saved* S, float* rstd, void* Xn, void* ws, size_t ws_bytes,
                          void* stream);

/*
 * qlora_mlp_bwd: gradients of <Y, dY> with sigma, silu and H recomputed from
 * the saved G and U:
 *   dH = dY Wd + s_d (dY Bd) Ad
 *   dU = dH * silu(G),  dG = dH * U * sigma(G) (1 + G (1 - sigma(G)))
 *   dX = dG Wg + s_g (dG Bg) Ag + dU Wu + s_u (dU Bu) Au      bf16 [M, D]
 *   LoRA gradients of the three layers as in qlora_linear_bwd (G_out).
 *   dG and dU live in the workspace.
 */
int qlora_mlp_bwd(const qlora_mlp* P, const void* dY, const void* X,
                  const qlora_mlp_saved* S, int64_t M, void* dX, const qlora_mlp_grads* G_out,
                  void* ws, size_t ws_bytes, void* stream);

/*
 * qlora_debug_force_arch: a test aid for the device check.  With a non-NULL
 * name, every entry point treats the current device as having that
 * gcnArchName: any name other than "gfx950..." makes each call that would
 * launch work return QLORA_ERR_UNSUPPORTED_DEVICE after validating its
 * arguments and before enqueuing anything.  NULL restores the query of the
 * real device.  Process-wide; set it while no other thread calls the library.
 * Returns QLORA_ERR_INVALID_ARG for a name of 64 characters or more.
 */
int qlora_debug_force_arch(const char* gcn_arch_name);

/*
 * qlora_trace_install: optional launch tracing, a profiling aid (off by
 * default).  While installed, every launch of a GEMM kernel (dequant-staged
 * or bf16-staged) records the caller-created events begin_events[i] and end_events[i]
 * (hipEvent_t handles) on its stream immediately before and after itself,
 * and stores its GEMM kind in kinds[i] (0 forward, 1 gate/up + SwiGLU
 * forward, 2 backward dX, 3 dH + SwiGLU backward, 4 dual-weight dX; plus 8
 * when the bf16-staged kernel ran, i.e. from 512 tokens on), for the
 * first `capacity` launches; *count is incremented for every launch seen.
 * Recording an event allocates nothing.  Pass capacity 0 (or NULL arrays)
 * to uninstall.  Process-wide and not thread-safe: install, run, uninstall
 * from one host thread.
 */
int qlora_trace_install(void** begin_events, void** end_events, int32_t* kinds, int32_t capacity,
                        int32_t* count);

#ifdef __cplusplus
}
#endif

#endif /* QLORA_H */
