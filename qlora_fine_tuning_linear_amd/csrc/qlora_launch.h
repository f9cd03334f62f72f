// Kernel launchers and their argument blocks (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qlora_plan.h"

// GEMM modes of qgemm_kernel.
enum {
  MODE_FWD = 0,         // Y  = X W^T + LoRA                 (weight [N, K], reduce over K)
  MODE_FWD_SWIGLU = 1,  // G, U = X Wg^T, X Wu^T + LoRA; H = silu(G) * U
  MODE_BWD = 2,         // dX = dY W + LoRA                  (weight [N, K], reduce over N)
  MODE_BWD_SWIGLU = 3,  // dH = dY Wd + LoRA; dG, dU from G, U
  MODE_BWD_DUAL = 4,    // dX = dG Wg + dU Wu + both LoRA terms (reduce over 2I)
};

struct Nf4Dev {
  const uint8_t* codes;
  const float* absmax;        // dq == 0
  const uint8_t* absmax_q;    // dq > 0
  const float* absmax_scale;  // dq > 0
  int64_t N, K;
  int32_t dq;
};

// One LoRA epilogue term: out[m, c] += s * sum_j V[m, j] * Wl(c, j),
// Wl(c, j) = Wl[c * wl_sc + j * wl_sj]  (B [N, r]: (r, 1); A [r, K]: (1, K)).
struct LoraSide {
  const float* V;
  const uint16_t* Wl;
  int64_t wl_sc, wl_sj;
  int32_t r;
  float s;
};

struct GemmArgs {
  const uint16_t* act0;
  const uint16_t* act1;
  int64_t M, Nout, Kred0, Kred1;
  Nf4Dev w0, w1;
  const float* codebook;   // table of w0
  const float* codebook1;  // table of w1 (dual-weight modes)
  LoraSide l0, l1;
  uint16_t* out0;
  uint16_t* out1;
  uint16_t* out2;
  const uint16_t* in0;
  const uint16_t* in1;
  float* partial;
  int64_t tiles_m, tiles_n;
  int32_t ktiles_per_split;
  // bgemm_kernel: the weight operand as bf16 rows (row = output column,
  // contiguous along the reduction), row stride ldw, rows [0, wrows) valid
  const uint16_t* wb;
  int64_t ldw, wrows;
  // bgemm_kernel, SwiGLU forward only: the rank-r product H A^T of the down
  // layer computed from the epilogue's H (A bf16 [r, Nout], r <= 32), written
  // as per-column-tile fp32 partials part[tiles_n][M][r] (null: not computed)
  const uint16_t* had_A;
  int32_t had_r;
  float* had_part;
  // bgemm_kernel only: row stride of act0 / act1 in elements (0: Kred0), and,
  // in the plain forward mode, fp32 results written to partial as [M][Nout]
  // instead of bf16 to out0
  int64_t lda;
  int32_t out_f32;
  // bgemm_kernel: row stride of act1 in elements when it differs from lda
  // (0: lda).  In the SwiGLU forward a nonzero Kred1 means that the LoRA
  // terms come as these extra reduction columns (act1 against columns
  // Kred0 .. Kred0 + Kred1 of the weight rows) instead of l0 / l1.
  int64_t lda1;
  // bgemm_kernel, SwiGLU backward only: the down layer's rank-r product
  // T^T H (T = l0.V fp32 [M, r], r = l0.r <= 32; H = silu(in0) in1 rounded
  // to bf16) as per-token-tile fp32 partials dad_part[tiles_m][Nout][r]
  // (null: not computed)
  float* dad_part;
  // with dad_part: T as bf16 transposed, dad_tt[j * dad_tt_ld + m] (rows
  // j < r, tokens m < dad_tt_ld, a multiple of 8; zero past M)
  const uint16_t* dad_tt;
  int64_t dad_tt_ld;
  // bgemm_kernel, SwiGLU forward only: every token row m of the product
  // (LoRA term included) is multiplied by row_scale[m] before the epilogue
  // (null: not scaled)
  const float* row_scale;
  // bgemm_kernel, plain forward only: the weight operand stored K-major,
  // wb[k ldw + n] for k < Kred0, n < wrows (ldw >= wrows, a multiple of 8)
  int32_t w_kmajor;
};

// Skinny-M forward GEMM (qlora_skinny.hip): out[m, n] = sum_k X[m, k]
// deq(w)[n, k] + s sum_j V[m, j] Wl(n, j), V = sum_z vpart[z] ([M, r] fp32
// partials of the down-projection, vsplits of them; when vout is set, V is
// also written there).  With part set, split z of the reduction writes fp32
// partials part[z][M][N] instead of out (LoRA term in split 0 only).
struct SkinnyArgs {
  const uint16_t* X;
  int64_t M, N, K;
  Nf4Dev w;
  const float* codebook;
  const float* vpart;
  int32_t vsplits;
  float* vout;
  const uint16_t* Wl;
  int64_t wl_sc, wl_sj;
  int32_t r;
  float s;
  uint16_t* out;
  float* part;
  int32_t kps;  // 64-wide reduction tiles per split
  // streaming form (skinny_fwd2_kernel): the activations re-laid out as
  // Xt[K/8][Mp][8] (Mp = M rounded up to 16, zero rows past M)
  const uint16_t* Xt;
  int32_t Mp;
};

// Skinny-M backward finish (qlora_skinny.hip): dX = sum of the split
// partials + s T A, dA = s T^T X, dB = s dY^T XA (T = sum of tpart), bf16
// outputs; M <= 64, r <= 128, K and N multiples of 64.
struct SkinnyFinishArgs {
  int64_t M, N, K;
  int32_t r;
  float s;
  const float* part;   // [splits][M][K]
  int32_t splits;
  const float* tpart;  // [tsplits][M][r]
  int32_t tsplits;
  const float* XA;     // [M][r]
  const uint16_t* X;   // [M][K]
  const uint16_t* dY;  // [M][N]
  const uint16_t* A;   // [r][K]
  uint16_t* dX;
  uint16_t* dA;
  uint16_t* dB;
};

// Skinny-M transposed product (qlora_skinny.hip): part[z][M][K] =
// dY[:, tiles of split z] deq(w)[those rows, :], 64-row tiles, kps per split.
struct SkinnyBwdArgs {
  const uint16_t* dY;  // [M][N]
  int64_t M, N, K;     // weight [N, K]
  Nf4Dev w;
  const float* codebook;
  float* part;
  int32_t kps;
};

hipError_t launch_nf4_quantize(const float* W, int64_t nblocks, const float* codebook, int dq, uint8_t* codes,
                               float* absmax, uint8_t* absmax_q, float* absmax_scale, hipStream_t st);
// out [N, K] 16-bit = round16(deq(w) + s B A) (f16: fp16, else bf16).
hipError_t launch_merge(const Nf4Dev& w, const float* codebook, const uint16_t* A, const uint16_t* B, int r,
                        float s, int f16, uint16_t* out, hipStream_t st);
// Packed LoRA groups: row ranges noff[g] .. noff[g+1] of the packed weight and
// rank columns roff[g] .. roff[g+1] belong to group g.
struct GroupDesc {
  const uint16_t* B[8];
  uint16_t* dB[8];
  int32_t noff[9], roff[9];
  float s[8];
  int32_t G;
};
// out [Nt, Rt] bf16 = block-diagonal of the bf16(s_g B_g)
hipError_t launch_grouped_bcat(const GroupDesc& d, int Nt, int Rt, uint16_t* out, hipStream_t st);
// dB_g = bf16(s_g * diagonal block g of dbcat [Nt, Rt])
hipError_t launch_grouped_db(const GroupDesc& d, int Nt, int Rt, const uint16_t* dbcat, hipStream_t st);
// dB_g = bf16(s_g Z_g^T V[:, roff_g .. roff_g + r_g)) straight from Z [M, P]
// (P = Nt columns, Z_g its group-g columns) and V fp32 [M, Rt], when every
// r_g <= 16, P % 8 == 0 and every group boundary is a multiple of 128
// (grouped_grad_ok); part fp32 [S][P][16] with S <= msplits.
bool grouped_grad_ok(const GroupDesc& d, int64_t P);
hipError_t launch_grouped_grad(const GroupDesc& d, const uint16_t* Z, int64_t M, int64_t P, const float* V, int Rt,
                               int msplits, float* part, hipStream_t st);
// RMSNorm: Y = X rstd w (rstd saved per row) and its backward; D % 8 == 0,
// D <= 8192.  The backward with dw needs part fp32 [rmsnorm_bwd_groups(M)][D].
int rmsnorm_bwd_groups(int64_t M);
// rows of A [rows, K] bf16 times w [K] bf16 -> out, bf16 (fp32 product rounded)
hipError_t launch_scale_cols(const uint16_t* A, int64_t rows, int64_t K, const uint16_t* w, uint16_t* out,
                             hipStream_t st);
// out[m, j] = in[m, j] * s[m], fp32 [M, r]
hipError_t launch_scale_rows(const float* in, int64_t M, int r, const float* s, float* out, hipStream_t st);
hipError_t launch_rmsnorm_fwd(const uint16_t* X, const uint16_t* w, int64_t M, int64_t D, float eps, uint16_t* Y,
                              float* rstd, hipStream_t st);
hipError_t launch_rmsnorm_bwd(const uint16_t* dY, const uint16_t* X, const uint16_t* w, const float* rstd,
                              int64_t M, int64_t D, uint16_t* dX, float* dw, float* part, hipStream_t st);
hipError_t launch_nf4_dequantize(const Nf4Dev& w, const float* codebook, int out_f32, void* out, hipStream_t st);
hipError_t launch_qgemm(int mode, const GemmArgs& a, const qplan::GemmPlan& pl, hipStream_t st);
hipError_t launch_bgemm(int mode, const GemmArgs& a, hipStream_t st);
// Sum of the H A^T partials of launch_bgemm (MODE_FWD_SWIGLU) in tile order.
hipError_t launch_had_finish(const float* part, int tiles, int64_t M, int r, float* out, hipStream_t st);
// out [r][ld] bf16 = T^T for T fp32 [M, r] (ld >= M, a multiple of 8; zero for
// M <= m < ld)
hipError_t launch_t_bf16_trans(const float* T, int64_t M, int r, int64_t ld, uint16_t* out, hipStream_t st);
// out = bf16(s * sum_z part[z]) over S fp32 partials [S][P][r], written as
// [P, r] (out_rp = 0) or [r, P] (out_rp = 1)
hipError_t launch_grad_finish(const float* part, int S, int64_t P, int r, float s, int out_rp, uint16_t* out,
                              hipStream_t st);
// Output head + cross-entropy helpers (qlora_ce.hip).
hipError_t launch_ce_count(const int32_t* targets, int64_t T, int64_t V, int32_t ignore, int32_t* n_valid,
                           hipStream_t st);
// z: fp32 logits [rows][V]; with want_grad each row's first 2V bytes are
// overwritten by the bf16 logit gradient (row stride 2V bf16 elements).
hipError_t launch_ce_rows(float* z, int64_t rows, int64_t V, const int32_t* targets, int32_t ignore,
                          const int32_t* n_valid, int want_grad, float* token_loss, hipStream_t st);
hipError_t launch_ce_loss(const float* token_loss, int64_t T, const int32_t* n_valid, float* loss, hipStream_t st);
// bf16 copy of the dequantized weight(s) for bgemm_kernel.
//   rows : out[R, 0:K] = deq(W)[src(R), :]; with w1 (SwiGLU pair) rows come in
//          blocks of 256 = 128 gate rows then the 128 up rows of the same
//          columns (rows past N are zero), else src(R) = R.
//   trans: out[k, col0 + n] = deq(W)[n, k] (row stride ldo).
hipError_t launch_dequant_rows(const Nf4Dev& w0, const Nf4Dev* w1, const float* codebook0, const float* codebook1,
                               int64_t rows_out, uint16_t* out, hipStream_t st,
                               const uint16_t* colw = nullptr, int64_t ldo = 0);
// The LoRA extension of a SwiGLU pair's expanded rows (row stride ldo):
// out[R, K + j] for j < ext = B_g[src(R), j] (j < rg) on gate rows,
// B_u[src(R), j - rg] (rg <= j < rg + ru) on up rows, 0 elsewhere and past N.
hipError_t launch_lora_ext_cols(const uint16_t* Bg, int rg, const uint16_t* Bu, int ru, int64_t N, int64_t rows_out,
                                int64_t K, int64_t ldo, int64_t ext, uint16_t* out, hipStream_t st);
// act [M, ext] bf16: bf16(sg Vg[m, j]) for j < rg, bf16(su Vu[m, j - rg]) for
// rg <= j < rg + ru, 0 past that (V fp32 [M, r]).
hipError_t launch_lora_ext_act(const float* Vg, int rg, float sg, const float* Vu, int ru, float su, int64_t M,
                               int64_t ext, uint16_t* act, hipStream_t st);
hipError_t launch_dequant_trans(const Nf4Dev& w, const float* codebook, uint16_t* out, int64_t ldo, int64_t col0,
                                hipStream_t st);
hipError_t launch_splitk_finish(const float* part, int splits, int64_t M, int64_t Nout, uint16_t* out,
                                hipStream_t st);
bool skinny_fwd_supported(int64_t M, int r);
bool skinny_fwd2_supported(int64_t M, int64_t N, int64_t K, int r);
// Xt[j][m][0..7] = X[m][8j..8j+7] (zero for M <= m < Mp)
hipError_t launch_xtile(const uint16_t* X, int64_t M, int64_t K, int Mp, uint16_t* Xt, hipStream_t st);
hipError_t launch_skinny_fwd2(const SkinnyArgs& a, const qplan::SkinnyPlan& pl, hipStream_t st);
bool skinny_finish_supported(int64_t M, int r);
bool skinny_bwd_supported(int64_t M, int64_t N, int64_t K);
hipError_t launch_skinny_bwd(const SkinnyBwdArgs& a, int splits, hipStream_t st);
hipError_t launch_skinny_bwd_finish(const SkinnyFinishArgs& a, hipStream_t st);
hipError_t launch_skinny_fwd(const SkinnyArgs& a, const qplan::SkinnyPlan& pl, hipStream_t st);
// V0 | V1 = Z W0^T | Z W1^T, W0 [r0, Kred], W1 [r1, Kred] (r0 + r1 <= 128).
// With finish = false and more than one split (qplan::down_splits_used) the
// fp32 partials stay in part[split][M][r0 + r1] for the consumer to sum.
// Rank <= 16 only: w_nr reads W0 stored [Kred, r0] (r1 = 0), i.e. V0 = Z W0;
// Xt (with Mp = M rounded up to 16) also receives Z re-laid out as
// Xt[Kred/8][Mp][8], rows M..Mp-1 zero.
hipError_t launch_lora_down(const uint16_t* Z, int64_t M, int64_t Kred, const uint16_t* W0, int r0,
                            const uint16_t* W1, int r1, float* V0, float* V1, int splits, float* part,
                            hipStream_t st, bool finish = true, bool w_nr = false, uint16_t* Xt = nullptr,
                            int Mp = 0);
// B [N, r] -> B^T [r, N]
hipError_t launch_transpose_rn(const uint16_t* B, int64_t N, int r, uint16_t* BT, hipStream_t st);

// Both LoRA products of one gradient-sized operand Z [M, P] (bf16) from a
// single read of Z: T = Z Bt^T ([M, r] fp32, Bt = B^T [r, P] bf16) and
// dB = s Z^T V ([P, r] bf16, V [M, r] fp32), r <= 16.  Up to two such jobs
// of the same M and P run in one launch; the kernel writes T partials per
// 512-column block (tpart [nb][M][r]) and dB partials per token split
// (gpart [S][P][r]); the finish launch adds them in fixed order.
struct PairJob {
  const uint16_t* Z;
  const uint16_t* Bt;
  const float* V;
  int32_t r;
  float s;
  float* tpart;
  float* gpart;
  float* T;
  uint16_t* dB;
  // optional: T also as bf16 T^T [r][tt_ld] (tokens past M zero), the dH
  // epilogue's dA_d operand
  uint16_t* Tt;
  int64_t tt_ld;
};
struct PairArgs {
  PairJob job[2];
  int32_t njobs;
  int64_t M, P;
  int64_t m_per_split;  // tokens per split (a multiple of 32)
  int32_t S;            // token splits
  int32_t nb;           // 512-column blocks
};
// Fills the split and block counts of a for M, P (r of the jobs <= 16) and
// njobs jobs in the launch; the partial buffers need
// qplan::pair_part_floats(M, P, r) floats per job (an upper bound: the split
// count may come out lower so that the launch fills whole rounds).
void plan_lora_pair(PairArgs& a, int64_t M, int64_t P, int r, int njobs = 1);
hipError_t launch_lora_pair(const PairArgs& a, hipStream_t st);
// Several transposes in one launch: job k, src [rows, cols] -> dst [cols, rows].
struct TransposeJobs {
  const uint16_t* src[6];
  uint16_t* dst[6];
  int64_t rows[6];
  int64_t cols[6];
  int32_t n;
};
struct TransposeBatch {
  TransposeJobs J{};
  void add(const uint16_t* src, int64_t rows, int64_t cols, uint16_t* dst) {
    const int k = J.n++;
    J.src[k] = src;
    J.dst[k] = dst;
    J.rows[k] = rows;
    J.cols[k] = cols;
  }
};
hipError_t launch_transpose_multi(const TransposeJobs& J, hipStream_t st);
// dA of two layers that share their input Z [M, P] from one pass over it:
// out_k = bf16(s_k V_k^T Z) as [r_k, P] (r_k <= 16, P % 8 == 0); part holds
// the token-split partials of both (lora_grad2_part_floats of them).
hipError_t launch_lora_grad2(const uint16_t* Z, int64_t M, int64_t P, const float* V0, int r0, float s0,
                             uint16_t* out0, const float* V1, int r1, float s1, uint16_t* out1, float* part,
                             hipStream_t st);
hipError_t launch_lora_grad(int zmode, const uint16_t* Z0, const uint16_t* Z1, int64_t M, int64_t P,
                            const float* V, int r, float s, int msplits, float* part, int out_rp, uint16_t* out,
                            hipStream_t st);
