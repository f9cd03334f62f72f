// Host-side planning shared by the launch code and the workspace queries.
// No HIP types here: this header is also compiled into the HIP-free
// argument-validation translation unit.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace qplan {

// Tile configurations of the dequant-staged MFMA GEMM (32x32x16 bf16 frags).
//   L256    : 4x2 waves, 2x4 frags per wave -> 256 tokens x 256 output columns,
//             activations staged through LDS (2 waves per SIMD)
//   SKINNY  : 1x2 waves, 2x1 frags per wave ->  64 tokens x  64 output columns,
//             activations loaded straight into registers
//   SKINNY_TR: 1x4 waves, 2x2 frags per wave -> 64 tokens x 256 output columns
//             of the transposed (backward) product, activations staged through
//             LDS: each weight row segment of a tile is one 128-byte line
enum GemmCfg { CFG_L256 = 0, CFG_SKINNY = 1, CFG_SKINNY_TR = 2 };

constexpr int kNumCUs = 256;
constexpr int64_t kBK = 64;  // reduction tile = one absmax block

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct GemmPlan {
  int cfg;
  int64_t bm, bn;
  int64_t tiles_m, tiles_n;
  int splits;            // reduction splits (fp32 partials + a reduce pass when > 1)
  int ktiles_per_split;  // 64-wide reduction tiles per split
};

// M tokens, Nout output columns, Kred reduction length (multiple of 64);
// trans: the single-linear backward product (the one transposed mode that
// may split its reduction).
inline GemmPlan plan_gemm(int64_t M, int64_t Nout, int64_t Kred, bool allow_split, bool trans = false) {
  GemmPlan p{};
  p.cfg = (M <= 128) ? CFG_SKINNY : CFG_L256;
  if (M <= 64 && trans && allow_split) p.cfg = CFG_SKINNY_TR;
  p.bm = (p.cfg == CFG_L256) ? 256 : 64;
  p.bn = (p.cfg == CFG_SKINNY) ? 64 : 256;
  p.tiles_m = cdiv(M, p.bm);
  p.tiles_n = cdiv(Nout, p.bn);
  const int64_t kt = Kred / kBK;
  int64_t splits = 1;
  const int64_t tiles = p.tiles_m * p.tiles_n;
  if (allow_split && tiles < kNumCUs) {
    splits = cdiv(kNumCUs, tiles);
    const int64_t max_splits = kt / 8 > 0 ? kt / 8 : 1;  // keep >= 8 tiles per split
    if (splits > max_splits) splits = max_splits;
    if (splits < 1) splits = 1;
  }
  int64_t per = cdiv(kt, splits);
  splits = cdiv(kt, per);
  p.splits = (int)splits;
  p.ktiles_per_split = (int)per;
  return p;
}

// Tokens per workgroup of the LoRA down-projection for a total rank rt: 64
// at ranks 33..64 (every workgroup reads its split's W columns whole, and at
// these ranks they are twice its token bytes with 32 tokens), else 32.
inline int down_tokens(int rt) { return (rt > 32 && rt <= 64) ? 64 : 32; }

// Reduction splits of the LoRA down-projection V = Z W^T (M x rt, reduce
// over Kred): one 8-wave workgroup per down_tokens(rt) tokens and split;
// enough splits to put one workgroup on every CU, each split keeping >= 2
// 64-wide chunks per wave.
inline int plan_down_splits(int64_t M, int64_t Kred, int rt) {
  const int64_t wgs = cdiv(M, down_tokens(rt));
  if (wgs >= kNumCUs) return 1;
  int64_t s = cdiv(kNumCUs, wgs);
  const int64_t max_s = Kred / 1024 > 0 ? Kred / 1024 : 1;
  if (s > max_s) s = max_s;
  return (int)(s < 1 ? 1 : s);
}

// Floats of split partials that any down-projection of total rank <= rmax
// over Kred may write (0: none).  The split count is not monotonic in the
// rank (more splits from rank 33, with 64-token workgroups), so this bounds
// both granularities.
inline size_t down_part_floats(int64_t M, int64_t Kred, int rmax) {
  size_t f = 0;
  const int s32 = plan_down_splits(M, Kred, 1);
  if (s32 > 1) f = (size_t)s32 * M * rmax;
  if (rmax > 32) {
    const int s64 = plan_down_splits(M, Kred, 64);
    const size_t f64 = s64 > 1 ? (size_t)s64 * M * (rmax < 64 ? rmax : 64) : 0;
    if (f64 > f) f = f64;
  }
  return f;
}

// Splits that launch_lora_down actually runs for a requested split count.
inline int down_splits_used(int64_t Kred, int splits) {
  const int64_t C = Kred / 64;
  if (C == 0 || splits <= 1) return 1;
  const int64_t per = cdiv(C, splits);
  return (int)cdiv(C, per);
}

// Skinny-M forward GEMM (M <= 64): one 4-wave workgroup per 16 * fn weight
// rows, fn from {1, 2, 4, 7, 8} the smallest that puts at most one
// workgroup on each CU; with fewer tiles than CUs the reduction is split
// (each wave keeping >= 2 of the 64-wide tiles), and it is split further
// while the workgroup's fp32 block absmax (16 fn rows x tiles) exceeds the
// 64 KB it stages in LDS.
struct SkinnyPlan {
  int fn;
  int splits;
  int kps;  // reduction tiles per split
};

inline SkinnyPlan plan_skinny_fwd(int64_t N, int64_t K) {
  static const int kFn[] = {1, 2, 4, 7, 8};
  SkinnyPlan p{8, 1, 0};
  for (int f : kFn)
    if (cdiv(N, 16 * f) <= kNumCUs) {
      p.fn = f;
      break;
    }
  const int64_t tiles = cdiv(N, 16 * p.fn);
  const int64_t kt = K / kBK;
  int64_t s = 1;
  if (tiles < kNumCUs) {
    s = kNumCUs / tiles;
    const int64_t max_s = kt / 8 > 0 ? kt / 8 : 1;
    if (s > max_s) s = max_s;
  }
  const int64_t max_tiles = (64 * 1024) / (4 * 16 * p.fn) - 4;  // row stride tiles + 4
  if (s < cdiv(kt, max_tiles)) s = cdiv(kt, max_tiles);
  const int64_t per = cdiv(kt, s > 0 ? s : 1);
  p.kps = (int)(per > 0 ? per : 1);
  p.splits = (int)(kt > 0 ? cdiv(kt, p.kps) : 1);
  return p;
}
inline bool use_skinny_fwd(int64_t M, int r) { return M >= 1 && M <= 64 && r <= 64; }

// Streaming skinny forward (M <= 64, K % 256 == 0): fn from {1, 2, 4, 7}, the
// smallest that puts at most one workgroup on each CU; with fewer tiles than
// CUs the reduction is split, each split a whole number of 4-tile groups and
// keeping >= 4 groups.
inline bool use_skinny_fwd2(int64_t M, int64_t N, int64_t K, int r) {
  return M >= 1 && M <= 64 && r <= 64 && K % 256 == 0 && N * (K / 16) < ((int64_t)1 << 31) &&
         K * 64 * 2 < ((int64_t)1 << 31);
}
inline int skinny_mp(int64_t M) { return (int)(16 * cdiv(M, 16)); }
inline SkinnyPlan plan_skinny_fwd2(int64_t N, int64_t K) {
  static const int kFn[] = {1, 2, 4, 7};
  SkinnyPlan p{7, 1, 0};
  for (int f : kFn)
    if (cdiv(N, 16 * f) <= kNumCUs) {
      p.fn = f;
      break;
    }
  const int64_t tiles = cdiv(N, 16 * p.fn);
  const int64_t groups = K / 256;
  int64_t s = 1;
  if (tiles < kNumCUs) {
    s = kNumCUs / tiles;
    const int64_t max_s = groups / 4 > 0 ? groups / 4 : 1;
    if (s > max_s) s = max_s;
  }
  const int64_t per = cdiv(groups, s > 0 ? s : 1);  // groups per split
  p.kps = (int)(4 * (per > 0 ? per : 1));
  p.splits = (int)(groups > 0 ? cdiv(groups, per) : 1);
  return p;
}

// Token splits of a LoRA-gradient reduction out[p, j] = sum_m Z[m, p] V[m, j].
// Each split writes an fp32 [P, r] partial; keep the partials small next to Z.
inline int plan_grad_msplits(int64_t M, int64_t P, int r) {
  const int64_t waves = cdiv(P, 256);
  int64_t s = cdiv(8 * kNumCUs, waves);  // ~8 waves per CU
  // partial bytes 4 * s * P * r must stay below ~1/4 of the Z bytes 2 * M * P
  int64_t cap = (M / (8 * (int64_t)r));
  if (cap < 1) cap = 1;
  if (s > cap) s = cap;
  const int64_t max_by_rows = cdiv(M, 64);  // >= 64 tokens per split
  if (s > max_by_rows) s = max_by_rows;
  return (int)(s < 1 ? 1 : s);
}

// Token count from which a GEMM runs as "expand the NF4 weight once into a
// bf16 workspace, then bf16 GEMM" (bgemm) instead of expanding it inside
// every 256-token tile (qgemm).
constexpr int64_t kBgemmMinTokens = 512;
inline bool use_bgemm(int64_t M) { return M >= kBgemmMinTokens; }
// Rows of the bf16 gate|up workspace: blocks of 128 gate rows + 128 up rows.
inline int64_t pair_rows(int64_t I) { return 256 * cdiv(I, 128); }

// The MLP backward takes T = Z B and dB = s Z^T V of each layer from one
// pass over Z (dY, dG, dU) when every rank is at most 16.  The pass splits
// tokens like the gradient reduction (32-token multiples) and columns in
// blocks of 512; its partials take nb M r + S P r floats per job.
inline bool use_lora_pair(int rg, int ru, int rd) {
  return rg >= 1 && rg <= 16 && ru >= 1 && ru <= 16 && rd >= 1 && rd <= 16;
}
// Token splits of the single-pass T + dB kernel: the gradient reduction's,
// capped at about two workgroups per CU per job (fewer dB partials to write
// and add).
inline int plan_pair_msplits(int64_t M, int64_t P, int r) {
  const int s = plan_grad_msplits(M, P, r);
  const int64_t cap = cdiv(2 * kNumCUs, cdiv(P, 512));
  return (int)(s < cap ? s : (cap < 1 ? 1 : cap));
}
inline size_t pair_part_floats(int64_t M, int64_t P, int r) {
  const int msplits = plan_pair_msplits(M, P, r);
  int64_t mps = (((M + msplits - 1) / msplits) + 31) / 32 * 32;
  if (mps <= 0) mps = 32;
  const int64_t S = cdiv(M, mps), nb = cdiv(P, 512);
  return (size_t)nb * M * r + (size_t)S * P * r;
}

struct LinearWs {
  size_t fwd_part, fwd_down;             // forward: split-K partials, down-proj partials
  size_t fwd_xt;                         // skinny forward: the re-laid-out activations
  size_t bwd_T, bwd_BT, bwd_part, bwd_down, bwd_grad;
  size_t wbuf;                           // bf16 weight copy (bgemm only), at the end
  size_t fwd_total, bwd_total, total;
};

inline LinearWs linear_ws(int64_t M, int64_t N, int64_t K, int r) {
  LinearWs w{};
  const bool bg = use_bgemm(M);
  GemmPlan pf = plan_gemm(M, N, K, true);
  w.fwd_part = (!bg && pf.splits > 1) ? align256((size_t)pf.splits * M * N * 4) : 0;
  if (use_skinny_fwd(M, r)) {
    const SkinnyPlan sp = plan_skinny_fwd(N, K);
    w.fwd_part = sp.splits > 1 ? align256((size_t)sp.splits * M * N * 4) : 0;
  }
  if (use_skinny_fwd2(M, N, K, r)) {
    const SkinnyPlan sp = plan_skinny_fwd2(N, K);
    w.fwd_part = sp.splits > 1 ? align256((size_t)sp.splits * M * N * 4) : 0;
    w.fwd_xt = align256((size_t)K * skinny_mp(M) * 2);
  }
  w.fwd_down = align256(down_part_floats(M, K, r) * 4);
  w.wbuf = bg ? align256((size_t)N * K * 2) : 0;
  w.fwd_total = w.fwd_part + w.fwd_down + w.fwd_xt + w.wbuf;

  GemmPlan pb = plan_gemm(M, K, N, true, true);
  w.bwd_T = align256((size_t)M * r * 4);
  w.bwd_BT = align256((size_t)N * r * 2) + align256((size_t)K * r * 2);  // B^T [r, N], A^T [K, r]
  w.bwd_part = (!bg && pb.splits > 1) ? align256((size_t)pb.splits * M * K * 4) : 0;
  // skinny backward: the transposed product always writes split partials
  if (pb.cfg == CFG_SKINNY_TR) w.bwd_part = align256((size_t)pb.splits * M * K * 4);
  w.bwd_down = align256(down_part_floats(M, N, r) * 4);
  const int gs_b = plan_grad_msplits(M, N, r);
  const int gs_a = plan_grad_msplits(M, K, r);
  size_t gb = align256((size_t)gs_b * N * r * 4), ga = align256((size_t)gs_a * K * r * 4);
  w.bwd_grad = gb > ga ? gb : ga;
  // T = dY B and dB from one pass over dY (rank <= 16) share that region
  if (r >= 1 && r <= 16) {
    const size_t pp = align256(pair_part_floats(M, N, r) * 4);
    if (pp > w.bwd_grad) w.bwd_grad = pp;
  }
  w.bwd_total = w.bwd_T + w.bwd_BT + w.bwd_part + w.bwd_down + w.bwd_grad + w.wbuf;
  w.total = w.fwd_total > w.bwd_total ? w.fwd_total : w.bwd_total;
  if (w.total == 0) w.total = 256;
  return w;
}

// SwiGLU backward on the bf16 path: the down layer's dA = s T^T H is
// computed in the dH GEMM's epilogue (from the G, U it reads anyway) for
// ranks up to 32.
inline bool fuse_dad(int rd) { return rd >= 1 && rd <= 32; }

// The gate/up GEMM on the bf16 path takes its LoRA terms as extra reduction
// columns: [s_g XA_g | s_u XA_u] (bf16) against [B_g | 0] on the gate rows and
// [0 | B_u] on the up rows of the expanded weight, zero-padded to whole
// 64-column reduction tiles.
inline int64_t lora_ext_cols(int rg, int ru) { return 64 * cdiv(rg + ru, 64); }

struct MlpWs {
  size_t fwd_H, fwd_down;                            // H bf16 [M, I], down-proj partials
  size_t fwd_ext;                                    // [s_g XA_g | s_u XA_u] bf16 [M, ext] (bgemm)
  size_t bwd_Td, bwd_dG, bwd_dU, bwd_Tg, bwd_Tu, bwd_BT, bwd_down, bwd_grad;
  size_t fwd_had;                                    // H A_d^T column-tile partials (bgemm, r_d <= 32)
  size_t bwd_pair;                                   // single-pass LoRA product partials (ranks <= 16)
  size_t bwd_tdt;                                    // T_d^T bf16 for the dH epilogue's dA_d (bgemm)
  size_t fwd_wbuf, bwd_wbuf;                         // bf16 weight copies (bgemm only), at the end
  size_t fwd_total, bwd_total, total;
};

inline MlpWs mlp_ws(int64_t M, int64_t D, int64_t I, int rg, int ru, int rd) {
  MlpWs w{};
  int rmax = rg > ru ? rg : ru;
  if (rd > rmax) rmax = rd;
  w.fwd_H = align256((size_t)M * I * 2);
  // X [A_g | A_u]^T (or one layer at a time) over D, H A_d^T over I
  size_t d1 = align256(down_part_floats(M, D, rg + ru) * 4);
  size_t d2 = align256(down_part_floats(M, I, rd) * 4);
  w.fwd_down = d1 > d2 ? d1 : d2;
  if (use_bgemm(M)) {
    const int64_t ext = lora_ext_cols(rg, ru);
    const size_t gu = (size_t)pair_rows(I) * (D + ext) * 2, dn = (size_t)D * I * 2;
    w.fwd_wbuf = align256(gu > dn ? gu : dn);
    w.fwd_ext = align256((size_t)M * ext * 2);
    w.bwd_wbuf = align256((size_t)2 * I * D * 2);
  }
  if (use_bgemm(M) && rd <= 32) w.fwd_had = align256((size_t)cdiv(I, 128) * M * rd * 4);
  w.fwd_total = w.fwd_H + w.fwd_down + w.fwd_had + w.fwd_ext + w.fwd_wbuf;

  w.bwd_Td = align256((size_t)M * rd * 4);
  w.bwd_dG = align256((size_t)M * I * 2);
  w.bwd_dU = align256((size_t)M * I * 2);
  w.bwd_Tg = align256((size_t)M * rg * 4);
  w.bwd_Tu = align256((size_t)M * ru * 4);
  // B_d^T [rd, D], B_g^T [rg, I], B_u^T [ru, I]; A_d^T [I, rd], A_g^T [D, rg], A_u^T [D, ru]
  w.bwd_BT = align256((size_t)rd * D * 2) + align256((size_t)rg * I * 2) + align256((size_t)ru * I * 2) +
             align256((size_t)I * rd * 2) + align256((size_t)D * rg * 2) + align256((size_t)D * ru * 2);
  // dY B_d over D; dG B_g, dU B_u over I
  size_t e1 = align256(down_part_floats(M, D, rd) * 4);
  size_t e2 = align256(down_part_floats(M, I, rmax) * 4);
  w.bwd_down = e1 > e2 ? e1 : e2;
  size_t g = 0;
  const int64_t Ps[6] = {D, I, I, D, I, D};
  const int Rs[6] = {rd, rd, rg, rg, ru, ru};
  for (int i = 0; i < 6; ++i) {
    const int ms = plan_grad_msplits(M, Ps[i], Rs[i]);
    size_t b = align256((size_t)ms * Ps[i] * Rs[i] * 4);
    if (b > g) g = b;
  }
  // the dH GEMM's per-token-tile partials of dA_d (bgemm, r_d <= 32), and
  // its T_d operand as bf16 [r_d][M rounded up to 8]
  if (use_bgemm(M) && fuse_dad(rd)) {
    const size_t b = align256((size_t)cdiv(M, 256) * I * rd * 4);
    if (b > g) g = b;
    w.bwd_tdt = align256((size_t)rd * (size_t)(8 * cdiv(M, 8)) * 2);
  }
  w.bwd_grad = g;
  if (use_lora_pair(rg, ru, rd)) {
    // dA_g and dA_u from one pass over X: both ranks' token-split partials
    const int rm = rg > ru ? rg : ru;
    const size_t b2 = align256((size_t)plan_grad_msplits(M, D, rm) * D * (rg + ru) * 4);
    if (b2 > w.bwd_grad) w.bwd_grad = b2;
    // the dY job (Td, dB_d), then the dG and dU jobs together
    const size_t a = pair_part_floats(M, D, rd);
    const size_t b = pair_part_floats(M, I, rg) + pair_part_floats(M, I, ru);
    w.bwd_pair = align256((a > b ? a : b) * 4);
  }
  w.bwd_total = w.bwd_Td + w.bwd_dG + w.bwd_dU + w.bwd_Tg + w.bwd_Tu + w.bwd_BT + w.bwd_down + w.bwd_grad +
                w.bwd_pair + w.bwd_tdt + w.bwd_wbuf;
  w.total = w.fwd_total > w.bwd_total ? w.fwd_total : w.bwd_total;
  if (w.total == 0) w.total = 256;
  return w;
}

// MLP forward with the RMSNorm folded in (qlora_mlp_fwd_rmsnorm): the MLP
// forward's workspace, then A_g w and A_u w (bf16), the unscaled X (A w)^T
// (fp32 [M, r_g + r_u]) and, below the bf16-GEMM threshold (where the norm
// runs as its own pass), the normalised input (bf16 [M, D]).
struct MlpRmsWs {
  size_t base, at_g, at_u, xa, xn, total;
};
inline MlpRmsWs mlp_rms_ws(int64_t M, int64_t D, int64_t I, int rg, int ru, int rd) {
  MlpRmsWs w{};
  w.base = mlp_ws(M, D, I, rg, ru, rd).fwd_total;
  w.at_g = align256((size_t)rg * D * 2);
  w.at_u = align256((size_t)ru * D * 2);
  w.xa = align256((size_t)M * (rg + ru) * 4);
  w.xn = use_bgemm(M) ? 0 : align256((size_t)M * D * 2);
  w.total = w.base + w.at_g + w.at_u + w.xa + w.xn;
  return w;
}

// Output head + cross-entropy: C tokens per chunk; the dX product of a chunk
// ([C, V] x [V, D]) splits its vocabulary reduction so that tiles x splits
// covers the chip about twice, with at least 32 vocabulary tiles per split.
struct CeWs {
  int64_t C;
  int splits, kps;
  size_t nvalid, tloss, logits, wt, part, total;
};

inline CeWs ce_ws(int64_t T, int64_t D, int64_t V, int64_t chunk, bool want_dx) {
  CeWs w{};
  w.C = T < chunk ? T : chunk;
  if (w.C < 1) w.C = 1;
  const int64_t kt = V / 64;
  const int64_t tiles = cdiv(w.C, 256) * cdiv(D, 256);
  int64_t splits = cdiv(2 * kNumCUs, tiles);
  const int64_t max_splits = kt / 32 > 0 ? kt / 32 : 1;
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  const int64_t per = cdiv(kt, splits);
  w.splits = (int)cdiv(kt, per);
  w.kps = (int)per;
  w.nvalid = 256;
  w.tloss = align256((size_t)T * 4);
  w.logits = align256((size_t)w.C * V * 4);  // fp32 logits; the bf16 gradient overwrites them
  w.wt = 0;  // the dX product reads the head as stored (K-major weight operand)
  w.part = (want_dx && w.splits > 1) ? align256((size_t)w.splits * w.C * D * 4) : 0;
  w.total = w.nvalid + w.tloss + w.logits + w.wt + w.part;
  return w;
}

}  // namespace qplan
