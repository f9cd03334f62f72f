// Skinny-M QLoRA GEMMs (M <= 64 tokens) for gfx950: the forward
// Y = X deq(W0)^T + s (X A^T) B^T of "LLM Fine-Tuning in 2026: Unsloth vs
// QLoRA vs Liger-Kernel" (section 1) when the token count is so small that
// the NF4 weight stream from HBM is the bound.
//
// Design.  With 64 tokens every weight element feeds 64 multiply-adds, so
// the kernel has to keep roughly 64 KB of loads in flight per CU and expand
// the codes with as few vector instructions as possible.  One 4-wave
// workgroup per CU (one wave per SIMD, 512 registers each) owns R = 16 FN
// weight rows; its waves split the reduction (wave w takes the w-th
// contiguous quarter of the workgroup's 64-wide reduction tiles) and each
// wave streams all R rows over its tiles:
//   * codes go straight from HBM into registers (8 bytes per lane per
//     16-row frag: the 32-byte row segment of a tile is read by 4 lanes),
//     are expanded in registers (codebook in LDS, times the block absmax,
//     rounded to bf16) and fed to v_mfma_f32_16x16x32_bf16 as the B operand
//     (columns = weight rows), so the expanded weight never touches LDS;
//   * the activation tile of each reduction tile is read by exactly one wave
//     (from L2, where the 64-token activation matrix stays resident) as the
//     A operand (rows = tokens);
//   * codes and activations of the next three tiles are in flight while the
//     current one is expanded and multiplied (a ring of four register sets);
//     the block absmax of the workgroup's rows and tiles is staged in LDS
//     once, as fp32.
// The four per-wave partial tiles are summed in LDS in wave order (results
// do not depend on timing), the LoRA term is added as one more MFMA step,
// and the tile is stored as bf16 (or as an fp32 split partial).
//
// Reduction order: lane group q (lanes 16q .. 16q+15) of MFMA step s holds
// reduction index 16q + 8s + e of the tile, e < 8, for both operands.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qlora_device.h"
#include "qlora_gemm_common.h"
#include "qlora_launch.h"

namespace qk {

// One 16x16x32 bf16 MFMA: C[16x16] += A[16x32] B[32x16].  Lane l holds
// A[l%16][k(l/16, e)] and B[k(l/16, e)][l%16] for e < 8 (the same reduction
// indices in both operands); accumulator element v of lane l is
// C[4*(l/16) + v][l%16].
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

constexpr int SK_WAVES = 4;   // one wave per SIMD: 512 registers each
constexpr int SK_TF = 4;      // token frags of 16: up to 64 tokens
constexpr int SK_DEPTH = 4;   // register sets of the load ring (tiles in flight + 1)
constexpr int SK_ABS_LDS = 64 * 1024;  // bytes of block absmax staged per workgroup

template <int FN, bool DQ>
__global__ __launch_bounds__(256) void skinny_fwd_kernel(SkinnyArgs p) {
  constexpr int TF = SK_TF;
  constexpr int R = 16 * FN;
  constexpr int D = SK_DEPTH;
  __shared__ float cb[16];
  __shared__ float red[SK_WAVES][TF * 4 * 64];
  __shared__ float vs[64 * 64];                 // V = sum of the down-projection partials, [M][r]
  __shared__ float absl[SK_ABS_LDS / 4];        // block absmax, [tile - kb][row - n0]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, q = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * R;
  const int KT = (int)(p.K / 64);
  const int kb = blockIdx.y * p.kps, ke = min(KT, kb + p.kps);
  const int kpw = (ke - kb + SK_WAVES - 1) / SK_WAVES;
  const int wb = min(ke, kb + wave * kpw), we = min(ke, wb + kpw);
  const int nt = we - wb;  // this wave's tiles
  const bool lora_here = blockIdx.y == 0 && p.r > 0;

  // ---- operand pointers (rows clamped into range; clamped rows are not stored)
  const uint8_t* cptr[FN];
#pragma unroll
  for (int f = 0; f < FN; ++f) {
    int64_t row = n0 + 16 * f + l16;
    if (row >= p.N) row = p.N - 1;
    cptr[f] = p.w.codes + row * (p.K / 2) + 8 * q;
  }
  const uint16_t* xptr[TF];
#pragma unroll
  for (int i = 0; i < TF; ++i) {
    int64_t m = 16 * i + l16;
    if (m >= p.M) m = p.M - 1;
    xptr[i] = p.X + m * p.K + 16 * q;
  }

  struct Regs {
    u32x4 x[TF][2];
    u32x2 c[FN];
  };
  auto load = [&](int kt, Regs& g) {
#pragma unroll
    for (int f = 0; f < FN; ++f) g.c[f] = *reinterpret_cast<const u32x2*>(cptr[f] + (int64_t)kt * 32);
#pragma unroll
    for (int i = 0; i < TF; ++i)
#pragma unroll
      for (int s = 0; s < 2; ++s) g.x[i][s] = *reinterpret_cast<const u32x4*>(xptr[i] + (int64_t)kt * 64 + 8 * s);
  };

  // the first D - 1 tiles are requested before anything else
  Regs g[D];
  if (nt > 0) {
#pragma unroll
    for (int u = 0; u < D - 1; ++u) load(wb + min(u, nt - 1), g[u]);
  }

  // ---- block absmax of the workgroup's rows and tiles into LDS (fp32).
  // Row rr's tiles are contiguous in memory; when they start and end on a
  // 4-tile boundary they are read 4 at a time (one 4-byte load of codes with
  // double quantization, one 16-byte load otherwise), all of a thread's
  // loads issued before the first is used.
  if (tid < 16) cb[tid] = p.codebook[tid];
  {
    const int ntile = ke - kb;
    if (((KT | kb | ntile) & 3) == 0) {
      const int nq = ntile >> 2, total = R * nq;  // 4-tile groups
      constexpr int PER = SK_ABS_LDS / 16 / 256;     // groups per thread at most
      uint32_t cq[PER];
      f32x4 af[PER];
      float sc[PER];
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int e = tid + 256 * j;
        const int rr = e / max(nq, 1), g4 = e - rr * max(nq, 1);
        int64_t row = n0 + rr;
        if (row >= p.N) row = p.N - 1;
        const int64_t blk = row * KT + kb + 4 * g4;
        if (e < total) {
          if constexpr (DQ) {
            cq[j] = *reinterpret_cast<const uint32_t*>(p.w.absmax_q + blk);
            sc[j] = p.w.absmax_scale[blk >> 8];
          } else {
            af[j] = *reinterpret_cast<const f32x4*>(p.w.absmax + blk);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int e = tid + 256 * j;
        if (e < total) {
          const int rr = e / nq, g4 = e - rr * nq;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            float a;
            if constexpr (DQ)
              a = (float)((cq[j] >> (8 * u)) & 0xFFu) * sc[j];
            else
              a = af[j][u];
            absl[(4 * g4 + u) * R + rr] = a;
          }
        }
      }
    } else {
      for (int e0 = 0; e0 < R * ntile; e0 += 256 * 8) {
        float a[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int e = min(e0 + tid + 256 * j, R * ntile - 1);
          const int rr = e / ntile, t = e - rr * ntile;
          int64_t row = n0 + rr;
          if (row >= p.N) row = p.N - 1;
          a[j] = absmax_at<DQ>(p.w, row * KT + kb + t);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int e = e0 + tid + 256 * j;
          if (e < R * ntile) {
            const int rr = e / ntile, t = e - rr * ntile;
            absl[t * R + rr] = a[j];
          }
        }
      }
    }
  }

  f32x4 acc[FN][TF];
#pragma unroll
  for (int f = 0; f < FN; ++f)
#pragma unroll
    for (int i = 0; i < TF; ++i) acc[f][i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // Expansion of one tile: the 16 codebook lookups of frag f + 1 are issued
  // before frag f is scaled, rounded and multiplied, so that their LDS
  // latency overlaps the matrix work of frag f.
  auto look = [&](const u32x2 c, float (&v)[16]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[e] = cb[(c[0] >> (4 * e)) & 15u];
      v[8 + e] = cb[(c[1] >> (4 * e)) & 15u];
    }
  };
  auto compute = [&](int kt, const Regs& gg) {
    const float* arow = absl + (kt - kb) * R + l16;
    float a[FN];
#pragma unroll
    for (int f = 0; f < FN; ++f) a[f] = arow[16 * f];
    float lv[2][16];
    look(gg.c[0], lv[0]);
#pragma unroll
    for (int f = 0; f < FN; ++f) {
      if (f + 1 < FN) look(gg.c[f + 1], lv[(f + 1) & 1]);
      const float* v = lv[f & 1];
      u32x4 w[2];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
        w[s2] = u32x4{pack_bf16x2(v[8 * s2 + 0] * a[f], v[8 * s2 + 1] * a[f]),
                      pack_bf16x2(v[8 * s2 + 2] * a[f], v[8 * s2 + 3] * a[f]),
                      pack_bf16x2(v[8 * s2 + 4] * a[f], v[8 * s2 + 5] * a[f]),
                      pack_bf16x2(v[8 * s2 + 6] * a[f], v[8 * s2 + 7] * a[f])};
#pragma unroll
      for (int i = 0; i < TF; ++i) {
        acc[f][i] = mfma16(gg.x[i][0], w[0], acc[f][i]);
        acc[f][i] = mfma16(gg.x[i][1], w[1], acc[f][i]);
      }
    }
  };

  __syncthreads();  // codebook and absmax in LDS
  {
    // load ring: tile t of the wave sits in g[t % D]; every step requests the
    // tile D - 1 ahead (clamped to the last tile: a redundant in-bounds load)
    int t = 0;
    for (; t + D <= nt; t += D) {
#pragma unroll
      for (int u = 0; u < D; ++u) {
        load(wb + min(t + u + D - 1, nt - 1), g[(u + D - 1) % D]);
        compute(wb + t + u, g[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < D - 1; ++u)
      if (t + u < nt) compute(wb + t + u, g[u]);
  }

  // ---- V = sum_z vpart[z] into LDS (summed in split order; after the main
  // loop so that its load latency does not delay the weight stream); the
  // first workgroup also writes it out (the forward keeps X A^T)
  if (lora_here) {
    // split z's partials are added in order z = 0, 1, ... for every entry;
    // the loads of 8 splits x 4 entries are issued together
    const int n = (int)p.M * p.r;
    for (int e0 = tid; e0 < n; e0 += 256 * 4) {
      float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      for (int z0 = 0; z0 < p.vsplits; z0 += 8) {
        float t[4][8];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int zz = 0; zz < 8; ++zz) {
            const int e = min(e0 + 256 * j, n - 1), z = min(z0 + zz, p.vsplits - 1);
            t[j][zz] = p.vpart[(int64_t)z * n + e];
          }
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int zz = 0; zz < 8; ++zz)
            if (z0 + zz < p.vsplits) v[j] += t[j][zz];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = e0 + 256 * j;
        if (e < n) {
          vs[e] = v[j];
          if (p.vout && blockIdx.x == 0) p.vout[e] = v[j];
        }
      }
    }
  }

  __syncthreads();

  // ---- LoRA term (wave 0): acc += (s V) Wl^T in steps of 32 ranks; s V is
  // rounded to bf16 like the other MFMA operands
  if (lora_here && wave == 0) {
    for (int j0 = 0; j0 < p.r; j0 += 32) {
      const int jq = j0 + 8 * q;  // this lane group's 8 ranks
      u32x4 va[TF];
#pragma unroll
      for (int i = 0; i < TF; ++i) {
        const int m = min(16 * i + l16, (int)p.M - 1);
        float y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = (jq + e < p.r) ? p.s * vs[m * p.r + jq + e] : 0.0f;
        va[i] = u32x4{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]),
                      pack_bf16x2(y[6], y[7])};
      }
#pragma unroll
      for (int f = 0; f < FN; ++f) {
        int64_t row = n0 + 16 * f + l16;
        if (row >= p.N) row = p.N - 1;
        uint32_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int j = jq + e;
          h[e] = j < p.r ? p.Wl[row * p.wl_sc + (int64_t)j * p.wl_sj] : 0u;
        }
        const u32x4 wb4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
#pragma unroll
        for (int i = 0; i < TF; ++i) acc[f][i] = mfma16(va[i], wb4, acc[f][i]);
      }
    }
  }

  // ---- sum the wave partials of each frag in wave order and store.
  // Value e = 256 i + 64 v + lane of a frag is token 16 i + 4 (lane/16) + v,
  // weight row n0 + 16 f + lane%16.
#pragma unroll
  for (int f = 0; f < FN; ++f) {
#pragma unroll
    for (int i = 0; i < TF; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) red[wave][256 * i + 64 * v + lane] = acc[f][i][v];
    __syncthreads();
#pragma unroll
    for (int h = 0; h < TF; ++h) {
      const int e = tid + 256 * h;
      float sum = 0.0f;
#pragma unroll
      for (int w = 0; w < SK_WAVES; ++w) sum += red[w][e];
      const int ln = e & 63;
      const int64_t m = 16 * (e >> 8) + 4 * (ln >> 4) + ((e >> 6) & 3);
      const int64_t n = n0 + 16 * f + (ln & 15);
      if (m < p.M && n < p.N) {
        if (p.part)
          p.part[((int64_t)blockIdx.y * p.M + m) * p.N + n] = sum;
        else
          p.out[m * p.N + n] = (uint16_t)(pack_bf16x2(sum, 0.0f) & 0xFFFFu);
      }
    }
    __syncthreads();
  }
}

template <int FN>
static hipError_t run_skinny_fwd(const SkinnyArgs& a, int splits, hipStream_t st) {
  dim3 grid((unsigned)((a.N + 16 * FN - 1) / (16 * FN)), (unsigned)splits);
  if (a.w.dq)
    skinny_fwd_kernel<FN, true><<<grid, 256, 0, st>>>(a);
  else
    skinny_fwd_kernel<FN, false><<<grid, 256, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace qk

using namespace qk;

bool skinny_fwd_supported(int64_t M, int r) { return M >= 1 && M <= 16 * SK_TF && r <= 64; }

hipError_t launch_skinny_fwd(const SkinnyArgs& a, const qplan::SkinnyPlan& pl, hipStream_t st) {
  if (!skinny_fwd_supported(a.M, a.r)) return hipErrorInvalidValue;
  switch (pl.fn) {
    case 1: return run_skinny_fwd<1>(a, pl.splits, st);
    case 2: return run_skinny_fwd<2>(a, pl.splits, st);
    case 4: return run_skinny_fwd<4>(a, pl.splits, st);
    case 7: return run_skinny_fwd<7>(a, pl.splits, st);
    case 8: return run_skinny_fwd<8>(a, pl.splits, st);
    default: return hipErrorInvalidValue;
  }
}
