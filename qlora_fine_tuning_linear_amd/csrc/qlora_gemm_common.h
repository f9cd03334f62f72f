// Tile geometry, mode traits and the shared epilogue of the MFMA GEMM
// kernels (the dequant-staged qgemm_kernel and the bf16-staged
// bgemm_kernel): LoRA term as extra MFMA steps on the accumulators, split
// partials, and the stores with the SwiGLU forward / backward variants.
#pragma once

#include "qlora_device.h"
#include "qlora_launch.h"

namespace qk {

// Absmax of NF4 block `blk`: fp32, or with double quantization the 8-bit code
// times the fp32 scale of its group of 256 blocks.
template <bool DQ>
__device__ __forceinline__ float absmax_at(const Nf4Dev& w, int64_t blk) {
  if constexpr (DQ) return (float)w.absmax_q[blk] * w.absmax_scale[blk >> 8];
  return w.absmax[blk];
}

// Expand 8 codes of one block into 8 bf16 values (4 packed dwords).
__device__ __forceinline__ u32x4 deq8(uint32_t c, float a, const float* cb) {
  u32x4 o;
  o[0] = pack_bf16x2(cb[c & 15u] * a, cb[(c >> 4) & 15u] * a);
  o[1] = pack_bf16x2(cb[(c >> 8) & 15u] * a, cb[(c >> 12) & 15u] * a);
  o[2] = pack_bf16x2(cb[(c >> 16) & 15u] * a, cb[(c >> 20) & 15u] * a);
  o[3] = pack_bf16x2(cb[(c >> 24) & 15u] * a, cb[(c >> 28) & 15u] * a);
  return o;
}

template <int MODE>
struct ModeTraits {
  static constexpr bool trans = (MODE == MODE_BWD || MODE == MODE_BWD_SWIGLU || MODE == MODE_BWD_DUAL);
  static constexpr bool swiglu_fwd = (MODE == MODE_FWD_SWIGLU);
};

template <int WM, int WN, int FM, int FN>
struct TileCfg {
  static constexpr int NT = WM * WN * 64;
  static constexpr int BM = WM * FM * 32;
  static constexpr int BN = WN * FN * 32;
  static constexpr int EPT = 64 * BN / NT;  // forward fill: elements per thread
  static constexpr int TPR = 64 / EPT;      // forward fill: threads per LDS row
  static constexpr int RPT = 8 * BN / NT;   // transposed fill: weight rows per thread
};

// LDS row (= output column within the tile) of frag f of wave column wn.
template <int MODE, int WN, int FN>
__device__ __forceinline__ int frag_row(int wn, int f) {
  if (ModeTraits<MODE>::swiglu_fwd) {
    constexpr int H = FN / 2;
    constexpr int BNH = WN * H * 32;
    return (f < H) ? (wn * H + f) * 32 : BNH + (wn * H + (f - H)) * 32;
  }
  return (wn * FN + f) * 32;
}

// Output column of lane-row l32 in output frag f of wave column wn (for the
// SwiGLU forward, frags f and f + FN/2 are the gate and up columns of the
// same intermediate column).
template <int MODE, int WN, int FN>
__device__ __forceinline__ int64_t out_col_of(int64_t n0, int wn, int f) {
  if (ModeTraits<MODE>::swiglu_fwd) {
    constexpr int H = FN / 2;
    return n0 + (int64_t)(wn * H + (f % H)) * 32;
  }
  return n0 + (int64_t)frag_row<MODE, WN, FN>(wn, f);
}

// LoRA term acc += s * V[m, :] Wl(col, :)^T as extra MFMA steps (rank r in
// steps of 16; s V rounded to bf16), done before the main reduction.
//
// Fast form (r a multiple of 8 and Wl rows contiguous in j, wl_sj == 1): the
// operands of a step are 16-byte vector loads (per lane two of V, one of Wl
// per frag), issued by lora_load; lora_apply packs and multiplies.  Callers
// issue step 0's loads before their own prologue loads so that the LoRA
// latency hides behind them.  Otherwise gemm_lora_scalar: clamped scalar
// loads, all issued before any use.
template <int FM, int FN>
struct LoraRegs {
  u32x4 v[FM][2];  // fp32 V[token][j .. j+7]
  u32x4 h[FN];     // bf16 Wl[col][j .. j+7]
};

__device__ __forceinline__ bool lora_fast(const LoraSide& L) { return (L.r & 7) == 0 && L.wl_sj == 1; }

template <int MODE, int WN, int FM, int FN>
__device__ __forceinline__ void lora_load(const GemmArgs& p, const LoraSide& L, int t, const int64_t (&arow)[FM],
                                          int64_t n0, int wn, int l32, int g, LoraRegs<FM, FN>& R) {
  int j0 = 16 * t + 8 * g;
  if (j0 > L.r - 8) j0 = L.r - 8;  // out-of-range group: any valid address, masked in lora_apply
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const u32x4* src = reinterpret_cast<const u32x4*>(L.V + arow[i] * L.r + j0);
    R.v[i][0] = src[0];
    R.v[i][1] = src[1];
  }
#pragma unroll
  for (int f = 0; f < FN; ++f) {
    int64_t c = out_col_of<MODE, WN, FN>(n0, wn, f) + l32;
    if (c >= p.Nout) c = p.Nout - 1;
    R.h[f] = *reinterpret_cast<const u32x4*>(L.Wl + c * L.wl_sc + j0);
  }
}

template <int FM, int FN>
__device__ __forceinline__ void lora_apply(const LoraSide& L, int t, int g, int f_lo, int f_hi,
                                           f32x16 (&acc)[FM][FN], const LoraRegs<FM, FN>& R) {
  const bool ok = 16 * t + 8 * g < L.r;
  u32x4 vop[FM];
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = ok ? L.s * __uint_as_float(R.v[i][e >> 2][e & 3]) : 0.0f;
    vop[i] = u32x4{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]),
                   pack_bf16x2(y[6], y[7])};
  }
#pragma unroll
  for (int f = 0; f < FN; ++f) {
    if (f < f_lo || f >= f_hi) continue;
    const u32x4 wop = ok ? R.h[f] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < FM; ++i) acc[i][f] = mfma32(wop, vop[i], acc[i][f]);
  }
}

template <int MODE, int WN, int FM, int FN>
__device__ __forceinline__ void lora_scalar(const GemmArgs& p, const LoraSide& L, int t0, f32x16 (&acc)[FM][FN],
                                            const int64_t (&arow)[FM], int64_t n0, int wn, int l32, int g, int f_lo,
                                            int f_hi) {
  const int steps = (L.r + 15) / 16;
  for (int t = t0; t < steps; ++t) {
    float x[FM][8];
    uint32_t h[FN][8];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = 16 * t + 8 * g + e;
        x[i][e] = L.V[arow[i] * L.r + (j < L.r ? j : L.r - 1)];
      }
#pragma unroll
    for (int f = 0; f < FN; ++f) {
      int64_t c = out_col_of<MODE, WN, FN>(n0, wn, f) + l32;
      if (c >= p.Nout) c = p.Nout - 1;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = 16 * t + 8 * g + e;
        h[f][e] = L.Wl[c * L.wl_sc + (int64_t)(j < L.r ? j : L.r - 1) * L.wl_sj];
      }
    }
    u32x4 vop[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = (16 * t + 8 * g + e < L.r) ? L.s * x[i][e] : 0.0f;
      vop[i] = u32x4{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]),
                     pack_bf16x2(y[6], y[7])};
    }
#pragma unroll
    for (int f = 0; f < FN; ++f) {
      if (f < f_lo || f >= f_hi) continue;
      uint32_t hh[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) hh[e] = (16 * t + 8 * g + e < L.r) ? h[f][e] : 0u;
      const u32x4 wop{hh[0] | (hh[1] << 16), hh[2] | (hh[3] << 16), hh[4] | (hh[5] << 16), hh[6] | (hh[7] << 16)};
#pragma unroll
      for (int i = 0; i < FM; ++i) acc[i][f] = mfma32(wop, vop[i], acc[i][f]);
    }
  }
}

// The LoRA sides of a mode: (side, output frags it adds to).  Split runs add
// the LoRA term in split 0 only.
template <int MODE, int FN, bool SPLIT>
__device__ __forceinline__ int lora_sides(const GemmArgs& p, const LoraSide* (&L)[2], int (&lo)[2], int (&hi)[2]) {
  if constexpr (MODE == MODE_FWD_SWIGLU) {
    L[0] = &p.l0; lo[0] = 0; hi[0] = FN / 2;
    L[1] = &p.l1; lo[1] = FN / 2; hi[1] = FN;
    return 2;
  } else if constexpr (MODE == MODE_BWD_DUAL) {
    L[0] = &p.l0; lo[0] = 0; hi[0] = FN;
    L[1] = &p.l1; lo[1] = 0; hi[1] = FN;
    return 2;
  } else {
    L[0] = &p.l0; lo[0] = 0; hi[0] = FN;
    L[1] = &p.l0; lo[1] = 0; hi[1] = 0;
    return (!SPLIT || blockIdx.y == 0) ? 1 : 0;
  }
}

// The whole LoRA term in one call (loads, then use).
template <int MODE, int WN, int FM, int FN, bool SPLIT>
__device__ __forceinline__ void gemm_lora(const GemmArgs& p, f32x16 (&acc)[FM][FN], const int64_t (&arow)[FM],
                                          int64_t n0, int wn, int l32, int g) {
  const LoraSide* L[2];
  int lo[2], hi[2];
  const int ns = lora_sides<MODE, FN, SPLIT>(p, L, lo, hi);
  for (int k = 0; k < ns; ++k) lora_scalar<MODE, WN, FM, FN>(p, *L[k], 0, acc, arow, n0, wn, l32, g, lo[k], hi[k]);
}

// Stores of one output tile.  acc[i][f]: token frag i (rows
// m0 + (wm*FM + i)*32 + l32, clamped copy in arow[i]) x output frag f of wave
// column wn; element v of lane (l32, g) is output column
// out_col(f) + 8*(v/4) + 4*g + v%4.
template <int MODE, int WM, int WN, int FM, int FN, bool SPLIT>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs& p, f32x16 (&acc)[FM][FN], const int64_t (&arow)[FM],
                                              int64_t m0, int64_t n0, int wm, int wn, int l32, int g) {
  auto out_col = [&](int f) -> int64_t { return out_col_of<MODE, WN, FN>(n0, wn, f); };
  {
    if constexpr (SPLIT) {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int64_t m = m0 + (int64_t)(wm * FM + i) * 32 + l32;
        if (m >= p.M) continue;
#pragma unroll
        for (int f = 0; f < FN; ++f) {
          const int64_t cb0 = out_col(f);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int64_t n = cb0 + 8 * q + 4 * g;
            if (n >= p.Nout) continue;
            f32x4 o{acc[i][f][4 * q], acc[i][f][4 * q + 1], acc[i][f][4 * q + 2], acc[i][f][4 * q + 3]};
            *reinterpret_cast<f32x4*>(p.partial + ((int64_t)blockIdx.y * p.M + m) * p.Nout + n) = o;
          }
        }
      }
      return;
    }

    // ---- SwiGLU backward: the G / U loads of token frag i+1 are issued
    // before frag i is computed and stored (one exposed memory latency per
    // tile); columns past Nout load a clamped address and are not stored.
    if constexpr (MODE == MODE_BWD_SWIGLU) {
      u32x2 gg[2][FN][4], uu[2][FN][4];
      auto load = [&](int i, int b) {
#pragma unroll
        for (int f = 0; f < FN; ++f)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            int64_t n = out_col(f) + 8 * q + 4 * g;
            if (n >= p.Nout) n = p.Nout - 4;
            gg[b][f][q] = *reinterpret_cast<const u32x2*>(p.in0 + arow[i] * p.Nout + n);
            uu[b][f][q] = *reinterpret_cast<const u32x2*>(p.in1 + arow[i] * p.Nout + n);
          }
      };
      load(0, 0);
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        if (i + 1 < FM) load(i + 1, (i + 1) & 1);
        const int b = i & 1;
        const int64_t m = m0 + (int64_t)(wm * FM + i) * 32 + l32;
        if (m >= p.M) continue;
#pragma unroll
        for (int f = 0; f < FN; ++f)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int64_t n = out_col(f) + 8 * q + 4 * g;
            if (n >= p.Nout) continue;
            const int64_t off = m * p.Nout + n;
            const float G[4] = {bf16_lo(gg[b][f][q][0]), bf16_hi(gg[b][f][q][0]), bf16_lo(gg[b][f][q][1]),
                                bf16_hi(gg[b][f][q][1])};
            const float U[4] = {bf16_lo(uu[b][f][q][0]), bf16_hi(uu[b][f][q][0]), bf16_lo(uu[b][f][q][1]),
                                bf16_hi(uu[b][f][q][1])};
            float dG[4], dU[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float dH = acc[i][f][4 * q + e];
              const float sg = sigmoid_fast(G[e]);
              dU[e] = dH * G[e] * sg;
              dG[e] = dH * U[e] * sg * (1.0f + G[e] * (1.0f - sg));
            }
            *reinterpret_cast<u32x2*>(p.out0 + off) = u32x2{pack_bf16x2(dG[0], dG[1]), pack_bf16x2(dG[2], dG[3])};
            *reinterpret_cast<u32x2*>(p.out1 + off) = u32x2{pack_bf16x2(dU[0], dU[1]), pack_bf16x2(dU[2], dU[3])};
          }
      }
      return;
    }

    // ---- stores
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int64_t m = m0 + (int64_t)(wm * FM + i) * 32 + l32;
      if (m >= p.M) continue;
      constexpr int FO = ModeTraits<MODE>::swiglu_fwd ? FN / 2 : FN;
#pragma unroll
      for (int f = 0; f < FO; ++f) {
        const int64_t cb0 = out_col(f);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t n = cb0 + 8 * q + 4 * g;
          if (n >= p.Nout) continue;
          const int64_t off = m * p.Nout + n;
          if constexpr (MODE == MODE_FWD_SWIGLU) {
            float G[4], U[4], H[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              G[e] = acc[i][f][4 * q + e];
              U[e] = acc[i][f + FN / 2][4 * q + e];
              H[e] = G[e] * sigmoid_fast(G[e]) * U[e];
            }
            *reinterpret_cast<u32x2*>(p.out0 + off) = u32x2{pack_bf16x2(G[0], G[1]), pack_bf16x2(G[2], G[3])};
            *reinterpret_cast<u32x2*>(p.out1 + off) = u32x2{pack_bf16x2(U[0], U[1]), pack_bf16x2(U[2], U[3])};
            *reinterpret_cast<u32x2*>(p.out2 + off) = u32x2{pack_bf16x2(H[0], H[1]), pack_bf16x2(H[2], H[3])};
          } else {
            const f32x16& a = acc[i][f];
            *reinterpret_cast<u32x2*>(p.out0 + off) =
                u32x2{pack_bf16x2(a[4 * q], a[4 * q + 1]), pack_bf16x2(a[4 * q + 2], a[4 * q + 3])};
          }
        }
      }
    }
  }
}

}  // namespace qk
