// RMSNorm forward and hand-derived backward, the normalisation in front of
// the MLP block ("LLM Fine-Tuning in 2026: Unsloth vs QLoRA vs Liger-Kernel",
// the fused RMSNorm of section 2: one inverse RMS saved per row, no
// full-size intermediate):
//
//   rstd = 1 / sqrt(mean(x^2) + eps),  y = x * rstd * w
//   g = dy * w,  dx = rstd g - rstd^3 / D (sum g x) x,  dw = sum_rows dy x rstd
//
// HBM-bound row kernels: one wave per row, the row held in registers (D <=
// 8192), fp32 arithmetic, fixed-order butterfly sums (results reproducible).
#include <hip/hip_runtime.h>

#include "qlora_device.h"
#include "qlora_launch.h"

namespace qk {

constexpr int RN_BWD_WG = 256;  // workgroups of the backward (rows dealt round-robin)

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ void unpack8(const u32x4& p, float (&f)[8]) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    f[2 * d] = bf16_lo(p[d]);
    f[2 * d + 1] = bf16_hi(p[d]);
  }
}

__device__ __forceinline__ u32x4 pack8(const float (&f)[8]) {
  return u32x4{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7])};
}

// Forward: wave -> row.  Lane l holds the 16-byte chunks l + 64 c (c < NC) of
// the row, 8 elements each.
template <int NC>
__global__ __launch_bounds__(256) void rmsnorm_fwd_kernel(const uint16_t* __restrict__ X,
                                                          const uint16_t* __restrict__ w, int64_t M, int D,
                                                          float eps, uint16_t* __restrict__ Y,
                                                          float* __restrict__ rstd) {
  const int lane = threadIdx.x & 63;
  const int64_t m = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (m >= M) return;
  const int nch = D / 8;
  const uint16_t* xr = X + m * D;
  u32x4 xv[NC];
  float ss = 0.0f;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int ch = lane + 64 * c;
    xv[c] = ch < nch ? *reinterpret_cast<const u32x4*>(xr + 8 * ch) : u32x4{0u, 0u, 0u, 0u};
    float f[8];
    unpack8(xv[c], f);
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += f[e] * f[e];
  }
  ss = wave_sum(ss);
  const float r = 1.0f / sqrtf(ss / (float)D + eps);
  if (lane == 0) rstd[m] = r;
  if (!Y) return;  // rstd only (the norm folded into the next GEMM)
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int ch = lane + 64 * c;
    if (ch >= nch) break;
    float f[8], g[8];
    unpack8(xv[c], f);
    unpack8(*reinterpret_cast<const u32x4*>(w + 8 * ch), g);
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = f[e] * r * g[e];
    *reinterpret_cast<u32x4*>(Y + m * D + 8 * ch) = pack8(f);
  }
}

// Backward: RN_BWD_WG workgroups, wave v of workgroup b takes rows
// 4 b + v + 4 RN_BWD_WG k.  x, dy and w stay packed (bf16) in registers and
// are unpacked where used.  With DW each lane keeps the dw sums of its
// columns; at the end the 4 waves' sums are added in LDS in wave order and
// workgroup b writes part[b][D].
template <int NC, bool DW>
__global__ __launch_bounds__(256) void rmsnorm_bwd_kernel(const uint16_t* __restrict__ dY,
                                                          const uint16_t* __restrict__ X,
                                                          const uint16_t* __restrict__ w,
                                                          const float* __restrict__ rstd, int64_t M, int D,
                                                          uint16_t* __restrict__ dX, float* __restrict__ part) {
  __shared__ float red[DW ? 4 * 512 : 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nch = D / 8;
  u32x4 wv[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int ch = lane + 64 * c;
    wv[c] = ch < nch ? *reinterpret_cast<const u32x4*>(w + 8 * ch) : u32x4{0u, 0u, 0u, 0u};
  }
  float acc[DW ? NC : 1][8];
#pragma unroll
  for (int c = 0; c < (DW ? NC : 1); ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[c][e] = 0.0f;

  // widest rows (NC == 16): two passes over the row (the second re-reads x
  // and dy from cache) instead of holding them, to stay clear of spills
  constexpr bool TWO = NC >= 16;
  for (int64_t m = (int64_t)blockIdx.x * 4 + wave; m < M; m += 4 * (int64_t)gridDim.x) {
    const float r = rstd[m];
    if constexpr (TWO) {
      float s = 0.0f;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int ch = lane + 64 * c;
        if (ch >= nch) break;
        float xf[8], df[8], wf[8];
        unpack8(*reinterpret_cast<const u32x4*>(X + m * D + 8 * ch), xf);
        unpack8(*reinterpret_cast<const u32x4*>(dY + m * D + 8 * ch), df);
        unpack8(wv[c], wf);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          s += df[e] * wf[e] * xf[e];
          if constexpr (DW) acc[c][e] += df[e] * xf[e] * r;
        }
      }
      s = wave_sum(s);
      const float k = r * r * r / (float)D * s;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int ch = lane + 64 * c;
        if (ch >= nch) break;
        float xf[8], df[8], wf[8], o[8];
        unpack8(*reinterpret_cast<const u32x4*>(X + m * D + 8 * ch), xf);
        unpack8(*reinterpret_cast<const u32x4*>(dY + m * D + 8 * ch), df);
        unpack8(wv[c], wf);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = r * (df[e] * wf[e]) - k * xf[e];
        *reinterpret_cast<u32x4*>(dX + m * D + 8 * ch) = pack8(o);
      }
      continue;
    }
    u32x4 xv[NC], dv[NC];
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int ch = lane + 64 * c;
      const bool ok = ch < nch;
      xv[c] = ok ? *reinterpret_cast<const u32x4*>(X + m * D + 8 * ch) : u32x4{0u, 0u, 0u, 0u};
      dv[c] = ok ? *reinterpret_cast<const u32x4*>(dY + m * D + 8 * ch) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      float xf[8], df[8], wf[8];
      unpack8(xv[c], xf);
      unpack8(dv[c], df);
      unpack8(wv[c], wf);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        s += df[e] * wf[e] * xf[e];
        if constexpr (DW) acc[c][e] += df[e] * xf[e] * r;
      }
    }
    s = wave_sum(s);
    const float k = r * r * r / (float)D * s;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int ch = lane + 64 * c;
      if (ch >= nch) break;
      float xf[8], df[8], wf[8], o[8];
      unpack8(xv[c], xf);
      unpack8(dv[c], df);
      unpack8(wv[c], wf);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = r * (df[e] * wf[e]) - k * xf[e];
      *reinterpret_cast<u32x4*>(dX + m * D + 8 * ch) = pack8(o);
    }
  }

  if constexpr (DW) {
    // per 64-chunk column group c: the 4 waves' sums, added in wave order
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int ch = lane + 64 * c;
      __syncthreads();  // the previous group's reads are done
#pragma unroll
      for (int e = 0; e < 8; ++e) red[wave * 512 + lane * 8 + e] = acc[c][e];
      __syncthreads();
      if (wave == 0 && ch < nch) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          part[(int64_t)blockIdx.x * D + 8 * ch + e] =
              ((red[lane * 8 + e] + red[512 + lane * 8 + e]) + red[1024 + lane * 8 + e]) + red[1536 + lane * 8 + e];
      }
    }
  }
}

__global__ __launch_bounds__(256) void zero_f32_kernel(float* __restrict__ out, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) out[i] = 0.0f;
}

// dw[d] = sum over workgroups b < G of part[b][d] in a fixed order:
// workgroup -> 32 columns; thread (column c, part p) adds b = p, p + 8, ... in
// order, then the 8 sums are added in order of p.
__global__ __launch_bounds__(256) void rmsnorm_dw_finish_kernel(const float* __restrict__ part, int G, int D,
                                                                float* __restrict__ dw) {
  __shared__ float red[8][32];
  const int c = threadIdx.x & 31, p = threadIdx.x >> 5;
  const int d = blockIdx.x * 32 + c;
  float s = 0.0f;
  if (d < D) {
    int b = p;
    for (; b + 56 < G; b += 64) {  // 8 loads in flight, added in order
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = part[(int64_t)(b + 8 * u) * D + d];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; b < G; b += 8) s += part[(int64_t)b * D + d];
  }
  red[p][c] = s;
  __syncthreads();
  if (p == 0 && d < D) {
    float t = red[0][c];
#pragma unroll
    for (int k = 1; k < 8; ++k) t += red[k][c];
    dw[d] = t;
  }
}

template <int NC>
static hipError_t run_rmsnorm_bwd(const uint16_t* dY, const uint16_t* X, const uint16_t* w, const float* rstd,
                                  int64_t M, int D, uint16_t* dX, float* dw, float* part, hipStream_t st) {
  const int G = rmsnorm_bwd_groups(M);
  if (dw) {
    rmsnorm_bwd_kernel<NC, true><<<G, 256, 0, st>>>(dY, X, w, rstd, M, D, dX, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    rmsnorm_dw_finish_kernel<<<(D + 31) / 32, 256, 0, st>>>(part, G, D, dw);
  } else {
    rmsnorm_bwd_kernel<NC, false><<<G, 256, 0, st>>>(dY, X, w, rstd, M, D, dX, part);
  }
  return hipGetLastError();
}

}  // namespace qk

using namespace qk;

int rmsnorm_bwd_groups(int64_t M) {
  const int64_t g = (M + 3) / 4;
  return (int)(g < RN_BWD_WG ? (g > 0 ? g : 1) : RN_BWD_WG);
}

// out[j, k] = bf16(A[j, k] w[k]): a rank-r matrix with the norm weight folded in
__global__ __launch_bounds__(256) void scale_cols_kernel(const uint16_t* __restrict__ A, int64_t n, int64_t K,
                                                         const uint16_t* __restrict__ w, uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int64_t k = i % K;
  out[i] = (uint16_t)(pack_bf16x2(bf16_lo(A[i]) * bf16_lo(w[k]), 0.0f) & 0xFFFFu);
}

// out[m, j] = in[m, j] s[m]
__global__ __launch_bounds__(256) void scale_rows_kernel(const float* __restrict__ in, int64_t n, int r,
                                                         const float* __restrict__ s, float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  out[i] = in[i] * s[i / r];
}

static int rmsnorm_nc(int64_t D) {
  for (int nc = 1; nc <= 16; nc *= 2)
    if (512 * nc >= D) return nc;
  return 0;
}

hipError_t launch_scale_cols(const uint16_t* A, int64_t rows, int64_t K, const uint16_t* w, uint16_t* out,
                             hipStream_t st) {
  const int64_t n = rows * K;
  if (n == 0) return hipSuccess;
  scale_cols_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(A, n, K, w, out);
  return hipGetLastError();
}

hipError_t launch_scale_rows(const float* in, int64_t M, int r, const float* s, float* out, hipStream_t st) {
  const int64_t n = M * r;
  if (n == 0) return hipSuccess;
  scale_rows_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(in, n, r, s, out);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_fwd(const uint16_t* X, const uint16_t* w, int64_t M, int64_t D, float eps, uint16_t* Y,
                              float* rstd, hipStream_t st) {
  if (M == 0) return hipSuccess;
  const unsigned grid = (unsigned)((M + 3) / 4);
  switch (rmsnorm_nc(D)) {
    case 1: rmsnorm_fwd_kernel<1><<<grid, 256, 0, st>>>(X, w, M, (int)D, eps, Y, rstd); break;
    case 2: rmsnorm_fwd_kernel<2><<<grid, 256, 0, st>>>(X, w, M, (int)D, eps, Y, rstd); break;
    case 4: rmsnorm_fwd_kernel<4><<<grid, 256, 0, st>>>(X, w, M, (int)D, eps, Y, rstd); break;
    case 8: rmsnorm_fwd_kernel<8><<<grid, 256, 0, st>>>(X, w, M, (int)D, eps, Y, rstd); break;
    case 16: rmsnorm_fwd_kernel<16><<<grid, 256, 0, st>>>(X, w, M, (int)D, eps, Y, rstd); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_rmsnorm_bwd(const uint16_t* dY, const uint16_t* X, const uint16_t* w, const float* rstd,
                              int64_t M, int64_t D, uint16_t* dX, float* dw, float* part, hipStream_t st) {
  if (M == 0) {
    if (dw) zero_f32_kernel<<<(unsigned)((D + 255) / 256), 256, 0, st>>>(dw, D);
    return hipGetLastError();
  }
  switch (rmsnorm_nc(D)) {
    case 1: return run_rmsnorm_bwd<1>(dY, X, w, rstd, M, (int)D, dX, dw, part, st);
    case 2: return run_rmsnorm_bwd<2>(dY, X, w, rstd, M, (int)D, dX, dw, part, st);
    case 4: return run_rmsnorm_bwd<4>(dY, X, w, rstd, M, (int)D, dX, dw, part, st);
    case 8: return run_rmsnorm_bwd<8>(dY, X, w, rstd, M, (int)D, dX, dw, part, st);
    case 16: return run_rmsnorm_bwd<16>(dY, X, w, rstd, M, (int)D, dX, dw, part, st);
    default: return hipErrorInvalidValue;
  }
}
