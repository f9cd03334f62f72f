// Merge of a trained LoRA pair into one 16-bit weight (qlora_merge): the
// export step after training ("LLM Fine-Tuning in 2026: Unsloth vs QLoRA vs
// Liger-Kernel", the listing's 16-bit merge save; the update h = W0 x +
// (alpha/r) B A x of section 1 folded into the weight).
//
//   out[n, k] = round16(fp32(codebook[q] * absmax')[n, k] + s (B A)[n, k])
//
// HBM-bound: per weight element 0.5 B of codes (+ absmax) read and 2 B
// written; the rank-r product B A comes from the matrix cores.
#include <hip/hip_runtime.h>

#include "qlora_device.h"
#include "qlora_gemm_common.h"
#include "qlora_launch.h"

namespace qk {

// ------------------------------------------------------------------------
// Workgroup: 128 weight rows x MG_COLS columns, 4 waves of 32 rows.  Per 32 x 32
// tile the matrix cores give C[k][n] = sum_j A[j][k] B[n][j] over ceil(r/16)
// v_mfma_f32_32x32x16_bf16 steps (j past r is zero on both operands).
// Accumulator v of lane l is then column k0 + 8(v/4) + 4(l/32) + v%4 of row
// n0 + l%32, i.e. of the lane's own row, whose code bytes and absmax values
// for the MG_COLS columns the lane loads up front.  A's columns are staged
// once per workgroup in LDS, transposed (A^T rows of 16-byte rank chunks),
// so that each MFMA A operand is one 16-byte LDS read.  The 16-bit results go to a
// per-wave LDS tile (rows padded by 16 bytes) and leave as whole row segments
// (2 * MG_COLS bytes), several rows per store instruction.
// ------------------------------------------------------------------------
constexpr int MG_COLS = 256;          // columns per workgroup
constexpr int MG_LD = MG_COLS + 8;    // LDS row stride of the [32][MG_COLS] output tile, elements
constexpr int MG_T = MG_COLS / 32;    // 32-column MFMA steps
constexpr int MG_CH = MG_COLS / 8;    // 16-byte chunks per output row
constexpr int MG_NB = 4;              // column blocks per workgroup

template <bool F16>
__global__ __launch_bounds__(256) void merge_kernel(Nf4Dev w, const float* __restrict__ codebook,
                                                    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
                                                    int r, float s, uint16_t* __restrict__ out) {
  __shared__ float cb[16];
  __shared__ __attribute__((aligned(16))) uint16_t tile[4][32 * MG_LD];
  // A^T of the current column block, [MG_COLS][16 JS + 8] (ranks past r
  // zero; the 16-byte pad keeps the 8-lane passes of the 16-byte reads and
  // writes on distinct banks): dynamic, 16 JS + 8 elements per column
  extern __shared__ __attribute__((aligned(16))) uint16_t at[];
  if (threadIdx.x < 16) cb[threadIdx.x] = codebook[threadIdx.x];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int64_t N = w.N, K = w.K;
  const int64_t nw = (int64_t)blockIdx.x * 128 + 32 * wave;  // the wave's first row
  const int64_t n = nw + l32;                                  // the lane's row
  const int64_t nr = n < N ? n : N - 1;
  const int JS = (r + 15) / 16;                               // 16-wide steps over the rank, <= 8
  const int ald = 16 * JS + 8;                                 // A^T row stride, elements
  uint16_t* T = tile[wave];
  // column blocks b0, b0 + 1, ... of this workgroup
  const int64_t nblk = (K + MG_COLS - 1) / MG_COLS;
  const int64_t b0 = (int64_t)blockIdx.y * MG_NB;
  const int64_t b1 = (b0 + MG_NB) < nblk ? (b0 + MG_NB) : nblk;

  // B operand of step js: lane (l32, g) holds B[nr][16 js + 8 g + i], i < 8 (0 past r)
  u32x4 bop[8];
#pragma unroll
  for (int js = 0; js < 8; ++js) {
    uint32_t h[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = 16 * js + 8 * g + i;
      h[i] = (js < JS && j < r) ? (uint32_t)B[nr * r + j] : 0u;
    }
    bop[js] = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
  }

  // the row's codes (32 columns per 16 bytes) and absmax (64 columns each) of
  // one block; the next block's are requested while this one is computed
  u32x4 cw[MG_T], cwn[MG_T];
  float am[MG_T / 2], amn[MG_T / 2];
  auto load_codes = [&](int64_t blk, u32x4 (&c)[MG_T], float (&a)[MG_T / 2]) {
    const int64_t kb = blk * MG_COLS;
    const int nc = (int)((K - kb) < MG_COLS ? (K - kb) : MG_COLS);
#pragma unroll
    for (int t = 0; t < MG_T; ++t)
      c[t] = 32 * t < nc ? *reinterpret_cast<const u32x4*>(w.codes + nr * (K / 2) + (kb + 32 * t) / 2)
                         : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int b = 0; b < MG_T / 2; ++b) {
      const int64_t bl = (nr * K + kb + 64 * (64 * b < nc ? b : 0)) / 64;
      a[b] = w.dq ? absmax_at<true>(w, bl) : absmax_at<false>(w, bl);
    }
  };
  if (b0 < b1) load_codes(b0, cw, am);

  for (int64_t blk = b0; blk < b1; ++blk) {
    const int64_t kb = blk * MG_COLS;
    const int ncols = (int)((K - kb) < MG_COLS ? (K - kb) : MG_COLS);  // multiple of 64
    if (blk + 1 < b1) load_codes(blk + 1, cwn, amn);
    __syncthreads();  // every wave is done reading the previous block's A^T
    {
      // thread c: column kb + c of A, 8 ranks per 16-byte LDS store
      const int c = threadIdx.x;
      const bool cok = c < ncols;
      for (int h = 0; h < 2 * JS; ++h) {
        uint32_t v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int j = 8 * h + i;
          v[i] = (cok && j < r) ? (uint32_t)A[(int64_t)j * K + kb + c] : 0u;
        }
        *reinterpret_cast<u32x4*>(at + c * ald + 8 * h) =
            u32x4{v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16), v[6] | (v[7] << 16)};
      }
    }
    __syncthreads();

#pragma unroll
    for (int t = 0; t < MG_T; ++t) {
      if (32 * t >= ncols) break;
      // A operand of step js: lane (l32, g) holds A[16 js + 8 g + i][kb + 32 t + l32]
      f32x16 acc;
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
#pragma unroll
      for (int js = 0; js < 8; ++js) {
        if (js >= JS) break;
        const u32x4 aop = *reinterpret_cast<const u32x4*>(at + (32 * t + l32) * ald + 16 * js + 8 * g);
        acc = mfma32(aop, bop[js], acc);
      }
      const float a = am[t >> 1];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        // columns 32 t + 8 q4 + 4 g + b: nibbles 16 g + 4 b of code dword q4
        float x[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const float d = cb[(cw[t][q4] >> (16 * g + 4 * b)) & 15u] * a;
          x[b] = d + s * acc[4 * q4 + b];
        }
        uint32_t p0, p1;
        if constexpr (F16) {
          p0 = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x[0]) |
               ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x[1]) << 16);
          p1 = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x[2]) |
               ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x[3]) << 16);
        } else {
          p0 = pack_bf16x2(x[0], x[1]);
          p1 = pack_bf16x2(x[2], x[3]);
        }
        *reinterpret_cast<u32x2*>(T + l32 * MG_LD + 32 * t + 8 * q4 + 4 * g) = u32x2{p0, p1};
      }
    }
    // the wave reads back only its own tile: LDS operations of a wave complete
    // in order, so no barrier is needed
    constexpr int RPI = 64 / MG_CH;  // rows per store instruction
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int row = RPI * i + lane / MG_CH, ch = lane % MG_CH;  // 16-byte chunk ch of the row
      if (8 * ch < ncols && nw + row < N)
        *reinterpret_cast<u32x4*>(out + (nw + row) * K + kb + 8 * ch) =
            *reinterpret_cast<const u32x4*>(T + row * MG_LD + 8 * ch);
    }
#pragma unroll
    for (int t = 0; t < MG_T; ++t) cw[t] = cwn[t];
#pragma unroll
    for (int b = 0; b < MG_T / 2; ++b) am[b] = amn[b];
  }
}

}  // namespace qk

using namespace qk;

hipError_t launch_merge(const Nf4Dev& w, const float* codebook, const uint16_t* A, const uint16_t* B, int r,
                        float s, int f16, uint16_t* out, hipStream_t st) {
  if (w.N == 0 || w.K == 0) return hipSuccess;
  if (r < 1 || r > 128 || w.K % 64 != 0) return hipErrorInvalidValue;
  const int64_t nblk = (w.K + MG_COLS - 1) / MG_COLS;
  const dim3 grid((unsigned)((w.N + 127) / 128), (unsigned)((nblk + MG_NB - 1) / MG_NB));
  const size_t at_bytes = (size_t)MG_COLS * (16 * ((r + 15) / 16) + 8) * 2;
  if (f16)
    merge_kernel<true><<<grid, 256, at_bytes, st>>>(w, codebook, A, B, r, s, out);
  else
    merge_kernel<false><<<grid, 256, at_bytes, st>>>(w, codebook, A, B, r, s, out);
  return hipGetLastError();
}
