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

#include <algorithm>

#include "qlora_device.h"
#include "qlora_gemm_common.h"
#include "qlora_launch.h"

namespace qk {

// ------------------------------------------------------------------------
// Workgroup: one block of MG_COLS columns, walking `nb` blocks of 128 weight
// rows (4 waves of 32 rows).  Per 32 x 32 tile the matrix cores give
// C[k][n] = sum_j A[j][k] B[n][j] over ceil(r/16) v_mfma_f32_32x32x16_bf16
// steps (j past r is zero on both operands).  Accumulator v of lane l is then
// column k0 + 8(v/4) + 4(l/32) + v%4 of row n0 + l%32, i.e. of the lane's own
// row, whose code bytes, absmax values and B row the lane loads one row block
// ahead.  A's columns are staged once per workgroup in LDS, transposed (A^T
// rows of 16-byte rank chunks), so that each MFMA A operand is one 16-byte LDS
// read.  The 16-bit results go to a per-wave LDS tile (rows padded by 16
// bytes) and leave as whole row segments (2 * MG_COLS bytes), four rows per
// non-temporal store instruction.  Every global load and store of the
// row-block loop is a buffer operation without a branch: rows past N and
// columns past K fall outside the buffer ranges, so loads there read zeros and
// stores there are dropped.  The number of memory operations in flight is
// then the same on every path, and the wait for one block's operands leaves
// the next block's loads and the previous block's stores in flight.
// ------------------------------------------------------------------------
constexpr int MG_COLS = 128;          // columns per workgroup
constexpr int MG_LD = MG_COLS + 8;    // LDS row stride of the [32][MG_COLS] output tile, elements
constexpr int MG_T = MG_COLS / 32;    // 32-column MFMA steps
constexpr int MG_CH = MG_COLS / 8;    // 16-byte chunks per output row
constexpr uint32_t MG_OFF = 0x80000000u;  // a buffer offset past every range
constexpr int64_t MG_TARGET_WG = 768;   // workgroups aimed for (three per CU)
// cache policy of the output stores: non-temporal (the merged weight is not
// read back by this pass; 35 us against 45.8 us with the default policy on the
// 14336 x 4096 weight)
constexpr int MG_NT = 2;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t mg_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// JSX: 16-wide rank steps provided for (r <= 16 JSX); BV: B rows load as
// 16-byte chunks (r % 8 == 0), else element by element; F16: fp16 output, else bf16
template <int JSX, bool DQ, bool BV, bool F16>
__global__ __launch_bounds__(256) void merge_kernel(Nf4Dev w, const float* __restrict__ codebook,
                                                    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
                                                    int r, float s, int nb, uint16_t* __restrict__ out) {
  __shared__ float cb[16];
  __shared__ __attribute__((aligned(16))) uint16_t tile[4][32 * MG_LD];
  // A^T of the column block, [MG_COLS][16 JS + 8] (ranks past r zero; the
  // 16-byte pad keeps the 8-lane passes of the 16-byte reads on distinct
  // banks): dynamic, 16 JS + 8 elements per column
  extern __shared__ __attribute__((aligned(16))) uint16_t at[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int64_t N = w.N, K = w.K;
  const int JS = (r + 15) / 16;  // <= JSX
  const int ald = 16 * JS + 8;   // A^T row stride, elements
  const int64_t kb = (int64_t)blockIdx.x * MG_COLS;
  const int ncols = (int)((K - kb) < MG_COLS ? (K - kb) : MG_COLS);  // 64 or 128
  const int64_t nrb = (N + 127) / 128;
  const int64_t rb0 = (int64_t)blockIdx.y * nb;
  const int64_t rb1 = (rb0 + nb) < nrb ? (rb0 + nb) : nrb;
  uint16_t* T = tile[wave];

  // one row block's per-lane operands: codes (32 columns per 16 bytes), the
  // absmax blocks, the B row as MFMA B operands
  struct Blk {
    u32x4 c[MG_T];
    float am[MG_T / 2];
    uint32_t aq[MG_T / 2];
    float sc[MG_T / 2];
    u32x4 b[JSX];
  };
  const int lrow = 32 * wave + l32;  // the lane's row within a row block
  auto load_blk = [&](int64_t rb, Blk& d) __attribute__((always_inline)) {
    const int64_t n0 = rb * 128;
    const int64_t nrows = (N - n0) < 128 ? (N - n0) : 128;
    const __amdgpu_buffer_rsrc_t crs = mg_rsrc(w.codes + n0 * (K / 2), nrows * (K / 2));
#pragma unroll
    for (int t = 0; t < MG_T; ++t)
      d.c[t] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(crs, (uint32_t)(lrow * (K / 2) + (kb + 32 * t) / 2), 0, 0));
    const int64_t kblk = K / 64;
    const int64_t blk0 = n0 * kblk;  // first absmax block of the row block
    const uint32_t lb = (uint32_t)(lrow * kblk + kb / 64);
    if constexpr (DQ) {
      const __amdgpu_buffer_rsrc_t ars = mg_rsrc(w.absmax_q + blk0, nrows * kblk);
      // the scales from the row block's first group to the end of the array
      const __amdgpu_buffer_rsrc_t srs =
          mg_rsrc(w.absmax_scale + (blk0 >> 8), ((N * kblk + 255) / 256 - (blk0 >> 8)) * 4);
#pragma unroll
      for (int b = 0; b < MG_T / 2; ++b) {
        d.aq[b] = __builtin_amdgcn_raw_buffer_load_b8(ars, lb + b, 0, 0);
        d.sc[b] = __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(srs, (uint32_t)((((blk0 & 255) + lb + b) >> 8) * 4), 0, 0));
      }
    } else {
      const __amdgpu_buffer_rsrc_t ars = mg_rsrc(w.absmax + blk0, nrows * kblk * 4);
#pragma unroll
      for (int b = 0; b < MG_T / 2; ++b)
        d.am[b] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ars, (lb + b) * 4, 0, 0));
    }
    // lane (l32, g), step js: B[n][16 js + 8 g + i], i < 8
    const __amdgpu_buffer_rsrc_t brs = mg_rsrc(B + n0 * r, nrows * r * 2);
#pragma unroll
    for (int js = 0; js < JSX; ++js) {
      const int j0 = 16 * js + 8 * g;
      if constexpr (BV) {
        const uint32_t o = j0 < r ? (uint32_t)((lrow * r + j0) * 2) : MG_OFF;
        d.b[js] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(brs, o, 0, 0));
      } else {
        uint32_t h[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t o = j0 + i < r ? (uint32_t)((lrow * r + j0 + i) * 2) : MG_OFF;
          h[i] = __builtin_amdgcn_raw_buffer_load_b16(brs, o, 0, 0);
        }
        d.b[js] = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
      }
    }
  };

  auto step = [&](int64_t rb, const Blk& d) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < MG_T; ++t) {
      if (32 * t >= ncols) break;
      // A operand of step js: lane (l32, g) holds A[16 js + 8 g + i][kb + 32 t + l32]
      f32x16 acc;
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[v] = 0.0f;
#pragma unroll
      for (int js = 0; js < JSX; ++js) {
        if (js >= JS) break;
        const u32x4 aop = *reinterpret_cast<const u32x4*>(at + (32 * t + l32) * ald + 16 * js + 8 * g);
        acc = mfma32(aop, d.b[js], acc);
      }
      const float a = DQ ? (float)d.aq[t >> 1] * d.sc[t >> 1] : d.am[t >> 1];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        // columns 32 t + 8 q4 + 4 g + b: nibbles 16 g + 4 b of code dword q4
        float x[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const float dv = cb[(d.c[t][q4] >> (16 * g + 4 * b)) & 15u] * a;
          x[b] = dv + s * acc[4 * q4 + b];
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
    const int64_t n0 = rb * 128;
    const int64_t nrows = (N - n0) < 128 ? (N - n0) : 128;
    const __amdgpu_buffer_rsrc_t ors = mg_rsrc(out + n0 * K, nrows * K * 2);
    constexpr int RPI = 64 / MG_CH;  // rows per store instruction
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int row = RPI * i + lane / MG_CH, ch = lane % MG_CH;  // 16-byte chunk ch of the row
      const uint32_t o = 8 * ch < ncols ? (uint32_t)(((32 * wave + row) * K + kb + 8 * ch) * 2) : MG_OFF;
      __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const u32x4*>(T + row * MG_LD + 8 * ch), ors, o, 0,
                                             MG_NT);
    }
  };

  // row blocks two at a time through two operand sets, each loaded one block
  // ahead (past the end the last block is loaded again); the first block's
  // operands are requested before A^T is staged
  Blk b0, b1;
  load_blk(rb0, b0);
  if (tid < 16) cb[tid] = codebook[tid];
  {
    // (rank j, 8-column chunk ch) pairs; ranks past r and chunks past K read
    // a valid address and store zeros
    for (int idx = tid; idx < 16 * JS * MG_CH; idx += 256) {
      const int j = idx / MG_CH, ch = idx % MG_CH;
      const bool ok = j < r && 8 * ch < ncols;
      const uint16_t* src = A + (int64_t)(ok ? j : 0) * K + kb + (ok ? 8 * ch : 0);
      uint16_t v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = src[i];
#pragma unroll
      for (int i = 0; i < 8; ++i) at[(8 * ch + i) * ald + j] = ok ? v[i] : (uint16_t)0;
    }
  }
  __syncthreads();
  for (int64_t rb = rb0; rb < rb1; rb += 2) {
    load_blk((rb + 1) < rb1 ? rb + 1 : rb1 - 1, b1);
    step(rb, b0);
    if (rb + 1 >= rb1) break;
    load_blk((rb + 2) < rb1 ? rb + 2 : rb1 - 1, b0);
    step(rb + 1, b1);
  }
}

}  // namespace qk

using namespace qk;

hipError_t launch_merge(const Nf4Dev& w, const float* codebook, const uint16_t* A, const uint16_t* B, int r,
                        float s, int f16, uint16_t* out, hipStream_t st) {
  if (w.N == 0 || w.K == 0) return hipSuccess;
  if (r < 1 || r > 128 || w.K % 64 != 0) return hipErrorInvalidValue;
  const int64_t ncb = (w.K + MG_COLS - 1) / MG_COLS, nrb = (w.N + 127) / 128;
  // row blocks per workgroup: about MG_TARGET_WG workgroups in all
  const int64_t nb = std::max<int64_t>(1, (ncb * nrb + MG_TARGET_WG - 1) / MG_TARGET_WG);
  const dim3 grid((unsigned)ncb, (unsigned)((nrb + nb - 1) / nb));
  const int js = (r + 15) / 16;
  const size_t at_bytes = (size_t)MG_COLS * (16 * js + 8) * 2;
  const bool dq = w.dq != 0, bv = r % 8 == 0;
#define MG_LAUNCH(JSX, DQ, BV)                                                                             \
  if (f16) merge_kernel<JSX, DQ, BV, true><<<grid, 256, at_bytes, st>>>(w, codebook, A, B, r, s, (int)nb, out); \
  else merge_kernel<JSX, DQ, BV, false><<<grid, 256, at_bytes, st>>>(w, codebook, A, B, r, s, (int)nb, out)
#define MG_BV(JSX, DQ) \
  if (bv) { MG_LAUNCH(JSX, DQ, true); } else { MG_LAUNCH(JSX, DQ, false); }
#define MG_DQ(JSX) \
  if (dq) { MG_BV(JSX, true); } else { MG_BV(JSX, false); }
  if (js == 1) { MG_DQ(1) }
  else if (js == 2) { MG_DQ(2) }
  else if (js <= 4) { MG_DQ(4) }
  else { MG_DQ(8) }
#undef MG_DQ
#undef MG_BV
#undef MG_LAUNCH
  return hipGetLastError();
}
