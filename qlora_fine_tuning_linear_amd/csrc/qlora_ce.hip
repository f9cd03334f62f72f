// Output head + cross-entropy for gfx950: the fused linear / cross-entropy
// step of "LLM Fine-Tuning in 2026: Unsloth vs QLoRA vs Liger-Kernel"
// (section 3), computed one token chunk at a time so that no [tokens, vocab]
// logit matrix is ever held.  Per chunk the entry point runs the bf16 GEMM
// for the chunk's fp32 logits, ce_rows_kernel for the loss terms and the
// bf16 logit gradient (in place), and the bf16 GEMM again (reduction over the vocabulary,
// split into fp32 partials, reading the head [V, D] as stored: a K-major
// weight operand) for dX.  The helpers here:
//   * ce_count_kernel      - number of tokens that carry a target;
//   * ce_rows_kernel       - one workgroup per token row of logits: log-sum-exp
//     (one pass, running maximum), the token's loss term and, in a second pass,
//     (softmax - onehot) / n rounded to bf16 in place of the logits;
//   * ce_loss_kernel       - the mean of the per-token terms in a fixed order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qlora_device.h"
#include "qlora_launch.h"

namespace qk {

// A target counts when it is a class index; ignore_index and any value
// outside [0, V) mark a token without a target.
__device__ __forceinline__ bool ce_valid(int32_t t, int64_t V, int32_t ignore) {
  return t != ignore && t >= 0 && (int64_t)t < V;
}

__global__ __launch_bounds__(1024) void ce_count_kernel(const int32_t* __restrict__ targets, int64_t T, int64_t V,
                                                        int32_t ignore, int32_t* __restrict__ n_valid) {
  __shared__ int32_t red[1024];
  int32_t c = 0;
  for (int64_t i = threadIdx.x; i < T; i += 1024) c += ce_valid(targets[i], V, ignore) ? 1 : 0;
  red[threadIdx.x] = c;
  __syncthreads();
  for (int s = 512; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) *n_valid = red[0];
}

// Running (max, sum of exp(x - max)) pairs, combined in a fixed order.
__device__ __forceinline__ void lse_combine(float& m, float& s, float m2, float s2) {
  if (s2 == 0.0f) return;
  if (s == 0.0f) {
    m = m2;
    s = s2;
    return;
  }
  const float mm = fmaxf(m, m2);
  s = s * __expf(m - mm) + s2 * __expf(m2 - mm);
  m = mm;
}

// One workgroup of 256 threads per token row of the chunk's logits z
// [rows, V] (fp32, V % 8 == 0).  Thread i takes the 32-byte chunks i, i + 256,
// ...; partial (max, sum) pairs are combined across lanes with a fixed xor
// pattern and across the four waves in wave order, so the result does not
// depend on timing.  Then token_loss[row] = lse - z[target] (0 without a
// target) and, with want_grad, bf16((softmax(z) - onehot) / n) (0 rows for
// tokens without a target) is written over the first half of the row's bytes
// (a bf16 row of stride 2V elements).  That pass goes in rounds of 256 chunks
// with a barrier between the reads and the writes of a round: the 16-byte
// bf16 chunk c lands in bytes [16c, 16c + 16), inside fp32 chunks that every
// thread has read by then (round k writes what rounds <= k read).
__global__ __launch_bounds__(256) void ce_rows_kernel(float* __restrict__ z, int64_t V,
                                                      const int32_t* __restrict__ targets, int32_t ignore,
                                                      const int32_t* __restrict__ n_valid, int want_grad,
                                                      float* __restrict__ token_loss) {
  __shared__ float wm[4], wsum[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.x;
  float* zr = z + row * V;
  const int32_t tgt = targets[row];
  const bool valid = ce_valid(tgt, V, ignore);
  const float zt = valid ? zr[tgt] : 0.0f;
  const int64_t nch = V / 8;

  float m = 0.0f, s = 0.0f;
  for (int64_t c = tid; c < nch; c += 256) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(zr + c * 8);
    const f32x4 b = *reinterpret_cast<const f32x4*>(zr + c * 8 + 4);
    const float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    float cm = x[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) cm = fmaxf(cm, x[e]);
    float cs = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) cs += __expf(x[e] - cm);
    lse_combine(m, s, cm, cs);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o), s2 = __shfl_xor(s, o);
    lse_combine(m, s, m2, s2);
  }
  if (lane == 0) {
    wm[wave] = m;
    wsum[wave] = s;
  }
  __syncthreads();
  float M = wm[0], S = wsum[0];
#pragma unroll
  for (int w = 1; w < 4; ++w) lse_combine(M, S, wm[w], wsum[w]);
  const float lse = M + __logf(S);
  if (tid == 0) token_loss[row] = valid ? lse - zt : 0.0f;
  if (!want_grad) return;

  const int32_t n = *n_valid;
  const float inv_n = (valid && n > 0) ? 1.0f / (float)n : 0.0f;
  uint16_t* gr = reinterpret_cast<uint16_t*>(zr);
  for (int64_t c0 = 0; c0 < nch; c0 += 256) {
    const int64_t c = c0 + tid;
    f32x4 a{}, b{};
    if (c < nch) {
      a = *reinterpret_cast<const f32x4*>(zr + c * 8);
      b = *reinterpret_cast<const f32x4*>(zr + c * 8 + 4);
    }
    __syncthreads();  // every read of this round is done before its writes
    if (c < nch) {
      const float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
      u32x4 o;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        float g[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int64_t col = c * 8 + 2 * d + e;
          g[e] = (__expf(x[2 * d + e] - lse) - (col == tgt ? 1.0f : 0.0f)) * inv_n;
        }
        o[d] = pack_bf16x2(g[0], g[1]);
      }
      *reinterpret_cast<u32x4*>(gr + c * 8) = o;
    }
  }
}

// loss = (1/n) sum_t token_loss[t] (0 when n == 0 or n_valid is null):
// thread i adds t = i, i + 1024, ... in order, then a fixed tree over the
// threads.
__global__ __launch_bounds__(1024) void ce_loss_kernel(const float* __restrict__ token_loss, int64_t T,
                                                       const int32_t* __restrict__ n_valid, float* __restrict__ loss) {
  __shared__ float red[1024];
  float s = 0.0f;
  for (int64_t i = threadIdx.x; i < T; i += 1024) s += token_loss[i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int k = 512; k > 0; k >>= 1) {
    if ((int)threadIdx.x < k) red[threadIdx.x] += red[threadIdx.x + k];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const int32_t n = n_valid ? *n_valid : 0;
    *loss = n > 0 ? red[0] / (float)n : 0.0f;
  }
}

}  // namespace qk

using namespace qk;

hipError_t launch_ce_count(const int32_t* targets, int64_t T, int64_t V, int32_t ignore, int32_t* n_valid,
                           hipStream_t st) {
  ce_count_kernel<<<1, 1024, 0, st>>>(targets, T, V, ignore, n_valid);
  return hipGetLastError();
}

hipError_t launch_ce_rows(float* z, int64_t rows, int64_t V, const int32_t* targets, int32_t ignore,
                          const int32_t* n_valid, int want_grad, float* token_loss, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  ce_rows_kernel<<<dim3((unsigned)rows), 256, 0, st>>>(z, V, targets, ignore, n_valid, want_grad, token_loss);
  return hipGetLastError();
}

hipError_t launch_ce_loss(const float* token_loss, int64_t T, const int32_t* n_valid, float* loss, hipStream_t st) {
  ce_loss_kernel<<<1, 1024, 0, st>>>(token_loss, T, n_valid, loss);
  return hipGetLastError();
}
