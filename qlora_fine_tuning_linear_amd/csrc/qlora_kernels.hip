// gfx950 (MI355X, CDNA4) kernels of the QLoRA linear / SwiGLU-MLP library.
//
// The method: a frozen NF4 base weight plus a trainable rank-r LoRA pair,
// h = W0 x + (alpha/r) B A x ("LLM Fine-Tuning in 2026: Unsloth vs QLoRA vs
// Liger-Kernel", section 1), with forward and backward written by hand
// (section 2 of that page) and the SwiGLU activation recomputed in the
// backward pass ("What is Unsloth", "Recompute instead of store").  The
// kernel design is this library's own, for CDNA4.  The GEMMs are split by
// token count M over three files:
//
//   M <= 64      qlora_skinny.hip: codes expanded straight into MFMA operand
//                registers (weight-streaming forward, split transposed
//                product + finish for the backward);
//   64 < M < 512 this file, qgemm_kernel: a dequant-staged bf16 MFMA GEMM
//                (v_mfma_f32_32x32x16_bf16, fp32 accumulation).  Per 64-wide
//                reduction tile all threads expand the NF4 codes of the
//                weight tile (codebook lookup in LDS, times the block absmax,
//                round to bf16) into a double-buffered LDS tile, written
//                transposed for the backward so both passes read it alike;
//                activations are staged through LDS (256 x 256 tiles) or
//                loaded straight in MFMA layout (64-wide tiles);
//   M >= 512     qlora_bgemm.hip: the weight expanded once per call into a
//                bf16 workspace, then a bf16 GEMM with direct-to-LDS loads.
//
// All GEMMs share the fused epilogue (qlora_gemm_common.h): the LoRA term as
// extra MFMA steps on the accumulators, and the SwiGLU forward / analytic
// backward variants, so G, U, H and dG, dU need no extra pass.  Also here:
//
// * lora_down_kernel - V = Z A^T (and T = dY B), the skinny rank-r products.
// * lora_grad_kernel / lora_grad16_kernel - dB = s dY^T XA and dA = s T^T X:
//   reductions over the tokens, with the token-major operand transposed in
//   registers and fed to the matrix cores (32x32x16, or 16x16x32 for ranks up
//   to 16); fixed-order partial sums, so results are reproducible.
// * nf4_quantize_kernel / nf4_dequantize_kernel - the bit-exact encoding.
// * transpose and packed-adapter helpers of the backward.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "qlora_device.h"
#include "qlora_gemm_common.h"
#include "qlora_launch.h"

namespace qk {

// ------------------------------------------------------------------------
// NF4 quantization.  One workgroup per group of 256 consecutive absmax
// blocks (64 elements each); thread t owns block t of the group.  With
// double quantization the group is exactly one DQ group.
// ------------------------------------------------------------------------
__global__ __launch_bounds__(256) void nf4_quantize_kernel(
    const float* __restrict__ W, int64_t nblocks, const float* __restrict__ codebook, int dq,
    uint8_t* __restrict__ codes, float* __restrict__ absmax, uint8_t* __restrict__ absmax_q,
    float* __restrict__ absmax_scale) {
  __shared__ double mids[15];
  __shared__ int zidx;
  __shared__ float wmax[4];
  const int t = threadIdx.x;
  if (t < 15) mids[t] = ((double)codebook[t] + (double)codebook[t + 1]) * 0.5;
  if (t < 16 && codebook[t] == 0.0f) zidx = t;
  __syncthreads();
  const int64_t b = (int64_t)blockIdx.x * 256 + t;
  const bool valid = b < nblocks;
  float a = 0.0f;
  f32x4 v[16];
  if (valid) {
    const f32x4* src = reinterpret_cast<const f32x4*>(W + b * 64);
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = src[i];
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) a = fmaxf(a, fabsf(v[i][e]));
    u32x4 out[2] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
    const int z = zidx;
#pragma unroll
    for (int e = 0; e < 64; ++e) {
      int q = z;
      if (a != 0.0f) {
        const float n = v[e >> 2][e & 3] / a;  // correctly rounded fp32 quotient
        const double nd = (double)n;
        q = 0;
#pragma unroll
        for (int j = 0; j < 15; ++j) q += (nd > mids[j]) ? 1 : 0;
      }
      out[e >> 5][(e & 31) >> 3] |= (uint32_t)q << (4 * (e & 7));
    }
    u32x4* dst = reinterpret_cast<u32x4*>(codes + b * 32);
    dst[0] = out[0];
    dst[1] = out[1];
    if (!dq) absmax[b] = a;
  }
  if (dq) {
    float g = a;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) g = fmaxf(g, __shfl_xor(g, off));
    if ((t & 63) == 0) wmax[t >> 6] = g;
    __syncthreads();
    g = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
    const float S = g / 255.0f;
    if (valid) {
      uint32_t c8 = 0;
      if (S != 0.0f) c8 = (uint32_t)fminf(255.0f, rintf(a / S));
      absmax_q[b] = (uint8_t)c8;
    }
    if (t == 0) absmax_scale[blockIdx.x] = S;
  }
}

__device__ __forceinline__ float block_absmax(const Nf4Dev& w, int64_t blk) {
  if (w.dq) return (float)w.absmax_q[blk] * w.absmax_scale[blk / w.dq];
  return w.absmax[blk];
}

// ------------------------------------------------------------------------
// NF4 dequantization (export): 8 elements per thread.
// ------------------------------------------------------------------------
__global__ __launch_bounds__(256) void nf4_dequantize_kernel(Nf4Dev w, const float* __restrict__ codebook,
                                                             int64_t n_groups8, int out_f32, void* out) {
  __shared__ float cb[16];
  if (threadIdx.x < 16) cb[threadIdx.x] = codebook[threadIdx.x];
  __syncthreads();
  const int64_t i8 = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i8 >= n_groups8) return;
  const uint32_t c = reinterpret_cast<const uint32_t*>(w.codes)[i8];
  const float a = block_absmax(w, i8 >> 3);
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = cb[(c >> (4 * e)) & 15u] * a;
  if (out_f32) {
    f32x4* o = reinterpret_cast<f32x4*>(static_cast<float*>(out) + i8 * 8);
    o[0] = f32x4{v[0], v[1], v[2], v[3]};
    o[1] = f32x4{v[4], v[5], v[6], v[7]};
  } else {
    u32x4 o;
    o[0] = pack_bf16x2(v[0], v[1]);
    o[1] = pack_bf16x2(v[2], v[3]);
    o[2] = pack_bf16x2(v[4], v[5]);
    o[3] = pack_bf16x2(v[6], v[7]);
    reinterpret_cast<u32x4*>(static_cast<uint16_t*>(out) + i8 * 8)[0] = o;
  }
}

// ------------------------------------------------------------------------
// The dequant-staged MFMA GEMM.
//
// Output tile: BM tokens x BN output columns; WM x WN waves, each FM x FN
// frags of 32 x 32.  The MFMA's "A" operand is the weight side (rows = output
// columns, from LDS), its "B" operand the activations (columns = tokens, from
// registers), so each lane ends up with 4 consecutive output columns of one
// token per accumulator quad and stores them as one 8-byte write.
//
// LDS weight tile: [BN rows][64 reduction values] bf16, rows = output columns,
// 16-byte chunks XOR-swizzled by swz(row); two buffers.
// ------------------------------------------------------------------------
// Per-thread expansion state of one weight tile: packed codes and the absmax
// of every weight row the thread expands, loaded one tile before expansion.
//   forward fill   : one weight row, EPT consecutive elements (one absmax)
//   transposed fill: RPT weight rows x 8 columns (RPT absmax values)
template <int NC, int NA>
struct FillRegs {
  uint32_t c[NC];
  float a[NA];
  int cbo;  // transposed fill: codebook of the tile (0: w0, 16: w1)
};


// ALDS: activations are staged through LDS.  Each 64-wide reduction tile of
// the BM token rows is fetched with direct global->LDS loads in whole 128-byte
// row segments (8 lanes per row), the 16-byte chunk each lane fetches chosen
// so that the LDS image is the swz()-swizzled [BM][64] layout; the MFMA
// operands are then read from LDS.  Without ALDS each lane loads its own
// operand rows straight into registers (fine when the token tile is small).
template <int MODE, int WM, int WN, int FM, int FN, bool SPLIT, bool DQ, bool ALDS>
__global__ __launch_bounds__(WM* WN * 64) void qgemm_kernel(GemmArgs p) {
  using C = TileCfg<WM, WN, FM, FN>;
  constexpr int BM = C::BM, BN = C::BN, NT = C::NT;
  constexpr bool TR = ModeTraits<MODE>::trans;
  constexpr int NC = TR ? C::RPT : C::EPT / 8;  // code dwords per thread per tile
  constexpr int NA = TR ? C::RPT : 1;           // absmax values per thread per tile
  static_assert(NC == 8 || NC == 4 || NC == 2, "fill shape");
  using Fill = FillRegs<NC, NA>;

  __shared__ __attribute__((aligned(16))) uint16_t lds[2][BN * 64];
  __shared__ __attribute__((aligned(16))) uint16_t alds[ALDS ? 2 : 1][ALDS ? BM * 64 : 8];
  __shared__ float cb[32];  // [0, 16): table of w0, [16, 32): table of w1

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int l32 = lane & 31, g = lane >> 5;

  // output columns per tile: the SwiGLU forward stacks gate and up rows of the
  // same BN/2 intermediate columns in one LDS tile
  constexpr int BNO = ModeTraits<MODE>::swiglu_fwd ? BN / 2 : BN;
  const int64_t tm = blockIdx.x % p.tiles_m;
  const int64_t tn = blockIdx.x / p.tiles_m;
  const int64_t m0 = tm * BM;
  const int64_t n0 = tn * BNO;  // first output column (I-index for the SwiGLU forward)

  const int KT0 = (int)(p.Kred0 / 64);
  const int KT = KT0 + (int)(p.Kred1 / 64);
  int kt_begin = 0, kt_end = KT;
  if (SPLIT) {
    kt_begin = blockIdx.y * p.ktiles_per_split;
    kt_end = min(KT, kt_begin + p.ktiles_per_split);
  }

  if (tid < 32) cb[tid] = (tid < 16 || !p.codebook1) ? p.codebook[tid & 15] : p.codebook1[tid & 15];

  // ---- activation operand: per-lane row pointers (rows clamped into [0, M))
  int64_t arow[FM];
  const uint16_t* aptr0[FM];
  const uint16_t* aptr1[FM];
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    int64_t r = m0 + (int64_t)(wm * FM + i) * 32 + l32;
    arow[i] = r < p.M ? r : p.M - 1;
    aptr0[i] = p.act0 + arow[i] * p.Kred0 + 8 * g;
    aptr1[i] = (p.act1 ? p.act1 + arow[i] * p.Kred1 + 8 * g : aptr0[i]) - p.Kred0;
  }
  auto load_act = [&](int kt, u32x4 (&dst)[FM][4]) {
    const bool second = kt >= KT0;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const uint16_t* src = (second ? aptr1[i] : aptr0[i]) + (int64_t)kt * 64;
#pragma unroll
      for (int s = 0; s < 4; ++s) dst[i][s] = *reinterpret_cast<const u32x4*>(src + 16 * s);
    }
  };

  // ---- ALDS staging: per tile, NI coalesced 16-byte loads per thread into
  // registers (8 lanes read one 128-byte row segment), written to LDS later
  // in the tile at the swz()-swizzled position.  Load i of wave w covers rows
  // (i*W + w)*8 + lane/8, chunk lane%8.  Rows past M are clamped.
  constexpr int NW = NT / 64;
  constexpr int NI = ALDS ? BM * 8 / NT : 1;
  uint32_t soff[NI];  // element offsets of the lane's chunks from the tile's first row
  int srow[NI];
  if constexpr (ALDS) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int row = (i * NW + wave) * 8 + (lane >> 3);
      int r = row;
      if (m0 + r >= p.M) r = (int)(p.M - 1 - m0);
      srow[i] = row;
      soff[i] = (uint32_t)r * (uint32_t)p.Kred0 + (uint32_t)(lane & 7) * 8;
    }
  }
  // the dual-reduction GEMM reads act0 then act1, both with row length Kred0
  const uint16_t* sbase0 = p.act0 + m0 * p.Kred0;
  const uint16_t* sbase1 = (p.act1 ? p.act1 + m0 * p.Kred0 : sbase0) - p.Kred0;
  auto stage_load = [&](int kt, u32x4 (&S)[NI]) {
    if constexpr (ALDS) {
      const uint16_t* base = (kt >= KT0 ? sbase1 : sbase0) + (int64_t)kt * 64;
#pragma unroll
      for (int i = 0; i < NI; ++i) S[i] = *reinterpret_cast<const u32x4*>(base + soff[i]);
    }
  };
  auto stage_store = [&](const u32x4 (&S)[NI], uint16_t* buf) {
    if constexpr (ALDS) {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int row = srow[i];
        *reinterpret_cast<u32x4*>(buf + row * 64 + (((lane & 7) ^ swz(row)) * 8)) = S[i];
      }
    }
  };
  // ---- weight tile expansion: per-thread source pointers
  // forward: thread -> (LDS row r, part); weight row clamped into [0, N)
  // transposed: thread -> (8 output columns kc, RPT reduction rows rg)
  const int fr = TR ? 0 : tid / C::TPR, fpart = TR ? 0 : tid % C::TPR;
  constexpr int KC = BN / 8;
  const int kc = tid % KC, rg = tid / KC;
  const uint8_t* csrc0;
  const uint8_t* csrc1;
  int64_t ablk0, ablk1, cstride0, cstride1, astride0, astride1;
  {
    if constexpr (!TR) {
      const Nf4Dev& w = (ModeTraits<MODE>::swiglu_fwd && fr >= BN / 2) ? p.w1 : p.w0;
      int64_t wrow = n0 + (fr % (ModeTraits<MODE>::swiglu_fwd ? BN / 2 : BN));
      if (wrow >= w.N) wrow = w.N - 1;
      csrc0 = csrc1 = w.codes + wrow * (w.K / 2) + fpart * (C::EPT / 2);
      ablk0 = ablk1 = wrow * (w.K / 64);
      cstride0 = cstride1 = astride0 = astride1 = 0;
    } else {
      int64_t col = n0 + 8 * kc;
      if (col > p.w0.K - 8) col = p.w0.K - 8;
      csrc0 = p.w0.codes + (int64_t)(rg * C::RPT) * (p.w0.K / 2) + col / 2;
      ablk0 = (int64_t)(rg * C::RPT) * (p.w0.K / 64) + col / 64;
      cstride0 = p.w0.K / 2;
      astride0 = p.w0.K / 64;
      const Nf4Dev& w1 = p.act1 ? p.w1 : p.w0;
      csrc1 = w1.codes + (int64_t)(rg * C::RPT) * (w1.K / 2) + col / 2 - (int64_t)KT0 * 64 * (w1.K / 2);
      ablk1 = (int64_t)(rg * C::RPT) * (w1.K / 64) + col / 64 - (int64_t)KT0 * 64 * (w1.K / 64);
      cstride1 = w1.K / 2;
      astride1 = w1.K / 64;
    }
  }
  const Nf4Dev& wsel1 = (TR && p.act1) ? p.w1 : p.w0;

  auto fill_load = [&](int kt, Fill& F) {
    if constexpr (!TR) {
      // the SwiGLU forward's second half of the rows reads the up weight
      const Nf4Dev& w = (ModeTraits<MODE>::swiglu_fwd && fr >= BN / 2) ? p.w1 : p.w0;
      const uint8_t* src = csrc0 + (int64_t)kt * 32;
      if constexpr (NC == 8) {
        const u32x4 x0 = reinterpret_cast<const u32x4*>(src)[0], x1 = reinterpret_cast<const u32x4*>(src)[1];
        F.c[0] = x0[0]; F.c[1] = x0[1]; F.c[2] = x0[2]; F.c[3] = x0[3];
        F.c[4] = x1[0]; F.c[5] = x1[1]; F.c[6] = x1[2]; F.c[7] = x1[3];
      } else if constexpr (NC == 4) {
        const u32x4 x0 = reinterpret_cast<const u32x4*>(src)[0];
        F.c[0] = x0[0]; F.c[1] = x0[1]; F.c[2] = x0[2]; F.c[3] = x0[3];
      } else {
        const u32x2 x0 = reinterpret_cast<const u32x2*>(src)[0];
        F.c[0] = x0[0]; F.c[1] = x0[1];
      }
      F.a[0] = absmax_at<DQ>(w, ablk0 + kt);
      F.cbo = 0;
    } else {
      const bool second = kt >= KT0;
      const Nf4Dev& w = second ? wsel1 : p.w0;
      const uint8_t* src = second ? csrc1 : csrc0;
      const int64_t cs = second ? cstride1 : cstride0;
      const int64_t ab = second ? ablk1 : ablk0;
      const int64_t as = second ? astride1 : astride0;
      const int64_t row = (int64_t)kt * 64;
      F.cbo = second ? 16 : 0;
#pragma unroll
      for (int i = 0; i < C::RPT; ++i) {
        F.c[i] = *reinterpret_cast<const uint32_t*>(src + (row + i) * cs);
        F.a[i] = absmax_at<DQ>(w, ab + (row + i) * as);
      }
    }
  };

  // Expand part `d` (of 8) of the thread's tile into LDS buffer `buf`.
  auto fill_part = [&](const Fill& F, uint16_t* buf, int d) {
    if constexpr (!TR) {
      constexpr int PER = NC;  // code dwords = LDS chunks of this thread
      if (d < PER) {
        const int chunk = fpart * PER + d;
        const u32x4 v = deq8(F.c[d], F.a[0], (ModeTraits<MODE>::swiglu_fwd && fr >= BN / 2) ? cb + 16 : cb);
        *reinterpret_cast<u32x4*>(buf + fr * 64 + ((chunk ^ swz(fr)) * 8)) = v;
      }
    } else {
      constexpr int RPT = C::RPT;
      const int n_off = rg * RPT;
      const int chunk = n_off >> 3, sub = n_off & 7;
      const int c = d;  // output column 8 kc + c
      float v[RPT];
      const float* tcb = cb + F.cbo;
#pragma unroll
      for (int i = 0; i < RPT; ++i) v[i] = tcb[(F.c[i] >> (4 * c)) & 15u] * F.a[i];
      const int row = 8 * kc + c;
      uint16_t* dst = buf + row * 64 + ((chunk ^ swz(row)) * 8) + sub;
      if constexpr (RPT == 8) {
        *reinterpret_cast<u32x4*>(dst) = u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                               pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
      } else if constexpr (RPT == 4) {
        *reinterpret_cast<u32x2*>(dst) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      } else {
        *reinterpret_cast<uint32_t*>(dst) = pack_bf16x2(v[0], v[1]);
      }
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int f = 0; f < FN; ++f)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][f][v] = 0.0f;

  // MFMAs of one reduction tile from LDS buffer `cur` with activations A.
  // With a next tile (`nxt` != null): each activation substep slot is
  // refilled from tile kt_next as soon as its MFMAs have been issued, and the
  // expansion of the next weight tile (codes F) into `nxt` is spread over the
  // four substeps, so the vector and LDS work overlaps the matrix cores.
  // staged activations of the next tiles: two register sets, loaded two tiles
  // ahead of their LDS store
  u32x4 Sa[NI], Sb[NI];
  auto mma_tile = [&](auto has_next, const uint16_t* cur, const uint16_t* acur, u32x4 (&A)[FM][4], int kt_next,
                      const Fill& F, uint16_t* nxt, uint16_t* anxt, const u32x4 (&Sst)[NI]) {
    constexpr bool NEXT = decltype(has_next)::value;
    const uint16_t* asrc[FM];
    if constexpr (NEXT && !ALDS) {
      const bool second = kt_next >= KT0;
#pragma unroll
      for (int i = 0; i < FM; ++i) asrc[i] = (second ? aptr1[i] : aptr0[i]) + (int64_t)kt_next * 64;
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 wa[FN];
#pragma unroll
      for (int f = 0; f < FN; ++f) {
        const int row = frag_row<MODE, WN, FN>(wn, f) + l32;
        wa[f] = *reinterpret_cast<const u32x4*>(cur + row * 64 + (((2 * s + g) ^ swz(row)) * 8));
      }
      if constexpr (ALDS) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int row = (wm * FM + i) * 32 + l32;
          A[i][s] = *reinterpret_cast<const u32x4*>(acur + row * 64 + (((2 * s + g) ^ swz(row)) * 8));
        }
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int f = 0; f < FN; ++f) acc[i][f] = mfma32(wa[f], A[i][s], acc[i][f]);
      if constexpr (NEXT) {
        // refill activation slots in pairs: substeps (0,1) and (2,3) of a row
        // are one contiguous 64-byte segment, fetched by back-to-back loads
        if (!ALDS && (s & 1)) {
#pragma unroll
          for (int i = 0; i < FM; ++i) {
            A[i][s - 1] = *reinterpret_cast<const u32x4*>(asrc[i] + 16 * (s - 1));
            A[i][s] = *reinterpret_cast<const u32x4*>(asrc[i] + 16 * s);
          }
          // keep the refill here: sinking it to the end of the tile would
          // expose its latency at the start of the next tile
          __builtin_amdgcn_sched_barrier(0);
        }
        // this substep's share of the expansion parts
        constexpr int NP = TR ? 8 : NC;
#pragma unroll
        for (int d = 0; d < NP; ++d)
          if (d * 4 / NP == s) fill_part(F, nxt, d);
        if (ALDS && s == 3) stage_store(Sst, anxt);  // next tile's activations, loaded two tiles ahead
      }
    }
  };

  // the LoRA term first: its loads are issued before the main reduction
  gemm_lora<MODE, WN, FM, FN, SPLIT>(p, acc, arow, n0, wn, l32, g);

  u32x4 A[FM][4];
  Fill Fa, Fb;
  __syncthreads();  // codebook in LDS
  if (kt_begin < kt_end) {
    if constexpr (ALDS) {
      stage_load(kt_begin, Sa);
      stage_store(Sa, alds[kt_begin & 1]);
      stage_load(min(kt_begin + 1, kt_end - 1), Sa);
    } else {
      load_act(kt_begin, A);
    }
    fill_load(kt_begin, Fa);
#pragma unroll
    for (int d = 0; d < 8; ++d) fill_part(Fa, lds[kt_begin & 1], d);
    fill_load(min(kt_begin + 1, kt_end - 1), Fa);
  }
  __syncthreads();

  // steady state: tile kt computes from LDS while tile kt+1 is expanded into
  // the other buffer; activations are fetched one tile ahead, codes two.
  // Two code-register sets alternate between consecutive tiles (unrolled by
  // two), so a prefetch is never copied - a copy would wait for the load.
  // (the staged activations of tile kt + 1 sit in Suse, those of kt + 2 are
  // requested into Sload; tiles past the end are clamped: redundant loads)
  auto step = [&](int kt, const Fill& Fuse, Fill& Fload, const u32x4 (&Suse)[NI], u32x4 (&Sload)[NI]) {
    stage_load(min(kt + 2, kt_end - 1), Sload);
    fill_load(min(kt + 2, kt_end - 1), Fload);
    __builtin_amdgcn_sched_barrier(0);  // issue the global loads first
    mma_tile(std::true_type{}, lds[kt & 1], alds[ALDS ? (kt & 1) : 0], A, kt + 1, Fuse, lds[(kt + 1) & 1],
             alds[ALDS ? ((kt + 1) & 1) : 0], Suse);
    lds_barrier();  // global prefetches stay in flight across it
  };
  int kt = kt_begin;
  for (; kt + 2 < kt_end; kt += 2) {
    step(kt, Fa, Fb, Sa, Sb);
    step(kt + 1, Fb, Fa, Sb, Sa);
  }
  if (kt + 1 < kt_end) {
    step(kt, Fa, Fb, Sa, Sb);
    ++kt;
  }
  if (kt_begin < kt_end)
    mma_tile(std::false_type{}, lds[(kt_end - 1) & 1], alds[ALDS ? ((kt_end - 1) & 1) : 0], A, 0, Fa, lds[0],
             alds[0], Sa);

  gemm_epilogue<MODE, WM, WN, FM, FN, SPLIT>(p, acc, arow, m0, n0, wm, wn, l32, g);
}

// Split-reduction finish for the linear GEMMs: out = bf16(sum_z part[z]) in
// split order (split 0 already holds the LoRA term).  4 columns per thread.
__global__ __launch_bounds__(256) void splitk_finish_kernel(const float* __restrict__ part, int splits,
                                                            int64_t MN, uint16_t* __restrict__ out) {
  const int64_t q = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (q >= MN) return;
  f32x4 s = *reinterpret_cast<const f32x4*>(part + q);
  for (int z = 1; z < splits; ++z) s += *reinterpret_cast<const f32x4*>(part + (int64_t)z * MN + q);
  *reinterpret_cast<u32x2*>(out + q) = u32x2{pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3])};
}

// ------------------------------------------------------------------------
// LoRA down-projection V[M, j] = sum_k Z[M, k] W[j, k] on the matrix cores,
// for the rank-r products X A^T, H A_d^T and (with W = B^T) dY B.  W rows
// j < r0 come from W0 into V0, rows r0 <= j < r0 + r1 from W1 into V1 (gate |
// up share one pass over Z).  Both W are [r, Kred] bf16, rows contiguous.
//
// Workgroup: 32 TF tokens (TF token frags of 32), 8 waves taking the 64-wide
// reduction chunks of their split in turn (consecutive chunks stream side by
// side).  Within a chunk lane (token l32 of each frag, half h) loads the 64
// contiguous bytes k0 + 32h .. +31 of its token row, and the W lane (row l32
// of the frag, half h) the same columns of its row: MFMA step t multiplies
// columns k0 + 32h + 8t + e, a permutation of the chunk shared by both
// operands.  Every workgroup reads its split's W columns whole, so TF = 2
// halves the W bytes per token (at ranks 33..64 they are twice the token
// bytes with TF = 1).  The next chunk's loads are issued before the current
// chunk's MFMAs.  The 8 wave partials are summed in LDS in wave order; with
// several splits (blockIdx.y) the sums go to part[split][M][r0 + r1] for
// down_finish_kernel.
// ------------------------------------------------------------------------
template <int JF, int TF>
__global__ __launch_bounds__(512) void lora_down_kernel(const uint16_t* __restrict__ Z, int64_t M, int64_t Kred,
                                                        const uint16_t* __restrict__ W0, int r0,
                                                        const uint16_t* __restrict__ W1, int r1,
                                                        float* __restrict__ V0, float* __restrict__ V1,
                                                        int64_t chunks_per_split, float* __restrict__ part) {
  __shared__ float red[8][JF * TF * 16 * 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, h = lane >> 5;
  const int rt = r0 + r1;
  const int64_t m0 = (int64_t)blockIdx.x * 32 * TF;
  const uint16_t* zrow[TF];
#pragma unroll
  for (int tf = 0; tf < TF; ++tf) {
    const int64_t m = (m0 + 32 * tf + l32 < M) ? m0 + 32 * tf + l32 : M - 1;
    zrow[tf] = Z + m * Kred + 32 * h;
  }
  const uint16_t* wrow[JF];
  bool wok[JF];
#pragma unroll
  for (int jf = 0; jf < JF; ++jf) {
    const int j = 32 * jf + l32;
    wok[jf] = j < rt;
    wrow[jf] = (j < r0 ? W0 + (int64_t)j * Kred : W1 + (int64_t)(j - r0) * Kred) + 32 * h;
    if (!wok[jf]) wrow[jf] = W0 + 32 * h;  // any valid address (one line for all such lanes); zeroed
  }
  const int64_t C = Kred / 64;
  const int64_t cb = (int64_t)blockIdx.y * chunks_per_split;
  const int64_t ce = (cb + chunks_per_split < C) ? cb + chunks_per_split : C;

  f32x16 acc[JF][TF];
#pragma unroll
  for (int jf = 0; jf < JF; ++jf)
#pragma unroll
    for (int tf = 0; tf < TF; ++tf)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[jf][tf][v] = 0.0f;

  u32x4 za[TF][4], wa[JF][4], zb[TF][4], wb[JF][4];
  auto load = [&](int64_t c, u32x4 (&z)[TF][4], u32x4 (&w)[JF][4]) {
#pragma unroll
    for (int tf = 0; tf < TF; ++tf)
#pragma unroll
      for (int t = 0; t < 4; ++t) z[tf][t] = *reinterpret_cast<const u32x4*>(zrow[tf] + c * 64 + 8 * t);
#pragma unroll
    for (int jf = 0; jf < JF; ++jf)
#pragma unroll
      for (int t = 0; t < 4; ++t) w[jf][t] = *reinterpret_cast<const u32x4*>(wrow[jf] + c * 64 + 8 * t);
  };
  auto mul = [&](const u32x4 (&z)[TF][4], const u32x4 (&w)[JF][4]) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int jf = 0; jf < JF; ++jf) {
        const u32x4 wz = wok[jf] ? w[jf][t] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int tf = 0; tf < TF; ++tf) acc[jf][tf] = mfma32(wz, z[tf][t], acc[jf][tf]);
      }
  };
  int64_t c = cb + wave;
  if (c < ce) load(c, za, wa);
  // two register sets alternate (a copy of a prefetch would wait for it)
  for (; c + 8 < ce; c += 16) {
    load(c + 8, zb, wb);
    mul(za, wa);
    if (c + 16 < ce) load(c + 16, za, wa);
    mul(zb, wb);
  }
  if (c < ce) mul(za, wa);

  // acc[jf][tf][v] = C[j = 32 jf + 8(v/4) + 4h + v%4][token 32 tf + l32]
#pragma unroll
  for (int jf = 0; jf < JF; ++jf)
#pragma unroll
    for (int tf = 0; tf < TF; ++tf)
#pragma unroll
      for (int v = 0; v < 16; ++v) red[wave][((jf * TF + tf) * 16 + v) * 64 + lane] = acc[jf][tf][v];
  __syncthreads();
  for (int idx = tid; idx < JF * TF * 16 * 64; idx += 512) {
    float sum = 0.0f;
#pragma unroll
    for (int w = 0; w < 8; ++w) sum += red[w][idx];
    const int ln = idx & 63, vv = (idx >> 6) & 15, jt = idx >> 10;
    const int jf = jt / TF, tf = jt - jf * TF;
    const int j = 32 * jf + 8 * (vv >> 2) + 4 * (ln >> 5) + (vv & 3);
    const int64_t mm = m0 + 32 * tf + (ln & 31);
    if (j >= rt || mm >= M) continue;
    if (part) {
      part[((int64_t)blockIdx.y * M + mm) * rt + j] = sum;
    } else if (j < r0) {
      V0[mm * r0 + j] = sum;
    } else {
      V1[mm * r1 + (j - r0)] = sum;
    }
  }
}

// One 16x16x32 bf16 MFMA: C[16x16] += A[16x32] B[32x16]; lane l holds
// A[l%16][8(l/16) + i] and B[8(l/16) + i][l%16], accumulator v of lane l is
// C[4(l/16) + v][l%16].
__device__ __forceinline__ f32x4 mfma16k32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

// The same down-projection when r0 + r1 <= 16, on 16x16x32 MFMAs: the W rows
// are the 16 rows of the A operand (none wasted), and each token frag is 16
// tokens.  Lane (c, q) (c = lane % 16, q = lane / 16) loads 16 bytes at
// k0 + 32 s + 8 q of its token row for step s of a 64-wide chunk, so one load
// instruction covers 64 contiguous bytes of 16 token rows (half lines; the
// 32-wide form reads 32-byte pieces of 32 rows).  Workgroup: 16 NF tokens (NF
// frags: 2, or 1 for at most 64 tokens, where two token blocks would leave
// most CUs idle), 8 waves taking the chunks of their split in turn; the 8
// wave partials are summed in LDS in wave order.
//
// WNR: W0 is stored [Kred, r0] (a LoRA B read as stored, r1 = 0); the lane
// gathers its 8 reduction rows of column c instead of one 16-byte load.
// XT: every token chunk the kernel loads is also written to Xt[Kred/8][Mp][8]
// (the skinny forward's activation layout; rows M..Mp-1 as zeros), so the
// activations need no separate re-layout pass.
template <bool WNR, bool XT, int NF>
__global__ __launch_bounds__(512) void lora_down16_kernel(const uint16_t* __restrict__ Z, int64_t M, int64_t Kred,
                                                          const uint16_t* __restrict__ W0, int r0,
                                                          const uint16_t* __restrict__ W1, int r1,
                                                          float* __restrict__ V0, float* __restrict__ V1,
                                                          int64_t chunks_per_split, float* __restrict__ part,
                                                          uint16_t* __restrict__ Xt, int Mp) {
  __shared__ float red[8][NF * 4 * 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, q = lane >> 4;
  const int rt = r0 + r1;
  const int64_t m0 = (int64_t)blockIdx.x * 16 * NF;
  const uint16_t* zrow[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int64_t m = (m0 + 16 * f + c < M) ? m0 + 16 * f + c : M - 1;
    zrow[f] = Z + m * Kred + 8 * q;
  }
  const bool wok = c < rt;
  const uint16_t* wrow = wok ? (c < r0 ? W0 + (int64_t)c * Kred : W1 + (int64_t)(c - r0) * Kred) + 8 * q
                             : W0 + 8 * q;  // any valid address; the operand is zeroed
  if constexpr (WNR) wrow = W0 + (wok ? c : 0) + (int64_t)(8 * q) * r0;
  // the lane's token rows for the re-laid-out copy (rows past Mp: none)
  int64_t xm[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) xm[f] = m0 + 16 * f + c;
  const int64_t C = Kred / 64;
  const int64_t cb = (int64_t)blockIdx.y * chunks_per_split;
  const int64_t ce = (cb + chunks_per_split < C) ? cb + chunks_per_split : C;

  f32x4 acc[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) acc[f] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  u32x4 za[NF][2], wa[2], zb[NF][2], wb[2];
  auto load = [&](int64_t ch, u32x4 (&z)[NF][2], u32x4 (&w)[2]) {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
#pragma unroll
      for (int f = 0; f < NF; ++f) z[f][st] = *reinterpret_cast<const u32x4*>(zrow[f] + ch * 64 + 32 * st);
      if constexpr (WNR) {
        const uint16_t* src = wrow + (ch * 64 + 32 * st) * r0;
        uint32_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = src[e * r0];
        w[st] = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
      } else {
        w[st] = *reinterpret_cast<const u32x4*>(wrow + ch * 64 + 32 * st);
      }
    }
  };
  auto mul = [&](int64_t ch, const u32x4 (&z)[NF][2], const u32x4 (&w)[2]) {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const u32x4 wz = wok ? w[st] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int f = 0; f < NF; ++f) acc[f] = mfma16k32(wz, z[f][st], acc[f]);
      if constexpr (XT) {
        // chunk ch * 8 + 4 st + q of token row xm[f]
#pragma unroll
        for (int f = 0; f < NF; ++f)
          if (xm[f] < Mp)
            *reinterpret_cast<u32x4*>(Xt + ((ch * 8 + 4 * st + q) * Mp + xm[f]) * 8) =
                xm[f] < M ? z[f][st] : u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  int64_t ch = cb + wave;
  if (ch < ce) load(ch, za, wa);
  // two register sets alternate (a copy of a prefetch would wait for it)
  for (; ch + 8 < ce; ch += 16) {
    load(ch + 8, zb, wb);
    mul(ch, za, wa);
    if (ch + 16 < ce) load(ch + 16, za, wa);
    mul(ch + 8, zb, wb);
  }
  if (ch < ce) mul(ch, za, wa);

  // acc[f][v] = C[j = 4q + v][token m0 + 16 f + c]
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[wave][(f * 4 + v) * 64 + lane] = acc[f][v];
  __syncthreads();
  if (tid < NF * 4 * 64) {
    float sum = 0.0f;
#pragma unroll
    for (int w = 0; w < 8; ++w) sum += red[w][tid];
    const int ln = tid & 63, v = (tid >> 6) & 3, f = tid >> 8;
    const int j = 4 * (ln >> 4) + v;
    const int64_t mm = m0 + 16 * f + (ln & 15);
    if (j < rt && mm < M) {
      if (part) {
        part[((int64_t)blockIdx.y * M + mm) * rt + j] = sum;
      } else if (j < r0) {
        V0[mm * r0 + j] = sum;
      } else {
        V1[mm * r1 + (j - r0)] = sum;
      }
    }
  }
}

// B [N, r] -> B^T [r, N] (bf16), so that dY B runs as a row-layout product.
__global__ __launch_bounds__(256) void transpose_rn_kernel(const uint16_t* __restrict__ B, int64_t N, int r,
                                                           uint16_t* __restrict__ BT) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // index into BT
  if (i >= N * r) return;
  const int64_t j = i / N, n = i % N;
  BT[i] = B[n * r + j];
}

// Packed LoRA groups run as one layer whose B is block-diagonal: element
// (n, j) of the [Nt, Rt] matrix belongs to the group whose row range holds n.
__device__ __forceinline__ int group_of(const GroupDesc& d, int n) {
  int g = 0;
  while (g < d.G - 1 && n >= d.noff[g + 1]) ++g;
  return g;
}

__global__ __launch_bounds__(256) void grouped_bcat_kernel(GroupDesc d, int Nt, int Rt, uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)Nt * Rt) return;
  const int n = (int)(i / Rt), j = (int)(i % Rt);
  const int g = group_of(d, n);
  float v = 0.0f;
  if (j >= d.roff[g] && j < d.roff[g + 1]) {
    const int rg = d.roff[g + 1] - d.roff[g];
    v = bf16_to_f32(d.B[g][(int64_t)(n - d.noff[g]) * rg + (j - d.roff[g])]) * d.s[g];
  }
  out[i] = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xFFFFu);
}

__global__ __launch_bounds__(256) void grouped_db_kernel(GroupDesc d, int Nt, int Rt,
                                                         const uint16_t* __restrict__ dbcat) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)Nt * Rt) return;
  const int n = (int)(i / Rt), j = (int)(i % Rt);
  const int g = group_of(d, n);
  if (j < d.roff[g] || j >= d.roff[g + 1]) return;
  const int rg = d.roff[g + 1] - d.roff[g];
  const float v = bf16_to_f32(dbcat[i]) * d.s[g];
  d.dB[g][(int64_t)(n - d.noff[g]) * rg + (j - d.roff[g])] = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xFFFFu);
}

// Several bf16 transposes in one launch: job k, src [rows, cols] -> dst
// [cols, rows].  Workgroup: one tile of 4096 elements of one job (jobs in
// order, tiles row-major within a job), shaped by the matrix: 256 x 16 when
// it has at most 16 columns (a LoRA B), 16 x 256 when it has at most 16 rows
// (a LoRA A), else 64 x 64.  Consecutive lanes read consecutive elements of a
// source row (whole rows when the tile spans them) and write consecutive
// elements of a destination row; the tile turns in LDS, whose rows are
// padded by two elements so that the column reads of the write phase fall on
// different banks.
// The same batch with one thread per element (the elements of all jobs
// numbered one after the other): for small batches, which are bound by load
// latency either way and do better with many short threads than with the
// tiled form's fewer, longer ones.
__global__ __launch_bounds__(256) void transpose_elem_kernel(TransposeJobs J) {
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  int k = 0;
  for (; k < J.n; ++k) {
    const int64_t n = J.rows[k] * J.cols[k];
    if (i < n) break;
    i -= n;
  }
  if (k >= J.n) return;
  const int64_t R = J.rows[k];
  const int64_t j = i / R, n = i - j * R;  // dst[k][j][n] = src[k][n][j]
  J.dst[k][i] = J.src[k][n * J.cols[k] + j];
}

__device__ __forceinline__ void transpose_tile_shape(int64_t rows, int64_t cols, int& lr, int& lc) {
  lc = cols <= 16 ? 4 : (rows <= 16 ? 8 : 6);  // log2 of the tile's columns
  lr = 12 - lc;
}

__global__ __launch_bounds__(256) void transpose_multi_kernel(TransposeJobs J) {
  __shared__ uint16_t t[4096 + 2 * 256];
  int64_t b = blockIdx.x, tc = 1;
  int k = 0, lr = 6, lc = 6;
  for (; k < J.n; ++k) {
    transpose_tile_shape(J.rows[k], J.cols[k], lr, lc);
    tc = (J.cols[k] + (1 << lc) - 1) >> lc;
    const int64_t tiles = ((J.rows[k] + (1 << lr) - 1) >> lr) * tc;
    if (b < tiles) break;
    b -= tiles;
  }
  if (k >= J.n) return;
  const int64_t R = J.rows[k], Cn = J.cols[k];
  const int TC = 1 << lc, TR = 1 << lr, LD = TC + 2;
  const int64_t r0 = (b / tc) << lr, c0 = (b % tc) << lc;
  const uint16_t* __restrict__ src = J.src[k];
  uint16_t* __restrict__ dst = J.dst[k];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int e = i * 256 + (int)threadIdx.x;
    const int row = e >> lc, col = e & (TC - 1);
    const int64_t r = r0 + row, c = c0 + col;
    if (r < R && c < Cn) t[row * LD + col] = src[r * Cn + c];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int e = i * 256 + (int)threadIdx.x;
    const int col = e >> lr, row = e & (TR - 1);
    const int64_t c = c0 + col, r = r0 + row;
    if (c < Cn && r < R) dst[c * R + r] = t[row * LD + col];
  }
}

// Sum of split partials [S][M][r0 + r1] in split order into V0 | V1.
__global__ __launch_bounds__(256) void down_finish_kernel(const float* __restrict__ part, int S, int64_t M,
                                                          int r0, int r1, float* __restrict__ V0,
                                                          float* __restrict__ V1) {
  const int rt = r0 + r1;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= M * rt) return;
  float s = 0.0f;
  for (int z = 0; z < S; ++z) s += part[(int64_t)z * M * rt + i];
  const int64_t m = i / rt;
  const int j = (int)(i % rt);
  if (j < r0)
    V0[m * r0 + j] = s;
  else
    V1[m * r1 + (j - r0)] = s;
}

// ------------------------------------------------------------------------
// LoRA gradient reduction over tokens: part[z][p][j] = sum_{m in split z}
// Z[m, p] V[m, j], for p in [0, P), j in [jb, jb + 32*JF).
//   ZMODE 0: Z is a bf16 [M, P] tensor.
//   ZMODE 1: Z = silu(G) * U recomputed from bf16 G, U [M, P].
// One wave per 256 columns p: per 16 tokens each lane loads 8 tokens x 8
// columns (16 B per token, coalesced along p), transposes them in registers
// (v_perm) into eight 32x16 operands whose row i is column p0 + 8 i + t,
// and runs 8 MFMAs per 32-wide j frag against V (rounded to bf16).
// ------------------------------------------------------------------------
template <int ZMODE, int JF>
__global__ __launch_bounds__(256) void lora_grad_kernel(const uint16_t* __restrict__ Z0,
                                                        const uint16_t* __restrict__ Z1, int64_t M,
                                                        int64_t P, const float* __restrict__ V, int r, int jb,
                                                        int64_t m_per_split, float* __restrict__ part) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int64_t p0 = ((int64_t)blockIdx.x * 4 + wave) * 256;
  if (p0 >= P) return;
  const int z = blockIdx.y;
  const int64_t mb = (int64_t)z * m_per_split;
  const int64_t me = min(M, mb + m_per_split);
  int64_t pc = p0 + 8 * l32;
  if (pc > P - 8) pc = P - 8;

  f32x16 acc[8][JF];
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int jf = 0; jf < JF; ++jf)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[t][jf][v] = 0.0f;

  // raw rows of one 16-token slab: token ms + 8 g + e, columns pc .. pc + 7
  // (ZMODE 1: G and U); tokens past the split are clamped and masked later
  constexpr int NZ = ZMODE == 0 ? 1 : 2;
  struct Slab {
    u32x4 raw[NZ][8];
    float x[JF][8];  // V[token][j] of the slab's tokens
  };
  auto load = [&](int64_t ms, Slab& S) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      int64_t mm = ms + 8 * g + e;
      if (mm >= me) mm = me - 1;
      S.raw[0][e] = *reinterpret_cast<const u32x4*>(Z0 + mm * P + pc);
      if constexpr (ZMODE == 1) S.raw[NZ - 1][e] = *reinterpret_cast<const u32x4*>(Z1 + mm * P + pc);
#pragma unroll
      for (int jf = 0; jf < JF; ++jf) {
        int j = jb + 32 * jf + l32;
        if (j >= r) j = r - 1;
        S.x[jf][e] = V[mm * r + j];
      }
    }
  };
  auto slab = [&](int64_t ms, const Slab& S) {
    const auto& raw = S.raw;
    u32x4 rows[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const bool ok = ms + 8 * g + e < me;
      if constexpr (ZMODE == 0) {
        rows[e] = ok ? raw[0][e] : u32x4{0u, 0u, 0u, 0u};
      } else {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const float g0 = bf16_lo(raw[0][e][d]), g1 = bf16_hi(raw[0][e][d]);
          const float h0 = g0 * sigmoid_fast(g0) * bf16_lo(raw[1][e][d]);
          const float h1 = g1 * sigmoid_fast(g1) * bf16_hi(raw[1][e][d]);
          rows[e][d] = ok ? pack_bf16x2(h0, h1) : 0u;
        }
      }
    }
    // operand t: lane (i, g) holds Z[ms + 8g + e][p0 + 8 i + t], e = 0..7
    u32x4 aop[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
      for (int d = 0; d < 4; ++d)
        aop[t][d] = __builtin_amdgcn_perm(rows[2 * d + 1][t >> 1], rows[2 * d][t >> 1], sel);
    }
#pragma unroll
    for (int jf = 0; jf < JF; ++jf) {
      const int j = jb + 32 * jf + l32;
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int64_t mm = ms + 8 * g + e;
        x[e] = (j < r && mm < me) ? S.x[jf][e] : 0.0f;
      }
      const u32x4 vop{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                      pack_bf16x2(x[6], x[7])};
#pragma unroll
      for (int t = 0; t < 8; ++t) acc[t][jf] = mfma32(aop[t], vop, acc[t][jf]);
    }
  };
  // two register sets alternate; the next slab is in flight during the current one
  Slab ra, rb;
  int64_t ms = mb;
  // unconditional prefetches (rows past the split are clamped to its last
  // row and masked), so that the compiler can count the loads in flight
  load(ms, ra);
  for (; ms + 16 < me; ms += 32) {
    load(ms + 16, rb);
    __builtin_amdgcn_sched_barrier(0);  // the prefetch is issued before the products
    slab(ms, ra);
    load(ms + 32, ra);
    __builtin_amdgcn_sched_barrier(0);
    slab(ms + 16, rb);
  }
  if (ms < me) slab(ms, ra);

  // acc[t][jf][v] = C[i = 8(v/4) + 4g + v%4][j = jb + 32 jf + l32], column p = p0 + 8 i + t
#pragma unroll
  for (int jf = 0; jf < JF; ++jf) {
    const int j = jb + 32 * jf + l32;
    if (j >= r) continue;
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int i = 8 * (v >> 2) + 4 * g + (v & 3);
        const int64_t pp = p0 + 8 * i + t;
        if (pp < P) part[((int64_t)z * P + pp) * r + j] = acc[t][jf][v];
      }
  }
}

// ------------------------------------------------------------------------
// The same reduction for r <= 16 on 16x16x32 MFMAs (no wasted accumulator
// columns, so a wave holds 32 accumulators and two waves fit a SIMD): one
// wave per 128 columns p, slabs of 32 tokens.  Lane (c, q) (c = lane % 16,
// q = lane / 16) loads tokens ms + 8q + e (e < 8), columns p0 + 8c .. + 7;
// after the register transpose operand t holds, for row c, column
// p0 + 8c + t of those 8 tokens, and the V operand holds V[token][j = c].
// ------------------------------------------------------------------------
// NV = 2: a second V (V1, rank r1, partials part1) against the same Z, so
// that two layers that share their input (gate and up) take their dA from one
// pass over it.
template <int ZMODE, int NV>
__device__ __forceinline__ void lora_grad16_body(const uint16_t* __restrict__ Z0,
                                                          const uint16_t* __restrict__ Z1, int64_t M, int64_t P,
                                                          const float* __restrict__ V, int r, int64_t m_per_split,
                                                          float* __restrict__ part, const float* __restrict__ V1 = nullptr,
                                                          int r1 = 0, float* __restrict__ part1 = nullptr,
                                                          int vs = 0, int ps = 0) {
  // vs: row stride of V (r unless V is a column slice of a wider matrix);
  // ps: row stride of the partials (r unless set)
  const int vstride = vs ? vs : r, pstride = ps ? ps : r;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, q = lane >> 4;
  const int64_t p0 = ((int64_t)blockIdx.x * 4 + wave) * 128;
  if (p0 >= P) return;
  const int z = blockIdx.y;
  const int64_t mb = (int64_t)z * m_per_split;
  const int64_t me = min(M, mb + m_per_split);
  int64_t pc = p0 + 8 * c;
  if (pc > P - 8) pc = P - 8;
  const int jv = c < r ? c : r - 1;
  const int jv1 = NV > 1 ? (c < r1 ? c : r1 - 1) : 0;

  f32x4 acc[NV][8];
#pragma unroll
  for (int k = 0; k < NV; ++k)
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[k][t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  constexpr int NZ = ZMODE == 0 ? 1 : 2;
  struct Slab {
    u32x4 raw[NZ][8];
    float x[NV][8];
  };
  auto load = [&](int64_t ms, Slab& S) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      int64_t mm = ms + 8 * q + e;
      if (mm >= me) mm = me - 1;
      S.raw[0][e] = *reinterpret_cast<const u32x4*>(Z0 + mm * P + pc);
      if constexpr (ZMODE == 1) S.raw[NZ - 1][e] = *reinterpret_cast<const u32x4*>(Z1 + mm * P + pc);
      S.x[0][e] = V[mm * vstride + jv];
      if constexpr (NV > 1) S.x[NV - 1][e] = V1[mm * r1 + jv1];
    }
  };
  auto slab = [&](int64_t ms, const Slab& S) {
    u32x4 rows[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const bool ok = ms + 8 * q + e < me;
      if constexpr (ZMODE == 0) {
        rows[e] = ok ? S.raw[0][e] : u32x4{0u, 0u, 0u, 0u};
      } else {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const float g0 = bf16_lo(S.raw[0][e][d]), g1 = bf16_hi(S.raw[0][e][d]);
          const float h0 = g0 * sigmoid_fast(g0) * bf16_lo(S.raw[1][e][d]);
          const float h1 = g1 * sigmoid_fast(g1) * bf16_hi(S.raw[1][e][d]);
          rows[e][d] = ok ? pack_bf16x2(h0, h1) : 0u;
        }
      }
    }
    u32x4 aop[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
      for (int d = 0; d < 4; ++d)
        aop[t][d] = __builtin_amdgcn_perm(rows[2 * d + 1][t >> 1], rows[2 * d][t >> 1], sel);
    }
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int rk = k == 0 ? r : r1;
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = (c < rk && ms + 8 * q + e < me) ? S.x[k][e] : 0.0f;
      const u32x4 vop{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                      pack_bf16x2(x[6], x[7])};
#pragma unroll
      for (int t = 0; t < 8; ++t) acc[k][t] = mfma16k32(aop[t], vop, acc[k][t]);
    }
  };
  Slab ra, rb;
  int64_t ms = mb;
  // unconditional prefetches (rows past the split are clamped to its last
  // row and masked), so that the compiler can count the loads in flight
  load(ms, ra);
  for (; ms + 32 < me; ms += 64) {
    load(ms + 32, rb);
    __builtin_amdgcn_sched_barrier(0);  // the prefetch is issued before the products
    slab(ms, ra);
    load(ms + 64, ra);
    __builtin_amdgcn_sched_barrier(0);
    slab(ms + 32, rb);
  }
  if (ms < me) slab(ms, ra);

  // acc[k][t][v] = C[row 4q + v][j = c]: column p = p0 + 8 (4q + v) + t
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int rk = k == 0 ? r : r1, sk = k == 0 ? pstride : r1;
    float* pk = k == 0 ? part : part1;
    if (c >= rk) continue;
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t pp = p0 + 8 * (4 * q + v) + t;
        if (pp < P) pk[((int64_t)z * P + pp) * sk + c] = acc[k][t][v];
      }
  }
}

template <int ZMODE>
__global__ __launch_bounds__(256) void lora_grad16_kernel(const uint16_t* __restrict__ Z0,
                                                          const uint16_t* __restrict__ Z1, int64_t M, int64_t P,
                                                          const float* __restrict__ V, int r, int64_t m_per_split,
                                                          float* __restrict__ part) {
  lora_grad16_body<ZMODE, 1>(Z0, Z1, M, P, V, r, m_per_split, part);
}

// Packed LoRA groups (one layer whose B is block-diagonal): dB_g only needs
// group g's own ranks of XA, so the wave over columns [p0, p0 + 128) (all of
// one group, its boundaries being multiples of 128) reduces against the
// column slice XA[:, roff_g .. roff_g + r_g) of the [M, Rt] matrix.  Partials
// [S][P][16], rank j of column p at p * 16 + j.
__global__ __launch_bounds__(256) void lora_grad16_grouped_kernel(GroupDesc d, const uint16_t* __restrict__ Z,
                                                                  int64_t M, int64_t P, const float* __restrict__ V,
                                                                  int Rt, int64_t m_per_split,
                                                                  float* __restrict__ part) {
  const int64_t p0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 128;
  if (p0 >= P) return;
  const int g = group_of(d, (int)p0);
  lora_grad16_body<0, 1>(Z, nullptr, M, P, V + d.roff[g], d.roff[g + 1] - d.roff[g], m_per_split, part, nullptr, 0,
                         nullptr, Rt, 16);
}

// dB_g = bf16(s_g sum_z part[z]) for the partials of lora_grad16_grouped_kernel
__global__ __launch_bounds__(256) void grouped_grad_finish_kernel(GroupDesc d, const float* __restrict__ part, int S,
                                                                  int64_t P) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= P * 16) return;
  const int p = (int)(i >> 4), j = (int)(i & 15);
  const int g = group_of(d, p);
  const int rg = d.roff[g + 1] - d.roff[g];
  if (j >= rg) return;
  float acc = 0.0f;
  const int64_t stride = P * 16;
  int z = 0;
  for (; z + 8 <= S; z += 8) {  // 8 loads in flight, added in split order
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = part[(int64_t)(z + u) * stride + i];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += v[u];
  }
  for (; z < S; ++z) acc += part[(int64_t)z * stride + i];
  d.dB[g][(int64_t)(p - d.noff[g]) * rg + j] = (uint16_t)(pack_bf16x2(d.s[g] * acc, 0.0f) & 0xFFFFu);
}

// the two-V form, held to two waves per SIMD
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void lora_grad16x2_kernel(
    const uint16_t* __restrict__ Z, int64_t M, int64_t P, const float* __restrict__ V0, int r0,
    int64_t m_per_split, float* __restrict__ part0, const float* __restrict__ V1, int r1,
    float* __restrict__ part1) {
  lora_grad16_body<0, 2>(Z, nullptr, M, P, V0, r0, m_per_split, part0, V1, r1, part1);
}

// ------------------------------------------------------------------------
// Both LoRA products of one gradient operand from a single pass over it
// ("Speed Up Fine-Tuning 2x with Unsloth", item 2, the adapters' fused
// backward): T = Z B (reduction over the P columns) and dB = s Z^T V
// (reduction over the M tokens), r <= 16.  Workgroup (x, y, z): columns
// [512 x, 512 x + 512) (wave w: 128 of them), token split y, job z.
//   dB side: as lora_grad16_kernel (lane (c, q) loads 8 tokens x 8 columns,
//     transposes them in registers, 8 MFMAs per 32-token slab against V).
//   T side: the wave's 32 x 128 slab goes to its own LDS region as loaded
//     (row-major, 16-byte chunk h of token row t at position h ^ (t % 16),
//     so that the writes and the reads below hit distinct banks); lane
//     (c, q) reads tokens 16 f + c at columns p0 + 32 s + 8 q, the B operand
//     of 16x16x32 MFMAs whose A operand is Bt (rank j = c, loaded once); the
//     four waves' 128-column sums of a slab are added in LDS in wave order
//     and written as this column block's partial.
// Z crosses HBM once; the operands never leave the CU.
// ------------------------------------------------------------------------
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void lora_pair16_kernel(PairArgs a) {
  __shared__ float tred[2][4][2 * 4 * 64];
  __shared__ __attribute__((aligned(16))) uint16_t zs[4][32 * 128];
  __shared__ u32x4 bts[4][4 * 64];
  const PairJob& J = a.job[blockIdx.z];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = lane & 15, q = lane >> 4;
  const int64_t M = a.M, P = a.P;
  const int r = J.r;
  const uint16_t* Z = J.Z;
  const int64_t p0 = ((int64_t)blockIdx.x * 4 + wave) * 128;
  const int64_t mb = (int64_t)blockIdx.y * a.m_per_split;
  const int64_t me = min(M, mb + a.m_per_split);
  int64_t pc = p0 + 8 * c;
  if (pc > P - 8) pc = P - 8;
  const int jv = c < r ? c : r - 1;
  // T side: rank c of Bt at this lane's 4 column chunks (zero past P / r),
  // kept in the wave's LDS slot [s][lane] (fewer live registers: two waves
  // per SIMD)
  u32x4* btw = bts[wave];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int64_t col = p0 + 32 * s + 8 * q;
    btw[s * 64 + lane] = (c < r && col < P) ? *reinterpret_cast<const u32x4*>(J.Bt + (int64_t)c * P + col)
                                            : u32x4{0u, 0u, 0u, 0u};
  }
  uint16_t* zw = zs[wave];
  // this workgroup's rows of the T partial (tokens [mb, me) of column block x)
  const __amdgpu_buffer_rsrc_t trs = __builtin_amdgcn_make_buffer_rsrc(
      J.tpart + ((int64_t)blockIdx.x * M + mb) * r, (short)0, (int)((me > mb ? me - mb : 0) * r * 4), 0x00020000);

  f32x4 acc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  struct Slab {
    u32x4 raw[8];
    float x[8];
  };
  auto load = [&](int64_t ms, Slab& S) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      int64_t mm = ms + 8 * q + e;
      if (mm >= me) mm = me - 1;
      S.raw[e] = *reinterpret_cast<const u32x4*>(Z + mm * P + pc);
      S.x[e] = J.V[mm * r + jv];
    }
  };
  auto slab = [&](int64_t ms, const Slab& S, int buf) {
    // the slab into this wave's region: token 8 q + e, chunk c
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int t = 8 * q + e;
      *reinterpret_cast<u32x4*>(zw + t * 128 + ((c ^ (t & 15)) * 8)) = S.raw[e];
    }
    // dB side
    u32x4 rows[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) rows[e] = (ms + 8 * q + e < me) ? S.raw[e] : u32x4{0u, 0u, 0u, 0u};
    u32x4 aop[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
      for (int d = 0; d < 4; ++d)
        aop[t][d] = __builtin_amdgcn_perm(rows[2 * d + 1][t >> 1], rows[2 * d][t >> 1], sel);
    }
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (c < r && ms + 8 * q + e < me) ? S.x[e] : 0.0f;
    const u32x4 vop{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                    pack_bf16x2(x[6], x[7])};
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[t] = mfma16k32(aop[t], vop, acc[t]);
    // T side: ta[f][v] = T partial [token ms + 16 f + c][j = 4 q + v]
    f32x4 ta[2];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      ta[f] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      const int t = 16 * f + c;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const u32x4 zt = *reinterpret_cast<const u32x4*>(zw + t * 128 + (((4 * s + q) ^ (t & 15)) * 8));
        ta[f] = mfma16k32(btw[s * 64 + lane], zt, ta[f]);
      }
    }
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int v = 0; v < 4; ++v) tred[buf][wave][(f * 4 + v) * 64 + lane] = ta[f][v];
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int e = tid + 256 * k;  // (f, v, lane)
      const float sum = tred[buf][0][e] + tred[buf][1][e] + tred[buf][2][e] + tred[buf][3][e];
      const int ln = e & 63, v = (e >> 6) & 3, f = e >> 8;
      const int64_t tok = ms + 16 * f + (ln & 15);
      const int j = 4 * (ln >> 4) + v;
      // a buffer store without a branch (dropped out of range), so that the
      // loads in flight stay countable
      const uint32_t o = (tok < me && j < r) ? (uint32_t)(((tok - mb) * r + j) * 4) : 0x80000000u;
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, sum), trs, o, 0, 0);
    }
  };
  Slab ra, rb;
  int64_t ms = mb;
  // unconditional prefetches (rows past the split are clamped to its last
  // row and masked), so that the compiler can count the loads in flight
  load(ms, ra);
  for (; ms + 32 < me; ms += 64) {
    load(ms + 32, rb);
    __builtin_amdgcn_sched_barrier(0);  // the prefetch is issued before the products
    slab(ms, ra, 0);
    load(ms + 64, ra);
    __builtin_amdgcn_sched_barrier(0);
    slab(ms + 32, rb, 1);
  }
  if (ms < me) slab(ms, ra, 0);

  // dB side: acc[t][v] = C[row 4q + v][j = c], column p = p0 + 8 (4q + v) + t
  if (c >= r) return;
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t pp = p0 + 8 * (4 * q + v) + t;
      if (pp < P) J.gpart[((int64_t)blockIdx.y * P + pp) * r + c] = acc[t][v];
    }
}

// sum_{i < n} src[i * stride], added in index order, 8 loads in flight
__device__ __forceinline__ float ordered_sum(const float* __restrict__ src, int n, int64_t stride) {
  float s = 0.0f;
  int i = 0;
  for (; i + 8 <= n; i += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = src[(int64_t)(i + u) * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += v[u];
  }
  for (; i < n; ++i) s += src[(int64_t)i * stride];
  return s;
}

// T = sum_b tpart[b] (fp32, [M, r]) and dB = bf16(s sum_z gpart[z]) ([P, r])
// of every job, each sum in fixed order.
__global__ __launch_bounds__(256) void pair_finish_kernel(PairArgs a) {
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (int k = 0; k < a.njobs; ++k) {
    const PairJob& J = a.job[k];
    const int64_t nt = a.M * J.r, ng = a.P * J.r;
    if (i < nt) {
      const float v = ordered_sum(J.tpart + i, a.nb, nt);
      J.T[i] = v;
      if (J.Tt) {
        const int64_t m = i / J.r;
        const int j = (int)(i - m * J.r);
        uint16_t* row = J.Tt + (int64_t)j * J.tt_ld;
        row[m] = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xFFFFu);
        if (m == a.M - 1)
          for (int64_t mm = a.M; mm < J.tt_ld; ++mm) row[mm] = 0;
      }
      return;
    }
    i -= nt;
    if (i < ng) {
      J.dB[i] = (uint16_t)(pack_bf16x2(J.s * ordered_sum(J.gpart + i, a.S, ng), 0.0f) & 0xFFFFu);
      return;
    }
    i -= ng;
  }
}

// out = bf16(s * sum_z part[z]), layout [P, r] (dB) or [r, P] (dA).
__global__ __launch_bounds__(256) void grad_finish_kernel(const float* __restrict__ part, int S, int64_t P, int r,
                                                          float s, int out_rp, uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= P * r) return;
  float acc = 0.0f;
  const int64_t stride = P * r;
  int z = 0;
  for (; z + 8 <= S; z += 8) {  // 8 loads in flight, added in split order
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = part[(int64_t)(z + u) * stride + i];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += v[u];
  }
  for (; z < S; ++z) acc += part[(int64_t)z * stride + i];
  acc *= s;
  const int64_t pp = i / r;
  const int j = (int)(i % r);
  const uint32_t b = pack_bf16x2(acc, 0.0f) & 0xFFFFu;
  if (out_rp)
    out[(int64_t)j * P + pp] = (uint16_t)b;
  else
    out[i] = (uint16_t)b;
}

__global__ __launch_bounds__(256) void zero_u16_kernel(uint16_t* __restrict__ out, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) out[i] = 0;
}

}  // namespace qk

// ==========================================================================
// Launchers (called by the C ABI in qlora_api.hip)
// ==========================================================================
using namespace qk;

static inline unsigned grid1(int64_t n, int per) { return (unsigned)((n + per - 1) / per); }

hipError_t launch_nf4_quantize(const float* W, int64_t nblocks, const float* codebook, int dq, uint8_t* codes,
                               float* absmax, uint8_t* absmax_q, float* absmax_scale, hipStream_t st) {
  if (nblocks == 0) return hipSuccess;
  nf4_quantize_kernel<<<grid1(nblocks, 256), 256, 0, st>>>(W, nblocks, codebook, dq, codes, absmax, absmax_q,
                                                           absmax_scale);
  return hipGetLastError();
}

hipError_t launch_nf4_dequantize(const Nf4Dev& w, const float* codebook, int out_f32, void* out, hipStream_t st) {
  const int64_t n8 = w.N * w.K / 8;
  if (n8 == 0) return hipSuccess;
  nf4_dequantize_kernel<<<grid1(n8, 256), 256, 0, st>>>(w, codebook, n8, out_f32, out);
  return hipGetLastError();
}

template <int MODE, int WM, int WN, int FM, int FN, bool DQ, bool ALDS>
static hipError_t run_gemm(GemmArgs a, const qplan::GemmPlan& pl, hipStream_t st) {
  constexpr int NT = WM * WN * 64;
  constexpr int BM = WM * FM * 32;
  constexpr int BNO = (MODE == MODE_FWD_SWIGLU ? WN * FN * 16 : WN * FN * 32);
  a.tiles_m = (a.M + BM - 1) / BM;
  a.tiles_n = (a.Nout + BNO - 1) / BNO;
  a.ktiles_per_split = pl.ktiles_per_split;
  dim3 grid((unsigned)(a.tiles_m * a.tiles_n), (unsigned)pl.splits);
  if (pl.splits > 1) {
    if constexpr (MODE == MODE_FWD || MODE == MODE_BWD) {
      qgemm_kernel<MODE, WM, WN, FM, FN, true, DQ, ALDS><<<grid, NT, 0, st>>>(a);
    } else {
      return hipErrorInvalidValue;
    }
  } else {
    qgemm_kernel<MODE, WM, WN, FM, FN, false, DQ, ALDS><<<grid, NT, 0, st>>>(a);
  }
  return hipGetLastError();
}

template <int MODE, bool DQ>
static hipError_t run_gemm_cfg(const GemmArgs& a, const qplan::GemmPlan& pl, hipStream_t st) {
  if (pl.cfg == qplan::CFG_L256) return run_gemm<MODE, 4, 2, 2, 4, DQ, true>(a, pl, st);
  if constexpr (MODE == MODE_BWD) {
    if (pl.cfg == qplan::CFG_SKINNY_TR) return run_gemm<MODE, 1, 8, 2, 1, DQ, true>(a, pl, st);
  }
  if constexpr (MODE == MODE_FWD_SWIGLU) {
    return run_gemm<MODE, 1, 2, 2, 2, DQ, false>(a, pl, st);
  } else {
    return run_gemm<MODE, 1, 2, 2, 1, DQ, false>(a, pl, st);
  }
}

template <int MODE>
static hipError_t run_mode(const GemmArgs& a, const qplan::GemmPlan& pl, hipStream_t st) {
  return a.w0.dq ? run_gemm_cfg<MODE, true>(a, pl, st) : run_gemm_cfg<MODE, false>(a, pl, st);
}

hipError_t launch_qgemm(int mode, const GemmArgs& a, const qplan::GemmPlan& pl, hipStream_t st) {
  switch (mode) {
    case MODE_FWD: return run_mode<MODE_FWD>(a, pl, st);
    case MODE_FWD_SWIGLU: return run_mode<MODE_FWD_SWIGLU>(a, pl, st);
    case MODE_BWD: return run_mode<MODE_BWD>(a, pl, st);
    case MODE_BWD_SWIGLU: return run_mode<MODE_BWD_SWIGLU>(a, pl, st);
    case MODE_BWD_DUAL: return run_mode<MODE_BWD_DUAL>(a, pl, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_splitk_finish(const float* part, int splits, int64_t M, int64_t Nout, uint16_t* out,
                                hipStream_t st) {
  const int64_t mn = M * Nout;
  if (mn == 0) return hipSuccess;
  splitk_finish_kernel<<<grid1(mn / 4, 256), 256, 0, st>>>(part, splits, mn, out);
  return hipGetLastError();
}

hipError_t launch_lora_down(const uint16_t* Z, int64_t M, int64_t Kred, const uint16_t* W0, int r0,
                            const uint16_t* W1, int r1, float* V0, float* V1, int splits, float* part,
                            hipStream_t st, bool finish, bool w_nr, uint16_t* Xt, int Mp) {
  if (M == 0) return hipSuccess;
  // rank <= 16: 16-token workgroups for at most 64 tokens (same splits, so
  // the partial layout [S][M][rt] is unchanged), else 32-token ones
  const int nf = (r0 + r1 <= 16 && M <= 64) ? 1 : 2;
  // the [Kred, r0] weight layout and the re-laid-out copy exist in the
  // rank <= 16 form only, one at a time
  if ((w_nr || Xt) && (r0 + r1 > 16 || (w_nr && (r1 != 0 || Xt)) || (Xt && (Mp < M || Mp > 16 * nf * grid1(M, 16 * nf)))))
    return hipErrorInvalidValue;
  const int64_t C = Kred / 64;
  const int64_t per = (C + splits - 1) / splits;
  const int S = (int)((C + per - 1) / per);
  // tokens per workgroup as qplan::down_tokens, which the split plan assumed
  const int tpw = qplan::down_tokens(r0 + r1);
  dim3 grid(grid1(M, tpw), (unsigned)S);
  float* pp = S > 1 ? part : nullptr;
  int jf = (r0 + r1 + 31) / 32;
  if (r0 + r1 <= 16) {
    const dim3 g16(grid1(M, 16 * nf), (unsigned)S);
    if (nf == 1) {
      if (w_nr)
        lora_down16_kernel<true, false, 1><<<g16, 512, 0, st>>>(Z, M, Kred, W0, r0, W1, r1, V0, V1, per, pp, nullptr,
                                                                0);
      else if (Xt)
        lora_down16_kernel<false, true, 1><<<g16, 512, 0, st>>>(Z, M, Kred, W0, r0, W1, r1, V0, V1, per, pp, Xt, Mp);
      else
        lora_down16_kernel<false, false, 1><<<g16, 512, 0, st>>>(Z, M, Kred, W0, r0, W1, r1, V0, V1, per, pp,
                                                                 nullptr, 0);
    } else {
      if (w_nr)
        lora_down16_kernel<true, false, 2><<<g16, 512, 0, st>>>(Z, M, Kred, W0, r0, W1, r1, V0, V1, per, pp, nullptr,
                                                                0);
      else if (Xt)
        lora_down16_kernel<false, true, 2><<<g16, 512, 0, st>>>(Z, M, Kred, W0, r0, W1, r1, V0, V1, per, pp, Xt, Mp);
      else
        lora_down16_kernel<false, false, 2><<<g16, 512, 0, st>>>(Z, M, Kred, W0, r0, W1, r1, V0, V1, per, pp,
                                                                 nullptr, 0);
    }
    jf = 0;
  }
  switch (jf) {
    case 0: break;
    case 1: lora_down_kernel<1, 1><<<grid, 512, 0, st>>>(Z, M, Kred, W0, r0, W1, r1, V0, V1, per, pp); break;
    case 2:
      if (tpw == 64)
        lora_down_kernel<2, 2><<<grid, 512, 0, st>>>(Z, M, Kred, W0, r0, W1, r1, V0, V1, per, pp);
      else
        lora_down_kernel<2, 1><<<grid, 512, 0, st>>>(Z, M, Kred, W0, r0, W1, r1, V0, V1, per, pp);
      break;
    case 3: lora_down_kernel<3, 1><<<grid, 512, 0, st>>>(Z, M, Kred, W0, r0, W1, r1, V0, V1, per, pp); break;
    case 4: lora_down_kernel<4, 1><<<grid, 512, 0, st>>>(Z, M, Kred, W0, r0, W1, r1, V0, V1, per, pp); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || S == 1 || !finish) return e;
  down_finish_kernel<<<grid1(M * (r0 + r1), 256), 256, 0, st>>>(part, S, M, r0, r1, V0, V1);
  return hipGetLastError();
}

hipError_t launch_grouped_bcat(const GroupDesc& d, int Nt, int Rt, uint16_t* out, hipStream_t st) {
  const int64_t n = (int64_t)Nt * Rt;
  if (n == 0) return hipSuccess;
  grouped_bcat_kernel<<<grid1(n, 256), 256, 0, st>>>(d, Nt, Rt, out);
  return hipGetLastError();
}

hipError_t launch_grouped_db(const GroupDesc& d, int Nt, int Rt, const uint16_t* dbcat, hipStream_t st) {
  const int64_t n = (int64_t)Nt * Rt;
  if (n == 0) return hipSuccess;
  grouped_db_kernel<<<grid1(n, 256), 256, 0, st>>>(d, Nt, Rt, dbcat);
  return hipGetLastError();
}

hipError_t launch_transpose_multi(const TransposeJobs& J, hipStream_t st) {
  if (J.n < 1 || J.n > 6) return hipErrorInvalidValue;
  int64_t tiles = 0, elems = 0;
  for (int k = 0; k < J.n; ++k) {
    // the kernel's tile shape (transpose_tile_shape)
    const int lc = J.cols[k] <= 16 ? 4 : (J.rows[k] <= 16 ? 8 : 6), lr = 12 - lc;
    tiles += ((J.rows[k] + (1 << lr) - 1) >> lr) * ((J.cols[k] + (1 << lc) - 1) >> lc);
    elems += J.rows[k] * J.cols[k];
  }
  if (elems == 0) return hipSuccess;
  if (elems < ((int64_t)1 << 21)) {
    // measured: 7.8 us per element-wise launch against 10-12 us tiled for the
    // six factors of a rank-16 Llama-3-8B MLP (0.9 M elements); tiled 15.6 us
    // against 40.5 us for the rank-64 Llama-3-70B MLP's (7.1 M)
    transpose_elem_kernel<<<grid1(elems, 256), 256, 0, st>>>(J);
    return hipGetLastError();
  }
  if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
  transpose_multi_kernel<<<(unsigned)tiles, 256, 0, st>>>(J);
  return hipGetLastError();
}

hipError_t launch_transpose_rn(const uint16_t* B, int64_t N, int r, uint16_t* BT, hipStream_t st) {
  if (N * r == 0) return hipSuccess;
  transpose_rn_kernel<<<grid1(N * r, 256), 256, 0, st>>>(B, N, r, BT);
  return hipGetLastError();
}

void plan_lora_pair(PairArgs& a, int64_t M, int64_t P, int r, int njobs) {
  int msplits = qplan::plan_pair_msplits(M, P, r);
  // Whole rounds of workgroups: two fit on a CU (64 KB of LDS each), and a
  // last round that is mostly empty leaves the chip idle for its duration
  // (the dG / dU launch of the Llama-3-8B MLP: 2 x 28 x 19 = 1064 = two
  // rounds and 40; with 18 splits, 1008: 118.7 -> 116.5 us).  Fewer splits
  // only shrink the partials, so the buffers sized by
  // qplan::pair_part_floats still hold them.
  const int64_t nbk = (P + 511) / 512, per_round = 2 * qplan::kNumCUs;
  const int64_t total = (int64_t)(njobs > 1 ? njobs : 1) * nbk * msplits;
  if (total > per_round && total % per_round != 0) {
    const int64_t s = (total / per_round) * per_round / ((njobs > 1 ? njobs : 1) * nbk);
    if (s >= 1 && s < msplits) msplits = (int)s;
  }
  const int64_t mps = (((M + msplits - 1) / msplits) + 31) / 32 * 32;
  a.M = M;
  a.P = P;
  a.m_per_split = mps > 0 ? mps : 32;
  a.S = (int)((M + a.m_per_split - 1) / a.m_per_split);
  a.nb = (int)((P + 511) / 512);
}

hipError_t launch_lora_pair(const PairArgs& a, hipStream_t st) {
  if (a.M == 0 || a.P == 0 || a.njobs < 1 || a.njobs > 2) return a.njobs < 1 || a.njobs > 2 ? hipErrorInvalidValue
                                                                                              : hipSuccess;
  for (int k = 0; k < a.njobs; ++k)
    if (a.job[k].r < 1 || a.job[k].r > 16) return hipErrorInvalidValue;
  if (a.P % 8 != 0) return hipErrorInvalidValue;
  lora_pair16_kernel<<<dim3((unsigned)a.nb, (unsigned)a.S, (unsigned)a.njobs), 256, 0, st>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int64_t n = 0;
  for (int k = 0; k < a.njobs; ++k) n += (a.M + a.P) * a.job[k].r;
  pair_finish_kernel<<<grid1(n, 256), 256, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_grad_finish(const float* part, int S, int64_t P, int r, float s, int out_rp, uint16_t* out,
                              hipStream_t st) {
  if (P * r == 0) return hipSuccess;
  grad_finish_kernel<<<grid1(P * r, 256), 256, 0, st>>>(part, S, P, r, s, out_rp, out);
  return hipGetLastError();
}

// Two finishes in one launch: out_k = bf16(s_k sum_z part_k[z]) as [r_k, P].
__global__ __launch_bounds__(256) void grad_finish2_kernel(const float* __restrict__ part0, int r0, float s0,
                                                           uint16_t* __restrict__ out0,
                                                           const float* __restrict__ part1, int r1, float s1,
                                                           uint16_t* __restrict__ out1, int S, int64_t P) {
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const float* part = part0;
  int r = r0;
  float s = s0;
  uint16_t* out = out0;
  if (i >= P * r0) {
    i -= P * r0;
    if (i >= P * r1) return;
    part = part1;
    r = r1;
    s = s1;
    out = out1;
  }
  float acc = 0.0f;
  const int64_t stride = P * r;
  int z = 0;
  for (; z + 8 <= S; z += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = part[(int64_t)(z + u) * stride + i];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += v[u];
  }
  for (; z < S; ++z) acc += part[(int64_t)z * stride + i];
  const int64_t pp = i / r;
  const int j = (int)(i % r);
  out[(int64_t)j * P + pp] = (uint16_t)(pack_bf16x2(s * acc, 0.0f) & 0xFFFFu);
}

hipError_t launch_lora_grad2(const uint16_t* Z, int64_t M, int64_t P, const float* V0, int r0, float s0,
                             uint16_t* out0, const float* V1, int r1, float s1, uint16_t* out1, float* part,
                             hipStream_t st) {
  if (M == 0 || P == 0) return hipSuccess;
  if (r0 < 1 || r0 > 16 || r1 < 1 || r1 > 16 || P % 8 != 0) return hipErrorInvalidValue;
  const int rmax = r0 > r1 ? r0 : r1;
  const int msplits = qplan::plan_grad_msplits(M, P, rmax);
  const int64_t mps = (((M + msplits - 1) / msplits) + 31) / 32 * 32;
  const int S = (int)((M + mps - 1) / mps);
  float* part1 = part + (size_t)S * P * r0;
  lora_grad16x2_kernel<<<dim3(grid1(P, 512), (unsigned)S), 256, 0, st>>>(Z, M, P, V0, r0, mps, part, V1, r1, part1);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  grad_finish2_kernel<<<grid1(P * (r0 + r1), 256), 256, 0, st>>>(part, r0, s0, out0, part1, r1, s1, out1, S, P);
  return hipGetLastError();
}

bool grouped_grad_ok(const GroupDesc& d, int64_t P) {
  if (P % 8 != 0) return false;
  for (int g = 0; g < d.G; ++g) {
    if (d.roff[g + 1] - d.roff[g] > 16) return false;
    if (g > 0 && d.noff[g] % 128 != 0) return false;
  }
  return true;
}

hipError_t launch_grouped_grad(const GroupDesc& d, const uint16_t* Z, int64_t M, int64_t P, const float* V, int Rt,
                               int msplits, float* part, hipStream_t st) {
  if (M == 0 || !grouped_grad_ok(d, P)) return hipErrorInvalidValue;
  const int64_t mps = (((M + msplits - 1) / msplits) + 31) / 32 * 32;
  const int S = (int)((M + mps - 1) / mps);
  lora_grad16_grouped_kernel<<<dim3(grid1(P, 512), (unsigned)S), 256, 0, st>>>(d, Z, M, P, V, Rt, mps, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  grouped_grad_finish_kernel<<<grid1(P * 16, 256), 256, 0, st>>>(d, part, S, P);
  return hipGetLastError();
}

hipError_t launch_lora_grad(int zmode, const uint16_t* Z0, const uint16_t* Z1, int64_t M, int64_t P,
                            const float* V, int r, float s, int msplits, float* part, int out_rp, uint16_t* out,
                            hipStream_t st) {
  if (M == 0) {
    zero_u16_kernel<<<grid1(P * r, 256), 256, 0, st>>>(out, P * r);
    return hipGetLastError();
  }
  if (r <= 16) {
    // 16x16x32 form: slabs of 32 tokens, two waves per SIMD (measured 25-30%
    // less time than the 32-wide form on the Llama-3-8B MLP's gradients)
    const int64_t mps = (((M + msplits - 1) / msplits) + 31) / 32 * 32;
    const int S = (int)((M + mps - 1) / mps);
    dim3 grid(grid1(P, 512), (unsigned)S);
    if (zmode == 0)
      lora_grad16_kernel<0><<<grid, 256, 0, st>>>(Z0, Z1, M, P, V, r, mps, part);
    else
      lora_grad16_kernel<1><<<grid, 256, 0, st>>>(Z0, Z1, M, P, V, r, mps, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    grad_finish_kernel<<<grid1(P * r, 256), 256, 0, st>>>(part, S, P, r, s, out_rp, out);
    return hipGetLastError();
  }
  const int64_t mps = (((M + msplits - 1) / msplits) + 15) / 16 * 16;
  const int S = (int)((M + mps - 1) / mps);
  for (int jb = 0; jb < r; jb += 64) {
    const int jf = (r - jb) > 32 ? 2 : 1;
    dim3 grid(grid1(P, 1024), (unsigned)S);
    if (zmode == 0) {
      if (jf == 2)
        lora_grad_kernel<0, 2><<<grid, 256, 0, st>>>(Z0, Z1, M, P, V, r, jb, mps, part);
      else
        lora_grad_kernel<0, 1><<<grid, 256, 0, st>>>(Z0, Z1, M, P, V, r, jb, mps, part);
    } else {
      if (jf == 2)
        lora_grad_kernel<1, 2><<<grid, 256, 0, st>>>(Z0, Z1, M, P, V, r, jb, mps, part);
      else
        lora_grad_kernel<1, 1><<<grid, 256, 0, st>>>(Z0, Z1, M, P, V, r, jb, mps, part);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  grad_finish_kernel<<<grid1(P * r, 256), 256, 0, st>>>(part, S, P, r, s, out_rp, out);
  return hipGetLastError();
}
