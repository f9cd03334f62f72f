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
//   * codes and activations of the next two tiles are in flight while the
//     current one is expanded and multiplied (a ring of three register sets);
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
constexpr int SK_DEPTH = 3;   // register sets of the load ring (tiles in flight + 1)
constexpr int SK_ABS_LDS = 64 * 1024;  // bytes of block absmax staged per workgroup

// Byte offset of a codebook entry: 4 * (bits [8B + 2, 8B + 6) of x), i.e.
// with x = c << 2 the low nibble of byte B of c, with x = c >> 2 its high
// nibble, selected and masked by one SDWA instruction (the codebook sits at
// LDS address 0, so this is the lookup's address).
#define SK_NIB(B)                                                                                             \
  __device__ __forceinline__ uint32_t nib_off##B(uint32_t x) {                                                \
    uint32_t r;                                                                                               \
    asm("v_and_b32_sdwa %0, 60, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_" #B \
        : "=v"(r)                                                                                             \
        : "v"(x));                                                                                            \
    return r;                                                                                                 \
  }
SK_NIB(0)
SK_NIB(1)
SK_NIB(2)
SK_NIB(3)
#undef SK_NIB

// 8 codes of one dword -> their 8 fp32 codebook values, element order (cb
// is the codebook at LDS address 0)
__device__ __forceinline__ void sk_lookup8(const float* cb, uint32_t c, float* v) {
  const uint32_t lo = c << 2, hi = c >> 2;
  const char* t = reinterpret_cast<const char*>(cb);
  v[0] = *reinterpret_cast<const float*>(t + nib_off0(lo));
  v[1] = *reinterpret_cast<const float*>(t + nib_off0(hi));
  v[2] = *reinterpret_cast<const float*>(t + nib_off1(lo));
  v[3] = *reinterpret_cast<const float*>(t + nib_off1(hi));
  v[4] = *reinterpret_cast<const float*>(t + nib_off2(lo));
  v[5] = *reinterpret_cast<const float*>(t + nib_off2(hi));
  v[6] = *reinterpret_cast<const float*>(t + nib_off3(lo));
  v[7] = *reinterpret_cast<const float*>(t + nib_off3(hi));
}

// LDS of the forward kernel, the codebook first (LDS address 0, which the
// lookups above rely on: it is the kernel's only LDS object).
struct SkFwdSmem {
  float cb[16];
  float vs[64 * 64];  // V = sum of the down-projection partials, [M][r]
  // block absmax [row - n0][tile - kb] (row stride ntile + 4) during the main
  // loop; afterwards the per-wave partial tiles of the reduction
  float absl[SK_ABS_LDS / 4];
};

template <int FN, bool DQ>
__global__ __launch_bounds__(256) void skinny_fwd_kernel(SkinnyArgs p) {
  constexpr int TF = SK_TF;
  constexpr int R = 16 * FN;
  constexpr int D = SK_DEPTH;
  __shared__ SkFwdSmem sm;
  float* cb = sm.cb;
  float* vs = sm.vs;
  float* absl = sm.absl;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, q = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * R;
  const int KT = (int)(p.K / 64);
  const int kb = blockIdx.y * p.kps, ke = min(KT, kb + p.kps);
  const int kpw = (ke - kb + SK_WAVES - 1) / SK_WAVES;
  const int wb = min(ke, kb + wave * kpw), we = min(ke, wb + kpw);
  const int nt = we - wb;  // this wave's tiles
  const bool lora_here = blockIdx.y == 0 && p.r > 0;

  // ---- operands through buffer resources (the workgroup's code rows, the
  // activations) with 32-bit lane offsets and the tile offset in the scalar
  // offset; rows are clamped into range (clamped rows are not stored)
  const int rows = (int)min((int64_t)R, p.N - n0);
  const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.w.codes + n0 * (p.K / 2)), (short)0, (int)(rows * (p.K / 2)), 0x00020000);
  const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(p.X), (short)0,
                                                                      (int)(p.M * p.K * 2), 0x00020000);
  uint32_t coff[FN];
#pragma unroll
  for (int f = 0; f < FN; ++f) coff[f] = (uint32_t)(min(16 * f + l16, rows - 1) * (p.K / 2) + 8 * q);
  uint32_t xoff[TF];
#pragma unroll
  for (int i = 0; i < TF; ++i) xoff[i] = (uint32_t)(min(16 * i + l16, (int)p.M - 1) * p.K * 2 + 32 * q);

  struct Regs {
    u32x4 x[TF][2];
    u32x2 c[FN];
  };
  auto load = [&](int kt, Regs& g) {
#pragma unroll
    for (int f = 0; f < FN; ++f)
      g.c[f] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(crs, coff[f], kt * 32, 0));
#pragma unroll
    for (int i = 0; i < TF; ++i)
#pragma unroll
      for (int s = 0; s < 2; ++s)
        g.x[i][s] =
            __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xrs, xoff[i], kt * 128 + 16 * s, 0));
  };

  // the first D - 1 tiles are requested before anything else
  Regs g[D];
  if (nt > 0) {
#pragma unroll
    for (int u = 0; u < D - 1; ++u) load(wb + min(u, nt - 1), g[u]);
  }

  // ---- block absmax of the workgroup's rows and tiles into LDS as fp32,
  // row-major with row stride ntile + 4.  Row rr's tiles are contiguous in
  // memory; when they start and end on a 4-tile boundary they are read 4 at a
  // time (a 4-byte load of codes with double quantization, a 16-byte load
  // otherwise) and written as one 16-byte LDS store, all of a thread's loads
  // issued before the first is used.
  if (tid < 16) cb[tid] = p.codebook[tid];
  const int ntile = ke - kb;
  const int astr = ntile + 4;
  {
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
          f32x4 a4;
          if constexpr (DQ) {
#pragma unroll
            for (int u = 0; u < 4; ++u) a4[u] = (float)((cq[j] >> (8 * u)) & 0xFFu) * sc[j];
          } else {
            a4 = af[j];
          }
          *reinterpret_cast<f32x4*>(absl + rr * astr + 4 * g4) = a4;
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
            absl[rr * astr + t] = a[j];
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

  // Expansion and products of one tile, frag by frag: 16 codebook lookups,
  // times the block absmax, rounded to bf16, then step 0 of all token frags
  // and step 1 (dependent MFMAs TF apart).
  auto compute = [&](int kt, const Regs& gg) {
    const float* arow = absl + l16 * astr + (kt - kb);
#pragma unroll
    for (int f = 0; f < FN; ++f) {
      const float a = arow[16 * f * astr];
      float v[16];
      sk_lookup8(cb, gg.c[f][0], v);
      sk_lookup8(cb, gg.c[f][1], v + 8);
      u32x4 w[2];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
        w[s2] = u32x4{pack_bf16x2(v[8 * s2 + 0] * a, v[8 * s2 + 1] * a), pack_bf16x2(v[8 * s2 + 2] * a, v[8 * s2 + 3] * a),
                      pack_bf16x2(v[8 * s2 + 4] * a, v[8 * s2 + 5] * a), pack_bf16x2(v[8 * s2 + 6] * a, v[8 * s2 + 7] * a)};
#pragma unroll
      for (int i = 0; i < TF; ++i) acc[f][i] = mfma16(gg.x[i][0], w[0], acc[f][i]);
#pragma unroll
      for (int i = 0; i < TF; ++i) acc[f][i] = mfma16(gg.x[i][1], w[1], acc[f][i]);
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

  // ---- sum the wave partials in wave order and store, up to 4 frags per
  // round through the (now free) absmax region: per frag and wave 1024 values,
  // value e = 256 i + 64 v + lane of a frag being token 16 i + 4 (lane/16) + v,
  // weight row n0 + 16 f + lane%16.  A thread sums 4 consecutive values (4
  // consecutive rows of one token) and stores them as one 8-byte write.
  float* red = absl;
  constexpr int FR = 4;
#pragma unroll
  for (int f0 = 0; f0 < FN; f0 += FR) {
    __syncthreads();  // the region is free: main loop (or the previous round) done
#pragma unroll
    for (int fl = 0; fl < FR; ++fl) {
      if (f0 + fl < FN) {
#pragma unroll
        for (int i = 0; i < TF; ++i)
#pragma unroll
          for (int v = 0; v < 4; ++v) red[(fl * SK_WAVES + wave) * 1024 + 256 * i + 64 * v + lane] = acc[f0 + fl][i][v];
      }
    }
    __syncthreads();
#pragma unroll
    for (int fl = 0; fl < FR; ++fl) {
      if (f0 + fl >= FN) continue;
      const int e = 4 * tid;  // values e .. e + 3 of frag f0 + fl
      f32x4 sum = *reinterpret_cast<const f32x4*>(red + (fl * SK_WAVES) * 1024 + e);
#pragma unroll
      for (int w = 1; w < SK_WAVES; ++w) sum += *reinterpret_cast<const f32x4*>(red + (fl * SK_WAVES + w) * 1024 + e);
      const int ln = e & 63;
      const int64_t m = 16 * (e >> 8) + 4 * (ln >> 4) + ((e >> 6) & 3);
      const int64_t n = n0 + 16 * (f0 + fl) + (ln & 15);  // first of 4 consecutive rows
      if (m < p.M) {
        if (p.part) {
#pragma unroll
          for (int u = 0; u < 4; ++u)
            if (n + u < p.N) p.part[((int64_t)blockIdx.y * p.M + m) * p.N + n + u] = sum[u];
        } else if (n + 3 < p.N) {
          *reinterpret_cast<u32x2*>(p.out + m * p.N + n) =
              u32x2{pack_bf16x2(sum[0], sum[1]), pack_bf16x2(sum[2], sum[3])};
        } else {
#pragma unroll
          for (int u = 0; u < 4; ++u)
            if (n + u < p.N) p.out[m * p.N + n + u] = (uint16_t)(pack_bf16x2(sum[u], 0.0f) & 0xFFFFu);
        }
      }
    }
  }

}


// ------------------------------------------------------------------------
// Skinny-M backward finish ("LLM Fine-Tuning in 2026: Unsloth vs QLoRA vs
// Liger-Kernel", section 2): one launch after the split transposed product.
// Workgroups [0, K/32) own 32 columns k of the input side:
//   dX[:, k] = sum_z part[z][:, k] + s T A[:, k]     (T = sum_z tpart[z])
//   dA[:, k] = s T^T X[:, k]
// workgroups [K/32, K/32 + N/64) own 64 rows n of B:
//   dB[n, :] = s dY[:, n]^T XA
// Every sum runs in fp32 in a fixed order.
// ------------------------------------------------------------------------
// LDS (dynamic, sized by the rank so that small ranks keep several
// workgroups per CU): vs [64][r] T or XA, zs [64][68] a 64-column block of X
// or dY (+4 pad), as [r][32] a 32-column block of A.
__global__ __launch_bounds__(256) void skinny_bwd_finish_kernel(SkinnyFinishArgs p) {
  extern __shared__ float fin_smem[];
  const int tid = threadIdx.x;
  const int M = (int)p.M, r = p.r;
  float* vs = fin_smem;
  float* zs = vs + 64 * r;
  float* as = zs + 64 * 68;
  const int nkb = (int)(p.K / 32);
  // bf16 [M][cols] block at src (row stride ld) -> zs as fp32, 8 columns per load
  auto stage_block = [&](const uint16_t* src, int64_t ld, int cols) {
    const int n8 = cols / 8;
    for (int e = tid; e < M * n8; e += 256) {
      const int m = e / n8, c8 = (e - m * n8) * 8;
      const u32x4 v = *reinterpret_cast<const u32x4*>(src + (int64_t)m * ld + c8);
      float* d = zs + m * 68 + c8;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        d[2 * u] = bf16_lo(v[u]);
        d[2 * u + 1] = bf16_hi(v[u]);
      }
    }
  };
  if ((int)blockIdx.x < nkb) {
    const int64_t k0 = (int64_t)blockIdx.x * 32;
    // dX: 8 threads per row, 4 columns each, rows tid / 8 and tid / 8 + 32.
    // With at most 8 splits the partials of both rows are requested first,
    // so they are in flight while T, X and A are staged.
    const int cq = (tid & 7) * 4;
    constexpr int PZ = 8;
    const bool early = p.splits <= PZ;
    f32x4 pre[2][PZ];
    if (early) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int m = min((tid >> 3) + 32 * h, M - 1);
        const float* src = p.part + (int64_t)m * p.K + k0 + cq;
#pragma unroll
        for (int zz = 0; zz < PZ; ++zz)
          pre[h][zz] = *reinterpret_cast<const f32x4*>(src + (int64_t)min(zz, p.splits - 1) * M * p.K);
      }
    }
    // T = sum_z tpart[z] (split order), loads of 8 splits in flight
    for (int e0 = tid; e0 < M * r; e0 += 256 * 4) {
      float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      for (int z0 = 0; z0 < p.tsplits; z0 += 8) {
        float t[4][8];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int zz = 0; zz < 8; ++zz)
            t[j][zz] = p.tpart[(int64_t)min(z0 + zz, p.tsplits - 1) * M * r + min(e0 + 256 * j, M * r - 1)];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int zz = 0; zz < 8; ++zz)
            if (z0 + zz < p.tsplits) v[j] += t[j][zz];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (e0 + 256 * j < M * r) vs[e0 + 256 * j] = v[j];
    }
    stage_block(p.X + k0, p.K, 32);
    for (int e = tid; e < r * 4; e += 256) {
      const int j = e >> 2, c8 = (e & 3) * 8;
      const u32x4 v = *reinterpret_cast<const u32x4*>(p.A + (int64_t)j * p.K + k0 + c8);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        as[j * 32 + c8 + 2 * u] = bf16_lo(v[u]);
        as[j * 32 + c8 + 2 * u + 1] = bf16_hi(v[u]);
      }
    }
    __syncthreads();
    // the split partials of a row are added in split order (loaded above,
    // or here 8 splits at a time)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int m = (tid >> 3) + 32 * h;
      if (m >= M) break;
      const float* src = p.part + (int64_t)m * p.K + k0 + cq;
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
      if (early) {
#pragma unroll
        for (int zz = 0; zz < PZ; ++zz)
          if (zz < p.splits) acc += pre[h][zz];
      } else {
        for (int z0 = 0; z0 < p.splits; z0 += 8) {
          f32x4 t[8];
#pragma unroll
          for (int zz = 0; zz < 8; ++zz)
            t[zz] = *reinterpret_cast<const f32x4*>(src + (int64_t)min(z0 + zz, p.splits - 1) * M * p.K);
#pragma unroll
          for (int zz = 0; zz < 8; ++zz)
            if (z0 + zz < p.splits) acc += t[zz];
        }
      }
      float lo[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      for (int j = 0; j < r; ++j) {
        const float v = vs[m * r + j];
#pragma unroll
        for (int u = 0; u < 4; ++u) lo[u] += v * as[j * 32 + cq + u];
      }
      *reinterpret_cast<u32x2*>(p.dX + (int64_t)m * p.K + k0 + cq) =
          u32x2{pack_bf16x2(acc[0] + p.s * lo[0], acc[1] + p.s * lo[1]),
                pack_bf16x2(acc[2] + p.s * lo[2], acc[3] + p.s * lo[3])};
    }
    // dA[j, k0 + c] = s sum_m T[m, j] X[m, k0 + c]; with an even rank each
    // thread takes ranks j, j + 1 (one 8-byte read of T per token)
    const int c = tid & 31;
    if ((r & 1) == 0) {
      for (int j = 2 * (tid >> 5); j < r; j += 16) {
        float a0 = 0.0f, a1 = 0.0f;
        for (int m = 0; m < M; ++m) {
          const float2 t = *reinterpret_cast<const float2*>(vs + m * r + j);
          const float x = zs[m * 68 + c];
          a0 += t.x * x;
          a1 += t.y * x;
        }
        p.dA[(int64_t)j * p.K + k0 + c] = (uint16_t)(pack_bf16x2(p.s * a0, 0.0f) & 0xFFFFu);
        p.dA[(int64_t)(j + 1) * p.K + k0 + c] = (uint16_t)(pack_bf16x2(p.s * a1, 0.0f) & 0xFFFFu);
      }
    } else {
      for (int j = tid >> 5; j < r; j += 8) {
        float acc = 0.0f;
        for (int m = 0; m < M; ++m) acc += vs[m * r + j] * zs[m * 68 + c];
        p.dA[(int64_t)j * p.K + k0 + c] = (uint16_t)(pack_bf16x2(p.s * acc, 0.0f) & 0xFFFFu);
      }
    }
  } else {
    const int64_t n0 = (int64_t)(blockIdx.x - nkb) * 64;
    for (int e = tid; e < M * r; e += 256) vs[e] = p.XA[e];
    stage_block(p.dY + n0, p.N, 64);
    __syncthreads();
    if ((r & 3) == 0) {
      // a thread takes 4 consecutive ranks of one row of dB (one 16-byte
      // read of XA per token), consecutive threads the next 4
      for (int e = 4 * tid; e < 64 * r; e += 1024) {
        const int nl = e / r, j = e - nl * r;
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int m = 0; m < M; ++m) acc += zs[m * 68 + nl] * *reinterpret_cast<const f32x4*>(vs + m * r + j);
        *reinterpret_cast<u32x2*>(p.dB + (n0 + nl) * r + j) =
            u32x2{pack_bf16x2(p.s * acc[0], p.s * acc[1]), pack_bf16x2(p.s * acc[2], p.s * acc[3])};
      }
    } else {
      // consecutive threads write consecutive ranks of one row of dB
      for (int e = tid; e < 64 * r; e += 256) {
        const int nl = e / r, j = e - nl * r;
        float acc = 0.0f;
        for (int m = 0; m < M; ++m) acc += zs[m * 68 + nl] * vs[m * r + j];
        p.dB[(n0 + nl) * r + j] = (uint16_t)(pack_bf16x2(p.s * acc, 0.0f) & 0xFFFFu);
      }
    }
  }
}

// ------------------------------------------------------------------------
// Skinny-M transposed product: the dequantized-weight part of dX = dY W0
// ("LLM Fine-Tuning in 2026: Unsloth vs QLoRA vs Liger-Kernel", section 2)
// for M <= 64 tokens, as split partials part[z] = dY[:, n-range z]
// deq(W0)[n-range z, :] (the finish kernel adds them and the LoRA term).
//
// Workgroup: 256 output columns k x the 64-row reduction tiles of one split,
// 8 waves (two per SIMD, so one wave's LDS waits overlap the other's work).
// Waves w and w + 4 own columns 64 (w % 4) .. + 63 and take reduction rows
// 0..31 and 32..63 of every tile; their sums are added at the end.  Per tile,
// the code rows (64 x 128 bytes), the dY tile (64 tokens x 64 reduction rows)
// and the absmax of the tile's rows arrive by direct global->LDS loads (whole
// 128-byte lines for codes and dY) in a 4-stage ring with one barrier per
// tile; every load of the kernel is a direct load, so each wait is the
// explicit vmcnt below.  Lane (l16, q) owns columns 4 l16 .. 4 l16 + 3 of its
// wave's 64 (frag f holds column 4 l16 + f): it reads 2 bytes of codes per
// reduction row and expands them straight into the B operands of
// v_mfma_f32_16x16x32_bf16 (reduction rows 32 h + 8 q + e, e < 8), so the
// expanded weight never goes through LDS.  Code rows are stored with 16-byte
// chunk c of row r at position c ^ ((r >> 3) & 7), dY rows with chunk c at
// c ^ (r & 7): the lanes of one LDS read then hit different banks.
// ------------------------------------------------------------------------
constexpr int SB_D = 4;  // stages of the load ring

struct __attribute__((aligned(16))) SkBwdStage {
  uint8_t codes[64 * 128];  // 64 reduction rows x 256 columns
  uint16_t dy[64 * 64];     // 64 tokens x 64 reduction rows
  // per row of the tile, one region per wave: DQ: waves 0..3 the row's 4
  // absmax codes (one dword), waves 4..7 the fp32 scale of those blocks;
  // else the fp32 absmax of the wave's block (waves 4..7: a copy)
  uint32_t aux[8 * 64];
};

// The codebook; the most strictly aligned LDS object, so that it sits at LDS
// address 0 (the lookups use the SDWA result as the address).
struct __attribute__((aligned(256))) SkBwdHead {
  float cb[16];
};

template <bool DQ>
__global__ __launch_bounds__(512) void skinny_bwd_kernel(SkinnyBwdArgs p) {
  __shared__ SkBwdHead hd;
  __shared__ SkBwdStage st0, st1, st2, st3;
  __shared__ f32x4 red[4 * 16 * 64];  // second-half sums of waves 4..7
  constexpr int TF = SK_TF;
  // direct loads per wave per tile: codes, dY and one absmax part, the same
  // three in every wave and without branches (a direct load under a branch
  // makes the compiler wait for all loads before every LDS read)
  constexpr int PT = 3;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cw = wave & 3, hh = wave >> 2;
  const int l16 = lane & 15, q = lane >> 4;
  const int64_t c0 = (int64_t)blockIdx.x * 256;
  const int64_t KB = p.K / 64;
  const int64_t kb0 = c0 / 64;
  const int NTL = (int)(p.N / 64);
  const int tb = blockIdx.y * p.kps, te = min(NTL, tb + p.kps);
  const int nt = te - tb;
  if (tid < 16) hd.cb[tid] = p.codebook[tid];

  // direct-load lane addresses for tile 0 (the tile offset is added per load):
  // wave w brings code rows and dY tokens 8 w .. 8 w + 7
  const int lrow = 8 * wave + (lane >> 3);
  const uint8_t* cg = p.w.codes + (int64_t)lrow * (p.K / 2) + c0 / 2 + 16 * ((lane & 7) ^ wave);
  // token rows past M read row M - 1 (never stored)
  const uint16_t* yg = p.dY + (int64_t)min(lrow, (int)p.M - 1) * p.N + 8 * ((lane & 7) ^ (lrow & 7));
  auto dma = [&](int t, SkBwdStage& S) {
    const int64_t n0 = (int64_t)t * 64;
    __builtin_amdgcn_global_load_lds(cg + n0 * (p.K / 2), LDS_PTR(S.codes + 8 * wave * 128), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(yg + n0, LDS_PTR(S.dy + 8 * wave * 64), 16, 0, 0);
    const int64_t blk = (n0 + lane) * KB + kb0;  // row lane's first block of the 256 columns
    const void* src;
    if constexpr (DQ)
      src = hh == 0 ? (const void*)(p.w.absmax_q + blk) : (const void*)(p.w.absmax_scale + ((blk + cw) >> 8));
    else
      src = p.w.absmax + blk + cw;
    __builtin_amdgcn_global_load_lds(src, LDS_PTR(S.aux + 64 * wave), 4, 0, 0);
  };

  f32x4 acc[4][TF];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int i = 0; i < TF; ++i) acc[f][i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  const int r0 = 32 * hh + 8 * q;         // the lane's 8 reduction rows within a tile
  const int cbyte = 32 * cw + 2 * l16;    // the lane's 2 code bytes within a row
  const int pc = ((cbyte >> 4) ^ ((4 * hh + q) & 7)) * 16 + (cbyte & 15);
  // the operands of one tile: built from its stage in one step, multiplied
  // in the next (interleaved with the next tile's LDS and VALU work)
  u32x4 wp[4], xp[TF];
#pragma unroll
  for (int f = 0; f < 4; ++f) wp[f] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < TF; ++i) xp[i] = u32x4{0u, 0u, 0u, 0u};
  auto mma = [&]() {
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int i = 0; i < TF; ++i) acc[f][i] = mfma16(xp[i], wp[f], acc[f][i]);
  };
  auto prepare = [&](const SkBwdStage& S, u32x4 (&w)[4], u32x4 (&x)[TF]) {
    // absmax of this wave's block for the tile's rows: lane r computes row r,
    // the lanes that need it read it with a cross-lane move
    float arow;
    if constexpr (DQ)
      arow = (float)((S.aux[64 * cw + lane] >> (8 * cw)) & 0xFFu) * __uint_as_float(S.aux[256 + 64 * cw + lane]);
    else
      arow = __uint_as_float(S.aux[64 * cw + lane]);
    float v[8][4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const uint32_t lo16 = *reinterpret_cast<const uint16_t*>(S.codes + (r0 + 2 * h) * 128 + pc);
      const uint32_t hi16 = *reinterpret_cast<const uint16_t*>(S.codes + (r0 + 2 * h + 1) * 128 + pc);
      const uint32_t d = lo16 | (hi16 << 16);
      float t8[8];
      sk_lookup8(hd.cb, d, t8);  // rows 2h (cols 0..3), 2h + 1 (cols 0..3)
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        v[2 * h][f] = t8[f];
        v[2 * h + 1][f] = t8[4 + f];
      }
    }
    float a[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] = __shfl(arow, r0 + e);
#pragma unroll
    for (int f = 0; f < 4; ++f)
      w[f] = u32x4{pack_bf16x2(v[0][f] * a[0], v[1][f] * a[1]), pack_bf16x2(v[2][f] * a[2], v[3][f] * a[3]),
                   pack_bf16x2(v[4][f] * a[4], v[5][f] * a[5]), pack_bf16x2(v[6][f] * a[6], v[7][f] * a[7])};
#pragma unroll
    for (int i = 0; i < TF; ++i) {
      const int tok = 16 * i + l16;
      x[i] = *reinterpret_cast<const u32x4*>(S.dy + tok * 64 + (((4 * hh + q) ^ (tok & 7)) * 8));
    }
  };

  // ring: tile t in stage t % 4; D - 1 tiles requested ahead (clamped to the
  // last tile, so every wave issues the same number of loads)
  if (nt > 0) {
    dma(tb + 0, st0);
    dma(tb + min(1, nt - 1), st1);
    dma(tb + min(2, nt - 1), st2);
  }
  auto step = [&](int t, SkBwdStage& cur, SkBwdStage& fill) {
    wait_vmcnt<(SB_D - 2) * PT>();  // tile t landed (this wave's part)
    stage_barrier();  // every wave's part landed; every wave done reading tile t - 1
    dma(tb + min(t + SB_D - 1, nt - 1), fill);
    u32x4 wn[4], xn[TF];
    prepare(cur, wn, xn);
    mma();  // tile t - 1 (zero operands before the first tile)
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      SCHED_GROUP(SG_DS_READ, 3);
      SCHED_GROUP(SG_VALU, 6);
      SCHED_GROUP(SG_MFMA, 1);
    }
#pragma unroll
    for (int f = 0; f < 4; ++f) wp[f] = wn[f];
#pragma unroll
    for (int i = 0; i < TF; ++i) xp[i] = xn[i];
  };
  int t = 0;
  for (; t + 4 <= nt; t += 4) {
    step(t, st0, st3);
    step(t + 1, st1, st0);
    step(t + 2, st2, st1);
    step(t + 3, st3, st2);
  }
  if (t < nt) step(t, st0, st3);
  if (t + 1 < nt) step(t + 1, st1, st0);
  if (t + 2 < nt) step(t + 2, st2, st1);
  wait_vmcnt<0>();  // no direct load may still target LDS at the end
  mma();            // the last tile

  // waves 4..7 hand their sums to waves 0..3 (lane-contiguous 16-byte slots)
  f32x4* rw = red + cw * 16 * 64 + lane;
  if (hh == 1) {
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int i = 0; i < TF; ++i) rw[(4 * f + i) * 64] = acc[f][i];
  }
  __syncthreads();
  if (hh == 1) return;
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int i = 0; i < TF; ++i) acc[f][i] += rw[(4 * f + i) * 64];

  // split partial: value v of acc[f][i] is token 16 i + 4 q + v, column
  // c0 + 64 cw + 4 l16 + f: 4 adjacent columns per (i, v), one 16-byte store
  float* dst = p.part + (int64_t)blockIdx.y * p.M * p.K + c0 + 64 * cw + 4 * l16;
#pragma unroll
  for (int i = 0; i < TF; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t m = 16 * i + 4 * q + v;
      if (m < p.M)
        *reinterpret_cast<f32x4*>(dst + m * p.K) = f32x4{acc[0][i][v], acc[1][i][v], acc[2][i][v], acc[3][i][v]};
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

bool skinny_finish_supported(int64_t M, int r) { return M >= 1 && M <= 64 && r >= 1 && r <= 128; }

hipError_t launch_skinny_bwd_finish(const SkinnyFinishArgs& a, hipStream_t st) {
  if (!skinny_finish_supported(a.M, a.r) || a.K % 64 != 0 || a.N % 64 != 0) return hipErrorInvalidValue;
  const unsigned grid = (unsigned)(a.K / 32 + a.N / 64);
  if (grid == 0) return hipSuccess;
  const size_t lds = (size_t)(64 * a.r + 64 * 68 + 32 * a.r) * sizeof(float);
  skinny_bwd_finish_kernel<<<grid, 256, lds, st>>>(a);
  return hipGetLastError();
}

bool skinny_bwd_supported(int64_t M, int64_t N, int64_t K) {
  return M >= 1 && M <= 64 && K % 256 == 0 && N % 64 == 0 && N > 0;
}

hipError_t launch_skinny_bwd(const SkinnyBwdArgs& a, int splits, hipStream_t st) {
  if (!skinny_bwd_supported(a.M, a.N, a.K) || splits < 1) return hipErrorInvalidValue;
  dim3 grid((unsigned)(a.K / 256), (unsigned)splits);
  if (a.w.dq)
    skinny_bwd_kernel<true><<<grid, 512, 0, st>>>(a);
  else
    skinny_bwd_kernel<false><<<grid, 512, 0, st>>>(a);
  return hipGetLastError();
}
