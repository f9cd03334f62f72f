// Skinny-M QLoRA forward for gfx950, streaming form: the forward
// Y = X deq(W0)^T + s (X A^T) B^T of "LLM Fine-Tuning in 2026: Unsloth vs
// QLoRA vs Liger-Kernel" (section 1) for M <= 64 tokens, where every weight
// element feeds at most 64 multiply-adds and the NF4 weight stream from HBM
// is the bound ("What is Unsloth?": memory bandwidth, not compute, limits).
//
// What bounds such a kernel on this chip, and the answer to each:
//   * global loads in MFMA operand layout put 16 different rows on 16
//     consecutive lanes and run at a third of the rate of whole-line loads.
//     The activations are therefore re-laid out once per call into
//     Xt[K/8][Mp][8] (Mp = tokens rounded up to 16, zero rows past M): the
//     8-element chunk that MFMA lane (token m, group q) needs sits next to the
//     chunks of tokens m +- 1, so one load instruction reads 4 runs of 256
//     contiguous bytes.  The NF4 codes (and block absmax) come by direct
//     global->LDS loads of whole 128-byte row segments;
//   * the expansion (codebook lookup, times the block absmax, rounded to
//     bf16) stays in registers and feeds the MFMA B operand directly, so the
//     accumulators never pass through vector ALU instructions and stay in the
//     accumulator registers.  The 16-entry fp32 codebook sits at LDS address 0
//     (one SDWA instruction yields the lookup address; a half-wave reads at
//     most 16 distinct dwords, without bank conflicts);
//   * the compiler orders LDS reads after direct loads that may alias them:
//     the two ring slots are separate LDS objects, so that reading one slot
//     never waits for the loads into the other.
//
// Workgroup: 16 FN weight rows x a range of 64-wide reduction tiles, 4 waves
// (one per SIMD).  Each wave takes a contiguous run of 4-tile groups (256
// reduction columns = one 128-byte line of codes per row) and streams all rows
// of the workgroup over it; there is no barrier in the main loop.  Per wave,
// group g's codes and absmax land in LDS ring g % 2 (the loads of group g + 2
// are issued when group g is done), and the activation operands of tile t are
// loaded into register set t % 4, three tiles ahead.  Loads complete in issue
// order, so one explicit vmcnt wait per tile (for tile t's activations) also
// covers its group's direct loads.
//
// Reduction order: MFMA step s (0, 1) of tile t, lane group q (lanes 16q ..
// 16q + 15) holds reduction columns 64t + 16q + 8s + e, e < 8, for both
// operands.  The wave partials are
// summed in LDS in wave order, the LoRA term is added as MFMA steps, and the
// tile is stored as bf16 (or as fp32 split partials).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qlora_device.h"
#include "qlora_gemm_common.h"
#include "qlora_launch.h"

namespace qk {

__device__ __forceinline__ f32x4 mfma16b(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

constexpr int S2_WAVES = 4;

// Byte offset of a codebook entry: 4 * (bits [8B + 2, 8B + 6) of x), i.e.
// with x = c << 2 the low nibble of byte B of c, with x = c >> 2 its high
// nibble, selected and masked by one SDWA instruction (the codebook sits at
// LDS address 0, so this is the lookup's address).
#define S2_NIB(B)                                                                                             \
  __device__ __forceinline__ uint32_t s2_nib##B(uint32_t x) {                                                 \
    uint32_t r;                                                                                               \
    asm("v_and_b32_sdwa %0, 60, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_" #B \
        : "=v"(r)                                                                                             \
        : "v"(x));                                                                                            \
    return r;                                                                                                 \
  }
S2_NIB(0)
S2_NIB(1)
S2_NIB(2)
S2_NIB(3)
#undef S2_NIB

// 8 codes of one dword -> 4 packed bf16 pairs of fp32(codebook[q] * a), in
// element order (cb: the codebook at LDS address 0)
__device__ __forceinline__ u32x4 s2_expand8(const float* cb, uint32_t c, float a) {
  const uint32_t lo = c << 2, hi = c >> 2;
  const char* t = reinterpret_cast<const char*>(cb);
  auto v = [&](uint32_t off) { return *reinterpret_cast<const float*>(t + off) * a; };
  return u32x4{pack_bf16x2(v(s2_nib0(lo)), v(s2_nib0(hi))), pack_bf16x2(v(s2_nib1(lo)), v(s2_nib1(hi))),
               pack_bf16x2(v(s2_nib2(lo)), v(s2_nib2(hi))), pack_bf16x2(v(s2_nib3(lo)), v(s2_nib3(hi)))};
}

// The codebook, the most strictly aligned LDS object of the kernel, so that
// it sits at LDS address 0.
struct __attribute__((aligned(1024))) Sk2Head {
  float cb[16];
};

// Activation re-layout for the skinny GEMMs: Xt[j][m][0..7] = X[m][8j..8j+7]
// for m < M, zero for M <= m < Mp.  One thread per 16-byte chunk; the
// threads of a wave take consecutive tokens of one chunk column, so the
// stores are contiguous.
__global__ __launch_bounds__(256) void xtile_kernel(const uint16_t* __restrict__ X, int64_t M, int64_t K, int Mp,
                                                    uint16_t* __restrict__ Xt) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t nchunk = K / 8;
  if (i >= nchunk * Mp) return;
  const int64_t j = i / Mp, m = i - j * Mp;
  u32x4 v = {0u, 0u, 0u, 0u};
  if (m < M) v = *reinterpret_cast<const u32x4*>(X + m * K + 8 * j);
  *reinterpret_cast<u32x4*>(Xt + i * 8) = v;
}

template <int FN, int TF, bool DQ>
struct Sk2Cfg {
  static_assert(FN <= 7 && TF <= 4, "offset arrays are sized for 7 frags and 4 token frags");
  static constexpr int R = 16 * FN;
  static constexpr int CODE_BYTES = R * 128;  // one group of codes
  static constexpr int NAX = (R + 63) / 64;   // absmax direct loads (per part), 64 rows each
  // absmax of a group: fp32 - 16 bytes per row; DQ - 4 code bytes per row,
  // then the row's fp32 scale (each direct load writes 64 lanes)
  static constexpr int AUX_BYTES = DQ ? 2 * 256 * NAX : 1024 * NAX;
  // fp32 absmax [row][4] of the group: the direct-loaded aux itself (fp32
  // mode), or written there from the codes and scales (DQ)
  static constexpr int AMF = DQ ? CODE_BYTES + AUX_BYTES : CODE_BYTES;
  static constexpr int SLOT = CODE_BYTES + AUX_BYTES + (DQ ? 16 * R : 0);
  static constexpr int ND = R / 8 + (DQ ? 2 : 1) * NAX;  // direct loads per group
  // after the main loop ring 0 holds 4 rounds of per-wave partial tiles,
  // ring 1 the LoRA operand V [64][64] fp32
  static constexpr int RED = 4 * S2_WAVES * TF * 256 * 4;
  static constexpr int RING0 = (S2_WAVES * SLOT > RED) ? S2_WAVES * SLOT : RED;
  static constexpr int RING1 = (S2_WAVES * SLOT > 64 * 64 * 4) ? S2_WAVES * SLOT : 64 * 64 * 4;
};

template <int FN, int TF, bool DQ>
__global__ __launch_bounds__(256) void skinny_fwd2_kernel(SkinnyArgs p) {
  using C = Sk2Cfg<FN, TF, DQ>;
  constexpr int R = C::R;
  constexpr int NX = 2 * TF;  // activation loads per tile
  __shared__ Sk2Head hd;
  __shared__ __attribute__((aligned(16))) uint8_t ring0[C::RING0];
  __shared__ __attribute__((aligned(16))) uint8_t ring1[C::RING1];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, q = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * R;
  const int KT = (int)(p.K / 64);
  const int kb = blockIdx.y * p.kps, ke = min(KT, kb + p.kps);
  const int ngr = (ke - kb) >> 2;  // 4-tile groups of this split
  const int gpw = (ngr + S2_WAVES - 1) / S2_WAVES;
  const int gb = min(ngr, wave * gpw), ge = min(ngr, gb + gpw);
  const int G = ge - gb;  // this wave's groups
  const int T = 4 * G;
  const int tile0 = kb + 4 * gb;  // first tile of the wave
  const bool lora_here = blockIdx.y == 0 && p.r > 0;
  const int rows = (int)min((int64_t)R, p.N - n0);

  if (tid < 16) hd.cb[tid] = p.codebook[tid];

  // ---- direct loads of one group into a ring slot: the codes of the R rows
  // (whole 128-byte segments; instruction i covers rows 8i .. 8i+7, lane l
  // loads 16-byte chunk (l % 8) ^ (l / 8) of row 8i + l/8, so chunk c of row r
  // lands at position c ^ (r % 8); rows past the weight read as zeros through
  // the buffer range), then the absmax of the rows' 4 blocks.
  const __amdgpu_buffer_rsrc_t crs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(p.w.codes + n0 * (p.K / 2)), (short)0, (int)(rows * (p.K / 2)), 0x00020000);
  const uint32_t cofs = (uint32_t)((lane >> 3) * (p.K / 2) + 16 * ((lane & 7) ^ (lane >> 3)));
  const int64_t nblk = p.N * (int64_t)KT;
  // DQ: the code bytes and the scales; else the fp32 absmax (twice)
  const __amdgpu_buffer_rsrc_t ars = __builtin_amdgcn_make_buffer_rsrc(
      DQ ? const_cast<void*>(static_cast<const void*>(p.w.absmax_q))
         : const_cast<void*>(static_cast<const void*>(p.w.absmax)),
      (short)0, (int)min(DQ ? nblk : nblk * 4, (int64_t)0x7FFFFFFF), 0x00020000);
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      DQ ? const_cast<void*>(static_cast<const void*>(p.w.absmax_scale))
         : const_cast<void*>(static_cast<const void*>(p.w.absmax)),
      (short)0, (int)min(DQ ? ((nblk + 255) >> 8) * 4 : nblk * 4, (int64_t)0x7FFFFFFF), 0x00020000);
  // (offset arrays passed to the load builtins have fixed sizes: with a
  // template-dependent size the host pass drops the kernel's launch stub)
  uint32_t aofs[2];
  int64_t ablk[2];
#pragma unroll
  for (int i = 0; i < C::NAX; ++i) {
    const int row = min(64 * i + lane, rows - 1);
    ablk[i] = (n0 + row) * (int64_t)KT;  // first block of the row
    aofs[i] = (uint32_t)(DQ ? ablk[i] : ablk[i] * 4);
  }
  auto dma_group = [&](uint8_t* slot, int g) __attribute__((always_inline)) {
    const int tg = tile0 + 4 * min(g, G - 1);  // past the end: reload the last group (in-bounds)
#pragma unroll
    for (int i = 0; i < R / 8; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(crs, LDS_PTR(slot + 1024 * i), 16, cofs,
                                               tg * 32 + i * 4 * (int)p.K, 0, 0);
    uint8_t* aux = slot + C::CODE_BYTES;
#pragma unroll
    for (int i = 0; i < C::NAX; ++i) {
      if constexpr (DQ) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ars, LDS_PTR(aux + 256 * i), 4, aofs[i], tg, 0, 0);
        const uint32_t so = (uint32_t)(((ablk[i] + tg) >> 8) * 4);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(srs, LDS_PTR(aux + 256 * C::NAX + 256 * i), 4, so, 0, 0, 0);
      } else {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ars, LDS_PTR(aux + 1024 * i), 16, aofs[i], tg * 4, 0, 0);
      }
    }
  };

  // ---- activation operands of tile t (register set t % 4): token frag i,
  // step s, lane (m, q) holds Xt[8t + 2q + s][16i + m][0..7]
  const int Mp = p.Mp;
  const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(p.Xt), (short)0, (int)min(p.K * (int64_t)Mp * 2, (int64_t)0x7FFFFFFF), 0x00020000);
  const uint32_t xofs = (uint32_t)(((2 * q) * Mp + l16) * 16);
  u32x4 xr[4][TF][2];
  auto load_x = [&](int t, u32x4 (&x)[TF][2]) __attribute__((always_inline)) {
    t = tile0 + min(t, T - 1);  // past the end: reload the last tile
#pragma unroll
    for (int i = 0; i < TF; ++i)
#pragma unroll
      for (int s = 0; s < 2; ++s)
        x[i][s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                xrs, xofs, t * 8 * Mp * 16 + (s * Mp + 16 * i) * 16, 0));
  };

  f32x4 acc[FN][TF];
#pragma unroll
  for (int f = 0; f < FN; ++f)
#pragma unroll
    for (int i = 0; i < TF; ++i) acc[f][i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // LDS byte offset of this lane's 8 code bytes (row l16 of frag 0, tile j of
  // the group); frag f adds 2048 f
  uint32_t crd[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) crd[j] = (uint32_t)(l16 * 128 + 16 * ((2 * j + (q >> 1)) ^ (l16 & 7)) + 8 * (q & 1));
  // DQ: absmax = code8 * scale of the group's rows into fp32 [row][4] (each
  // wave converts its own slot; lane l takes rows l and l + 64)
  auto group_absmax = [&](uint8_t* slot) __attribute__((always_inline)) {
    if constexpr (DQ) {
      const uint8_t* aux = slot + C::CODE_BYTES;
#pragma unroll
      for (int i = 0; i < C::NAX; ++i) {
        const int row = 64 * i + lane;
        if (row < R) {
          const uint32_t c4 = *reinterpret_cast<const uint32_t*>(aux + 4 * row);
          const float sc = *reinterpret_cast<const float*>(aux + 256 * C::NAX + 4 * row);
          *reinterpret_cast<f32x4*>(slot + C::AMF + 16 * row) =
              f32x4{(float)(c4 & 0xFFu) * sc, (float)((c4 >> 8) & 0xFFu) * sc, (float)((c4 >> 16) & 0xFFu) * sc,
                    (float)(c4 >> 24) * sc};
        }
      }
    }
  };
  // expansion and products of tile j of a group, software-pipelined over the
  // frags: round f issues the codebook lookups of frag f + 1, scales and packs
  // the bf16 operands of frag f and runs the MFMAs of frag f - 1, interleaved
  // (one MFMA, two lookups, a few vector instructions) so that the single wave
  // of the SIMD keeps the matrix core busy while its lookups are in flight
  auto compute_tile = [&](int j, const uint8_t* slot, const u32x4 (&x)[TF][2]) __attribute__((always_inline)) {
    u32x2 cw[FN];
    float av[FN];
#pragma unroll
    for (int f = 0; f < FN; ++f) {
      cw[f] = *reinterpret_cast<const u32x2*>(slot + crd[j] + 2048 * f);
      av[f] = *reinterpret_cast<const float*>(slot + C::AMF + 16 * (16 * f + l16) + 4 * j);
    }
    const char* t = reinterpret_cast<const char*>(hd.cb);
    float cv[2][16];
    u32x4 w[2][2];
    auto lookups = [&](int f, float (&v)[16]) __attribute__((always_inline)) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t lo = cw[f][h] << 2, hi = cw[f][h] >> 2;
        const uint32_t o[8] = {s2_nib0(lo), s2_nib0(hi), s2_nib1(lo), s2_nib1(hi),
                               s2_nib2(lo), s2_nib2(hi), s2_nib3(lo), s2_nib3(hi)};
#pragma unroll
        for (int e = 0; e < 8; ++e) v[8 * h + e] = *reinterpret_cast<const float*>(t + o[e]);
      }
    };
    auto operands = [&](int f, const float (&v)[16], u32x4 (&ww)[2]) __attribute__((always_inline)) {
      const float a = av[f];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int d = 0; d < 4; ++d) ww[h][d] = pack_bf16x2(v[8 * h + 2 * d] * a, v[8 * h + 2 * d + 1] * a);
    };
    auto products = [&](int f, const u32x4 (&ww)[2]) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < TF; ++i) acc[f][i] = mfma16b(x[i][0], ww[0], acc[f][i]);
#pragma unroll
      for (int i = 0; i < TF; ++i) acc[f][i] = mfma16b(x[i][1], ww[1], acc[f][i]);
    };
    lookups(0, cv[0]);
    if (FN > 1) lookups(1, cv[1]);
    operands(0, cv[0], w[0]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int f = 1; f <= FN; ++f) {
      if (f + 1 < FN) lookups(f + 1, cv[(f + 1) & 1]);
      if (f < FN) operands(f, cv[f & 1], w[f & 1]);
      products(f - 1, w[(f - 1) & 1]);
#pragma unroll
      for (int k = 0; k < 2 * TF; ++k) {
        SCHED_GROUP(SG_MFMA, 1);
        SCHED_GROUP(SG_DS_READ, 2);
        SCHED_GROUP(SG_VALU, 5);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // one group out of ring slot `slot`; then the loads of group g + 2 into it
  // (the empty asm statements keep the compiler from moving loads across the
  // explicit waits and LDS reads of direct-loaded data above them)
  auto group = [&](int g, uint8_t* slot) __attribute__((always_inline)) {
    load_x(4 * g + 3, xr[3]);
    asm volatile("" ::: "memory");
    wait_vmcnt<3 * NX + C::ND>();
    asm volatile("" ::: "memory");
    group_absmax(slot);
    compute_tile(0, slot, xr[0]);
    load_x(4 * g + 4, xr[0]);
    asm volatile("" ::: "memory");
    wait_vmcnt<3 * NX + C::ND>();
    asm volatile("" ::: "memory");
    compute_tile(1, slot, xr[1]);
    load_x(4 * g + 5, xr[1]);
    asm volatile("" ::: "memory");
    wait_vmcnt<3 * NX + C::ND>();
    asm volatile("" ::: "memory");
    compute_tile(2, slot, xr[2]);
    load_x(4 * g + 6, xr[2]);
    asm volatile("" ::: "memory");
    wait_vmcnt<3 * NX>();
    asm volatile("" ::: "memory");
    compute_tile(3, slot, xr[3]);
    // the slot is free once this wave's LDS reads of it are done
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    dma_group(slot, g + 2);
  };

  uint8_t* slot0 = ring0 + wave * C::SLOT;
  uint8_t* slot1 = ring1 + wave * C::SLOT;
  __syncthreads();  // the codebook is in place

  if (T > 0) {
    // prologue in the steady-state issue order: group 0, the activations of
    // tiles 0..2, group 1
    dma_group(slot0, 0);
    load_x(0, xr[0]);
    load_x(1, xr[1]);
    load_x(2, xr[2]);
    dma_group(slot1, 1);
    int g = 0;
    for (; g + 2 <= G; g += 2) {
      group(g, slot0);
      group(g + 1, slot1);
    }
    if (g < G) group(g, slot0);
    wait_vmcnt<0>();  // no direct load may still target LDS
  }

  __syncthreads();  // every wave is done with its slots

  // ---- V = sum_z vpart[z] into LDS (split order); the first workgroup
  // also writes it out (the forward keeps X A^T)
  float* vs = reinterpret_cast<float*>(ring1);  // [M][r], r <= 64
  if (lora_here) {
    // split z's partials are added in order z = 0, 1, ... for every entry;
    // the loads of 8 splits x 4 entries are issued together (one load and
    // its wait per split would put 4 x vsplits L2 round trips in a row)
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

  // ---- LoRA term (wave 0): acc += (s V) Wl^T in steps of 32 ranks, s V
  // rounded to bf16 like the other operands
  if (lora_here && wave == 0) {
    for (int j0 = 0; j0 < p.r; j0 += 32) {
      const int jq = j0 + 8 * q;
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
        for (int i = 0; i < TF; ++i) acc[f][i] = mfma16b(va[i], wb4, acc[f][i]);
      }
    }
  }

  // ---- sum the wave partials in wave order and store, up to 4 frags per
  // round: value e = 256 i + 64 v + lane of a frag is token 16 i + 4 (lane/16)
  // + v, weight row n0 + 16 f + lane % 16.  A thread sums 4 consecutive values
  // (4 consecutive rows of one token) and stores them together.
  float* red = reinterpret_cast<float*>(ring0);
  constexpr int FR = 4;
#pragma unroll
  for (int f0 = 0; f0 < FN; f0 += FR) {
    __syncthreads();
#pragma unroll
    for (int fl = 0; fl < FR; ++fl) {
      if (f0 + fl < FN) {
#pragma unroll
        for (int i = 0; i < TF; ++i)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            red[(fl * S2_WAVES + wave) * (TF * 256) + 256 * i + 64 * v + lane] = acc[f0 + fl][i][v];
      }
    }
    __syncthreads();
#pragma unroll
    for (int fl = 0; fl < FR; ++fl) {
      if (f0 + fl >= FN) continue;
      for (int e = 4 * tid; e < TF * 256; e += 1024) {
        f32x4 sum = *reinterpret_cast<const f32x4*>(red + (fl * S2_WAVES) * (TF * 256) + e);
#pragma unroll
        for (int w = 1; w < S2_WAVES; ++w)
          sum += *reinterpret_cast<const f32x4*>(red + (fl * S2_WAVES + w) * (TF * 256) + e);
        const int ln = e & 63;
        const int64_t m = 16 * (e >> 8) + 4 * (ln >> 4) + ((e >> 6) & 3);
        const int64_t n = n0 + 16 * (f0 + fl) + (ln & 15);
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
}

template <int FN, int TF>
static hipError_t run_fwd2(const SkinnyArgs& a, const qplan::SkinnyPlan& pl, hipStream_t st) {
  const dim3 grid((unsigned)qplan::cdiv(a.N, 16 * FN), (unsigned)pl.splits);
  if (a.w.dq)
    skinny_fwd2_kernel<FN, TF, true><<<grid, 256, 0, st>>>(a);
  else
    skinny_fwd2_kernel<FN, TF, false><<<grid, 256, 0, st>>>(a);
  return hipGetLastError();
}

template <int FN>
static hipError_t run_fwd2_tf(const SkinnyArgs& a, const qplan::SkinnyPlan& pl, hipStream_t st) {
  switch ((a.Mp + 15) / 16) {
    case 1: return run_fwd2<FN, 1>(a, pl, st);
    case 2: return run_fwd2<FN, 2>(a, pl, st);
    case 3: return run_fwd2<FN, 3>(a, pl, st);
    case 4: return run_fwd2<FN, 4>(a, pl, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qk

using namespace qk;

// M <= 64 tokens, whole 4-tile groups, and every buffer offset within 31 bits
// (fp32 absmax bytes N K / 16, activation bytes K Mp 2).
bool skinny_fwd2_supported(int64_t M, int64_t N, int64_t K, int r) {
  return M >= 1 && M <= 64 && r <= 64 && K % 256 == 0 && N * (K / 16) < ((int64_t)1 << 31) &&
         K * 64 * 2 < ((int64_t)1 << 31);
}

hipError_t launch_xtile(const uint16_t* X, int64_t M, int64_t K, int Mp, uint16_t* Xt, hipStream_t st) {
  const int64_t n = (K / 8) * Mp;
  if (n == 0) return hipSuccess;
  xtile_kernel<<<dim3((unsigned)((n + 255) / 256)), 256, 0, st>>>(X, M, K, Mp, Xt);
  return hipGetLastError();
}

hipError_t launch_skinny_fwd2(const SkinnyArgs& a, const qplan::SkinnyPlan& pl, hipStream_t st) {
  if (a.M == 0) return hipSuccess;
  switch (pl.fn) {
    case 1: return run_fwd2_tf<1>(a, pl, st);
    case 2: return run_fwd2_tf<2>(a, pl, st);
    case 4: return run_fwd2_tf<4>(a, pl, st);
    case 7: return run_fwd2_tf<7>(a, pl, st);
    default: return hipErrorInvalidValue;
  }
}
