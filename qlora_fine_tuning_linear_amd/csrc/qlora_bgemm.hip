// Large-token path of the QLoRA GEMMs on gfx950: the NF4 weight is expanded
// once per call into a bf16 workspace (coalesced, HBM-bound kernels below),
// then a bf16 x bf16 MFMA GEMM with both operands staged through LDS runs
// over it and finishes with the same fused epilogue as the dequant-staged
// kernel (LoRA term as extra MFMA steps, SwiGLU forward / backward).
//
// Why not expand inside the GEMM here: with T tokens and 256-token tiles an
// in-GEMM expansion redoes every weight element T/256 times (32 times at
// 8192 tokens), and its lookups and bf16 tile writes compete with the MFMA
// operand reads for LDS bandwidth.  One expansion pass costs 0.5 B read +
// 2 B written per weight element; the GEMM then re-reads 2 B per element
// per token tile from L2 instead of 0.5 B.  For few tokens (one token tile)
// the in-GEMM expansion of qgemm_kernel is used instead.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "qlora_device.h"
#include "qlora_gemm_common.h"
#include "qlora_launch.h"

namespace qk {

// ------------------------------------------------------------------------
// bgemm_kernel: output tile 256 tokens x 256 weight rows, 8 waves (two per
// SIMD) in a 2 x 4 grid, each 128 tokens x 64 weight rows = 4 x 2 frags of
// 32x32, fp32 accumulators.  Reduction tiles of 64 columns.  Two waves per
// SIMD let one wave's matrix instructions run while the other waits for its
// operands or at the barrier (measured against one 128 x 128 wave per SIMD:
// 3-9% less time per GEMM; the chip runs at a lower clock under the denser
// matrix work, so the gain in cycles is larger than the gain in time).
//
// Operands move global -> LDS by direct loads (buffer loads with the lds
// flag, 16 bytes per lane, no registers, no LDS write instructions; a fixed
// 32-bit lane offset, the tile's column offset in the scalar offset).  Each
// direct load fills 1 KB of LDS with 8 rows x 128 bytes, i.e. whole cache
// lines; a tile operand ([256][64] bf16, chunk c of row r stored at
// c ^ swz(r)) is 32 KB, 4 direct loads per wave.  The two operands of tile kt
// ("halves" 2kt and 2kt+1: the first half is the weight when the weight is
// the larger matrix, else the activations) rotate through five 32 KB buffers
// (all 160 KB of LDS; each buffer its own __shared__ object, so the
// compiler's dependency tracking adds no waits of its own).  While tile kt
// multiplies from its two buffers, the other three hold the next tile's
// halves and the following first half, in flight or landed (up to 96 KB per
// CU in flight; the L2-to-CU path measured about 9 TB/s with 64 KB in flight
// or half-line segments, 17-20 TB/s with 96-128 KB of whole lines).
//
// Per tile kt: step 0 requests the second half of tile kt+1 and step 1 the
// first half of tile kt+2, each into a buffer the previous tile freed, so
// that a wave's direct loads are spread over the tile instead of issued in
// one burst after the barrier (measured: 3-4% less time than refilling both
// freed buffers right after the barrier).  A first half is thus requested
// 1.5 tiles before its use and a second half 0.75 tile before; the first half
// is the operand that more often misses L2.  Steps 0-2 multiply while reading
// the next step's operands; then the wave waits until its loads of tile kt+1
// have landed (explicit vmcnt: the first half of kt+2 may stay in flight) and
// meets the others at the barrier, after which every wave has read its last
// operands of tile kt (its buffers are free) and every load of tile kt+1 has
// landed; step 3 multiplies while tile kt+1's first operands are read.
// ------------------------------------------------------------------------
constexpr int BG_WN = 4, BG_FM = 4, BG_FN = 2;  // 2 x 4 waves
constexpr int BG_LPH = 4;                        // direct loads per wave per operand half
constexpr int BG_BM = 256, BG_BN = 256;
constexpr int BG_HE = 256 * 64;  // elements per half (one operand of one tile)

// Block -> tile.  Workgroups are dealt round-robin over the 8 XCDs; the
// first part of the mapping gives each XCD a contiguous run of tile ids, the
// second walks them in groups of 8 token tiles, so the workgroups resident
// on one XCD share a few weight and activation tiles in its L2.
__device__ __forceinline__ void bg_tile(int64_t bid, int64_t tiles_m, int64_t tiles_n, int64_t& tm, int64_t& tn) {
  const int64_t n = tiles_m * tiles_n;
  const int64_t per = n / 8;
  int64_t t = bid;
  if (bid < per * 8) t = (bid % 8) * per + bid / 8;
  constexpr int64_t GM = 8;
  const int64_t group = t / (GM * tiles_n);
  const int64_t first = group * GM;
  const int64_t gs = (tiles_m - first) < GM ? (tiles_m - first) : GM;
  const int64_t in = t % (GM * tiles_n);
  tm = first + in % gs;
  tn = in / gs;
}

// Epilogue through LDS.  After the reduction each wave owns 128 tokens x 64
// weight rows (2 frags of 32) and a 16 KB LDS region.  Its results are
// written there in accumulator layout and read back as 16-byte row chunks,
// so that every global load and store of the epilogue covers whole row
// segments instead of 8-byte pieces of 32 different rows per instruction.
// Chunk c of row r sits at c ^ (r mod #chunks), which keeps both the writes
// and the row-chunk reads free of bank conflicts.
__device__ __forceinline__ f32x4 bg_mfma16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

// Position of H[token t][column c] in a wave's transposed H block [64
// columns][32 tokens] (bf16): the 16-byte chunk t / 8 of column c is stored at
// chunk (t / 8) ^ hsw(c), which keeps the column-wise MFMA operand reads (8
// columns per pass) and the token-wise writes of the epilogue off each
// other's banks.
__device__ __forceinline__ int bg_ht_index(int c, int t) {
  const int hsw = ((c >> 1) ^ (c >> 3)) & 3;
  return c * 32 + (((t >> 3) ^ hsw) << 3) + (t & 7);
}

// DAD: the SwiGLU backward also forms the dA_d partial (p.dad_part set)
template <int MODE, bool DAD>
// hp (SwiGLU forward): H of frag i at columns 8q + 4g .. + 3 as the two
// bf16 words that are stored, kept for the H A^T product.
__device__ __forceinline__ void bg_epilogue(const GemmArgs& p, f32x16 (&acc)[BG_FM][2], int64_t m0, int64_t n0,
                                             int wm, int wn, int lane, uint16_t* reg, f32x4 (&dad)[2][4],
                                             u32x2 (&hp)[BG_FM][4]) {
  constexpr int FM = BG_FM;
  const int l32 = lane & 31, g = lane >> 5;
  const int64_t mw = m0 + wm * 128;  // first token of the wave
  if constexpr (MODE == MODE_FWD_SWIGLU) {
    // G = acc[.][0], U = acc[.][1]: 32 intermediate columns per wave
    const int64_t cw = n0 + wn * 32;
    uint16_t* lg = reg;
    uint16_t* lu = reg + 128 * 32;
    auto wrw = [&](uint16_t* t, int i, int q, u32x2 w) {
      const int row = i * 32 + l32;
      *reinterpret_cast<u32x2*>(t + row * 32 + ((q ^ (row & 3)) * 8) + 4 * g) = w;
    };
    auto wr = [&](uint16_t* t, int i, int q, const float (&v)[4]) {
      wrw(t, i, q, u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])});
    };
    auto flush = [&](const uint16_t* t, uint16_t* out) {
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int row = it * 16 + (lane >> 2), c = lane & 3;
        const u32x4 v = *reinterpret_cast<const u32x4*>(t + row * 32 + ((c ^ (row & 3)) * 8));
        const int64_t m = mw + row, n = cw + c * 8;
        if (m < p.M && n < p.Nout) *reinterpret_cast<u32x4*>(out + m * p.Nout + n) = v;
      }
    };
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float G[4] = {acc[i][0][4 * q], acc[i][0][4 * q + 1], acc[i][0][4 * q + 2], acc[i][0][4 * q + 3]};
        const float U[4] = {acc[i][1][4 * q], acc[i][1][4 * q + 1], acc[i][1][4 * q + 2], acc[i][1][4 * q + 3]};
        wr(lg, i, q, G);
        wr(lu, i, q, U);
      }
    flush(lg, p.out0);
    flush(lu, p.out1);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float H[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float Gv = acc[i][0][4 * q + e], Uv = acc[i][1][4 * q + e];
          H[e] = Gv * sigmoid_fast(Gv) * Uv;
        }
        hp[i][q] = u32x2{pack_bf16x2(H[0], H[1]), pack_bf16x2(H[2], H[3])};
        wrw(lg, i, q, hp[i][q]);
      }
    flush(lg, p.out2);
  } else if constexpr (MODE == MODE_BWD_SWIGLU) {
    // dH (fp32) one token frag (32 rows x 64 columns, 8 KB) at a time through
    // the wave's LDS region.  G / U stream in as 16 row chunks (8 rows x 64
    // columns: one 16-byte piece per lane) kept LA = 6 chunks ahead of the chunk
    // being finished; buffer loads read rows past M as zeros and buffer
    // stores drop them (and columns past Nout), so that no memory operation
    // sits under a branch and every wait covers only what it must.
    const int64_t cw = n0 + wn * 64;
    const int c8 = lane & 7;  // this lane's 8-column group
    const int64_t ncol = cw + 8 * c8;
    const bool col_ok = ncol < p.Nout;
    const int64_t nc = col_ok ? ncol : p.Nout - 8;
    // resources over the tile's rows of G, U, dG, dU (at most 256 rows:
    // below 2 GiB for every accepted Nout)
    const int64_t tbytes = ((p.M - m0) < 256 ? (p.M - m0) : 256) * p.Nout * 2;
    auto trs = [&](const uint16_t* base) {
      return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base) + m0 * p.Nout, (short)0, (int)tbytes,
                                               0x00020000);
    };
    const __amdgpu_buffer_rsrc_t rsg = trs(p.in0), rsu = trs(p.in1), rsdg = trs(p.out0), rsdu = trs(p.out1);
    // byte offset of this lane's piece of chunk 0; chunk (i, it) adds the
    // wave-uniform (32 i + 8 it) rows
    const uint32_t lo = (uint32_t)(((int64_t)(wm * 128 + (lane >> 3)) * p.Nout + nc) * 2);
    const uint32_t lso = col_ok ? lo : 0x80000000u;
    auto chunk_so = [&](int c) { return (uint32_t)((32 * (c >> 2) + 8 * (c & 3)) * p.Nout * 2); };
    constexpr int NCH = FM * 4, LA = 6, SL = LA + 1;
    u32x4 gq[SL], uq[SL];
    // the whole offset goes in the lane offset: the range check covers the
    // lane offset only, not the scalar one
    auto ld = [&](int c) {
      const uint32_t o = lo + chunk_so(c);
      gq[c % SL] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsg, o, 0, 0));
      uq[c % SL] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsu, o, 0, 0));
    };
    // optional: the down layer's T^T H over this wave's 128 tokens x 64
    // columns, one 32-token frag at a time, with H = silu(G) U rounded to
    // bf16 and stored transposed after lf (T = l0.V, rank l0.r <= 32)
    constexpr bool with_dad = DAD;
    const int dr = p.l0.r;
    uint16_t* ht = reg + 4096;
    const int l16 = lane & 15, kq = lane >> 4;
    // T operand of frag i: ta[jf] = bf16 T[token 8 kq + e][j = 16 jf + l16]
    // for e < 8, one 16-byte load from the transposed copy (tokens past M
    // read as zeros: out-of-range offset; ranks past r masked at use)
    u32x4 ta[2];
    const __amdgpu_buffer_rsrc_t rst = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(p.dad_tt), (short)0, (int)(with_dad ? dr * p.dad_tt_ld * 2 : 0), 0x00020000);
    auto load_t = [&](int i) {
      const int64_t m = mw + i * 32 + 8 * kq;
      // bit 31 set past M: beyond the resource, reads zeros (arithmetic, not a
      // select, so that the loads stay out of branches)
      const uint32_t past = (uint32_t)(m >= p.M) << 31;
#pragma unroll
      for (int jf = 0; jf < 2; ++jf) {
        const int j = 16 * jf + l16;
        const uint32_t o = (uint32_t)(((j < dr ? j : dr - 1) * p.dad_tt_ld + (m < p.M ? m : 0)) * 2) | past;
        ta[jf] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rst, o, 0, 0));
      }
    };
    float* lf = reinterpret_cast<float*>(reg);
#pragma unroll
    for (int c = 0; c < LA; ++c) ld(c);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      if constexpr (DAD) load_t(i);
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = l32, c = 8 * f + 2 * q + g;  // 16-byte fp32 chunk of 16 per row
          *reinterpret_cast<f32x4*>(lf + row * 64 + ((c ^ (row & 15)) * 4)) =
              f32x4{acc[i][f][4 * q], acc[i][f][4 * q + 1], acc[i][f][4 * q + 2], acc[i][f][4 * q + 3]};
        }
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int ch = 4 * i + it;
        if (ch + LA < NCH) ld(ch + LA);
        const u32x4 gv = gq[ch % SL], uv = uq[ch % SL];
        const int row = it * 8 + (lane >> 3);
        const int c0 = 2 * c8;
        const f32x4 d0 = *reinterpret_cast<const f32x4*>(lf + row * 64 + ((c0 ^ (row & 15)) * 4));
        const f32x4 d1 = *reinterpret_cast<const f32x4*>(lf + row * 64 + (((c0 + 1) ^ (row & 15)) * 4));
        const float dH[8] = {d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
        u32x4 og, ou;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          float dG2[2], dU2[2];
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const float G = e ? bf16_hi(gv[d]) : bf16_lo(gv[d]);
            const float U = e ? bf16_hi(uv[d]) : bf16_lo(uv[d]);
            const float sg = sigmoid_fast(G);
            const float h = dH[2 * d + e];
            dU2[e] = h * G * sg;
            dG2[e] = h * U * sg * (1.0f + G * (1.0f - sg));
            if (with_dad)
              ht[bg_ht_index(8 * c8 + 2 * d + e, row)] = (uint16_t)(pack_bf16x2(G * sg * U, 0.0f) & 0xFFFFu);
          }
          og[d] = pack_bf16x2(dG2[0], dG2[1]);
          ou[d] = pack_bf16x2(dU2[0], dU2[1]);
        }
        const uint32_t so = lso + chunk_so(ch);
        __builtin_amdgcn_raw_buffer_store_b128(og, rsdg, so, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(ou, rsdu, so, 0, 0);
      }
      if (with_dad) {
        // A operand: T^T, lane (j, kq) holds T[token 8 kq + e][j] (zero past
        // M and past the rank); B operand: H^T rows, lane (column, kq) holds
        // H[token 8 kq + e][column]; result lane (column, q): j = 4 q + v
        u32x4 tb[2];
#pragma unroll
        for (int jf = 0; jf < 2; ++jf) {
          const bool jok = 16 * jf + l16 < dr;
#pragma unroll
          for (int d = 0; d < 4; ++d) tb[jf][d] = jok ? ta[jf][d] : 0u;
        }
#pragma unroll
        for (int cf = 0; cf < 4; ++cf) {
          const u32x4 hop = *reinterpret_cast<const u32x4*>(ht + bg_ht_index(16 * cf + l16, 8 * kq));
          dad[0][cf] = bg_mfma16(tb[0], hop, dad[0][cf]);
          if (dr > 16) dad[1][cf] = bg_mfma16(tb[1], hop, dad[1][cf]);
        }
      }
    }
  } else {
    // plain bf16 output: 128 tokens x 64 columns per wave, one pass
    const int64_t cw = n0 + wn * 64;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = i * 32 + l32, c = 4 * f + q;
          *reinterpret_cast<u32x2*>(reg + row * 64 + ((c ^ (row & 7)) * 8) + 4 * g) =
              u32x2{pack_bf16x2(acc[i][f][4 * q], acc[i][f][4 * q + 1]),
                    pack_bf16x2(acc[i][f][4 * q + 2], acc[i][f][4 * q + 3])};
        }
#pragma unroll
    for (int it = 0; it < 16; ++it) {
      const int row = it * 8 + (lane >> 3), c = lane & 7;
      const u32x4 v = *reinterpret_cast<const u32x4*>(reg + row * 64 + ((c ^ (row & 7)) * 8));
      const int64_t m = mw + row, n = cw + c * 8;
      if (m < p.M && n < p.Nout) *reinterpret_cast<u32x4*>(p.out0 + m * p.Nout + n) = v;
    }
  }
}

// SwiGLU forward, optional: the wave's share of H A^T (the down layer's
// rank-r product, A [r, Nout] bf16) from the bf16 H words the epilogue
// stored (hp).  Lane (token l32, g) holds H at columns cw + 8q + 4g + e
// (q, e < 4); taken as the A operand of two 32x32x16 MFMAs, step s covers
// q = 2s, 2s + 1, and the B operand reads A at the same columns, so no
// transpose is needed.  The 128 x 32 fp32 result goes to the wave's LDS
// region [token][j].
template <int MODE>
__device__ __forceinline__ void bg_had_wave(const GemmArgs& p, const u32x2 (&hp)[BG_FM][4], int64_t n0, int wn,
                                            int lane, float* reg) {
  const int l32 = lane & 31, g = lane >> 5;
  const int64_t cw = n0 + wn * 32;
  const bool jok = l32 < p.had_r;
  const uint16_t* arow = p.had_A + (int64_t)(jok ? l32 : 0) * p.Nout;
  u32x4 bop[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int64_t c0 = cw + 16 * s + 4 * g, c1 = c0 + 8;
    const u32x2 lo = (jok && c0 < p.Nout) ? *reinterpret_cast<const u32x2*>(arow + c0) : u32x2{0u, 0u};
    const u32x2 hi = (jok && c1 < p.Nout) ? *reinterpret_cast<const u32x2*>(arow + c1) : u32x2{0u, 0u};
    bop[s] = u32x4{lo[0], lo[1], hi[0], hi[1]};
  }
  // ranks past 16 hold zeros when r <= 16: not written (nor read back)
  const bool wj = l32 < (p.had_r <= 16 ? 16 : 32);
#pragma unroll
  for (int i = 0; i < BG_FM; ++i) {
    f32x16 h{};
#pragma unroll
    for (int s = 0; s < 2; ++s)
      h = mfma32(u32x4{hp[i][2 * s][0], hp[i][2 * s][1], hp[i][2 * s + 1][0], hp[i][2 * s + 1][1]}, bop[s], h);
    // h[v] = C[token 8(v/4) + 4g + v%4 of frag i][j = l32]
    if (wj) {
#pragma unroll
      for (int v = 0; v < 16; ++v) reg[(i * 32 + 8 * (v >> 2) + 4 * g + (v & 3)) * 32 + l32] = h[v];
    }
  }
}

// KMAJ: the weight operand is stored K-major, wb[k ldw + n] (an output head
// [V, D] read as the weight of the dX product, which reduces over V).  Its
// half-tile then sits in LDS as [64 k][256 n] (whole 512-byte row segments by
// direct loads; 16-byte chunk c of row k at c ^ 4 ((k / 8) % 2), so that the
// two lane halves of a read, 8 rows apart, hit different banks), and each
// A operand of the MFMA is gathered as 8 two-byte reads down a column.
template <int MODE, bool WLEAD, bool KMAJ = false, bool DAD = false>
__global__ __launch_bounds__(512) void bgemm_kernel(GemmArgs p) {
  constexpr int WN = BG_WN, FM = BG_FM, FN = BG_FN;
  constexpr int LPH = BG_LPH;
  constexpr int BM = BG_BM, BN = BG_BN;
  constexpr int BNO = ModeTraits<MODE>::swiglu_fwd ? BN / 2 : BN;

  __shared__ __attribute__((aligned(16))) uint16_t hb0[BG_HE];
  __shared__ __attribute__((aligned(16))) uint16_t hb1[BG_HE];
  __shared__ __attribute__((aligned(16))) uint16_t hb2[BG_HE];
  __shared__ __attribute__((aligned(16))) uint16_t hb3[BG_HE];
  __shared__ __attribute__((aligned(16))) uint16_t hb4[BG_HE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int l32 = lane & 31, g = lane >> 5;

  int64_t tm, tn;
  bg_tile(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
  const int64_t m0 = tm * BM;
  const int64_t n0 = tn * BNO;  // first output column
  const int64_t wr0 = tn * BN;  // first weight row of the tile
  const int KT0 = (int)(p.Kred0 / 64);
  const int64_t lda = p.lda > 0 ? p.lda : p.Kred0;  // activation row stride
  const int64_t lda1 = p.lda1 > 0 ? p.lda1 : lda;   // act1's
  // the SwiGLU forward's act1 (the LoRA extension) has its own row stride
  constexpr bool A1 = ModeTraits<MODE>::swiglu_fwd;
  // Reduction split (plain forward mode only, gridDim.y > 1): workgroup
  // (x, y) takes reduction tiles [kb, kb + KT) and writes fp32 partials.
  const int kb = gridDim.y > 1 ? (int)blockIdx.y * p.ktiles_per_split : 0;
  const int KTall = KT0 + (int)(p.Kred1 / 64);
  const int KT = gridDim.y > 1 ? min(KTall, kb + p.ktiles_per_split) - kb : KTall;

  // direct load i (0..7) of this wave: tile rows 8 (8 wave + i) + lane/8,
  // physical chunk lane%8 <- logical chunk (lane%8) ^ swz(row)
  uint32_t aoff[LPH], boff[LPH], aoff1[A1 ? LPH : 1];
#pragma unroll
  for (int i = 0; i < LPH; ++i) {
    const int row = 8 * (LPH * wave + i) + (lane >> 3);
    const int c = (lane & 7) ^ swz(row);
    int64_t ra = m0 + row;
    if (ra >= p.M) ra = p.M - 1;
    int64_t rb = wr0 + row;
    if (rb >= p.wrows) rb = p.wrows - 1;
    aoff[i] = (uint32_t)((ra - m0) * lda) + (uint32_t)c * 8;
    if constexpr (A1) aoff1[i] = (uint32_t)((ra - m0) * lda1) + (uint32_t)c * 8;
    boff[i] = (uint32_t)((rb - wr0) * p.ldw) + (uint32_t)c * 8;
    if constexpr (KMAJ) {
      // load i of this wave: reduction rows 2 (4 wave + i) + lane / 32 of the
      // tile, 16-byte chunk (lane % 32) ^ 4 ((row / 8) % 2) of its 256 columns
      const int kr = 2 * (LPH * wave + i) + (lane >> 5);
      const int kc = (lane & 31) ^ (((kr >> 3) & 1) * 4);
      boff[i] = (uint32_t)(kr * p.ldw) + (uint32_t)kc * 8;
    }
  }
  // Buffer resources over the tile's rows: the dual-reduction GEMM reads
  // act0 for the first KT0 tiles, then act1 (same row stride).  A direct load
  // is then one buffer load: fixed 32-bit lane offset, the tile's column
  // offset in the scalar offset, the LDS destination in M0.
  auto rsrc = [](const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0,
                                             (int)(bytes < 0x7FFFFFFF ? bytes : 0x7FFFFFFF), 0x00020000);
  };
  const int64_t abytes = (p.M - m0) * lda * 2;
  const __amdgpu_buffer_rsrc_t ra0 = rsrc(p.act0 + m0 * lda, abytes);
  const __amdgpu_buffer_rsrc_t ra1 = rsrc((p.act1 ? p.act1 : p.act0) + m0 * lda1, (p.M - m0) * lda1 * 2);
  const __amdgpu_buffer_rsrc_t rb = rsrc(p.wb + (KMAJ ? wr0 : wr0 * p.ldw), (p.wrows - wr0) * p.ldw * 2);

  // 8 direct loads of one operand half of tile kt (clamped to the last tile:
  // the tail re-loads it into a free buffer, which keeps vmcnt uniform)
#pragma unroll
  for (int i = 0; i < LPH; ++i) {
    aoff[i] *= 2;
    boff[i] *= 2;
    if constexpr (A1) aoff1[i] *= 2;
  }
  auto load_a = [&](uint16_t* buf, int kt) {
    kt = (kt < KT ? kt : KT - 1) + kb;
    const bool second = kt >= KT0;
    const int so = (second ? kt - KT0 : kt) * 128;
#pragma unroll
    for (int i = 0; i < LPH; ++i) {
      uint32_t off = aoff[i];
      if constexpr (A1) off = second ? aoff1[i] : off;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(second ? ra1 : ra0, LDS_PTR(buf + (LPH * wave + i) * 512), 16, off,
                                               so, 0, 0);
    }
  };
  auto load_b = [&](uint16_t* buf, int kt) {
    kt = (kt < KT ? kt : KT - 1) + kb;
    if constexpr (KMAJ) {
      // tile kt is rows 64 kt .. 64 kt + 63 of the weight: a resource based
      // at its first row (any weight size; offsets stay within the tile)
      const int64_t k0 = (int64_t)kt * 64;
      const __amdgpu_buffer_rsrc_t rk = rsrc(p.wb + k0 * p.ldw + wr0, ((p.Kred0 - k0) * p.ldw - wr0) * 2);
#pragma unroll
      for (int i = 0; i < LPH; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, LDS_PTR(buf + (LPH * wave + i) * 512), 16, boff[i], 0, 0, 0);
    } else {
#pragma unroll
      for (int i = 0; i < LPH; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, LDS_PTR(buf + (LPH * wave + i) * 512), 16, boff[i], kt * 128, 0,
                                                 0);
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int f = 0; f < FN; ++f)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][f][v] = 0.0f;

  // element offsets of this lane's operands within a half, per frag and
  // step (the same for every buffer, whose base goes to the read's offset)
  uint32_t aro[FM][4], bro[FN][4];
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int row = (wm * FM + i) * 32 + l32;
#pragma unroll
    for (int s = 0; s < 4; ++s) aro[i][s] = row * 64 + (((2 * s + g) ^ swz(row)) * 8);
  }
#pragma unroll
  for (int f = 0; f < FN; ++f) {
    const int row = frag_row<MODE, WN, FN>(wn, f) + l32;
#pragma unroll
    for (int s = 0; s < 4; ++s) bro[f][s] = row * 64 + (((2 * s + g) ^ swz(row)) * 8);
    if constexpr (KMAJ) {
      // column `row` of the [64][256] half: element (k, row) for k = 16 s +
      // 8 g + e lies at k 256 + bro[f][0] (chunk swizzle 4 g: (k / 8) % 2 = g)
      bro[f][0] = (8 * g) * 256 + ((((row >> 3) ^ (4 * g)) << 3) | (row & 7));
    }
  }

  // operands of 16-wide step s (0..3) of a tile held in halves (ha, hb)
  // The first half of each tile in the ring is requested half a tile earlier
  // than the second: WLEAD puts the weight operand first (chosen when it is
  // the larger matrix, whose tiles more often come from beyond L2).
  auto load_first = [&](uint16_t* buf, int kt) {
    if constexpr (WLEAD)
      load_b(buf, kt);
    else
      load_a(buf, kt);
  };
  auto load_second = [&](uint16_t* buf, int kt) {
    if constexpr (WLEAD)
      load_a(buf, kt);
    else
      load_b(buf, kt);
  };
  auto rd = [&](const uint16_t* h1, const uint16_t* h2, int s, u32x4 (&xa)[FM], u32x4 (&wa)[FN]) {
    const uint16_t* ha = WLEAD ? h2 : h1;
    const uint16_t* hb = WLEAD ? h1 : h2;
    if constexpr (KMAJ) {
#pragma unroll
      for (int f = 0; f < FN; ++f) {
        const uint16_t* col = hb + bro[f][0] + 16 * s * 256;
        uint32_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = col[e * 256];
        wa[f] = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
      }
    } else {
#pragma unroll
      for (int f = 0; f < FN; ++f) wa[f] = *reinterpret_cast<const u32x4*>(hb + bro[f][s]);
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) xa[i] = *reinterpret_cast<const u32x4*>(ha + aro[i][s]);
  };
  auto mm = [&](const u32x4 (&xa)[FM], const u32x4 (&wa)[FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int f = 0; f < FN; ++f) acc[i][f] = mfma32(wa[f], xa[i], acc[i][f]);
  };
  auto interleave_reads = [&]() {
#pragma unroll
    for (int j = 0; j < FM + FN; ++j) {
      SCHED_GROUP(SG_MFMA, 1);
      SCHED_GROUP(SG_DS_READ, 1);
    }
    SCHED_GROUP(SG_MFMA, FM * FN - FM - FN);
    __builtin_amdgcn_sched_barrier(0);
  };

  u32x4 x0[FM], w0[FN], x1[FM], w1[FN];
  // tile kt in halves (ca, cb); tile kt+1 goes to (na, nb), and fb is the
  // fifth buffer, which takes the first half of kt+2.  nb and fb were freed
  // by the barrier of tile kt-1.
  // The gate/up + SwiGLU kind raises its waves' priority over the three
  // matrix phases before the barrier, so that a wave with MFMAs ready issues
  // ahead of the other wave on its SIMD issuing loads (measured on the 8B
  // MLP: 1662 -> 1618 us; no gain for the other kinds).
  constexpr bool PRIO = ModeTraits<MODE>::swiglu_fwd;
  auto tile = [&](int kt, uint16_t* ca, uint16_t* cb, uint16_t* na, uint16_t* nb, uint16_t* fb) {
    rd(ca, cb, 1, x1, w1);
    load_second(nb, kt + 1);
    if constexpr (PRIO) __builtin_amdgcn_s_setprio(1);
    mm(x0, w0);
    interleave_reads();
    rd(ca, cb, 2, x0, w0);
    load_first(fb, kt + 2);
    mm(x1, w1);
    interleave_reads();
    rd(ca, cb, 3, x1, w1);
    mm(x0, w0);
    interleave_reads();
    if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
    wait_vmcnt<LPH>();  // tile kt+1 landed; the first half of kt+2 may be in flight
    stage_barrier();
    __builtin_amdgcn_sched_barrier(0);
    rd(na, nb, 0, x0, w0);
    mm(x1, w1);
    interleave_reads();
  };

  int64_t arow[FM];
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int64_t r = m0 + (int64_t)(wm * FM + i) * 32 + l32;
    arow[i] = r < p.M ? r : p.M - 1;
  }
  if (KT > 0) {
    // The LoRA term first.  Fast form: step 0 of every side is loaded before
    // the pipeline fill is issued (so the compiler's wait for it lets the
    // fill stay in flight) and applied after; remaining steps (rank > 16)
    // and the scalar form follow the fill.
    const LoraSide* L[2] = {&p.l0, &p.l0};
    int lo[2] = {0, 0}, hi[2] = {0, 0};
    // (none in the SwiGLU forward: it takes its LoRA terms as reduction
    // columns, act1 against the weight rows' extension)
    int ns = 0;
    if constexpr (!A1) ns = lora_sides<MODE, FN, true>(p, L, lo, hi);  // split runs: split 0 only
    const bool fast = lora_fast(*L[0]) && (ns < 2 || lora_fast(*L[1]));
    // One side's operands in registers at a time: with both sides' loads in
    // flight the prologue ran out of registers, and each spill store waited
    // for its load, a chain of memory round trips per tile.
    LoraRegs<FM, FN> R0;
    if (fast && ns > 0) lora_load<MODE, WN, FM, FN>(p, *L[0], 0, arow, n0, wn, l32, g, R0);
    load_first(hb0, 0);
    load_second(hb1, 0);
    load_first(hb2, 1);  // the second half of tile 1 is requested by tile 0
    if (fast) {
      if (ns > 0) lora_apply<FM, FN>(*L[0], 0, g, lo[0], hi[0], acc, R0);
      __builtin_amdgcn_sched_barrier(0);
      if (ns > 1) {
        lora_load<MODE, WN, FM, FN>(p, *L[1], 0, arow, n0, wn, l32, g, R0);
        lora_apply<FM, FN>(*L[1], 0, g, lo[1], hi[1], acc, R0);
      }
      for (int k = 0; k < ns; ++k)
        for (int t = 1; t < (L[k]->r + 15) / 16; ++t) {
          lora_load<MODE, WN, FM, FN>(p, *L[k], t, arow, n0, wn, l32, g, R0);
          lora_apply<FM, FN>(*L[k], t, g, lo[k], hi[k], acc, R0);
        }
    } else {
      for (int k = 0; k < ns; ++k)
        lora_scalar<MODE, WN, FM, FN>(p, *L[k], 0, acc, arow, n0, wn, l32, g, lo[k], hi[k]);
    }
    wait_vmcnt<LPH>();  // tile 0 landed
    stage_barrier();
    rd(hb0, hb1, 0, x0, w0);
    // half h of the sequence A0 B0 A1 B1 ... lives in buffer h % 5
    int kt = 0;
    for (; kt + 5 <= KT; kt += 5) {
      tile(kt, hb0, hb1, hb2, hb3, hb4);
      tile(kt + 1, hb2, hb3, hb4, hb0, hb1);
      tile(kt + 2, hb4, hb0, hb1, hb2, hb3);
      tile(kt + 3, hb1, hb2, hb3, hb4, hb0);
      tile(kt + 4, hb3, hb4, hb0, hb1, hb2);
    }
    const int rem = KT - kt;  // 0 .. 4
    if (rem > 0) tile(kt, hb0, hb1, hb2, hb3, hb4);
    if (rem > 1) tile(kt + 1, hb2, hb3, hb4, hb0, hb1);
    if (rem > 2) tile(kt + 2, hb4, hb0, hb1, hb2, hb3);
    if (rem > 3) tile(kt + 3, hb1, hb2, hb3, hb4, hb0);
    wait_vmcnt<0>();  // no direct load may still target LDS past this point
  }
  stage_barrier();  // every wave is done reading operands: LDS is free
  if constexpr (MODE == MODE_FWD) {
    if (gridDim.y > 1 || p.out_f32) {  // fp32 split partials, or fp32 results (partial[0])
      gemm_epilogue<MODE, 2, WN, FM, FN, true>(p, acc, arow, m0, n0, wm, wn, l32, g);
      return;
    }
  }
  if constexpr (MODE == MODE_FWD_SWIGLU) {
    if (p.row_scale) {
      // RMSNorm folded in: every token row of the product (LoRA term included)
      // times its inverse RMS; the norm weight is in the expanded weight
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const float rs = p.row_scale[arow[i]];
#pragma unroll
        for (int f = 0; f < FN; ++f)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[i][f][v] *= rs;
      }
    }
  }
  uint16_t* buf = wave < 2 ? hb0 : wave < 4 ? hb1 : wave < 6 ? hb2 : hb3;
  f32x4 dad[2][4];
#pragma unroll
  for (int jf = 0; jf < 2; ++jf)
#pragma unroll
    for (int cf = 0; cf < 4; ++cf) dad[jf][cf] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  u32x2 hp[FM][4];
  bg_epilogue<MODE, DAD>(p, acc, m0, n0, wm, wn, lane, buf + (wave & 1) * 8192, dad, hp);
  if constexpr (MODE == MODE_BWD_SWIGLU) {
    if (p.dad_part) {
      // the two token halves of each 64-column strip are added (waves 4..7
      // hand theirs to waves 0..3 through the fifth ring buffer) and written
      // as this token tile's partial dad_part[tm][column][j]
      float* xr = reinterpret_cast<float*>(hb4) + (wave & 3) * 2048;
      if (wm == 1) {
#pragma unroll
        for (int jf = 0; jf < 2; ++jf)
#pragma unroll
          for (int cf = 0; cf < 4; ++cf)
#pragma unroll
            for (int v = 0; v < 4; ++v) xr[((jf * 4 + cf) * 4 + v) * 64 + lane] = dad[jf][cf][v];
      }
      lds_barrier();  // an LDS exchange: the dG / dU stores need not land first
      if (wm == 0) {
        const int dr = p.l0.r;
        const int l16 = lane & 15, kq = lane >> 4;
#pragma unroll
        for (int jf = 0; jf < 2; ++jf)
#pragma unroll
          for (int cf = 0; cf < 4; ++cf) {
            const int64_t col = n0 + wn * 64 + 16 * cf + l16;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const int j = 16 * jf + 4 * kq + v;
              const float sum = dad[jf][cf][v] + xr[((jf * 4 + cf) * 4 + v) * 64 + lane];
              if (j < dr && col < p.Nout) p.dad_part[((int64_t)tm * p.Nout + col) * dr + j] = sum;
            }
          }
      }
    }
  }
  if constexpr (MODE == MODE_FWD_SWIGLU) {
    if (p.had_part) {
      // each wave's 128 tokens x 32 columns of H A^T into its region, then the
      // four waves of a token half are added in column order
      bg_had_wave<MODE>(p, hp, n0, wn, lane, reinterpret_cast<float*>(buf + (wave & 1) * 8192));
      lds_barrier();  // an LDS exchange: the G / U / H stores need not land first
      const int r = p.had_r;
      auto sum_out = [&](int hf, int t, int j) {
        float sum = 0.0f;
#pragma unroll
        for (int w4 = 0; w4 < 4; ++w4) {
          const int w = hf * 4 + w4;
          const uint16_t* bw = w < 2 ? hb0 : w < 4 ? hb1 : w < 6 ? hb2 : hb3;
          sum += reinterpret_cast<const float*>(bw + (w & 1) * 8192)[t * 32 + j];
        }
        const int64_t m = m0 + hf * 128 + t;
        if (j < r && m < p.M) p.had_part[((int64_t)tn * p.M + m) * r + j] = sum;
      };
      if (r <= 16) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int e = tid + 512 * k;  // [half][token][j < 16], 2 x 128 x 16
          sum_out(e >> 11, (e >> 4) & 127, e & 15);
        }
      } else {
#pragma unroll
        for (int k = 0; k < 16; ++k) {
          const int e = tid + 512 * k;  // [half][token][j], 2 x 128 x 32
          sum_out(e >> 12, (e >> 5) & 127, e & 31);
        }
      }
    }
  }
}

// ------------------------------------------------------------------------
// Weight expansion into bf16 rows.  The output is cut into 8-element
// chunks (16 bytes, one code dword); wave w expands chunks 256 w .. 256 w +
// 255, lane l taking chunks 256 w + 64 j + l (j < 4), so that every store
// instruction of a wave writes 1 KB of consecutive output and every code load
// reads 256 consecutive bytes.  With a SwiGLU pair the output rows come in
// blocks of 256: 128 gate rows, then the up rows of the same 128 columns;
// rows past N are written as zeros.
// ------------------------------------------------------------------------
__global__ __launch_bounds__(256) void dequant_rows_kernel(Nf4Dev w0, Nf4Dev w1, int pair,
                                                           const float* __restrict__ codebook0,
                                                           const float* __restrict__ codebook1, uint32_t cpr,
                                                           uint32_t nchunks, const uint16_t* __restrict__ colw,
                                                           int64_t ldo, uint16_t* __restrict__ out) {
  __shared__ float cb[32];  // tables of w0, w1
  if (threadIdx.x < 32) cb[threadIdx.x] = threadIdx.x < 16 ? codebook0[threadIdx.x] : codebook1[threadIdx.x & 15];
  __syncthreads();
  const int64_t K = w0.K;
  const uint32_t g0 = blockIdx.x * 1024u + (threadIdx.x >> 6) * 256u + (threadIdx.x & 63);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t g = g0 + 64u * j;
    if (g >= nchunks) break;
    const uint32_t R = g / cpr;
    const int64_t k0 = (int64_t)(g - R * cpr) * 8;
    bool up = false;
    int64_t src = R;
    if (pair) {
      const uint32_t within = R & 255u;
      up = within >= 128u;
      src = (int64_t)(R >> 8) * 128 + (within & 127u);
    }
    const Nf4Dev& w = up ? w1 : w0;
    u32x4 o = {0u, 0u, 0u, 0u};
    if (src < w.N) {
      const uint32_t c = *reinterpret_cast<const uint32_t*>(w.codes + src * (K / 2) + k0 / 2);
      const int64_t blk = (src * K + k0) / 64;
      const float a = w.dq ? absmax_at<true>(w, blk) : absmax_at<false>(w, blk);
      const float* t = up ? cb + 16 : cb;
      if (colw) {
        // column k scaled by colw[k]: fp32(fp32(codebook * absmax) * w), then bf16
        const u32x4 wv = *reinterpret_cast<const u32x4*>(colw + k0);
#pragma unroll
        for (int d = 0; d < 4; ++d)
          o[d] = pack_bf16x2(t[(c >> (8 * d)) & 15u] * a * bf16_lo(wv[d]), t[(c >> (8 * d + 4)) & 15u] * a * bf16_hi(wv[d]));
      } else {
        o = deq8(c, a, t);
      }
    }
    *reinterpret_cast<u32x4*>(out + (int64_t)R * ldo + k0) = o;
  }
}

// LoRA extension columns of the expanded SwiGLU pair rows: one thread per
// 8-column chunk of a row's ext columns.
__global__ __launch_bounds__(256) void lora_ext_cols_kernel(const uint16_t* __restrict__ Bg, int rg,
                                                            const uint16_t* __restrict__ Bu, int ru, int64_t N,
                                                            int64_t rows_out, int64_t K, int64_t ldo, int64_t ext,
                                                            uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t cpr = ext / 8;
  if (i >= rows_out * cpr) return;
  const int64_t R = i / cpr;
  const int q = (int)(i - R * cpr);
  const int64_t within = R & 255;
  const bool up = within >= 128;
  const int64_t src = (R >> 8) * 128 + (within & 127);
  uint32_t h[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int j = 8 * q + e;
    uint32_t v = 0u;
    if (src < N) {
      if (!up && j < rg) v = Bg[src * rg + j];
      if (up && j >= rg && j < rg + ru) v = Bu[src * ru + (j - rg)];
    }
    h[e] = v;
  }
  *reinterpret_cast<u32x4*>(out + R * ldo + K + 8 * q) =
      u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
}

// [s_g XA_g | s_u XA_u | 0] rounded to bf16, one thread per 8-column chunk.
__global__ __launch_bounds__(256) void lora_ext_act_kernel(const float* __restrict__ Vg, int rg, float sg,
                                                           const float* __restrict__ Vu, int ru, float su, int64_t M,
                                                           int64_t ext, uint16_t* __restrict__ act) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t cpr = ext / 8;
  if (i >= M * cpr) return;
  const int64_t m = i / cpr;
  const int q = (int)(i - m * cpr);
  float y[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int j = 8 * q + e;
    y[e] = j < rg ? sg * Vg[m * rg + j] : (j < rg + ru ? su * Vu[m * ru + (j - rg)] : 0.0f);
  }
  *reinterpret_cast<u32x4*>(act + m * ext + 8 * q) =
      u32x4{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]), pack_bf16x2(y[6], y[7])};
}

// T^T in bf16 for the dH epilogue's dA_d operand: out[j * ld + m] =
// bf16(T[m, j]), zero for M <= m < ld; one thread per 8 tokens of a rank.
__global__ __launch_bounds__(256) void t_bf16_trans_kernel(const float* __restrict__ T, int64_t M, int r,
                                                           int64_t ld, uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t per = ld / 8;
  if (i >= (int64_t)r * per) return;
  const int j = (int)(i / per);
  const int64_t m0 = (i - (int64_t)j * per) * 8;
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = m0 + e < M ? T[(m0 + e) * r + j] : 0.0f;
  *reinterpret_cast<u32x4*>(out + (int64_t)j * ld + m0) =
      u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
}

// ------------------------------------------------------------------------
// Transposed weight expansion: out[k, col0 + n] = deq(W)[n, k].  Workgroup
// -> 64 weight rows x 256 reduction columns.  Lane n of each wave expands
// 32 consecutive elements of weight row n0 + n and writes them down an LDS
// column (consecutive lanes -> consecutive halfwords); the tile is then
// written out as 128-byte row segments of out (8 lanes per row).
// ------------------------------------------------------------------------
constexpr int DT_LD = 72;  // LDS row stride (elements) of the [256 k][64 n] tile

__global__ __launch_bounds__(256) void dequant_trans_kernel(Nf4Dev w, const float* __restrict__ codebook,
                                                            uint16_t* __restrict__ out, int64_t ldo, int64_t col0) {
  __shared__ float cb[16];
  __shared__ __attribute__((aligned(16))) uint16_t tile[256 * DT_LD];
  if (threadIdx.x < 16) cb[threadIdx.x] = codebook[threadIdx.x];
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t n0 = (int64_t)blockIdx.x * 64;
  const int64_t k0 = (int64_t)blockIdx.y * 256;
  const int kn = (int)((w.K - k0) < 256 ? (w.K - k0) : 256);  // multiple of 64
  const int64_t n = n0 + lane;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = wave + 4 * j;  // 32-element chunk of the 256 columns
    if (32 * c >= kn) continue;
    const int64_t k = k0 + 32 * c;
    const u32x4 code = *reinterpret_cast<const u32x4*>(w.codes + n * (w.K / 2) + k / 2);
    const int64_t blk = (n * w.K + k) / 64;
    const float a = w.dq ? absmax_at<true>(w, blk) : absmax_at<false>(w, blk);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const u32x4 v = deq8(code[d], a, cb);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int kk = 32 * c + 8 * d + 2 * e;
        tile[kk * DT_LD + lane] = (uint16_t)(v[e] & 0xFFFFu);
        tile[(kk + 1) * DT_LD + lane] = (uint16_t)(v[e] >> 16);
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int kk = 32 * j + (threadIdx.x >> 3);
    if (kk >= kn) continue;
    const int ch = threadIdx.x & 7;
    const u32x4 v = *reinterpret_cast<const u32x4*>(&tile[kk * DT_LD + 8 * ch]);
    *reinterpret_cast<u32x4*>(out + (k0 + kk) * ldo + col0 + n0 + 8 * ch) = v;
  }
}

}  // namespace qk

using namespace qk;

template <int MODE>
static hipError_t run_bgemm(GemmArgs a, hipStream_t st) {
  constexpr int BNO = (MODE == MODE_FWD_SWIGLU) ? BG_BN / 2 : BG_BN;
  a.tiles_m = (a.M + BG_BM - 1) / BG_BM;
  a.tiles_n = (a.Nout + BNO - 1) / BNO;
  const int64_t n = a.tiles_m * a.tiles_n;
  if (n == 0) return hipSuccess;
  // the SwiGLU forward has no register-path LoRA term: its ranks must come as
  // act1 reduction columns
  if (MODE == MODE_FWD_SWIGLU && (a.l0.V || a.l1.V) && (a.Kred1 <= 0 || !a.act1)) return hipErrorInvalidValue;
  // the dA_d product reads T through its transposed bf16 copy
  if (MODE == MODE_BWD_SWIGLU && a.dad_part && (!a.dad_tt || a.dad_tt_ld < a.M || a.dad_tt_ld % 8 != 0))
    return hipErrorInvalidValue;
  // reduction splits (plain forward only): fp32 partials [splits][M][Nout]
  unsigned splits = 1;
  if (MODE == MODE_FWD && a.ktiles_per_split > 0 && a.partial) {
    const int64_t kt = (a.Kred0 + a.Kred1) / 64;
    splits = (unsigned)((kt + a.ktiles_per_split - 1) / a.ktiles_per_split);
  }
  if constexpr (MODE == MODE_FWD) {
    if (a.w_kmajor) {
      bgemm_kernel<MODE, false, true><<<dim3((unsigned)n, splits), 512, 0, st>>>(a);
      return hipGetLastError();
    }
  }
  if constexpr (MODE == MODE_BWD_SWIGLU) {
    if (a.dad_part) {
      if (a.wrows > a.M)
        bgemm_kernel<MODE, true, false, true><<<dim3((unsigned)n, splits), 512, 0, st>>>(a);
      else
        bgemm_kernel<MODE, false, false, true><<<dim3((unsigned)n, splits), 512, 0, st>>>(a);
      return hipGetLastError();
    }
  }
  if (a.wrows > a.M)
    bgemm_kernel<MODE, true><<<dim3((unsigned)n, splits), 512, 0, st>>>(a);
  else
    bgemm_kernel<MODE, false><<<dim3((unsigned)n, splits), 512, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_bgemm(int mode, const GemmArgs& a, hipStream_t st) {
  switch (mode) {
    case MODE_FWD: return run_bgemm<MODE_FWD>(a, st);
    case MODE_FWD_SWIGLU: return run_bgemm<MODE_FWD_SWIGLU>(a, st);
    case MODE_BWD: return run_bgemm<MODE_BWD>(a, st);
    case MODE_BWD_SWIGLU: return run_bgemm<MODE_BWD_SWIGLU>(a, st);
    case MODE_BWD_DUAL: return run_bgemm<MODE_BWD_DUAL>(a, st);
    default: return hipErrorInvalidValue;
  }
}

// out[m, j] = sum over column tiles t of part[t][m][j], in tile order.
__global__ __launch_bounds__(256) void had_finish_kernel(const float* __restrict__ part, int tiles, int64_t Mr,
                                                         float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= Mr) return;
  float s = 0.0f;
  int t = 0;
  for (; t + 8 <= tiles; t += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = part[(int64_t)(t + u) * Mr + i];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += v[u];
  }
  for (; t < tiles; ++t) s += part[(int64_t)t * Mr + i];
  out[i] = s;
}

hipError_t launch_had_finish(const float* part, int tiles, int64_t M, int r, float* out, hipStream_t st) {
  const int64_t n = M * r;
  if (n == 0) return hipSuccess;
  had_finish_kernel<<<dim3((unsigned)((n + 255) / 256)), 256, 0, st>>>(part, tiles, n, out);
  return hipGetLastError();
}

hipError_t launch_dequant_rows(const Nf4Dev& w0, const Nf4Dev* w1, const float* codebook0, const float* codebook1,
                               int64_t rows_out, uint16_t* out, hipStream_t st, const uint16_t* colw, int64_t ldo) {
  const int64_t cpr = w0.K / 8, chunks = rows_out * cpr;
  if (chunks == 0) return hipSuccess;
  if (chunks >= ((int64_t)1 << 32) - 1024) return hipErrorInvalidValue;  // 32-bit chunk index
  if (ldo == 0) ldo = w0.K;
  if (ldo < w0.K || ldo % 8 != 0) return hipErrorInvalidValue;
  dequant_rows_kernel<<<dim3((unsigned)((chunks + 1023) / 1024)), 256, 0, st>>>(
      w0, w1 ? *w1 : w0, w1 ? 1 : 0, codebook0, codebook1 ? codebook1 : codebook0, (uint32_t)cpr, (uint32_t)chunks,
      colw, ldo, out);
  return hipGetLastError();
}

hipError_t launch_t_bf16_trans(const float* T, int64_t M, int r, int64_t ld, uint16_t* out, hipStream_t st) {
  if (ld < M || ld % 8 != 0 || r < 1) return hipErrorInvalidValue;
  const int64_t n = (int64_t)r * (ld / 8);
  if (n == 0) return hipSuccess;
  t_bf16_trans_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(T, M, r, ld, out);
  return hipGetLastError();
}

hipError_t launch_lora_ext_cols(const uint16_t* Bg, int rg, const uint16_t* Bu, int ru, int64_t N, int64_t rows_out,
                                int64_t K, int64_t ldo, int64_t ext, uint16_t* out, hipStream_t st) {
  if (ext % 8 != 0 || K % 8 != 0 || ldo % 8 != 0 || ldo < K + ext || rg + ru > ext) return hipErrorInvalidValue;
  const int64_t n = rows_out * (ext / 8);
  if (n == 0) return hipSuccess;
  lora_ext_cols_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(Bg, rg, Bu, ru, N, rows_out, K, ldo, ext, out);
  return hipGetLastError();
}

hipError_t launch_lora_ext_act(const float* Vg, int rg, float sg, const float* Vu, int ru, float su, int64_t M,
                               int64_t ext, uint16_t* act, hipStream_t st) {
  if (ext % 8 != 0 || rg + ru > ext) return hipErrorInvalidValue;
  const int64_t n = M * (ext / 8);
  if (n == 0) return hipSuccess;
  lora_ext_act_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(Vg, rg, sg, Vu, ru, su, M, ext, act);
  return hipGetLastError();
}

hipError_t launch_dequant_trans(const Nf4Dev& w, const float* codebook, uint16_t* out, int64_t ldo, int64_t col0,
                                hipStream_t st) {
  if (w.N == 0 || w.K == 0) return hipSuccess;
  dim3 grid((unsigned)(w.N / 64), (unsigned)((w.K + 255) / 256));
  dequant_trans_kernel<<<grid, 256, 0, st>>>(w, codebook, out, ldo, col0);
  return hipGetLastError();
}
