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
// bgemm_kernel: output tile 256 tokens x 256 weight rows, 4 waves (one per
// SIMD) in a 2 x 2 grid, each 128 x 128 = 4 x 4 frags of 32x32, fp32
// accumulators.  Per 64-wide reduction tile both operand tiles ([256][64]
// bf16, 16-byte chunks swizzled by swz(row)) are double-buffered in LDS
// (128 KB).  Each thread stages 8 + 8 16-byte chunks of the next tile in
// registers: loaded right after the barrier that opens a tile, written to
// the other LDS buffer after the tile's MFMAs, so the global latency hides
// behind one tile of matrix work and one LDS-only barrier per tile suffices.
// ------------------------------------------------------------------------
constexpr int BG_WM = 2, BG_WN = 2, BG_FM = 4, BG_FN = 4;
constexpr int BG_BM = 256, BG_BN = 256;

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

template <int MODE>
__global__ __launch_bounds__(256) void bgemm_kernel(GemmArgs p) {
  constexpr int WM = BG_WM, WN = BG_WN, FM = BG_FM, FN = BG_FN;
  constexpr int BM = BG_BM, BN = BG_BN;
  constexpr int BNO = ModeTraits<MODE>::swiglu_fwd ? BN / 2 : BN;

  __shared__ __attribute__((aligned(16))) uint16_t sa[2][BM * 64];
  __shared__ __attribute__((aligned(16))) uint16_t sb[2][BN * 64];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int l32 = lane & 31, g = lane >> 5;

  int64_t tm, tn;
  bg_tile(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
  const int64_t m0 = tm * BM;
  const int64_t n0 = tn * BNO;        // first output column
  const int64_t wr0 = tn * BN;        // first weight row of the tile
  const int KT0 = (int)(p.Kred0 / 64);
  const int KT = KT0 + (int)(p.Kred1 / 64);

  // staging chunk i of this thread: tile row 32 i + 8 wave + lane/8, 16-byte
  // chunk lane%8 (8 lanes cover one 128-byte row segment)
  uint32_t aoff[8], boff[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = 32 * i + 8 * wave + (lane >> 3);
    int64_t ra = m0 + row;
    if (ra >= p.M) ra = p.M - 1;
    int64_t rb = wr0 + row;
    if (rb >= p.wrows) rb = p.wrows - 1;
    aoff[i] = (uint32_t)((ra - m0) * p.Kred0) + (uint32_t)(lane & 7) * 8;
    boff[i] = (uint32_t)((rb - wr0) * p.ldw) + (uint32_t)(lane & 7) * 8;
  }
  // the dual-reduction GEMM reads act0 for the first KT0 tiles, then act1
  const uint16_t* abase0 = p.act0 + m0 * p.Kred0;
  const uint16_t* abase1 = (p.act1 ? p.act1 + m0 * p.Kred0 : abase0) - (int64_t)KT0 * 64;
  const uint16_t* bbase = p.wb + wr0 * p.ldw;

  u32x4 ra[8], rb[8];
  auto gload = [&](int kt) {
    const uint16_t* a = (kt < KT0 ? abase0 : abase1) + (int64_t)kt * 64;
    const uint16_t* b = bbase + (int64_t)kt * 64;
#pragma unroll
    for (int i = 0; i < 8; ++i) {  // same order as the refills in lstore
      ra[i] = *reinterpret_cast<const u32x4*>(a + aoff[i]);
      rb[i] = *reinterpret_cast<const u32x4*>(b + boff[i]);
    }
  };
  // staged chunks [4h, 4h + 4) of both operands into LDS buffer `buf`; with
  // `reload`, each register is refilled from tile kt right after its store
  auto lstore = [&](int buf, int h, bool reload, int kt) {
    const uint16_t* a = (kt < KT0 ? abase0 : abase1) + (int64_t)kt * 64;
    const uint16_t* b = bbase + (int64_t)kt * 64;
#pragma unroll
    for (int i = 4 * h; i < 4 * h + 4; ++i) {
      const int row = 32 * i + 8 * wave + (lane >> 3);
      const int off = row * 64 + (((lane & 7) ^ swz(row)) * 8);
      *reinterpret_cast<u32x4*>(&sa[buf][off]) = ra[i];
      if (reload) ra[i] = *reinterpret_cast<const u32x4*>(a + aoff[i]);
      *reinterpret_cast<u32x4*>(&sb[buf][off]) = rb[i];
      if (reload) rb[i] = *reinterpret_cast<const u32x4*>(b + boff[i]);
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int f = 0; f < FN; ++f)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][f][v] = 0.0f;

  // LDS offsets (elements) of this lane's operand rows
  int arow_l[FM], brow_l[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) arow_l[i] = (wm * FM + i) * 32 + l32;
#pragma unroll
  for (int f = 0; f < FN; ++f) brow_l[f] = frag_row<MODE, WN, FN>(wn, f) + l32;

  // operands of one 16-wide reduction step s of LDS buffer `buf`
  auto rd = [&](int buf, int s, u32x4 (&xa)[FM], u32x4 (&wa)[FN]) {
#pragma unroll
    for (int f = 0; f < FN; ++f) {
      const int row = brow_l[f];
      wa[f] = *reinterpret_cast<const u32x4*>(&sb[buf][row * 64 + (((2 * s + g) ^ swz(row)) * 8)]);
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int row = arow_l[i];
      xa[i] = *reinterpret_cast<const u32x4*>(&sa[buf][row * 64 + (((2 * s + g) ^ swz(row)) * 8)]);
    }
  };
  auto mm = [&](const u32x4 (&xa)[FM], const u32x4 (&wa)[FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int f = 0; f < FN; ++f) acc[i][f] = mfma32(wa[f], xa[i], acc[i][f]);
  };
  auto mm_half = [&](const u32x4 (&xa)[FM], const u32x4 (&wa)[FN], int h) {
#pragma unroll
    for (int i = 2 * h; i < 2 * h + 2; ++i)
#pragma unroll
      for (int f = 0; f < FN; ++f) acc[i][f] = mfma32(wa[f], xa[i], acc[i][f]);
  };

  // Software pipeline over one reduction tile (4 steps x 16 MFMAs): the
  // operands of step s+1 are read while step s multiplies (two register
  // sets); during steps 2 and 3 the staged next tile goes to the other LDS
  // buffer, each staging register being refilled from the tile after that
  // right after its store, so every global load has one whole tile of matrix
  // work to arrive.  The group barriers pin the interleave: one LDS access
  // (and one global load) next to each MFMA.
  u32x4 x0[FM], w0[FN], x1[FM], w1[FN];
  auto tile = [&](int kt, auto more) {
    constexpr bool MORE = decltype(more)::value;  // a next tile exists
    const int cur = kt & 1, nxt = cur ^ 1;
    rd(cur, 1, x1, w1);
    mm(x0, w0);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      SCHED_GROUP(SG_MFMA, 1);
      SCHED_GROUP(SG_DS_READ, 1);
    }
    SCHED_GROUP(SG_MFMA, 8);
    __builtin_amdgcn_sched_barrier(0);
    rd(cur, 2, x0, w0);
    mm(x1, w1);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      SCHED_GROUP(SG_MFMA, 1);
      SCHED_GROUP(SG_DS_READ, 1);
    }
    SCHED_GROUP(SG_MFMA, 8);
    __builtin_amdgcn_sched_barrier(0);
    rd(cur, 3, x1, w1);
    if constexpr (MORE) lstore(nxt, 0, true, min(kt + 2, KT - 1));
    mm(x0, w0);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      SCHED_GROUP(SG_MFMA, 1);
      SCHED_GROUP(SG_DS_READ, 1);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      SCHED_GROUP(SG_MFMA, 1);
      if (MORE) {
        SCHED_GROUP(SG_DS_WRITE, 1);
        SCHED_GROUP(SG_VMEM_READ, 1);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (MORE) lstore(nxt, 1, true, min(kt + 2, KT - 1));
    mm_half(x1, w1, 0);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      SCHED_GROUP(SG_MFMA, 1);
      if (MORE) {
        SCHED_GROUP(SG_DS_WRITE, 1);
        SCHED_GROUP(SG_VMEM_READ, 1);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // Every LDS access of this wave to buffer `cur` and every store into
    // `nxt` is complete at this barrier, so the next tile's first operands
    // are read while the last MFMAs of this tile run.
    if constexpr (MORE) {
      lds_barrier();
      rd(nxt, 0, x0, w0);
    }
    mm_half(x1, w1, 1);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      SCHED_GROUP(SG_MFMA, 1);
      if (MORE) SCHED_GROUP(SG_DS_READ, 1);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  if (KT > 0) {
    gload(0);
    lstore(0, 0, true, min(1, KT - 1));
    lstore(0, 1, true, min(1, KT - 1));
    lds_barrier();
    rd(0, 0, x0, w0);
    int kt = 0;
    for (; kt + 1 < KT; ++kt) tile(kt, std::true_type{});
    tile(kt, std::false_type{});
  }

  int64_t arow[FM];
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int64_t r = m0 + (int64_t)(wm * FM + i) * 32 + l32;
    arow[i] = r < p.M ? r : p.M - 1;
  }
  gemm_epilogue<MODE, WM, WN, FM, FN, false>(p, acc, arow, m0, n0, wm, wn, l32, g);
}

// ------------------------------------------------------------------------
// Weight expansion into bf16 rows.  Thread -> 32 consecutive elements of one
// output row (16-byte code load, four 16-byte stores).  With a SwiGLU pair
// the output rows come in blocks of 256: 128 gate rows, then the up rows of
// the same 128 columns; rows past N are written as zeros.
// ------------------------------------------------------------------------
__global__ __launch_bounds__(256) void dequant_rows_kernel(Nf4Dev w0, Nf4Dev w1, int pair,
                                                           const float* __restrict__ codebook0,
                                                           const float* __restrict__ codebook1, int64_t rows_out,
                                                           uint16_t* __restrict__ out) {
  __shared__ float cb[32];  // tables of w0, w1
  if (threadIdx.x < 32) cb[threadIdx.x] = threadIdx.x < 16 ? codebook0[threadIdx.x] : codebook1[threadIdx.x & 15];
  __syncthreads();
  const int64_t K = w0.K;
  const int64_t per_row = K / 32;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= rows_out * per_row) return;
  const int64_t R = t / per_row;
  const int64_t k0 = (t % per_row) * 32;
  bool up = false;
  int64_t src = R;
  if (pair) {
    const int64_t within = R & 255;
    up = within >= 128;
    src = (R >> 8) * 128 + (within & 127);
  }
  const Nf4Dev& w = up ? w1 : w0;
  u32x4 o[4] = {};
  if (src < w.N) {
    const u32x4 c = *reinterpret_cast<const u32x4*>(w.codes + src * (K / 2) + k0 / 2);
    const int64_t blk = (src * K + k0) / 64;
    const float a = w.dq ? absmax_at<true>(w, blk) : absmax_at<false>(w, blk);
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = deq8(c[j], a, up ? cb + 16 : cb);
  }
  uint16_t* dst = out + R * K + k0;
#pragma unroll
  for (int j = 0; j < 4; ++j) reinterpret_cast<u32x4*>(dst)[j] = o[j];
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
  bgemm_kernel<MODE><<<dim3((unsigned)n), 256, 0, st>>>(a);
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

hipError_t launch_dequant_rows(const Nf4Dev& w0, const Nf4Dev* w1, const float* codebook0, const float* codebook1,
                               int64_t rows_out, uint16_t* out, hipStream_t st) {
  const int64_t threads = rows_out * (w0.K / 32);
  if (threads == 0) return hipSuccess;
  dequant_rows_kernel<<<dim3((unsigned)((threads + 255) / 256)), 256, 0, st>>>(
      w0, w1 ? *w1 : w0, w1 ? 1 : 0, codebook0, codebook1 ? codebook1 : codebook0, rows_out, out);
  return hipGetLastError();
}

hipError_t launch_dequant_trans(const Nf4Dev& w, const float* codebook, uint16_t* out, int64_t ldo, int64_t col0,
                                hipStream_t st) {
  if (w.N == 0 || w.K == 0) return hipSuccess;
  dim3 grid((unsigned)(w.N / 64), (unsigned)((w.K + 255) / 256));
  dequant_trans_kernel<<<grid, 256, 0, st>>>(w, codebook, out, ldo, col0);
  return hipGetLastError();
}
