// Device-side helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// Instruction-class masks for __builtin_amdgcn_sched_group_barrier: pin the
// interleave of matrix, LDS and global instructions in a scheduling region.
#define SCHED_GROUP(mask, n) __builtin_amdgcn_sched_group_barrier(mask, n, 0)
#define SG_VALU 0x002
#define SG_MFMA 0x008
#define SG_VMEM_READ 0x020
#define SG_DS_READ 0x100
#define SG_DS_WRITE 0x200

namespace qk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// fp32 -> bf16 round-to-nearest-even for two values, packed lo | hi << 16
// (gfx950 converts with v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// One 32x32x16 bf16 MFMA: C[32x32] += A[32x16] * B[16x32].
// Lane l holds A[l%32][8*(l/32) + 0..7] and B[8*(l/32) + 0..7][l%32];
// accumulator element v of lane l is C[8*(v/4) + 4*(l/32) + v%4][l%32].
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// 16-byte chunk swizzle for [row][64 bf16] LDS tiles (8 chunks per row): the
// 8 lanes that read one chunk column of 8 consecutive rows, and the 8 lanes
// that write one chunk of rows 8 apart, all hit different bank groups.
__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 7); }

// Workgroup barrier that orders LDS only: LDS writes before it are complete
// and visible to the workgroup after it, while global loads issued before it
// (register prefetches of later tiles) may still be in flight.  A plain
// __syncthreads() also waits for every outstanding global load.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// s_waitcnt with only the vector-memory counter: wait until at most N of this
// wave's vector memory operations are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for LDS data written by direct loads: LDS accesses of
// this wave complete (lgkmcnt), then s_barrier.  The memory clobber keeps the
// compiler from moving memory accesses across it.  The caller has already
// waited (vmcnt) for the direct loads that must be visible after it.
__device__ __forceinline__ void stage_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

__device__ __forceinline__ float sigmoidf_(float g) { return 1.0f / (1.0f + __expf(-g)); }

// sigmoid with the hardware reciprocal (v_rcp_f32, about 1 ulp) instead of
// the correctly rounded division: for values that are rounded to bf16 next.
__device__ __forceinline__ float sigmoid_fast(float g) { return __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

}  // namespace qk
