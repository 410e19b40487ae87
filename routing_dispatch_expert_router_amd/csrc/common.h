// Internal helpers shared by the gfx950 kernels of libmoe.so (not part of the ABI).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;

// ---------------------------------------------------------------- bf16 <-> f32
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}
// round to nearest, ties to even (inputs here are finite)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__host__ __device__ inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// storage type traits: activations / weights are either bf16 (uint16 bits) or f32
template <typename T> struct Elem;
template <> struct Elem<uint16_t> {
  static constexpr int kPer16B = 8;  // elements per 16-byte chunk
  __device__ __forceinline__ static float load(const uint16_t *p) { return bf16_to_f32(*p); }
  __device__ __forceinline__ static uint16_t from_f32(float f) { return f32_to_bf16(f); }
  __device__ __forceinline__ static float to_f32(uint16_t v) { return bf16_to_f32(v); }
};
template <> struct Elem<float> {
  static constexpr int kPer16B = 4;
  __device__ __forceinline__ static float load(const float *p) { return *p; }
  __device__ __forceinline__ static float from_f32(float f) { return f; }
  __device__ __forceinline__ static float to_f32(float v) { return v; }
};

// ---------------------------------------------------------------- MFMA
// One 16x16 output block, contraction over the 16 bytes each lane holds of A
// and B (8 bf16 or 4 f32).  Lane l holds A row (l % 16) and B column (l % 16);
// which k each byte stands for does not matter as long as A and B agree.
// Result layout: acc[i] = C[4*(l/16) + i][l % 16].
__device__ __forceinline__ f32x4 mma16(const u32x4 &a, const u32x4 &b, f32x4 acc, uint16_t) {
  bf16x8 av = __builtin_bit_cast(bf16x8, a);
  bf16x8 bv = __builtin_bit_cast(bf16x8, b);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(const u32x4 &a, const u32x4 &b, f32x4 acc, float) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[0]), __uint_as_float(b[0]), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[1]), __uint_as_float(b[1]), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[2]), __uint_as_float(b[2]), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[3]), __uint_as_float(b[3]), acc, 0, 0, 0);
  return acc;
}

// ---------------------------------------------------------------- gfx950 memory ops
// 16 bytes per lane straight from global memory into LDS (global_load_lds_dwordx4):
// lane l's data lands at lds_wave_base + 16*l, so lds_wave_base must be
// wave-uniform.  Tracked by vmcnt.
__device__ __forceinline__ void load_lds16(const void *gsrc, void *lds_wave_base) {
  __builtin_amdgcn_global_load_lds(gsrc, lds_wave_base, 16, 0, 0);
}
// 4 bytes per lane from global memory into LDS (global_load_lds_dword); used to
// pull a future cache line into L2 without holding a register for it
__device__ __forceinline__ void load_lds4(const void *gsrc, void *lds_wave_base) {
  __builtin_amdgcn_global_load_lds(gsrc, lds_wave_base, 4, 0, 0);
}
// wait until at most N vector-memory loads of this wave are outstanding
// (s_waitcnt vmcnt(N)); gfx9 encoding: vmcnt[3:0] | expcnt[6:4] |
// lgkmcnt[11:8] | vmcnt[5:4] << 14, expcnt and lgkmcnt left at "no wait"
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}
__device__ __forceinline__ void wait_vmcnt0() { wait_vmcnt<0>(); }
// wait until this wave's LDS (and scalar-memory) operations have completed
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Workgroup barrier without a memory fence, for the k-loops that stream
// operands into LDS with global -> LDS loads.  __syncthreads() also issues a
// workgroup release fence, and on gfx950 that fence waits for every
// outstanding vector-memory load (LDS DMA counts as an LDS write), so a chunk
// prefetched two steps ahead would be waited for at the next barrier.  The
// caller waits itself for what the other waves must see: its LDS reads
// (wait_lgkmcnt0) and its global -> LDS loads of the chunk about to be read
// (wait_vmcnt<N>).  The memory clobber keeps the compiler from moving LDS
// accesses across the barrier.
__device__ __forceinline__ void barrier_nofence() { asm volatile("s_barrier" ::: "memory"); }

// ---------------------------------------------------------------- wave helpers
__device__ __forceinline__ int lane_id() { return threadIdx.x & (WAVE - 1); }
// wave index in the workgroup, as a scalar (wave-uniform) value
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE); }

// order-preserving key of a float score: larger float -> larger key; -0.0 == +0.0
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float wave_max(float v, int width) {
  for (int o = width >> 1; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
  return v;
}
__device__ __forceinline__ float group_sum_fixed(float v, int width) {
  // butterfly: every lane of the group ends with the same value, and the
  // association order is fixed by the lane pattern (deterministic)
  for (int o = width >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}

}  // namespace moe
