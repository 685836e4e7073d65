// Device helpers shared by the gfx950 kernels: storage types, 8-element
// operand fragments and the 16x16 MFMA step that consumes them.
//
// MFMA operand layout used throughout (v_mfma_f32_16x16x32_bf16 and
// v_mfma_f32_16x16x4_f32 on CDNA4, wave64):
//   A fragment: lane l supplies row (l % 16), 8 consecutive k values of the
//               32-wide k step starting at 8 * (l / 16);
//   B fragment: lane l supplies column (l % 16), the same 8 k values;
//   C/D       : lane l holds column (l % 16), rows 4 * (l / 16) + 0..3.
// The kernels only rely on A and B agreeing on which k a lane supplies, so
// any consistent permutation of k inside a fragment is allowed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dflash {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// 8 storage elements as one MFMA operand fragment.
template <typename T> struct Frag8;
template <> struct Frag8<bf16> { typedef bf16x8 type; };
template <> struct Frag8<float> { typedef f32x8 type; };

__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f(float x) { return x; }

template <typename T> __device__ __forceinline__ T from_f(float x);
// round-to-nearest-even float -> bfloat16 (the compiler's conversion is RNE)
template <> __device__ __forceinline__ bf16 from_f<bf16>(float x) { return (bf16)x; }
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }

template <typename T>
__device__ __forceinline__ typename Frag8<T>::type load8(const T* p) {
  return *reinterpret_cast<const typename Frag8<T>::type*>(p);
}

template <typename T>
__device__ __forceinline__ typename Frag8<T>::type zero8() {
  typename Frag8<T>::type z;
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = (T)0.0f;
  return z;
}

// acc += A(16x32) * B(32x16) for one 32-wide k step.
__device__ __forceinline__ f32x4 mfma_step(bf16x8 a, bf16x8 b, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}
// fp32: the lane's 8 k values go to 8 separate 16x16x4 MFMAs; element e of
// every lane forms the 4-wide k step e.
__device__ __forceinline__ f32x4 mfma_step(f32x8 a, f32x8 b, f32x4 acc) {
#pragma unroll
  for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[e], b[e], acc, 0, 0, 0);
  return acc;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Element (m, k) of an activation matrix with K columns stored in MFMA
// fragment order, the order the tiled GEMM stages its operands in:
// [m / 16][k / 32][lane = m % 16 + 16 * (k % 32 / 8)][k % 8], so one
// fragment (16 rows x 32 k) is 1 KB of contiguous memory.  Four consecutive
// k from a multiple of 4 stay contiguous.
__device__ __forceinline__ long long frag_index(int m, int k, int K) {
  return ((((long long)(m >> 4) * (K >> 5) + (k >> 5)) * 64 + (m & 15) + 16 * ((k & 31) >> 3)) << 3) + (k & 7);
}

// Direct global -> LDS copy of 16 bytes per lane (no register staging): lane
// i's bytes land at lds_wave_base + 16 * i; the LDS address is wave-uniform.
// The copy counts as an outstanding vector-memory load until it has landed.
__device__ __forceinline__ void dma16(const void* src, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 0);
}
// The same with the nontemporal hint (data read once: weights, context K/V).
__device__ __forceinline__ void dma16_nt(const void* src, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)lds_wave_base, 16, 0, 2);
}

// At most N of this wave's vector-memory loads still outstanding and every
// LDS access of this wave complete, then the workgroup barrier.  The asm
// clobber keeps the compiler from moving memory accesses across it.
template <int N>
__device__ __forceinline__ void wait_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Stage ring of direct loads, NI per wave and stage: waits until at most
// min(ahead, A) later stages of this wave are still in flight, then joins the
// workgroup barrier.
template <int NI, int A>
__device__ __forceinline__ void wait_ring(int ahead) {
  if constexpr (A <= 0) {
    wait_barrier<0>();
  } else {
    if (ahead >= A)
      wait_barrier<A * NI>();
    else
      wait_ring<NI, A - 1>(ahead);
  }
}

// Sum over the 64 lanes of a wave (butterfly; every lane gets the result).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Order-preserving map of a float to an unsigned key (larger float, larger key).
__device__ __forceinline__ uint32_t float_key(float x) {
  uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_float(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

// Packed argmax key: larger logit wins, ties go to the lower id.
__device__ __forceinline__ uint64_t argmax_key(float logit, int id, int vocab) {
  return ((uint64_t)float_key(logit) << 32) | (uint32_t)(vocab - 1 - id);
}

__device__ __forceinline__ unsigned long long key_max(unsigned long long a, unsigned long long b) {
  return a > b ? a : b;
}
__device__ __forceinline__ unsigned long long key_min(unsigned long long a, unsigned long long b) {
  return a < b ? a : b;
}

// 16 adjacent lanes hold one key each (lane i of the group: index i); sort
// them descending (bitonic network over the group).
__device__ __forceinline__ unsigned long long sort16_desc(unsigned long long v, int i) {
#pragma unroll
  for (int k = 2; k <= 16; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const unsigned long long o = __shfl_xor(v, j, 64);
      const bool desc = (i & k) == 0;
      const bool lower = (i & j) == 0;
      v = (lower == desc) ? key_max(v, o) : key_min(v, o);
    }
  }
  return v;
}

// cur and nw are sorted descending over the same 16 lanes; returns the 16
// largest of both, sorted descending (lane i holds rank i).
__device__ __forceinline__ unsigned long long merge16_desc(unsigned long long cur, unsigned long long nw,
                                                           int i) {
  const int lane = threadIdx.x & 63;
  unsigned long long t = key_max(cur, __shfl(nw, (lane & 48) | (15 - i), 64));
#pragma unroll
  for (int j = 8; j > 0; j >>= 1) {
    const unsigned long long o = __shfl_xor(t, j, 64);
    t = ((i & j) == 0) ? key_max(t, o) : key_min(t, o);
  }
  return t;
}

// 64 keys, one per lane, sorted descending (bitonic network over the wave).
__device__ __forceinline__ unsigned long long sort64_desc(unsigned long long v, int lane) {
#pragma unroll
  for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const unsigned long long o = __shfl_xor(v, j, 64);
      const bool desc = (lane & k) == 0;
      const bool lower = (lane & j) == 0;
      v = (lower == desc) ? key_max(v, o) : key_min(v, o);
    }
  }
  return v;
}

// cur and nw are sorted descending over the 64 lanes; returns the 64 largest
// of both, sorted descending (the reversed second list against the first is
// bitonic, then a half-cleaner network).
__device__ __forceinline__ unsigned long long merge64_desc(unsigned long long cur, unsigned long long nw, int lane) {
  unsigned long long v = key_max(cur, __shfl(nw, 63 - lane, 64));
#pragma unroll
  for (int j = 32; j >= 1; j >>= 1) {
    const unsigned long long o = __shfl_xor(v, j, 64);
    v = ((lane & j) == 0) ? key_max(v, o) : key_min(v, o);
  }
  return v;
}

}  // namespace dflash
