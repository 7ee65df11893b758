// Shared device-side types and helpers for the gfx950 (CDNA4) kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dit {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte vector of element type T: 8 bf16 or 4 fp32 (one lane's share of an
// MFMA operand load).
template <class T> struct Vec;
template <> struct Vec<bf16> { typedef bf16x8 type; static constexpr int n = 8; };
template <> struct Vec<float> { typedef f32x4 type; static constexpr int n = 4; };

__device__ __forceinline__ float to_f(float x) { return x; }
__device__ __forceinline__ float to_f(bf16 x) { return (float)x; }
template <class T> __device__ __forceinline__ T from_f(float x);
template <> __device__ __forceinline__ float from_f<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f<bf16>(float x) { return (bf16)x; }

// Raw 16-byte global / LDS moves.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// 32x32 MFMA over one 16-byte operand vector per lane.
// bf16: one v_mfma_f32_32x32x16_bf16 (K = 16 = 2 lane groups x 8).
// fp32: four v_mfma_f32_32x32x2f32, element i of each lane's vector feeding
//       step i (K = 2 per step); both operands use the same element order, so
//       the 8 products summed are exactly the 8 k indices of the two vectors.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(f32x4 a, f32x4 b, f32x16 c) {
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[0], b[0], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[1], b[1], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[2], b[2], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[3], b[3], c, 0, 0, 0);
  return c;
}

template <class V> __device__ __forceinline__ V as_vec(u32x4 r) { return __builtin_bit_cast(V, r); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// GELU, tanh form: 0.5 x (1 + tanh(u)), u = sqrt(2/pi) (x + 0.044715 x^3).
// 1 + tanh(u) = 2 - 2 / (1 + e^{2u}) = 2 e^{2u} / (1 + e^{2u}); with e^{2u} from the
// hardware exp2 this is x * e / (1 + e) (saturating to x or 0 when e overflows/underflows).
__device__ __forceinline__ float gelu_tanh(float x) {
  const float k0 = 0.7978845608028654f;  // sqrt(2/pi)
  const float k1 = 0.044715f;
  const float u = k0 * fmaf(k1 * x, x * x, x);
  const float e = __builtin_amdgcn_exp2f(u * 2.8853900817779268f);  // e^{2u} = 2^{2u log2 e}
  return isinf(e) ? x : x * e * __builtin_amdgcn_rcpf(1.0f + e);
}

// Workgroups are dispatched round-robin over the 8 XCDs of the chip (each with its own
// L2).  Map dispatch index b to a logical index so that each XCD processes one
// contiguous range of logical work items: neighbours in the logical order then share
// an L2.
__device__ __forceinline__ int xcd_remap(int b, int total) {
  constexpr int NXCD = 8;
  const int x = b % NXCD, i = b / NXCD;
  const int q = total / NXCD, r = total % NXCD;
  return x * q + min(x, r) + i;
}
__device__ __forceinline__ float silu(float x) { return x / (1.0f + expf(-x)); }

// 4 consecutive elements <-> 4 floats (8-byte bf16 or 16-byte fp32 access).
template <class T> __device__ __forceinline__ void load4(const T* p, float v[4]);
template <> __device__ __forceinline__ void load4<float>(const float* p, float v[4]) {
  f32x4 r = *reinterpret_cast<const f32x4*>(p);
  v[0] = r[0]; v[1] = r[1]; v[2] = r[2]; v[3] = r[3];
}
template <> __device__ __forceinline__ void load4<bf16>(const bf16* p, float v[4]) {
  typedef bf16 b4 __attribute__((ext_vector_type(4)));
  b4 r = *reinterpret_cast<const b4*>(p);
  v[0] = (float)r[0]; v[1] = (float)r[1]; v[2] = (float)r[2]; v[3] = (float)r[3];
}
template <class T> __device__ __forceinline__ void store4(T* p, const float v[4]);
template <> __device__ __forceinline__ void store4<float>(float* p, const float v[4]) {
  f32x4 r = {v[0], v[1], v[2], v[3]};
  *reinterpret_cast<f32x4*>(p) = r;
}
template <> __device__ __forceinline__ void store4<bf16>(bf16* p, const float v[4]) {
  typedef bf16 b4 __attribute__((ext_vector_type(4)));
  b4 r = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
  *reinterpret_cast<b4*>(p) = r;
}


// Workgroup barrier that keeps direct-to-LDS loads in flight.  __syncthreads() carries
// a workgroup fence, which the compiler implements by draining every outstanding
// memory operation (vmcnt(0)), including global_load_lds transfers issued for later
// tiles.  Callers of this barrier instead wait explicitly (vmcnt(N) for their own
// older transfers, lgkmcnt(0) for their LDS reads) before it; the memory clobber
// keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

// s_waitcnt vmcnt(N) lgkmcnt(0); expcnt left at its maximum (7).
template <int N> __device__ __forceinline__ void wait_vm_lds() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

}  // namespace dit
