// Pieces shared by the attention kernels: the key tile size, the LDS chunk swizzle and
// the row sum of the bf16 P^T operand.
#pragma once
#include "common.h"

namespace dit {

// Row-sum accumulation from the P^T operand vector.
__device__ __forceinline__ float row_sum_add(bf16x8 p, float acc) {
  typedef bf16 b2 __attribute__((ext_vector_type(2)));
  const b2 one = {(bf16)1.0f, (bf16)1.0f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    b2 q = {p[2 * i], p[2 * i + 1]};
    acc = __builtin_amdgcn_fdot2_f32_bf16(q, one, acc, false);
  }
  return acc;
}
__device__ __forceinline__ float row_sum_add(f32x4 p, float acc) {
  return acc + p[0] + p[1] + p[2] + p[3];
}
constexpr int BKV = 64;  // keys per tile


// 16-byte chunk position of chunk c of row r in an unpadded LDS tile whose rows are RB
// bytes: consecutive rows reading the same chunk spread over all 64 banks.
template <int RB>
__device__ __forceinline__ int swz(int r, int c) {
  if constexpr (RB >= 256) return c ^ (r & 15);
  else return c ^ ((r >> 1) & 7);
}

}  // namespace dit
