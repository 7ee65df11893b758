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

// One 64-key tile of dh = 128 bf16 keys for the short-segment softmax: key row r at
// r * XK_RB bytes, its 16-byte chunk c at position swz<XK_RB>(r, c); rows past the
// segment hold zeros.
constexpr int XK_RB = 256;
constexpr int XK_TILE = BKV * XK_RB;

// Scores S^T = K Q^T of a wave's 32 queries against a staged key tile: qf[s] holds
// query l32's dh values s*16 + lg*8 + [0, 8); S[kb][r] is the score of key
// kb*32 + 8(r>>2) + 4lg + (r&3), -inf for keys >= n.
__device__ __forceinline__ void short_scores(const char* sk, const bf16x8 (&qf)[8], int n, int l32, int lg,
                                             f32x16 (&S)[2]) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) S[kb][r] = 0.f;
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const bf16x8 kf = __builtin_bit_cast(bf16x8, ld16(sk + (kb * 32 + l32) * XK_RB + swz<XK_RB>(l32, 2 * st + lg) * 16));
      S[kb] = mfma32(kf, qf[st], S[kb]);
    }
  }
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (kb * 32 + 8 * (r >> 2) + 4 * lg + (r & 3) >= n) S[kb][r] = -INFINITY;
}

// The exact softmax of short_scores' rows in place (exp2 domain: weight 2^(s scale - max)):
// S then holds the normalised probabilities, 0 for keys >= n.
__device__ __forceinline__ void short_probs(f32x16 (&S)[2], float scale) {
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[kb][r]);
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float ms = mx * scale;
  float l = 0.f;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      S[kb][r] = __builtin_amdgcn_exp2f(fmaf(S[kb][r], scale, -ms));
      l += S[kb][r];
    }
  const float lt = l + __shfl_xor(l, 32);
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) S[kb][r] *= inv;
}

}  // namespace dit
