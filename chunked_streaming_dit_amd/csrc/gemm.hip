// MFMA GEMM with fused epilogues: C = A W^T (+ bias) -> {store, GELU, gated residual,
// fp32 store, Euler update}.  A [M, K] and W [N, K] are both K-contiguous (W is a
// Linear weight stored [out, in]), fp32 accumulation.
//
// Work decomposition (gfx950, wave64):
//   - one workgroup of 256 threads (4 waves as 2 x 2) owns a BM x BN output tile;
//   - each K step stages a BM x 128-byte slice of A and a BN x 128-byte slice of W in
//     LDS (rows padded by 16 bytes so that the 16-byte fragment reads of 8
//     consecutive rows hit distinct banks), double-buffered with one barrier per step;
//     the next slice is fetched into registers while the current one is multiplied;
//   - each wave multiplies a (BM/2) x (BN/2) sub-tile with 32x32 MFMAs whose first
//     operand is W rows and second operand A rows, so each lane ends up holding 4
//     consecutive output columns of one output row: the epilogue reads bias, gate and
//     the fp32 residual as 16-byte vectors.
#include "common.h"
#include "kernels.h"

namespace dit {

namespace {

constexpr int ROWB = 128 + 16;  // LDS bytes per staged row (128 data + 16 pad)

template <class T, int BM, int BN, int EPI>
__global__ __launch_bounds__(256) void gemm_kernel(const T* __restrict__ A, int lda,
                                                   const T* __restrict__ W, int ldw, int M, int N,
                                                   int K, GemmEpi e) {
  typedef typename Vec<T>::type V;
  constexpr int VE = Vec<T>::n;
  constexpr int BK = 128 / (int)sizeof(T);
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int MB = WM / 32, NB = WN / 32;
  constexpr int CPT = (BM + BN) * 8 / 256;  // 16-byte chunks per thread per stage
  static_assert((BM + BN) * 8 % 256 == 0, "tile");
  __shared__ __attribute__((aligned(16))) char smem[2][(BM + BN) * ROWB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, lg = lane >> 5;

  // Grouped tile order: GM consecutive m-tiles share each W column block.
  const int num_m = (M + BM - 1) / BM, num_n = (N + BN - 1) / BN;
  constexpr int GM = 8;
  const int pid = blockIdx.x;
  const int group = pid / (GM * num_n);
  const int first_m = group * GM;
  const int gsz = min(num_m - first_m, GM);
  const int in_group = pid - group * GM * num_n;
  const int tm = first_m + in_group % gsz;
  const int tn = in_group / gsz;
  const int m0 = tm * BM, n0 = tn * BN;

  u32x4 stage[CPT];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + 256 * i;
      const int r = c >> 3, cc = c & 7;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (r < BM) {
        const int gm = m0 + r;
        if (gm < M) v = ld16(A + (size_t)gm * lda + k0 + cc * VE);
      } else {
        const int gn = n0 + r - BM;
        if (gn < N) v = ld16(W + (size_t)gn * ldw + k0 + cc * VE);
      }
      stage[i] = v;
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int c = tid + 256 * i;
      const int r = c >> 3, cc = c & 7;
      st16(&smem[buf][r * ROWB + cc * 16], stage[i]);
    }
  };

  f32x16 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = K / BK;
  gload(0);
  sstore(0);
  for (int it = 0; it < nk; ++it) {
    const int buf = it & 1;
    if (it + 1 < nk) gload((it + 1) * BK);
    __syncthreads();
    const char* sA = &smem[buf][0];
    const char* sW = &smem[buf][BM * ROWB];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      V af[MB], wf[NB];
#pragma unroll
      for (int i = 0; i < MB; ++i)
        af[i] = as_vec<V>(ld16(sA + (wm * WM + i * 32 + l32) * ROWB + s * 32 + lg * 16));
#pragma unroll
      for (int j = 0; j < NB; ++j)
        wf[j] = as_vec<V>(ld16(sW + (wn * WN + j * 32 + l32) * ROWB + s * 32 + lg * 16));
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = mfma32(wf[j], af[i], acc[i][j]);
    }
    if (it + 1 < nk) sstore(buf ^ 1);
  }

  // Epilogue: lane holds output row m = .. + l32, columns n = .. + 8q + 4lg + {0..3}.
  const T* bias = reinterpret_cast<const T*>(e.bias);
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int m = m0 + wm * WM + i * 32 + l32;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + wn * WN + j * 32 + 8 * q + 4 * lg;
        if (n >= N) continue;
        float v[4], b[4];
        load4<T>(bias + n, b);
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = acc[i][j][4 * q + r] + b[r];
        if constexpr (EPI == EPI_BIAS) {
          store4<T>(reinterpret_cast<T*>(e.out) + (size_t)m * e.ldo + n, v);
        } else if constexpr (EPI == EPI_GELU) {
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = gelu_tanh(v[r]);
          store4<T>(reinterpret_cast<T*>(e.out) + (size_t)m * e.ldo + n, v);
        } else if constexpr (EPI == EPI_F32) {
          store4<float>(reinterpret_cast<float*>(e.out) + (size_t)m * e.ldo + n, v);
        } else if constexpr (EPI == EPI_RESID) {
          float* hp = reinterpret_cast<float*>(e.out) + (size_t)m * e.ldo + n;
          float h[4], g[4] = {1.f, 1.f, 1.f, 1.f};
          load4<float>(hp, h);
          if (e.gate) load4<float>(e.gate + n, g);
#pragma unroll
          for (int r = 0; r < 4; ++r) h[r] += g[r] * v[r];
          store4<float>(hp, h);
        } else {  // EPI_EULER
          float* xp = reinterpret_cast<float*>(e.out) + (size_t)m * e.ldo + n;
          float x[4];
          load4<float>(xp, x);
#pragma unroll
          for (int r = 0; r < 4; ++r) x[r] = fmaf(e.dt, v[r], x[r]);
          store4<float>(xp, x);
          if (e.v_out) store4<float>(e.v_out + (size_t)m * e.ldo + n, v);
        }
      }
    }
  }
}

template <class T, int BM, int BN>
hipError_t launch_t(const void* A, int lda, const void* W, int ldw, int M, int N, int K,
                    const GemmEpi& e, hipStream_t s) {
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  dim3 grid(tiles), block(256);
  const T* a = reinterpret_cast<const T*>(A);
  const T* w = reinterpret_cast<const T*>(W);
  switch (e.kind) {
    case EPI_BIAS: gemm_kernel<T, BM, BN, EPI_BIAS><<<grid, block, 0, s>>>(a, lda, w, ldw, M, N, K, e); break;
    case EPI_GELU: gemm_kernel<T, BM, BN, EPI_GELU><<<grid, block, 0, s>>>(a, lda, w, ldw, M, N, K, e); break;
    case EPI_RESID: gemm_kernel<T, BM, BN, EPI_RESID><<<grid, block, 0, s>>>(a, lda, w, ldw, M, N, K, e); break;
    case EPI_F32: gemm_kernel<T, BM, BN, EPI_F32><<<grid, block, 0, s>>>(a, lda, w, ldw, M, N, K, e); break;
    case EPI_EULER: gemm_kernel<T, BM, BN, EPI_EULER><<<grid, block, 0, s>>>(a, lda, w, ldw, M, N, K, e); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t gemm(int dtype, const void* A, int lda, const void* W, int ldw, int M, int N, int K,
                const GemmEpi& e, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (dtype == BF16) {
    if (M >= 512 && N >= 512) return launch_t<bf16, 128, 128>(A, lda, W, ldw, M, N, K, e, s);
    return launch_t<bf16, 64, 64>(A, lda, W, ldw, M, N, K, e, s);
  }
  return launch_t<float, 64, 64>(A, lda, W, ldw, M, N, K, e, s);
}

}  // namespace dit
