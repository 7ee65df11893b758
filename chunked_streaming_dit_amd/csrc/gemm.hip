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
#include <algorithm>
#include <type_traits>

#include "attn_common.h"
#include "kernels.h"

namespace dit {

namespace {

constexpr int ROWB = 128 + 16;  // LDS bytes per staged row (128 data + 16 pad)
// Wave layout of gemm_lds_kernel (and patch_embed_kernel): 2 x 4 waves.
constexpr int LDS_WM = 2, LDS_WN = 4, LDS_THREADS = 64 * LDS_WM * LDS_WN;
// Rows from which bias / GELU launches take gemm_w4_kernel.
constexpr int W4_MIN_ROWS = 16384;

// Bias of a wave's NB x 32 columns, loaded into registers before the K loop so that its
// latency hides under it: lane columns n = nw + 32 j + 8 q + 4 lg + {0..3} in [j][q][0..3].
template <int NB, int EPI>
struct EpiCols {
  float b[NB][4][4];
};
template <class T, int NB, int EPI>
__device__ __forceinline__ void epi_cols_load(EpiCols<NB, EPI>& c, int nw, int lg, int N, const GemmEpi& e) {
  const T* bias = reinterpret_cast<const T*>(e.bias);
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int n = nw + j * 32 + 8 * q + 4 * lg;
#pragma unroll
      for (int r = 0; r < 4; ++r) c.b[j][q][r] = 0.f;
      if (n < N && bias) load4<T>(bias + n, c.b[j][q]);
    }
}

// Epilogue over a wave's (MB x 32) x (NB x 32) accumulator tile whose first row/column
// are mw, nw: lane holds output row m = mw + 32 i + l32 and columns
// n = nw + 32 j + 8 q + 4 lg + {0..3} in acc[i][j][4q .. 4q+3].  The residual gate is
// read before any store, and per 32-row block the values read back from the destination
// (residual h, latent x) are all requested before any store of that block, so their
// latencies overlap instead of adding up.
template <class T, int MB, int NB, int EPI>
__device__ __forceinline__ void epilogue(const f32x16 (&acc)[MB][NB], const EpiCols<NB, EPI>& c, int mw,
                                         int nw, int l32, int lg, int M, int N, const GemmEpi& e) {
  float gate[EPI == EPI_RESID ? NB : 1][4][4];
  if constexpr (EPI == EPI_RESID) {
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = nw + j * 32 + 8 * q + 4 * lg;
#pragma unroll
        for (int r = 0; r < 4; ++r) gate[j][q][r] = 1.f;
        if (e.gate && n < N) load4<float>(e.gate + n, gate[j][q]);
      }
  }
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int m = mw + i * 32 + l32;
    if (m >= M) continue;
    float* dst32 = reinterpret_cast<float*>(e.out) + (size_t)m * e.ldo;
    float old[EPI == EPI_RESID || EPI == EPI_EULER ? NB : 1][4][4];
    if constexpr (EPI == EPI_RESID || EPI == EPI_EULER) {
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = nw + j * 32 + 8 * q + 4 * lg;
          if (n < N) load4<float>(dst32 + n, old[j][q]);
        }
    }
#pragma unroll
    for (int j = 0; j < NB; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = nw + j * 32 + 8 * q + 4 * lg;
        if (n >= N) continue;
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = acc[i][j][4 * q + r] + c.b[j][q][r];
        if constexpr (EPI == EPI_BIAS) {
          store4<T>(reinterpret_cast<T*>(e.out) + (size_t)m * e.ldo + n, v);
        } else if constexpr (EPI == EPI_GELU) {
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = gelu_tanh(v[r]);
          store4<T>(reinterpret_cast<T*>(e.out) + (size_t)m * e.ldo + n, v);
        } else if constexpr (EPI == EPI_F32) {
          store4<float>(dst32 + n, v);
        } else if constexpr (EPI == EPI_RESID) {
          float h[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) h[r] = old[j][q][r] + gate[j][q][r] * v[r];
          store4<float>(dst32 + n, h);
        } else {  // EPI_EULER
          float x[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) x[r] = fmaf(e.dt, v[r], old[j][q][r]);
          store4<float>(dst32 + n, x);
          if (e.v_out) store4<float>(e.v_out + (size_t)m * e.ldo + n, v);
        }
      }
    }
  }
}

// EPI_QKNORM epilogue of gemm_lds_kernel (bf16, heads of 128 columns).  The tile's 256
// columns lie in one part of [q | k | v].  v columns are stored as computed (C + b).
// For q and k, a head's 128 columns are split over two waves (wn even / odd), so each
// row's sum of squares is completed through LDS (free once the K loop has ended); then
// each value is normalised, scaled by its gamma (and q_scale for q), pairs (2i, 2i+1)
// are rotated by the 3D RoPE of the row's token (axis t for the first d_t/2 pairs, then
// y, then x; pair j of an axis with d_a dims turns at theta^(-2j/d_a)), and the head is
// written in bf16.  k rows in [M, kpad) are written as zeros.  The rotation uses the
// hardware sine and cosine (v_sin_f32 / v_cos_f32, argument in turns) on the angle
// reduced to half a turn; their error is far below the bf16 rounding that follows.
// EPI_QKNORM_X layout of the ring after the K loop: the row sums of squares at 0, the
// normalised q tile (bf16, rows of XQ_PITCH bytes: 16-byte pad) from XQ_OFF, the tile's
// two heads' key tiles after it.
constexpr int XQ_OFF = 4096, XQ_PITCH = 512 + 16;
template <int BM>
constexpr int xattn_smem() { return XQ_OFF + BM * XQ_PITCH + 2 * XK_TILE; }

template <int BM, int MB, int NB, bool XATT, class Cols>
__device__ __forceinline__ void epilogue_qknorm(const f32x16 (&acc)[MB][NB], const Cols& cols,
                                                char* smem, int wm, int wn, int mw, int nw, int l32, int lg,
                                                int M, const GemmEpi& e) {
  constexpr int DH = 128;
  static_assert(NB == 2, "one wave covers half a head (64 columns)");
  const int part = nw / e.D;
  if constexpr (XATT) {
    // the tile's two heads' key tiles (rows past xn are zero in the source)
    const int head0 = (nw - nw % 256) / DH, D = e.D;
    char* sk = smem + XQ_OFF + BM * XQ_PITCH;
#pragma unroll
    for (int i = 0; i < 2 * BKV * 16 / LDS_THREADS; ++i) {
      const int c = threadIdx.x + LDS_THREADS * i;
      const int hh = c / (BKV * 16), cc = c - hh * BKV * 16, rk = cc >> 4, ck = cc & 15;
      const char* src = reinterpret_cast<const char*>(e.xk) + ((size_t)rk * D + (head0 + hh) * DH) * 2 + ck * 16;
      st16(sk + hh * XK_TILE + rk * XK_RB + swz<XK_RB>(rk, ck) * 16, ld16(src));
    }
  }
  if (!XATT && part == 2 && !e.vt_out) {
    epilogue<bf16, MB, NB, EPI_BIAS>(acc, reinterpret_cast<const EpiCols<NB, EPI_BIAS>&>(cols), mw, nw, l32, lg,
                                     M, 3 * e.D, e);
    return;
  }
  if (!XATT && part == 2) {
    // V^T: the tile (BM tokens x 256 columns) goes transposed through LDS, then each
    // thread writes one column's 16-token group in the attention layout (token offset
    // o of the group at position 8((o%8)/4) + 4(o/8) + o%4); tokens in [M, kpad) as 0.
    constexpr int P = BM;  // LDS row pitch (tokens) of a column: 256 x BM x 2 bytes fit the ring
    bf16* st = reinterpret_cast<bf16*>(smem);
    const int tid = threadIdx.x;
    const int c0 = nw - (nw / 256) * 256;  // wave's first column within the tile
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            st[(c0 + j * 32 + 8 * q + 4 * lg + r) * P + (mw % BM) + i * 32 + l32] =
                (bf16)(acc[i][j][4 * q + r] + cols.b[j][q][r]);
    __syncthreads();
    const int m0 = mw - mw % BM, ncol0 = nw - c0 - 2 * e.D;  // tile's first token / V column
    constexpr int G = BM / 16;
    bf16* vt = reinterpret_cast<bf16*>(e.vt_out);
    // Two lanes per 16-token group of a column, each reading 8 tokens (16 bytes; a wave
    // reads 1 KB of consecutive LDS, free of bank conflicts).  The group's output order
    // puts tokens 0-3, 8-11 in its first 16 bytes and 4-7, 12-15 in its second, so the
    // lanes swap 8 bytes and each stores one half.
    for (int it = tid; it < 2 * 256 * G; it += (int)blockDim.x) {
      const int col = it / (2 * G), rem = it - col * 2 * G, grp = rem >> 1, h = rem & 1;
      const int tok0 = m0 + grp * 16;
      if (tok0 >= e.kpad) continue;  // the same for both lanes of a group
      u32x4 raw = ld16(st + col * P + grp * 16 + h * 8);
      if (tok0 + 16 > M) {  // tokens in [M, kpad) as 0
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int t = tok0 + h * 8 + 2 * w;
          if (t >= M) raw[w] = 0u;
          else if (t + 1 >= M) raw[w] &= 0xffffu;
        }
      }
      const uint32_t s0 = h ? raw[0] : raw[2], s1 = h ? raw[1] : raw[3];  // half 0 sends 4-7, half 1 sends 8-11
      const uint32_t r0 = __shfl_xor(s0, 1), r1 = __shfl_xor(s1, 1);
      u32x4 o;
      if (h) { o[0] = r0; o[1] = r1; o[2] = raw[2]; o[3] = raw[3]; }  // 4-7 | 12-15
      else { o[0] = raw[0]; o[1] = raw[1]; o[2] = r0; o[3] = r1; }   // 0-3 | 8-11
      *reinterpret_cast<u32x4*>(vt + (size_t)(ncol0 + col) * e.vcap + tok0 + h * 8) = o;
    }
    return;
  }
  const bool isq = part == 0;
  const int col0 = nw - part * e.D;  // column of the wave's first value within its part
  const int half = (col0 % DH) / 64;
  float v[MB][NB][4][4], rs[MB];
  float* red = reinterpret_cast<float*>(smem);  // [2 wm][4 wn][MB * 32] row partial sums
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          v[i][j][q][r] = acc[i][j][4 * q + r] + cols.b[j][q][r];
          ss += v[i][j][q][r] * v[i][j][q][r];
        }
    ss += __shfl_xor(ss, 32);
    rs[i] = ss;
    if (lg == 0) red[(wm * 4 + wn) * MB * 32 + i * 32 + l32] = ss;
  }
  __syncthreads();
  void* outp = isq ? e.q_out : e.k_out;
  if (!XATT && !outp) return;  // q not needed (last block of a context pass)
  bf16* out = reinterpret_cast<bf16*>(outp);
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const float tot = rs[i] + red[(wm * 4 + (wn ^ 1)) * MB * 32 + i * 32 + l32];
    rs[i] = 1.0f / sqrtf(tot / (float)DH + e.eps);
  }
  // gamma (x q_scale for q) and rotation frequency of the lane's columns
  const bf16* gam = reinterpret_cast<const bf16*>(isq ? e.gq : e.gk);
  const float gs = isq ? e.q_scale : 1.0f;
  constexpr int D_HW = 2 * (DH / 6), D_T = DH - 2 * D_HW;
  float gm[NB][4][4], inv_freq[NB][4][2];
  int axis[NB][4][2];
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = half * 64 + j * 32 + 8 * q + 4 * lg;  // column within the head
      load4<bf16>(gam + c, gm[j][q]);
#pragma unroll
      for (int r = 0; r < 4; ++r) gm[j][q][r] *= gs;
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int pair = c / 2 + h2;
        int jj, da;
        if (pair < D_T / 2) { axis[j][q][h2] = 0; jj = pair; da = D_T; }
        else if (pair < D_T / 2 + D_HW / 2) { axis[j][q][h2] = 1; jj = pair - D_T / 2; da = D_HW; }
        else { axis[j][q][h2] = 2; jj = pair - D_T / 2 - D_HW / 2; da = D_HW; }
        // turns (revolutions) per position step
        inv_freq[j][q][h2] = exp2f(-(2.0f * (float)jj / (float)da) * e.log2_theta) * 0.15915494309189535f;
      }
    }
  const int hw = e.g.h * e.g.w;
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int m = mw + i * 32 + l32;
    bf16* orow = XATT ? reinterpret_cast<bf16*>(smem + XQ_OFF + (m % BM) * XQ_PITCH) + (nw % 256)
                      : out + (size_t)m * e.D + col0;
    if (m >= M) {
      if (!isq && m < e.kpad) {
        const float z[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) store4<bf16>(orow + j * 32 + 8 * q + 4 * lg, z);
      }
      continue;
    }
    float pt = 0.f, py = 0.f, px = 0.f;
    if (e.rope) {
      const int f = m / hw, rem = m - f * hw;
      const int y = rem / e.g.w;
      pt = (float)(e.g.t0 + f);
      py = (float)y;
      px = (float)(rem - y * e.g.w);
    }
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float o[4];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const float y0 = v[i][j][q][2 * h2] * rs[i] * gm[j][q][2 * h2];
          const float y1 = v[i][j][q][2 * h2 + 1] * rs[i] * gm[j][q][2 * h2 + 1];
          float sn = 0.f, cs = 1.f;
          if (e.rope) {  // hardware sin / cos of the angle reduced to [-1/2, 1/2] turn
            const int ax = axis[j][q][h2];
            const float turns = (ax == 0 ? pt : (ax == 1 ? py : px)) * inv_freq[j][q][h2];
            const float fr = turns - rintf(turns);
            sn = __builtin_amdgcn_sinf(fr);
            cs = __builtin_amdgcn_cosf(fr);
          }
          o[2 * h2] = y0 * cs - y1 * sn;
          o[2 * h2 + 1] = y0 * sn + y1 * cs;
        }
        store4<bf16>(orow + j * 32 + 8 * q + 4 * lg, o);
      }
  }
  if constexpr (XATT) {
    // the short softmax of every (head, 32-row block) of the tile from the LDS copies
    __syncthreads();
    const int head0 = (nw - nw % 256) / DH, m0 = mw - mw % BM;
    const char* sk = smem + XQ_OFF + BM * XQ_PITCH;
    const int wave = threadIdx.x >> 6;
    for (int u = wave; u < 2 * (BM / 32); u += LDS_THREADS / 64) {
      const int hh = u / (BM / 32), rb = u - hh * (BM / 32);
      const char* qrow = smem + XQ_OFF + (rb * 32 + l32) * XQ_PITCH + hh * DH * 2;
      bf16x8 qf[8];
#pragma unroll
      for (int st = 0; st < 8; ++st) qf[st] = __builtin_bit_cast(bf16x8, ld16(qrow + st * 32 + lg * 16));
      f32x16 S[2];
      short_scores(sk + hh * XK_TILE, qf, e.xn, l32, lg, S);
      short_probs(S, 1.0f);
      const int m = m0 + rb * 32 + l32;
      if (m >= M) continue;
      bf16* pp = reinterpret_cast<bf16*>(e.p_out) + (size_t)m * e.ldp + (head0 + hh) * BKV;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = S[kb][4 * q + r];
          store4<bf16>(pp + kb * 32 + 8 * q + 4 * lg, v);
        }
    }
  }
}

// Tile order: XCD-contiguous ranges of a grouped order in which GM consecutive
// m-tiles share each W column block.
__device__ __forceinline__ void tile_of(int b, int num_m, int num_n, int& tm, int& tn) {
  constexpr int GM = 8;
  const int pid = xcd_remap(b, num_m * num_n);
  const int group = pid / (GM * num_n);
  const int first_m = group * GM;
  const int gsz = min(num_m - first_m, GM);
  const int in_group = pid - group * GM * num_n;
  tm = first_m + in_group % gsz;
  tn = in_group / gsz;
}


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

  const int num_m = (M + BM - 1) / BM, num_n = (N + BN - 1) / BN;
  int tm, tn;
  tile_of(blockIdx.x, num_m, num_n, tm, tn);
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

  EpiCols<NB, EPI> cols;
  epi_cols_load<T, NB, EPI>(cols, n0 + wn * WN, lg, N, e);
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

  epilogue<T, MB, NB, EPI>(acc, cols, m0 + wm * WM, n0 + wn * WN, l32, lg, M, N, e);
}

template <class T, int BM, int BN>
hipError_t launch_t(const void* A, int lda, const void* W, int ldw, int M, int N, int K,
                    const GemmEpi& e, hipStream_t s, const hipEvent_t* ev) {
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  dim3 grid(tiles), block(256);
  const T* a = reinterpret_cast<const T*>(A);
  const T* w = reinterpret_cast<const T*>(W);
#define GK(EP) launch_k(gemm_kernel<T, BM, BN, EP>, grid, block, s, ev, a, lda, w, ldw, M, N, K, e)
  switch (e.kind) {
    case EPI_BIAS: return GK(EPI_BIAS);
    case EPI_GELU: return GK(EPI_GELU);
    case EPI_RESID: return GK(EPI_RESID);
    case EPI_F32: return GK(EPI_F32);
    case EPI_EULER: return GK(EPI_EULER);
    default: return hipErrorInvalidValue;
  }
#undef GK
}


// bf16 GEMM for large tiles, 8 waves (2 x 4) per workgroup, 2 waves per SIMD.
// Global -> LDS moves use direct-to-LDS buffer loads (buffer_load_dwordx4 ... lds: each
// wave instruction fills 1 KB = 8 rows of 128 bytes) into a 2-stage ring of unpadded
// 128-byte rows.  A and W are addressed through buffer resources (base in scalar
// registers, 32-bit per-lane offsets, the K step as the scalar offset), which measured
// 1.5-2% faster than 64-bit per-lane addresses; the resource's range check also turns
// any stray offset into zeros instead of a fault.  One wave per SIMD issues them (see
// the loader set-up below).  The 16-byte chunk c of row r sits at chunk position
// c ^ ((r >> 1) & 7), so that an MFMA fragment read (consecutive rows, same chunk)
// spreads over all 64 LDS banks.  Loads for step k+1 are in flight while step k is
// multiplied; one barrier per 64-wide K step.  Rows past M or N re-read the last valid
// row (their outputs are never stored).  While one wave of a SIMD waits on LDS the
// other issues MFMAs.

template <int BM, int BN, int EPI>
__global__ __launch_bounds__(LDS_THREADS) void gemm_lds_kernel(const bf16* __restrict__ A, int lda,
                                                               const bf16* __restrict__ W, int ldw,
                                                               int M, int N, int K, GemmEpi e) {
  typedef bf16x8 V;
  constexpr int NW = LDS_WM * LDS_WN;
  constexpr int WM = BM / LDS_WM, WN = BN / LDS_WN;
  constexpr int MB = WM / 32, NB = WN / 32;
  constexpr int ROWS = BM + BN;
  constexpr int STAGE = ROWS * 128;
  static_assert(WM % 32 == 0 && WN % 32 == 0 && ROWS % (8 * NW) == 0 && BM % (8 * NW) == 0, "tile");
  constexpr int SMEM = EPI == EPI_QKNORM_X && xattn_smem<BM>() > 2 * STAGE ? xattn_smem<BM>() : 2 * STAGE;
  __shared__ __attribute__((aligned(1024))) char smem[SMEM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / LDS_WN, wn = wave % LDS_WN;
  const int l32 = lane & 31, lg = lane >> 5;
  const int num_m = (M + BM - 1) / BM, num_n = (N + BN - 1) / BN;
  // EPI_PARTIAL: workgroup b takes K part b / tiles of tile b % tiles
  const int tiles = num_m * num_n;
  const int part = EPI == EPI_PARTIAL ? (int)blockIdx.x / tiles : 0;
  int tm, tn;
  tile_of((int)blockIdx.x - part * tiles, num_m, num_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  // Loaders: only waves 0-3, one per SIMD, move the tiles.  A wave that cannot issue
  // its next transfer (the CU's address unit busy with the others) stalls, and with
  // every wave loading, both waves of a SIMD stalled together and left its MFMA pipe
  // idle; with one loader per SIMD its partner keeps issuing MFMAs meanwhile (2-5%
  // faster on every block Linear shape, interleaved A/B on one board).
  // Instruction j of loader wave lw fills tile rows 8 (NLW j + lw) + [0, 8); the lane
  // covers row r = 8 (NLW j + lw) + lane/8 at chunk position lane & 7, i.e. source
  // chunk (lane & 7) ^ ((r >> 1) & 7).  Byte offsets from the matrix base are 32-bit
  // (matrices here are < 2 GB).
  constexpr int NLW = 4, NLDW = ROWS / (8 * NLW);  // loader waves, transfers per loader
  static_assert(ROWS % (8 * NLW) == 0 && BM % (8 * NLW) == 0, "loaders");
  const int lsub = lane >> 3, lw = wave % NLW;
  unsigned off[NLDW];
#pragma unroll
  for (int j = 0; j < NLDW; ++j) {
    const int r = 8 * (NLW * j + lw) + lsub;
    const int chunk = (lane & 7) ^ ((r >> 1) & 7);
    if (8 * NLW * j < BM)
      off[j] = (unsigned)(min(m0 + r, M - 1) * lda + chunk * 8) * 2u;
    else
      off[j] = (unsigned)(min(n0 + r - BM, N - 1) * ldw + chunk * 8) * 2u;
  }
  // Raw buffer resources over A and W (stride 0, size in bytes; the third word 0x00020000
  // is the gfx9-family format field for untyped dword accesses).
  const unsigned bytes_a = (unsigned)min((size_t)0xffffffffu, (size_t)M * lda * 2);
  const unsigned bytes_w = (unsigned)min((size_t)0xffffffffu, (size_t)N * ldw * 2);
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void*)A, (short)0, (int)bytes_a, 0x00020000);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc((void*)W, (short)0, (int)bytes_w, 0x00020000);
  auto issue = [&](int stage, int k0) {
    if (wave >= NLW) return;  // wave-uniform
    char* dst = smem + stage * STAGE + lw * 8 * 128;
#pragma unroll
    for (int j = 0; j < NLDW; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(8 * NLW * j < BM ? ra : rw,
                                               (__attribute__((address_space(3))) void*)(dst + j * NLW * 8 * 128), 16,
                                               (int)off[j], k0 * 2, 0, 0);
  };

  // EPI_PARTIAL stores the raw product of its K part as an fp32 tile of ws
  GemmEpi ep = e;
  if constexpr (EPI == EPI_PARTIAL) {
    ep.kind = EPI_F32;
    ep.bias = nullptr;
    ep.out = e.ws + (size_t)part * M * N;
    ep.ldo = N;
  }
  EpiCols<NB, EPI> cols;
  epi_cols_load<bf16, NB, EPI>(cols, n0 + wn * WN, lg, N, ep);
  f32x16 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // Fragment rows: all offsets are multiples of 32 rows, so the swizzle term of every
  // fragment this lane reads is the same: x = (l32 >> 1) & 7.
  const int x = (l32 >> 1) & 7;
  const int a_base = (wm * WM + l32) * 128;
  const int w_base = (BM + wn * WN + l32) * 128;

  // 64-wide K steps [it0, it1): all of them, or this workgroup's part of them
  const int nk = K / 64;
  const int it0 = EPI == EPI_PARTIAL ? (int)((long long)nk * part / e.ksplit) : 0;
  const int it1 = EPI == EPI_PARTIAL ? (int)((long long)nk * (part + 1) / e.ksplit) : nk;
  issue(0, it0 * 64);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int it = it0; it < it1; ++it) {
    const int buf = (it - it0) & 1;
    if (it + 1 < it1) issue(buf ^ 1, (it + 1) * 64);
    const char* st = smem + buf * STAGE;
    // Fragments of sub-step s+1 are requested before sub-step s multiplies and the
    // scheduler is asked to interleave them one per MFMA, so LDS latency hides under
    // the MFMAs of the same wave as well as under the other wave of the SIMD.
    V af[2][MB], wf[2][NB];
    auto frags = [&](int s, int set) {
      const int coff = ((2 * s + lg) ^ x) << 4;
#pragma unroll
      for (int i = 0; i < MB; ++i) af[set][i] = as_vec<V>(ld16(st + a_base + i * 32 * 128 + coff));
#pragma unroll
      for (int j = 0; j < NB; ++j) wf[set][j] = as_vec<V>(ld16(st + w_base + j * 32 * 128 + coff));
    };
    frags(0, 0);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s < 3) frags(s + 1, (s + 1) & 1);
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = mfma32(wf[s & 1][j], af[s & 1][i], acc[i][j]);
      if (s < 3) {
#pragma unroll
        for (int q = 0; q < MB + NB; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, MB * NB - (MB + NB), 0);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  if constexpr (EPI == EPI_QKNORM || EPI == EPI_QKNORM_X)
    epilogue_qknorm<BM, MB, NB, EPI == EPI_QKNORM_X>(acc, cols, smem, wm, wn, m0 + wm * WM, n0 + wn * WN, l32, lg,
                                                     M, e);
  else if constexpr (EPI == EPI_PARTIAL)
    epilogue<bf16, MB, NB, EPI_F32>(acc, reinterpret_cast<const EpiCols<NB, EPI_F32>&>(cols), m0 + wm * WM,
                                    n0 + wn * WN, l32, lg, M, N, ep);
  else
    epilogue<bf16, MB, NB, EPI>(acc, cols, m0 + wm * WM, n0 + wn * WN, l32, lg, M, N, e);
}

// Bias columns of a 256-column tile: every column exists, so the loads carry no per-lane
// condition and all of them are requested before the first wait.
template <int NB, int EPI>
__device__ __forceinline__ void cols_load_all(EpiCols<NB, EPI>& c, int nw, int lg, const GemmEpi& e) {
  const bf16* bias = reinterpret_cast<const bf16*>(e.bias);
  if (bias) {
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) load4<bf16>(bias + nw + j * 32 + 8 * q + 4 * lg, c.b[j][q]);
  } else {
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int r = 0; r < 4; ++r) c.b[j][q][r] = 0.f;
  }
}

// bf16 GEMM with a bias or bias + GELU epilogue for long launches (many 256 x 256
// tiles): 4 waves, one per SIMD, each with a 128 x 128 wave tile whose 256 accumulator
// registers live in the AGPRs.  Against gemm_lds_kernel's 8 waves of 128 x 64 it reads a
// third less LDS per MFMA.  K steps of 64 through two LDS stage buffers (separate arrays,
// so that the compiler knows the transfers into one never alias the fragment reads from
// the other and may interleave them); every wave moves a quarter of each stage with
// direct-to-LDS buffer loads (1 KB per instruction, the same row layout and swizzle as
// gemm_lds_kernel).  The fragments of all four 16-wide sub-steps of a stage are held in
// registers; the one barrier per K step sits after the second sub-step, when this
// stage's fragments are all read (so the next stage can be requested into its buffer)
// and the next stage has landed (so its first two sub-steps can be read under the last
// two sub-steps' MFMAs).  The next stage's transfers are spread at one per two MFMAs.
// Same arithmetic and summation order as gemm_lds_kernel: the results are bit for bit
// the same.
template <int EPI>
__global__ __launch_bounds__(256, 1) void gemm_w4_kernel(const bf16* __restrict__ A, int lda,
                                                       const bf16* __restrict__ W, int ldw,
                                                       int M, int N, int K, GemmEpi e) {
  typedef bf16x8 V;
  constexpr int BM = 256, BN = 256, MB = 4, NB = 4;
  constexpr int STAGE = (BM + BN) * 128;
  __shared__ __attribute__((aligned(1024))) char smem0[STAGE];
  __shared__ __attribute__((aligned(1024))) char smem1[STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, lg = lane >> 5;
  const int num_m = (M + BM - 1) / BM, num_n = N / BN;
  int tm, tn;
  tile_of((int)blockIdx.x, num_m, num_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  constexpr int NLD = 16;
  const int lsub = lane >> 3;
  unsigned off[NLD];
#pragma unroll
  for (int j = 0; j < NLD; ++j) {
    const int r = 8 * (4 * j + (tid >> 6)) + lsub;
    const int chunk = (lane & 7) ^ ((r >> 1) & 7);
    if (j < 8)
      off[j] = (unsigned)(min(m0 + r, M - 1) * lda + chunk * 8) * 2u;
    else
      off[j] = (unsigned)(min(n0 + r - BM, N - 1) * ldw + chunk * 8) * 2u;
  }
  const unsigned bytes_a = (unsigned)min((size_t)0xffffffffu, (size_t)M * lda * 2);
  const unsigned bytes_w = (unsigned)min((size_t)0xffffffffu, (size_t)N * ldw * 2);
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc((void*)A, (short)0, (int)bytes_a, 0x00020000);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc((void*)W, (short)0, (int)bytes_w, 0x00020000);
  auto issue = [&](char* sbuf, int k0, int j) __attribute__((always_inline)) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(j < 8 ? ra : rw,
                                             (__attribute__((address_space(3))) void*)(sbuf + (4 * j + wave) * 1024),
                                             16, (int)off[j], k0 * 2, 0, 0);
  };
  f32x16 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  const int x = (l32 >> 1) & 7;
  const int a_base = (wm * 128 + l32) * 128;
  const int w_base = (BM + wn * 128 + l32) * 128;
  V af[4][MB], wf[4][NB];
  auto frags = [&](const char* st, int s) __attribute__((always_inline)) {
    const int coff = ((2 * s + lg) ^ x) << 4;
#pragma unroll
    for (int i = 0; i < MB; ++i) af[s][i] = as_vec<V>(ld16(st + a_base + i * 32 * 128 + coff));
#pragma unroll
    for (int j = 0; j < NB; ++j) wf[s][j] = as_vec<V>(ld16(st + w_base + j * 32 * 128 + coff));
  };
  auto mfmas = [&](int s) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[i][j] = mfma32(wf[s][j], af[s][i], acc[i][j]);
  };
  const int nk = K / 64;
#pragma unroll
  for (int j = 0; j < NLD; ++j) issue(smem0, 0, j);
  if (nk > 1) {
#pragma unroll
    for (int j = 0; j < NLD; ++j) issue(smem1, 64, j);
    wait_vm_lds<NLD>();
  } else {
    wait_vm_lds<0>();
  }
  lds_barrier();
  frags(smem0, 0);
  frags(smem0, 1);
  auto step = [&](char* st, char* nst, int it, auto LOADS) __attribute__((always_inline)) {
    frags(st, 2);
    frags(st, 3);
    mfmas(0);
#pragma unroll
    for (int q = 0; q < 2 * (MB + NB); ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    mfmas(1);
    __builtin_amdgcn_sched_group_barrier(0x008, MB * NB, 0);
    __builtin_amdgcn_sched_barrier(0);
    wait_vm_lds<0>();
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
    frags(nst, 0);
    frags(nst, 1);
    if constexpr (decltype(LOADS)::value) {
#pragma unroll
      for (int j = 0; j < NLD; ++j) issue(st, (it + 2) * 64, j);
    }
    mfmas(2);
    mfmas(3);
    if constexpr (decltype(LOADS)::value) {
#pragma unroll
      for (int q = 0; q < (MB * NB) / 2; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
#pragma unroll
      for (int q = 0; q < (MB * NB) / 2; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 2 * (MB + NB); ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, MB * NB, 0);
    }
  };
  int it = 0;
  for (; it + 3 < nk; it += 2) {
    step(smem0, smem1, it, std::true_type{});
    step(smem1, smem0, it + 1, std::true_type{});
  }
  if (it + 2 < nk) { step(smem0, smem1, it, std::true_type{}); ++it; }
  char* st = (it & 1) ? smem1 : smem0;
  char* nst = (it & 1) ? smem0 : smem1;
  if (it + 1 < nk) { step(st, nst, it, std::false_type{}); ++it; char* t = st; st = nst; nst = t; }
  frags(st, 2);
  frags(st, 3);
  mfmas(0);
  mfmas(1);
  mfmas(2);
  mfmas(3);
  // Epilogue: bias (+ GELU) in registers, the bf16 tile staged row-major in the two stage
  // buffers (rows 0-127 in smem0, 128-255 in smem1; 512 bytes per row, the 16-byte chunk c
  // of row r at c ^ (r & 31)), then stored as whole rows, 16 bytes per lane (measured
  // +6-7% against each lane storing its 8-byte pieces of 32 rows).
  EpiCols<NB, EPI> cols;
  cols_load_all<NB, EPI>(cols, n0 + wn * 128, lg, e);
  __builtin_amdgcn_s_waitcnt(0xc07f);
  lds_barrier();
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int r = wm * 128 + i * 32 + l32;
    char* rowp = (wm ? smem1 : smem0) + (r & 127) * 512;
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = wn * 128 + j * 32 + 8 * q + 4 * lg;
        float v[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          v[t] = acc[i][j][4 * q + t] + cols.b[j][q][t];
          if constexpr (EPI == EPI_GELU) v[t] = gelu_tanh(v[t]);
        }
        store4<bf16>(reinterpret_cast<bf16*>(rowp + (((c >> 3) ^ (r & 31)) << 4) + (c & 7) * 2), v);
      }
  }
  __builtin_amdgcn_s_waitcnt(0xc07f);
  lds_barrier();
#pragma unroll 4
  for (int k = 0; k < 32; ++k) {
    const int r = wave * 64 + 2 * k + (lane >> 5), chunk = lane & 31;
    const int m = m0 + r;
    const u32x4 val = ld16((r < 128 ? smem0 : smem1) + (r & 127) * 512 + ((chunk ^ (r & 31)) << 4));
    if (m < M) st16(reinterpret_cast<bf16*>(e.out) + (size_t)m * e.ldo + n0 + chunk * 8, val);
  }
}


template <int EPI>
hipError_t launch_w4(const void* A, int lda, const void* W, int ldw, int M, int N, int K, const GemmEpi& e,
                     hipStream_t s, const hipEvent_t* ev) {
  const int tiles = ((M + 255) / 256) * (N / 256);
  return launch_k(gemm_w4_kernel<EPI>, dim3(tiles), dim3(256), s, ev, reinterpret_cast<const bf16*>(A), lda,
                  reinterpret_cast<const bf16*>(W), ldw, M, N, K, e);
}

// Split K: h[m, n] += gate[n] (sum_p ws[p, m, n] + b[n]) (gate NULL: 1), one thread per
// 4 consecutive columns.
template <class T>
__global__ __launch_bounds__(256) void splitk_resid_kernel(const float* __restrict__ ws, int parts, int M, int N,
                                                           const T* __restrict__ bias,
                                                           const float* __restrict__ gate,
                                                           float* __restrict__ h, int ldh) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long long)M * N / 4) return;
  const int m = (int)(i / (N / 4)), n = (int)(i - (long long)m * (N / 4)) * 4;
  float acc[4] = {0.f, 0.f, 0.f, 0.f}, v[4], b[4] = {0.f, 0.f, 0.f, 0.f}, g[4] = {1.f, 1.f, 1.f, 1.f}, hv[4];
  for (int p = 0; p < parts; ++p) {
    load4<float>(ws + ((size_t)p * M + m) * N + n, v);
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] += v[r];
  }
  if (bias) load4<T>(bias + n, b);
  if (gate) load4<float>(gate + n, g);
  load4<float>(h + (size_t)m * ldh + n, hv);
#pragma unroll
  for (int r = 0; r < 4; ++r) hv[r] += g[r] * (acc[r] + b[r]);
  store4<float>(h + (size_t)m * ldh + n, hv);
}

template <int BM, int BN>
hipError_t launch_lds(const void* A, int lda, const void* W, int ldw, int M, int N, int K,
                      const GemmEpi& e, hipStream_t s, const hipEvent_t* ev) {
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  dim3 grid(tiles), block(LDS_THREADS);
  const bf16* a = reinterpret_cast<const bf16*>(A);
  const bf16* w = reinterpret_cast<const bf16*>(W);
#define LK(EP) launch_k(gemm_lds_kernel<BM, BN, EP>, grid, block, s, ev, a, lda, w, ldw, M, N, K, e)
  switch (e.kind) {
    case EPI_BIAS: return LK(EPI_BIAS);
    case EPI_GELU: return LK(EPI_GELU);
    case EPI_RESID: return LK(EPI_RESID);
    case EPI_F32: return LK(EPI_F32);
    case EPI_EULER: return LK(EPI_EULER);
    case EPI_QKNORM: return LK(EPI_QKNORM);
    case EPI_QKNORM_X:
      if constexpr (BM <= 192) return LK(EPI_QKNORM_X);
      else return hipErrorInvalidValue;
    case EPI_PARTIAL:
      grid.x = tiles * e.ksplit;
      return LK(EPI_PARTIAL);
    default: return hipErrorInvalidValue;
  }
#undef LK
}

// EPI_RESID with the K range split into parts (see GemmEpi::ws): partial products of
// 128 x 256 tiles into ws, then the residual epilogue over their sum.
hipError_t gemm_resid_splitk(const void* A, int lda, const void* W, int ldw, int M, int N, int K, int parts,
                             const GemmEpi& e, hipStream_t s, const hipEvent_t* ev) {
  GemmEpi ep = e;
  ep.kind = EPI_PARTIAL;
  ep.ksplit = parts;
  const hipEvent_t ev0[2] = {ev ? ev[0] : nullptr, nullptr}, ev1[2] = {nullptr, ev ? ev[1] : nullptr};
  hipError_t err = launch_lds<128, 256>(A, lda, W, ldw, M, N, K, ep, s, ev0);
  if (err != hipSuccess) return err;
  const long long n4 = (long long)M * N / 4;
  return launch_k(splitk_resid_kernel<bf16>, dim3((unsigned)((n4 + 255) / 256)), dim3(256), s, ev1,
                  (const float*)e.ws, parts, M, N, reinterpret_cast<const bf16*>(e.bias), e.gate,
                  reinterpret_cast<float*>(e.out), e.ldo);
}


// Patch embed with the input assembly fused into the A-operand loads:
// out[n, N] (fp32) = [x || cond'] W^T + b, where cond' is zero (mode 0), cond per token
// (mode 1), or the nearest-2x upsample of a half-resolution cond (mode 2: token (f, y, x)
// channel 4c + 2dy + dx takes half-resolution token (f, y/2, x/2) channel 4c + 2(y%2) +
// (x%2)).  K = c_p + c_c is small (64 or 128), so the kernel is bound by its HBM
// traffic (x, cond, out); assembling the bf16 A tile from the fp32 sources in registers
// saves writing and re-reading the [n, K] input matrix.  Tile 128 x 256, 8 waves (2 x 4)
// as in gemm_lds_kernel, one 64-wide K stage at a time: the lanes convert 8 channels
// each into a 16-byte chunk written to the swizzled LDS row; W rows arrive by
// direct-to-LDS loads.  Rows past n repeat the last token (their outputs are not stored).
constexpr int PE_BM = 128, PE_BN = 256;

__global__ __launch_bounds__(LDS_THREADS) void patch_embed_kernel(
    const float* __restrict__ x, int n, int c_p, const float* __restrict__ cond, int c_c, int mode,
    RopeGrid g, const bf16* __restrict__ W, int N, GemmEpi e) {
  typedef bf16x8 V;
  constexpr int BM = PE_BM, BN = PE_BN;
  constexpr int NW = LDS_WM * LDS_WN;
  constexpr int WM = BM / LDS_WM, WN = BN / LDS_WN;
  constexpr int MB = WM / 32, NB = WN / 32;
  constexpr int NLW = BN / (8 * NW);        // W load instructions per wave per stage
  constexpr int ACH = BM * 8 / LDS_THREADS;  // A chunks (8 channels) per thread per stage
  __shared__ __attribute__((aligned(1024))) char smem[(BM + BN) * 128];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / LDS_WN, wn = wave % LDS_WN;
  const int l32 = lane & 31, lg = lane >> 5;
  const int K = c_p + c_c;
  const int num_m = (n + BM - 1) / BM, num_n = N / BN;
  int tm, tn;
  tile_of(blockIdx.x, num_m, num_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  // A chunk i of this thread: tile row r = c / 8, channels 8 (c % 8) of the stage; the
  // x half reads token xtok, the cond half token ctok (half-resolution in mode 2) at
  // channel offset cofs.
  int arow[ACH], xtok[ACH], ctok[ACH], cofs[ACH];
#pragma unroll
  for (int i = 0; i < ACH; ++i) {
    const int c = tid + LDS_THREADS * i;
    arow[i] = c >> 3;
    const int tok = min(m0 + arow[i], n - 1);
    xtok[i] = tok;
    ctok[i] = tok;
    cofs[i] = 0;
    if (mode == 2) {
      const int hw = g.h * g.w, f = tok / hw, rem = tok - f * hw;
      const int y = rem / g.w, xx = rem - y * g.w;
      ctok[i] = (f * (g.h / 2) + y / 2) * (g.w / 2) + xx / 2;
      cofs[i] = 2 * (y & 1) + (xx & 1);
    }
  }
  const int lsub = lane >> 3;
  unsigned woff[NLW];
#pragma unroll
  for (int j = 0; j < NLW; ++j) {
    const int r = 8 * (NW * j + wave) + lsub;
    const int chunk = (lane & 7) ^ ((r >> 1) & 7);
    woff[j] = (unsigned)(min(n0 + r, N - 1) * K + chunk * 8) * 2u;
  }

  EpiCols<NB, EPI_F32> cols;
  epi_cols_load<bf16, NB, EPI_F32>(cols, n0 + wn * WN, lg, N, e);
  f32x16 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int xs = (l32 >> 1) & 7;
  const int a_base = (wm * WM + l32) * 128;
  const int w_base = (BM + wn * WN + l32) * 128;
  const char* Wb = reinterpret_cast<const char*>(W);
  for (int k0 = 0; k0 < K; k0 += 64) {
    if (k0) __syncthreads();  // the previous stage's fragments have been read
    {
      char* dst = smem + BM * 128 + wave * 8 * 128;
#pragma unroll
      for (int j = 0; j < NLW; ++j)
        __builtin_amdgcn_global_load_lds((const void*)(Wb + (size_t)k0 * 2 + woff[j]),
                                         (void*)(dst + j * NW * 8 * 128), 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      const int cc = (tid + LDS_THREADS * i) & 7;
      const int ch = k0 + 8 * cc;  // first of the 8 channels (c_p, c_c are multiples of 8)
      f32x4 v0 = {0.f, 0.f, 0.f, 0.f}, v1 = v0;
      if (ch < c_p) {
        const float* p = x + (size_t)xtok[i] * c_p + ch;
        v0 = *reinterpret_cast<const f32x4*>(p);
        v1 = *reinterpret_cast<const f32x4*>(p + 4);
      } else if (mode == 1) {
        const float* p = cond + (size_t)ctok[i] * c_c + (ch - c_p);
        v0 = *reinterpret_cast<const f32x4*>(p);
        v1 = *reinterpret_cast<const f32x4*>(p + 4);
      } else if (mode == 2) {
        const float* p = cond + (size_t)ctok[i] * c_c + (ch - c_p) + cofs[i];
        const float a = p[0], b = p[4];
        v0 = f32x4{a, a, a, a};
        v1 = f32x4{b, b, b, b};
      }
      V h;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        h[q] = (bf16)v0[q];
        h[4 + q] = (bf16)v1[q];
      }
      const int r = arow[i];
      st16(smem + r * 128 + ((cc ^ ((r >> 1) & 7)) << 4), __builtin_bit_cast(u32x4, h));
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int coff = ((2 * s + lg) ^ xs) << 4;
      V af[MB], wf[NB];
#pragma unroll
      for (int i = 0; i < MB; ++i) af[i] = as_vec<V>(ld16(smem + a_base + i * 32 * 128 + coff));
#pragma unroll
      for (int j = 0; j < NB; ++j) wf[j] = as_vec<V>(ld16(smem + w_base + j * 32 * 128 + coff));
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = mfma32(wf[j], af[i], acc[i][j]);
    }
  }
  epilogue<bf16, MB, NB, EPI_F32>(acc, cols, m0 + wm * WM, n0 + wn * WN, l32, lg, n, N, e);
}

// Final layer with its pre-norm and the Euler update in one pass: for 32 tokens per
// workgroup, u = RMSNorm(h) (1 + scale) + shift is formed in registers from the fp32
// rows of h and kept in LDS as bf16 (the operand the unfused GEMM would read), then
// v = u W^T + b (N = 64 outputs) with the K range split over the 4 waves and the
// partial products summed through LDS; x += dt v and v_out = v.  h is read once and u
// never leaves the CU, against a norm pass writing u and a 122-workgroup GEMM reading it.
constexpr int FL_BM = 32, FL_N = 64, FL_THREADS = 256;

template <int IT>
__global__ __launch_bounds__(FL_THREADS) void final_layer_kernel(const float* __restrict__ h, int n,
                                                               const float* __restrict__ shift,
                                                               const float* __restrict__ scale, float eps,
                                                               const bf16* __restrict__ W,
                                                               const bf16* __restrict__ b, float dt,
                                                               float* __restrict__ x, float* __restrict__ v_out) {
  typedef bf16x8 V;
  constexpr int D = 256 * IT;
  constexpr int PITCH = D * 2 + 16;  // bytes per u row: 16-byte pad spreads a fragment read over the banks
  __shared__ __attribute__((aligned(16))) char su[FL_BM * PITCH];
  __shared__ float red[4][2][16][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, lg = lane >> 5;
  const int row0 = blockIdx.x * FL_BM;

  // u rows: wave w forms rows 8w .. 8w + 7 of the tile (rows past n repeat row n - 1)
  f32x4 sc[IT], sh[IT];
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    sc[i] = *reinterpret_cast<const f32x4*>(scale + i * 256 + lane * 4);
    sh[i] = *reinterpret_cast<const f32x4*>(shift + i * 256 + lane * 4);
  }
  for (int rr = 0; rr < FL_BM / 4; ++rr) {
    const int r = wave * (FL_BM / 4) + rr;
    const float* hr = h + (size_t)min(row0 + r, n - 1) * D + lane * 4;
    f32x4 v[IT];
#pragma unroll
    for (int i = 0; i < IT; ++i) v[i] = *reinterpret_cast<const f32x4*>(hr + i * 256);
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < IT; ++i) ss += v[i][0] * v[i][0] + v[i][1] * v[i][1] + v[i][2] * v[i][2] + v[i][3] * v[i][3];
    ss = wave_sum(ss);
    const float rs = 1.0f / sqrtf(ss / (float)D + eps);
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      float o[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] = fmaf(v[i][q] * rs, 1.0f + sc[i][q], sh[i][q]);
      store4<bf16>(reinterpret_cast<bf16*>(su + r * PITCH) + i * 256 + lane * 4, o);
    }
  }
  __syncthreads();

  // v^T partial over this wave's quarter of K: first MFMA operand W rows (outputs),
  // second u rows, so the lane holds token row0 + l32 and 16 outputs per 32-block
  f32x16 acc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int t = 0; t < 16; ++t) acc[j][t] = 0.f;
  constexpr int KW = D / 4;
  const int k_begin = wave * KW;
#pragma unroll 4
  for (int k0 = k_begin; k0 < k_begin + KW; k0 += 16) {
    const V af = as_vec<V>(ld16(su + l32 * PITCH + (k0 + lg * 8) * 2));
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const V wf = as_vec<V>(ld16(W + (size_t)(j * 32 + l32) * D + k0 + lg * 8));
      acc[j] = mfma32(wf, af, acc[j]);
    }
  }
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int t = 0; t < 16; ++t) red[wave][j][t][lane] = acc[j][t];
  __syncthreads();

  // wave w completes registers 4w .. 4w + 3 of both blocks: outputs j*32 + 8w + 4lg + {0..3}
  const int m = row0 + l32;
  if (m >= n) return;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = j * 32 + 8 * wave + 4 * lg;
    float bb[4], v[4], xo[4];
    load4<bf16>(b + c, bb);
    load4<float>(x + (size_t)m * FL_N + c, xo);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int t = 4 * wave + q;
      v[q] = red[0][j][t][lane] + red[1][j][t][lane] + red[2][j][t][lane] + red[3][j][t][lane] + bb[q];
      xo[q] = fmaf(dt, v[q], xo[q]);
    }
    store4<float>(x + (size_t)m * FL_N + c, xo);
    if (v_out) store4<float>(v_out + (size_t)m * FL_N + c, v);
  }
}

}  // namespace

bool gemm_qknorm_fits(int dtype, int M, int N, int dh) {
  return dtype == BF16 && dh == 128 && M >= 256 && N % 256 == 0;
}

hipError_t gemm(int dtype, const void* A, int lda, const void* W, int ldw, int M, int N, int K,
                const GemmEpi& e, hipStream_t s, const hipEvent_t* ev) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (e.kind == EPI_QKNORM && (!gemm_qknorm_fits(dtype, M, N, 128) || e.D % 256 || (N != e.D && N != 3 * e.D)))
    return hipErrorInvalidValue;
  if (e.kind == EPI_QKNORM_X && (!gemm_qknorm_fits(dtype, M, N, 128) || e.D % 256 || N != e.D || e.rope || !e.xk ||
                                 !e.p_out || e.xn < 1 || e.xn > 64 || e.ldp < e.D / 2))
    return hipErrorInvalidValue;
  if (dtype == BF16) {
    if (M >= 256 && N >= 256 && N % 256 == 0) {
      // Pick the tile height that minimises (waves of 256 workgroups) x tile area,
      // i.e. the padded work of the last, partly filled wave; ties go to taller tiles.
      const int cand[3] = {256, 192, 128};
      int best = 256;
      long long best_cost = -1;
      for (int bm : cand) {
        const long long tiles = (long long)((M + bm - 1) / bm) * (N / 256);
        const long long cost = (tiles + 255) / 256 * (long long)bm;
        if (best_cost < 0 || cost < best_cost) { best_cost = cost; best = bm; }
      }
      // Too few tiles to occupy the chip (short context passes): a residual GEMM with a
      // long K (>= 4096) and a workspace splits its K range over 128 x 256 tiles, as many
      // parts (2-4) as fit one wave of workgroups; other launches take smaller tiles.
      // (With K = 1536 the merge pass costs more than the split saves.)
      const long long t128 = (long long)((M + 127) / 128) * (N / 256);
      if (e.kind == EPI_RESID && e.ws && t128 < 160 && K >= 4096 && K % 64 == 0) {
        int parts = (int)std::min<long long>(4, 256 / t128);
        while (parts > 1 && (long long)parts * M * N > e.ws_floats) --parts;
        if (parts > 1) return gemm_resid_splitk(A, lda, W, ldw, M, N, K, parts, e, s, ev);
      }
      if (e.kind != EPI_QKNORM && e.kind != EPI_QKNORM_X && ((M + best - 1) / best) * (N / 256) < 160) {
        if ((long long)((M + 127) / 128) * ((N + 127) / 128) >= 240) return launch_t<bf16, 128, 128>(A, lda, W, ldw, M, N, K, e, s, ev);
        return launch_t<bf16, 64, 64>(A, lda, W, ldw, M, N, K, e, s, ev);
      }
      // Long bias / bias + GELU launches (the large chunk's MLP in): the 4-wave kernel, whose
      // 256-row tiles and whole-row stores pay off once the grid is many waves deep (on the
      // base chunk's 7800 rows it measured the same or slower).
      if ((e.kind == EPI_BIAS || e.kind == EPI_GELU) && M >= W4_MIN_ROWS && K % 64 == 0) {
        if (e.kind == EPI_BIAS) return launch_w4<EPI_BIAS>(A, lda, W, ldw, M, N, K, e, s, ev);
        return launch_w4<EPI_GELU>(A, lda, W, ldw, M, N, K, e, s, ev);
      }
      if (best == 256 && e.kind == EPI_QKNORM_X) best = 192;  // its LDS holds a 192-row q tile at most
      if (best == 256) return launch_lds<256, 256>(A, lda, W, ldw, M, N, K, e, s, ev);
      if (best == 192) return launch_lds<192, 256>(A, lda, W, ldw, M, N, K, e, s, ev);
      return launch_lds<128, 256>(A, lda, W, ldw, M, N, K, e, s, ev);
    }
    if (M >= 512 && N >= 512) return launch_t<bf16, 128, 128>(A, lda, W, ldw, M, N, K, e, s, ev);
    return launch_t<bf16, 64, 64>(A, lda, W, ldw, M, N, K, e, s, ev);
  }
  return launch_t<float, 64, 64>(A, lda, W, ldw, M, N, K, e, s, ev);
}

bool patch_embed_fits(int dtype, int c_p, int c_c, int N) {
  return dtype == BF16 && (c_p + c_c) % 64 == 0 && c_p % 8 == 0 && c_c % 8 == 0 && N % PE_BN == 0;
}

hipError_t patch_embed(const float* x, int n, int c_p, const float* cond, int c_c, int cond_mode,
                       RopeGrid g, const void* W, const void* bias, float* out, int N, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (!patch_embed_fits(BF16, c_p, c_c, N) || cond_mode < 0 || cond_mode > 2 ||
      (cond_mode && !cond) || (cond_mode == 2 && (g.h % 2 || g.w % 2 || (long long)g.frames * g.h * g.w != n)))
    return hipErrorInvalidValue;
  GemmEpi e{};
  e.kind = EPI_F32;
  e.bias = bias;
  e.out = out;
  e.ldo = N;
  const int tiles = ((n + PE_BM - 1) / PE_BM) * (N / PE_BN);
  patch_embed_kernel<<<tiles, LDS_THREADS, 0, s>>>(x, n, c_p, cond, c_c, cond_mode, g,
                                                   reinterpret_cast<const bf16*>(W), N, e);
  return hipGetLastError();
}

bool final_layer_fits(int dtype, int D, int c_p) {
  return dtype == BF16 && c_p == FL_N && (D == 1536 || D == 1024 || D == 512 || D == 256);
}

hipError_t final_layer(const float* h, int n, int D, const float* shift, const float* scale, float eps,
                       const void* W, const void* b, float dt, float* x, float* v_out, hipStream_t s,
                       const hipEvent_t* ev) {
  if (n <= 0) return hipSuccess;
  dim3 grid((n + FL_BM - 1) / FL_BM), block(FL_THREADS);
  const bf16* w = reinterpret_cast<const bf16*>(W);
  const bf16* bb = reinterpret_cast<const bf16*>(b);
#define FK(KD) launch_k(final_layer_kernel<KD>, grid, block, s, ev, h, n, shift, scale, eps, w, bb, dt, x, v_out)
  switch (D) {
    case 256: return FK(1);
    case 512: return FK(2);
    case 1024: return FK(4);
    case 1536: return FK(6);
    default: return hipErrorInvalidValue;
  }
#undef FK
}

}  // namespace dit
