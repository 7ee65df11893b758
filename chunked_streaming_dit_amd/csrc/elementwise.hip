// Bandwidth-bound kernels: RMSNorm + adaLN modulate, per-head QK-norm + 3D RoPE with
// K/V repacking into the attention layout, patch-embed input assembly (with the
// nearest-2x conditioning upsample), the Euler update, and the timestep-conditioning
// / modulation GEMVs.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace dit {

namespace {

// ---------------------------------------------------------------- RMSNorm + modulate
// One wave per row; each lane holds D/256 float4 groups in registers (D <= 4096).
template <class T>
__global__ __launch_bounds__(256) void rmsnorm_mod_kernel(const float* __restrict__ h, int n,
                                                          int D, const float* __restrict__ shift,
                                                          const float* __restrict__ scale,
                                                          float eps, T* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= n) return;
  const float* hr = h + (size_t)row * D;
  const int iters = D >> 8;
  f32x4 v[16];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (i < iters) {
      v[i] = *reinterpret_cast<const f32x4*>(hr + i * 256 + lane * 4);
      ss += v[i][0] * v[i][0] + v[i][1] * v[i][1] + v[i][2] * v[i][2] + v[i][3] * v[i][3];
    }
  }
  ss = wave_sum(ss);
  const float rs = 1.0f / sqrtf(ss / (float)D + eps);
  T* orow = out + (size_t)row * D;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (i < iters) {
      const int c = i * 256 + lane * 4;
      float o[4];
      if (scale) {
        f32x4 sc = *reinterpret_cast<const f32x4*>(scale + c);
        f32x4 sh = *reinterpret_cast<const f32x4*>(shift + c);
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = fmaf(v[i][r] * rs, 1.0f + sc[r], sh[r]);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = v[i][r] * rs;
      }
      store4<T>(orow + c, o);
    }
  }
}

// Fixed width D = 256 IT, two rows per wave: both rows' loads are in flight together and
// the modulation vectors are read once per two rows.
template <class T, int IT>
__global__ __launch_bounds__(256) void rmsnorm_mod2_kernel(const float* __restrict__ h, int n,
                                                           const float* __restrict__ shift,
                                                           const float* __restrict__ scale,
                                                           float eps, T* __restrict__ out) {
  constexpr int D = 256 * IT;
  const int lane = threadIdx.x & 63;
  const int row0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * 2;
  if (row0 >= n) return;
  const bool two = row0 + 1 < n;
  f32x4 v[2][IT];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const float* hr = h + (size_t)(two ? row0 + r : row0) * D + lane * 4;
#pragma unroll
    for (int i = 0; i < IT; ++i) v[r][i] = *reinterpret_cast<const f32x4*>(hr + i * 256);
  }
  float rs[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < IT; ++i)
      ss += v[r][i][0] * v[r][i][0] + v[r][i][1] * v[r][i][1] + v[r][i][2] * v[r][i][2] + v[r][i][3] * v[r][i][3];
    ss = wave_sum(ss);
    rs[r] = 1.0f / sqrtf(ss / (float)D + eps);
  }
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const int c = i * 256 + lane * 4;
    f32x4 sc = {0.f, 0.f, 0.f, 0.f}, sh = sc;
    if (scale) {
      sc = *reinterpret_cast<const f32x4*>(scale + c);
      sh = *reinterpret_cast<const f32x4*>(shift + c);
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      if (r == 1 && !two) break;
      float o[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] = fmaf(v[r][i][q] * rs[r], 1.0f + sc[q], sh[q]);
      store4<T>(out + (size_t)(row0 + r) * D + c, o);
    }
  }
}

// ---------------------------------------------------------------- QK-norm + RoPE + repack
// Grid: (round_up(n, 64) / 64, H).  A workgroup owns 64 tokens x one head.  A lane moves
// one 16-byte vector (VE elements, VE/2 rotation pairs) of a head row, so a row of dh
// elements is LPR = dh/VE lanes and a wave handles 64/LPR tokens at a time.  The row's
// sum of squares is reduced over its LPR lanes.  V rows are staged in LDS and written
// out transposed ([dh, cap] per head) in the attention kernel's key order.
template <class T, int DH>
__global__ __launch_bounds__(256) void qknorm_rope_kernel(
    int n, const T* __restrict__ q_in, const T* __restrict__ k_in, const T* __restrict__ v_in,
    int ld_in, const T* __restrict__ gq, const T* __restrict__ gk, int rope, RopeGrid g,
    float eps, float log2_theta, float q_scale, T* __restrict__ q_out, T* __restrict__ k_out,
    T* __restrict__ vt_out, int cap, int D) {
  typedef typename Vec<T>::type V;
  constexpr int VE = Vec<T>::n;
  constexpr int LPR = DH / VE;      // lanes per head row
  constexpr int TPW = 64 / LPR;     // tokens per wave step
  constexpr int NP = VE / 2;        // rotation pairs per lane
  __shared__ __attribute__((aligned(16))) T sv[64][DH + 8];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int head = blockIdx.y;
  const int tok0 = blockIdx.x * 64;
  const int c = lane % LPR;           // vector index within the row
  const int sub = lane / LPR;         // token within the wave step

  // Rotation frequency of each of this lane's pairs: axis t for the first d_t/2 pairs,
  // then y, then x; pair j of an axis with d_a dims turns at theta^(-2j/d_a).
  const int d_hw = 2 * (DH / 6);
  const int d_t = DH - 2 * d_hw;
  int axis[NP];
  float inv_freq[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int pair = c * NP + i;
    int j, d_a;
    if (pair < d_t / 2) { axis[i] = 0; j = pair; d_a = d_t; }
    else if (pair < d_t / 2 + d_hw / 2) { axis[i] = 1; j = pair - d_t / 2; d_a = d_hw; }
    else { axis[i] = 2; j = pair - d_t / 2 - d_hw / 2; d_a = d_hw; }
    inv_freq[i] = exp2f(-(2.0f * (float)j / (float)d_a) * log2_theta);
  }
  float gqv[VE], gkv[VE];
#pragma unroll
  for (int e = 0; e < VE; ++e) {
    gqv[e] = gq ? to_f(gq[c * VE + e]) * q_scale : 0.f;  // q_out carries q_scale
    gkv[e] = gk ? to_f(gk[c * VE + e]) : 0.f;
  }
  const int hw = g.h * g.w;

  // Normalise (per-head RMS over LPR lanes), scale by gamma and rotate one row vector.
  auto norm_rot = [&](V x, const float (&gam)[VE], const float (&cs)[NP], const float (&sn)[NP]) {
    float f[VE], ss = 0.f;
#pragma unroll
    for (int e = 0; e < VE; ++e) { f[e] = to_f(x[e]); ss += f[e] * f[e]; }
#pragma unroll
    for (int o = LPR / 2; o >= 1; o >>= 1) ss += __shfl_xor(ss, o);
    const float rs = 1.0f / sqrtf(ss / (float)DH + eps);
    V out;
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const float y0 = f[2 * i] * rs * gam[2 * i], y1 = f[2 * i + 1] * rs * gam[2 * i + 1];
      out[2 * i] = from_f<T>(y0 * cs[i] - y1 * sn[i]);
      out[2 * i + 1] = from_f<T>(y0 * sn[i] + y1 * cs[i]);
    }
    return out;
  };

  for (int it = wave * TPW + sub; it < 64; it += 4 * TPW) {
    const int tok = tok0 + it;
    const bool valid = tok < n;
    float cs[NP], sn[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) { cs[i] = 1.f; sn[i] = 0.f; }
    if (rope && valid) {
      const int f = tok / hw, rem = tok - f * hw;
      const int y = rem / g.w, x = rem - y * g.w;
      const int pv[3] = {g.t0 + f, y, x};
#pragma unroll
      for (int i = 0; i < NP; ++i) sincosf((float)pv[axis[i]] * inv_freq[i], &sn[i], &cs[i]);
    }
    const size_t src = (size_t)tok * ld_in + head * DH + c * VE;
    const size_t dst = (size_t)tok * D + head * DH + c * VE;
    V zero;
#pragma unroll
    for (int e = 0; e < VE; ++e) zero[e] = from_f<T>(0.f);
    if (q_in) {
      const V x = valid ? as_vec<V>(ld16(q_in + src)) : zero;
      const V y = norm_rot(x, gqv, cs, sn);
      if (valid) st16(q_out + dst, __builtin_bit_cast(u32x4, y));
    }
    if (k_in) {  // rows past n are written as zeros (x = 0 normalises to 0)
      const V x = valid ? as_vec<V>(ld16(k_in + src)) : zero;
      const V y = norm_rot(x, gkv, cs, sn);
      st16(k_out + dst, __builtin_bit_cast(u32x4, y));
    }
    if (v_in) {
      const V x = valid ? as_vec<V>(ld16(v_in + src)) : zero;
      *reinterpret_cast<V*>(&sv[it][c * VE]) = x;
    }
  }
  if (!v_in) return;
  __syncthreads();
  // V^T: row d of this head gets the 64 tokens of the tile, 16 bytes per thread-chunk.
  constexpr int CPR = 64 / VE;  // chunks per row
  for (int cc = tid; cc < DH * CPR; cc += 256) {
    const int d = cc / CPR, pos0 = (cc % CPR) * VE;
    V out;
#pragma unroll
    for (int e = 0; e < VE; ++e) {
      const int p = pos0 + e;
      int key = p;
      if constexpr (sizeof(T) == 2) {  // MFMA operand order within each 16-key group
        const int q16 = p & 15, gg = q16 >> 3, jj = q16 & 7;
        key = (p & ~15) + 8 * (jj >> 2) + 4 * gg + (jj & 3);
      }
      out[e] = sv[key][d];
    }
    *reinterpret_cast<V*>(vt_out + (size_t)(head * DH + d) * cap + tok0 + pos0) = out;
  }
}

// ---------------------------------------------------------------- patch-embed input
template <class T>
__global__ void patch_input_kernel(const float* __restrict__ x, int n, int c_p,
                                   const float* __restrict__ cond, int c_c, int mode, RopeGrid g,
                                   T* __restrict__ xin) {
  const int C = c_p + c_c;
  const long long total = (long long)n * C;
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < total;
       i += (long long)gridDim.x * blockDim.x) {
    const int tok = (int)(i / C), ch = (int)(i - (long long)tok * C);
    float v;
    if (ch < c_p) {
      v = x[(size_t)tok * c_p + ch];
    } else {
      const int cc = ch - c_p;
      if (mode == 0) {
        v = 0.f;
      } else if (mode == 1) {
        v = cond[(size_t)tok * c_c + cc];
      } else {
        // token (f, y, x), channel (c, dy, dx) <- half-res token (f, y/2, x/2),
        // channel (c, y%2, x%2): nearest 2x upsample in pixel space, re-patchified.
        const int hw = g.h * g.w;
        const int f = tok / hw, rem = tok - f * hw;
        const int y = rem / g.w, xx = rem - y * g.w;
        const int hl = g.h / 2, wl = g.w / 2;
        const int src_tok = (f * hl + y / 2) * wl + xx / 2;
        const int src_ch = (cc / 4) * 4 + (y % 2) * 2 + (xx % 2);
        v = cond[(size_t)src_tok * c_c + src_ch];
      }
    }
    xin[i] = from_f<T>(v);
  }
}

// x[i] = a z[i] + b e[i] (fp32): a point of the flow-matching path between data z
// (a = 1 - t) and noise e (b = t).
__global__ void noise_to_kernel(float* __restrict__ x, const float* __restrict__ z,
                                const float* __restrict__ e, float a, float b, long long n) {
  const long long n4 = n / 4;
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n4;
       i += (long long)gridDim.x * blockDim.x) {
    const f32x4 zz = reinterpret_cast<const f32x4*>(z)[i];
    const f32x4 ee = reinterpret_cast<const f32x4*>(e)[i];
    f32x4 r;
#pragma unroll
    for (int k = 0; k < 4; ++k) r[k] = fmaf(b, ee[k], a * zz[k]);
    reinterpret_cast<f32x4*>(x)[i] = r;
  }
  if (blockIdx.x == 0 && threadIdx.x < (n & 3)) {
    const long long i = n4 * 4 + threadIdx.x;
    x[i] = fmaf(b, e[i], a * z[i]);
  }
}

__global__ void euler_kernel(float* __restrict__ x, const float* __restrict__ v, float dt,
                             long long n) {
  const long long n4 = n / 4;
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < n4;
       i += (long long)gridDim.x * blockDim.x) {
    f32x4 a = reinterpret_cast<f32x4*>(x)[i];
    f32x4 b = reinterpret_cast<const f32x4*>(v)[i];
#pragma unroll
    for (int r = 0; r < 4; ++r) a[r] = fmaf(dt, b[r], a[r]);
    reinterpret_cast<f32x4*>(x)[i] = a;
  }
  if (blockIdx.x == 0 && threadIdx.x < (n & 3)) {
    const long long i = n4 * 4 + threadIdx.x;
    x[i] = fmaf(dt, v[i], x[i]);
  }
}

// ---------------------------------------------------------------- timestep conditioning
// phi(t) = [cos(s w_i) || sin(s w_i)], s = 1000 t, w_i = 10000^(-i/128), in double.
__device__ __forceinline__ void timestep_features_at(double t, float* __restrict__ phi) {
  const int i = threadIdx.x;  // 128 threads
  const double s = 1000.0 * t;
  const double w = pow(10000.0, -(double)i / 128.0);
  phi[i] = (float)cos(s * w);
  phi[128 + i] = (float)sin(s * w);
}
__global__ void timestep_features_kernel(double t, float* __restrict__ phi) { timestep_features_at(t, phi); }
// Features of up to MOD_BATCH timesteps, one workgroup each: phi[j] = features of t[j].
struct TimeBatch {
  double t[MOD_BATCH];
};
__global__ void timestep_features_batch_kernel(TimeBatch tb, float* __restrict__ phi) {
  timestep_features_at(tb.t[blockIdx.x], phi + (size_t)blockIdx.x * 256);
}

// y_j[r] = act(W[r, :] . x_j + b[r]) for r < R and nt <= NT vectors x_j (x_j at
// x + j ldx, y_j at y + j ldy).  One wave per RW consecutive output rows, so every
// weight row is read once for all nt vectors.  A lane reads 16 bytes of a row per step
// (8 bf16 or 4 fp32); K is a multiple of 256, and the steps are unrolled so that their
// loads are in flight together.  Per (row, vector) the products are accumulated by
// explicit operations in the same order for every NT and RW, so the results do not
// depend on them.
template <class T, int ACT, int NT, int RW>
__global__ __launch_bounds__(256) void gemv_kernel(const T* __restrict__ W,
                                                   const T* __restrict__ b, int R, int K,
                                                   const float* __restrict__ x, int ldx, int nt,
                                                   float* __restrict__ y, int ldy) {
  typedef typename Vec<T>::type V;
  constexpr int VE = Vec<T>::n;
  const int lane = threadIdx.x & 63;
  const int r0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * RW;
  if (r0 >= R) return;
  float acc[RW][NT];
#pragma unroll
  for (int rr = 0; rr < RW; ++rr)
#pragma unroll
    for (int v = 0; v < NT; ++v) acc[rr][v] = 0.f;
#pragma unroll(RW == 1 ? 4 : 2)
  for (int k = lane * VE; k < K; k += 64 * VE) {
    V w[RW];
#pragma unroll
    for (int rr = 0; rr < RW; ++rr) w[rr] = as_vec<V>(ld16(W + (size_t)min(r0 + rr, R - 1) * K + k));
#pragma unroll
    for (int v = 0; v < NT; ++v) {
      if (v < nt) {
        // explicit operations (a product, three fmas, an add per 4 terms): the same
        // rounding in every instantiation, with short dependency chains
#pragma unroll
        for (int j = 0; j < VE; j += 4) {
          const f32x4 x4 = *reinterpret_cast<const f32x4*>(x + (size_t)v * ldx + k + j);
#pragma unroll
          for (int rr = 0; rr < RW; ++rr) {
            float p = to_f(w[rr][j]) * x4[0];
            p = fmaf(to_f(w[rr][j + 1]), x4[1], p);
            p = fmaf(to_f(w[rr][j + 2]), x4[2], p);
            p = fmaf(to_f(w[rr][j + 3]), x4[3], p);
            acc[rr][v] += p;
          }
        }
      }
    }
  }
#pragma unroll
  for (int rr = 0; rr < RW; ++rr) {
    const int r = r0 + rr;
#pragma unroll
    for (int v = 0; v < NT; ++v) {
      if (v < nt && r < R) {
        const float a = wave_sum(acc[rr][v]);
        if (lane == 0) {
          float o = a + to_f(b[r]);
          if (ACT) o = silu(o);
          y[(size_t)v * ldy + r] = o;
        }
      }
    }
  }
}

// One row per wave for a single vector; two rows per wave for a batch (each vector
// fragment then serves both rows; the weight chunks are the only per-row registers).
template <class T, int NT>
void gemv_launch(const void* w, const void* b, int R, int K, const float* x, int ldx, int nt, float* y, int ldy,
                 int act, hipStream_t s) {
  constexpr int RW = NT == 1 ? 1 : 2;
  dim3 grid((R + 4 * RW - 1) / (4 * RW));
  if (act)
    gemv_kernel<T, 1, NT, RW><<<grid, 256, 0, s>>>((const T*)w, (const T*)b, R, K, x, ldx, nt, y, ldy);
  else
    gemv_kernel<T, 0, NT, RW><<<grid, 256, 0, s>>>((const T*)w, (const T*)b, R, K, x, ldx, nt, y, ldy);
}

template <class T>
hipError_t modulation_t(int D, int L, double t, const void* t1w, const void* t1b, const void* t2w,
                        const void* t2b, const void* const* modw, const void* const* modb,
                        const void* fmodw, const void* fmodb, float* tmp, float* mod_out,
                        float* fmod_out, hipStream_t s) {
  float* phi = tmp;            // [256]
  float* e1 = tmp + 256;       // [D]
  float* c = tmp + 256 + D;    // [D]
  timestep_features_kernel<<<1, 128, 0, s>>>(t, phi);
  auto G = [&](const void* w, const void* b, int R, int K, const float* x, float* y, int act) {
    gemv_launch<T, 1>(w, b, R, K, x, K, 1, y, R, act, s);
  };
  G(t1w, t1b, D, 256, phi, e1, 1);
  G(t2w, t2b, D, D, e1, c, 1);
  for (int l = 0; l < L; ++l) G(modw[l], modb[l], 6 * D, D, c, mod_out + (size_t)l * 6 * D, 0);
  G(fmodw, fmodb, 2 * D, D, c, fmod_out, 0);
  return hipGetLastError();
}

// Boundary by reuse: K rows [first, first + n) of a chunk's K (normed, rotated at time
// t_src) become rows [0, n) of the boundary K, their time-axis pairs turned by dt
// (= t_dst - t_src; rotations about the same axis add, so this places them at t_dst);
// rows [n, rows_pad) are zeroed.  One thread per (row, head, rotation pair).
template <class T, int DH>
__global__ __launch_bounds__(256) void bnd_reuse_k_kernel(const T* __restrict__ kc, int first, int n,
                                                          int rows_pad, int H, float dt,
                                                          float log2_theta, T* __restrict__ kb) {
  constexpr int NPAIR = DH / 2;
  const int d_t = DH - 4 * (DH / 6);  // time-axis dims (the first d_t / 2 pairs)
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long long)rows_pad * H * NPAIR) return;
  const int p = (int)(i % NPAIR);
  const int head = (int)((i / NPAIR) % H);
  const int j = (int)(i / ((long long)NPAIR * H));
  const int D = H * DH;
  T* dst = kb + (size_t)j * D + head * DH + 2 * p;
  if (j >= n) {
    dst[0] = from_f<T>(0.f);
    dst[1] = from_f<T>(0.f);
    return;
  }
  const T* src = kc + (size_t)(first + j) * D + head * DH + 2 * p;
  const float x0 = to_f(src[0]), x1 = to_f(src[1]);
  if (2 * p < d_t) {
    const float ang = dt * exp2f(-(2.0f * (float)p / (float)d_t) * log2_theta);
    float sn, cs;
    sincosf(ang, &sn, &cs);
    dst[0] = from_f<T>(x0 * cs - x1 * sn);
    dst[1] = from_f<T>(x0 * sn + x1 * cs);
  } else {
    dst[0] = src[0];
    dst[1] = src[1];
  }
}

// Stored column of key o in the V^T layout: bf16 keeps each aligned group of 16 keys
// in MFMA operand order (key offset q at 8 ((q % 8) / 4) + 4 (q / 8) + q % 4); fp32 is
// in natural order.
template <class T>
__device__ __forceinline__ int vt_col(int o) {
  if constexpr (sizeof(T) == 2) {
    const int q = o & 15;
    return (o & ~15) + 8 * ((q & 7) >> 2) + 4 * (q >> 3) + (q & 3);
  } else {
    return o;
  }
}

// V^T columns of keys [first, first + n) of a chunk (row pitch cap_src) become the
// columns of keys [0, n) of the boundary V^T (pitch cap_dst); keys [n, cols_pad) are
// zeroed.  One thread per (dim, key).
template <class T>
__global__ __launch_bounds__(256) void bnd_reuse_v_kernel(const T* __restrict__ vt, int cap_src, int first,
                                                          int n, int cols_pad, int D, T* __restrict__ vb,
                                                          int cap_dst) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long long)D * cols_pad) return;
  const int j = (int)(i % cols_pad);
  const int d = (int)(i / cols_pad);
  vb[(size_t)d * cap_dst + vt_col<T>(j)] =
      j < n ? vt[(size_t)d * cap_src + vt_col<T>(first + j)] : from_f<T>(0.f);
}

}  // namespace

hipError_t rmsnorm_mod(int dtype, const float* h, int n, int D, const float* shift,
                       const float* scale, float eps, void* out, hipStream_t s, const hipEvent_t* ev) {
  if (n <= 0) return hipSuccess;
  if (D % 256 || D > 4096) return hipErrorInvalidValue;
  if (D == 1536 || D == 3072) {
    const dim3 g2((n + 7) / 8), b(256);
#define RMS2(T, IT) return launch_k(rmsnorm_mod2_kernel<T, IT>, g2, b, s, ev, h, n, shift, scale, eps, (T*)out)
    if (dtype == BF16) { if (D == 1536) RMS2(bf16, 6); else RMS2(bf16, 12); }
    else { if (D == 1536) RMS2(float, 6); else RMS2(float, 12); }
#undef RMS2
  }
  const dim3 grid((n + 3) / 4), b(256);
  if (dtype == BF16) return launch_k(rmsnorm_mod_kernel<bf16>, grid, b, s, ev, h, n, D, shift, scale, eps, (bf16*)out);
  return launch_k(rmsnorm_mod_kernel<float>, grid, b, s, ev, h, n, D, shift, scale, eps, (float*)out);
}

hipError_t qknorm_rope(int dtype, int dh, int H, int n, const void* q_in, const void* k_in,
                       const void* v_in, int ld_in, const void* gq, const void* gk, int rope,
                       RopeGrid g, float eps, float theta, float q_scale, void* q_out,
                       void* k_out, void* vt_out, int cap, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int npad = (n + 63) / 64 * 64;
  if (npad > cap && (k_in || v_in)) return hipErrorInvalidValue;
  dim3 grid(npad / 64, H);
  const float l2t = log2f(theta);
  const int D = H * dh;
#define QKR(T, DHV)                                                                          \
  qknorm_rope_kernel<T, DHV><<<grid, 256, 0, s>>>(n, (const T*)q_in, (const T*)k_in,         \
                                                  (const T*)v_in, ld_in, (const T*)gq,       \
                                                  (const T*)gk, rope, g, eps, l2t, q_scale, (T*)q_out, \
                                                  (T*)k_out, (T*)vt_out, cap, D)
  if (dtype == BF16 && dh == 128) QKR(bf16, 128);
  else if (dtype == BF16 && dh == 64) QKR(bf16, 64);
  else if (dtype == F32 && dh == 128) QKR(float, 128);
  else if (dtype == F32 && dh == 64) QKR(float, 64);
  else return hipErrorInvalidValue;
#undef QKR
  return hipGetLastError();
}

hipError_t patch_input(int dtype, const float* x, int n, int c_p, const float* cond, int c_c,
                       int cond_mode, RopeGrid g, void* xin, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const long long total = (long long)n * (c_p + c_c);
  const int blocks = (int)((total + 255) / 256 < 4096 ? (total + 255) / 256 : 4096);
  if (dtype == BF16)
    patch_input_kernel<bf16><<<blocks, 256, 0, s>>>(x, n, c_p, cond, c_c, cond_mode, g, (bf16*)xin);
  else
    patch_input_kernel<float><<<blocks, 256, 0, s>>>(x, n, c_p, cond, c_c, cond_mode, g, (float*)xin);
  return hipGetLastError();
}

hipError_t noise_to(float* x, const float* z, const float* e, float a, float b, long long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  long long blocks = (n / 4 + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 8192) blocks = 8192;
  noise_to_kernel<<<(int)blocks, 256, 0, s>>>(x, z, e, a, b, n);
  return hipGetLastError();
}

hipError_t euler(float* x, const float* v, float dt, long long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  long long blocks = (n / 4 + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 8192) blocks = 8192;
  euler_kernel<<<(int)blocks, 256, 0, s>>>(x, v, dt, n);
  return hipGetLastError();
}

hipError_t modulation(int dtype, int D, int L, double t, const void* t1w, const void* t1b,
                      const void* t2w, const void* t2b, const void* const* modw,
                      const void* const* modb, const void* fmodw, const void* fmodb, float* tmp,
                      float* mod_out, float* fmod_out, hipStream_t s) {
  if (D % 256) return hipErrorInvalidValue;
  if (dtype == BF16)
    return modulation_t<bf16>(D, L, t, t1w, t1b, t2w, t2b, modw, modb, fmodw, fmodb, tmp, mod_out,
                              fmod_out, s);
  return modulation_t<float>(D, L, t, t1w, t1b, t2w, t2b, modw, modb, fmodw, fmodb, tmp, mod_out,
                             fmod_out, s);
}

// One thread per 16-byte chunk of the output (8 bf16 or 4 fp32).
template <class T>
__global__ __launch_bounds__(256) void head_blockdiag_kernel(const T* __restrict__ v, int M, int D, int dh,
                                                             T* __restrict__ out) {
  constexpr int VE = 16 / (int)sizeof(T);
  const int H = D / dh, cpr = D / VE;  // 16-byte chunks per row
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long long)H * 64 * cpr) return;
  const int row = (int)(i / cpr), c = (int)(i - (long long)row * cpr) * VE;
  const int h = row / 64, k = row - h * 64;
  u32x4 val = {0u, 0u, 0u, 0u};
  if (k < M && c / dh == h) val = ld16(v + (size_t)k * D + c);
  st16(out + (size_t)row * D + c, val);
}

hipError_t head_blockdiag(int dtype, const void* v, int M, int D, int dh, void* out, hipStream_t s) {
  if (M < 0 || M > 64 || D % 8 || dh % 8 || D % dh) return hipErrorInvalidValue;
  const long long n = (long long)(D / dh) * 64 * (D / (dtype == BF16 ? 8 : 4));
  dim3 grid((unsigned)((n + 255) / 256)), block(256);
  if (dtype == BF16)
    head_blockdiag_kernel<bf16><<<grid, block, 0, s>>>((const bf16*)v, M, D, dh, (bf16*)out);
  else
    head_blockdiag_kernel<float><<<grid, block, 0, s>>>((const float*)v, M, D, dh, (float*)out);
  return hipGetLastError();
}

hipError_t block_modulation(int dtype, int D, const void* w, const void* b, const float* c, float* out,
                            hipStream_t s) {
  if (D % 256) return hipErrorInvalidValue;
  if (dtype == BF16)
    gemv_launch<bf16, 1>(w, b, 6 * D, D, c, D, 1, out, 6 * D, 0, s);
  else
    gemv_launch<float, 1>(w, b, 6 * D, D, c, D, 1, out, 6 * D, 0, s);
  return hipGetLastError();
}

hipError_t timestep_cond_batch(int dtype, int D, const double* t, int nt, const void* t1w, const void* t1b,
                               const void* t2w, const void* t2b, float* tmp, float* c, hipStream_t s) {
  if (nt < 1 || nt > MOD_BATCH || D % 256) return hipErrorInvalidValue;
  TimeBatch tb{};
  for (int j = 0; j < nt; ++j) tb.t[j] = t[j];
  float* phi = tmp;                          // [nt, 256]
  float* e1 = tmp + (size_t)MOD_BATCH * 256;  // [nt, D]
  timestep_features_batch_kernel<<<nt, 128, 0, s>>>(tb, phi);
  if (dtype == BF16) {
    gemv_launch<bf16, MOD_BATCH>(t1w, t1b, D, 256, phi, 256, nt, e1, D, 1, s);
    gemv_launch<bf16, MOD_BATCH>(t2w, t2b, D, D, e1, D, nt, c, D, 1, s);
  } else {
    gemv_launch<float, MOD_BATCH>(t1w, t1b, D, 256, phi, 256, nt, e1, D, 1, s);
    gemv_launch<float, MOD_BATCH>(t2w, t2b, D, D, e1, D, nt, c, D, 1, s);
  }
  return hipGetLastError();
}

hipError_t gemv_batch(int dtype, int R, int K, const void* w, const void* b, const float* x, int ldx, int nt,
                      float* y, int ldy, hipStream_t s) {
  if (nt < 1 || nt > MOD_BATCH || K % 256) return hipErrorInvalidValue;
  if (dtype == BF16)
    gemv_launch<bf16, MOD_BATCH>(w, b, R, K, x, ldx, nt, y, ldy, 0, s);
  else
    gemv_launch<float, MOD_BATCH>(w, b, R, K, x, ldx, nt, y, ldy, 0, s);
  return hipGetLastError();
}

hipError_t boundary_reuse(int dtype, int dh, int H, const void* kc, const void* vtc, int cap_src, int first,
                          int n, float dt, float theta, void* kb, void* vtb, int cap_dst, hipStream_t s) {
  const int rows_pad = (n + 63) / 64 * 64;
  if (n <= 0 || rows_pad > cap_dst) return hipErrorInvalidValue;
  const int D = H * dh;
  const float l2t = log2f(theta);
  const long long nk = (long long)rows_pad * H * (dh / 2);
  const long long nv = (long long)D * rows_pad;
  dim3 gk((unsigned)((nk + 255) / 256)), gv((unsigned)((nv + 255) / 256)), b(256);
  if (dtype == BF16 && dh == 128) {
    bnd_reuse_k_kernel<bf16, 128><<<gk, b, 0, s>>>((const bf16*)kc, first, n, rows_pad, H, dt, l2t, (bf16*)kb);
    bnd_reuse_v_kernel<bf16><<<gv, b, 0, s>>>((const bf16*)vtc, cap_src, first, n, rows_pad, D, (bf16*)vtb, cap_dst);
  } else if (dtype == BF16 && dh == 64) {
    bnd_reuse_k_kernel<bf16, 64><<<gk, b, 0, s>>>((const bf16*)kc, first, n, rows_pad, H, dt, l2t, (bf16*)kb);
    bnd_reuse_v_kernel<bf16><<<gv, b, 0, s>>>((const bf16*)vtc, cap_src, first, n, rows_pad, D, (bf16*)vtb, cap_dst);
  } else if (dtype == F32 && dh == 128) {
    bnd_reuse_k_kernel<float, 128><<<gk, b, 0, s>>>((const float*)kc, first, n, rows_pad, H, dt, l2t, (float*)kb);
    bnd_reuse_v_kernel<float><<<gv, b, 0, s>>>((const float*)vtc, cap_src, first, n, rows_pad, D, (float*)vtb, cap_dst);
  } else if (dtype == F32 && dh == 64) {
    bnd_reuse_k_kernel<float, 64><<<gk, b, 0, s>>>((const float*)kc, first, n, rows_pad, H, dt, l2t, (float*)kb);
    bnd_reuse_v_kernel<float><<<gv, b, 0, s>>>((const float*)vtc, cap_src, first, n, rows_pad, D, (float*)vtb, cap_dst);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dit
