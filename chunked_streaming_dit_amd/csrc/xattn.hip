// Attention over one short key segment (the audio cross-attention): the exact softmax
// over a single 64-key tile per head, as output O or as the probabilities P.
#include "attn_common.h"
#include "kernels.h"

namespace dit {

namespace {

// Attention over one short key segment (at most one 64-key tile, e.g. the audio tokens
// of the cross-attention), bf16 with dh = 128.  A workgroup is 4 waves x 32 queries of
// one head; it stages the head's K and V^T tile in LDS once (swizzled as in the
// self-attention kernel) and each wave computes S^T = K Q^T, the exact softmax over the
// tile and O^T = V^T P^T.  With 32 KB of LDS and no pipeline state, several workgroups
// fit per CU, so the whole grid is resident at once: the kernel streams Q in and O out.
// POUT: the normalised probabilities themselves are written instead, P [nq, H*64] with
// head h's 64 key columns from h*64 (keys >= n exactly 0), and V is not read.
constexpr int XW = 4;           // waves per workgroup
constexpr int XBQ = 32 * XW;    // queries per workgroup

struct XArgs {
  const void* q;
  void* o;
  const void* k;
  const void* vt;
  int ldq, ldo, nq, n, cap, H;
  float scale;
};

template <bool POUT>
__global__ __launch_bounds__(64 * XW, 3) void xattn_kernel(XArgs a) {
  typedef bf16x8 V;
  typedef bf16 T;
  constexpr int DH = 128, VE = 8, SZ = 2, QV = DH / 16, DB = DH / 32;
  constexpr int RBK = DH * SZ, RBV = BKV * SZ;
  __shared__ __attribute__((aligned(1024))) char smem[BKV * RBK + DH * RBV];
  char* const sk = smem;
  char* const sv = smem + BKV * RBK;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, lg = lane >> 5;
  const int nqt = (a.nq + XBQ - 1) / XBQ;
  const int head = blockIdx.x / nqt, qt = blockIdx.x - head * nqt;
  const int qrow = qt * XBQ + wave * 32 + l32;
  const bool qvalid = qrow < a.nq;
  const int D = a.H * DH;

  // K tile: 64 rows x 16 chunks; V^T tile: 128 rows x 8 chunks (1024 chunks each);
  // chunk c of row r goes to position swz(r, c).  Rows / columns past n are zero in
  // the source (padded to cap).
  {
    const char* kg = reinterpret_cast<const char*>(a.k) + (size_t)head * DH * SZ;
    const char* vg = reinterpret_cast<const char*>(a.vt) + (size_t)head * DH * a.cap * SZ;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 256 * i;
      const int rk = c >> 4, ck = c & 15;
      st16(sk + rk * RBK + swz<RBK>(rk, ck) * 16, ld16(kg + (size_t)rk * D * SZ + ck * 16));
      if (!POUT) {
        const int rv = c >> 3, cv = c & 7;
        st16(sv + rv * RBV + swz<RBV>(rv, cv) * 16, ld16(vg + (size_t)rv * a.cap * SZ + cv * 16));
      }
    }
  }
  V qf[QV];
  {
    const char* qp = reinterpret_cast<const char*>(a.q) + ((size_t)(qvalid ? qrow : 0) * a.ldq + head * DH) * SZ;
#pragma unroll
    for (int s = 0; s < QV; ++s) {
      u32x4 r = {0u, 0u, 0u, 0u};
      if (qvalid) r = ld16(qp + s * 32 + lg * 16);
      qf[s] = as_vec<V>(r);
    }
  }
  __syncthreads();

  f32x16 S[2];
  short_scores(sk, qf, a.n, l32, lg, S);
  if constexpr (POUT) {
    short_probs(S, a.scale);
    if (!qvalid) return;
    T* pp = reinterpret_cast<T*>(a.o) + (size_t)qrow * a.ldo + head * BKV;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = S[kb][4 * q + r];
        store4<T>(pp + kb * 32 + 8 * q + 4 * lg, v);  // keys kb*32 + 8q + 4lg + r
      }
    return;
  }
  // exact softmax over the tile (keys past n have score -inf, so zero weight)
  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[kb][r]);
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float ms = mx * a.scale;
  f32x16 O[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) O[d][r] = 0.f;
  float l = 0.f;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      V pf;
#pragma unroll
      for (int j = 0; j < VE; ++j) pf[j] = from_f<T>(__builtin_amdgcn_exp2f(fmaf(S[kb][v * VE + j], a.scale, -ms)));
      l = row_sum_add(pf, l);
      const int pos = swz<RBV>(l32, (kb * 32 + v * 16 + lg * 8) * SZ / 16);
#pragma unroll
      for (int d = 0; d < DB; ++d)
        O[d] = mfma32(as_vec<V>(ld16(sv + (d * 32 + l32) * RBV + pos * 16)), pf, O[d]);
    }
  const float lt = l + __shfl_xor(l, 32);
  if (!qvalid) return;
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  T* op = reinterpret_cast<T*>(a.o) + (size_t)qrow * a.ldo + head * DH;
#pragma unroll
  for (int d = 0; d < DB; ++d)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = O[d][4 * q + r] * inv;
      store4<T>(op + d * 32 + 8 * q + 4 * lg, v);
    }
}

}  // namespace

bool short_attention_fits(int dtype, int dh, int nseg, const AttnSeg* segs) {
  return dtype == BF16 && dh == 128 && nseg == 1 && segs[0].n >= 1 && segs[0].n <= BKV && segs[0].cap >= BKV;
}

hipError_t short_attention(int dh, int H, const void* q, int ldq, void* o, int ldo, int nq, const AttnSeg& seg,
                           bool q_prescaled, hipStream_t s) {
  if (nq <= 0) return hipSuccess;
  if (dh != 128 || seg.n < 1 || seg.n > BKV || seg.cap < BKV) return hipErrorInvalidValue;
  XArgs a;
  a.q = q;
  a.o = o;
  a.k = seg.k;
  a.vt = seg.vt;
  a.ldq = ldq;
  a.ldo = ldo;
  a.nq = nq;
  a.n = seg.n;
  a.cap = seg.cap;
  a.H = H;
  a.scale = q_prescaled ? 1.0f : attention_q_scale(dh);
  const int nqt = (nq + XBQ - 1) / XBQ;
  xattn_kernel<false><<<nqt * H, 64 * XW, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t short_attention_probs(int dh, int H, const void* q, int ldq, void* p, int ldp, int nq, const AttnSeg& seg,
                                 bool q_prescaled, hipStream_t s) {
  if (nq <= 0) return hipSuccess;
  if (dh != 128 || seg.n < 1 || seg.n > BKV || seg.cap < BKV || ldp < H * BKV) return hipErrorInvalidValue;
  XArgs a;
  a.q = q;
  a.o = p;
  a.k = seg.k;
  a.vt = nullptr;
  a.ldq = ldq;
  a.ldo = ldp;
  a.nq = nq;
  a.n = seg.n;
  a.cap = seg.cap;
  a.H = H;
  a.scale = q_prescaled ? 1.0f : attention_q_scale(dh);
  const int nqt = (nq + XBQ - 1) / XBQ;
  xattn_kernel<true><<<nqt * H, 64 * XW, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace dit
