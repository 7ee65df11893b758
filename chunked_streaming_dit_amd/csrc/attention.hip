// Flash attention over segmented keys: [reference | boundary | chunk] (self-attention)
// or [audio] (cross-attention), one head per grid row.
//
// Per workgroup: 128 queries of one head (4 waves x 32 queries).  Key/value tiles of
// 64 keys are staged in LDS (double-buffered, one barrier per tile; the next tile is
// fetched into registers while the current one is used).  Each wave computes the
// transposed score tile S^T = K Q^T with 32x32 MFMAs, so that a lane holds scores of
// ONE query for 32 keys: the online-softmax row max needs one cross-lane exchange
// (lanes l and l^32), the row sum none until the end, and the rescale of the output
// accumulator O^T = V^T P^T touches only the lane's own registers.  The exponentiated
// scores feed the second MFMA directly from registers (no LDS round trip); the key
// order they are held in is matched by the stored order of V^T (see kernels.h).
// Softmax statistics and accumulation are fp32; exp2 with log2(e)/sqrt(dh) folded in.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace dit {

namespace {

struct AttnArgs {
  const void* q;
  void* o;
  int ldq, ldo, nq, ldk, H;
  int nseg;
  float scale;  // log2(e) / sqrt(dh)
  float thr;    // RESCALE_LOG2 / scale: lazy-rescale threshold in raw score units
  AttnSeg seg[ATTN_MAX_SEGS];
};

constexpr int BQ = 128;  // queries per workgroup
constexpr float RESCALE_LOG2 = 8.0f;

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

template <class T, int DH>
__global__ __launch_bounds__(256, 2) void attn_kernel(AttnArgs a) {
  typedef typename Vec<T>::type V;
  constexpr int VE = Vec<T>::n;
  constexpr int SZ = (int)sizeof(T);
  constexpr int QV = DH / (2 * VE);       // 16-byte vector steps over dh
  constexpr int KROWB = DH * SZ + 16;     // LDS bytes per key row
  constexpr int VROWB = BKV * SZ + 16;    // LDS bytes per V^T row
  constexpr int CK = DH * SZ / 16;        // 16-byte chunks per key row
  constexpr int CV = BKV * SZ / 16;       // 16-byte chunks per V^T row
  constexpr int KCH = BKV * CK / 256;     // K chunks per thread per tile
  constexpr int VCH = DH * CV / 256;      // V^T chunks per thread per tile
  constexpr int DB = DH / 32;             // 32-row blocks of dh
  constexpr int STAGE = BKV * KROWB + DH * VROWB;
  static_assert(BKV * CK % 256 == 0 && DH * CV % 256 == 0, "tile");
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, lg = lane >> 5;
  // 1-D grid over (head, q-tile), head-major, remapped so that each XCD works through
  // a contiguous range: the q-tiles of a head share that head's K/V in one L2.
  const int nqt = (a.nq + BQ - 1) / BQ;
  const int wi = xcd_remap(blockIdx.x, nqt * a.H);
  const int head = wi / nqt;
  const int qrow = (wi - head * nqt) * BQ + wave * 32 + l32;
  const bool qvalid = qrow < a.nq;

  // Q fragments (second MFMA operand): query qrow, dh = s*2VE + lg*VE + [0, VE).
  V qf[QV];
  {
    const char* qp = reinterpret_cast<const char*>(a.q) +
                     ((size_t)(qvalid ? qrow : 0) * a.ldq + head * DH) * SZ;
#pragma unroll
    for (int s = 0; s < QV; ++s) {
      u32x4 r = {0u, 0u, 0u, 0u};
      if (qvalid) r = ld16(qp + s * 32 + lg * 16);
      qf[s] = as_vec<V>(r);
    }
  }

  // Flattened walk over the tiles of all segments.
  int total = 0;
#pragma unroll
  for (int s = 0; s < ATTN_MAX_SEGS; ++s)
    if (s < a.nseg) total += (a.seg[s].n + BKV - 1) / BKV;

  u32x4 kst[KCH], vst[VCH];
  auto gload = [&](int si, int base) {
    const AttnSeg& sg = a.seg[si];
    const char* kp = reinterpret_cast<const char*>(sg.k);
    const char* vp = reinterpret_cast<const char*>(sg.vt);
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + 256 * i;
      const int r = c / CK, cc = c % CK;
      kst[i] = ld16(kp + ((size_t)(base + r) * a.ldk + head * DH) * SZ + cc * 16);
    }
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int c = tid + 256 * i;
      const int r = c / CV, cc = c % CV;
      vst[i] = ld16(vp + ((size_t)(head * DH + r) * sg.cap + base) * SZ + cc * 16);
    }
  };
  auto sstore = [&](int buf) {
    char* sk = smem + buf * STAGE;
    char* sv = sk + BKV * KROWB;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + 256 * i;
      st16(sk + (c / CK) * KROWB + (c % CK) * 16, kst[i]);
    }
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int c = tid + 256 * i;
      st16(sv + (c / CV) * VROWB + (c % CV) * 16, vst[i]);
    }
  };
  auto advance = [&](int& si, int& base) {
    base += BKV;
    if (base >= a.seg[si].n) {
      base = 0;
      ++si;
      while (si < a.nseg && a.seg[si].n == 0) ++si;
    }
  };

  f32x16 O[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) O[d][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  int si = 0, base = 0;
  while (si < a.nseg && a.seg[si].n == 0) ++si;
  int nsi = si, nbase = base;
  if (total > 0) {
    gload(si, base);
    sstore(0);
    advance(nsi, nbase);
  }

  for (int t = 0; t < total; ++t) {
    const int buf = t & 1;
    const bool more = t + 1 < total;
    if (more) gload(nsi, nbase);
    __syncthreads();
    const char* sk = smem + buf * STAGE;
    const char* sv = sk + BKV * KROWB;

    // S^T tile: 2 blocks of 32 keys x 32 queries.  Lane: query l32,
    // key = 32 kb + 8 (e/4) + 4 lg + e%4 for element e.
    f32x16 S[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) S[kb][r] = 0.f;
#pragma unroll
      for (int s = 0; s < QV; ++s) {
        V kf = as_vec<V>(ld16(sk + (kb * 32 + l32) * KROWB + s * 32 + lg * 16));
        S[kb] = mfma32(kf, qf[s], S[kb]);
      }
    }
    const int seg_n = a.seg[si].n;
    if (base + BKV > seg_n) {  // ragged tail of a segment: mask keys >= n
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = base + kb * 32 + 8 * (r >> 2) + 4 * lg + (r & 3);
          if (key >= seg_n) S[kb][r] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, S[kb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // Lazy rescale: keep the running max unless a score exceeds it by more than
    // RESCALE_LOG2 in the exp2 domain (then p stays <= 2^RESCALE_LOG2, which fp32
    // sums and bf16 operands hold exactly as well as p <= 1).  The decision is
    // wave-uniform; lanes l and l^32 hold the same query and the same max.
    if (__any(mx > m_run + a.thr)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * a.scale);
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < DB; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) O[d][r] *= alpha;
      m_run = m_new;
    }
    const float ms = m_run * a.scale;
    // P^T operands: elements [v*VE, v*VE+VE) of S[kb].  The row sum is taken from the
    // converted operand values, i.e. from exactly the weights the second MFMA uses.
    V pf[2][16 / VE];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16 / VE; ++v) {
#pragma unroll
        for (int j = 0; j < VE; ++j)
          pf[kb][v][j] = from_f<T>(__builtin_amdgcn_exp2f(fmaf(S[kb][v * VE + j], a.scale, -ms)));
        l_run = row_sum_add(pf[kb][v], l_run);
      }

    // O^T += V^T P^T; the V^T vector at key offset 32 kb + v*2VE + lg*VE holds the
    // same keys as pf[kb][v] (stored order).
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int v = 0; v < 16 / VE; ++v) {
#pragma unroll
        for (int d = 0; d < DB; ++d) {
          V vf = as_vec<V>(ld16(sv + (d * 32 + l32) * VROWB + (kb * 32 + v * 2 * VE + lg * VE) * SZ));
          O[d] = mfma32(vf, pf[kb][v], O[d]);
        }
      }
    }
    if (more) {
      sstore(buf ^ 1);
      si = nsi;
      base = nbase;
      advance(nsi, nbase);
    }
  }

  // Normalise and store: lane holds query qrow, dh = 32 d + 8 q + 4 lg + [0, 4).
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (!qvalid) return;
  const float inv = 1.0f / l_tot;
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

hipError_t attention(int dtype, int dh, int H, const void* q, int ldq, void* o, int ldo, int nq,
                     int ldk, const AttnSeg* segs, int nseg, hipStream_t s) {
  if (nq <= 0) return hipSuccess;
  if (nseg < 1 || nseg > ATTN_MAX_SEGS) return hipErrorInvalidValue;
  AttnArgs a;
  a.q = q;
  a.o = o;
  a.ldq = ldq;
  a.ldo = ldo;
  a.nq = nq;
  a.ldk = ldk;
  a.nseg = nseg;
  a.H = H;
  a.scale = (float)(1.4426950408889634 / sqrt((double)dh));
  a.thr = RESCALE_LOG2 / a.scale;
  for (int i = 0; i < ATTN_MAX_SEGS; ++i) a.seg[i] = i < nseg ? segs[i] : AttnSeg{nullptr, nullptr, 0, 64};
  dim3 grid(((nq + BQ - 1) / BQ) * H), block(256);
  if (dtype == BF16 && dh == 128) attn_kernel<bf16, 128><<<grid, block, 0, s>>>(a);
  else if (dtype == BF16 && dh == 64) attn_kernel<bf16, 64><<<grid, block, 0, s>>>(a);
  else if (dtype == F32 && dh == 64) attn_kernel<float, 64><<<grid, block, 0, s>>>(a);
  else if (dtype == F32 && dh == 128) attn_kernel<float, 128><<<grid, block, 0, s>>>(a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace dit
