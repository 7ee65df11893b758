// Host-side launchers of the device kernels (internal to libditchunk).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

namespace dit {

// Launch a kernel.  With ev (a start/stop event pair, either entry may be null) the
// dispatch itself stamps the kernel's start into ev[0] and its end into ev[1]
// (hipExtLaunchKernelGGL): timing without marker packets between launches.
template <typename... Args, typename F = void (*)(Args...)>
inline hipError_t launch_k(F kernel, dim3 grid, dim3 block, hipStream_t s, const hipEvent_t* ev, Args... args) {
  if (ev && (ev[0] || ev[1]))
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, ev[0], ev[1], 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
  return hipGetLastError();
}

enum Dtype { F32 = 0, BF16 = 1 };

// Token grid of a RoPE'd sequence: token i = (f, y, x) row-major, at position (t0 + f, y, x).
struct RopeGrid {
  int t0, frames, h, w;
};

// ---------------------------------------------------------------- GEMM (MFMA)
// C = A W^T (+ bias), A [M, K] (lda), W [N, K] (ldw), fp32 accumulation, then:
enum EpiKind {
  EPI_BIAS = 0,   // out[M, N] (dtype)  = C + b
  EPI_GELU = 1,   // out[M, N] (dtype)  = GELU_tanh(C + b)
  EPI_RESID = 2,  // h[M, N]   (fp32)  += gate (.) (C + b)      (gate NULL: 1)
  EPI_F32 = 3,    // out[M, N] (fp32)   = C + b
  EPI_EULER = 4,  // v = C + b; x[M, N] (fp32) += dt v; v_out (fp32, optional) = v
  EPI_QKNORM = 5, // y = C + b over N = [q | k | v] blocks of D columns (k, v optional):
                  //   q heads: QK-RMSNorm x gq x q_scale (+ 3D RoPE) -> q_out [M, D];
                  //   k heads: QK-RMSNorm x gk (+ RoPE) -> k_out [kpad, D], rows M..kpad zero;
                  //   v columns: V^T -> vt_out [D, vcap] in the attention layout (columns
                  //   M..kpad zero), or, with vt_out NULL, y -> out [M, ldo] (columns 2D..3D).
  EPI_PARTIAL = 6,  // internal (split K): the raw product of one K part -> ws (fp32)
  EPI_QKNORM_X = 7, // EPI_QKNORM for q only (N = D, no RoPE), followed in the epilogue by
                    //   the short-segment softmax of each head's q against the keys xk
                    //   ([>= 64, D], xn of them, 1..64): the normalised probabilities ->
                    //   p_out [M, ldp >= H*64] as short_attention_probs writes them; q
                    //   itself is not stored.
};
struct GemmEpi {
  int kind;
  const void* bias;   // [N] dtype, or NULL (no bias)
  void* out;          // EPI_BIAS/EPI_GELU/EPI_F32 output, EPI_RESID h, EPI_EULER x
  int ldo;
  const float* gate;  // EPI_RESID
  float* v_out;       // EPI_EULER
  float dt;           // EPI_EULER
  // EPI_QKNORM (bf16, dh = 128): gammas [dh]; q_out may be NULL (q not needed)
  const void* gq;
  const void* gk;
  void* q_out;
  void* k_out;
  void* vt_out;
  int D, kpad, rope, vcap;
  float q_scale, eps, log2_theta;
  RopeGrid g;
  // Optional fp32 workspace for EPI_RESID launches too small to fill the chip with large
  // tiles: the K range is then split over workgroups, their products summed by a second
  // kernel that applies the residual epilogue (needs splits x M x N floats).
  float* ws;
  long long ws_floats;
  int ksplit;  // internal: number of K parts of an EPI_PARTIAL launch
  // EPI_QKNORM_X: the keys (attention layout, rows >= xn zero), their count, and P
  const void* xk;
  int xn;
  void* p_out;
  int ldp;
};
// Whether gemm() can fuse EPI_QKNORM for this launch (else: EPI_BIAS + qknorm_rope).
// 32-bit operand offsets.  The LDS-staged GEMM forms each lane's offset into A and W as
// rows x row pitch in 32-bit integers (elements, then bytes), and the attention kernel
// forms the V^T offset of a head's rows (D x key capacity) in 32 bits.  Callers keep every
// GEMM operand (rows x pitch) under GEMM_MAX_ELEMS elements and every V^T buffer under
// VT_MAX_BYTES bytes; the host entry points reject larger shapes.
constexpr long long GEMM_MAX_ELEMS = (1LL << 31) - 64;
constexpr long long VT_MAX_BYTES = 1LL << 31;

// ---------------------------------------------------------------- measured ceilings
// The dense bf16 MFMA loop (flop: its algorithmic MFMA work) and the plain copy of
// probe.hip; sink holds PROBE_SINK_FLOATS floats (one per thread of the MFMA grid).
constexpr int PROBE_SINK_FLOATS = 512 * 256;
hipError_t probe_mfma(const void* data, int iters, float* sink, double* flop, hipStream_t s);
hipError_t probe_copy(const void* src, void* dst, long long bytes, hipStream_t s);

bool gemm_qknorm_fits(int dtype, int M, int N, int dh);
// ev: optional start/stop pair stamped by the first and the last kernel of the GEMM.
hipError_t gemm(int dtype, const void* A, int lda, const void* W, int ldw, int M, int N, int K,
                const GemmEpi& e, hipStream_t s, const hipEvent_t* ev = nullptr);

// ---------------------------------------------------------------- attention
// K/V segment in the attention layout:
//   k  [cap, ldk] row-major, head h at columns [h*dh, (h+1)*dh); rows >= n are zero.
//   vt [H*dh, cap] (V transposed); columns >= n are zero.  For bf16 the keys of each
//      aligned group of 16 are stored in MFMA operand order: key offset o sits at
//      position 8*((o%8)/4) + 4*(o/8) + o%4.  fp32 keeps natural order.
//   cap is a multiple of 64.
struct AttnSeg {
  const void* k;
  const void* vt;
  int n;
  int cap;
};
enum { ATTN_MAX_SEGS = 4 };  // reference | boundary | anchor | chunk
// Key-range split: nsplit > 1 makes attention() write normalised partial outputs
// opart [nsplit, nq, H*dh] and (running max of the exp2-domain logits, row sum) pairs
// ml [nsplit, nq, H, 2]
// (fp32), which attention_combine() merges into o.
// Key-range split of an attention launch: the q-tiles (ATTN_QTILE queries) from qt0 on
// are each split into nsplit contiguous parts of the key tiles, computed by separate
// workgroups into opart/ml and merged by attention_combine; q-tiles before qt0 take the
// whole key range and write o directly.  nsplit == 1: no split (qt0 ignored).
struct AttnSplit {
  int nsplit;
  int qt0;
  float* opart;
  float* ml;
};
constexpr int ATTN_QTILE = 256;
// o[nq, ldo] = softmax(q k^T / sqrt(dh)) v over the concatenated segments, per head.
// q_prescaled: q holds q * log2(e)/sqrt(dh) (as written by qknorm_rope with that
// q_scale), the form the kernels consume; otherwise the kernel scales q itself (for
// bf16 with dh = 128 that rounds the scaled q to bf16 a second time).
// norm (optional): q and k are QK-normed rows, q = q_fold * gq . q^, k = gk . k^ with
// q^, k^ RMS-normalised (gq, gk: dtype [dh]).  With q pre-scaled, the kernel then bounds
// the logits by q_fold dh max|gq| max|gk| and, when that bound is small, takes the
// softmax without a running max (same result up to rounding).
// ev (optional): a start/stop pair of timing events that the main kernel's dispatch
// stamps (hipExtLaunchKernel); the merge of split partials is not included.
struct AttnNorm {
  const void* gq;
  const void* gk;
  double q_fold;
};
enum { ATTN_SELF = 0, ATTN_CROSS = 1 };
hipError_t attention(int dtype, int dh, int H, const void* q, int ldq, void* o, int ldo, int nq,
                     int ldk, const AttnSeg* segs, int nseg, const AttnSplit& sp, bool q_prescaled,
                     hipStream_t s, int kind = ATTN_SELF, const AttnNorm* norm = nullptr,
                     const hipEvent_t* ev = nullptr);
// log2(e) / sqrt(dh): the q scale of the exp2-domain logits.
inline float attention_q_scale(int dh) { return (float)(1.4426950408889634 / __builtin_sqrt((double)dh)); }
// Whether a launch of nq queries with split sp splits any q-tile (then attention_combine
// launches its merge; with events, attention stamps only the start and the merge the end).
bool attention_splits(int nq, const AttnSplit& sp);
hipError_t attention_combine(int dtype, int dh, int H, int nq, const AttnSplit& sp, void* o, int ldo,
                             hipStream_t s, hipEvent_t stop = nullptr);
// One short key segment (1..64 keys, bf16, dh = 128): the exact softmax over one tile,
// o[nq, ldo] per head, in a kernel whose whole grid is resident at once.
bool short_attention_fits(int dtype, int dh, int nseg, const AttnSeg* segs);
hipError_t short_attention(int dh, int H, const void* q, int ldq, void* o, int ldo, int nq, const AttnSeg& seg,
                           bool q_prescaled, hipStream_t s);
// The same softmax, writing the normalised probabilities p [nq, ldp >= H*64] (bf16; head
// h's 64 key columns from h*64, keys >= n as 0) instead of O; seg.vt is not read.  With
// U_h = V_h W_o[:, h]^T per head, sum_h P_h U_h is the attention output times the output
// Linear W_o: for a short segment that product has H*64 terms per output against D.
hipError_t short_attention_probs(int dh, int H, const void* q, int ldq, void* p, int ldp, int nq,
                                 const AttnSeg& seg, bool q_prescaled, hipStream_t s);
// Split plan (nsplit, qt0; no buffers) minimising the modelled time for nq queries, H
// heads, key_tiles 64-key tiles, partial storage of partial_rows rows and `slots`
// concurrent workgroups.
AttnSplit attention_plan(int nq, int H, int key_tiles, int partial_rows, int slots);
int attention_key_tiles(const AttnSeg* segs, int nseg);
int device_cus();

// ---------------------------------------------------------------- elementwise
// out[n, D] (dtype) = RMSNorm(h) * (1 + scale) + shift  (shift/scale NULL: plain RMSNorm)
hipError_t rmsnorm_mod(int dtype, const float* h, int n, int D, const float* shift,
                       const float* scale, float eps, void* out, hipStream_t s, const hipEvent_t* ev = nullptr);

// Per-head QK-norm (+ optional 3D RoPE) and K/V repacking.
//   q_in/k_in/v_in: [n, ld_in] dtype (any may be NULL); gq/gk [dh] dtype.
//   q_out [n, D] (times q_scale), k_out [cap, D], vt_out [D, cap] (attention layout above).
//   Rows/columns in [n, round_up(n, 64)) of k_out/vt_out are zeroed.
//   rope: positions from the grid (t0 + f, y, x); rope == 0: no rotation.
hipError_t qknorm_rope(int dtype, int dh, int H, int n, const void* q_in, const void* k_in,
                       const void* v_in, int ld_in, const void* gq, const void* gk, int rope,
                       RopeGrid g, float eps, float theta, float q_scale, void* q_out,
                       void* k_out, void* vt_out, int cap, hipStream_t s);

// xin[n, c_p + c_c] (dtype) = [x rows (row_off..) || cond]; cond modes: 0 zero, 1 per-token
// [n, c_c], 2 nearest-2x upsample of [frames*(h/2)*(w/2), c_c] on grid g.
hipError_t patch_input(int dtype, const float* x, int n, int c_p, const float* cond, int c_c,
                       int cond_mode, RopeGrid g, void* xin, hipStream_t s);

// Fused patch embed (bf16 weights): out[n, N] (fp32) = [x || cond'] W^T + b, with the
// input row assembled as patch_input does (cond modes 0, 1, 2), without writing it out.
// W [N, c_p + c_c], b [N] bf16.  patch_embed_fits() tells whether the shapes qualify
// ((c_p + c_c) % 64 == 0, c_p % 8 == 0, c_c % 8 == 0, N % 256 == 0); otherwise
// patch_embed() returns hipErrorInvalidValue.
bool patch_embed_fits(int dtype, int c_p, int c_c, int N);
// Final layer with its pre-norm and the Euler step: v = (RMSNorm(h) (1 + scale) + shift)
// W^T + b with u rounded to bf16 as the GEMM operand, x += dt v, v_out (optional) = v.
// h [n, D] fp32, shift/scale [D] fp32, W [64, D] and b [64] bf16, x and v_out [n, 64]
// fp32.  final_layer_fits: the shapes it takes (bf16, c_p = 64, D in 256/512/1024/1536).
bool final_layer_fits(int dtype, int D, int c_p);
hipError_t final_layer(const float* h, int n, int D, const float* shift, const float* scale, float eps,
                       const void* W, const void* b, float dt, float* x, float* v_out, hipStream_t s,
                       const hipEvent_t* ev = nullptr);
hipError_t patch_embed(const float* x, int n, int c_p, const float* cond, int c_c, int cond_mode,
                       RopeGrid g, const void* W, const void* bias, float* out, int N, hipStream_t s);

// x[i] += dt * v[i]
hipError_t euler(float* x, const float* v, float dt, long long n, hipStream_t s);
// x = a z + b e over n fp32 elements (16-byte aligned pointers).
hipError_t noise_to(float* x, const float* z, const float* e, float a, float b, long long n, hipStream_t s);

// Boundary by reuse: keys [first, first + n) of a chunk's K [*, H*dh] and V^T
// [H*dh, cap_src] (layouts of qknorm_rope) become keys [0, n) of a boundary segment
// (kb [cap_dst, H*dh], vtb [H*dh, cap_dst]), K's time-axis RoPE pairs turned by dt;
// keys [n, round_up(n, 64)) are zeroed.
hipError_t boundary_reuse(int dtype, int dh, int H, const void* kc, const void* vtc, int cap_src, int first,
                          int n, float dt, float theta, void* kb, void* vtb, int cap_dst, hipStream_t s);

// Timestep conditioning c = SiLU(W2 SiLU(W1 phi(t) + b1) + b2) and per-block modulation
// mod[l] = Wmod_l c + bmod_l ([6D]) for l < L (L may be 0) and final fmod = Wf c + bf
// ([2D]).  tmp: fp32 scratch of 256 + 2 D floats; c is left in tmp[256 + D, 256 + 2 D).
hipError_t modulation(int dtype, int D, int L, double t, const void* t1w, const void* t1b,
                      const void* t2w, const void* t2b, const void* const* modw,
                      const void* const* modb, const void* fmodw, const void* fmodb, float* tmp,
                      float* mod_out, float* fmod_out, hipStream_t s);
// Head-block-diagonal copy of v [M, D] (dtype, heads of dh columns): out [H*64, D] with
// row h*64 + k = v row k restricted to head h's columns (other columns 0), rows k >= M 0.
// Requires M <= 64 and D % 8 == 0.
hipError_t head_blockdiag(int dtype, const void* v, int M, int D, int dh, void* out, hipStream_t s);
// One block's modulation out[6D] = Wmod c + bmod (W [6D, D] dtype, c [D] fp32).
hipError_t block_modulation(int dtype, int D, const void* w, const void* b, const float* c, float* out,
                            hipStream_t s);
// The same products for up to MOD_BATCH timesteps at once, each weight row read once
// for all of them; per timestep the arithmetic (and so the result, bit for bit) is that
// of modulation / block_modulation.
constexpr int MOD_BATCH = 16;
// c[j] ([D], rows D apart) for t[j], j < nt.  tmp: fp32 scratch of MOD_BATCH (256 + D).
hipError_t timestep_cond_batch(int dtype, int D, const double* t, int nt, const void* t1w, const void* t1b,
                               const void* t2w, const void* t2b, float* tmp, float* c, hipStream_t s);
// y[j][r] = W[r, :] . x[j] + b[r] for r < R, j < nt (x[j] at x + j ldx, y[j] at y + j ldy).
hipError_t gemv_batch(int dtype, int R, int K, const void* w, const void* b, const float* x, int ldx, int nt,
                      float* y, int ldy, hipStream_t s);

}  // namespace dit
