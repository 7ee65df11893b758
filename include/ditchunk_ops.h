/*
 * ditchunk_ops.h: kernel-level entry points of libditchunk.
 *
 * These expose the individual kernels that dit_chunk_step chains, so that each can be
 * checked against its definition and timed on its own.  Conventions as in ditchunk.h:
 *   - device pointers, dtype DIT_F32 or DIT_BF16 for "dtype" buffers, fp32 where stated;
 *   - asynchronous on the given hipStream_t (NULL: default stream);
 *   - arguments are validated on the host before any launch; failures return a
 *     negative DIT_E* code and set dit_last_error();
 *   - a call with zero rows (M, n or nq == 0) is validated like any other, then
 *     returns 0 without a launch; its row buffers (A, h, out, q, o, p, x, xin, cond)
 *     may then be NULL.  Weights, keys and the other arguments are still checked.
 * Linear weights are [out, in] row-major with a bias [out].
 */
#ifndef DITCHUNK_OPS_H
#define DITCHUNK_OPS_H

#include "ditchunk.h"

#ifdef __cplusplus
extern "C" {
#endif

enum { DITK_ACT_NONE = 0, DITK_ACT_GELU = 1, DITK_OUT_F32 = 2 };

/* out[M, N] = act(A W^T + b): A [M, K], W [N, K], b [N] (dtype).  act DITK_ACT_NONE
 * or DITK_ACT_GELU (tanh form) store dtype; DITK_OUT_F32 stores fp32 without
 * activation.  The Linear layers of the DiT block (QKV, cross q/k/v, FC1, patch embed).
 * K must be a multiple of 64; N a multiple of 4; A [M, K] and W [N, K] must each hold
 * fewer than 2^31 elements (32-bit operand offsets); DIT_ESHAPE otherwise. */
int ditk_linear(int dtype, const void* A, const void* W, const void* b, int M, int N, int K,
                int act, void* out, void* hip_stream);

/* h[M, N] (fp32) += gate[N] (.) (A W^T + b); gate fp32, NULL means 1.  The gated
 * residual of the adaLN DiT block (out-proj, cross out-proj, FC2).  workspace (fp32
 * device memory of workspace_floats floats, or NULL with 0): when given, a bf16 launch
 * whose large-tile grid would leave most of the chip idle (the context passes' MLP-out
 * Linear, K >= 4096) splits its K range into 2-4 parts computed by separate
 * workgroups and sums them in a second pass (needs parts x M x N floats; with less
 * workspace it is not split). */
int ditk_linear_residual(int dtype, const void* A, const void* W, const void* b, const float* gate,
                         int M, int N, int K, float* h, float* workspace, long long workspace_floats,
                         void* hip_stream);

/* out[n, D] (dtype) = RMSNorm(h) (.) (1 + scale) + shift, h fp32 [n, D], shift/scale fp32
 * [D] (both NULL: plain RMSNorm).  D a multiple of 256, <= 4096. */
int ditk_rmsnorm_modulate(int dtype, const float* h, int n, int D, const float* shift,
                          const float* scale, double eps, void* out, void* hip_stream);

/* Per-head QK-RMSNorm with gamma [dh] (dtype), 3D RoPE (rope != 0) at positions
 * (grid.t0 + f, y, x) of token f*h*w + y*w + x, and repacking into the attention layout:
 *   q_out  [n, H*dh]              q_scale times the normalised, rotated q (only if q_in);
 *                                 q_scale = log2(e)/sqrt(dh) gives the pre-scaled q that
 *                                 ditk_attention takes with q_prescaled != 0
 *   k_out  [cap, H*dh]            (rows n..round_up(n,64)-1 zeroed; only if k_in)
 *   vt_out [H*dh, cap]            V transposed (only if v_in); for bf16 the keys of each
 *                                 aligned group of 16 are stored so that key offset o
 *                                 sits at position 8*((o%8)/4) + 4*(o/8) + o%4; fp32
 *                                 keeps natural order; columns n..round_up(n,64)-1 zeroed.
 * q_in/k_in/v_in: [n, ld_in] (dtype), any may be NULL.  cap a multiple of 64, >= n. */
int ditk_qknorm_rope(int dtype, int dh, int H, int n, const void* q_in, const void* k_in,
                     const void* v_in, int ld_in, const void* gq, const void* gk, int rope,
                     dit_grid grid, double eps, double theta, double q_scale, void* q_out,
                     void* k_out, void* vt_out, int cap, void* hip_stream);

/* o[nq, H*dh] = softmax(q k^T / sqrt(dh)) v per head, keys the concatenation of nseg
 * (1..4) segments given in the layout of ditk_qknorm_rope (k[i] [cap[i], H*dh],
 * vt[i] [H*dh, cap[i]], n[i] valid keys; each V^T must be under 2^31 bytes, DIT_ESHAPE
 * otherwise).  q [nq, H*dh] (dtype).  fp32 needs dh = 64.
 * nsplit (1..8) splits the key tiles into contiguous parts computed by separate
 * workgroups and merged afterwards; nsplit > 1 needs partial: fp32 scratch of
 * nsplit * nq * (H*dh + 2*H) floats (NULL allowed when nothing is split).
 * unsplit_rows: queries [0, unsplit_rows) are not split (each 256-query tile takes the
 * whole key range in one workgroup); the split applies from there on.  It must be a
 * multiple of 256 or >= nq (then nothing is split); 0 splits every query (DIT_EINVAL
 * otherwise).
 * q_prescaled != 0: q holds q * log2(e)/sqrt(dh) (ditk_qknorm_rope with that q_scale;
 * the softmax is then taken in base 2 on q k^T directly).  q_prescaled == 0: plain q,
 * scaled inside the kernel (for bf16 with dh = 128 this rounds the scaled q to bf16
 * once more, i.e. slightly less accurate than the pre-scaled form).
 * gq, gk (dtype [dh], both or neither): q and k are QK-normed rows, q = q_fold gq . q^
 * and k = gk . k^ with q^, k^ RMS-normalised (ditk_qknorm_rope with q_scale q_fold and
 * 1).  With q pre-scaled, every exp2-domain logit is then at most q_fold dh max|gq|
 * max|gk| in magnitude; when that is small the kernel computes the softmax weights as
 * 2^s without a running max (the common factor cancels; same result up to rounding).
 * The caller guarantees the normalisation: for other q, k pass NULL.
 * One segment of 1..64 keys with bf16, dh = 128 and nsplit = 1 (the audio
 * cross-attention's shape) runs a single-tile kernel with the exact softmax. */
int ditk_attention(int dtype, int dh, int H, const void* q, int nq, int nseg,
                   const void* const* k, const void* const* vt, const int* n, const int* cap,
                   int nsplit, float* partial, int unsplit_rows, int q_prescaled, const void* gq,
                   const void* gk, double q_fold, void* o, void* hip_stream);

/* Allocation-free ditk_attention, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * arguments and results as ditk_attention, without `partial`; the key-range split's
 * partials live in a device array of the library, DITK_NOALLOC_SCRATCH_BYTES (64 MiB)
 * per GPU, held until the process ends.  The call allocates and frees nothing.
 *   - A split (nsplit > 1 with rows to split) needs nsplit * nq * (H*dh + 2*H) floats of
 *     that array: more is DIT_EWORKSPACE (checked before any HIP call).
 *   - The array used is the one of the calling thread's current device, whose address is
 *     looked up on the first call on that device; hip_stream must belong to that device.
 *   - Every call on one GPU shares the array, which keeps the last call's contents (each
 *     call writes every partial it reads): calls that can overlap on one GPU (other
 *     streams, other threads) race; serialise them.
 * Errors: those of ditk_attention, EWORKSPACE, EHIP (symbol lookup failed). */
#define DITK_NOALLOC_SCRATCH_BYTES (64LL << 20)
int ditk_attention_noalloc(int dtype, int dh, int H, const void* q, int nq, int nseg,
                           const void* const* k, const void* const* vt, const int* n, const int* cap,
                           int nsplit, int unsplit_rows, int q_prescaled, const void* gq, const void* gk,
                           double q_fold, void* o, void* hip_stream);

/* The softmax probabilities of one short key segment (bf16, dh = 128, 1..64 keys; the
 * audio cross-attention's shape): p [nq, H*64] (bf16), head h's 64 key columns from
 * h*64, p[i, h*64 + j] = softmax_j(q_i k_j / sqrt(dh)) for j < n and 0 for n <= j < 64.
 * q [nq, H*128] (q_prescaled as in ditk_attention), k [cap, H*128] in the layout of
 * ditk_qknorm_rope (rows >= n zero).  With U_h = V_h W_o[:, head h]^T this gives the
 * attention output already multiplied by the output Linear W_o as sum_h P_h U_h, a
 * product of H*64 terms per output instead of D (HeyGen, "Avatar inference at scale",
 * section "The underlying model architecture": the audio conditioning; folding the
 * output Linear into the values is this library's reading).
 * Errors: EINVAL (NULL pointer), ESHAPE (n outside 1..64, cap < 64 or not a multiple
 * of 64, H < 1, nq < 0). */
int ditk_attention_probs(int H, const void* q, int nq, const void* k, int n, int cap, int q_prescaled,
                         void* p, void* hip_stream);

/* Timestep conditioning and adaLN modulation for timestep t, from the weight table of
 * ditchunk.h: mod_out [L, 6, D] (fp32: shift_msa, scale_msa, gate_msa, shift_mlp,
 * scale_mlp, gate_mlp), fmod_out [2, D] (fp32: shift, scale).  tmp: fp32 scratch of
 * 256 + 2 D floats. */
int ditk_modulation(int dtype, int D, int L, double t, const void* const* weights,
                    float* mod_out, float* fmod_out, float* tmp, void* hip_stream);

/* xin[n, c_p + c_c] (dtype) = [x || cond]: cond_mode 0 zeros, 1 cond [n, c_c],
 * 2 nearest-2x upsample of cond [frames*(h/2)*(w/2), c_c] on the token grid. */
int ditk_patch_input(int dtype, const float* x, int n, int c_p, const float* cond, int c_c,
                     int cond_mode, dit_grid grid, void* xin, void* hip_stream);

/* Patch embed with the input rows assembled inside the GEMM's operand loads (bf16
 * weights): out[n, D] (fp32) = [x || cond'] W^T + b, cond' as in ditk_patch_input
 * (cond_mode 0 zeros, 1 cond [n, c_c], 2 the nearest-2x upsample of a half-resolution
 * cond: the super-resolution stage refines the low-resolution latents, HeyGen, "Avatar
 * inference at scale", section "The underlying model architecture"; how they enter
 * the model is not given, and channel concatenation of the upsampled latent is this
 * library's reading).  x [n, c_p] and cond fp32;
 * W [D, c_p + c_c] and b [D] bf16.  Needs (c_p + c_c) % 64 == 0, c_p % 8 == 0,
 * c_c % 8 == 0 and D % 256 == 0 (else DIT_ESHAPE); mode 2 needs an even grid with
 * frames * h * w == n.  This is the patch embed dit_chunk_step runs for bf16. */
int ditk_patch_embed(const float* x, int n, int c_p, const float* cond, int c_c, int cond_mode,
                     dit_grid grid, const void* w, const void* b, float* out, int D,
                     void* hip_stream);

/* Measured ceilings for the roofline figures (the spec peaks assume clocks and power a
 * real workload may not get):
 * ditk_probe_mfma: a dense bf16 MFMA loop, no memory traffic, 2 workgroups of 4 waves per
 *   CU on 256 CUs' worth of workgroups (512), each wave alternating two operand sets with
 *   unrelated bit patterns over independent accumulators for `iters` iterations.
 *   data: 4096 bytes of bf16 (device; random values give realistic operand toggling);
 *   sink: DITK_PROBE_SINK_FLOATS floats (device, written); *flop (host): the MFMA flop
 *   the launch performs.  Time it on the stream to get the sustained MFMA rate.
 * ditk_probe_copy: dst[0, bytes) = src[0, bytes), a plain grid-stride 16-byte copy
 *   (bytes a multiple of 16, both 16-byte aligned); with a buffer far larger than the
 *   caches it measures sustained HBM bandwidth (2 x bytes moved), and with a known size
 *   it calibrates the HBM traffic counters.
 * Errors: EINVAL (NULL, iters < 1, bad size or alignment), EWORKSPACE (sink too small),
 * EHIP. */
#define DITK_PROBE_SINK_FLOATS (512 * 256)
int ditk_probe_mfma(const void* data, int iters, float* sink, long long sink_floats, double* flop,
                    void* hip_stream);
int ditk_probe_copy(const void* src, void* dst, long long bytes, void* hip_stream);

#ifdef __cplusplus
}
#endif
#endif /* DITCHUNK_OPS_H */
