/*
 * ditchunk.h: C ABI of the chunked streaming DiT denoising step (MI355X, gfx950).
 *
 * What it computes.  HeyGen, "Avatar inference at scale":
 *   - "The underlying model architecture": the generator is a diffusion
 *     transformer trained with flow matching.  It is conditioned on rich
 *     reference tokens, not on a compressed identity embedding.  Long videos are
 *     made chunk by chunk: the first chunk relies on the static reference only,
 *     and later chunks on boundary data from the previous segment.
 *   - "The streaming framework and pipeline loop": the reference identity is
 *     encoded once per request.  The audio-to-video stage then runs a multi-step
 *     diffusion pass per chunk, conditioned on the previous chunk's boundary
 *     frames.
 *   - "Constant memory over duration": only the static reference conditioning
 *     and a minimal set of anchor tensors persist between chunks, so peak memory
 *     follows the chunk size, not the session length.
 * Hence the call cadence:
 *   ref_kv_precompute   once per request;
 *   boundary_kv_carry   once per chunk (a zero-frame grid clears it for chunk 0);
 *   interp_anchor_kv    once per interpolation chunk (see below; cleared for
 *                       ordinary chunks);
 *   audio_kv_precompute once per chunk: the audio K/V of every block, which the
 *                       chunk's steps then reuse;
 *   dit_modulation_table  once per request: the adaLN vectors of every timestep of
 *                       the schedule (and t = 0), which the passes then reuse;
 *   dit_chunk_step      once per denoising step: v = DiT(x, t), x += (t_next - t) v;
 *   dit_chunk_step_carry  alternatively the chunk's last step, which also leaves
 *                       that step's last-frame K/V as the next boundary;
 *   fm_euler_step       the bare Euler update, for callers with their own velocity;
 *   fm_noise_to         a point of the flow-matching path (frames held at known
 *                       latents, e.g. interpolation anchors inside the chunk's window).
 *
 * The block (readings of the pages, which give no internals): tokens are
 * patchified latents [N, c_p] (fp32).  A patch-embed Linear feeds L blocks.
 * Each block runs:
 *   - RMSNorm + adaLN shift/scale, QKV, per-head QK-RMSNorm with gamma, and a 3D
 *     RoPE over (t, y, x);
 *   - self-attention whose keys are [reference K | boundary K | anchor K | chunk K]
 *     (boundary and anchor when held);
 *   - a gated residual;
 *   - RMSNorm, audio cross-attention (q and k per-head normed), and a residual;
 *   - RMSNorm + adaLN, a GELU(tanh) MLP and a gated residual.
 * A final RMSNorm + adaLN and a Linear give v [N, c_p].  Context tokens
 * (reference, boundary, anchor) pass through the same blocks at t = 0: the
 * reference sees only itself, the boundary sees the reference and itself, and the
 * anchor sees the reference, the boundary and itself.  Their
 * per-block K (normed, rotated) and V are kept resident, read-only, in the
 * caller's state buffer.
 *
 * Ownership.  The caller owns ALL device memory:
 *   - weights, state (dit_state_bytes), workspace (dit_workspace_bytes), and every
 *     input and output buffer;
 *   - the library borrows pointers and allocates nothing on the device.
 * Every call is asynchronous on the handle's HIP stream.  A handle is not
 * thread-safe; separate handles are independent.
 *
 * Errors.  Every int-returning call returns DIT_OK (0) or a negative code.
 * Arguments and state are checked on the host before any HIP call; a failed
 * check launches nothing and changes no state.  dit_last_error() gives a
 * thread-local message for the last failure on the calling thread.
 */
#ifndef DITCHUNK_H
#define DITCHUNK_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  DIT_OK = 0,
  DIT_EINVAL = -1,     /* null pointer, bad enum, non-finite t, inconsistent config */
  DIT_ESHAPE = -2,     /* a size above the capacity fixed at create, or a bad grid  */
  DIT_ESTATE = -3,     /* call order: e.g. a step before ref_kv_precompute          */
  DIT_EWORKSPACE = -4, /* state or workspace smaller than required                  */
  DIT_EHIP = -5        /* a HIP runtime call failed                                 */
};

enum { DIT_F32 = 0, DIT_BF16 = 1 };

typedef struct dit_config {
  int L;          /* DiT blocks                                                     */
  int D;          /* hidden size; D == H * dh                                       */
  int H;          /* heads                                                          */
  int dh;         /* head dim: 64 or 128                                            */
  int mlp_ratio;  /* MLP width = mlp_ratio * D                                      */
  int c_p;        /* latent channels per token (x, v): 64                           */
  int c_c;        /* conditioning channels concatenated after x (0: none); c_p+c_c
                     must be a multiple of 64                                       */
  int cond_up;    /* 1: cond is per token [N, c_c]; 2: cond is given at half (h, w)
                     resolution [frames*(h/2)*(w/2), c_c] with (c, dy, dx) channel
                     layout and is nearest-upsampled 2x                             */
  int d_a;        /* audio feature dim (0: no audio cross-attention weights)        */
  int dtype;      /* DIT_F32 or DIT_BF16: weights, activations and K/V              */
  int max_tokens; /* capacity: chunk tokens N                                       */
  int max_ref;    /* capacity: reference tokens                                     */
  int max_bnd;    /* capacity: boundary tokens (one latent frame)                   */
  int max_audio;  /* capacity: audio tokens M                                       */
  double eps;     /* RMSNorm epsilon (1e-6)                                         */
  double rope_theta; /* RoPE base (10000)                                           */
} dit_config;

/* Token grid: frames x h x w tokens, row-major over (frame, y, x).  Token (f, y, x)
 * takes RoPE position (t0 + f, y, x). */
typedef struct dit_grid {
  int t0, frames, h, w;
} dit_grid;

typedef struct dit_handle dit_handle;

/* Weight table order.  Every pointer is device memory in the config's dtype.
 * Linear weights are [out, in] row-major (input-contiguous) with a bias [out].
 * Global entries come first; then block l's entries start at
 * DIT_W_GLOBAL_COUNT + l * DIT_W_BLOCK_COUNT.  Cross-attention entries
 * (DIT_WB_CQ_W .. DIT_WB_CO_B) may be NULL when d_a == 0. */
enum {
  DIT_W_PE_W = 0,   /* [D, c_p + c_c] patch embed                                    */
  DIT_W_PE_B,       /* [D]                                                           */
  DIT_W_T1_W,       /* [D, 256] timestep MLP layer 1 (input: sinusoid of 1000 t)     */
  DIT_W_T1_B,
  DIT_W_T2_W,       /* [D, D] timestep MLP layer 2                                   */
  DIT_W_T2_B,
  DIT_W_FMOD_W,     /* [2D, D] final adaLN (shift, scale)                            */
  DIT_W_FMOD_B,
  DIT_W_FIN_W,      /* [c_p, D] final Linear                                         */
  DIT_W_FIN_B,
  DIT_W_GLOBAL_COUNT
};
enum {
  DIT_WB_MOD_W = 0, /* [6D, D] adaLN: shift_msa, scale_msa, gate_msa, shift_mlp,
                       scale_mlp, gate_mlp                                           */
  DIT_WB_MOD_B,
  DIT_WB_QKV_W,     /* [3D, D] q | k | v, heads contiguous within each               */
  DIT_WB_QKV_B,
  DIT_WB_GQ,        /* [dh] QK-norm gamma for q                                      */
  DIT_WB_GK,        /* [dh] QK-norm gamma for k                                      */
  DIT_WB_O_W,       /* [D, D]                                                        */
  DIT_WB_O_B,
  DIT_WB_CQ_W,      /* [D, D] cross-attention query                                  */
  DIT_WB_CQ_B,
  DIT_WB_CK_W,      /* [D, d_a] cross-attention key                                  */
  DIT_WB_CK_B,
  DIT_WB_CV_W,      /* [D, d_a] cross-attention value                                */
  DIT_WB_CV_B,
  DIT_WB_GCQ,       /* [dh]                                                          */
  DIT_WB_GCK,       /* [dh]                                                          */
  DIT_WB_CO_W,      /* [D, D] cross-attention output                                 */
  DIT_WB_CO_B,
  DIT_WB_FC1_W,     /* [mlp_ratio*D, D]                                              */
  DIT_WB_FC1_B,
  DIT_WB_FC2_W,     /* [D, mlp_ratio*D]                                              */
  DIT_WB_FC2_B,
  DIT_W_BLOCK_COUNT
};

/* Number of entries of the weight table for this config (0 if the config is invalid). */
int dit_weight_count(const dit_config* cfg);

/* Capacity limit (checked with the config): the kernels address activation and V^T
 * buffers with 32-bit offsets, so the token capacity cap = max(max_tokens, max_ref,
 * max_bnd) rounded up to 64 must keep [cap, max(3 D, mlp_ratio D)] under 2^31 elements
 * and [D, cap] of the dtype under 2^31 bytes (e.g. cap < 174763 at D = 3072, mlp_ratio 4);
 * a larger config is invalid (DIT_EINVAL from dit_create, 0 from the size queries).
 *
 * Bytes of the resident state: per block, K and V of max_ref reference tokens, of
 * max_bnd boundary tokens, of max_bnd interpolation-anchor tokens and (d_a > 0) of
 * max_audio audio tokens (each rounded up to 64 tokens); (d_a > 0) the held audio
 * features [max_audio rounded up to 64, d_a]; for bf16 with dh = 128 and max_audio <= 64
 * per block the audio values folded into the cross-attention's output Linear
 * (D x H*64, see ditk_attention_probs); and the modulation table
 * (DIT_MOD_TABLE_MAX entries of (6 L + 2) D floats).  0 if the config is invalid (see
 * dit_last_error). */
size_t dit_state_bytes(const dit_config* cfg);

/* Bytes of per-call transients (activations of max(max_tokens, max_ref, max_bnd)
 * tokens, audio K/V, attention partials).  0 if the config is invalid. */
size_t dit_workspace_bytes(const dit_config* cfg);

/* Create a handle.  weights: host array of dit_weight_count(cfg) device
 * pointers (borrowed, must outlive the handle).  state/workspace: device
 * buffers of at least the reported sizes, 256-byte aligned (borrowed).
 * hip_stream: hipStream_t for every launch (NULL: the default stream).  No HIP
 * call is made.  The new handle holds no reference and no boundary. */
int dit_create(const dit_config* cfg, const void* const* weights, void* state,
               size_t state_bytes, void* workspace, size_t workspace_bytes,
               void* hip_stream, dit_handle** out);

/* Destroy a handle (NULL is allowed).  Does not synchronise the handle's stream; waits
 * for the weight-streaming copies it has enqueued (dit_weight_stream). */
int dit_destroy(dit_handle* h);

/* Per-block weight streaming: the single-GPU part of lazily unsharding a model block by
 * block from pinned host memory, with the transfer of the next blocks overlapped with
 * the compute of the current one (HeyGen, "Avatar inference at scale", section "Load and
 * offload phases within the pipeline").
 *
 * dit_block_weight_bytes: bytes of one block slot, i.e. the block entries of the weight
 * table (DIT_WB_*) in table order, each starting at a 256-byte aligned offset; absent
 * cross-attention entries (d_a == 0) take no space.  0 if the config is invalid.
 *
 * dit_weight_stream(h, host_blocks, ring, ring_bytes, nslot) switches the handle's
 * block weights to streaming:
 *   - host_blocks: host array of L * DIT_W_BLOCK_COUNT pointers (block l's entries at
 *     l * DIT_W_BLOCK_COUNT, shapes and dtype as in the weight table) to pinned host
 *     memory (hipHostMalloc); borrowed, contents must not change while streaming is on;
 *   - ring: device buffer of at least nslot * dit_block_weight_bytes(cfg) bytes,
 *     256-byte aligned, borrowed; 1 <= nslot <= L.
 * Every pass (reference, boundary, anchor, denoising step) uses blocks 0..L-1 in turn;
 * use u reads slot u % nslot.  The copy of the block needed nslot uses later is issued
 * on the handle's own copy stream as soon as use u's kernels have been enqueued, and
 * runs once they have finished; block kernels wait for their slot's copy.  So with
 * nslot >= 2 the next blocks (also the first ones of the next pass) transfer while the
 * current block computes; with nslot == L every block is copied once and stays.  The
 * global weight entries stay as given to dit_create, and results equal those of the
 * resident table bit for bit.
 * The call itself starts copying the first nslot blocks at once, on the copy stream,
 * without waiting for the handle's stream, so enabling streaming while earlier passes
 * still run (on the resident weights, or another model) overlaps the transfer with
 * them; the ring's memory must therefore not be read or written by any work still
 * enqueued (on any stream) when the call is made, e.g. a ring freshly taken from a
 * stream-ordered allocator is safe only after that allocator's pending work is done.
 * dit_weight_stream(h, NULL, NULL, 0, 0) switches back to the table of dit_create.
 * Before freeing the ring or the host memory, synchronise the device (the copies run
 * on the library's stream).  After a call that failed with DIT_EHIP the next pass
 * copies every block again.
 * Errors: EINVAL (null handle, nslot out of range, misaligned ring, a NULL host entry
 * that is not an absent cross-attention entry), EWORKSPACE (ring too small), EHIP. */
size_t dit_block_weight_bytes(const dit_config* cfg);
int dit_weight_stream(dit_handle* h, const void* const* host_blocks, void* ring, size_t ring_bytes,
                      int nslot);

/* Reference K/V: run the reference latent tokens ref [grid.frames*grid.h*grid.w,
 * c_p] (fp32, device) through all blocks at t = 0, each token at position
 * (grid.t0 + f, y, x), attending only to the reference, and store every block's
 * K and V in the state.  Once per request.  Clears any boundary and anchor.
 * Errors: EINVAL (null), ESHAPE (more than max_ref tokens, empty grid). */
int ref_kv_precompute(dit_handle* h, const float* ref, dit_grid grid);

/* Boundary K/V: take the last frame (frame prev.frames-1, h*w tokens) of the
 * previous chunk's final latent x_prev [prev.frames*prev.h*prev.w, c_p] (fp32,
 * device), run it through all blocks at t = 0 at positions (-1, y, x),
 * attending to the reference and itself, and store its K and V in the state.
 * prev.frames == 0 clears the boundary (first chunk: reference only).
 * Errors: EINVAL (null x_prev with frames > 0), ESHAPE (h*w > max_bnd),
 * ESTATE (no reference yet). */
int boundary_kv_carry(dit_handle* h, const float* x_prev, dit_grid prev);

/* Interpolation anchor K/V (HeyGen, "Avatar inference at scale", section "Boundary
 * continuity and chunk consistency": ordinary N-chunks make the timeline, and an
 * interpolation chunk between N_k and N_k+1, generated after both, smooths the
 * transition anchored on the final frame of N_k and one of the first frames of N_k+1;
 * the order is N0, N1, I0, N2, I1, ...).  Reading: both anchors are context
 * segments.  The boundary (boundary_kv_carry on N_k's final latent) is the first;
 * this call makes the second from frame 0 (h*w tokens) of N_k+1's final latent
 * x_next [next.frames*next.h*next.w, c_p] (fp32, device), run through all blocks at
 * t = 0 at positions (t_pos, y, x), usually t_pos = the interpolation chunk's frame
 * count, attending to the reference, the boundary (if held) and itself.  Anchors
 * are never denoised, so they yield no predictions to discard.  Until cleared,
 * dit_chunk_step attends to [reference | boundary | anchor | chunk].
 * next.frames == 0 clears the anchor; boundary_kv_carry and ref_kv_precompute also
 * clear it (its K/V depend on the boundary).
 * Errors: EINVAL (null x_next with frames > 0), ESHAPE (h*w > max_bnd),
 * ESTATE (no reference yet). */
int interp_anchor_kv(dit_handle* h, const float* x_next, dit_grid next, int t_pos);

/* Audio K/V, once per chunk: the chunk's audio features are the same at every
 * denoising step, so their cross-attention keys and values (per block: the K and V
 * Linears of audio [M, d_a] (fp32, device), K per-head normed) are computed once and
 * held in the state.  dit_chunk_step with audio NULL and M == DIT_AUDIO_HELD then
 * attends to them.  M == 0 (audio NULL) clears them.  The step's output is the same,
 * bit for bit, as when the audio is passed to every step.  While block weights stream
 * (dit_weight_stream) the features are held and each block's K/V is computed when the
 * next pass (any pass: step, context or modulation table) brings that block's weights
 * into the ring, so the audio adds no pass over the weights of its own.
 * Errors: EINVAL (null audio with M > 0, d_a == 0), ESHAPE (M > max_audio). */
enum { DIT_AUDIO_HELD = -1 };
int audio_kv_precompute(dit_handle* h, const float* audio, int M);

/* The modulation table of a schedule.  The adaLN vectors (per block shift, scale and
 * gate of the attention and MLP sublayers, and the final layer's shift and scale) depend
 * only on the timestep and the weights (HeyGen, "Avatar inference at scale", section
 * "The underlying model architecture" names the DiT; its conditioning is this library's
 * reading), so the table is computed once for the timesteps t[0..nt) of a request's
 * schedule (host array; t = 0 serves the context passes) and held in the state: each
 * weight row is read once for all nt timesteps instead of once per step.  Every later
 * pass whose timestep equals some t[j] exactly uses entry j; other timesteps are
 * computed per pass as before.  The results are the same, bit for bit.  nt == 0 clears
 * the table.  Errors: EINVAL (nt outside [0, DIT_MOD_TABLE_MAX], t NULL with nt > 0, a
 * non-finite t); on an error the table is unchanged, except that a HIP failure leaves
 * it cleared. */
enum { DIT_MOD_TABLE_MAX = 16 };
int dit_modulation_table(dit_handle* h, const double* t, int nt);

/* One denoising step of the chunk: v = DiT(x, t) and x += (t_next - t) v,
 * with dt computed in double on the host and applied in fp32.
 *   x     [N, c_p] fp32, device, updated in place; N = frames*h*w of chunk;
 *         token (f, y, x) at position (chunk.t0 + f, y, x).
 *   cond  fp32 conditioning (c_c > 0): [N, c_c] if cond_up == 1, else
 *         [frames*(h/2)*(w/2), c_c]; must be NULL when c_c == 0.
 *   audio [M, d_a] fp32 audio features (M == 0 or d_a == 0: no cross-attention);
 *         or audio NULL with M == DIT_AUDIO_HELD: the audio K/V held by
 *         audio_kv_precompute.
 *   v_out optional [N, c_p] fp32 copy of the velocity (NULL: not written).
 * Errors: EINVAL (null x, non-finite t/t_next, cond/audio mismatch), ESHAPE
 * (N > max_tokens, M > max_audio, odd h or w with cond_up == 2),
 * ESTATE (no reference yet; DIT_AUDIO_HELD with no audio held). */
int dit_chunk_step(dit_handle* h, float* x, const float* cond, const float* audio, int M,
                   dit_grid chunk, double t, double t_next, float* v_out);

/* The last denoising step of a chunk, with the boundary carried by reuse: the same
 * step as dit_chunk_step, and, block by block right after that block's
 * self-attention, the per-block K and V that this step forms for the chunk's last
 * frame (frame chunk.frames-1, h*w tokens) replace the boundary K/V, K turned from
 * t = chunk.t0 + frames - 1 to t = -1 (a rotation of the RoPE time pairs; rotations
 * about the same axis add).  The next chunk then needs no boundary_kv_carry pass.
 * Any anchor is cleared.  This is the alternative to boundary_kv_carry's clean t = 0
 * pass (HeyGen, "Avatar inference at scale": the boundary data of the previous segment
 * condition the next chunk, section "The underlying model architecture"; the pages do
 * not say how it is formed): the K/V come from the final step's input latent and
 * timestep instead, at the cost of a K/V copy instead of a forward pass.
 * Errors: as dit_chunk_step, and ESHAPE if h*w > max_bnd. */
int dit_chunk_step_carry(dit_handle* h, float* x, const float* cond, const float* audio, int M,
                         dit_grid chunk, double t, double t_next, float* v_out);

/* x[i] += (float)dt * v[i] for i < n (fp32, device) on hip_stream.
 * Errors: EINVAL (null pointer with n > 0, non-finite dt, n < 0). */
int fm_euler_step(float* x, const float* v, double dt, long long n, void* hip_stream);

/* x[i] = (float)(1 - t) * z[i] + (float)t * eps[i] for i < n (fp32, device) on hip_stream:
 * the point at time t of the flow-matching path from data z (t = 0) to noise eps (t = 1)
 * (HeyGen, "Avatar inference at scale": the generator is trained with flow matching,
 * section "The underlying model architecture").  It holds frames at known latents
 * during a pass, as the window reading of the interpolation anchors does: before every
 * step of an I-chunk whose window is [earlier N-chunk's last frame | F new frames |
 * later N-chunk's first frame] (grid t0 = -1, F + 2 frames, reference context only),
 * the two anchor frames are set to their latents at the step's t; the anchors'
 * predictions are dropped at the end (section "Boundary continuity and chunk
 * consistency").  x may alias z or eps.  Pointers 16-byte aligned.
 * Errors: EINVAL (null pointer with n > 0, misalignment, non-finite t, n < 0). */
int fm_noise_to(float* x, const float* z, const float* eps, double t, long long n, void* hip_stream);

/* Message of the last failure on this thread ("" if none). */
const char* dit_last_error(void);

/* Kernel timing on the handle's stream.  While a kind is enabled, each of its launches is
 * timed by a pair of HIP events that the dispatches themselves stamp with the kernels'
 * start and end (hipExtLaunchKernel: no marker packets between launches), at most 4096
 * pairs per window:
 *   DIT_TIME_ATTN  the self-attention of every pass (dit_chunk_step, ref_kv_precompute,
 *                  boundary_kv_carry, interp_anchor_kv), from the start of the main
 *                  kernel to the end of the merge of its key-range parts when the launch
 *                  is split; work = the method's 4 n_q n_kv D flop;
 *   DIT_TIME_GEMM  the Linears of the blocks (QKV with its QK-norm/RoPE epilogue,
 *                  out-projection, cross-attention q and out, MLP in and out, each with
 *                  its fused epilogue); work = 2 M N K flop;
 *   DIT_TIME_ELEM  the RMSNorm (+ adaLN) passes and the final layer (norm, Linear and
 *                  Euler update); work = the bytes they must move (fp32 h read, their
 *                  outputs written, x read and written, weights and vectors).
 * dit_timing_enable(h, mask): bit k of mask enables kind k (1: self-attention only; 0:
 * none) and opens a new window; it creates the events (once per kind), so a timed region
 * that follows does not include their creation.
 * dit_timing_read(h, kind, ...) synchronises that kind's events and returns its launch
 * count, summed milliseconds and summed work, then opens a new window for that kind.
 * Errors: EINVAL (NULL handle or output, mask or kind out of range), EHIP. */
enum { DIT_TIME_ATTN = 0, DIT_TIME_GEMM = 1, DIT_TIME_ELEM = 2, DIT_TIME_KINDS };
int dit_timing_enable(dit_handle* h, int enable);
int dit_timing_read(dit_handle* h, int kind, int* count, double* total_ms, double* total_work);

#ifdef __cplusplus
}
#endif
#endif /* DITCHUNK_H */
