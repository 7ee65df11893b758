// Kernel-level entry points (include/ditchunk_ops.h): host validation, then one launch.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "ditchunk.h"
#include "ditchunk_ops.h"
#include "kernels.h"

using namespace dit;

// Shared with ditchunk.cpp: the thread-local error message.
extern "C" const char* dit_last_error(void);
namespace dit {
int set_error(int code, const char* msg);
}

namespace {

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  return dit::set_error(code, buf);
}

int hipchk(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(DIT_EHIP, "%s: %s", what, hipGetErrorString(e));
  return DIT_OK;
}

bool dtype_ok(int d) { return d == DIT_F32 || d == DIT_BF16; }

int gemm_args(int dtype, const void* A, const void* W, const void* b, int M, int N, int K) {
  if (!dtype_ok(dtype)) return fail(DIT_EINVAL, "dtype %d", dtype);
  if ((M > 0 && !A) || !W || !b) return fail(DIT_EINVAL, "A, W and b must be non-NULL");
  if (M < 0 || N < 1 || K < 1) return fail(DIT_ESHAPE, "M=%d N=%d K=%d", M, N, K);
  if (K % 64) return fail(DIT_ESHAPE, "K=%d must be a multiple of 64", K);
  if (N % 4) return fail(DIT_ESHAPE, "N=%d must be a multiple of 4", N);
  if ((long long)M * K >= GEMM_MAX_ELEMS || (long long)N * K >= GEMM_MAX_ELEMS)
    return fail(DIT_ESHAPE, "M=%d N=%d K=%d: each operand must hold fewer than 2^31 elements", M, N, K);
  return DIT_OK;
}

}  // namespace

extern "C" {

int ditk_linear(int dtype, const void* A, const void* W, const void* b, int M, int N, int K,
                int act, void* out, void* stream) {
  int rc = gemm_args(dtype, A, W, b, M, N, K);
  if (rc) return rc;
  if (M > 0 && !out) return fail(DIT_EINVAL, "out is NULL");
  GemmEpi e{};
  if (act == DITK_ACT_NONE) e.kind = EPI_BIAS;
  else if (act == DITK_ACT_GELU) e.kind = EPI_GELU;
  else if (act == DITK_OUT_F32) e.kind = EPI_F32;
  else return fail(DIT_EINVAL, "act %d", act);
  if (M == 0) return DIT_OK;
  e.bias = b;
  e.out = out;
  e.ldo = N;
  return hipchk(gemm(dtype, A, K, W, K, M, N, K, e, (hipStream_t)stream), "gemm");
}

int ditk_linear_residual(int dtype, const void* A, const void* W, const void* b, const float* gate,
                         int M, int N, int K, float* h, float* workspace, long long workspace_floats,
                         void* stream) {
  int rc = gemm_args(dtype, A, W, b, M, N, K);
  if (rc) return rc;
  if (M > 0 && !h) return fail(DIT_EINVAL, "h is NULL");
  if (workspace_floats < 0 || (workspace_floats > 0 && !workspace))
    return fail(DIT_EINVAL, "workspace NULL with workspace_floats=%lld", workspace_floats);
  if (M == 0) return DIT_OK;
  GemmEpi e{};
  e.kind = EPI_RESID;
  e.bias = b;
  e.out = h;
  e.ldo = N;
  e.gate = gate;
  e.ws = workspace_floats > 0 ? workspace : nullptr;
  e.ws_floats = workspace_floats;
  return hipchk(gemm(dtype, A, K, W, K, M, N, K, e, (hipStream_t)stream), "gemm");
}

int ditk_rmsnorm_modulate(int dtype, const float* h, int n, int D, const float* shift,
                          const float* scale, double eps, void* out, void* stream) {
  if (!dtype_ok(dtype)) return fail(DIT_EINVAL, "dtype %d", dtype);
  if (n > 0 && (!h || !out)) return fail(DIT_EINVAL, "h/out NULL");
  if (!shift != !scale) return fail(DIT_EINVAL, "shift and scale must both be given or both NULL");
  if (n < 0 || D < 256 || D % 256 || D > 4096) return fail(DIT_ESHAPE, "n=%d D=%d", n, D);
  if (!(eps > 0) || !std::isfinite(eps)) return fail(DIT_EINVAL, "eps");
  if (n == 0) return DIT_OK;
  return hipchk(rmsnorm_mod(dtype, h, n, D, shift, scale, (float)eps, out, (hipStream_t)stream),
                "rmsnorm_mod");
}

int ditk_qknorm_rope(int dtype, int dh, int H, int n, const void* q_in, const void* k_in,
                     const void* v_in, int ld_in, const void* gq, const void* gk, int rope,
                     dit_grid grid, double eps, double theta, double q_scale, void* q_out,
                     void* k_out, void* vt_out, int cap, void* stream) {
  if (!dtype_ok(dtype)) return fail(DIT_EINVAL, "dtype %d", dtype);
  if (dh != 64 && dh != 128) return fail(DIT_EINVAL, "dh %d", dh);
  if (H < 1 || n < 0 || ld_in < H * dh) return fail(DIT_ESHAPE, "H=%d n=%d ld_in=%d", H, n, ld_in);
  if ((q_in && (!q_out || !gq)) || (k_in && (!k_out || !gk)) || (v_in && !vt_out))
    return fail(DIT_EINVAL, "missing output or gamma");
  if ((k_in || v_in) && (cap % 64 || cap < (n + 63) / 64 * 64))
    return fail(DIT_ESHAPE, "cap=%d must be a multiple of 64 >= n=%d", cap, n);
  if (rope && (grid.frames < 1 || grid.h < 1 || grid.w < 1 || (long long)grid.frames * grid.h * grid.w < n))
    return fail(DIT_ESHAPE, "grid does not cover n tokens");
  if (!(eps > 0) || !(theta > 1)) return fail(DIT_EINVAL, "eps/theta");
  if (!(q_scale > 0) || !std::isfinite(q_scale)) return fail(DIT_EINVAL, "q_scale");
  if (n == 0) return DIT_OK;
  RopeGrid g{grid.t0, grid.frames, grid.h, grid.w};
  return hipchk(qknorm_rope(dtype, dh, H, n, q_in, k_in, v_in, ld_in, gq, gk, rope, g, (float)eps,
                            (float)theta, (float)q_scale, q_out, k_out, vt_out, cap,
                            (hipStream_t)stream),
                "qknorm_rope");
}

int ditk_attention_probs(int H, const void* q, int nq, const void* k, int n, int cap, int q_prescaled,
                         void* p, void* stream) {
  if ((nq > 0 && (!q || !p)) || !k) return fail(DIT_EINVAL, "NULL argument");
  if (H < 1 || nq < 0) return fail(DIT_ESHAPE, "H=%d nq=%d", H, nq);
  if (n < 1 || n > 64 || cap < 64 || cap % 64) return fail(DIT_ESHAPE, "n=%d cap=%d: needs 1 <= n <= 64 <= cap", n, cap);
  if (nq == 0) return DIT_OK;
  const AttnSeg seg{k, nullptr, n, cap};
  return hipchk(short_attention_probs(128, H, q, H * 128, p, H * 64, nq, seg, q_prescaled != 0,
                                      (hipStream_t)stream),
                "short_attention_probs");
}

}  // extern "C"

namespace {

// The allocation-free attention's split scratch: a file-scope device array, one copy per
// GPU, kept until the process ends.  Host code must not pass `scratch` itself to a kernel
// (on the host it names a stand-in, not a device address): each device's address comes
// from hipGetSymbolAddress, taken once per device with that device current.
constexpr long long NOALLOC_SCRATCH_FLOATS = DITK_NOALLOC_SCRATCH_BYTES / 4;
__device__ __align__(256) float scratch[NOALLOC_SCRATCH_FLOATS];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
float* g_scratch[MAX_DEVICES] = {};

// The device address of `scratch` on the calling thread's current device.
int scratch_on_current_device(float** out) {
  int dev = -1;
  if (hipError_t e = hipGetDevice(&dev); e != hipSuccess)
    return fail(DIT_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= MAX_DEVICES) return fail(DIT_EHIP, "device %d beyond the %d supported", dev, MAX_DEVICES);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(DIT_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch[dev] = static_cast<float*>(p);
  }
  *out = g_scratch[dev];
  return DIT_OK;
}

// Validation and launch shared by ditk_attention (partial from the caller) and
// ditk_attention_noalloc (noalloc: the split scratch is the device's `scratch`, taken
// only after every check has passed, and bounded by its size).
int attention_entry(int dtype, int dh, int H, const void* q, int nq, int nseg, const void* const* k,
                    const void* const* vt, const int* n, const int* cap, int nsplit, float* partial,
                    bool noalloc, int unsplit_rows, int q_prescaled, const void* gq, const void* gk,
                    double q_fold, void* o, void* stream) {
  if (!dtype_ok(dtype)) return fail(DIT_EINVAL, "dtype %d", dtype);
  if ((gq != nullptr) != (gk != nullptr)) return fail(DIT_EINVAL, "gq and gk must both be given or both NULL");
  if (gq && !(q_fold > 0 && std::isfinite(q_fold))) return fail(DIT_EINVAL, "q_fold must be finite and > 0");
  if (dh != 64 && dh != 128) return fail(DIT_EINVAL, "dh %d", dh);
  if ((nq > 0 && (!q || !o)) || !k || !vt || !n || !cap) return fail(DIT_EINVAL, "NULL argument");
  if (dtype == DIT_F32 && dh != 64) return fail(DIT_EINVAL, "fp32 attention supports dh=64 only");
  if (H < 1 || nq < 0 || nseg < 1 || nseg > ATTN_MAX_SEGS) return fail(DIT_ESHAPE, "H/nq/nseg");
  AttnSeg seg[ATTN_MAX_SEGS];
  long long total = 0;
  for (int i = 0; i < nseg; ++i) {
    if (n[i] < 0 || cap[i] % 64 || cap[i] < (n[i] + 63) / 64 * 64)
      return fail(DIT_ESHAPE, "segment %d: n=%d cap=%d", i, n[i], cap[i]);
    if (n[i] > 0 && (!k[i] || !vt[i])) return fail(DIT_EINVAL, "segment %d NULL", i);
    if ((long long)H * dh * cap[i] * (dtype == DIT_BF16 ? 2 : 4) >= VT_MAX_BYTES)
      return fail(DIT_ESHAPE, "segment %d: V^T [%d, %d] must stay under 2^31 bytes", i, H * dh, cap[i]);
    seg[i] = AttnSeg{k[i], vt[i], n[i], cap[i]};
    total += n[i];
  }
  if (total < 1) return fail(DIT_ESHAPE, "no keys");
  if (nsplit < 1 || nsplit > 8) return fail(DIT_EINVAL, "nsplit=%d out of [1, 8]", nsplit);
  if (unsplit_rows < 0 || (unsplit_rows % ATTN_QTILE && unsplit_rows < nq))
    return fail(DIT_EINVAL, "unsplit_rows=%d: must be >= 0 and a multiple of %d or >= nq=%d", unsplit_rows,
                ATTN_QTILE, nq);
  if (unsplit_rows >= nq) nsplit = 1;  // nothing left to split
  const int D = H * dh;
  if (noalloc && nsplit > 1 && (long long)nsplit * nq * (D + 2LL * H) > NOALLOC_SCRATCH_FLOATS)
    return fail(DIT_EWORKSPACE, "split scratch of %d x %d x (%d + 2 x %d) floats exceeds the %lld of the "
                "allocation-free scratch", nsplit, nq, D, H, NOALLOC_SCRATCH_FLOATS);
  if (!noalloc && nsplit > 1 && !partial) return fail(DIT_EINVAL, "partial is NULL with nsplit=%d", nsplit);
  if (nq == 0) return DIT_OK;
  if (noalloc && nsplit > 1)
    if (int rc = scratch_on_current_device(&partial)) return rc;
  if (nsplit == 1 && short_attention_fits(dtype, dh, nseg, seg))
    return hipchk(short_attention(dh, H, q, D, o, D, nq, seg[0], q_prescaled != 0, (hipStream_t)stream),
                  "short_attention");
  AttnSplit sp{nsplit, unsplit_rows / ATTN_QTILE, partial, partial ? partial + (size_t)nsplit * nq * D : nullptr};
  const AttnNorm norm{gq, gk, q_fold};
  int rc = hipchk(attention(dtype, dh, H, q, D, o, D, nq, D, seg, nseg, sp, q_prescaled != 0,
                            (hipStream_t)stream, ATTN_SELF, gq ? &norm : nullptr),
                  "attention");
  if (rc) return rc;
  return hipchk(attention_combine(dtype, dh, H, nq, sp, o, D, (hipStream_t)stream), "attention_combine");
}

}  // namespace

extern "C" {

int ditk_attention(int dtype, int dh, int H, const void* q, int nq, int nseg,
                   const void* const* k, const void* const* vt, const int* n, const int* cap,
                   int nsplit, float* partial, int unsplit_rows, int q_prescaled, const void* gq,
                   const void* gk, double q_fold, void* o, void* stream) {
  return attention_entry(dtype, dh, H, q, nq, nseg, k, vt, n, cap, nsplit, partial, false, unsplit_rows,
                         q_prescaled, gq, gk, q_fold, o, stream);
}

int ditk_attention_noalloc(int dtype, int dh, int H, const void* q, int nq, int nseg,
                           const void* const* k, const void* const* vt, const int* n, const int* cap,
                           int nsplit, int unsplit_rows, int q_prescaled, const void* gq, const void* gk,
                           double q_fold, void* o, void* stream) {
  return attention_entry(dtype, dh, H, q, nq, nseg, k, vt, n, cap, nsplit, nullptr, true, unsplit_rows,
                         q_prescaled, gq, gk, q_fold, o, stream);
}

int ditk_modulation(int dtype, int D, int L, double t, const void* const* w, float* mod_out,
                    float* fmod_out, float* tmp, void* stream) {
  if (!dtype_ok(dtype)) return fail(DIT_EINVAL, "dtype %d", dtype);
  if (!w || !mod_out || !fmod_out || !tmp) return fail(DIT_EINVAL, "NULL argument");
  if (D < 256 || D % 256 || L < 1) return fail(DIT_ESHAPE, "D=%d L=%d", D, L);
  if (!std::isfinite(t)) return fail(DIT_EINVAL, "t not finite");
  const void* mw[256];
  const void* mb[256];
  if (L > 256) return fail(DIT_ESHAPE, "L > 256");
  for (int l = 0; l < L; ++l) {
    mw[l] = w[DIT_W_GLOBAL_COUNT + l * DIT_W_BLOCK_COUNT + DIT_WB_MOD_W];
    mb[l] = w[DIT_W_GLOBAL_COUNT + l * DIT_W_BLOCK_COUNT + DIT_WB_MOD_B];
  }
  return hipchk(modulation(dtype, D, L, t, w[DIT_W_T1_W], w[DIT_W_T1_B], w[DIT_W_T2_W],
                           w[DIT_W_T2_B], mw, mb, w[DIT_W_FMOD_W], w[DIT_W_FMOD_B], tmp, mod_out,
                           fmod_out, (hipStream_t)stream),
                "modulation");
}

int ditk_patch_input(int dtype, const float* x, int n, int c_p, const float* cond, int c_c,
                     int cond_mode, dit_grid grid, void* xin, void* stream) {
  if (!dtype_ok(dtype)) return fail(DIT_EINVAL, "dtype %d", dtype);
  if (n > 0 && (!x || !xin || (cond_mode && !cond))) return fail(DIT_EINVAL, "NULL argument");
  if (n < 0 || c_p < 1 || c_c < 0 || cond_mode < 0 || cond_mode > 2) return fail(DIT_ESHAPE, "shape");
  if (cond_mode == 2 && (grid.h % 2 || grid.w % 2 || c_c % 4 ||
                         (long long)grid.frames * grid.h * grid.w != n))
    return fail(DIT_ESHAPE, "upsample grid");
  if (n == 0) return DIT_OK;
  RopeGrid g{grid.t0, grid.frames, grid.h, grid.w};
  return hipchk(patch_input(dtype, x, n, c_p, cond, c_c, cond_mode, g, xin, (hipStream_t)stream),
                "patch_input");
}

static_assert(DITK_PROBE_SINK_FLOATS == PROBE_SINK_FLOATS, "probe sink size");

int ditk_probe_mfma(const void* data, int iters, float* sink, long long sink_floats, double* flop,
                    void* stream) {
  if (!data || !sink || !flop) return fail(DIT_EINVAL, "NULL argument");
  if (iters < 1) return fail(DIT_EINVAL, "iters=%d must be >= 1", iters);
  if (sink_floats < DITK_PROBE_SINK_FLOATS)
    return fail(DIT_EWORKSPACE, "sink of %lld floats < %d", sink_floats, DITK_PROBE_SINK_FLOATS);
  return hipchk(probe_mfma(data, iters, sink, flop, (hipStream_t)stream), "probe_mfma");
}

int ditk_probe_copy(const void* src, void* dst, long long bytes, void* stream) {
  if (bytes < 0 || bytes % 16) return fail(DIT_EINVAL, "bytes=%lld must be a non-negative multiple of 16", bytes);
  if (bytes == 0) return DIT_OK;
  if (!src || !dst) return fail(DIT_EINVAL, "NULL argument");
  if (((uintptr_t)src & 15) || ((uintptr_t)dst & 15)) return fail(DIT_EINVAL, "src, dst must be 16-byte aligned");
  return hipchk(probe_copy(src, dst, bytes, (hipStream_t)stream), "probe_copy");
}

int ditk_patch_embed(const float* x, int n, int c_p, const float* cond, int c_c, int cond_mode,
                     dit_grid grid, const void* w, const void* b, float* out, int D, void* stream) {
  if ((n > 0 && (!x || !out || (cond_mode && !cond))) || !w || !b) return fail(DIT_EINVAL, "NULL argument");
  if (n < 0 || c_p < 1 || c_c < 0 || D < 1 || cond_mode < 0 || cond_mode > 2) return fail(DIT_ESHAPE, "shape");
  if (!patch_embed_fits(BF16, c_p, c_c, D))
    return fail(DIT_ESHAPE, "patch_embed needs (c_p + c_c) %% 64 == 0, c_p and c_c %% 8 == 0, D %% 256 == 0");
  if (cond_mode == 2 && (grid.h % 2 || grid.w % 2 || (long long)grid.frames * grid.h * grid.w != n))
    return fail(DIT_ESHAPE, "upsample grid");
  if (n == 0) return DIT_OK;
  RopeGrid g{grid.t0, grid.frames, grid.h, grid.w};
  return hipchk(patch_embed(x, n, c_p, cond, c_c, cond_mode, g, w, b, out, D, (hipStream_t)stream),
                "patch_embed");
}

}  // extern "C"
