// libditchunk: host side of the C ABI (include/ditchunk.h).
//
// The handle borrows every device buffer (weights, state, workspace) from the caller
// and validates all arguments on the host before any HIP call.  A call enqueues a
// fixed kernel sequence on the handle's stream:
//
//   ref_kv_precompute / boundary_kv_carry / interp_anchor_kv (context pass at t = 0):
//     modulation(0) -> patch input -> patch embed ->
//     per block: RMSNorm+mod -> QKV -> QK-norm+RoPE (K, V written to the state) ->
//                [not last block] attention over earlier context + self -> out-proj
//                (gated residual) -> RMSNorm+mod -> FC1+GELU -> FC2 (gated residual)
//   dit_chunk_step:
//     modulation(t) -> patch input -> patch embed ->
//     per block: RMSNorm+mod -> QKV -> QK-norm+RoPE -> attention over
//                [ref | bnd | anchor | chunk] -> out-proj (gated residual) ->
//                [audio] RMSNorm -> q_c -> q-norm; audio K/V -> k-norm (or the
//                K/V held by audio_kv_precompute); cross attention -> out (residual) ->
//                RMSNorm+mod -> FC1+GELU -> FC2 (gated residual)
//     final RMSNorm+mod -> final Linear with the Euler update fused into its epilogue.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "ditchunk.h"
#include "kernels.h"

using namespace dit;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
int round64(long long x) { return (int)((x + 63) / 64 * 64); }

// Buffer layout of the state and the workspace (byte offsets).
struct Layout {
  size_t elt = 0;
  int cap_tok = 0, cap_ref = 0, cap_bnd = 0, cap_audio = 0, F = 0, C_in = 0, big_cols = 0;
  // state
  std::vector<size_t> kref, vref, kbnd, vbnd, kanc, vanc, kaud, vaud;
  size_t aud_in = 0;  // held audio features [cap_audio, d_a] (dtype), d_a > 0
  // Audio cross-attention folded into its output Linear (bf16, dh 128, at most 64 audio
  // tokens): per block U^T = W_co [V_a restricted to each head]^T, [D, H*64] (dtype), so
  // that the cross out-projection is P [n, H*64] U^T (see short_attention_probs).
  bool fold = false;
  std::vector<size_t> uta;  // held audio: per block U^T
  size_t modtab = 0;  // DIT_MOD_TABLE_MAX entries of mod_entry floats
  size_t mod_entry = 0;
  size_t state_total = 0;
  // workspace
  size_t wbd = 0, uta_ws = 0;  // fold: head-block-diagonal V_a [H*64, D]; U^T of per-step audio
  size_t xin = 0, h = 0, u = 0, big = 0, q = 0, kc = 0, vtc = 0, o = 0, ain = 0, ka_raw = 0,
         va_raw = 0, ka = 0, vat = 0, mod = 0, tmp = 0, opart = 0, ml = 0;
  int part_rows = 0;  // rows of key-range attention partials (split count x queries)
  size_t ws_total = 0;
};

int check_config(const dit_config* c) {
  if (!c) return fail(DIT_EINVAL, "config is NULL");
  if (c->dtype != DIT_F32 && c->dtype != DIT_BF16) return fail(DIT_EINVAL, "dtype %d", c->dtype);
  if (c->L < 1 || c->L > 256) return fail(DIT_EINVAL, "L=%d out of [1, 256]", c->L);
  if (c->dh != 64 && c->dh != 128) return fail(DIT_EINVAL, "dh=%d (64 or 128)", c->dh);
  if (c->dtype == DIT_F32 && c->dh != 64) return fail(DIT_EINVAL, "fp32 supports dh=64 only");
  if (c->H < 1 || c->D != c->H * c->dh) return fail(DIT_EINVAL, "D=%d != H*dh=%d*%d", c->D, c->H, c->dh);
  if (c->D % 256 || c->D > 4096) return fail(DIT_EINVAL, "D=%d must be a multiple of 256, <= 4096", c->D);
  if (c->mlp_ratio < 1 || c->mlp_ratio > 8) return fail(DIT_EINVAL, "mlp_ratio=%d", c->mlp_ratio);
  if (c->c_p < 4 || c->c_p % 4) return fail(DIT_EINVAL, "c_p=%d must be a positive multiple of 4", c->c_p);
  if (c->c_c < 0 || (c->c_p + c->c_c) % 64) return fail(DIT_EINVAL, "c_p+c_c=%d must be a multiple of 64", c->c_p + c->c_c);
  if (c->cond_up != 1 && c->cond_up != 2) return fail(DIT_EINVAL, "cond_up=%d (1 or 2)", c->cond_up);
  if (c->cond_up == 2 && c->c_c % 4) return fail(DIT_EINVAL, "cond_up=2 needs c_c multiple of 4");
  if (c->d_a < 0 || c->d_a % 64) return fail(DIT_EINVAL, "d_a=%d must be a multiple of 64", c->d_a);
  if (c->max_tokens < 1 || c->max_ref < 1 || c->max_bnd < 0 || c->max_audio < 0)
    return fail(DIT_EINVAL, "capacities must be max_tokens>=1, max_ref>=1, max_bnd>=0, max_audio>=0");
  if (c->max_tokens > (1 << 24) || c->max_ref > (1 << 24) || c->max_bnd > (1 << 24) || c->max_audio > 65536)
    return fail(DIT_EINVAL, "capacity too large");
  {
    // 32-bit operand offsets of the GEMM and attention kernels (GEMM_MAX_ELEMS,
    // VT_MAX_BYTES): the widest activation matrix is [token capacity, max(3D, mlp D)],
    // the largest V^T buffer [D, token capacity].
    long long cap = c->max_tokens;
    if (c->max_ref > cap) cap = c->max_ref;
    if (c->max_bnd > cap) cap = c->max_bnd;
    cap = (cap + 63) / 64 * 64;
    const long long elt = c->dtype == DIT_BF16 ? 2 : 4;
    const long long widest = 3LL * c->D > (long long)c->mlp_ratio * c->D ? 3LL * c->D : (long long)c->mlp_ratio * c->D;
    if (cap * widest >= GEMM_MAX_ELEMS || cap * c->D * elt >= VT_MAX_BYTES)
      return fail(DIT_EINVAL,
                  "token capacity %lld too large for D=%d, mlp_ratio=%d: activations [%lld, %lld] must stay under "
                  "2^31 elements and V^T [%d, %lld] under 2^31 bytes",
                  cap, c->D, c->mlp_ratio, cap, widest, c->D, cap);
  }
  if (!(c->eps > 0) || !std::isfinite(c->eps)) return fail(DIT_EINVAL, "eps must be finite and > 0");
  if (!(c->rope_theta > 1) || !std::isfinite(c->rope_theta)) return fail(DIT_EINVAL, "rope_theta must be finite and > 1");
  return DIT_OK;
}

Layout make_layout(const dit_config* c) {
  Layout L;
  L.elt = c->dtype == DIT_BF16 ? 2 : 4;
  const size_t D = c->D;
  L.F = c->mlp_ratio * c->D;
  L.C_in = c->c_p + c->c_c;
  int mx = c->max_tokens;
  if (c->max_ref > mx) mx = c->max_ref;
  if (c->max_bnd > mx) mx = c->max_bnd;
  L.cap_tok = round64(mx);
  L.cap_ref = round64(c->max_ref);
  L.cap_bnd = round64(c->max_bnd);
  L.cap_audio = round64(c->max_audio > 0 ? c->max_audio : 1);
  L.big_cols = 3 * c->D > L.F ? 3 * c->D : L.F;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t r = off; off += align256(bytes); return r; };
  for (int l = 0; l < c->L; ++l) {
    L.kref.push_back(take((size_t)L.cap_ref * D * L.elt));
    L.vref.push_back(take((size_t)L.cap_ref * D * L.elt));
    L.kbnd.push_back(take((size_t)L.cap_bnd * D * L.elt));
    L.vbnd.push_back(take((size_t)L.cap_bnd * D * L.elt));
    L.kanc.push_back(take((size_t)L.cap_bnd * D * L.elt));
    L.vanc.push_back(take((size_t)L.cap_bnd * D * L.elt));
    const size_t aud = c->d_a > 0 ? (size_t)L.cap_audio * D * L.elt : 0;
    L.kaud.push_back(take(aud));
    L.vaud.push_back(take(aud));
  }
  L.aud_in = take(c->d_a > 0 ? (size_t)L.cap_audio * c->d_a * L.elt : 0);
  L.fold = c->dtype == DIT_BF16 && c->dh == 128 && c->d_a > 0 && L.cap_audio == 64;
  const size_t ubytes = L.fold ? D * (size_t)c->H * 64 * L.elt : 0;
  for (int l = 0; l < c->L; ++l) L.uta.push_back(take(ubytes));
  L.mod_entry = ((size_t)c->L * 6 + 2) * D;
  L.modtab = take(DIT_MOD_TABLE_MAX * L.mod_entry * 4);
  L.state_total = off;
  off = 0;
  const size_t T = L.cap_tok;
  L.xin = take(T * L.C_in * L.elt);
  L.h = take(T * D * 4);
  L.u = take(T * D * L.elt);
  L.big = take(T * L.big_cols * L.elt);
  L.q = take(T * D * L.elt);
  L.kc = take(T * D * L.elt);
  L.vtc = take(T * D * L.elt);
  L.o = take(T * D * L.elt);
  const size_t A = L.cap_audio;
  L.ain = take(A * (c->d_a > 0 ? c->d_a : 64) * L.elt);
  L.ka_raw = take(A * D * L.elt);
  L.va_raw = take(A * D * L.elt);
  L.ka = take(A * D * L.elt);
  L.vat = take(A * D * L.elt);
  L.mod = take(((size_t)c->L * 6 * D + 2 * D) * 4);
  L.tmp = take((256 + 2 * D) * 4);
  L.part_rows = 2 * L.cap_tok;
  L.opart = take((size_t)L.part_rows * D * 4);
  L.ml = take((size_t)L.part_rows * c->H * 2 * 4);
  L.wbd = take(L.fold ? (size_t)c->H * 64 * D * L.elt : 0);
  L.uta_ws = take(L.fold ? D * (size_t)c->H * 64 * L.elt : 0);
  L.ws_total = off;
  return L;
}

constexpr int MAX_EVENT_PAIRS = 4096;

}  // namespace

namespace dit {
int set_error(int code, const char* msg) {
  g_err = msg;
  return code;
}
}  // namespace dit

// Per-block weight streaming (dit_weight_stream): block weights come from pinned host
// memory through a device ring of nslot block slots.  Block uses are numbered in pass
// order (every pass uses blocks 0..L-1 in turn); use u reads slot u % nslot, which holds
// block u % L.  The copy for use u + nslot is issued on the copy stream once use u has
// been enqueued, behind an event recorded after use u's last kernel, so while block l
// runs the next nslot - 1 blocks (also those of the next pass) are in flight.
struct Streaming {
  bool on = false;
  std::vector<const void*> host;  // L * DIT_W_BLOCK_COUNT host pointers
  char* ring = nullptr;
  int nslot = 0;
  size_t slot_bytes = 0;
  size_t off[DIT_W_BLOCK_COUNT] = {}, bytes[DIT_W_BLOCK_COUNT] = {};
  hipStream_t copy = nullptr;
  std::vector<hipEvent_t> ready, freed;  // per slot: copy landed / last reader done
  std::vector<int> holds;                // block copied into each slot (-1: none)
  std::vector<char> freed_rec;           // freed[slot] has been recorded
  long long base = 0;                    // use index of block 0 of the current pass
  long long issued = 0;                  // copies of uses [0, issued) are enqueued
};

struct dit_handle {
  dit_config cfg;
  Layout lay;
  std::vector<const void*> w;
  Streaming st;
  char* state = nullptr;
  char* ws = nullptr;
  hipStream_t stream = nullptr;
  bool has_ref = false;
  int n_ref = 0, n_bnd = 0, n_anc = 0, n_aud = 0;
  // Held audio K/V of block l still to compute (set by audio_kv_precompute while block
  // weights stream: each block's K/V is then computed when the next pass brings that
  // block's weights into the ring, instead of in a pass of its own).
  std::vector<char> aud_pend;
  std::vector<double> mod_t;  // timesteps of the modulation table entries
  // timing (dit_timing_enable): per kind, event pairs stamped by the timed dispatches
  struct Timing {
    bool on = false;
    std::vector<hipEvent_t> ev;  // 2 * MAX_EVENT_PAIRS, created by dit_timing_enable
    int used = 0;                // pairs stamped in this window
    double work = 0.0;           // their algorithmic flop (attention, GEMM) or bytes
  } tm[DIT_TIME_KINDS];

  const void* W(int i) const { return w[i]; }
  const void* B(int l, int i) const {
    if (st.on) {
      if (!st.bytes[i]) return nullptr;
      return st.ring + (size_t)((st.base + l) % st.nslot) * st.slot_bytes + st.off[i];
    }
    return w[DIT_W_GLOBAL_COUNT + l * DIT_W_BLOCK_COUNT + i];
  }
  template <class P = void> P* S(size_t off) const { return reinterpret_cast<P*>(state + off); }
  template <class P = void> P* X(size_t off) const { return reinterpret_cast<P*>(ws + off); }
};

namespace {

#define HIPCHK(expr)                                                                   \
  do {                                                                                 \
    hipError_t e_ = (expr);                                                            \
    if (e_ != hipSuccess) return fail(DIT_EHIP, "%s: %s", #expr, hipGetErrorString(e_)); \
  } while (0)

// The modulation table entry held for timestep t (dit_modulation_table), or NULL: then
// the pass computes its modulation itself.  Entry layout: [L, 6, D] then [2, D].
const float* mod_table_entry(const dit_handle* hd, double t) {
  for (size_t j = 0; j < hd->mod_t.size(); ++j)
    if (hd->mod_t[j] == t) return hd->S<float>(hd->lay.modtab) + j * hd->lay.mod_entry;
  return nullptr;
}

// Bytes of block weight entry i (0 for absent cross-attention entries).
size_t block_entry_bytes(const dit_config& c, int i) {
  const size_t D = c.D, F = (size_t)c.mlp_ratio * c.D, dh = c.dh, da = c.d_a;
  const size_t elt = c.dtype == DIT_BF16 ? 2 : 4;
  const bool cross = c.d_a > 0;
  size_t n = 0;
  switch (i) {
    case DIT_WB_MOD_W: n = 6 * D * D; break;
    case DIT_WB_MOD_B: n = 6 * D; break;
    case DIT_WB_QKV_W: n = 3 * D * D; break;
    case DIT_WB_QKV_B: n = 3 * D; break;
    case DIT_WB_GQ: case DIT_WB_GK: n = dh; break;
    case DIT_WB_O_W: n = D * D; break;
    case DIT_WB_O_B: n = D; break;
    case DIT_WB_CQ_W: case DIT_WB_CO_W: n = cross ? D * D : 0; break;
    case DIT_WB_CQ_B: case DIT_WB_CK_B: case DIT_WB_CV_B: case DIT_WB_CO_B: n = cross ? D : 0; break;
    case DIT_WB_CK_W: case DIT_WB_CV_W: n = D * da; break;
    case DIT_WB_GCQ: case DIT_WB_GCK: n = cross ? dh : 0; break;
    case DIT_WB_FC1_W: case DIT_WB_FC2_W: n = F * D; break;
    case DIT_WB_FC1_B: n = F; break;
    case DIT_WB_FC2_B: n = D; break;
    default: n = 0;
  }
  return n * elt;
}

// Slot layout: entries in table order, each 256-byte aligned.  Returns the slot size.
size_t block_slot_layout(const dit_config& c, size_t* off, size_t* bytes) {
  size_t o = 0;
  for (int i = 0; i < DIT_W_BLOCK_COUNT; ++i) {
    bytes[i] = block_entry_bytes(c, i);
    off[i] = o;
    o += align256(bytes[i]);
  }
  return o;
}

// Enqueue the copy of block use u into its slot (nothing if the slot already holds
// that block).
int stream_issue(dit_handle* hd, long long u) {
  Streaming& st = hd->st;
  const int slot = (int)(u % st.nslot), blk = (int)(u % hd->cfg.L);
  if (st.holds[slot] == blk) return DIT_OK;
  if (st.freed_rec[slot]) HIPCHK(hipStreamWaitEvent(st.copy, st.freed[slot], 0));
  char* dst = st.ring + (size_t)slot * st.slot_bytes;
  for (int i = 0; i < DIT_W_BLOCK_COUNT; ++i) {
    if (!st.bytes[i]) continue;
    HIPCHK(hipMemcpyAsync(dst + st.off[i], st.host[(size_t)blk * DIT_W_BLOCK_COUNT + i], st.bytes[i],
                          hipMemcpyHostToDevice, st.copy));
  }
  HIPCHK(hipEventRecord(st.ready[slot], st.copy));
  st.holds[slot] = blk;
  return DIT_OK;
}

int stream_issue_upto(dit_handle* hd, long long end) {
  Streaming& st = hd->st;
  for (; st.issued < end; ++st.issued)
    if (int rc = stream_issue(hd, st.issued)) return rc;
  return DIT_OK;
}

// Start of a pass: the first min(nslot, L) uses have their copies enqueued.
int pass_begin(dit_handle* hd) {
  Streaming& st = hd->st;
  if (!st.on) return DIT_OK;
  const int k = st.nslot < hd->cfg.L ? st.nslot : hd->cfg.L;
  return stream_issue_upto(hd, st.base + k);
}

int audio_kv(dit_handle* hd, int l, int M, const void* ain, void* ka, void* vat, void* uta);

// Block l of the pass: its kernels wait for its slot's copy.  A held audio K/V of block
// l still pending is computed first (its weights are now in place).
int block_begin(dit_handle* hd, int l) {
  Streaming& st = hd->st;
  if (st.on) HIPCHK(hipStreamWaitEvent(hd->stream, st.ready[(st.base + l) % st.nslot], 0));
  if (!hd->aud_pend.empty() && hd->aud_pend[l]) {
    const Layout& L = hd->lay;
    if (int rc = audio_kv(hd, l, hd->n_aud, hd->S(L.aud_in), hd->S(L.kaud[l]), hd->S(L.vaud[l]),
                          L.fold ? hd->S(L.uta[l]) : nullptr))
      return rc;
    hd->aud_pend[l] = 0;
  }
  return DIT_OK;
}

// After block l's last kernel is enqueued: mark its slot free once those kernels have
// run, and enqueue the copy of the use nslot later into it.
int block_end(dit_handle* hd, int l) {
  Streaming& st = hd->st;
  if (!st.on) return DIT_OK;
  const int slot = (int)((st.base + l) % st.nslot);
  HIPCHK(hipEventRecord(st.freed[slot], hd->stream));
  st.freed_rec[slot] = 1;
  return stream_issue_upto(hd, st.base + l + st.nslot + 1);
}

// End of a pass.  rc != DIT_OK (a pass cut short): forget what the slots hold so the
// next pass copies every block again, behind all work enqueued so far.
int pass_end(dit_handle* hd, int rc) {
  Streaming& st = hd->st;
  if (!st.on) return rc;
  if (rc == DIT_OK) {
    st.base += hd->cfg.L;
    return DIT_OK;
  }
  for (int k = 0; k < st.nslot; ++k) {
    (void)hipEventRecord(st.freed[k], hd->stream);
    st.freed_rec[k] = 1;
    st.holds[k] = -1;
  }
  st.issued = st.base;
  return rc;
}

// The start/stop event pair for the next launch of timing kind k, or NULL when that kind
// is not being timed (or the window is full).  The pair counts once timed_done has
// charged its work, i.e. only for a launch that was enqueued.
const hipEvent_t* timed_ev(dit_handle* h, int k) {
  dit_handle::Timing& t = h->tm[k];
  if (!t.on || t.used >= MAX_EVENT_PAIRS) return nullptr;
  return &t.ev[2 * (size_t)t.used];
}
void timed_done(dit_handle* h, int k, const hipEvent_t* ev, double work) {
  if (!ev) return;
  ++h->tm[k].used;
  h->tm[k].work += work;
}

// A GEMM of the block passes, timed as kind DIT_TIME_GEMM (flop 2 M N K).
int block_gemm(dit_handle* hd, const void* A, int lda, const void* W, int ldw, int M, int N, int K,
               const GemmEpi& e) {
  const hipEvent_t* ev = M > 0 ? timed_ev(hd, DIT_TIME_GEMM) : nullptr;
  HIPCHK(gemm(hd->cfg.dtype, A, lda, W, ldw, M, N, K, e, hd->stream, ev));
  timed_done(hd, DIT_TIME_GEMM, ev, 2.0 * M * N * K);
  return DIT_OK;
}

// RMSNorm (+ adaLN modulation when shift/scale are given) of h [n, D] into u, timed as
// kind DIT_TIME_ELEM (bytes: h read in fp32, u written in the dtype, the two vectors).
int block_norm(dit_handle* hd, const float* h, int n, const float* shift, const float* scale, void* u) {
  const dit_config& c = hd->cfg;
  const hipEvent_t* ev = n > 0 ? timed_ev(hd, DIT_TIME_ELEM) : nullptr;
  HIPCHK(rmsnorm_mod(c.dtype, h, n, c.D, shift, scale, (float)c.eps, u, hd->stream, ev));
  timed_done(hd, DIT_TIME_ELEM, ev, (double)n * c.D * (4 + hd->lay.elt) + (shift ? 2.0 * c.D * 4 : 0.0));
  return DIT_OK;
}

// Attention launch: picks the key-range split, times the main kernel when timing is on
// (the flop count is the method's 4 n_q n_kv D), then merges partials if split.  q and
// k are QK-normed with block l's gammas (self: gq/gk, cross: gcq/gck), q pre-scaled.
int run_attention(dit_handle* hd, int n, const AttnSeg* seg, int ns, bool timed, int kind, int l) {
  const dit_config& c = hd->cfg;
  const Layout& L = hd->lay;
  if (kind == ATTN_CROSS && short_attention_fits(c.dtype, c.dh, ns, seg)) {
    HIPCHK(short_attention(c.dh, c.H, hd->X(L.q), c.D, hd->X(L.o), c.D, n, seg[0], true, hd->stream));
    return DIT_OK;
  }
  AttnSplit sp = attention_plan(n, c.H, attention_key_tiles(seg, ns), L.part_rows, device_cus());
  sp.opart = hd->X<float>(L.opart);
  sp.ml = hd->X<float>(L.ml);
  // timed: the main kernel's dispatch stamps the start, the merge's (if split) the end
  const hipEvent_t* ev = timed && n > 0 ? timed_ev(hd, DIT_TIME_ATTN) : nullptr;
  const bool cross = kind == ATTN_CROSS;
  const AttnNorm norm{hd->B(l, cross ? DIT_WB_GCQ : DIT_WB_GQ), hd->B(l, cross ? DIT_WB_GCK : DIT_WB_GK),
                      (double)attention_q_scale(c.dh)};
  HIPCHK(attention(c.dtype, c.dh, c.H, hd->X(L.q), c.D, hd->X(L.o), c.D, n, c.D, seg, ns, sp, true, hd->stream,
                   kind, &norm, ev));
  HIPCHK(attention_combine(c.dtype, c.dh, c.H, n, sp, hd->X(L.o), c.D, hd->stream, ev ? ev[1] : nullptr));
  if (ev) {
    double nkv = 0;
    for (int i = 0; i < ns; ++i) nkv += seg[i].n;
    timed_done(hd, DIT_TIME_ATTN, ev, 4.0 * n * nkv * c.D);
  }
  return DIT_OK;
}

// Patch embed into h [n, D] (fp32): the tokens' input rows [x || cond'] (cond' zero,
// per token, or the nearest-2x upsample, by cond_mode) times W_pe, plus bias.  The
// fused kernel assembles the rows inside its operand loads; shapes it does not take
// (fp32 weights, odd widths) go through the assembled input matrix and a GEMM.
int embed(dit_handle* hd, const float* x, int n, const float* cond, int cond_mode, RopeGrid g, float* h) {
  const dit_config& c = hd->cfg;
  const Layout& L = hd->lay;
  if (patch_embed_fits(c.dtype, c.c_p, c.c_c, c.D)) {
    HIPCHK(patch_embed(x, n, c.c_p, cond, c.c_c, cond_mode, g, hd->W(DIT_W_PE_W), hd->W(DIT_W_PE_B), h,
                       c.D, hd->stream));
    return DIT_OK;
  }
  HIPCHK(patch_input(c.dtype, x, n, c.c_p, cond, c.c_c, cond_mode, g, hd->X(L.xin), hd->stream));
  GemmEpi e{};
  e.kind = EPI_F32; e.bias = hd->W(DIT_W_PE_B); e.out = h; e.ldo = c.D;
  HIPCHK(gemm(c.dtype, hd->X(L.xin), L.C_in, hd->W(DIT_W_PE_W), L.C_in, n, c.D, L.C_in, e, hd->stream));
  return DIT_OK;
}

// Block l's audio K (k-normed) and V^T (attention layout, capacity cap_audio) from the
// audio tokens ain [M, d_a] (dtype); with uta (the folded cross-attention) also
// U^T = W_co V_bd^T [D, H*64], V_bd the head-block-diagonal copy of V [M, D].
int audio_kv(dit_handle* hd, int l, int M, const void* ain, void* ka, void* vat, void* uta) {
  const dit_config& c = hd->cfg;
  const Layout& L = hd->lay;
  const int D = c.D;
  hipStream_t s = hd->stream;
  RopeGrid g0{0, 1, 1, 1};
  GemmEpi e{};
  e.kind = EPI_BIAS; e.bias = hd->B(l, DIT_WB_CK_B); e.out = hd->X(L.ka_raw); e.ldo = D;
  HIPCHK(gemm(c.dtype, ain, c.d_a, hd->B(l, DIT_WB_CK_W), c.d_a, M, D, c.d_a, e, s));
  e.bias = hd->B(l, DIT_WB_CV_B); e.out = hd->X(L.va_raw);
  HIPCHK(gemm(c.dtype, ain, c.d_a, hd->B(l, DIT_WB_CV_W), c.d_a, M, D, c.d_a, e, s));
  HIPCHK(qknorm_rope(c.dtype, c.dh, c.H, M, nullptr, hd->X(L.ka_raw), hd->X(L.va_raw), D, nullptr,
                     hd->B(l, DIT_WB_GCK), 0, g0, (float)c.eps, (float)c.rope_theta, 1.0f, nullptr, ka,
                     vat, L.cap_audio, s));
  if (uta) {
    const int HK = c.H * 64;
    HIPCHK(head_blockdiag(c.dtype, hd->X(L.va_raw), M, D, c.dh, hd->X(L.wbd), s));
    GemmEpi eu{};
    eu.kind = EPI_BIAS; eu.bias = nullptr; eu.out = uta; eu.ldo = HK;
    HIPCHK(gemm(c.dtype, hd->B(l, DIT_WB_CO_W), D, hd->X(L.wbd), D, D, HK, D, eu, s));
  }
  return DIT_OK;
}

// QKV of block l over n tokens (u in the workspace): q (QK-normed, pre-scaled, rotated)
// -> q_out (NULL: not needed), k (QK-normed, rotated) -> k_out [cap rows], V^T -> vt_out
// [D, cap].  When the launch allows it the QK-norm, the RoPE and the V^T repack all run
// in the GEMM's epilogue.
int qkv_project(dit_handle* hd, int l, int n, RopeGrid g, void* q_out, void* k_out, void* vt_out, int cap) {
  const dit_config& c = hd->cfg;
  const Layout& L = hd->lay;
  const int D = c.D;
  hipStream_t s = hd->stream;
  const char* big = hd->X<char>(L.big);
  GemmEpi e{};
  e.bias = hd->B(l, DIT_WB_QKV_B); e.out = hd->X(L.big); e.ldo = 3 * D;
  if (gemm_qknorm_fits(c.dtype, n, 3 * D, c.dh)) {
    e.kind = EPI_QKNORM;
    e.gq = hd->B(l, DIT_WB_GQ); e.gk = hd->B(l, DIT_WB_GK);
    e.q_out = q_out; e.k_out = k_out; e.vt_out = vt_out; e.vcap = cap;
    e.D = D; e.kpad = round64(n); e.rope = 1;
    e.q_scale = attention_q_scale(c.dh); e.eps = (float)c.eps; e.log2_theta = (float)std::log2(c.rope_theta);
    e.g = g;
    return block_gemm(hd, hd->X(L.u), D, hd->B(l, DIT_WB_QKV_W), D, n, 3 * D, D, e);
  }
  e.kind = EPI_BIAS;
  if (int rc = block_gemm(hd, hd->X(L.u), D, hd->B(l, DIT_WB_QKV_W), D, n, 3 * D, D, e)) return rc;
  HIPCHK(qknorm_rope(c.dtype, c.dh, c.H, n, q_out ? big : nullptr, big + (size_t)D * L.elt,
                     big + (size_t)2 * D * L.elt, 3 * D, hd->B(l, DIT_WB_GQ), hd->B(l, DIT_WB_GK), 1, g,
                     (float)c.eps, (float)c.rope_theta, attention_q_scale(c.dh), q_out, k_out, vt_out, cap, s));
  return DIT_OK;
}

// One context pass (reference, boundary or interpolation anchor) at t = 0: writes K
// (normed, rotated) and V of every block into kdst[l] / vdst[l] (capacity cap).  The
// tokens attend to the earlier context segments and themselves: nprior 0 (reference:
// itself only), 1 (boundary: reference), 2 (anchor: reference and, if held, boundary).
int context_pass_run(dit_handle* hd, const float* z, int n, RopeGrid g, const std::vector<size_t>& kdst,
                     const std::vector<size_t>& vdst, int cap, int nprior) {
  const dit_config& c = hd->cfg;
  const Layout& L = hd->lay;
  const int D = c.D, F = L.F;
  hipStream_t s = hd->stream;
  float* mod = hd->X<float>(L.mod);
  const float* tab = mod_table_entry(hd, 0.0);
  if (!tab)
    HIPCHK(modulation(c.dtype, D, 0, 0.0, hd->W(DIT_W_T1_W), hd->W(DIT_W_T1_B), hd->W(DIT_W_T2_W),
                      hd->W(DIT_W_T2_B), nullptr, nullptr, hd->W(DIT_W_FMOD_W), hd->W(DIT_W_FMOD_B),
                      hd->X<float>(L.tmp), mod, mod + (size_t)c.L * 6 * D, s));
  const float* cvec = hd->X<float>(L.tmp) + 256 + D;
  float* h = hd->X<float>(L.h);
  if (const int rc = embed(hd, z, n, nullptr, 0, g, h)) return rc;
  GemmEpi e{};
  for (int l = 0; l < c.L; ++l) {
    const float* m = (tab ? tab : mod) + (size_t)l * 6 * D;
    const bool last = l == c.L - 1;
    if (int rc = block_begin(hd, l)) return rc;
    if (!tab)
      HIPCHK(block_modulation(c.dtype, D, hd->B(l, DIT_WB_MOD_W), hd->B(l, DIT_WB_MOD_B), cvec,
                              mod + (size_t)l * 6 * D, s));
    if (int rc = block_norm(hd, h, n, m + 0 * D, m + 1 * D, hd->X(L.u))) return rc;
    if (int rc = qkv_project(hd, l, n, g, last ? nullptr : hd->X(L.q), hd->S(kdst[l]), hd->S(vdst[l]), cap))
      return rc;
    if (last) {
      if (int rc = block_end(hd, l)) return rc;
      break;
    }
    AttnSeg seg[3];
    int ns = 0;
    if (nprior >= 1) seg[ns++] = AttnSeg{hd->S(L.kref[l]), hd->S(L.vref[l]), hd->n_ref, L.cap_ref};
    if (nprior >= 2 && hd->n_bnd > 0) seg[ns++] = AttnSeg{hd->S(L.kbnd[l]), hd->S(L.vbnd[l]), hd->n_bnd, L.cap_bnd};
    seg[ns++] = AttnSeg{hd->S(kdst[l]), hd->S(vdst[l]), n, cap};
    int rc = run_attention(hd, n, seg, ns, true, ATTN_SELF, l);
    if (rc) return rc;
    e = GemmEpi{};
    e.kind = EPI_RESID; e.bias = hd->B(l, DIT_WB_O_B); e.out = h; e.ldo = D; e.gate = m + 2 * D;
    e.ws = hd->X<float>(L.opart); e.ws_floats = (long long)L.part_rows * D;
    if ((rc = block_gemm(hd, hd->X(L.o), D, hd->B(l, DIT_WB_O_W), D, n, D, D, e))) return rc;
    if ((rc = block_norm(hd, h, n, m + 3 * D, m + 4 * D, hd->X(L.u)))) return rc;
    e = GemmEpi{};
    e.kind = EPI_GELU; e.bias = hd->B(l, DIT_WB_FC1_B); e.out = hd->X(L.big); e.ldo = F;
    if ((rc = block_gemm(hd, hd->X(L.u), D, hd->B(l, DIT_WB_FC1_W), D, n, F, D, e))) return rc;
    e = GemmEpi{};
    e.kind = EPI_RESID; e.bias = hd->B(l, DIT_WB_FC2_B); e.out = h; e.ldo = D; e.gate = m + 5 * D;
    e.ws = hd->X<float>(L.opart); e.ws_floats = (long long)L.part_rows * D;
    if ((rc = block_gemm(hd, hd->X(L.big), F, hd->B(l, DIT_WB_FC2_W), F, n, D, F, e))) return rc;
    if ((rc = block_end(hd, l))) return rc;
  }
  return DIT_OK;
}

int context_pass(dit_handle* hd, const float* z, int n, RopeGrid g, const std::vector<size_t>& kdst,
                 const std::vector<size_t>& vdst, int cap, int nprior) {
  int rc = pass_begin(hd);
  if (!rc) rc = context_pass_run(hd, z, n, g, kdst, vdst, cap, nprior);
  return pass_end(hd, rc);
}

bool grid_ok(const dit_grid& g) { return g.frames >= 1 && g.h >= 1 && g.w >= 1; }
long long grid_n(const dit_grid& g) { return (long long)g.frames * g.h * g.w; }

}  // namespace

extern "C" {

int dit_weight_count(const dit_config* cfg) {
  if (check_config(cfg)) return 0;
  return DIT_W_GLOBAL_COUNT + cfg->L * DIT_W_BLOCK_COUNT;
}

size_t dit_state_bytes(const dit_config* cfg) {
  if (check_config(cfg)) return 0;
  return make_layout(cfg).state_total;
}

size_t dit_workspace_bytes(const dit_config* cfg) {
  if (check_config(cfg)) return 0;
  return make_layout(cfg).ws_total;
}

int dit_create(const dit_config* cfg, const void* const* weights, void* state, size_t state_bytes,
               void* workspace, size_t workspace_bytes, void* hip_stream, dit_handle** out) {
  if (!out) return fail(DIT_EINVAL, "out is NULL");
  *out = nullptr;
  int rc = check_config(cfg);
  if (rc) return rc;
  if (!weights) return fail(DIT_EINVAL, "weights is NULL");
  if (!state || !workspace) return fail(DIT_EINVAL, "state/workspace is NULL");
  if (((uintptr_t)state & 255) || ((uintptr_t)workspace & 255))
    return fail(DIT_EINVAL, "state/workspace must be 256-byte aligned");
  Layout L = make_layout(cfg);
  if (state_bytes < L.state_total)
    return fail(DIT_EWORKSPACE, "state %zu bytes < required %zu", state_bytes, L.state_total);
  if (workspace_bytes < L.ws_total)
    return fail(DIT_EWORKSPACE, "workspace %zu bytes < required %zu", workspace_bytes, L.ws_total);
  const int nw = DIT_W_GLOBAL_COUNT + cfg->L * DIT_W_BLOCK_COUNT;
  for (int i = 0; i < nw; ++i) {
    const int j = i < DIT_W_GLOBAL_COUNT ? -1 : (i - DIT_W_GLOBAL_COUNT) % DIT_W_BLOCK_COUNT;
    const bool cross = j >= DIT_WB_CQ_W && j <= DIT_WB_CO_B;
    if (!weights[i] && !(cross && cfg->d_a == 0)) return fail(DIT_EINVAL, "weight %d is NULL", i);
    if (weights[i] && ((uintptr_t)weights[i] & 15)) return fail(DIT_EINVAL, "weight %d not 16-byte aligned", i);
  }
  dit_handle* h = new dit_handle();
  h->cfg = *cfg;
  h->lay = L;
  h->w.assign(weights, weights + nw);
  h->state = static_cast<char*>(state);
  h->ws = static_cast<char*>(workspace);
  h->stream = static_cast<hipStream_t>(hip_stream);
  *out = h;
  return DIT_OK;
}

int dit_destroy(dit_handle* h) {
  if (!h) return DIT_OK;
  for (auto& t : h->tm)
    for (auto& e : t.ev) (void)hipEventDestroy(e);
  if (h->st.copy) {
    (void)hipStreamSynchronize(h->st.copy);
    for (auto& e : h->st.ready) (void)hipEventDestroy(e);
    for (auto& e : h->st.freed) (void)hipEventDestroy(e);
    (void)hipStreamDestroy(h->st.copy);
  }
  delete h;
  return DIT_OK;
}

size_t dit_block_weight_bytes(const dit_config* cfg) {
  if (check_config(cfg)) return 0;
  size_t off[DIT_W_BLOCK_COUNT], bytes[DIT_W_BLOCK_COUNT];
  return block_slot_layout(*cfg, off, bytes);
}

int dit_weight_stream(dit_handle* h, const void* const* host_blocks, void* ring, size_t ring_bytes,
                      int nslot) {
  if (!h) return fail(DIT_EINVAL, "handle is NULL");
  const dit_config& c = h->cfg;
  Streaming& st = h->st;
  if (!host_blocks) {
    if (ring || nslot) return fail(DIT_EINVAL, "host_blocks NULL: ring and nslot must be NULL/0");
    if (st.copy) HIPCHK(hipStreamSynchronize(st.copy));
    st.on = false;
    return DIT_OK;
  }
  if (nslot < 1 || nslot > c.L) return fail(DIT_EINVAL, "nslot=%d out of [1, L=%d]", nslot, c.L);
  if (!ring || ((uintptr_t)ring & 255)) return fail(DIT_EINVAL, "ring NULL or not 256-byte aligned");
  size_t off[DIT_W_BLOCK_COUNT], bytes[DIT_W_BLOCK_COUNT];
  const size_t slot = block_slot_layout(c, off, bytes);
  if (ring_bytes < slot * (size_t)nslot)
    return fail(DIT_EWORKSPACE, "ring %zu bytes < %d slots x %zu", ring_bytes, nslot, slot);
  for (int l = 0; l < c.L; ++l)
    for (int i = 0; i < DIT_W_BLOCK_COUNT; ++i)
      if (bytes[i] && !host_blocks[(size_t)l * DIT_W_BLOCK_COUNT + i])
        return fail(DIT_EINVAL, "host block %d entry %d is NULL", l, i);
  if (!st.copy) {
    HIPCHK(hipStreamCreateWithFlags(&st.copy, hipStreamNonBlocking));
  } else {
    HIPCHK(hipStreamSynchronize(st.copy));
  }
  for (int k = (int)st.ready.size(); k < nslot; ++k) {
    hipEvent_t a, b;
    HIPCHK(hipEventCreateWithFlags(&a, hipEventDisableTiming));
    st.ready.push_back(a);
    HIPCHK(hipEventCreateWithFlags(&b, hipEventDisableTiming));
    st.freed.push_back(b);
  }
  st.host.assign(host_blocks, host_blocks + (size_t)c.L * DIT_W_BLOCK_COUNT);
  st.ring = static_cast<char*>(ring);
  st.nslot = nslot;
  st.slot_bytes = slot;
  for (int i = 0; i < DIT_W_BLOCK_COUNT; ++i) { st.off[i] = off[i]; st.bytes[i] = bytes[i]; }
  st.holds.assign(nslot, -1);
  st.freed_rec.assign(nslot, 0);
  st.base = 0;
  st.issued = 0;
  st.on = true;
  // Prefetch: the first blocks start moving now, alongside whatever the handle's
  // stream is still running (e.g. passes on the resident weights).
  if (int rc = stream_issue_upto(h, nslot)) {
    st.on = false;
    return rc;
  }
  return DIT_OK;
}

int ref_kv_precompute(dit_handle* h, const float* ref, dit_grid grid) {
  if (!h) return fail(DIT_EINVAL, "handle is NULL");
  if (!ref) return fail(DIT_EINVAL, "ref is NULL");
  if (!grid_ok(grid)) return fail(DIT_ESHAPE, "empty reference grid");
  const long long n = grid_n(grid);
  if (n > h->cfg.max_ref) return fail(DIT_ESHAPE, "reference tokens %lld > max_ref %d", n, h->cfg.max_ref);
  h->has_ref = false;
  h->n_bnd = 0;
  h->n_anc = 0;
  RopeGrid g{grid.t0, grid.frames, grid.h, grid.w};
  int rc = context_pass(h, ref, (int)n, g, h->lay.kref, h->lay.vref, h->lay.cap_ref, 0);
  if (rc) return rc;
  h->n_ref = (int)n;
  h->has_ref = true;
  return DIT_OK;
}

int boundary_kv_carry(dit_handle* h, const float* x_prev, dit_grid prev) {
  if (!h) return fail(DIT_EINVAL, "handle is NULL");
  if (prev.frames == 0) {
    h->n_bnd = 0;
    h->n_anc = 0;
    return DIT_OK;
  }
  if (!x_prev) return fail(DIT_EINVAL, "x_prev is NULL");
  if (!grid_ok(prev)) return fail(DIT_ESHAPE, "bad previous-chunk grid");
  const long long n = (long long)prev.h * prev.w;
  if (n > h->cfg.max_bnd) return fail(DIT_ESHAPE, "boundary tokens %lld > max_bnd %d", n, h->cfg.max_bnd);
  if (!h->has_ref) return fail(DIT_ESTATE, "boundary_kv_carry before ref_kv_precompute");
  h->n_bnd = 0;
  h->n_anc = 0;  // an anchor's K/V depend on the boundary they were computed with
  const float* last = x_prev + (size_t)(prev.frames - 1) * n * h->cfg.c_p;
  RopeGrid g{-1, 1, prev.h, prev.w};
  int rc = context_pass(h, last, (int)n, g, h->lay.kbnd, h->lay.vbnd, h->lay.cap_bnd, 1);
  if (rc) return rc;
  h->n_bnd = (int)n;
  return DIT_OK;
}

int audio_kv_precompute(dit_handle* h, const float* audio, int M) {
  if (!h) return fail(DIT_EINVAL, "handle is NULL");
  const dit_config& c = h->cfg;
  if (M == 0) {
    if (audio) return fail(DIT_EINVAL, "audio given with M=0");
    h->n_aud = 0;
    h->aud_pend.clear();
    return DIT_OK;
  }
  if (!audio) return fail(DIT_EINVAL, "audio is NULL with M=%d", M);
  if (c.d_a == 0) return fail(DIT_EINVAL, "audio given but d_a=0");
  if (M < 0 || M > c.max_audio) return fail(DIT_ESHAPE, "M=%d out of [1, max_audio=%d]", M, c.max_audio);
  h->n_aud = 0;
  h->aud_pend.clear();
  RopeGrid g0{0, 1, 1, 1};
  HIPCHK(patch_input(c.dtype, audio, M, c.d_a, nullptr, 0, 0, g0, h->S(h->lay.aud_in), h->stream));
  if (h->st.on) {
    // Streamed weights: a pass of its own would copy every block slot for two small
    // Linears; instead each block's K/V is computed at the next pass's block_begin.
    h->aud_pend.assign(c.L, 1);
    h->n_aud = M;
    return DIT_OK;
  }
  int rc = pass_begin(h);
  for (int l = 0; l < c.L && !rc; ++l) {
    rc = block_begin(h, l);
    if (!rc)
      rc = audio_kv(h, l, M, h->S(h->lay.aud_in), h->S(h->lay.kaud[l]), h->S(h->lay.vaud[l]),
                    h->lay.fold ? h->S(h->lay.uta[l]) : nullptr);
    if (!rc) rc = block_end(h, l);
  }
  if ((rc = pass_end(h, rc))) return rc;
  h->n_aud = M;
  return DIT_OK;
}

int dit_modulation_table(dit_handle* h, const double* t, int nt) {
  if (!h) return fail(DIT_EINVAL, "handle is NULL");
  if (nt < 0 || nt > DIT_MOD_TABLE_MAX) return fail(DIT_EINVAL, "nt=%d out of [0, %d]", nt, DIT_MOD_TABLE_MAX);
  if (nt > 0 && !t) return fail(DIT_EINVAL, "t is NULL with nt=%d", nt);
  for (int j = 0; j < nt; ++j)
    if (!std::isfinite(t[j])) return fail(DIT_EINVAL, "t[%d] is not finite", j);
  static_assert(DIT_MOD_TABLE_MAX <= MOD_BATCH, "one batched launch per weight matrix");
  h->mod_t.clear();
  if (nt == 0) return DIT_OK;
  const dit_config& c = h->cfg;
  const Layout& L = h->lay;
  const int D = c.D;
  hipStream_t s = h->stream;
  // scratch: the attention partials, unused between passes; the conditioning c[j] after
  // the feature and hidden rows of timestep_cond_batch
  if ((size_t)MOD_BATCH * (256 + 2 * D) > (size_t)L.part_rows * D)
    return fail(DIT_EWORKSPACE, "modulation scratch exceeds the partial buffer");
  float* tmp = h->X<float>(L.opart);
  float* cv = tmp + (size_t)MOD_BATCH * (256 + D);
  float* tab = h->S<float>(L.modtab);
  const int E = (int)L.mod_entry;
  HIPCHK(timestep_cond_batch(c.dtype, D, t, nt, h->W(DIT_W_T1_W), h->W(DIT_W_T1_B), h->W(DIT_W_T2_W),
                             h->W(DIT_W_T2_B), tmp, cv, s));
  HIPCHK(gemv_batch(c.dtype, 2 * D, D, h->W(DIT_W_FMOD_W), h->W(DIT_W_FMOD_B), cv, D, nt,
                    tab + (size_t)c.L * 6 * D, E, s));
  int rc = pass_begin(h);
  for (int l = 0; l < c.L && !rc; ++l) {
    rc = block_begin(h, l);
    if (!rc && gemv_batch(c.dtype, 6 * D, D, h->B(l, DIT_WB_MOD_W), h->B(l, DIT_WB_MOD_B), cv, D, nt,
                          tab + (size_t)l * 6 * D, E, s) != hipSuccess)
      rc = fail(DIT_EHIP, "gemv_batch: %s", hipGetErrorString(hipGetLastError()));
    if (!rc) rc = block_end(h, l);
  }
  if ((rc = pass_end(h, rc))) return rc;
  h->mod_t.assign(t, t + nt);
  return DIT_OK;
}

int interp_anchor_kv(dit_handle* h, const float* x_next, dit_grid next, int t_pos) {
  if (!h) return fail(DIT_EINVAL, "handle is NULL");
  if (next.frames == 0) {
    h->n_anc = 0;
    return DIT_OK;
  }
  if (!x_next) return fail(DIT_EINVAL, "x_next is NULL");
  if (!grid_ok(next)) return fail(DIT_ESHAPE, "bad next-chunk grid");
  const long long n = (long long)next.h * next.w;
  if (n > h->cfg.max_bnd) return fail(DIT_ESHAPE, "anchor tokens %lld > max_bnd %d", n, h->cfg.max_bnd);
  if (!h->has_ref) return fail(DIT_ESTATE, "interp_anchor_kv before ref_kv_precompute");
  h->n_anc = 0;
  RopeGrid g{t_pos, 1, next.h, next.w};  // frame 0 of the next chunk, placed at t = t_pos
  int rc = context_pass(h, x_next, (int)n, g, h->lay.kanc, h->lay.vanc, h->lay.cap_bnd, 2);
  if (rc) return rc;
  h->n_anc = (int)n;
  return DIT_OK;
}

namespace {

// One denoising step; with carry, also the boundary by reuse (see dit_chunk_step_carry).
// The kernels of one denoising step (arguments checked by chunk_step).
int chunk_pass(dit_handle* hd, float* x, const float* cond, const float* audio, int M, dit_grid chunk,
               double t, double t_next, float* v_out, bool carry) {
  const dit_config& c = hd->cfg;
  const Layout& L = hd->lay;
  const long long hw = (long long)chunk.h * chunk.w;
  const int n = (int)grid_n(chunk), D = c.D, F = L.F;
  hipStream_t s = hd->stream;
  RopeGrid g{chunk.t0, chunk.frames, chunk.h, chunk.w};
  float* mod = hd->X<float>(L.mod);
  const float* tab = mod_table_entry(hd, t);
  const float* fmod = (tab ? tab : mod) + (size_t)c.L * 6 * D;
  if (!tab)
    HIPCHK(modulation(c.dtype, D, 0, t, hd->W(DIT_W_T1_W), hd->W(DIT_W_T1_B), hd->W(DIT_W_T2_W),
                      hd->W(DIT_W_T2_B), nullptr, nullptr, hd->W(DIT_W_FMOD_W), hd->W(DIT_W_FMOD_B),
                      hd->X<float>(L.tmp), mod, mod + (size_t)c.L * 6 * D, s));
  const float* cvec = hd->X<float>(L.tmp) + 256 + D;
  const bool held = M == DIT_AUDIO_HELD;
  const bool cross = held || (M > 0 && c.d_a > 0);
  if (cross && !held)
    HIPCHK(patch_input(c.dtype, audio, M, c.d_a, nullptr, 0, 0, g, hd->X(L.ain), s));
  float* h = hd->X<float>(L.h);
  if (const int rc = embed(hd, x, n, cond, c.c_c ? c.cond_up : 0, g, h)) return rc;
  GemmEpi e{};
  const char* big = hd->X<char>(L.big);
  for (int l = 0; l < c.L; ++l) {
    const float* m = (tab ? tab : mod) + (size_t)l * 6 * D;
    if (int rc = block_begin(hd, l)) return rc;
    if (!tab)
      HIPCHK(block_modulation(c.dtype, D, hd->B(l, DIT_WB_MOD_W), hd->B(l, DIT_WB_MOD_B), cvec,
                              mod + (size_t)l * 6 * D, s));
    // self-attention
    if (int rc = block_norm(hd, h, n, m + 0 * D, m + 1 * D, hd->X(L.u))) return rc;
    if (int rc = qkv_project(hd, l, n, g, hd->X(L.q), hd->X(L.kc), hd->X(L.vtc), L.cap_tok)) return rc;
    AttnSeg seg[ATTN_MAX_SEGS];
    int ns = 0;
    seg[ns++] = AttnSeg{hd->S(L.kref[l]), hd->S(L.vref[l]), hd->n_ref, L.cap_ref};
    if (hd->n_bnd > 0) seg[ns++] = AttnSeg{hd->S(L.kbnd[l]), hd->S(L.vbnd[l]), hd->n_bnd, L.cap_bnd};
    if (hd->n_anc > 0) seg[ns++] = AttnSeg{hd->S(L.kanc[l]), hd->S(L.vanc[l]), hd->n_anc, L.cap_bnd};
    seg[ns++] = AttnSeg{hd->X(L.kc), hd->X(L.vtc), n, L.cap_tok};
    int rc = run_attention(hd, n, seg, ns, true, ATTN_SELF, l);
    if (rc) return rc;
    if (carry) {
      // This block's attention has read its boundary slot; refill it with the last
      // frame's K (moved from t0 + frames - 1 to t = -1) and V of this step.
      const int first = (chunk.frames - 1) * (int)hw;
      const float dt = (float)(-1 - (chunk.t0 + chunk.frames - 1));
      HIPCHK(boundary_reuse(c.dtype, c.dh, c.H, hd->X(L.kc), hd->X(L.vtc), L.cap_tok, first, (int)hw, dt,
                            (float)c.rope_theta, hd->S(L.kbnd[l]), hd->S(L.vbnd[l]), L.cap_bnd, s));
    }
    e = GemmEpi{};
    e.kind = EPI_RESID; e.bias = hd->B(l, DIT_WB_O_B); e.out = h; e.ldo = D; e.gate = m + 2 * D;
    e.ws = hd->X<float>(L.opart); e.ws_floats = (long long)L.part_rows * D;
    if ((rc = block_gemm(hd, hd->X(L.o), D, hd->B(l, DIT_WB_O_W), D, n, D, D, e))) return rc;
    // audio cross-attention
    if (cross) {
      if ((rc = block_norm(hd, h, n, nullptr, nullptr, hd->X(L.u)))) return rc;
      // the audio keys and values: held, or from this step's audio
      AttnSeg aseg{hd->S(L.kaud[l]), hd->S(L.vaud[l]), hd->n_aud, L.cap_audio};
      void* uta = L.fold ? hd->S(L.uta[l]) : nullptr;
      if (!held) {
        uta = L.fold ? hd->X(L.uta_ws) : nullptr;
        if (int rc2 = audio_kv(hd, l, M, hd->X(L.ain), hd->X(L.ka), hd->X(L.vat), uta)) return rc2;
        aseg = AttnSeg{hd->X(L.ka), hd->X(L.vat), M, L.cap_audio};
      }
      const int HK = c.H * 64;
      e = GemmEpi{};
      e.bias = hd->B(l, DIT_WB_CQ_B); e.out = hd->X(L.big); e.ldo = D;
      if (uta && gemm_qknorm_fits(c.dtype, n, D, c.dh)) {
        // folded, and the softmax in the cross-q GEMM's epilogue: P [n, H*64] directly
        e.kind = EPI_QKNORM_X; e.gq = hd->B(l, DIT_WB_GCQ); e.D = D;
        e.q_scale = attention_q_scale(c.dh); e.eps = (float)c.eps; e.g = g;
        e.xk = aseg.k; e.xn = aseg.n; e.p_out = hd->X(L.o); e.ldp = HK;
        if ((rc = block_gemm(hd, hd->X(L.u), D, hd->B(l, DIT_WB_CQ_W), D, n, D, D, e))) return rc;
      } else {
        if (gemm_qknorm_fits(c.dtype, n, D, c.dh)) {  // q-norm in the GEMM epilogue (no RoPE)
          e.kind = EPI_QKNORM; e.gq = hd->B(l, DIT_WB_GCQ); e.q_out = hd->X(L.q); e.D = D;
          e.q_scale = attention_q_scale(c.dh); e.eps = (float)c.eps; e.g = g;
          if ((rc = block_gemm(hd, hd->X(L.u), D, hd->B(l, DIT_WB_CQ_W), D, n, D, D, e))) return rc;
        } else {
          e.kind = EPI_BIAS;
          if ((rc = block_gemm(hd, hd->X(L.u), D, hd->B(l, DIT_WB_CQ_W), D, n, D, D, e))) return rc;
          HIPCHK(qknorm_rope(c.dtype, c.dh, c.H, n, big, nullptr, nullptr, D, hd->B(l, DIT_WB_GCQ),
                             nullptr, 0, g, (float)c.eps, (float)c.rope_theta, attention_q_scale(c.dh),
                             hd->X(L.q), nullptr, nullptr, L.cap_tok, s));
        }
        if (uta) {  // folded: P [n, H*64] from the short softmax
          HIPCHK(short_attention_probs(c.dh, c.H, hd->X(L.q), D, hd->X(L.o), HK, n, aseg, true, s));
        } else {
          if (int rc2 = run_attention(hd, n, &aseg, 1, false, ATTN_CROSS, l)) return rc2;
        }
      }
      e = GemmEpi{};
      e.kind = EPI_RESID; e.bias = hd->B(l, DIT_WB_CO_B); e.out = h; e.ldo = D; e.gate = nullptr;
      e.ws = hd->X<float>(L.opart); e.ws_floats = (long long)L.part_rows * D;
      if (uta)  // h += P U^T + b_co
        rc = block_gemm(hd, hd->X(L.o), HK, uta, HK, n, D, HK, e);
      else
        rc = block_gemm(hd, hd->X(L.o), D, hd->B(l, DIT_WB_CO_W), D, n, D, D, e);
      if (rc) return rc;
    }
    // MLP
    if ((rc = block_norm(hd, h, n, m + 3 * D, m + 4 * D, hd->X(L.u)))) return rc;
    e = GemmEpi{};
    e.kind = EPI_GELU; e.bias = hd->B(l, DIT_WB_FC1_B); e.out = hd->X(L.big); e.ldo = F;
    if ((rc = block_gemm(hd, hd->X(L.u), D, hd->B(l, DIT_WB_FC1_W), D, n, F, D, e))) return rc;
    e = GemmEpi{};
    e.kind = EPI_RESID; e.bias = hd->B(l, DIT_WB_FC2_B); e.out = h; e.ldo = D; e.gate = m + 5 * D;
    e.ws = hd->X<float>(L.opart); e.ws_floats = (long long)L.part_rows * D;
    if ((rc = block_gemm(hd, hd->X(L.big), F, hd->B(l, DIT_WB_FC2_W), F, n, D, F, e))) return rc;
    if ((rc = block_end(hd, l))) return rc;
  }
  // final layer + Euler
  if (final_layer_fits(c.dtype, D, c.c_p)) {
    // bytes: h read (fp32), x read and written, v written, the weights and vectors
    const hipEvent_t* ev = timed_ev(hd, DIT_TIME_ELEM);
    HIPCHK(final_layer(h, n, D, fmod, fmod + D, (float)c.eps, hd->W(DIT_W_FIN_W), hd->W(DIT_W_FIN_B),
                       (float)(t_next - t), x, v_out, s, ev));
    timed_done(hd, DIT_TIME_ELEM, ev,
               (double)n * D * 4 + (double)n * c.c_p * 4 * (v_out ? 3 : 2) + (double)c.c_p * (D + 1) * L.elt +
                   2.0 * D * 4);
    return DIT_OK;
  }
  if (int rc = block_norm(hd, h, n, fmod, fmod + D, hd->X(L.u))) return rc;
  e = GemmEpi{};
  e.kind = EPI_EULER; e.bias = hd->W(DIT_W_FIN_B); e.out = x; e.ldo = c.c_p; e.v_out = v_out;
  e.dt = (float)(t_next - t);
  HIPCHK(gemm(c.dtype, hd->X(L.u), D, hd->W(DIT_W_FIN_W), D, n, c.c_p, D, e, s));
  return DIT_OK;
}

int chunk_step(dit_handle* hd, float* x, const float* cond, const float* audio, int M,
               dit_grid chunk, double t, double t_next, float* v_out, bool carry) {
  if (!hd) return fail(DIT_EINVAL, "handle is NULL");
  const dit_config& c = hd->cfg;
  const Layout& L = hd->lay;
  if (!x) return fail(DIT_EINVAL, "x is NULL");
  if (!std::isfinite(t) || !std::isfinite(t_next)) return fail(DIT_EINVAL, "t/t_next not finite");
  if (!grid_ok(chunk)) return fail(DIT_ESHAPE, "empty chunk grid");
  const long long nn = grid_n(chunk);
  if (nn > c.max_tokens) return fail(DIT_ESHAPE, "chunk tokens %lld > max_tokens %d", nn, c.max_tokens);
  if (c.c_c > 0 && !cond) return fail(DIT_EINVAL, "cond is NULL but c_c=%d", c.c_c);
  if (c.c_c == 0 && cond) return fail(DIT_EINVAL, "cond given but c_c=0");
  if (c.c_c > 0 && c.cond_up == 2 && (chunk.h % 2 || chunk.w % 2))
    return fail(DIT_ESHAPE, "cond_up=2 needs even h and w");
  if (M == DIT_AUDIO_HELD) {
    if (audio) return fail(DIT_EINVAL, "audio given with M=DIT_AUDIO_HELD");
    if (hd->n_aud == 0) return fail(DIT_ESTATE, "M=DIT_AUDIO_HELD but no audio K/V held (audio_kv_precompute)");
  } else if (M < 0 || M > c.max_audio) {
    return fail(DIT_ESHAPE, "M=%d out of [0, max_audio=%d]", M, c.max_audio);
  }
  if (M > 0 && !audio) return fail(DIT_EINVAL, "audio is NULL with M=%d", M);
  if (M > 0 && c.d_a == 0) return fail(DIT_EINVAL, "audio given but d_a=0");
  const long long hw = (long long)chunk.h * chunk.w;
  if (carry && hw > c.max_bnd)
    return fail(DIT_ESHAPE, "boundary by reuse: frame of %lld tokens > max_bnd %d", hw, c.max_bnd);
  if (!hd->has_ref) return fail(DIT_ESTATE, "dit_chunk_step before ref_kv_precompute");

  int rc = pass_begin(hd);
  if (!rc) rc = chunk_pass(hd, x, cond, audio, M, chunk, t, t_next, v_out, carry);
  if ((rc = pass_end(hd, rc))) return rc;
  if (carry) {
    hd->n_bnd = (int)hw;
    hd->n_anc = 0;
  }
  return DIT_OK;
}

}  // namespace

int dit_chunk_step(dit_handle* hd, float* x, const float* cond, const float* audio, int M,
                   dit_grid chunk, double t, double t_next, float* v_out) {
  return chunk_step(hd, x, cond, audio, M, chunk, t, t_next, v_out, false);
}

int dit_chunk_step_carry(dit_handle* hd, float* x, const float* cond, const float* audio, int M,
                         dit_grid chunk, double t, double t_next, float* v_out) {
  return chunk_step(hd, x, cond, audio, M, chunk, t, t_next, v_out, true);
}

int fm_euler_step(float* x, const float* v, double dt, long long n, void* hip_stream) {
  if (n < 0) return fail(DIT_EINVAL, "n < 0");
  if (n == 0) return DIT_OK;
  if (!x || !v) return fail(DIT_EINVAL, "x or v is NULL");
  if (!std::isfinite(dt)) return fail(DIT_EINVAL, "dt not finite");
  if (((uintptr_t)x & 15) || ((uintptr_t)v & 15)) return fail(DIT_EINVAL, "x, v must be 16-byte aligned");
  HIPCHK(euler(x, v, (float)dt, n, static_cast<hipStream_t>(hip_stream)));
  return DIT_OK;
}

int fm_noise_to(float* x, const float* z, const float* eps, double t, long long n, void* hip_stream) {
  if (n < 0) return fail(DIT_EINVAL, "n < 0");
  if (n == 0) return DIT_OK;
  if (!x || !z || !eps) return fail(DIT_EINVAL, "x, z or eps is NULL");
  if (!std::isfinite(t)) return fail(DIT_EINVAL, "t not finite");
  if (((uintptr_t)x & 15) || ((uintptr_t)z & 15) || ((uintptr_t)eps & 15))
    return fail(DIT_EINVAL, "x, z, eps must be 16-byte aligned");
  HIPCHK(noise_to(x, z, eps, (float)(1.0 - t), (float)t, n, static_cast<hipStream_t>(hip_stream)));
  return DIT_OK;
}

const char* dit_last_error(void) { return g_err.c_str(); }

int dit_timing_enable(dit_handle* h, int enable) {
  if (!h) return fail(DIT_EINVAL, "handle is NULL");
  if (enable < 0 || enable >= (1 << DIT_TIME_KINDS)) return fail(DIT_EINVAL, "enable mask %d", enable);
  for (int k = 0; k < DIT_TIME_KINDS; ++k) {
    dit_handle::Timing& t = h->tm[k];
    t.on = false;
    t.used = 0;
    t.work = 0.0;
    if (!(enable & (1 << k))) continue;
    // Timing-only events, created here (not inside a timed region): no system-scope
    // fence when they complete (it would write back and invalidate the caches around
    // the timed launch).  Elapsed times are read after hipEventSynchronize, which needs
    // no memory ordering with the timed work.
    while (t.ev.size() < 2 * (size_t)MAX_EVENT_PAIRS) {
      hipEvent_t e;
      HIPCHK(hipEventCreateWithFlags(&e, hipEventDisableSystemFence));
      t.ev.push_back(e);
    }
    t.on = true;
  }
  return DIT_OK;
}

int dit_timing_read(dit_handle* h, int kind, int* count, double* total_ms, double* total_work) {
  if (!h || !count || !total_ms) return fail(DIT_EINVAL, "NULL argument");
  if (kind < 0 || kind >= DIT_TIME_KINDS) return fail(DIT_EINVAL, "kind %d", kind);
  dit_handle::Timing& t = h->tm[kind];
  double ms = 0.0;
  for (int i = 0; i < t.used; ++i) {
    HIPCHK(hipEventSynchronize(t.ev[2 * (size_t)i + 1]));
    float f = 0.f;
    HIPCHK(hipEventElapsedTime(&f, t.ev[2 * (size_t)i], t.ev[2 * (size_t)i + 1]));
    ms += f;
  }
  *count = t.used;
  *total_ms = ms;
  if (total_work) *total_work = t.work;
  t.used = 0;
  t.work = 0.0;
  return DIT_OK;
}

}  // extern "C"
