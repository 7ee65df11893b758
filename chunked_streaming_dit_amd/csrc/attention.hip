// Flash attention over segmented keys: [reference | boundary | chunk] (self-attention)
// or [audio] (cross-attention), one head per grid row.
//
// Per workgroup: 256 queries of one head (8 waves x 32 queries).  Key and V^T tiles of
// 64 keys are brought into LDS by direct-to-LDS transfers through two 3-slot rings, each
// tile requested about two tiles ahead of its use; one workgroup barrier per tile.  Each
// wave computes the transposed score tile S^T = K Q^T with 32x32 MFMAs, so that a lane
// holds scores of ONE query for 32 keys: the online-softmax row max needs one
// cross-lane exchange (lanes l and l^32), the row sum none until the end, and the
// rescale of the output accumulator O^T = V^T P^T touches only the lane's own
// registers.  The exponentiated scores feed the second MFMA directly from registers (no
// LDS round trip); the key order they are held in is matched by the stored order of V^T
// (see kernels.h).  Softmax statistics and accumulation are fp32; the softmax is taken
// in base 2 with log2(e)/sqrt(dh) folded into q (given pre-scaled, or applied here).
// When q and k are QK-normed (per-head RMSNorm times gamma), every logit is bounded by
// |q||k| <= q_scale dh max|gq| max|gk|; if that bound is small the weights 2^s cannot
// overflow and the softmax needs no running max at all: the common factor of numerator
// and denominator cancels, so the row max, its cross-lane exchange, the rescale test
// and the shift all drop out of the loop.
#include <hip/hip_ext.h>
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "attn_common.h"
#include "kernels.h"

namespace dit {

namespace {

struct AttnArgs {
  const void* q;
  void* o;
  int ldq, ldo, nq, ldk, H;
  int nseg;
  float scale;  // log2(e) / sqrt(dh), or 1 when q comes pre-scaled
  float thr;    // RESCALE_LOG2 / scale: lazy-rescale threshold in raw score units
  int nsplit;   // key-range splits per (head, q-tile) from q-tile qt0 on; > 1 writes partials
  int qt0;      // q-tiles [0, qt0) take the whole key range and write o directly
  float* opart; // [nsplit, nq, H*DH] normalised partial outputs (nsplit > 1)
  float* ml;    // [nsplit, nq, H, 2] (running max * scale, row sum) per partial
  // QK-norm gammas of q and k (or NULL) and the logit bound coefficient: every exp2-domain
  // logit is at most bcoef * max|gq| * max|gk| in magnitude (see attention()).
  const void* gq;
  const void* gk;
  float bcoef;
  AttnSeg seg[ATTN_MAX_SEGS];
};

constexpr int AW = 8;          // waves per workgroup (32 queries each)
constexpr int BQ = 32 * AW;    // queries per workgroup
static_assert(BQ == ATTN_QTILE, "q-tile of the split plan");
constexpr int NSLOT = 4;       // ring depth of the K and of the V^T tile rings
constexpr float RESCALE_LOG2 = 8.0f;
// Logit bound (exp2 domain) up to which the softmax is taken without a running max:
// 2^60 per weight, summed over at most 2^24 keys, stays far inside the fp32 range.
constexpr float NOMAX_BOUND = 60.0f;


// KIND only names the launch site in profiles (0: self-attention over the segmented
// keys, 1: audio cross-attention); the code is the same.
template <class T, int DH, int KIND>
__global__ __launch_bounds__(64 * AW, 2) void attn_kernel(AttnArgs a) {
  typedef typename Vec<T>::type V;
  constexpr int VE = Vec<T>::n;
  constexpr int SZ = (int)sizeof(T);
  constexpr int QV = DH / (2 * VE);       // 16-byte vector steps over dh
  constexpr int RBK = DH * SZ;            // bytes per key row
  constexpr int RBV = BKV * SZ;           // bytes per V^T row
  constexpr int RPK = 1024 / RBK;         // key rows per 1-KB load instruction
  constexpr int RPV = 1024 / RBV;         // V^T rows per 1-KB load instruction
  // The K and V^T tiles are moved by 4 of the 8 waves, one per SIMD: a wave stalled on
  // issuing a transfer then leaves its SIMD's MFMA pipe to the other wave (2-3% faster
  // than every wave loading, interleaved A/B on one board).
  constexpr int LW = 4;                       // loader waves
  constexpr int NLK = BKV * RBK / 1024 / LW;  // K load instructions per loader wave per tile
  constexpr int NLV = DH * RBV / 1024 / LW;   // V^T load instructions per loader wave per tile
  constexpr int DB = DH / 32;             // 32-row blocks of dh
  constexpr int KTILE = BKV * RBK, VTILE = DH * RBV;
  static_assert(RBK >= 128 && RBV >= 128 && NLK >= 1 && NLV >= 1 &&
                BKV * RBK == 1024 * LW * NLK && DH * RBV == 1024 * LW * NLV && LW <= AW, "tile");
  // LDS: NSLOT K slots and NSLOT V^T slots (separate rings, see the loop below).
  __shared__ __attribute__((aligned(1024))) char smem[NSLOT * (KTILE + VTILE)];
  char* const ks = smem;
  char* const vs = smem + NSLOT * KTILE;

  // The wave index is uniform; saying so keeps the loader waves' LDS destinations (M0)
  // and their branches scalar instead of per-lane values read back with readfirstlane.
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, lg = lane >> 5;
  // 1-D grid of two parts.  The first qt0 * H workgroups take q-tiles [0, qt0) over the
  // whole key range; the rest take q-tiles [qt0, nqt), each (head, q-tile) split into
  // nsplit contiguous parts of the key tiles.  The whole-range items come first, so they
  // are dispatched first and the shorter split items fill the last wave.  Within each
  // part the order is head-major and remapped so that each XCD works through a
  // contiguous range: the q-tiles of a head share that head's K/V in one L2.
  const int nqt = (a.nq + BQ - 1) / BQ;
  const int n1 = a.qt0 * a.H;
  int head, split, nsp, qt;
  if ((int)blockIdx.x < n1) {
    const int wi = xcd_remap(blockIdx.x, n1);
    head = wi / a.qt0;
    qt = wi - head * a.qt0;
    split = 0;
    nsp = 1;
  } else {
    const int nqs = nqt - a.qt0;
    const int wi = xcd_remap(blockIdx.x - n1, nqs * a.H * a.nsplit);
    const int hs = wi / nqs;  // head * nsplit + split
    head = hs / a.nsplit;
    split = hs - head * a.nsplit;
    nsp = a.nsplit;
    qt = a.qt0 + (wi - hs * nqs);
  }
  const int qrow = qt * BQ + wave * 32 + l32;
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

  // Offset-free softmax when the QK-norm bound allows it (uniform over the launch).
  int nomax = 0;
  if (a.gq) {
    const T* gq = reinterpret_cast<const T*>(a.gq);
    const T* gk = reinterpret_cast<const T*>(a.gk);
    float mq = 0.f, mk = 0.f;
    for (int i = lane; i < DH; i += 64) {
      mq = fmaxf(mq, fabsf(to_f(gq[i])));
      mk = fmaxf(mk, fabsf(to_f(gk[i])));
    }
    nomax = a.bcoef * wave_max(mq) * wave_max(mk) <= NOMAX_BOUND;
    nomax = __builtin_amdgcn_readfirstlane(nomax);
  }

  // Tiles of all segments in order: tile t lies in segment si at key offset base.
  // Tile counts of the segments, and prefix sums e1 <= e2 <= e3 = ntiles.
  int c[ATTN_MAX_SEGS];
#pragma unroll
  for (int i = 0; i < ATTN_MAX_SEGS; ++i) c[i] = i < a.nseg ? (a.seg[i].n + BKV - 1) / BKV : 0;
  static_assert(ATTN_MAX_SEGS == 4, "segment walk below");
  const int e1 = c[0], e2 = e1 + c[1], e3 = e2 + c[2];
  const int ntiles = e3 + c[3];
  const int tb = (int)((long long)ntiles * split / nsp);
  const int total = (int)((long long)ntiles * (split + 1) / nsp);  // tiles [tb, total)
  auto locate = [&](int t, int& si, int& base) {
    if (t < e1) { si = 0; base = t * BKV; }
    else if (t < e2) { si = 1; base = (t - e1) * BKV; }
    else if (t < e3) { si = 2; base = (t - e2) * BKV; }
    else { si = 3; base = (t - e3) * BKV; }
  };
  // Segment fields by runtime index (read from the kernel arguments; used only when a
  // walker enters a segment).
  auto seg_k = [&](int si) { return reinterpret_cast<const char*>(a.seg[si].k); };
  auto seg_vt = [&](int si) { return reinterpret_cast<const char*>(a.seg[si].vt); };
  auto seg_cap = [&](int si) { return a.seg[si].cap; };
  auto seg_n = [&](int si) { return a.seg[si].n; };
  auto seg_tiles = [&](int si) { return (a.seg[si].n + BKV - 1) / BKV; };
  // A walker follows one stream of consecutive key tiles: segment si, tiles left in it
  // (the current one included), and the byte offset of the current tile's first key
  // row (K) or column (V^T).  Advancing costs a few scalar operations; the segment
  // fields are looked up only when it enters the next (non-empty) segment.
  struct Walk {
    int si, left;
    const char* kp;  // K rows of the current tile
    const char* vp;  // V^T columns of the current tile
    int cap;         // V^T row pitch (keys) of the segment
  };
  auto walk_at = [&](int t) {
    int si, base;
    locate(t, si, base);
    Walk w;
    w.si = si;
    w.left = seg_tiles(si) - base / BKV;
    w.kp = seg_k(si) + (size_t)base * a.ldk * SZ;
    w.vp = seg_vt(si) + (size_t)base * SZ;
    w.cap = seg_cap(si);
    return w;
  };
  auto walk_next = [&](Walk& w) {
    w.kp += (size_t)BKV * a.ldk * SZ;
    w.vp += BKV * SZ;
    if (--w.left == 0) {
      do { ++w.si; } while (w.si < a.nseg && seg_tiles(w.si) == 0);
      if (w.si < a.nseg) {
        w.left = seg_tiles(w.si);
        w.kp = seg_k(w.si);
        w.vp = seg_vt(w.si);
        w.cap = seg_cap(w.si);
      }
    }
  };
  // Direct-to-LDS loads (buffer_load_dwordx4 ... lds through a buffer resource whose base
  // is the tile's first key row or column, so a load needs no per-lane address
  // arithmetic): instruction g = lw + LW i of loader wave lw fills 1 KB of a slot = rows
  // [RP g, RP g + RP); the lane covers row RP g + lane/(64/RP) at chunk position
  // lane % (64/RP), i.e. source chunk swz(row, position).  The other waves issue none
  // (their waits pass at once).  All offsets lie inside the segment (V^T under 2^31
  // bytes), below the resource's unlimited size.
  const int lw = wave % LW;
  unsigned koff[NLK];
#pragma unroll
  for (int i = 0; i < NLK; ++i) {
    const int g = lw + LW * i;
    const int r = RPK * g + lane / (64 / RPK);
    const int c = swz<RBK>(r, lane % (64 / RPK));
    koff[i] = (unsigned)((r * a.ldk + head * DH) * SZ + c * 16);
  }
  // V^T lane offsets depend on the segment's row pitch: computed when a new pitch comes.
  unsigned vvoff[NLV];
  int vcap = -1;
  auto load_k = [&](const Walk& w, int slot) {
    if (wave >= LW) return;  // wave-uniform
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)w.kp, (short)0, -1, 0x00020000);
    char* dst = ks + slot * KTILE + lw * 1024;
#pragma unroll
    for (int i = 0; i < NLK; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(dst + i * LW * 1024), 16,
                                               (int)koff[i], 0, 0, 0);
  };
  auto load_v = [&](const Walk& w, int slot) {
    if (wave >= LW) return;
    if (w.cap != vcap) {  // uniform
      vcap = w.cap;
#pragma unroll
      for (int i = 0; i < NLV; ++i) {
        const int g = lw + LW * i;
        const int row = RPV * g + lane / (64 / RPV);
        vvoff[i] = ((unsigned)(head * DH + row) * (unsigned)vcap) * SZ + swz<RBV>(row, lane % (64 / RPV)) * 16;
      }
    }
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)w.vp, (short)0, -1, 0x00020000);
    char* dst = vs + slot * VTILE + lw * 1024;
#pragma unroll
    for (int i = 0; i < NLV; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(dst + i * LW * 1024), 16,
                                               (int)vvoff[i], 0, 0, 0);
  };
  // S^T tile from a K slot: 2 blocks of 32 keys x 32 queries.  Lane: query l32,
  // key = 32 kb + 8 (e/4) + 4 lg + e%4 for element e.
  const int kx = l32;  // swizzle row term: fragment rows are l32 + multiples of 32
  auto scores = [&](int slot, f32x16 (&S)[2]) {
    const char* sk = ks + slot * KTILE;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) S[kb][r] = 0.f;
#pragma unroll
      for (int s = 0; s < QV; ++s) {
        const int pos = swz<RBK>(kx, 2 * s + lg);
        V kf = as_vec<V>(ld16(sk + (kb * 32 + l32) * RBK + pos * 16));
        S[kb] = mfma32(kf, qf[s], S[kb]);
      }
    }
  };

  f32x16 O[DB];
#pragma unroll
  for (int d = 0; d < DB; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) O[d][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 Sc[2], Sn[2];  // scores of the current and of the next tile

  // Software pipeline over tiles.  Iteration t computes the scores of tile t+1 (MFMA)
  // before the softmax of tile t (VALU), then O += V_t P_t.  K and V^T have separate
  // 4-slot rings (tile i in slot (i - tb) % 4), and the tiles are taken in pairs with
  // one barrier per pair (see body below): half the barriers of a ring refilled every
  // tile, with the same two-iteration lead (1.3-2.2% faster, interleaved A/B on one
  // board).  Walkers: wk at the next K tile to load, wv at the next V^T tile to load,
  // wc at the tile being softmaxed.
  static_assert(NSLOT == 4, "pairs of tiles per barrier");
  Walk wk, wv, wc;
  int sl = 0;  // (current tile - tb) % NSLOT
  if (total > tb) {
    wk = walk_at(tb);
    wv = wk;
    wc = wk;
    // K tiles tb, tb+1, tb+2 and V tiles tb, tb+1 (slot i - tb)
    load_k(wk, 0);
    walk_next(wk);
    if (total > tb + 1) { load_k(wk, 1); walk_next(wk); }
    if (total > tb + 2) { load_k(wk, 2); walk_next(wk); }
    load_v(wv, 0);
    walk_next(wv);
    if (total > tb + 1) { load_v(wv, 1); walk_next(wv); }
    wait_vm_lds<0>();
    lds_barrier();
    scores(0, Sc);
  }
  // One iteration.  The softmax exponentials / P^T conversion / P V MFMAs of tile t and
  // the score MFMAs of tile t+1 form one branch-free block that the scheduler
  // interleaves (MFMA, LDS read, VALU), so the VALU softmax of one tile runs under the
  // MFMAs of the other.  Tiles go in pairs (t, t+1), t - tb even.  The pair's first
  // iteration (FIRST) starts with the barrier: every wave has finished tile t-1, so
  // the K slots of tiles <= t and the V^T slots of tiles <= t-1 are free, and it
  // issues K t+3, t+4 and V t+2, t+3 into them.  The pair reads K t+1, t+2 and V t, t+1,
  // issued by the previous pair.  The second iteration ends by waiting for all of this
  // wave's transfers, so after the next pair's barrier they have landed for every wave.
  // For the last tile the scores of a (stale) slot are computed and dropped, which
  // keeps the block free of branches; the slot address stays in LDS.
  auto body = [&](int t, f32x16 (&S)[2], f32x16 (&Snext)[2], auto DIRECT, auto FIRST) __attribute__((always_inline)) {
    const int sl1 = (sl + 1) & (NSLOT - 1);
    if (FIRST) {
      lds_barrier();
      const int sl3 = (sl + 3) & (NSLOT - 1);
      const int sl2 = (sl + 2) & (NSLOT - 1);
      if (t + 3 < total) { load_k(wk, sl3); walk_next(wk); }
      if (t + 4 < total) { load_k(wk, sl); walk_next(wk); }
      if (t + 2 < total) { load_v(wv, sl2); walk_next(wv); }
      if (t + 3 < total) { load_v(wv, sl3); walk_next(wv); }
    }

    if (wc.left == 1) {  // last tile of its segment: mask keys >= n (ragged tail)
      const int nk = seg_n(wc.si) - (seg_tiles(wc.si) - 1) * BKV;  // valid keys in this tile
      if (nk < BKV) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kb * 32 + 8 * (r >> 2) + 4 * lg + (r & 3);
            if (key >= nk) S[kb][r] = -INFINITY;
          }
      }
    }
    if (!DIRECT && !nomax) {  // uniform branch: the running max and its lazy rescale
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
    }
    const float ms = nomax ? 0.f : m_run * a.scale;
    const char* sv = vs + sl * VTILE;
    const char* sk = ks + sl1 * KTILE;
    // Softmax of tile t, P V of tile t and the scores of tile t+1, in NU phases.  Unit u
    // = (kb, v) covers keys [32 kb + v*2VE, +2VE) of tile t: VE exponentials per lane
    // (P^T operand elements [v*VE, v*VE+VE) of S[kb]), their row-sum contribution and
    // DB P V MFMAs with the V^T vector holding the same keys (stored order).  Phase u
    // first requests the K fragments of phase u+1 (scores of tile t+1, KPU fragments per
    // phase), then takes the exponentials of unit u+1 while its score MFMAs and the P V
    // MFMAs of unit u (whose weights the previous phase made) run: no MFMA of a phase
    // waits for that phase's VALU work (1.2% faster at the large chunk than
    // exponentiating and multiplying the same unit, interleaved A/B on one board).  The
    // scheduling barrier keeps each phase's instructions together so LDS latency hides
    // under the exponentials.  The row sum is taken from the converted operand values,
    // i.e. from exactly the weights the MFMA uses.
    constexpr int UPK = 16 / VE;       // units per 32-key block
    constexpr int NU = 2 * UPK;        // units (phases) per tile
    constexpr int KPU = 2 * QV / NU;   // score fragments per phase
    V kf[2][KPU];
    auto kread = [&](int u, int set) {
#pragma unroll
      for (int i = 0; i < KPU; ++i) {
        const int f = u * KPU + i, skb = f / QV, st = f % QV;
        const int pos = swz<RBK>(l32, 2 * st + lg);
        kf[set][i] = as_vec<V>(ld16(sk + (skb * 32 + l32) * RBK + pos * 16));
      }
    };
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) Snext[kb][r] = 0.f;
    auto expu = [&](int u) __attribute__((always_inline)) {
      const int kb = u / UPK, v = u % UPK;
      V p;
#pragma unroll
      for (int j = 0; j < VE; ++j)
        p[j] = from_f<T>(__builtin_amdgcn_exp2f(DIRECT ? S[kb][v * VE + j] : fmaf(S[kb][v * VE + j], a.scale, -ms)));
      return p;
    };
    kread(0, 0);
    V pcur = expu(0);
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      if (u + 1 < NU) kread(u + 1, (u + 1) & 1);
      const int kb = u / UPK, v = u % UPK;
      V pnext;
      if (u + 1 < NU) pnext = expu(u + 1);
      l_run = row_sum_add(pcur, l_run);
      const int pos = swz<RBV>(l32, (kb * 32 + v * 2 * VE + lg * VE) * SZ / 16);
      V vf[DB];
#pragma unroll
      for (int d = 0; d < DB; ++d) vf[d] = as_vec<V>(ld16(sv + (d * 32 + l32) * RBV + pos * 16));
#pragma unroll
      for (int i = 0; i < KPU; ++i) {
        const int f = u * KPU + i, skb = f / QV, st = f % QV;
        Snext[skb] = mfma32(kf[u & 1][i], qf[st], Snext[skb]);
      }
#pragma unroll
      for (int d = 0; d < DB; ++d) O[d] = mfma32(vf[d], pcur, O[d]);
      __builtin_amdgcn_sched_barrier(0);
      if (u + 1 < NU) pcur = pnext;
    }
    if (!FIRST) wait_vm_lds<0>();  // this wave's K t+2, t+3 and V t+1, t+2 (issued at t-1)
    walk_next(wc);
    sl = sl1;
  };
  // DIRECT: no running max and q pre-scaled (scale 1), so each weight is exp2 of the raw
  // score; the general form's fma(s, scale, -m) would be the identity and is left out
  // (a quarter of the loop's VALU instructions).
  auto run = [&](auto DIRECT) __attribute__((always_inline)) {
    int t = tb;
    for (; t + 1 < total; t += 2) {
      body(t, Sc, Sn, DIRECT, std::true_type{});
      body(t + 1, Sn, Sc, DIRECT, std::false_type{});
    }
    if (t < total) body(t, Sc, Sn, DIRECT, std::true_type{});
  };
  if (nomax && a.scale == 1.f)
    run(std::true_type{});
  else
    run(std::false_type{});

  // Normalise and store: lane holds query qrow, dh = 32 d + 8 q + 4 lg + [0, 4).
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  if (nsp == 1) {
    // The wave's 32 output rows go row-major through LDS (the rings are free once every
    // wave has passed this barrier), so that each store instruction writes whole rows,
    // 16 bytes per lane, instead of 8-byte pieces of 32 rows.  Row pitch padded by 16
    // bytes against bank conflicts.  No wave leaves before the barrier.
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS reads are done
    lds_barrier();
    constexpr int OP = DH + 16 / SZ;  // LDS row pitch (elements)
    constexpr int RB = DH * SZ;       // bytes per output row
    constexpr int LPR = RB / 16;      // lanes per row
    static_assert(RB % 16 == 0 && 64 % LPR == 0, "output rows of whole 16-byte pieces");
    T* ot = reinterpret_cast<T*>(smem) + wave * 32 * OP;
#pragma unroll
    for (int d = 0; d < DB; ++d)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = O[d][4 * q + r] * inv;
        store4<T>(ot + l32 * OP + d * 32 + 8 * q + 4 * lg, v);
      }
    const int row0 = qt * BQ + wave * 32;  // the wave's first query
    char* og = reinterpret_cast<char*>(a.o) + ((size_t)row0 * a.ldo + head * DH) * SZ;
#pragma unroll
    for (int k = 0; k < 32 * LPR / 64; ++k) {
      const int row = (64 / LPR) * k + lane / LPR, ch = lane % LPR;
      if (row0 + row < a.nq)
        st16(og + (size_t)row * a.ldo * SZ + ch * 16,
             ld16(reinterpret_cast<const char*>(ot) + row * OP * SZ + ch * 16));
    }
    return;
  }
  if (!qvalid) return;
  const int D = a.H * DH;
  float* op = a.opart + ((size_t)split * a.nq + qrow) * D + head * DH;
#pragma unroll
  for (int d = 0; d < DB; ++d)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = O[d][4 * q + r] * inv;
      store4<float>(op + d * 32 + 8 * q + 4 * lg, v);
    }
  if (lg == 0) {
    float* mp = a.ml + (((size_t)split * a.nq + qrow) * a.H + head) * 2;
    mp[0] = l_tot > 0.f ? (nomax ? 0.f : m_run * a.scale) : -INFINITY;
    mp[1] = l_tot;
  }
}

// Merge key-range partials of queries [r0, nq): o = sum_s w_s o_s / sum_s w_s,
// w_s = l_s 2^(m_s - max m).  One thread per (query, head, 4 consecutive dh).
template <class T, int DH>
__global__ __launch_bounds__(256) void attn_combine_kernel(const float* __restrict__ opart,
                                                           const float* __restrict__ ml, int nsplit,
                                                           int r0, int nq, int H, T* __restrict__ o,
                                                           int ldo) {
  const int D = H * DH;
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long long)(nq - r0) * D / 4) return;
  const int qrow = r0 + (int)(i / (D / 4));
  const int c = (int)(i - (long long)(qrow - r0) * (D / 4)) * 4;
  const int head = c / DH;
  float mmax = -INFINITY;
  for (int sp = 0; sp < nsplit; ++sp) mmax = fmaxf(mmax, ml[(((size_t)sp * nq + qrow) * H + head) * 2]);
  float acc[4] = {0.f, 0.f, 0.f, 0.f}, wsum = 0.f;
  for (int sp = 0; sp < nsplit; ++sp) {
    const float* mp = ml + (((size_t)sp * nq + qrow) * H + head) * 2;
    const float w = mp[1] > 0.f ? mp[1] * __builtin_amdgcn_exp2f(mp[0] - mmax) : 0.f;
    float v[4];
    load4<float>(opart + ((size_t)sp * nq + qrow) * D + c, v);
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = fmaf(w, v[r], acc[r]);
    wsum += w;
  }
  const float inv = 1.0f / wsum;
#pragma unroll
  for (int r = 0; r < 4; ++r) acc[r] *= inv;
  store4<T>(o + (size_t)qrow * ldo + c, acc);
}

}  // namespace

hipError_t attention(int dtype, int dh, int H, const void* q, int ldq, void* o, int ldo, int nq,
                     int ldk, const AttnSeg* segs, int nseg, const AttnSplit& sp, bool q_prescaled,
                     hipStream_t s, int kind, const AttnNorm* norm, const hipEvent_t* ev) {
  if (nq <= 0) return hipSuccess;
  if (nseg < 1 || nseg > ATTN_MAX_SEGS) return hipErrorInvalidValue;
  if (sp.nsplit < 1 || (sp.nsplit > 1 && (!sp.opart || !sp.ml))) return hipErrorInvalidValue;
  const int nqt = (nq + BQ - 1) / BQ;
  const int qt0 = sp.nsplit > 1 ? std::min(std::max(sp.qt0, 0), nqt) : 0;
  AttnArgs a;
  a.q = q;
  a.o = o;
  a.ldq = ldq;
  a.ldo = ldo;
  a.nq = nq;
  a.ldk = ldk;
  a.nseg = nseg;
  a.H = H;
  a.scale = q_prescaled ? 1.0f : attention_q_scale(dh);
  a.thr = RESCALE_LOG2 / a.scale;
  a.nsplit = sp.nsplit;
  a.qt0 = qt0;
  a.opart = sp.opart;
  a.ml = sp.ml;
  // q = q_fold (gq . q^) and k = gk . k^ with |q^|^2, |k^|^2 <= dh (RMS-normed rows), so
  // |q . k| <= q_fold dh max|gq| max|gk|; the factor covers the bf16 rounding of q and k.
  a.gq = (norm && q_prescaled && norm->gq && norm->gk) ? norm->gq : nullptr;
  a.gk = a.gq ? norm->gk : nullptr;
  a.bcoef = a.gq ? (float)(norm->q_fold * dh * 1.02) : 0.f;
  for (int i = 0; i < ATTN_MAX_SEGS; ++i) a.seg[i] = i < nseg ? segs[i] : AttnSeg{nullptr, nullptr, 0, 64};
  const dim3 grid(qt0 * H + (nqt - qt0) * H * sp.nsplit), block(64 * AW);
  const bool cross = kind == ATTN_CROSS;
  const void* fn;
  if (dtype == BF16 && dh == 128)
    fn = cross ? (const void*)attn_kernel<bf16, 128, 1> : (const void*)attn_kernel<bf16, 128, 0>;
  else if (dtype == BF16 && dh == 64)
    fn = cross ? (const void*)attn_kernel<bf16, 64, 1> : (const void*)attn_kernel<bf16, 64, 0>;
  else if (dtype == F32 && dh == 64)
    fn = cross ? (const void*)attn_kernel<float, 64, 1> : (const void*)attn_kernel<float, 64, 0>;
  else
    return hipErrorInvalidValue;
  // With events, the dispatch itself stamps the kernel's start and end into them: no
  // separate marker packets (and their waits) between this launch and its neighbours.
  // When q-tiles are split the merge (attention_combine) stamps the end instead.
  void* args[1] = {&a};
  if (ev) return hipExtLaunchKernel(fn, grid, block, args, 0, s, ev[0], attention_splits(nq, sp) ? nullptr : ev[1], 0);
  return hipLaunchKernel(fn, grid, block, args, 0, s);
}

bool attention_splits(int nq, const AttnSplit& sp) {
  return nq > 0 && sp.nsplit > 1 && std::min(std::max(sp.qt0, 0) * BQ, nq) < nq;
}

hipError_t attention_combine(int dtype, int dh, int H, int nq, const AttnSplit& sp, void* o, int ldo,
                             hipStream_t s, hipEvent_t stop) {
  if (!attention_splits(nq, sp)) return hipSuccess;
  const int r0 = std::min(std::max(sp.qt0, 0) * BQ, nq);  // rows before r0 were not split
  const long long n4 = (long long)(nq - r0) * H * dh / 4;
  const dim3 grid((unsigned)((n4 + 255) / 256)), block(256);
  const hipEvent_t ev[2] = {nullptr, stop};
  if (dtype == BF16 && dh == 128)
    return launch_k(attn_combine_kernel<bf16, 128>, grid, block, s, ev, (const float*)sp.opart, (const float*)sp.ml,
                    sp.nsplit, r0, nq, H, (bf16*)o, ldo);
  if (dtype == BF16 && dh == 64)
    return launch_k(attn_combine_kernel<bf16, 64>, grid, block, s, ev, (const float*)sp.opart, (const float*)sp.ml,
                    sp.nsplit, r0, nq, H, (bf16*)o, ldo);
  if (dtype == F32 && dh == 64)
    return launch_k(attn_combine_kernel<float, 64>, grid, block, s, ev, (const float*)sp.opart, (const float*)sp.ml,
                    sp.nsplit, r0, nq, H, (float*)o, ldo);
  return hipErrorInvalidValue;
}

int attention_key_tiles(const AttnSeg* segs, int nseg) {
  int t = 0;
  for (int i = 0; i < nseg; ++i) t += (segs[i].n + BKV - 1) / BKV;
  return t;
}

int device_cus() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      cus = n;
    else
      cus = 256;
  }
  return cus;
}

}  // namespace dit
