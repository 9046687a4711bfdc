// Host runtime and C ABI of the streaming KV-ring attention library.
//
// The ring state of a rollout is two integers (frames committed since the
// last reset, temporal origin t0); slots, positions and evictions follow in
// closed form, so no call ever reads device memory back.  Cache reading:
// S sink frames (the first S frames of a sequence, never evicted) plus a
// FIFO window of W frames in S + W fixed slots -- FlashDreams blog post,
// "Bounded Memory for Infinite Rollouts"; Cosmos3-H-Dreams model card,
// "Software Integration" (static-shape KV cache).
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <set>
#include <string>
#include <vector>

#include "wm.h"
#include "wm_internal.hpp"

namespace {

thread_local std::string g_err;

wm_status fail(wm_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

wm_status ok() {
  g_err.clear();
  return WM_OK;
}

std::mutex g_mu;
std::set<const void*> g_live;    // live ring handles
uint64_t g_serial = 0;           // rings created so far (a ring's serial number)
std::set<const void*> g_graphs;  // live rollout-graph handles

bool sync_check_enabled() {
  static const bool on = [] {
    const char* e = getenv("WM_SYNC_CHECK");
    return e && atoi(e) != 0;
  }();
  return on;
}

// WM_FAULT_INJECT=launch|rope|attn|append (read on every call): direct
// launches of that kind (every kind for "launch") fail as if the runtime had
// refused them; for tests of the error path.
bool fault_injected(const char* kind) {
  const char* e = getenv("WM_FAULT_INJECT");
  return e && (strcmp(e, "launch") == 0 || strcmp(e, kind) == 0);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// libm through volatile pointers: keeps the compiler from fusing cos/sin
// into sincos or vectorising them, so every entry is the scalar libm result.
double (*volatile g_cos)(double) = ::cos;
double (*volatile g_sin)(double) = ::sin;
double (*volatile g_pow)(double, double) = ::pow;

struct Bands {
  int dt, dh, dw;
};

bool bands_of(const wm_kvring_desc& d, Bands* b) {
  if (d.rope_dims[0] || d.rope_dims[1] || d.rope_dims[2]) {
    b->dt = d.rope_dims[0];
    b->dh = d.rope_dims[1];
    b->dw = d.rope_dims[2];
  } else {
    b->dh = b->dw = 2 * (d.head_dim / 6);
    b->dt = d.head_dim - b->dh - b->dw;
  }
  if (b->dt < 0 || b->dh < 0 || b->dw < 0) return false;
  if ((b->dt | b->dh | b->dw) & 1) return false;
  if (b->dt + b->dh + b->dw != d.head_dim) return false;
  if (b->dt / 2 > wm::kMaxTPairs) return false;
  return true;
}

constexpr int kMaxLayers = 256;
constexpr int kMaxViews = 16;

// Views per frame of a descriptor (0 means one) and tokens per stored frame.
int views_of(const wm_kvring_desc& d) { return d.n_views > 0 ? d.n_views : 1; }
int64_t ft_of(const wm_kvring_desc& d) { return (int64_t)views_of(d) * d.frame_h * d.frame_w; }

// Layers of a descriptor (0 means one).
int layers_of(const wm_kvring_desc& d) { return d.n_layers > 0 ? d.n_layers : 1; }

struct Layout {
  size_t k_off, v_off;  // layer 0; layer l adds l * layer_bytes
  size_t layer_bytes;
  size_t tab_off;
  size_t hw;        // byte offset of the (cos, sin) table of the h then w band
  size_t tab_bytes;
  size_t cnt_off, cnt_bytes;  // split-attention arrival counters (int32, zeroed at creation)
  size_t total;
};

wm_status check_desc(const wm_kvring_desc* d, Bands* bands) {
  if (!d) return fail(WM_E_ARG, "descriptor is NULL");
  if (d->batch < 1 || d->batch > WM_MAX_BATCH)
    return fail(WM_E_SHAPE, "batch %d not in [1, %d]", d->batch, WM_MAX_BATCH);
  if (d->n_q_heads < 1 || d->n_kv_heads < 1 || d->n_q_heads % d->n_kv_heads)
    return fail(WM_E_SHAPE, "heads: Hq=%d must be a positive multiple of Hkv=%d", d->n_q_heads,
                d->n_kv_heads);
  if (d->n_q_heads > 256) return fail(WM_E_SHAPE, "Hq=%d above 256", d->n_q_heads);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(WM_E_SHAPE, "head_dim %d: only 64 and 128 are built", d->head_dim);
  if (d->n_views < 0 || d->n_views > kMaxViews)
    return fail(WM_E_SHAPE, "n_views %d not in [0, %d]", d->n_views, kMaxViews);
  if (d->frame_h < 1 || d->frame_w < 1 || ft_of(*d) > (1 << 20))
    return fail(WM_E_SHAPE, "frame of %d views of %dx%d tokens out of range", views_of(*d), d->frame_h,
                d->frame_w);
  if (d->n_sink < 0 || d->window < 0 || d->n_sink + d->window > WM_MAX_RING)
    return fail(WM_E_SHAPE, "sink %d + window %d must be in [0, %d]", d->n_sink, d->window,
                WM_MAX_RING);
  if (d->max_chunk < 1 || d->max_chunk > WM_MAX_CHUNK)
    return fail(WM_E_SHAPE, "max_chunk %d not in [1, %d]", d->max_chunk, WM_MAX_CHUNK);
  if (d->evict_policy != WM_EVICT_SLIDE && d->evict_policy != WM_EVICT_RESET)
    return fail(WM_E_SHAPE, "evict_policy %d is neither WM_EVICT_SLIDE nor WM_EVICT_RESET",
                d->evict_policy);
  if (d->n_layers < 0 || d->n_layers > kMaxLayers)
    return fail(WM_E_SHAPE, "n_layers %d not in [0, %d]", d->n_layers, kMaxLayers);
  if (!(d->rope_theta > 1.0) || !isfinite(d->rope_theta))
    return fail(WM_E_SHAPE, "rope_theta must be finite and > 1");
  if (!bands_of(*d, bands))
    return fail(WM_E_SHAPE, "rope_dims {%d,%d,%d}: bands must be even, sum to d, d_t <= %d",
                d->rope_dims[0], d->rope_dims[1], d->rope_dims[2], 2 * wm::kMaxTPairs);
  const int64_t nq = (int64_t)d->max_chunk * ft_of(*d);
  if ((int64_t)(d->n_sink + d->window + d->max_chunk) * ft_of(*d) >= ((int64_t)1 << 24))
    return fail(WM_E_SHAPE, "visible keys (S+W+C)*Ft must stay below 2^24");
  // The kernels form offsets within one rollout's chunk tensor and within
  // one rollout's K (or V) half of a layer in 32 bits.
  if (nq * d->n_q_heads * d->head_dim >= (int64_t)1 << 31)
    return fail(WM_E_SHAPE, "chunk tensor of 2^31 elements or more per rollout");
  if ((int64_t)(d->n_sink + d->window) * d->n_kv_heads * ft_of(*d) * d->head_dim >= (int64_t)1 << 31)
    return fail(WM_E_SHAPE, "ring of 2^31 elements or more per rollout in the K (or V) half");
  return WM_OK;
}

// Attention wave tasks: 32 queries of one q head each, eight per workgroup
// (256 queries of one kv head's group).
constexpr int kWaveQ = 32;
constexpr int kWgWaves = 8;

int task_blocks_of(int64_t nq) { return (int)((nq + kWaveQ - 1) / kWaveQ); }

int wg_per_bg_of(const wm_kvring_desc& d, int64_t nq) {
  const int group = d.n_q_heads / d.n_kv_heads;
  return (group * task_blocks_of(nq) + kWgWaves - 1) / kWgWaves;
}

Layout layout_of(const wm_kvring_desc& d, const Bands& b) {
  Layout L;
  const size_t ft = (size_t)ft_of(d);
  const size_t half =
      (size_t)d.batch * (d.n_sink + d.window) * d.n_kv_heads * ft * d.head_dim * sizeof(uint16_t);
  L.k_off = 0;
  L.v_off = align_up(half, 256);
  L.layer_bytes = align_up(L.v_off + half, 256);
  L.tab_off = L.layer_bytes * layers_of(d);
  const size_t entries = (size_t)d.frame_h * (b.dh / 2) + (size_t)d.frame_w * (b.dw / 2);
  L.hw = L.tab_off;
  // At least one entry: the kernels read entry 0 (unused) for t-band pairs.
  L.tab_bytes = (entries ? entries : 1) * 2 * sizeof(double);
  // One counter per row block of the largest attention launch group.
  const size_t groups = (size_t)std::min(d.batch, wm::kAttnMaxB) * d.n_kv_heads *
                        wg_per_bg_of(d, (int64_t)d.max_chunk * ft_of(d));
  L.cnt_off = align_up(L.tab_off + L.tab_bytes, 256);
  L.cnt_bytes = align_up(groups * sizeof(int32_t), 256);
  L.total = L.cnt_off + L.cnt_bytes;
  return L;
}

// Inverse frequency of pair j in a band of width da: theta^(-(2j)/da), fp64.
double inv_freq(double theta, int j, int da) { return g_pow(theta, -(2.0 * j) / (double)da); }

}  // namespace

struct wm_kvring {
  wm_kvring_desc desc;
  Bands bands;
  Layout L;
  int ft, R, n_layers;
  bool meta_only;
  uint8_t* pool;
  std::vector<int64_t> n_committed, t0;
  std::vector<double> inv_t;
  // t-band (cos, sin) rows by absolute t, direct-mapped: a frame's row is
  // needed by every RoPE call of its denoise steps and by its append.
  struct TRow {
    int64_t t = INT64_MIN;
    float2 cs[wm::kMaxTPairs];
  };
  mutable TRow t_cache[64];
  // Overlapped finalize: ev_attn marks the last attention of a step on the
  // main stream, ev_fin the append on the finalize stream; once an append has
  // gone to a finalize stream, every later call that touches the pool waits
  // for ev_fin first (RoPE, which does not, overlaps it).
  hipEvent_t ev_attn = nullptr, ev_fin = nullptr;
  bool fin_recorded = false;
  uint64_t serial = 0;  // distinguishes a ring from a later one at the same address
};

namespace {
// One planned kernel launch: its shape and its parameter block.
struct PLaunch {
  wm::LaunchSpec spec;
  bool attn;             // parameters: ap (attention) or rp (RoPE / append)
  wm::RopeParams rp;
  wm::AttnParams ap;
  void* argv[1];
  void* args() { return attn ? static_cast<void*>(&ap) : static_cast<void*>(&rp); }
};
}  // namespace

struct wm_rollout_graph {
  wm_kvring* ring;
  uint64_t ring_serial;
  int D, n_frames;
  bool has_active;
  std::vector<uint8_t> active;
  std::vector<const wm_bf16*> q, k, v;
  std::vector<wm_bf16*> out;
  wm_bf16 *q_rot, *k_rot;
  void* ws;
  size_t ws_bytes;
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  hipEvent_t ev_done = nullptr;  // after the last launch; waited on before the exec is dropped
  bool launched = false;
  std::vector<hipGraphNode_t> nodes;
  std::vector<wm::LaunchSpec> shape;
  std::vector<PLaunch> held;  // the parameters each node of the instance holds
};

namespace {

wm_status check_ring(const wm_kvring* r) {
  if (!r) return fail(WM_E_ARG, "ring handle is NULL");
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_live.count(r)) return fail(WM_E_STATE, "ring handle is not live (destroyed?)");
  return WM_OK;
}

wm_status check_dev(const void* p, const char* name) {
  if (!p) return fail(WM_E_ARG, "%s is NULL", name);
  if (!aligned16(p)) return fail(WM_E_ARG, "%s is not 16-byte aligned", name);
  return WM_OK;
}

bool is_active(const uint8_t* active, int b) { return !active || active[b] != 0; }

int64_t next_t(const wm_kvring* r, int b) { return r->t0[b] + r->n_committed[b]; }

void t_row(const wm_kvring* r, int64_t t, float2* cs) {
  const int np = r->bands.dt / 2;
  wm_kvring::TRow& c = r->t_cache[(uint64_t)t & 63];
  if (c.t != t) {
    for (int j = 0; j < np; ++j) {
      const double ang = (double)t * r->inv_t[j];
      c.cs[j].x = (float)g_cos(ang);
      c.cs[j].y = (float)g_sin(ang);
    }
    c.t = t;
  }
  memcpy(cs, c.cs, sizeof(float2) * np);
}

// Multiplier and shift for wm::FastDiv (d >= 1, dividends below 2^31):
// l = ceil(log2 d), mul = floor(2^32 (2^l - d) / d) + 1.
wm::FastDiv fast_div_of(uint32_t d) {
  uint32_t l = 0;
  while ((1ull << l) < d) ++l;
  const uint64_t mul = ((((uint64_t)1 << l) - d) << 32) / d + 1;
  return wm::FastDiv{(uint32_t)mul, l};
}

void fill_tables_ptrs(const wm_kvring* r, wm::RopeParams* p, int n_heads) {
  p->hw = reinterpret_cast<const double2*>(r->pool + r->L.hw);
  p->w_base = r->desc.frame_h * (r->bands.dh / 2);
  p->n_heads = n_heads;
  p->lg_cpr = r->desc.head_dim == 128 ? 4 : 3;
  p->hg_first = (n_heads + wm::kRopeHeads - 1) / wm::kRopeHeads;
  p->div_fw = fast_div_of((uint32_t)r->desc.frame_w);
  p->div_fh = fast_div_of((uint32_t)r->desc.frame_h);
  p->fh = r->desc.frame_h;
  p->ft = r->ft;
  p->fw = r->desc.frame_w;
  p->d = r->desc.head_dim;
  p->dt2 = r->bands.dt / 2;
  p->dh2 = r->bands.dh / 2;
  p->dw2 = r->bands.dw / 2;
  p->ring_slots = r->R;
}

wm_status hip_fail(hipError_t e, const char* what) {
  return fail(WM_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

wm_status finish(hipStream_t s) {
  if (sync_check_enabled()) {
    hipError_t e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "stream synchronize");
    e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "asynchronous error");
  }
  return ok();
}

// --- where the workers' launches go ---------------------------------------
// A planned launch: its spec and the parameter struct it takes.

// Kernel-node parameters of a planned launch (points into L: L must stay put
// until the node is added or updated).
hipKernelNodeParams node_params(PLaunch& L) {
  hipKernelNodeParams kp;
  memset(&kp, 0, sizeof kp);
  L.argv[0] = L.args();
  kp.func = const_cast<void*>(L.spec.func);
  kp.gridDim = L.spec.grid;
  kp.blockDim = L.spec.block;
  kp.sharedMemBytes = 0;
  kp.kernelParams = L.argv;
  kp.extra = nullptr;
  return kp;
}

// Launches on a stream, or records the launches (for a HIP graph) instead.
struct Sink {
  hipStream_t s = nullptr;
  std::vector<PLaunch>* rec = nullptr;

  hipError_t put(const wm::LaunchSpec& sp, const wm::RopeParams* rp, const wm::AttnParams* ap,
                 const char* kind) {
    if (rec) {
      rec->emplace_back();
      PLaunch& L = rec->back();
      L.spec = sp;
      L.attn = ap != nullptr;
      if (rp) L.rp = *rp;
      if (ap) L.ap = *ap;
      return hipSuccess;
    }
    if (fault_injected(kind)) return hipErrorLaunchFailure;
    void* arg = ap ? (void*)ap : (void*)rp;
    void* args[] = {arg};
    return hipLaunchKernel(sp.func, sp.grid, sp.block, args, 0, s);
  }
  hipError_t rope(const wm::RopeParams& p) { return put(wm::rope3d_spec(p), &p, nullptr, "rope"); }
  hipError_t append(const wm::RopeParams& p) {
    return put(wm::kv_append_spec(p), &p, nullptr, "append");
  }
  hipError_t attn(wm::AttnParams p, int head_dim) {
    wm::LaunchSpec sp[2];
    const int n = wm::chunk_attn_specs(p, head_dim, sp);
    if (n == 0) return hipErrorInvalidValue;
    for (int i = 0; i < n; ++i) {
      hipError_t e = put(sp[i], nullptr, &p, "attn");
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
};

// --- the unchecked workers (arguments validated by the callers) -----------

// RoPE of x into y and, when x2 is given, of x2 into y2 in the same launch
// (Q and K of a denoise step: same frames, so the same rows and positions).
wm_status do_rope(const wm_kvring* r, const wm_bf16* x, wm_bf16* y, int n_heads, int n_frames,
                  const int64_t* t_first, const uint8_t* active, Sink& k,
                  const wm_bf16* x2 = nullptr, wm_bf16* y2 = nullptr, int n_heads2 = 0) {
  wm::RopeParams p;
  memset(&p, 0, sizeof p);
  fill_tables_ptrs(r, &p, n_heads);
  p.x = x;
  p.y = y;
  p.x_b_stride = (int64_t)n_frames * r->ft * n_heads * r->desc.head_dim;
  p.x2 = x2;
  p.y2 = y2;
  p.n_heads2 = n_heads2;
  p.x2_b_stride = (int64_t)n_frames * r->ft * n_heads2 * r->desc.head_dim;
  for (int b = 0; b < r->desc.batch; ++b) {
    if (!is_active(active, b)) continue;
    const int64_t t0 = t_first ? t_first[b] : next_t(r, b);
    for (int j = 0; j < n_frames; ++j) {
      wm::RopeRow& row = p.rows[p.n_rows];
      row.b = b;
      row.j = j;
      row.slot = -1;
      t_row(r, t0 + j, p.tcs[p.n_rows]);
      if (++p.n_rows == wm::kRopeRows) {
        hipError_t e = k.rope(p);
        if (e != hipSuccess) return hip_fail(e, "rope3d launch");
        p.n_rows = 0;
      }
    }
  }
  if (p.n_rows) {
    hipError_t e = k.rope(p);
    if (e != hipSuccess) return hip_fail(e, "rope3d launch");
  }
  return WM_OK;
}

// Closed-form plan of one append for rollout b (see the pool layout in wm.h).
struct Planned {
  int32_t slot;
  bool stored;
};

void plan_append(const wm_kvring* r, int b, int n_frames, wm_append_report* rep,
                 Planned* plan) {
  const int64_t S = r->desc.n_sink, W = r->desc.window;
  const int64_t m0 = r->n_committed[b], m_end = m0 + n_frames;
  rep->n_written = n_frames;
  rep->n_evicted = 0;
  for (int j = 0; j < n_frames; ++j) {
    const int64_t f = m0 + j;
    int32_t slot;
    if (f < S)
      slot = (int32_t)f;
    else if (W > 0)
      slot = (int32_t)(S + (f - S) % W);
    else
      slot = -1;
    rep->frame[j] = f;
    rep->slot[j] = slot;
    rep->t[j] = r->t0[b] + f;
    if (W > 0 && f >= S + W) rep->evicted[rep->n_evicted++] = f - W;
    plan[j].slot = slot;
    plan[j].stored = slot >= 0 && (f < S || f >= m_end - W);
  }
}

// Plans and launches (or records) one append; the bookkeeping advances only
// when `commit` is set, after every launch was accepted.
wm_status do_append(wm_kvring* r, const wm_bf16* k_raw, const wm_bf16* v, int n_frames,
                    const uint8_t* active, wm_append_report* rep, Sink& k, bool commit = true) {
  const int B = r->desc.batch;
  std::vector<wm_append_report> reps(B);
  std::vector<Planned> plan((size_t)B * n_frames);
  for (int b = 0; b < B; ++b) {
    memset(&reps[b], 0, sizeof(wm_append_report));
    if (is_active(active, b)) plan_append(r, b, n_frames, &reps[b], &plan[(size_t)b * n_frames]);
  }
  if (!r->meta_only) {
    wm::RopeParams p;
    memset(&p, 0, sizeof p);
    fill_tables_ptrs(r, &p, r->desc.n_kv_heads);
    p.x = k_raw;
    p.vsrc = v;
    p.y = reinterpret_cast<uint16_t*>(r->pool + r->L.k_off);
    p.vdst = reinterpret_cast<uint16_t*>(r->pool + r->L.v_off);
    p.x_b_stride = (int64_t)n_frames * r->ft * r->desc.n_kv_heads * r->desc.head_dim;
    p.n_layers = r->n_layers;
    p.x_layer_stride = p.x_b_stride * B;
    p.pool_layer_stride = (int64_t)(r->L.layer_bytes / sizeof(uint16_t));
    for (int b = 0; b < B; ++b) {
      if (!is_active(active, b)) continue;
      for (int j = 0; j < n_frames; ++j) {
        const Planned& pl = plan[(size_t)b * n_frames + j];
        if (!pl.stored) continue;
        wm::RopeRow& row = p.rows[p.n_rows];
        row.b = b;
        row.j = j;
        row.slot = pl.slot;
        t_row(r, reps[b].t[j], p.tcs[p.n_rows]);
        if (++p.n_rows == wm::kRopeRows) {
          hipError_t e = k.append(p);
          if (e != hipSuccess) return hip_fail(e, "kv_append launch");
          p.n_rows = 0;
        }
      }
    }
    if (p.n_rows) {
      hipError_t e = k.append(p);
      if (e != hipSuccess) return hip_fail(e, "kv_append launch");
    }
  } else if (fault_injected("append")) {  // a metadata-only ring fails where the launch would
    return hip_fail(hipErrorLaunchFailure, "kv_append launch");
  }
  // Commit only once every launch was accepted.
  if (commit)
    for (int b = 0; b < B; ++b)
      if (is_active(active, b)) r->n_committed[b] += n_frames;
  if (rep) memcpy(rep, reps.data(), sizeof(wm_append_report) * B);
  return WM_OK;
}

// Key-range split of an attention launch.  Launch time of s splits, in
// times of one workgroup's 64-key tile, a model fitted to launches with every
// forced count (1-6, 8) on four workloads (152 to 880 workgroups, 275 to 1100
// key tiles; it picks the fastest count on each):
//  - the n_wg * s workgroups run in rounds of one per CU; a round lasts the
//    tiles each walks, ceil(ntiles / s), plus a fixed kWgFixedTiles per
//    workgroup (Q load, pipeline fill and drain, partial write);
//  - a partly filled round is shorter, as the clock rises when fewer CUs
//    draw power (the card runs this kernel at its power limit): its time
//    scales by max(kRoundFloor, f^kRoundExp) at busy fraction f;
//  - the partials (written, then read by the merge) add kMergeTiles per 256
//    workgroups of the launch.
// Each split keeps at least two 64-key tiles.
constexpr int kCUs = 256;
constexpr int kMaxSplit = wm::kAttnMaxSplit;
constexpr double kWgFixedTiles = 4.0;
constexpr double kMergeTiles = 4.0;
constexpr double kRoundExp = 0.6;
constexpr double kRoundFloor = 0.7;

double split_cost(int n_wg, int ntiles, int s) {
  const int64_t n = (int64_t)n_wg * s;
  const int64_t full = n / kCUs, rem = n % kCUs;
  const double rounds =
      (double)full + (rem ? std::max(kRoundFloor, std::pow((double)rem / kCUs, kRoundExp)) : 0.0);
  double cost = rounds * ((double)((ntiles + s - 1) / s) + kWgFixedTiles);
  if (s > 1) cost += kMergeTiles * (double)n / kCUs;
  return cost;
}

// WM_ATTN_SPLIT=n (1..8) overrides the choice (tuning and tests); read on
// every call.
int forced_split() {
  const char* e = getenv("WM_ATTN_SPLIT");
  if (!e) return 0;
  const int v = atoi(e);
  return v < 1 ? 0 : (v > kMaxSplit ? kMaxSplit : v);
}

int choose_split(int n_wg, int ntiles) {
  const int forced = forced_split();
  if (forced) return std::max(1, std::min(forced, ntiles));
  int best = 1;
  double best_cost = split_cost(n_wg, ntiles, 1);
  for (int s = 2; s <= kMaxSplit && ntiles >= 2 * s; ++s) {
    const double cost = split_cost(n_wg, ntiles, s);
    if (cost < best_cost - 1e-9) {
      best = s;
      best_cost = cost;
    }
  }
  return best;
}

// Rows of split partials: every 32-query task block whole (the kernel keeps
// them in its lanes' register order, padding rows included).
size_t split_rows(int nsplit, int nb, int nq, int hq) {
  return (size_t)nsplit * nb * hq * task_blocks_of(nq) * kWaveQ;
}

size_t split_ws_bytes(int nsplit, int nb, int nq, int hq, int hd) {
  const size_t rows = split_rows(nsplit, nb, nq, hq);
  return align_up(rows * hd * sizeof(float), 256) + rows * 2 * sizeof(float);
}

int wg_per_bg_of(const wm_kvring* r, int n_frames) { return wg_per_bg_of(r->desc, (int64_t)n_frames * r->ft); }

// The attention launch groups of a call: up to kAttnMaxB active rollouts each,
// in batch order, with the split each would take given unlimited workspace.
struct AttnGroup {
  int nb = 0;
  int max_ring = 0;
  int nsplit = 1;
  int32_t b_index[wm::kAttnMaxB];
  int32_t n_ring[wm::kAttnMaxB];
};

std::vector<AttnGroup> attn_groups(const wm_kvring* r, int n_frames, const uint8_t* active) {
  const wm_kvring_desc& d = r->desc;
  std::vector<AttnGroup> groups;
  AttnGroup g;
  auto close = [&]() {
    const int ntiles = ((g.max_ring + n_frames) * r->ft + 63) / 64;
    g.nsplit = choose_split(g.nb * d.n_kv_heads * wg_per_bg_of(r, n_frames), ntiles);
    groups.push_back(g);
    g = AttnGroup();
  };
  for (int b = 0; b < d.batch; ++b) {
    if (!is_active(active, b)) continue;
    g.b_index[g.nb] = b;
    g.n_ring[g.nb] = (int32_t)std::min<int64_t>(r->n_committed[b], r->R);
    g.max_ring = std::max(g.max_ring, (int)g.n_ring[g.nb]);
    if (++g.nb == wm::kAttnMaxB) close();
  }
  if (g.nb) close();
  return groups;
}

// Workspace the largest group of a call needs for its split (0: no split).
size_t attn_ws_needed(const wm_kvring* r, int n_frames, const std::vector<AttnGroup>& groups) {
  size_t need = 0;
  for (const AttnGroup& g : groups)
    if (g.nsplit > 1)
      need = std::max(need, split_ws_bytes(g.nsplit, g.nb, n_frames * r->ft, r->desc.n_q_heads,
                                           r->desc.head_dim));
  return need;
}

wm_status do_attn(const wm_kvring* r, int layer, const wm_bf16* q, const wm_bf16* kc,
                  const wm_bf16* vc, int n_frames, const uint8_t* active, float scale,
                  wm_bf16* out, void* ws, size_t ws_bytes, Sink& k) {
  const wm_kvring_desc& d = r->desc;
  wm::AttnParams p;
  memset(&p, 0, sizeof p);
  p.q = q;
  p.kc = kc;
  p.vc = vc;
  p.pk = reinterpret_cast<const uint16_t*>(r->pool + (size_t)layer * r->L.layer_bytes + r->L.k_off);
  p.pv = reinterpret_cast<const uint16_t*>(r->pool + (size_t)layer * r->L.layer_bytes + r->L.v_off);
  p.out = out;
  p.hq = d.n_q_heads;
  p.hkv = d.n_kv_heads;
  p.group = d.n_q_heads / d.n_kv_heads;
  p.ft = r->ft;
  p.nq = n_frames * r->ft;
  p.ring_slots = r->R;
  p.nqb = task_blocks_of(p.nq);
  p.counters = reinterpret_cast<int32_t*>(r->pool + r->L.cnt_off);
  p.wg_per_bg = wg_per_bg_of(r, n_frames);
  const float sc = scale > 0.f ? scale : (float)(1.0 / sqrt((double)d.head_dim));
  p.scale_log2e = (float)((double)sc * 1.4426950408889634);
  // One launch per group of rollouts, split when it pays and the workspace
  // fits (a split that does not fit is reduced until it does).
  for (const AttnGroup& g : attn_groups(r, n_frames, active)) {
    p.nb = g.nb;
    memcpy(p.b_index, g.b_index, sizeof(int32_t) * g.nb);
    memcpy(p.n_ring, g.n_ring, sizeof(int32_t) * g.nb);
    int ns = g.nsplit;
    while (ns > 1 && (!ws || split_ws_bytes(ns, p.nb, p.nq, p.hq, d.head_dim) > ws_bytes)) --ns;
    p.nsplit = ns;
    p.part_o = nullptr;
    p.part_ml = nullptr;
    if (ns > 1) {
      const size_t rows = split_rows(ns, p.nb, p.nq, p.hq);
      p.part_o = static_cast<float*>(ws);
      p.part_ml = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) +
                                           align_up(rows * d.head_dim * sizeof(float), 256));
    }
    hipError_t e = k.attn(p, d.head_dim);
    if (e != hipSuccess) return hip_fail(e, "chunk_attn launch");
  }
  return WM_OK;
}

wm_status check_frames(const wm_kvring* r, int n_frames) {
  if (n_frames < 1 || n_frames > r->desc.max_chunk)
    return fail(WM_E_SHAPE, "n_frames %d not in [1, max_chunk=%d]", n_frames, r->desc.max_chunk);
  return WM_OK;
}

// WM_EVICT_RESET: every active rollout must hold n_frames more frames
// without evicting (its sinks and window not yet full).
wm_status check_room(const wm_kvring* r, int n_frames, const uint8_t* active) {
  if (r->desc.evict_policy != WM_EVICT_RESET) return WM_OK;
  for (int b = 0; b < r->desc.batch; ++b)
    if (is_active(active, b) && r->n_committed[b] + n_frames > r->R)
      return fail(WM_E_CAPACITY,
                  "rollout %d holds %lld of %d frames: a %d-frame append would evict (reset policy: "
                  "start a new window with wm_kvring_reset)",
                  b, (long long)r->n_committed[b], r->R, n_frames);
  return WM_OK;
}

wm_status make_events(wm_kvring* r) {
  hipError_t e = hipSuccess;
  if (!r->ev_attn) e = hipEventCreateWithFlags(&r->ev_attn, hipEventDisableTiming);
  if (e == hipSuccess && !r->ev_fin) e = hipEventCreateWithFlags(&r->ev_fin, hipEventDisableTiming);
  return e == hipSuccess ? WM_OK : hip_fail(e, "event create");
}

// Order s after the last append that went to a finalize stream.
wm_status wait_finalize(const wm_kvring* r, hipStream_t s) {
  if (!r->fin_recorded) return WM_OK;
  hipError_t e = hipStreamWaitEvent(s, r->ev_fin, 0);
  return e == hipSuccess ? WM_OK : hip_fail(e, "finalize wait");
}

wm_status check_device_ring(const wm_kvring* r) {
  if (r->meta_only) return fail(WM_E_STATE, "metadata-only ring has no device pool");
  return WM_OK;
}

// Arguments of a rollout step (wm_rollout_step, wm_rollout_graph_create).
wm_status check_step(const wm_kvring* ring, int n_denoise, const wm_bf16* const* q,
                     const wm_bf16* const* k, const wm_bf16* const* v, int n_frames,
                     const wm_bf16* q_rot, const wm_bf16* k_rot, wm_bf16* const* out,
                     const void* workspace) {
  wm_status st;
  if ((st = check_ring(ring)) != WM_OK) return st;
  if ((st = check_device_ring(ring)) != WM_OK) return st;
  if ((st = check_frames(ring, n_frames)) != WM_OK) return st;
  if (ring->n_layers != 1)
    return fail(WM_E_UNSUPPORTED, "a rollout step drives a one-layer ring (this one has %d layers)",
                ring->n_layers);
  if (n_denoise < 1 || n_denoise > 64) return fail(WM_E_ARG, "n_denoise %d not in [1, 64]", n_denoise);
  if (!q || !k || !v || !out) return fail(WM_E_ARG, "q/k/v/out pointer arrays must not be NULL");
  for (int i = 0; i < n_denoise; ++i) {
    if ((st = check_dev(q[i], "q[s]")) != WM_OK) return st;
    if ((st = check_dev(k[i], "k[s]")) != WM_OK) return st;
    if ((st = check_dev(v[i], "v[s]")) != WM_OK) return st;
    if ((st = check_dev(out[i], "out[s]")) != WM_OK) return st;
  }
  if ((st = check_dev(q_rot, "q_rot_scratch")) != WM_OK) return st;
  if ((st = check_dev(k_rot, "k_rot_scratch")) != WM_OK) return st;
  if (workspace && !aligned16(workspace)) return fail(WM_E_ARG, "workspace is not 16-byte aligned");
  return WM_OK;
}

// n_denoise x (RoPE of Q and K, attention), then, with `append`, the append
// of the last step's K and V (bookkeeping advanced only with `commit`).
// Launched directly, the first attention is ordered after a pending append on
// a finalize stream (the null stream is a stream like any other here); a
// recorded step leaves that to the graph launch.
wm_status do_step(wm_kvring* ring, int n_denoise, const wm_bf16* const* q, const wm_bf16* const* k,
                  const wm_bf16* const* v, int n_frames, const uint8_t* active, wm_bf16* q_rot,
                  wm_bf16* k_rot, wm_bf16* const* out, void* ws, size_t ws_bytes,
                  wm_append_report* rep, Sink& sink, bool append, bool commit = true) {
  wm_status st;
  const wm_kvring_desc& d = ring->desc;
  for (int i = 0; i < n_denoise; ++i) {
    if ((st = do_rope(ring, q[i], q_rot, d.n_q_heads, n_frames, nullptr, active, sink, k[i], k_rot,
                      d.n_kv_heads)) != WM_OK)
      return st;
    if (i == 0 && !sink.rec && (st = wait_finalize(ring, sink.s)) != WM_OK) return st;
    if ((st = do_attn(ring, 0, q_rot, k_rot, v[i], n_frames, active, 0.f, out[i], ws, ws_bytes,
                      sink)) != WM_OK)
      return st;
  }
  if (append)
    return do_append(ring, k[n_denoise - 1], v[n_denoise - 1], n_frames, active, rep, sink, commit);
  return WM_OK;
}

// The launches of one graph step for the ring's current state, recorded;
// nothing is committed.  reps (host [B]) receives the append reports.
wm_status plan_graph_step(wm_rollout_graph* g, std::vector<PLaunch>* plan, wm_append_report* reps) {
  Sink rec;
  rec.rec = plan;
  plan->reserve(4 * g->D + 4);
  return do_step(g->ring, g->D, g->q.data(), g->k.data(), g->v.data(), g->n_frames,
                 g->has_active ? g->active.data() : nullptr, g->q_rot, g->k_rot, g->out.data(), g->ws,
                 g->ws_bytes, reps, rec, true, false);
}

// A graph of the planned launches in one dependency chain, and its instance.
// A step with no active rollout plans no launch: then there is no graph and
// a launch enqueues only the completion event.
hipError_t build_graph(wm_rollout_graph* g, std::vector<PLaunch>& plan) {
  if (plan.empty()) return hipSuccess;
  hipError_t e = hipGraphCreate(&g->graph, 0);
  for (size_t i = 0; e == hipSuccess && i < plan.size(); ++i) {
    hipKernelNodeParams kp = node_params(plan[i]);
    hipGraphNode_t node;
    e = hipGraphAddKernelNode(&node, g->graph, i ? &g->nodes.back() : nullptr, i ? 1 : 0, &kp);
    if (e == hipSuccess) {
      g->nodes.push_back(node);
      g->shape.push_back(plan[i].spec);
    }
  }
  if (e == hipSuccess) e = hipGraphInstantiate(&g->exec, g->graph, nullptr, nullptr, 0);
  if (e == hipSuccess) g->held = plan;
  return e;
}

bool same_params(PLaunch& a, PLaunch& b) {
  return a.attn == b.attn &&
         memcmp(a.args(), b.args(), a.attn ? sizeof(wm::AttnParams) : sizeof(wm::RopeParams)) == 0;
}

// Drops the graph and its instance once their last launch has finished.
// Errors of these release calls are ignored: nothing is left to report to.
void drop_graph(wm_rollout_graph* g) {
  if (g->launched) (void)hipEventSynchronize(g->ev_done);
  g->launched = false;
  if (g->exec) (void)hipGraphExecDestroy(g->exec);
  if (g->graph) (void)hipGraphDestroy(g->graph);
  g->exec = nullptr;
  g->graph = nullptr;
  g->nodes.clear();
  g->shape.clear();
  g->held.clear();
}

// Arguments of wm_rope3d (for each tensor of wm_rope3d_pair).
// Arguments of an attention call (everything but the workspace).
wm_status check_attn(const wm_kvring* ring, int layer, const wm_bf16* q_rot, const wm_bf16* k_rot,
                     const wm_bf16* v, int n_frames, float softmax_scale, const wm_bf16* out) {
  wm_status st;
  if ((st = check_ring(ring)) != WM_OK) return st;
  if (layer < 0 || layer >= ring->n_layers)
    return fail(WM_E_ARG, "layer %d not in [0, %d)", layer, ring->n_layers);
  if ((st = check_device_ring(ring)) != WM_OK) return st;
  if ((st = check_dev(q_rot, "q_rot")) != WM_OK) return st;
  if ((st = check_dev(k_rot, "k_rot")) != WM_OK) return st;
  if ((st = check_dev(v, "v")) != WM_OK) return st;
  if ((st = check_dev(out, "out")) != WM_OK) return st;
  if ((st = check_frames(ring, n_frames)) != WM_OK) return st;
  if (!isfinite(softmax_scale)) return fail(WM_E_ARG, "softmax_scale is not finite");
  return WM_OK;
}

wm_status check_rope(const wm_kvring* ring, const wm_bf16* x, wm_bf16* y, int32_t n_heads,
                     int32_t n_frames, const int64_t* t_first, const uint8_t* active) {
  wm_status st;
  if ((st = check_ring(ring)) != WM_OK) return st;
  if ((st = check_device_ring(ring)) != WM_OK) return st;
  if ((st = check_dev(x, "x")) != WM_OK) return st;
  if ((st = check_dev(y, "y")) != WM_OK) return st;
  if ((st = check_frames(ring, n_frames)) != WM_OK) return st;
  if (n_heads < 1 || n_heads > 256) return fail(WM_E_SHAPE, "n_heads %d not in [1, 256]", n_heads);
  if ((int64_t)n_frames * ring->ft * n_heads * ring->desc.head_dim >= (int64_t)1 << 31)
    return fail(WM_E_SHAPE, "tensor of 2^31 elements or more per rollout");  // 32-bit offsets
  if (t_first)
    for (int b = 0; b < ring->desc.batch; ++b)
      if (is_active(active, b) && (t_first[b] < 0 || t_first[b] > ((int64_t)1 << 52)))
        return fail(WM_E_ARG, "t_first[%d] out of range [0, 2^52]", b);
  return WM_OK;
}

}  // namespace

extern "C" {

size_t wm_kvring_pool_bytes(const wm_kvring_desc* desc) {
  Bands b;
  if (check_desc(desc, &b) != WM_OK) return 0;
  return layout_of(*desc, b).total;
}

wm_status wm_kvring_create(const wm_kvring_desc* desc, void* dev_pool, size_t pool_bytes,
                           wm_kvring** out) {
  if (!out) return fail(WM_E_ARG, "out is NULL");
  Bands bands;
  wm_status st = check_desc(desc, &bands);
  if (st != WM_OK) return st;
  const Layout L = layout_of(*desc, bands);
  const bool meta = dev_pool == nullptr && pool_bytes == 0;
  if (!meta) {
    if (!dev_pool) return fail(WM_E_ARG, "dev_pool is NULL but pool_bytes is not 0");
    if (!aligned16(dev_pool)) return fail(WM_E_ARG, "dev_pool is not 16-byte aligned");
    if (pool_bytes < L.total)
      return fail(WM_E_CAPACITY, "pool of %zu bytes, ring needs %zu", pool_bytes, L.total);
  }
  wm_kvring* r = new wm_kvring();
  r->desc = *desc;
  r->bands = bands;
  r->L = L;
  r->ft = (int)ft_of(*desc);
  r->R = desc->n_sink + desc->window;
  r->n_layers = layers_of(*desc);
  r->meta_only = meta;
  r->pool = static_cast<uint8_t*>(dev_pool);
  r->n_committed.assign(desc->batch, 0);
  r->t0.assign(desc->batch, 0);
  for (int j = 0; j < bands.dt / 2; ++j) r->inv_t.push_back(inv_freq(desc->rope_theta, j, bands.dt));
  if (!meta && L.tab_bytes) {
    std::vector<uint8_t> host(L.tab_bytes, 0);
    // fp64 copies of the fp32-rounded values (exact), so the kernels skip
    // the widening.
    double* cs = reinterpret_cast<double*>(host.data());
    auto fill = [&](int n_pos, int da) {
      for (int pos = 0; pos < n_pos; ++pos)
        for (int j = 0; j < da / 2; ++j) {
          const double ang = (double)pos * inv_freq(desc->rope_theta, j, da);
          *cs++ = (double)(float)g_cos(ang);
          *cs++ = (double)(float)g_sin(ang);
        }
    };
    fill(desc->frame_h, bands.dh);
    fill(desc->frame_w, bands.dw);
    hipError_t e = hipMemcpy(r->pool + L.tab_off, host.data(), L.tab_bytes, hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipMemset(r->pool + L.cnt_off, 0, L.cnt_bytes);
    if (e != hipSuccess) {
      delete r;
      return hip_fail(e, "table upload");
    }
  }
  {
    std::lock_guard<std::mutex> lk(g_mu);
    r->serial = ++g_serial;
    g_live.insert(r);
  }
  *out = r;
  return ok();
}

wm_status wm_kvring_destroy(wm_kvring* ring) {
  wm_status st = check_ring(ring);
  if (st != WM_OK) return st;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    g_live.erase(ring);
  }
  if (ring->ev_attn) (void)hipEventDestroy(ring->ev_attn);
  if (ring->ev_fin) (void)hipEventDestroy(ring->ev_fin);
  delete ring;
  return ok();
}

wm_status wm_kvring_reset(wm_kvring* ring, int32_t b, int64_t t0) {
  wm_status st = check_ring(ring);
  if (st != WM_OK) return st;
  if (b < 0 || b >= ring->desc.batch) return fail(WM_E_ARG, "rollout %d out of range", b);
  if (t0 < 0 || t0 > ((int64_t)1 << 52)) return fail(WM_E_ARG, "t0 out of range [0, 2^52]");
  ring->n_committed[b] = 0;
  ring->t0[b] = t0;
  return ok();
}

wm_status wm_kvring_view(const wm_kvring* ring, int32_t b, wm_ring_view* out) {
  wm_status st = check_ring(ring);
  if (st != WM_OK) return st;
  if (!out) return fail(WM_E_ARG, "out is NULL");
  if (b < 0 || b >= ring->desc.batch) return fail(WM_E_ARG, "rollout %d out of range", b);
  const int64_t S = ring->desc.n_sink, W = ring->desc.window, m = ring->n_committed[b];
  memset(out, 0, sizeof *out);
  int n = 0;
  for (int64_t f = 0; f < std::min(S, m); ++f) {
    out->frame[n] = f;
    out->slot[n] = (int32_t)f;
    out->t[n] = ring->t0[b] + f;
    ++n;
  }
  if (W > 0)
    for (int64_t f = std::max(S, m - W); f < m; ++f) {
      out->frame[n] = f;
      out->slot[n] = (int32_t)(S + (f - S) % W);
      out->t[n] = ring->t0[b] + f;
      ++n;
    }
  out->n_retained = n;
  out->n_committed = m;
  out->t0 = ring->t0[b];
  return ok();
}

wm_status wm_rope3d(const wm_kvring* ring, const wm_bf16* x, wm_bf16* y, int32_t n_heads,
                    int32_t n_frames, const int64_t* t_first, const uint8_t* active,
                    void* stream) {
  wm_status st;
  if ((st = check_rope(ring, x, y, n_heads, n_frames, t_first, active)) != WM_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Sink k{s};
  if ((st = do_rope(ring, x, y, n_heads, n_frames, t_first, active, k)) != WM_OK) return st;
  return finish(s);
}

wm_status wm_rope3d_pair(const wm_kvring* ring, const wm_bf16* x, wm_bf16* y, int32_t n_heads,
                         const wm_bf16* x2, wm_bf16* y2, int32_t n_heads2, int32_t n_frames,
                         const int64_t* t_first, const uint8_t* active, void* stream) {
  wm_status st;
  if ((st = check_rope(ring, x, y, n_heads, n_frames, t_first, active)) != WM_OK) return st;
  if ((st = check_rope(ring, x2, y2, n_heads2, n_frames, t_first, active)) != WM_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Sink k{s};
  if ((st = do_rope(ring, x, y, n_heads, n_frames, t_first, active, k, x2, y2, n_heads2)) != WM_OK)
    return st;
  return finish(s);
}

size_t wm_chunk_attn_workspace_bytes(const wm_kvring* ring, int32_t n_frames) {
  if (check_ring(ring) != WM_OK) return 0;
  if (n_frames < 1 || n_frames > ring->desc.max_chunk) return 0;
  // Largest workspace any launch group (1 .. min(B, rollouts per launch)
  // rollouts, full window) would use.
  const wm_kvring_desc& d = ring->desc;
  const int ntiles = ((ring->R + n_frames) * ring->ft + 63) / 64;
  const int nq = n_frames * ring->ft;
  size_t best = 0;
  for (int nb = 1; nb <= std::min(d.batch, wm::kAttnMaxB); ++nb) {
    const int ns = choose_split(nb * d.n_kv_heads * wg_per_bg_of(ring, n_frames), ntiles);
    if (ns > 1) best = std::max(best, split_ws_bytes(ns, nb, nq, d.n_q_heads, d.head_dim));
  }
  return best;
}

wm_status wm_chunk_attn(const wm_kvring* ring, const wm_bf16* q_rot, const wm_bf16* k_rot,
                        const wm_bf16* v, int32_t n_frames, const uint8_t* active,
                        float softmax_scale, wm_bf16* out, void* workspace,
                        size_t workspace_bytes, void* stream) {
  return wm_chunk_attn_layer(ring, 0, q_rot, k_rot, v, n_frames, active, softmax_scale, out,
                             workspace, workspace_bytes, stream);
}

wm_status wm_chunk_attn_layer(const wm_kvring* ring, int32_t layer, const wm_bf16* q_rot,
                              const wm_bf16* k_rot, const wm_bf16* v, int32_t n_frames,
                              const uint8_t* active, float softmax_scale, wm_bf16* out,
                              void* workspace, size_t workspace_bytes, void* stream) {
  wm_status st;
  if ((st = check_attn(ring, layer, q_rot, k_rot, v, n_frames, softmax_scale, out)) != WM_OK)
    return st;
  if (workspace && !aligned16(workspace)) return fail(WM_E_ARG, "workspace is not 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = wait_finalize(ring, s)) != WM_OK) return st;
  Sink k{s};
  st = do_attn(ring, layer, q_rot, k_rot, v, n_frames, active, softmax_scale, out, workspace,
               workspace_bytes, k);
  if (st != WM_OK) return st;
  return finish(s);
}

static_assert(wm::kScratchBytes == WM_NOALLOC_SCRATCH_BYTES, "scratch size");

wm_status wm_chunk_attn_noalloc(const wm_kvring* ring, const wm_bf16* q_rot, const wm_bf16* k_rot,
                                const wm_bf16* v, int32_t n_frames, const uint8_t* active,
                                float softmax_scale, wm_bf16* out, void* stream) {
  wm_status st;
  if ((st = check_attn(ring, 0, q_rot, k_rot, v, n_frames, softmax_scale, out)) != WM_OK) return st;
  // The split wm_chunk_attn takes with a large enough workspace, or an error.
  const size_t need = attn_ws_needed(ring, n_frames, attn_groups(ring, n_frames, active));
  if (need > wm::kScratchBytes)
    return fail(WM_E_CAPACITY,
                "this call's key-range split needs %zu bytes of scratch, more than the %zu the "
                "allocation-free entry point holds per device (use wm_chunk_attn with a workspace)",
                need, wm::kScratchBytes);
  void* scratch = nullptr;
  hipError_t e = wm::scratch_region(&scratch);
  if (e != hipSuccess) return hip_fail(e, "scratch address (hipGetSymbolAddress)");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = wait_finalize(ring, s)) != WM_OK) return st;
  Sink k{s};
  st = do_attn(ring, 0, q_rot, k_rot, v, n_frames, active, softmax_scale, out, scratch,
               wm::kScratchBytes, k);
  if (st != WM_OK) return st;
  return finish(s);
}

wm_status wm_kvring_append_evict(wm_kvring* ring, const wm_bf16* k_raw, const wm_bf16* v,
                                 int32_t n_frames, const uint8_t* active,
                                 wm_append_report* rep, void* stream) {
  wm_status st;
  if ((st = check_ring(ring)) != WM_OK) return st;
  if ((st = check_frames(ring, n_frames)) != WM_OK) return st;
  if (!ring->meta_only) {
    if ((st = check_dev(k_raw, "k_raw")) != WM_OK) return st;
    if ((st = check_dev(v, "v")) != WM_OK) return st;
  }
  if ((st = check_room(ring, n_frames, active)) != WM_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!ring->meta_only && (st = wait_finalize(ring, s)) != WM_OK) return st;
  Sink k{s};
  if ((st = do_append(ring, k_raw, v, n_frames, active, rep, k)) != WM_OK) return st;
  if (ring->meta_only) return ok();
  return finish(s);
}

wm_status wm_rollout_step(wm_kvring* ring, int32_t n_denoise, const wm_bf16* const* q,
                          const wm_bf16* const* k, const wm_bf16* const* v, int32_t n_frames,
                          const uint8_t* active, wm_bf16* q_rot_scratch, wm_bf16* k_rot_scratch,
                          wm_bf16* const* out, void* workspace, size_t workspace_bytes,
                          wm_append_report* rep, void* stream, void* finalize_stream) {
  wm_status st;
  if ((st = check_step(ring, n_denoise, q, k, v, n_frames, q_rot_scratch, k_rot_scratch, out,
                       workspace)) != WM_OK)
    return st;
  if ((st = check_room(ring, n_frames, active)) != WM_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipStream_t fs = static_cast<hipStream_t>(finalize_stream);
  Sink main{s};
  if (!fs || fs == s) {
    st = do_step(ring, n_denoise, q, k, v, n_frames, active, q_rot_scratch, k_rot_scratch, out,
                 workspace, workspace_bytes, rep, main, true);
    if (st != WM_OK) return st;
    return finish(s);
  }
  // Overlapped finalize: the append waits only for this step's last
  // attention (it overwrites the slots that attention read) and runs on the
  // finalize stream; the next call's pool accesses wait for it.
  if ((st = make_events(ring)) != WM_OK) return st;
  st = do_step(ring, n_denoise, q, k, v, n_frames, active, q_rot_scratch, k_rot_scratch, out,
               workspace, workspace_bytes, rep, main, false);
  if (st != WM_OK) return st;
  hipError_t e = hipEventRecord(ring->ev_attn, s);
  if (e == hipSuccess) e = hipStreamWaitEvent(fs, ring->ev_attn, 0);
  if (e != hipSuccess) return hip_fail(e, "finalize ordering");
  Sink fin{fs};
  if ((st = do_append(ring, k[n_denoise - 1], v[n_denoise - 1], n_frames, active, rep, fin)) != WM_OK)
    return st;
  e = hipEventRecord(ring->ev_fin, fs);
  if (e != hipSuccess) return hip_fail(e, "finalize event");
  ring->fin_recorded = true;
  if ((st = finish(s)) != WM_OK) return st;
  return finish(fs);
}

wm_status wm_rollout_graph_create(wm_kvring* ring, int32_t n_denoise, const wm_bf16* const* q,
                                  const wm_bf16* const* k, const wm_bf16* const* v,
                                  int32_t n_frames, const uint8_t* active, wm_bf16* q_rot_scratch,
                                  wm_bf16* k_rot_scratch, wm_bf16* const* out, void* workspace,
                                  size_t workspace_bytes, wm_rollout_graph** graph_out) {
  wm_status st;
  if (!graph_out) return fail(WM_E_ARG, "graph_out is NULL");
  if ((st = check_step(ring, n_denoise, q, k, v, n_frames, q_rot_scratch, k_rot_scratch, out,
                       workspace)) != WM_OK)
    return st;
  wm_rollout_graph* g = new wm_rollout_graph();
  g->ring = ring;
  g->ring_serial = ring->serial;
  g->D = n_denoise;
  g->n_frames = n_frames;
  g->has_active = active != nullptr;
  if (active) g->active.assign(active, active + ring->desc.batch);
  g->q.assign(q, q + n_denoise);
  g->k.assign(k, k + n_denoise);
  g->v.assign(v, v + n_denoise);
  g->out.assign(out, out + n_denoise);
  g->q_rot = q_rot_scratch;
  g->k_rot = k_rot_scratch;
  g->ws = workspace;
  g->ws_bytes = workspace_bytes;
  // The launches of one step for the ring as it is now (nothing committed).
  std::vector<PLaunch> plan;
  if ((st = plan_graph_step(g, &plan, nullptr)) != WM_OK) {
    delete g;
    return st;
  }
  hipError_t e = hipEventCreateWithFlags(&g->ev_done, hipEventDisableTiming);
  if (e == hipSuccess) e = build_graph(g, plan);
  if (e != hipSuccess) {
    drop_graph(g);
    if (g->ev_done) (void)hipEventDestroy(g->ev_done);
    delete g;
    return hip_fail(e, "graph build");
  }
  {
    std::lock_guard<std::mutex> lk(g_mu);
    g_graphs.insert(g);
  }
  *graph_out = g;
  return ok();
}

wm_status wm_rollout_graph_launch(wm_rollout_graph* g, wm_append_report* rep, int32_t* rebuilt,
                                  void* stream) {
  {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g || !g_graphs.count(g)) return fail(WM_E_STATE, "graph handle is not live");
  }
  wm_status st;
  wm_kvring* ring = g->ring;
  if ((st = check_ring(ring)) != WM_OK) return st;
  if (ring->serial != g->ring_serial) return fail(WM_E_STATE, "the graph's ring was destroyed");
  const uint8_t* active = g->has_active ? g->active.data() : nullptr;
  if ((st = check_room(ring, g->n_frames, active)) != WM_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  std::vector<PLaunch> plan;
  std::vector<wm_append_report> reps(ring->desc.batch);
  if ((st = plan_graph_step(g, &plan, reps.data())) != WM_OK) return st;
  bool same = plan.size() == g->shape.size();
  for (size_t i = 0; same && i < plan.size(); ++i) {
    const wm::LaunchSpec &a = plan[i].spec, &b = g->shape[i];
    same = a.func == b.func && a.grid.x == b.grid.x && a.grid.y == b.grid.y && a.grid.z == b.grid.z &&
           a.block.x == b.block.x;
  }
  if ((st = wait_finalize(ring, s)) != WM_OK) return st;
  hipError_t e = hipSuccess;
  if (same) {
    // Only the nodes whose parameters changed since their last update (in
    // steady state: the RoPE rows' positions and the append's slots; an
    // attention over a full window keeps its parameters).
    for (size_t i = 0; e == hipSuccess && i < plan.size(); ++i) {
      if (same_params(plan[i], g->held[i])) continue;
      hipKernelNodeParams kp = node_params(plan[i]);
      e = hipGraphExecKernelNodeSetParams(g->exec, g->nodes[i], &kp);
      if (e == hipSuccess) g->held[i] = plan[i];
    }
  } else {
    // New launch shapes (the window filling, a different key split): a new
    // graph of this step's launches replaces the old one.
    drop_graph(g);
    e = build_graph(g, plan);
    if (e != hipSuccess) drop_graph(g);
  }
  if (e == hipSuccess && g->exec) e = hipGraphLaunch(g->exec, s);
  if (e == hipSuccess) e = hipEventRecord(g->ev_done, s);
  if (e != hipSuccess) return hip_fail(e, "graph launch");
  g->launched = true;
  for (int b = 0; b < ring->desc.batch; ++b)
    if (is_active(active, b)) ring->n_committed[b] += g->n_frames;
  if (rep) memcpy(rep, reps.data(), sizeof(wm_append_report) * ring->desc.batch);
  if (rebuilt) *rebuilt = same ? 0 : 1;
  return finish(s);
}

wm_status wm_rollout_graph_destroy(wm_rollout_graph* g) {
  {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g || !g_graphs.count(g)) return fail(WM_E_STATE, "graph handle is not live");
    g_graphs.erase(g);
  }
  drop_graph(g);
  (void)hipEventDestroy(g->ev_done);
  delete g;
  return ok();
}

const char* wm_last_error(void) { return g_err.c_str(); }

}  // extern "C"
