/*
 * wm.h -- streaming block-causal chunk attention over a bounded KV ring,
 *         for AMD Instinct MI355X (gfx950).
 *
 * One layer of the attention of a streaming autoregressive video world
 * model.  Each generated chunk of latent frames is denoised in a few steps;
 * in every step the chunk's queries attend, bidirectionally, to the chunk's
 * own keys and to a bounded cache of earlier frames: S persistent "sink"
 * (reference) frames plus a FIFO window of the W most recent frames.  After
 * the last step the chunk's K (rotated by 3D-RoPE at its absolute (t,h,w)
 * position) and V are appended to the cache and the oldest window frames are
 * evicted, so device memory stays flat over arbitrarily long rollouts.
 *
 * Sources (web pages; section names given):
 *  - FlashDreams blog post ("NVIDIA FlashDreams Is the Open-Source Inference
 *    Engine Robotics World Models Needed"), "Bounded Memory for Infinite
 *    Rollouts": every rollout owns a cache of fixed device memory and drops
 *    old entries by itself;
 *    "Hot-Path Generation, Background State Updates": each step splits into
 *    generate() (denoising) and finalize() (KV-cache update).
 *  - Cosmos3-H-Dreams model card, "Model Architecture": block-causal few-step
 *    student with a KV cache; the conditioning frame is prefilled once;
 *    "Software Integration": static-shape KV cache, BF16.
 *  - AlpaDreams GTC write-up, section VII: the causal DiT predicts each new
 *    frame from the earlier, already denoised frames together with the frame
 *    still being denoised.
 *  - DreamZero single-GPU page, "Sequential requests": frame positions and the
 *    cache persist across requests; explicit start frame / cache reset.
 *
 * Conventions that the pages leave open (cache reading, RoPE convention,
 * rounding) are fixed as documented at each call below.
 *
 * General rules
 *  - Every device pointer is a HIP device address, 16-byte aligned.
 *  - bf16 tensors are raw IEEE bfloat16 bit patterns (wm_bf16).
 *  - Token tensors are [B][n_frames*Ft][H][d] (row-major), token index =
 *    frame*Ft + view*frame_h*frame_w + h*frame_w + w (Ft = views * frame_h *
 *    frame_w; one view unless the descriptor says more), B = desc.batch (every
 *    rollout has a row block, active or not).
 *  - `active` (host [B] or NULL = all): a call whose mask names no rollout
 *    is valid and launches no kernel (stream-ordering events aside).
 *  - `stream` is a hipStream_t (NULL = the null stream).  Every launch of a
 *    call goes onto that stream; no call synchronizes the device or copies
 *    device data to the host, with two exceptions: wm_kvring_create (a
 *    synchronous table upload) and the replacement or destruction of a
 *    rollout graph, which first waits for that graph's last launch.
 *  - The library allocates no device memory.  The caller owns the pool, all
 *    tensors, workspaces, host report/view structs and streams.
 *  - Errors: every argument is validated before anything is enqueued.  A
 *    non-zero status other than WM_E_HIP means nothing was enqueued and the
 *    ring is unchanged; wm_last_error() then returns a message
 *    (thread-local).  WM_E_HIP from a launch the runtime refused: launches
 *    of the same call before it may have been enqueued, the ring's
 *    bookkeeping (frames, slots, positions) is unchanged, but slots this call
 *    would have written may hold part of the new data -- wm_kvring_reset of
 *    the affected rollouts recovers.  Device faults are asynchronous and
 *    surface at the caller's next synchronization; with the environment
 *    variable WM_SYNC_CHECK=1 every call synchronizes its stream and reports
 *    such errors as WM_E_HIP.  WM_FAULT_INJECT=launch|rope|attn|append (read
 *    on every call, for tests of this path) makes every direct launch of that
 *    kind ("launch": any) fail that way; on a metadata-only ring "append"
 *    fails wm_kvring_append_evict at the point of its launch.
 *  - A ring is not thread-safe; calls on one ring must be ordered on one
 *    stream (or by the caller's events).
 */
#ifndef WM_H_
#define WM_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define WM_MAX_CHUNK 16  /* frames per chunk (append / attention call)      */
#define WM_MAX_RING 256  /* sink + window slots per rollout                 */
#define WM_MAX_BATCH 1024

/* What an append does when a rollout's window is full (wm_kvring_desc.evict_policy). */
#define WM_EVICT_SLIDE 0 /* evict the oldest window frame (FIFO); the default     */
#define WM_EVICT_RESET 1 /* refuse: the caller starts a new window (reset)         */

typedef uint16_t wm_bf16;
typedef struct wm_kvring wm_kvring;
typedef struct wm_rollout_graph wm_rollout_graph;

typedef enum {
  WM_OK = 0,
  WM_E_ARG = 1,         /* NULL / misaligned pointer, out-of-range scalar   */
  WM_E_SHAPE = 2,       /* shape not allowed by the ring's descriptor      */
  WM_E_STATE = 3,       /* destroyed handle, metadata-only ring, bad state */
  WM_E_CAPACITY = 4,    /* pool or workspace too small                     */
  WM_E_HIP = 5,         /* a HIP call failed                               */
  WM_E_UNSUPPORTED = 6  /* valid request the library does not implement    */
} wm_status;

typedef struct {
  int32_t batch;        /* B >= 1 independent rollouts (no cross-rollout attention)   */
  int32_t n_q_heads;    /* Hq >= 1                                                    */
  int32_t n_kv_heads;   /* Hkv >= 1, Hq % Hkv == 0; q head h reads kv head h/(Hq/Hkv) */
  int32_t head_dim;     /* d: 64 or 128                                               */
  int32_t frame_h;      /* latent grid height (of one view)                           */
  int32_t frame_w;      /* latent grid width (of one view)                            */
  int32_t n_sink;       /* S >= 0: the first S frames of a sequence, never evicted    */
  int32_t window;       /* W >= 0: FIFO window of the most recent later frames        */
  int32_t max_chunk;    /* C in [1, WM_MAX_CHUNK]: frames per call                    */
  double rope_theta;    /* RoPE base (e.g. 10000.0), > 1                              */
  int32_t rope_dims[3]; /* {d_t,d_h,d_w} even, sum d; {0,0,0} = default split:
                           d_h = d_w = 2*floor(d/6), d_t = d - d_h - d_w             */
  int32_t n_layers;     /* L in [0, 256]: attention layers sharing the ring's frames,
                           slots and positions (0 = 1).  Each layer has its own K/V
                           in the pool; an append commits every layer at once     */
  int32_t n_views;      /* V in [0, 16]: camera views per frame (0 = 1).  A frame is
                           V grids of frame_h x frame_w tokens attended jointly;
                           Ft = V*frame_h*frame_w (AlpaDreams write-up, VII and
                           VIII: a four-view model, up to seven cameras, views
                           attended together by one Transformer)                 */
  int32_t evict_policy; /* WM_EVICT_SLIDE or WM_EVICT_RESET (DreamZero page,
                           "Sequential requests": at the local-attention window
                           boundary the old KV is released, the frame position
                           reset and a new window started)                         */
} wm_kvring_desc;

/* Per-rollout result of one append, in commit order.  A frame that is
 * committed but not stored (W == 0 and not a sink, or pushed out again by a
 * later frame of the same append) still appears in frame/slot/t; slot is -1
 * when it is never stored, and it is listed in `evicted` when a later frame
 * of the same append pushes it out. */
typedef struct {
  int32_t n_written;                 /* frames committed by this append       */
  int32_t n_evicted;                 /* frames evicted by this append         */
  int64_t frame[WM_MAX_CHUNK];       /* frame id within the sequence          */
  int32_t slot[WM_MAX_CHUNK];        /* ring slot it was assigned, or -1      */
  int64_t t[WM_MAX_CHUNK];           /* absolute temporal position t0 + frame */
  int64_t evicted[WM_MAX_CHUNK];     /* evicted frame ids, oldest first       */
} wm_append_report;

/* Frames a rollout holds, in temporal order. */
typedef struct {
  int32_t n_retained;
  int64_t frame[WM_MAX_RING];
  int32_t slot[WM_MAX_RING];
  int64_t t[WM_MAX_RING];
  int64_t n_committed;               /* frames committed since the last reset */
  int64_t t0;                        /* temporal origin of the sequence       */
} wm_ring_view;

/* ---------------------------------------------------------------------------
 * Pool
 *
 * Bytes of device memory a ring needs (0 if the descriptor is invalid).
 * Layout, all offsets from the pool base, per layer l = 0 .. L-1 at
 * l * layer bytes (layer bytes = K half + V half, each rounded up to 256):
 *   K half : bf16 [B][S+W][Hkv][Ft][d]   -- each (slot, kv head) one
 *                                           contiguous Ft x d block
 *   V half : bf16 [B][S+W][Hkv][Ft][d]   -- after the K half (256-aligned)
 * then, after the L layers, once:
 *   tables : (cos, sin) pairs of the h and w RoPE bands, [frame_h][d_h/2]
 *            then [frame_w][d_w/2]: fp64 copies of fp32-rounded values,
 *            256-byte aligned
 *   counters: int32, one per row block of the largest attention launch
 *            (min(B, 64) * Hkv * ceil(Hq/Hkv * ceil(C*Ft/32) / 8)), rounded up
 *            to 256 bytes: arrivals of the workgroups of a key-range split,
 *            zero between calls (the last arrival resets its counter)
 * Slot of frame f of a sequence: f if f < S, else S + (f - S) mod W.
 */
size_t wm_kvring_pool_bytes(const wm_kvring_desc* desc);

/* Create a ring over a caller-owned device pool of at least
 * wm_kvring_pool_bytes(desc) bytes (16-byte aligned, valid until destroy).
 * Writes the RoPE h/w tables into the pool's table area with a synchronous
 * host-to-device copy and zeroes the counters; K/V slot contents are left
 * as they are.  Every
 * rollout starts empty at t0 = 0.
 * dev_pool == NULL with pool_bytes == 0 creates a metadata-only ring: appends
 * update the bookkeeping and reports only (no device access), and
 * wm_rope3d / wm_chunk_attn / wm_rollout_step return WM_E_STATE.
 * Errors: WM_E_ARG (NULL desc/out, misaligned pool), WM_E_SHAPE (invalid
 * descriptor, including a rollout's chunk tensor max_chunk*Ft*Hq*d or its
 * K half (S+W)*Hkv*Ft*d reaching 2^31 elements, or (S+W+C)*Ft reaching 2^24
 * keys), WM_E_CAPACITY (pool too small), WM_E_HIP. */
wm_status wm_kvring_create(const wm_kvring_desc* desc, void* dev_pool, size_t pool_bytes,
                           wm_kvring** out);

/* Release the handle (host memory only; the pool stays the caller's).
 * Calls with a destroyed handle return WM_E_STATE. */
wm_status wm_kvring_destroy(wm_kvring* ring);

/* Start a new sequence on rollout b: no frames committed, temporal origin
 * t0 (DreamZero page, "Sequential requests": current start frame and cache
 * reset).  Old slot contents are simply no longer visible. */
wm_status wm_kvring_reset(wm_kvring* ring, int32_t b, int64_t t0);

/* Retained frames of rollout b in temporal order (sinks, then window). */
wm_status wm_kvring_view(const wm_kvring* ring, int32_t b, wm_ring_view* out);

/* ---------------------------------------------------------------------------
 * 3D-RoPE of a chunk's Q or K (one denoise step).
 *
 * x, y : bf16 [B][n_frames*Ft][n_heads][d] (y may equal x).  Token r of chunk
 * frame j of rollout b sits at t = t_first[b] + j and, within its view,
 * h = (r mod frame_h*frame_w) / frame_w, w = r mod frame_w (every view has
 * its own grid; views of one frame share t); t_first == NULL means each
 * rollout's next uncommitted frame (t0 + n_committed).  Bands [t | h | w] of
 * the head dim; in a band of width d_a, pair j = elements (2j, 2j+1) rotated
 * by angle pos*theta^(-2j/d_a); cos/sin are libm fp64 values rounded once to
 * fp32 (computed on the host);
 * y0 = x0*c - x1*s, y1 = x0*s + x1*c in fp64 (the products are exact), then
 * rounded to bf16 round-to-nearest-even.  Only active rollouts (active[b] !=
 * 0; NULL = all) are read or written.
 * Errors: WM_E_ARG, WM_E_SHAPE (n_frames not in [1, max_chunk], n_heads not
 * in [1, 256], n_frames*Ft*n_heads*d of 2^31 or more), WM_E_STATE
 * (metadata-only ring), WM_E_HIP. */
wm_status wm_rope3d(const wm_kvring* ring, const wm_bf16* x, wm_bf16* y, int32_t n_heads,
                    int32_t n_frames, const int64_t* t_first, const uint8_t* active, void* stream);

/* wm_rope3d of two tensors of the same chunk frames (the Q and K of one
 * denoise step) in one launch: x (n_heads) into y and x2 (n_heads2) into y2,
 * each with its own [B][n_frames*Ft][heads][d] layout and the same positions.
 * Results are bit-identical to two wm_rope3d calls.  y may equal x and y2
 * may equal x2; the pair (x, y) must not overlap (x2, y2).
 * Errors: as wm_rope3d, for either tensor. */
wm_status wm_rope3d_pair(const wm_kvring* ring, const wm_bf16* x, wm_bf16* y, int32_t n_heads,
                         const wm_bf16* x2, wm_bf16* y2, int32_t n_heads2, int32_t n_frames,
                         const int64_t* t_first, const uint8_t* active, void* stream);

/* ---------------------------------------------------------------------------
 * Chunk attention (one denoise step; FlashDreams generate()).
 *
 * For every active rollout b and q head h (kv head g = h / (Hq/Hkv)):
 *   out[b,i,h,:] = softmax_j( q_rot[b,i,h,:] . K_j / scale^-1 ) V_j
 * over the keys j of: the sink frames and window frames rollout b holds
 * (committed K_rot/V in the pool) and all n_frames frames of the chunk itself
 * (k_rot, v of this step) -- bidirectional inside the chunk, no other mask.
 * q_rot : bf16 [B][n_frames*Ft][Hq][d]     (already rotated, see wm_rope3d)
 * k_rot : bf16 [B][n_frames*Ft][Hkv][d]    (already rotated)
 * v     : bf16 [B][n_frames*Ft][Hkv][d]
 * out   : bf16 [B][n_frames*Ft][Hq][d], round-to-nearest-even of the fp32
 *         result (bf16 MFMA products, fp32 accumulation and softmax).
 * Inputs must be finite and every scaled score q.k*scale finite in fp32;
 * NaN or infinite inputs, or scores that overflow fp32, are outside the
 * contract (the kernel does not screen for them).
 * softmax_scale <= 0 selects 1/sqrt(d).
 * workspace: optional device scratch for splitting long key ranges across
 * workgroups (more parallelism when B*Hq*Nq is small); NULL/0 = no split.
 * wm_chunk_attn_workspace_bytes() gives the size that enables the split.  The
 * split count is chosen per launch from the workgroup count and key length;
 * the environment variable WM_ATTN_SPLIT=n (1..8) overrides it (tuning,
 * tests) and is also honoured by wm_chunk_attn_workspace_bytes().  A split
 * that does not fit the given workspace is reduced until it does.  The
 * workspace (like the RoPE scratch of wm_rollout_step) is written and read by
 * this call's launches on `stream`: calls that may run at the same time, on
 * other streams, need workspaces of their own.
 * Errors: WM_E_ARG, WM_E_SHAPE, WM_E_STATE, WM_E_HIP. */
wm_status wm_chunk_attn(const wm_kvring* ring, const wm_bf16* q_rot, const wm_bf16* k_rot,
                        const wm_bf16* v, int32_t n_frames, const uint8_t* active,
                        float softmax_scale, wm_bf16* out, void* workspace,
                        size_t workspace_bytes, void* stream);

/* wm_chunk_attn on layer `layer` (0 .. L-1) of a multi-layer ring: the same
 * computation over that layer's committed K/V (wm_chunk_attn is layer 0).
 * A whole model's cache then lives in one static pool whose size does not
 * grow with the rollout (FlashDreams post, "Bounded Memory for Infinite
 * Rollouts": per-rollout caches of fixed VRAM; Cosmos3-H-Dreams card,
 * "Software Integration": static-shape KV cache).
 * Errors: as wm_chunk_attn; WM_E_ARG for a layer out of range. */
wm_status wm_chunk_attn_layer(const wm_kvring* ring, int32_t layer, const wm_bf16* q_rot,
                              const wm_bf16* k_rot, const wm_bf16* v, int32_t n_frames,
                              const uint8_t* active, float softmax_scale, wm_bf16* out,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes that let wm_chunk_attn split the key range for a chunk of
 * n_frames frames (0 if splitting never pays for this ring's shapes). */
size_t wm_chunk_attn_workspace_bytes(const wm_kvring* ring, int32_t n_frames);

/* ---------------------------------------------------------------------------
 * Allocation-free attention: for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  The caller still passes the inputs and the output.
 *
 * Computes exactly what wm_chunk_attn (layer 0) computes with a workspace of
 * at least wm_chunk_attn_workspace_bytes(): the same launches with the same
 * key-range split, hence the same output bits.  The split partials live in a
 * static device array of WM_NOALLOC_SCRATCH_BYTES that the library holds on
 * every GPU it runs on until the process ends; its device address is looked
 * up once per device (the first call with that device current).  The call
 * allocates nothing (no hipMalloc/hipFree, no allocating library routine).
 * The array needs no clearing: every split partial a launch reads was
 * written by that launch.
 * All calls on one GPU share that GPU's array and it keeps the last call's
 * contents: calls that can overlap on one GPU (other streams, other threads,
 * other rings) race on it and must be ordered by the caller.
 * Errors: as wm_chunk_attn; WM_E_CAPACITY (nothing enqueued) when the call's
 * split needs more than WM_NOALLOC_SCRATCH_BYTES (e.g. many rollouts with
 * long key ranges): use wm_chunk_attn with a workspace there. */
#define WM_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
wm_status wm_chunk_attn_noalloc(const wm_kvring* ring, const wm_bf16* q_rot, const wm_bf16* k_rot,
                                const wm_bf16* v, int32_t n_frames, const uint8_t* active,
                                float softmax_scale, wm_bf16* out, void* stream);

/* ---------------------------------------------------------------------------
 * Append + evict (FlashDreams finalize()).
 *
 * Commits n_frames frames to every active rollout: frame ids n_committed ..
 * n_committed+n_frames-1, t = t0 + id.  K is rotated by the same rule as
 * wm_rope3d at each frame's t and stored with V in the frame's slot; the
 * oldest window frames are evicted FIFO; sinks are never evicted.  Frames
 * that would be evicted again within the same append are not written.
 * k_raw, v : bf16 [L][B][n_frames*Ft][Hkv][d] (unrotated K; L = the ring's
 *            layers, layer-major): one bookkeeping step and one launch write
 *            every layer's K and V into its own pool slice.
 * rep      : host array [B] or NULL; filled for active rollouts (inactive
 *            rollouts get n_written = n_evicted = 0).
 * With evict_policy WM_EVICT_RESET an append that would evict a frame (or,
 * with W == 0, commit one past the sinks) fails with WM_E_CAPACITY and
 * changes nothing: the caller starts a new window with wm_kvring_reset (new
 * origin, slots reused from 0) and prefills its conditioning again.
 * Classifier-free guidance runs its branches as separate rollouts of the
 * batch (each with its own cache); the guidance combine is outside this call.
 * Bookkeeping is host-side closed form: no device readback.  Stream order
 * matters: an append overwrites the slot of each frame it evicts, which the
 * chunk's own attention read, so it must follow that attention on the stream.
 * Prefill (conditioning frames committed without attention) is this call.
 * Errors: WM_E_ARG, WM_E_SHAPE, WM_E_CAPACITY (reset policy, window full),
 * WM_E_HIP. */
wm_status wm_kvring_append_evict(wm_kvring* ring, const wm_bf16* k_raw, const wm_bf16* v,
                                 int32_t n_frames, const uint8_t* active,
                                 wm_append_report* rep, void* stream);

/* ---------------------------------------------------------------------------
 * One whole chunk: n_denoise x (RoPE of Q and K, chunk attention), then the
 * append of the last step's K and V.
 * q[s], k[s], v[s] : host arrays of n_denoise device pointers (step s inputs,
 *                    unrotated), shapes as in wm_chunk_attn.
 * q_rot_scratch    : bf16 [B][n_frames*Ft][Hq][d] device scratch
 * k_rot_scratch    : bf16 [B][n_frames*Ft][Hkv][d] device scratch
 * out[s]           : host array of n_denoise device output pointers.
 * workspace        : as for wm_chunk_attn.
 * rep              : as for wm_kvring_append_evict.
 * finalize_stream  : NULL (or `stream`) = everything on `stream`.  Otherwise
 *                    the append (FlashDreams post, "Hot-Path Generation,
 *                    Background State Updates": finalize() off the critical
 *                    path) goes to finalize_stream, ordered after this step's
 *                    last attention only; every later call on the ring that
 *                    reads or writes the pool waits for it, so the next
 *                    step's RoPE overlaps it.  The append reads
 *                    k[n_denoise-1] and v[n_denoise-1] on finalize_stream
 *                    after this call returns: the caller keeps them
 *                    unchanged and allocated until finalize_stream has
 *                    passed this point (an event recorded there after the
 *                    call marks it).
 * One-layer rings only (a model with L layers interleaves other work between
 * its layers: it calls wm_rope3d / wm_chunk_attn_layer per layer and one
 * wm_kvring_append_evict for all of them).
 * Errors: as the calls it makes; WM_E_UNSUPPORTED for a multi-layer ring;
 * validation of everything happens first. */
wm_status wm_rollout_step(wm_kvring* ring, int32_t n_denoise, const wm_bf16* const* q,
                          const wm_bf16* const* k, const wm_bf16* const* v, int32_t n_frames,
                          const uint8_t* active, wm_bf16* q_rot_scratch, wm_bf16* k_rot_scratch,
                          wm_bf16* const* out, void* workspace, size_t workspace_bytes,
                          wm_append_report* rep, void* stream, void* finalize_stream);

/* ---------------------------------------------------------------------------
 * One rollout step as a HIP graph (Cosmos-H-Dreams news item: inference with
 * compilation and CUDA Graphs; Cosmos3-H-Dreams card, "Software
 * Integration": static shapes).
 *
 * wm_rollout_graph_create builds a graph of the launches wm_rollout_step
 * would make for these buffers (fixed for the graph's life) and this active
 * set, from the ring as it is now; it changes nothing.  The graph holds only
 * kernel nodes, in one dependency chain (none when no rollout is active: a
 * launch then runs nothing).
 * wm_rollout_graph_launch runs one step: it plans the step from the ring's
 * bookkeeping (positions, slots, visible frames), writes those parameters
 * into the graph's nodes and launches the graph on `stream`, then commits
 * the append like wm_kvring_append_evict.  When the planned launches differ
 * in kernel or grid from the graph's (the window still filling, a different
 * key split), the graph is first rebuilt for them, after its previous launch
 * has finished (the host waits for it); *rebuilt (may be NULL) is 1 then.
 * Results are those of wm_rollout_step either way.
 * The graph and its executable instance are HIP objects the library creates
 * (host and driver memory); the ring's pool and the tensors stay the
 * caller's.  wm_rollout_graph_destroy waits for the graph's last launch and
 * releases them.  Once its ring is destroyed a graph can only be destroyed.
 * Errors: as wm_rollout_step (create and launch: WM_E_HIP for a failed graph
 * call); WM_E_STATE for a dead graph handle or, at launch, once the graph's
 * ring has been destroyed. */
wm_status wm_rollout_graph_create(wm_kvring* ring, int32_t n_denoise, const wm_bf16* const* q,
                                  const wm_bf16* const* k, const wm_bf16* const* v,
                                  int32_t n_frames, const uint8_t* active, wm_bf16* q_rot_scratch,
                                  wm_bf16* k_rot_scratch, wm_bf16* const* out, void* workspace,
                                  size_t workspace_bytes, wm_rollout_graph** graph_out);
wm_status wm_rollout_graph_launch(wm_rollout_graph* graph, wm_append_report* rep,
                                  int32_t* rebuilt, void* stream);
wm_status wm_rollout_graph_destroy(wm_rollout_graph* graph);

/* Thread-local message for the last non-OK status ("" if none). */
const char* wm_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* WM_H_ */
