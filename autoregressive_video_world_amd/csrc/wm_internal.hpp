// Internal interface between the host runtime (wm_api.cpp) and the HIP
// kernels (kernels/*.hip).  Kernel parameters travel by value as kernel
// arguments; everything here is plain data.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wm {

// ---------------------------------------------------------------------------
// RoPE / append
// ---------------------------------------------------------------------------
constexpr int kRopeRows = 8;     // (rollout, frame) rows per launch
constexpr int kMaxTPairs = 32;   // d_t / 2 upper bound
constexpr int kRopeHeads = 4;    // heads per thread of the RoPE / append kernel

struct RopeRow {
  int32_t b;      // rollout index
  int32_t j;      // frame index within the chunk
  int32_t slot;   // append: destination ring slot (-1: not stored); rope: unused
  int32_t pad;
};

// n / d for n < 2^31 as (umulhi(n, mul) + n) >> shift (round-up multiplier
// method of Granlund and Montgomery, "Division by Invariant Integers using
// Multiplication", 1994); the host computes mul and shift for d >= 1.
struct FastDiv {
  uint32_t mul;
  uint32_t shift;
};

struct RopeParams {
  const uint16_t* x;      // rope: input chunk;  append: unrotated K of the chunk
  uint16_t* y;            // rope: output chunk; append: K half of the pool
  const uint16_t* vsrc;   // append only: V of the chunk
  uint16_t* vdst;         // append only: V half of the pool
  const double2* hw;      // (cos, sin) table: [frame_h][dh2] of the h band, then
                          // [frame_w][dw2] of the w band from entry w_base
  const uint16_t* x2;     // rope, paired: a second chunk tensor (K with Q), same rows
  uint16_t* y2;           // rope, paired: its output
  int64_t x_b_stride;     // elements per rollout in x / y (rope) or x / vsrc (append)
  int64_t x2_b_stride;    // elements per rollout in x2 / y2
  int32_t n_heads;        // heads of x
  int32_t n_heads2;       // heads of x2
  int32_t hg_first;       // rope: head groups of x; grid z beyond them covers x2
  int32_t d;              // head dim
  int32_t lg_cpr;         // log2(d / 8): 16-byte vectors per (token, head)
  int32_t ft;             // tokens per frame
  int32_t fw;             // frame width
  int32_t dt2, dh2, dw2;  // pairs per band
  int32_t ring_slots;     // S + W (append)
  int32_t w_base;         // first entry of the w band in hw
  int32_t n_rows;
  int32_t n_layers;       // append: layers written by one launch (rope: 1)
  int64_t x_layer_stride;     // append: elements between layers of x / vsrc
  int64_t pool_layer_stride;  // append: elements between layers of y / vdst
  FastDiv div_fw;         // division by frame width
  FastDiv div_fh;         // division by frame height (token -> row within its view)
  int32_t fh;             // frame height (rows of one view)
  RopeRow rows[kRopeRows];
  float2 tcs[kRopeRows][kMaxTPairs];  // (cos, sin) of the t band at each row's t
};

// One kernel launch of the library: kernel, grid and block.  Every kernel
// takes a single parameter struct by value; the host runtime launches a spec
// directly (hipLaunchKernel) or makes it a node of a HIP graph.
struct LaunchSpec {
  const void* func;
  dim3 grid;
  dim3 block;
};

LaunchSpec rope3d_spec(const RopeParams& p);
LaunchSpec kv_append_spec(const RopeParams& p);

// ---------------------------------------------------------------------------
// Chunk attention
// ---------------------------------------------------------------------------
constexpr int kAttnMaxB = 64;    // rollouts per launch
constexpr int kAttnMaxSplit = 8; // key-range splits per attention launch

struct AttnParams {
  const uint16_t* q;      // [B][Nq][Hq][d]
  const uint16_t* kc;     // [B][Nq][Hkv][d] chunk keys (rotated)
  const uint16_t* vc;     // [B][Nq][Hkv][d]
  const uint16_t* pk;     // pool K half [B][R][Hkv][Ft][d]
  const uint16_t* pv;     // pool V half
  uint16_t* out;          // [B][Nq][Hq][d]
  float* part_o;          // split-KV partial outputs (nullptr: no split)
  float* part_ml;         // split-KV (max, sum) per row
  int32_t* counters;      // split-KV arrival counters, one per row block (zero between launches)
  int32_t hq, hkv, group; // group = Hq / Hkv
  int32_t ft;             // tokens per frame
  int32_t nq;             // queries per rollout = n_frames * Ft
  int32_t ring_slots;     // R = S + W
  int32_t nqb;            // 32-query wave tasks per rollout and q head
  int32_t wg_per_bg;      // workgroups per (rollout, kv head) per split
  int32_t nsplit;         // key-range splits (1 = none)
  int32_t n_wg;           // logical workgroups (set by the launcher)
  int32_t per_xcd;        // logical workgroups per XCD (set by the launcher)
  float scale_log2e;      // softmax scale * log2(e)
  int32_t nb;             // rollouts in this launch
  int32_t b_index[kAttnMaxB];
  int32_t n_ring[kAttnMaxB];   // visible ring frames (slots 0 .. n_ring-1)
};

// Scratch of the allocation-free attention entry point (key-range split
// partials), one static device array per GPU; equal to the public
// WM_NOALLOC_SCRATCH_BYTES.
constexpr size_t kScratchBytes = (size_t)128 << 20;

// This device's address of that array: looked up with hipGetSymbolAddress on
// the first call with the device current, then cached per device.
hipError_t scratch_region(void** ptr);

// The launch of one attention group: fills p's derived fields (workgroup
// count, XCD stride) and returns the number of launches (1; 0 if the shape
// is not built).  A split launch merges its partials itself.
int chunk_attn_specs(AttnParams& p, int head_dim, LaunchSpec specs[2]);

}  // namespace wm
