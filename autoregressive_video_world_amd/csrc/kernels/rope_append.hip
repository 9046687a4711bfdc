// 3D-RoPE of a chunk and the RoPE-fused KV append (gfx950).
//
// Both kernels are HBM-bound streams over 16-byte vectors (8 bf16 = 4
// rotation pairs of one (token, head) row).  Each thread owns the same
// 16-byte slot of one token in kHeads heads and issues all of its loads
// before any arithmetic.  Results are written with the non-temporal hint
// (streamed out instead of being kept in the caches: measurably faster).
//
// Rotation, exactly: a bf16 value times an fp32 table entry is exact in fp64,
// so y0 = x0*c - x1*s and y1 = x0*s + x1*c are each rounded once to fp64 (one
// exact product plus one FMA), then once more, to nearest-even, to bf16 (the
// hardware fp32 -> bf16 pack, with a rare-case fix for double rounding).  NaN
// becomes the canonical quiet NaN 0x7FC0.
//
// Append (FlashDreams blog post, "Hot-Path Generation, Background State
// Updates": the KV update is the finalize() half of a step): K of each stored
// frame is rotated at the frame's absolute t and written, with V, into the
// frame's ring slot; the pool keeps each (slot, kv head) as one contiguous
// Ft x d block so attention reads whole frames with unit stride.
#include "../wm_internal.hpp"

namespace wm {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kHeads = kRopeHeads;  // heads per thread

__device__ __forceinline__ uint32_t fast_div(uint32_t n, FastDiv d) {
  return (__umulhi(n, d.mul) + n) >> d.shift;
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const bf16x2 v = {(__bf16)a, (__bf16)b};  // nearest-even
  return __builtin_bit_cast(uint32_t, v);
}

// Nearest-even bf16 of fp64 values, exactly.  Rounding first to fp32
// (nearest-even) and then to bf16 gives the same result unless the fp32 value
// lands exactly on a midpoint between two bf16 neighbours while the fp64 value
// does not (double rounding).  Such vectors, and NaN, are rare: the fast pass
// only detects them (midpoint: low 16 bits of the fp32 value are 0x8000; NaN:
// magnitude bits above those of infinity) and a second pass recomputes the
// vector with the fix (the fp32 value moves one fp32 unit toward the fp64
// value, off the midpoint to the correct side; NaN becomes 0x7FC0).
struct FixDetect {
  uint32_t mid = 1u;  // 0 once a midpoint was seen
  uint32_t mag = 0u;  // largest |fp32 bits| seen
  __device__ __forceinline__ void add(float f) {
    const uint32_t b = __float_as_uint(f);
    mid = min(mid, (b & 0xFFFFu) ^ 0x8000u);
    mag = max(mag, b << 1);
  }
  __device__ __forceinline__ bool needed() const { return mid == 0u || mag > 0xFF000000u; }
};

__device__ __forceinline__ float fix_f32(float f, double y) {
  const uint32_t bits = __float_as_uint(f);
  const double back = (double)f;
  if (y != y) return __uint_as_float(0x7FC00000u);
  if ((bits & 0xFFFFu) != 0x8000u || back == y) return f;
  return __uint_as_float(__builtin_fabs(back) > __builtin_fabs(y) ? bits - 1 : bits + 1);
}

// Rotate the 4 pairs of one 16-byte vector with per-pair (cos, sin).
// kExact: apply the double-rounding fix; otherwise feed the detector.
template <bool kExact>
__device__ __forceinline__ u32x4 rotate_vec(u32x4 x, const double (&c)[4], const double (&s)[4],
                                            FixDetect& det) {
  u32x4 o;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const double x0 = (double)__uint_as_float(x[k] << 16);
    const double x1 = (double)__uint_as_float(x[k] & 0xFFFF0000u);
    const double y0 = __builtin_fma(x0, c[k], -(x1 * s[k]));
    const double y1 = __builtin_fma(x0, s[k], x1 * c[k]);
    float f0 = (float)y0, f1 = (float)y1;
    if constexpr (kExact) {
      f0 = fix_f32(f0, y0);
      f1 = fix_f32(f1, y1);
    } else {
      // Opaque: stops the compiler from fusing the two conversions into its
      // own (exact but much longer) fp64 -> bf16 sequence.
      asm("" : "+v"(f0), "+v"(f1));
      det.add(f0);
      det.add(f1);
    }
    o[k] = pack_bf16(f0, f1);
  }
  return o;
}

// (cos, sin) of pair pr at the token (hpos, wpos): the t band from the row's
// kernel-argument values, the h and w bands from the pool table.  Both
// entries are loaded unconditionally (t pairs read pool entry 0, h/w pairs
// t entry 0) and blended as c = e_hw * keep + e_t with keep = 0, e_t = the t
// value for t pairs (e_hw is finite and the t rows hold no -0, so this is
// exactly the t value) and keep = 1, e_t = -0 for h/w pairs (exactly e_hw).
// No branch, so no wait on the earlier loads sits between the lookups.
__device__ __forceinline__ void pair_entry(const RopeParams& p, int row, int pr, uint32_t hpos,
                                           uint32_t wpos, double& c, double& s) {
  const bool in_t = pr < p.dt2;
  const bool in_h = pr < p.dt2 + p.dh2;
  const uint32_t e = in_t ? 0u
                          : (in_h ? hpos * p.dh2 + (pr - p.dt2)
                                  : p.w_base + wpos * p.dw2 + (pr - p.dt2 - p.dh2));
  const float2 t = p.tcs[row][in_t ? pr : 0];
  const double2 hw = p.hw[e];
  const double keep = in_t ? 0.0 : 1.0;
  c = __builtin_fma(hw.x, keep, in_t ? (double)t.x : -0.0);
  s = __builtin_fma(hw.y, keep, in_t ? (double)t.y : -0.0);
}

// grid: x = ceil(ft / tokens per block), y = row of p.rows,
//       z = head group (rope: those of x, then those of x2 when paired) or
//           2 * (layer * head groups + head group) + part
//       (append: part 0 rotates K, part 1 copies V -- separate waves, so the V
//       stream runs while K waves compute; all layers of a multi-layer ring in
//       one launch, each with its own input and pool slices).
// Thread = (token, 16-byte slot c8 of the head dim); it handles kHeads heads of
// that token, so its four pairs' table entries and its token's position are
// looked up once.  A wave covers 64 / (d/8) consecutive tokens: each head's
// rows are 256-byte (d = 128) runs in the chunk tensor and, in the pool
// ([head][token][d]), one contiguous run.
template <bool kAppend, int kLgCpr>
__global__ __launch_bounds__(kThreads) void rope_rows_kernel(const RopeParams p) {
  constexpr int kCpr = 1 << kLgCpr;  // 16-byte vectors per (token, head)
  constexpr int kTpb = kThreads / kCpr;
  const int row = blockIdx.y;
  const uint32_t c8 = threadIdx.x & (kCpr - 1);
  const uint32_t tok = blockIdx.x * kTpb + (threadIdx.x >> kLgCpr);
  if (tok >= (uint32_t)p.ft) return;
  int hgroup = kAppend ? (int)(blockIdx.z >> 1) : (int)blockIdx.z;
  const bool v_part = kAppend && (blockIdx.z & 1);
  // Paired rope: the second tensor (its own heads and stride, the same rows).
  const bool second = !kAppend && hgroup >= p.hg_first;
  const int n_heads = second ? p.n_heads2 : p.n_heads;
  const uint16_t* const xin = second ? p.x2 : p.x;
  const int64_t x_b_stride = second ? p.x2_b_stride : p.x_b_stride;
  if (second) hgroup -= p.hg_first;
  int64_t x_layer = 0, pool_layer = 0;
  if constexpr (kAppend) {
    const int n_hg = (n_heads + kHeads - 1) / kHeads;
    const int layer = hgroup / n_hg;
    hgroup -= layer * n_hg;
    x_layer = (int64_t)layer * p.x_layer_stride;
    pool_layer = (int64_t)layer * p.pool_layer_stride;
  }
  const int h0 = hgroup * kHeads;
  const int nh = min(kHeads, n_heads - h0);
  const int rb = p.rows[row].b;
  const int rj = p.rows[row].j;
  const uint32_t head_bytes = (uint32_t)kCpr * 16u;

  // A rollout's chunk tensor holds below 2^31 elements (checked at ring
  // creation), so byte offsets within a frame fit 32 bits.
  // Heads past the last are clamped on load; their stores are skipped.
  const int64_t row_base = x_layer + (int64_t)rb * x_b_stride + (int64_t)rj * p.ft * n_heads * (kCpr * 8);
  const uint32_t src_off = ((tok * (uint32_t)n_heads + h0) * kCpr + c8) * 16u;

  // Destinations: the chunk layout (rope) or the slot's [head][token][d] block.
  char* out;
  uint32_t dst_off, dst_head;
  if constexpr (kAppend) {
    const int64_t slot_base =
        pool_layer + ((int64_t)rb * p.ring_slots + p.rows[row].slot) * n_heads * p.ft * (kCpr * 8);
    out = reinterpret_cast<char*>((v_part ? p.vdst : p.y) + slot_base);
    dst_head = (uint32_t)p.ft * head_bytes;
    dst_off = (uint32_t)h0 * dst_head + (tok * kCpr + c8) * 16u;
  } else {
    out = reinterpret_cast<char*>((second ? p.y2 : p.y) + row_base);
    dst_head = head_bytes;
    dst_off = src_off;
  }

  if (v_part) {  // V: a plain copy into the slot
    const char* vs = reinterpret_cast<const char*>(p.vsrc + row_base) + src_off;
    u32x4 vx[kHeads];
#pragma unroll
    for (int g = 0; g < kHeads; ++g)
      vx[g] = *reinterpret_cast<const u32x4*>(vs + (uint32_t)(g < nh ? g : nh - 1) * head_bytes);
#pragma unroll
    for (int g = 0; g < kHeads; ++g)
      if (g < nh) __builtin_nontemporal_store(vx[g], reinterpret_cast<u32x4*>(out + dst_off + g * dst_head));
    return;
  }

  // Table entries first (L2 hits), then the K loads (HBM).  Token index
  // within the frame = view * (fh * fw) + h * fw + w.
  const uint32_t rows = fast_div(tok, p.div_fw);
  const uint32_t wpos = tok - rows * p.fw;
  const uint32_t hpos = rows - fast_div(rows, p.div_fh) * p.fh;
  double c[4], s[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) pair_entry(p, row, (int)c8 * 4 + k, hpos, wpos, c[k], s[k]);

  const char* xs = reinterpret_cast<const char*>(xin + row_base) + src_off;
  u32x4 kx[kHeads];
#pragma unroll
  for (int g = 0; g < kHeads; ++g)
    kx[g] = *reinterpret_cast<const u32x4*>(xs + (uint32_t)(g < nh ? g : nh - 1) * head_bytes);

  uint32_t fix_mask = 0;
#pragma unroll
  for (int g = 0; g < kHeads; ++g) {
    FixDetect det;
    const u32x4 o = rotate_vec<false>(kx[g], c, s, det);
    if (g >= nh) continue;
    fix_mask |= (uint32_t)det.needed() << g;
    __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(out + dst_off + g * dst_head));
  }

  // Rare second pass: exact recomputation of flagged vectors (same thread,
  // same address, so it simply overwrites the first result).
  if (__builtin_expect(fix_mask != 0, 0)) {
#pragma unroll
    for (int g = 0; g < kHeads; ++g) {
      if (!(fix_mask >> g & 1u)) continue;
      u32x4 x = kx[g];
      asm volatile("" : "+v"(x));  // keeps this pass from being folded into the first
      FixDetect unused;
      *reinterpret_cast<u32x4*>(out + dst_off + g * dst_head) = rotate_vec<true>(x, c, s, unused);
    }
  }
}

template <bool kAppend>
LaunchSpec rows_spec(const RopeParams& p) {
  const int lg = p.lg_cpr;
  const uint32_t tpb = kThreads >> lg;
  LaunchSpec sp;
  const int hg = (p.n_heads + kHeads - 1) / kHeads;
  const int hg2 = !kAppend && p.x2 ? (p.n_heads2 + kHeads - 1) / kHeads : 0;
  sp.grid = dim3((p.ft + tpb - 1) / tpb, p.n_rows, kAppend ? 2 * p.n_layers * hg : hg + hg2);
  sp.block = dim3(kThreads);
  sp.func = lg == 4 ? reinterpret_cast<const void*>(&rope_rows_kernel<kAppend, 4>)
                    : reinterpret_cast<const void*>(&rope_rows_kernel<kAppend, 3>);
  return sp;
}

}  // namespace

LaunchSpec rope3d_spec(const RopeParams& p) { return rows_spec<false>(p); }

LaunchSpec kv_append_spec(const RopeParams& p) { return rows_spec<true>(p); }

}  // namespace wm
