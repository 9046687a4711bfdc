// 3D-RoPE of a chunk and the RoPE-fused KV append (gfx950).
//
// Both kernels are HBM-bound streams over 16-byte vectors (8 bf16 = 4
// rotation pairs of one (token, head) row).  Each thread owns kVecs vectors,
// 256 vectors apart, and issues all of its loads before any arithmetic, so a
// wave keeps 4 (rope) or 8 (append) 16-byte loads in flight.
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
constexpr int kVecs = 4;  // 16-byte vectors per thread

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

// Per-thread constants of its four pairs.  A pair's band is fixed by its index
// within the head dim, which is the same for all of a thread's vectors (they
// are 256 apart), so the t-band entries are loaded once.  Every pair reads one
// pool-table entry (byte offset sel(pair) + off(pair) with sel the token's h or
// w row); t-band pairs read a valid but unused entry and blend it out with
// c = e*0 + c_t (e finite, and the t rows hold no -0, so this is exactly c_t),
// h/w pairs with c = e*1 + (-0) (exactly e).  The blend keeps the table loads
// unconditional (no branch per pair).
struct PairBands {
  bool in_h[4];
  uint32_t off16[4];    // byte offset of the pair's entry within its row
  double keep[4];       // 1 for h/w pairs, 0 for t pairs
  double tc[4], ts[4];  // t-band (cos, sin), or -0 for h/w pairs
};

__device__ __forceinline__ void pair_tables(const RopeParams& p, const PairBands& pb,
                                            uint32_t hrow16, uint32_t wrow16, double (&c)[4],
                                            double (&s)[4]) {
  const char* base = reinterpret_cast<const char*>(p.hw);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t off = (pb.in_h[k] ? hrow16 : wrow16) + pb.off16[k];
    const double2 e = *reinterpret_cast<const double2*>(base + off);
    c[k] = __builtin_fma(e.x, pb.keep[k], pb.tc[k]);
    s[k] = __builtin_fma(e.y, pb.keep[k], pb.ts[k]);
  }
}

// grid: x = ceil(row_vecs / (256 * kVecs)), y = row of p.rows
template <bool kAppend>
__global__ __launch_bounds__(kThreads, 4) void rope_rows_kernel(const RopeParams p) {
  const int row = blockIdx.y;
  const int rb = p.rows[row].b;
  const int rj = p.rows[row].j;
  const uint32_t nvec = (uint32_t)p.row_vecs;
  // A row's vectors are contiguous in the chunk tensor ([token][head][d]);
  // 32-bit byte offsets (a row holds below 2^28 vectors).
  const int64_t row_base = (int64_t)rb * p.x_b_stride + (int64_t)rj * nvec * 8;
  const char* xs = reinterpret_cast<const char*>(p.x + row_base);
  const char* vs = reinterpret_cast<const char*>(p.vsrc + row_base);

  // Loads first (indices clamped into the row; stores are predicated).
  uint32_t vi[kVecs];
  u32x4 kx[kVecs], vx[kVecs];
#pragma unroll
  for (int u = 0; u < kVecs; ++u) {
    vi[u] = (blockIdx.x * kVecs + u) * kThreads + threadIdx.x;
    const uint32_t off = (vi[u] < nvec ? vi[u] : nvec - 1) * 16u;
    kx[u] = *reinterpret_cast<const u32x4*>(xs + off);
    if constexpr (kAppend) vx[u] = *reinterpret_cast<const u32x4*>(vs + off);
  }

  const uint32_t c8 = threadIdx.x & ((1u << p.lg_cpr) - 1);
  const int ht = p.dt2 + p.dh2;
  PairBands pb;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int pr = (int)c8 * 4 + k;
    const bool in_t = pr < p.dt2;
    pb.in_h[k] = pr < ht;
    pb.off16[k] = in_t ? 0u : 16u * (uint32_t)(pr < ht ? pr - p.dt2 : pr - ht);
    pb.keep[k] = in_t ? 0.0 : 1.0;
    const float2 t = p.tcs[row][in_t ? pr : 0];
    pb.tc[k] = in_t ? (double)t.x : -0.0;
    pb.ts[k] = in_t ? (double)t.y : -0.0;
  }

  // Pool destination of a (head, token): per-row slot block + 32-bit offset.
  uint16_t* kdst = nullptr;
  uint16_t* vdst = nullptr;
  if constexpr (kAppend) {
    const int64_t slot_base =
        ((int64_t)rb * p.ring_slots + p.rows[row].slot) * p.n_heads * p.ft * p.d;
    kdst = p.y + slot_base;
    vdst = p.vdst + slot_base;
  }
  const uint32_t head_stride16 = (uint32_t)p.ft * p.d * 2u;

  // Token decomposition of vector vi: table rows and pool offset.
  struct Where {
    uint32_t hrow16, wrow16, dst16;
  };
  auto where = [&](uint32_t v) __attribute__((always_inline)) {
    const uint32_t th = v >> p.lg_cpr;  // token * n_heads + head
    const uint32_t tok = fast_div(th, p.div_heads);
    const uint32_t head = th - tok * p.n_heads;
    const uint32_t hpos = fast_div(tok, p.div_fw);
    const uint32_t wpos = tok - hpos * p.fw;
    Where r;
    r.hrow16 = hpos * (uint32_t)p.dh2 * 16u;
    r.wrow16 = (wpos * (uint32_t)p.dw2 + (uint32_t)p.w_base) * 16u;
    r.dst16 = kAppend ? head * head_stride16 + (tok * (uint32_t)p.d + c8 * 8u) * 2u : v * 16u;
    return r;
  };
  char* kout = kAppend ? reinterpret_cast<char*>(kdst) : reinterpret_cast<char*>(p.y + row_base);

  uint32_t fix_mask = 0;
#pragma unroll
  for (int u = 0; u < kVecs; ++u) {
    const Where at = where(vi[u]);
    double c[4], s[4];
    pair_tables(p, pb, at.hrow16, at.wrow16, c, s);
    FixDetect det;
    const u32x4 o = rotate_vec<false>(kx[u], c, s, det);
    if (vi[u] >= nvec) continue;
    fix_mask |= (uint32_t)det.needed() << u;
    *reinterpret_cast<u32x4*>(kout + at.dst16) = o;
    if constexpr (kAppend) *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(vdst) + at.dst16) = vx[u];
  }

  // Rare second pass: exact recomputation of flagged vectors (same thread,
  // same address, so it simply overwrites the first result).
  if (__builtin_expect(fix_mask != 0, 0)) {
#pragma unroll
    for (int u = 0; u < kVecs; ++u) {
      if (!(fix_mask >> u & 1u)) continue;
      // Opaque copies: keep the compiler from folding this pass into the first.
      u32x4 x = kx[u];
      uint32_t v = vi[u];
      asm volatile("" : "+v"(x), "+v"(v));
      const Where at = where(v);
      double c[4], s[4];
      pair_tables(p, pb, at.hrow16, at.wrow16, c, s);
      FixDetect unused;
      *reinterpret_cast<u32x4*>(kout + at.dst16) = rotate_vec<true>(x, c, s, unused);
    }
  }
}

dim3 rows_grid(const RopeParams& p) {
  const uint32_t per_block = kThreads * kVecs;
  return dim3(((uint32_t)p.row_vecs + per_block - 1) / per_block, p.n_rows, 1);
}

}  // namespace

hipError_t launch_rope3d(const RopeParams& p, hipStream_t s) {
  hipLaunchKernelGGL(rope_rows_kernel<false>, rows_grid(p), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_kv_append(const RopeParams& p, hipStream_t s) {
  hipLaunchKernelGGL(rope_rows_kernel<true>, rows_grid(p), dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace wm
