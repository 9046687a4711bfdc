// 3D-RoPE of a chunk and the RoPE-fused KV append (gfx950).
//
// Both kernels are HBM-bound streams: each thread moves one 16-byte vector
// (8 bf16 = 4 rotation pairs) of a (token, head) row.  The rotation follows
// the exact-product rule: a bf16 value times an fp32 table entry is exact in
// fp64, so y0 = x0*c - x1*s and y1 = x0*s + x1*c are each rounded once (fp64
// add/sub; contraction into an FMA gives the same bits), then rounded once
// more, to nearest-even, straight from fp64 to bf16.
//
// Append (FlashDreams blog post, "Hot-Path Generation, Background State
// Updates": the KV update is the finalize() half of a step): K of each stored
// frame is rotated at the frame's absolute t and written, with V, into the
// frame's ring slot; the pool keeps each (slot, kv head) as one contiguous
// Ft x d block so attention reads whole frames with unit stride.
#include "../wm_internal.hpp"

namespace wm {
namespace {

__device__ __forceinline__ double bf16_to_f64(uint32_t bits16) {
  return (double)__uint_as_float(bits16 << 16);
}

// Round-to-nearest-even from fp64 to bf16.
__device__ __forceinline__ uint32_t f64_to_bf16(double y) {
  const uint64_t u = (uint64_t)__double_as_longlong(y);
  const uint32_t sign = (uint32_t)(u >> 48) & 0x8000u;
  uint64_t a = u & 0x7FFFFFFFFFFFFFFFull;
  if (a >= 0x7FF0000000000000ull) return a == 0x7FF0000000000000ull ? (sign | 0x7F80u) : 0x7FC0u;
  const int e = (int)(a >> 52) - 1023;
  if (e < -126) {
    // bf16 subnormal range: quantum 2^-133; the power-of-two scaling is exact.
    const double n = __builtin_rint(__builtin_fabs(y) * 0x1p133);
    return sign | (uint32_t)n;
  }
  a += 0x00000FFFFFFFFFFFull + ((a >> 45) & 1u);  // keep 7 of 52 fraction bits, ties to even
  const uint64_t r = a >> 45;                      // 11 exponent bits | 7 fraction bits
  const int eb = (int)(r >> 7) - 1023 + 127;
  if (eb >= 255) return sign | 0x7F80u;
  return sign | ((uint32_t)eb << 7) | (uint32_t)(r & 0x7Fu);
}

// Rotate the 4 pairs held in one 16-byte vector; `pair0` is the index of the
// first pair within the head dim.
__device__ __forceinline__ uint4 rotate_vec(uint4 x, int pair0, const RopeParams& p, int row,
                                            int hpos, int wpos) {
  uint32_t w[4] = {x.x, x.y, x.z, x.w};
  uint32_t o[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int pr = pair0 + k;
    float c, s;
    if (pr < p.dt2) {
      c = p.tcos[row][pr];
      s = p.tsin[row][pr];
    } else if (pr < p.dt2 + p.dh2) {
      const int j = pr - p.dt2;
      c = p.hcos[hpos * p.dh2 + j];
      s = p.hsin[hpos * p.dh2 + j];
    } else {
      const int j = pr - p.dt2 - p.dh2;
      c = p.wcos[wpos * p.dw2 + j];
      s = p.wsin[wpos * p.dw2 + j];
    }
    const double x0 = bf16_to_f64(w[k] & 0xFFFFu);
    const double x1 = bf16_to_f64(w[k] >> 16);
    const double cd = (double)c, sd = (double)s;
    const double y0 = x0 * cd - x1 * sd;
    const double y1 = x0 * sd + x1 * cd;
    o[k] = f64_to_bf16(y0) | (f64_to_bf16(y1) << 16);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

constexpr int kThreads = 256;

// grid: x = vectors of one (rollout, frame) row / 256, y = row of p.rows
template <bool kAppend>
__global__ __launch_bounds__(kThreads) void rope_rows_kernel(const RopeParams p) {
  const int row = blockIdx.y;
  const int rb = p.rows[row].b;
  const int rj = p.rows[row].j;
  const int cpr = p.d >> 3;  // 16-byte vectors per (token, head)
  const uint32_t nvec = (uint32_t)p.ft * p.n_heads * cpr;
  const uint32_t i = blockIdx.x * kThreads + threadIdx.x;
  if (i >= nvec) return;
  const uint32_t c8 = i & (cpr - 1);
  const uint32_t th = i / cpr;
  const uint32_t head = th % p.n_heads;
  const uint32_t tok = th / p.n_heads;
  const uint32_t hpos = tok / p.fw;
  const uint32_t wpos = tok - hpos * p.fw;
  const int64_t src = (int64_t)rb * p.x_b_stride +
                      ((int64_t)(rj * p.ft + tok) * p.n_heads + head) * p.d + c8 * 8;
  const uint4 xv = *reinterpret_cast<const uint4*>(p.x + src);
  const uint4 yv = rotate_vec(xv, c8 * 4, p, row, hpos, wpos);
  if constexpr (!kAppend) {
    *reinterpret_cast<uint4*>(p.y + src) = yv;
  } else {
    const int slot = p.rows[row].slot;
    const int64_t dst =
        ((((int64_t)rb * p.ring_slots + slot) * p.n_heads + head) * p.ft + tok) * p.d + c8 * 8;
    const uint4 vv = *reinterpret_cast<const uint4*>(p.vsrc + src);
    *reinterpret_cast<uint4*>(p.y + dst) = yv;
    *reinterpret_cast<uint4*>(p.vdst + dst) = vv;
  }
}

dim3 rows_grid(const RopeParams& p) {
  const uint32_t nvec = (uint32_t)p.ft * p.n_heads * (p.d >> 3);
  return dim3((nvec + kThreads - 1) / kThreads, p.n_rows, 1);
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
