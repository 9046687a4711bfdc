// Block-causal chunk attention over a bounded KV ring (gfx950, bf16 MFMA).
//
// What it computes (Cosmos3-H-Dreams model card, "Model Architecture":
// block-causal student with a KV cache; AlpaDreams GTC write-up, section VII:
// next frame from historical clean frames + the current noisy frame): for
// each query of the current chunk, softmax attention over the keys of the
// frames the rollout holds (sinks + window, from the ring pool) and of every
// frame of the chunk itself.  The visible ring slots of a rollout that has
// committed m frames are exactly slots 0 .. min(m, S+W)-1, so the key list is
// two segments: ring frames (unit row stride inside a slot) and the chunk
// (row stride Hkv*d).  Softmax is order-invariant, so keys are visited in
// slot order, never concatenated.
//
// Design (one workgroup = 4 waves = 4 "wave tasks" that share one kv head):
//  * a wave task is 64 queries of one q head: two 32-query blocks;
//  * keys stream through LDS in 64-key tiles (K double-, V triple-buffered,
//    one barrier per tile); tile loads are issued two tiles ahead and are
//    branch-free: keys past the end are clamped to the last key and masked
//    out of the softmax;
//  * S^T = K * Q^T on v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = Q^T
//    held in registers for the whole kernel): in the 32x32 accumulator
//    layout each lane owns one query column and 16 keys, so the row max and
//    row sum need one cross-half exchange (v_permlane32_swap), no tree;
//  * O^T += V^T * P^T on the same MFMA: P^T comes straight from the S^T
//    accumulator (exp2, cvt_pk_bf16).  V stays in its natural [key][d] layout
//    in LDS and the V^T operand is read with ds_read_b64_tr_b16: in each
//    16-lane group, lane j receives element j%4 of the 8-byte chunks read by
//    lanes j/4, j/4+4, j/4+8, j/4+12, so when lane L reads row kbase + L/4 at
//    column dbase + 4*(L%4), lane j gets V[kbase .. kbase+3][dbase + j] --
//    four consecutive keys of one d, exactly the keys the S^T accumulator
//    layout gives that lane's P;
//  * LDS row pitches: K rows 272 B (8 consecutive rows of a 16-byte column
//    hit disjoint banks), V rows 288 B (the 4 rows x 32 B of a transposed
//    read hit disjoint banks);
//  * the two 32-query blocks of a wave are staggered so that the matrix
//    cores compute one block's S while the vector ALUs form the other
//    block's P (phase list at the main loop);
//  * online softmax in the log2 domain with a lazy rescale: the running max
//    only moves (and O, l are rescaled) when a row's new max exceeds it by
//    more than 8 (P stays <= 2^8); a wave-uniform branch, rarely taken;
//  * GQA: the 4 wave tasks of a workgroup are (q block, head-in-group) pairs
//    of one kv head, so a K/V tile in LDS serves every q head of the group.
// This file is compiled with -fno-honor-nans (max without NaN quieting):
// the softmax never produces NaN from finite inputs; -inf is still honoured.
#include "../wm_internal.hpp"

namespace wm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) uint16_t lds_u16;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kKT = 64;                // keys per tile
constexpr int kXcds = 8;               // MI355X: 8 accelerator complex dies
constexpr float kRescaleSlack = 8.0f;  // log2 units

template <int HD>
struct Cfg {
  static constexpr int KP = HD + 8;     // K row pitch (elements)
  static constexpr int VP = HD + 16;    // V row pitch (elements)
  static constexpr int NDC = HD / 16;   // 16-wide d chunks (QK^T contraction)
  static constexpr int NDB = HD / 32;   // 32-row d blocks (PV output)
  static constexpr int CPR = HD / 8;    // 16-byte vectors per row
  static constexpr int K_ELEMS = kKT * KP;
  static constexpr int V_ELEMS = kKT * VP;
  static constexpr int LDS_ELEMS = 2 * K_ELEMS + 3 * V_ELEMS;
};

__device__ __forceinline__ float xhalf_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float xhalf_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Register-class pins (empty asm, no side effects): MFMA-only data (O, Q) in
// AGPRs, data the vector ALUs touch (S) in VGPRs, so the allocator never
// shuttles them across the rare rescale branch.
template <typename T>
__device__ __forceinline__ void pin_agpr(T& x) {
  asm("" : "+a"(x));
}
template <typename T>
__device__ __forceinline__ void pin_vgpr(T& x) {
  asm("" : "+v"(x));
}

// Row max of one 32-query block over a 64-key tile (both 32-key halves).
__device__ __forceinline__ float tile_rowmax(const f32x16& a, const f32x16& b) {
  float m0 = fmaxf(a[0], fmaxf(a[1], a[2]));
  float m1 = fmaxf(b[0], fmaxf(b[1], b[2]));
#pragma unroll
  for (int i = 3; i < 15; i += 2) {
    m0 = fmaxf(m0, fmaxf(a[i], a[i + 1]));
    m1 = fmaxf(m1, fmaxf(b[i], b[i + 1]));
  }
  return xhalf_max(fmaxf(m0, fmaxf(a[15], fmaxf(m1, b[15]))));
}

template <int HD, bool kSmallFt>
__global__ __launch_bounds__(kThreads, 1) void chunk_attn_kernel(const AttnParams p) {
  using C = Cfg<HD>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[C::LDS_ELEMS];
  lds_u16* const kbuf0 = (lds_u16*)smem;
  lds_u16* const vbuf0 = kbuf0 + 2 * C::K_ELEMS;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // ---- which (rollout, kv head, workgroup, split) -------------------------
  // Workgroups are dispatched round-robin over the 8 XCDs; remap so that each
  // XCD gets a contiguous run of logical workgroups -- the q blocks of one kv
  // head then stream the same K/V tiles through that XCD's L2.
  int bid = (int)(blockIdx.x % kXcds) * p.per_xcd + (int)(blockIdx.x / kXcds);
  if (bid >= p.n_wg) return;
  const int split = bid % p.nsplit;
  bid /= p.nsplit;
  const int wgi = bid % p.wg_per_bg;
  bid /= p.wg_per_bg;
  const int g = bid % p.hkv;
  const int bi = bid / p.hkv;
  const int b = p.b_index[bi];
  const int ring_keys = p.n_ring[bi] * p.ft;
  const int nk = ring_keys + p.nq;
  const int ntiles = (nk + kKT - 1) / kKT;
  const int tps = (ntiles + p.nsplit - 1) / p.nsplit;
  const int t_begin = split * tps;
  const int n_local = min(ntiles, t_begin + tps) - t_begin;  // >= 1 by construction

  const int task = wgi * kWaves + wave;
  const bool has_task = task < p.group * p.nqb;
  const int qblk = has_task ? task / p.group : 0;
  const int h = g * p.group + (has_task ? task % p.group : 0);
  const int q0 = qblk * 64;

  // ---- Q^T operands: lane (l32, hi) holds query q0+qb*32+l32, d = dc*16+hi*8.. --
  bf16x8 qreg[2][C::NDC];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int q = min(q0 + qb * 32 + l32, p.nq - 1);
    const uint16_t* src = p.q + (((int64_t)b * p.nq + q) * p.hq + h) * HD + hi * 8;
#pragma unroll
    for (int dc = 0; dc < C::NDC; ++dc) {
      qreg[qb][dc] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(src + dc * 16));
      pin_agpr(qreg[qb][dc]);
    }
  }

  // ---- loader role: 4 consecutive keys x one 16-byte column chunk ----------
  const int lkg = tid >> 4;  // key group 0..15 -> keys 4*lkg .. 4*lkg+3
  const int lc = (tid & 15) % C::CPR;
  const bool loader = (tid & 15) < C::CPR;
  const int ft = p.ft;
  const float inv_ft = 1.0f / (float)ft;
  const uint16_t* const ring_k = p.pk + ((int64_t)b * p.ring_slots * p.hkv + g) * (int64_t)ft * HD + lc * 8;
  const uint16_t* const ring_v = p.pv + ((int64_t)b * p.ring_slots * p.hkv + g) * (int64_t)ft * HD + lc * 8;
  const uint32_t slot_stride = (uint32_t)p.hkv * ft * HD;  // elements; < 2^31 per rollout
  const uint16_t* const chunk_k = p.kc + ((int64_t)b * p.nq * p.hkv + g) * HD + lc * 8;
  const uint16_t* const chunk_v = p.vc + ((int64_t)b * p.nq * p.hkv + g) * HD + lc * 8;
  const uint32_t chunk_stride = (uint32_t)p.hkv * HD;

  u32x4 kreg[4], vreg[4];
  // Issue the loads of local tile u (keys clamped into range: always valid).
  auto load_tile = [&](int u) {
    const int j0 = (t_begin + u) * kKT + lkg * 4;
    int s0 = (int)((float)j0 * inv_ft);
    int r0 = j0 - s0 * ft;
    s0 += (r0 >= ft) - (r0 < 0);
    r0 = j0 - s0 * ft;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int j = min(j0 + i, nk - 1);
      int si, ri;
      if constexpr (kSmallFt) {
        si = (int)((float)j * inv_ft);
        ri = j - si * ft;
        si += (ri >= ft) - (ri < 0);
        ri = j - si * ft;
      } else {
        // ft >= 4: at most one frame boundary inside the 4 keys
        ri = r0 + i;
        si = s0;
        if (ri >= ft) {
          ri -= ft;
          ++si;
        }
      }
      const bool in_ring = j < ring_keys;
      const uint32_t ro = (uint32_t)si * slot_stride + (uint32_t)ri * HD;
      const uint32_t co = (uint32_t)(j - ring_keys) * chunk_stride;
      const uint16_t* kp = in_ring ? ring_k + ro : chunk_k + co;
      const uint16_t* vp = in_ring ? ring_v + ro : chunk_v + co;
      kreg[i] = *reinterpret_cast<const u32x4*>(kp);
      vreg[i] = *reinterpret_cast<const u32x4*>(vp);
    }
  };
  auto store_tile = [&](lds_u16* ks, lds_u16* vs) {
    if (!loader) return;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *(lds_u32x4*)(ks + (lkg * 4 + i) * C::KP + lc * 8) = kreg[i];
      *(lds_u32x4*)(vs + (lkg * 4 + i) * C::VP + lc * 8) = vreg[i];
    }
  };

  // ---- running state ------------------------------------------------------
  f32x16 oacc[C::NDB][2];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[db][qb][i] = 0.f;
  float m_run[2] = {-INFINITY, -INFINITY};  // running max (scaled, log2 domain)
  float l_run[2] = {0.f, 0.f};              // running sum over this lane's keys
  const float sl2 = p.scale_log2e;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  // Transposed-read role: the lane's row and column inside its 16-lane group.
  const int tr_l = lane & 15;
  const int tr_off = (hi * 4 + (tr_l >> 2)) * C::VP + ((lane >> 4) & 1) * 16 + 4 * (tr_l & 3);
  const uint32_t tr_base = (uint32_t)(uintptr_t)(vbuf0 + tr_off);

  // S^T of one 32-query block: S[kb], keys kb*32.., 16 fp32 per lane each.
  auto qk = [&](const lds_u16* ks, int qb, f32x16 (&S)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const bf16x8 kf = *(const lds_bf16x8*)(ks + (kb * 32 + l32) * C::KP + hi * 8);
      S[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qreg[qb][0], (f32x16){}, 0, 0, 0);
    }
#pragma unroll
    for (int dc = 1; dc < C::NDC; ++dc) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 kf = *(const lds_bf16x8*)(ks + (kb * 32 + l32) * C::KP + dc * 16 + hi * 8);
        S[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qreg[qb][dc], S[kb], 0, 0, 0);
      }
    }
    // pin_vgpr(S[0]);
    // pin_vgpr(S[1]);
  };
  // O^T[qb] += V^T P^T of one 32-query block; V^T fragments via transposed reads.
  // MFMA kc covers keys kc*16..: lane half hi takes keys +4*hi+{0..3} and +8+4*hi+{0..3}.
  // trv is the 32-bit LDS byte address of this lane's first read in the tile;
  // every other read is a compile-time byte offset from it.
  auto pv = [&](uint32_t trv, int qb, const bf16x8 (&P)[4]) {
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        const uint32_t a = trv + 2 * ((kc * 16) * C::VP + db * 32);
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)a);
        const s16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)(a + 2 * 8 * C::VP));
        const s16x8 v8 = {lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2], up[3]};
        oacc[db][qb] =
            __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, v8), P[kc], oacc[db][qb], 0, 0, 0);
      }
    }
  };
  // P^T fragments of one 32-key half of S: exp2(s*scale*log2e - m) in bf16, row sum.
  auto softmax_half = [&](const f32x16& S, int qb, bf16x8& Pa, bf16x8& Pb) {
    const float mneg = -m_run[qb];
    uint32_t pk[8];
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
      const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[i], sl2, mneg));
      const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[i + 1], sl2, mneg));
      const bf16x2 pr = {(__bf16)e0, (__bf16)e1};
      l_run[qb] = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, l_run[qb], false);
      pk[i >> 1] = __builtin_bit_cast(uint32_t, pr);
    }
    Pa = __builtin_bit_cast(bf16x8, make_uint4(pk[0], pk[1], pk[2], pk[3]));
    Pb = __builtin_bit_cast(bf16x8, make_uint4(pk[4], pk[5], pk[6], pk[7]));
  };
  // Mask keys >= nvalid of a tile (only the last tile of the key range).
  auto mask_tail = [&](f32x16 (&S)[2], int nvalid) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = kb * 32 + (i >> 2) * 8 + hi * 4 + (i & 3);
        if (key >= nvalid) S[kb][i] = -INFINITY;
      }
  };
  // Lazy rescale of one query block (wave-uniform branch).
  auto maybe_rescale = [&](int qb, float mxraw) {
    const bool need = mxraw * sl2 > m_run[qb] + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float m_new = fmaxf(m_run[qb], mxraw * sl2);
      const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - m_new);
      m_run[qb] = m_new;
      l_run[qb] *= alpha;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][qb][i] *= alpha;
        pin_agpr(oacc[db][qb]);
      }
    }
  };

  const int nk_last = nk - (t_begin + n_local - 1) * kKT;  // valid keys in the last local tile
  f32x16 S0[2], S1[2];
  bf16x8 P0[4], P1[4];

  // Prologue: K,V of tiles 0 and 1 in LDS; S of tile 0, block 0, and its row max.
  load_tile(0);
  store_tile(kbuf0, vbuf0);
  load_tile(1);
  store_tile(kbuf0 + C::K_ELEMS, vbuf0 + C::V_ELEMS);
  __syncthreads();
  qk(kbuf0, 0, S0);
  float mx0 = tile_rowmax(S0[0], S0[1]);

  // Per tile u (S0 = S(u, block 0) and its row max ready on entry):
  //   A: S(u, block 1) on the matrix cores  || P(u, block 0) on the vector ALUs
  //   B: O0 += V(u) P(u, block 0)             || first half of P(u, block 1)
  //   C: S(u+1, block 0)                      || second half of P(u, block 1)
  //   D: O1 += V(u) P(u, block 1)             || row max of S(u+1, block 0), LDS stores
  // K is double-buffered (tile u+1 is read in C), V triple-buffered; the loads
  // of tile u+2 are issued in A and land in LDS at the end of D.
  for (int u = 0; u < n_local; ++u) {
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
      pin_agpr(oacc[db][0]);
      pin_agpr(oacc[db][1]);
    }
    const lds_u16* kcur = kbuf0 + (u & 1) * C::K_ELEMS;
    const lds_u16* knext = kbuf0 + ((u + 1) & 1) * C::K_ELEMS;
    uint32_t trv = tr_base + (uint32_t)((u % 3) * C::V_ELEMS * 2);
    pin_vgpr(trv);  // opaque per-tile base: keeps base+const from being hoisted per read
    const bool tail = u == n_local - 1 && nk_last < kKT;
    if (tail) {
      mask_tail(S0, nk_last);
      mx0 = tile_rowmax(S0[0], S0[1]);
    }
    maybe_rescale(0, mx0);
    // A
    load_tile(u + 2);
    qk(kcur, 1, S1);
    softmax_half(S0[0], 0, P0[0], P0[1]);
    softmax_half(S0[1], 0, P0[2], P0[3]);
    if (tail) mask_tail(S1, nk_last);
    maybe_rescale(1, tile_rowmax(S1[0], S1[1]));
    // B
    pv(trv, 0, P0);
    softmax_half(S1[0], 1, P1[0], P1[1]);
    // C
    qk(knext, 0, S0);
    softmax_half(S1[1], 1, P1[2], P1[3]);
    // D
    pv(trv, 1, P1);
    mx0 = tile_rowmax(S0[0], S0[1]);
    store_tile(kbuf0 + (u & 1) * C::K_ELEMS, vbuf0 + ((u + 2) % 3) * C::V_ELEMS);
    __syncthreads();
  }

  if (!has_task) return;

  // ---- epilogue -------------------------------------------------------------
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int q = q0 + qb * 32 + l32;
    const float l_tot = xhalf_sum(l_run[qb]);
    if (q >= p.nq) continue;
    if (p.nsplit == 1) {
      const float inv = 1.0f / l_tot;
      uint16_t* dst = p.out + (((int64_t)b * p.nq + q) * p.hq + h) * HD;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int d = db * 32 + ii * 8 + hi * 4;
          const uint2 v = make_uint2(pack_bf16(oacc[db][qb][ii * 4 + 0] * inv, oacc[db][qb][ii * 4 + 1] * inv),
                                     pack_bf16(oacc[db][qb][ii * 4 + 2] * inv, oacc[db][qb][ii * 4 + 3] * inv));
          *reinterpret_cast<uint2*>(dst + d) = v;
        }
    } else {
      // Partial result of this key range: O / l (fp32) plus (max, sum).
      const int64_t row = (((int64_t)split * p.nb + bi) * p.nq + q) * p.hq + h;
      float* dst = p.part_o + row * HD;
      const float inv = 1.0f / l_tot;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const int d = db * 32 + ii * 8 + hi * 4;
          *reinterpret_cast<float4*>(dst + d) =
              make_float4(oacc[db][qb][ii * 4 + 0] * inv, oacc[db][qb][ii * 4 + 1] * inv,
                          oacc[db][qb][ii * 4 + 2] * inv, oacc[db][qb][ii * 4 + 3] * inv);
        }
      if (hi == 0) {
        p.part_ml[row * 2 + 0] = m_run[qb];
        p.part_ml[row * 2 + 1] = l_tot;
      }
    }
  }
}

}  // namespace

hipError_t launch_chunk_attn(const AttnParams& p_in, int head_dim, hipStream_t s) {
  AttnParams p = p_in;
  p.n_wg = p.nb * p.hkv * p.wg_per_bg * p.nsplit;
  p.per_xcd = (p.n_wg + kXcds - 1) / kXcds;
  const dim3 grid(p.per_xcd * kXcds);
  const bool small = p.ft < 4;
  if (head_dim == 128) {
    if (small)
      hipLaunchKernelGGL((chunk_attn_kernel<128, true>), grid, dim3(kThreads), 0, s, p);
    else
      hipLaunchKernelGGL((chunk_attn_kernel<128, false>), grid, dim3(kThreads), 0, s, p);
  } else {
    if (small)
      hipLaunchKernelGGL((chunk_attn_kernel<64, true>), grid, dim3(kThreads), 0, s, p);
    else
      hipLaunchKernelGGL((chunk_attn_kernel<64, false>), grid, dim3(kThreads), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace wm
