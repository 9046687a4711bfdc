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
//  * keys stream through LDS in 64-key tiles, double-buffered: while a tile
//    is consumed from LDS the next one is in flight from HBM/L2 in VGPRs;
//  * S^T = K * Q^T on v_mfma_f32_32x32x16_bf16 (A = K from LDS, B = Q^T held
//    in VGPRs for the whole kernel): in the 32x32 accumulator layout each
//    lane owns one query column and 16 keys, so the row max / row sum need
//    one cross-half exchange (v_permlane32_swap) instead of a reduction tree;
//  * O^T += V^T * P^T on the same MFMA: P^T comes straight from the S^T
//    accumulator (exp2, cvt_pk_bf16); V is stored transposed in LDS with the
//    keys permuted so that each lane's 8 keys are one 16-byte LDS read;
//  * online softmax in the log2 domain with fp32 running max and sum;
//  * GQA: the 4 wave tasks of a workgroup are (q block, head-in-group) pairs
//    of one kv head, so a K/V tile in LDS serves every q head of the group.
#include "../wm_internal.hpp"

namespace wm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kKT = 64;   // keys per tile
constexpr int kVP = kKT + 8;  // transposed-V row pitch (elements)

template <int HD>
struct Cfg {
  static constexpr int KP = HD + 8;            // K row pitch in LDS (elements)
  static constexpr int NDC = HD / 16;          // 16-wide d chunks (QK^T contraction)
  static constexpr int NDB = HD / 32;          // 32-row d blocks (PV output)
  static constexpr int CPR = HD / 8;           // 16-byte vectors per row
  static constexpr int K_ELEMS = kKT * KP;
  static constexpr int V_ELEMS = HD * kVP;
  static constexpr int STAGE = K_ELEMS + V_ELEMS;
};

// Position of key o (0..63) of a tile inside a transposed-V row: keys are
// grouped so that the 8 keys a lane feeds to one PV MFMA are contiguous.
__device__ __forceinline__ int vperm(int o) {
  const int kb = o >> 5, r = o & 31;
  return kb * 32 + (r >> 4) * 16 + ((r >> 2) & 1) * 8 + ((r >> 3) & 1) * 4 + (r & 3);
}

__device__ __forceinline__ float xhalf_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float xhalf_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

template <int HD>
__global__ __launch_bounds__(kThreads, 1) void chunk_attn_kernel(const AttnParams p) {
  using C = Cfg<HD>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * C::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // ---- which (rollout, kv head, workgroup, split) -------------------------
  int bid = blockIdx.x;
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
  const int t_end = min(ntiles, t_begin + tps);

  const int task = wgi * kWaves + wave;
  const bool has_task = task < p.group * p.nqb;
  const int qblk = has_task ? task / p.group : 0;
  const int h = g * p.group + (has_task ? task % p.group : 0);
  const int q0 = qblk * 64;

  // ---- Q^T operands: lane (l32, hi) holds query q0+qb*32+l32, d = dc*16+hi*8.. --
  bf16x8 qreg[2][C::NDC];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int q = q0 + qb * 32 + l32;
    const bool ok = has_task && q < p.nq;
    const uint16_t* src = p.q + (((int64_t)b * p.nq + (ok ? q : 0)) * p.hq + h) * HD + hi * 8;
#pragma unroll
    for (int dc = 0; dc < C::NDC; ++dc) {
      uint4 v = ok ? *reinterpret_cast<const uint4*>(src + dc * 16) : make_uint4(0, 0, 0, 0);
      qreg[qb][dc] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // ---- loader role: 4 consecutive keys x one 16-byte column chunk ----------
  const int lkg = tid >> 4;      // key group 0..15 -> keys 4*lkg .. 4*lkg+3
  const int lc = tid & 15;       // column chunk
  const bool loader = lc < C::CPR;
  const float inv_ft = 1.0f / (float)p.ft;
  const int64_t ring_base = ((int64_t)b * p.ring_slots * p.hkv + g) * (int64_t)p.ft * HD;
  const int64_t slot_stride = (int64_t)p.hkv * p.ft * HD;
  const int64_t chunk_base = ((int64_t)b * p.nq * p.hkv + g) * HD;
  const int64_t chunk_stride = (int64_t)p.hkv * HD;

  uint4 kreg[4], vreg[4];
  auto load_tile = [&](int tile) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = tile * kKT + lkg * 4 + i;
      uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
      if (loader && j < nk) {
        int64_t off;
        const uint16_t *kb_, *vb_;
        if (j < ring_keys) {
          int s = (int)((float)j * inv_ft);
          int r = j - s * p.ft;
          if (r < 0) {
            --s;
            r += p.ft;
          } else if (r >= p.ft) {
            ++s;
            r -= p.ft;
          }
          off = ring_base + s * slot_stride + (int64_t)r * HD;
          kb_ = p.pk;
          vb_ = p.pv;
        } else {
          off = chunk_base + (int64_t)(j - ring_keys) * chunk_stride;
          kb_ = p.kc;
          vb_ = p.vc;
        }
        off += lc * 8;
        kv = *reinterpret_cast<const uint4*>(kb_ + off);
        vv = *reinterpret_cast<const uint4*>(vb_ + off);
      }
      kreg[i] = kv;
      vreg[i] = vv;
    }
  };
  auto store_tile = [&](int buf) {
    if (!loader) return;
    uint16_t* ks = smem + buf * C::STAGE;
    uint16_t* vs = ks + C::K_ELEMS;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint4*>(ks + (lkg * 4 + i) * C::KP + lc * 8) = kreg[i];
    const int pos = vperm(lkg * 4);
    const uint32_t* v0 = reinterpret_cast<const uint32_t*>(&vreg[0]);
    const uint32_t* v1 = reinterpret_cast<const uint32_t*>(&vreg[1]);
    const uint32_t* v2 = reinterpret_cast<const uint32_t*>(&vreg[2]);
    const uint32_t* v3 = reinterpret_cast<const uint32_t*>(&vreg[3]);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      // d = lc*8 + 2w (low halves) and lc*8 + 2w + 1 (high halves)
      const uint2 lo = make_uint2((v0[w] & 0xFFFFu) | (v1[w] << 16), (v2[w] & 0xFFFFu) | (v3[w] << 16));
      const uint2 hi2 = make_uint2((v0[w] >> 16) | (v1[w] & 0xFFFF0000u),
                                   (v2[w] >> 16) | (v3[w] & 0xFFFF0000u));
      *reinterpret_cast<uint2*>(vs + (lc * 8 + 2 * w) * kVP + pos) = lo;
      *reinterpret_cast<uint2*>(vs + (lc * 8 + 2 * w + 1) * kVP + pos) = hi2;
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
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};
  const float sl2 = p.scale_log2e;

  if (t_begin < t_end) {
    load_tile(t_begin);
    store_tile(0);
  }
  __syncthreads();

  for (int t = t_begin; t < t_end; ++t) {
    const int buf = (t - t_begin) & 1;
    const bool more = t + 1 < t_end;
    if (more) load_tile(t + 1);

    if (has_task) {
      const uint16_t* ks = smem + buf * C::STAGE;
      const uint16_t* vs = ks + C::K_ELEMS;
      // S^T blocks: [kb][qb], keys kb*32.., queries qb*32..
      f32x16 sacc[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int i = 0; i < 16; ++i) sacc[kb][qb][i] = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int dc = 0; dc < C::NDC; ++dc) {
          const bf16x8 kf =
              *reinterpret_cast<const bf16x8*>(ks + (kb * 32 + l32) * C::KP + dc * 16 + hi * 8);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            sacc[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qreg[qb][dc], sacc[kb][qb], 0, 0, 0);
        }
      }
      // Mask keys past the end (only the last tile can hold any).
      const int kbase = t * kKT;
      if (kbase + kKT > nk) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = kbase + kb * 32 + (i >> 2) * 8 + hi * 4 + (i & 3);
            if (key >= nk) {
              sacc[kb][0][i] = -INFINITY;
              sacc[kb][1][i] = -INFINITY;
            }
          }
      }
      // Online softmax (log2 domain), P^T fragments for the PV MFMA.
      bf16x8 pfrag[2][4];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        float mx = sacc[0][qb][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][qb][i]);
        mx = xhalf_max(mx);
        const float m_new = fmaxf(m_run[qb], mx * sl2);
        const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - m_new);
        m_run[qb] = m_new;
        float rs = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          uint32_t pk[8];
#pragma unroll
          for (int i = 0; i < 16; i += 2) {
            const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][qb][i], sl2, -m_new));
            const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][qb][i + 1], sl2, -m_new));
            rs += e0 + e1;
            pk[i >> 1] = pack_bf16(e0, e1);
          }
          pfrag[qb][kb * 2 + 0] = __builtin_bit_cast(bf16x8, make_uint4(pk[0], pk[1], pk[2], pk[3]));
          pfrag[qb][kb * 2 + 1] = __builtin_bit_cast(bf16x8, make_uint4(pk[4], pk[5], pk[6], pk[7]));
        }
        l_run[qb] = l_run[qb] * alpha + rs;
#pragma unroll
        for (int db = 0; db < C::NDB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[db][qb][i] *= alpha;
      }
      // O^T += V^T P^T
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
          const bf16x8 vf =
              *reinterpret_cast<const bf16x8*>(vs + (db * 32 + l32) * kVP + kc * 16 + hi * 8);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
            oacc[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pfrag[qb][kc], oacc[db][qb], 0, 0, 0);
        }
      }
    }

    if (more) store_tile(buf ^ 1);
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
      const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
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

hipError_t launch_chunk_attn(const AttnParams& p, int head_dim, hipStream_t s) {
  const dim3 grid(p.nb * p.hkv * p.wg_per_bg * p.nsplit);
  if (head_dim == 128)
    hipLaunchKernelGGL(chunk_attn_kernel<128>, grid, dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL(chunk_attn_kernel<64>, grid, dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace wm
