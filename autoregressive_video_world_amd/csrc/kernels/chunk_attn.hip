// Block-causal chunk attention over a bounded KV ring (gfx950, bf16 MFMA).
//
// What it computes (Cosmos3-H-Dreams model card, "Model Architecture":
// block-causal student with a KV cache; AlpaDreams GTC write-up, section VII:
// a new frame is predicted from the denoised earlier frames and the noisy
// current one): for
// each query of the current chunk, softmax attention over the keys of the
// frames the rollout holds (sinks + window, from the ring pool) and of every
// frame of the chunk itself.  The visible ring slots of a rollout that has
// committed m frames are exactly slots 0 .. min(m, S+W)-1, so the key list is
// two segments: ring frames (unit row stride inside a slot) and the chunk
// (row stride Hkv*d).  Softmax is order-invariant, so keys are visited in
// slot order, never concatenated.
//
// Two forms share this file's helpers and the key-range split/combine:
//  * chunk_attn8_kernel (the one launched): eight waves per workgroup, two per
//    SIMD, 32 queries per wave -- described where it is defined below;
//  * chunk_attn_kernel: four waves, one per SIMD, 64 queries per wave
//    (selectable with WM_ATTN_FORM=4 for measurement), described here.
// Both cover 256 queries of one kv head per workgroup.
//
// Design of the four-wave form (one workgroup = 4 waves = 4 "wave tasks"
// that share one kv head):
//  * a wave task is 64 queries of one q head: two 32-query blocks;
//  * keys stream through LDS in 64-key tiles, K and V triple-buffered, with
//    direct global->LDS loads (global_load_lds_dwordx4): no staging
//    registers, no LDS store instructions.  A tile is stored column-major:
//    16-byte column c of all 64 key rows is one contiguous 1 KB run (column
//    pitch 1088 B), so one wave-wide DMA instruction fills one column with
//    lane = key row, and every lane computes one row address per tile.  Keys
//    past the end are clamped to the last key and masked out of the softmax;
//  * S^T = K * Q^T on v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = Q^T
//    held in AGPRs for the whole kernel): in the 32x32 accumulator layout
//    each lane owns one query column and 16 keys, so the row max and row sum
//    need one cross-half exchange (v_permlane32_swap), no tree;
//  * O^T += V^T * P^T on the same MFMA: P^T comes straight from the S^T
//    accumulator (exp2, cvt_pk_bf16); the row sum l adds the fp32
//    exponentials (plain adds: on this chip a v_dot2 does not issue beside a
//    running MFMA, fp32 adds do).  V^T operands are read with
//    ds_read_b64_tr_b16: in each 16-lane group, lane j receives element j%4
//    of the 8-byte chunks read by lanes j/4, j/4+4, j/4+8, j/4+12, so when
//    lane L reads key row kbase + L/4 at dims dbase + 4*(L%4), lane j gets
//    V[kbase .. kbase+3][dbase + j] -- four consecutive keys of one dim,
//    exactly the keys the S^T accumulator layout gives that lane's P;
//  * 32-key sub-tile pipeline: in sub-step j the matrix cores compute S of
//    sub-tile j+1 and O += V P of sub-tile j-1 while the vector ALUs form P of
//    sub-tile j, interleaved by hand (one MFMA per slot with a slice of the
//    vector work).  Each K and V fragment read from LDS feeds both query
//    blocks (LDS instruction count per tile halves compared with handling the
//    blocks apart -- LDS issue, not bandwidth, is the scarce resource);
//  * online softmax in the log2 domain with a lazy rescale: the running max
//    only moves (and O, l are rescaled) when a row's new max exceeds it by
//    more than 8 (P stays <= 2^8); a wave-uniform branch, rarely taken;
//  * GQA: the 4 wave tasks of a workgroup are (q block, head-in-group) pairs
//    of one kv head, so a K/V tile in LDS serves every q head of the group.
// This file is compiled with -fno-honor-nans (max without NaN quieting):
// the softmax never produces NaN from finite inputs; -inf is still honoured.
#include "../wm_internal.hpp"

#include <mutex>
#include <type_traits>

namespace wm {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;
typedef __attribute__((address_space(3))) uint8_t lds_u8;

constexpr int kKT = 64;                // keys per tile
constexpr int kXcds = 8;               // MI355X: 8 accelerator complex dies
constexpr float kRescaleSlack = 8.0f;  // log2 units
constexpr int kColPitch = kKT * 16 + 64;  // bytes per 16-byte column of a tile

// NQB = 32-query blocks per wave task: 2 -> 4 waves per workgroup, one per
// SIMD, 64 queries per wave (launched); 1 -> 8 waves, two per SIMD, 32
// queries each (kept compilable; slower, since each K/V fragment read from
// LDS then feeds half as many MFMAs).  A workgroup covers 256 queries of one
// kv head either way.
template <int HD, int NQB>
struct Cfg {
  static constexpr int WAVES = 8 / NQB;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int NDC = HD / 16;             // 16-wide d chunks (QK^T contraction)
  static constexpr int NDB = HD / 32;             // 32-row d blocks (PV output)
  static constexpr int NCOL = HD / 8;             // 16-byte columns per key row
  static constexpr int COLS_PER_WAVE = NCOL / WAVES;
  static constexpr int TILE_BYTES = NCOL * kColPitch;
  static constexpr int LDS_BYTES = 6 * TILE_BYTES;  // K x3, V x3
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
// AGPRs, so the allocator never shuttles them across the rare rescale branch.
template <typename T>
__device__ __forceinline__ void pin_agpr(T& x) {
  asm("" : "+a"(x));
}
template <typename T>
__device__ __forceinline__ void pin_vgpr(T& x) {
  asm("" : "+v"(x));
}
// Anchor: a side-effecting use that keeps a value's computation from being
// sunk past this point (the compiler otherwise moves the softmax out of the
// MFMA region, next to its first use, and nothing overlaps).
template <typename T>
__device__ __forceinline__ void anchor(const T& x) {
  asm volatile("" ::"v"(x));
}

// Wait until at most n of this wave's vector-memory operations are pending
// (s_waitcnt vmcnt(n), other counters untouched).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Tile barrier: this wave's LDS reads done, at most n of its DMA transfers
// still in flight, then s_barrier.  Written out instead of __syncthreads():
// the workgroup release fence of the latter makes the compiler wait for every
// outstanding DMA (vmcnt(0)), including the prefetch two tiles ahead.  The
// asm carries a memory clobber, so no memory access moves across it.
template <int n>
__device__ __forceinline__ void tile_barrier() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (0x7 << 4));  // lgkmcnt(0)
  asm volatile("s_barrier" ::: "memory");
}

template <int HD, int NQB>
__global__ __launch_bounds__(512 / NQB, 1) void chunk_attn_kernel(const AttnParams p) {
  using C = Cfg<HD, NQB>;
  // Six distinct LDS objects (not one array): the compiler can then prove that
  // a read of one buffer never aliases a DMA still writing another, and does
  // not stall the read on vmcnt(0).
  __shared__ __attribute__((aligned(16))) uint8_t k0s[C::TILE_BYTES], k1s[C::TILE_BYTES], k2s[C::TILE_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t v0s[C::TILE_BYTES], v1s[C::TILE_BYTES], v2s[C::TILE_BYTES];
  lds_u8* const K0 = (lds_u8*)k0s;
  lds_u8* const K1 = (lds_u8*)k1s;
  lds_u8* const K2 = (lds_u8*)k2s;
  lds_u8* const V0 = (lds_u8*)v0s;
  lds_u8* const V1 = (lds_u8*)v1s;
  lds_u8* const V2 = (lds_u8*)v2s;

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
  const int n_local = min(ntiles, t_begin + tps) - t_begin;

  const int task = wgi * C::WAVES + wave;
  const bool has_task = task < p.group * p.nqb;
  const int qblk = has_task ? task / p.group : 0;
  const int h = g * p.group + (has_task ? task % p.group : 0);
  const int q0 = qblk * 32 * NQB;

  // A key-range split past the end of a short rollout's keys (ragged batch):
  // record an empty partial (sum 0) and leave; the whole workgroup agrees.
  if (n_local <= 0) {
    if (has_task && lane < 32) {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        const int q = q0 + qb * 32 + lane;
        if (q < p.nq) {
          const int64_t row = (((int64_t)split * p.nb + bi) * p.nq + q) * p.hq + h;
          p.part_ml[row * 2 + 0] = -INFINITY;
          p.part_ml[row * 2 + 1] = 0.f;
        }
      }
    }
    return;
  }

  // ---- Q^T operands: lane (l32, hi) holds query q0+qb*32+l32, d = dc*16+hi*8.. --
  bf16x8 qreg[NQB][C::NDC];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int q = min(q0 + qb * 32 + l32, p.nq - 1);
    const uint16_t* src = p.q + (((int64_t)b * p.nq + q) * p.hq + h) * HD + hi * 8;
#pragma unroll
    for (int dc = 0; dc < C::NDC; ++dc) {
      qreg[qb][dc] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(src + dc * 16));
      pin_agpr(qreg[qb][dc]);
    }
  }

  // ---- tile loads: lane = key row, wave w fills columns w*CPW .. ------------
  const int ft = p.ft;
  const float inv_ft = 1.0f / (float)ft;
  // This wave's first column, as a wave-uniform value (readfirstlane): the
  // column offsets then fold into the base pointers and the LDS addresses
  // (M0) are formed with scalar instructions.
  const int col0 = __builtin_amdgcn_readfirstlane(wave) * C::COLS_PER_WAVE;
  const uint16_t* const ring_k = p.pk + ((int64_t)b * p.ring_slots * p.hkv + g) * (int64_t)ft * HD + col0 * 8;
  const uint16_t* const ring_v = p.pv + ((int64_t)b * p.ring_slots * p.hkv + g) * (int64_t)ft * HD + col0 * 8;
  // Offsets within one rollout's ring and chunk tensor stay below 2^31
  // elements (the descriptor check at ring creation enforces it).
  const uint32_t slot_stride = (uint32_t)p.hkv * ft * HD;
  const uint16_t* const chunk_k = p.kc + ((int64_t)b * p.nq * p.hkv + g) * HD + col0 * 8;
  const uint16_t* const chunk_v = p.vc + ((int64_t)b * p.nq * p.hkv + g) * HD + col0 * 8;
  const uint32_t chunk_stride = (uint32_t)p.hkv * HD;

  // Row pointers (K and V) of this lane's key row in local tile u.
  auto row_ptrs = [&](int u, const uint16_t*& kp, const uint16_t*& vp) __attribute__((always_inline)) {
    const int j = min((t_begin + u) * kKT + lane, nk - 1);
    int s = (int)((float)j * inv_ft);
    int r = j - s * ft;
    s += (r >= ft) - (r < 0);
    r = j - s * ft;
    const bool in_ring = j < ring_keys;
    const uint32_t ro = (uint32_t)s * slot_stride + (uint32_t)r * HD;
    const uint32_t co = (uint32_t)(j - ring_keys) * chunk_stride;
    kp = in_ring ? ring_k + ro : chunk_k + co;
    vp = in_ring ? ring_v + ro : chunk_v + co;
  };
  // rp: this lane's key row, already offset to column col0.
  auto dma_cols = [&](const uint16_t* rp, lds_u8* tile) __attribute__((always_inline)) {
    lds_u8* const t0 = tile + col0 * kColPitch;
#pragma unroll
    for (int i = 0; i < C::COLS_PER_WAVE; ++i) {
      __builtin_amdgcn_global_load_lds(rp + i * 8, t0 + i * kColPitch, 16, 0, 0);
    }
  };

  // ---- running state ------------------------------------------------------
  f32x16 oacc[C::NDB][NQB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db)
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[db][qb][i] = 0.f;
  float m_run[NQB], l_run[NQB];  // running max (scaled, log2 domain), sum over this lane's keys
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
  }
  const float sl2 = p.scale_log2e;

  // LDS byte offsets of this lane's reads inside a tile.
  //  K operand (A of S^T): key row kb*32 + l32, column 2*dc + hi.
  const uint32_t k_off = (uint32_t)(hi * kColPitch + l32 * 16);
  //  V^T operand: group lane L = lane & 15 reads key row +hi*4 + L/4, dims
  //  dsub*16 + 4*(L&3) -> column dsub*2 + (L&3)/2, byte (L&1)*8 inside it.
  const int tr_l = lane & 15;
  const uint32_t v_off = (uint32_t)((((lane >> 4) & 1) * 2 + ((tr_l & 3) >> 1)) * kColPitch +
                                    (hi * 4 + (tr_l >> 2)) * 16 + (tr_l & 1) * 8);

  // S^T of a 32-key sub-tile (keys kb*32.. of the tile) for both query blocks:
  // each K fragment read from LDS feeds two MFMAs.
  auto qk = [&](const lds_u8* tile, int kb, f32x16 (&S)[NQB]) __attribute__((always_inline)) {
#pragma unroll
    for (int dc = 0; dc < C::NDC; ++dc) {
      const bf16x8 kf = *(const lds_bf16x8*)(tile + k_off + 2 * dc * kColPitch + kb * 512);
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
        S[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qreg[qb][dc], dc == 0 ? (f32x16){} : S[qb], 0, 0, 0);
    }
  };
  // O^T += V^T P^T over a 32-key sub-tile, both query blocks; each V^T fragment
  // (two transposed reads) feeds two MFMAs.  MFMA half h covers keys kb*32+16h..:
  // lane half hi takes keys +4*hi+{0..3} and +8+4*hi+{0..3}.
  auto pv = [&](const lds_u8* tile, int kb, const bf16x8 (&P)[NQB][2]) __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const lds_u8* a = tile + v_off + db * 4 * kColPitch + (kb * 32 + half * 16) * 16;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)a);
        const s16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a + 8 * 16));
        const bf16x8 vf = __builtin_bit_cast(bf16x8, (s16x8){lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2], up[3]});
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
          oacc[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, P[qb][half], oacc[db][qb], 0, 0, 0);
      }
    }
  };
  // Row max over a 32-key sub-tile (lane pair holds the 32 keys of a query).
  auto sub_rowmax = [&](const auto& S) __attribute__((always_inline)) {
    float m0 = fmaxf(S[0], fmaxf(S[1], S[2]));
    float m1 = fmaxf(S[3], fmaxf(S[4], S[5]));
#pragma unroll
    for (int i = 6; i < 16; i += 4) {
      m0 = fmaxf(m0, fmaxf(S[i], S[i + 1]));
      m1 = fmaxf(m1, fmaxf(S[i + 2], S[i + 3]));
    }
    return xhalf_max(fmaxf(m0, m1));
  };
  // Mask keys >= nvalid of a sub-tile (only in the last tile of the key range).
  auto mask_sub = [&](auto& S, int nvalid) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = (i >> 2) * 8 + hi * 4 + (i & 3);
      if (key >= nvalid) {
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) S[qb][i] = -INFINITY;
      }
    }
  };
  // Lazy rescale (wave-uniform, rarely taken).  The decision for sub-tile j is
  // taken before its exponentials: the running max and sum move at once, but
  // O is rescaled only after the still-pending P(j-1)*V -- formed against the
  // old max -- has been accumulated (rescale_o at the end of the sub-step).
  auto rescale_decide = [&](const float (&mx)[NQB], float (&alpha)[NQB]) __attribute__((always_inline)) {
    bool need = false;
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) need |= mx[qb] * sl2 > m_run[qb] + kRescaleSlack;
    if (!__builtin_amdgcn_ballot_w64(need)) return false;
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const float m_new = fmaxf(m_run[qb], mx[qb] * sl2);
      alpha[qb] = __builtin_amdgcn_exp2f(m_run[qb] - m_new);
      m_run[qb] = m_new;
      l_run[qb] *= alpha[qb];
    }
    return true;
  };
  auto rescale_o = [&](const float (&alpha)[NQB]) __attribute__((always_inline)) {
    // A side-effecting marker keeps this block a real (rarely taken) branch:
    // if-converted, it would cost 3 x 128 VALU operations on every sub-step.
    asm volatile("; rescale O" ::: "memory");
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][qb][i] *= alpha[qb];
        pin_agpr(oacc[db][qb]);
      }
  };
  // Sub-tile j of the local key range: mask what lies past the end, then the
  // rescale decision on its row max.
  const int nk_local = nk - t_begin * kKT;  // keys of this split's range (last tile may be partial)
  auto prepare = [&](int j, auto& S, float (&mx)[NQB], float (&alpha)[NQB]) __attribute__((always_inline)) {
    const int nvalid = nk_local - j * 32;
    if (nvalid < 32) {
      mask_sub(S, nvalid);
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) mx[qb] = sub_rowmax(S[qb]);
    }
    return rescale_decide(mx, alpha);
  };
  f32x16 SA[NQB], SB[NQB];
  bf16x8 PA[NQB][2], PB[NQB][2];
  float mx[NQB];
  const uint16_t *kp, *vp;
  // S of the sub-tile whose softmax is next, copied once out of the MFMA
  // accumulators into VGPRs (the row max and the exponentials then read the
  // copy: one AGPR read per value instead of two).  Separate scalars, not a
  // vector: each value is then its own register, consumed independently.
  float Sv[NQB][16];
  auto take_s = [&](const f32x16 (&S)[NQB]) __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        Sv[qb][i] = S[qb][i];
        pin_vgpr(Sv[qb][i]);
      }
      mx[qb] = sub_rowmax(Sv[qb]);
    }
  };

  // One 32-key sub-step j, scheduled by hand.  Matrix op i is issued in slot i
  // together with a slice of the vector work, and sched_barrier(0) keeps every
  // slice in its slot (left alone, the scheduler clusters the matrix ops and
  // the vector work then runs beside only a few of them):
  //   slots [0, NQK):        S(j+1) = K Q^T, 2 MFMAs per K fragment
  //                          || P(j) = exp2(S(j) * scale - m): 8 key pairs per query block
  //   slots [NQK, NQK+NPV):  O += V^T P(j-1)^T, 2 MFMAs per V fragment
  //                          || S(j+1) copied out of the accumulators, its row max;
  //                             the DMA issue of this sub-step
  // K fragments are read KAHEAD slots ahead of their MFMAs, V fragments
  // during the last QK slots.
  constexpr int NQK = C::NDC * NQB;
  constexpr int NPV = C::NDB * 2 * NQB;
  constexpr int NE = 8 * NQB;                 // exponential units (2 keys of one query block)
  constexpr int E_PER = (NE + NQK - 1) / NQK;  // per QK slot
  constexpr int KAHEAD = 4;
  constexpr int NVF = C::NDB * 2;             // V fragments per sub-step
  constexpr int VSLOT0 = NQK - NVF / 2 > 0 ? NQK - NVF / 2 : 0;  // first slot with V reads (2 per slot)
  auto substep = [&](const lds_u8* kt, int kb, f32x16 (&Sn)[NQB], bf16x8 (&Po)[NQB][2],
                     const lds_u8* vt, int vkb, const bf16x8 (&Pi)[NQB][2], bool do_pv,
                     auto&& dma) __attribute__((always_inline)) {
    bf16x8 kfr[C::NDC];
    bf16x8 vfr[NVF];
    uint32_t pk[NQB][8];
    float mq[NQB][4];
    float mneg[NQB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) mneg[qb] = -m_run[qb];
    auto read_k = [&](int dc) __attribute__((always_inline)) {
      kfr[dc] = *(const lds_bf16x8*)(kt + k_off + 2 * dc * kColPitch + kb * 512);
    };
    auto read_v = [&](int f) __attribute__((always_inline)) {  // f = half * NDB + db
      const int half = f / C::NDB, db = f % C::NDB;
      const lds_u8* a = vt + v_off + db * 4 * kColPitch + (vkb * 32 + half * 16) * 16;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)a);
      const s16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a + 8 * 16));
      vfr[f] = __builtin_bit_cast(bf16x8, (s16x8){lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2], up[3]});
    };
    // The slot's inputs pass through a volatile empty asm and its results into
    // one: volatile asm keeps its order relative to sched_barrier, so neither
    // the IR optimizers nor the scheduler can move the work out of its slot.
    auto exp_unit = [&](int e) __attribute__((always_inline)) {
      const int qb = e / 8, pr = e % 8;
      float s0 = Sv[qb][2 * pr], s1 = Sv[qb][2 * pr + 1];
      asm volatile("" : "+v"(s0), "+v"(s1));
      const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s0, sl2, mneg[qb]));
      const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s1, sl2, mneg[qb]));
      const bf16x2 two = {(__bf16)e0, (__bf16)e1};
      l_run[qb] = (l_run[qb] + e0) + e1;  // fp32 adds: a dot instruction would not overlap the MFMAs
      pk[qb][pr] = __builtin_bit_cast(uint32_t, two);
      asm volatile("" ::"v"(pk[qb][pr]), "v"(l_run[qb]));
    };
    // copy 4 values of S(j+1) out of the accumulators, and their max
    auto copy_unit = [&](int t) __attribute__((always_inline)) {
      const int qb = t / 4, r = t % 4;
      float x[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        x[k] = Sn[qb][4 * r + k];
        asm volatile("" : "+v"(x[k]));
        Sv[qb][4 * r + k] = x[k];
      }
      mq[qb][r] = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      asm volatile("" ::"v"(mq[qb][r]));
    };
    auto max_unit = [&](int qb) __attribute__((always_inline)) {
      mx[qb] = xhalf_max(fmaxf(fmaxf(mq[qb][0], mq[qb][1]), fmaxf(mq[qb][2], mq[qb][3])));
      asm volatile("" ::"v"(mx[qb]));
    };

#pragma unroll
    for (int dc = 0; dc < KAHEAD && dc < C::NDC; ++dc) read_k(dc);
#pragma unroll
    for (int i = 0; i < NQK + NPV; ++i) {
      if (i < NQK) {
        const int dc = i / NQB, qb = i % NQB;
        Sn[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfr[dc], qreg[qb][dc], dc == 0 ? (f32x16){} : Sn[qb], 0, 0, 0);
        if (qb == NQB - 1 && dc + KAHEAD < C::NDC) read_k(dc + KAHEAD);
        if (i >= VSLOT0) {
          const int f = 2 * (i - VSLOT0);
          if (f < NVF) read_v(f);
          if (f + 1 < NVF) read_v(f + 1);
        }
#pragma unroll
        for (int k = 0; k < E_PER; ++k)
          if (i * E_PER + k < NE) exp_unit(i * E_PER + k);
        if (i == NQK - 1) {
#pragma unroll
          for (int qb2 = 0; qb2 < NQB; ++qb2) {
            Po[qb2][0] = __builtin_bit_cast(bf16x8, make_uint4(pk[qb2][0], pk[qb2][1], pk[qb2][2], pk[qb2][3]));
            Po[qb2][1] = __builtin_bit_cast(bf16x8, make_uint4(pk[qb2][4], pk[qb2][5], pk[qb2][6], pk[qb2][7]));
          }
        }
      } else {
        const int m = i - NQK;
        const int f = m / NQB, qb = m % NQB;  // V fragment f = half * NDB + db
        if (do_pv)
          oacc[f % C::NDB][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfr[f], Pi[qb][f / C::NDB],
                                                                          oacc[f % C::NDB][qb], 0, 0, 0);
        // S(j+1) copy: NT units from slot CS of this half on (the second, when
        // there is room: one more matrix op between the last write and the
        // first read); a query block's row max right after its 4 units.
        constexpr int NT = 4 * NQB;
        constexpr int CS = NPV > NT ? 1 : 0;
        constexpr int T_PER = (NT + (NPV - CS) - 1) / (NPV - CS);
#pragma unroll
        for (int k = 0; k < T_PER; ++k) {
          const int t = (m - CS) * T_PER + k;
          if (m >= CS && t < NT) {
            copy_unit(t);
            if (t % 4 == 3) max_unit(t / 4);
          }
        }
        if (m == (CS + (NT + T_PER - 1) / T_PER < NPV ? CS + (NT + T_PER - 1) / T_PER : NPV - 1)) dma();
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Prologue: tiles 0 and 1 into LDS; S and row max of sub-tile 0.
  row_ptrs(0, kp, vp);
  dma_cols(kp, K0);
  dma_cols(vp, V0);
  row_ptrs(1, kp, vp);
  dma_cols(kp, K1);
  dma_cols(vp, V1);
  tile_barrier<0>();
  qk(K0, 0, SA);
  take_s(SA);

  // Two 32-key sub-steps per 64-key tile u.  Sub-step j computes
  //   S(j+1) on the matrix cores (K fragments shared by both query blocks)
  //   || P(j) = exp(S(j) - m) on the vector ALUs
  //   || O += V P(j-1) on the matrix cores (V fragments shared likewise),
  // then the row max of S(j+1).  K of tile u is read in sub-steps 2u-1 and
  // 2u, V of tile u in 2u+1 and 2u+2.  The DMA of K(u+2) is issued at
  // sub-step 2u into the buffer K(u-1) left, that of V(u+2) at 2u+1 into the
  // buffer V(u-1) left; the one barrier per tile (end of sub-step 2u) is
  // preceded by a wait that lets only the two newest DMA groups be in flight.
  // Buffers rotate with period 3 (tile u uses K[u%3], V[u%3]); the caller
  // passes them explicitly so every LDS access names a fixed object:
  //   ku = K(u), kn = K(u+1), kf = K(u+2) (DMA target),
  //   vu = V(u), vp_ = V(u-1) = V(u+2) (read in sub-step 2u, then DMA target).
  auto tile_steps = [&](int u, bool first, lds_u8* ku, lds_u8* kn, lds_u8* kf, lds_u8* vu,
                        lds_u8* vp_) __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) pin_agpr(oacc[db][qb]);
    float alpha[NQB];
    // sub-step 2u: S(2u) in Sv, P(2u-1) in PB
    bool resc = prepare(2 * u, Sv, mx, alpha);
    substep(ku, 1, SB, PA, vp_, 1, PB, !first, [&]() __attribute__((always_inline)) {
      row_ptrs(u + 2, kp, vp);
      dma_cols(kp, kf);
    });
    if (resc) rescale_o(alpha);
    tile_barrier<2 * C::COLS_PER_WAVE>();
    // sub-step 2u+1: S(2u+1) in Sv, P(2u) in PA
    resc = prepare(2 * u + 1, Sv, mx, alpha);
    substep(kn, 0, SA, PB, vu, 0, PA, true, [&]() __attribute__((always_inline)) { dma_cols(vp, vp_); });
    if (resc) rescale_o(alpha);
  };
  tile_steps(0, true, K0, K1, K2, V0, V2);
  int u = 1;
  for (; u + 3 <= n_local; u += 3) {
    tile_steps(u, false, K1, K2, K0, V1, V0);
    tile_steps(u + 1, false, K2, K0, K1, V2, V1);
    tile_steps(u + 2, false, K0, K1, K2, V0, V2);
  }
  if (u < n_local) tile_steps(u++, false, K1, K2, K0, V1, V0);
  if (u < n_local) tile_steps(u++, false, K2, K0, K1, V2, V1);
  // P(2n-1): V of the last tile, keys 32..63.
  switch ((n_local - 1) % 3) {
    case 0: pv(V0, 1, PB); break;
    case 1: pv(V1, 1, PB); break;
    default: pv(V2, 1, PB); break;
  }
  // No DMA may still be writing this workgroup's LDS when it retires.
  wait_vmcnt<0>();

  if (!has_task) return;

  // ---- epilogue -------------------------------------------------------------
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
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

// ---------------------------------------------------------------------------
// Eight-wave form: two waves per SIMD, 32 queries per wave.
//
// One wave issues at most one vector instruction every ~5 cycles (an exp
// every ~10), so the ~100 softmax instructions that go with every 16 MFMAs of
// a 64-query wave cannot hide under its own 512 MFMA cycles.  With two waves
// per SIMD each wave has half the queries and half the vector work, and the
// SIMD issues both waves' vector instructions beside the other wave's MFMAs.
// Each K or V fragment read from LDS then feeds one MFMA instead of two,
// which the LDS read rate (~245 B/clk per CU for 16-byte reads) carries.
// Per wave and 32-key sub-tile j:
//   QK half (one MFMA slot per 16-wide d chunk): S(j+1) = K Q^T on the
//     matrix cores (K fragments already in registers) || P(j) = exp2(S(j)
//     * scale - m) on the vector ALUs || the V^T fragments of sub-tile j
//     read from LDS;
//   PV half (one slot per V fragment): O^T += V^T P(j)^T || the row max of
//     S(j+1) || the K fragments of sub-tile j+2 read from LDS.
// Every operand and accumulator lives in VGPRs (230 of the 256 a wave has at
// two waves per SIMD; no AGPRs), so the softmax reads S without accumulator
// copies.  Tiles of 64 keys stream through NBUF LDS buffers; one
// barrier per tile, in the middle of its first sub-step, after which the
// DMA of the tile NBUF-1 ahead is issued into the buffer the tile before
// freed.
// ---------------------------------------------------------------------------
template <int HD>
struct Cfg8 {
  static constexpr int WAVES = 8;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int NDC = HD / 16;             // QK MFMAs per sub-tile
  static constexpr int NDB = HD / 32;             // 32-row d blocks of O^T
  static constexpr int NCOL = HD / 8;             // 16-byte columns per key row
  static constexpr int COLS_PER_WAVE = NCOL / WAVES;
  static constexpr int TILE_BYTES = NCOL * kColPitch;
  static_assert(COLS_PER_WAVE >= 1, "every wave fills at least one column");
};

template <int HD, int NBUF>
__global__ __launch_bounds__(512, 1) void chunk_attn8_kernel(const AttnParams p) {
  using C = Cfg8<HD>;
  static_assert(NBUF == 3 || NBUF == 4, "three or four tile buffers");
  // Distinct LDS objects: a read of one buffer provably never aliases a DMA
  // still writing another, so reads do not wait for every pending DMA.
  __shared__ __attribute__((aligned(16))) uint8_t k0s[C::TILE_BYTES], k1s[C::TILE_BYTES], k2s[C::TILE_BYTES],
      k3s[NBUF == 4 ? C::TILE_BYTES : 16];
  __shared__ __attribute__((aligned(16))) uint8_t v0s[C::TILE_BYTES], v1s[C::TILE_BYTES], v2s[C::TILE_BYTES],
      v3s[NBUF == 4 ? C::TILE_BYTES : 16];
  lds_u8* const KB[4] = {(lds_u8*)k0s, (lds_u8*)k1s, (lds_u8*)k2s, (lds_u8*)k3s};
  lds_u8* const VB[4] = {(lds_u8*)v0s, (lds_u8*)v1s, (lds_u8*)v2s, (lds_u8*)v3s};

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

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
  const int n_local = min(ntiles, t_begin + tps) - t_begin;

  const int task = wgi * C::WAVES + wave;
  const bool has_task = task < p.group * p.nqb;
  const int qblk = has_task ? task / p.group : 0;
  const int h = g * p.group + (has_task ? task % p.group : 0);
  const int q0 = qblk * 32;

  if (n_local <= 0) {
    if (has_task && lane < 32) {
      const int q = q0 + lane;
      if (q < p.nq) {
        const int64_t row = (((int64_t)split * p.nb + bi) * p.nq + q) * p.hq + h;
        p.part_ml[row * 2 + 0] = -INFINITY;
        p.part_ml[row * 2 + 1] = 0.f;
      }
    }
    return;
  }

  // Q^T operands: lane (l32, hi) holds query q0+l32, d = dc*16 + hi*8 .. +8.
  bf16x8 qreg[C::NDC];
  {
    const int q = min(q0 + l32, p.nq - 1);
    const uint16_t* src = p.q + (((int64_t)b * p.nq + q) * p.hq + h) * HD + hi * 8;
#pragma unroll
    for (int dc = 0; dc < C::NDC; ++dc) {
      qreg[dc] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(src + dc * 16));
    }
  }

  // ---- tile loads: lane = key row, wave w fills columns w*CPW .. ---------
  const int ft = p.ft;
  const float inv_ft = 1.0f / (float)ft;
  const int col0 = __builtin_amdgcn_readfirstlane(wave) * C::COLS_PER_WAVE;
  const uint16_t* const ring_k = p.pk + ((int64_t)b * p.ring_slots * p.hkv + g) * (int64_t)ft * HD + col0 * 8;
  const uint16_t* const ring_v = p.pv + ((int64_t)b * p.ring_slots * p.hkv + g) * (int64_t)ft * HD + col0 * 8;
  const uint32_t slot_stride = (uint32_t)p.hkv * ft * HD;
  const uint16_t* const chunk_k = p.kc + ((int64_t)b * p.nq * p.hkv + g) * HD + col0 * 8;
  const uint16_t* const chunk_v = p.vc + ((int64_t)b * p.nq * p.hkv + g) * HD + col0 * 8;
  const uint32_t chunk_stride = (uint32_t)p.hkv * HD;

  // Tile loads: direct global->LDS DMA, lane = key row, wave w fills the
  // 16-byte columns w*CPW .. of K and of V (keys past the end clamp to the
  // last key).  A tile's DMA instructions are spread over the slots of two
  // sub-steps instead of issued together: the row addresses are formed once
  // (tile_rows), then each call of dma_col issues one column.
  const uint16_t* dkp;  // this lane's K and V row of the tile being fetched
  const uint16_t* dvp;
  auto tile_rows = [&](int u) __attribute__((always_inline)) {
    const int j = min((t_begin + u) * kKT + lane, nk - 1);
    int s = (int)((float)j * inv_ft);
    int r = j - s * ft;
    s += (r >= ft) - (r < 0);
    r = j - s * ft;
    const bool in_ring = j < ring_keys;
    const uint32_t ro = (uint32_t)s * slot_stride + (uint32_t)r * HD;
    const uint32_t co = (uint32_t)(j - ring_keys) * chunk_stride;
    dkp = in_ring ? ring_k + ro : chunk_k + co;
    dvp = in_ring ? ring_v + ro : chunk_v + co;
  };
  // column c of this wave's share (c < CPW: K, else V) into tile kt / vt
  auto dma_col = [&](int c, lds_u8* kt, lds_u8* vt) __attribute__((always_inline)) {
    if (c < C::COLS_PER_WAVE) {
      const uint16_t* src = dkp + c * 8;
      lds_u8* dst = kt + (col0 + c) * kColPitch;
      __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
    } else {
      const uint16_t* src = dvp + (c - C::COLS_PER_WAVE) * 8;
      lds_u8* dst = vt + (col0 + c - C::COLS_PER_WAVE) * kColPitch;
      __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
    }
  };
  constexpr int NDMA = 2 * C::COLS_PER_WAVE;  // DMA instructions per wave per tile

  // ---- running state ------------------------------------------------------
  f32x16 oacc[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;  // running max (scaled, log2), this lane's partial sum
  const float sl2 = p.scale_log2e;

  const uint32_t k_off = (uint32_t)(hi * kColPitch + l32 * 16);
  const int tr_l = lane & 15;
  const uint32_t v_off = (uint32_t)((((lane >> 4) & 1) * 2 + ((tr_l & 3) >> 1)) * kColPitch +
                                    (hi * 4 + (tr_l >> 2)) * 16 + (tr_l & 1) * 8);

  // K fragments of the next sub-tile's QK.
  bf16x8 kf[C::NDC];
  auto read_k = [&](const lds_u8* tile, int kb, int dc) __attribute__((always_inline)) {
    kf[dc] = *(const lds_bf16x8*)(tile + k_off + 2 * dc * kColPitch + kb * 512);
  };
  auto rowmax16 = [&](const f32x16& S) __attribute__((always_inline)) {
    float m0 = fmaxf(S[0], fmaxf(S[1], S[2]));
    float m1 = fmaxf(S[3], fmaxf(S[4], S[5]));
    m0 = fmaxf(m0, fmaxf(S[6], S[7]));
    m1 = fmaxf(m1, fmaxf(S[8], S[9]));
    m0 = fmaxf(m0, fmaxf(S[10], S[11]));
    m1 = fmaxf(m1, fmaxf(S[12], S[13]));
    m0 = fmaxf(m0, fmaxf(S[14], S[15]));
    return xhalf_max(fmaxf(m0, m1));
  };
  const int nk_local = nk - t_begin * kKT;
  // Lazy rescale.  The decision for sub-tile j is taken on its row max
  // before its exponentials: the running max and sum move at once.  O is
  // rescaled one sub-step later, once P(j-1) -- formed against the old max
  // and accumulated during sub-step j -- is in it (o_pending carries the
  // factor).  Keys past the end of the range (only in the last tile) are
  // masked first.
  float o_alpha = 1.f;
  bool o_pending = false;  // wave-uniform
  auto prepare = [&](int j, f32x16& S, float mx) __attribute__((always_inline)) {
    const int nvalid = nk_local - j * 32;
    if (nvalid < 32) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = (i >> 2) * 8 + hi * 4 + (i & 3);
        if (key >= nvalid) S[i] = -INFINITY;
      }
      mx = rowmax16(S);
    }
    const bool need = mx * sl2 > m_run + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float m_new = fmaxf(m_run, mx * sl2);
      o_alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= o_alpha;
      o_pending = true;
    }
  };
  auto rescale_o = [&]() __attribute__((always_inline)) {
    if (o_pending) {
      asm volatile("; rescale O" ::: "memory");
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= o_alpha;
      o_pending = false;
    }
  };

  constexpr int NQK = C::NDC;       // QK MFMAs per sub-step
  constexpr int NPV = 2 * C::NDB;   // PV MFMAs per sub-step (one per V fragment)
  static_assert(NQK == NPV, "QK and PV slots pair up");
  constexpr int NS = NQK + NPV;     // MFMA slots per sub-step
  constexpr int RA = NS / 2;        // fragment reads run RA slots ahead of their MFMA
  constexpr int NE = 8;             // exponential units (2 keys each) per sub-tile
  static_assert(NS % NE == 0, "exponential units spread evenly");
  constexpr int DMA_EVERY = (NS + RA) / NDMA;  // DMA issues spread over the slots after the barrier
  // Slot order of a sub-step: Q0 P0 Q1 P1 ... Q(n-3) P(n-3) Q(n-2) Q(n-1)
  // P(n-2) P(n-1) (Q = a QK MFMA, P = a PV MFMA): the last QK comes two slots
  // before the end, so S(j+1) is done when its row max is taken.
  constexpr auto slot_is_q = [](int i) { return i < 2 * (NQK - 2) ? i % 2 == 0 : i < 2 * (NQK - 2) + 2; };
  constexpr auto slot_idx = [](int i) {
    return i < 2 * (NQK - 2) ? i / 2 : (i < 2 * (NQK - 2) + 2 ? NQK - 2 + (i - 2 * (NQK - 2)) : NPV - 2 + (i - 2 * (NQK - 2) - 2));
  };

  // Operand fragments in flight: a ring of RA registers; the fragment of
  // slot i lives in fr[i % RA], read from LDS RA slots before slot i, into
  // the register the MFMA of slot i - RA has just read.
  bf16x8 fr[RA];
  struct Src {
    const lds_u8* t;
    int kb;
  };
  auto read_frag = [&](int slot, Src k, Src v) __attribute__((always_inline)) {
    const int idx = slot_idx(slot);
    if (slot_is_q(slot)) {
      fr[slot % RA] = *(const lds_bf16x8*)(k.t + k_off + 2 * idx * kColPitch + k.kb * 512);
    } else {
      const int half = idx / C::NDB, db = idx % C::NDB;
      const lds_u8* a = v.t + v_off + db * 4 * kColPitch + (v.kb * 32 + half * 16) * 16;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)a);
      const s16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a + 8 * 16));
      fr[slot % RA] = __builtin_bit_cast(bf16x8, (s16x8){lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2], up[3]});
    }
  };

  // One sub-step j.  On entry: Sc = S(j) (masked, max checked), Pp = P(j-1),
  // the ring holds the fragments of slots 0 .. RA-1.  The matrix cores
  // alternate S(j+1) = K(j+1) Q^T and O^T += V(j-1)^T P(j-1)^T; slot i also
  // reads the fragment of slot i+RA -- from K(j+1) / V(j-1) (cur) while that
  // is in this sub-step, else from K(j+2) / V(j) (nxt).  The vector ALUs form
  // P(j) = exp2(S(j) * scale - m) into Pn across the slots; mid() runs after
  // slot RA-1 (the tile barrier, when there is one), hook(i) after slot i.
  // Returns the row max of S(j+1).
  auto substep = [&](const f32x16& Sc, f32x16& Sn, const bf16x8 (&Pp)[2], bf16x8 (&Pn)[2], Src curK,
                     Src curV, Src nxtK, Src nxtV, auto&& mid, auto&& hook) __attribute__((always_inline)) {
    uint32_t pk[8];
    const float mneg = -m_run;
    auto exp_unit = [&](int e) __attribute__((always_inline)) {
      float s0 = Sc[2 * e], s1 = Sc[2 * e + 1];
      asm volatile("" : "+v"(s0), "+v"(s1));
      const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s0, sl2, mneg));
      const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s1, sl2, mneg));
      const bf16x2 two = {(__bf16)e0, (__bf16)e1};
      l_run = (l_run + e0) + e1;
      pk[e] = __builtin_bit_cast(uint32_t, two);
      asm volatile("" ::"v"(pk[e]), "v"(l_run));
    };
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int idx = slot_idx(i);
      if (slot_is_q(i)) {
        Sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[i % RA], qreg[idx], idx == 0 ? (f32x16){} : Sn, 0, 0, 0);
      } else {
        oacc[idx % C::NDB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[i % RA], Pp[idx / C::NDB],
                                                                      oacc[idx % C::NDB], 0, 0, 0);
      }
      if (i + RA < NS)
        read_frag(i + RA, curK, curV);
      else
        read_frag(i + RA - NS, nxtK, nxtV);
      if (i % (NS / NE) == NS / NE - 1) exp_unit(i / (NS / NE));
      if (i == RA - 1) {
        __builtin_amdgcn_sched_barrier(0);
        mid();
      }
      hook(i);
      __builtin_amdgcn_sched_barrier(0);
    }
    Pn[0] = __builtin_bit_cast(bf16x8, make_uint4(pk[0], pk[1], pk[2], pk[3]));
    Pn[1] = __builtin_bit_cast(bf16x8, make_uint4(pk[4], pk[5], pk[6], pk[7]));
    rescale_o();  // after P(j-1) V(j-1) was issued, before P(j) V(j)
    return rowmax16(Sn);
  };

  // ---- prologue -------------------------------------------------------------
  // Tiles 0 .. NBUF-2 in flight; buffer NBUF-1 stands for "tile -1" in the
  // first sub-step (V(-1), multiplied by P(-1) = 0) and is zeroed so that the
  // product is exactly 0.  Then S(0), its row max, the first ring fill.
#pragma unroll
  for (int u = 0; u < NBUF - 1; ++u) {
    tile_rows(u);
#pragma unroll
    for (int c = 0; c < NDMA; ++c) dma_col(c, KB[u], VB[u]);
  }
  for (int o = tid * 16; o < C::TILE_BYTES; o += C::THREADS * 16)
    *(lds_bf16x8*)(VB[NBUF - 1] + o) = (bf16x8){};
  wait_vmcnt<(NBUF - 2) * NDMA>();
  tile_barrier<(NBUF - 2) * NDMA>();
  f32x16 SA, SB;
  bf16x8 PA[2], PB[2];
  {
    bf16x8 k0[C::NDC];
#pragma unroll
    for (int dc = 0; dc < C::NDC; ++dc) k0[dc] = *(const lds_bf16x8*)(KB[0] + k_off + 2 * dc * kColPitch);
#pragma unroll
    for (int dc = 0; dc < C::NDC; ++dc)
      SA = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0[dc], qreg[dc], dc == 0 ? (f32x16){} : SA, 0, 0, 0);
  }
#pragma unroll
  for (int i = 0; i < RA; ++i) read_frag(i, Src{KB[0], 1}, Src{VB[NBUF - 1], 1});
  PB[0] = PB[1] = (bf16x8){};
  prepare(0, SA, rowmax16(SA));

  // Sub-steps 2u and 2u+1 of local tile u (buffer u % NBUF).  The barrier
  // after slot RA-1 of sub-step 2u: this wave's DMA of tile u+1 has landed
  // (its K is first read right after), every wave has read the last of
  // tile u-1 (V(2u-1), read up to slot RA-1 of sub-step 2u).  After it the
  // DMA of tile u+NBUF-1, into the buffer tile u-1 left, is issued one column
  // at a time over the remaining slots of the tile (only the DMA of tile
  // u+NBUF-2 may then be in flight at the next barrier when NBUF = 4; NBUF =
  // 3 waits for everything).
  auto tile_steps = [&](int u, auto ph_) __attribute__((always_inline)) {
    constexpr int ph = decltype(ph_)::value;
    constexpr int nx = (ph + 1) % NBUF;
    constexpr int pv = (ph + NBUF - 1) % NBUF;  // tile u-1, freed at the barrier
    auto dma = [&](int pos) __attribute__((always_inline)) {  // pos: slots since the barrier
      if (pos >= 0 && pos % DMA_EVERY == DMA_EVERY / 2 && pos / DMA_EVERY < NDMA)
        dma_col(pos / DMA_EVERY, KB[pv], VB[pv]);
    };
    float mx = substep(SA, SB, PB, PA, Src{KB[ph], 1}, Src{VB[pv], 1}, Src{KB[nx], 0}, Src{VB[ph], 0},
                       [&]() __attribute__((always_inline)) {
                         tile_barrier<(NBUF - 3) * NDMA>();
                         tile_rows(u + NBUF - 1);
                       },
                       [&](int i) __attribute__((always_inline)) { dma(i - RA); });
    prepare(2 * u + 1, SB, mx);
    mx = substep(SB, SA, PA, PB, Src{KB[nx], 0}, Src{VB[ph], 0}, Src{KB[nx], 1}, Src{VB[ph], 1},
                 []() {}, [&](int i) __attribute__((always_inline)) { dma(NS - RA + i); });
    prepare(2 * u + 2, SA, mx);
  };
  int u = 0;
  for (; u + NBUF <= n_local; u += NBUF) {
    tile_steps(u, std::integral_constant<int, 0>{});
    tile_steps(u + 1, std::integral_constant<int, 1>{});
    tile_steps(u + 2, std::integral_constant<int, 2>{});
    if constexpr (NBUF == 4) tile_steps(u + 3, std::integral_constant<int, 3>{});
  }
  // The remaining tiles, each with its phase (u % NBUF).
  if (u < n_local) tile_steps(u++, std::integral_constant<int, 0>{});
  if (u < n_local) tile_steps(u++, std::integral_constant<int, 1>{});
  if constexpr (NBUF == 4)
    if (u < n_local) tile_steps(u++, std::integral_constant<int, 2>{});
  // P(2n-1) V(2n-1): the last sub-tile's P*V (PB holds P(2n-1); V(2n-1) is
  // the second half of the last tile, in buffer (n_local-1) % NBUF).
  {
    const int lb = (n_local - 1) % NBUF;
    const lds_u8* vl = lb == 0 ? VB[0] : lb == 1 ? VB[1] : lb == 2 ? VB[2] : VB[3];
#pragma unroll
    for (int m = 0; m < NPV; ++m) {
      const int half = m / C::NDB, db = m % C::NDB;
      const lds_u8* a = vl + v_off + db * 4 * kColPitch + (32 + half * 16) * 16;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)a);
      const s16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(a + 8 * 16));
      const bf16x8 vf = __builtin_bit_cast(bf16x8, (s16x8){lo[0], lo[1], lo[2], lo[3], up[0], up[1], up[2], up[3]});
      oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, PB[half], oacc[db], 0, 0, 0);
    }
  }
  rescale_o();
  // No DMA may still be writing this workgroup's LDS when it retires.
  wait_vmcnt<0>();

  if (!has_task) return;

  // ---- epilogue -------------------------------------------------------------
  const int q = q0 + l32;
  const float l_tot = xhalf_sum(l_run);
  if (q >= p.nq) return;
  const float inv = 1.0f / l_tot;
  if (p.nsplit == 1) {
    uint16_t* dst = p.out + (((int64_t)b * p.nq + q) * p.hq + h) * HD;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int d = db * 32 + ii * 8 + hi * 4;
        const uint2 v = make_uint2(pack_bf16(oacc[db][ii * 4 + 0] * inv, oacc[db][ii * 4 + 1] * inv),
                                   pack_bf16(oacc[db][ii * 4 + 2] * inv, oacc[db][ii * 4 + 3] * inv));
        *reinterpret_cast<uint2*>(dst + d) = v;
      }
  } else {
    const int64_t row = (((int64_t)split * p.nb + bi) * p.nq + q) * p.hq + h;
    float* dst = p.part_o + row * HD;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int d = db * 32 + ii * 8 + hi * 4;
        *reinterpret_cast<float4*>(dst + d) =
            make_float4(oacc[db][ii * 4 + 0] * inv, oacc[db][ii * 4 + 1] * inv,
                        oacc[db][ii * 4 + 2] * inv, oacc[db][ii * 4 + 3] * inv);
      }
    if (hi == 0) {
      p.part_ml[row * 2 + 0] = m_run;
      p.part_ml[row * 2 + 1] = l_tot;
    }
  }
}

// Merge the key-range partials of a split launch: weights l_s * 2^(m_s - M)
// over the splits with keys (log-sum-exp combine), one thread per 8 output
// dims of one (rollout, query, head) row.
template <int HD>
__global__ __launch_bounds__(256) void attn_combine_kernel(const AttnParams p) {
  constexpr int kCpr = HD / 8;
  const int64_t rows = (int64_t)p.nb * p.nq * p.hq;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= rows * kCpr) return;
  const int c = (int)(idx % kCpr);
  const int64_t row = idx / kCpr;
  // Every split's (max, sum) and output slice are loaded before any is used,
  // so a thread waits for one round of memory latency, not two per split.
  // A split with an empty key range has sum 0 and an unwritten output slice:
  // its values are loaded but never used.
  float m[kAttnMaxSplit], l[kAttnMaxSplit];
  float4 a[kAttnMaxSplit], b[kAttnMaxSplit];
#pragma unroll
  for (int s = 0; s < kAttnMaxSplit; ++s) {
    if (s < p.nsplit) {
      const int64_t r = s * rows + row;
      const float2 ml = *reinterpret_cast<const float2*>(p.part_ml + r * 2);
      m[s] = ml.x;
      l[s] = ml.y;
      const float4* src = reinterpret_cast<const float4*>(p.part_o + r * HD + c * 8);
      a[s] = src[0];
      b[s] = src[1];
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < kAttnMaxSplit; ++s)
    if (s < p.nsplit && l[s] > 0.f) M = fmaxf(M, m[s]);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
#pragma unroll
  for (int s = 0; s < kAttnMaxSplit; ++s) {
    if (!(s < p.nsplit && l[s] > 0.f)) continue;
    const float w = l[s] * __builtin_amdgcn_exp2f(m[s] - M);
    wsum += w;
    acc[0] += w * a[s].x;
    acc[1] += w * a[s].y;
    acc[2] += w * a[s].z;
    acc[3] += w * a[s].w;
    acc[4] += w * b[s].x;
    acc[5] += w * b[s].y;
    acc[6] += w * b[s].z;
    acc[7] += w * b[s].w;
  }
  const float inv = 1.0f / wsum;
  const int h = (int)(row % p.hq);
  const int64_t qrow = row / p.hq;
  const int q = (int)(qrow % p.nq);
  const int bi = (int)(qrow / p.nq);
  uint16_t* dst = p.out + (((int64_t)p.b_index[bi] * p.nq + q) * p.hq + h) * HD + c * 8;
  *reinterpret_cast<uint4*>(dst) = make_uint4(pack_bf16(acc[0] * inv, acc[1] * inv), pack_bf16(acc[2] * inv, acc[3] * inv),
                                              pack_bf16(acc[4] * inv, acc[5] * inv), pack_bf16(acc[6] * inv, acc[7] * inv));
}

}  // namespace

// ---------------------------------------------------------------------------
// Scratch of the allocation-free entry point.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in): it passes the
// device address scratch_region() looked up for the current device.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch[kMaxDevices];
}  // namespace

hipError_t scratch_region(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return hipSuccess;
}

int chunk_attn_specs(AttnParams& p, int head_dim, LaunchSpec specs[2]) {
  if ((p.wave_qblocks != 1 && p.wave_qblocks != 2) || (head_dim != 128 && head_dim != 64)) return 0;
  p.n_wg = p.nb * p.hkv * p.wg_per_bg * p.nsplit;
  p.per_xcd = (p.n_wg + kXcds - 1) / kXcds;
  specs[0].grid = dim3(p.per_xcd * kXcds);
  if (p.wave_qblocks == 1) {
    specs[0].block = dim3(Cfg8<128>::THREADS);
    if (p.tile_bufs == 4)
      specs[0].func = head_dim == 128 ? reinterpret_cast<const void*>(&chunk_attn8_kernel<128, 4>)
                                      : reinterpret_cast<const void*>(&chunk_attn8_kernel<64, 4>);
    else
      specs[0].func = head_dim == 128 ? reinterpret_cast<const void*>(&chunk_attn8_kernel<128, 3>)
                                      : reinterpret_cast<const void*>(&chunk_attn8_kernel<64, 3>);
  } else {
    specs[0].block = dim3(Cfg<128, 2>::THREADS);
    specs[0].func = head_dim == 128 ? reinterpret_cast<const void*>(&chunk_attn_kernel<128, 2>)
                                    : reinterpret_cast<const void*>(&chunk_attn_kernel<64, 2>);
  }
  if (p.nsplit == 1) return 1;
  const int64_t threads = (int64_t)p.nb * p.nq * p.hq * (head_dim / 8);
  specs[1].grid = dim3((unsigned)((threads + 255) / 256));
  specs[1].block = dim3(256);
  specs[1].func = head_dim == 128 ? reinterpret_cast<const void*>(&attn_combine_kernel<128>)
                                  : reinterpret_cast<const void*>(&attn_combine_kernel<64>);
  return 2;
}

}  // namespace wm
