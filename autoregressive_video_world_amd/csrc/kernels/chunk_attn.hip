// Block-causal chunk attention over a bounded KV ring (gfx950, bf16 MFMA).
//
// What it computes (Cosmos3-H-Dreams model card, "Model Architecture":
// block-causal student with a KV cache; AlpaDreams GTC write-up, section VII:
// a new frame is predicted from the denoised earlier frames and the noisy
// current one): for each query of the current chunk, softmax attention over
// the keys of the frames the rollout holds (sinks + window, from the ring
// pool) and of every frame of the chunk itself.  The visible ring slots of a
// rollout that has committed m frames are exactly slots 0 .. min(m, S+W)-1,
// so the key list is two segments: ring frames (unit row stride inside a
// slot) and the chunk (row stride Hkv*d).  Softmax is order-invariant, so
// keys are visited in slot order, never concatenated.
//
// Design (one workgroup = 8 waves, two per SIMD, covering 256 queries of one
// kv head; each wave is a "task" of 32 queries of one q head):
//  * why two waves per SIMD: one wave issues at most one vector instruction
//    every ~5 cycles (an exp every ~10), so the softmax work that goes with a
//    wave's MFMAs cannot hide under them when one wave per SIMD does both;
//    with two, the SIMD issues one wave's vector work beside the other's
//    MFMAs.  Each K or V fragment read from LDS feeds one MFMA, which the LDS
//    read rate carries;
//  * keys stream through LDS in 64-key tiles, K and V in four buffers each,
//    filled by direct global->LDS loads (global_load_lds_dwordx4).  A tile
//    is stored column-major: 16-byte column c of all 64 key rows is one
//    contiguous 1 KB run (column pitch 1088 B), so one wave-wide load fills
//    one column with lane = key row and every lane forms one row address per
//    tile.  Keys past the end are clamped to the last key and masked out of
//    the softmax;
//  * S^T = K * Q^T on v_mfma_f32_32x32x16_bf16 (A = K fragment from LDS,
//    B = Q^T held in registers for the whole kernel): in the 32x32
//    accumulator layout each lane owns one query column and 16 keys, so the
//    row max and row sum need one cross-half exchange (v_permlane32_swap);
//  * O^T += V^T * P^T on the same MFMA: P^T comes straight from the S^T
//    accumulator (exp2, cvt_pk_bf16); the row sum adds the fp32
//    exponentials.  V^T operands are read with ds_read_b64_tr_b16: in each
//    16-lane group, lane j receives element j%4 of the 8-byte chunks read by
//    lanes j/4, j/4+4, j/4+8, j/4+12, so when lane L reads key row
//    kbase + L/4 at dims dbase + 4*(L%4), lane j gets V[kbase .. kbase+3]
//    [dbase + j] -- four consecutive keys of one dim, exactly the keys the
//    S^T accumulator layout gives that lane's P;
//  * 32-key sub-tile pipeline, scheduled by hand: in sub-step j the matrix
//    cores alternate S(j+1) = K Q^T and O^T += V(j-1)^T P(j-1)^T, one MFMA
//    per slot, while the vector ALUs form P(j); every operand fragment is
//    read from LDS eight slots before its MFMA into a ring of eight
//    registers;
//  * while a wave forms its exponentials it takes issue priority over the
//    other wave of its SIMD (s_setprio), so that its softmax, the longer
//    dependent chain, is not starved by the other wave's MFMA slots;
//  * online softmax in the log2 domain with a lazy rescale: the running max
//    only moves (and O, l are rescaled) when a row's new max exceeds it by
//    more than 8 (P stays <= 2^8); a wave-uniform branch, rarely taken;
//  * GQA: the tasks of a workgroup are (32-query block, head-in-group) pairs
//    of one kv head, so a K/V tile in LDS serves every q head of the group;
//  * a key-range split (several workgroups per row block when the grid is
//    small) writes fp32 partials (O/l, m, l) in each lane's register order,
//    with device-coherent 16-byte stores; the last workgroup of a row block
//    to finish (counted with a device-scope atomic on a per-ring counter that
//    it resets) reads them back the same way and merges by log-sum-exp, all
//    inside the one launch.
// This file is compiled with -fno-honor-nans (max without NaN quieting):
// the softmax never produces NaN from finite inputs; -inf is still honoured.
#include "../wm_internal.hpp"

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
constexpr int kBufs = 4;               // LDS buffers of K and of V

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

// Split partials are exchanged between workgroups that may run on different
// XCDs, whose L2 caches are not coherent with each other.  They move with
// 16-byte buffer loads and stores that carry the agent-scope coherence bit
// (sc1), the encoding the compiler itself gives agent-scope atomic loads
// and stores: such accesses are coherent across the device without any L2
// writeback or invalidation.  Ordering: each wave waits for its stores to
// complete (vmcnt 0) before the barrier that precedes the workgroup's
// arrival atomic, and the merging workgroup issues its loads only after its
// own atomic returned -- release and acquire for these accesses, without the
// whole-L2 writeback and invalidation a fence over plain accesses costs.
// A descriptor covers one wave's block, so its base must be wave-uniform
// (taken from the first active lane).  (m, l) pairs move as two 4-byte
// accesses: this compiler's 8-byte buffer-load builtin returns its first
// word in both halves.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kSc1 = 16;  // cache-policy operand bit for sc1
__device__ __forceinline__ __amdgpu_buffer_rsrc_t wave_rsrc(const void* base, int bytes);
__device__ __forceinline__ void store_ml(__amdgpu_buffer_rsrc_t r, int lane32, float m, float l) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, m), r, lane32 * 8, 0, kSc1);
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, l), r, lane32 * 8 + 4, 0, kSc1);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t wave_rsrc(const void* base, int bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint64_t u = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) << 32) |
                     (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(u), 0, bytes, 0x00020000);
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

template <int HD>
struct Cfg {
  static constexpr int WAVES = 8;
  static constexpr int THREADS = WAVES * 64;
  static constexpr int NDC = HD / 16;             // QK MFMAs per sub-tile
  static constexpr int NDB = HD / 32;             // 32-row d blocks of O^T
  static constexpr int NCOL = HD / 8;             // 16-byte columns per key row
  static constexpr int COLS_PER_WAVE = NCOL / WAVES;
  static constexpr int TILE_BYTES = NCOL * kColPitch;
  static_assert(COLS_PER_WAVE >= 1, "every wave fills at least one column");
};

template <int HD>
__global__ __launch_bounds__(512, 1) void chunk_attn_kernel(const AttnParams p) {
  using C = Cfg<HD>;
  constexpr int NBUF = kBufs;
  // Distinct LDS objects: a read of one buffer provably never aliases a DMA
  // still writing another, so reads do not wait for every pending DMA.
  __shared__ __attribute__((aligned(16))) uint8_t k0s[C::TILE_BYTES], k1s[C::TILE_BYTES], k2s[C::TILE_BYTES],
      k3s[C::TILE_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t v0s[C::TILE_BYTES], v1s[C::TILE_BYTES], v2s[C::TILE_BYTES],
      v3s[C::TILE_BYTES];
  static_assert(kBufs == 4, "four named buffers");
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
  // split partials: per (split, task) a block of 32 x HD floats in the
  // lanes' own register order, and 32 (m, l) pairs
  const int64_t n_tasks = (int64_t)p.nb * p.hq * p.nqb;
  const int64_t task_id = ((int64_t)bi * p.hq + h) * p.nqb + qblk;
  // O rows to the output in bf16: lane (l32, hi) holds query q0 + l32 at
  // dims db*32 + ii*8 + hi*4 .. +4 in acc[db][ii*4 ..].
  auto write_out = [&](const f32x16 (&acc)[C::NDB], float inv) __attribute__((always_inline)) {
    const int q = q0 + l32;
    if (q >= p.nq) return;
    uint16_t* dst = p.out + (((int64_t)b * p.nq + q) * p.hq + h) * HD;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int d = db * 32 + ii * 8 + hi * 4;
        *reinterpret_cast<uint2*>(dst + d) =
            make_uint2(pack_bf16(acc[db][ii * 4 + 0] * inv, acc[db][ii * 4 + 1] * inv),
                       pack_bf16(acc[db][ii * 4 + 2] * inv, acc[db][ii * 4 + 3] * inv));
      }
  };

  if (n_local <= 0) {
    // A key-range split past the end of a short rollout's keys (ragged
    // batch): an empty partial (sum 0) for the merge.
    if (has_task && hi == 0)
      store_ml(wave_rsrc(p.part_ml + (split * n_tasks + task_id) * 64, 256), l32, -INFINITY, 0.f);
  } else {

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
      // While a wave forms its exponentials (its longest-latency vector
      // work) it has issue priority over the other wave of its SIMD.
      if (i % (NS / NE) == NS / NE - 1) {
        __builtin_amdgcn_s_setprio(1);
        exp_unit(i / (NS / NE));
        __builtin_amdgcn_s_setprio(0);
      }
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
  // u+NBUF-2 may then be in flight at the next barrier).
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
                         tile_barrier<NDMA>();
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
    tile_steps(u + 3, std::integral_constant<int, 3>{});
  }
  // The remaining tiles, each with its phase (u % NBUF).
  if (u < n_local) tile_steps(u++, std::integral_constant<int, 0>{});
  if (u < n_local) tile_steps(u++, std::integral_constant<int, 1>{});
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

  // ---- this task's result: O / l, or the split partial (O / l, m, l) -----
  const float l_tot = xhalf_sum(l_run);
  if (has_task) {
    const float inv = 1.0f / l_tot;
    if (p.nsplit == 1) {
      write_out(oacc, inv);
    } else {
      const auto ro = wave_rsrc(p.part_o + (split * n_tasks + task_id) * (32 * HD), 32 * HD * 4);
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const float4 v = make_float4(oacc[db][ii * 4 + 0] * inv, oacc[db][ii * 4 + 1] * inv,
                                       oacc[db][ii * 4 + 2] * inv, oacc[db][ii * 4 + 3] * inv);
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), ro, ((db * 4 + ii) * 64 + lane) * 16,
                                                 0, kSc1);
        }
      if (hi == 0) store_ml(wave_rsrc(p.part_ml + (split * n_tasks + task_id) * 64, 256), l32, m_run, l_tot);
    }
  }
  }  // n_local > 0
  if (p.nsplit == 1) return;

  // ---- key-range merge: the last of the row block's splits to arrive ------
  // Every wave waits for its partial stores to complete before the barrier;
  // then one atomic counts the workgroup's arrival.  The last arrival resets
  // the counter (every split of this launch has counted) and merges: weights
  // l_s * 2^(m_s - M) over the splits with keys, each lane reading back
  // exactly the registers it would hold for its own split.
  __shared__ int merge_here;
  wait_vmcnt<0>();
  __syncthreads();
  if (tid == 0) {
    int* cnt = p.counters + ((int64_t)bi * p.hkv + g) * p.wg_per_bg + wgi;
    const int last = atomicAdd(cnt, 1) == p.nsplit - 1;
    if (last) atomicExch(cnt, 0);
    merge_here = last;
  }
  __syncthreads();
  if (!merge_here || !has_task) return;
  float ms[kAttnMaxSplit], ls[kAttnMaxSplit];
#pragma unroll
  for (int sp = 0; sp < kAttnMaxSplit; ++sp) {
    ms[sp] = -INFINITY;
    ls[sp] = 0.f;
    if (sp < p.nsplit) {
      const auto rml = wave_rsrc(p.part_ml + (sp * n_tasks + task_id) * 64, 256);
      ms[sp] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rml, l32 * 8, 0, kSc1));
      ls[sp] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rml, l32 * 8 + 4, 0, kSc1));
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int sp = 0; sp < kAttnMaxSplit; ++sp)
    if (ls[sp] > 0.f) M = fmaxf(M, ms[sp]);
  f32x16 acc[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) acc[db] = f32x16{};
  float wsum = 0.f;
#pragma unroll 1
  for (int sp = 0; sp < p.nsplit; ++sp) {
    if (!(ls[sp] > 0.f)) continue;
    const float w = ls[sp] * __builtin_amdgcn_exp2f(ms[sp] - M);
    const auto ro = wave_rsrc(p.part_o + (sp * n_tasks + task_id) * (32 * HD), 32 * HD * 4);
    float4 v[C::NDB * 4];
#pragma unroll
    for (int j = 0; j < C::NDB * 4; ++j)
      v[j] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(ro, (j * 64 + lane) * 16, 0, kSc1));
#pragma unroll
    for (int j = 0; j < C::NDB * 4; ++j) {
      acc[j / 4][(j % 4) * 4 + 0] += w * v[j].x;
      acc[j / 4][(j % 4) * 4 + 1] += w * v[j].y;
      acc[j / 4][(j % 4) * 4 + 2] += w * v[j].z;
      acc[j / 4][(j % 4) * 4 + 3] += w * v[j].w;
    }
    wsum += w;
  }
  write_out(acc, 1.0f / wsum);
}

}  // namespace

int chunk_attn_specs(AttnParams& p, int head_dim, LaunchSpec specs[2]) {
  if (head_dim != 128 && head_dim != 64) return 0;
  p.n_wg = p.nb * p.hkv * p.wg_per_bg * p.nsplit;
  p.per_xcd = (p.n_wg + kXcds - 1) / kXcds;
  specs[0].grid = dim3(p.per_xcd * kXcds);
  specs[0].block = dim3(Cfg<128>::THREADS);
  specs[0].func = head_dim == 128 ? reinterpret_cast<const void*>(&chunk_attn_kernel<128>)
                                  : reinterpret_cast<const void*>(&chunk_attn_kernel<64>);
  return 1;
}

}  // namespace wm
