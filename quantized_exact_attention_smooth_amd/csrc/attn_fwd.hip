// Fused quantized attention main loop for gfx950 (CDNA4).
//
// Experiment Log (vortex_exact_attention): "Phase 0 Import And Verification"
// lists QK traversal, online softmax, FP8 V/P, two-level PV accumulation,
// final conversion and ragged tails; "Phase 1 State-Ownership Decision" fixes
// strict tile order, exact FP8 score bytes and per-tile RO rescaling; "Phase 2A
// VEA-B Capability Decision" stages K and V in two 8 KiB slots (64 keys x 128
// bytes each). The SM121 ten-warp role split is prior art; this kernel is laid
// out for 64-wide waves and CDNA4 matrix cores instead:
//
//  * workgroup = 4 waves = 128 query rows of one (b, h); wave w owns 32 rows.
//    Grid order puts the heaviest causal tiles first; consecutive blocks walk
//    the heads, so with B*H a multiple of 8 every tile of a head runs on the
//    same XCD (blocks are dealt to the 8 XCDs round-robin) and shares its L2.
//  * per 64-key epoch the K tile (64 x D int8) and V tile (D x 64 e4m3, keys
//    contiguous) are copied straight from global memory into LDS (two slots
//    each; K(e+2) and V(e) fill while epoch e computes), no staging registers.
//  * QK: S^T = K . Q^T with v_mfma_i32_32x32x32_i8 (A = K rows from LDS,
//    B = Q codes held in registers for the whole kernel). The K rows are
//    loaded in a permuted order so that each lane ends with 32 consecutive
//    keys of ONE query: lane (h, q) holds S[q][32h .. 32h+31].
//  * softmax: the row max is taken on the exact int32 scores (the dequant
//    factor sq*sk*sm_scale*log2e is positive), then one cross-half exchange;
//    p = exp2(fma(S, c, -m)) in fp32; the row sum stays a per-half partial
//    until the epilogue.
//  * P -> E4M3 in registers; that register block IS the B operand of the PV
//    matrix-core step (O^T = V^T . P^T, v_mfma_f32_32x32x64_f8f6f4), so P
//    never goes through LDS, and each lane's outputs belong to its own query.
//  * two-level PV: RO *= alpha (skipped when no row max of the wave moved,
//    i.e. alpha == 1 in every lane), then the matrix core reduces the epoch's
//    64 keys in fp32 (inner level) and adds the result into RO, its C
//    operand (outer level).
//  * epilogue: r = 1/l (IEEE divide), out = bf16(RO * r * sv[c]) for rows < Lq.
//  * instantiations: TRACE records one wave's per-epoch state (debug).
#include <limits.h>

#include <type_traits>

#include "sage_device.h"
#include "sage_launch.h"

namespace sage {

// ---------------------------------------------------------------- staging

// Copy one K tile (64 x D int8, row-major) into LDS with the read swizzle.
template <int D, int NT>
struct KStage {
  static constexpr int kChunks = kBlock * D / 16 / NT;
  v4i r[kChunks];
  __device__ __forceinline__ void load(const int8_t* __restrict__ src) {
#pragma unroll
    for (int j = 0; j < kChunks; ++j)
      r[j] = *reinterpret_cast<const v4i*>(src + 16 * (threadIdx.x + NT * j));
  }
  __device__ __forceinline__ void store(uint8_t* lds) const {
#pragma unroll
    for (int j = 0; j < kChunks; ++j) {
      const int g = threadIdx.x + NT * j;
      *reinterpret_cast<v4i*>(lds + k_lds_off<D>(g / (D / 16), g % (D / 16))) = r[j];
    }
  }
};

// Copy one V tile (D x 64 e4m3, keys contiguous) into LDS with the swizzle.
template <int D, int NT>
struct VStage {
  static constexpr int kChunks = D * kBlock / 16 / NT;
  v4i r[kChunks];
  __device__ __forceinline__ void load(const uint8_t* __restrict__ src) {
#pragma unroll
    for (int j = 0; j < kChunks; ++j)
      r[j] = *reinterpret_cast<const v4i*>(src + 16 * (threadIdx.x + NT * j));
  }
  __device__ __forceinline__ void store(uint8_t* lds) const {
#pragma unroll
    for (int j = 0; j < kChunks; ++j) {
      const int g = threadIdx.x + NT * j;
      *reinterpret_cast<v4i*>(lds + v_lds_off(g / 4, g % 4)) = r[j];
    }
  }
};

// ------------------------------------------------------------ QK, codecs

// Exact int32 scores of one 64-key epoch for the 32 queries of a wave.
// lane = (h, q): acc_m[r] = S[q][32h + 16m + r] for m = 0, 1.
template <int D>
__device__ __forceinline__ void qk_epoch(const uint8_t* lk, const v4i* qreg, int lane, v16i& acc0,
                                         v16i& acc1) {
  const int row = lane & 31, h = lane >> 5;
  const int key0 = qk_row_key(row, 0), key1 = qk_row_key(row, 1);
  acc0 = v16i{};
  acc1 = v16i{};
#pragma unroll
  for (int s = 0; s < D / 32; ++s) {
    const v4i a0 = *reinterpret_cast<const v4i*>(lk + k_lds_off<D>(key0, 2 * s + h));
    const v4i a1 = *reinterpret_cast<const v4i*>(lk + k_lds_off<D>(key1, 2 * s + h));
    acc0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, qreg[s], acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, qreg[s], acc1, 0, 0, 0);
  }
}

// Maximum of one lane's 32 scores (v_max3 chain).
__device__ __forceinline__ int row_max32(const int (&x)[32]) {
  int mx = max(max(x[0], x[1]), x[2]);
#pragma unroll
  for (int t = 3; t < 31; t += 2) mx = max(max(mx, x[t]), x[t + 1]);
  return max(mx, x[31]);
}

// Four fp32 values -> four E4M3FN bytes (x0 in the low byte), hardware
// conversion, round to nearest even.
__device__ __forceinline__ int pack4_fp8(float x0, float x1, float x2, float x3) {
  // Both halves of the word are written, so its prior contents are irrelevant;
  // an empty asm output stands for them and saves a register clear.
  int w;
  asm volatile("" : "=v"(w));
  w = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, w, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, w, true);
}

// Two fp32 values -> two bf16 (x0 in the low half), round to nearest even.
__device__ __forceinline__ uint32_t pack2_bf16(float x0, float x1) {
  __bf16 b0 = (__bf16)x0, b1 = (__bf16)x1;
  return (uint32_t)__builtin_bit_cast(uint16_t, b0) | ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
}

// Direct global -> LDS copies (no staging registers) through buffer loads:
// a wave copies 64 consecutive 16-byte LDS chunks per instruction; each lane
// fetches the global chunk that the swizzled layout places at its LDS
// position. In the buffer form (rather than global_load_lds) the per-lane
// offsets stay loop-invariant and the tile offset is a scalar, so a fill
// costs no per-epoch address arithmetic, and the compiler can wait for the
// main loop's LDS reads one by one while copies are in flight. rsrc spans one
// head's tiles; tile is the byte offset of the tile in it.
typedef __attribute__((address_space(3))) void* lds_ptr_t;
constexpr int kRawBufferFlags = 0x00020000;  // untyped 32-bit access
template <int D>
__device__ __forceinline__ void k_tile_to_lds(__amdgpu_buffer_rsrc_t rsrc, int tile, uint8_t* lds, int w,
                                              int lane) {
  constexpr int kPerWave = kBlock * D / 16 / 4 / 64;  // instructions per wave
#pragma unroll
  for (int j = 0; j < kPerWave; ++j) {
    const int p0 = (w * kPerWave + j) * 64;
    const int p = p0 + lane;
    const int key = p / (D / 16), pc = p % (D / 16);
    const int c = (k_lds_off<D>(key, pc) - key * D) >> 4;  // logical chunk at physical pc
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr_t)(lds + 16 * p0), 16, key * D + 16 * c, tile, 0, 0);
  }
}
template <int D>
__device__ __forceinline__ void v_tile_to_lds(__amdgpu_buffer_rsrc_t rsrc, int tile, uint8_t* lds, int w,
                                              int lane) {
  constexpr int kPerWave = D * kBlock / 16 / 4 / 64;
#pragma unroll
  for (int j = 0; j < kPerWave; ++j) {
    const int p0 = (w * kPerWave + j) * 64;
    const int p = p0 + lane;
    const int row = p / 4, pc = p % 4;
    const int c = (v_lds_off(row, pc) - row * 64) >> 4;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr_t)(lds + 16 * p0), 16, row * 64 + 16 * c, tile, 0, 0);
  }
}

// Pairwise exchange between lane halves: returns f(own, other) in every lane.
// v_permlane32_swap with the same value in both operands leaves, per lane,
// its own value in one result and the other half's value in the other.
__device__ __forceinline__ int half_max(int x) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return max((int)r[0], (int)r[1]);
}
__device__ __forceinline__ float half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}

// s_waitcnt with lgkmcnt(0) and the vector-memory and export counters left
// at their maxima: LDS operations done, global loads and fills still in flight.
constexpr int kWaitLgkmOnly = 0xC07F;

// ------------------------------------------------------------ main kernel
//
// Software pipeline per wave, one body per epoch e:
//   1. start the LDS fills of K(e+2) and V(e) (buffers freed by the last
//      barrier);
//   2. softmax of epoch e (VALU) from the accumulators filled one body ago;
//      between groups of its exp2 evaluations the wave issues the QK
//      matrix-core steps of epoch e+1 (into the other accumulator set) and
//      the PV steps of epoch e-1 (RO += V(e-1)^T . P(e-1)^T);
//   3. RO *= alpha(e) when some row's running max moved (RO now holds the
//      epochs before e, exactly as in an undeferred order);
//   4. wait for this body's LDS fills, barrier.
// Every matrix-core step thus runs while the wave keeps issuing softmax work,
// and its result is consumed one body later. After the last body the PV step
// of the wave's final epoch completes RO.

template <int D, bool CAUSAL, bool TRACE>
__global__ __launch_bounds__(kThreads) void attn_fwd_kernel(AttnArgs a) {
  // Four separate LDS objects (not one array) so that the compiler can tell
  // the in-flight direct fills apart from the buffers being read.
  __shared__ __attribute__((aligned(16))) uint8_t s_k0[kBlock * D];
  __shared__ __attribute__((aligned(16))) uint8_t s_k1[kBlock * D];
  __shared__ __attribute__((aligned(16))) uint8_t s_v0[D * kBlock];
  __shared__ __attribute__((aligned(16))) uint8_t s_v1[D * kBlock];

  const int BH = a.B * a.H;
  const int tile = TRACE ? a.trace_tile : a.n_qtiles - 1 - (int)(blockIdx.x / BH);
  const long bh = TRACE ? (long)a.trace_bh : (long)(blockIdx.x % BH);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int h = lane >> 5, ql = lane & 31;
  const int q0 = tile * kQTile;
  const int wrow0 = q0 + 32 * w;
  const int qrow = wrow0 + ql;
  const int off = a.Lkv - a.Lq;

  // Epochs the workgroup stages, and the epochs this wave computes.
  int n_ep = a.nkb;
  if (CAUSAL) {
    const int x = min(a.Lq - 1, q0 + kQTile - 1) + off;
    n_ep = x < 0 ? 0 : min(a.nkb, x / kBlock + 1);
  }
  const bool wave_on = wrow0 < a.Lq;
  int w_ep = 0;
  if (wave_on) {
    const int x = CAUSAL ? min(a.Lq - 1, wrow0 + 31) + off : a.Lkv - 1;
    w_ep = x < 0 ? 0 : min(a.nkb, x / kBlock + 1);
  }
  // Keys beyond lim (this lane's last visible key) are masked. An epoch needs
  // the mask only when it reaches past the wave's smallest limit w_lim.
  const int lim = CAUSAL ? min(qrow + off, a.Lkv - 1) : a.Lkv - 1;
  const int w_lim = CAUSAL ? min(wrow0 + off, a.Lkv - 1) : a.Lkv - 1;

  // Buffer resources over this head's K and V tiles (the host bounds a head's
  // tiles below 2^31 bytes, so offsets and the record count fit).
  const int head_bytes = a.nkb * kBlock * D;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.k_i8 + bh * (long)head_bytes), (short)0, head_bytes, kRawBufferFlags);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.v_fp8 + bh * (long)head_bytes), (short)0, head_bytes, kRawBufferFlags);
  // k_scale is read-only for the kernel's lifetime: scalar (constant-space) loads.
  const __attribute__((address_space(4))) float* ksh =
      (const __attribute__((address_space(4))) float*)(a.k_scale + bh * a.nkb);
  // The first two K fills start before the Q codes are loaded, so that the
  // latencies overlap (V(0) is filled by the first body).
  if (n_ep > 0) {
    k_tile_to_lds<D>(krs, 0, s_k0, w, lane);
    if (n_ep > 1) k_tile_to_lds<D>(krs, kBlock * D, s_k1, w, lane);
  }

  v4i qreg[D / 32];
  const int8_t* qh = a.q_i8 + bh * (long)a.nqb * kBlock * D;
#pragma unroll
  for (int s = 0; s < D / 32; ++s)
    qreg[s] = (qrow < a.Lq) ? *reinterpret_cast<const v4i*>(qh + (long)qrow * D + 32 * s + 16 * h) : v4i{};
  const float sq = wave_on ? a.q_scale[bh * a.nqb + wrow0 / kBlock] : 0.0f;
  const float cq = sq * a.scale_log2;

  float m = -INFINITY, l = 0.0f;
  v16f ro[D / 32];
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb) ro[cb] = v16f{};

  v16i sa0 = {}, sa1 = {}, sb0 = {}, sb1 = {};
  v8i pba = {}, pbb = {};  // E4M3 P of even / odd epochs
  // The first body's deferred PV step ("epoch -1") multiplies a zero P with
  // s_v1; zeroing s_v1 keeps garbage (NaN codes) out of that product, so it
  // adds exactly +0 to RO.
#pragma unroll
  for (int i = threadIdx.x; i < D * kBlock / 16; i += kThreads) reinterpret_cast<v4i*>(s_v1)[i] = v4i{};
  __builtin_amdgcn_s_waitcnt(0);  // the first K fills (issued above) have landed
  __syncthreads();
  if (w_ep > 0) qk_epoch<D>(s_k0, qreg, lane, sa0, sa1);
  // The first epoch refills s_k0 with K(2): every wave must have read K(0) first.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // A operand of one PV step: channels 32 cb + ql, this lane's 32 keys.
  auto pv_frag = [&](const uint8_t* vb, int cb) -> v8i {
    const int ch = 32 * cb + ql;
    const v4i lo = *reinterpret_cast<const v4i*>(vb + v_lds_off(ch, 2 * h));
    const v4i hi = *reinterpret_cast<const v4i*>(vb + v_lds_off(ch, 2 * h + 1));
    return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  };
  // Whole PV step of one epoch (used where nothing is left to interleave).
  auto pv_step = [&](const uint8_t* vb, const v8i& pb) {
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb)
      ro[cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(pv_frag(vb, cb), pb, ro[cb], 0, 0, 0, 127, 0, 127);
  };
  // Trace checkpoint: RO after the PV step of epoch ep.
  auto trace_ro = [&](int ep) {
    if (TRACE && w == a.trace_wave) {
      float* rt = a.tr_ro + ((long)ql * a.nkb + ep) * D;
#pragma unroll
      for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) rt[32 * cb + 8 * (r / 4) + 4 * h + r % 4] = ro[cb][r];
    }
  };

  // One pipelined epoch: `cur` holds S(e), `nxt` receives S(e+1); `pbp` is
  // P(e-1), whose PV step runs in this body, `pbn` receives P(e). The epoch's
  // parity is a template argument so every LDS buffer is a fixed object.
  auto body = [&](auto parity, const int e, const v16i& cur0, const v16i& cur1, v16i& nxt0, v16i& nxt1,
                  const v8i& pbp, v8i& pbn) {
    constexpr int P = decltype(parity)::value;
    uint8_t* k_fill = P ? s_k1 : s_k0;   // K(e+2) replaces K(e)
    uint8_t* k_next = P ? s_k0 : s_k1;   // K(e+1)
    uint8_t* v_prev = P ? s_v0 : s_v1;   // V(e-1)
    uint8_t* v_fill = P ? s_v1 : s_v0;   // V(e) replaces V(e-2)
    if (e + 2 < n_ep) k_tile_to_lds<D>(krs, (e + 2) * kBlock * D, k_fill, w, lane);
    v_tile_to_lds<D>(vrs, e * D * kBlock, v_fill, w, lane);
    // A wave whose last epoch was e-1 (the workgroup stages more for the
    // other waves) runs one more body: every key of epoch e is past each of
    // its rows' limits, so p = 0, alpha = 1 and m, l stay, and the body only
    // completes the PV step of epoch e-1.
    if (e < w_ep || (e == w_ep && e > 0)) {
      // First K fragments of epoch e+1, read ahead of the row max.
      const int key0 = qk_row_key(ql, 0), key1 = qk_row_key(ql, 1);
      const v4i kf0 = *reinterpret_cast<const v4i*>(k_next + k_lds_off<D>(key0, h));
      const v4i kf1 = *reinterpret_cast<const v4i*>(k_next + k_lds_off<D>(key1, h));
      __builtin_amdgcn_sched_barrier(0);
      // log2-domain score per unit of the int32 accumulator
      const float c = cq * ksh[e];
      int x[32];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        x[r] = cur0[r];
        x[16 + r] = cur1[r];
      }
      const bool masked = kBlock * e + kBlock - 1 > w_lim;  // wave-uniform
      const int dlim = lim - (kBlock * e + 32 * h);          // x[t] visible iff t <= dlim
      // Hidden scores are left in x (their p is zeroed below) and only kept
      // out of the row max, so the unmasked path carries no select or copy.
      int mx;
      if (masked) {
        asm volatile("" ::: "memory");  // keeps the selects inside this branch
        int y[32];
#pragma unroll
        for (int t = 0; t < 32; ++t) y[t] = (t > dlim) ? INT_MIN : x[t];
        mx = row_max32(y);
      } else {
        mx = row_max32(x);
      }
      mx = half_max(mx);
      const float mt = (kBlock * e <= lim) ? (float)mx * c : -INFINITY;
      const float m_new = fmaxf(m, mt);
      const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m - m_use);
      const bool moved = __builtin_amdgcn_ballot_w64(m_new != m) != 0;  // wave-uniform

      // p = exp2(S c - m), with matrix-core steps spread through it so that
      // each runs while this wave keeps issuing VALU work (a burst would stall
      // the wave on each step's dependent successor). Per 32 channels, four
      // slots: QK of epoch e+1 into each accumulator, then the PV step of
      // epoch e-1 (RO += V(e-1)^T . P(e-1)^T, deferred one body so that it
      // overlaps this softmax; same operands and order as an undeferred step,
      // so RO then holds epochs < e and the rescale below applies alpha(e)
      // before the PV step of epoch e adds into it), then VALU only. On the
      // wave's last epoch the QK steps read a stale K buffer and go unused.
      constexpr int kG = D / 32;
      constexpr int kPer = 32 / (4 * kG);  // p values per slot
      // Each operand is read from LDS right after the step that frees its
      // registers, two or three slots ahead of its own step.
      float p[32];
      v4i ka = kf0, kb = kf1;
      v8i av;
#pragma unroll
      for (int j = 0; j < 4 * kG; ++j) {
        const int st = j >> 2, slot = j & 3;
        if (slot == 0) {
          if (st == 0) av = pv_frag(v_prev, 0);
          nxt0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(ka, qreg[st], st ? nxt0 : v16i{}, 0, 0, 0);
        } else if (slot == 1) {
          if (st + 1 < kG) ka = *reinterpret_cast<const v4i*>(k_next + k_lds_off<D>(key0, 2 * (st + 1) + h));
          nxt1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(kb, qreg[st], st ? nxt1 : v16i{}, 0, 0, 0);
        } else if (slot == 2) {
          if (st + 1 < kG) kb = *reinterpret_cast<const v4i*>(k_next + k_lds_off<D>(key1, 2 * (st + 1) + h));
          ro[st] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, pbp, ro[st], 0, 0, 0, 127, 0, 127);
        } else {
          if (st + 1 < kG) av = pv_frag(v_prev, st + 1);
        }
#pragma unroll
        for (int t = kPer * j; t < kPer * (j + 1); ++t)
          p[t] = __builtin_amdgcn_exp2f(__builtin_fmaf((float)x[t], c, -m_use));
        __builtin_amdgcn_sched_barrier(0);
      }
      if (masked) {
        asm volatile("" ::: "memory");
#pragma unroll
        for (int t = 0; t < 32; ++t) p[t] = (t > dlim) ? 0.0f : p[t];
      }
      float ps = p[0];
#pragma unroll
      for (int t = 1; t < 32; ++t) ps += p[t];
      l = __builtin_fmaf(l, alpha, ps);
#pragma unroll
      for (int d = 0; d < 8; ++d) pbn[d] = pack4_fp8(p[4 * d], p[4 * d + 1], p[4 * d + 2], p[4 * d + 3]);
      if (e > 0) trace_ro(e - 1);

      // Per-tile rescale; a no-op (alpha == 1 in every lane) when no row max moved.
      if (moved) {
#pragma unroll
        for (int cb = 0; cb < D / 32; ++cb) ro[cb] *= alpha;
      }
      m = m_new;
      if (TRACE && w == a.trace_wave && e < w_ep) {
        // Checkpoints of this epoch: m (log2 domain), l, alpha, P8 (RO follows
        // with the PV step in the next body).
        const float lt = half_sum(l);
        if (h == 0) {
          float* st = a.tr_stats + ((long)ql * (a.nkb + 1) + e) * 4;
          st[0] = m;
          st[1] = lt;
          st[2] = alpha;
          st[3] = 0.0f;
        }
        uint32_t* p8 = reinterpret_cast<uint32_t*>(a.tr_p8 + ((long)ql * a.nkb + e) * kBlock + 32 * h);
#pragma unroll
        for (int d = 0; d < 8; ++d) p8[d] = (uint32_t)pbn[d];
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  for (int e = 0; e < n_ep; e += 2) {
    body(std::integral_constant<int, 0>{}, e, sa0, sa1, sb0, sb1, pbb, pba);
    if (e + 1 < n_ep) body(std::integral_constant<int, 1>{}, e + 1, sb0, sb1, sa0, sa1, pba, pbb);
  }
  // The PV step of the last epoch, when it is this wave's (V(e) sits in
  // buffer e % 2; no fills are in flight any more).
  if (w_ep > 0 && w_ep == n_ep) {
    if ((n_ep - 1) & 1)
      pv_step(s_v1, pbb);
    else
      pv_step(s_v0, pba);
    trace_ro(n_ep - 1);
  }

  // Epilogue: the two halves of a query hold partial sums of l.
  const float lt = half_sum(l);
  const float rcp = (lt > 0.0f) ? 1.0f / lt : 0.0f;
  if (TRACE && w == a.trace_wave && h == 0) {
    float* st = a.tr_stats + ((long)ql * (a.nkb + 1) + a.nkb) * 4;
    st[0] = rcp;
    st[1] = lt;
    st[2] = 0.0f;
    st[3] = 0.0f;
  }
  if (qrow < a.Lq) {
    uint16_t* orow = a.out + (bh * a.Lq + qrow) * (long)D;
    const float* svh = a.v_scale + bh * D;
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c0 = 32 * cb + 8 * g + 4 * h;
        const float4 sv = *reinterpret_cast<const float4*>(svh + c0);
        const uint32_t w0 = pack2_bf16(ro[cb][4 * g + 0] * rcp * sv.x, ro[cb][4 * g + 1] * rcp * sv.y);
        const uint32_t w1 = pack2_bf16(ro[cb][4 * g + 2] * rcp * sv.z, ro[cb][4 * g + 3] * rcp * sv.w);
        *reinterpret_cast<uint2*>(orow + c0) = make_uint2(w0, w1);
      }
    }
  }
}

// ------------------------------------------------------------ debug kernels

// One 64x64 int32 QK tile per workgroup (2 waves = 64 queries), through the
// same staging and qk_epoch code as the main loop's first epoch (later epochs
// interleave the same MFMA steps, same operands, with the softmax).
template <int D>
__global__ __launch_bounds__(128) void qk_debug_kernel(QkDebugArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t s_k[kBlock * D];
  const int t = blockIdx.x;
  const long bh = (long)a.tiles[t][0] * a.H + a.tiles[t][1];
  const int qb = a.tiles[t][2], kb = a.tiles[t][3];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, h = lane >> 5, ql = lane & 31;
  const int qrow = qb * kBlock + 32 * w + ql;
  v4i qreg[D / 32];
  const int8_t* qh = a.q_i8 + bh * (long)a.nqb * kBlock * D;
#pragma unroll
  for (int s = 0; s < D / 32; ++s)
    qreg[s] = *reinterpret_cast<const v4i*>(qh + (long)qrow * D + 32 * s + 16 * h);
  KStage<D, 128> ks;
  ks.load(a.k_i8 + (bh * a.nkb + kb) * (long)kBlock * D);
  ks.store(s_k);
  __syncthreads();
  v16i acc0, acc1;
  qk_epoch<D>(s_k, qreg, lane, acc0, acc1);
  int32_t* o = a.acc_out + (long)t * kBlock * kBlock + (32 * w + ql) * kBlock + 32 * h;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    o[r] = acc0[r];
    o[16 + r] = acc1[r];
  }
}

__global__ __launch_bounds__(256) void codecs_debug_kernel(const float* __restrict__ x, int n,
                                                           uint8_t* __restrict__ p8,
                                                           uint16_t* __restrict__ bf) {
  const long i = 4L * ((long)blockIdx.x * blockDim.x + threadIdx.x);
  if (i >= n) return;
  float v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = (i + j < n) ? x[i + j] : 0.0f;
  const int w = pack4_fp8(v[0], v[1], v[2], v[3]);
  const uint32_t b01 = pack2_bf16(v[0], v[1]), b23 = pack2_bf16(v[2], v[3]);
  const uint32_t bb[4] = {b01 & 0xFFFFu, b01 >> 16, b23 & 0xFFFFu, b23 >> 16};
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (i + j < n) {
      p8[i + j] = (uint8_t)((uint32_t)w >> (8 * j));
      bf[i + j] = (uint16_t)bb[j];
    }
}

// ------------------------------------------------------------ launchers

template <int D, bool C, bool T>
static hipError_t launch_attn_t(const AttnArgs& a, hipStream_t stream) {
  const long blocks = T ? 1L : (long)a.n_qtiles * a.B * a.H;
  attn_fwd_kernel<D, C, T><<<dim3((unsigned)blocks), kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

template <bool T>
static hipError_t launch_attn_v(const AttnArgs& a, int D, bool causal, hipStream_t stream) {
  if (D == 128) return causal ? launch_attn_t<128, true, T>(a, stream) : launch_attn_t<128, false, T>(a, stream);
  return causal ? launch_attn_t<64, true, T>(a, stream) : launch_attn_t<64, false, T>(a, stream);
}

hipError_t launch_attn(const AttnArgs& a, int D, bool causal, hipStream_t stream) {
  return launch_attn_v<false>(a, D, causal, stream);
}
hipError_t launch_attn_trace(const AttnArgs& a, int D, bool causal, hipStream_t stream) {
  return launch_attn_v<true>(a, D, causal, stream);
}

hipError_t launch_qk_debug(const QkDebugArgs& a, int D, hipStream_t stream) {
  if (D == 128)
    qk_debug_kernel<128><<<a.n, 128, 0, stream>>>(a);
  else
    qk_debug_kernel<64><<<a.n, 128, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_codecs_debug(const float* x, int n, uint8_t* p8, uint16_t* bf16, hipStream_t stream) {
  const int groups = (n + 3) / 4;
  codecs_debug_kernel<<<(groups + 255) / 256, 256, 0, stream>>>(x, n, p8, bf16);
  return hipGetLastError();
}

}  // namespace sage
