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
//  * three workgroups per CU at D = 128 (four at D = 64): the loop keeps one
//    set of score registers and packs P as it is produced, so it fits 168
//    VGPRs and each SIMD holds three waves (four at D = 64), which cover each
//    other's matrix-core steps and stalls.
//  * per 64-key epoch the K tile (64 x D int8) and V tile (D x 64 e4m3, keys
//    contiguous) are copied straight from global memory into LDS (two slots
//    each; K(e+1) and V(e+1) fill while epoch e computes), no staging
//    registers.
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
//  * epilogue: r = 1/l (IEEE divide), out = bf16(RO * r * sv[c]) for rows < Lq,
//    with sv read into LDS at the start; a wave's 32 rows are consecutive in
//    memory, so they pass through LDS and leave as whole 16-byte chunks.
//  * instantiations: TRACE records one wave's per-epoch state (debug).
#include <limits.h>

#include <type_traits>

#include "sage_device.h"
#include "sage_launch.h"

namespace sage {

// ------------------------------------------------------------ QK, codecs

// LDS byte offsets of this lane's A-operand reads in qk_epoch: step s reads
// key qk_row_key(row, 0), chunk 2s + h at koff[s], and the key 16 rows
// further down at koff[s] + 16 D (the swizzle does not depend on key bit 4).
template <int D>
__device__ __forceinline__ void qk_offsets(int lane, int (&koff)[D / 32]) {
  const int row = lane & 31, h = lane >> 5;
  const int key0 = qk_row_key(row, 0);
#pragma unroll
  for (int s = 0; s < D / 32; ++s) koff[s] = k_lds_off<D>(key0, 2 * s + h);
}

// Exact int32 scores of one 64-key epoch for the 32 queries of a wave.
// lane = (h, q): acc_m[r] = S[q][32h + 16m + r] for m = 0, 1.
template <int D>
__device__ __forceinline__ void qk_epoch(const uint8_t* lk, const v4i* qreg, const int (&koff)[D / 32],
                                         v16i& acc0, v16i& acc1) {
  acc0 = v16i{};
  acc1 = v16i{};
#pragma unroll
  for (int s = 0; s < D / 32; ++s) {
    const v4i a0 = *reinterpret_cast<const v4i*>(lk + koff[s]);
    const v4i a1 = *reinterpret_cast<const v4i*>(lk + koff[s] + 16 * D);
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

// ------------------------------------------------------------ main kernel
//
// Per wave, one body per epoch e:
//   1. start the LDS fills of K(e+1) and V(e+1) (buffers freed by the last
//      barrier);
//   2. QK matrix-core steps of epoch e from the resident K(e);
//   3. softmax of epoch e (VALU): row max, alpha, then p in groups of four
//      keys, each group packed to E4M3 and added to the row sum at once;
//   4. RO *= alpha when some row's running max moved, then the PV step of
//      epoch e into RO;
//   5. wait for this body's LDS fills, barrier.
// A wave stalls on its own matrix-core steps; the other waves of the SIMD
// issue VALU work meanwhile.

// Waves per SIMD the register budget is set for: 3 at D = 128 (<= 168
// VGPRs), 4 at D = 64 (<= 128); the trace build stores extra state and runs
// one workgroup, so it keeps the compiler's default.
template <int D, bool TRACE>
constexpr int kWavesPerSimd = TRACE ? 1 : (D == 64 ? 4 : 3);

template <int D, bool CAUSAL, bool TRACE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kWavesPerSimd<D, TRACE>)))
void attn_fwd_kernel(AttnArgs a) {
  // Four separate LDS objects (not one array) so that the compiler can tell
  // the in-flight direct fills apart from the buffers being read.
  __shared__ __attribute__((aligned(16))) uint8_t s_k0[kBlock * D];
  __shared__ __attribute__((aligned(16))) uint8_t s_k1[kBlock * D];
  __shared__ __attribute__((aligned(16))) uint8_t s_v0[D * kBlock];
  __shared__ __attribute__((aligned(16))) uint8_t s_v1[D * kBlock];
  // The head's V channel scales, read at the start so that the epilogue does
  // not wait for a global load.
  __shared__ __attribute__((aligned(16))) float s_sv[D];

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
  // The first K and V fills start before the Q codes are loaded, so that the
  // latencies overlap.
  if (n_ep > 0) {
    k_tile_to_lds<D>(krs, 0, s_k0, w, lane);
    v_tile_to_lds<D>(vrs, 0, s_v0, w, lane);
  }

  v4i qreg[D / 32];
  const int8_t* qh = a.q_i8 + bh * (long)a.nqb * kBlock * D;
#pragma unroll
  for (int s = 0; s < D / 32; ++s)
    qreg[s] = (qrow < a.Lq) ? *reinterpret_cast<const v4i*>(qh + (long)qrow * D + 32 * s + 16 * h) : v4i{};
  const float sq = wave_on ? a.q_scale[bh * a.nqb + wrow0 / kBlock] : 0.0f;
  const float cq = sq * a.scale_log2;
  if (threadIdx.x < D) s_sv[threadIdx.x] = a.v_scale[bh * D + threadIdx.x];

  // The QK read offsets are computed once; the empty asm keeps the compiler
  // from rebuilding them from their parts in every epoch (four VALU adds).
  int koff[D / 32];
  qk_offsets<D>(lane, koff);
#pragma unroll
  for (int s = 0; s < D / 32; ++s) asm volatile("" : "+v"(koff[s]));

  float m = -INFINITY, l = 0.0f;
  v16f ro[D / 32];
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb) ro[cb] = v16f{};
  __builtin_amdgcn_s_waitcnt(0);  // the first fills (issued above) have landed
  __syncthreads();

  // p = exp2(S c - m) for 4 consecutive keys of this lane, packed to E4M3
  // and added to the row sum in key order.
  auto p4 = [&](const int (&x)[32], int d, float c, float m_use, float& ps) -> int {
    float p[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) p[j] = __builtin_amdgcn_exp2f(__builtin_fmaf((float)x[4 * d + j], c, -m_use));
#pragma unroll
    for (int j = 0; j < 4; ++j) ps = (d == 0 && j == 0) ? p[0] : ps + p[j];
    return pack4_fp8(p[0], p[1], p[2], p[3]);
  };
  auto p4_masked = [&](const int (&x)[32], int d, float c, float m_use, int dlim, float& ps) -> int {
    float p[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float e = __builtin_amdgcn_exp2f(__builtin_fmaf((float)x[4 * d + j], c, -m_use));
      p[j] = (4 * d + j > dlim) ? 0.0f : e;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) ps = (d == 0 && j == 0) ? p[0] : ps + p[j];
    return pack4_fp8(p[0], p[1], p[2], p[3]);
  };

  // One epoch. The epoch's parity is a template argument so every LDS buffer
  // is a fixed object.
  auto body = [&](auto parity, const int e) {
    constexpr int P = decltype(parity)::value;
    uint8_t* k_cur = P ? s_k1 : s_k0;   // K(e)
    uint8_t* v_cur = P ? s_v1 : s_v0;   // V(e)
    uint8_t* k_fill = P ? s_k0 : s_k1;  // K(e+1) replaces K(e-1)
    uint8_t* v_fill = P ? s_v0 : s_v1;  // V(e+1) replaces V(e-1)
    if (e + 1 < n_ep) {
      k_tile_to_lds<D>(krs, (e + 1) * kBlock * D, k_fill, w, lane);
      v_tile_to_lds<D>(vrs, (e + 1) * D * kBlock, v_fill, w, lane);
    }
    if (e < w_ep) {
      v16i acc0, acc1;
      qk_epoch<D>(k_cur, qreg, koff, acc0, acc1);
      // log2-domain score per unit of the int32 accumulator
      const float c = cq * ksh[e];
      int x[32];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        x[r] = acc0[r];
        x[16 + r] = acc1[r];
      }
      const bool masked = kBlock * e + kBlock - 1 > w_lim;  // wave-uniform
      const int dlim = lim - (kBlock * e + 32 * h);          // x[t] visible iff t <= dlim
      float ps;
      v8i pb;
      float alpha;
      bool moved;
      // Hidden scores are only kept out of the row max and have p = 0, so the
      // unmasked path carries no select.
      if (masked) {
        int y[32];
#pragma unroll
        for (int t = 0; t < 32; ++t) y[t] = (t > dlim) ? INT_MIN : x[t];
        const int mx = half_max(row_max32(y));
        const float mt = (kBlock * e <= lim) ? (float)mx * c : -INFINITY;
        // mt > m is the only way the running max changes (neither is NaN), so
        // one compare gives both the new max and the lanes that moved.
        const bool up = mt > m;
        const float m_new = up ? mt : m;
        const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
        alpha = __builtin_amdgcn_exp2f(m - m_use);
        moved = __builtin_amdgcn_ballot_w64(up) != 0;
#pragma unroll
        for (int d = 0; d < 8; ++d) pb[d] = p4_masked(x, d, c, m_use, dlim, ps);
        m = m_new;
      } else {
        const int mx = half_max(row_max32(x));
        const float mt = (float)mx * c;
        const bool up = mt > m;
        const float m_new = up ? mt : m;
        alpha = __builtin_amdgcn_exp2f(m - m_new);
        moved = __builtin_amdgcn_ballot_w64(up) != 0;
#pragma unroll
        for (int d = 0; d < 8; ++d) pb[d] = p4(x, d, c, m_new, ps);
        m = m_new;
      }
      l = __builtin_fmaf(l, alpha, ps);
      // Per-tile rescale; a no-op (alpha == 1 in every lane) when no row max moved.
      if (moved) {
#pragma unroll
        for (int cb = 0; cb < D / 32; ++cb) ro[cb] *= alpha;
      }
#pragma unroll
      for (int cb = 0; cb < D / 32; ++cb) {
        const int ch = 32 * cb + ql;
        const v4i lo = *reinterpret_cast<const v4i*>(v_cur + v_lds_off(ch, 2 * h));
        const v4i hi = *reinterpret_cast<const v4i*>(v_cur + v_lds_off(ch, 2 * h + 1));
        const v8i av = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        ro[cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, pb, ro[cb], 0, 0, 0, 127, 0, 127);
      }
      if (TRACE && w == a.trace_wave) {
        // Checkpoints of this epoch: m (log2 domain), l, alpha, P8, RO.
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
        for (int d = 0; d < 8; ++d) p8[d] = (uint32_t)pb[d];
        float* rt = a.tr_ro + ((long)ql * a.nkb + e) * D;
#pragma unroll
        for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
          for (int r = 0; r < 16; ++r) rt[32 * cb + 8 * (r / 4) + 4 * h + r % 4] = ro[cb][r];
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  for (int e = 0; e < n_ep; e += 2) {
    body(std::integral_constant<int, 0>{}, e);
    if (e + 1 < n_ep) body(std::integral_constant<int, 1>{}, e + 1);
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
  // A wave's 32 output rows are consecutive in memory. The bf16 values go
  // through LDS (one of the four K/V buffers per wave; every wave has passed
  // the last epoch's barrier, so none is read any more) and leave as whole
  // 16-byte chunks of consecutive rows: scattered 8-byte stores of the
  // register layout cost more than the arithmetic of the epilogue.
  uint8_t* stage = w == 0 ? s_k0 : w == 1 ? s_k1 : w == 2 ? s_v0 : s_v1;  // 32 rows x 2D bytes
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int c0 = 32 * cb + 8 * g + 4 * h;
      const float4 sv = *reinterpret_cast<const float4*>(s_sv + c0);
      const uint32_t w0 = pack2_bf16(ro[cb][4 * g + 0] * rcp * sv.x, ro[cb][4 * g + 1] * rcp * sv.y);
      const uint32_t w1 = pack2_bf16(ro[cb][4 * g + 2] * rcp * sv.z, ro[cb][4 * g + 3] * rcp * sv.w);
      *reinterpret_cast<uint2*>(stage + out_lds_off<D>(ql, 4 * cb + g) + 8 * h) = make_uint2(w0, w1);
    }
  }
  // A wave's LDS accesses complete in order; this keeps the compiler from
  // moving the reads below above the writes.
  asm volatile("" ::: "memory");
  constexpr int kChunksPerRow = D / 8;  // 16-byte chunks of one bf16 output row
  uint16_t* obase = a.out + (bh * a.Lq + wrow0) * (long)D;
#pragma unroll
  for (int i = 0; i < 32 * kChunksPerRow / 64; ++i) {
    const int gi = lane + 64 * i, row = gi / kChunksPerRow, chunk = gi % kChunksPerRow;
    const uint4 val = *reinterpret_cast<const uint4*>(stage + out_lds_off<D>(row, chunk));
    if (wrow0 + row < a.Lq) *reinterpret_cast<uint4*>(obase + (long)row * D + 8 * chunk) = val;
  }
}

// ------------------------------------------------------------ debug kernels

// One 64x64 int32 QK tile per workgroup (2 waves = 64 queries), through the
// main loop's own staging (direct buffer-to-LDS copies into the swizzled
// layout) and qk_epoch code.
template <int D>
__global__ __launch_bounds__(128) void qk_debug_kernel(QkDebugArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t s_k[kBlock * D];
  const int t = blockIdx.x;
  const long bh = (long)a.tiles[t][0] * a.H + a.tiles[t][1];
  const int qb = a.tiles[t][2], kb = a.tiles[t][3];
  const int lane = threadIdx.x & 63, h = lane >> 5, ql = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int qrow = qb * kBlock + 32 * w + ql;
  v4i qreg[D / 32];
  const int8_t* qh = a.q_i8 + bh * (long)a.nqb * kBlock * D;
#pragma unroll
  for (int s = 0; s < D / 32; ++s)
    qreg[s] = *reinterpret_cast<const v4i*>(qh + (long)qrow * D + 32 * s + 16 * h);
  // The two waves copy the four quarters of the tile that the main loop's
  // four waves copy (the host bounds a head's codes below 2^31 bytes).
  const int head_bytes = a.nkb * kBlock * D;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.k_i8 + bh * (long)head_bytes), (short)0, head_bytes, kRawBufferFlags);
  k_tile_to_lds<D>(krs, kb * kBlock * D, s_k, w, lane);
  k_tile_to_lds<D>(krs, kb * kBlock * D, s_k, w + 2, lane);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  v16i acc0, acc1;
  int koff[D / 32];
  qk_offsets<D>(lane, koff);
  qk_epoch<D>(s_k, qreg, koff, acc0, acc1);
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
