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
//    B = Q codes from the workgroup's LDS Q tile, copied in once per tile,
//    or coded there from bf16 Q by the entry design). The K rows are
//    loaded in a permuted order so that each lane ends with 32 consecutive
//    keys of ONE query: lane (h, q) holds S[q][32h .. 32h+31].
//  * softmax: the row max is taken on the exact int32 scores (the dequant
//    factor sq*sk*sm_scale*log2e is positive), then one cross-half exchange;
//    p = exp2(fma(S, c, -m)) in fp32 (relative to the integer row max once
//    the scores are very large); the row sum stays a per-half partial until
//    the epilogue.
//  * P -> E4M3 in registers; that register block IS the B operand of the PV
//    matrix-core step (O^T = V^T . P^T, v_mfma_f32_32x32x64_f8f6f4), so P
//    never goes through LDS, and each lane's outputs belong to its own query.
//  * two-level PV: RO *= alpha (skipped when no row max of the wave moved,
//    i.e. alpha == 1 in every lane), then the matrix core reduces the epoch's
//    64 keys in fp32 (inner level) and adds the result into RO, its C
//    operand (outer level); epoch 0 starts RO from a zero accumulator.
//  * epilogue: r = 1/l (IEEE divide), out = bf16(RO * r * sv[c]) for rows < Lq,
//    with sv read into LDS at the start; a wave's 32 rows are consecutive in
//    memory, so they pass through LDS and leave as whole 16-byte chunks.
//  * instantiations: TRACE records one wave's per-epoch state (debug);
//    PERSIST runs the tiles in persistent workgroups fed by work counters;
//    NW = 8 gives 256-row workgroups; ENTRY codes the Q tile from bf16 Q.
#include <type_traits>

#include "attn_common.h"

namespace sage {

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

// Waves per SIMD the register budget is set for: 3 at D = 128 with 4-wave
// workgroups (<= 168 VGPRs; the LDS of 4 such workgroups would not fit a CU),
// 4 at D = 64 and for 8-wave workgroups (<= 128); the trace build stores
// extra state and runs one workgroup, so it keeps the compiler's default.
template <int D, bool TRACE, int NW>
constexpr int kWavesPerSimd = TRACE ? 1 : (D == 64 || NW == 8 ? 4 : 3);

// The LDS of one workgroup. Four separate K/V objects (not one array) so
// that the compiler can tell the in-flight direct fills apart from the
// buffers being read; the head's V channel scales are read at the start so
// that the epilogue does not wait for a global load.
template <int D>
struct FusedLds {
  uint8_t* k0;
  uint8_t* k1;
  uint8_t* v0;
  uint8_t* v1;
  float* sv;
};

// Entry design: the Q codes of a tile, made by the main loop from the bf16
// rows as the preparation pass makes them (an INT8 scale per 64-row block:
// s = absmax / 127 over the block's rows < Lq; code = clamp(rint(x / s),
// +-127) with the quotient rounded as an IEEE division; rows >= Lq code 0),
// so for finite inputs the codes and scales are the same bits. Each wave
// codes its own 32 rows (wrow0 ..) into the LDS Q tile; the two waves of a
// 64-row block exchange their absmax through s_qmax (one slot per wave).
// Every wave of the workgroup calls it (it holds a barrier). Returns the
// block's s. Three shortcuts, exact for finite bf16 inputs:
//  * the absmax is a packed 16-bit unsigned max of the bf16 bits with the
//    sign cleared (finite magnitudes order like their bit patterns);
//  * |x / s| < 127.5 for every finite bf16 x (s = RN(absmax / 127) is within
//    2^-10 of absmax / 127 even when it is subnormal), so the clamp never
//    binds, and adding 1.5 * 2^23 rounds the quotient to the nearest integer,
//    ties to even, in one fp32 addition whose low byte is then the code;
//  * the block's scale is read as a wave-uniform value, so the choice of
//    quotient path is one branch.
template <int D, int NW>
__device__ __forceinline__ float q_code_tile(const uint16_t* __restrict__ qh, int Lq, int wrow0, uint8_t* s_q,
                                             float* s_qmax, int w, int lane) {
  constexpr int kChunks = D / 16;               // 16-code chunks per row
  constexpr int kPerLane = 32 * kChunks / 64;   // chunks per lane: 4 at D = 128, 2 at D = 64
  uint4 raw[kPerLane][2];
#pragma unroll
  for (int j = 0; j < kPerLane; ++j) {
    const int p = lane + 64 * j, row = wrow0 + p / kChunks, c = p % kChunks;
    if (row < Lq) {
      const uint4* src = reinterpret_cast<const uint4*>(qh + (long)row * D + 16 * c);
      raw[j][0] = src[0];
      raw[j][1] = src[1];
    } else {
      raw[j][0] = raw[j][1] = make_uint4(0, 0, 0, 0);
    }
  }
  // Rows >= Lq hold zeros, which leave the absmax as it is.
  typedef unsigned short v2u16 __attribute__((ext_vector_type(2)));
  v2u16 mx2 = {0, 0};
#pragma unroll
  for (int j = 0; j < kPerLane; ++j)
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const uint4 u = raw[j][hf];
      const uint32_t ws[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int t = 0; t < 4; ++t)
        mx2 = __builtin_elementwise_max(mx2, __builtin_bit_cast(v2u16, ws[t] & 0x7FFF7FFFu));
    }
  float amax = __uint_as_float((uint32_t)max(mx2[0], mx2[1]) << 16);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  if (lane == 0) s_qmax[w] = amax;
  __syncthreads();
  const float am = __uint_as_float(
      __builtin_amdgcn_readfirstlane(__float_as_uint(fmaxf(s_qmax[w], s_qmax[w ^ 1]))));
  const float s = am / 127.0f;
  uint32_t cw[kPerLane][4];
  // Codes of every chunk from the quotient function quot(x).
  auto code_all = [&](auto quot) {
#pragma unroll
    for (int j = 0; j < kPerLane; ++j)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        float f[8];
        unpack8(raw[j][hf], f);
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          uint32_t b[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) b[i] = __float_as_uint(quot(f[4 * g + i]) + 12582912.0f);
          // low bytes of b0..b3 -> bytes 0..3
          const uint32_t lo = __builtin_amdgcn_perm(b[1], b[0], 0x0c0c0400u);
          const uint32_t hi = __builtin_amdgcn_perm(b[3], b[2], 0x04000c0cu);
          cw[j][2 * hf + g] = lo | hi;
        }
      }
  };
  if (am == 0.0f) {  // every code 0
#pragma unroll
    for (int j = 0; j < kPerLane; ++j)
#pragma unroll
      for (int t = 0; t < 4; ++t) cw[j][t] = 0u;
  } else if (s >= kFastDivMinScale) {
    const float r = 1.0f / s;
    code_all([&](float x) { return div_rn(x, s, r); });
  } else {
    code_all([&](float x) { return x / s; });
  }
#pragma unroll
  for (int j = 0; j < kPerLane; ++j) {
    const int p = lane + 64 * j;
    *reinterpret_cast<uint4*>(s_q + q_lds_off<D>(32 * w + p / kChunks, p % kChunks)) =
        make_uint4(cw[j][0], cw[j][1], cw[j][2], cw[j][3]);
  }
  return s;
}

// One tile of 32 NW rows of head bh (NW waves of 32 rows each). ENTRY: the
// tile's Q codes are made here from bf16 Q (q_code_tile) instead of copied.
template <int D, bool CAUSAL, bool TRACE, int NW, bool ENTRY>
__device__ __forceinline__ void fused_tile(const AttnArgs& a, const int tile, const long bh, uint8_t* s_k0,
                                           uint8_t* s_k1, uint8_t* s_v0, uint8_t* s_v1, uint8_t* s_q,
                                           float* s_sv, float* s_qmax) {
  // The thread index is made opaque here, so that the per-lane offsets
  // derived from it are computed where they are used, in every tile, rather
  // than hoisted out of a persistent workgroup's tile loop (where they would
  // stay live through every epoch loop and push the kernel past its
  // registers).
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int h = lane >> 5, ql = lane & 31;
  constexpr int kRows = 32 * NW;
  const int q0 = tile * kRows;
  const int wrow0 = q0 + 32 * w;
  const int qrow = wrow0 + ql;
  const int off = a.Lkv - a.Lq;

  // Epochs the workgroup stages, and the epochs this wave computes.
  int n_ep = a.nkb;
  if (CAUSAL) {
    const int x = min(a.Lq - 1, q0 + kRows - 1) + off;
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
    k_tile_to_lds<D, NW>(krs, 0, s_k0, w, lane);
    v_tile_to_lds<D, NW>(vrs, 0, s_v0, w, lane);
  }

  if (tid < D) s_sv[tid] = a.v_scale[bh * D + tid];
  // The tile's Q codes go straight into LDS with the first fills (or are
  // made there from bf16 Q).
  float sq;
  if (ENTRY) {
    const float s = q_code_tile<D, NW>(a.q + bh * (long)a.Lq * D, a.Lq, wrow0, s_q, s_qmax, w, lane);
    sq = wave_on ? s : 0.0f;
  } else {
    const int q_bytes = a.nqb * kBlock * D;
    const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.q_i8 + bh * (long)q_bytes), (short)0, q_bytes, kRawBufferFlags);
    q_tile_to_lds<D, NW>(qrs, q0, s_q, w, lane);
    sq = wave_on ? a.q_scale[bh * a.nqb + wrow0 / kBlock] : 0.0f;
  }
  int qoff[D / 32];
#pragma unroll
  for (int s = 0; s < D / 32; ++s) qoff[s] = q_lds_off<D>(32 * w + ql, 2 * s + h);
  const float cq = sq * a.scale_log2;

  // The QK read offsets are computed once; the empty asm keeps the compiler
  // from rebuilding them from their parts in every epoch (four VALU adds).
  int koff[D / 32];
  qk_offsets<D>(lane, koff);
#pragma unroll
  for (int s = 0; s < D / 32; ++s) asm volatile("" : "+v"(koff[s]));

  float m = -INFINITY, l = 0.0f;
  // RO is first written by epoch 0's PV step (a wave that computes any epoch
  // computes epoch 0: every row that sees a key sees key 0); a wave with no
  // epoch clears it after the loop.
  v16f ro[D / 32];
  __builtin_amdgcn_s_waitcnt(0);  // the first fills (issued above) have landed
  __syncthreads();

  // One epoch. The epoch's parity is a template argument so every LDS buffer
  // is a fixed object; epoch 0 (first) has its own copy, with no rescale and
  // a zero accumulator for its PV step.
  auto body = [&](auto parity, auto first, const int e) {
    constexpr int P = decltype(parity)::value;
    constexpr bool F = decltype(first)::value;
    uint8_t* k_cur = P ? s_k1 : s_k0;   // K(e)
    uint8_t* v_cur = P ? s_v1 : s_v0;   // V(e)
    uint8_t* k_fill = P ? s_k0 : s_k1;  // K(e+1) replaces K(e-1)
    uint8_t* v_fill = P ? s_v0 : s_v1;  // V(e+1) replaces V(e-1)
    if (e + 1 < n_ep) {
      k_tile_to_lds<D, NW>(krs, (e + 1) * kBlock * D, k_fill, w, lane);
      v_tile_to_lds<D, NW>(vrs, (e + 1) * D * kBlock, v_fill, w, lane);
    }
    if (e < w_ep) {
      v16i acc0, acc1;
      qk_epoch_lq<D>(k_cur, s_q, qoff, koff, acc0, acc1);
      // log2-domain score per unit of the int32 accumulator
      const float c = cq * ksh[e];
      const bool masked = kBlock * e + kBlock - 1 > w_lim;  // wave-uniform
      const int dlim = lim - (kBlock * e + 32 * h);          // score t visible iff t <= dlim
      v8i pb;
      float alpha;
      bool moved;
      softmax_epoch(acc0, acc1, c, masked, dlim, kBlock * e <= lim, m, l, pb, alpha, moved);
      // Per-tile rescale; a no-op (alpha == 1 in every lane) when no row max moved.
      if (!F && moved) {
#pragma unroll
        for (int cb = 0; cb < D / 32; ++cb) ro[cb] *= alpha;
      }
      if (F)
        pv_epoch_first<D>(v_cur, pb, ro, h, ql);
      else
        pv_epoch<D>(v_cur, pb, ro, h, ql);
      if (TRACE && w == a.trace_wave) {
        // The epoch's own PV partial, run again into a zeroed accumulator.
        v16f pv[D / 32];
#pragma unroll
        for (int cb = 0; cb < D / 32; ++cb) pv[cb] = v16f{};
        pv_epoch<D>(v_cur, pb, pv, h, ql);
        trace_softmax(a, e, h, ql, m, l, alpha, pb);
        trace_pv<D>(a, e, h, ql, ro, pv);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  using Even = std::integral_constant<int, 0>;
  using Odd = std::integral_constant<int, 1>;
  using First = std::true_type;
  using Later = std::false_type;
  if (n_ep > 0) body(Even{}, First{}, 0);
  for (int e = 1; e < n_ep; e += 2) {
    body(Odd{}, Later{}, e);
    if (e + 1 < n_ep) body(Even{}, Later{}, e + 1);
  }
  if (w_ep == 0) {
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb) ro[cb] = v16f{};
  }

  // Epilogue: the two halves of a query hold partial sums of l. Each wave
  // stages its 32 rows (2D bytes each) in one of the four K/V buffers, waves
  // 4-7 of a wide workgroup in a quarter of the Q tile (every wave has passed
  // the last epoch's barrier, so none of them is read any more).
  const float lt = half_sum(l);
  const float rcp = (lt > 0.0f) ? 1.0f / lt : 0.0f;
  if (TRACE && w == a.trace_wave) trace_final(a, h, ql, rcp, lt);
  uint8_t* stage = w == 0 ? s_k0 : w == 1 ? s_k1 : w == 2 ? s_v0 : w == 3 ? s_v1 : s_q + (w - 4) * 64 * D;
  store_rows<D>(ro, rcp, s_sv, stage, a.out, bh, a.Lq, wrow0, lane, h, ql);
}

template <int D, bool CAUSAL, bool TRACE, bool PERSIST, int NW, bool ENTRY = false>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(kWavesPerSimd<D, TRACE, NW>)))
void attn_fwd_kernel(AttnArgs a) {
  static_assert(NW == 4 || NW == 8, "4- or 8-wave workgroups");
  __shared__ __attribute__((aligned(16))) uint8_t s_k0[kBlock * D];
  __shared__ __attribute__((aligned(16))) uint8_t s_k1[kBlock * D];
  __shared__ __attribute__((aligned(16))) uint8_t s_v0[D * kBlock];
  __shared__ __attribute__((aligned(16))) uint8_t s_v1[D * kBlock];
  __shared__ __attribute__((aligned(16))) uint8_t s_q[32 * NW * D];
  __shared__ __attribute__((aligned(16))) float s_sv[D];
  __shared__ float s_qmax[NW];
  if (TRACE) {
    fused_tile<D, CAUSAL, TRACE, NW, ENTRY>(a, a.trace_tile, a.trace_bh, s_k0, s_k1, s_v0, s_v1, s_q, s_sv,
                                            s_qmax);
    return;
  }
  if (!PERSIST) {
    int tile;
    long bh;
    work_item(a, blockIdx.x, tile, bh);
    fused_tile<D, CAUSAL, TRACE, NW, ENTRY>(a, tile, bh, s_k0, s_k1, s_v0, s_v1, s_q, s_sv, s_qmax);
    return;
  }
  // Persistent workgroups take work items from counters (fetch-and-add), one
  // per XCD: workgroups are dealt to the 8 XCDs round-robin, so workgroup b
  // runs on XCD x = b % 8 and takes the items n = x + 8 k, k = 0, 1, ... in
  // order (heaviest first), as the per-tile grid would place them: with B*H a
  // multiple of 8, every tile of a head then stays on one XCD and its L2.
  // Each workgroup's last fetch is past the end, so counter x serves exactly
  // items_x + wgs_x fetches in a launch; the workgroup that draws the last
  // of them returns it to 0 for the next launch on this counter (no other
  // workgroup of the launch touches that counter afterwards).
  __shared__ int s_item;
  constexpr int kXcds = 8;
  const int n_items = a.n_qtiles * a.B * a.H;
  const int x = blockIdx.x % kXcds;
  const int items_x = (n_items - x + kXcds - 1) / kXcds;
  const int wgs_x = ((int)gridDim.x - x + kXcds - 1) / kXcds;
  unsigned int* queue = a.queue + x;
  for (;;) {
    if (threadIdx.x == 0) s_item = (int)atomicAdd(queue, 1u);
    __syncthreads();
    const int k = s_item;
    if (k >= items_x) {
      if (threadIdx.x == 0 && k == items_x + wgs_x - 1) atomicExch(queue, 0u);
      return;
    }
    int tile;
    long bh;
    work_item(a, x + kXcds * k, tile, bh);
    fused_tile<D, CAUSAL, TRACE, NW, ENTRY>(a, tile, bh, s_k0, s_k1, s_v0, s_v1, s_q, s_sv, s_qmax);
    // Every wave is done with the LDS (the epilogue staged its rows in the
    // K/V buffers) and with s_item before the next item refills them.
    __syncthreads();
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

template <int D, bool C, bool T, bool P, int NW, bool E>
static hipError_t launch_attn_t(const AttnArgs& a, hipStream_t stream) {
  const long blocks = T ? 1L : P ? (long)a.persist_grid : (long)a.n_qtiles * a.B * a.H;
  attn_fwd_kernel<D, C, T, P, NW, E><<<dim3((unsigned)blocks), 64 * NW, 0, stream>>>(a);
  return hipGetLastError();
}

template <bool T, bool P, int NW, bool E = false>
static hipError_t launch_attn_v(const AttnArgs& a, int D, bool causal, hipStream_t stream) {
  if (D == 128)
    return causal ? launch_attn_t<128, true, T, P, NW, E>(a, stream)
                  : launch_attn_t<128, false, T, P, NW, E>(a, stream);
  return causal ? launch_attn_t<64, true, T, P, NW, E>(a, stream) : launch_attn_t<64, false, T, P, NW, E>(a, stream);
}

hipError_t launch_attn_fused(const AttnArgs& a, int D, bool causal, bool trace, hipStream_t stream) {
  return trace ? launch_attn_v<true, false, 4>(a, D, causal, stream)
               : launch_attn_v<false, false, 4>(a, D, causal, stream);
}
hipError_t launch_attn_wide(const AttnArgs& a, int D, bool causal, bool trace, hipStream_t stream) {
  return trace ? launch_attn_v<true, false, 8>(a, D, causal, stream)
               : launch_attn_v<false, false, 8>(a, D, causal, stream);
}
hipError_t launch_attn_persistent(const AttnArgs& a, int D, bool causal, hipStream_t stream) {
  return launch_attn_v<false, true, 4>(a, D, causal, stream);
}

hipError_t launch_attn_entry(const AttnArgs& a, int D, bool causal, hipStream_t stream) {
  return launch_attn_v<false, false, 4, true>(a, D, causal, stream);
}

hipError_t launch_attn(const AttnArgs& a, int D, bool causal, int kernel, hipStream_t stream) {
  if (kernel == kKernelSplit) return launch_attn_split(a, D, causal, false, stream);
  if (kernel == kKernelEntry) return launch_attn_entry(a, D, causal, stream);
  if (kernel == kKernelPersistent) return launch_attn_persistent(a, D, causal, stream);
  if (kernel == kKernelWide) return launch_attn_wide(a, D, causal, false, stream);
  return launch_attn_fused(a, D, causal, false, stream);
}
hipError_t launch_attn_trace(const AttnArgs& a, int D, bool causal, int kernel, hipStream_t stream) {
  if (kernel == kKernelSplit) return launch_attn_split(a, D, causal, true, stream);
  if (kernel == kKernelEntry) return launch_attn_v<true, false, 4, true>(a, D, causal, stream);
  if (kernel == kKernelWide) return launch_attn_wide(a, D, causal, true, stream);
  return launch_attn_fused(a, D, causal, true, stream);
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
