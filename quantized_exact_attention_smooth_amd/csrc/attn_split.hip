// Wave-specialised quantized attention main loop for gfx950 (CDNA4).
//
// Experiment Log (vortex_exact_attention): "Phase 1 State-Ownership
// Decision" chooses paired owners, one set of warps holding the QK/softmax
// state and another the PV/output state; "Phase 2A VEA-B Capability Decision"
// reports that the QK and PV role clocks overlap. This kernel keeps that
// ownership split in CDNA4 terms, with the same arithmetic as the fused
// kernel (attn_fwd.hip) step for step, so its output is bit-identical:
//
//  * workgroup = 8 waves = 128 query rows of one (b, h). Waves 0-3 (softmax
//    waves) own the Q codes, the scores, the running max m and the row sums
//    l of rows 32 g .. 32 g + 31 (g = wave & 3); waves 4-7 (PV waves) own
//    RO of the same rows. Neither role holds the other's registers, so the
//    kernel fits 128 VGPRs: four waves per SIMD (two workgroups per CU).
//  * a softmax wave runs the softmax of epoch t and refills each of its two
//    score accumulators with the QK matrix-core steps of epoch t + 1 as soon
//    as the softmax has consumed it, so half of those steps run under the
//    softmax's VALU work and half while the waves meet at the period's
//    barrier, with one set of score registers; it hands the E4M3 P block of epoch t (exactly the PV
//    step's B operand, 32 bytes per lane) and alpha to its PV wave through a
//    two-slot LDS ring.
//  * a PV wave takes P(t - 1) and alpha(t - 1), rescales RO (skipped when
//    alpha == 1 in every lane) and runs the PV step of epoch t - 1; the PV
//    waves also issue every direct global-to-LDS copy: K(t + 2) and V(t)
//    during period t (two slots each).
//  * one s_barrier per period orders the ring: period t writes P(t), K(t+2),
//    V(t) into the slots that period t - 1 finished reading.
//  * epilogue: the softmax waves pass 1/l through LDS; the PV waves write
//    bf16(RO * (1/l) * sv[c]) staged through LDS as whole 16-byte chunks.
#include <type_traits>

#include "attn_common.h"

namespace sage {

constexpr int kSplitThreads = 512;  // 4 softmax waves + 4 PV waves

// Waves per SIMD the register budget is set for (<= 128 VGPRs); the trace
// build stores extra state and runs one workgroup.
template <bool TRACE>
constexpr int kSplitWavesPerSimd = TRACE ? 1 : 4;

template <int D, bool CAUSAL, bool TRACE>
__global__ __launch_bounds__(kSplitThreads) __attribute__((amdgpu_waves_per_eu(kSplitWavesPerSimd<TRACE>)))
void attn_split_kernel(AttnArgs a) {
  // Separate LDS objects (not one array) so that the compiler can tell the
  // in-flight direct copies apart from the buffers being read.
  __shared__ __attribute__((aligned(16))) uint8_t s_k0[kBlock * D];
  __shared__ __attribute__((aligned(16))) uint8_t s_k1[kBlock * D];
  __shared__ __attribute__((aligned(16))) uint8_t s_v0[D * kBlock];
  __shared__ __attribute__((aligned(16))) uint8_t s_v1[D * kBlock];
  // P ring: [row group][half][lane][4 dwords], the B operand of the PV step
  // as the softmax wave's lane holds it (2 x 16 bytes per lane; each b128
  // access covers 1 KiB of consecutive 16-byte chunks, free of bank
  // conflicts).
  __shared__ __attribute__((aligned(16))) uint32_t s_p0[4 * 2 * 64 * 4];
  __shared__ __attribute__((aligned(16))) uint32_t s_p1[4 * 2 * 64 * 4];
  __shared__ float s_a0[4 * 32];  // alpha per row, even / odd epochs
  __shared__ float s_a1[4 * 32];
  __shared__ float s_rcp[4 * 32];  // 1/l per row, for the epilogue
  __shared__ __attribute__((aligned(16))) float s_sv[D];

  int tile = a.trace_tile;
  long bh = a.trace_bh;
  if (!TRACE) work_item(a, blockIdx.x, tile, bh);
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int g = wid & 3;                                              // row group
  const int h = lane >> 5, ql = lane & 31;
  const int q0 = tile * kQTile;
  const int wrow0 = q0 + 32 * g;
  const int qrow = wrow0 + ql;
  const int off = a.Lkv - a.Lq;

  // Epochs the workgroup stages, and the epochs of this row group.
  int n_ep = a.nkb;
  if (CAUSAL) {
    const int x = min(a.Lq - 1, q0 + kQTile - 1) + off;
    n_ep = x < 0 ? 0 : min(a.nkb, x / kBlock + 1);
  }
  const bool group_on = wrow0 < a.Lq;
  int w_ep = 0;
  if (group_on) {
    const int x = CAUSAL ? min(a.Lq - 1, wrow0 + 31) + off : a.Lkv - 1;
    w_ep = x < 0 ? 0 : min(a.nkb, x / kBlock + 1);
  }

  if (wid >= 4) {
    // ---------------------------------------------------------- PV wave
    // Buffer resources over this head's K and V tiles (the host bounds a
    // head's tiles below 2^31 bytes).
    const int head_bytes = a.nkb * kBlock * D;
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.k_i8 + bh * (long)head_bytes), (short)0, head_bytes, kRawBufferFlags);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.v_fp8 + bh * (long)head_bytes), (short)0, head_bytes, kRawBufferFlags);
    if (n_ep > 0) k_tile_to_lds<D>(krs, 0, s_k0, g, lane);
    if (n_ep > 1) k_tile_to_lds<D>(krs, kBlock * D, s_k1, g, lane);
    const int ti = threadIdx.x - 256;
    if (ti < D) s_sv[ti] = a.v_scale[bh * D + ti];
    // RO is first written by epoch 0's PV step (a group that computes any
    // epoch computes epoch 0); a group with no epoch clears it after the loop.
    v16f ro[D / 32];
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();  // K(0), K(1) resident
    __syncthreads();  // the softmax waves have read K(0): its slot may refill

    // Period t: copies of K(t+2) and V(t), then the PV step of epoch t - 1
    // (period 1, first, holds epoch 0's: no rescale, a zero accumulator).
    auto body = [&](auto parity, auto first, const int t) {
      constexpr int P = decltype(parity)::value;
      constexpr bool F = decltype(first)::value;
      uint8_t* k_fill = P ? s_k1 : s_k0;         // K(t+2) replaces K(t)
      uint8_t* v_fill = P ? s_v1 : s_v0;         // V(t) replaces V(t-2)
      const uint8_t* v_cur = P ? s_v0 : s_v1;    // V(t-1)
      const uint32_t* p_cur = P ? s_p0 : s_p1;   // P(t-1)
      const float* a_cur = P ? s_a0 : s_a1;      // alpha(t-1)
      if (t + 2 < n_ep) k_tile_to_lds<D>(krs, (t + 2) * kBlock * D, k_fill, g, lane);
      if (t < n_ep) v_tile_to_lds<D>(vrs, t * D * kBlock, v_fill, g, lane);
      const int e = t - 1;
      if (e >= 0 && e < w_ep) {
        const uint4* pp = reinterpret_cast<const uint4*>(p_cur) + g * 128 + lane;
        const uint4 p0 = pp[0], p1 = pp[64];
        const v8i pb = {(int)p0.x, (int)p0.y, (int)p0.z, (int)p0.w, (int)p1.x, (int)p1.y, (int)p1.z, (int)p1.w};
        const float alpha = a_cur[g * 32 + ql];
        // Per-tile rescale; a no-op (alpha == 1 in every lane) when no row
        // max of the group moved.
        if (!F && __builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
          for (int cb = 0; cb < D / 32; ++cb) ro[cb] *= alpha;
        }
        if (F)
          pv_epoch_first<D>(v_cur, pb, ro, h, ql);
        else
          pv_epoch<D>(v_cur, pb, ro, h, ql);
        if (TRACE && g == a.trace_wave) {
          v16f pv[D / 32];
#pragma unroll
          for (int cb = 0; cb < D / 32; ++cb) pv[cb] = v16f{};
          pv_epoch<D>(v_cur, pb, pv, h, ql);
          trace_pv<D>(a, e, h, ql, ro, pv);
        }
      }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    };
    using Even = std::integral_constant<int, 0>;
    using Odd = std::integral_constant<int, 1>;
    body(Even{}, std::false_type{}, 0);
    if (1 <= n_ep) body(Odd{}, std::true_type{}, 1);
    for (int t = 2; t <= n_ep; t += 2) {
      body(Even{}, std::false_type{}, t);
      if (t + 1 <= n_ep) body(Odd{}, std::false_type{}, t + 1);
    }
    if (w_ep == 0) {
#pragma unroll
      for (int cb = 0; cb < D / 32; ++cb) ro[cb] = v16f{};
    }
    __syncthreads();  // 1/l of every row is in s_rcp
    const float rcp = s_rcp[g * 32 + ql];
    uint8_t* stage = g == 0 ? s_k0 : g == 1 ? s_k1 : g == 2 ? s_v0 : s_v1;  // 32 rows x 2D bytes
    store_rows<D>(ro, rcp, s_sv, stage, a.out, bh, a.Lq, wrow0, lane, h, ql);
  } else {
    // ----------------------------------------------------- softmax wave
    // Keys beyond lim (this lane's last visible key) are masked. An epoch
    // needs the mask only when it reaches past the group's smallest limit.
    const int lim = CAUSAL ? min(qrow + off, a.Lkv - 1) : a.Lkv - 1;
    const int w_lim = CAUSAL ? min(wrow0 + off, a.Lkv - 1) : a.Lkv - 1;
    const __attribute__((address_space(4))) float* ksh =
        (const __attribute__((address_space(4))) float*)(a.k_scale + bh * a.nkb);
    v4i qreg[D / 32];
    const int8_t* qh = a.q_i8 + bh * (long)a.nqb * kBlock * D;
#pragma unroll
    for (int s = 0; s < D / 32; ++s)
      qreg[s] = (qrow < a.Lq) ? *reinterpret_cast<const v4i*>(qh + (long)qrow * D + 32 * s + 16 * h) : v4i{};
    const float sq = group_on ? a.q_scale[bh * a.nqb + wrow0 / kBlock] : 0.0f;
    const float cq = sq * a.scale_log2;
    int koff[D / 32];
    qk_offsets<D>(lane, koff);
#pragma unroll
    for (int s = 0; s < D / 32; ++s) asm volatile("" : "+v"(koff[s]));
    float m = -INFINITY, l = 0.0f;
    v16i acc0, acc1;  // scores of the current epoch
    __syncthreads();  // K(0), K(1) resident
    if (w_ep > 0) qk_epoch<D>(s_k0, qreg, koff, acc0, acc1);
    __syncthreads();  // K(0) read (its slot refills during period 0)

    // Period t: the softmax of epoch t; the QK steps of epoch t + 1 refill
    // each score accumulator as soon as the softmax has consumed it (the
    // first half after the first 16 keys' probabilities), so half of them
    // run under the softmax's VALU work and the rest while the waves meet
    // at the period's barrier.
    auto body = [&](auto parity, const int t) {
      constexpr int P = decltype(parity)::value;
      const uint8_t* k_next = P ? s_k0 : s_k1;  // K(t+1)
      uint32_t* p_out = P ? s_p1 : s_p0;        // P(t)
      float* a_out = P ? s_a1 : s_a0;           // alpha(t)
      const bool next = t + 1 < w_ep;
      auto refill = [&](int i) {
        if (next) {
          if (i == 0) qk_half<D, 0>(k_next, qreg, koff, acc0);
          else qk_half<D, 1>(k_next, qreg, koff, acc1);
        }
      };
      if (t < w_ep) {
        const float c = cq * ksh[t];  // log2-domain score per accumulator unit
        const bool masked = kBlock * t + kBlock - 1 > w_lim;  // wave-uniform
        const int dlim = lim - (kBlock * t + 32 * h);          // score j visible iff j <= dlim
        v8i pb;
        float alpha;
        bool moved;
        softmax_epoch(acc0, acc1, c, masked, dlim, kBlock * t <= lim, m, l, pb, alpha, moved, refill);
        uint4* pp = reinterpret_cast<uint4*>(p_out) + g * 128 + lane;
        pp[0] = make_uint4(pb[0], pb[1], pb[2], pb[3]);
        pp[64] = make_uint4(pb[4], pb[5], pb[6], pb[7]);
        if (h == 0) a_out[g * 32 + ql] = alpha;
        if (TRACE && g == a.trace_wave) trace_softmax(a, t, h, ql, m, l, alpha, pb);
      }
      __syncthreads();
    };
    for (int t = 0; t <= n_ep; t += 2) {
      body(std::integral_constant<int, 0>{}, t);
      if (t + 1 <= n_ep) body(std::integral_constant<int, 1>{}, t + 1);
    }
    // The two halves of a query hold partial sums of l.
    const float lt = half_sum(l);
    const float rcp = (lt > 0.0f) ? 1.0f / lt : 0.0f;
    if (h == 0) s_rcp[g * 32 + ql] = rcp;
    if (TRACE && g == a.trace_wave) trace_final(a, h, ql, rcp, lt);
    __syncthreads();
  }
}

template <int D, bool C, bool T>
static hipError_t launch_split_t(const AttnArgs& a, hipStream_t stream) {
  const long blocks = T ? 1L : (long)a.n_qtiles * a.B * a.H;
  attn_split_kernel<D, C, T><<<dim3((unsigned)blocks), kSplitThreads, 0, stream>>>(a);
  return hipGetLastError();
}

template <bool T>
static hipError_t launch_split_v(const AttnArgs& a, int D, bool causal, hipStream_t stream) {
  if (D == 128) return causal ? launch_split_t<128, true, T>(a, stream) : launch_split_t<128, false, T>(a, stream);
  return causal ? launch_split_t<64, true, T>(a, stream) : launch_split_t<64, false, T>(a, stream);
}

hipError_t launch_attn_split(const AttnArgs& a, int D, bool causal, bool trace, hipStream_t stream) {
  return trace ? launch_split_v<true>(a, D, causal, stream) : launch_split_v<false>(a, D, causal, stream);
}

}  // namespace sage
