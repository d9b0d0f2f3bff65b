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
//    contiguous) are staged in LDS, double-buffered through registers.
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
//  * two-level PV: the epoch's P.V is formed in fresh fp32 registers, then
//    RO = RO * alpha + PV per element (one fma).
//  * epilogue: r = 1/l (IEEE divide), out = bf16(RO * r * sv[c]) for rows < Lq.
#include <limits.h>

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

// Four fp32 values -> four E4M3FN bytes (x0 in the low byte), hardware
// conversion, round to nearest even.
__device__ __forceinline__ int pack4_fp8(float x0, float x1, float x2, float x3) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, w, true);
}

// Two fp32 values -> two bf16 (x0 in the low half), round to nearest even.
__device__ __forceinline__ uint32_t pack2_bf16(float x0, float x1) {
  __bf16 b0 = (__bf16)x0, b1 = (__bf16)x1;
  return (uint32_t)__builtin_bit_cast(uint16_t, b0) | ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
}

// ------------------------------------------------------------ main kernel

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void attn_fwd_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t s_k[2][kBlock * D];
  __shared__ __attribute__((aligned(16))) uint8_t s_v[2][D * kBlock];

  const int BH = a.B * a.H;
  const int tile = a.n_qtiles - 1 - (int)(blockIdx.x / BH);
  const long bh = blockIdx.x % BH;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
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
  // Keys beyond lim (this lane's last visible key) are masked; an epoch needs
  // the mask only when it reaches past the wave's smallest limit.
  const int lim = CAUSAL ? min(qrow + off, a.Lkv - 1) : a.Lkv - 1;
  const int w_lim = CAUSAL ? min(wrow0 + off, a.Lkv - 1) : a.Lkv - 1;

  v4i qreg[D / 32];
  {
    const int8_t* qh = a.q_i8 + bh * (long)a.nqb * kBlock * D;
#pragma unroll
    for (int s = 0; s < D / 32; ++s)
      qreg[s] = (qrow < a.Lq) ? *reinterpret_cast<const v4i*>(qh + (long)qrow * D + 32 * s + 16 * h)
                              : v4i{};
  }
  const float sq = wave_on ? a.q_scale[bh * a.nqb + wrow0 / kBlock] : 0.0f;

  float m = -INFINITY, l = 0.0f;
  v16f ro[D / 32];
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb) ro[cb] = v16f{};

  const int8_t* kh = a.k_i8 + bh * (long)a.nkb * kBlock * D;
  const uint8_t* vh = a.v_fp8 + bh * (long)a.nkb * D * kBlock;
  const float* ksh = a.k_scale + bh * a.nkb;
  KStage<D, kThreads> ks;
  VStage<D, kThreads> vs;
  if (n_ep > 0) {
    ks.load(kh);
    vs.load(vh);
    ks.store(s_k[0]);
    vs.store(s_v[0]);
  }
  __syncthreads();

  for (int e = 0; e < n_ep; ++e) {
    const int buf = e & 1;
    if (e + 1 < n_ep) {
      ks.load(kh + (long)(e + 1) * kBlock * D);
      vs.load(vh + (long)(e + 1) * D * kBlock);
    }
    if (e < w_ep) {
      v16i acc0, acc1;
      qk_epoch<D>(s_k[buf], qreg, lane, acc0, acc1);

      const float c = sq * ksh[e] * a.scale_log2;
      const int kbase = kBlock * e + 32 * h;
      const bool masked = kBlock * e + kBlock - 1 > w_lim;
      int x[32];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        x[r] = acc0[r];
        x[16 + r] = acc1[r];
      }
      if (masked) {
#pragma unroll
        for (int t = 0; t < 32; ++t)
          if (kbase + t > lim) x[t] = INT_MIN;
      }
      int mx = x[0];
#pragma unroll
      for (int t = 1; t < 32; ++t) mx = max(mx, x[t]);
      mx = max(mx, __shfl_xor(mx, 32, 64));
      const float mt = (kBlock * e <= lim) ? (float)mx * c : -INFINITY;
      const float m_new = fmaxf(m, mt);
      const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m - m_use);

      float p[32];
      float ps = 0.0f;
#pragma unroll
      for (int t = 0; t < 32; ++t) {
        p[t] = __builtin_amdgcn_exp2f(__builtin_fmaf((float)x[t], c, -m_use));
        if (masked && kbase + t > lim) p[t] = 0.0f;
        ps += p[t];
      }
      l = l * alpha + ps;

      v8i pb;
#pragma unroll
      for (int d = 0; d < 8; ++d) pb[d] = pack4_fp8(p[4 * d], p[4 * d + 1], p[4 * d + 2], p[4 * d + 3]);

      const uint8_t* lv = s_v[buf];
#pragma unroll
      for (int cb = 0; cb < D / 32; ++cb) {
        const int ch = 32 * cb + ql;
        const v4i lo = *reinterpret_cast<const v4i*>(lv + v_lds_off(ch, 2 * h));
        const v4i hi = *reinterpret_cast<const v4i*>(lv + v_lds_off(ch, 2 * h + 1));
        const v8i av = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        const v16f pv = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, pb, v16f{}, 0, 0, 0, 127, 0, 127);
#pragma unroll
        for (int r = 0; r < 16; ++r) ro[cb][r] = __builtin_fmaf(ro[cb][r], alpha, pv[r]);
      }
      m = m_new;
    }
    if (e + 1 < n_ep) {
      ks.store(s_k[buf ^ 1]);
      vs.store(s_v[buf ^ 1]);
    }
    __syncthreads();
  }

  // Epilogue: both halves of a query hold partial sums of l.
  const float lt = l + __shfl_xor(l, 32, 64);
  const float rcp = (lt > 0.0f) ? 1.0f / lt : 0.0f;
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
// same staging and qk_epoch code as the main loop.
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

template <int D, bool C>
static hipError_t launch_attn_t(const AttnArgs& a, hipStream_t stream) {
  const long blocks = (long)a.n_qtiles * a.B * a.H;
  attn_fwd_kernel<D, C><<<dim3((unsigned)blocks), kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_attn(const AttnArgs& a, int D, bool causal, hipStream_t stream) {
  if (D == 128) return causal ? launch_attn_t<128, true>(a, stream) : launch_attn_t<128, false>(a, stream);
  return causal ? launch_attn_t<64, true>(a, stream) : launch_attn_t<64, false>(a, stream);
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
