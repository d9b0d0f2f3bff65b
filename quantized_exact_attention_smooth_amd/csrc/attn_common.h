// Device code shared by the main-loop kernels (internal header): the QK
// matrix-core step, the row reductions, the E4M3 and bf16 packing, the
// direct global-to-LDS tile copies, the online softmax of one epoch, the PV
// step, the epilogue's output staging and the checkpoint records.
#pragma once

#include <limits.h>

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

// One half of qk_epoch: acc = the scores of keys 32h + 16 i .. + 15 (the
// accumulator acc_i of qk_epoch).
template <int D, int I>
__device__ __forceinline__ void qk_half(const uint8_t* lk, const v4i* qreg, const int (&koff)[D / 32], v16i& acc) {
  acc = v16i{};
#pragma unroll
  for (int s = 0; s < D / 32; ++s) {
    const v4i a = *reinterpret_cast<const v4i*>(lk + koff[s] + 16 * D * I);
    acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, qreg[s], acc, 0, 0, 0);
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

// Two fp32 values -> two bf16 (x0 in the low half), round to nearest even:
// one v_cvt_pk_bf16_f32 (two scalar conversions would each fill half a
// register and need a shift and an or to combine).
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack2_bf16(float x0, float x1) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){x0, x1}, v2bf));
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
// Copy instructions of one tile (64 lanes x 16 bytes each) are dealt to the
// NW waves of the workgroup round-robin: wave w issues instructions w,
// w + NW, ... (with fewer instructions than waves, the last waves issue none).
template <int kInstr, int NW>
constexpr int kInstrPerWave = (kInstr + NW - 1) / NW;

template <int D, int NW = 4>
__device__ __forceinline__ void k_tile_to_lds(__amdgpu_buffer_rsrc_t rsrc, int tile, uint8_t* lds, int w,
                                              int lane) {
  constexpr int kInstr = kBlock * D / 16 / 64;
#pragma unroll
  for (int j = 0; j < kInstrPerWave<kInstr, NW>; ++j) {
    const int i = w + NW * j;
    if (kInstr % NW != 0 && i >= kInstr) break;  // wave-uniform
    const int p0 = i * 64;
    const int p = p0 + lane;
    const int key = p / (D / 16), pc = p % (D / 16);
    const int c = (k_lds_off<D>(key, pc) - key * D) >> 4;  // logical chunk at physical pc
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr_t)(lds + 16 * p0), 16, key * D + 16 * c, tile, 0, 0);
  }
}
template <int D, int NW = 4>
__device__ __forceinline__ void v_tile_to_lds(__amdgpu_buffer_rsrc_t rsrc, int tile, uint8_t* lds, int w,
                                              int lane) {
  constexpr int kInstr = D * kBlock / 16 / 64;
#pragma unroll
  for (int j = 0; j < kInstrPerWave<kInstr, NW>; ++j) {
    const int i = w + NW * j;
    if (kInstr % NW != 0 && i >= kInstr) break;  // wave-uniform
    const int p0 = i * 64;
    const int p = p0 + lane;
    const int row = p / 4, pc = p % 4;
    const int c = (v_lds_off(row, pc) - row * 64) >> 4;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr_t)(lds + 16 * p0), 16, row * 64 + 16 * c, tile, 0, 0);
  }
}

// Byte offset of 16-byte chunk `chunk` of query row `row` in an LDS Q tile
// of 32 NW rows x D bytes. Rows r and r + 256/D start at the same bank, so the
// chunk index is XORed with row / (256/D): the 16 rows that one b128 read of
// the QK step touches (rows q .. q + 15, one chunk each) then cover all 64
// banks once.
template <int D>
__device__ __forceinline__ int q_swz(int row) {
  return (row / (256 / D)) & (D / 16 - 1);
}
template <int D>
__device__ __forceinline__ int q_lds_off(int row, int chunk) {
  return row * D + ((chunk ^ q_swz<D>(row)) << 4);
}

// The (32 NW) x D Q code tile of rows q0 .. q0 + 32 NW - 1 of one head,
// copied straight into LDS (direct buffer loads; wave w of NW copies its
// share). rsrc spans the head's NQB*64 code rows: rows past them read as 0.
template <int D, int NW = 4>
__device__ __forceinline__ void q_tile_to_lds(__amdgpu_buffer_rsrc_t rsrc, int q0, uint8_t* lds, int w, int lane) {
  constexpr int kInstr = 32 * NW * D / 16 / 64;
  constexpr int kChunksPerRow = D / 16;
#pragma unroll
  for (int j = 0; j < kInstrPerWave<kInstr, NW>; ++j) {
    const int p0 = (w + NW * j) * 64;
    const int p = p0 + lane;
    const int row = p / kChunksPerRow, pc = p % kChunksPerRow;
    const int c = pc ^ q_swz<D>(row);  // logical chunk at physical pc
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr_t)(lds + 16 * p0), 16, row * D + 16 * c, q0 * D, 0, 0);
  }
}

// QK of one epoch with the Q codes read from an LDS Q tile (qoff[s]: this
// lane's Q chunk offsets); otherwise as qk_epoch.
template <int D>
__device__ __forceinline__ void qk_epoch_lq(const uint8_t* lk, const uint8_t* lq, const int (&qoff)[D / 32],
                                            const int (&koff)[D / 32], v16i& acc0, v16i& acc1) {
  acc0 = v16i{};
  acc1 = v16i{};
#pragma unroll
  for (int s = 0; s < D / 32; ++s) {
    const v4i b = *reinterpret_cast<const v4i*>(lq + qoff[s]);
    const v4i a0 = *reinterpret_cast<const v4i*>(lk + koff[s]);
    const v4i a1 = *reinterpret_cast<const v4i*>(lk + koff[s] + 16 * D);
    acc0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a0, b, acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, b, acc1, 0, 0, 0);
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


// Work item n of the grid order. Workgroups are dealt to the 8 XCDs
// round-robin, so item n runs on XCD n % 8; with B*H a multiple of 8 both
// orders keep every tile of a head on one XCD and its L2.
//  * heaviest first (causal, or B*H not a multiple of 8): consecutive items
//    walk the heads, the causal tiles with the most keys first;
//  * head-grouped (a.grouped: not causal, B*H a multiple of 8): XCD x runs
//    heads x, x + 8, x + 16, ... one after another, so all its tiles in flight
//    stream one head's K and V (3x less HBM fetch and 2 % faster at
//    B1 H24 L32760 than heaviest first; causal grids lose more to the
//    imbalance of the tail).
__device__ __forceinline__ void work_item(const AttnArgs& a, int n, int& tile, long& bh) {
  const int BH = a.B * a.H;
  if (a.grouped) {
    const int k = n / 8;
    tile = a.n_qtiles - 1 - k % a.n_qtiles;
    bh = n % 8 + 8 * (k / a.n_qtiles);
    return;
  }
  tile = a.n_qtiles - 1 - n / BH;
  bh = n % BH;
}

// ------------------------------------------------------------ epoch steps

// Maximum of one lane's 32 scores with the hidden ones (index t > dlim) left
// out; INT_MIN when all are hidden. Streams through the scores, so no masked
// copy of them is held.
__device__ __forceinline__ int row_max32_masked(const int (&x)[32], int dlim) {
  auto v = [&](int t) { return t > dlim ? INT_MIN : x[t]; };
  int mx = max(max(v(0), v(1)), v(2));
#pragma unroll
  for (int t = 3; t < 31; t += 2) mx = max(max(mx, v(t)), v(t + 1));
  return max(mx, v(31));
}

// p = exp2(S c - m) for 4 consecutive keys of this lane (x[4d .. 4d+3]),
// packed to E4M3 and added to the row sum in key order; hidden keys (index
// > dlim) get p = 0.
template <bool MASKED>
__device__ __forceinline__ int p4(const int (&x)[32], int d, float c, float m_use, int dlim, float& ps) {
  float p[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float e = __builtin_amdgcn_exp2f(__builtin_fmaf((float)x[4 * d + j], c, -m_use));
    p[j] = (MASKED && 4 * d + j > dlim) ? 0.0f : e;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) ps = (d == 0 && j == 0) ? p[0] : ps + p[j];
  return pack4_fp8(p[0], p[1], p[2], p[3]);
}

// Online softmax of one 64-key epoch for the 32 queries of a wave.
//   acc0, acc1  exact int32 scores: lane (h, q) holds S[q][32h + 16i + r] in
//               acc_i[r] (i = 0, 1);
//   c           log2-domain score per accumulator unit (sq sk sm_scale log2e);
//   masked      (wave-uniform) some key of the epoch lies past some lane's
//               last visible key; then keys with index > dlim are hidden and
//               `sees` tells whether the lane's row sees any key of the epoch.
// Updates the running max m (log2 domain) and the lane's partial row sum l
// (the two lane halves of a query hold the sums of their 32 keys). Returns
// the E4M3 bytes of p (the PV step's B operand), alpha = exp2(m_old - m_new)
// and whether any lane's max moved (else alpha == 1 in every lane).
// Hidden scores are only kept out of the row max and have p = 0, so the
// unmasked path carries no select.
// hook(i) is called once the scores of acc_i have been consumed (i = 0
// after the first 16 keys' probabilities, i = 1 at the end), so that a
// caller can refill that accumulator; the default does nothing.
struct NoHook {
  __device__ __forceinline__ void operator()(int) const {}
};

// Large scores. The direct exponent fma(S, c, -m) carries the rounding error
// of the running max m = RN(Smax c) (up to half an ulp of m) into every key
// of the epoch. Within an epoch that factor multiplies P and l alike, and
// while |m| < 2^12 it is below 2^-13 of an exponent unit; but at very large
// scores it would push the top key's p far above 1, past the E4M3 range.
// When some row of the wave has |m| >= 2^12 (wave-uniform test, one compare
// per epoch), the epoch takes its scores relative to the row's integer max
// instead: p = exp2((S - Smax) c - (m - m_e)), with S - Smax exact (|S| <
// 2^22) and m - m_e >= 0 (m_e = RN(Smax c), the epoch's own max), so every
// exponent is <= 0 and the top key of the epoch that set m gets p = 1.
constexpr float kRebaseLog2 = 4096.0f;
__device__ __forceinline__ bool large_scores(float m_use) {
  return __builtin_amdgcn_ballot_w64(__builtin_fabsf(m_use) >= kRebaseLog2) != 0;
}

// p4 in the large-score form: x[t] - mx is taken in unsigned arithmetic (for
// a lane that sees no key of the epoch mx is INT_MIN and the difference
// wraps; such keys are hidden, p = 0), dm = m - m_e (+inf for such a lane).
template <bool MASKED>
__device__ __forceinline__ int p4_rebased(const int (&x)[32], int d, int mx, float c, float dm, int dlim,
                                          float& ps) {
  float p[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int t = 4 * d + j;
    const float e = __builtin_amdgcn_exp2f(__builtin_fmaf((float)(int)((unsigned)x[t] - (unsigned)mx), c, -dm));
    p[j] = (MASKED && t > dlim) ? 0.0f : e;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) ps = (d == 0 && j == 0) ? p[0] : ps + p[j];
  return pack4_fp8(p[0], p[1], p[2], p[3]);
}

template <typename Hook = NoHook>
__device__ __forceinline__ void softmax_epoch(const v16i& acc0, const v16i& acc1, float c, bool masked,
                                              int dlim, bool sees, float& m, float& l, v8i& pb, float& alpha,
                                              bool& moved, Hook hook = Hook{}) {
  int x[32];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    x[r] = acc0[r];
    x[16 + r] = acc1[r];
  }
  float ps;
  if (masked) {
    const int mx = half_max(row_max32_masked(x, dlim));
    const float mt = sees ? (float)mx * c : -INFINITY;
    // mt > m is the only way the running max changes (neither is NaN), so
    // one compare gives both the new max and the lanes that moved.
    const bool up = mt > m;
    const float m_new = up ? mt : m;
    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
    alpha = __builtin_amdgcn_exp2f(m - m_use);
    moved = __builtin_amdgcn_ballot_w64(up) != 0;
    if (large_scores(m_use)) {
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        pb[d] = p4_rebased<true>(x, d, mx, c, m_use - mt, dlim, ps);
        if (d == 3) hook(0);
      }
    } else {
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        pb[d] = p4<true>(x, d, c, m_use, dlim, ps);
        if (d == 3) hook(0);
      }
    }
    m = m_new;
  } else {
    const int mx = half_max(row_max32(x));
    const float mt = (float)mx * c;
    const bool up = mt > m;
    const float m_new = up ? mt : m;
    alpha = __builtin_amdgcn_exp2f(m - m_new);
    moved = __builtin_amdgcn_ballot_w64(up) != 0;
    if (large_scores(m_new)) {
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        pb[d] = p4_rebased<false>(x, d, mx, c, m_new - mt, dlim, ps);
        if (d == 3) hook(0);
      }
    } else {
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        pb[d] = p4<false>(x, d, c, m_new, dlim, ps);
        if (d == 3) hook(0);
      }
    }
    m = m_new;
  }
  hook(1);
  l = __builtin_fmaf(l, alpha, ps);
}

// PV step of one epoch: ro[cb] += V^T[32 cb .. 32 cb + 31][epoch keys] . P^T
// (v_mfma_f32_32x32x64_f8f6f4, fp32 accumulate; lane (h, q) of ro[cb] holds
// channels 32 cb + 8 (r / 4) + 4 h + r % 4 of query q).
template <int D>
__device__ __forceinline__ void pv_epoch(const uint8_t* v_cur, const v8i& pb, v16f* ro, int h, int ql) {
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb) {
    const int ch = 32 * cb + ql;
    const v4i lo = *reinterpret_cast<const v4i*>(v_cur + v_lds_off(ch, 2 * h));
    const v4i hi = *reinterpret_cast<const v4i*>(v_cur + v_lds_off(ch, 2 * h + 1));
    const v8i av = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    ro[cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, pb, ro[cb], 0, 0, 0, 127, 0, 127);
  }
}

// The first epoch's PV step: RO = PV, the accumulator operand a zero
// constant (RO needs no clearing, and 0 * alpha + PV is PV exactly).
template <int D>
__device__ __forceinline__ void pv_epoch_first(const uint8_t* v_cur, const v8i& pb, v16f* ro, int h, int ql) {
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb) {
    const int ch = 32 * cb + ql;
    const v4i lo = *reinterpret_cast<const v4i*>(v_cur + v_lds_off(ch, 2 * h));
    const v4i hi = *reinterpret_cast<const v4i*>(v_cur + v_lds_off(ch, 2 * h + 1));
    const v8i av = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    ro[cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, pb, v16f{}, 0, 0, 0, 127, 0, 127);
  }
}

// Channel of register r of ro[cb] in lane half h.
__device__ __forceinline__ int ro_channel(int cb, int r, int h) { return 32 * cb + 8 * (r / 4) + 4 * h + r % 4; }

// Epilogue of a wave's 32 rows: out = bf16(RO * rcp * sv[c]) for rows < Lq.
// A wave's 32 output rows are consecutive in memory, so the bf16 values go
// through the LDS area `stage` (32 rows x 2D bytes, free when called) and
// leave as whole 16-byte chunks of consecutive rows: scattered 8-byte stores
// of the register layout cost more than the arithmetic of the epilogue.
template <int D>
__device__ __forceinline__ void store_rows(const v16f* ro, float rcp, const float* s_sv, uint8_t* stage,
                                           uint16_t* out, long bh, int Lq, int wrow0, int lane, int h, int ql) {
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
  uint16_t* obase = out + (bh * Lq + wrow0) * (long)D;
#pragma unroll
  for (int i = 0; i < 32 * kChunksPerRow / 64; ++i) {
    const int gi = lane + 64 * i, row = gi / kChunksPerRow, chunk = gi % kChunksPerRow;
    const uint4 val = *reinterpret_cast<const uint4*>(stage + out_lds_off<D>(row, chunk));
    if (wrow0 + row < Lq) *reinterpret_cast<uint4*>(obase + (long)row * D + 8 * chunk) = val;
  }
}

// ------------------------------------------------------------ checkpoints

// Trace records of one epoch e for the traced wave's 32 rows (layouts in
// sage_attn.h): m, l, alpha and the P bytes (from the wave that ran the
// softmax), RO after the epoch and the epoch's own PV partial (from the wave
// that ran the PV step).
__device__ __forceinline__ void trace_softmax(const AttnArgs& a, int e, int h, int ql, float m, float l,
                                              float alpha, const v8i& pb) {
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
}
template <int D>
__device__ __forceinline__ void trace_pv(const AttnArgs& a, int e, int h, int ql, const v16f* ro,
                                         const v16f* pv) {
  float* rt = a.tr_ro + ((long)ql * a.nkb + e) * D;
  float* pt = a.tr_pv + ((long)ql * a.nkb + e) * D;
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      rt[ro_channel(cb, r, h)] = ro[cb][r];
      pt[ro_channel(cb, r, h)] = pv[cb][r];
    }
}
__device__ __forceinline__ void trace_final(const AttnArgs& a, int h, int ql, float rcp, float lt) {
  if (h == 0) {
    float* st = a.tr_stats + ((long)ql * (a.nkb + 1) + a.nkb) * 4;
    st[0] = rcp;
    st[1] = lt;
    st[2] = 0.0f;
    st[3] = 0.0f;
  }
}

}  // namespace sage
