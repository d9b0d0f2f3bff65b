// Preparation pass on gfx950: K channel mean, K smoothing, INT8 block codes
// of Q and K, per-channel E4M3FN codes of V.
//
// Experiment Log (vortex_exact_attention), "Phase 0 Import And Verification":
// the imported contract starts with Q/K preparation, K smoothing, INT8
// quantization and FP8 V. The pass is bound by HBM bandwidth; three launches:
//   stats    - one read of K and V: per (head, 256-row split) fp64 channel sums
//              of K and fp32 channel absmax of V (16-byte coalesced loads);
//   finalize - per head: mean = fp32(sum / Lkv), sv = absmax / 448 (the
//              splits spread over the workgroup);
//   quant    - one read of Q, K, V per 64-row block: block absmax, codes.
// With few splits per head the finalize launch is skipped: each K or V
// workgroup of the quantization pass reduces the splits of its head itself,
// and the head's first K and V workgroups write the means and scales. With
// short key sets the statistics launch is skipped as well: each K or V
// workgroup of the quantization pass reduces its whole head (head_stats).
// Every quotient is the correctly rounded fp32 (or fp64) one, as an IEEE
// division gives. The K channel sums are fp64 sums over 256-row splits, then
// over the splits: bf16 values carry 8 significant bits, so when a channel's
// nonzero magnitudes lie in [2^e_min, 2^(e_max + 1)) with
// e_max - e_min <= 45 - ceil(log2 Lkv), every partial sum is a multiple of
// 2^(e_min - 7) of magnitude below 2^53 such units: exact, so the split order
// cannot change a bit of the mean. Outside that range (values spread over more binades) the
// last bits of the sum, and rarely of the fp32 mean, may depend on the order.
#include "sage_device.h"
#include "sage_launch.h"

namespace sage {

constexpr int kStatRows = 256;  // key rows per statistics workgroup (one split)

template <int D>
__global__ __launch_bounds__(kThreads) void prep_stats_kernel(const uint16_t* __restrict__ k,
                                                              const uint16_t* __restrict__ v, int Lkv,
                                                              int n_split, double* __restrict__ psum,
                                                              float* __restrict__ pmax) {
  constexpr int kLanesPerRow = D / 8;
  constexpr int kRowsPerIter = kThreads / kLanesPerRow;
  __shared__ double s_sum[kRowsPerIter][D];
  __shared__ float s_max[kRowsPerIter][D];

  // One-dimensional grid (its y extent is capped at 2^16): split-minor.
  const int split = (int)(blockIdx.x % n_split);
  const long bh = blockIdx.x / n_split;
  const int tid = threadIdx.x;
  const int cg = tid % kLanesPerRow, rg = tid / kLanesPerRow;
  const int t0 = split * kStatRows;
  const int t1 = min(t0 + kStatRows, Lkv);
  const uint16_t* kh = k + bh * (long)Lkv * D;
  const uint16_t* vh = v + bh * (long)Lkv * D;

  // Rows are taken kBatch at a time with every load of a batch issued first
  // (rows past the end read as zero, which changes neither statistic).
  constexpr int kBatch = 4;
  static_assert(kStatRows % (kRowsPerIter * kBatch) == 0, "split is whole batches");
  double s[8];
  float mx[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) { s[i] = 0.0; mx[i] = 0.0f; }
  for (int t = t0 + rg; t < t0 + kStatRows; t += kBatch * kRowsPerIter) {
    uint4 uk[kBatch], uv[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int r = t + u * kRowsPerIter;
      uk[u] = r < t1 ? *reinterpret_cast<const uint4*>(kh + (long)r * D + 8 * cg) : make_uint4(0, 0, 0, 0);
      uv[u] = r < t1 ? *reinterpret_cast<const uint4*>(vh + (long)r * D + 8 * cg) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      float fk[8], fv[8];
      unpack8(uk[u], fk);
      unpack8(uv[u], fv);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        s[i] += (double)fk[i];
        mx[i] = fmaxf(mx[i], fabsf(fv[i]));
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    s_sum[rg][8 * cg + i] = s[i];
    s_max[rg][8 * cg + i] = mx[i];
  }
  __syncthreads();
  if (tid < D) {
    double a = 0.0;
    float m = 0.0f;
    for (int r = 0; r < kRowsPerIter; ++r) {
      a += s_sum[r][tid];
      m = fmaxf(m, s_max[r][tid]);
    }
    psum[(bh * n_split + split) * D + tid] = a;
    pmax[(bh * n_split + split) * D + tid] = m;
  }
}

// Per head: mean = fp32(sum / Lkv) and sv = absmax / 448 from the split
// partials. A workgroup takes kFinChannels channels of one head; its
// kThreads / kFinChannels thread groups each take every G-th split with four
// loads in flight, then combine through LDS (the order matters only when the
// channel sum is not exact; see the file header).
constexpr int kFinChannels = 32;
template <int D>
__global__ __launch_bounds__(kThreads) void prep_finalize_kernel(const double* __restrict__ psum,
                                                                 const float* __restrict__ pmax, int n_split,
                                                                 int Lkv, float* __restrict__ k_mean,
                                                                 float* __restrict__ v_scale) {
  constexpr int G = kThreads / kFinChannels;
  __shared__ double s_sum[G][kFinChannels];
  __shared__ float s_max[G][kFinChannels];
  const long bh = blockIdx.x / (D / kFinChannels);
  const int cl = threadIdx.x % kFinChannels, g = threadIdx.x / kFinChannels;
  const int c = (int)(blockIdx.x % (D / kFinChannels)) * kFinChannels + cl;
  const double* ps = psum + bh * n_split * (long)D + c;
  const float* pm = pmax + bh * n_split * (long)D + c;
  double a[4] = {0.0, 0.0, 0.0, 0.0};
  float m[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  int s = g;
  for (; s + 3 * G < n_split; s += 4 * G) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      a[u] += ps[(long)(s + u * G) * D];
      m[u] = fmaxf(m[u], pm[(long)(s + u * G) * D]);
    }
  }
  for (; s < n_split; s += G) {
    a[0] += ps[(long)s * D];
    m[0] = fmaxf(m[0], pm[(long)s * D]);
  }
  s_sum[g][cl] = (a[0] + a[1]) + (a[2] + a[3]);
  s_max[g][cl] = fmaxf(fmaxf(m[0], m[1]), fmaxf(m[2], m[3]));
  __syncthreads();
  if (g == 0) {
    double t = 0.0;
    float mx = 0.0f;
#pragma unroll
    for (int i = 0; i < G; ++i) {
      t += s_sum[i][cl];
      mx = fmaxf(mx, s_max[i][cl]);
    }
    k_mean[bh * D + c] = (float)(t / (double)Lkv);
    v_scale[bh * D + c] = mx / 448.0f;
  }
}

// Max over the workgroup of one float per thread (all threads get it).
__device__ __forceinline__ float block_max(float x, float* s_red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) s_red[w] = x;
  __syncthreads();
  x = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  __syncthreads();
  return x;
}

// This thread's share of one 64-row block of a [L][D] bf16 head: 16-byte
// chunks g = threadIdx.x + kThreads j, row g / (D / 8), columns 8 (g % (D / 8))
// .. +7; rows >= L read as zero.
template <int D>
struct Int8BlockLoad {
  static constexpr int kChunks = kBlock * D / 8 / kThreads;  // 8 values per chunk
  static constexpr int kLanesPerRow = D / 8;
  uint4 raw[kChunks];
  __device__ __forceinline__ void load(const uint16_t* __restrict__ x, int L, int blk) {
#pragma unroll
    for (int j = 0; j < kChunks; ++j) {
      const int g = threadIdx.x + kThreads * j;
      const int row = blk * kBlock + g / kLanesPerRow, c0 = 8 * (g % kLanesPerRow);
      raw[j] = (row < L) ? *reinterpret_cast<const uint4*>(x + (long)row * D + c0) : make_uint4(0, 0, 0, 0);
    }
  }
};

// INT8 codes of one loaded 64-row block (rows >= L are padding: excluded from
// the absmax and coded 0). sub[c] is subtracted from column c first (the K
// channel mean; nullptr for Q).
template <int D>
__device__ void quant_int8_block(const Int8BlockLoad<D>& ld, int L, int blk, const float* __restrict__ sub,
                                 int8_t* __restrict__ codes, float* __restrict__ scale, float* s_red) {
  constexpr int kChunks = Int8BlockLoad<D>::kChunks;
  constexpr int kLanesPerRow = Int8BlockLoad<D>::kLanesPerRow;
  const uint4* raw = ld.raw;
  float f[kChunks][8];
  float a = 0.0f;
#pragma unroll
  for (int j = 0; j < kChunks; ++j) {
    const int g = threadIdx.x + kThreads * j;
    const int row = blk * kBlock + g / kLanesPerRow, c0 = 8 * (g % kLanesPerRow);
    unpack8(raw[j], f[j]);
    if (row < L) {
      if (sub) {
#pragma unroll
        for (int i = 0; i < 8; ++i) f[j][i] = f[j][i] - sub[c0 + i];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(f[j][i]));
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) f[j][i] = 0.0f;
    }
  }
  a = block_max(a, s_red);
  const float s = a / 127.0f;
  if (threadIdx.x == 0) *scale = s;
  const bool fast = s >= kFastDivMinScale;  // uniform over the block
  const float r = fast ? 1.0f / s : 0.0f;
#pragma unroll
  for (int j = 0; j < kChunks; ++j) {
    const int g = threadIdx.x + kThreads * j;
    const int c0 = 8 * (g % kLanesPerRow);
    uint32_t w[2] = {0u, 0u};
    if (a != 0.0f) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float q = fast ? div_rn(f[j][i], s, r) : f[j][i] / s;
        w[i >> 2] |= code_i8(q) << (8 * (i & 3));
      }
    }
    *reinterpret_cast<uint2*>(codes + (long)(blk * kBlock) * D + (long)(g / kLanesPerRow) * D + c0) =
        make_uint2(w[0], w[1]);
  }
}

// E4M3FN codes of one 64-key block of V, written as a [D][64] tile (keys of a
// channel contiguous). Each work unit codes 4 consecutive keys x 8 channels,
// so every LDS write is a whole dword of one channel row. The quotient
// v / sv[c] is rounded to fp32 as an IEEE division would (div_rn, or a
// division when some scale of the head is tiny) and then converted by the
// hardware E4M3 conversion (nearest even; |v / sv| <= 448 up to rounding).
template <int D>
struct VBlockLoad {
  static constexpr int kUnits = (kBlock / 4) * (D / 8);
  static constexpr int kPerThread = (kUnits + kThreads - 1) / kThreads;
  uint4 raw[kPerThread][4];
  __device__ __forceinline__ void load(const uint16_t* __restrict__ v, int L, int blk) {
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
      const int u = threadIdx.x + kThreads * k;
      if (u >= kUnits) break;
      const int kq = u % (kBlock / 4), c0 = 8 * (u / (kBlock / 4));
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = blk * kBlock + 4 * kq + r;
        raw[k][r] = (row < L) ? *reinterpret_cast<const uint4*>(v + (long)row * D + c0) : make_uint4(0, 0, 0, 0);
      }
    }
  }
};

template <int D>
__device__ void quant_v_block(const VBlockLoad<D>& ld, int L, int blk, const float* __restrict__ sv,
                              const float* __restrict__ rv, bool fast, uint8_t* __restrict__ tile,
                              uint8_t* s_tile) {
  constexpr int kUnits = VBlockLoad<D>::kUnits;
#pragma unroll
  for (int k = 0; k < VBlockLoad<D>::kPerThread; ++k) {
    const int u = threadIdx.x + kThreads * k;
    if (u >= kUnits) break;
    const int kq = u % (kBlock / 4), c0 = 8 * (u / (kBlock / 4));
    const uint4* raw = ld.raw[k];
    float f[4][8];
#pragma unroll
    for (int r = 0; r < 4; ++r) unpack8(raw[r], f[r]);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float s = sv[c0 + i], rc = rv[c0 + i];
      float q[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool pad = blk * kBlock + 4 * kq + r >= L;
        q[r] = (pad || s == 0.0f) ? 0.0f : (fast ? div_rn(f[r][i], s, rc) : f[r][i] / s);
      }
      int word;
      asm volatile("" : "=v"(word));  // both halves are written below
      word = __builtin_amdgcn_cvt_pk_fp8_f32(q[0], q[1], word, false);
      word = __builtin_amdgcn_cvt_pk_fp8_f32(q[2], q[3], word, true);
      *reinterpret_cast<uint32_t*>(s_tile + (c0 + i) * kBlock + 4 * kq) = (uint32_t)word;
    }
  }
  __syncthreads();
  constexpr int kOut = D * kBlock / 16 / kThreads;
#pragma unroll
  for (int j = 0; j < kOut; ++j) {
    const int g = threadIdx.x + kThreads * j;
    *reinterpret_cast<uint4*>(tile + 16 * g) = *reinterpret_cast<const uint4*>(s_tile + 16 * g);
  }
}

// Most statistics splits per head for which the quantization workgroups reduce
// the splits themselves instead of a finalize launch (each K or V workgroup
// then reads n_split * D partials of its head).
constexpr int kFuseMaxSplits = 4;

// Channel c's mean and V scale of head bh from the split partials, with the
// finalize pass's arithmetic (exact sums, so the same bits as the finalize
// pass, under the condition in the file header).
// All of a channel's partials are loaded before any is added, so their
// latencies overlap (and overlap the block's own loads, issued earlier).
__device__ __forceinline__ float head_mean(const PrepArgs& a, long bh, int c) {
  const double* ps = a.psum + bh * (long)a.n_split * a.D + c;
  double x[kFuseMaxSplits];
#pragma unroll
  for (int s = 0; s < kFuseMaxSplits; ++s) x[s] = s < a.n_split ? ps[(long)s * a.D] : 0.0;
  double t = 0.0;
#pragma unroll
  for (int s = 0; s < kFuseMaxSplits; ++s) t += x[s];
  return (float)(t / (double)a.Lkv);
}
__device__ __forceinline__ float head_vscale(const PrepArgs& a, long bh, int c) {
  const float* pm = a.pmax + bh * (long)a.n_split * a.D + c;
  float x[kFuseMaxSplits];
#pragma unroll
  for (int s = 0; s < kFuseMaxSplits; ++s) x[s] = s < a.n_split ? pm[(long)s * a.D] : 0.0f;
  float m = 0.0f;
#pragma unroll
  for (int s = 0; s < kFuseMaxSplits; ++s) m = fmaxf(m, x[s]);
  return m / 448.0f;
}

// Short key sets: a K or V quantization workgroup computes its head's
// channel statistics itself, over all Lkv rows, with the statistics pass's
// loop (fp64 channel sums of K, fp32 channel absmax of V), so the whole
// preparation is one launch. Every K or V workgroup of a head reads the head
// (from L2 after the first), so K and V are read NKB times over; this is
// taken while those extra reads, (NKB - 1) * B * H * 2 * Lkv * D * 2 bytes,
// stay within kSelfStatsMaxBytes (they then cost less than a launch: the
// Q128 x KV192 fixture's preparation takes 6.3 instead of 9.3 us, while at
// B1 H8 L1000, 60 MB over, it would take 14.3 instead of 10.6 us). The sums
// are exact under the condition in the file header, so the means are the
// statistics pass's bits. Results go to out[c] (the mean, or the V scale
// absmax / 448) for every thread; red is the LDS area of the reduction.
constexpr double kSelfStatsMaxBytes = 8.0 * 1024 * 1024;
template <int D>
union SelfStatsLds {
  double sum[kThreads / (D / 8)][D];
  float max[kThreads / (D / 8)][D];
};
template <int D, bool IS_K>
__device__ void head_stats(const uint16_t* __restrict__ x, int L, SelfStatsLds<D>& red, float* out) {
  constexpr int kLanesPerRow = D / 8;
  constexpr int kRowsPerIter = kThreads / kLanesPerRow;
  constexpr int kBatch = 4;
  const int tid = threadIdx.x;
  const int cg = tid % kLanesPerRow, rg = tid / kLanesPerRow;
  double s[8];
  float mx[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) { s[i] = 0.0; mx[i] = 0.0f; }
  for (int t = rg; t < L; t += kBatch * kRowsPerIter) {
    uint4 u[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int r = t + b * kRowsPerIter;
      u[b] = r < L ? *reinterpret_cast<const uint4*>(x + (long)r * D + 8 * cg) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      float f[8];
      unpack8(u[b], f);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (IS_K) s[i] += (double)f[i];
        else mx[i] = fmaxf(mx[i], fabsf(f[i]));
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (IS_K) red.sum[rg][8 * cg + i] = s[i];
    else red.max[rg][8 * cg + i] = mx[i];
  }
  __syncthreads();
  if (tid < D) {
    double a = 0.0;
    float m = 0.0f;
    for (int r = 0; r < kRowsPerIter; ++r) {
      if (IS_K) a += red.sum[r][tid];
      else m = fmaxf(m, red.max[r][tid]);
    }
    out[tid] = IS_K ? (float)(a / (double)L) : m / 448.0f;
  }
}

// One workgroup per (tensor, 64-row block): job in [0, nq) codes a Q block,
// [nq, nq + nkb) a K block, [nq + nkb, nq + 2 nkb) a V block, with nq = nqb,
// or 0 when the main loop codes Q itself (skip_q).
template <int D, bool SELF>
__global__ __launch_bounds__(kThreads) void prep_quant_kernel(PrepArgs a) {
  __shared__ float s_red[4];
  __shared__ SelfStatsLds<D> s_self;  // referenced (and allocated) only when SELF
  __shared__ __attribute__((aligned(16))) uint8_t s_tile[D * kBlock];
  __shared__ float s_ch[D];  // K channel mean, or V channel scale
  __shared__ float s_rv[D];  // RN(1 / V channel scale)
  // One-dimensional grid (its y extent is capped at 2^16): job-minor.
  const int nq = a.skip_q ? 0 : a.nqb;
  const int n_jobs = nq + 2 * a.nkb;
  const int job = (int)(blockIdx.x % n_jobs);
  const long bh = blockIdx.x / n_jobs;
  // The block's data loads are issued before the per-head channel values are
  // read, so the two memory latencies overlap.
  if (job < nq) {
    Int8BlockLoad<D> ld;
    ld.load(a.q + bh * (long)a.Lq * D, a.Lq, job);
    quant_int8_block<D>(ld, a.Lq, job, nullptr, a.q_i8 + bh * (long)a.nqb * kBlock * D,
                        a.q_scale + bh * a.nqb + job, s_red);
  } else if (job < nq + a.nkb) {
    const int blk = job - nq;
    Int8BlockLoad<D> ld;
    ld.load(a.k + bh * (long)a.Lkv * D, a.Lkv, blk);
    if constexpr (SELF) {
      head_stats<D, true>(a.k + bh * (long)a.Lkv * D, a.Lkv, s_self, s_ch);
      __syncthreads();
      if (blk == 0 && threadIdx.x < D) a.k_mean[bh * D + threadIdx.x] = s_ch[threadIdx.x];
    } else if (threadIdx.x < D) {
      if (a.fuse_finalize) {
        const float mu = head_mean(a, bh, threadIdx.x);
        s_ch[threadIdx.x] = mu;
        if (blk == 0) a.k_mean[bh * D + threadIdx.x] = mu;
      } else {
        s_ch[threadIdx.x] = a.k_mean[bh * D + threadIdx.x];
      }
    }
    __syncthreads();
    quant_int8_block<D>(ld, a.Lkv, blk, s_ch, a.k_i8 + bh * (long)a.nkb * kBlock * D,
                        a.k_scale + bh * a.nkb + blk, s_red);
  } else {
    const int blk = job - nq - a.nkb;
    VBlockLoad<D> ld;
    ld.load(a.v + bh * (long)a.Lkv * D, a.Lkv, blk);
    bool tiny = false;
    if constexpr (SELF) {
      head_stats<D, false>(a.v + bh * (long)a.Lkv * D, a.Lkv, s_self, s_ch);
      __syncthreads();
    }
    if (threadIdx.x < D) {
      float s;
      if constexpr (SELF) {
        s = s_ch[threadIdx.x];
        if (blk == 0) a.v_scale[bh * D + threadIdx.x] = s;
      } else if (a.fuse_finalize) {
        s = head_vscale(a, bh, threadIdx.x);
        if (blk == 0) a.v_scale[bh * D + threadIdx.x] = s;
      } else {
        s = a.v_scale[bh * D + threadIdx.x];
      }
      s_ch[threadIdx.x] = s;
      tiny = s != 0.0f && !(s >= kFastDivMinScale);
      s_rv[threadIdx.x] = tiny || s == 0.0f ? 0.0f : 1.0f / s;
    }
    const bool fast = !__syncthreads_or(tiny);
    quant_v_block<D>(ld, a.Lkv, blk, s_ch, s_rv, fast,
                     a.v_fp8 + (bh * a.nkb + blk) * (long)D * kBlock, s_tile);
  }
}

int prep_n_split(int Lkv) { return (Lkv + kStatRows - 1) / kStatRows; }

template <int D>
static hipError_t launch_prep_t(PrepArgs a, hipStream_t stream) {
  const int BH = a.B * a.H;
  const int ns = a.n_split;
  // The host bounds every flattened grid below 2^31 workgroups.
  const dim3 g_stats((unsigned)((long)ns * BH)), g_fin((unsigned)((long)BH * (D / kFinChannels))),
      g_quant((unsigned)((long)((a.skip_q ? 0 : a.nqb) + 2 * a.nkb) * BH));
  if (a.self_stats) {
    prep_quant_kernel<D, true><<<g_quant, kThreads, 0, stream>>>(a);
    return hipGetLastError();
  }
  prep_stats_kernel<D><<<g_stats, kThreads, 0, stream>>>(a.k, a.v, a.Lkv, ns, a.psum, a.pmax);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (!a.fuse_finalize) {
    prep_finalize_kernel<D><<<g_fin, kThreads, 0, stream>>>(a.psum, a.pmax, ns, a.Lkv, a.k_mean, a.v_scale);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  prep_quant_kernel<D, false><<<g_quant, kThreads, 0, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_prep(const PrepArgs& args, hipStream_t stream) {
  PrepArgs a = args;
  a.n_split = prep_n_split(a.Lkv);
  const double kv_bytes = 2.0 * a.B * a.H * (double)a.Lkv * a.D * 2;
  a.self_stats = (a.nkb - 1) * kv_bytes <= kSelfStatsMaxBytes;
  a.fuse_finalize = a.n_split <= kFuseMaxSplits;
  return a.D == 128 ? launch_prep_t<128>(a, stream) : launch_prep_t<64>(a, stream);
}

}  // namespace sage
