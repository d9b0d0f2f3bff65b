// Kernel argument blocks and launchers of the HIP library (internal header).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sage {

constexpr int kBlock = 64;      // quant block rows == attention epoch keys
constexpr int kThreads = 256;   // 4 wave64 per workgroup
constexpr int kQTile = 128;     // query rows per main-loop workgroup (32 per wave)

struct PrepArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  int B, H, Lq, Lkv, D, nqb, nkb;
  int8_t* q_i8;
  float* q_scale;
  int8_t* k_i8;
  float* k_scale;
  float* k_mean;
  uint8_t* v_fp8;
  float* v_scale;
  double* psum;  // [B*H][n_split][D] fp64 channel partial sums of K
  float* pmax;   // [B*H][n_split][D] channel absmax partials of V
  int n_split;   // statistics splits per head
  int fuse_finalize;  // 1: the quantization workgroups reduce the splits themselves
  int skip_q;         // 1: Q is not coded (the main loop codes it from q)
  int self_stats;     // 1: no statistics launch; K/V workgroups reduce their head themselves
};

struct AttnArgs {
  const int8_t* q_i8;
  const float* q_scale;
  const int8_t* k_i8;
  const float* k_scale;
  const uint8_t* v_fp8;
  const float* v_scale;
  uint16_t* out;
  const uint16_t* q;  // bf16 Q [B][H][Lq][D]: the entry design codes it (q_i8, q_scale unused)
  int B, H, Lq, Lkv, nqb, nkb, n_qtiles;
  int grouped;       // 1: head-grouped tile order (not causal, B*H a multiple of 8)
  float scale_log2;  // sm_scale * log2(e)
  // Per-epoch checkpoints (trace launches only): the workgroup runs tile
  // trace_tile of head trace_bh, and wave trace_wave writes its 32 rows'
  // state after every epoch (layouts in sage_attn.h).
  int trace_bh, trace_tile, trace_wave;
  float* tr_stats;
  uint8_t* tr_p8;
  float* tr_ro;
  float* tr_pv;
  // Persistent design: the launch-wide work counter (0 when a launch starts;
  // each launch leaves it at 0) and the number of workgroups.
  unsigned int* queue;
  int persist_grid;
};

constexpr int kMaxDebugTiles = 64;
struct QkDebugArgs {
  const int8_t* q_i8;
  const int8_t* k_i8;
  int32_t* acc_out;
  int Lq, Lkv, nqb, nkb, H, n;
  int tiles[kMaxDebugTiles][4];
};

// Main-loop kernel designs (the values of SAGE_KERNEL_* in sage_attn.h).
constexpr int kKernelFused = 1;  // every wave runs QK, softmax and PV for its rows
constexpr int kKernelSplit = 2;  // softmax waves and PV waves own separate state
constexpr int kKernelPersistent = 3;  // fused waves in persistent workgroups fed by a work counter
constexpr int kKernelWide = 4;        // fused waves in 8-wave (256-row) workgroups
constexpr int kKernelEntry = 5;       // fused waves that code their Q tile from bf16 themselves

// Query rows per workgroup of a main-loop design.
constexpr int tile_rows(int kernel) { return kernel == kKernelWide ? 256 : kQTile; }

int prep_n_split(int Lkv);
hipError_t launch_prep(const PrepArgs& a, hipStream_t stream);
hipError_t launch_attn(const AttnArgs& a, int D, bool causal, int kernel, hipStream_t stream);
hipError_t launch_attn_trace(const AttnArgs& a, int D, bool causal, int kernel, hipStream_t stream);
hipError_t launch_attn_fused(const AttnArgs& a, int D, bool causal, bool trace, hipStream_t stream);
hipError_t launch_attn_split(const AttnArgs& a, int D, bool causal, bool trace, hipStream_t stream);
hipError_t launch_attn_wide(const AttnArgs& a, int D, bool causal, bool trace, hipStream_t stream);
hipError_t launch_attn_entry(const AttnArgs& a, int D, bool causal, hipStream_t stream);
hipError_t launch_qk_debug(const QkDebugArgs& a, int D, hipStream_t stream);
hipError_t launch_codecs_debug(const float* x, int n, uint8_t* p8, uint16_t* bf16, hipStream_t stream);

}  // namespace sage
