// C ABI of the quantized attention library: argument validation, workspace
// layout and kernel launches. Declarations and contracts: include/sage_attn.h.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "sage_attn.h"
#include "sage_launch.h"

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool misaligned(const void* p, size_t a) { return ((uintptr_t)p % a) != 0; }

int check_dims(int B, int H, int Lq, int Lkv, int D) {
  if (B < 1 || H < 1 || Lq < 1 || Lkv < 1) return SAGE_ERR_INVALID_ARG;
  if (D != 64 && D != 128) return SAGE_ERR_UNSUPPORTED;
  const double elems = (double)B * H * (double)(Lq > Lkv ? Lq : Lkv) * D;
  if (elems >= 1099511627776.0) return SAGE_ERR_INVALID_ARG;  // 2^40
  const double qtiles = (double)B * H * ((Lq + sage::kQTile - 1) / sage::kQTile);
  if (qtiles >= 2147483647.0) return SAGE_ERR_INVALID_ARG;
  // One-dimensional preparation grids: B*H times the splits, the blocks or the
  // 32-channel groups.
  const double nqb = (Lq + sage::kBlock - 1) / sage::kBlock, nkb = (Lkv + sage::kBlock - 1) / sage::kBlock;
  if ((double)B * H * (nqb + 2 * nkb) >= 2147483647.0) return SAGE_ERR_INVALID_ARG;
  if ((double)B * H * sage::prep_n_split(Lkv) >= 2147483647.0) return SAGE_ERR_INVALID_ARG;
  if ((double)B * H * (D / 32) >= 2147483647.0) return SAGE_ERR_INVALID_ARG;
  // The main loop addresses one head's Q, K or V codes with 32-bit buffer
  // offsets.
  const double head_codes = (double)((Lkv + sage::kBlock - 1) / sage::kBlock) * sage::kBlock * D;
  if (head_codes >= 2147483648.0) return SAGE_ERR_INVALID_ARG;
  const double head_q = (double)((Lq + sage::kBlock - 1) / sage::kBlock) * sage::kBlock * D;
  if (head_q >= 2147483648.0) return SAGE_ERR_INVALID_ARG;
  return SAGE_OK;
}

struct Layout {
  size_t q_i8, q_scale, k_i8, k_scale, k_mean, v_fp8, v_scale, psum, pmax, total;
};

Layout layout(int B, int H, int Lq, int Lkv, int D) {
  const size_t bh = (size_t)B * H;
  const size_t nqb = (Lq + sage::kBlock - 1) / sage::kBlock, nkb = (Lkv + sage::kBlock - 1) / sage::kBlock;
  const size_t ns = sage::prep_n_split(Lkv);
  Layout l;
  size_t o = 0;
  l.q_i8 = o;    o = align_up(o + bh * nqb * sage::kBlock * D);
  l.q_scale = o; o = align_up(o + bh * nqb * sizeof(float));
  l.k_i8 = o;    o = align_up(o + bh * nkb * sage::kBlock * D);
  l.k_scale = o; o = align_up(o + bh * nkb * sizeof(float));
  l.k_mean = o;  o = align_up(o + bh * D * sizeof(float));
  l.v_fp8 = o;   o = align_up(o + bh * nkb * sage::kBlock * D);
  l.v_scale = o; o = align_up(o + bh * D * sizeof(float));
  l.psum = o;    o = align_up(o + bh * ns * D * sizeof(double));
  l.pmax = o;    o = align_up(o + bh * ns * D * sizeof(float));
  l.total = o;
  return l;
}

size_t prep_scratch(int B, int H, int Lkv, int D) {
  const size_t n = (size_t)B * H * sage::prep_n_split(Lkv) * D;
  return align_up(n * sizeof(double)) + align_up(n * sizeof(float));
}

int hip_status(hipError_t e) { return e == hipSuccess ? SAGE_OK : SAGE_ERR_HIP; }

// Scratch of sage_quant_prep_noalloc (the preparation pass's fp64 channel
// partial sums and fp32 channel absmax partials): a file-scope device array.
// Each GPU holds its own copy until the process ends; every call on a GPU
// uses that GPU's copy. In host code `scratch` only names the symbol: its
// device address comes from hipGetSymbolAddress, taken once per device with
// that device current, and only that address is passed to kernels.
constexpr size_t kStaticScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;

// Work counters of the persistent main-loop design: one set of 8 (one per
// XCD) per stream that has used it (calls on one stream run in order, so a
// set never serves two launches at once). Every launch leaves its counters at
// 0.
constexpr int kQueueSlots = 64;
constexpr int kQueuesPerSlot = 8;  // one counter per XCD
static __device__ unsigned int work_queue[kQueueSlots * kQueuesPerSlot];

struct QueueTable {
  unsigned int* base = nullptr;  // device address of work_queue
  int cus = 0;                   // compute units
  void* streams[kQueueSlots] = {};
  int used = 0;
};

// This device's counter for `stream` and its compute-unit count; nullptr when
// every slot is taken by other streams (the caller then runs the
// non-persistent design) or on a HIP error (*status set).
unsigned int* queue_for(void* stream, int* cus, int* status) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *status = SAGE_ERR_HIP;
    return nullptr;
  }
  static std::mutex mu;
  static QueueTable table[kMaxDevices];
  std::lock_guard<std::mutex> lock(mu);
  QueueTable& t = table[dev];
  if (!t.base) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(work_queue)) != hipSuccess || !p ||
        hipDeviceGetAttribute(&t.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
      *status = SAGE_ERR_HIP;
      return nullptr;
    }
    t.base = (unsigned int*)p;
  }
  *cus = t.cus;
  for (int i = 0; i < t.used; ++i)
    if (t.streams[i] == stream) return t.base + kQueuesPerSlot * i;
  if (t.used == kQueueSlots) return nullptr;
  t.streams[t.used] = stream;
  return t.base + kQueuesPerSlot * t.used++;
}

// Device address of this device's `scratch` (nullptr and *status set on a
// HIP error).
void* static_scratch(int* status) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *status = SAGE_ERR_HIP;
    return nullptr;
  }
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      *status = SAGE_ERR_HIP;
      return nullptr;
    }
    addr[dev] = p;
  }
  return addr[dev];
}

// The main-loop design SAGE_KERNEL_AUTO selects on prepared operands. When
// the grid has fewer
// 128-row tiles than the GPU has compute units, the wave-specialised design
// finishes each tile sooner (twice the waves per tile: 0.0180 against
// 0.0204 ms at B1 H8 L1000 D128 causal); on full grids the fused design is
// faster (0.175 against 0.192 ms at B2 H32 L4096 D128 causal).
constexpr long kAutoSplitMaxTiles = 256;
int auto_kernel(int B, int H, int Lq) {
  const long tiles = (long)B * H * ((Lq + sage::kQTile - 1) / sage::kQTile);
  return tiles < kAutoSplitMaxTiles ? sage::kKernelSplit : sage::kKernelFused;
}

// The automatic choice of the whole path: on full grids the entry design
// (Q coded inside the main loop; the preparation pass codes K and V only) is
// faster end to end (0.249 against 0.256 ms at B2 H32 L4096 D128 causal,
// 0.521 against 0.532 ms at B4 H16 L8192 D64 causal, 7.83 against 7.92 ms at
// B1 H24 L32760 D128); below the split threshold the split design stays.
int auto_kernel_whole(int B, int H, int Lq) {
  const int k = auto_kernel(B, H, Lq);
  return k == sage::kKernelFused ? sage::kKernelEntry : k;
}

// SAGE_KERNEL_* -> launcher kind; -1 for an unknown value.
int resolve_kernel(int kernel, int B, int H, int Lq, bool whole_path = false) {
  if (kernel == SAGE_KERNEL_AUTO) return whole_path ? auto_kernel_whole(B, H, Lq) : auto_kernel(B, H, Lq);
  if (kernel == SAGE_KERNEL_FUSED) return sage::kKernelFused;
  if (kernel == SAGE_KERNEL_SPLIT) return sage::kKernelSplit;
  if (kernel == SAGE_KERNEL_PERSISTENT) return sage::kKernelPersistent;
  if (kernel == SAGE_KERNEL_WIDE) return sage::kKernelWide;
  if (kernel == SAGE_KERNEL_ENTRY) return sage::kKernelEntry;
  return -1;
}

// Shapes and the input/output pointers of the preparation pass.
// Shapes and the input/output pointers of the preparation pass (without Q's
// input and outputs when kv_only).
int check_prep_args(const void* q, const void* k, const void* v, int B, int H, int Lq, int Lkv, int D,
                    const int8_t* q_i8, const float* q_scale, const int8_t* k_i8, const float* k_scale,
                    const float* k_mean, const uint8_t* v_fp8, const float* v_scale, bool kv_only = false) {
  const int st = check_dims(B, H, Lq, Lkv, D);
  if (st != SAGE_OK) return st;
  if (!k || !v || !k_i8 || !k_scale || !k_mean || !v_fp8 || !v_scale) return SAGE_ERR_INVALID_ARG;
  if (!kv_only && (!q || !q_i8 || !q_scale)) return SAGE_ERR_INVALID_ARG;
  if (misaligned(k, 16) || misaligned(v, 16) || misaligned(k_i8, 16) || misaligned(v_fp8, 16) ||
      misaligned(k_scale, 4) || misaligned(k_mean, 16) || misaligned(v_scale, 16))
    return SAGE_ERR_INVALID_ARG;
  if (!kv_only && (misaligned(q, 16) || misaligned(q_i8, 16) || misaligned(q_scale, 4))) return SAGE_ERR_INVALID_ARG;
  return SAGE_OK;
}

// Body of sage_quant_prep (also run by sage_attn_fwd on its workspace);
// skip_q codes K and V only (q, q_i8 and q_scale are then not used).
int quant_prep(const void* q, const void* k, const void* v, int B, int H, int Lq, int Lkv, int D,
               int8_t* q_i8, float* q_scale, int8_t* k_i8, float* k_scale, float* k_mean, uint8_t* v_fp8,
               float* v_scale, void* scratch, size_t scratch_bytes, void* stream, bool skip_q = false) {
  const int st = check_prep_args(q, k, v, B, H, Lq, Lkv, D, q_i8, q_scale, k_i8, k_scale, k_mean, v_fp8, v_scale,
                                 skip_q);
  if (st != SAGE_OK) return st;
  if (!scratch || misaligned(scratch, 8)) return SAGE_ERR_INVALID_ARG;
  if (scratch_bytes < prep_scratch(B, H, Lkv, D)) return SAGE_ERR_WORKSPACE;
  const size_t n = (size_t)B * H * sage::prep_n_split(Lkv) * D;
  sage::PrepArgs a;
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.B = B; a.H = H; a.Lq = Lq; a.Lkv = Lkv; a.D = D;
  a.nqb = (Lq + sage::kBlock - 1) / sage::kBlock;
  a.nkb = (Lkv + sage::kBlock - 1) / sage::kBlock;
  a.q_i8 = q_i8; a.q_scale = q_scale; a.k_i8 = k_i8; a.k_scale = k_scale; a.k_mean = k_mean;
  a.v_fp8 = v_fp8; a.v_scale = v_scale;
  a.psum = (double*)scratch;
  a.pmax = (float*)((char*)scratch + align_up(n * sizeof(double)));
  a.skip_q = skip_q ? 1 : 0;
  return hip_status(sage::launch_prep(a, (hipStream_t)stream));
}


// Validation and argument block shared by the main-loop entry points.
// q_bf16 (the entry design: bf16 Q, coded by the main loop) replaces q_i8
// and q_scale when it is not null.
int attn_args(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8, const float* k_scale,
              const uint8_t* v_fp8, const float* v_scale, void* out, int B, int H, int Lq, int Lkv, int D,
              int causal, float sm_scale, sage::AttnArgs* a, const void* q_bf16 = nullptr) {
  const int st = check_dims(B, H, Lq, Lkv, D);
  if (st != SAGE_OK) return st;
  if (!k_i8 || !k_scale || !v_fp8 || !v_scale || !out) return SAGE_ERR_INVALID_ARG;
  if (!q_bf16 && (!q_i8 || !q_scale)) return SAGE_ERR_INVALID_ARG;
  if (misaligned(k_i8, 16) || misaligned(v_fp8, 16) || misaligned(out, 16) || misaligned(k_scale, 4) ||
      misaligned(v_scale, 16))
    return SAGE_ERR_INVALID_ARG;
  if (q_bf16 ? misaligned(q_bf16, 16) : (misaligned(q_i8, 16) || misaligned(q_scale, 4)))
    return SAGE_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return SAGE_ERR_INVALID_ARG;
  if (isnan(sm_scale) || isinf(sm_scale)) return SAGE_ERR_INVALID_ARG;
  if (sm_scale <= 0.0f) sm_scale = 1.0f / sqrtf((float)D);
  *a = sage::AttnArgs{};
  a->q_i8 = q_i8; a->q_scale = q_scale; a->k_i8 = k_i8; a->k_scale = k_scale;
  a->v_fp8 = v_fp8; a->v_scale = v_scale; a->out = (uint16_t*)out;
  a->B = B; a->H = H; a->Lq = Lq; a->Lkv = Lkv;
  a->nqb = (Lq + sage::kBlock - 1) / sage::kBlock;
  a->nkb = (Lkv + sage::kBlock - 1) / sage::kBlock;
  a->n_qtiles = (Lq + sage::kQTile - 1) / sage::kQTile;
  a->scale_log2 = sm_scale * 1.4426950408889634f;
  a->grouped = causal == 0 && (B * H) % 8 == 0;
  a->q = (const uint16_t*)q_bf16;
  return SAGE_OK;
}

}  // namespace

extern "C" {

const char* sage_status_str(int status) {
  switch (status) {
    case SAGE_OK: return "SAGE_OK";
    case SAGE_ERR_INVALID_ARG: return "SAGE_ERR_INVALID_ARG";
    case SAGE_ERR_UNSUPPORTED: return "SAGE_ERR_UNSUPPORTED";
    case SAGE_ERR_WORKSPACE: return "SAGE_ERR_WORKSPACE";
    case SAGE_ERR_HIP: return "SAGE_ERR_HIP";
    default: return "SAGE_ERR_UNKNOWN";
  }
}

int sage_prep_scratch_bytes(int B, int H, int Lq, int Lkv, int D, size_t* bytes) {
  if (!bytes) return SAGE_ERR_INVALID_ARG;
  const int st = check_dims(B, H, Lq, Lkv, D);
  if (st != SAGE_OK) return st;
  *bytes = prep_scratch(B, H, Lkv, D);
  return SAGE_OK;
}

int sage_workspace_bytes(int B, int H, int Lq, int Lkv, int D, size_t* bytes) {
  if (!bytes) return SAGE_ERR_INVALID_ARG;
  const int st = check_dims(B, H, Lq, Lkv, D);
  if (st != SAGE_OK) return st;
  *bytes = layout(B, H, Lq, Lkv, D).total;
  return SAGE_OK;
}

int sage_quant_prep(const void* q, const void* k, const void* v, int B, int H, int Lq, int Lkv, int D,
                    int8_t* q_i8, float* q_scale, int8_t* k_i8, float* k_scale, float* k_mean,
                    uint8_t* v_fp8, float* v_scale, void* scratch, size_t scratch_bytes, void* stream) {
  return quant_prep(q, k, v, B, H, Lq, Lkv, D, q_i8, q_scale, k_i8, k_scale, k_mean, v_fp8, v_scale, scratch,
                    scratch_bytes, stream);
}

// Tiles per head for the design's tile height.
void set_tiles(sage::AttnArgs* a, int kind) {
  const int rows = sage::tile_rows(kind);
  a->n_qtiles = (a->Lq + rows - 1) / rows;
}

// Counter and grid of a persistent launch: one workgroup per resident slot
// (three per compute unit at D = 128, four at D = 64), at most one per work
// item. Falls back to the non-persistent design (*kind) when no counter is
// free for the stream; false on a HIP error.
bool persistent_setup(sage::AttnArgs* a, int D, void* stream, int* kind) {
  int cus = 0, st = SAGE_OK;
  a->queue = queue_for(stream, &cus, &st);
  if (st != SAGE_OK) return false;
  if (!a->queue) {
    *kind = sage::kKernelFused;
    return true;
  }
  const long items = (long)a->n_qtiles * a->B * a->H;
  const long slots = (long)cus * (D == 64 ? 4 : 3);
  a->persist_grid = (int)(items < slots ? items : slots);
  return true;
}

int sage_quant_prep_noalloc(const void* q, const void* k, const void* v, int B, int H, int Lq, int Lkv, int D,
                            int8_t* q_i8, float* q_scale, int8_t* k_i8, float* k_scale, float* k_mean,
                            uint8_t* v_fp8, float* v_scale, void* stream) {
  const int st = check_prep_args(q, k, v, B, H, Lq, Lkv, D, q_i8, q_scale, k_i8, k_scale, k_mean, v_fp8, v_scale);
  if (st != SAGE_OK) return st;
  if (prep_scratch(B, H, Lkv, D) > kStaticScratchBytes) return SAGE_ERR_WORKSPACE;
  int hs = SAGE_OK;
  void* ws = static_scratch(&hs);
  if (!ws) return hs;
  return quant_prep(q, k, v, B, H, Lq, Lkv, D, q_i8, q_scale, k_i8, k_scale, k_mean, v_fp8, v_scale, ws,
                    kStaticScratchBytes, stream);
}

int sage_attn_fwd_prepped_kernel(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                                 const float* k_scale, const uint8_t* v_fp8, const float* v_scale, void* out,
                                 int B, int H, int Lq, int Lkv, int D, int causal, float sm_scale, int kernel,
                                 void* stream) {
  sage::AttnArgs a;
  const int st = attn_args(q_i8, q_scale, k_i8, k_scale, v_fp8, v_scale, out, B, H, Lq, Lkv, D, causal,
                           sm_scale, &a);
  if (st != SAGE_OK) return st;
  int kind = resolve_kernel(kernel, B, H, Lq);
  if (kind < 0 || kind == sage::kKernelEntry) return SAGE_ERR_INVALID_ARG;  // entry: bf16 Q needed
  set_tiles(&a, kind);
  if (kind == sage::kKernelPersistent && !persistent_setup(&a, D, stream, &kind)) return SAGE_ERR_HIP;
  return hip_status(sage::launch_attn(a, D, causal == 1, kind, (hipStream_t)stream));
}

int sage_attn_fwd_prepped(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                          const float* k_scale, const uint8_t* v_fp8, const float* v_scale, void* out,
                          int B, int H, int Lq, int Lkv, int D, int causal, float sm_scale, void* stream) {
  return sage_attn_fwd_prepped_kernel(q_i8, q_scale, k_i8, k_scale, v_fp8, v_scale, out, B, H, Lq, Lkv, D,
                                      causal, sm_scale, SAGE_KERNEL_AUTO, stream);
}

// The trace record setup shared by the two trace entry points.
int trace_setup(sage::AttnArgs* a, int kind, int H, int Lq, int B, int b, int h, int row0, float* stats,
                uint8_t* p8, float* pv, float* ro) {
  set_tiles(a, kind);
  if (b < 0 || b >= B || h < 0 || h >= H || row0 < 0 || row0 >= Lq || row0 % 32 != 0) return SAGE_ERR_INVALID_ARG;
  if (!stats || !p8 || !pv || !ro || misaligned(stats, 16) || misaligned(p8, 4) || misaligned(pv, 4) ||
      misaligned(ro, 4))
    return SAGE_ERR_INVALID_ARG;
  a->trace_bh = b * H + h;
  a->trace_tile = row0 / sage::tile_rows(kind);
  a->trace_wave = (row0 % sage::tile_rows(kind)) / 32;
  a->tr_stats = stats;
  a->tr_p8 = p8;
  a->tr_pv = pv;
  a->tr_ro = ro;
  return SAGE_OK;
}

int sage_debug_epoch_trace(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8, const float* k_scale,
                           const uint8_t* v_fp8, const float* v_scale, void* out, int B, int H, int Lq, int Lkv,
                           int D, int causal, float sm_scale, int kernel, int b, int h, int row0, float* stats,
                           uint8_t* p8, float* pv, float* ro, void* stream) {
  sage::AttnArgs a;
  int st = attn_args(q_i8, q_scale, k_i8, k_scale, v_fp8, v_scale, out, B, H, Lq, Lkv, D, causal, sm_scale, &a);
  if (st != SAGE_OK) return st;
  int kind = resolve_kernel(kernel, B, H, Lq);
  if (kind < 0 || kind == sage::kKernelEntry) return SAGE_ERR_INVALID_ARG;
  if (kind == sage::kKernelPersistent) kind = sage::kKernelFused;  // the same tile code, traced on one tile
  st = trace_setup(&a, kind, H, Lq, B, b, h, row0, stats, p8, pv, ro);
  if (st != SAGE_OK) return st;
  return hip_status(sage::launch_attn_trace(a, D, causal == 1, kind, (hipStream_t)stream));
}

int sage_debug_epoch_trace_kv(const void* q, const int8_t* k_i8, const float* k_scale, const uint8_t* v_fp8,
                              const float* v_scale, void* out, int B, int H, int Lq, int Lkv, int D, int causal,
                              float sm_scale, int b, int h, int row0, float* stats, uint8_t* p8, float* pv,
                              float* ro, void* stream) {
  if (!q) return SAGE_ERR_INVALID_ARG;
  sage::AttnArgs a;
  int st = attn_args(nullptr, nullptr, k_i8, k_scale, v_fp8, v_scale, out, B, H, Lq, Lkv, D, causal, sm_scale,
                     &a, q);
  if (st != SAGE_OK) return st;
  st = trace_setup(&a, sage::kKernelEntry, H, Lq, B, b, h, row0, stats, p8, pv, ro);
  if (st != SAGE_OK) return st;
  return hip_status(sage::launch_attn_trace(a, D, causal == 1, sage::kKernelEntry, (hipStream_t)stream));
}

int sage_attn_fwd_kernel(const void* q, const void* k, const void* v, void* out, int B, int H, int Lq, int Lkv,
                         int D, int causal, float sm_scale, int kernel, void* workspace, size_t workspace_bytes,
                         void* stream) {
  const int st = check_dims(B, H, Lq, Lkv, D);
  if (st != SAGE_OK) return st;
  if (!q || !k || !v || !out || !workspace) return SAGE_ERR_INVALID_ARG;
  if (misaligned(workspace, kAlign) || misaligned(out, 16)) return SAGE_ERR_INVALID_ARG;
  int kind = resolve_kernel(kernel, B, H, Lq, true);
  if (kind < 0) return SAGE_ERR_INVALID_ARG;
  const Layout l = layout(B, H, Lq, Lkv, D);
  if (workspace_bytes < l.total) return SAGE_ERR_WORKSPACE;
  char* ws = (char*)workspace;
  // Every argument is checked, and the persistent design's counter taken,
  // before anything is launched.
  int s = check_prep_args(q, k, v, B, H, Lq, Lkv, D, (int8_t*)(ws + l.q_i8), (float*)(ws + l.q_scale),
                          (int8_t*)(ws + l.k_i8), (float*)(ws + l.k_scale), (float*)(ws + l.k_mean),
                          (uint8_t*)(ws + l.v_fp8), (float*)(ws + l.v_scale));
  if (s != SAGE_OK) return s;
  const bool entry = kind == sage::kKernelEntry;
  sage::AttnArgs a;
  s = attn_args((const int8_t*)(ws + l.q_i8), (const float*)(ws + l.q_scale), (const int8_t*)(ws + l.k_i8),
                (const float*)(ws + l.k_scale), (const uint8_t*)(ws + l.v_fp8), (const float*)(ws + l.v_scale), out,
                B, H, Lq, Lkv, D, causal, sm_scale, &a, entry ? q : nullptr);
  if (s != SAGE_OK) return s;
  set_tiles(&a, kind);
  if (kind == sage::kKernelPersistent && !persistent_setup(&a, D, stream, &kind)) return SAGE_ERR_HIP;
  // The preparation pass writes the operands into the workspace (all but
  // Q's when the main loop codes Q), then the main loop runs on them.
  s = quant_prep(q, k, v, B, H, Lq, Lkv, D, (int8_t*)(ws + l.q_i8), (float*)(ws + l.q_scale),
                 (int8_t*)(ws + l.k_i8), (float*)(ws + l.k_scale), (float*)(ws + l.k_mean),
                 (uint8_t*)(ws + l.v_fp8), (float*)(ws + l.v_scale), ws + l.psum, l.total - l.psum, stream, entry);
  if (s != SAGE_OK) return s;
  return hip_status(sage::launch_attn(a, D, causal == 1, kind, (hipStream_t)stream));
}

int sage_attn_fwd(const void* q, const void* k, const void* v, void* out, int B, int H, int Lq, int Lkv,
                  int D, int causal, float sm_scale, void* workspace, size_t workspace_bytes,
                  void* stream) {
  return sage_attn_fwd_kernel(q, k, v, out, B, H, Lq, Lkv, D, causal, sm_scale, SAGE_KERNEL_AUTO, workspace,
                              workspace_bytes, stream);
}

int sage_quant_prep_kv(const void* k, const void* v, int B, int H, int Lkv, int D, int8_t* k_i8, float* k_scale,
                       float* k_mean, uint8_t* v_fp8, float* v_scale, void* scratch, size_t scratch_bytes,
                       void* stream) {
  return quant_prep(nullptr, k, v, B, H, 1, Lkv, D, nullptr, nullptr, k_i8, k_scale, k_mean, v_fp8, v_scale,
                    scratch, scratch_bytes, stream, true);
}

int sage_attn_fwd_kv_prepped(const void* q, const int8_t* k_i8, const float* k_scale, const uint8_t* v_fp8,
                             const float* v_scale, void* out, int B, int H, int Lq, int Lkv, int D, int causal,
                             float sm_scale, void* stream) {
  if (!q) return SAGE_ERR_INVALID_ARG;
  sage::AttnArgs a;
  const int st = attn_args(nullptr, nullptr, k_i8, k_scale, v_fp8, v_scale, out, B, H, Lq, Lkv, D, causal,
                           sm_scale, &a, q);
  if (st != SAGE_OK) return st;
  set_tiles(&a, sage::kKernelEntry);
  return hip_status(sage::launch_attn(a, D, causal == 1, sage::kKernelEntry, (hipStream_t)stream));
}

int sage_auto_design(int B, int H, int Lq, int Lkv, int D, int whole_path, int* design) {
  if (!design || (whole_path != 0 && whole_path != 1)) return SAGE_ERR_INVALID_ARG;
  const int st = check_dims(B, H, Lq, Lkv, D);
  if (st != SAGE_OK) return st;
  const int k = whole_path ? auto_kernel_whole(B, H, Lq) : auto_kernel(B, H, Lq);
  *design = k == sage::kKernelSplit ? SAGE_KERNEL_SPLIT : k == sage::kKernelEntry ? SAGE_KERNEL_ENTRY
                                                                                 : SAGE_KERNEL_FUSED;
  return SAGE_OK;
}

int sage_debug_qk_int32(const int8_t* q_i8, const int8_t* k_i8, int B, int H, int Lq, int Lkv, int D,
                        const int* tiles, int n_tiles, int32_t* acc_out, void* stream) {
  const int st = check_dims(B, H, Lq, Lkv, D);
  if (st != SAGE_OK) return st;
  if (!q_i8 || !k_i8 || !tiles || !acc_out || n_tiles < 0) return SAGE_ERR_INVALID_ARG;
  if (misaligned(q_i8, 16) || misaligned(k_i8, 16) || misaligned(acc_out, 16)) return SAGE_ERR_INVALID_ARG;
  sage::QkDebugArgs a;
  a.q_i8 = q_i8; a.k_i8 = k_i8;
  a.Lq = Lq; a.Lkv = Lkv; a.H = H;
  a.nqb = (Lq + sage::kBlock - 1) / sage::kBlock;
  a.nkb = (Lkv + sage::kBlock - 1) / sage::kBlock;
  for (int i = 0; i < n_tiles; ++i) {
    const int* t = tiles + 4 * i;
    if (t[0] < 0 || t[0] >= B || t[1] < 0 || t[1] >= H || t[2] < 0 || t[2] >= a.nqb || t[3] < 0 ||
        t[3] >= a.nkb)
      return SAGE_ERR_INVALID_ARG;
  }
  for (int base = 0; base < n_tiles; base += sage::kMaxDebugTiles) {
    a.n = n_tiles - base < sage::kMaxDebugTiles ? n_tiles - base : sage::kMaxDebugTiles;
    for (int i = 0; i < a.n; ++i)
      for (int j = 0; j < 4; ++j) a.tiles[i][j] = tiles[4 * (base + i) + j];
    a.acc_out = acc_out + (size_t)base * sage::kBlock * sage::kBlock;
    const int s = hip_status(sage::launch_qk_debug(a, D, (hipStream_t)stream));
    if (s != SAGE_OK) return s;
  }
  return SAGE_OK;
}

int sage_debug_codecs(const float* x, int n, uint8_t* p8, uint16_t* bf16, void* stream) {
  if (!x || !p8 || !bf16 || n < 0) return SAGE_ERR_INVALID_ARG;
  if (misaligned(x, 4) || misaligned(bf16, 2)) return SAGE_ERR_INVALID_ARG;
  if (n == 0) return SAGE_OK;
  return hip_status(sage::launch_codecs_debug(x, n, p8, bf16, (hipStream_t)stream));
}

}  // extern "C"
