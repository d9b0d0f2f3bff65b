/*
 * sage_attn.h - C ABI of the MI355X (gfx950) quantized exact attention library.
 *
 * The method is SageAttention2-style quantized attention with K smoothing, as
 * the "Experiment Log" page (vortex_exact_attention) lists its contract in
 * section "Phase 0 Import And Verification": Q/K preparation, K smoothing,
 * INT8 quantization, QK traversal, online softmax, FP8 V/P, two-level PV
 * accumulation, final conversion and ragged tails. Section "Phase 1
 * State-Ownership Decision" adds strict tile order, exact FP8 score bytes and
 * per-tile RO rescaling.
 *
 * Conventions shared by every entry point:
 *  - Pointers to tensors are DEVICE pointers owned by the caller. The library
 *    never allocates, frees or keeps a pointer after a call returns.
 *  - q is [B][H][Lq][D], k, v are [B][H][Lkv][D], out is [B][H][Lq][D]:
 *    bf16 (raw 16-bit storage), D contiguous, base address 16-byte aligned.
 *  - D is 64 or 128; B, H, Lq, Lkv >= 1; B*H*max(Lq,Lkv)*D < 2^40, and one
 *    head's Q and K codes fit in 2 GiB: NQB*64*D < 2^31 and NKB*64*D < 2^31
 *    (Lq, Lkv < 2^24 at D = 128);
 *    B*H*(NQB + 2*NKB) < 2^31 (workgroups of the preparation pass).
 *  - Quantization blocks and attention epochs are SAGE_BLOCK = 64 rows/keys;
 *    NQB = ceil(Lq/64), NKB = ceil(Lkv/64).
 *  - stream is a hipStream_t (NULL = the default stream). Calls only enqueue
 *    work; results are valid once the stream has synchronised. Calls keep no
 *    state between them and may be made from several host threads.
 *  - Arguments are validated before any GPU call; on an error nothing is
 *    enqueued. A failed launch is reported as SAGE_ERR_HIP. NaN or Inf inputs
 *    give unspecified output values, never a fault.
 */
#ifndef SAGE_ATTN_H
#define SAGE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SAGE_BLOCK 64

enum sage_status {
    SAGE_OK = 0,
    SAGE_ERR_INVALID_ARG = -1, /* null or misaligned pointer, size < 1, bad flag */
    SAGE_ERR_UNSUPPORTED = -2, /* D not in {64, 128} */
    SAGE_ERR_WORKSPACE = -3,   /* workspace or scratch too small */
    SAGE_ERR_HIP = -4          /* a HIP launch or runtime call failed */
};

/* Human-readable name of a status code (static storage). */
const char* sage_status_str(int status);

/*
 * Bytes of device scratch sage_quant_prep needs (fp64 channel partial sums
 * and fp32 channel absmax partials). Host-only; writes *bytes.
 */
int sage_prep_scratch_bytes(int B, int H, int Lq, int Lkv, int D, size_t* bytes);

/*
 * Bytes of device workspace sage_attn_fwd needs: every output of
 * sage_quant_prep laid out as below, each part 256-byte aligned, followed by
 * the preparation scratch. Host-only; writes *bytes.
 */
int sage_workspace_bytes(int B, int H, int Lq, int Lkv, int D, size_t* bytes);

/*
 * Preparation pass (Experiment Log, "Phase 0 Import And Verification":
 * Q/K preparation, K smoothing, INT8 quantization, FP8 V).
 * Inputs q, k, v as above. Outputs (device, caller-owned):
 *   k_mean  fp32 [B][H][D]        mean[c] = fp32(fp64 sum_t K[t][c] / Lkv);
 *                                  the fp64 sum runs in an unspecified order.
 *                                  It is exact, so the mean is order-free,
 *                                  when the channel's nonzero |K| lie in
 *                                  [2^e_min, 2^(e_max+1)), e_max - e_min <=
 *                                  45 - ceil(log2 Lkv) (bf16 has 8
 *                                  significant bits); otherwise its last
 *                                  bits may depend on the order
 *   k_i8    int8 [B][H][NKB*64][D] codes of Ks = fp32(K) - mean, per 64-row
 *                                  block: s = absmax/127, code =
 *                                  clamp(rint_even(Ks / s), -127, 127)
 *   k_scale fp32 [B][H][NKB]
 *   q_i8    int8 [B][H][NQB*64][D] the same block codes of raw Q
 *   q_scale fp32 [B][H][NQB]
 *   v_scale fp32 [B][H][D]         sv[c] = max_t |V[t][c]| / 448
 *   v_fp8   uint8 [B][H][NKB][D][64] E4M3FN codes of V / sv (nearest-even,
 *                                  saturating), stored per 64-key block with
 *                                  the keys of a channel contiguous
 * Padded rows/keys (beyond Lq or Lkv) hold code 0; an all-zero block or
 * channel has scale 0 and codes 0. The int8 outputs and v_fp8 must be 16-byte
 * aligned. scratch: device memory of at least sage_prep_scratch_bytes; its
 * contents on entry do not matter.
 */
int sage_quant_prep(const void* q, const void* k, const void* v, int B, int H, int Lq, int Lkv, int D,
                    int8_t* q_i8, float* q_scale, int8_t* k_i8, float* k_scale, float* k_mean,
                    uint8_t* v_fp8, float* v_scale, void* scratch, size_t scratch_bytes, void* stream);

/*
 * sage_quant_prep for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same outputs, bit for bit, with the preparation scratch taken from a
 * static device array of 16 MiB inside the library (one per GPU, held until
 * the process ends) instead of a caller buffer. The call allocates nothing.
 * Shapes whose scratch (sage_prep_scratch_bytes) exceeds 16 MiB return
 * SAGE_ERR_WORKSPACE before any GPU call (the scratch is 12 bytes per head,
 * 256-key split and channel: B*H*ceil(Lkv/256)*D up to about 1.39 million
 * fits; 64 heads at Lkv = 4096 and D = 128 need 1.5 MiB). The first call
 * on a device looks up that device's array (hipGetSymbolAddress; the current
 * device must be the stream's device). Calls on one GPU share its array:
 * calls whose execution overlaps on one GPU (different streams, or host
 * threads without ordering) race and give undefined outputs; calls ordered
 * on one stream do not.
 */
int sage_quant_prep_noalloc(const void* q, const void* k, const void* v, int B, int H, int Lq, int Lkv, int D,
                            int8_t* q_i8, float* q_scale, int8_t* k_i8, float* k_scale, float* k_mean,
                            uint8_t* v_fp8, float* v_scale, void* stream);

/*
 * Attention from prepared operands (the main loop alone, in the design
 * SAGE_KERNEL_AUTO selects for prepared operands), in the layouts
 * sage_quant_prep writes. Per query row i, strictly ascending 64-key
 * epochs (Experiment Log, "Phase 1 State-Ownership Decision"):
 *   S = q8 . k8 (exact int32), z = S * sq * sk * sm_scale, online max m and
 *   sum l, alpha = exp(m_old - m_new), P8 = e4m3(exp(z - m_new)),
 *   PV = P8 . V8 (fp32, one epoch), RO = RO * alpha + PV;
 *   out = bf16(RO * (1/l) * sv[c])   ("reciprocal" then BF16; Experiment
 *   Log, "Phase 2B Fixed Aligned Numerical Prototype").
 * causal = 1 masks key j > i + Lkv - Lq (bottom-right aligned); a row with no
 * visible key outputs 0. sm_scale <= 0 selects 1/sqrt(D). out is written for
 * rows < Lq only.
 */
int sage_attn_fwd_prepped(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                          const float* k_scale, const uint8_t* v_fp8, const float* v_scale, void* out,
                          int B, int H, int Lq, int Lkv, int D, int causal, float sm_scale, void* stream);

/*
 * Main-loop kernel designs. Every design computes the same values bit for
 * bit (the same per-epoch arithmetic in the same order); they differ in how
 * the work is laid out on the waves of a workgroup.
 *   SAGE_KERNEL_FUSED  each wave owns 32 query rows end to end: their Q
 *                      codes, scores, running max and sum, and RO.
 *   SAGE_KERNEL_SPLIT  wave-specialised ownership (Experiment Log, "Phase 1
 *                      State-Ownership Decision": paired QK/softmax and
 *                      PV/output owners; "Phase 2A": the role clocks
 *                      overlap): softmax waves hold the Q codes, scores, m
 *                      and l; PV waves hold RO; the E4M3 P block and alpha
 *                      of each epoch pass between them through LDS.
 *   SAGE_KERNEL_PERSISTENT  the FUSED waves in persistent workgroups (as
 *                      many as fit on the GPU at once) that take 128-row
 *                      tiles, heaviest first, from a work counter
 *                      (fetch-and-add). The library keeps one counter per
 *                      stream for up to 64 streams per device (a further
 *                      stream runs FUSED); each launch returns its counter to
 *                      0, and calls on one stream never overlap.
 *   SAGE_KERNEL_WIDE   the FUSED waves in 8-wave workgroups of 256 rows:
 *                      each K/V tile copied into LDS serves twice the rows,
 *                      and two such workgroups (four waves per SIMD) fit a
 *                      compute unit.
 *   SAGE_KERNEL_ENTRY  (sage_attn_fwd_kernel only) the FUSED waves with the
 *                      Q INT8 step moved into the main loop (Experiment Log,
 *                      "Closed Prior Work": the P1 entry fusion, reused
 *                      inside the attention pipeline): the preparation pass
 *                      codes K and V only, and each workgroup reads its 128
 *                      rows of bf16 Q and codes them straight into its LDS Q
 *                      tile with the preparation pass's arithmetic (the same
 *                      codes and scales for finite inputs), so Q codes
 *                      never pass through memory; the workspace's Q code and
 *                      Q scale areas are left unwritten. Its two stages are
 *                      also public: sage_quant_prep_kv and
 *                      sage_attn_fwd_kv_prepped. Calls on prepared Q codes
 *                      return SAGE_ERR_INVALID_ARG for it.
 *   SAGE_KERNEL_AUTO   the design measured faster for the shape: SPLIT when
 *                      B*H*ceil(Lq/128) < 256 (fewer 128-row tiles than
 *                      compute units); otherwise FUSED for calls on prepared
 *                      operands and ENTRY for the whole path (sage_attn_fwd),
 *                      where it is faster end to end. sage_auto_design
 *                      reports the choice.
 */
enum sage_kernel {
    SAGE_KERNEL_AUTO = 0,
    SAGE_KERNEL_FUSED = 1,
    SAGE_KERNEL_SPLIT = 2,
    SAGE_KERNEL_PERSISTENT = 3,
    SAGE_KERNEL_WIDE = 4,
    SAGE_KERNEL_ENTRY = 5
};

/*
 * sage_attn_fwd_prepped with an explicit main-loop design (enum
 * sage_kernel, other than SAGE_KERNEL_ENTRY); any other value returns
 * SAGE_ERR_INVALID_ARG.
 */
int sage_attn_fwd_prepped_kernel(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                                 const float* k_scale, const uint8_t* v_fp8, const float* v_scale, void* out,
                                 int B, int H, int Lq, int Lkv, int D, int causal, float sm_scale, int kernel,
                                 void* stream);

/*
 * The whole path with the automatic design (SAGE_KERNEL_AUTO): the
 * preparation pass into the workspace (its parts laid out as
 * sage_workspace_bytes describes), then the main loop on them, both on
 * stream. On full grids that is sage_quant_prep_kv + sage_attn_fwd_kv_prepped
 * (the entry design), otherwise sage_quant_prep + sage_attn_fwd_prepped; the
 * output is the same bits either way for finite inputs. workspace: device
 * memory of at least sage_workspace_bytes, 256-byte aligned; it is
 * overwritten.
 */
int sage_attn_fwd(const void* q, const void* k, const void* v, void* out, int B, int H, int Lq, int Lkv,
                  int D, int causal, float sm_scale, void* workspace, size_t workspace_bytes,
                  void* stream);

/*
 * sage_attn_fwd with an explicit main-loop design (enum sage_kernel,
 * SAGE_KERNEL_ENTRY included); any other value returns SAGE_ERR_INVALID_ARG.
 * Every argument is checked before anything is launched.
 */
int sage_attn_fwd_kernel(const void* q, const void* k, const void* v, void* out, int B, int H, int Lq, int Lkv,
                         int D, int causal, float sm_scale, int kernel, void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * The K/V half of the preparation pass (Experiment Log, "Phase 0 Import And
 * Verification": K smoothing, INT8 quantization, FP8 V), e.g. for a key and
 * value set that several query batches attend to: k_mean, k_i8, k_scale,
 * v_fp8 and v_scale exactly as sage_quant_prep writes them for the same k and
 * v. scratch: at least sage_prep_scratch_bytes for these B, H, Lkv, D (any
 * Lq). Arguments otherwise as sage_quant_prep.
 */
int sage_quant_prep_kv(const void* k, const void* v, int B, int H, int Lkv, int D, int8_t* k_i8, float* k_scale,
                       float* k_mean, uint8_t* v_fp8, float* v_scale, void* scratch, size_t scratch_bytes,
                       void* stream);

/*
 * The main loop of the entry design (SAGE_KERNEL_ENTRY) on K/V prepared by
 * sage_quant_prep_kv (or sage_quant_prep) and bf16 q [B][H][Lq][D] (16-byte
 * aligned): each workgroup codes its Q rows itself (Experiment Log, "Closed
 * Prior Work": the P1 entry fusion inside the attention pipeline), with the
 * arithmetic of the preparation pass, so for finite inputs the output equals
 * sage_quant_prep + sage_attn_fwd_prepped bit for bit. Other arguments as
 * sage_attn_fwd_prepped.
 */
int sage_attn_fwd_kv_prepped(const void* q, const int8_t* k_i8, const float* k_scale, const uint8_t* v_fp8,
                             const float* v_scale, void* out, int B, int H, int Lq, int Lkv, int D, int causal,
                             float sm_scale, void* stream);

/*
 * The design SAGE_KERNEL_AUTO selects for a shape: *design =
 * SAGE_KERNEL_SPLIT, _FUSED or _ENTRY; whole_path = 1 for sage_attn_fwd,
 * 0 for sage_attn_fwd_prepped. Invalid shapes return the status the calls
 * would.
 */
int sage_auto_design(int B, int H, int Lq, int Lkv, int D, int whole_path, int* design);

/*
 * Debug: the exact int32 QK accumulators of chosen 64x64 tiles, computed by
 * the same LDS staging and INT8 matrix-core code as the main loop
 * (Experiment Log, "Phase 2B": the "QK" checkpoint).
 * tiles: HOST array of n_tiles records {b, h, query block, key block}, each
 * checked against B, H, NQB, NKB. acc_out: device int32 [n_tiles][64][64],
 * row = query within the block, column = key within the block.
 */
int sage_debug_qk_int32(const int8_t* q_i8, const int8_t* k_i8, int B, int H, int Lq, int Lkv, int D,
                        const int* tiles, int n_tiles, int32_t* acc_out, void* stream);

/*
 * Debug: per-epoch checkpoints of 32 query rows (Experiment Log, "Phase 2B
 * Fixed Aligned Numerical Prototype": the QK, m, d, FP8 probability,
 * rescale, PV, FP32 RO and reciprocal checkpoints). Runs the main loop of
 * design `kernel` (enum sage_kernel, not SAGE_KERNEL_ENTRY) on the one tile
 * of head (b, h) that holds rows row0 .. row0 + 31 (row0 a multiple of 32,
 * < Lq); the waves
 * owning those rows write, for row t = row0 + i and every epoch e they
 * compute (e below the rows' epoch count; the caller pre-fills the buffers
 * to recognise the rest):
 *   stats [32][NKB+1][4] fp32: [i][e] = m (log2 domain: max of z * log2(e)),
 *         l, alpha (of this epoch), 0; [i][NKB] = 1/l, l at the end;
 *   p8    [32][NKB][64] uint8: the epoch's E4M3 P bytes, key 64e + j;
 *   pv    [32][NKB][D]  fp32: the epoch's own PV partial, sum over its 64
 *         keys of dec(P8) dec(V8) (the main loop adds it into RO inside
 *         the matrix-core step; the trace build runs that step once more
 *         into a zeroed accumulator to record it);
 *   ro    [32][NKB][D]  fp32: RO after the epoch (RO * alpha + PV).
 * out (bf16 [B][H][Lq][D]) receives that tile's rows as the main loop would
 * write them. Arguments otherwise as sage_attn_fwd_prepped; stats 16-byte
 * aligned, p8, pv and ro 4-byte aligned.
 */
int sage_debug_epoch_trace(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                           const float* k_scale, const uint8_t* v_fp8, const float* v_scale, void* out,
                           int B, int H, int Lq, int Lkv, int D, int causal, float sm_scale, int kernel, int b,
                           int h, int row0, float* stats, uint8_t* p8, float* pv, float* ro, void* stream);

/*
 * Debug: the same per-epoch checkpoints for the entry design's main loop
 * (sage_attn_fwd_kv_prepped: bf16 q, coded into the Q tile by the loop
 * itself) on K/V prepared by sage_quant_prep_kv or sage_quant_prep; the
 * records and the other arguments as sage_debug_epoch_trace.
 */
int sage_debug_epoch_trace_kv(const void* q, const int8_t* k_i8, const float* k_scale, const uint8_t* v_fp8,
                              const float* v_scale, void* out, int B, int H, int Lq, int Lkv, int D, int causal,
                              float sm_scale, int b, int h, int row0, float* stats, uint8_t* p8, float* pv,
                              float* ro, void* stream);

/*
 * Debug: run the device conversions the main loop uses on n fp32 values x
 * (device): p8[i] = FP8 E4M3FN code as the probability packing produces it,
 * bf16[i] = bf16 bits as the output conversion produces them.
 */
int sage_debug_codecs(const float* x, int n, uint8_t* p8, uint16_t* bf16, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SAGE_ATTN_H */
