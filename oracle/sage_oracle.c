/*
 * CPU oracle for SageAttention2-style quantized exact attention with K smoothing.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library. It shares no code, header, table or
 * helper with the HIP library, and the HIP library never calls it.
 *
 * Source: the "Experiment Log" page (vortex_exact_attention), section
 * "Phase 0 Import And Verification", names the contract's parts in order:
 * Q/K preparation, K smoothing, INT8 quantization, QK traversal, online
 * softmax, FP8 V/P, two-level PV accumulation, final conversion and ragged
 * tails. Section "Phase 1 State-Ownership Decision" adds strict tile order,
 * exact FP8 score bytes and per-tile RO rescaling; "Phase 2B Fixed Aligned
 * Numerical Prototype" lists the checkpoints QK, m, d, FP8 probability,
 * rescale, PV, FP32 RO, reciprocal and BF16 output. The page gives no
 * formulas, so the plainest reading is written out here step by step; each
 * reading is named where it is used.
 *
 * Three computations:
 *   (i)   orc_prep_head + orc_attn_rows: the quantized contract (the
 *         reference the GPU is compared to);
 *   (ii)  orc_attn_unquant_rows: the same 64-key epoch loop in fp64 with
 *         every quantizer replaced by the identity;
 *   (iii) orc_attn_ref_rows: brute-force fp64 softmax(Q K^T * scale) V.
 *
 * Build: plain C11, -O2 -ffp-contract=off (no fused multiply-add, so every
 * float operation below rounds once, as written), no fast-math, libm only.
 *
 * Parity pins (tests/test_oracle_*.py): codec tables and library casts, exact
 * summation of the mean, brute-force nearest-integer checks of the codes,
 * (ii) == (iii) on ragged/causal sweeps, smoothing invariance, constant V,
 * zero Q, one-hot keys and cosine >= 0.995 of (i) against (iii).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_BLOCK 64 /* quant block rows == attention epoch keys */

/* ------------------------------------------------------------------ codecs */

float orc_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* float -> bf16, round to nearest, ties to the even bf16 mantissa. The two
 * bf16 neighbours of x (toward and away from zero) are compared by their
 * exact distance to x in double. */
uint16_t orc_f32_to_bf16(float x)
{
    uint32_t u;
    memcpy(&u, &x, sizeof u);
    if (isnan(x))
        return (uint16_t)((u >> 16) | 0x0040u);
    if (isinf(x))
        return (uint16_t)(u >> 16);
    uint32_t lo = u & 0xFFFF0000u;
    uint32_t hi = lo + 0x10000u;
    float flo;
    memcpy(&flo, &lo, sizeof flo);
    double dlo = fabs((double)x - (double)flo);
    double vhi;
    if ((hi & 0x7F800000u) == 0x7F800000u) /* the away neighbour overflows */
        vhi = copysign(ldexp(1.0, 128), (double)x);
    else {
        float fhi;
        memcpy(&fhi, &hi, sizeof fhi);
        vhi = (double)fhi;
    }
    double dhi = fabs(vhi - (double)x);
    uint32_t pick;
    if (dlo < dhi)
        pick = lo;
    else if (dhi < dlo)
        pick = hi;
    else
        pick = ((lo >> 16) & 1u) ? hi : lo;
    return (uint16_t)(pick >> 16);
}

/* OCP FP8 E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent 0
 * holds subnormals m * 2^-9; S.1111.111 is NaN; no infinities; the largest
 * finite value is 1.75 * 2^8 = 448. */
double orc_e4m3_decode(uint8_t code)
{
    int s = code >> 7, e = (code >> 3) & 0xF, m = code & 7;
    if (e == 15 && m == 7)
        return NAN;
    double v = (e == 0) ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
    return s ? -v : v;
}

/* float -> E4M3FN, round to nearest, ties to even code, saturating to +-448.
 * The magnitude is located between two adjacent finite codes by bisection
 * over the monotone decode table, and the nearer one is taken. A zero
 * result keeps the sign of x. */
uint8_t orc_e4m3_encode(float x)
{
    if (isnan(x))
        return 0x7F;
    uint8_t sign = signbit(x) ? 0x80 : 0x00;
    double a = fabs((double)x);
    if (a >= 448.0)
        return (uint8_t)(sign | 0x7E);
    int lo = 0, hi = 126;
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (orc_e4m3_decode((uint8_t)mid) <= a)
            lo = mid;
        else
            hi = mid - 1;
    }
    double d0 = a - orc_e4m3_decode((uint8_t)lo);
    double d1 = orc_e4m3_decode((uint8_t)(lo + 1)) - a;
    int c;
    if (d0 < d1)
        c = lo;
    else if (d1 < d0)
        c = lo + 1;
    else
        c = (lo & 1) ? lo + 1 : lo;
    return (uint8_t)(sign | c);
}

void orc_bf16_round_array(const float* x, uint16_t* out, long n)
{
    for (long i = 0; i < n; ++i)
        out[i] = orc_f32_to_bf16(x[i]);
}

void orc_e4m3_encode_array(const float* x, uint8_t* out, long n)
{
    for (long i = 0; i < n; ++i)
        out[i] = orc_e4m3_encode(x[i]);
}

void orc_e4m3_decode_array(const uint8_t* c, double* out, long n)
{
    for (long i = 0; i < n; ++i)
        out[i] = orc_e4m3_decode(c[i]);
}

/* ------------------------------------------------------------ preparation */

/* INT8 code of x in a block with scale s = a / 127 (a = block absmax):
 * the fp32 quotient x / s rounded half-to-even to an integer and clamped to
 * [-127, 127]; an all-zero block (a == 0) codes to 0. */
static int8_t int8_code(float x, float s, float a)
{
    if (a == 0.0f)
        return 0;
    float t = x / s;    /* IEEE single division */
    float r = rintf(t); /* default rounding mode: nearest, ties to even */
    if (r > 127.0f)
        r = 127.0f;
    if (r < -127.0f)
        r = -127.0f;
    return (int8_t)r;
}

/* Quantize rows [0, L) of x (fp32 values, [L][D]) in 64-row blocks into
 * codes [nb*64][D] (padded rows 0) and one scale per block. */
static void quant_blocks(const float* x, int L, int D, int8_t* codes, float* scales)
{
    int nb = (L + ORC_BLOCK - 1) / ORC_BLOCK;
    for (int b = 0; b < nb; ++b) {
        int t0 = b * ORC_BLOCK;
        int t1 = t0 + ORC_BLOCK < L ? t0 + ORC_BLOCK : L;
        float a = 0.0f;
        for (int t = t0; t < t1; ++t)
            for (int c = 0; c < D; ++c) {
                float m = fabsf(x[(long)t * D + c]);
                if (m > a)
                    a = m;
            }
        float s = a / 127.0f;
        scales[b] = s;
        for (int t = t0; t < t0 + ORC_BLOCK; ++t)
            for (int c = 0; c < D; ++c)
                codes[(long)t * D + c] = (t < t1) ? int8_code(x[(long)t * D + c], s, a) : 0;
    }
}

/*
 * One (b, h) head of the preparation pass.
 *   q [Lq][D], k, v [Lkv][D]: bf16 bits.
 *   smooth: 1 = subtract K's per-channel mean (the contract), 0 = no smoothing
 *           (only for the ablation that shows what smoothing buys).
 * Outputs (caller-owned):
 *   q8 [nqb*64][D], q_scale [nqb]; k8 [nkb*64][D], k_scale [nkb]; k_mean [D];
 *   v8 [nkb*64][D] (token-major E4M3FN bytes), v_scale [D].
 * Returns 0, or 1 if a channel sum of K was not exact in fp64 (forward and
 * reverse sums differ), in which case the mean is order-dependent.
 *
 * Steps (Experiment Log, "Phase 0 Import And Verification": Q/K preparation,
 * K smoothing, INT8 quantization, FP8 V):
 *   1. mean[c] = fp32( (sum_t fp64 K[t,c]) / fp64 Lkv )          (fp64 sum)
 *   2. Ks[t,c] = fp32(K[t,c]) - mean[c]                           (one fp32 op)
 *   3. per 64-row block: s = absmax / 127, code = clamp(rint(Ks / s))
 *   4. same for raw Q (no smoothing of Q)
 *   5. per channel: sv[c] = max_t |V[t,c]| / 448, V8 = e4m3(V / sv)
 */
int orc_prep_head(const uint16_t* q, const uint16_t* k, const uint16_t* v, int Lq, int Lkv, int D,
                  int smooth, int8_t* q8, float* q_scale, int8_t* k8, float* k_scale, float* k_mean,
                  uint8_t* v8, float* v_scale)
{
    int inexact = 0;
    int nkb = (Lkv + ORC_BLOCK - 1) / ORC_BLOCK;

    for (int c = 0; c < D; ++c) {
        double fwd = 0.0, rev = 0.0;
        for (int t = 0; t < Lkv; ++t)
            fwd += (double)orc_bf16_to_f32(k[(long)t * D + c]);
        for (int t = Lkv - 1; t >= 0; --t)
            rev += (double)orc_bf16_to_f32(k[(long)t * D + c]);
        if (fwd != rev)
            inexact = 1;
        k_mean[c] = smooth ? (float)(fwd / (double)Lkv) : 0.0f;
    }

    float* tmp = (float*)malloc(sizeof(float) * (size_t)(Lq > Lkv ? Lq : Lkv) * (size_t)D);
    if (!tmp)
        return -1;

    for (long i = 0; i < (long)Lkv * D; ++i)
        tmp[i] = orc_bf16_to_f32(k[i]) - k_mean[i % D];
    quant_blocks(tmp, Lkv, D, k8, k_scale);

    for (long i = 0; i < (long)Lq * D; ++i)
        tmp[i] = orc_bf16_to_f32(q[i]);
    quant_blocks(tmp, Lq, D, q8, q_scale);
    free(tmp);

    for (int c = 0; c < D; ++c) {
        float a = 0.0f;
        for (int t = 0; t < Lkv; ++t) {
            float m = fabsf(orc_bf16_to_f32(v[(long)t * D + c]));
            if (m > a)
                a = m;
        }
        float s = a / 448.0f;
        v_scale[c] = s;
        for (int t = 0; t < nkb * ORC_BLOCK; ++t) {
            uint8_t code = 0;
            if (t < Lkv && a != 0.0f)
                code = orc_e4m3_encode(orc_bf16_to_f32(v[(long)t * D + c]) / s);
            v8[(long)t * D + c] = code;
        }
    }
    return inexact;
}

/* ------------------------------------------------ quantized attention (i) */

/*
 * The quantized contract for one query row i of one head, from the
 * prepared operands. Causal masking is bottom-right aligned: row i sees keys
 * j <= i + Lkv - Lq.
 *
 * Per row (strict ascending 64-key epochs; Experiment Log, "Phase 1
 * State-Ownership Decision": strict tile order, exact FP8 score bytes,
 * per-tile RO rescaling, two-level PV accumulation):
 *   acc_j  = sum_c q8[i,c] * k8[j,c]                          (exact integer)
 *   z_j    = (fp32(acc_j) * (sq * sk[e])) * sm_scale           (fp32), -inf if masked
 *   m'     = max(m, max_j z_j); skip the epoch while m' = -inf
 *   alpha  = exp(m - m')            (0 when m = -inf)          -> "rescale"
 *   p_j    = exp(z_j - m')                                     (fp32 result)
 *   l      = l * alpha + sum_j p_j  (ascending j)              -> "d"
 *   P8_j   = e4m3(p_j), no extra scale                         -> "FP8 probability"
 *   PV[c]  = sum_j dec(P8_j) * dec(V8[j,c])  (fp32, ascending)  -> inner level
 *   RO[c]  = RO[c] * alpha + PV[c]                             -> outer level, "FP32 RO"
 * Final conversion: r = 1 / l ("reciprocal"), out = bf16(RO * r * sv[c]);
 * a row with no visible key outputs 0. exp is evaluated in fp64 on the fp32
 * operands and rounded to fp32.
 *
 * When tr_stats is not NULL the
 * state after every epoch e (0 <= e < NKB) is copied out, and nothing else
 * changes: tr_stats[e*4 + 0..3] = m, l, alpha (1 for an epoch without a
 * visible key, whose state is carried over), 0; tr_stats[NKB*4 + 0..1] =
 * r, l after the last epoch; tr_p8[e*64 + jj] = P8 of key 64e + jj (0 where
 * masked); tr_pv[e*D + c] = the epoch's PV partial; tr_ro[e*D + c] = RO
 * after the epoch. Returns 2 if an accumulator reached 2^24, else 0. */
static int attn_row(const int8_t* q8, const float* q_scale, const int8_t* k8, const float* k_scale,
                    const uint8_t* v8, const float* v_scale, int Lq, int Lkv, int D, int causal,
                    float sm_scale, int i, float* RO, uint16_t* out_row, float* tr_stats, uint8_t* tr_p8,
                    float* tr_pv, float* tr_ro)
{
    int status = 0;
    int nkb = (Lkv + ORC_BLOCK - 1) / ORC_BLOCK;
    float z[ORC_BLOCK], p[ORC_BLOCK];
    uint8_t p8[ORC_BLOCK];
    long last = causal ? (long)i + Lkv - Lq : (long)Lkv - 1; /* last visible key */
    if (last > Lkv - 1)
        last = Lkv - 1;
    float m = -INFINITY, l = 0.0f;
    for (int c = 0; c < D; ++c)
        RO[c] = 0.0f;

    for (int e = 0; e < nkb; ++e) {
        long j0 = (long)e * ORC_BLOCK;
        int live = 0;
        float alpha = 1.0f;
        if (j0 <= last) { /* otherwise this and every later epoch is fully masked */
            float sqk = q_scale[i / ORC_BLOCK] * k_scale[e];
            float mx = -INFINITY;
            for (int jj = 0; jj < ORC_BLOCK; ++jj) {
                long j = j0 + jj;
                if (j > last) {
                    z[jj] = -INFINITY;
                    continue;
                }
                int64_t acc = 0;
                for (int c = 0; c < D; ++c)
                    acc += (int64_t)q8[(long)i * D + c] * (int64_t)k8[j * D + c];
                if (acc >= (1 << 24) || acc <= -(1 << 24))
                    status = 2;
                z[jj] = ((float)acc * sqk) * sm_scale;
                if (z[jj] > mx)
                    mx = z[jj];
            }
            float mn = m > mx ? m : mx;
            if (mn != -INFINITY) {
                live = 1;
                alpha = (m == -INFINITY) ? 0.0f : (float)exp((double)m - (double)mn);
                float ps = 0.0f;
                for (int jj = 0; jj < ORC_BLOCK; ++jj) {
                    p[jj] = (z[jj] == -INFINITY) ? 0.0f : (float)exp((double)z[jj] - (double)mn);
                    ps += p[jj];
                    p8[jj] = orc_e4m3_encode(p[jj]);
                }
                l = l * alpha + ps;
                for (int c = 0; c < D; ++c) {
                    float pv = 0.0f;
                    for (int jj = 0; jj < ORC_BLOCK; ++jj) {
                        long j = j0 + jj;
                        if (j >= Lkv)
                            break; /* padded keys have P8 = 0 and V8 = 0 */
                        pv += (float)orc_e4m3_decode(p8[jj]) * (float)orc_e4m3_decode(v8[j * D + c]);
                    }
                    RO[c] = RO[c] * alpha + pv;
                    if (tr_pv)
                        tr_pv[(long)e * D + c] = pv;
                }
                m = mn;
            }
        }
        if (tr_stats) {
            tr_stats[e * 4 + 0] = m;
            tr_stats[e * 4 + 1] = l;
            tr_stats[e * 4 + 2] = alpha;
            tr_stats[e * 4 + 3] = 0.0f;
            for (int jj = 0; jj < ORC_BLOCK; ++jj)
                tr_p8[(long)e * ORC_BLOCK + jj] = live ? p8[jj] : 0;
            for (int c = 0; c < D; ++c) {
                if (!live)
                    tr_pv[(long)e * D + c] = 0.0f;
                tr_ro[(long)e * D + c] = RO[c];
            }
        }
    }
    float r = (l > 0.0f) ? 1.0f / l : 0.0f;
    if (tr_stats) {
        tr_stats[nkb * 4 + 0] = r;
        tr_stats[nkb * 4 + 1] = l;
        tr_stats[nkb * 4 + 2] = 0.0f;
        tr_stats[nkb * 4 + 3] = 0.0f;
    }
    for (int c = 0; c < D; ++c)
        out_row[c] = orc_f32_to_bf16((RO[c] * r) * v_scale[c]);
    return status;
}

/* Rows [r0, r1) of one head's output. out: bf16 bits [Lq][D]; only rows
 * r0..r1-1 are written. Returns 0, or 2 if an INT8 dot product left the
 * int32-exact range. */
int orc_attn_rows(const int8_t* q8, const float* q_scale, const int8_t* k8, const float* k_scale,
                  const uint8_t* v8, const float* v_scale, int Lq, int Lkv, int D, int causal,
                  float sm_scale, int r0, int r1, uint16_t* out)
{
    int status = 0;
    float* RO = (float*)malloc(sizeof(float) * (size_t)D);
    if (!RO)
        return -1;
    for (int i = r0; i < r1; ++i) {
        int st = attn_row(q8, q_scale, k8, k_scale, v8, v_scale, Lq, Lkv, D, causal, sm_scale, i, RO,
                          out + (long)i * D, NULL, NULL, NULL, NULL);
        if (st)
            status = st;
    }
    free(RO);
    return status;
}

/* Per-epoch checkpoints of one row i (the Phase 2B checkpoint list: m, d,
 * FP8 probability, rescale, PV, FP32 RO, reciprocal), laid out as in
 * attn_row. out_row receives the row's bf16 output. */
int orc_attn_row_trace(const int8_t* q8, const float* q_scale, const int8_t* k8, const float* k_scale,
                       const uint8_t* v8, const float* v_scale, int Lq, int Lkv, int D, int causal,
                       float sm_scale, int i, uint16_t* out_row, float* tr_stats, uint8_t* tr_p8, float* tr_pv,
                       float* tr_ro)
{
    float* RO = (float*)malloc(sizeof(float) * (size_t)D);
    if (!RO)
        return -1;
    int st = attn_row(q8, q_scale, k8, k_scale, v8, v_scale, Lq, Lkv, D, causal, sm_scale, i, RO, out_row,
                      tr_stats, tr_p8, tr_pv, tr_ro);
    free(RO);
    return st;
}

/* ------------------------------------- unquantized epoch loop, fp64 (ii) */

/* The epoch loop above with identity quantizers: no codes, no scales, no
 * FP8, every value and operation in fp64. q [Lq][D], k, v [Lkv][D],
 * out [Lq][D] (rows r0..r1-1 written). */
int orc_attn_unquant_rows(const double* q, const double* k, const double* v, int Lq, int Lkv, int D,
                          int causal, double sm_scale, int r0, int r1, double* out)
{
    int nkb = (Lkv + ORC_BLOCK - 1) / ORC_BLOCK;
    double* RO = (double*)malloc(sizeof(double) * (size_t)D);
    if (!RO)
        return -1;
    double z[ORC_BLOCK];
    for (int i = r0; i < r1; ++i) {
        long last = causal ? (long)i + Lkv - Lq : (long)Lkv - 1;
        if (last > Lkv - 1)
            last = Lkv - 1;
        double m = -INFINITY, l = 0.0;
        for (int c = 0; c < D; ++c)
            RO[c] = 0.0;
        for (int e = 0; e < nkb; ++e) {
            long j0 = (long)e * ORC_BLOCK;
            if (j0 > last)
                break;
            double mx = -INFINITY;
            for (int jj = 0; jj < ORC_BLOCK; ++jj) {
                long j = j0 + jj;
                if (j > last) {
                    z[jj] = -INFINITY;
                    continue;
                }
                double acc = 0.0;
                for (int c = 0; c < D; ++c)
                    acc += q[(long)i * D + c] * k[j * D + c];
                z[jj] = acc * sm_scale;
                if (z[jj] > mx)
                    mx = z[jj];
            }
            double mn = m > mx ? m : mx;
            if (mn == -INFINITY)
                continue;
            double alpha = (m == -INFINITY) ? 0.0 : exp(m - mn);
            double ps = 0.0;
            for (int jj = 0; jj < ORC_BLOCK; ++jj) {
                double pj = (z[jj] == -INFINITY) ? 0.0 : exp(z[jj] - mn);
                z[jj] = pj;
                ps += pj;
            }
            l = l * alpha + ps;
            for (int c = 0; c < D; ++c) {
                double pv = 0.0;
                for (int jj = 0; jj < ORC_BLOCK && j0 + jj < Lkv; ++jj)
                    pv += z[jj] * v[(j0 + jj) * D + c];
                RO[c] = RO[c] * alpha + pv;
            }
            m = mn;
        }
        for (int c = 0; c < D; ++c)
            out[(long)i * D + c] = (l > 0.0) ? RO[c] / l : 0.0;
    }
    free(RO);
    return 0;
}

/* ------------------------------------------ brute-force attention (iii) */

/* out[i] = sum_j w_j v_j / sum_j w_j with w_j = exp(s_j - max s),
 * s_j = sm_scale * q_i . k_j over the visible keys j (same mask as above). */
int orc_attn_ref_rows(const double* q, const double* k, const double* v, int Lq, int Lkv, int D,
                      int causal, double sm_scale, int r0, int r1, double* out)
{
    double* s = (double*)malloc(sizeof(double) * (size_t)(Lkv > 0 ? Lkv : 1));
    if (!s)
        return -1;
    for (int i = r0; i < r1; ++i) {
        long last = causal ? (long)i + Lkv - Lq : (long)Lkv - 1;
        if (last > Lkv - 1)
            last = Lkv - 1;
        if (last < 0) {
            for (int c = 0; c < D; ++c)
                out[(long)i * D + c] = 0.0;
            continue;
        }
        double mx = -INFINITY;
        for (long j = 0; j <= last; ++j) {
            double acc = 0.0;
            for (int c = 0; c < D; ++c)
                acc += q[(long)i * D + c] * k[j * D + c];
            s[j] = acc * sm_scale;
            if (s[j] > mx)
                mx = s[j];
        }
        double den = 0.0;
        for (long j = 0; j <= last; ++j) {
            s[j] = exp(s[j] - mx);
            den += s[j];
        }
        for (int c = 0; c < D; ++c) {
            double num = 0.0;
            for (long j = 0; j <= last; ++j)
                num += s[j] * v[j * D + c];
            out[(long)i * D + c] = num / den;
        }
    }
    free(s);
    return 0;
}

/* ------------------------------------------- whole hot path for one head */

/* Preparation followed by the quantized epoch loop over all rows of one
 * head: bf16 q, k, v in, bf16 out [Lq][D]. Returns the first nonzero status
 * of the two steps. */
int orc_sage_head(const uint16_t* q, const uint16_t* k, const uint16_t* v, int Lq, int Lkv, int D,
                  int causal, float sm_scale, uint16_t* out)
{
    int nqb = (Lq + ORC_BLOCK - 1) / ORC_BLOCK, nkb = (Lkv + ORC_BLOCK - 1) / ORC_BLOCK;
    int8_t* q8 = (int8_t*)malloc((size_t)nqb * ORC_BLOCK * D);
    int8_t* k8 = (int8_t*)malloc((size_t)nkb * ORC_BLOCK * D);
    uint8_t* v8 = (uint8_t*)malloc((size_t)nkb * ORC_BLOCK * D);
    float* qs = (float*)malloc(sizeof(float) * (size_t)nqb);
    float* ks = (float*)malloc(sizeof(float) * (size_t)nkb);
    float* km = (float*)malloc(sizeof(float) * (size_t)D);
    float* vs = (float*)malloc(sizeof(float) * (size_t)D);
    int st = -1;
    if (q8 && k8 && v8 && qs && ks && km && vs) {
        st = orc_prep_head(q, k, v, Lq, Lkv, D, 1, q8, qs, k8, ks, km, v8, vs);
        if (st == 0)
            st = orc_attn_rows(q8, qs, k8, ks, v8, vs, Lq, Lkv, D, causal, sm_scale, 0, Lq, out);
    }
    free(q8);
    free(k8);
    free(v8);
    free(qs);
    free(ks);
    free(km);
    free(vs);
    return st;
}
