/*
 * Delta-KV CPU oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, sequential, deliberately slow C11 that spells out what the Delta-KV
 * path computes.  Only the test suite, the smoke check and the CPU-baseline leg
 * of the benchmark may load this file's library.  It shares no code, header,
 * table or helper with the HIP library, and the product path never calls it.
 *
 * Build: gcc -std=c11 -O2 -ffp-contract=off -fno-fast-math (SSE arithmetic,
 * default MXCSR: IEEE binary32 with round-to-nearest-even, no FTZ/DAZ).
 *
 * Sources (web pages, cited by title and section):
 *  [DKV]  "영상 압축 기법을 KV 캐시에 적용해 Q4 양자화 오차를 10,000배 줄인 Delta-KV"
 *         (jeff.news), sections "핵심 아이디어" (keyframe + token-to-token delta,
 *         4-bit like Q4_0), "벤치마크" (Q4_0 as the 4-bit format, kf=32),
 *         "컨텍스트 길이에 따른 안정성" (no error growth even at 512 delta frames).
 *  [VQ]   "KV 캐시 벡터 양자화와 주의 보존 변환" (llm-wiki.hwlabs.dev), section
 *         "왜 복원 오차가 틀린 기준인가" (attention = softmax(Q·K^T/sqrt(d)) then A·V).
 *
 * Readings taken where the pages are silent (each one is listed in the design
 * notes with its reason):
 *  - keyframe: the fp16 row itself, at every token t with t % kf == 0;
 *  - delta: closed loop, d_t = x_t - xhat_{t-1}, where xhat is the decoder's own
 *    reconstruction (so the quantisation error cannot accumulate);
 *  - Q4_0 block: 32 values, m = the signed value of largest magnitude (first
 *    index wins ties), s = m / -8, id = 1/s (0 if s == 0),
 *    code = min(15, trunc(v*id + 8.5)) with both operations rounded separately,
 *    the stored scale is fp16(s) rounded to nearest even, and byte i of the 16
 *    code bytes holds code i in its low nibble and code i+16 in its high nibble;
 *  - reconstruction: xhat_t = fp32(xhat_{t-1} + (code-8)*float(s16)), one
 *    rounding per token and channel, folded left to right from the keyframe;
 *  - attention: float64 over the reconstructed fp32 rows, scale given in fp32;
 *    an empty sequence yields a zero output row;
 *  - Q4-keyframe variant ([DKV] "벤치마크": the same 4-bit storage as Q4_0):
 *    the keyframe row is coded as Q4_0 against a zero reference and decoded
 *    as 0 + (code-8)*scale; every other row as in the delta rule above, so
 *    each row is one plain Q4_0 row and kf = 1 is plain Q4_0.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* IEEE binary16 <-> binary32                                               */
/* ------------------------------------------------------------------------ */

/* Exact widening of an fp16 bit pattern. */
float oracle_f16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1F;
    int mant = h & 0x3FF;
    float mag;
    if (expo == 0) {
        mag = ldexpf((float)mant, -24);              /* zero or subnormal */
    } else if (expo == 31) {
        mag = mant ? NAN : INFINITY;
    } else {
        mag = ldexpf((float)(1024 + mant), expo - 25);
    }
    return sign ? -mag : mag;
}

/* fp32 -> fp16, round to nearest, ties to even; overflow gives infinity. */
uint16_t oracle_f32_to_f16(float f)
{
    uint16_t sign = signbit(f) ? 0x8000 : 0;
    float a = fabsf(f);
    if (isnan(f)) return (uint16_t)(sign | 0x7E00);
    if (isinf(a)) return (uint16_t)(sign | 0x7C00);
    if (a == 0.0f) return sign;
    int e;
    frexpf(a, &e);            /* a = frac * 2^e, frac in [0.5, 1) */
    e -= 1;                   /* a in [2^e, 2^(e+1)) */
    if (e < -14) {
        /* subnormal range: quantum 2^-24; n == 1024 lands on the smallest normal */
        float n = rintf(ldexpf(a, 24));
        return (uint16_t)(sign | (uint16_t)n);
    }
    float n = rintf(ldexpf(a, 10 - e));   /* in [1024, 2048] */
    if (n >= 2048.0f) { n = 1024.0f; e += 1; }
    if (e + 15 >= 31) return (uint16_t)(sign | 0x7C00);
    return (uint16_t)(sign | ((e + 15) << 10) | ((int)n - 1024));
}

/* ------------------------------------------------------------------------ */
/* Q4_0 block quantiser ([DKV] "핵심 아이디어", "벤치마크": 4-bit Q4_0 blocks)     */
/* ------------------------------------------------------------------------ */

/* Quantise 32 values; codes are returned unpacked (0..15). */
void oracle_q40_block(const float *v, uint16_t *s16, uint8_t *codes)
{
    float amax = 0.0f;
    float m = 0.0f;
    for (int j = 0; j < 32; ++j) {
        float a = fabsf(v[j]);
        if (a > amax) {       /* strict: the first index of the maximum wins */
            amax = a;
            m = v[j];
        }
    }
    float s = m / -8.0f;
    float id = (s != 0.0f) ? 1.0f / s : 0.0f;
    for (int j = 0; j < 32; ++j) {
        float t = v[j] * id;
        t = t + 8.5f;
        int c = (int)t;       /* t >= 0 here, so truncation is floor */
        codes[j] = (uint8_t)(c > 15 ? 15 : c);
    }
    *s16 = oracle_f32_to_f16(s);
}

/* Pack 32 codes into the 16 Q4_0 bytes: byte i = code[i] | code[i+16] << 4. */
void oracle_q40_pack(const uint8_t *codes, uint8_t *bytes)
{
    for (int i = 0; i < 16; ++i)
        bytes[i] = (uint8_t)(codes[i] | (codes[i + 16] << 4));
}

void oracle_q40_unpack(const uint8_t *bytes, uint8_t *codes)
{
    for (int i = 0; i < 16; ++i) {
        codes[i] = bytes[i] & 0x0F;
        codes[i + 16] = bytes[i] >> 4;
    }
}

/* ------------------------------------------------------------------------ */
/* Delta-KV stream codec ([DKV] "핵심 아이디어": keyframe, then deltas)           */
/*                                                                          */
/* One stream = the K (or V) rows of one (sequence, kv-head): x[S][D] fp16.   */
/* Canonical (oracle) storage of an encoded stream:                          */
/*   kf_rows [ceil(S/kf)][D]  fp16 bits, the keyframe of each group          */
/*   codes   [n_delta][D/2]   Q4_0 bytes of each delta token, block-major      */
/*   scales  [n_delta][D/32]  fp16 bits of each delta block's scale            */
/* where delta token t (t % kf != 0) has index (t/kf)*(kf-1) + (t%kf) - 1.      */
/* ------------------------------------------------------------------------ */

long oracle_delta_index(long t, int kf)
{
    return (t / kf) * (long)(kf - 1) + (t % kf) - 1;
}

/*
 * Encode one token of a stream at position t, given the reconstruction state
 * xh[D] of token t-1 (ignored when t opens a group).  Updates xh to the
 * reconstruction of token t.  This is both the append step and, repeated,
 * the bulk encoder.
 */
void oracle_step(const uint16_t *x, long t, int D, int kf,
                 uint16_t *kf_rows, uint8_t *codes, uint16_t *scales, float *xh)
{
    if (t % kf == 0) {
        uint16_t *row = kf_rows + (t / kf) * (long)D;
        for (int c = 0; c < D; ++c) {
            row[c] = x[c];
            xh[c] = oracle_f16_to_f32(x[c]);
        }
        return;
    }
    long di = oracle_delta_index(t, kf);
    uint8_t *crow = codes + di * (long)(D / 2);
    uint16_t *srow = scales + di * (long)(D / 32);
    float d[32];
    uint8_t q[32];
    for (int b = 0; b < D / 32; ++b) {
        for (int j = 0; j < 32; ++j) {
            int c = 32 * b + j;
            d[j] = oracle_f16_to_f32(x[c]) - xh[c];
        }
        uint16_t s16;
        oracle_q40_block(d, &s16, q);
        srow[b] = s16;
        oracle_q40_pack(q, crow + 16 * b);
        float sf = oracle_f16_to_f32(s16);
        for (int j = 0; j < 32; ++j) {
            int c = 32 * b + j;
            float step = (float)((int)q[j] - 8) * sf;   /* exact product */
            xh[c] = xh[c] + step;                        /* one rounding */
        }
    }
}

/* Encode S tokens of one stream.  recon (optional) receives every xhat_t. */
void oracle_encode_stream(const uint16_t *x, long S, int D, int kf,
                          uint16_t *kf_rows, uint8_t *codes, uint16_t *scales,
                          float *recon, float *state)
{
    float *xh = (float *)calloc((size_t)D, sizeof(float));
    for (long t = 0; t < S; ++t) {
        oracle_step(x + t * (long)D, t, D, kf, kf_rows, codes, scales, xh);
        if (recon) memcpy(recon + t * (long)D, xh, sizeof(float) * (size_t)D);
    }
    if (state) memcpy(state, xh, sizeof(float) * (size_t)D);
    free(xh);
}

/* Decoder: the same recurrence, read back from the stored stream. */
void oracle_reconstruct_stream(const uint16_t *kf_rows, const uint8_t *codes,
                               const uint16_t *scales, long S, int D, int kf,
                               float *out)
{
    float *xh = (float *)calloc((size_t)D, sizeof(float));
    uint8_t q[32];
    for (long t = 0; t < S; ++t) {
        if (t % kf == 0) {
            const uint16_t *row = kf_rows + (t / kf) * (long)D;
            for (int c = 0; c < D; ++c) xh[c] = oracle_f16_to_f32(row[c]);
        } else {
            long di = oracle_delta_index(t, kf);
            for (int b = 0; b < D / 32; ++b) {
                oracle_q40_unpack(codes + di * (long)(D / 2) + 16 * b, q);
                float sf = oracle_f16_to_f32(scales[di * (long)(D / 32) + b]);
                for (int j = 0; j < 32; ++j) {
                    int c = 32 * b + j;
                    float step = (float)((int)q[j] - 8) * sf;
                    xh[c] = xh[c] + step;
                }
            }
        }
        memcpy(out + t * (long)D, xh, sizeof(float) * (size_t)D);
    }
    free(xh);
}

/* ------------------------------------------------------------------------ */
/* Plain Q4_0 of absolute values (the comparison cache of [DKV] "벤치마크")      */
/* ------------------------------------------------------------------------ */

void oracle_q40_abs_stream(const uint16_t *x, long S, int D,
                           uint8_t *codes, uint16_t *scales)
{
    float v[32];
    uint8_t q[32];
    for (long t = 0; t < S; ++t) {
        for (int b = 0; b < D / 32; ++b) {
            for (int j = 0; j < 32; ++j)
                v[j] = oracle_f16_to_f32(x[t * (long)D + 32 * b + j]);
            oracle_q40_block(v, &scales[t * (long)(D / 32) + b], q);
            oracle_q40_pack(q, codes + t * (long)(D / 2) + 16 * b);
        }
    }
}

void oracle_q40_dequant_stream(const uint8_t *codes, const uint16_t *scales,
                               long S, int D, float *out)
{
    uint8_t q[32];
    for (long t = 0; t < S; ++t) {
        for (int b = 0; b < D / 32; ++b) {
            oracle_q40_unpack(codes + t * (long)(D / 2) + 16 * b, q);
            float sf = oracle_f16_to_f32(scales[t * (long)(D / 32) + b]);
            for (int j = 0; j < 32; ++j)
                out[t * (long)D + 32 * b + j] = (float)((int)q[j] - 8) * sf;
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Q4-keyframe variant: the keyframe itself stored as Q4_0 of its absolute    */
/* values, so every row of a stream takes the 4-bit storage of Q4_0 ([DKV]    */
/* "벤치마크": Delta-KV keeps Q4_0's storage at 4 bits).  Row t of a stream:   */
/*   reference r_t = 0 when t % kf == 0 (a keyframe), else xhat_{t-1};        */
/*   d_t = x_t - r_t, quantised one Q4_0 block per 32 channels;               */
/*   xhat_t = fp32(r_t + (code-8)*float(s16)), one rounding per channel.      */
/* Storage per row: codes [D/2] and scales [D/32] exactly as a plain Q4_0 row */
/* (18 bytes per 32 values); with kf = 1 every row is a keyframe and the     */
/* stream is plain Q4_0 of x.                                                 */
/* ------------------------------------------------------------------------ */

void oracle_q4k_step(const uint16_t *x, long t, int D, int kf, uint8_t *codes, uint16_t *scales, float *xh)
{
    int key = (t % kf) == 0;
    float d[32];
    uint8_t q[32];
    for (int b = 0; b < D / 32; ++b) {
        for (int j = 0; j < 32; ++j) {
            int c = 32 * b + j;
            float ref = key ? 0.0f : xh[c];
            d[j] = oracle_f16_to_f32(x[c]) - ref;
        }
        uint16_t s16;
        oracle_q40_block(d, &s16, q);
        scales[t * (long)(D / 32) + b] = s16;
        oracle_q40_pack(q, codes + t * (long)(D / 2) + 16 * b);
        float sf = oracle_f16_to_f32(s16);
        for (int j = 0; j < 32; ++j) {
            int c = 32 * b + j;
            float ref = key ? 0.0f : xh[c];
            float step = (float)((int)q[j] - 8) * sf;     /* exact product */
            xh[c] = ref + step;                            /* one rounding */
        }
    }
}

void oracle_q4k_encode_stream(const uint16_t *x, long S, int D, int kf, uint8_t *codes, uint16_t *scales,
                              float *recon, float *state)
{
    float *xh = (float *)calloc((size_t)D, sizeof(float));
    for (long t = 0; t < S; ++t) {
        oracle_q4k_step(x + t * (long)D, t, D, kf, codes, scales, xh);
        if (recon) memcpy(recon + t * (long)D, xh, sizeof(float) * (size_t)D);
    }
    if (state) memcpy(state, xh, sizeof(float) * (size_t)D);
    free(xh);
}

/* Decoder of the Q4-keyframe stream: the same recurrence read back. */
void oracle_q4k_reconstruct_stream(const uint8_t *codes, const uint16_t *scales, long S, int D, int kf, float *out)
{
    float *xh = (float *)calloc((size_t)D, sizeof(float));
    uint8_t q[32];
    for (long t = 0; t < S; ++t) {
        int key = (t % kf) == 0;
        for (int b = 0; b < D / 32; ++b) {
            oracle_q40_unpack(codes + t * (long)(D / 2) + 16 * b, q);
            float sf = oracle_f16_to_f32(scales[t * (long)(D / 32) + b]);
            for (int j = 0; j < 32; ++j) {
                int c = 32 * b + j;
                float ref = key ? 0.0f : xh[c];
                xh[c] = ref + (float)((int)q[j] - 8) * sf;
            }
        }
        memcpy(out + t * (long)D, xh, sizeof(float) * (size_t)D);
    }
    free(xh);
}

/* ------------------------------------------------------------------------ */
/* Plain Q8_0 of absolute values: the 8-bit reference the Delta-KV article's   */
/* "벤치마크" section compares against (near-lossless next to F16).  The block */
/* rule is the publicly documented convention of that format: per 32 values,  */
/*   amax = max |v|,  d = amax / 127,  id = d != 0 ? 1/d : 0,                 */
/*   code_j = round-half-away-from-zero(v_j * id)  (|code| <= 127),            */
/*   stored scale = fp16(d) (round to nearest even);                          */
/*   dequantised value = code_j * float(stored scale).                        */
/* Each operation is one correctly rounded fp32 step (no FMA).               */
/* ------------------------------------------------------------------------ */

void oracle_q80_block(const float *v, uint16_t *d16, int8_t *codes)
{
    float amax = 0.0f;
    for (int j = 0; j < 32; ++j) {
        float a = fabsf(v[j]);
        if (a > amax) amax = a;
    }
    float d = amax / 127.0f;
    float id = (d != 0.0f) ? 1.0f / d : 0.0f;
    for (int j = 0; j < 32; ++j) {
        float t = v[j] * id;
        codes[j] = (int8_t)roundf(t);     /* |t| <= 127 up to rounding: no clamp needed */
    }
    *d16 = oracle_f32_to_f16(d);
}

void oracle_q80_abs_stream(const uint16_t *x, long S, int D, int8_t *codes, uint16_t *scales)
{
    float v[32];
    for (long t = 0; t < S; ++t)
        for (int b = 0; b < D / 32; ++b) {
            for (int j = 0; j < 32; ++j)
                v[j] = oracle_f16_to_f32(x[t * (long)D + 32 * b + j]);
            oracle_q80_block(v, &scales[t * (long)(D / 32) + b], codes + t * (long)D + 32 * b);
        }
}

void oracle_q80_dequant_stream(const int8_t *codes, const uint16_t *scales, long S, int D, float *out)
{
    for (long t = 0; t < S; ++t)
        for (int b = 0; b < D / 32; ++b) {
            float sf = oracle_f16_to_f32(scales[t * (long)(D / 32) + b]);
            for (int j = 0; j < 32; ++j)
                out[t * (long)D + 32 * b + j] = (float)codes[t * (long)D + 32 * b + j] * sf;
        }
}

/* ------------------------------------------------------------------------ */
/* Decode attention in float64 ([VQ] "왜 복원 오차가 틀린 기준인가")              */
/*                                                                          */
/* G query heads that share one kv-head: q[G][D], keys/values K[S][D],       */
/* V[S][D] (fp32 rows, e.g. the reconstruction), out[G][D] in float64:       */
/*   l_t = scale * sum_c q_c K_t,c ;  p_t = exp(l_t - max l) ;                */
/*   out = sum_t p_t V_t / sum_t p_t                                          */
/* ------------------------------------------------------------------------ */

void oracle_attention_f64(const float *q, int G, const float *K, const float *V,
                          long S, int D, float scale, double *out)
{
    double *l = (double *)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1));
    for (int h = 0; h < G; ++h) {
        const float *qh = q + (long)h * D;
        double *oh = out + (long)h * D;
        for (int c = 0; c < D; ++c) oh[c] = 0.0;
        if (S <= 0) continue;
        double mx = -INFINITY;
        for (long t = 0; t < S; ++t) {
            double acc = 0.0;
            for (int c = 0; c < D; ++c)
                acc += (double)qh[c] * (double)K[t * (long)D + c];
            l[t] = (double)scale * acc;
            if (l[t] > mx) mx = l[t];
        }
        double den = 0.0;
        for (long t = 0; t < S; ++t) {
            double p = exp(l[t] - mx);
            den += p;
            for (int c = 0; c < D; ++c) oh[c] += p * (double)V[t * (long)D + c];
        }
        for (int c = 0; c < D; ++c) oh[c] /= den;
    }
    free(l);
}

/* ------------------------------------------------------------------------ */
/* Strided-reference residual coding (the gist.science explainer of DeltaKV,
 * "3. 제안 방법론", A: "Strided Reference Selection", "Residual Encoding",
 * "Reconstruction"; section 2 motivates references far back in the history).
 *
 * References: the tokens at positions 0, stride, 2*stride, ... , kept as their
 * exact fp16 rows.  Token t chooses, among the references k with
 * k*stride <= t (and, when window > 0, k > t/stride - window), the one nearest
 * to it: smallest squared Euclidean distance between the fp16 rows.  The
 * distance is summed in double over channels 0..D-1 in order, each product
 * and each sum rounded on its own (the difference of two fp16 values is exact
 * in double); the lowest index wins ties.  The residual x_t - r (one fp32
 * subtraction per channel) is coded with the Q4_0 block rule above, and
 * xhat_t = r + (code - 8) * scale (exact product, one rounding).  A reference
 * token picks itself (distance 0) or an identical earlier row, so it is
 * reconstructed exactly.  Plain reading: the mean of the most similar
 * references is taken over one reference (the nearest); the residual coder is
 * Q4_0 instead of a trained compressor. */
double oracle_sqdist_f16(const uint16_t *a, const uint16_t *b, int D)
{
    double s = 0.0;
    for (int c = 0; c < D; ++c) {
        double d = (double)oracle_f16_to_f32(a[c]) - (double)oracle_f16_to_f32(b[c]);
        double sq = d * d;
        s = s + sq;
    }
    return s;
}

/* Order of two distances for the nearest-reference choice: the usual order of
 * numbers (+infinity included), with a NaN distance (a NaN in either row, or
 * infinities of one sign in the same channel of both) ranked above every
 * number and equal to another NaN.  Inputs are meant to be finite; this only
 * fixes which reference such a row takes. */
static int oracle_dist_less(double a, double b)
{
    if (isnan(a)) return 0;
    if (isnan(b)) return 1;
    return a < b;
}

void oracle_strided_encode_stream(const uint16_t *x, long S, int D, int stride, int window,
                                  uint16_t *refs, int32_t *ref_idx, uint8_t *codes, uint16_t *scales,
                                  float *recon)
{
    float v[32];
    uint8_t q[32];
    for (long k = 0; k * stride < S; ++k) memcpy(refs + k * (long)D, x + k * stride * (long)D, 2 * (size_t)D);
    for (long t = 0; t < S; ++t) {
        const uint16_t *xt = x + t * (long)D;
        const long kt = t / stride;
        const long k0 = (window > 0 && kt - window + 1 > 0) ? kt - window + 1 : 0;
        long best = k0;
        double bd = oracle_sqdist_f16(xt, refs + k0 * (long)D, D);
        for (long k = k0 + 1; k <= kt; ++k) {
            double d = oracle_sqdist_f16(xt, refs + k * (long)D, D);
            if (oracle_dist_less(d, bd)) {
                bd = d;
                best = k;
            }
        }
        ref_idx[t] = (int32_t)best;
        const uint16_t *r = refs + best * (long)D;
        for (int b = 0; b < D / 32; ++b) {
            for (int j = 0; j < 32; ++j) {
                int c = 32 * b + j;
                v[j] = oracle_f16_to_f32(xt[c]) - oracle_f16_to_f32(r[c]);
            }
            uint16_t s16;
            oracle_q40_block(v, &s16, q);
            scales[t * (long)(D / 32) + b] = s16;
            oracle_q40_pack(q, codes + t * (long)(D / 2) + 16 * b);
            float sf = oracle_f16_to_f32(s16);
            for (int j = 0; j < 32; ++j) {
                int c = 32 * b + j;
                float step = (float)((int)q[j] - 8) * sf;
                recon[t * (long)D + c] = oracle_f16_to_f32(r[c]) + step;
            }
        }
    }
}
