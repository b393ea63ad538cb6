// Strided-reference residual KV cache: encode and decode attention.
//
// The variant of the gist.science explainer of DeltaKV (section 3.A,
// "Strided Reference Selection", "Residual Encoding", "Reconstruction";
// section 2 on similar tokens far apart): the tokens at positions 0, stride,
// 2*stride, ... are kept as exact fp16 reference rows; every token stores the
// index of its nearest reference and the Q4_0 code of its residual against
// it, and decodes as reference + residual.  The residual coder is the Q4_0
// block rule of the Delta-KV codec (dkv_q40.h) in place of a trained
// compressor, and the "mean of the most similar references" is taken over the
// single nearest one.
//
// Nearest: smallest squared distance between the fp16 rows, summed in double
// over the channels in order with every product and sum rounded on its own
// (no fused multiply-add), lowest index on ties, among references k with
// k*stride <= t and, when window > 0, k > t/stride - window.  The difference of
// two fp16 values is exact in double, so the choice is a fixed function of the
// inputs.
//
// Layout of one stream (sequence b, kv-head h, K or V), streams [b][h][K,V]
// back to back, every plane 256-byte aligned:
//   refs    fp16 [nref][D]    nref = ceil(capacity / stride)
//   codes   u8   [cap][D/2]   Q4_0 bytes, byte i of a block: code i | code i+16 << 4
//   scales  fp16 [cap][D/32]
//   idx     u16  [cap]        reference index of every token
//
// Decode attention: one workgroup of 256 threads per run of 32-token tiles
// of one (sequence, kv-head), all the kv-head's query heads.  Per tile the
// threads rebuild K and V (reference row gathered by index + dequantised
// residual) in fp32, take the logits, run the online softmax and accumulate
// the weighted V rows; the partial (acc, m, l) goes to the split-K combine
// shared with the Delta-KV kernels.  HBM traffic per token is the two
// streams' codes, scales and index (74 bytes each at D = 128); the reference
// rows, 1/stride of the tokens, are gathered from the L2 and Infinity caches.
#include "dkv_fused_common.h"
#include "dkv_q40.h"

namespace dkv {

__host__ __device__ inline int64_t pad256(int64_t x) { return (x + 255) & ~int64_t(255); }

struct StridedLayout {
    int nref;
    int64_t off_codes, off_scales, off_idx, stream_bytes;
};

__host__ __device__ inline StridedLayout strided_layout(const dkv_config &c)
{
    StridedLayout l;
    const int64_t cap = c.max_tokens, D = c.head_dim;
    l.nref = (int)((cap + c.kf - 1) / c.kf);
    l.off_codes = pad256((int64_t)l.nref * D * 2);
    l.off_scales = l.off_codes + pad256(cap * D / 2);
    l.off_idx = l.off_scales + pad256(cap * (D / 32) * 2);
    l.stream_bytes = l.off_idx + pad256(cap * 2);
    return l;
}

constexpr int kStridedThreads = 256;
constexpr int kStridedMaxG = 16;

// Squared distance of two fp16 rows in double, channel order, no contraction.
template <int D>
__device__ inline double sqdist_rows(const uint16_t *__restrict__ a, const uint16_t *__restrict__ b)
{
#pragma clang fp contract(off)
    double s = 0.0;
#pragma unroll 2
    for (int c8 = 0; c8 < D / 8; ++c8) {
        const u4 av = ((const u4 *)a)[c8], bv = ((const u4 *)b)[c8];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const double d0 = (double)h2f((uint16_t)(av[w] & 0xFFFF)) - (double)h2f((uint16_t)(bv[w] & 0xFFFF));
            const double q0 = d0 * d0;
            s = s + q0;
            const double d1 = (double)h2f((uint16_t)(av[w] >> 16)) - (double)h2f((uint16_t)(bv[w] >> 16));
            const double q1 = d1 * d1;
            s = s + q1;
        }
    }
    return s;
}

// grid (ceil(s_max / 32), n_kv_heads * 2, batch): one 32-token tile of one stream.
template <int D>
__global__ void __launch_bounds__(kStridedThreads)
    k_strided_encode(dkv_config cfg, uint8_t *__restrict__ cache, const uint16_t *__restrict__ k,
                     const uint16_t *__restrict__ v, const int32_t *__restrict__ lens, int s_max, int window)
{
    constexpr int NB = D / 32;
    const StridedLayout ly = strided_layout(cfg);
    const int stride = cfg.kf;
    const int tile = blockIdx.x, h = blockIdx.y >> 1, s = blockIdx.y & 1, b = blockIdx.z;
    const int tid = threadIdx.x;
    const int L = max(0, min(lens[b], min(s_max, cfg.max_tokens)));
    const int t0 = tile * 32;
    if (t0 >= L) return;
    const uint16_t *x = (s ? v : k) + ((int64_t)b * cfg.n_kv_heads + h) * s_max * D;
    uint8_t *base = cache + (((int64_t)b * cfg.n_kv_heads + h) * 2 + s) * ly.stream_bytes;
    uint16_t *refs = (uint16_t *)base;
    uint8_t *codes = base + ly.off_codes;
    uint16_t *scales = (uint16_t *)(base + ly.off_scales);
    uint16_t *idx = (uint16_t *)(base + ly.off_idx);

    // the tile's reference rows, copied exactly
    for (int e = tid; e < 32 * D; e += kStridedThreads) {
        const int t = t0 + e / D, c = e % D;
        if (t < L && t % stride == 0) refs[(int64_t)(t / stride) * D + c] = x[(int64_t)t * D + c];
    }

    // nearest reference: 8 lanes per token, each scanning every 8th candidate
    __shared__ int sidx[32];
    {
        const int tt = tid >> 3, sl = tid & 7, t = t0 + tt;
        double bd = INFINITY;
        int bk = 0x7FFFFFFF;
        if (t < L) {
            const int kt = t / stride;
            const int k0 = (window > 0 && kt - window + 1 > 0) ? kt - window + 1 : 0;
            for (int kk = k0 + sl; kk <= kt; kk += 8) {
                const double d = sqdist_rows<D>(x + (int64_t)t * D, x + (int64_t)kk * stride * D);
                if (d < bd) {
                    bd = d;
                    bk = kk;
                }
            }
        }
#pragma unroll
        for (int off = 1; off < 8; off <<= 1) {
            const double d2 = __shfl_xor(bd, off, 8);
            const int k2 = __shfl_xor(bk, off, 8);
            if (d2 < bd || (d2 == bd && k2 < bk)) {
                bd = d2;
                bk = k2;
            }
        }
        if (sl == 0) {
            sidx[tt] = t < L ? bk : 0;
            if (t < L) idx[t] = (uint16_t)bk;
        }
    }
    __syncthreads();

    // Q4_0 residuals: one 32-lane half-wave per (token, block)
    const int hw = tid >> 5, ln = tid & 31;
    for (int p = hw; p < 32 * NB; p += kStridedThreads / 32) {
        const int tt = p / NB, blk = p % NB, t = t0 + tt;
        if (t >= L) continue;                       // uniform over the half-wave
        const int c = 32 * blk + ln;
        const float xv = h2f(x[(int64_t)t * D + c]);
        float xh = h2f(x[(int64_t)sidx[tt] * stride * D + c]);
        int code;
        uint16_t s16;
        q40_delta_step(xv, xh, code, s16);
        const int hi = __shfl_down(code, 16, 32);
        if (ln < 16) codes[(int64_t)t * (D / 2) + 16 * blk + ln] = (uint8_t)(code | (hi << 4));
        if (ln == 0) scales[(int64_t)t * NB + blk] = s16;
    }
}

// Raw data of channels [c0, c0 + D/8) of one token of one stream: its code
// bytes, block scale and reference row slice (the row found through the
// token's index, clamped so that a token never encoded reads a wrong row, not
// past the plane).
template <int D>
struct RowRaw {
    uint32_t cw[D / 32];     // D/8 code bytes
    uint32_t rw[D / 16];     // D/8 fp16 reference values
    uint32_t sc;             // fp16 scale bits
};

// The token's reference index, clamped to the plane.
__device__ inline int strided_ref(const uint8_t *__restrict__ base, const StridedLayout &ly, int t)
{
    return min((int)((const uint16_t *)(base + ly.off_idx))[t], ly.nref - 1);
}

// Codes, scale and reference slice of token t with reference index k.
template <int D>
__device__ inline void strided_fetch(const uint8_t *__restrict__ base, const StridedLayout &ly, int t, int k, int c0,
                                     RowRaw<D> &w)
{
    constexpr int NB = D / 32, CPT = D / 8;
    const int blk = c0 >> 5, e0 = c0 & 31;
    w.sc = ((const uint16_t *)(base + ly.off_scales))[(int64_t)t * NB + blk];
    const uint8_t *cb = base + ly.off_codes + (int64_t)t * (D / 2) + 16 * blk + (e0 & 15);
    if constexpr (CPT == 16) {
        const u4 x = *(const u4 *)cb;
#pragma unroll
        for (int i = 0; i < 4; ++i) w.cw[i] = x[i];
    } else {
        const u2 x = *(const u2 *)cb;
        w.cw[0] = x[0];
        w.cw[1] = x[1];
    }
    const uint16_t *r = (const uint16_t *)base + (int64_t)k * D + c0;
#pragma unroll
    for (int i = 0; i < CPT / 8; ++i) {
        const u4 x = ((const u4 *)r)[i];
#pragma unroll
        for (int j = 0; j < 4; ++j) w.rw[4 * i + j] = x[j];
    }
}

// One new token per sequence at positions[b] (negative: none), the same
// coding as the prefill encode: candidates are read from the reference plane,
// which holds the rows the prefill read from its input, and the token itself
// when it is a reference.  grid (1, n_kv_heads * 2, batch).
template <int D>
__global__ void __launch_bounds__(kStridedThreads)
    k_strided_append(dkv_config cfg, uint8_t *__restrict__ cache, const uint16_t *__restrict__ knew,
                     const uint16_t *__restrict__ vnew, const int32_t *__restrict__ positions, int window)
{
    constexpr int NB = D / 32;
    const StridedLayout ly = strided_layout(cfg);
    const int stride = cfg.kf;
    const int h = blockIdx.y >> 1, s = blockIdx.y & 1, b = blockIdx.z;
    const int tid = threadIdx.x;
    const int t = positions[b];
    if (t < 0 || t >= cfg.max_tokens) return;
    const uint16_t *x = (s ? vnew : knew) + ((int64_t)b * cfg.n_kv_heads + h) * D;
    uint8_t *base = cache + (((int64_t)b * cfg.n_kv_heads + h) * 2 + s) * ly.stream_bytes;
    uint16_t *refs = (uint16_t *)base;
    const int kt = t / stride;
    const bool is_ref = t % stride == 0;
    const int k0 = (window > 0 && kt - window + 1 > 0) ? kt - window + 1 : 0;

    __shared__ double sd[kStridedThreads / 64];
    __shared__ int sk[kStridedThreads / 64];
    double bd = INFINITY;
    int bk = 0x7FFFFFFF;
    for (int kk = k0 + tid; kk <= kt; kk += kStridedThreads) {
        const uint16_t *r = (is_ref && kk == kt) ? x : refs + (int64_t)kk * D;
        const double d = sqdist_rows<D>(x, r);
        if (d < bd) {
            bd = d;
            bk = kk;
        }
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const double d2 = __shfl_xor(bd, off);
        const int k2 = __shfl_xor(bk, off);
        if (d2 < bd || (d2 == bd && k2 < bk)) {
            bd = d2;
            bk = k2;
        }
    }
    if ((tid & 63) == 0) {
        sd[tid >> 6] = bd;
        sk[tid >> 6] = bk;
    }
    __syncthreads();
    bd = sd[0];
    bk = sk[0];
#pragma unroll
    for (int w = 1; w < kStridedThreads / 64; ++w)
        if (sd[w] < bd || (sd[w] == bd && sk[w] < bk)) {
            bd = sd[w];
            bk = sk[w];
        }
    const uint16_t *r = (is_ref && bk == kt) ? x : refs + (int64_t)bk * D;
    if (tid == 0) ((uint16_t *)(base + ly.off_idx))[t] = (uint16_t)bk;
    // Q4_0 residual: one half-wave per block
    const int hw = tid >> 5, ln = tid & 31;
    if (hw < NB) {
        const int c = 32 * hw + ln;
        const float xv = h2f(x[c]);
        float xh = h2f(r[c]);
        int code;
        uint16_t s16;
        q40_delta_step(xv, xh, code, s16);
        const int hi = __shfl_down(code, 16, 32);
        if (ln < 16) base[ly.off_codes + (int64_t)t * (D / 2) + 16 * hw + ln] = (uint8_t)(code | (hi << 4));
        if (ln == 0) ((uint16_t *)(base + ly.off_scales))[(int64_t)t * NB + hw] = s16;
    }
    if (is_ref && tid < D) refs[(int64_t)kt * D + tid] = x[tid];
}

// Rebuild the channels in fp32: reference + (code - 8) * scale.
template <int D>
__device__ inline void strided_rebuild(const RowRaw<D> &w, int c0, float (&out)[D / 8])
{
    constexpr int CPT = D / 8;
    const int sh = 4 * ((c0 & 31) >> 4);
    const float sf = h2f((uint16_t)w.sc);
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int code = (int)((w.cw[i >> 2] >> (8 * (i & 3) + sh)) & 15u);
        const uint16_t rh = (uint16_t)((i & 1) ? (w.rw[i >> 1] >> 16) : (w.rw[i >> 1] & 0xFFFF));
        out[i] = __builtin_fmaf((float)(code - 8), sf, h2f(rh));     // exact product, one rounding
    }
}

// Lane reductions in registers (DPP moves within a row of 16 lanes, the
// row-pair swap across rows): every lane of the group gets the result.
template <int CTRL>
__device__ inline float dpp_f(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
__device__ inline float sum8_lanes(float x)          // groups of 8 aligned lanes
{
    x += dpp_f<0xB1>(x);     // quad_perm [1,0,3,2]
    x += dpp_f<0x4E>(x);     // quad_perm [2,3,0,1]
    return x + dpp_f<0x141>(x);   // row_half_mirror: the other quad of the 8
}
__device__ inline float sum32_lanes(float x)         // groups of 32 aligned lanes
{
    x = sum8_lanes(x);
    x += dpp_f<0x140>(x);    // row_mirror: the other 8 of the row
    float a0, a1;
    swap16(x, a0, a1);
    return a0 + a1;
}
__device__ inline float max32_lanes(float x)
{
    x = fmaxf(x, dpp_f<0xB1>(x));
    x = fmaxf(x, dpp_f<0x4E>(x));
    x = fmaxf(x, dpp_f<0x141>(x));
    x = fmaxf(x, dpp_f<0x140>(x));
    float a0, a1;
    swap16(x, a0, a1);
    return fmaxf(a0, a1);
}

// grid (nsplit, n_kv_heads, batch): the split's run of 32-token tiles.
// Per tile the 256 threads rebuild K and V (8 lanes per token, 16 B loads)
// into LDS; the logits (32 tokens x 16 head columns over D channels) and the
// weighted V rows (16 head rows x D channels over 32 tokens) are fp32
// matrix-core products (v_mfma_f32_16x16x4_f32: lane 16*j + n supplies row n
// of A and column n of B at k = j; it holds rows 4j..4j+3 of column n of the
// result), the query held in registers.  Head columns beyond the group are
// zero.  The next tile's rows are fetched while the current one is processed.
template <int D>
__global__ void __launch_bounds__(kStridedThreads)
    k_strided_attn(dkv_config cfg, const uint8_t *__restrict__ cache, const float *__restrict__ q,
                   const int32_t *__restrict__ lens, float scale_log2, float *__restrict__ ws, int nsplit, int chunk)
{
    constexpr int CPT = D / 8;
    constexpr int KS = D + 4, VS = D + 16;       // LDS row strides: conflict-free operand reads
    constexpr int NKK = D / 8;                   // k-steps of 4 channels over half the channels
    constexpr int NCB = D / 64;                  // 16-channel column blocks per wave
    const StridedLayout ly = strided_layout(cfg);
    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
    const int Hq = cfg.n_q_heads, G = Hq / cfg.n_kv_heads;
    const int L = max(0, min(lens[b], cfg.max_tokens));
    const int ntile = (L + 31) / 32;
    const int tb0 = split * chunk, tb1 = min(ntile, tb0 + chunk);
    const int64_t row0 = (int64_t)b * Hq + (int64_t)h * G;
    const int wv = tid >> 6, lane = tid & 63, jj = lane >> 4, nn = lane & 15;
    const int th = wv & 1, ch = wv >> 1;         // logits: token half, channel half of this wave

    __shared__ __attribute__((aligned(16))) float kt[32 * KS];
    __shared__ __attribute__((aligned(16))) float vt[32 * VS];
    __shared__ float lgp[2][kStridedMaxG][32];
    __shared__ float lg[kStridedMaxG][32];
    __shared__ float al[kStridedMaxG];
    for (int e = tid; e < kStridedMaxG * 32; e += kStridedThreads) (&lg[0][0])[e] = 0.0f;
    if (tid < kStridedMaxG) al[tid] = 1.0f;

    // query operand: head nn, channels ch*D/2 + 4*kk + jj (zero beyond the group)
    float qb[NKK];
    {
        const float *qr = q + (row0 + min(nn, G - 1)) * D + ch * (D / 2) + jj;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            const float x = qr[4 * kk] * scale_log2;
            qb[kk] = nn < G ? x : 0.0f;
        }
    }
    __syncthreads();

    const uint8_t *kb = cache + (((int64_t)b * cfg.n_kv_heads + h) * 2) * ly.stream_bytes;
    const uint8_t *vb = kb + ly.stream_bytes;
    float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.0f, 0.0f};
    f4 acc[NCB];
#pragma unroll
    for (int u = 0; u < NCB; ++u) acc[u] = f4{0.0f, 0.0f, 0.0f, 0.0f};

    const int tt = tid >> 3, sl = tid & 7, c0 = sl * CPT;
    RowRaw<D> nk, nv;
    if (tb0 < tb1 && tb0 * 32 + tt < L) {
        strided_fetch<D>(kb, ly, tb0 * 32 + tt, strided_ref(kb, ly, tb0 * 32 + tt), c0, nk);
        strided_fetch<D>(vb, ly, tb0 * 32 + tt, strided_ref(vb, ly, tb0 * 32 + tt), c0, nv);
    }
    for (int tile = tb0; tile < tb1; ++tile) {
        const int t0 = tile * 32, nt = min(32, L - t0);
        {
            float kh[CPT], vh[CPT];
            if (tt < nt) {
                strided_rebuild<D>(nk, c0, kh);
                strided_rebuild<D>(nv, c0, vh);
            } else {
#pragma unroll
                for (int i = 0; i < CPT; ++i) kh[i] = vh[i] = 0.0f;
            }
            if (tile + 1 < tb1 && t0 + 32 + tt < L) {
                strided_fetch<D>(kb, ly, t0 + 32 + tt, strided_ref(kb, ly, t0 + 32 + tt), c0, nk);
                strided_fetch<D>(vb, ly, t0 + 32 + tt, strided_ref(vb, ly, t0 + 32 + tt), c0, nv);
            }
#pragma unroll
            for (int i = 0; i < CPT; i += 4) {
                *(f4 *)&kt[tt * KS + c0 + i] = f4{kh[i], kh[i + 1], kh[i + 2], kh[i + 3]};
                *(f4 *)&vt[tt * VS + c0 + i] = f4{vh[i], vh[i + 1], vh[i + 2], vh[i + 3]};
            }
        }
        __syncthreads();
        // logits of tokens 16*th + row over channels [ch*D/2, (ch+1)*D/2)
        {
            f4 C = f4{0.0f, 0.0f, 0.0f, 0.0f};
            const float *ka = kt + (16 * th + nn) * KS + ch * (D / 2) + jj;
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) C = __builtin_amdgcn_mfma_f32_16x16x4f32(ka[4 * kk], qb[kk], C, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) lgp[ch][nn][16 * th + 4 * jj + i] = C[i];
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int g = (tid >> 5) + 8 * i, t = tid & 31;
            if (g < G) {                             // uniform over the half-wave
                const float x = t < nt ? lgp[0][g][t] + lgp[1][g][t] : -INFINITY;
                const float mx = max32_lanes(x);
                const float m_new = fmaxf(m_run[i], mx);
                const float p = x == -INFINITY ? 0.0f : exp2f(x - m_new);
                const float alpha = exp2f(m_run[i] - m_new);
                const float sum = sum32_lanes(p);
                l_run[i] = l_run[i] * alpha + sum;
                m_run[i] = m_new;
                lg[g][t] = p;
                if (t == 0) al[g] = alpha;
            }
        }
        __syncthreads();
        // weighted V rows: heads 4*jj + i, channels 16*cb + nn
        {
            float alr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) alr[i] = al[4 * jj + i];
#pragma unroll
            for (int u = 0; u < NCB; ++u)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[u][i] *= alr[i];
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                const float pa = lg[nn][4 * kk + jj];
#pragma unroll
                for (int u = 0; u < NCB; ++u) {
                    const int cb = wv * NCB + u;
                    acc[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(pa, vt[(4 * kk + jj) * VS + 16 * cb + nn], acc[u],
                                                                  0, 0, 0);
                }
            }
        }
        __syncthreads();
    }
    constexpr int R = part_stride(D);
#pragma unroll
    for (int u = 0; u < NCB; ++u) {
        const int cb = wv * NCB + u;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int g = 4 * jj + i;
            if (g < G) ws[((row0 + g) * nsplit + split) * R + 16 * cb + nn] = acc[u][i];
        }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int g = (tid >> 5) + 8 * i;
        if (g < G && (tid & 31) == 0) {
            float *rec = ws + ((row0 + g) * nsplit + split) * R;
            rec[D] = m_run[i];
            rec[D + 1] = l_run[i];
        }
    }
}

int64_t strided_cache_bytes(const dkv_config &c)
{
    return strided_layout(c).stream_bytes * 2 * c.batch * c.n_kv_heads;
}

void strided_plane_offsets(const dkv_config &c, int64_t *off)
{
    const StridedLayout l = strided_layout(c);
    off[0] = 0;
    off[1] = l.off_codes;
    off[2] = l.off_scales;
    off[3] = l.off_idx;
    off[4] = l.stream_bytes;
    off[5] = l.nref;
}

hipError_t launch_strided_encode(const dkv_config &c, void *cache, const uint16_t *k, const uint16_t *v,
                                 const int32_t *lens, int s_max, int window, hipStream_t st)
{
    dim3 grid((s_max + 31) / 32, c.n_kv_heads * 2, c.batch);
    if (c.head_dim == 64)
        hipLaunchKernelGGL(k_strided_encode<64>, grid, dim3(kStridedThreads), 0, st, c, (uint8_t *)cache, k, v,
                           lens, s_max, window);
    else
        hipLaunchKernelGGL(k_strided_encode<128>, grid, dim3(kStridedThreads), 0, st, c, (uint8_t *)cache, k, v,
                           lens, s_max, window);
    return hipGetLastError();
}

hipError_t launch_strided_append(const dkv_config &c, void *cache, const uint16_t *knew, const uint16_t *vnew,
                                 const int32_t *positions, int window, hipStream_t st)
{
    dim3 grid(1, c.n_kv_heads * 2, c.batch);
    if (c.head_dim == 64)
        hipLaunchKernelGGL(k_strided_append<64>, grid, dim3(kStridedThreads), 0, st, c, (uint8_t *)cache, knew, vnew,
                           positions, window);
    else
        hipLaunchKernelGGL(k_strided_append<128>, grid, dim3(kStridedThreads), 0, st, c, (uint8_t *)cache, knew,
                           vnew, positions, window);
    return hipGetLastError();
}

hipError_t launch_strided_attn(const dkv_config &c, const void *cache, const float *q, const int32_t *lens,
                               float scale_log2, float *ws, int nsplit, int chunk, hipStream_t st)
{
    dim3 grid(nsplit, c.n_kv_heads, c.batch);
    if (c.head_dim == 64)
        hipLaunchKernelGGL(k_strided_attn<64>, grid, dim3(kStridedThreads), 0, st, c, (const uint8_t *)cache, q,
                           lens, scale_log2, ws, nsplit, chunk);
    else
        hipLaunchKernelGGL(k_strided_attn<128>, grid, dim3(kStridedThreads), 0, st, c, (const uint8_t *)cache, q,
                           lens, scale_log2, ws, nsplit, chunk);
    return hipGetLastError();
}

}  // namespace dkv
