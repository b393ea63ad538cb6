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
// Decode attention: one wave per run of 32-token tiles of one (sequence,
// kv-head), all the kv-head's query heads.  Per 16-token sub-tile the wave
// rebuilds K and V (reference row gathered by index + dequantised residual)
// in fp32, takes the logits and the weighted V rows on fp32 matrix cores and
// runs the online softmax; the partial (acc, m, l) goes to the split-K
// combine shared with the Delta-KV kernels.  HBM traffic per token is the two
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

// Ordering key of a distance for the nearest-reference choice: distances are
// +0 or positive, so their bit patterns order like the numbers (+infinity
// included); a NaN distance (a NaN in either row, or infinities of one sign
// in the same channel of both) is ranked above every number.  The nearest
// reference is the smallest (key, index) pair, so a row holding a NaN takes
// the first candidate.
__device__ inline uint64_t dist_key(double d)
{
    return d != d ? 0x7FF8000000000000ull : (uint64_t)__builtin_bit_cast(int64_t, d);
}
// (key, index) lexicographic minimum of two candidates, kept in (bd, bk).
__device__ inline void keep_nearer(uint64_t &bd, int &bk, uint64_t d2, int k2)
{
    if (d2 < bd || (d2 == bd && k2 < bk)) {
        bd = d2;
        bk = k2;
    }
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
        // a lane without candidates keeps the largest key and loses to every
        // real candidate; every token has at least one (k0 <= t / stride)
        uint64_t bd = ~0ull;
        int bk = 0x7FFFFFFF;
        const int kt = t / stride;
        if (t < L) {
            const int k0 = (window > 0 && kt - window + 1 > 0) ? kt - window + 1 : 0;
            for (int kk = k0 + sl; kk <= kt; kk += 8)
                keep_nearer(bd, bk, dist_key(sqdist_rows<D>(x + (int64_t)t * D, x + (int64_t)kk * stride * D)), kk);
        }
#pragma unroll
        for (int off = 1; off < 8; off <<= 1) {
            const uint64_t d2 = __shfl_xor(bd, off, 8);
            const int k2 = __shfl_xor(bk, off, 8);
            keep_nearer(bd, bk, d2, k2);
        }
        bk = min(bk, kt);
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

// The token's reference index, clamped to the plane.
__device__ inline int strided_ref(const uint8_t *__restrict__ base, const StridedLayout &ly, int t)
{
    return min((int)((const uint16_t *)(base + ly.off_idx))[t], ly.nref - 1);
}

// The append of one token t of one stream by one wave: candidates scanned
// by the 64 lanes, the argmin over
// (distance, index) across the wave, then the Q4_0 blocks two half-waves at a
// time, and the token's row kept when it is a reference.
template <int D>
__device__ inline void strided_append_wave(const StridedLayout &ly, int stride, uint8_t *base,
                                           const uint16_t *__restrict__ x, int t, int window, int lane)
{
    constexpr int NB = D / 32;
    uint16_t *refs = (uint16_t *)base;
    const int kt = t / stride;
    const bool is_ref = t % stride == 0;
    const int k0 = (window > 0 && kt - window + 1 > 0) ? kt - window + 1 : 0;
    uint64_t bd = ~0ull;        // as in k_strided_encode: no candidate loses to any
    int bk = 0x7FFFFFFF;
    for (int kk = k0 + lane; kk <= kt; kk += 64) {
        const uint16_t *r = (is_ref && kk == kt) ? x : refs + (int64_t)kk * D;
        keep_nearer(bd, bk, dist_key(sqdist_rows<D>(x, r)), kk);
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint64_t d2 = __shfl_xor(bd, off);
        const int k2 = __shfl_xor(bk, off);
        keep_nearer(bd, bk, d2, k2);
    }
    bk = min(bk, kt);
    const uint16_t *r = (is_ref && bk == kt) ? x : refs + (int64_t)bk * D;
    if (lane == 0) ((uint16_t *)(base + ly.off_idx))[t] = (uint16_t)bk;
    const int ln = lane & 31;
    for (int blk = lane >> 5; blk < NB; blk += 2) {       // the same count for both half-waves
        const int c = 32 * blk + ln;
        const float xv = h2f(x[c]);
        float xh = h2f(r[c]);
        int code;
        uint16_t s16;
        q40_delta_step(xv, xh, code, s16);
        const int hi = __shfl_down(code, 16, 32);
        if (ln < 16) base[ly.off_codes + (int64_t)t * (D / 2) + 16 * blk + ln] = (uint8_t)(code | (hi << 4));
        if (ln == 0) ((uint16_t *)(base + ly.off_scales))[(int64_t)t * NB + blk] = s16;
    }
    if (is_ref)
        for (int c = lane; c < D; c += 64) refs[(int64_t)kt * D + c] = x[c];
}

// One new token per sequence at positions[b] (negative: none), the same
// coding as the prefill encode: candidates are read from the reference plane,
// which holds the rows the prefill read from its input, and the token itself
// when it is a reference.  grid (1, n_kv_heads * 2, batch), one wave.
template <int D>
__global__ void __launch_bounds__(64)
    k_strided_append(dkv_config cfg, uint8_t *__restrict__ cache, const uint16_t *__restrict__ knew,
                     const uint16_t *__restrict__ vnew, const int32_t *__restrict__ positions, int window)
{
    const StridedLayout ly = strided_layout(cfg);
    const int h = blockIdx.y >> 1, s = blockIdx.y & 1, b = blockIdx.z;
    const int t = positions[b];
    if (t < 0 || t >= cfg.max_tokens) return;
    const uint16_t *x = (s ? vnew : knew) + ((int64_t)b * cfg.n_kv_heads + h) * D;
    uint8_t *base = cache + (((int64_t)b * cfg.n_kv_heads + h) * 2 + s) * ly.stream_bytes;
    strided_append_wave<D>(ly, cfg.kf, base, x, t, window, threadIdx.x);
}

// Raw data of D/4 channels [c0, c0 + D/4) of one token of one stream (one
// block at D = 128, half a block at D = 64): the block's 16 code bytes, its
// scale and the reference row slice.
template <int D>
struct RowQ {
    uint32_t cw[4];
    uint32_t rw[D / 8];
    uint32_t sc;
};

template <int D>
__device__ inline void strided_fetch_q(const uint8_t *__restrict__ base, const StridedLayout &ly, int t, int c0,
                                       RowQ<D> &w)
{
    constexpr int NB = D / 32;
    const int k = strided_ref(base, ly, t);
    const int blk = c0 >> 5;
    w.sc = ((const uint16_t *)(base + ly.off_scales))[(int64_t)t * NB + blk];
    const u4 x = *(const u4 *)(base + ly.off_codes + (int64_t)t * (D / 2) + 16 * blk);
#pragma unroll
    for (int i = 0; i < 4; ++i) w.cw[i] = x[i];
    const u4 *r = (const u4 *)((const uint16_t *)base + (int64_t)k * D + c0);
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
        const u4 y = r[i];
#pragma unroll
        for (int j = 0; j < 4; ++j) w.rw[4 * i + j] = y[j];
    }
}

// reference + (code - 8) * scale of the D/4 channels, written to an LDS row
template <int D>
__device__ inline void strided_rebuild_q(const RowQ<D> &w, int c0, float *__restrict__ dst)
{
    constexpr int CH = D / 4;
    const float sf = h2f((uint16_t)w.sc);
#pragma unroll
    for (int i = 0; i < CH; i += 4) {
        f4 o;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int ci = i + u;                                   // channel c0 + ci
            const int e = (c0 & 31) + ci;                           // its place in the block
            const int code = (int)((w.cw[(e & 15) >> 2] >> (8 * (e & 3) + 4 * (e >> 4))) & 15u);
            const uint16_t rh = (uint16_t)((ci & 1) ? (w.rw[ci >> 1] >> 16) : (w.rw[ci >> 1] & 0xFFFF));
            o[u] = __builtin_fmaf((float)(code - 8), sf, h2f(rh));   // exact product, one rounding
        }
        *(f4 *)&dst[i] = o;
    }
}

// K operands of one token for the fp16 matrix instructions: lane 16*j + n
// holds row n of A at k = 8j..8j+7, so for each block b it takes the
// reference channels 32b + 8j .. 32b + 8j + 7 (exact fp16) and the same
// channels' code bytes (8 bytes of the block, nibble plane j >> 1).
template <int D>
struct KOps {
    u4 ref[D / 32];
    u2 code[D / 32];
    uint32_t sc;                                 // scale bits of block min(j, D/32 - 1)
};

template <int D>
__device__ inline void strided_fetch_k(const uint8_t *__restrict__ base, const StridedLayout &ly, int t, int j,
                                       KOps<D> &o)
{
    constexpr int NB = D / 32;
    const int k = strided_ref(base, ly, t);
    const uint16_t *r = (const uint16_t *)base + (int64_t)k * D + 8 * j;
    const uint8_t *cb = base + ly.off_codes + (int64_t)t * (D / 2) + 8 * (j & 1);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        o.ref[b] = *(const u4 *)(r + 32 * b);
        o.code[b] = *(const u2 *)(cb + 16 * b);
    }
    o.sc = ((const uint16_t *)(base + ly.off_scales))[(int64_t)t * NB + min(j, NB - 1)];
}

// (c - 8) of 8 codes as exact fp16: 1024 + c built by placing each nibble in
// the low mantissa of 0x6400, then 1032 subtracted.
__device__ inline h8 codes_f16(u2 w, int sh)
{
    u4 o;
    const h2 off = h2{(_Float16)1032.0f, (_Float16)1032.0f};
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const uint32_t n4 = (w[i] >> sh) & 0x0F0F0F0Fu;
        const uint32_t p0 = __builtin_amdgcn_perm(0u, n4, 0x0C010C00u) | 0x64006400u;   // bytes 0, 1
        const uint32_t p1 = __builtin_amdgcn_perm(0u, n4, 0x0C030C02u) | 0x64006400u;   // bytes 2, 3
        o[2 * i] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, p0) - off);
        o[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, p1) - off);
    }
    return __builtin_bit_cast(h8, o);
}

// grid (nsplit, n_kv_heads, batch), one wave per workgroup: the split's run of
// 32-token tiles, taken as 16-token sub-tiles with no barrier between waves.
// Per sub-tile the logits are taken in the residual domain on fp16 matrix
// instructions (v_mfma_f32_16x16x32_f16: lane 16*j + n holds row n of A and
// column n of B at k = 8j..8j+7, and rows 4j..4j+3 of column n of the result):
//   q.khat_t = q.r_idx(t) + sum_b s_t,b * sum_(j in b) q_j (c_t,j - 8)
// with the reference rows (exact fp16) and the codes (c - 8, exact fp16) as A
// operands and q, scaled by 2^-E and split hi + lo, as B.  V is rebuilt in
// fp32 into the wave's LDS tile (lane: token lane/4, a quarter of the
// channels) and the weighted V rows (16 head rows x D channels over the 16
// tokens) are fp32 matrix products (v_mfma_f32_16x16x4_f32).  The softmax runs
// down each head column; head columns beyond the group are zero.  The next
// sub-tile's operands are fetched while the current one is processed.
// With positions (not null) the workgroup whose run holds a sequence's new
// token appends it first (k_new, v_new fp16 [B][Hkv][D]; the cache is written
// through the same pointer it is read through, hence no __restrict__ on it).
template <int D>
__global__ void __launch_bounds__(64)
    k_strided_attn(dkv_config cfg, const uint8_t *cache, const float *__restrict__ q,
                   const int32_t *__restrict__ lens, float scale_log2, float *__restrict__ ws, int nsplit, int chunk,
                   const uint16_t *__restrict__ knew, const uint16_t *__restrict__ vnew,
                   const int32_t *__restrict__ positions, int window)
{
    constexpr int VS = D + 16;                   // LDS row stride: conflict-free operand reads
    constexpr int NCB = D / 16;                  // 16-channel column blocks of the weighted V rows
    const StridedLayout ly = strided_layout(cfg);
    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
    const int jj = lane >> 4, nn = lane & 15;
    const int Hq = cfg.n_q_heads, G = Hq / cfg.n_kv_heads;
    if (positions) {
        const int pos = positions[b];
        if (pos >= 0 && pos < cfg.max_tokens && (pos >> 5) / chunk == split) {
            const int64_t sh = ((int64_t)b * cfg.n_kv_heads + h) * 2;
            uint8_t *wc = (uint8_t *)cache;
            const int64_t xo = ((int64_t)b * cfg.n_kv_heads + h) * D;
            strided_append_wave<D>(ly, cfg.kf, wc + sh * ly.stream_bytes, knew + xo, pos, window, lane);
            strided_append_wave<D>(ly, cfg.kf, wc + (sh + 1) * ly.stream_bytes, vnew + xo, pos, window, lane);
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        }
    }
    const int L = max(0, min(lens[b], cfg.max_tokens));
    const int t_begin = split * chunk * 32, t_end = min(L, t_begin + chunk * 32);
    const int64_t row0 = (int64_t)b * Hq + (int64_t)h * G;

    __shared__ __attribute__((aligned(16))) float vt[16 * VS];
    __shared__ float pl[kStridedMaxG][17];
    __shared__ float al[kStridedMaxG];
    __shared__ __attribute__((aligned(16))) float scl[16][4];   // the sub-tile's block scales [token][block]

    // query operand: head nn, channels 32b + 8jj + e, scaled by 2^-E (E from
    // the largest |q| of the kv-head's group) and split into hi + lo fp16
    constexpr int NB = D / 32;
    h8 qh[NB], ql[NB];
    float unq;
    {
        const float *qr = q + (row0 + min(nn, G - 1)) * D + 8 * jj;
        float qv[NB][8], qm = 0.0f;
#pragma unroll
        for (int bb = 0; bb < NB; ++bb)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = qr[32 * bb + e] * scale_log2;
                qv[bb][e] = nn < G ? x : 0.0f;
                qm = fmaxf(qm, fabsf(qv[bb][e]));
            }
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) qm = fmaxf(qm, __shfl_xor(qm, off));
        int E = 0;
        if (qm > 0.0f) frexpf(qm, &E);
        const float qsc = ldexpf(1.0f, -E);
        unq = ldexpf(1.0f, E);
#pragma unroll
        for (int bb = 0; bb < NB; ++bb)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float y = qv[bb][e] * qsc;
                const _Float16 hi = (_Float16)y;
                qh[bb][e] = hi;
                ql[bb][e] = (_Float16)(y - (float)hi);
            }
    }
    const uint8_t *kb = cache + (((int64_t)b * cfg.n_kv_heads + h) * 2) * ly.stream_bytes;
    const uint8_t *vb = kb + ly.stream_bytes;
    float m_run = -INFINITY, l_run = 0.0f;       // of head nn
    f4 acc[NCB];
#pragma unroll
    for (int u = 0; u < NCB; ++u) acc[u] = f4{0.0f, 0.0f, 0.0f, 0.0f};

    const int r = lane >> 2, c0 = (lane & 3) * (D / 4);
    const int csh = 4 * (jj >> 1);               // nibble plane of this lane's k-range
    KOps<D> ck;                                  // K operands of token t0 + nn
    RowQ<D> nv;                                  // V raw data of token t0 + r
    if (t_begin + nn < t_end) strided_fetch_k<D>(kb, ly, t_begin + nn, jj, ck);
    if (t_begin + r < t_end) strided_fetch_q<D>(vb, ly, t_begin + r, c0, nv);
    for (int t0 = t_begin; t0 < t_end; t0 += 16) {
        const int nt = min(16, t_end - t0);
        if (r < nt) {
            strided_rebuild_q<D>(nv, c0, vt + r * VS + c0);
        } else {
#pragma unroll
            for (int i = 0; i < D / 4; i += 4) *(f4 *)&vt[r * VS + c0 + i] = f4{0.0f, 0.0f, 0.0f, 0.0f};
        }
        if (jj < NB) scl[nn][jj] = nn < nt ? h2f((uint16_t)ck.sc) : 0.0f;
        // residual-domain logits of row token nn: reference part and per-block code parts
        f4 Cr = f4{0.0f, 0.0f, 0.0f, 0.0f};
        f4 Rb[NB];
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) {
            const h8 ar = __builtin_bit_cast(h8, ck.ref[bb]);
            Cr = mfma(ar, qh[bb], Cr);
            Cr = mfma(ar, ql[bb], Cr);
            const h8 ac = codes_f16(ck.code[bb], csh);
            Rb[bb] = mfma(ac, qh[bb], f4{0.0f, 0.0f, 0.0f, 0.0f});
            Rb[bb] = mfma(ac, ql[bb], Rb[bb]);
        }
        if (t0 + 16 + nn < t_end) strided_fetch_k<D>(kb, ly, t0 + 16 + nn, jj, ck);
        if (t0 + 16 + r < t_end) strided_fetch_q<D>(vb, ly, t0 + 16 + r, c0, nv);
        __syncthreads();
        float x[4], mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = 4 * jj + i;
            float lg = Cr[i];
#pragma unroll
            for (int bb = 0; bb < NB; ++bb) lg = __builtin_fmaf(scl[t][bb], Rb[bb][i], lg);
            x[i] = t < nt ? lg * unq : -INFINITY;
            mx = fmaxf(mx, x[i]);
        }
        mx = rows_max(mx);
        const float m_new = fmaxf(m_run, mx);
        const float alpha = exp2f(m_run - m_new);
        float ps = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float p = x[i] == -INFINITY ? 0.0f : exp2f(x[i] - m_new);
            pl[nn][4 * jj + i] = p;
            ps += p;
        }
        l_run = l_run * alpha + rows_sum(ps);
        m_run = m_new;
        if (jj == 0) al[nn] = alpha;
        __syncthreads();
        // weighted V rows: heads 4*jj + i, channels 16*cb + nn
        float alr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) alr[i] = al[4 * jj + i];
#pragma unroll
        for (int u = 0; u < NCB; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[u][i] *= alr[i];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const float pa = pl[nn][4 * kk + jj];
            const float *vr = vt + (4 * kk + jj) * VS + nn;
#pragma unroll
            for (int u = 0; u < NCB; ++u) acc[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(pa, vr[16 * u], acc[u], 0, 0, 0);
        }
        __syncthreads();
    }
    constexpr int R = part_stride(D);
#pragma unroll
    for (int u = 0; u < NCB; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int g = 4 * jj + i;
            if (g < G) ws[((row0 + g) * nsplit + split) * R + 16 * u + nn] = acc[u][i];
        }
    if (jj == 0 && nn < G) {
        float *rec = ws + ((row0 + nn) * nsplit + split) * R;
        rec[D] = m_run;
        rec[D + 1] = l_run;
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
        hipLaunchKernelGGL(k_strided_append<64>, grid, dim3(64), 0, st, c, (uint8_t *)cache, knew, vnew, positions,
                           window);
    else
        hipLaunchKernelGGL(k_strided_append<128>, grid, dim3(64), 0, st, c, (uint8_t *)cache, knew, vnew, positions,
                           window);
    return hipGetLastError();
}

// knew/vnew/positions null: decode only.
hipError_t launch_strided_attn(const dkv_config &c, const void *cache, const float *q, const int32_t *lens,
                               float scale_log2, float *ws, int nsplit, int chunk, const uint16_t *knew,
                               const uint16_t *vnew, const int32_t *positions, int window, hipStream_t st)
{
    dim3 grid(nsplit, c.n_kv_heads, c.batch);
    if (c.head_dim == 64)
        hipLaunchKernelGGL(k_strided_attn<64>, grid, dim3(64), 0, st, c, (const uint8_t *)cache, q, lens,
                           scale_log2, ws, nsplit, chunk, knew, vnew, positions, window);
    else
        hipLaunchKernelGGL(k_strided_attn<128>, grid, dim3(64), 0, st, c, (const uint8_t *)cache, q, lens,
                           scale_log2, ws, nsplit, chunk, knew, vnew, positions, window);
    return hipGetLastError();
}

}  // namespace dkv
