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

// Buffer resource over one stream (its planes are addressed with 32-bit
// offsets; loads past the stream return zeros).
__device__ inline __amdgpu_buffer_rsrc_t stream_rsrc(const uint8_t *base, int64_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, (int)bytes, 0x00020000);
}
// The token's reference index, clamped to the plane, through the stream's resource.
__device__ inline int strided_ref_rs(__amdgpu_buffer_rsrc_t rs, const StridedLayout &ly, int t)
{
    return min((int)(uint16_t)__builtin_amdgcn_raw_buffer_load_b16(rs, (int)ly.off_idx + 2 * t, 0, kStream),
               ly.nref - 1);
}

// K operands of token t with reference index k (loaded ahead: the row load
// does not wait for the index load).
template <int D>
__device__ inline void strided_fetch_k(__amdgpu_buffer_rsrc_t rs, const StridedLayout &ly, int t, int k, int j,
                                       KOps<D> &o)
{
    constexpr int NB = D / 32;
    const int ro = k * (2 * D) + 16 * j;
    const int co = (int)ly.off_codes + t * (D / 2) + 8 * (j & 1);
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        o.ref[b] = __builtin_amdgcn_raw_buffer_load_b128(rs, ro + 64 * b, 0, 0);
        o.code[b] = __builtin_amdgcn_raw_buffer_load_b64(rs, co + 16 * b, 0, kStream);
    }
    o.sc = (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(rs, (int)ly.off_scales + (t * NB + min(j, NB - 1)) * 2, 0,
                                                          kStream);
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
        // bytes 0, 1 (2, 3) of n4 under a 0x64 byte each
        const uint32_t p0 = __builtin_amdgcn_perm(0x64646464u, n4, 0x04010400u);
        const uint32_t p1 = __builtin_amdgcn_perm(0x64646464u, n4, 0x04030402u);
        o[2 * i] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, p0) - off);
        o[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, p1) - off);
    }
    return __builtin_bit_cast(h8, o);
}

// fp16 (c - 8) of the 8 codes in word w (byte i: code i of the block in the
// low nibble, code i + 16 in the high one) for 4 channels of each nibble
// plane: lo[0..1] = channels i..i+3 (low nibbles), hi[0..1] = i+16..i+19.
// 0x64 above a nibble is the fp16 1024 + c; 1032 is subtracted exactly.
__device__ inline void codes_pairs(uint32_t w, uint32_t (&lo)[2], uint32_t (&hi)[2])
{
    const h2 off = h2{(_Float16)1032.0f, (_Float16)1032.0f};
    const uint32_t nl = w & 0x0F0F0F0Fu, nh = (w >> 4) & 0x0F0F0F0Fu;
    const uint32_t p64 = 0x64646464u;
    const uint32_t l0 = __builtin_amdgcn_perm(p64, nl, 0x04010400u), l1 = __builtin_amdgcn_perm(p64, nl, 0x04030402u);
    const uint32_t h0 = __builtin_amdgcn_perm(p64, nh, 0x04010400u), h1 = __builtin_amdgcn_perm(p64, nh, 0x04030402u);
    lo[0] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, l0) - off);
    lo[1] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, l1) - off);
    hi[0] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, h0) - off);
    hi[1] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, h1) - off);
}

// V data of one token for one lane: half h of its channels, the reference
// row's slice (fp16), the code bytes of the same channels and their scales.
template <int D>
struct VHalf {
    u4 ref[D / 16];                 // D/2 channels: D bytes
    uint32_t code[D / 16];          // D/4 bytes of codes (D/2 channels)
    uint32_t sc;                    // scales of the half's blocks (D = 128: 2, D = 64: 1)
};

// fp16 transpose read (ds_read_b64_tr_b16): in each group of 16 lanes, lane L
// returns element L % 4 of the 8-byte pieces addressed by lanes L/4, L/4 + 4,
// L/4 + 8 and L/4 + 12 of its group.
__device__ inline u2 lds_tr16(const uint8_t *p)
{
    typedef short v4s __attribute__((ext_vector_type(4)));
    const v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4s *)(__attribute__((address_space(3))) uint8_t *)p);
    return __builtin_bit_cast(u2, r);
}

// grid (nsplit, n_kv_heads, batch), one wave per workgroup: the split's run of
// 32-token tiles.  Per tile:
//  - logits in the residual domain on fp16 matrix instructions
//    (v_mfma_f32_16x16x32_f16: lane 16*j + n holds row n of A and column n
//    of B at k = 8j..8j+7, and rows 4j..4j+3 of column n of the result):
//      q.khat_t = q.r_idx(t) + sum_b s_t,b * sum_(i in b) q_i (c_t,i - 8)
//    with the reference rows and the codes (c - 8) as exact fp16 A operands
//    (rows: tokens) and q, scaled by 2^-E and split hi + lo, as B;
//  - the online softmax down each head column (head columns past the group
//    have a zero query);
//  - the weighted V rows in the residual domain on the same instructions:
//      sum_t p_t vhat_t = sum_t p_t r_idx(t) + sum_b sum_t (p_t s_t,b)(c_t - 8)
//    The tile's reference rows and its codes (c - 8, exact fp16) are written
//    to LDS as token rows and read back transposed (ds_read_b64_tr_b16), so
//    A holds 16 channels x 32 tokens; B holds the weights p (for the
//    reference rows) and p * s_b (for the codes of block b), split hi + lo.
//    V is never rebuilt.
//  The next tile's operands are fetched while the current one is processed.
// PAIR (at most 8 query heads per kv-head): the 8 spare columns of B carry the
// same heads again, and the A rows of each instruction are 8 channels of a
// block b (rows 0..7) and 8 of block b + nb/2 (rows 8..15), so column half h
// takes the code weights of one block of each pair (half the weight work per
// lane); only the (row half, column half) pairs that match are kept.
// With positions (not null) the workgroup whose run holds a sequence's new
// token appends it first (k_new, v_new fp16 [B][Hkv][D]; the cache is written
// through the same pointer it is read through, hence no __restrict__ on it).
template <int D, bool PAIR>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2)))
    k_strided_attn(dkv_config cfg, const uint8_t *cache, const float *__restrict__ q,
                   const int32_t *__restrict__ lens, float scale_log2, float *__restrict__ ws, int nsplit, int chunk,
                   const uint16_t *__restrict__ knew, const uint16_t *__restrict__ vnew,
                   const int32_t *__restrict__ positions, int window)
{
    constexpr int NB = D / 32, NCB = D / 16;
    constexpr int VS = 4 * D + 32;               // LDS bytes per V token row: [reference 2D][codes 2D][pad]
    constexpr int PS = 36;                       // floats per weight row
    const StridedLayout ly = strided_layout(cfg);
    const int split = grid_split(), h = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
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

    // per token of the tile: its reference row and its codes as fp16 (c - 8);
    // the 32-byte pad puts the 4 rows of a transposed read on separate banks
    __shared__ __attribute__((aligned(16))) uint8_t vdat[32 * VS];
    __shared__ __attribute__((aligned(16))) float pl[kStridedMaxG * PS]; // p [head][token]
    __shared__ __attribute__((aligned(16))) uint16_t vsh[32 * NB];    // V scales (fp16) [token][block]
    __shared__ float ksl[32][NB];                                     // K scales [token][block]

    // query operand: head nn, channels 32b + 8jj + e, scaled by 2^-E (E from
    // the largest |q| of the kv-head's group) and split into hi + lo fp16
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
    const __amdgpu_buffer_rsrc_t krs = stream_rsrc(kb, ly.stream_bytes), vrs = stream_rsrc(vb, ly.stream_bytes);
    float m_run = -INFINITY, l_run = 0.0f;       // of head nn
    f4 acc[NCB];
#pragma unroll
    for (int u = 0; u < NCB; ++u) acc[u] = f4{0.0f, 0.0f, 0.0f, 0.0f};

    // V fetch: lane = token vt (of the tile) and half vh of the channels
    const int vt = lane >> 1, vh = lane & 1;
    const int csh = 4 * (jj >> 1);               // K: nibble plane of this lane's k-range
    // reference indices are loaded a tile before the rows they select
    auto kidx = [&](int t) { return strided_ref_rs(krs, ly, t < t_end ? t : t_begin); };
    auto vidx = [&](int t) { return strided_ref_rs(vrs, ly, t < t_end ? t : t_begin); };
    auto fetch_v_rest = [&](int t, VHalf<D> &v) {
        const int tc = t < t_end ? t : t_begin;  // past the end: a valid row (its weight is zero)
        const int co = (int)ly.off_codes + tc * (D / 2) + vh * (D / 4);
#pragma unroll
        for (int i = 0; i < D / 64; ++i) {
            const u4 x = __builtin_amdgcn_raw_buffer_load_b128(vrs, co + 16 * i, 0, kStream);
#pragma unroll
            for (int e = 0; e < 4; ++e) v.code[4 * i + e] = x[e];
        }
        if constexpr (NB == 4)
            v.sc = __builtin_amdgcn_raw_buffer_load_b32(vrs, (int)ly.off_scales + tc * 8 + 4 * vh, 0, kStream);
        else
            v.sc = (uint16_t)__builtin_amdgcn_raw_buffer_load_b16(vrs, (int)ly.off_scales + tc * 4 + 2 * vh, 0,
                                                                  kStream);
    };
    auto fetch_v_ref = [&](int k, VHalf<D> &v) {
        const int ro = k * (2 * D) + vh * D;
#pragma unroll
        for (int i = 0; i < D / 16; ++i) v.ref[i] = __builtin_amdgcn_raw_buffer_load_b128(vrs, ro + 16 * i, 0, 0);
    };
    // K operands of token t (row nn of the tile's half T) with its reference
    // index k; tokens past the end read token t_begin (their logits are masked)
    auto fetch_k = [&](int t, int k, KOps<D> &o) { strided_fetch_k<D>(krs, ly, t < t_end ? t : t_begin, k, jj, o); };

    KOps<D> ck[2];
    VHalf<D> cv;
    int ki0 = 0, ki1 = 0, vi = 0;             // reference indices of the next tile's tokens
    if (t_begin < t_end) {
        fetch_k(t_begin + nn, kidx(t_begin + nn), ck[0]);
        fetch_k(t_begin + 16 + nn, kidx(t_begin + 16 + nn), ck[1]);
        fetch_v_rest(t_begin + vt, cv);
        fetch_v_ref(vidx(t_begin + vt), cv);
        ki0 = kidx(t_begin + 32 + nn);
        ki1 = kidx(t_begin + 48 + nn);
        vi = vidx(t_begin + 32 + vt);
    }
    for (int t0 = t_begin; t0 < t_end; t0 += 32) {
        const int nt = min(32, t_end - t0);
        // stage the tile's V rows (reference slice and codes as fp16 (c - 8)),
        // its V scales and its K scales
        {
            uint8_t *rr = vdat + vt * VS + vh * D;
            uint8_t *cr = rr + 2 * D;
#pragma unroll
            for (int i = 0; i < D / 16; ++i) ((u4 *)rr)[i] = cv.ref[i];
            // code words: D/64 blocks per half, 4 words (16 bytes) each
#pragma unroll
            for (int bl = 0; bl < D / 64; ++bl) {
                uint32_t lo[8], hi[8];
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    uint32_t l2[2], h2_[2];
                    codes_pairs(cv.code[4 * bl + w], l2, h2_);
                    lo[2 * w] = l2[0];
                    lo[2 * w + 1] = l2[1];
                    hi[2 * w] = h2_[0];
                    hi[2 * w + 1] = h2_[1];
                }
                u4 *dst = (u4 *)(cr + 64 * bl);           // block: channels 0..15 (low nibbles), 16..31 (high)
                dst[0] = u4{lo[0], lo[1], lo[2], lo[3]};
                dst[1] = u4{lo[4], lo[5], lo[6], lo[7]};
                dst[2] = u4{hi[0], hi[1], hi[2], hi[3]};
                dst[3] = u4{hi[4], hi[5], hi[6], hi[7]};
            }
            if constexpr (NB == 4)
                ((uint32_t *)vsh)[vt * 2 + vh] = cv.sc;
            else
                vsh[vt * 2 + vh] = (uint16_t)cv.sc;
            if (nt < 32 && vt >= nt) {
                // rows past the end (re-reads of a valid token) become zeros:
                // their weights are zero, and zero rows keep 0 * inf out
#pragma unroll
                for (int i = 0; i < D / 16; ++i) ((u4 *)rr)[i] = u4{0, 0, 0, 0};
#pragma unroll
                for (int i = 0; i < D / 16; ++i) ((u4 *)cr)[i] = u4{0, 0, 0, 0};
                if constexpr (NB == 4)
                    ((uint32_t *)vsh)[vt * 2 + vh] = 0u;
                else
                    vsh[vt * 2 + vh] = (uint16_t)0;
            }
            if (jj < NB) {
                ksl[nn][jj] = h2f((uint16_t)ck[0].sc);
                ksl[16 + nn][jj] = h2f((uint16_t)ck[1].sc);
            }
        }
        // K side: both halves of the tile from the registers fetched last tile
        f4 Cr[2], Rb[2][NB];
#pragma unroll
        for (int T = 0; T < 2; ++T) {
            Cr[T] = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int bb = 0; bb < NB; ++bb) {
                const h8 ar = __builtin_bit_cast(h8, ck[T].ref[bb]);
                Cr[T] = mfma(ar, qh[bb], Cr[T]);
                Cr[T] = mfma(ar, ql[bb], Cr[T]);
                const h8 ac = codes_f16(ck[T].code[bb], csh);
                Rb[T][bb] = mfma(ac, qh[bb], f4{0.0f, 0.0f, 0.0f, 0.0f});
                Rb[T][bb] = mfma(ac, ql[bb], Rb[T][bb]);
            }
        }
        // fetch the next tile (the reference rows once their indices are in)
        const int t1 = t0 + 32;
        VHalf<D> nv;
        if (t1 < t_end) {
            fetch_k(t1 + nn, ki0, ck[0]);
            fetch_k(t1 + 16 + nn, ki1, ck[1]);
            fetch_v_rest(t1 + vt, nv);
            fetch_v_ref(vi, nv);
            ki0 = kidx(t1 + 32 + nn);
            ki1 = kidx(t1 + 48 + nn);
            vi = vidx(t1 + 32 + vt);
        }
        __syncthreads();
        // logits of tokens 16T + 4jj + i, the tile maximum, softmax weights
        float x[2][4], mx = -INFINITY;
#pragma unroll
        for (int T = 0; T < 2; ++T)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * T + 4 * jj + i;
                float lg = Cr[T][i];
#pragma unroll
                for (int bb = 0; bb < NB; ++bb) lg = __builtin_fmaf(ksl[t][bb], Rb[T][bb][i], lg);
                x[T][i] = t < nt ? lg * unq : -INFINITY;
                mx = fmaxf(mx, x[T][i]);
            }
        mx = rows_max(mx);
        const float m_new = fmaxf(m_run, mx);
        if (__any(m_new != m_run)) {
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            // PAIR: the accumulators of column half 1 hold head nn - 8, whose
            // softmax state is in lane nn - 8 of the row
            // (every lane takes part in the exchange: the empty asm keeps the
            // compiler from moving it under the lane condition, where the
            // lanes it reads would be switched off)
            float ao = other_half(alpha);
            asm volatile("" : "+v"(ao));
            const float av = (PAIR && (nn >> 3)) ? ao : alpha;
#pragma unroll
            for (int u = 0; u < NCB; ++u) acc[u] *= av;
            l_run *= alpha;
        }
        m_run = m_new;
        float ps = 0.0f;
#pragma unroll
        for (int T = 0; T < 2; ++T) {
            f4 pv;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p = __builtin_amdgcn_exp2f(x[T][i] - m_new);     // exp2(-inf) = 0
                pv[i] = p;
                ps += p;
            }
            *(f4 *)&pl[nn * PS + 16 * T + 4 * jj] = pv;
        }
        l_run += rows_sum(ps);
        __syncthreads();
        // weights of head hq for tokens 8jj..8jj+7: p (reference rows) and
        // p * s_b (codes of block b), each split hi + lo, token pairs per word;
        // PAIR: block wb + (nb/2)*h2 of each pair wb
        constexpr int NWB = PAIR ? NB / 2 : NB;
        const int h2 = nn >> 3, hq = PAIR ? (nn & 7) : nn;
        uint32_t wph[4], wpl[4], wsh[NWB][4], wsl[NWB][4];
        {
            const f4 p0 = *(const f4 *)&pl[hq * PS + 8 * jj], p1 = *(const f4 *)&pl[hq * PS + 8 * jj + 4];
            const float p[8] = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
            const uint32_t *sw = (const uint32_t *)vsh + 8 * jj * (NB / 2);
            constexpr uint32_t kOne = 0x3C003C00u;               // fp16 1.0 in both halves
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
                split_w<0>(kOne, kOne, p[2 * e2], p[2 * e2 + 1], wph[e2], wpl[e2]);
#pragma unroll
                for (int wb = 0; wb < NWB; ++wb) {
                    // block bb's scale: half bb & 1 of word bb >> 1 of the token's scales
                    const int bb = PAIR ? wb + (NB / 2) * h2 : wb;
                    uint32_t s0 = sw[(2 * e2) * (NB / 2) + (bb >> 1)], s1 = sw[(2 * e2 + 1) * (NB / 2) + (bb >> 1)];
                    if constexpr (PAIR && NB == 2) {          // bb = h2: a lane-dependent half
                        s0 = h2 ? s0 >> 16 : s0;
                        s1 = h2 ? s1 >> 16 : s1;
                        split_w<0>(s0, s1, p[2 * e2], p[2 * e2 + 1], wsh[wb][e2], wsl[wb][e2]);
                    } else if (wb & 1) {
                        split_w<1>(s0, s1, p[2 * e2], p[2 * e2 + 1], wsh[wb][e2], wsl[wb][e2]);
                    } else {
                        split_w<0>(s0, s1, p[2 * e2], p[2 * e2 + 1], wsh[wb][e2], wsl[wb][e2]);
                    }
                }
            }
        }
        // transposed reads: lane L of group jj gets the channel of row L of
        // tokens 8jj..8jj+3, then 8jj+4..8jj+7; lane L addresses token
        // 8jj + L/4 and the 4 channels its row quarter L % 4 takes:
        //  plain: rows = channels 16cb .. 16cb + 15;
        //  PAIR:  rows 0..7 = channels 8g .. 8g+7 of block wb, rows 8..15 those of block wb + nb/2
        const int rrow = (8 * jj + (nn >> 2)) * VS;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            const int ch = PAIR ? 32 * ((cb >> 2) + (NB / 2) * ((nn & 3) >> 1)) + 8 * (cb & 3) + 4 * (nn & 1)
                                : 16 * cb + 4 * (nn & 3);
            const uint8_t *pr = vdat + rrow + 2 * ch;
            const u2 r0 = lds_tr16(pr), r1 = lds_tr16(pr + 4 * VS);
            const u2 c0 = lds_tr16(pr + 2 * D), c1 = lds_tr16(pr + 2 * D + 4 * VS);
            const h8 ar = __builtin_bit_cast(h8, u4{r0[0], r0[1], r1[0], r1[1]});
            const h8 ac = __builtin_bit_cast(h8, u4{c0[0], c0[1], c1[0], c1[1]});
            const int wb = PAIR ? cb >> 2 : cb >> 1;
            acc[cb] = mfma(ar, as_h8(u4{wph[0], wph[1], wph[2], wph[3]}), acc[cb]);
            acc[cb] = mfma(ar, as_h8(u4{wpl[0], wpl[1], wpl[2], wpl[3]}), acc[cb]);
            acc[cb] = mfma(ac, as_h8(u4{wsh[wb][0], wsh[wb][1], wsh[wb][2], wsh[wb][3]}), acc[cb]);
            acc[cb] = mfma(ac, as_h8(u4{wsl[wb][0], wsl[wb][1], wsl[wb][2], wsl[wb][3]}), acc[cb]);
        }
        cv = nv;
        __syncthreads();
    }
    // plain: lane (jj, nn) holds channels 16cb + 4jj + i of head nn; PAIR:
    // lanes with (jj >> 1) == (nn >> 3) hold channels 8g + 4(jj & 1) + i of
    // block cb/4 + (nb/2)(nn >> 3) (cb = 4 * pair + g) of head nn & 7
    constexpr int R = part_stride(D);
    const int hq = PAIR ? (nn & 7) : nn;
    if (hq < G && (!PAIR || (jj >> 1) == (nn >> 3))) {
        float *rec = ws + ((row0 + hq) * nsplit + split) * R;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            const int ch = PAIR ? 32 * ((cb >> 2) + (NB / 2) * (nn >> 3)) + 8 * (cb & 3) + 4 * (jj & 1) : 16 * cb + 4 * jj;
            *(f4 *)&rec[ch] = acc[cb];
        }
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
    const bool pair = c.n_q_heads / c.n_kv_heads <= 8;
    if (c.head_dim == 64) {
        if (pair)
            hipLaunchKernelGGL((k_strided_attn<64, true>), grid, dim3(64), 0, st, c, (const uint8_t *)cache, q, lens,
                               scale_log2, ws, nsplit, chunk, knew, vnew, positions, window);
        else
            hipLaunchKernelGGL((k_strided_attn<64, false>), grid, dim3(64), 0, st, c, (const uint8_t *)cache, q, lens,
                               scale_log2, ws, nsplit, chunk, knew, vnew, positions, window);
    } else {
        if (pair)
            hipLaunchKernelGGL((k_strided_attn<128, true>), grid, dim3(64), 0, st, c, (const uint8_t *)cache, q, lens,
                               scale_log2, ws, nsplit, chunk, knew, vnew, positions, window);
        else
            hipLaunchKernelGGL((k_strided_attn<128, false>), grid, dim3(64), 0, st, c, (const uint8_t *)cache, q,
                               lens, scale_log2, ws, nsplit, chunk, knew, vnew, positions, window);
    }
    return hipGetLastError();
}

}  // namespace dkv
