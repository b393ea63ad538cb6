// Delta-KV encoder (bulk prefill and per-step append), decoder export and
// canonical export kernels for gfx950.
//
// The codec follows the Delta-KV article (jeff.news, "핵심 아이디어"): an fp16
// keyframe opens every group of kf tokens; each later token stores the
// difference to the previous *reconstructed* token (closed loop), quantised as
// 32-channel Q4_0 blocks.  One wavefront owns one stream (sequence, kv-head,
// K or V) of one group and walks its tokens in order; lanes own channels
// (lane l holds channels l and l+64 when D = 128), so a 32-lane half-wave is
// exactly one Q4_0 block and the block's max-magnitude search is a 5-step
// butterfly inside the half-wave.
//
// Arithmetic is written with explicitly rounded fp32 operations so that the
// result is bit-identical to a plain sequential fp32 implementation of the
// same steps (the library is also built with -ffp-contract=off):
//   d      = x - xhat
//   m      = d of largest |d| (lowest channel wins ties; +0 if all zero)
//   s      = m * -1/8,  id = s != 0 ? 1/s (correctly rounded) : 0
//   code   = min(15, trunc((d*id) + 8.5))
//   scale  = fp16(s) round-to-nearest-even
//   xhat  += (code-8) * float(scale)     (exact product, one rounding)
#include "dkv_append.h"

namespace dkv {

// ------------------------------------------------------------------------
// Bulk prefill: grid (groups, Hkv*2, B), one wavefront per (b, h, stream, group).
// ------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(64) k_encode_prefill(dkv_config cfg, uint8_t *cache, float *state,
                                                       const int32_t *bt, const uint16_t *kin,
                                                       const uint16_t *vin, const int32_t *seq_lens,
                                                       int s_max)
{
    constexpr int NC = D / 64;
    constexpr int nb = D / 32;
    const Geom g = make_geom(cfg);
    const int gi = blockIdx.x, h = blockIdx.y >> 1, s = blockIdx.y & 1, b = blockIdx.z;
    const int L = min(min(seq_lens[b], g.cap_tokens), s_max);
    const int t0 = gi * g.kf;
    if (t0 >= L) return;
    const int n = min(g.kf, L - t0);
    const int64_t off = group_offset(g, bt, b, h, gi);
    if (off < 0) return;
    StreamPtrs p = stream_ptrs(g, cache + off, s);
    const uint16_t *x = (s ? vin : kin) + (((int64_t)b * g.Hkv + h) * s_max + t0) * D;
    const int lane = threadIdx.x;

    float xh[NC];
    uint32_t vw[NC][4];
    uint16_t smax[NC];
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        smax[i] = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) vw[i][j] = 0x88888888u;
    }

    uint16_t xv[NC];
#pragma unroll
    for (int i = 0; i < NC; ++i) xv[i] = x[lane + 64 * i];

    for (int r = 0; r < n; ++r) {
        uint16_t xn[NC];
        if (r + 1 < n) {
#pragma unroll
            for (int i = 0; i < NC; ++i) xn[i] = x[(int64_t)(r + 1) * D + lane + 64 * i];
        }
        if (r == 0) {
#pragma unroll
            for (int i = 0; i < NC; ++i) {
                const int c = lane + 64 * i;
                ((uint16_t *)p.kf)[s ? vkf_pos(D, c, g.vbp) : kkf_pos(nb, c)] = xv[i];
                xh[i] = h2f(xv[i]);
            }
        } else {
            const int tau = r & 31;
#pragma unroll
            for (int i = 0; i < NC; ++i) {
                const int c = lane + 64 * i;
                const int blk = c >> 5;
                int code;
                uint16_t s16;
                q40_delta_step(h2f(xv[i]), xh[i], code, s16);
                if ((lane & 31) == 0) p.sc[r * nb + blk] = s16;
                smax[i] = (uint16_t)max((int)smax[i], (int)habs_bits(s16));
                if (s == 0) {
                    store_k_codes<D>(p.cd + (int64_t)(r - 1) * (D / 2), blk, code);
                } else {
                    const int j = (tau & 15) >> 2, sh = 4 * vcode_nibble(tau);
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj)
                        if (jj == j) vw[i][jj] = (vw[i][jj] & ~(0xFu << sh)) | ((uint32_t)code << sh);
                }
            }
        }
        // V: flush a finished tile of code words (a tile holding only the
        // keyframe slot has no codes; with kf == 1 there is no code plane)
        if (s == 1 && r > 0 && ((r & 31) == 31 || r == n - 1)) {
            uint32_t *tw = (uint32_t *)(p.cd + (int64_t)(r >> 5) * 16 * D);
#pragma unroll
            for (int i = 0; i < NC; ++i) {
                const int c = lane + 64 * i;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    tw[vcode_word(D, 4 * j, c, g.vbp)] = vw[i][j];
                    vw[i][j] = 0x88888888u;
                }
            }
        }
#pragma unroll
        for (int i = 0; i < NC; ++i) xv[i] = xn[i];
    }
    // slot 0 of the scale plane: largest |scale| per block over the group
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        const int c = lane + 64 * i;
        uint16_t mx = smax[i];
#pragma unroll
        for (int off2 = 16; off2 >= 1; off2 >>= 1) mx = (uint16_t)max((int)mx, __shfl_xor((int)mx, off2, 32));
        if ((lane & 31) == 0) p.sc[c >> 5] = mx;
    }
    if (t0 + n == L) {
        float *st = state + (((int64_t)b * g.Hkv + h) * 2 + s) * D;
#pragma unroll
        for (int i = 0; i < NC; ++i) st[lane + 64 * i] = xh[i];
    }
}

// ------------------------------------------------------------------------
// Append one token per sequence: grid (1, Hkv*2, B).
// ------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(64) k_append(dkv_config cfg, uint8_t *cache, float *state,
                                               const int32_t *bt, const uint16_t *knew,
                                               const uint16_t *vnew, const int32_t *positions)
{
    const Geom g = make_geom(cfg);
    const int h = blockIdx.y >> 1, s = blockIdx.y & 1, b = blockIdx.z;
    append_token_stream<D>(g, cache, state, bt, knew, vnew, positions[b], b, h, s, threadIdx.x);
}

// ------------------------------------------------------------------------
// Code / scale readers shared by the decoder kernels.
// ------------------------------------------------------------------------
template <int D>
__device__ inline int read_code(const StreamPtrs &p, int s, int r, int c, int bp)
{
    if (s == 0) {
        const int cb = c & 31;
        const uint8_t byte = p.cd[(int64_t)(r - 1) * (D / 2) + kcode_byte(D / 32, c >> 5, cb & 15)];
        return (byte >> (4 * (cb >> 4))) & 15;
    }
    const int tau = r & 31;
    const uint32_t w = ((const uint32_t *)(p.cd + (int64_t)(r >> 5) * 16 * D))[vcode_word(D, tau, c, bp)];
    return (w >> (4 * vcode_nibble(tau))) & 15;
}

// Dense fp32 reconstruction: grid (groups, Hkv*2, B).
template <int D>
__global__ void __launch_bounds__(64) k_reconstruct(dkv_config cfg, const uint8_t *cache,
                                                    const int32_t *bt, const int32_t *seq_lens,
                                                    int s_max, float *kout, float *vout)
{
    constexpr int NC = D / 64;
    constexpr int nb = D / 32;
    const Geom g = make_geom(cfg);
    const int gi = blockIdx.x, h = blockIdx.y >> 1, s = blockIdx.y & 1, b = blockIdx.z;
    const int L = min(min(seq_lens[b], g.cap_tokens), s_max);
    const int t0 = gi * g.kf;
    if (t0 >= L) return;
    const int n = min(g.kf, L - t0);
    const int64_t off = group_offset(g, bt, b, h, gi);
    if (off < 0) return;
    StreamPtrs p = stream_ptrs(g, (uint8_t *)cache + off, s);
    float *o = (s ? vout : kout) + (((int64_t)b * g.Hkv + h) * s_max + t0) * D;
    const int lane = threadIdx.x;
    float xh[NC];
    for (int r = 0; r < n; ++r) {
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            const int c = lane + 64 * i;
            if (r == 0) {
                xh[i] = h2f(((const uint16_t *)p.kf)[s ? vkf_pos(D, c, g.vbp) : kkf_pos(nb, c)]);
            } else {
                const int code = read_code<D>(p, s, r, c, g.vbp);
                const float sf = h2f(p.sc[r * nb + (c >> 5)]);
                xh[i] = __fadd_rn(xh[i], __fmul_rn((float)(code - 8), sf));
            }
            o[(int64_t)r * D + c] = xh[i];
        }
    }
}

// Canonical export: grid (groups, Hkv*2, B).
template <int D>
__global__ void __launch_bounds__(64) k_export(dkv_config cfg, const uint8_t *cache, const int32_t *bt,
                                               const int32_t *seq_lens, int s_max, uint16_t *okf,
                                               uint8_t *ocd, uint16_t *osc)
{
    constexpr int NC = D / 64;
    constexpr int nb = D / 32;
    const Geom g = make_geom(cfg);
    const int gi = blockIdx.x, h = blockIdx.y >> 1, s = blockIdx.y & 1, b = blockIdx.z;
    const int L = min(min(seq_lens[b], g.cap_tokens), s_max);
    const int t0 = gi * g.kf;
    if (t0 >= L) return;
    const int n = min(g.kf, L - t0);
    const int64_t off = group_offset(g, bt, b, h, gi);
    if (off < 0) return;
    StreamPtrs p = stream_ptrs(g, (uint8_t *)cache + off, s);
    const int ng = (s_max + g.kf - 1) / g.kf, nd = s_max - ng;
    const int64_t sidx = ((int64_t)b * g.Hkv + h) * 2 + s;
    const int lane = threadIdx.x;
    for (int r = 0; r < n; ++r) {
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            const int c = lane + 64 * i;
            if (r == 0) {
                okf[(sidx * ng + gi) * D + c] = ((const uint16_t *)p.kf)[s ? vkf_pos(D, c, g.vbp) : kkf_pos(nb, c)];
            } else {
                const int64_t di = (int64_t)gi * (g.kf - 1) + r - 1;
                const int code = read_code<D>(p, s, r, c, g.vbp);
                const int hi = __shfl_down(code, 16, 32);
                const int sl = lane & 31;
                if (sl < 16) ocd[(sidx * nd + di) * (D / 2) + (c >> 5) * 16 + sl] = (uint8_t)(code | (hi << 4));
                if (sl == 0) osc[(sidx * nd + di) * nb + (c >> 5)] = p.sc[r * nb + (c >> 5)];
            }
        }
    }
}

// ------------------------------------------------------------------------
// Host launchers
// ------------------------------------------------------------------------
#define DKV_DISPATCH_D(D_, ...)                       \
    do {                                              \
        if ((D_) == 64) {                             \
            constexpr int DD = 64;                    \
            __VA_ARGS__;                              \
        } else {                                      \
            constexpr int DD = 128;                   \
            __VA_ARGS__;                              \
        }                                             \
    } while (0)

hipError_t launch_encode_prefill(const dkv_config &c, void *cache, float *state, const int32_t *bt,
                                 const uint16_t *k, const uint16_t *v, const int32_t *lens, int s_max,
                                 hipStream_t st)
{
    const int ng = (min(s_max, make_geom(c).cap_tokens) + c.kf - 1) / c.kf;
    if (ng == 0) return hipSuccess;
    dim3 grid(ng, c.n_kv_heads * 2, c.batch);
    DKV_DISPATCH_D(c.head_dim, hipLaunchKernelGGL(k_encode_prefill<DD>, grid, dim3(64), 0, st, c,
                                                  (uint8_t *)cache, state, bt, k, v, lens, s_max));
    return hipGetLastError();
}

hipError_t launch_append(const dkv_config &c, void *cache, float *state, const int32_t *bt,
                         const uint16_t *k, const uint16_t *v, const int32_t *pos, hipStream_t st)
{
    dim3 grid(1, c.n_kv_heads * 2, c.batch);
    DKV_DISPATCH_D(c.head_dim, hipLaunchKernelGGL(k_append<DD>, grid, dim3(64), 0, st, c,
                                                  (uint8_t *)cache, state, bt, k, v, pos));
    return hipGetLastError();
}

hipError_t launch_reconstruct(const dkv_config &c, const void *cache, const int32_t *bt,
                              const int32_t *lens, int s_max, float *ko, float *vo, hipStream_t st)
{
    const int ng = (s_max + c.kf - 1) / c.kf;
    if (ng == 0) return hipSuccess;
    dim3 grid(ng, c.n_kv_heads * 2, c.batch);
    DKV_DISPATCH_D(c.head_dim, hipLaunchKernelGGL(k_reconstruct<DD>, grid, dim3(64), 0, st, c,
                                                  (const uint8_t *)cache, bt, lens, s_max, ko, vo));
    return hipGetLastError();
}

hipError_t launch_export(const dkv_config &c, const void *cache, const int32_t *bt, const int32_t *lens,
                         int s_max, uint16_t *okf, uint8_t *ocd, uint16_t *osc, hipStream_t st)
{
    const int ng = (s_max + c.kf - 1) / c.kf;
    if (ng == 0) return hipSuccess;
    dim3 grid(ng, c.n_kv_heads * 2, c.batch);
    DKV_DISPATCH_D(c.head_dim, hipLaunchKernelGGL(k_export<DD>, grid, dim3(64), 0, st, c,
                                                  (const uint8_t *)cache, bt, lens, s_max, okf, ocd, osc));
    return hipGetLastError();
}

}  // namespace dkv
