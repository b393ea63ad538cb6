// Appending one token to a stream of the Delta-KV cache (Delta-KV article,
// "핵심 아이디어": a keyframe every kf tokens, in between the 4-bit code of the
// closed-loop delta against the running reconstruction).  Shared by the append
// kernel and the decode kernel that appends the new token of each sequence
// before it attends over it, so both write the same bytes.
#pragma once
#include "dkv_q40.h"

namespace dkv {

struct StreamPtrs {
    uint8_t *kf;     // keyframe (fp16, permuted)
    uint16_t *sc;    // scales [kf][nb]
    uint8_t *cd;     // codes
};

__device__ inline StreamPtrs stream_ptrs(const Geom &g, uint8_t *rec, int s)
{
    StreamPtrs p;
    p.kf = rec + (s ? g.off_vkf : 0);
    p.sc = (uint16_t *)(rec + (s ? g.off_vsc : g.off_ksc));
    p.cd = rec + (s ? g.off_vcd : g.off_kcd);
    return p;
}

// One wavefront (64 lanes, lane = channel mod 64) appends token `pos` of
// stream s (0 = K, 1 = V) of (sequence b, kv-head h): at pos % kf == 0 the fp16
// row becomes the group's keyframe and the reconstruction; otherwise the delta
// against the reconstruction is quantised block by block (32-lane halves), its
// codes and scale are stored, the group's max-|scale| slot is raised and the
// reconstruction advances.  A position past the capacity or in an unmapped
// page writes nothing.
template <int D>
__device__ inline void append_token_stream(const Geom &g, uint8_t *cache, float *state, const int32_t *bt,
                                           const uint16_t *knew, const uint16_t *vnew, int pos, int b, int h,
                                           int s, int lane)
{
    constexpr int NC = D / 64;
    constexpr int nb = D / 32;
    if (pos < 0 || pos >= g.cap_tokens) return;
    const int gi = pos / g.kf, r = pos % g.kf;
    const int64_t off = group_offset(g, bt, b, h, gi);
    if (off < 0) return;
    StreamPtrs p = stream_ptrs(g, cache + off, s);
    const uint16_t *x = (s ? vnew : knew) + ((int64_t)b * g.Hkv + h) * D;
    float *st = state + (((int64_t)b * g.Hkv + h) * 2 + s) * D;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        const int c = lane + 64 * i;
        const int blk = c >> 5;
        const uint16_t xv = x[c];
        if (r == 0) {
            ((uint16_t *)p.kf)[s ? vkf_pos(D, c, g.vbp) : kkf_pos(nb, c)] = xv;
            if ((lane & 31) == 0) p.sc[blk] = 0;       // new group: reset the max-|scale| slot
            st[c] = h2f(xv);
        } else {
            float xh = st[c];
            int code;
            uint16_t s16;
            q40_delta_step(h2f(xv), xh, code, s16);
            if ((lane & 31) == 0) {
                p.sc[r * nb + blk] = s16;
                p.sc[blk] = (uint16_t)max((int)p.sc[blk], (int)habs_bits(s16));
            }
            if (s == 0) {
                store_k_codes<D>(p.cd + (int64_t)(r - 1) * (D / 2), blk, code);
            } else {
                const int tau = r & 31;
                uint32_t *w = (uint32_t *)(p.cd + (int64_t)(r >> 5) * 16 * D) + vcode_word(D, tau, c, g.vbp);
                const int sh = 4 * vcode_nibble(tau);
                *w = (*w & ~(0xFu << sh)) | ((uint32_t)code << sh);
            }
            st[c] = xh;
        }
    }
}

}  // namespace dkv
