// Q4_0 block quantiser on a 32-lane half-wave (one lane per channel of the
// block), shared by the Delta-KV codec and the plain Q4_0 comparison encoder.
//   m      = value of largest |v| (lowest channel wins ties; +0 if all zero)
//   s      = m * -1/8,  id = s != 0 ? 1/s (correctly rounded) : 0
//   code   = min(15, trunc((v*id) + 8.5))      (two separately rounded ops)
//   scale  = fp16(s) round-to-nearest-even
// The Delta-KV codec quantises v = x - xhat and then advances
// xhat += (code-8) * float(scale) (exact product, one rounding).
#pragma once
#include "dkv_common.h"

namespace dkv {

// Max-|v| search inside a 32-lane half-wave with the lowest lane winning ties.
__device__ inline void half_wave_argmax(float a, int idx, float &amax, int &imax)
{
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) {
        float a2 = __shfl_xor(a, off, 32);
        int i2 = __shfl_xor(idx, off, 32);
        bool take = (a2 > a) || (a2 == a && i2 < idx);
        a = take ? a2 : a;
        idx = take ? i2 : idx;
    }
    amax = a;
    imax = idx;
}

// Quantise one delta value per lane (the lane's channel in a 32-lane block)
// and advance the reconstruction.  All lanes of the half-wave get the block's
// fp16 scale; each lane gets its own code.
__device__ inline void q40_delta_step(float x, float &xh, int &code, uint16_t &s16)
{
    const int sl = threadIdx.x & 31;
    float d = __fsub_rn(x, xh);
    float amax;
    int imax;
    half_wave_argmax(fabsf(d), sl, amax, imax);
    float m = __shfl(d, imax, 32);
    if (amax == 0.0f) m = 0.0f;
    float s = __fmul_rn(m, -0.125f);
    float id = (s != 0.0f) ? (1.0f / s) : 0.0f;
    float t = __fadd_rn(__fmul_rn(d, id), 8.5f);
    int c = (int)t;
    code = c > 15 ? 15 : c;
    s16 = f2h_rn(s);
    float sf = h2f(s16);
    xh = __fadd_rn(xh, __fmul_rn((float)(code - 8), sf));
}

__device__ inline uint16_t habs_bits(uint16_t h) { return (uint16_t)(h & 0x7FFF); }

// Store the K code bytes of one delta token (row r-1).  Lanes 0..15 of each
// half-wave write byte i = code[i] | code[i+16] << 4 of their block.
template <int D>
__device__ inline void store_k_codes(uint8_t *row, int blk, int code)
{
    const int sl = threadIdx.x & 31;
    int hi = __shfl_down(code, 16, 32);
    if (sl < 16) row[kcode_byte(D / 32, blk, sl)] = (uint8_t)(code | (hi << 4));
}

}  // namespace dkv
