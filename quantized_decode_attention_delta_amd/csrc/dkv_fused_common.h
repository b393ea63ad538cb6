// Device building blocks shared by the matrix-core fused decode-attention
// kernels (32-token groups and longer keyframe intervals).
#pragma once
#include "dkv_common.h"

namespace dkv {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

__device__ inline h8 as_h8(u4 v) { return __builtin_bit_cast(h8, v); }

// Eight 4-bit codes -> eight fp16 subnormals.  Half hh holds nibble
// (hh>>1) + 4*(hh&1) of w, valued nibble * 2^-24 * f(hh) with f = 16 for
// hh in {2,3,6,7} and 1 otherwise.
__device__ inline h8 unpack8(uint32_t w)
{
    u4 r;
    r[0] = w & 0x000F000Fu;
    r[1] = w & 0x00F000F0u;
    const uint32_t w8 = w >> 8;
    r[2] = w8 & 0x000F000Fu;
    r[3] = w8 & 0x00F000F0u;
    return as_h8(r);
}

__device__ inline f4 mfma(h8 a, h8 b, f4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }

__device__ inline float hlo(uint32_t p) { return (float)__builtin_bit_cast(h2, p)[0]; }
__device__ inline float hhi(uint32_t p) { return (float)__builtin_bit_cast(h2, p)[1]; }
__device__ inline float half_at(const uint32_t *w, int k) { return (k & 1) ? hhi(w[k >> 1]) : hlo(w[k >> 1]); }

// Cross-row exchanges with gfx950 permlane swaps (VALU, no LDS round trip).
// The 64 lanes form 4 rows j of 16; these helpers combine the 4 values that
// one column n holds in rows 0..3.
// (Inline asm on two distinct registers: the compiler builtin models both
// results in one register.  The s_nop covers the VALU-write -> permlane-read
// gap; the asm has no side effects, so the scheduler may move it.)
__device__ inline void swap16(float x, float &r0, float &r1)
{
    // r0 = rows (x0, x0, x2, x2), r1 = rows (x1, x1, x3, x3)
    float a = x, b = x;
    asm("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
    r0 = a;
    r1 = b;
}
__device__ inline void swap32(float x, float &r0, float &r1)
{
    // r0 = rows (x0, x1, x0, x1), r1 = rows (x2, x3, x2, x3)
    float a = x, b = x;
    asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
    r0 = a;
    r1 = b;
}
// Inclusive prefix over rows 0..j of the column, and the column total.
__device__ inline void rows_prefix(float x, int j, float &incl, float &total)
{
    float a0, a1, b0, b1;
    swap16(x, a0, a1);
    const float t = a0 + a1;
    swap32(t, b0, b1);
    incl = ((j & 1) ? t : a0) + (j >= 2 ? b0 : 0.0f);
    total = b0 + b1;
}
// Inclusive suffix over rows j..3 of the column, and the column total.
__device__ inline void rows_suffix(float x, int j, float &incl, float &total)
{
    float a0, a1, b0, b1;
    swap16(x, a0, a1);
    const float t = a0 + a1;
    swap32(t, b0, b1);
    incl = ((j & 1) ? a1 : t) + (j < 2 ? b1 : 0.0f);
    total = b0 + b1;
}
// Sum over the 4 rows of a column (all rows get the total).
__device__ inline float rows_sum(float x)
{
    float a0, a1, b0, b1;
    swap16(x, a0, a1);
    swap32(a0 + a1, b0, b1);
    return b0 + b1;
}
// fp32 max without the quieting copies that fmaxf adds around operands the
// compiler cannot prove canonical (results of lane exchanges); the operands
// here are never signalling NaNs.
__device__ inline float fmax_nc(float a, float b)
{
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}
__device__ inline float rows_max(float x)
{
    float a0, a1, b0, b1;
    swap16(x, a0, a1);
    swap32(fmax_nc(a0, a1), b0, b1);
    return fmax_nc(b0, b1);
}

// Lane index computed afresh (not CSE-able), to keep it out of the register
// allocation of long loops.
__device__ inline int fresh_lane_id()
{
    int x;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(x));
    return x;
}

// Both fp16 halves of a word times 1/16.
__device__ inline uint32_t scale_h2_16th(uint32_t x)
{
    const h2 sc = {(_Float16)0.0625f, (_Float16)0.0625f};
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, x) * sc);
}

__device__ inline uint32_t pack_h2(float lo, float hi)
{
    h2 v;
    v[0] = (_Float16)lo;
    v[1] = (_Float16)hi;
    return __builtin_bit_cast(uint32_t, v);
}

// V weights of two token slots: w0 = s0 * x0 into the low half and w1 = s1 * x1
// into the high half of `hi` (fp16, round to nearest), and the fp16 residues
// x*s - w into `lo`.  s0, s1: fp16 in half SEL of sw0, sw1; the residue reads
// its w straight from the half of `hi` it sits in.
template <int SEL>
__device__ inline void split_w(uint32_t sw0, uint32_t sw1, float x0, float x1, uint32_t &hi, uint32_t &lo)
{
    if constexpr (SEL == 0)
        asm("v_fma_mixlo_f16 %0, %2, %4, 0 op_sel_hi:[1,0,0]\n\t"
            "v_fma_mixhi_f16 %0, %3, %5, 0 op_sel_hi:[1,0,0]\n\t"
            "v_fma_mixlo_f16 %1, %2, %4, -%0 op_sel_hi:[1,0,1]\n\t"
            "v_fma_mixhi_f16 %1, %3, %5, -%0 op_sel:[0,0,1] op_sel_hi:[1,0,1]"
            : "=&v"(hi), "=&v"(lo)
            : "v"(sw0), "v"(sw1), "v"(x0), "v"(x1));
    else
        asm("v_fma_mixlo_f16 %0, %2, %4, 0 op_sel:[1,0,0] op_sel_hi:[1,0,0]\n\t"
            "v_fma_mixhi_f16 %0, %3, %5, 0 op_sel:[1,0,0] op_sel_hi:[1,0,0]\n\t"
            "v_fma_mixlo_f16 %1, %2, %4, -%0 op_sel:[1,0,0] op_sel_hi:[1,0,1]\n\t"
            "v_fma_mixhi_f16 %1, %3, %5, -%0 op_sel:[1,0,1] op_sel_hi:[1,0,1]"
            : "=&v"(hi), "=&v"(lo)
            : "v"(sw0), "v"(sw1), "v"(x0), "v"(x1));
}

// Value of lane n ^ 8 within each row of 16 lanes (DPP row rotate by 8).
__device__ inline float other_half(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x128, 0xF, 0xF, false));
}

// Byte offsets of a lane's loads inside a group record (the same for every group).
struct LaneOffsets {
    int side, k0, k1, v;
};

// zero_kf_row: the keyframe row (token 0) of the K operand reads past the
// record (zeros) instead of a dummy code row.
template <int D>
__device__ inline LaneOffsets lane_offsets(const Geom &g, int lane, int j, int n, bool zero_kf_row = false)
{
    constexpr int NB = D / 32, NCC = D / 16, SIDE_LANES = D / 4;
    LaneOffsets o;
    // lanes beyond the side data read past the record: the buffer unit returns zeros
    o.side = lane < SIDE_LANES ? 16 * lane
           : lane < 2 * SIDE_LANES ? (int)g.off_vkf + 16 * (lane - SIDE_LANES) : 0x40000000;
    const int row0 = n > 0 ? n - 1 : 0;        // token n of tile 0 (token 0 is the keyframe)
    o.k0 = (zero_kf_row && n == 0) ? 0x40000000 : (int)g.off_kcd + row0 * (D / 2) + 4 * j * NB;
    o.k1 = (int)g.off_kcd + (15 + n) * (D / 2) + 4 * j * NB;
    o.v = (int)g.off_vcd + vcode_piece(D, j * 16 + n, 0);
    return o;
}

// Softmax / accumulation state of one wavefront.
template <int D>
struct RunState {
    f4 acc[D / 16];    // sum_t p_t Vhat_t, channels 16cc + 4j + i of head n, units 2^(beta-20)
    f4 Z[D / 32];      // the "-8" part of each block, same units
    float m, l;        // running max (log2 units) and sum of the softmax weights
    int beta;          // fp16 range bias of the V weights
    float bsc;         // 2^beta (kept by the GQA <= 8 kernels)
};

}  // namespace dkv
