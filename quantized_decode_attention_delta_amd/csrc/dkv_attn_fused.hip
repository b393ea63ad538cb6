// Matrix-core fused decode attention over the Delta-KV cache (gfx950).
//
// Attention (page "KV 캐시 벡터 양자화와 주의 보존 변환", section "왜 복원 오차가
// 틀린 기준인가") over a cache stored as keyframes plus closed-loop Q4_0 deltas
// (Delta-KV article, section "핵심 아이디어").  Decode reads every cached byte
// once (section "KV 캐시가 왜 병목인가": the K/V read is the bottleneck), so the
// kernel never rebuilds K or V: it works in the delta domain.
//
// Within a group of kf tokens with keyframe x_0 and deltas
// d_r = (c_r - 8) * s_r (per 32-channel block):
//   K side:  q.Khat_t = q.x_0 + sum_{r<=t} q.d_r
//            -> one 16x16x32 fp16 MFMA per (16 tokens, 32-channel block) on the
//               raw 4-bit codes, scale applied per (token, block) in fp32, then a
//               prefix sum over the group's tokens;
//   V side:  sum_t p_t Vhat_t = (sum_t p_t) x_0 + sum_r S_r d_r,
//            S_r = sum_{t>=r} p_t (suffix sums of the softmax weights)
//            -> one MFMA per (16 channels, 32 token slots) with the weights
//               S_r * s_r as the second operand.
// Codes enter the matrix cores as fp16 subnormals (nibble * 2^-24, obtained by
// masking, no conversion instructions); products with fp16 operands are exact
// and accumulate in fp32.  The "-8" of the Q4_0 code is applied through one
// extra small MFMA per side.  The query and the V weights are split in
// hi + lo fp16 parts so that the fp16 operands carry ~22 significant bits.
//
// Layout of the work: one wavefront per (sequence, kv-head, run of groups);
// lane = 16*j + n.  K side: MFMA rows are tokens (16 per tile, two tiles per
// 32-token group), columns are the G query heads (padded to 16).  A lane holds
// tokens 16T + 4j + i (i < 4) of head n, which is exactly the operand layout
// the V-side MFMA wants for its weights, so no data moves between the phases.
// The group's scales and keyframes (1 KB) are staged through LDS once.
#include "dkv_common.h"

namespace dkv {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

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

__device__ inline uint32_t pack_h2(float lo, float hi)
{
    h2 v;
    v[0] = (_Float16)lo;
    v[1] = (_Float16)hi;
    return __builtin_bit_cast(uint32_t, v);
}

bool fused_supported(const dkv_config &c)
{
    return c.kf == 32 && (c.head_dim == 64 || c.head_dim == 128) && c.n_q_heads / c.n_kv_heads <= 16;
}

// LDS image of a group's side data (kf = 32): [K keyframe][K scales][V keyframe][V scales], 2*D bytes each.
template <int D>
__global__ void __launch_bounds__(64)
    k_attn_fused32(dkv_config cfg, const uint8_t *__restrict__ cache, const int32_t *__restrict__ bt,
                   const float *__restrict__ q, const int32_t *__restrict__ seq_lens, float scale_log2,
                   float *__restrict__ ws, int nsplit, int chunk)
{
    constexpr int NB = D / 32;      // Q4_0 blocks per row
    constexpr int NCC = D / 16;     // 16-channel chunks
    constexpr int SIDE_LANES = D / 4; // lanes loading 16 B each per side range (4*D bytes)
    const Geom g = make_geom(cfg);
    const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x, j = lane >> 4, n = lane & 15;
    const int G = g.G;
    const int L = min(seq_lens[b], g.cap_tokens);
    const int ng = (L + 31) >> 5;
    const int g0 = split * chunk, g1 = min(ng, g0 + chunk);

    __shared__ float sq[16][D + 4];
    __shared__ __attribute__((aligned(16))) uint32_t side[2 * D];   // 8*D bytes

    // ---------------------------------------------------------------- query
    for (int i = lane; i < 16 * D; i += 64) {
        const int hh = i / D, c = i % D;
        sq[hh][c] = hh < G ? q[((int64_t)b * g.Hq + h * G + hh) * D + c] * scale_log2 : 0.0f;
    }
    __syncthreads();
    float qm = 0.0f;
    for (int c = j * (D / 4); c < (j + 1) * (D / 4); ++c) qm = fmaxf(qm, fabsf(sq[n][c]));
    qm = fmaxf(qm, __shfl_xor(qm, 16));
    qm = fmaxf(qm, __shfl_xor(qm, 32));
    int E = 0;
    if (qm > 0.0f) frexpf(qm, &E);         // |q'| * 2^-E < 1
    const float qscale = ldexpf(1.0f, -E);
    const float c2E = ldexpf(1.0f, E);

    h8 Bh[NB], Bl[NB];
    float Qs[NB];
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
        float qsum = 0.0f;
#pragma unroll
        for (int hh = 0; hh < 8; ++hh) {
            const bool f16x = ((hh >> 1) & 1) != 0;            // code half carries a factor 16
            const float x = sq[n][32 * bb + kf_k_channel(j, hh)] * qscale * (f16x ? 1.0f : 16.0f);
            const _Float16 hi = (_Float16)x;
            const _Float16 lo = (_Float16)(x - (float)hi);
            Bh[bb][hh] = hi;
            Bl[bb][hh] = lo;
            qsum += ((float)hi + (float)lo) * (f16x ? 1.0f : 0.0625f);
        }
        qsum += __shfl_xor(qsum, 16);
        qsum += __shfl_xor(qsum, 32);
        Qs[bb] = qsum;
    }
    // correction operand: -8 * Qs[block] at K index = block (lane group 0)
    h8 B2h, B2l;
#pragma unroll
    for (int hh = 0; hh < 8; ++hh) {
        const float x = (j == 0 && hh < NB) ? -8.0f * Qs[hh < NB ? hh : 0] : 0.0f;
        const _Float16 hi = (_Float16)x;
        B2h[hh] = hi;
        B2l[hh] = (_Float16)(x - (float)hi);
    }
    // V "-8" operand: -8 * 2^-24 * f(hh) as fp16 subnormals
    u4 azr;
    azr[0] = 0x80088008u;
    azr[1] = 0x80808080u;
    azr[2] = 0x80088008u;
    azr[3] = 0x80808080u;
    const h8 AZ = as_h8(azr);

    f4 acc[NCC];
    f4 Z[NB];
#pragma unroll
    for (int cc = 0; cc < NCC; ++cc) acc[cc] = f4{0, 0, 0, 0};
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) Z[bb] = f4{0, 0, 0, 0};
    float m_run = -INFINITY, l_run = 0.0f;
    int beta_run = 127;

    const uint8_t *side_b = (const uint8_t *)side;
    for (int gi = g0; gi < g1; ++gi) {
        const int64_t off = group_offset(g, bt, b, h, gi);
        if (off < 0) continue;
        const uint8_t *rec = cache + off;
        const int nval = min(32, L - gi * 32);

        // ---- loads: side data, K codes (two 16-token tiles), V codes
        u4 sidev = u4{0, 0, 0, 0};
        if (lane < SIDE_LANES) sidev = *(const u4 *)(rec + 16 * lane);
        else if (lane < 2 * SIDE_LANES) sidev = *(const u4 *)(rec + g.off_vkf + 16 * (lane - SIDE_LANES));
        uint32_t kc[2][NB];
#pragma unroll
        for (int T = 0; T < 2; ++T) {
            const int tau = 16 * T + n;
            const int row = tau > 0 ? tau - 1 : 0;
            const uint32_t *src = (const uint32_t *)(rec + g.off_kcd + (int64_t)row * (D / 2) + 4 * j * NB);
#pragma unroll
            for (int bb = 0; bb < NB; ++bb) kc[T][bb] = src[bb];
        }
        uint32_t vc[NCC];
        {
            const uint32_t *src = (const uint32_t *)(rec + g.off_vcd) + (j * 16 + n) * NCC;
#pragma unroll
            for (int cc = 0; cc < NCC; ++cc) vc[cc] = src[cc];
        }
        __syncthreads();
        if (lane < 2 * SIDE_LANES) ((u4 *)side)[lane] = sidev;
        __syncthreads();

        // ---- K side: delta logits per (token, head)
        float dl[2][4];
#pragma unroll
        for (int T = 0; T < 2; ++T) {
            // scales of tokens 16T + 4j + i (fp16 pairs over blocks)
            uint32_t sg[4][NB / 2];
            const uint32_t *sp = (const uint32_t *)(side_b + 2 * D + (16 * T + 4 * j) * 2 * NB);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int k = 0; k < NB / 2; ++k) sg[i][k] = sp[i * (NB / 2) + k];
            if (T == 0 && j == 0) {
#pragma unroll
                for (int k = 0; k < NB / 2; ++k) sg[0][k] = 0x00100010u;   // keyframe row: 2^-20
            }
            f4 u = f4{0, 0, 0, 0};
#pragma unroll
            for (int bb = 0; bb < NB; ++bb) {
                h8 A = unpack8(kc[T][bb]);
                if (T == 0 && n == 0) {
                    // keyframe row: fp16 keyframe values times f(hh)/16
                    u4 kv = *(const u4 *)(side_b + (j * NB + bb) * 16);
                    h8 kh = as_h8(kv);
#pragma unroll
                    for (int hh = 0; hh < 8; ++hh)
                        if (((hh >> 1) & 1) == 0) kh[hh] = kh[hh] * (_Float16)0.0625f;
                    A = kh;
                }
                f4 P = mfma(A, Bh[bb], f4{0, 0, 0, 0});
                P = mfma(A, Bl[bb], P);
#pragma unroll
                for (int i = 0; i < 4; ++i) u[i] = __builtin_fmaf(half_at(sg[i], bb), P[i], u[i]);
            }
            // correction: -8 * sum_b s_{t,b} Qs_b, with the token's scales at K index = block
            u4 a2 = u4{0, 0, 0, 0};
            if (j == 0 && !(T == 0 && n == 0)) {
                const uint32_t *ap = (const uint32_t *)(side_b + 2 * D + (16 * T + n) * 2 * NB);
#pragma unroll
                for (int k = 0; k < NB / 2; ++k) a2[k] = ap[k];
            }
            f4 C2 = mfma(as_h8(a2), B2h, f4{0, 0, 0, 0});
            C2 = mfma(as_h8(a2), B2l, C2);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tok = 16 * T + 4 * j + i;
                dl[T][i] = tok < nval ? __builtin_fmaf(u[i], 1048576.0f, C2[i]) : 0.0f;
            }
        }

        // ---- prefix over the group's tokens: order (T, j, i)
        float Lg[2][4];
        float tot[2], excl[2], all[2];
#pragma unroll
        for (int T = 0; T < 2; ++T) {
            Lg[T][0] = dl[T][0];
#pragma unroll
            for (int i = 1; i < 4; ++i) Lg[T][i] = Lg[T][i - 1] + dl[T][i];
            tot[T] = Lg[T][3];
            float x = tot[T];
            float y = __shfl_up(x, 16);
            if (j >= 1) x += y;
            y = __shfl_up(x, 32);
            if (j >= 2) x += y;
            excl[T] = x - tot[T];
            all[T] = __shfl(x, 48 + n);
        }
        float mx = -INFINITY;
#pragma unroll
        for (int T = 0; T < 2; ++T)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                Lg[T][i] += excl[T] + (T == 1 ? all[0] : 0.0f);
                const int tok = 16 * T + 4 * j + i;
                if (tok < nval) mx = fmaxf(mx, Lg[T][i]);
            }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_g = mx * c2E;

        // ---- V range: largest |scale| of the group sets the fp16 bias of the weights
        int vmax = 0;
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) {
            const uint16_t sv = ((const uint16_t *)(side_b + 6 * D))[bb] & 0x7FFF;
            vmax = max(vmax, (int)sv);
        }
        const int ev = (vmax >> 10) == 0 ? -14 : (vmax >> 10) - 15;
        const int beta_g = vmax == 0 ? 19 : 5 - ev;             // kf * 16 * |s| * 2^beta < 2^15

        const float m_new = fmaxf(m_run, m_g);
        const int beta_new = min(beta_run, beta_g);
        const float a_m = exp2f(m_run - m_new);
        const float alpha = a_m * ldexpf(1.0f, beta_new - beta_run);
        if (__any(alpha != 1.0f)) {
#pragma unroll
            for (int cc = 0; cc < NCC; ++cc) acc[cc] *= alpha;
#pragma unroll
            for (int bb = 0; bb < NB; ++bb) Z[bb] *= alpha;
        }
        l_run *= a_m;
        m_run = m_new;
        beta_run = beta_new;

        // ---- softmax weights and suffix sums
        float p[2][4], S[2][4];
#pragma unroll
        for (int T = 0; T < 2; ++T)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tok = 16 * T + 4 * j + i;
                p[T][i] = tok < nval ? exp2f(__builtin_fmaf(Lg[T][i], c2E, -m_new)) : 0.0f;
            }
        float stot[2], sexcl[2], sall[2];
#pragma unroll
        for (int T = 0; T < 2; ++T) {
            S[T][3] = p[T][3];
#pragma unroll
            for (int i = 2; i >= 0; --i) S[T][i] = S[T][i + 1] + p[T][i];
            stot[T] = S[T][0];
            float x = stot[T];
            float y = __shfl_down(x, 16);
            if (j <= 2) x += y;
            y = __shfl_down(x, 32);
            if (j <= 1) x += y;
            sexcl[T] = x - stot[T];
            sall[T] = __shfl(x, n);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            S[1][i] += sexcl[1];
            S[0][i] += sexcl[0] + sall[1];
        }
        const float Pg = sall[0] + sall[1];
        l_run += Pg;

        // ---- V weights W = S * s * 2^beta * 16/f, split hi + lo fp16 (slot 0 = keyframe: 0)
        uint32_t vs[2][4][NB / 2];
#pragma unroll
        for (int T = 0; T < 2; ++T) {
            const uint32_t *sp = (const uint32_t *)(side_b + 6 * D + (16 * T + 4 * j) * 2 * NB);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int k = 0; k < NB / 2; ++k) {
                    const int tok = 16 * T + 4 * j + i;
                    vs[T][i][k] = tok < nval ? sp[i * (NB / 2) + k] : 0u;
                }
        }
        const float bsc = ldexpf(1.0f, beta_run);
        float Sp[2][4];
#pragma unroll
        for (int T = 0; T < 2; ++T)
#pragma unroll
            for (int i = 0; i < 4; ++i) Sp[T][i] = S[T][i] * bsc * ((i & 1) ? 1.0f : 16.0f);
        if (j == 0) Sp[0][0] = 0.0f;
        h8 Wh[NB], Wl[NB];
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) {
            u4 rh, rl;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float w0 = Sp[0][i] * half_at(vs[0][i], bb);
                const float w1 = Sp[1][i] * half_at(vs[1][i], bb);
                const _Float16 h0 = (_Float16)w0, h1 = (_Float16)w1;
                rh[i] = pack_h2((float)h0, (float)h1);
                rl[i] = pack_h2(w0 - (float)h0, w1 - (float)h1);
            }
            Wh[bb] = as_h8(rh);
            Wl[bb] = as_h8(rl);
        }
        // ---- V side MFMAs
#pragma unroll
        for (int cc = 0; cc < NCC; ++cc) {
            const h8 A = unpack8(vc[cc]);
            acc[cc] = mfma(A, Wh[cc >> 1], acc[cc]);
            acc[cc] = mfma(A, Wl[cc >> 1], acc[cc]);
        }
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) {
            Z[bb] = mfma(AZ, Wh[bb], Z[bb]);
            Z[bb] = mfma(AZ, Wl[bb], Z[bb]);
        }
        // ---- keyframe: acc += P_g * x0 (in the accumulator's units 2^(beta-20))
        {
            const float pk = Pg * ldexpf(1.0f, beta_run - 20);
            const uint32_t *kp = (const uint32_t *)(side_b + 4 * D + j * NCC * 8);
#pragma unroll
            for (int cc = 0; cc < NCC; ++cc) {
                const uint32_t w01 = kp[2 * cc], w23 = kp[2 * cc + 1];
                acc[cc][0] = __builtin_fmaf(hlo(w01), pk, acc[cc][0]);
                acc[cc][1] = __builtin_fmaf(hhi(w01), pk, acc[cc][1]);
                acc[cc][2] = __builtin_fmaf(hlo(w23), pk, acc[cc][2]);
                acc[cc][3] = __builtin_fmaf(hhi(w23), pk, acc[cc][3]);
            }
        }
    }

    // ---------------------------------------------------------------- partials
    if (n < G) {
        float *rec = ws + (((int64_t)b * g.Hq + h * G + n) * nsplit + split) * part_stride(D);
        const float un = ldexpf(1.0f, 20 - beta_run);
#pragma unroll
        for (int cc = 0; cc < NCC; ++cc) {
            f4 o;
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = (acc[cc][i] + Z[cc >> 1][i]) * un;
            *(f4 *)(rec + 16 * cc + 4 * j) = o;
        }
        if (j == 0) {
            rec[D] = m_run;
            rec[D + 1] = l_run;
        }
    }
}

hipError_t launch_attn_fused(const dkv_config &c, const void *cache, const int32_t *bt, const float *q,
                             const int32_t *lens, float scale_log2, float *ws, int nsplit, int chunk,
                             hipStream_t st)
{
    dim3 grid(nsplit, c.n_kv_heads, c.batch);
    if (c.head_dim == 64)
        hipLaunchKernelGGL(k_attn_fused32<64>, grid, dim3(64), 0, st, c, (const uint8_t *)cache, bt, q, lens,
                           scale_log2, ws, nsplit, chunk);
    else
        hipLaunchKernelGGL(k_attn_fused32<128>, grid, dim3(64), 0, st, c, (const uint8_t *)cache, bt, q, lens,
                           scale_log2, ws, nsplit, chunk);
    return hipGetLastError();
}

}  // namespace dkv
