// Matrix-core fused decode attention for keyframe intervals kf = 32*NT with
// NT = 2..16 (e.g. kf = 64, 128 or 512).
//
// Same delta-domain arithmetic as the 32-token kernel (Delta-KV article,
// section "핵심 아이디어"; attention as on page "KV 캐시 벡터 양자화와 주의 보존
// 변환", section "왜 복원 오차가 틀린 기준인가"), applied to a group of NT
// 32-token tiles:
//   K pass, tiles 0..NT-1: delta logits by MFMA on the raw codes, prefix sums
//     carried across tiles from the keyframe logit, logits kept in LDS;
//   softmax update with the group maximum;
//   V pass, tiles NT-1..0: suffix sums of the softmax weights carried across
//     tiles from the end of the group, weighted V codes by MFMA;
//   keyframe: acc += (sum of the group's weights) * keyframe.
// One wavefront per (sequence, kv-head, run of groups); lane = 16*j + n.
#include "dkv_fused_common.h"

namespace dkv {

constexpr int kMaxTilesLong = 16;

template <int D>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2)))
    k_attn_fused_long(dkv_config cfg, const uint8_t *__restrict__ cache, const int32_t *__restrict__ bt,
                      const float *__restrict__ q, const int32_t *__restrict__ seq_lens, float scale_log2,
                      float *__restrict__ ws, int nsplit, int chunk)
{
    constexpr int NB = D / 32, NCC = D / 16;
    const Geom g = make_geom(cfg);
    const int NT = g.kf / 32;
    const int split = grid_split(), h = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x, j = lane >> 4, n = lane & 15;
    const int G = g.G;
    const int L = min(seq_lens[b], g.cap_tokens);
    const int ng = (L + g.kf - 1) / g.kf;
    const int g0 = split * chunk, g1 = min(ng, g0 + chunk);

    __shared__ __attribute__((aligned(16))) uint32_t side[2 * D];    // [K keyframe][K scales][V keyframe][V scales]
    __shared__ u4 qB[2 * NB * 64];
    // dynamic LDS: the scaled query during set-up, then the logits [tile][half][lane] of the current group
    extern __shared__ f4 dyn[];
    float(*sq)[D + 4] = (float(*)[D + 4])dyn;
    f4 *lg = dyn;

    // ---------------------------------------------------------------- query (as in the 32-token kernel)
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
    if (qm > 0.0f) frexpf(qm, &E);
    const float qscale = ldexpf(1.0f, -E);
    const float c2E = ldexpf(1.0f, E);
    float Qs[NB];
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
        float qsum = 0.0f;
        h8 Bh, Bl;
#pragma unroll
        for (int hh = 0; hh < 8; ++hh) {
            const bool f16x = ((hh >> 1) & 1) != 0;
            const float x = sq[n][32 * bb + kf_k_channel(j, hh)] * qscale * (f16x ? 1.0f : 16.0f);
            const _Float16 hi = (_Float16)x;
            const _Float16 lo = (_Float16)(x - (float)hi);
            Bh[hh] = hi;
            Bl[hh] = lo;
            qsum += ((float)hi + (float)lo) * (f16x ? 1.0f : 0.0625f);
        }
        qsum += __shfl_xor(qsum, 16);
        qsum += __shfl_xor(qsum, 32);
        Qs[bb] = qsum;
        qB[(2 * bb) * 64 + lane] = __builtin_bit_cast(u4, Bh);
        qB[(2 * bb + 1) * 64 + lane] = __builtin_bit_cast(u4, Bl);
    }
    h8 B2h, B2l;
#pragma unroll
    for (int hh = 0; hh < 8; ++hh) {
        const float x = (j == 0 && hh < NB) ? -8.0f * Qs[hh < NB ? hh : 0] : 0.0f;
        const _Float16 hi = (_Float16)x;
        B2h[hh] = hi;
        B2l[hh] = (_Float16)(x - (float)hi);
    }
    u4 azr;
    azr[0] = 0x80088008u;
    azr[1] = 0x80808080u;
    azr[2] = 0x80088008u;
    azr[3] = 0x80808080u;
    const h8 AZ = as_h8(azr);

    RunState<D> st;
#pragma unroll
    for (int cc = 0; cc < NCC; ++cc) st.acc[cc] = f4{0, 0, 0, 0};
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) st.Z[bb] = f4{0, 0, 0, 0};
    st.m = -INFINITY;
    st.l = 0.0f;
    st.beta = 127;

    const LaneOffsets lo = lane_offsets<D>(g, lane, j, n);
    const int rec_bytes = (int)g.rec;
    const uint8_t *sb = (const uint8_t *)side;

    for (int gi = g0; gi < g1; ++gi) {
        const int64_t off = group_offset(g, bt, b, h, gi);
        if (off < 0) continue;
        const uint8_t *rec = cache + off;
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc((void *)rec, (short)0, rec_bytes, 0x00020000);
        const int nvg = min(g.kf, L - gi * g.kf);          // valid tokens of the group
        const int ntl = (nvg + 31) >> 5;                   // tiles holding valid tokens

        // ---------------------------------------------------------- K pass
        float carry = 0.0f;                                // running logit (qn units) at the end of the last tile
        float mx = -INFINITY;
        for (int t = 0; t < ntl; ++t) {
            const int nvt = min(32, nvg - 32 * t);
            // stage: K keyframe (tile 0) and the K scales of this tile
            __syncthreads();
            if (lane < D / 8) {
                if (t == 0) {
                    u4 v = __builtin_amdgcn_raw_buffer_load_b128(rs, 16 * lane, 0, kStream);
                    const uint32_t w0 = v[0], w2 = v[2];
                    v[0] = scale_h2_16th(w0);
                    v[2] = scale_h2_16th(w2);
                    ((u4 *)side)[lane] = v;
                }
            } else if (lane < D / 4) {
                ((u4 *)side)[lane] = __builtin_amdgcn_raw_buffer_load_b128(
                    rs, (int)g.off_ksc + 64 * NB * t + 16 * (lane - D / 8), 0, kStream);
            }
            // K codes of tokens 32t + 16T + m (row = token - 1; the keyframe slot reads a dummy row)
            uint32_t kc[2][NB];
            {
                // token 32t + n is code row 32t + n - 1, except the keyframe (t = n = 0: a dummy row)
                const int k0t = (t == 0) ? lo.k0 : (int)g.off_kcd + (32 * t + n - 1) * (D / 2) + 4 * j * NB;
                const int k1t = lo.k1 + 32 * t * (D / 2);
                if constexpr (NB == 4) {
                    const u4 a = __builtin_amdgcn_raw_buffer_load_b128(rs, k0t, 0, kStream);
                    const u4 c = __builtin_amdgcn_raw_buffer_load_b128(rs, k1t, 0, kStream);
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        kc[0][k] = a[k];
                        kc[1][k] = c[k];
                    }
                } else {
                    const u2 a = __builtin_amdgcn_raw_buffer_load_b64(rs, k0t, 0, kStream);
                    const u2 c = __builtin_amdgcn_raw_buffer_load_b64(rs, k1t, 0, kStream);
#pragma unroll
                    for (int k = 0; k < 2; ++k) {
                        kc[0][k] = a[k];
                        kc[1][k] = c[k];
                    }
                }
            }
            __syncthreads();
            const bool first = t == 0;
            float dl[2][4];
#pragma unroll
            for (int T = 0; T < 2; ++T) {
                uint32_t sg[4][NB / 2];
                const uint32_t *sp = (const uint32_t *)(sb + 2 * D + (16 * T + 4 * j) * 2 * NB);
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int k = 0; k < NB / 2; ++k) sg[i][k] = sp[i * (NB / 2) + k];
                if (T == 0) {
#pragma unroll
                    for (int k = 0; k < NB / 2; ++k) sg[0][k] = (first && j == 0) ? 0x00100010u : sg[0][k];
                }
                f4 u = f4{0, 0, 0, 0};
#pragma unroll
                for (int bb = 0; bb < NB; ++bb) {
                    h8 A = unpack8(kc[T][bb]);
                    if (T == 0) {
                        const u4 k = *(const u4 *)(sb + (j * NB + bb) * 16);
                        u4 a = __builtin_bit_cast(u4, A);
#pragma unroll
                        for (int e = 0; e < 4; ++e) a[e] = (first && n == 0) ? k[e] : a[e];
                        A = as_h8(a);
                    }
                    const h8 bh = as_h8(qB[(2 * bb) * 64 + lane]);
                    const h8 bl = as_h8(qB[(2 * bb + 1) * 64 + lane]);
                    f4 P = mfma(A, bh, f4{0, 0, 0, 0});
                    P = mfma(A, bl, P);
#pragma unroll
                    for (int i = 0; i < 4; ++i) u[i] = __builtin_fmaf(half_at(sg[i], bb), P[i], u[i]);
                }
                u4 a2 = u4{0, 0, 0, 0};
                {
                    const uint32_t *ap = (const uint32_t *)(sb + 2 * D + (16 * T + n) * 2 * NB);
                    const bool use = j == 0 && !(first && T == 0 && n == 0);
#pragma unroll
                    for (int k = 0; k < NB / 2; ++k) a2[k] = use ? ap[k] : 0u;
                }
                f4 C2 = mfma(as_h8(a2), B2h, f4{0, 0, 0, 0});
                C2 = mfma(as_h8(a2), B2l, C2);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float d = __builtin_fmaf(u[i], 1048576.0f, C2[i]);
                    dl[T][i] = (16 * T + 4 * j + i < nvt) ? d : 0.0f;
                }
            }
            // prefix over the tile's tokens, carried from the previous tiles
            float excl[2], all[2];
            float Lg[2][4];
#pragma unroll
            for (int T = 0; T < 2; ++T) {
                Lg[T][0] = dl[T][0];
#pragma unroll
                for (int i = 1; i < 4; ++i) Lg[T][i] = Lg[T][i - 1] + dl[T][i];
                const float tot = Lg[T][3];
                float incl;
                rows_prefix(tot, j, incl, all[T]);
                excl[T] = incl - tot;
            }
#pragma unroll
            for (int T = 0; T < 2; ++T)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    Lg[T][i] += carry + excl[T] + (T == 1 ? all[0] : 0.0f);
                    if (16 * T + 4 * j + i < nvt) mx = fmaxf(mx, Lg[T][i]);
                }
            carry += all[0] + all[1];
#pragma unroll
            for (int T = 0; T < 2; ++T) lg[(2 * t + T) * 64 + lane] = f4{Lg[T][0], Lg[T][1], Lg[T][2], Lg[T][3]};
        }
        mx = rows_max(mx);
        const float m_g = mx * c2E;

        // ---------------------------------------------------------- softmax update
        uint32_t vmx = 0;
        {
            const u2 s0 = __builtin_amdgcn_raw_buffer_load_b64(rs, (int)g.off_vsc, 0, kStream);   // slot 0: max |scale|
#pragma unroll
            for (int k = 0; k < NB / 2; ++k) {
                const uint32_t w = s0[k] & 0x7FFF7FFFu;
                vmx = max(vmx, max(w & 0xFFFFu, w >> 16));
            }
        }
        const int ev = (vmx >> 10) == 0 ? -14 : (int)(vmx >> 10) - 15;
        const int lkf = 32 - __builtin_clz((unsigned)g.kf - 1u);       // kf <= 2^lkf
        const int beta_g = vmx == 0 ? 24 - lkf : 10 - lkf - ev;        // kf * 16 * |s| * 2^beta < 2^15
        const float m_new = fmaxf(st.m, m_g);
        const int beta_new = min(st.beta, beta_g);
        const float a_m = __builtin_amdgcn_exp2f(st.m - m_new);
        if (__any(m_new != st.m || beta_new != st.beta)) {
            const float alpha = a_m * ldexpf(1.0f, beta_new - st.beta);
#pragma unroll
            for (int cc = 0; cc < NCC; ++cc) st.acc[cc] *= alpha;
#pragma unroll
            for (int bb = 0; bb < NB; ++bb) st.Z[bb] *= alpha;
            st.l *= a_m;
        }
        st.m = m_new;
        st.beta = beta_new;
        const float bsc = ldexpf(1.0f, st.beta);

        // ---------------------------------------------------------- V pass (last tile first)
        float carryS = 0.0f;                               // sum of the weights of the later tiles
        for (int t = ntl - 1; t >= 0; --t) {
            const int nvt = min(32, nvg - 32 * t);
            __syncthreads();
            if (lane < D / 8) {
                if (t == 0)
                    ((u4 *)side)[D / 4 + lane] = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)g.off_vkf + 16 * lane,
                                                                                       0, kStream);
            } else if (lane < D / 4) {
                ((u4 *)side)[D / 4 + lane] = __builtin_amdgcn_raw_buffer_load_b128(
                    rs, (int)g.off_vsc + 64 * NB * t + 16 * (lane - D / 8), 0, kStream);
            }
            uint32_t vc[NCC];
#pragma unroll
            for (int q4 = 0; q4 < NCC / 4; ++q4) {
                const u4 a = __builtin_amdgcn_raw_buffer_load_b128(rs, lo.v + 16 * D * t + vcode_piece(D, 0, q4), 0,
                                                                   kStream);
#pragma unroll
                for (int k = 0; k < 4; ++k) vc[4 * q4 + k] = a[k];
            }
            __syncthreads();
            float S[2][4];
#pragma unroll
            for (int T = 0; T < 2; ++T) {
                const f4 lv = lg[(2 * t + T) * 64 + lane];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(lv[i], c2E, -m_new));
                    S[T][i] = (16 * T + 4 * j + i < nvt) ? p : 0.0f;
                }
            }
            float sexcl[2], sall[2];
#pragma unroll
            for (int T = 0; T < 2; ++T) {
#pragma unroll
                for (int i = 2; i >= 0; --i) S[T][i] += S[T][i + 1];
                const float tot = S[T][0];
                float incl;
                rows_suffix(tot, j, incl, sall[T]);
                sexcl[T] = incl - tot;
            }
            float Sp[2][4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float k16 = (i & 1) ? bsc : 16.0f * bsc;
                Sp[1][i] = (S[1][i] + sexcl[1] + carryS) * k16;
                Sp[0][i] = (S[0][i] + (sexcl[0] + sall[1] + carryS)) * k16;
            }
            if (t == 0) Sp[0][0] = j == 0 ? 0.0f : Sp[0][0];       // keyframe slot
            carryS += sall[0] + sall[1];
#pragma unroll
            for (int k = 0; k < NB / 2; ++k) {
                uint32_t vs[2][4];
#pragma unroll
                for (int T = 0; T < 2; ++T) {
                    const uint32_t *sp = (const uint32_t *)(sb + 6 * D + (16 * T + 4 * j) * 2 * NB);
#pragma unroll
                    for (int i = 0; i < 4; ++i) vs[T][i] = (16 * T + 4 * j + i < nvt) ? sp[i * (NB / 2) + k] : 0u;
                }
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int bb = 2 * k + e;
                    h8 Wh, Wl;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float s0 = e ? hhi(vs[0][i]) : hlo(vs[0][i]);
                        const float s1 = e ? hhi(vs[1][i]) : hlo(vs[1][i]);
                        const _Float16 h0 = (_Float16)__builtin_fmaf(s0, Sp[0][i], 0.0f);
                        const _Float16 h1 = (_Float16)__builtin_fmaf(s1, Sp[1][i], 0.0f);
                        Wh[2 * i] = h0;
                        Wh[2 * i + 1] = h1;
                        Wl[2 * i] = (_Float16)__builtin_fmaf(s0, Sp[0][i], -(float)h0);
                        Wl[2 * i + 1] = (_Float16)__builtin_fmaf(s1, Sp[1][i], -(float)h1);
                    }
#pragma unroll
                    for (int c2 = 0; c2 < 2; ++c2) {
                        const int cc = 2 * bb + c2;
                        const h8 A = unpack8(vc[cc]);
                        st.acc[cc] = mfma(A, Wh, st.acc[cc]);
                        st.acc[cc] = mfma(A, Wl, st.acc[cc]);
                    }
                    st.Z[bb] = mfma(AZ, Wh, st.Z[bb]);
                    st.Z[bb] = mfma(AZ, Wl, st.Z[bb]);
                }
            }
        }
        // ---------------------------------------------------------- keyframe and running sum
        const float Pg = carryS;
        st.l += Pg;
        const float pk = Pg * ldexpf(1.0f, st.beta - 20);
        const uint32_t *kp = (const uint32_t *)(sb + 4 * D + j * NCC * 8);
#pragma unroll
        for (int cc = 0; cc < NCC; ++cc) {
            const uint32_t w01 = kp[2 * cc], w23 = kp[2 * cc + 1];
            st.acc[cc][0] = __builtin_fmaf(hlo(w01), pk, st.acc[cc][0]);
            st.acc[cc][1] = __builtin_fmaf(hhi(w01), pk, st.acc[cc][1]);
            st.acc[cc][2] = __builtin_fmaf(hlo(w23), pk, st.acc[cc][2]);
            st.acc[cc][3] = __builtin_fmaf(hhi(w23), pk, st.acc[cc][3]);
        }
    }

    // ---------------------------------------------------------------- partials
    if (n < G) {
        float *recp = ws + (((int64_t)b * g.Hq + h * G + n) * nsplit + split) * part_stride(D);
        const float un = ldexpf(1.0f, 20 - st.beta);
#pragma unroll
        for (int cc = 0; cc < NCC; ++cc) {
            f4 o;
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = (st.acc[cc][i] + st.Z[cc >> 1][i]) * un;
            *(f4 *)(recp + 16 * cc + 4 * j) = o;
        }
        if (j == 0) {
            recp[D] = st.m;
            recp[D + 1] = st.l;
        }
    }
}

bool fused_long_supported(const dkv_config &c)
{
    const int kf = c.kf;
    return !vbp_layout(c) && kf > 32 && kf <= 32 * kMaxTilesLong && kf % 32 == 0 &&
           (c.head_dim == 64 || c.head_dim == 128) &&
           c.n_q_heads / c.n_kv_heads <= 16;
}

hipError_t launch_attn_fused_long(const dkv_config &c, const void *cache, const int32_t *bt, const float *q,
                                  const int32_t *lens, float scale_log2, float *ws, int nsplit, int chunk,
                                  hipStream_t st)
{
    dim3 grid(nsplit, c.n_kv_heads, c.batch);
    const size_t lg_bytes = (size_t)(c.kf / 32) * 2 * 64 * 16;
    const size_t sq_bytes = (size_t)16 * (c.head_dim + 4) * sizeof(float);
    const size_t lds = lg_bytes > sq_bytes ? lg_bytes : sq_bytes;
    if (c.head_dim == 64)
        hipLaunchKernelGGL(k_attn_fused_long<64>, grid, dim3(64), lds, st, c, (const uint8_t *)cache, bt, q, lens,
                           scale_log2, ws, nsplit, chunk);
    else
        hipLaunchKernelGGL(k_attn_fused_long<128>, grid, dim3(64), lds, st, c, (const uint8_t *)cache, bt, q, lens,
                           scale_log2, ws, nsplit, chunk);
    return hipGetLastError();
}

}  // namespace dkv
