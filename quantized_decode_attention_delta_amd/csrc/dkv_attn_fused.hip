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
#include "dkv_fused_common.h"

namespace dkv {

bool fused_supported(const dkv_config &c)
{
    return c.kf == 32 && (c.head_dim == 64 || c.head_dim == 128) && c.n_q_heads / c.n_kv_heads <= 16 &&
           !vbp_layout(c);
}

// Per-group inputs of the fused kernel, fetched one group ahead.
template <int D>
struct GroupRegs {
    u4 side;                          // 16 B of the group's side data (this lane's share)
    uint32_t kc[2][D / 32];           // K code pieces of tokens 16T + n (piece j)
    uint32_t vc[D / 16];              // V code words of channel n (piece j)
};

template <int D>
__device__ inline void load_group(GroupRegs<D> &r, const uint8_t *rec, int rec_bytes, const LaneOffsets &o)
{
    constexpr int NB = D / 32, NCC = D / 16;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void *)rec, (short)0, rec_bytes, 0x00020000);
    r.side = __builtin_amdgcn_raw_buffer_load_b128(rs, o.side, 0, kStream);
    if constexpr (NB == 4) {
        u4 a = __builtin_amdgcn_raw_buffer_load_b128(rs, o.k0, 0, kStream);
        u4 c = __builtin_amdgcn_raw_buffer_load_b128(rs, o.k1, 0, kStream);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            r.kc[0][k] = a[k];
            r.kc[1][k] = c[k];
        }
    } else {
        u2 a = __builtin_amdgcn_raw_buffer_load_b64(rs, o.k0, 0, kStream);
        u2 c = __builtin_amdgcn_raw_buffer_load_b64(rs, o.k1, 0, kStream);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            r.kc[0][k] = a[k];
            r.kc[1][k] = c[k];
        }
    }
#pragma unroll
    for (int q4 = 0; q4 < NCC / 4; ++q4) {
        u4 a = __builtin_amdgcn_raw_buffer_load_b128(rs, o.v + vcode_piece(D, 0, q4), 0, kStream);
#pragma unroll
        for (int k = 0; k < 4; ++k) r.vc[4 * q4 + k] = a[k];
    }
}

// One 32-token group: K-side logits, online-softmax update, V-side accumulation.
// FULL: all 32 tokens valid (no masking).  side_b: the group's side data in LDS.
template <int D, bool FULL>
__device__ inline void process_group(RunState<D> &st, const GroupRegs<D> &r, const uint8_t *side_b, int nval,
                                     int j, int n, const u4 *qB, float c2E, h8 B2h, h8 B2l, h8 AZ)
{
    constexpr int NB = D / 32, NCC = D / 16;
    const int lane = 16 * j + n;
    // ---- K side: delta logits per (token, head)
    float dl[2][4];
#pragma unroll
    for (int T = 0; T < 2; ++T) {
        uint32_t sg[4][NB / 2];
        const uint32_t *sp = (const uint32_t *)(side_b + 2 * D + (16 * T + 4 * j) * 2 * NB);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int k = 0; k < NB / 2; ++k) sg[i][k] = sp[i * (NB / 2) + k];
        if (T == 0) {
#pragma unroll
            for (int k = 0; k < NB / 2; ++k) sg[0][k] = j == 0 ? 0x00100010u : sg[0][k];   // keyframe row: 2^-20
        }
        f4 u = f4{0, 0, 0, 0};
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) {
            h8 A = unpack8(r.kc[T][bb]);
            if (T == 0) {
                // token 0 of the group is the keyframe (staged in LDS already scaled by f(hh)/16)
                const u4 k = *(const u4 *)(side_b + (j * NB + bb) * 16);
                u4 a = __builtin_bit_cast(u4, A);
#pragma unroll
                for (int e = 0; e < 4; ++e) a[e] = n == 0 ? k[e] : a[e];
                A = as_h8(a);
            }
            // query operand (hi, lo) of block bb for this lane, staged in LDS
            const h8 bh = as_h8(qB[(2 * bb) * 64 + 16 * j + n]);
            const h8 bl = as_h8(qB[(2 * bb + 1) * 64 + 16 * j + n]);
            f4 P = mfma(A, bh, f4{0, 0, 0, 0});
            P = mfma(A, bl, P);
#pragma unroll
            for (int i = 0; i < 4; ++i) u[i] = __builtin_fmaf(half_at(sg[i], bb), P[i], u[i]);
        }
        u4 a2 = u4{0, 0, 0, 0};
        {
            const uint32_t *ap = (const uint32_t *)(side_b + 2 * D + (16 * T + n) * 2 * NB);
            const bool use = j == 0 && !(T == 0 && n == 0);
#pragma unroll
            for (int k = 0; k < NB / 2; ++k) a2[k] = use ? ap[k] : 0u;
        }
        f4 C2 = mfma(as_h8(a2), B2h, f4{0, 0, 0, 0});
        C2 = mfma(as_h8(a2), B2l, C2);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float d = __builtin_fmaf(u[i], 1048576.0f, C2[i]);
            dl[T][i] = (FULL || 16 * T + 4 * j + i < nval) ? d : 0.0f;
        }
    }

    // ---- prefix over the group's tokens (order T, j, i)
    float Lg[2][4];
    float excl[2], all[2];
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
    float mx = -INFINITY;
#pragma unroll
    for (int T = 0; T < 2; ++T)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            Lg[T][i] += excl[T] + (T == 1 ? all[0] : 0.0f);
            if (FULL || 16 * T + 4 * j + i < nval) mx = fmaxf(mx, Lg[T][i]);
        }
    mx = rows_max(mx);
    const float m_g = mx * c2E;

    // ---- V range bias from the group's largest |scale| (slot 0 of the V scale plane)
    const uint32_t *vs0 = (const uint32_t *)(side_b + 6 * D);
    uint32_t vmx = 0;
#pragma unroll
    for (int k = 0; k < NB / 2; ++k) {
        const uint32_t w = vs0[k] & 0x7FFF7FFFu;
        vmx = max(vmx, max(w & 0xFFFFu, w >> 16));
    }
    const int ev = (vmx >> 10) == 0 ? -14 : (int)(vmx >> 10) - 15;
    const int beta_g = vmx == 0 ? 19 : 5 - ev;            // 32 * 16 * |s| * 2^beta < 2^15

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

    // ---- softmax weights and suffix sums
    float S[2][4];
#pragma unroll
    for (int T = 0; T < 2; ++T)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(Lg[T][i], c2E, -m_new));
            S[T][i] = (FULL || 16 * T + 4 * j + i < nval) ? p : 0.0f;
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
    const float Pg = sall[0] + sall[1];
    st.l += Pg;

    // ---- V weights W = S * s * 2^beta * 16/f in hi + lo fp16 (slot 0 = keyframe: weight 0)
    const float bsc = ldexpf(1.0f, st.beta);
    float Sp[2][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float k16 = (i & 1) ? bsc : 16.0f * bsc;
        Sp[1][i] = (S[1][i] + sexcl[1]) * k16;
        Sp[0][i] = (S[0][i] + (sexcl[0] + sall[1])) * k16;
    }
    Sp[0][0] = j == 0 ? 0.0f : Sp[0][0];
    // weights per block pair, then the V MFMAs of the two 16-channel chunks of each block
#pragma unroll
    for (int k = 0; k < NB / 2; ++k) {
        uint32_t vs[2][4];
#pragma unroll
        for (int T = 0; T < 2; ++T) {
            const uint32_t *sp = (const uint32_t *)(side_b + 6 * D + (16 * T + 4 * j) * 2 * NB);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                vs[T][i] = (FULL || 16 * T + 4 * j + i < nval) ? sp[i * (NB / 2) + k] : 0u;
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
                const h8 A = unpack8(r.vc[cc]);
                st.acc[cc] = mfma(A, Wh, st.acc[cc]);
                st.acc[cc] = mfma(A, Wl, st.acc[cc]);
            }
            st.Z[bb] = mfma(AZ, Wh, st.Z[bb]);
            st.Z[bb] = mfma(AZ, Wl, st.Z[bb]);
        }
    }
    // ---- keyframe: acc += P_g * x0 (accumulator units 2^(beta-20))
    const float pk = Pg * ldexpf(1.0f, st.beta - 20);
    const uint32_t *kp = (const uint32_t *)(side_b + 4 * D + j * NCC * 8);
#pragma unroll
    for (int cc = 0; cc < NCC; ++cc) {
        const uint32_t w01 = kp[2 * cc], w23 = kp[2 * cc + 1];
        st.acc[cc][0] = __builtin_fmaf(hlo(w01), pk, st.acc[cc][0]);
        st.acc[cc][1] = __builtin_fmaf(hhi(w01), pk, st.acc[cc][1]);
        st.acc[cc][2] = __builtin_fmaf(hlo(w23), pk, st.acc[cc][2]);
        st.acc[cc][3] = __builtin_fmaf(hhi(w23), pk, st.acc[cc][3]);
    }
}

// kf = 32.  LDS image of a group's side data: [K keyframe][K scales][V keyframe][V scales], 2*D bytes each,
// double-buffered so the next group's data lands while the current one is read.
template <int D>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2)))
    k_attn_fused32(dkv_config cfg, const uint8_t *__restrict__ cache, const int32_t *__restrict__ bt,
                   const float *__restrict__ q, const int32_t *__restrict__ seq_lens, float scale_log2,
                   float *__restrict__ ws, int nsplit, int chunk)
{
    constexpr int NB = D / 32;
    constexpr int NCC = D / 16;
    constexpr int SIDE_LANES = D / 4;
    const Geom g = make_geom(cfg);
    const int split = grid_split(), h = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x, j = lane >> 4, n = lane & 15;
    const int G = g.G;
    const int L = min(seq_lens[b], g.cap_tokens);
    const int ng = (L + 31) >> 5;
    const int g0 = split * chunk, g1 = min(ng, g0 + chunk);

    __shared__ float sq[16][D + 4];
    __shared__ __attribute__((aligned(16))) uint32_t side[2][2 * D];   // 2 x 8*D bytes
    // per lane: query operands (block, hi/lo), the K correction operand (hi, lo) and the V "-8" operand
    __shared__ u4 qB[(2 * NB + 3) * 64];

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

    // K-side operand: q * 2^-E * 16/f in hi + lo fp16, in the code unpack order
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
        qB[(2 * bb) * 64 + lane] = __builtin_bit_cast(u4, Bh[bb]);
        qB[(2 * bb + 1) * 64 + lane] = __builtin_bit_cast(u4, Bl[bb]);
    }
    // correction operand: -8 * Qs[block] at K index = block (lane group 0)
    {
        h8 B2h, B2l;
#pragma unroll
        for (int hh = 0; hh < 8; ++hh) {
            const float x = (j == 0 && hh < NB) ? -8.0f * Qs[hh < NB ? hh : 0] : 0.0f;
            const _Float16 hi = (_Float16)x;
            B2h[hh] = hi;
            B2l[hh] = (_Float16)(x - (float)hi);
        }
        qB[(2 * NB) * 64 + lane] = __builtin_bit_cast(u4, B2h);
        qB[(2 * NB + 1) * 64 + lane] = __builtin_bit_cast(u4, B2l);
        // V "-8" operand: -8 * 2^-24 * f(hh) as fp16 subnormals
        u4 azr;
        azr[0] = 0x80088008u;
        azr[1] = 0x80808080u;
        azr[2] = 0x80088008u;
        azr[3] = 0x80808080u;
        qB[(2 * NB + 2) * 64 + lane] = azr;
    }

    RunState<D> st;
#pragma unroll
    for (int cc = 0; cc < NCC; ++cc) st.acc[cc] = f4{0, 0, 0, 0};
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) st.Z[bb] = f4{0, 0, 0, 0};
    st.m = -INFINITY;
    st.l = 0.0f;
    st.beta = 127;

    const h8 B2hr = as_h8(qB[(2 * NB) * 64 + lane]), B2lr = as_h8(qB[(2 * NB + 1) * 64 + lane]);
    const h8 AZr = as_h8(qB[(2 * NB + 2) * 64 + lane]);
    const LaneOffsets lo = lane_offsets<D>(g, lane, j, n);

    const int rec_bytes = (int)g.rec;
    // first mapped group at or after x (paged mode may leave pages unmapped); uniform
    auto next_mapped = [&](int x, int64_t &o) {
        for (; x < g1; ++x) {
            o = group_offset(g, bt, b, h, x);
            if (o >= 0) break;
        }
        return x;
    };
    // stage a group's side data into LDS buffer `bf`; the K keyframe (lanes < D/8)
    // is scaled by f(hh)/16 here, once, for the keyframe row of the K-side MFMA
    auto stage = [&](const GroupRegs<D> &r, int bf) {
        if (lane < 2 * SIDE_LANES) {
            u4 v = r.side;
            if (lane < D / 8) {
                // (scalar temporaries: bit_cast of a vector element lvalue is miscompiled)
                const uint32_t w0 = v[0], w2 = v[2];
                v[0] = scale_h2_16th(w0);
                v[2] = scale_h2_16th(w2);
            }
            // lane id recomputed here (two VALU ops) rather than kept live across the loop
            ((u4 *)side[bf])[fresh_lane_id()] = v;
        }
    };
    auto run = [&](const GroupRegs<D> &r, int gcur, int bf) {
        __syncthreads();
        const int nval = min(32, L - gcur * 32);
        const uint8_t *sb = (const uint8_t *)side[bf];
        if (nval == 32)
            process_group<D, true>(st, r, sb, nval, j, n, qB, c2E, B2hr, B2lr, AZr);
        else
            process_group<D, false>(st, r, sb, nval, j, n, qB, c2E, B2hr, B2lr, AZr);
    };

    GroupRegs<D> ra, rb;
    int64_t off = -1, offn = -1;
    int gi = next_mapped(g0, off);
    if (gi < g1) load_group<D>(ra, cache + off, rec_bytes, lo);
    // two groups per trip: ra and rb alternate as current / prefetch buffers
    while (gi < g1) {
        int gn = next_mapped(gi + 1, offn);
        stage(ra, 0);
        // prefetch unconditionally so the wait counts stay exact (past the end it
        // re-reads the current record and the values are unused)
        load_group<D>(rb, cache + (gn < g1 ? offn : off), rec_bytes, lo);
        run(ra, gi, 0);
        gi = gn;
        off = offn;
        if (gi >= g1) break;
        gn = next_mapped(gi + 1, offn);
        stage(rb, 1);
        load_group<D>(ra, cache + (gn < g1 ? offn : off), rec_bytes, lo);
        run(rb, gi, 1);
        gi = gn;
        off = offn;
    }

    // ---------------------------------------------------------------- partials
    const int64_t row0 = (int64_t)b * g.Hq + h * G;       // first query head of this kv-head
    if (n < G) {
        float *rec = ws + ((row0 + n) * nsplit + split) * part_stride(D);
        const float un = ldexpf(1.0f, 20 - st.beta);
#pragma unroll
        for (int cc = 0; cc < NCC; ++cc) {
            f4 o;
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = (st.acc[cc][i] + st.Z[cc >> 1][i]) * un;
            *(f4 *)(rec + 16 * cc + 4 * j) = o;
        }
        if (j == 0) {
            rec[D] = st.m;
            rec[D + 1] = st.l;
        }
    }
}

hipError_t launch_attn_fused(const dkv_config &c, const void *cache, const int32_t *bt, const float *q,
                             const int32_t *lens, float scale_log2, float *ws, int nsplit, int chunk, hipStream_t st)
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
