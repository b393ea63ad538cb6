// In-run comparison paths of the Delta-KV article's "벤치마크" section: a
// plain Q4_0 cache of absolute values (the 4-bit baseline) and an F16 cache
// (the unquantised baseline), each with a matrix-core decode-attention kernel
// built like the Delta-KV one (same split-K partials, same combine), so that
// the three are compared on equal footing.
//
// Q4_0 cache (layout in dkv_common.h): exactly 18 bytes per 32 elements,
// laid out for the 16x16x32 fp16 matrix instruction.  With at most 8 query
// heads per kv-head the attention runs on the GQA<=8 kernel family
// (dkv_attn_g8.hip); this file keeps the general 16-column kernel.
#include "dkv_fused_common.h"
#include "dkv_q40.h"

namespace dkv {


// ------------------------------------------------------------------------
// Q4_0 encode: grid (tiles, Hkv*2, B), one wavefront per (tile, stream);
// lanes own channels as in the Delta-KV encoder, the quantiser sees the
// absolute value (reference 0).
// ------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(64) k_q40_encode(dkv_config cfg, uint8_t *q4, const int32_t *bt, const uint16_t *kin,
                                                   const uint16_t *vin, const int32_t *seq_lens, int s_max)
{
    constexpr int NC = D / 64, nb = D / 32;
    const int tile = blockIdx.x, h = blockIdx.y >> 1, s = blockIdx.y & 1, b = blockIdx.z;
    const int L = min(min(seq_lens[b], q40_ntiles(cfg) * 32), s_max);
    const int t0 = tile * 32;
    if (t0 >= L) return;
    const int64_t toff = q40_tile_offset(cfg, bt, b, h, tile);
    if (toff < 0) return;                       // unmapped page
    const int n = min(32, L - t0);
    uint8_t *base = q4 + toff + (s ? 18 * D : 0);
    uint16_t *sc = (uint16_t *)base;
    uint8_t *cd = base + 2 * D;
    const uint16_t *x = (s ? vin : kin) + (((int64_t)b * cfg.n_kv_heads + h) * s_max + t0) * D;
    const int lane = threadIdx.x;

    uint32_t vw[NC][4];
#pragma unroll
    for (int i = 0; i < NC; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) vw[i][j] = 0x88888888u;

    for (int r = 0; r < n; ++r) {
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            const int c = lane + 64 * i;
            const int blk = c >> 5;
            float ref = 0.0f;
            int code;
            uint16_t s16;
            q40_delta_step(h2f(x[(int64_t)r * D + c]), ref, code, s16);
            if ((lane & 31) == 0) sc[r * nb + blk] = s16;
            if (s == 0) {
                store_k_codes<D>(cd + r * (D / 2), blk, code);
            } else {
                const int j = (r & 15) >> 2, sh = 4 * vcode_nibble(r);
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    if (jj == j) vw[i][jj] = (vw[i][jj] & ~(0xFu << sh)) | ((uint32_t)code << sh);
            }
        }
    }
    if (s == 1) {
        uint32_t *tw = (uint32_t *)cd;
#pragma unroll
        for (int i = 0; i < NC; ++i) {
            const int c = lane + 64 * i;
#pragma unroll
            for (int j = 0; j < 4; ++j) tw[vcode_word(D, 4 * j, c, q40_vbp(cfg))] = vw[i][j];
        }
    }
}

// Canonical export: codes uint8 [B][Hkv][2][s_max][D/2] (byte i of a block =
// code i | code i+16 << 4), scales uint16 [B][Hkv][2][s_max][D/32].
// grid (ceil(s_max*D/2 / 256), Hkv*2, B), one thread per output code byte.
template <int D>
__global__ void __launch_bounds__(256) k_q40_export(dkv_config cfg, const uint8_t *q4, const int32_t *bt,
                                                    const int32_t *seq_lens, int s_max, uint8_t *codes,
                                                    uint16_t *scales)
{
    constexpr int nb = D / 32, RB = D / 2;
    const int h = blockIdx.y >> 1, s = blockIdx.y & 1, b = blockIdx.z;
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int t = (int)(e / RB), byte = (int)(e % RB);
    const int L = min(min(seq_lens[b], q40_ntiles(cfg) * 32), s_max);
    if (t >= L) return;
    const int64_t toff = q40_tile_offset(cfg, bt, b, h, t >> 5);
    if (toff < 0) return;                       // unmapped page: the row is left untouched
    const uint8_t *base = q4 + toff + (s ? 18 * D : 0);
    const int tau = t & 31, blk = byte >> 4, i = byte & 15;
    uint8_t out;
    if (s == 0) {
        out = base[2 * D + tau * RB + kcode_byte(nb, blk, i)];
    } else {
        const uint32_t *tw = (const uint32_t *)(base + 2 * D);
        const int sh = 4 * vcode_nibble(tau);
        const int bp = q40_vbp(cfg);
        const uint32_t lo = (tw[vcode_word(D, tau, 32 * blk + i, bp)] >> sh) & 0xFu;
        const uint32_t hi = (tw[vcode_word(D, tau, 32 * blk + i + 16, bp)] >> sh) & 0xFu;
        out = (uint8_t)(lo | (hi << 4));
    }
    const int64_t row = (((int64_t)b * cfg.n_kv_heads + h) * 2 + s) * s_max + t;
    codes[row * RB + byte] = out;
    if (byte < nb) scales[row * nb + byte] = ((const uint16_t *)base)[tau * nb + byte];
}

// ------------------------------------------------------------------------
// Shared set-up of the comparison attention kernels: the query of the G heads
// of one kv-head, scaled by softmax_scale*log2(e) and by 2^-E (E = exponent of
// its largest element), split in hi + lo fp16 as the K-side MFMA operand.
// natural = true: K channels in natural order (F16); false: the Q4_0 code
// unpack order with the 16/f factors (Q4_0).
// ------------------------------------------------------------------------
template <int D, bool NATURAL>
__device__ inline void setup_query(float (*sq)[D + 4], u4 *qB, const float *q, int64_t row0, int G, float scale_log2,
                                   int lane, int j, int n, float &c2E, float *Qs)
{
    constexpr int NB = D / 32;
    for (int i = lane; i < 16 * D; i += 64) {
        const int hh = i / D, c = i % D;
        sq[hh][c] = hh < G ? q[(row0 + hh) * D + c] * scale_log2 : 0.0f;
    }
    __syncthreads();
    float qm = 0.0f;
    for (int c = j * (D / 4); c < (j + 1) * (D / 4); ++c) qm = fmaxf(qm, fabsf(sq[n][c]));
    qm = fmaxf(qm, __shfl_xor(qm, 16));
    qm = fmaxf(qm, __shfl_xor(qm, 32));
    int E = 0;
    if (qm > 0.0f) frexpf(qm, &E);
    const float qscale = ldexpf(1.0f, -E);
    c2E = ldexpf(1.0f, E);
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
        float qsum = 0.0f;
        h8 Bh, Bl;
#pragma unroll
        for (int hh = 0; hh < 8; ++hh) {
            const bool f16x = !NATURAL && ((hh >> 1) & 1) != 0;
            const int ch = NATURAL ? 8 * j + hh : kf_k_channel(j, hh);
            const float x = sq[n][32 * bb + ch] * qscale * ((NATURAL || f16x) ? 1.0f : 16.0f);
            const _Float16 hi = (_Float16)x;
            const _Float16 lo = (_Float16)(x - (float)hi);
            Bh[hh] = hi;
            Bl[hh] = lo;
            qsum += ((float)hi + (float)lo) * ((NATURAL || f16x) ? 1.0f : 0.0625f);
        }
        qsum += __shfl_xor(qsum, 16);
        qsum += __shfl_xor(qsum, 32);
        if (Qs) Qs[bb] = qsum;
        qB[(2 * bb) * 64 + lane] = __builtin_bit_cast(u4, Bh);
        qB[(2 * bb + 1) * 64 + lane] = __builtin_bit_cast(u4, Bl);
    }
}


// ------------------------------------------------------------------------
// Q4_0 decode attention: grid (nsplit, Hkv, B), one wavefront per
// (sequence, kv-head, run of 32-token tiles); lane = 16*j + n.
// Per tile: logits of 32 tokens x 16 heads by MFMA on the raw codes (scale per
// (token, block) applied to the fp32 results, "-8" by one small MFMA), online
// softmax, then P.V by MFMA with the weights p*s*2^beta (hi + lo fp16).
// ------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2)))
    k_attn_q40(dkv_config cfg, const uint8_t *__restrict__ q4, const int32_t *__restrict__ bt,
               const float *__restrict__ q, const int32_t *__restrict__ seq_lens, float scale_log2,
               float *__restrict__ ws, int nsplit, int chunk)
{
    constexpr int NB = D / 32, NCC = D / 16;
    const int split = grid_split(), h = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x, j = lane >> 4, n = lane & 15;
    const int G = cfg.n_q_heads / cfg.n_kv_heads;
    const int ntiles = q40_ntiles(cfg);
    const int L = min(seq_lens[b], ntiles * 32);
    const int nt = (L + 31) >> 5;
    const int t0 = split * chunk, t1 = min(nt, t0 + chunk);
    const int64_t row0 = (int64_t)b * cfg.n_q_heads + h * G;

    __shared__ float sq[16][D + 4];
    __shared__ __attribute__((aligned(16))) uint32_t side[D];      // [K scales 2D bytes][V scales 2D bytes]
    __shared__ u4 qB[2 * NB * 64];

    float Qs[NB];
    float c2E;
    setup_query<D, false>(sq, qB, q, row0, G, scale_log2, lane, j, n, c2E, Qs);
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
    const uint8_t *sb = (const uint8_t *)side;
    const int tb = (int)q40_tile_bytes(D);

    for (int tl = t0; tl < t1; ++tl) {
        const int64_t toff = q40_tile_offset(cfg, bt, b, h, tl);
        if (toff < 0) continue;                 // unmapped page: its tokens are not attended
        const uint8_t *tp = q4 + toff;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void *)tp, (short)0, tb, 0x00020000);
        const int nvt = min(32, L - 32 * tl);
        __syncthreads();
        if (lane < D / 8)
            ((u4 *)side)[lane] = __builtin_amdgcn_raw_buffer_load_b128(rs, 16 * lane, 0, kStream);
        else if (lane < D / 4)
            ((u4 *)side)[lane] = __builtin_amdgcn_raw_buffer_load_b128(rs, 18 * D + 16 * (lane - D / 8), 0, kStream);
        uint32_t kc[2][NB];
#pragma unroll
        for (int T = 0; T < 2; ++T) {
            const int off = 2 * D + (16 * T + n) * (D / 2) + 4 * j * NB;
            if constexpr (NB == 4) {
                const u4 a = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kStream);
#pragma unroll
                for (int k = 0; k < 4; ++k) kc[T][k] = a[k];
            } else {
                const u2 a = __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, kStream);
#pragma unroll
                for (int k = 0; k < 2; ++k) kc[T][k] = a[k];
            }
        }
        uint32_t vc[NCC];
#pragma unroll
        for (int q4i = 0; q4i < NCC / 4; ++q4i) {
            const u4 a = __builtin_amdgcn_raw_buffer_load_b128(rs, 20 * D + vcode_piece(D, j * 16 + n, q4i), 0, kStream);
#pragma unroll
            for (int k = 0; k < 4; ++k) vc[4 * q4i + k] = a[k];
        }
        __syncthreads();

        // ---- logits
        float Lg[2][4];
#pragma unroll
        for (int T = 0; T < 2; ++T) {
            uint32_t sg[4][NB / 2];
            const uint32_t *sp = (const uint32_t *)(sb + (16 * T + 4 * j) * 2 * NB);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int k = 0; k < NB / 2; ++k) sg[i][k] = sp[i * (NB / 2) + k];
            f4 u = f4{0, 0, 0, 0};
#pragma unroll
            for (int bb = 0; bb < NB; ++bb) {
                const h8 A = unpack8(kc[T][bb]);
                const h8 bh = as_h8(qB[(2 * bb) * 64 + lane]);
                const h8 bl = as_h8(qB[(2 * bb + 1) * 64 + lane]);
                f4 P = mfma(A, bh, f4{0, 0, 0, 0});
                P = mfma(A, bl, P);
#pragma unroll
                for (int i = 0; i < 4; ++i) u[i] = __builtin_fmaf(half_at(sg[i], bb), P[i], u[i]);
            }
            u4 a2 = u4{0, 0, 0, 0};
            {
                const uint32_t *ap = (const uint32_t *)(sb + (16 * T + n) * 2 * NB);
#pragma unroll
                for (int k = 0; k < NB / 2; ++k) a2[k] = j == 0 ? ap[k] : 0u;
            }
            f4 C2 = mfma(as_h8(a2), B2h, f4{0, 0, 0, 0});
            C2 = mfma(as_h8(a2), B2l, C2);
#pragma unroll
            for (int i = 0; i < 4; ++i) Lg[T][i] = __builtin_fmaf(u[i], 1048576.0f, C2[i]);
        }
        float mx = -INFINITY;
#pragma unroll
        for (int T = 0; T < 2; ++T)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (16 * T + 4 * j + i < nvt) mx = fmaxf(mx, Lg[T][i]);
        mx = rows_max(mx);
        const float m_new = fmaxf(st.m, mx * c2E);

        // ---- V scales of this lane's 8 tokens (invalid tokens: 0) and the tile's max |scale|
        uint32_t vs[2][4][NB / 2];
        uint32_t vmx2 = 0;
#pragma unroll
        for (int T = 0; T < 2; ++T) {
            const uint32_t *sp = (const uint32_t *)(sb + 2 * D + (16 * T + 4 * j) * 2 * NB);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int k = 0; k < NB / 2; ++k) {
                    const uint32_t w = (16 * T + 4 * j + i < nvt) ? sp[i * (NB / 2) + k] : 0u;
                    vs[T][i][k] = w;
                    const uint32_t a = w & 0x7FFF7FFFu;
                    vmx2 = max(vmx2, max(a & 0xFFFFu, a >> 16));
                }
        }
        const int vmx = (int)rows_max((float)vmx2);
        const int ev = (vmx >> 10) == 0 ? -14 : (vmx >> 10) - 15;
        const int beta_g = vmx == 0 ? 127 : 10 - ev;                      // 16 * |s| * 2^beta < 2^15
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

        // ---- weights
        float p[2][4];
        float ps = 0.0f;
#pragma unroll
        for (int T = 0; T < 2; ++T)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(Lg[T][i], c2E, -m_new));
                p[T][i] = (16 * T + 4 * j + i < nvt) ? e : 0.0f;
                ps += p[T][i];
            }
        st.l += rows_sum(ps);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float k16 = (i & 1) ? bsc : 16.0f * bsc;
            p[0][i] *= k16;
            p[1][i] *= k16;
        }
#pragma unroll
        for (int k = 0; k < NB / 2; ++k) {
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int bb = 2 * k + e;
                h8 Wh, Wl;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float s0 = e ? hhi(vs[0][i][k]) : hlo(vs[0][i][k]);
                    const float s1 = e ? hhi(vs[1][i][k]) : hlo(vs[1][i][k]);
                    const _Float16 h0 = (_Float16)__builtin_fmaf(s0, p[0][i], 0.0f);
                    const _Float16 h1 = (_Float16)__builtin_fmaf(s1, p[1][i], 0.0f);
                    Wh[2 * i] = h0;
                    Wh[2 * i + 1] = h1;
                    Wl[2 * i] = (_Float16)__builtin_fmaf(s0, p[0][i], -(float)h0);
                    Wl[2 * i + 1] = (_Float16)__builtin_fmaf(s1, p[1][i], -(float)h1);
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

    if (n < G) {
        float *recp = ws + ((row0 + n) * nsplit + split) * part_stride(D);
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

// ------------------------------------------------------------------------
// F16 decode attention over token-major fp16 K/V [B][Hkv][s_max][D]:
// grid (nsplit, Hkv, B), one wavefront per (sequence, kv-head, run of tiles).
// K side: the 16-byte K row pieces are the MFMA A operand as loaded.  V side:
// lane (j, n) loads channels n*CPL..n*CPL+CPL-1 of its 8 tokens 16T+4j+i and
// regroups them (v_perm) into one A operand per channel offset r, so that MFMA
// r yields channels m*CPL + r; weights p*2^14 in hi + lo fp16.
// ------------------------------------------------------------------------
__device__ inline uint32_t pack_lo16(uint32_t a, uint32_t b) { return (a & 0xFFFFu) | (b << 16); }
__device__ inline uint32_t pack_hi16(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xFFFF0000u); }

// The fp16 cache streams with no cache line shared between loads; the
// nontemporal hint took the 70B-layer split kernel from 368 to 313 us.
constexpr int kStreamF16 = 2;

template <int D>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2)))
    k_attn_f16(dkv_config cfg, const uint16_t *__restrict__ kin, const uint16_t *__restrict__ vin,
               const int32_t *__restrict__ bt, const float *__restrict__ q, const int32_t *__restrict__ seq_lens,
               float scale_log2, float *__restrict__ ws, int nsplit, int chunk)
{
    constexpr int NB = D / 32;
    constexpr int CPL = D / 16;             // channels per lane per V token load
    constexpr int VW = CPL / 2;             // dwords per V load
    const int split = grid_split(), h = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x, j = lane >> 4, n = lane & 15;
    const int G = cfg.n_q_heads / cfg.n_kv_heads;
    const int L = min(seq_lens[b], cmp_ntiles(cfg) * 32);
    const int nt = (L + 31) >> 5;
    const int t0 = split * chunk, t1 = min(nt, t0 + chunk);
    const int64_t row0 = (int64_t)b * cfg.n_q_heads + h * G;
    if (t0 >= nt) return;                  // past the sequence's end: no record (the combine skips it)

    __shared__ float sq[16][D + 4];
    __shared__ u4 qB[2 * NB * 64];
    float c2E;
    setup_query<D, true>(sq, qB, q, row0, G, scale_log2, lane, j, n, c2E, nullptr);

    f4 acc[CPL];
#pragma unroll
    for (int r = 0; r < CPL; ++r) acc[r] = f4{0, 0, 0, 0};
    float m = -INFINITY, l = 0.0f;

    // Software pipeline over the run's mapped tiles: the next tile's K rows are
    // fetched (into the other of two K buffers) before the current tile's
    // logits, its V rows as soon as the current V rows have gone into the
    // matrix instructions.  Past the run (or where only unmapped tiles follow)
    // the current tile is fetched again (an L2 hit) and not used.
    struct KRegs {
        u4 kr[2][NB];
    };
    struct VRegs {
        uint32_t vr[2][4][VW];
    };
    auto next_mapped = [&](int t, int64_t &e) {
        for (; t < t1; ++t) {
            e = f16_tile_elem(cfg, bt, b, h, t);
            if (e >= 0) break;                  // unmapped page: its tokens are not attended
        }
        return t;
    };
    // the tile's rows (contiguous: up to the end of the stream; loads past it return 0)
    auto tile_rsrc = [&](const uint16_t *base, int tl, int64_t e0) {
        const int bytes = (cfg.page_tokens > 0 ? 32 : min(32, cfg.max_tokens - 32 * tl)) * D * 2;
        return __builtin_amdgcn_make_buffer_rsrc((void *)(base + e0), (short)0, bytes, 0x00020000);
    };
    auto load_k = [&](KRegs &r, int tl, int64_t e0) {
        const __amdgpu_buffer_rsrc_t rk = tile_rsrc(kin, tl, e0);
#pragma unroll
        for (int T = 0; T < 2; ++T)
#pragma unroll
            for (int bb = 0; bb < NB; ++bb)
                r.kr[T][bb] =
                    __builtin_amdgcn_raw_buffer_load_b128(rk, ((16 * T + n) * D + 32 * bb + 8 * j) * 2, 0, kStreamF16);
    };
    auto load_v = [&](VRegs &r, int tl, int64_t e0) {
        const __amdgpu_buffer_rsrc_t rv = tile_rsrc(vin, tl, e0);
#pragma unroll
        for (int T = 0; T < 2; ++T)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int off = ((16 * T + 4 * j + i) * D + CPL * n) * 2;
                if constexpr (VW == 4) {
                    const u4 a = __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, kStreamF16);
#pragma unroll
                    for (int k = 0; k < 4; ++k) r.vr[T][i][k] = a[k];
                } else {
                    const u2 a = __builtin_amdgcn_raw_buffer_load_b64(rv, off, 0, kStreamF16);
#pragma unroll
                    for (int k = 0; k < 2; ++k) r.vr[T][i][k] = a[k];
                }
            }
    };
    // tile tl from K rows rk and V rows r; then the V rows of tile tn (at e_n)
    // are fetched into r
    auto compute_tile = [&](const KRegs &rk, VRegs &r, int tl, int tn, int64_t e_n) {
        const int nvt = min(32, L - 32 * tl);
        // ---- logits (units: q * 2^-E)
        float Lg[2][4];
#pragma unroll
        for (int T = 0; T < 2; ++T) {
            f4 P = f4{0, 0, 0, 0};
#pragma unroll
            for (int bb = 0; bb < NB; ++bb) {
                const h8 A = as_h8(rk.kr[T][bb]);
                P = mfma(A, as_h8(qB[(2 * bb) * 64 + lane]), P);
                P = mfma(A, as_h8(qB[(2 * bb + 1) * 64 + lane]), P);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) Lg[T][i] = P[i];
        }
        float mx = -INFINITY;
#pragma unroll
        for (int T = 0; T < 2; ++T)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (16 * T + 4 * j + i < nvt) mx = fmaxf(mx, Lg[T][i]);
        mx = rows_max(mx);
        const float m_new = fmaxf(m, mx * c2E);
        const float a_m = __builtin_amdgcn_exp2f(m - m_new);
        if (__any(m_new != m)) {
#pragma unroll
            for (int c = 0; c < CPL; ++c) acc[c] *= a_m;
            l *= a_m;
        }
        m = m_new;

        // ---- weights p * 2^14, hi + lo fp16, in the operand order 2i + T
        h8 Wh, Wl;
        float ps = 0.0f;
#pragma unroll
        for (int T = 0; T < 2; ++T)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool ok = 16 * T + 4 * j + i < nvt;
                const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(Lg[T][i], c2E, -m_new));
                const float p = ok ? e : 0.0f;
                ps += p;
                const float w = p * 16384.0f;
                const _Float16 hi = (_Float16)w;
                Wh[2 * i + T] = hi;
                Wl[2 * i + T] = (_Float16)(w - (float)hi);
                if (!ok) {
#pragma unroll
                    for (int k = 0; k < VW; ++k) r.vr[T][i][k] = 0u;      // rows past the end may hold non-finite values
                }
            }
        l += rows_sum(ps);

        // ---- V operands per channel offset c, then P.V
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            u4 a;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t w0 = r.vr[0][i][c >> 1], w1 = r.vr[1][i][c >> 1];
                a[i] = (c & 1) ? pack_hi16(w0, w1) : pack_lo16(w0, w1);
            }
            acc[c] = mfma(as_h8(a), Wh, acc[c]);
            acc[c] = mfma(as_h8(a), Wl, acc[c]);
        }
        load_v(r, tn, e_n);
    };

    int64_t e_cur = -1;
    int tl = next_mapped(t0, e_cur);
    if (tl < t1) {
        KRegs ka, kb;
        VRegs vr;
        load_k(ka, tl, e_cur);
        load_v(vr, tl, e_cur);
        // one step: the next mapped tile's K into pf, then tile tl
        auto step = [&](const KRegs &cur, KRegs &pf) {
            int64_t e_n = -1;
            const int tn = next_mapped(tl + 1, e_n);
            const bool more = tn < t1;
            load_k(pf, more ? tn : tl, more ? e_n : e_cur);
            compute_tile(cur, vr, tl, more ? tn : tl, more ? e_n : e_cur);
            tl = tn;
            e_cur = e_n;
            return more;
        };
        while (step(ka, kb) && step(kb, ka)) {
        }
    }

    if (n < G) {
        float *recp = ws + ((row0 + n) * nsplit + split) * part_stride(D);
#pragma unroll
        for (int r = 0; r < CPL; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) recp[(4 * j + i) * CPL + r] = acc[r][i] * (1.0f / 16384.0f);
        if (j == 0) {
            recp[D] = m;
            recp[D + 1] = l;
        }
    }
}

// ------------------------------------------------------------------------
// Plain Q8_0 of absolute values (quality comparison only): the 8-bit reference
// of the Delta-KV article's "벤치마크" section.  Per block of 32 values:
// d = max|v| / 127, code = round-half-away-from-zero(v * (1/d)), scale fp16(d).
// One wavefront per run of kQ80Tokens tokens of a (sequence, kv-head, stream);
// each 32-lane half takes one block.  Writes the canonical arrays directly:
// codes int8 [B][Hkv][2][s_max][D], scales fp16 [B][Hkv][2][s_max][D/32].
// ------------------------------------------------------------------------
constexpr int kQ80Tokens = 16;

template <int D>
__global__ void __launch_bounds__(64) k_q80_encode(dkv_config cfg, const uint16_t *__restrict__ k,
                                                   const uint16_t *__restrict__ v, const int32_t *__restrict__ lens,
                                                   int s_max, int8_t *__restrict__ codes,
                                                   uint16_t *__restrict__ scales)
{
    const int h = blockIdx.y >> 1, s = blockIdx.y & 1, b = blockIdx.z;
    const int lane = threadIdx.x;
    const int L = min(lens[b], s_max);
    const int t0 = blockIdx.x * kQ80Tokens, t1 = min(L, t0 + kQ80Tokens);
    const int64_t row = (((int64_t)b * cfg.n_kv_heads + h) * 2 + s) * s_max;
    const uint16_t *x = (s ? v : k) + ((int64_t)b * cfg.n_kv_heads + h) * s_max * D;
    for (int t = t0; t < t1; ++t) {
#pragma unroll
        for (int i = 0; i < D / 64; ++i) {
            const int c = 64 * i + lane;
            const float val = h2f(x[(int64_t)t * D + c]);
            float amax = fabsf(val);
#pragma unroll
            for (int o = 16; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 32));
            const float d = amax / 127.0f;
            const float id = d != 0.0f ? 1.0f / d : 0.0f;
            codes[(row + t) * D + c] = (int8_t)roundf(val * id);
            if ((lane & 31) == 0) scales[(row + t) * (D / 32) + (c >> 5)] = f2h_rn(d);
        }
    }
}

// ------------------------------------------------------------------------
// Q4-keyframe variant (Delta-KV article, "벤치마크": the same 4-bit storage as
// Q4_0).  The cache is the plain Q4_0 tile layout; token t is one Q4_0 row,
// coded against zero at a keyframe (t % kf == 0) and against the running
// reconstruction otherwise, with the block quantiser of the Delta-KV codec.
// kf divides 32 or is a multiple of 32, so every group lies in whole tiles.
// ------------------------------------------------------------------------
__host__ __device__ inline int q4k_tiles_per_segment(int kf) { return kf >= 32 ? kf / 32 : 1; }

// One Q4-keyframe row of a stream: lane = channel mod 64 (NC channels per
// lane), xh the lanes' reconstruction of the previous token; writes the row's
// scales and K codes into the tile at `base` (the stream's part), slot tau.
// V codes: into the lane's tile words vw (the bulk encoder writes whole words
// per tile, unused slots holding code 8), or with RMW read-modify-write of the
// word in the cache (the append).
template <int D, bool RMW>
__device__ inline void q4k_row(const dkv_config &cfg, uint8_t *base, int s, int tau, bool key, const uint16_t *x,
                               float (&xh)[D / 64], uint32_t (&vw)[D / 64][4], int lane)
{
    constexpr int NC = D / 64, nb = D / 32;
    uint16_t *sc = (uint16_t *)base;
    uint8_t *cd = base + 2 * D;
    const int sh = 4 * vcode_nibble(tau);
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        const int c = lane + 64 * i;
        const int blk = c >> 5;
        float ref = key ? 0.0f : xh[i];
        int code;
        uint16_t s16;
        q40_delta_step(h2f(x[c]), ref, code, s16);
        if ((lane & 31) == 0) sc[tau * nb + blk] = s16;
        if (s == 0) {
            store_k_codes<D>(cd + tau * (D / 2), blk, code);
        } else if constexpr (RMW) {
            uint32_t *w = (uint32_t *)cd + vcode_word(D, tau, c, q40_vbp(cfg));
            *w = (*w & ~(0xFu << sh)) | ((uint32_t)code << sh);
        } else {
            const int j = (tau & 15) >> 2;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                if (jj == j) vw[i][jj] = (vw[i][jj] & ~(0xFu << sh)) | ((uint32_t)code << sh);
        }
        xh[i] = ref;
    }
}

// Bulk encode.  grid (segments, Hkv*2, B): a segment is one tile when kf
// divides 32 and one group (kf/32 tiles) otherwise; one wave per segment and
// stream, rows in order.  The segment holding a sequence's last token writes
// the reconstruction state.
template <int D>
__global__ void __launch_bounds__(64) k_q4k_encode(dkv_config cfg, uint8_t *q4, float *state, const int32_t *bt,
                                                   const uint16_t *kin, const uint16_t *vin, const int32_t *seq_lens,
                                                   int s_max)
{
    constexpr int NC = D / 64;
    const int seg = blockIdx.x, h = blockIdx.y >> 1, s = blockIdx.y & 1, b = blockIdx.z;
    const int L = min(min(seq_lens[b], q40_ntiles(cfg) * 32), s_max);
    const int tps = q4k_tiles_per_segment(cfg.kf);
    const int lane = threadIdx.x;
    const uint16_t *xs = (s ? vin : kin) + ((int64_t)b * cfg.n_kv_heads + h) * s_max * D;
    float xh[NC];
#pragma unroll
    for (int i = 0; i < NC; ++i) xh[i] = 0.0f;
    for (int tile = seg * tps; tile < (seg + 1) * tps && tile * 32 < L; ++tile) {
        const int64_t toff = q40_tile_offset(cfg, bt, b, h, tile);
        if (toff < 0) return;                   // unmapped page (a page holds whole groups)
        uint8_t *base = q4 + toff + (s ? 18 * D : 0);
        const int n = min(32, L - tile * 32);
        uint32_t vw[NC][4];
#pragma unroll
        for (int i = 0; i < NC; ++i)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) vw[i][jj] = 0x88888888u;
        for (int r = 0; r < n; ++r) {
            const int t = tile * 32 + r;
            q4k_row<D, false>(cfg, base, s, r, t % cfg.kf == 0, xs + (int64_t)t * D, xh, vw, lane);
        }
        if (s == 1) {
            uint32_t *tw = (uint32_t *)(base + 2 * D);
#pragma unroll
            for (int i = 0; i < NC; ++i)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) tw[vcode_word(D, 4 * jj, lane + 64 * i, q40_vbp(cfg))] = vw[i][jj];
        }
        if (tile * 32 + n == L) {
            float *st = state + (((int64_t)b * cfg.n_kv_heads + h) * 2 + s) * D;
#pragma unroll
            for (int i = 0; i < NC; ++i) st[lane + 64 * i] = xh[i];
        }
    }
}

// Append one token per sequence at positions[b] (negative: skipped).
// grid (Hkv*2, B), one wave per (sequence, kv-head, stream).
template <int D>
__global__ void __launch_bounds__(64) k_q4k_append(dkv_config cfg, uint8_t *q4, float *state, const int32_t *bt,
                                                   const uint16_t *knew, const uint16_t *vnew,
                                                   const int32_t *positions)
{
    constexpr int NC = D / 64;
    const int h = blockIdx.x >> 1, s = blockIdx.x & 1, b = blockIdx.y;
    const int pos = positions[b];
    if (pos < 0 || pos >= q40_ntiles(cfg) * 32) return;
    const int64_t toff = q40_tile_offset(cfg, bt, b, h, pos >> 5);
    if (toff < 0) return;
    const int lane = threadIdx.x;
    float *st = state + (((int64_t)b * cfg.n_kv_heads + h) * 2 + s) * D;
    float xh[NC];
    uint32_t vw[NC][4];                         // (unused: the append rewrites words in place)
#pragma unroll
    for (int i = 0; i < NC; ++i) xh[i] = st[lane + 64 * i];
    q4k_row<D, true>(cfg, q4 + toff + (s ? 18 * D : 0), s, pos & 31, pos % cfg.kf == 0,
                     (s ? vnew : knew) + ((int64_t)b * cfg.n_kv_heads + h) * D, xh, vw, lane);
#pragma unroll
    for (int i = 0; i < NC; ++i) st[lane + 64 * i] = xh[i];
}

// Reconstruction of every token t < seq_lens[b] (rows in order per segment):
// out_k, out_v float [B][Hkv][s_max][D].
template <int D>
__global__ void __launch_bounds__(64) k_q4k_reconstruct(dkv_config cfg, const uint8_t *q4, const int32_t *bt,
                                                        const int32_t *seq_lens, int s_max, float *ok, float *ov)
{
    constexpr int NC = D / 64, nb = D / 32;
    const int seg = blockIdx.x, h = blockIdx.y >> 1, s = blockIdx.y & 1, b = blockIdx.z;
    const int L = min(min(seq_lens[b], q40_ntiles(cfg) * 32), s_max);
    const int tps = q4k_tiles_per_segment(cfg.kf);
    const int lane = threadIdx.x;
    const int bp = q40_vbp(cfg);
    float *out = (s ? ov : ok) + ((int64_t)b * cfg.n_kv_heads + h) * s_max * D;
    float xh[NC];
#pragma unroll
    for (int i = 0; i < NC; ++i) xh[i] = 0.0f;
    for (int tile = seg * tps; tile < (seg + 1) * tps && tile * 32 < L; ++tile) {
        const int64_t toff = q40_tile_offset(cfg, bt, b, h, tile);
        if (toff < 0) return;
        const uint8_t *base = q4 + toff + (s ? 18 * D : 0);
        const uint16_t *sc = (const uint16_t *)base;
        const uint8_t *cd = base + 2 * D;
        const int n = min(32, L - tile * 32);
        for (int r = 0; r < n; ++r) {
            const int t = tile * 32 + r;
            const bool key = t % cfg.kf == 0;
#pragma unroll
            for (int i = 0; i < NC; ++i) {
                const int c = lane + 64 * i, blk = c >> 5, w = c & 31;
                int code;
                if (s == 0) {
                    const uint8_t byte = cd[r * (D / 2) + kcode_byte(nb, blk, w & 15)];
                    code = w < 16 ? (byte & 0xF) : (byte >> 4);
                } else {
                    code = (((const uint32_t *)cd)[vcode_word(D, r, c, bp)] >> (4 * vcode_nibble(r))) & 0xF;
                }
                const float ref = key ? 0.0f : xh[i];
                xh[i] = __fadd_rn(ref, __fmul_rn((float)(code - 8), h2f(sc[r * nb + blk])));
                out[(int64_t)t * D + c] = xh[i];
            }
        }
    }
}

// ------------------------------------------------------------------------
// Launchers
// ------------------------------------------------------------------------
hipError_t launch_q40_encode(const dkv_config &c, void *q4, const int32_t *bt, const uint16_t *k, const uint16_t *v,
                             const int32_t *lens, int s_max, hipStream_t st)
{
    const int tiles = min(q40_ntiles(c), (s_max + 31) / 32);
    dim3 grid(tiles, c.n_kv_heads * 2, c.batch);
    if (c.head_dim == 64)
        hipLaunchKernelGGL(k_q40_encode<64>, grid, dim3(64), 0, st, c, (uint8_t *)q4, bt, k, v, lens, s_max);
    else
        hipLaunchKernelGGL(k_q40_encode<128>, grid, dim3(64), 0, st, c, (uint8_t *)q4, bt, k, v, lens, s_max);
    return hipGetLastError();
}

hipError_t launch_q80_encode(const dkv_config &c, const uint16_t *k, const uint16_t *v, const int32_t *lens,
                             int s_max, int8_t *codes, uint16_t *scales, hipStream_t st)
{
    dim3 grid((s_max + kQ80Tokens - 1) / kQ80Tokens, c.n_kv_heads * 2, c.batch);
    if (c.head_dim == 64)
        hipLaunchKernelGGL(k_q80_encode<64>, grid, dim3(64), 0, st, c, k, v, lens, s_max, codes, scales);
    else
        hipLaunchKernelGGL(k_q80_encode<128>, grid, dim3(64), 0, st, c, k, v, lens, s_max, codes, scales);
    return hipGetLastError();
}

hipError_t launch_q40_export(const dkv_config &c, const void *q4, const int32_t *bt, const int32_t *lens, int s_max,
                             uint8_t *codes, uint16_t *scales, hipStream_t st)
{
    const int64_t per = (int64_t)s_max * (c.head_dim / 2);
    dim3 grid((unsigned)((per + 255) / 256), c.n_kv_heads * 2, c.batch);
    if (c.head_dim == 64)
        hipLaunchKernelGGL(k_q40_export<64>, grid, dim3(256), 0, st, c, (const uint8_t *)q4, bt, lens, s_max, codes,
                           scales);
    else
        hipLaunchKernelGGL(k_q40_export<128>, grid, dim3(256), 0, st, c, (const uint8_t *)q4, bt, lens, s_max, codes,
                           scales);
    return hipGetLastError();
}

hipError_t launch_attn_q40_g8(const dkv_config &c, const void *q4, const int32_t *bt, const float *q,
                              const int32_t *lens, float scale_log2, float *ws, int nsplit, int chunk, hipStream_t st,
                              bool delta);

hipError_t launch_attn_q40(const dkv_config &c, const void *q4, const int32_t *bt, const float *q, const int32_t *lens,
                           float scale_log2, float *ws, int nsplit, int chunk, hipStream_t st)
{
    if (q40_vbp(c)) return launch_attn_q40_g8(c, q4, bt, q, lens, scale_log2, ws, nsplit, chunk, st, false);
    dim3 grid(nsplit, c.n_kv_heads, c.batch);
    if (c.head_dim == 64)
        hipLaunchKernelGGL(k_attn_q40<64>, grid, dim3(64), 0, st, c, (const uint8_t *)q4, bt, q, lens, scale_log2, ws,
                           nsplit, chunk);
    else
        hipLaunchKernelGGL(k_attn_q40<128>, grid, dim3(64), 0, st, c, (const uint8_t *)q4, bt, q, lens, scale_log2,
                           ws, nsplit, chunk);
    return hipGetLastError();
}

hipError_t launch_attn_f16(const dkv_config &c, const uint16_t *k, const uint16_t *v, const int32_t *bt,
                           const float *q, const int32_t *lens, float scale_log2, float *ws, int nsplit, int chunk,
                           hipStream_t st)
{
    dim3 grid(nsplit, c.n_kv_heads, c.batch);
    if (c.head_dim == 64)
        hipLaunchKernelGGL(k_attn_f16<64>, grid, dim3(64), 0, st, c, k, v, bt, q, lens, scale_log2, ws, nsplit,
                           chunk);
    else
        hipLaunchKernelGGL(k_attn_f16<128>, grid, dim3(64), 0, st, c, k, v, bt, q, lens, scale_log2, ws, nsplit,
                           chunk);
    return hipGetLastError();
}

static int q4k_segments(const dkv_config &c, int s_max)
{
    const int tiles = min(q40_ntiles(c), (s_max + 31) / 32);
    const int tps = q4k_tiles_per_segment(c.kf);
    return (tiles + tps - 1) / tps;
}

hipError_t launch_q4k_encode(const dkv_config &c, void *q4, float *state, const int32_t *bt, const uint16_t *k,
                             const uint16_t *v, const int32_t *lens, int s_max, hipStream_t st)
{
    dim3 grid(q4k_segments(c, s_max), c.n_kv_heads * 2, c.batch);
    if (c.head_dim == 64)
        hipLaunchKernelGGL(k_q4k_encode<64>, grid, dim3(64), 0, st, c, (uint8_t *)q4, state, bt, k, v, lens, s_max);
    else
        hipLaunchKernelGGL(k_q4k_encode<128>, grid, dim3(64), 0, st, c, (uint8_t *)q4, state, bt, k, v, lens, s_max);
    return hipGetLastError();
}

hipError_t launch_q4k_append(const dkv_config &c, void *q4, float *state, const int32_t *bt, const uint16_t *k,
                             const uint16_t *v, const int32_t *pos, hipStream_t st)
{
    dim3 grid(c.n_kv_heads * 2, c.batch);
    if (c.head_dim == 64)
        hipLaunchKernelGGL(k_q4k_append<64>, grid, dim3(64), 0, st, c, (uint8_t *)q4, state, bt, k, v, pos);
    else
        hipLaunchKernelGGL(k_q4k_append<128>, grid, dim3(64), 0, st, c, (uint8_t *)q4, state, bt, k, v, pos);
    return hipGetLastError();
}

hipError_t launch_q4k_reconstruct(const dkv_config &c, const void *q4, const int32_t *bt, const int32_t *lens,
                                  int s_max, float *ok, float *ov, hipStream_t st)
{
    dim3 grid(q4k_segments(c, s_max), c.n_kv_heads * 2, c.batch);
    if (c.head_dim == 64)
        hipLaunchKernelGGL(k_q4k_reconstruct<64>, grid, dim3(64), 0, st, c, (const uint8_t *)q4, bt, lens, s_max, ok,
                           ov);
    else
        hipLaunchKernelGGL(k_q4k_reconstruct<128>, grid, dim3(64), 0, st, c, (const uint8_t *)q4, bt, lens, s_max, ok,
                           ov);
    return hipGetLastError();
}

// Decode attention over the Q4-keyframe cache: kf = 1 is plain Q4_0 (the
// plain kernel); kf = 32 the same kernel with prefix / suffix sums per tile.
hipError_t launch_attn_q4k(const dkv_config &c, const void *q4, const int32_t *bt, const float *q,
                           const int32_t *lens, float scale_log2, float *ws, int nsplit, int chunk, hipStream_t st)
{
    return launch_attn_q40_g8(c, q4, bt, q, lens, scale_log2, ws, nsplit, chunk, st, c.kf == 32);
}

}  // namespace dkv
