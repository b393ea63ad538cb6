// Matrix-core fused decode attention for GQA groups of at most 8 query heads
// per kv-head: the same delta-domain arithmetic as the general kernels
// (Delta-KV article, "핵심 아이디어"; attention as in "KV 캐시 벡터 양자화와 주의
// 보존 변환", "왜 복원 오차가 틀린 기준인가"), laid out so that the 8 operand
// columns such a group leaves free do useful work instead of padding.
//
// Lane = 16*j + n, column n = 8*h2 + hq: column half h2 in {0,1}, head hq.
//  K side: the two 16-token halves T of a 32-token tile go to the two column
//    halves.  The query operand of half T sits in columns 8T..8T+7 (zeros
//    elsewhere), so the four matrix instructions of a block (T = 0,1 x hi/lo
//    query) accumulate into one result whose column half h2 holds the logits of
//    tokens 16*h2 + row.  Every per-token step (scales, prefix sums, softmax
//    weights) then runs on 4 tokens per lane instead of 8.
//  V side: the V code tile rows are in block-pair order (rows 0..7 from block
//    p, rows 8..15 from block p + nb/2).  Column half h2 carries the weights of
//    block p + h2*nb/2, so one operand serves both blocks of a pair and every
//    lane forms the weights of one block instead of two; only the matching
//    (row half, column half) results are kept.
// Two kernels: kf = 32 (one tile per group, two groups in flight) and
// kf = 32*NT, NT = 2..16 (a K pass over the tiles keeps the prefix logits in
// LDS, a V pass runs over them in reverse carrying the suffix sums).
#include "dkv_append.h"
#include "dkv_fused_common.h"

namespace dkv {


bool fused_g8_supported(const dkv_config &c) { return vbp_layout(c) != 0 && c.kf == 32; }
bool fused_long_g8_supported(const dkv_config &c) { return vbp_layout(c) != 0 && c.kf > 32 && c.kf <= 512; }

// LDS images of the query-side operands, shared by all groups of a workgroup.
// Entry e = 8*j + hq of each image holds lane (j, n)'s operand for head hq; a
// lane of the other column half reads the all-zero image at the same index.
template <int D>
struct G8Shared {
    u4 qk[2 * (D / 32) * 32];   // query (block bb, hi/lo) at (2*bb + hl)*32 + e
    u4 qc[2 * 32];              // "-8" correction operand (hi/lo) at hl*32 + e
    u4 qz[2 * (D / 32) * 32];   // zeros
};

// LDS operand addresses of one lane, per token half T.
struct G8Ops {
    const u4 *qk[2];   // + (2*bb + hl) * 32
    const u4 *qc[2];   // + hl * 32
};

// The query elements of head n & 7 of the kv-head's group (rows row0 ..) that
// lane (j, n) prepares, in the K-code unpack order: the blocks of column half
// h2 = n >> 3 (blocks h2*NB/2 .. h2*NB/2 + NB/2 - 1), so that the two halves
// share the set-up.  Lanes of heads beyond the group read head 0 (every load
// is unconditional, so they all go out together) and setup_g8 zeroes them.
template <int D>
__device__ inline void load_q_g8(float (&xq)[D / 64][8], const float *q, int64_t row0, int G, int j, int n)
{
    constexpr int NH = D / 64;
    const int hq = n & 7, bb0 = (n >> 3) * NH;
    const float *qr = q + (row0 + (hq < G ? hq : 0)) * D;
#pragma unroll
    for (int k = 0; k < NH; ++k)
#pragma unroll
        for (int hh = 0; hh < 8; ++hh) xq[k][hh] = qr[32 * (bb0 + k) + kf_k_channel(j, hh)];
}

// Query set-up from load_q_g8's elements: head hq's query scaled by
// softmax_scale*log2(e) and by 2^-E (E = exponent of its largest element),
// split in hi + lo fp16 in the K-code unpack order with the 16/f factors; the
// "-8" operand -8*sum(q) per block.  Each column half prepares the operands of
// its own blocks (the head's maximum and the block sums are exchanged between
// the halves).  Returns 2^E.
template <int D>
__device__ inline float setup_g8(G8Shared<D> &sh, G8Ops &op, const float (&qraw)[D / 64][8], int G, float scale_log2,
                                 int j, int n, float *qs_out = nullptr)
{
    constexpr int NB = D / 32, NH = D / 64;
    const int h2 = n >> 3, hq = n & 7, e = 8 * j + hq, bb0 = h2 * NH;
    float xq[NH][8];
    float qm = 0.0f;
#pragma unroll
    for (int k = 0; k < NH; ++k)
#pragma unroll
        for (int hh = 0; hh < 8; ++hh) {
            const float x = hq < G ? qraw[k][hh] * scale_log2 : 0.0f;
            xq[k][hh] = x;
            qm = fmaxf(qm, fabsf(x));
        }
    qm = rows_max(qm);
    qm = fmax_nc(qm, other_half(qm));        // the head's other blocks
    int E = 0;
    if (qm > 0.0f) frexpf(qm, &E);         // |q'| * 2^-E < 1
    const float qscale = ldexpf(1.0f, -E);
    float Qo[NH];
#pragma unroll
    for (int k = 0; k < NH; ++k) {
        const int bb = bb0 + k;
        float qsum = 0.0f;
        h8 Bh, Bl;
#pragma unroll
        for (int hh = 0; hh < 8; ++hh) {
            const bool f16x = ((hh >> 1) & 1) != 0;            // code half carries a factor 16
            const float x = xq[k][hh] * qscale * (f16x ? 1.0f : 16.0f);
            const _Float16 hi = (_Float16)x;
            const _Float16 lo = (_Float16)(x - (float)hi);
            Bh[hh] = hi;
            Bl[hh] = lo;
            qsum += ((float)hi + (float)lo) * (f16x ? 1.0f : 0.0625f);
        }
        float incl, all;
        rows_prefix(qsum, j, incl, all);
        Qo[k] = all;
        sh.qk[(2 * bb) * 32 + e] = __builtin_bit_cast(u4, Bh);
        sh.qk[(2 * bb + 1) * 32 + e] = __builtin_bit_cast(u4, Bl);
        sh.qz[(2 * bb) * 32 + e] = u4{0, 0, 0, 0};
        sh.qz[(2 * bb + 1) * 32 + e] = u4{0, 0, 0, 0};
    }
    // block sums of every block: own half's and the other half's
    float Qs[NB];
#pragma unroll
    for (int k = 0; k < NH; ++k) {
        const float other = other_half(Qo[k]);
        Qs[k] = h2 ? other : Qo[k];
        Qs[NH + k] = h2 ? Qo[k] : other;
    }
    if (qs_out)
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) qs_out[bb] = Qs[bb];
    if (h2 == 0) {
        h8 B2h, B2l;
#pragma unroll
        for (int hh = 0; hh < 8; ++hh) {
            const float x = (j == 0 && hh < NB) ? -8.0f * Qs[hh < NB ? hh : 0] : 0.0f;
            const _Float16 hi = (_Float16)x;
            B2h[hh] = hi;
            B2l[hh] = (_Float16)(x - (float)hi);
        }
        sh.qc[e] = __builtin_bit_cast(u4, B2h);
        sh.qc[32 + e] = __builtin_bit_cast(u4, B2l);
    }
    op.qk[0] = (h2 == 0 ? sh.qk : sh.qz) + e;
    op.qk[1] = (h2 == 1 ? sh.qk : sh.qz) + e;
    op.qc[0] = (h2 == 0 ? sh.qc : sh.qz) + e;
    op.qc[1] = (h2 == 1 ? sh.qc : sh.qz) + e;
    return ldexpf(1.0f, E);
}

// K phase of one 32-token tile.  sb: the tile's K side data in LDS
// ([keyframe 2D bytes][scales 2D bytes]); FIRST: the tile opens a group (its
// token 0 is the keyframe: the code row reads as zeros and the keyframe logit
// enters through C2).  Lg: prefixed logits of this lane's 4 tokens (units
// q*2^-E) including `carry` (the sum over earlier tiles of the group); total:
// this tile's sum.  Returns the tile maximum in log2 units.
// DELTA = false: plain Q4_0 tile (absolute values: no prefix sums, no keyframe).
template <int D, bool FULL, bool FIRST, bool DELTA = true>
__device__ inline float k_phase_g8(const uint32_t *kc, const uint8_t *sb, const u4 *kf_row, int nval, int j, int n,
                                   const G8Ops &op, float c2E, float carry, float (&Lg)[4], float &total)
{
    constexpr int NB = D / 32, NP = NB / 2;
    const int h2 = n >> 3;
    const int tb = 16 * h2 + 4 * j;          // first of this lane's 4 tokens

    uint32_t sg[4][NP];
    {
        const uint32_t *sp = (const uint32_t *)(sb + 2 * D + tb * 2 * NB);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int k = 0; k < NP; ++k) sg[i][k] = sp[i * NP + k];
    }
    // C2: the "-8" correction of every delta token (and, in a first tile, the
    // keyframe logit in row 0: the keyframe, staged scaled by f(hh)/16 and read
    // as zeros by lanes n != 0, times the first half's query operand)
    f4 C2;
    {
        u4 a0 = u4{0, 0, 0, 0}, a1 = u4{0, 0, 0, 0};
        const uint32_t *p0 = (const uint32_t *)(sb + 2 * D + n * 2 * NB);
        const uint32_t *p1 = (const uint32_t *)(sb + 2 * D + (16 + n) * 2 * NB);
        // (loaded by every lane, then selected: a guarded load would split the code)
#pragma unroll
        for (int k = 0; k < NP; ++k) {
            const uint32_t w0 = p0[k], w1 = p1[k];
            a0[k] = (j == 0 && (!FIRST || n != 0)) ? w0 : 0u;
            a1[k] = j == 0 ? w1 : 0u;
        }
        C2 = mfma(as_h8(a0), as_h8(op.qc[0][0]), f4{0, 0, 0, 0});
        C2 = mfma(as_h8(a0), as_h8(op.qc[0][32]), C2);
        C2 = mfma(as_h8(a1), as_h8(op.qc[1][0]), C2);
        C2 = mfma(as_h8(a1), as_h8(op.qc[1][32]), C2);
    }
    f4 u = f4{0, 0, 0, 0};
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
        const h8 A0 = unpack8(kc[bb]);
        const h8 A1 = unpack8(kc[NB + bb]);
        const h8 bh0 = as_h8(op.qk[0][(2 * bb) * 32]), bl0 = as_h8(op.qk[0][(2 * bb + 1) * 32]);
        f4 P = mfma(A0, bh0, f4{0, 0, 0, 0});
        P = mfma(A0, bl0, P);
        P = mfma(A1, as_h8(op.qk[1][(2 * bb) * 32]), P);
        P = mfma(A1, as_h8(op.qk[1][(2 * bb + 1) * 32]), P);
        if constexpr (FIRST) {
            const h8 K = as_h8(kf_row[bb]);
            C2 = mfma(K, bh0, C2);
            C2 = mfma(K, bl0, C2);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) u[i] = __builtin_fmaf(half_at(sg[i], bb), P[i], u[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float d = __builtin_fmaf(u[i], 1048576.0f, C2[i]);
        Lg[i] = (FULL || tb + i < nval) ? d : 0.0f;
    }
    if constexpr (DELTA) {
        // prefix over the tile's tokens: in-lane, over rows j, then the first half's total
#pragma unroll
        for (int i = 1; i < 4; ++i) Lg[i] += Lg[i - 1];
        float incl, all;
        rows_prefix(Lg[3], j, incl, all);
        const float allx = other_half(all);           // (every lane takes part in the exchange)
        total = all + allx;
        const float off = (incl - Lg[3]) + (h2 ? allx : 0.0f) + carry;
#pragma unroll
        for (int i = 0; i < 4; ++i) Lg[i] += off;
    } else {
        total = 0.0f;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (FULL || tb + i < nval) mx = fmaxf(mx, Lg[i]);
    mx = rows_max(mx);
    mx = fmax_nc(mx, other_half(mx));
    return mx * c2E;
}

// K phase of one whole keyframe group of 32 tokens (kf = 32), with the two
// per-token terms that do not depend on the codes taken out of the code
// matrix instructions:
//  - the "-8" of every code: the accumulator of block bb starts at
//    bias[bb] = -8 * (sum of the head's query over the block) * 2^-20, the
//    units of the code products, so each block result is sum((c - 8) * q);
//  - the keyframe logit q.x0, computed for the whole run beforehand
//    (kf_logits_g8) and passed as `carry`, which the prefix sums add to every
//    token of the group.
// Token 0 is the keyframe: its code row reads as zeros and its scale slot
// holds the group's largest |scale| (used by the V side), so its delta term
// is dropped here and its logit is the carry alone.
// For a tile inside a long group (forward kernel below) `first` is false: the
// tile's token 0 is a delta like the others; `total` is the tile's sum.
template <int D, bool FULL>
__device__ inline float k_phase_g8b(const uint32_t *kc, const uint8_t *sb, int nval, int j, int n, const G8Ops &op,
                                    const h8 (&qh)[2][D / 32], const f4 (&bias)[D / 32], float c2E, float carry,
                                    float (&Lg)[4], bool first, float &total)
{
    constexpr int NB = D / 32, NP = NB / 2;
    const int h2 = n >> 3;
    const int tb = 16 * h2 + 4 * j;          // first of this lane's 4 tokens

    uint32_t sg[4][NP];
    {
        const uint32_t *sp = (const uint32_t *)(sb + 2 * D + tb * 2 * NB);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int k = 0; k < NP; ++k) sg[i][k] = sp[i * NP + k];
    }
    f4 u = f4{0, 0, 0, 0};
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
        const h8 A0 = unpack8(kc[bb]);
        const h8 A1 = unpack8(kc[NB + bb]);
        f4 P = mfma(A0, qh[0][bb], bias[bb]);
        P = mfma(A0, as_h8(op.qk[0][(2 * bb + 1) * 32]), P);
        P = mfma(A1, qh[1][bb], P);
        P = mfma(A1, as_h8(op.qk[1][(2 * bb + 1) * 32]), P);
#pragma unroll
        for (int i = 0; i < 4; ++i) u[i] = __builtin_fmaf(half_at(sg[i], bb), P[i], u[i]);
    }
    // logits stay in the units of the code products (2^-20 of the query
    // units); the factor 2^20 is folded into c2E
#pragma unroll
    for (int i = 0; i < 4; ++i) Lg[i] = (FULL || tb + i < nval) ? u[i] : 0.0f;
    Lg[0] = (first && tb == 0) ? 0.0f : Lg[0];
#pragma unroll
    for (int i = 1; i < 4; ++i) Lg[i] += Lg[i - 1];
    float incl, all;
    rows_prefix(Lg[3], j, incl, all);
    const float allx = other_half(all);           // (every lane takes part in the exchange)
    total = all + allx;
    const float off = (incl - Lg[3]) + (h2 ? allx : 0.0f) + carry;
#pragma unroll
    for (int i = 0; i < 4; ++i) Lg[i] += off;
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        if (FULL || tb + i < nval) mx = fmaxf(mx, Lg[i]);
    mx = rows_max(mx);
    mx = fmax_nc(mx, other_half(mx));
    return mx * c2E;
}

// Keyframe logits q.x0 of the first `cnt` (1..64) groups of a run (offsets in
// `list`), 16 groups per set of matrix instructions: row r of the K operand is
// the keyframe of group c + r (in the K-code operand order, scaled by f(hh)/16
// as the code operand expects), the B operand the query of column half 0.
// kf_load_g8 fetches lane (j, n)'s pieces of every 16-group set (positions past
// cnt re-read the last group), kf_logits_g8 writes out[x * 8 + hq]: the logit
// of head hq for the group at position x, in the units of k_phase_g8b's logits
// (2^-20 of the query units).
template <int D, int NSET = 4>
__device__ inline void kf_load_g8(u4 (&a)[NSET][D / 32], const int64_t *list, int cnt, const uint8_t *cache, int j,
                                  int n)
{
    constexpr int NB = D / 32;
#pragma unroll
    for (int c4 = 0; c4 < NSET; ++c4) {
        const u4 *kfp = (const u4 *)(cache + list[min(16 * c4 + n, cnt - 1)]) + j * NB;
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) a[c4][bb] = kfp[bb];
    }
}
template <int D, int NSET = 4>
__device__ inline void kf_logits_g8(float *out, const u4 (&a)[NSET][D / 32], int cnt, const G8Ops &op, int j, int n)
{
    constexpr int NB = D / 32;
#pragma unroll
    for (int c4 = 0; c4 < NSET; ++c4) {
        const int c = 16 * c4;
        if (c >= cnt) break;
        f4 C = f4{0, 0, 0, 0};
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) {
            u4 v = a[c4][bb];
            const uint32_t w0 = v[0], w2 = v[2];
            v[0] = scale_h2_16th(w0);
            v[2] = scale_h2_16th(w2);
            C = mfma(as_h8(v), as_h8(op.qk[0][(2 * bb) * 32]), C);
            C = mfma(as_h8(v), as_h8(op.qk[0][(2 * bb + 1) * 32]), C);
        }
        if (n < 8) {
#pragma unroll
            for (int i = 0; i < 4; ++i) out[(c + 4 * j + i) * 8 + n] = C[i] * 0x1p-20f;
        }
    }
}

// Lazy running max (log2 units): the reference max moves only when a group's
// maximum exceeds it by more than kLazyMax, so the softmax weights stay below
// 2^kLazyMax and the accumulators are rescaled rarely.  On slowly drifting
// logits (a random-walk cache) nearly every group used to raise the max and
// cost a rescale; with a fixed reference the 70B-layer split kernel measured
// 124 us against 136 us.  The partial records carry their reference max, so
// the split combine is unaffected.
constexpr int kLazyMax = 8;

// Softmax state update for a group with maximum m_g: new running max and V
// range bias from the group's largest |V scale| (slot 0 of the V scale plane,
// vs0) and kf <= 2^lkf; the accumulators are rescaled only when either changes,
// and with them `pend`, keyframe weights not yet added (same units).
template <int D>
__device__ inline void update_g8_vmx(RunState<D> &st, float m_g, uint32_t vmx, int lkf, float &pend)
{
    constexpr int NB = D / 32, NCC = D / 16, NP = NB / 2;
    const int ev = (vmx >> 10) == 0 ? -14 : (int)(vmx >> 10) - 15;
    // kf * 16 * |s| * 2^kLazyMax * 2^beta < 2^15 (weights below 2^kLazyMax)
    const int beta_g = (vmx == 0 ? 24 - lkf : 10 - lkf - ev) - kLazyMax;

    const float m_new = m_g > st.m + (float)kLazyMax ? m_g : st.m;
    const int beta_new = min(st.beta, beta_g);
    const float a_m = __builtin_amdgcn_exp2f(st.m - m_new);
    if (__any(m_new != st.m || beta_new != st.beta)) {
        st.bsc = ldexpf(1.0f, beta_new);
        const float alpha = a_m * ldexpf(1.0f, beta_new - st.beta);
#pragma unroll
        for (int cc = 0; cc < NCC; ++cc) st.acc[cc] *= alpha;
#pragma unroll
        for (int p = 0; p < NP; ++p) st.Z[p] *= alpha;
        st.l *= a_m;
        pend *= alpha;
    }
    st.m = m_new;
    st.beta = beta_new;
}
template <int D>
__device__ inline void update_g8(RunState<D> &st, float m_g, const uint32_t *vs0, int lkf)
{
    constexpr int NP = D / 64;
    uint32_t vmx = 0;
#pragma unroll
    for (int k = 0; k < NP; ++k) {
        const uint32_t w = vs0[k] & 0x7FFF7FFFu;
        vmx = max(vmx, max(w & 0xFFFFu, w >> 16));
    }
    float none = 0.0f;
    update_g8_vmx<D>(st, m_g, vmx, lkf, none);
}

// Keyframe term of a group: acc += pk * x0, pk = the group's weight in
// accumulator units 2^(beta-20); sb: the group's V side data in LDS.
template <int D>
__device__ inline void kf_fma_g8(RunState<D> &st, const uint8_t *sb, float pk, int j)
{
    constexpr int NCC = D / 16;
    const uint32_t *kp = (const uint32_t *)(sb + j * NCC * 8);
#pragma unroll
    for (int cc = 0; cc < NCC; ++cc) {
        const uint32_t w01 = kp[2 * cc], w23 = kp[2 * cc + 1];
        st.acc[cc][0] = __builtin_fmaf(hlo(w01), pk, st.acc[cc][0]);
        st.acc[cc][1] = __builtin_fmaf(hhi(w01), pk, st.acc[cc][1]);
        st.acc[cc][2] = __builtin_fmaf(hlo(w23), pk, st.acc[cc][2]);
        st.acc[cc][3] = __builtin_fmaf(hhi(w23), pk, st.acc[cc][3]);
    }
}

// The weighted V codes of one tile: Sp[T][i] is the weight (in the units
// 2^beta, times 16 on the slots i even) of token 16T + 4j + i for this lane's
// head column; it is multiplied by the token's scale of the lane's block of
// each pair, split hi + lo fp16, and the code tile's products accumulate
// into st.acc (the codes) and st.Z (their "-8").
template <int D, bool FULL>
__device__ inline void v_accumulate_g8(RunState<D> &st, const uint32_t *vc, const uint8_t *sb, const float (&Sp)[2][4],
                                       int nval, int j, int n, h8 AZ)
{
    constexpr int NB = D / 32, NP = NB / 2;
    const int h2 = n >> 3;
    // scales of the 8 token slots for this lane's block of each pair
    uint32_t vs[2][4];
    {
        const int wsel = NB == 4 ? h2 : 0;
#pragma unroll
        for (int T = 0; T < 2; ++T) {
            const uint32_t *sp = (const uint32_t *)(sb + 2 * D + (16 * T + 4 * j) * 2 * NB) + wsel;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t w = sp[i * NP];
                if constexpr (NB == 2) w >>= 16 * h2;        // block h2 of the single pair
                vs[T][i] = (FULL || 16 * T + 4 * j + i < nval) ? w : 0u;
            }
        }
    }
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        uint32_t whd[4], wld[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t hi, lo;
            if (NB == 4 && p == 1)
                split_w<1>(vs[0][i], vs[1][i], Sp[0][i], Sp[1][i], hi, lo);
            else
                split_w<0>(vs[0][i], vs[1][i], Sp[0][i], Sp[1][i], hi, lo);
            whd[i] = hi;
            wld[i] = lo;
        }
        const h8 Wh = __builtin_bit_cast(h8, u4{whd[0], whd[1], whd[2], whd[3]});
        const h8 Wl = __builtin_bit_cast(h8, u4{wld[0], wld[1], wld[2], wld[3]});
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
            const int cc = 4 * p + c4;
            const h8 A = unpack8(vc[cc]);
            st.acc[cc] = mfma(A, Wh, st.acc[cc]);
            st.acc[cc] = mfma(A, Wl, st.acc[cc]);
        }
        st.Z[p] = mfma(AZ, Wh, st.Z[p]);
        st.Z[p] = mfma(AZ, Wl, st.Z[p]);
    }
}

// V phase of one 32-token tile.  sb: the tile's V side data in LDS ([keyframe
// 2D bytes][scales 2D bytes]); Lg: the tile's prefixed logits from the K phase;
// carry: the sum of the softmax weights of the later tiles of the group.
// Adds the tile's weighted V codes to the accumulators; a FIRST tile (the last
// one processed) also adds the keyframe with the group's total weight.
// Returns the tile's weight sum.  DELTA = false: plain Q4_0 tile (the weight of
// token t is p_t itself, no suffix sums, no keyframe).
// KFD = false: a FIRST tile leaves the keyframe term to the caller (the return
// value plus carry is the group's weight).
template <int D, bool FULL, bool FIRST, bool DELTA = true, bool KFD = true>
__device__ inline float v_phase_g8(RunState<D> &st, const uint32_t *vc, const uint8_t *sb, const float (&Lg)[4],
                                   int nval, int j, int n, float c2E, h8 AZ, float carry)
{
    constexpr int NB = D / 32, NCC = D / 16, NP = NB / 2;
    const int h2 = n >> 3;
    const int tb = 16 * h2 + 4 * j;
    const float m_new = st.m;
    float S[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(Lg[i], c2E, -m_new));
        S[i] = (FULL || tb + i < nval) ? p : 0.0f;
    }
    float Pt;
    if constexpr (DELTA) {
#pragma unroll
        for (int i = 2; i >= 0; --i) S[i] += S[i + 1];
        float incl, all;
        rows_suffix(S[0], j, incl, all);
        const float allx = other_half(all);
        Pt = all + allx;
        const float off = (incl - S[0]) + (h2 ? 0.0f : allx) + carry;
#pragma unroll
        for (int i = 0; i < 4; ++i) S[i] += off;
    } else {
        const float all = rows_sum((S[0] + S[1]) + (S[2] + S[3]));
        Pt = all + other_half(all);
    }
    st.l += Pt;

    // suffix sums of both token halves: own half and the other column half's
    // (scaled to the weight units first: 2^beta, and 16 for the token slots
    // whose code nibble sits 4 bits up)
    const float bsc = st.bsc, bsc16 = 16.0f * bsc;
    float Sp[2][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float y = S[i] * ((i & 1) ? bsc : bsc16);
        const float x = other_half(y);
        Sp[0][i] = h2 ? x : y;
        Sp[1][i] = h2 ? y : x;
    }
    if constexpr (FIRST) Sp[0][0] = j == 0 ? 0.0f : Sp[0][0];      // keyframe slot
    v_accumulate_g8<D, FULL>(st, vc, sb, Sp, nval, j, n, AZ);
    if constexpr (FIRST && KFD) kf_fma_g8<D>(st, sb, (Pt + carry) * (st.bsc * 0x1p-20f), j);
    return Pt;
}

template <int D>
__device__ inline void init_state(RunState<D> &st)
{
#pragma unroll
    for (int cc = 0; cc < D / 16; ++cc) st.acc[cc] = f4{0, 0, 0, 0};
#pragma unroll
    for (int p = 0; p < D / 32; ++p) st.Z[p] = f4{0, 0, 0, 0};
    st.m = -INFINITY;
    st.l = 0.0f;
    st.beta = 127;
    st.bsc = 0x1p127f;
}

// The split-K combine as the kernel's tail (one launch per decode step), used
// where the launch is small enough that a second kernel launch costs more than
// the tail (the host picks it).  Every workgroup of a (sequence, kv-head) row
// writes its partial records for the row's G query heads and counts its
// arrival; the last of the row's nsplit workgroups resets the counter for the
// next call and merges the records into out.  The row's workgroups run on
// different XCDs, each with its own L2, so the records are published at device
// scope: written with device-scope (sc1) stores, which write through the
// writer's L2; the writer waits for them to complete (vmcnt(0)) before it
// counts its arrival; the merging workgroup's agent-scope acquire fence drops
// stale lines from its own L1 and L2 before it reads them.  (An agent-scope
// release fence in every workgroup instead writes back the whole L2, and
// device-scope loads instead of the acquire fence were slower still.)
constexpr int kCpolSc1 = 16;        // buffer cache-policy bit of gfx950: sc1 (device scope)

__device__ inline __amdgpu_buffer_rsrc_t ws_rsrc(const float *base, int nbytes)
{
    return __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, nbytes, 0x00020000);
}
// Record stores: write-through (wt) when the kernel merges its own records.
__device__ inline void store_rec4(float *p, f4 v, bool wt)
{
    if (wt)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4, v), ws_rsrc(p, 16), 0, 0, kCpolSc1);
    else
        *(f4 *)p = v;
}
__device__ inline void store_rec2(float *p, float a, float b, bool wt)
{
    if (wt)
        __builtin_amdgcn_raw_buffer_store_b64(u2{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b)},
                                              ws_rsrc(p, 8), 0, 0, kCpolSc1);
    else
        *(f2 *)p = f2{a, b};
}

// Split-K partial record of the wave's run: lane (j, n) keeps rows 4j..4j+3
// of each V slice; they belong to its column half's block when
// (j < 2) == (h2 == 0).
template <int D>
__device__ inline void write_partial_g8(const RunState<D> &st, float *ws, int64_t row0, int G, int nsplit, int split,
                                        int lane, int j, int n, bool wt)
{
    constexpr int NCC = D / 16;
    const int h2 = n >> 3, hq = n & 7;
    if (hq >= G) return;
    float *recp = ws + ((row0 + hq) * nsplit + split) * part_stride(D);
    const float un = ldexpf(1.0f, 20 - st.beta);
    if ((j < 2) == (h2 == 0)) {
#pragma unroll
        for (int cc = 0; cc < NCC; ++cc) {
            f4 o;
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = (st.acc[cc][i] + st.Z[cc >> 2][i]) * un;
            store_rec4(recp + vchan(D, cc, 4 * j, 1), o, wt);
        }
    }
    if (lane == hq) store_rec2(recp + D, st.m, st.l, wt);
}

// Merge of one row by the last workgroup, in one pass over the splits (running
// max in log2 units, the sums rescaled when it grows; splits with l = 0, i.e.
// runs past the end or on unmapped pages, are skipped; an empty row gives
// zeros).  The row's G heads are spread over the wave: GP = G rounded up to a
// power of two, 64/GP lanes per head, CPL = D*GP/64 channels per lane, so every
// lane carries the same running max and sum as the other lanes of its head and
// no lane-to-lane reduction is needed.  UB splits are loaded per batch, all
// their loads in flight before the first is used (each batch costs one round
// trip to the memory side).
template <int D, int GP>
__device__ __forceinline__ void merge_row_gp(const float *ws, float *out, int64_t row0, int G, int nsplit, int lane)
{
    constexpr int R = part_stride(D), LPH = 64 / GP, CPL = D / LPH;
    constexpr int UB = CPL >= 16 ? 8 : 16;
    const int hq = lane / LPH, sub = lane % LPH;
    const int hqc = hq < G ? hq : 0;          // lanes past the group read head 0 and discard it
    const float *rec0 = ws + (row0 + hqc) * nsplit * R;
    float M = -INFINITY, den = 0.0f;
    float num[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) num[c] = 0.0f;
    for (int s0 = 0; s0 < nsplit; s0 += UB) {
        f2 ml[UB];
        float a[UB][CPL];
#pragma unroll
        for (int u = 0; u < UB; ++u) {
            const float *r = rec0 + (int64_t)min(s0 + u, nsplit - 1) * R;
            ml[u] = *(const f2 *)(r + D);
            if constexpr (CPL >= 4) {
#pragma unroll
                for (int k = 0; k < CPL / 4; ++k) {
                    const f4 v = *(const f4 *)(r + sub * CPL + 4 * k);
#pragma unroll
                    for (int i = 0; i < 4; ++i) a[u][4 * k + i] = v[i];
                }
            } else if constexpr (CPL == 2) {
                const f2 v = *(const f2 *)(r + sub * CPL);
                a[u][0] = v[0];
                a[u][1] = v[1];
            } else {
                a[u][0] = r[sub];
            }
        }
#pragma unroll
        for (int u = 0; u < UB; ++u) {
            const float m = ml[u][0], l = ml[u][1];
            if (s0 + u < nsplit && l > 0.0f) {
                const float mn = fmaxf(M, m);
                const float al = exp2f(M - mn), w = exp2f(m - mn);
#pragma unroll
                for (int c = 0; c < CPL; ++c) num[c] = fmaf(w, a[u][c], num[c] * al);
                den = fmaf(w, l, den * al);
                M = mn;
            }
        }
    }
    if (hq >= G) return;
    float *o = out + (row0 + hq) * D + sub * CPL;
#pragma unroll
    for (int c = 0; c < CPL; ++c) o[c] = den > 0.0f ? num[c] / den : 0.0f;
}

template <int D>
__device__ __forceinline__ void merge_row_g8(const float *ws, float *out, int64_t row0, int G, int nsplit, int lane)
{
    if (G > 4) merge_row_gp<D, 8>(ws, out, row0, G, nsplit, lane);
    else if (G > 2) merge_row_gp<D, 4>(ws, out, row0, G, nsplit, lane);
    else if (G > 1) merge_row_gp<D, 2>(ws, out, row0, G, nsplit, lane);
    else merge_row_gp<D, 1>(ws, out, row0, G, nsplit, lane);
}

// After write_partial_g8 with wt = true: count this workgroup's arrival; the
// last of the row merges.
template <int D>
__device__ __forceinline__ void combine_tail_g8(const float *ws, const CombineTail &tl, int64_t row0, int G, int nsplit,
                                       int64_t pair, int lane)
{
    __builtin_amdgcn_s_waitcnt(0x0F70);          // vmcnt(0): the write-through record stores have completed
    __syncthreads();
    uint32_t *ctr = tl.counter + pair;
    uint32_t old = 0;
    if (lane == 0) old = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    old = __builtin_amdgcn_readfirstlane(old);
    if (old != (uint32_t)(nsplit - 1)) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    if (lane == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    merge_row_g8<D>(ws, tl.out, row0, G, nsplit, lane);
}

// "-8" operand of the V side: -8 * 2^-24 * f(hh) as fp16 subnormals
__device__ inline h8 v_minus8_operand()
{
    u4 azr;
    azr[0] = 0x80088008u;
    azr[1] = 0x80808080u;
    azr[2] = 0x80088008u;
    azr[3] = 0x80808080u;
    return as_h8(azr);
}

// ============================================================================ kf = 32
template <int D>
struct G8Regs {
    u4 side;                     // 16 B of the group's side data
    uint32_t kc[2 * (D / 32)];   // K code pieces of tokens n (first NB) and 16 + n (piece j)
    uint32_t vc[D / 16];         // V code words of tile row n (piece j)
};

template <int D>
__device__ inline void load_g8(G8Regs<D> &r, const uint8_t *rec, int rec_bytes, const LaneOffsets &o)
{
    constexpr int NB = D / 32, NCC = D / 16;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void *)rec, (short)0, rec_bytes, 0x00020000);
    r.side = __builtin_amdgcn_raw_buffer_load_b128(rs, o.side, 0, kStream);
    if constexpr (NB == 4) {
        u4 a = __builtin_amdgcn_raw_buffer_load_b128(rs, o.k0, 0, kStream);
        u4 c = __builtin_amdgcn_raw_buffer_load_b128(rs, o.k1, 0, kStream);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            r.kc[k] = a[k];
            r.kc[NB + k] = c[k];
        }
    } else {
        u2 a = __builtin_amdgcn_raw_buffer_load_b64(rs, o.k0, 0, kStream);
        u2 c = __builtin_amdgcn_raw_buffer_load_b64(rs, o.k1, 0, kStream);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            r.kc[k] = a[k];
            r.kc[NB + k] = c[k];
        }
    }
#pragma unroll
    for (int q4 = 0; q4 < NCC / 4; ++q4) {
        u4 a = __builtin_amdgcn_raw_buffer_load_b128(rs, o.v + vcode_piece(D, 0, q4), 0, kStream);
#pragma unroll
        for (int k = 0; k < 4; ++k) r.vc[4 * q4 + k] = a[k];
    }
}

// The kf = 32 kernel fetches the two parts of a group separately: the K part
// (side data and K code pieces) and the V part (V code words), each two groups
// ahead of its use.
template <int D>
struct G8KRegs {
    u4 side;
    uint32_t kc[2 * (D / 32)];
};
template <int D>
struct G8VRegs {
    uint32_t vc[D / 16];
};

template <int D>
__device__ inline void load_g8k(G8KRegs<D> &r, const uint8_t *rec, int rec_bytes, const LaneOffsets &o)
{
    constexpr int NB = D / 32;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void *)rec, (short)0, rec_bytes, 0x00020000);
    r.side = __builtin_amdgcn_raw_buffer_load_b128(rs, o.side, 0, kStream);
    if constexpr (NB == 4) {
        const u4 a = __builtin_amdgcn_raw_buffer_load_b128(rs, o.k0, 0, kStream);
        const u4 c = __builtin_amdgcn_raw_buffer_load_b128(rs, o.k1, 0, kStream);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            r.kc[k] = a[k];
            r.kc[NB + k] = c[k];
        }
    } else {
        const u2 a = __builtin_amdgcn_raw_buffer_load_b64(rs, o.k0, 0, kStream);
        const u2 c = __builtin_amdgcn_raw_buffer_load_b64(rs, o.k1, 0, kStream);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            r.kc[k] = a[k];
            r.kc[NB + k] = c[k];
        }
    }
}

template <int D>
__device__ inline void load_g8v(G8VRegs<D> &r, const uint8_t *rec, int rec_bytes, const LaneOffsets &o)
{
    constexpr int NCC = D / 16;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void *)rec, (short)0, rec_bytes, 0x00020000);
#pragma unroll
    for (int q4 = 0; q4 < NCC / 4; ++q4) {
        const u4 a = __builtin_amdgcn_raw_buffer_load_b128(rs, o.v + vcode_piece(D, 0, q4), 0, kStream);
#pragma unroll
        for (int k = 0; k < 4; ++k) r.vc[4 * q4 + k] = a[k];
    }
}

// Largest |V scale| of a group: slot 0 of its V scale plane (side data + 6*D).
template <int D>
__device__ inline uint32_t group_vmax(const uint8_t *sb)
{
    const uint32_t *vs0 = (const uint32_t *)(sb + 6 * D);
    uint32_t vmx = 0;
#pragma unroll
    for (int k = 0; k < D / 64; ++k) {
        const uint32_t w = vs0[k] & 0x7FFF7FFFu;
        vmx = max(vmx, max(w & 0xFFFFu, w >> 16));
    }
    return vmx;
}

// Steps between the fetch of a group part and its use in the kf = 32 kernel
// (2..4; each step of lead holds one more group, 20 registers, in flight).
constexpr int kG8Lead = 3;

template <int V>
struct IC {
    static constexpr int value = V;
};

// Offset of the k-th mapped group of a run as a wave-uniform value.
__device__ inline int64_t uniform_offset(const int64_t *list, int k)
{
    const int64_t v = list[k];
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// kf = 32: the groups of a run (at most 64) are software-pipelined.  Step i
// runs the V phase of group i and the K phase (with the softmax update) of
// group i + 1, two independent streams of work that the compiler interleaves
// in one block of code.  The keyframe terms of every 4 groups are added
// together by fp32 matrix instructions.  The last step's K phase re-reads the
// last group of the run: its maximum and V range are already in the state,
// so its update changes nothing and its logits are not used.
template <int D>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2)))
    k_attn_g8(dkv_config cfg, const uint8_t *cache, const int32_t *__restrict__ bt,
              const float *__restrict__ q, const int32_t *__restrict__ seq_lens, float scale_log2,
              float *ws, int nsplit, int chunk, AppendArgs ap, CombineTail ct)
{
    constexpr int NB = D / 32, NCC = D / 16;
    constexpr int SIDE_LANES = D / 4;
    constexpr int BATCH = 64;
    constexpr int LEAD = kG8Lead, NBUF = LEAD + 1;
    static_assert(NBUF == 4, "the keyframe batches of 4 groups close on the last step of an unrolled round");
    constexpr int NSLOT = 8;
    const Geom g = make_geom(cfg);
    const int split = grid_split(), h = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x, j = lane >> 4, n = lane & 15;
    const int G = g.G;
    if (ap.positions) {
        // the run that holds the new token's group appends it first (both
        // streams), and makes the bytes visible to its own loads below
        const int pos = ap.positions[b];
        if (pos >= 0 && pos < g.cap_tokens && (pos >> 5) / chunk == split) {
            append_token_stream<D>(g, ap.cache, ap.state, bt, ap.knew, ap.vnew, pos, b, h, 0, threadIdx.x);
            append_token_stream<D>(g, ap.cache, ap.state, bt, ap.knew, ap.vnew, pos, b, h, 1, threadIdx.x);
            // the stores complete (in this XCD's L2, which the loads below also
            // use), then the L1 lines the read-modify-write of the V codes
            // brought in are dropped
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        }
    }
    const int L = min(seq_lens[b], g.cap_tokens);
    const int ng = (L + 31) >> 5;
    const int g0 = split * chunk, g1 = min(ng, g0 + chunk);
    const int64_t row0 = (int64_t)b * g.Hq + h * G;

    // side data of the groups at positions x of the run in slot x % NSLOT:
    // [K keyframe][K scales][V keyframe][V scales], 2*D bytes each.  A group is
    // staged two steps before its V phase; its slot is rewritten six steps
    // after it, when the group's keyframe batch has long been added.
    __shared__ __attribute__((aligned(16))) uint32_t side[NSLOT][2 * D];
    __shared__ int64_t glist[BATCH];
    __shared__ G8Shared<D> sh;
    __shared__ float kls[BATCH * 8];          // keyframe logits [position][head]

    // The run's mapped groups (a run has at most BATCH groups: the split plan
    // caps it at 2048 tokens) listed in LDS.  The whole groups go through the
    // pipeline; a partial last group of the sequence is taken on its own after.
    const int x0 = g0 + lane;
    const int64_t o0 = x0 < g1 ? group_offset(g, bt, b, h, x0) : -1;
    const uint64_t mk = __ballot(o0 >= 0);
    const int cnt = __popcll(mk);
    const bool last_partial = (L & 31) != 0 && g1 == ng && ng > g0 && ((mk >> (ng - 1 - g0)) & 1) != 0;
    const int nfull = cnt - (last_partial ? 1 : 0);
    if (cnt == 0) {
        // a run past the sequence's end: no record (the combine reads only
        // the runs that start before the end), unless this launch merges
        // its own records, which counts every run's arrival
        if (g0 >= ng && !ct.out) return;
        // a wholly unmapped run: an empty record
        RunState<D> st;
        init_state<D>(st);
        write_partial_g8<D>(st, ws, row0, G, nsplit, split, lane, j, n, ct.out != nullptr);
        if (ct.out) combine_tail_g8<D>(ws, ct, row0, G, nsplit, (int64_t)b * g.Hkv + h, lane);
        return;
    }
    if (o0 >= 0) glist[__builtin_amdgcn_mbcnt_hi((uint32_t)(mk >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mk, 0u))] = o0;
    __syncthreads();
    // past the end of the whole groups the fetches re-read the last one (still
    // in L2: it was fetched a few steps earlier); a run whose only group is a
    // partial one fetches that group.  Every start-up load is unconditional, so
    // all of them go out together and each wait covers only what it needs.
    auto rec_at = [&](int k) { return cache + uniform_offset(glist, k < nfull ? k : max(nfull - 1, 0)); };

    LaneOffsets lo = lane_offsets<D>(g, lane, j, n, true);
    // the K keyframe (side lanes < D/8) is read once, by the keyframe-logit
    // prologue: these lanes' side loads read past the record (zeros)
    if (lane < D / 8) lo.side = 0x40000000;
    const int rec_bytes = (int)g.rec;
    // group x: K part in buffer x % NBUF (fetched LEAD steps before the step
    // that stages it), V part in buffer x % NBUF.  Start-up order: the parts
    // the first steps use, the query, the keyframes of the run's groups (one
    // set of 16 for runs of up to 16 groups), then the query set-up and the
    // keyframe logits, then the rest of the lead.  Every wave of the launch
    // starts at once, so the start-up loads are a burst; measured per
    // workgroup (s_memrealtime), issuing the first group's parts first and
    // no keyframe sets past the run cut the median start-up on the long
    // workload from 7.6 to 5.9 us.
    G8KRegs<D> kb[NBUF];
    G8VRegs<D> vb[NBUF];
    G8Ops op;
    float qs[NB];
    float c2E;
    auto prologue = [&](auto nset_c) {
        constexpr int NS = decltype(nset_c)::value;
        load_g8k<D>(kb[0], rec_at(0), rec_bytes, lo);
        load_g8v<D>(vb[0], rec_at(0), rec_bytes, lo);
        load_g8k<D>(kb[1], rec_at(1), rec_bytes, lo);
        float qraw[D / 64][8];
        load_q_g8<D>(qraw, q, row0, G, j, n);
        u4 kfa[NS][NB];
        kf_load_g8<D, NS>(kfa, glist, cnt, cache, j, n);
        c2E = setup_g8<D>(sh, op, qraw, G, scale_log2, j, n, qs);
        kf_logits_g8<D, NS>(kls, kfa, cnt, op, j, n);
        load_g8v<D>(vb[1], rec_at(1), rec_bytes, lo);
        load_g8k<D>(kb[2], rec_at(2), rec_bytes, lo);
        load_g8v<D>(vb[2], rec_at(2), rec_bytes, lo);
        load_g8k<D>(kb[3], rec_at(3), rec_bytes, lo);
    };
    if (cnt <= 16)
        prologue(IC<1>{});
    else
        prologue(IC<4>{});
    const h8 AZ = v_minus8_operand();
    // accumulator start of each block's code products: the "-8" term
    f4 kbias[NB];
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
        const float x = -8.0f * 0x1p-20f * qs[bb];
        kbias[bb] = f4{x, x, x, x};
    }
    auto klog = [&](int x) { return kls[x * 8 + (n & 7)]; };
    // the K phases' logits are in 2^-20 of the query units
    const float c2Eu = c2E * 1048576.0f;
    // the hi query operands of both token halves stay in registers
    h8 qh[2][NB];
#pragma unroll
    for (int T = 0; T < 2; ++T)
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) qh[T][bb] = as_h8(op.qk[T][(2 * bb) * 32]);

    RunState<D> st;
    init_state<D>(st);
    // keyframe weights of the open batch of 4 groups: lane (j, n) holds the
    // weight of head column n of the batch's group j (the B operand of an
    // fp32 16x16x4 matrix instruction whose A operand holds the 4 keyframes)
    float kfw = 0.0f;
    float tot_unused;                         // (runs of kf = 32 groups carry no logits between tiles)

    auto sbp = [&](int x) { return (const uint8_t *)side[x & (NSLOT - 1)]; };
    auto stage = [&](const G8KRegs<D> &r, int x) {
        if (2 * SIDE_LANES == 64 || lane < 2 * SIDE_LANES) ((u4 *)side[x & (NSLOT - 1)])[fresh_lane_id()] = r.side;
    };
    // add the keyframe terms of the batch whose last group is at position x:
    // lane (j, n) supplies channel row n of slice cc of group (x & ~3) + j
    // (rows past x, if any, are masked to zero)
    auto kf_flush = [&](int x, bool whole) {
        const int gj = (x & ~3) + j;
        const uint16_t *kfv = (const uint16_t *)(sbp(gj) + 4 * D) + (n >> 2) * NCC * 4 + (n & 3);
        const bool live = whole || gj <= x;
#pragma unroll
        for (int cc = 0; cc < NCC; ++cc) {
            const float a = live ? h2f(kfv[4 * cc]) : 0.0f;
            st.acc[cc] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, kfw, st.acc[cc], 0, 0, 0);
        }
        kfw = 0.0f;
    };

    // A group is one tile here: the V phases get no carry (-0.0, since
    // x + -0.0 == x for every x and the add folds away); the K phases get the
    // group's keyframe logit.
    if (nfull > 0) {
        float Lg[4];
        __syncthreads();
        stage(kb[0], 0);
        stage(kb[1], 1);
        __syncthreads();
        {
            const float m = k_phase_g8b<D, true>(kb[0].kc, sbp(0), 32, j, n, op, qh, kbias, c2Eu, klog(0), Lg,
                                                 true, tot_unused);
            update_g8_vmx<D>(st, m, group_vmax<D>(sbp(0)), 5, kfw);
        }
        // step i (u = i % NBUF): fetch the K part of group i + 1 + LEAD and the
        // V part of group i + LEAD, V phase of i (its keyframe weight joins the
        // open batch), K phase of i + 1, then stage the K part of group i + 2 for
        // the next step.  The wave is alone in its workgroup: its LDS accesses
        // stay in program order without barriers.
        auto step = [&](int i, auto uc) {
            constexpr int u = decltype(uc)::value;
            constexpr int un = (u + 1) % NBUF, u2 = (u + 2) % NBUF, ulast = (u + LEAD) % NBUF;
            load_g8k<D>(kb[u], rec_at(i + 1 + LEAD), rec_bytes, lo);
            load_g8v<D>(vb[ulast], rec_at(i + LEAD), rec_bytes, lo);
            const float pt =
                v_phase_g8<D, true, true, true, false>(st, vb[u].vc, sbp(i) + 4 * D, Lg, 32, j, n, c2Eu, AZ, -0.0f);
            kfw = j == u ? pt * (st.bsc * 0x1p-20f) : kfw;
            if constexpr (u == NBUF - 1) kf_flush(i, true);
            const float m = k_phase_g8b<D, true>(kb[un].kc, sbp(i + 1), 32, j, n, op, qh, kbias, c2Eu,
                                                 klog(min(i + 1, nfull - 1)), Lg, true, tot_unused);
            update_g8_vmx<D>(st, m, group_vmax<D>(sbp(i + 1)), 5, kfw);
            stage(kb[u2], i + 2);
            return i + 1 < nfull;
        };
        // Two waves share each SIMD, and the issue arbiter favours the older one:
        // with equal runs the first-dispatched half of the grid finished in
        // about 118 us and the second in about 151 us.  So the wave priority
        // falls with the run's progress (quarters), and the first-dispatched
        // half runs one level lower; a wave that falls behind wins the issue
        // slots until it has caught up.  (Order only: results are unaffected.)
        const bool older = (blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z)) <
                           (gridDim.x * gridDim.y * gridDim.z) / 2;
        const int q1 = nfull >> 2, q2 = nfull >> 1, q3 = (3 * nfull) >> 2;
        if (older) __builtin_amdgcn_s_setprio(2); else __builtin_amdgcn_s_setprio(3);
        // Whole rounds of 4 steps, then the remaining 0..3 steps.  (No exit from
        // inside a round: an exit path that shares the loop's back edge makes the
        // compiler drain every fetch in flight at the top of each round.)
        const int nround = nfull / NBUF, nrest = nfull % NBUF;
        for (int r = 0; r < nround; ++r) {
            const int i = r * NBUF;
            if (i >= q1) {
                const int lvl = (i >= q3 ? 0 : i >= q2 ? 1 : 2) - (older ? 1 : 0);
                if (lvl <= 0)
                    __builtin_amdgcn_s_setprio(0);
                else if (lvl == 1)
                    __builtin_amdgcn_s_setprio(1);
                else
                    __builtin_amdgcn_s_setprio(2);
            }
            step(i, IC<0>{});
            step(i + 1, IC<1>{});
            step(i + 2, IC<2>{});
            step(i + 3, IC<3>{});
        }
        if (nrest > 0) {
            const int i = nround * NBUF;
            step(i, IC<0>{});
            if (nrest > 1) step(i + 1, IC<1>{});
            if (nrest > 2) step(i + 2, IC<2>{});
        }
        if (((nfull - 1) & 3) != 3) kf_flush(nfull - 1, false);
        __builtin_amdgcn_s_setprio(0);
    }
    if (last_partial) {
        G8KRegs<D> kr;
        G8VRegs<D> vr;
        const uint8_t *rec = cache + uniform_offset(glist, cnt - 1);
        load_g8k<D>(kr, rec, rec_bytes, lo);
        load_g8v<D>(vr, rec, rec_bytes, lo);
        // position nfull: its slot holds no group of an open batch
        __syncthreads();
        stage(kr, nfull);
        __syncthreads();
        const int nval = L - (ng - 1) * 32;
        float Lg[4];
        const float m = k_phase_g8b<D, false>(kr.kc, sbp(nfull), nval, j, n, op, qh, kbias, c2Eu, klog(nfull), Lg,
                                              true, tot_unused);
        update_g8_vmx<D>(st, m, group_vmax<D>(sbp(nfull)), 5, kfw);
        v_phase_g8<D, false, true>(st, vr.vc, sbp(nfull) + 4 * D, Lg, nval, j, n, c2Eu, AZ, -0.0f);
    }
    write_partial_g8<D>(st, ws, row0, G, nsplit, split, lane, j, n, ct.out != nullptr);
    if (ct.out) combine_tail_g8<D>(ws, ct, row0, G, nsplit, (int64_t)b * g.Hkv + h, lane);
}

// ==================================================================== kf = 32*NT
// One step = one 32-token tile of one pass: the K pass visits tiles 0..nt-1 of
// a group, the V pass tiles nt-1..0.  The registers of the next step are
// fetched while the current one is processed.
template <int D>
struct TileRegs {
    u4 side;                  // 16 B of the tile's side data (keyframe / scales / V slot 0)
    uint32_t code[D / 16];    // K: pieces of rows n and 16 + n (NB words each); V: the lane's tile words
};

template <int D>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2)))
    k_attn_long_g8(dkv_config cfg, const uint8_t *__restrict__ cache, const int32_t *__restrict__ bt,
                   const float *__restrict__ q, const int32_t *__restrict__ seq_lens, float scale_log2,
                   float *ws, int nsplit, int chunk, CombineTail ct)
{
    constexpr int NB = D / 32, NCC = D / 16;
    const Geom g = make_geom(cfg);
    const int kf = g.kf;
    const int lkf = 32 - __builtin_clz((unsigned)kf - 1u);       // kf <= 2^lkf
    const int split = grid_split(), h = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x, j = lane >> 4, n = lane & 15;
    const int G = g.G;
    const int L = min(seq_lens[b], g.cap_tokens);
    const int ng = (L + kf - 1) / kf;
    const int g0 = split * chunk, g1 = min(ng, g0 + chunk);
    const int64_t row0 = (int64_t)b * g.Hq + h * G;
    if (g0 >= ng && !ct.out) return;       // past the sequence's end: no record (see k_attn_g8)

    // side: [keyframe 2D bytes][scales of the tile 2D bytes] of the current step;
    // vslot0: slot 0 (max |scale|) of the group's V scale plane
    __shared__ __attribute__((aligned(16))) uint32_t side[D];
    __shared__ __attribute__((aligned(16))) uint32_t vslot0[4];
    __shared__ G8Shared<D> sh;
    extern __shared__ f4 lgs[];               // prefixed logits [tile][row] of the current group

    G8Ops op;
    float c2E = 0.0f;                         // set once the first fetches are out
    const h8 AZ = v_minus8_operand();

    RunState<D> st;
    init_state<D>(st);

    const int rec_bytes = (int)g.rec;
    auto next_mapped = [&](int x, int64_t &o) {
        for (; x < g1; ++x) {
            o = group_offset(g, bt, b, h, x);
            if (o >= 0) break;
        }
        return x;
    };
    auto ntiles = [&](int gi) { return (min(kf, L - gi * kf) + 31) >> 5; };
    // step s of a group with nt tiles: s < nt -> K tile s, else V tile 2*nt-1-s.
    // Every step issues the same three loads (side data, two code pieces of NB
    // words); only the offsets differ, so the wait counts stay exact.
    auto load_step = [&](TileRegs<D> &r, int64_t off, int s, int nt) {
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc((void *)(cache + off), (short)0, rec_bytes, 0x00020000);
        const bool kp = s < nt;
        const int t = kp ? s : 2 * nt - 1 - s;
        // side: lanes < D/8 the keyframe, D/8..D/4 the tile's scales, lane D/4 (K pass) V slot 0
        int so;
        if (lane < D / 8)
            so = (kp ? 0 : (int)g.off_vkf) + 16 * lane;
        else if (lane < D / 4)
            so = (int)(kp ? g.off_ksc : g.off_vsc) + 64 * NB * t + 16 * (lane - D / 8);
        else
            so = (kp && lane == D / 4) ? (int)g.off_vsc : 0x40000000;
        // K: token 32t + n is code row 32t + n - 1 (the keyframe row of tile 0 reads
        // as zeros), token 32t + 16 + n row 32t + 15 + n.  V: the lane's 2*NB tile words.
        const int ov = (int)g.off_vcd + 16 * D * t + vcode_piece(D, lane, 0);
        const int o0 = kp ? ((t == 0 && n == 0) ? 0x40000000 : (int)g.off_kcd + (32 * t + n - 1) * (D / 2) + 4 * j * NB)
                          : ov;
        const int o1 = kp ? (int)g.off_kcd + (32 * t + 15 + n) * (D / 2) + 4 * j * NB
                          : ov + (NB == 4 ? vcode_piece(D, 0, 1) : 4 * NB);
        r.side = __builtin_amdgcn_raw_buffer_load_b128(rs, so, 0, kStream);
        if constexpr (NB == 4) {
            const u4 a = __builtin_amdgcn_raw_buffer_load_b128(rs, o0, 0, kStream);
            const u4 c = __builtin_amdgcn_raw_buffer_load_b128(rs, o1, 0, kStream);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                r.code[k] = a[k];
                r.code[4 + k] = c[k];
            }
        } else {
            const u2 a = __builtin_amdgcn_raw_buffer_load_b64(rs, o0, 0, kStream);
            const u2 c = __builtin_amdgcn_raw_buffer_load_b64(rs, o1, 0, kStream);
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                r.code[k] = a[k];
                r.code[2 + k] = c[k];
            }
        }
    };
    auto stage = [&](const TileRegs<D> &r, bool kpass) {
        u4 v = r.side;
        if (kpass && lane < D / 8) {
            const uint32_t w0 = v[0], w2 = v[2];
            v[0] = scale_h2_16th(w0);
            v[2] = scale_h2_16th(w2);
        }
        if (lane < D / 4) ((u4 *)side)[fresh_lane_id()] = v;
        if (kpass && lane == D / 4) *(u4 *)vslot0 = v;
    };
    const u4 *kf_row = n == 0 ? (const u4 *)((const uint8_t *)side + j * NB * 16) : sh.qz;

    // Logit rows of a tile: one f4 per lane.  With at most 4 query heads per
    // kv-head only the lanes of heads 0..3 carry logits, so a tile takes 32 rows
    // (lane (j, n) -> 8j + 4(n >> 3) + (n & 3)); the other lanes read those rows
    // (finite values they do not use) and write to one spare row past the tiles.
    const bool half_rows = G <= 4;
    const int lrow = half_rows ? 8 * j + 4 * (n >> 3) + (n & 3) : lane;
    const int lstride = half_rows ? 32 : 64;
    const int spare = ((kf + 31) >> 5) * 32;
    const bool wr_spare = half_rows && (n & 7) >= 4;

    float carry = 0.0f, mx = -INFINITY;       // per-group pass state
    // a position in the run: group g (record at off), step s of its 2*nt steps
    struct Cursor {
        int g;
        int64_t off;
        int s, nt;
    };
    auto next_pos = [&](Cursor c) {
        Cursor r = c;
        if (++r.s < 2 * r.nt) return r;
        r.g = next_mapped(c.g + 1, r.off);
        r.s = 0;
        r.nt = r.g < g1 ? ntiles(r.g) : 1;
        return r;
    };
    float qraw[D / 64][8];
    load_q_g8<D>(qraw, q, row0, G, j, n);
    Cursor cc0;
    cc0.off = -1;
    cc0.g = next_mapped(g0, cc0.off);
    if (cc0.g < g1) {
        cc0.s = 0;
        cc0.nt = ntiles(cc0.g);
        // two steps in flight: the registers of steps +1 and +2 are being fetched
        Cursor cc1 = next_pos(cc0), cc2 = cc1.g < g1 ? next_pos(cc1) : cc1;
        TileRegs<D> ra, rb, rc;
        load_step(ra, cc0.off, 0, cc0.nt);
        load_step(rb, cc1.g < g1 ? cc1.off : cc0.off, cc1.g < g1 ? cc1.s : 0, cc1.g < g1 ? cc1.nt : cc0.nt);
        // query set-up after the first fetches, so its loads overlap them
        c2E = setup_g8<D>(sh, op, qraw, G, scale_log2, j, n);
        // wave priority by progress through the run, one level lower for the
        // first-dispatched half of the grid (as in the kf = 32 kernel)
        const bool older = (blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z)) <
                           (gridDim.x * gridDim.y * gridDim.z) / 2;
        const int ntmax = (kf + 31) >> 5;
        const int run_steps = (g1 - g0) * 2 * ntmax;
        // quarter marks of the run (step counts), computed once: no division per step
        const int q1 = (run_steps + 3) / 4, q2 = (2 * run_steps + 3) / 4, q3 = (3 * run_steps + 3) / 4;
        auto set_priority = [&](int gc, int s) {
            const int done = (gc - g0) * 2 * ntmax + s;
            const int quarters = (done >= q1) + (done >= q2) + (done >= q3);
            const int lvl = 3 - quarters - (older ? 1 : 0);
            if (lvl <= 0)
                __builtin_amdgcn_s_setprio(0);
            else if (lvl == 1)
                __builtin_amdgcn_s_setprio(1);
            else if (lvl == 2)
                __builtin_amdgcn_s_setprio(2);
            else
                __builtin_amdgcn_s_setprio(3);
        };
        auto step = [&](const TileRegs<D> &cur, TileRegs<D> &pf) {
            const int gc = cc0.g, s = cc0.s, ntc = cc0.nt;
            set_priority(gc, s);
            __syncthreads();
            const bool kp = s < ntc;
            const int t = kp ? s : 2 * ntc - 1 - s;
            const int nval = min(kf, L - gc * kf) - 32 * t;     // valid tokens from the tile start
            stage(cur, kp);
            // prefetch two steps ahead (past the end: the current step again)
            const bool more = cc2.g < g1;
            load_step(pf, more ? cc2.off : cc0.off, more ? cc2.s : s, more ? cc2.nt : ntc);
            __syncthreads();
            const uint8_t *sb = (const uint8_t *)side;
            if (kp) {
                float Lg[4], tot, m;
                if (t == 0) {
                    carry = 0.0f;
                    if (nval >= 32)
                        m = k_phase_g8<D, true, true>(cur.code, sb, kf_row, nval, j, n, op, c2E, carry, Lg, tot);
                    else
                        m = k_phase_g8<D, false, true>(cur.code, sb, kf_row, nval, j, n, op, c2E, carry, Lg, tot);
                    mx = m;
                } else {
                    if (nval >= 32)
                        m = k_phase_g8<D, true, false>(cur.code, sb, kf_row, nval, j, n, op, c2E, carry, Lg, tot);
                    else
                        m = k_phase_g8<D, false, false>(cur.code, sb, kf_row, nval, j, n, op, c2E, carry, Lg, tot);
                    mx = fmaxf(mx, m);
                }
                carry += tot;
                lgs[wr_spare ? spare : t * lstride + lrow] = f4{Lg[0], Lg[1], Lg[2], Lg[3]};
                if (t == ntc - 1) {
                    update_g8<D>(st, mx, vslot0, lkf);
                    carry = 0.0f;            // from here on: the suffix carry of the V pass
                }
            } else {
                const f4 lv = lgs[t * lstride + lrow];
                const float Lg[4] = {lv[0], lv[1], lv[2], lv[3]};
                float pt;
                if (t == 0) {
                    if (nval >= 32)
                        pt = v_phase_g8<D, true, true>(st, cur.code, sb, Lg, nval, j, n, c2E, AZ, carry);
                    else
                        pt = v_phase_g8<D, false, true>(st, cur.code, sb, Lg, nval, j, n, c2E, AZ, carry);
                } else {
                    if (nval >= 32)
                        pt = v_phase_g8<D, true, false>(st, cur.code, sb, Lg, nval, j, n, c2E, AZ, carry);
                    else
                        pt = v_phase_g8<D, false, false>(st, cur.code, sb, Lg, nval, j, n, c2E, AZ, carry);
                }
                carry += pt;
            }
            // move to the next step
            cc0 = cc1;
            cc1 = cc2;
            if (cc2.g < g1) cc2 = next_pos(cc2);
            return cc0.g < g1;
        };
        // The run's steps: 2 per tile of each mapped group (only the sequence's
        // last group can be short).  Whole rounds of 3 steps, then the 0..2
        // left through one step that rotates the buffers by value: no exit
        // from inside a round (an exit path that shares the back edge makes
        // the compiler drain every fetch in flight at the top of each round).
        int total;
        {
            const int xg = g0 + lane;
            const uint64_t mm = __ballot(xg < g1 && group_offset(g, bt, b, h, xg) >= 0);
            total = 2 * ntmax * __popcll(mm);
            if (g1 == ng && ng > g0 && ((mm >> (ng - 1 - g0)) & 1) != 0) total += 2 * (ntiles(ng - 1) - ntmax);
        }
        const int nround = total / 3, nrest = total % 3;
        for (int r = 0; r < nround; ++r) {
            step(ra, rc);
            step(rb, ra);
            step(rc, rb);
        }
        for (int x = 0; x < nrest; ++x) {
            step(ra, rc);
            const TileRegs<D> t = ra;
            ra = rb;
            rb = rc;
            rc = t;
        }
        __builtin_amdgcn_s_setprio(0);
    }
    write_partial_g8<D>(st, ws, row0, G, nsplit, split, lane, j, n, ct.out != nullptr);
    if (ct.out) combine_tail_g8<D>(ws, ct, row0, G, nsplit, (int64_t)b * g.Hkv + h, lane);
}

// ============================================================ kf = 32*NT, G <= 4
// Long groups (kf = 64..512) with at most 4 query heads per kv-head, in one
// forward pass.  With P the group's total softmax weight, d_t the delta of
// token t and E_t the weight of the group's tokens before t, the weighted sum
// of the group's reconstructions is
//   sum_t p_t xhat_t = P * (x0 + sum_t d_t) - sum_t E_t * d_t,
// so every tile's V codes can be weighted as soon as its logits are known
// (with -E_t), and the K and V sides of a tile share one step, pipelined as
// in the kf = 32 kernel: step x runs the V phase of tile x and the K phase of
// tile x + 1.  Operand column 4 of each column half is spare when G <= 4; it
// weights every delta with 1 and so sums the group's deltas.  At the group's
// last tile every head adds P times its keyframe and that sum.  Against the
// two-pass kernel (K pass, then V pass in reverse) a tile takes one step
// instead of two and no logits go through LDS.

// Softmax state update of the forward kernel: as update_g8_vmx, but the
// lanes of the delta-sum column (dcol) are rescaled only for the change of
// the weight units, and the running weight of the open group (ecarry) with
// the max.
template <int D>
__device__ inline void update_fwd(RunState<D> &st, float m_g, uint32_t vmx, int lkf, bool dcol, float &ecarry)
{
    constexpr int NCC = D / 16, NP = D / 64;
    const int ev = (vmx >> 10) == 0 ? -14 : (int)(vmx >> 10) - 15;
    const int beta_g = (vmx == 0 ? 24 - lkf : 10 - lkf - ev) - kLazyMax;
    const float m_new = m_g > st.m + (float)kLazyMax ? m_g : st.m;
    const int beta_new = min(st.beta, beta_g);
    const float a_m = __builtin_amdgcn_exp2f(st.m - m_new);
    if (__any(m_new != st.m || beta_new != st.beta)) {
        st.bsc = ldexpf(1.0f, beta_new);
        const float ab = ldexpf(1.0f, beta_new - st.beta);
        const float alpha = dcol ? ab : a_m * ab;
#pragma unroll
        for (int cc = 0; cc < NCC; ++cc) st.acc[cc] *= alpha;
#pragma unroll
        for (int p = 0; p < NP; ++p) st.Z[p] *= alpha;
        st.l *= a_m;
        ecarry *= a_m;
    }
    st.m = m_new;
    st.beta = beta_new;
}

// V phase of one tile of a long group in the forward kernel: the weight of
// token t's codes is -E_t (E_t: the weight of the group's tokens before t,
// ecarry from the earlier tiles), 1 in the delta-sum column; the group's
// keyframe slot (token 0 of its first tile) gets none.  Returns the tile's
// weight sum.
template <int D, bool FULL>
__device__ inline float v_phase_fwd(RunState<D> &st, const uint32_t *vc, const uint8_t *sb, const float (&Lg)[4],
                                    int nval, int j, int n, float c2E, h8 AZ, float ecarry, bool first, bool dcol)
{
    const int h2 = n >> 3;
    const int tb = 16 * h2 + 4 * j;
    float S[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(Lg[i], c2E, -st.m));
        S[i] = (FULL || tb + i < nval) ? p : 0.0f;
    }
    // exclusive prefix: in-lane, over rows j, then the first half's total
    const float s01 = S[0] + S[1], s012 = s01 + S[2], s0123 = s012 + S[3];
    float incl, all;
    rows_prefix(s0123, j, incl, all);
    const float allx = other_half(all);
    const float Pt = all + allx;
    const float off = (incl - s0123) + (h2 ? allx : 0.0f) + ecarry;
    const float E[4] = {off, off + S[0], off + s01, off + s012};
    st.l += Pt;
    const float bsc = st.bsc, bsc16 = 16.0f * bsc;
    float Sp[2][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float w = dcol ? 1.0f : -E[i];
        const float y = w * ((i & 1) ? bsc : bsc16);
        const float x = other_half(y);
        Sp[0][i] = h2 ? x : y;
        Sp[1][i] = h2 ? y : x;
    }
    Sp[0][0] = (first && j == 0) ? 0.0f : Sp[0][0];      // keyframe slot
    v_accumulate_g8<D, FULL>(st, vc, sb, Sp, nval, j, n, AZ);
    return Pt;
}

// Close a group in the forward kernel: every head adds P (the group's total
// weight) times its keyframe (vkf: the group's V keyframe, 2D bytes in LDS)
// plus the group's delta sum, which the delta-sum column's lane of the same
// row and column half passes through LDS (rbuf, 8 x D/16 f4); the column then
// starts the next group at zero.  The barrier keeps the other lanes' reads
// after those stores: the stores are conditional, and without it the compiler
// may move a lane's read ahead of another lane's store (for the hardware one
// wave's LDS accesses are in order; for the compiler they are separate threads).
template <int D>
__device__ inline void group_end_fwd(RunState<D> &st, f4 *rbuf, const uint8_t *vkf, float P, int j, int n, bool dcol)
{
    constexpr int NCC = D / 16, NP = D / 64;
    f4 *rb = rbuf + ((n >> 3) * 4 + j) * NCC;
    if (dcol) {
#pragma unroll
        for (int cc = 0; cc < NCC; ++cc) rb[cc] = st.acc[cc] + st.Z[cc >> 2];
    }
    __syncthreads();
#pragma unroll
    for (int cc = 0; cc < NCC; ++cc) {
        const f4 r = rb[cc];
#pragma unroll
        for (int i = 0; i < 4; ++i) st.acc[cc][i] = __builtin_fmaf(P, r[i], st.acc[cc][i]);
    }
    kf_fma_g8<D>(st, vkf, P * (st.bsc * 0x1p-20f), j);
#pragma unroll
    for (int cc = 0; cc < NCC; ++cc)
#pragma unroll
        for (int i = 0; i < 4; ++i) st.acc[cc][i] = dcol ? 0.0f : st.acc[cc][i];
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int i = 0; i < 4; ++i) st.Z[p][i] = dcol ? 0.0f : st.Z[p][i];
}

// Fetch of one tile part: the side data (per-lane offset with the tile's
// term folded in) and the K code pieces, or the V code words; `soff` is the
// tile's offset in the code planes.
template <int D>
__device__ inline void load_tile_k(G8KRegs<D> &r, const uint8_t *rec, int rec_bytes, int side, int k0, int k1,
                                   int soff)
{
    constexpr int NB = D / 32;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void *)rec, (short)0, rec_bytes, 0x00020000);
    r.side = __builtin_amdgcn_raw_buffer_load_b128(rs, side, 0, kStream);
    if constexpr (NB == 4) {
        const u4 a = __builtin_amdgcn_raw_buffer_load_b128(rs, k0, soff, kStream);
        const u4 c = __builtin_amdgcn_raw_buffer_load_b128(rs, k1, soff, kStream);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            r.kc[k] = a[k];
            r.kc[NB + k] = c[k];
        }
    } else {
        const u2 a = __builtin_amdgcn_raw_buffer_load_b64(rs, k0, soff, kStream);
        const u2 c = __builtin_amdgcn_raw_buffer_load_b64(rs, k1, soff, kStream);
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            r.kc[k] = a[k];
            r.kc[NB + k] = c[k];
        }
    }
}
template <int D>
__device__ inline void load_tile_v(G8VRegs<D> &r, const uint8_t *rec, int rec_bytes, int v, int soff)
{
    constexpr int NCC = D / 16;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void *)rec, (short)0, rec_bytes, 0x00020000);
#pragma unroll
    for (int q4 = 0; q4 < NCC / 4; ++q4) {
        const u4 a = __builtin_amdgcn_raw_buffer_load_b128(rs, v + vcode_piece(D, 0, q4), soff, kStream);
#pragma unroll
        for (int k = 0; k < 4; ++k) r.vc[4 * q4 + k] = a[k];
    }
}

template <int D>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2)))
    k_attn_lfwd_g8(dkv_config cfg, const uint8_t *cache, const int32_t *__restrict__ bt,
                   const float *__restrict__ q, const int32_t *__restrict__ seq_lens, float scale_log2,
                   float *ws, int nsplit, int chunk, CombineTail ct)
{
    constexpr int NB = D / 32, NCC = D / 16;
    constexpr int SIDE_LANES = D / 4;
    constexpr int BATCH = 32;                 // groups per run (runs of at most 2048 tokens, kf >= 64)
    constexpr int LEAD = kG8Lead, NBUF = LEAD + 1;
    static_assert(NBUF == 4, "rounds of 4 steps rotate the 4 fetch buffers");
    constexpr int NSLOT = 4;                  // a tile's side data lives from its staging to its V phase
    const Geom g = make_geom(cfg);
    const int split = grid_split(), h = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x, j = lane >> 4, n = lane & 15;
    const int G = g.G;
    const int kf = g.kf, NT = kf >> 5;
    const int lkf = 32 - __builtin_clz((unsigned)kf - 1u);       // kf <= 2^lkf
    const int L = min(seq_lens[b], g.cap_tokens);
    const int ng = (L + kf - 1) / kf;
    const int g0 = split * chunk, g1 = min(ng, g0 + chunk);
    const int64_t row0 = (int64_t)b * g.Hq + h * G;
    const bool dcol = (n & 7) == 4;           // the delta-sum column of each column half

    __shared__ __attribute__((aligned(16))) uint32_t side[NSLOT][2 * D];
    __shared__ __attribute__((aligned(16))) uint32_t vkf[2][D / 2];     // V keyframes of the open groups
    __shared__ f4 rbuf[8 * NCC];                                       // delta sums at a group's end
    __shared__ int64_t glist[BATCH];
    __shared__ G8Shared<D> sh;
    __shared__ float kls[BATCH * 8];          // keyframe logits [position][head]

    const int x0 = g0 + lane;
    const int64_t o0 = (lane < BATCH && x0 < g1) ? group_offset(g, bt, b, h, x0) : -1;
    const uint64_t mk = __ballot(o0 >= 0);
    const int cnt = __popcll(mk);
    if (cnt == 0) {
        // past the sequence's end: no record (the combine reads only the runs
        // that start before the end), unless this launch merges its records
        if (g0 >= ng && !ct.out) return;
        RunState<D> st;
        init_state<D>(st);
        write_partial_g8<D>(st, ws, row0, G, nsplit, split, lane, j, n, ct.out != nullptr);
        if (ct.out) combine_tail_g8<D>(ws, ct, row0, G, nsplit, (int64_t)b * g.Hkv + h, lane);
        return;
    }
    if (o0 >= 0) glist[__builtin_amdgcn_mbcnt_hi((uint32_t)(mk >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mk, 0u))] = o0;
    __syncthreads();
    // the run's tiles: NT per group, fewer for the sequence's last group; a
    // partial last tile is taken on its own after the pipeline
    const bool lastg = g1 == ng && ng > g0 && ((mk >> (ng - 1 - g0)) & 1) != 0;
    const int ntot = lastg ? (cnt - 1) * NT + ((L - (ng - 1) * kf + 31) >> 5) : cnt * NT;
    const bool last_partial = lastg && (L & 31) != 0;
    const int nfull = ntot - (last_partial ? 1 : 0);
    const uint32_t magic = (65536u + (uint32_t)NT - 1u) / (uint32_t)NT;     // x / NT for x < 65536 / NT
    auto grp = [&](int x) { return (int)(((uint32_t)x * magic) >> 16); };

    // lane offsets in a group record for its first tile (t0) and for later
    // tiles (tn, to which the tile's code offset 16*D*t is added as soffset;
    // the scale lanes of the side data add 64*NB*t)
    const LaneOffsets lo = lane_offsets<D>(g, lane, j, n, true);
    const bool kf_lane = lane < D / 8, vkf_lane = lane >= SIDE_LANES && lane < SIDE_LANES + D / 8;
    const int side_t0 = kf_lane ? 0x40000000 : lo.side;              // K keyframes: read by the prologue
    const int side_tn = (kf_lane || vkf_lane) ? 0x40000000 : lo.side;
    const int side_mul = (lane < 2 * SIDE_LANES && !kf_lane && !vkf_lane) ? 64 * NB : 0;
    const int k0_t0 = lo.k0;                                         // token 0 of the group: zeros
    const int k0_tn = n == 0 ? (int)g.off_kcd - D / 2 + 4 * j * NB : lo.k0;
    const int rec_bytes = (int)g.rec;
    // tile x's record (past the whole tiles: the last whole one again, still in
    // L2; a run of only a partial tile fetches that one)
    auto rec_of = [&](int x) { return cache + uniform_offset(glist, grp(x)); };
    auto clampx = [&](int x) { return x < nfull ? x : max(nfull - 1, 0); };
    auto fetch_k = [&](G8KRegs<D> &r, int x) {
        const int xc = clampx(x), t = xc - grp(xc) * NT;
        load_tile_k<D>(r, rec_of(xc), rec_bytes, (t == 0 ? side_t0 : side_tn) + side_mul * t,
                       t == 0 ? k0_t0 : k0_tn, lo.k1, 16 * D * t);
    };
    auto fetch_v = [&](G8VRegs<D> &r, int x) {
        const int xc = clampx(x), t = xc - grp(xc) * NT;
        load_tile_v<D>(r, rec_of(xc), rec_bytes, lo.v, 16 * D * t);
    };

    // start-up order as in k_attn_g8
    G8KRegs<D> kb[NBUF];
    G8VRegs<D> vb[NBUF];
    G8Ops op;
    float qs[NB];
    float c2E;
    auto prologue = [&](auto nset_c) {
        constexpr int NS = decltype(nset_c)::value;
        fetch_k(kb[0], 0);
        fetch_v(vb[0], 0);
        fetch_k(kb[1], 1);
        float qraw[D / 64][8];
        load_q_g8<D>(qraw, q, row0, G, j, n);
        u4 kfa[NS][NB];
        kf_load_g8<D, NS>(kfa, glist, cnt, cache, j, n);
        c2E = setup_g8<D>(sh, op, qraw, G, scale_log2, j, n, qs);
        kf_logits_g8<D, NS>(kls, kfa, cnt, op, j, n);
        fetch_v(vb[1], 1);
        fetch_k(kb[2], 2);
        fetch_v(vb[2], 2);
        fetch_k(kb[3], 3);
    };
    if (cnt <= 16)
        prologue(IC<1>{});
    else
        prologue(IC<2>{});
    const h8 AZ = v_minus8_operand();
    f4 kbias[NB];
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
        const float xb = -8.0f * 0x1p-20f * qs[bb];
        kbias[bb] = f4{xb, xb, xb, xb};
    }
    auto klog = [&](int k) { return kls[k * 8 + (n & 7)]; };
    const float c2Eu = c2E * 1048576.0f;
    h8 qh[2][NB];
#pragma unroll
    for (int T = 0; T < 2; ++T)
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) qh[T][bb] = as_h8(op.qk[T][(2 * bb) * 32]);

    RunState<D> st;
    init_state<D>(st);
    float ecarry = 0.0f;                      // weight of the open group's earlier tokens
    float kcin = 0.0f, kcarry = 0.0f;         // logit carry into the last K phase, and out of it
    uint32_t vmx = 0;                         // the open group's largest |V scale|

    auto sbp = [&](int x) { return (const uint8_t *)side[x & (NSLOT - 1)]; };
    // staging of tile x (group k, tile t of it) in slot x % NSLOT: its side
    // data, and for a group's first tile its V keyframe, kept for the group's end
    auto stage_at = [&](const G8KRegs<D> &r, int x, int k, int t) {
        if (2 * SIDE_LANES == 64 || lane < 2 * SIDE_LANES) ((u4 *)side[x & (NSLOT - 1)])[fresh_lane_id()] = r.side;
        if (t == 0 && vkf_lane) ((u4 *)vkf[k & 1])[lane - SIDE_LANES] = r.side;
    };
    auto stage = [&](const G8KRegs<D> &r, int x) {
        const int xc = clampx(x), k = grp(xc);
        stage_at(r, x, k, xc - k * NT);
    };
    // K phase of tile x (FULL) with its carry; x past the whole tiles repeats
    // the last one with the carry it had, so its maximum changes nothing
    auto kphase = [&](const G8KRegs<D> &r, int x, float (&Lg)[4]) {
        const bool past = x >= nfull;
        const int xc = clampx(x), k = grp(xc), t = xc - k * NT;
        const bool first = t == 0;
        const float cin = past ? kcin : first ? klog(k) : kcarry;
        float tot;
        const float m = k_phase_g8b<D, true>(r.kc, sbp(x), 32, j, n, op, qh, kbias, c2Eu, cin, Lg, first, tot);
        kcin = cin;
        kcarry = cin + tot;
        vmx = first ? group_vmax<D>(sbp(x)) : vmx;
        update_fwd<D>(st, m, vmx, lkf, dcol, ecarry);
    };
    // after tile x's V phase (its weight already in ecarry) and the next K
    // phase's update: close x's group at the group's last tile
    auto close = [&](int x) {
        const int k = grp(x), t = x - k * NT;
        if (t == NT - 1 || x == ntot - 1) {
            group_end_fwd<D>(st, rbuf, (const uint8_t *)vkf[k & 1], ecarry, j, n, dcol);
            ecarry = 0.0f;
        }
    };

    if (nfull > 0) {
        float Lg[4];
        __syncthreads();
        stage(kb[0], 0);
        stage(kb[1], 1);
        __syncthreads();
        kphase(kb[0], 0, Lg);
        // step x (u = x % NBUF): fetch the K part of tile x + 1 + LEAD and the V
        // part of tile x + LEAD, V phase of x, K phase of x + 1, stage x + 2;
        // then close x's group if x is its last tile
        auto step = [&](int x, auto uc) {
            constexpr int u = decltype(uc)::value;
            constexpr int un = (u + 1) % NBUF, u2 = (u + 2) % NBUF, ulast = (u + LEAD) % NBUF;
            fetch_k(kb[u], x + 1 + LEAD);
            fetch_v(vb[ulast], x + LEAD);
            const int t = x - grp(x) * NT;
            ecarry += v_phase_fwd<D, true>(st, vb[u].vc, sbp(x) + 4 * D, Lg, 32, j, n, c2Eu, AZ, ecarry, t == 0,
                                           dcol);
            // (the V phase reads Lg before the K phase of x + 1 overwrites it)
            kphase(kb[un], x + 1, Lg);
            stage(kb[u2], x + 2);
            close(x);
        };
        const bool older = (blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z)) <
                           (gridDim.x * gridDim.y * gridDim.z) / 2;
        const int q1 = nfull >> 2, q2 = nfull >> 1, q3 = (3 * nfull) >> 2;
        if (older) __builtin_amdgcn_s_setprio(2); else __builtin_amdgcn_s_setprio(3);
        const int nround = nfull / NBUF, nrest = nfull % NBUF;
        for (int r = 0; r < nround; ++r) {
            const int x = r * NBUF;
            if (x >= q1) {
                const int lvl = (x >= q3 ? 0 : x >= q2 ? 1 : 2) - (older ? 1 : 0);
                if (lvl <= 0)
                    __builtin_amdgcn_s_setprio(0);
                else if (lvl == 1)
                    __builtin_amdgcn_s_setprio(1);
                else
                    __builtin_amdgcn_s_setprio(2);
            }
            step(x, IC<0>{});
            step(x + 1, IC<1>{});
            step(x + 2, IC<2>{});
            step(x + 3, IC<3>{});
        }
        if (nrest > 0) {
            const int x = nround * NBUF;
            step(x, IC<0>{});
            if (nrest > 1) step(x + 1, IC<1>{});
            if (nrest > 2) step(x + 2, IC<2>{});
        }
        __builtin_amdgcn_s_setprio(0);
    }
    if (last_partial) {
        const int x = ntot - 1, k = grp(x), t = x - k * NT;
        G8KRegs<D> kr;
        G8VRegs<D> vr;
        const uint8_t *rec = cache + uniform_offset(glist, k);
        load_tile_k<D>(kr, rec, rec_bytes, (t == 0 ? side_t0 : side_tn) + side_mul * t, t == 0 ? k0_t0 : k0_tn,
                       lo.k1, 16 * D * t);
        load_tile_v<D>(vr, rec, rec_bytes, lo.v, 16 * D * t);
        __syncthreads();
        stage_at(kr, x, k, t);
        __syncthreads();
        const int nval = L - (ng - 1) * kf - 32 * t;
        const float cin = t == 0 ? klog(k) : kcarry;
        float Lg[4], tot;
        const float m = k_phase_g8b<D, false>(kr.kc, sbp(x), nval, j, n, op, qh, kbias, c2Eu, cin, Lg, t == 0, tot);
        vmx = t == 0 ? group_vmax<D>(sbp(x)) : vmx;
        update_fwd<D>(st, m, vmx, lkf, dcol, ecarry);
        ecarry += v_phase_fwd<D, false>(st, vr.vc, sbp(x) + 4 * D, Lg, nval, j, n, c2Eu, AZ, ecarry, t == 0, dcol);
        close(x);
    }
    write_partial_g8<D>(st, ws, row0, G, nsplit, split, lane, j, n, ct.out != nullptr);
    if (ct.out) combine_tail_g8<D>(ws, ct, row0, G, nsplit, (int64_t)b * g.Hkv + h, lane);
}

// With `append` (kf = 32 only), the kernel appends each sequence's new token
// before it decodes: append->positions null means no append.
// With `tail` (non-null out), the kernel also merges the partial records
// into out (one launch per decode step).
hipError_t launch_attn_g8(const dkv_config &c, const void *cache, const int32_t *bt, const float *q,
                          const int32_t *lens, float scale_log2, float *ws, int nsplit, int chunk, hipStream_t st,
                          const AppendArgs *append, CombineTail ct)
{
    dim3 grid(nsplit, c.n_kv_heads, c.batch);
    if (c.kf == 32) {
        if (chunk > 64) return hipErrorInvalidValue;     // a run's group list holds 64 groups
        const AppendArgs ap = append ? *append : AppendArgs{nullptr, nullptr, nullptr, nullptr, nullptr};
        if (c.head_dim == 64)
            hipLaunchKernelGGL(k_attn_g8<64>, grid, dim3(64), 0, st, c, (const uint8_t *)cache, bt, q, lens,
                               scale_log2, ws, nsplit, chunk, ap, ct);
        else
            hipLaunchKernelGGL(k_attn_g8<128>, grid, dim3(64), 0, st, c, (const uint8_t *)cache, bt, q, lens,
                               scale_log2, ws, nsplit, chunk, ap, ct);
    } else {
        if (append && append->positions) return hipErrorInvalidValue;     // the long-interval kernels do not append
        if (chunk > 64) return hipErrorInvalidValue;     // a run's groups are counted over one wave
        if (c.n_q_heads / c.n_kv_heads <= 4 && chunk <= 32) {
            // one forward pass (operand column 4 is spare)
            if (c.head_dim == 64)
                hipLaunchKernelGGL(k_attn_lfwd_g8<64>, grid, dim3(64), 0, st, c, (const uint8_t *)cache, bt, q, lens,
                                   scale_log2, ws, nsplit, chunk, ct);
            else
                hipLaunchKernelGGL(k_attn_lfwd_g8<128>, grid, dim3(64), 0, st, c, (const uint8_t *)cache, bt, q, lens,
                                   scale_log2, ws, nsplit, chunk, ct);
            return hipGetLastError();
        }
        // logit rows (see the kernel): 32 per tile and a spare row when at most
        // 4 query heads share a kv-head, 64 per tile otherwise
        const int nt = (c.kf + 31) / 32;
        const size_t lds = (c.n_q_heads / c.n_kv_heads <= 4 ? (size_t)nt * 32 + 1 : (size_t)nt * 64) * sizeof(f4);
        if (c.head_dim == 64)
            hipLaunchKernelGGL(k_attn_long_g8<64>, grid, dim3(64), lds, st, c, (const uint8_t *)cache, bt, q, lens,
                               scale_log2, ws, nsplit, chunk, ct);
        else
            hipLaunchKernelGGL(k_attn_long_g8<128>, grid, dim3(64), lds, st, c, (const uint8_t *)cache, bt, q, lens,
                               scale_log2, ws, nsplit, chunk, ct);
    }
    return hipGetLastError();
}

// ============================================================ plain Q4_0, GQA <= 8
// The same layout tricks on the plain Q4_0 comparison cache: one 32-token tile
// per step, the next tile fetched while the current one is processed.  The
// tile's largest |V scale| (the V weight range) is reduced over the wave.
// DELTA: the Q4-keyframe cache at kf = 32 in the same tiles (row 0 of each tile
// coded against zero, rows 1..31 closed-loop deltas): the logits take prefix
// sums and the weights suffix sums over the tile, both starting at zero, and
// the V weight range allows suffix sums of up to 32 weights.
template <int D, bool DELTA>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2)))
    k_attn_q40_g8(dkv_config cfg, const uint8_t *__restrict__ q4, const int32_t *__restrict__ bt,
                  const float *__restrict__ q, const int32_t *__restrict__ seq_lens, float scale_log2,
                  float *__restrict__ ws, int nsplit, int chunk)
{
    constexpr int NB = D / 32;
    const int split = grid_split(), h = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x, j = lane >> 4, n = lane & 15;
    const int G = cfg.n_q_heads / cfg.n_kv_heads;
    const int L = min(seq_lens[b], q40_ntiles(cfg) * 32);
    const int nt = (L + 31) >> 5;
    const int t0 = split * chunk, t1 = min(nt, t0 + chunk);
    const int64_t row0 = (int64_t)b * cfg.n_q_heads + h * G;
    if (t0 >= nt) return;                  // past the sequence's end: no record (the combine skips it)
    const int tbytes = (int)q40_tile_bytes(D);

    // [unused 2D][K scales 2D][unused 2D][V scales 2D]: the side layout of the phases
    __shared__ __attribute__((aligned(16))) uint32_t side[2 * D];
    __shared__ G8Shared<D> sh;
    // the run's mapped tiles (a run has at most 64: the split plan caps it),
    // listed with their byte offsets; paged mode may leave pages unmapped
    __shared__ int64_t toffs[64];
    __shared__ int tnum[64];
    int ntl = max(t1 - t0, 0);              // contiguous: every tile of the run is mapped
    if (bt) {
        const int x = t0 + lane;
        const int64_t o = x < t1 ? q40_tile_offset(cfg, bt, b, h, x) : -1;
        const uint64_t mk = __ballot(o >= 0);
        ntl = __popcll(mk);
        if (o >= 0) {
            const int pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(mk >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mk, 0u));
            toffs[pos] = o;
            tnum[pos] = x;
        }
        __syncthreads();
    }

    G8Ops op;
    float qraw[D / 64][8];
    load_q_g8<D>(qraw, q, row0, G, j, n);
    const float c2E = setup_g8<D>(sh, op, qraw, G, scale_log2, j, n);
    const h8 AZ = v_minus8_operand();
    RunState<D> st;
    init_state<D>(st);

    // per-lane offsets inside a tile
    const int so = (lane >= D / 8 && lane < D / 4) ? 16 * (lane - D / 8)
                 : (lane >= 3 * D / 8 && lane < D / 2) ? 18 * D + 16 * (lane - 3 * D / 8) : 0x40000000;
    const int ok0 = 2 * D + n * (D / 2) + 4 * j * NB;
    const int ok1 = 2 * D + (16 + n) * (D / 2) + 4 * j * NB;
    const int ov = 20 * D + vcode_piece(D, lane, 0);
    auto load_tile = [&](G8Regs<D> &r, int k) {
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(q4 + (bt ? uniform_offset(toffs, k) : q40_tile_offset(cfg, nullptr, b, h, t0 + k))), (short)0,
            tbytes, 0x00020000);
        r.side = __builtin_amdgcn_raw_buffer_load_b128(rs, so, 0, kStream);
        if constexpr (NB == 4) {
            const u4 a = __builtin_amdgcn_raw_buffer_load_b128(rs, ok0, 0, kStream);
            const u4 c = __builtin_amdgcn_raw_buffer_load_b128(rs, ok1, 0, kStream);
            const u4 v0 = __builtin_amdgcn_raw_buffer_load_b128(rs, ov, 0, kStream);
            const u4 v1 = __builtin_amdgcn_raw_buffer_load_b128(rs, ov + vcode_piece(D, 0, 1), 0, kStream);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                r.kc[k] = a[k];
                r.kc[4 + k] = c[k];
                r.vc[k] = v0[k];
                r.vc[4 + k] = v1[k];
            }
        } else {
            const u2 a = __builtin_amdgcn_raw_buffer_load_b64(rs, ok0, 0, kStream);
            const u2 c = __builtin_amdgcn_raw_buffer_load_b64(rs, ok1, 0, kStream);
            const u4 v0 = __builtin_amdgcn_raw_buffer_load_b128(rs, ov, 0, kStream);
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                r.kc[k] = a[k];
                r.kc[2 + k] = c[k];
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) r.vc[k] = v0[k];
        }
    };
    auto run = [&](const G8Regs<D> &r, int k) {
        const int tl = bt ? __builtin_amdgcn_readfirstlane(tnum[k]) : t0 + k;    // contiguous: every tile mapped
        __syncthreads();
        if (lane < D / 2) ((u4 *)side)[fresh_lane_id()] = r.side;
        __syncthreads();
        const uint8_t *sb = (const uint8_t *)side;
        const int nval = min(32, L - 32 * tl);
        // largest |V scale| of the tile (2*D bytes = D/2 words over the wave)
        uint32_t vmx;
        {
            const uint32_t w = ((const uint32_t *)(sb + 6 * D))[lane & (D / 2 - 1)];
            const int valid_tok = (lane & (D / 2 - 1)) / (NB / 2) < nval;
            const uint32_t a = valid_tok ? (w & 0x7FFF7FFFu) : 0u;
            float m = (float)max(a & 0xFFFFu, a >> 16);
            m = rows_max(m);
#pragma unroll
            for (int sh2 = 8; sh2 >= 1; sh2 >>= 1)
                m = fmaxf(m, __shfl_xor(m, sh2, 16));
            vmx = (uint32_t)m;
        }
        float Lg[4], tot;
        const u4 *none = sh.qz;
        float mt;
        if (nval == 32)
            mt = k_phase_g8<D, true, false, DELTA>(r.kc, sb, none, nval, j, n, op, c2E, 0.0f, Lg, tot);
        else
            mt = k_phase_g8<D, false, false, DELTA>(r.kc, sb, none, nval, j, n, op, c2E, 0.0f, Lg, tot);
        float no_kf = 0.0f;
        update_g8_vmx<D>(st, mt, vmx, DELTA ? 5 : 0, no_kf);       // weights (suffix sums) <= 2^lkf
        if (nval == 32)
            v_phase_g8<D, true, false, DELTA>(st, r.vc, sb + 4 * D, Lg, nval, j, n, c2E, AZ, 0.0f);
        else
            v_phase_g8<D, false, false, DELTA>(st, r.vc, sb + 4 * D, Lg, nval, j, n, c2E, AZ, 0.0f);
    };
    if (ntl > 0) {
        G8Regs<D> ra, rb;
        int k = 0;
        load_tile(ra, k);
        auto step = [&](const G8Regs<D> &cur, G8Regs<D> &pf) {
            // prefetch unconditionally (past the end: the current tile again)
            load_tile(pf, k + 1 < ntl ? k + 1 : k);
            run(cur, k);
            ++k;
            return k < ntl;
        };
        while (step(ra, rb) && step(rb, ra)) {
        }
    }
    write_partial_g8<D>(st, ws, row0, G, nsplit, split, lane, j, n, false);
}

// delta: the Q4-keyframe cache at kf = 32 (see the kernel)
hipError_t launch_attn_q40_g8(const dkv_config &c, const void *q4, const int32_t *bt, const float *q,
                              const int32_t *lens, float scale_log2, float *ws, int nsplit, int chunk, hipStream_t st,
                              bool delta)
{
    if (chunk > 64) return hipErrorInvalidValue;      // the kernel lists at most 64 tiles per run
    dim3 grid(nsplit, c.n_kv_heads, c.batch);
    const uint8_t *p = (const uint8_t *)q4;
    if (c.head_dim == 64) {
        if (delta)
            hipLaunchKernelGGL((k_attn_q40_g8<64, true>), grid, dim3(64), 0, st, c, p, bt, q, lens, scale_log2, ws,
                               nsplit, chunk);
        else
            hipLaunchKernelGGL((k_attn_q40_g8<64, false>), grid, dim3(64), 0, st, c, p, bt, q, lens, scale_log2, ws,
                               nsplit, chunk);
    } else {
        if (delta)
            hipLaunchKernelGGL((k_attn_q40_g8<128, true>), grid, dim3(64), 0, st, c, p, bt, q, lens, scale_log2, ws,
                               nsplit, chunk);
        else
            hipLaunchKernelGGL((k_attn_q40_g8<128, false>), grid, dim3(64), 0, st, c, p, bt, q, lens, scale_log2, ws,
                               nsplit, chunk);
    }
    return hipGetLastError();
}

}  // namespace dkv
