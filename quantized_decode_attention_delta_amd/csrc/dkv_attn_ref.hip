// Reference fused decode attention over the Delta-KV cache (fp32, VALU), and
// the split-K combine shared by every decode-attention kernel of the library.
//
// Attention follows the definition on the page "KV 캐시 벡터 양자화와 주의 보존
// 변환" (section "왜 복원 오차가 틀린 기준인가"): logits q.K^T * scale, a
// softmax over the cached tokens, then the weighted sum of V rows.  This
// kernel rebuilds each 32-token tile of K and V in fp32 (the same bit-exact
// fold as the decoder) into LDS and runs plain fp32 attention with an online
// softmax; it is the straightforward counterpart of the matrix-core kernel.
//
// Split-K ("flash-decoding"): the groups of a sequence are cut into runs of
// whole groups (every group decodes from its own keyframe); each workgroup
// writes a partial (acc[D], m, l) with m in log2 units, and k_combine merges
// them.
#include "dkv_common.h"

namespace dkv {

constexpr int kRefThreads = 256;
constexpr int kMaxG = 16;

template <int D>
__device__ inline int ref_code(const uint8_t *cd, int s, int r, int c, int bp)
{
    if (s == 0) {
        const int cb = c & 31;
        const uint8_t byte = cd[(int64_t)(r - 1) * (D / 2) + kcode_byte(D / 32, c >> 5, cb & 15)];
        return (byte >> (4 * (cb >> 4))) & 15;
    }
    const int tau = r & 31;
    const uint32_t w = ((const uint32_t *)(cd + (int64_t)(r >> 5) * 16 * D))[vcode_word(D, tau, c, bp)];
    return (w >> (4 * vcode_nibble(tau))) & 15;
}

template <int D>
__global__ void __launch_bounds__(kRefThreads)
    k_attn_ref(dkv_config cfg, const uint8_t *cache, const int32_t *bt, const float *q,
               const int32_t *seq_lens, float scale_log2, float *ws, int nsplit, int chunk)
{
    constexpr int nb = D / 32;
    constexpr int ACC = (kMaxG * D + kRefThreads - 1) / kRefThreads;
    const Geom g = make_geom(cfg);
    const int split = grid_split(), h = blockIdx.y, b = blockIdx.z;
    const int G = g.G;
    const int tid = threadIdx.x;
    const int L = min(seq_lens[b], g.cap_tokens);
    const int ng = (L + g.kf - 1) / g.kf;
    const int g0 = split * chunk, g1 = min(ng, g0 + chunk);

    __shared__ float sK[32][D];
    __shared__ float sV[32][D];
    __shared__ float sq[kMaxG][D];
    __shared__ float sl[kMaxG][33];
    __shared__ float sm[kMaxG], sls[kMaxG], salpha[kMaxG];

    for (int i = tid; i < G * D; i += kRefThreads)
        sq[i / D][i % D] = q[((int64_t)b * g.Hq + h * G) * D + i] * scale_log2;
    if (tid < G) { sm[tid] = -INFINITY; sls[tid] = 0.0f; }
    float acc[ACC];
#pragma unroll
    for (int k = 0; k < ACC; ++k) acc[k] = 0.0f;
    __syncthreads();

    const int rs = tid / D;              // 0: K, 1: V (threads >= 2D idle in the fold)
    const int rc = tid % D;
    for (int gi = g0; gi < g1; ++gi) {
        const int64_t off = group_offset(g, bt, b, h, gi);
        if (off < 0) continue;              // unmapped page: uniform over the block
        const uint8_t *rec = cache + off;
        const uint8_t *pkf = rec + (rs ? g.off_vkf : 0);
        const uint16_t *psc = (const uint16_t *)(rec + (rs ? g.off_vsc : g.off_ksc));
        const uint8_t *pcd = rec + (rs ? g.off_vcd : g.off_kcd);
        const int ngt = min(g.kf, L - gi * g.kf);
        float xh = 0.0f;
        for (int tok0 = 0; tok0 < ngt; tok0 += 32) {
            const int nt = min(32, ngt - tok0);
            if (rs < 2) {
                for (int tt = 0; tt < nt; ++tt) {
                    const int r = tok0 + tt;
                    if (r == 0) {
                        xh = h2f(((const uint16_t *)pkf)[rs ? vkf_pos(D, rc, g.vbp) : kkf_pos(nb, rc)]);
                    } else {
                        const int code = ref_code<D>(pcd, rs, r, rc, g.vbp);
                        const float sf = h2f(psc[r * nb + (rc >> 5)]);
                        xh = __fadd_rn(xh, __fmul_rn((float)(code - 8), sf));
                    }
                    if (rs == 0) sK[tt][rc] = xh; else sV[tt][rc] = xh;
                }
            }
            __syncthreads();
            for (int i = tid; i < G * 32; i += kRefThreads) {
                const int hh = i >> 5, tt = i & 31;
                float dot = -INFINITY;
                if (tt < nt) {
                    dot = 0.0f;
                    for (int c = 0; c < D; ++c) dot = fmaf(sq[hh][c], sK[tt][c], dot);
                }
                sl[hh][tt] = dot;
            }
            __syncthreads();
            if (tid < G) {
                float mx = sm[tid];
                for (int tt = 0; tt < nt; ++tt) mx = fmaxf(mx, sl[tid][tt]);
                const float alpha = exp2f(sm[tid] - mx);
                float sum = 0.0f;
                for (int tt = 0; tt < nt; ++tt) {
                    const float p = exp2f(sl[tid][tt] - mx);
                    sl[tid][tt] = p;
                    sum += p;
                }
                sls[tid] = sls[tid] * alpha + sum;
                sm[tid] = mx;
                salpha[tid] = alpha;
            }
            __syncthreads();
#pragma unroll
            for (int k = 0; k < ACC; ++k) {
                const int i = tid + k * kRefThreads;
                if (i < G * D) {
                    const int hh = i / D, c = i % D;
                    float a = acc[k] * salpha[hh];
                    for (int tt = 0; tt < nt; ++tt) a = fmaf(sl[hh][tt], sV[tt][c], a);
                    acc[k] = a;
                }
            }
            __syncthreads();
        }
    }
    // partial record: acc[D], m, l
#pragma unroll
    for (int k = 0; k < ACC; ++k) {
        const int i = tid + k * kRefThreads;
        if (i < G * D) {
            const int hh = i / D, c = i % D;
            ws[(((int64_t)b * g.Hq + h * G + hh) * nsplit + split) * part_stride(D) + c] = acc[k];
        }
    }
    if (tid < G) {
        float *rec = ws + (((int64_t)b * g.Hq + h * G + tid) * nsplit + split) * part_stride(D);
        rec[D] = sm[tid];
        rec[D + 1] = sls[tid];
    }
}

// Merge split partials: grid (B*Hq), four wavefronts per output row; lane c
// holds channels c and c+64.  Wave w merges splits w, w+4, w+8, ...: all loads
// of a run of 8 of its splits are issued before the merge arithmetic, so a row
// costs about one memory round trip per 32 splits.  The four waves' (max, sum,
// numerators) are then merged through LDS by wave 0.  Only the splits whose
// run starts before the sequence's end are read: ceil(min(len, cap) /
// split_tokens) of them.
constexpr int kCombineWaves = 4;

template <int D>
__global__ void __launch_bounds__(64 * kCombineWaves) k_combine(const float *__restrict__ ws, int nsplit,
                                                                float *__restrict__ out,
                                                                const int32_t *__restrict__ lens, int Hq,
                                                                int cap_tokens, int split_tokens)
{
    constexpr int R = part_stride(D);
    constexpr int NCH = D / 64;
    const int64_t row = blockIdx.x;
    const int c = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int L = max(0, min(lens[row / Hq], cap_tokens));
    const int used = min(nsplit, (L + split_tokens - 1) / split_tokens);
    const float *p = ws + row * nsplit * R;
    float M = -INFINITY, den = 0.0f, num[NCH];
#pragma unroll
    for (int k = 0; k < NCH; ++k) num[k] = 0.0f;
    for (int s0 = wv; s0 < used; s0 += 8 * kCombineWaves) {
        float ms[8], ls[8], a[8][NCH];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int sp = s0 + u * kCombineWaves;
            const bool ok = sp < used;
            const float *r = p + (int64_t)(ok ? sp : 0) * R;
            ms[u] = r[D];
            ls[u] = ok ? r[D + 1] : 0.0f;
#pragma unroll
            for (int k = 0; k < NCH; ++k) a[u][k] = r[c + 64 * k];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (ls[u] > 0.0f) {
                const float mn = fmaxf(M, ms[u]);
                const float al = exp2f(M - mn), w = exp2f(ms[u] - mn);
#pragma unroll
                for (int k = 0; k < NCH; ++k) num[k] = fmaf(w, a[u][k], num[k] * al);
                den = fmaf(w, ls[u], den * al);
                M = mn;
            }
        }
    }
    __shared__ float sM[kCombineWaves], sden[kCombineWaves], snum[kCombineWaves][D];
    if (c == 0) {
        sM[wv] = M;
        sden[wv] = den;
    }
#pragma unroll
    for (int k = 0; k < NCH; ++k) snum[wv][c + 64 * k] = num[k];
    __syncthreads();
    if (wv == 0) {
        M = -INFINITY;
        den = 0.0f;
#pragma unroll
        for (int k = 0; k < NCH; ++k) num[k] = 0.0f;
#pragma unroll
        for (int w2 = 0; w2 < kCombineWaves; ++w2) {
            const float l2 = sden[w2];
            if (l2 > 0.0f) {
                const float mn = fmaxf(M, sM[w2]);
                const float al = exp2f(M - mn), w = exp2f(sM[w2] - mn);
#pragma unroll
                for (int k = 0; k < NCH; ++k) num[k] = fmaf(w, snum[w2][c + 64 * k], num[k] * al);
                den = fmaf(w, l2, den * al);
                M = mn;
            }
        }
#pragma unroll
        for (int k = 0; k < NCH; ++k) out[row * D + c + 64 * k] = den > 0.0f ? num[k] / den : 0.0f;
    }
}

hipError_t launch_attn_ref(const dkv_config &c, const void *cache, const int32_t *bt, const float *q,
                           const int32_t *lens, float scale_log2, float *ws, int nsplit, int chunk,
                           hipStream_t st)
{
    dim3 grid(nsplit, c.n_kv_heads, c.batch);
    if (c.head_dim == 64)
        hipLaunchKernelGGL(k_attn_ref<64>, grid, dim3(kRefThreads), 0, st, c, (const uint8_t *)cache, bt,
                           q, lens, scale_log2, ws, nsplit, chunk);
    else
        hipLaunchKernelGGL(k_attn_ref<128>, grid, dim3(kRefThreads), 0, st, c, (const uint8_t *)cache, bt,
                           q, lens, scale_log2, ws, nsplit, chunk);
    return hipGetLastError();
}

hipError_t launch_combine(const dkv_config &c, const float *ws, int nsplit, float *out, const int32_t *lens,
                          int cap_tokens, int split_tokens, hipStream_t st)
{
    if (split_tokens < 1) return hipErrorInvalidValue;
    dim3 grid(c.batch * c.n_q_heads);
    if (c.head_dim == 64)
        hipLaunchKernelGGL(k_combine<64>, grid, dim3(64 * kCombineWaves), 0, st, ws, nsplit, out, lens, c.n_q_heads,
                           cap_tokens, split_tokens);
    else
        hipLaunchKernelGGL(k_combine<128>, grid, dim3(64 * kCombineWaves), 0, st, ws, nsplit, out, lens,
                           c.n_q_heads, cap_tokens, split_tokens);
    return hipGetLastError();
}

}  // namespace dkv
