// Diagnostic: attention-preserving distortion of a reconstructed KV cache
// ("KV 캐시 벡터 양자화와 주의 보존 변환", section 어텐션 보존 왜곡).  The page
// measures a cache by what attention sees rather than by ||Khat - K||:
//   d_k = || q.Khat^T - q.K^T ||^2      (the logit row, unscaled dot products)
//   d_v = || A.Vhat - A.V ||^2          (A: the attention weights)
// per (sequence, query head) of one decode step, with A = softmax over the
// sequence's tokens of softmax_scale * q.K_t on the exact keys, so that d_v
// isolates the error of the values.
//
// One workgroup of 256 threads per (sequence, query head).  Every term is
// formed from the difference Khat - K (Vhat - V) first: both are fp32 values
// within a few percent of each other, so the difference is exact and the sums
// carry no cancellation.
#include "dkv_common.h"

namespace dkv {

constexpr int kDistThreads = 256;

__device__ inline float block_sum(float x, float *red)
{
    for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = x;
    __syncthreads();
    float s = 0.0f;
    for (int i = 0; i < kDistThreads / 64; ++i) s += red[i];
    return s;
}

__device__ inline float block_max(float x, float *red)
{
    for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[w] = x;
    __syncthreads();
    float s = -INFINITY;
    for (int i = 0; i < kDistThreads / 64; ++i) s = fmaxf(s, red[i]);
    return s;
}

template <int D>
__global__ void __launch_bounds__(kDistThreads)
    k_attn_distortion(int Hq, int Hkv, const float *__restrict__ khat, const float *__restrict__ vhat,
                      const uint16_t *__restrict__ k, const uint16_t *__restrict__ v, int s_max,
                      const float *__restrict__ q, const int32_t *__restrict__ lens, float scale,
                      float *__restrict__ logits, float *__restrict__ dk, float *__restrict__ dv)
{
    constexpr int SL = kDistThreads / D;      // token slices of the value pass
    const int hq = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int h = hq / (Hq / Hkv);
    const int L = min(lens[b], s_max);
    const int64_t row = (int64_t)b * Hq + hq;
    const int64_t base = ((int64_t)b * Hkv + h) * s_max * D;
    __shared__ float qs[D];
    __shared__ float red[kDistThreads / 64];
    __shared__ float part[SL][D];
    for (int c = tid; c < D; c += kDistThreads) qs[c] = q[row * D + c];
    __syncthreads();

    // keys: the logit error of every token, and the exact logits
    float* lrow = logits + row * s_max;
    float sk = 0.0f, mx = -INFINITY;
    for (int t = tid; t < L; t += kDistThreads) {
        const float *kh = khat + base + (int64_t)t * D;
        const uint16_t *kx = k + base + (int64_t)t * D;
        float e = 0.0f, l = 0.0f;
        for (int c = 0; c < D; ++c) {
            const float x = h2f(kx[c]);
            e = __builtin_fmaf(qs[c], kh[c] - x, e);
            l = __builtin_fmaf(qs[c], x, l);
        }
        l *= scale;
        lrow[t] = l;
        sk = __builtin_fmaf(e, e, sk);
        mx = fmaxf(mx, l);
    }
    sk = block_sum(sk, red);
    mx = block_max(mx, red);
    __syncthreads();            // every thread's logits are written before any is read

    float se = 0.0f;
    for (int t = tid; t < L; t += kDistThreads) se += expf(lrow[t] - mx);
    se = block_sum(se, red);

    // values: sum_t a_t (Vhat_t - V_t), channel c by the threads c (mod D)
    const int c = tid % D, sl = tid / D;
    float acc = 0.0f;
    for (int t = sl; t < L; t += SL) {
        const int64_t o = base + (int64_t)t * D + c;
        acc = __builtin_fmaf(expf(lrow[t] - mx), vhat[o] - h2f(v[o]), acc);
    }
    part[sl][c] = acc;
    __syncthreads();
    float y2 = 0.0f;
    if (sl == 0 && L > 0) {
        float y = 0.0f;
        for (int s = 0; s < SL; ++s) y += part[s][c];
        y /= se;
        y2 = y * y;
    }
    y2 = block_sum(y2, red);
    if (tid == 0) {
        dk[row] = L > 0 ? sk : 0.0f;
        dv[row] = y2;
    }
}

hipError_t launch_attn_distortion(const dkv_config &c, const float *khat, const float *vhat, const uint16_t *k,
                                  const uint16_t *v, int s_max, const float *q, const int32_t *lens, float scale,
                                  float *logits, float *dk, float *dv, hipStream_t st)
{
    const dim3 grid(c.n_q_heads, c.batch);
    if (c.head_dim == 64)
        hipLaunchKernelGGL(k_attn_distortion<64>, grid, dim3(kDistThreads), 0, st, c.n_q_heads, c.n_kv_heads, khat,
                           vhat, k, v, s_max, q, lens, scale, logits, dk, dv);
    else if (c.head_dim == 128)
        hipLaunchKernelGGL(k_attn_distortion<128>, grid, dim3(kDistThreads), 0, st, c.n_q_heads, c.n_kv_heads,
                           khat, vhat, k, v, s_max, q, lens, scale, logits, dk, dv);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace dkv
