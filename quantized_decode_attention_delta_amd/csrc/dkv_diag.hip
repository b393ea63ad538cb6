// Diagnostic: a plain streaming read of device memory, the bandwidth ceiling
// the decode kernels are compared against.  Decode attention is a streaming
// read of the compressed cache (the cost model of "KV 캐시 벡터 양자화와 주의
// 보존 변환", "KV 캐시가 왜 병목인가"); this kernel does nothing but that read.
//
// Each workgroup (one wave) reads a contiguous run of the buffer with 16-byte
// nontemporal loads, 8 in flight per lane, and folds them into one word per
// lane, which it writes to `sink` so that no load can be removed.
#include "dkv_common.h"

namespace dkv {

typedef uint32_t u4v __attribute__((ext_vector_type(4)));

constexpr int kReadWaves = 2048;     // one workgroup per wave slot at 2 waves per SIMD
constexpr int kReadUnroll = 8;

__global__ void __launch_bounds__(64) k_stream_read(const u4v *__restrict__ p, int64_t n16, int64_t per_wg,
                                                    uint32_t *__restrict__ sink)
{
    const int64_t base = (int64_t)blockIdx.x * per_wg;
    const int64_t end = min(base + per_wg, n16);
    uint32_t acc = 0;
    for (int64_t i = base + threadIdx.x; i < end; i += 64 * kReadUnroll) {
        u4v v[kReadUnroll];
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) {
            const int64_t k = i + 64 * u;
            v[u] = k < end ? __builtin_nontemporal_load(p + k) : u4v{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    sink[(int64_t)blockIdx.x * 64 + threadIdx.x] = acc;
}

size_t stream_read_sink_words() { return (size_t)kReadWaves * 64; }

hipError_t launch_stream_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t st)
{
    const int64_t n16 = (int64_t)(bytes / 16);
    const int64_t per_wg = (n16 + kReadWaves - 1) / kReadWaves;
    hipLaunchKernelGGL(k_stream_read, dim3(kReadWaves), dim3(64), 0, st, (const u4v *)buf, n16, per_wg, sink);
    return hipGetLastError();
}

}  // namespace dkv
