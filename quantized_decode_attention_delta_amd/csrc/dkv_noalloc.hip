// dkv_attn_decode_noalloc: dkv_attn_decode for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc).  The split-K partial results, which dkv_attn_decode
// writes to the caller's workspace, go to a fixed array of this library
// instead; the kernels and the split plan are dkv_attn_decode's own.
//
// `scratch` below is a device array; in host code its name is only a stand-in
// for the symbol.  Its device address is looked up once per device with
// hipGetSymbolAddress (each GPU holds its own copy at its own address) and
// only that address is ever handed to a kernel.
#include <hip/hip_runtime.h>

#include <atomic>

#include "dkv.h"
#include "dkv_common.h"

namespace dkv {

size_t decode_partials_bytes(const dkv_config &c);
dkv_status attn_decode_launch(const dkv_config &c, const void *cache, const int32_t *bt, const float *q,
                              const int32_t *lens, float scale, float *out, void *ws, hipStream_t st);

constexpr size_t kScratchBytes = size_t(160) << 20;  // 160 MiB per device
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// Device address of `scratch` per device ordinal, resolved on first use.
constexpr int kMaxDevices = 64;
static std::atomic<void *> g_scratch_ptr[kMaxDevices];

// The address of the current device's copy of `scratch`, or nullptr on error.
static void *scratch_on_current_device()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p) return p;
    void *addr = nullptr;
    if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) return nullptr;
    g_scratch_ptr[dev].store(addr, std::memory_order_release);   // racing threads store the same address
    return addr;
}

}  // namespace dkv

extern "C" dkv_status dkv_attn_decode_noalloc(const dkv_config *c, const void *cache, const int32_t *bt,
                                              const float *q, const int32_t *lens, float scale, float *out,
                                              dkv_stream_t stream)
{
    const dkv_status st = dkv_check_config(c);
    if (st != DKV_OK) return st;
    if (!cache || !q || !lens || !out) return DKV_ERR_ARG;
    if (c->page_tokens > 0 && !bt) return DKV_ERR_ARG;
    if (dkv::decode_partials_bytes(*c) > dkv::kScratchBytes) return DKV_ERR_SCRATCH;
    void *ws = dkv::scratch_on_current_device();
    if (!ws) return DKV_ERR_HIP;
    // every partial record the combine reads is written by the split phase of
    // the same call, and the arrival counters at the array's start are zero
    // from the load of the library (zero-filled static memory) and left at
    // zero by every call, so nothing in the array needs clearing
    return dkv::attn_decode_launch(*c, cache, bt, q, lens, scale, out, ws, (hipStream_t)stream);
}
