// C entry points of libdkv.so: argument validation, size queries, split
// planning and kernel dispatch.  Every check runs on the host before any
// launch; nothing here allocates device memory.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>

#include "dkv.h"
#include "dkv_common.h"

namespace dkv {
hipError_t launch_encode_prefill(const dkv_config &, void *, float *, const int32_t *, const uint16_t *,
                                 const uint16_t *, const int32_t *, int, hipStream_t);
hipError_t launch_append(const dkv_config &, void *, float *, const int32_t *, const uint16_t *,
                         const uint16_t *, const int32_t *, hipStream_t);
hipError_t launch_reconstruct(const dkv_config &, const void *, const int32_t *, const int32_t *, int,
                              float *, float *, hipStream_t);
hipError_t launch_export(const dkv_config &, const void *, const int32_t *, const int32_t *, int,
                         uint16_t *, uint8_t *, uint16_t *, hipStream_t);
hipError_t launch_attn_ref(const dkv_config &, const void *, const int32_t *, const float *,
                           const int32_t *, float, float *, int, int, hipStream_t);
hipError_t launch_combine(const dkv_config &, const float *, int, float *, const int32_t *, int, int,
                          hipStream_t);
hipError_t launch_stream_read(const void *, size_t, uint32_t *, hipStream_t);
hipError_t launch_q80_encode(const dkv_config &, const uint16_t *, const uint16_t *, const int32_t *, int, int8_t *,
                             uint16_t *, hipStream_t);
hipError_t launch_attn_distortion(const dkv_config &, const float *, const float *, const uint16_t *,
                                  const uint16_t *, int, const float *, const int32_t *, float, float *, float *,
                                  float *, hipStream_t);
size_t stream_read_sink_words();
int64_t strided_cache_bytes(const dkv_config &);
void strided_plane_offsets(const dkv_config &, int64_t *);
hipError_t launch_strided_encode(const dkv_config &, void *, const uint16_t *, const uint16_t *, const int32_t *, int,
                                 int, hipStream_t);
hipError_t launch_strided_attn(const dkv_config &, const void *, const float *, const int32_t *, float, float *, int,
                               int, const uint16_t *, const uint16_t *, const int32_t *, int, hipStream_t);
hipError_t launch_strided_append(const dkv_config &, void *, const uint16_t *, const uint16_t *, const int32_t *, int,
                                 hipStream_t);
hipError_t launch_attn_fused(const dkv_config &, const void *, const int32_t *, const float *,
                             const int32_t *, float, float *, int, int, hipStream_t);
bool fused_supported(const dkv_config &);
hipError_t launch_attn_fused_long(const dkv_config &, const void *, const int32_t *, const float *,
                                  const int32_t *, float, float *, int, int, hipStream_t);
bool fused_long_supported(const dkv_config &);
hipError_t launch_attn_g8(const dkv_config &, const void *, const int32_t *, const float *, const int32_t *,
                          float, float *, int, int, hipStream_t, const AppendArgs *, CombineTail);
bool fused_g8_supported(const dkv_config &);
bool fused_long_g8_supported(const dkv_config &);
hipError_t launch_q40_encode(const dkv_config &, void *, const int32_t *, const uint16_t *, const uint16_t *,
                             const int32_t *, int, hipStream_t);
hipError_t launch_q40_export(const dkv_config &, const void *, const int32_t *, const int32_t *, int, uint8_t *,
                             uint16_t *, hipStream_t);
hipError_t launch_attn_q40(const dkv_config &, const void *, const int32_t *, const float *, const int32_t *, float,
                           float *, int, int, hipStream_t);
hipError_t launch_q4k_encode(const dkv_config &, void *, float *, const int32_t *, const uint16_t *,
                             const uint16_t *, const int32_t *, int, hipStream_t);
hipError_t launch_q4k_append(const dkv_config &, void *, float *, const int32_t *, const uint16_t *,
                             const uint16_t *, const int32_t *, hipStream_t);
hipError_t launch_q4k_reconstruct(const dkv_config &, const void *, const int32_t *, const int32_t *, int, float *,
                                  float *, hipStream_t);
hipError_t launch_attn_q4k(const dkv_config &, const void *, const int32_t *, const float *, const int32_t *, float,
                           float *, int, int, hipStream_t);
hipError_t launch_attn_f16(const dkv_config &, const uint16_t *, const uint16_t *, const int32_t *, const float *,
                           const int32_t *, float, float *, int, int, hipStream_t);

// Split plan: runs of whole units (groups, or 32-token tiles) per workgroup,
// sized for about 2048 workgroups over the batch, and at most max_units
// (about 2048 tokens) per run so that ragged batches, where the capacity is far
// above most sequences' lengths, stay balanced: runs past a sequence's end exit
// at once and the combine skips their empty partial records.
struct Plan {
    int nsplit, chunk;
    int split_tokens;   // tokens per run (chunk units)
    int cap_tokens;     // tokens a sequence can hold: lengths are clamped to it
};
static Plan make_plan(int units_cap, int B, int Hkv, int max_units, int min_units)
{
    Plan p;
    const int64_t pairs = (int64_t)B * Hkv;
    int64_t ns = (2048 + pairs - 1) / pairs;
    if (ns < 1) ns = 1;
    // at least min_units (128 tokens) per run while that leaves 256 or more
    // workgroups: on a batch of a few (sequence, kv-head) pairs the
    // 2048-workgroup target would make runs of one group, each paying a whole
    // start-up (8B layer, 8 pairs of 4096 tokens: 32 runs of 4 groups against
    // 128 runs of one, 0.0124 against 0.0139 ms per layer-step in a 32-layer
    // graph).  Below 256 workgroups the runs' start-ups overlap anyway and
    // fewer, longer runs only lengthen the launch (one 256-token sequence:
    // 2 runs of 4 groups took 0.0088 ms per layer-step against 0.0071 for 8).
    const int64_t ns_floor = std::max<int64_t>(units_cap / min_units, (256 + pairs - 1) / pairs);
    if (ns > ns_floor) ns = ns_floor;
    if (ns > units_cap) ns = units_cap;
    if (ns < 1) ns = 1;
    p.chunk = (int)((units_cap + ns - 1) / ns);
    if (p.chunk > max_units) p.chunk = max_units;
    if (p.chunk < 1) p.chunk = 1;
    p.nsplit = (units_cap + p.chunk - 1) / p.chunk;
    if (p.nsplit < 1) p.nsplit = 1;
    p.split_tokens = 0;
    p.cap_tokens = 0;
    return p;
}
// Longest run: 2048 tokens for full (contiguous) caches, 1024 tokens for
// paged serving batches.  Ragged lengths leave a last, partly filled round of
// runs; shorter runs shorten that tail, longer ones start up less often.
// Measured step times (append + decode) of the mixed serving batch: 0.638 ms
// at 1024-token runs, 0.691 at 512, 0.652 at 2048; of a random-walk batch of
// the same shape: 0.656, 0.628 and 0.780 ms.
constexpr int kRunTokens = 2048, kRunTokensPaged = 1024;
// Shortest run: 128 tokens (whole units of unit_tokens).
static int min_units(int unit_tokens) { return unit_tokens >= 128 ? 1 : 128 / unit_tokens; }
static int run_units(const dkv_config &c, int unit_tokens)
{
    const int rt = c.page_tokens > 0 ? kRunTokensPaged : kRunTokens;
    return unit_tokens >= rt ? 1 : rt / unit_tokens;
}
Plan delta_plan(const dkv_config &c)
{
    const Geom g = make_geom(c);
    Plan p = make_plan(g.ng_cap, c.batch, c.n_kv_heads, run_units(c, c.kf), min_units(c.kf));
    p.split_tokens = p.chunk * c.kf;
    p.cap_tokens = g.cap_tokens;
    return p;
}
// Whether the GQA <= 8 decode kernels merge their own partial records (one
// launch per step) for plan p: only for launches of at most 256 workgroups with
// at most 16 splits per row.  The merge is a chain of memory round trips in
// the last workgroup of each row (records written through to memory, arrival
// count, L2 invalidate, loads); measured on MI355X it takes longer than a
// second launch on every larger workload (1 to 18 us per step), while on the
// launch-bound small ones it saves the second launch (about 2 us of 15).
static bool merge_in_kernel(const dkv_config &c, const Plan &p)
{
    return p.nsplit <= 16 && (int64_t)p.nsplit * c.batch * c.n_kv_heads <= 256;
}
// the comparison caches (32-token tiles, contiguous or paged)
Plan tile_plan(const dkv_config &c)
{
    Plan p = make_plan(cmp_ntiles(c), c.batch, c.n_kv_heads, run_units(c, 32), min_units(32));
    p.split_tokens = p.chunk * 32;
    p.cap_tokens = cmp_ntiles(c) * 32;
    return p;
}
// strided-reference decode: runs of at most 64 tiles (2048 tokens), as the
// Delta-KV decode (16-tile runs measured 3 % slower on the 70B layer)
Plan strided_plan(const dkv_config &c)
{
    const int tiles = (c.max_tokens + 31) / 32;
    Plan p = make_plan(tiles, c.batch, c.n_kv_heads, 64, min_units(32));
    p.split_tokens = p.chunk * 32;
    p.cap_tokens = c.max_tokens;
    return p;
}
static size_t ws_for(const dkv_config &c, const Plan &p)
{
    return (size_t)c.batch * c.n_q_heads * p.nsplit * part_stride(c.head_dim) * sizeof(float);
}
// [arrival counters, counter_bytes(c)][partial records of the largest plan]
static size_t workspace_total(const dkv_config &c)
{
    const size_t a = ws_for(c, delta_plan(c));
    const size_t b = (c.page_tokens == 0 || c.page_tokens % 32 == 0) ? ws_for(c, tile_plan(c)) : 0;
    const size_t d = c.page_tokens == 0 ? ws_for(c, strided_plan(c)) : 0;
    return (size_t)counter_bytes(c) + (a > b ? (a > d ? a : d) : (b > d ? b : d));
}
// the partial records start after the arrival counters
static float *partials(const dkv_config &c, void *ws) { return (float *)((uint8_t *)ws + counter_bytes(c)); }
// The split-K combine of plan p: each row merges the records of the splits
// whose run starts before its sequence's end (later runs hold no tokens and
// may leave their record unwritten).
static hipError_t combine(const dkv_config &c, void *ws, const Plan &p, const int32_t *lens, float *out,
                          hipStream_t st)
{
    return launch_combine(c, partials(c, ws), p.nsplit, out, lens, p.cap_tokens, p.split_tokens, st);
}

static dkv_status hip_status(hipError_t e) { return e == hipSuccess ? DKV_OK : DKV_ERR_HIP; }

static float resolve_scale(const dkv_config &c, float s)
{
    const float sc = (s == 0.0f) ? 1.0f / std::sqrt((float)c.head_dim) : s;
    return sc * 1.4426950408889634f;     // logits kept in log2 units
}

// Workspace bytes dkv_attn_decode uses for c: the arrival counters and its
// split plan's partial records.
size_t decode_partials_bytes(const dkv_config &c) { return (size_t)counter_bytes(c) + ws_for(c, delta_plan(c)); }

// The decode of dkv_attn_decode after its argument checks: split phase into
// `ws` (at least decode_partials_bytes(c) bytes), then the combine.
dkv_status attn_decode_launch(const dkv_config &c, const void *cache, const int32_t *bt, const float *q,
                              const int32_t *lens, float scale, float *out, void *ws, hipStream_t st);

}  // namespace dkv

using namespace dkv;

extern "C" {

const char *dkv_status_str(dkv_status s)
{
    switch (s) {
    case DKV_OK: return "ok";
    case DKV_ERR_ARG: return "invalid argument";
    case DKV_ERR_UNSUPPORTED: return "unsupported configuration";
    case DKV_ERR_WORKSPACE: return "workspace missing or too small";
    case DKV_ERR_HIP: return "HIP runtime error";
    case DKV_ERR_SCRATCH: return "needs more than the fixed scratch of the no-allocation entry point";
    }
    return "unknown status";
}

dkv_status dkv_check_config(const dkv_config *c)
{
    if (!c) return DKV_ERR_ARG;
    if (c->batch < 1 || c->n_kv_heads < 1 || c->n_q_heads < 1) return DKV_ERR_ARG;
    if (c->n_q_heads % c->n_kv_heads != 0) return DKV_ERR_ARG;
    if (c->head_dim <= 0 || c->head_dim % 32 != 0) return DKV_ERR_ARG;
    if (c->kf < 1) return DKV_ERR_ARG;
    if (c->page_tokens < 0) return DKV_ERR_ARG;
    if (c->page_tokens == 0) {
        if (c->max_tokens < 1) return DKV_ERR_ARG;
    } else {
        if (c->page_tokens % c->kf != 0) return DKV_ERR_ARG;
        if (c->n_pages < 1 || c->max_pages_per_seq < 1) return DKV_ERR_ARG;
        if ((int64_t)c->max_pages_per_seq * c->page_tokens > INT_MAX / 2) return DKV_ERR_ARG;
    }
    if (c->head_dim != 64 && c->head_dim != 128) return DKV_ERR_UNSUPPORTED;
    if (c->kf > kMaxKf) return DKV_ERR_UNSUPPORTED;
    if (c->n_q_heads / c->n_kv_heads > 16) return DKV_ERR_UNSUPPORTED;
    return DKV_OK;
}

size_t dkv_group_record_bytes(const dkv_config *c)
{
    if (dkv_check_config(c) != DKV_OK) return 0;
    return (size_t)make_geom(*c).rec;
}

size_t dkv_cache_bytes(const dkv_config *c)
{
    if (dkv_check_config(c) != DKV_OK) return 0;
    const Geom g = make_geom(*c);
    if (g.paged) return (size_t)c->n_pages * (size_t)g.page_bytes;
    return (size_t)c->batch * (size_t)g.page_bytes;
}

size_t dkv_state_bytes(const dkv_config *c)
{
    if (dkv_check_config(c) != DKV_OK) return 0;
    return (size_t)c->batch * c->n_kv_heads * 2 * c->head_dim * sizeof(float);
}

size_t dkv_workspace_bytes(const dkv_config *c)
{
    if (dkv_check_config(c) != DKV_OK) return 0;
    return workspace_total(*c);
}

dkv_status dkv_attn_decode_plan(const dkv_config *c, int32_t *nsplit, int32_t *split_tokens)
{
    const dkv_status st = dkv_check_config(c);
    if (st != DKV_OK) return st;
    if (!nsplit || !split_tokens) return DKV_ERR_ARG;
    const Plan p = delta_plan(*c);
    *nsplit = p.nsplit;
    *split_tokens = p.split_tokens;
    return DKV_OK;
}

int32_t dkv_attn_decode_launches(const dkv_config *c)
{
    if (dkv_check_config(c) != DKV_OK) return 0;
    const bool g8 = fused_g8_supported(*c) || fused_long_g8_supported(*c);
    return g8 && merge_in_kernel(*c, delta_plan(*c)) ? 1 : 2;
}

dkv_status dkv_encode_prefill(const dkv_config *c, void *cache, float *state, const int32_t *bt,
                              const uint16_t *k, const uint16_t *v, const int32_t *lens, int32_t s_max,
                              dkv_stream_t stream)
{
    dkv_status st = dkv_check_config(c);
    if (st != DKV_OK) return st;
    if (!cache || !state || !k || !v || !lens || s_max < 0) return DKV_ERR_ARG;
    if (c->page_tokens > 0 && !bt) return DKV_ERR_ARG;
    if (s_max == 0) return DKV_OK;
    return hip_status(launch_encode_prefill(*c, cache, state, c->page_tokens > 0 ? bt : nullptr, k, v, lens,
                                            s_max, (hipStream_t)stream));
}

dkv_status dkv_append(const dkv_config *c, void *cache, float *state, const int32_t *bt,
                      const uint16_t *k, const uint16_t *v, const int32_t *pos, dkv_stream_t stream)
{
    dkv_status st = dkv_check_config(c);
    if (st != DKV_OK) return st;
    if (!cache || !state || !k || !v || !pos) return DKV_ERR_ARG;
    if (c->page_tokens > 0 && !bt) return DKV_ERR_ARG;
    return hip_status(launch_append(*c, cache, state, c->page_tokens > 0 ? bt : nullptr, k, v, pos,
                                    (hipStream_t)stream));
}

static dkv_status attn_common(const dkv_config *c, const void *cache, const int32_t *bt, const float *q,
                              const int32_t *lens, float *out, void *ws, size_t ws_bytes)
{
    dkv_status st = dkv_check_config(c);
    if (st != DKV_OK) return st;
    if (!cache || !q || !lens || !out) return DKV_ERR_ARG;
    if (c->page_tokens > 0 && !bt) return DKV_ERR_ARG;
    if (!ws || ws_bytes < workspace_total(*c)) return DKV_ERR_WORKSPACE;
    return DKV_OK;
}

// With `ap` (non-null positions), each sequence's new token is appended first:
// inside the split kernel where the kf = 32, GQA <= 8 kernel runs, else by the
// append kernel ahead of it.
// With `out`, the split kernel merges its own partials into out where that is
// faster (the GQA <= 8 kernels on small launches, merge_in_kernel): one
// launch; *merged tells whether it did, else the caller launches the combine.
static hipError_t launch_split_phase(const dkv_config &c, const void *cache, const int32_t *bt, const float *q,
                                     const int32_t *lens, float scale, void *ws, const Plan &p, hipStream_t st,
                                     const AppendArgs *ap = nullptr, float *out = nullptr, bool *merged = nullptr)
{
    const int32_t *btp = c.page_tokens > 0 ? bt : nullptr;
    float *part = partials(c, ws);
    if (merged) *merged = false;
    if (ap && !fused_g8_supported(c)) {
        const hipError_t e = launch_append(c, ap->cache, ap->state, btp, ap->knew, ap->vnew, ap->positions, st);
        if (e != hipSuccess) return e;
        ap = nullptr;
    }
    if (fused_g8_supported(c) || fused_long_g8_supported(c)) {
        const bool mk = out != nullptr && merge_in_kernel(c, p);
        const CombineTail ct{mk ? out : nullptr, mk ? (uint32_t *)ws : nullptr};
        if (merged) *merged = mk;
        return launch_attn_g8(c, cache, btp, q, lens, resolve_scale(c, scale), part, p.nsplit, p.chunk, st, ap, ct);
    }
    if (fused_supported(c))
        return launch_attn_fused(c, cache, btp, q, lens, resolve_scale(c, scale), part, p.nsplit, p.chunk, st);
    if (fused_long_supported(c))
        return launch_attn_fused_long(c, cache, btp, q, lens, resolve_scale(c, scale), part, p.nsplit, p.chunk,
                                      st);
    return launch_attn_ref(c, cache, btp, q, lens, resolve_scale(c, scale), part, p.nsplit, p.chunk, st);
}

dkv_status dkv_attn_decode(const dkv_config *c, const void *cache, const int32_t *bt, const float *q,
                           const int32_t *lens, float scale, float *out, void *ws, size_t ws_bytes,
                           dkv_stream_t stream)
{
    dkv_status st = attn_common(c, cache, bt, q, lens, out, ws, ws_bytes);
    if (st != DKV_OK) return st;
    return dkv::attn_decode_launch(*c, cache, bt, q, lens, scale, out, ws, (hipStream_t)stream);
}

dkv_status dkv_append_attn_decode(const dkv_config *c, void *cache, float *state, const int32_t *bt,
                                  const uint16_t *k, const uint16_t *v, const int32_t *pos, const float *q,
                                  const int32_t *lens, float scale, float *out, void *ws, size_t ws_bytes,
                                  dkv_stream_t stream)
{
    dkv_status st = attn_common(c, cache, bt, q, lens, out, ws, ws_bytes);
    if (st != DKV_OK) return st;
    if (!state || !k || !v || !pos) return DKV_ERR_ARG;
    const Plan p = delta_plan(*c);
    const AppendArgs ap{(uint8_t *)cache, state, k, v, pos};
    bool merged = false;
    hipError_t e = launch_split_phase(*c, cache, bt, q, lens, scale, ws, p, (hipStream_t)stream, &ap, out, &merged);
    if (e != hipSuccess) return DKV_ERR_HIP;
    if (merged) return DKV_OK;
    return hip_status(combine(*c, ws, p, lens, out, (hipStream_t)stream));
}

dkv_status dkv_attn_decode_partial(const dkv_config *c, const void *cache, const int32_t *bt, const float *q,
                                   const int32_t *lens, float scale, void *ws, size_t ws_bytes,
                                   dkv_stream_t stream)
{
    dkv_status st = attn_common(c, cache, bt, q, lens, (float *)ws, ws, ws_bytes);
    if (st != DKV_OK) return st;
    return hip_status(launch_split_phase(*c, cache, bt, q, lens, scale, ws, delta_plan(*c), (hipStream_t)stream));
}

dkv_status dkv_attn_decode_ref(const dkv_config *c, const void *cache, const int32_t *bt, const float *q,
                               const int32_t *lens, float scale, float *out, void *ws, size_t ws_bytes,
                               dkv_stream_t stream)
{
    dkv_status st = attn_common(c, cache, bt, q, lens, out, ws, ws_bytes);
    if (st != DKV_OK) return st;
    const Plan p = delta_plan(*c);
    hipError_t e = launch_attn_ref(*c, cache, c->page_tokens > 0 ? bt : nullptr, q, lens,
                                   resolve_scale(*c, scale), partials(*c, ws), p.nsplit, p.chunk,
                                   (hipStream_t)stream);
    if (e != hipSuccess) return DKV_ERR_HIP;
    return hip_status(combine(*c, ws, p, lens, out, (hipStream_t)stream));
}

dkv_status dkv_reconstruct(const dkv_config *c, const void *cache, const int32_t *bt, const int32_t *lens,
                           int32_t s_max, float *ko, float *vo, dkv_stream_t stream)
{
    dkv_status st = dkv_check_config(c);
    if (st != DKV_OK) return st;
    if (!cache || !lens || !ko || !vo || s_max < 0) return DKV_ERR_ARG;
    if (c->page_tokens > 0 && !bt) return DKV_ERR_ARG;
    if (s_max == 0) return DKV_OK;
    return hip_status(launch_reconstruct(*c, cache, c->page_tokens > 0 ? bt : nullptr, lens, s_max, ko, vo,
                                         (hipStream_t)stream));
}

dkv_status dkv_q8_0_encode(const dkv_config *c, const uint16_t *k, const uint16_t *v, const int32_t *lens,
                           int32_t s_max, int8_t *codes, uint16_t *scales, dkv_stream_t stream)
{
    dkv_status st = dkv_check_config(c);
    if (st != DKV_OK) return st;
    if (!k || !v || !lens || !codes || !scales || s_max < 0) return DKV_ERR_ARG;
    if (s_max == 0) return DKV_OK;
    return hip_status(launch_q80_encode(*c, k, v, lens, s_max, codes, scales, (hipStream_t)stream));
}

dkv_status dkv_attn_distortion(const dkv_config *c, const float *khat, const float *vhat, const uint16_t *k,
                               const uint16_t *v, int32_t s_max, const float *q, const int32_t *lens,
                               float softmax_scale, float *logits, float *dk, float *dv, dkv_stream_t stream)
{
    if (!c || !khat || !vhat || !k || !v || !q || !lens || !logits || !dk || !dv || s_max < 1) return DKV_ERR_ARG;
    if (c->batch < 1 || c->n_kv_heads < 1 || c->n_q_heads < 1 || c->n_q_heads % c->n_kv_heads != 0)
        return DKV_ERR_ARG;
    if (c->head_dim != 64 && c->head_dim != 128) return DKV_ERR_UNSUPPORTED;
    const float sc = softmax_scale == 0.0f ? 1.0f / std::sqrt((float)c->head_dim) : softmax_scale;
    return hip_status(launch_attn_distortion(*c, khat, vhat, k, v, s_max, q, lens, sc, logits, dk, dv,
                                             (hipStream_t)stream));
}

dkv_status dkv_export(const dkv_config *c, const void *cache, const int32_t *bt, const int32_t *lens,
                      int32_t s_max, uint16_t *kf_rows, uint8_t *codes, uint16_t *scales,
                      dkv_stream_t stream)
{
    dkv_status st = dkv_check_config(c);
    if (st != DKV_OK) return st;
    if (!cache || !lens || !kf_rows || s_max < 0) return DKV_ERR_ARG;
    const int64_t nd = (int64_t)s_max - (s_max + c->kf - 1) / c->kf;   // delta rows (0 when kf == 1)
    if (nd > 0 && (!codes || !scales)) return DKV_ERR_ARG;
    if (c->page_tokens > 0 && !bt) return DKV_ERR_ARG;
    if (s_max == 0) return DKV_OK;
    return hip_status(launch_export(*c, cache, c->page_tokens > 0 ? bt : nullptr, lens, s_max, kf_rows,
                                    codes, scales, (hipStream_t)stream));
}

// The comparison caches are cut in 32-token tiles, so paged mode needs
// page_tokens % 32 == 0 (a tile never straddles two pages).
static dkv_status cmp_check(const dkv_config *c, const int32_t *bt)
{
    dkv_status st = dkv_check_config(c);
    if (st != DKV_OK) return st;
    if (c->page_tokens > 0 && c->page_tokens % 32 != 0) return DKV_ERR_UNSUPPORTED;
    if (c->page_tokens > 0 && !bt) return DKV_ERR_ARG;
    return DKV_OK;
}

size_t dkv_q4_0_cache_bytes(const dkv_config *c)
{
    if (dkv_check_config(c) != DKV_OK || (c->page_tokens > 0 && c->page_tokens % 32 != 0)) return 0;
    const int64_t tiles = c->page_tokens > 0 ? (int64_t)c->n_pages * (c->page_tokens / 32)
                                             : (int64_t)c->batch * cmp_ntiles(*c);
    return (size_t)tiles * c->n_kv_heads * (size_t)q40_tile_bytes(c->head_dim);
}

dkv_status dkv_q4_0_encode(const dkv_config *c, void *q4, const int32_t *bt, const uint16_t *k, const uint16_t *v,
                           const int32_t *lens, int32_t s_max, dkv_stream_t stream)
{
    dkv_status st = cmp_check(c, bt);
    if (st != DKV_OK) return st;
    if (!q4 || !k || !v || !lens || s_max < 0) return DKV_ERR_ARG;
    if (s_max == 0) return DKV_OK;
    return hip_status(launch_q40_encode(*c, q4, c->page_tokens > 0 ? bt : nullptr, k, v, lens, s_max,
                                        (hipStream_t)stream));
}

dkv_status dkv_q4_0_export(const dkv_config *c, const void *q4, const int32_t *bt, const int32_t *lens,
                           int32_t s_max, uint8_t *codes, uint16_t *scales, dkv_stream_t stream)
{
    dkv_status st = cmp_check(c, bt);
    if (st != DKV_OK) return st;
    if (!q4 || !lens || !codes || !scales || s_max < 0) return DKV_ERR_ARG;
    if (s_max == 0) return DKV_OK;
    return hip_status(launch_q40_export(*c, q4, c->page_tokens > 0 ? bt : nullptr, lens, s_max, codes, scales,
                                        (hipStream_t)stream));
}

dkv_status dkv_attn_decode_q4_0(const dkv_config *c, const void *q4, const int32_t *bt, const float *q,
                                const int32_t *lens, float scale, float *out, void *ws, size_t ws_bytes,
                                dkv_stream_t stream)
{
    dkv_status st = cmp_check(c, bt);
    if (st != DKV_OK) return st;
    if (!q4 || !q || !lens || !out) return DKV_ERR_ARG;
    const Plan p = tile_plan(*c);
    if (!ws || ws_bytes < workspace_total(*c)) return DKV_ERR_WORKSPACE;
    hipError_t e = launch_attn_q40(*c, q4, c->page_tokens > 0 ? bt : nullptr, q, lens, resolve_scale(*c, scale),
                                   partials(*c, ws), p.nsplit, p.chunk, (hipStream_t)stream);
    if (e != hipSuccess) return DKV_ERR_HIP;
    return hip_status(combine(*c, ws, p, lens, out, (hipStream_t)stream));
}

// ------------------------------------------------------- Q4-keyframe variant
// The plain Q4_0 tile layout and size; groups must lie in whole tiles.
static dkv_status q4k_check(const dkv_config *c, const int32_t *bt)
{
    dkv_status st = cmp_check(c, bt);
    if (st != DKV_OK) return st;
    if (32 % c->kf != 0 && c->kf % 32 != 0) return DKV_ERR_UNSUPPORTED;
    return DKV_OK;
}

dkv_status dkv_q4k_encode_prefill(const dkv_config *c, void *cache, float *state, const int32_t *bt,
                                  const uint16_t *k, const uint16_t *v, const int32_t *lens, int32_t s_max,
                                  dkv_stream_t stream)
{
    dkv_status st = q4k_check(c, bt);
    if (st != DKV_OK) return st;
    if (!cache || !state || !k || !v || !lens || s_max < 0) return DKV_ERR_ARG;
    if (s_max == 0) return DKV_OK;
    return hip_status(launch_q4k_encode(*c, cache, state, c->page_tokens > 0 ? bt : nullptr, k, v, lens, s_max,
                                        (hipStream_t)stream));
}

dkv_status dkv_q4k_append(const dkv_config *c, void *cache, float *state, const int32_t *bt, const uint16_t *k_new,
                          const uint16_t *v_new, const int32_t *positions, dkv_stream_t stream)
{
    dkv_status st = q4k_check(c, bt);
    if (st != DKV_OK) return st;
    if (!cache || !state || !k_new || !v_new || !positions) return DKV_ERR_ARG;
    return hip_status(launch_q4k_append(*c, cache, state, c->page_tokens > 0 ? bt : nullptr, k_new, v_new, positions,
                                        (hipStream_t)stream));
}

dkv_status dkv_q4k_reconstruct(const dkv_config *c, const void *cache, const int32_t *bt, const int32_t *lens,
                               int32_t s_max, float *k_out, float *v_out, dkv_stream_t stream)
{
    dkv_status st = q4k_check(c, bt);
    if (st != DKV_OK) return st;
    if (!cache || !lens || !k_out || !v_out || s_max < 0) return DKV_ERR_ARG;
    if (s_max == 0) return DKV_OK;
    return hip_status(launch_q4k_reconstruct(*c, cache, c->page_tokens > 0 ? bt : nullptr, lens, s_max, k_out, v_out,
                                             (hipStream_t)stream));
}

dkv_status dkv_attn_decode_q4k(const dkv_config *c, const void *cache, const int32_t *bt, const float *q,
                               const int32_t *lens, float scale, float *out, void *ws, size_t ws_bytes,
                               dkv_stream_t stream)
{
    dkv_status st = q4k_check(c, bt);
    if (st != DKV_OK) return st;
    if (c->kf != 1 && c->kf != 32) return DKV_ERR_UNSUPPORTED;
    if (!q40_vbp(*c)) return DKV_ERR_UNSUPPORTED;           // at most 8 query heads per kv-head
    if (!cache || !q || !lens || !out) return DKV_ERR_ARG;
    const Plan p = tile_plan(*c);
    if (!ws || ws_bytes < workspace_total(*c)) return DKV_ERR_WORKSPACE;
    hipError_t e = launch_attn_q4k(*c, cache, c->page_tokens > 0 ? bt : nullptr, q, lens, resolve_scale(*c, scale),
                                   partials(*c, ws), p.nsplit, p.chunk, (hipStream_t)stream);
    if (e != hipSuccess) return DKV_ERR_HIP;
    return hip_status(combine(*c, ws, p, lens, out, (hipStream_t)stream));
}

dkv_status dkv_attn_decode_f16(const dkv_config *c, const uint16_t *k, const uint16_t *v, const int32_t *bt,
                               const float *q, const int32_t *lens, float scale, float *out, void *ws,
                               size_t ws_bytes, dkv_stream_t stream)
{
    dkv_status st = cmp_check(c, bt);
    if (st != DKV_OK) return st;
    if (!k || !v || !q || !lens || !out) return DKV_ERR_ARG;
    const Plan p = tile_plan(*c);
    if (!ws || ws_bytes < workspace_total(*c)) return DKV_ERR_WORKSPACE;
    hipError_t e = launch_attn_f16(*c, k, v, c->page_tokens > 0 ? bt : nullptr, q, lens, resolve_scale(*c, scale),
                                   partials(*c, ws), p.nsplit, p.chunk, (hipStream_t)stream);
    if (e != hipSuccess) return DKV_ERR_HIP;
    return hip_status(combine(*c, ws, p, lens, out, (hipStream_t)stream));
}

// ---------------------------------------------------------- strided references
// Contiguous mode only; the reference index of a token is 16 bits.
static dkv_status strided_check(const dkv_config *c)
{
    dkv_status st = dkv_check_config(c);
    if (st != DKV_OK) return st;
    if (c->page_tokens != 0) return DKV_ERR_UNSUPPORTED;
    if ((c->max_tokens + (int64_t)c->kf - 1) / c->kf > 65536) return DKV_ERR_UNSUPPORTED;
    if (c->n_kv_heads > 32767 || c->batch > 65535) return DKV_ERR_UNSUPPORTED;
    return DKV_OK;
}

size_t dkv_strided_cache_bytes(const dkv_config *c)
{
    if (strided_check(c) != DKV_OK) return 0;
    return (size_t)strided_cache_bytes(*c);
}

dkv_status dkv_strided_layout(const dkv_config *c, int64_t *layout)
{
    dkv_status st = strided_check(c);
    if (st != DKV_OK) return st;
    if (!layout) return DKV_ERR_ARG;
    strided_plane_offsets(*c, layout);
    return DKV_OK;
}

dkv_status dkv_strided_encode_prefill(const dkv_config *c, void *cache, const uint16_t *k, const uint16_t *v,
                                      const int32_t *lens, int32_t s_max, int32_t window, dkv_stream_t stream)
{
    dkv_status st = strided_check(c);
    if (st != DKV_OK) return st;
    if (!cache || !k || !v || !lens || s_max < 0 || window < 0) return DKV_ERR_ARG;
    if (s_max == 0) return DKV_OK;
    return hip_status(launch_strided_encode(*c, cache, k, v, lens, s_max, window, (hipStream_t)stream));
}

dkv_status dkv_strided_append(const dkv_config *c, void *cache, const uint16_t *k_new, const uint16_t *v_new,
                              const int32_t *positions, int32_t window, dkv_stream_t stream)
{
    dkv_status st = strided_check(c);
    if (st != DKV_OK) return st;
    if (!cache || !k_new || !v_new || !positions || window < 0) return DKV_ERR_ARG;
    return hip_status(launch_strided_append(*c, cache, k_new, v_new, positions, window, (hipStream_t)stream));
}

dkv_status dkv_strided_attn_decode(const dkv_config *c, const void *cache, const float *q, const int32_t *lens,
                                   float scale, float *out, void *ws, size_t ws_bytes, dkv_stream_t stream)
{
    dkv_status st = strided_check(c);
    if (st != DKV_OK) return st;
    if (!cache || !q || !lens || !out) return DKV_ERR_ARG;
    if (!ws || ws_bytes < workspace_total(*c)) return DKV_ERR_WORKSPACE;
    const Plan p = strided_plan(*c);
    hipError_t e = launch_strided_attn(*c, cache, q, lens, resolve_scale(*c, scale), partials(*c, ws), p.nsplit, p.chunk,
                                       nullptr, nullptr, nullptr, 0, (hipStream_t)stream);
    if (e != hipSuccess) return DKV_ERR_HIP;
    return hip_status(combine(*c, ws, p, lens, out, (hipStream_t)stream));
}

dkv_status dkv_strided_append_attn_decode(const dkv_config *c, void *cache, const uint16_t *k_new,
                                          const uint16_t *v_new, const int32_t *positions, int32_t window,
                                          const float *q, const int32_t *lens, float scale, float *out, void *ws,
                                          size_t ws_bytes, dkv_stream_t stream)
{
    dkv_status st = strided_check(c);
    if (st != DKV_OK) return st;
    if (!cache || !k_new || !v_new || !positions || window < 0 || !q || !lens || !out) return DKV_ERR_ARG;
    if (!ws || ws_bytes < workspace_total(*c)) return DKV_ERR_WORKSPACE;
    const Plan p = strided_plan(*c);
    hipError_t e = launch_strided_attn(*c, cache, q, lens, resolve_scale(*c, scale), partials(*c, ws), p.nsplit, p.chunk,
                                       k_new, v_new, positions, window, (hipStream_t)stream);
    if (e != hipSuccess) return DKV_ERR_HIP;
    return hip_status(combine(*c, ws, p, lens, out, (hipStream_t)stream));
}

}  // extern "C"

size_t dkv_stream_read_sink_words(void) { return dkv::stream_read_sink_words(); }

dkv_status dkv_stream_read(const void *buf, size_t bytes, uint32_t *sink, size_t sink_words, dkv_stream_t stream)
{
    if (!buf || !sink || bytes < 16) return DKV_ERR_ARG;
    if (sink_words < dkv::stream_read_sink_words()) return DKV_ERR_WORKSPACE;
    return dkv::hip_status(dkv::launch_stream_read(buf, bytes, sink, (hipStream_t)stream));
}

dkv_status dkv::attn_decode_launch(const dkv_config &c, const void *cache, const int32_t *bt, const float *q,
                                   const int32_t *lens, float scale, float *out, void *ws, hipStream_t st)
{
    const Plan p = delta_plan(c);
    bool merged = false;
    hipError_t e = launch_split_phase(c, cache, bt, q, lens, scale, ws, p, st, nullptr, out, &merged);
    if (e != hipSuccess) return DKV_ERR_HIP;
    if (merged) return DKV_OK;
    return hip_status(combine(c, ws, p, lens, out, st));
}
