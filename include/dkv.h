/*
 * dkv.h -- Delta-KV compressed KV cache and fused decode attention on MI355X
 * (gfx950).  C ABI of libdkv.so.
 *
 * Method (web page "영상 압축 기법을 KV 캐시에 적용해 Q4 양자화 오차를 10,000배
 * 줄인 Delta-KV", jeff.news, sections "핵심 아이디어" and "벤치마크"): each K
 * and each V stream of one (sequence, kv-head) is stored as an fp16 keyframe
 * every kf tokens; every other token stores the closed-loop difference to the
 * previous reconstructed token, quantised Q4_0-style (32-element blocks, an
 * fp16 scale and 4-bit codes: 18 bytes per 32 elements).  Decode attention
 * (page "KV 캐시 벡터 양자화와 주의 보존 변환", llm-wiki.hwlabs.dev, sections
 * "KV 캐시가 왜 병목인가" and "왜 복원 오차가 틀린 기준인가") reads the
 * compressed cache directly: softmax(q.K^T * scale) . V with grouped-query
 * heads (query head hq uses kv-head hq / (Hq/Hkv)).
 *
 * Conventions for every entry point:
 *  - Pointers marked (device) are device memory on the current HIP device;
 *    (host) pointers are host memory read during the call.  The caller owns
 *    every buffer; the library allocates no memory and keeps no state.
 *  - Every launch is asynchronous on `stream` (0 = the null stream).
 *  - Arguments are validated on the host before anything is launched; a
 *    failed check returns a status and launches nothing.  A HIP launch error
 *    returns DKV_ERR_HIP.  No C++ exception crosses this interface.
 *  - Preconditions the library cannot check (caller's responsibility, as for
 *    any KV cache): K/V inputs are finite; positions and sequence lengths stay
 *    within the cache capacity; appends arrive in token order; device arrays
 *    have the documented sizes.
 *
 * Cache layout (one buffer holds one attention layer):
 *  A "group" is the kf tokens that start at a keyframe.  Each (sequence,
 *  kv-head, group) owns one group record of dkv_group_record_bytes() bytes
 *  holding, in order, for K then for V:
 *    keyframe  D fp16 values (channel order permuted for the matrix cores);
 *    scales    kf x D/32 fp16 -- slot 0 holds the largest |scale| of each
 *              block over the group's delta tokens, slots 1..kf-1 the scale
 *              of each delta token's blocks;
 *    codes     K: (kf-1) rows of D/2 bytes, one per delta token, each Q4_0
 *              block's 16 canonical bytes split into four 4-byte pieces;
 *              V: ceil(kf/32) tiles of 32 token slots, each channel's nibbles
 *              of 8 tokens packed in one 32-bit word (slot 0 of a group is the
 *              keyframe and carries no code);
 *  then padding to a multiple of 128 bytes (whole cache lines per record).
 *  Contiguous mode (page_tokens == 0): records are ordered
 *  [batch][n_kv_heads][ceil(max_tokens/kf)].  Paged mode (page_tokens > 0,
 *  page_tokens % kf == 0): a page holds page_tokens tokens of every kv-head,
 *  ordered [n_kv_heads][page_tokens/kf]; block_table (device, int32
 *  [batch][max_pages_per_seq]) maps a sequence's logical page to a physical
 *  page in [0, n_pages).
 *
 * Reconstruction (the decoder): xhat = float(keyframe); then per delta token,
 * per channel, xhat = fp32(xhat + (code-8)*float(scale)), folded in token
 * order -- bit-identical to the encoder's closed loop.
 */
#ifndef DKV_H
#define DKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *dkv_stream_t; /* a hipStream_t */

typedef enum {
    DKV_OK = 0,
    DKV_ERR_ARG = 1,         /* null pointer, non-positive size, inconsistent shape */
    DKV_ERR_UNSUPPORTED = 2, /* valid but not built: head_dim not 64/128, kf > 1024 ... */
    DKV_ERR_WORKSPACE = 3,   /* workspace missing or smaller than dkv_workspace_bytes() */
    DKV_ERR_HIP = 4,         /* a HIP runtime call or kernel launch failed */
    DKV_ERR_SCRATCH = 5      /* needs more than the fixed scratch of dkv_attn_decode_noalloc */
} dkv_status;

typedef struct {
    int32_t batch;             /* B, sequences per call, >= 1 */
    int32_t n_q_heads;         /* Hq, multiple of n_kv_heads */
    int32_t n_kv_heads;        /* Hkv >= 1 */
    int32_t head_dim;          /* D: 64 or 128 */
    int32_t kf;                /* keyframe interval, 1..1024 */
    int32_t max_tokens;        /* capacity per sequence (tokens), >= 1 */
    int32_t page_tokens;       /* 0 = contiguous; else tokens per page, multiple of kf */
    int32_t n_pages;           /* paged mode: physical pages in the buffer */
    int32_t max_pages_per_seq; /* paged mode: row length of block_table */
} dkv_config;

/* Human-readable name of a status code (static string). */
const char *dkv_status_str(dkv_status s);

/* Checks a configuration without touching the GPU. */
dkv_status dkv_check_config(const dkv_config *cfg);

/* Bytes of one group record (K and V of one kv-head, kf tokens). 0 if cfg is invalid. */
size_t dkv_group_record_bytes(const dkv_config *cfg);

/* Bytes of one layer's compressed cache for cfg (header-free). 0 if cfg is invalid. */
size_t dkv_cache_bytes(const dkv_config *cfg);

/* Bytes of the reconstruction state: fp32 [batch][n_kv_heads][2][head_dim]
 * (the last reconstructed K and V row of each sequence). */
size_t dkv_state_bytes(const dkv_config *cfg);

/* Bytes of the workspace the decode calls need for cfg.  Layout: one 32-bit
 * arrival counter per (sequence, kv-head), padded to a multiple of 256 bytes,
 * then the split-K partial records.  The counters must be zero before the
 * first call that uses the workspace (allocate it zero-filled); every decode
 * call leaves them at zero again.  The partial records need no initial
 * contents. */
size_t dkv_workspace_bytes(const dkv_config *cfg);

/* Kernel launches dkv_attn_decode issues for cfg: 1 where its split kernel
 * merges its own partial results, else 2 (split phase, combine); 0 if cfg is
 * invalid.  dkv_append_attn_decode issues the same number, plus one for the
 * append where it is not done inside the split launch (kf other than 32). */
int32_t dkv_attn_decode_launches(const dkv_config *cfg);

/*
 * Bulk prefill encode.  Encodes tokens [0, seq_lens[b]) of every sequence.
 *  k, v      (device) fp16 [batch][n_kv_heads][s_max][head_dim]
 *  seq_lens  (device) int32 [batch], each in [0, min(s_max, capacity)]
 *  cache     (device) dkv_cache_bytes(cfg) bytes, written
 *  state     (device) fp32 state, written for every sequence with seq_lens > 0
 *  block_table (device) int32 [batch][max_pages_per_seq] in paged mode, else NULL
 * Parallel over (sequence, kv-head, K/V, group); each group is encoded
 * token by token (closed loop).
 */
dkv_status dkv_encode_prefill(const dkv_config *cfg, void *cache, float *state,
                              const int32_t *block_table, const uint16_t *k,
                              const uint16_t *v, const int32_t *seq_lens, int32_t s_max,
                              dkv_stream_t stream);

/*
 * Append one token per sequence (one decode step).
 *  k_new, v_new (device) fp16 [batch][n_kv_heads][head_dim]
 *  positions    (device) int32 [batch]: index of the new token (= tokens
 *               already cached); a negative position skips the sequence.
 *               The caller advances it afterwards.
 * A token at a multiple of kf becomes a keyframe; any other token is
 * quantised against `state`, which is updated.
 */
dkv_status dkv_append(const dkv_config *cfg, void *cache, float *state,
                      const int32_t *block_table, const uint16_t *k_new,
                      const uint16_t *v_new, const int32_t *positions, dkv_stream_t stream);

/*
 * Fused decode attention over the compressed cache.
 *  q        (device) fp32 [batch][n_q_heads][head_dim]
 *  seq_lens (device) int32 [batch]: tokens attended (0 gives a zero row)
 *  softmax_scale: logit scale; 0 means 1/sqrt(head_dim)
 *  out      (device) fp32 [batch][n_q_heads][head_dim]
 *  workspace (device) at least dkv_workspace_bytes(cfg) bytes (see there:
 *           its arrival counters start at zero; calls that share a
 *           workspace must not run concurrently)
 * Launches: the split phase, then the split-K combine.  Where kf is a
 * multiple of 32 up to 512, at most 8 query heads share a kv-head and the
 * split launch is small (at most 256 workgroups, at most 16 splits per
 * (sequence, kv-head); on MI355X a second launch costs more than the merge
 * there), ONE kernel: the last workgroup of each (sequence, kv-head) to finish
 * merges that row's split-K partial results into out.
 */
dkv_status dkv_attn_decode(const dkv_config *cfg, const void *cache,
                           const int32_t *block_table, const float *q,
                           const int32_t *seq_lens, float softmax_scale, float *out,
                           void *workspace, size_t workspace_bytes, dkv_stream_t stream);

/*
 * dkv_attn_decode without a workspace, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, kernels, launches and results as
 * dkv_attn_decode, except that the split-K partial results go to a scratch
 * array of 160 MiB that the library holds in each GPU's memory (static device
 * memory, resolved once per device on the first call there, held until the
 * process ends).  It allocates nothing, on the device or the host.
 *  - Needs the arrival counters (4 * batch * n_kv_heads bytes, rounded up to
 *    256) plus batch * n_q_heads * nsplit * (head_dim + 4) * 4 bytes of
 *    scratch, nsplit being dkv_attn_decode's split count
 *    (dkv_workspace_bytes(cfg) is an upper bound); a configuration needing
 *    more than 160 MiB returns DKV_ERR_SCRATCH before anything is launched.
 *  - Every call on one GPU shares that GPU's scratch array: calls that may
 *    overlap on one GPU (several streams, several host threads) race and must
 *    be serialised by the caller.  Nothing in it needs clearing: each call
 *    writes every partial record it reads, and the arrival counters at its
 *    start (see dkv_workspace_bytes) are zero when the library is loaded
 *    (static device memory is zero-filled) and zero again after every call.
 *  - Errors: as dkv_attn_decode, DKV_ERR_SCRATCH, and DKV_ERR_HIP if the
 *    scratch array's device address cannot be obtained.
 */
dkv_status dkv_attn_decode_noalloc(const dkv_config *cfg, const void *cache,
                                   const int32_t *block_table, const float *q,
                                   const int32_t *seq_lens, float softmax_scale, float *out,
                                   dkv_stream_t stream);

/*
 * One serving step in one call: dkv_append of each sequence's new token, then
 * dkv_attn_decode over the grown cache (the decode step that follows an
 * append, Delta-KV article "구현"), with the same arguments as those two
 * calls.  seq_lens must already count the new token.  Where the kf = 32,
 * GQA <= 8 decode kernel runs (every benchmark workload), the append is done
 * inside its split launch by the workgroup whose run holds the new token's
 * group, before it reads that group: the launches of dkv_attn_decode and no
 * more (ONE launch per serving step where that kernel also merges its
 * partials).  Elsewhere the append kernel runs first.  The
 * cache bytes, state and output equal those of dkv_append followed by
 * dkv_attn_decode.  Errors as those two calls.
 */
dkv_status dkv_append_attn_decode(const dkv_config *cfg, void *cache, float *state,
                                  const int32_t *block_table, const uint16_t *k_new,
                                  const uint16_t *v_new, const int32_t *positions, const float *q,
                                  const int32_t *seq_lens, float softmax_scale, float *out,
                                  void *workspace, size_t workspace_bytes, dkv_stream_t stream);

/* Split plan of dkv_attn_decode for cfg: *nsplit splits per (sequence,
 * kv-head), split s covering tokens [s * split_tokens, (s + 1) * split_tokens)
 * of the sequence.  Runs are at most 2048 tokens, 1024 in paged mode (ragged
 * serving batches: shorter runs keep the last partial round of runs short),
 * and at least 128 tokens (whole keyframe intervals) while that leaves 256
 * or more workgroups.
 * Errors: as dkv_check_config, DKV_ERR_ARG for null outputs. */
dkv_status dkv_attn_decode_plan(const dkv_config *cfg, int32_t *nsplit, int32_t *split_tokens);

/* The split phase of dkv_attn_decode alone: writes the per-split partial
 * results to the workspace and merges nothing (the arrival counters are left
 * untouched).  Partial record of (sequence b, query head hq, split s), at float
 * offset ((b*n_q_heads + hq)*nsplit + s)*(head_dim + 4) after the counters
 * (nsplit from dkv_attn_decode_plan): acc[head_dim] (sum of softmax weights
 * times V over the split's tokens, the weights relative to the running max),
 * running max (log2 units: logits times log2(e)), running sum, 2 pad floats.
 * A split whose run starts at or past min(seq_lens[b], capacity) holds no
 * token: its record may be left unwritten, and a merge reads only splits
 * s < ceil(min(seq_lens[b], capacity) / split_tokens).  For callers that merge
 * the splits themselves, and for timing the split phase alone.  Same
 * arguments as dkv_attn_decode without `out`. */
dkv_status dkv_attn_decode_partial(const dkv_config *cfg, const void *cache,
                                   const int32_t *block_table, const float *q,
                                   const int32_t *seq_lens, float softmax_scale,
                                   void *workspace, size_t workspace_bytes,
                                   dkv_stream_t stream);

/* Same as dkv_attn_decode but through the plain (unfused-layout-agnostic)
 * reference kernel: reconstructs each tile in fp32 and runs fp32 attention.
 * Kept as a cross-check of the fused kernel. */
dkv_status dkv_attn_decode_ref(const dkv_config *cfg, const void *cache,
                               const int32_t *block_table, const float *q,
                               const int32_t *seq_lens, float softmax_scale, float *out,
                               void *workspace, size_t workspace_bytes,
                               dkv_stream_t stream);

/*
 * Diagnostics.  Dense fp32 reconstruction of every cached token:
 *  k_out, v_out (device) fp32 [batch][n_kv_heads][s_max][head_dim]; rows at
 *  t >= seq_lens[b] are left untouched.
 */
dkv_status dkv_reconstruct(const dkv_config *cfg, const void *cache,
                           const int32_t *block_table, const int32_t *seq_lens,
                           int32_t s_max, float *k_out, float *v_out, dkv_stream_t stream);

/*
 * Diagnostics.  The encoded stream in canonical Q4_0 form, for bit-exact checks.
 * With ng = ceil(s_max/kf) and nd = s_max - ng, for stream s (0 = K, 1 = V):
 *  kf_rows (device) uint16 [batch][n_kv_heads][2][ng][head_dim], fp16 keyframes
 *  codes   (device) uint8  [batch][n_kv_heads][2][nd][head_dim/2], delta token t
 *          at row (t/kf)*(kf-1) + t%kf - 1, byte i of a block = code i | code i+16 << 4
 *  scales  (device) uint16 [batch][n_kv_heads][2][nd][head_dim/32]
 * codes and scales may be NULL when nd == 0 (kf == 1).
 * Rows beyond a sequence's length are left untouched.
 */
dkv_status dkv_export(const dkv_config *cfg, const void *cache, const int32_t *block_table,
                      const int32_t *seq_lens, int32_t s_max, uint16_t *kf_rows,
                      uint8_t *codes, uint16_t *scales, dkv_stream_t stream);

/*
 * In-run comparisons (the Delta-KV article's "벤치마크" section sets Delta-KV
 * against an F16 cache and a plain Q4_0 cache of absolute values).  Both
 * comparison caches are cut in 32-token tiles:
 *  - contiguous mode (page_tokens == 0): per (sequence, kv-head) a run of
 *    ceil(max_tokens/32) tiles, sequences and kv-heads in order;
 *  - paged mode: page_tokens must be a multiple of 32 (else
 *    DKV_ERR_UNSUPPORTED); a physical page holds every kv-head's tiles,
 *    [n_kv_heads][page_tokens/32], and block_table (device, int32
 *    [batch][max_pages_per_seq]) maps logical pages as for the Delta-KV cache.
 *    Tokens on an unmapped page (id < 0 or >= n_pages) are not attended.
 * kf is ignored.  Errors: as dkv_check_config, DKV_ERR_UNSUPPORTED,
 * DKV_ERR_ARG (null pointer; no block table in paged mode; s_max < 0),
 * DKV_ERR_WORKSPACE (workspace below dkv_workspace_bytes), DKV_ERR_HIP.
 *
 * Plain Q4_0 cache: 18 bytes per 32 elements (Q4_0 of the absolute values,
 * the block rule of the Delta-KV deltas with reference 0).  One tile is 36*D
 * bytes: [K scales 2D][K codes 16D][V scales 2D][V codes 16D].
 */
size_t dkv_q4_0_cache_bytes(const dkv_config *cfg);   /* 0 if cfg is invalid or unsupported */
/* Encodes tokens [0, min(seq_lens[b], s_max)) of k, v (device, fp16
 * [batch][n_kv_heads][s_max][head_dim]) into q4_cache (dkv_q4_0_cache_bytes). */
dkv_status dkv_q4_0_encode(const dkv_config *cfg, void *q4_cache, const int32_t *block_table,
                           const uint16_t *k, const uint16_t *v, const int32_t *seq_lens,
                           int32_t s_max, dkv_stream_t stream);
/* Decode attention over the Q4_0 cache; arguments as dkv_attn_decode. */
dkv_status dkv_attn_decode_q4_0(const dkv_config *cfg, const void *q4_cache,
                                const int32_t *block_table, const float *q,
                                const int32_t *seq_lens, float softmax_scale, float *out,
                                void *workspace, size_t workspace_bytes, dkv_stream_t stream);
/* Canonical export of the Q4_0 cache: codes uint8 [batch][Hkv][2][s_max][D/2],
 * scales uint16 [batch][Hkv][2][s_max][D/32]; rows past a sequence's length or
 * on an unmapped page are left untouched. */
dkv_status dkv_q4_0_export(const dkv_config *cfg, const void *q4_cache, const int32_t *block_table,
                           const int32_t *seq_lens, int32_t s_max, uint8_t *codes,
                           uint16_t *scales, dkv_stream_t stream);

/*
 * Q4-keyframe variant of the Delta-KV cache: the keyframe itself is stored as
 * Q4_0 of its absolute values, so every token takes the 4-bit storage of
 * Q4_0 (Delta-KV article, "벤치마크": the same 4-bit storage).  Token t of a
 * stream is one Q4_0 row (18 bytes per 32 values): at t % kf == 0 the row is
 * coded against zero, otherwise its closed-loop delta against the running
 * reconstruction, with the block rule of the Delta-KV codec; the
 * reconstruction is ref + (code - 8) * scale, ref = 0 at a keyframe, else the
 * previous reconstruction (one fp32 rounding).  With kf = 1 the cache is plain
 * Q4_0 byte for byte.
 * Layout and size: those of the plain Q4_0 cache (dkv_q4_0_cache_bytes, 32-token
 * tiles, contiguous or paged with page_tokens % 32 == 0); dkv_q4_0_export
 * gives its canonical codes and scales.  state: as dkv_state_bytes (the last
 * reconstructed K and V row of each sequence).
 * kf must divide 32 or be a multiple of 32 (else DKV_ERR_UNSUPPORTED); paged
 * mode also needs page_tokens % kf == 0 (dkv_check_config).
 */
/* Bulk prefill encode: arguments as dkv_encode_prefill, cache of
 * dkv_q4_0_cache_bytes(cfg) bytes. */
dkv_status dkv_q4k_encode_prefill(const dkv_config *cfg, void *cache, float *state,
                                  const int32_t *block_table, const uint16_t *k,
                                  const uint16_t *v, const int32_t *seq_lens, int32_t s_max,
                                  dkv_stream_t stream);
/* One token per sequence: arguments as dkv_append (negative position skips). */
dkv_status dkv_q4k_append(const dkv_config *cfg, void *cache, float *state,
                          const int32_t *block_table, const uint16_t *k_new,
                          const uint16_t *v_new, const int32_t *positions, dkv_stream_t stream);
/* Reconstructed K and V of tokens [0, min(seq_lens[b], s_max)): k_out, v_out
 * (device) fp32 [batch][n_kv_heads][s_max][head_dim]; other rows untouched. */
dkv_status dkv_q4k_reconstruct(const dkv_config *cfg, const void *cache,
                               const int32_t *block_table, const int32_t *seq_lens, int32_t s_max,
                               float *k_out, float *v_out, dkv_stream_t stream);
/* Decode attention over the Q4-keyframe cache; arguments as dkv_attn_decode.
 * kf = 1 (plain Q4_0) or kf = 32, at most 8 query heads per kv-head; else
 * DKV_ERR_UNSUPPORTED.  Two launches: split phase (logits by prefix sums and
 * weights by suffix sums over each 32-token tile, as in the Delta-KV kernel),
 * then the split combine. */
dkv_status dkv_attn_decode_q4k(const dkv_config *cfg, const void *cache,
                               const int32_t *block_table, const float *q,
                               const int32_t *seq_lens, float softmax_scale, float *out,
                               void *workspace, size_t workspace_bytes, dkv_stream_t stream);

/*
 * Decode attention over an F16 cache (the unquantised baseline): k and v are
 * two arrays of fp16 token rows in the tile layout above, i.e. (device)
 *  contiguous: fp16 [batch][n_kv_heads][max_tokens][head_dim];
 *  paged:      fp16 [n_pages][n_kv_heads][page_tokens][head_dim].
 * Other arguments as dkv_attn_decode.
 */
dkv_status dkv_attn_decode_f16(const dkv_config *cfg, const uint16_t *k, const uint16_t *v,
                               const int32_t *block_table, const float *q,
                               const int32_t *seq_lens, float softmax_scale, float *out,
                               void *workspace, size_t workspace_bytes, dkv_stream_t stream);

/*
 * Quality comparison: plain Q8_0 of absolute values, the 8-bit reference the
 * Delta-KV article's "벤치마크" section sets Delta-KV against (34 bytes per 32
 * elements).  Per block of 32 channels of a token: d = max|x| / 127, code =
 * round-half-away-from-zero(x * (1/d)) in -127..127, stored scale fp16(d)
 * (round to nearest even); the value it stands for is code * scale.
 *  k, v     (device) fp16 bits [batch][n_kv_heads][s_max][head_dim]
 *  seq_lens (device) int32 [batch]; rows t >= min(seq_lens[b], s_max) are
 *           left untouched
 *  codes    (device) int8  [batch][n_kv_heads][2][s_max][head_dim]
 *  scales   (device) uint16 [batch][n_kv_heads][2][s_max][head_dim/32]
 * Only the quantised arrays are produced (no attention kernel reads them).
 * Errors: as dkv_check_config, DKV_ERR_ARG (null pointer, s_max < 0),
 * DKV_ERR_HIP.  Asynchronous on `stream`.
 */
dkv_status dkv_q8_0_encode(const dkv_config *cfg, const uint16_t *k, const uint16_t *v,
                           const int32_t *seq_lens, int32_t s_max, int8_t *codes, uint16_t *scales,
                           dkv_stream_t stream);

/*
 * Diagnostic: attention-preserving distortion of reconstructed keys and values
 * ("KV 캐시 벡터 양자화와 주의 보존 변환", section 어텐션 보존 왜곡), one
 * decode step, per (sequence b, query head hq) over the sequence's tokens
 * t < min(seq_lens[b], s_max), kv-head h = hq / (n_q_heads / n_kv_heads):
 *   d_k[b][hq] = sum_t ( q . (k_hat_t - k_t) )^2        (unscaled logit row)
 *   d_v[b][hq] = || sum_t a_t (v_hat_t - v_t) ||^2,
 *   a_t = softmax_t( softmax_scale * q . k_t )          (exact keys)
 * The page's expectation E[.] is the mean of these over the rows.
 *  k_hat, v_hat (device) float [batch][n_kv_heads][s_max][head_dim]: the
 *               reconstruction under test (dkv_reconstruct's output, or any other)
 *  k, v         (device) fp16 bits [batch][n_kv_heads][s_max][head_dim]: originals
 *  q            (device) float [batch][n_q_heads][head_dim]
 *  seq_lens     (device) int32 [batch]
 *  softmax_scale  0 => 1/sqrt(head_dim)
 *  logits       (device) float [batch][n_q_heads][s_max], caller-owned scratch
 *               (holds the exact scaled logits afterwards)
 *  d_k, d_v     (device) float [batch][n_q_heads]; a row with no tokens gets 0
 * Only batch, n_q_heads, n_kv_heads and head_dim of cfg are used (head_dim 64
 * or 128).  Errors: DKV_ERR_ARG (null pointer, s_max < 1, bad head counts),
 * DKV_ERR_UNSUPPORTED (head_dim), DKV_ERR_HIP.  Asynchronous on `stream`.
 */
dkv_status dkv_attn_distortion(const dkv_config *cfg, const float *k_hat, const float *v_hat,
                               const uint16_t *k, const uint16_t *v, int32_t s_max, const float *q,
                               const int32_t *seq_lens, float softmax_scale, float *logits,
                               float *d_k, float *d_v, dkv_stream_t stream);

/*
 * Diagnostic: the streaming-read ceiling.  Decode attention is a streaming
 * read of the cache (the cost model of "KV 캐시 벡터 양자화와 주의 보존 변환",
 * section "KV 캐시가 왜 병목인가"); this call only reads, with no arithmetic of
 * the method, so its rate is the practical bandwidth the decode kernels are
 * measured against.
 *  buf  (device) any readable buffer; the first floor(bytes/16)*16 bytes are
 *       read once with 16-byte loads.  bytes >= 16.
 *  sink (device) uint32 [dkv_stream_read_sink_words()], caller-owned: one word
 *       per work-item, the XOR of the 32-bit words it read (the XOR of all sink
 *       words is the XOR of all words read).
 * Errors: DKV_ERR_ARG (null pointer, bytes < 16), DKV_ERR_WORKSPACE (sink too
 * small), DKV_ERR_HIP (launch failure).  Asynchronous on `stream`.
 */
size_t dkv_stream_read_sink_words(void);
dkv_status dkv_stream_read(const void *buf, size_t bytes, uint32_t *sink, size_t sink_words,
                           dkv_stream_t stream);

/*
 * Strided-reference residual cache (the gist.science explainer of DeltaKV,
 * section 3.A: "Strided Reference Selection", "Residual Encoding",
 * "Reconstruction").  The tokens at positions 0, kf, 2*kf, ... (cfg->kf is the
 * stride) are kept as exact fp16 reference rows; every token stores the index
 * of its nearest reference and the Q4_0 code of its residual against it, and
 * decodes as reference + (code - 8) * scale.  Nearest: smallest squared
 * distance of the fp16 rows, summed in double over the channels in order
 * without fused multiply-add, lowest index on ties, among references
 * k <= t / kf (and k > t / kf - window when window > 0).  A NaN distance
 * (non-finite rows, outside the finite-input contract) ranks above every
 * number, so such a row still takes one of its candidates.  Contiguous mode only
 * (page_tokens must be 0), at most 65536 references per sequence; otherwise
 * DKV_ERR_UNSUPPORTED.
 *
 * Cache: streams [batch][n_kv_heads][K, V] of dkv_strided_layout()[4] bytes
 * each; inside a stream, at the offsets of dkv_strided_layout():
 *   [0] refs   fp16 [nref][head_dim]        nref = layout[5] = ceil(capacity / kf)
 *   [1] codes  u8   [capacity][head_dim/2]  Q4_0 bytes, byte i of a block: code i | code i+16 << 4
 *   [2] scales fp16 [capacity][head_dim/32]
 *   [3] idx    u16  [capacity]              reference index per token
 */
size_t dkv_strided_cache_bytes(const dkv_config *cfg);  /* 0 if cfg is invalid or unsupported */

/* layout (host) int64 [6]: plane offsets [0..3], stream bytes [4], nref [5]. */
dkv_status dkv_strided_layout(const dkv_config *cfg, int64_t *layout);

/*
 * Encode tokens [0, min(seq_lens[b], s_max, capacity)) of every sequence.
 *  k, v     (device) fp16 [batch][n_kv_heads][s_max][head_dim]
 *  seq_lens (device) int32 [batch]
 *  cache    (device) dkv_strided_cache_bytes(cfg) bytes; the encoded tokens'
 *           entries and references are written, the rest is left untouched
 *  window   0: every earlier reference is a candidate; else the last `window`
 * One workgroup per (32-token tile, kv-head, K/V, sequence).  Errors: as
 * dkv_check_config, DKV_ERR_UNSUPPORTED (see above), DKV_ERR_ARG (null
 * pointer, s_max < 0, window < 0), DKV_ERR_HIP.  Asynchronous on `stream`.
 */
dkv_status dkv_strided_encode_prefill(const dkv_config *cfg, void *cache, const uint16_t *k,
                                      const uint16_t *v, const int32_t *seq_lens, int32_t s_max,
                                      int32_t window, dkv_stream_t stream);

/*
 * Append one token per sequence to the strided-reference cache, coded exactly
 * as dkv_strided_encode_prefill codes it (the candidates are read from the
 * cache's reference rows; with the same window the bytes equal those of a
 * prefill over the grown sequence).
 *  k_new, v_new (device) fp16 [batch][n_kv_heads][head_dim]
 *  positions    (device) int32 [batch]: the token's index t; a sequence with
 *               t < 0 or t >= capacity is skipped.  Tokens 0..t-1 must
 *               already be encoded (prefill or earlier appends).
 * One workgroup per (kv-head, K/V, sequence).  Errors: as
 * dkv_strided_encode_prefill.  Asynchronous on `stream`.
 */
dkv_status dkv_strided_append(const dkv_config *cfg, void *cache, const uint16_t *k_new,
                              const uint16_t *v_new, const int32_t *positions, int32_t window,
                              dkv_stream_t stream);

/*
 * One serving step on the strided-reference cache in one call:
 * dkv_strided_append (k_new, v_new, positions, window) followed by
 * dkv_strided_attn_decode (q, seq_lens, ...), with the append done inside the
 * decode's split launch by the workgroup whose run holds the new token.  The
 * cache bytes and the output are identical to the two separate calls.
 * seq_lens must already count the new token (position + 1).  Errors: as the
 * two calls.  Two launches on `stream` (split phase with the append, combine).
 */
dkv_status dkv_strided_append_attn_decode(const dkv_config *cfg, void *cache, const uint16_t *k_new,
                                          const uint16_t *v_new, const int32_t *positions,
                                          int32_t window, const float *q, const int32_t *seq_lens,
                                          float softmax_scale, float *out, void *workspace,
                                          size_t workspace_bytes, dkv_stream_t stream);

/*
 * Decode attention over the strided-reference cache: out[b][hq] =
 * softmax(scale * q . K_hat^T) V_hat over tokens t < min(seq_lens[b], capacity),
 * arguments as dkv_attn_decode (workspace of dkv_workspace_bytes(cfg) bytes).
 * Two launches on `stream`: the split phase (one wave per run of 32-token
 * tiles; logits in the residual domain, q.r_idx + sum_b s_b q_b.(c_b - 8), on
 * fp16 matrix instructions; V rebuilt in fp32), then the split combine.  A
 * sequence of length 0 gives zero rows.
 */
dkv_status dkv_strided_attn_decode(const dkv_config *cfg, const void *cache, const float *q,
                                   const int32_t *seq_lens, float softmax_scale, float *out,
                                   void *workspace, size_t workspace_bytes, dkv_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DKV_H */
