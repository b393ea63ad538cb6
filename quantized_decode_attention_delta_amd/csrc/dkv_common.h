// Shared definitions of the Delta-KV HIP library: cache geometry, the
// channel permutations of the group record, and small device helpers.
//
// Geometry of one group record (K part, then V part; every piece 16-byte
// aligned).  nb = D/32 Q4_0 blocks per row.
//   keyframe   2*D bytes          fp16, permuted (see kf_k_channel / kf_v_channel)
//   scales     pad16(kf*nb*2)     fp16 [kf][nb]; slot 0 = per-block max |scale|
//   codes (K)  pad16((kf-1)*D/2)  one row per delta token; the 16 canonical
//                                 Q4_0 bytes of block b are split in four
//                                 32-bit pieces, piece j at word j*nb + b
//   codes (V)  ntiles*16*D        32-token tiles; word vcode_word: lane
//                                 16*j+m's word cc holds channel vchan(cc, m)
//                                 for the 8 token slots 16*e+4*j+r (r<4, e<2)
//                                 at nibble r+4*e
// The permutations line the data up with the operand layout of the gfx950
// 16x16x32 fp16 matrix instruction (lane = 16*j + m, eight K values per lane).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dkv.h"

namespace dkv {

constexpr int kMaxKf = 1024;
// Cache policy of the attention kernels' loads of the compressed cache: the
// default one.  With the nontemporal hint (2) the kf = 32 kernel fetched 5%
// more bytes from HBM (cache lines shared by neighbouring loads were fetched
// twice) at the same speed.
constexpr int kStream = 0;
constexpr int kWave = 64;

__host__ __device__ inline int64_t pad16(int64_t x) { return (x + 15) & ~int64_t(15); }

// Split-K partial record per (sequence, query head, split): acc[D], running
// max (log2 units), running sum, two pad floats (16-byte aligned records).
__host__ __device__ constexpr int part_stride(int D) { return D + 4; }

// Workspace of the decode calls: first one 32-bit arrival counter per
// (sequence, kv-head) (zero between calls: the split kernels that merge their
// own partials count their arrivals there and the last one resets it), padded
// to 256 bytes, then the split-K partial records.
__host__ __device__ inline int64_t counter_bytes(const dkv_config &c)
{
    return ((int64_t)c.batch * c.n_kv_heads * 4 + 255) & ~int64_t(255);
}

// Where a split kernel that merges its own partial records writes the result:
// out[B][Hq][D]; counter[B][Hkv] are the arrival counters.  out == nullptr:
// partial records only (a separate combine kernel merges them).
struct CombineTail {
    float *out;
    uint32_t *counter;
};

struct Geom {
    int D, nb, kf, Hkv, Hq, G, B;
    int ntiles_v;              // 32-token tiles of V codes per group
    int vbp;                   // V tiles in block-pair order (see vchan)
    int64_t off_ksc, off_kcd, off_vkf, off_vsc, off_vcd, rec;
    // addressing
    int paged;                 // 1 if paged
    int gpp;                   // groups per page (paged) or per sequence (contiguous)
    int64_t page_bytes;        // bytes of a page (paged) or of one sequence (contiguous)
    int max_pages;             // block-table row length (paged)
    int n_pages;               // physical pages (paged)
    int ng_cap;                // group capacity per sequence
    int cap_tokens;            // token capacity per sequence
};

// V code tiles use the block-pair row order when at most 8 query heads share
// a kv-head (the matrix-core kernels then spend the 8 spare operand columns
// on the second block of a pair), kf is a multiple of 32 up to 512 and D is
// 64 or 128.
__host__ __device__ inline int vbp_layout(const dkv_config &c)
{
    return c.kf % 32 == 0 && c.kf <= 512 && c.n_q_heads / c.n_kv_heads <= 8 &&
           (c.head_dim == 64 || c.head_dim == 128);
}

__host__ __device__ inline Geom make_geom(const dkv_config &c)
{
    Geom g{};
    g.D = c.head_dim;
    g.nb = c.head_dim / 32;
    g.kf = c.kf;
    g.Hkv = c.n_kv_heads;
    g.Hq = c.n_q_heads;
    g.G = c.n_q_heads / c.n_kv_heads;
    g.B = c.batch;
    g.ntiles_v = c.kf > 1 ? (c.kf + 31) / 32 : 0;
    g.vbp = vbp_layout(c);
    int64_t kfb = 2 * (int64_t)g.D;
    int64_t scb = pad16((int64_t)c.kf * g.nb * 2);
    int64_t kcb = pad16((int64_t)(c.kf - 1) * g.D / 2);
    g.off_ksc = kfb;
    g.off_kcd = g.off_ksc + scb;
    g.off_vkf = g.off_kcd + kcb;
    g.off_vsc = g.off_vkf + kfb;
    g.off_vcd = g.off_vsc + scb;
    // records padded to whole 128-byte cache lines: a record's lines are its
    // own, so the keyframe lines the decode reads ahead of the rest of the
    // record are never fetched a second time with a neighbour's data
    g.rec = (g.off_vcd + (int64_t)g.ntiles_v * 16 * g.D + 127) & ~int64_t(127);
    g.paged = c.page_tokens > 0;
    if (g.paged) {
        g.gpp = c.page_tokens / c.kf;
        g.page_bytes = (int64_t)g.Hkv * g.gpp * g.rec;
        g.max_pages = c.max_pages_per_seq;
        g.n_pages = c.n_pages;
        g.cap_tokens = c.max_pages_per_seq * c.page_tokens;
        g.ng_cap = g.cap_tokens / c.kf;
    } else {
        g.ng_cap = (c.max_tokens + c.kf - 1) / c.kf;
        g.gpp = g.ng_cap;
        g.page_bytes = (int64_t)g.Hkv * g.ng_cap * g.rec;
        g.max_pages = 1;
        g.n_pages = c.batch;
        g.cap_tokens = g.ng_cap * c.kf;
    }
    return g;
}

// Byte offset of the group record of (sequence b, kv-head h, group gi).
// Returns -1 for an unmapped (or out-of-range) page in paged mode.
// The new token of each sequence, appended by the decode kernel itself (one
// launch per serving step): null `positions` means no append.
struct AppendArgs {
    uint8_t *cache;                 // the cache the kernel reads, writable
    float *state;                   // reconstruction state [B][Hkv][2][D]
    const uint16_t *knew, *vnew;    // fp16 [B][Hkv][D]
    const int32_t *positions;       // [B]: index of the new token
};

__host__ __device__ inline int64_t group_offset(const Geom &g, const int32_t *block_table,
                                                int b, int h, int gi)
{
    if (g.paged) {
        int lp = gi / g.gpp;
        int phys = block_table[(int64_t)b * g.max_pages + lp];
        if (phys < 0 || phys >= g.n_pages) return -1;
        return (int64_t)phys * g.page_bytes + ((int64_t)h * g.gpp + gi % g.gpp) * g.rec;
    }
    return (int64_t)b * g.page_bytes + ((int64_t)h * g.gpp + gi) * g.rec;
}

// ---- comparison caches (plain Q4_0, F16): 32-token tiles ----------------------
// Both comparison caches are cut in 32-token tiles.  Contiguous mode: per
// (sequence, kv-head) a run of ceil(max_tokens/32) tiles.  Paged mode (the
// layout of the Delta-KV cache's pages, which needs page_tokens % 32 == 0 here):
// a page of page_tokens tokens holds every kv-head's tiles,
// [n_kv_heads][page_tokens/32], and block_table maps a sequence's logical page
// to a physical one.  cmp_tile_index returns the tile's index in units of one
// tile of one kv-head, or -1 for an unmapped (or out-of-range) page.
__host__ __device__ inline int cmp_ntiles(const dkv_config &c)
{
    return c.page_tokens > 0 ? c.max_pages_per_seq * (c.page_tokens / 32) : (c.max_tokens + 31) / 32;
}
__host__ __device__ inline int64_t cmp_tile_index(const dkv_config &c, const int32_t *block_table, int b, int h,
                                                  int tile)
{
    if (c.page_tokens > 0) {
        const int tpp = c.page_tokens / 32;
        const int phys = block_table[(int64_t)b * c.max_pages_per_seq + tile / tpp];
        if (phys < 0 || phys >= c.n_pages) return -1;
        return ((int64_t)phys * c.n_kv_heads + h) * tpp + tile % tpp;
    }
    return ((int64_t)b * c.n_kv_heads + h) * cmp_ntiles(c) + tile;
}

// Plain Q4_0 tile: 36*D bytes, [K scales 2D][K codes 16D][V scales 2D][V codes
// 16D], codes in the same orders as the Delta-KV K code rows and V code tiles
// (V in block-pair order under the same condition on G and D).
__host__ __device__ inline int64_t q40_tile_bytes(int D) { return 36LL * D; }
__host__ __device__ inline int q40_ntiles(const dkv_config &c) { return cmp_ntiles(c); }
__host__ __device__ inline int64_t q40_tile_offset(const dkv_config &c, const int32_t *block_table, int b, int h,
                                                   int tile)
{
    const int64_t t = cmp_tile_index(c, block_table, b, h, tile);
    return t < 0 ? -1 : t * q40_tile_bytes(c.head_dim);
}
// F16 tile: 32 token rows of D fp16 values, separately for K and V (two
// arrays of the same layout); element offset of the tile's first row, or -1.
__host__ __device__ inline int64_t f16_tile_elem(const dkv_config &c, const int32_t *block_table, int b, int h,
                                                 int tile)
{
    if (c.page_tokens > 0) {
        const int64_t t = cmp_tile_index(c, block_table, b, h, tile);
        return t < 0 ? -1 : t * 32 * c.head_dim;
    }
    return (((int64_t)b * c.n_kv_heads + h) * c.max_tokens + 32LL * tile) * c.head_dim;
}
__host__ __device__ inline int q40_vbp(const dkv_config &c)
{
    return c.n_q_heads / c.n_kv_heads <= 8 && (c.head_dim == 64 || c.head_dim == 128);
}

// ---- channel permutations -------------------------------------------------
// Within a 32-bit code piece (canonical bytes 4j..4j+3 of a block), nibble p
// is byte p/2, low (p even) or high (p odd) half, i.e. block channel
// 4j + p/2 + 16*(p&1).  The matrix-core unpack places nibble r+4e in half
// 2r+e of the eight K values.  kf_k_channel gives the block channel held in
// half h of lane group j.
__host__ __device__ inline int half_to_nibble(int h) { return (h >> 1) + 4 * (h & 1); }
__host__ __device__ inline int nibble_channel(int j, int p) { return 4 * j + (p >> 1) + 16 * (p & 1); }
__host__ __device__ inline int kf_k_channel(int j, int h) { return nibble_channel(j, half_to_nibble(h)); }

// K keyframe: element (j*nb + b)*8 + h holds channel 32*b + kf_k_channel(j, h).
__host__ __device__ inline int kkf_pos(int nb, int c)
{
    int b = c >> 5, cb = c & 31;
    int hi = cb >> 4, rem = cb & 15;           // cb = 4j + k + 16*hi
    int j = rem >> 2, k = rem & 3;
    int p = 2 * k + hi;                        // nibble position
    int h = 2 * (p & 3) + (p >> 2);            // inverse of half_to_nibble
    return (j * nb + b) * 8 + h;
}
// V tile rows.  A V code tile is D/16 slices of 16 rows (cc, m), each row one
// channel.  Plain order: vchan(cc, m) = 16*cc + m (slice cc lies in block
// cc/2).  Block-pair order (bp): with np = nb/2 block pairs (p, p+np), slice
// cc = 4p + c4 holds channels 8*c4 + (m & 7) of block p in rows m < 8 and of
// block p + np in rows m >= 8.
__host__ __device__ inline int vchan(int D, int cc, int m, int bp)
{
    if (!bp) return 16 * cc + m;
    const int np = D / 64, p = cc >> 2, c4 = cc & 3;
    return 32 * (p + (m >> 3) * np) + 8 * c4 + (m & 7);
}
// inverse of vchan: slice and row of channel c
__host__ __device__ inline void vslot(int D, int c, int bp, int &cc, int &m)
{
    if (!bp) {
        cc = c >> 4;
        m = c & 15;
        return;
    }
    const int np = D / 64, b = c >> 5, w = c & 31;
    const int hi = b >= np;
    cc = 4 * (b - hi * np) + (w >> 3);
    m = 8 * hi + (w & 7);
}
// V keyframe: element (j*(D/16) + cc)*4 + r holds channel vchan(cc, 4*j + r),
// the accumulator order of the V-side matrix instruction.
__host__ __device__ inline int vkf_pos(int D, int c, int bp)
{
    int cc, m;
    vslot(D, c, bp, cc, m);
    int j = m >> 2, r = m & 3;
    return (j * (D / 16) + cc) * 4 + r;
}
// K code row: byte offset of canonical byte i (0..15) of block b.
__host__ __device__ inline int kcode_byte(int nb, int b, int i) { return 4 * ((i >> 2) * nb + b) + (i & 3); }
// V code tile: lane l = 16*j + m of the decode kernels holds the D/16 words
// of row m (slices cc = 0 .. D/16-1) for its token slots.  With D/16 a
// multiple of 4 the words go in 16-byte pieces: piece q4 (words 4*q4 .. 4*q4+3
// of every lane) is one contiguous run over the 64 lanes, so that each
// 16-byte load of a wave reads whole cache lines; otherwise a lane's words
// are consecutive.  vcode_piece: byte offset of lane l's piece q4.
__host__ __device__ inline int vcode_piece(int D, int lane, int q4)
{
    return (D / 16) % 4 == 0 ? 1024 * q4 + 16 * lane : lane * (D / 16) * 4 + 16 * q4;
}
// V code tile: word index and nibble of (token slot tau in 0..31, channel c).
__host__ __device__ inline int vcode_word(int D, int tau, int c, int bp)
{
    int j = (tau & 15) >> 2;
    int cc, m;
    vslot(D, c, bp, cc, m);
    return vcode_piece(D, j * 16 + m, cc >> 2) / 4 + (cc & 3);
}
__host__ __device__ inline int vcode_nibble(int tau) { return (tau & 3) + 4 * (tau >> 4); }

// ---- small device helpers --------------------------------------------------
// Split (run) index of a workgroup of a (split, kv-head, batch) decode grid.
// The chip hands workgroups to its 8 XCDs round-robin in linear order, so
// with an even split count the same run positions of every row would land on
// the same XCDs; in a ragged batch those are the first runs, the ones every
// sequence has, and the XCDs that hold them get more work (10-13 % above the
// mean on 1K..64K-token batches with 64 splits).  Rotating row r's runs by r
// spreads them over all eight (an odd split count already does).
__device__ inline int grid_split()
{
    const unsigned row = blockIdx.z * gridDim.y + blockIdx.y;
    return (gridDim.x & 1u) ? (int)blockIdx.x : (int)((blockIdx.x + row) % gridDim.x);
}
// fp16 <-> fp32 through the compiler's _Float16 (v_cvt_f32_f16 / v_cvt_f16_f32,
// round to nearest even, subnormals kept).
__device__ inline float h2f(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }
__device__ inline uint16_t f2h_rn(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

}  // namespace dkv
