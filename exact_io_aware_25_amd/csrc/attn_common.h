// attn_common.h -- device and host helpers shared by the forward and the
// backward kernels (gfx950).  Internal to the library: not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRowsPerWave = 32;
constexpr int kBlockK = 64;  // keys per K/V tile

template <typename T> struct Vec8;
template <> struct Vec8<_Float16> { typedef f16x8 type; };
template <> struct Vec8<__bf16> { typedef bf16x8 type; };

__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}


// Row of the K tile that feeds A-operand row m: bits 2 and 3 swapped.  With
// this order, accumulator register r (0..15) of lane half `hi` in a 32-key
// block holds key 16*(r/8) + 8*hi + r%8, i.e. 8 consecutive keys per 16-key
// slice -- the layout the B operand of the second product needs.
__host__ __device__ __forceinline__ int k_row_for_lane(int m)
{
    return (m & ~0xC) | ((m & 4) << 1) | ((m & 8) >> 1);
}

template <bool CAUSAL, bool WINDOW>
__host__ __device__ __forceinline__ bool visible(int i, int j, int L, int window)
{
    if (j >= L) return false;
    if (CAUSAL && j > i) return false;
    if (WINDOW) {
        if (i - j > window) return false;
        if (!CAUSAL && j - i > window) return false;
    }
    return true;
}

// XOR swizzles of the 16-byte units of each LDS tile row (tiles are not
// padded).  A row of D 16-bit values has D/8 units; unit u of row r is stored
// at unit u ^ f(r).  The functions are chosen so that both reads are free of
// bank conflicts whether the LDS serves 8 lanes x 16 bytes (32 banks) or 16
// lanes x 16 bytes (64 banks) per cycle:
//  * K is read 16 bytes per lane from the 16 rows k_row_for_lane(0..15) of a
//    32-row block, all at the same logical unit: f must be a bijection on row
//    bits {0,1,3} (the first 8 of those rows) and on bits {1,2,3} for a fixed
//    bit 0 (16 rows over two 128-byte halves);
//  * V is read 8 bytes per lane by the transposing load, four consecutive rows
//    at a time with two (16 lanes) or four (32 lanes) consecutive units per
//    row: f must move the unit pair, and for 32 lanes the unit quad, of each
//    of the four rows to a different place.
template <int D> __host__ __device__ __forceinline__ int k_swizzle(int row)
{
    const int b0 = row & 1, b1 = (row >> 1) & 1, b2 = (row >> 2) & 1, b3 = (row >> 3) & 1;
    return (b0 ^ b2) | (b1 << 1) | (b3 << 2) | (D == 128 ? (b2 << 3) : 0);
}
template <int D> __host__ __device__ __forceinline__ int v_swizzle(int row)
{
    const int c = row & 3;
    return (c << 1) | (D == 128 ? ((c & 1) << 3) : 0);
}

// Copy 16 bytes per lane from a buffer into LDS without passing through
// VGPRs: lane i's bytes land at lds_dst + 16*i (lds_dst is wave-uniform).
__device__ __forceinline__ void copy_to_lds16(__amdgpu_buffer_rsrc_t src, void *lds_dst, int src_offset)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (__attribute__((address_space(3))) void *)lds_dst, 16,
                                             src_offset, 0, 0, 0);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Transposing 8-byte LDS read: within each group of 16 lanes, lane 4a+b gets
// element b of the 8-byte chunks addressed by lanes a, a+4, a+8 and a+12.
__device__ __forceinline__ s16x4 lds_read_tr16(const void *generic_lds_ptr)
{
    auto p = (__attribute__((address_space(3))) char *)(generic_lds_ptr);
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)p);
}

__device__ __forceinline__ float half_swap_max(float x)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x)
{
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float sum8(f16x8 v, float acc)
{
    const f16x2 one = {1, 1};
    acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(v, v, 0, 1), one, acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(v, v, 2, 3), one, acc, false);
    acc = __builtin_amdgcn_fdot2(__builtin_shufflevector(v, v, 4, 5), one, acc, false);
    return __builtin_amdgcn_fdot2(__builtin_shufflevector(v, v, 6, 7), one, acc, false);
}

// XOR swizzle for a tile that is read both ways: 16 bytes per lane from the
// rows k_row_for_lane(0..31) (as K above) and by the transposing load from
// four consecutive rows (as V above).  Found by exhaustive search over the
// linear (XOR) functions of the row bits under both LDS bank models: for
// d=64 f = b1 | (b0^b2)<<1 | (b1^b3)<<2, for d=128
// f = b0 | b1<<1 | (b0^b3)<<2 | (b1^b2)<<3.  It depends on bit 2 of the row,
// so the second transposing read (rows +4) needs its own offset.
template <int D> __host__ __device__ __forceinline__ int dual_swizzle(int row)
{
    const int b0 = row & 1, b1 = (row >> 1) & 1, b2 = (row >> 2) & 1, b3 = (row >> 3) & 1;
    if (D == 64) return b1 | ((b0 ^ b2) << 1) | ((b1 ^ b3) << 2);
    return b0 | (b1 << 1) | ((b0 ^ b3) << 2) | ((b1 ^ b2) << 3);
}

// ---- lane -> LDS offset and tile-range arithmetic shared by the kernels.
// Host-callable as well, so that tests can enumerate every lane, step and
// launch shape on the CPU and check each offset against its tile and each
// read against the element it must deliver.

// The swizzle a 16-bit tile was stored with.
enum SwizzleKind { kSwzK = 0, kSwzV = 1, kSwzDual = 2 };
template <int D, int KIND> __host__ __device__ __forceinline__ int swizzle_of(int row)
{
    return KIND == kSwzK ? k_swizzle<D>(row) : (KIND == kSwzV ? v_swizzle<D>(row) : dual_swizzle<D>(row));
}

// Byte offset of 16-byte logical unit `unit` of tile row `row`, stored at
// unit `unit ^ swz` of a row of `row_bytes` bytes.
__host__ __device__ __forceinline__ int swizzled_offset(int row, int unit, int swz, int row_bytes)
{
    return row * row_bytes + 16 * (unit ^ swz);
}

// K fragment (A operand of S^T = K Q^T, 32x32x16) of 16-bit tile rows: lane
// l reads 16 bytes, d = 16 ds + 8 (l / 32) .. + 7, of row k_row_for_lane(l %
// 32) of a 32-row block (add 32 kb rows for block kb).  KIND: the swizzle
// the tile was stored with.
template <int D, int KIND>
__host__ __device__ __forceinline__ int k_frag_offset(int lane, int ds)
{
    const int row = k_row_for_lane(lane % 32);
    return swizzled_offset(row, 2 * ds + lane / 32, swizzle_of<D, KIND>(row), 2 * D);
}

// Transposing 8-byte reads (ds_read_b64_tr_b16) of a row-major tile for d
// block db: within each 16-lane group, lane 4a + b receives element b of the
// chunks of lanes a, a+4, a+8, a+12, so after the read at r4 = 0 lane l holds
// rows 8 (l / 32) + 0..3 of column 32 db + l % 32, and after the read at
// r4 = 1 rows 8 (l / 32) + 4..7.  16-key slice ks adds 16 ks rows, which no
// swizzle here changes (they depend on row bits 0..3); the V and K swizzles
// depend on row & 3 only, so their r4 = 1 read is also the r4 = 0 address plus
// four rows.
template <int D, int KIND>
__host__ __device__ __forceinline__ int v_tr_offset(int lane, int db, int r4 = 0)
{
    const int row = 8 * (lane >> 5) + ((lane >> 2) & 3) + 4 * r4;
    const int unit = 4 * db + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    return swizzled_offset(row, unit, swizzle_of<D, KIND>(row), 2 * D) + 8 * (lane & 1);
}

// Source byte offset (within a tile of 16-bit rows of D values) of the 16
// bytes a lane copies into LDS unit `lds_unit`: the logical unit that the
// swizzle places there (a wave-wide copy fills 64 consecutive LDS units in
// lane order; XOR makes placement and lookup the same map).
template <int D, int KIND>
__host__ __device__ __forceinline__ int copy_src_offset(int lds_unit)
{
    const int row = lds_unit / (D / 8), phys = lds_unit % (D / 8);
    return swizzled_offset(row, phys, swizzle_of<D, KIND>(row), 2 * D);
}

// XOR swizzle of the 16-byte units of an fp8 tile row (D/16 units per row),
// found by exhaustive search over linear functions of the row bits so that
// both reads are free of bank conflicts (32- and 64-bank models): the K rows
// read 16 bytes per lane from rows k_row_for_lane(0..31), the V rows read by
// the 8-bit transposing load, 8 rows x 16 bytes per 16-lane group.
template <int D> __host__ __device__ __forceinline__ int f8_swizzle(int row)
{
    const int b0 = row & 1, b1 = (row >> 1) & 1, b2 = (row >> 2) & 1, b3 = (row >> 3) & 1;
    if (D == 64) return (b1 ^ b2) | ((b2 ^ b3) << 1);
    return b1 | ((b0 ^ b2) << 1) | ((b0 ^ b1 ^ b3) << 2);
}

// fp8 K fragment (A operand of the 32x32x64 fp8 product): lane l holds 32
// contiguous d-bytes 64 ds + 32 (l / 32) .. + 31 of row k_row_for_lane(l %
// 32), read as two 16-byte units (sp = 0, 1); add 32 kb rows for block kb.
template <int D>
__host__ __device__ __forceinline__ int f8_k_frag_offset(int lane, int ds, int sp)
{
    const int row = k_row_for_lane(lane % 32);
    return swizzled_offset(row, 4 * ds + 2 * (lane / 32) + sp, f8_swizzle<D>(row), D);
}

// 8-bit transposing V read (ds_read_b64_tr_b8) for d block db: read rho =
// 2 kb + t adds 32 kb + 16 t rows; the base addresses key row 8 (grp / 2) +
// li / 2 at d bytes 32 db + 16 (grp % 2) + 8 (li % 2), with grp = l / 16 and
// li = l % 16 (these row offsets keep the swizzle, which depends on row bits
// 0..3 only through rows 0..15 of each 16-row run).
template <int D>
__host__ __device__ __forceinline__ int f8_v_tr_offset(int lane, int db)
{
    const int grp = lane / 16, li = lane % 16;
    const int row = 8 * (grp / 2) + li / 2;
    return swizzled_offset(row, 2 * db + grp % 2, f8_swizzle<D>(row), D) + 8 * (li % 2);
}

// Source offset of the 16 bytes a lane copies into fp8 LDS unit `unit` of
// the [K | V] tile pair (units below 64 D / 16 are K's, the rest V's, each
// tile of 64 rows of D bytes): the logical unit the swizzle places there,
// within its own tile.
template <int D>
__host__ __device__ __forceinline__ int f8_copy_src_offset(int unit)
{
    const int u = unit % (64 * D / 16);
    const int row = u / (D / 16), phys = u % (D / 16);
    return swizzled_offset(row, phys, f8_swizzle<D>(row), D);
}

// Key tiles of a workgroup of query rows [q_first, q_last] (q_last < L): all
// tiles that may hold a visible key, cut into SPLIT equal consecutive shares;
// share grp is [t_begin, t_end), and every share runs t_stop - t_begin steps.
struct TileRange {
    int t_begin, t_end, t_stop;
};
template <bool CAUSAL, bool WINDOW, int SPLIT>
__host__ __device__ __forceinline__ TileRange key_tiles(int q_first, int q_last, int L, int window, int block_k,
                                                        int grp)
{
    int kv_begin = 0, kv_end = L;
    if (WINDOW) kv_begin = q_first - window > 0 ? q_first - window : 0;
    if (CAUSAL) kv_end = q_last + 1;
    else if (WINDOW) kv_end = q_last + window + 1 < L ? q_last + window + 1 : L;
    const int t_first = kv_begin / block_k;
    const int t_last = (kv_end + block_k - 1) / block_k;  // one past
    TileRange r;
    if (SPLIT > 1) {
        const int chunk = (t_last - t_first + SPLIT - 1) / SPLIT;
        r.t_begin = t_first + grp * chunk;
        r.t_end = t_last < r.t_begin + chunk ? t_last : r.t_begin + chunk;
        r.t_stop = r.t_begin + chunk;
    } else {
        r.t_begin = t_first;
        r.t_end = t_last;
        r.t_stop = t_last;
    }
    return r;
}

// How a wave with query rows [qa, qb] (qb < L) treats the key tile starting
// at key j0: 0 = skip (no visible key), 1 = full (every key visible from every
// row: no mask), 2 = edge (masked).
template <bool CAUSAL, bool WINDOW>
__host__ __device__ __forceinline__ int tile_class(int j0, int qa, int qb, int L, int window, int block_k)
{
    const int j_last = j0 + block_k - 1;
    bool skip = false;
    if (CAUSAL) skip = skip || j0 > qb;
    if (WINDOW) {
        skip = skip || j_last < qa - window;
        if (!CAUSAL) skip = skip || j0 > qb + window;
    }
    if (skip) return 0;
    bool full = j_last < L;
    if (CAUSAL) full = full && j_last <= qa;
    if (WINDOW) {
        full = full && j0 >= qb - window;
        if (!CAUSAL) full = full && j_last <= qa + window;
    }
    return full ? 1 : 2;
}

// Merge of the key-range groups' partial results (forward, SPLIT > 1): each
// wave of a group s > 0 writes its lanes' O^T (16 per d block), reference max
// and sum, kPart floats per lane, into a slot of one of the two idle stage
// buffers (each SPLIT * 2 * kTileBytes bytes); kBatch waves per round.
template <int D, int NW, int SPLIT>
struct MergeLayout {
    static constexpr int kPart = 16 * (D / 32) + 2;                  // floats per lane
    static constexpr int kSlotBytes = 64 * kPart * 4;                 // one wave's slot
    static constexpr int kBufferBytes = SPLIT * 2 * 64 * 2 * D;       // one stage buffer
    static constexpr int kPerBuffer = kBufferBytes / kSlotBytes;      // slots per buffer
    static constexpr int kBatch = 2 * kPerBuffer < NW ? 2 * kPerBuffer : NW;  // waves per round
    // float offset of slot i (i < kBatch) within its buffer, which is the
    // first buffer when i < kPerBuffer and the second otherwise
    __host__ __device__ static constexpr int slot_float_offset(int i) { return (i % kPerBuffer) * 64 * kPart; }
};

// ---- paged decode: the list of key tiles that the partial kernel splits into
// equal runs of P = max(ceil(total / W), kMinTiles) tiles over W waves.
constexpr int kDecTile = 32;     // keys per tile
constexpr int kMaxWaves = 4096;  // most waves of the partial kernel (bounds the workspace)
constexpr int kMinTiles = 8;     // fewest tiles per wave

// Row blocks (of up to 32 query rows of one K/V head), segments per sequence,
// rows per result slot, and the most waves a call of this shape can use (one
// wave per kMinTiles tiles of the longest possible list, at most kMaxWaves);
// each wave writes at most one result per segment it touches, and the runs
// are consecutive, so waves_cap + B * nseg slots hold them all.  Host side.
struct DecodeShape {
    int64_t rows, n_rowblk, nseg, rslot, waves_cap, n_slots;
};
inline DecodeShape decode_shape(int64_t B, int64_t H, int64_t H_kv, int64_t Lq, int64_t max_len)
{
    DecodeShape s;
    s.rows = H / H_kv * Lq;
    s.n_rowblk = (s.rows + 31) / 32;
    s.nseg = H_kv * s.n_rowblk;
    s.rslot = s.rows < 32 ? s.rows : 32;
    const int64_t tiles = B * s.nseg * ((max_len + kDecTile - 1) / kDecTile);
    const int64_t cap = (tiles + kMinTiles - 1) / kMinTiles;
    s.waves_cap = cap < 1 ? 1 : (cap > kMaxWaves ? kMaxWaves : cap);
    s.n_slots = s.waves_cap + B * s.nseg;
    return s;
}

// A sequence of n tokens (n already clamped) whose last Lq tokens are the
// query rows: the first key one of them sees, and the 32-key tiles
// [t_lo, t_hi) holding every such key (none when n = 0).
__host__ __device__ __forceinline__ int decode_first_key(int n, int Lq, int window)
{
    return window >= 0 && n - Lq - window > 0 ? n - Lq - window : 0;
}
struct DecSeqTiles {
    int t_lo, t_hi;
};
__host__ __device__ __forceinline__ DecSeqTiles decode_seq_tiles(int n, int Lq, int window)
{
    DecSeqTiles st;
    st.t_lo = decode_first_key(n, Lq, window) / kDecTile;
    st.t_hi = (n + kDecTile - 1) / kDecTile;
    return st;
}

// A position in the tile list: sequence b (n tokens, tiles [t_lo, t_hi)),
// K/V head g, row block rb, tile t.  The list runs over t, then rb, then g,
// then the sequences that have tiles.
struct DecCursor {
    int b, g, rb, t, t_lo, t_hi, n;
};

// The cursor at tile `off` (< tiles * H_kv * n_rowblk) of sequence b's part
// of the list.
__host__ __device__ __forceinline__ DecCursor decode_cursor_at(int b, int n, DecSeqTiles st, int64_t off,
                                                               int n_rowblk)
{
    DecCursor c;
    c.b = b;
    c.n = n;
    c.t_lo = st.t_lo;
    c.t_hi = st.t_hi;
    const int tiles = st.t_hi - st.t_lo;
    const int seg = (int)(off / tiles);
    c.t = st.t_lo + (int)(off % tiles);
    c.g = seg / n_rowblk;
    c.rb = seg % n_rowblk;
    return c;
}

// The tile after c; len(b) is sequence b's clamped length.  Sequences without
// tiles are skipped; past the last tile of the list the cursor stays inside
// the last sequence (a valid tile, not part of any run).
template <typename LenFn>
__host__ __device__ __forceinline__ DecCursor decode_next_tile(DecCursor c, int B, int H_kv, int n_rowblk, int Lq,
                                                               int window, LenFn len)
{
    if (++c.t < c.t_hi) return c;
    c.t = c.t_lo;
    if (++c.rb < n_rowblk) return c;
    c.rb = 0;
    if (++c.g < H_kv) return c;
    c.g = 0;
    while (c.b + 1 < B) {
        ++c.b;
        c.n = len(c.b);
        const DecSeqTiles st = decode_seq_tiles(c.n, Lq, window);
        c.t_lo = st.t_lo;
        c.t_hi = st.t_hi;
        if (c.t_hi > c.t_lo) break;
    }
    c.t = c.t_lo;
    return c;
}

// The waves whose runs of P consecutive tiles meet a segment of `tiles`
// tiles (> 0) that starts at list position f_seg: w_lo .. w_hi.
struct DecWaves {
    int64_t lo, hi;
};
__host__ __device__ __forceinline__ DecWaves decode_segment_waves(int64_t f_seg, int64_t tiles, int64_t P)
{
    DecWaves w;
    w.lo = f_seg / P;
    w.hi = (f_seg + tiles - 1) / P;
    return w;
}

// Do the byte ranges [a, a+na) and [b, b+nb) overlap?
inline bool overlaps(const void *a, size_t na, const void *b, size_t nb)
{
    const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
    return na && nb && pa < pb + nb && pb < pa + na;
}

}  // namespace
