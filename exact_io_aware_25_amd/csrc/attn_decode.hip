// attn_decode.hip -- attention of a few new queries over a paged KV cache
// (decode) for MI355X (CDNA4, gfx950).
//
// Each generated token reads the whole KV cache of its sequence, so decode
// is bound by HBM bandwidth («Что такое memory-efficient attention для long
// context на 8x H100?», section 1); the cache lives in fixed-size blocks
// reached through a page table (same page, section 3, PagedAttention).  The
// result is the forward definition for the last Lq positions of each
// sequence: query i of sequence b sits at p = n_b - Lq + i and sees keys
// j <= p (and p - j <= window).
//
// Two kernels:
//   1. partial (split-K over an even partition): the work is the list of
//      32-key tiles of every segment -- (sequence, K/V head, block of up to
//      32 query rows that read that head: the group's heads times Lq) --
//      laid end to end.  Each of W waves takes an equal run of P consecutive
//      tiles; W is as many waves as the device holds at once, so all of them
//      start at the launch and finish together (no later rounds of waves
//      behind a tail of unequal chunks).  A run may start or end inside a
//      segment and cross into the next ones; the wave writes one partial
//      result (max, sum, unnormalised O) per segment it touches.  Each wave
//      works alone -- its own LDS region, no barriers.  Per tile: the K rows
//      go straight from the cache into the A-operand registers of S^T = K Q^T
//      (16 contiguous bytes per lane), the V tile goes into LDS by
//      direct-to-LDS loads (for the transposing read of the second product),
//      both one tile ahead and the page-table entries two tiles ahead; the
//      online softmax is per lane.  When every V row is read by one wave only
//      (one row block per K/V head) and the waves have long runs, the V loads
//      carry the non-temporal hint: each one covers whole 128-byte lines, and
//      streaming them past L2 raised the read rate by about a tenth.  The K
//      loads keep the default policy: each covers 32 bytes of 32 rows, and
//      the tile's other loads need those lines to stay in L2.
//   2. merge: one workgroup per query row combines the partial results of the
//      waves that touched its segment exactly (the same rescale the online
//      softmax uses) and writes O and lse.
// The products run on the 32x32x16 MFMA although at most Lq*H/H_kv of the
// 32 query columns are live: the kernel is bound by bytes, not FLOPs.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "attn.h"
#include "attn_common.h"

namespace {

// One 16-byte direct-to-LDS load per lane (as copy_to_lds16), with the
// non-temporal cache policy (bit 1 of the instruction's cache-policy field)
// when STREAM is set.
template <bool STREAM>
__device__ __forceinline__ void copy_to_lds16_policy(__amdgpu_buffer_rsrc_t src, void *lds_dst, int src_offset)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (__attribute__((address_space(3))) void *)lds_dst, 16,
                                             src_offset, 0, 0, STREAM ? 2 : 0);
}

constexpr int kDecWaves = 4;     // independent waves per workgroup (tiles: kDecTile keys)
constexpr int kMaxDevices = 64;
constexpr float kLn2 = 0.69314718055994531f;

struct DecParams {
    const void *q, *kc, *vc;
    const int *table, *lens;
    void *o;
    float *lse;
    int64_t *hdr;  // workspace head: [B + 1] first tile of each sequence in the list (the last = total), then P
    float *part;   // [n_slots][rslot][D] unnormalised O, then [n_slots][rslot][2] (m, l)
    int B, H, H_kv, Lq, group, rows;  // rows = group * Lq: query rows per K/V head
    int d;                            // head size (host side: picks the kernel instance)
    int bs, bs_shift, max_blocks, num_blocks, max_len, window;
    int n_rowblk, nseg, rslot;  // row blocks per K/V head; segments per sequence (H_kv * n_rowblk); rows per slot
    int n_waves, n_slots;       // waves of the partial kernel; result slots (most waves + B * nseg)
    float scale_log2;
};

// Read through the constant address space: the lengths and the page table
// are not written while the kernels run, so a wave-uniform read of them can be
// a scalar load, which the wave's waits for its vector loads (vmcnt) do not
// include.
__device__ __forceinline__ int load_invariant(const int *ptr)
{
    return *(const __attribute__((address_space(4))) int *)ptr;
}

__device__ __forceinline__ int seq_len(const DecParams &p, int b)
{
    return min(max(load_invariant(p.lens + b), 0), p.max_len);
}

// Page-table entry for key j of sequence b (the logical block number is
// clamped), and the physical block it names (the entry is clamped too, so a
// bad table reads a wrong block, never out of bounds).
__device__ __forceinline__ int table_entry(const DecParams &p, int b, int j)
{
    const int lb = min(j >> p.bs_shift, p.max_blocks - 1);
    return load_invariant(p.table + (int64_t)b * p.max_blocks + lb);
}

__device__ __forceinline__ int64_t physical_block(const DecParams &p, int entry)
{
    return min(max(entry, 0), p.num_blocks - 1);
}

// Tiles of sequence b over all its segments.
__device__ __forceinline__ int64_t sequence_span(const DecParams &p, int b)
{
    const DecSeqTiles st = decode_seq_tiles(seq_len(p, b), p.Lq, p.window);
    return (int64_t)(st.t_hi - st.t_lo) * p.nseg;
}

// The tile after c (see decode_next_tile).
__device__ __forceinline__ DecCursor next_tile(const DecParams &p, DecCursor c)
{
    return decode_next_tile(c, p.B, p.H_kv, p.n_rowblk, p.Lq, p.window, [&](int b) { return seq_len(p, b); });
}

__device__ __forceinline__ int64_t uniform64(int64_t x)
{
    const uint64_t u = (uint64_t)x;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// s_waitcnt vmcnt(N): at most N of this wave's vector memory operations are
// still outstanding (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt has 6 bits");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int64_t wave_prefix_sum(int64_t x, int lane)
{
#pragma unroll
    for (int off = 1; off < 64; off *= 2) {
        const long long y = __shfl_up((long long)x, off);
        if (lane >= off) x += y;
    }
    return x;
}

// ---------------------------------------------------------------- 1. partial
template <typename T, int D, bool STREAM>
__global__ __launch_bounds__(64 * kDecWaves) void attn_decode_partial_kernel(DecParams p)
{
    typedef typename Vec8<T>::type vec8;
    constexpr int kRowBytes = 2 * D;
    constexpr int kTileBytes = kDecTile * kRowBytes;
    constexpr int kUnits = D / 8;
    constexpr int kHalfCopies = 16 * kUnits / 64;  // copy instructions per 16-row half tile
    constexpr int kDSteps = D / 16;
    constexpr int kDBlocks = D / 32;

    // per wave: two stages of one V tile
    __shared__ __attribute__((aligned(16))) char lds_a[kDecWaves][kTileBytes];
    __shared__ __attribute__((aligned(16))) char lds_b[kDecWaves][kTileBytes];

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    const int lane = threadIdx.x % 64;
    const int l32 = lane % 32;
    const int hi = lane / 32;
    const int w = blockIdx.x * kDecWaves + wave;  // this wave's run of the tile list
    if (w >= p.n_waves) return;

    // ---- the tile list: each sequence's first tile in it, the total, the run length P
    int64_t total = 0;
    int64_t span0 = 0, incl0 = 0;  // sequences 0..63 (kept for the search below)
    for (int b0 = 0; b0 < p.B; b0 += 64) {
        const int b = b0 + lane;
        const int64_t span = b < p.B ? sequence_span(p, b) : 0;
        const int64_t incl = wave_prefix_sum(span, lane);
        if (b0 == 0) {
            span0 = span;
            incl0 = incl;
        }
        if (w == 0 && b < p.B) p.hdr[b] = total + incl - span;
        total += uniform64(__shfl((long long)incl, 63));
    }
    const int64_t P = max((total + p.n_waves - 1) / p.n_waves, (int64_t)kMinTiles);
    if (w == 0 && lane == 0) {
        p.hdr[p.B] = total;
        p.hdr[p.B + 1] = P;
    }
    const int64_t f_begin = (int64_t)w * P;
    const int64_t f_end = min(total, f_begin + P);
    if (f_begin >= f_end) return;

    // ---- the cursor at f_begin: the sequence whose tiles hold it, then segment and tile
    DecCursor c0;
    {
        int64_t run = 0;
        for (int b0 = 0; b0 < p.B; b0 += 64) {
            const int b = b0 + lane;
            const int64_t span = b0 == 0 ? span0 : b < p.B ? sequence_span(p, b) : 0;
            const int64_t incl = b0 == 0 ? incl0 : wave_prefix_sum(span, lane);
            const uint64_t found = __ballot(b < p.B && run + incl > f_begin);
            if (found) {
                const int l = __builtin_ctzll(found);
                const int64_t off = f_begin - run - uniform64(__shfl((long long)(incl - span), l));
                const int n = seq_len(p, b0 + l);  // the sequence holds f_begin, so it has tiles
                c0 = decode_cursor_at(b0 + l, n, decode_seq_tiles(n, p.Lq, p.window), off, p.n_rowblk);
                break;
            }
            run += uniform64(__shfl((long long)incl, 63));
        }
    }

    const T *kc = static_cast<const T *>(p.kc);
    const T *vc = static_cast<const T *>(p.vc);
    const int krow = k_row_for_lane(l32);  // A-operand row order (bits 2 and 3 swapped)

    // transposing-read offsets of the V tile (rows 8hi + a and +4, as in the forward)
    int voff[kDBlocks];
#pragma unroll
    for (int db = 0; db < kDBlocks; ++db) voff[db] = v_tr_offset<D, kSwzV>(lane, db);
    int ld_v[kHalfCopies];  // source offsets within a 16-row half tile (swizzled placement)
#pragma unroll
    for (int cc = 0; cc < kHalfCopies; ++cc) ld_v[cc] = copy_src_offset<D, kSwzV>(cc * 64 + lane);

    // The page-table entries of the two 16-key halves of a tile (wave-uniform
    // scalar loads).  They are fetched two tiles ahead and clamped only where
    // used, so a tile's data loads never wait on a page-table load.
    struct Pages { int lo, hi; };
    auto pages_of = [&](const DecCursor &c) {
        Pages pg;
        pg.lo = table_entry(p, c.b, c.t * kDecTile);
        pg.hi = table_entry(p, c.b, c.t * kDecTile + 16);
        return pg;
    };
    // K fragments of a tile into registers; its V tile into this wave's stage
    auto load_k = [&](const DecCursor &c, Pages pg, vec8 (&kf)[kDSteps]) {
        const int j = c.t * kDecTile + krow;  // krow < 16 exactly when l32 < 16
        const int64_t page = physical_block(p, l32 < 16 ? pg.lo : pg.hi);
        const T *row = kc + ((page * p.H_kv + c.g) * p.bs + (j & (p.bs - 1))) * D;
#pragma unroll
        for (int s = 0; s < kDSteps; ++s) kf[s] = *reinterpret_cast<const vec8 *>(row + 16 * s + 8 * hi);
    };
    auto copy_v = [&](const DecCursor &c, Pages pg, char *stage) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const int j0 = c.t * kDecTile + 16 * hf;
            const int valid = min(max(c.n - j0, 0), 16);  // rows past n arrive as zeros
            const int64_t page = physical_block(p, __builtin_amdgcn_readfirstlane(hf ? pg.hi : pg.lo));
            const T *base = vc + ((page * p.H_kv + c.g) * p.bs + (j0 & (p.bs - 1))) * D;
            const __amdgpu_buffer_rsrc_t rv =
                __builtin_amdgcn_make_buffer_rsrc((void *)base, 0, valid * kRowBytes, 0x00020000);
#pragma unroll
            for (int cc = 0; cc < kHalfCopies; ++cc)
                copy_to_lds16_policy<STREAM>(rv, stage + hf * 16 * kRowBytes + cc * 1024, ld_v[cc]);
        }
    };

    // ---- the segment being accumulated and this lane's query row in it
    int seg_b = -1, seg_g = 0, seg_rb = 0;  // wave-uniform
    int k_begin = 0, k_end = 0, min_pos = 0, max_pos = 0;
    bool row_live = false;
    int pos = 0;
    vec8 qf[kDSteps];
    f32x16 acc_o[kDBlocks];
    float m_run = -INFINITY;  // running max of scale*log2(e)*s
    float l_run = 0.f;        // running sum of weights, this lane half's keys

    // the segment's partial result into slot w + (its index among all segments)
    auto flush = [&]() {
        const float l_tot = half_swap_sum(l_run);
        if (!row_live) return;
        const int64_t slot = (int64_t)w + ((int64_t)seg_b * p.H_kv + seg_g) * p.n_rowblk + seg_rb;
        float *po = p.part + (slot * p.rslot + l32) * D;
#pragma unroll
        for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                // register 4a+cc of block db holds d = 32db + 8a + 4hi + cc
                const float4 v4 = {acc_o[db][4 * a], acc_o[db][4 * a + 1], acc_o[db][4 * a + 2], acc_o[db][4 * a + 3]};
                *reinterpret_cast<float4 *>(po + 32 * db + 8 * a + 4 * hi) = v4;
            }
        if (hi == 0) {
            float *pml = p.part + (int64_t)p.n_slots * p.rslot * D + 2 * (slot * p.rslot + l32);
            pml[0] = m_run;
            pml[1] = l_tot;
        }
    };
    // start accumulating the segment of cursor c
    auto begin_segment = [&](const DecCursor &c) {
        seg_b = c.b;
        seg_g = c.g;
        seg_rb = c.rb;
        const int r = c.rb * 32 + l32;  // row (head in group, new-token index) of this lane
        row_live = r < p.rows;
        const int hh = row_live ? r / p.Lq : 0;
        const int qi = row_live ? r % p.Lq : 0;
        const int h = c.g * p.group + hh;
        pos = c.n - p.Lq + qi;  // its position (rows with pos < 0 see no key)
        k_begin = decode_first_key(c.n, p.Lq, p.window);
        k_end = c.n;
        max_pos = c.n - 1;
        min_pos = c.n - p.Lq;
        const T *qrow = static_cast<const T *>(p.q) + (((int64_t)c.b * p.H + h) * p.Lq + qi) * D;
#pragma unroll
        for (int s = 0; s < kDSteps; ++s)
            qf[s] = row_live ? *reinterpret_cast<const vec8 *>(qrow + 16 * s + 8 * hi) : vec8{};
        // Wait for them here (and for every load before them), and hide their
        // origin from the compiler: the products of every tile then wait only
        // for that tile's own loads, not for a query load on some other path.
        wait_vmcnt<0>();
#pragma unroll
        for (int s = 0; s < kDSteps; ++s) asm volatile("" : "+v"(qf[s]));
#pragma unroll
        for (int i = 0; i < kDBlocks; ++i) acc_o[i] = f32x16{};
        m_run = -INFINITY;
        l_run = 0.f;
    };

    auto process = [&](const DecCursor &c, const vec8 (&kf)[kDSteps], const char *tv) {
        if (c.b != seg_b || c.g != seg_g || c.rb != seg_rb) {
            if (seg_b >= 0) flush();
            begin_segment(c);
        }
        const int j0 = c.t * kDecTile;
        // S^T = K Q^T: register r holds key j0 + 16(r/8) + 8hi + r%8 of this lane's row
        f32x16 s = f32x16{};
#pragma unroll
        for (int ds = 0; ds < kDSteps; ++ds) s = mfma32(kf[ds], qf[ds], s);
        bool full = j0 + kDecTile - 1 <= min_pos && j0 >= k_begin && j0 + kDecTile <= k_end;
        if (p.window >= 0) full = full && max_pos - j0 <= p.window;
        if (!full) {
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) {
                const int j = j0 + 16 * (rr / 8) + 8 * hi + (rr % 8);
                bool ok = row_live && j >= k_begin && j < k_end && j <= pos;
                if (p.window >= 0) ok = ok && pos - j <= p.window;
                if (!ok) s[rr] = -INFINITY;
            }
        }
        float mt = -INFINITY;
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) mt = fmaxf(mt, s[rr]);
        const float m_new = fmaxf(m_run, half_swap_max(mt) * p.scale_log2);
        if (__any(m_new > m_run)) {
            const float alpha = m_new > m_run ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
            l_run *= alpha;
#pragma unroll
            for (int i = 0; i < kDBlocks; ++i) acc_o[i] *= alpha;
            m_run = m_new;
        }
        const float neg_m = m_run == -INFINITY ? 0.f : -m_run;
        vec8 pv[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            f32x8 pf;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                pf[e] = __builtin_amdgcn_exp2f(fmaf(s[8 * ks + e], p.scale_log2, neg_m));
                l_run += pf[e];
            }
            pv[ks] = __builtin_convertvector(pf, vec8);
        }
        // O^T += V^T P^T over the two 16-key slices
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int db = 0; db < kDBlocks; ++db) {
                const char *base = tv + 16 * ks * kRowBytes + voff[db];
                const s16x4 lo4 = lds_read_tr16(base);
                const s16x4 hi4 = lds_read_tr16(base + 4 * kRowBytes);
                const vec8 vf = __builtin_bit_cast(vec8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
                acc_o[db] = mfma32(vf, pv[ks], acc_o[db]);
            }
    };

    // Two tiles in flight: the loads of tile f+1 are issued before the wave
    // waits for tile f, and overlap its products.  The wave waits for its own
    // loads only (vmcnt, in issue order: all but the kTileLoads newest); before
    // a copy reuses a stage, its reads of that stage have completed (lgkmcnt).
    // Every step issues one tile's loads whether or not a tile is left (past
    // the end of the run it loads the tile just processed again: its K rows
    // are still in L2, its V rows too unless they were streamed), so every
    // path through the loop has the same loads in flight and the compiler's
    // own waits stay as loose as the ones here.
    // At the top of each step c0 is tile f (in stage a), c1 tile f+1, c2 tile
    // f+2, pg0 and pg1 the page entries of c0 and c1.
    constexpr int kTileLoads = kDSteps + 2 * kHalfCopies;  // vector memory instructions per tile
    char *stage_a = lds_a[wave];
    char *stage_b = lds_b[wave];
    vec8 kf_a[kDSteps], kf_b[kDSteps];
    DecCursor c1 = next_tile(p, c0);  // past the end of the run: a tile inside the list, not processed
    DecCursor c2 = next_tile(p, c1);
    Pages pg0 = pages_of(c0);
    Pages pg1 = pages_of(c1);
    load_k(c0, pg0, kf_a);
    copy_v(c0, pg0, stage_a);
    begin_segment(c0);  // its query rows load while the first tile is in flight
    for (int64_t f = f_begin; f < f_end; f += 2) {
        const bool has1 = f + 1 < f_end;
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        load_k(has1 ? c1 : c0, has1 ? pg1 : pg0, kf_b);
        copy_v(has1 ? c1 : c0, has1 ? pg1 : pg0, stage_b);
        const Pages pg2 = pages_of(c2);
        wait_vmcnt<kTileLoads>();
        process(c0, kf_a, stage_a);
        if (!has1) break;

        const bool has2 = f + 2 < f_end;
        const DecCursor c3 = next_tile(p, c2);
        __builtin_amdgcn_s_waitcnt(0xC07F);
        load_k(has2 ? c2 : c1, has2 ? pg2 : pg1, kf_a);
        copy_v(has2 ? c2 : c1, has2 ? pg2 : pg1, stage_a);
        const Pages pg3 = pages_of(c3);
        wait_vmcnt<kTileLoads>();
        process(c1, kf_b, stage_b);
        c0 = c2;
        pg0 = pg2;
        c1 = c3;
        pg1 = pg3;
        c2 = next_tile(p, c3);
    }
    wait_vmcnt<0>();  // no copy into LDS outlives the wave
    flush();
}

// ---------------------------------------------------------------- 2. merge
// One workgroup of NW waves per query row.  The waves of the partial kernel
// whose runs met the row's segment are w_lo..w_hi (the runs are consecutive
// and equal).  The merge is the online softmax's rescale over their results
// (max m_w, sum l_w, unnormalised O_w): in one pass, each lane keeps a running
// state, the states meet across lanes and then across waves in LDS (in wave
// order), each rescaled by 2^(m - M) to the largest maximum M.  A row with few
// results (many short segments) gets 4 waves, each taking one result per
// load; a row with many (few long segments) 16 waves, each taking several
// results per load.
template <typename T, int D, int NW>
__global__ __launch_bounds__(64 * NW) void attn_decode_merge_kernel(DecParams p)
{
    __shared__ float red_m[NW];
    __shared__ float red_o[NW][D + 1];
    const int wave = threadIdx.x / 64;
    const int lane = threadIdx.x % 64;
    const int row = blockIdx.x;  // (b*H + h)*Lq + i (B*H*Lq < 2^31)
    const int b = row / (p.H * p.Lq);
    const int h = row / p.Lq % p.H;
    const int i = row % p.Lq;
    const int g = h / p.group;
    const int r = (h % p.group) * p.Lq + i;  // row within the K/V head's rows
    const int rb = r / 32;
    const int seg = g * p.n_rowblk + rb;      // segment within the sequence
    const int64_t seq_first = p.hdr[b];
    const int64_t tiles = (p.hdr[b + 1] - seq_first) / p.nseg;  // tiles of each segment of sequence b
    const int64_t P = p.hdr[p.B + 1];
    DecWaves ws = {0, -1};  // none when the sequence has no tile
    if (tiles > 0) ws = decode_segment_waves(seq_first + seg * tiles, tiles, P);
    const int64_t w_lo = ws.lo, w_hi = ws.hi;
    const int64_t slot0 = (int64_t)b * p.nseg + seg;  // wave w's result for this segment: slot w + slot0
    const int64_t rs = r % 32;
    const float *pml = p.part + (int64_t)p.n_slots * p.rslot * D;

    // One pass over the results: each lane keeps a running (max, sum, O) and
    // rescales it when a larger maximum arrives, as the online softmax does;
    // the running states then meet across lanes and waves the same way.
    float m = -INFINITY, l = 0.f;
    if constexpr (NW == 4) {
        // wave v takes the results w_lo + v, + 4, ... (one per load, lanes over d)
        constexpr int kPer = D / 64;
        float acc[kPer];
#pragma unroll
        for (int e = 0; e < kPer; ++e) acc[e] = 0.f;
#pragma unroll 4
        for (int64_t w = w_lo + wave; w <= w_hi; w += NW) {
            const int64_t sr = (w + slot0) * p.rslot + rs;
            const float mc = pml[2 * sr];
            const float lc = pml[2 * sr + 1];
            float o[kPer];
#pragma unroll
            for (int e = 0; e < kPer; ++e) o[e] = p.part[sr * D + e * 64 + lane];
            // no branch, so the loads of the unrolled iterations issue together
            const float mn = fmaxf(m, mc);
            const float alpha = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mn);
            const float wt = mc == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mc - mn);
            l = alpha * l + wt * lc;
#pragma unroll
            for (int e = 0; e < kPer; ++e) acc[e] = alpha * acc[e] + wt * o[e];
            m = mn;
        }
#pragma unroll
        for (int e = 0; e < kPer; ++e) red_o[wave][e * 64 + lane] = acc[e];
    } else {
        // lanes over (result, 4 consecutive d): a wave reads 64 / (D / 4)
        // results per load, 16 bytes per lane, and combines them up the lane
        // bits above d
        constexpr int kLanesPerPart = D / 4;
        constexpr int kPartsPerWave = 64 / kLanesPerPart;
        const int sub = lane / kLanesPerPart;
        const int d4 = lane % kLanesPerPart;
        float4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
        for (int64_t w = w_lo + wave * kPartsPerWave + sub; w <= w_hi; w += NW * kPartsPerWave) {
            const int64_t sr = (w + slot0) * p.rslot + rs;
            const float mc = pml[2 * sr];
            const float lc = pml[2 * sr + 1];
            const float4 v = *reinterpret_cast<const float4 *>(p.part + sr * D + 4 * d4);
            const float mn = fmaxf(m, mc);
            const float alpha = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mn);
            const float wt = mc == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mc - mn);
            l = alpha * l + wt * lc;
            acc.x = alpha * acc.x + wt * v.x;
            acc.y = alpha * acc.y + wt * v.y;
            acc.z = alpha * acc.z + wt * v.z;
            acc.w = alpha * acc.w + wt * v.w;
            m = mn;
        }
#pragma unroll
        for (int off = kLanesPerPart; off < 64; off *= 2) {
            const float mo = __shfl_xor(m, off);
            const float lo = __shfl_xor(l, off);
            const float4 ao = {__shfl_xor(acc.x, off), __shfl_xor(acc.y, off), __shfl_xor(acc.z, off),
                               __shfl_xor(acc.w, off)};
            const float mn = fmaxf(m, mo);
            const float a = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mn);
            const float c = mo == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mo - mn);
            l = a * l + c * lo;
            acc.x = a * acc.x + c * ao.x;
            acc.y = a * acc.y + c * ao.y;
            acc.z = a * acc.z + c * ao.z;
            acc.w = a * acc.w + c * ao.w;
            m = mn;
        }
        if (lane < kLanesPerPart) {
            red_o[wave][4 * d4] = acc.x;
            red_o[wave][4 * d4 + 1] = acc.y;
            red_o[wave][4 * d4 + 2] = acc.z;
            red_o[wave][4 * d4 + 3] = acc.w;
        }
    }
    if (lane == 0) {
        red_m[wave] = m;
        red_o[wave][D] = l;
    }
    __syncthreads();
    if (wave != 0) return;
    float mx = red_m[0];
#pragma unroll
    for (int v = 1; v < NW; ++v) mx = fmaxf(mx, red_m[v]);
    float sc[NW];  // each wave's rescale to the largest maximum
    l = 0.f;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
        sc[v] = red_m[v] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(red_m[v] - mx);
        l += sc[v] * red_o[v][D];
    }
    m = mx;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    T *orow = static_cast<T *>(p.o) + (int64_t)row * D;
#pragma unroll
    for (int e = 0; e < D / 64; ++e) {
        const int d = e * 64 + lane;
        float o = 0.f;
#pragma unroll
        for (int v = 0; v < NW; ++v) o += sc[v] * red_o[v][d];
        orow[d] = (T)(o * inv);
    }
    if (lane == 0) p.lse[row] = l > 0.f ? (m + __log2f(l)) * kLn2 : -INFINITY;
}

// ------------------------------------------------------------------ host side

size_t decode_hdr_bytes(int64_t B)
{
    return (size_t)((B + 2) * 8 + 15) / 16 * 16;
}

size_t decode_workspace_bytes(int64_t B, int64_t H, int64_t H_kv, int64_t Lq, int d, int64_t max_len)
{
    const DecodeShape s = decode_shape(B, H, H_kv, Lq, max_len);
    const size_t part = (size_t)(s.n_slots * s.rslot * (d + 2) * (int64_t)sizeof(float));
    return (decode_hdr_bytes(B) + part + 15) / 16 * 16;
}

// Waves of the partial kernel the current device holds at once (queried
// once per device and kernel instance); 0 when the query fails.
std::mutex g_capacity_mutex;

template <typename T, int D, bool STREAM>
int resident_waves()
{
    static int cached[kMaxDevices];
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    std::lock_guard<std::mutex> lock(g_capacity_mutex);
    if (!cached[dev]) {
        int cus = 0, blocks = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &blocks, reinterpret_cast<const void *>(&attn_decode_partial_kernel<T, D, STREAM>), 64 * kDecWaves,
                0) !=
                hipSuccess ||
            cus < 1 || blocks < 1)
            return 0;
        cached[dev] = cus * blocks * kDecWaves;
    }
    return cached[dev];
}

// Whether the partial kernel's V loads stream past L2: only when each V row
// has one reader (a single row block per K/V head) and the waves' runs are
// long (at least kStreamTiles tiles each by the upper bound on the tile
// list); short runs are bound by latency, and the hint cost them about 2 %.
constexpr int64_t kStreamTiles = 16;
inline bool decode_streams_v(const DecParams &p)
{
    if (p.n_rowblk != 1) return false;
    const int64_t keys = p.window >= 0 ? std::min<int64_t>(p.max_len, (int64_t)p.window + p.Lq) : p.max_len;
    const int64_t tiles = (int64_t)p.B * p.nseg * ((keys + kDecTile - 1) / kDecTile + 1);
    return tiles >= kStreamTiles * p.n_waves;
}

template <typename T, int D, bool STREAM>
hipError_t launch_partial(DecParams &p, hipStream_t stream)
{
    const int resident = resident_waves<T, D, STREAM>();
    if (resident < 1) return hipErrorInvalidDevice;
    p.n_waves = std::min(p.n_waves, resident);  // n_slots keeps the workspace layout of the cap
    void *kargs[] = {&p};
    const int grid1 = (p.n_waves + kDecWaves - 1) / kDecWaves;
    return hipLaunchKernel(reinterpret_cast<const void *>(&attn_decode_partial_kernel<T, D, STREAM>),
                           dim3((unsigned)grid1), dim3(64 * kDecWaves), kargs, 0, stream);
}

template <typename T, int D>
hipError_t launch_decode(DecParams p, hipStream_t stream)
{
    // decided on the resident wave count, which both instances share (same
    // registers and LDS)
    const int resident = resident_waves<T, D, false>();
    if (resident < 1) return hipErrorInvalidDevice;
    DecParams probe = p;
    probe.n_waves = std::min(p.n_waves, resident);
    hipError_t err = decode_streams_v(probe) ? launch_partial<T, D, true>(p, stream)
                                             : launch_partial<T, D, false>(p, stream);
    if (err != hipSuccess) return err;
    void *kargs[] = {&p};
    // a row has at most about n_waves / (B * nseg) + 1 partial results (fewer
    // when the sequences are shorter than max_seq_len)
    const int64_t rows_total = (int64_t)p.B * p.H * p.Lq;
    if (p.n_waves >= (int64_t)128 * p.B * p.nseg)
        return hipLaunchKernel(reinterpret_cast<const void *>(&attn_decode_merge_kernel<T, D, 16>),
                               dim3((unsigned)rows_total), dim3(64 * 16), kargs, 0, stream);
    return hipLaunchKernel(reinterpret_cast<const void *>(&attn_decode_merge_kernel<T, D, 4>),
                           dim3((unsigned)rows_total), dim3(64 * 4), kargs, 0, stream);
}
// Checks every argument but the workspace and fills the launch parameters
// (all but p->part); *bytes_ws receives the workspace the call needs.  Makes
// no HIP call.  ATTN_OK with p->B == 0 is an empty problem.
template <typename T>
int decode_plan(const void *q, const void *k_cache, const void *v_cache, const int *block_table,
                const int *seq_lens, void *out, float *lse, int B, int H, int H_kv, int Lq, int d, int block_size,
                int max_blocks, int num_blocks, int max_seq_len, int window, float scale, DecParams *pp,
                size_t *bytes_ws_out)
{
    DecParams &p = *pp;
    p.B = 0;
    if (B < 0 || H < 1 || H_kv < 1 || H % H_kv != 0 || Lq < 1 || max_blocks < 1 || num_blocks < 1 ||
        max_seq_len < 1)
        return ATTN_ERR_SHAPE;
    if (block_size < 16 || block_size > 4096 || (block_size & (block_size - 1)) ||
        (int64_t)max_seq_len > (int64_t)max_blocks * block_size)
        return ATTN_ERR_SHAPE;
    if (d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
    if (window < -1) return ATTN_ERR_WINDOW;
    if (std::isinf(scale)) return ATTN_ERR_SCALE;
    if (B == 0) return ATTN_OK;
    if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !out || !lse)
        return ATTN_ERR_NULL;
    const uintptr_t a16 = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k_cache) |
                          reinterpret_cast<uintptr_t>(v_cache) | reinterpret_cast<uintptr_t>(out);
    const uintptr_t a4 = reinterpret_cast<uintptr_t>(lse) | reinterpret_cast<uintptr_t>(block_table) |
                         reinterpret_cast<uintptr_t>(seq_lens);
    if ((a16 & 15) || (a4 & 3)) return ATTN_ERR_ALIGN;

    const unsigned __int128 cache_elems = (unsigned __int128)num_blocks * H_kv * block_size * d;
    const unsigned __int128 q_elems = (unsigned __int128)B * H * Lq * d;
    if (cache_elems * sizeof(T) >= ((unsigned __int128)1 << 62) || q_elems * 16 >= ((unsigned __int128)1 << 62))
        return ATTN_ERR_SIZE;
    const DecodeShape sh = decode_shape(B, H, H_kv, Lq, max_seq_len);
    if (sh.n_slots * sh.rslot * (d + 2) > (int64_t)1 << 40 || (int64_t)B * H * Lq > INT_MAX ||
        B * sh.nseg > INT_MAX / 2)
        return ATTN_ERR_SIZE;

    const size_t bytes_q = (size_t)(q_elems * sizeof(T));
    const size_t bytes_cache = (size_t)(cache_elems * sizeof(T));
    const size_t bytes_table = (size_t)B * max_blocks * sizeof(int);
    const size_t bytes_lens = (size_t)B * sizeof(int);
    const size_t bytes_lse = (size_t)B * H * Lq * sizeof(float);
    const void *ins[] = {q, k_cache, v_cache, block_table, seq_lens};
    const size_t in_bytes[] = {bytes_q, bytes_cache, bytes_cache, bytes_table, bytes_lens};
    const void *outs[] = {out, lse};
    const size_t out_bytes[] = {bytes_q, bytes_lse};
    for (int i = 0; i < 2; ++i) {
        for (int j = 0; j < 5; ++j)
            if (overlaps(outs[i], out_bytes[i], ins[j], in_bytes[j])) return ATTN_ERR_ALIAS;
        for (int j = i + 1; j < 2; ++j)
            if (overlaps(outs[i], out_bytes[i], outs[j], out_bytes[j])) return ATTN_ERR_ALIAS;
    }
    *bytes_ws_out = decode_workspace_bytes(B, H, H_kv, Lq, d, max_seq_len);

    p.q = q;
    p.kc = k_cache;
    p.vc = v_cache;
    p.table = block_table;
    p.lens = seq_lens;
    p.o = out;
    p.lse = lse;
    p.hdr = nullptr;
    p.part = nullptr;
    p.B = B;
    p.H = H;
    p.H_kv = H_kv;
    p.Lq = Lq;
    p.group = H / H_kv;
    p.rows = (int)sh.rows;
    p.bs = block_size;
    p.bs_shift = __builtin_ctz((unsigned)block_size);
    p.max_blocks = max_blocks;
    p.num_blocks = num_blocks;
    p.max_len = max_seq_len;
    p.window = window;
    p.n_rowblk = (int)sh.n_rowblk;
    p.nseg = (int)sh.nseg;
    p.rslot = (int)sh.rslot;
    p.n_waves = (int)sh.waves_cap;
    p.n_slots = (int)sh.n_slots;
    p.scale_log2 = attn_resolve_scale(scale, d) * 1.4426950408889634f;
    p.d = d;
    return ATTN_OK;
}

template <typename T>
int decode_launch(const DecParams &p, void *stream)
{
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t err = p.d == 64 ? launch_decode<T, 64>(p, s) : launch_decode<T, 128>(p, s);
    return err == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

template <typename T>
int attn_decode_impl(const void *q, const void *k_cache, const void *v_cache, const int *block_table,
                     const int *seq_lens, void *out, float *lse, void *workspace, int B, int H, int H_kv, int Lq,
                     int d, int block_size, int max_blocks, int num_blocks, int max_seq_len, int window,
                     float scale, void *stream)
{
    DecParams p;
    size_t bytes_ws = 0;
    const int st = decode_plan<T>(q, k_cache, v_cache, block_table, seq_lens, out, lse, B, H, H_kv, Lq, d,
                                  block_size, max_blocks, num_blocks, max_seq_len, window, scale, &p, &bytes_ws);
    if (st != ATTN_OK || p.B == 0) return st;
    if (!workspace) return ATTN_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(workspace) & 15) return ATTN_ERR_ALIGN;
    const size_t bytes_q = (size_t)B * H * Lq * d * sizeof(T);
    const size_t bytes_cache = (size_t)num_blocks * H_kv * block_size * d * sizeof(T);
    const void *others[] = {q, k_cache, v_cache, block_table, seq_lens, out, lse};
    const size_t other_bytes[] = {bytes_q, bytes_cache, bytes_cache, (size_t)B * max_blocks * sizeof(int),
                                  (size_t)B * sizeof(int), bytes_q, (size_t)B * H * Lq * sizeof(float)};
    for (int j = 0; j < 7; ++j)
        if (overlaps(workspace, bytes_ws, others[j], other_bytes[j])) return ATTN_ERR_ALIAS;
    p.hdr = static_cast<int64_t *>(workspace);
    p.part = reinterpret_cast<float *>(static_cast<char *>(workspace) + decode_hdr_bytes(B));
    return decode_launch<T>(p, stream);
}

}  // namespace

// ---------------------------------------------------------------- allocation-free entry point
// The partial results of attn_decode_noalloc live in this array, one copy per
// device (the runtime loads it with the code object and keeps it until the
// process ends).  In host code `scratch` is only a stand-in for the device
// symbol: the device address comes from hipGetSymbolAddress, once per device,
// and only that address is ever handed to a kernel.
static constexpr size_t kDecodeScratchBytes = size_t(64) << 20;
static __device__ __align__(256) char scratch[kDecodeScratchBytes];

namespace {

std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device, once looked up

// The current device's copy of `scratch` (looked up on the first call made
// with that device current).
int scratch_pointer(void **ptr)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ATTN_ERR_LAUNCH;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return ATTN_ERR_LAUNCH;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_decode_noalloc(const void *q, const void *k_cache, const void *v_cache, const int *block_table,
                        const int *seq_lens, void *out, float *lse, int B, int H, int H_kv, int Lq, int d,
                        int block_size, int max_blocks_per_seq, int num_blocks, int max_seq_len, int window,
                        float scale, void *stream)
{
    DecParams p;
    size_t bytes_ws = 0;
    const int st = decode_plan<_Float16>(q, k_cache, v_cache, block_table, seq_lens, out, lse, B, H, H_kv, Lq, d,
                                         block_size, max_blocks_per_seq, num_blocks, max_seq_len, window, scale, &p,
                                         &bytes_ws);
    if (st != ATTN_OK || p.B == 0) return st;
    if (bytes_ws > kDecodeScratchBytes) return ATTN_ERR_SCRATCH;
    void *ws = nullptr;
    const int sp = scratch_pointer(&ws);
    if (sp != ATTN_OK) return sp;
    p.hdr = static_cast<int64_t *>(ws);
    p.part = reinterpret_cast<float *>(static_cast<char *>(ws) + decode_hdr_bytes(B));
    return decode_launch<_Float16>(p, stream);
}

size_t attn_decode_workspace_size(int B, int H, int H_kv, int Lq, int d, int max_seq_len)
{
    if (B <= 0 || H < 1 || H_kv < 1 || H % H_kv != 0 || Lq < 1 || max_seq_len < 1 || (d != 64 && d != 128))
        return 0;
    return decode_workspace_bytes(B, H, H_kv, Lq, d, max_seq_len);
}

int attn_decode(const void *q, const void *k_cache, const void *v_cache, const int *block_table,
                const int *seq_lens, void *out, float *lse, void *workspace, int B, int H, int H_kv, int Lq, int d,
                int block_size, int max_blocks_per_seq, int num_blocks, int max_seq_len, int window, float scale,
                void *stream)
{
    return attn_decode_impl<_Float16>(q, k_cache, v_cache, block_table, seq_lens, out, lse, workspace, B, H, H_kv,
                                      Lq, d, block_size, max_blocks_per_seq, num_blocks, max_seq_len, window, scale,
                                      stream);
}

int attn_decode_bf16(const void *q, const void *k_cache, const void *v_cache, const int *block_table,
                     const int *seq_lens, void *out, float *lse, void *workspace, int B, int H, int H_kv, int Lq,
                     int d, int block_size, int max_blocks_per_seq, int num_blocks, int max_seq_len, int window,
                     float scale, void *stream)
{
    return attn_decode_impl<__bf16>(q, k_cache, v_cache, block_table, seq_lens, out, lse, workspace, B, H, H_kv,
                                    Lq, d, block_size, max_blocks_per_seq, num_blocks, max_seq_len, window, scale,
                                    stream);
}

}  // extern "C"
