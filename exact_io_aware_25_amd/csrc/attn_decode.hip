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
//   1. partial (split-K): one wave owns a chunk of one sequence's keys for
//      one K/V head and all query rows that read that head (up to 32 rows:
//      the group's heads times Lq).  Each wave works alone -- its own LDS
//      region, no barriers.  Per 32-key tile: the K rows go straight from the
//      cache into the A-operand registers of S^T = K Q^T (16 contiguous bytes
//      per lane), the V tile goes into LDS by direct-to-LDS loads (for the
//      transposing read of the second product), both one tile ahead; the
//      online softmax is per lane; the chunk's (max, sum, unnormalised O)
//      go to the workspace.
//   2. merge: one workgroup per query row combines its chunks exactly (the
//      same rescale the online softmax uses) and writes O and lse.
// The products run on the 32x32x16 MFMA although at most Lq*H/H_kv of the
// 32 query columns are live: the kernel is bound by bytes, not FLOPs.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "attn.h"
#include "attn_common.h"

namespace {

constexpr int kDecTile = 32;  // keys per tile
constexpr int kDecWaves = 4;  // independent waves per workgroup
constexpr float kLn2 = 0.69314718055994531f;

struct DecParams {
    const void *q, *kc, *vc;
    const int *table, *lens;
    void *o;
    float *lse;
    float *part;        // [rows_total][n_chunks][D] unnormalised O, then [rows_total][n_chunks][2] (m, l)
    int B, H, H_kv, Lq, group, rows;  // rows = group * Lq: query rows per K/V head
    int d;                            // head size (host side: picks the kernel instance)
    int bs, bs_shift, max_blocks, num_blocks, max_len, window;
    int chunk, n_chunks, n_rowblk, n_cgroups;
    float scale_log2;
};

__device__ __forceinline__ int seq_len(const DecParams &p, int b)
{
    return min(max(p.lens[b], 0), p.max_len);
}

// First key any query row of a sequence of n tokens can see.
__device__ __forceinline__ int first_key(const DecParams &p, int n)
{
    return p.window >= 0 ? max(0, n - p.Lq - p.window) : 0;
}

// Physical block holding key j of sequence b (table entries and the block
// number are clamped, so a bad table reads a wrong block, never out of bounds).
__device__ __forceinline__ int64_t page_of(const DecParams &p, int b, int j)
{
    const int lb = min(j >> p.bs_shift, p.max_blocks - 1);
    const int phys = p.table[(int64_t)b * p.max_blocks + lb];
    return min(max(phys, 0), p.num_blocks - 1);
}

// ---------------------------------------------------------------- 1. partial
template <typename T, int D>
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

    const int wave = threadIdx.x / 64;
    const int lane = threadIdx.x % 64;
    const int l32 = lane % 32;
    const int hi = lane / 32;

    int idx = blockIdx.x;
    const int cg = idx % p.n_cgroups;
    idx /= p.n_cgroups;
    const int rowblk = idx % p.n_rowblk;
    idx /= p.n_rowblk;
    const int g = idx % p.H_kv;
    const int b = idx / p.H_kv;
    const int c = __builtin_amdgcn_readfirstlane(cg * kDecWaves + wave);  // this wave's chunk
    if (c >= p.n_chunks) return;
    const int n = seq_len(p, b);
    const int k_begin = max(c * p.chunk, first_key(p, n));
    const int k_end = min(n, (c + 1) * p.chunk);
    if (k_begin >= k_end) return;  // no key here: the merge skips this chunk

    // ---- this lane's query row: (head in group, new-token index)
    const int r = rowblk * 32 + l32;
    const bool row_live = r < p.rows;
    const int hh = row_live ? r / p.Lq : 0;
    const int qi = row_live ? r % p.Lq : 0;
    const int h = g * p.group + hh;
    const int pos = n - p.Lq + qi;  // its position (rows with pos < 0 see no key)
    const T *qrow = static_cast<const T *>(p.q) + (((int64_t)b * p.H + h) * p.Lq + qi) * D;
    vec8 qf[kDSteps];
#pragma unroll
    for (int s = 0; s < kDSteps; ++s)
        qf[s] = row_live ? *reinterpret_cast<const vec8 *>(qrow + 16 * s + 8 * hi) : vec8{};

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

    // The physical blocks of the two 16-key halves of tile t (wave-uniform).
    // They are fetched two tiles ahead, so a tile's data loads never wait on
    // a page-table load.
    struct Pages { int lo, hi; };
    auto pages_of = [&](int t) {
        Pages pg;
        pg.lo = (int)page_of(p, b, t * kDecTile);
        pg.hi = (int)page_of(p, b, t * kDecTile + 16);
        return pg;
    };
    // K fragments of tile t into registers; V tile t into this wave's stage
    auto load_k = [&](int t, Pages pg, vec8 (&kf)[kDSteps]) {
        const int j = t * kDecTile + krow;  // krow < 16 exactly when l32 < 16
        const int64_t page = l32 < 16 ? pg.lo : pg.hi;
        const T *row = kc + ((page * p.H_kv + g) * p.bs + (j & (p.bs - 1))) * D;
#pragma unroll
        for (int s = 0; s < kDSteps; ++s) kf[s] = *reinterpret_cast<const vec8 *>(row + 16 * s + 8 * hi);
    };
    auto copy_v = [&](int t, Pages pg, char *stage) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const int j0 = t * kDecTile + 16 * hf;
            const int valid = min(max(n - j0, 0), 16);  // rows past n arrive as zeros
            const int64_t page = __builtin_amdgcn_readfirstlane(hf ? pg.hi : pg.lo);
            const T *base = vc + ((page * p.H_kv + g) * p.bs + (j0 & (p.bs - 1))) * D;
            const __amdgpu_buffer_rsrc_t rv =
                __builtin_amdgcn_make_buffer_rsrc((void *)base, 0, valid * kRowBytes, 0x00020000);
#pragma unroll
            for (int cc = 0; cc < kHalfCopies; ++cc)
                copy_to_lds16(rv, stage + hf * 16 * kRowBytes + cc * 1024, ld_v[cc]);
        }
    };

    f32x16 acc_o[kDBlocks];
#pragma unroll
    for (int i = 0; i < kDBlocks; ++i) acc_o[i] = f32x16{};
    float m_run = -INFINITY;  // running max of scale*log2(e)*s
    float l_run = 0.f;        // running sum of weights, this lane half's keys

    const int t_first = k_begin / kDecTile;
    const int t_last = (k_end + kDecTile - 1) / kDecTile;  // one past
    const int max_pos = n - 1;
    const int min_pos = n - p.Lq;
    char *stage_a = lds_a[wave];
    char *stage_b = lds_b[wave];

    auto process = [&](int t, const vec8 (&kf)[kDSteps], const char *tv) {
        const int j0 = t * kDecTile;
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

    // two tiles in flight: loads of tile t+1 overlap the products of tile t.
    // The wave waits for its own loads only (vmcnt); before a copy reuses a
    // stage, its reads of that stage have completed (lgkmcnt).
    vec8 kf_a[kDSteps], kf_b[kDSteps];
    Pages pg_next = pages_of(t_first + 1 < t_last ? t_first + 1 : t_first);
    {
        const Pages pg0 = pages_of(t_first);
        load_k(t_first, pg0, kf_a);
        copy_v(t_first, pg0, stage_a);
    }
    for (int t = t_first; t < t_last; t += 2) {
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        if (t + 1 < t_last) {
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
            load_k(t + 1, pg_next, kf_b);
            copy_v(t + 1, pg_next, stage_b);
            if (t + 2 < t_last) pg_next = pages_of(t + 2);
        }
        process(t, kf_a, stage_a);
        if (t + 1 < t_last) {
            __builtin_amdgcn_s_waitcnt(0x0F70);
            if (t + 2 < t_last) {
                __builtin_amdgcn_s_waitcnt(0xC07F);
                load_k(t + 2, pg_next, kf_a);
                copy_v(t + 2, pg_next, stage_a);
                if (t + 3 < t_last) pg_next = pages_of(t + 3);
            }
            process(t + 1, kf_b, stage_b);
        }
    }

    // ---- this chunk's partial result: unnormalised O, max, sum
    if (!row_live) return;
    const int64_t pr = (((int64_t)b * p.H + h) * p.Lq + qi) * p.n_chunks + c;
    const int64_t rows_total = (int64_t)p.B * p.H * p.Lq;
    float *po = p.part + pr * D;
#pragma unroll
    for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            // register 4a+cc of block db holds d = 32db + 8a + 4hi + cc
            const float4 v4 = {acc_o[db][4 * a], acc_o[db][4 * a + 1], acc_o[db][4 * a + 2], acc_o[db][4 * a + 3]};
            *reinterpret_cast<float4 *>(po + 32 * db + 8 * a + 4 * hi) = v4;
        }
    const float l_tot = half_swap_sum(l_run);
    if (hi == 0) {
        float *pml = p.part + rows_total * p.n_chunks * D + 2 * pr;
        pml[0] = m_run;
        pml[1] = l_tot;
    }
}

// ---------------------------------------------------------------- 2. merge
// One workgroup of 4 waves per query row: every thread takes a share of the
// chunks' maxima, the block agrees on the largest M, then wave w sums the
// chunks c = w, w+4, ... with weights 2^(m_c - M) (lanes over d) and the
// four partial sums meet in LDS.
template <typename T, int D>
__global__ __launch_bounds__(256) void attn_decode_merge_kernel(DecParams p)
{
    constexpr int kPer = D / 64;  // elements of O per lane
    __shared__ float red_m[4];
    __shared__ float red_o[4][D + 1];
    const int wave = threadIdx.x / 64;
    const int lane = threadIdx.x % 64;
    const int64_t rows_total = (int64_t)p.B * p.H * p.Lq;
    const int64_t row = blockIdx.x;  // (b*H + h)*Lq + i
    const int b = (int)(row / ((int64_t)p.H * p.Lq));
    const int i = (int)(row % p.Lq);
    const int n = seq_len(p, b);
    const int pos = n - p.Lq + i;
    const int c_first = first_key(p, n) / p.chunk;
    const int c_last = (pos >= 0 && n > 0) ? (n - 1) / p.chunk : c_first - 1;  // empty when pos < 0
    const float *pml = p.part + rows_total * p.n_chunks * D + 2 * row * p.n_chunks;
    const float *po = p.part + row * p.n_chunks * D;

    float m = -INFINITY;
    for (int c = c_first + (int)threadIdx.x; c <= c_last; c += 256) m = fmaxf(m, pml[2 * c]);
#pragma unroll
    for (int off = 32; off > 0; off /= 2) m = fmaxf(m, __shfl_xor(m, off));
    if (lane == 0) red_m[wave] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red_m[0], red_m[1]), fmaxf(red_m[2], red_m[3]));

    float l = 0.f, acc[kPer];
#pragma unroll
    for (int e = 0; e < kPer; ++e) acc[e] = 0.f;
    if (m != -INFINITY) {
#pragma unroll 4
        for (int c = c_first + wave; c <= c_last; c += 4) {
            const float mc = pml[2 * c];
            const float w = mc == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mc - m);
            l += w * pml[2 * c + 1];
#pragma unroll
            for (int e = 0; e < kPer; ++e) acc[e] += w * po[(int64_t)c * D + e * 64 + lane];
        }
    }
#pragma unroll
    for (int e = 0; e < kPer; ++e) red_o[wave][e * 64 + lane] = acc[e];
    if (lane == 0) red_o[wave][D] = l;
    __syncthreads();
    if (wave != 0) return;
    l = (red_o[0][D] + red_o[1][D]) + (red_o[2][D] + red_o[3][D]);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    T *orow = static_cast<T *>(p.o) + row * D;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
        const int d = e * 64 + lane;
        const float o = (red_o[0][d] + red_o[1][d]) + (red_o[2][d] + red_o[3][d]);
        orow[d] = (T)(o * inv);
    }
    if (lane == 0) p.lse[row] = l > 0.f ? (m + __log2f(l)) * kLn2 : -INFINITY;
}

// ------------------------------------------------------------------ host side

// Keys per wave chunk: enough chunks for ~8192 waves over the batch, at least
// 256 keys (8 tiles) so the partial write stays small next to the keys read.
int decode_chunk(int64_t B, int64_t H_kv, int64_t n_rowblk, int64_t max_len)
{
    const int64_t target = 8192;
    int64_t c = (max_len * B * H_kv * n_rowblk + target - 1) / target;
    c = (c + kDecTile - 1) / kDecTile * kDecTile;
    return (int)std::min<int64_t>(std::max<int64_t>(c, 256), 1 << 20);
}

size_t decode_workspace_bytes(int64_t B, int64_t H, int64_t H_kv, int64_t Lq, int d, int64_t max_len)
{
    const int64_t rows = H / H_kv * Lq;
    const int64_t n_rowblk = (rows + 31) / 32;
    const int64_t chunk = decode_chunk(B, H_kv, n_rowblk, max_len);
    const int64_t n_chunks = (max_len + chunk - 1) / chunk;
    return (size_t)(B * H * Lq * n_chunks * (d + 2) * (int64_t)sizeof(float));
}

template <typename T, int D>
hipError_t launch_decode(DecParams p, hipStream_t stream)
{
    void *kargs[] = {&p};
    const int64_t grid1 = (int64_t)p.B * p.H_kv * p.n_rowblk * p.n_cgroups;
    hipError_t err = hipLaunchKernel(reinterpret_cast<const void *>(&attn_decode_partial_kernel<T, D>),
                                     dim3((unsigned)grid1), dim3(64 * kDecWaves), kargs, 0, stream);
    if (err != hipSuccess) return err;
    const int64_t rows_total = (int64_t)p.B * p.H * p.Lq;
    return hipLaunchKernel(reinterpret_cast<const void *>(&attn_decode_merge_kernel<T, D>),
                           dim3((unsigned)rows_total), dim3(256), kargs, 0, stream);
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
    const int rows = H / H_kv * Lq;
    const int n_rowblk = (rows + 31) / 32;
    const int chunk = decode_chunk(B, H_kv, n_rowblk, max_seq_len);
    const int n_chunks = (max_seq_len + chunk - 1) / chunk;
    const int n_cgroups = (n_chunks + kDecWaves - 1) / kDecWaves;
    if ((int64_t)B * H_kv * n_rowblk * n_cgroups > INT_MAX || (int64_t)B * H * Lq > INT_MAX)
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
    p.part = nullptr;
    p.B = B;
    p.H = H;
    p.H_kv = H_kv;
    p.Lq = Lq;
    p.group = H / H_kv;
    p.rows = rows;
    p.bs = block_size;
    p.bs_shift = __builtin_ctz((unsigned)block_size);
    p.max_blocks = max_blocks;
    p.num_blocks = num_blocks;
    p.max_len = max_seq_len;
    p.window = window;
    p.chunk = chunk;
    p.n_chunks = n_chunks;
    p.n_rowblk = n_rowblk;
    p.n_cgroups = n_cgroups;
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
    p.part = static_cast<float *>(workspace);
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

constexpr int kMaxDevices = 64;
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
    p.part = static_cast<float *>(ws);
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
