// attn_fwd.hip -- exact attention forward for MI355X (CDNA4, gfx950).
//
// The method: softmax(scale * Q K^T + mask) V computed tile by tile so the
// L x L score matrix never reaches device memory.  Q, K and V are split into
// blocks that fit on chip, a running row maximum and row sum make the softmax
// exact across blocks ("online softmax"), and only the final O and the row
// logsumexp are written («Что такое memory-efficient attention для long
// context на 8x H100?», section 2: tiling into on-chip blocks, partial softmax
// accumulated on chip, only O written back, O(n) memory).  Masks and heads:
// causal flag, sliding window, fewer K/V heads than query heads («Оптимизация
// внимания Flash», Quick start and Workflow 2, Steps 2-3).
//
// The pages' own kernels target NVIDIA parts (shared-memory tiling, TMA,
// warp groups).  This file is written for gfx950:
//   * a key-range group = 4 or 8 waves of 64 lanes = 128 or 256 query rows of
//     one (b, h); each wave owns 32 query rows for the whole pass; a
//     workgroup holds 1, 2 or 4 groups that split the key range and merge
//     their partial results exactly at the end (the launch shape is chosen
//     per problem, see launch_shape);
//   * S^T = K Q^T on v_mfma_f32_32x32x16_{f16,bf16} with K as the A operand
//     and Q^T (kept in registers) as the B operand.  In the 32x32 accumulator
//     layout a lane then holds 16 keys of ONE query, so the softmax row
//     statistics are per lane, and the only cross-lane step is between the
//     two 32-lane halves of the wave;
//   * the K rows feeding the A operand are permuted (bits 2 and 3 of the row
//     index swapped) so that the fp32 score registers, rounded to 16 bits,
//     are directly the B operand (P^T) of the second product O^T = V^T P^T;
//   * V stays row-major in LDS and the A operand V^T of the second product
//     comes from transposing LDS reads (ds_read_b64_tr_b16);
//   * K and V tiles go from device memory straight into LDS (buffer loads
//     with an LDS destination), double-buffered: the copy of tile t+1 is in
//     flight while tile t is multiplied;
//   * the softmax runs in the exp2 domain with scale*log2(e) folded in, and
//     O^T stays in fp32 accumulators until a single final write.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>
#include <type_traits>

#include "attn.h"
#include "attn_common.h"

namespace {

struct Params {
    const void *q, *k, *v;
    void *o;
    float *lse;
    int B, H, H_kv, L;
    int group;          // H / H_kv
    int window;         // -1 or the window size
    int n_qblk;         // ceil(L / kBlockQ)
    float scale_log2;   // scale * log2(e)
};

// Largest per-lane tile sum of softmax weights the fast path accepts.  It
// bounds every weight by 2^15, inside fp16 range, and keeps the sum of a
// whole row (at most 2^15 per key) far inside fp32 range.
constexpr float kMaxTileSum = 32768.0f;

// A workgroup owns NW*32 query rows of one (b, h).  Its waves form SPLIT
// groups of NW waves; wave w of group s takes rows 32w.. of the block and the
// s-th contiguous share of the block's key tiles.  The NW waves of a group
// share each K/V tile of their share.  With SPLIT > 1 the groups' partial
// results (O, reference max, sum) are merged at the end with the same exact
// rescale the online softmax uses; this shortens the serial key loop of short
// problems, whose grids are too small to fill the GPU.
template <typename T, int D, bool CAUSAL, bool WINDOW, int NW, int SPLIT>
__global__ __launch_bounds__(64 * NW * SPLIT) void attn_fwd_kernel(Params p)
{
    typedef typename Vec8<T>::type vec8;
    constexpr int kWaves = NW;
    constexpr int kThreads = 64 * NW;  // threads of one group
    constexpr int kBlockQ = kRowsPerWave * NW;  // query rows per workgroup
    constexpr int kRowBytes = 2 * D;                      // one K or V row in LDS
    constexpr int kTileBytes = kBlockK * kRowBytes;       // one K or V tile
    constexpr int kChunks = kBlockK * (D / 8) / kThreads;  // 16-byte units per thread per tile
    constexpr int kDSteps = D / 16;                       // k-steps of the first product
    constexpr int kDBlocks = D / 32;                      // 32-row blocks of O^T
    // fp16 row sums on the matrix cores (see weights() below); the 8-wave
    // shapes have the registers for it, the smaller ones keep VALU dot2 sums
    constexpr bool kSumOnMfma = std::is_same<T, _Float16>::value && NW == 8;

    // two stages of [group][K | V] tiles, as separate objects so the compiler
    // can tell copies into one stage from reads of the other
    __shared__ __attribute__((aligned(16))) char lds_a[SPLIT][2][kTileBytes];
    __shared__ __attribute__((aligned(16))) char lds_b[SPLIT][2][kTileBytes];

    const int tid = threadIdx.x;
    const int grp = SPLIT > 1 ? __builtin_amdgcn_readfirstlane(tid / 64 / NW) : 0;  // key-range group
    // wave-uniform (an SGPR): the row block and everything derived from it
    // (its first and last rows, liveness, skip tests) stay out of VGPRs
    const int wave = __builtin_amdgcn_readfirstlane((tid / 64) % NW);  // row block within the group
    const int lane = tid % 64;
    const int l32 = lane % 32;
    const int hi = lane / 32;

    // ---- work partition: heaviest query blocks first when causal
    const int BH = p.B * p.H;
    const int order = blockIdx.x / BH;
    const int bh = blockIdx.x % BH;
    const int qblk = CAUSAL ? (p.n_qblk - 1 - order) : order;
    const int b = bh / p.H;
    const int h = bh % p.H;
    const int g = h / p.group;
    const int L = p.L;

    const T *qh = static_cast<const T *>(p.q) + ((int64_t)b * p.H + h) * L * D;
    const T *kh = static_cast<const T *>(p.k) + ((int64_t)b * p.H_kv + g) * L * D;
    const T *vh = static_cast<const T *>(p.v) + ((int64_t)b * p.H_kv + g) * L * D;
    T *oh = static_cast<T *>(p.o) + ((int64_t)b * p.H + h) * L * D;
    float *lseh = p.lse + ((int64_t)b * p.H + h) * L;

    // ---- key range of the workgroup, and the tiles that cover it
    const int q_first = qblk * kBlockQ;
    const int q_last = min(L, q_first + kBlockQ) - 1;
    const TileRange tiles = key_tiles<CAUSAL, WINDOW, SPLIT>(q_first, q_last, L, p.window, kBlockK, grp);
    const int t_begin = tiles.t_begin;  // this group's tiles
    const int t_end = tiles.t_end;
    const int t_stop = tiles.t_stop;    // steps every group runs

    // ---- this wave's query rows
    const int qa = q_first + wave * kRowsPerWave;
    const int qb = min(qa + kRowsPerWave, L) - 1;
    const bool wave_live = qa < L;
    const int qi = qa + l32;  // this lane's query row

    // Q^T fragments (B operand of S^T = K Q^T), kept in registers
    vec8 qf[kDSteps];
#pragma unroll
    for (int s = 0; s < kDSteps; ++s) {
        if (qi < L)
            qf[s] = *reinterpret_cast<const vec8 *>(qh + (int64_t)qi * D + 16 * s + 8 * hi);
        else
            qf[s] = vec8{};
    }

    // ---- per-lane LDS byte offsets (swizzled), fixed for the whole pass
    int koff[kDSteps];
#pragma unroll
    for (int ds = 0; ds < kDSteps; ++ds) koff[ds] = k_frag_offset<D, kSwzK>(lane, ds);
    int voff[kDBlocks];  // + 16 ks rows per key slice, + 4 rows for the second read
#pragma unroll
    for (int db = 0; db < kDBlocks; ++db) voff[db] = v_tr_offset<D, kSwzV>(lane, db);
    f32x16 acc_o[kDBlocks];
#pragma unroll
    for (int i = 0; i < kDBlocks; ++i) acc_o[i] = f32x16{};
    float m_run = -INFINITY;  // reference max of scale*log2(e)*s (log2 domain), -inf until a key is seen
    float neg_m = 0.f;        // -m_run, or 0 while m_run is -inf
    // sum of the rounded weights: with kSumOnMfma the whole row's (every lane
    // of the query holds it), otherwise this lane's half of the keys
    float l_run = 0.f;
    // A operand of the row-sum product (16x16x32): the word 0x3C003C00 (two
    // fp16 ones) where row 4G of the selector picks the k-groups holding the
    // query of lane group G, else zero (see weights())
    const int sel_m = lane % 16, sel_g = lane / 16;
    const uint32_t ones_word = (sel_m % 4 == 0 && (sel_g & 1) == ((sel_m >> 2) & 1)) ? 0x3C003C00u : 0u;

    // ---- global -> LDS copies of one K/V tile, straight into LDS (no VGPR
    // staging).  A wave-wide copy instruction writes 64 consecutive 16-byte
    // LDS units, one per lane in lane order, so lane i fetches the logical unit
    // that the swizzle places at LDS unit i.  The buffer resource starts at the
    // tile and ends at key L: rows past L read as zeros, keeping every product
    // finite (those keys are masked).
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    int ld_k[kChunks], ld_v[kChunks];
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
        const int unit_idx = (c * kWaves + wave) * 64 + lane;  // LDS unit this lane fills
        ld_k[c] = copy_src_offset<D, kSwzK>(unit_idx);
        ld_v[c] = copy_src_offset<D, kSwzV>(unit_idx);
    }
    auto copy_tile = [&](int t, char (*stage)[2][kTileBytes]) {
        const int j0 = t * kBlockK;
        const int bytes = min(L - j0, kBlockK) * kRowBytes;  // keys j0 .. min(j0 + 63, L - 1)
        const __amdgpu_buffer_rsrc_t rk =
            __builtin_amdgcn_make_buffer_rsrc((void *)(kh + (int64_t)j0 * D), 0, bytes, 0x00020000);
        const __amdgpu_buffer_rsrc_t rv =
            __builtin_amdgcn_make_buffer_rsrc((void *)(vh + (int64_t)j0 * D), 0, bytes, 0x00020000);
#pragma unroll
        for (int c = 0; c < kChunks; ++c) {
            const int region = (c * kWaves + wave_u) * 1024;
            copy_to_lds16(rk, &stage[grp][0][region], ld_k[c]);
            copy_to_lds16(rv, &stage[grp][1][region], ld_v[c]);
        }
    };

    if (t_begin < t_end) copy_tile(t_begin, lds_a);

    // One tile: wait for this wave's copies, barrier (the tile is then in LDS
    // and every wave is done with the other stage), start copying the next
    // tile into the other stage, then compute on this one.
    // (Every wave runs the same number of steps, `chunk`; a group whose share
    // is shorter idles through the rest, still meeting every barrier.)
    auto process_tile = [&](int t, char (*cur)[2][kTileBytes], char (*nxt)[2][kTileBytes]) {
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's copies have landed
        __syncthreads();
        if (t + 1 < t_end) copy_tile(t + 1, nxt);

        const int j0 = t * kBlockK;
        const int cls = tile_class<CAUSAL, WINDOW>(j0, qa, qb, L, p.window, kBlockK);
        const bool skip = !wave_live || (SPLIT > 1 && t >= t_end) || cls == 0;
        if (!skip) {
            const bool full = cls == 1;

            // S^T for the two 32-key blocks of the tile
            const char *tk = cur[grp][0];
            f32x16 s[2];
            __builtin_amdgcn_s_setprio(1);
            {
                // every K fragment is read before the first product, so the LDS
                // latency is paid once per tile instead of once per product (the
                // registers are those of the previous tile's weights, dead here)
                vec8 kf[2][kDSteps];
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int ds = 0; ds < kDSteps; ++ds)
                        kf[kb][ds] = *reinterpret_cast<const vec8 *>(tk + 32 * kb * kRowBytes + koff[ds]);
                __builtin_amdgcn_sched_barrier(0);
                s[0] = f32x16{};
                s[1] = f32x16{};
#pragma unroll
                for (int ds = 0; ds < kDSteps; ++ds)
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb) s[kb] = mfma32(kf[kb][ds], qf[ds], s[kb]);
            }

            __builtin_amdgcn_s_setprio(0);
            // mask: register r of block kb holds key j0 + 32*kb + 16*(r/8) + 8*hi + r%8
            if (!full) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int j = j0 + 32 * kb + 16 * (r / 8) + 8 * hi + (r % 8);
                        if (!visible<CAUSAL, WINDOW>(qi, j, L, p.window)) s[kb][r] = -INFINITY;
                    }
            }

            // Online softmax in the exp2 domain.  Fast path: weights against the
            // current reference maximum, with no per-tile maximum.  If a weight
            // of some row in the wave could exceed 2^15 (its tile sum does), or
            // a row has no reference yet, the slow path takes the tile's true
            // row maxima, moves the reference, rescales O and the sum, and
            // recomputes the weights.  Either way the result is the exact
            // softmax: the reference cancels between O and the sum.
            vec8 pv[4];
            float l_tile = 0.f, part[4];
            auto weights = [&]() {
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    f32x8 pf;
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        pf[e] = __builtin_amdgcn_exp2f(fmaf(s[ks / 2][8 * (ks % 2) + e], p.scale_log2, neg_m));
                    pv[ks] = __builtin_convertvector(pf, vec8);
                    if constexpr (kSumOnMfma) {
                        (void)part;  // summed below on the matrix cores
                    } else if constexpr (std::is_same<T, _Float16>::value) {
                        part[ks] = sum8(pv[ks], 0.f);  // the rounded weights, as the product uses them
                    } else {
                        // bf16 rounding of the weights (2^-8) would reach the lse of
                        // short rows, so the sum takes them in fp32: one running
                        // sum over the tile, started from its first weight
#pragma unroll
                        for (int e = 0; e < 8; ++e) l_tile = (ks == 0 && e == 0) ? pf[0] : l_tile + pf[e];
                        // pack here: left to itself the compiler moves the packs past
                        // the sum check, keeping all 32 fp32 weights live across it
                        // (11 more VGPRs, one wave per SIMD fewer at d=64)
                        asm volatile("" : "+v"(pv[ks]));
                    }
                }
                if constexpr (kSumOnMfma) {
                    // Row sums of the rounded weights as a 16x16x32 product on the
                    // matrix cores instead of 16 dot2 per lane: the B operand is
                    // each 16-key slice of P^T as held for the second product
                    // (lane 16g + n: query n + 16(g & 1), keys 8(g >> 1)..+7 of
                    // the slice), the A operand a 0/1 selector whose row 4G sums
                    // the k-groups g with g & 1 == G & 1.  Result row 4G, column n
                    // sits in register 0 of lane 16G + n: that lane's own query,
                    // summed over all 64 keys of the tile.  Products with 1 and 0
                    // are exact and accumulate in fp32, as the dot2 sums did.  The
                    // selector word is rebuilt per tile so that its four registers
                    // are not live across the loop.
                    uint32_t w = ones_word;
                    asm volatile("" : "+v"(w));
                    const f16x8 sel = __builtin_bit_cast(f16x8, u32x4{w, w, w, w});
                    f32x4 ls = __builtin_amdgcn_mfma_f32_16x16x32_f16(sel, pv[0], f32x4{}, 0, 0, 0);
#pragma unroll
                    for (int ks = 1; ks < 4; ++ks) ls = __builtin_amdgcn_mfma_f32_16x16x32_f16(sel, pv[ks], ls, 0, 0, 0);
                    l_tile = ls[0];
                } else if constexpr (std::is_same<T, _Float16>::value) {
                    // four independent dot2 chains, combined pairwise (one chain
                    // of 16 dependent dot2 measured 4 % slower at the 128k shape)
                    l_tile = (part[0] + part[1]) + (part[2] + part[3]);
                }
            };
            weights();
            if (__any(!(l_tile <= kMaxTileSum) || m_run == -INFINITY)) {
                float mt = -INFINITY;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[kb][r]);
                const float m_new = fmaxf(m_run, half_swap_max(mt) * p.scale_log2);
                if (__any(m_new > m_run)) {
                    const float alpha = m_new > m_run ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
                    l_run *= alpha;
#pragma unroll
                    for (int i = 0; i < kDBlocks; ++i) acc_o[i] *= alpha;
                    m_run = m_new;
                    neg_m = (m_new == -INFINITY) ? 0.f : -m_new;
                    weights();
                }
            }
            l_run += l_tile;

            // O^T += V^T P^T over the four 16-key slices of the tile
            const char *tv = cur[grp][1];
            __builtin_amdgcn_s_setprio(1);
            auto read_v = [&](int ks, vec8 (&vf)[kDBlocks]) {
#pragma unroll
                for (int db = 0; db < kDBlocks; ++db) {
                    const char *base = tv + 16 * ks * kRowBytes + voff[db];
                    const s16x4 lo4 = lds_read_tr16(base);
                    const s16x4 hi4 = lds_read_tr16(base + 4 * kRowBytes);
                    vf[db] = __builtin_bit_cast(vec8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
                }
            };
            {
                // the V fragments of slice ks+1 are read while slice ks multiplies
                vec8 vf[2][kDBlocks];
                read_v(0, vf[0]);
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) {
                    if (ks + 1 < 4) read_v(ks + 1, vf[(ks + 1) & 1]);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int db = 0; db < kDBlocks; ++db) acc_o[db] = mfma32(vf[ks & 1][db], pv[ks], acc_o[db]);
                }
            }
            __builtin_amdgcn_s_setprio(0);
        }
    };

    for (int t = t_begin; t < t_stop; t += 2) {
        process_tile(t, lds_a, lds_b);
        if (t + 1 < t_stop) process_tile(t + 1, lds_b, lds_a);
    }

    // ---- merge the groups' partial results into group 0, one group per
    // round, through the now idle stage buffers: with M = max(m_0, m_s),
    // O = 2^(m_0-M) O_0 + 2^(m_s-M) O_s and likewise the sums
    if constexpr (SPLIT > 1) {
        typedef MergeLayout<D, NW, SPLIT> ML;
        constexpr int kPart = ML::kPart;  // floats per lane: O^T, reference max, sum
        constexpr int kPerBuffer = ML::kPerBuffer;  // wave slots per stage buffer
        constexpr int kBatch = ML::kBatch;          // row blocks merged per round
        static_assert(ML::kBufferBytes == (int)sizeof(lds_a) && kPerBuffer >= 1, "merge slot does not fit");
        for (int s = 1; s < SPLIT; ++s) {
            for (int first = 0; first < NW; first += kBatch) {
                const int i = wave - first;  // slot of this wave in the round
                const bool in_round = i >= 0 && i < kBatch;
                float *slot = reinterpret_cast<float *>(i < kPerBuffer ? &lds_a[0][0][0] : &lds_b[0][0][0]) +
                              ML::slot_float_offset(i);
                __syncthreads();  // the previous round (or the last tile) is done with the buffers
                if (grp == s && in_round) {
#pragma unroll
                    for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
                        for (int r = 0; r < 16; ++r) slot[(16 * db + r) * 64 + lane] = acc_o[db][r];
                    slot[(kPart - 2) * 64 + lane] = m_run;
                    slot[(kPart - 1) * 64 + lane] = l_run;
                }
                __syncthreads();
                if (grp == 0 && in_round) {
                    const float m_s = slot[(kPart - 2) * 64 + lane];
                    const float m_new = fmaxf(m_run, m_s);
                    const float a_own = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
                    const float a_s = m_s == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_s - m_new);
#pragma unroll
                    for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            acc_o[db][r] = a_own * acc_o[db][r] + a_s * slot[(16 * db + r) * 64 + lane];
                    l_run = a_own * l_run + a_s * slot[(kPart - 1) * 64 + lane];
                    m_run = m_new;
                }
            }
        }
    }

    // ---- epilogue: one write of O and lse
    if (grp != 0 || !wave_live || qi >= L) return;
    const float l_tot = kSumOnMfma ? l_run : half_swap_sum(l_run);
    const float inv = 1.f / l_tot;
    if (hi == 0) lseh[qi] = (m_run + __log2f(l_tot)) * 0.69314718055994531f;
    T *orow = oh + (int64_t)qi * D;
#pragma unroll
    for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            // register 4a+c of block db holds d = 32*db + 8*a + 4*hi + c
            T outv[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) outv[c] = (T)(acc_o[db][4 * a + c] * inv);
            *reinterpret_cast<uint64_t *>(orow + 32 * db + 8 * a + 4 * hi) =
                *reinterpret_cast<const uint64_t *>(outv);
        }
}

// ------------------------------------------------------------------ host side

template <typename T, int D, bool CAUSAL, bool WINDOW, int NW, int SPLIT>
hipError_t launch_waves(Params p, hipStream_t stream)
{
    p.n_qblk = (p.L + kRowsPerWave * NW - 1) / (kRowsPerWave * NW);
    const dim3 grid((unsigned)((int64_t)p.n_qblk * p.B * p.H));
    void *kargs[] = {&p};
    return hipLaunchKernel(reinterpret_cast<const void *>(&attn_fwd_kernel<T, D, CAUSAL, WINDOW, NW, SPLIT>),
                           grid, dim3(64 * NW * SPLIT), kargs, 0, stream);
}

// Workgroup shape: waves per key-range group (2 -> 64 query rows, 4 -> 128,
// 8 -> 256) and number of key-range groups.  Measured on MI355X: 8-wave
// groups halve K/V traffic per FLOP and win once the 256-row grid has >= 512
// blocks; plain causal grids have unequal blocks (the last one walks every
// key), so below 2048 blocks their serial key loop is split (2 groups of 8
// waves at d=64, else 4 groups of 4 waves).  The shortest plain causal grids
// (<= 256 blocks of 128 rows: 4k and 8k tokens at 4 heads) are held by the
// last block's walk on one CU; at d=64, 64-row workgroups of 4 groups of 2
// waves halve it (causal 4k, H=4: 38 -> 28 us; 8k: 70 -> 62 us).  Other small
// grids split in 2.  Limits: a 16-wave workgroup must fit 128 VGPRs per
// wave, which d=128 does not, and four d=128 splits would not fit LDS.
void launch_shape(int64_t B, int64_t H, int64_t L, int d, bool causal, int window, int *waves, int *splits)
{
    const int64_t g8 = (L + 255) / 256 * B * H;
    const int64_t g4 = (L + 127) / 128 * B * H;
    const bool unequal = causal && window < 0;
    *waves = 8;
    *splits = 1;
    if (g8 >= 2048 || (g8 >= 512 && !unequal)) return;
    if (g8 >= 512) {
        *splits = d == 64 ? 2 : 1;
        return;
    }
    *waves = 4;
    if (unequal) {
        *splits = d == 64 ? 4 : 2;
        if (d == 64 && g4 <= 256) *waves = 2;
    } else {
        *splits = g4 < 512 ? 2 : 1;
    }
}

template <typename T, int D, bool CAUSAL, bool WINDOW>
hipError_t launch_instance(const Params &p, hipStream_t stream)
{
    int waves, splits;
    launch_shape(p.B, p.H, p.L, D, CAUSAL, WINDOW ? p.window : -1, &waves, &splits);
    if (waves == 8) {
        if constexpr (D == 64) {
            if (splits == 2) return launch_waves<T, D, CAUSAL, WINDOW, 8, 2>(p, stream);
        }
        return launch_waves<T, D, CAUSAL, WINDOW, 8, 1>(p, stream);
    }
    if constexpr (D == 64 && CAUSAL && !WINDOW) {
        if (waves == 2) return launch_waves<T, D, CAUSAL, WINDOW, 2, 4>(p, stream);
    }
    if constexpr (D == 64) {
        if (splits == 4) return launch_waves<T, D, CAUSAL, WINDOW, 4, 4>(p, stream);
    }
    if (splits >= 2) return launch_waves<T, D, CAUSAL, WINDOW, 4, 2>(p, stream);
    return launch_waves<T, D, CAUSAL, WINDOW, 4, 1>(p, stream);
}

template <typename T, int D>
hipError_t launch_mask(const Params &p, bool causal, bool window, hipStream_t stream)
{
    if (causal)
        return window ? launch_instance<T, D, true, true>(p, stream)
                      : launch_instance<T, D, true, false>(p, stream);
    return window ? launch_instance<T, D, false, true>(p, stream)
                  : launch_instance<T, D, false, false>(p, stream);
}

template <typename T>
int attn_forward(const void *q, const void *k, const void *v, void *out, float *lse, int B, int H,
                 int H_kv, int L, int d, int causal, int window, float scale, void *stream)
{
    if (B < 0 || L < 0 || H < 1 || H_kv < 1 || H % H_kv != 0) return ATTN_ERR_SHAPE;
    if (d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
    if (window < -1) return ATTN_ERR_WINDOW;
    if (causal != 0 && causal != 1) return ATTN_ERR_FLAG;
    if (std::isinf(scale)) return ATTN_ERR_SCALE;
    if (B == 0 || L == 0) return ATTN_OK;
    if (!q || !k || !v || !out || !lse) return ATTN_ERR_NULL;
    // 16-byte vector loads and stores of q, k, v and out; 4-byte lse stores
    if (((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
          reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(out)) & 15) ||
        (reinterpret_cast<uintptr_t>(lse) & 3))
        return ATTN_ERR_ALIGN;

    // sizes in bytes, with overflow checks (2^62 keeps every product in range)
    const unsigned __int128 rows_q = (unsigned __int128)B * H * L;
    const unsigned __int128 rows_kv = (unsigned __int128)B * H_kv * L;
    if (rows_q * d * sizeof(T) >= ((unsigned __int128)1 << 62)) return ATTN_ERR_SIZE;
    const size_t bytes_q = (size_t)(rows_q * d * sizeof(T));
    const size_t bytes_kv = (size_t)(rows_kv * d * sizeof(T));
    const size_t bytes_lse = (size_t)(rows_q * sizeof(float));
    const int64_t blocks = (int64_t)((L + 127) / 128) * B * H;  // the finer of the two grids
    if (blocks > INT_MAX) return ATTN_ERR_SIZE;
    if (overlaps(out, bytes_q, q, bytes_q) || overlaps(out, bytes_q, k, bytes_kv) ||
        overlaps(out, bytes_q, v, bytes_kv) || overlaps(out, bytes_q, lse, bytes_lse) ||
        overlaps(lse, bytes_lse, q, bytes_q) || overlaps(lse, bytes_lse, k, bytes_kv) ||
        overlaps(lse, bytes_lse, v, bytes_kv))
        return ATTN_ERR_ALIAS;

    Params p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = out;
    p.lse = lse;
    p.B = B;
    p.H = H;
    p.H_kv = H_kv;
    p.L = L;
    p.group = H / H_kv;
    p.window = window;
    p.scale_log2 = attn_resolve_scale(scale, d) * 1.4426950408889634f;

    const hipStream_t s = static_cast<hipStream_t>(stream);
    const bool win = window >= 0;
    const hipError_t err = d == 64 ? launch_mask<T, 64>(p, causal, win, s)
                                   : launch_mask<T, 128>(p, causal, win, s);
    return err == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}

}  // namespace

extern "C" {

float attn_resolve_scale(float scale, int d)
{
    if (!(scale > 0.0f)) return (float)(1.0 / std::sqrt((double)(d > 0 ? d : 1)));
    return scale;
}

int attn_fwd(const void *q, const void *k, const void *v, void *out, float *lse, int B, int H,
             int H_kv, int L, int d, int causal, int window, float scale, void *stream)
{
    return attn_forward<_Float16>(q, k, v, out, lse, B, H, H_kv, L, d, causal, window, scale, stream);
}

int attn_fwd_bf16(const void *q, const void *k, const void *v, void *out, float *lse, int B, int H,
                  int H_kv, int L, int d, int causal, int window, float scale, void *stream)
{
    return attn_forward<__bf16>(q, k, v, out, lse, B, H, H_kv, L, d, causal, window, scale, stream);
}

int attn_launch_shape(int B, int H, int L, int d, int causal, int window, int *waves_per_group,
                      int *key_splits)
{
    if (!waves_per_group || !key_splits) return ATTN_ERR_NULL;
    if (B < 0 || L < 0 || H < 1) return ATTN_ERR_SHAPE;
    if (d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
    if (window < -1) return ATTN_ERR_WINDOW;
    if (causal != 0 && causal != 1) return ATTN_ERR_FLAG;
    launch_shape(B, H, L, d, causal == 1, window, waves_per_group, key_splits);
    return ATTN_OK;
}

const char *attn_status_string(int status)
{
    switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "a tensor pointer is NULL";
    case ATTN_ERR_SHAPE: return "bad shape: need B >= 0, L >= 0, H >= 1, H_kv >= 1, H % H_kv == 0";
    case ATTN_ERR_HEAD_DIM: return "head dimension must be 64 or 128";
    case ATTN_ERR_WINDOW: return "window must be -1 (none) or >= 0";
    case ATTN_ERR_ALIAS: return "an output overlaps another tensor";
    case ATTN_ERR_LAUNCH: return "kernel launch failed";
    case ATTN_ERR_SIZE: return "problem too large to index";
    case ATTN_ERR_FLAG: return "causal must be 0 or 1";
    case ATTN_ERR_SCALE: return "scale must be finite";
    case ATTN_ERR_ALIGN: return "tensors must be 16-byte aligned (lse 4-byte aligned)";
    case ATTN_ERR_SCRATCH: return "the call needs more workspace than the static scratch of attn_decode_noalloc holds";
    default: return "unknown status";
    }
}

}  // extern "C"
