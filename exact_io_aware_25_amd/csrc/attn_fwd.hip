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
//   * one workgroup = 4 waves of 64 lanes = 128 query rows of one (b, h);
//     each wave owns 32 query rows for the whole pass;
//   * S^T = K Q^T on v_mfma_f32_32x32x16_{f16,bf16} with K as the A operand
//     and Q^T (kept in registers) as the B operand.  In the 32x32 accumulator
//     layout a lane then holds 16 keys of ONE query, so the softmax row
//     statistics are per lane, and the only cross-lane step is between the
//     two 32-lane halves of the wave;
//   * the K rows feeding the A operand are permuted (bits 2 and 3 of the row
//     index swapped) so that the fp32 score registers, rounded to 16 bits,
//     are directly the B operand (P^T) of the second product O^T = V^T P^T;
//   * V is written to LDS transposed (V^T, keys contiguous) so the A operand
//     of O^T = V^T P^T is one 16-byte LDS read per lane;
//   * K and V tiles are double-buffered in LDS: global loads of tile t+1 are
//     in flight while tile t is multiplied;
//   * the softmax runs in the exp2 domain with scale*log2(e) folded in, and
//     O^T stays in fp32 accumulators until a single final write.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>

#include "attn.h"

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = 32;
constexpr int kBlockQ = kRowsPerWave * kWaves;  // query rows per workgroup
constexpr int kBlockK = 64;                     // keys per K/V tile
constexpr int kPad = 8;                         // 16 bytes of padding per LDS row

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

// Row of the K tile that feeds A-operand row m: bits 2 and 3 swapped.  With
// this order, accumulator register r (0..15) of lane half `hi` in a 32-key
// block holds key 16*(r/8) + 8*hi + r%8, i.e. 8 consecutive keys per 16-key
// slice -- the layout the B operand of the second product needs.
__device__ __forceinline__ int k_row_for_lane(int m)
{
    return (m & ~0xC) | ((m & 4) << 1) | ((m & 8) >> 1);
}

template <bool CAUSAL, bool WINDOW>
__device__ __forceinline__ bool visible(int i, int j, int L, int window)
{
    if (j >= L) return false;
    if (CAUSAL && j > i) return false;
    if (WINDOW) {
        if (i - j > window) return false;
        if (!CAUSAL && j - i > window) return false;
    }
    return true;
}

template <typename T, int D, bool CAUSAL, bool WINDOW>
__global__ __launch_bounds__(kThreads) void attn_fwd_kernel(Params p)
{
    typedef typename Vec8<T>::type vec8;
    constexpr int KS = D + kPad;        // K tile row stride (elements)
    constexpr int VS = kBlockK + kPad;  // V^T tile row stride (elements)
    constexpr int kTileK = kBlockK * KS;
    constexpr int kTileV = D * VS;
    constexpr int kChunks = kBlockK * D / 8 / kThreads;  // 16-byte chunks per thread per tile
    constexpr int kDSteps = D / 16;     // k-steps of the first product
    constexpr int kDBlocks = D / 32;    // 32-row blocks of O^T

    __shared__ __attribute__((aligned(16))) T lds_k[2][kTileK];
    __shared__ __attribute__((aligned(16))) T lds_v[2][kTileV];

    const int tid = threadIdx.x;
    const int wave = tid / 64;
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
    int kv_begin = 0, kv_end = L;
    if (WINDOW) kv_begin = max(0, q_first - p.window);
    if (CAUSAL) kv_end = q_last + 1;
    else if (WINDOW) kv_end = min(L, q_last + p.window + 1);
    const int t_begin = kv_begin / kBlockK;
    const int t_end = (kv_end + kBlockK - 1) / kBlockK;

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

    f32x16 acc_o[kDBlocks];
#pragma unroll
    for (int i = 0; i < kDBlocks; ++i) acc_o[i] = f32x16{};
    float m_run = -INFINITY;  // running max of scale*log2(e)*s over keys seen
    float l_run = 0.f;        // running sum of exp2 weights, this lane's half of the keys

    // ---- global -> register -> LDS staging of one K/V tile
    u32x4 reg_k[kChunks], reg_v[kChunks];
    auto load_tile = [&](int t) {
        const int j0 = t * kBlockK;
#pragma unroll
        for (int c = 0; c < kChunks; ++c) {
            const int chunk = tid + c * kThreads;
            const int row = chunk / (D / 8);
            const int col = (chunk % (D / 8)) * 8;
            if (j0 + row < L) {
                reg_k[c] = *reinterpret_cast<const u32x4 *>(kh + (int64_t)(j0 + row) * D + col);
                reg_v[c] = *reinterpret_cast<const u32x4 *>(vh + (int64_t)(j0 + row) * D + col);
            } else {
                reg_k[c] = u32x4{};  // keys past L: zeros keep the products finite
                reg_v[c] = u32x4{};
            }
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int c = 0; c < kChunks; ++c) {
            const int chunk = tid + c * kThreads;
            const int row = chunk / (D / 8);
            const int col = (chunk % (D / 8)) * 8;
            *reinterpret_cast<u32x4 *>(&lds_k[buf][row * KS + col]) = reg_k[c];
            const T *vals = reinterpret_cast<const T *>(&reg_v[c]);
#pragma unroll
            for (int e = 0; e < 8; ++e) lds_v[buf][(col + e) * VS + row] = vals[e];
        }
    };

    if (t_begin < t_end) {
        load_tile(t_begin);
        store_tile(0);
    }

    for (int t = t_begin; t < t_end; ++t) {
        const int buf = (t - t_begin) & 1;
        if (t + 1 < t_end) load_tile(t + 1);
        __syncthreads();

        const int j0 = t * kBlockK;
        const int j_last = j0 + kBlockK - 1;
        bool skip = !wave_live;
        if (CAUSAL) skip = skip || j0 > qb;
        if (WINDOW) {
            skip = skip || j_last < qa - p.window;
            if (!CAUSAL) skip = skip || j0 > qb + p.window;
        }
        if (!skip) {
            bool full = j_last < L;
            if (CAUSAL) full = full && j_last <= qa;
            if (WINDOW) {
                full = full && j0 >= qb - p.window;
                if (!CAUSAL) full = full && j_last <= qa + p.window;
            }

            // S^T for the two 32-key blocks of the tile
            const T *tk = lds_k[buf];
            f32x16 s[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                s[kb] = f32x16{};
                const T *krow = tk + (32 * kb + k_row_for_lane(l32)) * KS + 8 * hi;
#pragma unroll
                for (int ds = 0; ds < kDSteps; ++ds) {
                    vec8 a = *reinterpret_cast<const vec8 *>(krow + 16 * ds);
                    s[kb] = mfma32(a, qf[ds], s[kb]);
                }
            }

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

            // online softmax in the exp2 domain
            float mt = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[kb][r]);
            mt = fmaxf(mt, __shfl_xor(mt, 32));
            const float m_new = fmaxf(m_run, mt * p.scale_log2);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
            float psum = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float e = __builtin_amdgcn_exp2f(fmaf(s[kb][r], p.scale_log2, -m_use));
                    s[kb][r] = e;
                    psum += e;
                }
            l_run = l_run * alpha + psum;
            m_run = m_new;
#pragma unroll
            for (int i = 0; i < kDBlocks; ++i) acc_o[i] *= alpha;

            // O^T += V^T P^T over the four 16-key slices of the tile
            const T *tv = lds_v[buf];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                f32x8 pf;
#pragma unroll
                for (int e = 0; e < 8; ++e) pf[e] = s[ks / 2][8 * (ks % 2) + e];
                const vec8 pv = __builtin_convertvector(pf, vec8);
#pragma unroll
                for (int db = 0; db < kDBlocks; ++db) {
                    vec8 a = *reinterpret_cast<const vec8 *>(tv + (32 * db + l32) * VS + 16 * ks + 8 * hi);
                    acc_o[db] = mfma32(a, pv, acc_o[db]);
                }
            }
        }

        if (t + 1 < t_end) store_tile(buf ^ 1);
    }

    // ---- epilogue: one write of O and lse
    if (!wave_live || qi >= L) return;
    const float l_tot = l_run + __shfl_xor(l_run, 32);
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

bool overlaps(const void *a, size_t na, const void *b, size_t nb)
{
    const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
    return na && nb && pa < pb + nb && pb < pa + na;
}

template <typename T, int D, bool CAUSAL, bool WINDOW>
hipError_t launch_instance(const Params &p, dim3 grid, hipStream_t stream)
{
    Params args = p;
    void *kargs[] = {&args};
    return hipLaunchKernel(reinterpret_cast<const void *>(&attn_fwd_kernel<T, D, CAUSAL, WINDOW>),
                           grid, dim3(kThreads), kargs, 0, stream);
}

template <typename T, int D>
hipError_t launch_mask(const Params &p, bool causal, bool window, dim3 grid, hipStream_t stream)
{
    if (causal)
        return window ? launch_instance<T, D, true, true>(p, grid, stream)
                      : launch_instance<T, D, true, false>(p, grid, stream);
    return window ? launch_instance<T, D, false, true>(p, grid, stream)
                  : launch_instance<T, D, false, false>(p, grid, stream);
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
    const int n_qblk = (L + kBlockQ - 1) / kBlockQ;
    const int64_t blocks = (int64_t)n_qblk * B * H;
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
    p.n_qblk = n_qblk;
    p.scale_log2 = attn_resolve_scale(scale, d) * 1.4426950408889634f;

    const dim3 grid((unsigned)blocks);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const bool win = window >= 0;
    const hipError_t err = d == 64 ? launch_mask<T, 64>(p, causal, win, grid, s)
                                   : launch_mask<T, 128>(p, causal, win, grid, s);
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

const char *attn_status_string(int status)
{
    switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "a tensor pointer is NULL";
    case ATTN_ERR_SHAPE: return "bad shape: need B >= 0, L >= 0, H >= 1, H_kv >= 1, H % H_kv == 0";
    case ATTN_ERR_HEAD_DIM: return "head dimension must be 64 or 128";
    case ATTN_ERR_WINDOW: return "window must be -1 (none) or >= 0";
    case ATTN_ERR_ALIAS: return "out or lse overlaps another tensor";
    case ATTN_ERR_LAUNCH: return "kernel launch failed";
    case ATTN_ERR_SIZE: return "problem too large to index";
    case ATTN_ERR_FLAG: return "causal must be 0 or 1";
    case ATTN_ERR_SCALE: return "scale must be finite";
    case ATTN_ERR_ALIGN: return "q, k, v, out must be 16-byte aligned and lse 4-byte aligned";
    default: return "unknown status";
    }
}

}  // extern "C"
