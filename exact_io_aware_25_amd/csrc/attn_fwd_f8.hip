// attn_fwd_f8.hip -- exact attention forward with fp8 (OCP E4M3) inputs for
// MI355X (CDNA4, gfx950).
//
// «Оптимизация внимания Flash», Workflow 3: q, k, v cast to float8_e4m3fn and
// run through the same attention call, for up to twice the fp16 speed.  The
// result is still the forward definition of the decoded fp8 inputs; both
// products run on gfx950's 32x32x64 fp8 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4
// with unit scales), twice the work per instruction of the 16-bit one:
//   * S^T = K Q^T: a lane holds 32 contiguous d-bytes of one key row (A) or
//     one query (B); at d=64 one instruction covers the whole dot product of a
//     32x32 block.  The key rows feed the A operand in the bit-2/3-swapped
//     order of the 16-bit kernel, so lane half hi of block kb holds keys
//     32kb + 16t + 8hi + e (t, e < 2, 8) in registers 8t + e;
//   * P^T: the weights, packed to fp8 in register order, are exactly the B
//     operand of O^T += V^T P^T for the 64-key tile (byte 8(2kb+t) + e);
//   * V^T: four 8-bit transposing LDS reads (ds_read_b64_tr_b8) per 64-key
//     tile, each giving a lane 8 keys of its d row: within a 16-lane group,
//     lane i receives byte i%8 of the chunks addressed by lanes i/8 + 2e, so
//     lanes 2e and 2e+1 address key e's row at d offsets +0 and +8;
//   * weights are taken against the running reference plus 3 (2^3), so a
//     weight is at most 8 when the reference is the row's maximum and the
//     bulk stays in e4m3's normal range; a lane's tile sum above 448 (e4m3's
//     largest value) sends the tile to the exact slow path; the row sums stay
//     in fp32, so lse is not touched by the 8-bit rounding;
//   * O is written in bf16.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>

#include "attn.h"
#include "attn_common.h"

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

constexpr float kF8Max = 448.0f;
constexpr float kF8Shift = 3.0f;  // weights against reference + 2^3

struct F8Params {
    const uint8_t *q, *k, *v;
    __bf16 *o;
    float *lse;
    int B, H, H_kv, L;
    int group;
    int window;
    int n_qblk;
    float scale_log2;
};

__device__ __forceinline__ f32x16 mfma_f8(i32x8 a, i32x8 b, f32x16 c)
{
    // format 0 = fp8 E4M3 for both operands; scale exponents 127 = 2^0
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ i32x2 lds_read_tr8(const void *generic_lds_ptr)
{
    auto p = (__attribute__((address_space(3))) char *)(generic_lds_ptr);
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2 *)p);
}

// four fp32 values -> four E4M3 bytes of one dword (round to nearest even).
// Each conversion writes one half of the dword and keeps the other; the
// first keeps half of a's own bits, which the second then overwrites, so the
// result can take a's register (with 0 there it needs a zeroed register).
__device__ __forceinline__ int pack4_f8(float a, float b, float c, float d)
{
    int x = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __builtin_bit_cast(int, a), false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, x, true);
}

template <int D, bool CAUSAL, bool WINDOW, int NW>
__global__ __launch_bounds__(64 * NW) void attn_fwd_f8_kernel(F8Params p)
{
    constexpr int kThreads = 64 * NW;
    constexpr int kBlockQ = kRowsPerWave * NW;
    constexpr int kRowBytes = D;                  // one fp8 row
    constexpr int kTileBytes = kBlockK * kRowBytes;
    constexpr int kUnits = 2 * kTileBytes / 16;   // 16-byte units of the K and V tiles
    constexpr int kChunks = kUnits / kThreads;
    constexpr int kDSteps = D / 64;               // 64-deep k-steps of the first product
    constexpr int kDBlocks = D / 32;
    static_assert(kChunks * kThreads == kUnits, "tile copy must split evenly");

    __shared__ __attribute__((aligned(16))) char lds_a[2][kTileBytes];  // K | V
    __shared__ __attribute__((aligned(16))) char lds_b[2][kTileBytes];

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);  // wave-uniform: derived rows and tests stay in SGPRs
    const int lane = tid % 64;
    const int l32 = lane % 32;
    const int hi = lane / 32;

    const int BH = p.B * p.H;
    const int order = blockIdx.x / BH;
    const int bh = blockIdx.x % BH;
    const int qblk = CAUSAL ? (p.n_qblk - 1 - order) : order;
    const int b = bh / p.H;
    const int h = bh % p.H;
    const int g = h / p.group;
    const int L = p.L;

    const uint8_t *qh = p.q + ((int64_t)b * p.H + h) * L * D;
    const uint8_t *kh = p.k + ((int64_t)b * p.H_kv + g) * L * D;
    const uint8_t *vh = p.v + ((int64_t)b * p.H_kv + g) * L * D;
    __bf16 *oh = p.o + ((int64_t)b * p.H + h) * L * D;
    float *lseh = p.lse + ((int64_t)b * p.H + h) * L;

    const int q_first = qblk * kBlockQ;
    const int q_last = min(L, q_first + kBlockQ) - 1;
    int kv_begin = 0, kv_end = L;
    if (WINDOW) kv_begin = max(0, q_first - p.window);
    if (CAUSAL) kv_end = q_last + 1;
    else if (WINDOW) kv_end = min(L, q_last + p.window + 1);
    const int t_first = kv_begin / kBlockK;
    const int t_last = (kv_end + kBlockK - 1) / kBlockK;

    const int qa = q_first + wave * kRowsPerWave;
    const int qb = min(qa + kRowsPerWave, L) - 1;
    const bool wave_live = qa < L;
    const int qi = qa + l32;

    // Q^T fragments: 32 contiguous d-bytes per lane per 64-deep step
    i32x8 qf[kDSteps];
#pragma unroll
    for (int s = 0; s < kDSteps; ++s) {
        if (qi < L) {
            const i32x4 *src = reinterpret_cast<const i32x4 *>(qh + (int64_t)qi * D + 64 * s + 32 * hi);
            const i32x4 lo = src[0], hi4 = src[1];
            qf[s] = __builtin_shufflevector(lo, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
        } else {
            qf[s] = i32x8{};
        }
    }

    // LDS offsets (swizzled): K rows for the A operand, two 16-byte units per
    // 64-deep step; V rows for the transposing reads
    int koff[kDSteps][2];
#pragma unroll
    for (int ds = 0; ds < kDSteps; ++ds)
#pragma unroll
        for (int sp = 0; sp < 2; ++sp) koff[ds][sp] = f8_k_frag_offset<D>(lane, ds, sp);
    int voff[kDBlocks];
#pragma unroll
    for (int db = 0; db < kDBlocks; ++db) voff[db] = f8_v_tr_offset<D>(lane, db);

    f32x16 acc_o[kDBlocks];
#pragma unroll
    for (int i = 0; i < kDBlocks; ++i) acc_o[i] = f32x16{};
    float m_run = -INFINITY;  // reference (log2 domain), -inf until a key is seen
    float neg_m = 0.f;        // 3 - m_run, or 0 while m_run is -inf
    float l_run = 0.f;        // sum of the fp32 weights, this lane half's keys

    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    int ld_off[kChunks];
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
        ld_off[c] = f8_copy_src_offset<D>((c * NW + wave) * 64 + lane);  // the unit the swizzle puts here
    }
    auto copy_tile = [&](int t, char (*stage)[kTileBytes]) {
        const int j0 = t * kBlockK;
        const int bytes = min(L - j0, kBlockK) * kRowBytes;
        const __amdgpu_buffer_rsrc_t rk =
            __builtin_amdgcn_make_buffer_rsrc((void *)(kh + (int64_t)j0 * D), 0, bytes, 0x00020000);
        const __amdgpu_buffer_rsrc_t rv =
            __builtin_amdgcn_make_buffer_rsrc((void *)(vh + (int64_t)j0 * D), 0, bytes, 0x00020000);
#pragma unroll
        for (int c = 0; c < kChunks; ++c) {
            const int region = (c * NW + wave_u) * 1024;  // wave-uniform: which tile and where
            if (region < kTileBytes)
                copy_to_lds16(rk, &stage[0][region], ld_off[c]);
            else
                copy_to_lds16(rv, &stage[1][region - kTileBytes], ld_off[c]);
        }
    };

    if (t_first < t_last) copy_tile(t_first, lds_a);

    auto process_tile = [&](int t, char (*cur)[kTileBytes], char (*nxt)[kTileBytes]) {
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        __syncthreads();
        if (t + 1 < t_last) copy_tile(t + 1, nxt);

        const int j0 = t * kBlockK;
        const int j_last = j0 + kBlockK - 1;
        bool skip = !wave_live;
        if (CAUSAL) skip = skip || j0 > qb;
        if (WINDOW) {
            skip = skip || j_last < qa - p.window;
            if (!CAUSAL) skip = skip || j0 > qb + p.window;
        }
        if (skip) return;
        bool full = j_last < L;
        if (CAUSAL) full = full && j_last <= qa;
        if (WINDOW) {
            full = full && j0 >= qb - p.window;
            if (!CAUSAL) full = full && j_last <= qa + p.window;
        }

        const char *tk = cur[0];
        const char *tv = cur[1];
        f32x16 s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            s[kb] = f32x16{};
#pragma unroll
            for (int ds = 0; ds < kDSteps; ++ds) {
                const i32x4 lo = *reinterpret_cast<const i32x4 *>(tk + 32 * kb * kRowBytes + koff[ds][0]);
                const i32x4 hi4 = *reinterpret_cast<const i32x4 *>(tk + 32 * kb * kRowBytes + koff[ds][1]);
                s[kb] = mfma_f8(__builtin_shufflevector(lo, hi4, 0, 1, 2, 3, 4, 5, 6, 7), qf[ds], s[kb]);
            }
        }
        if (!full) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int j = j0 + 32 * kb + 16 * (r / 8) + 8 * hi + (r % 8);
                    if (!visible<CAUSAL, WINDOW>(qi, j, L, p.window)) s[kb][r] = -INFINITY;
                }
        }

        // weights against the reference + 3; fp32 sum; fp8 pack
        f32x16 w[2];
        float l_tile = 0.f;
        auto weights = [&]() {
            float part[4];  // four interleaved fp32 sums, each started from a weight
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    w[kb][r] = __builtin_amdgcn_exp2f(fmaf(s[kb][r], p.scale_log2, neg_m));
                    part[r % 4] = (kb == 0 && r < 4) ? w[0][r] : part[r % 4] + w[kb][r];
                }
            l_tile = (part[0] + part[1]) + (part[2] + part[3]);
        };
        weights();
        if (__any(!(l_tile <= kF8Max) || m_run == -INFINITY)) {
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
                neg_m = (m_new == -INFINITY) ? 0.f : kF8Shift - m_new;
                weights();
            }
        }
        l_run += l_tile;

        // P^T as the B operand: bytes 0..15 from block 0 registers 0..15, 16..31 from block 1
        i32x8 pf;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
                pf[4 * kb + q4] = pack4_f8(w[kb][4 * q4], w[kb][4 * q4 + 1], w[kb][4 * q4 + 2], w[kb][4 * q4 + 3]);

        // O^T += V^T P^T: per d block, four transposing reads (one per 8-key run)
#pragma unroll
        for (int db = 0; db < kDBlocks; ++db) {
            i32x8 vf;
#pragma unroll
            for (int rho = 0; rho < 4; ++rho) {
                const int kb = rho / 2, tt = rho % 2;
                const i32x2 x = lds_read_tr8(tv + (32 * kb + 16 * tt) * kRowBytes + voff[db]);
                vf[2 * rho] = x[0];
                vf[2 * rho + 1] = x[1];
            }
            acc_o[db] = mfma_f8(vf, pf, acc_o[db]);
        }
    };

    for (int t = t_first; t < t_last; t += 2) {
        process_tile(t, lds_a, lds_b);
        if (t + 1 < t_last) process_tile(t + 1, lds_b, lds_a);
    }

    // ---- epilogue: O/l in bf16, lse = (m - 3 + log2 l) ln 2
    if (!wave_live || qi >= L) return;
    const float l_tot = half_swap_sum(l_run);
    const float inv = 1.f / l_tot;
    if (hi == 0) lseh[qi] = (m_run - kF8Shift + __log2f(l_tot)) * 0.69314718055994531f;
    __bf16 *orow = oh + (int64_t)qi * D;
#pragma unroll
    for (int db = 0; db < kDBlocks; ++db)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            __bf16 outv[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) outv[c] = (__bf16)(acc_o[db][4 * a + c] * inv);
            *reinterpret_cast<uint64_t *>(orow + 32 * db + 8 * a + 4 * hi) = *reinterpret_cast<const uint64_t *>(outv);
        }
}

// ------------------------------------------------------------------ host side

template <int D, bool CAUSAL, bool WINDOW, int NW>
hipError_t launch_f8(F8Params p, hipStream_t stream)
{
    p.n_qblk = (p.L + kRowsPerWave * NW - 1) / (kRowsPerWave * NW);
    void *kargs[] = {&p};
    return hipLaunchKernel(reinterpret_cast<const void *>(&attn_fwd_f8_kernel<D, CAUSAL, WINDOW, NW>),
                           dim3((unsigned)((int64_t)p.n_qblk * p.B * p.H)), dim3(64 * NW), kargs, 0, stream);
}

template <int D, bool CAUSAL, bool WINDOW>
hipError_t launch_f8_shape(const F8Params &p, hipStream_t stream)
{
    // 8 waves (256 rows) once the grid of 256-row blocks fills the GPU twice
    const int64_t g8 = (int64_t)(p.L + 255) / 256 * p.B * p.H;
    return g8 >= 512 ? launch_f8<D, CAUSAL, WINDOW, 8>(p, stream) : launch_f8<D, CAUSAL, WINDOW, 4>(p, stream);
}

template <int D>
hipError_t launch_f8_mask(const F8Params &p, bool causal, bool window, hipStream_t stream)
{
    if (causal)
        return window ? launch_f8_shape<D, true, true>(p, stream) : launch_f8_shape<D, true, false>(p, stream);
    return window ? launch_f8_shape<D, false, true>(p, stream) : launch_f8_shape<D, false, false>(p, stream);
}

}  // namespace

extern "C" int attn_fwd_fp8(const void *q, const void *k, const void *v, void *out, float *lse, int B, int H,
                            int H_kv, int L, int d, int causal, int window, float scale, void *stream)
{
    if (B < 0 || L < 0 || H < 1 || H_kv < 1 || H % H_kv != 0) return ATTN_ERR_SHAPE;
    if (d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
    if (window < -1) return ATTN_ERR_WINDOW;
    if (causal != 0 && causal != 1) return ATTN_ERR_FLAG;
    if (std::isinf(scale)) return ATTN_ERR_SCALE;
    if (B == 0 || L == 0) return ATTN_OK;
    if (!q || !k || !v || !out || !lse) return ATTN_ERR_NULL;
    if (((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v) |
          reinterpret_cast<uintptr_t>(out)) & 15) ||
        (reinterpret_cast<uintptr_t>(lse) & 3))
        return ATTN_ERR_ALIGN;
    const unsigned __int128 rows_q = (unsigned __int128)B * H * L;
    const unsigned __int128 rows_kv = (unsigned __int128)B * H_kv * L;
    if (rows_q * d * 2 >= ((unsigned __int128)1 << 62)) return ATTN_ERR_SIZE;
    const size_t bytes_q = (size_t)(rows_q * d);        // fp8 q
    const size_t bytes_kv = (size_t)(rows_kv * d);
    const size_t bytes_o = (size_t)(rows_q * d * 2);    // bf16 out
    const size_t bytes_lse = (size_t)(rows_q * sizeof(float));
    if ((int64_t)((L + 127) / 128) * B * H > INT_MAX) return ATTN_ERR_SIZE;
    if (overlaps(out, bytes_o, q, bytes_q) || overlaps(out, bytes_o, k, bytes_kv) ||
        overlaps(out, bytes_o, v, bytes_kv) || overlaps(out, bytes_o, lse, bytes_lse) ||
        overlaps(lse, bytes_lse, q, bytes_q) || overlaps(lse, bytes_lse, k, bytes_kv) ||
        overlaps(lse, bytes_lse, v, bytes_kv))
        return ATTN_ERR_ALIAS;

    F8Params p;
    p.q = static_cast<const uint8_t *>(q);
    p.k = static_cast<const uint8_t *>(k);
    p.v = static_cast<const uint8_t *>(v);
    p.o = static_cast<__bf16 *>(out);
    p.lse = lse;
    p.B = B;
    p.H = H;
    p.H_kv = H_kv;
    p.L = L;
    p.group = H / H_kv;
    p.window = window;
    p.n_qblk = 0;
    p.scale_log2 = attn_resolve_scale(scale, d) * 1.4426950408889634f;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const bool win = window >= 0;
    const hipError_t err = d == 64 ? launch_f8_mask<64>(p, causal, win, s) : launch_f8_mask<128>(p, causal, win, s);
    return err == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH;
}
