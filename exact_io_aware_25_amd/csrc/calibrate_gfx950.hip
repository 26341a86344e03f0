// calibrate_gfx950.hip -- checks and measurements of the gfx950 features the
// attention kernel relies on.  Not part of the library.
//
//   calibrate_gfx950 --check   verify lane layouts (exit status 0 = all hold):
//       * ds_read_b64_tr_b16: within each 16-lane group, lane 4a+b receives
//         element b of the 8-byte chunks addressed by lanes a, a+4, a+8, a+12;
//       * v_permlane32_swap(x, x): first result = x of lane l%32, second =
//         x of lane l%32 + 32;
//       * buffer_load_dwordx4 ... lds: lane i's 16 bytes land at M0 + 16*i,
//         read from lane i's own offset, and out-of-range lanes write zeros;
//       * v_mfma_f32_16x16x32_f16 as the forward's row-sum product: with the
//         0/1 selector as A and lane 16g + n holding 8 values as B, register 0
//         of lane 16G + n is the sum of the 16 values of lanes 16g + n with
//         g & 1 == G & 1 (the lanes of one query in the 32x32 layout);
//       and reports (without failing) which SIMD each wave of an 8-wave
//       workgroup runs on (HW_REG_HW_ID bits 5:4): --rates places its two
//       wave roles on shared SIMDs by assuming waves w and w+4 share one.
//   calibrate_gfx950 --rates   issue rates per SIMD, no memory traffic:
//       MFMA 32x32x16 f16 alone, the softmax VALU mix of one 64-key tile
//       alone, both in one wave, and one MFMA wave beside one VALU wave on
//       every SIMD;
//       then the cost of single instructions (8 independent chains per
//       wave) with 1 and 4 waves per SIMD, and 4 MFMAs with 16 independent
//       FMAs of the same wave between them.
//   calibrate_gfx950 --fp8acc  how exactly one v_mfma_scale_f32_32x32x64_f8f6f4
//       (E4M3, unit scales) sums its 64 products: its 32x32 results against
//       the exact sums, for small random values, for one large product among
//       small ones, and for two large products that cancel.
//   calibrate_gfx950 --read    HBM read rate of a plain kernel over 3.3 GB,
//       the data read in 4 KiB blocks in order and in a random order (the
//       access pattern of a paged KV cache), with default and with
//       non-temporal loads.
//   calibrate_gfx950 --atomics fp32 atomic adds as an atomic dQ would issue
//       them in the backward at causal L = 131072, H = 4, d = 64: one
//       workgroup per 128-key block and head adds a 64 x 64 fp32 tile into dQ
//       for every 64-row query tile whose rows see its keys (1.72e10 adds,
//       no return value); the time, the adds per second, and a check of every
//       sum.
//
// Every memory access stays inside the buffers it is given.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <vector>

#define CHECK_HIP(x)                                                                  \
    do {                                                                              \
        hipError_t e_ = (x);                                                          \
        if (e_ != hipSuccess) {                                                       \
            std::printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            return 2;                                                                 \
        }                                                                             \
    } while (0)

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

// ------------------------------------------------------------------ wave placement
// SIMD of each wave of the workgroup: HW_REG_HW_ID (register 4), bits 5:4.
__global__ void simd_of_wave(int *out)
{
    const unsigned simd = __builtin_amdgcn_s_getreg((1 << 11) | (4 << 6) | 4);
    if (threadIdx.x % 64 == 0) out[blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64] = (int)simd;
}

// ------------------------------------------------------------------ layout checks
// One wave.  lds holds 1024 shorts; lane addresses stay below 2 KiB - 8 bytes.
__global__ void tr16_layout(short *out)
{
    __shared__ short lds[1024];
    const int lane = threadIdx.x;
    for (int i = lane; i < 1024; i += 64) lds[i] = (short)i;
    __syncthreads();
    const int byte_addr = (lane % 16) * 64 + (lane / 16) * 8;  // 16 rows of 64 B, 4 column chunks
    auto p = (__attribute__((address_space(3))) s16x4 *)((__attribute__((address_space(3))) char *)lds + byte_addr);
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p);
    for (int e = 0; e < 4; ++e) out[lane * 4 + e] = v[e];
}

__global__ void swap_layout(int *out)
{
    const int lane = threadIdx.x;
    const unsigned x = 1000 + lane;
    auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    out[lane * 2] = r[0];
    out[lane * 2 + 1] = r[1];
}

__device__ __forceinline__ void copy16(__amdgpu_buffer_rsrc_t src, void *lds_dst, int off)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (__attribute__((address_space(3))) void *)lds_dst, 16, off, 0, 0, 0);
}

// src: 64 chunks of 16 bytes; lane reads chunk (5*lane)%64; the resource
// covers `records` bytes, so lanes whose chunk lies past it read zeros.
__global__ void dma_layout(const unsigned *src, unsigned *out, int records)
{
    __shared__ __attribute__((aligned(16))) unsigned lds[1024];
    const int lane = threadIdx.x;
    for (int i = lane; i < 1024; i += 64) lds[i] = 0xdeadbeefu;
    __syncthreads();
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void *)src, 0, records, 0x00020000);
    copy16(r, lds + 256, ((5 * lane) % 64) * 16);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    for (int i = lane; i < 1024; i += 64) out[i] = lds[i];
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

// One wave: the forward's row-sum product on known B values.
__global__ void rowsum_layout(float *out)
{
    const int lane = threadIdx.x;
    const int m = lane % 16, g = lane / 16;
    const _Float16 one = (m % 4 == 0 && (g & 1) == ((m >> 2) & 1)) ? (_Float16)1 : (_Float16)0;
    f16x8 a, b;
    for (int j = 0; j < 8; ++j) {
        a[j] = one;
        b[j] = (_Float16)((lane * 8 + j) % 61);
    }
    const f32x4 d = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, f32x4{}, 0, 0, 0);
    out[lane] = d[0];
}

static int run_checks()
{
    int failures = 0;
    short *d_s;
    int *d_i;
    unsigned *d_src, *d_out;
    CHECK_HIP(hipMalloc(&d_s, 256 * sizeof(short)));
    CHECK_HIP(hipMalloc(&d_i, 128 * sizeof(int)));
    CHECK_HIP(hipMalloc(&d_src, 256 * sizeof(unsigned)));
    CHECK_HIP(hipMalloc(&d_out, 1024 * sizeof(unsigned)));

    hipLaunchKernelGGL(tr16_layout, dim3(1), dim3(64), 0, 0, d_s);
    CHECK_HIP(hipDeviceSynchronize());
    std::vector<short> hs(256);
    CHECK_HIP(hipMemcpy(hs.data(), d_s, 256 * sizeof(short), hipMemcpyDeviceToHost));
    for (int lane = 0; lane < 64; ++lane) {
        const int grp = lane / 16, a = (lane % 16) / 4, b = lane % 4;
        for (int c = 0; c < 4; ++c) {
            const int src_lane = 16 * grp + a + 4 * c;
            const int want = (src_lane % 16) * 32 + (src_lane / 16) * 4 + b;  // element b of that lane's chunk
            if (hs[lane * 4 + c] != want) ++failures;
        }
    }
    std::printf("ds_read_b64_tr_b16 layout: %s\n", failures ? "MISMATCH" : "ok");

    const int before_swap = failures;
    hipLaunchKernelGGL(swap_layout, dim3(1), dim3(64), 0, 0, d_i);
    CHECK_HIP(hipDeviceSynchronize());
    std::vector<int> hi(128);
    CHECK_HIP(hipMemcpy(hi.data(), d_i, 128 * sizeof(int), hipMemcpyDeviceToHost));
    for (int lane = 0; lane < 64; ++lane)
        if (hi[2 * lane] != 1000 + lane % 32 || hi[2 * lane + 1] != 1000 + lane % 32 + 32) ++failures;
    std::printf("v_permlane32_swap layout: %s\n", failures > before_swap ? "MISMATCH" : "ok");

    std::vector<unsigned> src(256);
    for (int i = 0; i < 256; ++i) src[i] = i;
    CHECK_HIP(hipMemcpy(d_src, src.data(), 256 * sizeof(unsigned), hipMemcpyHostToDevice));
    std::vector<unsigned> ho(1024);
    for (int records : {64 * 16, 32 * 16}) {
        const int before = failures;
        hipLaunchKernelGGL(dma_layout, dim3(1), dim3(64), 0, 0, d_src, d_out, records);
        CHECK_HIP(hipDeviceSynchronize());
        CHECK_HIP(hipMemcpy(ho.data(), d_out, 1024 * sizeof(unsigned), hipMemcpyDeviceToHost));
        for (int i = 0; i < 1024; ++i) {
            unsigned want = 0xdeadbeefu;
            if (i >= 256 && i < 512) {
                const int lane = (i - 256) / 4, word = (i - 256) % 4;
                const int chunk = (5 * lane) % 64;
                want = chunk * 16 < records ? (unsigned)(4 * chunk + word) : 0u;
            }
            if (ho[i] != want) ++failures;
        }
        std::printf("buffer_load ... lds placement (%d-byte range): %s\n", records,
                    failures > before ? "MISMATCH" : "ok");
    }
    {
        const int before = failures;
        float *d_f;
        CHECK_HIP(hipMalloc(&d_f, 64 * sizeof(float)));
        hipLaunchKernelGGL(rowsum_layout, dim3(1), dim3(64), 0, 0, d_f);
        CHECK_HIP(hipDeviceSynchronize());
        std::vector<float> hf(64);
        CHECK_HIP(hipMemcpy(hf.data(), d_f, 64 * sizeof(float), hipMemcpyDeviceToHost));
        CHECK_HIP(hipFree(d_f));
        for (int lane = 0; lane < 64; ++lane) {
            const int G = lane / 16, n = lane % 16;
            int want = 0;
            for (int g = 0; g < 4; ++g)
                if ((g & 1) == (G & 1))
                    for (int j = 0; j < 8; ++j) want += ((16 * g + n) * 8 + j) % 61;
            if (hf[lane] != (float)want) ++failures;
        }
        std::printf("v_mfma_f32_16x16x32_f16 row-sum selector layout: %s\n", failures > before ? "MISMATCH" : "ok");
    }
    // wave placement (reported, not checked): 16 workgroups of 8 waves
    hipLaunchKernelGGL(simd_of_wave, dim3(16), dim3(512), 0, 0, d_i);
    CHECK_HIP(hipDeviceSynchronize());
    CHECK_HIP(hipMemcpy(hi.data(), d_i, 128 * sizeof(int), hipMemcpyDeviceToHost));
    bool pairs = true;
    for (int b = 0; b < 16; ++b) {
        int seen = 0;
        for (int w = 0; w < 4; ++w) {
            pairs = pairs && hi[8 * b + w] == hi[8 * b + w + 4];
            seen |= 1 << hi[8 * b + w];
        }
        pairs = pairs && seen == 15;
    }
    std::printf("wave placement, workgroup 0, SIMD of waves 0..7: %d %d %d %d %d %d %d %d; waves w and w+4 "
                "share a SIMD, waves 0..3 on four SIMDs, in all 16 workgroups: %s\n",
                hi[0], hi[1], hi[2], hi[3], hi[4], hi[5], hi[6], hi[7], pairs ? "yes" : "NO");
    CHECK_HIP(hipFree(d_s));
    CHECK_HIP(hipFree(d_i));
    CHECK_HIP(hipFree(d_src));
    CHECK_HIP(hipFree(d_out));
    std::printf("%s\n", failures ? "CHECKS FAILED" : "all checks passed");
    return failures ? 1 : 0;
}

// ------------------------------------------------------------------ issue rates
// MODE 0: 16 MFMA per iteration (4 independent accumulators)
// MODE 1: softmax VALU mix of one wave-tile (32 fma+exp2, 16 cvt, 16 dot2)
// MODE 2: both, in every wave
// MODE 3: the first half of the waves MFMA only, the second half VALU only
//         (waves w and w+4 share a SIMD, so at 2 waves per SIMD every SIMD
//         holds one wave of each kind)
template <int MODE>
__global__ void rates(float *out, int iters, long long *cycles)
{
    const int wave = threadIdx.x / 64;
    f16x8 a, b;
    for (int i = 0; i < 8; ++i) {
        a[i] = (_Float16)(threadIdx.x * 1e-4f);
        b[i] = (_Float16)1e-3f;
    }
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {}, s0, s1;
    for (int i = 0; i < 16; ++i) {
        s0[i] = threadIdx.x * 1e-3f + i;
        s1[i] = -i * 1e-2f;
    }
    float acc = 0.f;
    const bool first_half = wave < (int)blockDim.x / 128;
    const bool do_mfma = MODE == 0 || MODE == 2 || (MODE == 3 && first_half);
    const bool do_valu = MODE == 1 || MODE == 2 || (MODE == 3 && !first_half);
    const long long t0 = clock64();
    for (int it = 0; it < iters; ++it) {
        if (do_mfma) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c0, 0, 0, 0);
                c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c1, 0, 0, 0);
                c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c2, 0, 0, 0);
                c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c3, 0, 0, 0);
            }
        }
        if (do_valu) {
            float part[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                f32x8 pf;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    pf[e] = __builtin_amdgcn_exp2f(fmaf(ks < 2 ? s0[8 * (ks % 2) + e] : s1[8 * (ks % 2) + e], 0.18f, acc));
                const f16x8 pv = __builtin_convertvector(pf, f16x8);
                const f16x2 one = {1, 1};
                float t = __builtin_amdgcn_fdot2(__builtin_shufflevector(pv, pv, 0, 1), one, 0.f, false);
                t = __builtin_amdgcn_fdot2(__builtin_shufflevector(pv, pv, 2, 3), one, t, false);
                t = __builtin_amdgcn_fdot2(__builtin_shufflevector(pv, pv, 4, 5), one, t, false);
                part[ks] = __builtin_amdgcn_fdot2(__builtin_shufflevector(pv, pv, 6, 7), one, t, false);
            }
            acc = ((part[0] + part[1]) + (part[2] + part[3])) * 1e-12f;
            s0[0] += acc;
        }
    }
    const long long t1 = clock64();
    float r = acc;
    for (int i = 0; i < 16; ++i) r += c0[i] + c1[i] + c2[i] + c3[i] + s0[i] + s1[i];
    out[blockIdx.x * blockDim.x + threadIdx.x] = r;
    if (threadIdx.x % 64 == 0 && blockIdx.x == 0) cycles[threadIdx.x / 64] = t1 - t0;  // every wave of block 0
}

template <int MODE>
static int time_mode(const char *name, int waves_per_simd, int cus, float *out, long long *cyc)
{
    const int threads = 256 * waves_per_simd, iters = 1000;
    hipLaunchKernelGGL(rates<MODE>, dim3(cus), dim3(threads), 0, 0, out, iters, cyc);
    hipEvent_t e0, e1;
    CHECK_HIP(hipEventCreate(&e0));
    CHECK_HIP(hipEventCreate(&e1));
    CHECK_HIP(hipEventRecord(e0));
    hipLaunchKernelGGL(rates<MODE>, dim3(cus), dim3(threads), 0, 0, out, iters, cyc);
    CHECK_HIP(hipEventRecord(e1));
    CHECK_HIP(hipEventSynchronize(e1));
    float ms = 0;
    CHECK_HIP(hipEventElapsedTime(&ms, e0, e1));
    long long c[16] = {};
    CHECK_HIP(hipMemcpy(c, cyc, sizeof c, hipMemcpyDeviceToHost));
    const double mfma_waves = MODE == 0 || MODE == 2 ? threads / 64.0 : (MODE == 3 ? threads / 128.0 : 0.0);
    const double tflops = mfma_waves * 16 * 32768.0 * iters * cus / (ms * 1e-3) / 1e12;
    std::printf("%-44s waves/SIMD %d  %8.3f ms  %7.1f clocks/iteration (wave 0)  MFMA %7.1f TFLOP/s", name,
                waves_per_simd, ms, (double)c[0] / iters, tflops);
    // MODE 3: wave 0 runs MFMAs, wave threads/128 (on the same SIMD) the VALU mix
    if (MODE == 3) std::printf("  VALU wave %7.1f clocks/iteration", (double)c[threads / 128] / iters);
    std::printf("\n");
    CHECK_HIP(hipEventDestroy(e0));
    CHECK_HIP(hipEventDestroy(e1));
    return 0;
}

// ------------------------------------------------------------------ MFMA on random operands
// 16 MFMA 32x32x16 f16 per iteration (4 accumulators), the A and B operands
// taken in turn from 8 fragments per lane of N(0,1) fp16 values (read once
// from `src`, 64 lanes x 8 fragments x 8 halves per wave), so the operand
// bits change from one instruction to the next as they do in the attention
// kernel.  MFMA power, and so the clock, depends on those bits.
__global__ void mfma_random(const f16x8 *src, float *out, int iters, long long *cycles)
{
    const int lane = threadIdx.x % 64;
    f16x8 frag[8];
    for (int i = 0; i < 8; ++i) frag[i] = src[(threadIdx.x / 64 % 4) * 512 + i * 64 + lane];
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    const long long t0 = clock64();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(frag[2 * i], frag[2 * i + 1], c0, 0, 0, 0);
            c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(frag[(2 * i + 2) % 8], frag[(2 * i + 5) % 8], c1, 0, 0, 0);
            c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(frag[(2 * i + 4) % 8], frag[(2 * i + 1) % 8], c2, 0, 0, 0);
            c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(frag[(2 * i + 6) % 8], frag[(2 * i + 7) % 8], c3, 0, 0, 0);
        }
    }
    const long long t1 = clock64();
    float r = 0.f;
    for (int i = 0; i < 16; ++i) r += c0[i] + c1[i] + c2[i] + c3[i];
    out[blockIdx.x * blockDim.x + threadIdx.x] = r;
    if (threadIdx.x == 0 && blockIdx.x == 0) cycles[0] = t1 - t0;
}

static int time_mfma_random(int waves_per_simd, int cus, float *out, long long *cyc)
{
    // 4 waves' worth of fragments (2048 x 8 halves), N(0,1) by Box-Muller on a
    // seeded 64-bit LCG, rounded to fp16; waves w and w+4 share a set
    std::vector<_Float16> h(4 * 512 * 8);
    unsigned long long st = 2024;
    auto uni = [&]() {
        st = st * 6364136223846793005ULL + 1442695040888963407ULL;
        return ((st >> 11) + 0.5) * (1.0 / 9007199254740992.0);
    };
    for (size_t i = 0; i < h.size(); i += 2) {
        const double r = std::sqrt(-2.0 * std::log(uni())), t = 6.283185307179586 * uni();
        h[i] = (_Float16)(r * std::cos(t));
        h[i + 1] = (_Float16)(r * std::sin(t));
    }
    f16x8 *src;
    CHECK_HIP(hipMalloc(&src, h.size() * sizeof(_Float16)));
    CHECK_HIP(hipMemcpy(src, h.data(), h.size() * sizeof(_Float16), hipMemcpyHostToDevice));
    const int threads = 256 * waves_per_simd, iters = 1000;
    hipLaunchKernelGGL(mfma_random, dim3(cus), dim3(threads), 0, 0, src, out, iters, cyc);
    CHECK_HIP(hipDeviceSynchronize());
    hipEvent_t e0, e1;
    CHECK_HIP(hipEventCreate(&e0));
    CHECK_HIP(hipEventCreate(&e1));
    CHECK_HIP(hipEventRecord(e0));
    for (int r = 0; r < 20; ++r)
        hipLaunchKernelGGL(mfma_random, dim3(cus), dim3(threads), 0, 0, src, out, iters, cyc);
    CHECK_HIP(hipEventRecord(e1));
    CHECK_HIP(hipEventSynchronize(e1));
    float ms = 0;
    CHECK_HIP(hipEventElapsedTime(&ms, e0, e1));
    ms /= 20;
    const double tflops = threads / 64.0 * 16 * 32768.0 * iters * cus / (ms * 1e-3) / 1e12;
    std::printf("%-44s waves/SIMD %d  %8.3f ms  MFMA %7.1f TFLOP/s\n", "16 MFMA 32x32x16 f16, N(0,1) operands",
                waves_per_simd, ms, tflops);
    CHECK_HIP(hipFree(src));
    CHECK_HIP(hipEventDestroy(e0));
    CHECK_HIP(hipEventDestroy(e1));
    return 0;
}

// ------------------------------------------------------------------ single instructions
// OP 0: v_exp_f32; 1: v_fma_f32; 2: v_cvt_pk_f16_f32; 3: v_dot2c_f32_f16;
// 4: 4 MFMA 32x32x16 f16 with 16 independent v_fma_f32 between them;
// 5: v_exp_f16 on the low half, then its SDWA form on the high half of the
// same register, keeping the other half (a pair of fp16 weights in place).
// 8 independent dependency chains per wave; each iteration issues 8 of the
// instruction (OP 4: 4 MFMAs and 16 FMAs).  Registers only.
template <int OP>
__global__ void op_rate(float *out, int iters, long long *cycles)
{
    float x[8];
    for (int i = 0; i < 8; ++i) x[i] = 1e-3f * (threadIdx.x + i);
    f16x8 a;
    for (int i = 0; i < 8; ++i) a[i] = (_Float16)(1e-3f * i);
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    const f16x2 one = {1, 1};
    const long long t0 = clock64();
    for (int it = 0; it < iters; ++it) {
        if (OP == 4) {
            c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, a, c0, 0, 0, 0);
            for (int i = 0; i < 4; ++i) x[i] = fmaf(x[i], 0.999f, 1e-3f);
            c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, a, c1, 0, 0, 0);
            for (int i = 4; i < 8; ++i) x[i] = fmaf(x[i], 0.999f, 1e-3f);
            c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, a, c2, 0, 0, 0);
            for (int i = 0; i < 4; ++i) x[i] = fmaf(x[i], 0.999f, 1e-3f);
            c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, a, c3, 0, 0, 0);
            for (int i = 4; i < 8; ++i) x[i] = fmaf(x[i], 0.999f, 1e-3f);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if (OP == 0) x[i] = __builtin_amdgcn_exp2f(-x[i]);
                if (OP == 1) x[i] = fmaf(x[i], 0.999f, 1e-3f);
                if (OP == 2) {
                    const f16x2 h = __builtin_convertvector((float __attribute__((ext_vector_type(2)))){x[i], x[(i + 1) % 8]}, f16x2);
                    x[i] = __builtin_bit_cast(float, h);
                }
                if (OP == 3) x[i] = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, x[(i + 1) % 8]), one, x[i], false);
                if (OP == 5)
                    asm volatile("v_exp_f16 %0, %0\n\t"
                                 "v_exp_f16_sdwa %0, %0 dst_sel:WORD_1 dst_unused:UNUSED_PRESERVE src0_sel:WORD_1"
                                 : "+v"(x[i]));
            }
        }
    }
    const long long t1 = clock64();
    float r = 0.f;
    for (int i = 0; i < 8; ++i) r += x[i];
    for (int i = 0; i < 16; ++i) r += c0[i] + c1[i] + c2[i] + c3[i];
    out[blockIdx.x * blockDim.x + threadIdx.x] = r;
    if (threadIdx.x % 64 == 0) cycles[blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64] = t1 - t0;
}

template <int OP>
static int time_op(const char *name, int waves_per_simd, int cus, float *out, long long *cyc)
{
    const int threads = 256 * waves_per_simd, iters = 2000;
    hipLaunchKernelGGL(op_rate<OP>, dim3(cus), dim3(threads), 0, 0, out, iters, cyc);
    CHECK_HIP(hipDeviceSynchronize());
    hipLaunchKernelGGL(op_rate<OP>, dim3(cus), dim3(threads), 0, 0, out, iters, cyc);
    CHECK_HIP(hipDeviceSynchronize());
    // the slowest wave's cycles: with several waves per SIMD the oldest one
    // runs ahead, and only the last one to finish shows what the SIMD does
    const int n = cus * threads / 64;
    std::vector<long long> c(n);
    CHECK_HIP(hipMemcpy(c.data(), cyc, sizeof(long long) * n, hipMemcpyDeviceToHost));
    long long slowest = 0;
    for (long long v : c) slowest = v > slowest ? v : slowest;
    const double per_wave = (double)slowest / iters / (OP == 4 ? 1 : OP == 5 ? 16 : 8);
    std::printf("%-44s waves/SIMD %d  %7.2f clocks per %s per wave (slowest wave), %6.2f per SIMD\n", name,
                waves_per_simd, per_wave, OP == 4 ? "iteration" : "instruction", per_wave / waves_per_simd);
    return 0;
}

static int run_rates()
{
    hipDeviceProp_t prop;
    CHECK_HIP(hipGetDeviceProperties(&prop, 0));
    const int cus = prop.multiProcessorCount;
    std::printf("device %s (%s), %d CUs, max clock %.2f GHz\n", prop.name, prop.gcnArchName, cus,
                prop.clockRate * 1e-6);
    float *out;
    long long *cyc;
    CHECK_HIP(hipMalloc(&out, (size_t)cus * 1024 * sizeof(float)));
    CHECK_HIP(hipMalloc(&cyc, (size_t)cus * 16 * sizeof(long long)));  // one per wave, up to 16 per CU
    int rc = 0;
    rc |= time_mode<0>("16 MFMA 32x32x16 f16", 1, cus, out, cyc);
    rc |= time_mode<1>("softmax VALU mix of one 64-key tile", 1, cus, out, cyc);
    rc |= time_mode<1>("softmax VALU mix of one 64-key tile", 4, cus, out, cyc);
    rc |= time_mode<2>("both in every wave", 1, cus, out, cyc);
    rc |= time_mode<2>("both in every wave", 2, cus, out, cyc);
    rc |= time_mode<3>("MFMA-only wave beside VALU-only wave, one SIMD", 2, cus, out, cyc);
    rc |= time_mfma_random(1, cus, out, cyc);
    rc |= time_mfma_random(2, cus, out, cyc);
    for (int w : {1, 4}) {
        rc |= time_op<0>("v_exp_f32", w, cus, out, cyc);
        rc |= time_op<1>("v_fma_f32", w, cus, out, cyc);
        rc |= time_op<2>("v_cvt_pk_f16_f32", w, cus, out, cyc);
        rc |= time_op<3>("v_dot2c_f32_f16", w, cus, out, cyc);
        rc |= time_op<5>("v_exp_f16 (low half, then SDWA high half)", w, cus, out, cyc);
    }
    rc |= time_op<4>("4 MFMA (128 clocks) + 16 independent fma", 1, cus, out, cyc);
    CHECK_HIP(hipFree(out));
    CHECK_HIP(hipFree(cyc));
    return rc;
}

// ------------------------------------------------------------------ fp8 MFMA sums
typedef int i32x8 __attribute__((ext_vector_type(8)));

// One wave: lane l holds 32 E4M3 bytes of A row l%32 and of B column l%32 (k
// bytes 32*(l/32)..+31 of each; the instruction pairs A and B bytes by lane
// half and byte position), C = 0; result register r of lane l is
// C[8*(r/4) + 4*(l/32) + r%4][l%32].
__global__ void fp8_mfma_once(const i32x8 *a, const i32x8 *b, float *c)
{
    const int lane = threadIdx.x;
    const f32x16 r = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[lane], b[lane], f32x16{}, 0, 0, 0, 127, 0, 127);
    for (int i = 0; i < 16; ++i) c[lane * 16 + i] = r[i];
}

static double e4m3_value(unsigned char x)
{
    const int sgn = x >> 7, e = (x >> 3) & 15, m = x & 7;
    const double v = e == 0 ? m * std::ldexp(1.0, -9) : (8 + m) * std::ldexp(1.0, e - 10);
    return sgn ? -v : v;
}

static unsigned char e4m3_nearest(double v)  // by search: exact for the values used here
{
    unsigned char best = 0;
    for (int x = 0; x < 256; ++x) {
        if ((x & 0x7f) == 0x7f) continue;  // NaN patterns
        if (std::fabs(e4m3_value((unsigned char)x) - v) < std::fabs(e4m3_value(best) - v)) best = (unsigned char)x;
    }
    return best;
}

static int run_fp8acc()
{
    unsigned long long st = 77;
    auto uni = [&]() {
        st = st * 6364136223846793005ULL + 1442695040888963407ULL;
        return ((st >> 11) + 0.5) * (1.0 / 9007199254740992.0);
    };
    std::vector<unsigned char> A(64 * 32), Bm(64 * 32);  // lane-major: lane l's 32 bytes
    i32x8 *da, *db;
    float *dc;
    CHECK_HIP(hipMalloc(&da, 64 * sizeof(i32x8)));
    CHECK_HIP(hipMalloc(&db, 64 * sizeof(i32x8)));
    CHECK_HIP(hipMalloc(&dc, 64 * 16 * sizeof(float)));
    const char *names[3] = {"random |x| < 1", "one product 240*6 among small ones", "240*6 - 240*6 among small ones"};
    for (int cs = 0; cs < 3; ++cs) {
        for (int l = 0; l < 64; ++l)
            for (int k = 0; k < 32; ++k) {
                A[l * 32 + k] = e4m3_nearest((uni() - 0.5) * 1.0);
                Bm[l * 32 + k] = e4m3_nearest((uni() - 0.5) * 1.0);
            }
        if (cs >= 1)
            for (int l = 0; l < 32; ++l) {  // byte 0 of lane half 0 of every row and column
                A[l * 32] = e4m3_nearest(240.0);
                Bm[l * 32] = e4m3_nearest(6.0);
                if (cs == 2) {  // and byte 0 of lane half 1: -240 * 6
                    A[(l + 32) * 32] = e4m3_nearest(-240.0);
                    Bm[(l + 32) * 32] = e4m3_nearest(6.0);
                }
            }
        CHECK_HIP(hipMemcpy(da, A.data(), A.size(), hipMemcpyHostToDevice));
        CHECK_HIP(hipMemcpy(db, Bm.data(), Bm.size(), hipMemcpyHostToDevice));
        hipLaunchKernelGGL(fp8_mfma_once, dim3(1), dim3(64), 0, 0, da, db, dc);
        CHECK_HIP(hipDeviceSynchronize());
        std::vector<float> c(64 * 16);
        CHECK_HIP(hipMemcpy(c.data(), dc, c.size() * sizeof(float), hipMemcpyDeviceToHost));
        double max_err = 0, max_mag = 0;
        for (int l = 0; l < 64; ++l)
            for (int r = 0; r < 16; ++r) {
                const int row = 8 * (r / 4) + 4 * (l / 32) + r % 4, col = l % 32;
                double exact = 0, mag = 0;
                for (int h = 0; h < 2; ++h)
                    for (int k = 0; k < 32; ++k) {
                        const double t = e4m3_value(A[(row + 32 * h) * 32 + k]) * e4m3_value(Bm[(col + 32 * h) * 32 + k]);
                        exact += t;
                        mag = std::max(mag, std::fabs(t));
                    }
                max_err = std::max(max_err, std::fabs((double)c[l * 16 + r] - exact));
                max_mag = std::max(max_mag, mag);
            }
        std::printf("fp8 MFMA, %-36s largest |product| %8.3f, max |result - exact sum| %.3e (%.2e of it)\n",
                    names[cs], max_mag, max_err, max_err / max_mag);
    }
    CHECK_HIP(hipFree(da));
    CHECK_HIP(hipFree(db));
    CHECK_HIP(hipFree(dc));
    return 0;
}

// ------------------------------------------------------------------ HBM read rate
// Wave w reads 4 KiB blocks order[w*per .. w*per+per-1] (entries past nblk
// are skipped), 16 bytes per lane per load (each load 1 KiB contiguous);
// one word per lane is written.  NT: the loads carry the non-temporal hint.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
template <bool NT>
__global__ __launch_bounds__(256) void read_blocks(const u32x4 *x, const int *order, int per, int nblk, unsigned *out)
{
    const int w = blockIdx.x * 4 + threadIdx.x / 64, lane = threadIdx.x % 64;
    unsigned acc = 0;
    for (int i = 0; i < per; ++i) {
        const int bi = w * per + i;
        if (bi >= nblk) break;
        const int64_t blk = order[bi];
        u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const u32x4 *src = x + blk * 256 + u * 64 + lane;
            v[u] = NT ? __builtin_nontemporal_load(src) : *src;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) acc ^= v[u].x ^ v[u].w;
    }
    out[w * 64 + lane] = acc;
}

static int run_read()
{
    const int nblk = 810652;  // 3.32 GB
    const int waves = 4096;
    const int per = (nblk + waves - 1) / waves;
    u32x4 *x;
    unsigned *out;
    int *order;
    CHECK_HIP(hipMalloc(&x, (size_t)nblk * 4096));
    CHECK_HIP(hipMalloc(&out, sizeof(unsigned) * 64 * waves));
    CHECK_HIP(hipMalloc(&order, sizeof(int) * nblk));
    CHECK_HIP(hipMemset(x, 1, (size_t)nblk * 4096));
    std::vector<int> h(nblk);
    for (int pass = 0; pass < 4; ++pass) {
        const bool nt = pass >= 2;
        auto kernel = nt ? read_blocks<true> : read_blocks<false>;
        for (int i = 0; i < nblk; ++i) h[i] = i;
        if (pass % 2 == 1) {  // seeded Fisher-Yates shuffle (64-bit LCG)
            unsigned long long st = 12345;
            for (int i = nblk - 1; i > 0; --i) {
                st = st * 6364136223846793005ULL + 1442695040888963407ULL;
                const int j = (int)((st >> 33) % (unsigned long long)(i + 1));
                const int t = h[i];
                h[i] = h[j];
                h[j] = t;
            }
        }
        CHECK_HIP(hipMemcpy(order, h.data(), sizeof(int) * nblk, hipMemcpyHostToDevice));
        hipLaunchKernelGGL(kernel, dim3(waves / 4), dim3(256), 0, 0, x, order, per, nblk, out);
        CHECK_HIP(hipDeviceSynchronize());
        hipEvent_t e0, e1;
        CHECK_HIP(hipEventCreate(&e0));
        CHECK_HIP(hipEventCreate(&e1));
        CHECK_HIP(hipEventRecord(e0));
        for (int r = 0; r < 10; ++r)
            hipLaunchKernelGGL(kernel, dim3(waves / 4), dim3(256), 0, 0, x, order, per, nblk, out);
        CHECK_HIP(hipEventRecord(e1));
        CHECK_HIP(hipEventSynchronize(e1));
        float ms = 0;
        CHECK_HIP(hipEventElapsedTime(&ms, e0, e1));
        ms /= 10;
        std::printf("read %.2f GB as 4 KiB blocks, %-6s order, %-12s loads: %.3f ms  %.0f GB/s\n", nblk * 4096e-9,
                    pass % 2 ? "random" : "linear", nt ? "non-temporal" : "default", ms,
                    nblk * 4096.0 / (ms * 1e-3) / 1e9);
    }
    CHECK_HIP(hipFree(x));
    CHECK_HIP(hipFree(out));
    CHECK_HIP(hipFree(order));
    return 0;
}

// ------------------------------------------------------------------ fp32 atomics
// Workgroup (h, kb) adds 1 to every element of the 64 x 64 tiles qt >= 2 kb
// of head h; element i of a tile is added by thread i % 256.
__global__ __launch_bounds__(256) void dq_atomics(float *dq, int n_qtiles, int kblocks)
{
    const int kb = blockIdx.x % kblocks;
    const int h = blockIdx.x / kblocks;
    float *dqh = dq + (int64_t)h * n_qtiles * 4096;
    for (int qt = 2 * kb; qt < n_qtiles; ++qt) {
        float *tile = dqh + (int64_t)qt * 4096;
#pragma unroll
        for (int i = 0; i < 16; ++i)
            __hip_atomic_fetch_add(tile + i * 256 + threadIdx.x, 1.0f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

static int run_atomics()
{
    const int H = 4, n_qtiles = 131072 / 64, kblocks = 131072 / 128;
    const size_t n = (size_t)H * n_qtiles * 4096;
    float *dq;
    CHECK_HIP(hipMalloc(&dq, n * sizeof(float)));
    double adds = 0;
    for (int kb = 0; kb < kblocks; ++kb) adds += (double)(n_qtiles - std::min(2 * kb, n_qtiles)) * 4096 * H;
    std::vector<float> h(n);
    int bad = 0;
    for (int rep = 0; rep < 3; ++rep) {
        CHECK_HIP(hipMemset(dq, 0, n * sizeof(float)));
        CHECK_HIP(hipDeviceSynchronize());
        hipEvent_t e0, e1;
        CHECK_HIP(hipEventCreate(&e0));
        CHECK_HIP(hipEventCreate(&e1));
        CHECK_HIP(hipEventRecord(e0));
        hipLaunchKernelGGL(dq_atomics, dim3(H * kblocks), dim3(256), 0, 0, dq, n_qtiles, kblocks);
        CHECK_HIP(hipEventRecord(e1));
        CHECK_HIP(hipEventSynchronize(e1));
        float ms = 0;
        CHECK_HIP(hipEventElapsedTime(&ms, e0, e1));
        CHECK_HIP(hipMemcpy(h.data(), dq, n * sizeof(float), hipMemcpyDeviceToHost));
        for (size_t i = 0; i < n; ++i) {
            const int qt = (int)(i / 4096 % n_qtiles);
            if (h[i] != (float)std::min(qt / 2 + 1, kblocks)) ++bad;
        }
        std::printf("fp32 atomic adds, atomic-dQ pattern of causal 128k H=4 d=64: %.3g adds in %.2f ms = %.3g adds/s "
                    "(%.0f GB/s of fp32 payload)\n", adds, ms, adds / (ms * 1e-3), adds * 4 / (ms * 1e-3) / 1e9);
    }
    std::printf("every sum equals the number of key blocks that add to it: %s\n", bad ? "NO" : "yes");
    CHECK_HIP(hipFree(dq));
    return bad ? 1 : 0;
}

int main(int argc, char **argv)
{
    const char *mode = argc > 1 ? argv[1] : "";
    if (std::strcmp(mode, "--check") == 0) return run_checks();
    if (std::strcmp(mode, "--rates") == 0) return run_rates();
    if (std::strcmp(mode, "--read") == 0) return run_read();
    if (std::strcmp(mode, "--fp8acc") == 0) return run_fp8acc();
    if (std::strcmp(mode, "--atomics") == 0) return run_atomics();
    std::printf("usage: %s --check | --rates | --read | --fp8acc | --atomics\n", argv[0]);
    return 2;
}
