// bench_peaks.hip -- box-measured throughput ceilings for the roofline of the
// attention kernels.  Built into librattn_bench.so; NOT part of the product ABI.
//
// The attention's arithmetic splits between the matrix cores (the two
// contractions) and the vector ALUs (per score: the scaling fma, the exp2 and
// the bookkeeping of the online softmax).  These probes measure, on the box,
// what each can sustain:
//   * dense bf16 MFMA (v_mfma_f32_16x16x32_bf16, eight independent
//     accumulator chains per wavefront, nothing else in the loop);
//   * the per-score softmax pair, one fma feeding one v_exp_f32;
//   * v_exp_f32 alone;
//   * float32 fma (not packed: the library is built without packed-fp32
//     instruction selection);
//   * co-issue: each MFMA followed by one exp2 of an independent chain in
//     the same wavefront, and MFMA wavefronts beside wavefronts of fma/exp2
//     chains on the same SIMDs (workgroups of eight wavefronts, four of
//     each kind, one of each on every SIMD).
// Every lane runs eight independent chains, so dependent-issue latency does
// not bound the rate; each thread writes its final value, so no chain is dead.
#include <hip/hip_runtime.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kChains = 8;

__global__ __launch_bounds__(kThreads) void peak_mfma_kernel(float *out, int iters, float seed) {
    const float s = seed + 1e-3f * (float)threadIdx.x;
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(s * 1e-3f * (float)(i + 1));
        b[i] = (__bf16)(0.5f - 0.01f * (float)i);
    }
    f32x4 acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
    // The MFMA is written as an instruction with its accumulator tied to its
    // result: with the builtin, the ROCm 7.2 code generator moves every
    // loop-carried accumulator between AGPRs and VGPRs on each iteration
    // (108 v_accvgpr moves per eight MFMAs), and the loop then measures those
    // moves instead of the matrix cores.  This loop holds the eight MFMAs,
    // the counter and the branch only.
    asm volatile("s_nop 4" ::: "memory");  // vector writes of a, b, acc before their MFMA reads
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < kChains; ++c)
            asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc[c]) : "v"(a), "v"(b));
    }
    // the code generator does not know the instructions above are MFMAs, so
    // it inserts none of the wait states a vector read of their results needs
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    float r = 0.f;
#pragma unroll
    for (int c = 0; c < kChains; ++c) r += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
    out[(size_t)blockIdx.x * kThreads + threadIdx.x] = r;
}

// x <- exp2(x * c - m): x stays in (0.5, 0.57] for x in (0, 1]
__global__ __launch_bounds__(kThreads) void peak_fma_exp_kernel(float *out, int iters, float seed) {
    float x[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) x[c] = 0.5f + 1e-4f * (float)(threadIdx.x + c) + 0.f * seed;
    const float cc = 0.18033688f, m = seed;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < kChains; ++c) x[c] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[c], cc, -m));
    }
    float r = 0.f;
#pragma unroll
    for (int c = 0; c < kChains; ++c) r += x[c];
    out[(size_t)blockIdx.x * kThreads + threadIdx.x] = r;
}

// x <- exp2(-x): x stays in [0.5, 1) for x in (0, 1]
__global__ __launch_bounds__(kThreads) void peak_exp_kernel(float *out, int iters, float seed) {
    float x[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) x[c] = seed + 1e-4f * (float)(threadIdx.x + c);
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < kChains; ++c) x[c] = __builtin_amdgcn_exp2f(-x[c]);
    }
    float r = 0.f;
#pragma unroll
    for (int c = 0; c < kChains; ++c) r += x[c];
    out[(size_t)blockIdx.x * kThreads + threadIdx.x] = r;
}

// x <- x * a + b: a fixed point near 1, finite throughout
__global__ __launch_bounds__(kThreads) void peak_fma_kernel(float *out, int iters, float seed) {
    float x[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) x[c] = seed + 1e-4f * (float)(threadIdx.x + c);
    const float a = 0.999f, b = 1e-3f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < kChains; ++c) x[c] = __builtin_fmaf(x[c], a, b);
    }
    float r = 0.f;
#pragma unroll
    for (int c = 0; c < kChains; ++c) r += x[c];
    out[(size_t)blockIdx.x * kThreads + threadIdx.x] = r;
}

#define RATTN_PEAK_MFMA(acc) \
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b))

// Each MFMA of the eight chains followed by one exp2 of an independent
// float chain, in one wavefront.
__global__ __launch_bounds__(kThreads) void peak_mfma_exp_kernel(float *out, int iters, float seed) {
    const float s = seed + 1e-3f * (float)threadIdx.x;
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(s * 1e-3f * (float)(i + 1));
        b[i] = (__bf16)(0.5f - 0.01f * (float)i);
    }
    f32x4 acc[kChains];
    float x[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) {
        acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
        x[c] = s + 1e-4f * (float)c;
    }
    asm volatile("s_nop 4" ::: "memory");
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < kChains; ++c) {
            RATTN_PEAK_MFMA(acc[c]);
            x[c] = __builtin_amdgcn_exp2f(-x[c]);
        }
    }
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    float r = 0.f;
#pragma unroll
    for (int c = 0; c < kChains; ++c) r += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3] + x[c];
    out[(size_t)blockIdx.x * kThreads + threadIdx.x] = r;
}

// Workgroups of eight wavefronts (two per SIMD).  KIND 0: wavefronts 0-3 run
// the eight MFMA chains and wavefronts 4-7 two fma and one exp2 per chain
// step; KIND 1: all eight run MFMA chains; KIND 2: all eight the fma/exp2
// chains.
constexpr int kSplitThreads = 512;
template <int KIND>
__global__ __launch_bounds__(kSplitThreads) void split_kernel(float *out, int iters, float seed) {
    const int w = threadIdx.x >> 6;
    const float s = seed + 1e-3f * (float)threadIdx.x;
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(s * 1e-3f * (float)(i + 1));
        b[i] = (__bf16)(0.5f - 0.01f * (float)i);
    }
    f32x4 acc[kChains];
    float x[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) {
        acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
        x[c] = 0.5f + 1e-4f * (float)(threadIdx.x + c);
    }
    asm volatile("s_nop 4" ::: "memory");
    if (KIND == 1 || (KIND == 0 && w < 4)) {
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int c = 0; c < kChains; ++c) RATTN_PEAK_MFMA(acc[c]);
        }
    } else {
        for (int it = 0; it < iters; ++it) {
#pragma unroll
            for (int c = 0; c < kChains; ++c) {
                x[c] = __builtin_fmaf(x[c], 0.999f, 1e-3f);
                x[(c + 1) & 7] = __builtin_fmaf(x[(c + 1) & 7], 0.999f, 1e-3f);
                x[(c + 2) & 7] = __builtin_amdgcn_exp2f(-x[(c + 2) & 7]);
            }
        }
    }
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    float r = 0.f;
#pragma unroll
    for (int c = 0; c < kChains; ++c) r += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3] + x[c];
    out[(size_t)blockIdx.x * kSplitThreads + threadIdx.x] = r;
}

// Runs `kernel` on `grid` workgroups (once to warm up, then timed with HIP
// events) and returns the elapsed seconds, or a negative value on error.
template <typename K>
double timed(K kernel, int grid, int iters, float seed, float *out, hipStream_t s,
             int threads = kThreads) {
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(threads), 0, s, out, iters, seed);
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess) return -1.0;
    if (hipEventCreate(&e1) != hipSuccess) {
        (void)hipEventDestroy(e0);
        return -1.0;
    }
    (void)hipEventRecord(e0, s);
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(threads), 0, s, out, iters, seed);
    (void)hipEventRecord(e1, s);
    float ms = -1.f;
    const bool ok = hipGetLastError() == hipSuccess && hipEventSynchronize(e1) == hipSuccess &&
                    hipEventElapsedTime(&ms, e0, e1) == hipSuccess;
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    return ok ? ms * 1e-3 : -1.0;
}

}  // namespace

extern "C" {

typedef struct bench_peaks_result {
    double mfma_bf16_tflops;   // dense bf16 MFMA, TFLOP/s (2 * 16 * 16 * 32 per MFMA)
    double fma_exp_per_s;      // softmax pairs (one fma feeding one exp2) per second
    double exp_per_s;          // v_exp_f32 results per second
    double fma_f32_tflops;     // float32 fma, TFLOP/s (2 per fma)
    double mfma_ns;            // ns per MFMA per SIMD, MFMA chains alone
    double mfma_exp_ns;        // ns per (MFMA + independent exp2) per SIMD, one wavefront
    double split_mixed_s;      // MFMA wavefronts beside fma/exp2 wavefronts, seconds
    double split_mfma_s;       // the same launch, all wavefronts MFMA, seconds
    double split_valu_s;       // the same launch, all wavefronts fma/exp2, seconds
} bench_peaks_result;

// The probes on `grid` workgroups of 256 threads (a few per CU; the split
// probes on grid / 2 workgroups of 512), each thread running `iters`
// iterations of eight chains.  0 on success.
int bench_peaks(int grid, int iters, void *stream, bench_peaks_result *res) {
    if (grid < 2 || iters < 1 || !res) return 1;
    hipStream_t s = (hipStream_t)stream;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        return 2;
    float *out = nullptr;
    // the split probes run grid / 2 workgroups of 512 threads: no more lanes
    if (hipMalloc(&out, (size_t)grid * kThreads * sizeof(float)) != hipSuccess) return 2;
    const double lanes = (double)grid * kThreads;
    const double per_lane = (double)iters * kChains;
    const double t_mfma = timed(peak_mfma_kernel, grid, iters, 1.f, out, s);
    const double t_fe = timed(peak_fma_exp_kernel, grid, iters, 1.f, out, s);
    const double t_exp = timed(peak_exp_kernel, grid, iters, 0.5f, out, s);
    const double t_fma = timed(peak_fma_kernel, grid, iters, 0.5f, out, s);
    const double t_me = timed(peak_mfma_exp_kernel, grid, iters, 0.5f, out, s);
    const int g2 = grid / 2;
    const double t_mix = timed(split_kernel<0>, g2, iters, 1.f, out, s, kSplitThreads);
    const double t_smf = timed(split_kernel<1>, g2, iters, 1.f, out, s, kSplitThreads);
    const double t_sva = timed(split_kernel<2>, g2, iters, 1.f, out, s, kSplitThreads);
    const bool ok = hipFree(out) == hipSuccess && t_mfma > 0 && t_fe > 0 && t_exp > 0 && t_fma > 0 &&
                    t_me > 0 && t_mix > 0 && t_smf > 0 && t_sva > 0;
    if (!ok) return 3;
    // one MFMA per wavefront of 64 lanes per chain step
    const double mfma_per_simd = lanes / 64.0 * per_lane / (4.0 * cus);
    res->mfma_bf16_tflops = lanes / 64.0 * per_lane * 16.0 * 16.0 * 32.0 * 2.0 / t_mfma * 1e-12;
    res->fma_exp_per_s = lanes * per_lane / t_fe;
    res->exp_per_s = lanes * per_lane / t_exp;
    res->fma_f32_tflops = lanes * per_lane * 2.0 / t_fma * 1e-12;
    res->mfma_ns = t_mfma / mfma_per_simd * 1e9;
    res->mfma_exp_ns = t_me / mfma_per_simd * 1e9;
    res->split_mixed_s = t_mix;
    res->split_mfma_s = t_smf;
    res->split_valu_s = t_sva;
    return 0;
}

}  // extern "C"
