// internal.h -- kernel launch descriptors shared by the library's translation
// units (api.hip calls the launchers defined in pack.hip, attention.hip and
// repack.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <cstddef>
#include <cstring>

namespace rattn {

// ---------------------------------------------------------------------------
// Kernel launch.  The arguments are written straight into one kernel-argument
// block, in the kernel's parameter layout (each parameter at its natural
// alignment, in order), and the block goes to hipModuleLaunchKernel with the
// kernel's hipFunction_t, resolved once per device by hipGetFuncBySymbol: no
// per-call lookup of the kernel by its host address and no per-argument
// marshalling in the runtime, the kind of launch stub the pages credit with
// the lower dispatch floor (radpulse.milrad-way.com write-up, section on the
// 40 us Triton kernel).  Built with RATTN_LAUNCH_GGL, the launchers take the
// plain hipLaunchKernelGGL + hipGetLastError path instead (the CPU emulation
// of these sources, and the comparison of the two paths).
// ---------------------------------------------------------------------------
constexpr int kMaxDevices = 64;
constexpr size_t kMaxKernArgBytes = 512;

template <typename T> struct same_type { typedef T type; };

#if !defined(RATTN_LAUNCH_GGL)
template <auto Kernel>
hipFunction_t kernel_function() {
    static std::atomic<hipFunction_t> fn[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    hipFunction_t f = fn[dev].load(std::memory_order_acquire);
    if (!f) {
        if (hipGetFuncBySymbol(&f, reinterpret_cast<const void *>(Kernel)) != hipSuccess)
            return nullptr;
        fn[dev].store(f, std::memory_order_release);
    }
    return f;
}
#endif

template <auto Kernel, typename... P>
hipError_t launch_with(void (*)(P...), dim3 grid, dim3 block, hipStream_t s,
                       typename same_type<P>::type... args) {
#if defined(RATTN_LAUNCH_GGL)
    hipLaunchKernelGGL(Kernel, grid, block, 0, s, args...);
    return hipGetLastError();
#else
    alignas(16) unsigned char blk[kMaxKernArgBytes];
    size_t off = 0;
    ((off = (off + alignof(P) - 1) & ~(alignof(P) - 1), std::memcpy(blk + off, &args, sizeof(P)),
      off += sizeof(P)),
     ...);
    static_assert(((sizeof(P) + alignof(P)) + ... + 0) <= kMaxKernArgBytes, "kernel arguments");
    hipFunction_t f = kernel_function<Kernel>();
    if (!f) return hipErrorInvalidDeviceFunction;
    void *extra[] = {HIP_LAUNCH_PARAM_BUFFER_POINTER, blk, HIP_LAUNCH_PARAM_BUFFER_SIZE, &off,
                     HIP_LAUNCH_PARAM_END};
    return hipModuleLaunchKernel(f, grid.x, grid.y, grid.z, block.x, block.y, block.z, 0, s,
                                 nullptr, extra);
#endif
}

// launch<kernel>(grid, block, stream, arguments...): one enqueue, no sync.
template <auto Kernel, typename... A>
hipError_t launch(dim3 grid, dim3 block, hipStream_t s, A... args) {
    return launch_with<Kernel>(Kernel, grid, block, s, args...);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kMaxTensors = 3;

// Token-chunking of one image for the pack / unpack kernels: one workgroup per
// (image, chunk of <= 64 consecutive token positions), so that one wavefront
// ballot ranks a whole chunk.
struct Chunking {
    int nchunks;  // chunks per image
    int chunk;    // token positions per chunk (<= 64)
};

inline Chunking chunking_for(int N) {
    Chunking c;
    c.nchunks = (N + 63) / 64;
    c.chunk = (N + c.nchunks - 1) / c.nchunks;
    return c;
}

// Moves `total` 16-byte vector slots of NT tensors with a workgroup of
// NThreads threads: slot idx goes from vector so of each source tensor to
// vector d of the matching destination, as map(idx, so, d) sets them.  Each
// thread issues the loads of U slots (U * NT vectors in flight) before its
// first store, so a workgroup waits for one memory round trip per
// U * NThreads slots instead of per NThreads.  The destinations must not
// overlap the sources.
//
// The tensor count is a compile-time constant on purpose: behind a run-time
// branch on the count (1, 2 or 3 tensors), the gfx950 code generator of ROCm
// 7.2 structurized the three cases so that on the three-tensor path the
// register holding the second destination's base address was never written,
// and that store went to an unrelated address.
template <int NT, int U, int NThreads, typename Map>
__device__ __forceinline__ void copy_batched(const u32x4 *const (&src)[kMaxTensors],
                                             u32x4 *const (&dst)[kMaxTensors], int total,
                                             Map map) {
    static_assert(NT >= 1 && NT <= kMaxTensors, "1-3 tensors");
    for (int i0 = (int)threadIdx.x; i0 < total; i0 += NThreads * U) {
        u32x4 x[U][NT];
        int64_t dv[U];
        bool ok[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int idx = i0 + u * NThreads;
            ok[u] = idx < total;
            int64_t sv = 0;
            dv[u] = 0;
            if (ok[u]) map(idx, sv, dv[u]);
#pragma unroll
            for (int t = 0; t < NT; ++t) x[u][t] = ok[u] ? src[t][sv] : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (ok[u]) {
#pragma unroll
                for (int t = 0; t < NT; ++t) dst[t][dv[u]] = x[u][t];
            }
        }
    }
}

struct PackArgs {
    const u32x4 *src[kMaxTensors];
    u32x4 *dst[kMaxTensors];
    const uint8_t *keep;
    int32_t *cu;         // [B+1] output
    int32_t *max_out;    // nullable
    int32_t *total_out;  // nullable
    int B, N;
    int row_vec;         // 16-byte vectors per token row
    int n_tensors;
    Chunking ch;
};

struct UnpackArgs {
    const u32x4 *src;
    u32x4 *dst;          // nullable
    u32x4 *cls;          // nullable
    const uint8_t *keep;
    const int32_t *cu;
    int B, N;
    int row_vec;
    Chunking ch;
};

struct RepackArgs {
    const u32x4 *src[kMaxTensors];  // flat [>= T, row] (T = cu[B])
    u32x4 *dst[kMaxTensors];        // flat [>= T2, row]
    const uint8_t *keep2;           // [>= T], nonzero = keep the flat row
    const int32_t *cu;              // [B+1] of src
    int32_t *cu2;                   // [B+1] output
    int32_t *total_out;             // nullable
    int B;
    int row_vec;                    // 16-byte vectors per row
    int n_tensors;
    int slices;                     // workgroups per image (set by the launcher)
};

enum class Elem { F32, F16, BF16 };

struct AttnArgs {
    const void *q, *k, *v;
    void *o;
    const int32_t *cu;
    int B, H;
    int max_seqlen;
    float scale;
    Elem dt;
};

struct FusedArgs {
    const void *q, *k, *v;  // padded [B, N, H, 64]
    const uint8_t *keep;    // [B, N]
    void *out;              // padded [B, N, H, 64] (nullable)
    void *cls;              // [B, H, 64] (nullable)
    int B, N, H;
    int max_seqlen;
    int pad;                // 0: ragged; > 0: padded comparator, every image at this length
    float scale;
    Elem dt;
};

// Longest padded sequence the fused kernel accepts: its workgroups keep the
// image's kept positions as an int16 list in LDS (2048 entries = 4 KiB, which
// keeps the 64-row-tile workgroup within 40 KiB so four fit on one CU).
constexpr int kMaxFusedN = 2048;

// Packs with a single launch when B*N is at most this many tokens (each
// workgroup then derives its own output offset from the mask); above it a
// one-workgroup scan runs first and the gather reads cu_seqlens.
constexpr int kSelfScanMaxTokens = 16384;

hipError_t launch_pack(const PackArgs &a, hipStream_t s);
hipError_t launch_unpack(const UnpackArgs &a, hipStream_t s);
hipError_t launch_attention(const AttnArgs &a, hipStream_t s);
hipError_t launch_fused(const FusedArgs &a, hipStream_t s);
hipError_t launch_repack(const RepackArgs &a, hipStream_t s);

}  // namespace rattn
