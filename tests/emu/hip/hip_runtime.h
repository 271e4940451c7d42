// CPU emulation shim of the subset of HIP that the rattn kernels use; test
// infrastructure only.  With it the kernel sources compile for x86 (clang++,
// AddressSanitizer), so every global and LDS access of a launch is bounds-checked
// on the CPU.
//
// One OS thread per lane; a block's threads run together, blocks run one after
// another.  Wave intrinsics exchange values through per-wave slots between two
// wave barriers.  MFMA builtins follow the documented CDNA lane layouts
// (A[row = l%16][k], B[k][col = l%16], D rows 4*(l/16)+i); global_load_lds and
// ds_read_b64_tr_b16 follow the lane mappings measured on gfx950.
#pragma once
#include <stdint.h>
#include <math.h>
#include <barrier>
#include <thread>
#include <vector>
#include <functional>
#include <atomic>
#include <cstring>
#include <cstdio>
#include <cstdlib>
#include <algorithm>

#define __global__
#define __device__
#define __host__
#define __forceinline__ inline
#define __launch_bounds__(...)
#define __shared__ static
typedef int hipError_t;
#define hipSuccess 0
#define hipErrorInvalidValue 1
typedef void *hipStream_t;
struct dim3 { unsigned x, y, z; dim3(unsigned a = 1, unsigned b = 1, unsigned c = 1) : x(a), y(b), z(c) {} };
struct emu_idx { unsigned x, y, z; };
extern thread_local emu_idx threadIdx, blockIdx;
extern thread_local dim3 blockDim, gridDim;
using std::min; using std::max;

// Barrier for the emulation's lane threads, which far outnumber the host's
// CPUs: a waiter spins briefly, then yields its CPU to the threads it waits
// for (cheaper here than sleeping on a futex and being woken per arrival).
struct EmuBarrier {
    explicit EmuBarrier(int n) : n_(n) {}
    void arrive_and_wait() {
        const unsigned g = gen_.load(std::memory_order_acquire);
        if (count_.fetch_add(1, std::memory_order_acq_rel) == n_ - 1) {
            count_.store(0, std::memory_order_relaxed);
            gen_.fetch_add(1, std::memory_order_acq_rel);
            return;
        }
        for (int spin = 0; gen_.load(std::memory_order_acquire) == g; ++spin)
            if (spin > 16) std::this_thread::yield();
    }
    int n_;
    std::atomic<int> count_{0};
    std::atomic<unsigned> gen_{0};
};

struct EmuBlock {
    int nthreads;
    EmuBarrier *block_bar;
    std::vector<EmuBarrier *> wave_bar;
    std::vector<std::vector<uint64_t>> slot;      // per wave, 2 x 64 lanes, generic 8-byte payload
};
extern EmuBlock *g_emu;
// Every lane of a wave makes the same sequence of wave exchanges, and each
// exchange uses the slot set of its parity: a lane writes set n+1 only after
// all lanes passed exchange n's barrier, i.e. finished reading set n-1, so one
// barrier per exchange suffices.
extern thread_local unsigned emu_phase;
inline unsigned emu_next_set() { return 64u * ((emu_phase++) & 1u); }

inline void __syncthreads() { g_emu->block_bar->arrive_and_wait(); }
inline int emu_lane() { return threadIdx.x & 63; }
inline int emu_wave() { return threadIdx.x >> 6; }
inline void emu_wave_sync() { g_emu->wave_bar[emu_wave()]->arrive_and_wait(); }

template <typename T> inline T emu_exchange_get(T v, int src_lane) {
    static_assert(sizeof(T) <= 8, "");
    const unsigned set = emu_next_set();
    uint64_t bits = 0; std::memcpy(&bits, &v, sizeof(T));
    g_emu->slot[emu_wave()][set + emu_lane()] = bits;
    emu_wave_sync();
    uint64_t got = g_emu->slot[emu_wave()][set + (src_lane & 63)];
    T r; std::memcpy(&r, &got, sizeof(T)); return r;
}
template <typename T> inline T __shfl_xor(T v, int m, int w = 64) { return emu_exchange_get(v, emu_lane() ^ m); }
template <typename T> inline T __shfl_up(T v, unsigned d, int w = 64) {
    int l = emu_lane(); return emu_exchange_get(v, l >= (int)d ? l - (int)d : l);
}
inline uint64_t __ballot(int pred) {
    const unsigned set = emu_next_set();
    g_emu->slot[emu_wave()][set + emu_lane()] = pred ? 1 : 0;
    emu_wave_sync();
    uint64_t m = 0;
    for (int i = 0; i < 64; ++i) if (g_emu->slot[emu_wave()][set + i]) m |= 1ull << i;
    return m;
}
inline int __popc(uint32_t x) { return __builtin_popcount(x); }
inline int __popcll(uint64_t x) { return __builtin_popcountll(x); }
inline unsigned __umul24(unsigned a, unsigned b) { return (a & 0xFFFFFFu) * (b & 0xFFFFFFu); }
inline int atomicAdd(int *p, int v) { return __atomic_fetch_add(p, v, __ATOMIC_SEQ_CST); }

typedef float emu_f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 emu_bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 emu_f16x8 __attribute__((ext_vector_type(8)));

// generic 16x16xK MFMA: each lane gives KP elements of A and of B.
// A[row = l%16][k = (l/16)*KP + j], B[k = (l/16)*KP + j][col = l%16],
// D[row = 4*(l/16) + i][col = l%16].
template <int KP>
inline emu_f32x4 emu_mfma16(const float *a, const float *b, emu_f32x4 c) {
    struct Ent { float a[8], b[8]; };
    static Ent buf[16][128];  // per wave, two sets of 64 lanes
    Ent *w = buf[emu_wave()] + emu_next_set();
    Ent &e = w[emu_lane()];
    for (int j = 0; j < KP; ++j) { e.a[j] = a[j]; e.b[j] = b[j]; }
    emu_wave_sync();
    const int l = emu_lane(), col = l & 15, g = l >> 4;
    emu_f32x4 d;
    for (int i = 0; i < 4; ++i) {
        const int row = 4 * g + i;
        double acc = 0.0;
        for (int k = 0; k < 4 * KP; ++k) {
            const int kg = k / KP, kj = k % KP;
            acc += (double)w[row + 16 * kg].a[kj] * (double)w[col + 16 * kg].b[kj];
        }
        d[i] = (float)(c[i] + acc);
    }
    return d;
}
inline emu_f32x4 emu_mfma_bf16(emu_bf16x8 a, emu_bf16x8 b, emu_f32x4 c, int, int, int) {
    float fa[8], fb[8]; for (int j = 0; j < 8; ++j) { fa[j] = (float)a[j]; fb[j] = (float)b[j]; }
    return emu_mfma16<8>(fa, fb, c);
}
inline emu_f32x4 emu_mfma_f16(emu_f16x8 a, emu_f16x8 b, emu_f32x4 c, int, int, int) {
    float fa[8], fb[8]; for (int j = 0; j < 8; ++j) { fa[j] = (float)a[j]; fb[j] = (float)b[j]; }
    return emu_mfma16<8>(fa, fb, c);
}
inline emu_f32x4 emu_mfma_f32(float a, float b, emu_f32x4 c, int, int, int) { return emu_mfma16<1>(&a, &b, c); }
#define __builtin_amdgcn_mfma_f32_16x16x32_bf16 emu_mfma_bf16
#define __builtin_amdgcn_mfma_f32_16x16x32_f16 emu_mfma_f16
#define __builtin_amdgcn_mfma_f32_16x16x4f32 emu_mfma_f32
#define __builtin_amdgcn_exp2f exp2f
#define __builtin_amdgcn_rcpf(X) (1.0f / (X))

// readfirstlane: lane 0's value (every caller passes a wave-uniform value)
template <typename T> inline T emu_readfirstlane(T v) { return emu_exchange_get(v, 0); }
#define __builtin_amdgcn_readfirstlane(X) emu_readfirstlane(X)

// v_permlane32_swap / v_permlane16_swap (gfx950): {new vdst, new vsrc} after
// swapping the upper 32 lanes of vdst with the lower 32 of vsrc, resp. the odd
// 16-lane rows of vdst with the even rows of vsrc.
typedef uint32_t emu_u32x2 __attribute__((ext_vector_type(2)));
inline emu_u32x2 emu_permlane_swap(uint32_t old, uint32_t src, int width) {
    const uint32_t o_self = old, s_self = src;
    const int l = emu_lane();
    const unsigned set = emu_next_set();
    g_emu->slot[emu_wave()][set + l] = ((uint64_t)s_self << 32) | o_self;
    emu_wave_sync();
    auto o_at = [&](int i) { return (uint32_t)(g_emu->slot[emu_wave()][set + i] & 0xFFFFFFFFu); };
    auto s_at = [&](int i) { return (uint32_t)(g_emu->slot[emu_wave()][set + i] >> 32); };
    emu_u32x2 r;
    const bool upper = (l / width) & 1;  // odd block of `width` lanes
    r[0] = upper ? s_at(l - width) : o_at(l);
    r[1] = upper ? s_at(l) : o_at(l + width);
    return r;
}
#define __builtin_amdgcn_permlane32_swap(O, S, FI, BC) emu_permlane_swap((O), (S), 32)
#define __builtin_amdgcn_permlane16_swap(O, S, FI, BC) emu_permlane_swap((O), (S), 16)

void emu_launch(dim3 grid, dim3 block, const std::function<void()> &body);
#define hipLaunchKernelGGL(K, G, Bk, SH, S, ...) emu_launch(dim3(G), dim3(Bk), [&] { K(__VA_ARGS__); })
inline hipError_t hipGetLastError() { return hipSuccess; }

// --- host API subset used by api.hip (emulation: one fake gfx950 device) ---
struct hipDeviceProp_t { char gcnArchName[256]; };
// device memory is host memory here, and launches run to completion when
// they are made, so a device-to-host copy is a memcpy and a stream is always idle
enum hipMemcpyKind { hipMemcpyHostToDevice = 1, hipMemcpyDeviceToHost = 2, hipMemcpyDeviceToDevice = 3 };
inline hipError_t hipMemcpyAsync(void *dst, const void *src, size_t n, hipMemcpyKind, hipStream_t) {
    memcpy(dst, src, n);
    return hipSuccess;
}
inline hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
inline hipError_t hipGetDeviceCount(int *n) { *n = 1; return hipSuccess; }
inline hipError_t hipGetDevice(int *d) { *d = 0; return hipSuccess; }
inline hipError_t hipGetDeviceProperties(hipDeviceProp_t *p, int) { strcpy(p->gcnArchName, "gfx950:sramecc+:xnack-"); return hipSuccess; }

// --- gfx950 data-movement builtins ---
// global_load_lds: this lane's 16 bytes land at lds + 16 * lane
inline void emu_global_load_lds(const void *g, void *lds, int size, int, int) {
    std::memcpy((char *)lds + size * emu_lane(), g, size);
}
#define __builtin_amdgcn_global_load_lds(G, L, SZ, OFF, AUX) emu_global_load_lds((const void *)(G), (void *)(L), SZ, OFF, AUX)
// ds_read_b64_tr_b16: in each 16-lane group, lane i element j = element (i%4)
// of the 4-element word addressed by lane 4*j + i/4 of the group
typedef short emu_s16x4 __attribute__((ext_vector_type(4)));
inline emu_s16x4 emu_ds_read_tr16(const void *p) {
    const uint64_t addr = (uint64_t)(uintptr_t)p;
    const unsigned set = emu_next_set();
    g_emu->slot[emu_wave()][set + emu_lane()] = addr;
    emu_wave_sync();
    const int l = emu_lane(), g0 = l & ~15, i = l & 15;
    emu_s16x4 r;
    for (int j = 0; j < 4; ++j) {
        const short *w = (const short *)(uintptr_t)g_emu->slot[emu_wave()][set + g0 + 4 * j + i / 4];
        r[j] = w[i % 4];
    }
    return r;
}
#define __builtin_amdgcn_ds_read_tr16_b64_v4i16(P) emu_ds_read_tr16((const void *)(P))
#define __builtin_amdgcn_s_waitcnt(X) ((void)0)
#define __builtin_amdgcn_sched_barrier(X) ((void)0)
#define __builtin_amdgcn_wave_barrier() emu_wave_sync()
