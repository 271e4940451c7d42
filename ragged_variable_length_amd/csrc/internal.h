// internal.h -- kernel launch descriptors shared by the library's translation
// units (api.hip calls the launchers defined in pack.hip and attention.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rattn {

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
// keeps the workgroup within 40 KiB so four fit on one CU).
constexpr int kMaxFusedN = 2048;

// Packs with a single launch when B*N is at most this many tokens (each
// workgroup then derives its own output offset from the mask); above it a
// one-workgroup scan runs first and the gather reads cu_seqlens.
constexpr int kSelfScanMaxTokens = 16384;

hipError_t launch_pack(const PackArgs &a, hipStream_t s);
hipError_t launch_unpack(const UnpackArgs &a, hipStream_t s);
hipError_t launch_attention(const AttnArgs &a, hipStream_t s);
hipError_t launch_fused(const FusedArgs &a, hipStream_t s);

}  // namespace rattn
