// repack.hip -- compaction of an already packed ragged buffer under a second
// keep mask (a later pruning stage), for gfx950.
//
// Pages on "Dispatch-Aware Ragged Attention for Pruned Vision Transformers"
// (arXiv 2604.15408), radpulse.milrad-way.com write-up, section on the
// integrated packing pipeline: the packed buffer is kept across blocks and the
// pipeline does not depend on the pruning method -- including methods that
// prune again at later blocks.  Re-packing keeps the buffer ragged from one
// stage to the next instead of going back through the padded layout.
//
// Design on CDNA4: each image's rows are split into `slices` contiguous
// slices, one workgroup each (the host picks the count from B alone so that
// small batches still fill the chip).  A workgroup counts the kept flags of
// all rows before its slice itself (16-byte loads, SWAR byte popcount, one
// block reduction), so the whole re-pack is ONE launch with no
// inter-workgroup communication.  Its own rows are ranked 256 at a time with
// one wavefront ballot per 64 rows; the kept rows then move as 16-byte
// vectors, lanes of the workgroup covering consecutive pieces of consecutive
// rows.  The last slice of an image writes that image's new cu_seqlens
// entry.
#include <algorithm>

#include "internal.h"

namespace rattn {
namespace {

constexpr int kRepackThreads = 256;
constexpr int kRepackWaves = kRepackThreads / 64;

__device__ __forceinline__ int nonzero_bytes4(uint32_t w) {
    // bit 7 of each byte of t is set iff that byte of w is nonzero
    const uint32_t t = ((w & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | w;
    return __popc(t & 0x80808080u);
}

template <int NT>
__global__ __launch_bounds__(kRepackThreads) void repack_kernel(RepackArgs a) {
    __shared__ int red[kRepackWaves];
    __shared__ int wave_cnt[kRepackWaves];
    __shared__ int list[kRepackThreads];
    const int b = blockIdx.x / a.slices, slice = blockIdx.x - b * a.slices;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int img0 = a.cu[b], len = a.cu[b + 1] - img0;
    const int s = img0 + (int)((int64_t)len * slice / a.slices);
    const int e = img0 + (int)((int64_t)len * (slice + 1) / a.slices);

    // kept flags of rows [0, s): whole 16-byte words, then the tail bytes
    int c = 0;
    const int words = s >> 4;
    for (int w = tid; w < words; w += kRepackThreads) {
        const u32x4 x = *(const u32x4 *)(a.keep2 + (int64_t)w * 16);
        c += nonzero_bytes4(x[0]) + nonzero_bytes4(x[1]) + nonzero_bytes4(x[2]) +
             nonzero_bytes4(x[3]);
    }
    if (tid < s - (words << 4)) c += a.keep2[(words << 4) + tid] != 0;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) c += __shfl_xor(c, d);
    if (lane == 0) red[wid] = c;
    __syncthreads();
    int base = 0;
#pragma unroll
    for (int w = 0; w < kRepackWaves; ++w) base += red[w];

    // the image's own rows, 256 per round
    const int rv = a.row_vec;
    int carry = 0;
    for (int g0 = s; g0 < e; g0 += kRepackThreads) {
        const int r = g0 + tid;
        const bool kept = r < e && a.keep2[r] != 0;
        const uint64_t m = __ballot(kept);
        const int before_in_wave = __popcll(m & ((1ull << lane) - 1ull));
        if (lane == 0) wave_cnt[wid] = __popcll(m);
        __syncthreads();
        int off = 0, total = 0;
#pragma unroll
        for (int w = 0; w < kRepackWaves; ++w) {
            off += w < wid ? wave_cnt[w] : 0;
            total += wave_cnt[w];
        }
        if (kept) list[off + before_in_wave] = r;
        __syncthreads();
        const int64_t dst_row0 = (int64_t)base + carry;
        copy_batched<NT, 4, kRepackThreads>(
            a.src, a.dst, total * rv, [&](int idx, int64_t &so, int64_t &d) {
                const int j = idx / rv;
                const int p = idx - j * rv;
                so = (int64_t)list[j] * rv + p;
                d = (dst_row0 + j) * rv + p;
            });
        carry += total;
        __syncthreads();  // list and wave_cnt are rewritten by the next round
    }
    if (tid == 0 && slice == a.slices - 1) {
        if (b == 0) a.cu2[0] = 0;
        a.cu2[b + 1] = base + carry;
        if (a.total_out && b == a.B - 1) *a.total_out = base + carry;
    }
}

}  // namespace

hipError_t launch_repack(const RepackArgs &args, hipStream_t s) {
    // about 512 workgroups whatever the batch: up to 16 slices per image
    RepackArgs a = args;
    a.slices = (int)std::min<int64_t>(16, std::max<int64_t>(1, (512 + (int64_t)a.B - 1) / a.B));
    const dim3 grid((unsigned)((int64_t)a.B * a.slices)), block(kRepackThreads);
    switch (a.n_tensors) {
        case 1: return launch<repack_kernel<1>>(grid, block, s, a);
        case 2: return launch<repack_kernel<2>>(grid, block, s, a);
        case 3: return launch<repack_kernel<3>>(grid, block, s, a);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace rattn
