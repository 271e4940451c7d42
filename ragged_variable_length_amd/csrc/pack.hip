// pack.hip -- cu_seqlens scan, coalesced pack-gather and unpack / CLS scatter
// for gfx950.
//
// Pages on "Dispatch-Aware Ragged Attention for Pruned Vision Transformers"
// (arXiv 2604.15408), radpulse.milrad-way.com write-up, section on the
// integrated packing pipeline: compute cu_seqlens, copy the surviving tokens
// with coalesced accesses into a contiguous flat tensor, and after the blocks
// run on it, take the CLS token out.
//
// Design on CDNA4:
//  * A token's destination row is the number of kept tokens before it in the
//    flattened [B*N] mask.  A workgroup owns one (image, chunk of <= 64
//    positions); one wavefront ballot over the chunk gives every kept token
//    its rank, so ordering is stable and bit-exact with no atomics.
//  * Rows are moved as 16-byte vectors (global_load/store_dwordx4); lanes of a
//    wavefront cover consecutive 16-byte pieces of a row, so every access is a
//    full-line, coalesced transfer.  q, k and v share one mask and are copied
//    by the same workgroup in one launch.
//  * The prefix over images is either read from cu_seqlens written by a
//    one-workgroup scan launched first (large B*N), or, for small B*N, counted
//    by each workgroup from the mask itself with 16-byte loads, so that the
//    whole pack is ONE launch -- at ViT serving sizes launch count is what
//    the dispatch floor is made of.
#include "internal.h"

namespace rattn {
namespace {

constexpr int kPackThreads = 256;
constexpr int kScanThreads = 1024;
constexpr int kScanTileBig = 8192;    // image counts per LDS tile, 1024-thread scan
constexpr int kScanTileSmall = 2048;  // same, 256-thread scan inside the pack launch

__device__ __forceinline__ int nonzero_bytes(uint32_t w) {
    // bit 7 of each byte of t is set iff that byte of w is nonzero
    uint32_t t = ((w & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | w;
    return __popc(t & 0x80808080u);
}

// Block-wide exclusive prefix sum of one int per thread.  `red` is LDS scratch
// of at least NT/64 ints.  Returns the exclusive prefix; *total the block sum.
template <int NT>
__device__ int block_exclusive_scan(int v, int *red, int *total) {
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        int y = __shfl_up(x, d);
        if (lane >= d) x += y;
    }
    if (lane == 63) red[wid] = x;
    __syncthreads();
    if (wid == 0) {
        int t = lane < NW ? red[lane] : 0;
#pragma unroll
        for (int d = 1; d < NW; d <<= 1) {
            int y = __shfl_up(t, d);
            if (lane >= d) t += y;
        }
        if (lane < NW) red[lane] = t;
    }
    __syncthreads();
    const int before = wid ? red[wid - 1] : 0;
    *total = red[NW - 1];
    __syncthreads();  // red may be reused by the caller
    return before + x - v;
}

template <int NT>
__device__ int block_max(int v, int *red) {
    constexpr int NW = NT / 64;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v = max(v, __shfl_xor(v, d));
    if (lane == 0) red[wid] = v;
    __syncthreads();
    int m = red[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) m = max(m, red[i]);
    __syncthreads();
    return m;
}

template <int NT>
__device__ int block_sum(int v, int *red) {
    int total;
    block_exclusive_scan<NT>(v, red, &total);
    return total;
}

// Load the 16-byte word w of the mask, zero-filling bytes at or past `nbytes`
// (only the final word of the mask can be partial; it is read bytewise).
__device__ __forceinline__ u32x4 load_mask_word(const uint8_t *keep, int64_t w, int64_t nbytes) {
    const int64_t p = w * 16;
    if (p + 16 <= nbytes) return *(const u32x4 *)(keep + p);
    u32x4 r = {0u, 0u, 0u, 0u};
    for (int j = 0; j < 16 && p + j < nbytes; ++j)
        r[j >> 2] |= (uint32_t)keep[p + j] << (8 * (j & 3));
    return r;
}

// cu_seqlens[0..B], max kept count and total, computed by one workgroup.
// Per-image counts of a tile of images are accumulated in LDS from 16-byte
// words of the flat mask (a word may straddle image boundaries), then scanned.
template <int NT, int TILE>
__device__ void scan_images(const uint8_t *keep, int B, int N, int32_t *cu, int32_t *max_out,
                            int32_t *total_out, int *cnt, int *red) {
    const int tid = threadIdx.x;
    const int64_t nbytes = (int64_t)B * N;
    int carry = 0, mx = 0;
    if (tid == 0) cu[0] = 0;
    for (int b0 = 0; b0 < B; b0 += TILE) {
        const int nb = min(TILE, B - b0);
        for (int i = tid; i < nb; i += NT) cnt[i] = 0;
        __syncthreads();
        const int64_t lo = (int64_t)b0 * N, hi = (int64_t)(b0 + nb) * N;
        for (int64_t w = (lo >> 4) + tid; w < (hi + 15) >> 4; w += NT) {
            const u32x4 x = load_mask_word(keep, w, nbytes);
            int64_t pos = w * 16;
            int img = (int)(pos / N);
            int64_t bound = (int64_t)(img + 1) * N;
            int c = 0;
#pragma unroll
            for (int j = 0; j < 16; ++j, ++pos) {
                if (pos >= bound) {
                    if (c) atomicAdd(&cnt[img - b0], c);
                    c = 0;
                    ++img;
                    bound += N;
                }
                const uint32_t byte = (x[j >> 2] >> (8 * (j & 3))) & 0xFFu;
                if (pos >= lo && pos < hi) c += byte != 0u;
            }
            if (c) atomicAdd(&cnt[img - b0], c);
        }
        __syncthreads();
        // each thread scans a contiguous segment of the tile's counts
        const int seg = (nb + NT - 1) / NT;
        const int i0 = min(nb, tid * seg), i1 = min(nb, i0 + seg);
        int s = 0, m = 0;
        for (int i = i0; i < i1; ++i) {
            s += cnt[i];
            m = max(m, cnt[i]);
        }
        int tile_total;
        int run = carry + block_exclusive_scan<NT>(s, red, &tile_total);
        for (int i = i0; i < i1; ++i) {
            run += cnt[i];
            cu[b0 + i + 1] = run;
        }
        mx = max(mx, block_max<NT>(m, red));
        carry += tile_total;
        __syncthreads();  // cnt is reused by the next tile
    }
    if (tid == 0) {
        if (max_out) *max_out = mx;
        if (total_out) *total_out = carry;
    }
}

__global__ __launch_bounds__(kScanThreads) void scan_kernel(const uint8_t *keep, int B, int N,
                                                            int32_t *cu, int32_t *max_out,
                                                            int32_t *total_out) {
    __shared__ int cnt[kScanTileBig];
    __shared__ int red[kScanThreads / 64];
    scan_images<kScanThreads, kScanTileBig>(keep, B, N, cu, max_out, total_out, cnt, red);
}

// Rank the kept tokens of positions [cs, ce) of image b with one ballot.
// Wave 0 writes list[r] = position of the r-th kept token; returns the count
// (valid in wave 0 only).
__device__ __forceinline__ int rank_chunk(const uint8_t *keep_img, int cs, int ce, int *list) {
    const int lane = threadIdx.x & 63;
    const int n = cs + lane;
    const bool kept = n < ce && keep_img[n] != 0;
    const uint64_t m = __ballot(kept);
    if (kept) list[__popcll(m & ((1ull << lane) - 1ull))] = n;
    return __popcll(m);
}

// Kept tokens among positions [0, cs) of one image, counted by wave 0.
__device__ __forceinline__ int count_prefix_in_image(const uint8_t *keep_img, int cs) {
    const int lane = threadIdx.x & 63;
    int c = 0;
    for (int n0 = 0; n0 < cs; n0 += 64) {
        const int n = n0 + lane;
        c += __popcll(__ballot(n < cs && keep_img[n] != 0));
    }
    return c;
}

template <bool kSelfScan, int NT>
__global__ __launch_bounds__(kPackThreads) void pack_kernel(PackArgs a) {
    __shared__ int list[64];
    __shared__ int red[kPackThreads / 64];
    __shared__ int64_t s_base;
    __shared__ int s_cnt;
    int wg = blockIdx.x;
    if constexpr (kSelfScan) {
        if (wg == 0) {
            __shared__ int cnt[kScanTileSmall];
            scan_images<kPackThreads, kScanTileSmall>(a.keep, a.B, a.N, a.cu, a.max_out,
                                                      a.total_out, cnt, red);
            return;
        }
        wg -= 1;
    }
    const int b = wg / a.ch.nchunks, s = wg - b * a.ch.nchunks;
    const int cs = s * a.ch.chunk, ce = min(a.N, cs + a.ch.chunk);
    if (cs >= ce) return;
    const uint8_t *keep_img = a.keep + (int64_t)b * a.N;
    const int tid = threadIdx.x;

    int64_t base;
    if constexpr (kSelfScan) {
        // kept tokens in the flat mask before (b, cs): 16-byte words plus a tail
        const int64_t p = (int64_t)b * a.N + cs;
        int c = 0;
        for (int64_t w = tid; w < (p >> 4); w += kPackThreads) {
            const u32x4 x = *(const u32x4 *)(a.keep + w * 16);
            c += nonzero_bytes(x[0]) + nonzero_bytes(x[1]) + nonzero_bytes(x[2]) +
                 nonzero_bytes(x[3]);
        }
        const int64_t tail = (p >> 4) << 4;
        if (tid < p - tail) c += a.keep[tail + tid] != 0;
        base = block_sum<kPackThreads>(c, red);
    }
    if (tid < 64) {
        const int k = rank_chunk(keep_img, cs, ce, list);
        if constexpr (!kSelfScan) {
            const int before = count_prefix_in_image(keep_img, cs);
            if (tid == 0) s_base = (int64_t)a.cu[b] + before;
        }
        if (tid == 0) s_cnt = k;
    }
    __syncthreads();
    if constexpr (!kSelfScan) base = s_base;
    const int kc = s_cnt;
    const int rv = a.row_vec;
    const int total = kc * rv;
    const int64_t img_row0 = (int64_t)b * a.N;
    for (int idx = tid; idx < total; idx += kPackThreads) {
        const int j = idx / rv;
        const int e = idx - j * rv;
        const int64_t so = (img_row0 + list[j]) * rv + e;
        const int64_t d = (base + j) * rv + e;
        copy_vec<NT>(a.src, a.dst, so, d);
    }
}

// out[b, n] = kept ? src[rank] : 0 for the positions of one chunk; the chunk
// holding position 0 also writes the CLS row.
__global__ __launch_bounds__(kPackThreads) void unpack_kernel(UnpackArgs a) {
    __shared__ int src_row[64];
    const int wg = blockIdx.x;
    const int b = wg / a.ch.nchunks, s = wg - b * a.ch.nchunks;
    const int cs = s * a.ch.chunk, ce = min(a.N, cs + a.ch.chunk);
    if (cs >= ce) return;
    const uint8_t *keep_img = a.keep + (int64_t)b * a.N;
    const int tid = threadIdx.x;
    if (tid < 64) {
        const int before = count_prefix_in_image(keep_img, cs);
        const int n = cs + tid;
        const bool kept = n < ce && keep_img[n] != 0;
        const uint64_t m = __ballot(kept);
        const int base = a.cu[b] + before;
        if (n < ce) src_row[tid] = kept ? base + __popcll(m & ((1ull << tid) - 1ull)) : -1;
    }
    __syncthreads();
    const int rv = a.row_vec;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    if (a.dst) {
        const int total = (ce - cs) * rv;
        const int64_t out0 = ((int64_t)b * a.N + cs) * rv;
        for (int idx = tid; idx < total; idx += kPackThreads) {
            const int j = idx / rv;
            const int e = idx - j * rv;
            const int r = src_row[j];
            a.dst[out0 + idx] = r >= 0 ? a.src[(int64_t)r * rv + e] : zero;
        }
    }
    if (a.cls && cs == 0) {
        const int r = src_row[0];
        for (int e = tid; e < rv; e += kPackThreads)
            a.cls[(int64_t)b * rv + e] = r >= 0 ? a.src[(int64_t)r * rv + e] : zero;
    }
}

}  // namespace

namespace {

template <int NT>
hipError_t launch_pack_nt(const PackArgs &a, hipStream_t s) {
    const int64_t tokens = (int64_t)a.B * a.N;
    const int64_t wgs = (int64_t)a.B * a.ch.nchunks;
    if (tokens <= kSelfScanMaxTokens) {
        hipLaunchKernelGGL((pack_kernel<true, NT>), dim3((unsigned)(wgs + 1)), dim3(kPackThreads),
                           0, s, a);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kScanThreads), 0, s, a.keep, a.B, a.N, a.cu,
                       a.max_out, a.total_out);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((pack_kernel<false, NT>), dim3((unsigned)wgs), dim3(kPackThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_pack(const PackArgs &a, hipStream_t s) {
    switch (a.n_tensors) {
        case 1: return launch_pack_nt<1>(a, s);
        case 2: return launch_pack_nt<2>(a, s);
        case 3: return launch_pack_nt<3>(a, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_unpack(const UnpackArgs &a, hipStream_t s) {
    UnpackArgs b = a;
    if (!a.dst) {  // CLS rows only: one workgroup per image, first chunk only
        b.ch.nchunks = 1;
        b.ch.chunk = 1;
    }
    const int64_t wgs = (int64_t)b.B * b.ch.nchunks;
    hipLaunchKernelGGL(unpack_kernel, dim3((unsigned)wgs), dim3(kPackThreads), 0, s, b);
    return hipGetLastError();
}

}  // namespace rattn
