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
constexpr int kCopyBatch = 4;  // row-copy slots per thread with their loads in flight together
constexpr int kScanThreads = 1024;
constexpr int kScanWordsBig = 8;    // 16-byte mask words per thread and round, 1024-thread scan
constexpr int kScanWordsSmall = 4;  // same, 256-thread scan inside the pack launch

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

// The nonzero bytes of a 16-byte mask word as 16 flag bits of one 32-bit
// word: byte i of dword d sets bit 8*i + 7 - d.  (Bit 7 of each byte of
// ((w & 0x7F7F7F7F) + 0x7F7F7F7F) | w is set iff that byte of w is nonzero;
// the four dwords' flags are then interleaved by shifting dword d right d.)
__device__ __forceinline__ uint32_t nonzero_flags(u32x4 x) {
    uint32_t r = 0;
#pragma unroll
    for (int d = 0; d < 4; ++d)
        r |= ((((x[d] & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | x[d]) & 0x80808080u) >> d;
    return r;
}

// The flag bits of nonzero_flags for bytes 0 .. k-1 of the word (k < 16):
// dwords d < k/4 whole, then the first k%4 bytes of dword k/4.
__device__ __forceinline__ uint32_t flags_below(int k) {
    const int D = k >> 2, rb = k & 3;
    const uint32_t whole = ((0xFF00u >> D) & 0xFFu) * 0x01010101u;
    const uint32_t part = ((1u << (8 * rb)) - 1u) & (0x80808080u >> D);
    return whole | part;
}

// cu_seqlens[0..B], max kept count and total, computed by one workgroup of NT
// threads.  The flat [B*N] mask is read as 16-byte words, WPT consecutive
// words per thread and NT*WPT words per round, all of a thread's loads issued
// before the first is used.  Each word's nonzero flags go to LDS (`flg`), and
// one block scan of the per-thread counts gives every word's exclusive prefix
// (`pre`).  The kept count before byte e is then
// pre[e/16] + popcount(flg[e/16] & flags_below(e%16)): cu[b] is that value at
// e = b*N, wherever the image boundary falls inside a word.  An image's kept
// count is the difference of its two boundary values; one whose boundaries
// lie in different rounds takes its first value from the previous round
// (`carry_v`).  No atomics, no per-byte loop, no second pass over the mask.
template <int NT, int WPT>
__device__ __forceinline__ void scan_images(const uint8_t *keep, int B, int N, int32_t *cu,
                                            int32_t *max_out, int32_t *total_out, int *pre,
                                            uint32_t *flg, int *red) {
    constexpr int TW = NT * WPT;
    __shared__ int carry_v, last_b;  // value and index of the last boundary computed
    const int tid = threadIdx.x;
    const int64_t nbytes = (int64_t)B * N;
    const int64_t nwords = (nbytes + 15) >> 4;
    const u32x4 zero4 = {0u, 0u, 0u, 0u};
    if (tid == 0) last_b = -1;
    __syncthreads();
    int carry = 0, m = 0;
    for (int64_t w0 = 0; w0 < nwords; w0 += TW) {
        // the previous round's last boundary, read before this round's first
        // barrier (it is rewritten only after that)
        const int prev_v = carry_v, prev_b = last_b;
        const int64_t wt = w0 + (int64_t)tid * WPT;
        u32x4 x[WPT];
#pragma unroll
        for (int j = 0; j < WPT; ++j) x[j] = wt + j < nwords ? load_mask_word(keep, wt + j, nbytes) : zero4;
        uint32_t fl[WPT];
        int c = 0;
#pragma unroll
        for (int j = 0; j < WPT; ++j) {
            fl[j] = nonzero_flags(x[j]);
            c += __popc(fl[j]);
        }
        int round_total;
        int run = block_exclusive_scan<NT>(c, red, &round_total);
#pragma unroll
        for (int j = 0; j < WPT; ++j) {
            pre[tid * WPT + j] = run;
            flg[tid * WPT + j] = fl[j];
            run += __popc(fl[j]);
        }
        __syncthreads();
        // kept count before byte e, for e inside this round's words
        const int64_t lo = w0 * 16, hi = min(w0 + TW, nwords) * 16;
        auto value_at = [&](int64_t e) {
            const int i = (int)((e >> 4) - w0);
            return carry + pre[i] + __popc(flg[i] & flags_below((int)(e & 15)));
        };
        // images whose first byte b*N lies in this round's words
        const int64_t b0 = (lo + N - 1) / N;
        const int64_t b_end = min((int64_t)B + 1, (hi + N - 1) / N);
        for (int64_t b = b0 + tid; b < b_end; b += NT) {
            const int v = value_at(b * N);
            cu[b] = v;
            if (b < B && (b + 1) * N < hi) m = max(m, value_at((b + 1) * N) - v);
            if (b == b0 && b > 0 && prev_b == b - 1) m = max(m, v - prev_v);  // image b-1 began earlier
            if (b == b_end - 1) {
                carry_v = v;
                last_b = (int)b;
            }
        }
        carry += round_total;
        __syncthreads();  // pre, flg and the carried boundary are rewritten next round
    }
    if (tid == 0) {
        cu[0] = 0;
        cu[B] = carry;  // also when B*N is a multiple of 16 (no word holds byte B*N)
        if (total_out) *total_out = carry;
        if (B > 0 && last_b == B - 1) m = max(m, carry - carry_v);  // the last image ends at byte B*N
    }
    m = block_max<NT>(m, red);
    if (tid == 0 && max_out) *max_out = m;
}

__global__ __launch_bounds__(kScanThreads) void scan_kernel(const uint8_t *keep, int B, int N,
                                                            int32_t *cu, int32_t *max_out,
                                                            int32_t *total_out) {
    __shared__ int pre[kScanThreads * kScanWordsBig];
    __shared__ uint32_t flg[kScanThreads * kScanWordsBig];
    __shared__ int red[kScanThreads / 64];
    scan_images<kScanThreads, kScanWordsBig>(keep, B, N, cu, max_out, total_out, pre, flg, red);
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

// Kept tokens among positions [0, cs) of one image, counted by wave 0: eight
// 64-position chunks per round, their mask loads issued together (one memory
// round trip per 512 positions), then one ballot each.
__device__ __forceinline__ int count_prefix_in_image(const uint8_t *keep_img, int cs) {
    const int lane = threadIdx.x & 63;
    int c = 0;
    for (int n0 = 0; n0 < cs; n0 += 64 * 8) {
        uint8_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int n = n0 + 64 * u + lane;
            v[u] = n < cs ? keep_img[n] : 0;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) c += __popcll(__ballot(v[u] != 0));
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
            __shared__ int pre[kPackThreads * kScanWordsSmall];
            __shared__ uint32_t flg[kPackThreads * kScanWordsSmall];
            scan_images<kPackThreads, kScanWordsSmall>(a.keep, a.B, a.N, a.cu, a.max_out,
                                                       a.total_out, pre, flg, red);
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
    copy_batched<NT, kCopyBatch, kPackThreads>(
        a.src, a.dst, total, [&](int idx, int64_t &so, int64_t &d) {
            const int j = idx / rv;
            const int e = idx - j * rv;
            so = (img_row0 + list[j]) * rv + e;
            d = (base + j) * rv + e;
        });
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
        // kCopyBatch loads of a thread in flight before its first store
        const int total = (ce - cs) * rv;
        const int64_t out0 = ((int64_t)b * a.N + cs) * rv;
        for (int i0 = tid; i0 < total; i0 += kPackThreads * kCopyBatch) {
            u32x4 x[kCopyBatch];
#pragma unroll
            for (int u = 0; u < kCopyBatch; ++u) {
                const int idx = i0 + u * kPackThreads;
                const int j = idx / rv;
                const int r = idx < total ? src_row[j] : -1;
                x[u] = r >= 0 ? a.src[(int64_t)r * rv + (idx - j * rv)] : zero;
            }
#pragma unroll
            for (int u = 0; u < kCopyBatch; ++u) {
                const int idx = i0 + u * kPackThreads;
                if (idx < total) a.dst[out0 + idx] = x[u];
            }
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
    if (tokens <= kSelfScanMaxTokens)
        return launch<pack_kernel<true, NT>>(dim3((unsigned)(wgs + 1)), dim3(kPackThreads), s, a);
    hipError_t e = launch<scan_kernel>(dim3(1), dim3(kScanThreads), s, a.keep, a.B, a.N, a.cu,
                                       a.max_out, a.total_out);
    if (e != hipSuccess) return e;
    return launch<pack_kernel<false, NT>>(dim3((unsigned)wgs), dim3(kPackThreads), s, a);
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
    return launch<unpack_kernel>(dim3((unsigned)wgs), dim3(kPackThreads), s, b);
}

}  // namespace rattn
