// attention.hip -- bidirectional ragged multi-head attention for gfx950, on the
// flat ragged buffer (rattn_forward) and fused with the pack and the unpack in
// one launch straight from / to the padded layout (rattn_fused).
//
// Pages on "Dispatch-Aware Ragged Attention for Pruned Vision Transformers"
// (arXiv 2604.15408): the abstract (attention over the variable-length token
// sets left by pruning; host dispatch is the cost to cut) and the
// radpulse.milrad-way.com write-up, sections on FlashAttention-2's dispatch
// ceiling (one flat ragged buffer plus cumulative sequence lengths), on the
// Triton bidirectional kernel (no causal mask, no KV cache, no softmax_lse
// workspace) and on the integrated packing pipeline (cu_seqlens, coalesced
// copy of the survivors, attention, CLS extract).  Per image b, head h and
// kept query row i:  o_i = sum_j softmax_j(scale * q_i . k_j) v_j  over the
// kept rows j of the same image.
//
// CDNA4 mapping (16-bit inputs):
//  * A workgroup is W wavefronts, each owning QB blocks of 16 query rows, so
//    a query tile is 16*W*QB rows (4x1: 64 rows up to 256 positions, 4x2:
//    128 rows beyond).  The query tiles of one (image, head) go to G
//    workgroups (tiles g, g+G, ...): G > 1 when the batch has fewer heads
//    than the chip has CUs, and in the flat kernel with 128-row tiles (up to
//    three per head).  Workgroup ids are laid out so that the G workgroups of
//    one (image, head) land on the same XCD (ids are dealt to the 8 XCDs
//    round-robin), keeping that head's K/V rows in one L2.
//  * Keys stream through LDS in chunks of 64, double-buffered, copied by
//    global->LDS DMA (global_load_lds_dwordx4, 16 bytes per lane straight
//    into the lane's LDS slot).  The copy of the next step's chunk is in
//    flight while the current one is computed, one barrier per step; a
//    sequence of at most two chunks stays resident.  Query rows of odd
//    256-row blocks take the chunks in reverse, so that a workgroup's tile
//    crossing such a boundary starts with the two chunks still in its
//    buffers.  16-byte pieces of each K and V row are XOR-permuted so that
//    the operand reads hit distinct banks without padding.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_16x16x32_{bf16,f16}: in the accumulator layout each lane holds
//    4 keys of ONE query, so the running max and sum are per-lane scalars (the
//    max needs two cross-lane steps per chunk, the sum none: it comes from one
//    more MFMA against an all-ones operand).
//  * The probabilities feed O^T = V^T P^T directly as the MFMA B operand;
//    V^T is read with the transposing LDS read ds_read_b64_tr_b16, its key
//    order matching the score accumulators slot for slot.
//  * Online softmax in base 2 (scores times scale*log2(e), v_exp_f32).  For
//    scale > 0 the reference max may lag the running max by 8 in log2 units:
//    the output and row sum are rescaled only when some row's max grows past
//    that, and the final division cancels whichever reference was used.
//  * With two blocks per wavefront (4x2) each wavefront copies its own Q rows
//    into LDS by the same DMA and reads its operands from there every step,
//    which keeps 32 VGPRs of current and prefetched Q rows out of the loop.
//  * Copies of keys past the sequence end read the last key's row (finite
//    values): their scores repeat a valid score, so the row max needs no
//    mask, and they are set to -inf before the exponentials, so every copy
//    runs with all lanes active.  Query rows past the end are computed on
//    zeros (4x1) or copies of the last row (4x2) and never stored.
//  * Fused path: the workgroup first ranks its image's kept tokens with one
//    wavefront ballot per 64 positions into an LDS list of positions; Q/K/V
//    rows are then copied from those positions of the padded tensors and the
//    outputs written to the same positions of the padded output.  After its
//    attention, the last workgroup of each (image, head) writes zeros to the
//    pruned rows and, when position 0 was pruned, the CLS row.
// The float32 path has the same structure on v_mfma_f32_16x16x4_f32 with
// 32-key chunks, row-padded LDS and probabilities kept in float32.
#include <algorithm>

#include "internal.h"

namespace rattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 64;        // head_dim
constexpr int kKC = 64;       // keys per LDS chunk, 16-bit path
constexpr int kKC32 = 32;     // keys per LDS chunk, float32 path
constexpr int kWaves = 4;     // wavefronts per workgroup
constexpr int kQW = 16;       // query rows per wavefront
constexpr int kQT = kWaves * kQW;
constexpr int kThreads = kWaves * 64;
constexpr int kLd32 = 68;     // LDS row pitch of the float32 path, in floats
constexpr float kLog2e = 1.4426950408889634f;

template <typename T> struct Mma;
template <> struct Mma<__bf16> {
    typedef bf16x8 v8;
    static constexpr uint32_t kOnePair = 0x3F803F80u;  // two bf16 1.0
    static __device__ __forceinline__ f32x4 run(v8 a, v8 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};
template <> struct Mma<_Float16> {
    typedef f16x8 v8;
    static constexpr uint32_t kOnePair = 0x3C003C00u;  // two fp16 1.0
    static __device__ __forceinline__ f32x4 run(v8 a, v8 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
};

// Lanes l, l^16, l^32 and l^48 hold the same query row: two lane swaps
// (v_permlane32_swap, v_permlane16_swap) give every lane the maximum of the four.
__device__ __forceinline__ float max_across_groups(float x) {
    uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    x = __builtin_elementwise_maximum(__builtin_bit_cast(float, (uint32_t)a[0]),
                                      __builtin_bit_cast(float, (uint32_t)a[1]));
    u = __builtin_bit_cast(uint32_t, x);
    const auto b = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return __builtin_elementwise_maximum(__builtin_bit_cast(float, (uint32_t)b[0]),
                                         __builtin_bit_cast(float, (uint32_t)b[1]));
}

__device__ __forceinline__ float sum_across_groups(float x) {
    uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    x = __builtin_bit_cast(float, (uint32_t)a[0]) + __builtin_bit_cast(float, (uint32_t)a[1]);
    u = __builtin_bit_cast(uint32_t, x);
    const auto b = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return __builtin_bit_cast(float, (uint32_t)b[0]) + __builtin_bit_cast(float, (uint32_t)b[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// max(a, b) as IEEE maximum (NaN-propagating, v_maximum3_f32 on gfx950):
// unlike fmaxf it needs no canonicalizing of MFMA results before the compare.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two floats rounded to nearest even and packed (v_cvt_pk_bf16_f32 /
// v_cvt_pk_f16_f32).
template <typename T>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    typedef T T2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, T2));
}

// Element offset, from the (image, head) base, of the 64-element head slice
// of kept row r: in the flat ragged buffer (rows consecutive) or in the padded
// tensor (row at its original position).  32-bit: the host checks that one
// image's rows span less than 2^31 bytes.
struct FlatRows {
    uint32_t rs;  // elements per token row
    __device__ __forceinline__ uint32_t off(int r) const { return (uint32_t)r * rs; }
};
struct PaddedRows {
    uint32_t rs;
    const int16_t *pos;  // LDS: position of the r-th kept token
    // full-rate 24-bit multiply: pos < 2^11 and rs < 2^24, and the host keeps
    // one image's rows under 2^31 bytes, so the product fits 32 bits
    __device__ __forceinline__ uint32_t off(int r) const { return __umul24((uint32_t)pos[r], rs); }
};

// LDS tiles of the 16-bit path are 64 rows x 128 bytes, written by
// global->LDS DMA (each lane's 16 bytes land at base + 16*lane) and read as
// MFMA operands.  The 16-byte pieces of each row are XOR-permuted so that the
// reads hit distinct banks: K and Q rows (read as 16-byte row slices, one row
// per lane of each group of 16) by (row >> 1) & 7, V rows (read transposed, 8
// bytes per lane) by 2 * ((row ^ row>>1) & 3).  A lane fetches from global
// memory whichever piece belongs in its LDS slot, so the permutation costs
// nothing at staging time.  On gfx950 the K/Q permutation was chosen by the
// LDS bank-conflict counter: (row ^ row>>3) & 7, which has no conflict if a
// 16-byte read is served 8 or 16 consecutive lanes at a time, left 1.8e6
// conflict cycles per 384-px forward launch (0.15e6 per operand read per
// step); (row >> 1) & 7 leaves none and took that launch from 39.1 to 38.1 us.
__device__ __forceinline__ int kpiece(int row, int p) { return p ^ ((row >> 1) & 7); }
__device__ __forceinline__ int vpiece(int row, int p) { return p ^ (((row ^ (row >> 1)) & 3) << 1); }

#define RATTN_LDS(p) ((__attribute__((address_space(3))) void *)(p))
typedef short s16x4 __attribute__((ext_vector_type(4)));

// Transposing 8-byte LDS read (ds_read_b64_tr_b16): in each group of 16
// lanes, lane i receives element (i % 4) of the 4-element words that lanes
// i/4, 4 + i/4, 8 + i/4, 12 + i/4 address.
__device__ __forceinline__ u32x2 lds_read_tr(const uint16_t *p) {
    const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4 *)(p));
    return __builtin_bit_cast(u32x2, r);
}

// s_waitcnt vmcnt(0) alone (expcnt and lgkmcnt left at their maxima): the
// global->LDS copies this wavefront issued have landed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// s_waitcnt vmcnt(N): all but the N most recent vector memory operations of
// this wavefront have completed (N < 16).
template <int N>
__device__ __forceinline__ void wait_vmem_but() {
    static_assert(N >= 0 && N < 16, "vmcnt field");
    __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// ---------------------------------------------------------------------------
// 16-bit core: the query tiles g, g+G, ... of one (image, head).  W
// wavefronts per workgroup, each owning QB blocks of 16 query rows (a tile is
// 16*QB*W rows).  The blocks of one wavefront share every K and V operand
// read from LDS, and their MFMA and softmax work is independent, so the
// wavefront always has one block's arithmetic to overlap with the other's.
// ---------------------------------------------------------------------------
// kTag only tells specializations apart: the kernels for batches of few heads
// use attend16 with kTag = 1, the same code as the other kernels' kTag = 0
// (the host compilation pass of ROCm 7.2 rejects one specialization called
// from both kernel families).
template <typename T, bool kPos, int W, int QB, typename Rows, int kTag = 0>
__device__ __forceinline__ void attend16(const uint16_t *__restrict__ qh,
                                         const uint16_t *__restrict__ kh,
                                         const uint16_t *__restrict__ vh,
                                         uint16_t *__restrict__ oh, const Rows &R, int L, int Lp,
                                         float c, int g, int G, uint16_t *sK, uint16_t *sV,
                                         uint16_t *sQ, uint16_t *__restrict__ cls_dst) {
    // Lp >= L is the length processed: L for ragged attention; for the padded
    // comparator, the padded length, whose extra keys are masked and whose
    // extra query rows are computed (on zeros, or with two blocks per
    // wavefront on copies of the last row) and discarded
    typedef typename Mma<T>::v8 V8;
    constexpr uint32_t kOneBits = Mma<T>::kOnePair;
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 15, grp = lane >> 4;
    const u32x4 zero4 = {0u, 0u, 0u, 0u};

    // Staging: a 64-key chunk is 16 DMA instructions of 8 rows (1 KB) -- 8
    // for K, 8 for V -- dealt evenly to the W wavefronts; lane l fills row
    // l/8, slot l%8 of its 8-row block.  Every instruction is issued with all
    // lanes active, so each wavefront has exactly kDmaPerWave copies in
    // flight per chunk and a partial s_waitcnt can wait for one chunk alone.
    // Keys past the sequence end copy the last key's row: finite values whose
    // scores are masked to -inf (K) and whose probability 0 makes them add
    // exactly 0 (V).
    constexpr int kRowsPerWave = QB * kQW;
    constexpr int kQT16 = W * kRowsPerWave;  // query rows per tile
    constexpr int kDmaPerWave = 16 / W;
    const int srow = lane >> 3, sslot = lane & 7;
    auto stage = [&](int chunk, int buf) {
        // the row offsets of all of this wavefront's copies first (in the
        // padded layout they are LDS reads), then the copies
        uint32_t ro[kDmaPerWave];
#pragma unroll
        for (int i = 0; i < kDmaPerWave; ++i) {
            const int idx = wid * kDmaPerWave + i;  // 0..7: K blocks, 8..15: V blocks
            ro[i] = R.off(min(chunk * kKC + 8 * (idx & 7) + srow, L - 1));
        }
#pragma unroll
        for (int i = 0; i < kDmaPerWave; ++i) {
            const int idx = wid * kDmaPerWave + i;
            const bool is_v = idx >= 8;
            const int row0 = 8 * (idx & 7);
            const int row = row0 + srow;
            uint16_t *dst = (is_v ? sV : sK) + buf * (kKC * 64) + row0 * 64;
            const uint16_t *src = is_v ? vh + ro[i] + 8 * vpiece(row, sslot)
                                       : kh + ro[i] + 8 * kpiece(row, sslot);
            __builtin_amdgcn_global_load_lds(src, RATTN_LDS(dst), 16, 0, 0);
        }
    };
    // B operand of S^T = K Q^T for block qb of query tile `tile`: row `col`
    // of the block, dims 8*grp .. +7 and 32 + 8*grp .. +7
    auto load_q = [&](int tile, u32x4 (&a)[QB], u32x4 (&b)[QB]) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const int qr = tile * kQT16 + wid * kRowsPerWave + qb * kQW + col;
            a[qb] = zero4;
            b[qb] = zero4;
            if (qr < L) {
                const uint16_t *src = qh + R.off(qr);
                a[qb] = *(const u32x4 *)(src + 8 * grp);
                b[qb] = *(const u32x4 *)(src + 32 + 8 * grp);
            }
        }
    };
    // With two blocks per wavefront the Q rows live in LDS instead of
    // registers (32 VGPRs for the current and the prefetched tile would
    // otherwise be live across the loop): each wavefront copies its own rows
    // of a query tile by global->LDS DMA, in K's swizzled layout, and reads
    // its B operands from there every step.  No other wavefront touches
    // them, so no barrier guards them; the next tile's rows are copied as
    // soon as the last chunk's S^T has read the current ones.  Rows past the
    // sequence end copy the last row (finite values, never stored).
    constexpr bool kQL = QB == 2;
    auto stage_q = [&](int tile) {
        constexpr int kQDma = kRowsPerWave / 8;
        uint32_t ro[kQDma];
#pragma unroll
        for (int i = 0; i < kQDma; ++i)
            ro[i] = R.off(min(tile * kQT16 + wid * kRowsPerWave + 8 * i + srow, L - 1));
#pragma unroll
        for (int i = 0; i < kQDma; ++i) {
            const int row0 = wid * kRowsPerWave + 8 * i;
            __builtin_amdgcn_global_load_lds(qh + ro[i] + 8 * kpiece(row0 + srow, sslot),
                                             RATTN_LDS(sQ + row0 * 64), 16, 0, 0);
        }
    };

    // This workgroup owns query tiles g, g+G, g+2G, ... of the sequence; G
    // workgroups share one (image, head).  Keys come in nch chunks of 64.
    // The work is one pipeline of steps (tile, chunk): the copy of the
    // following step's K/V chunk -- the next chunk, or chunk 0 of the next
    // tile -- and the next tile's Q rows are in flight while the current step
    // computes.  With at most two chunks the double buffer holds the whole
    // sequence, so only the first tile stages.
    const int nch = (Lp + kKC - 1) / kKC;
    const int ntile = (Lp + kQT16 - 1) / kQT16;
    if (g >= ntile) return;
    const bool resident = nch <= 2;
    // Chunk order: query rows of even 256-row blocks take the key chunks in
    // order, those of odd blocks in reverse.  Where a workgroup's
    // consecutive tiles cross such a boundary they meet at the same chunks:
    // the last two chunks of one tile, still in the double buffer, are the
    // first two of the next and are not copied again.  The order depends on
    // a row's index only, so the results do not depend on the tile shape,
    // the workgroups per head or the sequence bound.  The 64-row-tile shape
    // serves bounds up to 256 only, where every row is in block 0, so it
    // always runs in order.  Only the nreal chunks that hold kept keys are
    // reversed: the padded comparator's all-masked chunks always come last,
    // as in the ragged order, so that its bits stay those of the ragged
    // kernel.  (A resident sequence has at most 128 rows, all in order.)
    const int nreal = (L + kKC - 1) / kKC;
    auto chunk_at = [&](int tile, int i) {
        if constexpr (QB == 1) return i;
        else return (i < nreal && (((tile * kQT16) >> 8) & 1)) ? nreal - 1 - i : i;
    };
    // Tile order.  Several workgroups per head: tiles g, g+G, ...  One
    // workgroup per head with 128-row tiles: within each pair of 256-row
    // blocks the tiles go 0, 2, 1, 3, so that every tile after the first
    // starts with the two chunks the previous one ended with (the blocks
    // take the chunks in opposite orders), still in the double buffer.
    auto next_tile_of = [&](int tile) {
        if (QB == 1 || G != 1) return tile + G;
        constexpr int kOrder[4] = {0, 2, 1, 3};
        const int base = tile & ~3, pos = tile & 3;
        int i = 0;
        while (kOrder[i] != pos) ++i;
        for (++i; i < 4; ++i)
            if (base + kOrder[i] < ntile) return base + kOrder[i];
        return base + 4;  // next group (tile 0 of it, or past the end)
    };
    int t = g, idx = 0, step = 0;
    int ch = chunk_at(t, 0);
    int buf = resident ? ch : 0;
    int held[2] = {ch, -1};  // the chunk each buffer holds (streamed sequences)
    u32x4 qf0[QB], qf1[QB], qn0[QB], qn1[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) qf0[qb] = qf1[qb] = qn0[qb] = qn1[qb] = zero4;
    if constexpr (kQL) stage_q(t);
    else load_q(t, qf0, qf1);
    stage(ch, buf);
    if (resident && nch == 2) {
        // both chunks in flight at once; wait for the Q rows and chunk 0
        // only (loads complete in issue order)
        stage(1, 1);
        wait_vmem_but<kDmaPerWave>();
    } else {
        wait_vmem();
    }
    __syncthreads();

    // all-ones A operand: its product with P^T gives P's row sums
    const V8 ones = __builtin_bit_cast(V8, u32x4{kOneBits, kOneBits, kOneBits, kOneBits});
    const int vr = 4 * grp + (col >> 2);
    const int vp = (col & 3) >> 1, vhalf = 4 * (col & 1);
    constexpr float kLag = 8.f;
    // in raw units; finite even when c is so small that 8 / c overflows
    // (scale below about 1.6e-38), so that m + lag stays -inf on the first
    // chunk and the first chunk always sets the reference
    const float lag = kPos ? fminf(kLag / c, 3.4028234663852886e38f) : 0.f;
    float m[QB], mc[QB];
    f32x4 acc[QB][4], accl[QB];
    auto reset = [&]() {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            m[qb] = -INFINITY;
            mc[qb] = -INFINITY;
            accl[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) acc[qb][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    };
    reset();
    while (true) {
        int nt = t, ni = idx + 1;
        if (ni == nch) {
            nt = next_tile_of(t);
            ni = 0;
        }
        const bool has_next = nt < ntile;
        const bool next_tile = has_next && ni == 0;
        // the next step's chunk: already in a buffer, or copied into the one
        // this step does not read
        const int nc = QB == 1 ? ni : (has_next ? chunk_at(nt, ni) : ch);
        int nbuf = resident ? nc : (QB == 1 ? (step + 1) & 1 : buf ^ 1);
        bool load_next = !resident && has_next;
        if constexpr (QB == 2) {
            if (load_next && held[buf] == nc) {
                nbuf = buf;
                load_next = false;
            } else if (load_next && held[nbuf] == nc) {
                load_next = false;
            }
            if (load_next) held[nbuf] = nc;
        }
        if (load_next) stage(nc, nbuf);
        if (!kQL && next_tile) load_q(nt, qn0, qn1);

        if constexpr (QB == 1) buf = resident ? ch : (step & 1);
        const uint16_t *Ks = sK + buf * (kKC * 64);
        const uint16_t *Vs = sV + buf * (kKC * 64);
        const int valid = L - ch * kKC;    // keys of this chunk inside the sequence
        const int valid_p = Lp - ch * kKC; // keys of this chunk that are processed

        // A wavefront whose query rows all lie past the sequence end has
        // nothing to compute (it still stages and meets every barrier).
        const bool active = t * kQT16 + wid * kRowsPerWave < Lp;
        f32x4 s[QB][4];
        float mx[QB];
        if (active) {
            if constexpr (kQL) {
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    const int r = wid * kRowsPerWave + qb * kQW + col;
                    qf0[qb] = *(const u32x4 *)(sQ + r * 64 + 8 * kpiece(r, grp));
                    qf1[qb] = *(const u32x4 *)(sQ + r * 64 + 8 * kpiece(r, 4 + grp));
                }
            }
            // S^T for the 64 keys of the chunk, with each block's row maximum
            // taken as soon as its scores are done.  Every block is computed:
            // rows of keys past the end hold copies of the last key, so no
            // branch sits between the reads, their scores repeat a valid one
            // (the maximum over all 64 is the maximum over the valid keys),
            // and they are masked to -inf only before the exponentials.  Each
            // K operand serves all QB query blocks.
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) mx[qb] = -INFINITY;
#pragma unroll
            for (int blk = 0; blk < 4; ++blk) {
                const int row = 16 * blk + col;
                const u32x4 a0 = *(const u32x4 *)(Ks + row * 64 + 8 * kpiece(row, grp));
                const u32x4 a1 = *(const u32x4 *)(Ks + row * 64 + 8 * kpiece(row, 4 + grp));
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    f32x4 z = {0.f, 0.f, 0.f, 0.f};
                    z = Mma<T>::run(__builtin_bit_cast(V8, a0), __builtin_bit_cast(V8, qf0[qb]), z);
                    s[qb][blk] = Mma<T>::run(__builtin_bit_cast(V8, a1),
                                             __builtin_bit_cast(V8, qf1[qb]), z);
                    if constexpr (kPos) {
                        const float t3 = vmax(vmax(s[qb][blk][0], s[qb][blk][1]), s[qb][blk][2]);
                        mx[qb] = vmax(vmax(mx[qb], t3), s[qb][blk][3]);
                    }
                }
            }
        }
        // the Q operands of this tile have been read: copy the next tile's
        if (kQL && next_tile) stage_q(nt);
        if (active) {
            if constexpr (kPos) {
                // scale > 0: the largest score is the largest raw dot
                // product, so the reference max m is kept in raw units and
                // each probability is one fma and one exp2.  m may lag the
                // running max by up to kLag / c (probabilities up to 2^kLag):
                // the output and the row sum are rescaled only when some
                // row's max grows past that, which after the first chunk is
                // rare, and the final division cancels whichever reference
                // was used.  One test covers all blocks, on each lane's own
                // maximum: some lane's exceeds m + lag exactly when the
                // maximum over the four lanes of that query does, so the
                // cross-lane reduction runs only when rescaling.  Inside the
                // branch each query row decides for itself: only a row whose
                // own maximum passed its lag moves its reference (to that
                // maximum, exactly); every other row keeps its reference and
                // multiplies by exactly 1.  So a row's probabilities, and
                // their rounding, depend on that row's scores alone, not on
                // the other rows of the wavefront, the tile shape or the
                // sequence bound.
                bool grow = false;
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) grow = grow || mx[qb] > m[qb] + lag;
                if (__ballot(grow)) {
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) {
                        const float mxa = max_across_groups(mx[qb]);
                        const bool row_grows = mxa > m[qb] + lag;
                        const float alpha = row_grows ? fast_exp2((m[qb] - mxa) * c) : 1.f;
                        m[qb] = row_grows ? mxa : m[qb];
                        mc[qb] = m[qb] * c;
#pragma unroll
                        for (int dt = 0; dt < 4; ++dt) acc[qb][dt] *= alpha;
                        accl[qb][0] *= alpha;
                    }
                }
            }
            if (valid < kKC) {
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                    for (int blk = 0; blk < 4; ++blk)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (16 * blk + 4 * grp + i >= valid) s[qb][blk][i] = -INFINITY;
            }
            if constexpr (!kPos) {
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    // scale <= 0 (degenerate but valid): scale, then the
                    // exact running max (masked scores stay -inf)
                    float mxn = -INFINITY;
#pragma unroll
                    for (int blk = 0; blk < 4; ++blk)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float x = s[qb][blk][i] == -INFINITY ? -INFINITY : s[qb][blk][i] * c;
                            s[qb][blk][i] = x;
                            mxn = fmaxf(mxn, x);
                        }
                    mxn = max_across_groups(mxn);
                    // while every key so far is masked (a reversed tile of the
                    // padded comparator can start with such a chunk) nothing
                    // is rescaled and every probability is 0
                    const float mn = fmaxf(m[qb], mxn);
                    const float alpha = m[qb] == mn ? 1.f : fast_exp2(m[qb] - mn);
                    const float mref = mn == -INFINITY ? 0.f : mn;
                    m[qb] = mn;
#pragma unroll
                    for (int blk = 0; blk < 4; ++blk)
#pragma unroll
                        for (int i = 0; i < 4; ++i) s[qb][blk][i] = fast_exp2(s[qb][blk][i] - mref);
#pragma unroll
                    for (int dt = 0; dt < 4; ++dt) acc[qb][dt] *= alpha;
                    accl[qb][0] *= alpha;
                }
            }

            // O^T += V^T P^T.  Operand slot (lane group g, slot s) of the
            // 32-key step ks is key 32*ks + 16*(s/4) + 4*g + s%4: the key whose
            // score the lane already holds in slot s%4 of block 2*ks + s/4.
            // The V^T operand is read transposed out of row-major V: lane r of
            // group g addresses key 32*ks + 16*h + 4*g + r/4, dims 16*dt + 4*(r%4).
            // The row sums of the rounded P come from the same B operand
            // against an all-ones A operand.  Each V operand serves all QB
            // query blocks.  For scale > 0 the probabilities of each 32-key
            // half are computed here, next to the MFMAs that consume them.
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                if (ks == 0 || valid_p > 32) {
                    const int r0 = 32 * ks + vr, r1 = r0 + 16;
                    const uint16_t *v0 = Vs + r0 * 64 + vhalf;
                    const uint16_t *v1 = Vs + r1 * 64 + vhalf;
                    auto expo = [&](int qb, int blk, int i0) {
#pragma unroll
                        for (int i = i0; i < i0 + 2; ++i)
                            s[qb][blk][i] = fast_exp2(__builtin_fmaf(s[qb][blk][i], c, -mc[qb]));
                    };
                    auto pack_b = [&](int qb) {
                        u32x4 pb;
                        pb[0] = pack2<T>(s[qb][2 * ks][0], s[qb][2 * ks][1]);
                        pb[1] = pack2<T>(s[qb][2 * ks][2], s[qb][2 * ks][3]);
                        pb[2] = pack2<T>(s[qb][2 * ks + 1][0], s[qb][2 * ks + 1][1]);
                        pb[3] = pack2<T>(s[qb][2 * ks + 1][2], s[qb][2 * ks + 1][3]);
                        return __builtin_bit_cast(V8, pb);
                    };
                    if constexpr (kPos && QB == 2) {
                        // Explicit order (the compiler otherwise issues every
                        // exponential before the first MFMA, leaving the matrix
                        // pipe idle): the half's V^T operands first, then block
                        // 0's probabilities, then each of block 0's MFMAs
                        // followed by a quarter of block 1's exponentials, which
                        // run while the MFMA does.
                        u32x4 va[4];
#pragma unroll
                        for (int dt = 0; dt < 4; ++dt) {
                            const u32x2 lo = lds_read_tr(v0 + 8 * vpiece(r0, 2 * dt + vp));
                            const u32x2 hi = lds_read_tr(v1 + 8 * vpiece(r1, 2 * dt + vp));
                            va[dt] = u32x4{lo[0], lo[1], hi[0], hi[1]};
                        }
#pragma unroll
                        for (int blk = 2 * ks; blk < 2 * ks + 2; ++blk) {
                            expo(0, blk, 0);
                            expo(0, blk, 2);
                        }
                        const V8 b0 = pack_b(0);
                        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                        for (int dt = 0; dt < 4; ++dt) {
                            acc[0][dt] = Mma<T>::run(__builtin_bit_cast(V8, va[dt]), b0, acc[0][dt]);
                            expo(1, 2 * ks + (dt >> 1), 2 * (dt & 1));
                            __builtin_amdgcn_sched_barrier(0);
                        }
                        accl[0] = Mma<T>::run(ones, b0, accl[0]);
                        const V8 b1 = pack_b(1);
                        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                        for (int dt = 0; dt < 4; ++dt)
                            acc[1][dt] = Mma<T>::run(__builtin_bit_cast(V8, va[dt]), b1, acc[1][dt]);
                        accl[1] = Mma<T>::run(ones, b1, accl[1]);
                    } else {
                        if constexpr (kPos) {
#pragma unroll
                            for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                                for (int blk = 2 * ks; blk < 2 * ks + 2; ++blk) {
                                    expo(qb, blk, 0);
                                    expo(qb, blk, 2);
                                }
                        }
                        V8 b[QB];
#pragma unroll
                        for (int qb = 0; qb < QB; ++qb) b[qb] = pack_b(qb);
#pragma unroll
                        for (int dt = 0; dt < 4; ++dt) {
                            const u32x2 lo = lds_read_tr(v0 + 8 * vpiece(r0, 2 * dt + vp));
                            const u32x2 hi = lds_read_tr(v1 + 8 * vpiece(r1, 2 * dt + vp));
                            const u32x4 a = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
                            for (int qb = 0; qb < QB; ++qb)
                                acc[qb][dt] = Mma<T>::run(__builtin_bit_cast(V8, a), b[qb], acc[qb][dt]);
                        }
#pragma unroll
                        for (int qb = 0; qb < QB; ++qb) accl[qb] = Mma<T>::run(ones, b[qb], accl[qb]);
                    }
                }
            }
        }

        if ((QB == 1 ? ch : idx) == nch - 1) {
            // tile t done: normalise and store; start the next tile afresh
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const int qrow = t * kQT16 + wid * kRowsPerWave + qb * kQW + col;
                if (qrow < L) {
                    const float inv = __builtin_amdgcn_rcpf(accl[qb][0]);
                    const f32x4 *a4 = acc[qb];
                    // lane holds o[qrow][16*dt + 4*grp + i], i = 0..3
                    const u32x2 w0 = {pack2<T>(a4[0][0] * inv, a4[0][1] * inv), pack2<T>(a4[0][2] * inv, a4[0][3] * inv)};
                    const u32x2 w1 = {pack2<T>(a4[1][0] * inv, a4[1][1] * inv), pack2<T>(a4[1][2] * inv, a4[1][3] * inv)};
                    const u32x2 w2 = {pack2<T>(a4[2][0] * inv, a4[2][1] * inv), pack2<T>(a4[2][2] * inv, a4[2][3] * inv)};
                    const u32x2 w3 = {pack2<T>(a4[3][0] * inv, a4[3][1] * inv), pack2<T>(a4[3][2] * inv, a4[3][3] * inv)};
                    if (oh) {
                        uint16_t *orow = oh + R.off(qrow) + 4 * grp;
                        *(u32x2 *)(orow) = w0;
                        *(u32x2 *)(orow + 16) = w1;
                        *(u32x2 *)(orow + 32) = w2;
                        *(u32x2 *)(orow + 48) = w3;
                    }
                    if (cls_dst && qrow == 0) {
                        uint16_t *crow = cls_dst + 4 * grp;
                        *(u32x2 *)(crow) = w0;
                        *(u32x2 *)(crow + 16) = w1;
                        *(u32x2 *)(crow + 32) = w2;
                        *(u32x2 *)(crow + 48) = w3;
                    }
                }
            }
            reset();
        }
        // the next step's chunk has landed: the one staged in this step, or,
        // resident, chunk 1 staged up front
        if (load_next || (kQL && next_tile) || (resident && step == 0 && nch == 2)) wait_vmem();
        __syncthreads();
        if (!has_next) break;
        if (!kQL && next_tile) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                qf0[qb] = qn0[qb];
                qf1[qb] = qn1[qb];
            }
        }
        t = nt;
        idx = ni;
        ch = nc;
        buf = nbuf;
        ++step;
    }
}

// ---------------------------------------------------------------------------
// 16-bit core for batches of few heads: the 16-query tiles g, g+G, ... of one
// (image, head).  Wavefront w takes the tile's 64-key chunks w, w+4, ...,
// each copied by its own DMA into an LDS slab of its own (K and V in the
// swizzled layout of attend16), so a short sequence's chunks run on four
// SIMDs at once instead of one after another.  Per chunk the arithmetic is
// attend16's for one block of 16 rows: S^T on the matrix cores, the lazy
// per-row reference maximum, probabilities rounded to T, O^T and the row
// sums on the matrix cores.  The four partial states (reference maximum,
// row sum, unnormalised output) are then merged in LDS in wavefront order
// 0, 1, 2, 3.  A chunk with no key inside the sequence (the padded
// comparator's) is skipped, so padding changes nothing.
// ---------------------------------------------------------------------------
constexpr int kSlab16 = 2 * kKC * 64;  // 16-bit elements: one chunk of K and of V

template <typename T, bool kPos, typename Rows>
__device__ __forceinline__ void attend16_split(const uint16_t *__restrict__ qh,
                                               const uint16_t *__restrict__ kh,
                                               const uint16_t *__restrict__ vh,
                                               uint16_t *__restrict__ oh, const Rows &R, int L,
                                               int Lp, float c, int g, int G, uint16_t *slabs,
                                               uint16_t *__restrict__ cls_dst) {
    typedef typename Mma<T>::v8 V8;
    constexpr uint32_t kOneBits = Mma<T>::kOnePair;
    const int lane = threadIdx.x & 63;
    const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int col = lane & 15, grp = lane >> 4;
    const u32x4 zero4 = {0u, 0u, 0u, 0u};
    uint16_t *sK = slabs + wid * kSlab16, *sV = sK + kKC * 64;
    float *part = (float *)sK;  // the partial state, once the chunks are done

    // a chunk is 16 DMA instructions of 8 rows (1 KB): 8 for K, 8 for V;
    // lane l fills row l/8, slot l%8 of each 8-row block.  Keys past the
    // sequence end copy the last key's row (finite, masked or weighted 0).
    const int srow = lane >> 3, sslot = lane & 7;
    auto stage = [&](int chunk) {
        uint32_t ro[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) ro[i] = R.off(min(chunk * kKC + 8 * i + srow, L - 1));
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int row = 8 * i + srow;
            __builtin_amdgcn_global_load_lds(kh + ro[i] + 8 * kpiece(row, sslot),
                                             RATTN_LDS(sK + 8 * i * 64), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(vh + ro[i] + 8 * vpiece(row, sslot),
                                             RATTN_LDS(sV + 8 * i * 64), 16, 0, 0);
        }
    };

    const V8 ones = __builtin_bit_cast(V8, u32x4{kOneBits, kOneBits, kOneBits, kOneBits});
    const int vr = 4 * grp + (col >> 2);
    const int vp = (col & 3) >> 1, vhalf = 4 * (col & 1);
    const float lag = kPos ? fminf(8.f / c, 3.4028234663852886e38f) : 0.f;
    const int nch = (Lp + kKC - 1) / kKC;
    const int ntile = (Lp + kQW - 1) / kQW;
    for (int t = g; t < ntile; t += G) {
        // every wavefront has read the previous tile's partial states
        if (t != g) __syncthreads();
        // B operand of S^T: query row t*16 + col, dims 8*grp.. and 32 + 8*grp..
        const int qr = t * kQW + col;
        u32x4 qf0 = zero4, qf1 = zero4;
        if (qr < L) {
            const uint16_t *src = qh + R.off(qr);
            qf0 = *(const u32x4 *)(src + 8 * grp);
            qf1 = *(const u32x4 *)(src + 32 + 8 * grp);
        }
        float m = -INFINITY, mc = -INFINITY;
        f32x4 acc[4], accl = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) acc[dt] = accl;
        for (int ch = wid; ch < nch; ch += kWaves) {
            const int valid = L - ch * kKC;
            if (valid <= 0) continue;
            const int valid_p = Lp - ch * kKC;
            // this wavefront's earlier reads of the slab are done before the
            // copies overwrite it; the copies (and the Q rows) have landed
            // before the reads below
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
            stage(ch);
            wait_vmem();
            __builtin_amdgcn_wave_barrier();
            f32x4 s[4];
            float mx = -INFINITY;
#pragma unroll
            for (int blk = 0; blk < 4; ++blk) {
                const int row = 16 * blk + col;
                const u32x4 a0 = *(const u32x4 *)(sK + row * 64 + 8 * kpiece(row, grp));
                const u32x4 a1 = *(const u32x4 *)(sK + row * 64 + 8 * kpiece(row, 4 + grp));
                f32x4 z = {0.f, 0.f, 0.f, 0.f};
                z = Mma<T>::run(__builtin_bit_cast(V8, a0), __builtin_bit_cast(V8, qf0), z);
                s[blk] = Mma<T>::run(__builtin_bit_cast(V8, a1), __builtin_bit_cast(V8, qf1), z);
                if constexpr (kPos) {
                    const float t3 = vmax(vmax(s[blk][0], s[blk][1]), s[blk][2]);
                    mx = vmax(vmax(mx, t3), s[blk][3]);
                }
            }
            if constexpr (kPos) {
                // the lazy reference of attend16: a row moves its reference
                // (raw units) only when its own maximum passed it by the lag
                if (__ballot(mx > m + lag)) {
                    const float mxa = max_across_groups(mx);
                    const bool row_grows = mxa > m + lag;
                    const float alpha = row_grows ? fast_exp2((m - mxa) * c) : 1.f;
                    m = row_grows ? mxa : m;
                    mc = m * c;
#pragma unroll
                    for (int dt = 0; dt < 4; ++dt) acc[dt] *= alpha;
                    accl[0] *= alpha;
                }
            }
            if (valid < kKC) {
#pragma unroll
                for (int blk = 0; blk < 4; ++blk)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (16 * blk + 4 * grp + i >= valid) s[blk][i] = -INFINITY;
            }
            if constexpr (!kPos) {
                // scale <= 0: scale, then the exact running maximum
                float mxn = -INFINITY;
#pragma unroll
                for (int blk = 0; blk < 4; ++blk)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float x = s[blk][i] == -INFINITY ? -INFINITY : s[blk][i] * c;
                        s[blk][i] = x;
                        mxn = fmaxf(mxn, x);
                    }
                mxn = max_across_groups(mxn);
                const float mn = fmaxf(m, mxn);
                const float alpha = m == mn ? 1.f : fast_exp2(m - mn);
                const float mref = mn == -INFINITY ? 0.f : mn;
                m = mn;
#pragma unroll
                for (int blk = 0; blk < 4; ++blk)
#pragma unroll
                    for (int i = 0; i < 4; ++i) s[blk][i] = fast_exp2(s[blk][i] - mref);
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) acc[dt] *= alpha;
                accl[0] *= alpha;
            }
            // O^T += V^T P^T and the row sums, in 32-key halves, as attend16
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                if (ks == 0 || valid_p > 32) {
                    if constexpr (kPos) {
#pragma unroll
                        for (int blk = 2 * ks; blk < 2 * ks + 2; ++blk)
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                s[blk][i] = fast_exp2(__builtin_fmaf(s[blk][i], c, -mc));
                    }
                    u32x4 pb;
                    pb[0] = pack2<T>(s[2 * ks][0], s[2 * ks][1]);
                    pb[1] = pack2<T>(s[2 * ks][2], s[2 * ks][3]);
                    pb[2] = pack2<T>(s[2 * ks + 1][0], s[2 * ks + 1][1]);
                    pb[3] = pack2<T>(s[2 * ks + 1][2], s[2 * ks + 1][3]);
                    const V8 b = __builtin_bit_cast(V8, pb);
                    const int r0 = 32 * ks + vr, r1 = r0 + 16;
                    const uint16_t *v0 = sV + r0 * 64 + vhalf;
                    const uint16_t *v1 = sV + r1 * 64 + vhalf;
#pragma unroll
                    for (int dt = 0; dt < 4; ++dt) {
                        const u32x2 lo = lds_read_tr(v0 + 8 * vpiece(r0, 2 * dt + vp));
                        const u32x2 hi = lds_read_tr(v1 + 8 * vpiece(r1, 2 * dt + vp));
                        const u32x4 a = {lo[0], lo[1], hi[0], hi[1]};
                        acc[dt] = Mma<T>::run(__builtin_bit_cast(V8, a), b, acc[dt]);
                    }
                    accl = Mma<T>::run(ones, b, accl);
                }
            }
        }
        // partial state into the own slab: output block dt at 256 dt + 4 lane,
        // then the 16 reference maxima and the 16 row sums
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the slab's reads are done
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) *(f32x4 *)(part + 256 * dt + 4 * lane) = acc[dt];
        if (grp == 0) {
            part[1024 + col] = m;
            part[1040 + col] = accl[0];
        }
        __syncthreads();
        // wavefront w merges output block w (dimensions 16 w .. 16 w + 15)
        float mw[kWaves], lw[kWaves];
        f32x4 aw[kWaves];
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float *pw = (const float *)(slabs + w * kSlab16);
            mw[w] = pw[1024 + col];
            lw[w] = pw[1040 + col];
            aw[w] = *(const f32x4 *)(pw + 256 * wid + 4 * lane);
        }
        const float M = fmaxf(fmaxf(mw[0], mw[1]), fmaxf(mw[2], mw[3]));
        float l = 0.f;
        f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            // a wavefront with no valid chunk has reference -inf: weight 0
            const float f = fast_exp2(kPos ? (mw[w] - M) * c : mw[w] - M);
            l += f * lw[w];
            o += f * aw[w];
        }
        const int qrow = t * kQW + col;
        if (qrow < L) {
            const float inv = __builtin_amdgcn_rcpf(l);
            const u32x2 wv = {pack2<T>(o[0] * inv, o[1] * inv), pack2<T>(o[2] * inv, o[3] * inv)};
            if (oh) *(u32x2 *)(oh + R.off(qrow) + 16 * wid + 4 * grp) = wv;
            if (cls_dst && qrow == 0) *(u32x2 *)(cls_dst + 16 * wid + 4 * grp) = wv;
        }
    }
}

// One 32-key chunk of the float32 online softmax for the 16 query rows of a
// wavefront: the chunk's scores S^T = K Q^T (keys at or past `valid` masked),
// the running row maximum m and row sum, and O^T += V^T P^T.  Ks and Vs hold
// the chunk's K and V rows in LDS at a pitch of kLd32 floats; qf[kk] is the B
// operand Q[query col][4*kk + grp].  acc_j[i] is O^T[16*j + 4*grp + i][col].
__device__ __forceinline__ void step32(const float *Ks, const float *Vs, const float (&qf)[16],
                                       int valid, float c, float &m, float &lsum, f32x4 &acc0,
                                       f32x4 &acc1, f32x4 &acc2, f32x4 &acc3) {
    const int lane = threadIdx.x & 63, col = lane & 15, grp = lane >> 4;
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0;
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
        s0 = __builtin_amdgcn_mfma_f32_16x16x4f32(Ks[col * kLd32 + 4 * kk + grp], qf[kk], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x4f32(Ks[(16 + col) * kLd32 + 4 * kk + grp], qf[kk], s1, 0, 0, 0);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float x0 = s0[i] * c, x1 = s1[i] * c;
        if (4 * grp + i >= valid) x0 = -INFINITY;
        if (16 + 4 * grp + i >= valid) x1 = -INFINITY;
        s0[i] = x0;
        s1[i] = x1;
        mx = fmaxf(mx, fmaxf(x0, x1));
    }
    mx = max_across_groups(mx);
    const float mn = fmaxf(m, mx);
    const float alpha = fast_exp2(m - mn);
    m = mn;
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        s0[i] = fast_exp2(s0[i] - mn);
        s1[i] = fast_exp2(s1[i] - mn);
        ps += s0[i] + s1[i];
    }
    lsum = lsum * alpha + ps;
    acc0 *= alpha;
    acc1 *= alpha;
    acc2 *= alpha;
    acc3 *= alpha;
    // O^T += V^T P^T, one key per 16x16x4 step: lane group g supplies key
    // 16*blk + 4*g + i, which is exactly the score it holds in slot i
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float *v0 = Vs + (4 * grp + i) * kLd32 + col;
        const float *v1 = Vs + (16 + 4 * grp + i) * kLd32 + col;
        acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(v0[0], s0[i], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(v0[16], s0[i], acc1, 0, 0, 0);
        acc2 = __builtin_amdgcn_mfma_f32_16x16x4f32(v0[32], s0[i], acc2, 0, 0, 0);
        acc3 = __builtin_amdgcn_mfma_f32_16x16x4f32(v0[48], s0[i], acc3, 0, 0, 0);
        acc0 = __builtin_amdgcn_mfma_f32_16x16x4f32(v1[0], s1[i], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_16x16x4f32(v1[16], s1[i], acc1, 0, 0, 0);
        acc2 = __builtin_amdgcn_mfma_f32_16x16x4f32(v1[32], s1[i], acc2, 0, 0, 0);
        acc3 = __builtin_amdgcn_mfma_f32_16x16x4f32(v1[48], s1[i], acc3, 0, 0, 0);
    }
}

// ---------------------------------------------------------------------------
// float32 core: the 64-query tiles g, g+G, ... of one (image, head), 32-key
// chunks
// ---------------------------------------------------------------------------
template <typename Rows>
__device__ __forceinline__ void attend32(const float *__restrict__ q, const float *__restrict__ k,
                                         const float *__restrict__ v, float *__restrict__ o,
                                         const Rows &R, int L, int Lp, float c, int g, int G,
                                         float *sK, float *sV, float *__restrict__ cls_dst) {
    // Lp >= L: length processed (padded comparator), as in the 16-bit core
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const u32x4 zero4 = {0u, 0u, 0u, 0u};

    // staging: a chunk is 32 keys x 16 four-float vectors per tensor; thread
    // t stages vectors t and t + 256 of K and of V
    const int key_a = tid >> 4, key_b = (tid + kThreads) >> 4, c4 = tid & 15;
    u32x4 ka, kb, va, vb;
#define RATTN_LOAD32(CH)                                                               \
    {                                                                                  \
        const int k0_ = (CH) * kKC32;                                                  \
        ka = zero4; va = zero4; kb = zero4; vb = zero4;                                \
        if (k0_ + key_a < L) {                                                         \
            ka = *(const u32x4 *)(k + R.off(k0_ + key_a) + 4 * c4);                     \
            va = *(const u32x4 *)(v + R.off(k0_ + key_a) + 4 * c4);                     \
        }                                                                              \
        if (k0_ + key_b < L) {                                                         \
            kb = *(const u32x4 *)(k + R.off(k0_ + key_b) + 4 * c4);                     \
            vb = *(const u32x4 *)(v + R.off(k0_ + key_b) + 4 * c4);                     \
        }                                                                              \
    }
#define RATTN_STORE32(BUF)                                                             \
    {                                                                                  \
        float *dk_ = sK + (BUF) * (kKC32 * kLd32);                                     \
        float *dv_ = sV + (BUF) * (kKC32 * kLd32);                                     \
        *(u32x4 *)(dk_ + key_a * kLd32 + 4 * c4) = ka;                                 \
        *(u32x4 *)(dv_ + key_a * kLd32 + 4 * c4) = va;                                 \
        *(u32x4 *)(dk_ + key_b * kLd32 + 4 * c4) = kb;                                 \
        *(u32x4 *)(dv_ + key_b * kLd32 + 4 * c4) = vb;                                 \
    }

    const int nch = (Lp + kKC32 - 1) / kKC32;
    const int ntile = (Lp + kQT - 1) / kQT;
    const bool resident = nch <= 2;
    for (int t = g; t < ntile; t += G) {
        // B operand of score step kk: Q[query col][4*kk + grp]
        const int qrow = t * kQT + wid * kQW + col;
        float qf[16];
        {
            const float *src = q + (qrow < L ? R.off(qrow) : 0u);
#pragma unroll
            for (int kk = 0; kk < 16; ++kk) qf[kk] = qrow < L ? src[4 * kk + grp] : 0.f;
        }
        const bool stage = !resident || t == g;
        if (stage) {
            RATTN_LOAD32(0)
            RATTN_STORE32(0)
            __syncthreads();
        }
        float m = -INFINITY, lsum = 0.f;
        f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0, acc2 = acc0, acc3 = acc0;
        for (int ch = 0; ch < nch; ++ch) {
            const int buf = ch & 1;
            const bool more = stage && ch + 1 < nch;
            if (more) RATTN_LOAD32(ch + 1)
            step32(sK + buf * (kKC32 * kLd32), sV + buf * (kKC32 * kLd32), qf,
                   L - ch * kKC32, c, m, lsum, acc0, acc1, acc2, acc3);
            if (more) RATTN_STORE32(buf ^ 1)
            __syncthreads();
        }
        lsum = sum_across_groups(lsum);
        const float inv = 1.f / lsum;
        if (qrow < L) {
            if (o) {
                float *orow = o + R.off(qrow) + 4 * grp;
                *(f32x4 *)(orow) = acc0 * inv;
                *(f32x4 *)(orow + 16) = acc1 * inv;
                *(f32x4 *)(orow + 32) = acc2 * inv;
                *(f32x4 *)(orow + 48) = acc3 * inv;
            }
            if (cls_dst && qrow == 0) {
                float *crow = cls_dst + 4 * grp;
                *(f32x4 *)(crow) = acc0 * inv;
                *(f32x4 *)(crow + 16) = acc1 * inv;
                *(f32x4 *)(crow + 32) = acc2 * inv;
                *(f32x4 *)(crow + 48) = acc3 * inv;
            }
        }
    }
#undef RATTN_LOAD32
#undef RATTN_STORE32
}

// ---------------------------------------------------------------------------
// float32 core for batches of few heads: the 16-query tiles g, g+G, ... of one
// (image, head).  Wavefront w takes the tile's 32-key chunks w, w+4, ... into
// an LDS slab of its own, so a short sequence's chunks run on four SIMDs at
// once instead of one after another.  The four partial softmax states (row
// maximum, row sum, unnormalised output) are then merged in LDS in wavefront
// order 0, 1, 2, 3, whatever order the wavefronts finished in.
// ---------------------------------------------------------------------------
constexpr int kSlab32 = 2 * kKC32 * kLd32;  // floats: one chunk of K and of V

template <typename Rows>
__device__ __forceinline__ void attend32_split(const float *__restrict__ q,
                                               const float *__restrict__ k,
                                               const float *__restrict__ v, float *__restrict__ o,
                                               const Rows &R, int L, int Lp, float c, int g, int G,
                                               float *slabs, float *__restrict__ cls_dst) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const u32x4 zero4 = {0u, 0u, 0u, 0u};
    float *sK = slabs + wid * kSlab32, *sV = sK + kKC32 * kLd32;
    // a chunk is 32 keys x 16 four-float vectors per tensor; lane l copies
    // vector l & 15 of keys (l >> 4) + 4 j, j = 0..7
    const int c4 = lane & 15, key0 = lane >> 4;
    u32x4 kr[8], vr[8];
    auto load = [&](int ch) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int key = ch * kKC32 + key0 + 4 * j;
            kr[j] = zero4;
            vr[j] = zero4;
            if (key < L) {
                kr[j] = *(const u32x4 *)(k + R.off(key) + 4 * c4);
                vr[j] = *(const u32x4 *)(v + R.off(key) + 4 * c4);
            }
        }
    };
    const int nch = (Lp + kKC32 - 1) / kKC32;
    const int ntile = (Lp + kQW - 1) / kQW;
    for (int t = g; t < ntile; t += G) {
        // every wavefront has read the previous tile's partial states
        if (t != g) __syncthreads();
        const int qrow = t * kQW + col;
        float qf[16];
        {
            const float *src = q + (qrow < L ? R.off(qrow) : 0u);
#pragma unroll
            for (int kk = 0; kk < 16; ++kk) qf[kk] = qrow < L ? src[4 * kk + grp] : 0.f;
        }
        // finite, so that a chunk with no valid key (padded length) leaves
        // the state unchanged instead of giving exp2(-inf + inf)
        float m = -__FLT_MAX__, lsum = 0.f;
        f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0, acc2 = acc0, acc3 = acc0;
        if (wid < nch) load(wid);
        for (int ch = wid; ch < nch; ch += kWaves) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                *(u32x4 *)(sK + (key0 + 4 * j) * kLd32 + 4 * c4) = kr[j];
                *(u32x4 *)(sV + (key0 + 4 * j) * kLd32 + 4 * c4) = vr[j];
            }
            // LDS serves one wavefront's instructions in order: the slab is
            // written before this wavefront's reads below, and read before
            // its next writes
            __builtin_amdgcn_wave_barrier();
            if (ch + kWaves < nch) load(ch + kWaves);
            step32(sK, sV, qf, L - ch * kKC32, c, m, lsum, acc0, acc1, acc2, acc3);
            __builtin_amdgcn_wave_barrier();
        }
        // partial state into the own slab: output block j at 256 j + 4 lane,
        // then the 16 row maxima and the 16 row sums
        lsum = sum_across_groups(lsum);
        *(f32x4 *)(sK + 4 * lane) = acc0;
        *(f32x4 *)(sK + 256 + 4 * lane) = acc1;
        *(f32x4 *)(sK + 512 + 4 * lane) = acc2;
        *(f32x4 *)(sK + 768 + 4 * lane) = acc3;
        if (grp == 0) {
            sK[1024 + col] = m;
            sK[1040 + col] = lsum;
        }
        __syncthreads();
        // wavefront w merges output block w (dimensions 16 w .. 16 w + 15)
        float mw[kWaves], lw[kWaves];
        f32x4 aw[kWaves];
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float *part = slabs + w * kSlab32;
            mw[w] = part[1024 + col];
            lw[w] = part[1040 + col];
            aw[w] = *(const f32x4 *)(part + 256 * wid + 4 * lane);
        }
        const float M = fmaxf(fmaxf(mw[0], mw[1]), fmaxf(mw[2], mw[3]));
        float l = 0.f;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float f = fast_exp2(mw[w] - M);
            l += f * lw[w];
            acc += f * aw[w];
        }
        const float inv = 1.f / l;
        if (qrow < L) {
            if (o) *(f32x4 *)(o + R.off(qrow) + 16 * wid + 4 * grp) = acc * inv;
            if (cls_dst && qrow == 0) *(f32x4 *)(cls_dst + 16 * wid + 4 * grp) = acc * inv;
        }
    }
}

// (image, head, tile group) of this workgroup; false if the id is padding.
// Workgroup ids are dealt to the 8 XCDs round-robin; the G workgroups of one
// (image, head) get ids on the same XCD so the head's K/V rows, which each of
// them streams, are read into one L2.
__device__ __forceinline__ bool decode_group(int BH, int H, int G, int *b, int *h, int *g) {
    const int id = blockIdx.x;
    const int xcd = id & 7, local = id >> 3;
    const int pair = (local / G) * 8 + xcd;
    *g = local - (local / G) * G;
    if (pair >= BH) return false;
    *b = pair / H;
    *h = pair - *b * H;
    return true;
}

// One workgroup per (image, head) when the batch has at least as many heads
// as the chip has CUs; otherwise each head's query tiles (16*W rows) are
// dealt to G workgroups (tiles g, g+G, ...), G = CUs / heads, at most one per
// tile.  In the fused kernel splitting further only adds workgroups that
// re-rank the image (384 px, three workgroups per head: 47.3 -> 50.3 us).
// The last of a head's workgroups writes the pruned rows' zeros; while the
// chip has room (`spare_for_zeros`) a head gets at least two workgroups so
// that those stores overlap the attention of the first.  The flat kernel has
// no ranking to repeat: with 128-row tiles its heads are dealt to up to three
// workgroups, whose copies of each K/V chunk, made at about the same time on
// one XCD, share its L2, and the smaller units even out the load over the
// dispatch rounds (384 px: 41.3 -> 39.0 us; four or five workgroups per head
// were slower, 51.9 and 39.8 us).  With 64-row tiles (bounds up to 256) it
// keeps the plain rule: at batch 512 four workgroups per head took 37.4 ->
// 60.3 us.
constexpr int64_t kComputeUnits = 256;

int tile_groups(int B, int H, int max_seqlen, int rows, bool spare_for_zeros, int per_cu = 1) {
    const int ntiles = max_seqlen > 0 ? (max_seqlen + rows - 1) / rows : 1;
    const int64_t pairs = std::max<int64_t>((int64_t)B * H, 1);
    int64_t G = per_cu * kComputeUnits / pairs;
    if (spare_for_zeros && pairs < kComputeUnits) G = std::max<int64_t>(G, 2);
    if (!spare_for_zeros && rows == 128) G = std::max<int64_t>(G, std::min(ntiles, 3));
    return (int)std::max<int64_t>(1, std::min<int64_t>(G, std::max(ntiles, spare_for_zeros ? 2 : 1)));
}

// Shape of the 16-bit workgroups: W wavefronts, each owning QB blocks of 16
// query rows.  A workgroup computes 16*W*QB query rows against each K/V chunk
// it stages, so longer sequences get larger tiles and stream their K/V rows
// fewer times; two blocks per wavefront also halve the LDS operand reads per
// score, at the cost of registers (three wavefronts per SIMD instead of four).
struct Shape {
    int W, QB;
};

Shape shape_for(int max_seqlen) {
    // measured on MI355X (rattn_fused, back to back): up to 256 positions
    // 4x1 is best (batch 512: 52 us; 4x2 56, 8x1 61); at 577 positions 4x2
    // (56 us) beats 8x1 (60) and 4x1 (69): its 128-row tiles stream K/V three
    // times instead of five, and at three workgroups per CU all 768 heads of
    // a 64-image batch run in one round
    if (max_seqlen <= 256) return Shape{4, 1};
    return Shape{4, 2};
}

// Each path splits a tile's keys over its four wavefronts (attend32_split,
// attend16_split) when the batch has at most this many heads.  The rule reads
// B and H only, never the length bound, so every entry point picks the same
// core for the same batch and their outputs stay bitwise equal.
constexpr int64_t kSplit32Heads = 64;
constexpr int64_t kSplit16Heads = 24;
bool split32(int B, int H) { return (int64_t)B * H <= kSplit32Heads; }
bool split16(int B, int H) { return (int64_t)B * H <= kSplit16Heads; }
// Workgroups per head of a split core (16-row tiles).  One per CU while that
// runs at least half of each head's tiles under the bound at once; else up to
// two per CU, which their 68-74 KB of LDS leave room for.  Measured on float32
// batches of 197 positions, half kept (rattn_fused): 24 heads 7.7 us with one
// per CU against 9.8 with two (two split workgroups sharing a CU's SIMDs),
// 48 heads 12.1 against 10.1.
int split_groups(int B, int H, int bound, bool spare_for_zeros) {
    const int ntiles = bound > 0 ? (bound + kQW - 1) / kQW : 1;
    const int one = tile_groups(B, H, bound, kQW, spare_for_zeros);
    return 2 * one >= ntiles ? one : tile_groups(B, H, bound, kQW, spare_for_zeros, 2);
}
// The 16-bit split's steps are light enough that two of its workgroups on one
// CU still beat a workgroup running a second tile after its first: up to two
// per CU always.  DeiT-B at batch 2 (24 heads, 197 positions, rattn_fused
// back to back): unpruned 6.1 -> 5.5 us, 80 % pruned 4.35 -> 4.0 us.
int split16_groups(int B, int H, int bound, bool spare_for_zeros) {
    return tile_groups(B, H, bound, kQW, spare_for_zeros, 2);
}

int64_t grid_for(int B, int H, int G) { return 8 * (((int64_t)B * H + 7) / 8) * G; }

// ---------------------------------------------------------------------------
// kernels on the flat ragged buffer: one workgroup per (image, head)
// ---------------------------------------------------------------------------
template <typename T, int W, int QB>
__global__ __launch_bounds__(64 * W, QB == 1 ? 4 : 3) void attn_fwd16(const uint16_t *__restrict__ q,
                                                        const uint16_t *__restrict__ k,
                                                        const uint16_t *__restrict__ v,
                                                        uint16_t *__restrict__ o,
                                                        const int32_t *__restrict__ cu, int B,
                                                        int H, int G, int max_seqlen, float c) {
    __shared__ __attribute__((aligned(16))) uint16_t sK[2 * kKC * 64];
    __shared__ __attribute__((aligned(16))) uint16_t sV[2 * kD * 64];
    __shared__ __attribute__((aligned(16))) uint16_t sQ[QB == 2 ? 16 * W * QB * kD : 8];
    int b, h, g;
    if (!decode_group(B * H, H, G, &b, &h, &g)) return;
    const int seq0 = cu[b];
    const int L = cu[b + 1] - seq0;
    // an image longer than the caller's bound is outside the contract; it is
    // skipped (its rows are left unwritten) rather than read out of range
    if (L <= 0 || L > max_seqlen) return;
    const int64_t rs = (int64_t)H * kD;
    const int64_t base = (int64_t)seq0 * rs + (int64_t)h * kD;
    const FlatRows R = {(uint32_t)rs};
    if (c > 0.f)
        attend16<T, true, W, QB>(q + base, k + base, v + base, o + base, R, L, L, c, g, G, sK, sV,
                                 sQ, nullptr);
    else
        attend16<T, false, W, QB>(q + base, k + base, v + base, o + base, R, L, L, c, g, G, sK,
                                  sV, sQ, nullptr);
}

template <bool SPLIT>
__global__ __launch_bounds__(kThreads) void attn_fwd32(const float *__restrict__ q,
                                                       const float *__restrict__ k,
                                                       const float *__restrict__ v,
                                                       float *__restrict__ o,
                                                       const int32_t *__restrict__ cu, int B,
                                                       int H, int G, int max_seqlen, float c) {
    __shared__ __attribute__((aligned(16))) float lds[SPLIT ? kWaves * kSlab32 : 2 * kSlab32];
    int b, h, g;
    if (!decode_group(B * H, H, G, &b, &h, &g)) return;
    const int seq0 = cu[b];
    const int L = cu[b + 1] - seq0;
    if (L <= 0 || L > max_seqlen) return;
    const int64_t rs = (int64_t)H * kD;
    const int64_t base = (int64_t)seq0 * rs + (int64_t)h * kD;
    const FlatRows R = {(uint32_t)rs};
    if (SPLIT)
        attend32_split(q + base, k + base, v + base, o + base, R, L, L, c, g, G, lds, nullptr);
    else
        attend32(q + base, k + base, v + base, o + base, R, L, L, c, g, G, lds, lds + kSlab32,
                 nullptr);
}

// ---------------------------------------------------------------------------
// fused kernels: padded in, padded out, one launch, one workgroup per
// (image, head)
// ---------------------------------------------------------------------------
// Ranking an image of at most C 64-position chunks (N <= 64 C, C a multiple
// of W): every wavefront loads and ballots all C chunks in one round trip and
// counts the kept positions before each chunk in scalar registers;
// wavefront w writes the positions and the keep bits of chunks w, w+W, ...,
// and one barrier publishes them.
template <int W, int C>
__device__ __forceinline__ int rank_all(const uint8_t *__restrict__ keep_img, int N,
                                        int16_t *pos, uint64_t *keep_bits) {
    static_assert(C % W == 0, "chunks dealt evenly");
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nchunk = (N + 63) / 64;
    uint8_t byte[C];
#pragma unroll
    for (int i = 0; i < C; ++i) byte[i] = keep_img[min(64 * i + lane, N - 1)];
    int total = 0;  // kept positions before chunk i
#pragma unroll
    for (int i = 0; i < C; ++i) {
        const bool kept = 64 * i + lane < N && byte[i] != 0;
        const uint64_t m = __ballot(kept);
        if (i % W == w && i < nchunk) {
            if (kept) pos[total + __popcll(m & ((1ull << lane) - 1ull))] = (int16_t)(64 * i + lane);
            if (lane == 0) keep_bits[i] = m;
        }
        total += __popcll(m);
    }
    __syncthreads();
    return total;
}

// Kept positions of image b, in order, into pos[]; returns the count.  The
// keep bitmap (one 64-bit ballot per 64-position chunk) goes to keep_bits.
// Up to 1024 positions every wavefront ranks the whole image (rank_all);
// longer images: chunk c belongs to wavefront c % W, the ballots go to LDS,
// and after one exchange of per-chunk counts each wavefront writes its kept
// positions at their ranks.
template <int W>
__device__ __forceinline__ int rank_image(const uint8_t *__restrict__ keep_img, int N,
                                          int16_t *pos, uint64_t *keep_bits) {
    if (N <= 64 * W) return rank_all<W, W>(keep_img, N, pos, keep_bits);
    if (N <= 1024) return rank_all<W, 16>(keep_img, N, pos, keep_bits);
    constexpr int kChunksPerWave = (kMaxFusedN + 64 * W - 1) / (64 * W);
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int nchunk = (N + 63) / 64;
    // every load is issued before the first is used: positions past the end
    // read the last byte of the row and are discarded
    uint8_t byte[kChunksPerWave];
#pragma unroll
    for (int i = 0; i < kChunksPerWave; ++i)
        byte[i] = keep_img[min(64 * (wid + W * i) + lane, N - 1)];
    bool kept[kChunksPerWave];
#pragma unroll
    for (int i = 0; i < kChunksPerWave; ++i)
        kept[i] = 64 * (wid + W * i) + lane < N && byte[i] != 0;
    uint64_t m[kChunksPerWave];
#pragma unroll
    for (int i = 0; i < kChunksPerWave; ++i) {
        m[i] = __ballot(kept[i]);
        const int chunk = wid + W * i;
        if (lane == 0 && chunk < nchunk) keep_bits[chunk] = m[i];
    }
    __syncthreads();
    int total = 0;
    for (int cidx = 0; cidx < nchunk; ++cidx) total += __popcll(keep_bits[cidx]);
#pragma unroll
    for (int i = 0; i < kChunksPerWave; ++i) {
        const int chunk = wid + W * i;
        if (chunk >= nchunk) break;
        int before = 0;
        for (int cidx = 0; cidx < chunk; ++cidx) before += __popcll(keep_bits[cidx]);
        if (kept[i]) pos[before + __popcll(m[i] & ((1ull << lane) - 1ull))] = (int16_t)(64 * chunk + lane);
    }
    __syncthreads();
    return total;
}

// Zero rows of head h at the pruned positions of image b (and the CLS row
// when position 0 was pruned), reading the keep bitmap from LDS; every
// thread writes 16-byte pieces, 8 or 16 threads per 128/256-byte row.
template <int kPiecesPerRow, int kNThreads>
__device__ __forceinline__ void zero_pruned(const uint64_t *keep_bits, int N,
                                            u32x4 *__restrict__ out_head0, int64_t row_vec,
                                            u32x4 *__restrict__ cls_head) {
    const u32x4 zero4 = {0u, 0u, 0u, 0u};
    if (out_head0) {
        for (int idx = threadIdx.x; idx < N * kPiecesPerRow; idx += kNThreads) {
            const int n = idx / kPiecesPerRow, p = idx - n * kPiecesPerRow;
            if (!((keep_bits[n >> 6] >> (n & 63)) & 1ull)) out_head0[(int64_t)n * row_vec + p] = zero4;
        }
    }
    if (cls_head && !(keep_bits[0] & 1ull) && threadIdx.x < kPiecesPerRow) cls_head[threadIdx.x] = zero4;
}

template <typename T, int W, int QB>
__global__ __launch_bounds__(64 * W, QB == 1 ? 4 : 3) void fused16(const uint16_t *__restrict__ q,
                                                     const uint16_t *__restrict__ k,
                                                     const uint16_t *__restrict__ v,
                                                     const uint8_t *__restrict__ keep,
                                                     uint16_t *__restrict__ out,
                                                     uint16_t *__restrict__ cls, int B, int N,
                                                     int H, int G, int pad, float c) {
    __shared__ __attribute__((aligned(16))) uint16_t sK[2 * kKC * 64];
    __shared__ __attribute__((aligned(16))) uint16_t sV[2 * kD * 64];
    __shared__ __attribute__((aligned(16))) uint16_t sQ[QB == 2 ? 16 * W * QB * kD : 8];
    __shared__ int16_t pos[kMaxFusedN];
    __shared__ uint64_t keep_bits[kMaxFusedN / 64];
    int b, h, g;
    if (!decode_group(B * H, H, G, &b, &h, &g)) return;
    const uint8_t *keep_img = keep + (int64_t)b * N;
    const int L = rank_image<W>(keep_img, N, pos, keep_bits);
    const int64_t rs = (int64_t)H * kD;
    const int64_t head0 = (int64_t)b * N * rs + (int64_t)h * kD;  // (b, 0, h)
    uint16_t *cls_head = cls ? cls + ((int64_t)b * H + h) * kD : nullptr;
    uint16_t *out_head = out ? out + head0 : nullptr;
    if (L > 0) {
        const PaddedRows R = {(uint32_t)rs, pos};
        // the output row of query rank 0 is the CLS row iff position 0 was kept
        uint16_t *cls_dst = (cls_head && pos[0] == 0) ? cls_head : nullptr;
        // padded comparator (pad > 0): every image processed at length pad
        const int Lp = max(L, pad);
        int gg = g, GG = G;
        bool run = true;
        if (!out) {
            // CLS rows only: only the workgroup holding query tile 0 has work,
            // and it computes that tile alone
            run = cls_dst && g == 0;
            GG = (Lp + 16 * W * QB - 1) / (16 * W * QB);
            gg = 0;
        }
        if (run) {
            if (c > 0.f)
                attend16<T, true, W, QB>(q + head0, k + head0, v + head0, out_head, R, L, Lp, c, gg, GG,
                                     sK, sV, sQ, cls_dst);
            else
                attend16<T, false, W, QB>(q + head0, k + head0, v + head0, out_head, R, L, Lp, c, gg, GG,
                                      sK, sV, sQ, cls_dst);
        }
    }
    // zeros for the pruned rows: by the last workgroup of the head, after its
    // attention, so that the attention's loads never wait for these stores
    if (g == G - 1)
        zero_pruned<kD * 2 / 16, 64 * W>(keep_bits, N, out_head ? (u32x4 *)out_head : nullptr,
                                         rs * 2 / 16, (u32x4 *)cls_head);
}

// Kernels for batches of few heads.  The core for one (image, head) is
// chosen by the image's kept count L, the same in every entry point whatever
// the bound or the padded length: an image of one 64-key chunk has no keys
// to split and runs attend16 on one 64-row tile, exactly as in a batch of
// many heads; a longer one runs the key-split core on 16-row tiles.  The G
// workgroups of a head are dealt 16-row tiles (g, g+G, ...); with 64-row
// tiles only g = 0 has one.  attend16's two K and two V chunk buffers use
// the first two slabs (its Q buffer serves two-block wavefronts only).
#define RATTN_ATTEND_FEW(RT, QH, KH, VH, OH, R, L, LP, C, G_, GG, SLABS, CLS)                \
    do {                                                                                    \
        uint16_t *sK_ = (SLABS), *sV_ = (SLABS) + 2 * kKC * 64, *sQ_ = (SLABS) + 4 * kKC * 64; \
        if ((L) <= kKC && (C) > 0.f)                                                        \
            attend16<T, true, kWaves, 1, RT, 1>(QH, KH, VH, OH, R, L, LP, C, G_, GG, sK_, sV_, sQ_, \
                                                CLS);                                        \
        else if ((L) <= kKC)                                                                \
            attend16<T, false, kWaves, 1, RT, 1>(QH, KH, VH, OH, R, L, LP, C, G_, GG, sK_, sV_, sQ_, \
                                                 CLS);                                       \
        else if ((C) > 0.f)                                                                 \
            attend16_split<T, true>(QH, KH, VH, OH, R, L, LP, C, G_, GG, SLABS, CLS);        \
        else                                                                                \
            attend16_split<T, false>(QH, KH, VH, OH, R, L, LP, C, G_, GG, SLABS, CLS);       \
    } while (0)

// rattn_forward for batches of few heads
template <typename T>
__global__ __launch_bounds__(kThreads) void attn_fwd16s(const uint16_t *__restrict__ q,
                                                        const uint16_t *__restrict__ k,
                                                        const uint16_t *__restrict__ v,
                                                        uint16_t *__restrict__ o,
                                                        const int32_t *__restrict__ cu, int B,
                                                        int H, int G, int max_seqlen, float c) {
    __shared__ __attribute__((aligned(16))) uint16_t slabs[kWaves * kSlab16];
    int b, h, g;
    if (!decode_group(B * H, H, G, &b, &h, &g)) return;
    const int seq0 = cu[b];
    const int L = cu[b + 1] - seq0;
    if (L <= 0 || L > max_seqlen) return;
    const int64_t rs = (int64_t)H * kD;
    const int64_t base = (int64_t)seq0 * rs + (int64_t)h * kD;
    const FlatRows R = {(uint32_t)rs};
    RATTN_ATTEND_FEW(FlatRows, q + base, k + base, v + base, o + base, R, L, L, c, g, G, slabs,
                     nullptr);
}

// rattn_fused for batches of few heads
template <typename T>
__global__ __launch_bounds__(kThreads) void fused16s(const uint16_t *__restrict__ q,
                                                     const uint16_t *__restrict__ k,
                                                     const uint16_t *__restrict__ v,
                                                     const uint8_t *__restrict__ keep,
                                                     uint16_t *__restrict__ out,
                                                     uint16_t *__restrict__ cls, int B, int N,
                                                     int H, int G, int pad, float c) {
    __shared__ __attribute__((aligned(16))) uint16_t slabs[kWaves * kSlab16];
    __shared__ int16_t pos[kMaxFusedN];
    __shared__ uint64_t keep_bits[kMaxFusedN / 64];
    int b, h, g;
    if (!decode_group(B * H, H, G, &b, &h, &g)) return;
    const uint8_t *keep_img = keep + (int64_t)b * N;
    const int L = rank_image<kWaves>(keep_img, N, pos, keep_bits);
    const int64_t rs = (int64_t)H * kD;
    const int64_t head0 = (int64_t)b * N * rs + (int64_t)h * kD;
    uint16_t *cls_head = cls ? cls + ((int64_t)b * H + h) * kD : nullptr;
    uint16_t *out_head = out ? out + head0 : nullptr;
    if (L > 0) {
        const PaddedRows R = {(uint32_t)rs, pos};
        uint16_t *cls_dst = (cls_head && pos[0] == 0) ? cls_head : nullptr;
        const int Lp = max(L, pad);
        int gg = g, GG = G;
        bool run = true;
        if (!out) {
            // CLS rows only: the workgroup holding query tile 0 computes that
            // tile alone
            run = cls_dst && g == 0;
            GG = (Lp + kQW - 1) / kQW;
            gg = 0;
        }
        if (run)
            RATTN_ATTEND_FEW(PaddedRows, q + head0, k + head0, v + head0, out_head, R, L, Lp, c, gg,
                             GG, slabs, cls_dst);
    }
    // zeros for the pruned rows: by the last workgroup of the head, after its
    // attention
    if (g == G - 1)
        zero_pruned<kD * 2 / 16, kThreads>(keep_bits, N, out_head ? (u32x4 *)out_head : nullptr,
                                           rs * 2 / 16, (u32x4 *)cls_head);
}
#undef RATTN_ATTEND_FEW


template <bool SPLIT>
__global__ __launch_bounds__(kThreads) void fused32(const float *__restrict__ q,
                                                    const float *__restrict__ k,
                                                    const float *__restrict__ v,
                                                    const uint8_t *__restrict__ keep,
                                                    float *__restrict__ out,
                                                    float *__restrict__ cls, int B, int N,
                                                    int H, int G, int pad, float c) {
    __shared__ __attribute__((aligned(16))) float lds[SPLIT ? kWaves * kSlab32 : 2 * kSlab32];
    __shared__ int16_t pos[kMaxFusedN];
    __shared__ uint64_t keep_bits[kMaxFusedN / 64];
    int b, h, g;
    if (!decode_group(B * H, H, G, &b, &h, &g)) return;
    const uint8_t *keep_img = keep + (int64_t)b * N;
    const int L = rank_image<kWaves>(keep_img, N, pos, keep_bits);
    const int64_t rs = (int64_t)H * kD;
    const int64_t head0 = (int64_t)b * N * rs + (int64_t)h * kD;
    float *cls_head = cls ? cls + ((int64_t)b * H + h) * kD : nullptr;
    float *out_head = out ? out + head0 : nullptr;
    if (L > 0) {
        const PaddedRows R = {(uint32_t)rs, pos};
        float *cls_dst = (cls_head && pos[0] == 0) ? cls_head : nullptr;
        const int Lp = max(L, pad);
        int gg = g, GG = G;
        bool run = true;
        if (!out) {
            // CLS rows only: the workgroup holding query tile 0 computes that
            // tile alone
            run = cls_dst && g == 0;
            GG = (Lp + (SPLIT ? kQW : kQT) - 1) / (SPLIT ? kQW : kQT);
            gg = 0;
        }
        if (run && SPLIT)
            attend32_split(q + head0, k + head0, v + head0, out_head, R, L, Lp, c, gg, GG, lds,
                           cls_dst);
        else if (run)
            attend32(q + head0, k + head0, v + head0, out_head, R, L, Lp, c, gg, GG, lds,
                     lds + kSlab32, cls_dst);
    }
    // zeros for the pruned rows: by the last workgroup of the head, after its
    // attention
    if (g == G - 1)
        zero_pruned<kD * 4 / 16, kThreads>(keep_bits, N, out_head ? (u32x4 *)out_head : nullptr,
                                           rs * 4 / 16, (u32x4 *)cls_head);
}

template <typename T, int W, int QB>
hipError_t launch_fwd16(const AttnArgs &a, float c, hipStream_t s) {
    const int G = tile_groups(a.B, a.H, a.max_seqlen, 16 * W * QB, false);
    const unsigned grid = (unsigned)grid_for(a.B, a.H, G);
    return launch<attn_fwd16<T, W, QB>>(dim3(grid), dim3(64 * W), s, (const uint16_t *)a.q,
                                        (const uint16_t *)a.k, (const uint16_t *)a.v,
                                        (uint16_t *)a.o, a.cu, a.B, a.H, G, a.max_seqlen, c);
}

template <typename T>
hipError_t launch_fwd16_shape(const AttnArgs &a, float c, hipStream_t s) {
    if (split16(a.B, a.H)) {
        const int G = split16_groups(a.B, a.H, a.max_seqlen, false);
        return launch<attn_fwd16s<T>>(dim3((unsigned)grid_for(a.B, a.H, G)), dim3(kThreads), s,
                                      (const uint16_t *)a.q, (const uint16_t *)a.k,
                                      (const uint16_t *)a.v, (uint16_t *)a.o, a.cu, a.B, a.H, G,
                                      a.max_seqlen, c);
    }
    const Shape sh = shape_for(a.max_seqlen);
    if (sh.QB == 1) return launch_fwd16<T, 4, 1>(a, c, s);
    return launch_fwd16<T, 4, 2>(a, c, s);
}

template <typename T, int W, int QB>
hipError_t launch_fused16(const FusedArgs &a, float c, hipStream_t s) {
    // without the padded output only tile 0 (the CLS row) is computed
    const int G = a.out ? tile_groups(a.B, a.H, std::min(a.max_seqlen, a.N), 16 * W * QB, true) : 1;
    const unsigned grid = (unsigned)grid_for(a.B, a.H, G);
    return launch<fused16<T, W, QB>>(dim3(grid), dim3(64 * W), s, (const uint16_t *)a.q,
                                     (const uint16_t *)a.k, (const uint16_t *)a.v, a.keep,
                                     (uint16_t *)a.out, (uint16_t *)a.cls, a.B, a.N, a.H, G, a.pad,
                                     c);
}

template <typename T>
hipError_t launch_fused16_shape(const FusedArgs &a, float c, hipStream_t s) {
    if (split16(a.B, a.H)) {
        // without the padded output only tile 0 (the CLS row) is computed
        const int G = a.out ? split16_groups(a.B, a.H, std::min(a.max_seqlen, a.N), true) : 1;
        return launch<fused16s<T>>(dim3((unsigned)grid_for(a.B, a.H, G)), dim3(kThreads), s,
                                   (const uint16_t *)a.q, (const uint16_t *)a.k,
                                   (const uint16_t *)a.v, a.keep, (uint16_t *)a.out,
                                   (uint16_t *)a.cls, a.B, a.N, a.H, G, a.pad, c);
    }
    // the CLS-only mode computes one tile per head: the smallest workgroup
    const Shape sh = a.out ? shape_for(std::min(a.max_seqlen, a.N)) : Shape{4, 1};
    if (sh.QB == 1) return launch_fused16<T, 4, 1>(a, c, s);
    return launch_fused16<T, 4, 2>(a, c, s);
}

}  // namespace

hipError_t launch_attention(const AttnArgs &a, hipStream_t s) {
    const float c = a.scale * kLog2e;
    switch (a.dt) {
    case Elem::BF16: return launch_fwd16_shape<__bf16>(a, c, s);
    case Elem::F16: return launch_fwd16_shape<_Float16>(a, c, s);
    case Elem::F32: {
        const bool split = split32(a.B, a.H);
        const int G = split ? split_groups(a.B, a.H, a.max_seqlen, false)
                            : tile_groups(a.B, a.H, a.max_seqlen, kQT, false);
        const dim3 grid((unsigned)grid_for(a.B, a.H, G));
        if (split)
            return launch<attn_fwd32<true>>(grid, dim3(kThreads), s, (const float *)a.q,
                                            (const float *)a.k, (const float *)a.v, (float *)a.o,
                                            a.cu, a.B, a.H, G, a.max_seqlen, c);
        return launch<attn_fwd32<false>>(grid, dim3(kThreads), s, (const float *)a.q,
                                         (const float *)a.k, (const float *)a.v, (float *)a.o,
                                         a.cu, a.B, a.H, G, a.max_seqlen, c);
    }
    }
    return hipErrorInvalidValue;
}

hipError_t launch_fused(const FusedArgs &a, hipStream_t s) {
    const float c = a.scale * kLog2e;
    switch (a.dt) {
    case Elem::BF16: return launch_fused16_shape<__bf16>(a, c, s);
    case Elem::F16: return launch_fused16_shape<_Float16>(a, c, s);
    case Elem::F32: {
        const bool split = split32(a.B, a.H);
        // without the padded output only tile 0 (the CLS row) is computed
        const int bound = std::min(a.max_seqlen, a.N);
        const int G = !a.out ? 1
                      : split ? split_groups(a.B, a.H, bound, true)
                              : tile_groups(a.B, a.H, bound, kQT, true);
        const dim3 grid((unsigned)grid_for(a.B, a.H, G));
        if (split)
            return launch<fused32<true>>(grid, dim3(kThreads), s, (const float *)a.q,
                                         (const float *)a.k, (const float *)a.v, a.keep,
                                         (float *)a.out, (float *)a.cls, a.B, a.N, a.H, G, a.pad,
                                         c);
        return launch<fused32<false>>(grid, dim3(kThreads), s, (const float *)a.q,
                                      (const float *)a.k, (const float *)a.v, a.keep,
                                      (float *)a.out, (float *)a.cls, a.B, a.N, a.H, G, a.pad, c);
    }
    }
    return hipErrorInvalidValue;
}

}  // namespace rattn
