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
//  * One workgroup = 4 wavefronts = one (image, head, 64-query tile); each
//    wavefront owns 16 query rows.  Workgroup ids are laid out so all query
//    tiles of one (image, head) land on the same XCD (ids are dealt to the 8
//    XCDs round-robin), keeping that head's K/V rows in one L2.
//  * Keys stream through LDS in chunks of 64, double-buffered: the global
//    loads of chunk c+1 are in flight while chunk c is computed, one barrier
//    per chunk.  K is stored row-major, V transposed (dims x keys) so each
//    MFMA operand is one 16-byte LDS read per lane; 16-byte pieces of a row
//    are XOR-swizzled by (row & 7) so the 16 rows one operand read touches hit
//    distinct banks without padding.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_16x16x32_{bf16,f16}: in the accumulator layout each lane holds
//    4 keys of ONE query, so the running max / sum are per-lane scalars (the
//    max needs two cross-lane steps per chunk, the sum none until the end).
//  * The probabilities feed O^T = V^T P^T directly as the MFMA B operand: the
//    V^T column order is permuted so operand slot (lane group g, slot s) of a
//    32-key step carries the same key in V^T and in the score accumulators.
//  * Online softmax in base 2: scores times scale*log2(e), v_exp_f32, running
//    output rescaled by exp2(m_old - m_new) per chunk, one division at the end.
//  * Keys past the sequence end inside the last chunk are zero-filled in LDS
//    and get score -inf; query rows past the end are computed on zeros and
//    never stored.
//  * Fused path: the workgroup first ranks its image's kept tokens with one
//    wavefront ballot per 64 positions into an LDS list of positions; Q/K/V
//    rows are then read from those positions of the padded tensors and the
//    outputs written to the same positions of the padded output.  Tile 0 of
//    each (image, head) also writes zeros to the pruned rows and the CLS row.
// The float32 path has the same structure on v_mfma_f32_16x16x4_f32 with
// 32-key chunks, row-padded LDS and probabilities kept in float32.
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
    static __device__ __forceinline__ f32x4 run(v8 a, v8 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};
template <> struct Mma<_Float16> {
    typedef f16x8 v8;
    static __device__ __forceinline__ f32x4 run(v8 a, v8 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
};

__device__ __forceinline__ float max_across_groups(float x) {
    // lanes l, l^16, l^32, l^48 hold the same query row
    x = fmaxf(x, __shfl_xor(x, 16));
    x = fmaxf(x, __shfl_xor(x, 32));
    return x;
}

__device__ __forceinline__ float sum_across_groups(float x) {
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <typename T>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    T a = (T)lo, b = (T)hi;  // round to nearest even
    return (uint32_t)__builtin_bit_cast(uint16_t, a) |
           ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// (image, head, query tile) of this workgroup; false if the id is padding.
__device__ __forceinline__ bool decode_tile(int B, int H, int ntiles, int *b, int *h,
                                            int *tile) {
    const int id = blockIdx.x;
    const int xcd = id & 7, local = id >> 3;
    const int pair = (local / ntiles) * 8 + xcd;
    *tile = local - (local / ntiles) * ntiles;
    if (pair >= B * H) return false;
    *b = pair / H;
    *h = pair - *b * H;
    return true;
}

// Element offset of the 64-element head slice of kept row r of one
// (image, head), in the flat ragged buffer or in the padded tensor.
struct FlatRows {
    int64_t base, rs;  // offset of (cu[b], h); elements per token row
    __device__ __forceinline__ int64_t at(int r) const { return base + (int64_t)r * rs; }
};
struct PaddedRows {
    int64_t base, rs;    // offset of (b, 0, h); elements per token row
    const int16_t *pos;  // LDS: position of the r-th kept token
    __device__ __forceinline__ int64_t at(int r) const { return base + (int64_t)pos[r] * rs; }
};

// 16-byte piece p of LDS row `row` (128-byte rows), XOR-swizzled.
__device__ __forceinline__ int swz(int row, int piece) { return row * 64 + 8 * (piece ^ (row & 7)); }

// ---------------------------------------------------------------------------
// 16-bit core: one 64-query tile of one (image, head)
// ---------------------------------------------------------------------------
template <typename T, typename Rows>
__device__ __forceinline__ void attend16(const uint16_t *__restrict__ q,
                                         const uint16_t *__restrict__ k,
                                         const uint16_t *__restrict__ v,
                                         uint16_t *__restrict__ o, const Rows &R, int L, int q0,
                                         float c, uint16_t *sK, uint16_t *sV,
                                         uint16_t *__restrict__ cls_dst) {
    typedef typename Mma<T>::v8 V8;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const u32x4 zero4 = {0u, 0u, 0u, 0u};

    // B operand of S^T = K Q^T: query row `col` of this wavefront, dims
    // 32*kk + 8*grp .. +7
    const int qrow = q0 + wid * kQW + col;
    u32x4 qf0 = zero4, qf1 = zero4;
    if (qrow < L) {
        const uint16_t *src = q + R.at(qrow);
        qf0 = *(const u32x4 *)(src + 8 * grp);
        qf1 = *(const u32x4 *)(src + 32 + 8 * grp);
    }

    // Staging roles: threads 0..127 stage V (keys 4*sr .. 4*sr+3, dims
    // 8*sc .. +7, transposed on the way into LDS); threads 128..255 stage K
    // (keys sr + 16*i, dims 8*sc .. +7, row copies).
    const bool vrole = tid < 128;
    const int sr = (tid & 127) >> 3;
    const int sc = tid & 7;
    const uint16_t *stage_src = vrole ? v : k;
    u32x4 g0, g1, g2, g3;

#define RATTN_LOAD_CHUNK(CH)                                                            \
    {                                                                                   \
        const int k0_ = (CH) * kKC;                                                     \
        const int key0_ = k0_ + (vrole ? 4 * sr : sr);                                 \
        const int step_ = vrole ? 1 : 16;                                               \
        g0 = key0_ < L ? *(const u32x4 *)(stage_src + R.at(key0_) + 8 * sc) : zero4;   \
        g1 = key0_ + step_ < L ? *(const u32x4 *)(stage_src + R.at(key0_ + step_) + 8 * sc) : zero4; \
        g2 = key0_ + 2 * step_ < L ? *(const u32x4 *)(stage_src + R.at(key0_ + 2 * step_) + 8 * sc) : zero4; \
        g3 = key0_ + 3 * step_ < L ? *(const u32x4 *)(stage_src + R.at(key0_ + 3 * step_) + 8 * sc) : zero4; \
    }

    // V^T column of key j inside a chunk: (j & ~31) + 8*((j>>2)&3) + 4*((j>>4)&1) + (j&3)
    const int vcol = (4 * sr & ~31) + 8 * ((sr) & 3) + 4 * ((4 * sr >> 4) & 1);
#define RATTN_STORE_CHUNK(BUF)                                                          \
    {                                                                                   \
        if (vrole) {                                                                    \
            uint16_t *dstv_ = sV + (BUF) * (kD * 64);                                   \
            _Pragma("unroll") for (int e = 0; e < 8; ++e) {                             \
                const int sh_ = 16 * (e & 1);                                           \
                const uint32_t x0_ = (g0[e >> 1] >> sh_) & 0xFFFFu;                     \
                const uint32_t x1_ = (g1[e >> 1] >> sh_) & 0xFFFFu;                     \
                const uint32_t x2_ = (g2[e >> 1] >> sh_) & 0xFFFFu;                     \
                const uint32_t x3_ = (g3[e >> 1] >> sh_) & 0xFFFFu;                     \
                const u32x2 w_ = {x0_ | (x1_ << 16), x2_ | (x3_ << 16)};                \
                const int row_ = 8 * sc + e;                                            \
                *(u32x2 *)(dstv_ + swz(row_, vcol >> 3) + (vcol & 7)) = w_;             \
            }                                                                           \
        } else {                                                                        \
            uint16_t *dstk_ = sK + (BUF) * (kKC * 64);                                  \
            *(u32x4 *)(dstk_ + swz(sr, sc)) = g0;                                       \
            *(u32x4 *)(dstk_ + swz(sr + 16, sc)) = g1;                                  \
            *(u32x4 *)(dstk_ + swz(sr + 32, sc)) = g2;                                  \
            *(u32x4 *)(dstk_ + swz(sr + 48, sc)) = g3;                                  \
        }                                                                               \
    }

    float m = -INFINITY, lsum = 0.f;
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0, acc2 = acc0, acc3 = acc0;

    const int nch = (L + kKC - 1) / kKC;
    RATTN_LOAD_CHUNK(0)
    RATTN_STORE_CHUNK(0)
    __syncthreads();

    for (int ch = 0; ch < nch; ++ch) {
        const int buf = ch & 1;
        const bool more = ch + 1 < nch;
        if (more) RATTN_LOAD_CHUNK(ch + 1)
        const uint16_t *Ks = sK + buf * (kKC * 64);
        const uint16_t *Vs = sV + buf * (kD * 64);

        f32x4 s[4];
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
            const int row = 16 * blk + col;
            const u32x4 a0 = *(const u32x4 *)(Ks + swz(row, grp));
            const u32x4 a1 = *(const u32x4 *)(Ks + swz(row, 4 + grp));
            f32x4 z = {0.f, 0.f, 0.f, 0.f};
            z = Mma<T>::run(__builtin_bit_cast(V8, a0), __builtin_bit_cast(V8, qf0), z);
            s[blk] = Mma<T>::run(__builtin_bit_cast(V8, a1), __builtin_bit_cast(V8, qf1), z);
        }

        const int valid = L - ch * kKC;
        float mx = -INFINITY;
#pragma unroll
        for (int blk = 0; blk < 4; ++blk)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float x = s[blk][i] * c;
                if (16 * blk + 4 * grp + i >= valid) x = -INFINITY;
                s[blk][i] = x;
                mx = fmaxf(mx, x);
            }
        mx = max_across_groups(mx);
        const float mn = fmaxf(m, mx);
        const float alpha = fast_exp2(m - mn);
        m = mn;
        float ps = 0.f;
#pragma unroll
        for (int blk = 0; blk < 4; ++blk)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p = fast_exp2(s[blk][i] - mn);
                s[blk][i] = p;
                ps += p;
            }
        lsum = lsum * alpha + ps;
        acc0 *= alpha;
        acc1 *= alpha;
        acc2 *= alpha;
        acc3 *= alpha;

#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            u32x4 pb;
            pb[0] = pack2<T>(s[2 * ks][0], s[2 * ks][1]);
            pb[1] = pack2<T>(s[2 * ks][2], s[2 * ks][3]);
            pb[2] = pack2<T>(s[2 * ks + 1][0], s[2 * ks + 1][1]);
            pb[3] = pack2<T>(s[2 * ks + 1][2], s[2 * ks + 1][3]);
            const V8 b = __builtin_bit_cast(V8, pb);
            const int piece = 4 * ks + grp;
            acc0 = Mma<T>::run(__builtin_bit_cast(V8, *(const u32x4 *)(Vs + swz(col, piece))), b, acc0);
            acc1 = Mma<T>::run(__builtin_bit_cast(V8, *(const u32x4 *)(Vs + swz(16 + col, piece))), b, acc1);
            acc2 = Mma<T>::run(__builtin_bit_cast(V8, *(const u32x4 *)(Vs + swz(32 + col, piece))), b, acc2);
            acc3 = Mma<T>::run(__builtin_bit_cast(V8, *(const u32x4 *)(Vs + swz(48 + col, piece))), b, acc3);
        }
        if (more) RATTN_STORE_CHUNK(buf ^ 1)
        __syncthreads();
    }
#undef RATTN_LOAD_CHUNK
#undef RATTN_STORE_CHUNK

    lsum = sum_across_groups(lsum);
    const float inv = 1.f / lsum;
    if (qrow < L) {
        // lane holds o[qrow][16*dt + 4*grp + i], i = 0..3
        const u32x2 w0 = {pack2<T>(acc0[0] * inv, acc0[1] * inv), pack2<T>(acc0[2] * inv, acc0[3] * inv)};
        const u32x2 w1 = {pack2<T>(acc1[0] * inv, acc1[1] * inv), pack2<T>(acc1[2] * inv, acc1[3] * inv)};
        const u32x2 w2 = {pack2<T>(acc2[0] * inv, acc2[1] * inv), pack2<T>(acc2[2] * inv, acc2[3] * inv)};
        const u32x2 w3 = {pack2<T>(acc3[0] * inv, acc3[1] * inv), pack2<T>(acc3[2] * inv, acc3[3] * inv)};
        if (o) {
            uint16_t *orow = o + R.at(qrow) + 4 * grp;
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

// ---------------------------------------------------------------------------
// float32 core
// ---------------------------------------------------------------------------
template <typename Rows>
__device__ __forceinline__ void attend32(const float *__restrict__ q, const float *__restrict__ k,
                                         const float *__restrict__ v, float *__restrict__ o,
                                         const Rows &R, int L, int q0, float c, float *sK,
                                         float *sV, float *__restrict__ cls_dst) {
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const u32x4 zero4 = {0u, 0u, 0u, 0u};

    // B operand of score step kk: Q[query col][4*kk + grp]
    const int qrow = q0 + wid * kQW + col;
    float qf[16];
    {
        const float *src = q + (qrow < L ? R.at(qrow) : R.at(0));
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) qf[kk] = qrow < L ? src[4 * kk + grp] : 0.f;
    }

    // staging: a chunk is 32 keys x 16 four-float vectors per tensor; thread
    // t stages vectors t and t + 256 of K and of V
    const int key_a = tid >> 4, key_b = (tid + kThreads) >> 4, c4 = tid & 15;
    u32x4 ka, kb, va, vb;
#define RATTN_LOAD32(CH)                                                               \
    {                                                                                  \
        const int k0_ = (CH) * kKC32;                                                  \
        ka = zero4; va = zero4; kb = zero4; vb = zero4;                                \
        if (k0_ + key_a < L) {                                                         \
            ka = *(const u32x4 *)(k + R.at(k0_ + key_a) + 4 * c4);                     \
            va = *(const u32x4 *)(v + R.at(k0_ + key_a) + 4 * c4);                     \
        }                                                                              \
        if (k0_ + key_b < L) {                                                         \
            kb = *(const u32x4 *)(k + R.at(k0_ + key_b) + 4 * c4);                     \
            vb = *(const u32x4 *)(v + R.at(k0_ + key_b) + 4 * c4);                     \
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

    float m = -INFINITY, lsum = 0.f;
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = acc0, acc2 = acc0, acc3 = acc0;
    const int nch = (L + kKC32 - 1) / kKC32;
    RATTN_LOAD32(0)
    RATTN_STORE32(0)
    __syncthreads();
    for (int ch = 0; ch < nch; ++ch) {
        const int buf = ch & 1;
        const bool more = ch + 1 < nch;
        if (more) RATTN_LOAD32(ch + 1)
        const float *Ks = sK + buf * (kKC32 * kLd32);
        const float *Vs = sV + buf * (kKC32 * kLd32);
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0;
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
            s0 = __builtin_amdgcn_mfma_f32_16x16x4f32(Ks[col * kLd32 + 4 * kk + grp], qf[kk], s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_16x16x4f32(Ks[(16 + col) * kLd32 + 4 * kk + grp], qf[kk], s1, 0, 0, 0);
        }
        const int valid = L - ch * kKC32;
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
        if (more) RATTN_STORE32(buf ^ 1)
        __syncthreads();
    }
#undef RATTN_LOAD32
#undef RATTN_STORE32
    lsum = sum_across_groups(lsum);
    const float inv = 1.f / lsum;
    if (qrow < L) {
        if (o) {
            float *orow = o + R.at(qrow) + 4 * grp;
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

// ---------------------------------------------------------------------------
// kernels on the flat ragged buffer
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kThreads) void attn_fwd16(const uint16_t *__restrict__ q,
                                                       const uint16_t *__restrict__ k,
                                                       const uint16_t *__restrict__ v,
                                                       uint16_t *__restrict__ o,
                                                       const int32_t *__restrict__ cu, int B,
                                                       int H, int ntiles, float c) {
    __shared__ __attribute__((aligned(16))) uint16_t sK[2 * kKC * 64];
    __shared__ __attribute__((aligned(16))) uint16_t sV[2 * kD * 64];
    int b, h, tile;
    if (!decode_tile(B, H, ntiles, &b, &h, &tile)) return;
    const int seq0 = cu[b];
    const int L = cu[b + 1] - seq0;
    const int q0 = tile * kQT;
    if (q0 >= L) return;
    const int64_t rs = (int64_t)H * kD;
    const FlatRows R = {(int64_t)seq0 * rs + (int64_t)h * kD, rs};
    attend16<T>(q, k, v, o, R, L, q0, c, sK, sV, nullptr);
}

__global__ __launch_bounds__(kThreads) void attn_fwd32(const float *__restrict__ q,
                                                       const float *__restrict__ k,
                                                       const float *__restrict__ v,
                                                       float *__restrict__ o,
                                                       const int32_t *__restrict__ cu, int B,
                                                       int H, int ntiles, float c) {
    __shared__ __attribute__((aligned(16))) float sK[2 * kKC32 * kLd32];
    __shared__ __attribute__((aligned(16))) float sV[2 * kKC32 * kLd32];
    int b, h, tile;
    if (!decode_tile(B, H, ntiles, &b, &h, &tile)) return;
    const int seq0 = cu[b];
    const int L = cu[b + 1] - seq0;
    const int q0 = tile * kQT;
    if (q0 >= L) return;
    const int64_t rs = (int64_t)H * kD;
    const FlatRows R = {(int64_t)seq0 * rs + (int64_t)h * kD, rs};
    attend32(q, k, v, o, R, L, q0, c, sK, sV, nullptr);
}

// ---------------------------------------------------------------------------
// fused kernels: padded in, padded out, one launch
// ---------------------------------------------------------------------------
// Kept positions of image b, in order, into pos[]; returns the count.  Wave 0
// walks the mask 64 positions at a time with one ballot each.
__device__ __forceinline__ int rank_image(const uint8_t *__restrict__ keep_img, int N,
                                          int16_t *pos, int *s_count) {
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        int count = 0;
        for (int n0 = 0; n0 < N; n0 += 64) {
            const int n = n0 + lane;
            const bool kept = n < N && keep_img[n] != 0;
            const uint64_t m = __ballot(kept);
            if (kept) pos[count + __popcll(m & ((1ull << lane) - 1ull))] = (int16_t)n;
            count += __popcll(m);
        }
        if (lane == 0) *s_count = count;
    }
    __syncthreads();
    return *s_count;
}

// Zero rows of head h at the pruned positions of image b (and the CLS row
// when position 0 was pruned); every thread writes 16-byte pieces.
template <int kPiecesPerRow>
__device__ __forceinline__ void zero_pruned(const uint8_t *__restrict__ keep_img, int N,
                                            u32x4 *__restrict__ out_head0, int64_t row_vec,
                                            u32x4 *__restrict__ cls_head) {
    const u32x4 zero4 = {0u, 0u, 0u, 0u};
    if (out_head0) {
        for (int idx = threadIdx.x; idx < N * kPiecesPerRow; idx += kThreads) {
            const int n = idx / kPiecesPerRow, p = idx - n * kPiecesPerRow;
            if (keep_img[n] == 0) out_head0[(int64_t)n * row_vec + p] = zero4;
        }
    }
    if (cls_head && keep_img[0] == 0 && threadIdx.x < kPiecesPerRow) cls_head[threadIdx.x] = zero4;
}

template <typename T>
__global__ __launch_bounds__(kThreads) void fused16(const uint16_t *__restrict__ q,
                                                    const uint16_t *__restrict__ k,
                                                    const uint16_t *__restrict__ v,
                                                    const uint8_t *__restrict__ keep,
                                                    uint16_t *__restrict__ out,
                                                    uint16_t *__restrict__ cls, int B, int N,
                                                    int H, int ntiles, float c) {
    __shared__ __attribute__((aligned(16))) uint16_t sK[2 * kKC * 64];
    __shared__ __attribute__((aligned(16))) uint16_t sV[2 * kD * 64];
    __shared__ int16_t pos[kMaxFusedN];
    __shared__ int s_count;
    int b, h, tile;
    if (!decode_tile(B, H, ntiles, &b, &h, &tile)) return;
    const uint8_t *keep_img = keep + (int64_t)b * N;
    const int L = rank_image(keep_img, N, pos, &s_count);
    const int64_t rs = (int64_t)H * kD;
    const int64_t head0 = (int64_t)b * N * rs + (int64_t)h * kD;  // (b, 0, h)
    uint16_t *cls_head = cls ? cls + ((int64_t)b * H + h) * kD : nullptr;
    if (tile == 0)
        zero_pruned<kD * 2 / 16>(keep_img, N, out ? (u32x4 *)(out + head0) : nullptr, rs * 2 / 16,
                                 (u32x4 *)cls_head);
    const int q0 = tile * kQT;
    if (q0 >= L) return;
    const PaddedRows R = {head0, rs, pos};
    // the output row of query rank 0 is the CLS row iff position 0 was kept
    uint16_t *cls_dst = (cls_head && pos[0] == 0) ? cls_head : nullptr;
    if (out) {
        attend16<T>(q, k, v, out, R, L, q0, c, sK, sV, cls_dst);
    } else {
        // CLS rows only: only the tile holding rank 0 has work
        if (tile != 0 || !cls_dst) return;
        attend16<T>(q, k, v, nullptr, R, L, q0, c, sK, sV, cls_dst);
    }
}

__global__ __launch_bounds__(kThreads) void fused32(const float *__restrict__ q,
                                                    const float *__restrict__ k,
                                                    const float *__restrict__ v,
                                                    const uint8_t *__restrict__ keep,
                                                    float *__restrict__ out,
                                                    float *__restrict__ cls, int B, int N, int H,
                                                    int ntiles, float c) {
    __shared__ __attribute__((aligned(16))) float sK[2 * kKC32 * kLd32];
    __shared__ __attribute__((aligned(16))) float sV[2 * kKC32 * kLd32];
    __shared__ int16_t pos[kMaxFusedN];
    __shared__ int s_count;
    int b, h, tile;
    if (!decode_tile(B, H, ntiles, &b, &h, &tile)) return;
    const uint8_t *keep_img = keep + (int64_t)b * N;
    const int L = rank_image(keep_img, N, pos, &s_count);
    const int64_t rs = (int64_t)H * kD;
    const int64_t head0 = (int64_t)b * N * rs + (int64_t)h * kD;
    float *cls_head = cls ? cls + ((int64_t)b * H + h) * kD : nullptr;
    if (tile == 0)
        zero_pruned<kD * 4 / 16>(keep_img, N, out ? (u32x4 *)(out + head0) : nullptr, rs * 4 / 16,
                                 (u32x4 *)cls_head);
    const int q0 = tile * kQT;
    if (q0 >= L) return;
    const PaddedRows R = {head0, rs, pos};
    float *cls_dst = (cls_head && pos[0] == 0) ? cls_head : nullptr;
    if (out) {
        attend32(q, k, v, out, R, L, q0, c, sK, sV, cls_dst);
    } else {
        if (tile != 0 || !cls_dst) return;
        attend32(q, k, v, nullptr, R, L, q0, c, sK, sV, cls_dst);
    }
}

int64_t grid_for(int B, int H, int ntiles) {
    const int64_t pairs = (int64_t)B * H;
    return 8 * ((pairs + 7) / 8) * ntiles;
}

}  // namespace

hipError_t launch_attention(const AttnArgs &a, hipStream_t s) {
    const int ntiles = (a.max_seqlen + kQT - 1) / kQT;
    const unsigned grid = (unsigned)grid_for(a.B, a.H, ntiles);
    const float c = a.scale * kLog2e;
    switch (a.dt) {
    case Elem::BF16:
        hipLaunchKernelGGL(attn_fwd16<__bf16>, dim3(grid), dim3(kThreads), 0, s,
                           (const uint16_t *)a.q, (const uint16_t *)a.k, (const uint16_t *)a.v,
                           (uint16_t *)a.o, a.cu, a.B, a.H, ntiles, c);
        break;
    case Elem::F16:
        hipLaunchKernelGGL(attn_fwd16<_Float16>, dim3(grid), dim3(kThreads), 0, s,
                           (const uint16_t *)a.q, (const uint16_t *)a.k, (const uint16_t *)a.v,
                           (uint16_t *)a.o, a.cu, a.B, a.H, ntiles, c);
        break;
    case Elem::F32:
        hipLaunchKernelGGL(attn_fwd32, dim3(grid), dim3(kThreads), 0, s, (const float *)a.q,
                           (const float *)a.k, (const float *)a.v, (float *)a.o, a.cu, a.B, a.H,
                           ntiles, c);
        break;
    }
    return hipGetLastError();
}

hipError_t launch_fused(const FusedArgs &a, hipStream_t s) {
    const int ntiles = (a.max_seqlen + kQT - 1) / kQT;
    const unsigned grid = (unsigned)grid_for(a.B, a.H, ntiles > 0 ? ntiles : 1);
    const int nt = ntiles > 0 ? ntiles : 1;
    const float c = a.scale * kLog2e;
    switch (a.dt) {
    case Elem::BF16:
        hipLaunchKernelGGL(fused16<__bf16>, dim3(grid), dim3(kThreads), 0, s,
                           (const uint16_t *)a.q, (const uint16_t *)a.k, (const uint16_t *)a.v,
                           a.keep, (uint16_t *)a.out, (uint16_t *)a.cls, a.B, a.N, a.H, nt, c);
        break;
    case Elem::F16:
        hipLaunchKernelGGL(fused16<_Float16>, dim3(grid), dim3(kThreads), 0, s,
                           (const uint16_t *)a.q, (const uint16_t *)a.k, (const uint16_t *)a.v,
                           a.keep, (uint16_t *)a.out, (uint16_t *)a.cls, a.B, a.N, a.H, nt, c);
        break;
    case Elem::F32:
        hipLaunchKernelGGL(fused32, dim3(grid), dim3(kThreads), 0, s, (const float *)a.q,
                           (const float *)a.k, (const float *)a.v, a.keep, (float *)a.out,
                           (float *)a.cls, a.B, a.N, a.H, nt, c);
        break;
    }
    return hipGetLastError();
}

}  // namespace rattn
