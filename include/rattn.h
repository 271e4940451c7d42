/*
 * rattn.h -- C ABI of librattn.so: the pack -> attend -> unpack hot path of
 * token-pruned Vision Transformers on AMD Instinct MI355X (gfx950).
 *
 * Source of the operations (pages on "Dispatch-Aware Ragged Attention for
 * Pruned Vision Transformers", arXiv 2604.15408):
 *   [Abstract]  paper abstract: bidirectional attention over ragged
 *               (variable-length) token sets after pruning, at ViT lengths;
 *               host-side dispatch cost is the quantity to drive down.
 *   [FA2]       radpulse.milrad-way.com write-up, section on FlashAttention-2's
 *               62 us dispatch ceiling: survivors compressed into one contiguous
 *               ragged buffer, described by cumulative sequence lengths, and
 *               handed to a variable-length attention call; validation, binding
 *               crossings, output allocation and launch make up the floor.
 *   [Triton]    same write-up, section on the 40 us Triton bidirectional
 *               kernel: no causal mask, no KV cache, no per-call softmax_lse
 *               workspace, arguments written straight into the launch.
 *   [Pipeline]  same write-up, section on the integrated packing pipeline:
 *               compute cu_seqlens, copy surviving tokens with coalesced
 *               accesses into a contiguous flat tensor, attend, extract CLS.
 *   [Padding]   same write-up, section on why pruning plus padding makes the
 *               dense path regress: every image padded to the longest
 *               survivor, the padding masked, the padded work still done.
 *
 * Conventions shared by every entry point:
 *   - All data pointers are DEVICE pointers owned by the caller (hipMalloc,
 *     torch, ...).  The library allocates nothing per call and keeps no
 *     pointer after the call returns.
 *   - Calls are asynchronous and stream-ordered: they enqueue work on
 *     `stream` (a hipStream_t; NULL = the default stream of the current
 *     device) and return without synchronising.  Results are visible to later
 *     work on the same stream.
 *   - Data pointers (tensors, keep) must be 16-byte aligned; cu_seqlens and
 *     the optional int32 outputs 4-byte aligned.  Tensors are dense,
 *     row-major, with no padding between rows.
 *   - Keep mask: uint8 [B, N]; a nonzero byte keeps the token.
 *   - cu_seqlens: int32 [B+1], cu[0] = 0, cu[b+1] - cu[b] = kept tokens of
 *     image b.  Inside the flat buffer images are in ascending b and tokens of
 *     one image in ascending position (a stable compaction).
 *   - Errors: every argument check runs on the host before any HIP call and
 *     returns RATTN_ERR_INVALID_ARG / RATTN_ERR_UNSUPPORTED with nothing
 *     enqueued.  A failed launch returns RATTN_ERR_HIP.  Faults inside kernels
 *     surface, as usual for HIP, at the caller's next synchronisation.
 *   - Contract the host cannot check without a device round trip: cu_seqlens
 *     must agree with the buffers' capacities, and max_seqlen must be >= every
 *     image's kept count.  Any such upper bound (N always is one) gives
 *     bitwise-identical results.  The opt-in debug-validate mode
 *     (rattn_set_validate) checks the bound and the shape of cu_seqlens with a
 *     device-to-host read before launching.
 *   - Order of the softmax accumulation: in a batch of few heads (B * H <= 24
 *     for RATTN_BF16 / RATTN_F16, <= 64 for RATTN_F32) an image longer than
 *     one key chunk (64 keys; every image for RATTN_F32) has its keys split
 *     over four partial softmax states, merged in a fixed order; otherwise
 *     each query row takes the keys in one sequence.  An image's output bits
 *     can therefore differ, within rounding, between batches whose head counts
 *     fall on different sides of those limits.  They never depend on the
 *     other images' contents, the bound, the padded length or the entry point
 *     (fused, three calls or padded comparator).
 *   - Thread safety: entry points may be called from several threads, on
 *     the same or different streams; the only global state is the one-time
 *     device check of rattn_init, the debug-validate flag, and a per-device
 *     table of kernel handles that each kernel's first launch on a device
 *     fills (atomically; a racing second lookup stores the same handle).
 *     No call keeps anything on the device between calls, so calls on
 *     different streams share nothing but their arguments.
 */
#ifndef RATTN_H
#define RATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum rattn_status {
    RATTN_OK = 0,
    RATTN_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad size, bad enum  */
    RATTN_ERR_UNSUPPORTED = 2, /* valid but not implemented (e.g. head_dim != 64) */
    RATTN_ERR_NO_DEVICE = 3,   /* no HIP device, or not a gfx950 device           */
    RATTN_ERR_HIP = 4          /* a HIP runtime call (launch) failed              */
} rattn_status;

typedef enum rattn_dtype {
    RATTN_F32 = 0,  /* IEEE binary32                       */
    RATTN_F16 = 1,  /* IEEE binary16                       */
    RATTN_BF16 = 2  /* bfloat16 (upper half of a binary32) */
} rattn_dtype;

#define RATTN_HEAD_DIM 64      /* the only head_dim rattn_forward accepts     */
#define RATTN_MAX_TENSORS 3    /* rattn_pack copies up to q, k and v at once  */
#define RATTN_MAX_TOKENS 2147483647 /* B*N and T must fit in int32            */
#define RATTN_MAX_FUSED_N 2048 /* longest padded sequence rattn_fused accepts  */
/* Largest span, in bytes, of one image's rows of one tensor (max_seqlen rows
 * for rattn_forward, N rows for rattn_fused): row offsets inside an image are
 * 32-bit in the kernels.  Larger configurations return RATTN_ERR_UNSUPPORTED. */
#define RATTN_MAX_IMAGE_BYTES 2147483648LL

/* Checks once that a gfx950 device is present.  Idempotent and thread-safe;
 * called implicitly by the entry points.  RATTN_ERR_NO_DEVICE otherwise. */
rattn_status rattn_init(void);

/* Static, human-readable name of a status code (never NULL). */
const char *rattn_status_string(rattn_status s);

/* ABI version of this header: (major << 16) | minor. */
int rattn_version(void);

/*
 * rattn_set_validate -- opt-in debug-validate mode for the contract a call
 * cannot check from its host arguments alone ([FA2]: the flat buffer and its
 * cumulative lengths are only as good as the caller's bookkeeping).
 *
 *   on          nonzero switches the mode on for the whole process, 0 off
 *               (the default).  Returns the previous setting (0 or 1).
 *
 * In the mode, after the host checks and before any launch, an entry point
 * copies what it needs to host memory, ordered after the earlier work on its
 * stream, waits for it, and returns RATTN_ERR_INVALID_ARG with nothing
 * launched when:
 *   rattn_forward       cu_seqlens[0] != 0, cu_seqlens decreases, or an image
 *                       has more rows than max_seqlen;
 *   rattn_fused         an image keeps more tokens than max_seqlen;
 *   rattn_fused_padded  an image keeps more tokens than pad_len;
 *   rattn_unpack        cu_seqlens is not the prefix sum of keep's counts;
 *   rattn_repack        cu_seqlens[0] != 0 or cu_seqlens decreases.
 * A failed copy or wait returns RATTN_ERR_HIP.  The mode makes those calls
 * synchronous and costs a device-to-host round trip each: it is for
 * debugging, and cannot be used under stream capture.  rattn_pack computes
 * cu_seqlens itself and is unaffected.  Thread-safe (an atomic flag).
 */
int rattn_set_validate(int on);

/* Current debug-validate setting: 1 on, 0 off. */
int rattn_get_validate(void);

/*
 * rattn_pack -- [Pipeline] steps 1 and 2: cu_seqlens and the coalesced pack.
 *
 *   src[i]      device, [B, N, row_elems] elements of `dt` (padded input i)
 *   dst[i]      device, [>= T, row_elems]: receives the kept rows of src[i],
 *               row r = r-th kept token in (b, n) order; capacity B*N rows is
 *               always enough.  Rows >= T are not written.
 *   n_tensors   1..RATTN_MAX_TENSORS (src and dst are host arrays of that
 *               many device pointers; all tensors share keep and row_elems)
 *   keep        device, uint8 [B, N]
 *   B, N        images and padded tokens per image; B >= 0, N >= 1,
 *               B*N <= RATTN_MAX_TOKENS
 *   row_elems   elements per token row (H*head_dim); row bytes must be a
 *               positive multiple of 16
 *   cu_seqlens  device, int32 [B+1] (output)
 *   max_seqlen_dev, total_dev  device int32 scalars (outputs, each nullable):
 *               largest kept count, and T = cu[B]
 * The copy is bitwise.  B = 0 writes cu[0] = 0 (and zeros to the scalars).
 */
rattn_status rattn_pack(const void *const *src, void *const *dst, int n_tensors,
                        const uint8_t *keep, int B, int N, int row_elems,
                        rattn_dtype dt, int32_t *cu_seqlens, int32_t *max_seqlen_dev,
                        int32_t *total_dev, void *stream);

/*
 * rattn_forward -- [Abstract], [FA2], [Triton]: bidirectional multi-head
 * attention over the ragged buffer.  For image b, head h and every query row i
 * in [cu[b], cu[b+1]):
 *     o[i,h,:] = sum_j softmax_j(scale * <q[i,h,:], k[j,h,:]>) v[j,h,:]
 * with j ranging over the rows of the same image only.  No causal mask, no KV
 * cache, no log-sum-exp output.
 *
 *   q, k, v     device, [>= T, H, head_dim] of `dt` (T = cu[B])
 *   o           device, [>= T, H, head_dim] of `dt` (output; only rows < T
 *               are written)
 *   cu_seqlens  device, int32 [B+1]
 *   B           images (>= 0)
 *   max_seqlen  host upper bound on every kept count (>= 0; 0 = nothing to do;
 *               max_seqlen * H * head_dim * element size must not exceed
 *               RATTN_MAX_IMAGE_BYTES).  An image whose kept count exceeds it
 *               breaks the contract: its output rows are left unwritten, or,
 *               in debug-validate mode, the call returns
 *               RATTN_ERR_INVALID_ARG before launching.
 *   H           heads (>= 1);  head_dim must be RATTN_HEAD_DIM
 *   scale       finite float multiplying the dot products (1/sqrt(64) for ViT)
 * Arithmetic: q.k and p.v contractions on the matrix cores with float32
 * accumulation (bf16/fp16 inputs; probabilities rounded to the input type for
 * the second contraction), float32 online softmax, output rounded to nearest
 * even.  RATTN_F32 inputs keep every step in float32.
 */
rattn_status rattn_forward(const void *q, const void *k, const void *v, void *o,
                           const int32_t *cu_seqlens, int B, int max_seqlen, int H,
                           int head_dim, float scale, rattn_dtype dt, void *stream);

/*
 * rattn_unpack -- [Pipeline] final step: back to the padded layout, and the
 * CLS rows.
 *
 *   src         device, [>= T, row_elems] of `dt` (flat, e.g. rattn_forward's o)
 *   dst_padded  device, [B, N, row_elems] (nullable): kept positions receive
 *               their flat row, pruned positions all-zero bytes (+0.0)
 *   cls         device, [B, row_elems] (nullable): row (b, 0) of the padded
 *               result, i.e. the CLS token's row, zeros when it was pruned
 *   keep, cu_seqlens, B, N, row_elems, dt: as for rattn_pack
 * At least one of dst_padded / cls must be non-NULL.  The copy is bitwise.
 */
rattn_status rattn_unpack(const void *src, void *dst_padded, void *cls,
                          const uint8_t *keep, const int32_t *cu_seqlens, int B, int N,
                          int row_elems, rattn_dtype dt, void *stream);

/*
 * rattn_fused -- [Pipeline] in ONE launch: the pack, the attention and the
 * unpack / CLS extract of a whole batch, from the padded tensors to the padded
 * output, with no flat intermediate and no cu_seqlens.  Each workgroup ranks
 * its image's kept tokens from the mask itself, gathers the kept q/k/v rows
 * from their padded positions and writes each output row back to its own
 * position.  Same arithmetic, and bit-for-bit the same outputs, as
 * rattn_pack + rattn_forward + rattn_unpack; the per-call dispatch cost the
 * pages put first ([Abstract], [FA2], [Triton]) is paid once instead of three
 * times, and the flat buffers' traffic disappears.
 *
 *   q, k, v     device, padded [B, N, H, head_dim] of `dt`
 *   keep        device, uint8 [B, N]
 *   out_padded  device, [B, N, H, head_dim] (nullable): kept positions get
 *               the attention output, pruned positions all-zero bytes
 *   cls         device, [B, H, head_dim] (nullable): row (b, 0) of that
 *               output (zeros when the CLS token was pruned)
 *   B, N, H     B >= 0, 1 <= N <= RATTN_MAX_FUSED_N, 1 <= H, H * head_dim
 *               < 2^24, and N * H * head_dim * element size <=
 *               RATTN_MAX_IMAGE_BYTES
 *   head_dim    must be RATTN_HEAD_DIM
 *   max_seqlen  host upper bound on every kept count (N is always valid)
 *   scale, dt   as for rattn_forward
 * At least one of out_padded / cls must be non-NULL.
 */
rattn_status rattn_fused(const void *q, const void *k, const void *v, const uint8_t *keep,
                         void *out_padded, void *cls, int B, int N, int H, int head_dim,
                         int max_seqlen, float scale, rattn_dtype dt, void *stream);

/*
 * rattn_repack -- [Pipeline] with a later pruning stage: compact an already
 * packed buffer under a second keep flag per flat row, so that the buffer
 * stays ragged from one stage to the next.  Within each image the kept rows
 * keep their order; images stay in order.  Bitwise row copies.
 *
 *   src         n_tensors (1..3) device pointers, [>= T, row_elems] of `dt`
 *               each, T = cu_seqlens[B]
 *   dst         n_tensors device pointers, [>= T2, row_elems] each (T2 = rows
 *               kept; T is always enough); must not overlap src
 *   keep2       device uint8 [>= T], 16-byte aligned: nonzero keeps the row
 *   cu_seqlens  device int32 [B+1] of src
 *   cu_seqlens_out  device int32 [B+1] (output), must not overlap cu_seqlens
 *   total_dev   device int32 scalar (output, nullable): T2
 * The longest image cannot grow, so a max_seqlen bound valid before the
 * re-pack stays valid after it.
 */
rattn_status rattn_repack(const void *const *src, void *const *dst, int n_tensors,
                          const uint8_t *keep2, const int32_t *cu_seqlens, int B, int row_elems,
                          rattn_dtype dt, int32_t *cu_seqlens_out, int32_t *total_dev,
                          void *stream);

/*
 * rattn_fused_padded -- [Padding]: the dense comparator of rattn_fused.  Every
 * image is processed as if it had pad_len tokens: its kept tokens first, the
 * rest padding whose keys are masked out and whose query rows are computed
 * and discarded -- the work a padded, masked attention does when each image
 * is padded to the longest survivor (pad_len = max kept count) or not pruned
 * at all (pad_len = N).  The outputs are bit-for-bit those of rattn_fused
 * (masked keys contribute exactly zero); only the work differs.
 *
 *   pad_len     1 <= pad_len <= N, and >= every image's kept count (an image
 *               with more kept tokens is processed at its own length)
 *   all other arguments as for rattn_fused (max_seqlen is pad_len)
 */
rattn_status rattn_fused_padded(const void *q, const void *k, const void *v, const uint8_t *keep,
                                void *out_padded, void *cls, int B, int N, int H, int head_dim,
                                int pad_len, float scale, rattn_dtype dt, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* RATTN_H */
