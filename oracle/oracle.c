/*
 * oracle.c -- plain, slow, obviously correct CPU reference of the token-pruned
 * ViT pack -> attend -> unpack path.  TEST INFRASTRUCTURE ONLY: the tests, the
 * smoke check and the benchmark's CPU-baseline leg may call it; the product
 * path never does.  It shares no code, header, table or helper with the HIP
 * library.
 *
 * Citations (pages on "Dispatch-Aware Ragged Attention for Pruned Vision
 * Transformers", arXiv 2604.15408):
 *   [Abstract]   the paper abstract: ragged attention over the kept tokens of
 *                each image, bidirectional, at ViT lengths.
 *   [Padding]    radpulse.milrad-way.com write-up, section on how pruning plus
 *                padding makes PyTorch regress: the dense alternative pads every
 *                image to the longest survivor and masks the rest.
 *   [FA2]        same write-up, section on FlashAttention-2's 62 us dispatch
 *                ceiling: survivors are compressed into one contiguous ragged
 *                buffer described by cumulative sequence lengths (cu_seqlens).
 *   [Triton]     same write-up, section on the 40 us Triton bidirectional
 *                kernel: no causal mask and no KV cache.
 *   [Pipeline]   same write-up, section on the integrated packing pipeline:
 *                compute cu_seqlens, copy the surviving tokens into a
 *                contiguous flat tensor, attend, then take the CLS token; the
 *                pipeline is agnostic to the pruning method, including methods
 *                that prune again at later blocks.
 *
 * Readings where the pages leave a step open:
 *   - keep mask is one byte per token, nonzero = kept;
 *   - cu_seqlens is int32 [B+1] with cu[0] = 0 (exclusive prefix sum);
 *   - inside the flat buffer, images are in ascending b and, within an image,
 *     tokens are in ascending position n (a stable compaction);
 *   - pruned rows of the unpacked output are all-zero bytes (+0.0);
 *   - the CLS row of image b is the unpacked row (b, 0).
 *
 * Precision: every attention quantity is double; inputs arrive already widened
 * exactly from their storage type.  The softmax is the textbook two-pass one:
 * maximum, exponentials, sum, weighted sum, one division.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* [Pipeline] step 1: per-image kept count, exclusive prefix sum over images.
 * Writes cu[0..B]; *max_seqlen = largest count; *total = cu[B].
 * Returns 0, or -1 on a bad argument. */
int oracle_scan(const uint8_t *keep, int B, int N, int32_t *cu,
                int32_t *max_seqlen, int32_t *total)
{
    if (B < 0 || N < 0 || (B > 0 && (!keep || !cu))) return -1;
    int32_t running = 0, mx = 0;
    if (cu) cu[0] = 0;
    for (int b = 0; b < B; ++b) {
        int32_t cnt = 0;
        for (int n = 0; n < N; ++n)
            if (keep[(int64_t)b * N + n] != 0) cnt += 1;
        running += cnt;
        cu[b + 1] = running;
        if (cnt > mx) mx = cnt;
    }
    if (max_seqlen) *max_seqlen = mx;
    if (total) *total = running;
    return 0;
}

/* [Pipeline] step 2: copy the rows of kept tokens, in order, into a flat
 * buffer.  src is [B, N, row_bytes], dst receives [T, row_bytes].  Bitwise.
 * Returns the number of rows written. */
int64_t oracle_pack(const uint8_t *src, uint8_t *dst, const uint8_t *keep,
                    int B, int N, int64_t row_bytes)
{
    int64_t r = 0;
    for (int b = 0; b < B; ++b)
        for (int n = 0; n < N; ++n) {
            int64_t t = (int64_t)b * N + n;
            if (keep[t] != 0) {
                memcpy(dst + r * row_bytes, src + t * row_bytes, (size_t)row_bytes);
                r += 1;
            }
        }
    return r;
}

/* [Pipeline], a second pruning stage: compact an already packed buffer under a
 * second keep flag per flat row.  src is [T, row_bytes] with T = cu[B]; keep2
 * is [T] (nonzero = keep); dst receives the kept rows, images in order and rows
 * in order within each image; cu2[0..B] is the prefix sum of the new per-image
 * counts.  Bitwise.  Returns the number of rows written, or -1 when cu
 * decreases. */
int64_t oracle_repack(const uint8_t *src, uint8_t *dst, const uint8_t *keep2,
                      const int32_t *cu, int B, int64_t row_bytes, int32_t *cu2)
{
    int64_t r = 0;
    cu2[0] = 0;
    for (int b = 0; b < B; ++b) {
        if (cu[b + 1] < cu[b]) return -1;
        for (int64_t t = cu[b]; t < cu[b + 1]; ++t)
            if (keep2[t] != 0) {
                memcpy(dst + r * row_bytes, src + t * row_bytes, (size_t)row_bytes);
                r += 1;
            }
        cu2[b + 1] = (int32_t)r;
    }
    return r;
}

/* Image that owns flat row t, found by walking cu (cu is nondecreasing). */
static int owner_image(const int32_t *cu, int B, int64_t t)
{
    for (int b = 0; b < B; ++b)
        if (t >= cu[b] && t < cu[b + 1]) return b;
    return -1;
}

/* [Abstract], [FA2], [Triton]: bidirectional multi-head attention over the
 * ragged buffer.  q, k, v are [T, H, D] doubles (T = cu[B]).  For query row i
 * of image b and head h, the keys are exactly the rows of image b:
 *     s_j = scale * <q_i, k_j>,   p_j = exp(s_j - max s),   o_i = sum p_j v_j / sum p_j.
 * No causal mask, no cache, nothing from another image.
 *
 * rows == NULL: every flat row, o is [T, H, D].
 * rows != NULL: only the nrows listed flat rows, o is [nrows, H, D].
 * absw (nullable, same shape as o) receives sum_j p_j |v_j| / sum_j p_j, a
 * magnitude used to size rounding tolerances.
 * Returns 0, or -1 on a bad argument / allocation failure. */
int oracle_attention(const double *q, const double *k, const double *v,
                     const int32_t *cu, int B, int H, int D, double scale,
                     const int64_t *rows, int64_t nrows, double *o, double *absw)
{
    if (B < 0 || H <= 0 || D <= 0 || !cu) return -1;
    int64_t T = cu[B];
    int64_t count = rows ? nrows : T;
    int32_t maxlen = 0;
    for (int b = 0; b < B; ++b)
        if (cu[b + 1] - cu[b] > maxlen) maxlen = cu[b + 1] - cu[b];
    double *s = (double *)malloc(sizeof(double) * (size_t)(maxlen > 0 ? maxlen : 1));
    if (!s) return -1;
    const int64_t rs = (int64_t)H * D; /* row stride of [T, H, D] */

    for (int64_t c = 0; c < count; ++c) {
        int64_t i = rows ? rows[c] : c;
        int b = owner_image(cu, B, i);
        if (b < 0) { free(s); return -1; }
        int64_t j0 = cu[b], L = cu[b + 1] - cu[b];
        for (int h = 0; h < H; ++h) {
            const double *qi = q + i * rs + (int64_t)h * D;
            /* pass 1: scores and their maximum */
            double m = -INFINITY;
            for (int64_t jj = 0; jj < L; ++jj) {
                const double *kj = k + (j0 + jj) * rs + (int64_t)h * D;
                double dot = 0.0;
                for (int d = 0; d < D; ++d) dot += qi[d] * kj[d];
                s[jj] = scale * dot;
                if (s[jj] > m) m = s[jj];
            }
            /* pass 2: exponentials, their sum, weighted sum of values */
            double l = 0.0;
            for (int64_t jj = 0; jj < L; ++jj) {
                s[jj] = exp(s[jj] - m);
                l += s[jj];
            }
            double *oi = o + c * rs + (int64_t)h * D;
            double *ai = absw ? absw + c * rs + (int64_t)h * D : NULL;
            for (int d = 0; d < D; ++d) {
                double acc = 0.0, aacc = 0.0;
                for (int64_t jj = 0; jj < L; ++jj) {
                    double vj = v[(j0 + jj) * rs + (int64_t)h * D + d];
                    acc += s[jj] * vj;
                    aacc += s[jj] * fabs(vj);
                }
                oi[d] = acc / l;
                if (ai) ai[d] = aacc / l;
            }
        }
    }
    free(s);
    return 0;
}

/* [Pipeline] last step, and the inverse of the packing copy: row r of the flat
 * buffer goes back to the position of the r-th kept token; pruned positions
 * become zero bytes.  src is [T, row_bytes] with T = cu[B]; dst (nullable) is
 * [B, N, row_bytes]; cls (nullable) is [B, row_bytes] and receives row (b, 0)
 * of the unpacked output, i.e. the CLS token when it was kept, zeros if not.
 * Returns 0, or -1 when an image's kept count disagrees with cu. */
int oracle_unpack(const uint8_t *src, uint8_t *dst, uint8_t *cls,
                  const uint8_t *keep, const int32_t *cu, int B, int N,
                  int64_t row_bytes)
{
    for (int b = 0; b < B; ++b) {
        int64_t r = cu[b];
        for (int n = 0; n < N; ++n) {
            int64_t t = (int64_t)b * N + n;
            const uint8_t *from = NULL;
            if (keep[t] != 0) {
                from = src + r * row_bytes;
                r += 1;
            }
            if (dst) {
                if (from) memcpy(dst + t * row_bytes, from, (size_t)row_bytes);
                else memset(dst + t * row_bytes, 0, (size_t)row_bytes);
            }
            if (cls && n == 0) {
                if (from) memcpy(cls + (int64_t)b * row_bytes, from, (size_t)row_bytes);
                else memset(cls + (int64_t)b * row_bytes, 0, (size_t)row_bytes);
            }
        }
        if (r != cu[b + 1]) return -1;
    }
    return 0;
}
