// api.hip -- the extern "C" entry points of librattn.so (declared, with their
// contracts, in include/rattn.h).
//
// The host path is deliberately thin, because per-call host dispatch is the
// cost the pages single out (paper abstract; radpulse.milrad-way.com write-up,
// sections on FlashAttention-2's 62 us dispatch ceiling and on the Triton
// kernel that writes its arguments straight into the launch): plain-int
// argument checks, one kernel-argument struct built on the stack, one launch
// per kernel, no allocation, no device-to-host traffic, no synchronisation.
// The one exception is the debug-validate mode a caller may switch on
// (rattn_set_validate), which reads the kept counts back to check the
// contract before launching.
#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>
#include <vector>

#include "internal.h"
#include "rattn.h"

using namespace rattn;

namespace {

std::once_flag g_once;
rattn_status g_init = RATTN_ERR_NO_DEVICE;
// debug-validate mode (rattn_set_validate): off unless a caller opts in
std::atomic<int> g_validate{0};

inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
inline bool aligned4(const void *p) { return ((uintptr_t)p & 3u) == 0; }

inline int elem_size(rattn_dtype dt) {
    switch (dt) {
    case RATTN_F32: return 4;
    case RATTN_F16: return 2;
    case RATTN_BF16: return 2;
    }
    return 0;
}

inline Elem to_elem(rattn_dtype dt) {
    return dt == RATTN_F32 ? Elem::F32 : dt == RATTN_F16 ? Elem::F16 : Elem::BF16;
}

// Row geometry shared by pack and unpack; 0 rows-of-16-bytes means invalid.
inline int row_vectors(int row_elems, rattn_dtype dt) {
    const int es = elem_size(dt);
    if (es == 0 || row_elems <= 0) return 0;
    const int64_t bytes = (int64_t)row_elems * es;
    if (bytes % 16 != 0 || bytes / 16 > (1 << 24)) return 0;
    return (int)(bytes / 16);
}

// ---------------------------------------------------------------------------
// debug-validate mode: the parts of the contract the host cannot see without
// reading device memory.  Each check copies what it needs to host memory,
// ordered after the earlier work on the caller's stream, and waits for it.
// ---------------------------------------------------------------------------
inline bool validating() { return g_validate.load(std::memory_order_relaxed) != 0; }

rattn_status read_back(void *host, const void *dev, size_t n, hipStream_t s) {
    if (n == 0) return RATTN_OK;
    if (hipMemcpyAsync(host, dev, n, hipMemcpyDeviceToHost, s) != hipSuccess) return RATTN_ERR_HIP;
    return hipStreamSynchronize(s) == hipSuccess ? RATTN_OK : RATTN_ERR_HIP;
}

// cu_seqlens must start at 0 and never decrease; *longest = its largest step.
rattn_status validate_cu(const int32_t *cu_dev, int B, hipStream_t s, std::vector<int32_t> &cu,
                         int *longest) {
    cu.assign((size_t)B + 1, 0);
    rattn_status st = read_back(cu.data(), cu_dev, cu.size() * sizeof(int32_t), s);
    if (st != RATTN_OK) return st;
    if (cu[0] != 0) return RATTN_ERR_INVALID_ARG;
    int m = 0;
    for (int b = 0; b < B; ++b) {
        const int64_t d = (int64_t)cu[b + 1] - cu[b];
        if (d < 0) return RATTN_ERR_INVALID_ARG;
        if (d > m) m = (int)d;
    }
    *longest = m;
    return RATTN_OK;
}

// Kept count of every image of a [B, N] mask.
rattn_status kept_counts(const uint8_t *keep_dev, int B, int N, hipStream_t s,
                         std::vector<int32_t> &cnt) {
    std::vector<uint8_t> keep((size_t)B * N);
    rattn_status st = read_back(keep.data(), keep_dev, keep.size(), s);
    if (st != RATTN_OK) return st;
    cnt.assign((size_t)B, 0);
    for (int b = 0; b < B; ++b) {
        const uint8_t *row = keep.data() + (size_t)b * N;
        int c = 0;
        for (int n = 0; n < N; ++n) c += row[n] != 0;
        cnt[b] = c;
    }
    return RATTN_OK;
}

// The bound passed with a padded batch must cover every image's kept count.
rattn_status validate_bound(const uint8_t *keep_dev, int B, int N, int bound, hipStream_t s) {
    std::vector<int32_t> cnt;
    rattn_status st = kept_counts(keep_dev, B, N, s, cnt);
    if (st != RATTN_OK) return st;
    for (int b = 0; b < B; ++b)
        if (cnt[b] > bound) return RATTN_ERR_INVALID_ARG;
    return RATTN_OK;
}

// cu_seqlens must be the prefix sum of the mask's kept counts.
rattn_status validate_cu_against_mask(const int32_t *cu_dev, const uint8_t *keep_dev, int B,
                                      int N, hipStream_t s) {
    std::vector<int32_t> cu, cnt;
    int longest = 0;
    rattn_status st = validate_cu(cu_dev, B, s, cu, &longest);
    if (st != RATTN_OK) return st;
    st = kept_counts(keep_dev, B, N, s, cnt);
    if (st != RATTN_OK) return st;
    for (int b = 0; b < B; ++b)
        if ((int64_t)cu[b + 1] - cu[b] != cnt[b]) return RATTN_ERR_INVALID_ARG;
    return RATTN_OK;
}

}  // namespace

extern "C" {

rattn_status rattn_init(void) {
    std::call_once(g_once, [] {
        int n = 0;
        if (hipGetDeviceCount(&n) != hipSuccess || n <= 0) return;
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess) return;
        hipDeviceProp_t p;
        if (hipGetDeviceProperties(&p, dev) != hipSuccess) return;
        if (std::strncmp(p.gcnArchName, "gfx950", 6) != 0) return;
        g_init = RATTN_OK;
    });
    return g_init;
}

const char *rattn_status_string(rattn_status s) {
    switch (s) {
    case RATTN_OK: return "RATTN_OK";
    case RATTN_ERR_INVALID_ARG: return "RATTN_ERR_INVALID_ARG: invalid argument";
    case RATTN_ERR_UNSUPPORTED: return "RATTN_ERR_UNSUPPORTED: unsupported configuration";
    case RATTN_ERR_NO_DEVICE: return "RATTN_ERR_NO_DEVICE: no gfx950 HIP device";
    case RATTN_ERR_HIP: return "RATTN_ERR_HIP: HIP runtime call failed";
    }
    return "RATTN_ERR_UNKNOWN";
}

int rattn_version(void) { return (1 << 16) | 1; }

int rattn_set_validate(int on) { return g_validate.exchange(on != 0 ? 1 : 0); }

int rattn_get_validate(void) { return g_validate.load(); }

rattn_status rattn_pack(const void *const *src, void *const *dst, int n_tensors,
                        const uint8_t *keep, int B, int N, int row_elems, rattn_dtype dt,
                        int32_t *cu_seqlens, int32_t *max_seqlen_dev, int32_t *total_dev,
                        void *stream) {
    if (n_tensors < 1 || n_tensors > RATTN_MAX_TENSORS || !src || !dst) return RATTN_ERR_INVALID_ARG;
    if (B < 0 || N < 1 || (int64_t)B * N > RATTN_MAX_TOKENS) return RATTN_ERR_INVALID_ARG;
    const int rv = row_vectors(row_elems, dt);
    if (rv == 0) return RATTN_ERR_INVALID_ARG;
    if (!cu_seqlens || !aligned4(cu_seqlens)) return RATTN_ERR_INVALID_ARG;
    if (max_seqlen_dev && !aligned4(max_seqlen_dev)) return RATTN_ERR_INVALID_ARG;
    if (total_dev && !aligned4(total_dev)) return RATTN_ERR_INVALID_ARG;
    if (B > 0 && (!keep || !aligned16(keep))) return RATTN_ERR_INVALID_ARG;
    PackArgs a = {};
    for (int i = 0; i < n_tensors; ++i) {
        if (!src[i] || !dst[i] || !aligned16(src[i]) || !aligned16(dst[i])) return RATTN_ERR_INVALID_ARG;
        a.src[i] = (const u32x4 *)src[i];
        a.dst[i] = (u32x4 *)dst[i];
    }
    rattn_status st = rattn_init();
    if (st != RATTN_OK) return st;
    a.keep = keep;
    a.cu = cu_seqlens;
    a.max_out = max_seqlen_dev;
    a.total_out = total_dev;
    a.B = B;
    a.N = N;
    a.row_vec = rv;
    a.n_tensors = n_tensors;
    a.ch = chunking_for(N);
    return launch_pack(a, (hipStream_t)stream) == hipSuccess ? RATTN_OK : RATTN_ERR_HIP;
}

rattn_status rattn_forward(const void *q, const void *k, const void *v, void *o,
                           const int32_t *cu_seqlens, int B, int max_seqlen, int H, int head_dim,
                           float scale, rattn_dtype dt, void *stream) {
    if (elem_size(dt) == 0) return RATTN_ERR_INVALID_ARG;
    if (B < 0 || H < 1 || max_seqlen < 0 || !std::isfinite(scale)) return RATTN_ERR_INVALID_ARG;
    if (head_dim != RATTN_HEAD_DIM) return RATTN_ERR_UNSUPPORTED;
    if ((int64_t)H * head_dim > (1 << 24)) return RATTN_ERR_INVALID_ARG;
    // row offsets inside one image are 32-bit in the kernels
    if ((int64_t)max_seqlen * H * head_dim * elem_size(dt) > RATTN_MAX_IMAGE_BYTES)
        return RATTN_ERR_UNSUPPORTED;
    if (B == 0 || max_seqlen == 0) return RATTN_OK;  // nothing to attend
    if (!q || !k || !v || !o || !cu_seqlens) return RATTN_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned4(cu_seqlens))
        return RATTN_ERR_INVALID_ARG;
    // grid = 8 * ceil(B*H/8) * ceil(max_seqlen/64) workgroups must fit a 32-bit x dimension
    if ((((int64_t)B * H + 7) / 8) * 8 * (((int64_t)max_seqlen + 63) / 64) > 0x7FFFFFFF)
        return RATTN_ERR_INVALID_ARG;
    rattn_status st = rattn_init();
    if (st != RATTN_OK) return st;
    if (validating()) {
        std::vector<int32_t> cu;
        int longest = 0;
        st = validate_cu(cu_seqlens, B, (hipStream_t)stream, cu, &longest);
        if (st != RATTN_OK) return st;
        if (longest > max_seqlen) return RATTN_ERR_INVALID_ARG;
    }
    AttnArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.cu = cu_seqlens;
    a.B = B;
    a.H = H;
    a.max_seqlen = max_seqlen;
    a.scale = scale;
    a.dt = to_elem(dt);
    return launch_attention(a, (hipStream_t)stream) == hipSuccess ? RATTN_OK : RATTN_ERR_HIP;
}

rattn_status rattn_unpack(const void *src, void *dst_padded, void *cls, const uint8_t *keep,
                          const int32_t *cu_seqlens, int B, int N, int row_elems, rattn_dtype dt,
                          void *stream) {
    if (B < 0 || N < 1 || (int64_t)B * N > RATTN_MAX_TOKENS) return RATTN_ERR_INVALID_ARG;
    const int rv = row_vectors(row_elems, dt);
    if (rv == 0) return RATTN_ERR_INVALID_ARG;
    if (!dst_padded && !cls) return RATTN_ERR_INVALID_ARG;
    if (B == 0) return RATTN_OK;
    if (!src || !keep || !cu_seqlens) return RATTN_ERR_INVALID_ARG;
    if (!aligned16(src) || !aligned16(keep) || !aligned4(cu_seqlens)) return RATTN_ERR_INVALID_ARG;
    if ((dst_padded && !aligned16(dst_padded)) || (cls && !aligned16(cls))) return RATTN_ERR_INVALID_ARG;
    rattn_status st = rattn_init();
    if (st != RATTN_OK) return st;
    if (validating()) {
        st = validate_cu_against_mask(cu_seqlens, keep, B, N, (hipStream_t)stream);
        if (st != RATTN_OK) return st;
    }
    UnpackArgs a;
    a.src = (const u32x4 *)src;
    a.dst = (u32x4 *)dst_padded;
    a.cls = (u32x4 *)cls;
    a.keep = keep;
    a.cu = cu_seqlens;
    a.B = B;
    a.N = N;
    a.row_vec = rv;
    a.ch = chunking_for(N);
    return launch_unpack(a, (hipStream_t)stream) == hipSuccess ? RATTN_OK : RATTN_ERR_HIP;
}

rattn_status rattn_repack(const void *const *src, void *const *dst, int n_tensors,
                          const uint8_t *keep2, const int32_t *cu_seqlens, int B, int row_elems,
                          rattn_dtype dt, int32_t *cu_seqlens_out, int32_t *total_dev,
                          void *stream) {
    if (n_tensors < 1 || n_tensors > RATTN_MAX_TENSORS || !src || !dst) return RATTN_ERR_INVALID_ARG;
    if (B < 0) return RATTN_ERR_INVALID_ARG;
    const int rv = row_vectors(row_elems, dt);
    if (rv == 0) return RATTN_ERR_INVALID_ARG;
    if (B == 0) return RATTN_OK;
    if (!keep2 || !aligned16(keep2) || !cu_seqlens || !aligned4(cu_seqlens) || !cu_seqlens_out ||
        !aligned4(cu_seqlens_out) || (total_dev && !aligned4(total_dev)))
        return RATTN_ERR_INVALID_ARG;
    if (cu_seqlens_out == cu_seqlens) return RATTN_ERR_INVALID_ARG;
    for (int i = 0; i < n_tensors; ++i) {
        if (!src[i] || !dst[i] || !aligned16(src[i]) || !aligned16(dst[i]) || src[i] == dst[i])
            return RATTN_ERR_INVALID_ARG;
    }
    rattn_status st = rattn_init();
    if (st != RATTN_OK) return st;
    if (validating()) {
        std::vector<int32_t> cu;
        int longest = 0;
        st = validate_cu(cu_seqlens, B, (hipStream_t)stream, cu, &longest);
        if (st != RATTN_OK) return st;
    }
    RepackArgs a;
    for (int i = 0; i < kMaxTensors; ++i) {
        a.src[i] = i < n_tensors ? (const u32x4 *)src[i] : nullptr;
        a.dst[i] = i < n_tensors ? (u32x4 *)dst[i] : nullptr;
    }
    a.keep2 = keep2;
    a.cu = cu_seqlens;
    a.cu2 = cu_seqlens_out;
    a.total_out = total_dev;
    a.B = B;
    a.row_vec = rv;
    a.n_tensors = n_tensors;
    return launch_repack(a, (hipStream_t)stream) == hipSuccess ? RATTN_OK : RATTN_ERR_HIP;
}

namespace {

rattn_status fused_common(const void *q, const void *k, const void *v, const uint8_t *keep,
                          void *out_padded, void *cls, int B, int N, int H, int head_dim,
                          int max_seqlen, int pad, float scale, rattn_dtype dt, void *stream) {
    if (elem_size(dt) == 0) return RATTN_ERR_INVALID_ARG;
    if (B < 0 || N < 1 || H < 1 || max_seqlen < 0 || !std::isfinite(scale))
        return RATTN_ERR_INVALID_ARG;
    // row strides below 2^24 elements: the kernels form padded row offsets
    // with a 24-bit multiply
    if ((int64_t)B * N > RATTN_MAX_TOKENS || (int64_t)H * RATTN_HEAD_DIM >= (1 << 24))
        return RATTN_ERR_INVALID_ARG;
    if (head_dim != RATTN_HEAD_DIM || N > RATTN_MAX_FUSED_N) return RATTN_ERR_UNSUPPORTED;
    if ((int64_t)N * H * head_dim * elem_size(dt) > RATTN_MAX_IMAGE_BYTES) return RATTN_ERR_UNSUPPORTED;
    if (!out_padded && !cls) return RATTN_ERR_INVALID_ARG;
    if (B == 0) return RATTN_OK;
    if (!q || !k || !v || !keep) return RATTN_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(keep))
        return RATTN_ERR_INVALID_ARG;
    if ((out_padded && !aligned16(out_padded)) || (cls && !aligned16(cls))) return RATTN_ERR_INVALID_ARG;
    if ((((int64_t)B * H + 7) / 8) * 8 * (((int64_t)max_seqlen + 63) / 64 + 1) > 0x7FFFFFFF)
        return RATTN_ERR_INVALID_ARG;
    rattn_status st = rattn_init();
    if (st != RATTN_OK) return st;
    if (validating()) {
        // the bound (pad_len for the padded comparator) must cover every image
        st = validate_bound(keep, B, N, max_seqlen, (hipStream_t)stream);
        if (st != RATTN_OK) return st;
    }
    FusedArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.keep = keep;
    a.out = out_padded;
    a.cls = cls;
    a.B = B;
    a.N = N;
    a.H = H;
    a.max_seqlen = max_seqlen;
    a.pad = pad;
    a.scale = scale;
    a.dt = to_elem(dt);
    return launch_fused(a, (hipStream_t)stream) == hipSuccess ? RATTN_OK : RATTN_ERR_HIP;
}

}  // namespace

rattn_status rattn_fused(const void *q, const void *k, const void *v, const uint8_t *keep,
                         void *out_padded, void *cls, int B, int N, int H, int head_dim,
                         int max_seqlen, float scale, rattn_dtype dt, void *stream) {
    return fused_common(q, k, v, keep, out_padded, cls, B, N, H, head_dim, max_seqlen, 0, scale,
                        dt, stream);
}

rattn_status rattn_fused_padded(const void *q, const void *k, const void *v, const uint8_t *keep,
                                void *out_padded, void *cls, int B, int N, int H, int head_dim,
                                int pad_len, float scale, rattn_dtype dt, void *stream) {
    if (pad_len < 1 || pad_len > N) return RATTN_ERR_INVALID_ARG;
    return fused_common(q, k, v, keep, out_padded, cls, B, N, H, head_dim, pad_len, pad_len,
                        scale, dt, stream);
}

}  // extern "C"
