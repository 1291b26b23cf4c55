// fa_api.hip -- the C ABI (include/fa.h): argument checks, then launches.
//
// Every check runs on the host before anything is enqueued, so an invalid call
// returns its status synchronously and touches no device state.
#include <math.h>
#include <stdint.h>

#include "fa.h"
#include "fa_launch.hpp"

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shape checks shared by every entry point.
int check_shape(int B, int H, int S, int D, int dtype) {
    if (B <= 0 || H <= 0 || S <= 0 || D <= 0) return FA_EINVAL;
    if (S > (1 << 30)) return FA_EINVAL;  // tile positions (a few tiles past S) stay within int
    const long long bh = (long long)B * H;
    if (bh > 0x7fffffffLL) return FA_EINVAL;
    // elements per tensor must fit comfortably in 63 bits
    const long long per_head = (long long)S * D;
    if (bh > (0x3fffffffffffffffLL / per_head)) return FA_EINVAL;
    if (dtype != FA_F32 && dtype != FA_BF16) return FA_EUNSUPPORTED;
    if (!fa::head_dim_supported(D)) return FA_EUNSUPPORTED;
    return FA_OK;
}

int check_scale(float scale) {
    if (!isfinite(scale) || !(scale > 0.f)) return FA_EINVAL;
    return FA_OK;
}

int map_launch(int rc) {
    if (rc == 0) return FA_OK;
    if (rc == -2) return FA_EUNSUPPORTED;
    if (rc == -1) return FA_EINVAL;
    return FA_EHIP;
}

}  // namespace

extern "C" {

int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H, int S,
           int D, float scale, int causal, fa_dtype dtype, hipStream_t stream) {
    if (!q || !k || !v || !o || !lse) return FA_EINVAL;
    if (causal != 0 && causal != 1) return FA_EINVAL;
    if (int rc = check_scale(scale)) return rc;
    if (int rc = check_shape(B, H, S, D, dtype)) return rc;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
        return FA_EALIGN;
    return map_launch(fa::launch_fwd(dtype, q, k, v, o, lse, B * H, S, D, scale, causal, stream));
}

int fa_bwd_preprocess(const void *o, const void *dout, float *delta, int B, int H, int S, int D,
                      fa_dtype dtype, hipStream_t stream) {
    if (!o || !dout || !delta) return FA_EINVAL;
    if (int rc = check_shape(B, H, S, D, dtype)) return rc;
    if (!aligned16(o) || !aligned16(dout) || !aligned16(delta)) return FA_EALIGN;
    return map_launch(fa::launch_delta(dtype, o, dout, delta, B * H, S, D, stream));
}

// The part of the backward workspace every call needs: the base-2 copy of
// lse, one fp32 per row, rounded up to 256 bytes.
static size_t bwd_base_workspace(int B, int H, int S) {
    return ((size_t)B * H * S * sizeof(float) + 255) & ~(size_t)255;
}

size_t fa_bwd_workspace_size(int B, int H, int S, int D, fa_dtype dtype) {
    if (check_shape(B, H, S, D, dtype) != FA_OK) return 0;
    const size_t bytes = bwd_base_workspace(B, H, S);
    // bf16 problems with few key tiles per CU: fp32 partial dQ, dK, dV of
    // each chunk of the split backward
    const fa::BwdSplit sp = fa::bwd_split(dtype, B * H, S, D);
    if (sp.n <= 1) return bytes;
    return bytes + 3 * (size_t)sp.n * B * H * S * D * sizeof(float);
}

int fa_bwd(const void *q, const void *k, const void *v, const void *dout, const float *lse,
           const float *delta, void *dq, void *dk, void *dv, void *workspace, size_t workspace_bytes,
           int B, int H, int S, int D, float scale, int causal, fa_dtype dtype, hipStream_t stream) {
    if (!q || !k || !v || !dout || !lse || !delta || !dq || !dk || !dv) return FA_EINVAL;
    if (causal != 0 && causal != 1) return FA_EINVAL;
    if (int rc = check_scale(scale)) return rc;
    if (int rc = check_shape(B, H, S, D, dtype)) return rc;
    if (!workspace) return FA_EINVAL;
    const void *ptrs[] = {q, k, v, dout, lse, delta, dq, dk, dv, workspace};
    for (const void *p : ptrs)
        if (!aligned16(p)) return FA_EALIGN;
    if (workspace_bytes < bwd_base_workspace(B, H, S)) return FA_EWORKSPACE;
    // the split backward runs only when the workspace holds its partials
    const bool split = workspace_bytes >= fa_bwd_workspace_size(B, H, S, D, dtype);
    return map_launch(fa::launch_bwd(dtype, q, k, v, dout, lse, delta, dq, dk, dv,
                                     static_cast<float *>(workspace), B * H, S, D, scale, causal, split,
                                     stream));
}

int fa_fwd_partial(const void *q, const void *k, const void *v, float *o_parts, float *lse_parts,
                   int B, int H, int Sq, int Sk, int D, float scale, int causal, int q_offset,
                   int n_split, fa_dtype dtype, hipStream_t stream) {
    if (!q || !k || !v || !o_parts || !lse_parts) return FA_EINVAL;
    if (causal != 0 && causal != 1) return FA_EINVAL;
    if (n_split < 1 || n_split > 65535) return FA_EINVAL;
    if (int rc = check_scale(scale)) return rc;
    if (int rc = check_shape(B, H, Sq, D, dtype)) return rc;
    if (int rc = check_shape(B, H, Sk, D, dtype)) return rc;
    // positions and their sums with the offset (at most Sq + Sk + a tile) stay within int
    if (Sq > (1 << 29) || Sk > (1 << 29)) return FA_EINVAL;
    // n_split copies of the output must still be addressable
    const long long per_split = (long long)B * H * Sq * D;
    if (per_split > 0x3fffffffffffffffLL / n_split) return FA_EINVAL;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o_parts) || !aligned16(lse_parts))
        return FA_EALIGN;
    const long long per = ((long long)Sk + 64LL * n_split - 1) / (64LL * n_split);
    const long long chunk = 64 * per;
    if (chunk * n_split > 0x7fffffffLL) return FA_EINVAL;
    // offsets beyond [-Sq, Sk] change nothing (every key allowed / none)
    const int off = (int)(q_offset < -Sq ? -Sq : (q_offset > Sk ? Sk : q_offset));
    return map_launch(fa::launch_fwd_partial(dtype, q, k, v, o_parts, lse_parts, B * H, Sq, Sk, D, scale,
                                             causal, off, n_split, (int)chunk, stream));
}

int fa_merge(const float *o_parts, const float *lse_parts, int n_parts, void *o, float *lse, int B,
             int H, int S, int D, fa_dtype dtype, hipStream_t stream) {
    if (!o_parts || !lse_parts || !o || !lse) return FA_EINVAL;
    if (n_parts < 1) return FA_EINVAL;
    if (int rc = check_shape(B, H, S, D, dtype)) return rc;
    const long long per_part = (long long)B * H * S * D;
    if (per_part > 0x3fffffffffffffffLL / n_parts) return FA_EINVAL;
    if (!aligned16(o_parts) || !aligned16(lse_parts) || !aligned16(o) || !aligned16(lse)) return FA_EALIGN;
    return map_launch(fa::launch_merge(dtype, o_parts, lse_parts, n_parts, o, lse, (long long)B * H * S, D,
                                       stream));
}

int fa_bwd_partial(const void *q, const void *k, const void *v, const void *dout, const float *lse,
                   const float *delta, float *dq_acc, float *dk_acc, float *dv_acc, int accumulate, int B,
                   int H, int Sq, int Sk, int D, float scale, int causal, int q_offset, fa_dtype dtype,
                   hipStream_t stream) {
    if (!q || !k || !v || !dout || !lse || !delta || !dq_acc || !dk_acc || !dv_acc) return FA_EINVAL;
    if (causal != 0 && causal != 1) return FA_EINVAL;
    if (accumulate != 0 && accumulate != 1) return FA_EINVAL;
    if (int rc = check_scale(scale)) return rc;
    if (int rc = check_shape(B, H, Sq, D, dtype)) return rc;
    if (int rc = check_shape(B, H, Sk, D, dtype)) return rc;
    // positions and their sums with the offset (at most Sq + Sk + a tile) stay within int
    if (Sq > (1 << 29) || Sk > (1 << 29)) return FA_EINVAL;
    const void *ptrs[] = {q, k, v, dout, lse, delta, dq_acc, dk_acc, dv_acc};
    for (const void *p : ptrs)
        if (!aligned16(p)) return FA_EALIGN;
    // offsets beyond [-Sq, Sk] change nothing (every key allowed / none)
    const int off = (int)(q_offset < -Sq ? -Sq : (q_offset > Sk ? Sk : q_offset));
    return map_launch(fa::launch_bwd_partial(dtype, q, k, v, dout, lse, delta, dq_acc, dk_acc, dv_acc,
                                             accumulate, B * H, Sq, Sk, D, scale, causal, off, stream));
}

const char *fa_strerror(int status) {
    switch (status) {
    case FA_OK: return "success";
    case FA_EINVAL: return "invalid argument (null pointer, non-positive size, causal not 0/1, bad scale or size overflow)";
    case FA_EUNSUPPORTED: return "unsupported head dimension or dtype";
    case FA_EALIGN: return "pointer not 16-byte aligned";
    case FA_EWORKSPACE: return "workspace too small";
    case FA_EHIP: return "HIP kernel launch failed";
    default: return "unknown status";
    }
}

}  // extern "C"
