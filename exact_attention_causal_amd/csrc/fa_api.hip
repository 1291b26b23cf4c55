// fa_api.hip -- the C ABI (include/fa.h): argument checks, then launches.
//
// Every check runs on the host before anything is enqueued, so an invalid call
// returns its status synchronously and touches no device state.
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>

#include "fa.h"
#include "fa_launch.hpp"

namespace fa {

namespace {
constexpr int kMaxDevices = 64;
std::atomic<int> g_cu[kMaxDevices];  // 0: not read yet
}  // namespace

int stream_cu_count(hipStream_t stream) {
    int dev = -1;
    if (stream ? hipStreamGetDevice(stream, &dev) != hipSuccess : hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    if (dev < 0 || dev >= kMaxDevices) return 0;
    int n = g_cu[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
        (void)hipGetLastError();
        return 0;
    }
    g_cu[dev].store(n, std::memory_order_relaxed);
    return n;
}

}  // namespace fa

namespace {

// Compute units a size query assumes when no device is visible: those of one
// MI355X.  (Launches always read the count of the device they run on.)
constexpr int kAssumedCU = 256;

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

// Argument checks shared by fa_fwd and fa_fwd_ws (all before the device query).
int check_fwd(const void *q, const void *k, const void *v, const void *o, const float *lse, int B, int H,
              int S, int D, float scale, int causal, int dtype) {
    if (!q || !k || !v || !o || !lse) return FA_EINVAL;
    if (causal != 0 && causal != 1) return FA_EINVAL;
    if (int rc = check_scale(scale)) return rc;
    if (int rc = check_shape(B, H, S, D, dtype)) return rc;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
        return FA_EALIGN;
    // one workgroup per 256 queries of every head must fit a launch grid (the
    // 512-query tile needs fewer; the 128-query one is chosen only for small grids)
    if ((long long)((S + 255) / 256) * B * H > 0x7fffffffLL) return FA_EINVAL;
    return FA_OK;
}

}  // namespace

extern "C" {

int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H, int S,
           int D, float scale, int causal, int dtype, hipStream_t stream) {
    if (int rc = check_fwd(q, k, v, o, lse, B, H, S, D, scale, causal, dtype)) return rc;
    const int ncu = fa::stream_cu_count(stream);
    if (ncu <= 0) return FA_EHIP;
    return map_launch(fa::launch_fwd(dtype, q, k, v, o, lse, B * H, S, D, scale, causal, ncu, stream));
}

size_t fa_fwd_workspace_size(int B, int H, int S, int D, int dtype) {
    if (check_shape(B, H, S, D, dtype) != FA_OK) return 0;
    int ncu = fa::stream_cu_count(nullptr);
    if (ncu <= 0) ncu = kAssumedCU;
    const int n = fa::fwd_split(dtype, B * H, S, D, 1, ncu, fa::kMaxSplitBytes);  // (causal: the most chunks)
    return fa::fwd_part_bytes(n, (long long)B * H, S, D);
}

int fa_fwd_ws(const void *q, const void *k, const void *v, void *o, float *lse, void *workspace,
              size_t workspace_bytes, int B, int H, int S, int D, float scale, int causal, int dtype,
              hipStream_t stream) {
    if (int rc = check_fwd(q, k, v, o, lse, B, H, S, D, scale, causal, dtype)) return rc;
    if (workspace && !aligned16(workspace)) return FA_EALIGN;
    const int ncu = fa::stream_cu_count(stream);
    if (ncu <= 0) return FA_EHIP;
    const long long BH = (long long)B * H;
    // as many key chunks as the rule asks for and the workspace holds (1: the plain forward)
    const int n = fa::fwd_split(dtype, (int)BH, S, D, causal, ncu,
                                workspace ? std::min(workspace_bytes, fa::kMaxSplitBytes) : 0);
    if (n <= 1) return map_launch(fa::launch_fwd(dtype, q, k, v, o, lse, (int)BH, S, D, scale, causal, ncu, stream));
    // chunks of whole 64-key tiles; the partials: O parts, then L parts
    const int chunk = 64 * ((S + 64 * n - 1) / (64 * n));
    const int parts = (S + chunk - 1) / chunk;
    float *o_parts = static_cast<float *>(workspace);
    float *lse_parts = reinterpret_cast<float *>(static_cast<char *>(workspace) +
                                                 fa::fwd_part_o_bytes(parts, BH, S, D));
    int rc = fa::launch_fwd_partial(dtype, q, k, v, o_parts, lse_parts, (int)BH, S, S, D, scale, causal, 0,
                                    parts, chunk, stream);
    if (rc != 0) return map_launch(rc);
    return map_launch(fa::launch_merge(dtype, o_parts, lse_parts, parts, o, lse, BH * S, D, stream));
}

int fa_bwd_preprocess(const void *o, const void *dout, float *delta, int B, int H, int S, int D,
                      int dtype, hipStream_t stream) {
    if (!o || !dout || !delta) return FA_EINVAL;
    if (int rc = check_shape(B, H, S, D, dtype)) return rc;
    if (!aligned16(o) || !aligned16(dout) || !aligned16(delta)) return FA_EALIGN;
    return map_launch(fa::launch_delta(dtype, o, dout, delta, B * H, S, D, stream));
}

size_t fa_bwd_workspace_size(int B, int H, int S, int D, int dtype) {
    if (check_shape(B, H, S, D, dtype) != FA_OK) return 0;
    const long long BH = (long long)B * H;
    // bf16 problems with few key tiles per CU: fp32 partial dQ, dK, dV of
    // each chunk of the split backward, for the current device's CU count
    int ncu = fa::stream_cu_count(nullptr);
    if (ncu <= 0) ncu = kAssumedCU;
    const fa::BwdSplit sp = fa::bwd_split(dtype, (int)BH, S, D, 1, ncu, fa::kMaxSplitBytes);  // (causal: the most chunks)
    return fa::bwd_lse2_bytes(BH * S) + fa::bwd_part_bytes(sp, BH, S, D);
}

// Checks shared by fa_bwd and fa_bwd_noalloc.
static int check_bwd(const void *q, const void *k, const void *v, const void *dout, const float *lse,
                     const float *delta, void *dq, void *dk, void *dv, int B, int H, int S, int D, float scale,
                     int causal, int dtype) {
    if (!q || !k || !v || !dout || !lse || !delta || !dq || !dk || !dv) return FA_EINVAL;
    if (causal != 0 && causal != 1) return FA_EINVAL;
    if (int rc = check_scale(scale)) return rc;
    if (int rc = check_shape(B, H, S, D, dtype)) return rc;
    const void *ptrs[] = {q, k, v, dout, lse, delta, dq, dk, dv};
    for (const void *p : ptrs)
        if (!aligned16(p)) return FA_EALIGN;
    // one workgroup per 128 keys of every head (the smallest key tile) must fit a launch grid
    if ((long long)((S + 127) / 128) * B * H > 0x7fffffffLL) return FA_EINVAL;
    return FA_OK;
}

int fa_bwd(const void *q, const void *k, const void *v, const void *dout, const float *lse,
           const float *delta, void *dq, void *dk, void *dv, void *workspace, size_t workspace_bytes,
           int B, int H, int S, int D, float scale, int causal, int dtype, hipStream_t stream) {
    if (int rc = check_bwd(q, k, v, dout, lse, delta, dq, dk, dv, B, H, S, D, scale, causal, dtype)) return rc;
    if (!workspace) return FA_EINVAL;
    if (!aligned16(workspace)) return FA_EALIGN;
    const long long BH = (long long)B * H;
    const size_t base = fa::bwd_lse2_bytes(BH * S);
    if (workspace_bytes < base) return FA_EWORKSPACE;
    const int ncu = fa::stream_cu_count(stream);
    if (ncu <= 0) return FA_EHIP;
    // the split backward takes as many chunks as the workspace holds partials for
    const size_t budget = workspace_bytes - base < fa::kMaxSplitBytes ? workspace_bytes - base : fa::kMaxSplitBytes;
    const fa::BwdSplit sp = fa::bwd_split(dtype, (int)BH, S, D, causal, ncu, budget);
    return map_launch(fa::launch_bwd(dtype, q, k, v, dout, lse, delta, dq, dk, dv,
                                     static_cast<float *>(workspace), (int)BH, S, D, scale, causal, sp, stream));
}

int fa_bwd_noalloc(const void *q, const void *k, const void *v, const void *dout, const float *lse,
                   const float *delta, void *dq, void *dk, void *dv, int B, int H, int S, int D, float scale,
                   int causal, int dtype, hipStream_t stream) {
    if (int rc = check_bwd(q, k, v, dout, lse, delta, dq, dk, dv, B, H, S, D, scale, causal, dtype)) return rc;
    const long long BH = (long long)B * H;
    const size_t base = fa::bwd_lse2_bytes(BH * S);
    if (base > fa::kNoAllocScratchBytes) return FA_ESCRATCH;
    const int ncu = fa::stream_cu_count(stream);
    if (ncu <= 0) return FA_EHIP;
    float *scratch = fa::noalloc_scratch(stream);
    if (!scratch) return FA_EHIP;
    const fa::BwdSplit sp = fa::bwd_split(dtype, (int)BH, S, D, causal, ncu, fa::kNoAllocScratchBytes - base);
    return map_launch(fa::launch_bwd(dtype, q, k, v, dout, lse, delta, dq, dk, dv, scratch, (int)BH, S, D,
                                     scale, causal, sp, stream));
}

int fa_get_plan(int B, int H, int S, int D, int dtype, int num_cu, fa_plan *plan) {
    if (!plan) return FA_EINVAL;
    if (int rc = check_shape(B, H, S, D, dtype)) return rc;
    if (num_cu <= 0) {
        num_cu = fa::stream_cu_count(nullptr);
        if (num_cu <= 0) return FA_EHIP;
    }
    const int BH = B * H;
    const fa::FwdPlan f = fa::fwd_plan(dtype, BH, S, D, num_cu);
    const fa::BwdSplit sp = fa::bwd_split(dtype, BH, S, D, 1, num_cu, fa::kMaxSplitBytes);
    plan->num_cu = num_cu;
    plan->fwd_block_queries = f.bq;
    plan->fwd_key_groups = f.groups;
    plan->fwd_key_tile = f.bk;
    plan->fwd_band = f.band;
    plan->bwd_chunks = sp.n;
    plan->bwd_chunk_rows = sp.chunk;
    return FA_OK;
}

int fa_fwd_partial(const void *q, const void *k, const void *v, float *o_parts, float *lse_parts,
                   int B, int H, int Sq, int Sk, int D, float scale, int causal, int q_offset,
                   int n_split, int dtype, hipStream_t stream) {
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
             int H, int S, int D, int dtype, hipStream_t stream) {
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
                   int H, int Sq, int Sk, int D, float scale, int causal, int q_offset, int dtype,
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
    case FA_EHIP: return "HIP runtime error (no device visible, device query or kernel launch failed)";
    case FA_ESCRATCH: return "problem too large for the fixed device scratch of fa_bwd_noalloc (B*H*S above 16777216)";
    default: return "unknown status";
    }
}

}  // extern "C"
