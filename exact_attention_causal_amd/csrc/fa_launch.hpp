// fa_launch.hpp -- internal interface between the C ABI (argument checks)
// and the kernel translation units (tile selection and launches).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa {

// Head dimensions with built kernels.
constexpr int kHeadDims[] = {16, 32, 64, 80, 96, 128};

inline bool head_dim_supported(int D) {
    for (int d : kHeadDims)
        if (d == D) return true;
    return false;
}

// Compute units of the device a launch on `stream` runs on (the null stream:
// the current device), read from the runtime once per device and cached; 0
// if no device is visible.  Every launch-shape threshold below takes it as an
// argument.
int stream_cu_count(hipStream_t stream);

// XCDs of the GPU: workgroup i of a launch runs on XCD i % kNumXcd (the
// dispatcher deals workgroups to the XCDs in turn; each has its own L2).
constexpr int kNumXcd = 8;

// Forward tile configuration of a self-attention problem: queries per
// workgroup, key groups per workgroup (2: two wave groups split the key tiles
// and merge), keys per LDS tile, and the workgroup order (band: see
// tile_order; 0 = consecutive workgroups take consecutive heads).
struct FwdPlan {
    int bq, groups, bk, band;
};
FwdPlan fwd_plan(int dtype, int BH, int S, int D, int ncu);

// Key chunks for a self-attention forward that has a workspace (fa_fwd_ws):
// 1 runs the plain forward; n > 1 runs n key chunks side by side (fp32
// partial O and L, fwd_part_bytes of them) and merges them.  At most as many
// chunks as max_part_bytes holds.
int fwd_split(int dtype, int BH, int S, int D, int causal, int ncu, size_t max_part_bytes);
// Bytes of the partials of n chunks: O parts, then L parts, each rounded up to 256 bytes.
inline size_t fwd_part_o_bytes(int n, long long BH, int S, int D) {
    return ((size_t)n * BH * S * D * sizeof(float) + 255) & ~(size_t)255;
}
inline size_t fwd_part_bytes(int n, long long BH, int S, int D) {
    if (n <= 1) return 0;
    return fwd_part_o_bytes(n, BH, S, D) + (((size_t)n * BH * S * sizeof(float) + 255) & ~(size_t)255);
}

// Each returns 0 on success, -2 (unsupported D/dtype) or -5 (launch refused).
// Sizes are already validated; BH = B*H; ncu as stream_cu_count.
int launch_fwd(int dtype, const void *q, const void *k, const void *v, void *o, float *lse,
               int BH, int S, int D, float scale, int causal, int ncu, hipStream_t stream);

// Shifted / split-key forward with fp32 partial outputs; `chunk` keys per split.
int launch_fwd_partial(int dtype, const void *q, const void *k, const void *v, float *o_parts,
                       float *lse_parts, int BH, int Sq, int Sk, int D, float scale, int causal,
                       int q_offset, int n_split, int chunk, hipStream_t stream);

// Merge of n partial results (rows = B*H*S).
int launch_merge(int dtype, const float *o_parts, const float *lse_parts, int n, void *o, float *lse,
                 long long rows, int D, hipStream_t stream);

int launch_delta(int dtype, const void *o, const void *dout, float *delta, int BH, int S, int D,
                 hipStream_t stream);

// How the backward of a problem with few key tiles per CU is split: n
// chunks of `chunk` rows per pass (n = 1: not split), with at most
// `max_part_bytes` of fp32 partial results.  A causal problem never takes
// fewer chunks than the same problem without the mask, so size queries,
// which do not know the mask, ask with causal = 1.
struct BwdSplit {
    int n, chunk;
};
constexpr size_t kMaxSplitBytes = (size_t)256 << 20;  // partials of the caller-workspace backward
BwdSplit bwd_split(int dtype, int BH, int S, int D, int causal, int ncu, size_t max_part_bytes);

// Bytes of the base-2 copy of lse at the start of the backward workspace (one
// fp32 per row, rounded up to 256 bytes); the split's partials follow it.
inline size_t bwd_lse2_bytes(long long rows) { return ((size_t)rows * sizeof(float) + 255) & ~(size_t)255; }
// Bytes of the partials of a split into sp.n chunks.
inline size_t bwd_part_bytes(const BwdSplit &sp, long long BH, int S, int D) {
    return sp.n <= 1 ? 0 : 3 * (size_t)sp.n * BH * S * D * sizeof(float);
}

// lse2: workspace of bwd_lse2_bytes(BH*S), followed -- when sp.n > 1 -- by
// bwd_part_bytes(sp, ...) of partial results.  sp comes from bwd_split.
int launch_bwd(int dtype, const void *q, const void *k, const void *v, const void *dout,
               const float *lse, const float *delta, void *dq, void *dk, void *dv, float *lse2,
               int BH, int S, int D, float scale, int causal, BwdSplit sp, hipStream_t stream);

// The allocation-free backward's device scratch (a fixed array in device
// memory, one per GPU): its address on the device `stream` runs on, looked up
// once per device; nullptr if the lookup failed.  kNoAllocScratchBytes is its size.
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
float *noalloc_scratch(hipStream_t stream);

// Gradient contributions of one key set (fp32, stored or added).
int launch_bwd_partial(int dtype, const void *q, const void *k, const void *v, const void *dout,
                       const float *lse, const float *delta, float *dq, float *dk, float *dv,
                       int accumulate, int BH, int Sq, int Sk, int D, float scale, int causal,
                       int q_offset, hipStream_t stream);

}  // namespace fa
