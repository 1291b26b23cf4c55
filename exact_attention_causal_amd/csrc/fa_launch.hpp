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

// Each returns 0 on success, -2 (unsupported D/dtype) or -5 (launch refused).
// Sizes are already validated; BH = B*H.
int launch_fwd(int dtype, const void *q, const void *k, const void *v, void *o, float *lse,
               int BH, int S, int D, float scale, int causal, hipStream_t stream);

// Shifted / split-key forward with fp32 partial outputs; `chunk` keys per split.
int launch_fwd_partial(int dtype, const void *q, const void *k, const void *v, float *o_parts,
                       float *lse_parts, int BH, int Sq, int Sk, int D, float scale, int causal,
                       int q_offset, int n_split, int chunk, hipStream_t stream);

// Merge of n partial results (rows = B*H*S).
int launch_merge(int dtype, const float *o_parts, const float *lse_parts, int n, void *o, float *lse,
                 long long rows, int D, hipStream_t stream);

int launch_delta(int dtype, const void *o, const void *dout, float *delta, int BH, int S, int D,
                 hipStream_t stream);

// How the bf16 backward of a problem with few key tiles per CU is split: n
// chunks of `chunk` rows per pass (n = 1: not split).
struct BwdSplit {
    int n, chunk;
};
BwdSplit bwd_split(int dtype, int BH, int S, int D);

// lse2: workspace of at least BH*S floats (the base-2 copy of lse), rounded
// up to 64 floats, followed -- when bwd_split gives n > 1 -- by 3*n*BH*S*D
// floats of partial results (used only with allow_split).
int launch_bwd(int dtype, const void *q, const void *k, const void *v, const void *dout,
               const float *lse, const float *delta, void *dq, void *dk, void *dv, float *lse2,
               int BH, int S, int D, float scale, int causal, bool allow_split, hipStream_t stream);

// Gradient contributions of one key set (fp32, stored or added).
int launch_bwd_partial(int dtype, const void *q, const void *k, const void *v, const void *dout,
                       const float *lse, const float *delta, float *dq, float *dk, float *dv,
                       int accumulate, int BH, int Sq, int Sk, int D, float scale, int causal,
                       int q_offset, hipStream_t stream);

}  // namespace fa
