// fa_merge.hip -- merge of attention results over disjoint key sets.
//
// The ring-attention page ("[Attention]FlashAttention/Ring-Attention/
// 混合序列并行的统一原理", section "online attention") splits the keys of one
// attention into parts and combines the parts' normalised outputs by their
// shares of the common softmax denominator.  Each part carries its output
// O_r and logsumexp L_r (its denominator times e^{its max} is e^{L_r}), so
// with M = max_r L_r and w_r = 2^{(L_r - M) log2 e}:
//   O = sum_r w_r O_r / sum_r w_r,   L = M + ln sum_r w_r,
// and a row that is empty in every part (all L_r = -inf) stays O = 0,
// L = -inf.  Parts are added in index order (reproducible).
//
// Bound by HBM: a row moves n*D*4 bytes in and D*sizeof(T) + 4 out.  A
// group of D/4 lanes owns one row (16-byte loads of O_r), so a 256-thread
// workgroup covers 1024/D rows.
#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {

template <typename T, int D>
__global__ __launch_bounds__(256) void merge_kernel(const float *__restrict__ o_parts,
                                                    const float *__restrict__ lse_parts, int n,
                                                    T *__restrict__ o, float *__restrict__ lse,
                                                    long long rows) {
    constexpr int LPR = D / 4;              // lanes per row
    constexpr int RPB = 256 / LPR;          // rows per workgroup
    const int t = threadIdx.x;
    if (t >= RPB * LPR) return;             // (D = 80, 96: the last lanes have no row)
    const long long row = (long long)blockIdx.x * RPB + t / LPR;
    const int c4 = (t % LPR) * 4;           // first of this lane's 4 columns
    if (row >= rows) return;
    float M = -INFINITY;
    for (int r = 0; r < n; ++r) M = fmaxf(M, lse_parts[(long long)r * rows + row]);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float wsum = 0.f;
    if (M != -INFINITY) {
        auto part = [&](int r) {
            const float lr = lse_parts[(long long)r * rows + row];
            const float w = fast_exp2((lr - M) * kLog2e);  // 0 for an empty part
            wsum += w;
            const f32x4 x = *reinterpret_cast<const f32x4 *>(o_parts + ((long long)r * rows + row) * D + c4);
            acc += w * x;
        };
        // four parts per round keep four 16-byte loads in flight per lane
        int r = 0;
        for (; r + 4 <= n; r += 4) {
#pragma unroll
            for (int u = 0; u < 4; ++u) part(r + u);
        }
        for (; r < n; ++r) part(r);
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    if constexpr (sizeof(T) == 2) {
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        bf16x4 y;
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = (__bf16)(acc[e] * inv);
        *reinterpret_cast<bf16x4 *>(o + row * D + c4) = y;
    } else {
        *reinterpret_cast<f32x4 *>(o + row * D + c4) = acc * inv;
    }
    if (c4 == 0) lse[row] = wsum > 0.f ? M + log2f(wsum) * kLn2 : -INFINITY;
}

template <typename T, int D>
static int run_merge(const float *op, const float *lp, int n, void *o, float *lse, long long rows,
                     hipStream_t stream) {
    constexpr int RPB = 256 / (D / 4);
    const long long grid = (rows + RPB - 1) / RPB;
    if (grid > 0x7fffffffLL) return -1;
    hipLaunchKernelGGL((merge_kernel<T, D>), dim3((unsigned)grid), dim3(256), 0, stream, op, lp, n, (T *)o,
                       lse, rows);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

template <typename T>
static int merge_dispatch(int D, const float *op, const float *lp, int n, void *o, float *lse, long long rows,
                          hipStream_t stream) {
    switch (D) {
    case 16: return run_merge<T, 16>(op, lp, n, o, lse, rows, stream);
    case 32: return run_merge<T, 32>(op, lp, n, o, lse, rows, stream);
    case 64: return run_merge<T, 64>(op, lp, n, o, lse, rows, stream);
    case 80: return run_merge<T, 80>(op, lp, n, o, lse, rows, stream);
    case 96: return run_merge<T, 96>(op, lp, n, o, lse, rows, stream);
    case 128: return run_merge<T, 128>(op, lp, n, o, lse, rows, stream);
    default: return -2;
    }
}

int launch_merge(int dtype, const float *o_parts, const float *lse_parts, int n, void *o, float *lse,
                 long long rows, int D, hipStream_t stream) {
    if (dtype == 1) return merge_dispatch<bf16>(D, o_parts, lse_parts, n, o, lse, rows, stream);
    if (dtype == 0) return merge_dispatch<float>(D, o_parts, lse_parts, n, o, lse, rows, stream);
    return -2;
}

}  // namespace fa
