// fa_fwd.hip -- causal FlashAttention-2 forward pass for gfx950.
//
// Follows the CS336 Assignment 2 handout, section 4.2.2 (Algorithm 1): one
// workgroup owns a tile of BQ queries of one head, keeps Q in registers and
// streams key/value tiles of BK rows through LDS; the running row maximum m,
// the running denominator l and the output accumulator are updated online
// (the handout's m^(j), l^(j), O^(j) recurrences), and the epilogue writes
// O = O^(Tk) / l and L = m + log l.  Key tiles that lie wholly above the
// diagonal are not visited; only tiles that cross the diagonal or the end of
// the sequence are masked (the handout's "Improve FlashAttention" ideas in
// its leaderboard problem; lecture notes "A2 系统", section on online softmax:
// skip fully masked blocks).
//
// gfx950 specifics:
//   * scores are formed transposed, S^T = K Q^T, so every lane owns one query
//     column: the row max / row sum are in-lane reductions plus one exchange
//     with the partner lane 32 away, and the output O^T = V^T P^T uses the
//     score registers directly as its B operand (no shuffles, no LDS trip);
//   * exponentials are exp2 with scale*log2(e) folded into one FMA, and the
//     stored L is converted back to the natural-log convention (lecture notes
//     "A2 系统" at courses-9tz.pages.dev/llm/systems, section "从公式到 Triton 程序");
//   * K and V tiles sit row-major in LDS with a padded pitch; V^T operand
//     fragments come straight from the row-major tile through the gfx950
//     transposing LDS read, so nothing is transposed on the way in;
//   * the accumulator is rescaled only when a new score exceeds the running
//     maximum by 2^8 (exactness is kept because O and l share the stale max);
//   * K/V tiles are loaded straight into LDS (global_load_lds_dwordx4) into
//     three stages, so the next two tiles stream in while the current one is
//     used and no registers or VALU work are spent staging them;
//   * workgroups are dispatched longest-first (highest query tile first) so
//     the short causal tiles fill in the tail.
#include "fa_common.hpp"
#include "fa_launch.hpp"

namespace fa {

template <typename T, int D_, int NQB_, int BK_, int NW_>
struct FwdTile {
    static constexpr int D = D_, NQB = NQB_, BK = BK_;
    static constexpr int NW = NW_, NT = NW * kWave;
    static constexpr int BQ = NW * NQB * 32;          // queries per workgroup
    static constexpr int KPL = Mma<T>::KPL;
    static constexpr int NSD = D / 2 / KPL;           // MFMAs over d per 32x32 block
    static constexpr int NKB = BK / 32;               // 32-key blocks per tile
    static constexpr int ND = (D + 31) / 32;          // 32-row output blocks over d
    static constexpr int NI = 16 / KPL;               // MFMAs per 32-key reduction block
    using DMA = TileDma<T, D, BK, NW / 2>;           // half the waves load K, half V
    static constexpr int TILE = DMA::ELEMS;           // elements per K or V tile
    static_assert(D % 16 == 0 && BK % 32 == 0 && NW % 2 == 0, "tile shape");
};

// Scores more than 2^kRescaleSlack above the running maximum force a rescale;
// below that, p = exp2(s - m) stays <= 2^kRescaleSlack, which fp32 and bf16
// hold exactly as well as values <= 1, and O and l keep the same stale m.
constexpr float kRescaleSlack = 8.f;

template <typename T, typename C>
__global__ __launch_bounds__(C::NT) void fwd_kernel(const T *__restrict__ q, const T *__restrict__ k,
                                                    const T *__restrict__ v, T *__restrict__ o,
                                                    float *__restrict__ lse, int BH, int S, float c,
                                                    int causal, int nqt) {
    using M = Mma<T>;
    using frag = typename M::frag;
    constexpr int D = C::D, NQB = C::NQB, BK = C::BK;
    // Three stages of K and V tiles: two tiles stream in while one is used.
    // Each stage is its own array and the loop is unrolled by three, so the
    // compiler can see that reads of one stage never alias the DMA into the
    // others and does not wait for the tiles in flight.
    __shared__ __attribute__((aligned(1024))) T sK0[C::TILE], sK1[C::TILE], sK2[C::TILE];
    __shared__ __attribute__((aligned(1024))) T sV0[C::TILE], sV1[C::TILE], sV2[C::TILE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, l32 = lane & 31;
    const int bid = blockIdx.x;
    const int qt = causal ? (nqt - 1 - bid / BH) : (bid / BH);
    const int bh = bid % BH;
    const size_t hoff = (size_t)bh * S * D;
    q += hoff;
    k += hoff;
    v += hoff;
    o += hoff;
    lse += (size_t)bh * S;
    const int q0 = qt * C::BQ;
    const int qw0 = q0 + wave * NQB * 32;

    // Q^T fragments (B operand): lane owns query qw0 + 32*qb + l32, d-run of half h.
    frag qf[NQB][C::NSD];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        const int qi = qw0 + qb * 32 + l32;
        if (qi < S)
            load_run<T, C::NSD>(qf[qb], q + (size_t)qi * D + h * (D / 2));
        else
            zero_run<T, C::NSD>(qf[qb]);
    }
    TransReader<T, D> vt;
    vt.init(lane);

    f32x16 acc[NQB][C::ND];
    float mrow[NQB], lrow[NQB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        mrow[qb] = -INFINITY;
        lrow[qb] = 0.f;
#pragma unroll
        for (int db = 0; db < C::ND; ++db) acc[qb][db] = f32x16{};
    }

    const int qend = min(q0 + C::BQ, S);
    int nkt = (S + BK - 1) / BK;
    if (causal) nkt = min(nkt, (qend - 1) / BK + 1);

    typename C::DMA dma;
    const int half = wave / (C::NW / 2), hw = wave % (C::NW / 2);
    dma.init(lane, hw);
    // this wave's share of key/value tile j: K (first half of the waves) or V
    auto issue = [&](T *nK, T *nV, int j) { dma.issue(half ? nV : nK, half ? v : k, j * BK, S, hw); };
    issue(sK0, sV0, 0);
    issue(sK1, sV1, 1);

    auto step = [&](const T *tK, const T *tV, T *nK, T *nV, int j) {
        const int j0 = j * BK;
        wait_vmcnt<C::DMA::IPW>();  // this wave's part of tile j has landed (j+1 may be in flight)
        lds_barrier();              // every part of tile j landed; stage of tile j-1 released
        // Prefetch tile j+2 into the stage tile j-1 used, one instruction at
        // a time spread over this step's work.  It is issued unconditionally
        // -- past the last tile its range is empty and it fetches nothing --
        // because a conditional issue makes the compiler wait for every DMA
        // before the next LDS read.
        // (parts: one before each S^T block and each O^T block)
        constexpr int NP = 2 * C::NKB;
        const auto rs = C::DMA::range(half ? v : k, (j + 2) * BK, S);
        T *const nT = half ? nV : nK;
        const bool active = qw0 < S && !(causal && j0 > qw0 + NQB * 32 - 1);
        if (!active) {
            dma.issue(nT, half ? v : k, (j + 2) * BK, S, hw);
        } else {
            // S^T block (kb, qb): rows = keys j0 + 32*kb + ridx(r, h), col = query.
            f32x16 s[NQB][C::NKB];
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb) {
                dma.template issue_part<NP>(kb, nT, rs, hw);
                // K fragments are read in groups of KG (each feeds NQB
                // products; an odd count ends with a single one): with two
                // query blocks per wave the registers would not hold them all
                constexpr int KG = NQB > 1 ? 2 : C::NSD;
                const T *krow = tK + (kb * 32 + rsigma(l32)) * C::DMA::PD::PITCH + h * (D / 2);
                auto group = [&](auto n, int f0) {
                    constexpr int N = decltype(n)::value;
                    frag kf[N];
                    load_run<T, N>(kf, krow + f0 * C::KPL);
#pragma unroll
                    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
                        for (int st = 0; st < N; ++st) s[qb][kb] = M::run(kf[st], qf[qb][f0 + st], s[qb][kb]);
                };
#pragma unroll
                for (int qb = 0; qb < NQB; ++qb) s[qb][kb] = f32x16{};
#pragma unroll
                for (int g = 0; g < C::NSD / KG; ++g) group(std::integral_constant<int, KG>{}, g * KG);
                if constexpr (C::NSD % KG != 0)
                    group(std::integral_constant<int, C::NSD % KG>{}, C::NSD / KG * KG);
            }
            const bool need_mask = (causal && j0 + BK - 1 > qw0) || (j0 + BK > S);
            if (need_mask) {
                // (the empty volatile asm keeps this block a real branch: only
                // tiles crossing the diagonal or the sequence end pay for masking)
                asm volatile("");
                // key j0 + 32*kb + ridx(r, h) is kept iff it is below `lim`
#pragma unroll
                for (int qb = 0; qb < NQB; ++qb) {
                    const int qi = qw0 + qb * 32 + l32;
                    const int lim = causal ? min(qi + 1, S) : S;
                    const int t = lim - j0 - 2 * h;
#pragma unroll
                    for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            s[qb][kb][r] = (32 * kb + ridx(r, 0) < t) ? s[qb][kb][r] : -INFINITY;
                }
            }
            // Online softmax in base 2 (scores scaled by c = scale*log2 e).  The
            // running maximum only moves when a score exceeds it by kRescaleSlack.
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb) {
                float mx = -INFINITY;
#pragma unroll
                for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[qb][kb][r]);
                mx = wave_xor32_max(mx) * c;
                const bool grow = mx > mrow[qb] + kRescaleSlack;
                if (__ballot(grow) != 0) {  // wave-uniform: rare after the first tile
                    const float mnew = grow ? mx : mrow[qb];
                    const float alpha = fast_exp2(mrow[qb] - mnew);
                    lrow[qb] *= alpha;
#pragma unroll
                    for (int db = 0; db < C::ND; ++db) acc[qb][db] *= alpha;
                    mrow[qb] = mnew;
                }
                // a row whose maximum is still -inf has seen only masked keys: use 0
                const float muse = (mrow[qb] == -INFINITY) ? 0.f : mrow[qb];
                float ps = 0.f;
#pragma unroll
                for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float p = fast_exp2(fmaf(s[qb][kb][r], c, -muse));
                        s[qb][kb][r] = p;
                        ps += p;
                    }
                lrow[qb] += ps;
            }
            // O^T += V^T P^T
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb) {
                dma.template issue_part<NP>(C::NKB + kb, nT, rs, hw);
                frag pf[NQB][C::NI];
#pragma unroll
                for (int qb = 0; qb < NQB; ++qb) to_bfrag<T>(pf[qb], s[qb][kb]);
#pragma unroll
                for (int db = 0; db < C::ND; ++db) {
                    frag vf[C::NI];
                    vt.load(vf, tV, kb, db);
#pragma unroll
                    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
                        for (int i = 0; i < C::NI; ++i) acc[qb][db] = M::run(vf[i], pf[qb][i], acc[qb][db]);
                }
            }
        }
        wait_lgkm0();  // this wave's reads of the stage are complete before the next barrier
    };
    for (int j = 0; j < nkt; j += 3) {
        step(sK0, sV0, sK2, sV2, j);
        if (j + 1 < nkt) step(sK1, sV1, sK0, sV0, j + 1);
        if (j + 2 < nkt) step(sK2, sV2, sK1, sV1, j + 2);
    }
    wait_vmcnt<0>();  // no DMA may still be writing this workgroup's LDS when it exits

    // Epilogue: O = acc / l, L = (m + log2 l) * ln 2 (natural log of the scaled scores).
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        const int qi = qw0 + qb * 32 + l32;
        const float lt = wave_xor32_sum(lrow[qb]);
        if (qi < S) {
            const float inv = 1.f / lt;
#pragma unroll
            for (int db = 0; db < C::ND; ++db)
#pragma unroll
                for (int hr = 0; hr < 2; ++hr) {
                    const int d0 = db * 32 + 16 * hr + 8 * h;
                    if (d0 < D) store8<T>(o + (size_t)qi * D + d0, acc[qb][db], 8 * hr, inv);
                }
            if (h == 0) lse[qi] = (mrow[qb] + log2f(lt)) * kLn2;
        }
    }
}

template <typename T, typename C>
static int run_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int BH, int S,
                   float scale, int causal, hipStream_t stream) {
    const int nqt = (S + C::BQ - 1) / C::BQ;
    const long long grid = (long long)nqt * BH;
    if (grid > 0x7fffffffLL) return -1;
    hipLaunchKernelGGL((fwd_kernel<T, C>), dim3((unsigned)grid), dim3(C::NT), 0, stream,
                       (const T *)q, (const T *)k, (const T *)v, (T *)o, lse, BH, S, scale * kLog2e,
                       causal, nqt);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

template <typename T, int D>
static int fwd_for(const void *q, const void *k, const void *v, void *o, float *lse, int BH, int S,
                   float scale, int causal, hipStream_t stream) {
    // fp32 rows are twice the bytes: wide fp32 heads take 32-key tiles to fit three stages
    constexpr int BK = (sizeof(T) == 4 && D > 80) ? 32 : 64;
    // bf16 D=128: 64 queries per wave over 32-key tiles halves the K/V reads
    // per FLOP, but makes the query tiles twice as long; keep it for problems
    // with at least four such tiles per CU (short causal problems lose more
    // to the uneven tile lengths than they gain).  Measured slower at D=80.
    using C2 = FwdTile<T, D, 2, 32, 8>;
    if constexpr (sizeof(T) == 2 && D == 128) {
        const long long tiles2 = (long long)((S + C2::BQ - 1) / C2::BQ) * BH;
        if (tiles2 >= 4 * kNumCU) return run_fwd<T, C2>(q, k, v, o, lse, BH, S, scale, causal, stream);
    }
    return run_fwd<T, FwdTile<T, D, 1, BK, 8>>(q, k, v, o, lse, BH, S, scale, causal, stream);
}

template <typename T>
static int fwd_dispatch(int D, const void *q, const void *k, const void *v, void *o, float *lse,
                        int BH, int S, float scale, int causal, hipStream_t stream) {
    switch (D) {
    case 16: return fwd_for<T, 16>(q, k, v, o, lse, BH, S, scale, causal, stream);
    case 32: return fwd_for<T, 32>(q, k, v, o, lse, BH, S, scale, causal, stream);
    case 64: return fwd_for<T, 64>(q, k, v, o, lse, BH, S, scale, causal, stream);
    case 80: return fwd_for<T, 80>(q, k, v, o, lse, BH, S, scale, causal, stream);
    case 96: return fwd_for<T, 96>(q, k, v, o, lse, BH, S, scale, causal, stream);
    case 128: return fwd_for<T, 128>(q, k, v, o, lse, BH, S, scale, causal, stream);
    default: return -2;
    }
}

int launch_fwd(int dtype, const void *q, const void *k, const void *v, void *o, float *lse, int BH,
               int S, int D, float scale, int causal, hipStream_t stream) {
    if (dtype == 1) return fwd_dispatch<bf16>(D, q, k, v, o, lse, BH, S, scale, causal, stream);
    if (dtype == 0) return fwd_dispatch<float>(D, q, k, v, o, lse, BH, S, scale, causal, stream);
    return -2;
}

}  // namespace fa
