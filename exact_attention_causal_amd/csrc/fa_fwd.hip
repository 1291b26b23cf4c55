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
//   * the running maximum is allowed to lag: a tile is exponentiated against
//     it as it stands and kept when the probabilities stay below 2^8, so most
//     tiles form no row maximum and rescale nothing (exactness is kept because
//     O and l share the stale max);
//   * K/V tiles are loaded straight into LDS (global_load_lds_dwordx4) into
//     three stages, so the next two tiles stream in while the current one is
//     used and no registers or VALU work are spent staging them;
//   * workgroups are dispatched longest-first (highest query tile first) so
//     the short causal tiles fill in the tail.
#include "fa_common.hpp"
#include "fa_launch.hpp"

#include <algorithm>

namespace fa {

// NG = 2 (problems with few query tiles): the waves form two groups that
// share their queries and split the key tiles (group g takes tiles g, g+2,
// ...), each with its own LDS ring; group 1 hands its (m, l, O) to group 0,
// which merges and stores.  Halves the longest tile's key walk.
template <typename T, int D_, int NQB_, int BK_, int NW_, int NG_ = 1>
struct FwdTile {
    static constexpr int D = D_, NQB = NQB_, BK = BK_;
    static constexpr int NW = NW_, NT = NW * kWave;
    static constexpr int NG = NG_, NWG = NW / NG;    // key groups, waves per group
    static constexpr int BQ = NWG * NQB * 32;         // queries per workgroup
    static constexpr int KPL = Mma<T>::KPL;
    static constexpr int NSD = D / 2 / KPL;           // MFMAs over d per 32x32 block
    static constexpr int NKB = BK / 32;               // 32-key blocks per tile
    // bf16 D = 16 (mod 32): the last 16 output rows form a 16-row tail
    static constexpr bool TAIL = KPL == 8 && D % 32 == 16;
    static constexpr int ND = TAIL ? D / 32 : (D + 31) / 32;  // 32-row output blocks over d
    static constexpr int NI = 16 / KPL;               // MFMAs per 32-key reduction block
    using DMA = TileDma<T, D, BK, NWG / 2>;          // half a group's waves load K, half V
    static constexpr int TILE = DMA::ELEMS;           // elements per K or V tile
    static_assert(D % 16 == 0 && BK % 32 == 0 && NW % 2 == 0, "tile shape");
    static_assert(NG == 1 || (NG == 2 && NQB == 1 && NWG % 2 == 0), "key groups");
    // the merge hands 8 floats per lane at a time through the first K stage
    static_assert(NG == 1 || TILE * (int)sizeof(T) >= NWG * kWave * 8 * 4, "merge buffer");
};

// The running maximum m may lag the scores: a tile whose probabilities
// p = exp2(s - m) sum to at most 2^kRescaleSlack per lane (16 or 32 of them)
// is accepted as it is -- such p are held by fp32 and bf16 exactly as well as
// values <= 1, and O and l share the stale m -- and only a larger sum makes
// the tile take the exact path, which moves m to the tile's maximum.
constexpr float kRescaleSlack = 8.f;
constexpr float kRescaleSum = 256.f;  // 2^kRescaleSlack
static_assert(kRescaleSum == (float)(1 << (int)kRescaleSlack), "sum limit");

// Problem shape of one launch.  Query i of a head sits `off` positions after
// key 0, so the causal mask allows key j iff j <= i + off (off = 0 and
// Sq = Sk for self-attention).  The keys may be split into chunks of `chunk`
// rows, one per blockIdx.y, each producing its own normalised O and L over
// its keys (outputs `o_split` / `l_split` elements apart).
struct FwdShape {
    int BH, Sq, Sk, off, chunk, causal, nqt;
    float c;  // scale * log2(e)
    long long o_split, l_split;
    int band;  // workgroup order (tile_order): 0, or bands of this many tiles per XCD
};

// GEN = false is self-attention (no shift, one chunk of all keys): the shift
// is then a compile-time zero, which the register allocator needs to keep the
// 64-queries-per-wave tile within 256 registers.  The bf16 D=80 tile is held to
// 128 registers (four waves per SIMD), so two workgroups share a CU: 5 %
// faster than one workgroup with 150 registers.
template <typename T, typename C, typename OutT, bool GEN>
__global__ __launch_bounds__(C::NT, (!GEN && C::D == 80 && C::KPL == 8 && C::NQB == 1) ? 4 : 1) void fwd_kernel(const T *__restrict__ q, const T *__restrict__ k,
                                                    const T *__restrict__ v, OutT *__restrict__ o,
                                                    float *__restrict__ lse, FwdShape a) {
    using M = Mma<T>;
    using frag = typename M::frag;
    constexpr int D = C::D, NQB = C::NQB, BK = C::BK;
    // Three stages of K and V tiles: two tiles stream in while one is used.
    // Each stage is its own array and the loop is unrolled by three, so the
    // compiler can see that reads of one stage never alias the DMA into the
    // others and does not wait for the tiles in flight.
    __shared__ __attribute__((aligned(1024))) T sK0[C::NG * C::TILE], sK1[C::NG * C::TILE], sK2[C::NG * C::TILE];
    __shared__ __attribute__((aligned(1024))) T sV0[C::NG * C::TILE], sV1[C::NG * C::TILE], sV2[C::NG * C::TILE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave_all = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = C::NG == 1 ? 0 : wave_all / C::NWG;          // key group
    const int wave = C::NG == 1 ? wave_all : wave_all % C::NWG;  // wave within its group
    const int gofs = grp * C::TILE;                              // the group's LDS ring
    const int h = lane >> 5, l32 = lane & 31;
    const int BH = a.BH, S = a.Sq, causal = a.causal;
    const float c = a.c;
    const int bid = blockIdx.x;
    int rank, bh;  // longest query tile first (see tile_order)
    tile_order(bid, BH, a.nqt, a.band, rank, bh);
    const int qt = causal ? a.nqt - 1 - rank : rank;
    // this launch's keys: chunk blockIdx.y of the head's key rows
    const int kbeg = GEN ? blockIdx.y * a.chunk : 0;
    // (readfirstlane keeps these wave-uniform in scalar registers: the clamp
    // is selected as vector min/max, which would make every branch on them
    // look divergent)
    const int Sk = GEN ? __builtin_amdgcn_readfirstlane(max(0, min(a.chunk, a.Sk - kbeg))) : S;
    const int off = GEN ? __builtin_amdgcn_readfirstlane(a.off - kbeg) : 0;
    q += (size_t)bh * S * D;
    k += ((size_t)bh * a.Sk + kbeg) * D;
    v += ((size_t)bh * a.Sk + kbeg) * D;
    o += blockIdx.y * a.o_split + (size_t)bh * S * D;
    lse += blockIdx.y * a.l_split + (size_t)bh * S;
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
    TailReader<D> tt;  // (16-row tail only)
    if constexpr (C::TAIL) tt.init(lane);

    f32x16 acc[NQB][C::ND > 0 ? C::ND : 1];
    f32x4 tacc[NQB][2];  // 16-row tail: queries 0..15 and 16..31 of the block
    float mrow[NQB], lrow[NQB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        mrow[qb] = -INFINITY;
        lrow[qb] = 0.f;
#pragma unroll
        for (int db = 0; db < C::ND; ++db) acc[qb][db] = f32x16{};
        tacc[qb][0] = f32x4{};
        tacc[qb][1] = f32x4{};
    }

    const int qend = min(q0 + C::BQ, S);
    int nkt = (Sk + BK - 1) / BK;
    if (causal) {
        const int last = qend - 1 + off;  // last key any query of the tile may see
        nkt = last < 0 ? 0 : min(nkt, last / BK + 1);
    }

    typename C::DMA dma;
    const int half = wave / (C::NWG / 2), hw = wave % (C::NWG / 2);
    dma.init(lane, hw);
    // this wave's share of key/value tile j: K (first half of the waves) or V
    auto issue = [&](T *nK, T *nV, int j) { dma.issue(half ? nV : nK, half ? v : k, j * BK, Sk, hw); };
    // the group's tiles: grp, grp + NG, grp + 2 NG, ...
    issue(sK0 + gofs, sV0 + gofs, grp);
    issue(sK1 + gofs, sV1 + gofs, C::NG + grp);

    // The prefetch of a tile goes out one instruction at a time, spread over a
    // step's work (parts: one before each S^T block and each O^T block).  It
    // is issued unconditionally -- past the last tile its range is empty and
    // it fetches nothing -- because a conditional issue makes the compiler
    // wait for every DMA before the next LDS read.
    constexpr int NP = 2 * C::NKB;
    auto rs = C::DMA::range(k, 0, 0);  // range of the tile being prefetched
    T *nT = sK2 + gofs;                // and the stage it lands in
    auto part = [&](int p) {
        if (p >= 0) dma.issue_part(p, NP, nT, rs, hw);
    };
    auto all_parts = [&]() {
#pragma unroll
        for (int p = 0; p < NP; ++p) part(p);
    };
    // whether tile j holds any key this wave's queries may see
    auto active = [&](int j) {
        return j >= 0 && j < nkt && qw0 < S && !(causal && j * BK > qw0 + NQB * 32 - 1 + off);
    };

    // S^T of a tile, block (kb, qb): rows = keys j0 + 32*kb + ridx(r, h), col = query.
    // Prefetch part p0 + kb goes out before key block kb (p0 < 0: none).
    f32x16 s[NQB][C::NKB];
    auto qk = [&](const T *tK, int p0) {
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) {
            part(p0 < 0 ? -1 : p0 + kb);
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
    };
    // scores of tile j that a query may not see become -inf
    auto mask = [&](int j) {
        const int j0 = j * BK;
        const bool need_mask = (causal && j0 + BK - 1 > qw0 + off) || (j0 + BK > Sk);
        if (need_mask) {
            // (the empty volatile asm keeps this block a real branch: only
            // tiles crossing the diagonal or the sequence end pay for masking)
            asm volatile("");
            // key j0 + 32*kb + ridx(r, h) is kept iff it is below `lim`
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb) {
                const int qi = qw0 + qb * 32 + l32;
                const int lim = causal ? min(qi + 1 + off, Sk) : Sk;
                const int t = lim - j0 - 2 * h;
#pragma unroll
                for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        s[qb][kb][r] = (32 * kb + ridx(r, 0) < t) ? s[qb][kb][r] : -INFINITY;
            }
        }
    };
    // Online softmax of tile j in base 2 (scores scaled by c = scale*log2 e),
    // P left in s and its row sums added to l.  Fast path: exponentiate against
    // the running maxima as they stand, and keep the result when every lane's
    // sum (so every p) is at most 2^kRescaleSlack: no row maximum is formed.
    // Otherwise the tile's scores are formed again and the exact path moves
    // each row's maximum to the tile's own.  A row that has seen no key yet
    // (m = -inf) always takes the exact path: its fast sum is inf or NaN.
    auto softmax = [&](const T *tK, int j) {
        mask(j);
        float ps[NQB];
        bool ok = true;
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
            ps[qb] = 0.f;
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = fast_exp2(fmaf(s[qb][kb][r], c, -mrow[qb]));
                    s[qb][kb][r] = p;
                    ps[qb] += p;
                }
            ok = ok && ps[qb] <= kRescaleSum;  // (false for inf and NaN)
        }
        if (__ballot(!ok) != 0) {  // wave-uniform: rare after a row's first tile
            qk(tK, -1);
            mask(j);
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb) {
                float mx = -INFINITY;
#pragma unroll
                for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[qb][kb][r]);
                mx = wave_xor32_max(mx) * c;
                const bool grow = mx > mrow[qb];
                if (__ballot(grow) != 0) {
                    const float mnew = grow ? mx : mrow[qb];
                    // (a row that has seen no key yet keeps -inf: its alpha is
                    // 1, not exp2(-inf - -inf))
                    const float alpha = (mnew == -INFINITY) ? 1.f : fast_exp2(mrow[qb] - mnew);
                    lrow[qb] *= alpha;
#pragma unroll
                    for (int db = 0; db < C::ND; ++db) acc[qb][db] *= alpha;
                    if constexpr (C::TAIL) {
                        float a0, a1;
                        tail_cols(alpha, a0, a1);
                        tacc[qb][0] *= a0;
                        tacc[qb][1] *= a1;
                    }
                    mrow[qb] = mnew;
                }
                // a row whose maximum is still -inf has seen only masked keys: use 0
                const float muse = (mrow[qb] == -INFINITY) ? 0.f : mrow[qb];
                ps[qb] = 0.f;
#pragma unroll
                for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float p = fast_exp2(fmaf(s[qb][kb][r], c, -muse));
                        s[qb][kb][r] = p;
                        ps[qb] += p;
                    }
            }
        }
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) lrow[qb] += ps[qb];
    };
    // O^T += V^T P^T; prefetch part p0 + kb goes out before key block kb (p0 < 0: none)
    auto pv = [&](const T *tV, int p0) {
#pragma unroll
        for (int kb = 0; kb < C::NKB; ++kb) {
            part(p0 < 0 ? -1 : p0 + kb);
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
            if constexpr (C::TAIL) {
                const bf16x8 ta = tt.load(tV, kb, 32 * C::ND);
#pragma unroll
                for (int qb = 0; qb < NQB; ++qb) {
                    bf16x8 b0, b1;
                    tail_bfrag(pf[qb], b0, b1);
                    tacc[qb][0] = mma16(ta, b0, tacc[qb][0]);
                    tacc[qb][1] = mma16(ta, b1, tacc[qb][1]);
                }
            }
        }
    };
    // start of step j: tile j has landed everywhere, then the group's tile
    // two steps on (j + 2 NG) is aimed at (nK, nV)
    auto begin_step = [&](T *nK, T *nV, int j) {
        wait_vmcnt<C::DMA::IPW>();  // this wave's part of tile j has landed (the next may be in flight)
        lds_barrier();              // every part of it; the stage the next-but-one tile goes to is released
        rs = C::DMA::range(half ? v : k, (j + 2 * C::NG) * BK, Sk);
        nT = half ? nV : nK;
    };

    // Three stages: step j uses tile j, tile j+1 is in flight and tile j+2
    // goes to the stage tile j-1 used.
    auto step = [&](const T *tK, const T *tV, T *nK, T *nV, int j) {
        begin_step(nK, nV, j);
        if (!active(j)) {
            all_parts();
        } else {
            qk(tK, 0);
            softmax(tK, j);
            pv(tV, C::NKB);
        }
        wait_lgkm0();  // this wave's reads of the stage are complete before the next barrier
    };
    // (every wave runs the same number of steps; a group's tile past nkt is inactive)
    const int nst = (nkt + C::NG - 1) / C::NG;
    for (int t = 0; t < nst; t += 3) {
        step(sK0 + gofs, sV0 + gofs, sK2 + gofs, sV2 + gofs, C::NG * t + grp);
        if (t + 1 < nst) step(sK1 + gofs, sV1 + gofs, sK0 + gofs, sV0 + gofs, C::NG * (t + 1) + grp);
        if (t + 2 < nst) step(sK2 + gofs, sV2 + gofs, sK1 + gofs, sV1 + gofs, C::NG * (t + 2) + grp);
    }
    wait_vmcnt<0>();  // no DMA may still be writing this workgroup's LDS when it exits

    if constexpr (C::NG == 2) {
        // Group 1 hands its (m, l, O^T) to group 0 through the first K stage,
        // 8 floats per lane at a time; group 0 rescales both to the larger m
        // and adds (O and l of either half share that half's m).
        float *xb = reinterpret_cast<float *>(sK0) + wave * kWave + lane;
        constexpr int XS = C::NWG * kWave;  // floats per handed register
        // lds_barrier() does not wait for this wave's LDS accesses (the
        // hardware does not either), so each side waits for its own before
        // the barrier that publishes them: group 1's writes must have landed
        // before group 0 reads, and group 0's reads must be done before the
        // next round's writes reuse the buffer.
        auto hand = [&](auto put, auto take) {
            lds_barrier();  // the buffer is free (every earlier read done)
            if (grp == 1) put();
            wait_lgkm0();
            lds_barrier();  // the writes are visible
            if (grp == 0) take();
            wait_lgkm0();
        };
        float a0 = 1.f, a1 = 0.f;
        hand([&] { xb[0] = mrow[0]; xb[XS] = lrow[0]; },
             [&] {
                 const float m1 = xb[0], l1 = xb[XS];
                 const float m0 = mrow[0];
                 const float mn = fmaxf(m0, m1);
                 // (a half that saw no key has m = -inf and l = 0: weight 0)
                 a0 = (m0 == -INFINITY) ? 0.f : fast_exp2(m0 - mn);
                 a1 = (m1 == -INFINITY) ? 0.f : fast_exp2(m1 - mn);
                 lrow[0] = a0 * lrow[0] + a1 * l1;
                 mrow[0] = mn;
             });
#pragma unroll
        for (int db = 0; db < C::ND; ++db)
#pragma unroll
            for (int hr = 0; hr < 2; ++hr)
                hand([&] {
#pragma unroll
                         for (int t = 0; t < 8; ++t) xb[t * XS] = acc[0][db][8 * hr + t];
                     },
                     [&] {
#pragma unroll
                         for (int t = 0; t < 8; ++t)
                             acc[0][db][8 * hr + t] = a0 * acc[0][db][8 * hr + t] + a1 * xb[t * XS];
                     });
        if constexpr (C::TAIL) {
            // tail lanes hold queries of other lanes: their factors come by the same swap
            float b0, b1, c0, c1;
            tail_cols(a0, b0, b1);
            tail_cols(a1, c0, c1);
            hand([&] {
#pragma unroll
                     for (int t = 0; t < 4; ++t) {
                         xb[t * XS] = tacc[0][0][t];
                         xb[(4 + t) * XS] = tacc[0][1][t];
                     }
                 },
                 [&] {
#pragma unroll
                     for (int t = 0; t < 4; ++t) {
                         tacc[0][0][t] = b0 * tacc[0][0][t] + c0 * xb[t * XS];
                         tacc[0][1][t] = b1 * tacc[0][1][t] + c1 * xb[(4 + t) * XS];
                     }
                 });
        }
        if (grp == 1) return;
    }

    // Epilogue: O = acc / l, L = (m + log2 l) * ln 2 (natural log of the scaled scores).
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        const int qi = qw0 + qb * 32 + l32;
        const float lt = wave_xor32_sum(lrow[qb]);
        // a row that allows no key of this launch (shifted or split keys
        // only) has the empty result O = 0, L = -inf
        const bool empty = !(lt > 0.f);
        const float inv = empty ? 0.f : 1.f / lt;
        if constexpr (C::TAIL) {
            // tail lane 16g + i holds rows 4g..4g+3 of queries i and 16 + i
            float i0, i1;
            tail_cols(inv, i0, i1);
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int qt_ = qw0 + qb * 32 + 16 * t + (lane & 15);
                if (qt_ < S)
                    store4<OutT>(o + (size_t)qt_ * D + 32 * C::ND + 4 * (lane >> 4), tacc[qb][t], t ? i1 : i0);
            }
        }
        if (qi < S) {
#pragma unroll
            for (int db = 0; db < C::ND; ++db)
#pragma unroll
                for (int hr = 0; hr < 2; ++hr) {
                    const int d0 = db * 32 + 16 * hr + 8 * h;
                    if (d0 < D) store8<OutT>(o + (size_t)qi * D + d0, acc[qb][db], 8 * hr, inv);
                }
            if (h == 0) lse[qi] = empty ? -INFINITY : (mrow[qb] + log2f(lt)) * kLn2;
        }
    }
}

template <typename T, typename C, typename OutT, bool GEN>
static int run_fwd(const void *q, const void *k, const void *v, OutT *o, float *lse, FwdShape a,
                   int n_split, hipStream_t stream) {
    a.nqt = (a.Sq + C::BQ - 1) / C::BQ;
    const long long grid = (long long)a.nqt * a.BH;
    if (grid > 0x7fffffffLL || n_split > 65535) return -1;
    hipLaunchKernelGGL((fwd_kernel<T, C, OutT, GEN>), dim3((unsigned)grid, (unsigned)n_split), dim3(C::NT), 0,
                       stream, (const T *)q, (const T *)k, (const T *)v, o, lse, a);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

// Key-tile rows: fp32 rows are twice the bytes, so wide fp32 heads take
// 32-key tiles to fit three stages.
template <typename T, int D>
constexpr int fwd_bk() { return (sizeof(T) == 4 && D > 80) ? 32 : 64; }

// Key tiles of the two-group tile (bf16, D >= 64): its LDS holds two rings.
template <int D>
constexpr int fwd_bk2() { return D > 80 ? 32 : 64; }

FwdPlan fwd_plan(int dtype, int BH, int S, int D, int ncu) {
    const bool bf = dtype == 1;
    const long long cu = ncu > 0 ? ncu : 1;
    // Few 256-query tiles per CU: two key groups per workgroup on 128-query
    // tiles (the longest tile walks half the keys per group). Measured
    // 1.4-1.9x faster at one tile per CU or fewer (one head, S = 1024 to
    // 65536; four heads at S = 16384).  Past one tile per CU the walk must be
    // long enough to pay for the merge and the shorter tiles (every tile
    // count at S = 512 .. 32768, D = 64, 80, 128): D = 64 and 80 gain 3-10 %
    // at two tiles per CU from S = 4096 on but lose 14-18 % at S = 2048;
    // D = 96 and 128 gain up to 1.5 tiles per CU from S = 2048 on, lose 4 %
    // at one tile per CU at S = 1024, and are 10 % slower at 1.75 and 2.
    if (bf && D >= 64) {
        const long long tiles1 = (long long)((S + 255) / 256) * BH;
        const bool two = D <= 80 ? tiles1 <= cu || (tiles1 <= 2 * cu && S >= 4096)
                                 : 2 * tiles1 <= cu || (2 * tiles1 <= 3 * cu && S >= 2048);
        if (two) return FwdPlan{128, 2, D > 80 ? 32 : 64, 0};
    }
    // bf16 D=128: 64 queries per wave over 32-key tiles halves the K/V reads
    // per FLOP, but makes the query tiles twice as long: the masked half of
    // the diagonal tile and the uneven tile lengths cost more at short
    // sequences.  Measured against the 256-query tile: 19.6 % slower at
    // S = 8192 with 4 tiles of 512 per CU, 2.5-6 % faster from S = 16384 on
    // with 2 tiles per CU, 50 % slower with one.  Measured slower at D=80.
    // Its workgroups go to the XCDs head by head in bands of 64 tiles
    // (tile_order): at S = 65536, H = 16 that halves the kernel's HBM
    // traffic (FETCH_SIZE + WRITE_SIZE 9.51 -> 4.67 GB) and runs 0.5-1 %
    // faster; the same order made the D = 80 tile 4-9 % slower.
    if (bf && D == 128) {
        const long long tiles2 = (long long)((S + 511) / 512) * BH;
        if (S >= 16384 && tiles2 >= 2 * cu) return FwdPlan{512, 1, 32, BH % kNumXcd == 0 ? 64 : 0};
    }
    return FwdPlan{256, 1, (!bf && D > 80) ? 32 : 64, 0};
}

int fwd_split(int dtype, int BH, int S, int D, int causal, int ncu, size_t max_part_bytes) {
    if ((dtype != 0 && dtype != 1) || !head_dim_supported(D)) return 1;
    const long long cu = ncu > 0 ? ncu : 1;
    // 256-query tiles of the plain forward; the longest causal one walks all
    // keys.  Key chunks shorten that walk n-fold at the price of writing and
    // merging n fp32 partial results.  Measured against the plain forward
    // (every chunk count 2..32; B*H = 1..32, S = 512..32768, D = 64, 128):
    const long long tiles = (long long)BH * ((S + 255) / 256);
    long long n = 1;
    if (dtype == 1) {
        // bf16 (whose forward already runs two key groups when tiles are
        // few, from D = 64 on): only long walks over very few tiles gain, 1.1-2.3x
        if (S >= 2048 && 4 * tiles <= cu && 64 * tiles <= S)
            n = 8 * tiles <= cu ? 8 : 4;
        else if (D <= 32 && S >= 4096) {
            // D = 16 and 32 have no two-group tile: up to two tiles per CU
            // the chunks pay as well (B*H = 1..32, S = 2048..65536, every
            // count up to 32, causal and not): 6 causal chunks 1.1-2.3x
            // faster than none, within about 10 % of the best count; without
            // the mask 2-4 chunks, 1.05-2x.  Below S = 4096 with as many tiles,
            // and past one tile per CU below S = 16384, none pay.
            if (2 * tiles <= cu)
                n = causal ? 6 : 4;
            else if (tiles <= cu || (tiles <= 2 * cu && S >= 16384))
                n = causal ? 6 : 2;
        } else if (D >= 64 && causal && 2 * tiles <= cu && S >= 8192) {
            // at up to CU/2 tiles 3 causal chunks beat the two-group tile
            // by 12-28 % (B*H = 1..4, S = 8192..32768, D = 64, 80, 128);
            // at one tile per CU, and without the mask, no count does
            n = 3;
        }
    } else if (D == 128) {
        // fp32 D = 128, whose chunk tile has 128 queries (fwd_gen_nw): about
        // one chunk tile per CU, fewer chunks past CU/4 tiles (each chunk's
        // merge input grows with n).  Measured at B*H = 1..16, S = 2048..32768
        // against every n up to 16, causal and not: 4-44 % faster than the
        // rule below, and within 3 % of the best count except at one point
        // (one causal head at S = 8192: 16 chunks 11 % faster).  Without the
        // mask every tile walks all keys: 3 chunks would leave half a round
        // of tiles, and past CU tiles the plain forward already fills the GPU.
        const long long t = (long long)BH * ((S + 127) / 128);
        if (4 * t <= cu)
            n = cu / t;
        else if (2 * t <= cu)
            n = causal ? 3 : 2;
        else if (t <= (causal ? 2 * cu : cu))
            n = 2;
    } else {
        // fp32 (long steps, no two-group tile): 1.5-10x up to one tile per CU
        if (8 * tiles <= cu)
            n = (cu + tiles - 1) / tiles;
        else if (2 * tiles <= cu)
            n = S >= 4096 ? 16 : 4;
        else if (tiles <= cu && causal)
            // (the causal imbalance of one tile per CU; level or slower
            // without the mask.  D >= 64: 2 chunks 1.5-1.6x faster, within
            // 10 % of the best count; D = 16 and 32 gain little from 2
            // (0.96-1.0) but 1.1-1.7x from 8 (B*H = 1..32, S = 2048..65536))
            n = D <= 32 ? 8 : 2;
    }
    n = std::min<long long>(n, std::min<long long>(32, S / 64));  // chunks of 64 keys or more
    while (n > 1 && fwd_part_bytes((int)n, BH, S, D) > max_part_bytes) --n;
    return n < 2 ? 1 : (int)n;
}

// Launch tile C if it is the one the plan names.
template <typename T, typename C, typename OutT, bool GEN>
static bool pick(const FwdPlan &p, int &rc, const void *q, const void *k, const void *v, OutT *o, float *lse,
                 const FwdShape &a, int n_split, hipStream_t stream) {
    if (p.bq != C::BQ || p.groups != C::NG || p.bk != C::BK) return false;
    rc = run_fwd<T, C, OutT, GEN>(q, k, v, o, lse, a, n_split, stream);
    return true;
}

// Waves of the shifted / split-key tile.
template <typename T, int D>
constexpr int fwd_gen_nw() { return (sizeof(T) == 4 && D == 128) ? 4 : 8; }

template <typename T, int D, typename OutT, bool GEN>
static int fwd_for(const void *q, const void *k, const void *v, OutT *o, float *lse, const FwdShape &a,
                   int n_split, int ncu, hipStream_t stream) {
    if constexpr (GEN) {
        // shifted / split keys: always the 32-query-per-wave tile
        return run_fwd<T, FwdTile<T, D, 1, fwd_bk<T, D>(), fwd_gen_nw<T, D>()>, OutT, GEN>(q, k, v, o, lse, a,
                                                                                           n_split, stream);
    } else {
        const FwdPlan p = fwd_plan(sizeof(T) == 2 ? 1 : 0, a.BH, a.Sq, D, ncu);
        FwdShape b = a;
        b.band = p.band;
        int rc = -5;
        if constexpr (sizeof(T) == 2 && D >= 64)
            if (pick<T, FwdTile<T, D, 1, fwd_bk2<D>(), 8, 2>, OutT, GEN>(p, rc, q, k, v, o, lse, b, n_split, stream))
                return rc;
        if constexpr (sizeof(T) == 2 && D == 128)
            if (pick<T, FwdTile<T, D, 2, 32, 8>, OutT, GEN>(p, rc, q, k, v, o, lse, b, n_split, stream)) return rc;
        if (pick<T, FwdTile<T, D, 1, fwd_bk<T, D>(), 8>, OutT, GEN>(p, rc, q, k, v, o, lse, b, n_split, stream))
            return rc;
        return -5;  // (a plan with no matching tile: fwd_plan and the tiles disagree)
    }
}

template <typename T, bool GEN, typename OutT>
static int fwd_dispatch(int D, const void *q, const void *k, const void *v, OutT *o, float *lse,
                        const FwdShape &a, int n_split, int ncu, hipStream_t stream) {
    switch (D) {
    case 16: return fwd_for<T, 16, OutT, GEN>(q, k, v, o, lse, a, n_split, ncu, stream);
    case 32: return fwd_for<T, 32, OutT, GEN>(q, k, v, o, lse, a, n_split, ncu, stream);
    case 64: return fwd_for<T, 64, OutT, GEN>(q, k, v, o, lse, a, n_split, ncu, stream);
    case 80: return fwd_for<T, 80, OutT, GEN>(q, k, v, o, lse, a, n_split, ncu, stream);
    case 96: return fwd_for<T, 96, OutT, GEN>(q, k, v, o, lse, a, n_split, ncu, stream);
    case 128: return fwd_for<T, 128, OutT, GEN>(q, k, v, o, lse, a, n_split, ncu, stream);
    default: return -2;
    }
}

int launch_fwd(int dtype, const void *q, const void *k, const void *v, void *o, float *lse, int BH,
               int S, int D, float scale, int causal, int ncu, hipStream_t stream) {
    FwdShape a{BH, S, S, 0, S, causal, 0, scale * kLog2e, 0, 0, 0};
    if (dtype == 1) return fwd_dispatch<bf16, false>(D, q, k, v, (bf16 *)o, lse, a, 1, ncu, stream);
    if (dtype == 0) return fwd_dispatch<float, false>(D, q, k, v, (float *)o, lse, a, 1, ncu, stream);
    return -2;
}

int launch_fwd_partial(int dtype, const void *q, const void *k, const void *v, float *o_parts,
                       float *lse_parts, int BH, int Sq, int Sk, int D, float scale, int causal,
                       int q_offset, int n_split, int chunk, hipStream_t stream) {
    FwdShape a{BH, Sq, Sk, q_offset, chunk, causal, 0, scale * kLog2e, (long long)BH * Sq * D,
               (long long)BH * Sq, 0};
    if (dtype == 1) return fwd_dispatch<bf16, true>(D, q, k, v, o_parts, lse_parts, a, n_split, 0, stream);
    if (dtype == 0) return fwd_dispatch<float, true>(D, q, k, v, o_parts, lse_parts, a, n_split, 0, stream);
    return -2;
}

// Every kernel the dispatch above can launch, instantiated explicitly: the
// host compilation pass has been seen to drop the launch stubs of some
// implicitly instantiated kernel templates (an undefined symbol at load
// time), so the list is spelled out.
#define COMMA ,
#define FA_FWD_KERNEL(T, C, OUT, GEN)                                                                         \
    template __global__ void fwd_kernel<T, C, OUT, GEN>(const T *, const T *, const T *, OUT *, float *,     \
                                                        FwdShape);
#define FA_FWD_HEAD(T, D)                                                                        \
    FA_FWD_KERNEL(T, FwdTile<T COMMA D COMMA 1 COMMA fwd_bk<T COMMA D>() COMMA 8>, T, false)    \
    FA_FWD_KERNEL(T, FwdTile<T COMMA D COMMA 1 COMMA fwd_bk<T COMMA D>() COMMA fwd_gen_nw<T COMMA D>()>, float, true)
FA_FWD_HEAD(bf16, 16)
FA_FWD_HEAD(bf16, 32)
FA_FWD_HEAD(bf16, 64)
FA_FWD_HEAD(bf16, 80)
FA_FWD_HEAD(bf16, 96)
FA_FWD_HEAD(bf16, 128)
FA_FWD_HEAD(float, 16)
FA_FWD_HEAD(float, 32)
FA_FWD_HEAD(float, 64)
FA_FWD_HEAD(float, 80)
FA_FWD_HEAD(float, 96)
FA_FWD_HEAD(float, 128)
FA_FWD_KERNEL(bf16, FwdTile<bf16 COMMA 128 COMMA 2 COMMA 32 COMMA 8>, bf16, false)
FA_FWD_KERNEL(bf16, FwdTile<bf16 COMMA 64 COMMA 1 COMMA fwd_bk2<64>() COMMA 8 COMMA 2>, bf16, false)
FA_FWD_KERNEL(bf16, FwdTile<bf16 COMMA 80 COMMA 1 COMMA fwd_bk2<80>() COMMA 8 COMMA 2>, bf16, false)
FA_FWD_KERNEL(bf16, FwdTile<bf16 COMMA 96 COMMA 1 COMMA fwd_bk2<96>() COMMA 8 COMMA 2>, bf16, false)
FA_FWD_KERNEL(bf16, FwdTile<bf16 COMMA 128 COMMA 1 COMMA fwd_bk2<128>() COMMA 8 COMMA 2>, bf16, false)
#undef FA_FWD_HEAD
#undef FA_FWD_KERNEL
#undef COMMA

}  // namespace fa
