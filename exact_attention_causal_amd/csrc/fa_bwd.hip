// fa_bwd.hip -- causal FlashAttention-2 backward pass for gfx950.
//
// Follows the CS336 Assignment 2 handout, section 4.2.3 (Algorithm 2) and
// Eq. 13-19: the probabilities are recomputed from the saved logsumexp,
// P_ij = exp(S_ij - L_i), with the per-query statistic
// D_i = rowsum(O o dO) computed beforehand, and the work is split into
//   * a key/value-outer pass: one workgroup per tile of keys (32 per wave,
//     or per pair of waves for fp32) accumulates dV = P^T dO and
//     dK = dS^T Q * scale over the query tiles at or below the diagonal;
//   * a query-outer pass: one workgroup per tile of queries accumulates
//     dQ = dS K * scale over the key tiles at or before the diagonal.
// P (and dS) are computed twice, once in each pass, so no partial sums ever
// cross workgroups: no atomics, bit-reproducible results (the handout's
// argument for Algorithm 2).  The only workspace is a base-2 copy of L.
//
// Register/LDS mapping (see fa_common.hpp): in the key-outer pass the scores
// are formed as S = Q K^T so that each lane owns one key column; P and dS
// then feed dV^T = dO^T P and dK^T = Q^T dS directly as B operands, with the
// Q^T and dO^T operands read out of the row-major Q and dO tiles by the
// transposing LDS read.  In the query-outer pass the scores are S^T = K Q^T
// (each lane owns one query), and dS^T feeds dQ^T = K^T dS^T, K^T again read
// transposed from the row-major K tile.
#include "fa_common.hpp"
#include "fa_launch.hpp"

#include <algorithm>
#include <atomic>
#include <mutex>

namespace fa {

// ---------------------------------------------------------------- delta ---
// D_i = sum_d O_id dO_id (handout Algorithm 2, first step), fp32 accumulation.
// A workgroup reduces 64 rows: each thread multiplies 16-byte chunks, partial
// sums meet in LDS, and 64 threads add a row's chunks in order.

template <typename T, int D>
__global__ __launch_bounds__(256) void delta_kernel(const T *__restrict__ o, const T *__restrict__ dout,
                                                    float *__restrict__ delta, long long rows) {
    constexpr int VEC = 16 / sizeof(T), CPR = D / VEC, RB = 64;
    __shared__ float part[RB][CPR + 1];
    const int tid = threadIdx.x;
    const long long r0 = (long long)blockIdx.x * RB;
    for (int u = tid; u < RB * CPR; u += 256) {
        const int rr = u / CPR, c = u % CPR;
        const long long row = r0 + rr;
        float acc = 0.f;
        if (row < rows) {
            const size_t off = (size_t)row * D + c * VEC;
            if constexpr (sizeof(T) == 2) {
                bf16x8 a = *reinterpret_cast<const bf16x8 *>(o + off);
                bf16x8 b = *reinterpret_cast<const bf16x8 *>(dout + off);
#pragma unroll
                for (int t = 0; t < 8; ++t) acc = fmaf((float)a[t], (float)b[t], acc);
            } else {
                f32x4 a = *reinterpret_cast<const f32x4 *>(o + off);
                f32x4 b = *reinterpret_cast<const f32x4 *>(dout + off);
#pragma unroll
                for (int t = 0; t < 4; ++t) acc = fmaf(a[t], b[t], acc);
            }
        }
        part[rr][c] = acc;
    }
    __syncthreads();
    if (tid < RB && r0 + tid < rows) {
        float s = 0.f;
#pragma unroll
        for (int c = 0; c < CPR; ++c) s += part[tid][c];
        delta[r0 + tid] = s;
    }
}

// L * log2(e) for every row, so that the two passes recompute
// P = 2^(S * scale * log2 e - L * log2 e) with one FMA per probability.
__global__ __launch_bounds__(256) void lse2_kernel(const float *__restrict__ lse, float *__restrict__ lse2,
                                                   long long rows) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i < rows) lse2[i] = lse[i] * kLog2e;
}

// --------------------------------------------------------- key-outer dK/dV ---
//
// Each 32-key block is owned by a pair of waves that split the block's four
// products between them (no product is computed twice):
//   * the P wave forms S = Q K^T, P = exp(S - L) (Eq. 13-14), hands P to its
//     partner through LDS and accumulates dV^T += dO^T P (Eq. 15);
//   * the dS wave forms dP = dO V^T (Eq. 16), and dS = P o (dP - D) (Eq. 17)
//     once its partner's P is there, and accumulates dK^T += Q^T dS (Eq. 19).
// So each wave keeps one B operand (K^T or V^T) and one accumulator in
// registers, which leaves room for two waves per SIMD.  The pair runs one
// query tile apart: in step i the P wave accumulates dV for tile i-1 and then
// forms P of tile i, while the dS wave does all of its work for tile i-1
// (whose P its partner wrote in step i-1).  One workgroup barrier per step
// separates them, and each wave's vector work (exponentials, dS) overlaps its
// partner's matrix products on the shared SIMD.

// Problem shape of one backward launch.  Query i sits `off` positions after
// key 0, so the causal mask allows key j iff j <= i + off (off = 0 and
// Sq = Sk for self-attention).  With GEN = false (self-attention) the shift is
// a compile-time zero, the gradients are written in the input dtype and the
// row statistic the kernels read is L * log2(e) (prepared once per launch);
// with GEN = true they are fp32 contributions of this key set, added to the
// outputs when `accumulate` is set, and the statistic is the natural-log L.  L and D are the statistics of the whole
// attention, so a row with L = -inf allows no key of this set either: every
// tile holding such a row crosses the causal boundary, and the mask zeroes
// the row's P (the infinite exponential is selected away, never multiplied).
struct BwdShape {
    int BH, Sq, Sk, off, causal, nqt, accumulate;
    float c, scale;  // c = scale * log2(e)
    // key-set calls (GEN) may cut the reduction of a pass into chunks, one per
    // blockIdx.y, each writing its own partial result: dK/dV over chunks of
    // `qchunk` queries (partials BH*Sk*D elements apart), dQ over chunks of
    // `kchunk` keys (BH*Sq*D apart).  One chunk each is the plain call.
    int qchunk, kchunk;
    int band;  // workgroup order of the two passes (tile_order)
};

// 8 consecutive gradient values of one lane, times `mul`, stored or (GEN)
// added to the fp32 output.
template <bool GEN, typename OutT>
__device__ inline void out8(OutT *dst, const f32x16 &acc, int r0, float mul, int accumulate) {
    if constexpr (GEN) {
        f32x16 x = acc;
        if (accumulate) {
            const f32x4 a = *reinterpret_cast<const f32x4 *>(dst);
            const f32x4 b = *reinterpret_cast<const f32x4 *>(dst + 4);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                x[r0 + t] = fmaf(x[r0 + t], mul, a[t]);
                x[r0 + 4 + t] = fmaf(x[r0 + 4 + t], mul, b[t]);
            }
            store8<OutT>(dst, x, r0, 1.f);
        } else {
            store8<OutT>(dst, x, r0, mul);
        }
    } else {
        store8<OutT>(dst, acc, r0, mul);
    }
}
// The same for the 4 consecutive elements a lane holds of a 16-row tail block.
template <bool GEN, typename OutT>
__device__ inline void out4(OutT *dst, const f32x4 &acc, float mul, int accumulate) {
    if constexpr (GEN) {
        if (accumulate) {
            const f32x4 a = *reinterpret_cast<const f32x4 *>(dst);
            store4<OutT>(dst, f32x4{fmaf(acc[0], mul, a[0]), fmaf(acc[1], mul, a[1]),
                                    fmaf(acc[2], mul, a[2]), fmaf(acc[3], mul, a[3])}, 1.f);
        } else {
            store4<OutT>(dst, acc, mul);
        }
    } else {
        store4<OutT>(dst, acc, mul);
    }
}

template <typename T, int D_, int BQ2_>
struct KvTile {
    static constexpr int D = D_, BQ2 = BQ2_;
    static constexpr int NW = 8, NT = NW * kWave;
    static constexpr int NPAIR = NW / 2;
    static constexpr int BKV = NPAIR * 32;            // keys per workgroup
    static constexpr int NQ2 = BQ2 / 32;              // 32-query blocks per query tile
    static constexpr int KPL = Mma<T>::KPL;
    static constexpr int NSD = D / 2 / KPL;
    static constexpr int ND = (D + 31) / 32;
    static constexpr int NI = 16 / KPL;
    using DMA = TileDma<T, D, BQ2, NW / 2>;           // the P waves load Q, the dS waves dO
    using PD = typename DMA::PD;
    // a Q (dO) tile array also carries the tile's L (D) values, 64 per P (dS) wave
    static constexpr int XOFF = DMA::ELEMS;           // element offset of those values
    static constexpr int TILE = DMA::ELEMS + NPAIR * kWave * 4 / (int)sizeof(T);
    // P values of one 32x32 block (elements), fragment-major: fragment i of
    // lane l at i*64*KPL + l*KPL, so the 16-byte accesses of consecutive
    // lanes are contiguous (a 32-byte lane stride costs LDS bank conflicts)
    static constexpr int PBLK = 64 * 16;
    static constexpr int PBUF = NPAIR * NQ2 * PBLK;   // P of one query tile (one of two buffers)
    static_assert(D % 16 == 0 && BQ2 % 32 == 0 && BQ2 <= kWave, "tile shape");
};

template <typename T, typename C, typename OutT, bool GEN>
__global__ __launch_bounds__(C::NT) void dkdv_kernel(const T *__restrict__ q, const T *__restrict__ k,
                                                     const T *__restrict__ v, const T *__restrict__ dout,
                                                     const float *__restrict__ lse,
                                                     const float *__restrict__ delta, OutT *__restrict__ dk,
                                                     OutT *__restrict__ dv, BwdShape a) {
    using M = Mma<T>;
    using frag = typename M::frag;
    constexpr int D = C::D, BQ2 = C::BQ2;
    // Three stages of Q and dO tiles, each its own array (see the forward
    // kernel): tile i-1 (read transposed), tile i (read by rows) and tile i+1
    // (in flight).  A Q array also holds the tile's L values, a dO array its
    // D values -- keeping the number of DMA targets within what the compiler
    // tracks.  Two P buffers: the one written in this step and the one read.
    __shared__ __attribute__((aligned(1024))) T sQ0[C::TILE], sQ1[C::TILE], sQ2[C::TILE];
    __shared__ __attribute__((aligned(1024))) T sdO0[C::TILE], sdO1[C::TILE], sdO2[C::TILE];
    __shared__ __attribute__((aligned(16))) T sP[2 * C::PBUF];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int role = wave / C::NPAIR;   // 0: P / dV wave, 1: dS / dK wave
    const int pair = wave % C::NPAIR;
    const int h = lane >> 5, l32 = lane & 31;
    const int BH = a.BH, Sh = a.Sq, causal = a.causal;
    // this launch's queries: chunk blockIdx.y of the head's query rows
    // (key-set calls; uniform values kept in scalar registers, see the forward kernel)
    const int qbeg = GEN ? blockIdx.y * a.qchunk : 0;
    const int S = GEN ? __builtin_amdgcn_readfirstlane(min(a.qchunk, Sh - qbeg)) : Sh;
    const int Sk = GEN ? a.Sk : Sh;   // keys of the head
    // query i of the chunk sits off positions after key 0
    const int off = GEN ? __builtin_amdgcn_readfirstlane(a.off + qbeg) : 0;
    const float c = a.c;
    const int bid = blockIdx.x;
    const int kt = bid / BH;  // ascending: the tiles with the most query tiles go first
    const int bh = bid % BH;
    q += ((size_t)bh * Sh + qbeg) * D;
    dout += ((size_t)bh * Sh + qbeg) * D;
    k += (size_t)bh * Sk * D;
    v += (size_t)bh * Sk * D;
    const size_t part = GEN ? (size_t)blockIdx.y * BH * Sk * D : 0;
    dk += part + (size_t)bh * Sk * D;
    dv += part + (size_t)bh * Sk * D;
    lse += (size_t)bh * Sh + qbeg;
    delta += (size_t)bh * Sh + qbeg;
    const int k0 = kt * C::BKV;
    const int kw0 = k0 + pair * 32;
    const int key = kw0 + l32;  // this lane's key column

    // B operand of this wave's first product: K^T (P wave) or V^T (dS wave);
    // lane owns key `key`, d-run of half h.
    frag bf[C::NSD];
    if (key < Sk)
        load_run<T, C::NSD>(bf, (role ? v : k) + (size_t)key * D + h * (D / 2));
    else
        zero_run<T, C::NSD>(bf);
    // The dS wave keeps V^T negated: its dP products start from D and yield
    // D - dP, so dS = P o (dP - D) comes out negated with one multiply per
    // element (the accumulated -dK^T is negated back at the store).
    if (role) neg_run<T, C::NSD>(bf);
    TransReader<T, D> tr;
    tr.init(lane);

    f32x16 acc[C::ND];  // dV^T (P wave) or -dK^T (dS wave)
#pragma unroll
    for (int db = 0; db < C::ND; ++db) acc[db] = f32x16{};

    const int nq2 = (S + BQ2 - 1) / BQ2;
    // first query tile that sees key k0 (none at all: i0 = nq2, one empty step)
    const int i0 = !causal ? 0
                   : GEN   ? __builtin_amdgcn_readfirstlane(min(max(0, k0 - off) / BQ2, nq2))
                           : k0 / BQ2;
    const int ntile = nq2 - i0;

    typename C::DMA dma;
    dma.init(lane, pair);
    typedef __attribute__((address_space(3))) void lds_void;
    // Q (P waves) or dO (dS waves) rows, and L (P waves) or D (dS waves) of
    // query tile `it` (rows past the end are out of range and land as zeros;
    // the statistics of those rows repeat the last row's; all are masked)
    auto issue = [&](T *nQ, T *ndO, int it) {
        T *dst = role ? ndO : nQ;
        dma.issue(dst, role ? dout : q, it * BQ2, S, pair);
        // slot j holds the query a lane half reads as registers 8u..8u+7 of its
        // 32-query block: slot 16u + 8h + 4rr + e <-> query ridx(8u + 4rr + e, h),
        // so each half reads two runs of 8 slots
        const int jq = 32 * (lane >> 5) + 16 * ((lane >> 4) & 1) + 4 * (lane & 3) +
                       2 * ((lane >> 3) & 1) + ((lane >> 2) & 1);
        const int qi = min(it * BQ2 + jq, S - 1);
        __builtin_amdgcn_global_load_lds((const void *)((role ? delta : lse) + qi),
                                         (lds_void *)(dst + C::XOFF + pair * kWave * 4 / (int)sizeof(T)), 4, 0, 0);
    };
    // this wave's per-query statistic (L from a Q tile, D from a dO tile)
    // for registers r of block qb (the tile is named directly in each role
    // so the compiler knows which DMA target the read depends on)
    auto stat = [&](float (&x)[16], const T *tile, int qb, float mul) {
        const float *wX = reinterpret_cast<const float *>(tile + C::XOFF) + pair * kWave;
#pragma unroll
        for (int hr = 0; hr < 2; ++hr) {
            const int base = qb * 32 + 16 * hr + 8 * h;
            const f32x4 a = *reinterpret_cast<const f32x4 *>(wX + base);
            const f32x4 b = *reinterpret_cast<const f32x4 *>(wX + base + 4);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                x[8 * hr + t] = a[t] * mul;
                x[8 * hr + 4 + t] = b[t] * mul;
            }
        }
    };
    issue(sQ0, sdO0, i0);
    // Step 0 has no tile before it: its "previous" stages get an empty range
    // (the DMA lands zeros) and the P buffer it reads is cleared, so the
    // lagged products of step 0 add exact zeros.  Every step then runs the
    // same straight-line code (tiles a pair does not need are masked to P = 0),
    // which lets the compiler interleave each wave's matrix and vector work.
    issue(sQ2, sdO2, nq2);
    {
        typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
        u32x4 *z = reinterpret_cast<u32x4 *>(sP);
        for (int i = tid; i < 2 * C::PBUF * (int)sizeof(T) / 16; i += C::NT) z[i] = u32x4{0u, 0u, 0u, 0u};
    }
    wait_lgkm0();

    // Step u (query tile it = i0 + u): stage tQ holds Q of tile it, pQ/pdO
    // hold tile it-1; nQ/ndO receive tile it+1 (the stages of tile it-2).
    auto step = [&](const T *tQ, const T *pQ, const T *pdO, T *nQ, T *ndO, int u) {
        const int it = i0 + u;
        const int q0 = it * BQ2;
        wait_vmcnt<0>();  // this wave's part of tile it has landed
        lds_barrier();    // every part of it; P of tile it-1 is written; the stages of tile it-2 are free
        // Tile it+1 is issued whole and unconditionally (see the forward
        // kernel); past the last tile its range is empty.
        issue(nQ, ndO, it + 1);
        T *pw = sP + (u & 1) * C::PBUF + pair * C::NQ2 * C::PBLK + lane * C::KPL;        // P of tile it
        const T *pr = sP + ((u + 1) & 1) * C::PBUF + pair * C::NQ2 * C::PBLK + lane * C::KPL;  // P of it-1
        if (role == 0) {
            // dV^T += dO^T P for tile it-1 (P read back from the buffer this
            // wave wrote in the previous step), and S, P of tile it
            frag pp[C::NQ2][C::NI];
#pragma unroll
            for (int qb = 0; qb < C::NQ2; ++qb)
#pragma unroll
                for (int i = 0; i < C::NI; ++i) pp[qb][i] = *reinterpret_cast<const frag *>(pr + qb * C::PBLK + i * (kWave * C::KPL));
            f32x16 s[C::NQ2];
#pragma unroll
            for (int qb = 0; qb < C::NQ2; ++qb) {
                // S block: rows = queries q0 + 32*qb + ridx(r, h), col = key.
                s[qb] = f32x16{};
                frag qa[C::NSD];
                load_row_frags<T, D>(qa, tQ, qb * 32 + rsigma(l32), h);
#pragma unroll
                for (int st = 0; st < C::NSD; ++st) s[qb] = M::run(qa[st], bf[st], s[qb]);
            }
#pragma unroll
            for (int qb = 0; qb < C::NQ2; ++qb) {
                float lv[16];
                stat(lv, tQ, qb, GEN ? kLog2e : 1.f);  // (self-attention: already base 2)
#pragma unroll
                for (int r = 0; r < 16; ++r) s[qb][r] = fast_exp2(fmaf(s[qb][r], c, -lv[r]));  // Eq. 14
            }
#pragma unroll
            for (int qb = 0; qb < C::NQ2; ++qb)
#pragma unroll
                for (int db = 0; db < C::ND; ++db) {
                    frag a[C::NI];
                    tr.load(a, pdO, qb, db);
#pragma unroll
                    for (int i = 0; i < C::NI; ++i) acc[db] = M::run(a[i], pp[qb][i], acc[db]);  // Eq. 15
                }
            const bool need_mask = (causal && kw0 + 31 > q0 + off) || (q0 + BQ2 > S);
            if (need_mask) {
                asm volatile("");  // a real branch: only diagonal / tail tiles pay for masking
                // query q0 + 32*qb + ridx(r, h) is kept iff it is at least `lo` and below `hi`
#pragma unroll
                for (int qb = 0; qb < C::NQ2; ++qb) {
                    const int lo = (causal ? key - off : 0) - q0 - 32 * qb - 2 * h;
                    const int hi = S - q0 - 32 * qb - 2 * h;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int e = ridx(r, 0);
                        s[qb][r] = (e >= lo && e < hi) ? s[qb][r] : 0.f;
                    }
                }
            }
            // hand P to the partner (same lane layout on both sides)
#pragma unroll
            for (int qb = 0; qb < C::NQ2; ++qb) {
                frag pf[C::NI];
                to_bfrag<T>(pf, s[qb]);
#pragma unroll
                for (int i = 0; i < C::NI; ++i) *reinterpret_cast<frag *>(pw + qb * C::PBLK + i * (kWave * C::KPL)) = pf[i];
            }
        } else {
            // tile it-1: dP = dO V^T, dS = P o (dP - D), dK^T += Q^T dS
            f32x16 dp[C::NQ2];  // D - dP (Eq. 16, with -V^T)
#pragma unroll
            for (int qb = 0; qb < C::NQ2; ++qb) {
                float dl[16];
                stat(dl, pdO, qb, 1.f);
#pragma unroll
                for (int r = 0; r < 16; ++r) dp[qb][r] = dl[r];
                frag da[C::NSD];
                load_row_frags<T, D>(da, pdO, qb * 32 + rsigma(l32), h);
#pragma unroll
                for (int st = 0; st < C::NSD; ++st) dp[qb] = M::run(da[st], bf[st], dp[qb]);
            }
#pragma unroll
            for (int qb = 0; qb < C::NQ2; ++qb) {
                frag pp[C::NI];
#pragma unroll
                for (int i = 0; i < C::NI; ++i) pp[i] = *reinterpret_cast<const frag *>(pr + qb * C::PBLK + i * (kWave * C::KPL));
                f32x16 ds;  // -dS (Eq. 17)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    float p;
                    if constexpr (C::KPL == 8)
                        p = (float)pp[r / 8][r % 8];
                    else
                        p = pp[r];
                    ds[r] = p * dp[qb][r];
                }
                frag sf[C::NI];
                to_bfrag<T>(sf, ds);
#pragma unroll
                for (int db = 0; db < C::ND; ++db) {
                    frag a[C::NI];
                    tr.load(a, pQ, qb, db);
#pragma unroll
                    for (int i = 0; i < C::NI; ++i) acc[db] = M::run(a[i], sf[i], acc[db]);  // Eq. 19
                }
            }
        }
        wait_lgkm0();  // this wave's reads of the stages and of P are complete
    };
    // steps 0 .. ntile: step u finishes tile it-1 and starts tile it
    for (int u = 0; u <= ntile; u += 3) {
        step(sQ0, sQ2, sdO2, sQ1, sdO1, u);
        if (u + 1 <= ntile) step(sQ1, sQ0, sdO0, sQ2, sdO2, u + 1);
        if (u + 2 <= ntile) step(sQ2, sQ1, sdO1, sQ0, sdO0, u + 2);
    }
    wait_vmcnt<0>();

    if (key < Sk) {
        OutT *out = role ? dk : dv;
        const float mul = role ? -a.scale : 1.f;
#pragma unroll
        for (int db = 0; db < C::ND; ++db)
#pragma unroll
            for (int hr = 0; hr < 2; ++hr) {
                const int d0 = db * 32 + 16 * hr + 8 * h;
                if (d0 < D) out8<GEN>(out + (size_t)key * D + d0, acc[db], 8 * hr, mul, a.accumulate);
            }
    }
}

// ----------------------------------------- key-outer dK/dV, one wave per key block ---
//
// The same pass with every 32-key block owned by a single wave that forms all
// four products of a 32-query tile itself: S = Q K^T and P = 2^(S c - L)
// (Eq. 13-14), dV^T += dO^T P (Eq. 15), D - dP = D - dO V^T (Eq. 16, V^T kept
// negated, the chain started from D), -dS = P o (D - dP) (Eq. 17) and
// -dK^T += Q^T (-dS) (Eq. 19).  P and dS go from the accumulator registers
// straight into the next products (no LDS hand-off, no bf16 round trip of P
// before dS), so the vector work per product is smaller than with pairs; the
// price is both K^T and V^T and both accumulators in registers, which the
// narrower head dimensions afford at two waves per SIMD.

template <typename T, int D_, int NW_, bool VLDS_ = false, int NQB_ = 1, int NSTAGE_ = 3, int VREG_ = 0>
struct KvTile1 {
    static constexpr int D = D_, NW = NW_, NT = NW * kWave;
    static constexpr int NQB = NQB_;                  // 32-query blocks per step
    // LDS stages of Q/dO tiles: 3 (two tiles in flight) or 2 (one)
    static constexpr int NSTAGE = NSTAGE_;
    // -V^T partly in LDS (written there once, read every step): the first
    // VREG fragments of a lane's run stay in registers, the other VL in LDS
    // (4 * KPL * VL / 8 fewer registers per lane, VL reads per block)
    static constexpr bool VLDS = VLDS_;
    static constexpr int BQ = 32 * NQB;               // queries per step
    static constexpr int BKV = NW * 32;               // keys per workgroup
    static constexpr int KPL = Mma<T>::KPL;
    static constexpr int NSD = D / 2 / KPL;
    static constexpr int VREG = VREG_, VL = NSD - VREG_;
    // LDS row of a key's -V^T part: both lane halves' VL fragments plus a
    // 16-byte pad (4 (mod 8) words, conflict-free like every tile)
    static constexpr int VPITCH = 2 * VL * KPL + 16 / (int)sizeof(T);
    // bf16 D = 16 (mod 32): the last 16 rows of dV^T, dK^T form a 16-row tail
    static constexpr bool TAIL = KPL == 8 && D % 32 == 16;
    static constexpr int ND = TAIL ? D / 32 : (D + 31) / 32;
    static constexpr int NI = 16 / KPL;
    using DMA = TileDma<T, D, BQ, NW / 2>;           // half the waves load Q, half dO
    // a Q (dO) tile array also carries the tile's L (D) values: 64 slots per
    // loading wave (every wave issues the same number of loads per tile)
    static constexpr int XOFF = DMA::ELEMS;
    static constexpr int TILE = DMA::ELEMS + (NW / 2) * kWave * 4 / (int)sizeof(T);
    static_assert(D % 16 == 0 && NW % 2 == 0 && (NQB == 1 || NQB == 2), "tile shape");
    static_assert(VREG >= 0 && VREG < NSD && (VLDS || VREG == 0), "-V^T split");
    static_assert(NSTAGE == 2 || NSTAGE == 3, "stages");
};

template <typename T, typename C, typename OutT, bool GEN>
__global__ __launch_bounds__(C::NT) void dkdv1_kernel(const T *__restrict__ q, const T *__restrict__ k,
                                                      const T *__restrict__ v, const T *__restrict__ dout,
                                                      const float *__restrict__ lse,
                                                      const float *__restrict__ delta, OutT *__restrict__ dk,
                                                      OutT *__restrict__ dv, BwdShape a) {
    using M = Mma<T>;
    using frag = typename M::frag;
    constexpr int D = C::D;
    // two or three stages of Q and dO tiles, each its own array (see the forward kernel)
    constexpr int T3 = C::NSTAGE == 3 ? C::TILE : 8;
    __shared__ __attribute__((aligned(1024))) T sQ0[C::TILE], sQ1[C::TILE], sQ2[T3];
    __shared__ __attribute__((aligned(1024))) T sdO0[C::TILE], sdO1[C::TILE], sdO2[T3];
    __shared__ __attribute__((aligned(16))) T sV[C::VLDS ? C::BKV * C::VPITCH : 8];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, l32 = lane & 31;
    const int BH = a.BH, Sh = a.Sq, causal = a.causal;
    // this launch's queries: chunk blockIdx.y of the head's query rows
    // (uniform values kept in scalar registers, see the forward kernel)
    const int qbeg = GEN ? blockIdx.y * a.qchunk : 0;
    const int S = GEN ? __builtin_amdgcn_readfirstlane(min(a.qchunk, Sh - qbeg)) : Sh;
    const int Sk = GEN ? a.Sk : Sh;
    const int off = GEN ? __builtin_amdgcn_readfirstlane(a.off + qbeg) : 0;
    const float c = a.c;
    const int bid = blockIdx.x;
    // ascending key tiles: the tiles with the most query tiles go first (tile_order)
    int kt, bh;
    tile_order(bid, BH, (Sk + C::BKV - 1) / C::BKV, a.band, kt, bh);
    q += ((size_t)bh * Sh + qbeg) * D;
    dout += ((size_t)bh * Sh + qbeg) * D;
    k += (size_t)bh * Sk * D;
    v += (size_t)bh * Sk * D;
    const size_t part = GEN ? (size_t)blockIdx.y * BH * Sk * D : 0;
    dk += part + (size_t)bh * Sk * D;
    dv += part + (size_t)bh * Sk * D;
    lse += (size_t)bh * Sh + qbeg;
    delta += (size_t)bh * Sh + qbeg;
    const int k0 = kt * C::BKV;
    const int kw0 = k0 + wave * 32;
    const int key = kw0 + l32;  // this lane's key column

    // B operands: K^T and -V^T (the dP chain then yields D - dP)
    frag bk[C::NSD], bv[C::VLDS ? (C::VREG > 0 ? C::VREG : 1) : C::NSD];
    // this lane's -V^T run in LDS (its own row: no other wave reads it)
    T *const sVl = sV + (C::VLDS ? (wave * 32 + l32) * C::VPITCH + h * C::VL * C::KPL : 0);
    if (key < Sk) {
        load_run<T, C::NSD>(bk, k + (size_t)key * D + h * (D / 2));
    } else {
        zero_run<T, C::NSD>(bk);
    }
    {
        frag vt0[C::NSD];
        if (key < Sk)
            load_run<T, C::NSD>(vt0, v + (size_t)key * D + h * (D / 2));
        else
            zero_run<T, C::NSD>(vt0);
        neg_run<T, C::NSD>(vt0);
        if constexpr (C::VLDS) {
#pragma unroll
            for (int i = 0; i < C::NSD; ++i) {
                if (i < C::VREG) bv[i < C::VREG ? i : 0] = vt0[i];  // (index kept in range for the compiler)
                else *reinterpret_cast<frag *>(sVl + (i - C::VREG) * C::KPL) = vt0[i];
            }
        } else {
#pragma unroll
            for (int i = 0; i < C::NSD; ++i) bv[i] = vt0[i];
        }
    }
    TransReader<T, D> tr;
    tr.init(lane);
    TailReader<D> tt;  // (16-row tail only)
    if constexpr (C::TAIL) tt.init(lane);

    f32x16 accV[C::ND > 0 ? C::ND : 1], accK[C::ND > 0 ? C::ND : 1];  // dV^T and -dK^T
    f32x4 tailV[2] = {f32x4{}, f32x4{}}, tailK[2] = {f32x4{}, f32x4{}};  // 16-row tails: keys 0..15, 16..31
#pragma unroll
    for (int db = 0; db < C::ND; ++db) {
        accV[db] = f32x16{};
        accK[db] = f32x16{};
    }

    const int nq = (S + C::BQ - 1) / C::BQ;
    const int i0 = !causal ? 0
                   : GEN   ? __builtin_amdgcn_readfirstlane(min(max(0, k0 - off) / C::BQ, nq))
                           : k0 / C::BQ;

    typename C::DMA dma;
    const int half = wave / (C::NW / 2), hw = wave % (C::NW / 2);
    dma.init(lane, hw);
    typedef __attribute__((address_space(3))) void lds_void;
    // slot j of a wave's statistics holds the query that a lane half reads as
    // registers of its 32-query block: slot 32b + 16u + 8h + 4rr + e <->
    // query 32b + ridx(8u + 4rr + e, h) (with one block per tile, lanes
    // 32..63 repeat lanes 0..31)
    const int jq = (C::NQB > 1 ? 32 * (lane >> 5) : 0) + 16 * ((lane >> 4) & 1) + 4 * (lane & 3) +
                   2 * ((lane >> 3) & 1) + ((lane >> 2) & 1);
    auto issue = [&](T *nQ, T *ndO, int it) {
        T *dst = half ? ndO : nQ;
        dma.issue(dst, half ? dout : q, it * C::BQ, S, hw);
        const int qi = min(it * C::BQ + jq, S - 1);
        __builtin_amdgcn_global_load_lds((const void *)((half ? delta : lse) + qi),
                                         (lds_void *)(dst + C::XOFF + hw * kWave * 4 / (int)sizeof(T)), 4, 0, 0);
    };
    // this wave's L (from a Q tile) or D (from a dO tile) for its 16 rows of block qb
    auto stat = [&](float (&x)[16], const T *tile, int qb, float mul) {
        const float *wX = reinterpret_cast<const float *>(tile + C::XOFF) + hw * kWave;
#pragma unroll
        for (int hr = 0; hr < 2; ++hr) {
            const int base = 32 * qb + 16 * hr + 8 * h;
            const f32x4 p0 = *reinterpret_cast<const f32x4 *>(wX + base);
            const f32x4 p1 = *reinterpret_cast<const f32x4 *>(wX + base + 4);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                x[8 * hr + t] = p0[t] * mul;
                x[8 * hr + 4 + t] = p1[t] * mul;
            }
        }
    };
    issue(sQ0, sdO0, i0);
    if constexpr (C::NSTAGE == 3) issue(sQ1, sdO1, i0 + 1);

    auto step = [&](const T *tQ, const T *tdO, T *nQ, T *ndO, int it) {
        const int q0 = it * C::BQ;
        if constexpr (C::NSTAGE == 3) {
            wait_vmcnt<C::DMA::IPW + 1>();  // this wave's part of tile it has landed (it+1 may be in flight)
            lds_barrier();                  // every part of it; the stage of tile it-1 is released
            issue(nQ, ndO, it + 2);         // unconditionally (see the forward kernel)
        } else {
            wait_vmcnt<0>();  // this wave's part of tile it has landed
            lds_barrier();    // every part of it; the other stage (tile it-1) is released
            issue(nQ, ndO, it + 1);
        }
        // one 32-query block: queries q0 + 32*qb + ridx(r, h)
        auto block = [&](int qb) {
            const int qb0 = q0 + 32 * qb;
            if (causal && kw0 > qb0 + 31 + off) return;  // no key of this wave is visible yet
            // S block: rows = queries qb0 + ridx(r, h), col = key; P = 2^(S c - L)
            f32x16 s = f32x16{};
            {
                frag qa[C::NSD];
                load_row_frags<T, D>(qa, tQ, 32 * qb + rsigma(l32), h);
#pragma unroll
                for (int st = 0; st < C::NSD; ++st) s = M::run(qa[st], bk[st], s);
            }
            // D - dP (Eq. 16).  Up to D = 96 its products are issued before the
            // exponentials, which then run while they execute (0.7 % faster at
            // D = 80); at D = 128 holding S and dP together spills.
            f32x16 dp;
            auto form_dp = [&]() {
                {
                    float dl[16];
                    stat(dl, tdO, qb, 1.f);
#pragma unroll
                    for (int r = 0; r < 16; ++r) dp[r] = dl[r];
                    frag da[C::NSD];
                    load_row_frags<T, D>(da, tdO, 32 * qb + rsigma(l32), h);
                    if constexpr (C::VLDS) {
                        frag bvl[C::VL];
                        load_run<T, C::VL>(bvl, sVl);
#pragma unroll
                        for (int st = 0; st < C::NSD; ++st)
                            dp = M::run(da[st], st < C::VREG ? bv[st < C::VREG ? st : 0] : bvl[st < C::VREG ? 0 : st - C::VREG], dp);
                    } else {
#pragma unroll
                        for (int st = 0; st < C::NSD; ++st) dp = M::run(da[st], bv[st], dp);
                    }
                }
            };
            if constexpr (C::D <= 96) form_dp();
            {
                float lv[16];
                stat(lv, tQ, qb, GEN ? kLog2e : 1.f);  // (self-attention: already base 2)
#pragma unroll
                for (int r = 0; r < 16; ++r) s[r] = fast_exp2(fmaf(s[r], c, -lv[r]));  // Eq. 14
            }
            const bool need_mask = (causal && kw0 + 31 > qb0 + off) || (qb0 + 32 > S);
            if (need_mask) {
                asm volatile("");  // a real branch: only diagonal / tail tiles pay for masking
                // query qb0 + ridx(r, h) is kept iff it is at least `lo` and below `hi`
                const int lo = (causal ? key - off : 0) - qb0 - 2 * h;
                const int hi = S - qb0 - 2 * h;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int e = ridx(r, 0);
                    s[r] = (e >= lo && e < hi) ? s[r] : 0.f;
                }
            }
            // dV^T += dO^T P (Eq. 15)
            {
                frag pf[C::NI];
                to_bfrag<T>(pf, s);
#pragma unroll
                for (int db = 0; db < C::ND; ++db) {
                    frag at[C::NI];
                    tr.load(at, tdO, qb, db);
#pragma unroll
                    for (int i = 0; i < C::NI; ++i) accV[db] = M::run(at[i], pf[i], accV[db]);
                }
                if constexpr (C::TAIL) {
                    bf16x8 b0, b1;
                    tail_bfrag(pf, b0, b1);
                    const bf16x8 ta = tt.load(tdO, qb, 32 * C::ND);
                    tailV[0] = mma16(ta, b0, tailV[0]);
                    tailV[1] = mma16(ta, b1, tailV[1]);
                }
            }
            if constexpr (C::D > 96) form_dp();
            // -dS = P o (D - dP) (Eq. 17)
#pragma unroll
            for (int r = 0; r < 16; ++r) dp[r] *= s[r];
            // -dK^T += Q^T (-dS) (Eq. 19)
            {
                frag sf[C::NI];
                to_bfrag<T>(sf, dp);
#pragma unroll
                for (int db = 0; db < C::ND; ++db) {
                    frag at[C::NI];
                    tr.load(at, tQ, qb, db);
#pragma unroll
                    for (int i = 0; i < C::NI; ++i) accK[db] = M::run(at[i], sf[i], accK[db]);
                }
                if constexpr (C::TAIL) {
                    bf16x8 b0, b1;
                    tail_bfrag(sf, b0, b1);
                    const bf16x8 ta = tt.load(tQ, qb, 32 * C::ND);
                    tailK[0] = mma16(ta, b0, tailK[0]);
                    tailK[1] = mma16(ta, b1, tailK[1]);
                }
            }
        };
#pragma unroll
        for (int qb = 0; qb < C::NQB; ++qb) block(qb);
        wait_lgkm0();  // this wave's reads of the stage are complete before the next barrier
    };
    if constexpr (C::NSTAGE == 3) {
        for (int it = i0; it < nq; it += 3) {
            step(sQ0, sdO0, sQ2, sdO2, it);
            if (it + 1 < nq) step(sQ1, sdO1, sQ0, sdO0, it + 1);
            if (it + 2 < nq) step(sQ2, sdO2, sQ1, sdO1, it + 2);
        }
    } else {
        for (int it = i0; it < nq; it += 2) {
            step(sQ0, sdO0, sQ1, sdO1, it);
            if (it + 1 < nq) step(sQ1, sdO1, sQ0, sdO0, it + 1);
        }
    }
    wait_vmcnt<0>();  // no DMA may still be writing this workgroup's LDS when it exits

    if (key < Sk) {
#pragma unroll
        for (int db = 0; db < C::ND; ++db)
#pragma unroll
            for (int hr = 0; hr < 2; ++hr) {
                const int d0 = db * 32 + 16 * hr + 8 * h;
                if (d0 < D) {
                    out8<GEN>(dv + (size_t)key * D + d0, accV[db], 8 * hr, 1.f, a.accumulate);
                    out8<GEN>(dk + (size_t)key * D + d0, accK[db], 8 * hr, -a.scale, a.accumulate);
                }
            }
    }
    if constexpr (C::TAIL) {
        // tail lane 16g + i holds rows 4g..4g+3 of the wave's keys i and 16 + i
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int kt_ = kw0 + 16 * t + (lane & 15);
            const int d0 = 32 * C::ND + 4 * (lane >> 4);
            if (kt_ < Sk) {
                out4<GEN>(dv + (size_t)kt_ * D + d0, tailV[t], 1.f, a.accumulate);
                out4<GEN>(dk + (size_t)kt_ * D + d0, tailK[t], -a.scale, a.accumulate);
            }
        }
    }
}

// -------------------------------------------------------- query-outer dQ ---

template <typename T, int D_, int NQB_, int BK_, int NW_>
struct QTile {
    static constexpr int D = D_, NQB = NQB_, BK = BK_;
    static constexpr int NW = NW_, NT = NW * kWave;
    static constexpr int BQ = NW * NQB * 32;
    static constexpr int KPL = Mma<T>::KPL;
    static constexpr int NSD = D / 2 / KPL;
    static constexpr int NKB = BK / 32;
    // bf16 D = 16 (mod 32): the last 16 rows of dQ^T form a 16-row tail
    static constexpr bool TAIL = KPL == 8 && D % 32 == 16;
    static constexpr int ND = TAIL ? D / 32 : (D + 31) / 32;
    static constexpr int NI = 16 / KPL;
    using DMA = TileDma<T, D, BK, NW / 2>;           // half the waves load K, half V
    static constexpr int TILE = DMA::ELEMS;           // elements per K or V tile
    static_assert(D % 16 == 0 && BK % 32 == 0 && NW % 2 == 0, "tile shape");
};

template <typename T, typename C, typename OutT, bool GEN>
__global__ __launch_bounds__(C::NT) void dq_kernel(const T *__restrict__ q, const T *__restrict__ k,
                                                   const T *__restrict__ v, const T *__restrict__ dout,
                                                   const float *__restrict__ lse,
                                                   const float *__restrict__ delta, OutT *__restrict__ dq,
                                                   BwdShape a) {
    using M = Mma<T>;
    using frag = typename M::frag;
    constexpr int D = C::D, NQB = C::NQB, BK = C::BK;
    // three stages of K and V tiles, each its own array (see the forward kernel)
    __shared__ __attribute__((aligned(1024))) T sK0[C::TILE], sK1[C::TILE], sK2[C::TILE];
    __shared__ __attribute__((aligned(1024))) T sV0[C::TILE], sV1[C::TILE], sV2[C::TILE];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5, l32 = lane & 31;
    const int BH = a.BH, S = a.Sq, causal = a.causal;
    // this launch's keys: chunk blockIdx.y of the head's key rows
    const int kbeg = GEN ? blockIdx.y * a.kchunk : 0;
    const int Skh = GEN ? a.Sk : S;  // keys per head (queries: S)
    const int Sk = GEN ? __builtin_amdgcn_readfirstlane(min(a.kchunk, Skh - kbeg)) : S;
    // query i sits off positions after key 0 of this launch
    const int off = GEN ? __builtin_amdgcn_readfirstlane(a.off - kbeg) : 0;
    const float c = a.c;
    const int bid = blockIdx.x;
    int rank, bh;  // longest query tile first (tile_order)
    tile_order(bid, BH, a.nqt, a.band, rank, bh);
    const int qt = causal ? a.nqt - 1 - rank : rank;
    q += (size_t)bh * S * D;
    dout += (size_t)bh * S * D;
    dq += (GEN ? (size_t)blockIdx.y * BH * S * D : 0) + (size_t)bh * S * D;
    k += ((size_t)bh * Skh + kbeg) * D;
    v += ((size_t)bh * Skh + kbeg) * D;
    lse += (size_t)bh * S;
    delta += (size_t)bh * S;
    const int q0 = qt * C::BQ;
    const int qw0 = q0 + wave * NQB * 32;

    // Q^T, dO^T fragments (B operands) and the row statistics of this lane's query.
    frag qf[NQB][C::NSD], df[NQB][C::NSD];
    float lq[NQB], dl[NQB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        const int qi = qw0 + qb * 32 + l32;
        if (qi < S) {
            load_run<T, C::NSD>(qf[qb], q + (size_t)qi * D + h * (D / 2));
            load_run<T, C::NSD>(df[qb], dout + (size_t)qi * D + h * (D / 2));
            lq[qb] = GEN ? lse[qi] * kLog2e : lse[qi];  // (self-attention: already base 2)
            // a row without probability mass (L = -inf) gives P = 0
            if (GEN && lq[qb] == -INFINITY) lq[qb] = INFINITY;
            dl[qb] = delta[qi];
        } else {
            zero_run<T, C::NSD>(qf[qb]);
            zero_run<T, C::NSD>(df[qb]);
            lq[qb] = 0.f;
            dl[qb] = 0.f;
        }
    }
    // dO^T is kept negated: the dP^T products then start from D and yield
    // D - dP^T, so dS^T = P o (dP^T - D) comes out negated with one multiply
    // per element (the accumulated -dQ^T is negated back at the store).
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) neg_run<T, C::NSD>(df[qb]);
    TransReader<T, D> tr;
    tr.init(lane);
    TailReader<D> tt;  // (16-row tail only)
    if constexpr (C::TAIL) tt.init(lane);

    f32x16 acc[NQB][C::ND > 0 ? C::ND : 1];
    f32x4 tacc[NQB][2];  // 16-row tail: queries 0..15 and 16..31 of the block
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
#pragma unroll
        for (int db = 0; db < C::ND; ++db) acc[qb][db] = f32x16{};
        tacc[qb][0] = f32x4{};
        tacc[qb][1] = f32x4{};
    }

    const int qend = min(q0 + C::BQ, S);
    int nkt = (Sk + BK - 1) / BK;
    if (causal) {
        const int last = qend - 1 + off;  // last key any query of the tile sees
        nkt = last < 0 ? 0 : min(nkt, last / BK + 1);
    }

    typename C::DMA dma;
    const int half = wave / (C::NW / 2), hw = wave % (C::NW / 2);
    dma.init(lane, hw);
    auto issue = [&](T *nK, T *nV, int j) { dma.issue(half ? nV : nK, half ? v : k, j * BK, Sk, hw); };
    issue(sK0, sV0, 0);
    issue(sK1, sV1, 1);
    // bf16 up to D = 96: the tile's products are issued block-phased (registers
    // allow holding both blocks' S^T and dP^T).  Backward, interleaved A/B with
    // replicate builds: D = 16 and 32 -1.8 %, D = 64 -1.6 %, D = 96 -1.0 %;
    // D = 80 measured 0.3 % slower and keeps one block at a time.
    constexpr bool kPhased = C::KPL == 8 && C::D <= 96 && C::D != 80 && NQB == 1;
    // bf16 D = 128 (no registers for two score blocks and two dP blocks): only
    // block 1's S^T goes out early.  Backward 1.0-1.3 % faster at S = 65536 and
    // 0.3 % at S = 16384 (replicate builds, interleaved); 0.7 % slower at D = 80.
    constexpr bool kHalfPhased = C::KPL == 8 && C::D == 128 && NQB == 1 && C::NKB == 2;

    auto step = [&](const T *tK, const T *tV, T *nK, T *nV, int j) {
        const int j0 = j * BK;
        wait_vmcnt<C::DMA::IPW>();
        lds_barrier();
        // prefetch of tile j+2, unconditional and spread over the key blocks
        // (see the forward kernel)
        const auto rs = C::DMA::range(half ? v : k, (j + 2) * BK, Sk);
        T *const nT = half ? nV : nK;
        const bool active = qw0 < S && !(causal && j0 > qw0 + NQB * 32 - 1 + off);
        if (!active) {
            dma.issue(nT, half ? v : k, (j + 2) * BK, Sk, hw);
        } else if constexpr (kPhased) {
            // All S^T and dP^T products of the tile first, then each block's
            // exponentials, -dS^T and dQ^T products: a block's vector work runs
            // while the wave's other products execute.
            const bool need_mask = (causal && j0 + BK - 1 > qw0 + off) || (j0 + BK > Sk);
            f32x16 s[C::NKB], dp[C::NKB];
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb) {
                dma.issue_part(kb, C::NKB, nT, rs, hw);
                s[kb] = f32x16{};
#pragma unroll
                for (int r = 0; r < 16; ++r) dp[kb][r] = dl[0];
                {
                    frag ka[C::NSD];
                    load_row_frags<T, D>(ka, tK, kb * 32 + rsigma(l32), h);
#pragma unroll
                    for (int st = 0; st < C::NSD; ++st) s[kb] = M::run(ka[st], qf[0][st], s[kb]);
                }
                {
                    frag va[C::NSD];
                    load_row_frags<T, D>(va, tV, kb * 32 + rsigma(l32), h);
#pragma unroll
                    for (int st = 0; st < C::NSD; ++st) dp[kb] = M::run(va[st], df[0][st], dp[kb]);
                }
            }
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) s[kb][r] = fast_exp2(fmaf(s[kb][r], c, -lq[0]));  // Eq. 14
            if (need_mask) {
                asm volatile("");  // a real branch: only diagonal / tail tiles pay for masking
                const int qi = qw0 + l32;
#pragma unroll
                for (int kb = 0; kb < C::NKB; ++kb) {
                    const int t = (causal ? min(qi + 1 + off, Sk) : Sk) - j0 - 32 * kb - 2 * h;
#pragma unroll
                    for (int r = 0; r < 16; ++r) s[kb][r] = (ridx(r, 0) < t) ? s[kb][r] : 0.f;
                }
            }
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) dp[kb][r] = s[kb][r] * dp[kb][r];  // -dS^T (Eq. 17)
                frag sf[C::NI];
                to_bfrag<T>(sf, dp[kb]);
#pragma unroll
                for (int db = 0; db < C::ND; ++db) {
                    frag a[C::NI];
                    tr.load(a, tK, kb, db);
#pragma unroll
                    for (int i = 0; i < C::NI; ++i) acc[0][db] = M::run(a[i], sf[i], acc[0][db]);  // Eq. 18
                }
                if constexpr (C::TAIL) {
                    bf16x8 b0, b1;
                    tail_bfrag(sf, b0, b1);
                    const bf16x8 ta = tt.load(tK, kb, 32 * C::ND);
                    tacc[0][0] = mma16(ta, b0, tacc[0][0]);
                    tacc[0][1] = mma16(ta, b1, tacc[0][1]);
                }
            }
        } else if constexpr (kHalfPhased) {
            // Block 1's S^T products go out before block 0's exponentials, -dS^T
            // and dQ^T products (and its dP^T products after them), so those run
            // while block 1's scores are formed; holds one more score block.
            const bool need_mask = (causal && j0 + BK - 1 > qw0 + off) || (j0 + BK > Sk);
            const int qi = qw0 + l32;
            f32x16 s[2], dp[2];
            auto s_prod = [&](int kb) {
                s[kb] = f32x16{};
                frag ka[C::NSD];
                load_row_frags<T, D>(ka, tK, kb * 32 + rsigma(l32), h);
#pragma unroll
                for (int st = 0; st < C::NSD; ++st) s[kb] = M::run(ka[st], qf[0][st], s[kb]);
            };
            auto dp_prod = [&](int kb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) dp[kb][r] = dl[0];
                frag va[C::NSD];
                load_row_frags<T, D>(va, tV, kb * 32 + rsigma(l32), h);
#pragma unroll
                for (int st = 0; st < C::NSD; ++st) dp[kb] = M::run(va[st], df[0][st], dp[kb]);
            };
            auto rest = [&](int kb) {
#pragma unroll
                for (int r = 0; r < 16; ++r) s[kb][r] = fast_exp2(fmaf(s[kb][r], c, -lq[0]));  // Eq. 14
                if (need_mask) {
                    asm volatile("");  // a real branch: only diagonal / tail tiles pay for masking
                    const int t = (causal ? min(qi + 1 + off, Sk) : Sk) - j0 - 32 * kb - 2 * h;
#pragma unroll
                    for (int r = 0; r < 16; ++r) s[kb][r] = (ridx(r, 0) < t) ? s[kb][r] : 0.f;
                }
#pragma unroll
                for (int r = 0; r < 16; ++r) dp[kb][r] = s[kb][r] * dp[kb][r];  // -dS^T (Eq. 17)
                frag sf[C::NI];
                to_bfrag<T>(sf, dp[kb]);
#pragma unroll
                for (int db = 0; db < C::ND; ++db) {
                    frag a[C::NI];
                    tr.load(a, tK, kb, db);
#pragma unroll
                    for (int i = 0; i < C::NI; ++i) acc[0][db] = M::run(a[i], sf[i], acc[0][db]);  // Eq. 18
                }
                if constexpr (C::TAIL) {
                    bf16x8 b0, b1;
                    tail_bfrag(sf, b0, b1);
                    const bf16x8 ta = tt.load(tK, kb, 32 * C::ND);
                    tacc[0][0] = mma16(ta, b0, tacc[0][0]);
                    tacc[0][1] = mma16(ta, b1, tacc[0][1]);
                }
            };
            static_assert(C::NKB == 2, "two key blocks per tile");
            __builtin_amdgcn_sched_barrier(0);
            dma.issue_part(0, C::NKB, nT, rs, hw);
            s_prod(0);
            __builtin_amdgcn_sched_barrier(0);
            dp_prod(0);
            __builtin_amdgcn_sched_barrier(0);
            dma.issue_part(1, C::NKB, nT, rs, hw);
            s_prod(1);
            rest(0);
            __builtin_amdgcn_sched_barrier(0);
            dp_prod(1);
            rest(1);
        } else {
            const bool need_mask = (causal && j0 + BK - 1 > qw0 + off) || (j0 + BK > Sk);
#pragma unroll
            for (int kb = 0; kb < C::NKB; ++kb) {
                __builtin_amdgcn_sched_barrier(0);
                dma.issue_part(kb, C::NKB, nT, rs, hw);
#pragma unroll
                for (int qb = 0; qb < NQB; ++qb) {
                    // S^T block: rows = keys j0 + 32*kb + ridx(r, h), col = query.
                    // (K and V fragments are not live at the same time: keeps two
                    // waves' worth of registers per SIMD)
                    f32x16 s = f32x16{}, dp;
#pragma unroll
                    for (int r = 0; r < 16; ++r) dp[r] = dl[qb];
                    {
                        frag ka[C::NSD];
                        load_row_frags<T, D>(ka, tK, kb * 32 + rsigma(l32), h);
#pragma unroll
                        for (int st = 0; st < C::NSD; ++st) s = M::run(ka[st], qf[qb][st], s);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    {
                        frag va[C::NSD];
                        load_row_frags<T, D>(va, tV, kb * 32 + rsigma(l32), h);
#pragma unroll
                        for (int st = 0; st < C::NSD; ++st) dp = M::run(va[st], df[qb][st], dp);
                    }
                    const int qi = qw0 + qb * 32 + l32;
                    const int t = (causal ? min(qi + 1 + off, Sk) : Sk) - j0 - 32 * kb - 2 * h;
#pragma unroll
                    for (int r = 0; r < 16; ++r) s[r] = fast_exp2(fmaf(s[r], c, -lq[qb]));  // Eq. 14
                    if (need_mask) {
                        asm volatile("");  // a real branch: only diagonal / tail tiles pay for masking
#pragma unroll
                        for (int r = 0; r < 16; ++r) s[r] = (ridx(r, 0) < t) ? s[r] : 0.f;
                    }
#pragma unroll
                    for (int r = 0; r < 16; ++r) dp[r] = s[r] * dp[r];  // -dS^T (Eq. 17)
                    frag sf[C::NI];
                    to_bfrag<T>(sf, dp);
#pragma unroll
                    for (int db = 0; db < C::ND; ++db) {
                        frag a[C::NI];
                        tr.load(a, tK, kb, db);
#pragma unroll
                        for (int i = 0; i < C::NI; ++i) acc[qb][db] = M::run(a[i], sf[i], acc[qb][db]);  // Eq. 18
                    }
                    if constexpr (C::TAIL) {
                        bf16x8 b0, b1;
                        tail_bfrag(sf, b0, b1);
                        const bf16x8 ta = tt.load(tK, kb, 32 * C::ND);
                        tacc[qb][0] = mma16(ta, b0, tacc[qb][0]);
                        tacc[qb][1] = mma16(ta, b1, tacc[qb][1]);
                    }
                }
            }
        }
        wait_lgkm0();
    };
    for (int j = 0; j < nkt; j += 3) {
        step(sK0, sV0, sK2, sV2, j);
        if (j + 1 < nkt) step(sK1, sV1, sK0, sV0, j + 1);
        if (j + 2 < nkt) step(sK2, sV2, sK1, sV1, j + 2);
    }
    wait_vmcnt<0>();

#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
        const int qi = qw0 + qb * 32 + l32;
        if (qi < S) {
#pragma unroll
            for (int db = 0; db < C::ND; ++db)
#pragma unroll
                for (int hr = 0; hr < 2; ++hr) {
                    const int d0 = db * 32 + 16 * hr + 8 * h;
                    if (d0 < D) out8<GEN>(dq + (size_t)qi * D + d0, acc[qb][db], 8 * hr, -a.scale, a.accumulate);
                }
        }
        if constexpr (C::TAIL) {
            // tail lane 16g + i holds rows 4g..4g+3 of queries i and 16 + i of the block
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int qt_ = qw0 + qb * 32 + 16 * t + (lane & 15);
                if (qt_ < S)
                    out4<GEN>(dq + (size_t)qt_ * D + 32 * C::ND + 4 * (lane >> 4), tacc[qb][t], -a.scale,
                              a.accumulate);
            }
        }
    }
}

// ---------------------------------------------- sum of partial results ---

// out_g = sum of n fp32 partial results `stride` elements apart, in a fixed
// order (so the split backward stays bit-reproducible), rounded to T; four
// elements per thread (count4 = elements / 4).  One launch for the three
// gradients: blockIdx.y = g selects out_g, whose partials start g*n*stride
// elements into `parts`.
template <typename T>
__global__ __launch_bounds__(256) void sum_parts_kernel(const float *__restrict__ parts, int n,
                                                        long long stride, T *__restrict__ out0,
                                                        T *__restrict__ out1, T *__restrict__ out2,
                                                        long long count4) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i >= count4) return;
    const int g = blockIdx.y;
    T *const out = g == 0 ? out0 : g == 1 ? out1 : out2;
    parts += (size_t)g * n * stride;
    f32x4 acc = *reinterpret_cast<const f32x4 *>(parts + 4 * i);
    for (int p = 1; p < n; ++p) acc += *reinterpret_cast<const f32x4 *>(parts + p * stride + 4 * i);
    store4<T>(out + 4 * i, acc, 1.f);
}

// ------------------------------------------------------------- launches ---

template <typename T, int D>
static int delta_for(const void *o, const void *dout, float *delta, int BH, int S, hipStream_t stream) {
    const long long rows = (long long)BH * S;
    const long long grid = (rows + 63) / 64;
    if (grid > 0x7fffffffLL) return -1;
    hipLaunchKernelGGL((delta_kernel<T, D>), dim3((unsigned)grid), dim3(256), 0, stream, (const T *)o,
                       (const T *)dout, delta, rows);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

// Tile shapes: fp32 rows are twice the bytes, so wider fp32 heads take
// shorter tiles to fit three stages in LDS.
template <typename T, int D>
using KvTileFor = KvTile<T, D, (sizeof(T) == 4 && D > 32) ? 32 : 64>;
// (fp32 D = 128: Q^T, -dO^T and the dQ^T accumulator take 64 registers each,
// so with two waves per SIMD the pass spilled 81 registers to scratch.  Four
// waves per workgroup, one per SIMD, spill them into the accumulation
// registers instead: the fp32 backward ran 25-33 % faster at D = 128, with
// bit-identical results (each query's sum over key tiles keeps its order).
// The same at D = 96 (7 spilled registers) was level.)
template <typename T, int D>
using QTileFor = QTile<T, D, 1, (sizeof(T) == 4 && D > 80) ? 32 : 64, (sizeof(T) == 4 && D == 128) ? 4 : 8>;
// (bf16 D = 128 keeps half of -V^T in LDS: with all of it in registers the
// kernel spills; half in registers (254 VGPRs) reads half as much LDS per
// block: the backward ran 1.3 % faster than with all of it in LDS.  Two 32-query blocks per
// step halve the barriers and DMA issues per product: 4-5 % faster up to
// D = 96; at D = 128 the LDS holds them beside -V^T only with two stages
// (1 % faster than one block with three).)
template <typename T, int D>
using KvTile1For = KvTile1<T, D, 8, sizeof(T) == 2 && D == 128, sizeof(T) == 2 ? 2 : 1,
                           (sizeof(T) == 2 && D == 128) ? 2 : 3, (sizeof(T) == 2 && D == 128) ? 4 : 0>;
// dK/dV with one wave per key block for bf16 (faster than pairs by 6 % at
// D = 80, 10 % at D = 64 and 5 % at D = 128); pairs of waves for fp32, whose
// wider fragments do not fit two waves per SIMD with both operands held
template <typename T, int D>
constexpr bool kv_single() { return sizeof(T) == 2; }

// ny > 1 (key-set calls only): dK/dV over ny query chunks and dQ over ny key
// chunks of a.qchunk / a.kchunk rows, side by side (blockIdx.y).
template <typename T, int D, typename OutT, bool GEN>
static int bwd_for(const void *q, const void *k, const void *v, const void *dout, const float *lse,
                   const float *delta, OutT *dq, OutT *dk, OutT *dv, BwdShape a, hipStream_t stream,
                   int ny = 1) {
    using KC = KvTileFor<T, D>;
    using K1 = KvTile1For<T, D>;
    using QC = QTileFor<T, D>;
    constexpr int BKV = kv_single<T, D>() ? K1::BKV : KC::BKV;
    const long long g1 = (long long)((a.Sk + BKV - 1) / BKV) * a.BH;
    a.nqt = (a.Sq + QC::BQ - 1) / QC::BQ;
    const long long g2 = (long long)a.nqt * a.BH;
    if (g1 > 0x7fffffffLL || g2 > 0x7fffffffLL || ny < 1 || ny > 65535) return -1;
    if (ny > 1 && !GEN) return -1;  // (chunks are key-set calls)
    if constexpr (kv_single<T, D>())
        hipLaunchKernelGGL((dkdv1_kernel<T, K1, OutT, GEN>), dim3((unsigned)g1, ny), dim3(K1::NT), 0, stream,
                           (const T *)q, (const T *)k, (const T *)v, (const T *)dout, lse, delta, dk, dv, a);
    else
        hipLaunchKernelGGL((dkdv_kernel<T, KC, OutT, GEN>), dim3((unsigned)g1, ny), dim3(KC::NT), 0, stream,
                           (const T *)q, (const T *)k, (const T *)v, (const T *)dout, lse, delta, dk, dv, a);
    if (hipGetLastError() != hipSuccess) return -5;
    hipLaunchKernelGGL((dq_kernel<T, QC, OutT, GEN>), dim3((unsigned)g2, ny), dim3(QC::NT), 0, stream,
                       (const T *)q, (const T *)k, (const T *)v, (const T *)dout, lse, delta, dq, a);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

#define FA_D_SWITCH(D, CALL)              \
    switch (D) {                          \
    case 16: { constexpr int DD = 16; return CALL; }   \
    case 32: { constexpr int DD = 32; return CALL; }   \
    case 64: { constexpr int DD = 64; return CALL; }   \
    case 80: { constexpr int DD = 80; return CALL; }   \
    case 96: { constexpr int DD = 96; return CALL; }   \
    case 128: { constexpr int DD = 128; return CALL; } \
    default: return -2;                   \
    }

// (as FA_D_SWITCH, but falls through on success)
#define FA_D_SWITCH_INT(D, CALL)                                          \
    {                                                                      \
        int rc_ = -2;                                                      \
        switch (D) {                                                       \
        case 16: { constexpr int DD = 16; rc_ = CALL; break; }             \
        case 32: { constexpr int DD = 32; rc_ = CALL; break; }             \
        case 64: { constexpr int DD = 64; rc_ = CALL; break; }             \
        case 80: { constexpr int DD = 80; rc_ = CALL; break; }             \
        case 96: { constexpr int DD = 96; rc_ = CALL; break; }             \
        case 128: { constexpr int DD = 128; rc_ = CALL; break; }           \
        default: break;                                                    \
        }                                                                  \
        if (rc_ != 0) return rc_;                                          \
    }

template <typename T>
static int delta_dispatch(int D, const void *o, const void *dout, float *delta, int BH, int S,
                          hipStream_t stream) {
    FA_D_SWITCH(D, (delta_for<T, DD>(o, dout, delta, BH, S, stream)))
}

template <typename T, typename OutT, bool GEN>
static int bwd_dispatch(int D, const void *q, const void *k, const void *v, const void *dout,
                        const float *lse, const float *delta, OutT *dq, OutT *dk, OutT *dv,
                        const BwdShape &a, hipStream_t stream) {
    FA_D_SWITCH(D, (bwd_for<T, DD, OutT, GEN>(q, k, v, dout, lse, delta, dq, dk, dv, a, stream)))
}

int launch_delta(int dtype, const void *o, const void *dout, float *delta, int BH, int S, int D,
                 hipStream_t stream) {
    if (dtype == 1) return delta_dispatch<bf16>(D, o, dout, delta, BH, S, stream);
    if (dtype == 0) return delta_dispatch<float>(D, o, dout, delta, BH, S, stream);
    return -2;
}

BwdSplit bwd_split(int dtype, int BH, int S, int D, int causal, int ncu, size_t max_part_bytes) {
    BwdSplit r{1, S};
    if ((dtype != 0 && dtype != 1) || !head_dim_supported(D) || S <= (dtype == 0 ? 64 : 256)) return r;  // (>= 2 chunks of 64)
    const long long cu = ncu > 0 ? ncu : 1;
    // The longest causal dK/dV workgroup walks the whole sequence.  Splitting
    // shortens that walk n-fold but writes and sums n sets of fp32 partials.
    // The counts below were measured (every chunk count, interleaved).
    long long n = 1;
    if (dtype == 1) {
        // bf16, 256 keys per dK/dV workgroup.  Over B*H = 1..128, S = 512..16384,
        // D = 64/80/128: about one busy workgroup per CU in flight is best; at
        // S <= 512 the walk is too short to pay for the partials unless only
        // a few tiles exist; with one to two tiles per CU, two chunks still
        // pay from S = 4096 on.
        const long long tiles = (long long)BH * ((S + 255) / 256);
        if (S <= 512)
            n = tiles * 16 <= cu ? 4 : 1;
        else if (D <= 16 && tiles < 2 * cu && S >= 2048)
            // D = 16 fits two workgroups per CU, placed together as the launch
            // starts: finer chunks keep two long causal walks off one CU
            // (B*H = 1..32, S = 2048..65536: 1.3-1.8x faster than 2 chunks)
            n = std::max<long long>(S >= 4096 ? 8 : 3, (cu + tiles - 1) / tiles);
        else if (2 * tiles <= cu)
            // (causal, from S = 4096 on, at least 3: with 2, half of the first
            // chunk's key tiles see no query of it; 3 chunks were 12-27 %
            // faster at CU/2 tiles, D = 32..128, but 13 % slower at S = 1024
            // and 13-20 % slower without the mask)
            n = std::max<long long>(causal && S >= 4096 ? 3 : 1, (cu + tiles - 1) / tiles);
        else if (tiles < cu)
            n = 2;
        else if (tiles < 2 * cu && S >= 4096)
            n = 2;
    } else {
        // fp32, 128 keys per (pair) dK/dV workgroup; each step is long (fp32
        // matrix cores), so splitting pays more and at more workgroups.  Over
        // B*H = 1..32, S = 512..16384, D = 64 and 128 (2.3-6.8x faster below
        // one workgroup per CU): 8 chunks up to a quarter workgroup per CU or
        // while the walk is long (S >= 32 tiles), 4 up to half, 2 up to two
        // per CU -- within 5 % of the best count at every measured point.
        const long long t = (long long)BH * ((S + 127) / 128);
        if (D == 128)
            // (D = 128: the dQ pass runs 4-wave, 128-query workgroups, twice as
            // many per chunk.  Over B*H = 1..32, S = 1024..16384 against every
            // count up to the rule below: 8 chunks up to an eighth workgroup per
            // CU, 4 up to a quarter, 3 up to half, 2 up to two; 3-39 % faster
            // where it differs.  Without the mask 2 up to half (3 were 31 %
            // slower) and none past it (2: 1 % slower).)
            n = 8 * t <= cu ? 8 : 4 * t <= cu ? 4 : 2 * t <= cu ? (causal ? 3 : 2) : (causal && t <= 2 * cu) ? 2 : 1;
        else
            n = (4 * t <= cu || 32 * t <= S) ? 8 : 2 * t <= cu ? 4 : t <= 2 * cu ? 2 : 1;
        // S <= 256 (one or two tiles per head; bf16 does not split there):
        // 1.3-2.4x faster up to CU/2 tiles (B*H = 1..16, D = 32..128), 10 %
        // slower at one tile per CU (B*H = 128, S = 256, 2 chunks)
        if (S <= 256 && 2 * t > cu) n = 1;
    }
    // at most 8 chunks (16 were no faster overall and hold twice the
    // partials), and no more partial results than the budget
    const long long per = 3LL * BH * S * D * 4;
    n = std::min<long long>(n, std::min<long long>(8, (long long)(max_part_bytes / (size_t)per)));
    if (n < 2) return r;
    const int chunk = (int)(((S + n - 1) / n + 63) / 64 * 64);  // whole 64-row tiles
    r.n = (S + chunk - 1) / chunk;
    r.chunk = chunk;
    if (r.n < 2) r = BwdSplit{1, S};
    return r;
}

int launch_bwd(int dtype, const void *q, const void *k, const void *v, const void *dout,
               const float *lse, const float *delta, void *dq, void *dk, void *dv, float *lse2, int BH,
               int S, int D, float scale, int causal, BwdSplit sp, hipStream_t stream) {
    if (dtype != 0 && dtype != 1) return -2;
    if (!head_dim_supported(D)) return -2;
    if (sp.n > 1) {
        // Few key tiles for the CUs: dK/dV over sp.n query chunks and dQ over
        // sp.n key chunks run side by side as key-set products (natural-log L,
        // fp32 partials in the workspace after the lse2 region), then summed.
        const size_t n_el = (size_t)BH * S * D;
        float *parts = lse2 + bwd_lse2_bytes((long long)BH * S) / sizeof(float);
        float *pq = parts, *pk = parts + (size_t)sp.n * n_el, *pv = parts + 2 * (size_t)sp.n * n_el;
        const BwdShape a{BH, S, S, 0, causal, 0, 0, scale * kLog2e, scale, sp.chunk, sp.chunk, 0};
        const long long count4 = (long long)(n_el / 4);
        const long long grid = (count4 + 255) / 256;
        if (grid > 0x7fffffffLL) return -1;
        // (the partials of dQ, dK, dV follow each other: pk = pq + n*n_el, pv = pk + n*n_el)
        if (dtype == 1) {
            FA_D_SWITCH_INT(D, (bwd_for<bf16, DD, float, true>(q, k, v, dout, lse, delta, pq, pk, pv, a, stream, sp.n)))
            hipLaunchKernelGGL(sum_parts_kernel<bf16>, dim3((unsigned)grid, 3), dim3(256), 0, stream, pq, sp.n,
                               (long long)n_el, (bf16 *)dq, (bf16 *)dk, (bf16 *)dv, count4);
        } else {
            FA_D_SWITCH_INT(D, (bwd_for<float, DD, float, true>(q, k, v, dout, lse, delta, pq, pk, pv, a, stream, sp.n)))
            hipLaunchKernelGGL(sum_parts_kernel<float>, dim3((unsigned)grid, 3), dim3(256), 0, stream, pq, sp.n,
                               (long long)n_el, (float *)dq, (float *)dk, (float *)dv, count4);
        }
        return hipGetLastError() == hipSuccess ? 0 : -5;
    }
    const long long rows = (long long)BH * S;
    const long long grid = (rows + 255) / 256;
    if (grid > 0x7fffffffLL) return -1;
    hipLaunchKernelGGL(lse2_kernel, dim3((unsigned)grid), dim3(256), 0, stream, lse, lse2, rows);
    if (hipGetLastError() != hipSuccess) return -5;
    // (consecutive workgroups take consecutive heads: the banded XCD order of
    // the forward cut both passes' HBM traffic by 35-60 % at S = 65536, D = 128
    // but ran 0.3 % slower there and 2 % slower at S = 16000, D = 80)
    const BwdShape a{BH, S, S, 0, causal, 0, 0, scale * kLog2e, scale, S, S, 0};
    if (dtype == 1)
        return bwd_dispatch<bf16, bf16, false>(D, q, k, v, dout, lse2, delta, (bf16 *)dq, (bf16 *)dk,
                                               (bf16 *)dv, a, stream);
    return bwd_dispatch<float, float, false>(D, q, k, v, dout, lse2, delta, (float *)dq, (float *)dk,
                                             (float *)dv, a, stream);
}

// ------------------------------------------- allocation-free backward ---
//
// For callers that cannot allocate device memory (code under graph capture,
// serving loops, harnesses that forbid it), the backward can run out of a
// fixed array in device memory instead of a caller's workspace: the base-2
// copy of lse and, when they fit, the split's partials.  Each GPU the library
// runs on holds its own copy until the process ends; every call on a GPU
// shares it, so calls that overlap on one GPU race.  Nothing in it needs to
// start at zero: every call overwrites what it reads.
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<float *> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

// The device address of `scratch` on the device of `stream`.  In host code
// the array's name is only a stand-in for the symbol; its address on a device
// comes from the runtime, looked up once per device with that device current.
float *noalloc_scratch(hipStream_t stream) {
    int dev = -1;
    if (stream ? hipStreamGetDevice(stream, &dev) != hipSuccess : hipGetDevice(&dev) != hipSuccess) return nullptr;
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    if (float *p = g_scratch[dev].load(std::memory_order_acquire)) return p;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (float *p = g_scratch[dev].load(std::memory_order_acquire)) return p;
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return nullptr;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || p == nullptr) {
        (void)hipGetLastError();  // (clear the sticky error the failed lookup left)
        return nullptr;
    }
    g_scratch[dev].store(static_cast<float *>(p), std::memory_order_release);
    return static_cast<float *>(p);
}

int launch_bwd_partial(int dtype, const void *q, const void *k, const void *v, const void *dout,
                       const float *lse, const float *delta, float *dq, float *dk, float *dv,
                       int accumulate, int BH, int Sq, int Sk, int D, float scale, int causal,
                       int q_offset, hipStream_t stream) {
    const BwdShape a{BH, Sq, Sk, q_offset, causal, 0, accumulate, scale * kLog2e, scale, Sq, Sk, 0};
    if (dtype == 1)
        return bwd_dispatch<bf16, float, true>(D, q, k, v, dout, lse, delta, dq, dk, dv, a, stream);
    if (dtype == 0)
        return bwd_dispatch<float, float, true>(D, q, k, v, dout, lse, delta, dq, dk, dv, a, stream);
    return -2;
}

// Every kernel the dispatch above can launch, instantiated explicitly (the
// host compilation pass has been seen to drop the launch stubs of some
// implicitly instantiated kernel templates).
// (dK/dV: the one-wave kernel for bf16, the pair kernel for fp32; see kv_single)
#define FA_BWD_KERNELS(T, D, OUT, GEN)                                                                       \
    template __global__ void dq_kernel<T, QTileFor<T, D>, OUT, GEN>(                                        \
        const T *, const T *, const T *, const T *, const float *, const float *, OUT *, BwdShape);
#define FA_BWD_KV1(T, D, OUT, GEN)                                                                           \
    template __global__ void dkdv1_kernel<T, KvTile1For<T, D>, OUT, GEN>(                                   \
        const T *, const T *, const T *, const T *, const float *, const float *, OUT *, OUT *, BwdShape);
#define FA_BWD_KV2(T, D, OUT, GEN)                                                                           \
    template __global__ void dkdv_kernel<T, KvTileFor<T, D>, OUT, GEN>(                                     \
        const T *, const T *, const T *, const T *, const float *, const float *, OUT *, OUT *, BwdShape);
#define FA_BWD_HEAD(T, D)                                                                   \
    static_assert(kv_single<T, D>() == (sizeof(T) == 2), "dK/dV kernel instantiated below"); \
    FA_BWD_KERNELS(T, D, T, false)                                                          \
    FA_BWD_KERNELS(T, D, float, true)                                                       \
    FA_BWD_KV_FOR_##T(T, D, T, false)                                                       \
    FA_BWD_KV_FOR_##T(T, D, float, true)
#define FA_BWD_KV_FOR_bf16 FA_BWD_KV1
#define FA_BWD_KV_FOR_float FA_BWD_KV2
FA_BWD_HEAD(bf16, 16)
FA_BWD_HEAD(bf16, 32)
FA_BWD_HEAD(bf16, 64)
FA_BWD_HEAD(bf16, 80)
FA_BWD_HEAD(bf16, 96)
FA_BWD_HEAD(bf16, 128)
FA_BWD_HEAD(float, 16)
FA_BWD_HEAD(float, 32)
FA_BWD_HEAD(float, 64)
FA_BWD_HEAD(float, 80)
FA_BWD_HEAD(float, 96)
FA_BWD_HEAD(float, 128)
#undef FA_BWD_HEAD
#undef FA_BWD_KV_FOR_bf16
#undef FA_BWD_KV_FOR_float
#undef FA_BWD_KV2
#undef FA_BWD_KV1
#undef FA_BWD_KERNELS

}  // namespace fa
