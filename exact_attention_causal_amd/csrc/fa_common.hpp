// fa_common.hpp -- shared device building blocks of the gfx950 attention kernels.
//
// Matrix-core conventions (CDNA3/CDNA4 32x32 MFMA, one 64-lane wavefront):
//   * 32x32 output block C (16 fp32 per lane): lane l, register r holds
//     C[row = 8*(r/4) + 4*(l/32) + r%4][col = l%32].
//   * A operand (32 rows x K): lane l holds A[row = l%32][k-slots of half l/32];
//     B operand (K x 32 cols): lane l holds B[k-slots of half l/32][col = l%32].
//     bf16 (v_mfma_f32_32x32x16_bf16): 8 consecutive k-slots per lane per
//     instruction; fp32 (v_mfma_f32_32x32x2f32): one k-slot per lane.
//
// Because a reduction does not care in which order its terms are summed, the
// kernels choose the mapping from MFMA rows and k-slots to real indices:
//   * A-operand row rho of a 32-row block is the real index sigma(rho), chosen
//     so that output register r of half h belongs to index
//         idx(r, h) = 16*(r/8) + 8*h + r%8,
//     i.e. registers 0..7 of a half are 8 consecutive indices and 8..15 the
//     next 8 + 8.  An output block can therefore be fed straight back as the
//     B operand of the next product (k-slots of instruction u = registers
//     u*KPL ..), and the matching A operand is two runs of 8 consecutive
//     elements per lane -- one 16-byte LDS read each for bf16.
//   * For products reducing over the head dimension, half h of the lanes owns
//     d in [h*D/2, (h+1)*D/2); instruction s takes KPL consecutive d of it.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kWave = 64;

template <typename T> struct Mma;

template <> struct Mma<bf16> {
    static constexpr int KPL = 8;  // k-slots per lane per instruction
    typedef bf16x8 frag;
    __device__ static inline f32x16 run(frag a, frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    __device__ static inline frag zero() { return frag{}; }
};

template <> struct Mma<float> {
    static constexpr int KPL = 1;
    typedef float frag;
    __device__ static inline f32x16 run(frag a, frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
    __device__ static inline frag zero() { return 0.f; }
};

// Real index of output register r for lane half h (see header).
__device__ __host__ constexpr inline int idx_of(int r, int h) { return 16 * (r / 8) + 8 * h + (r % 8); }

// Real index that A-operand row rho stands for, so that output rows line up with idx_of.
__device__ __host__ constexpr inline int sigma(int rho) {
    return idx_of(4 * (rho / 8) + (rho % 4), (rho / 4) % 2);
}

// ---- fragments ------------------------------------------------------------

// N fragments = N*KPL consecutive elements from a 16-byte-aligned address
// (global or LDS).
template <typename T, int N>
__device__ inline void load_run(typename Mma<T>::frag (&dst)[N], const T *src) {
    if constexpr (Mma<T>::KPL == 8) {
#pragma unroll
        for (int i = 0; i < N; ++i) dst[i] = *reinterpret_cast<const bf16x8 *>(src + 8 * i);
    } else {
        static_assert(N % 4 == 0, "fp32 runs are read 4 at a time");
#pragma unroll
        for (int i = 0; i < N / 4; ++i) {
            f32x4 v = *reinterpret_cast<const f32x4 *>(src + 4 * i);
            dst[4 * i + 0] = v[0];
            dst[4 * i + 1] = v[1];
            dst[4 * i + 2] = v[2];
            dst[4 * i + 3] = v[3];
        }
    }
}

template <typename T, int N>
__device__ inline void zero_run(typename Mma<T>::frag (&dst)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) dst[i] = Mma<T>::zero();
}

// A-operand fragments reducing over one 32-index block of a transposed LDS
// tile row: elements idx_of(r, h) for r = 0..15, i.e. runs [8h, 8h+8) and
// [16+8h, 24+8h) of `row` (16/KPL instructions).
template <typename T>
__device__ inline void load_kblock(typename Mma<T>::frag (&dst)[16 / Mma<T>::KPL], const T *row, int h) {
    constexpr int H = 8 / Mma<T>::KPL;
    typename Mma<T>::frag a[H], b[H];
    load_run<T, H>(a, row + 8 * h);
    load_run<T, H>(b, row + 16 + 8 * h);
#pragma unroll
    for (int i = 0; i < H; ++i) {
        dst[i] = a[i];
        dst[H + i] = b[i];
    }
}

// An fp32 output block (16 registers) as B-operand fragments (rounded to T).
template <typename T>
__device__ inline void to_bfrag(typename Mma<T>::frag (&dst)[16 / Mma<T>::KPL], const f32x16 &c) {
    if constexpr (Mma<T>::KPL == 8) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            bf16x8 f;
#pragma unroll
            for (int t = 0; t < 8; ++t) f[t] = (bf16)c[8 * u + t];
            dst[u] = f;
        }
    } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) dst[r] = c[r];
    }
}

// ---- global <-> registers <-> LDS tiles ------------------------------------
//
// A tile is R rows x D columns of a [S][D] head.  It is moved in units of
// 4 rows x 16 bytes: unit u covers column chunk c = u % CPR (CPR = 16-byte
// chunks per row) of rows 4*(u / CPR) .. +3, so consecutive threads read
// consecutive 16-byte chunks of a row.  Rows at or beyond S read as zero.

template <typename T, int R, int D, int NT>
struct TileIO {
    static constexpr int VEC = 16 / sizeof(T);       // elements per 16-byte chunk
    static constexpr int CPR = D / VEC;              // chunks per row
    static constexpr int UNITS = (R / 4) * CPR;
    static constexpr int UPT = (UNITS + NT - 1) / NT;  // units per thread
    static_assert(D % VEC == 0, "D must be a multiple of 16 bytes");
    static_assert(R % 4 == 0, "tile rows must be a multiple of 4");

    u32x4 reg[UPT][4];

    __device__ inline void load(const T *base, int row0, int S, int tid) {
#pragma unroll
        for (int i = 0; i < UPT; ++i) {
            const int u = tid + i * NT;
            const int c = u % CPR, rg = u / CPR;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int row = row0 + 4 * rg + rr;
                u32x4 x = {0u, 0u, 0u, 0u};
                if ((UNITS % NT == 0 || u < UNITS) && row < S)
                    x = *reinterpret_cast<const u32x4 *>(base + (size_t)row * D + c * VEC);
                reg[i][rr] = x;
            }
        }
    }

    // Row-major LDS tile, row stride LD elements.
    template <int LD>
    __device__ inline void store_rows(T *lds, int tid) const {
#pragma unroll
        for (int i = 0; i < UPT; ++i) {
            const int u = tid + i * NT;
            if (UNITS % NT != 0 && u >= UNITS) continue;
            const int c = u % CPR, rg = u / CPR;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
                *reinterpret_cast<u32x4 *>(lds + (4 * rg + rr) * LD + c * VEC) = reg[i][rr];
        }
    }

    // Transposed LDS tile: element (row, d) goes to lds[d * LD + row].
    template <int LD>
    __device__ inline void store_cols(T *lds, int tid) const {
#pragma unroll
        for (int i = 0; i < UPT; ++i) {
            const int u = tid + i * NT;
            if (UNITS % NT != 0 && u >= UNITS) continue;
            const int c = u % CPR, rg = u / CPR;
            if constexpr (sizeof(T) == 2) {
                // 8 columns of 4 rows: 8 writes of 4 bf16 (8 bytes)
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const int w = t / 2, sh = 16 * (t % 2);
                    uint32_t e0 = (reg[i][0][w] >> sh) & 0xffffu, e1 = (reg[i][1][w] >> sh) & 0xffffu;
                    uint32_t e2 = (reg[i][2][w] >> sh) & 0xffffu, e3 = (reg[i][3][w] >> sh) & 0xffffu;
                    u32x2 p = {e0 | (e1 << 16), e2 | (e3 << 16)};
                    *reinterpret_cast<u32x2 *>(lds + (c * 8 + t) * LD + 4 * rg) = p;
                }
            } else {
                // 4 columns of 4 rows: 4 writes of 4 fp32 (16 bytes)
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    u32x4 p = {reg[i][0][t], reg[i][1][t], reg[i][2][t], reg[i][3][t]};
                    *reinterpret_cast<u32x4 *>(lds + (c * 4 + t) * LD + 4 * rg) = p;
                }
            }
        }
    }
};

// Zero rows [r0, r1) of a row-major LDS array with LD elements per row.
template <typename T, int LD, int NT>
__device__ inline void zero_lds_rows(T *lds, int r0, int r1, int tid) {
    static_assert((LD * sizeof(T)) % 16 == 0, "row stride must be 16-byte aligned");
    constexpr int CH = LD * sizeof(T) / 16;
    for (int u = tid; u < (r1 - r0) * CH; u += NT) {
        const int r = r0 + u / CH, c = u % CH;
        *reinterpret_cast<u32x4 *>(reinterpret_cast<char *>(lds + r * LD) + 16 * c) = u32x4{0u, 0u, 0u, 0u};
    }
}

// Store 8 consecutive output elements (fp32 values * mul, rounded to T).
template <typename T>
__device__ inline void store8(T *dst, const f32x16 &c, int r0, float mul) {
    if constexpr (sizeof(T) == 2) {
        bf16x8 v;
#pragma unroll
        for (int t = 0; t < 8; ++t) v[t] = (bf16)(c[r0 + t] * mul);
        *reinterpret_cast<bf16x8 *>(dst) = v;
    } else {
        f32x4 a = {c[r0] * mul, c[r0 + 1] * mul, c[r0 + 2] * mul, c[r0 + 3] * mul};
        f32x4 b = {c[r0 + 4] * mul, c[r0 + 5] * mul, c[r0 + 6] * mul, c[r0 + 7] * mul};
        *reinterpret_cast<f32x4 *>(dst) = a;
        *reinterpret_cast<f32x4 *>(dst + 4) = b;
    }
}

__device__ inline float wave_xor32_max(float x) { return fmaxf(x, __shfl_xor(x, 32)); }
__device__ inline float wave_xor32_sum(float x) { return x + __shfl_xor(x, 32); }

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace fa
