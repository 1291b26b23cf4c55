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

// ---- swizzled row-major LDS tiles -----------------------------------------
//
// Every LDS tile is row-major with a power-of-two pitch of 8, 16 or 32
// 16-byte chunks per row, and logical chunk c of row r sits at physical chunk
// c ^ f(r).  f is chosen so that both read patterns the kernels use are free
// of bank conflicts on the 64 four-byte LDS banks:
//   * "row" reads (A operand reducing over columns): 16 lanes read one
//     16-byte chunk each from 16 different rows;
//   * "transposed" reads (ds_read_b64_tr_b16, A operand reducing over rows):
//     32 lanes read 4 consecutive rows x 64 bytes.
// Chunks at or beyond the logical row length stay zero (the tile is cleared
// once), which is how head dimensions pad to whole 32-row output blocks.

template <typename T, int D>
struct Swz {
    static constexpr int CW = 16 / sizeof(T);                            // elements per chunk
    static constexpr int CPR = D / CW;                                   // logical chunks per row
    static constexpr int PCH = CPR <= 8 ? 8 : (CPR <= 16 ? 16 : 32);     // physical chunks per row
    static constexpr int PITCH = PCH * CW;                               // elements per row
    static_assert(D % CW == 0, "rows must be whole 16-byte chunks");
    __device__ static constexpr inline int f(int r) {
        return PCH == 8 ? 4 * ((r >> 1) & 1) + ((r >> 2) & 3) : 4 * (r & 3) + ((r >> 2) & 3);
    }
    // element offset of logical chunk c of row r
    __device__ static constexpr inline int off(int r, int c) { return r * PITCH + ((c ^ f(r)) * CW); }
    // element offset of column `col` of row r
    __device__ static constexpr inline int at(int r, int col) { return off(r, col / CW) + col % CW; }
};

// Global -> registers -> LDS mover for an R-row tile of a [S][D] head.
// Unit u is chunk u % CPR of row u / CPR, so consecutive threads read
// consecutive 16-byte chunks.  Rows at or beyond S read as zero.
template <typename T, int D, int R, int NT>
struct TileLoader {
    using SW = Swz<T, D>;
    static constexpr int UNITS = R * SW::CPR;
    static constexpr int UPT = (UNITS + NT - 1) / NT;
    u32x4 reg[UPT];

    __device__ inline void load(const T *base, int row0, int S, int tid) {
#pragma unroll
        for (int i = 0; i < UPT; ++i) {
            const int u = tid + i * NT;
            const int r = u / SW::CPR, c = u % SW::CPR;
            u32x4 x = {0u, 0u, 0u, 0u};
            if ((UNITS % NT == 0 || u < UNITS) && row0 + r < S)
                x = *reinterpret_cast<const u32x4 *>(base + (size_t)(row0 + r) * D + c * SW::CW);
            reg[i] = x;
        }
    }
    __device__ inline void store(T *lds, int tid) const {
#pragma unroll
        for (int i = 0; i < UPT; ++i) {
            const int u = tid + i * NT;
            if (UNITS % NT != 0 && u >= UNITS) continue;
            const int r = u / SW::CPR, c = u % SW::CPR;
            *reinterpret_cast<u32x4 *>(lds + SW::off(r, c)) = reg[i];
        }
    }
};

// Direct global -> LDS tile loads (global_load_lds_dwordx4): each instruction
// of a wave writes 1 KiB of consecutive LDS (16 bytes per lane, in lane
// order), so a lane is told which global chunk belongs at its LDS position of
// the swizzled tile.  Rows past the end of the sequence load the last row and
// padding chunks load the row's last chunk: the values are finite, and the
// kernels mask those rows or never store the outputs they feed.
template <typename T, int D, int R, int NW>
struct TileDma {
    using SW = Swz<T, D>;
    static constexpr int ROW_BYTES = SW::PITCH * (int)sizeof(T);
    static constexpr int RPI = 1024 / ROW_BYTES;      // rows per instruction
    static constexpr int NINS = R / RPI;              // instructions per tile
    static constexpr int IPW = NINS / NW;             // instructions per wave
    static_assert(1024 % ROW_BYTES == 0 && R % RPI == 0 && NINS % NW == 0, "tile/DMA shape");
    int row[IPW];  // row within the tile
    int col[IPW];  // element column of the chunk

    __device__ inline void init(int lane, int wave) {
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
            const int p = (wave * IPW + i) * 64 + lane;  // 16-byte slot within the tile
            const int r = p / SW::PCH, pc = p % SW::PCH;
            const int c = min(pc ^ SW::f(r), SW::CPR - 1);
            row[i] = r;
            col[i] = c * SW::CW;
        }
    }
    // Issue this wave's share of the tile holding rows row0 .. row0 + R - 1.
    __device__ inline void issue(T *lds, const T *base, int row0, int S, int wave) const {
        typedef __attribute__((address_space(3))) void lds_void;
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
            const int r = min(row0 + row[i], S - 1);
            T *dst = lds + (wave * IPW + i) * (1024 / (int)sizeof(T));
            __builtin_amdgcn_global_load_lds((const void *)(base + (size_t)r * D + col[i]),
                                             (lds_void *)dst, 16, 0, 0);
        }
    }
};

// s_waitcnt with only the vector-memory counter limited to n (gfx9 encoding).
template <int N>
__device__ inline void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// s_waitcnt lgkmcnt(0) (LDS reads and writes of this wave completed).
__device__ inline void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (3 << 14)); }

// Workgroup barrier that does not wait for outstanding global loads (so LDS
// DMA of the next tile stays in flight); the empty asm statements keep the
// compiler from moving memory accesses across it.
__device__ inline void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Clear n elements of LDS (n a multiple of 8 bytes' worth is not required; 16-byte steps).
template <typename T, int N, int NT>
__device__ inline void zero_lds(T *lds, int tid) {
    static_assert((N * sizeof(T)) % 16 == 0, "tile bytes must be a multiple of 16");
    constexpr int CH = N * sizeof(T) / 16;
    for (int u = tid; u < CH; u += NT) reinterpret_cast<u32x4 *>(lds)[u] = u32x4{0u, 0u, 0u, 0u};
}

// A-operand fragments reducing over the head dimension, from rows of a tile:
// lane (h, l32) takes row `row` and columns [h*D/2, (h+1)*D/2) (D/2/KPL fragments).
template <typename T, int D>
__device__ inline void load_row_frags(typename Mma<T>::frag (&dst)[D / 2 / Mma<T>::KPL], const T *tile,
                                      int row, int h) {
    using SW = Swz<T, D>;
    constexpr int KPL = Mma<T>::KPL;
    constexpr int NCH = D / 2 / SW::CW;  // chunks per half row
    const T *rp = tile + row * SW::PITCH;
    const int fx = SW::f(row);
#pragma unroll
    for (int q = 0; q < NCH; ++q) {
        const u32x4 x = *reinterpret_cast<const u32x4 *>(rp + (((h * NCH + q) ^ fx) * SW::CW));
        if constexpr (KPL == 8) {
            dst[q] = __builtin_bit_cast(bf16x8, x);
        } else {
            const f32x4 v = __builtin_bit_cast(f32x4, x);
            dst[4 * q + 0] = v[0];
            dst[4 * q + 1] = v[1];
            dst[4 * q + 2] = v[2];
            dst[4 * q + 3] = v[3];
        }
    }
}

// A-operand fragments reducing over 32 rows of a tile (rows 32*kb + idx_of(r, h)),
// output row = column 32*cb + sigma(l32).  bf16 uses the LDS transpose read
// ds_read_b64_tr_b16: in each 16-lane group, destination lane i receives
// column i of the 4 x 16 block whose row k, columns 4c..4c+3 the source lane
// 4k + c points at.  fp32 reads single elements.
template <typename T, int D>
struct TransReader {
    using SW = Swz<T, D>;
    static constexpr int NCB = (D + 31) / 32;  // 32-column output blocks
    static constexpr int NI = 16 / Mma<T>::KPL;
    int off[NCB][2];  // bf16: per output block and half-fragment, lane offset within a 16-row slab

    __device__ inline void init(int lane) {
        if constexpr (Mma<T>::KPL == 8) {
            const int g = lane >> 4, j = lane & 15, k = j >> 2, c = j & 3;
            const int h = g >> 1, sub = g & 1;
            constexpr int perm4[4] = {0, 8, 4, 12};
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                for (int rr = 0; rr < 2; ++rr) {
                    const int row = 4 * rr + 8 * h + k;          // row within a 16-row slab
                    const int col = 32 * cb + 16 * sub + perm4[c];
                    off[cb][rr] = SW::at(row, col);
                }
        }
    }

    __device__ inline void load(typename Mma<T>::frag (&dst)[NI], const T *tile, int kb, int cb, int lane) const {
        if constexpr (Mma<T>::KPL == 8) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const T *slab = tile + (32 * kb + 16 * u) * SW::PITCH;  // rows 32kb+16u .. +15
                typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
                const bf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                    (lds_bf16x4 *)(slab + off[cb][0]));
                const bf16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                    (lds_bf16x4 *)(slab + off[cb][1]));
                dst[u] = bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
            }
        } else {
            const int h = lane >> 5, col = 32 * cb + sigma(lane & 31);
#pragma unroll
            for (int r = 0; r < 16; ++r) dst[r] = tile[SW::at(32 * kb + idx_of(r, h), col)];
        }
    }
};

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
