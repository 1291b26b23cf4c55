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
// kernels choose which real index each A-operand row and each k-slot stands
// for.  Two mappings are used:
//   * reduction rows (keys in the forward and dQ passes, queries in the dK/dV
//     pass): output register r of half h is index
//         ridx(r, h) = 16*(r/8) + 4*(r%4) + 2*h + (r/4)%2.
//     An output block is then the B operand of the next product as it stands
//     (instruction u takes registers 8u..8u+7), and the matching A operand --
//     read with the LDS transpose instruction -- takes every 4th row of the
//     tile, which with a padded row pitch keeps LDS banks conflict-free;
//   * head-dimension rows of the outputs: register r of half h is
//         didx(r, h) = 16*(r/8) + 8*h + r%8,
//     so registers 0..7 and 8..15 of a lane are runs of 8 consecutive d and
//     the epilogue stores 16 bytes at a time.
// For products reducing over the head dimension, half h of the lanes owns d
// in [h*D/2, (h+1)*D/2); instruction s takes KPL consecutive d of it.
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

// Reduction-row index of output register r of half h (see header).
__device__ __host__ constexpr inline int ridx(int r, int h) {
    return 16 * (r / 8) + 4 * (r % 4) + 2 * h + (r / 4) % 2;
}
// Reduction-row index that A-operand row rho stands for (so output rows line up with ridx).
__device__ __host__ constexpr inline int rsigma(int rho) {
    return 16 * (rho / 16) + 4 * (rho % 4) + 2 * ((rho / 4) % 2) + (rho / 8) % 2;
}
// Head-dimension index of output register r of half h.
__device__ __host__ constexpr inline int didx(int r, int h) { return 16 * (r / 8) + 8 * h + (r % 8); }
// Head-dimension index that A-operand row rho stands for.
__device__ __host__ constexpr inline int dsigma(int rho) {
    return 16 * (rho / 16) + 8 * ((rho / 4) % 2) + 4 * ((rho / 8) % 2) + rho % 4;
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

// Negate fragments in place (sign flips only: exact).
template <typename T, int N>
__device__ inline void neg_run(typename Mma<T>::frag (&x)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
        if constexpr (Mma<T>::KPL == 8) {
            typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
            x[i] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, x[i]) ^ 0x80008000u);
        } else {
            x[i] = -x[i];
        }
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

// ---- padded row-major LDS tiles --------------------------------------------
//
// Every LDS tile is row-major with a row pitch of D + 16 bytes' worth of
// elements, i.e. 4 (mod 8) four-byte words for every head dimension used.  On
// the 64 four-byte LDS banks that makes both read patterns conflict-free:
//   * row reads (A operand reducing over the head dimension): 16 lanes read
//     one 16-byte chunk each from 16 consecutive rows -> 16 distinct 4-bank
//     groups;
//   * transposed reads (ds_read_b64_tr_b16, A operand reducing over rows):
//     32 lanes read 4 rows spaced 4 apart x 64 bytes -> 4 disjoint 16-bank
//     windows.
// Every per-lane address is then one base register plus an immediate offset.

template <typename T, int D>
struct Pad {
    static constexpr int CW = 16 / sizeof(T);          // elements per 16-byte chunk
    static constexpr int CPR = D / CW;                 // data chunks per row
    static constexpr int SLOTS = CPR + 1;              // 16-byte slots per row (one pad)
    static constexpr int PITCH = SLOTS * CW;           // elements per row
    static_assert(D % CW == 0, "rows must be whole 16-byte chunks");
    static_assert(((PITCH * sizeof(T) / 4) % 8) == 4, "pitch must be 4 (mod 8) words");
};

// Direct global -> LDS tile loads (buffer_load_dwordx4 ... lds): each
// instruction of a wave writes 1 KiB of consecutive LDS (16 bytes per lane, in
// lane order), so each lane fetches the global chunk that belongs at its LDS
// slot.  The tile's slots are rounded up to whole instructions for every wave.
// The loads go through a buffer descriptor whose range ends at the last row of
// the tile that exists: slots past the tile's last row, pad slots and rows past
// the end of the sequence are out of range, so they fetch nothing from memory
// and land as zeros (the kernels mask those rows or never read the pad).
template <typename T, int D, int R, int NW>
struct TileDma {
    using PD = Pad<T, D>;
    static constexpr int NSLOT = R * PD::SLOTS;
    static constexpr int IPW = (NSLOT + 64 * NW - 1) / (64 * NW);  // instructions per wave
    static constexpr int ELEMS = IPW * NW * 64 * PD::CW;          // tile allocation (elements)
    static constexpr int kNone = 0x40000000;                      // beyond any tile's range
    // transposed reads of the last 32-column block may run up to 32 elements past a row
    static_assert(R * PD::PITCH + 32 <= ELEMS || PD::CPR * PD::CW % 32 == 0, "tile slack");
    static_assert((long long)R * D * sizeof(T) < kNone, "tile range");
    int voff[IPW];  // byte offset of this lane's chunk from the tile's first row, or kNone

    __device__ inline void init(int lane, int wave) {
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
            const int p = (wave * IPW + i) * 64 + lane;  // 16-byte slot within the tile
            const int r = p / PD::SLOTS, cc = p % PD::SLOTS;
            voff[i] = (r < R && cc < PD::CPR) ? (r * D + cc * PD::CW) * (int)sizeof(T) : kNone;
        }
    }
    // Descriptor of rows row0 .. min(row0 + R, S) - 1 of a [S, D] matrix
    // (empty when row0 >= S).  All arguments are wave-uniform.
    static __device__ inline __amdgpu_buffer_rsrc_t range(const T *base, int row0, int S) {
        // (the clamp is selected as a vector min/max; readfirstlane hands the
        // uniform result back to the scalar unit, where the descriptor lives)
        const int rows = __builtin_amdgcn_readfirstlane(max(0, min(R, S - row0)));
        // dword 3: 32-bit data format (the raw-buffer setting for gfx9 parts)
        return __builtin_amdgcn_make_buffer_rsrc((void *)(base + (size_t)row0 * D), 0,
                                                 rows * D * (int)sizeof(T), 0x00020000);
    }
    // Issue instruction i of this wave's share of the tile described by `rs`
    // (kernels spread the instructions over their work so the waves of a
    // workgroup do not all queue at the memory pipeline at once).
    __device__ inline void issue_one(int i, T *lds, __amdgpu_buffer_rsrc_t rs, int wave) const {
        typedef __attribute__((address_space(3))) void lds_void;
        T *dst = lds + (wave * IPW + i) * (1024 / (int)sizeof(T));
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)dst, 16, voff[i], 0, 0, 0);
    }
    // Issue part p of np near-equal parts of this wave's share (np is a
    // compile-time constant at every call; it is a plain argument because a
    // member template taking the descriptor type does not substitute in the
    // host compilation pass).
    __device__ inline void issue_part(int p, int np, T *lds, __amdgpu_buffer_rsrc_t rs, int wave) const {
        const int a = (IPW * p + np - 1) / np, b = (IPW * (p + 1) + np - 1) / np;
#pragma unroll
        for (int i = 0; i < IPW; ++i)
            if (i >= a && i < b) issue_one(i, lds, rs, wave);
    }
    // Issue this wave's whole share of the tile holding rows row0 .. row0 + R - 1.
    __device__ inline void issue(T *lds, const T *base, int row0, int S, int wave) const {
        const __amdgpu_buffer_rsrc_t rs = range(base, row0, S);
#pragma unroll
        for (int i = 0; i < IPW; ++i) issue_one(i, lds, rs, wave);
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

// A-operand fragments reducing over the head dimension, from row `row` of a
// tile: lane half h takes columns [h*D/2, (h+1)*D/2) (D/2/KPL fragments).
template <typename T, int D>
__device__ inline void load_row_frags(typename Mma<T>::frag (&dst)[D / 2 / Mma<T>::KPL], const T *tile,
                                      int row, int h) {
    load_run<T, D / 2 / Mma<T>::KPL>(dst, tile + row * Pad<T, D>::PITCH + h * (D / 2));
}

// A-operand fragments reducing over 32 rows of a tile (rows 32*kb + ridx(r, h)),
// output row = column 32*cb + dsigma(l32).  bf16 uses the LDS transpose read
// ds_read_b64_tr_b16: in each 16-lane group, destination lane i receives
// column i of the 4 x 16 block whose row e, columns 4c..4c+3 source lane
// 4e + c points at.  fp32 reads single elements.
template <typename T, int D>
struct TransReader {
    using PD = Pad<T, D>;
    static constexpr int NI = 16 / Mma<T>::KPL;
    int base;  // per-lane element offset; everything else is an immediate

    __device__ inline void init(int lane) {
        const int h = lane >> 5;
        if constexpr (Mma<T>::KPL == 8) {
            const int g = lane >> 4, j = lane & 15, e = j >> 2, c = j & 3;
            const int sub = g & 1;
            // source row 4e + 2h (+1 for the second read) of a 16-row slab;
            // the four 4-column chunks of a group cover dsigma of its 16 lanes
            base = (4 * e + 2 * h) * PD::PITCH + 16 * sub + 4 * ((c & 1) * 2 + (c >> 1));
        } else {
            base = 2 * h * PD::PITCH + dsigma(lane & 31);
        }
    }

    __device__ inline void load(typename Mma<T>::frag (&dst)[NI], const T *tile, int kb, int cb) const {
        if constexpr (Mma<T>::KPL == 8) {
            typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const T *p = tile + base + (32 * kb + 16 * u) * PD::PITCH + 32 * cb;
                const bf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)p);
                const bf16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(p + PD::PITCH));
                dst[u] = bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
            }
        } else {
            const T *p = tile + base + 32 * kb * PD::PITCH + 32 * cb;
#pragma unroll
            for (int r = 0; r < 16; ++r) dst[r] = p[ridx(r, 0) * PD::PITCH];
        }
    }
};

// ---- 16-row output tails (bf16, D = 16 (mod 32)) --------------------------
//
// A head dimension of 32k + 16 leaves a last output block of 16 rows.  It is
// formed with v_mfma_f32_16x16x32_bf16 (half the matrix-core time of a padded
// 32x32x16 pair) as two 16-column blocks, one per 16 columns of the 32x32
// block whose B operand it shares:
//   * output (16 x 16): lane 16g + i, register r holds C[row 4g + r][col i];
//   * B operand (32 x 16): lane 16g + i holds 8 k-slots for column i.  From
//     the two B fragments of a 32x32 output block (registers 0..7 and 8..15,
//     i.e. reduction rows 16u + 2h + {0,4,8,12,1,5,9,13}), one half-row swap
//     (v_permlane16_swap: odd 16-lane rows of the first with even rows of the
//     second) leaves in the first fragment the operand of columns 0..15 and in
//     the second that of columns 16..31, with lane group g holding reduction
//     rows b_g + {0,4,8,12,1,5,9,13}, b_g = 16*(g&1) + 2*(g>>1);
//   * A operand (16 x 32): lane 16g + i holds row i at those reduction rows,
//     which two transposing LDS reads deliver (TailReader).
__device__ inline f32x4 mma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// B operands of the two 16-column tail blocks from the two B fragments of a
// 32x32 output block (see above).
__device__ inline void tail_bfrag(const bf16x8 (&pf)[2], bf16x8 &b0, bf16x8 &b1) {
    u32x4 x = __builtin_bit_cast(u32x4, pf[0]), y = __builtin_bit_cast(u32x4, pf[1]);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const auto r = __builtin_amdgcn_permlane16_swap(x[w], y[w], false, false);
        x[w] = r[0];
        y[w] = r[1];
    }
    b0 = __builtin_bit_cast(bf16x8, x);
    b1 = __builtin_bit_cast(bf16x8, y);
}

// A value held per 32x32 column (lane l and l ^ 32 hold column l % 32), as the
// two tail blocks need it: lane 16g + i gets column i (first) and 16 + i (second).
__device__ inline void tail_cols(float x, float &c0, float &c1) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    c0 = __uint_as_float(r[0]);
    c1 = __uint_as_float(r[1]);
}

// A operand of a 16-row tail: rows are columns c0..c0+15 of a padded tile,
// reducing over tile rows 32*kb + b_g + {0,4,8,12,1,5,9,13}.  In each 16-lane
// group the transposing read gives lane i column i of the four rows that
// lanes 4e..4e+3 point at (row b_g + 4e, columns 4c..4c+3 for lane 4e + c).
template <int D>
struct TailReader {
    using PD = Pad<bf16, D>;
    int base;
    __device__ inline void init(int lane) {
        const int g = lane >> 4, j = lane & 15, e = j >> 2, c = j & 3;
        base = (16 * (g & 1) + 2 * (g >> 1) + 4 * e) * PD::PITCH + 4 * c;
    }
    __device__ inline bf16x8 load(const bf16 *tile, int kb, int c0) const {
        typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
        const bf16 *p = tile + base + 32 * kb * PD::PITCH + c0;
        const bf16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)p);
        const bf16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(p + PD::PITCH));
        return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    }
};

// Store 4 consecutive output elements (fp32 values * mul, rounded to T).
template <typename T>
__device__ inline void store4(T *dst, const f32x4 &c, float mul) {
    if constexpr (sizeof(T) == 2) {
        bf16x4 v;
#pragma unroll
        for (int t = 0; t < 4; ++t) v[t] = (bf16)(c[t] * mul);
        *reinterpret_cast<bf16x4 *>(dst) = v;
    } else {
        *reinterpret_cast<f32x4 *>(dst) = f32x4{c[0] * mul, c[1] * mul, c[2] * mul, c[3] * mul};
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

// Reductions over lane pairs (l, l ^ 32): the gfx950 half swap exchanges the
// two 32-lane halves in registers (a shuffle would round-trip through LDS).
// Swapping x with itself leaves each lane its own value and its partner's.
__device__ inline float wave_xor32_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float wave_xor32_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Workgroup order over the (tile, head) pairs of a launch, longest tile first
// (rank 0 = the tile with the most work).  Workgroup i runs on XCD i % 8 (the
// dispatcher deals workgroups to the 8 XCDs in turn; each has its own L2).
// band = 0: consecutive workgroups take consecutive heads.  band > 0 (B*H a
// multiple of 8): XCD x takes only heads x, x + 8, ..., in bands of `band`
// tiles -- the band's tiles of its first head, then the same band of its next
// head, and so on -- so the workgroups in flight on one XCD, which share its
// L2, mostly stream the same head's tiles, while every head's longest tiles
// still start first.  All arguments are wave-uniform.
__device__ inline void tile_order(int bid, int BH, int ntiles, int band, int &rank, int &bh) {
    if (band > 0) {
        const int x = bid & 7, slot = bid >> 3, J = BH >> 3;
        const int full = ntiles / band, per = band * J;  // full bands, slots per full band
        int j, k;
        if (slot < full * per) {
            const int b = slot / per, w = slot - b * per;
            j = w / band;
            k = w - j * band;
            rank = b * band + k;
        } else {  // the last, shorter band
            const int rem = ntiles - full * band, w = slot - full * per;
            j = w / rem;
            k = w - j * rem;
            rank = full * band + k;
        }
        bh = x + 8 * j;
    } else {
        rank = bid / BH;
        bh = bid % BH;
    }
}

}  // namespace fa
