// kd_device.h -- device-side building blocks shared by the gfx950 kernels.
//
// MFMA fragment conventions (CDNA3/CDNA4 16x16 tiles, wave64):
//   * A operand of a 16xK tile: lane l holds row (l % 16) and the K slice of
//     lane group g = l / 16.
//   * B operand of a Kx16 tile: lane l holds column (l % 16) and the K slice
//     of lane group g.
//   * C/D accumulator (floatx4): lane l holds rows 4g + r (r = 0..3) of
//     column (l % 16).
// The order of K inside a contraction is free as long as A and B agree; the
// kernels use two orders:
//   "natural": lane group g holds K = KS*ks + 8g + e (bf16, e < 8) or
//              K = KS*ks + g (fp32);
//   "state"  : the K order in which an fp32 accumulator tile already sits in
//              registers (rows 4g + r), so a state held as accumulators can be
//              fed straight back as a B operand without an LDS transpose.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 halfx8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int CH = 64;        // chunk length (tokens per chunk)
// The Gram tiles of a chunk take their decay relative to the 16-token
// sub-blocks (every operand a product of gates, at most 1).  A diagonal tile
// divides by its sub-block's decay; a key channel whose decay over one
// sub-block falls below this floor (an exact reset f = 0 among them) has its
// diagonal-tile terms computed apart.
constexpr float kSafeFloor = 7.888609052210118e-31f;  // 2^-100
constexpr int SB = 16;        // sub-block edge = MFMA tile edge
constexpr int NSB = CH / SB;  // sub-blocks per chunk

// Workgroup barrier that waits for this wave's LDS traffic only, so global
// prefetch loads stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// A zero the compiler cannot see through: adding it to a per-lane index inside
// a loop keeps the addresses derived from that index from being hoisted out of
// the loop (where they would hold registers across the whole loop).
__device__ __forceinline__ int opaque_zero() {
    int z;
    asm volatile("v_mov_b32 %0, 0" : "=v"(z));
    return z;
}

__device__ __forceinline__ float readlane_f(float x, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

// Maximum over the 64 lanes of a wave of non-negative floats (compared as
// their bit patterns), returned wave-uniform.  DPP quad/mirror steps reduce
// each row of 16 lanes, then the four row maxima are read out as scalars.
#define KD_DPP_UMAX(x, ctrl) max((x), (unsigned)__builtin_amdgcn_mov_dpp((int)(x), (ctrl), 0xf, 0xf, false))
__device__ __forceinline__ float wave_max_nonneg(float v) {
    unsigned x = __float_as_uint(v);
    x = KD_DPP_UMAX(x, 0xB1);    // quad_perm [1,0,3,2]
    x = KD_DPP_UMAX(x, 0x4E);    // quad_perm [2,3,0,1]
    x = KD_DPP_UMAX(x, 0x141);   // row_half_mirror
    x = KD_DPP_UMAX(x, 0x140);   // row_mirror
    const unsigned r0 = (unsigned)__builtin_amdgcn_readlane((int)x, 0);
    const unsigned r1 = (unsigned)__builtin_amdgcn_readlane((int)x, 16);
    const unsigned r2 = (unsigned)__builtin_amdgcn_readlane((int)x, 32);
    const unsigned r3 = (unsigned)__builtin_amdgcn_readlane((int)x, 48);
    return __uint_as_float(max(max(r0, r1), max(r2, r3)));
}
#undef KD_DPP_UMAX

// Sum over the 64 lanes of a wave, returned wave-uniform: DPP steps reduce
// each row of 16 lanes, then the four row sums are read out as scalars and
// added in a fixed order.
#define KD_DPP_FADD(x, ctrl) ((x) + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), (ctrl), 0xf, 0xf, false)))
__device__ __forceinline__ float wave_sum(float x) {
    x = KD_DPP_FADD(x, 0xB1);    // quad_perm [1,0,3,2]
    x = KD_DPP_FADD(x, 0x4E);    // quad_perm [2,3,0,1]
    x = KD_DPP_FADD(x, 0x141);   // row_half_mirror
    x = KD_DPP_FADD(x, 0x140);   // row_mirror
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
    return (r0 + r1) + (r2 + r3);
}
#undef KD_DPP_FADD

// 2^-e for the exponent e of x (x = m 2^e, 0.5 <= m < 1): scales x into
// [0.5, 1).  Returns 1 for x == 0 (or non-finite x).
__device__ __forceinline__ float pow2_scale(float x) {
    if (!(x > 0.f) || !(x < 3.0e38f)) return 1.f;
    return ldexpf(1.f, -__builtin_amdgcn_frexp_expf(x));
}
// The exponent e of pow2_scale(x) = 2^-e (0 where pow2_scale returns 1).
__device__ __forceinline__ int pow2_exp(float x) {
    if (!(x > 0.f) || !(x < 3.0e38f)) return 0;
    return __builtin_amdgcn_frexp_expf(x);
}

// ---------------------------------------------------------------- bf16 path
struct Bf16T {
    typedef __bf16 E;
    typedef bf16x8 Frag;
    static constexpr int KS = 32;     // K per MFMA
    static constexpr int PAD = 8;     // LDS row padding (elements)

    static __device__ __forceinline__ floatx4 mma(Frag a, Frag b, floatx4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ E cvt(float x) { return (__bf16)x; }
    static __device__ __forceinline__ float tof(E x) { return (float)x; }

    // natural-order fragment from a row (K contiguous): K = 32ks + 8g + e
    static __device__ __forceinline__ Frag ld_nat(const E* row, int ks, int g) {
        return *reinterpret_cast<const Frag*>(row + KS * ks + 8 * g);
    }
    // state-order fragment from a row: K = 32ks + {4g..4g+3, 16+4g..16+4g+3}
    static __device__ __forceinline__ Frag ld_state(const E* row, int ks, int g) {
        const E* p = row + KS * ks + 4 * g;
        bf16x4 lo = *reinterpret_cast<const bf16x4*>(p);
        bf16x4 hi = *reinterpret_cast<const bf16x4*>(p + 16);
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    // Column order of the forward's row-major LDS operands: inside every block
    // of 32 columns, column j goes to 8*((j % 16) / 4) + 4*((j / 16) % 2) + j % 4,
    // so the "state" K slice of lane group g is one contiguous 16-byte run.
    // Contractions over j (the Gram tiles) read both operands in this order,
    // which leaves their sums unchanged.
    static __device__ __forceinline__ int pcol(int j) {
        return (j & ~31) | (((j >> 2) & 3) << 3) | (((j >> 4) & 1) << 2) | (j & 3);
    }
    // state-order fragment from a row stored in pcol order
    static __device__ __forceinline__ Frag ld_state_p(const E* row, int ks, int g) {
        return *reinterpret_cast<const Frag*>(row + KS * ks + 8 * g);
    }
    // B operand from accumulator tiles holding X[j][n] (j = 16mt + 4g + r):
    // K-step ks takes tiles 2ks and 2ks+1, already in the "state" K order.
    static __device__ __forceinline__ Frag state_frag(const floatx4* acc, int ks) {
        const floatx4 a = acc[2 * ks];
        const floatx4 b = acc[2 * ks + 1];
        Frag r;
        r[0] = cvt(a[0]); r[1] = cvt(a[1]); r[2] = cvt(a[2]); r[3] = cvt(a[3]);
        r[4] = cvt(b[0]); r[5] = cvt(b[1]); r[6] = cvt(b[2]); r[7] = cvt(b[3]);
        return r;
    }
    // state_frag with each key channel j scaled by s[j]: s is a row of D
    // factors in pcol order, so the fragment's eight channels sit at
    // s[32ks + 8g .. 32ks + 8g + 7]
    static __device__ __forceinline__ Frag state_frag_scaled(const floatx4* acc, int ks, const float* s, int g) {
        const floatx4 a = acc[2 * ks] * *reinterpret_cast<const floatx4*>(s + KS * ks + 8 * g);
        const floatx4 b = acc[2 * ks + 1] * *reinterpret_cast<const floatx4*>(s + KS * ks + 8 * g + 4);
        Frag r;
        r[0] = cvt(a[0]); r[1] = cvt(a[1]); r[2] = cvt(a[2]); r[3] = cvt(a[3]);
        r[4] = cvt(b[0]); r[5] = cvt(b[1]); r[6] = cvt(b[2]); r[7] = cvt(b[3]);
        return r;
    }
    // Column reads of a row-major LDS tile through the transpose read
    // (ds_read_b64_tr_b16).  In each 16-lane block, lanes 4e .. 4e + 3 each
    // name four consecutive elements of row e (together columns c0 .. c0 + 15)
    // and lane j of the block receives column c0 + j of the four rows.  col
    // points at column c0 + cl of the first row (cl = lane % 16, c0 a multiple
    // of 4 and ld a multiple of 4, so every address is 8-byte aligned); every
    // lane of the wave takes part, so callers stay in wave-uniform code.
    static __device__ __forceinline__ s16x4 ld_tr4(const E* col, int ld) {
        const int cl = (int)__lane_id() & 15;
        const E* p = col - cl + (cl >> 2) * ld + 4 * (cl & 3);
        typedef __attribute__((__vector_size__(4 * sizeof(short)))) short v4s;
        return __builtin_bit_cast(s16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                             (__attribute__((address_space(3))) v4s*)(p)));
    }
    // natural-order fragment from a column: K = 32ks + 8g + e at col[K * ld]
    // (a transposed operand read in place: two transpose reads of 4 rows)
    static __device__ __forceinline__ Frag ld_col(const E* col, int ld, int ks, int g) {
        const E* p = col + (KS * ks + 8 * g) * ld;
        const s16x4 lo = ld_tr4(p, ld), hi = ld_tr4(p + 4 * ld, ld);
        return __builtin_bit_cast(Frag, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
    // Column fragments of a row-major matrix without strided loads: B operand
    // with K = rows 32ks .. 32ks + 31 (in the "state" order) and N = columns
    // c0 + cl (c0 a multiple of 16).  Two rows-by-16 tiles pass through the
    // matrix core against a 0/1 selection of the 16 columns (one term per
    // output, so the values are exact); tiles[hh] receives them as
    // accumulators (rows 32ks + 16hh + 4g + r of column c0 + cl).
    static __device__ __forceinline__ Frag col_sel(int c0, int g, int cl) {
        Frag r;
#pragma unroll
        for (int e = 0; e < 8; ++e) r[e] = cvt(8 * g + e == (c0 & 31) + cl ? 1.f : 0.f);
        return r;
    }
    static __device__ __forceinline__ Frag col_frag(const E* m, int ld, int ks, int c0, Frag sel,
                                                    int g, int cl, floatx4* tiles) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
            tiles[hh] = mma(ld_nat(m + (uint32_t)(KS * ks + 16 * hh + cl) * ld + (c0 & ~31), 0, g), sel,
                            floatx4{0.f, 0.f, 0.f, 0.f});
        return state_frag(tiles, 0);
    }
    // A operand along the same K order as col_frag (rows of the contraction)
    static __device__ __forceinline__ Frag ld_colmatch(const E* row, int ks, int g) { return ld_state(row, ks, g); }
    // every element times s (one row or column of an operand scaled)
    static __device__ __forceinline__ Frag scale(Frag x, float s) {
        Frag r;
#pragma unroll
        for (int e = 0; e < 8; ++e) r[e] = cvt(tof(x[e]) * s);
        return r;
    }
    // element e times s * sv[K] for the fragment's K = 32ks + 8g + e
    static __device__ __forceinline__ Frag scale_k(Frag x, float s, const float* sv, int ks, int g) {
        const floatx4 a = *reinterpret_cast<const floatx4*>(sv + KS * ks + 8 * g);
        const floatx4 b = *reinterpret_cast<const floatx4*>(sv + KS * ks + 8 * g + 4);
        Frag r;
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = cvt(tof(x[e]) * (s * a[e]));
#pragma unroll
        for (int e = 0; e < 4; ++e) r[4 + e] = cvt(tof(x[4 + e]) * (s * b[e]));
        return r;
    }
    // Contractions of length 16 (one sub-block): one 16x16x16 MFMA, lane group
    // g holding K = 4g .. 4g + 3.  From a row (K contiguous) or a column (K
    // strided by ld).
    typedef s16x4 F16;
    static __device__ __forceinline__ F16 ld16_row(const E* row, int g) {
        return *reinterpret_cast<const F16*>(row + 4 * g);
    }
    static __device__ __forceinline__ F16 ld16_col(const E* col, int ld, int g) {
        return ld_tr4(col + 4 * g * ld, ld);
    }
    static __device__ __forceinline__ floatx4 mma16(F16 a, F16 b, floatx4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
    }
    // operands that need more than bf16 precision are stored as hi + lo
    static constexpr bool SPLIT = true;
    static __device__ __forceinline__ E lo_part(float x, E hi) { return cvt(x - tof(hi)); }
    // natural-order fragment along K = token index t from a row that is
    // contiguous in t, each element scaled by u[t]
    static __device__ __forceinline__ Frag row_times(const E* row, const float* u, int ks, int g) {
        const int t0 = KS * ks + 8 * g;
        const Frag x = *reinterpret_cast<const Frag*>(row + t0);
        const floatx4 u0 = *reinterpret_cast<const floatx4*>(u + t0);
        const floatx4 u1 = *reinterpret_cast<const floatx4*>(u + t0 + 4);
        Frag r;
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = cvt(u0[e] * tof(x[e]));
#pragma unroll
        for (int e = 0; e < 4; ++e) r[4 + e] = cvt(u1[e] * tof(x[4 + e]));
        return r;
    }

    // State update operands in fp16 (11-bit mantissa; values pre-scaled by
    // exact powers of two so they stay inside fp16's range).
    typedef _Float16 H;
    typedef halfx8 FragH;
    static __device__ __forceinline__ floatx4 mma_h(FragH a, FragH b, floatx4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ FragH ld_nat_h(const H* row, int ks, int g) {
        return *reinterpret_cast<const FragH*>(row + KS * ks + 8 * g);
    }
    static __device__ __forceinline__ FragH row_times_h(const E* row, const float* u, float su,
                                                        int ks, int g) {
        const int t0 = KS * ks + 8 * g;
        const Frag x = *reinterpret_cast<const Frag*>(row + t0);
        const floatx4 u0 = *reinterpret_cast<const floatx4*>(u + t0);
        const floatx4 u1 = *reinterpret_cast<const floatx4*>(u + t0 + 4);
        FragH r;
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = (_Float16)((u0[e] * su) * tof(x[e]));
#pragma unroll
        for (int e = 0; e < 4; ++e) r[4 + e] = (_Float16)((u1[e] * su) * tof(x[4 + e]));
        return r;
    }
    // row_times (bf16) and row_times_h (fp16, u scaled by su) from one read of
    // the row and of u
    static __device__ __forceinline__ void row_times_both(const E* row, const float* u, float su, int ks,
                                                          int g, Frag& wa, FragH& wb) {
        const int t0 = KS * ks + 8 * g;
        const Frag x = *reinterpret_cast<const Frag*>(row + t0);
        const floatx4 u0 = *reinterpret_cast<const floatx4*>(u + t0);
        const floatx4 u1 = *reinterpret_cast<const floatx4*>(u + t0 + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            wa[e] = cvt(u0[e] * tof(x[e]));
            wa[4 + e] = cvt(u1[e] * tof(x[4 + e]));
            wb[e] = (_Float16)((u0[e] * su) * tof(x[e]));
            wb[4 + e] = (_Float16)((u1[e] * su) * tof(x[4 + e]));
        }
    }
    // bf16 ua[t] x[t] and fp16 ub[t] x[t] from one read of the row
    static __device__ __forceinline__ void row_times_pair(const E* row, const float* ua, const float* ub,
                                                          int ks, int g, Frag& wa, FragH& wb) {
        const int t0 = KS * ks + 8 * g;
        const Frag x = *reinterpret_cast<const Frag*>(row + t0);
        const floatx4 a0 = *reinterpret_cast<const floatx4*>(ua + t0);
        const floatx4 a1 = *reinterpret_cast<const floatx4*>(ua + t0 + 4);
        const floatx4 b0 = *reinterpret_cast<const floatx4*>(ub + t0);
        const floatx4 b1 = *reinterpret_cast<const floatx4*>(ub + t0 + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            wa[e] = cvt(a0[e] * tof(x[e]));
            wa[4 + e] = cvt(a1[e] * tof(x[4 + e]));
            wb[e] = (_Float16)(b0[e] * tof(x[e]));
            wb[4 + e] = (_Float16)(b1[e] * tof(x[4 + e]));
        }
    }
    // the same for two rows sharing one scaled slice of u
    static __device__ __forceinline__ void rows_times_h2(const E* row0, const E* row1, const float* u,
                                                         float su, int ks, int g, FragH& r0, FragH& r1) {
        const int t0 = KS * ks + 8 * g;
        const Frag x0 = *reinterpret_cast<const Frag*>(row0 + t0);
        const Frag x1 = *reinterpret_cast<const Frag*>(row1 + t0);
        const floatx4 u0 = *reinterpret_cast<const floatx4*>(u + t0) * su;
        const floatx4 u1 = *reinterpret_cast<const floatx4*>(u + t0 + 4) * su;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            r0[e] = (_Float16)(u0[e] * tof(x0[e]));
            r1[e] = (_Float16)(u0[e] * tof(x1[e]));
            r0[4 + e] = (_Float16)(u1[e] * tof(x0[4 + e]));
            r1[4 + e] = (_Float16)(u1[e] * tof(x1[4 + e]));
        }
    }
};

// ---------------------------------------------------------------- fp32 path
struct F32T {
    typedef float E;
    typedef float Frag;
    static constexpr int KS = 4;
    static constexpr int PAD = 4;

    static __device__ __forceinline__ floatx4 mma(Frag a, Frag b, floatx4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ E cvt(float x) { return x; }
    static __device__ __forceinline__ float tof(E x) { return x; }

    static __device__ __forceinline__ Frag ld_nat(const E* row, int ks, int g) {
        return row[KS * ks + g];
    }
    // state order: step ks covers accumulator tile ks/4, register ks%4
    static __device__ __forceinline__ Frag ld_state(const E* row, int ks, int g) {
        return row[16 * (ks >> 2) + 4 * g + (ks & 3)];
    }
    // fp32 fragments are single elements: no column permutation
    static __device__ __forceinline__ int pcol(int j) { return j; }
    static __device__ __forceinline__ Frag ld_state_p(const E* row, int ks, int g) { return ld_state(row, ks, g); }
    static __device__ __forceinline__ Frag state_frag(const floatx4* acc, int ks) {
        return acc[ks >> 2][ks & 3];
    }
    // key channel j = 16 (ks / 4) + 4g + ks % 4 scaled by s[j] (no column
    // permutation for fp32)
    static __device__ __forceinline__ Frag state_frag_scaled(const floatx4* acc, int ks, const float* s, int g) {
        return acc[ks >> 2][ks & 3] * s[16 * (ks >> 2) + 4 * g + (ks & 3)];
    }
    static __device__ __forceinline__ Frag ld_col(const E* col, int ld, int ks, int g) {
        return col[(KS * ks + g) * ld];
    }
    // fp32: one element per lane and K-step, read in place
    static __device__ __forceinline__ Frag col_sel(int, int, int) { return 0.f; }
    static __device__ __forceinline__ Frag col_frag(const E* m, int ld, int ks, int c0, Frag, int g, int cl,
                                                    floatx4*) {
        return m[(uint32_t)(KS * ks + g) * ld + c0 + cl];
    }
    static __device__ __forceinline__ Frag ld_colmatch(const E* row, int ks, int g) { return ld_nat(row, ks, g); }
    static __device__ __forceinline__ Frag scale(Frag x, float s) { return x * s; }
    static __device__ __forceinline__ Frag scale_k(Frag x, float s, const float* sv, int ks, int g) {
        return x * (s * sv[KS * ks + g]);
    }
    // Contractions of length 16: four 16x16x4 MFMAs, step e taking K = 4e + g.
    typedef floatx4 F16;
    static __device__ __forceinline__ F16 ld16_row(const E* row, int g) {
        return F16{row[g], row[4 + g], row[8 + g], row[12 + g]};
    }
    static __device__ __forceinline__ F16 ld16_col(const E* col, int ld, int g) {
        return F16{col[g * ld], col[(4 + g) * ld], col[(8 + g) * ld], col[(12 + g) * ld]};
    }
    static __device__ __forceinline__ floatx4 mma16(F16 a, F16 b, floatx4 c) {
#pragma unroll
        for (int e = 0; e < 4; ++e) c = mma(a[e], b[e], c);
        return c;
    }
    static constexpr bool SPLIT = false;
    static __device__ __forceinline__ E lo_part(float, E) { return 0.f; }
    static __device__ __forceinline__ Frag row_times(const E* row, const float* u, int ks, int g) {
        const int t = KS * ks + g;
        return u[t] * row[t];
    }
    typedef float H;
    typedef float FragH;
    static __device__ __forceinline__ floatx4 mma_h(FragH a, FragH b, floatx4 c) { return mma(a, b, c); }
    static __device__ __forceinline__ FragH ld_nat_h(const H* row, int ks, int g) { return ld_nat(row, ks, g); }
    static __device__ __forceinline__ FragH row_times_h(const E* row, const float* u, float su,
                                                        int ks, int g) {
        const int t = KS * ks + g;
        return (u[t] * su) * row[t];
    }
    static __device__ __forceinline__ void rows_times_h2(const E* row0, const E* row1, const float* u,
                                                         float su, int ks, int g, FragH& r0, FragH& r1) {
        const int t = KS * ks + g;
        const float us = u[t] * su;
        r0 = us * row0[t];
        r1 = us * row1[t];
    }
};

// Two consecutive tokens of eight adjacent channels (16-byte aligned group
// ch0 .. ch0 + 7), held in registers between the global load and its use
// (the prefetch buffer).  One 16-byte load per row for bf16.
template <class TR> struct Row2x8;

template <> struct Row2x8<Bf16T> {
    uint4 w[2];   // row e, channels 2i (low half) and 2i + 1 (high half) in w[e][i]
    // p: wave-uniform base; row e at element offset off_e (32-bit).
    __device__ __forceinline__ void load(const __bf16* p, uint32_t off0, uint32_t off1) {
        const char* base = reinterpret_cast<const char*>(p);
        w[0] = *reinterpret_cast<const uint4*>(base + off0 * 2u);
        w[1] = *reinterpret_cast<const uint4*>(base + off1 * 2u);
    }
    __device__ __forceinline__ uint32_t word(int e, int i) const {
        return i == 0 ? w[e].x : i == 1 ? w[e].y : i == 2 ? w[e].z : w[e].w;
    }
    __device__ __forceinline__ float get(int e, int c) const {
        const uint32_t x = word(e, c >> 1);
        return __uint_as_float((c & 1) ? (x & 0xffff0000u) : (x << 16));
    }
    // row e becomes `fill` (0 or 1; exact in bf16)
    __device__ __forceinline__ void clear(int e, float fill) {
        const uint32_t fb = __float_as_uint(fill) >> 16;
        const uint32_t x = fb | (fb << 16);
        w[e] = make_uint4(x, x, x, x);
    }
    __device__ __forceinline__ void store(__bf16* dst, int e) const {
        *reinterpret_cast<uint4*>(dst) = w[e];
    }
};

template <> struct Row2x8<F32T> {
    floatx4 w[2][2];
    __device__ __forceinline__ void load(const float* p, uint32_t off0, uint32_t off1) {
        const char* base = reinterpret_cast<const char*>(p);
        w[0][0] = *reinterpret_cast<const floatx4*>(base + off0 * 4u);
        w[0][1] = *reinterpret_cast<const floatx4*>(base + off0 * 4u + 16u);
        w[1][0] = *reinterpret_cast<const floatx4*>(base + off1 * 4u);
        w[1][1] = *reinterpret_cast<const floatx4*>(base + off1 * 4u + 16u);
    }
    __device__ __forceinline__ float get(int e, int c) const { return w[e][c >> 2][c & 3]; }
    __device__ __forceinline__ void clear(int e, float fill) {
        w[e][0] = floatx4{fill, fill, fill, fill};
        w[e][1] = w[e][0];
    }
    __device__ __forceinline__ void store(float* dst, int e) const {
        reinterpret_cast<floatx4*>(dst)[0] = w[e][0];
        reinterpret_cast<floatx4*>(dst)[1] = w[e][1];
    }
};

// Products over the eight lanes l & 7 = 0..7 of each aligned 8-lane group:
// inclusive prefix product of x in lane order (DPP row shifts, masked at the
// group boundary).
template <int S>
__device__ __forceinline__ float dpp_row_shr(float x) {   // lane i <- lane i-S of its 16-lane row (1 if none)
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(1.f), __float_as_int(x),
                                                      0x110 + S, 0xf, 0xf, false));
}
__device__ __forceinline__ float group8_prefix_prod(float x, int r8) {
    float y = dpp_row_shr<1>(x);
    x = (r8 >= 1) ? x * y : x;
    y = dpp_row_shr<2>(x);
    x = (r8 >= 2) ? x * y : x;
    y = dpp_row_shr<4>(x);
    x = (r8 >= 4) ? x * y : x;
    return x;
}
// Value of x in the previous lane of the 8-lane group (1 for the first lane).
__device__ __forceinline__ float group8_shift1(float x, int r8) {
    const float y = dpp_row_shr<1>(x);
    return r8 >= 1 ? y : 1.f;
}
// Sums over the same 8-lane groups in reverse lane order.  Every DPP move is
// issued by all lanes before the lane-dependent select.
template <int S>
__device__ __forceinline__ float dpp_row_shl0(float x) {   // lane i <- lane i+S of its 16-lane row (0 if none)
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x100 + S, 0xf, 0xf, false));
}
// inclusive suffix sum: lanes r8 .. 7 of the group
__device__ __forceinline__ float group8_suffix_sum(float x, int r8) {
    float y = dpp_row_shl0<1>(x);
    x = (r8 <= 6) ? x + y : x;
    y = dpp_row_shl0<2>(x);
    x = (r8 <= 5) ? x + y : x;
    y = dpp_row_shl0<4>(x);
    x = (r8 <= 3) ? x + y : x;
    return x;
}
// product over the lanes after this one in its aligned 8-lane group (1 for
// the last lane): the exclusive suffix product
template <int S>
__device__ __forceinline__ float dpp_row_shl1(float x) {   // lane i <- lane i+S of its 16-lane row (1 if none)
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(1.f), __float_as_int(x), 0x100 + S, 0xf, 0xf, false));
}
__device__ __forceinline__ float group8_excl_suffix_prod(float x, int r8) {
    float y = dpp_row_shl1<1>(x);
    x = (r8 <= 6) ? x * y : x;        // lanes r8 .. r8+1
    y = dpp_row_shl1<2>(x);
    x = (r8 <= 5) ? x * y : x;        // r8 .. r8+3
    y = dpp_row_shl1<4>(x);
    x = (r8 <= 3) ? x * y : x;        // r8 .. 7: inclusive suffix
    y = dpp_row_shl1<1>(x);
    return r8 <= 6 ? y : 1.f;
}
// value of x in the next lane of the group (0 for the last lane)
__device__ __forceinline__ float group8_next1(float x, int r8) {
    const float y = dpp_row_shl0<1>(x);
    return r8 <= 6 ? y : 0.f;
}

// Element order of the per-chunk state records of bf16 runs (the entering
// state S0 and the state gradient dS of every chunk, D x D, D a multiple of
// 32): blocks of 16 rows i by 32 columns j, each block 64 runs of eight
// elements; run g * 16 + i % 16 holds row i's columns 4g .. 4g + 3 and
// 16 + 4g .. 16 + 4g + 3 of the block.  That is the order in which an MFMA
// accumulator lane holds a row of the state (tiles 2kb and 2kb + 1, rows
// 4g .. 4g + 3 of each), so a writer's lane stores its values as 16-byte runs
// and one store instruction covers 1 KB.  rec_run: element offset of a run.
template <int D>
__device__ __forceinline__ uint32_t rec_run(int i, int kb, int g) {
    return ((uint32_t)((i >> 4) * (D / 32) + kb) * 64u + (uint32_t)(g * 16 + (i & 15))) * 8u;
}
template <int D>
__device__ __forceinline__ uint32_t rec_idx(int i, int j) {
    return rec_run<D>(i, j >> 5, (j >> 2) & 3) + (uint32_t)((((j >> 4) & 1) << 2) | (j & 3));
}
// One run from two accumulator tiles (times s): elements 0 .. 3 from a, 4 .. 7 from b.
__device__ __forceinline__ void st_run_nt(__bf16* p, floatx4 a, floatx4 b, float s) {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) { r[e] = (__bf16)(a[e] * s); r[4 + e] = (__bf16)(b[e] * s); }
    __builtin_nontemporal_store(__builtin_bit_cast(floatx4, r), reinterpret_cast<floatx4*>(p));
}
__device__ __forceinline__ void st_run(__bf16* p, floatx4 a, floatx4 b) {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) { r[e] = (__bf16)a[e]; r[4 + e] = (__bf16)b[e]; }
    *reinterpret_cast<bf16x8*>(p) = r;
}

// Store eight values as one 16-byte row segment.
__device__ __forceinline__ void st8v(__bf16* p, const float* x) {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (__bf16)x[e];
    *reinterpret_cast<bf16x8*>(p) = r;
}
__device__ __forceinline__ void st8v(float* p, const float* x) {
    reinterpret_cast<floatx4*>(p)[0] = floatx4{x[0], x[1], x[2], x[3]};
    reinterpret_cast<floatx4*>(p)[1] = floatx4{x[4], x[5], x[6], x[7]};
}
// the same as streaming stores (outputs no kernel of the launch reads back)
__device__ __forceinline__ void st8v_nt(__bf16* p, const float* x) {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (__bf16)x[e];
    __builtin_nontemporal_store(__builtin_bit_cast(floatx4, r), reinterpret_cast<floatx4*>(p));
}
__device__ __forceinline__ void st8v_nt(float* p, const float* x) {
    __builtin_nontemporal_store(floatx4{x[0], x[1], x[2], x[3]}, reinterpret_cast<floatx4*>(p));
    __builtin_nontemporal_store(floatx4{x[4], x[5], x[6], x[7]}, reinterpret_cast<floatx4*>(p) + 1);
}
// Two adjacent values of one row as a streaming store.
__device__ __forceinline__ void st2_nt(__bf16* p, float a, float b) {
    const __bf16 __attribute__((ext_vector_type(2))) r = {(__bf16)a, (__bf16)b};
    __builtin_nontemporal_store(__builtin_bit_cast(unsigned, r), reinterpret_cast<unsigned*>(p));
}
__device__ __forceinline__ void st2_nt(float* p, float a, float b) {
    typedef float f2v __attribute__((ext_vector_type(2)));
    __builtin_nontemporal_store(f2v{a, b}, reinterpret_cast<f2v*>(p));
}
// Store two consecutive values (a transposed-array entry pair).
__device__ __forceinline__ void st2h(_Float16* p, float a, float b) {
    _Float16 __attribute__((ext_vector_type(2))) x;
    x[0] = (_Float16)a;
    x[1] = (_Float16)b;
    *reinterpret_cast<decltype(x)*>(p) = x;
}
__device__ __forceinline__ void st2h(float* p, float a, float b) {
    *reinterpret_cast<float2*>(p) = make_float2(a, b);
}

// Four consecutive tokens of eight adjacent channels (16-byte aligned group
// ch0 .. ch0 + 7): the producer's prefetch buffer.  One 16-byte load per row
// for bf16.
template <class TR> struct Raw4x8;

template <> struct Raw4x8<Bf16T> {
    uint4 w[4];   // row e: channels 2i (low half) and 2i + 1 (high half) in word i
    // p: wave-uniform base; row e at 32-bit element offset off + min(e, last)*stride.
    __device__ __forceinline__ void load(const __bf16* p, uint32_t off, uint32_t stride, int last) {
        const char* base = reinterpret_cast<const char*>(p);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            w[e] = *reinterpret_cast<const uint4*>(base + (off + (uint32_t)(e < last ? e : last) * stride) * 2u);
    }
    __device__ __forceinline__ uint32_t word(int e, int i) const {
        return i == 0 ? w[e].x : i == 1 ? w[e].y : i == 2 ? w[e].z : w[e].w;
    }
    __device__ __forceinline__ float get(int e, int c) const {
        const uint32_t x = word(e, c >> 1);
        return __uint_as_float((c & 1) ? (x & 0xffff0000u) : (x << 16));
    }
    __device__ __forceinline__ void clear(int e, float fill) {
        const uint32_t fb = __float_as_uint(fill) >> 16;
        const uint32_t x = fb | (fb << 16);
        w[e] = make_uint4(x, x, x, x);
    }
    __device__ __forceinline__ void store(__bf16* dst, int e) const {
        *reinterpret_cast<uint4*>(dst) = w[e];
    }
};

template <> struct Raw4x8<F32T> {
    floatx4 w[4][2];
    __device__ __forceinline__ void load(const float* p, uint32_t off, uint32_t stride, int last) {
        const char* base = reinterpret_cast<const char*>(p);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t b = (off + (uint32_t)(e < last ? e : last) * stride) * 4u;
            w[e][0] = *reinterpret_cast<const floatx4*>(base + b);
            w[e][1] = *reinterpret_cast<const floatx4*>(base + b + 16u);
        }
    }
    __device__ __forceinline__ float get(int e, int c) const { return w[e][c >> 2][c & 3]; }
    __device__ __forceinline__ void clear(int e, float fill) {
        w[e][0] = floatx4{fill, fill, fill, fill};
        w[e][1] = w[e][0];
    }
    __device__ __forceinline__ void store(float* dst, int e) const {
        reinterpret_cast<floatx4*>(dst)[0] = w[e][0];
        reinterpret_cast<floatx4*>(dst)[1] = w[e][1];
    }
};

// Sixteen consecutive tokens (one sub-block) of two adjacent channels ch0,
// ch0 + 1: the producer's prefetch buffer.  One 4-byte load per row for bf16
// (8-byte for fp32); the lanes of a wave cover adjacent channel pairs, so every
// load instruction reads whole rows.
template <class TR> struct Raw16x2;

template <> struct Raw16x2<Bf16T> {
    uint32_t w[16];   // row e: channel ch0 in the low half, ch0 + 1 in the high half
    // p: wave-uniform base; row e at 32-bit element offset off + min(e, last)*stride.
    __device__ __forceinline__ void load(const __bf16* p, uint32_t off, uint32_t stride, int last) {
        const char* base = reinterpret_cast<const char*>(p);
#pragma unroll
        for (int e = 0; e < 16; ++e)
            w[e] = *reinterpret_cast<const uint32_t*>(base + (off + (uint32_t)(e < last ? e : last) * stride) * 2u);
    }
    __device__ __forceinline__ float get(int e, int cc) const {
        return __uint_as_float(cc ? (w[e] & 0xffff0000u) : (w[e] << 16));
    }
    __device__ __forceinline__ void clear(int e, float fill) {
        const uint32_t fb = __float_as_uint(fill) >> 16;
        w[e] = fb | (fb << 16);
    }
    __device__ __forceinline__ void store(__bf16* dst, int e) const { *reinterpret_cast<uint32_t*>(dst) = w[e]; }
    // max |x| over the 32 values
    __device__ __forceinline__ float absmax() const {
        typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
        u16x2 m = {0, 0};
#pragma unroll
        for (int e = 0; e < 16; ++e)   // bf16 magnitudes order like unsigned integers
            m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w[e] & 0x7fff7fffu));
        const uint32_t hi = m[0] > m[1] ? m[0] : m[1];
        return __uint_as_float(hi << 16);
    }
};

template <> struct Raw16x2<F32T> {
    float2 w[16];
    __device__ __forceinline__ void load(const float* p, uint32_t off, uint32_t stride, int last) {
        const char* base = reinterpret_cast<const char*>(p);
#pragma unroll
        for (int e = 0; e < 16; ++e)
            w[e] = *reinterpret_cast<const float2*>(base + (off + (uint32_t)(e < last ? e : last) * stride) * 4u);
    }
    __device__ __forceinline__ float get(int e, int cc) const { return cc ? w[e].y : w[e].x; }
    __device__ __forceinline__ void clear(int e, float fill) { w[e] = make_float2(fill, fill); }
    __device__ __forceinline__ void store(float* dst, int e) const { *reinterpret_cast<float2*>(dst) = w[e]; }
    __device__ __forceinline__ float absmax() const {
        float m = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) m = fmaxf(m, fmaxf(fabsf(w[e].x), fabsf(w[e].y)));
        return m;
    }
};

// Sixteen consecutive tokens of one channel, kept from the producer's prep
// until they are written as one transposed entry (32 bytes for bf16 and fp16,
// 64 bytes for fp32).
template <class T> struct Col16;
template <> struct Col16<__bf16> {
    uint32_t w[8];
    __device__ __forceinline__ void set_raw(const Raw16x2<Bf16T>& r, int cc) {
        const uint32_t sel = cc ? 0x07060302u : 0x05040100u;
#pragma unroll
        for (int k = 0; k < 8; ++k) w[k] = __builtin_amdgcn_perm(r.w[2 * k + 1], r.w[2 * k], sel);
    }
    __device__ __forceinline__ void store(__bf16* p) const {
        reinterpret_cast<uint4*>(p)[0] = make_uint4(w[0], w[1], w[2], w[3]);
        reinterpret_cast<uint4*>(p)[1] = make_uint4(w[4], w[5], w[6], w[7]);
    }
};
template <> struct Col16<_Float16> {
    uint32_t w[8];
    __device__ __forceinline__ void set_pair(int k, float a, float b) {
        _Float16 __attribute__((ext_vector_type(2))) x;
        x[0] = (_Float16)a;
        x[1] = (_Float16)b;
        w[k] = __builtin_bit_cast(uint32_t, x);
    }
    __device__ __forceinline__ void store(_Float16* p) const {
        reinterpret_cast<uint4*>(p)[0] = make_uint4(w[0], w[1], w[2], w[3]);
        reinterpret_cast<uint4*>(p)[1] = make_uint4(w[4], w[5], w[6], w[7]);
    }
};
template <> struct Col16<float> {
    float w[16];
    __device__ __forceinline__ void set_raw(const Raw16x2<F32T>& r, int cc) {
#pragma unroll
        for (int e = 0; e < 16; ++e) w[e] = r.get(e, cc);
    }
    __device__ __forceinline__ void set_pair(int k, float a, float b) { w[2 * k] = a; w[2 * k + 1] = b; }
    __device__ __forceinline__ void store(float* p) const {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            reinterpret_cast<floatx4*>(p)[k] = floatx4{w[4 * k], w[4 * k + 1], w[4 * k + 2], w[4 * k + 3]};
    }
};

// Eight consecutive tokens of two adjacent channels ch0, ch0 + 1 (bf16): one
// 4-byte load per row, so a wave whose lanes cover adjacent channel pairs
// reads whole rows.
// The mixer's gates (KronLSTM summary page, section on how the rule is used):
// sigmoid(x) = 1 / (1 + 2^(-x log2 e)), and the forget gate
// sigmoid(x)^a = 2^(-a log2(1 + 2^(-x log2 e))), on the hardware base-2 exp,
// log and reciprocal.  Large negative x gives 1 + inf, so the gate is exactly
// 0; large positive x gives log2(1) = 0, a gate within fp32's spacing of 1.
// The pre-processing kernel and the forward's fused gates share these, so
// both give the same bits.
constexpr float kLog2e = 1.4426950408889634f;
template <int CTRL>
__device__ __forceinline__ float mix_dpp(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}
// sum over the LPR adjacent lanes of a row (LPR in {4, 8, 16}, rows aligned
// to LPR lanes), on DPP lane moves: the partner quad lane, the other quad of
// the 8-lane half row (half-row mirror), the other half of the 16-lane row
// (row mirror)
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
    static_assert(LPR == 4 || LPR == 8 || LPR == 16, "rows of 4, 8 or 16 lanes");
    x += mix_dpp<0xB1>(x);                   // quad_perm(1, 0, 3, 2): lane ^ 1
    x += mix_dpp<0x4E>(x);                   // quad_perm(2, 3, 0, 1): lane ^ 2
    if (LPR >= 8) x += mix_dpp<0x141>(x);    // row_half_mirror
    if (LPR >= 16) x += mix_dpp<0x140>(x);   // row_mirror
    return x;
}

__device__ __forceinline__ float gate_sigmoid(float x) {
    return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-kLog2e * x));
}
__device__ __forceinline__ float forget_gate(float x, float a) {
    return __builtin_amdgcn_exp2f(-a * __builtin_amdgcn_logf(1.f + __builtin_amdgcn_exp2f(-kLog2e * x)));
}

struct Raw8x2 {
    uint32_t w[8];   // row e: channel ch0 in the low half, ch0 + 1 in the high half
    // p: wave-uniform base; row e at 32-bit element offset off + min(e, last)*stride.
    __device__ __forceinline__ void load(const __bf16* p, uint32_t off, uint32_t stride, int last) {
        const char* base = reinterpret_cast<const char*>(p);
#pragma unroll
        for (int e = 0; e < 8; ++e)
            w[e] = *reinterpret_cast<const uint32_t*>(base + (off + (uint32_t)(e < last ? e : last) * stride) * 2u);
    }
    __device__ __forceinline__ float get(int e, int cc) const {
        return __uint_as_float(cc ? (w[e] & 0xffff0000u) : (w[e] << 16));
    }
    __device__ __forceinline__ void clear(int e, float fill) {
        const uint32_t fb = __float_as_uint(fill) >> 16;
        w[e] = fb | (fb << 16);
    }
    __device__ __forceinline__ void store(__bf16* dst, int e) const { *reinterpret_cast<uint32_t*>(dst) = w[e]; }
    // every value x replaced by fn(x), rounded to bf16 (nearest even)
    template <class F>
    __device__ __forceinline__ void map(F fn) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            bf16x2 r;
            r[0] = (__bf16)fn(get(e, 0));
            r[1] = (__bf16)fn(get(e, 1));
            w[e] = __builtin_bit_cast(uint32_t, r);
        }
    }
    // max |x| over the 16 values
    __device__ __forceinline__ float absmax() const {
        typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
        u16x2 m = {0, 0};
#pragma unroll
        for (int e = 0; e < 8; ++e)   // bf16 magnitudes order like unsigned integers
            m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, w[e] & 0x7fff7fffu));
        const uint32_t hi = m[0] > m[1] ? m[0] : m[1];
        return __uint_as_float(hi << 16);
    }
};

// Eight consecutive tokens of one channel (16 bytes), written as one
// transposed entry.
struct Col8 {
    uint32_t w[4];
    // channel cc of raw rows, taken as 16-bit halves of the loaded words
    __device__ __forceinline__ void set_raw(const Raw8x2& r, int cc) {
        const uint32_t sel = cc ? 0x07060302u : 0x05040100u;
#pragma unroll
        for (int k = 0; k < 4; ++k) w[k] = __builtin_amdgcn_perm(r.w[2 * k + 1], r.w[2 * k], sel);
    }
    // tokens 2k, 2k + 1 as fp16
    __device__ __forceinline__ void set_pair_h(int k, float a, float b) {
        _Float16 __attribute__((ext_vector_type(2))) x;
        x[0] = (_Float16)a;
        x[1] = (_Float16)b;
        w[k] = __builtin_bit_cast(uint32_t, x);
    }
    __device__ __forceinline__ void store(void* p) const {
        *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
    }
};

// max |x| over the 32 values of four raw rows, as a float.
__device__ __forceinline__ float raw_absmax(const Raw4x8<Bf16T>& r) {
    typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
    u16x2 m = {0, 0};
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int i = 0; i < 4; ++i)   // bf16 magnitudes order like unsigned integers
            m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, r.word(e, i) & 0x7fff7fffu));
    const uint32_t hi = m[0] > m[1] ? m[0] : m[1];
    return __uint_as_float(hi << 16);
}
__device__ __forceinline__ float raw_absmax(const Raw4x8<F32T>& r) {
    float m = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int c = 0; c < 8; ++c) m = fmaxf(m, fabsf(r.get(e, c)));
    return m;
}

// Four consecutive values of one channel, held from the producer's prep until
// they are written as one 8-byte (bf16/fp16) or 16-byte (fp32) transposed
// entry.
template <class T> struct Col4;
template <> struct Col4<__bf16> {
    uint32_t w[2];
    __device__ __forceinline__ void set(const float* x) {
        bf16x2 a, b;
        a[0] = (__bf16)x[0]; a[1] = (__bf16)x[1];
        b[0] = (__bf16)x[2]; b[1] = (__bf16)x[3];
        w[0] = __builtin_bit_cast(uint32_t, a);
        w[1] = __builtin_bit_cast(uint32_t, b);
    }
    __device__ __forceinline__ void store(__bf16* p) const { *reinterpret_cast<uint2*>(p) = make_uint2(w[0], w[1]); }
    // channel c of four raw rows, taken as 16-bit halves of the loaded words
    __device__ __forceinline__ void set_raw(const Raw4x8<Bf16T>& r, int c) {
        const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
        w[0] = __builtin_amdgcn_perm(r.word(1, c >> 1), r.word(0, c >> 1), sel);
        w[1] = __builtin_amdgcn_perm(r.word(3, c >> 1), r.word(2, c >> 1), sel);
    }
};
template <> struct Col4<_Float16> {
    uint32_t w[2];
    __device__ __forceinline__ void set(const float* x) {
        _Float16 __attribute__((ext_vector_type(2))) a, b;
        a[0] = (_Float16)x[0]; a[1] = (_Float16)x[1];
        b[0] = (_Float16)x[2]; b[1] = (_Float16)x[3];
        w[0] = __builtin_bit_cast(uint32_t, a);
        w[1] = __builtin_bit_cast(uint32_t, b);
    }
    __device__ __forceinline__ void store(_Float16* p) const { *reinterpret_cast<uint2*>(p) = make_uint2(w[0], w[1]); }
};
template <> struct Col4<float> {
    floatx4 w;
    __device__ __forceinline__ void set(const float* x) { w = floatx4{x[0], x[1], x[2], x[3]}; }
    __device__ __forceinline__ void set_raw(const Raw4x8<F32T>& r, int c) {
        w = floatx4{r.get(0, c), r.get(1, c), r.get(2, c), r.get(3, c)};
    }
    __device__ __forceinline__ void store(float* p) const { *reinterpret_cast<floatx4*>(p) = w; }
};

// Store four consecutive fp32 values in the path's element type.
__device__ __forceinline__ void st4(__bf16* p, floatx4 x) {
    bf16x4 r;
    r[0] = (__bf16)x[0]; r[1] = (__bf16)x[1]; r[2] = (__bf16)x[2]; r[3] = (__bf16)x[3];
    *reinterpret_cast<bf16x4*>(p) = r;
}
__device__ __forceinline__ void st4(float* p, floatx4 x) { *reinterpret_cast<floatx4*>(p) = x; }
// The same as a non-temporal (streaming) store: for outputs no kernel of the
// launch reads back, so they do not take cache space from the inputs still
// to be read.
__device__ __forceinline__ void st4_nt(__bf16* p, floatx4 x) {
    bf16x4 r;
    r[0] = (__bf16)x[0]; r[1] = (__bf16)x[1]; r[2] = (__bf16)x[2]; r[3] = (__bf16)x[3];
    __builtin_nontemporal_store(__builtin_bit_cast(unsigned long long, r), reinterpret_cast<unsigned long long*>(p));
}
__device__ __forceinline__ void st4_nt(float* p, floatx4 x) {
    __builtin_nontemporal_store(x, reinterpret_cast<floatx4*>(p));
}
__device__ __forceinline__ void st_nt(float* p, float x) { __builtin_nontemporal_store(x, p); }
// 16-byte copy, streaming store
__device__ __forceinline__ void cp16_nt(void* dst, const void* src) {
    __builtin_nontemporal_store(*reinterpret_cast<const floatx4*>(src), reinterpret_cast<floatx4*>(dst));
}

// Quad (4-lane group) scans of products, r4 = lane & 3.
template <int CTRL>
__device__ __forceinline__ float dpp_quad(float x) {
    // a quad permutation always has a source lane, so no "old" value is needed
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}
// exclusive prefix product (product over lanes r' < r4; 1 for r4 = 0) and the
// exclusive suffix product (product over lanes r' > r4; 1 for r4 = 3)
// Every DPP move is issued by all four lanes before any lane-dependent select:
// a move placed under a condition becomes a branch, and a lane masked off by
// that branch cannot be read.
__device__ __forceinline__ void quad_excl_prod(float x, int r4, float& pre, float& suf) {
    const float x1 = dpp_quad<0x90>(x);                  // quad_perm [0,0,1,2]
    const float y1 = dpp_quad<0xF9>(x);                  // quad_perm [1,2,3,3]
    const float a1 = (r4 >= 1) ? x * x1 : x;             // product of lanes r4-1 .. r4
    const float b1 = (r4 <= 2) ? x * y1 : x;             // product of lanes r4 .. r4+1
    const float x2 = dpp_quad<0x40>(a1);                 // quad_perm [0,0,0,1]
    const float y2 = dpp_quad<0xFE>(b1);                 // quad_perm [2,3,3,3]
    const float a2 = (r4 >= 2) ? a1 * x2 : a1;           // inclusive prefix
    const float b2 = (r4 <= 1) ? b1 * y2 : b1;           // inclusive suffix
    const float x3 = dpp_quad<0x90>(a2);
    const float y3 = dpp_quad<0xF9>(b2);
    pre = (r4 >= 1) ? x3 : 1.f;
    suf = (r4 <= 2) ? y3 : 1.f;
}

// The sum over the 16 lanes of a DPP row, in every lane of the row, as the
// butterfly over lane ^ 1, ^ 2, ^ 4, ^ 8.  The last two partners come from the
// half-row and row mirrors: at that point they hold the same partial sums as
// lane ^ 4 and lane ^ 8, so every addition has the butterfly's operands.
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp_quad<0xB1>(x);   // quad_perm [1,0,3,2]: lane ^ 1
    x += dpp_quad<0x4E>(x);   // quad_perm [2,3,0,1]: lane ^ 2
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xf, 0xf, false));   // half-row mirror
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xf, 0xf, false));   // row mirror
    return x;
}

// One step of a transpose-reduce over the 16 lanes of a DPP row: x[0 .. 2M)
// of every lane are summed in pairs with a partner lane whose bit M of the
// row index differs, and each lane keeps the half selected by that bit (the
// partner comes from a mirror or quad swap, so it need not be lane ^ M: it
// only has to share the bits above M).  After the steps M = 8, 4, 2, 1,
// lane l of the row holds the row's sum of element l in x[0].  The DPP moves
// run on every lane; only the selects depend on the lane.
template <int M>
__device__ __forceinline__ void row16_reduce_step(float* x, int cl) {
    constexpr int CTRL = M == 8 ? 0x140 : M == 4 ? 0x141 : M == 2 ? 0x4E : 0xB1;
    const bool up = (cl & M) != 0;
#pragma unroll
    for (int e = 0; e < M; ++e) {
        const float send = up ? x[e] : x[e + M];
        const float keep = up ? x[e + M] : x[e];
        x[e] = keep + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(send), CTRL, 0xf, 0xf, false));
    }
}

// x[0 .. 3] of every lane summed over the four lane groups (rows of 16
// lanes): lane (g, cl) returns the sum over g' of x[g] held by lane (g', cl).
// Two exchange steps, each lane keeping the half of its values that its
// partner sends back summed (partners 32, then 16 lanes apart).
__device__ __forceinline__ float group4_transpose_sum(const float (&x)[4], int g) {
    const bool hi2 = (g & 2) != 0;
    const float k0 = hi2 ? x[2] : x[0], k1 = hi2 ? x[3] : x[1];
    const float s0 = hi2 ? x[0] : x[2], s1 = hi2 ? x[1] : x[3];
    const float y0 = k0 + __shfl_xor(s0, 32, 64);
    const float y1 = k1 + __shfl_xor(s1, 32, 64);
    const bool hi1 = (g & 1) != 0;
    const float kk = hi1 ? y1 : y0, ss = hi1 ? y0 : y1;
    return kk + __shfl_xor(ss, 16, 64);
}

// Store two adjacent channels' values (as the path's element type).
__device__ __forceinline__ void st2(__bf16* p, float a, float b) {
    bf16x2 x;
    x[0] = (__bf16)a;
    x[1] = (__bf16)b;
    *reinterpret_cast<bf16x2*>(p) = x;
}
__device__ __forceinline__ void st2(float* p, float a, float b) {
    *reinterpret_cast<float2*>(p) = make_float2(a, b);
}
// Load eight consecutive values (16-byte aligned) as fp32.
__device__ __forceinline__ void ld8f(const __bf16* p, float* x) {
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (float)v[e];
}
__device__ __forceinline__ void ld8f(const float* p, float* x) {
    const floatx4 a = reinterpret_cast<const floatx4*>(p)[0], b = reinterpret_cast<const floatx4*>(p)[1];
#pragma unroll
    for (int e = 0; e < 4; ++e) { x[e] = a[e]; x[4 + e] = b[e]; }
}

// Store eight consecutive values (16 bytes of bf16 / 32 bytes of fp32).
__device__ __forceinline__ void st8(__bf16* p, const float* x) {
    bf16x8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (__bf16)x[e];
    *reinterpret_cast<bf16x8*>(p) = r;
}
__device__ __forceinline__ void st8(_Float16* p, const float* x) {
    halfx8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = (_Float16)x[e];
    *reinterpret_cast<halfx8*>(p) = r;
}
__device__ __forceinline__ void st8(float* p, const float* x) {
    reinterpret_cast<floatx4*>(p)[0] = floatx4{x[0], x[1], x[2], x[3]};
    reinterpret_cast<floatx4*>(p)[1] = floatx4{x[4], x[5], x[6], x[7]};
}

// Per-chunk records that the checkpointing forward leaves for the backward,
// each an array over (b, h, chunk) units in that order.
// Gates computed inside the forward from their logits (the mixer path): f
// holds forget-gate logits, beta and c the erase and write logits; then
// f = forget_gate(f, exp(a_log[h])), beta = beta_scale * sigmoid, c = sigmoid.
struct FwdGates {
    const float* a_log;   // [H]
    float beta_scale;
    // with og set: o leaves as y = o / sqrt(mean_i o_i^2 + norm_eps) * norm_w[h]
    // * sigmoid(og), per (b, t, h) (og [B, T, H, D] bf16 gate logits, norm_w [H, D])
    const __bf16* og;
    const float* norm_w;
    float norm_eps;
};

struct FwdCkpt {
    void* S;    // entering state S[i][j], input dtype, d*d per unit
    float* U;   // u, then r0: 2*CH fp32 per unit
    float* M;   // M, [CH][CH] fp32 per unit
    void* P;    // P, [CH][CH] input dtype per unit
};

// Number of MFMA K-steps of each path that cover a contraction of length n.
template <class TR, int N>
struct KSteps { static constexpr int value = N / TR::KS; };

}  // namespace kd
