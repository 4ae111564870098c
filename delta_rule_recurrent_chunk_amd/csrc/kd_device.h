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
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int CH = 64;        // chunk length (tokens per chunk)
constexpr int SB = 16;        // sub-block edge = MFMA tile edge
constexpr int NSB = CH / SB;  // sub-blocks per chunk

// Workgroup barrier that waits for this wave's LDS traffic only, so global
// prefetch loads stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ float readlane_f(float x, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
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
    // B operand from accumulator tiles holding X[j][n] (j = 16mt + 4g + r),
    // each K row j scaled by sc[j] (fp32, before rounding to bf16).
    static __device__ __forceinline__ Frag state_frag(const floatx4* acc, int ks, const float* sc, int g) {
        const floatx4 s0 = *reinterpret_cast<const floatx4*>(sc + KS * ks + 4 * g);
        const floatx4 s1 = *reinterpret_cast<const floatx4*>(sc + KS * ks + 16 + 4 * g);
        const floatx4 a = acc[2 * ks] * s0;
        const floatx4 b = acc[2 * ks + 1] * s1;
        Frag r;
        r[0] = cvt(a[0]); r[1] = cvt(a[1]); r[2] = cvt(a[2]); r[3] = cvt(a[3]);
        r[4] = cvt(b[0]); r[5] = cvt(b[1]); r[6] = cvt(b[2]); r[7] = cvt(b[3]);
        return r;
    }
    // natural-order fragment scaled element-wise by sc[K] (K = 32ks + 8g + e)
    static __device__ __forceinline__ Frag scale_nat(Frag x, const float* sc, int ks, int g) {
        const floatx4 s0 = *reinterpret_cast<const floatx4*>(sc + KS * ks + 8 * g);
        const floatx4 s1 = *reinterpret_cast<const floatx4*>(sc + KS * ks + 8 * g + 4);
        Frag r;
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = cvt(tof(x[e]) * s0[e]);
#pragma unroll
        for (int e = 0; e < 4; ++e) r[4 + e] = cvt(tof(x[4 + e]) * s1[e]);
        return r;
    }
    // natural-order fragment along K = token index t: value(t) = u[t] * col[t*ld]
    static __device__ __forceinline__ Frag col_times(const E* col, int ld, const float* u, int ks, int g) {
        const int t0 = KS * ks + 8 * g;
        const floatx4 u0 = *reinterpret_cast<const floatx4*>(u + t0);
        const floatx4 u1 = *reinterpret_cast<const floatx4*>(u + t0 + 4);
        Frag r;
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = cvt(u0[e] * tof(col[(t0 + e) * ld]));
#pragma unroll
        for (int e = 0; e < 4; ++e) r[4 + e] = cvt(u1[e] * tof(col[(t0 + 4 + e) * ld]));
        return r;
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
    static __device__ __forceinline__ Frag state_frag(const floatx4* acc, int ks, const float* sc, int g) {
        return acc[ks >> 2][ks & 3] * sc[16 * (ks >> 2) + 4 * g + (ks & 3)];
    }
    static __device__ __forceinline__ Frag scale_nat(Frag x, const float* sc, int ks, int g) {
        return x * sc[KS * ks + g];
    }
    static __device__ __forceinline__ Frag col_times(const E* col, int ld, const float* u, int ks, int g) {
        const int t = KS * ks + g;
        return u[t] * col[t * ld];
    }
};

// Eight consecutive tokens of two adjacent channels (j0 = even, j0 + 1) held
// in registers between the global load and its use (the prefetch buffer).
// One 32-bit load fetches both bf16 channels of a row.
template <class TR> struct Pair8;

template <> struct Pair8<Bf16T> {
    uint32_t w[8];   // low half: channel j0, high half: channel j0 + 1
    // p: wave-uniform base; row m at p[off + min(m, last)*stride] (32-bit
    // element offsets, off even).  Loads are unconditional: rows past the
    // sequence end re-read row `last` (in bounds) and are masked at use.
    __device__ __forceinline__ void load(const __bf16* p, uint32_t off, uint32_t stride, int last) {
#pragma unroll
        for (int m = 0; m < 8; ++m)
            w[m] = *reinterpret_cast<const uint32_t*>(p + off + (uint32_t)(m < last ? m : last) * stride);
    }
    __device__ __forceinline__ float get(int m, int c) const {
        return __uint_as_float(c ? (w[m] & 0xffff0000u) : (w[m] << 16));
    }
};

template <> struct Pair8<F32T> {
    float w[8][2];
    __device__ __forceinline__ void load(const float* p, uint32_t off, uint32_t stride, int last) {
#pragma unroll
        for (int m = 0; m < 8; ++m) {
            const float2 x = *reinterpret_cast<const float2*>(p + off + (uint32_t)(m < last ? m : last) * stride);
            w[m][0] = x.x;
            w[m][1] = x.y;
        }
    }
    __device__ __forceinline__ float get(int m, int c) const { return w[m][c]; }
};

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

// Number of MFMA K-steps of each path that cover a contraction of length n.
template <class TR, int N>
struct KSteps { static constexpr int value = N / TR::KS; };

}  // namespace kd
