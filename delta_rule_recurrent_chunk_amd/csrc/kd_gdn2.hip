// kd_gdn2.hip -- chunkwise forward of the Gated Delta Rule-2 (decoupled erase
// and write), bf16 inputs at d = 128, gfx950.
//
// Rule (aitrends.kr Gated DeltaNet-2 summary, sections 핵심 기여 and 방법론
// steps 1-4): per (b, h), state S in R^{dk x dv} (keys as rows),
//     Sbar = diag(alpha_t) S_{t-1};  u_t = w_t v_t - Sbar^T (b_t k_t);
//     S_t = Sbar + k_t u_t^T;  o_t = S_t^T q_t.
// Chunked form used here (C = 64 tokens; gamma_t = product of alpha over the
// chunk up to t, per key channel, referenced to the chunk start):
//     Ebar = gamma * b * k,  Kbar = k / gamma,  Qbar = gamma * q,
//     Ktil = k * gamma_C / gamma,  Z = w * v,
//     T = tril(Ebar Kbar^T, -1),  P = tril(Qbar Kbar^T, 0),
//     U = (I + T)^{-1} (Z - Ebar S0)        (the WY step of 방법론 step 3:
//                                            U = A Z - (A Ebar) S0),
//     O = Qbar S0 + P U,  S_C = diag(gamma_C) S0 + Ktil^T U.
// Kbar divides by gamma; a key channel whose decay over a chunk falls below
// 2^-100 gets a zero Kbar column and its T and P terms are added exactly
// (rare path), as in the Kronecker kernels.
//
// One workgroup of eight waves per (b, h); phases separated by barriers:
//   1. every wave prepares 8 rows of the chunk (two key channels per lane):
//      decay products, the operands above into LDS (the next chunk's rows are
//      loaded during phases 2 and 3);
//   2. Gram tiles of T and P; each wave forms Ebar S0 and Qbar S0 for its 16
//      value columns (the state lives in its MFMA accumulators, keys as rows);
//      the wave of each diagonal Gram tile inverts that 16 x 16 block of I + T;
//   3. each wave solves (I + T) U = Z - Ebar S0 for its value columns block by
//      block with 16 x 16 x 16 MFMAs on bf16 hi + lo splits (fp32-like
//      products), then the readout O = Qbar S0 + P U and the update
//      S <- diag(gamma_C) S + Ktil^T U (Ktil and U also split hi + lo).
#include "kd_device.h"

// Phase markers: no-ops here; a profiling build may define them to record
// timestamps at the phase boundaries of the chunk loop.
#ifndef KD_PHASE_MARK
#define KD_PHASE_MARK(chunk, id) ((void)0)
#endif

namespace kd {

namespace g2w {
constexpr int D = 128;
constexpr int NT = 512;
constexpr int NW = 8;             // waves
constexpr int RB = CH / NW;       // rows per wave in phase 1
constexpr int LD = D + 16;        // row-major [CH][D] operands (key columns in pcol order)
constexpr int LDT = CH + 8;       // transposed [D][CH] operands
constexpr int LDM = CH + 4;       // fp32 T (and the fallback scratch)
constexpr int LDP = CH + 8;       // P (token columns in pcol order)
constexpr int LDX = 16 + 4;       // fp32 inverses of the diagonal blocks
}  // namespace g2w

struct Gdn2Smem {
    alignas(16) __bf16 Qb[CH * g2w::LD];       // q * gamma
    alignas(16) __bf16 Eb[CH * g2w::LD];       // b * k * gamma
    alignas(16) __bf16 Kc[CH * g2w::LD];       // k / gamma (0 for fallback channels)
    alignas(16) __bf16 KtH[g2w::D * g2w::LDT]; // Ktil^T, high bf16 part (token columns in pcol order)
    alignas(16) __bf16 KtL[g2w::D * g2w::LDT]; // Ktil^T, low part
    alignas(16) __bf16 ZT[g2w::D * g2w::LDT];  // (w * v)^T, natural token order
    alignas(16) float Tm[CH * g2w::LDM];       // T; fallback scratch
    alignas(16) __bf16 P[CH * g2w::LDP];
    alignas(16) float X[4][16 * g2w::LDX];     // (I + T_II)^{-1}
    alignas(16) float bprod[g2w::NW][g2w::D];  // product of alpha over each 8-row block
    alignas(16) float gam[g2w::D];             // gamma_C
    unsigned unsafe;
};

typedef short s16x4 __attribute__((ext_vector_type(4)));

// fp32 x as bf16 hi + lo (x - hi rounded again): products of two such splits
// taken as hi*hi + hi*lo + lo*hi carry about 16 significant bits.
__device__ __forceinline__ void split_hl(floatx4 x, s16x4& hi, s16x4& lo) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const __bf16 hh = (__bf16)x[e];
        hi[e] = __builtin_bit_cast(short, hh);
        lo[e] = __builtin_bit_cast(short, (__bf16)(x[e] - (float)hh));
    }
}
__device__ __forceinline__ floatx4 mma16(s16x4 a, s16x4 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 mma16_3(s16x4 ah, s16x4 al, s16x4 bh, s16x4 bl, floatx4 c) {
    c = mma16(ah, bh, c);
    c = mma16(ah, bl, c);
    return mma16(al, bh, c);
}
// low bf16 parts of Bf16T::state_frag(acc, ks)
__device__ __forceinline__ Bf16T::Frag state_frag_lo(const floatx4* acc, int ks, Bf16T::Frag hi) {
    const floatx4 a = acc[2 * ks], b = acc[2 * ks + 1];
    Bf16T::Frag r;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        r[e] = (__bf16)(a[e] - (float)hi[e]);
        r[4 + e] = (__bf16)(b[e] - (float)hi[4 + e]);
    }
    return r;
}

__global__ __launch_bounds__(g2w::NT) void kd_gdn2_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ al, const __bf16* __restrict__ bg, const __bf16* __restrict__ wg,
    const float* __restrict__ S0, __bf16* __restrict__ o, float* __restrict__ ST, int T, int H)
{
    using namespace g2w;
    typedef Bf16T TR;
    typedef __bf16 E;
    typedef TR::Frag Frag;
    constexpr int KD_ = D / TR::KS;    // K-steps over d
    constexpr int KC_ = CH / TR::KS;   // K-steps over a chunk

    __shared__ Gdn2Smem sm;

    const int tid = threadIdx.x;
    const int lane = tid & 63, g = lane >> 4, cl = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int bh = blockIdx.x, b = bh / H, h = bh % H;
    const uint32_t rs = (uint32_t)H * D;               // elements between tokens
    const size_t bbase = (size_t)b * T * H * D;
    const E *qb = q + bbase, *kb = k + bbase, *vb = v + bbase;
    const E *ab = al + bbase, *bgb = bg + bbase, *wgb = wg + bbase;
    const uint32_t hoff = (uint32_t)h * D;
    const int NC = (T + CH - 1) / CH;
    const size_t sbase = (size_t)bh * D * D;

    if (NC == 0) {   // empty sequence: S_T = S0
        if (ST)
            for (int x = tid; x < D * D; x += NT) ST[sbase + x] = S0 ? S0[sbase + x] : 0.f;
        return;
    }

    // one-time init: the upper triangles of T and P are never written
    for (int x = tid; x < CH * LDM; x += NT) sm.Tm[x] = 0.f;
    for (int x = tid; x < CH * LDP; x += NT) sm.P[x] = (E)0.f;
    if (tid == 0) sm.unsafe = 0u;

    // state: this wave's value columns i0 .. i0 + 15, S[16mj + 4g + r][i0 + cl] in S[mj][r]
    const int i0 = 16 * w;
    floatx4 S[D / 16];
#pragma unroll
    for (int mj = 0; mj < D / 16; ++mj)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            S[mj][r] = S0 ? S0[sbase + (size_t)(16 * mj + 4 * g + r) * D + i0 + cl] : 0.f;

    // phase-1 lane mapping: rows rb .. rb + 7 of the chunk, channels ch0, ch0 + 1
    const int rb = RB * w;
    const int ch0 = 2 * lane;
    const int pc0 = TR::pcol(ch0);   // adjacent under pcol
    Raw8x2 rq, rk, rv, ra, rbb, rw;
    // Rows past the end re-read the last row (in bounds) and are cleared
    // before use; loads are clamped to the last chunk.
    auto row_off = [&](int n, int& last) {
        const int t0 = min(n * CH + rb, T - 1);
        last = min(RB - 1, T - 1 - t0);
        return (uint32_t)t0 * rs + hoff + ch0;
    };
    auto load_rows_a = [&](int n) {   // q, k, alpha
        int last;
        const uint32_t off = row_off(n, last);
        rq.load(qb, off, rs, last);
        rk.load(kb, off, rs, last);
        ra.load(ab, off, rs, last);
    };
    auto load_rows_b = [&](int n) {   // v, b, w
        int last;
        const uint32_t off = row_off(n, last);
        rv.load(vb, off, rs, last);
        rbb.load(bgb, off, rs, last);
        rw.load(wgb, off, rs, last);
    };
    load_rows_a(0);
    load_rows_b(0);
    lds_barrier();

    for (int n = 0; n < NC; ++n) {
        KD_PHASE_MARK(n, 0);
        // =========================================== phase 1: operands of chunk n
        if (n * CH + CH > T) {   // ragged last chunk: rows past the end contribute nothing
#pragma unroll
            for (int e = 0; e < RB; ++e)
                if (n * CH + rb + e >= T) {
                    rq.clear(e, 0.f); rk.clear(e, 0.f); rv.clear(e, 0.f);
                    ra.clear(e, 1.f); rbb.clear(e, 0.f); rw.clear(e, 0.f);
                }
        }
        {
            float tot[2];
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) {
                const float x0 = ra.get(0, c2) * ra.get(1, c2), x1 = ra.get(2, c2) * ra.get(3, c2);
                const float x2 = ra.get(4, c2) * ra.get(5, c2), x3 = ra.get(6, c2) * ra.get(7, c2);
                tot[c2] = (x0 * x1) * (x2 * x3);
            }
            st2(&sm.bprod[w][ch0], tot[0], tot[1]);
        }
        lds_barrier();
        unsigned pmask = 0;   // fallback channels (bit c: ch0 + c)
        {
            // gamma before this block (plt), after it (pgt) and over the chunk
            // (gC, multiplied in one fixed order so every wave agrees on it)
            float plt[2] = {1.f, 1.f}, pgt[2] = {1.f, 1.f}, gC[2] = {1.f, 1.f}, rgC[2];
#pragma unroll
            for (int p = 0; p < NW; ++p) {
                const float2 xb = *reinterpret_cast<const float2*>(&sm.bprod[p][ch0]);
                gC[0] *= xb.x; gC[1] *= xb.y;
                if (p < w) { plt[0] *= xb.x; plt[1] *= xb.y; }
                if (p > w) { pgt[0] *= xb.x; pgt[1] *= xb.y; }
            }
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) {
                const bool un = !(gC[c2] >= kSafeFloor);
                if (un) pmask |= 1u << c2;
                rgC[c2] = un ? 0.f : 1.f / gC[c2];
            }
            if (w == 0) st2(&sm.gam[ch0], gC[0], gC[1]);
            if (pmask) atomicOr(&sm.unsafe, 1u);
            // gamma_C / gamma at each row: suffix products within the block
            float om[RB][2];
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) {
                om[RB - 1][c2] = pgt[c2];
#pragma unroll
                for (int e = RB - 2; e >= 0; --e) om[e][c2] = om[e + 1][c2] * ra.get(e + 1, c2);
            }
            float ga[2] = {plt[0], plt[1]};
            uint32_t kth[2][RB / 2], ktl[2][RB / 2], zt[2][RB / 2];   // transposed pairs of tokens
#pragma unroll
            for (int e = 0; e < RB; ++e) {
                float qo[2], eo[2], co[2], kt[2], zo[2];
#pragma unroll
                for (int c2 = 0; c2 < 2; ++c2) {
                    ga[c2] *= ra.get(e, c2);
                    const float kf = rk.get(e, c2);
                    kt[c2] = kf * om[e][c2];              // k gamma_C / gamma
                    qo[c2] = rq.get(e, c2) * ga[c2];
                    eo[c2] = rbb.get(e, c2) * kf * ga[c2];
                    co[c2] = kt[c2] * rgC[c2];            // k / gamma
                    zo[c2] = rw.get(e, c2) * rv.get(e, c2);
                }
                st2(&sm.Qb[(rb + e) * LD + pc0], qo[0], qo[1]);
                st2(&sm.Eb[(rb + e) * LD + pc0], eo[0], eo[1]);
                st2(&sm.Kc[(rb + e) * LD + pc0], co[0], co[1]);
                // (token e, token e + 1) pairs per channel for the transposed stores
#pragma unroll
                for (int c2 = 0; c2 < 2; ++c2) {
                    const __bf16 hh = (__bf16)kt[c2];
                    const uint32_t hb = (uint32_t)__builtin_bit_cast(unsigned short, hh);
                    const uint32_t lb = (uint32_t)__builtin_bit_cast(unsigned short, (__bf16)(kt[c2] - (float)hh));
                    const uint32_t zb = (uint32_t)__builtin_bit_cast(unsigned short, (__bf16)zo[c2]);
                    if (e & 1) {
                        kth[c2][e >> 1] |= hb << 16;
                        ktl[c2][e >> 1] |= lb << 16;
                        zt[c2][e >> 1] |= zb << 16;
                    } else {
                        kth[c2][e >> 1] = hb;
                        ktl[c2][e >> 1] = lb;
                        zt[c2][e >> 1] = zb;
                    }
                }
            }
            // transposed operands: channel ch0 + c2, tokens rb .. rb + 7.  Ktil^T
            // columns are in pcol order (tokens rb .. rb+3 and rb+4 .. rb+7 are two
            // runs of four); Z^T in natural order.
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) {
                const int row = (ch0 + c2) * LDT;
                *reinterpret_cast<uint2*>(&sm.KtH[row + TR::pcol(rb)]) = make_uint2(kth[c2][0], kth[c2][1]);
                *reinterpret_cast<uint2*>(&sm.KtH[row + TR::pcol(rb + 4)]) = make_uint2(kth[c2][2], kth[c2][3]);
                *reinterpret_cast<uint2*>(&sm.KtL[row + TR::pcol(rb)]) = make_uint2(ktl[c2][0], ktl[c2][1]);
                *reinterpret_cast<uint2*>(&sm.KtL[row + TR::pcol(rb + 4)]) = make_uint2(ktl[c2][2], ktl[c2][3]);
                *reinterpret_cast<uint4*>(&sm.ZT[row + rb]) = make_uint4(zt[c2][0], zt[c2][1], zt[c2][2], zt[c2][3]);
            }
        }
        lds_barrier();

        // =========================================== exact fallback terms (rare)
        const bool fbk = sm.unsafe != 0u;
        if (fbk) {
            // Exact T and P terms of the key channels whose decay over the chunk
            // falls below the floor: T[t,s] (s<t) accumulates at Tm[t][s], P[t,s]
            // (s<t) at Tm[s][t], P[t,t] at Tm[t][t].  Rows are re-read from
            // global memory.
            for (int x = tid; x < CH * LDM; x += NT) sm.Tm[x] = 0.f;
            lds_barrier();
            if (w == 0 && pmask) {
                const int t0 = n * CH;
#pragma unroll 1
                for (int c = 0; c < 2; ++c) {
                    if (!((pmask >> c) & 1u)) continue;
                    const uint32_t off = (uint32_t)t0 * rs + hoff + ch0 + c;
#pragma unroll 1
                    for (int s = 0; s < CH && t0 + s < T; ++s) {
                        const float ks_ = (float)kb[off + s * rs];
                        atomicAdd(&sm.Tm[s * LDM + s], (float)qb[off + s * rs] * ks_);
                        float prod = 1.f;
#pragma unroll 1
                        for (int t = s + 1; t < CH && t0 + t < T; ++t) {
                            prod *= (float)ab[off + t * rs];
                            const float kt_ = (float)kb[off + t * rs];
                            atomicAdd(&sm.Tm[t * LDM + s], (float)bgb[off + t * rs] * kt_ * ks_ * prod);
                            atomicAdd(&sm.Tm[s * LDM + t], (float)qb[off + t * rs] * ks_ * prod);
                        }
                    }
                }
            }
            lds_barrier();
        }

        KD_PHASE_MARK(n, 1);
        // =========================================== phase 2: Grams, state products
        // next chunk's rows, in flight through the rest of this chunk (the raw
        // rows of this chunk were last read in phase 1)
        if (n + 1 < NC) load_rows_a(n + 1);
        // Gram tile (I_ >= J_) of T and P: waves 0..7 take tiles 0..7, waves 0, 1
        // also tiles 8, 9.  The wave of a diagonal tile (I_ == J_) then inverts
        // that 16 x 16 block of I + T: it alone wrote the block, and a wave's LDS
        // accesses complete in order.
        auto gram_tile = [&](int tile) {
            const int I_ = tile < 1 ? 0 : tile < 3 ? 1 : tile < 6 ? 2 : 3;
            const int J_ = tile - (I_ * (I_ + 1)) / 2;
            const E* aE = &sm.Eb[(SB * I_ + cl) * LD];
            const E* aQ = &sm.Qb[(SB * I_ + cl) * LD];
            const E* bK = &sm.Kc[(SB * J_ + cl) * LD];
            floatx4 gt = {0.f, 0.f, 0.f, 0.f}, pp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KD_; ++ks) {
                const Frag kk = TR::ld_nat(bK, ks, g);
                gt = TR::mma(TR::ld_nat(aE, ks, g), kk, gt);
                pp = TR::mma(TR::ld_nat(aQ, ks, g), kk, pp);
            }
            const int s_ = SB * J_ + cl;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t_ = SB * I_ + 4 * g + r;
                if (fbk) {
                    if (s_ < t_) gt[r] += sm.Tm[t_ * LDM + s_];
                    if (s_ <= t_) {
                        pp[r] += sm.Tm[s_ * LDM + t_];
                        if (s_ < t_) sm.Tm[s_ * LDM + t_] = 0.f;
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t_ = SB * I_ + 4 * g + r;
                if (s_ < t_) sm.Tm[t_ * LDM + s_] = gt[r];
                else if (s_ == t_) sm.Tm[t_ * LDM + s_] = 0.f;   // clears the P diagonal scratch
                sm.P[t_ * LDP + TR::pcol(s_)] = (E)((s_ <= t_) ? pp[r] : 0.f);
            }
            if (I_ == J_) {
                // (I + T_II)^{-1}: lane c < 16 runs forward substitution down column c
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                if (lane < 16) {
                    const int c = lane;
                    const float* Tb = &sm.Tm[(16 * I_) * LDM + 16 * I_];
                    float x[16];
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        // the row of T as four 16-byte reads, the sum over s < r in
                        // four independent chains
                        floatx4 tr[4];
#pragma unroll
                        for (int q4 = 0; q4 < 4; ++q4)
                            if (4 * q4 < r) tr[q4] = *reinterpret_cast<const floatx4*>(&Tb[r * LDM + 4 * q4]);
                        float a4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int s = 0; s < r; ++s) a4[s & 3] = fmaf(tr[s >> 2][s & 3], x[s], a4[s & 3]);
                        const float acc = ((r == c) ? 1.f : 0.f) - ((a4[0] + a4[1]) + (a4[2] + a4[3]));
                        x[r] = (r < c) ? 0.f : acc;
                    }
#pragma unroll
                    for (int r = 0; r < 16; ++r) sm.X[I_][r * LDX + c] = x[r];
                }
            }
        };
        gram_tile(w);
        if (w < 2) gram_tile(8 + w);

        // X = Op S0 for this wave's value columns (Op rows = tokens 16tt + cl;
        // K = keys in the state order of the accumulators)
        floatx4 R[NSB], OQ[NSB];
        {
            const floatx4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int tt = 0; tt < NSB; ++tt) { R[tt] = z; OQ[tt] = z; }
#pragma unroll
            for (int ks = 0; ks < KD_; ++ks) {
                const Frag sf = TR::state_frag(S, ks);
#pragma unroll
                for (int tt = 0; tt < NSB; ++tt) {
                    R[tt] = TR::mma(TR::ld_state_p(&sm.Eb[(SB * tt + cl) * LD], ks, g), sf, R[tt]);
                    OQ[tt] = TR::mma(TR::ld_state_p(&sm.Qb[(SB * tt + cl) * LD], ks, g), sf, OQ[tt]);
                }
            }
            // R = Z - Ebar S0 (Z^T row i0 + cl holds tokens in natural order)
#pragma unroll
            for (int tt = 0; tt < NSB; ++tt) {
                const bf16x4 zz = *reinterpret_cast<const bf16x4*>(&sm.ZT[(i0 + cl) * LDT + SB * tt + 4 * g]);
#pragma unroll
                for (int r = 0; r < 4; ++r) R[tt][r] = (float)zz[r] - R[tt][r];
            }
        }
        lds_barrier();

        KD_PHASE_MARK(n, 2);
        // =========================================== phase 3: solve, readout, update
        if (n + 1 < NC) load_rows_b(n + 1);
        floatx4 U[NSB];
#pragma unroll
        for (int I_ = 0; I_ < NSB; ++I_) {
            floatx4 acc = R[I_];
#pragma unroll
            for (int J_ = 0; J_ < I_; ++J_) {   // acc -= T_IJ U_J
                const floatx4 tv = -*reinterpret_cast<const floatx4*>(&sm.Tm[(16 * I_ + cl) * LDM + 16 * J_ + 4 * g]);
                s16x4 th, tl, uh, ul;
                split_hl(tv, th, tl);
                split_hl(U[J_], uh, ul);
                acc = mma16_3(th, tl, uh, ul, acc);
            }
            const floatx4 xv = *reinterpret_cast<const floatx4*>(&sm.X[I_][cl * LDX + 4 * g]);
            s16x4 xh, xl, ah, alo;
            split_hl(xv, xh, xl);
            split_hl(acc, ah, alo);
            U[I_] = mma16_3(xh, xl, ah, alo, floatx4{0.f, 0.f, 0.f, 0.f});
        }
        // O = Qbar S0 + P U
#pragma unroll
        for (int ks = 0; ks < KC_; ++ks) {
            const Frag uf = TR::state_frag(U, ks);
#pragma unroll
            for (int tt = 0; tt < NSB; ++tt)
                OQ[tt] = TR::mma(TR::ld_state_p(&sm.P[(SB * tt + cl) * LDP], ks, g), uf, OQ[tt]);
        }
        if (o) {
            // O goes out through LDS (the wave's own 16 columns of the Qbar
            // tile, last read in phase 2): each lane then stores 16 bytes,
            // eight adjacent columns of one token, instead of sixteen 2-byte
            // values; no other wave reads these columns, so no barrier
            E* ost = sm.Qb;
#pragma unroll
            for (int tt = 0; tt < NSB; ++tt)
#pragma unroll
                for (int r = 0; r < 4; ++r) ost[(SB * tt + 4 * g + r) * LD + i0 + cl] = (E)OQ[tt][r];
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this wave's writes before its reads
#pragma unroll
            for (int it = 0; it < 2; ++it) {
                const int pce = 64 * it + lane, tk = pce >> 1, half = pce & 1;
                const int t = n * CH + tk;
                const uint4 val = *reinterpret_cast<const uint4*>(&ost[tk * LD + i0 + 8 * half]);
                if (t < T) cp16_nt(o + bbase + (size_t)t * rs + hoff + i0 + 8 * half, &val);
            }
        }
        // S <- diag(gamma_C) S + Ktil^T U
#pragma unroll
        for (int mj = 0; mj < D / 16; ++mj)
            S[mj] = S[mj] * *reinterpret_cast<const floatx4*>(&sm.gam[16 * mj + 4 * g]);
#pragma unroll
        for (int ks = 0; ks < KC_; ++ks) {
            const Frag uh = TR::state_frag(U, ks);
            const Frag ul = state_frag_lo(U, ks, uh);
#pragma unroll
            for (int mj = 0; mj < D / 16; ++mj) {
                const Frag kh = TR::ld_state_p(&sm.KtH[(16 * mj + cl) * LDT], ks, g);
                const Frag kl = TR::ld_state_p(&sm.KtL[(16 * mj + cl) * LDT], ks, g);
                S[mj] = TR::mma(kh, uh, S[mj]);
                S[mj] = TR::mma(kh, ul, S[mj]);
                S[mj] = TR::mma(kl, uh, S[mj]);
            }
        }
        if (tid == 0) sm.unsafe = 0u;
        KD_PHASE_MARK(n, 3);
        lds_barrier();
    }
    if (ST) {
#pragma unroll
        for (int mj = 0; mj < D / 16; ++mj)
#pragma unroll
            for (int r = 0; r < 4; ++r) st_nt(&ST[sbase + (size_t)(16 * mj + 4 * g + r) * D + i0 + cl], S[mj][r]);
    }
}

hipError_t launch_gdn2(const void* q, const void* k, const void* v, const void* alpha, const void* b,
                       const void* w, const float* S0, void* o, float* ST, int B, int T, int H,
                       hipStream_t st)
{
    typedef __bf16 E;
    hipLaunchKernelGGL(kd_gdn2_kernel, dim3((unsigned)(B * H)), dim3(g2w::NT), 0, st, (const E*)q,
                       (const E*)k, (const E*)v, (const E*)alpha, (const E*)b, (const E*)w, S0, (E*)o, ST,
                       T, H);
    return hipGetLastError();
}

}  // namespace kd
