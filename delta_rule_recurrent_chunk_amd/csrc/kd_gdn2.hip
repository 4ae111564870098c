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
//   2. Gram tiles of T and P (waves 4..7 take the four diagonal tiles and
//      invert that 16 x 16 block of I + T, four lanes per column); each wave
//      forms Ebar S0 and Qbar S0 for its 16 value columns (the state lives in
//      its MFMA accumulators, keys as rows).  The off-diagonal T blocks and
//      the block inverses go to LDS once, as bf16 hi + lo operand fragments;
//   3. each wave solves (I + T) U = Z - Ebar S0 for its value columns block by
//      block with 16x16x32 products of the hi + lo parts (fp32-like), then
//      the readout O = Qbar S0 + P U and the update S <- diag(gamma_C) S +
//      Ktil^T U, whose operands go in fp16 with exact power-of-two scales.
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
constexpr int LDM = CH + 4;       // fp32 exact-term scratch
constexpr int LDO = 2 * LDM;      // bf16 o staging rows over the same bytes
constexpr int LDP = CH + 8;       // P (token columns in pcol order)
}  // namespace g2w

struct Gdn2Smem {
    alignas(16) __bf16 Qb[CH * g2w::LD];       // q * gamma
    alignas(16) __bf16 Eb[CH * g2w::LD];       // b * k * gamma
    alignas(16) __bf16 Kc[CH * g2w::LD];       // k / gamma (0 for fallback channels)
    alignas(16) _Float16 Kt[2][g2w::D * g2w::LDT]; // (Ktil 2^-ek)^T in fp16 (token columns in pcol order), by chunk parity
    alignas(16) __bf16 ZT[g2w::D * g2w::LDT];  // (w * v)^T, natural token order
    alignas(16) float Tm[CH * g2w::LDM];       // exact terms of the fallback channels; o staging in phase 3
    alignas(16) __bf16 P[CH * g2w::LDP];
    alignas(16) float X[4][16 * 16];           // scratch of the block inverses
    // A operands of the block solve, ready for 16x16x32 products: per lane,
    // the bf16 hi and lo parts of four adjacent entries of one row
    alignas(16) __bf16 TF[6][64 * 8];          // -T_IJ (I > J)
    alignas(16) __bf16 XF[4][64 * 8];          // (I + T_II)^{-1}
    alignas(16) float bprod[g2w::NW][g2w::D];  // product of alpha over each 8-row block
    alignas(16) float gam[2][g2w::D];          // gamma_C, by chunk parity
    float kmx[g2w::NW];                        // largest |k| of each wave's rows
    unsigned unsafe[2];                        // a fallback channel in the chunk, by parity
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
// Entry (i, k) of a 16 x 16 block into the x32 A-operand layout: lane
// 16 (k / 4) + i holds row i, columns 4 (k / 4) .. + 3, hi parts first.
__device__ __forceinline__ void put_frag(__bf16* f, int i, int k, float x) {
    const __bf16 hh = (__bf16)x;
    __bf16* p = f + (16 * (k >> 2) + i) * 8 + (k & 3);
    p[0] = hh;
    p[4] = (__bf16)(x - (float)hh);
}
// x of lane k of each quad, to all four lanes of the quad
__device__ __forceinline__ float quad_bcast(float x, int k) {
    switch (k) {
    case 0: return dpp_quad<0x00>(x);
    case 1: return dpp_quad<0x55>(x);
    case 2: return dpp_quad<0xAA>(x);
    default: return dpp_quad<0xFF>(x);
    }
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
    if (tid < 2) sm.unsafe[tid] = 0u;

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
    // Chunk m's operands are prepared one phase ahead: its block products at
    // the end of phase 2 of chunk m - 1, the rest during phase 3 of chunk m - 1.
    // In phase 3 the waves of one SIMD (w and w + 4) take the two jobs in
    // opposite orders, so the preparation's vector arithmetic runs beside the
    // other wave's products.
    // chunk m's decay products over each wave's 8 rows and its largest |k|
    auto prep_a = [&](int m) __attribute__((always_inline)) {
        if (m * CH + CH > T) {   // ragged last chunk: rows past the end contribute nothing
#pragma unroll
            for (int e = 0; e < RB; ++e)
                if (m * CH + rb + e >= T) {
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
            float km = 0.f;
#pragma unroll
            for (int e = 0; e < RB; ++e)
#pragma unroll
                for (int c2 = 0; c2 < 2; ++c2) km = fmaxf(km, fabsf(rk.get(e, c2)));
            km = wave_max_nonneg(km);
            if (lane == 0) sm.kmx[w] = km;
        }
    };
    // chunk m's operands into LDS: Qbar, Ebar, Kbar, Z^T and the K~ and gamma_C
    // buffers of its parity; ek_out is its K~ scale exponent and pmask_out the
    // lane's fallback channels
    auto prep_b = [&](int m, int& ek_out, unsigned& pmask_out) __attribute__((always_inline)) {
        // Ktil = k gamma_C / gamma is at most |k| in size: with the chunk's
        // largest |k| = x 2^ek (1/2 <= x < 1), Ktil 2^-ek lies in (-1, 1) and
        // goes to the update in fp16
        {
            float kmax = 0.f;
#pragma unroll
            for (int p = 0; p < NW; ++p) kmax = fmaxf(kmax, sm.kmx[p]);
            ek_out = pow2_exp(kmax);
        }
        const float ksc = ldexpf(1.f, -ek_out);
        pmask_out = 0u;   // fallback channels (bit c: ch0 + c)
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
                if (un) pmask_out |= 1u << c2;
                rgC[c2] = un ? 0.f : 1.f / gC[c2];
            }
            if (w == 0) st2(&sm.gam[m & 1][2 * (lane + opaque_zero())], gC[0], gC[1]);   // address formed here, not held
            if (pmask_out) atomicOr(&sm.unsafe[m & 1], 1u);
            // gamma_C / gamma at each row: suffix products within the block
            float om[RB][2];
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) {
                om[RB - 1][c2] = pgt[c2];
#pragma unroll
                for (int e = RB - 2; e >= 0; --e) om[e][c2] = om[e + 1][c2] * ra.get(e + 1, c2);
            }
            float ga[2] = {plt[0], plt[1]};
            uint32_t kth[2][RB / 2], zt[2][RB / 2];   // transposed pairs of tokens
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
                    const uint32_t hb = (uint32_t)__builtin_bit_cast(unsigned short, (_Float16)(kt[c2] * ksc));
                    const uint32_t zb = (uint32_t)__builtin_bit_cast(unsigned short, (__bf16)zo[c2]);
                    if (e & 1) {
                        kth[c2][e >> 1] |= hb << 16;
                        zt[c2][e >> 1] |= zb << 16;
                    } else {
                        kth[c2][e >> 1] = hb;
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
                *reinterpret_cast<uint2*>(&sm.Kt[m & 1][row + TR::pcol(rb)]) = make_uint2(kth[c2][0], kth[c2][1]);
                *reinterpret_cast<uint2*>(&sm.Kt[m & 1][row + TR::pcol(rb + 4)]) = make_uint2(kth[c2][2], kth[c2][3]);
                *reinterpret_cast<uint4*>(&sm.ZT[row + rb]) = make_uint4(zt[c2][0], zt[c2][1], zt[c2][2], zt[c2][3]);
            }
        }
    };
    load_rows_a(0);
    load_rows_b(0);
    lds_barrier();
    prep_a(0);
    lds_barrier();
    int ek_cur, ek_next = 0;
    unsigned pmask, pmask_next = 0u;
    prep_b(0, ek_cur, pmask);
    lds_barrier();

    for (int n = 0; n < NC; ++n) {
        KD_PHASE_MARK(n, 0);
        // =========================================== exact fallback terms (rare)
        const bool fbk = sm.unsafe[n & 1] != 0u;
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
        // the next chunk's rows (this chunk's rows were last read in its
        // preparation), in flight through the rest of the phase: waves 0..3
        // issue them first, waves 4..7 after their inverses, which the solve
        // waits for
        auto load_next = [&]() {
            if (n + 1 < NC) {
                load_rows_a(n + 1);
                load_rows_b(n + 1);
            }
        };
        if (w < 4) load_next();
        // Gram tile (I_ >= J_) of T and P.  The diagonal tiles 0, 2, 5, 9 go to
        // waves 4..7, which then invert that 16 x 16 block of I + T; waves 0..3
        // take the six off-diagonal tiles (waves 0 and 1 two each).
        auto gram_tile = [&](int tile) __attribute__((always_inline)) {
            const int I_ = tile < 1 ? 0 : tile < 3 ? 1 : tile < 6 ? 2 : 3;
            const int J_ = tile - (I_ * (I_ + 1)) / 2;
            const E* aE = &sm.Eb[(SB * I_ + cl) * LD];
            const E* aQ = &sm.Qb[(SB * I_ + cl) * LD];
            const E* bK = &sm.Kc[(SB * J_ + cl) * LD];
            // all twelve fragments are read before the first product, so the
            // LDS latency is paid once
            Frag fk[KD_], fe[KD_], fq[KD_];
#pragma unroll
            for (int ks = 0; ks < KD_; ++ks) {
                fk[ks] = TR::ld_nat(bK, ks, g);
                fe[ks] = TR::ld_nat(aE, ks, g);
                fq[ks] = TR::ld_nat(aQ, ks, g);
            }
            floatx4 gt = {0.f, 0.f, 0.f, 0.f}, pp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KD_; ++ks) {
                gt = TR::mma(fe[ks], fk[ks], gt);
                pp = TR::mma(fq[ks], fk[ks], pp);
            }
            const int s_ = SB * J_ + cl;
            if (fbk) {   // the exact terms of this tile (every entry is read by one tile)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t_ = SB * I_ + 4 * g + r;
                    if (s_ < t_) gt[r] += sm.Tm[t_ * LDM + s_];
                    if (s_ <= t_) pp[r] += sm.Tm[s_ * LDM + t_];
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t_ = SB * I_ + 4 * g + r;
                sm.P[t_ * LDP + TR::pcol(s_)] = (E)((s_ <= t_) ? pp[r] : 0.f);
            }
            if (I_ > J_) {
#pragma unroll
                for (int r = 0; r < 4; ++r) put_frag(sm.TF[tile - I_], 4 * g + r, cl, -gt[r]);
            }
            if (I_ == J_) {
                // (I + T_II)^{-1} by forward substitution down the 16 columns,
                // right-looking: lane 4c + q holds column c of the rows t = q
                // (mod 4).  Once row r is final, its owner's value goes to the
                // other lanes of the quad (a DPP broadcast) and every lane takes
                // T[t][r] x_r off its later rows, so each row adds one broadcast
                // and one multiply-add to the chain.  The strict lower triangle
                // goes through X[I_] with T[4j + q][s] at (16 q + s) 4 + j.
                float* Tq = sm.X[I_];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t16 = 4 * g + r;
                    Tq[(16 * r + cl) * 4 + g] = (cl < t16) ? gt[r] : 0.f;
                }
                const int c = lane >> 2, q = lane & 3;
                float tq[16][4];   // tq[r][j] = T[4j + q][r], needed for 4j + 3 > r
#pragma unroll
                for (int r = 0; r < 15; ++r)
#pragma unroll
                    for (int j = r >> 2; j < 4; ++j) tq[r][j] = Tq[(16 * q + r) * 4 + j];
                float xs[4];   // x[4j + q]
#pragma unroll
                for (int j = 0; j < 4; ++j) xs[j] = (4 * j + q == c) ? 1.f : 0.f;
#pragma unroll
                for (int r = 0; r < 15; ++r) {
                    const float xr = quad_bcast(xs[r >> 2], r & 3);
#pragma unroll
                    for (int j = r >> 2; j < 4; ++j) xs[j] = fmaf(-tq[r][j], xr, xs[j]);
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) put_frag(sm.XF[I_], 4 * j + q, c, xs[j]);
            }
        };
        if (w >= 4) {
            // the diagonal tiles and their inverses feed the whole solve: these
            // waves issue first until the inverses are out
            __builtin_amdgcn_s_setprio(2);
            gram_tile(w == 4 ? 0 : w == 5 ? 2 : w == 6 ? 5 : 9);
            __builtin_amdgcn_s_setprio(0);
            load_next();
        } else {
            gram_tile(w == 0 ? 1 : w == 1 ? 3 : w == 2 ? 4 : 8);
            if (w < 2) gram_tile(w == 0 ? 6 : 7);
        }

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
        if (n + 1 < NC) prep_a(n + 1);
        lds_barrier();

        KD_PHASE_MARK(n, 2);
        // =========================================== phase 3: solve, readout, update
        auto phase3 = [&]() __attribute__((always_inline)) {
            // the solve is a chain of dependent products: it issues ahead of
            // the next chunk's preparation on the same SIMD
            __builtin_amdgcn_s_setprio(1);
            // U = (I + T)^{-1} R by 16-row blocks, right-looking: as soon as U_J is
            // known, its terms -T_IJ U_J go into every later R_I, so the chain runs
            // through one product per block step.  Products carry about 16 bits:
            // (hi + lo) x (hi + lo) bf16 splits as two 16x16x32 products,
            // [hi | lo] [hi ; hi] and [hi | lo] [lo ; lo].
            floatx4 U[NSB];
            {
                auto prod = [&](Frag a2, s16x4 bh, s16x4 bl, floatx4 c) {
                    const Frag bh2 = __builtin_bit_cast(Frag, __builtin_shufflevector(bh, bh, 0, 1, 2, 3, 4, 5, 6, 7));
                    const Frag bl2 = __builtin_bit_cast(Frag, __builtin_shufflevector(bl, bl, 0, 1, 2, 3, 4, 5, 6, 7));
                    c = TR::mma(a2, bh2, c);
                    return TR::mma(a2, bl2, c);
                };
#pragma unroll
                for (int J_ = 0; J_ < NSB; ++J_) {
                    s16x4 bh, bl;
                    split_hl(R[J_], bh, bl);
                    U[J_] = prod(*reinterpret_cast<const Frag*>(&sm.XF[J_][8 * lane]), bh, bl,
                                 floatx4{0.f, 0.f, 0.f, 0.f});
                    if (J_ + 1 < NSB) {
                        split_hl(U[J_], bh, bl);
#pragma unroll
                        for (int I_ = J_ + 1; I_ < NSB; ++I_) {
                            const int ij = I_ * (I_ - 1) / 2 + J_;
                            R[I_] = prod(*reinterpret_cast<const Frag*>(&sm.TF[ij][8 * lane]), bh, bl, R[I_]);
                        }
                    }
                }
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
                // O goes out through LDS (the wave's own 16 columns of a bf16 tile
                // over Tm, which holds nothing in this phase): each lane then
                // stores 16 bytes, eight adjacent columns of one token, instead of
                // sixteen 2-byte values; no other wave reads these columns, so no
                // barrier
                E* ost = reinterpret_cast<E*>(sm.Tm);
#pragma unroll
                for (int tt = 0; tt < NSB; ++tt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) ost[(SB * tt + 4 * g + r) * LDO + i0 + cl] = (E)OQ[tt][r];
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this wave's writes before its reads
#pragma unroll
                for (int it = 0; it < 2; ++it) {
                    const int pce = 64 * it + lane, tk = pce >> 1, half = pce & 1;
                    const int t = n * CH + tk;
                    const uint4 val = *reinterpret_cast<const uint4*>(&ost[tk * LDO + i0 + 8 * half]);
                    if (t < T) cp16_nt(o + bbase + (size_t)t * rs + hoff + i0 + 8 * half, &val);
                }
            }
            // S <- diag(gamma_C) S + Ktil^T U: Ktil 2^-ek and U 2^-eu (eu from this
            // wave's largest |U|) in fp16, their product in fresh accumulators,
            // scaled back by 2^(ek + eu) and added to the decayed state
            {
                float um = 0.f;
#pragma unroll
                for (int tt = 0; tt < NSB; ++tt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) um = fmaxf(um, fabsf(U[tt][r]));
                const int eu = pow2_exp(wave_max_nonneg(um));
                const float usc = ldexpf(1.f, -eu);
                const int es = ek_cur + eu;
                TR::FragH uf[KC_];
#pragma unroll
                for (int ks = 0; ks < KC_; ++ks)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        uf[ks][e] = (_Float16)(U[2 * ks][e] * usc);
                        uf[ks][4 + e] = (_Float16)(U[2 * ks + 1][e] * usc);
                    }
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    floatx4 dS[D / 32];
#pragma unroll
                    for (int m = 0; m < D / 32; ++m) dS[m] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < KC_; ++ks)
#pragma unroll
                        for (int m = 0; m < D / 32; ++m) {
                            const int mj = (D / 32) * half + m;
                            dS[m] = TR::mma_h(*reinterpret_cast<const TR::FragH*>(
                                                  &sm.Kt[n & 1][(16 * mj + cl) * LDT + TR::KS * ks + 8 * g]),
                                              uf[ks], dS[m]);
                        }
#pragma unroll
                    for (int m = 0; m < D / 32; ++m) {
                        const int mj = (D / 32) * half + m;
                        const floatx4 gm = *reinterpret_cast<const floatx4*>(&sm.gam[n & 1][16 * mj + 4 * g]);
#pragma unroll
                        for (int r = 0; r < 4; ++r) S[mj][r] = fmaf(S[mj][r], gm[r], ldexpf(dS[m][r], es));
                    }
                }
            }
            __builtin_amdgcn_s_setprio(0);
        };
        if (w < 4) {
            phase3();
            if (n + 1 < NC) prep_b(n + 1, ek_next, pmask_next);
        } else {
            if (n + 1 < NC) prep_b(n + 1, ek_next, pmask_next);
            phase3();
        }
        // chunk n's fallback flag was read before the phase-2 barrier; chunk
        // n + 2 sets it during the next phase 3
        if (tid == 0) sm.unsafe[n & 1] = 0u;
        ek_cur = ek_next;
        pmask = pmask_next;
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
