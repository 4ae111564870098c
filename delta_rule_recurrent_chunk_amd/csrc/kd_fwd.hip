// kd_fwd.hip -- fused chunkwise forward of the Kronecker delta rule, gfx950.
//
// Method (onedev.kr KronLSTM summary, sections "어떻게 동작하나" and "어떻게
// 쓰나"): per (b, h), state S in R^{dv x dk}; per token
//     Sbar = S diag(f_t);  r_t = v_t^T Sbar k_t;  S = Sbar + (c_t - beta_t r_t) v_t k_t^T;
//     o_t = S q_t.
// Chunkwise form (chunk of C = 64 tokens, local index t; the same page's
// section "무엇과 다른가" states DeltaNet's chunk-parallel training applies; the
// Gated DeltaNet-2 summary on aitrends.kr, section "방법론" steps 3-4 and
// section "기술 상세", gives the WY pattern with a strictly lower triangular
// T, A = (I + T)^{-1} by forward substitution, C = 64).  With S0 the state
// entering the chunk and gamma_t = prod_{s<=t} f_s (per key channel):
//     r_t = v_t^T S0 (gamma_t * k_t) + sum_{s<t} u_s (v_t.v_s) (k_t . k_s gamma_t/gamma_s)
//     u_t = c_t - beta_t r_t   =>   (I + M) u = c - beta * r0,
//     M[t,s] = beta_t (v_t.v_s) sum_j k_tj k_sj gamma_tj/gamma_sj   (s < t)
// so the WY pseudo-targets u are scalars (the lifted features a = k (x) v have
// Gram a_t.a_s = (k_t.k_s)(v_t.v_s)).  Then
//     O   = (Q * gamma) S0^T + P (u * V),   P[t,s] = sum_j q_tj k_sj gamma_tj/gamma_sj  (s <= t)
//     S_C = S0 diag(gamma_C) + (u * V)^T (K * gamma_C/gamma).
//
// MI355X design
//  * One workgroup per (b, h), 4*d threads = d/16 waves, chunk loop inside
//    the kernel.  The waves split into two teams that run a software pipeline
//    over chunks, so matrix-core work of one chunk overlaps the vector work of
//    the next:
//      consumers (waves 0 .. d/32-1) own the fp32 state, TRANSPOSED (S^T, key
//        index j as rows) as MFMA accumulators, 32 value columns per wave.
//        Accumulator registers are directly an MFMA operand of the state reads
//        (Y^T = S Kbar^T, O^T = S Qbar^T), so the state never goes through LDS.
//        They do the state reads, the forward substitution (one wave) and the
//        readout and state update of chunk n.
//      producers (the other half) load chunk n+1 from HBM, fold the decay into
//        the operands and build its Gram tiles M, P on MFMA.
//    Per iteration: stage A (consumer: state reads n | producer: transposed
//    operands of n, decay scans of n+1) -- stage B (consumer: substitution n |
//    producer: operands of n+1, loads of n+2) -- stage C (consumer: readout
//    and update n | producer: Gram of n+1), one barrier after each stage.
//  * Decay folding.  The Gram tiles take their decay relative to the four
//    16-token sub-blocks: a_t = prod of f from the start of t's sub-block
//    through t, b_s = prod of f after s through the end of s's sub-block, and
//    the stored operands Qloc = q a, Kloc = k a, Kr = k b are products of gates
//    (at most 1).  Tile (I, J < I) is Kloc_I diag(D_IJ) Kr_J^T with D_IJ the
//    decay of the whole sub-blocks between them (1 for neighbours); a diagonal
//    tile divides Kr by its sub-block's decay.  A channel whose decay over one
//    sub-block is below 2^-100 (a reset f = 0 among them) is left out of that
//    diagonal tile and its terms are added exactly on the vector units before
//    the tile is read, so every input in [0, 1] is handled exactly.  The state
//    reads go sub-block by sub-block on the state decayed in place to the
//    sub-block's start, so (S diag(gamma before I)) Kloc^T = S Kbar^T; the
//    update then needs only the last sub-block's decay.  K * gamma_C/gamma
//    comes from suffix products and never divides.
//  * Precision: Grams and state reads take bf16 operands; the rank-64 state
//    update takes fp16 operands with exact power-of-two scales (max |k|,
//    max |u| * max |v| per chunk), its accumulation is fp32.
#include <type_traits>

#include "kd_device.h"

// Phase markers: no-ops here; a profiling build may define them to record
// timestamps at the stage boundaries of the chunk loop.
#ifndef KD_PHASE_MARK
#define KD_PHASE_MARK(chunk, id) ((void)0)
#endif

namespace kd {

template <class TR, int D>
struct FwdSmem {
    typedef typename TR::E E;
    typedef typename TR::H Hh;
    // row-major [CH][D] arrays; for bf16 a row stride of D + 16 elements
    // (72 dwords at d = 128) keeps the 16-byte fragment loads of 16 rows off
    // each other's LDS banks (measured: a third of the conflicts of D + 8)
    static constexpr int LD = D + (sizeof(E) == 2 ? 16 : TR::PAD);
    static constexpr int LDT = CH + TR::PAD;   // transposed [D][CH] arrays
    static constexpr int LDM = CH + 4;         // fp32 M
    static constexpr int LDP = CH + TR::PAD;   // P
    static constexpr int NWC = D / 32;         // consumer waves
    // row-major [CH][LD] operands, columns in TR::pcol order
    alignas(16) E Qb[CH * LD];     // q * a                         (chunk n+1 from stage B)
    alignas(16) E Kb[CH * LD];     // k * a
    alignas(16) E Kc[CH * LD];     // k * b
    alignas(16) E V[CH * LD];      // v
    alignas(16) E VT[D * LDT];     // v^T                           (chunk n from stage A)
    alignas(16) Hh KtT[D * LDT];   // (k gamma_C / gamma)^T * kscale
    alignas(16) float M[CH * LDM]; // beta_t tril_{-1}(G_K * G_V)
    alignas(16) E P[2][CH * LDP];  // tril_0 of the decayed Q K^T, by chunk parity
    alignas(16) float beta[2][CH];
    alignas(16) float c[2][CH];
    alignas(16) float u[CH];
    alignas(16) float r0p[NWC][CH];
    alignas(16) float bprod[NSB][D];   // product of f over each 16-token sub-block
    alignas(16) float gam[2][D];       // decay over the last sub-block, by chunk parity
    // decay factors of the prepared chunk: rows 0..3, 1 / (decay over sub-block
    // I) (0 below the floor); 4, 5, 6 the decay between the sub-blocks of tiles
    // (2,0), (3,1), (3,0) (pcol order); 7..9 the decay over sub-blocks 0..2
    // (natural order, the state's)
    alignas(16) float fac[10][D];
    unsigned kmax[3], vmax[3];              // per chunk mod 3: max |k|, max |v| (bits)
    unsigned fbm[2][NSB][(D + 31) / 32];    // channels below the floor per sub-block, by chunk parity
    unsigned fbany[2];
    unsigned umax;                          // max |u| of the current chunk (bits)
};

// CKPT: also store, per chunk, the records of FwdCkpt for the backward: the
// entering state (input dtype), the WY targets u and r0,
// and M (fp32) and P (input dtype) as [CH][CH] row-major.  A separate
// instantiation, so the plain forward carries none of its registers.
template <class TR, int D, bool CKPT>
__global__ __launch_bounds__(4 * D) void kd_fwd_kernel(
    const typename TR::E* __restrict__ q, const typename TR::E* __restrict__ k,
    const typename TR::E* __restrict__ v, const typename TR::E* __restrict__ f,
    const float* __restrict__ beta, const float* __restrict__ cc,
    const float* __restrict__ S0, typename TR::E* __restrict__ o, float* __restrict__ ST,
    FwdCkpt ck, const int* __restrict__ cu, int T_, int H)
{
    typedef typename TR::E E;
    typedef typename TR::H Hh;
    typedef typename TR::Frag Frag;
    typedef typename TR::FragH FragH;
    typedef FwdSmem<TR, D> SM;
    constexpr int NT = 4 * D;
    constexpr int NWC = SM::NWC;       // consumer waves (32 value columns each)
    constexpr int NWP = D / 32;        // producer waves
    constexpr int KD_ = D / TR::KS;    // K-steps over a d-long contraction
    constexpr int KC_ = CH / TR::KS;   // K-steps over a chunk-long contraction
    constexpr int LD = SM::LD, LDT = SM::LDT, LDM = SM::LDM, LDP = SM::LDP;

    __shared__ SM sm;

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6, g = lane >> 4, cl = lane & 15;
    const bool consumer = w < NWC;
    const int bh = blockIdx.x, b = bh / H, h = bh % H;
    // Per batch element, every [T, H, D] tensor is addressed from a wave-uniform
    // base with 32-bit element offsets (the host checks T*H*D fits).
    const uint32_t rs = (uint32_t)H * D;         // token stride (elements)
    // Batch element b holds tokens tok0 .. tok0 + T - 1: T_ tokens each, or,
    // for packed sequences, those between the offsets cu[b] and cu[b + 1]
    // (clamped to [0, T_], so bad offsets cannot reach outside the tensors).
    int tok0 = b * T_, T = T_;
    if (cu) {
        tok0 = min(max(cu[b], 0), T_);
        T = min(max(cu[b + 1], tok0), T_) - tok0;
    }
    const size_t bbase = (size_t)tok0 * H * D;
    const E* qb = q + bbase;
    const E* kb = k + bbase;
    const E* vb = v + bbase;
    const E* fb = f + bbase;
    E* ob = o ? o + bbase : nullptr;
    const uint32_t hoff = (uint32_t)h * D;
    const int NC = (T + CH - 1) / CH;

    // ---- producer ownership: the 16 rows rb .. rb+15 of sub-block I and the two
    // channels ch0, ch0 + 1 (the decay scans stay inside the lane); at d = 128
    // each producer wave owns one whole sub-block, so I is wave-uniform.
    const int ptid = tid - NWC * 64;
    const int I = (D == 128) ? __builtin_amdgcn_readfirstlane(w - NWC) : ptid / (D / 2);
    const int ch0 = 2 * (ptid % (D / 2));
    const int pc0 = TR::pcol(ch0);   // ch0 and ch0 + 1 stay adjacent under pcol
    const int rb = SB * I;
    // ---- consumer ownership: value columns 32w .. 32w+31
    const int i0 = 32 * w;

    if (NC == 0) {   // empty sequence: S_T = S0
        if (ST)
            for (int x = tid; x < D * D; x += NT)
                ST[(size_t)bh * D * D + x] = S0 ? S0[(size_t)bh * D * D + x] : 0.f;
        return;
    }

    // ---- one-time init: the upper triangles of M and P are never written
    constexpr int NFW = (D + 31) / 32;
    for (int x = tid; x < 2 * CH * LDP; x += NT) (&sm.P[0][0])[x] = TR::cvt(0.f);
    for (int x = tid; x < CH * LDM; x += NT) sm.M[x] = 0.f;
    if (tid < 2 * NSB * NFW) (&sm.fbm[0][0][0])[tid] = 0u;
    if (tid == 0) {
        for (int s = 0; s < 3; ++s) { sm.kmax[s] = 0u; sm.vmax[s] = 0u; }
        sm.fbany[0] = sm.fbany[1] = 0u;
        sm.umax = 0u;
    }

    lds_barrier();

    // Both teams run the same loop of barriers, one per stage.  Each team's
    // registers live only in its own loop.
    if (consumer) {
        floatx4 S[2][D / 16];   // S^T[16mj + 4g + r][i0 + 16nt + cl] in S[nt][mj]
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int mj = 0; mj < D / 16; ++mj)   // four adjacent columns: one 16-byte load
                S[nt][mj] = S0 ? *reinterpret_cast<const floatx4*>(
                                     &S0[(size_t)bh * D * D + (size_t)(i0 + 16 * nt + cl) * D + 16 * mj + 4 * g])
                               : floatx4{0.f, 0.f, 0.f, 0.f};

        for (int n = -1; n < NC; ++n) {
            const int nn = n + 1;
            // ======================================================= stage A
            KD_PHASE_MARK(n, 0);
            floatx4 Ot[2][NSB];   // O^T[i0 + 16mt + 4g + r][16tt + cl], lives to stage C
            if (n >= 0) {
                if (CKPT) {   // chunk-start state for the backward: S[i][j] (bf16: in record order)
                    E* dst = static_cast<E*>(ck.S) + ((size_t)bh * NC + n) * D * D;
                    if constexpr (std::is_same<TR, Bf16T>::value) {
#pragma unroll
                        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                            for (int kb = 0; kb < D / 32; ++kb)
                                st_run_nt(dst + rec_run<D>(i0 + 16 * nt + cl, kb, g), S[nt][2 * kb], S[nt][2 * kb + 1], 1.f);
                    } else {
#pragma unroll
                        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                            for (int mj = 0; mj < D / 16; ++mj)
                                st4_nt(dst + ((uint32_t)(i0 + 16 * nt + cl) * D + 16 * mj + 4 * g), S[nt][mj]);
                    }
                }
                // Y^T = S Kbar^T and O^T = S Qbar^T (M = value index i, N = token t),
                // sub-block by sub-block as S_tt Kloc^T and S_tt Qloc^T, the state
                // decayed in place to the start of sub-block tt
                floatx4 Yt[2][NSB];
#pragma unroll
                for (int tt = 0; tt < NSB; ++tt) {
#pragma unroll
                    for (int ks = 0; ks < KD_; ++ks) {
                        const Frag a0 = TR::state_frag(S[0], ks);
                        const Frag a1 = TR::state_frag(S[1], ks);
                        const floatx4 z = {0.f, 0.f, 0.f, 0.f};   // first K-step: inline-zero accumulator
                        const Frag bk = TR::ld_state_p(&sm.Kb[(SB * tt + cl) * LD], ks, g);
                        const Frag bq = TR::ld_state_p(&sm.Qb[(SB * tt + cl) * LD], ks, g);
                        Yt[0][tt] = TR::mma(a0, bk, ks ? Yt[0][tt] : z);
                        Yt[1][tt] = TR::mma(a1, bk, ks ? Yt[1][tt] : z);
                        Ot[0][tt] = TR::mma(a0, bq, ks ? Ot[0][tt] : z);
                        Ot[1][tt] = TR::mma(a1, bq, ks ? Ot[1][tt] : z);
                    }
                    if (tt + 1 < NSB) {
#pragma unroll
                        for (int mj = 0; mj < D / 16; ++mj) {
                            const floatx4 dc = *reinterpret_cast<const floatx4*>(&sm.fac[7 + tt][16 * mj + 4 * g]);
                            S[0][mj] = S[0][mj] * dc;
                            S[1][mj] = S[1][mj] * dc;
                        }
                    }
                }
                // partial r0[t] = sum over this wave's 32 value columns of Y[t,i] v[t,i]
#pragma unroll
                for (int tt = 0; tt < NSB; ++tt) {
                    float x = 0.f;
#pragma unroll
                    for (int mt = 0; mt < 2; ++mt) {
                        const E* vr = &sm.V[(SB * tt + cl) * LD + TR::pcol(i0 + 16 * mt + 4 * g)];
#pragma unroll
                        for (int r = 0; r < 4; ++r) x += Yt[mt][tt][r] * TR::tof(vr[r]);
                    }
                    x += __shfl_xor(x, 16, 64);
                    x += __shfl_xor(x, 32, 64);
                    if (g == 0) sm.r0p[w][SB * tt + cl] = x;
                }
            }
            KD_PHASE_MARK(n, 3);
            lds_barrier();
            // ======================================================= stage B
            KD_PHASE_MARK(n, 1);
            if (n >= 0 && w == 0) {   // forward substitution (I + M) u = c - beta r0
                const int t_ = lane;
                float r0 = 0.f;
#pragma unroll
                for (int ww = 0; ww < NWC; ++ww) r0 += sm.r0p[ww][t_];
                float x = sm.c[n & 1][t_] - sm.beta[n & 1][t_] * r0;
                float Mrow[CH];
#pragma unroll
                for (int s4 = 0; s4 < CH / 4; ++s4) {
                    const floatx4 m4 = *reinterpret_cast<const floatx4*>(&sm.M[t_ * LDM + 4 * s4]);
                    Mrow[4 * s4] = m4[0]; Mrow[4 * s4 + 1] = m4[1]; Mrow[4 * s4 + 2] = m4[2]; Mrow[4 * s4 + 3] = m4[3];
                }
                // M is strictly lower triangular (zeros elsewhere), so the update
                // needs no lane mask: lane t only changes while s < t.
#pragma unroll
                for (int s = 0; s < CH - 1; ++s) x = fmaf(-Mrow[s], readlane_f(x, s), x);
                sm.u[t_] = x;
                if (CKPT) {   // u and r0 of the chunk for the backward
                    float* du = ck.U + ((size_t)bh * NC + n) * 2 * CH;
                    st_nt(&du[t_], x);
                    st_nt(&du[CH + t_], r0);
                }
                const float um = wave_max_nonneg(fabsf(x));
                if (lane == 0) sm.umax = __float_as_uint(um);
            }
            if (CKPT && n >= 0) {
                // M and P of chunk n are complete and nobody writes them in this
                // stage: the consumer waves copy them out ([CH][CH] row-major)
                constexpr int EPV = 16 / sizeof(E);   // elements per 16-byte move
                float* dm = ck.M + ((size_t)bh * NC + n) * CH * CH;
                E* dp = static_cast<E*>(ck.P) + ((size_t)bh * NC + n) * CH * CH;
                for (int x = tid; x < CH * CH / 4; x += NWC * 64) {
                    const int t = x / (CH / 4), s4 = x % (CH / 4);
                    cp16_nt(dm + t * CH + 4 * s4, &sm.M[t * LDM + 4 * s4]);
                }
                for (int x = tid; x < CH * CH / EPV; x += NWC * 64) {
                    const int t = x / (CH / EPV), sv = x % (CH / EPV);
                    cp16_nt(dp + t * CH + EPV * sv, &sm.P[n & 1][t * LDP + EPV * sv]);
                }
            }
            if (tid == 0 && n >= 0) {
                // slot (n+2)%3 = chunks n-1 and n+2: the former's last reader ran in
                // the previous stage C, the latter's first writer runs in stage A(n+1)
                sm.kmax[(n + 2) % 3] = 0u; sm.vmax[(n + 2) % 3] = 0u;
            }
            if (tid < NSB * NFW && n >= 0) {
                // chunk n's flags were last read in stage A; chunk n + 2 sets them
                // in stage B(n + 1)
                (&sm.fbm[n & 1][0][0])[tid] = 0u;
                if (tid == 0) sm.fbany[n & 1] = 0u;
            }
            KD_PHASE_MARK(n, 4);
            lds_barrier();
            // ======================================================= stage C
            KD_PHASE_MARK(n, 2);
            if (n >= 0) {   // readout and state update of chunk n
                const float usc = pow2_scale(__uint_as_float(sm.umax) * __uint_as_float(sm.vmax[n % 3]));
                const float ksc = pow2_scale(__uint_as_float(sm.kmax[n % 3]));
                const float inv = 1.f / (usc * ksc);
                // O^T += W^T P^T with W = u * V (bf16), then O leaves as 8-byte rows
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
                    for (int ks = 0; ks < KC_; ++ks) {
                        const Frag wa = TR::row_times(&sm.VT[(i0 + 16 * mt + cl) * LDT], sm.u, ks, g);
#pragma unroll
                        for (int tt = 0; tt < NSB; ++tt)
                            Ot[mt][tt] = TR::mma(wa, TR::ld_nat(&sm.P[n & 1][(SB * tt + cl) * LDP], ks, g), Ot[mt][tt]);
                    }
                }
                if (ob) {
#pragma unroll
                    for (int tt = 0; tt < NSB; ++tt) {
                        const int t = n * CH + SB * tt + cl;
                        if (t < T) {
#pragma unroll
                            for (int mt = 0; mt < 2; ++mt)
                                st4_nt(ob + (uint32_t)t * rs + hoff + i0 + 16 * mt + 4 * g, Ot[mt][tt]);
                        }
                    }
                }
                // S <- (S diag(gamma_C) s + K~'^T W') / s with s = usc * ksc (exact powers of 2)
                FragH wb[2][KC_];
#pragma unroll
                for (int ks = 0; ks < KC_; ++ks)
                    TR::rows_times_h2(&sm.VT[(i0 + cl) * LDT], &sm.VT[(i0 + 16 + cl) * LDT], sm.u, usc,
                                      ks, g, wb[0][ks], wb[1][ks]);
#pragma unroll
                for (int mj = 0; mj < D / 16; ++mj) {
                    const floatx4 gm = *reinterpret_cast<const floatx4*>(&sm.gam[n & 1][16 * mj + 4 * g]) * (usc * ksc);
                    S[0][mj] = S[0][mj] * gm;
                    S[1][mj] = S[1][mj] * gm;
#pragma unroll
                    for (int ks = 0; ks < KC_; ++ks) {
                        const FragH ak = TR::ld_nat_h(&sm.KtT[(16 * mj + cl) * LDT], ks, g);
                        S[0][mj] = TR::mma_h(ak, wb[0][ks], S[0][mj]);
                        S[1][mj] = TR::mma_h(ak, wb[1][ks], S[1][mj]);
                    }
                    S[0][mj] = S[0][mj] * inv;
                    S[1][mj] = S[1][mj] * inv;
                }
            }
            KD_PHASE_MARK(n, 5);
            lds_barrier();
        }
        if (ST) {
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
#pragma unroll
                for (int mj = 0; mj < D / 16; ++mj)   // four adjacent columns: one 16-byte store
                    st4_nt(&ST[(size_t)bh * D * D + (size_t)(i0 + 16 * nt + cl) * D + 16 * mj + 4 * g], S[nt][mj]);
        }
    } else {
        Raw16x2<TR> rq, rk, rv, rf;         // raw rows of the chunk being prepared
        float rb_beta = 0.f, rb_c = 0.f;    // beta_t, c_t for t = ptid (ptid < CH)
        float tot[2];                       // product of f over the sub-block, per channel
        Col16<E> keep_v[2];                 // v and K-tilde of the prepared chunk, written
        Col16<Hh> keep_kt[2];               //   transposed in the following stage A
        // Rows past the sequence end re-read the last row (in bounds) and are
        // cleared before use (q = k = v = 0, f = 1, beta = c = 0).  Every load
        // is unconditional (clamped to the last chunk), so the prefetch
        // registers are never merged with older values: a merge makes the
        // compiler copy them and wait for the loads right away.
        auto row_off = [&](int n, int& last) {
            const int t0 = min(n * CH + rb, T - 1);
            last = min(SB - 1, T - 1 - t0);
            return (uint32_t)t0 * rs + hoff + ch0;
        };
        auto load_q = [&](int n) {   // with beta and c (lanes past the first wave re-read its tokens)
            int last;
            const uint32_t off = row_off(n, last);
            rq.load(qb, off, rs, last);
            const int t = min(n * CH + (ptid & (CH - 1)), T - 1);
            const uint32_t gi = ((uint32_t)t * H + h);
            rb_beta = beta[(size_t)tok0 * H + gi];
            rb_c = cc[(size_t)tok0 * H + gi];
        };
        auto load_k = [&](int n) { int last; const uint32_t off = row_off(n, last); rk.load(kb, off, rs, last); };
        auto load_v = [&](int n) { int last; const uint32_t off = row_off(n, last); rv.load(vb, off, rs, last); };
        auto load_f = [&](int n) { int last; const uint32_t off = row_off(n, last); rf.load(fb, off, rs, last); };
        load_q(0);
        load_k(0);
        load_v(0);
        load_f(0);
        // Exact terms of the diagonal tile I_ of chunk ch for the key channels
        // whose decay over that sub-block is below the floor (left out of the
        // tile's matrix product), added to M and P in LDS before they are read:
        // lane (g, cl) takes the entries t = 4g + r, s = cl (rows of the
        // sub-block) and sums over those channels k_t k_s E (G_K, s < t) and
        // q_t k_s E (P, s <= t), E = prod_{s<u<=t} f_u; then M[t][s] += beta_t
        // dG_K G_V[t][s] (G_V again from V) and P[t][s] += dP.  Rare path: the
        // rows are re-read from global memory.
        auto diag_exact = [&](int I_, int ch) {
            const unsigned* fm = sm.fbm[ch & 1][I_];
            const int row0 = ch * CH + SB * I_;
            floatx4 dk = {0.f, 0.f, 0.f, 0.f}, dp = dk;
#pragma unroll 1
            for (int wd = 0; wd < NFW; ++wd) {
                unsigned bits = __builtin_amdgcn_readfirstlane(fm[wd]);
#pragma unroll 1
                while (bits) {
                    const int j = 32 * wd + __builtin_ctz(bits);
                    bits &= bits - 1u;
                    const uint32_t cj = hoff + (uint32_t)j;
                    auto ldv = [&](const E* p, int x) {
                        const int t = row0 + x;
                        return t < T ? TR::tof(p[(uint32_t)t * rs + cj]) : 0.f;
                    };
                    const float fl = row0 + cl < T ? TR::tof(fb[(uint32_t)(row0 + cl) * rs + cj]) : 1.f;
                    const float ksv = ldv(kb, cl);
                    float e4[4] = {1.f, 1.f, 1.f, 1.f};
#pragma unroll 1
                    for (int u = 1; u < SB; ++u) {
                        const float fu = readlane_f(fl, u);
#pragma unroll
                        for (int r = 0; r < 4; ++r) e4[r] = (u > cl && u <= 4 * g + r) ? e4[r] * fu : e4[r];
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int t = 4 * g + r;
                        const float w_ = ksv * e4[r];
                        if (t > cl) dk[r] += ldv(kb, t) * w_;
                        if (t >= cl) dp[r] += ldv(qb, t) * w_;
                    }
                }
            }
            floatx4 gv = {0.f, 0.f, 0.f, 0.f};
            const E* aV = &sm.V[(SB * I_ + cl) * LD];
#pragma unroll
            for (int ks = 0; ks < KD_; ++ks) gv = TR::mma(TR::ld_nat(aV, ks, g), TR::ld_nat(aV, ks, g), gv);
            const int s_ = SB * I_ + cl;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t_ = SB * I_ + 4 * g + r;
                if (s_ < t_) sm.M[t_ * LDM + s_] += sm.beta[ch & 1][t_] * dk[r] * gv[r];
                if (s_ <= t_) {
                    E& pe = sm.P[ch & 1][t_ * LDP + s_];
                    pe = TR::cvt(TR::tof(pe) + dp[r]);
                }
            }
        };
        // One lower-triangular 16 x 16 tile (I_ >= J_) of M (DO_M) and / or P
        // (DO_P) for chunk ch, whose operands are in LDS.  The M part writes
        // only the strictly lower entries of M (the diagonal and the upper
        // triangle stay zero), the P part the tile's entries of P: the two parts
        // never touch the same entry, so they may run on different waves in any
        // order.  The decay between the two sub-blocks goes on the Kr fragment
        // (fac row fr).
        auto gram_tile = [&](auto do_m, auto do_p, int tile, int ch) {
            constexpr bool DO_M = decltype(do_m)::value, DO_P = decltype(do_p)::value;
            const int I_ = tile < 1 ? 0 : tile < 3 ? 1 : tile < 6 ? 2 : 3;
            const int J_ = tile - (I_ * (I_ + 1)) / 2;
            const int fr = I_ == J_ ? I_ : I_ - J_ == 2 ? (J_ == 0 ? 4 : 5) : I_ - J_ == 3 ? 6 : -1;
            floatx4 gk, pp, gv;
            const E* aK = &sm.Kb[(SB * I_ + cl) * LD];
            const E* aQ = &sm.Qb[(SB * I_ + cl) * LD];
            const E* aV = &sm.V[(SB * I_ + cl) * LD];
            const E* bK = &sm.Kc[(SB * J_ + cl) * LD];
            const E* bV = &sm.V[(SB * J_ + cl) * LD];
#pragma unroll
            for (int ks = 0; ks < KD_; ++ks) {
                const floatx4 z = {0.f, 0.f, 0.f, 0.f};
                Frag fk = TR::ld_nat(bK, ks, g);
                if (fr >= 0) fk = TR::scale_k(fk, 1.f, sm.fac[fr], ks, g);
                if (DO_M) gk = TR::mma(TR::ld_nat(aK, ks, g), fk, ks ? gk : z);
                if (DO_P) pp = TR::mma(TR::ld_nat(aQ, ks, g), fk, ks ? pp : z);
                if (DO_M) gv = TR::mma(TR::ld_nat(aV, ks, g), TR::ld_nat(bV, ks, g), ks ? gv : z);
            }
            const int s_ = SB * J_ + cl;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t_ = SB * I_ + 4 * g + r;
                if (DO_M && s_ < t_) sm.M[t_ * LDM + s_] = sm.beta[ch & 1][t_] * gk[r] * gv[r];
                if (DO_P) sm.P[ch & 1][t_ * LDP + s_] = TR::cvt((s_ <= t_) ? pp[r] : 0.f);
            }
        };
        typedef std::integral_constant<bool, true> kYes;
        typedef std::integral_constant<bool, false> kNo;
        // Gram tiles per producer wave.  At d = 128 tiles 8 and 9 wait for the
        // next stage A, where the producers have slack (their M entries are
        // first read by the forward substitution of stage B, their P entries by
        // the readout of stage C), split over the four producer waves: the M
        // parts on the first two, the P parts on the other two.
        constexpr int NTPW = (10 + NWP - 1) / NWP;
        constexpr int NTPW_C = (D == 128) ? 2 : NTPW;

        for (int n = -1; n < NC; ++n) {
            const int nn = n + 1;             // chunk the producers prepare
            const bool prod_on = nn < NC;
            // ======================================================= stage A
            KD_PHASE_MARK(n, 0);
            if (n >= 0) {   // transposed operands of chunk n, and its remaining Gram tiles
#pragma unroll
                for (int c2 = 0; c2 < 2; ++c2) {
                    keep_v[c2].store(&sm.VT[(ch0 + c2) * LDT + rb]);
                    keep_kt[c2].store(&sm.KtT[(ch0 + c2) * LDT + rb]);
                }
                if (D == 128) {
                    const int pw = w - NWC;   // producer wave 0..3
                    if (pw >= 2) gram_tile(kNo(), kYes(), 8 + (pw & 1), n);
                    else gram_tile(kYes(), kNo(), 8 + (pw & 1), n);
                }
                // every tile of chunk n is done (D < 128: in the last stage C)
                if (D < 128 && sm.fbany[n & 1] != 0u) {
                    const int pw = w - NWC;
#pragma unroll 1
                    for (int I2 = pw; I2 < NSB; I2 += NWP) diag_exact(I2, n);
                }
            }
            if (prod_on) {   // decay products of chunk nn
                if (nn * CH + CH > T) {   // ragged last chunk: clear rows past the end
#pragma unroll
                    for (int e = 0; e < SB; ++e)
                        if (nn * CH + rb + e >= T) {
                            rq.clear(e, 0.f); rk.clear(e, 0.f); rv.clear(e, 0.f); rf.clear(e, 1.f);
                        }
                    if (ptid < CH && nn * CH + ptid >= T) { rb_beta = 0.f; rb_c = 0.f; }
                }
#pragma unroll
                for (int c2 = 0; c2 < 2; ++c2) {   // pairwise tree over the 16 rows
                    float x[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[e] = rf.get(2 * e, c2) * rf.get(2 * e + 1, c2);
                    tot[c2] = ((x[0] * x[1]) * (x[2] * x[3])) * ((x[4] * x[5]) * (x[6] * x[7]));
                }
                st2(&sm.bprod[I][ch0], tot[0], tot[1]);   // sub-block products
                const float km = wave_max_nonneg(rk.absmax());
                const float vm = wave_max_nonneg(rv.absmax());
                if (lane == 0) {   // non-negative floats order like their bit patterns
                    atomicMax(&sm.kmax[nn % 3], __float_as_uint(km));
                    atomicMax(&sm.vmax[nn % 3], __float_as_uint(vm));
                }
                if (ptid < CH) {
                    sm.beta[nn & 1][ptid] = rb_beta;
                    sm.c[nn & 1][ptid] = rb_c;
                }
            }
            KD_PHASE_MARK(n, 3);
            lds_barrier();
            // ======================================================= stage B
            KD_PHASE_MARK(n, 1);
            if (prod_on) {   // operands of chunk nn into LDS
                // decay over each sub-block (bp), the factor rows this lane
                // writes, and the decay of the sub-blocks after this one
                float bp[NSB][2];
#pragma unroll
                for (int I2 = 0; I2 < NSB; ++I2) {
                    const float2 x = *reinterpret_cast<const float2*>(&sm.bprod[I2][ch0]);
                    bp[I2][0] = x.x; bp[I2][1] = x.y;
                }
                float after[2] = {1.f, 1.f};
#pragma unroll
                for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
                    for (int I2 = 1; I2 < NSB; ++I2)
                        if (I2 > I) after[c2] *= bp[I2][c2];
                auto facv = [&](int row, int c2) {
                    if (row < 4) return bp[row][c2] >= kSafeFloor ? __builtin_amdgcn_rcpf(bp[row][c2]) : 0.f;
                    if (row == 4) return bp[1][c2];
                    if (row == 5) return bp[2][c2];
                    if (row == 6) return bp[1][c2] * bp[2][c2];
                    return bp[row - 7][c2];
                };
                // the lanes of sub-block I write rows I, I + 4 (and 8 + I for I < 2)
                st2(&sm.fac[I][pc0], facv(I, 0), facv(I, 1));
                if (I < 3) st2(&sm.fac[4 + I][pc0], facv(4 + I, 0), facv(4 + I, 1));
                if (I == 3) st2(&sm.fac[7][ch0], facv(7, 0), facv(7, 1));
                if (I < 2) st2(&sm.fac[8 + I][ch0], facv(8 + I, 0), facv(8 + I, 1));
                {   // channels of sub-block I below the floor (rare)
                    const unsigned fl2 = (bp[I][0] >= kSafeFloor ? 0u : 1u) | (bp[I][1] >= kSafeFloor ? 0u : 2u);
                    if (fl2) {
                        atomicOr(&sm.fbm[nn & 1][I][ch0 >> 5], fl2 << (ch0 & 31));
                        atomicOr(&sm.fbany[nn & 1], 1u);
                    }
                }
                if (I == NSB - 1) st2(&sm.gam[nn & 1][ch0], bp[NSB - 1][0], bp[NSB - 1][1]);
                const float ksc = pow2_scale(__uint_as_float(sm.kmax[nn % 3]));
                // b (to the sub-block end) as suffix products within the
                // sub-block; gamma_C / gamma = b * after
                float bs[SB][2];
#pragma unroll
                for (int c2 = 0; c2 < 2; ++c2) {
                    bs[SB - 1][c2] = 1.f;
#pragma unroll
                    for (int e = SB - 2; e >= 0; --e) bs[e][c2] = bs[e + 1][c2] * rf.get(e + 1, c2);
                }
                float ga[2] = {1.f, 1.f};   // a at the current row (running prefix)
                float kprev[2] = {0.f, 0.f};
#pragma unroll
                for (int e = 0; e < SB; ++e) {
                    float qo[2], ko[2], co[2];
#pragma unroll
                    for (int c2 = 0; c2 < 2; ++c2) {
                        ga[c2] *= rf.get(e, c2);
                        const float kf = rk.get(e, c2), qf = rq.get(e, c2);
                        const float kt = kf * (bs[e][c2] * after[c2]);   // K-tilde
                        qo[c2] = qf * ga[c2];
                        ko[c2] = kf * ga[c2];
                        co[c2] = kf * bs[e][c2];
                        if (e & 1) keep_kt[c2].set_pair(e >> 1, kprev[c2], kt * ksc);
                        else kprev[c2] = kt * ksc;
                    }
                    st2(&sm.Qb[(rb + e) * LD + pc0], qo[0], qo[1]);
                    st2(&sm.Kb[(rb + e) * LD + pc0], ko[0], ko[1]);
                    st2(&sm.Kc[(rb + e) * LD + pc0], co[0], co[1]);
                    rv.store(&sm.V[(rb + e) * LD + pc0], e);
                }
#pragma unroll
                for (int c2 = 0; c2 < 2; ++c2) keep_v[c2].set_raw(rv, c2);
            }
            // Prefetch of chunk nn + 1, spread over the end of this stage and the
            // Gram of the next: when every workgroup requested its whole chunk at
            // once, the issuing wave stalled until HBM drained the burst.
            const int npf = min(nn + 1, NC - 1);
            load_q(npf);
            KD_PHASE_MARK(n, 4);
            lds_barrier();
            // ======================================================= stage C
            KD_PHASE_MARK(n, 2);
            load_k(npf);
#pragma unroll
            for (int it = 0; it < NTPW_C; ++it) {   // Gram tiles of chunk nn: M and P
                const int tile = w - NWC + it * NWP;
                if (prod_on && tile < 10) gram_tile(kYes(), kYes(), tile, nn);
                // (it is a compile-time constant in each unrolled copy: no branch)
                if (it == 0) load_v(npf);
                if (it == 1) load_f(npf);
            }
            KD_PHASE_MARK(n, 5);
            lds_barrier();
        }
    }
}

// --------------------------------------------------------------- launchers
template <class TR, int D>
static hipError_t launch_fwd_t(const void* q, const void* k, const void* v, const void* f,
                               const float* beta, const float* c, const float* S0, void* o,
                               float* ST, const FwdCkpt* ck, const int* cu, int B, int T, int H,
                               hipStream_t st)
{
    typedef typename TR::E E;
    if (ck)
        hipLaunchKernelGGL((kd_fwd_kernel<TR, D, true>), dim3((unsigned)(B * H)), dim3(4 * D), 0, st,
                           (const E*)q, (const E*)k, (const E*)v, (const E*)f, beta, c, S0, (E*)o, ST,
                           *ck, (const int*)nullptr, T, H);
    else
        hipLaunchKernelGGL((kd_fwd_kernel<TR, D, false>), dim3((unsigned)(B * H)), dim3(4 * D), 0, st,
                           (const E*)q, (const E*)k, (const E*)v, (const E*)f, beta, c, S0, (E*)o, ST,
                           FwdCkpt{}, cu, T, H);
    return hipGetLastError();
}

hipError_t launch_fwd16(const void* q, const void* k, const void* v, const void* f, const float* beta,
                        const float* c, const float* S0, void* o, float* ST, const FwdCkpt* ck,
                        const int* cu, int B, int T, int H, hipStream_t st);

// ck: the checkpoint records to fill (the backward's recompute), or null.
// cu: null, or the B + 1 token offsets of packed sequences (T = total tokens;
// not combined with ck).
hipError_t launch_fwd(int bf16, int d, const void* q, const void* k, const void* v, const void* f,
                      const float* beta, const float* c, const float* S0, void* o, float* ST,
                      const FwdCkpt* ck, const int* cu, int B, int T, int H, hipStream_t st)
{
#define KD_FWD_ARGS q, k, v, f, beta, c, S0, o, ST, ck, cu, B, T, H, st
    if (bf16) {
        switch (d) {
        case 32: return launch_fwd_t<Bf16T, 32>(KD_FWD_ARGS);
        case 64: return launch_fwd_t<Bf16T, 64>(KD_FWD_ARGS);
        case 128: return launch_fwd16(KD_FWD_ARGS);   // sixteen-wave kernel (kd_fwd16.hip)
        }
    } else {
        switch (d) {
        case 32: return launch_fwd_t<F32T, 32>(KD_FWD_ARGS);
        case 64: return launch_fwd_t<F32T, 64>(KD_FWD_ARGS);
        }
    }
#undef KD_FWD_ARGS
    return hipErrorInvalidValue;
}

}  // namespace kd
