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
//  * One workgroup per (b, h); 4*d threads = d/16 waves; the chunk loop runs
//    inside the kernel, so the fp32 state never leaves the chip.  The state is
//    held TRANSPOSED (S^T, key index j as rows) as MFMA accumulators, wave w
//    owning value columns i in [16w, 16w + 16).  In that orientation the
//    accumulator registers are directly the B operand of both products that
//    read the state (O_inter = Qbar S0^T and Y = Kbar S0^T), so the state needs
//    no LDS round trip.
//  * Decay folding: Qbar = q*gamma, Kbar = k*gamma and Kc = k/gamma are the
//    MFMA operands of every Gram tile and of the state reads (one operand set,
//    no per-tile rescaling).  Kc needs gamma >= 2^-100; a key channel whose
//    decay over the chunk falls below that has its Kc column zeroed and its
//    Gram terms accumulated exactly by a scalar fallback, so every input in
//    [0, 1] is handled exactly.  K * gamma_C/gamma is built from suffix
//    products, which never divide.
//  * Per chunk: prep (decay products, operands into LDS) -> Gram tiles and
//    state reads (MFMA) -> forward substitution (one wave, lane t owns row t,
//    readlane broadcast) -> O and state update (MFMA).  The next chunk's
//    global loads are issued right after the prep so they overlap the MFMA
//    phases; O leaves through LDS as full 16-byte row segments.
#include "kd_device.h"

// Phase markers: no-ops here; a profiling build may define them to record
// timestamps at the phase boundaries of the chunk loop.
#ifndef KD_PHASE_MARK
#define KD_PHASE_MARK(chunk, id) ((void)0)
#endif

namespace kd {

constexpr float kSafeFloor = 7.888609052210118e-31f;  // 2^-100

template <class TR, int D>
struct FwdSmem {
    typedef typename TR::E E;
    static constexpr int LD = D + TR::PAD;     // row-major [CH][D] arrays
    static constexpr int LDT = CH + TR::PAD;   // transposed [D][CH] arrays
    static constexpr int LDM = CH + 4;         // fp32 M
    static constexpr int LDP = CH + TR::PAD;   // P
    alignas(16) E Qb[CH * LD];     // q * gamma
    alignas(16) E Kb[CH * LD];     // k * gamma
    alignas(16) E Kc[CH * LD];     // k / gamma (0 for fallback channels); O staging after the Gram
    alignas(16) E V[CH * LD];      // v
    alignas(16) E VT[D * LDT];     // v^T
    alignas(16) typename TR::H KtT[D * LDT];   // (k * gamma_C / gamma)^T * kscale (state-update precision)
    alignas(16) float M[CH * LDM]; // beta_t tril_{-1}(G_K * G_V); fallback scratch
    alignas(16) E P[CH * LDP];     // tril_0 of the decayed Q K^T
    alignas(16) float beta[CH];
    alignas(16) float c[CH];
    alignas(16) float u[CH];
    alignas(16) float r0p[D / 16][CH];
    alignas(16) float bprod[NSB][D];   // product of f over each 16-token sub-block
    alignas(16) float gam[D];          // gamma_C
    unsigned unsafe_any;
    unsigned kmax_bits;                // max |k| over the chunk (fp32 bits)
    unsigned vmax_bits[2];             // max |v| over the chunk (fp32 bits), by chunk parity
    unsigned umax_bits;                // max |u| over the chunk (fp32 bits)
};

template <class TR, int D>
__global__ __launch_bounds__(4 * D) void kd_fwd_kernel(
    const typename TR::E* __restrict__ q, const typename TR::E* __restrict__ k,
    const typename TR::E* __restrict__ v, const typename TR::E* __restrict__ f,
    const float* __restrict__ beta, const float* __restrict__ cc,
    const float* __restrict__ S0, typename TR::E* __restrict__ o, float* __restrict__ ST,
    float* __restrict__ ckpt, int T, int H)
{
    typedef typename TR::E E;
    typedef typename TR::Frag Frag;
    typedef FwdSmem<TR, D> SM;
    constexpr int NT = 4 * D;
    constexpr int NW = D / 16;
    constexpr int KD_ = D / TR::KS;   // K-steps over a d-long contraction
    constexpr int KC_ = CH / TR::KS;  // K-steps over a chunk-long contraction
    constexpr int LD = SM::LD, LDT = SM::LDT, LDM = SM::LDM, LDP = SM::LDP;
    constexpr int EPV = 16 / sizeof(E);   // elements per 16-byte vector

    __shared__ SM sm;

    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6, g = lane >> 4, cl = lane & 15;
    // prep ownership: rows row0, row0 + 1 of the chunk and channels ch0 .. ch0+7;
    // the eight row pairs of a 16-row sub-block sit in one aligned 8-lane group.
    const int r8 = lane & 7;
    const int qd = w * 8 + (lane >> 3);
    const int I = qd / (D / 8), ch0 = 8 * (qd % (D / 8));
    const int row0 = SB * I + 2 * r8;
    const int bh = blockIdx.x, b = bh / H, h = bh % H;
    // Per batch element, every [T, H, D] tensor is addressed from a wave-uniform
    // base with 32-bit element offsets (the host checks T*H*D fits).
    const uint32_t rs = (uint32_t)H * D;         // token stride (elements)
    const size_t bbase = (size_t)b * T * H * D;
    const E* qb = q + bbase;
    const E* kb = k + bbase;
    const E* vb = v + bbase;
    const E* fb = f + bbase;
    E* ob = o ? o + bbase : nullptr;
    const float* gsrc = (tid < CH ? beta : cc) + (size_t)b * T * H;
    const uint32_t hoff = (uint32_t)h * D;
    const int NC = (T + CH - 1) / CH;

    // ---- one-time init
    for (int x = tid; x < CH * LDP; x += NT) sm.P[x] = TR::cvt(0.f);
    if (tid == 0) {
        sm.unsafe_any = 0u; sm.kmax_bits = 0u; sm.umax_bits = 0u;
        sm.vmax_bits[0] = 0u; sm.vmax_bits[1] = 0u;
    }

    floatx4 S[D / 16];   // S^T[16mt + 4g + r][16w + cl]
#pragma unroll
    for (int mt = 0; mt < D / 16; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            S[mt][r] = S0 ? S0[(size_t)bh * D * D + (size_t)(16 * w + cl) * D + 16 * mt + 4 * g + r] : 0.f;

    // ---- prefetch registers (rows row0, row0 + 1; channels ch0 .. ch0 + 7)
    Row2x8<TR> rq, rk, rv, rf;
    float rbc = 0.f;
    auto load_chunk = [&](int n) {
        // Rows past the sequence end re-read the last row (in bounds) and are
        // cleared in the prep (q = k = v = 0, f = 1, beta = c = 0).
        const int ta = min(n * CH + row0, T - 1), tb = min(n * CH + row0 + 1, T - 1);
        const uint32_t oa = (uint32_t)ta * rs + hoff + ch0, ob2 = (uint32_t)tb * rs + hoff + ch0;
        rq.load(qb, oa, ob2);
        rk.load(kb, oa, ob2);
        rv.load(vb, oa, ob2);
        rf.load(fb, oa, ob2);
        if (tid < 2 * CH) {
            const int t = min(n * CH + (tid & (CH - 1)), T - 1);
            rbc = gsrc[(uint32_t)t * H + h];
        }
    };
    // Coalesced output of a staged O tile (rows in sm.Kc).
    auto store_o = [&](int n) {
        constexpr int VPR = D / EPV;   // 16-byte vectors per row
        for (int x = tid; x < CH * VPR; x += NT) {
            const int t = x / VPR, cv = x % VPR;
            const int tg = n * CH + t;
            if (tg < T)
                *reinterpret_cast<uint4*>(ob + (uint32_t)tg * rs + hoff + cv * EPV) =
                    *reinterpret_cast<const uint4*>(&sm.Kc[t * LD + cv * EPV]);
        }
    };
    if (NC > 0) load_chunk(0);
    lds_barrier();

    for (int n = 0; n < NC; ++n) {
        if (ckpt) {   // chunk-start state, stored as S[i][j]
            float* dst = ckpt + ((size_t)bh * NC + n) * D * D;
#pragma unroll
            for (int mt = 0; mt < D / 16; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    dst[(size_t)(16 * w + cl) * D + 16 * mt + 4 * g + r] = S[mt][r];
        }
        KD_PHASE_MARK(n, 0);
        if (n > 0 && ob) store_o(n - 1);   // previous chunk's O, staged in Kc
        // ================= prep (a): decay products within the sub-block
        if (n * CH + CH > T) {   // ragged last chunk: clear rows past the end
#pragma unroll
            for (int e = 0; e < 2; ++e)
                if (n * CH + row0 + e >= T) {
                    rq.clear(e, 0.f); rk.clear(e, 0.f); rv.clear(e, 0.f); rf.clear(e, 1.f);
                }
            if (tid < 2 * CH && n * CH + (tid & (CH - 1)) >= T) rbc = 0.f;
        }
        float incl[8], excl[8];   // products of f from the sub-block start through row0+1 / before row0
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            incl[c] = group8_prefix_prod(rf.get(0, c) * rf.get(1, c), r8);
            excl[c] = group8_shift1(incl[c], r8);
        }
        if (r8 == 7) st8v(&sm.bprod[I][ch0], incl);   // sub-block products
        {   // chunk max |k| and |v|: exact power-of-two scales of the fp16
            // state-update operands
            float km = 0.f, vm = 0.f;
#pragma unroll
            for (int e = 0; e < 2; ++e)
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    km = fmaxf(km, fabsf(rk.get(e, c)));
                    vm = fmaxf(vm, fabsf(rv.get(e, c)));
                }
            km = wave_max_nonneg(km);
            vm = wave_max_nonneg(vm);
            if (lane == 0) {   // non-negative floats order like their bit patterns
                atomicMax(&sm.kmax_bits, __float_as_uint(km));
                atomicMax(&sm.vmax_bits[n & 1], __float_as_uint(vm));
            }
        }
        // clear M: it doubles as the scratch of the exact fallback
        for (int x = tid; x < CH * LDM / 4; x += NT)
            reinterpret_cast<floatx4*>(sm.M)[x] = floatx4{0.f, 0.f, 0.f, 0.f};
        lds_barrier();

        KD_PHASE_MARK(n, 1);
        // ================= prep (b): operands into LDS
        float ksc;            // 2^-e scaling the chunk's max |k| into [0.5, 1)
        unsigned unsafe = 0;  // bit c: channel ch0 + c decays below the floor in this chunk
        {
            float plt[8], gC[8];
#pragma unroll
            for (int c = 0; c < 8; ++c) { plt[c] = 1.f; gC[c] = 1.f; }
#pragma unroll
            for (int I2 = 0; I2 < NSB; ++I2) {
#pragma unroll
                for (int c4 = 0; c4 < 2; ++c4) {
                    const floatx4 x = *reinterpret_cast<const floatx4*>(&sm.bprod[I2][ch0 + 4 * c4]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        gC[4 * c4 + e] *= x[e];
                        if (I2 < I) plt[4 * c4 + e] *= x[e];
                    }
                }
            }
#pragma unroll
            for (int c = 0; c < 8; ++c)
                if (!(gC[c] >= kSafeFloor)) unsafe |= 1u << c;
            if (I == 0 && r8 == 0) st8v(&sm.gam[ch0], gC);
            if (unsafe) atomicOr(&sm.unsafe_any, 1u);
            ksc = pow2_scale(__uint_as_float(sm.kmax_bits));
            float kt[2][8], vt[2][8];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                float qo[8], ko[8], co[8];
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const float ga = plt[c] * (e == 0 ? excl[c] * rf.get(0, c) : incl[c]);
                    const float kf = rk.get(e, c), qf = rq.get(e, c);
                    const float kr = kf * __builtin_amdgcn_rcpf(ga);
                    const bool un = (unsafe >> c) & 1u;
                    qo[c] = qf * ga;
                    ko[c] = kf * ga;
                    co[c] = un ? 0.f : kr;
                    kt[e][c] = un ? 0.f : kr * (gC[c] * ksc);   // fallback channels: filled in later
                    vt[e][c] = rv.get(e, c);
                }
                st8v(&sm.Qb[(row0 + e) * LD + ch0], qo);
                st8v(&sm.Kb[(row0 + e) * LD + ch0], ko);
                st8v(&sm.Kc[(row0 + e) * LD + ch0], co);
                rv.store(&sm.V[(row0 + e) * LD + ch0], e);
            }
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                st2h(&sm.KtT[(ch0 + c) * LDT + row0], kt[0][c], kt[1][c]);
                st2(&sm.VT[(ch0 + c) * LDT + row0], vt[0][c], vt[1][c]);
            }
            if (I == 0 && r8 == 0 && unsafe) {
                // Exact Gram terms of a key channel whose chunk decay is below the
                // floor (its Kc column is zero, so the MFMA tiles leave it out):
                // G_K[t,s] (s<t) accumulates at M[t][s], P[t,s] (s<t) at M[s][t],
                // P[t,t] at M[t][t].  Rare path: rows are re-read from global memory.
                const int t0 = n * CH;
#pragma unroll 1
                for (int c = 0; c < 8; ++c) {
                    if (!((unsafe >> c) & 1u)) continue;
                    const uint32_t off = (uint32_t)t0 * rs + hoff + ch0 + c;
#pragma unroll 1
                    for (int s = 0; s < CH && t0 + s < T; ++s) {
                        const float ks_ = TR::tof(kb[off + s * rs]);
                        atomicAdd(&sm.M[s * LDM + s], TR::tof(qb[off + s * rs]) * ks_);
                        float prod = 1.f;
#pragma unroll 1
                        for (int t = s + 1; t < CH && t0 + t < T; ++t) {
                            prod *= TR::tof(fb[off + t * rs]);
                            atomicAdd(&sm.M[t * LDM + s], TR::tof(kb[off + t * rs]) * ks_ * prod);
                            atomicAdd(&sm.M[s * LDM + t], TR::tof(qb[off + t * rs]) * ks_ * prod);
                        }
                    }
                }
            }
            if (tid < CH) sm.beta[tid] = rbc;
            else if (tid < 2 * CH) sm.c[tid - CH] = rbc;
        }
        lds_barrier();

        KD_PHASE_MARK(n, 2);
        // ================= Gram tiles: M and P
        const bool fallback = sm.unsafe_any != 0u;
        if (I == 0 && r8 == 0 && unsafe) {
            // K-tilde of the fallback channels by suffix products (no division);
            // read only after two more barriers.
            const int t0 = n * CH;
#pragma unroll 1
            for (int c = 0; c < 8; ++c) {
                if (!((unsafe >> c) & 1u)) continue;
                const uint32_t off = (uint32_t)t0 * rs + hoff + ch0 + c;
                float suf = 1.f;
#pragma unroll 1
                for (int t = CH - 1; t >= 0; --t) {
                    if (t0 + t < T) {
                        sm.KtT[(ch0 + c) * LDT + t] = (typename TR::H)(TR::tof(kb[off + t * rs]) * ksc * suf);
                        suf *= TR::tof(fb[off + t * rs]);
                    }
                }
            }
        }
        // Reset the other parity's max |v|: its last reader (the previous chunk's
        // update) finished before the prep barriers, its next writer (the next
        // chunk's prep) comes after this chunk's closing barrier.
        if (tid == 0) sm.vmax_bits[(n + 1) & 1] = 0u;
        for (int tile = w; tile < 10; tile += NW) {
            // lower-triangular tile list (I_, J_), I_ >= J_
            const int I_ = tile < 1 ? 0 : tile < 3 ? 1 : tile < 6 ? 2 : 3;
            const int J_ = tile - (I_ * (I_ + 1)) / 2;
            floatx4 gk = {0.f, 0.f, 0.f, 0.f}, pp = gk, gv = gk;
            const E* aK = &sm.Kb[(SB * I_ + cl) * LD];
            const E* aQ = &sm.Qb[(SB * I_ + cl) * LD];
            const E* aV = &sm.V[(SB * I_ + cl) * LD];
            const E* bK = &sm.Kc[(SB * J_ + cl) * LD];
            const E* bV = &sm.V[(SB * J_ + cl) * LD];
#pragma unroll
            for (int ks = 0; ks < KD_; ++ks) {
                const Frag fk = TR::ld_nat(bK, ks, g);
                gk = TR::mma(TR::ld_nat(aK, ks, g), fk, gk);
                pp = TR::mma(TR::ld_nat(aQ, ks, g), fk, pp);
                gv = TR::mma(TR::ld_nat(aV, ks, g), TR::ld_nat(bV, ks, g), gv);
            }
            const int s_ = SB * J_ + cl;
            if (fallback) {
                float ck[4], cp[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t_ = SB * I_ + 4 * g + r;
                    ck[r] = (s_ < t_) ? sm.M[t_ * LDM + s_] : 0.f;
                    cp[r] = (s_ <= t_) ? sm.M[s_ * LDM + t_] : 0.f;
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    gk[r] += ck[r];
                    pp[r] += cp[r];
                    const int t_ = SB * I_ + 4 * g + r;
                    if (I_ != J_) sm.M[s_ * LDM + t_] = 0.f;   // mirror upper tile back to zero
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t_ = SB * I_ + 4 * g + r;
                sm.M[t_ * LDM + s_] = (s_ < t_) ? sm.beta[t_] * gk[r] * gv[r] : 0.f;
                sm.P[t_ * LDP + s_] = TR::cvt((s_ <= t_) ? pp[r] : 0.f);
            }
        }

        KD_PHASE_MARK(n, 3);
        // ================= state reads: Y = Kbar S0^T, O = Qbar S0^T
        floatx4 Y[NSB], Oa[NSB];
#pragma unroll
        for (int I_ = 0; I_ < NSB; ++I_) { Y[I_] = floatx4{0.f, 0.f, 0.f, 0.f}; Oa[I_] = Y[I_]; }
#pragma unroll
        for (int ks = 0; ks < KD_; ++ks) {
            const Frag bS = TR::state_frag(S, ks);
#pragma unroll
            for (int I_ = 0; I_ < NSB; ++I_) {
                Y[I_] = TR::mma(TR::ld_state(&sm.Kb[(SB * I_ + cl) * LD], ks, g), bS, Y[I_]);
                Oa[I_] = TR::mma(TR::ld_state(&sm.Qb[(SB * I_ + cl) * LD], ks, g), bS, Oa[I_]);
            }
        }
        // partial r0[t] = sum over this wave's 16 value columns of Y[t,i] v[t,i]
        {
            float x[16];
#pragma unroll
            for (int I_ = 0; I_ < NSB; ++I_)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    x[4 * I_ + r] = Y[I_][r] * TR::tof(sm.V[(SB * I_ + 4 * g + r) * LD + 16 * w + cl]);
            // butterfly reduce-scatter over the 16 lanes of a row group: lane cl
            // ends with the full sum of entry cl.
#pragma unroll
            for (int m = 8; m >= 1; m >>= 1) {
                const bool up = (cl & m) != 0;
#pragma unroll
                for (int e = 0; e < m; ++e) {
                    const float send = up ? x[e] : x[e + m];
                    const float keep = up ? x[e + m] : x[e];
                    x[e] = keep + __shfl_xor(send, m, 64);
                }
            }
            sm.r0p[w][SB * (cl >> 2) + 4 * g + (cl & 3)] = x[0];
        }
        lds_barrier();

        KD_PHASE_MARK(n, 4);
        // ================= forward substitution (I + M) u = c - beta r0
        // The next chunk's loads are issued where each wave is otherwise idle:
        // waves 1.. while wave 0 solves, wave 0 right after.  Issue stalls
        // while HBM drains the requests then cost no compute time.
        if (w != 0 && n + 1 < NC) load_chunk(n + 1);
        if (w == 0) {
            const int t_ = lane;
            float r0 = 0.f;
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) r0 += sm.r0p[ww][t_];
            float x = sm.c[t_] - sm.beta[t_] * r0;
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
            const float um = wave_max_nonneg(fabsf(x));
            if (lane == 0) {
                sm.umax_bits = __float_as_uint(um);
                // all reads of these flags for this chunk are done (prep b, Gram)
                sm.unsafe_any = 0u;
                sm.kmax_bits = 0u;
            }
            if (n + 1 < NC) load_chunk(n + 1);
        }
        lds_barrier();

        KD_PHASE_MARK(n, 5);
        // ================= O += P (u * V); state update
        {
            // Scales of the fp16 state-update operands (exact powers of two).
            const float usc = pow2_scale(__uint_as_float(sm.umax_bits) * __uint_as_float(sm.vmax_bits[n & 1]));
            const float inv = 1.f / (usc * ksc);
            Frag bW[KC_];
#pragma unroll
            for (int ks = 0; ks < KC_; ++ks) bW[ks] = TR::row_times(&sm.VT[(16 * w + cl) * LDT], sm.u, ks, g);
#pragma unroll
            for (int I_ = 0; I_ < NSB; ++I_)
#pragma unroll
                for (int ks = 0; ks < KC_; ++ks)
                    Oa[I_] = TR::mma(TR::ld_nat(&sm.P[(SB * I_ + cl) * LDP], ks, g), bW[ks], Oa[I_]);
            if (ob) {   // stage O in the (now free) Kc array
#pragma unroll
                for (int I_ = 0; I_ < NSB; ++I_)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        sm.Kc[(SB * I_ + 4 * g + r) * LD + 16 * w + cl] = TR::cvt(Oa[I_][r]);
            }
            typename TR::FragH hW[KC_];
#pragma unroll
            for (int ks = 0; ks < KC_; ++ks)
                hW[ks] = TR::row_times_h(&sm.VT[(16 * w + cl) * LDT], sm.u, usc, ks, g);
            // S <- (S diag(gamma_C) * s + K~'^T W') / s with s = usc * ksc
#pragma unroll
            for (int mt = 0; mt < D / 16; ++mt) {
                const floatx4 gm = *reinterpret_cast<const floatx4*>(&sm.gam[16 * mt + 4 * g]);
                S[mt] = S[mt] * (gm * (usc * ksc));
#pragma unroll
                for (int ks = 0; ks < KC_; ++ks)
                    S[mt] = TR::mma_h(TR::ld_nat_h(&sm.KtT[(16 * mt + cl) * LDT], ks, g), hW[ks], S[mt]);
                S[mt] = S[mt] * inv;
            }
        }
        lds_barrier();
        KD_PHASE_MARK(n, 6);
    }
    if (NC > 0 && ob) store_o(NC - 1);

    if (ST) {
#pragma unroll
        for (int mt = 0; mt < D / 16; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                ST[(size_t)bh * D * D + (size_t)(16 * w + cl) * D + 16 * mt + 4 * g + r] = S[mt][r];
    }
}

// --------------------------------------------------------------- launchers
template <class TR, int D>
static hipError_t launch_fwd_t(const void* q, const void* k, const void* v, const void* f,
                               const float* beta, const float* c, const float* S0, void* o,
                               float* ST, float* ckpt, int B, int T, int H, hipStream_t st)
{
    typedef typename TR::E E;
    hipLaunchKernelGGL((kd_fwd_kernel<TR, D>), dim3((unsigned)(B * H)), dim3(4 * D), 0, st,
                       (const E*)q, (const E*)k, (const E*)v, (const E*)f, beta, c, S0, (E*)o, ST,
                       ckpt, T, H);
    return hipGetLastError();
}

hipError_t launch_fwd(int bf16, int d, const void* q, const void* k, const void* v, const void* f,
                      const float* beta, const float* c, const float* S0, void* o, float* ST,
                      float* ckpt, int B, int T, int H, hipStream_t st)
{
    if (bf16) {
        switch (d) {
        case 32: return launch_fwd_t<Bf16T, 32>(q, k, v, f, beta, c, S0, o, ST, ckpt, B, T, H, st);
        case 64: return launch_fwd_t<Bf16T, 64>(q, k, v, f, beta, c, S0, o, ST, ckpt, B, T, H, st);
        case 128: return launch_fwd_t<Bf16T, 128>(q, k, v, f, beta, c, S0, o, ST, ckpt, B, T, H, st);
        }
    } else {
        switch (d) {
        case 32: return launch_fwd_t<F32T, 32>(q, k, v, f, beta, c, S0, o, ST, ckpt, B, T, H, st);
        case 64: return launch_fwd_t<F32T, 64>(q, k, v, f, beta, c, S0, o, ST, ckpt, B, T, H, st);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace kd
