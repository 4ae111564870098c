// kd_fwd16.hip -- chunkwise forward for bf16 inputs at d = 128, sixteen waves
// per (b, h).
//
// Same method, chunk algebra and software pipeline as the generic forward
// kernel (kd_fwd.hip; onedev.kr KronLSTM summary, sections "어떻게 동작하나"
// and "어떻게 쓰나"; aitrends.kr Gated DeltaNet-2 summary, section "방법론"
// steps 3-4): per chunk n,
//     (I + M) u = c - beta * r0,  r0_t = v_t^T S0 Kbar_t,
//     O = Qbar S0^T + P (u * V),  S_C = S0 diag(gamma_C) + (u * V)^T Ktilde.
// What changes is the split of the work: each role has eight waves, so every
// SIMD holds two consumer and two producer waves (128 registers each) and
// one wave's LDS, matrix-core or dependency wait is covered by the others.
//   consumers (waves 0..7): 16 value columns of the fp32 state each, held
//     transposed as MFMA accumulators (S^T[j][i], key index j as rows);
//     state reads, the forward substitution (wave 0), readout and update.
//   producers (waves 8..15): 8 rows of the chunk being prepared each, two
//     adjacent key channels per lane; decay products, operands, Gram tiles.
// Stage A: state reads of n | transposed operands of n, decay products of n+1.
// Stage B: substitution of n | operands of n+1, first prefetch of n+2.
// Stage C: readout and update of n | Gram tiles of n+1, rest of the prefetch.
#include <type_traits>

#include "kd_device.h"

// Phase markers: no-ops here; a profiling build may define them to record
// timestamps at the stage boundaries of the chunk loop.
#ifndef KD_PHASE_MARK
#define KD_PHASE_MARK(chunk, id) ((void)0)
#endif

namespace kd {

namespace f16w {
constexpr int D = 128;
constexpr int NT = 1024;
constexpr int NWC = 8;            // consumer waves
constexpr int NWP = 8;            // producer waves
constexpr int RB = CH / NWP;      // rows per producer wave
constexpr int LD = D + 16;        // row-major [CH][D] operands (columns in pcol order)
constexpr int LDT = CH + 8;       // transposed [D][CH] operands
constexpr int LDM = CH + 4;       // fp32 M
constexpr int LDP = CH + 8;       // P
constexpr int LDR = 4 * NWC + 4;  // r0 partials per token (row stride 36: conflict-free stores)
}  // namespace f16w

struct Fwd16Smem {
    alignas(16) __bf16 Qb[CH * f16w::LD];       // q * gamma
    alignas(16) __bf16 Kb[CH * f16w::LD];       // k * gamma
    alignas(16) __bf16 Kc[CH * f16w::LD];       // k / gamma (0 for fallback channels)
    alignas(16) __bf16 V[CH * f16w::LD];        // v
    alignas(16) __bf16 VT[f16w::D * f16w::LDT];     // v^T
    alignas(16) _Float16 KtT[f16w::D * f16w::LDT];  // (k gamma_C / gamma)^T * kscale
    alignas(16) float M[CH * f16w::LDM];        // beta_t tril_{-1}(G_K * G_V); fallback scratch
    alignas(16) __bf16 P[2][CH * f16w::LDP];    // tril_0 of the decayed Q K^T, by chunk parity
    alignas(16) float beta[2][CH];
    alignas(16) float c[2][CH];
    alignas(16) float u[CH];                   // u * s_prev (readout operand, see below)
    alignas(16) float us[CH];                  // u * usc (update operand)
    alignas(16) float gs[f16w::D];             // gamma_C * s / s_prev (state decay and rescale)
    alignas(16) float r0q[CH * f16w::LDR];     // r0 partials: [t][4 * wave + lane group]
    alignas(16) float bprod[f16w::NWP][f16w::D];   // product of f over each 8-row block
    alignas(16) float gam[2][f16w::D];             // gamma_C, by chunk parity
    unsigned kmax[3], vmax[3], unsafe[3];   // per chunk mod 3: max |k|, max |v| (bits), fallback flag
    float oinv, sinv;                       // 1 / s_prev and 1 / s of the current chunk
};

// CKPT: also store, per chunk, the records of FwdCkpt: the entering state
// (bf16), u and r0, and the chunk's M and P.  GATES: f, beta and c hold the
// gates' logits, turned into the gates by the producers as they load them
// (FwdGates).
template <bool CKPT, bool GATES>
__global__ __launch_bounds__(f16w::NT) void kd_fwd16_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ f, const float* __restrict__ beta, const float* __restrict__ cc,
    const float* __restrict__ S0, __bf16* __restrict__ o, float* __restrict__ ST,
    FwdCkpt ck, FwdGates gt, const int* __restrict__ cu, int T_, int H)
{
    using namespace f16w;
    typedef Bf16T TR;
    typedef __bf16 E;
    typedef TR::Frag Frag;
    typedef TR::FragH FragH;
    constexpr int KD_ = D / TR::KS;    // K-steps over d
    constexpr int KC_ = CH / TR::KS;   // K-steps over a chunk

    __shared__ Fwd16Smem sm;

    const int tid = threadIdx.x;
    const int lane = tid & 63, g = lane >> 4, cl = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool consumer = w < NWC;
    const int bh = blockIdx.x, b = bh / H, h = bh % H;
    // per batch element, [T, H, D] tensors are addressed from a wave-uniform
    // base with 32-bit element offsets (the host checks T*H*D fits)
    const uint32_t rs = (uint32_t)H * D;
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

    if (NC == 0) {   // empty sequence: S_T = S0
        if (ST)
            for (int x = tid; x < D * D; x += NT)
                ST[(size_t)bh * D * D + x] = S0 ? S0[(size_t)bh * D * D + x] : 0.f;
        return;
    }

    // one-time init: the upper triangles of M and P are never written
    for (int x = tid; x < 2 * CH * LDP; x += NT) (&sm.P[0][0])[x] = TR::cvt(0.f);
    for (int x = tid; x < CH * LDM; x += NT) sm.M[x] = 0.f;
    if (tid == 0) {
        for (int s = 0; s < 3; ++s) { sm.kmax[s] = 0u; sm.vmax[s] = 0u; sm.unsafe[s] = 0u; }
        sm.oinv = 1.f;
        sm.sinv = 1.f;
    }
    lds_barrier();

    // Both teams run the same sequence of barriers (three per chunk, two more
    // in a stage C whose next chunk takes the exact fallback).
    if (consumer) {
        // The state is kept multiplied by the exact power of two s = usc * ksc
        // of the last update (the fp16 operand scales below), so that the
        // update needs one multiply per element: S <- S diag(gamma_C) s / s_prev
        // + K~'^T W'.  Reads of the state come out scaled by s_prev and are
        // rescaled once: r0 on the substitution wave, o at the store, S_T at the
        // end.  Powers of two commute with rounding, so the results are those
        // of the unscaled state.
        const int i0 = 16 * w;   // value columns i0 .. i0 + 15
        int e_prev = 0;          // s_prev = 2^-e_prev (substitution wave)
        const uint32_t o_lane = (uint32_t)cl * rs + hoff + i0 + 4 * g;
        floatx4 S[D / 16];       // S^T[16mj + 4g + r][i0 + cl] in S[mj][r]
#pragma unroll
        for (int mj = 0; mj < D / 16; ++mj)   // four adjacent columns: one 16-byte load
            S[mj] = S0 ? *reinterpret_cast<const floatx4*>(&S0[(size_t)bh * D * D + (size_t)(i0 + cl) * D + 16 * mj + 4 * g])
                       : floatx4{0.f, 0.f, 0.f, 0.f};

        for (int n = -1; n < NC; ++n) {
            const int nn = n + 1;
            // ======================================================= stage A
            KD_PHASE_MARK(n, 0);
            floatx4 Ot[NSB];   // O^T[i0 + 4g + r][16tt + cl], lives to stage C
            if (n >= 0) {
                if (CKPT) {
                    E* dst = static_cast<E*>(ck.S) + ((size_t)bh * NC + n) * D * D;
                    const float si = sm.sinv;
#pragma unroll
                    for (int mj = 0; mj < D / 16; ++mj)
                        st4_nt(dst + ((uint32_t)(i0 + cl) * D + 16 * mj + 4 * g), S[mj] * si);
                }
                // Y^T = S Kbar^T, then O^T = S Qbar^T (M = value index, N = token).
                // The B fragments of the next K-step are loaded before the MFMAs
                // of this one.
                auto state_pass = [&](const E* op, floatx4* acc) {
                    Frag bc[NSB];
#pragma unroll
                    for (int tt = 0; tt < NSB; ++tt) bc[tt] = TR::ld_state_p(&op[(SB * tt + cl) * LD], 0, g);
#pragma unroll
                    for (int ks = 0; ks < KD_; ++ks) {
                        Frag bn[NSB];
                        if (ks + 1 < KD_) {
#pragma unroll
                            for (int tt = 0; tt < NSB; ++tt) bn[tt] = TR::ld_state_p(&op[(SB * tt + cl) * LD], ks + 1, g);
                        }
                        const Frag a = TR::state_frag(S, ks);
                        const floatx4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int tt = 0; tt < NSB; ++tt) acc[tt] = TR::mma(a, bc[tt], ks ? acc[tt] : z);
                        if (ks + 1 < KD_) {
#pragma unroll
                            for (int tt = 0; tt < NSB; ++tt) bc[tt] = bn[tt];
                        }
                    }
                };
                {
                    floatx4 Yt[NSB];
                    state_pass(sm.Kb, Yt);
                    // partial r0[t] over value columns i0 + 4g .. i0 + 4g + 3 (adjacent
                    // under pcol); the substitution wave adds the 32 partials of t
#pragma unroll
                    for (int tt = 0; tt < NSB; ++tt) {
                        const bf16x4 vr = *reinterpret_cast<const bf16x4*>(
                            &sm.V[(SB * tt + cl) * LD + TR::pcol(i0 + 4 * g)]);
                        float x = 0.f;
#pragma unroll
                        for (int r = 0; r < 4; ++r) x += Yt[tt][r] * TR::tof(vr[r]);
                        sm.r0q[(SB * tt + cl) * LDR + 4 * w + g] = x;
                    }
                }
                state_pass(sm.Qb, Ot);
            }
            KD_PHASE_MARK(n, 3);
            lds_barrier();
            // ======================================================= stage B
            KD_PHASE_MARK(n, 1);
            if (n >= 0 && w == 0) {   // forward substitution (I + M) u = c - beta r0
                const int t_ = lane;
                __builtin_amdgcn_s_setprio(3);   // the chain every other wave waits for
                float r0;
                {
                    const floatx4* pr = reinterpret_cast<const floatx4*>(&sm.r0q[t_ * LDR]);
                    floatx4 a = pr[0] + pr[4], b = pr[1] + pr[5];
                    a += pr[2] + pr[6];
                    b += pr[3] + pr[7];
                    a += b;
                    r0 = ((a[0] + a[1]) + (a[2] + a[3])) * ldexpf(1.f, e_prev);
                }
                float x = sm.c[n & 1][t_] - sm.beta[n & 1][t_] * r0;
                // M is strictly lower triangular (zeros elsewhere): lane t only
                // changes while s < t, no mask needed
#pragma unroll
                for (int sb = 0; sb < CH / 16; ++sb) {
                    float Mrow[16];
#pragma unroll
                    for (int s4 = 0; s4 < 4; ++s4) {
                        const floatx4 m4 = *reinterpret_cast<const floatx4*>(&sm.M[t_ * LDM + 16 * sb + 4 * s4]);
                        Mrow[4 * s4] = m4[0]; Mrow[4 * s4 + 1] = m4[1];
                        Mrow[4 * s4 + 2] = m4[2]; Mrow[4 * s4 + 3] = m4[3];
                    }
#pragma unroll
                    for (int s = 0; s < 16; ++s)
                        if (16 * sb + s < CH - 1) x = fmaf(-Mrow[s], readlane_f(x, 16 * sb + s), x);
                }
                if (CKPT) {
                    float* du = ck.U + ((size_t)bh * NC + n) * 2 * CH;
                    st_nt(&du[t_], x);
                    st_nt(&du[CH + t_], r0);
                }
                // scales of this chunk's update: usc = 2^-eu, ksc = 2^-ek, s = 2^-e
                const float um = wave_max_nonneg(fabsf(x));
                const int eu = pow2_exp(um * __uint_as_float(sm.vmax[n % 3]));
                const int e = eu + pow2_exp(__uint_as_float(sm.kmax[n % 3]));
                sm.u[t_] = x * ldexpf(1.f, -e_prev);
                sm.us[t_] = x * ldexpf(1.f, -eu);
                const float rs_ = ldexpf(1.f, e_prev - e);
                const float2 gm = *reinterpret_cast<const float2*>(&sm.gam[n & 1][2 * t_]);
                *reinterpret_cast<float2*>(&sm.gs[2 * t_]) = make_float2(gm.x * rs_, gm.y * rs_);
                if (lane == 0) {
                    sm.oinv = ldexpf(1.f, e_prev);
                    sm.sinv = ldexpf(1.f, e);
                }
                e_prev = e;
                __builtin_amdgcn_s_setprio(0);
            }
            if (CKPT && n >= 0 && w >= 1) {
                // M and P of chunk n are complete (their last tiles ran in stage
                // A) and nobody writes them in this stage: the idle consumer waves
                // copy them out
                float* dm = ck.M + ((size_t)bh * NC + n) * CH * CH;
                E* dp = static_cast<E*>(ck.P) + ((size_t)bh * NC + n) * CH * CH;
                for (int x = tid - 64; x < CH * CH / 4; x += (NWC - 1) * 64) {
                    const int t = x >> 4, s4 = x & 15;
                    cp16_nt(dm + t * CH + 4 * s4, &sm.M[t * LDM + 4 * s4]);
                }
                for (int x = tid - 64; x < CH * CH / 8; x += (NWC - 1) * 64) {
                    const int t = x >> 3, s8 = x & 7;
                    cp16_nt(dp + t * CH + 8 * s8, &sm.P[n & 1][t * LDP + 8 * s8]);
                }
            }
            if (tid == 0 && n >= 0) {
                // slot (n+2)%3 = chunks n-1 and n+2: the former's last reader ran in
                // the previous stage C, the latter's first writer runs in stage A(n+1)
                sm.kmax[(n + 2) % 3] = 0u; sm.vmax[(n + 2) % 3] = 0u; sm.unsafe[(n + 2) % 3] = 0u;
            }
            KD_PHASE_MARK(n, 4);
            lds_barrier();
            // ======================================================= stage C
            KD_PHASE_MARK(n, 2);
            if (nn < NC && sm.unsafe[nn % 3] != 0u) {   // producers run the exact fallback
                lds_barrier();
                lds_barrier();
            }
            if (n >= 0) {
                // W = u * V of this wave's value columns: bf16 scaled by s_prev for
                // the readout, fp16 scaled by usc for the update
                Frag wa[KC_];
                FragH wb[KC_];
#pragma unroll
                for (int ks = 0; ks < KC_; ++ks) TR::row_times_pair(&sm.VT[(i0 + cl) * LDT], sm.u, sm.us, ks, g, wa[ks], wb[ks]);
                // O^T += W^T P^T (the P fragments of a K-step loaded together)
#pragma unroll
                for (int ks = 0; ks < KC_; ++ks) {
                    Frag pf[NSB];
#pragma unroll
                    for (int tt = 0; tt < NSB; ++tt) pf[tt] = TR::ld_nat(&sm.P[n & 1][(SB * tt + cl) * LDP], ks, g);
#pragma unroll
                    for (int tt = 0; tt < NSB; ++tt) Ot[tt] = TR::mma(wa[ks], pf[tt], Ot[tt]);
                }
                if (ob) {
                    const float oi = sm.oinv;
#pragma unroll
                    for (int tt = 0; tt < NSB; ++tt) {
                        // row offset = scalar part + this lane's part (one register
                        // across the loop instead of one per tt)
                        const uint32_t srow = __builtin_amdgcn_readfirstlane((uint32_t)(n * CH + SB * tt) * rs);
                        if (n * CH + SB * tt + cl < T) st4_nt(ob + (srow + o_lane), Ot[tt] * oi);
                    }
                }
                // S <- S diag(gamma_C) s / s_prev + K~'^T W'; K-steps outermost, so
                // consecutive MFMAs go to different accumulators
#pragma unroll
                for (int mj = 0; mj < D / 16; ++mj)
                    S[mj] = S[mj] * *reinterpret_cast<const floatx4*>(&sm.gs[16 * mj + 4 * g]);
#pragma unroll
                for (int ks = 0; ks < KC_; ++ks) {
                    FragH ak[D / 16];
#pragma unroll
                    for (int mj = 0; mj < D / 16; ++mj) ak[mj] = TR::ld_nat_h(&sm.KtT[(16 * mj + cl) * LDT], ks, g);
#pragma unroll
                    for (int mj = 0; mj < D / 16; ++mj) S[mj] = TR::mma_h(ak[mj], wb[ks], S[mj]);
                }
            }
            KD_PHASE_MARK(n, 5);
            lds_barrier();
        }
        if (ST) {
            const float si = sm.sinv;
#pragma unroll
            for (int mj = 0; mj < D / 16; ++mj)   // four adjacent columns: one 16-byte store
                st4_nt(&ST[(size_t)bh * D * D + (size_t)(i0 + cl) * D + 16 * mj + 4 * g], S[mj] * si);
        }
    } else {
        const int pw = w - NWC;          // producer wave 0..7 (wave-uniform)
        const int rb = RB * pw;          // rows rb .. rb + 7 of the chunk
        const int ch0 = 2 * lane;        // channels ch0, ch0 + 1
        const int pc0 = TR::pcol(ch0);   // adjacent under pcol
        Raw8x2 rq, rk, rv, rf;           // raw rows of the chunk being prepared
        float rb_beta = 0.f, rb_c = 0.f; // beta_t, c_t for t = lane (used by wave 0)
        float tot[2];                    // product of f over the 8 rows, per channel
        Col8 keep_v[2], keep_kt[2];      // v and K-tilde of the prepared chunk, written
                                         //   transposed in the following stage A
        unsigned pmask = 0;              // fallback channels (bit cc: ch0 + cc)
        const float gex = GATES ? __expf(gt.a_log[h]) : 0.f;   // forget-gate exponent
        // Rows past the sequence end re-read the last row (in bounds) and are
        // cleared before use.  Loads are unconditional (clamped to the last
        // chunk) so the prefetch registers never merge with older values.
        auto row_off = [&](int n, int& last) {
            const int t0 = min(n * CH + rb, T - 1);
            last = min(RB - 1, T - 1 - t0);
            return (uint32_t)t0 * rs + hoff + ch0;
        };
        auto load_q = [&](int n) {
            int last;
            const uint32_t off = row_off(n, last);
            rq.load(qb, off, rs, last);
            const int t = min(n * CH + lane, T - 1);
            const uint32_t gi = (uint32_t)t * H + h;
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
        // One lower-triangular 16 x 16 tile (I_ >= J_) of M (DO_M) and / or P
        // (DO_P) for chunk ch.  The M part writes only the strictly lower
        // entries of M; after the exact fallback, whose P terms sit on and
        // above the diagonal of M, the P part reads and clears them.  The two
        // parts never touch the same entry.
        auto gram_tile = [&](auto do_m, auto do_p, int tile, int ch, bool fbk) {
            constexpr bool DO_M = decltype(do_m)::value, DO_P = decltype(do_p)::value;
            const int I_ = tile < 1 ? 0 : tile < 3 ? 1 : tile < 6 ? 2 : 3;
            const int J_ = tile - (I_ * (I_ + 1)) / 2;
            floatx4 gk, pp, gv;
            const E* aK = &sm.Kb[(SB * I_ + cl) * LD];
            const E* aQ = &sm.Qb[(SB * I_ + cl) * LD];
            const E* aV = &sm.V[(SB * I_ + cl) * LD];
            const E* bK = &sm.Kc[(SB * J_ + cl) * LD];
            const E* bV = &sm.V[(SB * J_ + cl) * LD];
            // operands of one K-step; those of the next are loaded before the
            // MFMAs of the current one
            struct GF { Frag k, a, q, v, w; };
            auto ldg = [&](int ks) {
                GF r;
                r.k = TR::ld_nat(bK, ks, g);
                if (DO_M) { r.a = TR::ld_nat(aK, ks, g); r.v = TR::ld_nat(aV, ks, g); r.w = TR::ld_nat(bV, ks, g); }
                if (DO_P) r.q = TR::ld_nat(aQ, ks, g);
                return r;
            };
            GF cur = ldg(0);
#pragma unroll
            for (int ks = 0; ks < KD_; ++ks) {
                const floatx4 z = {0.f, 0.f, 0.f, 0.f};
                GF nxt;
                if (ks + 1 < KD_) nxt = ldg(ks + 1);
                if (DO_M) gk = TR::mma(cur.a, cur.k, ks ? gk : z);
                if (DO_P) pp = TR::mma(cur.q, cur.k, ks ? pp : z);
                if (DO_M) gv = TR::mma(cur.v, cur.w, ks ? gv : z);
                if (ks + 1 < KD_) cur = nxt;
            }
            const int s_ = SB * J_ + cl;
            if (fbk) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t_ = SB * I_ + 4 * g + r;
                    if (DO_M && s_ < t_) gk[r] += sm.M[t_ * LDM + s_];
                    if (DO_P && s_ <= t_) {
                        pp[r] += sm.M[s_ * LDM + t_];
                        sm.M[s_ * LDM + t_] = 0.f;
                    }
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t_ = SB * I_ + 4 * g + r;
                if (DO_M && s_ < t_) sm.M[t_ * LDM + s_] = sm.beta[ch & 1][t_] * gk[r] * gv[r];
                if (DO_P) sm.P[ch & 1][t_ * LDP + s_] = TR::cvt((s_ <= t_) ? pp[r] : 0.f);
            }
        };
        typedef std::integral_constant<bool, true> kYes;
        typedef std::integral_constant<bool, false> kNo;

        for (int n = -1; n < NC; ++n) {
            const int nn = n + 1;             // chunk the producers prepare
            const bool prod_on = nn < NC;
            // ======================================================= stage A
            KD_PHASE_MARK(n, 0);
            if (n >= 0) {   // transposed operands of chunk n and its last two Gram tiles
#pragma unroll
                for (int c2 = 0; c2 < 2; ++c2) {
                    keep_v[c2].store(&sm.VT[(ch0 + c2) * LDT + rb]);
                    keep_kt[c2].store(&sm.KtT[(ch0 + c2) * LDT + rb]);
                }
                // tiles 8 and 9 (rows 48..63) are first read by the substitution
                // (M) and the readout (P) of chunk n: their M and P parts run
                // here on producer waves 0..3, one SIMD each
                if (pw < 4) {
                    const bool fbk = sm.unsafe[n % 3] != 0u;
                    if (pw >= 2) gram_tile(kNo(), kYes(), 8 + (pw & 1), n, fbk);
                    else gram_tile(kYes(), kNo(), 8 + (pw & 1), n, fbk);
                }
            }
            if (prod_on) {   // decay products of chunk nn
                if (GATES) {   // the gates of chunk nn from their logits
                    rf.map([&](float x) { return forget_gate(x, gex); });
                    rb_beta = gt.beta_scale * gate_sigmoid(rb_beta);
                    rb_c = gate_sigmoid(rb_c);
                }
                if (nn * CH + CH > T) {   // ragged last chunk: clear rows past the end
#pragma unroll
                    for (int e = 0; e < RB; ++e)
                        if (nn * CH + rb + e >= T) {
                            rq.clear(e, 0.f); rk.clear(e, 0.f); rv.clear(e, 0.f); rf.clear(e, 1.f);
                        }
                    if (nn * CH + lane >= T) { rb_beta = 0.f; rb_c = 0.f; }
                }
#pragma unroll
                for (int c2 = 0; c2 < 2; ++c2) {   // pairwise tree over the 8 rows
                    const float x0 = rf.get(0, c2) * rf.get(1, c2), x1 = rf.get(2, c2) * rf.get(3, c2);
                    const float x2 = rf.get(4, c2) * rf.get(5, c2), x3 = rf.get(6, c2) * rf.get(7, c2);
                    tot[c2] = (x0 * x1) * (x2 * x3);
                }
                st2(&sm.bprod[pw][ch0], tot[0], tot[1]);
                const float km = wave_max_nonneg(rk.absmax());
                const float vm = wave_max_nonneg(rv.absmax());
                if (lane == 0) {   // non-negative floats order like their bit patterns
                    atomicMax(&sm.kmax[nn % 3], __float_as_uint(km));
                    atomicMax(&sm.vmax[nn % 3], __float_as_uint(vm));
                }
                if (pw == 0) {
                    sm.beta[nn & 1][lane] = rb_beta;
                    sm.c[nn & 1][lane] = rb_c;
                }
            }
            KD_PHASE_MARK(n, 3);
            lds_barrier();
            // ======================================================= stage B
            KD_PHASE_MARK(n, 1);
            if (prod_on) {   // operands of chunk nn into LDS
                // gamma before this block (plt), after it (pgt), and over the chunk
                // (gC, multiplied in one fixed order so every wave agrees on it).
                // pw is wave-uniform: one straight-line case per value.
                float plt[2] = {1.f, 1.f}, pgt[2] = {1.f, 1.f}, gC[2] = {1.f, 1.f}, rgC[2];
                {
                    float2 xb[NWP];
#pragma unroll
                    for (int p = 0; p < NWP; ++p) xb[p] = *reinterpret_cast<const float2*>(&sm.bprod[p][ch0]);
                    auto prods = [&](auto pw_c) {
                        constexpr int PW = decltype(pw_c)::value;
#pragma unroll
                        for (int p = 0; p < NWP; ++p) {
                            gC[0] *= xb[p].x; gC[1] *= xb[p].y;
                            if (p < PW) { plt[0] *= xb[p].x; plt[1] *= xb[p].y; }
                            if (p > PW) { pgt[0] *= xb[p].x; pgt[1] *= xb[p].y; }
                        }
                    };
                    switch (pw) {
                    case 0: prods(std::integral_constant<int, 0>()); break;
                    case 1: prods(std::integral_constant<int, 1>()); break;
                    case 2: prods(std::integral_constant<int, 2>()); break;
                    case 3: prods(std::integral_constant<int, 3>()); break;
                    case 4: prods(std::integral_constant<int, 4>()); break;
                    case 5: prods(std::integral_constant<int, 5>()); break;
                    case 6: prods(std::integral_constant<int, 6>()); break;
                    default: prods(std::integral_constant<int, 7>()); break;
                    }
                }
                pmask = 0;
#pragma unroll
                for (int c2 = 0; c2 < 2; ++c2) {
                    // fallback channels get a zero Kc column (their Gram terms are
                    // added exactly in stage C)
                    const bool un = !(gC[c2] >= kSafeFloor);
                    if (un) pmask |= 1u << c2;
                    rgC[c2] = un ? 0.f : __builtin_amdgcn_rcpf(gC[c2]);
                }
                if (pw == 0) st2(&sm.gam[nn & 1][ch0], gC[0], gC[1]);
                if (pmask) atomicOr(&sm.unsafe[nn % 3], 1u);
                // K-tilde is kept scaled by ksc (a power of 2) for the fp16 update;
                // Kc = K-tilde / gamma_C takes 1 / ksc back through rgC
                const int ek = pow2_exp(__uint_as_float(sm.kmax[nn % 3]));
                const float ksc = ldexpf(1.f, -ek), iksc = ldexpf(1.f, ek);
                // ksc * gamma_C / gamma at each row: suffix products within the block
                float om[RB][2];
#pragma unroll
                for (int c2 = 0; c2 < 2; ++c2) {
                    rgC[c2] *= iksc;
                    om[RB - 1][c2] = pgt[c2] * ksc;
#pragma unroll
                    for (int e = RB - 2; e >= 0; --e) om[e][c2] = om[e + 1][c2] * rf.get(e + 1, c2);
                }
                float ga[2] = {plt[0], plt[1]};   // gamma at the current row
                float kprev[2] = {0.f, 0.f};
#pragma unroll
                for (int e = 0; e < RB; ++e) {
                    float qo[2], ko[2], co[2];
#pragma unroll
                    for (int c2 = 0; c2 < 2; ++c2) {
                        ga[c2] *= rf.get(e, c2);
                        const float kf = rk.get(e, c2), qf = rq.get(e, c2);
                        const float kt = kf * om[e][c2];   // K-tilde * ksc
                        qo[c2] = qf * ga[c2];
                        ko[c2] = kf * ga[c2];
                        co[c2] = kt * rgC[c2];             // k / gamma = K-tilde / gamma_C
                        if (e & 1) keep_kt[c2].set_pair_h(e >> 1, kprev[c2], kt);
                        else kprev[c2] = kt;
                    }
                    st2(&sm.Qb[(rb + e) * LD + pc0], qo[0], qo[1]);
                    st2(&sm.Kb[(rb + e) * LD + pc0], ko[0], ko[1]);
                    st2(&sm.Kc[(rb + e) * LD + pc0], co[0], co[1]);
                    rv.store(&sm.V[(rb + e) * LD + pc0], e);
                }
#pragma unroll
                for (int c2 = 0; c2 < 2; ++c2) keep_v[c2].set_raw(rv, c2);
            }
            const int npf = min(nn + 1, NC - 1);   // prefetch of chunk nn + 1
            load_q(npf);
            KD_PHASE_MARK(n, 4);
            lds_barrier();
            // ======================================================= stage C
            KD_PHASE_MARK(n, 2);
            const bool fallback = prod_on && sm.unsafe[nn % 3] != 0u;
            if (fallback) {
                // Exact Gram terms of the key channels of chunk nn whose decay is
                // below the floor: G_K[t,s] (s<t) accumulates at M[t][s], P[t,s]
                // (s<t) at M[s][t], P[t,t] at M[t][t].  Rare path: rows are
                // re-read from global memory.
                for (int x = tid - NWC * 64; x < CH * LDM / 4; x += NWP * 64)
                    reinterpret_cast<floatx4*>(sm.M)[x] = floatx4{0.f, 0.f, 0.f, 0.f};
                lds_barrier();
                if (pw == 0 && pmask) {
                    const int t0 = nn * CH;
#pragma unroll 1
                    for (int c = 0; c < 2; ++c) {
                        if (!((pmask >> c) & 1u)) continue;
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
                lds_barrier();
            }
            load_k(npf);
            if (prod_on) gram_tile(kYes(), kYes(), pw, nn, fallback);   // tiles 0..7
            load_v(npf);
            load_f(npf);
            KD_PHASE_MARK(n, 5);
            lds_barrier();
        }
    }
}

hipError_t launch_fwd16(const void* q, const void* k, const void* v, const void* f, const float* beta,
                        const float* c, const float* S0, void* o, float* ST, const FwdCkpt* ck,
                        const int* cu, int B, int T, int H, hipStream_t st)
{
    typedef __bf16 E;
    if (ck)
        hipLaunchKernelGGL((kd_fwd16_kernel<true, false>), dim3((unsigned)(B * H)), dim3(f16w::NT), 0, st,
                           (const E*)q, (const E*)k, (const E*)v, (const E*)f, beta, c, S0, (E*)o, ST,
                           *ck, FwdGates{}, (const int*)nullptr, T, H);
    else
        hipLaunchKernelGGL((kd_fwd16_kernel<false, false>), dim3((unsigned)(B * H)), dim3(f16w::NT), 0, st,
                           (const E*)q, (const E*)k, (const E*)v, (const E*)f, beta, c, S0, (E*)o, ST,
                           FwdCkpt{}, FwdGates{}, cu, T, H);
    return hipGetLastError();
}

// The forward with the gates made from their logits (f_raw [B,T,H,D] bf16,
// beta_raw and c_raw [B,T,H] fp32) as the producers load them.
hipError_t launch_fwd16_gates(const void* q, const void* k, const void* v, const void* f_raw,
                              const float* beta_raw, const float* c_raw, const float* a_log, float beta_scale,
                              const float* S0, void* o, float* ST, int B, int T, int H, hipStream_t st)
{
    typedef __bf16 E;
    FwdGates gt;
    gt.a_log = a_log;
    gt.beta_scale = beta_scale;
    hipLaunchKernelGGL((kd_fwd16_kernel<false, true>), dim3((unsigned)(B * H)), dim3(f16w::NT), 0, st,
                       (const E*)q, (const E*)k, (const E*)v, (const E*)f_raw, beta_raw, c_raw, S0, (E*)o, ST,
                       FwdCkpt{}, gt, (const int*)nullptr, T, H);
    return hipGetLastError();
}

}  // namespace kd
