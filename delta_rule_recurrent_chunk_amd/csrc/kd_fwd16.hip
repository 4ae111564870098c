// kd_fwd16.hip -- chunkwise forward for bf16 inputs at d = 128, sixteen waves
// per (b, h).
//
// Same method, chunk algebra and software pipeline as the generic forward
// kernel (kd_fwd.hip; onedev.kr KronLSTM summary, sections "어떻게 동작하나"
// and "어떻게 쓰나"; aitrends.kr Gated DeltaNet-2 summary, section "방법론"
// steps 3-4): per chunk n,
//     (I + M) u = c - beta * r0,  r0_t = v_t^T S0 Kbar_t,
//     O = Qbar S0^T + P (u * V),  S_C = S0 diag(gamma_C) + (u * V)^T Ktilde.
// Decay references: two, chosen per chunk by a vote of the producers (every
// producer wave holds every key channel, so all reach the same vote).
//   Chunk start, when every channel's decay over the chunk is at least 2^-100:
//     Qb = q gamma, Kb = k gamma, Kc = k / gamma (= k b after / gamma_C),
//     gamma from the chunk start; the Gram tiles need no factors and the
//     consumers read the state as it entered the chunk.
//   16-token sub-blocks otherwise, so that every stored operand is a product
//   of gates (at most 1, never a quotient):
//     a_t = prod of f from the start of t's sub-block through t,
//     b_s = prod of f after s through the end of s's sub-block,
//     Qloc = q a, Kloc = k a, Kr = k b   (LDS arrays Qb, Kb, Kc),
//     G_K[t,s] = sum_j Kloc_tj Kr_sj D_IJ,j   (t in sub-block I, s in J < I),
//   where D_IJ is the decay of the whole sub-blocks between J and I (1 for
//   neighbours).  A diagonal tile (I = J) divides by its sub-block's decay
//   (Kr / prod over the sub-block); a channel whose sub-block decay is below
//   2^-100 is left out of that tile's matrix product and its terms are added
//   exactly on the vector units.  The state reads go sub-block by sub-block,
//   decaying the state in place by each sub-block's decay after its reads, so
//   that sub-block I reads (S diag(gamma before I)) Kloc^T = S Kbar^T; after
//   the last one the update needs only the last sub-block's decay.
// The split of the work: each role has eight waves, so every
// SIMD holds two consumer and two producer waves (128 registers each) and
// one wave's LDS, matrix-core or dependency wait is covered by the others.
//   consumers (waves 0..7): 16 value columns of the fp32 state each, held
//     transposed as MFMA accumulators (S^T[j][i], key index j as rows);
//     state reads, the forward substitution (wave 0), readout and update;
//     o leaves through an LDS staging tile as whole rows (written out by
//     waves 1..7 during the next substitution).
//   producers (waves 8..15): 8 rows of the chunk being prepared each, two
//     adjacent key channels per lane; decay products, operands, Gram tiles.
// Stage A: state reads of n, o of n-1 staged | K-tilde^T of n, tiles 8-9 of
//          n, decay products of n+1.
// Stage B: substitution of n, o rows of n-1 out | operands of n+1, first
//          prefetch of n+2.
// Stage C: readout and update of n | Gram tiles 0-7 of n+1, rest of the
//          prefetch.
#include <atomic>
#include <ctime>
#include <type_traits>

#include "kd_device.h"
#include "kd_handoff.h"
#include "kd_mixer_conv.h"

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
constexpr int LDO = D + 8;        // o staging rows
constexpr int LDM = CH + 4;       // fp32 M
constexpr int LDP = CH + 8;       // P
}  // namespace f16w

// Rows of the factor table Fwd16Smem::fac (key channels in pcol order).
// Rows DIAG .. D30 are the Gram tiles' (pcol order); rows SUB + I are the
// decay over sub-block I in natural channel order (the state's decay).
// parts of a Gram tile (gram_tile)
constexpr int GT_MP = 0, GT_P = 1, GT_GK = 2, GT_GV = 3;

namespace facrow {
constexpr int DIAG = 0;    // DIAG + I: 1 / (decay over sub-block I), 0 for a channel below the floor
constexpr int D20 = 4;     // decay over sub-block 1 (tile I=2, J=0)
constexpr int D31 = 5;     // decay over sub-block 2 (tile I=3, J=1)
constexpr int D30 = 6;     // decay over sub-blocks 1 and 2 (tile I=3, J=0)
constexpr int SUB = 7;     // SUB + I (I = 0..2): decay over sub-block I, natural order
constexpr int N = 10;
}  // namespace facrow

struct Fwd16Smem {
    alignas(16) __bf16 Qb[CH * f16w::LD];       // q * a (decay from the sub-block start)
    alignas(16) __bf16 Kb[CH * f16w::LD];       // k * a
    alignas(16) __bf16 Kc[CH * f16w::LD];       // k * b (decay to the sub-block end)
    alignas(16) __bf16 V[CH * f16w::LD];        // v
    alignas(16) __bf16 Os[CH * f16w::LDO];      // o of the chunk, natural columns (staging)
    alignas(16) _Float16 KtT[f16w::D * f16w::LDT];  // (k gamma_C / gamma)^T * kscale
    alignas(16) float M[CH * f16w::LDM];        // beta_t tril_{-1}(G_K * G_V); rows 48..63 of tiles
                                                 //   (3,2), (3,3): beta_t G_K only (times G3 when read)
    alignas(16) float G3[2][SB * SB];           // G_V of tiles (3,2), (3,3), [tile][t][s]
    alignas(16) __bf16 P[2][CH * f16w::LDP];    // tril_0 of the decayed Q K^T, by chunk parity
    alignas(16) float beta[2][CH];
    alignas(16) float c[2][CH];
    alignas(16) float u[CH];                   // u * s_prev (readout operand, see below)
    alignas(16) float us[CH];                  // u * usc (update operand)
    alignas(16) float gs[f16w::D];             // gamma_C * s / s_prev (state decay and rescale)
    alignas(16) float r0p[CH * f16w::NWC];     // r0 partials: [t][consumer wave, rotated by t / 4]
    alignas(16) float bprod[f16w::NWP][f16w::D];   // product of f over each 8-row block
    alignas(16) float gam[2][f16w::D];             // decay over the last sub-block, by chunk parity
    alignas(16) float fac[facrow::N][f16w::D];     // decay factors of the prepared chunk (facrow)
    unsigned kmax[3], vmax[3];              // per chunk mod 3: max |k|, max |v| (bits)
    unsigned fbm[2][NSB][f16w::D / 32];     // channels below the floor per sub-block, by chunk parity
    unsigned fbany[2];                      // any such channel in the chunk, by chunk parity
    unsigned slow[2];                       // chunk-start references (see below), by chunk parity
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
    FwdCkpt ck, FwdGates gt, ConvFeed cf, const int* __restrict__ cu, int T_, int H)
{
    using namespace f16w;
    typedef Bf16T TR;
    typedef __bf16 E;
    typedef TR::Frag Frag;
    typedef TR::FragH FragH;
    constexpr int KD_ = D / TR::KS;    // K-steps over d
    constexpr int KC_ = CH / TR::KS;   // K-steps over a chunk

    __shared__ Fwd16Smem sm;

    // GATES with a convolution feed: blocks BHpad and up convolve q, k, v for
    // the forward blocks 0 .. BH - 1 (conv_feed_worker), which publish their XCD
    const bool feed = GATES && cf.nwork > 0;
    if constexpr (GATES) {
        if (feed) {
            if ((int)blockIdx.x >= cf.BHpad) {
                conv_feed_worker(cf, &sm, T_, H);
                return;
            }
            if ((int)blockIdx.x >= cf.BH) return;
            if (threadIdx.x == 0)
                __hip_atomic_store(&cf.hdr[blockIdx.x], pub_word(cf.epoch, xcc_id()), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
    }

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
    if (tid < 2 * NSB * (D / 32)) (&sm.fbm[0][0][0])[tid] = 0u;
    if (tid < 2) sm.fbany[tid] = 0u;
    if (tid == 0) {
        for (int s = 0; s < 3; ++s) { sm.kmax[s] = 0u; sm.vmax[s] = 0u; }
        sm.oinv = 1.f;
        sm.sinv = 1.f;
    }
    lds_barrier();

    // Both teams run the same sequence of barriers, three per chunk.
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
        // chunk nc's o from the staging rows to global memory: 16 lanes per
        // row (one DPP row), 16 bytes each, so every store instruction writes
        // whole rows.  With the gated norm (GATES and og set) the row leaves
        // as y: its sum of squares over the 16 lanes, then the norm weight
        // and the output gate, in the arithmetic order of the stand-alone
        // post-processing kernel.  At most 3 rows per lane (nthr >= 448); the
        // gate logits of all of them are loaded first.
        auto copy_o = [&](int nc, int tid0, int nthr) {
            if (!ob) return;
            if (GATES && gt.og) {
                const int c8 = 8 * (lane & 15);   // the same columns on every row of this lane
                // the row indices are formed here on every call (an opaque zero on
                // the thread index): hoisted out of the chunk loop they were
                // spilled, and each reload waited for every load and store in flight
                const int tx = tid - tid0 + opaque_zero();
                constexpr int MAXR = 3;
                bf16x8 gv[MAXR];   // raw logits, widened when used
#pragma unroll
                for (int it = 0; it < MAXR; ++it) {
                    const int x = tx + it * nthr;
                    const int tok = min(nc * CH + (x >> 4), T - 1);
                    if (x < CH * D / 8)
                        gv[it] = *reinterpret_cast<const bf16x8*>(gt.og + bbase + ((uint32_t)tok * rs + hoff + c8));
                }
                float wv[8];
                ld8f(gt.norm_w + (uint32_t)h * D + c8, wv);
#pragma unroll
                for (int it = 0; it < MAXR; ++it) {
                    const int x = tx + it * nthr;
                    if (x < CH * D / 8) {   // the same for all 16 lanes of the row
                        const int t = x >> 4;
                        float xv[8];
                        ld8f(&sm.Os[t * LDO + c8], xv);
                        float ss = 0.f;
#pragma unroll
                        for (int e = 0; e < 8; ++e) ss = fmaf(xv[e], xv[e], ss);
                        const float sc = rsqrtf(row_sum<16>(ss) * (1.f / D) + gt.norm_eps);
#pragma unroll
                        for (int e = 0; e < 8; ++e) xv[e] = xv[e] * sc * wv[e] * gate_sigmoid((float)gv[it][e]);
                        if (nc * CH + t < T) st8v_nt(ob + ((uint32_t)(nc * CH + t) * rs + hoff + c8), xv);
                    }
                }
                return;
            }
            for (int x = tid - tid0; x < CH * D / 8; x += nthr) {
                const int t = x >> 4, c8 = 8 * (x & 15);
                const int tok = nc * CH + t;
                if (tok < T) cp16_nt(ob + ((uint32_t)tok * rs + hoff + c8), &sm.Os[t * LDO + c8]);
            }
        };
        floatx4 S[D / 16];       // S^T[16mj + 4g + r][i0 + cl] in S[mj][r]
#pragma unroll
        for (int mj = 0; mj < D / 16; ++mj)   // four adjacent columns: one 16-byte load
            S[mj] = S0 ? *reinterpret_cast<const floatx4*>(&S0[(size_t)bh * D * D + (size_t)(i0 + cl) * D + 16 * mj + 4 * g])
                       : floatx4{0.f, 0.f, 0.f, 0.f};

        floatx4 Ot[NSB];   // O^T[i0 + 4g + r][16tt + cl]: from stage A to the next stage A
        // o of the previous chunk (this wave's columns) into the staging rows,
        // scaled by 1 / s_prev of that chunk; written out as whole rows in the
        // following stage B
        auto stage_o = [&]() {
            const float oi = sm.oinv;
            __bf16* od = &sm.Os[(uint32_t)cl * LDO + i0 + 4 * g + opaque_zero()];
#pragma unroll
            for (int tt = 0; tt < NSB; ++tt) {
                const floatx4 y = Ot[tt] * oi;
                bf16x4 r;
                r[0] = (__bf16)y[0]; r[1] = (__bf16)y[1]; r[2] = (__bf16)y[2]; r[3] = (__bf16)y[3];
                *reinterpret_cast<bf16x4*>(od + SB * tt * LDO) = r;
            }
        };
        for (int n = -1; n < NC; ++n) {
            const int nn = n + 1;
            // ======================================================= stage A
            KD_PHASE_MARK(n, 0);
            if (n >= 1) stage_o();
            Frag vw[KC_];      // v of value column i0 + cl, tokens 32ks + 8g .. + 7 (to stage C)
            if (n >= 0) {
                if (CKPT) {
                    E* dst = static_cast<E*>(ck.S) + ((size_t)bh * NC + n) * D * D;
                    const float si = sm.sinv;   // in record order (16-byte runs)
#pragma unroll
                    for (int kb = 0; kb < D / 32; ++kb)
                        st_run_nt(dst + rec_run<D>(i0 + cl, kb, g), S[2 * kb], S[2 * kb + 1], si);
                }
                // Y^T = S Kbar^T and O^T = S Qbar^T (M = value index, N = token)
                // per token sub-block tt, as S_tt Kloc^T and S_tt Qloc^T with S_tt
                // the state decayed to the start of sub-block tt (in place);
                // partial r0[t] over value columns i0 + 4g .. i0 + 4g + 3 (adjacent
                // under pcol) for the tokens t = 16tt + cl
                float x[NSB];
                // token sub-block tt with the state operand of K-step ks from a_of
                auto read_sub = [&](auto tt_c, auto a_of) {
                    constexpr int tt = decltype(tt_c)::value;
                    floatx4 Yt;
#pragma unroll
                    for (int ks = 0; ks < KD_; ++ks) {
                        const floatx4 z = {0.f, 0.f, 0.f, 0.f};
                        const Frag a = a_of(ks);
                        const Frag bk = TR::ld_state_p(&sm.Kb[(SB * tt + cl) * LD], ks, g);
                        const Frag bq = TR::ld_state_p(&sm.Qb[(SB * tt + cl) * LD], ks, g);
                        Yt = TR::mma(a, bk, ks ? Yt : z);
                        Ot[tt] = TR::mma(a, bq, ks ? Ot[tt] : z);
                    }
                    const bf16x4 vr = *reinterpret_cast<const bf16x4*>(
                        &sm.V[(SB * tt + cl) * LD + TR::pcol(i0 + 4 * g)]);
                    x[tt] = 0.f;
#pragma unroll
                    for (int r = 0; r < 4; ++r) x[tt] += Yt[r] * TR::tof(vr[r]);
                };
                typedef std::integral_constant<int, 0> T0;
                typedef std::integral_constant<int, 1> T1;
                typedef std::integral_constant<int, 2> T2;
                typedef std::integral_constant<int, 3> T3;
                if (sm.slow[n & 1]) {
                    // operands referenced to the chunk start: the state as it
                    // entered the chunk, converted once
                    Frag a[KD_];
#pragma unroll
                    for (int ks = 0; ks < KD_; ++ks) a[ks] = TR::state_frag(S, ks);
                    auto a_of = [&](int ks) { return a[ks]; };
                    read_sub(T0(), a_of); read_sub(T1(), a_of); read_sub(T2(), a_of); read_sub(T3(), a_of);
                } else {
                    // operands referenced to each sub-block's start: the state
                    // decayed in place past every sub-block as it is read
                    auto a_dec = [&](auto tt_c) {
                        constexpr int tt = decltype(tt_c)::value;
                        return [&](int ks) {
                            const Frag a = TR::state_frag(S, ks);
                            if (tt + 1 < NSB) {   // the two state tiles of this K-step, decayed past sub-block tt
                                const float* dc = &sm.fac[facrow::SUB + tt][32 * ks + 4 * g];
                                S[2 * ks] = S[2 * ks] * *reinterpret_cast<const floatx4*>(dc);
                                S[2 * ks + 1] = S[2 * ks + 1] * *reinterpret_cast<const floatx4*>(dc + 16);
                            }
                            return a;
                        };
                    };
                    read_sub(T0(), a_dec(T0())); read_sub(T1(), a_dec(T1()));
                    read_sub(T2(), a_dec(T2())); read_sub(T3(), a_dec(T3()));
                }
                {   // V holds chunk n until stage B; read after the state so as not to
                    // hold up its operand loads
                    const E* vcol = &sm.V[(uint32_t)(8 * g) * LD + TR::pcol(i0 + cl) + opaque_zero()];
#pragma unroll
                    for (int ks = 0; ks < KC_; ++ks)
#pragma unroll
                        for (int e = 0; e < 8; ++e) vw[ks][e] = vcol[(TR::KS * ks + e) * LD];
                }
                // the producers' exact pass over chunk n's diagonal tiles (rare)
                if (sm.fbany[n & 1] != 0u) lds_barrier();
                {
                    // summed over the lane groups: lane (g, cl) then holds this
                    // wave's partial of token 16g + cl
                    const float xs = group4_transpose_sum(x, g);
                    const int t = SB * g + cl;
                    sm.r0p[t * NWC + ((w + (t >> 2)) & (NWC - 1))] = xs;
                }
            }
            KD_PHASE_MARK(n, 3);
            lds_barrier();
            // ======================================================= stage B
            KD_PHASE_MARK(n, 1);
            if (n >= 0 && w == 0) {   // forward substitution (I + M) u = c - beta r0
                const int t_ = lane + opaque_zero();   // its addresses are formed here, not hoisted
                __builtin_amdgcn_s_setprio(3);   // the chain every other wave waits for
                float r0;
                {
                    const floatx4* pr = reinterpret_cast<const floatx4*>(&sm.r0p[t_ * NWC]);
                    const floatx4 a = pr[0] + pr[1];
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
                        floatx4 m4 = *reinterpret_cast<const floatx4*>(&sm.M[t_ * LDM + 16 * sb + 4 * s4]);
                        if (sb >= 2) {   // tiles (3,2), (3,3): G_V on M's beta G_K (1 on rows < 48)
                            const floatx4 g4 = *reinterpret_cast<const floatx4*>(&sm.G3[sb - 2][(t_ & 15) * SB + 4 * s4]);
                            m4 = t_ >= 48 ? m4 * g4 : m4;
                        }
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
            if (n >= 1 && w >= 1) copy_o(n - 1, 64, (NWC - 1) * 64);   // chunk n - 1's o rows
            if (CKPT && n >= 0 && w >= 1) {
                // M and P of chunk n are complete (their last tiles ran in stage
                // A) and nobody writes them in this stage: the idle consumer waves
                // copy them out
                float* dm = ck.M + ((size_t)bh * NC + n) * CH * CH;
                E* dp = static_cast<E*>(ck.P) + ((size_t)bh * NC + n) * CH * CH;
                const int tc = tid - 64 + opaque_zero();   // formed here, not hoisted out of the loop
                for (int x = tc; x < CH * CH / 4; x += (NWC - 1) * 64) {
                    const int t = x >> 4, s4 = x & 15;
                    floatx4 m4 = *reinterpret_cast<const floatx4*>(&sm.M[t * LDM + 4 * s4]);
                    if (t >= 48 && s4 >= 8)   // tiles (3,2), (3,3): times G_V, as the substitution read them
                        m4 = m4 * *reinterpret_cast<const floatx4*>(&sm.G3[(s4 >> 2) - 2][(t - 48) * SB + 4 * (s4 & 3)]);
                    __builtin_nontemporal_store(m4, reinterpret_cast<floatx4*>(dm + t * CH + 4 * s4));
                }
                for (int x = tc; x < CH * CH / 8; x += (NWC - 1) * 64) {
                    const int t = x >> 3, s8 = x & 7;
                    cp16_nt(dp + t * CH + 8 * s8, &sm.P[n & 1][t * LDP + 8 * s8]);
                }
            }
            if (tid == 0 && n >= 0) {
                // slot (n+2)%3 = chunks n-1 and n+2: the former's last reader ran in
                // the previous stage C, the latter's first writer runs in stage A(n+1)
                sm.kmax[(n + 2) % 3] = 0u; sm.vmax[(n + 2) % 3] = 0u;
            }
            if (tid < NSB * (D / 32) && n >= 0) {
                // chunk n's flags were last read in stage A; chunk n + 2 sets them
                // in stage B(n + 1)
                (&sm.fbm[n & 1][0][0])[tid + opaque_zero()] = 0u;
                if (tid == 0) sm.fbany[n & 1] = 0u;
            }
            KD_PHASE_MARK(n, 4);
            lds_barrier();
            // ======================================================= stage C
            KD_PHASE_MARK(n, 2);
            if (n >= 0) {
                // W = u * V of this wave's value columns: bf16 scaled by s_prev for
                // the readout, fp16 scaled by usc for the update
                // (value column i0 + cl, tokens 32ks + 8g .. + 7, read in stage A)
                Frag wa[KC_];
                FragH wb[KC_];
                {
#pragma unroll
                    for (int ks = 0; ks < KC_; ++ks) {
                        const int t0 = TR::KS * ks + 8 * g;
                        const floatx4 a0 = *reinterpret_cast<const floatx4*>(&sm.u[t0]);
                        const floatx4 a1 = *reinterpret_cast<const floatx4*>(&sm.u[t0 + 4]);
                        const floatx4 b0 = *reinterpret_cast<const floatx4*>(&sm.us[t0]);
                        const floatx4 b1 = *reinterpret_cast<const floatx4*>(&sm.us[t0 + 4]);
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const float xv = TR::tof(vw[ks][e]);
                            const float ua = e < 4 ? a0[e] : a1[e - 4], ub = e < 4 ? b0[e] : b1[e - 4];
                            wa[ks][e] = TR::cvt(ua * xv);
                            wb[ks][e] = (_Float16)(ub * xv);
                        }
                    }
                }
                // O^T += W^T P^T (the P fragments of a K-step loaded together)
#pragma unroll
                for (int ks = 0; ks < KC_; ++ks) {
                    Frag pf[NSB];
#pragma unroll
                    for (int tt = 0; tt < NSB; ++tt) pf[tt] = TR::ld_nat(&sm.P[n & 1][(SB * tt + cl) * LDP], ks, g);
#pragma unroll
                    for (int tt = 0; tt < NSB; ++tt) Ot[tt] = TR::mma(wa[ks], pf[tt], Ot[tt]);
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
        stage_o();        // the last chunk's o rows
        lds_barrier();    // (the producers' matching barrier follows their loop)
        copy_o(NC - 1, 0, NWC * 64);
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
        bool slow_p = true;              // the prepared chunk's references (see stage B)
        Col8 keep_kt[2];                 // K-tilde of the prepared chunk, written
                                         //   transposed in the following stage A
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
        // the convolution feed: a chunk's q, k, v rows are read only after its
        // unit is published (its flag read a stage early: a unit that is ready
        // costs no poll); a wait that runs out makes the rows NaN from there on
        bool feed_dead = false;
        unsigned long long feed_pk = 0ull;
        const unsigned feed_me = feed ? xcc_id() : 0u;
        auto feed_peek = [&](int nc) {
            if (feed && !feed_dead)
                feed_pk = __hip_atomic_load(&cf.flags[(size_t)bh * NC + nc], __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
        };
        auto feed_wait = [&](int nc) {
            if (!feed || feed_dead) return;
            unsigned long long wd = feed_pk;
            bool ok = ((unsigned)(wd >> 32) == cf.epoch && (wd & 1ull) != 0ull) ||
                      pub_wait(&cf.flags[(size_t)bh * NC + nc], cf.epoch, 1ull, wd, cf.spin);
            if (ok && ((unsigned)(wd >> 24) & 0xffu) != feed_me) {   // written back by a writer elsewhere
                ok = (wd & PUB_FLUSHED) != 0ull;
                if (ok) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            }
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");   // no row read moves above the wait
            feed_dead = !ok;
        };
        auto feed_poison = [&](Raw8x2& r) {
            if (feed && feed_dead)
#pragma unroll
                for (int e = 0; e < RB; ++e) r.clear(e, __builtin_nanf(""));
        };
        feed_wait(0);
        load_q(0);
        load_k(0);
        load_v(0);
        load_f(0);
        feed_poison(rq);
        feed_poison(rk);
        feed_poison(rv);
        // Exact terms of the diagonal tile I_ of chunk ch for the key channels
        // whose decay over that sub-block is below the floor (left out of the
        // tile's matrix product), added to M and P in LDS: lane (g, cl) takes
        // the entries t = 4g + r, s = cl (rows of the sub-block) and sums over
        // those channels k_t k_s E (G_K, s < t) and q_t k_s E (P, s <= t),
        // E = prod_{s<u<=t} f_u; then M[t][s] += beta_t dG_K G_V[t][s] (G_V again
        // from V) and P[t][s] += dP.  Rare path: the rows are re-read from
        // global memory, and the forget gate is made again from its logit
        // (GATES) with the producers' function and rounding.
        auto diag_exact = [&](int I_, int ch) {
            const unsigned* fm = sm.fbm[ch & 1][I_];
            unsigned any = 0u;
#pragma unroll
            for (int wd = 0; wd < D / 32; ++wd) any |= fm[wd];
            if (__builtin_amdgcn_readfirstlane(any) == 0u) return;
            const int row0 = ch * CH + SB * I_;
            floatx4 dk = {0.f, 0.f, 0.f, 0.f}, dp = dk;
#pragma unroll 1
            for (int wd = 0; wd < D / 32; ++wd) {
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
                    float fl = 1.f;   // f of row cl (1 past the end)
                    if (row0 + cl < T) {
                        fl = TR::tof(fb[(uint32_t)(row0 + cl) * rs + cj]);
                        if (GATES) fl = TR::tof(TR::cvt(forget_gate(fl, gex)));
                    }
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
                if (s_ < t_) {   // tile (3,3) holds beta G_K (its G_V goes on when read)
                    if (I_ == NSB - 1) sm.M[t_ * LDM + s_] += sm.beta[ch & 1][t_] * dk[r];
                    else sm.M[t_ * LDM + s_] += sm.beta[ch & 1][t_] * dk[r] * gv[r];
                }
                if (s_ <= t_) {
                    E& pe = sm.P[ch & 1][t_ * LDP + s_];
                    pe = TR::cvt(TR::tof(pe) + dp[r]);
                }
            }
        };
        // One lower-triangular 16 x 16 tile (I_ >= J_) of M (DO_M) and / or P
        // (DO_P) for chunk ch.  The M part writes only the strictly lower
        // entries of M, the P part the tile's entries of P; the two parts never
        // touch the same entry.  The decay between the two sub-blocks goes on
        // the Kr fragment (fac row fr).
        // MODE: GT_MP both parts; GT_P the P part; GT_GK M's rows as beta G_K
        // (tiles 8, 9; G_V goes on when M is read); GT_GV G_V into G3 (tiles 8, 9).
        auto gram_tile = [&](auto mode_c, int tile, int ch) {
            constexpr int MODE = decltype(mode_c)::value;
            constexpr bool DO_GK = MODE == GT_MP || MODE == GT_GK, DO_GV = MODE == GT_MP || MODE == GT_GV;
            constexpr bool DO_M = DO_GK || DO_GV, DO_P = MODE == GT_MP || MODE == GT_P;
            const int I_ = tile < 1 ? 0 : tile < 3 ? 1 : tile < 6 ? 2 : 3;
            const int J_ = tile - (I_ * (I_ + 1)) / 2;
            const int fr = I_ == J_ ? facrow::DIAG + I_
                         : I_ - J_ == 2 ? (J_ == 0 ? facrow::D20 : facrow::D31)
                         : I_ - J_ == 3 ? facrow::D30 : -1;
            floatx4 gk, pp, gv;
            const E* aK = &sm.Kb[(SB * I_ + cl) * LD];
            const E* aQ = &sm.Qb[(SB * I_ + cl) * LD];
            const E* aV = &sm.V[(SB * I_ + cl) * LD];
            const E* bK = &sm.Kc[(SB * J_ + cl) * LD];
            const E* bV = &sm.V[(SB * J_ + cl) * LD];
            // operands of one K-step (not prefetched a step ahead: the registers
            // are needed elsewhere, and the other waves of the SIMD cover the
            // LDS latency)
            struct GF { Frag k, a, q, v, w; };
            auto ldg = [&](int ks) {
                GF r;
                if (DO_GK || DO_P) {
                    r.k = TR::ld_nat(bK, ks, g);
                    if (fr >= 0 && !slow_p) r.k = TR::scale_k(r.k, 1.f, sm.fac[fr], ks, g);
                }
                if (DO_GK) r.a = TR::ld_nat(aK, ks, g);
                if (DO_GV) { r.v = TR::ld_nat(aV, ks, g); r.w = TR::ld_nat(bV, ks, g); }
                if (DO_P) r.q = TR::ld_nat(aQ, ks, g);
                return r;
            };
#pragma unroll
            for (int ks = 0; ks < KD_; ++ks) {
                const floatx4 z = {0.f, 0.f, 0.f, 0.f};
                const GF cur = ldg(ks);
                if (DO_GK) gk = TR::mma(cur.a, cur.k, ks ? gk : z);
                if (DO_P) pp = TR::mma(cur.q, cur.k, ks ? pp : z);
                if (DO_GV) gv = TR::mma(cur.v, cur.w, ks ? gv : z);
            }
            const int s_ = SB * J_ + cl + opaque_zero();   // addresses formed here, not hoisted
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t_ = SB * I_ + 4 * g + r;
                if (MODE == GT_MP && s_ < t_) sm.M[t_ * LDM + s_] = sm.beta[ch & 1][t_] * gk[r] * gv[r];
                if (MODE == GT_GK && s_ < t_) sm.M[t_ * LDM + s_] = sm.beta[ch & 1][t_] * gk[r];
                if (MODE == GT_GV) sm.G3[tile - 8][(4 * g + r) * SB + cl] = gv[r];
                if (DO_P) sm.P[ch & 1][t_ * LDP + s_] = TR::cvt((s_ <= t_) ? pp[r] : 0.f);
            }
        };
        typedef std::integral_constant<int, GT_MP> kMP;
        typedef std::integral_constant<int, GT_P> kP;
        typedef std::integral_constant<int, GT_GK> kGK;
        typedef std::integral_constant<int, GT_GV> kGV;

        for (int n = -1; n < NC; ++n) {
            const int nn = n + 1;             // chunk the producers prepare
            const bool prod_on = nn < NC;
            feed_peek(min(nn + 1, NC - 1));   // the chunk whose rows this iteration loads
            const int oz = opaque_zero();     // per-lane LDS addresses stay inside the loop
            // ======================================================= stage A
            KD_PHASE_MARK(n, 0);
            // the producer waves with a Gram product in this stage (beta G_K and
            // P) would finish last: they issue before the others
            if (pw < 2 || pw >= 6) __builtin_amdgcn_s_setprio(1);
            if (n >= 0) {   // transposed K-tilde of chunk n and its last two Gram tiles
#pragma unroll
                for (int c2 = 0; c2 < 2; ++c2) {
                    keep_kt[c2].store(&sm.KtT[(ch0 + c2) * LDT + rb]);
                }
                // tiles 8 and 9 (rows 48..63) are first read by the substitution
                // (M) and the readout (P) of chunk n: they run here on producer
                // waves 0..3 and 6, 7, one matrix product each (beta G_K into M,
                // G_V into G3, P), so that no wave carries two; producer waves
                // pw and pw + 4 share a SIMD, so the G_K waves (with the decay
                // factors) have theirs alone
                if (pw < 2) gram_tile(kGK(), 8 + pw, n);
                else if (pw < 4) gram_tile(kGV(), 8 + (pw & 1), n);
                else if (pw >= 6) gram_tile(kP(), 8 + (pw & 1), n);
                if (sm.fbany[n & 1] != 0u) {   // every tile of chunk n is done: exact pass
                    lds_barrier();
                    if ((pw & 1) == 0) diag_exact(pw >> 1, n);
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
            __builtin_amdgcn_s_setprio(0);
            lds_barrier();
            // ======================================================= stage B
            KD_PHASE_MARK(n, 1);
            // the producers' work bounds stages B and C, where the consumers
            // other than the substitution's wave have slack: their instructions
            // issue first (the substitution itself runs at a higher level).  With
            // the gates, the consumers' row writes carry the gated norm in stage
            // B, so there the boost starts in stage C.
            if (!GATES) __builtin_amdgcn_s_setprio(2);
            if (prod_on) {   // operands of chunk nn into LDS
                // Decay products from the 8-row blocks of the producer waves
                // (bprod[p]; sub-block I2 = blocks 2 I2 and 2 I2 + 1), per wave:
                // astart / bstart = decay of its sub-block's rows before / after
                // its own, after = decay of the sub-blocks after its own, and the
                // factor-table rows it writes (row pw; waves 0, 1 also row pw + 8).
                // pw is wave-uniform: one straight-line case per value.
                float astart[2], bstart[2], after[2], fv0[2], fv1[2], lastsub[2], gcv[2], gst[2];
                const float* bpb = &sm.bprod[0][ch0 + oz];   // one base, constant offsets
                unsigned fl2 = 0u;
                auto consts = [&](auto pw_c) {
                    constexpr int PW = decltype(pw_c)::value, I = PW >> 1, H2 = PW & 1;
                    auto xbp = [&](int p) { return *reinterpret_cast<const float2*>(bpb + p * D); };
                    auto sub = [&](int I2) { const float2 a = xbp(2 * I2), b = xbp(2 * I2 + 1); return make_float2(a.x * b.x, a.y * b.y); };
                    auto mul = [](float2 a, float2 b) { return make_float2(a.x * b.x, a.y * b.y); };
                    auto facv = [&](auto row_c) {
                        constexpr int R = decltype(row_c)::value;
                        if constexpr (R < facrow::D20) {
                            const float2 x = sub(R - facrow::DIAG);
                            return make_float2(x.x >= kSafeFloor ? __builtin_amdgcn_rcpf(x.x) : 0.f,
                                               x.y >= kSafeFloor ? __builtin_amdgcn_rcpf(x.y) : 0.f);
                        } else if constexpr (R == facrow::D20) {
                            return sub(1);
                        } else if constexpr (R == facrow::D31) {
                            return sub(2);
                        } else if constexpr (R == facrow::D30) {
                            return mul(sub(1), sub(2));
                        } else {
                            return sub(R - facrow::SUB);
                        }
                    };
                    const float2 h0 = xbp(2 * I), h1 = xbp(2 * I + 1);
                    astart[0] = H2 ? h0.x : 1.f; astart[1] = H2 ? h0.y : 1.f;
                    bstart[0] = H2 ? 1.f : h1.x; bstart[1] = H2 ? 1.f : h1.y;
                    float2 af = make_float2(1.f, 1.f);
                    if constexpr (I < 3) af = sub(3);
                    if constexpr (I < 2) af = mul(sub(2), af);
                    if constexpr (I < 1) af = mul(sub(1), af);
                    after[0] = af.x; after[1] = af.y;
                    const float2 f0 = facv(std::integral_constant<int, PW>());
                    fv0[0] = f0.x; fv0[1] = f0.y;
                    if constexpr (PW + NWP < facrow::N) {
                        const float2 f1 = facv(std::integral_constant<int, PW + NWP>());
                        fv1[0] = f1.x; fv1[1] = f1.y;
                    }
                    if constexpr (H2 == 0) {   // channels of sub-block I below the floor
                        const float2 x = mul(h0, h1);
                        fl2 = (x.x >= kSafeFloor ? 0u : 1u) | (x.y >= kSafeFloor ? 0u : 2u);
                    }
                    if constexpr (PW == 0) {   // the state's decay over the last sub-block
                        const float2 x = sub(NSB - 1);
                        lastsub[0] = x.x; lastsub[1] = x.y;
                    }
                    // decay before sub-block I and over the whole chunk (one
                    // association, the same in every wave)
                    const float2 p1 = sub(0), p2 = mul(p1, sub(1)), p3 = mul(p2, sub(2)), pc = mul(p3, sub(3));
                    const float2 ps = I == 0 ? make_float2(1.f, 1.f) : I == 1 ? p1 : I == 2 ? p2 : p3;
                    gst[0] = ps.x; gst[1] = ps.y;
                    gcv[0] = pc.x; gcv[1] = pc.y;
                };
                switch (pw) {
                case 0: consts(std::integral_constant<int, 0>()); break;
                case 1: consts(std::integral_constant<int, 1>()); break;
                case 2: consts(std::integral_constant<int, 2>()); break;
                case 3: consts(std::integral_constant<int, 3>()); break;
                case 4: consts(std::integral_constant<int, 4>()); break;
                case 5: consts(std::integral_constant<int, 5>()); break;
                case 6: consts(std::integral_constant<int, 6>()); break;
                default: consts(std::integral_constant<int, 7>()); break;
                }
                // A chunk with every channel's decay at or above the floor takes
                // operands referenced to the chunk start: Qb = q gamma, Kb = k gamma,
                // Kc = k / gamma (gamma: decay from the chunk start), so its Gram
                // tiles need no factors and the consumers read the state as it
                // entered the chunk.  Otherwise the sub-block references above.
                // Every wave holds every channel: the vote is the same in all.
                slow_p = __builtin_amdgcn_ballot_w64(!(gcv[0] >= kSafeFloor && gcv[1] >= kSafeFloor)) == 0ull;
                if (pw == 0 && lane == 0) sm.slow[nn & 1] = slow_p ? 1u : 0u;
                // Gram rows in pcol order, the state's rows in natural order
                st2(&sm.fac[pw][pw < facrow::SUB ? pc0 : ch0], fv0[0], fv0[1]);
                if (pw + NWP < facrow::N) st2(&sm.fac[pw + NWP][ch0], fv1[0], fv1[1]);
                if (fl2) {
                    atomicOr(&sm.fbm[nn & 1][pw >> 1][ch0 >> 5], fl2 << (ch0 & 31));
                    atomicOr(&sm.fbany[nn & 1], 1u);
                }
                // the state's decay in stage C: over the chunk, or over its last
                // sub-block when the earlier ones were applied as it was read
                if (pw == 0) st2(&sm.gam[nn & 1][ch0], slow_p ? gcv[0] : lastsub[0], slow_p ? gcv[1] : lastsub[1]);
                // K-tilde is kept scaled by ksc (a power of 2) for the fp16 update
                const int ek = pow2_exp(__uint_as_float(sm.kmax[nn % 3]));
                const float ksc = ldexpf(1.f, -ek);
                // suffix products within the wave's rows: b (to the sub-block end);
                // ksc * gamma_C / gamma (to the chunk end) is b times tk
                float bs[RB][2], tk[2];
#pragma unroll
                for (int c2 = 0; c2 < 2; ++c2) {
                    tk[c2] = after[c2] * ksc;
                    bs[RB - 1][c2] = bstart[c2];
#pragma unroll
                    for (int e = RB - 2; e >= 0; --e) bs[e][c2] = bs[e + 1][c2] * rf.get(e + 1, c2);
                }
                // chunk-start references: a times the decay before the sub-block,
                // and Kc = k b (decay after the sub-block) / gamma_C
                float ga[2], cm[2];   // a (or gamma) at the current row; Kc = k bs cm
#pragma unroll
                for (int c2 = 0; c2 < 2; ++c2) {
                    ga[c2] = slow_p ? astart[c2] * gst[c2] : astart[c2];
                    cm[c2] = slow_p ? after[c2] * __builtin_amdgcn_rcpf(gcv[c2]) : 1.f;
                }
                float kprev[2] = {0.f, 0.f};
                const int pcz = pc0 + oz;
#pragma unroll
                for (int e = 0; e < RB; ++e) {
                    float qo[2], ko[2], co[2];
#pragma unroll
                    for (int c2 = 0; c2 < 2; ++c2) {
                        ga[c2] *= rf.get(e, c2);
                        const float kf = rk.get(e, c2), qf = rq.get(e, c2);
                        const float kt = kf * (bs[e][c2] * tk[c2]);   // K-tilde * ksc
                        qo[c2] = qf * ga[c2];
                        ko[c2] = kf * ga[c2];
                        co[c2] = kf * (bs[e][c2] * cm[c2]);
                        if (e & 1) keep_kt[c2].set_pair_h(e >> 1, kprev[c2], kt);
                        else kprev[c2] = kt;
                    }
                    st2(&sm.Qb[(rb + e) * LD + pcz], qo[0], qo[1]);
                    st2(&sm.Kb[(rb + e) * LD + pcz], ko[0], ko[1]);
                    st2(&sm.Kc[(rb + e) * LD + pcz], co[0], co[1]);
                    rv.store(&sm.V[(rb + e) * LD + pcz], e);
                }
            }
            const int npf = min(nn + 1, NC - 1);   // prefetch of chunk nn + 1
            feed_wait(npf);
            load_q(npf);
            feed_poison(rq);
            KD_PHASE_MARK(n, 4);
            lds_barrier();
            // ======================================================= stage C
            KD_PHASE_MARK(n, 2);
            if (GATES) __builtin_amdgcn_s_setprio(2);
            load_k(npf);
            feed_poison(rk);
            if (prod_on) gram_tile(kMP(), pw, nn);   // tiles 0..7
            load_v(npf);
            feed_poison(rv);
            load_f(npf);
            KD_PHASE_MARK(n, 5);
            __builtin_amdgcn_s_setprio(0);
            lds_barrier();
        }
        lds_barrier();   // the consumers stage the last chunk's o
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
                           *ck, FwdGates{}, ConvFeed{}, (const int*)nullptr, T, H);
    else
        hipLaunchKernelGGL((kd_fwd16_kernel<false, false>), dim3((unsigned)(B * H)), dim3(f16w::NT), 0, st,
                           (const E*)q, (const E*)k, (const E*)v, (const E*)f, beta, c, S0, (E*)o, ST,
                           FwdCkpt{}, FwdGates{}, ConvFeed{}, cu, T, H);
    return hipGetLastError();
}

// The forward with the gates made from their logits (f_raw [B,T,H,D] bf16,
// beta_raw and c_raw [B,T,H] fp32) as the producers load them; with og set,
// o leaves through the gated per-head norm (FwdGates).
hipError_t launch_fwd16_gates(const void* q, const void* k, const void* v, const void* f_raw,
                              const float* beta_raw, const float* c_raw, const float* a_log, float beta_scale,
                              const void* og, const float* norm_w, float norm_eps,
                              const float* S0, void* o, float* ST, int B, int T, int H, hipStream_t st)
{
    typedef __bf16 E;
    FwdGates gt;
    gt.a_log = a_log;
    gt.beta_scale = beta_scale;
    gt.og = static_cast<const E*>(og);
    gt.norm_w = norm_w;
    gt.norm_eps = norm_eps;
    hipLaunchKernelGGL((kd_fwd16_kernel<false, true>), dim3((unsigned)(B * H)), dim3(f16w::NT), 0, st,
                       (const E*)q, (const E*)k, (const E*)v, (const E*)f_raw, beta_raw, c_raw, S0, (E*)o, ST,
                       FwdCkpt{}, gt, ConvFeed{}, (const int*)nullptr, T, H);
    return hipGetLastError();
}

int compute_units();
unsigned bwd_wait_polls();

// launch epochs of the fused mixer forward (see ConvFeed)
static unsigned next_feed_epoch() {
    static std::atomic<unsigned> e{0u};
    unsigned v = e.fetch_add(1u) + 1u;
    if (v == 1u) {   // first launch of the process: start from the clock
        const unsigned t = (unsigned)time(nullptr) * 3266489917u;
        e.fetch_add(t);
        v += t;
    }
    return v;
}

// Zeroes the hand-off words of a fused mixer launch (a kernel rather than a
// memset, so that a captured graph replays it correctly).
__global__ void kd_fwd16_feed_clear_kernel(unsigned long long* __restrict__ w, int n)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) w[i] = 0ull;
}

// Convolution workers a forward block can take beside the B*H forward blocks
// (0: the feed does not fit; then the convolution runs as its own kernel
// first): one per free compute unit, in multiples of 8, at least 64.
int fwd16_feed_workers(int BH) {
    const int BHpad = (BH + 7) & ~7;
    const int nwork = ((compute_units() - BHpad) / 8) * 8;
    return nwork >= 64 ? nwork : 0;
}

// The mixer forward in one launch: the convolution of q, k, v (conv_size 4,
// into q, k, v) by workers beside the forward with the gates from their
// logits (launch_fwd16_gates); hw: 8 * (B*H + B*H*NC) bytes of hand-off words.
hipError_t launch_fwd16_mixer_fed(const void* const raw[3], void* const out[3], const float* const conv[3],
                                  const void* f_raw, const float* beta_raw, const float* c_raw,
                                  const float* a_log, float beta_scale, const void* og, const float* norm_w,
                                  float norm_eps, const float* S0, void* o, float* ST, void* hw, int nwork,
                                  int B, int T, int H, hipStream_t st)
{
    typedef __bf16 E;
    MixPreArgs mx{};
    for (int i = 0; i < 3; ++i) { mx.raw[i] = raw[i]; mx.out[i] = out[i]; mx.conv[i] = conv[i]; }
    mx.K = 4;
    FwdGates gt;
    gt.a_log = a_log;
    gt.beta_scale = beta_scale;
    gt.og = static_cast<const E*>(og);
    gt.norm_w = norm_w;
    gt.norm_eps = norm_eps;
    const int NC = (T + CH - 1) / CH;
    ConvFeed cf;
    cf.mx = mx;
    cf.BH = B * H;
    cf.BHpad = (cf.BH + 7) & ~7;
    cf.nwork = nwork;
    cf.hdr = static_cast<unsigned long long*>(hw);
    cf.flags = cf.hdr + cf.BH;
    cf.epoch = next_feed_epoch();
    cf.spin = bwd_wait_polls();
    const int nw = cf.BH + cf.BH * NC;
    hipLaunchKernelGGL(kd_fwd16_feed_clear_kernel, dim3((unsigned)((nw + 255) / 256)), dim3(256), 0, st, cf.hdr, nw);
    hipLaunchKernelGGL((kd_fwd16_kernel<false, true>), dim3((unsigned)(cf.BHpad + nwork)), dim3(f16w::NT), 0, st,
                       (const E*)mx.out[0], (const E*)mx.out[1], (const E*)mx.out[2], (const E*)f_raw, beta_raw,
                       c_raw, S0, (E*)o, ST, FwdCkpt{}, gt, cf, (const int*)nullptr, T, H);
    return hipGetLastError();
}

}  // namespace kd
