// kd_fwd16s.hip -- the chunkwise forward for few heads (bf16 inputs, d = 128):
// a chunk-parallel preparation launch, then one streaming state pass per
// (b, h).
//
// Same recurrence and chunk algebra as the one-launch forward (kd_fwd16.hip;
// onedev.kr KronLSTM summary, sections "어떻게 동작하나" and "어떻게 쓰나";
// aitrends.kr Gated DeltaNet-2 summary, section "방법론" steps 3-4, which
// states the chunk's triangular system and the inverse T = (I + M)^{-1}):
// per 64-token chunk,
//     u = A (c - beta r0),  A = (I + M)^{-1},  r0_t = v_t^T S0 Kbar_t,
//     O = Qbar S0^T + P (u * V),  S_C = S0 diag(gamma_C) + (u * V)^T Ktilde.
// Everything but r0, u, O and S_C depends on the chunk's own inputs only, so
// with few heads (B*H well under the compute-unit count) the one-launch
// forward leaves most of the chip idle while each head's chain runs.  Here:
//   1. kd_fwd16_prep_kernel, one workgroup per (b, h, chunk), all chunks at
//      once: decay products, the state operands Kbar = k gamma, Qbar = q gamma
//      (gamma from the chunk start), Ktilde = k gamma_C / gamma, the Gram
//      matrices M and P (chunk-start or 16-token sub-block references with
//      the exact pass, as in the one-launch kernel), and A = (I + M)^{-1} by
//      blocks of 16: the diagonal blocks by substitution, then
//      A_IJ = -A_II sum_{J <= K < I} M_IK A_KJ, one block diagonal at a time.
//      Each unit leaves an image of exactly the LDS layout the state pass
//      uses (f16s::G1_* and G2_* offsets) in the workspace.
//   2. kd_fwd16_state_kernel, one workgroup per (b, h): four consumer waves
//      hold 32 value columns of the fp32 state each (two 16-column halves
//      sharing every operand fragment read); four loader waves stream the
//      images in: group 1 (Kbar, Qbar, V; read in stage A) of chunk n + 1 is
//      written to LDS during stage C of chunk n, group 2 (Ktilde^T, P, A, the
//      gates) of chunk n during its stage A, each from registers loaded a
//      whole chunk earlier.  Per chunk: A: state reads (MFMA), r0 partials;
//      B: u = A b on one wave (64 broadcasts), the loaders write the previous
//      chunk's o rows; C: readout and update (MFMA).
#include <atomic>
#include <ctime>
#include <type_traits>

#include "kd_device.h"
#include "kd_handoff.h"

// Phase markers: no-ops here; a profiling build may define them to record
// timestamps at the stage boundaries of the state pass.
#ifndef KD_PHASE_MARK
#define KD_PHASE_MARK(chunk, id) ((void)0)
#endif

namespace kd {

namespace f16s {
constexpr int D = 128;
constexpr int LD = D + 16;     // row-major [CH][D] operands, pcol columns
constexpr int LDT = CH + 8;    // Ktilde^T [D][CH] (fp16)
constexpr int LDP = CH + 8;    // P [CH][CH] (bf16)
constexpr int LDA = CH + 4;    // M and A [CH][CH] (fp32)
constexpr int LDO = D + 8;     // o staging rows
// the image of one (b, h, chunk) unit, byte offsets
constexpr uint32_t ROWB = CH * LD * 2;
constexpr uint32_t G1_KB = 0, G1_QB = ROWB, G1_V = 2 * ROWB, G1_BYTES = 3 * ROWB;
constexpr uint32_t G2_KT = 0;
constexpr uint32_t G2_P = G2_KT + D * LDT * 2;
constexpr uint32_t G2_A = G2_P + CH * LDP * 2;
constexpr uint32_t G2_GAM = G2_A + CH * LDA * 4;   // gamma_C per key channel (fp32)
constexpr uint32_t G2_BETA = G2_GAM + D * 4;
constexpr uint32_t G2_C = G2_BETA + CH * 4;
constexpr uint32_t G2_SCAL = G2_C + CH * 4;        // [0] ek (Ktilde carries 2^-ek), [1] max |v| bits
constexpr uint32_t G2_BYTES = G2_SCAL + 256;
constexpr uint32_t UNIT_BYTES = G1_BYTES + G2_BYTES;
static_assert(G1_BYTES % 256 == 0 && G2_BYTES % 256 == 0, "images of whole 256-byte blocks");
// preparation: eight waves of eight rows
constexpr int PNT = 512, PNW = 8, PRB = CH / PNW;
// state pass: four consumer waves (32 value columns each), four loader waves
#ifndef KD_FWD16S_NWC
#define KD_FWD16S_NWC 4
#endif
constexpr int NWC = KD_FWD16S_NWC, NWL = 4, SNT = 64 * (NWC + NWL), CPW = D / NWC, NHV = CPW / 16;
constexpr int G1_SLOTS = (G1_BYTES / 16 + NWL * 64 - 1) / (NWL * 64);
constexpr int G2_SLOTS = (G2_BYTES / 16 + NWL * 64 - 1) / (NWL * 64);
// factor rows of the Gram tiles (sub-block references), pcol order
namespace frow {
constexpr int DIAG = 0;    // DIAG + I: 1 / (decay over sub-block I), 0 below the floor
constexpr int D20 = 4;     // decay over sub-block 1 (tile I=2, J=0)
constexpr int D31 = 5;     // decay over sub-block 2 (tile I=3, J=1)
constexpr int D30 = 6;     // decay over sub-blocks 1 and 2 (tile I=3, J=0)
constexpr int N = 7;
}  // namespace frow
}  // namespace f16s

// Workspace of the few-heads forward: one image per (b, h, chunk), then the
// hand-off words of the fused launch: hdr [B*H], flags [B*H*NC].
size_t fwd16_split_ws_bytes(int B, int T, int H) {
    const size_t nc = (size_t)((T + CH - 1) / CH);
    const size_t units = (size_t)B * H * nc;
    return units * f16s::UNIT_BYTES + 8 * ((size_t)B * H + units);
}

struct PrepSmem {
    alignas(16) __bf16 Qg[CH * f16s::LD];   // Gram operands; later A (fp32) and block scratch
    alignas(16) __bf16 Kg[CH * f16s::LD];
    alignas(16) __bf16 Kc[CH * f16s::LD];
    alignas(16) __bf16 V[CH * f16s::LD];
    alignas(16) float M[CH * f16s::LDA];    // beta_t tril_{-1}(G_K * G_V)
    alignas(16) __bf16 P[CH * f16s::LDP];   // tril_0 of the decayed Q K^T
    alignas(16) float beta[CH];
    alignas(16) float bprod[f16s::PNW][f16s::D];
    alignas(16) float fac[f16s::frow::N][f16s::D];
    unsigned kmax, vmax;
    unsigned fbm[NSB][f16s::D / 32];
    unsigned fbany;
};

// One preparation unit (b, h, chunk n) with the block's LDS sm: the image of
// chunk n of head bh into img.  Every thread of the block calls it.
__device__ __forceinline__ void prep_unit(
    PrepSmem& sm, const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ f, const float* __restrict__ beta, const float* __restrict__ cc,
    unsigned char* __restrict__ img, int n, int bh, int T, int H)
{
    using namespace f16s;
    typedef Bf16T TR;
    typedef __bf16 E;
    typedef TR::Frag Frag;
    constexpr int KD_ = D / TR::KS;
    const int tid = threadIdx.x;
    const int lane = tid & 63, g = lane >> 4, cl = lane & 15;
    const int pw = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int b = bh / H, h = bh % H;
    const int NC = (T + CH - 1) / CH;
    const uint32_t rs = (uint32_t)H * D;
    const size_t bbase = (size_t)b * T * H * D;
    const E* qb = q + bbase;
    const E* kb = k + bbase;
    const E* vb = v + bbase;
    const E* fb = f + bbase;
    const uint32_t hoff = (uint32_t)h * D;
    unsigned char* g1 = img + ((size_t)bh * NC + n) * UNIT_BYTES;
    unsigned char* g2 = g1 + G1_BYTES;

    for (int x = tid; x < CH * LDP; x += PNT) sm.P[x] = TR::cvt(0.f);
    for (int x = tid; x < CH * LDA; x += PNT) sm.M[x] = 0.f;
    if (tid < NSB * (D / 32)) (&sm.fbm[0][0])[tid] = 0u;
    if (tid == 0) { sm.fbany = 0u; sm.kmax = 0u; sm.vmax = 0u; }

    // rows rb .. rb + 7, channels ch0, ch0 + 1 (rows past the end: the last
    // row, in bounds, cleared below)
    const int rb = PRB * pw;
    const int ch0 = 2 * lane;
    const int pc0 = TR::pcol(ch0);
    Raw8x2 rq, rk, rv, rf;
    {
        const int t0 = min(n * CH + rb, T - 1);
        const int last = min(PRB - 1, T - 1 - t0);
        const uint32_t off = (uint32_t)t0 * rs + hoff + ch0;
        rq.load(qb, off, rs, last);
        rk.load(kb, off, rs, last);
        rv.load(vb, off, rs, last);
        rf.load(fb, off, rs, last);
    }
#pragma unroll
    for (int e = 0; e < PRB; ++e)
        if (n * CH + rb + e >= T) { rq.clear(e, 0.f); rk.clear(e, 0.f); rv.clear(e, 0.f); rf.clear(e, 1.f); }
    lds_barrier();   // the clears above are done before any atomic below
    {
        float tot[2];
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
            atomicMax(&sm.kmax, __float_as_uint(km));
            atomicMax(&sm.vmax, __float_as_uint(vm));
        }
        if (pw == 0) {
            const int t = n * CH + lane;
            const uint32_t gi = (uint32_t)min(t, T - 1) * H + h;
            const float bt = t < T ? beta[(size_t)b * T * H + gi] : 0.f;
            const float ct = t < T ? cc[(size_t)b * T * H + gi] : 0.f;
            sm.beta[lane] = bt;
            reinterpret_cast<float*>(g2 + G2_BETA)[lane] = bt;
            reinterpret_cast<float*>(g2 + G2_C)[lane] = ct;
        }
    }
    lds_barrier();

    // ---------------------------------------------------- decay products
    // per wave (pw wave-uniform, one straight-line case per value):
    // astart / bstart = decay of its sub-block's rows before / after its own
    // eight, after = decay of the sub-blocks after its own, gst = decay before
    // its sub-block, gcv = decay over the chunk (one association in every
    // wave), fv = its factor-table row (waves 0 .. 6), fl2 = its sub-block's
    // channels below the floor (even waves)
    float astart[2], bstart[2], after[2], gst[2], gcv[2], fv[2] = {1.f, 1.f};
    unsigned fl2 = 0u;
    {
        const float* bpb = &sm.bprod[0][ch0];
        auto consts = [&](auto pw_c) {
            constexpr int PW = decltype(pw_c)::value, I = PW >> 1, H2 = PW & 1;
            auto xbp = [&](int p) { return *reinterpret_cast<const float2*>(bpb + p * D); };
            auto mul = [](float2 a, float2 c) { return make_float2(a.x * c.x, a.y * c.y); };
            auto sub = [&](int I2) { return mul(xbp(2 * I2), xbp(2 * I2 + 1)); };
            const float2 h0 = xbp(2 * I), h1 = xbp(2 * I + 1);
            astart[0] = H2 ? h0.x : 1.f; astart[1] = H2 ? h0.y : 1.f;
            bstart[0] = H2 ? 1.f : h1.x; bstart[1] = H2 ? 1.f : h1.y;
            float2 af = make_float2(1.f, 1.f);
            if constexpr (I < 3) af = sub(3);
            if constexpr (I < 2) af = mul(sub(2), af);
            if constexpr (I < 1) af = mul(sub(1), af);
            after[0] = af.x; after[1] = af.y;
            const float2 p1 = sub(0), p2 = mul(p1, sub(1)), p3 = mul(p2, sub(2)), pc = mul(p3, sub(3));
            const float2 ps = I == 0 ? make_float2(1.f, 1.f) : I == 1 ? p1 : I == 2 ? p2 : p3;
            gst[0] = ps.x; gst[1] = ps.y;
            gcv[0] = pc.x; gcv[1] = pc.y;
            if constexpr (PW < frow::D20) {
                const float2 x = sub(PW - frow::DIAG);
                fv[0] = x.x >= kSafeFloor ? __builtin_amdgcn_rcpf(x.x) : 0.f;
                fv[1] = x.y >= kSafeFloor ? __builtin_amdgcn_rcpf(x.y) : 0.f;
            } else if constexpr (PW == frow::D20) {
                const float2 x = sub(1); fv[0] = x.x; fv[1] = x.y;
            } else if constexpr (PW == frow::D31) {
                const float2 x = sub(2); fv[0] = x.x; fv[1] = x.y;
            } else if constexpr (PW == frow::D30) {
                const float2 x = mul(sub(1), sub(2)); fv[0] = x.x; fv[1] = x.y;
            }
            if constexpr (H2 == 0) {
                const float2 x = mul(h0, h1);
                fl2 = (x.x >= kSafeFloor ? 0u : 1u) | (x.y >= kSafeFloor ? 0u : 2u);
            }
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
    }
    // chunk-start Gram references when every channel's chunk decay is at or
    // above the floor (the same vote in every wave: each holds all channels)
    const bool slow = __builtin_amdgcn_ballot_w64(!(gcv[0] >= kSafeFloor && gcv[1] >= kSafeFloor)) == 0ull;
    if (pw < frow::N) st2(&sm.fac[pw][pc0], fv[0], fv[1]);
    if (fl2) {
        atomicOr(&sm.fbm[pw >> 1][ch0 >> 5], fl2 << (ch0 & 31));
        atomicOr(&sm.fbany, 1u);
    }
    const int ek = pow2_exp(__uint_as_float(sm.kmax));
    const float ksc = ldexpf(1.f, -ek);
    if (pw == 0) {
        *reinterpret_cast<float2*>(g2 + G2_GAM + 4 * ch0) = make_float2(gcv[0], gcv[1]);
        if (lane == 0) {
            reinterpret_cast<int*>(g2 + G2_SCAL)[0] = ek;
            reinterpret_cast<unsigned*>(g2 + G2_SCAL)[1] = sm.vmax;
        }
    }
    {
        // per row: a (from the sub-block start), gamma = a * gst (from the
        // chunk start), bs (after the row to the sub-block end), Ktilde * ksc =
        // k bs after ksc; Gram operands Qg, Kg, Kc by the chunk's references
        float bs[PRB][2], tk[2], cm[2], ga[2];
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
            tk[c2] = after[c2] * ksc;
            cm[c2] = slow ? after[c2] * __builtin_amdgcn_rcpf(gcv[c2]) : 1.f;
            ga[c2] = astart[c2];
            bs[PRB - 1][c2] = bstart[c2];
#pragma unroll
            for (int e = PRB - 2; e >= 0; --e) bs[e][c2] = bs[e + 1][c2] * rf.get(e + 1, c2);
        }
        Col8 kt8[2];
        float kprev[2] = {0.f, 0.f};
        E* ikb = reinterpret_cast<E*>(g1 + G1_KB);
        E* iqb = reinterpret_cast<E*>(g1 + G1_QB);
        E* iv = reinterpret_cast<E*>(g1 + G1_V);
#pragma unroll
        for (int e = 0; e < PRB; ++e) {
            float qo[2], ko[2], co[2], qs[2], kss[2];
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) {
                ga[c2] *= rf.get(e, c2);
                const float gm = ga[c2] * gst[c2];   // gamma at this row
                const float kf = rk.get(e, c2), qf = rq.get(e, c2);
                const float kt = kf * (bs[e][c2] * tk[c2]);
                qs[c2] = qf * gm;
                kss[c2] = kf * gm;
                qo[c2] = slow ? qs[c2] : qf * ga[c2];
                ko[c2] = slow ? kss[c2] : kf * ga[c2];
                co[c2] = kf * (bs[e][c2] * cm[c2]);
                if (e & 1) kt8[c2].set_pair_h(e >> 1, kprev[c2], kt);
                else kprev[c2] = kt;
            }
            const uint32_t ro = (uint32_t)(rb + e) * LD + pc0;
            st2(&sm.Qg[ro], qo[0], qo[1]);
            st2(&sm.Kg[ro], ko[0], ko[1]);
            st2(&sm.Kc[ro], co[0], co[1]);
            rv.store(&sm.V[ro], e);
            st2(iqb + ro, qs[0], qs[1]);
            st2(ikb + ro, kss[0], kss[1]);
            rv.store(iv + ro, e);
        }
        _Float16* ikt = reinterpret_cast<_Float16*>(g2 + G2_KT);
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) kt8[c2].store(ikt + (ch0 + c2) * LDT + rb);
    }
    lds_barrier();

    // ---------------------------------------------------- Gram tiles
    // One lower-triangular 16 x 16 tile (I_ >= J_) of M (DO_M) and / or P
    // (DO_P); the factor between the sub-blocks on the Kc fragment (sub-block
    // references only).
    auto gram_tile = [&](auto do_m, auto do_p, int tile) {
        constexpr bool DO_M = decltype(do_m)::value, DO_P = decltype(do_p)::value;
        const int I_ = tile < 1 ? 0 : tile < 3 ? 1 : tile < 6 ? 2 : 3;
        const int J_ = tile - (I_ * (I_ + 1)) / 2;
        const int fr = I_ == J_ ? frow::DIAG + I_
                     : I_ - J_ == 2 ? (J_ == 0 ? frow::D20 : frow::D31)
                     : I_ - J_ == 3 ? frow::D30 : -1;
        floatx4 gk, pp, gv;
        const E* aK = &sm.Kg[(SB * I_ + cl) * LD];
        const E* aQ = &sm.Qg[(SB * I_ + cl) * LD];
        const E* aV = &sm.V[(SB * I_ + cl) * LD];
        const E* bK = &sm.Kc[(SB * J_ + cl) * LD];
        const E* bV = &sm.V[(SB * J_ + cl) * LD];
#pragma unroll
        for (int ks = 0; ks < KD_; ++ks) {
            const floatx4 z = {0.f, 0.f, 0.f, 0.f};
            Frag kk = TR::ld_nat(bK, ks, g);
            if (fr >= 0 && !slow) kk = TR::scale_k(kk, 1.f, sm.fac[fr], ks, g);
            if (DO_M) {
                gk = TR::mma(TR::ld_nat(aK, ks, g), kk, ks ? gk : z);
                gv = TR::mma(TR::ld_nat(aV, ks, g), TR::ld_nat(bV, ks, g), ks ? gv : z);
            }
            if (DO_P) pp = TR::mma(TR::ld_nat(aQ, ks, g), kk, ks ? pp : z);
        }
        const int s_ = SB * J_ + cl;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t_ = SB * I_ + 4 * g + r;
            if (DO_M && s_ < t_) sm.M[t_ * LDA + s_] = sm.beta[t_] * gk[r] * gv[r];
            if (DO_P) sm.P[t_ * LDP + s_] = TR::cvt((s_ <= t_) ? pp[r] : 0.f);
        }
    };
    typedef std::integral_constant<bool, true> kYes;
    typedef std::integral_constant<bool, false> kNo;
    gram_tile(kYes(), kYes(), pw);   // tiles 0 .. 7
    if (pw < 4) {                    // tiles 8, 9 as M and P halves
        if (pw >= 2) gram_tile(kNo(), kYes(), 8 + (pw & 1));
        else gram_tile(kYes(), kNo(), 8 + (pw & 1));
    }
    lds_barrier();
    if (sm.fbany != 0u) {
        // Exact terms of diagonal tile I_ for the channels whose decay over
        // sub-block I_ is below the floor (left out of the tile's product):
        // lane (g, cl) adds, for t = 4g + r and s = cl of the sub-block, the
        // terms k_t k_s E (G_K, s < t) and q_t k_s E (P, s <= t) with
        // E = prod_{s<u<=t} f_u over those channels, from the global rows.
        if ((pw & 1) == 0) {
            const int I_ = pw >> 1;
            const unsigned* fm = sm.fbm[I_];
            unsigned any = 0u;
#pragma unroll
            for (int wd = 0; wd < D / 32; ++wd) any |= fm[wd];
            if (__builtin_amdgcn_readfirstlane(any) != 0u) {
                const int row0 = n * CH + SB * I_;
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
                    if (s_ < t_) sm.M[t_ * LDA + s_] += sm.beta[t_] * dk[r] * gv[r];
                    if (s_ <= t_) {
                        E& pe = sm.P[t_ * LDP + s_];
                        pe = TR::cvt(TR::tof(pe) + dp[r]);
                    }
                }
            }
        }
        lds_barrier();
    }

    // ---------------------------------------------------- P out, A = (I + M)^-1
    {
        const uint4* src = reinterpret_cast<const uint4*>(sm.P);
        uint4* dst = reinterpret_cast<uint4*>(g2 + G2_P);
        for (int x = tid; x < CH * LDP * 2 / 16; x += PNT) dst[x] = src[x];
    }
    float* Ai = reinterpret_cast<float*>(sm.Qg);      // [CH][LDA], the Gram operands are done
    float* Tb = reinterpret_cast<float*>(sm.Kg);      // per wave a 16 x 16 block, [16][16]
    for (int x = tid; x < CH * LDA; x += PNT) Ai[x] = 0.f;
    lds_barrier();
    if (pw == 0) {
        // diagonal blocks, column j of block I per lane: forward substitution
        // of (I + M_II) x = e_j
        const int I_ = lane >> 4, j = lane & 15;
        const float* Mb = &sm.M[(SB * I_) * LDA + SB * I_];
        float x[SB];
#pragma unroll
        for (int i = 0; i < SB; ++i) {
            float acc = i == j ? 1.f : 0.f;
#pragma unroll
            for (int s = 0; s < i; ++s) acc = fmaf(-Mb[i * LDA + s], x[s], acc);
            x[i] = acc;
        }
#pragma unroll
        for (int i = 0; i < SB; ++i) Ai[(SB * I_ + i) * LDA + SB * I_ + j] = x[i];
    }
    lds_barrier();
    // Off-diagonal blocks, one block diagonal at a time: wave w takes block
    // (I, J) = (J + dist, J) with J = w; lane (r = lane / 4, c0 = 4 (lane % 4))
    // makes four entries of row r.
    {
        const int r = lane >> 2, c0 = 4 * (lane & 3);
#pragma unroll 1
        for (int dist = 1; dist < NSB; ++dist) {
            const int J_ = pw, I_ = pw + dist;
            const bool mine = I_ < NSB;
            float tv[4] = {0.f, 0.f, 0.f, 0.f};
            if (mine) {   // T = sum_{J <= K < I} M_IK A_KJ
#pragma unroll 1
                for (int K_ = J_; K_ < I_; ++K_) {
                    const float* mrow = &sm.M[(SB * I_ + r) * LDA + SB * K_];
#pragma unroll
                    for (int s = 0; s < SB; ++s) {
                        const float mv = mrow[s];
                        const floatx4 a4 = *reinterpret_cast<const floatx4*>(&Ai[(SB * K_ + s) * LDA + SB * J_ + c0]);
#pragma unroll
                        for (int e = 0; e < 4; ++e) tv[e] = fmaf(mv, a4[e], tv[e]);
                    }
                }
                *reinterpret_cast<floatx4*>(&Tb[pw * 256 + r * 16 + c0]) = floatx4{tv[0], tv[1], tv[2], tv[3]};
            }
            lds_barrier();
            if (mine) {   // A_IJ = -A_II T
                float av[4] = {0.f, 0.f, 0.f, 0.f};
                const float* arow = &Ai[(SB * I_ + r) * LDA + SB * I_];
#pragma unroll
                for (int s = 0; s < SB; ++s) {
                    const float a = arow[s];
                    const floatx4 t4 = *reinterpret_cast<const floatx4*>(&Tb[pw * 256 + s * 16 + c0]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) av[e] = fmaf(-a, t4[e], av[e]);
                }
                *reinterpret_cast<floatx4*>(&Ai[(SB * I_ + r) * LDA + SB * J_ + c0]) = floatx4{av[0], av[1], av[2], av[3]};
            }
            lds_barrier();
        }
    }
    {
        const uint4* src = reinterpret_cast<const uint4*>(Ai);
        uint4* dst = reinterpret_cast<uint4*>(g2 + G2_A);
        for (int x = tid; x < CH * LDA * 4 / 16; x += PNT) dst[x] = src[x];
    }
}

__global__ __launch_bounds__(f16s::PNT) void kd_fwd16_prep_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ f, const float* __restrict__ beta, const float* __restrict__ cc,
    unsigned char* __restrict__ img, int T, int H)
{
    __shared__ PrepSmem sm;
    prep_unit(sm, q, k, v, f, beta, cc, img, blockIdx.x, blockIdx.y, T, H);
}

struct StateSmem {
    alignas(16) unsigned char g1[f16s::G1_BYTES];
    alignas(16) unsigned char g2[f16s::G2_BYTES];
    alignas(16) __bf16 Os[CH * f16s::LDO];   // o of the previous chunk, natural columns
    alignas(16) float r0p[CH * f16s::NWC];   // r0 partials: [t][consumer wave, rotated by t / 4]
    alignas(16) float bvec[CH];              // c - beta r0 of the chunk
    alignas(16) float u[CH];                 // u * s_prev (readout operand)
    alignas(16) float us[CH];                // u * usc (update operand)
    alignas(16) float gs[f16s::D];           // gamma_C * s / s_prev
    float oinv, sinv;
};

// Hand-off of the preparation images to the state pass when both run in one
// launch (kd_fwd16_split_fused_kernel): flags[bh * NC + n] is published once
// unit (bh, n)'s image is in memory, hdr[bh] carries the XCD of the state
// block of head bh (both words as pub_word; cleared before the launch).
struct SplitPub {
    unsigned long long* flags;   // [B*H*NC]
    unsigned long long* hdr;     // [B*H]
    unsigned epoch;
    unsigned spin;               // polls of a bounded wait before it gives up
};

// The state pass of head bh with the block's LDS sm.  FUSED: the images come
// from preparation units running in the same launch; the loader waves wait
// for each unit's flag before reading its image (a wait that runs out of its
// bound makes that chunk's images, and all later ones, NaN).
template <bool FUSED>
__device__ __forceinline__ void state_pass(
    StateSmem& sm, const unsigned char* __restrict__ img, const float* __restrict__ S0, __bf16* __restrict__ o,
    float* __restrict__ ST, int T, int H, int bh, const SplitPub& pub)
{
    using namespace f16s;
    typedef Bf16T TR;
    typedef __bf16 E;
    typedef TR::Frag Frag;
    typedef TR::FragH FragH;
    constexpr int KD_ = D / TR::KS;
    constexpr int KC_ = CH / TR::KS;
    const int tid = threadIdx.x;
    const int lane = tid & 63, g = lane >> 4, cl = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int b = bh / H, h = bh % H;
    const int NC = (T + CH - 1) / CH;
    const uint32_t rs = (uint32_t)H * D;
    E* ob = o + (size_t)b * T * H * D;
    const uint32_t hoff = (uint32_t)h * D;
    const unsigned char* himg = img + (size_t)bh * NC * UNIT_BYTES;

    const E* Kb = reinterpret_cast<const E*>(sm.g1 + G1_KB);
    const E* Qb = reinterpret_cast<const E*>(sm.g1 + G1_QB);
    const E* Vr = reinterpret_cast<const E*>(sm.g1 + G1_V);
    const _Float16* KtT = reinterpret_cast<const _Float16*>(sm.g2 + G2_KT);
    const E* Pm = reinterpret_cast<const E*>(sm.g2 + G2_P);
    const float* Am = reinterpret_cast<const float*>(sm.g2 + G2_A);
    const float* gam = reinterpret_cast<const float*>(sm.g2 + G2_GAM);
    const float* betaL = reinterpret_cast<const float*>(sm.g2 + G2_BETA);
    const float* cL = reinterpret_cast<const float*>(sm.g2 + G2_C);
    const unsigned* scal = reinterpret_cast<const unsigned*>(sm.g2 + G2_SCAL);

    // chunk nc's o rows from the staging tile to global memory: 16 lanes per
    // row, 16 bytes each
    auto copy_o = [&](int nc, int tid0, int nthr) {
        for (int x = tid - tid0; x < CH * D / 8; x += nthr) {
            const int t = x >> 4, c8 = 8 * (x & 15);
            const int tok = nc * CH + t;
            if (tok < T) cp16_nt(ob + ((uint32_t)tok * rs + hoff + c8), &sm.Os[t * LDO + c8]);
        }
    };

    if (w < NWC) {
        // ---------------------------------------------------- consumers
        // The state is kept multiplied by the power of two s = usc * ksc of
        // the last update, as in the one-launch forward: reads come out scaled
        // by s_prev and are rescaled once (r0 here, o at staging, S_T at the end).
        const int i0 = CPW * w;
        int e_prev = 0;   // s_prev = 2^-e_prev (wave 0)
        floatx4 S[NHV][D / 16];   // S^T[16mj + 4g + r][i0 + 16hv + cl]
#pragma unroll
        for (int hv = 0; hv < NHV; ++hv)
#pragma unroll
            for (int mj = 0; mj < D / 16; ++mj)
                S[hv][mj] = S0 ? *reinterpret_cast<const floatx4*>(
                                     &S0[(size_t)bh * D * D + (size_t)(i0 + 16 * hv + cl) * D + 16 * mj + 4 * g])
                               : floatx4{0.f, 0.f, 0.f, 0.f};
        floatx4 Ot[NHV][NSB];   // O^T[i0 + 16hv + 4g + r][16tt + cl]
        auto stage_o = [&]() {
            const float oi = sm.oinv;
#pragma unroll
            for (int hv = 0; hv < NHV; ++hv)
#pragma unroll
                for (int tt = 0; tt < NSB; ++tt) {
                    const floatx4 y = Ot[hv][tt] * oi;
                    bf16x4 r;
                    r[0] = (__bf16)y[0]; r[1] = (__bf16)y[1]; r[2] = (__bf16)y[2]; r[3] = (__bf16)y[3];
                    *reinterpret_cast<bf16x4*>(&sm.Os[(SB * tt + cl) * LDO + i0 + 16 * hv + 4 * g]) = r;
                }
        };
        lds_barrier();   // the prologue's group 1 of chunk 0
        for (int n = 0; n < NC; ++n) {
            // ============================================== stage A
            KD_PHASE_MARK(n, 0);
            if (n >= 1) stage_o();
            Frag vw[NHV][KC_];   // v of value column i0 + 16hv + cl, tokens 32ks + 8g .. + 7
            float x[NSB];
            {
                Frag a[NHV][KD_];
#pragma unroll
                for (int hv = 0; hv < NHV; ++hv)
#pragma unroll
                    for (int ks = 0; ks < KD_; ++ks) a[hv][ks] = TR::state_frag(S[hv], ks);
                // one wave per SIMD: the operand fragments of sub-block tt + 1
                // are loaded while sub-block tt's MFMAs run (ping-pong)
                Frag fk[2][KD_], fq[2][KD_];
                bf16x4 fv[2][NHV];
                auto ldf = [&](int tt, int p) {
#pragma unroll
                    for (int ks = 0; ks < KD_; ++ks) {
                        fk[p][ks] = TR::ld_state_p(&Kb[(SB * tt + cl) * LD], ks, g);
                        fq[p][ks] = TR::ld_state_p(&Qb[(SB * tt + cl) * LD], ks, g);
                    }
#pragma unroll
                    for (int hv = 0; hv < NHV; ++hv)
                        fv[p][hv] = *reinterpret_cast<const bf16x4*>(
                            &Vr[(SB * tt + cl) * LD + TR::pcol(i0 + 16 * hv + 4 * g)]);
                };
                ldf(0, 0);
#pragma unroll
                for (int tt = 0; tt < NSB; ++tt) {
                    const int p = tt & 1;
                    if (tt + 1 < NSB) ldf(tt + 1, p ^ 1);
                    floatx4 Yt[NHV];
#pragma unroll
                    for (int ks = 0; ks < KD_; ++ks) {
                        const floatx4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int hv = 0; hv < NHV; ++hv) {
                            Yt[hv] = TR::mma(a[hv][ks], fk[p][ks], ks ? Yt[hv] : z);
                            Ot[hv][tt] = TR::mma(a[hv][ks], fq[p][ks], ks ? Ot[hv][tt] : z);
                        }
                    }
                    x[tt] = 0.f;
#pragma unroll
                    for (int hv = 0; hv < NHV; ++hv)
#pragma unroll
                        for (int r = 0; r < 4; ++r) x[tt] += Yt[hv][r] * TR::tof(fv[p][hv][r]);
                }
            }
#pragma unroll
            for (int hv = 0; hv < NHV; ++hv) {
                const E* vcol = &Vr[(uint32_t)(8 * g) * LD + TR::pcol(i0 + 16 * hv + cl)];
#pragma unroll
                for (int ks = 0; ks < KC_; ++ks)
#pragma unroll
                    for (int e = 0; e < 8; ++e) vw[hv][ks][e] = vcol[(TR::KS * ks + e) * LD];
            }
            {
                const float xs = group4_transpose_sum(x, g);
                const int t = SB * g + cl;
                sm.r0p[t * NWC + ((w + (t >> 2)) & (NWC - 1))] = xs;
            }
            KD_PHASE_MARK(n, 3);
            lds_barrier();
            // ============================================== stage B
            KD_PHASE_MARK(n, 1);
            if (w == 0) {   // u = A (c - beta r0), then this chunk's scales
                const int t_ = lane;
                float r0;
                {
                    const floatx4* pr = reinterpret_cast<const floatx4*>(&sm.r0p[t_ * NWC]);
                    floatx4 a = pr[0];
#pragma unroll
                    for (int i = 1; i < NWC / 4; ++i) a = a + pr[i];
                    r0 = ((a[0] + a[1]) + (a[2] + a[3])) * ldexpf(1.f, e_prev);
                }
                // b = c - beta r0 through LDS (this wave's own stores, read back
                // in order), then u_t = sum_s A[t][s] b_s on four partial sums
                sm.bvec[t_] = cL[t_] - betaL[t_] * r0;
                __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the stores are done
                __builtin_amdgcn_wave_barrier();
                float uq[4] = {0.f, 0.f, 0.f, 0.f};
                const float* arow = &Am[t_ * LDA];
#pragma unroll
                for (int s4 = 0; s4 < CH / 4; ++s4) {
                    const floatx4 a4 = *reinterpret_cast<const floatx4*>(&arow[4 * s4]);
                    const floatx4 b4 = *reinterpret_cast<const floatx4*>(&sm.bvec[4 * s4]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) uq[e] = fmaf(a4[e], b4[e], uq[e]);
                }
                const float uu = (uq[0] + uq[1]) + (uq[2] + uq[3]);
                const float um = wave_max_nonneg(fabsf(uu));
                const int eu = pow2_exp(um * __uint_as_float(scal[1]));
                const int e = eu + (int)scal[0];
                sm.u[t_] = uu * ldexpf(1.f, -e_prev);
                sm.us[t_] = uu * ldexpf(1.f, -eu);
                const float rs_ = ldexpf(1.f, e_prev - e);
                const float2 gm = *reinterpret_cast<const float2*>(&gam[2 * t_]);
                *reinterpret_cast<float2*>(&sm.gs[2 * t_]) = make_float2(gm.x * rs_, gm.y * rs_);
                if (lane == 0) {
                    sm.oinv = ldexpf(1.f, e_prev);
                    sm.sinv = ldexpf(1.f, e);
                }
                e_prev = e;
            }
            KD_PHASE_MARK(n, 4);
            lds_barrier();
            // ============================================== stage C
            KD_PHASE_MARK(n, 2);
            {
                // the P fragments and the first K-step's Ktilde^T fragments are
                // loaded before the W arithmetic, which covers their latency
                Frag pf[KC_][NSB];
#pragma unroll
                for (int ks = 0; ks < KC_; ++ks)
#pragma unroll
                    for (int tt = 0; tt < NSB; ++tt) pf[ks][tt] = TR::ld_nat(&Pm[(SB * tt + cl) * LDP], ks, g);
                FragH ak[2][D / 16];
#pragma unroll
                for (int mj = 0; mj < D / 16; ++mj) ak[0][mj] = TR::ld_nat_h(&KtT[(16 * mj + cl) * LDT], 0, g);
                Frag wa[NHV][KC_];
                FragH wb[NHV][KC_];
#pragma unroll
                for (int ks = 0; ks < KC_; ++ks) {
                    const int t0 = TR::KS * ks + 8 * g;
                    const floatx4 a0 = *reinterpret_cast<const floatx4*>(&sm.u[t0]);
                    const floatx4 a1 = *reinterpret_cast<const floatx4*>(&sm.u[t0 + 4]);
                    const floatx4 b0 = *reinterpret_cast<const floatx4*>(&sm.us[t0]);
                    const floatx4 b1 = *reinterpret_cast<const floatx4*>(&sm.us[t0 + 4]);
#pragma unroll
                    for (int hv = 0; hv < NHV; ++hv)
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const float xv = TR::tof(vw[hv][ks][e]);
                            const float ua = e < 4 ? a0[e] : a1[e - 4], ub = e < 4 ? b0[e] : b1[e - 4];
                            wa[hv][ks][e] = TR::cvt(ua * xv);
                            wb[hv][ks][e] = (_Float16)(ub * xv);
                        }
                }
                // O^T += W^T P^T
#pragma unroll
                for (int ks = 0; ks < KC_; ++ks)
#pragma unroll
                    for (int hv = 0; hv < NHV; ++hv)
#pragma unroll
                        for (int tt = 0; tt < NSB; ++tt) Ot[hv][tt] = TR::mma(wa[hv][ks], pf[ks][tt], Ot[hv][tt]);
                // S <- S diag(gamma_C) s / s_prev + Ktilde'^T W'
#pragma unroll
                for (int mj = 0; mj < D / 16; ++mj) {
                    const floatx4 gsv = *reinterpret_cast<const floatx4*>(&sm.gs[16 * mj + 4 * g]);
#pragma unroll
                    for (int hv = 0; hv < NHV; ++hv) S[hv][mj] = S[hv][mj] * gsv;
                }
#pragma unroll
                for (int ks = 0; ks < KC_; ++ks) {
                    if (ks + 1 < KC_)   // the next K-step's fragments under this one's MFMAs
#pragma unroll
                        for (int mj = 0; mj < D / 16; ++mj)
                            ak[(ks + 1) & 1][mj] = TR::ld_nat_h(&KtT[(16 * mj + cl) * LDT], ks + 1, g);
#pragma unroll
                    for (int mj = 0; mj < D / 16; ++mj)
#pragma unroll
                        for (int hv = 0; hv < NHV; ++hv) S[hv][mj] = TR::mma_h(ak[ks & 1][mj], wb[hv][ks], S[hv][mj]);
                }
            }
            KD_PHASE_MARK(n, 5);
            lds_barrier();
        }
        stage_o();
        lds_barrier();   // the loaders write the last chunk's rows
        if (ST) {
            const float si = sm.sinv;
#pragma unroll
            for (int hv = 0; hv < NHV; ++hv)
#pragma unroll
                for (int mj = 0; mj < D / 16; ++mj)
                    st4_nt(&ST[(size_t)bh * D * D + (size_t)(i0 + 16 * hv + cl) * D + 16 * mj + 4 * g],
                           S[hv][mj] * si);
        }
    } else {
        // ---------------------------------------------------- loaders
        // 16-byte piece li + 256 s of a group's image in register slot s
        // (straight-line copies at each use, so the slots stay registers)
        const int li = tid - NWC * 64;
        constexpr int G1N = G1_BYTES / 16, G2N = G2_BYTES / 16, LS = NWL * 64;
        typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
        u32x4 r1[G1_SLOTS], r2[G2_SLOTS];
        u32x4* d1 = reinterpret_cast<u32x4*>(sm.g1);
        u32x4* d2 = reinterpret_cast<u32x4*>(sm.g2);
        // FUSED: chunk nc's flag before its first read (group 1 of a chunk is
        // always loaded before its group 2); dead: a wait ran out
        bool dead = false;
        const unsigned me = FUSED ? xcc_id() : 0u;
        auto wait_unit = [&](int nc) {
            if (!FUSED || dead) return;
            unsigned long long wd = 0;
            bool ok = pub_wait(&pub.flags[(size_t)bh * NC + nc], pub.epoch, 1ull, wd, pub.spin);
            // a writer on another XCD wrote its L2 back before publishing: drop
            // this XCD's copies before reading
            if (ok && ((unsigned)(wd >> 24) & 0xffu) != me) {
                ok = (wd & PUB_FLUSHED) != 0ull;
                if (ok) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            }
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");   // no image read moves above the wait
            dead = !ok;
        };
#define KD_LOAD1(nc)                                                                              \
    {                                                                                             \
        wait_unit(nc);                                                                            \
        const u32x4* src_ = reinterpret_cast<const u32x4*>(himg + (size_t)(nc) * UNIT_BYTES);     \
        if (FUSED && dead) {                                                                      \
            _Pragma("unroll") for (int s = 0; s < G1_SLOTS; ++s) r1[s] = u32x4{0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u}; \
        } else {                                                                                  \
            _Pragma("unroll") for (int s = 0; s < G1_SLOTS; ++s) if (li + LS * s < G1N) r1[s] = src_[li + LS * s]; \
        }                                                                                         \
    }
#define KD_LOAD2(nc)                                                                              \
    {                                                                                             \
        const u32x4* src_ = reinterpret_cast<const u32x4*>(himg + (size_t)(nc) * UNIT_BYTES + G1_BYTES); \
        if (FUSED && dead) {                                                                      \
            _Pragma("unroll") for (int s = 0; s < G2_SLOTS; ++s) r2[s] = u32x4{0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u, 0x7fc07fc0u}; \
        } else {                                                                                  \
            _Pragma("unroll") for (int s = 0; s < G2_SLOTS; ++s) if (li + LS * s < G2N) r2[s] = src_[li + LS * s]; \
        }                                                                                         \
    }
#define KD_PUT1() _Pragma("unroll") for (int s = 0; s < G1_SLOTS; ++s) if (li + LS * s < G1N) d1[li + LS * s] = r1[s];
#define KD_PUT2() _Pragma("unroll") for (int s = 0; s < G2_SLOTS; ++s) if (li + LS * s < G2N) d2[li + LS * s] = r2[s];
        KD_LOAD1(0)
        KD_PUT1()
        KD_LOAD2(0)
        if (NC > 1) KD_LOAD1(1)
        lds_barrier();
        for (int n = 0; n < NC; ++n) {
            // stage A: group 2 of chunk n (its previous readers ran in stage C
            // of chunk n - 1), then the loads of chunk n + 1's
            KD_PHASE_MARK(n, 0);
            KD_PUT2()
            if (n + 1 < NC) KD_LOAD2(n + 1)
            KD_PHASE_MARK(n, 3);
            lds_barrier();
            // stage B: chunk n - 1's o rows
            KD_PHASE_MARK(n, 1);
            if (n >= 1) copy_o(n - 1, NWC * 64, NWL * 64);
            KD_PHASE_MARK(n, 4);
            lds_barrier();
            // stage C: group 1 of chunk n + 1 (its previous readers ran in
            // stage A), then the loads of chunk n + 2's
            KD_PHASE_MARK(n, 2);
            if (n + 1 < NC) {
                KD_PUT1()
                if (n + 2 < NC) KD_LOAD1(n + 2)
            }
            KD_PHASE_MARK(n, 5);
            lds_barrier();
        }
#undef KD_LOAD1
#undef KD_LOAD2
#undef KD_PUT1
#undef KD_PUT2
        lds_barrier();   // the consumers stage the last chunk's o
        copy_o(NC - 1, NWC * 64, NWL * 64);
    }
}

__global__ __launch_bounds__(f16s::SNT) void kd_fwd16_state_kernel(
    const unsigned char* __restrict__ img, const float* __restrict__ S0, __bf16* __restrict__ o,
    float* __restrict__ ST, int T, int H)
{
    __shared__ StateSmem sm;
    state_pass<false>(sm, img, S0, o, ST, T, H, blockIdx.x, SplitPub{});
}

static_assert(f16s::PNT == f16s::SNT, "the fused launch runs both roles with one block size");

// Both launches of the few-heads forward in one, so the state passes start as
// soon as their first chunk is prepared instead of after every chunk is.
// Blocks 0 .. BHpad - 1 run the state passes (one per (b, h); blocks past B*H
// have no head and leave).  The others are persistent workers that prepare
// units: under round-robin placement blocks x and x + 8 share an XCD, so the
// workers with x = c (mod 8) take the units of the heads bh = c (mod 8), in
// chunk order, r, r + R, ... for the r-th of the R workers of XCD c, and the
// state block of head bh reads them through the XCD's L2.  Dispatch is in
// block order, so every state block is resident before any worker, and the
// workers never wait: the state blocks' waits end.  A worker that finds the
// state block of a unit's head on another XCD (or not yet known) writes its
// L2 back to memory before publishing (PUB_FLUSHED).
__global__ __launch_bounds__(f16s::SNT) void kd_fwd16_split_fused_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ f, const float* __restrict__ beta, const float* __restrict__ cc,
    unsigned char* __restrict__ img, const float* __restrict__ S0, __bf16* __restrict__ o,
    float* __restrict__ ST, SplitPub pub, int BH, int BHpad, int nwork, int T, int H)
{
    union Smem {
        PrepSmem p;
        StateSmem s;
    };
    __shared__ Smem sm;
    const int x = blockIdx.x;
    if (x < BHpad) {
        if (x < BH) {
            if (threadIdx.x == 0)
                __hip_atomic_store(&pub.hdr[x], pub_word(pub.epoch, xcc_id()), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            state_pass<true>(sm.s, img, S0, o, ST, T, H, x, pub);
        }
        return;
    }
    const int NC = (T + CH - 1) / CH;
    const int c = x & 7, r = (x - BHpad) >> 3, R = nwork >> 3;
    const int nh = c < BH ? (BH - c + 7) / 8 : 0;   // heads c, c + 8, ... on this XCD
    const int total = nh * NC;
    const unsigned me = xcc_id();
#pragma unroll 1
    for (int u = r; u < total; u += R) {
        const int n = u / nh, bh = c + 8 * (u % nh);
        prep_unit(sm.p, q, k, v, f, beta, cc, img, n, bh, T, H);
        // every thread's image stores have reached L2; the flag goes out after
        // the barrier (which also frees the LDS for the next unit)
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        lds_barrier();
        if (threadIdx.x == 0) {
            const unsigned long long hw =
                __hip_atomic_load(&pub.hdr[bh], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            unsigned long long extra = 0ull;
            if ((unsigned)(hw >> 32) != pub.epoch || ((unsigned)(hw >> 24) & 0xffu) != me) {
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
                extra = PUB_FLUSHED;
            }
            __hip_atomic_store(&pub.flags[(size_t)bh * NC + n], pub_word(pub.epoch, me) | extra, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// Zeroes the hand-off words of a fused launch (a kernel rather than a memset,
// so that a captured graph replays it correctly).
__global__ void kd_fwd16_split_clear_kernel(unsigned long long* __restrict__ w, int n)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) w[i] = 0ull;
}

int compute_units();
unsigned bwd_wait_polls();

// preparation workers of the fused launch (at most one per compute unit the
// state passes leave free)
#ifndef KD_FWD16S_MAXWORK
#define KD_FWD16S_MAXWORK 1024
#endif

// launch epochs of the fused few-heads forward (see SplitPub)
static unsigned next_split_epoch() {
    static std::atomic<unsigned> e{0u};
    unsigned v = e.fetch_add(1u) + 1u;
    if (v == 1u) {   // first launch of the process: start from the clock
        const unsigned t = (unsigned)time(nullptr) * 2246822519u;
        e.fetch_add(t);
        v += t;
    }
    return v;
}

hipError_t launch_fwd16_split(const void* q, const void* k, const void* v, const void* f, const float* beta,
                              const float* c, const float* S0, void* o, float* ST, void* ws, int B, int T,
                              int H, hipStream_t st)
{
    typedef __bf16 E;
    const int NC = (T + CH - 1) / CH;
    const int BH = B * H, BHpad = (BH + 7) & ~7;
    // about four workers per head keep ahead of the state passes; more only
    // crowd the memory system the state passes read from
    const int nwork = min(min(((compute_units() - BHpad) / 8) * 8, KD_FWD16S_MAXWORK),
                          max(64, ((4 * BH + 7) / 8) * 8));
    if (NC > 0 && nwork >= 64) {   // one launch: the state passes beside the preparation workers
        unsigned char* wb = static_cast<unsigned char*>(ws);
        SplitPub pub;
        pub.hdr = reinterpret_cast<unsigned long long*>(wb + (size_t)BH * NC * f16s::UNIT_BYTES);
        pub.flags = pub.hdr + BH;
        pub.epoch = next_split_epoch();
        pub.spin = bwd_wait_polls();
        const int nw = BH + BH * NC;
        hipLaunchKernelGGL(kd_fwd16_split_clear_kernel, dim3((unsigned)((nw + 255) / 256)), dim3(256), 0, st,
                           pub.hdr, nw);
        hipLaunchKernelGGL(kd_fwd16_split_fused_kernel, dim3((unsigned)(BHpad + nwork)), dim3(f16s::SNT), 0, st,
                           (const E*)q, (const E*)k, (const E*)v, (const E*)f, beta, c, wb, S0, (E*)o, ST, pub,
                           BH, BHpad, nwork, T, H);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(kd_fwd16_prep_kernel, dim3((unsigned)NC, (unsigned)(B * H)), dim3(f16s::PNT), 0, st,
                       (const E*)q, (const E*)k, (const E*)v, (const E*)f, beta, c,
                       static_cast<unsigned char*>(ws), T, H);
    hipLaunchKernelGGL(kd_fwd16_state_kernel, dim3((unsigned)(B * H)), dim3(f16s::SNT), 0, st,
                       static_cast<const unsigned char*>(ws), S0, (E*)o, ST, T, H);
    return hipGetLastError();
}

}  // namespace kd
