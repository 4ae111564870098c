// kd_bwd.hip -- gate-aware chunkwise backward of the Kronecker delta rule, gfx950.
//
// Reverse mode of the chunked forward (the forward kernel's header gives the
// chunk algebra; the pages are the onedev.kr KronLSTM summary, sections
// "어떻게 동작하나" and "어떻게 쓰나", and the aitrends.kr Gated DeltaNet-2
// summary, sections "방법론" steps 3-4 and "핵심 기여", which names a
// gate-aware backward through the WY form).  Per chunk, with dS the gradient
// of the state leaving the chunk and drho = (I + M)^{-T} du:
//   du   = rowsum((P^T dO + Kt dS^T) * V)            (Kt = K gamma_C / gamma)
//   dS0  = dS diag(gamma_C) + dO^T Qbar + V^T diag(dr0) Kbar,  dr0 = -beta * drho
//   dM   = -drho u^T (strictly lower), dGK = beta dM * GV, dGV = beta dM * GK
//   dV   = diag(u) (P^T dO + Kt dS^T) + (dGV + dGV^T) V + diag(dr0) Kbar S0^T
//   dKbar = dGK Kc + diag(dr0) V S0,   dKc = dGK^T Kbar + dP^T Qbar,
//   dQbar = dO S0 + dP Kc,   dKt = W dS,   dP = tril_0(dO W^T),  W = u * V
//   dbeta = -r0 drho + rowsum(dM * GK * GV),   dc = drho
// and the decay enters through g = d/d(log gamma):
//   g_t = dQbar Qbar + dKbar Kbar - dKc Kc - dKt Kt,
//   g_C = gamma_C colsum(dS * S0) + sum_t dKt Kt,
//   d log f_s = sum_{t >= s} g_t + g_C,   df = d log f / f.
//
// Three launches on the caller's stream:
//   1. the forward kernel with checkpoints: per chunk the entering state (in
//      the input dtype, S[i][j]), u, r0, and the chunk's M and P;
//   2. kd_bwd_state_kernel: one workgroup per (b, h), chunks in reverse, the
//      fp32 dS^T held as MFMA accumulators (the mirror of the forward state):
//      state read, back substitution, rank-128 update; stores dS and drho.
//      M and P come from the forward, and each chunk's inputs are loaded
//      while the previous chunk is processed;
//   3. kd_bwd_chunk_kernel: one workgroup per (b, h, chunk), all chunks in
//      parallel: every local gradient.
// A chunk with a key channel whose decay over the chunk falls below 2^-100
// (the forward's exact-fallback case, which includes f = 0) is not handled
// here: all its gradients are NaN, and so is every gradient that depends on
// it through the state gradient (dk, dv, df, dbeta, dc of the earlier chunks
// of that (b, h), and dS0); dq of the earlier chunks does not and stays exact.
#include <type_traits>

#include <time.h>

#include <atomic>

#include "kd_device.h"

namespace kd {

hipError_t launch_fwd(int bf16, int d, const void* q, const void* k, const void* v, const void* f,
                      const float* beta, const float* c, const float* S0, void* o, float* ST,
                      const FwdCkpt* ck, const int* cu, int B, int T, int H, hipStream_t st);

// Workspace: [S0 | u, r0 | dS | drho | M | P] per (b, h, chunk) unit,
// 256-byte aligned parts (per unit: d*d*e, 2*CH*4, d*d*e, CH*4, CH*CH*4,
// CH*CH*e bytes).
struct BwdWs {
    size_t s0, ur, ds, rho, mm, pp, fl, total;   // fl: 8 claim counters, then one flag per (b, h, chunk) at +256
};

// Hand-off of the reverse sweep's per-chunk results (dS, rho) to the chunk
// workers of the fused launch (kd_bwd_fused_kernel).  A flag word carries the
// launch's epoch (flags of earlier launches never match), the writer's XCD id
// and bit 1 = PUB_FLUSHED: set only on chunk 0's flag, which goes out after
// the sweep has written its XCD's L2 back to memory, so a reader on another
// XCD can wait for that flag and read everything the sweep wrote.
// The chunks of the heads on one XCD are handed out in the sweep's order by
// a claim counter per XCD (ctr[c]: epoch in the high word, units claimed in
// the low word), which the launch's block c sets at its start.
struct BwdPub {
    unsigned long long* flags;   // [B*H*NC]
    unsigned long long* ctr;     // [8]
    unsigned epoch;
};
constexpr unsigned long long PUB_FLUSHED = 2ull;

__device__ __forceinline__ unsigned xcc_id() {
    return __builtin_amdgcn_s_getreg(20 | (0 << 6) | (3 << 11));   // HW_REG_XCC_ID[3:0]
}
__device__ __forceinline__ unsigned long long pub_word(unsigned epoch, unsigned xcc) {
    return ((unsigned long long)epoch << 32) | ((unsigned long long)(xcc & 0xffu) << 24) | 1ull;
}
// bounded wait of one thread for a flag of this launch that has the bits
// `need`; false when the bound ran out (then nothing may be read)
__device__ __forceinline__ bool pub_wait(const unsigned long long* fp, unsigned epoch, unsigned long long need,
                                         unsigned long long& w) {
    for (int s = 0; s < (1 << 23); ++s) {
        w = __hip_atomic_load(fp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((unsigned)(w >> 32) == epoch && (w & need) == need) return true;
        __builtin_amdgcn_s_sleep(2);
    }
    return false;
}
static BwdWs bwd_ws_layout(size_t esz, int d, int B, int T, int H) {
    const size_t nc = (size_t)(T + CH - 1) / CH;
    const size_t units = (size_t)B * H * nc;
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    BwdWs w;
    w.s0 = 0;
    w.ur = up(units * d * d * esz);
    w.ds = w.ur + up(units * 2 * CH * sizeof(float));
    w.rho = w.ds + up(units * d * d * esz);
    w.mm = w.rho + up(units * CH * sizeof(float));
    w.pp = w.mm + up(units * CH * CH * sizeof(float));
    w.fl = w.pp + up(units * CH * CH * esz);
    w.total = w.fl + up(256 + units * sizeof(unsigned long long));
    return w;
}

size_t bwd_workspace_bytes(int bf16, int d, int B, int T, int H) {
    return bwd_ws_layout(bf16 ? 2 : 4, d, B, T, H).total;
}

// Common prep of both backward kernels: thread owns rows row0, row0 + 1 of the
// chunk and channels ch0 .. ch0 + 7 (the eight row pairs of a 16-row
// sub-block sit in one aligned 8-lane group).
struct PrepIdx {
    int r8, I, ch0, row0;
    __device__ PrepIdx(int tid, int D) {
        const int lane = tid & 63, w = tid >> 6;
        r8 = lane & 7;
        const int qd = w * 8 + (lane >> 3);
        I = qd / (D / 8);
        ch0 = 8 * (qd % (D / 8));
        row0 = SB * I + 2 * r8;
    }
};

// ======================================================================
// Serial dS recurrence
// ======================================================================
template <class TR, int D>
struct BwdStateSmem {
    typedef typename TR::E E;
    static constexpr int LD = D + TR::PAD;     // [CH][D] row-major operands
    static constexpr int LDT = CH + TR::PAD;   // [D][CH] transposed operands
    static constexpr int LDM = CH + 4;         // fp32 M
    static constexpr int LDP = CH + TR::PAD;
    static constexpr int NW = D / 16;
    alignas(16) E Kt[CH * LD];                        // K-tilde rows
    alignas(16) E V[CH * LD];
    alignas(16) E VT[D * LDT];                        // v^T
    alignas(16) E OT[D * LDT];                        // dO^T
    alignas(16) E QT[D * LDT];                        // (q gamma)^T
    alignas(16) E KT[D * LDT];                        // (k gamma)^T
    alignas(16) E PT[CH * LDP];                       // PT[s][t] = P[t][s]
    alignas(16) float M[CH * LDM];                    // M of the chunk (strictly lower)
    alignas(16) float beta[CH];
    alignas(16) float dr0[CH];
    alignas(16) float dup[NW][CH];                    // partial du per wave
    alignas(16) float bprod[NSB][D];
    alignas(16) float gam[D];
    unsigned unsafe_any;
};

// One chunk's inputs as held in registers between its prefetch and its prep:
// two rows x eight channels of q, k, v, f, dO per thread, beta of one token,
// and a slice of the chunk's M and P from the forward.
template <class TR, int D>
struct BwdStateRegs {
    typedef typename TR::E E;
    static constexpr int MV = CH * CH / (4 * 4 * D);             // float4 of M per thread
    static constexpr int PV = CH * CH * sizeof(E) / (16 * 4 * D);  // 16-byte slices of P per thread
    Row2x8<TR> q, k, v, f, o;
    float beta;
    floatx4 m[MV];
    uint4 p[PV];
};

// Publishing arguments of the fused launch, in LDS: only the publishing
// thread reads them, when it publishes, so they hold no register across the
// sweep's loop.
__shared__ BwdPub g_pub;

// The sweep of one (b, h); with PUB, each chunk's dS and rho are published
// (flags of g_pub) once every wave's stores of them have reached L2.
template <class TR, int D, bool PUB>
__device__ __forceinline__ void bwd_state_body(
    BwdStateSmem<TR, D>& sm, int bh,
    const typename TR::E* __restrict__ q, const typename TR::E* __restrict__ k,
    const typename TR::E* __restrict__ v, const typename TR::E* __restrict__ f,
    const float* __restrict__ beta, const typename TR::E* __restrict__ dO,
    const float* __restrict__ ckM, const typename TR::E* __restrict__ ckP,
    const float* __restrict__ dST, typename TR::E* __restrict__ wsdS, float* __restrict__ wsrho,
    float* __restrict__ dS0, int T, int H)
{
    typedef typename TR::E E;
    typedef typename TR::Frag Frag;
    typedef BwdStateSmem<TR, D> SM;
    typedef BwdStateRegs<TR, D> RG;
    constexpr int NT = 4 * D;
    constexpr int NW = SM::NW;
    constexpr int KD_ = D / TR::KS;
    constexpr int KC_ = CH / TR::KS;
    constexpr int LD = SM::LD, LDT = SM::LDT, LDM = SM::LDM, LDP = SM::LDP;
    constexpr int EPV = 16 / sizeof(E);   // P elements per 16-byte slice


    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6, g = lane >> 4, cl = lane & 15;
    const PrepIdx pi(tid, D);
    const int r8 = pi.r8, I = pi.I, ch0 = pi.ch0, row0 = pi.row0;
    const int b = bh / H, h = bh % H;
    const uint32_t rs = (uint32_t)H * D;
    const size_t bbase = (size_t)b * T * H * D;
    const uint32_t hoff = (uint32_t)h * D;
    const int NC = (T + CH - 1) / CH;
    auto publish = [&](int n, unsigned long long extra) {   // chunk n's dS and rho are in L2 (see the loop's end)
        __hip_atomic_store(&g_pub.flags[(size_t)bh * NC + n], pub_word(g_pub.epoch, xcc_id()) | extra,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };

    floatx4 dSt[D / 16];   // dS^T[16mj + 4g + r][16w + cl] = dS[16w + cl][16mj + 4g + r]
#pragma unroll
    for (int mj = 0; mj < D / 16; ++mj)   // four adjacent columns: one 16-byte load
        dSt[mj] = dST ? *reinterpret_cast<const floatx4*>(&dST[(size_t)bh * D * D + (size_t)(16 * w + cl) * D + 16 * mj + 4 * g])
                      : floatx4{0.f, 0.f, 0.f, 0.f};

    // Loads of chunk n into registers; unconditional (n is clamped by the
    // caller, rows past the end re-read the last row and are cleared in the
    // prep), so the next chunk's loads stay in flight across the current one.
    // The loads of the next chunk are issued in three parts over the stages
    // that follow the prep, so no wave issues the whole chunk at once.
    RG cur;
    auto row_offs = [&](int n, uint32_t& oa, uint32_t& ob) {
        const int ta = min(n * CH + row0, T - 1), tb = min(n * CH + row0 + 1, T - 1);
        oa = (uint32_t)ta * rs + hoff + ch0;
        ob = (uint32_t)tb * rs + hoff + ch0;
    };
    auto load_part1 = [&](int n) {
        uint32_t oa, ob;
        row_offs(n, oa, ob);
        cur.q.load(q + bbase, oa, ob);
        cur.k.load(k + bbase, oa, ob);
        cur.f.load(f + bbase, oa, ob);
    };
    auto load_part2 = [&](int n) {
        uint32_t oa, ob;
        row_offs(n, oa, ob);
        cur.v.load(v + bbase, oa, ob);
        cur.o.load(dO + bbase, oa, ob);
    };
    auto load_part3 = [&](int n) {
        cur.beta = beta[((size_t)b * T + min(n * CH + (tid & (CH - 1)), T - 1)) * H + h];
        const float* mg = ckM + ((size_t)bh * NC + n) * CH * CH;
        const E* pg = ckP + ((size_t)bh * NC + n) * CH * CH;
#pragma unroll
        for (int i = 0; i < RG::MV; ++i) cur.m[i] = reinterpret_cast<const floatx4*>(mg)[tid + NT * i];
#pragma unroll
        for (int i = 0; i < RG::PV; ++i) cur.p[i] = reinterpret_cast<const uint4*>(pg)[tid + NT * i];
    };
    if (NC > 0) {
        if (tid == 0) sm.unsafe_any = 0u;
        load_part1(NC - 1);
        load_part2(NC - 1);
        load_part3(NC - 1);
    }

    // gradient of the state leaving chunk n, dS[i][j], for the chunk-local kernel
    auto store_dS = [&](int n) {
        E* dst = wsdS + ((size_t)bh * NC + n) * D * D;
#pragma unroll
        for (int mj = 0; mj < D / 16; ++mj)
            st4(dst + ((uint32_t)(16 * w + cl) * D + 16 * mj + 4 * g), dSt[mj]);
    };

    for (int n = NC - 1; n >= 0; --n) {
        if (PUB && tid == 0 && n + 1 < NC) publish(n + 1, 0ull);
        // ---------------- prep (a): decay products within the sub-block; M and P
        if (n * CH + CH > T) {   // ragged last chunk: rows past the end are inert
#pragma unroll
            for (int e = 0; e < 2; ++e)
                if (n * CH + row0 + e >= T) {
                    cur.q.clear(e, 0.f); cur.k.clear(e, 0.f); cur.v.clear(e, 0.f); cur.f.clear(e, 1.f);
                    cur.o.clear(e, 0.f);
                }
            if (n * CH + (tid & (CH - 1)) >= T) cur.beta = 0.f;
        }
        float incl[8], excl[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            incl[c] = group8_prefix_prod(cur.f.get(0, c) * cur.f.get(1, c), r8);
            excl[c] = group8_shift1(incl[c], r8);
        }
        if (r8 == 7) st8v(&sm.bprod[I][ch0], incl);
        if (tid < CH) sm.beta[tid] = cur.beta;
#pragma unroll
        for (int i = 0; i < RG::MV; ++i) {
            const int x = tid + NT * i, t = x / (CH / 4), s4 = x % (CH / 4);
            *reinterpret_cast<floatx4*>(&sm.M[t * LDM + 4 * s4]) = cur.m[i];
        }
#pragma unroll
        for (int i = 0; i < RG::PV; ++i) {   // transposed: PT[s][t] = P[t][s]
            const int x = tid + NT * i, t = x / (CH / EPV), s0 = EPV * (x % (CH / EPV));
            const E* pe = reinterpret_cast<const E*>(&cur.p[i]);
#pragma unroll
            for (int e = 0; e < EPV; ++e) sm.PT[(s0 + e) * LDP + t] = pe[e];
        }
        lds_barrier();

        // ---------------- prep (b): operands
        {
            float plt[8], gC[8];
#pragma unroll
            for (int c = 0; c < 8; ++c) { plt[c] = 1.f; gC[c] = 1.f; }
#pragma unroll
            for (int I2 = 0; I2 < NSB; ++I2)
#pragma unroll
                for (int c4 = 0; c4 < 2; ++c4) {
                    const floatx4 x = *reinterpret_cast<const floatx4*>(&sm.bprod[I2][ch0 + 4 * c4]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        gC[4 * c4 + e] *= x[e];
                        if (I2 < I) plt[4 * c4 + e] *= x[e];
                    }
                }
            unsigned unsafe = 0;
#pragma unroll
            for (int c = 0; c < 8; ++c)
                if (!(gC[c] >= kSafeFloor)) unsafe |= 1u << c;
            if (I == 0 && r8 == 0) st8v(&sm.gam[ch0], gC);
            if (unsafe) atomicOr(&sm.unsafe_any, 1u);
            float qo[2][8], ko[2][8];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                float kt[8];
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    const float ga = plt[c] * (e == 0 ? excl[c] * cur.f.get(0, c) : incl[c]);
                    const float kf = cur.k.get(e, c);
                    const bool un = (unsafe >> c) & 1u;
                    qo[e][c] = cur.q.get(e, c) * ga;
                    ko[e][c] = kf * ga;
                    kt[c] = un ? 0.f : kf * __builtin_amdgcn_rcpf(ga) * gC[c];   // K-tilde
                }
                st8v(&sm.Kt[(row0 + e) * LD + ch0], kt);
                cur.v.store(&sm.V[(row0 + e) * LD + ch0], e);
            }
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                st2(&sm.VT[(ch0 + c) * LDT + row0], cur.v.get(0, c), cur.v.get(1, c));
                st2(&sm.OT[(ch0 + c) * LDT + row0], cur.o.get(0, c), cur.o.get(1, c));
                st2(&sm.QT[(ch0 + c) * LDT + row0], qo[0][c], qo[1][c]);
                st2(&sm.KT[(ch0 + c) * LDT + row0], ko[0][c], ko[1][c]);
            }
        }
        const int npf = max(n - 1, 0);   // the next chunk's loads run under this one
        load_part1(npf);
        lds_barrier();

        // ---------------- state read: dW = Kt dS^T + P^T dO (rows t, this wave's 16 columns i)
        floatx4 dW[NSB];
        {
            Frag ac[NSB];
#pragma unroll
            for (int tt = 0; tt < NSB; ++tt) ac[tt] = TR::ld_state(&sm.Kt[(SB * tt + cl) * LD], 0, g);
#pragma unroll
            for (int ks = 0; ks < KD_; ++ks) {
                Frag an[NSB];
                if (ks + 1 < KD_) {
#pragma unroll
                    for (int tt = 0; tt < NSB; ++tt) an[tt] = TR::ld_state(&sm.Kt[(SB * tt + cl) * LD], ks + 1, g);
                }
                const Frag bS = TR::state_frag(dSt, ks);
                const floatx4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int tt = 0; tt < NSB; ++tt) dW[tt] = TR::mma(ac[tt], bS, ks ? dW[tt] : z);
                if (ks + 1 < KD_) {
#pragma unroll
                    for (int tt = 0; tt < NSB; ++tt) ac[tt] = an[tt];
                }
            }
        }
#pragma unroll
        for (int ks = 0; ks < KC_; ++ks) {
            const Frag bO = TR::ld_nat(&sm.OT[(16 * w + cl) * LDT], ks, g);
            Frag ap[NSB];
#pragma unroll
            for (int tt = 0; tt < NSB; ++tt) ap[tt] = TR::ld_nat(&sm.PT[(SB * tt + cl) * LDP], ks, g);
#pragma unroll
            for (int tt = 0; tt < NSB; ++tt) dW[tt] = TR::mma(ap[tt], bO, dW[tt]);
        }
        load_part2(npf);
        {   // partial du[t] over this wave's 16 value columns: transpose-reduce
            // over the 16 lanes of a row with DPP partners (row mirror, half-row
            // mirror, quad swaps), after which lane cl holds element cl
            float x[16];
#pragma unroll
            for (int tt = 0; tt < NSB; ++tt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    x[4 * tt + r] = dW[tt][r] * TR::tof(sm.V[(SB * tt + 4 * g + r) * LD + 16 * w + cl]);
            row16_reduce_step<8>(x, cl);
            row16_reduce_step<4>(x, cl);
            row16_reduce_step<2>(x, cl);
            row16_reduce_step<1>(x, cl);
            sm.dup[w][SB * (cl >> 2) + 4 * g + (cl & 3)] = x[0];
        }
        lds_barrier();

        // ---------------- back substitution (I + M)^T drho = du; every wave
        // then stores dS and issues the rest of the next chunk's loads (the
        // others while wave 0 solves)
        if (w == 0) {
            const int t_ = lane;
            float x = 0.f;
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) x += sm.dup[ww][t_];
            float Mcol[CH];
#pragma unroll
            for (int s = 0; s < CH; ++s) Mcol[s] = sm.M[s * LDM + t_];
            // lane t takes the finished drho_s of every later row s; the mask
            // keeps a non-finite drho_s of an earlier row out of lane t
#pragma unroll
            for (int s = CH - 1; s >= 1; --s) {
                const float y = fmaf(-Mcol[s], readlane_f(x, s), x);
                x = (t_ < s) ? y : x;
            }
            if (sm.unsafe_any) x = __builtin_nanf("");
            wsrho[((size_t)bh * NC + n) * CH + t_] = x;
            sm.dr0[t_] = -sm.beta[t_] * x;
        }
        store_dS(n);
        load_part3(npf);
        lds_barrier();

        // ---------------- dS <- dS diag(gamma_C) + dO^T Qbar + V^T diag(dr0) Kbar
        if (tid == 0) sm.unsafe_any = 0u;   // read for the last time above
        {
            Frag bO[KC_], bR[KC_];
#pragma unroll
            for (int ks = 0; ks < KC_; ++ks) {
                bO[ks] = TR::ld_nat(&sm.OT[(16 * w + cl) * LDT], ks, g);
                bR[ks] = TR::row_times(&sm.VT[(16 * w + cl) * LDT], sm.dr0, ks, g);
            }
#pragma unroll
            for (int mj = 0; mj < D / 16; ++mj)
                dSt[mj] = dSt[mj] * *reinterpret_cast<const floatx4*>(&sm.gam[16 * mj + 4 * g]);
#pragma unroll
            for (int ks = 0; ks < KC_; ++ks)
#pragma unroll
                for (int mj = 0; mj < D / 16; ++mj) {
                    dSt[mj] = TR::mma(TR::ld_nat(&sm.QT[(16 * mj + cl) * LDT], ks, g), bO[ks], dSt[mj]);
                    dSt[mj] = TR::mma(TR::ld_nat(&sm.KT[(16 * mj + cl) * LDT], ks, g), bR[ks], dSt[mj]);
                }
        }
        // this wave's stores of chunk n (and everything before them) have
        // reached L2 before the barrier; the flag goes out after it
        if (PUB) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        lds_barrier();
    }
    if (PUB && tid == 0 && NC > 0) {   // every wave's stores are in L2: write it back, then the last flag
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        publish(0, PUB_FLUSHED);
    }

    if (dS0) {
#pragma unroll
        for (int mj = 0; mj < D / 16; ++mj)   // four adjacent columns: one 16-byte store
            st4_nt(&dS0[(size_t)bh * D * D + (size_t)(16 * w + cl) * D + 16 * mj + 4 * g], dSt[mj]);
    }
}

// ======================================================================
// Chunk-local gradients, every chunk in parallel
// ======================================================================
template <class TR, int D>
struct BwdChunkSmem {
    typedef typename TR::E E;
    static constexpr int LD = D + TR::PAD;     // [CH][D] operands
    static constexpr int LDP = CH + TR::PAD;   // [CH][CH] matrices
    static constexpr int LDF = D + 4;          // fp32 staging of the results
    static constexpr size_t ROWB = (size_t)CH * LD * sizeof(E);
    static constexpr size_t SQB = (size_t)CH * LDP * sizeof(E);
    static constexpr size_t OPB = 5 * ROWB + 6 * SQB;
    static constexpr size_t STB = 4 * (size_t)CH * LDF * sizeof(float);
    // operands (Qb, Kb, Kc, V, dO, then P, dGK hi/lo, dP hi/lo, Gsym); later the staging
    alignas(16) unsigned char big[OPB > STB ? OPB : STB];
    alignas(16) float gam[D];          // gamma_C
    alignas(16) float beta[CH];
    alignas(16) float u[CH];
    alignas(16) float r0[CH];
    alignas(16) float drho[CH];
    alignas(16) float dr0[CH];
    alignas(16) float dbp[NSB][CH];    // dbeta partial of row t from column block J (J <= t / 16)
    alignas(16) float bprod[NSB][D];
    alignas(16) float gC2[D];          // sum_i dS[i][j] S0[i][j]
    alignas(16) float gsub[NSB][D];    // sub-block sums of g
    alignas(16) float hsub[NSB][D];    // sub-block sums of dKt * Kt
    unsigned unsafe_any;
};

// The gradients of chunk n of (b, h) = bh.  stale (thread 0's is read):
// nonzero when dS and rho of the unit could not be received; every output of
// the unit is then NaN, as for an unsafe decay.
template <class TR, int D>
__device__ __forceinline__ void bwd_chunk_body(
    BwdChunkSmem<TR, D>& sm, int bh, int n, int tid, unsigned stale,
    const typename TR::E* __restrict__ q, const typename TR::E* __restrict__ k,
    const typename TR::E* __restrict__ v, const typename TR::E* __restrict__ f,
    const float* __restrict__ beta, const typename TR::E* __restrict__ dO,
    const typename TR::E* __restrict__ ckptS, const float* __restrict__ ckptU,
    const typename TR::E* __restrict__ wsdS, const float* __restrict__ wsrho,
    typename TR::E* __restrict__ dq, typename TR::E* __restrict__ dk,
    typename TR::E* __restrict__ dv, typename TR::E* __restrict__ df,
    float* __restrict__ dbeta, float* __restrict__ dc, int T, int H)
{
    typedef typename TR::E E;
    typedef typename TR::Frag Frag;
    typedef BwdChunkSmem<TR, D> SM;
    constexpr int NT = 4 * D;
    constexpr int NW = D / 16;
    constexpr int KD_ = D / TR::KS;
    constexpr int KC_ = CH / TR::KS;
    constexpr int LD = SM::LD, LDP = SM::LDP, LDF = SM::LDF;

    E* Qb = reinterpret_cast<E*>(sm.big);
    E* Kb = Qb + CH * LD;
    E* Kc = Kb + CH * LD;
    E* Vs = Kc + CH * LD;
    E* Do = Vs + CH * LD;
    E* P = Do + CH * LD;
    E* dGK = P + CH * LDP;     // hi part (bf16) ...
    E* dGKl = dGK + CH * LDP;  // ... and the rest
    E* dP = dGKl + CH * LDP;
    E* dPl = dP + CH * LDP;
    E* Gs = dPl + CH * LDP;
    float* stQ = reinterpret_cast<float*>(sm.big);
    float* stK = stQ + CH * LDF;
    float* stC = stK + CH * LDF;
    float* stT = stC + CH * LDF;

    // tid: threadIdx.x (see the fused kernel)
    const int lane = tid & 63, w = tid >> 6, g = lane >> 4, cl = lane & 15;
    const PrepIdx pi(tid, D);
    const int r8 = pi.r8, I = pi.I, ch0 = pi.ch0, row0 = pi.row0;
    const int NC = (T + CH - 1) / CH;
    const int b = bh / H, h = bh % H;
    const uint32_t rs = (uint32_t)H * D;
    const size_t bbase = (size_t)b * T * H * D;
    const uint32_t hoff = (uint32_t)h * D;
    const size_t unit = (size_t)bh * NC + n;

    // ---------------- prep (a)
    // q, k, f and the decay factors are needed again by the elementwise stage
    // at the end; they are re-read there (L2) rather than held in registers
    // through the contractions.
    const int ta = min(n * CH + row0, T - 1), tb = min(n * CH + row0 + 1, T - 1);
    const uint32_t oa = (uint32_t)ta * rs + hoff + ch0, ob = (uint32_t)tb * rs + hoff + ch0;
    const bool ragged = n * CH + CH > T;
    auto load_qkf = [&](Row2x8<TR>& rq_, Row2x8<TR>& rk_, Row2x8<TR>& rf_) {
        rq_.load(q + bbase, oa, ob);
        rk_.load(k + bbase, oa, ob);
        rf_.load(f + bbase, oa, ob);
    };
    auto clear_qkf = [&](Row2x8<TR>& rq_, Row2x8<TR>& rk_, Row2x8<TR>& rf_) {
        if (ragged) {
#pragma unroll
            for (int e = 0; e < 2; ++e)
                if (n * CH + row0 + e >= T) { rq_.clear(e, 0.f); rk_.clear(e, 0.f); rf_.clear(e, 1.f); }
        }
    };
    // gamma at this thread's two rows and gamma_C, from f and the sub-block
    // products in sm.bprod (the same arithmetic every time it is called)
    auto gammas = [&](const Row2x8<TR>& rf_, float (&ga_)[2][8], float (&gC_)[8]) {
        float plt[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) { plt[c] = 1.f; gC_[c] = 1.f; }
#pragma unroll
        for (int I2 = 0; I2 < NSB; ++I2)
#pragma unroll
            for (int c4 = 0; c4 < 2; ++c4) {
                const floatx4 x = *reinterpret_cast<const floatx4*>(&sm.bprod[I2][ch0 + 4 * c4]);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    gC_[4 * c4 + e] *= x[e];
                    if (I2 < I) plt[4 * c4 + e] *= x[e];
                }
            }
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const float incl = group8_prefix_prod(rf_.get(0, c) * rf_.get(1, c), r8);
            const float excl = group8_shift1(incl, r8);
            ga_[0][c] = plt[c] * (excl * rf_.get(0, c));
            ga_[1][c] = plt[c] * incl;
        }
    };
    Row2x8<TR> pq, pk, rv, pf, ro;   // prep copies of q, k, f
    load_qkf(pq, pk, pf);
    rv.load(v + bbase, oa, ob);
    ro.load(dO + bbase, oa, ob);
    if (tid < CH) {
        const bool valid = n * CH + tid < T;
        const int t = min(n * CH + tid, T - 1);
        sm.beta[tid] = valid ? beta[((size_t)b * T + t) * H + h] : 0.f;
        sm.u[tid] = valid ? ckptU[unit * 2 * CH + tid] : 0.f;
        sm.r0[tid] = valid ? ckptU[unit * 2 * CH + CH + tid] : 0.f;
        sm.drho[tid] = valid ? wsrho[unit * CH + tid] : 0.f;
    }
    clear_qkf(pq, pk, pf);
    if (ragged) {
#pragma unroll
        for (int e = 0; e < 2; ++e)
            if (n * CH + row0 + e >= T) { rv.clear(e, 0.f); ro.clear(e, 0.f); }
    }
    // the upper triangles of P, dGK, dP (hi and lo) are never written
    for (int x = tid; x < 5 * CH * LDP * (int)sizeof(E) / 16; x += NT)
        reinterpret_cast<uint4*>(P)[x] = make_uint4(0u, 0u, 0u, 0u);
    if (tid == 0) sm.unsafe_any = stale;
    {
        float incl[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) incl[c] = group8_prefix_prod(pf.get(0, c) * pf.get(1, c), r8);
        if (r8 == 7) st8v(&sm.bprod[I][ch0], incl);
    }
    lds_barrier();

    // ---------------- prep (b): operands
    {
        float ga[2][8], gC[8];
        gammas(pf, ga, gC);
        unsigned unsafe = 0;
#pragma unroll
        for (int c = 0; c < 8; ++c)
            if (!(gC[c] >= kSafeFloor)) unsafe |= 1u << c;
        if (unsafe) atomicOr(&sm.unsafe_any, 1u);
        if (I == 0 && r8 == 0) st8v(&sm.gam[ch0], gC);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            float qo[8], ko[8], co[8];
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const float kf = pk.get(e, c);
                const bool un = (unsafe >> c) & 1u;
                const float kr = kf * __builtin_amdgcn_rcpf(ga[e][c]);
                qo[c] = pq.get(e, c) * ga[e][c];
                ko[c] = kf * ga[e][c];
                co[c] = un ? 0.f : kr;
            }
            st8v(&Qb[(row0 + e) * LD + ch0], qo);
            st8v(&Kb[(row0 + e) * LD + ch0], ko);
            st8v(&Kc[(row0 + e) * LD + ch0], co);
            rv.store(&Vs[(row0 + e) * LD + ch0], e);
            ro.store(&Do[(row0 + e) * LD + ch0], e);
        }
    }
    if (tid < CH) sm.dr0[tid] = -sm.beta[tid] * sm.drho[tid];
    lds_barrier();

    // ---------------- C x C tiles: P, dP, dGK, dGV (+ its transpose), dbeta
    for (int tile = w; tile < 10; tile += NW) {
        const int I_ = tile < 1 ? 0 : tile < 3 ? 1 : tile < 6 ? 2 : 3;
        const int J_ = tile - (I_ * (I_ + 1)) / 2;
        const int s_ = SB * J_ + cl;
        floatx4 gk = {0.f, 0.f, 0.f, 0.f}, gv = gk, pp = gk, dp = gk;
        const float us = sm.u[s_];
#pragma unroll
        for (int ks = 0; ks < KD_; ++ks) {
            const Frag fk = TR::ld_nat(&Kc[(SB * J_ + cl) * LD], ks, g);
            const Frag fv = TR::ld_nat(&Vs[(SB * J_ + cl) * LD], ks, g);
            gk = TR::mma(TR::ld_nat(&Kb[(SB * I_ + cl) * LD], ks, g), fk, gk);
            pp = TR::mma(TR::ld_nat(&Qb[(SB * I_ + cl) * LD], ks, g), fk, pp);
            gv = TR::mma(TR::ld_nat(&Vs[(SB * I_ + cl) * LD], ks, g), fv, gv);
            dp = TR::mma(TR::ld_nat(&Do[(SB * I_ + cl) * LD], ks, g), fv, dp);
        }
        dp = dp * us;   // dP[t][s] = u_s (dO V^T)[t][s]: column s = this lane's
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t_ = SB * I_ + 4 * g + r;
            const bool low = s_ < t_, inc = s_ <= t_;
            const float dM = low ? -sm.drho[t_] * us : 0.f;
            const float bt = sm.beta[t_];
            const float dgv = bt * dM * gk[r];
            P[t_ * LDP + s_] = TR::cvt(inc ? pp[r] : 0.f);
            const float dpv = inc ? dp[r] : 0.f, dgkv = bt * dM * gv[r];
            const E dph = TR::cvt(dpv), dgkh = TR::cvt(dgkv);
            dP[t_ * LDP + s_] = dph;
            dPl[t_ * LDP + s_] = TR::lo_part(dpv, dph);
            dGK[t_ * LDP + s_] = dgkh;
            dGKl[t_ * LDP + s_] = TR::lo_part(dgkv, dgkh);
            if (low) {
                Gs[t_ * LDP + s_] = TR::cvt(dgv);
                Gs[s_ * LDP + t_] = TR::cvt(dgv);
            } else if (s_ == t_) {
                Gs[t_ * LDP + t_] = TR::cvt(0.f);
            }
            float db = dM * gk[r] * gv[r];
            db += __shfl_xor(db, 1, 64);
            db += __shfl_xor(db, 2, 64);
            db += __shfl_xor(db, 4, 64);
            db += __shfl_xor(db, 8, 64);
            if (cl == 0) sm.dbp[J_][t_] = db;
        }
    }
    const int jc = 16 * w + cl;   // this lane's output column (key j, or value i for dV)
    const E* S0n = ckptS + unit * D * D;   // S0[i][j]
    const E* dSn = wsdS + unit * D * D;    // dS[i][j]
    if (!std::is_same<TR, Bf16T>::value) {   // colsum(dS * S0) for column jc (bf16: below)
        float acc = 0.f;
        for (int x = 0; x < D / 4; ++x) {
            const int i = g * (D / 4) + x;
            acc += TR::tof(S0n[i * D + jc]) * TR::tof(dSn[i * D + jc]);
        }
        acc += __shfl_xor(acc, 16, 64);
        acc += __shfl_xor(acc, 32, 64);
        if (g == 0) sm.gC2[jc] = acc;
    }
    lds_barrier();

    // ---------------- C x D results, this wave's 16 columns, all 64 rows
    // Scalings by u[t] or dr0[t] of the output row t are applied to the
    // accumulators, not to the operands: aK and aT start as V S0 and V dS, and
    // dV is accumulated in two parts, aVu = Kt dS^T + P^T dO (times u) and
    // aVr = dr0 (Kbar S0^T) + (dGV + dGV^T) V.  The key-channel scaling of
    // Kt = Kc gamma_C goes on the dS fragment, once per K-step.
    floatx4 aQ[NSB], aK[NSB], aC[NSB], aT[NSB], aVu[NSB], aVr[NSB];
#pragma unroll
    for (int tt = 0; tt < NSB; ++tt) {
        aQ[tt] = floatx4{0.f, 0.f, 0.f, 0.f};
        aK[tt] = aQ[tt]; aC[tt] = aQ[tt]; aT[tt] = aQ[tt]; aVu[tt] = aQ[tt]; aVr[tt] = aQ[tt];
    }
    // contractions over a d-long index, B operands from the state checkpoints
    // in global memory (L2): rows directly, columns through col_frag (whose
    // tiles also give colsum(dS * S0) for bf16)
    {
        const Frag csel = TR::col_sel(16 * w, g, cl);
        float gc2 = 0.f;
#pragma unroll
        for (int ks = 0; ks < KD_; ++ks) {
            floatx4 ts[2], td[2];
            const Frag b_s0t = TR::col_frag(S0n, D, ks, 16 * w, csel, g, cl, ts);   // B[i][j] = S0[i][j]
            const Frag b_dst = TR::col_frag(dSn, D, ks, 16 * w, csel, g, cl, td);   // B[i][j] = dS[i][j]
            if (std::is_same<TR, Bf16T>::value) {
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                    for (int r = 0; r < 4; ++r) gc2 += ts[hh][r] * td[hh][r];
            }
            const Frag b_dsg = TR::scale_k(TR::ld_nat(dSn + jc * D, ks, g), 1.f, sm.gam, ks, g);   // B[j][i] = dS[i][j] gamma_C[j]
            const Frag b_s0 = TR::ld_nat(S0n + jc * D, ks, g);     // B[j][i] = S0[i][j]
#pragma unroll
            for (int tt = 0; tt < NSB; ++tt) {
                const int tr = SB * tt + cl;
                const Frag a_v = TR::ld_colmatch(&Vs[tr * LD], ks, g);
                aQ[tt] = TR::mma(TR::ld_colmatch(&Do[tr * LD], ks, g), b_s0t, aQ[tt]);   // dO S0
                aK[tt] = TR::mma(a_v, b_s0t, aK[tt]);                                      // V S0
                aT[tt] = TR::mma(a_v, b_dst, aT[tt]);                                      // V dS
                aVu[tt] = TR::mma(TR::ld_nat(&Kc[tr * LD], ks, g), b_dsg, aVu[tt]);       // Kt dS^T
                aVr[tt] = TR::mma(TR::ld_nat(&Kb[tr * LD], ks, g), b_s0, aVr[tt]);        // Kbar S0^T
            }
        }
        if (std::is_same<TR, Bf16T>::value) {
            gc2 += __shfl_xor(gc2, 16, 64);
            gc2 += __shfl_xor(gc2, 32, 64);
            if (g == 0) sm.gC2[jc] = gc2;
        }
    }
#pragma unroll
    for (int tt = 0; tt < NSB; ++tt) {
        const floatx4 r0v = *reinterpret_cast<const floatx4*>(&sm.dr0[SB * tt + 4 * g]);
        const floatx4 uv = *reinterpret_cast<const floatx4*>(&sm.u[SB * tt + 4 * g]);
        aK[tt] = aK[tt] * r0v;    // dr0 (V S0)
        aT[tt] = aT[tt] * uv;     // W dS
        aVr[tt] = aVr[tt] * r0v;  // dr0 (Kbar S0^T)
    }
    // contractions over the chunk: transposed operands read in place
#pragma unroll
    for (int ks = 0; ks < KC_; ++ks) {
        const Frag b_kc = TR::ld_col(&Kc[jc], LD, ks, g);   // B[s][j] = Kc[s][j]
        const Frag b_kb = TR::ld_col(&Kb[jc], LD, ks, g);   // B[t][j] = Kbar[t][j]
        const Frag b_qb = TR::ld_col(&Qb[jc], LD, ks, g);   // B[t][j] = Qbar[t][j]
        const Frag b_v = TR::ld_col(&Vs[jc], LD, ks, g);    // B[s][i] = V[s][i]
        const Frag b_do = TR::ld_col(&Do[jc], LD, ks, g);   // B[t][i] = dO[t][i]
#pragma unroll
        for (int tt = 0; tt < NSB; ++tt) {
            const int tr = SB * tt + cl;
            // dP and dGK enter as hi + lo (their bf16 rounding would dominate the
            // error of dq and df)
            aQ[tt] = TR::mma(TR::ld_nat(&dP[tr * LDP], ks, g), b_kc, aQ[tt]);            // dP Kc
            aK[tt] = TR::mma(TR::ld_nat(&dGK[tr * LDP], ks, g), b_kc, aK[tt]);           // dGK Kc
            aC[tt] = TR::mma(TR::ld_col(&dGK[tr], LDP, ks, g), b_kb, aC[tt]);            // dGK^T Kbar
            aC[tt] = TR::mma(TR::ld_col(&dP[tr], LDP, ks, g), b_qb, aC[tt]);             // dP^T Qbar
            if (TR::SPLIT) {
                aQ[tt] = TR::mma(TR::ld_nat(&dPl[tr * LDP], ks, g), b_kc, aQ[tt]);
                aK[tt] = TR::mma(TR::ld_nat(&dGKl[tr * LDP], ks, g), b_kc, aK[tt]);
                aC[tt] = TR::mma(TR::ld_col(&dGKl[tr], LDP, ks, g), b_kb, aC[tt]);
                aC[tt] = TR::mma(TR::ld_col(&dPl[tr], LDP, ks, g), b_qb, aC[tt]);
            }
            aVr[tt] = TR::mma(TR::ld_nat(&Gs[tr * LDP], ks, g), b_v, aVr[tt]);           // (dGV + dGV^T) V
            aVu[tt] = TR::mma(TR::ld_col(&P[tr], LDP, ks, g), b_do, aVu[tt]);            // P^T dO
        }
    }
    floatx4 aV[NSB];   // dV = u (Kt dS^T + P^T dO) + aVr
#pragma unroll
    for (int tt = 0; tt < NSB; ++tt)
        aV[tt] = aVu[tt] * *reinterpret_cast<const floatx4*>(&sm.u[SB * tt + 4 * g]) + aVr[tt];
    // q, k, f again for the elementwise stage (in flight during the staging)
    Row2x8<TR> rq, rk, rf;
    load_qkf(rq, rk, rf);
    lds_barrier();   // every operand read is done: the staging reuses the space
#pragma unroll
    for (int tt = 0; tt < NSB; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = SB * tt + 4 * g + r;
            stQ[row * LDF + jc] = aQ[tt][r];
            stK[row * LDF + jc] = aK[tt][r];
            stC[row * LDF + jc] = aC[tt][r];
            stT[row * LDF + jc] = aT[tt][r];
        }
    lds_barrier();

    // ---------------- elementwise: dq, dk, and the decay gradient (prep layout)
    clear_qkf(rq, rk, rf);
    float ga[2][8], gC[8];
    gammas(rf, ga, gC);   // bitwise the values the prep used
    const bool poison = sm.unsafe_any != 0u;
    float dqv[2][8], dkv[2][8], suf0[8], suf1[8], totg[8], toth[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        float gg[2], hh[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int idx = (row0 + e) * LDF + ch0 + c;
            const float dQ = stQ[idx], dKb = stK[idx], dKc = stC[idx], dKt = stT[idx];
            const float gm = ga[e][c], rg = __builtin_amdgcn_rcpf(gm);
            const float qf = rq.get(e, c), kf = rk.get(e, c);
            // Qbar, Kbar, Kc exactly as the MFMA products saw them (same fp32
            // arithmetic as the prep, same rounding): each Gram pair (t, s)
            // then enters g_t and g_s with equal and opposite values, and the
            // suffix sums below cancel it exactly.  Kt enters no product whose
            // result feeds g, so it is taken exact.
            const float kr = kf * rg;
            const float Qbar = TR::tof(TR::cvt(qf * gm)), Kbar = TR::tof(TR::cvt(kf * gm));
            const float Kcv = TR::tof(TR::cvt(kr)), Ktv = kr * gC[c];
            dqv[e][c] = dQ * gm;
            dkv[e][c] = dKb * gm + dKc * rg + dKt * (gC[c] * rg);
            gg[e] = dQ * Qbar + dKb * Kbar - dKc * Kcv - dKt * Ktv;
            hh[e] = dKt * Ktv;
        }
        const float pair = gg[0] + gg[1];
        const float inc = group8_suffix_sum(pair, r8);
        const float nxt = group8_next1(inc, r8);
        toth[c] = group8_suffix_sum(hh[0] + hh[1], r8);
        totg[c] = inc;
        suf1[c] = nxt + gg[1];
        suf0[c] = suf1[c] + gg[0];
    }
    if (r8 == 0) {
        st8v(&sm.gsub[I][ch0], totg);
        st8v(&sm.hsub[I][ch0], toth);
    }
    lds_barrier();
    {
        float dfv[2][8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            float later = 0.f, htot = 0.f;
#pragma unroll
            for (int I2 = 0; I2 < NSB; ++I2) {
                if (I2 > I) later += sm.gsub[I2][ch0 + c];
                htot += sm.hsub[I2][ch0 + c];
            }
            const float base = later + gC[c] * sm.gC2[ch0 + c] + htot;
            dfv[0][c] = (suf0[c] + base) / rf.get(0, c);
            dfv[1][c] = (suf1[c] + base) / rf.get(1, c);
        }
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int t = n * CH + row0 + e;
            if (t < T) {
                if (poison) {
#pragma unroll
                    for (int c = 0; c < 8; ++c) {
                        dqv[e][c] = __builtin_nanf("");
                        dkv[e][c] = dqv[e][c];
                        dfv[e][c] = dqv[e][c];
                    }
                }
                const uint32_t off = (uint32_t)t * rs + hoff + ch0;
                st8v_nt(dq + bbase + off, dqv[e]);
                st8v_nt(dk + bbase + off, dkv[e]);
                st8v_nt(df + bbase + off, dfv[e]);
            }
        }
    }
    lds_barrier();   // staging reads done before dV reuses it
#pragma unroll
    for (int tt = 0; tt < NSB; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r) stQ[(SB * tt + 4 * g + r) * LDF + jc] = aV[tt][r];
    lds_barrier();
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int t = n * CH + row0 + e;
        if (t < T) {
            float x[8];
#pragma unroll
            for (int c = 0; c < 8; ++c) x[c] = poison ? __builtin_nanf("") : stQ[(row0 + e) * LDF + ch0 + c];
            st8v_nt(dv + bbase + (uint32_t)t * rs + hoff + ch0, x);
        }
    }
    if (tid < CH && n * CH + tid < T) {
        const size_t gi = ((size_t)b * T + n * CH + tid) * H + h;
        float db = -sm.r0[tid] * sm.drho[tid];
        for (int J = 0; J <= tid / SB; ++J) db += sm.dbp[J][tid];   // fixed order: bitwise reproducible
        st_nt(&dbeta[gi], poison ? __builtin_nanf("") : db);
        st_nt(&dc[gi], poison ? __builtin_nanf("") : sm.drho[tid]);
    }
}

template <class TR, int D>
__global__ __launch_bounds__(4 * D) void kd_bwd_state_kernel(
    const typename TR::E* __restrict__ q, const typename TR::E* __restrict__ k,
    const typename TR::E* __restrict__ v, const typename TR::E* __restrict__ f,
    const float* __restrict__ beta, const typename TR::E* __restrict__ dO,
    const float* __restrict__ ckM, const typename TR::E* __restrict__ ckP,
    const float* __restrict__ dST, typename TR::E* __restrict__ wsdS, float* __restrict__ wsrho,
    float* __restrict__ dS0, int T, int H)
{
    __shared__ BwdStateSmem<TR, D> sm;
    bwd_state_body<TR, D, false>(sm, blockIdx.x, q, k, v, f, beta, dO, ckM, ckP, dST, wsdS, wsrho, dS0, T, H);
}

template <class TR, int D>
__global__ __launch_bounds__(4 * D) void kd_bwd_chunk_kernel(
    const typename TR::E* __restrict__ q, const typename TR::E* __restrict__ k,
    const typename TR::E* __restrict__ v, const typename TR::E* __restrict__ f,
    const float* __restrict__ beta, const typename TR::E* __restrict__ dO,
    const typename TR::E* __restrict__ ckptS, const float* __restrict__ ckptU,
    const typename TR::E* __restrict__ wsdS, const float* __restrict__ wsrho,
    typename TR::E* __restrict__ dq, typename TR::E* __restrict__ dk,
    typename TR::E* __restrict__ dv, typename TR::E* __restrict__ df,
    float* __restrict__ dbeta, float* __restrict__ dc, int T, int H)
{
    __shared__ BwdChunkSmem<TR, D> sm;
    const int NC = (T + CH - 1) / CH;
    bwd_chunk_body<TR, D>(sm, blockIdx.x / NC, blockIdx.x % NC, threadIdx.x, 0u, q, k, v, f, beta, dO, ckptS, ckptU,
                          wsdS, wsrho, dq, dk, dv, df, dbeta, dc, T, H);
}

// Both backward kernels in one launch, so the chunk gradients run on the CUs
// the sweep leaves idle while the sweep goes on.  Blocks 0 .. BHpad - 1 sweep
// (one per (b, h); blocks past B*H have no head) and then join the others,
// persistent workers that take (b, h, chunk) units from their XCD's claim
// counter.  Dispatch is in block order on each XCD, so every sweep block is
// resident before any worker, and a sweep never waits: the workers' waits
// always end.  Blocks x and x + 8 share an XCD under round-robin placement,
// so the blocks with x = c (mod 8) share the chunks of the heads bh = c
// (mod 8), handed out in the sweep's order (newest chunk first, then the
// heads in turn), and read their dS and rho through the XCD's L2.  Block c
// sets the counter of XCD c before any claim is made (a claimer waits for
// this launch's epoch in it).  Should a worker find the writer on
// another XCD (the flag's id), it waits for the sweep's closing L2 write-back
// (chunk 0's flag) and acquires at agent scope before reading.  A wait that
// runs out of its bound turns the unit's outputs into NaN.
template <class TR, int D>
__global__ __launch_bounds__(4 * D) void kd_bwd_fused_kernel(
    const typename TR::E* __restrict__ q, const typename TR::E* __restrict__ k,
    const typename TR::E* __restrict__ v, const typename TR::E* __restrict__ f,
    const float* __restrict__ beta, const typename TR::E* __restrict__ dO,
    const float* __restrict__ ckM, const typename TR::E* __restrict__ ckP,
    const typename TR::E* __restrict__ ckptS, const float* __restrict__ ckptU,
    const float* __restrict__ dST, typename TR::E* __restrict__ wsdS, float* __restrict__ wsrho,
    float* __restrict__ dS0, typename TR::E* __restrict__ dq, typename TR::E* __restrict__ dk,
    typename TR::E* __restrict__ dv, typename TR::E* __restrict__ df,
    float* __restrict__ dbeta, float* __restrict__ dc, int BH, int BHpad, int nwork, BwdPub pub,
    int T, int H)
{
    union Smem {
        BwdStateSmem<TR, D> s;
        BwdChunkSmem<TR, D> c;
    };
    __shared__ Smem sm;
    __shared__ int g_unit;
    const int x = blockIdx.x;
    const int NC = (T + CH - 1) / CH;
    int c;   // this block's XCD under round-robin placement: x mod 8
    if (x < BHpad) {
        if (x < 8 && threadIdx.x == 0)
            __hip_atomic_store(&pub.ctr[x], (unsigned long long)pub.epoch << 32, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        if (x < BH) {
            if (threadIdx.x == 0) g_pub = pub;   // read after the sweep's first barriers
            bwd_state_body<TR, D, true>(sm.s, x, q, k, v, f, beta, dO, ckM, ckP, dST, wsdS, wsrho, dS0, T, H);
            lds_barrier();   // the sweep's LDS is done with: the block joins the workers
        }
        c = x & 7;
    } else {
        c = (x - BHpad) & 7;
    }
    const int nh = c < BH ? (BH - c + 7) / 8 : 0;   // heads c, c + 8, ... on this XCD
    const int total = nh * NC;
    const unsigned me = xcc_id();
    // thread 0 only: dyn, units come from the claim counter (pending: the
    // claim in flight); otherwise, if the counter never showed this launch's
    // epoch, a worker takes the units r, r + R, ... (next); dead: a wait ran
    // out, so every unit taken from then on is NaN
    bool dyn = false, dead = false;
    int next = -1;
    unsigned long long pending = 0;
    if (threadIdx.x == 0 && total > 0) {
        unsigned long long w = 0;
        if (pub_wait(&pub.ctr[c], pub.epoch, 0ull, w)) {
            dyn = true;
            pending = __hip_atomic_fetch_add(&pub.ctr[c], 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            dead = true;
            next = x < BHpad ? -1 : (x - BHpad) >> 3;
        }
    }
#pragma unroll 1
    for (;;) {
        if (threadIdx.x == 0) {
            int u = -1;
            if (dyn) {
                const unsigned k = (unsigned)pending;   // units claimed before this one
                if (k < (unsigned)total) {
                    u = (int)k;
                    // the claim of the unit after this one is in flight during the body
                    pending = __hip_atomic_fetch_add(&pub.ctr[c], 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                } else {
                    dyn = false;
                }
            } else if (next >= 0 && next < total) {
                u = next;
                next += nwork >> 3;
            }
            if (u >= 0 && !dead) {
                const int n = NC - 1 - u / nh, bh = c + 8 * (u % nh);
                unsigned long long w = 0;
                dead = !pub_wait(&pub.flags[(size_t)bh * NC + n], pub.epoch, 1ull, w);
                // a writer on another XCD: wait for its L2 write-back, then drop
                // this XCD's copies
                if (!dead && ((unsigned)(w >> 24) & 0xffu) != me) {
                    dead = !pub_wait(&pub.flags[(size_t)bh * NC], pub.epoch, PUB_FLUSHED, w);
                    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                }
            }
            g_unit = u < 0 ? -1 : (dead ? -2 - u : u);   // -2 - u: unit u, as NaN
        }
        lds_barrier();
        const int gu = g_unit;
        if (gu == -1) break;
        const int u = gu >= 0 ? gu : -2 - gu;
        const int n = NC - 1 - u / nh, bh = c + 8 * (u % nh);
        // the thread index through an opaque zero: nothing the body derives
        // from it is invariant across units, so nothing is hoisted out of this
        // loop to hold registers through the body
        int z;
        asm volatile("v_mov_b32 %0, 0" : "=v"(z));
        bwd_chunk_body<TR, D>(sm.c, bh, n, (int)threadIdx.x + z, gu < 0 ? 1u : 0u, q, k, v, f, beta, dO, ckptS,
                              ckptU, wsdS, wsrho, dq, dk, dv, df, dbeta, dc, T, H);
        lds_barrier();   // the next unit reuses the LDS (and g_unit)
    }
}

// --------------------------------------------------------------- launchers
// compute units of the current device (the fused backward sizes its worker
// pool to the CUs the sweep leaves free)
static int compute_units() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int n = cache[dev].load();
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n = 0;
        cache[dev].store(n);
    }
    return n;
}

// launch epochs of the fused backward: each launch's flags differ from every
// earlier launch's, so flags left in a reused workspace never match
static unsigned next_bwd_epoch() {
    static std::atomic<unsigned> e{0u};
    unsigned v = e.fetch_add(1u) + 1u;
    if (v == 1u) {   // first launch of the process: start from the clock
        const unsigned t = (unsigned)time(nullptr) * 2654435761u;
        e.fetch_add(t);
        v += t;
    }
    return v;
}

// the forward's records of each chunk, where the backward workspace keeps them
static FwdCkpt ckpt_in(void* ws, size_t esize, int D, int B, int T, int H) {
    const BwdWs L = bwd_ws_layout(esize, D, B, T, H);
    char* wb = static_cast<char*>(ws);
    FwdCkpt ck;
    ck.S = wb + L.s0;
    ck.U = reinterpret_cast<float*>(wb + L.ur);
    ck.M = reinterpret_cast<float*>(wb + L.mm);
    ck.P = wb + L.pp;
    return ck;
}

// Forward for training: o, S_T and the per-chunk records the backward reads.
hipError_t launch_fwd_train(int bf16, int d, const void* q, const void* k, const void* v, const void* f,
                            const float* beta, const float* c, const float* S0, void* o, float* ST,
                            void* ws, int B, int T, int H, hipStream_t st)
{
    const FwdCkpt ck = ckpt_in(ws, bf16 ? 2 : 4, d, B, T, H);
    return launch_fwd(bf16, d, q, k, v, f, beta, c, S0, o, ST, &ck, nullptr, B, T, H, st);
}

// recompute: run the recording forward first (otherwise the records of a
// preceding launch_fwd_train on the same inputs and workspace are used)
template <class TR, int D>
static hipError_t launch_bwd_t(const void* q, const void* k, const void* v, const void* f,
                               const float* beta, const float* c, const float* S0, const void* dO,
                               const float* dST, void* dq, void* dk, void* dv, void* df,
                               float* dbeta, float* dc, float* dS0, void* ws, int B, int T, int H,
                               int recompute, hipStream_t st)
{
    typedef typename TR::E E;
    const BwdWs L = bwd_ws_layout(sizeof(E), D, B, T, H);
    char* wb = static_cast<char*>(ws);
    const FwdCkpt ck = ckpt_in(ws, sizeof(E), D, B, T, H);
    E* wdS = reinterpret_cast<E*>(wb + L.ds);
    float* wrho = reinterpret_cast<float*>(wb + L.rho);
    const int NC = (T + CH - 1) / CH;
    if (NC > 0 && recompute) {
        hipError_t e = launch_fwd(sizeof(E) == 2, D, q, k, v, f, beta, c, S0, nullptr, nullptr, &ck,
                                  nullptr, B, T, H, st);
        if (e != hipSuccess) return e;
    }
    // The fused launch when at least 64 workers fit beside the sweep blocks.
    const int BH = B * H, BHpad = (BH + 7) & ~7;
    const int nwork = ((compute_units() - BHpad) / 8) * 8;
    if (NC > 0 && nwork >= 64) {
        BwdPub pub;
        pub.ctr = reinterpret_cast<unsigned long long*>(wb + L.fl);
        pub.flags = reinterpret_cast<unsigned long long*>(wb + L.fl + 256);
        pub.epoch = next_bwd_epoch();
        hipLaunchKernelGGL((kd_bwd_fused_kernel<TR, D>), dim3((unsigned)(BHpad + nwork)), dim3(4 * D), 0, st,
                           (const E*)q, (const E*)k, (const E*)v, (const E*)f, beta, (const E*)dO,
                           (const float*)ck.M, (const E*)ck.P, (const E*)ck.S, (const float*)ck.U, dST, wdS,
                           wrho, dS0, (E*)dq, (E*)dk, (E*)dv, (E*)df, dbeta, dc, BH, BHpad, nwork, pub, T, H);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((kd_bwd_state_kernel<TR, D>), dim3((unsigned)(B * H)), dim3(4 * D), 0, st,
                       (const E*)q, (const E*)k, (const E*)v, (const E*)f, beta, (const E*)dO,
                       (const float*)ck.M, (const E*)ck.P, dST, wdS, wrho, dS0, T, H);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || NC == 0) return e;
    hipLaunchKernelGGL((kd_bwd_chunk_kernel<TR, D>), dim3((unsigned)(B * H * NC)), dim3(4 * D), 0, st,
                       (const E*)q, (const E*)k, (const E*)v, (const E*)f, beta, (const E*)dO,
                       (const E*)ck.S, (const float*)ck.U, (const E*)wdS, (const float*)wrho,
                       (E*)dq, (E*)dk, (E*)dv, (E*)df, dbeta, dc, T, H);
    return hipGetLastError();
}

hipError_t launch_bwd(int bf16, int d, const void* q, const void* k, const void* v, const void* f,
                      const float* beta, const float* c, const float* S0, const void* dO,
                      const float* dST, void* dq, void* dk, void* dv, void* df, float* dbeta,
                      float* dc, float* dS0, void* ws, int B, int T, int H, int recompute,
                      hipStream_t st)
{
#define KD_BWD_ARGS q, k, v, f, beta, c, S0, dO, dST, dq, dk, dv, df, dbeta, dc, dS0, ws, B, T, H, recompute, st
    if (bf16) {
        switch (d) {
        case 32: return launch_bwd_t<Bf16T, 32>(KD_BWD_ARGS);
        case 64: return launch_bwd_t<Bf16T, 64>(KD_BWD_ARGS);
        case 128: return launch_bwd_t<Bf16T, 128>(KD_BWD_ARGS);
        }
    } else if (d == 32) {
        return launch_bwd_t<F32T, 32>(KD_BWD_ARGS);
    }
#undef KD_BWD_ARGS
    return hipErrorInvalidValue;
}

}  // namespace kd
