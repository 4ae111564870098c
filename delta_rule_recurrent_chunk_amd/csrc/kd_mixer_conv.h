// kd_mixer_conv.h -- the KronLSTM mixer's short causal depthwise convolution
// on q, k, v, then SiLU and the L2 norm per (token, head) (onedev.kr KronLSTM
// summary, section "어떻게 쓰나"), as a block-level device function shared by
// the stand-alone convolution kernel and the forward's convolution workers.
#pragma once

#include <hip/hip_runtime.h>

#include "kd_device.h"
#include "kd_handoff.h"

namespace kd {

constexpr int MIX_TT = 32;     // tokens walked by one thread (gates, post-processing)
constexpr int MIX_TB = 8;      // tokens whose loads are in flight together
constexpr int MIX_CT = 64;     // tokens of one convolution block
constexpr int MIX_NT = 256;    // threads per block
constexpr int MIX_KMAX = 4;    // widest convolution
constexpr float MIX_EPS_L2 = 1e-6f;

struct MixPreArgs {
    const void* raw[4];        // q, k, v, f projections [B, T, H, d]
    void* out[4];              // q, k, v, f
    const float* conv[3];      // [H, d, K] taps of q, k, v (tap K-1 on the current token)
    const float* a_log;        // [H]
    const float* beta_raw;     // [B, T, H]
    const float* c_raw;        // [B, T, H]
    float* beta;
    float* c;
    float beta_scale;
    int K;
};

// LDS of one convolution block: the raw rows of its tokens and the K - 1
// before them, and the head's taps
template <class E, int D, int K>
struct ConvLds {
    alignas(16) E st[(MIX_CT + K - 1) * D];
    alignas(16) float sw[D * K];   // taps of (h, channel i) at i*K
};

// Tokens t0 .. t0 + MIX_CT - 1 of tensor z (0: q, 1: k, 2: v) of (b, h), by
// MIX_NT threads (tid = 0 .. MIX_NT - 1), in three steps: conv_fetch loads the
// raw rows of the tokens and the K - 1 before them (zero before the first
// token; rows past the last token are never read) and the head's taps into
// registers, every load issued before any is used; conv_stage puts them in
// LDS; after a barrier, conv_rows makes the outputs, each row of D/8 lanes
// one token from K staged rows: convolution, SiLU, the row's sum of squares
// on DPP lane moves, the scale, one 16-byte store per lane (NT_STORE:
// streaming stores, for outputs no kernel of the launch reads back).
template <class E, int D, int K>
struct ConvRegs {
    static constexpr int ROWS = MIX_CT + K - 1;
    static constexpr int PPR = D * (int)sizeof(E) / 16;   // 16-byte pieces per row
    static constexpr int NPC = (ROWS * PPR + MIX_NT - 1) / MIX_NT;
    uint4 pcs[NPC];
    floatx4 tw;
};

template <class E, int D, int K>
__device__ __forceinline__ void conv_fetch(const MixPreArgs& a, int T, int H, int b, int h, int z, int t0,
                                           int tid, ConvRegs<E, D, K>& R) {
    typedef ConvRegs<E, D, K> CR;
    static_assert(D * K <= 4 * MIX_NT, "one float4 of taps per thread");
    const uint32_t rs = (uint32_t)H * D;   // token stride (elements); one batch element fits 2^31 bytes
    const E* __restrict__ src = static_cast<const E*>(a.raw[z]) + (size_t)b * T * rs + (size_t)h * D;
    R.tw = floatx4{0.f, 0.f, 0.f, 0.f};
    if (tid < D * K / 4) R.tw = reinterpret_cast<const floatx4*>(a.conv[z] + (size_t)h * D * K)[tid];
#pragma unroll
    for (int i = 0; i < CR::NPC; ++i) {
        const int x = tid + i * MIX_NT;
        const int r = x / CR::PPR, pc = x % CR::PPR;
        const int t = t0 - (K - 1) + r;
        R.pcs[i] = make_uint4(0u, 0u, 0u, 0u);
        if (x < CR::ROWS * CR::PPR && t >= 0 && t < T)
            R.pcs[i] = *reinterpret_cast<const uint4*>(src + (uint32_t)t * rs + pc * (16 / sizeof(E)));
    }
}

template <class E, int D, int K>
__device__ __forceinline__ void conv_stage(ConvLds<E, D, K>& L, const ConvRegs<E, D, K>& R, int tid) {
    typedef ConvRegs<E, D, K> CR;
#pragma unroll
    for (int i = 0; i < CR::NPC; ++i) {
        const int x = tid + i * MIX_NT;
        if (x < CR::ROWS * CR::PPR)
            *reinterpret_cast<uint4*>(&L.st[(x / CR::PPR) * D + (x % CR::PPR) * (16 / sizeof(E))]) = R.pcs[i];
    }
    if (tid < D * K / 4) reinterpret_cast<floatx4*>(L.sw)[tid] = R.tw;
}

template <class E, int D, int K, bool NT_STORE>
__device__ __forceinline__ void conv_rows(const MixPreArgs& a, int T, int H, int b, int h, int z, int t0,
                                          const ConvLds<E, D, K>& L, int tid) {
    constexpr int LPR = D / 8;                  // lanes per row
    constexpr int TPP = MIX_NT / LPR;           // tokens per pass
    static_assert(MIX_CT % TPP == 0, "a block's tokens are whole passes");
    const uint32_t rs = (uint32_t)H * D;
    E* __restrict__ dst = static_cast<E*>(a.out[z]) + (size_t)b * T * rs + (size_t)h * D;
    // taps of this lane's eight channels: wt[e][j] multiplies the token t - (K-1) + j
    const int o8 = tid % LPR, slot = tid / LPR;
    float wt[8][K];
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int j = 0; j < K; ++j) wt[e][j] = L.sw[(8 * o8 + e) * K + j];
#pragma unroll
    for (int ps = 0; ps < MIX_CT / TPP; ++ps) {
        const int r = ps * TPP + slot;   // output token t0 + r, staged rows r .. r + 3
        const int t = t0 + r;
        if (t >= T) break;               // the row's lanes leave together
        float y[8], ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = 0.f;
#pragma unroll
        for (int j = 0; j < K; ++j) {
            float x[8];
            ld8f(&L.st[(r + j) * D + 8 * o8], x);
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = fmaf(wt[e][j], x[e], y[e]);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            y[e] = y[e] * gate_sigmoid(y[e]);   // SiLU
            ss = fmaf(y[e], y[e], ss);
        }
        const float sc = rsqrtf(row_sum<LPR>(ss) + MIX_EPS_L2);
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] *= sc;
        if (NT_STORE) st8v_nt(dst + (uint32_t)t * rs + 8 * o8, y);
        else st8v(dst + (uint32_t)t * rs + 8 * o8, y);
    }
}

// The convolution feeding the mixer forward inside one launch (bf16, d = 128,
// conv_size 4): workers convolve the chunks of q, k, v in order and publish
// each (b, h, chunk) unit in flags; the forward's producers read a chunk's
// rows only after its unit is published.  nwork = 0: no feed (q, k, v are
// in memory before the launch).
struct ConvFeed {
    MixPreArgs mx;
    unsigned long long* hdr;     // [B*H]: the XCD of the forward block of each head
    unsigned long long* flags;   // [B*H*NC]
    unsigned epoch;
    unsigned spin;               // polls of a bounded wait before it gives up
    int BH, BHpad, nwork;
};

// A convolution worker of the fused mixer forward (blocks BHpad and up of a
// launch of 1024 threads): under round-robin placement blocks x and x + 8
// share an XCD, so the workers with x = c (mod 8) take the (b, h, chunk) units
// of the heads bh = c (mod 8) in chunk order, r, r + R, ... for the r-th of
// the R workers of XCD c.  A unit is three tensor jobs (its q, k, v); the
// four groups of 256 threads take the worker's jobs four at a time, and each
// round's raw rows are loaded while the round before computes.  A unit is
// published once its three jobs are stored; one whose forward block is not
// known to share the XCD is first written back to memory (PUB_FLUSHED).
__device__ __forceinline__ void conv_feed_worker(const ConvFeed& cf, void* lds, int T, int H) {
    typedef __bf16 E;
    constexpr int D = 128, K = 4;
    ConvLds<E, D, K>* L = reinterpret_cast<ConvLds<E, D, K>*>(lds);   // one per group
    const int NC = (T + CH - 1) / CH;
    const int x = blockIdx.x, c = x & 7, r = (x - cf.BHpad) >> 3, R = cf.nwork >> 3;
    const int nh = c < cf.BH ? (cf.BH - c + 7) / 8 : 0;   // heads c, c + 8, ... on this XCD
    const int total = nh * NC;
    const int mine = r < total ? (total - r + R - 1) / R : 0;   // units of this worker
    const int njobs = 3 * mine;
    const int g = threadIdx.x >> 8, tid = threadIdx.x & 255;
    const unsigned me = xcc_id();
    auto job = [&](int jb, int& b, int& h, int& z, int& t0) {   // job jb: tensor z of the worker's unit jb / 3
        const int i = jb / 3, u = r + i * R, n = u / nh, bh = c + 8 * (u % nh);
        z = jb - 3 * i;
        b = bh / H;
        h = bh % H;
        t0 = n * CH;
    };
    ConvRegs<E, D, K> cur;
    int b = 0, h = 0, z = 0, t0 = 0;
    bool act = g < njobs;
    if (act) {
        job(g, b, h, z, t0);
        conv_fetch<E, D, K>(cf.mx, T, H, b, h, z, t0, tid, cur);
    }
#pragma unroll 1
    for (int k = 0; 4 * k < njobs; ++k) {
        if (act) conv_stage<E, D, K>(L[g], cur, tid);
        __syncthreads();
        const int jn = 4 * (k + 1) + g;
        const bool actn = jn < njobs;
        int bn = 0, hn = 0, zn = 0, tn = 0;
        ConvRegs<E, D, K> nxt;
        if (actn) {
            job(jn, bn, hn, zn, tn);
            conv_fetch<E, D, K>(cf.mx, T, H, bn, hn, zn, tn, tid, nxt);
        }
        if (act) conv_rows<E, D, K, false>(cf.mx, T, H, b, h, z, t0, L[g], tid);
        // every thread's stores have reached L2 (the next round's loads too);
        // the flags go out after the barrier, which also frees the LDS
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (threadIdx.x == 0) {
            for (int jb = 4 * k; jb < 4 * k + 4 && jb < njobs; ++jb) {
                if (jb % 3 != 2) continue;   // a unit is complete with its third job
                const int u = r + (jb / 3) * R, n = u / nh, bh = c + 8 * (u % nh);
                const unsigned long long hw =
                    __hip_atomic_load(&cf.hdr[bh], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                unsigned long long extra = 0ull;
                if ((unsigned)(hw >> 32) != cf.epoch || ((unsigned)(hw >> 24) & 0xffu) != me) {
                    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
                    extra = PUB_FLUSHED;
                }
                __hip_atomic_store(&cf.flags[(size_t)bh * NC + n], pub_word(cf.epoch, me) | extra,
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        cur = nxt;
        act = actn;
        b = bn; h = hn; z = zn; t0 = tn;
    }
}

}  // namespace kd
