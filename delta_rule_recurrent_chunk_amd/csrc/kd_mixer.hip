// kd_mixer.hip -- the KronLSTM mixer's pre- and post-processing around the
// Kronecker delta rule (onedev.kr KronLSTM summary, section "어떻게 쓰나"):
//   pre:  q, k, v = L2norm(SiLU(short causal depthwise conv(projection)))
//         f = sigmoid(x)^exp(a_log[h]),  beta = beta_scale * sigmoid(.),  c = sigmoid(.)
//   post: y = o / sqrt(mean o^2 + eps) * w[h] * sigmoid(g)      (per head)
// Both are row-wise and bound by HBM: one pass over their inputs and outputs.
//
// Layout of a launch: a thread owns eight adjacent channels of one head (a
// 16-byte bf16 segment) and walks MIX_TT consecutive tokens, so the
// convolution's window of earlier tokens stays in registers and each raw
// element is read once (plus MIX_KMAX - 1 tokens of history per walk).  The
// D/8 lanes of a row are adjacent, so a wave reads whole rows of adjacent
// heads (one contiguous run per token) and sums a row with lane shuffles.
#include <hip/hip_runtime.h>

#include "kd_device.h"

namespace kd {

constexpr int MIX_TT = 32;     // tokens walked by one thread
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

__device__ __forceinline__ float mix_sigmoid(float x) {
    return __builtin_amdgcn_rcpf(1.f + __expf(-x));
}
// softplus(z) = log(1 + e^z), without overflow for large z
__device__ __forceinline__ float mix_softplus(float z) {
    return fmaxf(z, 0.f) + log1pf(__expf(-fabsf(z)));
}

// sum over the LPR adjacent lanes of a row (LPR a power of two <= 16)
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
#pragma unroll
    for (int m = 1; m < LPR; m <<= 1) x += __shfl_xor(x, m, 64);
    return x;
}

template <class E, int D>
__global__ __launch_bounds__(MIX_NT) void kd_mixer_pre_kernel(MixPreArgs a, int T, int H) {
    constexpr int LPR = D / 8;   // lanes per row
    static_assert(MIX_NT % LPR == 0, "a block holds whole rows");
    const int z = blockIdx.z & 3, b = blockIdx.z >> 2;
    const int lin = blockIdx.x * MIX_NT + threadIdx.x;
    const int h = lin / LPR, o8 = lin % LPR;
    // rows past the last head leave as a whole (all their lanes), so every
    // shuffle below reads lanes of its own, active row
    if (h >= H) return;
    const int t0 = blockIdx.y * MIX_TT;
    const int t1 = min(t0 + MIX_TT, T);
    const uint32_t rs = (uint32_t)H * D;   // token stride (elements); one batch element fits 2^31 bytes
    const size_t bbase = (size_t)b * T * rs;
    const uint32_t off = (uint32_t)h * D + 8 * o8;
    const E* src = static_cast<const E*>(a.raw[z]) + bbase + off;
    E* dst = static_cast<E*>(a.out[z]) + bbase + off;

    if (z == 3) {   // forget gate, and the head's scalar gates on the row's first lane
        const float ex = __expf(a.a_log[h]);
#pragma unroll 4
        for (int t = t0; t < t1; ++t) {
            float x[8];
            ld8f(src + (uint32_t)t * rs, x);
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = __expf(-ex * mix_softplus(-x[e]));
            st8(dst + (uint32_t)t * rs, x);
            if (o8 == 0) {
                const size_t gi = ((size_t)b * T + t) * H + h;
                a.beta[gi] = a.beta_scale * mix_sigmoid(a.beta_raw[gi]);
                a.c[gi] = mix_sigmoid(a.c_raw[gi]);
            }
        }
        return;
    }

    // taps, aligned right: wt[e][j] multiplies the token t - (MIX_KMAX - 1) + j
    const int K = a.K;
    float wt[8][MIX_KMAX];
    const float* cw = a.conv[z] + ((size_t)h * D + 8 * o8) * K;
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int j = 0; j < MIX_KMAX; ++j) {
            const int tau = j - (MIX_KMAX - K);
            wt[e][j] = tau >= 0 ? cw[e * K + tau] : 0.f;
        }
    // the window: raw rows of tokens t-3, t-2, t-1 (zero before the first token)
    float win[MIX_KMAX - 1][8];
#pragma unroll
    for (int j = 0; j < MIX_KMAX - 1; ++j) {
        const int t = t0 - (MIX_KMAX - 1) + j;
        if (t >= 0 && j >= MIX_KMAX - K) {
            ld8f(src + (uint32_t)t * rs, win[j]);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) win[j][e] = 0.f;
        }
    }
#pragma unroll 4
    for (int t = t0; t < t1; ++t) {
        float x[8], y[8];
        ld8f(src + (uint32_t)t * rs, x);
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float acc = wt[e][MIX_KMAX - 1] * x[e];
#pragma unroll
            for (int j = 0; j < MIX_KMAX - 1; ++j) acc = fmaf(wt[e][j], win[j][e], acc);
            y[e] = acc * mix_sigmoid(acc);   // SiLU
            ss = fmaf(y[e], y[e], ss);
        }
#pragma unroll
        for (int j = 0; j + 1 < MIX_KMAX - 1; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e) win[j][e] = win[j + 1][e];
#pragma unroll
        for (int e = 0; e < 8; ++e) win[MIX_KMAX - 2][e] = x[e];
        const float sc = rsqrtf(row_sum<LPR>(ss) + MIX_EPS_L2);
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] *= sc;
        st8(dst + (uint32_t)t * rs, y);
    }
}

template <class E, int D>
__global__ __launch_bounds__(MIX_NT) void kd_mixer_post_kernel(const E* __restrict__ o, const E* __restrict__ g,
                                                               const float* __restrict__ w, float eps,
                                                               E* __restrict__ y, int T, int H) {
    constexpr int LPR = D / 8;
    const int b = blockIdx.z;
    const int lin = blockIdx.x * MIX_NT + threadIdx.x;
    const int h = lin / LPR, o8 = lin % LPR;
    if (h >= H) return;   // whole rows, as in the pre kernel
    const int t0 = blockIdx.y * MIX_TT;
    const int t1 = min(t0 + MIX_TT, T);
    const uint32_t rs = (uint32_t)H * D;
    const size_t bbase = (size_t)b * T * rs;
    const uint32_t off = (uint32_t)h * D + 8 * o8;
    float wv[8];
    ld8f(w + (size_t)h * D + 8 * o8, wv);
#pragma unroll 4
    for (int t = t0; t < t1; ++t) {
        float x[8], gv[8];
        ld8f(o + bbase + (uint32_t)t * rs + off, x);
        ld8f(g + bbase + (uint32_t)t * rs + off, gv);
        float ss = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = fmaf(x[e], x[e], ss);
        const float sc = rsqrtf(row_sum<LPR>(ss) * (1.f / D) + eps);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = x[e] * sc * wv[e] * mix_sigmoid(gv[e]);
        st8(y + bbase + (uint32_t)t * rs + off, x);
    }
}

// ---------------------------------------------------------------- launchers
static dim3 mix_grid(int B, int T, int H, int D, int zmul) {
    const int rows_per_block = MIX_NT / (D / 8);
    return dim3((unsigned)((H + rows_per_block - 1) / rows_per_block), (unsigned)((T + MIX_TT - 1) / MIX_TT),
                (unsigned)(B * zmul));
}

// grid limits of the two launches (checked by the caller before any launch)
bool mixer_grid_ok(int B, int T) {
    return (T + MIX_TT - 1) / MIX_TT <= 65535 && (long long)B * 4 <= 65535;
}

template <class E, int D>
static hipError_t launch_pre_t(const MixPreArgs& a, int B, int T, int H, hipStream_t st) {
    hipLaunchKernelGGL((kd_mixer_pre_kernel<E, D>), mix_grid(B, T, H, D, 4), dim3(MIX_NT), 0, st, a, T, H);
    return hipGetLastError();
}

hipError_t launch_mixer_pre(int bf16, int d, const void* const raw[4], void* const out[4],
                            const float* const conv[3], int K, const float* a_log, const float* beta_raw,
                            const float* c_raw, float beta_scale, float* beta, float* c, int B, int T, int H,
                            hipStream_t st) {
    if (T == 0) return hipSuccess;
    MixPreArgs a;
    for (int i = 0; i < 4; ++i) { a.raw[i] = raw[i]; a.out[i] = out[i]; }
    for (int i = 0; i < 3; ++i) a.conv[i] = conv[i];
    a.a_log = a_log;
    a.beta_raw = beta_raw;
    a.c_raw = c_raw;
    a.beta = beta;
    a.c = c;
    a.beta_scale = beta_scale;
    a.K = K;
    if (bf16) {
        switch (d) {
        case 32: return launch_pre_t<__bf16, 32>(a, B, T, H, st);
        case 64: return launch_pre_t<__bf16, 64>(a, B, T, H, st);
        default: return launch_pre_t<__bf16, 128>(a, B, T, H, st);
        }
    }
    switch (d) {
    case 32: return launch_pre_t<float, 32>(a, B, T, H, st);
    case 64: return launch_pre_t<float, 64>(a, B, T, H, st);
    default: return launch_pre_t<float, 128>(a, B, T, H, st);
    }
}

template <class E, int D>
static hipError_t launch_post_t(const void* o, const void* g, const float* w, float eps, void* y, int B, int T,
                                int H, hipStream_t st) {
    hipLaunchKernelGGL((kd_mixer_post_kernel<E, D>), mix_grid(B, T, H, D, 1), dim3(MIX_NT), 0, st,
                       (const E*)o, (const E*)g, w, eps, (E*)y, T, H);
    return hipGetLastError();
}

hipError_t launch_mixer_post(int bf16, int d, const void* o, const void* g, const float* w, float eps, void* y,
                             int B, int T, int H, hipStream_t st) {
    if (T == 0) return hipSuccess;
    if (bf16) {
        switch (d) {
        case 32: return launch_post_t<__bf16, 32>(o, g, w, eps, y, B, T, H, st);
        case 64: return launch_post_t<__bf16, 64>(o, g, w, eps, y, B, T, H, st);
        default: return launch_post_t<__bf16, 128>(o, g, w, eps, y, B, T, H, st);
        }
    }
    switch (d) {
    case 32: return launch_post_t<float, 32>(o, g, w, eps, y, B, T, H, st);
    case 64: return launch_post_t<float, 64>(o, g, w, eps, y, B, T, H, st);
    default: return launch_post_t<float, 128>(o, g, w, eps, y, B, T, H, st);
    }
}

}  // namespace kd
