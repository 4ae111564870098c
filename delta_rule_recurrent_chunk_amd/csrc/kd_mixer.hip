// kd_mixer.hip -- the KronLSTM mixer's pre- and post-processing around the
// Kronecker delta rule (onedev.kr KronLSTM summary, section "어떻게 쓰나"):
//   pre:  q, k, v = L2norm(SiLU(short causal depthwise conv(projection)))
//         f = sigmoid(x)^exp(a_log[h]),  beta = beta_scale * sigmoid(.),  c = sigmoid(.)
//   post: y = o / sqrt(mean o^2 + eps) * w[h] * sigmoid(g)      (per head)
// All three kernels are row-wise and bound by HBM: one pass over their inputs
// and outputs.  A lane owns eight adjacent channels of a row (16 bytes of
// bf16); the D/8 lanes of a row are adjacent, so a row's sum of squares is a
// few DPP lane moves, and a wave reads whole 256-byte rows.
#include <hip/hip_runtime.h>

#include "kd_device.h"

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

// q, k, v: one block per (b, h, tensor) and MIX_CT consecutive tokens.  The
// block stages the raw rows of its tokens and the K - 1 before them, and the
// head's taps, in LDS (one coalesced pass), then each row of D/8 lanes makes
// one output token from K staged rows: convolution, SiLU, the row's sum of
// squares on DPP lane moves, the scale, one 16-byte store per lane.
template <class E, int D, int K>
__global__ __launch_bounds__(MIX_NT) void kd_mixer_conv_kernel(MixPreArgs a, int T, int H) {
    constexpr int LPR = D / 8;                  // lanes per row
    constexpr int TPP = MIX_NT / LPR;           // tokens per pass
    static_assert(MIX_CT % TPP == 0, "a block's tokens are whole passes");
    constexpr int ROWS = MIX_CT + K - 1;
    constexpr int PPR = D * (int)sizeof(E) / 16; // 16-byte pieces per row
    static_assert(D * K <= 4 * MIX_NT, "one float4 of taps per thread");
    __shared__ __align__(16) E st[ROWS * D];
    __shared__ __align__(16) float sw[D * K];   // taps of (h, channel i) at i*K
    const int z = blockIdx.z % 3, b = blockIdx.z / 3, h = blockIdx.y;
    const int t0 = blockIdx.x * MIX_CT;
    const uint32_t rs = (uint32_t)H * D;   // token stride (elements); one batch element fits 2^31 bytes
    const size_t base = (size_t)b * T * rs + (size_t)h * D;
    const E* __restrict__ src = static_cast<const E*>(a.raw[z]) + base;
    E* __restrict__ dst = static_cast<E*>(a.out[z]) + base;
    const int tid = threadIdx.x;
    // stage rows t0 - (K-1) .. t0 + MIX_CT - 1 (zero before the first token;
    // rows past the last token are never read) and the taps: every load is
    // issued before the first LDS store
    constexpr int NPC = (ROWS * PPR + MIX_NT - 1) / MIX_NT;
    uint4 pcs[NPC];
    floatx4 tw = {0.f, 0.f, 0.f, 0.f};
    if (tid < D * K / 4) tw = reinterpret_cast<const floatx4*>(a.conv[z] + (size_t)h * D * K)[tid];
#pragma unroll
    for (int i = 0; i < NPC; ++i) {
        const int x = tid + i * MIX_NT;
        const int r = x / PPR, pc = x % PPR;
        const int t = t0 - (K - 1) + r;
        pcs[i] = make_uint4(0u, 0u, 0u, 0u);
        if (x < ROWS * PPR && t >= 0 && t < T)
            pcs[i] = *reinterpret_cast<const uint4*>(src + (uint32_t)t * rs + pc * (16 / sizeof(E)));
    }
#pragma unroll
    for (int i = 0; i < NPC; ++i) {
        const int x = tid + i * MIX_NT;
        if (x < ROWS * PPR)
            *reinterpret_cast<uint4*>(&st[(x / PPR) * D + (x % PPR) * (16 / sizeof(E))]) = pcs[i];
    }
    if (tid < D * K / 4) reinterpret_cast<floatx4*>(sw)[tid] = tw;
    __syncthreads();
    // taps of this lane's eight channels: wt[e][j] multiplies the token t - (K-1) + j
    const int o8 = tid % LPR, slot = tid / LPR;
    float wt[8][K];
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int j = 0; j < K; ++j) wt[e][j] = sw[(8 * o8 + e) * K + j];
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
            ld8f(&st[(r + j) * D + 8 * o8], x);
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
        st8v_nt(dst + (uint32_t)t * rs + 8 * o8, y);
    }
}

// f, beta, c: elementwise over the B*T token rows.  A lane owns eight
// channels of one head and walks MIX_TT token rows, MIX_TB loads in flight at
// a time; the first lane of a head's row also makes that row's beta and c.
template <class E, int D>
__global__ __launch_bounds__(MIX_NT) void kd_mixer_gate_kernel(MixPreArgs a, int BT, int H) {
    constexpr int LPR = D / 8;
    const int lin = blockIdx.y * MIX_NT + threadIdx.x;
    const int h = lin / LPR, o8 = lin % LPR;
    if (h >= H) return;
    const int t0 = blockIdx.x * MIX_TT;
    const int t1 = min(t0 + MIX_TT, BT);
    const size_t rs = (size_t)H * D;
    const E* __restrict__ src = static_cast<const E*>(a.raw[3]) + (size_t)h * D + 8 * o8;
    E* __restrict__ dst = static_cast<E*>(a.out[3]) + (size_t)h * D + 8 * o8;
    const float ex = __expf(a.a_log[h]);
    for (int tb = t0; tb < t1; tb += MIX_TB) {
        float x[MIX_TB][8], br[MIX_TB], cr[MIX_TB];
#pragma unroll
        for (int i = 0; i < MIX_TB; ++i) {
            const size_t t = (size_t)min(tb + i, t1 - 1);
            ld8f(src + t * rs, x[i]);
            if (o8 == 0) {
                br[i] = a.beta_raw[t * H + h];
                cr[i] = a.c_raw[t * H + h];
            }
        }
#pragma unroll
        for (int i = 0; i < MIX_TB; ++i) {
            const int t = tb + i;
            if (t >= t1) break;
#pragma unroll
            for (int e = 0; e < 8; ++e) x[i][e] = forget_gate(x[i][e], ex);
            st8v_nt(dst + (size_t)t * rs, x[i]);
            if (o8 == 0) {
                a.beta[(size_t)t * H + h] = a.beta_scale * gate_sigmoid(br[i]);
                a.c[(size_t)t * H + h] = gate_sigmoid(cr[i]);
            }
        }
    }
}

template <class E, int D>
__global__ __launch_bounds__(MIX_NT) void kd_mixer_post_kernel(const E* __restrict__ o, const E* __restrict__ g,
                                                               const float* __restrict__ w, float eps,
                                                               E* __restrict__ y, int T, int H) {
    constexpr int LPR = D / 8;
    const int b = blockIdx.z;
    const int lin = blockIdx.y * MIX_NT + threadIdx.x;
    const int h = lin / LPR, o8 = lin % LPR;
    // rows past the last head leave as a whole (all their lanes), so every
    // lane move of row_sum reads lanes of its own, active row
    if (h >= H) return;
    const int t0 = blockIdx.x * MIX_TT;
    const int t1 = min(t0 + MIX_TT, T);
    const uint32_t rs = (uint32_t)H * D;
    const size_t bbase = (size_t)b * T * rs;
    const uint32_t off = (uint32_t)h * D + 8 * o8;
    float wv[8];
    ld8f(w + (size_t)h * D + 8 * o8, wv);
    for (int tb = t0; tb < t1; tb += MIX_TB) {
        float x[MIX_TB][8], gv[MIX_TB][8];
#pragma unroll
        for (int i = 0; i < MIX_TB; ++i) {
            const uint32_t r = (uint32_t)min(tb + i, t1 - 1) * rs + off;
            ld8f(o + bbase + r, x[i]);
            ld8f(g + bbase + r, gv[i]);
        }
#pragma unroll
        for (int i = 0; i < MIX_TB; ++i) {
            const int t = tb + i;
            if (t >= t1) break;
            float ss = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) ss = fmaf(x[i][e], x[i][e], ss);
            const float sc = rsqrtf(row_sum<LPR>(ss) * (1.f / D) + eps);
#pragma unroll
            for (int e = 0; e < 8; ++e) x[i][e] = x[i][e] * sc * wv[e] * gate_sigmoid(gv[i][e]);
            st8v_nt(y + bbase + (uint32_t)t * rs + off, x[i]);
        }
    }
}

// ---------------------------------------------------------------- launchers
// grid limits of the launches (checked by the caller before any launch)
bool mixer_grid_ok(int B, int T, int H) {
    return H <= 65535 && (long long)B * 3 <= 65535 && (long long)B * T <= 0x7fffffffLL;
}

template <class E, int D, int K>
static void launch_conv_t(const MixPreArgs& a, int B, int T, int H, hipStream_t st) {
    // token tiles vary fastest over the grid
    hipLaunchKernelGGL((kd_mixer_conv_kernel<E, D, K>), dim3((unsigned)((T + MIX_CT - 1) / MIX_CT), (unsigned)H,
                                                             (unsigned)(B * 3)),
                       dim3(MIX_NT), 0, st, a, T, H);
}

template <class E, int D>
static hipError_t launch_pre_t(const MixPreArgs& a, int B, int T, int H, int gates, hipStream_t st) {
    switch (a.K) {
    case 1: launch_conv_t<E, D, 1>(a, B, T, H, st); break;
    case 2: launch_conv_t<E, D, 2>(a, B, T, H, st); break;
    case 3: launch_conv_t<E, D, 3>(a, B, T, H, st); break;
    default: launch_conv_t<E, D, 4>(a, B, T, H, st); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !gates) return e;
    const int BT = B * T, rows_per_block = MIX_NT / (D / 8);
    hipLaunchKernelGGL((kd_mixer_gate_kernel<E, D>),
                       dim3((unsigned)((BT + MIX_TT - 1) / MIX_TT), (unsigned)((H + rows_per_block - 1) / rows_per_block)),
                       dim3(MIX_NT), 0, st, a, BT, H);
    return hipGetLastError();
}

// gates = 0: q, k, v only (the forward then makes the gates from their logits)
hipError_t launch_mixer_pre(int bf16, int d, const void* const raw[4], void* const out[4],
                            const float* const conv[3], int K, const float* a_log, const float* beta_raw,
                            const float* c_raw, float beta_scale, float* beta, float* c, int B, int T, int H,
                            int gates, hipStream_t st) {
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
        case 32: return launch_pre_t<__bf16, 32>(a, B, T, H, gates, st);
        case 64: return launch_pre_t<__bf16, 64>(a, B, T, H, gates, st);
        default: return launch_pre_t<__bf16, 128>(a, B, T, H, gates, st);
        }
    }
    switch (d) {
    case 32: return launch_pre_t<float, 32>(a, B, T, H, gates, st);
    case 64: return launch_pre_t<float, 64>(a, B, T, H, gates, st);
    default: return launch_pre_t<float, 128>(a, B, T, H, gates, st);
    }
}

template <class E, int D>
static hipError_t launch_post_t(const void* o, const void* g, const float* w, float eps, void* y, int B, int T,
                                int H, hipStream_t st) {
    const int rows_per_block = MIX_NT / (D / 8);
    hipLaunchKernelGGL((kd_mixer_post_kernel<E, D>),
                       dim3((unsigned)((T + MIX_TT - 1) / MIX_TT), (unsigned)((H + rows_per_block - 1) / rows_per_block),
                            (unsigned)B),
                       dim3(MIX_NT), 0, st,
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
