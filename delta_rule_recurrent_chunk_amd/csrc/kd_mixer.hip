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
#include "kd_mixer_conv.h"

namespace kd {

// q, k, v: one block per (b, h, tensor) and MIX_CT consecutive tokens
// (conv_fetch, conv_stage, conv_rows).
template <class E, int D, int K>
__global__ __launch_bounds__(MIX_NT) void kd_mixer_conv_kernel(MixPreArgs a, int T, int H) {
    __shared__ ConvLds<E, D, K> L;
    const int b = blockIdx.z / 3, h = blockIdx.y, z = blockIdx.z % 3, t0 = blockIdx.x * MIX_CT;
    ConvRegs<E, D, K> R;
    conv_fetch<E, D, K>(a, T, H, b, h, z, t0, threadIdx.x, R);
    conv_stage<E, D, K>(L, R, threadIdx.x);
    __syncthreads();
    conv_rows<E, D, K, true>(a, T, H, b, h, z, t0, L, threadIdx.x);
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
