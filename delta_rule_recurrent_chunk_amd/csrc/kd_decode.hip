// kd_decode.hip -- token-by-token recurrence on a carried state (serving), gfx950.
//
// For each (b, h) and each of the T tokens, in order (onedev.kr KronLSTM
// summary, sections "어떻게 동작하나" and "어떻게 쓰나"):
//     Sbar = S diag(f_t);  r = v_t^T Sbar k_t;  S = Sbar + (c_t - beta_t r) v_t k_t^T;
//     o_t = S q_t = Sbar q_t + (c_t - beta_t r) v_t (k_t . q_t).
// No chunking: T is small in decoding (typically 1), and the state (d x d
// fp32) is the only large operand, so the kernel is bound by reading and
// writing it once per call.
//
// One workgroup of 256 threads per (b, h).  The state lives in registers for
// the whole call.  It is read and written in whole 4 KiB runs: load x of
// thread t is the 16 bytes at float offset 4 (256 x + t), so one load
// instruction of a wave covers 1 KiB of contiguous memory.  Thread t then holds
// four adjacent columns 4 (t mod RL) .. of the rows (256 x + t) / RL, x < NV,
// with RL = D / 4 lanes per row; a row's sums over its columns are
// reductions over those RL adjacent lanes.
#include "kd_device.h"

namespace kd {

template <class E, int D>
__global__ __launch_bounds__(256) void kd_decode_kernel(
    const E* __restrict__ q, const E* __restrict__ k, const E* __restrict__ v, const E* __restrict__ f,
    const float* __restrict__ beta, const float* __restrict__ cc, const float* S_in,
    E* __restrict__ o, float* S_out, const int* __restrict__ cu, int T_, int H)
{
    constexpr int NT = 256;
    constexpr int RL = D / 4;             // lanes per state row
    constexpr int RPX = NT / RL;          // rows per load step
    constexpr int NV = D * D / (4 * NT);  // float4 per thread
    __shared__ float sq[D], sk[D], sf[D], sv[D];
    __shared__ float red[2][NT / 64];     // per-wave partials of r and k.q
    __shared__ float bc[2];               // beta_t, c_t

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int bh = blockIdx.x, b = bh / H, h = bh % H;
    const int i0 = tid / RL, j0 = 4 * (tid % RL);   // first row, first column
    // (b, h) walks tokens tok0 .. tok0 + T - 1: T_ tokens each, or, for packed
    // sequences, those between the offsets cu[b] and cu[b + 1] (clamped to
    // [0, T_], so bad offsets cannot reach outside the tensors)
    int tok0 = b * T_, T = T_;
    if (cu) {
        tok0 = min(max(cu[b], 0), T_);
        T = min(max(cu[b + 1], tok0), T_) - tok0;
    }
    const bool lead = tid % RL == 0;                  // counts its rows once

    floatx4 S[NV];   // S[x] = S[i0 + RPX x][j0 .. j0 + 3]
    const size_t sbase = (size_t)bh * D * D + 4 * (size_t)tid;
#pragma unroll
    for (int x = 0; x < NV; ++x)
        S[x] = S_in ? *reinterpret_cast<const floatx4*>(S_in + sbase + 4 * (size_t)NT * x) : floatx4{0.f, 0.f, 0.f, 0.f};

    for (int t = 0; t < T; ++t) {
        const size_t row = ((size_t)tok0 + t) * H + h;   // token (b, t, h)
        if (tid < D) {
            sq[tid] = (float)q[row * D + tid];
            sk[tid] = (float)k[row * D + tid];
            sf[tid] = (float)f[row * D + tid];
            sv[tid] = (float)v[row * D + tid];
        }
        if (tid == 0) { bc[0] = beta[row]; bc[1] = cc[row]; }
        __syncthreads();
        // Sbar = S diag(f); y = Sbar k and z = Sbar q of each held row, over its RL lanes
        const floatx4 fj = *reinterpret_cast<const floatx4*>(&sf[j0]);
        const floatx4 kj = *reinterpret_cast<const floatx4*>(&sk[j0]);
        const floatx4 qj = *reinterpret_cast<const floatx4*>(&sq[j0]);
        float y[NV], z[NV];
#pragma unroll
        for (int x = 0; x < NV; ++x) {
            S[x] = S[x] * fj;
            y[x] = S[x][0] * kj[0] + S[x][1] * kj[1] + S[x][2] * kj[2] + S[x][3] * kj[3];
            z[x] = S[x][0] * qj[0] + S[x][1] * qj[1] + S[x][2] * qj[2] + S[x][3] * qj[3];
        }
#pragma unroll
        for (int m = 1; m < RL; m <<= 1)
#pragma unroll
            for (int x = 0; x < NV; ++x) {
                y[x] += __shfl_xor(y[x], m, 64);
                z[x] += __shfl_xor(z[x], m, 64);
            }
        // r = sum_i v_i y_i (each row once, on its lead lane) and k.q
        float pr = 0.f;
        if (lead)
#pragma unroll
            for (int x = 0; x < NV; ++x) pr = fmaf(sv[i0 + RPX * x], y[x], pr);
        float pk = (tid < D) ? sk[tid] * sq[tid] : 0.f;
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) {
            pr += __shfl_xor(pr, m, 64);
            pk += __shfl_xor(pk, m, 64);
        }
        if (lane == 0) { red[0][w] = pr; red[1][w] = pk; }
        __syncthreads();
        float r = 0.f, kq = 0.f;
#pragma unroll
        for (int ww = 0; ww < NT / 64; ++ww) { r += red[0][ww]; kq += red[1][ww]; }
        const float a = bc[1] - bc[0] * r;
        // S = Sbar + a v k^T;  o = Sbar q + a v (k.q)
#pragma unroll
        for (int x = 0; x < NV; ++x) {
            const float av = a * sv[i0 + RPX * x];
            S[x] = S[x] + av * kj;
            if (lead) o[row * D + i0 + RPX * x] = (E)(z[x] + av * kq);
        }
        __syncthreads();   // the token vectors and partials are reused
    }
    if (S_out) {   // NULL when a caller does not want the final state
#pragma unroll
        for (int x = 0; x < NV; ++x) st4_nt(S_out + sbase + 4 * (size_t)NT * x, S[x]);
    }
}

// cu: NULL, or the B + 1 offsets of packed sequences (device memory)
hipError_t launch_decode(int bf16, int d, const void* q, const void* k, const void* v, const void* f,
                         const float* beta, const float* c, const float* S_in, void* o, float* S_out,
                         int B, int T, int H, hipStream_t st, const int* cu)
{
#define KD_DEC(E, D)                                                                                     \
    hipLaunchKernelGGL((kd_decode_kernel<E, D>), dim3((unsigned)(B * H)), dim3(256), 0, st, (const E*)q,  \
                       (const E*)k, (const E*)v, (const E*)f, beta, c, S_in, (E*)o, S_out, cu, T, H)
    if (bf16) {
        switch (d) {
        case 32: KD_DEC(__bf16, 32); break;
        case 64: KD_DEC(__bf16, 64); break;
        case 128: KD_DEC(__bf16, 128); break;
        default: return hipErrorInvalidValue;
        }
    } else {
        switch (d) {
        case 32: KD_DEC(float, 32); break;
        case 64: KD_DEC(float, 64); break;
        case 128: KD_DEC(float, 128); break;
        default: return hipErrorInvalidValue;
        }
    }
#undef KD_DEC
    return hipGetLastError();
}

}  // namespace kd
