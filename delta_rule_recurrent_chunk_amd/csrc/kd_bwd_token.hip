// kd_bwd_token.hip -- exact fp32 backward by the per-token recurrence (d = 128), gfx950.
//
// The rule, token by token (onedev.kr KronLSTM summary, sections "어떻게
// 동작하나" and "어떻게 쓰나"):
//     Sbar_t = S_{t-1} diag(f_t),  r_t = v_t^T Sbar_t k_t,  e_t = c_t - beta_t r_t,
//     S_t = Sbar_t + e_t v_t k_t^T,  o_t = S_t q_t.
// Its reverse mode, with G the adjoint of S_t (dS_T at the end, plus what the
// later tokens send back), for t = T-1 .. 0:
//     G    += dO_t q_t^T                  dq_t = S_t^T dO_t
//     de_t  = v_t^T G k_t                 dc_t = de_t,  dbeta_t = -r_t de_t,  dr_t = -beta_t de_t
//     dv_t  = e_t G k_t + dr_t Sbar_t k_t
//     dk_t  = (e_t G + dr_t Sbar_t)^T v_t
//     Gbar  = G + dr_t v_t k_t^T          df_t = column sums of Gbar .* S_{t-1}
//     G     = Gbar diag(f_t)              (and dS0 = G after token 0)
// The gate enters only as a product, so every f in [0, 1] is exact.
//
// The chunked backward keeps its fp32 operands in LDS only up to d = 64; at
// d = 128 fp32 is a diagnostic precision, so it takes this form: one
// workgroup of 256 threads per (b, h), the state and its adjoint in
// registers, sequential in t.  The states the reverse pass needs are
// recomputed by chunks of 64 tokens: a first pass stores the state entering
// every chunk (ck), then for each chunk from the last one the states entering
// its tokens are recomputed into tb and the chunk's tokens are reversed.
// Every thread reads back only what it wrote itself, so ck and tb need no
// synchronisation between threads.
//
// Thread layout (as the decode kernel): thread t holds four adjacent columns
// 4 (t mod RL) .. of the rows t / RL + RPX x, x < NV, RL = D / 4 lanes per
// row; a row sum is a reduction over RL adjacent lanes, a column sum one over
// the row groups of a wave (lane xor RL, ...) and then over the waves (LDS).
#include "kd_device.h"

namespace kd {

namespace {

constexpr int TOK_NT = 256;

__device__ __forceinline__ float dot4(floatx4 a, floatx4 b) {
    return a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3];
}
__device__ __forceinline__ floatx4 ld4(const float* p) { return *reinterpret_cast<const floatx4*>(p); }

// sum over the RL adjacent lanes that hold one row
template <int RL>
__device__ __forceinline__ float tok_row_sum(float x) {
#pragma unroll
    for (int m = 1; m < RL; m <<= 1) x += __shfl_xor(x, m, 64);
    return x;
}
__device__ __forceinline__ float tok_wave_sum(float x) {
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) x += __shfl_xor(x, m, 64);
    return x;
}

// Token vectors of one step, staged in LDS.
template <int D>
struct TokLds {
    float q[D], k[D], v[D], f[D], g[D];   // g: dO
    float bc[2];                          // beta_t, c_t
    float red[2][TOK_NT / 64];            // per-wave partials of r and de
    floatx4 col[3][TOK_NT / 64][D / 4];   // per-wave column partials of dq, dk, df
};

// One forward step of the state S (held as in the layout above) over token
// `row`: S = Sbar + (c - beta r) v k^T.  Three barriers; the LDS is free
// again when it returns.
template <int D>
__device__ __forceinline__ void tok_fwd_step(floatx4 (&S)[D * D / (4 * TOK_NT)], TokLds<D>& L,
                                             const float* __restrict__ k, const float* __restrict__ v,
                                             const float* __restrict__ f, const float* __restrict__ beta,
                                             const float* __restrict__ cc, size_t row, int tid)
{
    constexpr int RL = D / 4, RPX = TOK_NT / RL, NV = D * D / (4 * TOK_NT);
    const int i0 = tid / RL, j0 = 4 * (tid % RL), lane = tid & 63, w = tid >> 6;
    if (tid < D) {
        L.k[tid] = k[row * D + tid];
        L.v[tid] = v[row * D + tid];
        L.f[tid] = f[row * D + tid];
    }
    if (tid == 0) { L.bc[0] = beta[row]; L.bc[1] = cc[row]; }
    __syncthreads();
    const floatx4 fj = ld4(&L.f[j0]), kj = ld4(&L.k[j0]);
    float y[NV];
#pragma unroll
    for (int x = 0; x < NV; ++x) {
        S[x] = S[x] * fj;
        y[x] = tok_row_sum<RL>(dot4(S[x], kj));
    }
    float pr = 0.f;
    if (tid % RL == 0)
#pragma unroll
        for (int x = 0; x < NV; ++x) pr = fmaf(L.v[i0 + RPX * x], y[x], pr);
    pr = tok_wave_sum(pr);
    if (lane == 0) L.red[0][w] = pr;
    __syncthreads();
    float r = 0.f;
#pragma unroll
    for (int ww = 0; ww < TOK_NT / 64; ++ww) r += L.red[0][ww];
    const float e = L.bc[1] - L.bc[0] * r;
#pragma unroll
    for (int x = 0; x < NV; ++x) S[x] = S[x] + (e * L.v[i0 + RPX * x]) * kj;
    __syncthreads();
}

}  // namespace

template <int D>
__global__ __launch_bounds__(TOK_NT) void kd_bwd_token_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ f, const float* __restrict__ beta, const float* __restrict__ cc,
    const float* __restrict__ S0, const float* __restrict__ dO, const float* __restrict__ dST,
    float* __restrict__ dq, float* __restrict__ dk, float* __restrict__ dv, float* __restrict__ df,
    float* __restrict__ dbeta, float* __restrict__ dc, float* __restrict__ dS0,
    float* __restrict__ ck, float* __restrict__ tb, int T, int H)
{
    constexpr int RL = D / 4, RPX = TOK_NT / RL, NV = D * D / (4 * TOK_NT), NW = TOK_NT / 64;
    __shared__ TokLds<D> L;

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int bh = blockIdx.x, b = bh / H, h = bh % H;
    const int i0 = tid / RL, j0 = 4 * (tid % RL);
    const bool lead = tid % RL == 0;
    const int NC = (T + CH - 1) / CH;
    const size_t DD = (size_t)D * D;
    const size_t sb = 4 * (size_t)tid;   // this thread's first float of a d x d block
    float* ckb = ck + (size_t)bh * NC * DD;
    float* tbb = tb + (size_t)bh * CH * DD;
    auto tok = [&](int t) { return ((size_t)b * T + t) * H + h; };

    // pass 1: the state entering every chunk
    floatx4 S[NV];
#pragma unroll
    for (int x = 0; x < NV; ++x)
        S[x] = S0 ? ld4(S0 + (size_t)bh * DD + sb + 4 * (size_t)TOK_NT * x) : floatx4{0.f, 0.f, 0.f, 0.f};
    for (int n = 0; n < NC; ++n) {
#pragma unroll
        for (int x = 0; x < NV; ++x) st4(ckb + n * DD + sb + 4 * (size_t)TOK_NT * x, S[x]);
        if (n + 1 < NC)
            for (int t = n * CH; t < (n + 1) * CH; ++t) tok_fwd_step<D>(S, L, k, v, f, beta, cc, tok(t), tid);
    }

    // pass 2: chunks in reverse; the adjoint G of the state in registers
    floatx4 G[NV];
#pragma unroll
    for (int x = 0; x < NV; ++x)
        G[x] = dST ? ld4(dST + (size_t)bh * DD + sb + 4 * (size_t)TOK_NT * x) : floatx4{0.f, 0.f, 0.f, 0.f};
    for (int n = NC - 1; n >= 0; --n) {
        const int t0 = n * CH, t1 = min(T, t0 + CH);
        // the states entering the chunk's tokens
#pragma unroll
        for (int x = 0; x < NV; ++x) S[x] = ld4(ckb + n * DD + sb + 4 * (size_t)TOK_NT * x);
        for (int t = t0; t < t1; ++t) {
#pragma unroll
            for (int x = 0; x < NV; ++x) st4(tbb + (t - t0) * DD + sb + 4 * (size_t)TOK_NT * x, S[x]);
            if (t + 1 < t1) tok_fwd_step<D>(S, L, k, v, f, beta, cc, tok(t), tid);
        }
        for (int t = t1 - 1; t >= t0; --t) {
            const size_t row = tok(t);
            floatx4 P[NV];   // S_{t-1}
#pragma unroll
            for (int x = 0; x < NV; ++x) P[x] = ld4(tbb + (t - t0) * DD + sb + 4 * (size_t)TOK_NT * x);
            if (tid < D) {
                L.q[tid] = q[row * D + tid];
                L.k[tid] = k[row * D + tid];
                L.v[tid] = v[row * D + tid];
                L.f[tid] = f[row * D + tid];
                L.g[tid] = dO[row * D + tid];
            }
            if (tid == 0) { L.bc[0] = beta[row]; L.bc[1] = cc[row]; }
            __syncthreads();
            const floatx4 fj = ld4(&L.f[j0]), kj = ld4(&L.k[j0]), qj = ld4(&L.q[j0]);
            // y = Sbar k and g = G k per row, with G += dO q^T first
            float y[NV], g[NV];
#pragma unroll
            for (int x = 0; x < NV; ++x) {
                G[x] = G[x] + L.g[i0 + RPX * x] * qj;
                y[x] = tok_row_sum<RL>(dot4(P[x] * fj, kj));
                g[x] = tok_row_sum<RL>(dot4(G[x], kj));
            }
            float pr = 0.f, pg = 0.f;
            if (lead)
#pragma unroll
                for (int x = 0; x < NV; ++x) {
                    const float vi = L.v[i0 + RPX * x];
                    pr = fmaf(vi, y[x], pr);
                    pg = fmaf(vi, g[x], pg);
                }
            pr = tok_wave_sum(pr);
            pg = tok_wave_sum(pg);
            if (lane == 0) { L.red[0][w] = pr; L.red[1][w] = pg; }
            __syncthreads();
            float r = 0.f, de = 0.f;
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) { r += L.red[0][ww]; de += L.red[1][ww]; }
            const float bt = L.bc[0], e = L.bc[1] - bt * r, dr = -bt * de;
            if (lead)
#pragma unroll
                for (int x = 0; x < NV; ++x) dv[row * D + i0 + RPX * x] = e * g[x] + dr * y[x];
            if (tid == 0) { dc[row] = de; dbeta[row] = -r * de; }
            // column partials of dq, dk, df; G <- Gbar diag(f)
            floatx4 aq = {0.f, 0.f, 0.f, 0.f}, ak = aq, af = aq;
#pragma unroll
            for (int x = 0; x < NV; ++x) {
                const float vi = L.v[i0 + RPX * x], oi = L.g[i0 + RPX * x];
                const floatx4 Sb = P[x] * fj;
                aq = aq + oi * (Sb + (e * vi) * kj);
                ak = ak + vi * (e * G[x] + dr * Sb);
                const floatx4 Gb = G[x] + (dr * vi) * kj;
                af = af + Gb * P[x];
                G[x] = Gb * fj;
            }
#pragma unroll
            for (int m = RL; m < 64; m <<= 1)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    aq[c] += __shfl_xor(aq[c], m, 64);
                    ak[c] += __shfl_xor(ak[c], m, 64);
                    af[c] += __shfl_xor(af[c], m, 64);
                }
            if (lane < RL) { L.col[0][w][lane] = aq; L.col[1][w][lane] = ak; L.col[2][w][lane] = af; }
            __syncthreads();
            if (tid < D) {
                const int jl = tid >> 2, c = tid & 3;
                float sq = 0.f, sk = 0.f, sf = 0.f;
#pragma unroll
                for (int ww = 0; ww < NW; ++ww) {
                    sq += L.col[0][ww][jl][c];
                    sk += L.col[1][ww][jl][c];
                    sf += L.col[2][ww][jl][c];
                }
                dq[row * D + tid] = sq;
                dk[row * D + tid] = sk;
                df[row * D + tid] = sf;
            }
        }
    }
    if (dS0) {
#pragma unroll
        for (int x = 0; x < NV; ++x) st4_nt(dS0 + (size_t)bh * DD + sb + 4 * (size_t)TOK_NT * x, G[x]);
    }
}

// Workspace of the per-token backward: the state entering each chunk, per
// (b, h, chunk), then the states entering one chunk's tokens, per (b, h).
size_t bwd_token_ws_states(int d, int B, int T, int H, size_t* tb_off) {
    const size_t nc = (size_t)(T + CH - 1) / CH;
    const size_t dd = (size_t)d * d * sizeof(float);
    auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
    *tb_off = up((size_t)B * H * nc * dd);
    return *tb_off + (nc ? up((size_t)B * H * CH * dd) : 0);
}

hipError_t launch_bwd_token(int d, const void* q, const void* k, const void* v, const void* f,
                            const float* beta, const float* c, const float* S0, const void* dO,
                            const float* dST, void* dq, void* dk, void* dv, void* df, float* dbeta,
                            float* dc, float* dS0, void* ws, int B, int T, int H, hipStream_t st)
{
    if (d != 128) return hipErrorInvalidValue;
    size_t tb_off = 0;
    bwd_token_ws_states(d, B, T, H, &tb_off);
    float* ck = static_cast<float*>(ws);
    float* tb = reinterpret_cast<float*>(static_cast<char*>(ws) + tb_off);
    hipLaunchKernelGGL((kd_bwd_token_kernel<128>), dim3((unsigned)(B * H)), dim3(TOK_NT), 0, st,
                       (const float*)q, (const float*)k, (const float*)v, (const float*)f, beta, c, S0,
                       (const float*)dO, dST, (float*)dq, (float*)dk, (float*)dv, (float*)df, dbeta, dc, dS0,
                       ck, tb, T, H);
    return hipGetLastError();
}

}  // namespace kd
