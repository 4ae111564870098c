// kd_api.hip -- the C ABI declared in include/kron_delta.h: argument checks,
// workspace sizing and kernel dispatch on the caller's stream.  No
// allocation, no synchronisation.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include <atomic>

#include "kron_delta.h"

namespace kd {
struct FwdCkpt;
hipError_t launch_fwd(int bf16, int d, const void* q, const void* k, const void* v, const void* f,
                      const float* beta, const float* c, const float* S0, void* o, float* ST,
                      const FwdCkpt* ck, const int* cu, int B, int T, int H, hipStream_t st);
hipError_t launch_bwd(int bf16, int d, const void* q, const void* k, const void* v, const void* f,
                      const float* beta, const float* c, const float* S0, const void* dO,
                      const float* dST, void* dq, void* dk, void* dv, void* df, float* dbeta,
                      float* dc, float* dS0, void* ws, int B, int T, int H, int recompute,
                      hipStream_t st);
hipError_t launch_fwd_train(int bf16, int d, const void* q, const void* k, const void* v, const void* f,
                            const float* beta, const float* c, const float* S0, void* o, float* ST,
                            void* ws, int B, int T, int H, hipStream_t st);
size_t bwd_workspace_bytes(int bf16, int d, int B, int T, int H);
hipError_t launch_gdn2(const void* q, const void* k, const void* v, const void* alpha, const void* b,
                       const void* w, const float* S0, void* o, float* ST, int B, int T, int H,
                       hipStream_t st);
hipError_t launch_decode(int bf16, int d, const void* q, const void* k, const void* v, const void* f,
                         const float* beta, const float* c, const float* S_in, void* o, float* S_out,
                         int B, int T, int H, hipStream_t st, const int* cu = nullptr);
bool mixer_grid_ok(int B, int T, int H);
hipError_t launch_mixer_pre(int bf16, int d, const void* const raw[4], void* const out[4],
                            const float* const conv[3], int K, const float* a_log, const float* beta_raw,
                            const float* c_raw, float beta_scale, float* beta, float* c, int B, int T, int H,
                            int gates, hipStream_t st);
hipError_t launch_fwd16_gates(const void* q, const void* k, const void* v, const void* f_raw,
                              const float* beta_raw, const float* c_raw, const float* a_log, float beta_scale,
                              const void* og, const float* norm_w, float norm_eps,
                              const float* S0, void* o, float* ST, int B, int T, int H, hipStream_t st);
hipError_t launch_mixer_post(int bf16, int d, const void* o, const void* g, const float* w, float eps, void* y,
                             int B, int T, int H, hipStream_t st);
size_t fwd16_split_ws_bytes(int B, int T, int H);
int fwd16_feed_workers(int BH);
hipError_t launch_fwd16_mixer_fed(const void* const raw[3], void* const out[3], const float* const conv[3],
                                  const void* f_raw, const float* beta_raw, const float* c_raw,
                                  const float* a_log, float beta_scale, const void* og, const float* norm_w,
                                  float norm_eps, const float* S0, void* o, float* ST, void* hw, int nwork,
                                  int B, int T, int H, hipStream_t st);
void set_bwd_wait_polls(unsigned polls);
size_t bwd_status_offset(int bf16, int d, int B, int T, int H);
hipError_t launch_fwd16_split(const void* q, const void* k, const void* v, const void* f, const float* beta,
                              const float* c, const float* S0, void* o, float* ST, void* ws, int B, int T,
                              int H, hipStream_t st);
}  // namespace kd

namespace {

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void* p, size_t bytes) {
    Range r;
    r.lo = (uintptr_t)p;
    r.hi = r.lo + bytes;
    return r;
}

bool overlap(Range a, Range b) {
    if (a.lo == a.hi || b.lo == b.hi || a.lo == 0 || b.lo == 0) return false;
    return a.lo < b.hi && b.lo < a.hi;
}

bool misaligned(const void* p) { return p != nullptr && ((uintptr_t)p & 15u) != 0; }

// fp32_d128: whether the entry point supports fp32 at d = 128 (decode only)
kd_status check_desc(const kd_desc* d, bool fp32_d128 = false) {
    if (!d) return KD_ERR_NULL;
    if (d->dtype != KD_F32 && d->dtype != KD_BF16) return KD_ERR_DTYPE;
    if (d->B < 1 || d->H < 1 || d->T < 0) return KD_ERR_SHAPE;
    if (d->dk != d->dv) return KD_ERR_SHAPE;
    if (d->dk != 32 && d->dk != 64 && d->dk != 128) return KD_ERR_SHAPE;
    if (d->dtype == KD_F32 && d->dk == 128 && !fp32_d128) return KD_ERR_DTYPE;
    if ((int64_t)d->B * (int64_t)d->H > (int64_t)INT32_MAX) return KD_ERR_SHAPE;
    // kernels address one batch element's [T, H, d] tensor with 32-bit byte offsets
    const int64_t es = d->dtype == KD_BF16 ? 2 : 4;
    if ((int64_t)d->T * d->H * d->dk * es > (int64_t)INT32_MAX) return KD_ERR_SHAPE;
    return KD_OK;
}

size_t esize(const kd_desc* d) { return d->dtype == KD_BF16 ? 2 : 4; }

size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }

// The mixer forward's workspace: q, k, v, f (desc dtype), beta, c (fp32), the
// read-out o, and the hand-off words of the one-launch form (8 bytes per
// head and per (head, 64-token chunk)), each part 256-byte aligned.
struct MixWs {
    size_t x[4], beta, c, o, hw, total;
};
MixWs mixer_ws(const kd_desc* d) {
    const size_t ntok = (size_t)d->B * d->T * d->H;
    const size_t xb = up256(ntok * d->dk * esize(d)), gb = up256(ntok * sizeof(float));
    const size_t bh = (size_t)d->B * d->H, nc = ((size_t)d->T + 63) / 64;
    MixWs w;
    for (int i = 0; i < 4; ++i) w.x[i] = i * xb;
    w.beta = 4 * xb;
    w.c = w.beta + gb;
    w.o = w.c + gb;
    w.hw = w.o + xb;
    w.total = w.hw + up256(8 * (bh + bh * nc));
    return w;
}

// checks of the mixer's parameters: pre (conv, a_log) and/or post (norm_w)
kd_status check_mixer(const kd_desc* d, const kd_mixer_params* p, bool pre, bool post) {
    if (!p) return KD_ERR_NULL;
    if (!kd::mixer_grid_ok(d->B, d->T, d->H)) return KD_ERR_SHAPE;
    if (pre) {
        if (!p->conv_q || !p->conv_k || !p->conv_v || !p->a_log) return KD_ERR_NULL;
        if (p->conv_size < 1 || p->conv_size > 4) return KD_ERR_SHAPE;
        const void* ptrs[] = {p->conv_q, p->conv_k, p->conv_v, p->a_log};
        for (const void* q : ptrs)
            if (misaligned(q)) return KD_ERR_ALIGN;
    }
    if (post) {
        if (!p->norm_w) return KD_ERR_NULL;
        if (misaligned(p->norm_w)) return KD_ERR_ALIGN;
        if (!(p->norm_eps >= 0.f)) return KD_ERR_SHAPE;
    }
    return KD_OK;
}

// The allocation-free backward's workspace: one fixed array in device memory,
// which every GPU the library runs on holds until the process ends.  Host
// code never uses the array's name as an address (on the host it is a
// stand-in): the device address comes from hipGetSymbolAddress, once per
// device.
constexpr size_t kScratchBytes = KRON_DELTA_NOALLOC_SCRATCH_BYTES;

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
// Device address of `scratch` on the current device, looked up the first time
// the device is seen (null when the lookup fails).
void* scratch_address() {
    static std::atomic<void*> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    void* p = cache[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        void* q = nullptr;
        if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr) return nullptr;
        cache[dev].store(q, std::memory_order_release);
        p = q;
    }
    return p;
}
}  // namespace

extern "C" {

int kron_delta_abi_version(void) { return KRON_DELTA_ABI_VERSION; }

const char* kron_delta_status_string(int s) {
    switch (s) {
    case KD_OK: return "ok";
    case KD_ERR_NULL: return "a required pointer is NULL";
    case KD_ERR_SHAPE: return "unsupported shape (need B,H>=1, T>=0, dk==dv in {32,64,128})";
    case KD_ERR_DTYPE: return "unsupported dtype for this call (bf16: d in {32,64,128}; fp32: d in {32,64}, and 128 in the forward, decode, backward and training pair)";
    case KD_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case KD_ERR_WORKSPACE: return "workspace missing or too small";
    case KD_ERR_LAUNCH: return "kernel launch failed";
    case KD_ERR_ALIAS: return "an output overlaps an input";
    case KD_ERR_TIMEOUT:
        return "a chunk worker of the backward gave up waiting for the reverse sweep (its gradients are NaN)";
    case KD_ERR_SCRATCH:
        return "the problem needs more workspace than kron_delta_bwd_noalloc's fixed scratch "
               "(KRON_DELTA_NOALLOC_SCRATCH_BYTES = 64 MiB)";
    default: return "unknown status";
    }
}

// Workspace of kron_delta_fwd: the few-heads path (bf16, d = 128, at most
// KRON_DELTA_FWD_SPLIT_MAX_HEADS heads B*H, T > 0) takes one hand-off image
// per (b, h, chunk); 0 otherwise.
static size_t fwd_ws_bytes(const kd_desc* d) {
    if (d->dtype != KD_BF16 || d->dk != 128 || d->dv != 128 || d->T <= 0) return 0;
    if ((long long)d->B * d->H > KRON_DELTA_FWD_SPLIT_MAX_HEADS) return 0;
    return kd::fwd16_split_ws_bytes(d->B, d->T, d->H);
}

size_t kron_delta_workspace_bytes(const kd_desc* d, int which) {
    if (check_desc(d, true) != KD_OK) return 0;
    switch (which) {
    case KD_WS_FWD: return fwd_ws_bytes(d);
    case KD_WS_BWD: return kd::bwd_workspace_bytes(d->dtype == KD_BF16, d->dk, d->B, d->T, d->H);
    case KD_WS_MIXER: return mixer_ws(d).total;
    default: return 0;
    }
}

kd_status kron_delta_fwd(const kd_desc* d, const void* q, const void* k, const void* v,
                         const void* f, const float* beta, const float* c, const float* S0,
                         void* o, float* ST, void* ws, size_t ws_bytes, void* stream) {
    kd_status st = check_desc(d, true);
    if (st != KD_OK) return st;
    const size_t ntok = (size_t)d->B * d->T * d->H;
    const size_t xb = ntok * d->dk * esize(d);
    const size_t gb = ntok * sizeof(float);
    const size_t sb = (size_t)d->B * d->H * d->dv * d->dk * sizeof(float);
    if (ntok > 0 && (!q || !k || !v || !f || !beta || !c || !o)) return KD_ERR_NULL;
    const void* ptrs[] = {q, k, v, f, beta, c, S0, o, ST};
    for (const void* p : ptrs)
        if (misaligned(p)) return KD_ERR_ALIGN;
    const Range ins[] = {range_of(q, xb), range_of(k, xb), range_of(v, xb), range_of(f, xb),
                         range_of(beta, gb), range_of(c, gb), range_of(S0, S0 ? sb : 0)};
    const Range outs[] = {range_of(o, ntok ? xb : 0), range_of(ST, ST ? sb : 0)};
    for (const Range& a : outs)
        for (const Range& b : ins)
            if (overlap(a, b)) return KD_ERR_ALIAS;
    if (overlap(outs[0], outs[1])) return KD_ERR_ALIAS;
    if (ntok == 0 && !ST) return KD_OK;
    if (d->dtype == KD_F32 && d->dk == 128) {
        // fp32 at d = 128: the chunk kernels' fp32 operands do not fit the LDS,
        // so the tokens go through the per-token recurrence (the decode kernel,
        // state in registers across all T tokens): exact in fp32, sequential in t
        hipError_t e = kd::launch_decode(0, 128, q, k, v, f, beta, c, S0, o, ST, d->B, d->T, d->H,
                                         (hipStream_t)stream);
        return e == hipSuccess ? KD_OK : KD_ERR_LAUNCH;
    }
    const size_t need = fwd_ws_bytes(d);
    if (need > 0 && ws && ws_bytes >= need) {   // few heads: preparation, then the state pass
        if (misaligned(ws)) return KD_ERR_ALIGN;
        const Range wr = range_of(ws, need);
        for (const Range& b : ins)
            if (overlap(wr, b)) return KD_ERR_ALIAS;
        if (overlap(wr, outs[0]) || overlap(wr, outs[1])) return KD_ERR_ALIAS;
        hipError_t e = kd::launch_fwd16_split(q, k, v, f, beta, c, S0, o, ST, ws, d->B, d->T, d->H,
                                              (hipStream_t)stream);
        return e == hipSuccess ? KD_OK : KD_ERR_LAUNCH;
    }
    hipError_t e = kd::launch_fwd(d->dtype == KD_BF16, d->dk, q, k, v, f, beta, c, S0, o, ST,
                                  nullptr, nullptr, d->B, d->T, d->H, (hipStream_t)stream);
    return e == hipSuccess ? KD_OK : KD_ERR_LAUNCH;
}

kd_status kron_delta_fwd_varlen(const kd_desc* d, const int32_t* cu_seqlens, const void* q,
                                const void* k, const void* v, const void* f, const float* beta,
                                const float* c, const float* S0, void* o, float* ST, void* stream) {
    kd_status st = check_desc(d, true);
    if (st != KD_OK) return st;
    if (!cu_seqlens) return KD_ERR_NULL;
    if (((uintptr_t)cu_seqlens & 3u) != 0) return KD_ERR_ALIGN;
    const size_t ntok = (size_t)d->T * d->H;   // all sequences packed along T
    const size_t xb = ntok * d->dk * esize(d);
    const size_t gb = ntok * sizeof(float);
    const size_t sb = (size_t)d->B * d->H * d->dv * d->dk * sizeof(float);
    if (ntok > 0 && (!q || !k || !v || !f || !beta || !c || !o)) return KD_ERR_NULL;
    const void* ptrs[] = {q, k, v, f, beta, c, S0, o, ST};
    for (const void* p : ptrs)
        if (misaligned(p)) return KD_ERR_ALIGN;
    const Range ins[] = {range_of(q, xb), range_of(k, xb), range_of(v, xb), range_of(f, xb),
                         range_of(beta, gb), range_of(c, gb), range_of(S0, S0 ? sb : 0),
                         range_of(cu_seqlens, (size_t)(d->B + 1) * sizeof(int32_t))};
    const Range outs[] = {range_of(o, ntok ? xb : 0), range_of(ST, ST ? sb : 0)};
    for (const Range& a : outs)
        for (const Range& b : ins)
            if (overlap(a, b)) return KD_ERR_ALIAS;
    if (overlap(outs[0], outs[1])) return KD_ERR_ALIAS;
    if (ntok == 0 && !ST) return KD_OK;
    // fp32 at d = 128: the per-token recurrence over each sequence (as kron_delta_fwd)
    hipError_t e = d->dtype == KD_F32 && d->dk == 128
                       ? kd::launch_decode(0, 128, q, k, v, f, beta, c, S0, o, ST, d->B, d->T, d->H,
                                           (hipStream_t)stream, cu_seqlens)
                       : kd::launch_fwd(d->dtype == KD_BF16, d->dk, q, k, v, f, beta, c, S0, o, ST,
                                        nullptr, cu_seqlens, d->B, d->T, d->H, (hipStream_t)stream);
    return e == hipSuccess ? KD_OK : KD_ERR_LAUNCH;
}

kd_status kron_delta_decode(const kd_desc* d, const void* q, const void* k, const void* v,
                            const void* f, const float* beta, const float* c, const float* S_in,
                            void* o, float* S_out, void* stream) {
    kd_status st = check_desc(d, true);
    if (st != KD_OK) return st;
    const size_t ntok = (size_t)d->B * d->T * d->H;
    const size_t xb = ntok * d->dk * esize(d);
    const size_t gb = ntok * sizeof(float);
    const size_t sb = (size_t)d->B * d->H * d->dv * d->dk * sizeof(float);
    if (!S_out) return KD_ERR_NULL;
    if (ntok > 0 && (!q || !k || !v || !f || !beta || !c || !o)) return KD_ERR_NULL;
    const void* ptrs[] = {q, k, v, f, beta, c, S_in, o, S_out};
    for (const void* p : ptrs)
        if (misaligned(p)) return KD_ERR_ALIGN;
    // S_out may be S_in itself (update in place); any other overlap is rejected
    const bool inplace = S_in != nullptr && S_in == S_out;
    const Range ins[] = {range_of(q, xb), range_of(k, xb), range_of(v, xb), range_of(f, xb),
                         range_of(beta, gb), range_of(c, gb), range_of(inplace ? nullptr : S_in, sb)};
    const Range outs[] = {range_of(o, ntok ? xb : 0), range_of(S_out, sb)};
    for (const Range& a : outs)
        for (const Range& b : ins)
            if (overlap(a, b)) return KD_ERR_ALIAS;
    if (overlap(outs[0], outs[1])) return KD_ERR_ALIAS;
    if (inplace && (overlap(outs[0], range_of(S_in, sb)))) return KD_ERR_ALIAS;
    hipError_t e = kd::launch_decode(d->dtype == KD_BF16, d->dk, q, k, v, f, beta, c, S_in, o, S_out,
                                     d->B, d->T, d->H, (hipStream_t)stream);
    return e == hipSuccess ? KD_OK : KD_ERR_LAUNCH;
}

namespace {
kd_status bwd_impl(const kd_desc* d, const void* q, const void* k, const void* v,
                   const void* f, const float* beta, const float* c, const float* S0,
                   const void* dO, const float* dST, void* dq, void* dk, void* dv,
                   void* df, float* dbeta, float* dc, float* dS0, void* ws,
                   size_t ws_bytes, void* stream, int recompute) {
    // fp32 at d = 128 takes the per-token backward (the chunk kernels hold their
    // fp32 operands in LDS only up to d = 64)
    kd_status st = check_desc(d, true);
    if (st != KD_OK) return st;
    const size_t ntok = (size_t)d->B * d->T * d->H;
    const size_t xb = ntok * d->dk * esize(d);
    const size_t gb = ntok * sizeof(float);
    const size_t sb = (size_t)d->B * d->H * d->dv * d->dk * sizeof(float);
    if (ntok > 0 && (!q || !k || !v || !f || !beta || !c || !dO || !dq || !dk || !dv || !df ||
                     !dbeta || !dc))
        return KD_ERR_NULL;
    const void* ptrs[] = {q, k, v, f, beta, c, S0, dO, dST, dq, dk, dv, df, dbeta, dc, dS0, ws};
    for (const void* p : ptrs)
        if (misaligned(p)) return KD_ERR_ALIGN;
    if (ntok == 0 && !dS0) return KD_OK;   // nothing to compute, nothing launched
    const size_t need = kron_delta_workspace_bytes(d, 1);
    if (need > 0 && (!ws || ws_bytes < need)) return KD_ERR_WORKSPACE;
    const Range ins[] = {range_of(q, xb), range_of(k, xb), range_of(v, xb), range_of(f, xb),
                         range_of(beta, gb), range_of(c, gb), range_of(S0, S0 ? sb : 0),
                         range_of(dO, xb), range_of(dST, dST ? sb : 0)};
    const Range outs[] = {range_of(dq, xb), range_of(dk, xb), range_of(dv, xb), range_of(df, xb),
                          range_of(dbeta, gb), range_of(dc, gb), range_of(dS0, dS0 ? sb : 0),
                          range_of(ws, need)};
    for (const Range& a : outs)
        for (const Range& b : ins)
            if (overlap(a, b)) return KD_ERR_ALIAS;
    for (size_t a = 0; a < sizeof(outs) / sizeof(outs[0]); ++a)
        for (size_t b = a + 1; b < sizeof(outs) / sizeof(outs[0]); ++b)
            if (overlap(outs[a], outs[b])) return KD_ERR_ALIAS;
    hipError_t e = kd::launch_bwd(d->dtype == KD_BF16, d->dk, q, k, v, f, beta, c, S0, dO, dST,
                                  dq, dk, dv, df, dbeta, dc, dS0, ws, d->B, d->T, d->H, recompute,
                                  (hipStream_t)stream);
    return e == hipSuccess ? KD_OK : KD_ERR_LAUNCH;
}
}  // namespace

kd_status kron_delta_bwd(const kd_desc* d, const void* q, const void* k, const void* v,
                         const void* f, const float* beta, const float* c, const float* S0,
                         const void* dO, const float* dST, void* dq, void* dk, void* dv,
                         void* df, float* dbeta, float* dc, float* dS0, void* ws,
                         size_t ws_bytes, void* stream) {
    return bwd_impl(d, q, k, v, f, beta, c, S0, dO, dST, dq, dk, dv, df, dbeta, dc, dS0, ws, ws_bytes,
                    stream, 1);
}

kd_status kron_delta_bwd_noalloc(const kd_desc* d, const void* q, const void* k, const void* v,
                                 const void* f, const float* beta, const float* c, const float* S0,
                                 const void* dO, const float* dST, void* dq, void* dk, void* dv,
                                 void* df, float* dbeta, float* dc, float* dS0, void* stream) {
    kd_status st = check_desc(d, true);
    if (st != KD_OK) return st;
    const size_t need = kron_delta_workspace_bytes(d, 1);
    if (need > kScratchBytes) return KD_ERR_SCRATCH;
    void* ws = nullptr;   // looked up only for a call that launches
    const bool launches = (size_t)d->B * d->T * d->H > 0 || dS0 != nullptr;
    if (need > 0 && launches) {
        ws = scratch_address();
        if (ws == nullptr) return KD_ERR_LAUNCH;
    }
    return bwd_impl(d, q, k, v, f, beta, c, S0, dO, dST, dq, dk, dv, df, dbeta, dc, dS0, ws, need, stream, 1);
}

kd_status kron_delta_bwd_status(const kd_desc* d, const void* ws, size_t ws_bytes, void* stream) {
    kd_status st = check_desc(d, true);
    if (st != KD_OK) return st;
    const size_t need = kron_delta_workspace_bytes(d, 1);
    if (ws == nullptr) {   // the fixed scratch of kron_delta_bwd_noalloc on the current device
        if (need > kScratchBytes) return KD_ERR_SCRATCH;
        ws = scratch_address();
        if (ws == nullptr) return KD_ERR_LAUNCH;
    } else {
        if (misaligned(ws)) return KD_ERR_ALIGN;
        if (ws_bytes < need) return KD_ERR_WORKSPACE;
    }
    const size_t off = kd::bwd_status_offset(d->dtype == KD_BF16, d->dk, d->B, d->T, d->H);
    unsigned long long word = 0;
    if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return KD_ERR_LAUNCH;
    if (hipMemcpy(&word, static_cast<const char*>(ws) + off, sizeof(word), hipMemcpyDeviceToHost) != hipSuccess)
        return KD_ERR_LAUNCH;
    return word ? KD_ERR_TIMEOUT : KD_OK;
}

void kron_delta_bwd_set_wait_limit(uint32_t polls) { kd::set_bwd_wait_polls(polls); }

kd_status kron_delta_bwd_saved(const kd_desc* d, const void* q, const void* k, const void* v,
                               const void* f, const float* beta, const float* c, const float* S0,
                               const void* dO, const float* dST, void* dq, void* dk, void* dv,
                               void* df, float* dbeta, float* dc, float* dS0, void* ws,
                               size_t ws_bytes, void* stream) {
    return bwd_impl(d, q, k, v, f, beta, c, S0, dO, dST, dq, dk, dv, df, dbeta, dc, dS0, ws, ws_bytes,
                    stream, 0);
}

kd_status kron_delta_fwd_train(const kd_desc* d, const void* q, const void* k, const void* v,
                               const void* f, const float* beta, const float* c, const float* S0,
                               void* o, float* ST, void* ws, size_t ws_bytes, void* stream) {
    kd_status st = check_desc(d, true);
    if (st != KD_OK) return st;
    const size_t ntok = (size_t)d->B * d->T * d->H;
    const size_t xb = ntok * d->dk * esize(d);
    const size_t gb = ntok * sizeof(float);
    const size_t sb = (size_t)d->B * d->H * d->dv * d->dk * sizeof(float);
    if (ntok > 0 && (!q || !k || !v || !f || !beta || !c || !o)) return KD_ERR_NULL;
    const void* ptrs[] = {q, k, v, f, beta, c, S0, o, ST, ws};
    for (const void* p : ptrs)
        if (misaligned(p)) return KD_ERR_ALIGN;
    const size_t need = kron_delta_workspace_bytes(d, 1);
    if (need > 0 && (!ws || ws_bytes < need)) return KD_ERR_WORKSPACE;
    const Range ins[] = {range_of(q, xb), range_of(k, xb), range_of(v, xb), range_of(f, xb),
                         range_of(beta, gb), range_of(c, gb), range_of(S0, S0 ? sb : 0)};
    const Range outs[] = {range_of(o, ntok ? xb : 0), range_of(ST, ST ? sb : 0), range_of(ws, need)};
    for (const Range& a : outs)
        for (const Range& b : ins)
            if (overlap(a, b)) return KD_ERR_ALIAS;
    for (size_t a = 0; a < 3; ++a)
        for (size_t b = a + 1; b < 3; ++b)
            if (overlap(outs[a], outs[b])) return KD_ERR_ALIAS;
    if (ntok == 0 && !ST) return KD_OK;
    hipError_t e = kd::launch_fwd_train(d->dtype == KD_BF16, d->dk, q, k, v, f, beta, c, S0, o, ST, ws,
                                        d->B, d->T, d->H, (hipStream_t)stream);
    return e == hipSuccess ? KD_OK : KD_ERR_LAUNCH;
}

}  // extern "C"

kd_status kron_delta_gdn2_fwd(const kd_desc* d, const void* q, const void* k, const void* v,
                              const void* alpha, const void* b, const void* w, const float* S0,
                              void* o, float* ST, void* stream) {
    kd_status st = check_desc(d);
    if (st != KD_OK) return st;
    if (d->dtype != KD_BF16) return KD_ERR_DTYPE;
    if (d->dk != 128) return KD_ERR_SHAPE;
    const size_t ntok = (size_t)d->B * d->T * d->H;
    const size_t xb = ntok * d->dk * esize(d);
    const size_t sb = (size_t)d->B * d->H * d->dv * d->dk * sizeof(float);
    if (ntok > 0 && (!q || !k || !v || !alpha || !b || !w || !o)) return KD_ERR_NULL;
    const void* ptrs[] = {q, k, v, alpha, b, w, S0, o, ST};
    for (const void* p : ptrs)
        if (misaligned(p)) return KD_ERR_ALIGN;
    const Range ins[] = {range_of(q, xb), range_of(k, xb), range_of(v, xb), range_of(alpha, xb),
                         range_of(b, xb), range_of(w, xb), range_of(S0, S0 ? sb : 0)};
    const Range outs[] = {range_of(o, ntok ? xb : 0), range_of(ST, ST ? sb : 0)};
    for (const Range& a : outs)
        for (const Range& c : ins)
            if (overlap(a, c)) return KD_ERR_ALIAS;
    if (overlap(outs[0], outs[1])) return KD_ERR_ALIAS;
    if (ntok == 0 && !ST) return KD_OK;
    hipError_t e = kd::launch_gdn2(q, k, v, alpha, b, w, S0, o, ST, d->B, d->T, d->H, (hipStream_t)stream);
    return e == hipSuccess ? KD_OK : KD_ERR_LAUNCH;
}

kd_status kron_delta_mixer_pre(const kd_desc* d, const kd_mixer_params* p, const void* q_raw, const void* k_raw,
                               const void* v_raw, const void* f_raw, const float* beta_raw, const float* c_raw,
                               void* q, void* k, void* v, void* f, float* beta, float* c, void* stream) {
    kd_status st = check_desc(d, true);
    if (st != KD_OK) return st;
    st = check_mixer(d, p, true, false);
    if (st != KD_OK) return st;
    const size_t ntok = (size_t)d->B * d->T * d->H;
    const size_t xb = ntok * d->dk * esize(d), gb = ntok * sizeof(float);
    if (ntok == 0) return KD_OK;
    const void* ptrs[] = {q_raw, k_raw, v_raw, f_raw, beta_raw, c_raw, q, k, v, f, beta, c};
    for (const void* x : ptrs)
        if (!x) return KD_ERR_NULL;
    for (const void* x : ptrs)
        if (misaligned(x)) return KD_ERR_ALIGN;
    const size_t hd = (size_t)d->H * d->dk * p->conv_size * sizeof(float);
    const Range ins[] = {range_of(q_raw, xb), range_of(k_raw, xb), range_of(v_raw, xb), range_of(f_raw, xb),
                         range_of(beta_raw, gb), range_of(c_raw, gb), range_of(p->conv_q, hd),
                         range_of(p->conv_k, hd), range_of(p->conv_v, hd),
                         range_of(p->a_log, (size_t)d->H * sizeof(float))};
    const Range outs[] = {range_of(q, xb), range_of(k, xb), range_of(v, xb), range_of(f, xb), range_of(beta, gb),
                          range_of(c, gb)};
    for (const Range& a : outs)
        for (const Range& b : ins)
            if (overlap(a, b)) return KD_ERR_ALIAS;
    for (int i = 0; i < 6; ++i)
        for (int j = i + 1; j < 6; ++j)
            if (overlap(outs[i], outs[j])) return KD_ERR_ALIAS;
    const void* raw[4] = {q_raw, k_raw, v_raw, f_raw};
    void* out[4] = {q, k, v, f};
    const float* conv[3] = {p->conv_q, p->conv_k, p->conv_v};
    hipError_t e = kd::launch_mixer_pre(d->dtype == KD_BF16, d->dk, raw, out, conv, p->conv_size, p->a_log,
                                        beta_raw, c_raw, p->beta_scale, beta, c, d->B, d->T, d->H, 1,
                                        (hipStream_t)stream);
    return e == hipSuccess ? KD_OK : KD_ERR_LAUNCH;
}

kd_status kron_delta_mixer_post(const kd_desc* d, const kd_mixer_params* p, const void* o, const void* g,
                                void* y, void* stream) {
    kd_status st = check_desc(d, true);
    if (st != KD_OK) return st;
    st = check_mixer(d, p, false, true);
    if (st != KD_OK) return st;
    const size_t ntok = (size_t)d->B * d->T * d->H;
    const size_t xb = ntok * d->dv * esize(d);
    if (ntok == 0) return KD_OK;
    if (!o || !g || !y) return KD_ERR_NULL;
    if (misaligned(o) || misaligned(g) || misaligned(y)) return KD_ERR_ALIGN;
    const Range ry = range_of(y, xb);
    if (overlap(ry, range_of(o, xb)) || overlap(ry, range_of(g, xb)) ||
        overlap(ry, range_of(p->norm_w, (size_t)d->H * d->dv * sizeof(float))))
        return KD_ERR_ALIAS;
    hipError_t e = kd::launch_mixer_post(d->dtype == KD_BF16, d->dv, o, g, p->norm_w, p->norm_eps, y, d->B, d->T,
                                         d->H, (hipStream_t)stream);
    return e == hipSuccess ? KD_OK : KD_ERR_LAUNCH;
}

kd_status kron_delta_mixer_fwd(const kd_desc* d, const kd_mixer_params* p, const void* q_raw, const void* k_raw,
                               const void* v_raw, const void* f_raw, const float* beta_raw, const float* c_raw,
                               const void* g, const float* S0, void* y, float* ST, void* ws, size_t ws_bytes,
                               void* stream) {
    kd_status st = check_desc(d);
    if (st != KD_OK) return st;
    st = check_mixer(d, p, true, true);
    if (st != KD_OK) return st;
    const size_t ntok = (size_t)d->B * d->T * d->H;
    const size_t xb = ntok * d->dk * esize(d), gb = ntok * sizeof(float);
    const size_t sb = (size_t)d->B * d->H * d->dv * d->dk * sizeof(float);
    const MixWs L = mixer_ws(d);
    if (ntok > 0 && (!q_raw || !k_raw || !v_raw || !f_raw || !beta_raw || !c_raw || !g || !y)) return KD_ERR_NULL;
    const void* ptrs[] = {q_raw, k_raw, v_raw, f_raw, beta_raw, c_raw, g, S0, y, ST, ws};
    for (const void* x : ptrs)
        if (misaligned(x)) return KD_ERR_ALIGN;
    if (ntok > 0 && (!ws || ws_bytes < L.total)) return KD_ERR_WORKSPACE;
    const size_t hd = (size_t)d->H * d->dk * p->conv_size * sizeof(float);
    const Range ins[] = {range_of(q_raw, xb), range_of(k_raw, xb), range_of(v_raw, xb), range_of(f_raw, xb),
                         range_of(beta_raw, gb), range_of(c_raw, gb), range_of(g, xb), range_of(S0, S0 ? sb : 0),
                         range_of(p->conv_q, hd), range_of(p->conv_k, hd), range_of(p->conv_v, hd),
                         range_of(p->a_log, (size_t)d->H * sizeof(float)),
                         range_of(p->norm_w, (size_t)d->H * d->dv * sizeof(float))};
    const Range outs[] = {range_of(y, ntok ? xb : 0), range_of(ST, ST ? sb : 0),
                          range_of(ws, ntok ? L.total : 0)};
    for (const Range& a : outs)
        for (const Range& b : ins)
            if (overlap(a, b)) return KD_ERR_ALIAS;
    if (overlap(outs[0], outs[1]) || overlap(outs[0], outs[2]) || overlap(outs[1], outs[2])) return KD_ERR_ALIAS;
    if (ntok == 0) {
        if (!ST) return KD_OK;
        hipError_t e = kd::launch_fwd(d->dtype == KD_BF16, d->dk, nullptr, nullptr, nullptr, nullptr, nullptr,
                                      nullptr, S0, nullptr, ST, nullptr, nullptr, d->B, d->T, d->H,
                                      (hipStream_t)stream);
        return e == hipSuccess ? KD_OK : KD_ERR_LAUNCH;
    }
    char* wb = static_cast<char*>(ws);
    void* x[4];
    for (int i = 0; i < 4; ++i) x[i] = wb + L.x[i];
    float* beta = reinterpret_cast<float*>(wb + L.beta);
    float* c = reinterpret_cast<float*>(wb + L.c);
    void* o = wb + L.o;
    const void* raw[4] = {q_raw, k_raw, v_raw, f_raw};
    const float* conv[3] = {p->conv_q, p->conv_k, p->conv_v};
    const hipStream_t sm = (hipStream_t)stream;
    const int bf = d->dtype == KD_BF16;
    // bf16 at d = 128: the forward makes the gates from their logits as it
    // loads them (the gate kernel's arithmetic, so the same bits) and writes
    // y through the gated norm as it stores each chunk's rows (the
    // post-processing kernel's arithmetic)
    const bool fused_gates = bf && d->dk == 128;
    // and with conv_size 4, when the compute units the forward blocks leave
    // free hold enough workers, the convolution runs on them inside the same
    // launch, each chunk published to the forward as soon as it is done
    const int nwork = fused_gates && p->conv_size == 4 ? kd::fwd16_feed_workers(d->B * d->H) : 0;
    if (nwork > 0) {
        hipError_t e = kd::launch_fwd16_mixer_fed(raw, x, conv, f_raw, beta_raw, c_raw, p->a_log, p->beta_scale, g,
                                                  p->norm_w, p->norm_eps, S0, y, ST, wb + L.hw, nwork, d->B, d->T,
                                                  d->H, sm);
        return e == hipSuccess ? KD_OK : KD_ERR_LAUNCH;
    }
    hipError_t e = kd::launch_mixer_pre(bf, d->dk, raw, x, conv, p->conv_size, p->a_log, beta_raw, c_raw,
                                        p->beta_scale, beta, c, d->B, d->T, d->H, fused_gates ? 0 : 1, sm);
    if (e == hipSuccess)
        e = fused_gates ? kd::launch_fwd16_gates(x[0], x[1], x[2], f_raw, beta_raw, c_raw, p->a_log, p->beta_scale,
                                                 g, p->norm_w, p->norm_eps, S0, y, ST, d->B, d->T, d->H, sm)
                        : kd::launch_fwd(bf, d->dk, x[0], x[1], x[2], x[3], beta, c, S0, o, ST, nullptr, nullptr,
                                         d->B, d->T, d->H, sm);
    if (e == hipSuccess && !fused_gates)
        e = kd::launch_mixer_post(bf, d->dv, o, g, p->norm_w, p->norm_eps, y, d->B, d->T, d->H, sm);
    return e == hipSuccess ? KD_OK : KD_ERR_LAUNCH;
}

