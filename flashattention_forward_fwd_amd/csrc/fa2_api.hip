// fa2_api.hip -- the C ABI of libfa2.so (declared in include/fa2.h): argument
// validation, device check, launch geometry and dispatch to the kernels.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <atomic>

#include "fa2.h"
#include "fa2_internal.h"

namespace {

// Per-device result of the architecture check: 0 unknown, 1 gfx950, 2 other.
constexpr int kMaxDevices = 64;
std::atomic<int> g_device_ok[kMaxDevices];

int check_device()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return FA2_ERR_DEVICE;
    if (dev < kMaxDevices) {
        const int known = g_device_ok[dev].load(std::memory_order_relaxed);
        if (known == 1) return FA2_OK;
        if (known == 2) return FA2_ERR_DEVICE;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
        return FA2_ERR_DEVICE;
    const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev < kMaxDevices)
        g_device_ok[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
    return ok ? FA2_OK : FA2_ERR_DEVICE;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// a*b*c*d fits in int64 (all positive)?
bool product_fits(int64_t a, int64_t b, int64_t c, int64_t d)
{
    const int64_t lim = INT64_MAX;
    if (a > lim / b) return false;
    a *= b;
    if (a > lim / c) return false;
    a *= c;
    return a <= lim / d;
}

int prepare(const void *q, const void *k, const void *v, const void *o, const float *lse,
            int B, int H, int Lq, int Lk, int d, float scale, int causal, int elem_bytes,
            fa2::FwdParams *out)
{
    if (!q || !k || !v || !o || !lse) return FA2_ERR_NULL;
    if (B <= 0 || H <= 0 || Lq <= 0 || Lk <= 0) return FA2_ERR_DIM;
    if (d != 64 && d != 128) return FA2_ERR_UNSUPPORTED_D;
    if (causal != 0 && causal != 1) return FA2_ERR_ARG;
    if (!(scale > 0.f) || !isfinite(scale)) return FA2_ERR_ARG;
    if (elem_bytes != 2 && elem_bytes != 4) return FA2_ERR_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
        return FA2_ERR_ALIGN;
    const int64_t L = Lq > Lk ? Lq : Lk;
    if (!product_fits(B, H, L, (int64_t)d * elem_bytes)) return FA2_ERR_DIM;
    const int64_t n_qtiles = (Lq + fa2::kBr - 1) / fa2::kBr;
    if ((int64_t)B * H > INT32_MAX / n_qtiles) return FA2_ERR_DIM;   // grid size
    if (out) {
        out->q = q; out->k = k; out->v = v; out->o = const_cast<void *>(o);
        out->lse = const_cast<float *>(lse);
        out->B = B; out->H = H; out->Lq = Lq; out->Lk = Lk;
        out->scale_log2 = (float)((double)scale * 1.4426950408889634074);
        out->n_qtiles = (int)n_qtiles;
        out->n_wg = (int)(n_qtiles * B * H);
    }
    return FA2_OK;
}

}  // namespace

extern "C" {

int fa2_check_args(const void *q, const void *k, const void *v, const void *o, const float *lse,
                   int B, int H, int Lq, int Lk, int d, float scale, int causal, int elem_bytes)
{
    return prepare(q, k, v, o, lse, B, H, Lq, Lk, d, scale, causal, elem_bytes, nullptr);
}

int fa2_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
            int B, int H, int Lq, int Lk, int d, float scale, int causal, void *stream)
{
    fa2::FwdParams p;
    int st = prepare(q, k, v, o, lse, B, H, Lq, Lk, d, scale, causal, 2, &p);
    if (st != FA2_OK) return st;
    if ((st = check_device()) != FA2_OK) return st;
    if (fa2::launch_fwd_bf16(p, d, causal != 0, static_cast<hipStream_t>(stream)) != hipSuccess)
        return FA2_ERR_LAUNCH;
    return FA2_OK;
}

int fa2_fwd_f32(const float *q, const float *k, const float *v, float *o, float *lse,
                int B, int H, int Lq, int Lk, int d, float scale, int causal, void *stream)
{
    fa2::FwdParams p;
    int st = prepare(q, k, v, o, lse, B, H, Lq, Lk, d, scale, causal, 4, &p);
    if (st != FA2_OK) return st;
    if ((st = check_device()) != FA2_OK) return st;
    if (fa2::launch_fwd_f32(p, d, causal != 0, static_cast<hipStream_t>(stream)) != hipSuccess)
        return FA2_ERR_LAUNCH;
    return FA2_OK;
}

const char *fa2_status_string(int status)
{
    switch (status) {
    case FA2_OK: return "ok";
    case FA2_ERR_NULL: return "a tensor pointer is NULL";
    case FA2_ERR_DIM: return "B, H, Lq, Lk must be positive and the sizes must fit";
    case FA2_ERR_UNSUPPORTED_D: return "head dimension d must be 64 or 128";
    case FA2_ERR_ARG: return "causal must be 0 or 1 and scale finite and positive";
    case FA2_ERR_ALIGN: return "tensor pointers must be 16-byte aligned";
    case FA2_ERR_DEVICE: return "no usable gfx950 HIP device";
    case FA2_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
    }
}

}  // extern "C"
