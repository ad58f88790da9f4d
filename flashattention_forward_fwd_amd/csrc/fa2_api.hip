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
std::atomic<int> g_device_cus[kMaxDevices];     // compute units, 0 = not queried yet

// Work-groups of the forward kernels that one compute unit holds at once.
constexpr int kWorkgroupsPerCU = 2;
// Fewest K/V tiles a split-KV range should have, so the partial kernel's
// software pipeline and double buffering have something to overlap.
constexpr int kMinTilesPerSplit = 8;
// The decoding kernel (Lq <= 4): work-groups per CU the automatic split count
// aims for, and the fewest keys per range.
constexpr int kDecodeWorkgroupsPerCU = 2;
constexpr int kMinDecodeKeys = 256;

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

// Compute units of the current device (0 if it cannot be queried).
int device_cus()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    if (dev < kMaxDevices) {
        const int known = g_device_cus[dev].load(std::memory_order_relaxed);
        if (known > 0) return known;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return 0;
    if (dev < kMaxDevices) g_device_cus[dev].store(cus, std::memory_order_relaxed);
    return cus;
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

// Head-dimension sets: the fp32 forward (32, 64, 128) and every 16-bit kernel
// and the merge (also 96 and 256).
enum DimSet { kDimsF32, kDims16 };
bool head_dim_ok(int d, DimSet dims)
{
    if (d == 32 || d == 64 || d == 128) return true;
    return dims == kDims16 && (d == 96 || d == 256);
}

int prepare(const void *q, const void *k, const void *v, const void *o, const float *lse,
            int B, int H, int Lq, int Lk, int d, float scale, int causal, int elem_bytes,
            fa2::FwdParams *out, DimSet dims = kDimsF32)
{
    if (!q || !k || !v || !o || !lse) return FA2_ERR_NULL;
    if (B <= 0 || H <= 0 || Lq <= 0 || Lk <= 0) return FA2_ERR_DIM;
    if (!head_dim_ok(d, dims)) return FA2_ERR_UNSUPPORTED_D;
    if (causal != 0 && causal != 1) return FA2_ERR_ARG;
    if (!(scale > 0.f) || !isfinite(scale)) return FA2_ERR_ARG;
    if (elem_bytes != 2 && elem_bytes != 4) return FA2_ERR_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
        return FA2_ERR_ALIGN;
    const int64_t L = Lq > Lk ? Lq : Lk;
    if (!product_fits(B, H, L, (int64_t)d * elem_bytes)) return FA2_ERR_DIM;
    // One head's K (or V), plus one tile, must stay below 2 GiB: tiles are
    // addressed with 32-bit buffer offsets.
    if (((int64_t)Lk + fa2::kBc) * d * elem_bytes > INT32_MAX) return FA2_ERR_DIM;
    const int64_t n_qtiles = (Lq + fa2::kBr - 1) / fa2::kBr;
    if ((int64_t)B * H > INT32_MAX / n_qtiles) return FA2_ERR_DIM;   // grid size
    if (out) {
        out->q = q; out->k = k; out->v = v; out->o = const_cast<void *>(o);
        out->lse = const_cast<float *>(lse);
        out->B = B; out->H = H; out->Lq = Lq; out->Lk = Lk;
        out->scale_log2 = (float)((double)scale * 1.4426950408889634074);
        out->n_qtiles = (int)n_qtiles;
        out->n_splits = 1;
        out->n_wg = (int)(n_qtiles * B * H);
        out->wl = -1;
        out->wr = causal ? 0 : -1;
        out->drop = fa2::DropoutParams{0u, 0u, 0u, 256u, 1.0f};
    }
    return FA2_OK;
}

// Dropout settings: keep threshold t = round(256 (1 - p)) (ties to even) in
// 1..256, scale 256 / t.  p must lie in [0, 1).
int dropout_setup(double p_drop, uint64_t seed, uint32_t offset, fa2::DropoutParams *dp)
{
    if (!(p_drop >= 0.0 && p_drop < 1.0)) return FA2_ERR_ARG;
    double t = nearbyint(256.0 * (1.0 - p_drop));
    if (t < 1.0) t = 1.0;
    if (t > 256.0) t = 256.0;
    dp->seed_lo = (uint32_t)(seed & 0xFFFFFFFFu);
    dp->seed_hi = (uint32_t)(seed >> 32);
    dp->offset = offset;
    dp->threshold = (uint32_t)t;
    dp->keep_scale = (float)(256.0 / t);
    return FA2_OK;
}

// Split count for num_splits == 0 (Lq <= 4: the decoding kernel's rule below):
// the fewest ranges that put one work-group on every compute unit, or two under
// the causal mask (query tiles then differ in length, and finer pieces even out
// the end of the launch).  Measured on MI355X, more splits than that cost more in
// partial-result traffic and per work-group start-up than they gain.  Every range
// keeps at least kMinTilesPerSplit K/V tiles.
int auto_splits(int B, int H, int Lq, int Lk, int causal)
{
    const int cus = device_cus();
    if (cus <= 0) return 1;
    if (Lq <= fa2::kDecodeMaxRows) {
        // Decoding kernel: two work-groups per CU keep enough loads in flight;
        // every range keeps at least kMinDecodeKeys keys.
        const int64_t keys = causal ? (Lq < Lk ? Lq : Lk) : Lk;
        int64_t S = ((int64_t)kDecodeWorkgroupsPerCU * cus + (int64_t)B * H - 1) / ((int64_t)B * H);
        if (S > keys / kMinDecodeKeys) S = keys / kMinDecodeKeys;
        if (S > FA2_MAX_SPLITS) S = FA2_MAX_SPLITS;
        return S < 1 ? 1 : (int)S;
    }
    const int64_t target = (int64_t)cus * (causal ? kWorkgroupsPerCU : 1);
    const int64_t n_qtiles = (Lq + fa2::kBr - 1) / fa2::kBr;
    const int64_t base = n_qtiles * B * H;
    if (base >= target) return 1;
    // K/V tiles of the longest query tile (the last one).
    const int tiles = fa2::kv_tiles_for((int)n_qtiles - 1, Lq, Lk, causal != 0);
    int64_t S = (target + base - 1) / base;
    if (S > tiles / kMinTilesPerSplit) S = tiles / kMinTilesPerSplit;
    if (S > FA2_MAX_SPLITS) S = FA2_MAX_SPLITS;
    return S < 1 ? 1 : (int)S;
}

// Byte size of the partial outputs [S, rows, d] fp32, rounded up so the
// partial logsumexps that follow start on a 256-byte boundary.
size_t partial_o_bytes(int64_t S, int64_t rows, int d)
{
    const size_t b = (size_t)S * rows * d * sizeof(float);
    return (b + 255) & ~(size_t)255;
}

// The merge grid (d/4 threads per row, 256 per work-group) fits in a launch.
bool merge_grid_fits(int64_t rows, int d)
{
    return rows <= (int64_t)INT32_MAX / (d / 4) * 256;
}

// Workspace size for S splits, 0 if it overflows.
size_t workspace_bytes(int64_t S, int B, int H, int Lq, int d)
{
    const int64_t rows = (int64_t)B * H * Lq;
    if (!product_fits(S, rows, d + 1, sizeof(float))) return 0;
    return partial_o_bytes(S, rows, d) + (size_t)S * rows * sizeof(float);
}

// Backward workspace: lse * log2(e) for every query row, then (at a 256-byte
// boundary) D = rowsum(dO * O) for every query row, both fp32.  0 on overflow.
size_t bwd_lse2_bytes(int64_t rows)
{
    return ((size_t)rows * sizeof(float) + 255) & ~(size_t)255;
}
size_t bwd_workspace_bytes(int B, int H, int Lq)
{
    if (B <= 0 || H <= 0 || Lq <= 0) return 0;
    if (!product_fits(B, H, Lq, 2 * sizeof(float))) return 0;
    const int64_t rows = (int64_t)B * H * Lq;
    return bwd_lse2_bytes(rows) + (size_t)rows * sizeof(float);
}

int prepare_bwd(const void *q, const void *k, const void *v, const void *o, const float *lse, const void *dout,
                const void *dq, const void *dk, const void *dv, int B, int H, int Lq, int Lk, int d,
                float scale, int causal, const void *workspace, size_t workspace_bytes_given,
                fa2::BwdParams *out)
{
    if (!dout || !dq || !dk || !dv) return FA2_ERR_NULL;
    int st = prepare(q, k, v, o, lse, B, H, Lq, Lk, d, scale, causal, 2, nullptr, kDims16);
    if (st != FA2_OK) return st;
    if (!aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv)) return FA2_ERR_ALIGN;
    // Query tiles of one head are addressed with 32-bit buffer offsets too.
    if (((int64_t)Lq + fa2::kBr) * d * 2 > INT32_MAX) return FA2_ERR_DIM;
    const int64_t key_block = d == 256 ? 64 : 128;    // keys per dK/dV work-group
    const int64_t key_blocks = (Lk + key_block - 1) / key_block;
    if ((int64_t)B * H > INT32_MAX / key_blocks) return FA2_ERR_DIM;          // dK/dV grid
    const int64_t rows = (int64_t)B * H * Lq;
    if (rows * (d == 96 ? 16 : d / 8) / 256 + 1 > INT32_MAX) return FA2_ERR_DIM;  // prep grid
    const size_t need = bwd_workspace_bytes(B, H, Lq);
    if (need == 0) return FA2_ERR_DIM;
    if (!workspace) return FA2_ERR_WORKSPACE;
    if (!aligned16(workspace)) return FA2_ERR_ALIGN;
    if (workspace_bytes_given < need) return FA2_ERR_WORKSPACE;
    if (out) {
        out->q = q; out->k = k; out->v = v; out->dout = dout;
        out->dq = const_cast<void *>(dq); out->dk = const_cast<void *>(dk); out->dv = const_cast<void *>(dv);
        float *ws = static_cast<float *>(const_cast<void *>(workspace));
        out->lse2 = ws;
        out->delta = reinterpret_cast<const float *>(reinterpret_cast<const char *>(ws) + bwd_lse2_bytes(rows));
        out->B = B; out->H = H; out->Lq = Lq; out->Lk = Lk;
        out->scale = scale;
        out->scale_log2 = (float)((double)scale * 1.4426950408889634074);
        out->n_blocks = 0;
        out->n_wg = 0;
        out->wl = -1;
        out->wr = causal ? 0 : -1;
        out->drop = fa2::DropoutParams{0u, 0u, 0u, 256u, 1.0f};
    }
    return FA2_OK;
}

// ---- the 16-bit entry points, shared by the bf16 and fp16 (f16) names

int fwd16(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H, int Lq, int Lk, int d,
          float scale, int causal, bool f16, void *stream)
{
    fa2::FwdParams p;
    int st = prepare(q, k, v, o, lse, B, H, Lq, Lk, d, scale, causal, 2, &p, kDims16);
    if (st != FA2_OK) return st;
    if ((st = check_device()) != FA2_OK) return st;
    if (fa2::launch_fwd16(p, d, causal != 0, f16, fa2::FwdVariant::kPlain, static_cast<hipStream_t>(stream)) !=
        hipSuccess)
        return FA2_ERR_LAUNCH;
    return FA2_OK;
}

int fwd_window16(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H, int Lq, int Lk,
                 int d, float scale, int window_left, int window_right, bool f16, void *stream)
{
    fa2::FwdParams p;
    int st = prepare(q, k, v, o, lse, B, H, Lq, Lk, d, scale, 0, 2, &p, kDims16);
    if (st != FA2_OK) return st;
    if ((st = check_device()) != FA2_OK) return st;
    // Negative bounds all mean "unbounded"; keep them as -1.
    p.wl = window_left < 0 ? -1 : window_left;
    p.wr = window_right < 0 ? -1 : window_right;
    if (fa2::launch_fwd16(p, d, false, f16, fa2::FwdVariant::kWindow, static_cast<hipStream_t>(stream)) !=
        hipSuccess)
        return FA2_ERR_LAUNCH;
    return FA2_OK;
}

int fwd_dropout16(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H, int Lq, int Lk,
                  int d, float scale, int causal, double dropout_p, uint64_t seed, uint32_t offset, bool f16,
                  void *stream)
{
    fa2::FwdParams p;
    int st = prepare(q, k, v, o, lse, B, H, Lq, Lk, d, scale, causal, 2, &p, kDims16);
    if (st != FA2_OK) return st;
    if ((st = dropout_setup(dropout_p, seed, offset, &p.drop)) != FA2_OK) return st;
    if ((st = check_device()) != FA2_OK) return st;
    if (fa2::launch_fwd16(p, d, causal != 0, f16, fa2::FwdVariant::kDropout, static_cast<hipStream_t>(stream)) !=
        hipSuccess)
        return FA2_ERR_LAUNCH;
    return FA2_OK;
}

// Launches the split-KV forward for S >= 1 ranges with the partial results in
// `workspace` (big enough for S; unused when S == 1): the partial kernel (or the
// decoding kernel for a few query rows), then the merge.
int splitkv_launch(const fa2::FwdParams &p, int S, int d, int causal, bool f16, void *workspace, void *o,
                   float *lse, hipStream_t s)
{
    if (S == 1) {                             // one range: the one-pass kernel
        if (fa2::launch_fwd16(p, d, causal != 0, f16, fa2::FwdVariant::kPlain, s) != hipSuccess)
            return FA2_ERR_LAUNCH;
        return FA2_OK;
    }
    const int64_t rows = (int64_t)p.B * p.H * p.Lq;
    float *o_parts = static_cast<float *>(workspace);
    float *lse_parts = reinterpret_cast<float *>(static_cast<char *>(workspace) + partial_o_bytes(S, rows, d));
    fa2::FwdParams pp = p;
    pp.o = o_parts;
    pp.lse = lse_parts;
    pp.n_splits = S;
    if (p.Lq <= fa2::kDecodeMaxRows) {        // a few query rows: the decoding kernel
        pp.n_wg = p.B * p.H * S;
        if (fa2::launch_decode(pp, d, f16, s) != hipSuccess) return FA2_ERR_LAUNCH;
    } else {
        pp.n_wg = p.n_wg * S;
        if (fa2::launch_fwd16(pp, d, causal != 0, f16, fa2::FwdVariant::kSplit, s) != hipSuccess)
            return FA2_ERR_LAUNCH;
    }
    if (fa2::launch_merge(o_parts, lse_parts, S, rows, d, f16, o, lse, s) != hipSuccess) return FA2_ERR_LAUNCH;
    return FA2_OK;
}

// Range count of a split-KV call and the partial-result bytes it needs; the
// status of the size checks.  num_splits == 0 asks the device (auto_splits).
int splitkv_size(const fa2::FwdParams &p, int num_splits, int d, int causal, int *S_out, size_t *need_out)
{
    const int S = num_splits == 0 ? auto_splits(p.B, p.H, p.Lq, p.Lk, causal) : num_splits;
    if ((int64_t)p.n_wg * S > INT32_MAX) return FA2_ERR_DIM;
    if (!merge_grid_fits((int64_t)p.B * p.H * p.Lq, d)) return FA2_ERR_DIM;
    const size_t need = workspace_bytes(S, p.B, p.H, p.Lq, d);
    if (need == 0) return FA2_ERR_DIM;
    *S_out = S;
    *need_out = need;
    return FA2_OK;
}

int fwd_splitkv16(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H, int Lq, int Lk,
                  int d, float scale, int causal, int num_splits, void *workspace, size_t workspace_bytes_given,
                  bool f16, void *stream)
{
    fa2::FwdParams p;
    int st = prepare(q, k, v, o, lse, B, H, Lq, Lk, d, scale, causal, 2, &p, kDims16);
    if (st != FA2_OK) return st;
    if (num_splits < 0 || num_splits > FA2_MAX_SPLITS) return FA2_ERR_ARG;
    if (!workspace) return FA2_ERR_WORKSPACE;
    if (!aligned16(workspace)) return FA2_ERR_ALIGN;
    if ((st = check_device()) != FA2_OK) return st;
    int S = 0;
    size_t need = 0;
    if ((st = splitkv_size(p, num_splits, d, causal, &S, &need)) != FA2_OK) return st;
    if (workspace_bytes_given < need) return FA2_ERR_WORKSPACE;
    return splitkv_launch(p, S, d, causal, f16, workspace, o, lse, static_cast<hipStream_t>(stream));
}

// ---- fa2_fwd_splitkv_static: the partial results in a static device array

// Device memory of the library, one copy on every device it runs on (held
// until the process ends).  Host code never uses this name as an address: the
// host-side symbol is a stand-in, and a kernel given it would fault.  Each
// device's own address comes from hipGetSymbolAddress (scratch_on_device).
static __device__ __align__(256) char scratch[FA2_STATIC_SCRATCH_BYTES];

std::atomic<void *> g_scratch_ptr[kMaxDevices];

// The current device's address of `scratch`: looked up once per device (with
// that device current) and kept; NULL if the lookup fails.
void *scratch_on_device()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void *ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (ptr) return ptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev].store(ptr, std::memory_order_release);
    return ptr;
}

int merge16(const float *o_parts, const float *lse_parts, int n_parts, int64_t rows, int d, void *o, float *lse,
            bool f16, void *stream)
{
    if (!o_parts || !lse_parts || !o || !lse) return FA2_ERR_NULL;
    if (n_parts < 1 || n_parts > FA2_MAX_SPLITS) return FA2_ERR_ARG;
    if (rows < 1) return FA2_ERR_DIM;
    if (!head_dim_ok(d, kDims16)) return FA2_ERR_UNSUPPORTED_D;
    if (!aligned16(o_parts) || !aligned16(lse_parts) || !aligned16(o) || !aligned16(lse))
        return FA2_ERR_ALIGN;
    if (!product_fits(n_parts, rows, d, sizeof(float))) return FA2_ERR_DIM;
    if (!merge_grid_fits(rows, d)) return FA2_ERR_DIM;
    int st = check_device();
    if (st != FA2_OK) return st;
    if (fa2::launch_merge(o_parts, lse_parts, n_parts, rows, d, f16, o, lse, static_cast<hipStream_t>(stream)) !=
        hipSuccess)
        return FA2_ERR_LAUNCH;
    return FA2_OK;
}

struct Window {
    int left, right;
};
struct Dropout {
    double p;
    uint64_t seed;
    uint32_t offset;
};

// The backward entry points: causal, or a window (w), with or without dropout (dr).
int bwd16(const void *q, const void *k, const void *v, const void *o, const float *lse, const void *dout, void *dq,
          void *dk, void *dv, int B, int H, int Lq, int Lk, int d, float scale, int causal, const Window *w,
          const Dropout *dr, void *workspace, size_t workspace_bytes_given, bool f16, void *stream)
{
    fa2::BwdParams p;
    int st = prepare_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, H, Lq, Lk, d, scale, causal, workspace,
                         workspace_bytes_given, &p);
    if (st != FA2_OK) return st;
    if (dr && (st = dropout_setup(dr->p, dr->seed, dr->offset, &p.drop)) != FA2_OK) return st;
    if ((st = check_device()) != FA2_OK) return st;
    if (w) {
        p.wl = w->left < 0 ? -1 : w->left;
        p.wr = w->right < 0 ? -1 : w->right;
    }
    if (fa2::launch_bwd16(p, d, f16, dr != nullptr, o, lse, static_cast<hipStream_t>(stream)) != hipSuccess)
        return FA2_ERR_LAUNCH;
    return FA2_OK;
}

}  // namespace

extern "C" {

int fa2_check_args(const void *q, const void *k, const void *v, const void *o, const float *lse,
                   int B, int H, int Lq, int Lk, int d, float scale, int causal, int elem_bytes)
{
    return prepare(q, k, v, o, lse, B, H, Lq, Lk, d, scale, causal, elem_bytes, nullptr,
                   elem_bytes == 2 ? kDims16 : kDimsF32);
}

int fa2_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
            int B, int H, int Lq, int Lk, int d, float scale, int causal, void *stream)
{
    return fwd16(q, k, v, o, lse, B, H, Lq, Lk, d, scale, causal, false, stream);
}

int fa2_fwd_f16(const void *q, const void *k, const void *v, void *o, float *lse,
                int B, int H, int Lq, int Lk, int d, float scale, int causal, void *stream)
{
    return fwd16(q, k, v, o, lse, B, H, Lq, Lk, d, scale, causal, true, stream);
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

int fa2_fwd_window(const void *q, const void *k, const void *v, void *o, float *lse,
                   int B, int H, int Lq, int Lk, int d, float scale, int window_left, int window_right,
                   void *stream)
{
    return fwd_window16(q, k, v, o, lse, B, H, Lq, Lk, d, scale, window_left, window_right, false, stream);
}

int fa2_fwd_window_f16(const void *q, const void *k, const void *v, void *o, float *lse,
                       int B, int H, int Lq, int Lk, int d, float scale, int window_left, int window_right,
                       void *stream)
{
    return fwd_window16(q, k, v, o, lse, B, H, Lq, Lk, d, scale, window_left, window_right, true, stream);
}

int fa2_fwd_dropout(const void *q, const void *k, const void *v, void *o, float *lse,
                    int B, int H, int Lq, int Lk, int d, float scale, int causal,
                    double dropout_p, uint64_t seed, uint32_t offset, void *stream)
{
    return fwd_dropout16(q, k, v, o, lse, B, H, Lq, Lk, d, scale, causal, dropout_p, seed, offset, false, stream);
}

int fa2_fwd_dropout_f16(const void *q, const void *k, const void *v, void *o, float *lse,
                        int B, int H, int Lq, int Lk, int d, float scale, int causal,
                        double dropout_p, uint64_t seed, uint32_t offset, void *stream)
{
    return fwd_dropout16(q, k, v, o, lse, B, H, Lq, Lk, d, scale, causal, dropout_p, seed, offset, true, stream);
}

int fa2_splitkv_num_splits(int B, int H, int Lq, int Lk, int d, int causal)
{
    if (B <= 0 || H <= 0 || Lq <= 0 || Lk <= 0 || !head_dim_ok(d, kDims16)) return 1;
    return auto_splits(B, H, Lq, Lk, causal);
}

size_t fa2_splitkv_workspace_bytes(int B, int H, int Lq, int Lk, int d, int causal, int num_splits)
{
    // Size checks of fa2_fwd_splitkv, on stand-in aligned pointers.
    const void *fake = reinterpret_cast<const void *>(uintptr_t(256));
    if (prepare(fake, fake, fake, fake, static_cast<const float *>(fake), B, H, Lq, Lk, d, 1.0f,
                causal, 2, nullptr, kDims16) != FA2_OK)
        return 0;
    if (num_splits < 0 || num_splits > FA2_MAX_SPLITS) return 0;
    const int S = num_splits == 0 ? auto_splits(B, H, Lq, Lk, causal) : num_splits;
    return workspace_bytes(S, B, H, Lq, d);
}

int fa2_fwd_splitkv_static(const void *q, const void *k, const void *v, void *o, float *lse,
                           int B, int H, int Lq, int Lk, int d, float scale, int causal, int num_splits, void *stream)
{
    fa2::FwdParams p;
    int st = prepare(q, k, v, o, lse, B, H, Lq, Lk, d, scale, causal, 2, &p, kDims16);
    if (st != FA2_OK) return st;
    if (num_splits < 0 || num_splits > FA2_MAX_SPLITS) return FA2_ERR_ARG;
    int S = 0;
    size_t need = 0;
    if (num_splits > 0) {                     // sizes known: reject before any HIP call
        if ((st = splitkv_size(p, num_splits, d, causal, &S, &need)) != FA2_OK) return st;
        if (S > 1 && need > (size_t)FA2_STATIC_SCRATCH_BYTES) return FA2_ERR_SCRATCH;
    }
    if ((st = check_device()) != FA2_OK) return st;
    if ((st = splitkv_size(p, num_splits, d, causal, &S, &need)) != FA2_OK) return st;
    if (S > 1 && need > (size_t)FA2_STATIC_SCRATCH_BYTES) return FA2_ERR_SCRATCH;
    void *ws = S > 1 ? scratch_on_device() : nullptr;
    if (S > 1 && !ws) return FA2_ERR_DEVICE;
    return splitkv_launch(p, S, d, causal, false, ws, o, lse, static_cast<hipStream_t>(stream));
}

int fa2_fwd_splitkv(const void *q, const void *k, const void *v, void *o, float *lse,
                    int B, int H, int Lq, int Lk, int d, float scale, int causal,
                    int num_splits, void *workspace, size_t workspace_bytes_given, void *stream)
{
    return fwd_splitkv16(q, k, v, o, lse, B, H, Lq, Lk, d, scale, causal, num_splits, workspace,
                         workspace_bytes_given, false, stream);
}

int fa2_fwd_splitkv_f16(const void *q, const void *k, const void *v, void *o, float *lse,
                        int B, int H, int Lq, int Lk, int d, float scale, int causal,
                        int num_splits, void *workspace, size_t workspace_bytes_given, void *stream)
{
    return fwd_splitkv16(q, k, v, o, lse, B, H, Lq, Lk, d, scale, causal, num_splits, workspace,
                         workspace_bytes_given, true, stream);
}

int fa2_merge_partials(const float *o_parts, const float *lse_parts, int n_parts, int64_t rows,
                       int d, void *o, float *lse, void *stream)
{
    return merge16(o_parts, lse_parts, n_parts, rows, d, o, lse, false, stream);
}

int fa2_merge_partials_f16(const float *o_parts, const float *lse_parts, int n_parts, int64_t rows,
                           int d, void *o, float *lse, void *stream)
{
    return merge16(o_parts, lse_parts, n_parts, rows, d, o, lse, true, stream);
}

size_t fa2_bwd_workspace_bytes(int B, int H, int Lq)
{
    return bwd_workspace_bytes(B, H, Lq);
}

int fa2_bwd(const void *q, const void *k, const void *v, const void *o, const float *lse, const void *dout,
            void *dq, void *dk, void *dv, int B, int H, int Lq, int Lk, int d, float scale, int causal,
            void *workspace, size_t workspace_bytes_given, void *stream)
{
    return bwd16(q, k, v, o, lse, dout, dq, dk, dv, B, H, Lq, Lk, d, scale, causal, nullptr, nullptr,
                 workspace, workspace_bytes_given, false, stream);
}

int fa2_bwd_f16(const void *q, const void *k, const void *v, const void *o, const float *lse, const void *dout,
                void *dq, void *dk, void *dv, int B, int H, int Lq, int Lk, int d, float scale, int causal,
                void *workspace, size_t workspace_bytes_given, void *stream)
{
    return bwd16(q, k, v, o, lse, dout, dq, dk, dv, B, H, Lq, Lk, d, scale, causal, nullptr, nullptr,
                 workspace, workspace_bytes_given, true, stream);
}

int fa2_bwd_window(const void *q, const void *k, const void *v, const void *o, const float *lse, const void *dout,
                   void *dq, void *dk, void *dv, int B, int H, int Lq, int Lk, int d, float scale,
                   int window_left, int window_right, void *workspace, size_t workspace_bytes_given,
                   void *stream)
{
    const Window w{window_left, window_right};
    return bwd16(q, k, v, o, lse, dout, dq, dk, dv, B, H, Lq, Lk, d, scale, 0, &w, nullptr, workspace,
                 workspace_bytes_given, false, stream);
}

int fa2_bwd_window_f16(const void *q, const void *k, const void *v, const void *o, const float *lse,
                       const void *dout, void *dq, void *dk, void *dv, int B, int H, int Lq, int Lk, int d,
                       float scale, int window_left, int window_right, void *workspace,
                       size_t workspace_bytes_given, void *stream)
{
    const Window w{window_left, window_right};
    return bwd16(q, k, v, o, lse, dout, dq, dk, dv, B, H, Lq, Lk, d, scale, 0, &w, nullptr, workspace,
                 workspace_bytes_given, true, stream);
}

int fa2_bwd_dropout(const void *q, const void *k, const void *v, const void *o, const float *lse, const void *dout,
                    void *dq, void *dk, void *dv, int B, int H, int Lq, int Lk, int d, float scale, int causal,
                    double dropout_p, uint64_t seed, uint32_t offset, void *workspace,
                    size_t workspace_bytes_given, void *stream)
{
    const Dropout dr{dropout_p, seed, offset};
    return bwd16(q, k, v, o, lse, dout, dq, dk, dv, B, H, Lq, Lk, d, scale, causal, nullptr, &dr, workspace,
                 workspace_bytes_given, false, stream);
}

int fa2_bwd_dropout_f16(const void *q, const void *k, const void *v, const void *o, const float *lse,
                        const void *dout, void *dq, void *dk, void *dv, int B, int H, int Lq, int Lk, int d,
                        float scale, int causal, double dropout_p, uint64_t seed, uint32_t offset,
                        void *workspace, size_t workspace_bytes_given, void *stream)
{
    const Dropout dr{dropout_p, seed, offset};
    return bwd16(q, k, v, o, lse, dout, dq, dk, dv, B, H, Lq, Lk, d, scale, causal, nullptr, &dr, workspace,
                 workspace_bytes_given, true, stream);
}

const char *fa2_status_string(int status)
{
    switch (status) {
    case FA2_OK: return "ok";
    case FA2_ERR_NULL: return "a tensor pointer is NULL";
    case FA2_ERR_DIM: return "B, H, Lq, Lk must be positive and the sizes must fit (one head's K below 2 GiB)";
    case FA2_ERR_UNSUPPORTED_D: return "head dimension d must be 32, 64 or 128 (or 96 or 256 for 16-bit data)";
    case FA2_ERR_ARG:
        return "an argument is out of range: causal must be 0 or 1, scale finite and positive, "
               "num_splits in [0, FA2_MAX_SPLITS], dropout_p in [0, 1)";
    case FA2_ERR_ALIGN: return "tensor pointers must be 16-byte aligned";
    case FA2_ERR_DEVICE: return "no usable gfx950 HIP device";
    case FA2_ERR_LAUNCH: return "kernel launch failed";
    case FA2_ERR_WORKSPACE: return "workspace missing or too small";
    case FA2_ERR_SCRATCH:
        return "the split-KV partial results need more than the library's static scratch "
               "(FA2_STATIC_SCRATCH_BYTES); use fa2_fwd_splitkv with a workspace";
    default: return "unknown status";
    }
}

}  // extern "C"
