// C ABI of the fused conv / GEMM-logsumexp library: argument validation, the
// per-(device, stream) workspace cache, and dispatch to the kernels.
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <map>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "../../include/fconv.h"
#include "internal.h"

#define FCONV_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
    g_last_error = msg;
    return code;
}

int ok() {
    g_last_error.clear();
    return FCONV_OK;
}

constexpr long long kMaxElems = (1LL << 31) - 1;

struct Workspace {
    void* ptr = nullptr;
    size_t bytes = 0;
};

std::mutex g_ws_mutex;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;

// Returns a device buffer of at least `bytes` owned by the library for (current device,
// stream). Growing it waits for the stream first (earlier work on it may still read the
// old buffer) and then replaces the buffer; calls on other streams use their own.
int get_workspace(hipStream_t stream, size_t bytes, void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(FCONV_EHIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    Workspace& ws = g_ws[std::make_pair(dev, stream)];
    if (ws.bytes < bytes) {
        if (ws.ptr) {
            e = hipStreamSynchronize(stream);
            if (e != hipSuccess)
                return fail(FCONV_EHIP, std::string("hipStreamSynchronize: ") + hipGetErrorString(e));
            (void)hipFree(ws.ptr);
            ws.ptr = nullptr;
            ws.bytes = 0;
        }
        const size_t want = bytes < (1u << 20) ? (1u << 20) : bytes;
        e = hipMalloc(&ws.ptr, want);
        if (e != hipSuccess) {
            ws.ptr = nullptr;
            (void)hipGetLastError();
            return fail(FCONV_ENOMEM, "workspace hipMalloc(" + std::to_string(want) + "): " + hipGetErrorString(e));
        }
        ws.bytes = want;
    }
    *out = ws.ptr;
    return FCONV_OK;
}

// Per-kernel event timing (fconv_profile / fconv_profile_read).
struct EventTimer final : fconv::KernelTimer {
    struct Pending {
        std::string kernel;
        hipEvent_t start, stop;
    };
    std::mutex mu;
    std::atomic<bool> enabled{false};
    std::vector<Pending> pending;
    // start events of the kernels in flight, per (kernel, stream): calls on several
    // streams may be timed at once
    std::map<std::pair<std::string, hipStream_t>, hipEvent_t> open;
    std::map<std::string, std::pair<double, long long>> totals;  // ms, launches

    void begin(const char* kernel, hipStream_t s) override {
        hipEvent_t e;
        if (hipEventCreate(&e) != hipSuccess) return;
        (void)hipEventRecord(e, s);
        std::lock_guard<std::mutex> lock(mu);
        hipEvent_t& slot = open[std::make_pair(std::string(kernel), s)];
        if (slot) (void)hipEventDestroy(slot);  // a begin without its end: drop the stale start
        slot = e;
    }
    void end(const char* kernel, hipStream_t s) override {
        hipEvent_t e;
        if (hipEventCreate(&e) != hipSuccess) return;
        (void)hipEventRecord(e, s);
        std::lock_guard<std::mutex> lock(mu);
        auto it = open.find(std::make_pair(std::string(kernel), s));
        if (it == open.end()) {
            (void)hipEventDestroy(e);
            return;
        }
        pending.push_back({std::string(kernel), it->second, e});
        open.erase(it);
    }
    // Waits for recorded events and folds them into the totals.
    int drain() {
        std::lock_guard<std::mutex> lock(mu);
        int rc = FCONV_OK;
        for (auto& p : pending) {
            float ms = 0.f;
            if (hipEventSynchronize(p.stop) != hipSuccess || hipEventElapsedTime(&ms, p.start, p.stop) != hipSuccess)
                rc = FCONV_EHIP;
            auto& t = totals[p.kernel];
            t.first += ms;
            t.second += 1;
            (void)hipEventDestroy(p.start);
            (void)hipEventDestroy(p.stop);
        }
        pending.clear();
        return rc;
    }
};

EventTimer g_timer;

fconv::KernelTimer* active_timer() { return g_timer.enabled.load() ? &g_timer : nullptr; }

// Brackets a single-kernel entry point with the timer (when profiling is on).
struct ActivePlanTimer {
    fconv::KernelTimer* t;
    const char* name;
    hipStream_t s;
    ActivePlanTimer(fconv::KernelTimer* t_, const char* n, hipStream_t s_) : t(t_), name(n), s(s_) {
        if (t) t->begin(name, s);
    }
    ~ActivePlanTimer() {
        if (t) t->end(name, s);
    }
};

bool overlaps(const void* a, size_t abytes, const void* b, size_t bbytes) {
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + bbytes && b0 < a0 + abytes;
}

bool known_act(int a) {
    return a == FCONV_ACT_NONE || a == FCONV_ACT_GELU || a == FCONV_ACT_MISH2 || a == FCONV_ACT_GELU_TANH;
}

}  // namespace

FCONV_API int fconv_version(void) { return 100; }

FCONV_API const char* fconv_last_error(void) { return g_last_error.c_str(); }

namespace {

// Scratch of fconv_act_pool_noalloc: a file-scope device array, so the entry point needs
// no allocation. Each GPU the library runs on holds its own copy (at its own address) until
// the process ends. In host code `scratch` names a host-side stand-in; its device address
// comes from hipGetSymbolAddress, looked up once per device with that device current.
constexpr size_t kNoAllocScratchBytes = FCONV_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device.
int noalloc_scratch(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(FCONV_EHIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(FCONV_EUNSUPPORTED, "device index beyond the scratch table");
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(FCONV_EHIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return FCONV_OK;
}

int conv_impl(const char* name, const void* x, const void* w, const float* b, int N, int Cin, int H, int W,
              int Cout, int K, int stride, int pad, int act, int pool, float* out, hipStream_t stream,
              bool noalloc = false) {
    const std::string fn(name);
    if (!x || !w || !b || !out) return fail(FCONV_EINVAL, fn + ": null pointer argument");
    if (N < 1 || Cin < 1 || Cout < 1) return fail(FCONV_EINVAL, fn + ": N, Cin and Cout must be >= 1");
    if (K < 1 || stride < 1 || pad < 0) return fail(FCONV_EINVAL, fn + ": need K >= 1, stride >= 1, pad >= 0");
    if (H < 1 || W < 1 || H + 2 * pad < K || W + 2 * pad < K)
        return fail(FCONV_EINVAL, fn + ": the padded input is smaller than the kernel (H and W must be >= 3 for "
                                       "a 3x3 valid conv)");
    const int kind = act & 0xFF, dt = act & ~0xFF;
    if (!known_act(kind)) return fail(FCONV_EINVAL, fn + ": unknown activation " + std::to_string(kind));
    if (dt != FCONV_DT_F32 && dt != FCONV_DT_BF16) return fail(FCONV_EINVAL, fn + ": unknown dtype bits in act");
    if (pool != 0 && pool != 1) return fail(FCONV_EINVAL, fn + ": pool must be 0 or 1");
    const bool bf16_in = (act & ~0xFF) == FCONV_DT_BF16;
    // 3x3 stride 1: valid layers, and bf16 "same" layers (pad 1) of 256 or more output channels
    // with 16-byte halo runs, take the 3x3 kernels
    const bool fast = K == 3 && stride == 1 && (pad == 0 || (pad == 1 && fconv::conv3x3_same_wide(bf16_in, W, Cout, x)));
    if (!fast && !fconv::conv_general_supported(K, stride))
        return fail(FCONV_EUNSUPPORTED, fn + ": kernel size must be 1, 3 or 5 and stride 1 or 2");
    if (pad >= K) return fail(FCONV_EUNSUPPORTED, fn + ": padding must be smaller than the kernel size");
    const long long OH = (H + 2LL * pad - K) / stride + 1, OW = (W + 2LL * pad - K) / stride + 1;
    const long long nx = (long long)N * Cin * H * W, nw = (long long)Cout * Cin * K * K;
    const long long nout = pool ? (long long)N * Cout : (long long)N * Cout * OH * OW;
    if (nx > kMaxElems || nw > kMaxElems || nout > kMaxElems)
        return fail(FCONV_EINVAL, fn + ": a tensor has 2^31 or more elements");
    const size_t esz = dt == FCONV_DT_BF16 ? 2 : 4;
    const size_t ob = (size_t)nout * 4;
    if (overlaps(out, ob, x, nx * esz) || overlaps(out, ob, w, nw * esz) || overlaps(out, ob, b, (size_t)Cout * 4))
        return fail(FCONV_EINVAL, fn + ": out overlaps an input");

    const bool bf16 = dt == FCONV_DT_BF16;
    const fconv::ConvPlan plan = fast ? fconv::plan_conv(bf16, kind, pool, N, Cin, H, W, Cout, x, pad)
                                      : fconv::plan_conv_general(bf16, kind, pool, N, Cin, H, W, Cout, K, stride, pad);
    if (plan.grid() > 0x7FFFFFFFLL) return fail(FCONV_EUNSUPPORTED, fn + ": launch grid too large");
    // The kernels address one image of x, and the repacked weights, with 32-bit byte offsets.
    if ((long long)Cin * H * W * (long long)esz > 0x7FFF0000LL || (long long)plan.wpack_bytes > 0x7FFF0000LL)
        return fail(FCONV_EUNSUPPORTED, fn + ": one image (or the weights) exceeds 2 GiB");
    void* ws = nullptr;
    if (noalloc) {
        if (plan.workspace_bytes() > kNoAllocScratchBytes)
            return fail(FCONV_EINVAL, fn + ": needs " + std::to_string(plan.workspace_bytes()) +
                                          " bytes of scratch (repacked weights + pool partials); the static scratch "
                                          "holds " + std::to_string(kNoAllocScratchBytes));
        int rc = noalloc_scratch(&ws);
        if (rc != FCONV_OK) return rc;
    } else {
        int rc = get_workspace(stream, plan.workspace_bytes(), &ws);
        if (rc != FCONV_OK) return rc;
    }
    // the allocation-free entry point records no timing events either
    fconv::KernelTimer* timer = noalloc ? nullptr : active_timer();
    hipError_t e = fast ? fconv::launch_conv(plan, x, w, b, out, ws, stream, timer)
                        : fconv::launch_conv_general(plan, x, w, b, out, ws, stream, timer);
    if (e != hipSuccess) return fail(FCONV_EHIP, fn + " launch: " + hipGetErrorString(e));
    return ok();
}

}  // namespace

FCONV_API int fconv_act_pool(const void* x, const void* w, const float* b, int N, int Cin, int H, int W,
                             int Cout, int act, int pool, float* out, hipStream_t stream) {
    return conv_impl("fconv_act_pool", x, w, b, N, Cin, H, W, Cout, 3, 1, 0, act, pool, out, stream);
}

FCONV_API int fconv_act_pool_noalloc(const void* x, const void* w, const float* b, int N, int Cin, int H, int W,
                                     int Cout, int act, int pool, float* out, hipStream_t stream) {
    return conv_impl("fconv_act_pool_noalloc", x, w, b, N, Cin, H, W, Cout, 3, 1, 0, act, pool, out, stream, true);
}

FCONV_API int fconv2d_act_pool(const void* x, const void* w, const float* b, int N, int Cin, int H, int W,
                               int Cout, int K, int stride, int pad, int act, int pool, float* out,
                               hipStream_t stream) {
    return conv_impl("fconv2d_act_pool", x, w, b, N, Cin, H, W, Cout, K, stride, pad, act, pool, out, stream);
}

namespace {

int gemm_lse_mish_impl(const char* name, bool bf16, const void* x, const void* w, const float* b, int M, int K,
                       int N, float scale, float cmin, float cmax, float* out, hipStream_t stream) {
    const std::string fn(name);
    if (!x || !w || !b || !out) return fail(FCONV_EINVAL, fn + ": null pointer argument");
    if (M < 1 || K < 1 || N < 1) return fail(FCONV_EINVAL, fn + ": M, K and N must be >= 1");
    if (!std::isfinite(scale)) return fail(FCONV_EINVAL, fn + ": scale must be finite");
    if (std::isnan(cmin) || std::isnan(cmax) || cmin > cmax)
        return fail(FCONV_EINVAL, fn + ": need cmin <= cmax (not NaN)");
    const long long nx = (long long)M * K, nw = (long long)N * K;
    if (nx > kMaxElems || nw > kMaxElems) return fail(FCONV_EINVAL, fn + ": a tensor has 2^31 or more elements");
    const size_t esz = bf16 ? 2 : 4, ob = (size_t)M * 4;
    if (overlaps(out, ob, x, nx * esz) || overlaps(out, ob, w, nw * esz) || overlaps(out, ob, b, (size_t)N * 4))
        return fail(FCONV_EINVAL, fn + ": out overlaps an input");

    const fconv::GemmPlan plan = fconv::plan_gemm(bf16, M, K, N, x, w);
    if ((long long)plan.tilesM * plan.tilesN > 0x7FFFFFFFLL) return fail(FCONV_EUNSUPPORTED, fn + ": launch grid too large");
    void* ws = nullptr;
    int rc = get_workspace(stream, plan.workspace_bytes(), &ws);
    if (rc != FCONV_OK) return rc;
    hipError_t e = fconv::launch_gemm_lse(plan, x, w, b, scale, cmin, cmax, out, ws, stream, active_timer());
    if (e != hipSuccess) return fail(FCONV_EHIP, fn + " launch: " + hipGetErrorString(e));
    return ok();
}

}  // namespace

FCONV_API int fgemm_lse_mish(const float* x, const float* w, const float* b, int M, int K, int N, float scale,
                             float cmin, float cmax, float* out, hipStream_t stream) {
    return gemm_lse_mish_impl("fgemm_lse_mish", false, x, w, b, M, K, N, scale, cmin, cmax, out, stream);
}

FCONV_API int fgemm_lse_mish_bf16(const void* x, const void* w, const float* b, int M, int K, int N, float scale,
                                  float cmin, float cmax, float* out, hipStream_t stream) {
    return gemm_lse_mish_impl("fgemm_lse_mish_bf16", true, x, w, b, M, K, N, scale, cmin, cmax, out, stream);
}

FCONV_API int fact_pool(const float* x, int N, int C, int H, int W, int act, float* out, hipStream_t stream) {
    if (!x || !out) return fail(FCONV_EINVAL, "fact_pool: null pointer argument");
    if (N < 1 || C < 1 || H < 1 || W < 1) return fail(FCONV_EINVAL, "fact_pool: N, C, H and W must be >= 1");
    if (!known_act(act))
        return fail(FCONV_EINVAL, "fact_pool: act must be FCONV_ACT_NONE, _GELU, _MISH2 or _GELU_TANH (float32 only)");
    const long long nx = (long long)N * C * H * W, nout = (long long)N * C;
    if (nx > kMaxElems) return fail(FCONV_EINVAL, "fact_pool: a tensor has 2^31 or more elements");
    if (overlaps(out, (size_t)nout * 4, x, (size_t)nx * 4)) return fail(FCONV_EINVAL, "fact_pool: out overlaps x");
    ActivePlanTimer t(active_timer(), "act_pool_map", stream);
    hipError_t e = fconv::launch_act_pool_map(x, N, C, H, W, act, out, stream);
    if (e != hipSuccess) return fail(FCONV_EHIP, std::string("fact_pool launch: ") + hipGetErrorString(e));
    return ok();
}

FCONV_API int fact_elementwise(const float* x, long long count, int act, float* out, hipStream_t stream) {
    if (!x || !out) return fail(FCONV_EINVAL, "fact_elementwise: null pointer argument");
    if (count < 0) return fail(FCONV_EINVAL, "fact_elementwise: count must be >= 0");
    if (!known_act(act))
        return fail(FCONV_EINVAL,
                    "fact_elementwise: act must be FCONV_ACT_NONE, _GELU, _MISH2 or _GELU_TANH (float32 only)");
    if (count > (1LL << 40)) return fail(FCONV_EINVAL, "fact_elementwise: count too large");
    if (out != x && overlaps(out, (size_t)count * 4, x, (size_t)count * 4))
        return fail(FCONV_EINVAL, "fact_elementwise: out partially overlaps x (only out == x is allowed)");
    ActivePlanTimer t(active_timer(), "act_elementwise", stream);
    hipError_t e = fconv::launch_act_elementwise(x, count, act, out, stream);
    if (e != hipSuccess) return fail(FCONV_EHIP, std::string("fact_elementwise launch: ") + hipGetErrorString(e));
    return ok();
}

FCONV_API int flse_mish_rows(const float* y, int M, int N, float scale, float cmin, float cmax, float* out,
                             hipStream_t stream) {
    if (!y || !out) return fail(FCONV_EINVAL, "flse_mish_rows: null pointer argument");
    if (M < 1 || N < 1) return fail(FCONV_EINVAL, "flse_mish_rows: M and N must be >= 1");
    if (!std::isfinite(scale)) return fail(FCONV_EINVAL, "flse_mish_rows: scale must be finite");
    if (std::isnan(cmin) || std::isnan(cmax) || cmin > cmax)
        return fail(FCONV_EINVAL, "flse_mish_rows: need cmin <= cmax (not NaN)");
    const long long ny = (long long)M * N;
    if (ny > kMaxElems) return fail(FCONV_EINVAL, "flse_mish_rows: y has 2^31 or more elements");
    if (overlaps(out, (size_t)M * 4, y, (size_t)ny * 4)) return fail(FCONV_EINVAL, "flse_mish_rows: out overlaps y");
    ActivePlanTimer t(active_timer(), "scale_clamp_lse", stream);
    hipError_t e = fconv::launch_scale_clamp_lse(y, M, N, scale, cmin, cmax, out, stream);
    if (e != hipSuccess) return fail(FCONV_EHIP, std::string("flse_mish_rows launch: ") + hipGetErrorString(e));
    return ok();
}

FCONV_API int fconv_mfma_rate_probe(int dtype, int iters, float* sink, double* flops, hipStream_t stream) {
    if (!sink || !flops) return fail(FCONV_EINVAL, "fconv_mfma_rate_probe: null pointer argument");
    if (dtype != FCONV_DT_F32 && dtype != FCONV_DT_BF16)
        return fail(FCONV_EINVAL, "fconv_mfma_rate_probe: dtype must be FCONV_DT_F32 or FCONV_DT_BF16");
    if (iters < 1 || iters > (1 << 20)) return fail(FCONV_EINVAL, "fconv_mfma_rate_probe: iters must be 1 .. 2^20");
    const bool bf16 = dtype == FCONV_DT_BF16;
    ActivePlanTimer t(active_timer(), "mfma_rate_probe", stream);
    hipError_t e = fconv::launch_mfma_probe(bf16, iters, sink, stream);
    if (e != hipSuccess) return fail(FCONV_EHIP, std::string("fconv_mfma_rate_probe launch: ") + hipGetErrorString(e));
    *flops = fconv::mfma_probe_flops(bf16, iters);
    return ok();
}

FCONV_API int fconv_release(void) {
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    int rc = FCONV_OK;
    int cur = 0;
    const bool have_dev = hipGetDevice(&cur) == hipSuccess;
    for (auto& kv : g_ws) {
        if (!kv.second.ptr) continue;
        // A device-wide sync: the stream itself may already have been destroyed.
        if (hipSetDevice(kv.first.first) != hipSuccess || hipDeviceSynchronize() != hipSuccess ||
            hipFree(kv.second.ptr) != hipSuccess)
            rc = fail(FCONV_EHIP, "fconv_release: HIP error while freeing a workspace");
    }
    g_ws.clear();
    if (have_dev) (void)hipSetDevice(cur);
    if (rc == FCONV_OK) return ok();
    return rc;
}

FCONV_API int fconv_profile(int enable) {
    int rc = g_timer.drain();
    {
        std::lock_guard<std::mutex> lock(g_timer.mu);
        g_timer.totals.clear();
        g_timer.enabled = enable != 0;
    }
    if (rc != FCONV_OK) return fail(rc, "fconv_profile: HIP error while draining events");
    return ok();
}

FCONV_API int fconv_profile_read(const char* kernel, double* total_ms, long long* launches) {
    if (!kernel || !total_ms || !launches) return fail(FCONV_EINVAL, "fconv_profile_read: null argument");
    int rc = g_timer.drain();
    if (rc != FCONV_OK) return fail(rc, "fconv_profile_read: HIP error while draining events");
    std::lock_guard<std::mutex> lock(g_timer.mu);
    auto it = g_timer.totals.find(kernel);
    *total_ms = it == g_timer.totals.end() ? 0.0 : it->second.first;
    *launches = it == g_timer.totals.end() ? 0 : it->second.second;
    return ok();
}
