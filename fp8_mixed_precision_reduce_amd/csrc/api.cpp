// extern "C" entry points of libfp8lin: argument validation (on the host,
// before anything is enqueued), dispatch to the kernel launchers, the layer
// compositions, error reporting and the optional launch timer.
//
// Every entry point follows the same shape: validate -> launch(es) on the
// caller's stream -> return a status.  No entry point synchronises, allocates
// device memory, or lets a C++ exception escape.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "fp8lin.h"
#include "common.h"

namespace fp8lin {

// ------------------------------------------------------------ error reporting
namespace {
thread_local char g_err[512] = "";

int32_t fail(int32_t status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return status;
}

int32_t ok() {
    g_err[0] = '\0';
    return FP8LIN_OK;
}

int32_t hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(FP8LIN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
bool is_hp(int32_t dt) { return dt == FP8LIN_F32 || dt == FP8LIN_BF16; }
bool is_fp8(int32_t dt) { return dt == FP8LIN_E4M3 || dt == FP8LIN_E5M2; }
int64_t elem_size(int32_t dt) { return dt == FP8LIN_F32 ? 4 : dt == FP8LIN_BF16 ? 2 : 1; }

// [lo, hi) byte ranges of two buffers overlap?
bool overlap(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
    if (!a || !b || abytes <= 0 || bbytes <= 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

constexpr int64_t kMaxElems = int64_t(1) << 40;
constexpr int64_t kCtMaxRows = int64_t(1) << 24, kCtMaxCols = int64_t(1) << 22;
constexpr int64_t kMaxK = int64_t(1) << 23;

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }
}  // namespace

// ---------------------------------------------------------------- launch timer
namespace {
struct Timer {
    std::mutex mu;
    std::vector<hipEvent_t> ev;     // 2 per record
    std::vector<int32_t> kinds;
    int32_t used = 0;
    std::atomic<int32_t> capacity{0};   // read without the lock on every launch (0: timing off)
    int32_t pending_kind = -1;
};
Timer g_timer;
}  // namespace

void timing_before(int kind, hipStream_t stream) {
    if (g_timer.capacity.load(std::memory_order_relaxed) == 0) return;
    std::lock_guard<std::mutex> lk(g_timer.mu);
    if (g_timer.used >= g_timer.capacity) return;
    if (hipEventRecord(g_timer.ev[2 * g_timer.used], stream) != hipSuccess) return;   // launch goes untimed
    g_timer.pending_kind = kind;
}

void timing_after(hipStream_t stream) {
    if (g_timer.capacity.load(std::memory_order_relaxed) == 0) return;
    std::lock_guard<std::mutex> lk(g_timer.mu);
    if (g_timer.pending_kind < 0) return;
    if (hipEventRecord(g_timer.ev[2 * g_timer.used + 1], stream) != hipSuccess) {
        g_timer.pending_kind = -1;
        return;
    }
    g_timer.kinds[g_timer.used] = g_timer.pending_kind;
    g_timer.pending_kind = -1;
    ++g_timer.used;
}

}  // namespace fp8lin

using namespace fp8lin;

extern "C" {

int32_t fp8lin_abi_version(void) { return FP8LIN_ABI_VERSION; }

const char* fp8lin_last_error(void) { return g_err; }

const char* fp8lin_status_name(int32_t s) {
    switch (s) {
        case FP8LIN_OK: return "FP8LIN_OK";
        case FP8LIN_ERR_NULL: return "FP8LIN_ERR_NULL";
        case FP8LIN_ERR_SHAPE: return "FP8LIN_ERR_SHAPE";
        case FP8LIN_ERR_ALIGN: return "FP8LIN_ERR_ALIGN";
        case FP8LIN_ERR_DTYPE: return "FP8LIN_ERR_DTYPE";
        case FP8LIN_ERR_ARG: return "FP8LIN_ERR_ARG";
        case FP8LIN_ERR_HIP: return "FP8LIN_ERR_HIP";
        case FP8LIN_ERR_UNSUPPORTED: return "FP8LIN_ERR_UNSUPPORTED";
        default: return "FP8LIN_UNKNOWN_STATUS";
    }
}

int64_t fp8lin_dbias_workspace_bytes(int64_t rows, int64_t cols) {
    return cast_transpose_dbias_ws_bytes(rows, cols);
}

int32_t fp8lin_clock_sample(uint64_t* out, int32_t wait_us, void* stream) {
    if (!out) return fail(FP8LIN_ERR_NULL, "fp8lin_clock_sample: out is null");
    if (!aligned(out, 8)) return fail(FP8LIN_ERR_ALIGN, "fp8lin_clock_sample: out not 8-byte aligned");
    if (wait_us < 1 || wait_us > 1000000)
        return fail(FP8LIN_ERR_ARG, "fp8lin_clock_sample: wait_us=%d outside 1..1000000", wait_us);
    return hip_status(launch_clock_sample(reinterpret_cast<unsigned long long*>(out), (int64_t)wait_us * 100,
                                          as_stream(stream)),
                      "fp8lin_clock_sample");
}

int32_t fp8lin_stream_probe(const void* src, void* dst, int64_t bytes, int32_t mode, void* stream) {
    const char* fn = "fp8lin_stream_probe";
    if (mode < 0 || mode > 4)
        return fail(FP8LIN_ERR_ARG, "%s: mode %d is not 0 (read), 1 / 2 (copy) or 3 / 4 (copy twice)", fn, mode);
    if (bytes < 0 || bytes % 16 || bytes > kMaxElems) return fail(FP8LIN_ERR_SHAPE, "%s: bytes=%lld", fn, (long long)bytes);
    if (bytes > 0 && (!src || !dst)) return fail(FP8LIN_ERR_NULL, "%s: null pointer", fn);
    if (!aligned(src, 16) || !aligned(dst, 16)) return fail(FP8LIN_ERR_ALIGN, "%s: misaligned pointer", fn);
    if (overlap(src, bytes, dst, mode == 0 ? 8192 : mode <= 2 ? bytes : 2 * bytes))
        return fail(FP8LIN_ERR_ARG, "%s: dst overlaps src", fn);
    return hip_status(launch_stream_probe(src, dst, bytes, mode, as_stream(stream)), fn);
}

int32_t fp8lin_timing_enable(int32_t capacity) {
    std::lock_guard<std::mutex> lk(g_timer.mu);
    for (hipEvent_t e : g_timer.ev) (void)hipEventDestroy(e);
    g_timer.ev.clear();
    g_timer.kinds.clear();
    g_timer.used = 0;
    g_timer.capacity = 0;
    g_timer.pending_kind = -1;
    if (capacity < 0 || capacity > (1 << 20)) return fail(FP8LIN_ERR_ARG, "timing capacity %d out of range", capacity);
    if (capacity == 0) return ok();
    g_timer.ev.resize(2 * (size_t)capacity);
    g_timer.kinds.assign(capacity, 0);
    for (size_t i = 0; i < g_timer.ev.size(); ++i) {
        const hipError_t r = hipEventCreate(&g_timer.ev[i]);
        if (r != hipSuccess) {
            for (size_t j = 0; j < i; ++j) (void)hipEventDestroy(g_timer.ev[j]);
            g_timer.ev.clear();
            g_timer.kinds.clear();
            return hip_status(r, "hipEventCreate");
        }
    }
    g_timer.capacity = capacity;
    return ok();
}

int32_t fp8lin_timing_read(int32_t* kinds, float* ms, int32_t max) {
    std::lock_guard<std::mutex> lk(g_timer.mu);
    const int32_t n = g_timer.used < max ? g_timer.used : max;
    for (int32_t i = 0; i < n; ++i) {
        float t = -1.0f;                // -1: the events could not be read
        if (hipEventSynchronize(g_timer.ev[2 * i + 1]) != hipSuccess ||
            hipEventElapsedTime(&t, g_timer.ev[2 * i], g_timer.ev[2 * i + 1]) != hipSuccess)
            t = -1.0f;
        if (kinds) kinds[i] = g_timer.kinds[i];
        if (ms) ms[i] = t;
    }
    g_timer.used = 0;
    return n;
}

// ------------------------------------------------------------------- amax
// ------------------------------------------------------ saturation counters
namespace {
// Counters registered per amax slot, process-wide.  Looked up at each cast
// launch; with none registered the lookup is one atomic load.
constexpr int kMaxSatCounters = 256;
struct SatEntry {
    const float* slot;
    uint32_t* counter;
};
std::mutex g_sat_mu;
SatEntry g_sat[kMaxSatCounters];
std::atomic<int> g_sat_n{0};

uint32_t* sat_counter(const float* slot) {
    if (!slot || g_sat_n.load(std::memory_order_acquire) == 0) return nullptr;
    std::lock_guard<std::mutex> lk(g_sat_mu);
    const int n = g_sat_n.load(std::memory_order_relaxed);
    for (int i = 0; i < n; ++i)
        if (g_sat[i].slot == slot) return g_sat[i].counter;
    return nullptr;
}
}  // namespace

int32_t fp8lin_count_saturation(const float* amax_slot, uint32_t* counter) {
    const char* fn = "fp8lin_count_saturation";
    if (!amax_slot) return fail(FP8LIN_ERR_NULL, "%s: null amax slot", fn);
    if (!aligned(amax_slot, 4) || !aligned(counter, 4)) return fail(FP8LIN_ERR_ALIGN, "%s: misaligned pointer", fn);
    std::lock_guard<std::mutex> lk(g_sat_mu);
    const int n = g_sat_n.load(std::memory_order_relaxed);
    for (int i = 0; i < n; ++i) {
        if (g_sat[i].slot != amax_slot) continue;
        if (counter) {
            g_sat[i].counter = counter;
        } else {
            g_sat[i] = g_sat[n - 1];
            g_sat_n.store(n - 1, std::memory_order_release);
        }
        return FP8LIN_OK;
    }
    if (!counter) return FP8LIN_OK;
    if (n == kMaxSatCounters) return fail(FP8LIN_ERR_ARG, "%s: %d counters already registered", fn, n);
    g_sat[n] = SatEntry{amax_slot, counter};
    g_sat_n.store(n + 1, std::memory_order_release);
    return FP8LIN_OK;
}

int32_t fp8_amax(const void* x, int32_t x_dtype, int64_t n, float* amax_slot, void* stream) {
    if (!is_hp(x_dtype)) return fail(FP8LIN_ERR_DTYPE, "fp8_amax: x_dtype %d must be F32 or BF16", x_dtype);
    if (n < 0 || n > kMaxElems) return fail(FP8LIN_ERR_SHAPE, "fp8_amax: n=%lld out of range", (long long)n);
    if (!amax_slot || (n > 0 && !x)) return fail(FP8LIN_ERR_NULL, "fp8_amax: null pointer");
    if (!aligned(x, 16) || !aligned(amax_slot, 4)) return fail(FP8LIN_ERR_ALIGN, "fp8_amax: misaligned pointer");
    return hip_status(launch_amax(x, x_dtype, n, amax_slot, as_stream(stream)), "fp8_amax");
}

// ----------------------------------------------------------- scale update
namespace {
int32_t check_scale_args(const char* fn, float* amax_history, float* scale, float* scale_inv, const uint8_t* formats,
                         int32_t n_tensors, const fp8lin_recipe* recipe) {
    if (!amax_history || !scale || !scale_inv || !formats || !recipe) return fail(FP8LIN_ERR_NULL, "%s: null pointer", fn);
    if (n_tensors < 1 || n_tensors > 4096)
        return fail(FP8LIN_ERR_SHAPE, "%s: n_tensors=%d not in [1, 4096]", fn, n_tensors);
    if (recipe->history_len < 1 || recipe->history_len > 65536)
        return fail(FP8LIN_ERR_ARG, "%s: history_len=%d not in [1, 65536]", fn, recipe->history_len);
    if (recipe->margin < 0 || recipe->margin > 127)
        return fail(FP8LIN_ERR_ARG, "%s: margin=%d not in [0, 127]", fn, recipe->margin);
    if (recipe->amax_compute_algo != FP8LIN_AMAX_MAX)
        return fail(FP8LIN_ERR_UNSUPPORTED, "%s: amax_compute_algo %d (only max)", fn, recipe->amax_compute_algo);
    for (int32_t t = 0; t < n_tensors; ++t)
        if (!is_fp8(formats[t])) return fail(FP8LIN_ERR_DTYPE, "%s: formats[%d]=%d is not E4M3/E5M2", fn, t, formats[t]);
    if (!aligned(amax_history, 4) || !aligned(scale, 4) || !aligned(scale_inv, 4))
        return fail(FP8LIN_ERR_ALIGN, "%s: misaligned pointer", fn);
    const int64_t hb = (int64_t)n_tensors * recipe->history_len * 4, sb = (int64_t)n_tensors * 4;
    if (overlap(amax_history, hb, scale, sb) || overlap(amax_history, hb, scale_inv, sb) ||
        overlap(scale, sb, scale_inv, sb))
        return fail(FP8LIN_ERR_ARG, "%s: history, scale and scale_inv overlap", fn);
    return FP8LIN_OK;
}
}  // namespace

int32_t fp8_amax_scale_update(float* amax_history, float* scale, float* scale_inv, const uint8_t* formats,
                              int32_t n_tensors, const fp8lin_recipe* recipe, void* stream) {
    const char* fn = "fp8_amax_scale_update";
    const int32_t v = check_scale_args(fn, amax_history, scale, scale_inv, formats, n_tensors, recipe);
    if (v != FP8LIN_OK) return v;
    return hip_status(launch_scale_update(amax_history, scale, scale_inv, formats, n_tensors, recipe->history_len,
                                          recipe->margin, as_stream(stream)),
                      fn);
}

int32_t fp8_scale_from_current_amax(float* amax_history, float* scale, float* scale_inv, const uint8_t* formats,
                                    int32_t n_tensors, const fp8lin_recipe* recipe, void* stream) {
    const char* fn = "fp8_scale_from_current_amax";
    const int32_t v = check_scale_args(fn, amax_history, scale, scale_inv, formats, n_tensors, recipe);
    if (v != FP8LIN_OK) return v;
    return hip_status(launch_scale_from_current(amax_history, recipe->history_len, scale, scale_inv, formats,
                                                n_tensors, recipe->margin, as_stream(stream)),
                      fn);
}

// ------------------------------------------------------------------- cast
int32_t fp8_cast(const void* x, int32_t x_dtype, int64_t n, int32_t fp8_dtype, const float* scale, uint8_t* q,
                 float* amax_slot, void* stream) {
    if (!is_hp(x_dtype)) return fail(FP8LIN_ERR_DTYPE, "fp8_cast: x_dtype %d must be F32 or BF16", x_dtype);
    if (!is_fp8(fp8_dtype)) return fail(FP8LIN_ERR_DTYPE, "fp8_cast: fp8_dtype %d must be E4M3 or E5M2", fp8_dtype);
    if (n < 0 || n > kMaxElems) return fail(FP8LIN_ERR_SHAPE, "fp8_cast: n=%lld out of range", (long long)n);
    if (!scale || (n > 0 && (!x || !q))) return fail(FP8LIN_ERR_NULL, "fp8_cast: null pointer");
    if (!aligned(x, 16) || !aligned(q, 16) || !aligned(scale, 4) || !aligned(amax_slot, 4))
        return fail(FP8LIN_ERR_ALIGN, "fp8_cast: misaligned pointer");
    if (overlap(x, n * elem_size(x_dtype), q, n))
        return fail(FP8LIN_ERR_ARG, "fp8_cast: output overlaps input");
    return hip_status(launch_cast(x, x_dtype, n, fp8_dtype, scale, q, amax_slot, as_stream(stream), SinvSnap{},
                                  SatCounts{sat_counter(amax_slot)}),
                      "fp8_cast");
}

namespace {
int32_t check_ct(const char* fn, const void* x, const void* z, int32_t x_dtype, int64_t rows, int64_t cols,
                 int32_t fp8_dtype, const float* scale, uint8_t* q, uint8_t* q_t, float* amax_slot, float* dbias,
                 float* dbias_ws, void* dz_out, bool need_qt = true) {
    if (!is_hp(x_dtype)) return fail(FP8LIN_ERR_DTYPE, "%s: x_dtype %d must be F32 or BF16", fn, x_dtype);
    if (!is_fp8(fp8_dtype)) return fail(FP8LIN_ERR_DTYPE, "%s: fp8_dtype %d must be E4M3 or E5M2", fn, fp8_dtype);
    if (rows < 0 || cols < 0 || rows % 16 || cols % 16 || rows * cols > kMaxElems)
        return fail(FP8LIN_ERR_SHAPE, "%s: rows=%lld cols=%lld must be >= 0 multiples of 16", fn, (long long)rows,
                    (long long)cols);
    // The kernels address a 128 x 128 tile with 32-bit byte offsets below 2^31.
    if (cols >= kCtMaxCols || rows >= kCtMaxRows)
        return fail(FP8LIN_ERR_SHAPE, "%s: rows=%lld cols=%lld (cast-transpose needs rows < 2^24, cols < 2^22)", fn,
                    (long long)rows, (long long)cols);
    const int64_t n = rows * cols;
    if (!scale || (n > 0 && (!x || (need_qt && !q_t)))) return fail(FP8LIN_ERR_NULL, "%s: null pointer", fn);
    if (dbias && cols > 0 && !dbias_ws && rows > 0) return fail(FP8LIN_ERR_NULL, "%s: dbias needs dbias_ws", fn);
    if (!aligned(x, 16) || !aligned(z, 16) || !aligned(q, 16) || !aligned(q_t, 16) || !aligned(dz_out, 16) ||
        !aligned(scale, 4) || !aligned(amax_slot, 4) || !aligned(dbias, 4) || !aligned(dbias_ws, 4))
        return fail(FP8LIN_ERR_ALIGN, "%s: misaligned pointer", fn);
    const int64_t xb = n * elem_size(x_dtype);
    const int64_t wsb = cast_transpose_dbias_ws_bytes(rows, cols);
    const void* outs[4] = {q, q_t, dz_out, dbias ? (const void*)dbias_ws : nullptr};
    const int64_t ob[4] = {n, n, xb, wsb};
    for (int i = 0; i < 4; ++i) {
        if (overlap(outs[i], ob[i], x, xb) || overlap(outs[i], ob[i], z, z ? xb : 0))
            return fail(FP8LIN_ERR_ARG, "%s: an output overlaps an input", fn);
        for (int j = i + 1; j < 4; ++j)
            if (overlap(outs[i], ob[i], outs[j], ob[j])) return fail(FP8LIN_ERR_ARG, "%s: outputs overlap", fn);
    }
    if (dbias && (overlap(dbias, cols * 4, x, xb) || overlap(dbias, cols * 4, dbias_ws, wsb)))
        return fail(FP8LIN_ERR_ARG, "%s: dbias overlaps another buffer", fn);
    return FP8LIN_OK;
}
}  // namespace

int32_t fp8_cast_transpose(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, int32_t fp8_dtype,
                           const float* scale, uint8_t* q, uint8_t* q_t, float* amax_slot, float* dbias,
                           float* dbias_ws, void* stream) {
    const int32_t v = check_ct("fp8_cast_transpose", x, nullptr, x_dtype, rows, cols, fp8_dtype, scale, q, q_t,
                               amax_slot, dbias, dbias_ws, nullptr);
    if (v != FP8LIN_OK) return v;
    return hip_status(launch_cast_transpose(x, nullptr, x_dtype, rows, cols, fp8_dtype, scale, q, q_t, amax_slot,
                                            dbias, dbias_ws, nullptr, as_stream(stream), SinvSnap{},
                                            SatCounts{sat_counter(amax_slot)}),
                      "fp8_cast_transpose");
}

int32_t fp8_cast_transpose_dbias_noalloc(const void* x, int32_t x_dtype, int64_t rows, int64_t cols,
                                         int32_t fp8_dtype, const float* scale, uint8_t* q, uint8_t* q_t,
                                         float* amax_slot, float* dbias, void* stream) {
    const char* fn = "fp8_cast_transpose_dbias_noalloc";
    int32_t v = check_ct(fn, x, nullptr, x_dtype, rows, cols, fp8_dtype, scale, q, q_t, amax_slot, nullptr,
                         nullptr, nullptr);
    if (v != FP8LIN_OK) return v;
    const int64_t n = rows * cols;
    if (!dbias && cols > 0) return fail(FP8LIN_ERR_NULL, "%s: dbias is null", fn);
    if (!aligned(dbias, 4)) return fail(FP8LIN_ERR_ALIGN, "%s: misaligned dbias", fn);
    if (overlap(dbias, cols * 4, x, n * elem_size(x_dtype)) || overlap(dbias, cols * 4, q, n) ||
        overlap(dbias, cols * 4, q_t, n))
        return fail(FP8LIN_ERR_ARG, "%s: dbias overlaps another buffer", fn);
    const int64_t need = cast_transpose_dbias_ws_bytes(rows, cols);
    if (need > kNoAllocScratchBytes)
        return fail(FP8LIN_ERR_ARG, "%s: rows=%lld cols=%lld need %lld bytes of scratch, more than its %lld", fn,
                    (long long)rows, (long long)cols, (long long)need, (long long)kNoAllocScratchBytes);
    float* ws = nullptr;
    if (n > 0) {
        const hipError_t e = noalloc_scratch(as_stream(stream), &ws);
        if (e != hipSuccess) return hip_status(e, fn);
    }
    return hip_status(launch_cast_transpose(x, nullptr, x_dtype, rows, cols, fp8_dtype, scale, q, q_t, amax_slot,
                                            dbias, ws, nullptr, as_stream(stream), SinvSnap{},
                                            SatCounts{sat_counter(amax_slot)}),
                      fn);
}

int32_t fp8_cast_transpose_dgelu(const void* dh, const void* z, int32_t x_dtype, int64_t rows, int64_t cols,
                                 int32_t fp8_dtype, const float* scale, uint8_t* q, uint8_t* q_t, float* amax_slot,
                                 float* dbias, float* dbias_ws, void* dz_out, void* stream) {
    if (rows * cols > 0 && !z) return fail(FP8LIN_ERR_NULL, "fp8_cast_transpose_dgelu: z is null");
    const int32_t v = check_ct("fp8_cast_transpose_dgelu", dh, z, x_dtype, rows, cols, fp8_dtype, scale, q, q_t,
                               amax_slot, dbias, dbias_ws, dz_out);
    if (v != FP8LIN_OK) return v;
    return hip_status(launch_cast_transpose(dh, z, x_dtype, rows, cols, fp8_dtype, scale, q, q_t, amax_slot, dbias,
                                            dbias_ws, dz_out, as_stream(stream), SinvSnap{},
                                            SatCounts{sat_counter(amax_slot)}),
                      "fp8_cast_transpose_dgelu");
}

int32_t fp8_cast_transpose_dual(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, const float* scale_e4m3,
                                uint8_t* q_e4m3, uint8_t* q_e4m3_t, float* amax_slot_e4m3, const float* scale_e5m2,
                                uint8_t* q_e5m2, uint8_t* q_e5m2_t, float* amax_slot_e5m2, void* stream) {
    const char* fn = "fp8_cast_transpose_dual";
    int32_t v;
    // each format's outputs are checked as one cast-transpose, then the two sets against each other
    if ((v = check_ct(fn, x, nullptr, x_dtype, rows, cols, FP8LIN_E4M3, scale_e4m3, q_e4m3, q_e4m3_t,
                      amax_slot_e4m3, nullptr, nullptr, nullptr, false)))
        return v;
    if ((v = check_ct(fn, x, nullptr, x_dtype, rows, cols, FP8LIN_E5M2, scale_e5m2, q_e5m2, q_e5m2_t,
                      amax_slot_e5m2, nullptr, nullptr, nullptr, false)))
        return v;
    const int64_t n = rows * cols;
    if (n > 0 && !q_e4m3 && !q_e4m3_t && !q_e5m2 && !q_e5m2_t) return fail(FP8LIN_ERR_NULL, "%s: no output", fn);
    const uint8_t* a[2] = {q_e4m3, q_e4m3_t};
    const uint8_t* b[2] = {q_e5m2, q_e5m2_t};
    for (int i = 0; i < 2; ++i)
        for (int j = 0; j < 2; ++j)
            if (overlap(a[i], n, b[j], n)) return fail(FP8LIN_ERR_ARG, "%s: outputs overlap", fn);
    return hip_status(launch_cast_transpose_dual(x, x_dtype, rows, cols, scale_e4m3, q_e4m3, q_e4m3_t, amax_slot_e4m3,
                                                 scale_e5m2, q_e5m2, q_e5m2_t, amax_slot_e5m2, as_stream(stream),
                                                 SatCounts{sat_counter(amax_slot_e4m3), sat_counter(amax_slot_e5m2)}),
                      fn);
}

int32_t fp8_cast_transpose_dual_update(const void* x, int32_t x_dtype, int64_t rows, int64_t cols, uint8_t* q_e4m3,
                                       uint8_t* q_e4m3_t, uint8_t* q_e5m2, uint8_t* q_e5m2_t, float* amax_history,
                                       float* scale, float* scale_inv, const fp8lin_recipe* recipe, uint32_t* ticket,
                                       void* stream) {
    const char* fn = "fp8_cast_transpose_dual_update";
    static const uint8_t fmts[2] = {FP8LIN_E4M3, FP8LIN_E5M2};
    int32_t v;
    if ((v = check_scale_args(fn, amax_history, scale, scale_inv, fmts, 2, recipe))) return v;
    const int64_t L = recipe->history_len;
    if ((v = check_ct(fn, x, nullptr, x_dtype, rows, cols, FP8LIN_E4M3, scale, q_e4m3, q_e4m3_t, amax_history,
                      nullptr, nullptr, nullptr, false)))
        return v;
    if ((v = check_ct(fn, x, nullptr, x_dtype, rows, cols, FP8LIN_E5M2, scale + 1, q_e5m2, q_e5m2_t,
                      amax_history + L, nullptr, nullptr, nullptr, false)))
        return v;
    const int64_t n = rows * cols;
    if (n > 0 && !q_e4m3 && !q_e4m3_t && !q_e5m2 && !q_e5m2_t) return fail(FP8LIN_ERR_NULL, "%s: no output", fn);
    if (n > 0 && !ticket) return fail(FP8LIN_ERR_NULL, "%s: ticket is null", fn);
    if (!aligned(ticket, 4)) return fail(FP8LIN_ERR_ALIGN, "%s: misaligned ticket", fn);
    const uint8_t* outs[4] = {q_e4m3, q_e4m3_t, q_e5m2, q_e5m2_t};
    for (int i = 0; i < 4; ++i)
        for (int j = i + 1; j < 4; ++j)
            if (overlap(outs[i], n, outs[j], n)) return fail(FP8LIN_ERR_ARG, "%s: outputs overlap", fn);
    const void* state[4] = {amax_history, scale, scale_inv, ticket};
    const int64_t sb[4] = {2 * L * 4, 8, 8, 4};
    const int64_t xb = n * elem_size(x_dtype);
    for (int i = 0; i < 4; ++i) {
        if (overlap(state[i], sb[i], x, xb)) return fail(FP8LIN_ERR_ARG, "%s: state overlaps the input", fn);
        for (int j = 0; j < 4; ++j)
            if (overlap(state[i], sb[i], outs[j], n)) return fail(FP8LIN_ERR_ARG, "%s: state overlaps an output", fn);
        if (i < 3 && overlap(state[i], sb[i], ticket, 4)) return fail(FP8LIN_ERR_ARG, "%s: ticket overlaps", fn);
    }
    return hip_status(launch_cast_transpose_dual_update(x, x_dtype, rows, cols, q_e4m3, q_e4m3_t, q_e5m2, q_e5m2_t,
                                                        amax_history, scale, scale_inv, (int32_t)L, recipe->margin,
                                                        ticket, as_stream(stream),
                                                        SatCounts{sat_counter(amax_history),
                                                                  sat_counter(amax_history + L)}),
                      fn);
}

// ---------------------------------------------------------------- dequant
int32_t fp8_dequant(const uint8_t* q, int32_t fp8_dtype, int64_t n, const float* scale_inv, void* out,
                    int32_t out_dtype, void* stream) {
    if (!is_fp8(fp8_dtype)) return fail(FP8LIN_ERR_DTYPE, "fp8_dequant: fp8_dtype %d must be E4M3 or E5M2", fp8_dtype);
    if (!is_hp(out_dtype)) return fail(FP8LIN_ERR_DTYPE, "fp8_dequant: out_dtype %d must be F32 or BF16", out_dtype);
    if (n < 0 || n > kMaxElems) return fail(FP8LIN_ERR_SHAPE, "fp8_dequant: n=%lld out of range", (long long)n);
    if (!scale_inv || (n > 0 && (!q || !out))) return fail(FP8LIN_ERR_NULL, "fp8_dequant: null pointer");
    if (!aligned(q, 16) || !aligned(out, 16) || !aligned(scale_inv, 4))
        return fail(FP8LIN_ERR_ALIGN, "fp8_dequant: misaligned pointer");
    if (overlap(q, n, out, n * elem_size(out_dtype))) return fail(FP8LIN_ERR_ARG, "fp8_dequant: output overlaps input");
    return hip_status(launch_dequant(q, fp8_dtype, n, scale_inv, out, out_dtype, as_stream(stream)), "fp8_dequant");
}

// ------------------------------------------------------------------- GEMM
namespace {
int32_t check_gemm(const char* fn, const uint8_t* a, int32_t a_dtype, const uint8_t* b, int32_t b_dtype, int64_t m,
                   int64_t n, int64_t k, const float* sinv_a, const float* sinv_b, const void* bias,
                   int32_t bias_dtype, int32_t epilogue, void* d, int32_t d_dtype, void* aux, const void* residual,
                   float* amax_d, const fp8lin_qout* q_out = nullptr) {
    if (!is_fp8(a_dtype) || !is_fp8(b_dtype))
        return fail(FP8LIN_ERR_DTYPE, "%s: operand types %d, %d must be E4M3/E5M2", fn, a_dtype, b_dtype);
    if (!is_hp(d_dtype)) return fail(FP8LIN_ERR_DTYPE, "%s: output type %d must be F32 or BF16", fn, d_dtype);
    if (bias && !is_hp(bias_dtype)) return fail(FP8LIN_ERR_DTYPE, "%s: bias type %d must be F32 or BF16", fn, bias_dtype);
    if (m < 0 || n < 0 || k < 0 || m % 16 || n % 16 || k % 16 || k >= kMaxK || m > (int64_t(1) << 31) ||
        n > (int64_t(1) << 31) || m * n > kMaxElems)
        return fail(FP8LIN_ERR_SHAPE, "%s: m=%lld n=%lld k=%lld must be >= 0 multiples of 16, k < 2^23", fn,
                    (long long)m, (long long)n, (long long)k);
    if (epilogue & ~(FP8LIN_EPI_GELU | FP8LIN_EPI_ACCUMULATE | FP8LIN_EPI_FAST_ACCUM))
        return fail(FP8LIN_ERR_ARG, "%s: unknown epilogue flags 0x%x", fn, epilogue);
    if ((epilogue & FP8LIN_EPI_GELU) && (epilogue & FP8LIN_EPI_ACCUMULATE))
        return fail(FP8LIN_ERR_ARG, "%s: GELU and ACCUMULATE cannot be combined", fn);
    if ((epilogue & FP8LIN_EPI_ACCUMULATE) && d_dtype != FP8LIN_F32)
        return fail(FP8LIN_ERR_DTYPE, "%s: ACCUMULATE needs an F32 output", fn);
    if (aux && !(epilogue & FP8LIN_EPI_GELU)) return fail(FP8LIN_ERR_ARG, "%s: aux is only written with GELU", fn);
    if (!sinv_a || !sinv_b) return fail(FP8LIN_ERR_NULL, "%s: null scale pointer", fn);
    if (q_out) {
        if (d_dtype != FP8LIN_BF16) return fail(FP8LIN_ERR_UNSUPPORTED, "%s: an FP8 copy of the output needs BF16", fn);
        if (a_dtype != FP8LIN_E4M3 || b_dtype != FP8LIN_E4M3)
            return fail(FP8LIN_ERR_UNSUPPORTED, "%s: an FP8 copy of the output needs E4M3 x E4M3 operands", fn);
        if (!is_fp8(q_out->fp8_dtype)) return fail(FP8LIN_ERR_DTYPE, "%s: q_out fp8_dtype %d", fn, q_out->fp8_dtype);
        if (!q_out->scale) return fail(FP8LIN_ERR_NULL, "%s: q_out has no scale", fn);
        if (m * n > 0 && !q_out->q && !q_out->q_t) return fail(FP8LIN_ERR_NULL, "%s: q_out has no output", fn);
        if (!aligned(q_out->scale, 4) || !aligned(q_out->q, 16) || !aligned(q_out->q_t, 16))
            return fail(FP8LIN_ERR_ALIGN, "%s: q_out misaligned", fn);
        const int64_t db = m * n * 2;
        const void* others[7] = {a, b, bias, d, aux, residual, q_out->q_t};
        const int64_t ob[7] = {m * k, n * k, bias ? n * elem_size(bias_dtype) : 0, d ? db : 0, aux ? db : 0,
                               residual ? db : 0, q_out->q_t ? m * n : 0};
        for (int i = 0; i < 7; ++i) {
            if (q_out->q && overlap(q_out->q, m * n, others[i], ob[i]))
                return fail(FP8LIN_ERR_ARG, "%s: q_out->q overlaps another buffer", fn);
            if (i < 6 && q_out->q_t && overlap(q_out->q_t, m * n, others[i], ob[i]))
                return fail(FP8LIN_ERR_ARG, "%s: q_out->q_t overlaps another buffer", fn);
        }
    }
    if (m * n > 0 && !d && !q_out) return fail(FP8LIN_ERR_NULL, "%s: null output", fn);
    if (m * n * k > 0 && (!a || !b)) return fail(FP8LIN_ERR_NULL, "%s: null operand", fn);
    if (!aligned(a, 16) || !aligned(b, 16) || !aligned(d, 16) || !aligned(aux, 16) || !aligned(bias, 16) ||
        !aligned(residual, 16) || !aligned(sinv_a, 4) || !aligned(sinv_b, 4) || !aligned(amax_d, 4))
        return fail(FP8LIN_ERR_ALIGN, "%s: misaligned pointer", fn);
    if (residual && (epilogue & FP8LIN_EPI_ACCUMULATE))
        return fail(FP8LIN_ERR_ARG, "%s: a residual cannot be combined with ACCUMULATE", fn);
    const int64_t db = m * n * elem_size(d_dtype);
    // the residual may be the output itself (each element is read before it is
    // written by the same lane) but must not partly overlap it or any other buffer
    if (residual && residual != d && overlap(residual, db, d, db))
        return fail(FP8LIN_ERR_ARG, "%s: residual partly overlaps d", fn);
    if (residual && overlap(residual, db, aux, aux ? db : 0))
        return fail(FP8LIN_ERR_ARG, "%s: residual overlaps aux", fn);
    const void* ins[3] = {a, b, bias};
    const int64_t ib[3] = {m * k, n * k, bias ? n * elem_size(bias_dtype) : 0};
    for (int i = 0; i < 3; ++i)
        if (overlap(d, db, ins[i], ib[i]) || overlap(aux, aux ? db : 0, ins[i], ib[i]))
            return fail(FP8LIN_ERR_ARG, "%s: an output overlaps an input", fn);
    if (overlap(d, db, aux, aux ? db : 0)) return fail(FP8LIN_ERR_ARG, "%s: d and aux overlap", fn);
    return FP8LIN_OK;
}
}  // namespace

int32_t fp8_gemm(const uint8_t* a, int32_t a_dtype, const uint8_t* b, int32_t b_dtype, int64_t m, int64_t n, int64_t k,
                 const float* sinv_a, const float* sinv_b, const void* bias, int32_t bias_dtype, int32_t epilogue,
                 void* d, int32_t d_dtype, void* aux, const void* residual, float* amax_d, const fp8lin_qout* q_out,
                 void* stream) {
    const int32_t v = check_gemm("fp8_gemm", a, a_dtype, b, b_dtype, m, n, k, sinv_a, sinv_b, bias, bias_dtype,
                                 epilogue, d, d_dtype, aux, residual, amax_d, q_out);
    if (v != FP8LIN_OK) return v;
    return hip_status(launch_gemm(a, a_dtype, b, b_dtype, m, n, k, sinv_a, sinv_b, bias, bias_dtype, epilogue, d,
                                  d_dtype, aux, residual, amax_d, q_out ? q_out->scale : nullptr,
                                  q_out ? q_out->q : nullptr, q_out ? q_out->q_t : nullptr,
                                  q_out ? q_out->fp8_dtype : 0, as_stream(stream)),
                      "fp8_gemm");
}

// ---------------------------------------------------------- linear layer
namespace {
int32_t check_recipe(const char* fn, const fp8lin_recipe* r) {
    if (!r) return fail(FP8LIN_ERR_NULL, "%s: null recipe", fn);
    if (r->format != FP8LIN_FORMAT_E4M3 && r->format != FP8LIN_FORMAT_HYBRID)
        return fail(FP8LIN_ERR_ARG, "%s: recipe format %d", fn, r->format);
    if (r->amax_compute_algo != FP8LIN_AMAX_MAX)
        return fail(FP8LIN_ERR_UNSUPPORTED, "%s: amax_compute_algo %d (only max)", fn, r->amax_compute_algo);
    if (r->margin < 0 || r->margin > 127) return fail(FP8LIN_ERR_ARG, "%s: margin=%d not in [0, 127]", fn, r->margin);
    return FP8LIN_OK;
}

// Just-in-time scaling of one tensor: amax(x) into the meta's slot 0 (or, for
// the GeLU backward, amax of dZ formed on the fly), then its scale from that
// amax.  The cast that follows needs no amax slot.
hipError_t jit_scale(const void* x, const void* gelu_z, int32_t dtype, int64_t rows, int64_t cols, int32_t fmt,
                     const fp8lin_meta* mt, int32_t margin, hipStream_t s) {
    hipError_t e = gelu_z ? launch_cast_transpose(x, gelu_z, dtype, rows, cols, fmt, mt->scale, nullptr, nullptr,
                                                  mt->amax_history, nullptr, nullptr, nullptr, s)
                          : launch_amax(x, dtype, rows * cols, mt->amax_history, s);
    if (e != hipSuccess) return e;
    const uint8_t f = (uint8_t)fmt;
    return launch_scale_from_current(mt->amax_history, 1, mt->scale, mt->scale_inv, &f, 1, margin, s);
}

int32_t check_meta(const char* fn, const char* which, const fp8lin_meta* mt) {
    if (!mt || !mt->amax_history || !mt->scale || !mt->scale_inv)
        return fail(FP8LIN_ERR_NULL, "%s: meta %s has a null pointer", fn, which);
    if (!aligned(mt->amax_history, 4) || !aligned(mt->scale, 4) || !aligned(mt->scale_inv, 4))
        return fail(FP8LIN_ERR_ALIGN, "%s: meta %s misaligned", fn, which);
    return FP8LIN_OK;
}
}  // namespace

int32_t fp8_linear_fwd(int64_t m, int64_t n, int64_t k, const void* x, int32_t x_dtype, const void* w,
                       int32_t w_dtype, const void* bias, int32_t bias_dtype, int32_t epilogue, void* y,
                       int32_t y_dtype, void* y_aux, const void* residual, float* y_amax_slot, const fp8lin_qout* y_q,
                       const fp8lin_recipe* recipe, const fp8lin_meta* mx, const fp8lin_meta* mw,
                       const fp8lin_saved* saved, void* stream) {
    const char* fn = "fp8_linear_fwd";
    int32_t v;
    if ((v = check_recipe(fn, recipe)) || (v = check_meta(fn, "x", mx)) || (v = check_meta(fn, "w", mw))) return v;
    if (!saved || !saved->xq || !saved->wq || !saved->sinv) return fail(FP8LIN_ERR_NULL, "%s: saved needs xq, wq, sinv", fn);
    if (!is_hp(x_dtype) || !is_hp(w_dtype)) return fail(FP8LIN_ERR_DTYPE, "%s: x/w types must be F32 or BF16", fn);
    if (epilogue & ~FP8LIN_EPI_GELU) return fail(FP8LIN_ERR_ARG, "%s: the forward epilogue is 0 or GELU", fn);
    const int32_t fast = recipe->fast_accum ? FP8LIN_EPI_FAST_ACCUM : 0;
    if (m < 0 || n < 0 || k < 0 || m % 16 || n % 16 || k % 16)
        return fail(FP8LIN_ERR_SHAPE, "%s: m=%lld n=%lld k=%lld must be >= 0 multiples of 16", fn, (long long)m,
                    (long long)n, (long long)k);
    const bool x_quantised = x == nullptr;      // X's codes are already in saved (cast by the producer)
    const bool w_quantised = w == nullptr;      // W's codes are already in saved (cast by fp8_sgd_step_cast)
    if ((x_quantised || w_quantised) && recipe->just_in_time)
        return fail(FP8LIN_ERR_ARG, "%s: a pre-quantised X or W cannot be scaled just in time", fn);
    if (!aligned(saved->sinv, 4)) return fail(FP8LIN_ERR_ALIGN, "%s: saved->sinv misaligned", fn);
    // Validate every sub-call before launching any of them.
    if (!x_quantised && (v = check_ct(fn, x, nullptr, x_dtype, m, k, FP8LIN_E4M3, mx->scale, saved->xq, saved->xq_t,
                                      mx->amax_history, nullptr, nullptr, nullptr, false)))
        return v;
    if (x_quantised && (!aligned(saved->xq, 16) || !aligned(saved->xq_t, 16)))
        return fail(FP8LIN_ERR_ALIGN, "%s: saved codes misaligned", fn);
    if (!w_quantised && (v = check_ct(fn, w, nullptr, w_dtype, n, k, FP8LIN_E4M3, mw->scale, saved->wq, saved->wq_t,
                                      mw->amax_history, nullptr, nullptr, nullptr, false)))
        return v;
    if (w_quantised && (!aligned(saved->wq, 16) || !aligned(saved->wq_t, 16)))
        return fail(FP8LIN_ERR_ALIGN, "%s: saved codes misaligned", fn);
    if ((v = check_gemm(fn, saved->xq, FP8LIN_E4M3, saved->wq, FP8LIN_E4M3, m, n, k, saved->sinv, saved->sinv + 1,
                        bias, bias_dtype, epilogue | fast, y, y_dtype, y_aux, residual, y_amax_slot, y_q)))
        return v;
    if (overlap(y, m * n * elem_size(y_dtype), x, m * k * elem_size(x_dtype)) ||
        overlap(y, m * n * elem_size(y_dtype), w, n * k * elem_size(w_dtype)))
        return fail(FP8LIN_ERR_ARG, "%s: y overlaps an input", fn);
    if (y_q) {
        const void* mine[4] = {saved->xq, saved->xq_t, saved->wq, saved->wq_t};
        const int64_t mb[4] = {m * k, saved->xq_t ? m * k : 0, n * k, saved->wq_t ? n * k : 0};
        for (int i = 0; i < 4; ++i)
            if (overlap(y_q->q, y_q->q ? m * n : 0, mine[i], mb[i]) ||
                overlap(y_q->q_t, y_q->q_t ? m * n : 0, mine[i], mb[i]))
                return fail(FP8LIN_ERR_ARG, "%s: y_q overlaps this layer's saved codes", fn);
    }

    hipStream_t s = as_stream(stream);
    hipError_t e;
    const bool jit = recipe->just_in_time != 0;
    // the W cast also snapshots the two inverse scales into saved->sinv (an
    // empty W launches no cast, so a one-thread copy does it)
    const SinvSnap snap{mx->scale_inv, mw->scale_inv, saved->sinv};
    if (!x_quantised && !w_quantised && saved->xq_t && saved->wq_t && x_dtype == w_dtype && m * k > 0 && n * k > 0) {
        // X and W in one launch (same kernel variant, independent tensors)
        if (jit && (e = jit_scale(x, nullptr, x_dtype, m, k, FP8LIN_E4M3, mx, recipe->margin, s)) != hipSuccess)
            return hip_status(e, "fp8_linear_fwd: just-in-time scale of X");
        if (jit && (e = jit_scale(w, nullptr, w_dtype, n, k, FP8LIN_E4M3, mw, recipe->margin, s)) != hipSuccess)
            return hip_status(e, "fp8_linear_fwd: just-in-time scale of W");
        e = launch_cast_transpose_pair(x, w, x_dtype, m, k, n, k, FP8LIN_E4M3, mx->scale, saved->xq, saved->xq_t,
                                       jit ? nullptr : mx->amax_history, mw->scale, saved->wq, saved->wq_t,
                                       jit ? nullptr : mw->amax_history, s, snap,
                                       SatCounts{sat_counter(mx->amax_history), sat_counter(mw->amax_history)});
        if (e != hipSuccess) return hip_status(e, "fp8_linear_fwd: cast X and W");
        return hip_status(launch_gemm(saved->xq, FP8LIN_E4M3, saved->wq, FP8LIN_E4M3, m, n, k, saved->sinv,
                                      saved->sinv + 1, bias, bias_dtype, epilogue | fast, y, y_dtype, y_aux, residual,
                                      y_amax_slot, y_q ? y_q->scale : nullptr, y_q ? y_q->q : nullptr,
                                      y_q ? y_q->q_t : nullptr, y_q ? y_q->fp8_dtype : 0, s),
                          "fp8_linear_fwd: gemm");
    }
    // the snapshot of the inverse scales rides on the last cast of the call
    // (none of an empty tensor), else a one-thread copy takes it
    const bool w_cast = !w_quantised && n * k > 0;
    if (!x_quantised) {
        if (jit && (e = jit_scale(x, nullptr, x_dtype, m, k, FP8LIN_E4M3, mx, recipe->margin, s)) != hipSuccess)
            return hip_status(e, "fp8_linear_fwd: just-in-time scale of X");
        float* xslot = jit ? nullptr : mx->amax_history;
        const SatCounts xsat{sat_counter(mx->amax_history)};
        const SinvSnap xsnap = !w_cast && m * k > 0 ? snap : SinvSnap{};
        if (saved->xq_t) e = launch_cast_transpose(x, nullptr, x_dtype, m, k, FP8LIN_E4M3, mx->scale, saved->xq,
                                                   saved->xq_t, xslot, nullptr, nullptr, nullptr, s, xsnap, xsat);
        else e = launch_cast(x, x_dtype, m * k, FP8LIN_E4M3, mx->scale, saved->xq, xslot, s, xsnap, xsat);
        if (e != hipSuccess) return hip_status(e, "fp8_linear_fwd: cast X");
    }
    if (!w_quantised) {
        if (jit && (e = jit_scale(w, nullptr, w_dtype, n, k, FP8LIN_E4M3, mw, recipe->margin, s)) != hipSuccess)
            return hip_status(e, "fp8_linear_fwd: just-in-time scale of W");
        float* wslot = jit ? nullptr : mw->amax_history;
        const SatCounts wsat{sat_counter(mw->amax_history)};
        if (saved->wq_t) e = launch_cast_transpose(w, nullptr, w_dtype, n, k, FP8LIN_E4M3, mw->scale, saved->wq,
                                                   saved->wq_t, wslot, nullptr, nullptr, nullptr, s, snap, wsat);
        else e = launch_cast(w, w_dtype, n * k, FP8LIN_E4M3, mw->scale, saved->wq, wslot, s, snap, wsat);
        if (e != hipSuccess) return hip_status(e, "fp8_linear_fwd: cast W");
    }
    if (!w_cast && (x_quantised || m * k == 0)) {
        e = launch_copy_scalars(mx->scale_inv, mw->scale_inv, saved->sinv, s);
        if (e != hipSuccess) return hip_status(e, "fp8_linear_fwd: save scale_inv");
    }
    e = launch_gemm(saved->xq, FP8LIN_E4M3, saved->wq, FP8LIN_E4M3, m, n, k, saved->sinv, saved->sinv + 1, bias,
                    bias_dtype, epilogue | fast, y, y_dtype, y_aux, residual, y_amax_slot, y_q ? y_q->scale : nullptr,
                    y_q ? y_q->q : nullptr, y_q ? y_q->q_t : nullptr, y_q ? y_q->fp8_dtype : 0, s);
    return hip_status(e, "fp8_linear_fwd: gemm");
}

int32_t fp8_linear_bwd(int64_t m, int64_t n, int64_t k, const void* dy, int32_t dy_dtype, const void* gelu_z,
                       void* dz_out, const fp8lin_recipe* recipe, const fp8lin_meta* mdy, const fp8lin_saved* saved,
                       uint8_t* dyq_ws, uint8_t* dyq_t_ws, void* dx, int32_t dx_dtype, const void* dx_residual,
                       float* dw, int32_t accumulate_dw, float* dbias, float* dbias_ws, void* stream) {
    const char* fn = "fp8_linear_bwd";
    int32_t v;
    if ((v = check_recipe(fn, recipe)) || (v = check_meta(fn, "dy", mdy))) return v;
    if (!saved || !saved->sinv) return fail(FP8LIN_ERR_NULL, "%s: saved needs sinv", fn);
    if (!is_hp(dy_dtype)) return fail(FP8LIN_ERR_DTYPE, "%s: dy type must be F32 or BF16", fn);
    if (dz_out && !gelu_z) return fail(FP8LIN_ERR_ARG, "%s: dz_out needs gelu_z", fn);
    if (m < 0 || n < 0 || k < 0 || m % 16 || n % 16 || k % 16)
        return fail(FP8LIN_ERR_SHAPE, "%s: m=%lld n=%lld k=%lld must be >= 0 multiples of 16", fn, (long long)m,
                    (long long)n, (long long)k);
    if (m * n > 0 && !dy) return fail(FP8LIN_ERR_NULL, "%s: null dy", fn);
    if (dx && (!dyq_ws || !saved->wq_t)) return fail(FP8LIN_ERR_NULL, "%s: dx needs dyq_ws and saved->wq_t", fn);
    if (dw && (!dyq_t_ws || !saved->xq_t)) return fail(FP8LIN_ERR_NULL, "%s: dw needs dyq_t_ws and saved->xq_t", fn);
    if (!dx && !dw && !dbias) return ok();
    const int32_t gfmt = recipe->format == FP8LIN_FORMAT_HYBRID ? FP8LIN_E5M2 : FP8LIN_E4M3;
    const int32_t fast = recipe->fast_accum ? FP8LIN_EPI_FAST_ACCUM : 0;
    // Row-major codes feed dgrad, transposed codes feed wgrad; each is written
    // only when its GEMM is wanted.
    uint8_t* qr = dx ? dyq_ws : nullptr;
    uint8_t* qt = dw ? dyq_t_ws : nullptr;
    if ((v = check_ct(fn, dy, gelu_z, dy_dtype, m, n, gfmt, mdy->scale, qr, qt, mdy->amax_history, dbias, dbias_ws,
                      dz_out, false)))
        return v;
    if (dx_residual && !dx) return fail(FP8LIN_ERR_ARG, "%s: dx_residual needs dx", fn);
    if (dx && (v = check_gemm(fn, dyq_ws, gfmt, saved->wq_t, FP8LIN_E4M3, m, k, n, mdy->scale_inv, saved->sinv + 1,
                              nullptr, FP8LIN_F32, fast, dx, dx_dtype, nullptr, dx_residual, nullptr)))
        return v;
    if (dw && (v = check_gemm(fn, dyq_t_ws, gfmt, saved->xq_t, FP8LIN_E4M3, n, k, m, mdy->scale_inv, saved->sinv,
                              nullptr, FP8LIN_F32, (accumulate_dw ? FP8LIN_EPI_ACCUMULATE : 0) | fast, dw, FP8LIN_F32,
                              nullptr, nullptr, nullptr)))
        return v;
    if (dx && dw && overlap(dx, m * k * elem_size(dx_dtype), dw, n * k * 4))
        return fail(FP8LIN_ERR_ARG, "%s: dx and dw overlap", fn);
    if (dx && (overlap(dx, m * k * elem_size(dx_dtype), dy, m * n * elem_size(dy_dtype)) ||
               overlap(dx, m * k * elem_size(dx_dtype), gelu_z, gelu_z ? m * n * elem_size(dy_dtype) : 0)))
        return fail(FP8LIN_ERR_ARG, "%s: dx overlaps dy or gelu_z", fn);

    hipStream_t s = as_stream(stream);
    hipError_t e;
    const bool jit = recipe->just_in_time != 0;
    if (jit && (e = jit_scale(dy, gelu_z, dy_dtype, m, n, gfmt, mdy, recipe->margin, s)) != hipSuccess)
        return hip_status(e, "fp8_linear_bwd: just-in-time scale of dY");
    e = launch_cast_transpose(dy, gelu_z, dy_dtype, m, n, gfmt, mdy->scale, qr, qt, jit ? nullptr : mdy->amax_history,
                              dbias, dbias_ws, dz_out, s, SinvSnap{}, SatCounts{sat_counter(mdy->amax_history)});
    if (e != hipSuccess) return hip_status(e, "fp8_linear_bwd: cast dY");
    if (dx) {
        e = launch_gemm(dyq_ws, gfmt, saved->wq_t, FP8LIN_E4M3, m, k, n, mdy->scale_inv, saved->sinv + 1, nullptr,
                        FP8LIN_F32, fast, dx, dx_dtype, nullptr, dx_residual, nullptr, nullptr, nullptr, nullptr, 0, s);
        if (e != hipSuccess) return hip_status(e, "fp8_linear_bwd: dgrad");
    }
    if (dw) {
        e = launch_gemm(dyq_t_ws, gfmt, saved->xq_t, FP8LIN_E4M3, n, k, m, mdy->scale_inv, saved->sinv, nullptr,
                        FP8LIN_F32, (accumulate_dw ? FP8LIN_EPI_ACCUMULATE : 0) | fast, dw, FP8LIN_F32, nullptr,
                        nullptr, nullptr, nullptr, nullptr, nullptr, 0, s);
        if (e != hipSuccess) return hip_status(e, "fp8_linear_bwd: wgrad");
    }
    return ok();
}

// --------------------------------------------------- loss scaling and SGD
int32_t fp8_loss_scale_update(const float* grad_amaxes, int32_t n, int64_t stride, float* state,
                              int32_t growth_interval, float backoff, float growth, void* stream) {
    const char* fn = "fp8_loss_scale_update";
    if (!grad_amaxes || !state) return fail(FP8LIN_ERR_NULL, "%s: null pointer", fn);
    if (n < 1 || n > 4096 || stride < 1) return fail(FP8LIN_ERR_SHAPE, "%s: n=%d stride=%lld", fn, n, (long long)stride);
    if (growth_interval < 1 || !(backoff > 0.0f && backoff < 1.0f) || !(growth > 1.0f))
        return fail(FP8LIN_ERR_ARG, "%s: need growth_interval >= 1, 0 < backoff < 1 < growth", fn);
    if (!aligned(grad_amaxes, 4) || !aligned(state, 4)) return fail(FP8LIN_ERR_ALIGN, "%s: misaligned pointer", fn);
    if (overlap(state, 16, grad_amaxes, ((int64_t)(n - 1) * stride + 1) * 4))
        return fail(FP8LIN_ERR_ARG, "%s: state overlaps the amaxes", fn);
    return hip_status(launch_loss_scale_update(grad_amaxes, n, stride, state, growth_interval, backoff, growth,
                                               as_stream(stream)), fn);
}

int32_t fp8_loss_scale_apply(const void* g, int32_t dtype, int64_t n, const float* state, void* out, void* stream) {
    const char* fn = "fp8_loss_scale_apply";
    if (!is_hp(dtype)) return fail(FP8LIN_ERR_DTYPE, "%s: dtype %d must be F32 or BF16", fn, dtype);
    if (n < 0 || n > kMaxElems) return fail(FP8LIN_ERR_SHAPE, "%s: n=%lld", fn, (long long)n);
    if (!state || (n > 0 && (!g || !out))) return fail(FP8LIN_ERR_NULL, "%s: null pointer", fn);
    if (!aligned(g, 16) || !aligned(out, 16) || !aligned(state, 4)) return fail(FP8LIN_ERR_ALIGN, "%s: misaligned", fn);
    if (g != out && overlap(g, n * elem_size(dtype), out, n * elem_size(dtype)))
        return fail(FP8LIN_ERR_ARG, "%s: out partly overlaps g", fn);
    return hip_status(launch_scale_by(g, dtype, n, state, out, as_stream(stream)), fn);
}

int32_t fp8_sgd_step(float* w, const float* g, int64_t n, float lr, const float* state, void* stream) {
    const char* fn = "fp8_sgd_step";
    if (n < 0 || n > kMaxElems) return fail(FP8LIN_ERR_SHAPE, "%s: n=%lld", fn, (long long)n);
    if (!state || (n > 0 && (!w || !g))) return fail(FP8LIN_ERR_NULL, "%s: null pointer", fn);
    if (!aligned(w, 16) || !aligned(g, 16) || !aligned(state, 4)) return fail(FP8LIN_ERR_ALIGN, "%s: misaligned", fn);
    if (overlap(w, n * 4, g, n * 4) || overlap(w, n * 4, state, 16))
        return fail(FP8LIN_ERR_ARG, "%s: w overlaps g or the state", fn);
    return hip_status(launch_sgd(w, g, n, lr, state, as_stream(stream)), fn);
}

int32_t fp8_sgd_step_cast(float* w, const float* g, int64_t rows, int64_t cols, float lr, const float* state,
                          const float* scale, uint8_t* q, uint8_t* q_t, float* amax_slot, void* stream) {
    const char* fn = "fp8_sgd_step_cast";
    int32_t v = check_ct(fn, w, nullptr, FP8LIN_F32, rows, cols, FP8LIN_E4M3, scale, q, q_t, amax_slot, nullptr,
                         nullptr, nullptr);
    if (v != FP8LIN_OK) return v;
    const int64_t n = rows * cols;
    if (!state || (n > 0 && !g)) return fail(FP8LIN_ERR_NULL, "%s: null pointer", fn);
    if (!aligned(g, 16) || !aligned(state, 4)) return fail(FP8LIN_ERR_ALIGN, "%s: misaligned", fn);
    // w is written: nothing else may share its bytes; g, state and scale are read
    if (overlap(w, n * 4, g, n * 4) || overlap(w, n * 4, state, 16) || overlap(w, n * 4, scale, 4) ||
        overlap(w, n * 4, amax_slot, 4))
        return fail(FP8LIN_ERR_ARG, "%s: w overlaps g, the state, the scale or the amax slot", fn);
    const void* outs[3] = {q, q_t, amax_slot};
    const int64_t ob[3] = {n, n, 4};
    for (int i = 0; i < 3; ++i)
        if (overlap(outs[i], ob[i], g, n * 4) || overlap(outs[i], ob[i], state, 16))
            return fail(FP8LIN_ERR_ARG, "%s: an output overlaps g or the state", fn);
    return hip_status(launch_sgd_cast_transpose(w, g, rows, cols, lr, state, scale, q, q_t, amax_slot,
                                                as_stream(stream), SatCounts{sat_counter(amax_slot)}),
                      fn);
}


// ------------------------------------------------------------ attention core
namespace {
// Validates the shape; on success sets the element counts of one head-split
// tensor (batch*seq*heads*128) and returns FP8LIN_OK.
int32_t check_attn_shape(const char* fn, int64_t batch, int64_t seq, int64_t heads, int64_t head_dim, int64_t* n) {
    if (head_dim != 128) return fail(FP8LIN_ERR_UNSUPPORTED, "%s: head_dim=%lld (only 128)", fn, (long long)head_dim);
    if (batch < 1 || heads < 1 || seq < 256 || seq % 256 != 0)
        return fail(FP8LIN_ERR_SHAPE, "%s: batch=%lld heads=%lld seq=%lld (seq a multiple of 256)", fn,
                    (long long)batch, (long long)heads, (long long)seq);
    if (batch > (1 << 20) || heads > (1 << 20) || seq > (1 << 24) || batch * seq * heads * 128 >= (int64_t(1) << 31))
        return fail(FP8LIN_ERR_SHAPE, "%s: batch*seq*heads*head_dim must be < 2^31", fn);
    // The kernels stage tiles with buffer loads whose byte offsets, from the
    // start of one (batch, head), stay below 2^31: a sequence of the qkv rows
    // (3 * heads * 128 bf16 each) and 128 rows of a transposed operand (row
    // length batch * seq bf16).
    if (seq * heads * 768 >= (int64_t(1) << 31) || batch * seq * 256 >= (int64_t(1) << 31))
        return fail(FP8LIN_ERR_SHAPE, "%s: seq*heads must be < 2796203 and batch*seq < 2^23", fn);
    *n = batch * seq * heads * 128;
    return FP8LIN_OK;
}
}  // namespace

int64_t bf16_attention_workspace_bytes(int64_t batch, int64_t seq, int64_t heads, int64_t head_dim, int32_t backward) {
    int64_t n = 0;
    if (check_attn_shape("bf16_attention_workspace_bytes", batch, seq, heads, head_dim, &n) != FP8LIN_OK) return -1;
    return backward ? 2 * n * 2 + batch * heads * seq * 4 : n * 2;
}

int32_t bf16_attention_fwd(const void* qkv, int64_t batch, int64_t seq, int64_t heads, int64_t head_dim, void* ctx,
                           float* lse, void* workspace, void* stream) {
    const char* fn = "bf16_attention_fwd";
    int64_t n = 0;
    const int32_t st = check_attn_shape(fn, batch, seq, heads, head_dim, &n);
    if (st != FP8LIN_OK) return st;
    if (!qkv || !ctx || !lse || !workspace) return fail(FP8LIN_ERR_NULL, "%s: null pointer", fn);
    if (!aligned(qkv, 16) || !aligned(ctx, 16) || !aligned(lse, 16) || !aligned(workspace, 16))
        return fail(FP8LIN_ERR_ALIGN, "%s: misaligned pointer", fn);
    const int64_t lb = batch * heads * seq * 4;
    const void* bufs[4] = {qkv, ctx, lse, workspace};
    const int64_t bytes[4] = {3 * n * 2, n * 2, lb, n * 2};
    for (int i = 0; i < 4; ++i)
        for (int j = i + 1; j < 4; ++j)
            if (overlap(bufs[i], bytes[i], bufs[j], bytes[j])) return fail(FP8LIN_ERR_ARG, "%s: buffers overlap", fn);
    const uint16_t* q = static_cast<const uint16_t*>(qkv);
    return hip_status(launch_attention_fwd(q, batch, seq, heads, static_cast<uint16_t*>(ctx), lse,
                                           static_cast<uint16_t*>(workspace), as_stream(stream)), fn);
}

int32_t bf16_attention_bwd(const void* qkv, const void* ctx, const float* lse, const void* dctx, int64_t batch,
                           int64_t seq, int64_t heads, int64_t head_dim, void* dqkv, void* workspace, void* stream) {
    const char* fn = "bf16_attention_bwd";
    int64_t n = 0;
    const int32_t st = check_attn_shape(fn, batch, seq, heads, head_dim, &n);
    if (st != FP8LIN_OK) return st;
    if (!qkv || !ctx || !lse || !dctx || !dqkv || !workspace) return fail(FP8LIN_ERR_NULL, "%s: null pointer", fn);
    if (!aligned(qkv, 16) || !aligned(ctx, 16) || !aligned(lse, 16) || !aligned(dctx, 16) || !aligned(dqkv, 16) ||
        !aligned(workspace, 16))
        return fail(FP8LIN_ERR_ALIGN, "%s: misaligned pointer", fn);
    const int64_t lb = batch * heads * seq * 4;
    const int64_t wsb = 2 * n * 2 + lb;           // Q^T and dO^T (bf16), then rowsum(dO * O) (fp32)
    const void* ins[4] = {qkv, ctx, lse, dctx};
    const int64_t inb[4] = {3 * n * 2, n * 2, lb, n * 2};
    for (int i = 0; i < 4; ++i)
        if (overlap(dqkv, 3 * n * 2, ins[i], inb[i]) || overlap(workspace, wsb, ins[i], inb[i]))
            return fail(FP8LIN_ERR_ARG, "%s: an output or the workspace overlaps an input", fn);
    if (overlap(dqkv, 3 * n * 2, workspace, wsb)) return fail(FP8LIN_ERR_ARG, "%s: dqkv overlaps the workspace", fn);
    return hip_status(launch_attention_bwd(static_cast<const uint16_t*>(qkv), static_cast<const uint16_t*>(ctx), lse,
                                           static_cast<const uint16_t*>(dctx), batch, seq, heads,
                                           static_cast<uint16_t*>(dqkv), static_cast<uint16_t*>(workspace),
                                           static_cast<uint16_t*>(workspace) + n,
                                           reinterpret_cast<float*>(static_cast<uint16_t*>(workspace) + 2 * n),
                                           as_stream(stream)),
                      fn);
}

}  // extern "C"
