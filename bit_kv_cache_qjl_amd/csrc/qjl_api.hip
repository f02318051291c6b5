// C ABI of libqjl: argument validation, workspace layout, dispatch onto the caller's stream, the
// optional launch timer.  Declarations and the contract of every entry point are in include/qjl.h.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>
#include <string>
#include <vector>

#include "../../include/qjl.h"
#include "qjl_common.h"

namespace qjl {
bool decode_shape_supported(int m, int m_out);
}

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return QJL_OK;
    return fail(QJL_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// shape rules shared by all entry points
int check_sketch_shape(int d, int m, int m_out, int n_out) {
    if (m <= 0 || m_out < 0 || n_out < 0) return fail(QJL_ERR_INVALID_ARG, "m=%d m_out=%d n_out=%d must be >= 0 (m > 0)", m, m_out, n_out);
    if (d != qjl::kD) return fail(QJL_ERR_UNSUPPORTED, "d=%d unsupported (only d=128)", d);
    if (m % 128 || m_out % 128) return fail(QJL_ERR_UNSUPPORTED, "m=%d and m_out=%d must be multiples of 128", m, m_out);
    if (m + m_out > qjl::kMaxBits) return fail(QJL_ERR_UNSUPPORTED, "m + m_out = %d exceeds %d", m + m_out, qjl::kMaxBits);
    if (n_out > qjl::kMaxOutliers) return fail(QJL_ERR_UNSUPPORTED, "n_out=%d exceeds %d", n_out, qjl::kMaxOutliers);
    if (n_out > 0 && m_out == 0) return fail(QJL_ERR_INVALID_ARG, "n_out=%d outlier channels need an outlier sketch (m_out > 0)", n_out);
    return QJL_OK;
}

// ------------------------------------------------------------------ launch timer
struct TimerRec {
    hipEvent_t start, stop;
};
std::mutex g_timer_mu;
bool g_timer_on = false;
std::vector<TimerRec> g_timer_open[qjl::TK_COUNT];
std::vector<TimerRec> g_timer_done[qjl::TK_COUNT];
std::vector<hipEvent_t> g_event_pool;

hipEvent_t pool_event() {
    if (!g_event_pool.empty()) {
        hipEvent_t e = g_event_pool.back();
        g_event_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

const char* kKernelNames[qjl::TK_COUNT] = {"quantize_keys", "quantize_values", "query_project", "decode", "combine",
                                           "append_project", "select_outliers"};

}  // namespace

namespace qjl {

void timer_begin(TimedKernel k, hipStream_t s) {
    std::lock_guard<std::mutex> lk(g_timer_mu);
    if (!g_timer_on) return;
    TimerRec r{pool_event(), pool_event()};
    if (!r.start || !r.stop) return;
    hipEventRecord(r.start, s);
    g_timer_open[k].push_back(r);
}

void timer_end(TimedKernel k, hipStream_t s) {
    std::lock_guard<std::mutex> lk(g_timer_mu);
    if (!g_timer_on || g_timer_open[k].empty()) return;
    TimerRec r = g_timer_open[k].back();
    g_timer_open[k].pop_back();
    hipEventRecord(r.stop, s);
    g_timer_done[k].push_back(r);
}

}  // namespace qjl

extern "C" {

const char* qjl_status_string(int status) {
    switch (status) {
        case QJL_OK: return "ok";
        case QJL_ERR_INVALID_ARG: return "invalid argument";
        case QJL_ERR_UNSUPPORTED: return "unsupported shape";
        case QJL_ERR_MISALIGNED: return "misaligned pointer or stride";
        case QJL_ERR_WORKSPACE: return "workspace missing or too small";
        case QJL_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char* qjl_last_error(void) { return g_last_error.c_str(); }

int qjl_timer_enable(int on) {
    std::lock_guard<std::mutex> lk(g_timer_mu);
    g_timer_on = on != 0;
    return QJL_OK;
}

int qjl_timer_read(const char* kernel, int64_t* launches, double* total_ms) {
    if (!kernel || !launches || !total_ms) return fail(QJL_ERR_INVALID_ARG, "qjl_timer_read: null argument");
    int k = -1;
    for (int i = 0; i < qjl::TK_COUNT; ++i)
        if (std::string(kernel) == kKernelNames[i]) k = i;
    if (k < 0) return fail(QJL_ERR_INVALID_ARG, "qjl_timer_read: unknown kernel '%s'", kernel);
    std::lock_guard<std::mutex> lk(g_timer_mu);
    double tot = 0.0;
    int64_t n = 0;
    for (const TimerRec& r : g_timer_done[k]) {
        hipError_t e = hipEventSynchronize(r.stop);
        if (e != hipSuccess) return hip_status(e, "qjl_timer_read");
        float ms = 0.f;
        e = hipEventElapsedTime(&ms, r.start, r.stop);
        if (e != hipSuccess) return hip_status(e, "qjl_timer_read");
        tot += ms;
        ++n;
        g_event_pool.push_back(r.start);
        g_event_pool.push_back(r.stop);
    }
    g_timer_done[k].clear();
    *launches = n;
    *total_ms = tot;
    return QJL_OK;
}

int qjl_quantize_keys(const void* K, int kdt, int B, int64_t T, int Hkv, int d, int64_t sK_b, int64_t sK_t,
                      int64_t sK_h, const void* S_in, int m, const void* S_out, int m_out,
                      const int32_t* outlier_idx, int n_out, uint32_t* bits, uint16_t* norms, int64_t Ncap,
                      int64_t t0, hipStream_t stream) {
    g_last_error.clear();
    if (kdt != QJL_BF16 && kdt != QJL_F32) return fail(QJL_ERR_INVALID_ARG, "kdt=%d is not a qjl_dtype", kdt);
    if (B < 0 || T < 0 || Hkv <= 0 || Ncap < 0 || t0 < 0)
        return fail(QJL_ERR_INVALID_ARG, "bad sizes B=%d T=%lld Hkv=%d Ncap=%lld t0=%lld", B, (long long)T, Hkv,
                    (long long)Ncap, (long long)t0);
    int st = check_sketch_shape(d, m, m_out, n_out);
    if (st) return st;
    if (t0 + T > Ncap) return fail(QJL_ERR_INVALID_ARG, "t0 + T = %lld exceeds Ncap = %lld", (long long)(t0 + T), (long long)Ncap);
    if (B == 0 || T == 0) return QJL_OK;
    if (!K || !S_in || !bits || !norms || (m_out && !S_out) || (n_out && !outlier_idx))
        return fail(QJL_ERR_INVALID_ARG, "null device pointer");
    if (sK_b < 0 || sK_t < 0 || sK_h < 0) return fail(QJL_ERR_INVALID_ARG, "negative stride");
    const int64_t vec = kdt == QJL_BF16 ? 8 : 4;
    if (!aligned16(K) || !aligned16(S_in) || (m_out && !aligned16(S_out)) || !aligned16(bits) || !aligned16(norms) ||
        sK_b % vec || sK_t % vec || sK_h % vec)
        return fail(QJL_ERR_MISALIGNED, "pointers must be 16-byte aligned and strides multiples of %lld elements", (long long)vec);
    qjl::KeyQuantArgs a{};
    a.K = K;
    a.sKb = sK_b;
    a.sKt = sK_t;
    a.sKh = sK_h;
    a.S_in = S_in;
    a.S_out = S_out;
    a.oidx = outlier_idx;
    a.bits = bits;
    a.norms = norms;
    a.T = T;
    a.Ncap = Ncap;
    a.t0 = t0;
    a.Hkv = Hkv;
    a.m = m;
    a.m_out = m_out;
    a.n_out = n_out;
    a.W = (m + m_out) / 32;
    // one round of workgroups over 256 CUs (one per CU for the kernel that keeps the JL matrices in
    // LDS, two for the other), in whole 64-token chunks
    const int64_t slots =
        kdt == QJL_BF16 && qjl::quantize_keys_lds_shape(m, m_out) && T * sK_t * 2 + 256 < ((int64_t)1 << 31) ? 256 : 512;
    int64_t per = ((int64_t)B * Hkv * T + slots - 1) / slots;
    per = ((per + 63) / 64) * 64;
    if (per < 64) per = 64;
    if (per > 8192) per = 8192;
    if (per > ((T + 63) / 64) * 64) per = ((T + 63) / 64) * 64;
    a.tokens_per_block = (int)per;
    qjl::timer_begin(qjl::TK_QUANT_KEYS, stream);
    hipError_t e = kdt == QJL_BF16 ? qjl::launch_quantize_keys_bf16(a, B, stream) : qjl::launch_quantize_keys_f32(a, B, stream);
    qjl::timer_end(qjl::TK_QUANT_KEYS, stream);
    return hip_status(e, "qjl_quantize_keys launch");
}

int qjl_quantize_values(const void* V, int vdt, int B, int64_t T, int Hkv, int d, int64_t sV_b, int64_t sV_t,
                        int64_t sV_h, int nbits, uint32_t* codes, uint16_t* meta, int64_t Ncap, int64_t t0,
                        hipStream_t stream) {
    g_last_error.clear();
    if (vdt != QJL_BF16 && vdt != QJL_F32) return fail(QJL_ERR_INVALID_ARG, "vdt=%d is not a qjl_dtype", vdt);
    if (B < 0 || T < 0 || Hkv <= 0 || Ncap < 0 || t0 < 0)
        return fail(QJL_ERR_INVALID_ARG, "bad sizes B=%d T=%lld Hkv=%d Ncap=%lld t0=%lld", B, (long long)T, Hkv,
                    (long long)Ncap, (long long)t0);
    if (d != qjl::kD) return fail(QJL_ERR_UNSUPPORTED, "d=%d unsupported (only d=128)", d);
    if (nbits != 2 && nbits != 3 && nbits != 4) return fail(QJL_ERR_UNSUPPORTED, "nbits=%d unsupported (2, 3 or 4)", nbits);
    if (t0 + T > Ncap) return fail(QJL_ERR_INVALID_ARG, "t0 + T = %lld exceeds Ncap = %lld", (long long)(t0 + T), (long long)Ncap);
    if (B == 0 || T == 0) return QJL_OK;
    if (!V || !codes || !meta) return fail(QJL_ERR_INVALID_ARG, "null device pointer");
    if (sV_b < 0 || sV_t < 0 || sV_h < 0) return fail(QJL_ERR_INVALID_ARG, "negative stride");
    const int64_t vec = vdt == QJL_BF16 ? 8 : 4;
    if (!aligned16(V) || !aligned16(codes) || !aligned16(meta) || sV_b % vec || sV_t % vec || sV_h % vec)
        return fail(QJL_ERR_MISALIGNED, "pointers must be 16-byte aligned and strides multiples of %lld elements", (long long)vec);
    qjl::ValueQuantArgs a{};
    a.V = V;
    a.sVb = sV_b;
    a.sVt = sV_t;
    a.sVh = sV_h;
    a.codes = codes;
    a.meta = meta;
    a.T = T;
    a.Ncap = Ncap;
    a.t0 = t0;
    a.B = B;
    a.Hkv = Hkv;
    a.nbits = nbits;
    qjl::timer_begin(qjl::TK_QUANT_VALUES, stream);
    hipError_t e = qjl::launch_quantize_values(a, vdt, stream);
    qjl::timer_end(qjl::TK_QUANT_VALUES, stream);
    return hip_status(e, "qjl_quantize_values launch");
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

namespace {

// workspace regions: query operands, per-head constants, chunk partials
struct WsLayout {
    size_t sq, qconst, part, total;
};
WsLayout ws_layout(int B, int Hq, int d, int m, int m_out, int ns) {
    WsLayout w;
    w.sq = 0;
    w.qconst = w.sq + align256((size_t)B * Hq * (m + m_out) * sizeof(float));
    w.part = w.qconst + align256((size_t)B * Hq * 4 * sizeof(float));
    w.total = w.part + align256((size_t)B * Hq * ns * (d + 2) * sizeof(float));
    return w;
}

// Checks shared by the decode entry points (everything but the value arguments and the pointers),
// then the launch descriptor.
int prepare_decode(qjl::DecodeArgs& a, int qdt, int B, int Hq, int Hkv, int d, int64_t N, int m, int m_out, int n_out,
                   int64_t Ncap, int vmode, int nbits, float sm_scale, int estimator, int path, int nsplit) {
    if (qdt != QJL_BF16 && qdt != QJL_F32) return fail(QJL_ERR_INVALID_ARG, "qdt=%d is not a qjl_dtype", qdt);
    if (path != QJL_PATH_AUTO && path != QJL_PATH_MATRIX && path != QJL_PATH_VECTOR)
        return fail(QJL_ERR_INVALID_ARG, "path=%d is not a qjl_decode_path", path);
    if (estimator != QJL_EST_ONE_SIDED && estimator != QJL_EST_TWO_SIDED)
        return fail(QJL_ERR_INVALID_ARG, "estimator=%d is not a qjl_estimator", estimator);
    if (vmode != QJL_V_CODES && vmode != QJL_V_F32) return fail(QJL_ERR_INVALID_ARG, "vmode=%d is not a qjl_vmode", vmode);
    if (B < 0 || Hq <= 0 || Hkv <= 0 || N < 0 || Ncap < 0)
        return fail(QJL_ERR_INVALID_ARG, "bad sizes B=%d Hq=%d Hkv=%d N=%lld Ncap=%lld", B, Hq, Hkv, (long long)N, (long long)Ncap);
    if (Hq % Hkv) return fail(QJL_ERR_INVALID_ARG, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
    if (N > Ncap) return fail(QJL_ERR_INVALID_ARG, "N=%lld exceeds Ncap=%lld", (long long)N, (long long)Ncap);
    if (Ncap * (int64_t)((m + m_out) / 32) >= ((int64_t)1 << 30) || Ncap * (int64_t)qjl::kD >= ((int64_t)1 << 30))
        return fail(QJL_ERR_UNSUPPORTED, "Ncap=%lld too large for one (sequence, KV head) row (32-bit offsets)", (long long)Ncap);
    int st = check_sketch_shape(d, m, m_out, n_out);
    if (st) return st;
    if (!qjl::decode_shape_supported(m, m_out))
        return fail(QJL_ERR_UNSUPPORTED, "decode supports m in {128, 256, 512} with m_out in {0, m}; got m=%d m_out=%d", m, m_out);
    if (vmode == QJL_V_CODES && (nbits < 2 || nbits > 4))
        return fail(QJL_ERR_UNSUPPORTED, "decode of %d-bit value codes unsupported (2, 3 or 4)", nbits);
    if (vmode == QJL_V_CODES && nbits != 2 && !qjl::decode_uses_mfma(m, m_out, QJL_V_CODES, nbits))
        return fail(QJL_ERR_UNSUPPORTED, "decode of %d-bit value codes needs m + m_out <= 512 (got m=%d m_out=%d)", nbits, m,
                    m_out);
    if (path == QJL_PATH_MATRIX && !qjl::decode_uses_mfma(m, m_out, vmode, nbits))
        return fail(QJL_ERR_UNSUPPORTED, "the matrix-core decode needs value codes and (m, m_out) in {(128|256|512, 0), "
                    "(128, 128), (256, 256)}; got m=%d m_out=%d %s", m, m_out, vmode == QJL_V_CODES ? "codes" : "fp32 values");
    if (path == QJL_PATH_VECTOR && vmode == QJL_V_CODES && nbits != 2)
        return fail(QJL_ERR_UNSUPPORTED, "the vector-unit decode reads 2-bit value codes or fp32 values (got %d-bit codes)", nbits);
    if (nsplit > qjl::kMaxSplits) return fail(QJL_ERR_UNSUPPORTED, "nsplit=%d exceeds %d", nsplit, qjl::kMaxSplits);
    const int g = Hq / Hkv;
    const int ns = nsplit > 0 ? nsplit : qjl::decode_pick_nsplit(B, Hkv, g, N, m, m_out);
    a.ws_need = ws_layout(B, Hq, d, m, m_out, ns).total;
    a.N = N;
    a.Ncap = Ncap;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.g = g;
    a.m = m;
    a.m_out = m_out;
    a.n_out = n_out;
    a.nsplit = ns;
    a.nbits = vmode == QJL_V_CODES ? nbits : 2;
    a.chunk = qjl::decode_chunk(N, ns);
    const float scale = sm_scale > 0.f ? sm_scale : 1.0f / sqrtf((float)d);
    a.z_scale = scale * qjl::kLog2e;
    a.estimator = estimator;
    a.path = path;
    return QJL_OK;
}

// after the other pointer checks: the workspace the launch descriptor points into (its regions are
// laid out from the sizes prepare_decode recorded)
int bind_workspace(qjl::DecodeArgs& a, void* workspace, size_t ws_bytes) {
    if (!workspace || ws_bytes < a.ws_need)
        return fail(QJL_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", a.ws_need, workspace ? ws_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(QJL_ERR_MISALIGNED, "device pointers must be 16-byte aligned");
    const WsLayout w = ws_layout(a.B, a.Hq, qjl::kD, a.m, a.m_out, a.nsplit);
    char* base = static_cast<char*>(workspace);
    a.sq = reinterpret_cast<float*>(base + w.sq);
    a.qconst = reinterpret_cast<float*>(base + w.qconst);
    a.part = reinterpret_cast<float*>(base + w.part);
    return QJL_OK;
}

}  // namespace

size_t qjl_decode_workspace_size(int B, int Hq, int Hkv, int d, int64_t N, int m, int m_out, int nsplit) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || N < 0 || m <= 0 || m_out < 0 || d <= 0) return 0;
    const int ns = nsplit > 0 ? nsplit : qjl::decode_pick_nsplit(B, Hkv, Hq / Hkv, N, m, m_out);
    return ws_layout(B, Hq, d, m, m_out, ns).total;
}

int qjl_decode_attention(const void* Q, int qdt, int B, int Hq, int Hkv, int d, int64_t N, const void* S_in, int m,
                         const void* S_out, int m_out, const int32_t* outlier_idx, int n_out, const uint32_t* bits,
                         const uint16_t* norms, int64_t Ncap, int vmode, const uint32_t* codes, const uint16_t* meta,
                         const float* V_f32, int nbits, float sm_scale, int estimator, int path, float* out, float* scores_dbg,
                         int nsplit, void* workspace, size_t ws_bytes, hipStream_t stream) {
    g_last_error.clear();
    qjl::DecodeArgs a{};
    int st = prepare_decode(a, qdt, B, Hq, Hkv, d, N, m, m_out, n_out, Ncap, vmode, nbits, sm_scale, estimator, path, nsplit);
    if (st) return st;
    if (B == 0) return QJL_OK;
    if (!Q || !S_in || !bits || !norms || !out || (m_out && !S_out) || (n_out && !outlier_idx) ||
        (vmode == QJL_V_CODES && (!codes || !meta)) || (vmode == QJL_V_F32 && !V_f32))
        return fail(QJL_ERR_INVALID_ARG, "null device pointer");
    if (!aligned16(Q) || !aligned16(S_in) || (m_out && !aligned16(S_out)) || !aligned16(bits) || !aligned16(norms) ||
        !aligned16(out) || (scores_dbg && !aligned16(scores_dbg)) ||
        (vmode == QJL_V_CODES && (!aligned16(codes) || !aligned16(meta))) || (vmode == QJL_V_F32 && !aligned16(V_f32)))
        return fail(QJL_ERR_MISALIGNED, "device pointers must be 16-byte aligned");
    st = bind_workspace(a, workspace, ws_bytes);
    if (st) return st;
    a.Q = Q;
    a.S_in = S_in;
    a.S_out = S_out;
    a.oidx = outlier_idx;
    a.bits = bits;
    a.norms = norms;
    a.codes = codes;
    a.meta = meta;
    a.V_f32 = V_f32;
    a.out = out;
    a.scores_dbg = scores_dbg;
    return hip_status(qjl::launch_decode(a, qdt, vmode, stream), "qjl_decode_attention launch");
}

}  // extern "C"

// ------------------------------------------------------------------ allocation-free decode step
// The workspace of qjl_decode_step_no_alloc: a fixed array in device memory, one copy per GPU.  In
// host code `scratch` names a host-side stand-in, not device memory: its device address on each GPU
// comes from hipGetSymbolAddress (with that GPU current) and only that address is ever passed on.
static __device__ __align__(256) uint8_t scratch[QJL_NO_ALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

int scratch_of_current_device(void** ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxScratchDevices) return fail(QJL_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxScratchDevices);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
        if (!p) return fail(QJL_ERR_HIP, "hipGetSymbolAddress(scratch) returned a null address");
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return QJL_OK;
}

// qjl_decode_step and qjl_decode_step_no_alloc: every argument is checked first; then the workspace is
// the caller's (no_alloc false) or the current device's scratch array (no_alloc true).
int decode_step_impl(const void* Q, const void* K_new, const void* V_new, int dt, int B, int Hq, int Hkv, int d, int64_t N,
                     int64_t sK_b, int64_t sK_h, int64_t sV_b, int64_t sV_h, const void* S_in, int m, const void* S_out,
                     int m_out, const int32_t* outlier_idx, int n_out, uint32_t* bits, uint16_t* norms, uint32_t* codes,
                     uint16_t* meta, int64_t Ncap, int nbits, float sm_scale, int estimator, int path, float* out,
                     float* scores_dbg, int nsplit, void* workspace, size_t ws_bytes, bool no_alloc, hipStream_t stream) {
    g_last_error.clear();
    if (N < 1) return fail(QJL_ERR_INVALID_ARG, "N=%lld: a decode step appends one token, so N >= 1", (long long)N);
    qjl::DecodeArgs a{};
    int st = prepare_decode(a, dt, B, Hq, Hkv, d, N, m, m_out, n_out, Ncap, QJL_V_CODES, nbits, sm_scale, estimator, path, nsplit);
    if (st) return st;
    if (B == 0) return QJL_OK;
    if (!Q || !K_new || !V_new || !S_in || !bits || !norms || !codes || !meta || !out || (m_out && !S_out) ||
        (n_out && !outlier_idx))
        return fail(QJL_ERR_INVALID_ARG, "null device pointer");
    if (sK_b < 0 || sK_h < 0 || sV_b < 0 || sV_h < 0) return fail(QJL_ERR_INVALID_ARG, "negative stride");
    const int64_t vec = dt == QJL_BF16 ? 8 : 4;
    if (!aligned16(Q) || !aligned16(K_new) || !aligned16(V_new) || !aligned16(S_in) || (m_out && !aligned16(S_out)) ||
        !aligned16(bits) || !aligned16(norms) || !aligned16(codes) || !aligned16(meta) || !aligned16(out) ||
        (scores_dbg && !aligned16(scores_dbg)) || sK_b % vec || sK_h % vec || sV_b % vec || sV_h % vec)
        return fail(QJL_ERR_MISALIGNED, "pointers must be 16-byte aligned and strides multiples of %lld elements", (long long)vec);
    if (no_alloc) {
        if (a.ws_need > QJL_NO_ALLOC_SCRATCH_BYTES)
            return fail(QJL_ERR_WORKSPACE, "qjl_decode_step_no_alloc: these sizes need %zu bytes of workspace; the fixed scratch holds %zu",
                        a.ws_need, (size_t)QJL_NO_ALLOC_SCRATCH_BYTES);
        st = scratch_of_current_device(&workspace);
        if (st) return st;
        ws_bytes = QJL_NO_ALLOC_SCRATCH_BYTES;
    }
    st = bind_workspace(a, workspace, ws_bytes);
    if (st) return st;
    if (dt == QJL_BF16 && path != QJL_PATH_VECTOR && qjl::decode_uses_mfma(m, m_out, QJL_V_CODES, nbits)) {
        a.Q = Q;
        a.S_in = S_in;
        a.S_out = S_out;
        a.oidx = outlier_idx;
        a.bits = bits;
        a.norms = norms;
        a.codes = codes;
        a.meta = meta;
        a.out = out;
        a.scores_dbg = scores_dbg;
        qjl::AppendArgs ap{};
        ap.K = static_cast<const uint16_t*>(K_new);
        ap.sKb = sK_b;
        ap.sKh = sK_h;
        ap.V = static_cast<const uint16_t*>(V_new);
        ap.sVb = sV_b;
        ap.sVh = sV_h;
        ap.bits = bits;
        ap.norms = norms;
        ap.codes = codes;
        ap.meta = meta;
        ap.pos = N - 1;
        return hip_status(qjl::launch_decode_step_mfma(a, ap, stream), "qjl_decode_step launch");
    }
    // other shapes, fp32 and the vector-unit path: the three operations one after the other (arguments
    // checked above)
    st = qjl_quantize_keys(K_new, dt, B, 1, Hkv, d, sK_b, 0, sK_h, S_in, m, S_out, m_out, outlier_idx, n_out, bits, norms,
                           Ncap, N - 1, stream);
    if (st) return st;
    st = qjl_quantize_values(V_new, dt, B, 1, Hkv, d, sV_b, 0, sV_h, nbits, codes, meta, Ncap, N - 1, stream);
    if (st) return st;
    return qjl_decode_attention(Q, dt, B, Hq, Hkv, d, N, S_in, m, S_out, m_out, outlier_idx, n_out, bits, norms, Ncap,
                                QJL_V_CODES, codes, meta, nullptr, nbits, sm_scale, estimator, path, out, scores_dbg, nsplit,
                                workspace, ws_bytes, stream);
}

}  // namespace

extern "C" {

int qjl_decode_step(const void* Q, const void* K_new, const void* V_new, int dt, int B, int Hq, int Hkv, int d, int64_t N,
                    int64_t sK_b, int64_t sK_h, int64_t sV_b, int64_t sV_h, const void* S_in, int m, const void* S_out,
                    int m_out, const int32_t* outlier_idx, int n_out, uint32_t* bits, uint16_t* norms, uint32_t* codes,
                    uint16_t* meta, int64_t Ncap, int nbits, float sm_scale, int estimator, int path, float* out,
                    float* scores_dbg, int nsplit, void* workspace, size_t ws_bytes, hipStream_t stream) {
    return decode_step_impl(Q, K_new, V_new, dt, B, Hq, Hkv, d, N, sK_b, sK_h, sV_b, sV_h, S_in, m, S_out, m_out, outlier_idx,
                            n_out, bits, norms, codes, meta, Ncap, nbits, sm_scale, estimator, path, out, scores_dbg, nsplit,
                            workspace, ws_bytes, false, stream);
}

int qjl_decode_step_no_alloc(const void* Q, const void* K_new, const void* V_new, int dt, int B, int Hq, int Hkv, int d,
                             int64_t N, int64_t sK_b, int64_t sK_h, int64_t sV_b, int64_t sV_h, const void* S_in, int m,
                             const void* S_out, int m_out, const int32_t* outlier_idx, int n_out, uint32_t* bits,
                             uint16_t* norms, uint32_t* codes, uint16_t* meta, int64_t Ncap, int nbits, float sm_scale,
                             int estimator, int path, float* out, float* scores_dbg, int nsplit, hipStream_t stream) {
    return decode_step_impl(Q, K_new, V_new, dt, B, Hq, Hkv, d, N, sK_b, sK_h, sV_b, sV_h, S_in, m, S_out, m_out, outlier_idx,
                            n_out, bits, norms, codes, meta, Ncap, nbits, sm_scale, estimator, path, out, scores_dbg, nsplit,
                            nullptr, 0, true, stream);
}

size_t qjl_select_outliers_workspace_size(int B, int64_t T, int Hkv, int d) {
    if (B < 0 || T < 0 || Hkv <= 0 || d != qjl::kD) return 0;
    const int64_t nb = qjl::outlier_token_blocks(B, T, Hkv);
    return align256((size_t)(nb > 0 ? nb : 1) * (size_t)(B > 0 ? B : 1) * Hkv * qjl::kD * sizeof(double));
}

int qjl_select_outliers(const void* K, int kdt, int B, int64_t T, int Hkv, int d, int64_t sK_b, int64_t sK_t,
                        int64_t sK_h, int n_out, int32_t* outlier_idx, void* workspace, size_t ws_bytes,
                        hipStream_t stream) {
    g_last_error.clear();
    if (kdt != QJL_BF16 && kdt != QJL_F32) return fail(QJL_ERR_INVALID_ARG, "kdt=%d is not a qjl_dtype", kdt);
    if (B < 0 || T < 0 || Hkv <= 0 || n_out < 0)
        return fail(QJL_ERR_INVALID_ARG, "bad sizes B=%d T=%lld Hkv=%d n_out=%d", B, (long long)T, Hkv, n_out);
    if (d != qjl::kD) return fail(QJL_ERR_UNSUPPORTED, "d=%d unsupported (only d=128)", d);
    if (n_out > qjl::kMaxOutliers) return fail(QJL_ERR_UNSUPPORTED, "n_out=%d exceeds %d", n_out, qjl::kMaxOutliers);
    if (n_out == 0) return QJL_OK;
    if (!outlier_idx || (B > 0 && T > 0 && !K)) return fail(QJL_ERR_INVALID_ARG, "null device pointer");
    if (sK_b < 0 || sK_t < 0 || sK_h < 0) return fail(QJL_ERR_INVALID_ARG, "negative stride");
    const int64_t vec = kdt == QJL_BF16 ? 8 : 4;
    if ((K && !aligned16(K)) || !aligned16(outlier_idx) || sK_b % vec || sK_t % vec || sK_h % vec)
        return fail(QJL_ERR_MISALIGNED, "pointers must be 16-byte aligned and strides multiples of %lld elements", (long long)vec);
    const size_t need = qjl_select_outliers_workspace_size(B, T, Hkv, d);
    if (!workspace || ws_bytes < need)
        return fail(QJL_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? ws_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(QJL_ERR_MISALIGNED, "device pointers must be 16-byte aligned");
    qjl::OutlierArgs a{};
    a.K = K;
    a.sKb = sK_b;
    a.sKt = sK_t;
    a.sKh = sK_h;
    a.partial = static_cast<double*>(workspace);
    a.outlier_idx = outlier_idx;
    a.T = B > 0 ? T : 0;
    a.Hkv = Hkv;
    a.n_out = n_out;
    qjl::timer_begin(qjl::TK_SELECT, stream);
    const hipError_t e = qjl::launch_select_outliers(a, B, kdt, stream);
    qjl::timer_end(qjl::TK_SELECT, stream);
    return hip_status(e, "qjl_select_outliers launch");
}

}  // extern "C"
