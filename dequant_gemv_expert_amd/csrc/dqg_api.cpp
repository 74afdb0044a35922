// C-ABI layer of libdqg: argument validation, dispatch to the kernels,
// counters, fault injection and the expert table.  Every argument is
// checked before any HIP call, so a rejected call launches nothing and
// writes nothing.
#include "../../include/dqg.h"
#include "dqg_internal.h"

#include <atomic>
#include <mutex>
#include <vector>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

using namespace dqg;

struct dqg_expert_table {
    ExpertDev *dev;       // device array [n]
    int32_t n;
    int device;
    int codec_gu, codec_down;
    int32_t H, I;
    float swiglu_limit;   // +inf: plain SwiGLU
    int32_t act;          // DQG_ACT_SWIGLU or DQG_ACT_SWIGLU_V4
};

namespace {

thread_local char g_err[512] = "";

std::atomic<uint64_t> g_calls_matmul{0}, g_calls_gate_up{0}, g_calls_dequant{0},
    g_calls_group{0}, g_calls_route{0}, g_launches{0}, g_bytes{0};
std::atomic<long> g_launch_attempts{0};

int fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

// DQG_FAULT=n: the n-th launch attempt of the process fails before
// reaching the GPU (host-side fault injection for error-path tests).
bool inject_fault() {
    static const long fault_at = [] {
        const char *v = std::getenv("DQG_FAULT");
        return v ? std::strtol(v, nullptr, 10) : 0L;
    }();
    const long n = ++g_launch_attempts;
    return fault_at > 0 && n == fault_at;
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool pow2(long v) { return v > 0 && (v & (v - 1)) == 0; }

int ilog2(long v) {
    int r = 0;
    while ((1L << r) < v) ++r;
    return r;
}

int codec_of(int fmt) {
    switch (fmt) {
    case DQG_I8_ROW:
    case DQG_I8_GS: return C_I8;
    case DQG_I4_ROW:
    case DQG_I4_GS: return C_I4;
    case DQG_I3_G64: return C_I3;
    case DQG_MXFP4: return C_FP4;
    case DQG_F32: return C_F32;
    case DQG_BF16: return C_BF16;
    case DQG_FP8_BLOCK: return C_FP8;
    case DQG_F16: return C_F16;
    }
    return 0;
}

bool has_scales(int fmt) { return fmt != DQG_F32 && fmt != DQG_BF16 && fmt != DQG_F16; }

// Inputs of one 16-byte code chunk (a whole group of 64 for int3).
int chunk_inputs(int fmt) {
    switch (fmt) {
    case DQG_I8_ROW:
    case DQG_I8_GS:
    case DQG_FP8_BLOCK: return 16;
    case DQG_I3_G64: return 64;
    case DQG_F32: return 4;
    case DQG_BF16:
    case DQG_F16: return 8;
    default: return 32;
    }
}

// Bytes of codes per input, times 8.
int code_bits(int fmt) {
    switch (fmt) {
    case DQG_I8_ROW:
    case DQG_I8_GS:
    case DQG_FP8_BLOCK: return 8;
    case DQG_I3_G64: return 3;
    case DQG_F32: return 32;
    case DQG_BF16:
    case DQG_F16: return 16;
    default: return 4;
    }
}

// Validate one matrix and translate it to the kernels' view.
int check_matrix(const dqg_matrix *W, const char *what, MatDev *out) {
    if (!W) return fail(DQG_EINVAL, "%s: matrix is NULL", what);
    const int fmt = W->fmt;
    if (!codec_of(fmt)) return fail(DQG_EFORMAT, "%s: unknown format %d", what, fmt);
    if (W->O < 1 || W->K < 1) return fail(DQG_ESHAPE, "%s: O=%d K=%d must be positive", what, W->O, W->K);
    const int cw = chunk_inputs(fmt);
    if (W->K % cw)
        return fail(DQG_ESHAPE, "%s: K=%d is not a multiple of %d for format %d", what, W->K, cw, fmt);
    switch (fmt) {
    case DQG_I8_ROW:
    case DQG_I4_ROW:
        if (W->gs != W->K) return fail(DQG_EFORMAT, "%s: format %d has one scale per row (gs must be K=%d, got %d)", what, fmt, W->K, W->gs);
        break;
    case DQG_I4_GS:
    case DQG_I8_GS:
        if (!pow2(W->gs) || W->gs < 32)
            return fail(DQG_EFORMAT, "%s: gs=%d must be a power of two >= 32", what, W->gs);
        if (W->K % W->gs) return fail(DQG_ESHAPE, "%s: K=%d is not a multiple of gs=%d", what, W->K, W->gs);
        break;
    case DQG_FP8_BLOCK:
        if (W->gs != 128) return fail(DQG_EFORMAT, "%s: format 12 has 128 x 128 blocks (gs must be 128, got %d)", what, W->gs);
        if (W->K % 128) return fail(DQG_ESHAPE, "%s: K=%d is not a multiple of 128 for format 12", what, W->K);
        break;
    case DQG_F32:
    case DQG_BF16:
    case DQG_F16:
        if (W->gs != 0 && W->gs != W->K)
            return fail(DQG_EFORMAT, "%s: format %d has no scales (gs must be 0 or K=%d, got %d)", what, fmt, W->K, W->gs);
        if (W->scales) return fail(DQG_EINVAL, "%s: format %d has no scales (scales must be NULL)", what, fmt);
        break;
    case DQG_I3_G64:
        if (W->gs != 64) return fail(DQG_EFORMAT, "%s: format 5 has gs 64 (got %d)", what, W->gs);
        break;
    case DQG_MXFP4:
        if (W->gs != 32) return fail(DQG_EFORMAT, "%s: format 7 has gs 32 (got %d)", what, W->gs);
        break;
    }
    if (!W->q || !aligned(W->q, 16)) return fail(DQG_EINVAL, "%s: q must be a 16-byte aligned device pointer", what);
    if (has_scales(fmt) && (!W->scales || !aligned(W->scales, 4)))
        return fail(DQG_EINVAL, "%s: scales must be a 4-byte aligned device pointer", what);
    if (fmt == DQG_I3_G64 && (!W->q2 || !aligned(W->q2, 16)))
        return fail(DQG_EINVAL, "%s: format 5 needs a 16-byte aligned q2 (the 1-bit plane)", what);
    MatDev m{};
    m.q = static_cast<const uint8_t *>(W->q);
    m.q2 = fmt == DQG_I3_G64 ? static_cast<const uint8_t *>(W->q2) : nullptr;
    m.s = W->scales;
    m.O = W->O;
    m.K = W->K;
    if (fmt == DQG_I3_G64) {
        m.qstride = W->K / 4;
        m.q2stride = W->K / 8;
    } else {
        m.qstride = (int32_t)((int64_t)W->K * code_bits(fmt) / 8);
    }
    m.srow = 0;
    if (!has_scales(fmt)) {
        m.s = nullptr;
        m.sstride = 0;
        m.shift = 31;
    } else if (fmt == DQG_I8_ROW || fmt == DQG_I4_ROW) {
        m.sstride = 1;
        m.shift = 31;
    } else {
        m.sstride = W->K / W->gs;
        m.shift = ilog2(W->gs / cw);
        if (fmt == DQG_FP8_BLOCK) m.srow = 7;   // 128 rows share a row of block scales
    }
    *out = m;
    return DQG_OK;
}

int check_vec(const void *p, const char *what) {
    if (!p || !aligned(p, 16)) return fail(DQG_EINVAL, "%s must be a 16-byte aligned device pointer", what);
    return DQG_OK;
}

int launched(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(DQG_ELAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
    return DQG_OK;
}

uint64_t matrix_bytes(const dqg_matrix *W) {
    const uint64_t codes = (uint64_t)W->O * W->K * code_bits(W->fmt) / 8;
    uint64_t scales = 0;
    if (W->fmt == DQG_FP8_BLOCK)
        scales = (uint64_t)((W->O + 127) / 128) * (W->K / 128);
    else if (has_scales(W->fmt))
        scales = (uint64_t)W->O * (W->K / W->gs);
    return codes + scales * 4;
}

void prof_call();   // event timing: counts an API call (below)

constexpr int32_t MAX_S = 256, MAX_K = 64, MAX_SLOTS = 2048;

// Scratch: a fixed header (the error flag at byte 0; the rest is reserved),
// then h [S*k + S][I] f32 from byte DQG_SCRATCH_H_OFFSET.  The header sits
// at the same place for every S, so one scratch serves calls of any size.
// The gate/up launch clears the flag, so the scratch needs no initialisation.
size_t group_h_bytes(int32_t S, int32_t k, int32_t I) {
    const size_t slots = (size_t)S * k + S;
    return (slots * I * sizeof(float) + 255) / 256 * 256;
}
constexpr size_t FLAG_OFFSET = 0;

// scratch == nullptr with use_static: the library's static per-device
// scratch (dqg_expert_group_noalloc), resolved after every argument check.
int group_common(const dqg_expert_table *t, int32_t S, int32_t k, const int32_t *ids,
                 const float *w, int32_t shared, const float *x, float *y, void *scratch,
                 size_t scratch_bytes, void *stream, int32_t **flag_out, bool use_static = false) {
    ++g_calls_group;
    prof_call();
    if (!t) return fail(DQG_EINVAL, "expert_group: table is NULL");
    if (S < 1 || S > MAX_S) return fail(DQG_EINVAL, "expert_group: S=%d outside [1, %d]", S, MAX_S);
    if (k < 1 || k > MAX_K) return fail(DQG_EINVAL, "expert_group: k=%d outside [1, %d]", k, MAX_K);
    if ((long)S * k + S > MAX_SLOTS) return fail(DQG_EINVAL, "expert_group: S*(k+1)=%ld exceeds %d", (long)S * (k + 1), MAX_SLOTS);
    if (shared < -1 || shared >= t->n) return fail(DQG_EINVAL, "expert_group: shared=%d outside [-1, %d)", shared, t->n);
    if (!ids || !aligned(ids, 4)) return fail(DQG_EINVAL, "expert_group: ids must be a 4-byte aligned device pointer");
    if (!w || !aligned(w, 4)) return fail(DQG_EINVAL, "expert_group: w must be a 4-byte aligned device pointer");
    int rc;
    if ((rc = check_vec(x, "expert_group: x")) || (rc = check_vec(y, "expert_group: y")) ||
        (!use_static && (rc = check_vec(scratch, "expert_group: scratch"))))
        return rc;
    const size_t need = dqg_expert_group_scratch_bytes(t, S, k);
    if (use_static) {
        if (need > STATIC_SCRATCH_BYTES)
            return fail(DQG_ENOMEM, "expert_group_noalloc: S=%d, k=%d, I=%d need %zu bytes of scratch, more than "
                                    "the %zu the library holds", S, k, t->I, need, STATIC_SCRATCH_BYTES);
        const hipError_t e = static_scratch(&scratch);
        if (e != hipSuccess)
            return fail(DQG_EDEVICE, "expert_group_noalloc: the scratch's device address: %s", hipGetErrorString(e));
        scratch_bytes = STATIC_SCRATCH_BYTES;
    }
    if (scratch_bytes < need)
        return fail(DQG_ENOMEM, "expert_group: scratch holds %zu bytes, %zu needed", scratch_bytes, need);
    if (inject_fault()) return fail(DQG_ELAUNCH, "expert_group: injected launch failure (DQG_FAULT)");
    GroupArgs a{};
    a.table = t->dev;
    a.n_experts = t->n;
    a.S = S;
    a.k = k;
    a.ids = ids;
    a.w = w;
    a.shared = shared;
    a.x = x;
    a.y = y;
    char *base = static_cast<char *>(scratch);
    a.h = reinterpret_cast<float *>(base + DQG_SCRATCH_H_OFFSET);
    a.flag = reinterpret_cast<int32_t *>(base + FLAG_OFFSET);
    a.H = t->H;
    a.I = t->I;
    a.limit = t->swiglu_limit;
    a.act = t->act == DQG_ACT_SWIGLU_V4 ? ACT_SWIGLU_V4 : ACT_SWIGLU;
    int nl = 0;
    const hipError_t e = launch_group(t->codec_gu, t->codec_down, a, static_cast<hipStream_t>(stream), &nl);
    g_launches += nl;
    if ((rc = launched(e, "expert_group"))) return rc;
    if (flag_out) *flag_out = a.flag;
    return DQG_OK;
}

// Event timing of launches (dqg_prof_begin / dqg_prof_end).
struct Prof {
    std::mutex mu;
    std::atomic<bool> on{false};
    std::vector<hipEvent_t> ev;       // 2 per launch
    std::vector<const char *> name;   // per launch
    int used = 0;
    int every = 1;                    // time the launches of every every-th call
    std::atomic<long> calls{0};       // calls since dqg_prof_begin
};
Prof g_prof;
// Whether the calling thread's current API call has its launches timed.
thread_local bool t_prof_sampled = true;

// Called once at the start of every entry point that launches kernels.
void prof_call() {
    if (!g_prof.on.load(std::memory_order_relaxed)) return;
    t_prof_sampled = g_prof.calls.fetch_add(1, std::memory_order_relaxed) % g_prof.every == 0;
}

void prof_release() {
    for (hipEvent_t e : g_prof.ev) (void)hipEventDestroy(e);
    g_prof.ev.clear();
    g_prof.name.clear();
    g_prof.used = 0;
}

}  // namespace

bool dqg::prof_slot(const char *kernel, hipEvent_t *start, hipEvent_t *stop) {
    if (!g_prof.on.load(std::memory_order_relaxed) || !t_prof_sampled) return false;
    std::lock_guard<std::mutex> lock(g_prof.mu);
    if (g_prof.used >= (int)g_prof.name.size()) return false;
    *start = g_prof.ev[2 * g_prof.used];
    *stop = g_prof.ev[2 * g_prof.used + 1];
    g_prof.name[g_prof.used] = kernel;
    ++g_prof.used;
    return true;
}

extern "C" {

int dqg_prof_begin(int32_t capacity) { return dqg_prof_begin_sampled(capacity, 1); }

int dqg_prof_begin_sampled(int32_t capacity, int32_t every) {
    if (capacity < 1) return fail(DQG_EINVAL, "prof_begin: capacity=%d must be >= 1", capacity);
    if (every < 1) return fail(DQG_EINVAL, "prof_begin: every=%d must be >= 1", every);
    std::lock_guard<std::mutex> lock(g_prof.mu);
    prof_release();
    g_prof.every = every;
    g_prof.calls = 0;
    g_prof.ev.resize(2 * (size_t)capacity, nullptr);
    g_prof.name.assign(capacity, nullptr);
    for (auto &e : g_prof.ev) {
        if (hipEventCreate(&e) != hipSuccess) {
            e = nullptr;
            prof_release();
            return fail(DQG_EDEVICE, "prof_begin: hipEventCreate failed");
        }
    }
    g_prof.on = true;
    return DQG_OK;
}

int dqg_prof_end(dqg_prof_record *out, int32_t max, int32_t *n) {
    std::lock_guard<std::mutex> lock(g_prof.mu);
    g_prof.on = false;
    int count = 0, rc = DQG_OK;
    for (int i = 0; i < g_prof.used && rc == DQG_OK; ++i) {
        float ms = 0.f;
        hipError_t e = hipEventSynchronize(g_prof.ev[2 * i + 1]);
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, g_prof.ev[2 * i], g_prof.ev[2 * i + 1]);
        if (e != hipSuccess) {
            rc = fail(DQG_EDEVICE, "prof_end: %s", hipGetErrorString(e));
            break;
        }
        int j = 0;
        while (j < count && std::strcmp(out[j].kernel, g_prof.name[i]) != 0) ++j;
        if (j == count) {
            if (count >= max || !out) continue;
            std::memset(&out[j], 0, sizeof out[j]);
            std::snprintf(out[j].kernel, sizeof out[j].kernel, "%s", g_prof.name[i]);
            ++count;
        }
        out[j].launches += 1;
        out[j].total_ms += ms;
    }
    if (n) *n = count;
    prof_release();
    return rc;
}

int dqg_prof_end_launches(dqg_prof_launch *out, int32_t max, int32_t *n) {
    std::lock_guard<std::mutex> lock(g_prof.mu);
    g_prof.on = false;
    int count = 0, rc = DQG_OK;
    for (int i = 0; i < g_prof.used; ++i) {
        float ms = 0.f;
        hipError_t e = hipEventSynchronize(g_prof.ev[2 * i + 1]);
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, g_prof.ev[2 * i], g_prof.ev[2 * i + 1]);
        if (e != hipSuccess) {
            rc = fail(DQG_EDEVICE, "prof_end_launches: %s", hipGetErrorString(e));
            break;
        }
        if (!out || count >= max) continue;
        std::memset(&out[count], 0, sizeof out[count]);
        std::snprintf(out[count].kernel, sizeof out[count].kernel, "%s", g_prof.name[i]);
        out[count].ms = ms;
        ++count;
    }
    if (n) *n = count;
    prof_release();
    return rc;
}

int dqg_matmul(const dqg_matrix *W, const float *x, int32_t S, float *y, void *stream) {
    ++g_calls_matmul;
    prof_call();
    MatDev m;
    int rc;
    if ((rc = check_matrix(W, "matmul: W", &m))) return rc;
    if (S < 1) return fail(DQG_EINVAL, "matmul: S=%d must be >= 1", S);
    if ((rc = check_vec(x, "matmul: x")) || (rc = check_vec(y, "matmul: y"))) return rc;
    if (inject_fault()) return fail(DQG_ELAUNCH, "matmul: injected launch failure (DQG_FAULT)");
    hipError_t e = launch_matmul(codec_of(W->fmt), m, x, S, y, static_cast<hipStream_t>(stream));
    if ((rc = launched(e, "matmul"))) return rc;
    ++g_launches;
    g_bytes += matrix_bytes(W) + (uint64_t)S * (W->K + W->O) * 4;
    return DQG_OK;
}

namespace {

// A SwiGLU limit: positive (clamped) or +inf (plain).  Zero and negative
// limits are refused, as the backend's shader runs only above 0.
int check_limit(float limit, const char *what) {
    if (!(limit > 0.f)) return fail(DQG_EINVAL, "%s: swiglu limit %g must be > 0 (or +inf for none)", what, (double)limit);
    return DQG_OK;
}

int gate_up_common(const dqg_matrix *G, const dqg_matrix *U, const float *x, int32_t S, float limit, float *h,
                   void *stream) {
    ++g_calls_gate_up;
    prof_call();
    MatDev g, u;
    int rc;
    if ((rc = check_matrix(G, "gate_up: G", &g)) || (rc = check_matrix(U, "gate_up: U", &u))) return rc;
    if (G->fmt != U->fmt || G->O != U->O || G->K != U->K || G->gs != U->gs)
        return fail(DQG_ESHAPE, "gate_up: G and U must share format, shape and group size");
    if (S < 1) return fail(DQG_EINVAL, "gate_up: S=%d must be >= 1", S);
    if ((rc = check_limit(limit, "gate_up"))) return rc;
    if ((rc = check_vec(x, "gate_up: x")) || (rc = check_vec(h, "gate_up: h"))) return rc;
    if (inject_fault()) return fail(DQG_ELAUNCH, "gate_up: injected launch failure (DQG_FAULT)");
    hipError_t e = launch_gate_up(codec_of(G->fmt), g, u, x, S, h, limit, static_cast<hipStream_t>(stream));
    if ((rc = launched(e, "gate_up"))) return rc;
    ++g_launches;
    g_bytes += 2 * matrix_bytes(G) + (uint64_t)S * (G->K + G->O) * 4;
    return DQG_OK;
}

}  // namespace

int dqg_gate_up(const dqg_matrix *G, const dqg_matrix *U, const float *x, int32_t S, float *h,
                void *stream) {
    return gate_up_common(G, U, x, S, INFINITY, h, stream);
}

int dqg_gate_up_clamped(const dqg_matrix *G, const dqg_matrix *U, const float *x, int32_t S, float limit,
                        float *h, void *stream) {
    return gate_up_common(G, U, x, S, limit, h, stream);
}

int dqg_expert_table_set_swiglu_limit(dqg_expert_table *t, float limit) {
    if (!t) return fail(DQG_EINVAL, "expert_table_set_swiglu_limit: table is NULL");
    int rc;
    if ((rc = check_limit(limit, "expert_table_set_swiglu_limit"))) return rc;
    t->swiglu_limit = limit;
    return DQG_OK;
}

int dqg_expert_table_set_activation(dqg_expert_table *t, int32_t act) {
    if (!t) return fail(DQG_EINVAL, "expert_table_set_activation: table is NULL");
    if (act != DQG_ACT_SWIGLU && act != DQG_ACT_SWIGLU_V4)
        return fail(DQG_EINVAL, "expert_table_set_activation: unknown activation %d", act);
    if (act == DQG_ACT_SWIGLU_V4 && t->I % 128)
        return fail(DQG_EINVAL, "expert_table_set_activation: DeepSeek V4's activation rounds blocks of 128, "
                                "I=%d is not a multiple of 128", t->I);
    t->act = act;
    return DQG_OK;
}

int dqg_dequant(const dqg_matrix *W, float *out, void *stream) {
    ++g_calls_dequant;
    prof_call();
    MatDev m;
    int rc;
    if ((rc = check_matrix(W, "dequant: W", &m))) return rc;
    if ((rc = check_vec(out, "dequant: out"))) return rc;
    if (inject_fault()) return fail(DQG_ELAUNCH, "dequant: injected launch failure (DQG_FAULT)");
    hipError_t e = launch_dequant(codec_of(W->fmt), m, out, static_cast<hipStream_t>(stream));
    if ((rc = launched(e, "dequant"))) return rc;
    ++g_launches;
    g_bytes += matrix_bytes(W) + (uint64_t)W->O * W->K * 4;
    return DQG_OK;
}

int dqg_read_bytes(const void *p, uint64_t nbytes, uint32_t *sink, void *stream) {
    prof_call();
    if (!p || !aligned(p, 16)) return fail(DQG_EINVAL, "read_bytes: p must be a 16-byte aligned device pointer");
    if (nbytes == 0 || nbytes % 1024)
        return fail(DQG_EINVAL, "read_bytes: nbytes=%llu must be a positive multiple of 1024",
                    (unsigned long long)nbytes);
    if (!sink || !aligned(sink, 4)) return fail(DQG_EINVAL, "read_bytes: sink must be a 4-byte aligned device pointer");
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        return fail(DQG_EDEVICE, "read_bytes: no device");
    int rc;
    if ((rc = launched(launch_read(p, nbytes, sink, cus, static_cast<hipStream_t>(stream)), "read_bytes"))) return rc;
    ++g_launches;
    return DQG_OK;
}

int dqg_route(const float *logits, int32_t S, int32_t E, int32_t k, int32_t mode, int32_t renorm,
              const float *bias, float w_scale, int32_t *ids, float *w, void *stream) {
    ++g_calls_route;
    prof_call();
    if (S < 1) return fail(DQG_EINVAL, "route: S=%d, need S >= 1", S);
    if (E < 1 || E > ROUTE_MAX_E) return fail(DQG_EINVAL, "route: E=%d outside [1, %d]", E, ROUTE_MAX_E);
    if (k < 1 || k > E || k > 64) return fail(DQG_EINVAL, "route: k=%d outside [1, min(E, 64)]", k);
    if (mode != DQG_ROUTE_SOFTMAX && mode != DQG_ROUTE_SIGMOID)
        return fail(DQG_EINVAL, "route: mode=%d is neither DQG_ROUTE_SOFTMAX nor DQG_ROUTE_SIGMOID", mode);
    if (renorm != 0 && renorm != 1) return fail(DQG_EINVAL, "route: renorm=%d, need 0 or 1", renorm);
    if (!std::isfinite(w_scale)) return fail(DQG_EINVAL, "route: w_scale is not finite");
    if (!logits || !aligned(logits, 4)) return fail(DQG_EINVAL, "route: logits must be a 4-byte aligned device pointer");
    if (bias && !aligned(bias, 4)) return fail(DQG_EINVAL, "route: bias must be NULL or a 4-byte aligned device pointer");
    if (!ids || !aligned(ids, 4)) return fail(DQG_EINVAL, "route: ids must be a 4-byte aligned device pointer");
    if (!w || !aligned(w, 4)) return fail(DQG_EINVAL, "route: w must be a 4-byte aligned device pointer");
    if (inject_fault()) return fail(DQG_ELAUNCH, "route: injected launch failure (DQG_FAULT)");
    RouteArgs a{logits, S, E, k, mode, renorm, bias, w_scale, ids, w};
    int rc;
    if ((rc = launched(launch_route(a, static_cast<hipStream_t>(stream)), "route"))) return rc;
    ++g_launches;
    return DQG_OK;
}

int dqg_expert_table_create(const dqg_expert *experts, int32_t n, dqg_expert_table **out) {
    if (!out) return fail(DQG_EINVAL, "expert_table_create: out is NULL");
    *out = nullptr;
    if (!experts || n < 1) return fail(DQG_EINVAL, "expert_table_create: need n >= 1 experts");
    ExpertDev *host = static_cast<ExpertDev *>(std::calloc((size_t)n, sizeof(ExpertDev)));
    if (!host) return fail(DQG_ENOMEM, "expert_table_create: host allocation failed");
    const dqg_expert &e0 = experts[0];
    int rc = DQG_OK;
    for (int32_t i = 0; i < n && rc == DQG_OK; ++i) {
        const dqg_expert &e = experts[i];
        char what[64];
        snprintf(what, sizeof what, "expert %d gate", i);
        if ((rc = check_matrix(&e.gate, what, &host[i].gate))) break;
        snprintf(what, sizeof what, "expert %d up", i);
        if ((rc = check_matrix(&e.up, what, &host[i].up))) break;
        snprintf(what, sizeof what, "expert %d down", i);
        if ((rc = check_matrix(&e.down, what, &host[i].down))) break;
        if (e.up.fmt != e.gate.fmt || e.up.gs != e.gate.gs || e.up.O != e.gate.O || e.up.K != e.gate.K)
            rc = fail(DQG_ESHAPE, "expert %d: up must match gate's format, group size and shape", i);
        else if (e.down.O != e.gate.K || e.down.K != e.gate.O)
            rc = fail(DQG_ESHAPE, "expert %d: down must be [H x I] = [%d x %d]", i, e.gate.K, e.gate.O);
        else if (e.gate.fmt != e0.gate.fmt || e.gate.gs != e0.gate.gs || e.gate.O != e0.gate.O ||
                 e.gate.K != e0.gate.K || e.down.fmt != e0.down.fmt || e.down.gs != e0.down.gs)
            rc = fail(DQG_ESHAPE, "expert %d: every expert must share expert 0's formats and shapes", i);
    }
    if (rc != DQG_OK) {
        std::free(host);
        return rc;
    }
    dqg_expert_table *t = static_cast<dqg_expert_table *>(std::calloc(1, sizeof(dqg_expert_table)));
    if (!t) {
        std::free(host);
        return fail(DQG_ENOMEM, "expert_table_create: host allocation failed");
    }
    t->n = n;
    t->codec_gu = codec_of(e0.gate.fmt);
    t->codec_down = codec_of(e0.down.fmt);
    t->H = e0.gate.K;
    t->I = e0.gate.O;
    t->swiglu_limit = INFINITY;
    t->act = DQG_ACT_SWIGLU;
    hipError_t e = hipGetDevice(&t->device);
    if (e == hipSuccess) e = hipMalloc(reinterpret_cast<void **>(&t->dev), (size_t)n * sizeof(ExpertDev));
    if (e == hipSuccess) e = hipMemcpy(t->dev, host, (size_t)n * sizeof(ExpertDev), hipMemcpyHostToDevice);
    std::free(host);
    if (e != hipSuccess) {
        if (t->dev) (void)hipFree(t->dev);
        std::free(t);
        return fail(DQG_EDEVICE, "expert_table_create: %s", hipGetErrorString(e));
    }
    *out = t;
    return DQG_OK;
}

void dqg_expert_table_destroy(dqg_expert_table *t) {
    if (!t) return;
    if (t->dev) {
        int cur = 0;
        (void)hipGetDevice(&cur);
        (void)hipSetDevice(t->device);
        (void)hipFree(t->dev);
        (void)hipSetDevice(cur);
    }
    std::free(t);
}

size_t dqg_expert_group_scratch_bytes(const dqg_expert_table *t, int32_t S, int32_t k) {
    if (!t || S < 1 || k < 1) return 0;
    return DQG_SCRATCH_H_OFFSET + group_h_bytes(S, k, t->I);
}

int dqg_expert_group(const dqg_expert_table *t, int32_t S, int32_t k, const int32_t *ids,
                     const float *w, int32_t shared, const float *x, float *y, void *scratch,
                     size_t scratch_bytes, void *stream) {
    return group_common(t, S, k, ids, w, shared, x, y, scratch, scratch_bytes, stream, nullptr);
}

int dqg_expert_group_noalloc(const dqg_expert_table *t, int32_t S, int32_t k, const int32_t *ids,
                             const float *w, int32_t shared, const float *x, float *y, void *stream) {
    static_assert(STATIC_SCRATCH_BYTES == DQG_NOALLOC_SCRATCH_BYTES, "dqg.h states the static scratch's size");
    return group_common(t, S, k, ids, w, shared, x, y, nullptr, 0, stream, nullptr, true);
}

int dqg_expert_group_issue(const dqg_expert_table *t, int32_t S, int32_t k, const int32_t *ids,
                           const float *w, int32_t shared, const float *x, float *y, void *scratch,
                           size_t scratch_bytes, void *stream, dqg_ticket *ticket) {
    if (!ticket) return fail(DQG_EINVAL, "expert_group_issue: ticket is NULL");
    ticket->event = nullptr;
    ticket->flag = nullptr;
    ticket->status = DQG_OK;
    int32_t *flag = nullptr;
    int rc = group_common(t, S, k, ids, w, shared, x, y, scratch, scratch_bytes, stream, &flag);
    if (rc) return rc;
    hipEvent_t ev = nullptr;
    hipError_t e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventRecord(ev, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) {
        if (ev) (void)hipEventDestroy(ev);
        return fail(DQG_EDEVICE, "expert_group_issue: %s", hipGetErrorString(e));
    }
    ticket->event = ev;
    ticket->flag = flag;
    return DQG_OK;
}

int dqg_expert_group_take(dqg_ticket *ticket) {
    if (!ticket || !ticket->event) return fail(DQG_EINVAL, "expert_group_take: no issued call in this ticket");
    hipEvent_t ev = static_cast<hipEvent_t>(ticket->event);
    hipError_t e = hipEventSynchronize(ev);
    int32_t flag = 0;
    if (e == hipSuccess) e = hipMemcpy(&flag, ticket->flag, sizeof flag, hipMemcpyDeviceToHost);
    (void)hipEventDestroy(ev);
    ticket->event = nullptr;
    if (e != hipSuccess) {
        ticket->status = DQG_EDEVICE;
        return fail(DQG_EDEVICE, "expert_group_take: %s", hipGetErrorString(e));
    }
    if (flag) {
        ticket->status = DQG_EROUTE;
        return fail(DQG_EROUTE, "expert_group_take: an expert id was out of range (its token's row is NaN)");
    }
    ticket->status = DQG_OK;
    return DQG_OK;
}

const char *dqg_last_error(void) { return g_err; }

void dqg_stats(dqg_counters *out) {
    if (!out) return;
    out->calls_matmul = g_calls_matmul;
    out->calls_gate_up = g_calls_gate_up;
    out->calls_dequant = g_calls_dequant;
    out->calls_expert_group = g_calls_group;
    out->calls_route = g_calls_route;
    out->launches = g_launches;
    out->bytes = g_bytes;
}

void dqg_stats_reset(void) {
    g_calls_matmul = g_calls_gate_up = g_calls_dequant = g_calls_group = g_calls_route = 0;
    g_launches = g_bytes = 0;
}

}  // extern "C"
