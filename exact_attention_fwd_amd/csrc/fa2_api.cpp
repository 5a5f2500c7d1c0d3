// C-ABI entry points of libfa2 (declared in include/fa2.h).
//
// Every argument check runs before the first HIP call, so argument errors are
// reported the same way on a machine without a GPU.
#include "fa2.h"

#include <cfloat>
#include <cmath>
#include <cstddef>
#include <cstdint>
#include <utility>

#include "fa2_launch.h"

namespace {

thread_local int g_last_hip_error = 0;

bool overlaps(const void* a, size_t a_bytes, const void* b, size_t b_bytes) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a);
    const uintptr_t b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + b_bytes && b0 < a0 + a_bytes;
}

// A finite scale whose scores all stay finite in fp32: the largest score of
// fp16 inputs is d * 65504^2, and the kernels form scale * log2(e) * score
// (the exp2 argument) in fp32, so that product must not exceed FLT_MAX.
bool scale_ok(float scale, int d) {
    if (!std::isfinite(scale)) return false;
    const double top = 1.4426950408889634 * 65504.0 * 65504.0 * double(d);
    return std::fabs(double(scale)) * top <= double(FLT_MAX);
}

// Sizes, scale and head dim of the square-attention entry points (forward,
// backward, FA1 order); 0 when valid.
int check_sizes(int B, int H, int N, int d, float scale, int max_d) {
    if (B < 1 || H < 1 || N < 1) return FA2_ERR_INVALID_ARG;
    // Per-head byte offsets are 32-bit buffer offsets: N * d * 2 plus a few
    // tiles of prefetch must stay below 2^31.
    if (N > (1 << 22)) return FA2_ERR_INVALID_ARG;
    if (int64_t(B) * H * N > INT32_MAX) return FA2_ERR_INVALID_ARG;
    if ((d != 32 && d != 64 && d != 96 && d != 128 && d != 256) || d > max_d)
        return FA2_ERR_UNSUPPORTED;
    if (!scale_ok(scale, d)) return FA2_ERR_INVALID_ARG;
    if (int64_t(N) * d > (int64_t(1) << 29)) return FA2_ERR_INVALID_ARG;
    return 0;
}

int launch_status(hipError_t err) {
    if (err == hipSuccess) return FA2_OK;
    g_last_hip_error = static_cast<int>(err);
    switch (err) {
        case hipErrorNoDevice:
        case hipErrorInvalidDevice:
        case hipErrorInsufficientDriver:
        case hipErrorNoBinaryForGpu:
        case hipErrorNotInitialized:
            return FA2_ERR_NO_DEVICE;
        default:
            return FA2_ERR_LAUNCH;
    }
}

}  // namespace

extern "C" int fa2_fwd(const void* q, const void* k, const void* v, void* o,
                       float* lse, int B, int H, int N, int d, float scale,
                       int causal, void* stream) {
    if (!q || !k || !v || !o || !lse) return FA2_ERR_INVALID_ARG;
    if (const int st = check_sizes(B, H, N, d, scale, /*max_d=*/256)) return st;
    const int64_t rows = int64_t(B) * H * N;
    const uintptr_t bits = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                           reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(o) |
                           reinterpret_cast<uintptr_t>(lse);
    if (bits & 15u) return FA2_ERR_MISALIGNED;
    const size_t t_bytes = size_t(rows) * size_t(d) * 2;
    const size_t l_bytes = size_t(rows) * 4;
    for (const void* in : {q, k, v}) {
        if (overlaps(o, t_bytes, in, t_bytes) || overlaps(lse, l_bytes, in, t_bytes))
            return FA2_ERR_INVALID_ARG;
    }
    if (overlaps(lse, l_bytes, o, t_bytes)) return FA2_ERR_INVALID_ARG;

    return launch_status(fa2::launch_fwd(q, k, v, o, lse, B * H, N, d, scale, causal != 0,
                                         static_cast<hipStream_t>(stream)));
}

extern "C" int fa2_bwd(const void* q, const void* k, const void* v, const void* o,
                       const float* lse, const void* dout, void* dq, void* dk, void* dv,
                       float* delta, int B, int H, int N, int d, float scale, int causal,
                       void* stream) {
    if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !delta)
        return FA2_ERR_INVALID_ARG;
    if (const int st = check_sizes(B, H, N, d, scale, /*max_d=*/128)) return st;
    const uintptr_t bits = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                           reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(o) |
                           reinterpret_cast<uintptr_t>(lse) | reinterpret_cast<uintptr_t>(dout) |
                           reinterpret_cast<uintptr_t>(dq) | reinterpret_cast<uintptr_t>(dk) |
                           reinterpret_cast<uintptr_t>(dv) | reinterpret_cast<uintptr_t>(delta);
    if (bits & 15u) return FA2_ERR_MISALIGNED;
    const size_t rows = size_t(B) * H * N;
    const size_t t_bytes = rows * size_t(d) * 2;
    const size_t l_bytes = rows * 4;
    const struct { const void* p; size_t n; } ins[] = {
        {q, t_bytes}, {k, t_bytes}, {v, t_bytes}, {o, t_bytes}, {lse, l_bytes}, {dout, t_bytes}};
    const struct { const void* p; size_t n; } outs[] = {
        {dq, t_bytes}, {dk, t_bytes}, {dv, t_bytes}, {delta, l_bytes}};
    for (const auto& w : outs) {
        for (const auto& r : ins)
            if (overlaps(w.p, w.n, r.p, r.n)) return FA2_ERR_INVALID_ARG;
        for (const auto& w2 : outs)
            if (&w2 != &w && overlaps(w.p, w.n, w2.p, w2.n)) return FA2_ERR_INVALID_ARG;
    }
    return launch_status(fa2::launch_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B * H, N, d,
                                         scale, causal != 0, static_cast<hipStream_t>(stream)));
}

extern "C" size_t fa1_workspace_bytes(int B, int H, int N, int d) {
    if (B < 1 || H < 1 || N < 1 || d < 1 || int64_t(B) * H * N > INT32_MAX) return 0;
    return fa2::fa1_workspace_floats(B * H, N, d) * sizeof(float);
}

extern "C" int fa1_fwd(const void* q, const void* k, const void* v, void* o, float* lse, void* ws,
                       size_t ws_bytes, int B, int H, int N, int d, float scale, int causal,
                       void* stream) {
    if (!q || !k || !v || !o || !lse || !ws) return FA2_ERR_INVALID_ARG;
    if (const int st = check_sizes(B, H, N, d, scale, /*max_d=*/256)) return st;
    if (d != 64) return FA2_ERR_UNSUPPORTED;
    // fp32 per-head offsets of the workspace are 32-bit: N * d * 4 < 2^31.
    if (int64_t(N) * d > (int64_t(1) << 27)) return FA2_ERR_INVALID_ARG;
    const size_t rows = size_t(B) * H * N;
    const size_t t_bytes = rows * size_t(d) * 2;
    const size_t l_bytes = rows * 4;
    const size_t w_bytes = fa2::fa1_workspace_floats(B * H, N, d) * sizeof(float);
    if (ws_bytes < w_bytes) return FA2_ERR_INVALID_ARG;
    const uintptr_t bits = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                           reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(o) |
                           reinterpret_cast<uintptr_t>(lse) | reinterpret_cast<uintptr_t>(ws);
    if (bits & 15u) return FA2_ERR_MISALIGNED;
    const struct { const void* p; size_t n; } outs[] = {{o, t_bytes}, {lse, l_bytes}, {ws, w_bytes}};
    for (const auto& w : outs) {
        for (const void* in : {q, k, v})
            if (overlaps(w.p, w.n, in, t_bytes)) return FA2_ERR_INVALID_ARG;
        for (const auto& w2 : outs)
            if (&w2 != &w && overlaps(w.p, w.n, w2.p, w2.n)) return FA2_ERR_INVALID_ARG;
    }
    return launch_status(fa2::launch_fa1(q, k, v, o, lse, ws, B * H, N, d, scale, causal != 0,
                                         static_cast<hipStream_t>(stream)));
}

namespace {

// Sizes of the split key/value call; 0 when valid.
int check_splitkv_sizes(int B, int H, int Nq, int Nk, int d, float scale, int n_splits) {
    if (B < 1 || H < 1 || Nq < 1 || Nk < 1) return FA2_ERR_INVALID_ARG;
    if (Nq > (1 << 22) || Nk > (1 << 22)) return FA2_ERR_INVALID_ARG;
    if (int64_t(B) * H * Nq > INT32_MAX || int64_t(B) * H * Nk > INT32_MAX) return FA2_ERR_INVALID_ARG;
    if (n_splits < 0 || n_splits > 4096) return FA2_ERR_INVALID_ARG;
    if (d != 32 && d != 64 && d != 96 && d != 128) return FA2_ERR_UNSUPPORTED;
    if (!scale_ok(scale, d)) return FA2_ERR_INVALID_ARG;
    if (int64_t(Nq) * d > (int64_t(1) << 29) || int64_t(Nk) * d > (int64_t(1) << 29))
        return FA2_ERR_INVALID_ARG;
    return 0;
}

size_t splitkv_ws_bytes(int B, int H, int Nq, int d, const fa2::SplitPlan& p) {
    if (p.n_splits <= 1) return 0;
    return size_t(p.n_splits) * size_t(B) * H * Nq * (size_t(d) + 1) * sizeof(float);
}

}  // namespace

extern "C" int fa2_splitkv_splits(int B, int H, int Nq, int Nk, int d, int n_splits) {
    if (check_splitkv_sizes(B, H, Nq, Nk, d, 1.0f, n_splits)) return 0;
    return fa2::plan_splits(B * H, Nq, Nk, n_splits).n_splits;
}

extern "C" size_t fa2_splitkv_workspace_bytes(int B, int H, int Nq, int Nk, int d, int n_splits) {
    if (check_splitkv_sizes(B, H, Nq, Nk, d, 1.0f, n_splits)) return 0;
    return splitkv_ws_bytes(B, H, Nq, d, fa2::plan_splits(B * H, Nq, Nk, n_splits));
}

namespace {

// The checks of a split key/value call that do not involve its workspace,
// all before any HIP call; on success fills the plan and the workspace bytes
// it needs.
int check_splitkv_call(const void* q, const void* k, const void* v, const void* o,
                       const float* lse, int B, int H, int Nq, int Nk, int d, float scale,
                       int n_splits, fa2::SplitPlan* plan, size_t* w_bytes) {
    if (!q || !k || !v || !o || !lse) return FA2_ERR_INVALID_ARG;
    if (const int st = check_splitkv_sizes(B, H, Nq, Nk, d, scale, n_splits)) return st;
    *plan = fa2::plan_splits(B * H, Nq, Nk, n_splits);
    // one workgroup per (32-query tile, key range, batch * head)
    if (int64_t(B) * H * ((Nq + 31) / 32) * plan->n_splits > INT32_MAX) return FA2_ERR_INVALID_ARG;
    *w_bytes = splitkv_ws_bytes(B, H, Nq, d, *plan);
    const uintptr_t bits = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                           reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(o) |
                           reinterpret_cast<uintptr_t>(lse);
    if (bits & 15u) return FA2_ERR_MISALIGNED;
    const size_t q_bytes = size_t(B) * H * Nq * size_t(d) * 2;
    const size_t kv_bytes = size_t(B) * H * Nk * size_t(d) * 2;
    const size_t l_bytes = size_t(B) * H * Nq * 4;
    const struct { const void* p; size_t n; } ins[] = {{q, q_bytes}, {k, kv_bytes}, {v, kv_bytes}};
    for (const auto& r : ins) {
        if (overlaps(o, q_bytes, r.p, r.n) || overlaps(lse, l_bytes, r.p, r.n))
            return FA2_ERR_INVALID_ARG;
    }
    if (overlaps(o, q_bytes, lse, l_bytes)) return FA2_ERR_INVALID_ARG;
    return 0;
}

}  // namespace

extern "C" int fa2_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                               void* ws, size_t ws_bytes, int B, int H, int Nq, int Nk, int d,
                               float scale, int n_splits, void* stream) {
    fa2::SplitPlan plan;
    size_t w_bytes = 0;
    if (const int st = check_splitkv_call(q, k, v, o, lse, B, H, Nq, Nk, d, scale, n_splits, &plan,
                                          &w_bytes))
        return st;
    if (w_bytes) {
        if (!ws || ws_bytes < w_bytes) return FA2_ERR_INVALID_ARG;
        if (reinterpret_cast<uintptr_t>(ws) & 15u) return FA2_ERR_MISALIGNED;
        const size_t q_bytes = size_t(B) * H * Nq * size_t(d) * 2;
        const size_t kv_bytes = size_t(B) * H * Nk * size_t(d) * 2;
        const size_t l_bytes = size_t(B) * H * Nq * 4;
        const struct { const void* p; size_t n; } others[] = {
            {q, q_bytes}, {k, kv_bytes}, {v, kv_bytes}, {o, q_bytes}, {lse, l_bytes}};
        for (const auto& r : others)
            if (overlaps(ws, w_bytes, r.p, r.n)) return FA2_ERR_INVALID_ARG;
    }
    return launch_status(fa2::launch_splitkv(q, k, v, o, lse, w_bytes ? ws : nullptr, B * H, Nq, Nk,
                                             d, scale, plan, static_cast<hipStream_t>(stream)));
}

extern "C" int fa2_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o,
                                       float* lse, int B, int H, int Nq, int Nk, int d, float scale,
                                       int n_splits, void* stream) {
    fa2::SplitPlan plan;
    size_t w_bytes = 0;
    if (const int st = check_splitkv_call(q, k, v, o, lse, B, H, Nq, Nk, d, scale, n_splits, &plan,
                                          &w_bytes))
        return st;
    if (w_bytes > FA2_NOALLOC_SCRATCH_BYTES) return FA2_ERR_SCRATCH_LIMIT;
    void* ws = nullptr;
    if (w_bytes) {
        // The library's own buffer (no allocation); its per-device address
        // is looked up on the first call on a device.
        const hipError_t e = fa2::noalloc_scratch(static_cast<hipStream_t>(stream), &ws);
        if (e != hipSuccess) return launch_status(e);
    }
    return launch_status(fa2::launch_splitkv(q, k, v, o, lse, ws, B * H, Nq, Nk, d, scale, plan,
                                             static_cast<hipStream_t>(stream)));
}

extern "C" int fa2_lse_merge(const float* o_parts, const float* lse_parts, void* o, float* lse,
                             int n_parts, int rows, int d, void* stream) {
    if (!o_parts || !lse_parts || !o || !lse) return FA2_ERR_INVALID_ARG;
    if (n_parts < 1 || rows < 1 || int64_t(n_parts) * rows > INT32_MAX) return FA2_ERR_INVALID_ARG;
    if (d != 32 && d != 64 && d != 96 && d != 128) return FA2_ERR_UNSUPPORTED;
    const uintptr_t bits = reinterpret_cast<uintptr_t>(o_parts) |
                           reinterpret_cast<uintptr_t>(lse_parts) |
                           reinterpret_cast<uintptr_t>(o) | reinterpret_cast<uintptr_t>(lse);
    if (bits & 15u) return FA2_ERR_MISALIGNED;
    const size_t op_bytes = size_t(n_parts) * rows * size_t(d) * 4;
    const size_t lp_bytes = size_t(n_parts) * rows * 4;
    const size_t o_bytes = size_t(rows) * d * 2;
    const size_t l_bytes = size_t(rows) * 4;
    for (const auto& w : {std::make_pair(static_cast<const void*>(o), o_bytes),
                          std::make_pair(static_cast<const void*>(lse), l_bytes)}) {
        if (overlaps(w.first, w.second, o_parts, op_bytes) ||
            overlaps(w.first, w.second, lse_parts, lp_bytes))
            return FA2_ERR_INVALID_ARG;
    }
    if (overlaps(o, o_bytes, lse, l_bytes)) return FA2_ERR_INVALID_ARG;
    return launch_status(fa2::launch_lse_merge(o_parts, lse_parts, o, lse, n_parts, rows, d,
                                               static_cast<hipStream_t>(stream)));
}

extern "C" const char* fa2_status_string(int status) {
    switch (status) {
        case FA2_OK: return "ok";
        case FA2_ERR_INVALID_ARG: return "invalid argument";
        case FA2_ERR_UNSUPPORTED:
            return "unsupported head dimension (forward: 32, 64, 96, 128, 256; backward: 32 to 128)";
        case FA2_ERR_MISALIGNED: return "pointer not 16-byte aligned";
        case FA2_ERR_NO_DEVICE: return "no usable gfx950 device";
        case FA2_ERR_LAUNCH: return "kernel launch failed";
        case FA2_ERR_SCRATCH_LIMIT:
            return "the call needs more scratch than fa2_fwd_splitkv_noalloc's fixed buffer "
                   "(FA2_NOALLOC_SCRATCH_BYTES) holds: use fewer key ranges or fa2_fwd_splitkv";
        default: return "unknown status";
    }
}

extern "C" int fa2_last_hip_error(void) { return g_last_hip_error; }

extern "C" const char* fa2_version(void) { return "fa2-gfx950 0.1.0"; }
