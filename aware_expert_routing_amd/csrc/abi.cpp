// libmoe C ABI: host-side argument checks, then kernel launches on the
// caller's stream.  No call allocates memory or synchronises; invalid
// arguments return a negative status before anything is enqueued.
#include <stdio.h>
#include <string.h>

#include "internal.h"
#include "../../include/moe_probe.h"

#define MOE_API extern "C" __attribute__((visibility("default")))

namespace moe {
namespace {
thread_local char g_last_error[256] = "";
}

int fail(int status, const char* msg) {
    snprintf(g_last_error, sizeof g_last_error, "%s", msg);
    return status;
}

int hip_status(hipError_t e, const char* where) {
    if (e == hipSuccess) return MOE_OK;
    snprintf(g_last_error, sizeof g_last_error, "%s: %s", where, hipGetErrorString(e));
    return MOE_EHIP;
}

const char* last_error() { return g_last_error; }

}  // namespace moe

using moe::fail;
using moe::hip_status;

namespace {

int check_sizes(int B, int N, int k) {
    if (N < 1 || N > moe::kMaxExperts) return fail(MOE_EINVAL, "N must be in [1, 128]");
    if (k < 1 || k > N || k > moe::kMaxTopK) return fail(MOE_EINVAL, "k must be in [1, min(N, 16)]");
    if (B < 1) return fail(MOE_EINVAL, "B must be >= 1");
    if (B > moe::kMaxBatch) return fail(MOE_EUNSUPPORTED, "B > 128 is not supported");
    return MOE_OK;
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

}  // namespace

MOE_API const char* moe_status_str(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_EINVAL: return "invalid argument";
        case MOE_EUNSUPPORTED: return "unsupported size";
        case MOE_EHIP: return "HIP runtime error";
        case MOE_EFULL: return "no free block (retry later)";
        default: return "unknown status";
    }
}

MOE_API const char* moe_last_error(void) { return moe::last_error(); }

MOE_API int moe_router_logits(const void* x, int x_dtype, const float* w_r, int B, int H, int N,
                              float* logits, void* stream) {
    if (!x || !w_r || !logits) return fail(MOE_EINVAL, "null pointer");
    if (x_dtype != MOE_DT_F32 && x_dtype != MOE_DT_BF16) return fail(MOE_EINVAL, "bad x_dtype");
    if (N < 1 || N > moe::kMaxExperts) return fail(MOE_EINVAL, "N must be in [1, 128]");
    if (B < 1) return fail(MOE_EINVAL, "B must be >= 1");
    if (B > moe::kMaxBatch) return fail(MOE_EUNSUPPORTED, "B > 128 is not supported");
    if (H < 8 || H % 8) return fail(MOE_EINVAL, "H must be a positive multiple of 8");
    return hip_status(moe::launch_router_logits(x, x_dtype, w_r, B, H, N, logits, as_stream(stream)),
                      "moe_router_logits");
}

MOE_API int moe_route_topk(const float* logits, int B, int N, int k, int renorm, int32_t* idx,
                           float* w, void* stream) {
    if (!logits || !idx || !w) return fail(MOE_EINVAL, "null pointer");
    int st = check_sizes(B, N, k);
    if (st) return st;
    return hip_status(moe::launch_route(logits, B, N, k, k, 1.0f, 0, renorm ? 1 : 0, idx, w,
                                        nullptr, nullptr, nullptr, as_stream(stream)),
                      "moe_route_topk");
}

MOE_API int moe_route_oea(const float* logits, int B, int N, int k0, float p, int k, int32_t* idx,
                          float* w, int32_t* n_base, uint32_t* sbase_mask, int32_t* T,
                          void* stream) {
    if (!logits || !idx || !w) return fail(MOE_EINVAL, "null pointer");
    int st = check_sizes(B, N, k);
    if (st) return st;
    if (k0 < 1 || k0 > k) return fail(MOE_EINVAL, "k0 must be in [1, k]");
    if (!(p > 0.0f)) return fail(MOE_EINVAL, "p must be > 0 (p >= 1 disables top-p)");
    return hip_status(moe::launch_route(logits, B, N, k, k0, p, 1, 1, idx, w, n_base, sbase_mask, T,
                                        as_stream(stream)),
                      "moe_route_oea");
}

MOE_API int moe_dispatch(const int32_t* idx, int B, int N, int k, int32_t* cnt, int32_t* offsets,
                         int32_t* perm, int32_t* active, int32_t* T, void* stream) {
    if (!idx || !cnt || !offsets || !perm || !active || !T) return fail(MOE_EINVAL, "null pointer");
    int st = check_sizes(B, N, k);
    if (st) return st;
    return hip_status(moe::launch_dispatch(idx, B, N, k, cnt, offsets, perm, active, T,
                                           as_stream(stream)),
                      "moe_dispatch");
}

MOE_API int moe_route_dispatch(const float* logits, int B, int N, int k, int mode, int k0, float p, int max_p,
                               int renorm, const int32_t* n_valid, const int32_t* k0_by_batch, int32_t* idx,
                               float* w, int32_t* n_base,
                               uint32_t* sbase_mask, int32_t* cnt, int32_t* offsets, int32_t* perm,
                               int32_t* active, int32_t* T, int32_t* sync, void* stream) {
    if (!logits || !idx || !w || !cnt || !offsets || !perm || !active || !T) return fail(MOE_EINVAL, "null pointer");
    int st = check_sizes(B, N, k);
    if (st) return st;
    if (mode != MOE_ROUTE_TOPK && mode != MOE_ROUTE_OEA && mode != MOE_ROUTE_PRUNED)
        return fail(MOE_EINVAL, "bad routing mode");
    if (mode != MOE_ROUTE_TOPK) {
        if (k0 < 1 || k0 > k) return fail(MOE_EINVAL, "k0 must be in [1, k]");
        if (!(p > 0.0f)) return fail(MOE_EINVAL, "p must be > 0 (p >= 1 disables top-p)");
        if (mode == MOE_ROUTE_OEA && (max_p < k0 || max_p > N)) return fail(MOE_EINVAL, "max_p must be in [k0, N]");
    }
    const bool oea_like = mode != MOE_ROUTE_TOPK;
    return hip_status(moe::launch_route_dispatch(logits, B, N, k, mode, k0, p, mode == MOE_ROUTE_OEA ? max_p : N,
                                                 renorm, n_valid, oea_like ? k0_by_batch : nullptr, idx, w,
                                                 oea_like ? n_base : nullptr,
                                                 oea_like ? sbase_mask : nullptr, cnt, offsets, perm, active, T,
                                                 sync, as_stream(stream)),
                      "moe_route_dispatch");
}

MOE_API int moe_router_route_dispatch(const void* x, int x_dtype, const float* w_r, int B, int H, int N, int k,
                                      int mode, int k0, float p, int max_p, int renorm, const int32_t* n_valid,
                                      const int32_t* k0_by_batch, float* logits, int32_t* idx, float* w,
                                      int32_t* n_base, uint32_t* sbase_mask, int32_t* cnt, int32_t* offsets,
                                      int32_t* perm, int32_t* active, int32_t* T, int32_t* sync, void* stream) {
    if (!x || !w_r || !logits || !idx || !w || !cnt || !offsets || !perm || !active || !T || !sync)
        return fail(MOE_EINVAL, "null pointer");
    if (x_dtype != MOE_DT_F32 && x_dtype != MOE_DT_BF16) return fail(MOE_EINVAL, "bad x_dtype");
    if (H < 8 || H % 8) return fail(MOE_EINVAL, "H must be a positive multiple of 8");
    int st = check_sizes(B, N, k);
    if (st) return st;
    if (mode != MOE_ROUTE_TOPK && mode != MOE_ROUTE_OEA && mode != MOE_ROUTE_PRUNED)
        return fail(MOE_EINVAL, "bad routing mode");
    if (mode != MOE_ROUTE_TOPK) {
        if (k0 < 1 || k0 > k) return fail(MOE_EINVAL, "k0 must be in [1, k]");
        if (!(p > 0.0f)) return fail(MOE_EINVAL, "p must be > 0 (p >= 1 disables top-p)");
        if (mode == MOE_ROUTE_OEA && (max_p < k0 || max_p > N)) return fail(MOE_EINVAL, "max_p must be in [k0, N]");
    }
    const bool oea_like = mode != MOE_ROUTE_TOPK;
    return hip_status(moe::launch_router_route_dispatch(x, x_dtype, w_r, B, H, N, k, mode, k0, p, max_p, renorm,
                                                        n_valid, oea_like ? k0_by_batch : nullptr, logits, idx, w,
                                                        oea_like ? n_base : nullptr, oea_like ? sbase_mask : nullptr,
                                                        cnt, offsets, perm, active, T, sync, as_stream(stream)),
                      "moe_router_route_dispatch");
}

MOE_API size_t moe_ffn_workspace_bytes(int B, int k, int H, int I) {
    if (B < 1 || k < 1 || H < 1 || I < 1) return 0;
    return moe::ffn_workspace_bytes(B, k, H, I);
}

namespace {

// Checks shared by both expert-FFN entry points (everything but the workspace).
int check_ffn(const moe_expert_handle* table, int N, int H, int I, const void* x, int x_dtype, const int32_t* idx,
              const float* w, const int32_t* offsets, const int32_t* perm, const int32_t* active, const int32_t* T,
              int B, int k, float* y) {
    if (!table || !x || !idx || !w || !offsets || !perm || !active || !T || !y)
        return fail(MOE_EINVAL, "null pointer");
    int st = check_sizes(B, N, k);
    if (st) return st;
    if (x_dtype != MOE_DT_F32 && x_dtype != MOE_DT_BF16) return fail(MOE_EINVAL, "bad x_dtype");
    if (H < 32 || H % 32 || I < 32 || I % 32) return fail(MOE_EINVAL, "H and I must be positive multiples of 32");
    if (H > 16384 || I > 16384) return fail(MOE_EUNSUPPORTED, "H and I above 16384 are not supported");
    if (!moe::ffn_cost_fits(B, k, N, H, I)) return fail(MOE_EUNSUPPORTED, "B*k too large for H and I");
    if (reinterpret_cast<uintptr_t>(table) % 16 != 0) return fail(MOE_EINVAL, "handle table must be 16-byte aligned");
    return MOE_OK;
}

moe::FfnArgs ffn_args(const moe_expert_handle* table, int N, int H, int I, const void* x, int x_dtype,
                      const int32_t* idx, const float* w, const int32_t* offsets, const int32_t* perm,
                      const int32_t* active, const int32_t* T, int B, int k, float* y) {
    moe::FfnArgs a{};
    a.table = table;
    a.N = N; a.H = H; a.I = I; a.B = B; a.k = k;
    a.x = x; a.x_dtype = x_dtype;
    a.idx = idx; a.w = w; a.offsets = offsets; a.perm = perm; a.active = active; a.T = T;
    a.y = y;
    return a;
}

}  // namespace

MOE_API int moe_expert_ffn(const moe_expert_handle* table, int N, int H, int I, const void* x,
                           int x_dtype, const int32_t* idx, const float* w, const int32_t* offsets,
                           const int32_t* perm, const int32_t* active, const int32_t* T, int B,
                           int k, float* y, void* ws, size_t ws_bytes, void* stream) {
    if (!ws) return fail(MOE_EINVAL, "null pointer");
    int st = check_ffn(table, N, H, I, x, x_dtype, idx, w, offsets, perm, active, T, B, k, y);
    if (st) return st;
    if (ws_bytes < moe::ffn_workspace_bytes(B, k, H, I)) return fail(MOE_EINVAL, "workspace too small");
    if (reinterpret_cast<uintptr_t>(ws) % 256 != 0) return fail(MOE_EINVAL, "workspace must be 256-byte aligned");
    const moe::FfnArgs a = ffn_args(table, N, H, I, x, x_dtype, idx, w, offsets, perm, active, T, B, k, y);
    return hip_status(moe::launch_expert_ffn(a, ws, as_stream(stream)), "moe_expert_ffn");
}

MOE_API int moe_expert_ffn_noalloc(const moe_expert_handle* table, int N, int H, int I, const void* x,
                                   int x_dtype, const int32_t* idx, const float* w, const int32_t* offsets,
                                   const int32_t* perm, const int32_t* active, const int32_t* T, int B, int k,
                                   float* y, void* stream) {
    int st = check_ffn(table, N, H, I, x, x_dtype, idx, w, offsets, perm, active, T, B, k, y);
    if (st) return st;
    if (moe::ffn_workspace_bytes(B, k, H, I) > MOE_FFN_NOALLOC_WORKSPACE_BYTES)
        return fail(MOE_EUNSUPPORTED, "moe_ffn_workspace_bytes(B, k, H, I) exceeds the 32 MiB static workspace of "
                                      "moe_expert_ffn_noalloc");
    void* ws = nullptr;
    st = hip_status(moe::ffn_noalloc_workspace(&ws), "moe_expert_ffn_noalloc: static workspace lookup");
    if (st) return st;
    const moe::FfnArgs a = ffn_args(table, N, H, I, x, x_dtype, idx, w, offsets, perm, active, T, B, k, y);
    return hip_status(moe::launch_expert_ffn(a, ws, as_stream(stream)), "moe_expert_ffn_noalloc");
}

MOE_API int moe_handle_publish(moe_expert_handle* table, int e, const moe_expert_handle* h,
                               void* stream) {
    if (!table || !h) return fail(MOE_EINVAL, "null pointer");
    if (e < 0 || e >= moe::kMaxExperts) return fail(MOE_EINVAL, "expert index out of range");
    if (h->fmt != MOE_W_F32 && h->fmt != MOE_W_BF16 && h->fmt != MOE_W_INT4_G128)
        return fail(MOE_EINVAL, "bad weight format");
    if (!h->w_gate || !h->w_up || !h->w_down) return fail(MOE_EINVAL, "null weight pointer");
    if (h->fmt == MOE_W_INT4_G128 && (h->group != 128 || !h->s_gate || !h->s_up || !h->s_down))
        return fail(MOE_EINVAL, "INT4 handle needs group 128 and scale pointers");
    auto misaligned = [](const void* p, uintptr_t a) { return reinterpret_cast<uintptr_t>(p) % a != 0; };
    if (misaligned(h->w_gate, 16) || misaligned(h->w_up, 16) || misaligned(h->w_down, 16))
        return fail(MOE_EINVAL, "packed weights must be 16-byte aligned");
    if (h->fmt == MOE_W_INT4_G128 && (misaligned(h->s_gate, 8) || misaligned(h->s_up, 8) || misaligned(h->s_down, 8)))
        return fail(MOE_EINVAL, "packed scales must be 8-byte aligned");
    return hip_status(moe::launch_handle_publish(table, e, *h, as_stream(stream)), "moe_handle_publish");
}

MOE_API int moe_quantize_int4_g128(const uint16_t* w, int rows, int cols, uint8_t* q,
                                   uint16_t* scales, void* stream) {
    if (!w || !q || !scales) return fail(MOE_EINVAL, "null pointer");
    if (rows < 1 || cols < 128 || cols % 128) return fail(MOE_EINVAL, "cols must be a positive multiple of 128");
    return hip_status(moe::launch_quantize_int4(w, rows, cols, q, scales, as_stream(stream)),
                      "moe_quantize_int4_g128");
}

MOE_API int moe_pack_weights(int fmt, const void* src, const uint16_t* src_scales, int rows, int cols,
                             void* dst, uint16_t* dst_scales, void* stream) {
    if (fmt != MOE_W_F32 && fmt != MOE_W_BF16 && fmt != MOE_W_INT4_G128) return fail(MOE_EINVAL, "bad weight format");
    if (!src || !dst) return fail(MOE_EINVAL, "null pointer");
    if (fmt == MOE_W_INT4_G128 && (!src_scales || !dst_scales)) return fail(MOE_EINVAL, "INT4 needs scale pointers");
    if (rows < 16 || rows % 16) return fail(MOE_EINVAL, "rows must be a positive multiple of 16");
    const int tc = moe::tile_cols(fmt);
    if (cols < tc || cols % tc) return fail(MOE_EINVAL, "cols must be a positive multiple of 16/32/128 (fp32/bf16/INT4)");
    if (static_cast<long>(rows) * cols > (1L << 31)) return fail(MOE_EUNSUPPORTED, "matrix above 2^31 elements");
    if (reinterpret_cast<uintptr_t>(src) % 16 || reinterpret_cast<uintptr_t>(dst) % 16)
        return fail(MOE_EINVAL, "src and dst must be 16-byte aligned");
    const size_t bytes = static_cast<size_t>(rows) * moe::weight_row_bytes(fmt, cols);
    const char* s0 = static_cast<const char*>(src);
    char* d0 = static_cast<char*>(dst);
    if (s0 < d0 + bytes && d0 < s0 + bytes) return fail(MOE_EINVAL, "src and dst overlap");
    return hip_status(moe::launch_pack_weights(fmt, src, src_scales, rows, cols, dst, dst_scales, as_stream(stream)),
                      "moe_pack_weights");
}

MOE_API int moe_hotness_ema(float* S, const int32_t* cnt, int N, float alpha, void* stream) {
    if (!S || !cnt) return fail(MOE_EINVAL, "null pointer");
    if (N < 1 || N > moe::kMaxExperts) return fail(MOE_EINVAL, "N must be in [1, 128]");
    if (!(alpha >= 0.0f && alpha <= 1.0f)) return fail(MOE_EINVAL, "alpha must be in [0, 1]");
    return hip_status(moe::launch_hotness_ema(S, cnt, N, alpha, as_stream(stream)), "moe_hotness_ema");
}

MOE_API int moe_expert_ffn_phase_events(const moe_expert_handle* table, int N, int H, int I, const void* x,
                                        int x_dtype, const int32_t* idx, const float* w, const int32_t* offsets,
                                        const int32_t* perm, const int32_t* active, const int32_t* T, int B, int k,
                                        float* y, void* ws, size_t ws_bytes, void* const* events, void* stream) {
    if (!events) return fail(MOE_EINVAL, "null events array");
    int st = check_ffn(table, N, H, I, x, x_dtype, idx, w, offsets, perm, active, T, B, k, y);
    if (st) return st;
    if (!ws) return fail(MOE_EINVAL, "null workspace");
    if (ws_bytes < moe::ffn_workspace_bytes(B, k, H, I)) return fail(MOE_EINVAL, "workspace too small");
    if (reinterpret_cast<uintptr_t>(ws) % 256 != 0) return fail(MOE_EINVAL, "workspace must be 256-byte aligned");
    hipEvent_t ev[4];
    for (int i = 0; i < 4; ++i) ev[i] = static_cast<hipEvent_t>(events[i]);
    const moe::FfnArgs a = ffn_args(table, N, H, I, x, x_dtype, idx, w, offsets, perm, active, T, B, k, y);
    return hip_status(moe::launch_expert_ffn(a, ws, as_stream(stream), ev), "moe_expert_ffn_phase_events");
}

MOE_API int moe_stream_read(const void* buf, size_t bytes, int waves_per_cu, uint32_t* out, void* stream) {
    if (!buf || !out) return fail(MOE_EINVAL, "null pointer");
    if (bytes < 16 || bytes % 16) return fail(MOE_EINVAL, "bytes must be a positive multiple of 16");
    if (waves_per_cu < 4 || waves_per_cu > 32 || waves_per_cu % 4)
        return fail(MOE_EINVAL, "waves_per_cu must be 4, 8, ..., 32");
    if (reinterpret_cast<uintptr_t>(buf) % 16 || reinterpret_cast<uintptr_t>(out) % 4)
        return fail(MOE_EINVAL, "buf must be 16-byte aligned");
    return hip_status(moe::launch_stream_read(buf, bytes, waves_per_cu, out, moe::device_cus(), as_stream(stream)),
                      "moe_stream_read");
}
