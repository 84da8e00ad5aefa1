// Internal declarations shared by the libmoe translation units (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

constexpr int kMaxExperts = 128;
constexpr int kMaxTopK = 16;
constexpr int kMaxBatch = 128;

#ifdef __HIPCC__
// Inclusive prefix sum over the 64 lanes of a wavefront (all lanes active),
// in registers: DPP row shifts by 1, 2, 4 and 8 scan each row of 16 lanes,
// then the last lane of row 0 is added to row 1, of row 2 to row 3, and of
// row 1 (by then the total of rows 0-1) to rows 2 and 3.  Lanes a move does
// not reach add 0.
__device__ __forceinline__ int wave_incl_scan(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);   // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);   // row_bcast:15 -> rows 1, 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);   // row_bcast:31 -> rows 2, 3
    return v;
}
#endif

// Launchers: called after argument validation; return the launch status.
hipError_t launch_router_logits(const void* x, int x_dtype, const float* w_r, int B, int H, int N,
                                float* logits, hipStream_t s);
hipError_t launch_route(const float* logits, int B, int N, int k, int k0, float p, int oea,
                        int renorm, int32_t* idx, float* w, int32_t* n_base, uint32_t* mask,
                        int32_t* T, hipStream_t s);
hipError_t launch_route_dispatch(const float* logits, int B, int N, int k, int mode, int k0, float p, int max_p,
                                 int renorm, const int32_t* n_valid, const int32_t* k0_by_batch, int32_t* idx,
                                 float* w, int32_t* n_base,
                                 uint32_t* mask, int32_t* cnt, int32_t* offsets, int32_t* perm, int32_t* active,
                                 int32_t* T, int32_t* sync, hipStream_t s);
hipError_t launch_router_route_dispatch(const void* x, int x_dtype, const float* w_r, int B, int H, int N, int k,
                                        int mode, int k0, float p, int max_p, int renorm, const int32_t* n_valid,
                                        const int32_t* k0_by_batch, float* logits, int32_t* idx, float* w,
                                        int32_t* n_base, uint32_t* mask, int32_t* cnt, int32_t* offsets,
                                        int32_t* perm, int32_t* active, int32_t* T, int32_t* sync, hipStream_t s);
hipError_t launch_dispatch(const int32_t* idx, int B, int N, int k, int32_t* cnt,
                           int32_t* offsets, int32_t* perm, int32_t* active, int32_t* T,
                           hipStream_t s);
hipError_t launch_hotness_ema(float* S, const int32_t* cnt, int N, float alpha, hipStream_t s);
hipError_t launch_hotness_accumulate(int32_t* c, const int32_t* cnt, int N, hipStream_t s);
hipError_t launch_hotness_fold(float* S, int32_t* c, int N, float alpha, hipStream_t s);

// Error reporting shared by the C ABI sources: set the calling thread's
// message and return the status.
int fail(int status, const char* msg);
int hip_status(hipError_t e, const char* where);
const char* last_error();
hipError_t launch_handle_publish(moe_expert_handle* table, int e, moe_expert_handle h,
                                 hipStream_t s);
hipError_t launch_quantize_int4(const uint16_t* w, int rows, int cols, uint8_t* q,
                                uint16_t* scales, hipStream_t s);
hipError_t launch_pack_weights(int fmt, const void* src, const uint16_t* src_scales, int rows, int cols,
                               void* dst, uint16_t* dst_scales, hipStream_t s);

// Bytes of one weight row of `cols` input columns in format fmt.
__host__ __device__ inline int weight_row_bytes(int fmt, int cols) {
    return fmt == MOE_W_F32 ? cols * 4 : (fmt == MOE_W_BF16 ? cols * 2 : cols / 2);
}
// Input columns covered by one 64-byte tile row segment.
__host__ __device__ inline int tile_cols(int fmt) {
    return fmt == MOE_W_F32 ? 16 : (fmt == MOE_W_BF16 ? 32 : 128);
}

struct FfnArgs {
    const moe_expert_handle* table;
    int N, H, I, B, k;
    const void* x;
    int x_dtype;
    const int32_t* idx;
    const float* w;
    const int32_t* offsets;
    const int32_t* perm;
    const int32_t* active;
    const int32_t* T;
    float* y;
    float* hbuf;   // [B*k, I] fp32: SwiGLU activations per routed pair
    float* dbuf;   // [B*k, H] fp32: weighted down-projection per routed pair
};

size_t ffn_workspace_bytes(int B, int k, int H, int I);
bool ffn_cost_fits(int B, int k, int N, int H, int I);   // the device partition's 32-bit cost sums
// ev: null, or four events recorded on s before phase A, after phase A, after
// phase B and after the combine (null entries are skipped).
hipError_t launch_expert_ffn(const FfnArgs& a, void* ws, hipStream_t s, hipEvent_t const* ev = nullptr);
hipError_t ffn_noalloc_workspace(void** out);   // this device's static workspace
hipError_t launch_stream_read(const void* buf, size_t bytes, int waves_per_cu, uint32_t* out, int cus,
                              hipStream_t s);
int device_cus();   // compute units of the current device (cached per device)

}  // namespace moe
