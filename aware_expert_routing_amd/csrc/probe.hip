// HBM read-stream reference: one pass over a buffer with the expert FFN's
// kind of load (16 bytes per lane, non-temporal), nothing else.  Its rate is
// the ceiling the weight-streaming kernels are compared against, measured on
// the same machine, beside the nominal HBM peak.
#include "internal.h"

namespace moe {
namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 8;   // 16-byte loads in flight per lane

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(1))) u32x4* gptr_u32x4;

// Each wave reads its own contiguous run of whole kilobytes (one 16-byte
// load per lane is one contiguous kilobyte per wave, as in the expert FFN's
// weight streaming), kProbeUnroll kilobytes in flight; the bytes past the last
// whole kilobyte go to wave 0.  The XOR of every 32-bit word is kept (so no
// load is dead) and folded into *out with an order-independent atomic, so the
// result is deterministic and checkable.
__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const u32x4* __restrict__ p, size_t n16,
                                                                     uint32_t* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const size_t waves = static_cast<size_t>(gridDim.x) * (kProbeThreads / 64);
    const size_t w = static_cast<size_t>(blockIdx.x) * (kProbeThreads / 64) + threadIdx.x / 64;
    const size_t n1k = n16 / 64;                  // whole kilobytes
    const size_t per = (n1k + waves - 1) / waves;
    size_t c = w * per;
    const size_t end = c + per < n1k ? c + per : n1k;
    uint32_t acc = 0u;
    for (; c + kProbeUnroll <= end; c += kProbeUnroll) {
        u32x4 v[kProbeUnroll];
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load((gptr_u32x4)(p + (c + u) * 64 + lane));
#pragma unroll
        for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; c < end; ++c) {
        const u32x4 v = __builtin_nontemporal_load((gptr_u32x4)(p + c * 64 + lane));
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (w == 0)
        for (size_t i = n1k * 64 + lane; i < n16; i += 64) {
            const u32x4 v = __builtin_nontemporal_load((gptr_u32x4)(p + i));
            acc ^= v.x ^ v.y ^ v.z ^ v.w;
        }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(acc), off, 64));
    if (lane == 0) atomicXor(out, acc);
}

}  // namespace

hipError_t launch_stream_read(const void* buf, size_t bytes, int waves_per_cu, uint32_t* out, int cus,
                              hipStream_t s) {
    const size_t n16 = bytes / 16;
    const int grid = (cus > 0 ? cus : 256) * waves_per_cu / (kProbeThreads / 64);
    stream_read_kernel<<<grid, kProbeThreads, 0, s>>>(static_cast<const u32x4*>(buf), n16, out);
    return hipGetLastError();
}

}  // namespace moe
