// INT4 group-128 low-precision expert versions.
//
// Page "DynaExq", section 3.2 (each expert keeps a high- and a low-precision
// version, INT4 for cold experts) and section 3.4 (versions are prepacked in
// kernel-ready form).  Format: per row and group of 128 input columns,
// s = fp16(absmax / 7), q = clamp(rint(w / s), -8, 7), stored as the unsigned
// nibble q + 8, two per byte with the even column in the low nibble.
// Quotients are IEEE fp32 divisions (correctly rounded), conversions round to
// nearest even, and contraction is off, so the packed bytes are exact.
#pragma clang fp contract(off)

#include "internal.h"

namespace moe {
namespace {

constexpr int kWave = 64;

// One wavefront per (row, group): lane l owns columns 2l and 2l+1.
__global__ __launch_bounds__(256) void quantize_int4_kernel(const uint16_t* __restrict__ w,
                                                            int rows, int cols,
                                                            uint8_t* __restrict__ q,
                                                            uint16_t* __restrict__ scales) {
    const int groups = cols / 128;
    const int lane = threadIdx.x & (kWave - 1);
    const long wid = static_cast<long>(blockIdx.x) * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (wid >= static_cast<long>(rows) * groups) return;
    const int r = static_cast<int>(wid / groups);
    const int g = static_cast<int>(wid - static_cast<long>(r) * groups);
    const size_t at = static_cast<size_t>(r) * cols + g * 128 + 2 * lane;
    const uint32_t pairbits = *reinterpret_cast<const uint32_t*>(w + at);
    const float v0 = __uint_as_float(pairbits << 16);
    const float v1 = __uint_as_float(pairbits & 0xffff0000u);
    float amax = fmaxf(fabsf(v0), fabsf(v1));
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, kWave));
    const _Float16 sh = static_cast<_Float16>(amax / 7.0f);
    const float s = static_cast<float>(sh);
    int q0 = 0, q1 = 0;
    if (s != 0.0f) {
        q0 = static_cast<int>(fminf(fmaxf(__builtin_rintf(v0 / s), -8.0f), 7.0f));
        q1 = static_cast<int>(fminf(fmaxf(__builtin_rintf(v1 / s), -8.0f), 7.0f));
    }
    q[at / 2] = static_cast<uint8_t>((q0 + 8) | ((q1 + 8) << 4));
    if (lane == 0) scales[static_cast<size_t>(r) * groups + g] = __builtin_bit_cast(uint16_t, sh);
}

}  // namespace

hipError_t launch_quantize_int4(const uint16_t* w, int rows, int cols, uint8_t* q,
                                uint16_t* scales, hipStream_t s) {
    const long waves = static_cast<long>(rows) * (cols / 128);
    const long blocks = (waves + 3) / 4;
    quantize_int4_kernel<<<static_cast<unsigned>(blocks), 256, 0, s>>>(w, rows, cols, q, scales);
    return hipGetLastError();
}

}  // namespace moe
