// Packing of expert weight versions into the tiled, kernel-ready layout.
//
// Page "DynaExq", section 3.4: expert versions are prepacked once into the
// form the kernel consumes, so the forward path only follows a handle.  The
// expert FFN reads every matrix as tiles of 16 rows x 64 bytes: one wave's
// 16-byte load per lane covers a whole 1 KB tile, lane l = 16 q + m taking
// row m, bytes [16 q, 16 q + 16) of the tile's 64-byte row segment, which is
// the operand order of v_mfma_f32_16x16x32_bf16 (row = lane % 16, eight
// consecutive k per lane).  Tiles run along the row first: tile (rb, s) of
// a matrix with S = row_bytes / 64 tiles per row block sits at (rb S + s) KB.
//
// fp32 and bf16 rows are copied byte for byte.  INT4 rows (two nibbles per
// byte, even column low, as written by the quantiser) are re-ordered inside
// each lane's four dwords: dword j holds columns 8 j .. 8 j + 7 of the
// lane's 32, with column 2 i in nibble i and column 2 i + 1 in nibble i + 4,
// so (d >> 4 i) & 0x000F000F is the natural-order pair (2 i, 2 i + 1).
// INT4 scales [rows, cols/128] become [rows/16][cols/128][16]: the 16 row
// scales of one tile are contiguous.
#include "internal.h"

namespace moe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t nib(const uint32_t (&w)[4], int k) {   // k in [0, 32)
    return (w[k >> 3] >> ((k & 7) * 4)) & 0xFu;
}

// One thread per 16-byte chunk of the packed matrix.
__global__ __launch_bounds__(256) void pack_kernel(const char* __restrict__ src, int fmt, int rows,
                                                   int row_bytes, char* __restrict__ dst) {
    const long chunks = static_cast<long>(rows) * row_bytes / 16;
    const int S = row_bytes / 64;
    for (long c = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x; c < chunks;
         c += static_cast<long>(gridDim.x) * blockDim.x) {
        const long tile = c >> 6;
        const int lane = static_cast<int>(c & 63);
        const int m = lane & 15, q = lane >> 4;
        const long rb = tile / S;
        const int s = static_cast<int>(tile - rb * S);
        const char* p = src + (rb * 16 + m) * static_cast<long>(row_bytes) + s * 64 + q * 16;
        u32x4 v = *reinterpret_cast<const u32x4*>(p);
        if (fmt == MOE_W_INT4_G128) {
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
            uint32_t o[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                uint32_t d = 0;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    d |= nib(w, 8 * j + 2 * i) << (4 * i);
                    d |= nib(w, 8 * j + 2 * i + 1) << (4 * i + 16);
                }
                o[j] = d;
            }
            v = u32x4{o[0], o[1], o[2], o[3]};
        }
        *reinterpret_cast<u32x4*>(dst + c * 16) = v;
    }
}

// One thread per scale: [rows, groups] -> [rows/16][groups][16].
__global__ __launch_bounds__(256) void pack_scales_kernel(const uint16_t* __restrict__ src, int rows,
                                                          int groups, uint16_t* __restrict__ dst) {
    const long n = static_cast<long>(rows) * groups;
    for (long i = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
         i += static_cast<long>(gridDim.x) * blockDim.x) {
        const long r = i / groups;
        const int g = static_cast<int>(i - r * groups);
        dst[((r >> 4) * groups + g) * 16 + (r & 15)] = src[i];
    }
}

unsigned grid_for(long items) {
    const long b = (items + 255) / 256;
    return static_cast<unsigned>(b < 4096 ? (b > 0 ? b : 1) : 4096);
}

}  // namespace

hipError_t launch_pack_weights(int fmt, const void* src, const uint16_t* src_scales, int rows, int cols,
                               void* dst, uint16_t* dst_scales, hipStream_t s) {
    const int row_bytes = weight_row_bytes(fmt, cols);
    const long chunks = static_cast<long>(rows) * row_bytes / 16;
    pack_kernel<<<grid_for(chunks), 256, 0, s>>>(static_cast<const char*>(src), fmt, rows, row_bytes,
                                                 static_cast<char*>(dst));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || fmt != MOE_W_INT4_G128) return e;
    const int groups = cols / 128;
    pack_scales_kernel<<<grid_for(static_cast<long>(rows) * groups), 256, 0, s>>>(src_scales, rows, groups,
                                                                                   dst_scales);
    return hipGetLastError();
}

}  // namespace moe
