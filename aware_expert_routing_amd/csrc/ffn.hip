// Expert FFN (SwiGLU) and weighted combine for a decode batch.
//
// Page "Opportunistic Expert Activation (OEA) - L2", section 4 (Eq. 2 and
// check 4): in decode each activated expert costs a fixed weight fetch b
// plus a small per-token term a, and batched kernels must still load every
// activated expert's weights.  This file therefore streams each active
// expert's gate/up/down weights from HBM once per call, with all of the
// expert's tokens (up to 16 per pass) applied to every weight that is loaded.
// Page "DynaExq", section 2.2 / 3.2: each expert is reached through a handle
// giving the active version's pointers and quantisation parameters, resolved
// here per work item, so experts of one layer may be bf16, fp32 or INT4.
//
// Work decomposition (memory-bound GEMV, not a GEMM):
//   * phase A (gate/up + SwiGLU): items are (active expert, 16 rows of I);
//     a 256-thread workgroup takes a contiguous range of items; each wave
//     owns 4 rows, 16 lanes per row, and every lane reads 16 contiguous bytes
//     per chunk of 256 row bytes, so one wave instruction reads four 256-byte
//     row segments.  A lane handles the gate row and the up row of the same
//     index, so the SwiGLU product needs no exchange.
//   * phase B (down + routing weight): items are (active expert, 32 rows of
//     H); each lane handles two rows.
//   * combine: y[i] = sum over token i's filled slots, in slot order.
// Activations of the expert's tokens are staged once per item range in LDS
// in the weight format's layout (fp32 activations as bf16 hi/lo pairs); partial dot products are reduced across the
// 16 lanes of a row with DPP moves.  Arithmetic is fp32: bf16 pairs use
// v_dot2_f32_bf16, INT4 nibbles become bf16 (128 + nibble) pairs by bit
// operations and the offset is removed with a per-block activation sum.
#include "internal.h"

namespace moe {
namespace {

constexpr int kWave = 64;
constexpr int kLanesPerRow = 16;
constexpr int kRowsPerInstr = kWave / kLanesPerRow;   // 4
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;               // 4
constexpr int kChunkBytes = kLanesPerRow * 16;          // 256 row bytes per chunk
constexpr int kMaxTok = 16;                             // tokens per pass
constexpr int kMaxTokInt4 = 4;                          // INT4: fewer live registers
constexpr int kRowsA = kWaves * kRowsPerInstr;          // 16 rows of I per item
constexpr int kRowsPerLaneB = 2;
constexpr int kRowsB = kWaves * kRowsPerInstr * kRowsPerLaneB;   // 32 rows of H per item
constexpr int kLdsBytes = 64 * 1024;
constexpr int kChunkBlock = 4;                          // chunks in flight per row

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), c, false);
}

// Sum over the 16 lanes of a row group (DPP within a row of 16 lanes).
__device__ __forceinline__ float row16_sum(float v) {
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));  // quad [1,0,3,2]
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));  // quad [2,3,0,1]
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false)); // half-row mirror
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false)); // row mirror
    return v;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) {
    return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// Bytes of one staged activation row and of one weight row, per format.
// With `split`, an fp32 activation a is staged for bf16/INT4 weights as the
// pair hi = bf16(a), lo = bf16(a - hi) (two bf16 rows), so that products with
// bf16 weights keep about 16 significant bits of a; without it a is rounded to
// bf16 once (exact for bf16 inputs).
__host__ __device__ __forceinline__ int act_row_bytes(int fmt, int cols, bool split) {
    return fmt == MOE_W_F32 ? cols * 4 : cols * 2 * (split ? 2 : 1);
}
__host__ __device__ __forceinline__ int act_sum_bytes(int fmt, int cols) {
    return fmt == MOE_W_INT4_G128 ? (cols / 32) * 4 : 0;
}
__host__ __device__ __forceinline__ int weight_row_bytes(int fmt, int cols) {
    return fmt == MOE_W_F32 ? cols * 4 : (fmt == MOE_W_BF16 ? cols * 2 : cols / 2);
}
__host__ __device__ __forceinline__ int tokens_per_pass(int fmt, int cols, bool split) {
    int per = act_row_bytes(fmt, cols, split) + act_sum_bytes(fmt, cols);
    int t = (kLdsBytes - 256) / per;
    const int cap = fmt == MOE_W_INT4_G128 ? kMaxTokInt4 : kMaxTok;
    return t < cap ? t : cap;
}

// ---------------------------------------------------------------------------
// Staging: activations of `ct` pairs into LDS in the layout of format FMT.
//   F32 : fp32 row;  BF16 : bf16 row (RNE from fp32 sources);
//   INT4: bf16 row with each 8-column block stored as pairs (c, c+4), plus
//         the fp32 sum of every 32-column block.
// src_kind 0: x rows (x_dtype) indexed by token = pair / k; 1: fp32 hbuf rows
// indexed by pair.
// ---------------------------------------------------------------------------
struct StageSrc {
    const void* base;
    int dtype;      // MOE_DT_F32 or MOE_DT_BF16
    int by_token;   // 1: row = pair / k, 0: row = pair
    int k;
};

__device__ __forceinline__ void load8_as_f32(const StageSrc& src, int row, int cols, int c,
                                             float (&v)[8]) {
    if (src.dtype == MOE_DT_BF16) {
        const uint4 a = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(src.base) +
                                                        static_cast<size_t>(row) * cols + c);
        const uint32_t u[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            v[2 * q] = __uint_as_float(u[q] << 16);
            v[2 * q + 1] = __uint_as_float(u[q] & 0xffff0000u);
        }
    } else {
        const float* p = static_cast<const float*>(src.base) + static_cast<size_t>(row) * cols + c;
        const float4 a = *reinterpret_cast<const float4*>(p);
        const float4 b = *reinterpret_cast<const float4*>(p + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
}

__device__ void stage_rows(int fmt, bool split, const StageSrc& src, const int32_t* pairs_g, int ct,
                           int cols, char* lds, int* lds_pairs) {
    const int tid = threadIdx.x;
    if (tid < ct) lds_pairs[tid] = pairs_g[tid];
    const int arow = act_row_bytes(fmt, cols, split);
    const int half = cols * 2;   // byte offset of the lo row when split
    const int blocks = cols / 8;
    float* sums = reinterpret_cast<float*>(lds + ct * arow);
    for (int j = tid; j < ct * blocks; j += kThreads) {
        const int t = j / blocks, b = j - t * blocks;
        const int pair = pairs_g[t];
        const int row = src.by_token ? pair / src.k : pair;
        float v[8];
        load8_as_f32(src, row, cols, 8 * b, v);
        char* dst = lds + t * arow;
        if (fmt == MOE_W_F32) {
            float4* d = reinterpret_cast<float4*>(dst + b * 32);
            d[0] = make_float4(v[0], v[1], v[2], v[3]);
            d[1] = make_float4(v[4], v[5], v[6], v[7]);
            continue;
        }
        uint32_t h[8], l[8];
        float s = 0.0f;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            h[q] = f32_to_bf16_rne(v[q]);
            const float hv = __uint_as_float(h[q] << 16);
            l[q] = split ? f32_to_bf16_rne(v[q] - hv) : 0u;
            s += split ? hv + __uint_as_float(l[q] << 16) : hv;
        }
        // BF16 weights pair columns (c, c+1); INT4 weights pair (c, c+4).
        const bool by4 = fmt == MOE_W_INT4_G128;
        const uint4 oh = by4 ? make_uint4(h[0] | (h[4] << 16), h[1] | (h[5] << 16), h[2] | (h[6] << 16),
                                          h[3] | (h[7] << 16))
                             : make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                                          h[6] | (h[7] << 16));
        *reinterpret_cast<uint4*>(dst + b * 16) = oh;
        if (split) {
            const uint4 ol = by4 ? make_uint4(l[0] | (l[4] << 16), l[1] | (l[5] << 16), l[2] | (l[6] << 16),
                                              l[3] | (l[7] << 16))
                                 : make_uint4(l[0] | (l[1] << 16), l[2] | (l[3] << 16), l[4] | (l[5] << 16),
                                              l[6] | (l[7] << 16));
            *reinterpret_cast<uint4*>(dst + half + b * 16) = ol;
        }
        if (by4) {
            // sum over a 32-column block: lanes j..j+3 hold its four 8-column blocks
            s += __shfl_xor(s, 1, kWave);
            s += __shfl_xor(s, 2, kWave);
            if ((b & 3) == 0) sums[t * (cols / 32) + b / 4] = s;
        }
    }
}

// ---------------------------------------------------------------------------
// Core: NR weight rows per lane against MT staged activation rows.
// Lane `g` (0..15 within its row group) reads 16 bytes at byte offset
// 256*c + 16*g of every row, for chunks c = 0 .. nchunks-1.
// ---------------------------------------------------------------------------
template <int FMT, bool SPLIT, int NR, int MT>
__device__ __forceinline__ void chunk_fma(const u32x4 (&wv)[NR], int c, int g, int ct,
                                          const char* lds, int arow, int half, const float* sums,
                                          int cols, const float (&scale)[NR], float (&acc)[NR][MT]) {
    const int off = c * kChunkBytes + g * 16;   // weight byte offset in the row
    if constexpr (FMT == MOE_W_F32) {
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            if (t < ct) {
                const uint4 xv = *reinterpret_cast<const uint4*>(lds + t * arow + off);
#pragma unroll
                for (int r = 0; r < NR; ++r) {
                    float a = acc[r][t];
                    a = __builtin_fmaf(__uint_as_float(wv[r].x), __uint_as_float(xv.x), a);
                    a = __builtin_fmaf(__uint_as_float(wv[r].y), __uint_as_float(xv.y), a);
                    a = __builtin_fmaf(__uint_as_float(wv[r].z), __uint_as_float(xv.z), a);
                    a = __builtin_fmaf(__uint_as_float(wv[r].w), __uint_as_float(xv.w), a);
                    acc[r][t] = a;
                }
            }
        }
    } else if constexpr (FMT == MOE_W_BF16) {
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            if (t < ct) {
                const uint4 xv = *reinterpret_cast<const uint4*>(lds + t * arow + off);
                uint4 xl = make_uint4(0u, 0u, 0u, 0u);
                if constexpr (SPLIT) xl = *reinterpret_cast<const uint4*>(lds + t * arow + half + off);
#pragma unroll
                for (int r = 0; r < NR; ++r) {
                    float a = acc[r][t];
                    a = dot2_bf16(wv[r].x, xv.x, a);
                    a = dot2_bf16(wv[r].y, xv.y, a);
                    a = dot2_bf16(wv[r].z, xv.z, a);
                    a = dot2_bf16(wv[r].w, xv.w, a);
                    if constexpr (SPLIT) {
                        a = dot2_bf16(wv[r].x, xl.x, a);
                        a = dot2_bf16(wv[r].y, xl.y, a);
                        a = dot2_bf16(wv[r].z, xl.z, a);
                        a = dot2_bf16(wv[r].w, xl.w, a);
                    }
                    acc[r][t] = a;
                }
            }
        }
    } else {
        // INT4: 32 weights (columns col0 .. col0+31, one 128-group) per lane.
        // Each 32-bit word holds 8 nibbles; (w >> 4s) & 0x000f000f | 0x43004300
        // is the bf16 pair (128 + u_s, 128 + u_{s+4}), matching the staged
        // activation pairs (c, c+4).
        const int col0 = off * 2;
        uint32_t pk[NR][16];
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    pk[r][4 * q + s] = ((wv[r][q] >> (4 * s)) & 0x000f000fu) | 0x43004300u;
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            if (t < ct) {
                const char* xr = lds + t * arow + col0 * 2;
                float d[NR];
#pragma unroll
                for (int r = 0; r < NR; ++r) d[r] = 0.0f;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint4 xv = *reinterpret_cast<const uint4*>(xr + 16 * q);
#pragma unroll
                    for (int r = 0; r < NR; ++r) {
                        d[r] = dot2_bf16(pk[r][4 * q + 0], xv.x, d[r]);
                        d[r] = dot2_bf16(pk[r][4 * q + 1], xv.y, d[r]);
                        d[r] = dot2_bf16(pk[r][4 * q + 2], xv.z, d[r]);
                        d[r] = dot2_bf16(pk[r][4 * q + 3], xv.w, d[r]);
                    }
                    if constexpr (SPLIT) {
                        const uint4 xl = *reinterpret_cast<const uint4*>(xr + half + 16 * q);
#pragma unroll
                        for (int r = 0; r < NR; ++r) {
                            d[r] = dot2_bf16(pk[r][4 * q + 0], xl.x, d[r]);
                            d[r] = dot2_bf16(pk[r][4 * q + 1], xl.y, d[r]);
                            d[r] = dot2_bf16(pk[r][4 * q + 2], xl.z, d[r]);
                            d[r] = dot2_bf16(pk[r][4 * q + 3], xl.w, d[r]);
                        }
                    }
                }
                const float xs = sums[t * (cols / 32) + col0 / 32];
#pragma unroll
                for (int r = 0; r < NR; ++r)   // sum (128 + u) x - 136 sum x = sum (u - 8) x
                    acc[r][t] = __builtin_fmaf(scale[r], __builtin_fmaf(-136.0f, xs, d[r]), acc[r][t]);
                // keep the scheduler from hoisting every token's LDS reads at once
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
}

template <int FMT, bool SPLIT, int NR, int MT>
__device__ __forceinline__ void rows_dot(const char* const (&rowp)[NR], const uint16_t* const (&srow)[NR],
                                         bool row_ok, int rbytes, int cols, int g, int ct,
                                         const char* lds, float (&acc)[NR][MT]) {
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[r][t] = 0.0f;
    if (!row_ok) return;
    const int arow = act_row_bytes(FMT, cols, SPLIT);
    const int half = cols * 2;
    const float* sums = reinterpret_cast<const float*>(lds + ct * arow);
    const int nchunks = (rbytes + kChunkBytes - 1) / kChunkBytes;
    // an INT4 chunk carries 32 weights per lane (a bf16 chunk 8): fewer per block
    constexpr int CB = FMT == MOE_W_INT4_G128 ? 1 : kChunkBlock;
    for (int c0 = 0; c0 < nchunks; c0 += CB) {
        u32x4 wv[CB][NR];
        float sc[CB][NR];
#pragma unroll
        for (int b = 0; b < CB; ++b) {
            const int off = (c0 + b) * kChunkBytes + g * 16;
            const bool ok = (c0 + b) < nchunks && off < rbytes;
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                wv[b][r] = ok ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(rowp[r] + off))
                              : u32x4{0u, 0u, 0u, 0u};
                if constexpr (FMT == MOE_W_INT4_G128)
                    sc[b][r] = ok ? f16_bits_to_f32(srow[r][(off * 2) / 128]) : 0.0f;
                else
                    sc[b][r] = 1.0f;
            }
        }
#pragma unroll
        for (int b = 0; b < CB; ++b) {
            const int off = (c0 + b) * kChunkBytes + g * 16;
            if ((c0 + b) < nchunks && off < rbytes)
                chunk_fma<FMT, SPLIT, NR, MT>(wv[b], c0 + b, g, ct, lds, arow, half, sums, cols, sc[b], acc);
        }
    }
}

// ---------------------------------------------------------------------------
// Phase A: gate/up rows and SwiGLU.
// ---------------------------------------------------------------------------
template <int FMT, bool SPLIT, int MT>
__device__ void gateup_item(const FfnArgs& a, const moe_expert_handle& h, int row0, int ct,
                            const char* lds, const int* lds_pairs) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int g = lane & (kLanesPerRow - 1);
    const int row = row0 + wave * kRowsPerInstr + lane / kLanesPerRow;
    const bool row_ok = row < a.I;
    const int rbytes = weight_row_bytes(FMT, a.H);
    const int rr = row_ok ? row : 0;
    const char* rowp[2] = {static_cast<const char*>(h.w_gate) + static_cast<size_t>(rr) * rbytes,
                           static_cast<const char*>(h.w_up) + static_cast<size_t>(rr) * rbytes};
    const uint16_t* srow[2] = {nullptr, nullptr};
    if constexpr (FMT == MOE_W_INT4_G128) {
        srow[0] = h.s_gate + static_cast<size_t>(rr) * (a.H / 128);
        srow[1] = h.s_up + static_cast<size_t>(rr) * (a.H / 128);
    }
    float acc[2][MT];
    rows_dot<FMT, SPLIT, 2, MT>(rowp, srow, row_ok, rbytes, a.H, g, ct, lds, acc);
    float mine_g = 0.0f, mine_u = 0.0f;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        const float sg = row16_sum(acc[0][t]);
        const float su = row16_sum(acc[1][t]);
        if (g == t) { mine_g = sg; mine_u = su; }
    }
    if (row_ok && g < ct) a.hbuf[static_cast<size_t>(lds_pairs[g]) * a.I + row] = silu(mine_g) * mine_u;
}

// ---------------------------------------------------------------------------
// Phase B: down rows, scaled by the pair's routing weight.
// ---------------------------------------------------------------------------
template <int FMT, bool SPLIT, int MT>
__device__ void down_item(const FfnArgs& a, const moe_expert_handle& h, int row0, int ct,
                          const char* lds, const int* lds_pairs) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int g = lane & (kLanesPerRow - 1);
    const int rbytes = weight_row_bytes(FMT, a.I);
    const int base = row0 + wave * (kRowsPerInstr * kRowsPerLaneB) + lane / kLanesPerRow;
    const bool row_ok = base < a.H;   // rows base, base+4 share validity when H % 8 == 0
    const char* rowp[kRowsPerLaneB];
    const uint16_t* srow[kRowsPerLaneB];
#pragma unroll
    for (int r = 0; r < kRowsPerLaneB; ++r) {
        const int row = row_ok ? base + r * kRowsPerInstr : 0;
        rowp[r] = static_cast<const char*>(h.w_down) + static_cast<size_t>(row) * rbytes;
        srow[r] = (FMT == MOE_W_INT4_G128) ? h.s_down + static_cast<size_t>(row) * (a.I / 128) : nullptr;
    }
    float acc[kRowsPerLaneB][MT];
    rows_dot<FMT, SPLIT, kRowsPerLaneB, MT>(rowp, srow, row_ok, rbytes, a.I, g, ct, lds, acc);
#pragma unroll
    for (int r = 0; r < kRowsPerLaneB; ++r) {
        float mine = 0.0f;
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            const float s = row16_sum(acc[r][t]);
            if (g == t) mine = s;
        }
        if (row_ok && g < ct) {
            const int pair = lds_pairs[g];
            a.dbuf[static_cast<size_t>(pair) * a.H + base + r * kRowsPerInstr] = a.w[pair] * mine;
        }
    }
}

template <int FMT, bool SPLIT, int PHASE>
__device__ __forceinline__ void run_item(const FfnArgs& a, const moe_expert_handle& h, int row0,
                                         int ct, const char* lds, const int* lds_pairs) {
#define MOE_ITEM_CASE(MTV)                                                              \
    if (ct <= MTV) {                                                                    \
        if constexpr (PHASE == 0) gateup_item<FMT, SPLIT, MTV>(a, h, row0, ct, lds, lds_pairs); \
        else down_item<FMT, SPLIT, MTV>(a, h, row0, ct, lds, lds_pairs);                \
        return;                                                                         \
    }
    MOE_ITEM_CASE(1)
    MOE_ITEM_CASE(2)
    MOE_ITEM_CASE(4)
    if constexpr (FMT != MOE_W_INT4_G128) {
        MOE_ITEM_CASE(8)
        MOE_ITEM_CASE(16)
    }
#undef MOE_ITEM_CASE
}

// Persistent workgroups; workgroup b takes items [b*total/G, (b+1)*total/G).
template <int PHASE>
__global__ __launch_bounds__(kThreads, 2) void ffn_kernel(FfnArgs a) {
    extern __shared__ __attribute__((aligned(16))) char lds_raw[];
    int* lds_pairs = reinterpret_cast<int*>(lds_raw + kLdsBytes - 64);
    const int T = *a.T;
    const int rows = PHASE == 0 ? a.I : a.H;
    const int cols = PHASE == 0 ? a.H : a.I;
    const int rows_per_item = PHASE == 0 ? kRowsA : kRowsB;
    const int tiles = (rows + rows_per_item - 1) / rows_per_item;
    const long total = static_cast<long>(T) * tiles;
    const long begin = total * blockIdx.x / gridDim.x;
    const long end = total * (blockIdx.x + 1) / gridDim.x;
    int staged_slot = -1, staged_t0 = -1;
    for (long it = begin; it < end; ++it) {
        const int slot = static_cast<int>(it / tiles);
        const int tile = static_cast<int>(it - static_cast<long>(slot) * tiles);
        const int e = a.active[slot];
        const moe_expert_handle h = a.table[e];
        const int first = a.offsets[e];
        const int cnt = a.offsets[e + 1] - first;
        // fp32 activations meet bf16/INT4 weights as hi/lo bf16 pairs
        const bool split = h.fmt != MOE_W_F32 && (PHASE == 1 || a.x_dtype == MOE_DT_F32);
        const int per_pass = tokens_per_pass(h.fmt, cols, split);
        for (int t0 = 0; t0 < cnt; t0 += per_pass) {
            const int ct = min(per_pass, cnt - t0);
            if (slot != staged_slot || t0 != staged_t0) {
                __syncthreads();
                StageSrc src;
                if (PHASE == 0) src = StageSrc{a.x, a.x_dtype, 1, a.k};
                else src = StageSrc{a.hbuf, MOE_DT_F32, 0, a.k};
                stage_rows(h.fmt, split, src, a.perm + first + t0, ct, cols, lds_raw, lds_pairs);
                __syncthreads();
                staged_slot = slot;
                staged_t0 = t0;
            }
            const int row0 = tile * rows_per_item;
            if (h.fmt == MOE_W_BF16) {
                if (split) run_item<MOE_W_BF16, true, PHASE>(a, h, row0, ct, lds_raw, lds_pairs);
                else run_item<MOE_W_BF16, false, PHASE>(a, h, row0, ct, lds_raw, lds_pairs);
            } else if (h.fmt == MOE_W_INT4_G128) {
                if (split) run_item<MOE_W_INT4_G128, true, PHASE>(a, h, row0, ct, lds_raw, lds_pairs);
                else run_item<MOE_W_INT4_G128, false, PHASE>(a, h, row0, ct, lds_raw, lds_pairs);
            } else {
                run_item<MOE_W_F32, false, PHASE>(a, h, row0, ct, lds_raw, lds_pairs);
            }
        }
    }
}

// y[i, o] = sum over filled slots s of token i (slot order) of dbuf[i*k+s, o].
__global__ __launch_bounds__(256) void combine_kernel(FfnArgs a) {
    const int i = blockIdx.y;
    const int o = (blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (o >= a.H) return;
    float4 s = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    for (int q = 0; q < a.k; ++q) {
        if (a.idx[i * a.k + q] < 0) continue;
        const float4 d = *reinterpret_cast<const float4*>(a.dbuf + static_cast<size_t>(i * a.k + q) * a.H + o);
        s.x += d.x; s.y += d.y; s.z += d.z; s.w += d.w;
    }
    *reinterpret_cast<float4*>(a.y + static_cast<size_t>(i) * a.H + o) = s;
}

int g_num_cus[64] = {0};

int device_cus() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (g_num_cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        g_num_cus[dev] = n;
    }
    return g_num_cus[dev];
}

}  // namespace

size_t ffn_workspace_bytes(int B, int k, int H, int I) {
    const size_t pairs = static_cast<size_t>(B) * k;
    size_t hb = (pairs * I * sizeof(float) + 255) & ~size_t(255);
    size_t db = (pairs * H * sizeof(float) + 255) & ~size_t(255);
    return hb + db;
}

hipError_t launch_expert_ffn(const FfnArgs& in, void* ws, hipStream_t s) {
    FfnArgs a = in;
    const size_t pairs = static_cast<size_t>(a.B) * a.k;
    char* p = static_cast<char*>(ws);
    a.hbuf = reinterpret_cast<float*>(p);
    a.dbuf = reinterpret_cast<float*>(p + ((pairs * a.I * sizeof(float) + 255) & ~size_t(255)));
    const int G = 2 * device_cus();
    ffn_kernel<0><<<G, kThreads, kLdsBytes, s>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    ffn_kernel<1><<<G, kThreads, kLdsBytes, s>>>(a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    dim3 cg((a.H / 4 + 255) / 256, a.B);
    combine_kernel<<<cg, 256, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace moe
