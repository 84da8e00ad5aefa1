// Expert FFN (SwiGLU) and weighted combine for a decode batch.
//
// Page "Opportunistic Expert Activation (OEA) - L2", section 4 (Eq. 2 and
// check 4): in decode each activated expert costs a fixed weight fetch b
// plus a small per-token term a, and batched kernels must still load every
// activated expert's weights.  This file streams each active expert's
// gate/up/down weights from HBM once per call (per pass of up to 8 of the
// expert's tokens) and applies every token of the pass to each loaded weight.
// Page "DynaExq", section 2.2 / 3.2: each expert is reached through a handle
// giving the active version's pointers and quantisation parameters, resolved
// per work item, so one layer may mix bf16, fp32 and INT4 experts.
//
// Work decomposition (a memory-bound GEMV, not a GEMM):
//   * phase A (gate/up + SwiGLU): work items are (active expert, 16 rows of
//     I); a lane owns the gate row and the up row of the same index, so the
//     SwiGLU product needs no exchange.  16 lanes share a row: lane g reads
//     bytes [256c + 16g, 256c + 16g + 16) of the row for chunks c, so one
//     wave instruction reads four 256-byte row segments.
//   * phase B (down + routing weight): items are (active expert, 32 rows of
//     H); a lane owns two rows.
//   * combine: y[i] = sum over token i's filled slots, in slot order.
// Each 256-thread workgroup takes a contiguous range of items of about equal
// streaming cost (every workgroup first prices the active experts).  A wave keeps
// the weight loads of its next block of chunks in flight while it computes
// the current block, and at the end of an item it has already issued the
// loads of the next item's first block, so the weight stream does not stop
// at item boundaries.  Activations of the pass's tokens are staged in LDS in
// the weight format's layout (fp32 activations as bf16 hi/lo pairs for
// bf16/INT4 weights); partial sums are reduced across the 16 lanes of a row
// with DPP moves.  bf16 products use v_dot2_f32_bf16; INT4 nibbles become the
// bf16 pair (128 + u, 128 + u') by bit operations, and the offset is removed
// with the staged sum of the activations of each 32-column block.
#include "internal.h"

namespace moe {
namespace {

constexpr int kWave = 64;
constexpr int kLanesPerRow = 16;
constexpr int kRowsPerInstr = kWave / kLanesPerRow;   // 4
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;               // 4
constexpr int kChunkBytes = kLanesPerRow * 16;          // 256 row bytes per chunk
constexpr int kMaxTok = 8;                              // tokens per pass
constexpr int kMaxTokInt4 = 2;                          // INT4: fewer live registers
constexpr int kLdsBytes = 56 * 1024;   // staged activations (dynamic LDS; static LDS adds ~6.7 KB)

// phase A: 2 rows per lane (gate, up), 16 rows per item, 4 chunks per block
constexpr int kNrA = 2, kRowsA = kWaves * kRowsPerInstr, kCbA = 4;
// phase B: 2 rows per lane, 32 rows per item, 3 chunks per block
constexpr int kNrB = 2, kRowsB = kWaves * kRowsPerInstr * kNrB, kCbB = 3;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(1))) u32x4* gptr_u32x4;

// 16-byte streaming load through the global (not flat) address space.
__device__ __forceinline__ u32x4 load_nt16(const char* p) {
    return __builtin_nontemporal_load((gptr_u32x4)(p));
}

// Values that are equal across the wavefront, moved to scalar registers so
// tests on them become scalar branches.
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), c, false);
}

// Sum over the 16 lanes of a row group (DPP within each row of 16 lanes).
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
// pair hi = bf16(a), lo = bf16(a - hi) (two bf16 rows), so products with bf16
// weights keep about 16 significant bits of a; without it a is rounded to
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
    const int per = act_row_bytes(fmt, cols, split) + act_sum_bytes(fmt, cols);
    const int t = kLdsBytes / per;
    const int cap = fmt == MOE_W_INT4_G128 ? kMaxTokInt4 : kMaxTok;
    return t < cap ? t : cap;
}

// ---------------------------------------------------------------------------
// Staging of one pass's activations into LDS.
//   F32 : fp32 row;  BF16 : bf16 row (pairs (c, c+1));
//   INT4: bf16 row with each 8-column block stored as pairs (c, c+4), plus
//         the fp32 sum of every 32-column block (after the rows).
// Phase A reads x rows (x_dtype) of token pair / k; phase B reads fp32 rows
// of the SwiGLU buffer indexed by pair.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void load8_as_f32(const void* base, int dtype, int row, int cols, int c,
                                             float (&v)[8]) {
    if (dtype == MOE_DT_BF16) {
        const uint4 a = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) +
                                                        static_cast<size_t>(row) * cols + c);
        const uint32_t u[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            v[2 * q] = __uint_as_float(u[q] << 16);
            v[2 * q + 1] = __uint_as_float(u[q] & 0xffff0000u);
        }
    } else {
        const float* p = static_cast<const float*>(base) + static_cast<size_t>(row) * cols + c;
        const float4 a = *reinterpret_cast<const float4*>(p);
        const float4 b = *reinterpret_cast<const float4*>(p + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
}

__device__ void stage_rows(int fmt, bool split, const void* base, int dtype, int by_token_k,
                           const int32_t* pairs_g, int ct, int cols, char* lds, const float* wts_g,
                           int* lds_pair, float* lds_wt) {
    const int tid = threadIdx.x;
    if (tid < ct) {
        const int pr = pairs_g[tid];
        lds_pair[tid] = pr;
        lds_wt[tid] = wts_g[pr];
    }
    const int arow = act_row_bytes(fmt, cols, split);
    const int half = cols * 2;   // byte offset of the lo row when split
    const int blocks = cols / 8;
    float* sums = reinterpret_cast<float*>(lds + ct * arow);
    for (int j = tid; j < ct * blocks; j += kThreads) {
        const int t = j / blocks, b = j - t * blocks;
        const int pair = pairs_g[t];
        const int row = by_token_k > 0 ? pair / by_token_k : pair;
        float v[8];
        load8_as_f32(base, dtype, row, cols, 8 * b, v);
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
            // a 32-column block is held by lanes j..j+3 (cols % 128 == 0)
            s += __shfl_xor(s, 1, kWave);
            s += __shfl_xor(s, 2, kWave);
            if ((b & 3) == 0) sums[t * (cols / 32) + b / 4] = s;
        }
    }
}

// ---------------------------------------------------------------------------
// Cost-balanced partition.  Each workgroup first prices every active expert
// (one thread per active slot, records kept in LDS): the cost of a row tile
// is the sum over the expert's token passes of (16 + tokens), since for the
// same weight bytes a pass of 8 tokens takes about 1.4x a pass of one
// (measured) and every extra pass streams the tile again.  Workgroup b then
// takes the items whose cost ranges start in [b*C/G, (b+1)*C/G) of the total
// cost C, so experts with many tokens are spread over more workgroups.
// ---------------------------------------------------------------------------
struct SlotRec {                  // one phase's view of an active expert
    const char* m0;               // phase A: gate, phase B: down
    const char* m1;               // phase A: up
    const uint16_t* s0;           // INT4 scales (or null)
    const uint16_t* s1;
    int32_t fmt, first, cnt, pad;
};

__device__ __forceinline__ int tile_cost(int cnt, int per_pass) {
    int c = 0;
    for (int t0 = 0; t0 < cnt; t0 += per_pass) c += 16 + min(per_pass, cnt - t0);
    return c;
}

// ---------------------------------------------------------------------------
// One unit of work of a workgroup: an item (active expert, row tile) and one
// pass of that expert's tokens.  All fields are wave-uniform.
// ---------------------------------------------------------------------------
struct Unit {
    int slot, tile, t0, ct;   // active slot, row tile, first token of the pass, tokens in it
    int fmt;
    bool split;
    int first;                // first routed pair of the expert in perm
    const char* m0;           // phase A: gate, phase B: down
    const char* m1;           // phase A: up
    const uint16_t* s0;
    const uint16_t* s1;
};

template <int PHASE>
__device__ __forceinline__ Unit make_unit(const SlotRec* recs, int x_dtype, long item, int t0, int tiles,
                                          int cols, int& cnt) {
    Unit u;
    u.slot = uni(static_cast<int>(item / tiles));
    u.tile = uni(static_cast<int>(item - static_cast<long>(u.slot) * tiles));
    const SlotRec& r = recs[u.slot];
    u.fmt = uni(r.fmt);
    u.split = u.fmt != MOE_W_F32 && (PHASE == 1 || x_dtype == MOE_DT_F32);
    u.first = uni(r.first);
    cnt = uni(r.cnt);
    const int per_pass = tokens_per_pass(u.fmt, cols, u.split);
    u.t0 = uni(t0);
    u.ct = uni(min(per_pass, cnt - t0));
    u.m0 = r.m0;
    u.m1 = r.m1;
    u.s0 = r.s0;
    u.s1 = r.s1;
    return u;
}

// Per-lane row addresses of a unit: phase A -> (gate r, up r); phase B ->
// rows base + 4j of the down matrix.  Rows at or beyond `rows` are clamped to
// row 0 so every load stays inside the matrix; their results are not stored.
template <int NR>
struct Rows {
    const char* p[NR];
    const uint16_t* s[NR];
    int id[NR];
    int rbytes;     // bytes per weight row
    int nchunks;    // 256-byte chunks per row (the last may be partial)
};

template <int PHASE, int NR>
__device__ __forceinline__ Rows<NR> unit_rows(const Unit& u, int rows, int cols) {
    Rows<NR> R;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    R.rbytes = uni(weight_row_bytes(u.fmt, cols));
    R.nchunks = uni((R.rbytes + kChunkBytes - 1) / kChunkBytes);
    const int sgroups = cols / 128;
    if constexpr (PHASE == 0) {
        const int row = u.tile * kRowsA + wave * kRowsPerInstr + lane / kLanesPerRow;
        const int rr = row < rows ? row : 0;
        R.p[0] = u.m0 + static_cast<size_t>(rr) * R.rbytes;
        R.p[1] = u.m1 + static_cast<size_t>(rr) * R.rbytes;
        R.s[0] = u.s0 + static_cast<size_t>(rr) * sgroups;
        R.s[1] = u.s1 + static_cast<size_t>(rr) * sgroups;
        R.id[0] = R.id[1] = row;
    } else {
        const int base = u.tile * kRowsB + wave * (kRowsPerInstr * NR) + lane / kLanesPerRow;
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            const int row = base + r * kRowsPerInstr;
            const int rr = row < rows ? row : 0;
            R.p[r] = u.m0 + static_cast<size_t>(rr) * R.rbytes;
            R.s[r] = u.s0 + static_cast<size_t>(rr) * sgroups;
            R.id[r] = row;
        }
    }
    return R;
}

// Weight block: CB chunks of NR rows, raw 16-byte loads.
template <int NR, int CB>
struct Block {
    u32x4 w[CB][NR];
};

// Issue the loads of block `blk`, unconditionally: offsets are clamped to the
// row's last 16 bytes, so chunks past the row (skipped when computing) and the
// lanes past the end of a partial chunk (masked when computing) re-read bytes
// of the same row instead of branching around the load.
template <int NR, int CB>
__device__ __forceinline__ void load_block(const Rows<NR>& R, int blk, Block<NR, CB>& b) {
    const int g = threadIdx.x & (kLanesPerRow - 1);
#pragma unroll
    for (int c = 0; c < CB; ++c) {
        const int off = min((blk * CB + c) * kChunkBytes + g * 16, R.rbytes - 16);
#pragma unroll
        for (int r = 0; r < NR; ++r) b.w[c][r] = load_nt16(R.p[r] + off);
    }
}

// Multiply-accumulate one chunk of NR rows against the pass's MT tokens.
template <int FMT, bool SPLIT, int NR, int MT>
__device__ __forceinline__ void chunk_fma(const u32x4 (&wv)[NR], const float (&scale)[NR], int off,
                                          int ct, const char* lds, int arow, int half,
                                          const float* sums, int cols, float (&acc)[NR][MT]) {
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
        // INT4: 32 weights (columns col0 .. col0+31 of one 128-group) per lane.
        // (w >> 4s) & 0x000f000f | 0x43004300 is the bf16 pair (128 + u_s,
        // 128 + u_{s+4}) of the word's nibbles, matching the staged pairs (c, c+4).
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
                __builtin_amdgcn_sched_barrier(0);   // one token's LDS reads at a time
            }
        }
    }
}

// Run one unit: blocks 0..nblk-1 with the next block's loads in flight while
// the current one is computed; the last block issues the loads of the next
// unit's first block into `pre`.  Then reduce across the 16 lanes of each row
// and write the results.
template <int PHASE, int FMT, bool SPLIT, int NR, int CB, int MT>
__device__ __forceinline__ void run_unit(const FfnArgs& a, const Unit& u, const Rows<NR>& R,
                                         const Rows<NR>& NRws, bool has_next, int rows, int cols,
                                         const char* lds, const int* lds_pair, const float* lds_wt,
                                         Block<NR, CB>& pre) {
    const int g = threadIdx.x & (kLanesPerRow - 1);
    const int nblk = (R.nchunks + CB - 1) / CB;
    const int arow = act_row_bytes(FMT, cols, SPLIT);
    const int half = cols * 2;
    const float* sums = reinterpret_cast<const float*>(lds + u.ct * arow);
    const bool partial = (R.rbytes % kChunkBytes) != 0;
    float acc[NR][MT];
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int t = 0; t < MT; ++t) acc[r][t] = 0.0f;
    // the block after the unit's last one: the next unit's first, or (at the
    // end of the range) a harmless re-read of this unit's first block
    const Rows<NR>& after = has_next ? NRws : R;
    for (int blk = 0; blk < nblk; ++blk) {
        Block<NR, CB> cur = pre;
        if (blk + 1 < nblk) load_block<NR, CB>(R, blk + 1, pre);
        else load_block<NR, CB>(after, 0, pre);
#pragma unroll
        for (int c = 0; c < CB; ++c) {
            const int chunk = blk * CB + c;
            if (chunk >= R.nchunks) break;
            const int off_raw = chunk * kChunkBytes + g * 16;
            const bool lane_ok = off_raw < R.rbytes;
            const int off = min(off_raw, R.rbytes - 16);
            float sc[NR];
#pragma unroll
            for (int r = 0; r < NR; ++r) {
                sc[r] = 1.0f;
                if constexpr (FMT == MOE_W_INT4_G128) sc[r] = f16_bits_to_f32(R.s[r][(off * 2) / 128]);
            }
            u32x4 w[NR];
#pragma unroll
            for (int r = 0; r < NR; ++r) w[r] = cur.w[c][r];
            if (partial && chunk == R.nchunks - 1) {   // wave-uniform test
#pragma unroll
                for (int r = 0; r < NR; ++r) {
                    if constexpr (FMT == MOE_W_INT4_G128) sc[r] = lane_ok ? sc[r] : 0.0f;
                    else w[r] = lane_ok ? w[r] : u32x4{0u, 0u, 0u, 0u};
                }
            }
            chunk_fma<FMT, SPLIT, NR, MT>(w, sc, off, u.ct, lds, arow, half, sums, cols, acc);
        }
    }
    const bool writer = g < u.ct;
    const int pair = writer ? lds_pair[g] : 0;
    if constexpr (PHASE == 0) {
        float mg = 0.0f, mu = 0.0f;
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            const float sg = row16_sum(acc[0][t]);
            const float su = row16_sum(acc[1][t]);
            if (g == t) { mg = sg; mu = su; }
        }
        if (writer && R.id[0] < rows) a.hbuf[static_cast<size_t>(pair) * a.I + R.id[0]] = silu(mg) * mu;
    } else {
        const float wgt = writer ? lds_wt[g] : 0.0f;
#pragma unroll
        for (int r = 0; r < NR; ++r) {
            float mine = 0.0f;
#pragma unroll
            for (int t = 0; t < MT; ++t) {
                const float s = row16_sum(acc[r][t]);
                if (g == t) mine = s;
            }
            if (writer && R.id[r] < rows)
                a.dbuf[static_cast<size_t>(pair) * a.H + R.id[r]] = wgt * mine;
        }
    }
}

template <int PHASE, int FMT, bool SPLIT, int NR, int CB>
__device__ __forceinline__ void run_unit_mt(const FfnArgs& a, const Unit& u, const Rows<NR>& R,
                                            const Rows<NR>& NRws, bool has_next, int rows, int cols,
                                            const char* lds, const int* lds_pair, const float* lds_wt,
                                            Block<NR, CB>& pre) {
#define MOE_RUN(MTV) \
    run_unit<PHASE, FMT, SPLIT, NR, CB, MTV>(a, u, R, NRws, has_next, rows, cols, lds, lds_pair, lds_wt, pre)
    if (u.ct <= 1) {
        MOE_RUN(1);
    } else if (u.ct <= 2) {
        MOE_RUN(2);
    } else if constexpr (FMT != MOE_W_INT4_G128) {   // INT4 passes hold at most 2 tokens
        if (u.ct <= 4) MOE_RUN(4);
        else MOE_RUN(8);
    }
#undef MOE_RUN
}

// Prologue of both phases: thread s < T reads active slot s's expert, its
// handle and token range into recs[s]; pref[s] receives the inclusive prefix
// of the slots' costs (slots >= T cost 0, so pref[127] is the total).
template <int PHASE>
__device__ __forceinline__ void price_slots(const FfnArgs& a, int T, int tiles, int cols, SlotRec* recs,
                                            int* pref, int* wave_total) {
    const int s = threadIdx.x;
    const int lane = s & (kWave - 1);
    int cost = 0;
    if (s < T) {
        const int e = a.active[s];
        const moe_expert_handle& h = a.table[e];
        SlotRec r;
        r.fmt = h.fmt;
        r.m0 = static_cast<const char*>(PHASE == 0 ? h.w_gate : h.w_down);
        r.m1 = PHASE == 0 ? static_cast<const char*>(h.w_up) : nullptr;
        r.s0 = PHASE == 0 ? h.s_gate : h.s_down;
        r.s1 = PHASE == 0 ? h.s_up : nullptr;
        r.first = a.offsets[e];
        r.cnt = a.offsets[e + 1] - r.first;
        r.pad = 0;
        recs[s] = r;
        const bool split = r.fmt != MOE_W_F32 && (PHASE == 1 || a.x_dtype == MOE_DT_F32);
        cost = tiles * tile_cost(r.cnt, tokens_per_pass(r.fmt, cols, split));
    }
    if (s < kMaxExperts) {              // waves 0 and 1: inclusive scan of 64 slots each
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const int v = __shfl_up(cost, off);
            if (lane >= off) cost += v;
        }
        if (lane == kWave - 1) wave_total[s / kWave] = cost;
    }
    __syncthreads();
    if (s < kMaxExperts) pref[s] = cost + (s >= kWave ? wave_total[0] : 0);
    __syncthreads();
}

// The item whose cost range holds position P: slot = number of prefix entries
// <= P (one ballot per 64 slots), tile = offset in the slot / per-tile cost.
__device__ __forceinline__ long item_at(const int* pref, int T, int tiles, long P) {
    const int lane = threadIdx.x & (kWave - 1);
    int slot = 0;
    for (int base = 0; base < kMaxExperts; base += kWave)
        slot += __popcll(__ballot(pref[base + lane] <= P));
    slot = uni(slot);
    if (slot >= T) return static_cast<long>(T) * tiles;
    const int lo = slot > 0 ? pref[slot - 1] : 0;
    const int per_tile = (pref[slot] - lo) / tiles;
    return static_cast<long>(slot) * tiles + (P - lo) / per_tile;
}

// Persistent workgroups; workgroup b takes the items (active expert, row
// tile) whose cost ranges start in [b*C/G, (b+1)*C/G) of the total cost C
// and, within each item, the passes of up to 8 tokens of its expert.
template <int PHASE>
__global__ __launch_bounds__(kThreads, 2) void ffn_kernel(FfnArgs a) {
    constexpr int NR = PHASE == 0 ? kNrA : kNrB;
    constexpr int CB = PHASE == 0 ? kCbA : kCbB;
    extern __shared__ __attribute__((aligned(16))) char lds[];
    __shared__ int lds_pair[kMaxTok];
    __shared__ float lds_wt[kMaxTok];
    __shared__ int pref[kMaxExperts];
    __shared__ int wave_total[2];
    __shared__ SlotRec recs[kMaxExperts];
    const int T = uni(*a.T);
    const int rows = PHASE == 0 ? a.I : a.H;
    const int cols = PHASE == 0 ? a.H : a.I;
    const int rows_per_item = PHASE == 0 ? kRowsA : kRowsB;
    const int tiles = (rows + rows_per_item - 1) / rows_per_item;
    price_slots<PHASE>(a, T, tiles, cols, recs, pref, wave_total);
    const long C = pref[kMaxExperts - 1];
    const long begin = item_at(pref, T, tiles, C * blockIdx.x / gridDim.x);
    const long end = item_at(pref, T, tiles, C * (blockIdx.x + 1) / gridDim.x);
    if (begin >= end) return;
    const void* src = PHASE == 0 ? a.x : static_cast<const void*>(a.hbuf);
    const int src_dtype = PHASE == 0 ? a.x_dtype : MOE_DT_F32;
    const int by_token = PHASE == 0 ? a.k : 0;

    long item = begin;
    int cnt = 0;
    Unit u = make_unit<PHASE>(recs, a.x_dtype, item, 0, tiles, cols, cnt);
    Rows<NR> R = unit_rows<PHASE, NR>(u, rows, cols);
    Block<NR, CB> pre;
    load_block<NR, CB>(R, 0, pre);
    stage_rows(u.fmt, u.split, src, src_dtype, by_token, a.perm + u.first + u.t0, u.ct, cols, lds, a.w,
               lds_pair, lds_wt);
    __syncthreads();
    while (true) {
        // the unit after u: the next pass of this item, else the next item
        long nitem = item;
        int nt0 = u.t0 + u.ct;
        if (nt0 >= cnt) { nitem = item + 1; nt0 = 0; }
        const bool has_next = nitem < end;
        int ncnt = cnt;
        const Unit nu = has_next ? make_unit<PHASE>(recs, a.x_dtype, nitem, nt0, tiles, cols, ncnt) : u;
        const Rows<NR> NRws = unit_rows<PHASE, NR>(nu, rows, cols);
        if (u.fmt == MOE_W_BF16) {
            if (u.split) run_unit_mt<PHASE, MOE_W_BF16, true, NR, CB>(a, u, R, NRws, has_next, rows, cols, lds, lds_pair, lds_wt, pre);
            else run_unit_mt<PHASE, MOE_W_BF16, false, NR, CB>(a, u, R, NRws, has_next, rows, cols, lds, lds_pair, lds_wt, pre);
        } else if (u.fmt == MOE_W_INT4_G128) {
            if (u.split) run_unit_mt<PHASE, MOE_W_INT4_G128, true, NR, CB>(a, u, R, NRws, has_next, rows, cols, lds, lds_pair, lds_wt, pre);
            else run_unit_mt<PHASE, MOE_W_INT4_G128, false, NR, CB>(a, u, R, NRws, has_next, rows, cols, lds, lds_pair, lds_wt, pre);
        } else {
            run_unit_mt<PHASE, MOE_W_F32, false, NR, CB>(a, u, R, NRws, has_next, rows, cols, lds, lds_pair, lds_wt, pre);
        }
        if (!has_next) break;
        if (nu.slot != u.slot || nu.t0 != u.t0) {
            __syncthreads();
            stage_rows(nu.fmt, nu.split, src, src_dtype, by_token, a.perm + nu.first + nu.t0, nu.ct, cols, lds,
                       a.w, lds_pair, lds_wt);
            __syncthreads();
        }
        u = nu;
        R = NRws;
        item = nitem;
        cnt = ncnt;
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

size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

}  // namespace

// Workspace: SwiGLU activations [B*k, I] fp32, then weighted down
// projections [B*k, H] fp32.
size_t ffn_workspace_bytes(int B, int k, int H, int I) {
    const size_t pairs = static_cast<size_t>(B) * k;
    return align256(pairs * I * sizeof(float)) + align256(pairs * H * sizeof(float));
}

hipError_t launch_expert_ffn(const FfnArgs& in, void* ws, hipStream_t s) {
    FfnArgs a = in;
    const size_t pairs = static_cast<size_t>(a.B) * a.k;
    char* p = static_cast<char*>(ws);
    a.hbuf = reinterpret_cast<float*>(p);
    a.dbuf = reinterpret_cast<float*>(p + align256(pairs * a.I * sizeof(float)));
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
