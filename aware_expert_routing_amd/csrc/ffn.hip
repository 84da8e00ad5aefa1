// Expert FFN (SwiGLU) and weighted combine for a decode batch.
//
// Page "Opportunistic Expert Activation (OEA) - L2", section 4 (Eq. 2 and
// check 4): in decode each activated expert costs a fixed weight fetch b
// plus a small per-token term a, and batched kernels must still load every
// activated expert's weights.  An expert with at most 32 tokens (16 for
// INT4) is streamed from HBM once, every one of its tokens applied to each
// loaded tile.  A larger expert is handled in token passes of that size; its
// passes over the same row blocks run side by side on one CU with cached
// weight loads, so the later passes read the tiles mostly from the L2 (HBM
// counters: 1.07x the algorithmic weight bytes in phase A at B = 128 with
// Zipf routing, against 1.26x when each pass streamed on its own).
// Page "DynaExq", sections 2.2 / 3.2 / 3.4: each expert is reached through a
// handle giving the active version's (prepacked) pointers and quantisation
// parameters, resolved per work item, so one layer may mix formats.
//
// Work decomposition.  Weights are tiled (16 rows x 64 bytes per 1 KB tile,
// in MFMA operand order; see pack.hip), so one wave load instruction reads a
// whole contiguous kilobyte.  The contraction of a tile with the tokens uses
// v_mfma_f32_16x16x32_bf16 (bf16 and INT4 weights) or
// v_mfma_f32_16x16x4f32 (fp32 weights): A = the weight tile (row = lane%16),
// B = 16 tokens' activations (token = lane%16), C = 16 rows x 16 tokens.
// Its cost does not depend on how many of the 16 columns hold real tokens,
// so one path serves experts with 1..16 tokens; up to 32 tokens use two
// column tiles against the same weight tile (weights still read once), and
// an expert with more tokens is handled in passes of 32 tokens (16 for
// INT4 experts) that share its weight tiles through the L2.  At these
// token counts the MFMA units are nearly idle and the kernel is bound by HBM.
//   * phase A: work items are (active expert, 2 row blocks of 16 rows of I);
//     the wave streams the gate and up tiles of those rows over all of H and
//     ends with h = silu(g) * u for every token of the expert.
//   * phase B: items are (active expert, 2 row blocks of H; 4 for experts
//     with more than 16 tokens in a pass) over all of I;
//     the result is scaled by the pair's routing weight.
//   * combine: y[i] = sum over token i's filled slots, in slot order.
// Items belong to single waves (no barriers, no LDS staging): each wave owns
// an equal share of the total streaming cost, keeps several tiles of loads
// in flight (a register ring of D stages) and reads its tokens' activation
// fragments straight from global memory (they stay in L1/L2).  Calls of at
// most 8 routed pairs instead give each item to a workgroup whose waves
// split its input columns and add their partial sums in LDS (see
// ffn_small_kernel): there the items are too few to occupy the chip.
// INT4 tiles are one quantisation group: nibbles become the bf16 values
// 128 + u by bit operations, one MFMA per 32 columns accumulates them, a
// second MFMA with the constant -136 removes the offset (u - 8 = q), and the
// group's per-row fp16 scale multiplies the result into the accumulator.
// fp32 activations meeting bf16/INT4 weights enter as bf16 hi + lo pairs.
// Phase A stores h of a bf16 expert already in that form (per 8 columns:
// 8 bf16 hi, then 8 bf16 lo; 4 bytes per value as in fp32), so phase B,
// which reads each h fragment once per row block, does no splitting; an
// fp32 expert's h stays fp32; an INT4 expert's h is stored in bf16 (W4A16:
// its down projection takes bf16 activations, as its gate/up take bf16 x).
#include "internal.h"

#include <algorithm>
#include <mutex>

namespace moe {
namespace {

constexpr int kWave = 64;
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kTileBytes = 1024;
// Row blocks per work item.  Every weight position also loads the tokens'
// activation fragments, once per item, so an item of more row blocks spends
// fewer activation loads per weight byte.  Two row blocks, except in phase B
// for experts with more than 16 tokens in a pass (two column tiles, and h
// fragments as large as the weight tile per token): four.
template <int PHASE, int NT>
constexpr int rb_per_item() { return PHASE == 1 && NT == 2 ? 4 : 2; }
__host__ __device__ __forceinline__ int rb_per_item(int phase, int nt) { return phase == 1 && nt == 2 ? 4 : 2; }
constexpr int kXcds = 8;  // MI355X: 8 XCDs; the grid is a multiple of 8 workgroups

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef const __attribute__((address_space(1))) u32x4* gptr_u32x4;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef const __attribute__((address_space(1))) u32x2* gptr_u32x2;

// Weight tiles: streamed once, non-temporal.  Activations: cached.
__device__ __forceinline__ u32x4 load_w(const char* p) {
    return __builtin_nontemporal_load((gptr_u32x4)p);
}
__device__ __forceinline__ u32x4 load_a(const char* p) { return *(gptr_u32x4)p; }
__device__ __forceinline__ u32x2 load_a8(const char* p) { return *(gptr_u32x2)p; }
__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }
template <typename T>
__device__ __forceinline__ const T* uni_ptr(const T* p) {   // wave-uniform pointer into SGPRs
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
    return reinterpret_cast<const T*>((static_cast<uint64_t>(hi) << 32) | lo);
}

__device__ __forceinline__ f32x4 mma_bf16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                  c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

__device__ __forceinline__ uint32_t bf16_rne(float f) {   // finite inputs
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
// 8 fp32 (two 16-byte chunks) -> bf16x8 hi and lo with hi + lo ~= f.
__device__ __forceinline__ void split8(u32x4 c0, u32x4 c1, u32x4& hi, u32x4& lo) {
    const uint32_t v[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
    uint32_t h[4], l[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float f0 = __uint_as_float(v[2 * j]), f1 = __uint_as_float(v[2 * j + 1]);
        const uint32_t a = bf16_rne(f0), b = bf16_rne(f1);
        h[j] = a | (b << 16);
        l[j] = bf16_rne(f0 - __uint_as_float(a << 16)) | (bf16_rne(f1 - __uint_as_float(b << 16)) << 16);
    }
    hi = u32x4{h[0], h[1], h[2], h[3]};
    lo = u32x4{l[0], l[1], l[2], l[3]};
}
// INT4 dword (nibble i = column 2i, nibble i+4 = column 2i+1) -> bf16x8 of 128 + u.
__device__ __forceinline__ u32x4 int4_as_bf16(uint32_t d) {
    return u32x4{(d & 0x000F000Fu) | 0x43004300u, ((d >> 4) & 0x000F000Fu) | 0x43004300u,
                 ((d >> 8) & 0x000F000Fu) | 0x43004300u, ((d >> 12) & 0x000F000Fu) | 0x43004300u};
}
constexpr uint32_t kBf16Neg136x2 = 0xC308C308u;   // bf16 pair (-136, -136)

// ---------------------------------------------------------------------------
// Activation fragments.  For the tile covering input columns [c0, c0 + CT),
// lane (n, q) needs columns c0 + q*CT/4 .. + CT/4 of token n: LANE_BYTES
// bytes at byte offset s*TILE_BYTES + q*LANE_BYTES of the token's row, read
// as NRAW 16-byte chunks (8 bytes for fp32 weights with bf16 activations).
// ---------------------------------------------------------------------------
template <int FMT, bool XF32>
struct Act {
    static constexpr int kCols = FMT == MOE_W_F32 ? 16 : (FMT == MOE_W_BF16 ? 32 : 128);
    static constexpr int kLaneBytes = kCols / 4 * (XF32 ? 4 : 2);
    static constexpr int kTileBytes = kLaneBytes * 4;
    static constexpr int kRaw = kLaneBytes >= 16 ? kLaneBytes / 16 : 1;
};

// Ring depths of a wave: weight tiles are loaded D positions ahead of the
// multiply, activation fragments X positions ahead.  X = D except where the
// activation fragments are much larger than the weights (INT4 with fp32
// activations: 128 columns of fp32 per 1 KB tile), where one activation
// stage frees the registers for a deeper weight ring.  The depths come from
// a register budget per case (the rest holds addresses and temporaries; the
// split and INT4 paths need more temporaries).
template <int PHASE, int FMT, bool XF32, int NT, int RB = rb_per_item<PHASE, NT>()>
struct Ring {
    static constexpr int kMatN = PHASE == 0 ? 2 : 1;
    static constexpr int kRbN = RB;
    static constexpr int kW = kMatN * kRbN * (FMT == MOE_W_INT4_G128 ? 6 : 4);   // registers per weight stage
    static constexpr int kX = NT * Act<FMT, XF32>::kRaw * 4;                      // per activation stage
    static constexpr int kAcc = kMatN * kRbN * NT * 4;
    static constexpr int kBudget = (FMT == MOE_W_INT4_G128 && XF32) ? (PHASE == 1 ? 70 : 110)
                                                                    : (PHASE == 1 ? (NT == 2 ? 110 : 90) : ((FMT == MOE_W_INT4_G128 || XF32) ? 150 : 200));
    static constexpr bool kSplit = FMT == MOE_W_INT4_G128 && XF32;
    static constexpr int depth(int x_fixed) {   // x_fixed = 0: X = D
        for (int d = 8; d >= 1; d /= 2)
            if (kW * d + kX * (x_fixed ? x_fixed : d) + kAcc <= kBudget) return d;
        return 1;
    }
    static constexpr int D = kSplit ? depth(1) : (FMT == MOE_W_INT4_G128 && NT > 1 ? 1 : depth(0));
    static constexpr int X = kSplit ? 1 : D;
};

template <int PHASE, int FMT, bool XF32, int NT, int RB = rb_per_item<PHASE, NT>()>
struct WStage {
    static constexpr int kMat = PHASE == 0 ? 2 : 1;
    static constexpr int kRb = RB;
    u32x4 w[kMat][kRb];
    u32x2 sc[kMat][kRb];                       // INT4 only
};
template <int FMT, bool XF32, int NT>
struct XStage {
    u32x4 x[NT][Act<FMT, XF32>::kRaw];
};

// Accumulate one tile (all row blocks, matrices and column tiles).  `keep`
// is all ones, or zero for a padding position: the activation bits are
// ANDed with it, so a padding tile adds exact zeros without a branch.
template <int PHASE, int FMT, bool XF32, int NT, int RB>
__device__ __forceinline__ void tile_mma(const WStage<PHASE, FMT, XF32, NT, RB>& ws, const XStage<FMT, XF32, NT>& xs_in,
                                         uint32_t keep,
                                         f32x4 (&acc)[PHASE == 0 ? 2 : 1][RB][NT]) {
    using S = WStage<PHASE, FMT, XF32, NT, RB>;
    struct {
        const u32x4 (&w)[S::kMat][S::kRb];
        const u32x2 (&sc)[S::kMat][S::kRb];
        u32x4 x[NT][Act<FMT, XF32>::kRaw];
    } st{ws.w, ws.sc, {}};
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int c = 0; c < Act<FMT, XF32>::kRaw; ++c) st.x[t][c] = xs_in.x[t][c] & keep;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        if constexpr (FMT == MOE_W_BF16) {
            if constexpr (!XF32) {
#pragma unroll
                for (int m = 0; m < S::kMat; ++m)
#pragma unroll
                    for (int r = 0; r < S::kRb; ++r) acc[m][r][t] = mma_bf16(st.w[m][r], st.x[t][0], acc[m][r][t]);
            } else {
                u32x4 hi = st.x[t][0], lo = st.x[t][1];   // phase B: h arrives split
                if constexpr (PHASE == 0) split8(st.x[t][0], st.x[t][1], hi, lo);
#pragma unroll
                for (int m = 0; m < S::kMat; ++m)
#pragma unroll
                    for (int r = 0; r < S::kRb; ++r) {
                        acc[m][r][t] = mma_bf16(st.w[m][r], hi, acc[m][r][t]);
                        acc[m][r][t] = mma_bf16(st.w[m][r], lo, acc[m][r][t]);
                    }
            }
        } else if constexpr (FMT == MOE_W_F32) {
            float xv[4];
            if constexpr (XF32) {
                xv[0] = __uint_as_float(st.x[t][0].x);
                xv[1] = __uint_as_float(st.x[t][0].y);
                xv[2] = __uint_as_float(st.x[t][0].z);
                xv[3] = __uint_as_float(st.x[t][0].w);
            } else {
                xv[0] = __uint_as_float(st.x[t][0].x << 16);
                xv[1] = __uint_as_float(st.x[t][0].x & 0xffff0000u);
                xv[2] = __uint_as_float(st.x[t][0].y << 16);
                xv[3] = __uint_as_float(st.x[t][0].y & 0xffff0000u);
            }
#pragma unroll
            for (int m = 0; m < S::kMat; ++m)
#pragma unroll
                for (int r = 0; r < S::kRb; ++r) {
                    const u32x4 wv = st.w[m][r];
                    acc[m][r][t] = mma_f32(__uint_as_float(wv.x), xv[0], acc[m][r][t]);
                    acc[m][r][t] = mma_f32(__uint_as_float(wv.y), xv[1], acc[m][r][t]);
                    acc[m][r][t] = mma_f32(__uint_as_float(wv.z), xv[2], acc[m][r][t]);
                    acc[m][r][t] = mma_f32(__uint_as_float(wv.w), xv[3], acc[m][r][t]);
                }
        } else {   // INT4: one tile = one group of 128 columns = 4 MFMA steps
            constexpr int kParts = XF32 ? 2 : 1;
            u32x4 xb[4][kParts];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if constexpr (XF32 && PHASE == 0) {
                    split8(st.x[t][2 * j], st.x[t][2 * j + 1], xb[j][0], xb[j][1]);
                } else if constexpr (XF32) {   // phase B: h arrives split
                    xb[j][0] = st.x[t][2 * j];
                    xb[j][kParts - 1] = st.x[t][2 * j + 1];
                } else {
                    xb[j][0] = st.x[t][j];
                }
            }
            const u32x4 neg = {kBf16Neg136x2, kBf16Neg136x2, kBf16Neg136x2, kBf16Neg136x2};
            f32x4 corr = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int h = 0; h < kParts; ++h) corr = mma_bf16(neg, xb[j][h], corr);
#pragma unroll
            for (int m = 0; m < S::kMat; ++m)
#pragma unroll
                for (int r = 0; r < S::kRb; ++r) {
                    const u32x4 wv = st.w[m][r];
                    const uint32_t wd[4] = {wv.x, wv.y, wv.z, wv.w};
                    f32x4 tmp = corr;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const u32x4 av = int4_as_bf16(wd[j]);
#pragma unroll
                        for (int h = 0; h < kParts; ++h) tmp = mma_bf16(av, xb[j][h], tmp);
                    }
                    const u32x2 sc = st.sc[m][r];
                    const float s0 = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(sc.x)));
                    const float s1 = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(sc.x >> 16)));
                    const float s2 = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(sc.y)));
                    const float s3 = static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(sc.y >> 16)));
                    f32x4& c = acc[m][r][t];
                    c.x = fmaf(s0, tmp.x, c.x);
                    c.y = fmaf(s1, tmp.y, c.y);
                    c.z = fmaf(s2, tmp.z, c.z);
                    c.w = fmaf(s3, tmp.w, c.w);
                }
        }
    }
}

// ---------------------------------------------------------------------------
// Active-expert records and the cost-balanced partition.  Every workgroup
// prices the active experts first (one thread per active slot): an expert
// has ceil(row_blocks / rb) items; an item's cost is its tile count times a
// per-tile weight (INT4 tiles also carry 4x the activation traffic; every
// extra 16-token column tile adds MFMA work).  Wave w of W takes the items
// whose cost ranges start in [w*C/W, (w+1)*C/W) of the total cost C.
// ---------------------------------------------------------------------------
struct SlotRec {
    const char* m0;          // phase A: gate, phase B: down (packed tiles)
    const char* m1;          // phase A: up
    const char* s0;          // INT4 packed scales (or null)
    const char* s1;
    int32_t fmt, first, cnt, ipp;   // ipp: items per token pass
    int32_t nt;                     // column tiles of the expert's first pass
};

// Tokens per pass: two 16-token column tiles (one for INT4, whose
// activation fragments are four times larger).
__host__ __device__ __forceinline__ int pass_tokens(int fmt) { return fmt == MOE_W_INT4_G128 ? 16 : 32; }

__host__ __device__ __forceinline__ int col_tiles_for(int cnt) { return cnt <= 16 ? 1 : 2; }

template <int PHASE>
__device__ __forceinline__ void price_slots(const FfnArgs& a, int T, const moe_expert_handle* table,
                                            const int* active, const int* offsets, SlotRec* recs, int* pref_cost,
                                            int* pref_item, int* wave_tot) {
    const int s = threadIdx.x;
    const int lane = s & (kWave - 1);
    const int rows = PHASE == 0 ? a.I : a.H, cols = PHASE == 0 ? a.H : a.I;
    int cost = 0, items = 0;
    if (s < T) {
        const int e = active[s];
        const moe_expert_handle& h = table[e];
        SlotRec r;
        r.fmt = h.fmt;
        r.m0 = static_cast<const char*>(PHASE == 0 ? h.w_gate : h.w_down);
        r.m1 = PHASE == 0 ? static_cast<const char*>(h.w_up) : nullptr;
        r.s0 = reinterpret_cast<const char*>(PHASE == 0 ? h.s_gate : h.s_down);
        r.s1 = PHASE == 0 ? reinterpret_cast<const char*>(h.s_up) : nullptr;
        r.first = offsets[e];
        r.cnt = offsets[e + 1] - r.first;
        // pass tokens (16 or 32), row blocks per item (2 or 4) and tile
        // columns (16, 32 or 128) are powers of two: shifts and masks
        const int lpt = r.fmt == MOE_W_INT4_G128 ? 4 : 5;
        const int nt = col_tiles_for(min(r.cnt, 1 << lpt));
        const int lrb = rb_per_item(PHASE, nt) == 4 ? 2 : 1;
        const int rb = 1 << lrb;
        r.nt = nt;
        r.ipp = (rows / 16 + rb - 1) >> lrb;
        recs[s] = r;
        const bool fits = (r.fmt == MOE_W_F32 || r.fmt == MOE_W_BF16 || r.fmt == MOE_W_INT4_G128) &&
                          (cols & (tile_cols(r.fmt) - 1)) == 0 && r.cnt > 0;
        if (fits) {
            const int passes = (r.cnt + (1 << lpt) - 1) >> lpt;
            items = passes * r.ipp;
            const int tiles = rb * (weight_row_bytes(r.fmt, cols) / 64);
            const int per_tile = r.fmt == MOE_W_INT4_G128 ? 12 + 2 * nt : 8 + nt;
            cost = items * tiles * per_tile;
        }
    }
    if (s < 2 * kWave) {   // waves 0 and 1: inclusive scans of 64 slots each
        cost = wave_incl_scan(cost);
        items = wave_incl_scan(items);
        if (lane == kWave - 1) { wave_tot[2 * (s / kWave)] = cost; wave_tot[2 * (s / kWave) + 1] = items; }
    }
    __syncthreads();
    if (s < 2 * kWave) {
        pref_cost[s] = cost + (s >= kWave ? wave_tot[0] : 0);
        pref_item[s] = items + (s >= kWave ? wave_tot[1] : 0);
    }
    __syncthreads();
}

// floor(n / d) for 0 <= n < 2^31 and 0 < d whose quotient is below 2^20:
// a float reciprocal estimate is within one of the quotient (relative error
// about 2^-22), and one correction step in each direction makes it exact.
__device__ __forceinline__ int div_small(int n, int d) {
    int q = static_cast<int>(static_cast<float>(n) * __builtin_amdgcn_rcpf(static_cast<float>(d)));
    const int r = n - q * d;
    q += (r >= d ? 1 : 0) - (r < 0 ? 1 : 0);
    return q;
}

// Number of prefix entries <= v (the slot whose range holds v), per wave.
__device__ __forceinline__ int count_le(const int* pref, int v) {
    const int lane = threadIdx.x & (kWave - 1);
    int n = 0;
#pragma unroll
    for (int base = 0; base < kMaxExperts; base += kWave) n += __popcll(__ballot(pref[base + lane] <= v));
    return uni(n);
}

// The item whose cost range holds position P (the total item count past the end).
__device__ __forceinline__ int item_at(const int* pref_cost, const int* pref_item, int T, int P) {
    const int slot = count_le(pref_cost, P);
    if (slot >= T) return pref_item[kMaxExperts - 1];
    const int c_lo = slot > 0 ? pref_cost[slot - 1] : 0;
    const int i_lo = slot > 0 ? pref_item[slot - 1] : 0;
    const int n_items = pref_item[slot] - i_lo;
    const int per_item = div_small(pref_cost[slot] - c_lo, n_items);   // quotients: item cost, item index
    return i_lo + div_small(P - c_lo, per_item);
}

// Write one item's results for every real token of its column tiles:
// phase A h = silu(g) * u in the expert's h format, phase B the pair's
// routing weight times the down projection.  acc[m][r][t]: matrix m (gate,
// up), row block r (first row block rb0), column tile t (tokens 16 t + n).
template <int PHASE, int FMT, int KMAT, int KRB, int NT>
__device__ __forceinline__ void store_item(const f32x4 (&acc)[KMAT][KRB][NT], const int (&pair)[NT],
                                           const float (&wt)[NT], float* hbuf, float* dbuf, int H, int I,
                                           int rb0, int nrb, int cnt, int n, int q) {
    constexpr int kMat = KMAT, kRb = KRB;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        if (16 * t + n >= cnt) continue;
        if constexpr (PHASE == 0) {
            float* hrow = hbuf + static_cast<size_t>(pair[t]) * I;
#pragma unroll
            for (int r = 0; r < kRb; ++r) {
                if (rb0 + r >= nrb) continue;
                const f32x4 g = acc[0][r][t], u = acc[kMat - 1][r][t];
                const float hv[4] = {silu(g.x) * u.x, silu(g.y) * u.y, silu(g.z) * u.z, silu(g.w) * u.w};
                const int c = (rb0 + r) * 16 + 4 * q;   // first of this lane's 4 columns of h
                if constexpr (FMT == MOE_W_F32) {
                    *reinterpret_cast<float4*>(hrow + c) = make_float4(hv[0], hv[1], hv[2], hv[3]);
                } else if constexpr (FMT == MOE_W_INT4_G128) {
                    // INT4 experts take h in bf16 (W4A16), row-major in the row's first 2 I bytes
                    const uint2 hb = make_uint2(bf16_rne(hv[0]) | (bf16_rne(hv[1]) << 16),
                                                bf16_rne(hv[2]) | (bf16_rne(hv[3]) << 16));
                    *reinterpret_cast<uint2*>(reinterpret_cast<char*>(hrow) + 2 * c) = hb;
                } else {
                    // split layout: per 8 columns, 8 bf16 hi then 8 bf16 lo
                    uint32_t hi[2], lo[2];
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const uint32_t a = bf16_rne(hv[2 * j]), b = bf16_rne(hv[2 * j + 1]);
                        hi[j] = a | (b << 16);
                        lo[j] = bf16_rne(hv[2 * j] - __uint_as_float(a << 16)) |
                                (bf16_rne(hv[2 * j + 1] - __uint_as_float(b << 16)) << 16);
                    }
                    char* gp = reinterpret_cast<char*>(hrow) + (c / 8) * 32 + (c % 8) * 2;
                    *reinterpret_cast<uint2*>(gp) = make_uint2(hi[0], hi[1]);
                    *reinterpret_cast<uint2*>(gp + 16) = make_uint2(lo[0], lo[1]);
                }
            }
        } else {
            float* drow = dbuf + static_cast<size_t>(pair[t]) * H;
#pragma unroll
            for (int r = 0; r < kRb; ++r) {
                if (rb0 + r >= nrb) continue;
                const f32x4 v = acc[0][r][t];
                *reinterpret_cast<float4*>(drow + (rb0 + r) * 16 + 4 * q) =
                    make_float4(wt[t] * v.x, wt[t] * v.y, wt[t] * v.z, wt[t] * v.w);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// One wave streams `count` consecutive items of one expert, starting at item
// `local0` of that expert.  Positions (item, tile) run through a ring of D
// stages: while tile p is multiplied, the loads of tile p + D are issued.
// Each item's tile count is padded to a multiple of D; padding positions
// re-load the item's last tile (cache hits) and skip the multiply.  Row
// blocks past the matrix end are clamped to the last one and not stored.
// ---------------------------------------------------------------------------
// Arguments are plain values (no struct in private memory); every one is
// wave-uniform and is moved to SGPRs, so the ring's loads and waits are
// scheduled per stage rather than behind divergent branches.
// SHARED: the expert has several token passes, which run side by side (see
// the item order in ffn_kernel): its weight tiles are loaded through the
// caches, so the passes after the first read them from the L2, not from HBM.
template <int PHASE, int FMT, bool XF32, int NT, int PRE = 0, bool KSPLIT = false, int RB = rb_per_item<PHASE, NT>(),
          bool SHARED = false>
__device__ __forceinline__ void run_items(const char* x_in, const int32_t* perm_in, const float* w_in,
                                       float* hbuf_in, float* dbuf_in, int k_in, int H_in, int I_in,
                                       const char* m0, const char* m1, const char* s0, const char* s1,
                                       int first_in, int cnt_in, int local0_in, int count_in,
                                       const WStage<PHASE, FMT, XF32, NT, RB>* pre = nullptr, int pre_pair = 0,
                                       int t_lo_in = 0, int t_n_in = 0, f32x4* part = nullptr) {
    const int local0 = uni(local0_in), count = uni(count_in);
    const int k = uni(k_in), H = uni(H_in), I = uni(I_in);
    const char* xg = uni_ptr(x_in);
    const int32_t* perm = uni_ptr(perm_in);
    const float* wg = uni_ptr(w_in);
    float* hbuf = const_cast<float*>(uni_ptr(hbuf_in));
    float* dbuf = const_cast<float*>(uni_ptr(dbuf_in));
    using Wst = WStage<PHASE, FMT, XF32, NT, RB>;
    using Xst = XStage<FMT, XF32, NT>;
    using Ac = Act<FMT, XF32>;
    constexpr int kMat = Wst::kMat, kRb = Wst::kRb;
    // weight stages in flight, and activation stages (X divides D); a slice
    // of a column-split item has few tiles and keeps at most 4 stages (2 for
    // INT4, whose activation stages are four times larger)
    using Rg = Ring<PHASE, FMT, XF32, NT, RB>;
    constexpr int D = KSPLIT ? std::min(FMT == MOE_W_INT4_G128 ? 2 : 4, Rg::D) : Rg::D;
    constexpr int X = std::min(D, Rg::X);
    const int lane = threadIdx.x & (kWave - 1);
    const int n = lane & 15, q = lane >> 4;
    const int rows = PHASE == 0 ? I : H, cols = PHASE == 0 ? H : I;
    const int nrb = rows / 16;
    const int S = uni(weight_row_bytes(FMT, cols) / 64);     // tiles per row block
    // KSPLIT: the wave streams only tile columns [t_lo, t_lo + Sl) of its
    // (single) item and leaves the partial sums in part[] (LDS)
    const int t_lo = KSPLIT ? uni(t_lo_in) : 0;
    const int Sl = KSPLIT ? uni(t_n_in) : S;
    const int Sp = uni((Sl + D - 1) / D * D);
    const int first = uni(first_in), cnt = uni(cnt_in);
    const char* mb[kMat];
    const char* sb[kMat];
    mb[0] = uni_ptr(m0);
    sb[0] = uni_ptr(s0);
    if constexpr (kMat == 2) { mb[1] = uni_ptr(m1); sb[1] = uni_ptr(s1); }

    const char* arow[NT];   // activation rows of this lane's tokens (column tile t: token 16 t + n)
    int pair[NT];
    float wt[NT];           // phase B: the pairs' routing weights

    // PRE: the caller has already issued the first PRE weight stages of the
    // first item (the same tiles this function would load) into pre[], and
    // this lane's perm entry into pre_pair (one column tile).
    static_assert(PRE == 0 || NT == 1, "pre-issued runs have one column tile");
    Wst ring[D];
    Xst xring[X];
    auto issue = [&](Wst& st, int item, int s) {
        const int se = t_lo + (s < Sl ? s : Sl - 1);
#pragma unroll
        for (int m = 0; m < kMat; ++m)
#pragma unroll
            for (int r = 0; r < kRb; ++r) {
                int rb = (local0 + item) * kRb + r;
                rb = rb < nrb ? rb : nrb - 1;
                const long tile = static_cast<long>(rb) * S + se;
                st.w[m][r] = SHARED ? load_a(mb[m] + tile * kTileBytes + lane * 16)
                                    : load_w(mb[m] + tile * kTileBytes + lane * 16);
                if constexpr (FMT == MOE_W_INT4_G128) st.sc[m][r] = load_a8(sb[m] + (tile * 16 + 4 * q) * 2);
            }
    };
    // activation fragments depend on the tile column only, not on the item
    auto issue_x = [&](Xst& st, int s) {
        const int se = t_lo + (s < Sl ? s : Sl - 1);
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int c = 0; c < Ac::kRaw; ++c) {
                const char* p = arow[t] + static_cast<long>(se) * Ac::kTileBytes + 16 * c;
                if constexpr (Ac::kLaneBytes == 8) {
                    const u32x2 v = load_a8(p);
                    st.x[t][c] = u32x4{v.x, v.y, 0u, 0u};
                } else {
                    st.x[t][c] = load_a(p);
                }
            }
    };

    f32x4 acc[kMat][kRb][NT];
    auto zero = [&]() {
#pragma unroll
        for (int m = 0; m < kMat; ++m)
#pragma unroll
            for (int r = 0; r < kRb; ++r)
#pragma unroll
                for (int t = 0; t < NT; ++t) acc[m][r][t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    };
    zero();
    // The perm entries go out first, then the weight stages: loads return in
    // order, so the wait for the perm entries does not cover the weights, and
    // the activation rows they address are requested while the weights are
    // still in flight.
    if constexpr (PRE == 0) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const int tok = 16 * t + n;
            pair[t] = ((const __attribute__((address_space(1))) int32_t*)perm)[first + (tok < cnt ? tok : 0)];
        }
        // keep the weight loads below (the perm loads stay first)
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int d = 0; d < D; ++d) {
        if (d < PRE) ring[d] = pre[d];
        else issue(ring[d], 0, d);
    }
    // and the address arithmetic on the perm entries (which waits for them) below them
    if constexpr (PRE == 0) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        if constexpr (PRE > 0) pair[t] = pre_pair;
        if constexpr (PHASE == 0)
            arow[t] = xg + static_cast<size_t>(pair[t] / k) * H * (XF32 ? 4 : 2);
        else
            arow[t] = reinterpret_cast<const char*>(hbuf + static_cast<size_t>(pair[t]) * I);
        arow[t] += q * Ac::kLaneBytes;
        wt[t] = PHASE == 1 ? ((const __attribute__((address_space(1))) float*)wg)[pair[t]] : 0.0f;
    }
#pragma unroll
    for (int d = 0; d < X; ++d) issue_x(xring[d], d);

    const int nblk = count * (Sp / D);
    int ci = 0, cs = 0;   // item and first tile of the block being multiplied
    int ii = 0, is = 0;   // item and first tile of the block being issued
    // The stage loop has no branches (padding is masked, the last block is
    // peeled), so the waits before each multiply cover only that stage.
    for (int blk = 0; blk < nblk; ++blk) {
        const bool last = blk + 1 == nblk;
        is += D;
        if (is == Sp) { is = 0; ++ii; }
        if (!last) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                tile_mma<PHASE, FMT, XF32, NT, RB>(ring[d], xring[d % X], cs + d < Sl ? ~0u : 0u, acc);
                issue(ring[d], ii, is + d);
                if constexpr (X == D) {
                    issue_x(xring[d], is + d);
                } else {
                    const int ta = cs + d + X;   // tile column X positions ahead (wraps into the next item)
                    issue_x(xring[d % X], ta < Sp ? ta : ta - Sp);
                }
            }
        } else {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                tile_mma<PHASE, FMT, XF32, NT, RB>(ring[d], xring[d % X], cs + d < Sl ? ~0u : 0u, acc);
                if constexpr (X < D) {
                    if (d + X < D) issue_x(xring[d % X], cs + d + X);
                }
            }
        }
        cs += D;
        if (cs == Sp) {   // item done: write its rows for every real token
            if constexpr (KSPLIT) {
#pragma unroll
                for (int m = 0; m < kMat; ++m)
#pragma unroll
                    for (int r = 0; r < kRb; ++r)
#pragma unroll
                        for (int t = 0; t < NT; ++t) part[((m * kRb + r) * NT + t) * kWave + lane] = acc[m][r][t];
            } else {
                store_item<PHASE, FMT, kMat, kRb, NT>(acc, pair, wt, hbuf, dbuf, H, I, (local0 + ci) * kRb, nrb, cnt,
                                                      n, q);
            }
            zero();
            cs = 0;
            ++ci;
        }
    }
}

// Out-of-line copy for the formats off the hot path (fp32, INT4, bf16 with
// fp32 activations in phase A): a call keeps their register needs apart
// from the inlined bf16 path.
template <int PHASE, int FMT, bool XF32, int NT, bool SHARED>
__device__ __noinline__ void run_items_call(const char* x, const int32_t* perm, const float* w, float* hbuf,
                                            float* dbuf, int k, int H, int I, const char* m0, const char* m1,
                                            const char* s0, const char* s1, int first, int cnt, int local0,
                                            int count) {
    run_items<PHASE, FMT, XF32, NT, 0, false, rb_per_item<PHASE, NT>(), SHARED>(x, perm, w, hbuf, dbuf, k, H, I, m0,
                                                                             m1, s0, s1, first, cnt, local0, count);
}

template <int PHASE, int FMT, bool XF32, bool SHARED>
__device__ __forceinline__ void run_nt(const FfnArgs& a, const SlotRec& rec, int local0, int count) {
    // bf16 weights with bf16 activations (phase A) or fp32 h (phase B) run inline
    constexpr bool hot = FMT == MOE_W_BF16 && XF32 == (PHASE == 1);
#define MOE_RUN_INLINE(NTV)                                                                                       \
    run_items<PHASE, FMT, XF32, NTV, 0, false, rb_per_item<PHASE, NTV>(), SHARED>(                              \
        static_cast<const char*>(a.x), a.perm, a.w, a.hbuf, a.dbuf, a.k, a.H, a.I, rec.m0, rec.m1, rec.s0, rec.s1, \
        rec.first, rec.cnt, local0, count)
#define MOE_RUN_CALL(NTV)                                                                                      \
    run_items_call<PHASE, FMT, XF32, NTV, SHARED>(static_cast<const char*>(a.x), a.perm, a.w, a.hbuf, a.dbuf,  \
                                                  a.k, a.H, a.I, rec.m0, rec.m1, rec.s0, rec.s1, rec.first,    \
                                                  rec.cnt, local0, count)
    // Phase A picks the column tiles per pass; phase B keeps the expert's
    // (its items' row blocks depend on them), so a last pass of at most 16
    // tokens of a larger expert runs with a masked second column tile.
    const bool one = (PHASE == 0 ? rec.cnt : 16 * rec.nt) <= 16;
    if constexpr (hot) {
        if (one) MOE_RUN_INLINE(1);
        else MOE_RUN_INLINE(2);
    } else {
        if (FMT == MOE_W_INT4_G128 || one) MOE_RUN_CALL(1);
        else MOE_RUN_CALL(FMT == MOE_W_INT4_G128 ? 1 : 2);
    }
#undef MOE_RUN_INLINE
#undef MOE_RUN_CALL
}

template <int PHASE, bool XF32, bool SHARED>
__device__ __forceinline__ void run_fmt_s(const FfnArgs& a, const SlotRec& rec, int local0, int count) {
    if (rec.fmt == MOE_W_BF16) run_nt<PHASE, MOE_W_BF16, XF32, SHARED>(a, rec, local0, count);
    else if (rec.fmt == MOE_W_INT4_G128) run_nt<PHASE, MOE_W_INT4_G128, PHASE == 0 && XF32, SHARED>(a, rec, local0, count);
    else run_nt<PHASE, MOE_W_F32, XF32, SHARED>(a, rec, local0, count);
}

template <int PHASE, bool XF32>
__device__ __forceinline__ void run_fmt(const FfnArgs& a, const SlotRec& rec, int local0, int count, bool shared) {
    if (shared) run_fmt_s<PHASE, XF32, true>(a, rec, local0, count);
    else run_fmt_s<PHASE, XF32, false>(a, rec, local0, count);
}

// ---------------------------------------------------------------------------
// Small batches (at most kSmallPairs routed pairs, so T <= 16 and every
// expert has at most 16 tokens).  There the per-wave items above leave most
// of the chip idle (B = 1, T = 3: 72 phase-A items), and each phase lasts as
// long as one wave needs to stream an item.  Here an item (expert, one or
// two row blocks) belongs to a workgroup of kSlices waves; wave j streams the j-th
// contiguous share of the item's tile columns, the partial sums meet in
// LDS, and wave 0 adds them in slice order (so results are deterministic)
// and writes the item as the per-wave path does.
// ---------------------------------------------------------------------------
constexpr int kSmallPairs = 8;
constexpr int kSmallThreads = 256;
constexpr int kSlices = kSmallThreads / kWave;
// row blocks per item: one in phase A (twice the workgroups), two in phase B
// (whose items are small: 16 rows of I)
template <int PHASE>
constexpr int small_rb() { return PHASE == 0 ? 1 : 2; }

template <int PHASE, int FMT, bool XF32, int RB = small_rb<PHASE>()>
__device__ __forceinline__ void small_item(const FfnArgs& a, const moe_expert_handle& h, int first, int cnt,
                                           int item, f32x4* part_l) {
    using Wst = WStage<PHASE, FMT, XF32, 1, RB>;
    constexpr int kMat = Wst::kMat, kRb = Wst::kRb;
    constexpr int kPart = kMat * kRb * kWave;   // f32x4 per slice
    const int cols = PHASE == 0 ? a.H : a.I, nrb = (PHASE == 0 ? a.I : a.H) / 16;
    const int S = weight_row_bytes(FMT, cols) / 64;
    const int ns = min(kSlices, S);   // slices with at least one tile column
    const int j = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const char* m0 = static_cast<const char*>(PHASE == 0 ? h.w_gate : h.w_down);
    const char* m1 = static_cast<const char*>(PHASE == 0 ? h.w_up : h.w_down);
    const char* s0 = reinterpret_cast<const char*>(PHASE == 0 ? h.s_gate : h.s_down);
    const char* s1 = reinterpret_cast<const char*>(PHASE == 0 ? h.s_up : h.s_down);
    if (j < ns) {
        const int lo = j * S / ns, hi = (j + 1) * S / ns;   // hi > lo since ns <= S
        run_items<PHASE, FMT, XF32, 1, 0, true, RB>(static_cast<const char*>(a.x), a.perm, a.w, a.hbuf, a.dbuf, a.k,
                                                a.H, a.I, m0, m1, s0, s1, first, cnt, item, 1, nullptr, 0, lo,
                                                hi - lo, part_l + j * kPart);
    }
    __syncthreads();
    if (j == 0) {
        f32x4 acc[kMat][kRb][1];
#pragma unroll
        for (int m = 0; m < kMat; ++m)
#pragma unroll
            for (int r = 0; r < kRb; ++r) {
                f32x4 v = part_l[(m * kRb + r) * kWave + lane];
                for (int jj = 1; jj < ns; ++jj) v += part_l[jj * kPart + (m * kRb + r) * kWave + lane];
                acc[m][r][0] = v;
            }
        const int n = lane & 15, q = lane >> 4;
        const int pair[1] = {((const __attribute__((address_space(1))) int32_t*)a.perm)[first + (n < cnt ? n : 0)]};
        const float wt[1] = {PHASE == 1 ? ((const __attribute__((address_space(1))) float*)a.w)[pair[0]] : 0.0f};
        store_item<PHASE, FMT, kMat, kRb, 1>(acc, pair, wt, a.hbuf, a.dbuf, a.H, a.I, item * kRb, nrb, cnt, n, q);
    }
}

// One (expert, item) of the column-split path, in the expert's format; the
// caller's whole workgroup calls it (it holds a barrier).  An expert whose
// format does not fit the sizes contributes nothing, as in the per-wave path.
template <int PHASE, int RB = small_rb<PHASE>()>
__device__ __forceinline__ void small_unit(const FfnArgs& a, const moe_expert_handle& h, int first, int cnt,
                                           int item, f32x4* part_l) {
    const int fmt = uni(h.fmt);
    const bool known = fmt == MOE_W_F32 || fmt == MOE_W_BF16 || fmt == MOE_W_INT4_G128;
    if (!known || ((PHASE == 0 ? a.H : a.I) & (tile_cols(fmt) - 1)) != 0) return;
    if (fmt == MOE_W_BF16) {
        if (PHASE == 1 || a.x_dtype == MOE_DT_F32) small_item<PHASE, MOE_W_BF16, true, RB>(a, h, first, cnt, item, part_l);
        else small_item<PHASE, MOE_W_BF16, false, RB>(a, h, first, cnt, item, part_l);
    } else if (fmt == MOE_W_INT4_G128) {
        if (PHASE == 0 && a.x_dtype == MOE_DT_F32) small_item<PHASE, MOE_W_INT4_G128, true, RB>(a, h, first, cnt, item, part_l);
        else small_item<PHASE, MOE_W_INT4_G128, false, RB>(a, h, first, cnt, item, part_l);
    } else {
        if (PHASE == 1 || a.x_dtype == MOE_DT_F32) small_item<PHASE, MOE_W_F32, true, RB>(a, h, first, cnt, item, part_l);
        else small_item<PHASE, MOE_W_F32, false, RB>(a, h, first, cnt, item, part_l);
    }
}

// Resident waves per SIMD: phase A keeps 2 (deep rings of gate+up tiles),
// phase B 3 (more waves with smaller items).
template <int PHASE>
constexpr int waves_per_simd() { return PHASE == 0 ? 2 : 3; }

template <int PHASE>
__global__ __launch_bounds__(kThreads, waves_per_simd<PHASE>()) void ffn_kernel(FfnArgs a) {
    __shared__ SlotRec recs[kMaxExperts];
    __shared__ int pref_cost[kMaxExperts];
    __shared__ int pref_item[kMaxExperts];
    __shared__ int wave_tot[4];
    __shared__ u32x4 table_l[kMaxExperts * 4];   // the N handles, 4 x 16 bytes each
    __shared__ int active_l[kMaxExperts];
    __shared__ int offsets_l[kMaxExperts + 1];
    __shared__ int odd_l[kWaves];
    __shared__ int big_l[kWaves];
    __shared__ f32x4 part_l[kSlices * 2 * kWave];   // column-split path
    static_assert(kSmallThreads == kThreads, "the column-split path runs on this kernel's workgroups");
    // Stage the handle table, active list and offsets with independent loads
    // (one round trip) instead of following active -> handle per slot.  The
    // loads take clamped (in-bounds) addresses and are all issued before the
    // first LDS write, so no load waits behind another.
    static_assert(kMaxExperts * 4 <= 2 * kThreads && kMaxExperts + 1 <= kThreads, "staging layout");
    const int T = uni(*a.T);
    const int tid = threadIdx.x, nc = a.N * 4;
    const char* tb = reinterpret_cast<const char*>(a.table);
    const u32x4 t0 = load_a(tb + 16 * min(tid, nc - 1));
    const u32x4 t1 = load_a(tb + 16 * min(tid + kThreads, nc - 1));
    const int act = ((const __attribute__((address_space(1))) int32_t*)a.active)[min(tid, a.N - 1)];
    const int off = ((const __attribute__((address_space(1))) int32_t*)a.offsets)[min(tid, a.N)];
    const int off1 = ((const __attribute__((address_space(1))) int32_t*)a.offsets)[min(tid + 1, a.N)];
    const int fmt = ((const __attribute__((address_space(1))) int32_t*)tb)[16 * min(tid, a.N - 1)];
    if (tid < nc) table_l[tid] = t0;
    if (tid + kThreads < nc) table_l[tid + kThreads] = t1;
    if (tid < a.N) active_l[tid] = act;
    if (tid <= a.N) offsets_l[tid] = off;
    // Expert tid outside the uniform case below: active and not bf16 with at most 16 tokens.
    const uint64_t odd = __ballot(tid < a.N && off1 > off && (fmt != MOE_W_BF16 || off1 - off > 16));
    if ((tid & (kWave - 1)) == 0) odd_l[tid / kWave] = odd != 0;
    // expert tid has more than 16 tokens (more than one column tile)
    const uint64_t big = __ballot(tid < a.N && off1 - off > 16);
    if ((tid & (kWave - 1)) == 0) big_l[tid / kWave] = big != 0;
    __syncthreads();
    if constexpr (PHASE == 0) {
        // Few items: when every (expert, row block) gets a workgroup of its own
        // and every expert fits one column tile, phase A takes the column-split
        // path (the per-wave items would leave most CUs idle).  T decides it,
        // so padding tokens do not change the path.
        bool one_tile = true;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) one_tile = one_tile && big_l[w] == 0;
        const int ipp_s = a.I / 16;   // small_rb<0>() == 1
        if (one_tile && T * ipp_s <= static_cast<int>(gridDim.x)) {
            const int s = div_small(blockIdx.x, ipp_s), item = blockIdx.x - s * ipp_s;
            if (s < T) {   // the same for the whole workgroup
                const int e = active_l[s];
                small_unit<0>(a, reinterpret_cast<const moe_expert_handle*>(table_l)[e], offsets_l[e],
                              offsets_l[e + 1] - offsets_l[e], item, part_l);
            }
            return;
        }
    } else {
        // phase B likewise, with items of one row block (the per-wave path's
        // register budget holds their slices; two row blocks would not fit)
        bool one_tile = true;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) one_tile = one_tile && big_l[w] == 0;
        const int ipp_s = a.H / 16;
        if (one_tile && T * ipp_s <= static_cast<int>(gridDim.x)) {
            const int s = div_small(blockIdx.x, ipp_s), item = blockIdx.x - s * ipp_s;
            if (s < T) {
                const int e = active_l[s];
                small_unit<1, 1>(a, reinterpret_cast<const moe_expert_handle*>(table_l)[e], offsets_l[e],
                                 offsets_l[e + 1] - offsets_l[e], item, part_l);
            }
            return;
        }
    }
    const int Wn = gridDim.x * kWaves;
    // XCD- and CU-aware numbering.  Workgroups are dealt to the 8 XCDs
    // round-robin (blockIdx % 8) and, inside an XCD, to its CUs round-robin,
    // so workgroup b sits on CU (b / 8) % cus_per_xcd of XCD b % 8.  The
    // virtual order runs XCD by XCD and, inside an XCD, CU by CU: each XCD
    // takes 1/8 of the total cost, the waves of one CU take consecutive items
    // (usually one expert, whose activation rows they share in L1/L2), and
    // when items are fewer than waves the idle waves spread evenly over CUs.
    const int xcd = blockIdx.x % kXcds, per_xcd = gridDim.x / kXcds, lb = blockIdx.x / kXcds;
    constexpr int wps = waves_per_simd<PHASE>();   // workgroups per CU
    const int cus = per_xcd / wps, lq = div_small(lb, cus > 0 ? cus : 1);
    const int slot = per_xcd % wps == 0 ? (lb - lq * cus) * wps + lq : lb;
    const int gw = (xcd * per_xcd + slot) * kWaves + threadIdx.x / kWave;
    // Speculative first ring stages.  When every active expert is bf16 with
    // at most 16 tokens (and phase A's activations are bf16), every item
    // costs the same and wave gw's first item is floor(T ipp gw / Wn): the
    // wave issues that item's first weight stages now, while the pricing
    // below runs, and uses them if the pricing agrees (they are the tiles the
    // run would load first).  Other batches skip it: there a wrong guess
    // would cost HBM reads.
    using WsHot = WStage<PHASE, MOE_W_BF16, PHASE == 1, 1>;
    constexpr int DH = Ring<PHASE, MOE_W_BF16, PHASE == 1, 1>::D;
    WsHot spec[DH];
    int s_g = -1, l0_g = -1, pair_g = 0;
    bool uniform = PHASE == 1 || a.x_dtype == MOE_DT_BF16;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) uniform = uniform && odd_l[w] == 0;
    {
        const int nrb = (PHASE == 0 ? a.I : a.H) / 16, ipp = (nrb + 1) / 2;   // two row blocks per item
        const int ng = T * ipp, bg = ng * gw / Wn, eg = ng * (gw + 1) / Wn;   // < 2^31
        if (uniform && bg < eg) {
            const int sg = div_small(bg, ipp), lg = bg - sg * ipp;
            const int e = active_l[sg];
            const moe_expert_handle& h = reinterpret_cast<const moe_expert_handle*>(table_l)[e];
            s_g = uni(sg);
            l0_g = uni(lg);
            // the perm entry first: the run waits for it alone, not for the weights behind it
            const int f = offsets_l[e], c = offsets_l[e + 1] - f, n = threadIdx.x & 15;
            pair_g = ((const __attribute__((address_space(1))) int32_t*)a.perm)[f + (n < c ? n : 0)];
            const char* m[2] = {uni_ptr(static_cast<const char*>(PHASE == 0 ? h.w_gate : h.w_down)),
                                uni_ptr(static_cast<const char*>(PHASE == 0 ? h.w_up : h.w_down))};
            const int S = weight_row_bytes(MOE_W_BF16, PHASE == 0 ? a.H : a.I) / 64;
            const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
            for (int d = 0; d < DH; ++d)
#pragma unroll
                for (int mm = 0; mm < WsHot::kMat; ++mm)
#pragma unroll
                    for (int r = 0; r < WsHot::kRb; ++r) {
                        const int rb = min(l0_g * WsHot::kRb + r, nrb - 1);
                        const long tile = static_cast<long>(rb) * S + min(d, S - 1);
                        spec[d].w[mm][r] = load_w(m[mm] + tile * kTileBytes + lane * 16);
                    }
        }
    }
    price_slots<PHASE>(a, T, reinterpret_cast<const moe_expert_handle*>(table_l), active_l, offsets_l, recs,
                       pref_cost, pref_item, wave_tot);
    // Range start of wave w: floor(C w / Wn), in 32-bit arithmetic (C is
    // below 2^31: the launcher checks its bound; (C mod Wn) w < 2^24).
    const int C = pref_cost[kMaxExperts - 1];
    const int cq = C / Wn, cr = C - cq * Wn;
    const int begin = item_at(pref_cost, pref_item, T, cq * gw + cr * gw / Wn);
    const int end = item_at(pref_cost, pref_item, T, cq * (gw + 1) + cr * (gw + 1) / Wn);
    int it = begin;
    // The speculated item: the range starts at item 0 of the first pass of a
    // bf16 expert with at most 16 tokens.  Peeled out of the loop so that the
    // speculative stages are not live across the other runs.
    if (s_g >= 0 && it < end) {
        const int slot = count_le(pref_item, it);
        const int i_lo = slot > 0 ? pref_item[slot - 1] : 0;
        const SlotRec rec = recs[slot];
        const int ipp = uni(rec.ipp);
        if (slot == s_g && it - i_lo == l0_g && rec.fmt == MOE_W_BF16 && rec.cnt <= 16) {
            const int count = uni(min(end, i_lo + ipp) - it);
            // no use of the perm entry may move above this point (its wait would stall the pricing)
            asm volatile("" : "+v"(pair_g));
            run_items<PHASE, MOE_W_BF16, PHASE == 1, 1, DH>(static_cast<const char*>(a.x), a.perm, a.w, a.hbuf,
                a.dbuf, a.k, a.H, a.I, rec.m0, rec.m1, rec.s0, rec.s1, rec.first, rec.cnt, l0_g, count, spec,
                pair_g);
            it += count;
        }
    }
    // One run per (expert, pass) touched by the range.  A single-pass
    // expert's items run in row order, many per run.  An expert with several
    // token passes has its items ordered row block first, pass second, so the
    // passes over the same weight tiles are consecutive items: they land on
    // the same CU at about the same time, and the tiles, loaded through the
    // caches, reach HBM once.
    while (it < end) {
        const int slot = count_le(pref_item, it);   // < T because it < total items
        const int i_lo = slot > 0 ? pref_item[slot - 1] : 0;
        SlotRec rec = recs[slot];
        const int ipp = uni(rec.ipp);
        const int pt = pass_tokens(rec.fmt);
        const int passes = uni((rec.cnt + pt - 1) / pt);
        int pass, local0, count;
        if (passes == 1) {
            pass = 0;
            local0 = it - i_lo;
            count = uni(min(end, i_lo + ipp) - it);
        } else {
            local0 = div_small(it - i_lo, passes);
            pass = it - i_lo - local0 * passes;
            count = 1;
        }
        rec.first += pass * pt;
        rec.cnt = min(pt, rec.cnt - pass * pt);
        if (PHASE == 1 || a.x_dtype == MOE_DT_F32) run_fmt<PHASE, true>(a, rec, local0, count, passes > 1);
        else run_fmt<PHASE, false>(a, rec, local0, count, passes > 1);
        it += count;
    }
}

// One workgroup per (active slot, item); workgroups past T exit at once.
template <int PHASE>
__global__ __launch_bounds__(kSmallThreads, 2) void ffn_small_kernel(FfnArgs a) {
    __shared__ f32x4 part_l[kSlices * 2 * kWave];   // slices x (matrices x row blocks = 2) x lanes
    static_assert((PHASE == 0 ? 2 : 1) * small_rb<PHASE>() == 2, "partial sums layout");
    const int nrb = (PHASE == 0 ? a.I : a.H) / 16, ipp = (nrb + small_rb<PHASE>() - 1) / small_rb<PHASE>();
    const int s = blockIdx.x / ipp, item = blockIdx.x - s * ipp;
    // T and the slot's expert in one round trip (s < N: the grid covers at most N slots)
    const int T = uni(*a.T);
    const int e = uni(((const __attribute__((address_space(1))) int32_t*)a.active)[s]);
    if (s >= T) return;
    const moe_expert_handle h = a.table[e];
    const int first = uni(a.offsets[e]), cnt = uni(a.offsets[e + 1]) - first;
    small_unit<PHASE>(a, h, first, cnt, item, part_l);
}

// y[i, o] = sum over filled slots s of token i (slot order) of dbuf[i*k+s, o].
// One wavefront per (token, 256 outputs).  All of the token's slot rows
// are loaded first (unfilled slots' rows are read and ignored); lane j < k
// then reads slot j's expert index and a ballot makes the filled-slot mask,
// so every load shares one round trip.  KS >= k slots are loaded.
template <int KS>
__device__ __forceinline__ void combine_token(const FfnArgs& a) {
    const int i = blockIdx.y, k = a.k, lane = threadIdx.x;
    const int o = (blockIdx.x * kWave + lane) * 4;
    const float* d0 = a.dbuf + static_cast<size_t>(i) * k * a.H + (o < a.H ? o : a.H - 4);
    float4 d[KS];
#pragma unroll
    for (int j = 0; j < KS; ++j)
        d[j] = *reinterpret_cast<const float4*>(d0 + static_cast<size_t>(j < k ? j : k - 1) * a.H);
    const int32_t* idx = a.idx + static_cast<size_t>(i) * k;
    const uint64_t filled = __ballot(lane < k && idx[lane < k ? lane : 0] >= 0);
    if (o >= a.H) return;
    float4 s = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
    for (int j = 0; j < KS; ++j) {
        const bool f = (filled >> j) & 1;   // bit j is clear for j >= k
        s.x = f ? s.x + d[j].x : s.x;
        s.y = f ? s.y + d[j].y : s.y;
        s.z = f ? s.z + d[j].z : s.z;
        s.w = f ? s.w + d[j].w : s.w;
    }
    *reinterpret_cast<float4*>(a.y + static_cast<size_t>(i) * a.H + o) = s;
}

__global__ __launch_bounds__(kWave) void combine_kernel(FfnArgs a) {
    static_assert(kMaxTopK <= 16, "combine loads at most 16 slots");
    if (a.k <= 8) combine_token<8>(a);
    else combine_token<16>(a);
}

int g_num_cus[64] = {0};

}  // namespace

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

namespace {

size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

// The allocation-free entry point's workspace: one copy per device, held
// until the process ends.  In host code `scratch` names a host-side stand-in,
// not device memory: its device address comes from hipGetSymbolAddress, per
// device, and only that address is ever passed to a kernel.
static __device__ __align__(256) char scratch[MOE_FFN_NOALLOC_WORKSPACE_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {nullptr};

}  // namespace

// Device address of the current device's `scratch`, looked up on the first
// call on that device (with that device current) and kept.
hipError_t ffn_noalloc_workspace(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr || reinterpret_cast<uintptr_t>(p) % 256 != 0) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

// The partition sums item costs in 32-bit integers on the device.  Whatever
// the formats in the handle table, an expert with c tokens has at most
// c / pass_tokens + 1 passes and sum(c) <= B k, which bounds the total.  At
// the largest accepted sizes (B = 128, k = 16, H = I = 16384) the bound is
// about 2.01e9, so the check is a guard for future limits.
bool ffn_cost_fits(int B, int k, int N, int H, int I) {
    long long worst = 0;
    for (int phase = 0; phase < 2; ++phase) {
        const int rows = phase == 0 ? I : H, cols = phase == 0 ? H : I;
        for (int nt = 1; nt <= 2; ++nt) {
            const int rb = rb_per_item(phase, nt);
            const long long ipp = (rows / 16 + rb - 1) / rb;
            for (int fmt : {MOE_W_F32, MOE_W_BF16, MOE_W_INT4_G128}) {
                const long long tiles = static_cast<long long>(rb) * (weight_row_bytes(fmt, cols) / 64);
                const long long per_tile = fmt == MOE_W_INT4_G128 ? 14 : 10;
                const long long passes = static_cast<long long>(B) * k / pass_tokens(fmt) + N;
                worst = std::max(worst, passes * ipp * tiles * per_tile);
            }
        }
    }
    return worst < (1LL << 31);
}

// Workspace: SwiGLU activations [B*k, I] (4 bytes per value: fp32, or the
// split bf16 hi/lo form), then weighted down projections [B*k, H] fp32.
size_t ffn_workspace_bytes(int B, int k, int H, int I) {
    const size_t pairs = static_cast<size_t>(B) * k;
    return align256(pairs * I * sizeof(float)) + align256(pairs * H * sizeof(float));
}

hipError_t launch_expert_ffn(const FfnArgs& in, void* ws, hipStream_t s, hipEvent_t const* ev) {
    auto mark = [&](int i) { return ev != nullptr && ev[i] != nullptr ? hipEventRecord(ev[i], s) : hipSuccess; };
    FfnArgs a = in;
    const size_t pairs = static_cast<size_t>(a.B) * a.k;
    char* p = static_cast<char*>(ws);
    a.hbuf = reinterpret_cast<float*>(p);
    a.dbuf = reinterpret_cast<float*>(p + align256(pairs * a.I * sizeof(float)));
    hipError_t e = mark(0);
    if (e != hipSuccess) return e;
    if (pairs <= static_cast<size_t>(kSmallPairs)) {
        // one workgroup per (slot, item) for every slot that T can reach
        const int slots = std::min(static_cast<int>(pairs), a.N);
        ffn_small_kernel<0><<<slots * ((a.I / 16 + small_rb<0>() - 1) / small_rb<0>()), kSmallThreads, 0, s>>>(a);
        if ((e = hipGetLastError()) != hipSuccess || (e = mark(1)) != hipSuccess) return e;
        ffn_small_kernel<1><<<slots * ((a.H / 16 + small_rb<1>() - 1) / small_rb<1>()), kSmallThreads, 0, s>>>(a);
        if ((e = hipGetLastError()) != hipSuccess || (e = mark(2)) != hipSuccess) return e;
    } else {
        const int cus = device_cus();
        // grids are whole multiples of kXcds workgroups (the virtual numbering needs it)
        const int g0 = (waves_per_simd<0>() * cus) / kXcds * kXcds;
        const int g1 = (waves_per_simd<1>() * cus) / kXcds * kXcds;
        ffn_kernel<0><<<g0 > 0 ? g0 : kXcds, kThreads, 0, s>>>(a);
        if ((e = hipGetLastError()) != hipSuccess || (e = mark(1)) != hipSuccess) return e;
        ffn_kernel<1><<<g1 > 0 ? g1 : kXcds, kThreads, 0, s>>>(a);
        if ((e = hipGetLastError()) != hipSuccess || (e = mark(2)) != hipSuccess) return e;
    }
    dim3 cg((a.H / 4 + kWave - 1) / kWave, a.B);
    combine_kernel<<<cg, kWave, 0, s>>>(a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return mark(3);
}

}  // namespace moe
