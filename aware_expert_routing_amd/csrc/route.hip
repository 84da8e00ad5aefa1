// Router logits, vanilla top-k / OEA routing, dispatch and the hotness score.
//
// Page "Opportunistic Expert Activation (OEA) - L2":
//   section 2 Q1   router top-k of N experts per token;
//   section 2 Q2   OEA Phase 1 (top-n_i baseline, n_i = min(k0, t_i), t_i an
//                  adaptive top-p count), the union S_base, Phase 2 piggyback
//                  of experts already in S_base, renormalised scores;
//   section 3      Algorithm 1 flow: a candidate is kept only if it is a member of S_base;
//   section 4      Eq. 2: cnt_i per expert and T = #{i : cnt_i > 0}.
// Page "DynaExq" section 2.5: hotness score S <- alpha S + (1 - alpha) c.
//
// Layout on the GPU: one row of 16 lanes per token (four tokens per
// wavefront); lane l of a row owns experts 8l .. 8l+7 (N <= 128).  A
// selection step is a lane-local maximum over 8 keys and a 4-step DPP
// maximum inside the row, so the four tokens of a wavefront select together;
// the softmax normaliser is a 3-level lane-local tree followed by 4 DPP
// levels, the balanced pairwise tree over 128 slots.  S_base is a 128-bit
// set in LDS built with integer OR, so its value does not depend on the
// order in which tokens finish.
//
// Floating-point contraction is off in this file: the top-p decision must be
// reproducible bit for bit, so every fused multiply-add is written out.
#pragma clang fp contract(off)

#include "internal.h"

namespace moe {
namespace {

constexpr int kWave = 64;

// Exponential used for routing decisions: Cody-Waite reduction
// x = n ln2 + r with ln 2 split into a 16-significant-bit head (so n * head is
// exact for |n| < 256) and an fp32 tail, then a degree-7 Taylor polynomial
// for e^r evaluated by Horner's rule with fused multiply-adds, then scaling by
// 2^n through the exponent field.  Inputs are l - max(l) <= 0; below -80 the
// result is 0, so no subnormal appears.
__device__ __forceinline__ float route_exp(float x) {
    if (x < -80.0f) return 0.0f;
    const float inv_ln2 = 1.44269504088896341f;
    const float ln2_head = 0.693145751953125f;
    const float ln2_tail = 1.42860682030941723e-6f;
    float n = __builtin_rintf(x * inv_ln2);
    float r = __builtin_fmaf(-n, ln2_head, x);
    r = __builtin_fmaf(-n, ln2_tail, r);
    float q = 1.0f / 5040.0f;
    q = __builtin_fmaf(q, r, 1.0f / 720.0f);
    q = __builtin_fmaf(q, r, 1.0f / 120.0f);
    q = __builtin_fmaf(q, r, 1.0f / 24.0f);
    q = __builtin_fmaf(q, r, 1.0f / 6.0f);
    q = __builtin_fmaf(q, r, 0.5f);
    q = __builtin_fmaf(q, r, 1.0f);
    q = __builtin_fmaf(q, r, 1.0f);
    int ni = static_cast<int>(n);
    return q * __int_as_float((ni + 127) << 23);
}

// Rank order is (logit descending, expert index ascending).  A lane holds its
// two candidates as 32-bit order keys: the logit's bits mapped to an
// order-preserving unsigned value (-0 is folded to +0 first, so equal logits
// compare equal as floats do); key 0 means "no candidate" (no finite or
// infinite logit maps to 0).  The index tie-break is taken separately: among
// the lanes holding the maximum key the lowest lane wins, and inside a lane
// expert 2l comes before 2l+1.
__device__ __forceinline__ uint32_t order_key(float l) {
    const uint32_t b = __float_as_uint(l == 0.0f ? 0.0f : l);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_logit(uint32_t o) {
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

// DPP cross-lane moves (all 64 lanes active).  Row masks select which rows of
// 16 lanes receive the moved value; the others keep `old`.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t dpp32(uint32_t old, uint32_t v) {
    return static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(static_cast<int>(old), static_cast<int>(v), CTRL, ROWS, 0xF, false));
}
constexpr int kQuadXor1 = 0xB1, kQuadXor2 = 0x4E, kHalfMirror = 0x141, kMirror = 0x140;

constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;

template <int CTRL>
__device__ __forceinline__ double dpp_move_f64(double v) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const int lo = __builtin_amdgcn_mov_dpp(static_cast<int>(b), CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_mov_dpp(static_cast<int>(b >> 32), CTRL, 0xF, 0xF, false);
    return __builtin_bit_cast(double, (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) | static_cast<uint32_t>(lo));
}
__device__ __forceinline__ double lane_f64(double v, int l) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(b), l));
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(b >> 32), l));
    return __builtin_bit_cast(double, (static_cast<uint64_t>(hi) << 32) | lo);
}

// A token is handled by a group of G lanes: G = 64 (a whole wavefront, two
// experts per lane; the lowest latency, for small batches) or G = 16 (a row,
// eight experts per lane, four tokens per wavefront; for large batches).
// Lane l of a group owns experts kPer l .. kPer l + kPer - 1.  Reductions
// give their result in every lane of the group.
template <int G>
struct Grp;

// max(v, v moved by a DPP control): 0 is the identity of the unsigned max,
// so lanes a move does not reach (and rows the mask leaves out) keep v, and
// the move folds into the max instruction itself (one v_max_u32 with DPP).
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t max_dpp(uint32_t v) {
    return max(v, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, ROWS, 0xF, true)));
}

template <>
struct Grp<16> {
    static constexpr int kPer = kMaxExperts / 16;
    static constexpr int kPerWave = kWave / 16;
    static constexpr int kRounds = kMaxBatch / (16 * kPerWave);   // 16 wavefronts cover 128 tokens
    __device__ static uint32_t max_u32(uint32_t v) {
        v = max_dpp<kQuadXor1, 0xF>(v);
        v = max_dpp<kQuadXor2, 0xF>(v);
        v = max_dpp<kHalfMirror, 0xF>(v);
        v = max_dpp<kMirror, 0xF>(v);
        return v;
    }
    // levels 4..7 of the balanced tree over 128 slots: lane pairs, quads, half rows, rows
    __device__ static float tree_sum(float x) {
        uint32_t s = __float_as_uint(x);
        s = __float_as_uint(__uint_as_float(s) + __uint_as_float(dpp32<kQuadXor1, 0xF>(s, s)));
        s = __float_as_uint(__uint_as_float(s) + __uint_as_float(dpp32<kQuadXor2, 0xF>(s, s)));
        s = __float_as_uint(__uint_as_float(s) + __uint_as_float(dpp32<kHalfMirror, 0xF>(s, s)));
        s = __float_as_uint(__uint_as_float(s) + __uint_as_float(dpp32<kMirror, 0xF>(s, s)));
        return __uint_as_float(s);
    }
    __device__ static double sum_f64(double v) {
        v += dpp_move_f64<kQuadXor1>(v);
        v += dpp_move_f64<kQuadXor2>(v);
        v += dpp_move_f64<kHalfMirror>(v);
        v += dpp_move_f64<kMirror>(v);
        return v;
    }
    // lowest lane (group-relative) whose ballot bit is set, -1 if none
    __device__ static int lowest(uint64_t ballot) {
        const int row0 = (threadIdx.x & (kWave - 1)) & ~15;
        return __ffs(static_cast<uint32_t>(ballot >> row0) & 0xFFFFu) - 1;
    }
};

template <>
struct Grp<64> {
    static constexpr int kPer = kMaxExperts / 64;
    static constexpr int kPerWave = 1;
    static constexpr int kRounds = 1;   // B <= 16 tokens, one per wavefront
    __device__ static uint32_t max_u32(uint32_t v) {
        v = Grp<16>::max_u32(v);
        v = max_dpp<kRowBcast15, 0xA>(v);   // rows 1, 3 take rows 0, 2
        v = max_dpp<kRowBcast31, 0xC>(v);   // rows 2, 3 take row 1
        return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
    }
    // levels 2..7 of the balanced tree: as Grp<16>, then row pairs, then the halves
    __device__ static float tree_sum(float x) {
        uint32_t s = __float_as_uint(Grp<16>::tree_sum(x));
        s = __float_as_uint(__uint_as_float(s) + __uint_as_float(dpp32<kRowBcast15, 0xA>(s, s)));   // rows 1, 3
        s = __float_as_uint(__uint_as_float(s) + __uint_as_float(dpp32<kRowBcast31, 0xC>(s, s)));   // row 3
        return __uint_as_float(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(s), 63)));
    }
    __device__ static double sum_f64(double v) {
        v = Grp<16>::sum_f64(v);
        return (lane_f64(v, 0) + lane_f64(v, 16)) + (lane_f64(v, 32) + lane_f64(v, 48));
    }
    __device__ static int lowest(uint64_t ballot) {
        return __ffsll(static_cast<unsigned long long>(ballot)) - 1;
    }
};

// Lane-local maximum and the lane's level-1..3 (or level-1) tree sum.
template <int P>
__device__ __forceinline__ uint32_t lane_max(const uint32_t (&k)[P]) {
    if constexpr (P == 8) return max(max(max(k[0], k[1]), max(k[2], k[3])), max(max(k[4], k[5]), max(k[6], k[7])));
    else return max(k[0], k[1]);
}
template <int P>
__device__ __forceinline__ float lane_tree_sum(const float (&v)[P]) {
    if constexpr (P == 8) return ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
    else return v[0] + v[1];
}

// One token per group.  Each lane keeps its experts' logits, keys and slots.
template <int P>
struct Tok {
    float l[P];
    uint32_t key[P];   // order keys still selectable (0 = none)
    int slot[P];       // rank slot of a selected expert, else -1
};

// Select the group's experts of ranks r0 .. count-1 in rank order (count is
// per group; a group with active == false selects nothing).  The owner lane
// of the r-th selection records r in slot[] and clears the key: the lowest
// lane holding the maximum key wins, and inside a lane the lowest expert, so
// ties go to the lower expert index.  Returns the number selected; top_key
// holds the first selected key (set by the caller when r0 > 0).  With p_z > 0
// a group also stops after the first rank at which the running sum of
// exp(l - l_top) in rank order (fp32, one addition per rank) reaches p_z
// (the top-p count).  The loop ends when every group of the wavefront is done.
template <int G, bool kTopP>
__device__ __forceinline__ int group_select(Tok<Grp<G>::kPer>& t, bool active, int r0, int count, uint32_t& top_key,
                                            float p_z) {
    constexpr int P = Grp<G>::kPer;
    const int l = threadIdx.x & (G - 1);
    if constexpr (G == 64) {
        // One token per wavefront: every condition is uniform, so the loop
        // runs on scalar registers and only the owner lane's update is a
        // per-lane select.
        if (!__builtin_amdgcn_readfirstlane(static_cast<int>(active))) return r0;
        int got = r0;
        float c = 0.0f, top = 0.0f;
        const int end = min(count, kMaxTopK);
        for (int r = r0; r < end; ++r) {
            const uint32_t lmax = max(t.key[0], t.key[1]);
            const uint32_t m = Grp<64>::max_u32(lmax);
            if (m == 0u) break;
            const int owner = __ffsll(static_cast<unsigned long long>(__ballot(lmax == m))) - 1;
            const bool mine = l == owner;
            const bool first = t.key[0] == m;
            t.key[0] = (mine && first) ? 0u : t.key[0];
            t.slot[0] = (mine && first) ? r : t.slot[0];
            t.key[1] = (mine && !first) ? 0u : t.key[1];
            t.slot[1] = (mine && !first) ? r : t.slot[1];
            got = r + 1;
            if (r == 0) {
                top_key = m;
                top = key_logit(m);
            }
            if constexpr (kTopP) {
                c = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(c + route_exp(key_logit(m) - top))));
                if (c >= p_z) break;
            }
        }
        return got;
    }
    int got = r0;
    bool live = active;
    float c = 0.0f, top = 0.0f;
    for (int r = r0; r < kMaxTopK; ++r) {
        const uint32_t lmax = lane_max<P>(t.key);
        const uint32_t m = Grp<G>::max_u32(lmax);
        const bool act = live && r < count && m != 0u;
        if (!__any(act)) break;
        const bool mine = act && l == Grp<G>::lowest(__ballot(act && lmax == m));
        // the owner's lowest expert holding m: clear it and record its rank
        bool hit = false;
#pragma unroll
        for (int j = 0; j < P; ++j) {
            const bool take = mine && !hit && t.key[j] == m;
            hit = hit || take;
            t.key[j] = take ? 0u : t.key[j];
            t.slot[j] = take ? r : t.slot[j];
        }
        got = act ? r + 1 : got;
        if (r == 0) {
            top_key = m;
            top = key_logit(m);
        }
        if constexpr (kTopP) {
            const float cn = c + route_exp(key_logit(m) - top);
            c = act ? cn : c;
            live = live && !(act && cn >= p_z);
        }
    }
    return got;
}

// Write one token's selected experts: the lane owning the expert of slot r
// writes idx[i k + r] and w[i k + r] = e / denom, e = exp(l - l_top); denom is
// the sum of e over the kept experts (renorm) or Z (raw softmax), formed in
// double as e times the double reciprocal of denom (one division per lane)
// and rounded once to fp32.  Slots got..k-1 get expert -1 and weight 0.
template <int G>
__device__ __forceinline__ void group_write(const Tok<Grp<G>::kPer>& t, int i, int k, int got, float top, bool renorm,
                                            float Z, int32_t* idx, float* w, int32_t* idx_copy) {
    constexpr int P = Grp<G>::kPer;
    const int l = threadIdx.x & (G - 1);
    double ev[P];
    double loc = 0.0;
#pragma unroll
    for (int j = 0; j < P; ++j) {
        ev[j] = t.slot[j] >= 0 ? static_cast<double>(route_exp(t.l[j] - top)) : 0.0;
        loc += ev[j];
    }
    const double denom = renorm ? Grp<G>::sum_f64(loc) : static_cast<double>(Z);
    const double inv = 1.0 / denom;
#pragma unroll
    for (int j = 0; j < P; ++j) {
        if (t.slot[j] < 0) continue;
        const int q = i * k + t.slot[j];
        idx[q] = P * l + j;
        if (idx_copy != nullptr) idx_copy[q] = P * l + j;
        w[q] = static_cast<float>(ev[j] * inv);
    }
    if (l >= got && l < k) {
        idx[i * k + l] = -1;
        if (idx_copy != nullptr) idx_copy[i * k + l] = -1;
        w[i * k + l] = 0.0f;
    }
}

// Key and expert of the group's kth-ranked expert (kth >= 1; with fewer
// candidates, the last one), by kth selections over copies of the keys.
template <int G>
__device__ __forceinline__ void group_kth(const uint32_t (&key_in)[Grp<G>::kPer], bool active, int kth, uint32_t& th,
                                          int& eth) {
    constexpr int P = Grp<G>::kPer;
    const int lane = threadIdx.x & (kWave - 1);
    const int l = lane & (G - 1);
    const int g0 = lane - l;
    uint32_t key[P];
#pragma unroll
    for (int j = 0; j < P; ++j) key[j] = key_in[j];
    th = 0u;
    eth = -1;
    for (int r = 0; r < kMaxExperts; ++r) {
        const uint32_t lmax = lane_max<P>(key);
        const uint32_t m = Grp<G>::max_u32(lmax);
        const bool act = active && r < kth && m != 0u;
        if (!__any(act)) break;
        const int L = Grp<G>::lowest(__ballot(act && lmax == m));
        const bool mine = act && l == L;
        int jsel = P;
#pragma unroll
        for (int j = P - 1; j >= 0; --j)
            if (key[j] == m) jsel = j;
#pragma unroll
        for (int j = 0; j < P; ++j)
            if (mine && j == jsel) key[j] = 0u;
        const int jgrp = __shfl(jsel, g0 + (L >= 0 ? L : 0), kWave);   // the owner's choice
        if (act) {
            th = m;
            eth = P * L + jgrp;
        }
    }
}

// Dispatch of one workgroup: histogram, exclusive scan, (expert, token)-
// ordered permutation and the active list.  A token's position inside its
// expert's bucket is the number of lower-numbered tokens routed to the same
// expert, read off a per-expert token bitmask, so the result needs no
// ordering of atomics.  `idx` may live in LDS or in global memory.
// The dispatch's LDS: per-expert counts and token bitmasks, then offsets.
struct DispLds {
    int cnt[kMaxExperts];
    int off[kMaxExperts + 1];
    unsigned long long tokmask[kMaxExperts][kMaxBatch / 64];
};
__device__ __forceinline__ void disp_clear(DispLds& d) {
    for (int e = threadIdx.x; e < kMaxExperts; e += blockDim.x) {
        d.cnt[e] = 0;
        d.tokmask[e][0] = 0ull;
        d.tokmask[e][1] = 0ull;
    }
}
// Count the routed pair (token t, expert e) (e valid).
__device__ __forceinline__ void disp_add(DispLds& d, int t, int e) {
    atomicAdd(&d.cnt[e], 1);
    atomicOr(&d.tokmask[e][t >> 6], 1ull << (t & 63));
}

// kCounted: the caller cleared d and counted every pair with disp_add (and
// synchronised the workgroup after); otherwise this function does both.
template <bool kCounted = false>
__device__ __forceinline__ void dispatch_block(const int32_t* idx, int B, int N, int k, int32_t* cnt,
                                               int32_t* offsets, int32_t* perm, int32_t* active,
                                               int32_t* T_out, DispLds& d) {
    int* const cnt_s = d.cnt;
    int* const off_s = d.off;
    const int tid = threadIdx.x;
    const int pairs = B * k;
    if constexpr (!kCounted) {
        disp_clear(d);
        __syncthreads();
        for (int q = tid; q < pairs; q += blockDim.x) {
            const int e = idx[q];
            if (e >= 0 && e < N) disp_add(d, q / k, e);
        }
        __syncthreads();
    }
    if (tid < kWave) {
        const int lane = tid;
        const int c0 = 2 * lane < N ? cnt_s[2 * lane] : 0;
        const int c1 = 2 * lane + 1 < N ? cnt_s[2 * lane + 1] : 0;
        int sum = c0 + c1;
        int act = (c0 > 0) + (c1 > 0);
        sum = wave_incl_scan(sum);   // inclusive scans over lanes
        act = wave_incl_scan(act);
        const int excl = sum - (c0 + c1);
        const int aexcl = act - ((c0 > 0) + (c1 > 0));
        if (2 * lane < N) {
            off_s[2 * lane] = excl;
            offsets[2 * lane] = excl;
            cnt[2 * lane] = c0;
        }
        if (2 * lane + 1 < N) {
            off_s[2 * lane + 1] = excl + c0;
            offsets[2 * lane + 1] = excl + c0;
            cnt[2 * lane + 1] = c1;
        }
        const int total = __builtin_amdgcn_readlane(sum, kWave - 1);
        const int tact = __builtin_amdgcn_readlane(act, kWave - 1);
        if (lane == 0) {
            off_s[N] = total;
            offsets[N] = total;
            *T_out = tact;
        }
        int pos = aexcl;   // active list, ascending, then -1
        if (2 * lane < N && c0 > 0) active[pos++] = 2 * lane;
        if (2 * lane + 1 < N && c1 > 0) active[pos++] = 2 * lane + 1;
        for (int e = tact + lane; e < N; e += kWave) active[e] = -1;
    }
    __syncthreads();
    const int total = off_s[N];
    for (int q = tid; q < pairs; q += blockDim.x) {
        const int e = idx[q];
        if (e >= 0 && e < N) {
            const int t = q / k;
            const unsigned long long lo = d.tokmask[e][0], hi = d.tokmask[e][1];
            const int below = t < 64 ? __popcll(lo & ((1ull << t) - 1ull))
                                     : __popcll(lo) + __popcll(hi & ((1ull << (t - 64)) - 1ull));
            perm[off_s[e] + below] = q;
        }
        if (q >= total) perm[q] = -1;
    }
}

template <bool kCoherent>
__device__ __forceinline__ float load_logit(const float* p) {
    if constexpr (kCoherent) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else return *p;
}
// Two adjacent logits (p 8-byte aligned) in one load.
template <bool kCoherent>
__device__ __forceinline__ void load_logit2(const float* p, float& a, float& b) {
    uint64_t v;
    if constexpr (kCoherent)
        v = __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
        v = *reinterpret_cast<const uint64_t*>(p);
    a = __uint_as_float(static_cast<uint32_t>(v));
    b = __uint_as_float(static_cast<uint32_t>(v >> 32));
}

// The routing of a whole batch by the calling workgroup, one token per group
// of G lanes: token i = kPerWave (wave + r nwaves) + group.  The launch has
// enough wavefronts for Grp<G>::kRounds rounds.  Every lane first loads the
// logits of its experts for all of its tokens (one round trip) and keeps
// them in registers; Phase 2 continues from Phase 1's selections.
// kCoherent: the logits were written by other workgroups of the same launch
// and are read with device-scope loads.
template <bool kOea, bool kDispatch, bool kCoherent, int G>
__device__ __forceinline__ void route_block(const float* __restrict__ logits, int B, int N, int k, int k0, float p,
                                            int renorm, int32_t* __restrict__ idx, float* __restrict__ w,
                                            int32_t* __restrict__ n_base, uint32_t* __restrict__ mask_out,
                                            int32_t* __restrict__ T_out, int32_t* __restrict__ cnt,
                                            int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
                                            int32_t* __restrict__ active, int pruned, int max_p,
                                            const int32_t* __restrict__ n_valid,
                                            const int32_t* __restrict__ k0_by_batch) {
    using Gr = Grp<G>;
    constexpr int P = Gr::kPer;
    constexpr int R = Gr::kRounds;
    __shared__ uint32_t sbase[kMaxExperts / 32];
    __shared__ int32_t idx_l[kDispatch ? kMaxBatch * kMaxTopK : 1];
    __shared__ DispLds disp_l;   // with dispatch: pairs are counted as they are written
    // tokens at or past n_valid are padding: no experts, nothing added to S_base
    const int B_real = n_valid != nullptr ? min(max(*n_valid, 0), B) : B;
    // batch-size-dependent k0, looked up on the device from the real batch size
    if (kOea && k0_by_batch != nullptr) k0 = min(max(k0_by_batch[B_real], 1), k);
    const int lane = threadIdx.x & (kWave - 1);
    const int l = lane & (G - 1);
    const int wave = threadIdx.x / kWave;
    const int nwaves = blockDim.x / kWave;
    const int e_first = P * l;
    if (threadIdx.x < kMaxExperts / 32) sbase[threadIdx.x] = 0u;
    if constexpr (kDispatch) disp_clear(disp_l);

    float L[R][P];
    if ((N & 1) == 0) {   // every lane's experts come in 8-byte aligned pairs (e_first and i N are even)
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int i = Gr::kPerWave * (wave + r * nwaves) + lane / G;
#pragma unroll
            for (int j = 0; j < P; j += 2) {
                const int e = e_first + j;
                if (i < B_real && e < N) {
                    load_logit2<kCoherent>(logits + i * N + e, L[r][j], L[r][j + 1]);
                } else {
                    L[r][j] = kNegInf;
                    L[r][j + 1] = kNegInf;
                }
            }
        }
    } else {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int i = Gr::kPerWave * (wave + r * nwaves) + lane / G;
#pragma unroll
            for (int j = 0; j < P; ++j) {
                const int e = e_first + j;
                L[r][j] = (i < B_real && e < N) ? load_logit<kCoherent>(logits + i * N + e) : kNegInf;
            }
        }
    }
    __syncthreads();
    int32_t* idx_copy = kDispatch ? idx_l : nullptr;

    // Vanilla top-k, or OEA Phase 1 (kept in registers for Phase 2).
    Tok<P> tok[R];
    int got1[R];
    uint32_t top1[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        got1[r] = 0;
        top1[r] = 0u;
        const int base = Gr::kPerWave * (wave + r * nwaves);
        if (base >= B) break;   // wave-uniform
        const int i = base + lane / G;
        const bool real = i < B_real;
        Tok<P>& t = tok[r];
#pragma unroll
        for (int j = 0; j < P; ++j) {
            t.l[j] = L[r][j];
            t.key[j] = (real && e_first + j < N) ? order_key(t.l[j]) : 0u;
            t.slot[j] = -1;
        }
        const bool need_z = kOea ? (p < 1.0f) : (renorm == 0);
        float Z = 0.0f;
        if (need_z) {   // normaliser over all experts, relative to the top logit
            const float m = key_logit(Gr::max_u32(lane_max<P>(t.key)));
            float sj[P];
#pragma unroll
            for (int j = 0; j < P; ++j) sj[j] = t.key[j] != 0u ? route_exp(t.l[j] - m) : 0.0f;
            Z = Gr::tree_sum(lane_tree_sum<P>(sj));
        }
        uint32_t top_key = 0u;
        const float p_z = (kOea && p < 1.0f) ? p * Z : 0.0f;
        const int got = p_z > 0.0f ? group_select<G, true>(t, real, 0, kOea ? k0 : k, top_key, p_z)
                                   : group_select<G, false>(t, real, 0, kOea ? k0 : k, top_key, p_z);
        got1[r] = got;
        top1[r] = top_key;
        if (i < B) {
            if (!kOea) {
                group_write<G>(t, i, k, got, key_logit(top_key), renorm != 0, Z, idx, w, idx_copy);
                if constexpr (kDispatch)
#pragma unroll
                    for (int j = 0; j < P; ++j)
                        if (t.slot[j] >= 0) disp_add(disp_l, i, e_first + j);
            } else {
                if (l == 0 && n_base != nullptr) n_base[i] = got;
#pragma unroll
                for (int j = 0; j < P; ++j)
                    if (t.slot[j] >= 0) atomicOr(&sbase[(e_first + j) >> 5], 1u << ((e_first + j) & 31));
            }
        }
    }
    if constexpr (kOea) {
        __syncthreads();
        int T = 0;   // |S_base|, counted by every thread
#pragma unroll
        for (int wd = 0; wd < kMaxExperts / 32; ++wd) T += __popc(sbase[wd]);
        if (threadIdx.x == 0 && T_out != nullptr && !kDispatch) *T_out = T;   // with dispatch, T comes from there
        if (mask_out != nullptr && threadIdx.x < (N + 31) / 32) mask_out[threadIdx.x] = sbase[threadIdx.x];
        const int keep = T < k ? T : k;

        // Phase 2: token i keeps the first min(k, T) members of S_base in its
        // rank order -- its baseline first (already selected: the top-ranked
        // experts are in S_base), then lower-ranked experts that other tokens
        // already activated.  With max_p < N only the token's top-max_p ranks
        // may be taken; pruned keeps the baseline alone (its n_i experts).
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int base = Gr::kPerWave * (wave + r * nwaves);
            if (base >= B) break;
            const int i = base + lane / G;
            const bool real = i < B_real;
            Tok<P>& t = tok[r];
            uint32_t th = 0u;
            int eth = kMaxExperts;
            if (!pruned && max_p < N) {
                uint32_t full[P];
#pragma unroll
                for (int j = 0; j < P; ++j) full[j] = (real && e_first + j < N) ? order_key(t.l[j]) : 0u;
                group_kth<G>(full, real, max_p, th, eth);
            }
            // a lane's P experts (P divides 32) share one word of the S_base mask
            const uint32_t sw = sbase[e_first >> 5] >> (e_first & 31);
#pragma unroll
            for (int j = 0; j < P; ++j) {
                const int e = e_first + j;
                bool a = t.key[j] != 0u && ((sw >> j) & 1u);
                if (!pruned && max_p < N) a = a && (t.key[j] > th || (t.key[j] == th && e <= eth));
                if (!a) t.key[j] = 0u;
            }
            uint32_t top_key = top1[r];
            const int count = pruned ? got1[r] : keep;
            const int got = group_select<G, false>(t, real, got1[r], count, top_key, 0.0f);
            if (i < B) {
                group_write<G>(t, i, k, got, key_logit(top_key), true, 0.0f, idx, w, idx_copy);
                if constexpr (kDispatch)
#pragma unroll
                    for (int j = 0; j < P; ++j)
                        if (t.slot[j] >= 0) disp_add(disp_l, i, e_first + j);
            }
        }
    }
    if constexpr (kDispatch) {
        __syncthreads();
        dispatch_block<true>(idx_l, B, N, k, cnt, offsets, perm, active, T_out, disp_l);
    }
}

// Routing of a batch by one workgroup: one wavefront per token for B <= 16
// (G = 64), else one row of 16 lanes per token, four per wavefront, on up to
// 16 wavefronts and two rounds (G = 16).  kOea: OEA
// Phase 1, the union S_base (LDS bitmask built with integer OR, independent
// of the order tokens finish), Phase 2; otherwise vanilla top-k.  kDispatch:
// the same workgroup then dispatches the routed pairs from LDS.
template <bool kOea, bool kDispatch, int G>
__global__ __launch_bounds__(1024) void route_kernel(const float* __restrict__ logits, int B, int N, int k,
                                                     int k0, float p, int renorm, int32_t* __restrict__ idx,
                                                     float* __restrict__ w, int32_t* __restrict__ n_base,
                                                     uint32_t* __restrict__ mask_out, int32_t* __restrict__ T_out,
                                                     int32_t* __restrict__ cnt, int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ perm, int32_t* __restrict__ active,
                                                     int pruned, int max_p, const int32_t* __restrict__ n_valid,
                                                     const int32_t* __restrict__ k0_by_batch) {
    route_block<kOea, kDispatch, false, G>(logits, B, N, k, k0, p, renorm, idx, w, n_base, mask_out, T_out, cnt,
                                           offsets, perm, active, pruned, max_p, n_valid, k0_by_batch);
}

// Dispatch on its own (idx from global memory).
__global__ __launch_bounds__(512) void dispatch_kernel(const int32_t* __restrict__ idx, int B, int N, int k,
                                                       int32_t* __restrict__ cnt, int32_t* __restrict__ offsets,
                                                       int32_t* __restrict__ perm, int32_t* __restrict__ active,
                                                       int32_t* __restrict__ T_out) {
    __shared__ DispLds d;
    dispatch_block(idx, B, N, k, cnt, offsets, perm, active, T_out, d);
}

// Router logits: one workgroup per (expert, group of 16 tokens); its 4 waves split the hidden
// dimension (lane l of wave w owns columns 8l + 512w + 2048i), and every lane
// issues its router-weight and activation loads for a group of 16 tokens at
// once, so the whole product costs about one memory round trip.  Partial sums
// are reduced over the 16 lanes of a row with DPP, then over rows and waves
// through LDS.  fp32 accumulation.
constexpr int kGemvTok = 16;
constexpr int kGemvThreads = 256;

template <typename XT>
__device__ __forceinline__ void load_x8(const XT* x, float (&v)[8]);

template <>
__device__ __forceinline__ void load_x8<float>(const float* x, float (&v)[8]) {
    const float4 a = *reinterpret_cast<const float4*>(x);
    const float4 b = *reinterpret_cast<const float4*>(x + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

template <>
__device__ __forceinline__ void load_x8<uint16_t>(const uint16_t* x, float (&v)[8]) {
    const uint4 a = *reinterpret_cast<const uint4*>(x);
    const uint32_t u[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        v[2 * q] = __uint_as_float(u[q] << 16);
        v[2 * q + 1] = __uint_as_float(u[q] & 0xffff0000u);
    }
}

__device__ __forceinline__ float row16_sum_f(float v) {
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, false));
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xF, 0xF, false));
    return v;
}

// Logits of expert e for tokens t0 .. t0 + nt - 1 by one group of
// kGemvThreads threads (tid = the thread's index in the group): partial sums
// per row of 16 lanes land in part[row][token]; the caller sums the rows.
template <typename XT>
__device__ __forceinline__ void gemv_expert(const XT* __restrict__ x, const float* __restrict__ w_r, int H, int e,
                                            int t0, int nt, int tid, float (*part)[kGemvTok]) {
    // activations stay in their storage format until the multiply (bf16: 4
    // registers per token per 8 columns); fp32 activations go 8 tokens at a time
    constexpr int kGroup = sizeof(XT) == 2 ? kGemvTok : kGemvTok / 2;
    constexpr int kRaw = sizeof(XT) == 2 ? 1 : 2;   // 16-byte chunks per 8 columns
    const int lane = tid & (kWave - 1);
    const int col0 = 8 * lane + 512 * (tid / kWave);     // this lane's first column
    const int stride = 8 * kGemvThreads;                  // 2048 columns per sweep
    const float* wrow = w_r + static_cast<size_t>(e) * H;
    float acc[kGemvTok];
#pragma unroll
    for (int t = 0; t < kGemvTok; ++t) acc[t] = 0.0f;
    for (int c = col0; c < H; c += stride) {
        float wv[8];
        load_x8<float>(wrow + c, wv);
#pragma unroll
        for (int g0 = 0; g0 < kGemvTok; g0 += kGroup) {
            uint4 raw[kGroup][kRaw];
#pragma unroll
            for (int t = 0; t < kGroup; ++t)
                if (g0 + t < nt)
#pragma unroll
                    for (int q = 0; q < kRaw; ++q)
                        raw[t][q] = *reinterpret_cast<const uint4*>(x + static_cast<size_t>(t0 + g0 + t) * H + c +
                                                                     4 * q);
#pragma unroll
            for (int t = 0; t < kGroup; ++t) {
                if (g0 + t >= nt) continue;
                float xv[8];
                if constexpr (sizeof(XT) == 2) {
                    const uint32_t u[4] = {raw[t][0].x, raw[t][0].y, raw[t][0].z, raw[t][0].w};
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        xv[2 * q] = __uint_as_float(u[q] << 16);
                        xv[2 * q + 1] = __uint_as_float(u[q] & 0xffff0000u);
                    }
                } else {
#pragma unroll
                    for (int q = 0; q < 2; ++q) {
                        xv[4 * q] = __uint_as_float(raw[t][q].x);
                        xv[4 * q + 1] = __uint_as_float(raw[t][q].y);
                        xv[4 * q + 2] = __uint_as_float(raw[t][q].z);
                        xv[4 * q + 3] = __uint_as_float(raw[t][q].w);
                    }
                }
#pragma unroll
                for (int q = 0; q < 8; ++q) acc[g0 + t] = __builtin_fmaf(wv[q], xv[q], acc[g0 + t]);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < kGemvTok; ++t) {
        const float sum = row16_sum_f(acc[t]);
        if ((tid & 15) == 0) part[tid / 16][t] = sum;
    }
}

template <typename XT>
__global__ __launch_bounds__(kGemvThreads) void router_logits_kernel(const XT* __restrict__ x,
                                                                     const float* __restrict__ w_r,
                                                                     int B, int H, int N,
                                                                     float* __restrict__ logits) {
    __shared__ float part[kGemvThreads / 16][kGemvTok];   // [row of 16 lanes][token]
    const int e = blockIdx.x;
    const int tid = threadIdx.x;
    for (int t0 = blockIdx.y * kGemvTok; t0 < B; t0 += gridDim.y * kGemvTok) {
        const int nt = min(kGemvTok, B - t0);
        gemv_expert<XT>(x, w_r, H, e, t0, nt, tid, part);
        __syncthreads();
        if (tid < nt) {
            float sum = 0.0f;
#pragma unroll
            for (int r = 0; r < kGemvThreads / 16; ++r) sum += part[r][tid];
            logits[static_cast<size_t>(t0 + tid) * N + e] = sum;
        }
        __syncthreads();
    }
}

// Logits of the kE experts e0 .. for tokens t0 + 4 g .. + 3 by group g of
// kGemvThreads threads: each thread multiplies its 8 columns of the kE
// experts' router rows with the same columns of the 4 tokens, so one
// workgroup reads the activations of its 16 tokens once (not once per
// expert).  Each group reads the kE router rows itself, so few experts per
// workgroup keep the bytes through one CU low (two experts and 16 tokens:
// 4 x 16 KB of router rows and 64 KB of activations).  Partial sums per row
// of 16 lanes land in part[row][4 e + t].
template <typename XT, int kE>
__device__ __forceinline__ void gemv_4x4(const XT* __restrict__ x, const float* __restrict__ w_r, int H, int N,
                                         int e0, int t0, int nt, int g, int tid, float (*part)[4 * kE]) {
    constexpr int kT = 4;
    const int lane = tid & (kWave - 1);
    const int col0 = 8 * lane + 512 * (tid / kWave);
    const int stride = 8 * kGemvThreads;
    float acc[kE][kT];
#pragma unroll
    for (int e = 0; e < kE; ++e)
#pragma unroll
        for (int t = 0; t < kT; ++t) acc[e][t] = 0.0f;
    for (int c = col0; c < H; c += stride) {
        float wv[kE][8];
#pragma unroll
        for (int e = 0; e < kE; ++e) {
            if (e0 + e < N) {
                load_x8<float>(w_r + static_cast<size_t>(e0 + e) * H + c, wv[e]);
            } else {
#pragma unroll
                for (int q = 0; q < 8; ++q) wv[e][q] = 0.0f;
            }
        }
#pragma unroll
        for (int t = 0; t < kT; ++t) {
            if (kT * g + t >= nt) continue;
            float xv[8];
            load_x8<XT>(x + static_cast<size_t>(t0 + kT * g + t) * H + c, xv);
#pragma unroll
            for (int e = 0; e < kE; ++e)
#pragma unroll
                for (int q = 0; q < 8; ++q) acc[e][t] = __builtin_fmaf(wv[e][q], xv[q], acc[e][t]);
        }
    }
#pragma unroll
    for (int e = 0; e < kE; ++e)
#pragma unroll
        for (int t = 0; t < kT; ++t) {
            const float sum = row16_sum_f(acc[e][t]);
            if ((tid & 15) == 0) part[tid / 16][kT * e + t] = sum;
        }
}

// Router logits, routing and dispatch in one launch.  Workgroup (gx, gy)
// computes the logits of experts kFusedExperts gx .. + kFusedExperts - 1 for
// tokens 16 gy .. 16 gy + 15 (group g of kFusedGroups groups of kGemvThreads
// threads takes tokens 4 g .. 4 g + 3 of those experts), writes them with
// device-scope stores, waits for those stores and counts itself done.  The workgroup that completes the
// count routes and dispatches the whole batch (its 16 wavefronts, one token
// per wavefront at a time), reading the logits with device-scope loads, and
// clears the count for the next call.  No workgroup waits for another.
constexpr int kFusedGroups = 4;    // thread groups per workgroup, 4 tokens each
// Experts per workgroup: 2 while the grid of (N/2) x (B/16) workgroups fits
// the chip in one round (B <= 64: 256 workgroups; one 1024-thread workgroup
// per CU at this kernel's register use), 4 for larger batches, which would
// otherwise take two rounds.
constexpr int kFusedMaxB2 = 64;

__device__ __forceinline__ void wait_vmem() {   // s_waitcnt vmcnt(0)
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

template <typename XT, bool kOea, int G, int kFusedExperts>
__global__ __launch_bounds__(kGemvThreads * kFusedGroups) void router_route_kernel(
        const XT* __restrict__ x, const float* __restrict__ w_r, int B, int H, int N, float* __restrict__ logits,
        int k, int k0, float p, int renorm, int32_t* __restrict__ idx, float* __restrict__ w,
        int32_t* __restrict__ n_base, uint32_t* __restrict__ mask_out, int32_t* __restrict__ T_out,
        int32_t* __restrict__ cnt, int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
        int32_t* __restrict__ active, int pruned, int max_p, const int32_t* __restrict__ n_valid,
        const int32_t* __restrict__ k0_by_batch, int32_t* __restrict__ sync) {
    __shared__ float part[kFusedGroups][kGemvThreads / 16][4 * kFusedExperts];
    __shared__ int last_s;
    static_assert(kFusedGroups * 4 == kGemvTok && kFusedExperts * kGemvTok <= kGemvThreads * kFusedGroups,
                  "gemv_4x4 layout");
    const int g = threadIdx.x / kGemvThreads;
    const int tid = threadIdx.x - g * kGemvThreads;
    const int e0 = blockIdx.x * kFusedExperts;
    const int t0 = blockIdx.y * kGemvTok;
    const int nt = min(kGemvTok, B - t0);
    gemv_4x4<XT, kFusedExperts>(x, w_r, H, N, e0, t0, nt, g, tid, part[g]);
    __syncthreads();
    if (threadIdx.x < kFusedExperts * kGemvTok) {   // (expert, token) = (threadIdx / 16, threadIdx % 16)
        const int el = threadIdx.x / kGemvTok, t = threadIdx.x % kGemvTok;
        if (e0 + el < N && t < nt) {
            float sum = 0.0f;
#pragma unroll
            for (int r = 0; r < kGemvThreads / 16; ++r) sum += part[t / 4][r][4 * el + t % 4];
            __hip_atomic_store(logits + static_cast<size_t>(t0 + t) * N + e0 + el, sum, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    // Hand-off: every wave waits for its logit stores to complete, the
    // workgroup barrier orders them before thread 0's count, and the count is
    // an agent-scope release (publishing this workgroup's logits) and acquire
    // (in the workgroup that completes it, of every other workgroup's logits);
    // the barrier after it passes the acquire on to the routing waves.
    wait_vmem();
    __syncthreads();
    if (threadIdx.x == 0)
        last_s = __hip_atomic_fetch_add(sync, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) ==
                 static_cast<int>(gridDim.x * gridDim.y) - 1;
    __syncthreads();
    if (!last_s) return;
    route_block<kOea, true, true, G>(logits, B, N, k, k0, p, kOea ? 1 : renorm, idx, w, n_base, mask_out, T_out,
                                     cnt, offsets, perm, active, pruned, max_p, n_valid, k0_by_batch);
    if (threadIdx.x == 0) __hip_atomic_store(sync, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Router logits for batches of more than 16 tokens: workgroup (gx, gy)
// computes experts kE gx .. kE gx + kE - 1 for tokens 16 gy .. 16 gy + 15 with
// the fused kernel's layout (four groups of 256 threads, 4 tokens each), so a
// workgroup reads its tokens' activations once for kE experts.  Each logit is
// summed in the same order as in router_logits_kernel and the fused kernel
// (the same column slices per thread, the same trees), so all three give the
// same bits.
template <typename XT, int kE>
__global__ __launch_bounds__(kGemvThreads * kFusedGroups) void router_logits_wide_kernel(
        const XT* __restrict__ x, const float* __restrict__ w_r, int B, int H, int N, float* __restrict__ logits) {
    __shared__ float part[kFusedGroups][kGemvThreads / 16][4 * kE];
    static_assert(kFusedGroups * 4 == kGemvTok && kE * kGemvTok <= kGemvThreads * kFusedGroups, "gemv_4x4 layout");
    const int g = threadIdx.x / kGemvThreads;
    const int tid = threadIdx.x - g * kGemvThreads;
    const int e0 = blockIdx.x * kE;
    const int t0 = blockIdx.y * kGemvTok;
    const int nt = min(kGemvTok, B - t0);
    gemv_4x4<XT, kE>(x, w_r, H, N, e0, t0, nt, g, tid, part[g]);
    __syncthreads();
    if (threadIdx.x < kE * kGemvTok) {   // (expert, token) = (threadIdx / 16, threadIdx % 16)
        const int el = threadIdx.x / kGemvTok, t = threadIdx.x % kGemvTok;
        if (e0 + el < N && t < nt) {
            float sum = 0.0f;
#pragma unroll
            for (int r = 0; r < kGemvThreads / 16; ++r) sum += part[t / 4][r][4 * el + t % 4];
            logits[static_cast<size_t>(t0 + t) * N + e0 + el] = sum;
        }
    }
}

// ---------------------------------------------------------------------------
// Batches of more than kGroupMinBatch (48) tokens with vanilla top-k or
// simplified OEA (no rank limit, not pruned), routed by token groups: workgroup g routes tokens
// 16 g .. 16 g + 15, one token per wavefront as for small batches, so a large
// batch's selections run on B/16 CUs side by side instead of on one.
//   Vanilla top-k: route_group_kernel<false> writes idx and w; the dispatch
//   (dispatch_kernel) follows, or, when the caller passes a completion count
//   (a sync word that is zero on entry), runs in the routing launch's last
//   workgroup.
//   OEA: route_group_kernel<true> runs Phase 1 and leaves each token's
//   baseline in its idx row (slots 0 .. n_i - 1, then -1); in the next
//   launch every workgroup rebuilds S_base from those rows (integer OR in
//   LDS) and runs Phase 2 for its tokens, and the workgroup that completes
//   the count dispatches the batch.  A row that another workgroup has
//   already extended in Phase 2 only adds members of S_base, so the union is
//   the same whichever it reads.
// Every selection depends only on the token's own logits and on S_base, so
// idx, n_base, the mask and T equal the one-workgroup path's bit for bit.
// ---------------------------------------------------------------------------
constexpr int kGroupTok = 16;

// Token i's logits (two experts per lane) and fresh selection state.
template <bool kCoherent>
__device__ __forceinline__ void group_token_load(const float* __restrict__ logits, int i, int N, bool real,
                                                 Tok<2>& t) {
    const int e_first = 2 * (threadIdx.x & (kWave - 1));
    float L[2];
    if ((N & 1) == 0) {
        if (real && e_first < N) load_logit2<kCoherent>(logits + static_cast<size_t>(i) * N + e_first, L[0], L[1]);
        else L[0] = L[1] = kNegInf;
    } else {
#pragma unroll
        for (int j = 0; j < 2; ++j)
            L[j] = (real && e_first + j < N) ? load_logit<kCoherent>(logits + static_cast<size_t>(i) * N + e_first + j)
                                             : kNegInf;
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        t.l[j] = L[j];
        t.key[j] = (real && e_first + j < N) ? order_key(L[j]) : 0u;
        t.slot[j] = -1;
    }
}

// The hand-off after a token-group kernel's writes: every wavefront waits
// for its stores, the barrier orders them before thread 0's count (an
// agent-scope release and, in the workgroup that completes the count,
// acquire), and that workgroup writes S_base (when given) and dispatches the
// batch from idx.  The dispatch writes T to T_out, which may be the count
// itself; with reset the count is stored back to zero afterwards.
__device__ __forceinline__ void group_dispatch_last(int32_t* __restrict__ idx, int B, int N, int k,
                                                    int32_t* __restrict__ count, bool reset,
                                                    int32_t* __restrict__ cnt, int32_t* __restrict__ offsets,
                                                    int32_t* __restrict__ perm, int32_t* __restrict__ active,
                                                    int32_t* __restrict__ T_out, uint32_t* __restrict__ mask_out,
                                                    const uint32_t* sbase) {
    __shared__ int last_s;
    __shared__ int32_t idx_l[kMaxBatch * kMaxTopK];
    __shared__ DispLds disp_l;
    const int tid = threadIdx.x;
    wait_vmem();
    __syncthreads();
    if (tid == 0)
        last_s = __hip_atomic_fetch_add(count, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) ==
                 static_cast<int>(gridDim.x) - 1;
    __syncthreads();
    if (!last_s) return;
    if (mask_out != nullptr && tid < (N + 31) / 32) mask_out[tid] = sbase[tid];
    disp_clear(disp_l);
    __syncthreads();
    for (int q = tid; q < B * k; q += blockDim.x) {   // copy and count the routed pairs
        const int e = idx[q];
        idx_l[q] = e;
        if (e >= 0 && e < N) disp_add(disp_l, q / k, e);
    }
    __syncthreads();
    dispatch_block<true>(idx_l, B, N, k, cnt, offsets, perm, active, T_out, disp_l);
    if (reset && tid == 0) *count = 0;   // the next call's launches come after this one
}

// One token of route_group_kernel: its selection and its writes.
template <bool kOea>
__device__ __forceinline__ void group_route_token(const float* __restrict__ logits, int N, int k, int k0, float p,
                                                  int renorm, int32_t* __restrict__ idx, float* __restrict__ w,
                                                  int32_t* __restrict__ n_base, int i, bool real, int lane) {
    Tok<2> t;
    group_token_load<false>(logits, i, N, real, t);
    const bool need_z = kOea ? (p < 1.0f) : (renorm == 0);
    float Z = 0.0f;
    if (need_z) {   // normaliser over all experts, relative to the top logit
        const float m = key_logit(Grp<64>::max_u32(lane_max<2>(t.key)));
        float sj[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) sj[j] = t.key[j] != 0u ? route_exp(t.l[j] - m) : 0.0f;
        Z = Grp<64>::tree_sum(lane_tree_sum<2>(sj));
    }
    uint32_t top_key = 0u;
    const float p_z = (kOea && p < 1.0f) ? p * Z : 0.0f;
    const int got = p_z > 0.0f ? group_select<64, true>(t, real, 0, kOea ? k0 : k, top_key, p_z)
                               : group_select<64, false>(t, real, 0, kOea ? k0 : k, top_key, p_z);
    if (!kOea) {
        group_write<64>(t, i, k, got, key_logit(top_key), renorm != 0, Z, idx, w, nullptr);
    } else {
#pragma unroll
        for (int j = 0; j < 2; ++j)
            if (t.slot[j] >= 0) idx[i * k + t.slot[j]] = 2 * lane + j;
        if (lane >= got && lane < k) idx[i * k + lane] = -1;
        if (lane == 0 && n_base != nullptr) n_base[i] = got;
    }
}

// Launch: ceil(B / 16) workgroups of 1024 threads.  kOea: Phase 1 and the
// baseline rows (and n_base); else vanilla top-k written in full.  Workgroup
// 0 also clears *T_out, the next launch's completion count (OEA).  Top-k
// with a completion count `count` (zero on entry, left at zero): the
// workgroup that completes it dispatches the batch, as Phase 2 does for OEA.
template <bool kOea>
__global__ __launch_bounds__(1024) void route_group_kernel(const float* __restrict__ logits, int B, int N, int k,
                                                           int k0, float p, int renorm, int32_t* __restrict__ idx,
                                                           float* __restrict__ w, int32_t* __restrict__ n_base,
                                                           int32_t* __restrict__ T_out,
                                                           const int32_t* __restrict__ n_valid,
                                                           const int32_t* __restrict__ k0_by_batch,
                                                           int32_t* __restrict__ count, int32_t* __restrict__ cnt,
                                                           int32_t* __restrict__ offsets, int32_t* __restrict__ perm,
                                                           int32_t* __restrict__ active) {
    const int B_real = n_valid != nullptr ? min(max(*n_valid, 0), B) : B;
    if (kOea && k0_by_batch != nullptr) k0 = min(max(k0_by_batch[B_real], 1), k);
    if (kOea && blockIdx.x == 0 && threadIdx.x == 0) *T_out = 0;
    const int lane = threadIdx.x & (kWave - 1);
    const int i = kGroupTok * blockIdx.x + threadIdx.x / kWave;
    if (!kOea && count != nullptr) {   // every wavefront reaches the hand-off's barriers
        if (i < B) group_route_token<kOea>(logits, N, k, k0, p, renorm, idx, w, n_base, i, i < B_real, lane);
        group_dispatch_last(idx, B, N, k, count, true, cnt, offsets, perm, active, T_out, nullptr, nullptr);
        return;
    }
    if (i >= B) return;   // whole wavefronts; no barrier follows
    group_route_token<kOea>(logits, N, k, k0, p, renorm, idx, w, n_base, i, i < B_real, lane);
}

// OEA Phase 2 of token group blockIdx.x and, in the workgroup that completes
// the count in *T_out, the dispatch of the whole batch (which then writes T
// there).  Launch: ceil(B / 16) workgroups of 1024 threads.
__global__ __launch_bounds__(1024) void route_group_p2_kernel(const float* __restrict__ logits, int B, int N, int k,
                                                              int32_t* __restrict__ idx, float* __restrict__ w,
                                                              uint32_t* __restrict__ mask_out,
                                                              const int32_t* __restrict__ n_valid,
                                                              int32_t* __restrict__ cnt, int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ perm, int32_t* __restrict__ active,
                                                              int32_t* __restrict__ T_out) {
    __shared__ uint32_t sbase[kMaxExperts / 32];
    const int B_real = n_valid != nullptr ? min(max(*n_valid, 0), B) : B;
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    if (tid < kMaxExperts / 32) sbase[tid] = 0u;
    __syncthreads();
    for (int q = tid; q < B * k; q += blockDim.x) {   // the union of every token's baseline
        const int e = idx[q];
        if (e >= 0 && e < N) atomicOr(&sbase[e >> 5], 1u << (e & 31));
    }
    __syncthreads();
    int T = 0;
#pragma unroll
    for (int wd = 0; wd < kMaxExperts / 32; ++wd) T += __popc(sbase[wd]);
    const int keep = T < k ? T : k;
    const int i = kGroupTok * blockIdx.x + tid / kWave;
    if (i < B) {   // whole wavefronts
        const bool real = i < B_real;
        Tok<2> t;
        group_token_load<false>(logits, i, N, real, t);
        // the rank-0 key (the token's largest) and the baseline slots from Phase 1
        uint32_t top_key = Grp<64>::max_u32(lane_max<2>(t.key));
        const int e_first = 2 * lane;
        const int32_t my = lane < k ? idx[i * k + lane] : -1;
        const int got1 = real ? __popcll(__ballot(lane < k && my >= 0)) : 0;   // baselines fill slots 0 .. n_i - 1
        for (int r = 0; r < got1; ++r) {
            const int e = __shfl(my, r, kWave);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                if (e == e_first + j) {
                    t.slot[j] = r;
                    t.key[j] = 0u;
                }
        }
        const uint32_t sw = sbase[e_first >> 5] >> (e_first & 31);
#pragma unroll
        for (int j = 0; j < 2; ++j)
            if (!(t.key[j] != 0u && ((sw >> j) & 1u))) t.key[j] = 0u;
        const int got = group_select<64, false>(t, real, got1, keep, top_key, 0.0f);
        group_write<64>(t, i, k, got, key_logit(top_key), true, 0.0f, idx, w, nullptr);
    }
    // the count is T_out (cleared by the Phase-1 launch); the dispatch then writes T there
    group_dispatch_last(idx, B, N, k, T_out, false, cnt, offsets, perm, active, T_out, mask_out, sbase);
}

__global__ void hotness_kernel(float* S, const int32_t* cnt, int N, float alpha) {
    int e = blockIdx.x * blockDim.x + threadIdx.x;
    if (e < N) S[e] = alpha * S[e] + (1.0f - alpha) * static_cast<float>(cnt[e]);
}

// Interval counters: c += cnt per forward call; at an update S <- alpha S +
// (1 - alpha) c and c <- 0 (a kernel, not a memset, so it may be captured).
__global__ void hotness_accumulate_kernel(int32_t* c, const int32_t* cnt, int N) {
    int e = blockIdx.x * blockDim.x + threadIdx.x;
    if (e < N) c[e] += cnt[e];
}

__global__ void hotness_fold_kernel(float* S, int32_t* c, int N, float alpha) {
    int e = blockIdx.x * blockDim.x + threadIdx.x;
    if (e < N) {
        S[e] = alpha * S[e] + (1.0f - alpha) * static_cast<float>(c[e]);
        c[e] = 0;
    }
}

__global__ void publish_kernel(moe_expert_handle* table, int e, moe_expert_handle h) {
    if (threadIdx.x == 0) table[e] = h;
}

}  // namespace

hipError_t launch_router_logits(const void* x, int x_dtype, const float* w_r, int B, int H, int N,
                                float* logits, hipStream_t s) {
    if (B > kGemvTok) {   // kRlE experts per workgroup, the activations read once for them
        // (2 measured fastest for 32-128 tokens: 4.3-5.9 us at H = 2048 against 5.4-7.6 one expert per workgroup)
        constexpr int kRlE = 2;
        const dim3 wgrid((N + kRlE - 1) / kRlE, (B + kGemvTok - 1) / kGemvTok);
        if (x_dtype == MOE_DT_BF16)
            router_logits_wide_kernel<uint16_t, kRlE><<<wgrid, kGemvThreads * kFusedGroups, 0, s>>>(
                static_cast<const uint16_t*>(x), w_r, B, H, N, logits);
        else
            router_logits_wide_kernel<float, kRlE><<<wgrid, kGemvThreads * kFusedGroups, 0, s>>>(
                static_cast<const float*>(x), w_r, B, H, N, logits);
        return hipGetLastError();
    }
    const dim3 grid(N, (B + kGemvTok - 1) / kGemvTok);   // one workgroup per (expert, 16 tokens)
    if (x_dtype == MOE_DT_BF16)
        router_logits_kernel<uint16_t><<<grid, kGemvThreads, 0, s>>>(static_cast<const uint16_t*>(x), w_r,
                                                                     B, H, N, logits);
    else
        router_logits_kernel<float><<<grid, kGemvThreads, 0, s>>>(static_cast<const float*>(x), w_r, B, H,
                                                                  N, logits);
    return hipGetLastError();
}

// Batches up to kSmallBatch route one token per wavefront, larger ones one
// token per 16-lane row (four per wavefront, at most 16 wavefronts).
constexpr int kSmallBatch = 16;
int route_threads(int B) {
    const int waves = B <= kSmallBatch ? B : (B + Grp<16>::kPerWave - 1) / Grp<16>::kPerWave;
    return kWave * (waves < 16 ? waves : 16);
}

hipError_t launch_route(const float* logits, int B, int N, int k, int k0, float p, int oea,
                        int renorm, int32_t* idx, float* w, int32_t* n_base, uint32_t* mask,
                        int32_t* T, hipStream_t s) {
#define MOE_ROUTE(G_, OEA_)                                                                                      \
    route_kernel<OEA_, false, G_><<<1, route_threads(B), 0, s>>>(                                                \
        logits, B, N, k, OEA_ ? k0 : k, OEA_ ? p : 1.0f, OEA_ ? 1 : renorm, idx, w, OEA_ ? n_base : nullptr,      \
        OEA_ ? mask : nullptr, OEA_ ? T : nullptr, nullptr, nullptr, nullptr, nullptr, 0, N, nullptr, nullptr)
    if (B <= kSmallBatch) {
        if (oea) MOE_ROUTE(64, true);
        else MOE_ROUTE(64, false);
    } else {
        if (oea) MOE_ROUTE(16, true);
        else MOE_ROUTE(16, false);
    }
#undef MOE_ROUTE
    return hipGetLastError();
}

namespace {

// Batches above kGroupMinBatch with vanilla top-k or simplified OEA take the
// token-group kernels (logits already in memory).  Below it one workgroup
// selects faster than a second launch costs: measured at N = 128, k = 8 the
// split is 1-2 us slower at 32 tokens, even at 64 and 7-10 us faster at 128.
constexpr int kGroupMinBatch = 48;
bool route_by_groups(int B, int N, int mode, int max_p) {
    return B > kGroupMinBatch && (mode == MOE_ROUTE_TOPK || (mode == MOE_ROUTE_OEA && max_p >= N));
}

// count: null, or a caller's word that is zero on entry (and left at zero):
// vanilla top-k then dispatches in the routing launch's last workgroup
// instead of a launch of its own.
hipError_t launch_route_groups(const float* logits, int B, int N, int k, int mode, int k0, float p, int renorm,
                               const int32_t* n_valid, const int32_t* k0_by_batch, int32_t* idx, float* w,
                               int32_t* n_base, uint32_t* mask, int32_t* cnt, int32_t* offsets, int32_t* perm,
                               int32_t* active, int32_t* T, int32_t* count, hipStream_t s) {
    const int groups = (B + kGroupTok - 1) / kGroupTok;
    if (mode == MOE_ROUTE_TOPK) {
        route_group_kernel<false><<<groups, kGroupTok * kWave, 0, s>>>(logits, B, N, k, k, 1.0f, renorm, idx, w,
                                                                        nullptr, T, n_valid, nullptr, count, cnt,
                                                                        offsets, perm, active);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess || count != nullptr) return e;
        dispatch_kernel<<<1, 512, 0, s>>>(idx, B, N, k, cnt, offsets, perm, active, T);
        return hipGetLastError();
    }
    route_group_kernel<true><<<groups, kGroupTok * kWave, 0, s>>>(logits, B, N, k, k0, p, 1, idx, w, n_base, T,
                                                                   n_valid, k0_by_batch, nullptr, nullptr, nullptr,
                                                                   nullptr, nullptr);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    route_group_p2_kernel<<<groups, kGroupTok * kWave, 0, s>>>(logits, B, N, k, idx, w, mask, n_valid, cnt, offsets,
                                                               perm, active, T);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_route_dispatch(const float* logits, int B, int N, int k, int mode, int k0, float p, int max_p,
                                 int renorm, const int32_t* n_valid, const int32_t* k0_by_batch, int32_t* idx,
                                 float* w, int32_t* n_base,
                                 uint32_t* mask, int32_t* cnt, int32_t* offsets, int32_t* perm, int32_t* active,
                                 int32_t* T, int32_t* sync, hipStream_t s) {
    if (route_by_groups(B, N, mode, max_p))
        return launch_route_groups(logits, B, N, k, mode, k0, p, renorm, n_valid, k0_by_batch, idx, w, n_base, mask,
                                   cnt, offsets, perm, active, T, sync, s);
    const bool oea = mode != MOE_ROUTE_TOPK;
#define MOE_ROUTE(G_, OEA_)                                                                                      \
    route_kernel<OEA_, true, G_><<<1, route_threads(B), 0, s>>>(                                                 \
        logits, B, N, k, OEA_ ? k0 : k, OEA_ ? p : 1.0f, OEA_ ? 1 : renorm, idx, w, OEA_ ? n_base : nullptr,      \
        OEA_ ? mask : nullptr, T, cnt, offsets, perm, active, OEA_ ? (mode == MOE_ROUTE_PRUNED) : 0,             \
        OEA_ ? max_p : N, n_valid, OEA_ ? k0_by_batch : nullptr)
    if (B <= kSmallBatch) {
        if (oea) MOE_ROUTE(64, true);
        else MOE_ROUTE(64, false);
    } else {
        if (oea) MOE_ROUTE(16, true);
        else MOE_ROUTE(16, false);
    }
#undef MOE_ROUTE
    return hipGetLastError();
}

hipError_t launch_router_route_dispatch(const void* x, int x_dtype, const float* w_r, int B, int H, int N, int k,
                                        int mode, int k0, float p, int max_p, int renorm, const int32_t* n_valid,
                                        const int32_t* k0_by_batch, float* logits, int32_t* idx, float* w,
                                        int32_t* n_base, uint32_t* mask, int32_t* cnt, int32_t* offsets,
                                        int32_t* perm, int32_t* active, int32_t* T, int32_t* sync, hipStream_t s) {
    if (route_by_groups(B, N, mode, mode == MOE_ROUTE_OEA ? max_p : N)) {
        // large batches: the logits in their own launch, then the token-group
        // kernels (top-k dispatches in its routing launch, counting in sync)
        hipError_t e = launch_router_logits(x, x_dtype, w_r, B, H, N, logits, s);
        if (e != hipSuccess) return e;
        return launch_route_groups(logits, B, N, k, mode, k0, p, renorm, n_valid, k0_by_batch, idx, w, n_base, mask,
                                   cnt, offsets, perm, active, T, sync, s);
    }
    const int fe = B <= kFusedMaxB2 ? 2 : 4;
    const dim3 grid((N + fe - 1) / fe, (B + kGemvTok - 1) / kGemvTok);
    const int threads = kGemvThreads * kFusedGroups;
    const bool oea = mode != MOE_ROUTE_TOPK;
    const int pruned = mode == MOE_ROUTE_PRUNED;
    const int mp = mode == MOE_ROUTE_OEA ? max_p : N;
#define MOE_FUSED_E(XT_, G_, OEA_, E_)                                                                          \
    router_route_kernel<XT_, OEA_, G_, E_><<<grid, threads, 0, s>>>(                                             \
        static_cast<const XT_*>(x), w_r, B, H, N, logits, k, OEA_ ? k0 : k, OEA_ ? p : 1.0f, OEA_ ? 1 : renorm,  \
        idx, w, OEA_ ? n_base : nullptr, OEA_ ? mask : nullptr, T, cnt, offsets, perm, active, OEA_ ? pruned : 0,  \
        OEA_ ? mp : N, n_valid, OEA_ ? k0_by_batch : nullptr, sync)
#define MOE_FUSED(XT_, G_, OEA_)                                     \
    do {                                                             \
        if (fe == 2) MOE_FUSED_E(XT_, G_, OEA_, 2);                  \
        else MOE_FUSED_E(XT_, G_, OEA_, 4);                          \
    } while (0)
#define MOE_FUSED_G(XT_)                                  \
    if (B <= kSmallBatch) {                               \
        if (oea) MOE_FUSED(XT_, 64, true);                \
        else MOE_FUSED(XT_, 64, false);                   \
    } else {                                              \
        if (oea) MOE_FUSED(XT_, 16, true);                \
        else MOE_FUSED(XT_, 16, false);                   \
    }
    if (x_dtype == MOE_DT_BF16) {
        MOE_FUSED_G(uint16_t)
    } else {
        MOE_FUSED_G(float)
    }
#undef MOE_FUSED_G
#undef MOE_FUSED
#undef MOE_FUSED_E
    return hipGetLastError();
}

hipError_t launch_dispatch(const int32_t* idx, int B, int N, int k, int32_t* cnt,
                           int32_t* offsets, int32_t* perm, int32_t* active, int32_t* T,
                           hipStream_t s) {
    dispatch_kernel<<<1, 512, 0, s>>>(idx, B, N, k, cnt, offsets, perm, active, T);
    return hipGetLastError();
}

hipError_t launch_hotness_ema(float* S, const int32_t* cnt, int N, float alpha, hipStream_t s) {
    hotness_kernel<<<1, 128, 0, s>>>(S, cnt, N, alpha);
    return hipGetLastError();
}

hipError_t launch_hotness_accumulate(int32_t* c, const int32_t* cnt, int N, hipStream_t s) {
    hotness_accumulate_kernel<<<1, 128, 0, s>>>(c, cnt, N);
    return hipGetLastError();
}

hipError_t launch_hotness_fold(float* S, int32_t* c, int N, float alpha, hipStream_t s) {
    hotness_fold_kernel<<<1, 128, 0, s>>>(S, c, N, alpha);
    return hipGetLastError();
}

hipError_t launch_handle_publish(moe_expert_handle* table, int e, moe_expert_handle h,
                                 hipStream_t s) {
    publish_kernel<<<1, 64, 0, s>>>(table, e, h);
    return hipGetLastError();
}

}  // namespace moe
