// Router logits, vanilla top-k / OEA routing, dispatch and the hotness score.
//
// Page "Opportunistic Expert Activation (OEA) - L2":
//   section 2 Q1   router top-k of N experts per token;
//   section 2 Q2   OEA Phase 1 (top-n_i baseline, n_i = min(k0, t_i), t_i an
//                  adaptive top-p count), the union S_base, Phase 2 piggyback
//                  of experts already in S_base, renormalised scores;
//   section 3      Algorithm 1 flow: the "if e_ij in S_base" gate;
//   section 4      Eq. 2: cnt_i per expert and T = #{i : cnt_i > 0}.
// Page "DynaExq" section 2.5: hotness score S <- alpha S + (1 - alpha) c.
//
// Layout on the GPU: one wavefront per token, lane l owns experts 2l and 2l+1
// (N <= 128), so the softmax normaliser is an xor butterfly over 64 lanes
// and every selection step is one wavefront argmax.  S_base is a 128-bit set
// in LDS built with integer OR, so its value does not depend on the order in
// which tokens finish.
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

// (v, j) precedes (ov, oj) in rank order: larger logit, then smaller index.
__device__ __forceinline__ bool precedes(float v, int j, float ov, int oj) {
    return v > ov || (v == ov && j < oj);
}

// Wavefront argmax in rank order; every lane ends with the same winner.
__device__ __forceinline__ void wave_best(float& v, int& j) {
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) {
        float ov = __shfl_xor(v, off, kWave);
        int oj = __shfl_xor(j, off, kWave);
        if (precedes(ov, oj, v, j)) { v = ov; j = oj; }
    }
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
    return v;
}

// Normaliser Z: lane sum of experts (2l, 2l+1), then the xor butterfly,
// which is exactly the balanced pairwise tree over 128 slots in expert order.
__device__ __forceinline__ float wave_tree_sum(float s) {
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) s = s + __shfl_xor(s, off, kWave);
    return s;
}

constexpr int kNoExpert = 0x7fffffff;
constexpr float kNegInf = -__builtin_huge_valf();

// Select up to `count` experts of the calling token in rank order among the
// lane's two candidates that are still available.  Results are uniform
// across the wavefront.  Stops early when nothing is left.
__device__ __forceinline__ int select_ranked(float l0, float l1, bool avail0, bool avail1,
                                             int e0, int e1, int count, float (&selv)[kMaxTopK],
                                             int (&selj)[kMaxTopK]) {
    int got = 0;
#pragma unroll
    for (int r = 0; r < kMaxTopK; ++r) {
        if (r >= count) break;
        float v0 = avail0 ? l0 : kNegInf;
        int j0 = avail0 ? e0 : kNoExpert;
        float v1 = avail1 ? l1 : kNegInf;
        int j1 = avail1 ? e1 : kNoExpert;
        float v = v0;
        int j = j0;
        if (precedes(v1, j1, v, j)) { v = v1; j = j1; }
        wave_best(v, j);
        if (j == kNoExpert) break;
        selv[r] = v;
        selj[r] = j;
        if (j == e0) avail0 = false;
        if (j == e1) avail1 = false;
        got = r + 1;
    }
    return got;
}

// Write the kept experts of one token: lane r < k writes slot r.
// Weights: e_r / sum_{kept} e (renorm) or e_r / Z (raw softmax), with the
// quotient taken in double and rounded once to fp32.
__device__ __forceinline__ void write_token(int lane, int i, int k, int kept, float m, bool renorm,
                                            float Z, const float (&selv)[kMaxTopK],
                                            const int (&selj)[kMaxTopK], int32_t* idx, float* w) {
    float ev[kMaxTopK];
    double denom = 0.0;
#pragma unroll
    for (int r = 0; r < kMaxTopK; ++r) {
        ev[r] = 0.0f;
        if (r < kept) {
            ev[r] = route_exp(selv[r] - m);
            denom += static_cast<double>(ev[r]);
        }
    }
    if (!renorm) denom = static_cast<double>(Z);
    int my_j = -1;
    float my_w = 0.0f;
#pragma unroll
    for (int r = 0; r < kMaxTopK; ++r) {
        if (lane == r && r < kept) {
            my_j = selj[r];
            my_w = static_cast<float>(static_cast<double>(ev[r]) / denom);
        }
    }
    if (lane < k) {
        idx[i * k + lane] = my_j;
        w[i * k + lane] = my_w;
    }
}

template <bool kOea>
__global__ __launch_bounds__(1024) void route_kernel(const float* __restrict__ logits, int B,
                                                     int N, int k, int k0, float p, int renorm,
                                                     int32_t* __restrict__ idx,
                                                     float* __restrict__ w,
                                                     int32_t* __restrict__ n_base,
                                                     uint32_t* __restrict__ mask_out,
                                                     int32_t* __restrict__ T_out) {
    __shared__ uint32_t sbase[kMaxExperts / 32];
    __shared__ int sbase_count;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const int nwaves = blockDim.x / kWave;
    const int e0 = 2 * lane, e1 = 2 * lane + 1;
    if (threadIdx.x < kMaxExperts / 32) sbase[threadIdx.x] = 0u;
    __syncthreads();

    float selv[kMaxTopK];
    int selj[kMaxTopK];

    // Vanilla top-k, or OEA Phase 1.
    for (int i = wave; i < B; i += nwaves) {
        const float l0 = e0 < N ? logits[i * N + e0] : kNegInf;
        const float l1 = e1 < N ? logits[i * N + e1] : kNegInf;
        const bool v0 = e0 < N, v1 = e1 < N;
        const bool need_z = kOea ? (p < 1.0f) : (renorm == 0);
        float Z = 0.0f;
        if (need_z) {
            float m = wave_max(fmaxf(l0, l1));
            float s0 = v0 ? route_exp(l0 - m) : 0.0f;
            float s1 = v1 ? route_exp(l1 - m) : 0.0f;
            Z = wave_tree_sum(s0 + s1);
        }
        if (!kOea) {
            int kept = select_ranked(l0, l1, v0, v1, e0, e1, k, selv, selj);
            write_token(lane, i, k, kept, selv[0], renorm != 0, Z, selv, selj, idx, w);
        } else {
            int kept = select_ranked(l0, l1, v0, v1, e0, e1, k0, selv, selj);
            int n = kept;
            if (p < 1.0f) {
                const float m = selv[0];
                const float pz = p * Z;
                float c = 0.0f;
#pragma unroll
                for (int r = 0; r < kMaxTopK; ++r) {
                    if (r >= kept) break;
                    c = c + route_exp(selv[r] - m);
                    if (c >= pz) { n = r + 1; break; }
                }
            }
            if (lane == 0 && n_base != nullptr) n_base[i] = n;
#pragma unroll
            for (int r = 0; r < kMaxTopK; ++r) {
                if (r < n && lane == r) atomicOr(&sbase[selj[r] >> 5], 1u << (selj[r] & 31));
            }
        }
    }
    if (!kOea) return;
    __syncthreads();
    if (threadIdx.x == 0) {
        int c = 0;
        for (int wd = 0; wd < kMaxExperts / 32; ++wd) c += __popc(sbase[wd]);
        sbase_count = c;
        if (T_out != nullptr) *T_out = c;
    }
    if (mask_out != nullptr && threadIdx.x < (N + 31) / 32) mask_out[threadIdx.x] = sbase[threadIdx.x];
    __syncthreads();
    const int T = sbase_count;
    const int keep = T < k ? T : k;

    // Phase 2: token i keeps the first min(k, T) members of S_base in its rank
    // order -- its baseline first (the top-ranked experts are in S_base), then
    // lower-ranked experts that other tokens already activated.
    for (int i = wave; i < B; i += nwaves) {
        const float l0 = e0 < N ? logits[i * N + e0] : kNegInf;
        const float l1 = e1 < N ? logits[i * N + e1] : kNegInf;
        const bool a0 = e0 < N && ((sbase[e0 >> 5] >> (e0 & 31)) & 1u);
        const bool a1 = e1 < N && ((sbase[e1 >> 5] >> (e1 & 31)) & 1u);
        int kept = select_ranked(l0, l1, a0, a1, e0, e1, keep, selv, selj);
        write_token(lane, i, k, kept, selv[0], true, 0.0f, selv, selj, idx, w);
    }
}

// Dispatch: histogram, exclusive scan, (expert, token)-ordered permutation and
// the active list.  A token's position inside its expert's bucket is the
// number of lower-numbered tokens routed to the same expert, read off a
// per-expert token bitmask, so the result needs no ordering of atomics.
__global__ __launch_bounds__(1024) void dispatch_kernel(const int32_t* __restrict__ idx, int B,
                                                        int N, int k, int32_t* __restrict__ cnt,
                                                        int32_t* __restrict__ offsets,
                                                        int32_t* __restrict__ perm,
                                                        int32_t* __restrict__ active,
                                                        int32_t* __restrict__ T_out) {
    __shared__ int cnt_s[kMaxExperts];
    __shared__ int off_s[kMaxExperts + 1];
    __shared__ unsigned long long tokmask[kMaxExperts][kMaxBatch / 64];
    const int tid = threadIdx.x;
    const int pairs = B * k;
    for (int e = tid; e < kMaxExperts; e += blockDim.x) {
        cnt_s[e] = 0;
        tokmask[e][0] = 0ull;
        tokmask[e][1] = 0ull;
    }
    __syncthreads();
    for (int q = tid; q < pairs; q += blockDim.x) {
        int e = idx[q];
        if (e >= 0 && e < N) {
            int t = q / k;
            atomicAdd(&cnt_s[e], 1);
            atomicOr(&tokmask[e][t >> 6], 1ull << (t & 63));
        }
    }
    __syncthreads();
    if (tid < kWave) {
        const int lane = tid;
        const int c0 = 2 * lane < N ? cnt_s[2 * lane] : 0;
        const int c1 = 2 * lane + 1 < N ? cnt_s[2 * lane + 1] : 0;
        int s = c0 + c1;
        int a = (c0 > 0) + (c1 > 0);
        // inclusive scans over lanes
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            int os = __shfl_up(s, off, kWave);
            int oa = __shfl_up(a, off, kWave);
            if (lane >= off) { s += os; a += oa; }
        }
        const int excl = s - (c0 + c1);
        const int aexcl = a - ((c0 > 0) + (c1 > 0));
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
        const int total = __shfl(s, kWave - 1, kWave);
        const int tact = __shfl(a, kWave - 1, kWave);
        if (lane == 0) {
            off_s[N] = total;
            offsets[N] = total;
            *T_out = tact;
        }
        // active list, ascending, then -1
        int pos = aexcl;
        if (2 * lane < N && c0 > 0) active[pos++] = 2 * lane;
        if (2 * lane + 1 < N && c1 > 0) active[pos++] = 2 * lane + 1;
        for (int e = tact + lane; e < N; e += kWave) active[e] = -1;
    }
    __syncthreads();
    const int total = off_s[N];
    for (int q = tid; q < pairs; q += blockDim.x) {
        int e = idx[q];
        if (e >= 0 && e < N) {
            int t = q / k;
            unsigned long long lo = tokmask[e][0], hi = tokmask[e][1];
            int below;
            if (t < 64) {
                below = __popcll(lo & ((1ull << t) - 1ull));
            } else {
                below = __popcll(lo) + __popcll(hi & ((1ull << (t - 64)) - 1ull));
            }
            perm[off_s[e] + below] = q;
        }
        if (q >= total) perm[q] = -1;
    }
}

// Router logits: one wavefront per (expert, group of up to 16 tokens); lanes
// stride over the hidden dimension 8 columns at a time; fp32 accumulation.
constexpr int kGemvTok = 16;

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

template <typename XT>
__global__ __launch_bounds__(256) void router_logits_kernel(const XT* __restrict__ x,
                                                            const float* __restrict__ w_r, int B,
                                                            int H, int N,
                                                            float* __restrict__ logits) {
    const int lane = threadIdx.x & (kWave - 1);
    const int e = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    const int t0 = blockIdx.y * kGemvTok;
    if (e >= N) return;
    const int nt = min(kGemvTok, B - t0);
    float acc[kGemvTok];
#pragma unroll
    for (int t = 0; t < kGemvTok; ++t) acc[t] = 0.0f;
    const float* wrow = w_r + static_cast<size_t>(e) * H;
    for (int c = 8 * lane; c < H; c += 8 * kWave) {
        float wv[8];
        load_x8<float>(wrow + c, wv);
#pragma unroll
        for (int t = 0; t < kGemvTok; ++t) {
            if (t < nt) {
                float xv[8];
                load_x8<XT>(x + static_cast<size_t>(t0 + t) * H + c, xv);
#pragma unroll
                for (int q = 0; q < 8; ++q) acc[t] = __builtin_fmaf(wv[q], xv[q], acc[t]);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < kGemvTok; ++t) {
        float s = acc[t];
#pragma unroll
        for (int off = kWave / 2; off > 0; off >>= 1) s = s + __shfl_xor(s, off, kWave);
        if (lane == 0 && t < nt) logits[static_cast<size_t>(t0 + t) * N + e] = s;
    }
}

__global__ void hotness_kernel(float* S, const int32_t* cnt, int N, float alpha) {
    int e = blockIdx.x * blockDim.x + threadIdx.x;
    if (e < N) S[e] = alpha * S[e] + (1.0f - alpha) * static_cast<float>(cnt[e]);
}

__global__ void publish_kernel(moe_expert_handle* table, int e, moe_expert_handle h) {
    if (threadIdx.x == 0) table[e] = h;
}

}  // namespace

hipError_t launch_router_logits(const void* x, int x_dtype, const float* w_r, int B, int H, int N,
                                float* logits, hipStream_t s) {
    dim3 grid((N + 3) / 4, (B + kGemvTok - 1) / kGemvTok);
    if (x_dtype == MOE_DT_BF16)
        router_logits_kernel<uint16_t><<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(x), w_r,
                                                            B, H, N, logits);
    else
        router_logits_kernel<float><<<grid, 256, 0, s>>>(static_cast<const float*>(x), w_r, B, H,
                                                         N, logits);
    return hipGetLastError();
}

hipError_t launch_route(const float* logits, int B, int N, int k, int k0, float p, int oea,
                        int renorm, int32_t* idx, float* w, int32_t* n_base, uint32_t* mask,
                        int32_t* T, hipStream_t s) {
    const int threads = kWave * (B < 16 ? B : 16);
    if (oea)
        route_kernel<true><<<1, threads, 0, s>>>(logits, B, N, k, k0, p, 1, idx, w, n_base, mask, T);
    else
        route_kernel<false><<<1, threads, 0, s>>>(logits, B, N, k, k, 1.0f, renorm, idx, w,
                                                  nullptr, nullptr, nullptr);
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

hipError_t launch_handle_publish(moe_expert_handle* table, int e, moe_expert_handle h,
                                 hipStream_t s) {
    publish_kernel<<<1, 64, 0, s>>>(table, e, h);
    return hipGetLastError();
}

}  // namespace moe
