/*
 * moe.h -- C ABI of libmoe, a decode-time Mixture-of-Experts layer for
 * AMD Instinct MI355X (gfx950) with Opportunistic Expert Activation routing.
 *
 * Conventions for every entry point
 *   - Pointers are DEVICE pointers unless the comment says (host).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued on it; the call returns without synchronising and
 *     never allocates device or host memory.
 *   - Arguments are validated on the host before anything is enqueued; an
 *     invalid call returns a negative status and enqueues nothing.
 *   - Results that size later work (T, counts, offsets) stay in device memory;
 *     no call reads them back to the host.
 *   - The caller owns every buffer.  Buffers must not overlap unless stated.
 *   - Limits: 1 <= N <= 128 experts, 1 <= k <= min(N, 16), 1 <= B <= 128.
 *   - Non-finite logits, and idx entries outside [-1, N) or repeated within a
 *     token's row, are undefined behaviour (not checked on the device).
 *
 * Page citations
 *   [OEA]  "Opportunistic Expert Activation (OEA) - L2" (zhaifeiyue.github.io)
 *   [DYN]  "Dynamic Expert Quantization for Scalable MoE Inference" notes
 *          (hotelren.com), sections 2.1-2.5 / 3.1-3.5.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
enum {
    MOE_OK = 0,
    MOE_EINVAL = -1,         /* argument out of range or null pointer           */
    MOE_EUNSUPPORTED = -2,   /* valid but beyond the library's limits (B > 128) */
    MOE_EHIP = -3,           /* a HIP runtime call or kernel launch failed      */
    MOE_EFULL = -4           /* a pool has no free block (backpressure; retry   */
                             /* later), see moe_residency.h                     */
};

/* activation element type */
enum { MOE_DT_F32 = 0, MOE_DT_BF16 = 1 };

/* expert weight formats */
enum {
    MOE_W_F32 = 0,           /* fp32                                            */
    MOE_W_BF16 = 1,          /* bf16                                            */
    MOE_W_INT4_G128 = 2      /* symmetric INT4, groups of 128 input columns,    */
                             /* fp16 scales (see moe_quantize_int4_g128)        */
};

/*
 * Per-expert stable handle [DYN section 2.2 "versioned expert residency" /
 * 3.2: a handle's identity never changes; it resolves at run time to the
 * active version's pointer and quantisation parameters, so a version change
 * rewrites the handle and never the kernel arguments].
 *
 * Matrices are [out, in]: w_gate, w_up : [I, H]   w_down : [H, I].  The
 * forward path reads them in the PACKED layout written by moe_pack_weights
 * (16-byte aligned), not row-major:
 *   Each matrix of `rows` x `cols` is cut into tiles of 16 rows x 64 bytes
 *   of row data (16 fp32, 32 bf16 or 128 INT4 columns); tile (rb, s) -- row
 *   block rb, column segment s, S = row_bytes / 64 -- is the 1 KB block at
 *   (rb * S + s) KB.  Inside a tile, the 16 bytes at 16 * l hold row m =
 *   l % 16, bytes [16 * (l / 16), + 16) of that row's segment (the operand
 *   order of the 16x16 MFMA instructions).  fp32/bf16 bytes are unchanged;
 *   INT4 bytes are re-ordered within each 4-byte word (see moe_pack_weights).
 *   MOE_W_INT4_G128 scales (fp16 bits, 8-byte aligned) are packed as
 *   [rows/16][cols/128][16]; s_gate, s_up, s_down are NULL for other formats.
 * The table is an array of N handles in device memory.  64 bytes each.
 */
typedef struct moe_expert_handle {
    int32_t fmt;             /* MOE_W_*                                         */
    int32_t group;           /* 128 for MOE_W_INT4_G128, else 0                 */
    const void *w_gate;
    const void *w_up;
    const void *w_down;
    const uint16_t *s_gate;
    const uint16_t *s_up;
    const uint16_t *s_down;
    int64_t reserved;        /* keeps the record at 64 bytes; set to 0          */
} moe_expert_handle;

/*
 * Router logits [OEA section 2 Q1: each token's router scores over N experts].
 *   logits[b, e] = sum_h x[b, h] * w_r[e, h], accumulated in fp32.
 *   x      : [B, H], element type x_dtype (MOE_DT_F32 or MOE_DT_BF16)
 *   w_r    : [N, H] fp32
 *   logits : [B, N] fp32 (written)
 * H must be a multiple of 8.
 */
int moe_router_logits(const void *x, int x_dtype, const float *w_r, int B, int H, int N,
                      float *logits, void *stream);

/*
 * Vanilla top-k routing [OEA section 2 Q1: each token routes to k of N
 * experts by router score].
 *   Ranking is (logit descending, expert index ascending).
 *   idx : [B, k] int32, the k best experts of each token in rank order.
 *   w   : [B, k] fp32.  renorm != 0: softmax restricted to the kept experts
 *         (sums to 1); renorm == 0: the full softmax probability.
 */
int moe_route_topk(const float *logits, int B, int N, int k, int renorm, int32_t *idx,
                   float *w, void *stream);

/*
 * OEA routing [OEA section 2 Q2 and section 3 (Algorithm 1 flow); section 5
 * Figure 3 for the simplified form].
 *   Phase 1: t_i = length of the shortest rank prefix whose softmax mass
 *     reaches p (the crossing expert included; p >= 1 turns top-p off, so
 *     t_i = N); n_i = min(k0, t_i); token i's baseline is its top n_i experts.
 *     S_base = union of the baselines, T = |S_base|.
 *   Phase 2: token i keeps the first min(k, T) members of S_base in its own
 *     rank order (its baseline first, then lower-ranked experts already in
 *     S_base); the kept softmax scores are renormalised to sum to 1.
 *   The top-p decision uses a fixed fp32 arithmetic so it is reproducible:
 *     m = top logit, e_j = exp(l_j - m) by Cody-Waite reduction and a
 *     degree-7 Taylor polynomial (0 below -80), Z = pairwise tree sum over
 *     128 slots in expert order, prefix sums in rank order, test c >= p * Z.
 *   idx        : [B, k] int32 in rank order, -1 in unused slots
 *   w          : [B, k] fp32, 0 in unused slots
 *   n_base     : [B] int32, n_i (may be NULL)
 *   sbase_mask : [ceil(N/32)] uint32, bit e%32 of word e/32 set iff e in S_base
 *                (may be NULL)
 *   T          : [1] int32, |S_base| (may be NULL)
 * Requires 1 <= k0 <= k and p > 0.
 */
int moe_route_oea(const float *logits, int B, int N, int k0, float p, int k, int32_t *idx,
                  float *w, int32_t *n_base, uint32_t *sbase_mask, int32_t *T, void *stream);

/*
 * Dispatch [OEA section 4, Eq. 2: cnt_i tokens per expert, T = number of
 * experts with cnt_i > 0; section 7: inserted before the expert dispatch].
 *   cnt     : [N]   tokens routed to each expert
 *   offsets : [N+1] exclusive prefix sum of cnt (offsets[N] = routed pairs)
 *   perm    : [B*k] pair ids token*k + slot sorted by (expert, token);
 *             entries past offsets[N] are -1
 *   active  : [N]   experts with cnt > 0 in ascending order, then -1
 *   T       : [1]   number of active experts
 * idx entries outside [0, N) (e.g. -1) are skipped.
 */
int moe_dispatch(const int32_t *idx, int B, int N, int k, int32_t *cnt, int32_t *offsets,
                 int32_t *perm, int32_t *active, int32_t *T, void *stream);

/*
 * Routing and dispatch, with the general OEA knobs [OEA sections 2 Q1/Q2, 3,
 * 4 (Eq. 2), 5 (maxP, k_max, pruned vs OEA) and 7 (padding tokens must not
 * inflate T)].  One launch, in which one workgroup routes and dispatches the
 * batch, for batches of up to 48 tokens and for pruned and max_p < N modes;
 * above 48 tokens vanilla top-k and simplified OEA route 16 tokens per
 * workgroup and take two launches (top-k: routing, then dispatch; OEA: Phase
 * 1, then Phase 2 with the dispatch in the workgroup that finishes last).
 * The results are the same either way.
 *   mode MOE_ROUTE_TOPK   : vanilla top-k (renorm as in moe_route_topk)
 *   mode MOE_ROUTE_OEA    : OEA; Phase 2 may take only experts the token
 *                           ranks within its top max_p (k0 <= max_p <= N;
 *                           max_p = N is the simplified router), until the
 *                           token holds k experts (k plays k_max and may
 *                           exceed the model's top-k)
 *   mode MOE_ROUTE_PRUNED : OEA Phase 1 only: each token keeps its n_i
 *                           baseline experts (same S_base and T as OEA)
 *   n_valid : NULL, or a device int32: tokens i >= *n_valid are padding;
 *             they get no experts (idx -1, w 0) and add nothing to S_base,
 *             so a fixed-size (e.g. graph-captured) batch serves smaller
 *             real batches without inflating T
 *   k0_by_batch : NULL, or a device int32 [B+1] table for OEA and pruned
 *             modes [OEA section 7 notes: piggybacking does nothing at B = 1
 *             and the natural tuning axis is a batch-size-dependent k0,
 *             larger at small B]: the call uses k0 = k0_by_batch[b] with b
 *             the number of real tokens (*n_valid, else B), clamped to
 *             [1, k]; the k0 argument then only bounds max_p's check.  The
 *             table is read on the device, so a captured graph follows the
 *             real batch size of each replay.
 *   sync : NULL, or a device int32 [1], zero before the first call and left
 *          at zero by every call (calls sharing it must be ordered, e.g. on
 *          one stream): with it, vanilla top-k above 48 tokens dispatches in
 *          its routing launch's last workgroup instead of a launch of its own
 *   Outputs as moe_route_oea (n_base, sbase_mask may be NULL; ignored for
 *   top-k) followed by moe_dispatch on idx; T = number of active experts
 *   (for OEA and pruned also |S_base|).  In the one-launch form the routed
 *   pairs stay on chip between routing and dispatch.
 */
enum { MOE_ROUTE_TOPK = 0, MOE_ROUTE_OEA = 1, MOE_ROUTE_PRUNED = 2 };
int moe_route_dispatch(const float *logits, int B, int N, int k, int mode, int k0, float p, int max_p,
                       int renorm, const int32_t *n_valid, const int32_t *k0_by_batch, int32_t *idx,
                       float *w, int32_t *n_base,
                       uint32_t *sbase_mask, int32_t *cnt, int32_t *offsets, int32_t *perm, int32_t *active,
                       int32_t *T, int32_t *sync, void *stream);

/*
 * Router logits, routing and dispatch [OEA section 2 Q1: the router scores
 * every expert for every token; then as moe_route_dispatch].
 *   x, x_dtype, w_r, H : as moe_router_logits; logits [B, N] fp32 receives
 *                        the router output (the routing decisions use it)
 *   the remaining arguments are those of moe_route_dispatch, but sync is
 *          required here (the router's workgroups count themselves in it).
 * Where moe_route_dispatch takes one launch, this is one launch too: its
 * workgroups each compute a slice of the logits, and the one that finishes
 * last routes and dispatches the batch, so no workgroup waits.  Otherwise
 * (above 48 tokens, vanilla top-k or simplified OEA) the logits are computed
 * as by moe_router_logits and the token-group routing follows (vanilla top-k
 * counts its workgroups in sync and dispatches in the last one; sync is again
 * left at zero).  The logits have the same bits on every path.
 * Requires H a positive multiple of 8, plus the conditions of
 * moe_route_dispatch.
 */
int moe_router_route_dispatch(const void *x, int x_dtype, const float *w_r, int B, int H, int N, int k, int mode,
                              int k0, float p, int max_p, int renorm, const int32_t *n_valid,
                              const int32_t *k0_by_batch, float *logits, int32_t *idx, float *w,
                              int32_t *n_base, uint32_t *sbase_mask, int32_t *cnt, int32_t *offsets,
                              int32_t *perm, int32_t *active, int32_t *T, int32_t *sync, void *stream);

/* Workspace bytes moe_expert_ffn needs for these sizes (host call):
 * B*k*(I + H)*4 (per routed pair, its SwiGLU activations and weighted down
 * projection), each part rounded up to 256 bytes. */
size_t moe_ffn_workspace_bytes(int B, int k, int H, int I);

/*
 * Expert FFN and weighted combine [OEA section 4, Eq. 2 and check 4: every
 * activated expert's weights are fetched once; the cost is b*T + a*sum(cnt)].
 *   For every active expert e and each routed pair (token i, slot s):
 *     g = W_gate,e x_i, u = W_up,e x_i, a = silu(g) * u, d = W_down,e a,
 *     y_i = sum over token i's filled slots of w[i, s] * d.
 *   table  : [N] moe_expert_handle (device, 16-byte aligned); each expert's
 *            format may differ
 *   x      : [B, H] (x_dtype); with bf16/INT4 experts an fp32 activation a
 *            enters the products as hi = bf16(a) plus lo = bf16(a - hi)
 *            (about 16 significant bits); bf16 inputs are used exactly.
 *            The SwiGLU output a enters the down projection the same split
 *            way for bf16 experts, exactly for fp32 experts, and rounded to
 *            bf16 for INT4 experts (4-bit weights, 16-bit activations)
 *   idx, w : routing output [B, k]; offsets, perm, active, T: dispatch output
 *   y      : [B, H] fp32, overwritten
 *   ws     : workspace of at least moe_ffn_workspace_bytes(B, k, H, I) bytes,
 *            256-byte aligned (scratch: the SwiGLU activations and the
 *            weighted down projections; no contents need be preset; calls
 *            that share a workspace must be ordered, e.g. on one stream).
 * Accumulation is fp32.  H and I must be multiples of 32, and of 128 for
 * INT4 experts (an expert whose format does not fit contributes nothing to
 * y; its pairs' outputs are undefined).  An active expert's weights are
 * streamed from HBM once when it has at most 32 tokens (16 for INT4 experts);
 * a larger expert is handled in passes of that many tokens, which run side by
 * side and read its weight tiles through the caches, so the later passes
 * mostly hit the L2.
 * Every call is deterministic.  Calls with B*k <= 8, and in each phase
 * calls whose items (T * I/16 in phase A, T * H/16 in phase B) fit the
 * launch with at most 16 tokens per expert, split each expert's input
 * columns over four waves and add the partial sums in a fixed order; other
 * calls sum each item in one wave.  A token's y
 * is bit-identical across calls that take the same paths (padding tokens
 * never change them) and agrees to fp32 rounding otherwise.
 * Errors: MOE_EINVAL for null pointers, sizes out of range, a short or
 * misaligned workspace or table; MOE_EUNSUPPORTED for H or I above 16384 (or,
 * as a guard that the current size limits never reach, when the work
 * partition's total cost could exceed 2^31).
 */
int moe_expert_ffn(const moe_expert_handle *table, int N, int H, int I, const void *x,
                   int x_dtype, const int32_t *idx, const float *w, const int32_t *offsets,
                   const int32_t *perm, const int32_t *active, const int32_t *T, int B, int k,
                   float *y, void *ws, size_t ws_bytes, void *stream);

/*
 * moe_expert_ffn without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, serving loops and
 * harnesses that forbid allocation.  Arguments, results, limits and errors
 * are those of moe_expert_ffn; the workspace is instead a fixed device array
 * of MOE_FFN_NOALLOC_WORKSPACE_BYTES inside the library (one per GPU, held
 * until the process ends; its address is looked up once per GPU, on the first
 * call made with that GPU current).  Nothing is allocated or freed.
 *   Limit: moe_ffn_workspace_bytes(B, k, H, I) <= MOE_FFN_NOALLOC_WORKSPACE_BYTES
 *   (e.g. B*k <= 2978 pairs at H = 2048, I = 768; B*k <= 1489 at H = 4096,
 *   I = 1536); larger calls return MOE_EUNSUPPORTED and enqueue nothing.
 *   Every call on a GPU uses that GPU's one array, which keeps the last call's
 *   contents (no contents need be preset): calls that may overlap on one GPU
 *   (several streams or threads) race and must be ordered by the caller.
 */
#define MOE_FFN_NOALLOC_WORKSPACE_BYTES ((size_t)32 << 20)
int moe_expert_ffn_noalloc(const moe_expert_handle *table, int N, int H, int I, const void *x,
                           int x_dtype, const int32_t *idx, const float *w, const int32_t *offsets,
                           const int32_t *perm, const int32_t *active, const int32_t *T, int B, int k,
                           float *y, void *stream);

/*
 * Publish a new version of expert e's handle [DYN section 2.2 / 3.2
 * "publish-then-switch": a version becomes visible only after its data is
 * complete; the forward path keeps using the previous version until then].
 *   h (host) is copied by value into the launch, so it may be freed on return.
 *   The write is ordered on `stream`: work enqueued on the stream before the
 *   call sees the old handle, work after it sees the new one.  A version
 *   copied on another stream must be made visible to `stream` (an event wait)
 *   before publishing.  The old weights may be freed only after work that can
 *   read them has completed.
 */
int moe_handle_publish(moe_expert_handle *table, int e, const moe_expert_handle *h, void *stream);

/*
 * Build the INT4 low-precision version of a bf16 matrix [DYN section 3.2:
 * each expert keeps a high- and a low-precision version; section 3.4:
 * versions are prepacked in kernel-ready form].
 *   w      : [rows, cols] bf16 bits, cols a multiple of 128
 *   q      : [rows, cols/2] row-major nibbles: each byte holds two weights,
 *            the even column in the low nibble, as the unsigned value q + 8
 *   scales : [rows, cols/128] fp16 bits
 *   Per row and group of 128 columns: s = fp16(absmax / 7) (fp32 quotient,
 *   rounded to nearest even), q = clamp(rint(w / s), -8, 7) with the fp32
 *   quotient (q = 0 when s = 0).
 */
int moe_quantize_int4_g128(const uint16_t *w, int rows, int cols, uint8_t *q, uint16_t *scales,
                           void *stream);

/*
 * Pack one row-major matrix into the layout the expert FFN reads [DYN
 * section 3.4: expert versions are prepacked once into kernel-ready form].
 *   fmt        : MOE_W_F32, MOE_W_BF16 or MOE_W_INT4_G128
 *   src        : [rows, cols] row-major (INT4: the bytes moe_quantize_int4_g128
 *                writes); dst receives the same number of bytes, packed.
 *   src_scales : INT4 only: [rows, cols/128] fp16 bits; dst_scales receives
 *                them as [rows/16][cols/128][16].  NULL for other formats.
 *   rows must be a multiple of 16 and cols of 16 (fp32), 32 (bf16) or 128
 *   (INT4); src and dst 16-byte aligned and not overlapping.
 *   INT4: in each 4-byte word of a packed tile (8 consecutive columns c..c+7
 *   of one row), nibble i holds column c + 2i and nibble i + 4 holds column
 *   c + 2i + 1 (i = 0..3), each as the unsigned value q + 8.
 */
int moe_pack_weights(int fmt, const void *src, const uint16_t *src_scales, int rows, int cols,
                     void *dst, uint16_t *dst_scales, void *stream);

/*
 * Hotness estimate [DYN section 2.5: per-expert counters c folded into a
 * smoothed score S <- alpha * S + (1 - alpha) * c].
 *   S : [N] fp32, updated in place;  cnt : [N] int32 (e.g. dispatch's cnt).
 */
int moe_hotness_ema(float *S, const int32_t *cnt, int N, float alpha, void *stream);

/* Static description of a status code (host). */
const char *moe_status_str(int status);

/* Message of the last failure on the calling thread ("" if none) (host). */
const char *moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H_ */
