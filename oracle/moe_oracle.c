/*
 * moe_oracle.c -- CPU oracle for the decode-time MoE layer with Opportunistic
 * Expert Activation (OEA) routing.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plain, obviously-correct
 * reference that the GPU library is checked against.  Only the test-suite, the
 * smoke check and the benchmark's CPU-baseline leg may load it.  It shares no
 * code, header, table or constant with the GPU library.
 *
 * Sources (page "Opportunistic Expert Activation (OEA) - L2", zhaifeiyue.github.io):
 *   - section 2 Q1/Q2: the router picks top-k of N experts per token; OEA Phase 1
 *     keeps each token's top-n_i with n_i = min(k0, t_i), t_i an adaptive top-p
 *     count; S_base is the union; Phase 2 adds lower-ranked experts only if they
 *     are already in S_base; kept scores are renormalised.
 *   - section 3 (Algorithm 1 flow: a candidate is kept only if it is a member of S_base), section 5
 *     (Figure 3: simplified OEA drops p and maxP and sets k_max = k).
 *   - section 4, Eq. 2: cnt_i is the number of tokens routed to expert i,
 *     T the number of experts with cnt_i > 0.
 * Page "DynaExq" (hotelren.com), section 2.2 / 3.2: each expert is reached
 * through a stable handle that carries the active version's pointer and its
 * quantisation parameters; cold experts are kept in INT4.
 *
 * Readings where the pages are silent (listed again in the design notes):
 *   - ranking order is (logit descending, expert index ascending);
 *   - t_i is the smallest t whose cumulative sorted probability is >= p
 *     (the crossing expert is included); p >= 1 switches top-p off;
 *   - Phase 2 scans ranks n_i+1..N in the token's rank order and stops at k;
 *   - the top-p decision is taken in the GPU's precision (fp32) with a fixed
 *     arithmetic: Cody-Waite exp, pairwise-tree normaliser, sequential prefix;
 *   - vanilla top-k weights are renormalised too (renorm = 1);
 *   - the expert FFN is SwiGLU: y = W_down (silu(W_gate x) * (W_up x)),
 *     weights stored [out, in] row-major;
 *   - INT4: symmetric, groups of 128 along the input dimension, fp16 scale
 *     s = fp16(absmax / 7), q = clamp(rint(w / s), -8, 7), stored as the
 *     nibble q + 8, two per byte, even column in the low nibble.
 *
 * Parity pins: every function here is checked in tests/test_oracle_pins.py
 * against closed forms, brute force, special cases or library routines.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------- */
/* fp32 <-> bits helpers (plain IEEE-754 definitions)                          */
/* ------------------------------------------------------------------------- */
static float f_from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits_from_f(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* bf16 -> fp32 is exact: the bf16 pattern is the top half of the fp32 one. */
float orc_bf16_to_f32(uint16_t b) { return f_from_bits((uint32_t)b << 16); }

/* fp16 -> fp32 (exact), straight from the binary16 definition. */
float orc_f16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1, ex = (h >> 10) & 0x1f, man = h & 0x3ff;
    double v;
    if (ex == 0)
        v = ldexp((double)man, -24);                  /* subnormal: man * 2^-24 */
    else if (ex == 31)
        v = man ? NAN : INFINITY;
    else
        v = ldexp((double)(man | 0x400), ex - 25);    /* 1.man * 2^(ex-15) */
    return (float)(sign ? -v : v);
}

/* fp32 -> fp16, round to nearest, ties to even, from the definition:
 * pick the representable binary16 value nearest to x; on an exact tie pick
 * the one with an even significand.  Overflow rounds to infinity. */
uint16_t orc_f32_to_f16(float x)
{
    uint16_t sign = (bits_from_f(x) >> 31) ? 0x8000 : 0;
    double a = fabs((double)x);
    if (isnan(x)) return 0x7e00;
    /* quantum (spacing) of binary16 around a */
    double q;
    if (a < ldexp(1.0, -14)) {
        q = ldexp(1.0, -24);                           /* subnormal spacing */
    } else {
        int e;
        frexp(a, &e);                                  /* a = f * 2^e, f in [0.5,1) */
        q = ldexp(1.0, (e - 1) - 10);
    }
    double n = floor(a / q);                           /* a/q is exact (power of 2) */
    double rem = a - n * q;
    if (rem > 0.5 * q || (rem == 0.5 * q && fmod(n, 2.0) != 0.0)) n += 1.0;
    double r = n * q;
    if (r > 65504.0) return sign | 0x7c00;             /* beyond max finite */
    /* encode r */
    if (r < ldexp(1.0, -14)) return sign | (uint16_t)(r / ldexp(1.0, -24));
    int e;
    double f = frexp(r, &e);                           /* r = f * 2^e */
    int ex = e - 1 + 15;
    uint16_t man = (uint16_t)((f * 2.0 - 1.0) * 1024.0);
    return sign | (uint16_t)(ex << 10) | man;
}

/* ------------------------------------------------------------------------- */
/* Canonical fp32 exponential for the top-p decision.                         */
/* Method: Cody & Waite argument reduction (x = n ln2 + r, ln2 split in two    */
/* parts so n*ln2_hi is exact), a degree-7 Taylor polynomial for e^r in Horner */
/* form with fused multiply-adds, and scaling by 2^n through the exponent     */
/* field.  Domain used here: x in [-80, 0]; x < -80 returns 0.                 */
/* ------------------------------------------------------------------------- */
float orc_cexpf(float x)
{
    if (x < -80.0f) return 0.0f;
    /* log2(e) and the two-part ln 2 (ln2_hi has 16 significant bits). */
    const float log2e  = 1.44269504088896341f;
    const float ln2_hi = 0.693145751953125f;          /* 45426 / 65536 */
    const float ln2_lo = 1.42860682030941723e-6f;     /* ln 2 - ln2_hi */
    float t = x * log2e;
    float n = rintf(t);                                /* ties to even */
    float r = fmaf(-n, ln2_hi, x);
    r = fmaf(-n, ln2_lo, r);
    /* Taylor coefficients 1/j!, j = 7..0 */
    float p = 1.0f / 5040.0f;
    p = fmaf(p, r, 1.0f / 720.0f);
    p = fmaf(p, r, 1.0f / 120.0f);
    p = fmaf(p, r, 1.0f / 24.0f);
    p = fmaf(p, r, 1.0f / 6.0f);
    p = fmaf(p, r, 0.5f);
    p = fmaf(p, r, 1.0f);
    p = fmaf(p, r, 1.0f);
    int ni = (int)n;                                   /* in [-116, 0] */
    float scale = f_from_bits((uint32_t)(ni + 127) << 23);
    return p * scale;
}

/* ------------------------------------------------------------------------- */
/* Ranking: (logit descending, expert index ascending), a strict total order. */
/* ------------------------------------------------------------------------- */
static int ranks_before(float la, int ia, float lb, int ib)
{
    if (la > lb) return 1;
    if (la < lb) return 0;
    return ia < ib;
}

/* order[0..N-1] = expert ids in rank order.  Plain insertion sort. */
void orc_rank(const float *l, int N, int32_t *order)
{
    for (int j = 0; j < N; ++j) {
        int pos = j;
        while (pos > 0 && ranks_before(l[j], j, l[order[pos - 1]], order[pos - 1])) {
            order[pos] = order[pos - 1];
            --pos;
        }
        order[pos] = j;
    }
}

/* Softmax terms in the canonical fp32 arithmetic:
 *   m = the top-ranked logit, e_j = cexp(l_j - m),
 *   Z = balanced pairwise tree sum of e over 128 slots in expert-index order
 *       (slots N..127 hold 0), i.e. level 1 adds (2j, 2j+1), level 2 adds
 *       pairs of those, and so on. */
void orc_softmax_terms(const float *l, int N, float *e, float *Z)
{
    float m = l[0];
    for (int j = 1; j < N; ++j)
        if (l[j] > m) m = l[j];
    float v[128];
    for (int j = 0; j < 128; ++j) v[j] = 0.0f;
    for (int j = 0; j < N; ++j) {
        float d = l[j] - m;
        e[j] = orc_cexpf(d);
        v[j] = e[j];
    }
    for (int width = 128; width > 1; width /= 2)
        for (int j = 0; j < width / 2; ++j)
            v[j] = v[2 * j] + v[2 * j + 1];
    *Z = v[0];
}

/* Adaptive top-p count t (section 2 Q2: "adaptive top-p"): the length of the
 * shortest rank prefix whose cumulative probability reaches p.  Cumulation is
 * sequential in rank order in fp32; the test is c >= p*Z (fp32 product).
 * p >= 1 disables top-p (t = N); if rounding keeps c below p*Z, t = N. */
int orc_topp_count(const float *e, float Z, const int32_t *order, int N, float p)
{
    if (p >= 1.0f) return N;
    float pz = p * Z;
    float c = 0.0f;
    for (int t = 1; t <= N; ++t) {
        c = c + e[order[t - 1]];
        if (c >= pz) return t;
    }
    return N;
}

/* ------------------------------------------------------------------------- */
/* Routing.                                                                    */
/*   oea = 0: vanilla top-k (section 2 Q1).  renorm selects renormalised       */
/*            weights over the k kept experts (1) or raw softmax (0).          */
/*   oea = 1: OEA (section 2 Q2 / section 3): Phase 1 baseline top-n_i,        */
/*            union S_base, Phase 2 piggyback from S_base up to k, then        */
/*            renormalise.                                                     */
/* Outputs: idx[B*k] (rank order, -1 padded), w[B*k] (double, 0 padded),      */
/* n_base[B], mask[ceil(N/32)] (bit e of word e/32 = e in S_base; for vanilla  */
/* the union of the kept sets), T[0] = number of experts in that union.       */
/* Weights are the plain softmax definition in double with libm exp.           */
/* ------------------------------------------------------------------------- */
/*
 * General routing.  mode 0 = vanilla top-k, 1 = OEA, 2 = pruned (OEA Phase 1
 * only: each token keeps just its baseline).  For OEA, Phase 2 scans the
 * token's ranks n_i+1 .. max_p (page OEA section 5: "maxP", the deepest rank
 * that may be piggybacked; max_p = N is the simplified router) and keeps an
 * expert only if it is in S_base, until the token holds k experts (k plays
 * the page's k_max).  Tokens i >= n_valid are padding: they route to no
 * expert and add nothing to S_base (page OEA section 7: padding tokens must
 * not inflate T).
 */
void orc_route_general(const float *logits, int B, int N, int k, int k0, float p, int mode, int max_p,
                       int renorm, int n_valid, int32_t *idx, double *w, int32_t *n_base, uint32_t *mask,
                       int32_t *T)
{
    int32_t order[128];
    float e[128];
    unsigned char in_base[128];
    memset(in_base, 0, sizeof in_base);
    const int oea = mode != 0;
    if (n_valid > B) n_valid = B;
    if (n_valid < 0) n_valid = 0;

    /* Phase 1 for every real token (for vanilla: the k kept experts). */
    for (int i = 0; i < B; ++i) {
        if (i >= n_valid) { n_base[i] = 0; continue; }
        const float *l = logits + (size_t)i * N;
        orc_rank(l, N, order);
        int n;
        if (oea) {
            float Z;
            orc_softmax_terms(l, N, e, &Z);
            int t = orc_topp_count(e, Z, order, N, p);
            n = k0 < t ? k0 : t;
        } else {
            n = k;
        }
        n_base[i] = n;
        for (int r = 0; r < n; ++r) in_base[order[r]] = 1;
    }
    int nwords = (N + 31) / 32;
    for (int wd = 0; wd < nwords; ++wd) mask[wd] = 0;
    int count = 0;
    for (int j = 0; j < N; ++j)
        if (in_base[j]) { mask[j / 32] |= 1u << (j % 32); ++count; }
    *T = count;

    /* Phase 2 (OEA), the baseline alone (pruned) or the vanilla selection,
       then the weights. */
    for (int i = 0; i < B; ++i) {
        int32_t sel[128];
        int ns = 0;
        const float *l = logits + (size_t)i * N;
        if (i < n_valid) {
            orc_rank(l, N, order);
            if (oea) {
                int n = n_base[i];
                for (int r = 0; r < n; ++r) sel[ns++] = order[r];
                if (mode == 1) {
                    /* literal scan: ranks n+1..max_p, keep an expert only if in S_base */
                    for (int r = n; r < max_p && r < N && ns < k; ++r)
                        if (in_base[order[r]]) sel[ns++] = order[r];
                }
            } else {
                for (int r = 0; r < k; ++r) sel[ns++] = order[r];
            }
        }
        double m = ns > 0 ? (double)l[order[0]] : 0.0;
        double denom = 0.0;
        if (oea || renorm) {
            for (int s = 0; s < ns; ++s) denom += exp((double)l[sel[s]] - m);
        } else if (ns > 0) {
            for (int j = 0; j < N; ++j) denom += exp((double)l[j] - m);
        }
        for (int s = 0; s < k; ++s) {
            if (s < ns) {
                idx[(size_t)i * k + s] = sel[s];
                w[(size_t)i * k + s] = exp((double)l[sel[s]] - m) / denom;
            } else {
                idx[(size_t)i * k + s] = -1;
                w[(size_t)i * k + s] = 0.0;
            }
        }
    }
}

/* Vanilla (oea = 0) or simplified-form OEA (oea = 1, max_p = N), all tokens real. */
void orc_route(const float *logits, int B, int N, int k, int k0, float p, int oea, int renorm,
               int32_t *idx, double *w, int32_t *n_base, uint32_t *mask, int32_t *T)
{
    orc_route_general(logits, B, N, k, k0, p, oea ? 1 : 0, N, renorm, B, idx, w, n_base, mask, T);
}

/* ------------------------------------------------------------------------- */
/* Dispatch (Eq. 2's cnt_i and T): per-expert counts, exclusive offsets, the   */
/* permutation sorted by (expert asc, token asc) whose entries are             */
/* token*k + slot, and the ascending list of active experts.                   */
/* perm entries past the last pair and active entries past T are -1.          */
/* ------------------------------------------------------------------------- */
void orc_dispatch(const int32_t *idx, int B, int N, int k, int32_t *cnt, int32_t *offsets,
                  int32_t *perm, int32_t *active, int32_t *T)
{
    for (int e = 0; e < N; ++e) cnt[e] = 0;
    for (int i = 0; i < B; ++i)
        for (int s = 0; s < k; ++s) {
            int e = idx[(size_t)i * k + s];
            if (e >= 0) cnt[e] += 1;
        }
    offsets[0] = 0;
    for (int e = 0; e < N; ++e) offsets[e + 1] = offsets[e] + cnt[e];
    for (int q = 0; q < B * k; ++q) perm[q] = -1;
    int pos = 0;
    for (int e = 0; e < N; ++e)
        for (int i = 0; i < B; ++i)
            for (int s = 0; s < k; ++s)
                if (idx[(size_t)i * k + s] == e) perm[pos++] = i * k + s;
    int t = 0;
    for (int e = 0; e < N; ++e) active[e] = -1;
    for (int e = 0; e < N; ++e)
        if (cnt[e] > 0) active[t++] = e;
    *T = t;
}

/* ------------------------------------------------------------------------- */
/* Router logits in double: logits[b, e] = sum_h x[b, h] * W_r[e, h].          */
/* ------------------------------------------------------------------------- */
void orc_router_logits(const double *x, const double *wr, int B, int H, int N, double *logits)
{
    for (int b = 0; b < B; ++b)
        for (int e = 0; e < N; ++e) {
            double acc = 0.0;
            for (int h = 0; h < H; ++h) acc += x[(size_t)b * H + h] * wr[(size_t)e * H + h];
            logits[(size_t)b * N + e] = acc;
        }
}

/* ------------------------------------------------------------------------- */
/* Expert weights as seen by the oracle: one record per expert.               */
/* fmt 0 = fp32, 1 = bf16 (uint16 bits), 2 = INT4 groups of 128 (uint8 nibble */
/* pairs + fp16 scale bits [out, in/128]).  Matrices are [out, in] row-major:  */
/* gate and up are [I, H], down is [H, I].                                     */
/* ------------------------------------------------------------------------- */
typedef struct {
    int32_t fmt;
    int32_t pad;
    const void *gate, *up, *down;
    const uint16_t *s_gate, *s_up, *s_down;
} orc_expert;

/* exact widening of one stored weight to double */
static double weight_at(int fmt, const void *m, const uint16_t *sc, int cols, int r, int c)
{
    size_t at = (size_t)r * cols + c;
    if (fmt == 0) return (double)((const float *)m)[at];
    if (fmt == 1) return (double)orc_bf16_to_f32(((const uint16_t *)m)[at]);
    const uint8_t *qb = (const uint8_t *)m;
    uint8_t byte = qb[at / 2];
    int nib = (at % 2 == 0) ? (byte & 0xf) : (byte >> 4);
    int q = nib - 8;
    double s = (double)orc_f16_to_f32(sc[(size_t)r * (cols / 128) + c / 128]);
    return (double)q * s;
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* Expert FFN and weighted combine, all in double, for every routed pair
 * (token i, slot s) with expert e = idx[i, s]:
 *   g = W_gate x_i, u = W_up x_i, a = silu(g) * u, d = W_down a,
 *   y[i] = sum over token i's filled slots, in slot (rank) order, of w[i, s] * d.
 * x is [B, H] (already widened), w is [B, k], idx is [B, k] (-1 = empty).
 * The work runs in three loops: the SwiGLU activations a of every (pair, row
 * of I), then the down projections d of every (pair, row of H), then the
 * combine, one output element at a time.  Each a and d element is one plain
 * dot product in index order, whichever thread computes it, and the combine
 * is sequential, so the result does not depend on the thread count
 * (orc_set_threads; OpenMP across pairs and rows). */
static int g_threads = 1;

void orc_set_threads(int n) { g_threads = n > 0 ? n : 1; }

int orc_get_threads(void) { return g_threads; }

void orc_expert_ffn(const orc_expert *ex, int H, int I, const double *x, const int32_t *idx,
                    const double *w, int B, int k, double *y)
{
    long pairs = (long)B * k;
    double *a = (double *)malloc(sizeof(double) * (size_t)pairs * (size_t)I);
    double *d = (double *)malloc(sizeof(double) * (size_t)pairs * (size_t)H);
    long n_a = pairs * I, n_d = pairs * H;
#pragma omp parallel for schedule(static) num_threads(g_threads)
    for (long t = 0; t < n_a; ++t) {
        long q = t / I;
        int j = (int)(t % I);
        int e = idx[q];
        if (e < 0) continue;
        const orc_expert *E = &ex[e];
        const double *xi = x + (size_t)(q / k) * H;
        double g = 0.0, u = 0.0;
        for (int h = 0; h < H; ++h) {
            g += weight_at(E->fmt, E->gate, E->s_gate, H, j, h) * xi[h];
            u += weight_at(E->fmt, E->up, E->s_up, H, j, h) * xi[h];
        }
        a[(size_t)q * I + j] = silu(g) * u;
    }
#pragma omp parallel for schedule(static) num_threads(g_threads)
    for (long t = 0; t < n_d; ++t) {
        long q = t / H;
        int o = (int)(t % H);
        int e = idx[q];
        if (e < 0) continue;
        const orc_expert *E = &ex[e];
        const double *aq = a + (size_t)q * I;
        double acc = 0.0;
        for (int j = 0; j < I; ++j) acc += weight_at(E->fmt, E->down, E->s_down, I, o, j) * aq[j];
        d[(size_t)q * H + o] = acc;
    }
    for (int i = 0; i < B; ++i) {
        double *yi = y + (size_t)i * H;
        for (int o = 0; o < H; ++o) yi[o] = 0.0;
        for (int s = 0; s < k; ++s) {
            long q = (long)i * k + s;
            if (idx[q] < 0) continue;
            for (int o = 0; o < H; ++o) yi[o] += w[q] * d[(size_t)q * H + o];
        }
    }
    free(a);
    free(d);
}

/* ------------------------------------------------------------------------- */
/* INT4 quantiser for one [rows, cols] bf16 matrix (cols % 128 == 0).          */
/* Per row and group of 128 consecutive columns: absmax of the widened values, */
/* s = fp16(absmax / 7) with the fp32 quotient rounded to nearest-even,        */
/* q = clamp(rint(w / s), -8, 7) with the fp32 quotient (q = 0 when s = 0),    */
/* stored as the nibble q + 8, even column in the low nibble.                  */
/* ------------------------------------------------------------------------- */
void orc_quantize_int4(const uint16_t *wb, int rows, int cols, uint8_t *q, uint16_t *scales)
{
    int groups = cols / 128;
    for (int r = 0; r < rows; ++r) {
        for (int g = 0; g < groups; ++g) {
            float amax = 0.0f;
            for (int c = g * 128; c < (g + 1) * 128; ++c) {
                float v = fabsf(orc_bf16_to_f32(wb[(size_t)r * cols + c]));
                if (v > amax) amax = v;
            }
            float quot = amax / 7.0f;
            uint16_t sh = orc_f32_to_f16(quot);
            scales[(size_t)r * groups + g] = sh;
            float s = orc_f16_to_f32(sh);
            for (int c = g * 128; c < (g + 1) * 128; ++c) {
                int qi = 0;
                if (s != 0.0f) {
                    float v = orc_bf16_to_f32(wb[(size_t)r * cols + c]);
                    float t = rintf(v / s);
                    if (t > 7.0f) t = 7.0f;
                    if (t < -8.0f) t = -8.0f;
                    qi = (int)t;
                }
                uint8_t nib = (uint8_t)(qi + 8);
                size_t at = (size_t)r * cols + c;
                if (at % 2 == 0) q[at / 2] = (uint8_t)((q[at / 2] & 0xf0) | nib);
                else q[at / 2] = (uint8_t)((q[at / 2] & 0x0f) | (nib << 4));
            }
        }
    }
}

/* ------------------------------------------------------------------------- */
/* Hotness estimate (DynaExq section 2.5): S <- alpha * S + (1 - alpha) * c.   */
/* ------------------------------------------------------------------------- */
void orc_hotness_ema(double *S, const int32_t *c, int N, double alpha)
{
    for (int e = 0; e < N; ++e) S[e] = alpha * S[e] + (1.0 - alpha) * (double)c[e];
}
