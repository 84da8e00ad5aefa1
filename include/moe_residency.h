/*
 * moe_residency.h -- online precision residency for the experts of one MoE
 * layer (libmoe, MI355X).
 *
 * Page citations
 *   [DYN]  "Dynamic Expert Quantization for Scalable MoE Inference" notes
 *          (hotelren.com): 2.2 / 3.2 versioned expert residency, 2.3 / 3.3
 *          GPU memory management (partitioned pools, fixed-size blocks,
 *          budget tracker), 2.4 / 3.4 non-blocking transition pipeline,
 *          2.5 / 3.5 online scheduling policy with hysteresis.
 *
 * The forward path is unchanged by anything here: kernels read the handle
 * table (moe.h) and nothing else.  These calls decide which experts hold a
 * high-precision version, copy those versions in on a migration stream and
 * publish them into the table between forward calls.
 *
 * Unless stated, objects are owned by one host thread (not thread-safe);
 * the budget tracker alone may be shared between threads.
 */
#ifndef MOE_RESIDENCY_H_
#define MOE_RESIDENCY_H_

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

/* ---- fixed-block pool [DYN 2.3 / 3.3: pool_hi and pool_lo hand out
 * fixed-size blocks of about one expert version each from a constant-time
 * free list, so promotions never reach a general-purpose allocator] ------ */
typedef struct moe_pool moe_pool;

/*
 * arena       : device memory owned by the caller (never dereferenced here),
 *               256-byte aligned; it must outlive the pool and every block.
 * block_bytes : a positive multiple of 256.  The pool has
 *               floor(arena_bytes / block_bytes) blocks (at least one).
 * *out receives the pool (host memory, freed by moe_pool_destroy).
 */
int moe_pool_create(void *arena, size_t arena_bytes, size_t block_bytes, moe_pool **out);
void moe_pool_destroy(moe_pool *pool);
/* *block = a free block's device address; MOE_EFULL (and *block = NULL) when none is free. O(1). */
int moe_pool_alloc(moe_pool *pool, void **block);
/* Return a block.  MOE_EINVAL for an address that is not a block of this pool or is already free. O(1). */
int moe_pool_free(moe_pool *pool, void *block);
int moe_pool_free_blocks(const moe_pool *pool);
int moe_pool_total_blocks(const moe_pool *pool);
size_t moe_pool_block_bytes(const moe_pool *pool);

/* ---- budget tracker [DYN 2.3 / 3.3: the device budget M_total minus the
 * fixed part M_fixed (KV cache, dense weights, activations, framework) is
 * what expert versions may use; every promotion reserves first] ---------- */
typedef struct moe_budget moe_budget;

int moe_budget_create(size_t total_bytes, size_t fixed_bytes, moe_budget **out);   /* fixed <= total */
void moe_budget_destroy(moe_budget *b);
/* 1: reserved; 0: it does not fit (nothing changes); negative: error.  Thread-safe. */
int moe_budget_try_reserve(moe_budget *b, size_t bytes);
/* MOE_EINVAL if more than is reserved.  Thread-safe. */
int moe_budget_release(moe_budget *b, size_t bytes);
size_t moe_budget_used(const moe_budget *b);
size_t moe_budget_capacity(const moe_budget *b);

/* ---- scheduling policy [DYN 2.5 / 3.5] (host, pure) ---------------------
 * One update of the high-precision set from scores S (fp32, [N]):
 *   - while the set has free capacity, the hottest outsiders with S > 0
 *     enter (no margin);
 *   - then the j-th hottest outsider replaces the j-th coldest member while
 *     S_out > fp32(S_mem + margin) (hysteresis), stopping at the first pair
 *     that fails;
 *   - if the set is larger than n_hi, its coldest members leave first;
 *   - experts with locked[e] != 0 keep their membership and are never paired;
 *   - ranks: higher score first, ties to the lower index.
 * in_hi, locked (may be NULL), target : [N] uint8 flags (target may alias in_hi).
 * promote / demote : [N] int32 each, hottest-first / coldest-first;
 * *n_promote, *n_demote receive their lengths.  1 <= N <= 128.
 */
int moe_residency_select(const float *S, const uint8_t *in_hi, const uint8_t *locked, int N, int n_hi,
                         float margin, uint8_t *target, int32_t *promote, int *n_promote, int32_t *demote,
                         int *n_demote);

/* ---- residency manager [DYN 2.2-2.5, 3.2-3.5] -------------------------- */
typedef struct moe_residency moe_residency;

typedef struct {
    int N, H, I;                    /* the layer: H, I positive multiples of 128 */
    moe_expert_handle *table;       /* device [N]: the layer's handle table */
    const moe_expert_handle *lo;    /* (host) [N]: each expert's resident low-precision version;
                                       the table is assumed to hold exactly these at creation */
    const void *const *hi_src;      /* (host) [N]: pinned host buffers of hi_bytes each, the expert's
                                       bf16 matrices in the packed layout of moe_pack_weights, laid
                                       out gate [I,H] | up [I,H] | down [H,I]; hi_bytes = 6 H I */
    moe_pool *pool_hi;              /* blocks of at least hi_bytes; not shared with other owners */
    moe_budget *budget;             /* each promoted expert holds one block's bytes of it */
    float *S;                       /* device [N]: hotness scores (caller initialises, e.g. zeros) */
    int32_t *c;                     /* device [N]: counts of the current interval (caller zeroes) */
    float *S_host;                  /* (host, pinned) [N]: the scores of the last update */
    int n_hi;                       /* high-precision capacity in experts, >= 0 */
    float alpha;                    /* EMA factor in [0, 1) */
    float margin;                   /* hysteresis margin on scores, >= 0 */
    double interval_s;              /* update cadence T_u in seconds (< 0: only forced updates) */
    void *compute_stream;           /* hipStream_t of the forward path */
    void *mig_stream;               /* hipStream_t for copies, distinct from compute_stream */
} moe_residency_config;

/* expert states: the handle always resolves to a complete version */
enum {
    MOE_RES_LO = 0,          /* the low-precision version is published                        */
    MOE_RES_PROMOTING = 1,   /* a block is reserved and its copy is in flight; still LO to kernels */
    MOE_RES_HI = 2,          /* the high-precision version is published                       */
    MOE_RES_EVICTING = 3     /* LO is published again; the block returns once that publish is done */
};

/* moe_residency_step flags */
enum {
    MOE_RES_FORCE_UPDATE = 1,   /* start a policy update now, whatever the cadence               */
    MOE_RES_WAIT = 2            /* block until every transition this call can start has finished  */
};

typedef struct {
    int64_t steps, updates, decisions;
    int64_t promotions_started, promotions_published, demotions, evictions;
    int64_t deferred;             /* admissions refused by the budget or the pool (backpressure) */
    int64_t bytes_h2d;
} moe_residency_stats;

/* Validates cfg, creates the HIP events it needs and copies the host arrays
 * (lo, hi_src pointers).  Everything else stays owned by the caller. */
int moe_residency_create(const moe_residency_config *cfg, moe_residency **out);

/*
 * One window boundary, called between forward calls on the calling thread.
 *   cnt : device [N] int32, the routing counts of the forward call just
 *         enqueued (dispatch's cnt), added to the interval counters on the
 *         compute stream; NULL adds nothing.
 * In this order, without blocking unless MOE_RES_WAIT:
 *   1. counts folded in; an update is started if due or forced: on the
 *      compute stream S <- alpha S + (1 - alpha) c, c <- 0, then a copy of S
 *      to S_host on the migration stream;
 *   2. if the last update's scores have arrived: moe_residency_select with
 *      in_hi = HI or PROMOTING and locked = PROMOTING or EVICTING; each
 *      demotion publishes the low version on the compute stream (state
 *      EVICTING); the promotions become the pending list, hottest first;
 *   3. EVICTING experts whose publish has completed return their block to
 *      the pool and its bytes to the budget;
 *   4. pending promotions are admitted in order while the budget reserves
 *      and the pool gives a block: the copy from hi_src runs on the
 *      migration stream, followed by an event (state PROMOTING); the first
 *      refusal stops admission until a later call (counted as deferred);
 *   5. PROMOTING experts whose copy has completed are published on the
 *      compute stream behind a wait on that copy's event (state HI).
 * Forward calls enqueued after this call see the table as it was left by it.
 */
int moe_residency_step(moe_residency *r, const int32_t *cnt, int flags);

int moe_residency_state(const moe_residency *r, int e);     /* MOE_RES_* or MOE_EINVAL */
int moe_residency_pending(const moe_residency *r);          /* promotions waiting for admission */
int moe_residency_get_stats(const moe_residency *r, moe_residency_stats *out);

/* Waits for the migration stream and frees the manager.  The table, the
 * pool's blocks still in use and the budget's reservations are left as they
 * are (the caller may keep running the layer). */
int moe_residency_destroy(moe_residency *r);

#ifdef __cplusplus
}
#endif
#endif /* MOE_RESIDENCY_H_ */
