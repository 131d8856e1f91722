/*
 * bsa.h -- C ABI of the MI355X (gfx950) block-sparse attention library.
 *
 * Forward pass of dynamic block-sparse attention (BSA) as described in
 * "Decoupling Logical Masks from GPU Execution for Dynamic Block-Sparse
 * Attention" (Tessera):
 *   - a request carries a logical block mask M over block geometry
 *     B = (B_Q, B_KV), tensor properties (dtype, head dim, layout) and the
 *     request dimensions (heads, sequence length)      [paper section 3,
 *     "Online request path"; section 4.4 request R = <A, M, B, x>]
 *   - plan creation builds the shared mask state (block-CSR plus scalar
 *     statistics) on the GPU, copies only the statistics to the host, looks
 *     up the performance regime, scans its ranking for the first eligible
 *     plan and prepares only that plan's metadata     [section 5.2]
 *   - run executes the plan's kernels: the attention mainloop and, for
 *     split-K plans, the partial-state merge          [sections 4.2, 4.3]
 *
 * Semantics of the output (section 1, section 2.2): for each head h and
 * query i < N, the keys j < N whose logical block M[h][i/B_Q][j/B_KV] is
 * nonzero enter softmax(q_i k_j^T / sqrt(d)) v_j; a query row with no active
 * key outputs zeros.  Non-causal.
 *
 * Conventions for every entry point:
 *   - Pointers named "device" are HIP device pointers; "host" pointers are
 *     ordinary CPU memory.  The caller owns every buffer it passes in.
 *   - Streams are hipStream_t values passed as void* (NULL = null stream).
 *   - Every call returns a bsa_status; no C++ exception crosses the ABI.
 *     Arguments are validated before anything is launched, so an error
 *     status leaves outputs untouched.  bsa_last_error() gives the text of
 *     the most recent error on the calling thread.
 */
#ifndef BSA_H
#define BSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BSA_OK = 0,
  BSA_ERR_INVALID_ARG = 1, /* malformed request, bad pointer or size        */
  BSA_ERR_UNSUPPORTED = 2, /* no eligible plan (dtype, d, geometry, limits)  */
  BSA_ERR_NO_MEMORY = 3,   /* device or host allocation failed               */
  BSA_ERR_HIP = 4,         /* a HIP runtime call failed                      */
  BSA_ERR_TABLE = 5        /* plan table missing, corrupt or mismatched      */
} bsa_status;

enum { BSA_DTYPE_BF16 = 1 };
/* Q, K, V and O share one layout, d contiguous, no padding:
 *   BSA_LAYOUT_HND  [batch][H][N][d]  (heads outermost within a batch entry)
 *   BSA_LAYOUT_NHD  [batch][N][H][d]  (a token's heads adjacent; rows of one
 *                                      head are H*d elements apart) */
enum { BSA_LAYOUT_HND = 0, BSA_LAYOUT_NHD = 1 };
enum { BSA_SPLIT_STREAM = -2 };

/* Opaque prepared plan: owns the block-CSR, the selected plan's metadata
 * (tile lists, membership bits, tasks) and its split-K workspace. */
typedef struct bsa_plan bsa_plan;

/* A runtime request (paper section 4.4: R = <A, M, B, x>; section 3 and
 * section 5.1: batch, head count and sequence length).  Every (batch entry,
 * head) pair is an independent attention head: planning, the regime
 * features and the task list see batch * H heads. */
typedef struct {
  int32_t H;         /* heads per batch entry, >= 1                             */
  int32_t N;         /* sequence length (queries = keys), >= 1                  */
  int32_t d;         /* head dimension: 32, 64, 128 or 256                      */
  int32_t block_q;   /* B_Q: 16, 32, 64, 128 or 256                             */
  int32_t block_kv;  /* B_KV: 16, 32, 64, 128 or 256                            */
  int32_t dtype;     /* BSA_DTYPE_BF16                                          */
  int32_t layout;    /* BSA_LAYOUT_HND or BSA_LAYOUT_NHD; NHD needs
                        N * H * d * 2 < 2^31 bytes (BSA_ERR_UNSUPPORTED)      */
  int32_t force_plan;  /* -1: regime table selection; >= 0: that catalog entry
                          (must be eligible, else BSA_ERR_UNSUPPORTED)          */
  int32_t force_split; /* -1: the plan's own split rule; 0: never split;
                          k > 0: at most k K/V items per task;
                          BSA_SPLIT_STREAM: equal ranges of the concatenated
                          tile-list entries, one per resident workgroup       */
  int32_t batch;       /* batch entries, 0 or 1 = one                          */
  int64_t workspace_limit; /* bytes of split-K workspace allowed; 0 = no limit */
  /* device, uint8 [batch][H][ceil(N/B_Q)][ceil(N/B_KV)], nonzero = active
   * (the same for both layouts).  Read
   * by kernels that bsa_plan_create queues on its stream: the caller may
   * overwrite it with work ordered after them on that stream, or once that
   * stream has been synchronized. */
  const uint8_t* mask;
} bsa_request;

/* Scalar facts about a prepared plan (host copy). */
typedef struct {
  int32_t plan_id;      /* catalog index of the selected plan                   */
  int32_t regime;       /* regime index in the plan table; -1 = lookup miss     */
  int32_t tile_q, tile_kv;       /* physical tile T = (T_Q, T_KV)                */
  int32_t coarsen_q, coarsen_kv; /* logical blocks per tile (1 if not coarsened)*/
  int32_t refine_q, refine_kv;   /* tiles per logical block (1 if not refined)  */
  int32_t split_items;  /* max K/V items per task; 0 = no split                 */
  int32_t max_row_nnz;  /* largest active-block count of a query-block row      */
  int64_t nnz_blocks;   /* active logical blocks                                */
  int64_t n_tile_rows;  /* rows of the tile list (query tiles or tile rows)     */
  int64_t n_items;      /* -1: the tile-list length lives on the device
                           (bsa_plan_export_tiles returns the tile count)       */
  int64_t n_tasks;      /* -1: the task count lives on the device
                           (bsa_plan_export_tasks returns it)                   */
  int64_t grid;         /* workgroups launched (>= n_tasks)                     */
  int64_t workspace_bytes; /* split-K workspace bound to the plan               */
  int64_t long_run_blocks; /* active blocks inside runs of length >= 2          */
  double density;       /* active / all logical blocks (section 5.1)            */
  double run_coverage;  /* long_run_blocks / active, 0 for an empty mask        */
  double row_skew;      /* max_row_nnz * rows / active blocks (>= 1), 0 if empty */
  double host_select_us;   /* host time spent in regime lookup + ranking scan   */
  int32_t tasks_predicted; /* 1: the task list was built speculatively for the
                              entry this request key selected last time, queued
                              before the statistics reached the host, and the
                              selection agreed; 0: built after the selection */
  int32_t split_threshold; /* rows (query tiles' tile-list rows) of more entries
                              than this are split into partitions of at most
                              split_items entries; 0 = no split (section 4.3
                              leaves the rule open: the balance rule keeps rows
                              of up to twice the mean length whole)          */
} bsa_plan_info;

/* Description of one catalog entry (paper section 4.4: native catalog). */
typedef struct {
  int32_t id;
  int32_t tile_q, tile_kv, d;
  int32_t split;        /* 0 = never split; s >= 1 = balance rule, partitions of
                           at most 2/s of the even share of entries per slot   */
  int32_t xcd_remap;    /* > 0: runs of this many consecutive tasks per XCD      */
  int32_t order;        /* 0 = query-tile order, 1 = longest task first, 2 = by
                           head, then by the median K/V column of the query
                           tile's row (tiles sharing K/V dispatched together) */
  char name[48];
} bsa_catalog_entry;

/* Create a plan for a request (paper section 3, "Online request path";
 * section 5.2: mask state, regime lookup, ranked fallback, launch
 * preparation).  Builds the mask state on `stream`, copies the statistics to
 * the host (the single synchronization of the request path), selects the
 * plan and prepares its metadata on `stream`.  On BSA_OK, *out
 * owns device memory until bsa_plan_destroy.  Errors: BSA_ERR_INVALID_ARG
 * (null pointers, non-positive sizes), BSA_ERR_UNSUPPORTED (dtype, layout,
 * d, geometry or forced plan not eligible), BSA_ERR_NO_MEMORY, BSA_ERR_HIP. */
bsa_status bsa_plan_create(const bsa_request* req, void* stream, bsa_plan** out);

/* Run a prepared plan: O = BSA(Q, K, V) (paper section 2.3: the attention
 * mainloop over the plan's tiles; section 4.3: the split-K merge).  Q, K, V, O are device bf16
 * buffers of batch * H * N * d elements in the request's layout; O is fully
 * written (zeros for empty rows).  Stream-ordered and asynchronous.  One run per plan may be in
 * flight at a time (the split-K workspace and, for the XCD organizations, the
 * task queues that each run resets are per plan).  Q/K/V may alias each
 * other; O must not alias Q, K or V. */
bsa_status bsa_run(const bsa_plan* plan, const void* q, const void* k, const void* v, void* o,
                   void* stream);

/* Same as bsa_run, and also returns the attention kernel's own duration in
 * milliseconds (kernel latency in the sense of paper section 7.1), measured with HIP events recorded on `stream` around that
 * launch (the call synchronizes on the end event). */
bsa_status bsa_run_timed(const bsa_plan* plan, const void* q, const void* k, const void* v,
                         void* o, void* stream, float* attn_ms, float* merge_ms);

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc: O = BSA(Q, K,
 * V) for `req` in one call, the same computation as bsa_plan_create +
 * bsa_run + bsa_plan_destroy, with tensors as for bsa_run, but every device
 * buffer of the request (mask state, tile and task lists, split-K workspace)
 * is carved from a fixed scratch array of 128 MiB per device that the
 * library holds until the process ends.  No hipMalloc, hipFree or pinned
 * host allocation is made (the array's address is looked up once per
 * device).  Plans whose buffers do not fit the space left after the mask
 * state are not eligible, so the ranked selection may pick a different plan
 * than bsa_plan_create; no task list is built speculatively.
 * Synchronizes `stream` once (for the mask statistics) and returns once O's
 * kernels are queued.  Every call on one GPU uses that GPU's one scratch
 * array, which keeps the last call's contents: calls that overlap on one GPU
 * (on different streams or threads) race and must be ordered by the caller;
 * calls on one stream are ordered by it.  Errors: those of bsa_plan_create
 * and bsa_run, checked before any launch; BSA_ERR_UNSUPPORTED with the sizes
 * in bsa_last_error() when the request's mask state, or every eligible
 * plan, needs more than the scratch (the block-CSR size is known only after
 * the mask-state kernels have run; O is then left untouched). */
bsa_status bsa_attention_noalloc(const bsa_request* req, const void* q, const void* k, const void* v,
                                 void* o, void* stream);

/* Release a plan and the metadata it prepared (paper section 5.2, "Launch
 * preparation").  Waits for the plan's latest stream work (its creation or
 * its most recent run) first; runs must not be in flight on other streams.
 * NULL is accepted. */
bsa_status bsa_plan_destroy(bsa_plan* plan);

/* Copy the plan's scalar facts to *info (host): the plan tuple
 * <g_Q, g_KV, sigma, e> of paper section 4.1 as chosen, plus the request's
 * mask statistics (section 5.1). */
bsa_status bsa_plan_get_info(const bsa_plan* plan, bsa_plan_info* info);

/* Export the physical tiles the attention kernels will visit (paper section
 * 2.2: a plan must cover exactly the interactions E(M); section 4.2: the
 * Direct, Coarsened and Refined mappings), in task order,
 * to host arrays of capacity `cap` records: head, query-tile index, K/V tile
 * index (in units of T_Q and T_KV tokens) and the membership bits of the
 * tile (bit a*coarsen_kv + b set = logical block (a, b) inside the tile is
 * active; all bits of the tile's coarsen_q*coarsen_kv set when not
 * coarsened).  *count receives the number of records; BSA_ERR_INVALID_ARG if
 * cap is too small (count still set).  For coverage checks only. */
bsa_status bsa_plan_export_tiles(const bsa_plan* plan, int32_t* head, int32_t* q_tile,
                                 int32_t* kv_tile, uint32_t* bits, int64_t cap, int64_t* count);

/* Export the plan's task list in dispatch order (paper section 3: the task
 * organization's grouping, traversal order and K/V partitions) to host arrays
 * of capacity `cap`: head, query-tile index, first and one-past-last entry of
 * the tile-list row (offsets into the plan's tile list, whose row for query
 * tile qt of head h is h * rows_per_head + qt / refine_q) and the split-K
 * workspace slot (-1 when the query tile is not split).  *count receives the
 * number of tasks; BSA_ERR_INVALID_ARG if cap is too small (count still set).
 * Synchronizes the device.  For organization checks only. */
bsa_status bsa_plan_export_tasks(const bsa_plan* plan, int32_t* head, int32_t* q_tile,
                                 int32_t* begin, int32_t* end, int32_t* slot, int64_t cap,
                                 int64_t* count);

/* Copy the shared block-CSR (paper section 3 and section 5.2: the mask state
 * mu(M) every plan of the request reads; row offsets [H*ceil(N/B_Q)+1] and
 * column indices [nnz_blocks]) to host arrays. */
bsa_status bsa_plan_export_csr(const bsa_plan* plan, int32_t* row_ptr, int32_t* cols,
                               int64_t cap_cols);

/* Catalog introspection (paper section 4.4: the native catalog C_A). */
int32_t bsa_catalog_size(void);
bsa_status bsa_catalog_get(int32_t id, bsa_catalog_entry* out);

/* Eligibility predicate Eligible(P, R) for catalog entry `id` and the
 * request's geometry and tensor properties (section 4.4); host only, touches
 * no GPU.  *eligible receives 1 or 0. */
bsa_status bsa_plan_eligible(int32_t id, const bsa_request* req, int32_t* eligible);

/* Regime lookup and ranked fallback (section 5.2) on host-side features
 * (density, run coverage, row skew -- see bsa_plan_info): returns the selected
 * catalog id, the regime index (-1 on a lookup miss, in which case the key's
 * base plan is the sole candidate) and BSA_OK, or BSA_ERR_UNSUPPORTED when no
 * candidate is eligible.  Touches no GPU. */
bsa_status bsa_select(const bsa_request* req, double density, double run_coverage, double row_skew,
                      int32_t* plan_id, int32_t* regime);

/* Base plan of the request's key (paper section 5.1: the catalog plan that
 * ends every ranking of the key and is the sole candidate on a lookup miss):
 * Direct (T = B) with the default organization when the catalog has it, else
 * the eligible entry with the smallest tile.  Host only.  *plan_id receives
 * the catalog id, or -1 with BSA_ERR_UNSUPPORTED when no entry is eligible. */
bsa_status bsa_base_plan(const bsa_request* req, int32_t* plan_id);

/* Plan cache for warm exact repeats (paper section 7.4: repeats of a request
 * reuse its prepared plan state instead of planning again).  A cache holds up
 * to `capacity` prepared plans (1..64) together with a device copy of each
 * plan's mask, at most `max_mask_bytes` of copies in total (0 = no limit),
 * and evicts the least recently used.  Host object; the mask copies and
 * plans live on the device that is current at bsa_plan_cache_get.  Errors:
 * BSA_ERR_INVALID_ARG, BSA_ERR_NO_MEMORY. */
typedef struct bsa_plan_cache bsa_plan_cache;
bsa_status bsa_plan_cache_create(int32_t capacity, int64_t max_mask_bytes, bsa_plan_cache** out);

/* Returns a prepared plan for `req`.  Cached plans of the same request
 * (H, N, d, B, dtype, layout, force_plan, force_split, workspace_limit) are
 * compared with req->mask byte for byte on the GPU (one compare kernel, the
 * result read back through host-coherent memory); an identical one is
 * returned with *hit = 1 and no planning work.  Otherwise a plan is created
 * as by bsa_plan_create, the mask is copied (stream-ordered) into the cache
 * and *hit = 0.  The returned plan belongs to the cache: it stays valid until
 * a later bsa_plan_cache_get evicts it or the cache is destroyed, and must
 * not be passed to bsa_plan_destroy.  A returned plan must not have a run in
 * flight on another stream (one run per plan at a time).  Errors: those of
 * bsa_plan_create. */
bsa_status bsa_plan_cache_get(bsa_plan_cache* cache, const bsa_request* req, void* stream, bsa_plan** out,
                              int32_t* hit);

/* O = BSA(Q, K, V) for `req` through the cache: bsa_plan_cache_get followed
 * by bsa_run of the returned plan, with tensors as for bsa_run.  On a
 * repeat the most recently used candidate plan is queued right behind the
 * mask comparison, its kernels guarded by the comparison's verdict (they do
 * nothing when it differs), so the host's wait for the verdict overlaps the
 * attention work; another matching candidate or a new plan then runs after
 * it and writes O.  *hit as for bsa_plan_cache_get.  Stream-ordered; returns
 * once O's kernels are queued.  Errors: those of bsa_plan_cache_get and
 * bsa_run. */
bsa_status bsa_plan_cache_run(bsa_plan_cache* cache, const bsa_request* req, const void* q, const void* k,
                              const void* v, void* o, void* stream, int32_t* hit);

/* Destroys every cached plan (after their latest stream work) and the cache. */
bsa_status bsa_plan_cache_destroy(bsa_plan_cache* cache);

/* Load a versioned plan table (text artifact; paper section 5.1: the regime
 * table compiled offline per architecture) replacing the built-in one.
 * BSA_ERR_TABLE if unreadable, malformed, or built for another architecture
 * or catalog.  NULL restores the built-in table. */
bsa_status bsa_table_load(const char* path);

/* Version strings of the loaded table and of the catalog (the versioning of
 * paper section 5.1's table against section 4.4's catalog). */
const char* bsa_table_version(void);
const char* bsa_catalog_hash(void);

/* Error reporting (library utilities with no counterpart in the paper):
 * the name of a status code, and the calling thread's last error message. */
const char* bsa_status_string(int32_t status);
const char* bsa_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* BSA_H */
