/*
 * tt_bag.h -- C ABI of libttbag: TT-EmbeddingBag on AMD MI355X (gfx950).
 *
 * An EmbeddingBag whose num_embeddings x embedding_dim table W is never stored.
 * "FBTT-Embedding" README, sections "Parameters" and "Initialization": W is held
 * as three Tensor-Train cores; core k has logical shape R_{k-1} x p_k x q_k x R_k
 * with ranks {1, R1, R2, 1}, prod(p) >= num_embeddings and prod(q) == embedding_dim.
 * Row i splits into (i1,i2,i3) and column j into (j1,j2,j3), both row-major mixed
 * radix (i = (i1*p2 + i2)*p3 + i3), and
 *     W[i][j] = sum_{r1,r2} G1[0][i1][j1][r1] G2[r1][i2][j2][r2] G3[r2][i3][j3][0].
 * The forward pass pools the requested rows per bag like PyTorch's EmbeddingBag
 * (README intro; "EmbeddingBag and Product-Key Memory Layers", tensorflow/addons
 * #2201: gather + weighted sum, without materialising the gathered rows).  The
 * backward pass forms the core gradients and applies SGD in place ("Parameters",
 * entry `sparse`; "Fused Kernel").  An optional HBM cache of decompressed rows
 * serves frequent indices ("Software Cache").  Several tables of one shape can be
 * batched in one call ("TableBatchedTTEmbeddingBag").
 *
 * Conventions for every entry point
 *  - Pointers are DEVICE pointers unless the comment says host.  `stream` is a
 *    hipStream_t (NULL = the default stream).  Every call is asynchronous on
 *    `stream` and does not synchronise the host, except tt_cache_populate (which
 *    reads a size back) and the diagnostic tt_bag_dedup_counts.
 *  - HIP graphs: the calls that enqueue kernels only (the grouping, forward and
 *    backward calls, planned or not, tt_cache_lookup) may be captured into a HIP
 *    graph and replayed.  Their grid-wide flags and counters carry a tag made of
 *    a host part and the workspace's own count of groupings / forwards, which the
 *    kernels move on themselves, so a replay tags them afresh.  Calls that read
 *    back or clear memory with a memset (tt_cache_create, tt_cache_populate,
 *    tt_cache_import, tt_bag_route with nnz = 0) are not for capture.
 *  - Ownership: the caller owns every buffer it passes, including the workspace.
 *    The library allocates device memory only inside tt_cache_create and frees it
 *    only in tt_cache_destroy; it keeps no caller pointer between calls.
 *  - Return value: TT_OK (0) or a negative TT_E* code.  A negative return means
 *    the arguments were rejected on the host and NOTHING was enqueued.
 *  - Content errors that only the device can see (an index outside [0, E), a
 *    non-CSR offsets array, a cache slot outside [0, cache_size), a full count
 *    table) OR bits into the sticky word *dev_status (device memory, never
 *    cleared by the library).  The offending elements are skipped without any
 *    out-of-bounds access; the outputs are then unspecified.
 *  - One workspace must not be used by two calls that may run concurrently.
 *
 * Core storage (device, fp32): cores[k] points to T consecutive tables of core k,
 * each stored slice-major [p_k][R_{k-1}][q_k][R_k], so the slice for one index
 * i_k is contiguous.  (The pages give only the logical order R_{k-1} x p_k x q_k
 * x R_k; slice-major is that order with the first two axes swapped.)
 *
 * Supported shapes (others return TT_ESHAPE): 1 <= T; 1 <= R1, R2 <= 64;
 * q1 in {1, 2, 4}; 1 <= q2; 1 <= q3 <= 16; D <= 1024; T*p_k + 1 <= 8192 for each
 * k (with a cache: T*p1 + 513 <= 8192); num_embeddings <= prod(p) < 2^40.
 */
#ifndef TT_BAG_H
#define TT_BAG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* return codes */
#define TT_OK          0
#define TT_EINVAL     (-1)  /* null pointer, negative size, lr not finite, ...  */
#define TT_ESHAPE     (-2)  /* descriptor inconsistent or outside the envelope */
#define TT_EWORKSPACE (-3)  /* workspace too small or not 256-byte aligned     */
#define TT_EHIP       (-4)  /* a HIP runtime call failed                       */
#define TT_EFULL      (-5)  /* cache capacity exceeded at create               */

/* bits OR-ed into *dev_status by the device */
#define TT_DEV_BAD_INDEX   1  /* index < 0 or >= num_embeddings (element skipped) */
#define TT_DEV_BAD_OFFSETS 2  /* offsets[0] != 0, offsets not non-decreasing, or
                                 offsets[T*B] != nnz                             */
#define TT_DEV_BAD_SLOT    4  /* cache slot >= cache_size (element skipped)       */
#define TT_DEV_HASH_FULL   8  /* frequency table full: new keys were not counted  */
#define TT_DEV_STALE_PLAN 16  /* a planned call found another call's plan in ws  */
#define TT_DEV_SYNC_TIMEOUT 32 /* grouping: a grid-wide barrier of the cooperative
                                  launch was not reached in time (no plan made)  */

/* Shape of one TT table ("Parameters": num_embeddings, embedding_dim = prod(q),
 * tt_p_shapes, tt_q_shapes, tt_ranks) and the number of tables batched
 * ("TableBatchedTTEmbeddingBag": num_tables, all of one shape). */
typedef struct tt_desc {
    int32_t num_tables;      /* T >= 1                                        */
    int64_t num_embeddings;  /* E, 1 <= E <= p[0]*p[1]*p[2]                    */
    int32_t p[3];            /* tt_p_shapes                                    */
    int32_t q[3];            /* tt_q_shapes; embedding_dim D = q[0]*q[1]*q[2]  */
    int32_t ranks[2];        /* tt_ranks (R1, R2); full ranks {1, R1, R2, 1}   */
    int32_t pooling;         /* TT_POOL_SUM (0) or TT_POOL_MEAN (1)            */
} tt_desc;
/* Pooling of a bag (PyTorch EmbeddingBag's modes "sum" and "mean"): the mean is the
 * (weighted) sum divided by the bag's number of elements; an empty bag gives zeros.
 * The backward scales each element's gradient by the same 1 / length. */
#define TT_POOL_SUM  0
#define TT_POOL_MEAN 1

/* A view of the software cache for one forward/backward call ("Software Cache").
 * slots[n] >= 0 makes element n a hit: the forward reads rows[slots[n]] instead
 * of the TT row, and the backward applies SGD to that row instead of the cores
 * (write-back).  slots[n] < 0 is a miss.  Only with num_tables == 1. */
typedef struct tt_cache_view {
    const int32_t *slots;    /* [nnz], from tt_cache_lookup                    */
    float *rows;             /* [cache_size][D] decompressed rows              */
    int64_t cache_size;
} tt_cache_view;

/* Bytes of workspace that tt_bag_forward / tt_bag_backward_sgd / tt_bag_route
 * need for nnz indices, num_bags bags per table and a cache of cache_size rows
 * (0 = no cache).  Returns 0 if the descriptor is rejected. */
size_t tt_bag_workspace_size(const tt_desc *desc, int64_t nnz, int64_t num_bags,
                             int64_t cache_size);

/*
 * Forward (README "How FBTT-Embedding works": same semantics as EmbeddingBag's
 * sum mode, with optional per-sample weights as in tensorflow/addons #2201).
 *   indices  [nnz] int64, rows of each table in [0, E)
 *   offsets  [T*num_bags + 1] int64, CSR: bag b holds positions
 *            [offsets[b], offsets[b+1]); offsets[0] = 0, offsets[T*num_bags] = nnz.
 *            Bags are table-major: bag b belongs to table b / num_bags.
 *   per_sample_weights [nnz] fp32 or NULL (all ones)
 *   cache    NULL, or a cache view (hits are pooled from cache rows)
 *   out      [T*num_bags][D] fp32, fully overwritten; an empty bag gives zeros.
 *   ws       workspace of ws_bytes >= tt_bag_workspace_size(...), 256-B aligned
 */
int tt_bag_forward(const tt_desc *desc, const float *const cores[3],
                   const int64_t *indices, int64_t nnz, const int64_t *offsets,
                   int64_t num_bags, const float *per_sample_weights,
                   const tt_cache_view *cache, float *out,
                   void *ws, size_t ws_bytes, int32_t *dev_status, void *stream);

/*
 * Backward with fused SGD ("Parameters", `sparse`=True with OptimType.SGD;
 * "Fused Kernel"): with L = sum_b <grad_out[b], out[b]>, computes the gradient of
 * every core slice and cache row touched by this batch at the current values and
 * applies  x <- x - lr * dL/dx  in place to exactly those slices/rows.  Gradients
 * are not returned.  Duplicate indices add up.  No gradient with respect to the
 * per-sample weights is formed.  Same argument meaning as tt_bag_forward;
 * grad_out is [T*num_bags][D] fp32.  The result is bit-reproducible run to run
 * (the reductions have a fixed order).
 */
int tt_bag_backward_sgd(const tt_desc *desc, float *const cores[3],
                        const int64_t *indices, int64_t nnz, const int64_t *offsets,
                        int64_t num_bags, const float *per_sample_weights,
                        const tt_cache_view *cache, const float *grad_out, float lr,
                        void *ws, size_t ws_bytes, int32_t *dev_status, void *stream);

/*
 * Forward for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): tt_bag_forward
 * without a workspace argument.  The grouping and the forward run in a scratch array
 * that the library holds in static device storage, TT_STATIC_SCRATCH_BYTES per GPU
 * (each GPU the library runs on keeps its copy until the process ends); the call
 * allocates nothing.  The batch may use at most that much of it: the forward's share
 * of tt_bag_workspace_size (about 80 bytes per index plus the bin tables: under 1 MiB
 * for 10,240 indices of the README shape); a larger batch returns TT_EWORKSPACE and
 * enqueues nothing.  Every call on one GPU shares that GPU's array, so calls that may
 * overlap on one GPU (other streams, other host threads) race and must be ordered by
 * the caller.  Arguments and results as tt_bag_forward.
 */
#define TT_STATIC_SCRATCH_BYTES 8388608
int tt_bag_forward_static(const tt_desc *desc, const float *const cores[3],
                          const int64_t *indices, int64_t nnz, const int64_t *offsets,
                          int64_t num_bags, const float *per_sample_weights,
                          const tt_cache_view *cache, float *out, int32_t *dev_status,
                          void *stream);

/*
 * Split of one training step into its grouping and its arithmetic.  tt_bag_plan
 * runs the grouping step (index split, bag ids, validation, the stable sorts) and
 * leaves the result in `ws`.  tt_bag_forward_planned / tt_bag_backward_sgd_planned
 * take exactly the arguments of tt_bag_forward / tt_bag_backward_sgd but reuse
 * that grouping, so a forward and backward over one batch group it only once.
 * The plan also holds each element's per-sample weight (NULL = all ones).
 * The workspace records a fingerprint of the plan's shape, sizes and input
 * pointers (indices, offsets, weights, cache slots); a planned call whose arguments do not
 * match it does nothing but set TT_DEV_STALE_PLAN in *dev_status.  The caller
 * must re-plan after changing the CONTENTS of those buffers (the fingerprint
 * cannot see that).  tt_bag_forward = plan + forward_planned, and
 * tt_bag_backward_sgd = plan + backward_sgd_planned (the same for the Adagrad and
 * gradient variants below).
 */
int tt_bag_plan(const tt_desc *desc, const int64_t *indices, int64_t nnz,
                const int64_t *offsets, int64_t num_bags, const float *per_sample_weights,
                const tt_cache_view *cache, void *ws, size_t ws_bytes, int32_t *dev_status,
                void *stream);

int tt_bag_forward_planned(const tt_desc *desc, const float *const cores[3],
                           const int64_t *indices, int64_t nnz, const int64_t *offsets,
                           int64_t num_bags, const float *per_sample_weights,
                           const tt_cache_view *cache, float *out,
                           void *ws, size_t ws_bytes, int32_t *dev_status, void *stream);

int tt_bag_backward_sgd_planned(const tt_desc *desc, float *const cores[3],
                                const int64_t *indices, int64_t nnz, const int64_t *offsets,
                                int64_t num_bags, const float *per_sample_weights,
                                const tt_cache_view *cache, const float *grad_out, float lr,
                                void *ws, size_t ws_bytes, int32_t *dev_status, void *stream);

/*
 * Backward with fused Adagrad ("Parameters": `sparse`=True with the Adagrad
 * optimizer type, whose `eps` is added to the denominator; the update itself is the
 * diagonal Adagrad of Duchi, Hazan and Singer 2011).  Same gradient as
 * tt_bag_backward_sgd; then, for every element x of a touched core slice or cache
 * row, with its gradient g and its running sum of squared gradients S:
 *     S <- S + g*g;   x <- x - lr * g / (sqrt(S) + eps)
 * Untouched slices/rows keep x and S.
 *   state      [3] device pointers, state[k] in the layout of cores[k] (fp32; start
 *              at zero or any non-negative value); updated in place
 *   state_rows [cache_size][D] fp32 running sums of the cache rows (required with a
 *              cache, ignored without)
 *   eps        finite and >= 0; lr finite
 * Bit-reproducible run to run like tt_bag_backward_sgd.
 */
int tt_bag_backward_adagrad(const tt_desc *desc, float *const cores[3],
                            const int64_t *indices, int64_t nnz, const int64_t *offsets,
                            int64_t num_bags, const float *per_sample_weights,
                            const tt_cache_view *cache, const float *grad_out, float lr, float eps,
                            float *const state[3], float *state_rows,
                            void *ws, size_t ws_bytes, int32_t *dev_status, void *stream);

int tt_bag_backward_adagrad_planned(const tt_desc *desc, float *const cores[3],
                                    const int64_t *indices, int64_t nnz, const int64_t *offsets,
                                    int64_t num_bags, const float *per_sample_weights,
                                    const tt_cache_view *cache, const float *grad_out, float lr,
                                    float eps, float *const state[3], float *state_rows,
                                    void *ws, size_t ws_bytes, int32_t *dev_status, void *stream);

/*
 * Backward without an update ("Parameters": `sparse`=False, the gradient with
 * respect to the TT cores or the cache is returned to an external optimizer).  The
 * cores and cache rows are only read.
 *   grad_cores [3] device pointers, grad_cores[k] in the layout of cores[k] (T
 *              tables, slice-major), fully overwritten: dL/dG on the slices this
 *              batch touches, zero elsewhere
 *   grad_rows  [cache_size][D] fp32, fully overwritten: dL/d(row) for rows with
 *              hits (the sum of w * grad_out over them), zero elsewhere (required
 *              with a cache, ignored without)
 * An empty batch (nnz = 0) writes all-zero gradients.  Bit-reproducible run to run.
 */
int tt_bag_backward_grad(const tt_desc *desc, const float *const cores[3],
                         const int64_t *indices, int64_t nnz, const int64_t *offsets,
                         int64_t num_bags, const float *per_sample_weights,
                         const tt_cache_view *cache, const float *grad_out,
                         float *const grad_cores[3], float *grad_rows,
                         void *ws, size_t ws_bytes, int32_t *dev_status, void *stream);

int tt_bag_backward_grad_planned(const tt_desc *desc, const float *const cores[3],
                                 const int64_t *indices, int64_t nnz, const int64_t *offsets,
                                 int64_t num_bags, const float *per_sample_weights,
                                 const tt_cache_view *cache, const float *grad_out,
                                 float *const grad_cores[3], float *grad_rows,
                                 void *ws, size_t ws_bytes, int32_t *dev_status, void *stream);

/*
 * Gradient with respect to the per-sample weights (the survey's N4 variant; PyTorch's
 * EmbeddingBag returns it when the weights require a gradient): for every element n,
 *     grad_weights[n] = <grad_out[bag n], W[indices[n]]>   (times 1 / bag length with
 *                                                         mean pooling),
 * the row being the cache row for a hit; skipped elements get 0.  Cores and rows are
 * only read.  grad_weights [nnz] fp32, fully overwritten.  TT_ESHAPE when a work
 * item's rows (32 x D floats) do not fit the forward kernel's LDS (D > 512).  Bit-
 * reproducible run to run.
 */
int tt_bag_weight_grad(const tt_desc *desc, const float *const cores[3],
                       const int64_t *indices, int64_t nnz, const int64_t *offsets,
                       int64_t num_bags, const float *per_sample_weights,
                       const tt_cache_view *cache, const float *grad_out, float *grad_weights,
                       void *ws, size_t ws_bytes, int32_t *dev_status, void *stream);

int tt_bag_weight_grad_planned(const tt_desc *desc, const float *const cores[3],
                               const int64_t *indices, int64_t nnz, const int64_t *offsets,
                               int64_t num_bags, const float *per_sample_weights,
                               const tt_cache_view *cache, const float *grad_out,
                               float *grad_weights, void *ws, size_t ws_bytes,
                               int32_t *dev_status, void *stream);

/*
 * The grouping step of both passes, exposed for inspection and tests: splits
 * every index, finds its bag, and sorts the elements stably so that misses come
 * first ordered by (table, i2, i1) and then by position, followed by cache hits
 * ordered by (slot, position), followed by the skipped elements by position.
 *   order_out     [nnz] int32: element positions in that order
 *   group_off_out [T*p2 + 2] int32: misses of group g = table*p2 + i2 occupy
 *                 order_out[group_off_out[g] .. group_off_out[g+1]); hits occupy
 *                 [group_off_out[T*p2], group_off_out[T*p2+1]).
 */
int tt_bag_route(const tt_desc *desc, const int64_t *indices, int64_t nnz,
                 const int64_t *offsets, int64_t num_bags, const int32_t *slots,
                 int64_t cache_size, int32_t *order_out, int32_t *group_off_out,
                 void *ws, size_t ws_bytes, int32_t *dev_status, void *stream);

/* ---------------------------------------------------------------- cache
 * "Software Cache": the access frequency of every looked-up index is counted in
 * an open-addressing hash table of hashtbl_size entries; tt_cache_populate fills
 * the cache with the (at most cache_size) most frequent indices, ties broken by
 * the smaller index, slot = rank in that order, each row decompressed from the
 * current cores.  Counts are never reset.  The pages describe a 32-way
 * set-associative LFU; this cache is fully associative exact top-K (the
 * replacement policy only decides which rows are cached, not the arithmetic).
 */
typedef struct tt_cache tt_cache;

/* Replacement policies of tt_cache_populate:
 *  TT_CACHE_TOPK   fully associative: the cache_size most frequent indices, slot = rank;
 *                  every populate rebuilds every row from the cores.
 *  TT_CACHE_LFU32  the pages' 32-way set-associative LFU ("Software Cache"; hash, ways
 *                  and row handling are this library's reading): slot = set * 32 + way,
 *                  set = (splitmix64(index) >> 32) mod (cache_size / 32), splitmix64 being
 *                  the output finalizer of Steele, Lea and Flood (2014).  Each populate
 *                  keeps in every set the 32 counted indices of that set with the highest
 *                  counts (ties: smaller index).  An index that stays keeps its slot and
 *                  its row (with the updates the backward applied to it); newcomers take
 *                  the freed ways in ascending order, in (count desc, index asc) order,
 *                  and only their rows are rebuilt from the cores.  Evicted rows are
 *                  dropped (their updates are not written back to the cores).
 *                  cache_size must be a multiple of 32. */
#define TT_CACHE_TOPK  0
#define TT_CACHE_LFU32 1

/* Allocates the count table, the index->slot map and populate's scratch for a
 * table of shape *desc (num_tables must be 1).  *out receives a host handle.
 * tt_cache_create is tt_cache_create_policy with TT_CACHE_TOPK. */
int tt_cache_create(tt_cache **out, const tt_desc *desc, int64_t cache_size,
                    int64_t hashtbl_size);
int tt_cache_create_policy(tt_cache **out, const tt_desc *desc, int64_t cache_size,
                           int64_t hashtbl_size, int policy);

/* slot_out[n] = slot of indices[n] in the cache, or -1.  With count_freq != 0 every
 * element with an index in [0, E) also adds one to its index's count. */
int tt_cache_lookup(tt_cache *c, const int64_t *indices, int64_t nnz, int32_t *slot_out,
                    int count_freq, int32_t *dev_status, void *stream);

/* Re-selects the cached indices from the counts (policy above) and writes the rows
 * it rebuilds into rows ([cache_size][D] fp32): TT_CACHE_TOPK fills slots
 * 0 .. n_filled-1; TT_CACHE_LFU32 rebuilds the newcomers' slots and n_filled is the
 * number of occupied slots.  *n_filled is a HOST pointer; this call synchronises
 * `stream`. */
int tt_cache_populate(tt_cache *c, const float *const cores[3], float *rows,
                      int64_t *n_filled, void *stream);

/* cached_out[s] = index held in slot s for s < n_filled (int64 device buffer of
 * cache_size entries; entries past n_filled are -1). */
int tt_cache_cached_indices(tt_cache *c, int64_t *cached_out, void *stream);

/* The cache state (the rows are the caller's): the index of every slot
 * (cached [cache_size] int64, -1 = empty) and the raw frequency table (keys
 * [hashtbl_size] int64, -1 = unused entry; counts [hashtbl_size] int32).  Device
 * buffers, asynchronous on `stream`.  tt_cache_import restores a state exported from a
 * cache created with the same descriptor, sizes and policy (its content is not
 * checked) and rebuilds the index->slot map; lookups and populates then behave as in
 * the exporting cache. */
int tt_cache_export(tt_cache *c, int64_t *cached_out, int64_t *keys_out, int32_t *counts_out,
                    void *stream);
int tt_cache_import(tt_cache *c, const int64_t *cached, const int64_t *keys,
                    const int32_t *counts, void *stream);

int tt_cache_destroy(tt_cache *c);

/* ---------------------------------------------------------------- initialisation
 * "Parameters" (`weight_dist`): the cores are drawn i.i.d. from the named distribution,
 * or ("approx-" variants) so that the entries of the full table follow it; the TT-Rec
 * abstract recommends sampled-Gaussian cores (= TT_INIT_APPROX_NORMAL here).  A table
 * entry sums R1*R2 products of one entry per core, so zero-mean i.i.d. cores of
 * variance v give Var(W) = R1 R2 v^3; the approx- variants pick v to match the target's
 * mean (0) and variance:
 *   TT_INIT_UNIFORM         cores U(-scale, scale)
 *   TT_INIT_NORMAL          cores N(0, scale^2)
 *   TT_INIT_APPROX_UNIFORM  W with the variance of U(-scale, scale): cores U(-c, c),
 *                           c^2 / 3 = (scale^2 / (3 R1 R2))^(1/3)
 *   TT_INIT_APPROX_NORMAL   W with the variance of N(0, scale^2): cores N(0, v),
 *                           v = (scale^2 / (R1 R2))^(1/3)
 * Random numbers: Philox4x32-10 (Salmon et al., SC 2011), key = seed (low word first),
 * counter = (n mod 2^32, n >> 32, k, 0) for element n of core k in its stored array
 * (all tables, slice-major); u = ((x >> 9) + 1/2) 2^-23 from the counter's words x0, x1;
 * uniform a (2 u0 - 1); normal by Box-Muller, a sqrt(-2 ln u0) cos(2 pi u1).
 * Fills cores[0..2] (device, the layout of the forward) on `stream`; scale finite, >= 0. */
#define TT_INIT_UNIFORM        0
#define TT_INIT_NORMAL         1
#define TT_INIT_APPROX_UNIFORM 2
#define TT_INIT_APPROX_NORMAL  3
int tt_init_cores(const tt_desc *desc, float *const cores[3], int dist, float scale,
                  uint64_t seed, void *stream);

/* Automatic shapes ("Initialization": without p / q shapes the sizes are factored
 * automatically; the pages state no rule).  Host function, 1 <= n < 2^31.
 *   exact != 0 (q: q1 q2 q3 == n, q1 in {1, 2, 4}, q3 <= 16 as the kernels require;
 *              TT_ESHAPE if there is none): the triple with the smallest largest
 *              factor, then the largest smallest factor, then the smallest q1, then the
 *              largest q2;
 *   exact == 0 (p: p1 p2 p3 >= n): p3 = the smallest m with m^3 >= n, p1 <= p2 <= p3
 *              with the smallest product, then the smallest p1. */
int tt_factorize(int64_t n, int exact, int32_t out[3]);

/* ---------------------------------------------------------------- full weight
 * Rows first .. first+count-1 of table `table` decompressed ("Initialization": a row is
 * the chain G1[i1] G2[i2] G3[i3]) into out [count][D] fp32 (device, fully overwritten),
 * on `stream`.  first + count <= num_embeddings.  TT_ESHAPE when q3 > 16 or when
 * T = G1[i1] G2[i2], a G2 slice, a G1 slice and one G3 slice do not fit the 160 KiB of
 * LDS together. */
int tt_full_weight(const tt_desc *desc, const float *const cores[3], int table, int64_t first,
                   int64_t count, float *out, void *stream);

/* ---------------------------------------------------------------- backward over distinct indices
 * The loss is linear in the rows, so the gradient of a batch equals that of a virtual
 * batch with one element per distinct (table, index) u, weight 1, alone in its bag, whose
 * grad_out row is sum_{n: idx_n = u} w_n grad_out[bag n] (times 1/len with mean pooling).
 * With repeated indices (Zipf-skewed batches) the virtual batch is smaller and a hot index
 * costs one element.  No cache.
 *   tt_bag_plan_dedup: the grouping of the batch (as tt_bag_plan, so tt_bag_forward_planned
 *     on the same ws runs the forward), the sort by index, the runs of equal indices, and
 *     the grouping of the virtual batch.  The number of distinct indices stays on the
 *     device: the virtual batch's launches are sized by its bounds (nnz elements, nnz bags
 *     per table) and its kernels read the count, so the call does not wait on the device
 *     and may be captured.  info (host array) receives those bounds, info[0] = info[1] =
 *     nnz; pass it unchanged to the backward, which rejects anything else (TT_EINVAL).
 *   tt_bag_backward_sgd_dedup / _grad_dedup: the grad_out sums of the runs (fixed order:
 *     32-element chunks of the sorted order, then each run's pieces in order), then the
 *     planned three-core backward (SGD, or dense gradients fully overwritten) on the
 *     virtual batch.  Same arguments as the planned calls plus info.
 * Workspace: tt_bag_workspace_size_dedup bytes (256-byte aligned); TT_ESHAPE when T * nnz
 * reaches 2^30 or the sort key (bits of T*E plus bits of nnz) exceeds 64 bits. */
size_t tt_bag_workspace_size_dedup(const tt_desc *desc, int64_t nnz, int64_t num_bags);
int tt_bag_plan_dedup(const tt_desc *desc, const int64_t *indices, int64_t nnz,
                      const int64_t *offsets, int64_t num_bags, const float *per_sample_weights,
                      void *ws, size_t ws_bytes, int32_t *dev_status, int64_t info[2],
                      void *stream);
int tt_bag_backward_sgd_dedup(const tt_desc *desc, float *const cores[3], const int64_t *indices,
                              int64_t nnz, const int64_t *offsets, int64_t num_bags,
                              const float *per_sample_weights, const float *grad_out, float lr,
                              const int64_t info[2], void *ws, size_t ws_bytes,
                              int32_t *dev_status, void *stream);
int tt_bag_backward_grad_dedup(const tt_desc *desc, const float *const cores[3],
                               const int64_t *indices, int64_t nnz, const int64_t *offsets,
                               int64_t num_bags, const float *per_sample_weights,
                               const float *grad_out, float *const grad_cores[3],
                               const int64_t info[2], void *ws, size_t ws_bytes,
                               int32_t *dev_status, void *stream);
/* Diagnostics (host-synchronous: waits for `stream`): the distinct-index counts of the
 * batch last planned by tt_bag_plan_dedup in ws, into the host array counts[T + 1]:
 * counts[t] = distinct (index) of the tables before t, counts[T] = all of them (invalid
 * indices not counted).  Same sizes as the plan; not for capture. */
int tt_bag_dedup_counts(const tt_desc *desc, int64_t nnz, int64_t num_bags, const void *ws,
                        size_t ws_bytes, int64_t *counts, void *stream);

/* ---------------------------------------------------------------- d-core tables
 * Tables of any number d of cores ("FBTT-Embedding" README, "Parameters": tt_p_shapes,
 * tt_q_shapes and tt_ranks are lists of one length; "Initialization": core k has shape
 * R_{k-1} x p_k x q_k x R_k with R_0 = R_d = 1).  The row index is split over p and the
 * column index over q row-major; the row is the product of the d slice matrices.
 * Cores are stored slice-major [p_k][R_{k-1}][q_k][R_k], T tables one after the other in
 * each core's buffer, as for three cores.
 *
 * The d cores are cut into three groups of consecutive cores; each group is multiplied
 * out into one (dense) core in the workspace, the three-core kernels run on those, and
 * their gradients are split back onto the d cores by the product rule.  The cut is the
 * one with the least dense work among those the three-core path accepts (q of the first
 * group in {1, 2, 4}, of the last <= 16, at most 8191 / T slices per group, ranks <= 64);
 * TT_ESHAPE when there is none.  No cache.  Semantics as tt_bag_forward /
 * tt_bag_backward_sgd / tt_bag_backward_grad, with d core pointers (host arrays of
 * device pointers).  Gradients (grad_d) are dense and fully overwritten: zero on slices
 * no index touched.  SGD (sgd_d) changes only entries with a nonzero gradient.
 * The workspace (tt_bag_workspace_size_d bytes, 256-byte aligned) holds the three-core
 * workspace, the multiplied-out cores with their gradients and d gradient buffers. */
#define TT_MAX_CORES 8
typedef struct tt_desc_d {
    int32_t num_tables;              /* T >= 1                                       */
    int32_t d;                       /* 3 <= d <= TT_MAX_CORES                       */
    int64_t num_embeddings;          /* E, 1 <= E <= prod(p)                         */
    int32_t p[TT_MAX_CORES];         /* p[0 .. d)                                    */
    int32_t q[TT_MAX_CORES];         /* q[0 .. d); D = prod(q)                       */
    int32_t ranks[TT_MAX_CORES - 1]; /* ranks[0 .. d-1), each in [1, 64]             */
    int32_t pooling;                 /* TT_POOL_SUM or TT_POOL_MEAN                  */
} tt_desc_d;

size_t tt_bag_workspace_size_d(const tt_desc_d *desc, int64_t nnz, int64_t num_bags);
/* the chosen cut: groups [0, cut[0]), [cut[0], cut[1]), [cut[1], d) */
int tt_bag_groups_d(const tt_desc_d *desc, int32_t cut[2]);
int tt_bag_forward_d(const tt_desc_d *desc, const float *const *cores, const int64_t *indices,
                     int64_t nnz, const int64_t *offsets, int64_t num_bags,
                     const float *per_sample_weights, float *out, void *ws, size_t ws_bytes,
                     int32_t *dev_status, void *stream);
int tt_bag_backward_sgd_d(const tt_desc_d *desc, float *const *cores, const int64_t *indices,
                          int64_t nnz, const int64_t *offsets, int64_t num_bags,
                          const float *per_sample_weights, const float *grad_out, float lr,
                          void *ws, size_t ws_bytes, int32_t *dev_status, void *stream);
int tt_bag_backward_grad_d(const tt_desc_d *desc, const float *const *cores,
                           const int64_t *indices, int64_t nnz, const int64_t *offsets,
                           int64_t num_bags, const float *per_sample_weights,
                           const float *grad_out, float *const *grad_cores, void *ws,
                           size_t ws_bytes, int32_t *dev_status, void *stream);
/* The grouping of a batch done once (as tt_bag_plan, into the three-core part of the
 * d-core workspace) and reused by the _planned calls below, which otherwise behave as
 * the calls above (same arguments; a plan made for other inputs sets
 * TT_DEV_STALE_PLAN and leaves the outputs unspecified). */
int tt_bag_plan_d(const tt_desc_d *desc, const int64_t *indices, int64_t nnz,
                  const int64_t *offsets, int64_t num_bags, const float *per_sample_weights,
                  void *ws, size_t ws_bytes, int32_t *dev_status, void *stream);
int tt_bag_forward_d_planned(const tt_desc_d *desc, const float *const *cores,
                             const int64_t *indices, int64_t nnz, const int64_t *offsets,
                             int64_t num_bags, const float *per_sample_weights, float *out,
                             void *ws, size_t ws_bytes, int32_t *dev_status, void *stream);
int tt_bag_backward_sgd_d_planned(const tt_desc_d *desc, float *const *cores,
                                  const int64_t *indices, int64_t nnz, const int64_t *offsets,
                                  int64_t num_bags, const float *per_sample_weights,
                                  const float *grad_out, float lr, void *ws, size_t ws_bytes,
                                  int32_t *dev_status, void *stream);
int tt_bag_backward_grad_d_planned(const tt_desc_d *desc, const float *const *cores,
                                   const int64_t *indices, int64_t nnz, const int64_t *offsets,
                                   int64_t num_bags, const float *per_sample_weights,
                                   const float *grad_out, float *const *grad_cores, void *ws,
                                   size_t ws_bytes, int32_t *dev_status, void *stream);

/* ---------------------------------------------------------------- timing
 * Optional per-kernel timing for benchmarks: while enabled, every kernel the
 * library enqueues is bracketed by two HIP events recorded on the stream it is
 * launched on (this adds a little time between kernels).  tt_profile_enable
 * clears the totals; tt_profile_read waits for the recorded events (host
 * blocking) and returns the summed milliseconds and the number of launches of
 * kernel kernel_id in [0, tt_profile_num_kernels()). */
int tt_profile_enable(int on);
int tt_profile_num_kernels(void);
const char *tt_profile_kernel_name(int kernel_id);
int tt_profile_read(int kernel_id, double *total_ms, int64_t *launches);

/* Bound of every wait a kernel of this library makes for other workgroups of its own
 * launch (the grouping's grid-wide barriers, the forward's check that out is cleared):
 * the number of polls after which a waiting workgroup gives up, reports
 * TT_DEV_SYNC_TIMEOUT and leaves (every workgroup still ends normally).  polls < 0
 * restores the default (2^22 polls).  Takes effect for calls made after it, in every
 * thread; meant for tests that drive the give-up path from the host. */
int tt_debug_sync_poll_limit(int64_t polls);

/* Static description of a return code. */
const char *tt_status_string(int code);

#ifdef __cplusplus
}
#endif
#endif /* TT_BAG_H */
