// tt_internal.h -- shared declarations of the libttbag HIP sources (not installed).
//
// Pipeline of one call (all kernels on the caller's stream):
//   route:  k_route_coop    (or k_route_a, _b, _c) split indices, find bags, validate;
//                           stable orders by (table,i3) and (table,i1); final order
//                           (table, i2, i1, position), hits after misses by
//                           (slot, position), skipped elements last; group table and
//                           work items.
//   yinit:  k_yinit         out = zeros, or the pooled cache hits.
//   forward: k_fwd          one workgroup per work item (piece of an i2 group).
//   backward: k_bwd         one workgroup per work item; with a cache, extra
//                           workgroups sum w * dY over the cache-hit runs of one slot.
//             k_seg         core-1 / core-3 segment sums + SGD; cache-row SGD.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tt_bag.h"

namespace ttb {

constexpr int RB = 1024;        // routing block: elements per block
constexpr int RT = 256;         // routing block: threads (4 elements each)
constexpr int HB = 512;         // cache slots per hit bin
constexpr int MAX_BINS = 8192;  // digit range of one counting-sort pass
constexpr int PIECE = 64;       // run-sum: positions per wave
constexpr int ITEM_MAX = 64;    // most positions of one contraction work item
constexpr int WG = 512;         // contraction workgroup: 8 waves
constexpr int NW = WG / 64;
constexpr int MBW = 1;          // forward: M-blocks (16 rows of (pair, j1)) per wave
constexpr int P_MAX = 32;       // positions per work item: P * q1 <= 16 * NW rows
constexpr int MAXQ3 = 16;
constexpr int STAGE_U = 8;      // global loads in flight per thread when staging into LDS
constexpr int COOP_TILES = 256; // blocks of the one-launch grouping kernel (one per CU)
constexpr int FWD_ZERO_BLOCKS = 64;  // forward blocks that clear out when it does
constexpr int COOP_CELLS = 65536;  // its bins x tiles per digit (each block reads them all)
constexpr int COOP_LDS_CELLS = 12288;  // (t,i2) x tile counts gathered in LDS up to this size
// dynamic LDS a contraction workgroup may take: the CU's 160 KiB less room for the
// kernels' few static LDS words (kept out of the plans, so that static + dynamic fit)
constexpr int LDS_DYN_MAX = 160 * 1024 - 256;

// header words inside the workspace (after three 64-bit "last block" counters)
enum {
  H_NFWD = 3,       // number of forward work items
  H_HIT_BEG = 4, H_HIT_END = 5,  // hit region [beg, end) of the final order
  H_VALID = 6,      // number of valid (non-skipped) elements
  H_PLAN = 7,       // fingerprint of the call that made the grouping (tt_bag_plan)
  H_REPOCH = 10,    // groupings run on this workspace (moved on by k_meta)
  H_FEPOCH = 11,    // forward calls that cleared out on this workspace (moved on by the
                    // last block of each)
  H_FCNT = 12,      // blocks of the running forward that are done (zeroed by k_meta and
                    // by the last block of each forward)
  H_SIZE0 = 16,     // [P_MAX + 1] work items handed a place so far, per size
  H_WORDS = 64
};

// Metadata of one contraction work item, written by the grouping (k_meta) and read whole
// into LDS by the contraction kernels: the item's elements (final-order positions s0 ..
// s0 + n_el), its "items" (distinct indices, numbered by their first element) and its
// "pairs" (distinct (i1, i2), runs of the grouping order).  Offsets inside a work item
// fit a byte (P <= 32 positions); i1 and i3 (< 8192) fit a short.
constexpr int META_INTS = 192;  // 768 bytes per work item
struct WorkMeta {
  int n_el, nI, nP, grp, s0;
  int item;                         // the work item's index (its slot is its workgroup)
  int t;                            // the table of its group
  int pad;
  int e_bag[P_MAX];                 // bag of each element
  float e_w[P_MAX];                 // its weight (times 1 / length with mean pooling)
  short pr_i1[P_MAX];               // i1 of each pair (inside its table)
  short it_i3[P_MAX];               // i3 of each item (inside its table)
  unsigned char e_perm[P_MAX];      // item-major slot -> element
  unsigned char e_it[P_MAX];        // element -> item
  unsigned char it_pair[P_MAX];     // item -> pair
  unsigned char it_first[P_MAX];    // item -> its first element
  unsigned char it_beg[P_MAX + 4];  // item -> first item-major slot; [nI] = n_el
  unsigned char pr_it[P_MAX + 4];   // pair -> first item; [nP] = nI
  unsigned char gcnt[P_MAX];        // lane group (4 rows) -> items of the pairs starting in it
  unsigned char mbf[8];             // M-block (16 rows) -> most items of one of its pairs
  unsigned char mbb[8];             // M-block -> most gcnt of its four lane groups
  unsigned char mb_slot[8];         // backward: placement slot -> M-block (see k_meta)
  unsigned char mb_fslot[8];        // forward: the same, by its stage-2 work
};
static_assert(sizeof(WorkMeta) <= META_INTS * 4, "work-item metadata too large");
static_assert(H_SIZE0 + P_MAX + 1 <= H_WORDS, "header words");

struct DevArgs {
  // shape
  int T, p1, p2, p3, q1, q2, q3, R1, R2, D;
  int64_t E;
  int B, NB;
  int nnz, nblk;
  int binsA, binsB, binsI3;
  int has_cache;
  int mean;         // mean pooling: element weights carry 1 / (bag length)
  int64_t cache_size;
  int NHB;
  int P;            // work item: positions per piece (8, 16 or 32; divides PIECE)
  int NRED;         // backward: LDS slots of the cross-wave dG2 reduction (divides NW)
  int JBf, JBb;     // forward / backward: G2 column blocks (j2) staged in LDS at once
  int lq1;          // log2(q1)
  unsigned mq3, mD; // fdiv multipliers of q3 and D
  double rp23, rp3; // 1 / (p2 * p3), 1 / p3 (row split)
  int fwd_sw;       // forward: 1 = rows of a work item kept in LDS and pooled at the end
  unsigned plan_fp;  // fingerprint of (shape, sizes, input pointers) of the plan
  int ncu;           // compute units of the device (0: unknown), for the item placement
  // inputs / outputs
  const int64_t *idx;
  const int64_t *off;
  const int64_t *nnz_dev;  // element count decided on the device (<= nnz), or null
  const float *psw;
  const int32_t *slots;
  float *crows;
  float *G1, *G2, *G3;
  float *Y;
  const float *dY;
  float lr;
  int upd;          // UPD_SGD, UPD_ADAGRAD or UPD_GRAD: what the backward does with a gradient
  float eps;        // Adagrad: added to the root of the running sum
  float *gw;        // gradient with respect to the per-sample weights [nnz] (or null)
  float *X1, *X2, *X3, *Xc;  // per core / cache rows, in their layout: Adagrad running
                             // sums (UPD_ADAGRAD) or the gradient outputs (UPD_GRAD)
  int32_t *status;
  // workspace
  unsigned long long *ctr;  // [3] epoch-tagged completion counters (no zeroing needed)
  unsigned long long *flag;  // [COOP_TILES] grid-barrier arrival words (epoch << 32 | k)
  unsigned long long *fflag; // [FWD_ZERO_BLOCKS] forward: "my slice of out is cleared" words
  int fzero;                 // forward: its first blocks clear out (no separate kernel)
  unsigned epoch;           // tag of the grid-wide flags and counters: unique per call
                            // (< 2^31) when enqueued directly; in a launch being captured
                            // into a graph, a per-process salt to which the kernels add the
                            // workspace's count of groupings / forwards (hdr[H_REPOCH] /
                            // hdr[H_FEPOCH]) and set the top bit, so that every replay
                            // tags its flags afresh
  int devtag;               // 1: the launch is being captured (the device count above)
  unsigned sync_polls;      // bound of every device-side wait (polls before giving up)
  int *hdr;
  int4 *einfo;      // per element: dA (t,i1), dB (t,i2), dI3 (t,i3), bag
  int *histA, *histB, *histI3;
  int *rec;         // [nnz][8] element records in the (t,i1) order (grouping only)
  int *segI3, *segA;  // first position of each (t,i3) / (t,i1) bin in orderI3 / orderA
  int4 *srec;       // final order, 2 int4 per position: (element n, dA, dB, dI3),
                    // (bag, position in orderI3, weight bits, position in orderA)
  int4 *fitem;      // work items: (group, first position, end position, workgroup slot)
  int *meta;        // [items][META_INTS] work-item metadata (WorkMeta)
  int *grp_off;     // [binsB + 1]
  int *chunk_pre;   // [T*p2 + 1]
  int *link1, *link3;  // orderA / orderI3 position -> final position of the partial, or -1
  float *part1, *part3, *frag;
  float *part2;     // dG2 partial per work item [items][R1][q2][R2]
};

// ---------------------------------------------------------------- helpers
// one position of the final order
struct SPos {
  int n, dA, dB, dI3, bag, posI3, posA;
  float w;
};
__device__ __forceinline__ SPos load_spos(const int4 *srec, int s) {
  const int4 u = srec[2 * (size_t)s], v = srec[2 * (size_t)s + 1];
  SPos p;
  p.n = u.x; p.dA = u.y; p.dB = u.z; p.dI3 = u.w;
  p.bag = v.x; p.posI3 = v.y; p.w = __int_as_float(v.z); p.posA = v.w;
  return p;
}
// floor(k / d) for 0 <= k < 2^16 and 1 <= d <= 2^16 with one high multiply by
// m = ceil(2^32 / d) (m = 0 stands for d = 1).  Exact: k * m / 2^32 exceeds k / d by
// less than k / 2^32 < 2^-16 <= 1 / d, which cannot carry it past the next integer.
inline unsigned fdiv_magic(unsigned d) {
  return d == 1 ? 0u : (unsigned)(((1ull << 32) + d - 1) / d);
}
__device__ __forceinline__ int fdiv(int k, unsigned m) {
  return m ? (int)__umulhi((unsigned)k, m) : k;
}
template <int RP>
constexpr int log2_rp() { return RP == 16 ? 4 : (RP == 32 ? 5 : 6); }

__device__ __forceinline__ void set_status(int32_t *st, int bit) {
  if (st) atomicOr(st, bit);
}

// update modes of the backward
enum { UPD_SGD = 0, UPD_ADAGRAD = 1, UPD_GRAD = 2 };

// The update of parameter x[i] (aux[i] in the same layout) with gradient g:
//   SGD      x -= lr g
//   Adagrad  S = aux + g^2 -> aux;  x -= lr g / (sqrt(S) + eps)
//   gradient aux = g (x unchanged)
// x_old / aux_old: the values of x[i] / aux[i] (already loaded by the caller).
template <int UPD>
__device__ __forceinline__ void apply_update(const DevArgs &a, float *x, float *aux, size_t i,
                                             float g, float x_old, float aux_old) {
  if constexpr (UPD == UPD_GRAD) {
    aux[i] = g;
  } else if constexpr (UPD == UPD_ADAGRAD) {
    const float S = aux_old + g * g;
    aux[i] = S;
    x[i] = x_old - a.lr * g / (sqrtf(S) + a.eps);
  } else {
    x[i] = x_old - a.lr * g;
  }
}

// device status bit for a planned call whose workspace holds another plan
constexpr int DEV_STALE_PLAN = 16;


// kernels named by the optional per-kernel timer (tt_prof.hip)
enum KernelId {
  K_ROUTE_COOP, K_ROUTE_A, K_ROUTE_B, K_ROUTE_C, K_FWD, K_BWD, K_SEG,
  K_CACHE_LOOKUP, K_YINIT, K_ZERO, K_DMERGE, K_DSPLIT, K_DAPPLY, K_DD_FRAG, K_DD_GU, K_META,
  K_COUNT
};
// Start / stop events for one launch of kernel `id`, recorded by the kernel's own
// dispatch (so they time the kernel alone), or null events while timing is off.
void prof_events(int id, hipEvent_t *start, hipEvent_t *stop);

template <typename... KArgs, typename... Args>
inline void tt_launch(int id, void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t lds,
                      hipStream_t s, Args... args) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  prof_events(id, &e0, &e1);
  if (e0)
    hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, s, e0, e1, 0u, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
}

// The grouping of a batch whose element count only the device knows: nnz (host) bounds it,
// *nnz_dev (device, read by the grouping kernels) is the count; positions from *nnz_dev on
// are not elements.  Offsets end at *nnz_dev.  No host synchronisation.
int plan_devcount(const tt_desc *desc, const int64_t *indices, int64_t nnz,
                  const int64_t *offsets, int64_t num_bags, const int64_t *nnz_dev, void *ws,
                  size_t ws_bytes, int32_t *dev_status, void *stream);

// header pointer and fingerprint of the three-core plan of these arguments in ws (no
// cache); TT_OK or the descriptor's rejection code
int plan_identity(const tt_desc *desc, int64_t nnz, int64_t num_bags, const void *idx,
                  const void *off, const void *psw, void *ws, int **hdr, unsigned *fp);

// compute units of the current device (cached per device; 0 if the query fails)
int device_cus();

// a copy of the arguments for a launch on stream s: when s is capturing a graph, devtag
// set and the tag's host part replaced by the per-process salt
DevArgs tag_for_launch(const DevArgs &a, hipStream_t s);
// the tag a kernel uses: the call's own, or in a captured launch (salt + the workspace's
// count in *count) | 2^31 -- the count is read only then (a load at kernel start otherwise)
__device__ __forceinline__ unsigned launch_tag(const DevArgs &a, const int *count) {
  return a.devtag ? ((a.epoch + (unsigned)*count) | 0x80000000u) : a.epoch;
}

// stable LSD radix sort of n 64-bit keys by bits [lo, hi); returns a or b (the result)
unsigned long long *radix_sort64_bits(unsigned long long *a, unsigned long long *b, int n,
                                      int *hist, int lo, int hi, hipStream_t s);

// host launchers (each kernel is launched from the file that defines it)
hipError_t launch_route(const DevArgs &a, hipStream_t s);   // the grouping kernels
hipError_t launch_yinit(const DevArgs &a, hipStream_t s);
hipError_t launch_seg(const DevArgs &a, hipStream_t s);
hipError_t launch_zero(float *x, size_t n, hipStream_t s);  // x[0 .. n) = 0
hipError_t launch_fwd(const DevArgs &a, int RP, size_t lds, hipStream_t s);
// dL/dw of the misses (the forward's rows dotted with grad_out, needs fwd_sw) / of the hits
hipError_t launch_wgrad(const DevArgs &a, int RP, size_t lds, hipStream_t s);
hipError_t launch_wgrad_hits(const DevArgs &a, hipStream_t s);
hipError_t launch_bwd(const DevArgs &a, int RP, size_t lds, hipStream_t s);
size_t fwd_lds_bytes(int RP, int JB, int P, int q3, int D, int sw);
size_t bwd_lds_bytes(int RP, int JB, int P, int q3, int D, int nred);

// the batch's element count in the grouping kernels: the host's, or the device word of a
// batch sized on the device (at most the host's)
__device__ __forceinline__ int elem_count(const DevArgs &a) {
  if (!a.nnz_dev) return a.nnz;
  const int64_t n = *a.nnz_dev;
  return n < 0 ? 0 : (n < a.nnz ? (int)n : a.nnz);
}

// Work items of both contraction kernels: every overlap of a miss group with a
// P-aligned piece of the final order.  Upper bound of their number:
__host__ __device__ inline int items_max(const DevArgs &a) {
  return a.T * a.p2 + (a.nnz + a.P - 1) / a.P;
}

}  // namespace ttb
