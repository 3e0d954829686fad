// tt_api.hip -- the C ABI (include/tt_bag.h): argument checks, workspace layout,
// launch sequence.  Device work lives in tt_route.hip, tt_fwd.hip, tt_bwd.hip and
// tt_cache.hip.
#include <unistd.h>

#include <atomic>
#include <chrono>
#include <cmath>
#include <cstring>
#include <mutex>
#include <new>

#include "tt_internal.h"

namespace ttb {
hipError_t cache_lookup_launch(const int64_t *idx, int nnz, int64_t E, long long *hkeys,
                               int *hcnt, long long H, const long long *mkeys, const int *mslot,
                               long long M, int32_t *slot_out, int count_freq, int32_t *status,
                               hipStream_t s);
hipError_t cache_compact_launch(const long long *hkeys, const int *hcnt, long long H, int kbits,
                                unsigned long long *out, int *n_out, hipStream_t s);
hipError_t radix_sort64(unsigned long long *a, unsigned long long *b, int n, int *hist,
                        hipStream_t s);
hipError_t cache_assign_launch(const unsigned long long *sorted, int nf, int kbits,
                               int64_t cache_size, int64_t *cached, long long *mkeys, int *mslot,
                               long long M, hipStream_t s);
hipError_t iota64_launch(int64_t *a, long long n, hipStream_t s);
hipError_t lfu_setkey_launch(const unsigned long long *prio, int n, int kbits, long long nsets,
                             unsigned long long *out, hipStream_t s);
hipError_t lfu_first_launch(const unsigned long long *sk, int n, int *set_first, hipStream_t s);
hipError_t lfu_assign_launch(const unsigned long long *prio, const unsigned long long *sk, int n,
                             int kbits, const int *set_first, long long nsets, int64_t *cached,
                             int *fresh_slot, int64_t *fresh_idx, int *counters, hipStream_t s);
hipError_t map_insert_launch(const int64_t *cached, long long K, long long *mkeys, int *mslot,
                             long long M, hipStream_t s);
hipError_t scatter_rows_launch(const float *tmp, const int *slot, int nf, int D, float *rows,
                               hipStream_t s);
}  // namespace ttb

using namespace ttb;

namespace {

constexpr size_t ALIGN = 256;
constexpr size_t LDS_LIMIT = LDS_DYN_MAX;  // dynamic LDS of one contraction workgroup
std::atomic<unsigned> g_epoch{1};
constexpr unsigned SYNC_POLLS = 1u << 22;  // default bound of a device-side wait
std::atomic<unsigned> g_sync_polls{SYNC_POLLS};

struct Plan {
  DevArgs a;
  int RP = 0;
  size_t lds_fwd = 0, lds_bwd = 0;
  size_t ws_total = 0;
  size_t ws_fwd = 0;  // the prefix the grouping and the forward use (no backward partials)
  // byte offsets inside the workspace
  size_t o_ctr, o_flag, o_fflag, o_hdr, o_einfo, o_histA, o_histB, o_histI3, o_rec, o_segI3, o_segA, o_srec,
      o_fitem, o_meta, o_grp, o_chunk,
      o_l1, o_l3, o_p1, o_p3, o_frag, o_p2;
};

size_t carve(size_t &cur, size_t bytes) {
  const size_t o = cur;
  cur += (bytes + ALIGN - 1) / ALIGN * ALIGN;
  return o;
}

int make_plan(const tt_desc *d, int64_t nnz, int64_t num_bags, int64_t cache_size, Plan *P) {
  if (!d || !P) return TT_EINVAL;
  if (nnz < 0 || nnz >= (int64_t)1 << 30 || num_bags < 1 || cache_size < 0) return TT_EINVAL;
  const int T = d->num_tables;
  if (T < 1) return TT_ESHAPE;
  for (int k = 0; k < 3; ++k)
    if (d->p[k] < 1 || d->q[k] < 1) return TT_ESHAPE;
  if (d->ranks[0] < 1 || d->ranks[1] < 1 || d->ranks[0] > 64 || d->ranks[1] > 64) return TT_ESHAPE;
  if (d->pooling != TT_POOL_SUM && d->pooling != TT_POOL_MEAN) return TT_EINVAL;
  if (!(d->q[0] == 1 || d->q[0] == 2 || d->q[0] == 4)) return TT_ESHAPE;
  if (d->q[2] > MAXQ3) return TT_ESHAPE;
  const int64_t D = (int64_t)d->q[0] * d->q[1] * d->q[2];
  if (D > 1024) return TT_ESHAPE;
  const double prodp = (double)d->p[0] * d->p[1] * d->p[2];
  if (prodp >= 1099511627776.0) return TT_ESHAPE;  // 2^40
  if (d->num_embeddings < 1 || (double)d->num_embeddings > prodp) return TT_ESHAPE;
  const int has_cache = cache_size > 0;
  if (has_cache && T != 1) return TT_ESHAPE;
  const int64_t NB = (int64_t)T * num_bags;
  if (NB >= (int64_t)1 << 30) return TT_EINVAL;
  const int NHB = has_cache ? (int)((cache_size + HB - 1) / HB) : 0;
  const int64_t binsA = (int64_t)T * d->p[0] + (has_cache ? HB : 0) + 1;
  const int64_t binsB = (int64_t)T * d->p[1] + NHB + 1;
  const int64_t binsI3 = (int64_t)T * d->p[2] + 1;
  if (binsA > MAX_BINS || binsB > MAX_BINS || binsI3 > MAX_BINS) return TT_ESHAPE;

  DevArgs &a = P->a;
  memset(&a, 0, sizeof(a));
  a.T = T;
  a.mean = d->pooling == TT_POOL_MEAN;
  a.p1 = d->p[0]; a.p2 = d->p[1]; a.p3 = d->p[2];
  a.q1 = d->q[0]; a.q2 = d->q[1]; a.q3 = d->q[2];
  a.R1 = d->ranks[0]; a.R2 = d->ranks[1];
  a.D = (int)D;
  a.E = d->num_embeddings;
  a.B = (int)num_bags;
  a.NB = (int)NB;
  a.nnz = (int)nnz;
  a.nblk = (int)((nnz + RB - 1) / RB);
  a.binsA = (int)binsA; a.binsB = (int)binsB; a.binsI3 = (int)binsI3;
  a.has_cache = has_cache;
  a.cache_size = cache_size;
  a.NHB = NHB;
  a.lq1 = a.q1 == 4 ? 2 : (a.q1 == 2 ? 1 : 0);
  a.mq3 = fdiv_magic((unsigned)a.q3);
  a.mD = fdiv_magic((unsigned)a.D);
  a.rp23 = 1.0 / ((double)a.p2 * a.p3);
  a.rp3 = 1.0 / (double)a.p3;
  const int Rmax = a.R1 > a.R2 ? a.R1 : a.R2;
  P->RP = Rmax <= 16 ? 16 : (Rmax <= 32 ? 32 : 64);
  // work items of P positions (P * q1 rows fill at most one M-block per wave); P shrinks
  // only when a work item's rows of width D would not fit the backward's LDS
  a.P = P_MAX;
  while (a.P > 8 && bwd_lds_bytes(P->RP, 1, a.P, a.q3, a.D, 1) > LDS_LIMIT) a.P >>= 1;
  if (bwd_lds_bytes(P->RP, 1, a.P, a.q3, a.D, 1) > LDS_LIMIT) return TT_ESHAPE;
  // LDS plans that let two workgroups share a CU where possible: G2 staged whole (fewer
  // column blocks only when needed), backward reduction slots 8 -> 2 first.  The rank-64
  // backward holds a whole CU by its register count, so its plan may take all of the LDS.
  const size_t half = LDS_LIMIT / 2 - 1024;
  const size_t bwd_budget = P->RP == 64 ? LDS_LIMIT : half;
  int nred = NW, JBb = a.q2;
  while (bwd_lds_bytes(P->RP, JBb, a.P, a.q3, a.D, nred) > bwd_budget && nred > 2) nred >>= 1;
  while (bwd_lds_bytes(P->RP, JBb, a.P, a.q3, a.D, nred) > bwd_budget && JBb > 1) --JBb;
  while (bwd_lds_bytes(P->RP, JBb, a.P, a.q3, a.D, nred) > bwd_budget && nred > 1) nred >>= 1;
  a.NRED = nred;
  a.JBb = JBb;
  P->lds_bwd = bwd_lds_bytes(P->RP, JBb, a.P, a.q3, a.D, nred);
  a.fwd_sw = (size_t)a.P * a.D * 4 <= 64 * 1024;
  a.JBf = a.q2;
  while (a.JBf > 1 && fwd_lds_bytes(P->RP, a.JBf, a.P, a.q3, a.D, a.fwd_sw) > half) --a.JBf;
  P->lds_fwd = fwd_lds_bytes(P->RP, a.JBf, a.P, a.q3, a.D, a.fwd_sw);
  if (P->lds_bwd > LDS_LIMIT || P->lds_fwd > LDS_LIMIT) return TT_ESHAPE;

  const size_t n = (size_t)nnz, nb = (size_t)a.nblk, G = (size_t)T * a.p2;
  size_t cur = 0;
  P->o_ctr = carve(cur, 3 * sizeof(unsigned long long));
  P->o_flag = carve(cur, COOP_TILES * sizeof(unsigned long long));
  P->o_fflag = carve(cur, FWD_ZERO_BLOCKS * sizeof(unsigned long long));
  P->o_hdr = carve(cur, H_WORDS * sizeof(int));
  P->o_einfo = carve(cur, n * sizeof(int4));
  P->o_histA = carve(cur, (size_t)binsA * nb * 4);
  P->o_histB = carve(cur, (size_t)binsB * nb * 4);
  P->o_histI3 = carve(cur, (size_t)binsI3 * nb * 4);
  P->o_rec = carve(cur, n * 32);
  P->o_segI3 = carve(cur, ((size_t)binsI3 + 1) * 4);
  P->o_segA = carve(cur, ((size_t)binsA + 1) * 4);
  P->o_srec = carve(cur, n * 32);
  P->o_fitem = carve(cur, (size_t)items_max(a) * sizeof(int4));
  P->o_meta = carve(cur, (size_t)items_max(a) * META_INTS * 4);
  P->o_grp = carve(cur, ((size_t)binsB + 1) * 4);
  P->o_chunk = carve(cur, (G + 1) * 4);
  P->o_l1 = carve(cur, n * 4);
  P->o_l3 = carve(cur, n * 4);
  P->ws_fwd = cur;  // from here on: parts only the backward writes
  P->o_p1 = carve(cur, n * (size_t)a.q1 * a.R1 * 4);
  P->o_p3 = carve(cur, n * (size_t)a.R2 * a.q3 * 4);
  P->o_frag = carve(cur, n * (size_t)a.D * 4);
  P->o_p2 = carve(cur, (size_t)items_max(a) * a.R1 * a.q2 * a.R2 * 4);
  P->ws_total = cur;
  return TT_OK;
}

void bind_ws(Plan *P, void *ws) {
  char *b = (char *)ws;
  DevArgs &a = P->a;
  a.ctr = (unsigned long long *)(b + P->o_ctr);
  a.flag = (unsigned long long *)(b + P->o_flag);
  a.fflag = (unsigned long long *)(b + P->o_fflag);
  a.hdr = (int *)(b + P->o_hdr);
  a.einfo = (int4 *)(b + P->o_einfo);
  a.histA = (int *)(b + P->o_histA);
  a.histB = (int *)(b + P->o_histB);
  a.histI3 = (int *)(b + P->o_histI3);
  a.rec = (int *)(b + P->o_rec);
  a.segI3 = (int *)(b + P->o_segI3);
  a.segA = (int *)(b + P->o_segA);
  a.srec = (int4 *)(b + P->o_srec);
  a.fitem = (int4 *)(b + P->o_fitem);
  a.meta = (int *)(b + P->o_meta);
  a.grp_off = (int *)(b + P->o_grp);
  a.chunk_pre = (int *)(b + P->o_chunk);
  a.link1 = (int *)(b + P->o_l1);
  a.link3 = (int *)(b + P->o_l3);
  a.part1 = (float *)(b + P->o_p1);
  a.part3 = (float *)(b + P->o_p3);
  a.frag = (float *)(b + P->o_frag);
  a.part2 = (float *)(b + P->o_p2);
  a.epoch = g_epoch.fetch_add(1) & 0x7fffffffu;  // (captured launches set the top bit)
  if (a.epoch == 0) a.epoch = g_epoch.fetch_add(1) & 0x7fffffffu;
  a.devtag = 0;
  a.sync_polls = g_sync_polls.load(std::memory_order_relaxed);
}

// fwd_only: the call runs the grouping and the forward only, which use ws_fwd bytes
int check_ws(const Plan &P, void *ws, size_t ws_bytes, bool fwd_only = false) {
  if (!ws) return TT_EINVAL;
  if (((uintptr_t)ws) % ALIGN) return TT_EWORKSPACE;
  if (ws_bytes < (fwd_only ? P.ws_fwd : P.ws_total)) return TT_EWORKSPACE;
  return TT_OK;
}

int set_cache(Plan *P, const tt_cache_view *cache, int64_t nnz) {
  DevArgs &a = P->a;
  if (!cache) return TT_OK;
  if (cache->cache_size != a.cache_size) return TT_EINVAL;
  if (cache->cache_size > 0 && (!cache->rows || (nnz > 0 && !cache->slots))) return TT_EINVAL;
  a.slots = cache->slots;
  a.crows = cache->rows;
  return TT_OK;
}

}  // namespace

extern "C" {

const char *tt_status_string(int code) {
  switch (code) {
    case TT_OK: return "ok";
    case TT_EINVAL: return "invalid argument (null pointer, negative size or non-finite value)";
    case TT_ESHAPE: return "descriptor inconsistent or outside the supported shapes";
    case TT_EWORKSPACE: return "workspace too small or not 256-byte aligned";
    case TT_EHIP: return "HIP runtime error";
    case TT_EFULL: return "cache capacity exceeded";
    default: return "unknown status";
  }
}

int tt_debug_sync_poll_limit(int64_t polls) {
  if (polls > (int64_t)0xffffffffu) return TT_EINVAL;
  g_sync_polls.store(polls < 0 ? SYNC_POLLS : (unsigned)polls, std::memory_order_relaxed);
  return TT_OK;
}

size_t tt_bag_workspace_size(const tt_desc *desc, int64_t nnz, int64_t num_bags,
                             int64_t cache_size) {
  Plan P;
  if (make_plan(desc, nnz, num_bags, cache_size, &P) != TT_OK) return 0;
  return P.ws_total;
}

static int finish(hipError_t e) { return e == hipSuccess ? TT_OK : TT_EHIP; }

// FNV-1a over the call's shape, sizes and input pointers: names the plan in a workspace.
static unsigned plan_fingerprint(const tt_desc *d, int64_t nnz, int64_t num_bags,
                                 int64_t cache_size, const void *idx, const void *off,
                                 const void *psw, const void *slots) {
  unsigned h = 2166136261u;
  auto mix = [&h](uint64_t v) {
    for (int i = 0; i < 8; ++i) {
      h ^= (unsigned)(v & 0xff);
      h *= 16777619u;
      v >>= 8;
    }
  };
  mix((uint64_t)d->num_tables);
  mix((uint64_t)d->num_embeddings);
  for (int k = 0; k < 3; ++k) { mix((uint64_t)d->p[k]); mix((uint64_t)d->q[k]); }
  mix((uint64_t)d->ranks[0]);
  mix((uint64_t)d->ranks[1]);
  mix((uint64_t)d->pooling);
  mix((uint64_t)nnz);
  mix((uint64_t)num_bags);
  mix((uint64_t)cache_size);
  mix((uint64_t)(uintptr_t)idx);
  mix((uint64_t)(uintptr_t)off);
  mix((uint64_t)(uintptr_t)psw);
  mix((uint64_t)(uintptr_t)slots);
  return h;
}

// argument checks shared by every call that takes a batch; fills P and binds ws
static int prepare(Plan *P, const tt_desc *desc, const int64_t *indices, int64_t nnz,
                   const int64_t *offsets, int64_t num_bags, const float *psw,
                   const tt_cache_view *cache, void *ws, size_t ws_bytes, int32_t *dev_status,
                   bool fwd_only = false) {
  const int64_t csize = cache ? cache->cache_size : 0;
  int rc = make_plan(desc, nnz, num_bags, csize, P);
  if (rc) return rc;
  if (!offsets || (nnz > 0 && !indices)) return TT_EINVAL;
  if ((rc = check_ws(*P, ws, ws_bytes, fwd_only))) return rc;
  if ((rc = set_cache(P, cache, nnz))) return rc;
  bind_ws(P, ws);
  DevArgs &a = P->a;
  a.idx = indices;
  a.off = offsets;
  a.psw = psw;
  a.status = dev_status;
  a.plan_fp = plan_fingerprint(desc, nnz, num_bags, csize, indices, offsets, psw,
                               cache ? (const void *)cache->slots : nullptr);
  return TT_OK;
}

static int check_cores(const float *const cores[3]) {
  return (!cores || !cores[0] || !cores[1] || !cores[2]) ? TT_EINVAL : TT_OK;
}

}  // extern "C"

namespace ttb {
DevArgs tag_for_launch(const DevArgs &a, hipStream_t s) {
  // one salt for the whole process: every graph captured here, whichever workspace it
  // uses, adds the same host part to the workspace's own count
  static const unsigned salt = [] {
    const unsigned long long t = (unsigned long long)std::chrono::steady_clock::now()
                                     .time_since_epoch().count();
    return (unsigned)(t ^ (t >> 32) ^ ((unsigned long long)getpid() << 16)) | 1u;
  }();
  DevArgs b = a;
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &st) == hipSuccess && st == hipStreamCaptureStatusActive) {
    b.devtag = 1;
    b.epoch = salt;
  }
  return b;
}

// Where a three-core plan keeps its header inside ws, and the fingerprint a plan made
// for these arguments carries (no cache).  Used by the backward over distinct indices,
// whose kernels read the real batch's plan and must see whether it is this batch's.
int plan_identity(const tt_desc *desc, int64_t nnz, int64_t num_bags, const void *idx,
                  const void *off, const void *psw, void *ws, int **hdr, unsigned *fp) {
  Plan P;
  const int rc = make_plan(desc, nnz, num_bags, 0, &P);
  if (rc) return rc;
  *hdr = (int *)((char *)ws + P.o_hdr);
  *fp = plan_fingerprint(desc, nnz, num_bags, 0, idx, off, psw, nullptr);
  return TT_OK;
}
}  // namespace ttb

// the grouping / the planned forward; fwd_only: ws holds only the forward's part
static int plan_call(const tt_desc *desc, const int64_t *indices, int64_t nnz,
                     const int64_t *offsets, int64_t num_bags, const float *per_sample_weights,
                     const tt_cache_view *cache, void *ws, size_t ws_bytes, int32_t *dev_status,
                     void *stream, bool fwd_only) {
  Plan P;
  int rc = prepare(&P, desc, indices, nnz, offsets, num_bags, per_sample_weights, cache, ws,
                   ws_bytes, dev_status, fwd_only);
  if (rc) return rc;
  return finish(launch_route(P.a, (hipStream_t)stream));
}

namespace ttb {
int plan_devcount(const tt_desc *desc, const int64_t *indices, int64_t nnz,
                  const int64_t *offsets, int64_t num_bags, const int64_t *nnz_dev, void *ws,
                  size_t ws_bytes, int32_t *dev_status, void *stream) {
  if (!nnz_dev) return TT_EINVAL;
  Plan P;
  int rc = prepare(&P, desc, indices, nnz, offsets, num_bags, nullptr, nullptr, ws, ws_bytes,
                   dev_status);
  if (rc) return rc;
  P.a.nnz_dev = nnz_dev;
  return finish(launch_route(P.a, (hipStream_t)stream));
}
}  // namespace ttb

static int forward_planned_call(const tt_desc *desc, const float *const cores[3],
                                const int64_t *indices, int64_t nnz, const int64_t *offsets,
                                int64_t num_bags, const float *per_sample_weights,
                                const tt_cache_view *cache, float *out, void *ws,
                                size_t ws_bytes, int32_t *dev_status, void *stream,
                                bool fwd_only) {
  Plan P;
  int rc = prepare(&P, desc, indices, nnz, offsets, num_bags, per_sample_weights, cache, ws,
                   ws_bytes, dev_status, fwd_only);
  if (rc) return rc;
  if ((rc = check_cores(cores)) || !out) return rc ? rc : TT_EINVAL;
  DevArgs &a = P.a;
  a.psw = per_sample_weights;
  a.G1 = (float *)cores[0]; a.G2 = (float *)cores[1]; a.G3 = (float *)cores[2];
  a.Y = out;
  hipStream_t s = (hipStream_t)stream;
  // without a cache the forward kernel clears out itself; with one, k_yinit pools the hits
  a.fzero = !a.has_cache && a.nnz > 0;
  hipError_t e = a.fzero ? hipSuccess : launch_yinit(a, s);
  if (e == hipSuccess && a.nnz > 0) e = launch_fwd(a, P.RP, P.lds_fwd, s);
  return finish(e);
}

// the stateless forward: argument checks, then grouping + planned forward in ws
static int forward_call(const tt_desc *desc, const float *const cores[3], const int64_t *indices,
                        int64_t nnz, const int64_t *offsets, int64_t num_bags,
                        const float *per_sample_weights, const tt_cache_view *cache, float *out,
                        void *ws, size_t ws_bytes, int32_t *dev_status, void *stream,
                        bool fwd_only) {
  Plan P;
  int rc = prepare(&P, desc, indices, nnz, offsets, num_bags, per_sample_weights, cache, ws,
                   ws_bytes, dev_status, fwd_only);
  if (rc) return rc;
  if ((rc = check_cores(cores)) || !out) return rc ? rc : TT_EINVAL;
  rc = plan_call(desc, indices, nnz, offsets, num_bags, per_sample_weights, cache, ws, ws_bytes,
                 dev_status, stream, fwd_only);
  if (rc) return rc;
  return forward_planned_call(desc, cores, indices, nnz, offsets, num_bags, per_sample_weights,
                              cache, out, ws, ws_bytes, dev_status, stream, fwd_only);
}

extern "C" {

int tt_bag_plan(const tt_desc *desc, const int64_t *indices, int64_t nnz, const int64_t *offsets,
                int64_t num_bags, const float *per_sample_weights, const tt_cache_view *cache,
                void *ws, size_t ws_bytes, int32_t *dev_status, void *stream) {
  return plan_call(desc, indices, nnz, offsets, num_bags, per_sample_weights, cache, ws, ws_bytes,
                   dev_status, stream, false);
}

int tt_bag_forward_planned(const tt_desc *desc, const float *const cores[3],
                           const int64_t *indices, int64_t nnz, const int64_t *offsets,
                           int64_t num_bags, const float *per_sample_weights,
                           const tt_cache_view *cache, float *out, void *ws, size_t ws_bytes,
                           int32_t *dev_status, void *stream) {
  return forward_planned_call(desc, cores, indices, nnz, offsets, num_bags, per_sample_weights,
                              cache, out, ws, ws_bytes, dev_status, stream, false);
}

}  // extern "C"

namespace {

// what the backward does with the gradients (see apply_update)
struct Update {
  int mode;
  float lr, eps;
  float *const *aux;  // [3] per core: Adagrad running sums or gradient outputs
  float *aux_rows;    // the same for the cache rows
};

// Every backward entry point: argument checks, then (plan_first) the grouping, then
// the run sums of cache hits, the contraction and the segment sums with the update.
int backward_call(const tt_desc *desc, float *const cores[3], const int64_t *indices, int64_t nnz,
                  const int64_t *offsets, int64_t num_bags, const float *psw,
                  const tt_cache_view *cache, const float *grad_out, const Update &u, void *ws,
                  size_t ws_bytes, int32_t *dev_status, void *stream, bool plan_first) {
  Plan P;
  int rc = prepare(&P, desc, indices, nnz, offsets, num_bags, psw, cache, ws, ws_bytes,
                   dev_status);
  if (rc) return rc;
  if ((rc = check_cores(cores)) || !grad_out) return rc ? rc : TT_EINVAL;
  DevArgs &a = P.a;
  if (u.mode != UPD_GRAD && !std::isfinite(u.lr)) return TT_EINVAL;
  if (u.mode == UPD_ADAGRAD && !(std::isfinite(u.eps) && u.eps >= 0.f)) return TT_EINVAL;
  if (u.mode != UPD_SGD) {
    if (!u.aux || !u.aux[0] || !u.aux[1] || !u.aux[2]) return TT_EINVAL;
    if (a.cache_size > 0 && !u.aux_rows) return TT_EINVAL;
    a.X1 = u.aux[0]; a.X2 = u.aux[1]; a.X3 = u.aux[2];
    a.Xc = u.aux_rows;
  }
  a.upd = u.mode;
  a.lr = u.lr;
  a.eps = u.eps;
  a.psw = psw;
  a.G1 = cores[0]; a.G2 = cores[1]; a.G3 = cores[2];
  a.dY = grad_out;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  if (u.mode == UPD_GRAD) {
    // gradient outputs are overwritten whole: rows without hits are cleared here, core
    // slices without contributions by the segment sums (or here for an empty batch)
    if (a.cache_size > 0) e = launch_zero(a.Xc, (size_t)a.cache_size * a.D, s);
    if (nnz == 0) {
      const size_t T = (size_t)a.T;
      if (e == hipSuccess) e = launch_zero(a.X1, T * a.p1 * a.q1 * a.R1, s);
      if (e == hipSuccess) e = launch_zero(a.X2, T * a.p2 * a.R1 * a.q2 * a.R2, s);
      if (e == hipSuccess) e = launch_zero(a.X3, T * a.p3 * a.R2 * a.q3, s);
      return finish(e);
    }
  } else if (nnz == 0) {
    return TT_OK;
  }
  if (e == hipSuccess && plan_first) e = launch_route(a, s);
  if (e == hipSuccess) e = launch_bwd(a, P.RP, P.lds_bwd, s);
  if (e == hipSuccess) e = launch_seg(a, s);
  return finish(e);
}

}  // namespace

extern "C" {

int tt_bag_backward_sgd_planned(const tt_desc *desc, float *const cores[3],
                                const int64_t *indices, int64_t nnz, const int64_t *offsets,
                                int64_t num_bags, const float *per_sample_weights,
                                const tt_cache_view *cache, const float *grad_out, float lr,
                                void *ws, size_t ws_bytes, int32_t *dev_status, void *stream) {
  const Update u{UPD_SGD, lr, 0.f, nullptr, nullptr};
  return backward_call(desc, cores, indices, nnz, offsets, num_bags, per_sample_weights, cache,
                       grad_out, u, ws, ws_bytes, dev_status, stream, false);
}

int tt_bag_backward_adagrad_planned(const tt_desc *desc, float *const cores[3],
                                    const int64_t *indices, int64_t nnz, const int64_t *offsets,
                                    int64_t num_bags, const float *per_sample_weights,
                                    const tt_cache_view *cache, const float *grad_out, float lr,
                                    float eps, float *const state[3], float *state_rows, void *ws,
                                    size_t ws_bytes, int32_t *dev_status, void *stream) {
  const Update u{UPD_ADAGRAD, lr, eps, state, state_rows};
  return backward_call(desc, cores, indices, nnz, offsets, num_bags, per_sample_weights, cache,
                       grad_out, u, ws, ws_bytes, dev_status, stream, false);
}

int tt_bag_backward_grad_planned(const tt_desc *desc, const float *const cores[3],
                                 const int64_t *indices, int64_t nnz, const int64_t *offsets,
                                 int64_t num_bags, const float *per_sample_weights,
                                 const tt_cache_view *cache, const float *grad_out,
                                 float *const grad_cores[3], float *grad_rows, void *ws,
                                 size_t ws_bytes, int32_t *dev_status, void *stream) {
  const Update u{UPD_GRAD, 0.f, 0.f, grad_cores, grad_rows};
  return backward_call(desc, (float *const *)cores, indices, nnz, offsets, num_bags,
                       per_sample_weights, cache, grad_out, u, ws, ws_bytes, dev_status, stream,
                       false);
}

int tt_bag_forward(const tt_desc *desc, const float *const cores[3], const int64_t *indices,
                   int64_t nnz, const int64_t *offsets, int64_t num_bags,
                   const float *per_sample_weights, const tt_cache_view *cache, float *out,
                   void *ws, size_t ws_bytes, int32_t *dev_status, void *stream) {
  return forward_call(desc, cores, indices, nnz, offsets, num_bags, per_sample_weights, cache,
                      out, ws, ws_bytes, dev_status, stream, false);
}

int tt_bag_backward_sgd(const tt_desc *desc, float *const cores[3], const int64_t *indices,
                        int64_t nnz, const int64_t *offsets, int64_t num_bags,
                        const float *per_sample_weights, const tt_cache_view *cache,
                        const float *grad_out, float lr, void *ws, size_t ws_bytes,
                        int32_t *dev_status, void *stream) {
  const Update u{UPD_SGD, lr, 0.f, nullptr, nullptr};
  return backward_call(desc, cores, indices, nnz, offsets, num_bags, per_sample_weights, cache,
                       grad_out, u, ws, ws_bytes, dev_status, stream, true);
}

int tt_bag_backward_adagrad(const tt_desc *desc, float *const cores[3], const int64_t *indices,
                            int64_t nnz, const int64_t *offsets, int64_t num_bags,
                            const float *per_sample_weights, const tt_cache_view *cache,
                            const float *grad_out, float lr, float eps, float *const state[3],
                            float *state_rows, void *ws, size_t ws_bytes, int32_t *dev_status,
                            void *stream) {
  const Update u{UPD_ADAGRAD, lr, eps, state, state_rows};
  return backward_call(desc, cores, indices, nnz, offsets, num_bags, per_sample_weights, cache,
                       grad_out, u, ws, ws_bytes, dev_status, stream, true);
}

int tt_bag_backward_grad(const tt_desc *desc, const float *const cores[3],
                         const int64_t *indices, int64_t nnz, const int64_t *offsets,
                         int64_t num_bags, const float *per_sample_weights,
                         const tt_cache_view *cache, const float *grad_out,
                         float *const grad_cores[3], float *grad_rows, void *ws, size_t ws_bytes,
                         int32_t *dev_status, void *stream) {
  const Update u{UPD_GRAD, 0.f, 0.f, grad_cores, grad_rows};
  return backward_call(desc, (float *const *)cores, indices, nnz, offsets, num_bags,
                       per_sample_weights, cache, grad_out, u, ws, ws_bytes, dev_status, stream,
                       true);
}

static int weight_grad_call(const tt_desc *desc, const float *const cores[3],
                            const int64_t *indices, int64_t nnz, const int64_t *offsets,
                            int64_t num_bags, const float *psw, const tt_cache_view *cache,
                            const float *grad_out, float *grad_w, void *ws, size_t ws_bytes,
                            int32_t *dev_status, void *stream, bool plan_first) {
  Plan P;
  int rc = prepare(&P, desc, indices, nnz, offsets, num_bags, psw, cache, ws, ws_bytes,
                   dev_status);
  if (rc) return rc;
  if ((rc = check_cores(cores)) || !grad_out || (nnz > 0 && !grad_w)) return rc ? rc : TT_EINVAL;
  DevArgs &a = P.a;
  if (!a.fwd_sw) return TT_ESHAPE;  // the rows of a work item must fit the forward's LDS
  if (nnz == 0) return TT_OK;
  a.psw = psw;
  a.G1 = (float *)cores[0]; a.G2 = (float *)cores[1]; a.G3 = (float *)cores[2];
  a.dY = grad_out;
  a.gw = grad_w;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = launch_zero(grad_w, (size_t)nnz, s);  // skipped elements keep 0
  if (e == hipSuccess && plan_first) e = launch_route(a, s);
  if (e == hipSuccess) e = launch_wgrad(a, P.RP, P.lds_fwd, s);
  if (e == hipSuccess) e = launch_wgrad_hits(a, s);
  return finish(e);
}

int tt_bag_weight_grad(const tt_desc *desc, const float *const cores[3], const int64_t *indices,
                       int64_t nnz, const int64_t *offsets, int64_t num_bags,
                       const float *per_sample_weights, const tt_cache_view *cache,
                       const float *grad_out, float *grad_weights, void *ws, size_t ws_bytes,
                       int32_t *dev_status, void *stream) {
  return weight_grad_call(desc, cores, indices, nnz, offsets, num_bags, per_sample_weights, cache,
                          grad_out, grad_weights, ws, ws_bytes, dev_status, stream, true);
}

int tt_bag_weight_grad_planned(const tt_desc *desc, const float *const cores[3],
                               const int64_t *indices, int64_t nnz, const int64_t *offsets,
                               int64_t num_bags, const float *per_sample_weights,
                               const tt_cache_view *cache, const float *grad_out,
                               float *grad_weights, void *ws, size_t ws_bytes,
                               int32_t *dev_status, void *stream) {
  return weight_grad_call(desc, cores, indices, nnz, offsets, num_bags, per_sample_weights, cache,
                          grad_out, grad_weights, ws, ws_bytes, dev_status, stream, false);
}

// copies the grouping order: valid elements first (see tt_bag.h)
__global__ void k_copy_route(const int4 *srec, int nnz, const int *grp_off, int G, int binsB,
                             int *order_out, int *group_off_out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < nnz) order_out[i] = srec[2 * (size_t)i].x;
  if (i <= G) group_off_out[i] = grp_off[i];
  if (i == G + 1) group_off_out[G + 1] = grp_off[binsB - 1];
}

int tt_bag_route(const tt_desc *desc, const int64_t *indices, int64_t nnz,
                 const int64_t *offsets, int64_t num_bags, const int32_t *slots,
                 int64_t cache_size, int32_t *order_out, int32_t *group_off_out, void *ws,
                 size_t ws_bytes, int32_t *dev_status, void *stream) {
  if (!order_out || !group_off_out) return TT_EINVAL;
  tt_cache_view view{slots, nullptr, cache_size};
  Plan P;
  const tt_cache_view *cv = slots ? &view : nullptr;
  if (slots && cache_size < 1) return TT_EINVAL;
  // the rows pointer is not needed for grouping
  const int64_t csize = cv ? cache_size : 0;
  int rc = make_plan(desc, nnz, num_bags, csize, &P);
  if (rc) return rc;
  if (!offsets || (nnz > 0 && !indices)) return TT_EINVAL;
  if ((rc = check_ws(P, ws, ws_bytes))) return rc;
  bind_ws(&P, ws);
  DevArgs &a = P.a;
  a.idx = indices; a.off = offsets; a.slots = slots; a.status = dev_status;
  a.plan_fp = plan_fingerprint(desc, nnz, num_bags, csize, indices, offsets, nullptr, slots);
  hipStream_t s = (hipStream_t)stream;
  const int G = a.T * a.p2;
  hipError_t e = hipSuccess;
  if (nnz == 0) return finish(hipMemsetAsync(group_off_out, 0, (G + 2) * sizeof(int32_t), s));
  e = launch_route(a, s);
  if (e == hipSuccess) {
    const int n = (int)nnz > G + 2 ? (int)nnz : G + 2;
    hipLaunchKernelGGL(k_copy_route, dim3((n + 255) / 256), dim3(256), 0, s, a.srec, a.nnz,
                       a.grp_off, G, a.binsB, order_out, group_off_out);
    e = hipGetLastError();
  }
  return finish(e);
}

// ---------------------------------------------------------------- cache
struct tt_cache {
  tt_desc desc;
  int policy = TT_CACHE_TOPK;
  int64_t cache_size = 0, H = 0, M = 0;
  int kbits = 1;
  long long *hkeys = nullptr;
  int *hcnt = nullptr;
  long long *mkeys = nullptr;
  int *mslot = nullptr;
  int64_t *cached = nullptr;
  unsigned long long *sk0 = nullptr, *sk1 = nullptr;
  int *shist = nullptr;
  int *nent = nullptr;
  int64_t *bag_off = nullptr;
  void *fws = nullptr;
  size_t fws_bytes = 0;
  int device = 0;
  // set-associative LFU only: set-major sort keys, set starts, newcomers, their rows
  unsigned long long *lk0 = nullptr, *lk1 = nullptr;
  int *set_first = nullptr, *fresh_slot = nullptr, *lcnt = nullptr;
  int64_t *fresh_idx = nullptr;
  float *rows_tmp = nullptr;
};

static void cache_free(tt_cache *c) {
  if (!c) return;
  void *ptrs[] = {c->hkeys, c->hcnt, c->mkeys, c->mslot, c->cached, c->sk0, c->sk1,
                  c->shist, c->nent, c->bag_off, c->fws, c->lk0, c->lk1, c->set_first,
                  c->fresh_slot, c->lcnt, c->fresh_idx, c->rows_tmp};
  for (void *p : ptrs)
    if (p) (void)hipFree(p);
  delete c;
}

int tt_cache_create(tt_cache **out, const tt_desc *desc, int64_t cache_size,
                    int64_t hashtbl_size) {
  return tt_cache_create_policy(out, desc, cache_size, hashtbl_size, TT_CACHE_TOPK);
}

int tt_cache_create_policy(tt_cache **out, const tt_desc *desc, int64_t cache_size,
                           int64_t hashtbl_size, int policy) {
  if (!out || !desc || cache_size < 1 || hashtbl_size < 1) return TT_EINVAL;
  if (policy != TT_CACHE_TOPK && policy != TT_CACHE_LFU32) return TT_EINVAL;
  if (policy == TT_CACHE_LFU32 && cache_size % 32 != 0) return TT_EINVAL;
  if (desc->num_tables != 1) return TT_ESHAPE;
  if (cache_size >= (int64_t)1 << 29 || hashtbl_size >= (int64_t)1 << 31) return TT_EFULL;
  Plan P;
  int rc = make_plan(desc, cache_size, cache_size, 0, &P);
  if (rc) return rc;
  tt_cache *c = new (std::nothrow) tt_cache();
  if (!c) return TT_EINVAL;
  c->desc = *desc;
  c->policy = policy;
  c->cache_size = cache_size;
  c->H = hashtbl_size;
  int64_t M = 1;
  while (M < 2 * cache_size) M <<= 1;
  c->M = M;
  int kb = 1;
  while (kb < 63 && ((int64_t)1 << kb) < desc->num_embeddings) ++kb;
  c->kbits = kb;
  c->fws_bytes = P.ws_total;
  const size_t nsort = (size_t)hashtbl_size;
  const size_t nblk = (nsort + RB - 1) / RB;
  bool ok = hipGetDevice(&c->device) == hipSuccess;
  ok = ok && hipMalloc(&c->hkeys, (size_t)c->H * 8) == hipSuccess;
  ok = ok && hipMalloc(&c->hcnt, (size_t)c->H * 4) == hipSuccess;
  ok = ok && hipMalloc(&c->mkeys, (size_t)M * 8) == hipSuccess;
  ok = ok && hipMalloc(&c->mslot, (size_t)M * 4) == hipSuccess;
  ok = ok && hipMalloc(&c->cached, (size_t)cache_size * 8) == hipSuccess;
  ok = ok && hipMalloc(&c->sk0, nsort * 8) == hipSuccess;
  ok = ok && hipMalloc(&c->sk1, nsort * 8) == hipSuccess;
  ok = ok && hipMalloc(&c->shist, 256 * nblk * 4 + 4) == hipSuccess;
  ok = ok && hipMalloc(&c->nent, 4) == hipSuccess;
  ok = ok && hipMalloc(&c->bag_off, (size_t)(cache_size + 1) * 8) == hipSuccess;
  ok = ok && hipMalloc(&c->fws, c->fws_bytes) == hipSuccess;
  if (policy == TT_CACHE_LFU32) {
    const size_t D = (size_t)desc->q[0] * desc->q[1] * desc->q[2];
    ok = ok && hipMalloc(&c->lk0, nsort * 8) == hipSuccess;
    ok = ok && hipMalloc(&c->lk1, nsort * 8) == hipSuccess;
    ok = ok && hipMalloc(&c->set_first, (size_t)(cache_size / 32) * 4) == hipSuccess;
    ok = ok && hipMalloc(&c->fresh_slot, (size_t)cache_size * 4) == hipSuccess;
    ok = ok && hipMalloc(&c->fresh_idx, (size_t)cache_size * 8) == hipSuccess;
    ok = ok && hipMalloc(&c->lcnt, 8) == hipSuccess;
    ok = ok && hipMalloc(&c->rows_tmp, (size_t)cache_size * D * 4) == hipSuccess;
  }
  ok = ok && hipMemset(c->hkeys, 0xff, (size_t)c->H * 8) == hipSuccess;
  ok = ok && hipMemset(c->hcnt, 0, (size_t)c->H * 4) == hipSuccess;
  ok = ok && hipMemset(c->mkeys, 0xff, (size_t)M * 8) == hipSuccess;
  ok = ok && hipMemset(c->cached, 0xff, (size_t)cache_size * 8) == hipSuccess;
  ok = ok && iota64_launch(c->bag_off, cache_size + 1, nullptr) == hipSuccess;
  ok = ok && hipDeviceSynchronize() == hipSuccess;
  if (!ok) {
    cache_free(c);
    return TT_EHIP;
  }
  *out = c;
  return TT_OK;
}

int tt_cache_lookup(tt_cache *c, const int64_t *indices, int64_t nnz, int32_t *slot_out,
                    int count_freq, int32_t *dev_status, void *stream) {
  if (!c || nnz < 0 || nnz >= (int64_t)1 << 30) return TT_EINVAL;
  if (nnz > 0 && (!indices || !slot_out)) return TT_EINVAL;
  return finish(cache_lookup_launch(indices, (int)nnz, c->desc.num_embeddings, c->hkeys, c->hcnt,
                                    c->H, c->mkeys, c->mslot, c->M, slot_out, count_freq ? 1 : 0,
                                    dev_status, (hipStream_t)stream));
}

// Set-associative LFU populate: counts -> priority order -> set-major order -> one wave
// per set keeps / replaces ways -> map rebuilt -> newcomers' rows rebuilt and scattered.
static int populate_lfu(tt_cache *c, const float *const cores[3], float *rows, int64_t *n_filled,
                        int n, hipStream_t s) {
  const long long nsets = c->cache_size / 32;
  hipError_t e = hipSuccess;
  if (n > 0) e = radix_sort64(c->sk0, c->sk1, n, c->shist, s);
  if (e == hipSuccess) e = lfu_setkey_launch(c->sk0, n, c->kbits, nsets, c->lk0, s);
  if (e == hipSuccess && n > 0) e = radix_sort64(c->lk0, c->lk1, n, c->shist, s);
  if (e == hipSuccess) e = hipMemsetAsync(c->set_first, 0xff, (size_t)nsets * 4, s);
  if (e == hipSuccess) e = lfu_first_launch(c->lk0, n, c->set_first, s);
  if (e == hipSuccess) e = hipMemsetAsync(c->lcnt, 0, 8, s);
  if (e == hipSuccess)
    e = lfu_assign_launch(c->sk0, c->lk0, n, c->kbits, c->set_first, nsets, c->cached,
                          c->fresh_slot, c->fresh_idx, c->lcnt, s);
  if (e == hipSuccess) e = hipMemsetAsync(c->mkeys, 0xff, (size_t)c->M * 8, s);
  if (e == hipSuccess) e = map_insert_launch(c->cached, c->cache_size, c->mkeys, c->mslot, c->M, s);
  int cnt[2] = {0, 0};
  if (e == hipSuccess) e = hipMemcpyAsync(cnt, c->lcnt, 8, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return TT_EHIP;
  const int nfresh = cnt[0];
  if (nfresh > 0) {
    int rc = tt_bag_forward(&c->desc, cores, c->fresh_idx, nfresh, c->bag_off, nfresh, nullptr,
                            nullptr, c->rows_tmp, c->fws, c->fws_bytes, nullptr, s);
    if (rc) return rc;
    const int D = c->desc.q[0] * c->desc.q[1] * c->desc.q[2];
    e = scatter_rows_launch(c->rows_tmp, c->fresh_slot, nfresh, D, rows, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return TT_EHIP;
  }
  *n_filled = cnt[1];
  return TT_OK;
}

int tt_cache_populate(tt_cache *c, const float *const cores[3], float *rows, int64_t *n_filled,
                      void *stream) {
  if (!c || !cores || !cores[0] || !cores[1] || !cores[2] || !rows || !n_filled) return TT_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipMemsetAsync(c->nent, 0, 4, s);
  if (e == hipSuccess) e = cache_compact_launch(c->hkeys, c->hcnt, c->H, c->kbits, c->sk0, c->nent, s);
  int n = 0;
  if (e == hipSuccess) e = hipMemcpyAsync(&n, c->nent, 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return TT_EHIP;
  if (c->policy == TT_CACHE_LFU32) return populate_lfu(c, cores, rows, n_filled, n, s);
  e = radix_sort64(c->sk0, c->sk1, n, c->shist, s);
  const int nf = (int)(n < c->cache_size ? n : c->cache_size);
  if (e == hipSuccess) e = hipMemsetAsync(c->mkeys, 0xff, (size_t)c->M * 8, s);
  if (e == hipSuccess)
    e = cache_assign_launch(c->sk0, nf, c->kbits, c->cache_size, c->cached, c->mkeys, c->mslot,
                            c->M, s);
  if (e != hipSuccess) return TT_EHIP;
  if (nf > 0) {
    int rc = tt_bag_forward(&c->desc, cores, c->cached, nf, c->bag_off, nf, nullptr, nullptr, rows,
                            c->fws, c->fws_bytes, nullptr, stream);
    if (rc) return rc;
  }
  e = hipStreamSynchronize(s);
  if (e != hipSuccess) return TT_EHIP;
  *n_filled = nf;
  return TT_OK;
}

int tt_cache_export(tt_cache *c, int64_t *cached_out, int64_t *keys_out, int32_t *counts_out,
                    void *stream) {
  if (!c || !cached_out || !keys_out || !counts_out) return TT_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(cached_out, c->cached, (size_t)c->cache_size * 8,
                                hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(keys_out, c->hkeys, (size_t)c->H * 8, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(counts_out, c->hcnt, (size_t)c->H * 4, hipMemcpyDeviceToDevice, s);
  return finish(e);
}

int tt_cache_import(tt_cache *c, const int64_t *cached, const int64_t *keys,
                    const int32_t *counts, void *stream) {
  if (!c || !cached || !keys || !counts) return TT_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(c->cached, cached, (size_t)c->cache_size * 8,
                                hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(c->hkeys, keys, (size_t)c->H * 8, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(c->hcnt, counts, (size_t)c->H * 4, hipMemcpyDeviceToDevice, s);
  if (e == hipSuccess) e = hipMemsetAsync(c->mkeys, 0xff, (size_t)c->M * 8, s);
  if (e == hipSuccess) e = map_insert_launch(c->cached, c->cache_size, c->mkeys, c->mslot, c->M, s);
  return finish(e);
}

int tt_cache_cached_indices(tt_cache *c, int64_t *cached_out, void *stream) {
  if (!c || !cached_out) return TT_EINVAL;
  return finish(hipMemcpyAsync(cached_out, c->cached, (size_t)c->cache_size * 8,
                               hipMemcpyDeviceToDevice, (hipStream_t)stream));
}

int tt_cache_destroy(tt_cache *c) {
  if (!c) return TT_EINVAL;
  (void)hipDeviceSynchronize();
  cache_free(c);
  return TT_OK;
}

}  // extern "C"

// ---------------------------------------------------------------- forward without allocation
// For callers that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid it): tt_bag_forward_static runs the grouping and
// the forward in a scratch array of the library instead of a caller workspace.  Each GPU
// holds its own copy of `scratch` (static storage, zero at load; nothing in it needs
// clearing: histograms are cleared by the grouping kernels themselves and the flag and
// counter words carry each call's epoch).  Host code never takes the array's name for an
// address: the device address comes from hipGetSymbolAddress once per device.
static __device__ __align__(256) unsigned char scratch[TT_STATIC_SCRATCH_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void *g_scratch[MAX_DEVICES];

// the current device's copy of `scratch` (looked up on the first call on that device)
void *scratch_of_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch[dev] = ptr;
  }
  return g_scratch[dev];
}
}  // namespace

extern "C" int tt_bag_forward_static(const tt_desc *desc, const float *const cores[3],
                                     const int64_t *indices, int64_t nnz, const int64_t *offsets,
                                     int64_t num_bags, const float *per_sample_weights,
                                     const tt_cache_view *cache, float *out, int32_t *dev_status,
                                     void *stream) {
  Plan P;
  int rc = make_plan(desc, nnz, num_bags, cache ? cache->cache_size : 0, &P);
  if (rc) return rc;
  if (P.ws_fwd > (size_t)TT_STATIC_SCRATCH_BYTES) return TT_EWORKSPACE;  // batch too large
  void *ws = scratch_of_current_device();
  if (!ws) return TT_EHIP;
  return forward_call(desc, cores, indices, nnz, offsets, num_bags, per_sample_weights, cache,
                      out, ws, TT_STATIC_SCRATCH_BYTES, dev_status, stream, true);
}
