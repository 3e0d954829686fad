// tt_route.hip -- grouping of the looked-up indices (index split, bag ids,
// validation, stable counting sorts) and the per-run sums of the upstream grad.
//
// "FBTT-Embedding" README, "Parameters"/"Initialization": row i of a table is
// addressed by (i1,i2,i3), a mixed-radix split of i over tt_p_shapes (row-major:
// i = (i1*p2 + i2)*p3 + i3).  Bags follow EmbeddingBag's CSR offsets.  Grouping
// the elements by the core-2 slice i2 lets one workgroup reuse a G2 slice for all
// its elements and share the G1*G2 product between elements with the same
// (i1,i2); the page's kernel relies on cub for its device-wide primitives, here
// each pass is a hand-written stable counting sort (LSD, three digits).
#include "tt_device.h"
#include "tt_mfma.h"

namespace ttb {

static __device__ __forceinline__ bool a_le(const int64_t *off, int c, int n) {
  return off[c] <= (int64_t)n;
}

// Largest b in [0, NB) with off[b] <= n, found by 128 threads (`half` = 0: threads
// 0..127, 1: threads 128..255) with a 128-ary search: one global load per thread per
// round.  Every thread of the block calls it (barriers); threads from 256 on only
// take part in the barriers.
static __device__ int half_find_bag(const int64_t *off, int NB, int n, int half, int *s_red) {
  const int t = threadIdx.x - half * 128, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const bool searcher = threadIdx.x < 256;
  int lo = 0;
  // invariant: the answer lies in [lo, lo + span).  The number of rounds depends on NB
  // only, so both halves meet every barrier.
  for (int span = NB; span > 1;) {
    const int step = (span + 127) / 128;
    const int c = lo + t * step;
    const bool ok = searcher && t * step < span && c < NB && a_le(off, c, n);
    int best = wave_max(ok ? t : -1);
    if (lane == 0 && searcher) s_red[w] = best;
    __syncthreads();
    best = max(s_red[half * 2], s_red[half * 2 + 1]);
    __syncthreads();
    if (best > 0) lo += best * step;  // best < 0 only with invalid offsets: keep lo
    span = step;
  }
  return lo;
}

constexpr int ROUTE_MAX_BAGS = 2048;  // offsets of one routing block kept in LDS

// ---------------------------------------------------------------- shared pieces
// A tile is RB = 1024 consecutive positions, held by a block of NT threads with
// EPT = RB / NT elements each: element r of thread tid of wave w sits at position
// w*64*EPT + r*64 + lane of the tile (the order the block ranks keep).
template <int NT>
static __device__ __forceinline__ int tile_pos(int blk, int r) {
  return blk * RB + (threadIdx.x >> 6) * (64 * (RB / NT)) + r * 64 + (threadIdx.x & 63);
}

// Word accesses for data that other blocks of the same launch read after a grid
// barrier (DEV = true): device-coherent (L2-bypassing) stores and loads, so that the
// barrier needs no cache write-back.  Plain accesses otherwise (kernel boundaries
// order them).
template <bool DEV>
static __device__ __forceinline__ void st_w(int *p, int v) {
  if (DEV) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *p = v;
}
template <bool DEV>
static __device__ __forceinline__ int ld_w(const int *p) {
  if (DEV) return __hip_atomic_load((int *)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return *p;
}

// One element on its way through the passes (a "record": 8 words in the workspace).
struct Rec {
  int e, dA, dB, dI, bag, posI3;
  float w;
};
constexpr int REC_WORDS = 8;

static __device__ __forceinline__ void store_rec(int *rec, int pos, const Rec &r) {
  int4 *q = (int4 *)(rec + (size_t)pos * REC_WORDS);
  q[0] = make_int4(r.e, r.dA, r.dB, r.dI);
  q[1] = make_int4(r.bag, r.posI3, __float_as_int(r.w), 0);
}
static __device__ __forceinline__ Rec load_rec(const int *rec, int pos) {
  const int4 *q = (const int4 *)(rec + (size_t)pos * REC_WORDS);
  const int4 u = q[0], v = q[1];
  Rec r;
  r.e = u.x; r.dA = u.y; r.dB = u.z; r.dI = u.w;
  r.bag = v.x; r.posI3 = v.y; r.w = __int_as_float(v.z);
  return r;
}

// Tile decode: bag, digits dA (t,i1), dB (t,i2), dI (t,i3) and weight of the tile's
// elements (digits -1 past the end); bad indices / slots reported.  Needs LDS s_off
// [ROUTE_MAX_BAGS], s_red [8], s_b [2].  Whole block.
template <int NT>
static __device__ void tile_decode(const DevArgs &a, int blk, int *s_off, int *s_red, int *s_b,
                                   Rec el[RB / NT]) {
  const int tid = threadIdx.x;
  // the element loads first: they do not depend on the bags
  int64_t iv[RB / NT];
  int sv[RB / NT];
#pragma unroll
  for (int r = 0; r < RB / NT; ++r) iv[r] = a.idx[min(tile_pos<NT>(blk, r), a.nnz - 1)];
  if (a.has_cache && a.slots) {
#pragma unroll
    for (int r = 0; r < RB / NT; ++r) sv[r] = a.slots[min(tile_pos<NT>(blk, r), a.nnz - 1)];
  } else {
#pragma unroll
    for (int r = 0; r < RB / NT; ++r) sv[r] = -1;
  }
  if (a.psw) {
#pragma unroll
    for (int r = 0; r < RB / NT; ++r) el[r].w = a.psw[min(tile_pos<NT>(blk, r), a.nnz - 1)];
  } else {
#pragma unroll
    for (int r = 0; r < RB / NT; ++r) el[r].w = 1.f;
  }
  // the bags that may hold the tile's positions: all of them when their offsets fit in
  // LDS, else the ones overlapping the tile (one 128-ary search per half of the block)
  int b_lo = 0, nbag = a.NB;
  if (a.NB + 1 > ROUTE_MAX_BAGS) {
    const int base = blk * RB, last = min(base + RB, a.nnz) - 1;
    const int half = min(tid >> 7, 1);
    const int b = half_find_bag(a.off, a.NB, half ? last : base, half, s_red);
    if (tid == 0 || tid == 128) s_b[half] = b;
    __syncthreads();
    b_lo = s_b[0];
    nbag = max(s_b[1], s_b[0]) - b_lo + 1;
  }
  const bool in_lds = nbag + 1 <= ROUTE_MAX_BAGS;
  if (in_lds) {  // ROUTE_MAX_BAGS / NT = 8 loads per thread, all in flight
    int64_t o[ROUTE_MAX_BAGS / NT];
#pragma unroll
    for (int u = 0; u < ROUTE_MAX_BAGS / NT; ++u) o[u] = a.off[b_lo + min(tid + u * NT, nbag)];
#pragma unroll
    for (int u = 0; u < ROUTE_MAX_BAGS / NT; ++u)
      if (tid + u * NT <= nbag) s_off[tid + u * NT] = (int)(o[u] < 0 ? 0 : (o[u] > a.nnz ? a.nnz : o[u]));
  }
  __syncthreads();
  // bag = last b with off[b] <= e: binary lifting over the offsets in LDS, the four
  // elements in lockstep (or a search in global memory for tiles of very many bags)
  int bag[RB / NT];
  if (in_lds) {
    int lo[RB / NT];
#pragma unroll
    for (int r = 0; r < RB / NT; ++r) lo[r] = 0;
    int top = 1;
    while (top < nbag + 1) top <<= 1;
    for (int span = top >> 1; span > 0; span >>= 1) {
      int ov[RB / NT];
#pragma unroll
      for (int r = 0; r < RB / NT; ++r) ov[r] = s_off[min(lo[r] + span, nbag)];
#pragma unroll
      for (int r = 0; r < RB / NT; ++r)
        lo[r] = (lo[r] + span <= nbag && ov[r] <= tile_pos<NT>(blk, r)) ? lo[r] + span : lo[r];
    }
#pragma unroll
    for (int r = 0; r < RB / NT; ++r) bag[r] = b_lo + min(lo[r], nbag - 1);
  } else {
#pragma unroll
    for (int r = 0; r < RB / NT; ++r) bag[r] = find_bag(a.off, a.NB, min(tile_pos<NT>(blk, r), a.nnz - 1));
  }
  if (a.mean) {  // mean pooling: the weight carries 1 / (bag length)
#pragma unroll
    for (int r = 0; r < RB / NT; ++r) {
      int64_t len;
      if (in_lds) {
        const int k = min(bag[r] - b_lo, nbag - 1);
        len = s_off[k + 1] - s_off[k];
      } else {
        len = a.off[bag[r] + 1] - a.off[bag[r]];
      }
      el[r].w = el[r].w / (float)(len > 0 ? len : 1);
    }
  }
  const int dropA = a.binsA - 1, dropB = a.binsB - 1, dropI = a.binsI3 - 1;
  const int64_t p23 = (int64_t)a.p2 * a.p3;
  const int n = elem_count(a);
  bool bad_slot = false, bad_index = false;
#pragma unroll
  for (int r = 0; r < RB / NT; ++r) {
    const int e = tile_pos<NT>(blk, r);
    Rec &x = el[r];
    x.e = e;
    x.bag = bag[r];
    x.posI3 = -1;
    x.dA = x.dB = x.dI = -1;
    if (e >= n) continue;
    const int t = a.T == 1 ? 0 : bag[r] / a.B;
    const int slot = sv[r];
    const int64_t i = iv[r];
    if (slot >= 0) {
      if (slot >= a.cache_size) {
        bad_slot = true;
        x.dA = dropA; x.dB = dropB; x.dI = dropI;
      } else {
        x.dA = a.T * a.p1 + slot % HB;
        x.dB = a.T * a.p2 + slot / HB;
        x.dI = dropI;
      }
    } else if (i < 0 || i >= a.E) {
      bad_index = true;
      x.dA = dropA; x.dB = dropB; x.dI = dropI;
    } else {
      int i1, i2, i3;
      split_index(i, a.p3, p23, a.rp23, a.rp3, i1, i2, i3);
      x.dA = t * a.p1 + i1;
      x.dB = t * a.p2 + i2;
      x.dI = t * a.p3 + i3;
    }
  }
  if (bad_slot) set_status(a.status, TT_DEV_BAD_SLOT);
  if (bad_index) set_status(a.status, TT_DEV_BAD_INDEX);
}

// Offsets must be a CSR over [0, nnz]; checked grid-strided by the nblk blocks.
template <int NT>
static __device__ void check_offsets(const DevArgs &a, int blk) {
  const int gt = blk * NT + threadIdx.x, gn = a.nblk * NT, n = elem_count(a);
  for (int k = gt; k <= a.NB; k += gn) {
    const int64_t o = a.off[k], o1 = a.off[min(k + 1, a.NB)];
    if ((k == 0 && o != 0) || (k == a.NB && o != (int64_t)n) || (k < a.NB && o1 < o))
      set_status(a.status, TT_DEV_BAD_OFFSETS);
  }
}

// Tile histogram of digit d; column blk of the [bin][tile] matrix (TILE_MAJOR false)
// or row blk of the [tile][bin] matrix (true).
template <int NT, bool DEV, bool TILE_MAJOR>
static __device__ void tile_hist(const int d[RB / NT], int *lds_h, int nb, int *hist, int blk) {
  const int tid = threadIdx.x;
  for (int i = tid; i < nb; i += NT) lds_h[i] = 0;
  __syncthreads();
#pragma unroll
  for (int r = 0; r < RB / NT; ++r)
    if (d[r] >= 0) atomicAdd(&lds_h[d[r]], 1);
  __syncthreads();
  for (int i = tid; i < nb; i += NT)
    st_w<DEV>(TILE_MAJOR ? hist + (size_t)blk * nb + i : hist + (size_t)i * gridDim.x + blk,
              lds_h[i]);
}

// Stable ranks of the tile's elements by digit d (order: position) and their output
// positions start[d * ss + so] + rank.
template <int NT>
static __device__ void tile_place(const int d[RB / NT], int pos[RB / NT], unsigned short *lds_c, int nb,
                                  const int *start, int ss, int so) {
  int rk[RB / NT];
  block_rank<NT, RB / NT>(d, rk, lds_c, nb, nbits_for(nb));
#pragma unroll
  for (int r = 0; r < RB / NT; ++r) pos[r] = d[r] >= 0 ? start[(size_t)d[r] * ss + so] + rk[r] : -1;
}

// Workgroup slot of the j-th largest of n work items (the contraction kernels run work
// item k in the workgroup of slot k).  The dispatcher hands out workgroups round-robin
// over the XCDs and their CUs, so with C CUs, workgroups w and w + C share a CU when a
// launch has between C and 2C of them.  Then the 2C - n largest items get a CU of their
// own and the others share one in pairs, the largest with the smallest, so that the CUs
// finish at about the same time; with n <= C or n > 2C the largest go first.  Only the
// placement depends on this: every result is keyed by the item, not by its slot.
__device__ __forceinline__ int item_slot(int j, int n, int C) {
  if (C <= 0 || n <= C || n > 2 * C) return j;
  const int pairs = n - C, alone = C - pairs;
  if (j < alone) return pairs + j;
  const int k = j - alone;
  return k < pairs ? k : C + (2 * pairs - 1 - k);
}

// Work items from the group table gs[0..binsB] (starts of the (t,i2) bins in the final
// order, gs[binsB] = nnz; LDS or global): a miss group of m elements becomes ceil(m / P)
// items (two near-equal halves, or P positions each but the last when there are three or
// more), numbered group by group; also
// grp_off, chunk_pre and the header words.  Every block of a launch may call it with
// its own part: all compute the item numbering (cnt: G + 1 ints of scratch, LDS or
// global), part k of nparts writes the entries of the groups g = k (mod nparts).
static __device__ void build_items(const DevArgs &a, const int *gs, int *cnt, int *s_scan,
                                   int part, int nparts) {
  const int G = a.T * a.p2, tid = threadIdx.x, nt = blockDim.x, lane = tid & 63, w = tid >> 6;
  const int lP = 31 - __clz(a.P), P1 = a.P - 1;  // P is a power of two
  // exclusive scan of the item counts on contiguous runs per thread
  const int per = (G + nt) / nt, beg = min(tid * per, G + 1), end = min(beg + per, G + 1);
  int sum = 0;
  for (int g = beg; g < end; ++g) sum += g < G ? (gs[g + 1] - gs[g] + P1) >> lP : 0;
  const int incl = wave_incl_scan(sum);
  if (lane == 63) s_scan[w] = incl;
  __syncthreads();
  int run = incl - sum;
  for (int v = 0; v < w; ++v) run += s_scan[v];
  for (int g = beg; g < end; ++g) {
    cnt[g] = run;
    run += g < G ? (gs[g + 1] - gs[g] + P1) >> lP : 0;
  }
  __threadfence_block();
  __syncthreads();
  // items per size (piece_cut below), then the number of items larger than each size
  __shared__ int s_above[P_MAX + 2];
  for (int k = tid; k < P_MAX + 2; k += nt) s_above[k] = 0;
  __syncthreads();
  for (int g = tid; g < G; g += nt) {
    const int nc = cnt[g + 1] - cnt[g], m = gs[g + 1] - gs[g];
    if (nc == 0) continue;
    if (nc <= 2) {  // near-equal: m mod nc of size m / nc + 1, the rest m / nc
      const int q = m / nc, r = m - q * nc;
      if (r) atomicAdd(&s_above[q + 1], r);
      if (nc > r) atomicAdd(&s_above[q], nc - r);
    } else {  // nc - 1 of P and the rest
      atomicAdd(&s_above[a.P], nc - 1);
      atomicAdd(&s_above[m - (nc - 1) * a.P], 1);
    }
  }
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int k = P_MAX + 1; k >= 0; --k) {
      const int c = s_above[k];
      s_above[k] = run;
      run += c;
    }
  }
  __syncthreads();
  const int nitems = cnt[G];
  for (int b = part + tid * nparts; b <= a.binsB; b += nt * nparts) a.grp_off[b] = gs[b];
  for (int g = part + tid * nparts; g <= G; g += nt * nparts) a.chunk_pre[g] = cnt[g];
  for (int g = part + tid * nparts; g < G; g += nt * nparts) {
    const int first = cnt[g], nc = cnt[g + 1] - first;
    const int gb = gs[g], m = gs[g + 1] - gb;
    if (nc == 0) continue;
    // piece_cut: a group in two items is cut in near-equal halves; a larger one into items of
    // P positions and the rest (fewer partly filled M-blocks where groups are large)
    const int q = m / nc, r = m - q * nc;
    auto cut = [&](int c) { return nc <= 2 ? gb + q * c + (r * c) / nc : gb + c * a.P; };
    int lo = gb;
    for (int c = 0; c < nc; ++c) {
      const int hi = c + 1 < nc ? cut(c + 1) : gb + m;
      // its rank among the items of its size (any order: only the placement uses it)
      const int j = s_above[hi - lo] + atomicAdd(&a.hdr[H_SIZE0 + hi - lo], 1);
      a.fitem[first + c] = make_int4(g, lo, hi, item_slot(j, nitems, a.ncu));
      lo = hi;
    }
  }
  if (part == 0 && tid == 0) {
    a.hdr[H_NFWD] = cnt[G];
    a.hdr[H_HIT_BEG] = gs[G];
    a.hdr[H_HIT_END] = gs[a.binsB - 1];
    a.hdr[H_VALID] = gs[a.binsB - 1];
  }
}

// orderI3 / orderA places of the tile's elements (from their bin starts); the records
// go to their orderA positions.  Returns the orderA positions (-1: none).
template <int NT>
static __device__ void tile_place_ia(const DevArgs &a, Rec el[RB / NT], int pA[RB / NT], unsigned short *lds_c,
                                     const int *startI, const int *startA, int ss, int so) {
  int d[RB / NT], pI[RB / NT];
#pragma unroll
  for (int r = 0; r < RB / NT; ++r) d[r] = el[r].dI;
  tile_place<NT>(d, pI, lds_c, a.binsI3, startI, ss, so);
  __syncthreads();
#pragma unroll
  for (int r = 0; r < RB / NT; ++r) d[r] = el[r].dA;
  tile_place<NT>(d, pA, lds_c, a.binsA, startA, ss, so);
#pragma unroll
  for (int r = 0; r < RB / NT; ++r) {
    if (pA[r] < 0) continue;
    el[r].posI3 = pI[r];
    store_rec(a.rec, pA[r], el[r]);
  }
}

// The records of tile blk of orderA (positions past the end repeat the last record).
template <int NT>
static __device__ void tile_load(const DevArgs &a, int blk, Rec x[RB / NT]) {
#pragma unroll
  for (int r = 0; r < RB / NT; ++r) x[r] = load_rec(a.rec, min(tile_pos<NT>(blk, r), a.nnz - 1));
}

// Final pass of a tile of orderA (its records x, from tile_load): placed by (t,i2) into
// the final order.
template <int NT>
static __device__ void tile_final(const DevArgs &a, int blk, unsigned short *lds_c,
                                  const int *start, int ss, int so, const Rec x[RB / NT]) {
  int d[RB / NT], pos[RB / NT];
  const int n = elem_count(a);
#pragma unroll
  for (int r = 0; r < RB / NT; ++r) d[r] = tile_pos<NT>(blk, r) < n ? x[r].dB : -1;
  tile_place<NT>(d, pos, lds_c, a.binsB, start, ss, so);
#pragma unroll
  for (int r = 0; r < RB / NT; ++r) {
    if (pos[r] < 0) continue;
    const int p = pos[r];
    a.srec[2 * (size_t)p] = make_int4(x[r].e, x[r].dA, x[r].dB, x[r].dI);
    a.srec[2 * (size_t)p + 1] = make_int4(x[r].bag, x[r].posI3, __float_as_int(x[r].w),
                                          tile_pos<NT>(blk, r));
  }
}

// ---------------------------------------------------------------- one-launch path
constexpr int CT = 1024;               // threads of a block of that launch (one element each)
constexpr int COOP_BINS = 2048;        // bins per digit

// Compute units of the current device (cached per device).
int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (!cus[dev] && hipDeviceGetAttribute(&cus[dev], hipDeviceAttributeMultiprocessorCount, dev) !=
                       hipSuccess)
    cus[dev] = 0;
  return cus[dev];
}

static bool coop_route_ok(const DevArgs &a) {
  return a.nblk <= COOP_TILES && a.nblk <= device_cus() && a.binsA <= COOP_BINS &&
         a.binsB <= COOP_BINS && a.binsI3 <= COOP_BINS &&
         (int64_t)a.binsA * a.nblk <= COOP_CELLS && (int64_t)a.binsB * a.nblk <= COOP_CELLS &&
         (int64_t)a.binsI3 * a.nblk <= COOP_CELLS;
}

// All blocks of the launch meet here (k-th barrier).  Data crossing the barrier is
// either written with device-coherent stores or atomics, complete before the block
// arrives (FENCE = false), or made visible by device-scope fences around the barrier
// (FENCE = true: plain stores and loads, at the price of an L2 write-back).  Arrival
// is one device-coherent store of (epoch << 32 | k) into the block's own flag word (no
// read-modify-write, so arrivals never contend); the first wave then reads all flags
// until each holds this call's epoch and a count >= k.  Words left by another call
// carry another epoch, so the flags never need clearing.  The wait is bounded: a block
// that gives up reports TT_DEV_SYNC_TIMEOUT and returns false (its caller leaves the
// kernel; no plan is marked valid).
template <bool FENCE>
static __device__ bool grid_sync(const DevArgs &a, unsigned k) {
  __shared__ int s_ok;
  const int tid = threadIdx.x, nblk = gridDim.x;
  // every wave's stores are complete; one thread then fences for the whole block (the
  // L2 write-back / invalidate act on the caches the block's waves share)
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0) {
    if (FENCE) __threadfence();
    __hip_atomic_store(&a.flag[blockIdx.x], ((unsigned long long)a.epoch << 32) | k,
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (tid < 64) {
    int ok = 1;
    for (unsigned polls = 0;; ++polls) {
      if (polls >= a.sync_polls) {  // (a limit of 0 gives up before the first poll)
        ok = 0;
        if (tid == 0) set_status(a.status, TT_DEV_SYNC_TIMEOUT);
        break;
      }
      bool mine = true;  // this lane's flags (blocks tid, tid + 64, ...) have arrived
      for (int b = tid; b < nblk; b += 64) {
        const unsigned long long v =
            __hip_atomic_load(&a.flag[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        mine = mine && (unsigned)(v >> 32) == a.epoch && (unsigned)v >= k;
      }
      if (__ballot(!mine) == 0ull) break;
      __builtin_amdgcn_s_sleep(1);
    }
    if (tid == 0) {
      if (FENCE) __threadfence();
      s_ok = ok;
    }
  }
  __syncthreads();
  return s_ok != 0;
}

// Per-tile bin starts of two digits from their [tile][bin] count matrices (read whole
// by every block): start[d] = (elements in smaller bins) + (elements of bin d in tiles
// < blk); gsum[d] = the global bin starts.  LDS arrays of nb (+1) ints.  Thread t sums
// the column of bin t (then t + CT, ...) over 16 tiles per round of loads (all in
// flight); threads without a bin issue no loads.  The exclusive scan over bins then
// runs on contiguous runs of the LDS totals.
constexpr int SCAN_TCH = 16;
static __device__ void tile_starts2(const int *h0, int nb0, int *start0, int *gs0, const int *h1,
                                   int nb1, int *start1, int *gs1, int blk, int *s_scan) {
  const int nblk = gridDim.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int nbt = nb0 + nb1;
  for (int j = tid; j < nbt; j += CT) {
    const bool first = j < nb0;
    const int *col = first ? h0 + j : h1 + (j - nb0);
    const int nb = first ? nb0 : nb1;
    int tot = 0, pre = 0;
    for (int t0 = 0; t0 < nblk; t0 += SCAN_TCH) {
      int v[SCAN_TCH];
#pragma unroll
      for (int u = 0; u < SCAN_TCH; ++u)
        v[u] = ld_w<true>(col + (size_t)min(t0 + u, nblk - 1) * nb);
#pragma unroll
      for (int u = 0; u < SCAN_TCH; ++u) {
        const int t = t0 + u;
        tot += t < nblk ? v[u] : 0;
        pre += t < blk ? v[u] : 0;
      }
    }
    if (first) { gs0[j] = tot; start0[j] = pre; }
    else { gs1[j - nb0] = tot; start1[j - nb0] = pre; }
  }
  __syncthreads();
  // exclusive scans over the bins of each digit, on contiguous runs per thread
  const int per = (nbt + CT - 1) / CT;
  int run0 = 0, run1 = 0;
  for (int k = 0; k < per; ++k) {
    const int j = tid * per + k;
    if (j < nb0) run0 += gs0[j];
    else if (j < nbt) run1 += gs1[j - nb0];
  }
  int x0 = run0, x1 = run1;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y0 = __shfl_up(x0, o), y1 = __shfl_up(x1, o);
    if (lane >= o) { x0 += y0; x1 += y1; }
  }
  if (lane == 63) { s_scan[w] = x0; s_scan[CT / 64 + w] = x1; }
  __syncthreads();
  int b0 = x0 - run0, b1 = x1 - run1;
  for (int v = 0; v < w; ++v) { b0 += s_scan[v]; b1 += s_scan[CT / 64 + v]; }
  for (int k = 0; k < per; ++k) {
    const int j = tid * per + k;
    if (j < nb0) {
      const int c = gs0[j];
      gs0[j] = b0;
      start0[j] += b0;
      b0 += c;
    } else if (j < nbt) {
      const int c = gs1[j - nb0];
      gs1[j - nb0] = b1;
      start1[j - nb0] += b1;
      b1 += c;
    }
  }
  __syncthreads();
}

// LDS of the one-launch kernel (ints, sized by the call's bins and tiles), phases overlap:
//   decode:  s_off [ROUTE_MAX_BAGS] | hist [max(binsI3, binsA)]
//   passes:  rank counts (u16, waves x bins) | startI, gsI | startA, gsA | (t,i2) cells
//            (the tiles' matrix, or this tile's row)
struct CoopLds {
  int c, sI, gI, sA, gA, cell, total;
};
__host__ __device__ inline CoopLds coop_lds(const DevArgs &a) {
  const int mb = max(a.binsI3, max(a.binsA, a.binsB));
  const int nX = max(a.binsI3, a.binsB) + 1, nY = max(a.binsA, a.binsB) + 1;
  CoopLds L;
  L.c = 0;
  L.sI = (CT / 64) * mb / 2 + 1;  // u16 counts per wave and bin
  L.gI = L.sI + nX;
  L.sA = L.gI + nX;
  L.gA = L.sA + nY;
  L.cell = L.gA + nY;
  // the [tile][bin] (t,i2) counts, or one row of them
  const int cells = a.binsB * a.nblk <= COOP_LDS_CELLS ? a.binsB * a.nblk : a.binsB;
  L.total = max(L.cell + cells, ROUTE_MAX_BAGS + max(a.binsI3, a.binsA));
  return L;
}

__global__ __launch_bounds__(CT) void k_route_coop(DevArgs a) {
  a.epoch = launch_tag(a, a.hdr + H_REPOCH);  // this grouping's tag
  extern __shared__ int lds_i[];
  __shared__ int s_scan[2 * (CT / 64) + 1];
  __shared__ int s_red[8];
  __shared__ int s_b[2];
  const int tid = threadIdx.x, blk = blockIdx.x, nblk = gridDim.x;
  const CoopLds L = coop_lds(a);
  unsigned short *lds_c = (unsigned short *)(lds_i + L.c);  // [waves][bins] rank counts
  int *startI = lds_i + L.sI, *gsI = lds_i + L.gI, *startA = lds_i + L.sA, *gsA = lds_i + L.gA;
  int *cellB = lds_i + L.cell;  // [binsB][nblk] (t,i2) counts of the orderA tiles
  Rec el[RB / CT];
  // whatever plan ws held stops being valid before any of it is rewritten (a grouping
  // that gives up at a barrier then leaves no plan that a later call could take for whole)
  if (blk == 0 && tid == 0) a.hdr[H_PLAN] = (int)~a.plan_fp;

  // (t,i2) counts per orderA tile: when that [tile][bin] matrix fits in LDS, each block
  // gathers its elements' contributions there and adds them to histB (cleared first)
  // before the second barrier; otherwise (most of a block's elements would need an atomic
  // of their own) a third barrier follows the placing, and each block counts its own
  // orderA tile and writes its row of histB whole
  const bool in_lds = a.binsB * nblk <= COOP_LDS_CELLS;

  // ---- histB cleared for the atomics; decode; (t,i3) and (t,i1) histograms of the tile
  if (in_lds)
    for (int k = blk * CT + tid; k < a.binsB * nblk; k += nblk * CT) st_w<true>(a.histB + k, 0);
  if (blk == 0)
    for (int k = tid; k <= P_MAX; k += CT) st_w<true>(a.hdr + H_SIZE0 + k, 0);
  tile_decode<CT>(a, blk, lds_i, s_red, s_b, el);
  check_offsets<CT>(a, blk);
  {
    int d[RB / CT];
#pragma unroll
    for (int r = 0; r < RB / CT; ++r) d[r] = el[r].dI;
    tile_hist<CT, true, true>(d, lds_i + ROUTE_MAX_BAGS, a.binsI3, a.histI3, blk);
    __syncthreads();
#pragma unroll
    for (int r = 0; r < RB / CT; ++r) d[r] = el[r].dA;
    tile_hist<CT, true, true>(d, lds_i + ROUTE_MAX_BAGS, a.binsA, a.histA, blk);
  }
  if (!grid_sync<false>(a, 1)) return;

  // ---- orderI3 / orderA places; the (t,i2) counts of the orderA tiles gathered per
  //      block in LDS, then added to histB
  tile_starts2(a.histI3, a.binsI3, startI, gsI, a.histA, a.binsA, startA, gsA, blk, s_scan);
  if (blk == 0) {
    for (int d = tid; d < a.binsI3; d += CT) a.segI3[d] = gsI[d];
    for (int d = tid; d < a.binsA; d += CT) a.segA[d] = gsA[d];
  }
  if (in_lds)
    for (int i = tid; i < a.binsB * nblk; i += CT) cellB[i] = 0;
  int pA[RB / CT];
  tile_place_ia<CT>(a, el, pA, lds_c, startI, startA, 1, 0);
  if (in_lds) {
#pragma unroll
    for (int r = 0; r < RB / CT; ++r)
      if (pA[r] >= 0) atomicAdd(&cellB[el[r].dB * nblk + pA[r] / RB], 1);
    __syncthreads();
    for (int i = tid; i < a.binsB * nblk; i += CT)
      if (cellB[i]) atomicAdd(&a.histB[(i % nblk) * a.binsB + i / nblk], cellB[i]);
  }
  if (!grid_sync<true>(a, 2)) return;
  Rec x[RB / CT];  // this block's tile of orderA
  tile_load<CT>(a, blk, x);
  if (!in_lds) {
    const int n = elem_count(a);
    int d[RB / CT];
#pragma unroll
    for (int r = 0; r < RB / CT; ++r) d[r] = tile_pos<CT>(blk, r) < n ? x[r].dB : -1;
    tile_hist<CT, true, true>(d, lds_i + L.cell, a.binsB, a.histB, blk);
    if (!grid_sync<false>(a, 3)) return;
  }

  // ---- work items (each block writes its share); final order: the orderA tiles placed
  //      by (t,i2)
  tile_starts2(a.histB, a.binsB, startI, gsI, nullptr, 0, nullptr, nullptr, blk, s_scan);
  if (tid == 0) gsI[a.binsB] = elem_count(a);
  __syncthreads();
  build_items(a, gsI, startA, s_scan, blk, nblk);
  tile_final<CT>(a, blk, lds_c, startI, 1, 0, x);
  if (blk == 0 && tid == 0) a.hdr[H_PLAN] = (int)a.plan_fp;
}

// ---------------------------------------------------------------- three-kernel path
// k_route_a: decode, (t,i3) and (t,i1) tile histograms; the last block scans both
// [bin][tile] matrices (bin-major: entry (d, t) becomes the first position of bin d's
// elements of tile t) and records the bin starts.
__global__ __launch_bounds__(RT) void k_route_a(DevArgs a) {
  a.epoch = launch_tag(a, a.hdr + H_REPOCH);  // this grouping's tag
  extern __shared__ int lds_i[];  // s_off [ROUTE_MAX_BAGS] | hist [max(binsI3, binsA)]
  __shared__ int s_scan[RT / 64 + 1];
  __shared__ int s_red[8];
  __shared__ int s_b[2];
  const int blk = blockIdx.x, tid = threadIdx.x;
  Rec el[4];
  if (blk == 0 && tid == 0) a.hdr[H_PLAN] = (int)~a.plan_fp;  // the old plan is void from here
  tile_decode<RT>(a, blk, lds_i, s_red, s_b, el);
  check_offsets<RT>(a, blk);
  for (int k = blk * RT + tid; k < a.binsB * a.nblk; k += a.nblk * RT) a.histB[k] = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r)
    if (el[r].e < elem_count(a)) a.einfo[el[r].e] = make_int4(el[r].dA, el[r].dB, el[r].dI, el[r].bag);
  int d[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) d[r] = el[r].dI;
  tile_hist<RT, false, false>(d, lds_i + ROUTE_MAX_BAGS, a.binsI3, a.histI3, blk);
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 4; ++r) d[r] = el[r].dA;
  tile_hist<RT, false, false>(d, lds_i + ROUTE_MAX_BAGS, a.binsA, a.histA, blk);
  if (!last_block(&a.ctr[0], a.nblk, a.epoch)) return;
  block_exclusive_scan(a.histI3, a.binsI3 * a.nblk, s_scan);
  block_exclusive_scan(a.histA, a.binsA * a.nblk, s_scan);
  for (int k = tid; k < a.binsI3; k += RT) a.segI3[k] = a.histI3[(size_t)k * a.nblk];
  for (int k = tid; k < a.binsA; k += RT) a.segA[k] = a.histA[(size_t)k * a.nblk];
}

// k_route_b: orderI3 / orderA places of the tile (records to orderA); (t,i2) counts
// over the orderA tiles; the last block scans them and builds the group table and the
// work items.
__global__ __launch_bounds__(RT) void k_route_b(DevArgs a) {
  a.epoch = launch_tag(a, a.hdr + H_REPOCH);  // this grouping's tag
  extern __shared__ unsigned short lds_c[];  // [4][max(binsI3, binsA)]
  __shared__ int s_scan[RT / 64 + 1];
  const int blk = blockIdx.x, n = elem_count(a);
  Rec el[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int e = tile_pos<RT>(blk, r), ec = min(e, a.nnz - 1);
    const int4 info = a.einfo[ec];
    const bool v = e < n;
    el[r].e = e;
    el[r].dA = v ? info.x : -1;
    el[r].dB = v ? info.y : -1;
    el[r].dI = v ? info.z : -1;
    el[r].bag = info.w;
    el[r].w = a.psw ? a.psw[ec] : 1.f;
    if (a.mean && v) {  // mean pooling: the weight carries 1 / (bag length)
      const int64_t len = a.off[info.w + 1] - a.off[info.w];
      el[r].w = el[r].w / (float)(len > 0 ? len : 1);
    }
  }
  int pA[4];
  tile_place_ia<RT>(a, el, pA, lds_c, a.histI3, a.histA, a.nblk, blk);
#pragma unroll
  for (int r = 0; r < 4; ++r)
    if (pA[r] >= 0) atomicAdd(&a.histB[(size_t)el[r].dB * a.nblk + pA[r] / RB], 1);
  if (!last_block(&a.ctr[1], a.nblk, a.epoch)) return;
  block_exclusive_scan(a.histB, a.binsB * a.nblk, s_scan);
  for (int d = threadIdx.x; d < a.binsB; d += RT) a.grp_off[d] = a.histB[(size_t)d * a.nblk];
  if (threadIdx.x == 0) a.grp_off[a.binsB] = elem_count(a);
  for (int k = threadIdx.x; k <= P_MAX; k += RT) a.hdr[H_SIZE0 + k] = 0;
  __threadfence();
  __syncthreads();
  build_items(a, a.grp_off, a.chunk_pre, s_scan, 0, 1);
}

// k_route_c: the orderA tiles placed by (t,i2) into the final order.
__global__ __launch_bounds__(RT) void k_route_c(DevArgs a) {
  a.epoch = launch_tag(a, a.hdr + H_REPOCH);  // this grouping's tag
  extern __shared__ unsigned short lds_c[];  // [4][binsB]
  Rec x[RB / RT];
  tile_load<RT>(a, blockIdx.x, x);
  tile_final<RT>(a, blockIdx.x, lds_c, a.histB, a.nblk, blockIdx.x, x);
  if (blockIdx.x == 0 && threadIdx.x == 0) a.hdr[H_PLAN] = (int)a.plan_fp;
}

// Forward: out[b] = sum of the weighted cache rows of bag b (zero when it has none);
// the contraction kernel then adds the misses.  One wave per bag: the slots and
// weights of 64 elements per load, then the hit rows eight at a time (summed in
// position order).
__global__ __launch_bounds__(RT) void k_yinit(DevArgs a) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int b = blockIdx.x * (RT / 64) + w;
  if (b >= a.NB) return;
  if (a.nnz > 0 && a.hdr[H_PLAN] != (int)a.plan_fp) {  // another call's plan: touch nothing
    if (b == 0 && lane == 0) set_status(a.status, DEV_STALE_PLAN);
    return;
  }
  int64_t lo = 0, hi = 0;
  if (a.has_cache) {
    lo = a.off[b];
    hi = a.off[b + 1];
    lo = lo < 0 ? 0 : (lo > a.nnz ? a.nnz : lo);
    hi = hi < lo ? lo : (hi > a.nnz ? a.nnz : hi);
  }
  const float inv = (a.mean && hi > lo) ? 1.f / (float)(hi - lo) : 1.f;
  constexpr int MAXC = 16;  // columns per lane (D <= 1024)
  float acc[MAXC];
#pragma unroll
  for (int k = 0; k < MAXC; ++k) acc[k] = 0.f;
  for (int64_t n0 = lo; n0 < hi; n0 += 64) {
    const int64_t n = n0 + lane;
    const int sl = n < hi ? a.slots[n] : -1;
    const bool hit = sl >= 0 && sl < a.cache_size;
    const float wt = hit ? (a.psw ? a.psw[n] : 1.f) * inv : 0.f;
    unsigned long long m = __ballot(hit);
    while (m) {
      int li[8];
      int cnt = 0;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        li[k] = m ? __ffsll((long long)m) - 1 : -1;
        if (m) { m &= m - 1ull; ++cnt; }
      }
      int rs[8];
      float rw[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int l = li[k] >= 0 ? li[k] : 0;
        rs[k] = __shfl(sl, l);
        rw[k] = li[k] >= 0 ? __shfl(wt, l) : 0.f;
        if (rs[k] < 0) rs[k] = 0;
      }
#pragma unroll
      for (int k2 = 0; k2 < MAXC; ++k2) {
        const int d = lane + 64 * k2;
        if (d >= a.D) break;
        float v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = a.crows[(size_t)rs[k] * a.D + d];
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (k < cnt) acc[k2] += rw[k] * v[k];
      }
    }
  }
#pragma unroll
  for (int k2 = 0; k2 < MAXC; ++k2) {
    const int d = lane + 64 * k2;
    if (d < a.D) a.Y[(size_t)b * a.D + d] = acc[k2];
  }
}

// dL/dw of the cache hits: one thread per position of the hit region,
// <cache row, grad_out[bag]> (times 1 / bag length with mean pooling), 8 loads in flight.
__global__ __launch_bounds__(256) void k_wgrad_hits(DevArgs a) {
  const int hb = a.hdr[H_HIT_BEG], he = a.hdr[H_HIT_END];
  if (a.hdr[H_PLAN] != (int)a.plan_fp) return;  // stale plan: the caller's status shows it
  const int s = hb + blockIdx.x * 256 + threadIdx.x;
  if (s >= he) return;
  const SPos sp = load_spos(a.srec, s);
  const int slot = (sp.dB - a.T * a.p2) * HB + (sp.dA - a.T * a.p1);
  const float *row = a.crows + (size_t)slot * a.D, *dy = a.dY + (size_t)sp.bag * a.D;
  float acc = 0.f;
  for (int d0 = 0; d0 < a.D; d0 += 8) {
    float x[8], y[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int d = min(d0 + u, a.D - 1);
      x[u] = row[d];
      y[u] = dy[d];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (d0 + u < a.D) acc += x[u] * y[u];
  }
  float scale = 1.f;
  if (a.mean) {
    const long long len = a.off[sp.bag + 1] - a.off[sp.bag];
    scale = 1.f / (float)(len > 0 ? len : 1);
  }
  a.gw[sp.n] = acc * scale;
}

hipError_t launch_wgrad_hits(const DevArgs &a, hipStream_t s) {
  if (a.has_cache && a.nnz > 0)
    hipLaunchKernelGGL(k_wgrad_hits, dim3((a.nnz + 255) / 256), dim3(256), 0, s, a);
  return hipGetLastError();
}

// Metadata of every work item (WorkMeta), one wave per work item, after the final order
// and the work items exist: the elements' bags and weights, the items (distinct indices,
// found by wave ballots on i3 inside each pair) and the pairs (runs of equal (t, i1) in
// the (t, i2, i1) order), and the per-M-block loop bounds of the contraction kernels.  It
// also writes the links of the segment sums: the position of each (t,i1)- / (t,i3)-ordered
// element's partial (its pair's / item's first element), or -1.  The contraction kernels
// read the metadata in one round of loads instead of working it out themselves, from the
// workgroup slot the grouping gave the item.  It runs right after the grouping on the
// same stream, so a plan marked valid has its metadata.
// Slot of M-block k among nmb by weight w[0 .. nmb) (larger first, ties by index): the
// heaviest get the slots with a SIMD of their own (sh .. al - 1), the others the shared
// pairs (j, j + 4), the heaviest left in j and the lightest left in j + 4.  Slots >= nmb
// keep their idle M-block.  (All eight weights are read at once.)
__device__ __forceinline__ int weighted_slot(int k, int nmb, const int *w) {
  int x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = w[i];
  const int wk = w[k];
  int p = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) p += (i < nmb && (x[i] > wk || (x[i] == wk && i < k))) ? 1 : 0;
  const int sh = max(nmb - 4, 0), al = min(nmb, 4), q = p - (al - sh);
  if (k >= nmb) return k;
  return q < 0 ? sh + p : (q < sh ? q : (2 * sh - 1 - q) + 4);
}

constexpr int META_WAVES = 4;
__global__ __launch_bounds__(64 * META_WAVES) void k_meta(DevArgs a) {
  __shared__ int s_m[META_WAVES][META_INTS];
  __shared__ int s_cnt[META_WAVES][P_MAX + 24];  // gcnt [32] | mbf [8] | mbb [8] | fwd [8]
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wi = blockIdx.x * META_WAVES + w;
  const int plan = a.hdr[H_PLAN], nitems = a.hdr[H_NFWD];
  // every grouping kernel of this call is done with its tag: the next grouping on this
  // workspace counts one more; and a forward after this grouping starts its block count
  // from zero
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    a.hdr[H_REPOCH] = a.hdr[H_REPOCH] + 1;
    a.hdr[H_FCNT] = 0;
  }
  if (plan != (int)a.plan_fp || wi >= nitems) return;  // (wave-uniform)
  const int4 item = a.fitem[wi];
  const int grp = item.x, s0 = item.y, n_el = item.z - item.y;
  const int t = grp / a.p2;
  const bool v = lane < n_el;
  const int s = s0 + min(lane, n_el - 1);
  const SPos sp = load_spos(a.srec, s);
  const int dA = v ? sp.dA : -1, i3 = v ? sp.dI3 - t * a.p3 : 0;
  const WaveItems r = wave_items(v, dA, i3, nbits_for(a.p3));
  WorkMeta &M = *(WorkMeta *)s_m[w];
  int *cnt = s_cnt[w];
  for (int k = lane; k < META_INTS; k += 64) s_m[w][k] = 0;
  if (lane < P_MAX + 8) cnt[lane] = 0;
  wave_lds_sync();
  if (v) {
    a.link1[sp.posA] = r.pair_st ? s : -1;
    a.link3[sp.posI3] = r.item_st ? s : -1;
    M.e_perm[r.item_pos] = (unsigned char)lane;
    M.e_it[lane] = (unsigned char)r.e_it;
  }
  if (lane < P_MAX) {
    M.e_bag[lane] = sp.bag;
    M.e_w[lane] = sp.w;
  }
  if (r.item_st) {
    M.it_beg[r.it] = (unsigned char)r.it_beg;
    M.it_first[r.it] = (unsigned char)lane;
    M.it_i3[r.it] = (short)i3;
    M.it_pair[r.it] = (unsigned char)r.pair_of;
  }
  if (r.pair_st) {
    M.pr_it[r.pr] = (unsigned char)r.it;
    M.pr_i1[r.pr] = (short)(dA - t * a.p1);
    atomicAdd(&cnt[(r.pr * a.q1) >> 2], r.pair_items);       // rows of a lane group
    atomicMax(&cnt[P_MAX + ((r.pr * a.q1) >> 4)], r.pair_items);  // rows of an M-block
  }
  if (lane == 0) {
    const int nI = __popcll(r.mi), nP = __popcll(r.mp);
    M.n_el = n_el; M.nI = nI; M.nP = nP; M.grp = grp; M.s0 = s0; M.item = wi; M.t = t;
    M.it_beg[nI] = (unsigned char)n_el;
    M.pr_it[nP] = (unsigned char)nI;
  }
  wave_lds_sync();
  if (lane < P_MAX) M.gcnt[lane] = (unsigned char)cnt[lane];
  if (lane < 8) {
    const int mbb = max(max(cnt[4 * lane], cnt[4 * lane + 1]),
                        max(cnt[4 * lane + 2], cnt[4 * lane + 3]));
    M.mbf[lane] = (unsigned char)cnt[P_MAX + lane];
    M.mbb[lane] = (unsigned char)mbb;
    cnt[P_MAX + 8 + lane] = mbb;  // backward weight
    // forward weight: matrix-core stage 2 once per four items of the M-block (q1 = q3 = 4),
    // else the VALU stage 2's mbf
    const int nP = __popcll(r.mp), ppm = 16 >> a.lq1;  // pairs per M-block
    const int p0 = min(lane * ppm, nP), p1 = min(p0 + ppm, nP);
    cnt[P_MAX + 16 + lane] = (a.q1 == 4 && a.q3 == 4) ? (M.pr_it[p1] - M.pr_it[p0] + 3) >> 2
                                                       : cnt[P_MAX + lane];
  }
  wave_lds_sync();
  // M-blocks by placement slot.  The contraction kernels' waves take slots 0 .. 7, slots s
  // and s + 4 on one SIMD (placed_mblock), and a workgroup waits for its slowest SIMD (the
  // backward at every column's barrier, the forward before pooling).  The weights above: the
  // backward's item loop runs mbb times, the forward's stage 2 as noted.  The heaviest
  // M-blocks get the slots that have a SIMD of their own (nmb - 4 .. 3 when there are more
  // than four), the others share one in pairs, the heaviest left with the lightest left.
  // Only the placement depends on this.
  if (lane < 8) {
    const int nmb = min((__popcll(r.mp) * a.q1 + 15) >> 4, 8);
    M.mb_slot[weighted_slot(lane, nmb, cnt + P_MAX + 8)] = (unsigned char)lane;
    M.mb_fslot[weighted_slot(lane, nmb, cnt + P_MAX + 16)] = (unsigned char)lane;
  }
  wave_lds_sync();
  if ((unsigned)item.w >= (unsigned)nitems) return;  // (the slots are a permutation)
  int *dst = a.meta + (size_t)item.w * META_INTS;     // the item's workgroup slot
  for (int k = lane; k < META_INTS; k += 64) dst[k] = s_m[w][k];
}

static hipError_t launch_meta(const DevArgs &a, hipStream_t s) {
  const int nb = (items_max(a) + META_WAVES - 1) / META_WAVES;
  tt_launch(K_META, k_meta, dim3(nb), dim3(64 * META_WAVES), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_route(const DevArgs &args, hipStream_t s) {
  DevArgs a = tag_for_launch(args, s);
  a.ncu = device_cus();
  if (a.nblk == 0) return hipGetLastError();
  if (coop_route_ok(a)) {
    static size_t attr_lds = 64 * 1024;  // dynamic LDS above 64 KiB is opt-in per kernel
    const size_t lds = (size_t)coop_lds(a).total * 4;
    if (lds > attr_lds) {
      const hipError_t e = hipFuncSetAttribute((const void *)k_route_coop,
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
      attr_lds = lds;
    }
    // One block per CU at most (LDS), launched on an otherwise idle stream position:
    // every block is resident at once.  The barriers are bounded waits in any case.
    tt_launch(K_ROUTE_COOP, k_route_coop, dim3(a.nblk), dim3(CT), lds, s, a);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? launch_meta(a, s) : e;
  }
  const size_t bins_ia = (size_t)(a.binsI3 > a.binsA ? a.binsI3 : a.binsA);
  tt_launch(K_ROUTE_A, k_route_a, dim3(a.nblk), dim3(RT), (ROUTE_MAX_BAGS + bins_ia) * 4, s, a);
  tt_launch(K_ROUTE_B, k_route_b, dim3(a.nblk), dim3(RT), bins_ia * 8, s, a);
  tt_launch(K_ROUTE_C, k_route_c, dim3(a.nblk), dim3(RT), (size_t)a.binsB * 8, s, a);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? launch_meta(a, s) : e;
}

hipError_t launch_yinit(const DevArgs &a, hipStream_t s) {
  if (a.NB > 0) {
    tt_launch(K_YINIT, k_yinit, dim3((a.NB + RT / 64 - 1) / (RT / 64)), dim3(RT), 0, s, a);
  }
  return hipGetLastError();
}


}  // namespace ttb
