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

// Largest b in [0, NB) with off[b] <= n, found by half of the block (128 threads,
// `half` = 0 or 1) with a 128-ary search: one global load per thread per round.
static __device__ int half_find_bag(const int64_t *off, int NB, int n, int half, int *s_red) {
  const int t = threadIdx.x - half * 128, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int lo = 0;
  // invariant: the answer lies in [lo, lo + span).  The number of rounds depends on NB
  // only, so both halves meet every barrier.
  for (int span = NB; span > 1;) {
    const int step = (span + 127) / 128;
    const int c = lo + t * step;
    const bool ok = t * step < span && c < NB && a_le(off, c, n);
    int best = wave_max(ok ? t : -1);
    if (lane == 0) s_red[w] = best;
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
// Positions of the 4 elements of thread tid in tile blk (RB = 1024 per tile).
static __device__ __forceinline__ int tile_pos(int blk, int r) {
  return blk * RB + (threadIdx.x >> 6) * 256 + r * 64 + (threadIdx.x & 63);
}

// Tile decode: bag, digits dA (t,i1), dB (t,i2), dI (t,i3) of the tile's elements (-1 past
// the end), einfo written, bad indices / slots reported.  Needs LDS s_off
// [ROUTE_MAX_BAGS], s_red [8], s_b [2].  Whole block.
static __device__ void tile_decode(const DevArgs &a, int blk, int *s_off, int *s_red, int *s_b,
                                   int dA[4], int dB[4], int dI[4]) {
  const int tid = threadIdx.x;
  const int base = blk * RB, last = min(base + RB, a.nnz) - 1;
  // bags overlapping [base, last]: one 128-ary search per half of the block (lockstep)
  {
    const int half = tid >> 7;
    const int b = half_find_bag(a.off, a.NB, half ? last : base, half, s_red);
    if ((tid & 127) == 0) s_b[half] = b;
  }
  __syncthreads();
  const int b_lo = s_b[0], b_hi = max(s_b[1], s_b[0]);
  const int nbag = b_hi - b_lo + 1;
  const bool in_lds = nbag + 1 <= ROUTE_MAX_BAGS;
  if (in_lds)
    for (int j = tid; j <= nbag; j += RT) {
      const int64_t o = a.off[b_lo + j];
      s_off[j] = (int)(o < 0 ? 0 : (o > a.nnz ? a.nnz : o));
    }
  __syncthreads();
  int64_t iv[4];
  int sv[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) iv[r] = a.idx[min(tile_pos(blk, r), a.nnz - 1)];
  if (a.has_cache && a.slots) {
#pragma unroll
    for (int r = 0; r < 4; ++r) sv[r] = a.slots[min(tile_pos(blk, r), a.nnz - 1)];
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) sv[r] = -1;
  }
  // bag = last b with off[b] <= e: binary lifting over the tile's offsets, the four
  // elements in lockstep (or a search in global memory for tiles of very many bags)
  int bag[4];
  if (in_lds) {
    int lo[4] = {0, 0, 0, 0};
    int top = 1;
    while (top < nbag + 1) top <<= 1;
    for (int span = top >> 1; span > 0; span >>= 1) {
      int ov[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) ov[r] = s_off[min(lo[r] + span, nbag)];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        lo[r] = (lo[r] + span <= nbag && ov[r] <= tile_pos(blk, r)) ? lo[r] + span : lo[r];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) bag[r] = b_lo + min(lo[r], nbag - 1);
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) bag[r] = find_bag(a.off, a.NB, min(tile_pos(blk, r), a.nnz - 1));
  }
  const int dropA = a.binsA - 1, dropB = a.binsB - 1, dropI = a.binsI3 - 1;
  const int64_t p23 = (int64_t)a.p2 * a.p3;
  bool bad_slot = false, bad_index = false;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int e = tile_pos(blk, r);
    dA[r] = dB[r] = dI[r] = -1;
    if (e >= a.nnz) continue;
    const int b = bag[r];
    const int t = a.T == 1 ? 0 : b / a.B;
    const int slot = sv[r];
    const int64_t i = iv[r];
    if (slot >= 0) {
      if (slot >= a.cache_size) {
        bad_slot = true;
        dA[r] = dropA; dB[r] = dropB; dI[r] = dropI;
      } else {
        dA[r] = a.T * a.p1 + slot % HB;
        dB[r] = a.T * a.p2 + slot / HB;
        dI[r] = dropI;
      }
    } else if (i < 0 || i >= a.E) {
      bad_index = true;
      dA[r] = dropA; dB[r] = dropB; dI[r] = dropI;
    } else {
      int i1, i2, i3;
      split_index(i, a.p3, p23, a.rp23, a.rp3, i1, i2, i3);
      dA[r] = t * a.p1 + i1;
      dB[r] = t * a.p2 + i2;
      dI[r] = t * a.p3 + i3;
    }
    a.einfo[e] = make_int4(dA[r], dB[r], dI[r], b);
  }
  if (bad_slot) set_status(a.status, TT_DEV_BAD_SLOT);
  if (bad_index) set_status(a.status, TT_DEV_BAD_INDEX);
}

// Offsets must be a CSR over [0, nnz]; checked grid-strided by the nblk blocks.
static __device__ void check_offsets(const DevArgs &a, int blk) {
  const int gt = blk * RT + threadIdx.x, gn = a.nblk * RT;
  for (int k = gt; k <= a.NB; k += gn) {
    const int64_t o = a.off[k], o1 = a.off[min(k + 1, a.NB)];
    if ((k == 0 && o != 0) || (k == a.NB && o != (int64_t)a.nnz) || (k < a.NB && o1 < o))
      set_status(a.status, TT_DEV_BAD_OFFSETS);
  }
}

// Tile histogram of digit d into column blk of the [bin][tile] matrix hist.
static __device__ void tile_hist(const int d[4], int *lds_h, int nb, int *hist, int blk) {
  const int tid = threadIdx.x;
  for (int i = tid; i < nb; i += RT) lds_h[i] = 0;
  __syncthreads();
#pragma unroll
  for (int r = 0; r < 4; ++r)
    if (d[r] >= 0) atomicAdd(&lds_h[d[r]], 1);
  __syncthreads();
  for (int i = tid; i < nb; i += RT) hist[(size_t)i * gridDim.x + blk] = lds_h[i];
}

// Stable ranks of the tile's elements by digit d (order: position) and their output
// positions start[d * ss + so] + rank.
static __device__ void tile_place(const int d[4], int pos[4], unsigned short *lds_c, int nb,
                                  const int *start, int ss, int so) {
  int rk[4];
  block_rank4(d, rk, lds_c, nb, nbits_for(nb), nullptr, 0);
#pragma unroll
  for (int r = 0; r < 4; ++r) pos[r] = d[r] >= 0 ? start[(size_t)d[r] * ss + so] + rk[r] : -1;
}

// Work items from the group table gs[0..binsB] (starts of the (t,i2) bins in the final
// order, gs[binsB] = nnz; LDS or global): a miss group of m elements becomes ceil(m / P)
// items of near-equal size (at most P positions each), numbered group by group; also
// grp_off and the header words.  Whole block; cnt: G + 1 ints of scratch (LDS or global).
static __device__ void build_items(const DevArgs &a, const int *gs, int *cnt, int *s_scan) {
  const int G = a.T * a.p2, tid = threadIdx.x, nt = blockDim.x;
  for (int g = tid; g <= G; g += nt) {
    const int m = g < G ? gs[g + 1] - gs[g] : 0;
    cnt[g] = (m + a.P - 1) / a.P;
  }
  for (int b = tid; b <= a.binsB; b += nt) a.grp_off[b] = gs[b];
  __threadfence_block();
  __syncthreads();
  block_exclusive_scan(cnt, G + 1, s_scan);
  for (int g = tid; g <= G; g += nt) a.chunk_pre[g] = cnt[g];
  for (int g = tid; g < G; g += nt) {
    const int first = cnt[g], nc = cnt[g + 1] - first;
    const int gb = gs[g], m = gs[g + 1] - gb;
    for (int c = 0; c < nc; ++c)
      a.fitem[first + c] = make_int4(g, gb + (int)((int64_t)m * c / nc),
                                     gb + (int)((int64_t)m * (c + 1) / nc), 0);
  }
  if (tid == 0) {
    a.hdr[H_NFWD] = cnt[G];
    a.hdr[H_HIT_BEG] = gs[G];
    a.hdr[H_HIT_END] = gs[a.binsB - 1];
    a.hdr[H_VALID] = gs[a.binsB - 1];
  }
}

// Final pass of a tile of orderA: the elements' data gathered, placed by (t,i2).
static __device__ void tile_final(const DevArgs &a, int blk, unsigned short *lds_c,
                                  const int *start, int ss, int so) {
  int e[4], d[4], pos[4], pI[4];
  int4 info[4];
  float wv[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) e[r] = a.orderA[min(tile_pos(blk, r), a.nnz - 1)];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    info[r] = a.einfo[e[r]];
    pI[r] = a.posI3_of[e[r]];
  }
  if (a.psw) {
#pragma unroll
    for (int r = 0; r < 4; ++r) wv[r] = a.psw[e[r]];
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) wv[r] = 1.f;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) d[r] = tile_pos(blk, r) < a.nnz ? info[r].y : -1;
  tile_place(d, pos, lds_c, a.binsB, start, ss, so);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (pos[r] < 0) continue;
    const int p = pos[r];
    a.s_n[p] = e[r];
    a.s_dA[p] = info[r].x;
    a.s_dB[p] = info[r].y;
    a.s_dI3[p] = info[r].z;
    a.s_bag[p] = info[r].w;
    a.s_w[p] = wv[r];
    a.s_posI3[p] = pI[r];
    a.s_posA[p] = tile_pos(blk, r);
  }
}

// ---------------------------------------------------------------- cooperative path
constexpr int COOP_TILES = 256;        // blocks of one barrier launch (and at most one per CU)
constexpr int COOP_BINS = 2048;        // bins per digit
constexpr int COOP_CELLS = 12288;      // bins x tiles per digit (each block reads them all)
constexpr unsigned SYNC_POLLS = 1u << 22;  // bounded wait of a grid barrier

// Compute units of the current device (cached per device).
static int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (!cus[dev] && hipDeviceGetAttribute(&cus[dev], hipDeviceAttributeMultiprocessorCount, dev) !=
                       hipSuccess)
    cus[dev] = 0;
  return cus[dev];
}

static bool coop_route_ok(const DevArgs &a) {
  return a.nblk <= COOP_TILES && a.nblk <= device_cus() && a.binsA <= COOP_BINS && a.binsB <= COOP_BINS &&
         a.binsI3 <= COOP_BINS && (int64_t)a.binsA * a.nblk <= COOP_CELLS &&
         (int64_t)a.binsB * a.nblk <= COOP_CELLS && (int64_t)a.binsI3 * a.nblk <= COOP_CELLS;
}

// All blocks of the cooperative launch meet here (k-th barrier: target k * nblk).  The
// counter holds (epoch << 32 | arrivals); a word of another call counts as zero.  The
// wait is bounded: a block that gives up reports TT_DEV_SYNC_TIMEOUT and returns false
// (its caller then leaves the kernel; nothing of the plan is marked valid).
static __device__ bool grid_sync(const DevArgs &a, unsigned target) {
  __shared__ int s_ok;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long *ctr = &a.ctr[0];
    unsigned long long old = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    while (true) {
      const unsigned long long nw = ((unsigned)(old >> 32) == a.epoch)
                                        ? old + 1ull
                                        : (((unsigned long long)a.epoch << 32) | 1ull);
      const unsigned long long prev = atomicCAS(ctr, old, nw);
      if (prev == old) break;
      old = prev;
    }
    int ok = 1;
    for (unsigned polls = 0;; ++polls) {
      const unsigned long long v = __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if ((unsigned)(v >> 32) == a.epoch && (unsigned)v >= target) break;
      if (polls >= SYNC_POLLS) {
        ok = 0;
        set_status(a.status, TT_DEV_SYNC_TIMEOUT);
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
    s_ok = ok;
  }
  __syncthreads();
  __threadfence();
  return s_ok != 0;
}

// Per-tile bin starts from the [bin][tile] count matrix hist (read whole by every
// block): start[d] = (elements in smaller bins) + (elements of bin d in tiles < blk);
// gsum[d] = the global bin starts.  LDS arrays of nb (+1) ints.
static __device__ void tile_starts(const int *hist, int nb, int blk, int *start, int *gsum,
                                   int *s_scan) {
  const int nblk = gridDim.x;
  for (int d = threadIdx.x; d < nb; d += RT) {
    const int *row = hist + (size_t)d * nblk;
    int tot = 0, pre = 0;
    for (int t0 = 0; t0 < nblk; t0 += 8) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = row[min(t0 + u, nblk - 1)];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int t = t0 + u;
        tot += t < nblk ? v[u] : 0;
        pre += t < blk ? v[u] : 0;
      }
    }
    start[d] = pre;
    gsum[d] = tot;
  }
  __syncthreads();
  block_exclusive_scan(gsum, nb, s_scan);
  for (int d = threadIdx.x; d < nb; d += RT) start[d] += gsum[d];
  __syncthreads();
}

// LDS of the cooperative kernel (ints), phases overlap:
//   decode:  s_off [ROUTE_MAX_BAGS] | hist [max bins]
//   passes:  lds_c (u16 4 x bins) [2 * COOP_BINS] | startI, gsI, startA, gsA [COOP_BINS + 1]
//            each | (t,i2) cells [COOP_CELLS]
constexpr int COOP_LDS_INTS = 2 * COOP_BINS + 4 * (COOP_BINS + 1) + COOP_CELLS;

__global__ __launch_bounds__(RT) void k_route_coop(DevArgs a) {
  extern __shared__ int lds_i[];
  __shared__ int s_scan[RT / 64 + 1];
  __shared__ int s_red[8];
  __shared__ int s_b[2];
  const int tid = threadIdx.x, blk = blockIdx.x, nblk = gridDim.x;
  unsigned short *lds_c = (unsigned short *)lds_i;   // [4][bins] rank counts
  int *startI = lds_i + 2 * COOP_BINS, *gsI = startI + COOP_BINS + 1;
  int *startA = gsI + COOP_BINS + 1, *gsA = startA + COOP_BINS + 1;
  int *cellB = gsA + COOP_BINS + 1;  // [binsB][nblk] (t,i2) counts of the orderA tiles
  int dA[4], dB[4], dI[4];

  // ---- decode; (t,i3) and (t,i1) histograms of the tile; histB cleared for the atomics
  tile_decode(a, blk, lds_i, s_red, s_b, dA, dB, dI);
  check_offsets(a, blk);
  for (int k = blk * RT + tid; k < a.binsB * nblk; k += nblk * RT) a.histB[k] = 0;
  tile_hist(dI, lds_i + ROUTE_MAX_BAGS, a.binsI3, a.histI3, blk);
  __syncthreads();
  tile_hist(dA, lds_i + ROUTE_MAX_BAGS, a.binsA, a.histA, blk);
  if (!grid_sync(a, nblk)) return;

  // ---- orderI3 and orderA: stable places by (t,i3) and (t,i1); the (t,i2) counts of
  //      the orderA tiles gathered per block in LDS, then added to histB
  tile_starts(a.histI3, a.binsI3, blk, startI, gsI, s_scan);
  tile_starts(a.histA, a.binsA, blk, startA, gsA, s_scan);
  if (blk == 0) {
    for (int d = tid; d < a.binsI3; d += RT) a.segI3[d] = gsI[d];
    for (int d = tid; d < a.binsA; d += RT) a.segA[d] = gsA[d];
  }
  for (int i = tid; i < a.binsB * nblk; i += RT) cellB[i] = 0;
  int pI[4], pA[4];
  tile_place(dI, pI, lds_c, a.binsI3, startI, 1, 0);
  __syncthreads();
  tile_place(dA, pA, lds_c, a.binsA, startA, 1, 0);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (pA[r] < 0) continue;
    const int e = tile_pos(blk, r);
    a.posI3_of[e] = pI[r];
    a.orderA[pA[r]] = e;
    atomicAdd(&cellB[dB[r] * nblk + pA[r] / RB], 1);
  }
  __syncthreads();
  for (int i = tid; i < a.binsB * nblk; i += RT)
    if (cellB[i]) atomicAdd(&a.histB[i], cellB[i]);
  if (!grid_sync(a, 2 * nblk)) return;

  // ---- final order: the orderA tiles placed by (t,i2); block 0 builds the work items
  tile_starts(a.histB, a.binsB, blk, startI, gsI, s_scan);
  tile_final(a, blk, lds_c, startI, 1, 0);
  if (blk == 0) {
    if (tid == 0) gsI[a.binsB] = a.nnz;
    __syncthreads();
    build_items(a, gsI, startA, s_scan);
    __syncthreads();
    if (tid == 0) a.hdr[H_PLAN] = (int)a.plan_fp;
  }
}

// ---------------------------------------------------------------- three-kernel path
// k_route_a: decode, (t,i3) and (t,i1) tile histograms; the last block scans both
// [bin][tile] matrices (bin-major: entry (d, t) becomes the first position of bin d's
// elements of tile t) and records the bin starts.
__global__ __launch_bounds__(RT) void k_route_a(DevArgs a) {
  extern __shared__ int lds_i[];  // s_off [ROUTE_MAX_BAGS] | hist [max(binsI3, binsA)]
  __shared__ int s_scan[RT / 64 + 1];
  __shared__ int s_red[8];
  __shared__ int s_b[2];
  const int blk = blockIdx.x, tid = threadIdx.x;
  int dA[4], dB[4], dI[4];
  tile_decode(a, blk, lds_i, s_red, s_b, dA, dB, dI);
  check_offsets(a, blk);
  for (int k = blk * RT + tid; k < a.binsB * a.nblk; k += a.nblk * RT) a.histB[k] = 0;
  tile_hist(dI, lds_i + ROUTE_MAX_BAGS, a.binsI3, a.histI3, blk);
  __syncthreads();
  tile_hist(dA, lds_i + ROUTE_MAX_BAGS, a.binsA, a.histA, blk);
  if (!last_block(&a.ctr[0], a.nblk, a.epoch)) return;
  block_exclusive_scan(a.histI3, a.binsI3 * a.nblk, s_scan);
  block_exclusive_scan(a.histA, a.binsA * a.nblk, s_scan);
  for (int d = tid; d < a.binsI3; d += RT) a.segI3[d] = a.histI3[(size_t)d * a.nblk];
  for (int d = tid; d < a.binsA; d += RT) a.segA[d] = a.histA[(size_t)d * a.nblk];
}

// k_route_b: orderI3 / orderA places of the tile; (t,i2) counts over the orderA tiles;
// the last block scans them and builds the group table and the work items.
__global__ __launch_bounds__(RT) void k_route_b(DevArgs a) {
  extern __shared__ unsigned short lds_c[];  // [4][max(binsI3, binsA)]
  __shared__ int s_scan[RT / 64 + 1];
  const int blk = blockIdx.x;
  int dA[4], dB[4], dI[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int e = tile_pos(blk, r);
    const int4 info = a.einfo[min(e, a.nnz - 1)];
    const bool v = e < a.nnz;
    dA[r] = v ? info.x : -1;
    dB[r] = v ? info.y : -1;
    dI[r] = v ? info.z : -1;
  }
  int pI[4], pA[4];
  tile_place(dI, pI, lds_c, a.binsI3, a.histI3, a.nblk, blk);
  __syncthreads();
  tile_place(dA, pA, lds_c, a.binsA, a.histA, a.nblk, blk);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (pA[r] < 0) continue;
    const int e = tile_pos(blk, r);
    a.posI3_of[e] = pI[r];
    a.orderA[pA[r]] = e;
    atomicAdd(&a.histB[(size_t)dB[r] * a.nblk + pA[r] / RB], 1);
  }
  if (!last_block(&a.ctr[1], a.nblk, a.epoch)) return;
  block_exclusive_scan(a.histB, a.binsB * a.nblk, s_scan);
  for (int d = threadIdx.x; d < a.binsB; d += RT) a.grp_off[d] = a.histB[(size_t)d * a.nblk];
  if (threadIdx.x == 0) a.grp_off[a.binsB] = a.nnz;
  __threadfence_block();
  __syncthreads();
  build_items(a, a.grp_off, a.chunk_pre, s_scan);
}

// k_route_c: the orderA tiles placed by (t,i2) into the final order.
__global__ __launch_bounds__(RT) void k_route_c(DevArgs a) {
  extern __shared__ unsigned short lds_c[];  // [4][binsB]
  tile_final(a, blockIdx.x, lds_c, a.histB, a.nblk, blockIdx.x);
  if (blockIdx.x == 0 && threadIdx.x == 0) a.hdr[H_PLAN] = (int)a.plan_fp;
}

// Forward: out[b] = sum of the weighted cache rows of bag b (zero when it has none);
// the contraction kernel then adds the misses.  One wave per bag.
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
  for (int d = lane; d < a.D; d += 64) {
    float acc = 0.f;
    for (int64_t n = lo; n < hi; ++n) {
      const int s = a.slots[n];
      if (s >= 0 && s < a.cache_size) {
        const float wt = a.psw ? a.psw[n] : 1.f;
        acc += wt * a.crows[(size_t)s * a.D + d];
      }
    }
    a.Y[(size_t)b * a.D + d] = acc;
  }
}

// Backward, cache hits: frag[s] = sum over positions of one run fragment of
// w_n * dY[bag n], where a run is a maximal range of equal (dB, dA, dI3) in the final
// order (one cache slot) and fragments are the pieces of a run inside P-position
// pieces.  One wave per 64 positions; the summation order is the position order.
// (Misses sum their runs inside the backward contraction kernel.)
__global__ __launch_bounds__(RT) void k_runsum(DevArgs a) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int piece = blockIdx.x * (RT / 64) + w;
  const int V = a.hdr[H_VALID];
  const int beg = piece * PIECE;
  if (a.hdr[H_PLAN] != (int)a.plan_fp) {  // the workspace holds another call's plan
    if (piece == 0 && lane == 0) set_status(a.status, DEV_STALE_PLAN);
    return;
  }
  if (beg >= V || beg + PIECE <= a.hdr[H_HIT_BEG]) return;
  const int len = min(PIECE, V - beg);
  const int s = beg + min(lane, len - 1);
  const int kA = a.s_dA[s], kB = a.s_dB[s], kI = a.s_dI3[s], bag = a.s_bag[s];
  const float wt = lane < len ? a.s_w[s] : 0.f;
  const int pA = __shfl_up(kA, 1), pB = __shfl_up(kB, 1), pI = __shfl_up(kI, 1);
  // fragments start at run starts and at every multiple of P (work item boundaries)
  const unsigned long long starts = __ballot(
      lane < len && ((lane == 0) || kA != pA || kB != pB || kI != pI || (s % a.P) == 0));
  for (int d0 = 0; d0 < a.D; d0 += 64) {
    const int d = min(d0 + lane, a.D - 1);
    float v[PIECE];
#pragma unroll
    for (int l = 0; l < PIECE; ++l) {
      const int b = __builtin_amdgcn_readlane(bag, l);
      v[l] = a.dY[(size_t)b * a.D + d];
    }
    float acc = 0.f;
    int cur = beg;
#pragma unroll
    for (int l = 0; l < PIECE; ++l) {
      if (((starts >> l) & 1ull) && l > 0) {
        if (d0 + lane < a.D) a.frag[(size_t)cur * a.D + d] = acc;
        acc = 0.f;
        cur = beg + l;
      }
      if (l < len) acc += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wt), l)) * v[l];
    }
    if (d0 + lane < a.D) a.frag[(size_t)cur * a.D + d] = acc;
  }
}

hipError_t launch_route(const DevArgs &a, hipStream_t s) {
  if (a.nblk == 0) return hipGetLastError();
  if (coop_route_ok(a)) {
    static bool attr_set = false;  // dynamic LDS above 64 KiB is opt-in per kernel
    const size_t lds = (size_t)COOP_LDS_INTS * 4;
    if (!attr_set) {
      (void)hipFuncSetAttribute((const void *)k_route_coop,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      attr_set = true;
    }
    // One block per CU at most (LDS), launched on an otherwise idle stream position:
    // every block is resident at once.  The barriers are bounded waits in any case.
    prof_begin(K_ROUTE_COOP, s);
    hipLaunchKernelGGL(k_route_coop, dim3(a.nblk), dim3(RT), lds, s, a);
    prof_end(K_ROUTE_COOP, s);
    return hipGetLastError();
  }
  const size_t bins_ia = (size_t)(a.binsI3 > a.binsA ? a.binsI3 : a.binsA);
  prof_begin(K_ROUTE_A, s);
  hipLaunchKernelGGL(k_route_a, dim3(a.nblk), dim3(RT), (ROUTE_MAX_BAGS + bins_ia) * 4, s, a);
  prof_end(K_ROUTE_A, s);
  prof_begin(K_ROUTE_B, s);
  hipLaunchKernelGGL(k_route_b, dim3(a.nblk), dim3(RT), bins_ia * 8, s, a);
  prof_end(K_ROUTE_B, s);
  prof_begin(K_ROUTE_C, s);
  hipLaunchKernelGGL(k_route_c, dim3(a.nblk), dim3(RT), (size_t)a.binsB * 8, s, a);
  prof_end(K_ROUTE_C, s);
  return hipGetLastError();
}

hipError_t launch_yinit(const DevArgs &a, hipStream_t s) {
  if (a.NB > 0) {
    prof_begin(K_YINIT, s);
    hipLaunchKernelGGL(k_yinit, dim3((a.NB + RT / 64 - 1) / (RT / 64)), dim3(RT), 0, s, a);
    prof_end(K_YINIT, s);
  }
  return hipGetLastError();
}

hipError_t launch_runsum(const DevArgs &a, hipStream_t s) {
  const int pieces = (a.nnz + PIECE - 1) / PIECE;
  if (pieces > 0 && a.has_cache) {
    prof_begin(K_RUNSUM, s);
    hipLaunchKernelGGL(k_runsum, dim3((pieces + 3) / 4), dim3(RT), 0, s, a);
    prof_end(K_RUNSUM, s);
  }
  return hipGetLastError();
}

}  // namespace ttb
