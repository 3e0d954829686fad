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

// Work items from the group table grp_off[0..binsB] (starts of the (table, i2) bins
// in the final order): a miss group of n elements becomes ceil(n / P) items of
// near-equal size (at most P positions each), numbered group by group.  Also the
// header words of the grouping.  Run by one whole block.
static __device__ void build_items(const DevArgs &a, int *s_scan) {
  const int G = a.T * a.p2, tid = threadIdx.x, nt = blockDim.x;
  for (int g = tid; g <= G; g += nt) {
    const int gb = a.grp_off[g], ge = g < G ? a.grp_off[g + 1] : gb;
    a.chunk_pre[g] = (ge - gb + a.P - 1) / a.P;
  }
  __threadfence_block();
  __syncthreads();
  block_exclusive_scan(a.chunk_pre, G + 1, s_scan);
  for (int g = tid; g < G; g += nt) {
    const int first = a.chunk_pre[g], nc = a.chunk_pre[g + 1] - first;
    const int gb = a.grp_off[g], n = a.grp_off[g + 1] - gb;
    for (int c = 0; c < nc; ++c)
      a.fitem[first + c] = make_int4(g, gb + (int)((int64_t)n * c / nc),
                                     gb + (int)((int64_t)n * (c + 1) / nc), 0);
  }
  if (tid == 0) {
    a.hdr[H_NFWD] = a.chunk_pre[G];
    a.hdr[H_HIT_BEG] = a.grp_off[G];
    a.hdr[H_HIT_END] = a.grp_off[a.binsB - 1];
    a.hdr[H_VALID] = a.grp_off[a.binsB - 1];
  }
}

__global__ __launch_bounds__(RT) void k_route_first(DevArgs a) {
  extern __shared__ int lds_i[];       // [binsI3] histogram, then the block's offsets
  __shared__ int s_scan[RT + 1];
  __shared__ int s_red[8];
  __shared__ int s_b[2];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int blk = blockIdx.x;
  const int base = blk * RB, last = min(base + RB, a.nnz) - 1;
  int *hist = lds_i;
  int *s_off = lds_i + a.binsI3;
  // bags overlapping [base, last]: one 128-ary search per half of the block.  The
  // two halves search in lockstep (same NB, same number of rounds).
  {
    const int half = tid >> 7;
    const int b = half_find_bag(a.off, a.NB, half ? last : base, half, s_red);
    if ((tid & 127) == 0) s_b[half] = b;
  }
  for (int i = tid; i < a.binsI3; i += RT) hist[i] = 0;
  __syncthreads();
  const int b_lo = s_b[0], b_hi = max(s_b[1], s_b[0]);
  const int nbag = b_hi - b_lo + 1;
  const bool in_lds = nbag + 1 <= ROUTE_MAX_BAGS;
  if (in_lds)
    for (int j = tid; j <= nbag; j += RT) {
      int64_t o = a.off[b_lo + j];
      s_off[j] = (int)(o < 0 ? 0 : (o > a.nnz ? a.nnz : o));
    }
  __syncthreads();
  const int dropA = a.binsA - 1, dropB = a.binsB - 1, dropI = a.binsI3 - 1;
  // all loads of the block's elements first (clamped addresses), then the arithmetic
  int64_t iv[4];
  int sv[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int e = min(base + w * 256 + r * 64 + lane, a.nnz - 1);
    iv[r] = a.idx[e];
    sv[r] = (a.has_cache && a.slots) ? a.slots[e] : -1;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int e = base + w * 256 + r * 64 + lane;
    if (e >= a.nnz) continue;
    int b;
    if (in_lds) {
      int lo = 0, hi = nbag;  // largest j with s_off[j] <= e
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_off[mid] <= e) lo = mid; else hi = mid;
      }
      b = b_lo + lo;
    } else {
      b = find_bag(a.off, a.NB, e);
    }
    const int t = b / a.B;
    int dA, dB, dI;
    const int slot = sv[r];
    if (slot >= 0) {
      if (slot >= a.cache_size) {
        set_status(a.status, TT_DEV_BAD_SLOT);
        dA = dropA; dB = dropB; dI = dropI;
      } else {
        dA = a.T * a.p1 + slot % HB;
        dB = a.T * a.p2 + slot / HB;
        dI = dropI;
      }
    } else {
      const int64_t i = iv[r];
      if (i < 0 || i >= a.E) {
        set_status(a.status, TT_DEV_BAD_INDEX);
        dA = dropA; dB = dropB; dI = dropI;
      } else {
        int i1, i2, i3;
        split_index(i, a.p3, (int64_t)a.p2 * a.p3, a.rp23, a.rp3, i1, i2, i3);
        dA = t * a.p1 + i1;
        dB = t * a.p2 + i2;
        dI = t * a.p3 + i3;
      }
    }
    a.einfo[e] = make_int4(dA, dB, dI, b);
    atomicAdd(&hist[dI], 1);
  }
  // offsets must be a CSR over [0, nnz]
  const int gt = blk * RT + tid, gn = a.nblk * RT;
  for (int k = gt; k <= a.NB; k += gn) {
    bool bad = false;
    if (k == 0 && a.off[0] != 0) bad = true;
    if (k == a.NB && a.off[a.NB] != (int64_t)a.nnz) bad = true;
    if (k < a.NB && a.off[k + 1] < a.off[k]) bad = true;
    if (bad) set_status(a.status, TT_DEV_BAD_OFFSETS);
  }
  // the two later digits are histogrammed with atomics: clear them here
  for (int k = gt; k < a.binsA * a.nblk; k += gn) a.histA[k] = 0;
  for (int k = gt; k < a.binsB * a.nblk; k += gn) a.histB[k] = 0;
  __syncthreads();
  for (int i = tid; i < a.binsI3; i += RT) a.histI3[(size_t)i * a.nblk + blk] = hist[i];
  if (last_block(&a.ctr[0], a.nblk, a.epoch)) block_exclusive_scan(a.histI3, a.binsI3 * a.nblk, s_scan);
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

// pass 1: original order -> orderI3 by (t,i3); histogram (t,i1) over destination blocks.
// pass 2: orderI3 -> orderA by (t,i1); histogram (t,i2) over destination blocks, then
//         the group table.
__global__ __launch_bounds__(RT) void k_route_pass(DevArgs a, int pass) {
  extern __shared__ unsigned short lds_c[];
  __shared__ int s_scan[RT + 1];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, blk = blockIdx.x;
  const int *in = pass == 1 ? nullptr : a.orderI3;
  int *out = pass == 1 ? a.orderI3 : a.orderA;
  const int *offs = pass == 1 ? a.histI3 : a.histA;
  int *hnext = pass == 1 ? a.histA : a.histB;
  const int nbins = pass == 1 ? a.binsI3 : a.binsA;
  int e[4], d[4], dn[4], rk[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int s = blk * RB + w * 256 + r * 64 + lane;
    e[r] = -1; d[r] = -1; dn[r] = 0;
    if (s < a.nnz) {
      e[r] = in ? in[s] : s;
      const int4 info = a.einfo[e[r]];
      d[r] = pass == 1 ? info.z : info.x;
      dn[r] = pass == 1 ? info.x : info.y;
    }
  }
  block_rank4(d, rk, lds_c, nbins, nbits_for(nbins), nullptr, a.nblk);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (e[r] < 0) continue;
    const int pos = offs[(size_t)d[r] * a.nblk + blk] + rk[r];
    out[pos] = e[r];
    (pass == 1 ? a.posI3_of : a.posA_of)[e[r]] = pos;
    atomicAdd(&hnext[(size_t)dn[r] * a.nblk + pos / RB], 1);
  }
  if (!last_block(&a.ctr[pass], a.nblk, a.epoch)) return;
  const int binsN = pass == 1 ? a.binsA : a.binsB;
  block_exclusive_scan(hnext, binsN * a.nblk, s_scan);
  if (pass == 2) {
    for (int b = tid; b < a.binsB; b += RT) a.grp_off[b] = a.histB[(size_t)b * a.nblk];
    if (tid == 0) a.grp_off[a.binsB] = a.nnz;
    __threadfence_block();
    __syncthreads();
    build_items(a, s_scan);
  }
}

__global__ __launch_bounds__(RT) void k_route_final(DevArgs a) {
  extern __shared__ unsigned short lds_c[];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, blk = blockIdx.x;
  if (blk == 0 && tid == 0) a.hdr[H_PLAN] = (int)a.plan_fp;
  int e[4], d[4], rk[4], pI[4], pA[4];
  float wv[4];
  int4 info[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int s = min(blk * RB + w * 256 + r * 64 + lane, a.nnz - 1);
    e[r] = a.orderA[s];
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    info[r] = a.einfo[e[r]];
    pI[r] = a.posI3_of[e[r]];
    pA[r] = a.posA_of[e[r]];
    wv[r] = a.psw ? a.psw[e[r]] : 1.f;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int s = blk * RB + w * 256 + r * 64 + lane;
    d[r] = s < a.nnz ? info[r].y : -1;
    if (s >= a.nnz) e[r] = -1;
  }
  block_rank4(d, rk, lds_c, a.binsB, nbits_for(a.binsB), nullptr, a.nblk);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    if (e[r] < 0) continue;
    const int pos = a.histB[(size_t)d[r] * a.nblk + blk] + rk[r];
    a.s_n[pos] = e[r];
    a.s_dA[pos] = info[r].x;
    a.s_dB[pos] = info[r].y;
    a.s_dI3[pos] = info[r].z;
    a.s_bag[pos] = info[r].w;
    a.s_w[pos] = wv[r];
    a.s_posI3[pos] = pI[r];
    a.s_posA[pos] = pA[r];
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

// ---------------------------------------------------------------- one-block route
// Batches of at most SR_MAX elements with at most SR_BINS bins per digit and at most
// SR_OFF - 1 bags are grouped by a single 1024-thread workgroup with everything in
// LDS: the same three stable counting passes (by (t,i3), (t,i1), (t,i2)) and the
// same outputs as the multi-block kernels, without their grid-wide scans.
constexpr int SR_T = 1024, SR_W = SR_T / 64;
constexpr int SR_MAX = 12288;               // elements (u16 positions)
constexpr int SR_K = SR_MAX / SR_T;         // positions per lane and pass
constexpr int SR_BINS = 1024;
constexpr int SR_OFF = 8192;                // offsets kept in LDS (in the count area)
constexpr size_t SR_LDS = (size_t)5 * SR_MAX * 2 + (size_t)SR_W * SR_BINS * 2 + (SR_BINS + 1) * 4;

static bool small_route_ok(const DevArgs &a) {
  return a.nnz <= SR_MAX && a.binsA <= SR_BINS && a.binsB <= SR_BINS && a.binsI3 <= SR_BINS &&
         a.NB + 1 <= SR_OFF;
}

// Loads here are written unconditionally (clamped addresses, selects afterwards): a
// load under a per-lane condition becomes a branch with a wait of its own, which
// serialises the unrolled loops.
__global__ __launch_bounds__(SR_T) void k_route_small(DevArgs a) {
  extern __shared__ int4 lds4[];
  unsigned short *dig = (unsigned short *)lds4;   // [3][SR_MAX] digits by element; the
                                                  // first two later hold posI3 / posA
  unsigned short *ord = dig + 3 * SR_MAX;         // [2][SR_MAX] order ping-pong
  unsigned short *cnt = ord + 2 * SR_MAX;         // [SR_W][SR_BINS] per-wave bin counts
  int *base = (int *)(cnt + SR_W * SR_BINS);      // [SR_BINS + 1]
  int *s_off = (int *)cnt;                        // phase 0: offsets [NB + 1]
  __shared__ int s_scan[SR_W + 1];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int n = a.nnz, NB = a.NB;

  // offsets (clamped copy in LDS) and their validation: a CSR over [0, n]
  for (int b = tid; b <= NB; b += SR_T) {
    const int64_t o = a.off[b];
    const int64_t o1 = a.off[min(b + 1, NB)];
    s_off[b] = (int)(o < 0 ? 0 : (o > n ? n : o));
    if ((b == 0 && o != 0) || (b == NB && o != (int64_t)n) || (b < NB && o1 < o))
      set_status(a.status, TT_DEV_BAD_OFFSETS);
  }
  __syncthreads();
  // elements: split, bag, digits (three parts: register budget)
  bool bad_slot = false, bad_index = false;
  for (int h = 0; h < 3; ++h) {
    constexpr int KH = SR_K / 3;
    int64_t iv[KH];
    int sv[KH], lo[KH];
#pragma unroll
    for (int k = 0; k < KH; ++k) iv[k] = a.idx[min(tid + (h * KH + k) * SR_T, n - 1)];
    if (a.has_cache && a.slots) {
#pragma unroll
      for (int k = 0; k < KH; ++k) sv[k] = a.slots[min(tid + (h * KH + k) * SR_T, n - 1)];
    } else {
#pragma unroll
      for (int k = 0; k < KH; ++k) sv[k] = -1;
    }
    // bag = last b < NB with off[b] <= e: binary lifting, all elements in lockstep
#pragma unroll
    for (int k = 0; k < KH; ++k) lo[k] = 0;
    int top = 1;
    while (top < NB) top <<= 1;
    for (int span = top >> 1; span > 0; span >>= 1) {
      int ov[KH];
#pragma unroll
      for (int k = 0; k < KH; ++k) ov[k] = s_off[min(lo[k] + span, NB - 1)];
#pragma unroll
      for (int k = 0; k < KH; ++k)
        lo[k] = (lo[k] + span < NB && ov[k] <= tid + (h * KH + k) * SR_T) ? lo[k] + span : lo[k];
    }
    const int dropA = a.binsA - 1, dropB = a.binsB - 1, dropI = a.binsI3 - 1;
    const int64_t p23 = (int64_t)a.p2 * a.p3;
#pragma unroll
    for (int k = 0; k < KH; ++k) {
      const int e = tid + (h * KH + k) * SR_T;
      const int b = lo[k], t = a.T == 1 ? 0 : b / a.B;
      const int slot = sv[k];
      const int64_t i = iv[k];
      const bool hit = slot >= 0, slot_ok = hit && slot < a.cache_size;
      const bool idx_ok = !hit && i >= 0 && i < a.E;
      const int64_t ic = idx_ok ? i : 0;
      const int sc = slot_ok ? slot : 0;
      int i1, i2, i3;
      split_index(ic, a.p3, p23, a.rp23, a.rp3, i1, i2, i3);
      int dA = t * a.p1 + i1;
      int dB = t * a.p2 + i2;
      int dI = t * a.p3 + i3;
      if (slot_ok) { dA = a.T * a.p1 + sc % HB; dB = a.T * a.p2 + sc / HB; dI = dropI; }
      if (!slot_ok && !idx_ok) { dA = dropA; dB = dropB; dI = dropI; }
      if (e < n) {
        bad_slot |= hit && !slot_ok;
        bad_index |= !hit && !idx_ok;
        a.einfo[e] = make_int4(dA, dB, dI, b);
        dig[e] = (unsigned short)dI;
        dig[SR_MAX + e] = (unsigned short)dA;
        dig[2 * SR_MAX + e] = (unsigned short)dB;
        ord[e] = (unsigned short)e;
      }
    }
  }
  if (bad_slot) set_status(a.status, TT_DEV_BAD_SLOT);
  if (bad_index) set_status(a.status, TT_DEV_BAD_INDEX);
  __syncthreads();

  // three stable counting passes; wave w ranks the positions [w*per, (w+1)*per) of the
  // current order, 64 at a time, by ballot matching
  const int per = (n + SR_W * 64 - 1) / (SR_W * 64) * 64;
  const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int pass = 0; pass < 3; ++pass) {
    const unsigned short *in = ord + (pass & 1) * SR_MAX;
    unsigned short *out = ord + ((pass + 1) & 1) * SR_MAX;
    const unsigned short *dg = dig + pass * SR_MAX;
    const int nb = pass == 0 ? a.binsI3 : (pass == 1 ? a.binsA : a.binsB);
    const int nbits = nbits_for(nb);
    for (int i = tid; i < SR_W * SR_BINS / 2; i += SR_T) ((unsigned *)cnt)[i] = 0u;
    // xd[k] = element | (digit + 1) << 14 (digit -1: no position); rk[k] = rank in wave
    int xd[SR_K], rk[SR_K];
#pragma unroll
    for (int k = 0; k < SR_K; ++k) xd[k] = in[min(w * per + k * 64 + lane, n - 1)];
#pragma unroll
    for (int k = 0; k < SR_K; ++k) {
      const int p = w * per + k * 64 + lane;
      const bool act = k * 64 < per && p < n;
      const int d = dg[xd[k]];
      xd[k] |= (act ? d + 1 : 0) << 14;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < SR_K; ++k) {
      const int dk = (xd[k] >> 14) - 1;
      const bool act = dk >= 0;
      unsigned long long m = __ballot(act);
      for (int b = 0; b < nbits; ++b) {
        const bool bit = act && ((dk >> b) & 1);
        const unsigned long long bb = __ballot(bit);
        m &= bit ? bb : ~bb;
      }
      const int before = __popcll(m & lt);
      const int ci = w * SR_BINS + (act ? dk : 0);
      const int c0 = cnt[ci];
      rk[k] = c0 + before;
      // every lane of the group has read the count before its leader writes it back
      __builtin_amdgcn_wave_barrier();
      if (act && before == 0) cnt[ci] = (unsigned short)(c0 + __popcll(m));
      __builtin_amdgcn_wave_barrier();
    }
    __syncthreads();
    // per bin: exclusive prefix over the waves, then the bin starts (block scan)
    int tot = 0;
    {
      int cv[SR_W];
      const int bi = min(tid, SR_BINS - 1);
#pragma unroll
      for (int v = 0; v < SR_W; ++v) cv[v] = cnt[v * SR_BINS + bi];
      if (tid < nb) {
#pragma unroll
        for (int v = 0; v < SR_W; ++v) {
          cnt[v * SR_BINS + bi] = (unsigned short)tot;
          tot += cv[v];
        }
      }
    }
    const int incl = wave_incl_scan(tot);
    if (lane == 63) s_scan[w] = incl;
    __syncthreads();
    if (w == 0) {
      const int v = lane < SR_W ? s_scan[lane] : 0;
      const int vi = wave_incl_scan(v);
      if (lane < SR_W) s_scan[lane] = vi - v;
    }
    __syncthreads();
    if (tid < nb) {
      const int start = s_scan[w] + incl - tot;
      base[tid] = start;
      if (pass == 0) a.histI3[(size_t)tid * a.nblk] = start;
      else if (pass == 1) a.histA[(size_t)tid * a.nblk] = start;
      else a.grp_off[tid] = start;
    }
    if (tid == 0 && pass == 2) base[nb] = n;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < SR_K; ++k) {
      const int dk = (xd[k] >> 14) - 1, d = dk >= 0 ? dk : 0;
      rk[k] += base[d] + cnt[w * SR_BINS + d];
    }
#pragma unroll
    for (int k = 0; k < SR_K; ++k) {
      if ((xd[k] >> 14) > 0) {
        const int x = xd[k] & 0x3fff;
        out[rk[k]] = (unsigned short)x;
        if (pass < 2) dig[pass * SR_MAX + x] = (unsigned short)rk[k];  // posI3 / posA
      }
    }
    __syncthreads();
  }

  // final order (ord[1]) -> the per-position arrays (two halves: register budget)
  for (int h = 0; h < 2; ++h) {
    constexpr int KH = SR_K / 2;
    const unsigned short *fin = ord + SR_MAX;
    int ek[KH], pI[KH], pA[KH];
    int4 info[KH];
    float wv[KH];
#pragma unroll
    for (int k = 0; k < KH; ++k) ek[k] = fin[min(tid + (h * KH + k) * SR_T, n - 1)];
#pragma unroll
    for (int k = 0; k < KH; ++k) {
      info[k] = a.einfo[ek[k]];
      pI[k] = dig[ek[k]];
      pA[k] = dig[SR_MAX + ek[k]];
    }
    if (a.psw) {
#pragma unroll
      for (int k = 0; k < KH; ++k) wv[k] = a.psw[ek[k]];
    } else {
#pragma unroll
      for (int k = 0; k < KH; ++k) wv[k] = 1.f;
    }
#pragma unroll
    for (int k = 0; k < KH; ++k) {
      const int s = tid + (h * KH + k) * SR_T;
      if (s < n) {
        a.s_n[s] = ek[k];
        a.s_dA[s] = info[k].x;
        a.s_dB[s] = info[k].y;
        a.s_dI3[s] = info[k].z;
        a.s_bag[s] = info[k].w;
        a.s_w[s] = wv[k];
        a.s_posI3[s] = pI[k];
        a.s_posA[s] = pA[k];
      }
    }
  }
  // work items from the group starts in LDS (base[0..binsB], base[binsB] = n): a
  // group of m elements gives ceil(m / P) items of near-equal size
  {
    const int G = a.T * a.p2;  // G < binsB <= SR_T
    const int gb = base[min(tid, G)], ge = base[min(tid + 1, a.binsB)];
    const int m = tid < G ? ge - gb : 0;
    const int nc = (m + a.P - 1) / a.P;
    const int incl = wave_incl_scan(nc);
    if (lane == 63) s_scan[w] = incl;
    __syncthreads();
    if (w == 0) {
      const int v = lane < SR_W ? s_scan[lane] : 0;
      const int vi = wave_incl_scan(v);
      if (lane < SR_W) s_scan[lane] = vi - v;
      if (lane == SR_W - 1) s_scan[SR_W] = vi;
    }
    __syncthreads();
    const int first = s_scan[w] + incl - nc;
    if (tid <= G) a.chunk_pre[tid] = first;
    for (int c = 0; c < nc; ++c)
      a.fitem[first + c] = make_int4(tid, gb + (int)((int64_t)m * c / nc),
                                     gb + (int)((int64_t)m * (c + 1) / nc), 0);
    if (tid == 0) {
      a.grp_off[a.binsB] = n;
      a.hdr[H_NFWD] = s_scan[SR_W];
      a.hdr[H_HIT_BEG] = base[G];
      a.hdr[H_HIT_END] = base[a.binsB - 1];
      a.hdr[H_VALID] = base[a.binsB - 1];
      a.hdr[H_PLAN] = (int)a.plan_fp;
    }
  }
}

hipError_t launch_route(const DevArgs &a, hipStream_t s) {
  if (a.nblk == 0) return hipGetLastError();
  if (small_route_ok(a)) {
    static bool attr_set = false;  // dynamic LDS above 64 KiB is opt-in per kernel
    if (!attr_set) {
      (void)hipFuncSetAttribute((const void *)k_route_small,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)SR_LDS);
      attr_set = true;
    }
    prof_begin(K_ROUTE_SMALL, s);
    hipLaunchKernelGGL(k_route_small, dim3(1), dim3(SR_T), SR_LDS, s, a);
    prof_end(K_ROUTE_SMALL, s);
    return hipGetLastError();
  }
  prof_begin(K_ROUTE_FIRST, s);
  hipLaunchKernelGGL(k_route_first, dim3(a.nblk), dim3(RT),
                     (size_t)(a.binsI3 + ROUTE_MAX_BAGS) * 4, s, a);
  prof_end(K_ROUTE_FIRST, s);
  prof_begin(K_ROUTE_PASS1, s);
  hipLaunchKernelGGL(k_route_pass, dim3(a.nblk), dim3(RT), (size_t)a.binsI3 * 8, s, a, 1);
  prof_end(K_ROUTE_PASS1, s);
  prof_begin(K_ROUTE_PASS2, s);
  hipLaunchKernelGGL(k_route_pass, dim3(a.nblk), dim3(RT), (size_t)a.binsA * 8, s, a, 2);
  prof_end(K_ROUTE_PASS2, s);
  prof_begin(K_ROUTE_FINAL, s);
  hipLaunchKernelGGL(k_route_final, dim3(a.nblk), dim3(RT), (size_t)a.binsB * 8, s, a);
  prof_end(K_ROUTE_FINAL, s);
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
