// tt_device.h -- device helpers shared by the routing and cache kernels.
#pragma once
#include "tt_internal.h"

namespace ttb {

// Row split i -> (i1, i2, i3) of a valid row i (0 <= i < p1*p2*p3 < 2^40), with
// i = (i1*p2 + i2)*p3 + i3.  The quotients come from double reciprocals (rp23 = 1/(p2*p3),
// rp3 = 1/p3): their products are within a few ulps of the exact quotients, so the
// truncation is exact or one too small, which one remainder check corrects.
static __device__ __forceinline__ void split_index(int64_t i, int p3, int64_t p23, double rp23,
                                                   double rp3, int &i1, int &i2, int &i3) {
  int q1 = (int)((double)i * rp23);
  int64_t r = i - (int64_t)q1 * p23;
  if (r >= p23) { ++q1; r -= p23; } else if (r < 0) { --q1; r += p23; }
  const int rr = (int)r;
  int q2 = (int)((double)rr * rp3);
  int r3 = rr - q2 * p3;
  if (r3 >= p3) { ++q2; r3 -= p3; } else if (r3 < 0) { --q2; r3 += p3; }
  i1 = q1; i2 = q2; i3 = r3;
}

// inclusive scan across the 64 lanes of a wave
static __device__ __forceinline__ int wave_incl_scan(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

// exclusive scan of arr[0..len) in global memory by one whole block (blockDim a
// multiple of 64, at most 1024).  Each thread owns a contiguous run of the array;
// the per-thread sums are scanned with wave shuffles.  s_tmp: >= 17 ints of LDS.
static __device__ void block_exclusive_scan(int *arr, int len, int *s_tmp) {
  const int nt = blockDim.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int per = (len + nt - 1) / nt;
  const int beg = min(tid * per, len), end = min(beg + per, len);
  int sum = 0;
  for (int i0 = beg; i0 < end; i0 += 8) {  // eight loads in flight
    int v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = arr[min(i0 + u, len - 1)];
#pragma unroll
    for (int u = 0; u < 8; ++u) sum += (i0 + u < end) ? v[u] : 0;
  }
  const int incl = wave_incl_scan(sum);
  if (lane == 63) s_tmp[w] = incl;
  __syncthreads();
  if (w == 0) {
    const int nw = nt >> 6;
    const int v = lane < nw ? s_tmp[lane] : 0;
    const int vi = wave_incl_scan(v);
    if (lane < nw) s_tmp[lane] = vi - v;
  }
  __syncthreads();
  int run = s_tmp[w] + incl - sum;
  for (int i0 = beg; i0 < end; i0 += 8) {
    int v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = arr[min(i0 + u, len - 1)];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (i0 + u < end) {
        arr[i0 + u] = run;
        run += v[u];
      }
  }
  __threadfence_block();
  __syncthreads();
}

// Items and pairs of one work item, worked out by one wave (lane = element offset in
// the work item, v = a real element).  Pairs are the runs of equal dA (the grouping
// order sorts by (t,i2,i1)); items are the distinct i3 inside a pair, numbered in the
// order of their first element (the "leader").  item_pos is the lane's slot in the
// item-major element list (items in order, an item's elements in position order).
struct WaveItems {
  unsigned long long mi, mp;  // leaders, pair starts
  bool item_st, pair_st;
  int e_it;        // item of this lane
  int it, pr;      // item index (leaders), pair index (pair starts)
  int pair_of;     // pair of this lane
  int it_beg;      // leaders: first slot of the item in the item-major list
  int item_pos;    // this lane's slot in the item-major list
  int pair_items;  // pair starts: number of items of the pair
};

static __device__ WaveItems wave_items(bool v, int dA, int i3, int nbits3) {
  const int lane = threadIdx.x & 63;
  const unsigned long long self = 1ull << lane;
  const unsigned long long lt = self - 1ull;
  WaveItems r;
  const int pdA = __shfl_up(dA, 1);
  r.pair_st = v && (lane == 0 || dA != pdA);
  r.mp = __ballot(r.pair_st);
  const unsigned long long vm = __ballot(v);
  const unsigned long long upto = r.mp & (lt | self), above = r.mp & ~(lt | self);
  const int ps = upto ? 63 - __clzll(upto) : 0;
  const int pe = above ? __ffsll((long long)above) - 1 : 64;
  const unsigned long long pmask = (pe >= 64 ? ~0ull : ((1ull << pe) - 1ull)) & ~((1ull << ps) - 1ull);
  unsigned long long m = vm & pmask;  // lanes of the same pair with the same i3
  for (int b = 0; b < nbits3; ++b) {
    const bool bit = (i3 >> b) & 1;
    const unsigned long long bb = __ballot(v && bit);
    m &= bit ? bb : ~bb;
  }
  const int lead = (v && m) ? __ffsll((long long)m) - 1 : lane;
  r.item_st = v && lead == lane;
  r.mi = __ballot(r.item_st);
  r.e_it = __popcll(r.mi & ((1ull << lead) - 1ull));
  r.it = __popcll(r.mi & lt);
  r.pr = __popcll(r.mp & lt);
  r.pair_of = __popcll(upto) - 1;
  const int sz = r.item_st ? __popcll(m) : 0;
  r.it_beg = wave_incl_scan(sz) - sz;
  r.item_pos = __shfl(r.it_beg, lead) + __popcll(m & lt);
  r.pair_items = __popcll(r.mi & pmask);
  return r;
}

// Stable ranks of the block's elements by digit (d < 0: no element).  Thread tid of
// wave w holds EPT elements, element r at position w*64*EPT + r*64 + lane of the block's
// order; rank = number of earlier elements with the same digit.  cnt: NW*nbins u16 of LDS
// (per-wave counts).  Whole block of NT threads.
template <int NT, int EPT>
static __device__ void block_rank(const int *d, int *rank, unsigned short *cnt, int nbins,
                                  int nbits) {
  constexpr int NW = NT / 64;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int i = threadIdx.x; i < NW * nbins; i += NT) cnt[i] = 0;
  __syncthreads();
  int rw[EPT];
  const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int r = 0; r < EPT; ++r) {
    const bool act = d[r] >= 0;
    unsigned long long m = __ballot(act);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = act && ((d[r] >> b) & 1);
      const unsigned long long bb = __ballot(bit);
      m &= bit ? bb : ~bb;
    }
    const int before = __popcll(m & lt);
    const int ci = w * nbins + (act ? d[r] : 0);
    const int base = cnt[ci];
    rw[r] = base + before;
    // every lane of the group has read `base` before the leader writes it back
    __builtin_amdgcn_wave_barrier();
    if (act && before == 0) cnt[ci] = (unsigned short)(base + __popcll(m));
    __builtin_amdgcn_wave_barrier();
  }
  __syncthreads();
  for (int bin = threadIdx.x; bin < nbins; bin += NT) {
    int c[NW];
#pragma unroll
    for (int v = 0; v < NW; ++v) c[v] = cnt[v * nbins + bin];
    int run = 0;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      cnt[v * nbins + bin] = (unsigned short)run;
      run += c[v];
    }
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < EPT; ++r) rank[r] = d[r] >= 0 ? (int)cnt[w * nbins + d[r]] + rw[r] : 0;
}

static __device__ __forceinline__ int nbits_for(int nbins) {
  return nbins <= 1 ? 1 : 32 - __clz(nbins - 1);
}

// bag of position n: the last b with off[b] <= n (off clamped to [0, nnz]).
static __device__ __forceinline__ int find_bag(const int64_t *off, int NB, int n) {
  int lo = 0, hi = NB;  // answer in [0, NB-1]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (off[mid] <= (int64_t)n) lo = mid; else hi = mid;
  }
  return lo;
}

// last-block detection: returns true in every thread of the block that finishes last.
// The counter word holds (epoch << 32 | count); a word left by another call (or
// garbage) carries another epoch and counts as zero, so it never needs clearing.
static __device__ bool last_block(unsigned long long *ctr, int nblocks, unsigned epoch) {
  __shared__ int s_last;
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long old = *(volatile unsigned long long *)ctr, nw;
    while (true) {
      nw = ((unsigned)(old >> 32) == epoch) ? old + 1ull
                                              : (((unsigned long long)epoch << 32) | 1ull);
      const unsigned long long prev = atomicCAS(ctr, old, nw);
      if (prev == old) break;
      old = prev;
    }
    s_last = ((nw & 0xffffffffull) == (unsigned long long)nblocks);
  }
  __syncthreads();
  if (s_last) __threadfence();
  return s_last != 0;
}

// One wave's part of the cache-hit run sums: the w_n * dY[bag n] of piece `piece` (64
// positions of the final order) summed per fragment (run starts and the piece start) in
// position order.  Runs of the same slot are cache hits of one row; misses sum theirs in
// the backward contraction itself.
static __device__ __forceinline__ void runsum_piece(const DevArgs &a, int piece, int lane) {
  const int V = a.hdr[H_VALID];
  const int beg = piece * PIECE;
  if (beg >= V || beg + PIECE <= a.hdr[H_HIT_BEG]) return;
  const int len = min(PIECE, V - beg);
  const int s = beg + min(lane, len - 1);
  const SPos sp = load_spos(a.srec, s);
  const int kA = sp.dA, kB = sp.dB, kI = sp.dI3, bag = sp.bag;
  const float wt = lane < len ? sp.w : 0.f;
  const int pA = __shfl_up(kA, 1), pB = __shfl_up(kB, 1), pI = __shfl_up(kI, 1);
  // fragments start at run starts and at the piece start
  const unsigned long long starts =
      __ballot(lane < len && ((lane == 0) || kA != pA || kB != pB || kI != pI));
  constexpr int HALF = PIECE / 2;  // dY rows in flight (two halves keep registers low)
  for (int d0 = 0; d0 < a.D; d0 += 64) {
    const int d = min(d0 + lane, a.D - 1);
    float acc = 0.f;
    int cur = beg;
#pragma unroll
    for (int h = 0; h < PIECE; h += HALF) {
      float v[HALF];
#pragma unroll
      for (int l = 0; l < HALF; ++l) {
        const int b = __builtin_amdgcn_readlane(bag, h + l);
        v[l] = a.dY[(size_t)b * a.D + d];
      }
#pragma unroll
      for (int l = 0; l < HALF; ++l) {
        const int ll = h + l;
        if (((starts >> ll) & 1ull) && ll > 0) {
          if (d0 + lane < a.D) a.frag[(size_t)cur * a.D + d] = acc;
          acc = 0.f;
          cur = beg + ll;
        }
        if (ll < len)
          acc += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wt), ll)) * v[l];
      }
    }
    if (d0 + lane < a.D) a.frag[(size_t)cur * a.D + d] = acc;
  }
}

}  // namespace ttb
