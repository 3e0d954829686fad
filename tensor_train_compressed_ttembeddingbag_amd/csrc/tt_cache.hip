// tt_cache.hip -- the software cache of decompressed rows.
//
// "FBTT-Embedding" README, "Software Cache": the most frequently queried rows are
// kept uncompressed so that a hit skips the TT arithmetic; access frequencies are
// counted in an open-addressing hash table (hashtbl_size entries) during lookups,
// and the cache content changes only when populate is called, which picks rows by
// frequency and initialises each from the TT cores.  Here: exact top-K by (count
// descending, index ascending), slot = rank in that order; a second open-addressing
// table maps index -> slot for lookups.
#include "tt_device.h"

namespace ttb {

constexpr long long EMPTY_KEY = -1;

// splitmix64 finalizer (Steele, Lea, Flood 2014) as the hash of an index.
static __device__ __forceinline__ unsigned long long mix64(unsigned long long x) {
  x ^= x >> 30;
  x *= 0xbf58476d1ce4e5b9ull;
  x ^= x >> 27;
  x *= 0x94d049bb133111ebull;
  x ^= x >> 31;
  return x;
}

// find or insert key in the count table; returns the entry or -1 if the table is full
static __device__ long long count_slot(long long *keys, long long H, long long key) {
  long long h = (long long)(mix64((unsigned long long)key) % (unsigned long long)H);
  for (long long probe = 0; probe < H; ++probe) {
    const long long k = __atomic_load_n(&keys[h], __ATOMIC_RELAXED);
    if (k == key) return h;
    if (k == EMPTY_KEY) {
      const long long prev = (long long)atomicCAS((unsigned long long *)&keys[h],
                                                  (unsigned long long)EMPTY_KEY,
                                                  (unsigned long long)key);
      if (prev == EMPTY_KEY || prev == key) return h;
    }
    h = (h + 1 == H) ? 0 : h + 1;
  }
  return -1;
}

// slot of key in the index -> slot map (M a power of two), or -1.  h: the key's home
// entry; k, sl: that entry's key and slot, loaded by the caller together with its other
// loads (later probes load an entry's key and slot together).
static __device__ int map_find(const long long *mkeys, const int *mslot, long long M,
                               long long key, long long h, long long k, int sl) {
  for (long long probe = 0; probe < M; ++probe) {
    if (probe > 0) {
      k = mkeys[h];
      sl = mslot[h];
    }
    if (k == key) return sl;
    if (k == EMPTY_KEY) return -1;
    h = (h + 1) & (M - 1);
  }
  return -1;
}

// slot lookup + frequency count.  Duplicated keys inside a wave are merged first
// (match on 16 hash bits with ballots, confirmed against the group leader's key), then the
// block's waves in a small LDS table (one entry per distinct key of the block), so a hot
// index costs one atomic on the count table per 1024 positions instead of one per
// occurrence (same-address atomics serialise in the L2).  The counts are integer sums:
// the same whatever the merging.
constexpr int LK_T = 1024;   // positions per lookup block (16 waves)
constexpr int LK_HT = 2048;  // its merge table: a power of two, at least twice LK_T
__global__ __launch_bounds__(LK_T) void k_cache_lookup(const int64_t *idx, int nnz, int64_t E,
                                                        long long *hkeys, int *hcnt, long long H,
                                                        const long long *mkeys, const int *mslot,
                                                        long long M, int32_t *slot_out,
                                                        int count_freq, int32_t *status) {
  __shared__ long long s_key[LK_HT];
  __shared__ int s_add[LK_HT];
  const int n = blockIdx.x * LK_T + threadIdx.x;
  const int lane = threadIdx.x & 63;
  const bool in = n < nnz;
  const long long key = in ? (long long)idx[n] : -1;
  const bool valid = in && key >= 0 && key < E;
  // the slot map's first probe goes out now and is looked at after the counting
  const unsigned long long hk = mix64((unsigned long long)key);
  const long long hm = (long long)(hk & (unsigned long long)(M - 1));
  long long km = EMPTY_KEY;
  int sm = -1;
  if (valid) {
    km = mkeys[hm];
    sm = mslot[hm];
  }
  if (count_freq) {  // (uniform)
    for (int i = threadIdx.x; i < LK_HT; i += LK_T) {
      s_key[i] = EMPTY_KEY;
      s_add[i] = 0;
    }
    const unsigned h16 = (unsigned)(hk >> 48);
    unsigned long long m = __ballot(valid);
    for (int b = 0; b < 16; ++b) {
      const bool bit = valid && ((h16 >> b) & 1u);
      const unsigned long long bb = __ballot(bit);
      m &= bit ? bb : ~bb;
    }
    const int leader = valid ? (__ffsll((long long)m) - 1) : lane;
    const long long lk = __shfl(key, leader);
    const unsigned long long same = m & __ballot(valid && key == lk);
    int add = 0;
    if (valid) {
      if (lane == leader) add = __popcll(same);
      else if (key != lk) add = 1;
    }
    __syncthreads();  // the table is clear
    if (add > 0) {    // at most LK_T keys in LK_HT entries: a free entry is always found
      unsigned h = (unsigned)hk & (LK_HT - 1);
      for (;;) {
        const long long prev = (long long)atomicCAS((unsigned long long *)&s_key[h],
                                                    (unsigned long long)EMPTY_KEY,
                                                    (unsigned long long)key);
        if (prev == EMPTY_KEY || prev == key) {
          atomicAdd(&s_add[h], add);
          break;
        }
        h = (h + 1) & (LK_HT - 1);
      }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < LK_HT; i += LK_T) {
      const long long k2 = s_key[i];
      if (k2 == EMPTY_KEY) continue;
      const long long e = count_slot(hkeys, H, k2);
      if (e < 0) { if (status) atomicOr(status, TT_DEV_HASH_FULL); }
      else atomicAdd(&hcnt[e], s_add[i]);
    }
  }
  if (in) slot_out[n] = valid ? map_find(mkeys, mslot, M, key, hm, km, sm) : -1;
}

// populate, step 1: compact the used count entries into sortable 64-bit keys
// ((cmax - count) << kbits) | index, so ascending order = count desc, index asc.
__global__ __launch_bounds__(256) void k_cache_compact(const long long *hkeys, const int *hcnt,
                                                        long long H, int kbits,
                                                        unsigned long long *out, int *n_out) {
  const long long h = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (h >= H) return;
  const long long k = hkeys[h];
  if (k == EMPTY_KEY) return;
  const unsigned long long cmax = (kbits >= 64) ? 0ull : ((~0ull) >> kbits);
  unsigned long long c = (unsigned long long)(unsigned)hcnt[h];
  if (c > cmax) c = cmax;
  const int pos = atomicAdd(n_out, 1);
  out[pos] = ((cmax - c) << kbits) | (unsigned long long)k;
}

// LSD radix sort of 64-bit keys, 8 bits per pass: block histograms ...
__global__ __launch_bounds__(RT) void k_sort_hist(const unsigned long long *keys, int n,
                                                   int shift, int *hist, int nblk) {
  __shared__ int h[256];
  const int tid = threadIdx.x;
  h[tid] = 0;
  __syncthreads();
  for (int r = 0; r < 4; ++r) {
    const int i = blockIdx.x * RB + r * 256 + tid;
    if (i < n) atomicAdd(&h[(int)((keys[i] >> shift) & 255ull)], 1);
  }
  __syncthreads();
  hist[tid * nblk + blockIdx.x] = h[tid];
}

// ... one-block exclusive scan ...
constexpr int SCAN_T = 1024;  // the histogram scan: one block, a short run per thread
__global__ __launch_bounds__(SCAN_T) void k_sort_scan(int *hist, int len) {
  __shared__ int s[SCAN_T / 64 + 1];
  block_exclusive_scan(hist, len, s);
}

// ... and a stable scatter (ranks inside the block keep the input order).
__global__ __launch_bounds__(RT) void k_sort_scatter(const unsigned long long *in, int n,
                                                      int shift, const int *off, int nblk,
                                                      unsigned long long *out) {
  __shared__ unsigned short cnt[4 * 256];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int d[4], rk[4];
  unsigned long long k[4];
  for (int r = 0; r < 4; ++r) {
    const int i = blockIdx.x * RB + w * 256 + r * 64 + lane;
    k[r] = 0;
    d[r] = -1;
    if (i < n) { k[r] = in[i]; d[r] = (int)((k[r] >> shift) & 255ull); }
  }
  block_rank<RT, 4>(d, rk, cnt, 256, 8);
  for (int r = 0; r < 4; ++r)
    if (d[r] >= 0) out[off[d[r] * nblk + blockIdx.x] + rk[r]] = k[r];
}

// populate, step 3: slots 0..n_filled-1 take the sorted indices; fill the map.
__global__ __launch_bounds__(256) void k_cache_assign(const unsigned long long *sorted, int nf,
                                                       int kbits, int64_t cache_size,
                                                       int64_t *cached, long long *mkeys,
                                                       int *mslot, long long M) {
  const long long s = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= cache_size) return;
  if (s >= nf) { cached[s] = -1; return; }
  const unsigned long long mask = (kbits >= 64) ? ~0ull : ((1ull << kbits) - 1ull);
  const long long key = (long long)(sorted[s] & mask);
  cached[s] = key;
  long long h = (long long)(mix64((unsigned long long)key) & (unsigned long long)(M - 1));
  for (long long probe = 0; probe < M; ++probe) {
    const long long prev = (long long)atomicCAS((unsigned long long *)&mkeys[h],
                                                (unsigned long long)EMPTY_KEY,
                                                (unsigned long long)key);
    if (prev == EMPTY_KEY) { mslot[h] = (int)s; return; }
    h = (h + 1) & (M - 1);
  }
}

// ---------------------------------------------------------------- set-associative LFU
// "Software Cache" names a 32-way set-associative LFU cache.  slot = set * 32 + way; the
// set of index i is (splitmix64(i) >> 32) mod nsets.  A populate keeps in every set the
// 32 counted indices of the set with the highest counts (ties: smaller index); indices
// that stay keep their way (and their row); newcomers take the freed ways in ascending
// order, in (count desc, index asc) order, and only their rows are rebuilt.
constexpr int LFU_WAYS = 32;

__device__ __forceinline__ long long lfu_set(long long key, long long nsets) {
  return (long long)((mix64((unsigned long long)key) >> 32) % (unsigned long long)nsets);
}

// key[r] = (set << 32) | r for the r-th entry of the priority order (sorting these keys
// orders the entries by set, then priority)
__global__ __launch_bounds__(256) void k_lfu_setkey(const unsigned long long *prio, int n,
                                                     int kbits, long long nsets,
                                                     unsigned long long *out) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= n) return;
  const unsigned long long mask = (kbits >= 64) ? ~0ull : ((1ull << kbits) - 1ull);
  const long long key = (long long)(prio[r] & mask);
  out[r] = ((unsigned long long)lfu_set(key, nsets) << 32) | (unsigned)r;
}

// first position of every set in the set-major order (-1: no candidate)
__global__ __launch_bounds__(256) void k_lfu_first(const unsigned long long *sk, int n,
                                                    int *set_first) {
  const int p = blockIdx.x * 256 + threadIdx.x;
  if (p >= n) return;
  const unsigned s = (unsigned)(sk[p] >> 32);
  if (p == 0 || (unsigned)(sk[p - 1] >> 32) != s) set_first[s] = p;
}

// one wave per set: lanes 0..31 are the ways (old occupants) and the new members
__global__ __launch_bounds__(256) void k_lfu_assign(const unsigned long long *prio,
                                                     const unsigned long long *sk, int n,
                                                     int kbits, const int *set_first,
                                                     long long nsets, int64_t *cached,
                                                     int *fresh_slot, int64_t *fresh_idx,
                                                     int *counters) {
  const int lane = threadIdx.x & 63;
  const long long s = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (s >= nsets) return;
  const unsigned long long mask = (kbits >= 64) ? ~0ull : ((1ull << kbits) - 1ull);
  const int first = set_first[s];
  long long m = -1;  // member `lane` of the set (priority order), or -1
  if (first >= 0 && lane < LFU_WAYS && first + lane < n) {
    const unsigned long long k = sk[first + lane];
    if ((long long)(k >> 32) == s) m = (long long)(prio[(unsigned)k] & mask);
  }
  const long long o = lane < LFU_WAYS ? (long long)cached[s * LFU_WAYS + lane] : -1;
  bool kept = false, is_new = m >= 0;
  for (int j = 0; j < LFU_WAYS; ++j) {
    const long long mj = __shfl(m, j), oj = __shfl(o, j);
    kept = kept || (o >= 0 && o == mj);
    is_new = is_new && m != oj;
  }
  const unsigned long long keep_m = __ballot(lane < LFU_WAYS && kept);
  const unsigned long long new_m = __ballot(lane < LFU_WAYS && is_new);
  const unsigned long long free_m = ~keep_m & 0xffffffffull;
  // way `lane`: kept, or the r-th free way takes the r-th newcomer, or empty
  long long v = kept ? o : -1;
  bool fresh = false;
  if (lane < LFU_WAYS && !kept) {
    const int r = __popcll(free_m & ((1ull << lane) - 1ull));
    unsigned long long nm = new_m;
    for (int t = 0; t < r && nm; ++t) nm &= nm - 1ull;  // drop the first r newcomers
    if (nm) {
      const int j = __ffsll((long long)nm) - 1;
      v = j;  // lane of the newcomer; its index is read below
      fresh = true;
    }
  }
  const long long mv = __shfl(m, fresh ? (int)v : 0);
  if (fresh) v = mv;
  if (lane < LFU_WAYS) {
    const long long slot = s * LFU_WAYS + lane;
    cached[slot] = v;
    if (fresh) {
      const int f = atomicAdd(&counters[0], 1);
      fresh_slot[f] = (int)slot;
      fresh_idx[f] = v;
    }
  }
  const unsigned long long valid = __ballot(lane < LFU_WAYS && v >= 0);
  if (lane == 0 && valid) atomicAdd(&counters[1], __popcll(valid));
}

// the index -> slot map from the slot table
__global__ __launch_bounds__(256) void k_map_insert(const int64_t *cached, long long K,
                                                     long long *mkeys, int *mslot, long long M) {
  const long long s = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= K) return;
  const long long key = (long long)cached[s];
  if (key < 0) return;
  long long h = (long long)(mix64((unsigned long long)key) & (unsigned long long)(M - 1));
  for (long long probe = 0; probe < M; ++probe) {
    const long long prev = (long long)atomicCAS((unsigned long long *)&mkeys[h],
                                                (unsigned long long)EMPTY_KEY,
                                                (unsigned long long)key);
    if (prev == EMPTY_KEY) { mslot[h] = (int)s; return; }
    h = (h + 1) & (M - 1);
  }
}

// rows[slot[f]] = tmp[f]
__global__ __launch_bounds__(256) void k_scatter_rows(const float *tmp, const int *slot, int nf,
                                                       int D, float *rows) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long long)nf * D) return;
  const long long f = i / D, d = i - f * D;
  rows[(size_t)slot[f] * D + d] = tmp[i];
}

__global__ void k_iota64(int64_t *a, long long n) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) a[i] = i;
}

// ---------------------------------------------------------------- host side
hipError_t cache_lookup_launch(const int64_t *idx, int nnz, int64_t E, long long *hkeys,
                               int *hcnt, long long H, const long long *mkeys, const int *mslot,
                               long long M, int32_t *slot_out, int count_freq, int32_t *status,
                               hipStream_t s) {
  if (nnz > 0) {
    tt_launch(K_CACHE_LOOKUP, k_cache_lookup, dim3((nnz + LK_T - 1) / LK_T), dim3(LK_T), 0, s,
              idx, nnz, E,
                       hkeys, hcnt, H, mkeys, mslot, M, slot_out, count_freq, status);
  }
  return hipGetLastError();
}

hipError_t cache_compact_launch(const long long *hkeys, const int *hcnt, long long H, int kbits,
                                unsigned long long *out, int *n_out, hipStream_t s) {
  hipLaunchKernelGGL(k_cache_compact, dim3((unsigned)((H + 255) / 256)), dim3(256), 0, s, hkeys,
                     hcnt, H, kbits, out, n_out);
  return hipGetLastError();
}

// stable sort of n keys by their bits [lo, hi) (8 per pass); returns the buffer that holds
// the result (a after an even number of passes, else b)
unsigned long long *radix_sort64_bits(unsigned long long *a, unsigned long long *b, int n,
                                      int *hist, int lo, int hi, hipStream_t s) {
  const int nblk = (n + RB - 1) / RB;
  if (nblk == 0) return a;
  for (int shift = lo; shift < hi; shift += 8) {
    hipLaunchKernelGGL(k_sort_hist, dim3(nblk), dim3(RT), 0, s, a, n, shift, hist, nblk);
    hipLaunchKernelGGL(k_sort_scan, dim3(1), dim3(SCAN_T), 0, s, hist, 256 * nblk);
    hipLaunchKernelGGL(k_sort_scatter, dim3(nblk), dim3(RT), 0, s, a, n, shift, hist, nblk, b);
    unsigned long long *t = a; a = b; b = t;
  }
  return a;
}

// sorts n keys in place (a is input and output, b scratch), 64 bits
hipError_t radix_sort64(unsigned long long *a, unsigned long long *b, int n, int *hist,
                        hipStream_t s) {
  const int nblk = (n + RB - 1) / RB;
  if (nblk == 0) return hipSuccess;
  for (int shift = 0; shift < 64; shift += 8) {
    hipLaunchKernelGGL(k_sort_hist, dim3(nblk), dim3(RT), 0, s, a, n, shift, hist, nblk);
    hipLaunchKernelGGL(k_sort_scan, dim3(1), dim3(SCAN_T), 0, s, hist, 256 * nblk);
    hipLaunchKernelGGL(k_sort_scatter, dim3(nblk), dim3(RT), 0, s, a, n, shift, hist, nblk, b);
    unsigned long long *t = a; a = b; b = t;
  }
  return hipGetLastError();  // 8 passes: the result is back in the first buffer
}

hipError_t cache_assign_launch(const unsigned long long *sorted, int nf, int kbits,
                               int64_t cache_size, int64_t *cached, long long *mkeys, int *mslot,
                               long long M, hipStream_t s) {
  if (cache_size > 0)
    hipLaunchKernelGGL(k_cache_assign, dim3((unsigned)((cache_size + 255) / 256)), dim3(256), 0,
                       s, sorted, nf, kbits, cache_size, cached, mkeys, mslot, M);
  return hipGetLastError();
}

hipError_t lfu_setkey_launch(const unsigned long long *prio, int n, int kbits, long long nsets,
                             unsigned long long *out, hipStream_t s) {
  if (n > 0) hipLaunchKernelGGL(k_lfu_setkey, dim3((n + 255) / 256), dim3(256), 0, s, prio, n, kbits,
                                nsets, out);
  return hipGetLastError();
}

hipError_t lfu_first_launch(const unsigned long long *sk, int n, int *set_first, hipStream_t s) {
  if (n > 0) hipLaunchKernelGGL(k_lfu_first, dim3((n + 255) / 256), dim3(256), 0, s, sk, n, set_first);
  return hipGetLastError();
}

hipError_t lfu_assign_launch(const unsigned long long *prio, const unsigned long long *sk, int n,
                             int kbits, const int *set_first, long long nsets, int64_t *cached,
                             int *fresh_slot, int64_t *fresh_idx, int *counters, hipStream_t s) {
  hipLaunchKernelGGL(k_lfu_assign, dim3((unsigned)((nsets + 3) / 4)), dim3(256), 0, s, prio, sk, n,
                     kbits, set_first, nsets, cached, fresh_slot, fresh_idx, counters);
  return hipGetLastError();
}

hipError_t map_insert_launch(const int64_t *cached, long long K, long long *mkeys, int *mslot,
                             long long M, hipStream_t s) {
  if (K > 0) hipLaunchKernelGGL(k_map_insert, dim3((unsigned)((K + 255) / 256)), dim3(256), 0, s,
                                cached, K, mkeys, mslot, M);
  return hipGetLastError();
}

hipError_t scatter_rows_launch(const float *tmp, const int *slot, int nf, int D, float *rows,
                               hipStream_t s) {
  const long long n = (long long)nf * D;
  if (n > 0) hipLaunchKernelGGL(k_scatter_rows, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                                tmp, slot, nf, D, rows);
  return hipGetLastError();
}

hipError_t iota64_launch(int64_t *a, long long n, hipStream_t s) {
  if (n > 0) hipLaunchKernelGGL(k_iota64, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a, n);
  return hipGetLastError();
}

}  // namespace ttb
