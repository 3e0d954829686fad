// tt_dedup.hip -- backward over distinct indices.  The loss L = sum_b <dY[b], Y[b]> is
// linear in the rows W[idx], so (README intro: the backward is EmbeddingBag's)
//   dL/dW[u] = sum_{n : idx_n = u} w_n dY[bag n]          (w_n times 1/len with mean pooling)
// and the backward of a batch equals the backward of a virtual batch with one element
// per distinct (table, index) u, weight 1, in a bag of its own whose grad_out row is that
// sum.  When indices repeat (Zipf-skewed batches) the virtual batch is much smaller, and
// a hot index costs one element instead of thousands.
//
// Plan (no host synchronisation): keys (table*E + index, position) sorted stably by the
// key's index bits, runs of equal keys, the virtual indices and offsets (table-major,
// nnz bags per table -- a bound on every table's count of distinct indices -- of which
// the first count are filled), and the grouping of both the real batch (for the forward)
// and the virtual one, whose element count the grouping kernels read from the device.  Backward: the grad_out sums of the runs in two fixed-order passes (32-element
// chunks of the sorted order, then each run's chunk pieces in order), then the planned
// three-core backward on the virtual batch.
#include <algorithm>
#include <cmath>
#include <cstring>

#include "tt_device.h"

namespace ttb {
namespace {

constexpr int DD_T = 256;   // threads of the small kernels
constexpr int DD_CH = 32;   // sorted elements per chunk of the grad_out sums

__device__ __forceinline__ bool dd_valid(unsigned long long key, int pbits,
                                         unsigned long long inv) {
  return (key >> pbits) != inv;
}

// key = ((t * E + idx) << pbits) | n for a valid index, (T * E) << pbits | n otherwise;
// bag of every position
__global__ __launch_bounds__(DD_T) void k_dd_keys(const int64_t *__restrict__ idx,
                                                  const int64_t *__restrict__ off, int nnz,
                                                  int NB, int B, long long E, int pbits,
                                                  unsigned long long inv,
                                                  unsigned long long *__restrict__ keys,
                                                  int *__restrict__ bagv) {
  const int n = blockIdx.x * DD_T + threadIdx.x;
  if (n >= nnz) return;
  int lo = 0, hi = NB - 1;  // the last bag b with off[b] <= n
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= n) lo = mid; else hi = mid - 1;
  }
  const long long i = idx[n];
  const long long t = lo / B;
  const unsigned long long hiv = (i >= 0 && i < E) ? (unsigned long long)(t * E + i) : inv;
  keys[n] = (hiv << pbits) | (unsigned long long)n;
  bagv[n] = lo;
}

// run starts per block of RB sorted elements (cnt[nblk] cleared for the scan's total)
__global__ __launch_bounds__(RT) void k_dd_count(const unsigned long long *__restrict__ keys,
                                                 int nnz, int pbits, unsigned long long inv,
                                                 int *__restrict__ cnt, int nblk) {
  __shared__ int s;
  if (threadIdx.x == 0) s = 0;
  __syncthreads();
  int c = 0;
  for (int r = 0; r < RB / RT; ++r) {
    const int m = blockIdx.x * RB + r * RT + threadIdx.x;
    if (m < nnz) {
      const unsigned long long k = keys[m];
      const bool st = dd_valid(k, pbits, inv) && (m == 0 || (keys[m - 1] >> pbits) != (k >> pbits));
      c += st;
    }
  }
  atomicAdd(&s, c);
  __syncthreads();
  if (threadIdx.x == 0) {
    cnt[blockIdx.x] = s;
    if (blockIdx.x == 0) cnt[nblk] = 0;
  }
}

__global__ __launch_bounds__(RT) void k_dd_scan(int *cnt, int len) {
  __shared__ int tmp[RT + 1];
  block_exclusive_scan(cnt, len, tmp);
}

// runs: index, table, first and end sorted position; Rt[t] = first run of table t
__global__ __launch_bounds__(RT) void k_dd_emit(const unsigned long long *__restrict__ keys,
                                                int nnz, int pbits, unsigned long long inv,
                                                long long E, int T, const int *__restrict__ cnt,
                                                int nblk, int64_t *__restrict__ vidx,
                                                int *__restrict__ rtab, int *__restrict__ rstart,
                                                int *__restrict__ rend, int64_t *__restrict__ Rt) {
  __shared__ int s_w[RB / 64];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int base = blockIdx.x * RB;
  // element m = base + 4 * tid + r: the block's flags in element order
  bool st[4], vl[4];
  unsigned long long k[4];
  int c = 0;
  for (int r = 0; r < 4; ++r) {
    const int m = base + 4 * tid + r;
    k[r] = m < nnz ? keys[m] : (inv << pbits);
    vl[r] = m < nnz && dd_valid(k[r], pbits, inv);
    st[r] = vl[r] && (m == 0 || (keys[m - 1] >> pbits) != (k[r] >> pbits));
    c += st[r];
  }
  const int incl = wave_incl_scan(c);
  if (lane == 63) s_w[w] = incl;
  __syncthreads();
  int before = cnt[blockIdx.x];
  for (int i = 0; i < w; ++i) before += s_w[i];
  int run = before + incl - c - 1;  // run of the element before this thread's first
  const int U = cnt[nblk];
  for (int r = 0; r < 4; ++r) {
    const int m = base + 4 * tid + r;
    if (!vl[r]) continue;
    if (st[r]) {
      ++run;
      const unsigned long long h = k[r] >> pbits;
      const long long t = (long long)(h / (unsigned long long)E);
      vidx[run] = (int64_t)(h - (unsigned long long)t * (unsigned long long)E);
      rtab[run] = (int)t;
      rstart[run] = m;
      const long long tp = m > 0 ? (long long)((keys[m - 1] >> pbits) / (unsigned long long)E) : -1;
      for (long long x = tp + 1; x <= t; ++x) Rt[x] = run;  // tables tp+1 .. t start here
    }
    const bool last = m + 1 >= nnz || (keys[m + 1] >> pbits) != (k[r] >> pbits);
    if (last) {
      rend[run] = m + 1;
      if (m + 1 >= nnz || !dd_valid(keys[m + 1], pbits, inv)) {  // the last valid element
        const long long t = (long long)((k[r] >> pbits) / (unsigned long long)E);
        for (long long x = t + 1; x <= T; ++x) Rt[x] = U;
      }
    }
  }
}

__global__ __launch_bounds__(DD_T) void k_dd_fill64(int64_t *__restrict__ x, long long n,
                                                    int64_t v) {
  const long long i = blockIdx.x * (long long)DD_T + threadIdx.x;
  if (i < n) x[i] = v;
}

int fill64(int64_t *x, long long n, int64_t v, hipStream_t s) {
  if (n > 0)
    hipLaunchKernelGGL(k_dd_fill64, dim3((unsigned)((n + DD_T - 1) / DD_T)), dim3(DD_T), 0, s, x, n,
                       v);
  return hipGetLastError() == hipSuccess ? TT_OK : TT_EHIP;
}

// virtual offsets: bag t * Bp + j holds run Rt[t] + j when j < (runs of table t)
__global__ __launch_bounds__(DD_T) void k_dd_voff(const int64_t *__restrict__ Rt, int T, int Bp,
                                                  int64_t *__restrict__ voff) {
  const long long b = blockIdx.x * (long long)DD_T + threadIdx.x;
  const long long nb = (long long)T * Bp;
  if (b > nb) return;
  if (b == nb) { voff[b] = Rt[T]; return; }
  const int t = (int)(b / Bp), j = (int)(b % Bp);
  const long long cntt = Rt[t + 1] - Rt[t];
  voff[b] = Rt[t] + (j < cntt ? j : cntt);
}

// The plan both passes read (sorted keys, bags, runs) belongs to the batch of the call
// only if the real batch's plan header holds this call's fingerprint.  Otherwise they
// touch nothing, report DEV_STALE_PLAN and mark the virtual batch's plan invalid, so
// that the planned backward that follows leaves the cores alone as well.
__device__ __forceinline__ bool dd_plan_ok(const int *rhdr, unsigned rfp, int *vhdr,
                                           unsigned vfp, int32_t *status) {
  if (rhdr[H_PLAN] == (int)rfp) return true;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    set_status(status, DEV_STALE_PLAN);
    vhdr[H_PLAN] = (int)~vfp;
  }
  return false;
}

// pass 1: per 32-element chunk of the sorted order, the sum of w_n dY[bag n] of each run's
// piece in the chunk, stored at the piece's first sorted position
__global__ __launch_bounds__(DD_T) void k_dd_frag(const unsigned long long *__restrict__ keys,
                                                  int nnz, int pbits, unsigned long long inv,
                                                  const int *__restrict__ bagv, int NB,
                                                  const int64_t *__restrict__ off,
                                                  const float *__restrict__ psw, int mean,
                                                  const float *__restrict__ dY, int D,
                                                  float *__restrict__ frag, const int *rhdr,
                                                  unsigned rfp, int *vhdr, unsigned vfp,
                                                  int32_t *status) {
  __shared__ float s_w[DD_CH];
  __shared__ int s_b[DD_CH], s_cut[DD_CH];
  if (!dd_plan_ok(rhdr, rfp, vhdr, vfp, status)) return;
  const int m0 = blockIdx.x * DD_CH;
  const unsigned long long pmask = (1ull << pbits) - 1ull;
  if (threadIdx.x < DD_CH) {
    const int m = m0 + threadIdx.x;
    float wv = 0.f;
    int bv = 0, cut = 1;
    if (m < nnz) {
      const unsigned long long k = keys[m];
      if (dd_valid(k, pbits, inv)) {
        const int n = min((int)(k & pmask), nnz - 1);
        bv = min(max(bagv[n], 0), NB - 1);
        wv = psw ? psw[n] : 1.f;
        if (mean) {
          const long long len = off[bv + 1] - off[bv];
          wv *= 1.f / (float)(len > 0 ? len : 1);
        }
        // the piece ends here when the chunk or the run ends
        cut = (threadIdx.x == DD_CH - 1 || m + 1 >= nnz ||
               (keys[m + 1] >> pbits) != (k >> pbits)) ? 1 : 0;
      } else {
        cut = -1;  // invalid elements (sorted last) take no part
      }
    } else {
      cut = -1;
    }
    s_w[threadIdx.x] = wv;
    s_b[threadIdx.x] = bv;
    s_cut[threadIdx.x] = cut;
  }
  __syncthreads();
  for (int d = threadIdx.x; d < D; d += DD_T) {
    float acc = 0.f;
    int first = m0;
    for (int e = 0; e < DD_CH; ++e) {
      const int cut = s_cut[e];
      if (cut < 0) break;
      acc = fmaf(s_w[e], dY[(size_t)s_b[e] * D + d], acc);
      if (cut) {
        frag[(size_t)first * D + d] = acc;
        acc = 0.f;
        first = m0 + e + 1;
      }
    }
  }
}

// pass 2: each run's pieces in sorted order -> the grad_out row of its virtual bag.  A
// run's pieces start at its first position and then at every chunk boundary inside it.
// NG = DD_T / D groups of D threads (one group when D >= DD_T) take contiguous ranges of
// the pieces, eight loads in flight, and the group sums are added in group order.
__global__ __launch_bounds__(DD_T) void k_dd_gu(const int *__restrict__ rstart,
                                                const int *__restrict__ rend,
                                                const int *__restrict__ rtab,
                                                const int64_t *__restrict__ Rt, int T, int Bp,
                                                int D, const float *__restrict__ frag,
                                                float *__restrict__ Gu, const int *rhdr,
                                                unsigned rfp, int *vhdr, unsigned vfp,
                                                int32_t *status) {
  __shared__ float s_part[DD_T];
  if (!dd_plan_ok(rhdr, rfp, vhdr, vfp, status)) return;
  const int u = blockIdx.x;
  if (u >= Rt[T]) return;  // (the launch covers every position; the runs are Rt[T])
  const int a = rstart[u], z = rend[u], t = rtab[u];
  const long long vb = (long long)t * Bp + (u - Rt[t]);
  const int c0 = a / DD_CH, nf = (z - 1) / DD_CH - c0 + 1;
  const int NG = D < DD_T ? DD_T / D : 1;
  const int g = D < DD_T ? (int)threadIdx.x / D : 0;
  const int per = (nf + NG - 1) / NG;
  const int k0 = min(nf, g * per), k1 = min(nf, k0 + per);
  for (int d0 = 0; d0 < D; d0 += DD_T) {  // more than one pass only when D > DD_T
    const int d = D < DD_T ? (int)threadIdx.x - g * D : d0 + (int)threadIdx.x;
    const bool act = g < NG && d < D;
    float acc = 0.f;
    if (act) {
      int k = k0;
      for (; k + 8 <= k1; k += 8) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int f = (k + j == 0) ? a : (c0 + k + j) * DD_CH;
          v[j] = frag[(size_t)f * D + d];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) acc += v[j];
      }
      for (; k < k1; ++k) acc += frag[(size_t)(k == 0 ? a : (c0 + k) * DD_CH) * D + d];
    }
    if (NG > 1) {
      if (act) s_part[threadIdx.x] = acc;
      __syncthreads();
      if (g == 0 && act) {
        float tot = 0.f;
        for (int x = 0; x < NG; ++x) tot += s_part[x * D + d];
        Gu[vb * D + d] = tot;
      }
    } else if (act) {
      Gu[vb * D + d] = acc;
    }
  }
}

int bits_for(unsigned long long v) {  // bits to hold 0 .. v
  int b = 0;
  while (b < 64 && (v >> b) != 0ull) ++b;
  return b > 0 ? b : 1;
}

size_t al(size_t x) { return (x + 255) & ~(size_t)255; }

struct DDPlan {
  tt_desc vdesc;  // the virtual batch: sum pooling
  int T, nnz, nblk, pbits, kbits, D;
  unsigned long long inv;
  size_t ws1, ws2;
  size_t o_ws2, o_k0, o_k1, o_hist, o_cnt, o_bag, o_vidx, o_rtab, o_rs, o_re, o_Rt, o_voff,
      o_frag, o_gu, total;
};

int make_ddplan(const tt_desc *desc, int64_t nnz, int64_t num_bags, DDPlan *P) {
  if (!desc || nnz < 0 || nnz >= (1LL << 30) || num_bags < 1) return TT_EINVAL;
  memset(P, 0, sizeof(*P));
  const size_t w1 = tt_bag_workspace_size(desc, nnz, num_bags, 0);
  if (w1 == 0) return TT_ESHAPE;
  P->T = desc->num_tables;
  P->nnz = (int)nnz;
  P->D = desc->q[0] * desc->q[1] * desc->q[2];
  P->vdesc = *desc;
  P->vdesc.pooling = TT_POOL_SUM;
  const int64_t vb = nnz > 0 ? nnz : 1;  // bags per table of the virtual batch: at most nnz
  if ((int64_t)P->T * vb >= (1LL << 30)) return TT_ESHAPE;
  const size_t w2 = tt_bag_workspace_size(&P->vdesc, nnz, vb, 0);
  if (w2 == 0) return TT_ESHAPE;
  P->pbits = bits_for(nnz > 1 ? (unsigned long long)(nnz - 1) : 1ull);
  const unsigned long long TE = (unsigned long long)P->T * (unsigned long long)desc->num_embeddings;
  P->inv = TE;
  P->kbits = bits_for(TE);
  if (P->pbits + P->kbits > 64) return TT_ESHAPE;
  P->nblk = (int)((nnz + RB - 1) / RB);
  const size_t n = (size_t)(nnz > 0 ? nnz : 1);
  size_t cur = al(w1);
  P->ws1 = w1;
  P->ws2 = w2;
  P->o_ws2 = cur; cur = al(cur + w2);
  P->o_k0 = cur; cur = al(cur + n * 8);
  P->o_k1 = cur; cur = al(cur + n * 8);
  P->o_hist = cur; cur = al(cur + (size_t)256 * (P->nblk + 1) * 4);
  P->o_cnt = cur; cur = al(cur + (size_t)(P->nblk + 2) * 4);
  P->o_bag = cur; cur = al(cur + n * 4);
  P->o_vidx = cur; cur = al(cur + n * 8);
  P->o_rtab = cur; cur = al(cur + n * 4);
  P->o_rs = cur; cur = al(cur + n * 4);
  P->o_re = cur; cur = al(cur + n * 4);
  P->o_Rt = cur; cur = al(cur + (size_t)(P->T + 1) * 8);
  P->o_voff = cur; cur = al(cur + ((size_t)P->T * n + 1) * 8);
  P->o_frag = cur; cur = al(cur + n * P->D * 4);
  P->o_gu = cur; cur = al(cur + (size_t)P->T * n * P->D * 4);
  P->total = cur;
  return TT_OK;
}

template <class X>
X *at(void *ws, size_t off) { return (X *)((char *)ws + off); }

// the virtual batch's sorted keys sit in k0 or k1 (by the parity of the sort's passes)
unsigned long long *sorted_keys(const DDPlan &P, void *ws) {
  const int passes = (P.kbits + 7) / 8;
  return (passes & 1) ? at<unsigned long long>(ws, P.o_k1) : at<unsigned long long>(ws, P.o_k0);
}

int check_ws_dd(const DDPlan &P, void *ws, size_t ws_bytes) {
  if (!ws || ((uintptr_t)ws & 255)) return TT_EINVAL;
  return ws_bytes < P.total ? TT_EWORKSPACE : TT_OK;
}

}  // namespace
}  // namespace ttb

using namespace ttb;

extern "C" {

size_t tt_bag_workspace_size_dedup(const tt_desc *desc, int64_t nnz, int64_t num_bags) {
  DDPlan P;
  if (make_ddplan(desc, nnz, num_bags, &P) != TT_OK) return 0;
  return P.total;
}

int tt_bag_plan_dedup(const tt_desc *desc, const int64_t *indices, int64_t nnz,
                      const int64_t *offsets, int64_t num_bags, const float *per_sample_weights,
                      void *ws, size_t ws_bytes, int32_t *dev_status, int64_t info[2],
                      void *stream) {
  if (!info || !offsets || (nnz > 0 && !indices)) return TT_EINVAL;
  DDPlan P;
  int rc = make_ddplan(desc, nnz, num_bags, &P);
  if (rc != TT_OK) return rc;
  if ((rc = check_ws_dd(P, ws, ws_bytes)) != TT_OK) return rc;
  hipStream_t s = (hipStream_t)stream;
  // the real batch's grouping (for the forward)
  rc = tt_bag_plan(desc, indices, nnz, offsets, num_bags, per_sample_weights, nullptr, ws, P.ws1,
                   dev_status, stream);
  if (rc != TT_OK) return rc;
  info[0] = info[1] = 0;
  if (nnz == 0) return TT_OK;
  const int NB = (int)((int64_t)P.T * num_bags);
  unsigned long long *k0 = at<unsigned long long>(ws, P.o_k0), *k1 = at<unsigned long long>(ws, P.o_k1);
  int *cnt = at<int>(ws, P.o_cnt);
  int64_t *Rt = at<int64_t>(ws, P.o_Rt);
  hipLaunchKernelGGL(k_dd_keys, dim3((P.nnz + DD_T - 1) / DD_T), dim3(DD_T), 0, s, indices, offsets,
                     P.nnz, NB, (int)num_bags, (long long)desc->num_embeddings, P.pbits, P.inv, k0,
                     at<int>(ws, P.o_bag));
  unsigned long long *sk = radix_sort64_bits(k0, k1, P.nnz, at<int>(ws, P.o_hist), P.pbits,
                                             P.pbits + P.kbits, s);
  if (sk != sorted_keys(P, ws)) return TT_EHIP;  // (cannot happen: same pass count)
  hipLaunchKernelGGL(k_dd_count, dim3(P.nblk), dim3(RT), 0, s, sk, P.nnz, P.pbits, P.inv, cnt,
                     P.nblk);
  hipLaunchKernelGGL(k_dd_scan, dim3(1), dim3(RT), 0, s, cnt, P.nblk + 1);
  // tables without valid elements keep Rt = 0 unless a later table sets them
  if (fill64(Rt, P.T + 1, 0, s) != TT_OK) return TT_EHIP;
  hipLaunchKernelGGL(k_dd_emit, dim3(P.nblk), dim3(RT), 0, s, sk, P.nnz, P.pbits, P.inv,
                     (long long)desc->num_embeddings, P.T, cnt, P.nblk, at<int64_t>(ws, P.o_vidx),
                     at<int>(ws, P.o_rtab), at<int>(ws, P.o_rs), at<int>(ws, P.o_re), Rt);
  if (hipGetLastError() != hipSuccess) return TT_EHIP;
  // the virtual batch: one element per distinct index, Rt[T] of them (a device word: the
  // host never reads it), sized here by its bounds -- nnz elements, vb bags per table
  const int64_t vb = nnz;
  const long long nvb = (long long)P.T * vb + 1;
  int64_t *voff = at<int64_t>(ws, P.o_voff);
  hipLaunchKernelGGL(k_dd_voff, dim3((unsigned)((nvb + DD_T - 1) / DD_T)), dim3(DD_T), 0, s, Rt,
                     P.T, (int)vb, voff);
  if (hipGetLastError() != hipSuccess) return TT_EHIP;
  info[0] = nnz;
  info[1] = vb;
  // the virtual batch's grouping, its element count read on the device
  return plan_devcount(&P.vdesc, at<int64_t>(ws, P.o_vidx), nnz, voff, vb, Rt + P.T,
                       at<char>(ws, P.o_ws2), P.ws2, dev_status, stream);
}

static int backward_dedup(const tt_desc *desc, float *const cores[3], const int64_t *indices,
                          int64_t nnz, const int64_t *offsets, int64_t num_bags,
                          const float *psw, const float *grad_out, float lr,
                          float *const grad_cores[3], const int64_t info[2], void *ws,
                          size_t ws_bytes, int32_t *dev_status, void *stream) {
  if (!info || !grad_out || !offsets || (nnz > 0 && !indices)) return TT_EINVAL;
  DDPlan P;
  int rc = make_ddplan(desc, nnz, num_bags, &P);
  if (rc != TT_OK) return rc;
  if ((rc = check_ws_dd(P, ws, ws_bytes)) != TT_OK) return rc;
  // info: the virtual batch's bounds from tt_bag_plan_dedup (nnz elements and nnz bags
  // per table; 0 and 0 for an empty batch)
  if (info[0] != nnz || info[1] != nnz) return TT_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  float *Gu = at<float>(ws, P.o_gu);
  const int64_t U = nnz, vb = nnz;
  int64_t *vidx = at<int64_t>(ws, P.o_vidx), *voff = at<int64_t>(ws, P.o_voff);
  if (nnz > 0) {
    // the plans the passes check: the real batch's (this call's inputs) and the virtual one's
    int *rhdr = nullptr, *vhdr = nullptr;
    unsigned rfp = 0, vfp = 0;
    if ((rc = plan_identity(desc, nnz, num_bags, indices, offsets, psw, ws, &rhdr, &rfp)) ||
        (rc = plan_identity(&P.vdesc, U, vb, vidx, voff, nullptr, at<char>(ws, P.o_ws2), &vhdr,
                            &vfp)))
      return rc;
    unsigned long long *sk = sorted_keys(P, ws);
    float *frag = at<float>(ws, P.o_frag);
    const int NB = (int)((int64_t)P.T * num_bags);
    tt_launch(K_DD_FRAG, k_dd_frag, dim3((P.nnz + DD_CH - 1) / DD_CH), dim3(DD_T), 0, s,
              (const unsigned long long *)sk, P.nnz, P.pbits, P.inv,
              (const int *)at<int>(ws, P.o_bag), NB, offsets, psw,
              desc->pooling == TT_POOL_MEAN ? 1 : 0, grad_out, P.D, frag, (const int *)rhdr,
              rfp, vhdr, vfp, dev_status);
    tt_launch(K_DD_GU, k_dd_gu, dim3((unsigned)U), dim3(DD_T), 0, s,
              (const int *)at<int>(ws, P.o_rs), (const int *)at<int>(ws, P.o_re),
              (const int *)at<int>(ws, P.o_rtab), (const int64_t *)at<int64_t>(ws, P.o_Rt),
              P.T, (int)vb, P.D, (const float *)frag, Gu, (const int *)rhdr, rfp, vhdr, vfp,
              dev_status);
    if (hipGetLastError() != hipSuccess) return TT_EHIP;
  }
  if (nnz == 0) {  // an empty batch: zero gradients, no update
    if (!grad_cores) return TT_OK;
    if (fill64(voff, P.T + 1, 0, s) != TT_OK) return TT_EHIP;  // T tables of one empty bag
    return tt_bag_backward_grad(&P.vdesc, cores, vidx, 0, voff, 1, nullptr, nullptr, Gu,
                                grad_cores, nullptr, at<char>(ws, P.o_ws2), P.ws2, dev_status,
                                stream);
  }
  // the virtual batch's planned backward (its element count on the device: a batch with
  // no valid index has no work item, the update leaves the cores alone and the gradient
  // mode writes zeros)
  if (grad_cores)
    return tt_bag_backward_grad_planned(&P.vdesc, cores, vidx, U, voff, vb, nullptr, nullptr, Gu,
                                        grad_cores, nullptr, at<char>(ws, P.o_ws2), P.ws2,
                                        dev_status, stream);
  return tt_bag_backward_sgd_planned(&P.vdesc, cores, vidx, U, voff, vb, nullptr, nullptr, Gu, lr,
                                     at<char>(ws, P.o_ws2), P.ws2, dev_status, stream);
}

int tt_bag_backward_sgd_dedup(const tt_desc *desc, float *const cores[3], const int64_t *indices,
                              int64_t nnz, const int64_t *offsets, int64_t num_bags,
                              const float *per_sample_weights, const float *grad_out, float lr,
                              const int64_t info[2], void *ws, size_t ws_bytes,
                              int32_t *dev_status, void *stream) {
  if (!std::isfinite(lr)) return TT_EINVAL;
  return backward_dedup(desc, cores, indices, nnz, offsets, num_bags, per_sample_weights,
                        grad_out, lr, nullptr, info, ws, ws_bytes, dev_status, stream);
}

int tt_bag_dedup_counts(const tt_desc *desc, int64_t nnz, int64_t num_bags, const void *ws,
                        size_t ws_bytes, int64_t *counts, void *stream) {
  if (!counts) return TT_EINVAL;
  DDPlan P;
  int rc = make_ddplan(desc, nnz, num_bags, &P);
  if (rc != TT_OK) return rc;
  if ((rc = check_ws_dd(P, (void *)ws, ws_bytes)) != TT_OK) return rc;
  if (nnz == 0) {
    for (int t = 0; t <= P.T; ++t) counts[t] = 0;
    return TT_OK;
  }
  hipStream_t s = (hipStream_t)stream;
  const int64_t *Rt = at<int64_t>((void *)ws, P.o_Rt);
  if (hipMemcpyAsync(counts, Rt, (size_t)(P.T + 1) * 8, hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return TT_EHIP;
  return TT_OK;
}

int tt_bag_backward_grad_dedup(const tt_desc *desc, const float *const cores[3],
                               const int64_t *indices, int64_t nnz, const int64_t *offsets,
                               int64_t num_bags, const float *per_sample_weights,
                               const float *grad_out, float *const grad_cores[3],
                               const int64_t info[2], void *ws, size_t ws_bytes,
                               int32_t *dev_status, void *stream) {
  if (!grad_cores) return TT_EINVAL;
  return backward_dedup(desc, (float *const *)cores, indices, nnz, offsets, num_bags,
                        per_sample_weights, grad_out, 0.f, grad_cores, info, ws, ws_bytes,
                        dev_status, stream);
}

}  // extern "C"
