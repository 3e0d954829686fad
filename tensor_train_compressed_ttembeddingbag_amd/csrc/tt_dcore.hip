// tt_dcore.hip -- tables of d cores ("FBTT-Embedding" README, "Parameters": the shape
// lists may have any length d).  The row of a d-core table is the product of its d slice
// matrices, and a product of consecutive slices is again a slice of one core: the
// Kronecker-structured core M = G_lo (x) ... (x) G_{hi-1} with slice index
// (i_lo, ..., i_{hi-1}) and column index (j_lo, ..., j_{hi-1}), both row-major.  The
// d cores are cut into three groups of consecutive cores, each group is multiplied out
// into one core (a group of one core is used as it is), and the three-core kernels run
// on those.  Their gradients with respect to the multiplied-out cores are split back
// onto the d cores by the product rule, one core at a time:
//   M_k = M_{k-1} (x) G_k:  M_k[iX*p_k + i_k][a][jX*q_k + j_k][b]
//                             = sum_s M_{k-1}[iX][a][jX][s] G_k[i_k][s][j_k][b]
//   dG_k[i_k][s][j_k][b]  = sum_{iX, a, jX} M_{k-1}[iX][a][jX][s] dM_k[...][a][...][b]
//   dM_{k-1}[iX][a][jX][s] = sum_{i_k, j_k, b} dM_k[...][a][...][b] G_k[i_k][s][j_k][b]
// The multiplied-out cores and their gradients are dense (every slice): the grouping is
// chosen to keep them small (groups at the ends of the chain have an outer rank of 1).
// All sums run in a fixed order, so results are reproducible bit for bit.
#include <cstring>

#include "tt_internal.h"

namespace ttb {
namespace {

constexpr int GBLK = 256;

__global__ __launch_bounds__(GBLK) void k_dmerge(const float *__restrict__ X,
                                                 const float *__restrict__ G,
                                                 float *__restrict__ Y, long long n, int PX,
                                                 int pk, int Rl, int QX, int qk, int Rm, int Rr) {
  const long long PY = (long long)PX * pk, QY = (long long)QX * qk;
  for (long long e = blockIdx.x * (long long)GBLK + threadIdx.x; e < n;
       e += (long long)gridDim.x * GBLK) {
    long long v = e;
    const int r = (int)(v % Rr); v /= Rr;
    const int jY = (int)(v % QY); v /= QY;
    const int a = (int)(v % Rl); v /= Rl;
    const long long iY = v % PY;
    const long long t = v / PY;
    const long long iX = iY / pk, ik = iY % pk;
    const int jX = jY / qk, jk = jY % qk;
    const float *x = X + (((t * PX + iX) * Rl + a) * QX + jX) * (long long)Rm;
    const float *g = G + ((t * pk + ik) * Rm * (long long)qk + jk) * Rr + r;
    float acc = 0.f;
    for (int s = 0; s < Rm; ++s) acc = fmaf(x[s], g[(long long)s * qk * Rr], acc);
    Y[e] = acc;
  }
}

// dG_k from M_{k-1} (X) and dM_k (dY)
__global__ __launch_bounds__(GBLK) void k_dsplit_g(const float *__restrict__ X,
                                                   const float *__restrict__ dY,
                                                   float *__restrict__ dG, long long n, int PX,
                                                   int pk, int Rl, int QX, int qk, int Rm,
                                                   int Rr) {
  const long long PY = (long long)PX * pk, QY = (long long)QX * qk;
  for (long long e = blockIdx.x * (long long)GBLK + threadIdx.x; e < n;
       e += (long long)gridDim.x * GBLK) {
    long long v = e;
    const int r = (int)(v % Rr); v /= Rr;
    const int jk = (int)(v % qk); v /= qk;
    const int s = (int)(v % Rm); v /= Rm;
    const long long ik = v % pk;
    const long long t = v / pk;
    float acc = 0.f;
    for (long long iX = 0; iX < PX; ++iX)
      for (int a = 0; a < Rl; ++a) {
        const float *x = X + (((t * PX + iX) * Rl + a) * QX) * (long long)Rm + s;
        const float *y = dY + (((t * PY + iX * pk + ik) * Rl + a) * QY + jk) * Rr + r;
        for (int jX = 0; jX < QX; ++jX)
          acc = fmaf(x[(long long)jX * Rm], y[(long long)jX * qk * Rr], acc);
      }
    dG[e] = acc;
  }
}

// dM_{k-1} from dM_k (dY) and G_k
__global__ __launch_bounds__(GBLK) void k_dsplit_x(const float *__restrict__ dY,
                                                   const float *__restrict__ G,
                                                   float *__restrict__ dX, long long n, int PX,
                                                   int pk, int Rl, int QX, int qk, int Rm,
                                                   int Rr) {
  const long long PY = (long long)PX * pk, QY = (long long)QX * qk;
  for (long long e = blockIdx.x * (long long)GBLK + threadIdx.x; e < n;
       e += (long long)gridDim.x * GBLK) {
    long long v = e;
    const int s = (int)(v % Rm); v /= Rm;
    const int jX = (int)(v % QX); v /= QX;
    const int a = (int)(v % Rl); v /= Rl;
    const long long iX = v % PX;
    const long long t = v / PX;
    float acc = 0.f;
    for (int ik = 0; ik < pk; ++ik)
      for (int jk = 0; jk < qk; ++jk) {
        const float *y = dY + (((t * PY + iX * pk + ik) * Rl + a) * QY + (long long)jX * qk + jk) * Rr;
        const float *g = G + (((t * pk + ik) * Rm + s) * (long long)qk + jk) * Rr;
        for (int r = 0; r < Rr; ++r) acc = fmaf(y[r], g[r], acc);
      }
    dX[e] = acc;
  }
}

// The same two sums with one wavefront per output when they are long: lane l adds the
// terms l, l + 64, ... in order, then the 64 partials are added by a fixed butterfly,
// so the result does not depend on timing.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__global__ __launch_bounds__(GBLK) void k_dsplit_g_wave(const float *__restrict__ X,
                                                        const float *__restrict__ dY,
                                                        float *__restrict__ dG, long long n,
                                                        int PX, int pk, int Rl, int QX, int qk,
                                                        int Rm, int Rr) {
  const long long PY = (long long)PX * pk, QY = (long long)QX * qk;
  const long long L = (long long)PX * Rl * QX;  // terms (iX, a, jX), jX fastest
  const int lane = threadIdx.x & 63;
  for (long long e = (blockIdx.x * (long long)GBLK + threadIdx.x) >> 6; e < n;
       e += ((long long)gridDim.x * GBLK) >> 6) {
    long long v = e;
    const int r = (int)(v % Rr); v /= Rr;
    const int jk = (int)(v % qk); v /= qk;
    const int s = (int)(v % Rm); v /= Rm;
    const long long ik = v % pk;
    const long long t = v / pk;
    float acc = 0.f;
    for (long long m = lane; m < L; m += 64) {
      const int jX = (int)(m % QX);
      const long long ia = m / QX;  // iX * Rl + a
      const long long iX = ia / Rl, a = ia % Rl;
      const float x = X[((t * PX + iX) * Rl + a) * QX * (long long)Rm + (long long)jX * Rm + s];
      const float y = dY[(((t * PY + iX * pk + ik) * Rl + a) * QY + (long long)jX * qk + jk) * Rr + r];
      acc = fmaf(x, y, acc);
    }
    acc = wave_sum(acc);
    if (lane == 0) dG[e] = acc;
  }
}

__global__ __launch_bounds__(GBLK) void k_dsplit_x_wave(const float *__restrict__ dY,
                                                        const float *__restrict__ G,
                                                        float *__restrict__ dX, long long n,
                                                        int PX, int pk, int Rl, int QX, int qk,
                                                        int Rm, int Rr) {
  const long long PY = (long long)PX * pk, QY = (long long)QX * qk;
  const long long L = (long long)pk * qk * Rr;  // terms (ik, jk, r), r fastest
  const int lane = threadIdx.x & 63;
  for (long long e = (blockIdx.x * (long long)GBLK + threadIdx.x) >> 6; e < n;
       e += ((long long)gridDim.x * GBLK) >> 6) {
    long long v = e;
    const int s = (int)(v % Rm); v /= Rm;
    const int jX = (int)(v % QX); v /= QX;
    const int a = (int)(v % Rl); v /= Rl;
    const long long iX = v % PX;
    const long long t = v / PX;
    float acc = 0.f;
    for (long long m = lane; m < L; m += 64) {
      const int r = (int)(m % Rr);
      const long long u = m / Rr;
      const int jk = (int)(u % qk);
      const long long ik = u / qk;
      const float y = dY[(((t * PY + iX * pk + ik) * Rl + a) * QY + (long long)jX * qk + jk) * Rr + r];
      const float g = G[(((t * pk + ik) * Rm + s) * (long long)qk + jk) * Rr + r];
      acc = fmaf(y, g, acc);
    }
    acc = wave_sum(acc);
    if (lane == 0) dX[e] = acc;
  }
}

// SGD on every core in one launch: entries with a zero gradient (every entry of an
// untouched slice) keep their bits
struct ApplyArgs {
  float *x[TT_MAX_CORES];
  const float *g[TT_MAX_CORES];
  long long end[TT_MAX_CORES];  // running sum of the cores' sizes
  int ncores;
  float lr;
};

__global__ __launch_bounds__(GBLK) void k_dapply(ApplyArgs A) {
  const long long n = A.end[A.ncores - 1];
  for (long long e = blockIdx.x * (long long)GBLK + threadIdx.x; e < n;
       e += (long long)gridDim.x * GBLK) {
    int k = 0;
    while (k < A.ncores - 1 && e >= A.end[k]) ++k;
    const long long i = e - (k > 0 ? A.end[k - 1] : 0);
    const float ge = A.g[k][i];
    if (ge != 0.f) A.x[k][i] = A.x[k][i] - A.lr * ge;
  }
}

int grid_for(long long n) {
  const long long b = (n + GBLK - 1) / GBLK;
  return (int)(b < 8192 ? (b > 0 ? b : 1) : 8192);
}

constexpr long long WAVE_SUM_MIN = 64;  // sums at least this long take a wavefront each

struct DPlan {
  int d, T;
  int lo[3], hi[3];
  long long R[TT_MAX_CORES + 1];  // full ranks, R[0] = R[d] = 1
  tt_desc d3;
  size_t ws3;                     // bytes of the three-core workspace (at offset 0)
  size_t offP[TT_MAX_CORES];      // prefix product ending at core k (k > group start)
  size_t offdP[TT_MAX_CORES];     // its gradient (k > group start)
  size_t offdG[TT_MAX_CORES];     // gradient of core k (SGD)
  long long numelG[TT_MAX_CORES];
  long long numelP[TT_MAX_CORES];
  size_t total;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// numel of the prefix product of group [lo, k] (k inclusive)
long long prefix_numel(const tt_desc_d *d, const long long *R, int T, int lo, int k) {
  long long P = 1, Q = 1;
  for (int m = lo; m <= k; ++m) {
    P *= d->p[m];
    Q *= d->q[m];
  }
  return (long long)T * P * R[lo] * Q * R[k + 1];
}

// dense work (multiply-adds) of the merges and the splits of group [lo, hi)
double group_cost(const tt_desc_d *d, const long long *R, int T, int lo, int hi) {
  double c = 0.0;
  long long PX = d->p[lo], QX = d->q[lo];
  for (int k = lo + 1; k < hi; ++k) {
    const double nP = (double)prefix_numel(d, R, T, lo, k);
    const double nG = (double)T * d->p[k] * R[k] * d->q[k] * R[k + 1];
    const double nX = (double)prefix_numel(d, R, T, lo, k - 1);
    c += nP * R[k];                                  // merge
    c += nG * (double)PX * R[lo] * QX;               // dG_k
    c += nX * (double)d->p[k] * d->q[k] * R[k + 1];  // dM_{k-1}
    PX *= d->p[k];
    QX *= d->q[k];
  }
  return c;
}

int validate_d(const tt_desc_d *d) {
  if (!d) return TT_EINVAL;
  if (d->d < 3 || d->d > TT_MAX_CORES || d->num_tables < 1) return TT_ESHAPE;
  if (d->pooling != TT_POOL_SUM && d->pooling != TT_POOL_MEAN) return TT_EINVAL;
  double prodp = 1.0;
  for (int k = 0; k < d->d; ++k) {
    if (d->p[k] < 1 || d->q[k] < 1) return TT_ESHAPE;
    prodp *= d->p[k];
  }
  for (int k = 0; k < d->d - 1; ++k)
    if (d->ranks[k] < 1 || d->ranks[k] > 64) return TT_ESHAPE;
  if (d->num_embeddings < 1 || (double)d->num_embeddings > prodp) return TT_ESHAPE;
  return TT_OK;
}

int make_dplan(const tt_desc_d *d, int64_t nnz, int64_t num_bags, DPlan *P) {
  const int rc = validate_d(d);
  if (rc != TT_OK) return rc;
  memset(P, 0, sizeof(*P));
  P->d = d->d;
  P->T = d->num_tables;
  P->R[0] = P->R[d->d] = 1;
  for (int k = 1; k < d->d; ++k) P->R[k] = d->ranks[k - 1];
  // the cheapest cut [0, a) [a, b) [b, d) that the three-core path accepts
  double best = -1.0;
  for (int a = 1; a < d->d - 1; ++a)
    for (int b = a + 1; b < d->d; ++b) {
      const int lo[3] = {0, a, b}, hi[3] = {a, b, d->d};
      tt_desc t3;
      memset(&t3, 0, sizeof(t3));
      t3.num_tables = d->num_tables;
      t3.num_embeddings = d->num_embeddings;
      t3.pooling = d->pooling;
      bool fits = true;
      for (int g = 0; g < 3; ++g) {
        long long pp = 1, qq = 1;
        for (int k = lo[g]; k < hi[g]; ++k) {
          pp *= d->p[k];
          qq *= d->q[k];
        }
        if (pp >= (1LL << 31) || qq > 1024) fits = false;
        t3.p[g] = (int32_t)(fits ? pp : 1);
        t3.q[g] = (int32_t)(fits ? qq : 1);
      }
      t3.ranks[0] = (int32_t)P->R[a];
      t3.ranks[1] = (int32_t)P->R[b];
      if (!fits) continue;
      const size_t w3 = tt_bag_workspace_size(&t3, nnz, num_bags, 0);
      if (w3 == 0) continue;
      double cost = 0.0;
      for (int g = 0; g < 3; ++g) cost += group_cost(d, P->R, P->T, lo[g], hi[g]);
      if (best < 0.0 || cost < best) {
        best = cost;
        for (int g = 0; g < 3; ++g) { P->lo[g] = lo[g]; P->hi[g] = hi[g]; }
        P->d3 = t3;
        P->ws3 = w3;
      }
    }
  if (best < 0.0) return TT_ESHAPE;
  size_t cur = align256(P->ws3);
  for (int k = 0; k < d->d; ++k) {
    P->numelG[k] = (long long)P->T * d->p[k] * P->R[k] * d->q[k] * P->R[k + 1];
    P->offdG[k] = cur;
    cur = align256(cur + (size_t)P->numelG[k] * 4);
  }
  for (int g = 0; g < 3; ++g)
    for (int k = P->lo[g] + 1; k < P->hi[g]; ++k) {
      P->numelP[k] = prefix_numel(d, P->R, P->T, P->lo[g], k);
      P->offP[k] = cur;
      cur = align256(cur + (size_t)P->numelP[k] * 4);
      P->offdP[k] = cur;
      cur = align256(cur + (size_t)P->numelP[k] * 4);
    }
  P->total = cur;
  return TT_OK;
}

float *wsf(void *ws, size_t off) { return (float *)((char *)ws + off); }

// shape arguments of the step M_k = M_{k-1} (x) G_k inside group g
struct Step {
  int PX, pk, Rl, QX, qk, Rm, Rr;
};

Step step_of(const tt_desc_d *d, const DPlan &P, int g, int k) {
  long long PX = 1, QX = 1;
  for (int m = P.lo[g]; m < k; ++m) {
    PX *= d->p[m];
    QX *= d->q[m];
  }
  return {(int)PX, d->p[k], (int)P.R[P.lo[g]], (int)QX, d->q[k], (int)P.R[k], (int)P.R[k + 1]};
}

// the three multiplied-out cores (merges enqueued on s)
hipError_t merge_all(const tt_desc_d *d, const DPlan &P, const float *const *cores, void *ws,
                     const float *S[3], hipStream_t s) {
  for (int g = 0; g < 3; ++g) {
    const float *cur = cores[P.lo[g]];
    for (int k = P.lo[g] + 1; k < P.hi[g]; ++k) {
      const Step st = step_of(d, P, g, k);
      float *out = wsf(ws, P.offP[k]);
      const long long n = P.numelP[k];
      tt_launch(K_DMERGE, k_dmerge, dim3(grid_for(n)), dim3(GBLK), 0, s, cur, cores[k], out, n,
                st.PX, st.pk, st.Rl, st.QX, st.qk, st.Rm, st.Rr);
      cur = out;
    }
    S[g] = cur;
  }
  return hipGetLastError();
}

int check_call(const tt_desc_d *d, const void *cores, const int64_t *indices, int64_t nnz,
               const int64_t *offsets, void *ws, size_t ws_bytes, DPlan *P, int64_t num_bags) {
  if (!cores || !offsets || !ws || (nnz > 0 && !indices)) return TT_EINVAL;
  const int rc = make_dplan(d, nnz, num_bags, P);
  if (rc != TT_OK) return rc;
  if (ws_bytes < P->total || ((uintptr_t)ws & 255)) return TT_EWORKSPACE;
  return TT_OK;
}

// backward of the d-core table: gradients of every core into dG[k] (fully overwritten)
int backward_d(const tt_desc_d *d, const DPlan &P, const float *const *cores,
               const int64_t *indices, int64_t nnz, const int64_t *offsets, int64_t num_bags,
               const float *psw, const float *grad_out, float *const *dG, void *ws,
               int32_t *dev_status, hipStream_t s, bool planned) {
  const float *S[3];
  hipError_t e = merge_all(d, P, cores, ws, S, s);
  if (e != hipSuccess) return TT_EHIP;
  float *dS[3];
  for (int g = 0; g < 3; ++g)
    dS[g] = P.hi[g] - P.lo[g] == 1 ? dG[P.lo[g]] : wsf(ws, P.offdP[P.hi[g] - 1]);
  int rc = (planned ? tt_bag_backward_grad_planned : tt_bag_backward_grad)(
      &P.d3, S, indices, nnz, offsets, num_bags, psw, nullptr, grad_out, dS, nullptr, ws, P.ws3,
      dev_status, s);
  if (rc != TT_OK) return rc;
  for (int g = 0; g < 3; ++g)
    for (int k = P.hi[g] - 1; k > P.lo[g]; --k) {
      const Step st = step_of(d, P, g, k);
      const float *X = k - 1 == P.lo[g] ? cores[P.lo[g]] : wsf(ws, P.offP[k - 1]);
      const float *dY = wsf(ws, P.offdP[k]);
      const long long nG = P.numelG[k];
      if ((long long)st.PX * st.Rl * st.QX >= WAVE_SUM_MIN)
        tt_launch(K_DSPLIT, k_dsplit_g_wave, dim3(grid_for(nG * 64)), dim3(GBLK), 0, s, X, dY,
                  dG[k], nG, st.PX, st.pk, st.Rl, st.QX, st.qk, st.Rm, st.Rr);
      else
        tt_launch(K_DSPLIT, k_dsplit_g, dim3(grid_for(nG)), dim3(GBLK), 0, s, X, dY, dG[k], nG,
                  st.PX, st.pk, st.Rl, st.QX, st.qk, st.Rm, st.Rr);
      float *dX = k - 1 == P.lo[g] ? dG[P.lo[g]] : wsf(ws, P.offdP[k - 1]);
      const long long nX = k - 1 == P.lo[g] ? P.numelG[P.lo[g]] : P.numelP[k - 1];
      if ((long long)st.pk * st.qk * st.Rr >= WAVE_SUM_MIN)
        tt_launch(K_DSPLIT, k_dsplit_x_wave, dim3(grid_for(nX * 64)), dim3(GBLK), 0, s, dY,
                  cores[k], dX, nX, st.PX, st.pk, st.Rl, st.QX, st.qk, st.Rm, st.Rr);
      else
        tt_launch(K_DSPLIT, k_dsplit_x, dim3(grid_for(nX)), dim3(GBLK), 0, s, dY, cores[k], dX,
                  nX, st.PX, st.pk, st.Rl, st.QX, st.qk, st.Rm, st.Rr);
    }
  return hipGetLastError() == hipSuccess ? TT_OK : TT_EHIP;
}

}  // namespace
}  // namespace ttb

using namespace ttb;

namespace ttb {
namespace {

int forward_d(const tt_desc_d *desc, const float *const *cores, const int64_t *indices,
              int64_t nnz, const int64_t *offsets, int64_t num_bags,
              const float *per_sample_weights, float *out, void *ws, size_t ws_bytes,
              int32_t *dev_status, void *stream, bool planned) {
  DPlan P;
  int rc = check_call(desc, cores, indices, nnz, offsets, ws, ws_bytes, &P, num_bags);
  if (rc != TT_OK) return rc;
  if (!out) return TT_EINVAL;
  for (int k = 0; k < desc->d; ++k)
    if (!cores[k]) return TT_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  const float *S[3];
  if (merge_all(desc, P, cores, ws, S, s) != hipSuccess) return TT_EHIP;
  return (planned ? tt_bag_forward_planned : tt_bag_forward)(
      &P.d3, S, indices, nnz, offsets, num_bags, per_sample_weights, nullptr, out, ws, P.ws3,
      dev_status, stream);
}

int grad_d(const tt_desc_d *desc, const float *const *cores, const int64_t *indices,
           int64_t nnz, const int64_t *offsets, int64_t num_bags,
           const float *per_sample_weights, const float *grad_out, float *const *grad_cores,
           void *ws, size_t ws_bytes, int32_t *dev_status, void *stream, bool planned) {
  DPlan P;
  int rc = check_call(desc, cores, indices, nnz, offsets, ws, ws_bytes, &P, num_bags);
  if (rc != TT_OK) return rc;
  if (!grad_out || !grad_cores) return TT_EINVAL;
  for (int k = 0; k < desc->d; ++k)
    if (!cores[k] || !grad_cores[k]) return TT_EINVAL;
  return backward_d(desc, P, cores, indices, nnz, offsets, num_bags, per_sample_weights,
                    grad_out, grad_cores, ws, dev_status, (hipStream_t)stream, planned);
}

int sgd_d(const tt_desc_d *desc, float *const *cores, const int64_t *indices, int64_t nnz,
          const int64_t *offsets, int64_t num_bags, const float *per_sample_weights,
          const float *grad_out, float lr, void *ws, size_t ws_bytes, int32_t *dev_status,
          void *stream, bool planned) {
  DPlan P;
  int rc = check_call(desc, cores, indices, nnz, offsets, ws, ws_bytes, &P, num_bags);
  if (rc != TT_OK) return rc;
  if (!grad_out) return TT_EINVAL;
  for (int k = 0; k < desc->d; ++k)
    if (!cores[k]) return TT_EINVAL;
  float *dG[TT_MAX_CORES];
  for (int k = 0; k < desc->d; ++k) dG[k] = wsf(ws, P.offdG[k]);
  hipStream_t s = (hipStream_t)stream;
  rc = backward_d(desc, P, cores, indices, nnz, offsets, num_bags, per_sample_weights, grad_out,
                  dG, ws, dev_status, s, planned);
  if (rc != TT_OK) return rc;
  ApplyArgs A;
  memset(&A, 0, sizeof(A));
  A.ncores = desc->d;
  A.lr = lr;
  long long run = 0;
  for (int k = 0; k < desc->d; ++k) {
    A.x[k] = cores[k];
    A.g[k] = dG[k];
    run += P.numelG[k];
    A.end[k] = run;
  }
  tt_launch(K_DAPPLY, k_dapply, dim3(grid_for(run)), dim3(GBLK), 0, s, A);
  return hipGetLastError() == hipSuccess ? TT_OK : TT_EHIP;
}

}  // namespace
}  // namespace ttb

extern "C" {

size_t tt_bag_workspace_size_d(const tt_desc_d *desc, int64_t nnz, int64_t num_bags) {
  DPlan P;
  if (make_dplan(desc, nnz, num_bags, &P) != TT_OK) return 0;
  return P.total;
}

int tt_bag_groups_d(const tt_desc_d *desc, int32_t cut[2]) {
  if (!cut) return TT_EINVAL;
  DPlan P;
  const int rc = make_dplan(desc, 1, 1, &P);
  if (rc != TT_OK) return rc;
  cut[0] = P.lo[1];
  cut[1] = P.lo[2];
  return TT_OK;
}

int tt_bag_plan_d(const tt_desc_d *desc, const int64_t *indices, int64_t nnz,
                  const int64_t *offsets, int64_t num_bags, const float *per_sample_weights,
                  void *ws, size_t ws_bytes, int32_t *dev_status, void *stream) {
  DPlan P;
  if (!offsets || !ws || (nnz > 0 && !indices)) return TT_EINVAL;
  const int rc = make_dplan(desc, nnz, num_bags, &P);
  if (rc != TT_OK) return rc;
  if (ws_bytes < P.total || ((uintptr_t)ws & 255)) return TT_EWORKSPACE;
  return tt_bag_plan(&P.d3, indices, nnz, offsets, num_bags, per_sample_weights, nullptr, ws,
                     P.ws3, dev_status, stream);
}

int tt_bag_forward_d(const tt_desc_d *desc, const float *const *cores, const int64_t *indices,
                     int64_t nnz, const int64_t *offsets, int64_t num_bags,
                     const float *per_sample_weights, float *out, void *ws, size_t ws_bytes,
                     int32_t *dev_status, void *stream) {
  return forward_d(desc, cores, indices, nnz, offsets, num_bags, per_sample_weights, out, ws,
                   ws_bytes, dev_status, stream, false);
}

int tt_bag_forward_d_planned(const tt_desc_d *desc, const float *const *cores,
                             const int64_t *indices, int64_t nnz, const int64_t *offsets,
                             int64_t num_bags, const float *per_sample_weights, float *out,
                             void *ws, size_t ws_bytes, int32_t *dev_status, void *stream) {
  return forward_d(desc, cores, indices, nnz, offsets, num_bags, per_sample_weights, out, ws,
                   ws_bytes, dev_status, stream, true);
}

int tt_bag_backward_grad_d(const tt_desc_d *desc, const float *const *cores,
                           const int64_t *indices, int64_t nnz, const int64_t *offsets,
                           int64_t num_bags, const float *per_sample_weights,
                           const float *grad_out, float *const *grad_cores, void *ws,
                           size_t ws_bytes, int32_t *dev_status, void *stream) {
  return grad_d(desc, cores, indices, nnz, offsets, num_bags, per_sample_weights, grad_out,
                grad_cores, ws, ws_bytes, dev_status, stream, false);
}

int tt_bag_backward_grad_d_planned(const tt_desc_d *desc, const float *const *cores,
                                   const int64_t *indices, int64_t nnz, const int64_t *offsets,
                                   int64_t num_bags, const float *per_sample_weights,
                                   const float *grad_out, float *const *grad_cores, void *ws,
                                   size_t ws_bytes, int32_t *dev_status, void *stream) {
  return grad_d(desc, cores, indices, nnz, offsets, num_bags, per_sample_weights, grad_out,
                grad_cores, ws, ws_bytes, dev_status, stream, true);
}

int tt_bag_backward_sgd_d(const tt_desc_d *desc, float *const *cores, const int64_t *indices,
                          int64_t nnz, const int64_t *offsets, int64_t num_bags,
                          const float *per_sample_weights, const float *grad_out, float lr,
                          void *ws, size_t ws_bytes, int32_t *dev_status, void *stream) {
  return sgd_d(desc, cores, indices, nnz, offsets, num_bags, per_sample_weights, grad_out, lr,
               ws, ws_bytes, dev_status, stream, false);
}

int tt_bag_backward_sgd_d_planned(const tt_desc_d *desc, float *const *cores,
                                  const int64_t *indices, int64_t nnz, const int64_t *offsets,
                                  int64_t num_bags, const float *per_sample_weights,
                                  const float *grad_out, float lr, void *ws, size_t ws_bytes,
                                  int32_t *dev_status, void *stream) {
  return sgd_d(desc, cores, indices, nnz, offsets, num_bags, per_sample_weights, grad_out, lr,
               ws, ws_bytes, dev_status, stream, true);
}

}  // extern "C"
