// tt_init.hip -- initialisation of the TT cores on the device, and the automatic
// factorisation of the table's shape (host).
//
// "FBTT-Embedding" README, "Parameters" (`weight_dist`): the cores are either drawn
// i.i.d. from the named distribution, or drawn so that the entries of the full table
// follow it ("approx-" variants); the TT-Rec abstract proposes sampled-Gaussian cores.
// Every entry of W is a sum over R1*R2 products of one entry of each core, so with
// zero-mean i.i.d. cores of variances v1, v2, v3, Var(W) = R1 R2 v1 v2 v3 (and by the
// central limit theorem W is close to normal).  The approx- variants choose one core
// variance v with R1 R2 v^3 = the target's variance:
//   approx-normal  N(0, scale^2):       cores N(0, v),  v = (scale^2 / (R1 R2))^(1/3)
//   approx-uniform U(-scale, scale):    cores U(-c, c), c^2 / 3 = (scale^2 / (3 R1 R2))^(1/3)
// Random numbers: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC 2011) with key = seed and
// counter (n mod 2^32, n / 2^32, k, 0) for element n of core k (its position in the
// stored slice-major array of all tables); uniforms from the top 23 bits of a word,
// u = (x >> 9 + 1/2) 2^-23 in (0, 1) (exact in fp32); U(-a, a) = a (2 u0 - 1); normal
// by Box-Muller (1958): a sqrt(-2 ln u0) cos(2 pi u1).
#include <algorithm>
#include <cmath>
#include <vector>

#include "tt_internal.h"

namespace ttb {

struct Philox4 {
  unsigned x[4];
};

__device__ __forceinline__ Philox4 philox4x32_10(unsigned c0, unsigned c1, unsigned c2,
                                                 unsigned c3, unsigned k0, unsigned k1) {
  for (int r = 0; r < 10; ++r) {
    const unsigned long long p0 = 0xD2511F53ull * c0, p1 = 0xCD9E8D57ull * c2;
    const unsigned n0 = (unsigned)(p1 >> 32) ^ c1 ^ k0, n2 = (unsigned)(p0 >> 32) ^ c3 ^ k1;
    c1 = (unsigned)p1;
    c3 = (unsigned)p0;
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  Philox4 o;
  o.x[0] = c0; o.x[1] = c1; o.x[2] = c2; o.x[3] = c3;
  return o;
}

__global__ __launch_bounds__(256) void k_init(float *core, long long n, int k, int dist,
                                               float a, unsigned k0, unsigned k1) {
  const long long stride = (long long)gridDim.x * 256;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) {
    const Philox4 r = philox4x32_10((unsigned)i, (unsigned)(i >> 32), (unsigned)k, 0u, k0, k1);
    const float u0 = ((float)(r.x[0] >> 9) + 0.5f) * (1.0f / 8388608.0f);
    float v;
    if (dist == TT_INIT_NORMAL || dist == TT_INIT_APPROX_NORMAL) {
      const float u1 = ((float)(r.x[1] >> 9) + 0.5f) * (1.0f / 8388608.0f);
      v = a * sqrtf(-2.0f * logf(u0)) * cosf(6.283185307179586f * u1);
    } else {
      v = a * (2.0f * u0 - 1.0f);
    }
    core[i] = v;
  }
}

// the parameter of the core distribution (std of a normal, half-width of a uniform)
static double core_param(int dist, double scale, int R1, int R2) {
  const double rr = (double)R1 * (double)R2;
  switch (dist) {
    case TT_INIT_APPROX_NORMAL: return std::sqrt(std::cbrt(scale * scale / rr));
    case TT_INIT_APPROX_UNIFORM: return std::sqrt(3.0 * std::cbrt(scale * scale / (3.0 * rr)));
    default: return scale;
  }
}

}  // namespace ttb

using namespace ttb;

extern "C" {

int tt_init_cores(const tt_desc *desc, float *const cores[3], int dist, float scale,
                  uint64_t seed, void *stream) {
  if (!desc || !cores || !cores[0] || !cores[1] || !cores[2]) return TT_EINVAL;
  if (dist < TT_INIT_UNIFORM || dist > TT_INIT_APPROX_NORMAL) return TT_EINVAL;
  if (!std::isfinite(scale) || scale < 0.f) return TT_EINVAL;
  if (desc->num_tables < 1 || desc->ranks[0] < 1 || desc->ranks[1] < 1) return TT_ESHAPE;
  for (int k = 0; k < 3; ++k)
    if (desc->p[k] < 1 || desc->q[k] < 1) return TT_ESHAPE;
  const int R[4] = {1, desc->ranks[0], desc->ranks[1], 1};
  const float a = (float)core_param(dist, scale, desc->ranks[0], desc->ranks[1]);
  hipStream_t s = (hipStream_t)stream;
  for (int k = 0; k < 3; ++k) {
    const long long n = (long long)desc->num_tables * desc->p[k] * R[k] * desc->q[k] * R[k + 1];
    const unsigned nb = (unsigned)std::min<long long>((n + 255) / 256, 16384);
    hipLaunchKernelGGL(k_init, dim3(nb), dim3(256), 0, s, cores[k], n, k, dist, a,
                       (unsigned)seed, (unsigned)(seed >> 32));
  }
  return hipGetLastError() == hipSuccess ? TT_OK : TT_EHIP;
}

// Automatic shapes ("Initialization": with no p / q shapes given, num_embeddings and
// embedding_dim are factored automatically; the rule is not stated).  Reading taken:
//  exact (q, product == n, among the shapes the kernels take: q1 in {1, 2, 4},
//    q3 <= 16): the triple with the smallest largest factor; then the largest smallest
//    factor; then the smallest first factor; then the largest second.
//  not exact (p, product >= n): largest factor m = the smallest m with m^3 >= n; then
//    the smallest product; then the smallest first factor; factors ascending.
int tt_factorize(int64_t n, int exact, int32_t out[3]) {
  if (!out || n < 1 || n >= ((int64_t)1 << 31)) return TT_EINVAL;
  if (exact) {
    std::vector<int64_t> divs;
    for (int64_t d = 1; d * d <= n; ++d)
      if (n % d == 0) {
        divs.push_back(d);
        if (d * d != n) divs.push_back(n / d);
      }
    int64_t best[3] = {0, 0, 0};
    for (int64_t a : divs)
      for (int64_t b : divs) {
        if ((n / a) % b) continue;
        const int64_t c = n / a / b;
        if (!(a == 1 || a == 2 || a == 4) || c > 16) continue;  // shapes the kernels take
        const int64_t mx = std::max(a, std::max(b, c)), mn = std::min(a, std::min(b, c));
        const int64_t bmx = std::max(best[0], std::max(best[1], best[2]));
        const int64_t bmn = std::min(best[0], std::min(best[1], best[2]));
        const bool better =
            best[0] == 0 || mx < bmx ||
            (mx == bmx && (mn > bmn || (mn == bmn && (a < best[0] || (a == best[0] && b > best[1])))));
        if (better) { best[0] = a; best[1] = b; best[2] = c; }
      }
    if (best[0] == 0) return TT_ESHAPE;
    for (int k = 0; k < 3; ++k) out[k] = (int32_t)best[k];
    return TT_OK;
  }
  int64_t m = (int64_t)std::cbrt((double)n);
  while (m > 1 && (m - 1) * (m - 1) * (m - 1) >= n) --m;
  while (m * m * m < n) ++m;
  int64_t bp = -1, b1 = 0, b2 = 0;
  for (int64_t p2 = 1; p2 <= m; ++p2) {
    const int64_t need = (n + m * p2 - 1) / (m * p2);  // smallest p1 with p1 p2 m >= n
    const int64_t p1 = std::max<int64_t>(need, 1);
    if (p1 > p2) continue;
    const int64_t prod = p1 * p2;
    if (bp < 0 || prod < bp || (prod == bp && p1 < b1)) { bp = prod; b1 = p1; b2 = p2; }
  }
  out[0] = (int32_t)b1; out[1] = (int32_t)b2; out[2] = (int32_t)m;
  return TT_OK;
}

}  // extern "C"
