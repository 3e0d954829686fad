// tt_full.hip -- rows of the full table decompressed into a dense buffer.
//
// "FBTT-Embedding" README, "Initialization": core k has logical shape
// R_{k-1} x p_k x q_k x R_k and a row is the chain G1[i1] G2[i2] G3[i3].  Rows with the
// same (i1, i2) are p3 consecutive indices and share T = G1[i1] G2[i2] ([q1 q2][R2]),
// so each workgroup builds T once per pair in LDS and writes the pair's rows as
// row[j1 j2][j3] = sum_r2 T[j1 j2][r2] G3[i3][r2][j3], with a chunk of the table's G3
// slices staged in LDS (the whole of G3 when it fits, then kept across pairs).
#include <algorithm>

#include "tt_internal.h"

namespace ttb {

constexpr int FULL_T = 256;
constexpr size_t FULL_G3_BYTES = 96 * 1024;  // LDS for G3 slices

struct FullArgs {
  const float *G1, *G2, *G3;  // table t's cores (slice-major)
  float *out;
  long long first, count;     // rows [first, first + count) -> out[0 ..)
  int p2, p3, q1, q2, q3, R1, R2, D;
  int i3c;                    // G3 slices per LDS chunk
};

__global__ __launch_bounds__(FULL_T) void k_full(FullArgs f) {
  extern __shared__ float lds[];
  const int tid = threadIdx.x;
  const int W3 = f.R2 * f.q3, W2 = f.R1 * f.q2 * f.R2, W1 = f.q1 * f.R1;
  const int nT = f.q1 * f.q2 * f.R2;
  float *sG3 = lds;                                  // [i3c][R2][q3]
  float *sG2 = sG3 + (size_t)f.i3c * W3;             // [R1][q2][R2]
  float *sG1 = sG2 + W2;                             // [q1][R1]
  float *sT = sG1 + W1;                              // [q1 q2][R2]
  const long long last = f.first + f.count - 1;
  const long long u0 = f.first / f.p3, u1 = last / f.p3;  // pairs (i1 * p2 + i2)
  const bool whole = f.i3c >= f.p3;
  if (whole) {
    for (int e = tid; e < f.p3 * W3; e += FULL_T) sG3[e] = f.G3[e];
  }
  for (long long u = u0 + blockIdx.x; u <= u1; u += gridDim.x) {
    const long long i1 = u / f.p2, i2 = u - i1 * f.p2;
    __syncthreads();  // the previous pair's T and G3 chunk are no longer read
    for (int e = tid; e < W2; e += FULL_T) sG2[e] = f.G2[(size_t)i2 * W2 + e];
    for (int e = tid; e < W1; e += FULL_T) sG1[e] = f.G1[(size_t)i1 * W1 + e];
    __syncthreads();
    // T[j1 j2][r2] = sum_r1 G1[i1][j1][r1] G2[i2][r1][j2][r2]
    for (int e = tid; e < nT; e += FULL_T) {
      const int r2 = e % f.R2, jj = e / f.R2, j2 = jj % f.q2, j1 = jj / f.q2;
      float acc = 0.f;
      for (int r1 = 0; r1 < f.R1; ++r1)
        acc += sG1[j1 * f.R1 + r1] * sG2[(r1 * f.q2 + j2) * f.R2 + r2];
      sT[e] = acc;
    }
    // the pair's rows inside the requested range
    const long long base = u * f.p3;
    const int a0 = (int)std::max<long long>(0, f.first - base);
    const int a1 = (int)std::min<long long>(f.p3 - 1, last - base);
    for (int c0 = a0; c0 <= a1; c0 += f.i3c) {
      const int c1 = std::min(a1, c0 + f.i3c - 1);
      if (!whole) {
        __syncthreads();
        for (int e = tid; e < (c1 - c0 + 1) * W3; e += FULL_T) sG3[e] = f.G3[(size_t)c0 * W3 + e];
      }
      __syncthreads();
      const int g0 = whole ? c0 : 0;  // chunk row of i3 = c0
      const long long nout = (long long)(c1 - c0 + 1) * f.D;
      for (long long e = tid; e < nout; e += FULL_T) {
        const int r = (int)(e / f.D), d = (int)(e - (long long)r * f.D);
        const int j3 = d % f.q3, jj = d / f.q3;
        const float *t = sT + jj * f.R2, *g = sG3 + (size_t)(g0 + r) * W3 + j3;
        float acc = 0.f;
        for (int r2 = 0; r2 < f.R2; ++r2) acc += t[r2] * g[r2 * f.q3];
        f.out[(size_t)(base + c0 + r - f.first) * f.D + d] = acc;
      }
    }
  }
}

static int device_cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 256;
  return n > 0 ? n : 256;
}

}  // namespace ttb

using namespace ttb;

extern "C" {

int tt_full_weight(const tt_desc *desc, const float *const cores[3], int table, int64_t first,
                   int64_t count, float *out, void *stream) {
  if (!desc || !cores || !cores[0] || !cores[1] || !cores[2] || !out) return TT_EINVAL;
  if (table < 0 || table >= desc->num_tables || first < 0 || count < 0 ||
      first + count > desc->num_embeddings)
    return TT_EINVAL;
  const int q1 = desc->q[0], q2 = desc->q[1], q3 = desc->q[2], R1 = desc->ranks[0],
            R2 = desc->ranks[1];
  if (desc->p[0] < 1 || desc->p[1] < 1 || desc->p[2] < 1 || q1 < 1 || q2 < 1 || q3 < 1 ||
      R1 < 1 || R2 < 1)
    return TT_ESHAPE;
  const size_t W1 = (size_t)q1 * R1, W2 = (size_t)R1 * q2 * R2, W3 = (size_t)R2 * q3;
  const size_t nT = (size_t)q1 * q2 * R2;
  const size_t fixed = (W2 + W1 + nT) * 4;
  if (fixed + W3 * 4 > 160 * 1024) return TT_ESHAPE;  // one G3 slice must fit beside T, G2
  const size_t g3_room = std::max<size_t>(W3 * 4, std::min<size_t>(FULL_G3_BYTES, 160 * 1024 - fixed));
  int i3c = (int)std::min<size_t>((size_t)desc->p[2], g3_room / (W3 * 4));
  if (count == 0) return TT_OK;
  FullArgs f;
  const size_t t = (size_t)table;
  f.G1 = cores[0] + t * desc->p[0] * W1;
  f.G2 = cores[1] + t * desc->p[1] * W2;
  f.G3 = cores[2] + t * desc->p[2] * W3;
  f.out = out;
  f.first = first;
  f.count = count;
  f.p2 = desc->p[1]; f.p3 = desc->p[2];
  f.q1 = q1; f.q2 = q2; f.q3 = q3; f.R1 = R1; f.R2 = R2; f.D = q1 * q2 * q3;
  f.i3c = i3c;
  const size_t lds = fixed + (size_t)i3c * W3 * 4;
  static size_t attr = 64 * 1024;
  if (lds > attr) {
    if (hipFuncSetAttribute((const void *)k_full, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)lds) != hipSuccess)
      return TT_EHIP;
    attr = lds;
  }
  const long long pairs = (first + count - 1) / f.p3 - first / f.p3 + 1;
  const long long nb = std::min<long long>(pairs, 4LL * device_cu_count());
  hipLaunchKernelGGL(k_full, dim3((unsigned)nb), dim3(FULL_T), lds, (hipStream_t)stream, f);
  return hipGetLastError() == hipSuccess ? TT_OK : TT_EHIP;
}

}  // extern "C"
