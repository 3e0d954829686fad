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

constexpr int FULL_T = 512;
constexpr size_t FULL_G3_BYTES = 96 * 1024;  // LDS for G3 slices

struct FullArgs {
  const float *G1, *G2, *G3;  // table t's cores (slice-major)
  float *out;
  long long first, count;     // rows [first, first + count) -> out[0 ..)
  int p2, p3, q1, q2, q3, R1, R2, D;
  int i3c;                    // G3 slices per LDS chunk
};

// dst[(e / w) * ld + e % w] = src[e] for e < n, whole block, 8 loads in flight per thread
static __device__ void stage(float *dst, const float *src, int n, int w, int ld) {
  const int tid = threadIdx.x;
  for (int b = tid; b < n; b += FULL_T * 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = src[min(b + u * FULL_T, n - 1)];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int e = b + u * FULL_T;
      if (e < n) dst[ld == w ? e : (e / w) * ld + e % w] = v[u];
    }
  }
}

// padded LDS strides: T rows (one per (j1, j2)) and G3 slices, against bank conflicts
__host__ __device__ inline int full_ts(int R2) { return R2 + 1; }
__host__ __device__ inline int full_g3s(int W3) { return W3 + 4; }

// q3 <= Q3M (a power of two); EXACT: q3 == Q3M (contiguous vector reads and stores)
template <int Q3M, bool EXACT>
__global__ __launch_bounds__(FULL_T) void k_full(FullArgs f) {
  extern __shared__ float lds[];
  const int tid = threadIdx.x;
  const int W3 = f.R2 * f.q3, W2 = f.R1 * f.q2 * f.R2, W1 = f.q1 * f.R1;
  const int nT = f.q1 * f.q2 * f.R2;
  const int TS = full_ts(f.R2), G3S = full_g3s(W3);
  float *sG3 = lds;                                  // [i3c][G3S]: [R2][q3] + pad
  float *sG2 = sG3 + (size_t)f.i3c * G3S;            // [R1][q2][R2]
  float *sG1 = sG2 + W2;                             // [q1][R1]
  float *sT = sG1 + W1;                              // [q1 q2][TS]
  const long long last = f.first + f.count - 1;
  const long long u0 = f.first / f.p3, u1 = last / f.p3;  // pairs (i1 * p2 + i2)
  const bool whole = f.i3c >= f.p3;
  if (whole) stage(sG3, f.G3, f.p3 * W3, W3, G3S);
  for (long long u = u0 + blockIdx.x; u <= u1; u += gridDim.x) {
    const long long i1 = u / f.p2, i2 = u - i1 * f.p2;
    __syncthreads();  // the previous pair's T and G3 chunk are no longer read
    stage(sG2, f.G2 + (size_t)i2 * W2, W2, W2, W2);
    stage(sG1, f.G1 + (size_t)i1 * W1, W1, W1, W1);
    __syncthreads();
    // T[j1 j2][r2] = sum_r1 G1[i1][j1][r1] G2[i2][r1][j2][r2]
    for (int e = tid; e < nT; e += FULL_T) {
      const int r2 = e % f.R2, jj = e / f.R2, j2 = jj % f.q2, j1 = jj / f.q2;
      float acc = 0.f;
      for (int r1 = 0; r1 < f.R1; ++r1)
        acc += sG1[j1 * f.R1 + r1] * sG2[(r1 * f.q2 + j2) * f.R2 + r2];
      sT[jj * TS + r2] = acc;
    }
    // the pair's rows inside the requested range
    const long long base = u * f.p3;
    const int a0 = (int)std::max<long long>(0, f.first - base);
    const int a1 = (int)std::min<long long>(f.p3 - 1, last - base);
    for (int c0 = a0; c0 <= a1; c0 += f.i3c) {
      const int c1 = std::min(a1, c0 + f.i3c - 1);
      if (!whole) {
        __syncthreads();
        stage(sG3, f.G3 + (size_t)c0 * W3, (c1 - c0 + 1) * W3, W3, G3S);
      }
      __syncthreads();
      const int g0 = whole ? c0 : 0;  // chunk row of i3 = c0
      // task = 4 rows x (all q3 columns) of one (j1, j2); tasks with consecutive (j1, j2)
      // write consecutive q3-float pieces of a row
      const int nrow = c1 - c0 + 1, njj = f.q1 * f.q2, ntask = ((nrow + 3) >> 2) * njj;
      for (int task = tid; task < ntask; task += FULL_T) {
        const int jj = task % njj, r0 = (task / njj) * 4;
        float acc[4][Q3M];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
#pragma unroll
          for (int j3 = 0; j3 < Q3M; ++j3) acc[rr][j3] = 0.f;
        const float *t = sT + jj * TS;
        const float *g[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) g[rr] = sG3 + (size_t)(g0 + min(r0 + rr, nrow - 1)) * G3S;
        // reads clamped instead of guarded (a guard becomes a branch around each read)
        int jc[Q3M];
#pragma unroll
        for (int j3 = 0; j3 < Q3M; ++j3) jc[j3] = EXACT ? j3 : min(j3, f.q3 - 1);
        const int q3 = EXACT ? Q3M : f.q3;
        for (int r2 = 0; r2 < f.R2; ++r2) {
          const float tv = t[r2];
          float gv[4][Q3M];
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
#pragma unroll
            for (int j3 = 0; j3 < Q3M; ++j3) gv[rr][j3] = g[rr][r2 * q3 + jc[j3]];
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
#pragma unroll
            for (int j3 = 0; j3 < Q3M; ++j3) acc[rr][j3] += tv * gv[rr][j3];
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          if (r0 + rr >= nrow) break;
          float *o = f.out + (size_t)(base + c0 + r0 + rr - f.first) * f.D + jj * q3;
          if constexpr (EXACT && Q3M % 4 == 0) {
#pragma unroll
            for (int j3 = 0; j3 < Q3M; j3 += 4)
              *(float4 *)(o + j3) =
                  make_float4(acc[rr][j3], acc[rr][j3 + 1], acc[rr][j3 + 2], acc[rr][j3 + 3]);
          } else {
#pragma unroll
            for (int j3 = 0; j3 < Q3M; ++j3)
              if (j3 < q3) o[j3] = acc[rr][j3];
          }
        }
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

template <int Q3M, bool EXACT>
static hipError_t launch_full_t(const FullArgs &f, dim3 grid, size_t lds, hipStream_t s) {
  static size_t attr = 64 * 1024;  // dynamic LDS above 64 KiB is opt-in per kernel
  if (lds > attr) {
    const hipError_t e = hipFuncSetAttribute((const void *)k_full<Q3M, EXACT>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr = lds;
  }
  hipLaunchKernelGGL((k_full<Q3M, EXACT>), grid, dim3(FULL_T), lds, s, f);
  return hipGetLastError();
}

// vector stores need 16-byte aligned rows: out aligned and D a multiple of 4
template <int Q3M>
static hipError_t launch_full(const FullArgs &f, dim3 grid, size_t lds, hipStream_t s) {
  const bool exact = f.q3 == Q3M && ((uintptr_t)f.out & 15) == 0 && f.D % 4 == 0;
  return exact ? launch_full_t<Q3M, true>(f, grid, lds, s) : launch_full_t<Q3M, false>(f, grid, lds, s);
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
      R1 < 1 || R2 < 1 || q3 > 16)
    return TT_ESHAPE;
  const size_t W1 = (size_t)q1 * R1, W2 = (size_t)R1 * q2 * R2, W3 = (size_t)R2 * q3;
  const size_t nT = (size_t)q1 * q2 * full_ts(R2), G3S = (size_t)full_g3s((int)W3);
  const size_t fixed = (W2 + W1 + nT) * 4;
  if (fixed + G3S * 4 > 160 * 1024) return TT_ESHAPE;  // one G3 slice must fit beside T, G2
  const size_t g3_room = std::max<size_t>(G3S * 4, std::min<size_t>(FULL_G3_BYTES, 160 * 1024 - fixed));
  int i3c = (int)std::min<size_t>((size_t)desc->p[2], g3_room / (G3S * 4));
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
  const size_t lds = fixed + (size_t)i3c * G3S * 4;
  const long long pairs = (first + count - 1) / f.p3 - first / f.p3 + 1;
  const dim3 grid((unsigned)std::min<long long>(pairs, (long long)device_cu_count()));
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (q3 <= 1) e = launch_full<1>(f, grid, lds, s);
  else if (q3 <= 2) e = launch_full<2>(f, grid, lds, s);
  else if (q3 <= 4) e = launch_full<4>(f, grid, lds, s);
  else if (q3 <= 8) e = launch_full<8>(f, grid, lds, s);
  else e = launch_full<16>(f, grid, lds, s);
  return e == hipSuccess ? TT_OK : TT_EHIP;
}

}  // extern "C"
