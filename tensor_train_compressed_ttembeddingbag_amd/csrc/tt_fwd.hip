// tt_fwd.hip -- forward TT contraction + bag pooling.
//
// "FBTT-Embedding" README, "Software Cache": a lookup rebuilds a row by two
// consecutive GEMMs; "TT-Rec" (MLSys 2021) abstract: lookups are batched into
// matrix multiplications.  With the row split i -> (i1,i2,i3):
//   stage 1  T[j1][j2][r2] = sum_r1 G1[i1][j1][r1] * G2[i2][r1][j2][r2]
//   stage 2  W[i][(j1 q2 + j2) q3 + j3] = sum_r2 T[j1][j2][r2] * G3[i3][r2][j3]
// and EmbeddingBag pooling out[b] += w_n * W[idx_n] (tensorflow/addons #2201: the
// gathered rows are never materialised).
//
// One workgroup takes up to 64 consecutive elements of one (table, i2) group of
// the grouping order (so all of them share one G2 slice).  Stage 1 runs once per
// distinct (i1, i2) pair ("pair"), as a GEMM on the fp32 matrix cores:
//     T^T[r2][(pair, j1)] = sum_r1 G2[r1][j2][r2] * G1[i1(pair)][j1][r1]
// with the G2 column block j2 staged in LDS (transposed to [r2][r1]) and the
// (pair, j1) rows in the MFMA column dimension, 16 per "M-block".  Stage 2 runs
// once per distinct index ("item") in VALU, reducing over the four lane groups,
// and each element of the item adds w * row into out with an fp32 atomic.
// Bits of out may therefore depend on the order of the atomics (the tolerance,
// not bit equality, is the contract for out).
#include "tt_internal.h"
#include "tt_mfma.h"

namespace ttb {

template <int RP>
struct FwdLds {
  static constexpr int LD = RP + 4;
  static constexpr int G2F = 2 * RP * LD;            // floats: double-buffered G2 column block
  static constexpr int BYTES = G2F * 4 + (64 * 4 + 65 + 64 + 65 + 64 + 4) * 4;
};

template <int RP>
__global__ __launch_bounds__(WG) void k_fwd(DevArgs a) {
  constexpr int KS = RP / 4;   // k-steps: lane group g covers r1 = g*KS + ks
  constexpr int NM = RP / 16;  // 16-row blocks of r2
  constexpr int LD = FwdLds<RP>::LD;
  extern __shared__ float smem[];
  float *sG2 = smem;
  int *e_dA = (int *)(smem + FwdLds<RP>::G2F);
  int *e_bag = e_dA + 64;
  float *e_w = (float *)(e_bag + 64);
  int *e_i3 = (int *)(e_w + 64);
  int *it_beg = e_i3 + 64;   // [65]
  int *it_i3 = it_beg + 65;  // [64]
  int *pr_it = it_i3 + 64;   // [65]
  int *pr_i1 = pr_it + 65;   // [64]
  int *s_cnt = pr_i1 + 64;   // [4]

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, c = lane & 15;
  const int wi = blockIdx.x;
  if (wi >= a.hdr[H_NFWD]) return;
  const int G = a.T * a.p2;
  int lo = 0, hi = G;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.chunk_pre[mid] <= wi) lo = mid; else hi = mid;
  }
  const int grp = lo;
  const int s0 = a.grp_off[grp] + (wi - a.chunk_pre[grp]) * FWD_CHE;
  const int s1 = min(s0 + FWD_CHE, a.grp_off[grp + 1]);
  const int n_el = s1 - s0;
  const int t = grp / a.p2, i2 = grp % a.p2;
  const int q1 = a.q1, q2 = a.q2, q3 = a.q3, R1 = a.R1, R2 = a.R2, D = a.D;

  if (tid < 64) {
    const bool v = tid < n_el;
    int dA = -1, i3 = -1;
    if (v) {
      const int s = s0 + tid;
      dA = a.s_dA[s];
      i3 = a.s_dI3[s] - t * a.p3;
      e_dA[tid] = dA;
      e_i3[tid] = i3;
      e_bag[tid] = a.s_bag[s];
      e_w[tid] = a.psw ? a.psw[a.s_n[s]] : 1.f;
    }
    const int pdA = __shfl_up(dA, 1), pi3 = __shfl_up(i3, 1);
    const bool item_st = v && (tid == 0 || dA != pdA || i3 != pi3);
    const bool pair_st = v && (tid == 0 || dA != pdA);
    const unsigned long long mi = __ballot(item_st), mp = __ballot(pair_st);
    const unsigned long long lt = (tid == 0) ? 0ull : (~0ull >> (64 - tid));
    const int it = __popcll(mi & lt), pr = __popcll(mp & lt);
    if (item_st) { it_beg[it] = tid; it_i3[it] = i3; }
    if (pair_st) { pr_it[pr] = it; pr_i1[pr] = dA - t * a.p1; }
    if (tid == 0) {
      const int nI = __popcll(mi), nP = __popcll(mp);
      it_beg[nI] = n_el;
      pr_it[nP] = nI;
      s_cnt[0] = nI;
      s_cnt[1] = nP;
    }
  }
  __syncthreads();
  const int nP = s_cnt[1];
  const int nmb = (nP * q1 + 15) / 16;

  // B operand of stage 1 (G1 rows of the M-block's pairs), kept for all j2
  float bv[MBW][KS];
#pragma unroll
  for (int mbi = 0; mbi < MBW; ++mbi) {
    const int row = (w + mbi * NW) * 16 + c;
    const int pr = row / q1, j1 = row - pr * q1;
    const bool ok = (w + mbi * NW) < nmb && pr < nP;
    const float *src = a.G1 + ((size_t)(t * a.p1 + (ok ? pr_i1[pr] : 0)) * q1 + j1) * R1;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int r1 = g * KS + ks;
      bv[mbi][ks] = (ok && r1 < R1) ? src[r1] : 0.f;
    }
  }

  const size_t g2base = (size_t)(t * a.p2 + i2) * R1 * q2 * R2;
  const float *G3t = a.G3 + (size_t)t * a.p3 * R2 * q3;
  for (int j2 = 0; j2 < q2; ++j2) {
    float *buf = sG2 + (j2 & 1) * RP * LD;
    for (int i = tid; i < RP * RP; i += WG) {
      const int r1 = i / RP, r2 = i - r1 * RP;
      buf[r2 * LD + r1] = (r1 < R1 && r2 < R2) ? a.G2[g2base + ((size_t)r1 * q2 + j2) * R2 + r2] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int mbi = 0; mbi < MBW; ++mbi) {
      const int mb = w + mbi * NW;
      if (mb >= nmb) break;
      f4 acc[NM];
#pragma unroll
      for (int m = 0; m < NM; ++m) acc[m] = zero4();
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int m = 0; m < NM; ++m)
          acc[m] = mfma4(buf[(16 * m + c) * LD + g * KS + ks], bv[mbi][ks], acc[m]);
      }
      // stage 2: lane (g, c) holds T^T[r2 = 16m + 4g + v][row c] of this j2
      const int row = mb * 16 + c;
      const int pr = row / q1, j1 = row - pr * q1;
      const bool okp = pr < nP;
      const int ib = okp ? pr_it[pr] : 0, ie = okp ? pr_it[pr + 1] : 0;
      const int nk = wave_max(ie - ib);
      for (int kk = 0; kk < nk; ++kk) {
        const int it = ib + kk;
        const bool act = it < ie;
        const int i3 = act ? it_i3[it] : 0;
        const float *a3 = G3t + (size_t)i3 * R2 * q3;
        for (int j3 = 0; j3 < q3; ++j3) {
          float part = 0.f;
#pragma unroll
          for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const int r2 = 16 * m + 4 * g + v;
              if (act && r2 < R2) part += acc[m][v] * a3[r2 * q3 + j3];
            }
          part += __shfl_xor(part, 16);
          part += __shfl_xor(part, 32);
          if (act && g == (j3 & 3)) {
            const int col = (j1 * q2 + j2) * q3 + j3;
            for (int e = it_beg[it]; e < it_beg[it + 1]; ++e)
              unsafeAtomicAdd(a.Y + (size_t)e_bag[e] * D + col, e_w[e] * part);
          }
        }
      }
    }
  }
}

size_t fwd_lds_bytes(int RP) {
  switch (RP) {
    case 16: return FwdLds<16>::BYTES;
    case 32: return FwdLds<32>::BYTES;
    default: return FwdLds<64>::BYTES;
  }
}

template <int RP>
static hipError_t launch_fwd_t(const DevArgs &a, size_t lds, hipStream_t s) {
  static bool attr_set = false;  // dynamic LDS above 64 KiB is opt-in per kernel
  if (!attr_set) {
    (void)hipFuncSetAttribute((const void *)k_fwd<RP>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              160 * 1024);
    attr_set = true;
  }
  const int grid = a.T * a.p2 + (a.nnz + FWD_CHE - 1) / FWD_CHE;
  prof_begin(K_FWD, s);
  hipLaunchKernelGGL(k_fwd<RP>, dim3(grid), dim3(WG), lds, s, a);
  prof_end(K_FWD, s);
  return hipGetLastError();
}

hipError_t launch_fwd(const DevArgs &a, int RP, size_t lds, hipStream_t s) {
  switch (RP) {
    case 16: return launch_fwd_t<16>(a, lds, s);
    case 32: return launch_fwd_t<32>(a, lds, s);
    default: return launch_fwd_t<64>(a, lds, s);
  }
}

}  // namespace ttb
