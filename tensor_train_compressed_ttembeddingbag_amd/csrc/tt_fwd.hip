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
// One workgroup takes one work item: the elements of one (table, i2) group that
// fall in one P-aligned piece of the grouping order (at most 64; all of them share
// one G2 slice).  Stage 1 runs once per
// distinct (i1, i2) pair ("pair"), as a GEMM on the fp32 matrix cores:
//     T^T[r2][(pair, j1)] = sum_r1 G2[r1][j2][r2] * G1[i1(pair)][j1][r1]
// with the column block j2 of G2 in LDS (transposed to [r2][r1], double-buffered,
// the next block prefetched into registers during the MFMAs) and 16 (pair, j1)
// rows per "M-block" in the MFMA column dimension.  Stage 2 runs once per
// distinct index ("item") in VALU from the item's G3 slice staged in LDS, reducing
// over the four lane groups; each element of the item then adds w * row into out
// with fp32 atomics.  Bits of out may depend on the order of the atomics.
#include "tt_internal.h"
#include "tt_mfma.h"

namespace ttb {

template <int RP>
struct FwdLds {
  static constexpr int LD = RP + 4;
  static constexpr int G2F = 2 * RP * LD;  // floats: double-buffered G2 column block
  __host__ __device__ static size_t g3_floats(int q3) { return (size_t)ITEM_MAX * RP * q3; }
  static constexpr int INTS = 64 * 2 + 65 + 64 + 65 + 64 + 8;
  static size_t bytes(int q3) { return (G2F + g3_floats(q3)) * 4 + INTS * 4; }
};

template <int RP>
__global__ __launch_bounds__(WG) void k_fwd(DevArgs a) {
  constexpr int KS = RP / 4;   // k-steps: lane group g covers r1 = g*KS + ks
  constexpr int NM = RP / 16;  // 16-row blocks of r2
  constexpr int LD = FwdLds<RP>::LD;
  constexpr int KP = (RP * RP + WG - 1) / WG;  // G2 column-block floats per thread
  extern __shared__ float smem[];
  const int q1 = a.q1, q2 = a.q2, q3 = a.q3, R1 = a.R1, R2 = a.R2, D = a.D;
  float *sG2 = smem;
  float *sG3 = smem + FwdLds<RP>::G2F;                     // [item][RP][q3]
  int *e_bag = (int *)(sG3 + FwdLds<RP>::g3_floats(q3));  // [64]
  float *e_w = (float *)(e_bag + 64);                      // [64]
  int *it_beg = (int *)(e_w + 64);                         // [65]
  int *it_i3 = it_beg + 65;                                // [64]
  int *pr_it = it_i3 + 64;                                 // [65]
  int *pr_i1 = pr_it + 65;                                 // [64]
  int *s_cnt = pr_i1 + 64;                                 // [8]

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, c = lane & 15;
  const int wi = blockIdx.x;
  const int plan = a.hdr[H_PLAN], nitems = a.hdr[H_NFWD];
  const int4 item = a.fitem[wi];
  if (plan != (int)a.plan_fp || wi >= nitems) return;
  const int grp = item.x, s0 = item.y, s1 = item.z;
  const int n_el = s1 - s0;
  const int t = grp / a.p2, i2 = grp - t * a.p2;
  const size_t g2base = (size_t)(t * a.p2 + i2) * R1 * q2 * R2;
  const float *G3t = a.G3 + (size_t)t * a.p3 * R2 * q3;

  // G2 column block j2 -> registers (clamped addresses, zero padding)
  float pf[KP];
  auto fetch_g2 = [&](int j2) {
#pragma unroll
    for (int k = 0; k < KP; ++k) {
      const int i = tid + k * WG;
      const int r1 = i / RP, r2 = i - r1 * RP;
      const bool ok = i < RP * RP && r1 < R1 && r2 < R2;
      const float v = a.G2[g2base + ((size_t)(ok ? r1 : 0) * q2 + j2) * R2 + (ok ? r2 : 0)];
      pf[k] = ok ? v : 0.f;
    }
  };
  auto store_g2 = [&](float *buf) {
#pragma unroll
    for (int k = 0; k < KP; ++k) {
      const int i = tid + k * WG;
      if (i < RP * RP) {
        const int r1 = i / RP, r2 = i - r1 * RP;
        buf[r2 * LD + r1] = pf[k];
      }
    }
  };
  fetch_g2(0);
  if (tid < 64) {
    const int s = s0 + min(tid, n_el - 1);
    const bool v = tid < n_el;
    const int dAv = a.s_dA[s], dIv = a.s_dI3[s], bagv = a.s_bag[s];
    const float wv = a.s_w[s];
    const int dA = v ? dAv : -1, i3 = v ? dIv - t * a.p3 : -1;
    if (v) { e_bag[tid] = bagv; e_w[tid] = wv; }
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
  store_g2(sG2);
  __syncthreads();
  const int nI = s_cnt[0], nP = s_cnt[1];
  const int nmb = (nP * q1 + 15) / 16;

  // B operand of stage 1 (G1 rows of the wave's M-blocks), kept for all j2
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
      const float v = src[min(r1, R1 - 1)];
      bv[mbi][ks] = (ok && r1 < R1) ? v : 0.f;
    }
  }
  // the G3 slices of the chunk's items -> LDS [item][r2 < RP][j3] (zero padding),
  // STAGE_U loads in flight per thread
  {
    const int per_item = RP * q3, total = nI * per_item;
    for (int base = tid; base < total; base += WG * STAGE_U) {
      float v[STAGE_U];
#pragma unroll
      for (int u = 0; u < STAGE_U; ++u) {
        const int i = min(base + u * WG, total - 1);
        const int it = i / per_item, rem = i - it * per_item;
        const int r2 = rem / q3;
        v[u] = G3t[(size_t)it_i3[it] * R2 * q3 + (r2 < R2 ? rem : 0)];
      }
#pragma unroll
      for (int u = 0; u < STAGE_U; ++u) {
        const int i = base + u * WG;
        if (i < total) {
          const int rem = i % per_item;
          sG3[i] = (rem / q3 < R2) ? v[u] : 0.f;
        }
      }
    }
  }
  if (q2 > 1) fetch_g2(1);
  __syncthreads();

  for (int j2 = 0; j2 < q2; ++j2) {
    const float *buf = sG2 + (j2 & 1) * RP * LD;
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
        const float *g3 = sG3 + (size_t)(act ? it : 0) * RP * q3;
        float part[MAXQ3];
#pragma unroll
        for (int j3 = 0; j3 < MAXQ3; ++j3) {
          part[j3] = 0.f;
          if (j3 < q3) {
            float sacc = 0.f;
#pragma unroll
            for (int m = 0; m < NM; ++m)
#pragma unroll
              for (int v = 0; v < 4; ++v) sacc += acc[m][v] * g3[(16 * m + 4 * g + v) * q3 + j3];
            sacc += __shfl_xor(sacc, 16);
            sacc += __shfl_xor(sacc, 32);
            part[j3] = sacc;
          }
        }
        if (act) {
          const int colbase = (j1 * q2 + j2) * q3;
          for (int e = it_beg[it]; e < it_beg[it + 1]; ++e) {
            float *yrow = a.Y + (size_t)e_bag[e] * D + colbase;
            const float we = e_w[e];
#pragma unroll
            for (int j3 = 0; j3 < MAXQ3; ++j3)
              if (j3 < q3 && (j3 & 3) == g) unsafeAtomicAdd(yrow + j3, we * part[j3]);
          }
        }
      }
    }
    if (j2 + 1 < q2) {
      store_g2(sG2 + ((j2 + 1) & 1) * RP * LD);
      if (j2 + 2 < q2) fetch_g2(j2 + 2);
      __syncthreads();
    }
  }
}

size_t fwd_lds_bytes(int RP, int q3) {
  switch (RP) {
    case 16: return FwdLds<16>::bytes(q3);
    case 32: return FwdLds<32>::bytes(q3);
    default: return FwdLds<64>::bytes(q3);
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
  const int grid = items_max(a);
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
