// tt_bwd.hip -- backward TT contraction with fused SGD.
//
// "FBTT-Embedding" README, "Software Cache": the gradient of each core is a chain
// of matrix multiplications in reverse order; "Parameters" (`sparse`) and "Fused
// Kernel": the update is applied during the backward pass instead of returning
// gradients.  With G_u = sum over the elements n of index u of w_n * dY[bag n]
// (viewed as [j1][j2][j3]) and T the stage-1 product of u's (i1, i2) pair:
//   dT[j1][j2][r2]    = sum_{u in pair} sum_j3 G_u[j1][j2][j3] * G3[i3(u)][r2][j3]
//   dG3[i3][r2][j3]  += sum_{j1,j2} T[j1][j2][r2] * G_u[j1][j2][j3]        (per u)
//   dG2[i2][r1][j2][r2] += sum_{pairs, j1} G1[i1][j1][r1] * dT[j1][j2][r2]
//   dG1[i1][j1][r1]  += sum_{j2, r2} dT[j1][j2][r2] * G2[i2][r1][j2][r2]    (per pair)
// then G <- G - lr * dG on the touched slices.  Every sum has a fixed order, so the
// result is reproducible bit for bit (tensorflow/addons #2201 discusses the same
// concern for EmbeddingBag's dense gradient: sort, then accumulate without races).
//
// k_bwd: one workgroup per work item (the elements of one (table, i2) group inside
// one P-aligned piece of the grouping order; at most P <= 32 elements, so its
// (pair, j1) rows fit one 16-row M-block per wave).  Three dependent rounds of
// global loads -- the work item; its elements and G2 slice; the items' G3 slices,
// the pairs' G1 rows and the elements' dY rows -- and everything else runs from
// LDS and registers.  Per column block j2 of G2: recompute T (MFMA), form dT and
// the dG3 partial per item (VALU), accumulate dG2 (MFMA, K = the rows (pair, j1))
// and dG1 per pair (MFMA after an LDS transpose of dT).  dG2 is reduced over the 8
// waves in a fixed order into the work item's partial.  The dG1 / dG3 partials go
// to the workspace at the final-order position of their first element, and the
// links record where they are.  k_seg then sums every partial per slice in a fixed
// order and applies SGD: dG1 / dG3 in the (t,i1)- / (t,i3)-order, dG2 in
// work-item order.  With a cache, workgroups after the work items sum w * dY over the
// cache-hit runs (runsum_piece), beside the contraction.
#include <algorithm>

#include "tt_device.h"
#include "tt_mfma.h"

namespace ttb {

// LDS carve of one backward workgroup (float words, then int words)
template <int RP>
struct BwdLds {
  static constexpr int LD = RP + 4;
  static constexpr int INTS = META_INTS;
  // the dG2 reduction slots alias the dT transpose tiles and the w * dY staging
  __host__ __device__ static size_t red_floats(int nred, int P, int D) {
    size_t r = (size_t)nred * RP * LD;
    const size_t t = (size_t)NW * 16 * LD, y = (size_t)P * D;
    r = r > t ? r : t;
    return r > y ? r : y;
  }
  static size_t bytes(int JB, int P, int q3, int D, int nred) {
    return ((size_t)JB * RP * LD + red_floats(nred, P, D) + (size_t)P * D +
            2 * (size_t)P * q3 * RP) * 4 + INTS * 4;
  }
};

size_t bwd_lds_bytes(int RP, int JB, int P, int q3, int D, int nred) {
  switch (RP) {
    case 16: return BwdLds<16>::bytes(JB, P, q3, D, nred);
    case 32: return BwdLds<32>::bytes(JB, P, q3, D, nred);
    default: return BwdLds<64>::bytes(JB, P, q3, D, nred);
  }
}

// two workgroups per CU need <= 128 VGPRs (rank-64 tiles take one CU each).  F44: the
// instance for q1 = q3 = 4 (a lane group's four rows are one pair; each item's G3 / dG3
// rows of four j3 move as 16-byte LDS vectors); otherwise q1 and q3 come from the
// arguments.  HITS: the instance for calls with a
// cache, whose extra workgroups sum the cache-hit runs (an instance of its own, so that
// the register budget of the others is not shared with that path).
template <int RP, bool F44, bool HITS>
__global__ __launch_bounds__(WG) __attribute__((amdgpu_waves_per_eu(RP == 64 ? 2 : 4)))
void k_bwd(DevArgs a) {
  constexpr int Q3 = F44 ? 4 : 0;  // q3 fixed at compile time with q1 = q3 = 4
  constexpr int KS = RP / 4, NM = RP / 16, LD = BwdLds<RP>::LD, LRP = log2_rp<RP>();
  constexpr int JU = 2;  // j3 per batch of the item loop with a runtime q3 (register budget)
  extern __shared__ float4 smem4[];
  float *smem = (float *)smem4;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, c = lane & 15;
  const int q1 = a.q1, q2 = a.q2, q3 = Q3 ? Q3 : a.q3, R1 = a.R1, R2 = a.R2, D = a.D;
  const int JB = a.JBb, P = a.P, nred = a.NRED;
  float *sG2 = smem;                                              // [JB][r2 < RP][LD]
  float *sRed = sG2 + (size_t)JB * RP * LD;                       // slots / dT tiles / w*dY
  float *sT = sRed;
  float *sYe = sRed;
  float *sGu = sRed + BwdLds<RP>::red_floats(nred, P, D);         // [item][D]
  float *sG3 = sGu + (size_t)P * D;                               // [item][r2 < RP][j3]
  float *sdA3 = sG3 + (size_t)P * q3 * RP;                        // [item][r2 < RP][j3]
  int *s_meta = (int *)(sdA3 + (size_t)P * q3 * RP);              // [META_INTS]
  const WorkMeta &M = *(const WorkMeta *)s_meta;

  // workgroups past the work items' part of the grid: the cache-hit run sums, one wave
  // per 64-position piece (they need only the plan and grad_out, so they run beside the
  // contraction; the segment sums read their fragments after this launch)
  const int nwi = items_max(a);
  if (HITS && (int)blockIdx.x >= nwi) {
    if (a.hdr[H_PLAN] != (int)a.plan_fp) return;  // stale plan: k_seg reports it
    const int piece = ((int)blockIdx.x - nwi) * NW + (int)(threadIdx.x >> 6);
    runsum_piece(a, piece, (int)(threadIdx.x & 63));
    return;
  }
  // round 1: plan check and the work item's metadata (built by the grouping)
  const int wi = blockIdx.x;
  const int plan = a.hdr[H_PLAN], nitems = a.hdr[H_NFWD];
  __shared__ int s_pl[NW];
  if (tid < META_INTS) s_meta[tid] = a.meta[(size_t)wi * META_INTS + tid];
  note_placement(s_pl);
  lds_barrier();
  if (plan != (int)a.plan_fp || wi >= nitems) return;
  // the record's counts are the same for the whole workgroup: scalar registers
  const int grp = wave_uniform(M.grp), s0 = wave_uniform(M.s0), n_el = wave_uniform(M.n_el);
  const int nI = wave_uniform(M.nI), nP = wave_uniform(M.nP);
  const int t = wave_uniform(M.t);
  const size_t W1 = (size_t)q1 * R1, W3 = (size_t)R2 * q3;
  const size_t slice2 = (size_t)R1 * q2 * R2;
  const float *G2g = a.G2 + (size_t)grp * slice2;
  const float *G1t = a.G1 + (size_t)t * a.p1 * W1;
  const float *G3t = a.G3 + (size_t)t * a.p3 * W3;
  float *part2 = a.part2 + (size_t)wave_uniform(M.item) * slice2;  // keyed by the item

  // G2 columns [j0, j0 + nj) -> LDS as G2^T blocks, STAGE_U loads per thread per batch
  auto load2 = [&](int j0, int nj, int base, float *v) {
    const int total = nj * RP * RP;
#pragma unroll
    for (int u = 0; u < STAGE_U; ++u) {
      const int i = min(base + u * WG, total - 1);
      const int jj = i >> (2 * LRP), r1 = (i >> LRP) & (RP - 1), r2 = i & (RP - 1);
      const bool ok = r1 < R1 && r2 < R2;
      v[u] = G2g[((size_t)(ok ? r1 : 0) * q2 + j0 + jj) * R2 + (ok ? r2 : 0)];
    }
  };
  auto store2 = [&](int nj, int base, const float *v) {
    const int total = nj * RP * RP;
#pragma unroll
    for (int u = 0; u < STAGE_U; ++u) {
      const int i = base + u * WG;
      if (i < total) {
        const int jj = i >> (2 * LRP), r1 = (i >> LRP) & (RP - 1), r2 = i & (RP - 1);
        sG2[(size_t)jj * RP * LD + r2 * LD + r1] = (r1 < R1 && r2 < R2) ? v[u] : 0.f;
      }
    }
  };
  auto stage_g2 = [&](int j0, int nj, int first) {
    for (int base = first; base < nj * RP * RP; base += WG * STAGE_U) {
      float v[STAGE_U];
      load2(j0, nj, base, v);
      store2(nj, base, v);
    }
  };

  // round 2: the first G2 stage, the items' G3 slices (-> LDS, with the dG3 accumulators
  // cleared), the pairs' G1 rows in the two operand layouts and the elements' w * dY rows,
  // the first batch of everything in flight at once
  const int nj0 = min(JB, q2);
  const int nmb = (nP * q1 + 15) >> 4;
  // one M-block per wave (P * q1 <= 16 * NW), by the slot the grouping gave it
  const int mb = wave_uniform(M.mb_slot[placed_mblock<NW>(s_pl)]);
  const int per_item = RP * q3, total3 = nI * per_item, totalY = n_el * D;
  // i = (item * RP + r2) * q3 + j3 -> (item * RP + r2, j3)
  auto split3 = [&](int i, int &jr, int &j3) {
    jr = Q3 ? i / Q3 : fdiv(i, a.mq3);
    j3 = i - jr * q3;
  };
  auto load3 = [&](int base, float *v) {
#pragma unroll
    for (int u = 0; u < STAGE_U; ++u) {
      const int i = min(base + u * WG, total3 - 1);
      int jr, j3;
      split3(i, jr, j3);
      const int it = jr >> LRP, r2 = jr & (RP - 1);
      v[u] = G3t[M.it_i3[it] * (int)W3 + (r2 < R2 ? r2 : 0) * q3 + j3];
    }
  };
  auto store3 = [&](int base, const float *v) {
#pragma unroll
    for (int u = 0; u < STAGE_U; ++u) {
      const int i = base + u * WG;
      if (i < total3) {
        int jr, j3;
        split3(i, jr, j3);
        sG3[i] = (jr & (RP - 1)) < R2 ? v[u] : 0.f;
        sdA3[i] = 0.f;
      }
    }
  };
  auto loadY = [&](int base, float *v) {
#pragma unroll
    for (int u = 0; u < STAGE_U; ++u) {
      const int i = min(base + u * WG, totalY - 1);
      const int e = fdiv(i, a.mD), d = i - e * D;
      v[u] = a.dY[(size_t)M.e_bag[e] * D + d];
    }
  };
  auto storeY = [&](int base, const float *v) {
#pragma unroll
    for (int u = 0; u < STAGE_U; ++u) {
      const int i = base + u * WG;
      if (i < totalY) sYe[i] = M.e_w[fdiv(i, a.mD)] * v[u];
    }
  };
  float aT[KS];          // A1[row = 16mb + c][r1 = g*KS + ks]     (stage 1)
  float aG[4][NM];       // A1[row = 16mb + 4g + sr][r1 = 16mr + c] (dG2)
  // G1 rows of the wave's M-block: aT as 16-byte vectors when the ranks fill RP
  auto load_g1 = [&](bool vec) {
    if (F44) {
      // q1 = 4: row r of the M-block is j1 = r % 4 of pair 4 mb + r / 4, so lane group g's
      // rows 4g .. 4g+3 are the four j1 of pair 4 mb + g (offsets under 2^21: i1 < 2^13)
      const unsigned oA = __umul24((unsigned)M.pr_i1[min(mb * 4 + (c >> 2), nP - 1)] * 4u +
                                       (unsigned)(c & 3), (unsigned)R1);
      const unsigned oB = __umul24((unsigned)M.pr_i1[min(mb * 4 + g, nP - 1)] * 4u, (unsigned)R1);
      if (vec) {
#pragma unroll
        for (int k4 = 0; k4 < KS / 4; ++k4) {
          const float4 x = *(const float4 *)&G1t[oA + g * KS + 4 * k4];
          aT[4 * k4] = x.x; aT[4 * k4 + 1] = x.y; aT[4 * k4 + 2] = x.z; aT[4 * k4 + 3] = x.w;
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) aT[ks] = G1t[oA + min(g * KS + ks, R1 - 1)];
      }
#pragma unroll
      for (int sr = 0; sr < 4; ++sr)
#pragma unroll
        for (int mr = 0; mr < NM; ++mr) aG[sr][mr] = G1t[oB + sr * R1 + min(16 * mr + c, R1 - 1)];
      return;
    }
    const int row = mb * 16 + c;
    const int pr = row >> a.lq1, j1 = row & (q1 - 1);
    const float *src = G1t + ((size_t)M.pr_i1[min(pr, nP - 1)] * q1 + j1) * R1;
    if (vec) {
#pragma unroll
      for (int k4 = 0; k4 < KS / 4; ++k4) {
        const float4 x = *(const float4 *)&src[g * KS + 4 * k4];
        aT[4 * k4] = x.x; aT[4 * k4 + 1] = x.y; aT[4 * k4 + 2] = x.z; aT[4 * k4 + 3] = x.w;
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) aT[ks] = src[min(g * KS + ks, R1 - 1)];
    }
#pragma unroll
    for (int sr = 0; sr < 4; ++sr) {
      const int row2 = mb * 16 + 4 * g + sr;
      const int pr2 = row2 >> a.lq1, j12 = row2 & (q1 - 1);
      const float *src2 = G1t + ((size_t)M.pr_i1[min(pr2, nP - 1)] * q1 + j12) * R1;
#pragma unroll
      for (int mr = 0; mr < NM; ++mr) aG[sr][mr] = src2[min(16 * mr + c, R1 - 1)];
    }
  };
  const bool vec = F44 && R1 == RP && R2 == RP;
  const bool rep = n_el > nI;  // some index repeats in the work item
  if (vec) {
    // 16-byte loads throughout (ranks fill RP, q3 = 4, D a multiple of 4): G2 along r2,
    // an item's G3 slice as one (r2, four j3) vector per lane, and the dY rows along d.
    // When every element of the work item is a distinct index (the usual case) the weighted
    // row of each element is its item's G_u and goes straight to sGu; when an index repeats,
    // the weighted rows go to sYe in position order, every row in flight at once, and each
    // item's rows are summed after the barrier.  The number of memory instructions, not the
    // bytes, bounds this round.
    constexpr int SV = 2;
    float *sWY = rep ? sYe : sGu;
    const int n2 = nj0 * RP * RP / 4, n3 = nI * RP, D4 = D >> 2, nY = n_el * D4;
    // 32-bit offsets from the slices' bases (a G2 slice is under 2^18 floats, a G3 table
    // under 2^21 here)
    auto ld2 = [&](int i4) {
      const int jj = i4 >> (2 * LRP - 2), r1 = (i4 >> (LRP - 2)) & (RP - 1);
      const int r2 = (i4 & (RP / 4 - 1)) * 4;
      return *(const float4 *)&G2g[((__umul24((unsigned)r1, (unsigned)q2) + jj) << LRP) + r2];
    };
    auto st2 = [&](int i4, float4 x) {
      const int jj = i4 >> (2 * LRP - 2), r1 = (i4 >> (LRP - 2)) & (RP - 1);
      const int r2 = (i4 & (RP / 4 - 1)) * 4;
      float *d = &sG2[(size_t)jj * RP * LD + r2 * LD + r1];
      d[0] = x.x; d[LD] = x.y; d[2 * LD] = x.z; d[3 * LD] = x.w;
    };
    auto ld3 = [&](int i4) {
      return *(const float4 *)&G3t[((unsigned)M.it_i3[i4 >> LRP] << (LRP + 2)) +
                                   (i4 & (RP - 1)) * 4];  // (W3 = 4 RP)
    };
    // vector i4 = (q, d4): row q of sWY -- element q in position order, or, with no repeated
    // index, item q (whose one element sits at item-major slot q)
    auto row_of = [&](int i4) { return fdiv(i4 << 2, a.mD); };  // i4 / D4 (4 i4 < P D < 2^16)
    auto elem_of = [&](int i4) {
      const int q = row_of(i4);
      return rep ? q : (int)M.e_perm[q];
    };
    auto ldY = [&](int i4, int e) {
      const int d4 = i4 - (int)__umul24((unsigned)row_of(i4), (unsigned)D4);
      return *(const float4 *)&a.dY[(size_t)M.e_bag[e] * D + d4 * 4];
    };
    auto stY = [&](int i4, int e, float4 y) {
      const float w = M.e_w[e];
      *(float4 *)&sWY[4 * i4] = make_float4(w * y.x, w * y.y, w * y.z, w * y.w);
    };
    float4 v2[SV], v3[SV], vy[SV];
    int ey[SV];
#pragma unroll
    for (int u = 0; u < SV; ++u) {
      const int iy = min(tid + u * WG, nY - 1);
      ey[u] = elem_of(iy);
      v2[u] = ld2(min(tid + u * WG, n2 - 1));
      v3[u] = ld3(min(tid + u * WG, n3 - 1));
      vy[u] = ldY(iy, ey[u]);
    }
    load_g1(true);
    const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int u = 0; u < SV; ++u) {
      const int i4 = tid + u * WG;
      if (i4 < n2) st2(i4, v2[u]);
      if (i4 < n3) {
        *(float4 *)&sG3[4 * i4] = v3[u];
        *(float4 *)&sdA3[4 * i4] = z4;
      }
      if (i4 < nY) stY(i4, ey[u], vy[u]);
    }
    for (int i4 = tid + SV * WG; i4 < n2; i4 += WG) st2(i4, ld2(i4));
    for (int i4 = tid + SV * WG; i4 < n3; i4 += WG) {
      *(float4 *)&sG3[4 * i4] = ld3(i4);
      *(float4 *)&sdA3[4 * i4] = z4;
    }
    for (int i4 = tid + SV * WG; i4 < nY; i4 += WG) {
      const int e = elem_of(i4);
      stY(i4, e, ldY(i4, e));
    }
  } else {
    float v2[STAGE_U], v3[STAGE_U], vy[STAGE_U];
    load2(0, nj0, tid, v2);
    load3(tid, v3);
    loadY(tid, vy);
    load_g1(false);
    store2(nj0, tid, v2);
    stage_g2(0, nj0, tid + WG * STAGE_U);
    store3(tid, v3);
    storeY(tid, vy);
    for (int base = tid + WG * STAGE_U; base < total3; base += WG * STAGE_U) {
      float v[STAGE_U];
      load3(base, v);
      store3(base, v);
    }
    for (int base = tid + WG * STAGE_U; base < totalY; base += WG * STAGE_U) {
      float v[STAGE_U];
      loadY(base, v);
      storeY(base, v);
    }
  }
  {
    const int row = mb * 16 + c;
    const bool ok = mb < nmb && (row >> a.lq1) < nP;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const float x = keep(aT[ks]);
      aT[ks] = (ok && g * KS + ks < R1) ? x : 0.f;
    }
#pragma unroll
    for (int sr = 0; sr < 4; ++sr) {
      const int row2 = mb * 16 + 4 * g + sr;
      const bool ok2 = mb < nmb && (row2 >> a.lq1) < nP;
#pragma unroll
      for (int mr = 0; mr < NM; ++mr) {
        const float x = keep(aG[sr][mr]);
        aG[sr][mr] = (ok2 && 16 * mr + c < R1) ? x : 0.f;
      }
    }
  }
  vmem_drain();
  lds_barrier();
  if (!vec || rep) {
    // G_u of every item: its elements' w * dY rows summed in position order
    for (int i = tid; i < nI * D; i += WG) {
      const int it = fdiv(i, a.mD), d = i - it * D;
      float acc = 0.f;
      for (int k = M.it_beg[it]; k < M.it_beg[it + 1]; ++k)
        acc += sYe[(size_t)M.e_perm[k] * D + d];
      sGu[i] = acc;
    }
    lds_barrier();
  }

  f4 dA1[NM];  // dG1^T[r1 = 16mr + 4g + v][row = c]
#pragma unroll
  for (int mr = 0; mr < NM; ++mr) dA1[mr] = zero4();
  const int rb = mb * 16 + 4 * g;  // the lane group's rows rb .. rb+3
  int j1v[4], prv[4];              // their j1 and pair
#pragma unroll
  for (int v = 0; v < 4; ++v) { j1v[v] = (rb + v) & (q1 - 1); prv[v] = (rb + v) >> a.lq1; }
  const int plo = rb >> a.lq1, phi = min((rb + 3) >> a.lq1, nP - 1);
  const int ib = (mb < nmb && plo < nP) ? M.pr_it[plo] : 0;
  const int ie = (mb < nmb && plo < nP) ? M.pr_it[phi + 1] : 0;
  const int nk = mb < nmb ? M.mbb[mb] : 0;

  for (int j0 = 0; j0 < q2; j0 += JB) {
    if (j0 > 0) {  // next G2 stage (only when the slice does not fit at once)
      lds_barrier();
      stage_g2(j0, min(JB, q2 - j0), tid);
      vmem_drain();
      lds_barrier();
    }
    const int jend = min(q2, j0 + JB);
    // stage 1 of column j2: T[row = 16mb + 4g + v][r2 = 16m + c] (the first product starts
    // from 0).  It runs one column ahead: the products of column j2 + 1 are issued before
    // the reduction of column j2, so the matrix cores work through its barriers.
    auto stage1 = [&](int j2, f4 *T) {
      const float *bufj = sG2 + (size_t)(j2 - j0) * RP * LD;
#pragma unroll
      for (int kq = 0; kq < KS / 4; ++kq)
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          const float4 bv = *(const float4 *)&bufj[(16 * m + c) * LD + g * KS + 4 * kq];
          T[m] = mfma4(aT[4 * kq + 0], bv.x, kq == 0 ? zero4() : T[m]);
          T[m] = mfma4(aT[4 * kq + 1], bv.y, T[m]);
          T[m] = mfma4(aT[4 * kq + 2], bv.z, T[m]);
          T[m] = mfma4(aT[4 * kq + 3], bv.w, T[m]);
        }
    };
    f4 Tn[NM];
    if (mb < nmb) stage1(j0, Tn);
    for (int j2 = j0; j2 < jend; ++j2) {
      const float *buf = sG2 + (size_t)(j2 - j0) * RP * LD;
      f4 gacc[NM][NM];  // dG2[r1 = 16mr + 4g + v][r2 = 16m2 + c]
      if (mb < nmb) {
        f4 T[NM], dT[NM];
#pragma unroll
        for (int m = 0; m < NM; ++m) { T[m] = Tn[m]; dT[m] = zero4(); }
        // the items of the pairs owning the lane group's rows
        if (F44) {
          // q1 = q3 = 4: a lane group's four rows are one pair (j1 = v); each lane group
          // runs its own pair's items (inactive lanes simply sit out), all four j3 of an
          // item's G_u, G3 and dG3 rows as 16-byte vectors
          for (int kk = 0; kk < nk; ++kk) {
            const int it = ib + kk;
            if (it < ie) {
              const float *g3 = sG3 + (size_t)it * per_item + c * 4;  // + 64 m
              const float *gu = sGu + (size_t)it * D + j2 * 4;        // + 4 q2 j1
              float *da3 = sdA3 + (size_t)it * per_item + c * 4;
              float4 gx[4];
#pragma unroll
              for (int v = 0; v < 4; ++v) gx[v] = *(const float4 *)&gu[v * q2 * 4];
#pragma unroll
              for (int m = 0; m < NM; ++m) {
                const float4 a3 = *(const float4 *)&g3[64 * m];
                float4 d3 = *(const float4 *)&da3[64 * m];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                  d3.x = fmaf(T[m][v], gx[v].x, d3.x);
                  d3.y = fmaf(T[m][v], gx[v].y, d3.y);
                  d3.z = fmaf(T[m][v], gx[v].z, d3.z);
                  d3.w = fmaf(T[m][v], gx[v].w, d3.w);
                  dT[m][v] = fmaf(gx[v].x, a3.x, dT[m][v]);
                  dT[m][v] = fmaf(gx[v].y, a3.y, dT[m][v]);
                  dT[m][v] = fmaf(gx[v].z, a3.z, dT[m][v]);
                  dT[m][v] = fmaf(gx[v].w, a3.w, dT[m][v]);
                }
                *(float4 *)&da3[64 * m] = d3;
              }
            }
          }
        } else {
          for (int kk = 0; kk < nk; ++kk) {
            const int it = ib + kk;
            const bool act = it < ie;
            const int itc = act ? it : 0;
            const int pr = act ? M.it_pair[itc] : -1;
            const float *g3 = sG3 + (size_t)itc * per_item + c * q3;  // + 16 m q3 + j3
            const float *gu = sGu + (size_t)itc * D;
            float *da3 = sdA3 + (size_t)itc * per_item + c * q3;
            // JU j3 at a time: all LDS reads of the block first, then the arithmetic,
            // then the updated dG3 partials (one writer lane per element); rows of
            // another pair (q1 < 4: a lane group spans several pairs) get weight 0
            float mk[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) mk[v] = (act && prv[v] == pr) ? 1.f : 0.f;
            for (int j30 = 0; j30 < q3; j30 += JU) {
              float gx[JU][4], a3[JU][NM], d3[JU][NM];
#pragma unroll
              for (int u = 0; u < JU; ++u) {
                const int j3 = min(j30 + u, q3 - 1);
#pragma unroll
                for (int v = 0; v < 4; ++v)
                  gx[u][v] = mk[v] * gu[((j1v[v]) * q2 + j2) * q3 + j3];
#pragma unroll
                for (int m = 0; m < NM; ++m) {
                  a3[u][m] = g3[16 * m * q3 + j3];
                  d3[u][m] = da3[16 * m * q3 + j3];
                }
              }
#pragma unroll
              for (int u = 0; u < JU; ++u) {
                const bool ok3 = j30 + u < q3;
#pragma unroll
                for (int m = 0; m < NM; ++m) {
                  float sacc = 0.f;
#pragma unroll
                  for (int v = 0; v < 4; ++v) {
                    const float gv = ok3 ? gx[u][v] : 0.f;
                    sacc += T[m][v] * gv;
                    dT[m][v] += gv * a3[u][m];
                  }
                  d3[u][m] += sacc;
                }
              }
              if (act) {
#pragma unroll
                for (int u = 0; u < JU; ++u)
                  if (j30 + u < q3)
#pragma unroll
                    for (int m = 0; m < NM; ++m) da3[16 * m * q3 + j30 + u] = d3[u][m];
              }
            }
          }
        }
        // dG2 += A1^T dT   (K = the 16 rows; lane group g feeds rows 4g + sr)
#pragma unroll
        for (int sr = 0; sr < 4; ++sr)
#pragma unroll
          for (int mr = 0; mr < NM; ++mr)
#pragma unroll
            for (int m2 = 0; m2 < NM; ++m2)
              gacc[mr][m2] = mfma4(aG[sr][mr], dT[m2][sr], sr == 0 ? zero4() : gacc[mr][m2]);
        // dG1^T += G2_j2 dT^T  (K = r2; dT transposed through the wave's LDS tile)
        float *tt = sT + (size_t)w * 16 * LD;
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int v = 0; v < 4; ++v) tt[(4 * g + v) * LD + 16 * m + c] = dT[m][v];
        wave_lds_sync();
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          const float4 bT = *(const float4 *)&tt[c * LD + 16 * m + 4 * g];
#pragma unroll
          for (int mr = 0; mr < NM; ++mr) {
            dA1[mr] = mfma4(buf[(16 * m + 4 * g + 0) * LD + 16 * mr + c], bT.x, dA1[mr]);
            dA1[mr] = mfma4(buf[(16 * m + 4 * g + 1) * LD + 16 * mr + c], bT.y, dA1[mr]);
            dA1[mr] = mfma4(buf[(16 * m + 4 * g + 2) * LD + 16 * mr + c], bT.z, dA1[mr]);
            dA1[mr] = mfma4(buf[(16 * m + 4 * g + 3) * LD + 16 * mr + c], bT.w, dA1[mr]);
          }
        }
        if (j2 + 1 < jend) stage1(j2 + 1, Tn);
      } else {
#pragma unroll
        for (int mr = 0; mr < NM; ++mr)
#pragma unroll
          for (int m2 = 0; m2 < NM; ++m2) gacc[mr][m2] = zero4();
      }
      // reduce dG2 over the waves in M-block order (the order does not depend on which
      // wave holds which M-block, so the sum is reproducible): M-block mb adds into slot
      // mb % nred in round mb / nred, then the slots are summed in slot order.  A slot holds
      // [r2][r1] (row pitch LD), so a lane's four r1 = 16mr + 4g .. +3 of one r2 move as
      // one 16-byte vector.
      lds_barrier();  // the transpose tiles (aliased by the slots) are free
      const int nsl = min(nmb, nred);  // slots in use
      // (only the M-blocks with rows take part: the first min(nmb, nred) slots, and a round
      // only when an M-block has it; nmb is the workgroup's)
      for (int rr = 0; rr < NW / nred && rr * nred < nmb; ++rr) {
        if (mb / nred == rr && mb < nmb) {
          float *slot = sRed + (size_t)(mb % nred) * RP * LD;
          // the slot's partial sums of one row of tiles (all of them up to RP = 32) read
          // before any is written
          constexpr int MRB = NM <= 2 ? NM : 1;
#pragma unroll
          for (int mr0 = 0; mr0 < NM; mr0 += MRB) {
            float4 o[MRB][NM];
            if (rr > 0)
#pragma unroll
              for (int mr = 0; mr < MRB; ++mr)
#pragma unroll
                for (int m2 = 0; m2 < NM; ++m2)
                  o[mr][m2] = *(const float4 *)&slot[(16 * m2 + c) * LD + 16 * (mr0 + mr) + 4 * g];
#pragma unroll
            for (int mr = 0; mr < MRB; ++mr)
#pragma unroll
              for (int m2 = 0; m2 < NM; ++m2) {
                const f4 &ga = gacc[mr0 + mr][m2];
                float4 x = make_float4(ga[0], ga[1], ga[2], ga[3]);
                if (rr > 0) {
                  x.x += o[mr][m2].x; x.y += o[mr][m2].y; x.z += o[mr][m2].z; x.w += o[mr][m2].w;
                }
                *(float4 *)&slot[(16 * m2 + c) * LD + 16 * (mr0 + mr) + 4 * g] = x;
              }
          }
        }
        lds_barrier();
      }
      // thread t: r2 = t mod RP, r1 = 4 (t / RP) .. +3, summed over the slots in order (all
      // slots read at once); the partial keeps the slice layout [r1][j2][r2] (consecutive
      // threads, consecutive r2; offsets inside the slice fit 32 bits)
      for (int t4 = tid; t4 < RP * RP / 4; t4 += WG) {
        const int r2 = t4 & (RP - 1), r1 = (t4 >> LRP) * 4;
        constexpr int KF = F44 ? 4 : 1;  // slots in flight (the F44 instances have the room)
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int k0 = 0; k0 < nsl; k0 += KF) {
          float4 o[KF];
#pragma unroll
          for (int k = 0; k < KF; ++k)
            if (k0 + k < nsl)
              o[k] = *(const float4 *)&sRed[(size_t)(k0 + k) * RP * LD + r2 * LD + r1];
#pragma unroll
          for (int k = 0; k < KF; ++k)
            if (k0 + k < nsl) {
              if (k0 + k == 0) acc = o[0];
              else { acc.x += o[k].x; acc.y += o[k].y; acc.z += o[k].z; acc.w += o[k].w; }
            }
        }
        const unsigned st = (unsigned)(q2 * R2);
        float *dst = part2 + (__umul24((unsigned)r1, (unsigned)q2) + j2) * (unsigned)R2 + r2;
        if (R1 == RP && R2 == RP) {  // (every r1, r2 of the slot is in the slice)
          dst[0] = acc.x; dst[st] = acc.y; dst[2 * st] = acc.z; dst[3 * st] = acc.w;
        } else if (r2 < R2) {
          if (r1 + 0 < R1) dst[0] = acc.x;
          if (r1 + 1 < R1) dst[st] = acc.y;
          if (r1 + 2 < R1) dst[2 * st] = acc.z;
          if (r1 + 3 < R1) dst[3 * st] = acc.w;
        }
      }
      lds_barrier();
    }
  }
  // dG1 partial per pair, dG3 partial per item, at their first positions
  if (mb < nmb) {
    const int row = mb * 16 + c;
    const int pr = row >> a.lq1, j1 = row & (q1 - 1);
    if (pr < nP) {
      float *dst = a.part1 + (size_t)(s0 + M.it_first[M.pr_it[pr]]) * W1 + (size_t)j1 * R1;
#pragma unroll
      for (int mr = 0; mr < NM; ++mr) {
        if (vec) {  // four r1 of the lane as one 16-byte store (R1 = RP)
          *(float4 *)&dst[16 * mr + 4 * g] =
              make_float4(dA1[mr][0], dA1[mr][1], dA1[mr][2], dA1[mr][3]);
        } else {
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int r1 = 16 * mr + 4 * g + v;
            if (r1 < R1) dst[r1] = dA1[mr][v];
          }
        }
      }
    }
  }
  if (vec) {  // q3 = 4, R2 = RP: an (item, r2) row of four j3 per 16-byte store
    for (int i4 = tid; i4 < total3 / 4; i4 += WG) {
      const int it = i4 >> LRP, r2 = i4 & (RP - 1);
      *(float4 *)&a.part3[(size_t)(s0 + M.it_first[it]) * W3 + r2 * 4] =
          *(const float4 *)&sdA3[4 * i4];
    }
  } else {
    for (int i = tid; i < total3; i += WG) {  // i = (item * RP + r2) * q3 + j3
      int jr, j3;
      split3(i, jr, j3);
      const int it = jr >> LRP, r2 = jr & (RP - 1);
      if (r2 < R2) a.part3[(size_t)(s0 + M.it_first[it]) * W3 + r2 * q3 + j3] = sdA3[i];
    }
  }
}

template <int RP, bool F44, bool HITS>
static hipError_t launch_bwd_k(const DevArgs &a, size_t lds, hipStream_t s) {
  static bool attr_set = false;  // dynamic LDS above 64 KiB is opt-in per kernel
  if (!attr_set) {
    (void)hipFuncSetAttribute((const void *)k_bwd<RP, F44, HITS>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, LDS_DYN_MAX);
    attr_set = true;
  }
  // with a cache, extra workgroups (eight 64-position pieces each) sum the hit runs
  const int pieces = HITS ? (a.nnz + PIECE - 1) / PIECE : 0;
  const int grid = items_max(a) + (pieces + NW - 1) / NW;
  tt_launch(K_BWD, k_bwd<RP, F44, HITS>, dim3(grid), dim3(WG), lds, s, a);
  return hipGetLastError();
}

template <int RP, bool F44>
static hipError_t launch_bwd_t(const DevArgs &a, size_t lds, hipStream_t s) {
  return a.has_cache ? launch_bwd_k<RP, F44, true>(a, lds, s)
                     : launch_bwd_k<RP, F44, false>(a, lds, s);
}

template <bool F44>
static hipError_t launch_bwd_q(const DevArgs &a, int RP, size_t lds, hipStream_t s) {
  switch (RP) {
    case 16: return launch_bwd_t<16, F44>(a, lds, s);
    case 32: return launch_bwd_t<32, F44>(a, lds, s);
    default: return launch_bwd_t<64, F44>(a, lds, s);
  }
}

hipError_t launch_bwd(const DevArgs &a, int RP, size_t lds, hipStream_t s) {
  return (a.q1 == 4 && a.q3 == 4) ? launch_bwd_q<true>(a, RP, lds, s)
                                  : launch_bwd_q<false>(a, RP, lds, s);
}

// ---------------------------------------------------------------- k_seg
// Blocks of 256 threads, three kinds of task:
//  * one block = one core-1 slice (t, i1) or core-3 slice (t, i3): the slice's segment
//    of the (t,i1)- / (t,i3)-ordered element list names, through the links, the final-
//    order positions of its partials; they are listed in segment order (up to 1024
//    positions per pass), then summed by 8 row groups (row group k takes the pass's rows
//    k, k+8, ...; a fixed assignment), the group sums added in group order, and SGD
//    applied;
//  * one block = one column chunk of a core-2 slice (t, i2): the dG2 partials of the
//    group's work items are summed in item order, then the update;
//  * four waves = four 64-position pieces of the cache-hit region: a cache run (one
//    slot) is finished by the piece that holds its first position, which sums the
//    run's fragments (its first position, then every piece start inside the run) in
//    position order.
constexpr int SEG_T = 256;
constexpr int SEG_ROWS = 4;   // partial rows in flight per thread
constexpr int SEG_LPT = 4;    // core-1/3 slices: links per thread per pass
constexpr int SEG_CW = 4;     // core-2 slices: columns per thread,
constexpr int SEG_IB = 8;     // work items in flight,
constexpr int SEG_COLS = SEG_T * SEG_CW;  // and columns per block
__host__ __device__ inline int seg_chunks(const DevArgs &a) {
  return (a.R1 * a.q2 * a.R2 + SEG_COLS - 1) / SEG_COLS;
}

template <int UPD>
__global__ __launch_bounds__(SEG_T) void k_seg(DevArgs a) {
  __shared__ int s_rows[SEG_T * SEG_LPT];
  __shared__ int s_wc[SEG_LPT][SEG_T / 64];
  __shared__ float s_red[SEG_T * 4];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int nA = a.T * a.p1, nC = a.T * a.p3, G = a.T * a.p2;
  const int bid = blockIdx.x;
  // the plan check and the task's first loads go out together
  const bool one = bid < nA;
  const int seg = one ? bid : bid - nA;
  const int *seg_start = one ? a.segA : a.segI3;
  const int nch = seg_chunks(a);
  const int gi = min(max(bid - nA - nC, 0) / nch, G - 1);
  const int plan = a.hdr[H_PLAN];
  const int beg = seg_start[min(seg, one ? nA : nC)], end = seg_start[min(seg + 1, one ? nA : nC)];
  const int i0 = a.chunk_pre[gi], i1 = a.chunk_pre[gi + 1];
  if (plan != (int)a.plan_fp) {  // the workspace holds another call's plan
    if (bid == 0 && tid == 0) set_status(a.status, DEV_STALE_PLAN);
    return;
  }
  if (bid < nA + nC) {
    const int *link = one ? a.link1 : a.link3;
    const float *part = one ? a.part1 : a.part3;
    const int W = one ? a.q1 * a.R1 : a.R2 * a.q3;
    float *dst = one ? a.G1 + (size_t)seg * W : a.G3 + (size_t)seg * W;
    float *aux = one ? a.X1 + (size_t)seg * W : a.X3 + (size_t)seg * W;
    // the values the update reads, loaded beside the segment bounds (thread t: column t
    // of the first column block, where the update puts thread t)
    float x_pre = 0.f, aux_pre = 0.f;
    if (tid < W) {
      if (UPD != UPD_GRAD) x_pre = dst[tid];
      if (UPD == UPD_ADAGRAD) aux_pre = aux[tid];
    }
    if (beg >= end) {  // an untouched slice: a zero gradient, no update
      if (UPD == UPD_GRAD)
        for (int c = tid; c < W; c += SEG_T) aux[c] = 0.f;
      return;
    }
    // columns: 4 per lane when W allows 16-byte rows, lanes per row LPR, row groups NRG
    const int VEC = (W & 3) == 0 ? 4 : 1;
    const int LPR = min(SEG_T, (W + VEC - 1) / VEC), NRG = SEG_T / LPR;
    const int rg = tid / LPR, cl = tid - rg * LPR;
    for (int c0 = 0; c0 < W; c0 += LPR * VEC) {  // column blocks (one unless W > 1024)
      const int col = c0 + cl * VEC;
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
      for (int p0 = beg; p0 < end; p0 += SEG_T * SEG_LPT) {
        // the pass's partial rows, in segment order (thread t takes positions
        // p0 + u SEG_T + t, all loads of the pass in flight at once)
        int lk[SEG_LPT];
#pragma unroll
        for (int u = 0; u < SEG_LPT; ++u) {
          const int p = p0 + u * SEG_T + tid;
          lk[u] = p < end ? link[p] : -1;
        }
        const unsigned long long lt = (1ull << lane) - 1ull;
        unsigned long long m[SEG_LPT];
#pragma unroll
        for (int u = 0; u < SEG_LPT; ++u) {
          m[u] = __ballot(lk[u] >= 0);
          if (lane == 0) s_wc[u][w] = __popcll(m[u]);
        }
        __syncthreads();
        int n = 0;
#pragma unroll
        for (int u = 0; u < SEG_LPT; ++u) {
          int before = n, tot = 0;
          for (int v = 0; v < SEG_T / 64; ++v) {
            before += v < w ? s_wc[u][v] : 0;
            tot += s_wc[u][v];
          }
          if (lk[u] >= 0) s_rows[before + __popcll(m[u] & lt)] = lk[u];
          n += tot;
        }
        __syncthreads();
        if (rg < NRG && col < W) {
          for (int k0 = rg; k0 < n; k0 += NRG * SEG_ROWS) {
            float4 v[SEG_ROWS];
#pragma unroll
            for (int u = 0; u < SEG_ROWS; ++u) {
              v[u] = make_float4(0.f, 0.f, 0.f, 0.f);
              if (k0 + u * NRG < n) {  // only the rows there are
                const float *row = part + (size_t)s_rows[k0 + u * NRG] * W + col;
                if (VEC == 4) v[u] = *(const float4 *)row;
                else v[u].x = row[0];
              }
            }
#pragma unroll
            for (int u = 0; u < SEG_ROWS; ++u)
              if (k0 + u * NRG < n) {
                acc[0] += v[u].x; acc[1] += v[u].y; acc[2] += v[u].z; acc[3] += v[u].w;
              }
          }
        }
        __syncthreads();
      }
      // row groups summed in group order, then the update
      if (rg < NRG)
#pragma unroll
        for (int j = 0; j < 4; ++j) s_red[(rg * LPR + cl) * 4 + j] = acc[j];
      __syncthreads();
      for (int t2 = tid; t2 < LPR * VEC; t2 += SEG_T) {
        const int c = c0 + t2;
        float sum = 0.f;
        for (int r = 0; r < NRG; ++r) sum += s_red[(r * LPR + t2 / VEC) * 4 + t2 % VEC];
        if (c < W) {
          const bool pre = c == tid;  // (the first column block)
          apply_update<UPD>(a, dst, aux, c, sum,
                            UPD == UPD_GRAD ? 0.f : (pre ? x_pre : dst[c]),
                            UPD == UPD_ADAGRAD ? (pre ? aux_pre : aux[c]) : 0.f);
        }
      }
      __syncthreads();
    }
    return;
  }
  if (bid < nA + nC + G * nch) {
    // one column chunk of one core-2 slice: SEG_COLS columns, SEG_CW per thread, the
    // values the update reads and SEG_IB items' partials in flight; items summed in
    // item order
    const int g = gi, c0 = (bid - nA - nC - g * nch) * SEG_COLS + tid;
    const int slice2 = a.R1 * a.q2 * a.R2;  // <= 64 * 64 * 64
    float *dst = a.G2 + (size_t)g * slice2, *aux = a.X2 + (size_t)g * slice2;
    if (i0 >= i1) {  // an untouched slice: a zero gradient, no update
      if (UPD == UPD_GRAD)
#pragma unroll
        for (int u = 0; u < SEG_CW; ++u)
          if (c0 + u * SEG_T < slice2) aux[c0 + u * SEG_T] = 0.f;
      return;
    }
    float acc[SEG_CW], old[SEG_CW], oaux[SEG_CW];
#pragma unroll
    for (int u = 0; u < SEG_CW; ++u) {
      acc[u] = 0.f;
      const int e = min(c0 + u * SEG_T, slice2 - 1);
      old[u] = UPD != UPD_GRAD ? dst[e] : 0.f;
      oaux[u] = UPD == UPD_ADAGRAD ? aux[e] : 0.f;
    }
    for (int it0 = i0; it0 < i1; it0 += SEG_IB) {
      float v[SEG_IB][SEG_CW];
#pragma unroll
      for (int k = 0; k < SEG_IB; ++k) {
        if (it0 + k < i1) {  // (uniform: only the items there are)
          const float *src = a.part2 + (size_t)(it0 + k) * slice2;
#pragma unroll
          for (int u = 0; u < SEG_CW; ++u) v[k][u] = src[min(c0 + u * SEG_T, slice2 - 1)];
        }
      }
#pragma unroll
      for (int k = 0; k < SEG_IB; ++k)
        if (it0 + k < i1)
#pragma unroll
          for (int u = 0; u < SEG_CW; ++u) acc[u] += v[k][u];
    }
#pragma unroll
    for (int u = 0; u < SEG_CW; ++u)
      if (c0 + u * SEG_T < slice2)
        apply_update<UPD>(a, dst, aux, c0 + u * SEG_T, acc[u], old[u], oaux[u]);
    return;
  }
  if (!a.has_cache) return;
  // cache hits: the wave's piece of the hit region; run starts from one load per lane
  const int k = (bid - nA - nC - G * nch) * 4 + w;
  const int hb = a.hdr[H_HIT_BEG], he = a.hdr[H_HIT_END];
  const int lo = max(k * PIECE, hb), hi = min((k + 1) * PIECE, he);
  if (lo >= hi) return;
  const int sl = min(lo + lane, hi - 1);
  const int4 cur = a.srec[2 * (size_t)sl], prev = a.srec[2 * (size_t)max(sl - 1, 0)];
  const bool st = lo + lane < hi && (sl == hb || prev.y != cur.y || prev.z != cur.z);
  unsigned long long starts = __ballot(st);
  // every run but the piece's last one ends inside the piece (one fragment): four of them
  // at a time, lane group q = lane / 16 takes run q and its 16 lanes the columns
  if (starts) {
    const int lastl = 63 - __clzll((long long)starts);
    unsigned long long early = starts & ~(1ull << lastl);
    starts = 1ull << lastl;
    const int q = lane >> 4, cq = lane & 15;
    while (early) {
      int lq = -1;
      for (int k = 0; k < 4 && early; ++k) {
        const int l = __ffsll((long long)early) - 1;
        early &= early - 1ull;
        if (k == q) lq = l;
      }
      const int l = lq >= 0 ? lq : 0;
      const int kA = __shfl(cur.y, l), kB = __shfl(cur.z, l);
      if (lq < 0) continue;
      const int s0 = lo + l;
      const int slot = (kB - a.T * a.p2) * HB + (kA - a.T * a.p1);
      for (int c0 = cq; c0 < a.D; c0 += 64) {  // 4 columns of 16 lanes in flight
        float fv[4], xv[4], av[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int c = min(c0 + 16 * k, a.D - 1);
          const size_t e = (size_t)slot * a.D + c;
          fv[k] = a.frag[(size_t)s0 * a.D + c];
          xv[k] = UPD == UPD_GRAD ? 0.f : a.crows[e];
          av[k] = UPD == UPD_ADAGRAD ? a.Xc[e] : 0.f;
        }
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (c0 + 16 * k < a.D)
            apply_update<UPD>(a, a.crows, a.Xc, (size_t)slot * a.D + c0 + 16 * k, fv[k], xv[k],
                              av[k]);
      }
    }
  }
  while (starts) {  // the last run: it may continue into the next pieces
    const int l = __ffsll((long long)starts) - 1;
    starts &= starts - 1ull;
    const int s0 = lo + l;
    const int kA = __shfl(cur.y, l), kB = __shfl(cur.z, l);
    const int slot = (kB - a.T * a.p2) * HB + (kA - a.T * a.p1);
    // the run's fragments: s0, then every piece start inside the run (runsum_piece);
    // their number, 64 piece starts per round
    const int pb = (s0 / PIECE + 1) * PIECE;
    int nfr = 0;
    for (;;) {
      const int pj = pb + (nfr + lane) * PIECE;
      bool in = pj < he;
      if (in) {
        const int4 q = a.srec[2 * (size_t)pj];
        in = q.y == kA && q.z == kB;
      }
      const unsigned long long out = __ballot(!in);
      if (out) { nfr += __ffsll((long long)out) - 1; break; }
      nfr += 64;
    }
    for (int d = lane; d < a.D; d += 64) {
      float acc = a.frag[(size_t)s0 * a.D + d];
      for (int j0 = 0; j0 < nfr; j0 += 16) {  // 16 fragments in flight, summed in order
        float v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u)
          v[u] = a.frag[(size_t)(pb + min(j0 + u, nfr - 1) * PIECE) * a.D + d];
#pragma unroll
        for (int u = 0; u < 16; ++u)
          if (j0 + u < nfr) acc += v[u];
      }
      const size_t e = (size_t)slot * a.D + d;
      apply_update<UPD>(a, a.crows, a.Xc, e, acc, UPD == UPD_GRAD ? 0.f : a.crows[e],
                        UPD == UPD_ADAGRAD ? a.Xc[e] : 0.f);
    }
  }
}

// x[0 .. n) = 0 (gradient outputs of rows that get no contribution)
__global__ __launch_bounds__(256) void k_zero(float *x, size_t n) {
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) x[i] = 0.f;
}

hipError_t launch_zero(float *x, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const unsigned nb = (unsigned)std::min<size_t>((n + 1023) / 1024, 16384);
  tt_launch(K_ZERO, k_zero, dim3(nb), dim3(256), 0, s, x, n);
  return hipGetLastError();
}

hipError_t launch_seg(const DevArgs &a, hipStream_t s) {
  const int nseg = a.T * a.p1 + a.T * a.p3;
  const int nbh = a.has_cache ? ((a.nnz + PIECE - 1) / PIECE + 3) / 4 : 0;
  const dim3 grid(nseg + a.T * a.p2 * seg_chunks(a) + nbh);
  if (a.upd == UPD_GRAD) tt_launch(K_SEG, k_seg<UPD_GRAD>, grid, dim3(SEG_T), 0, s, a);
  else if (a.upd == UPD_ADAGRAD) tt_launch(K_SEG, k_seg<UPD_ADAGRAD>, grid, dim3(SEG_T), 0, s, a);
  else tt_launch(K_SEG, k_seg<UPD_SGD>, grid, dim3(SEG_T), 0, s, a);
  return hipGetLastError();
}

}  // namespace ttb
