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
// one P-aligned piece of the grouping order), cut into chunks of at most CHPb pairs
// and CHI items (distinct indices).  Per chunk, G_u, the items' G3 slices and the
// pairs' G1 rows are fetched once; then per column block j2 of G2 (double-buffered
// in LDS, prefetched into registers): recompute T (MFMA), form dT and the dG3
// partial per item (VALU, LDS only), accumulate dG2 (MFMA, K = the rows (pair, j1))
// and dG1 per pair (MFMA after an LDS transpose of dT).  dG2 is reduced over the 8
// waves in a fixed order into the work item's partial.  The dG1 / dG3 partials go
// to the workspace at the final-order position of their first element.  k_seg then
// sums every partial per slice in a fixed order and applies SGD: dG1 / dG3 in the
// (t,i1)- / (t,i3)-order (which the links name), dG2 in work-item order.
#include "tt_internal.h"
#include "tt_mfma.h"

namespace ttb {

template <int RP>
struct BwdLds {
  static constexpr int LD = RP + 4;
  __host__ __device__ static size_t red_floats(int nred) {
    const size_t r = (size_t)nred * RP * LD, t = (size_t)NW * 16 * LD;
    return r > t ? r : t;  // the dG2 reduction slots alias the dT transpose tiles
  }
  static size_t floats(int CHI, int D, int q3, int nred) {
    return (size_t)2 * RP * LD + red_floats(nred) + (size_t)CHI * D + 2 * (size_t)CHI * RP * q3;
  }
  static size_t ints(int CHI) { return (size_t)(CHI + 1) + 2 * CHI + (CHP + 1) + CHP + 2 * NW + 16; }
  static size_t bytes(int CHI, int D, int q3, int nred) {
    return floats(CHI, D, q3, nred) * 4 + ints(CHI) * 4;
  }
};

size_t bwd_lds_bytes(int RP, int CHI, int D, int q3, int nred) {
  switch (RP) {
    case 16: return BwdLds<16>::bytes(CHI, D, q3, nred);
    case 32: return BwdLds<32>::bytes(CHI, D, q3, nred);
    default: return BwdLds<64>::bytes(CHI, D, q3, nred);
  }
}

// block-wide exclusive prefixes of two 0/1 flags (WG threads).  Totals land in
// tot[0], tot[1] (LDS, valid after the call).
static __device__ __forceinline__ void block_prefix2(bool f0, bool f1, int *s_w, int *tot, int &p0,
                                                     int &p1) {
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const unsigned long long m0 = __ballot(f0), m1 = __ballot(f1);
  const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  if (lane == 0) { s_w[w] = __popcll(m0); s_w[NW + w] = __popcll(m1); }
  __syncthreads();
  if (tid < 64) {
    const int v0 = lane < NW ? s_w[lane] : 0, v1 = lane < NW ? s_w[NW + lane] : 0;
    int x0 = v0, x1 = v1;
#pragma unroll
    for (int o = 1; o < NW; o <<= 1) {
      const int y0 = __shfl_up(x0, o), y1 = __shfl_up(x1, o);
      if (lane >= o) { x0 += y0; x1 += y1; }
    }
    if (lane < NW) { s_w[lane] = x0 - v0; s_w[NW + lane] = x1 - v1; }
    if (lane == NW - 1) { tot[0] = x0; tot[1] = x1; }
  }
  __syncthreads();
  p0 = s_w[w] + __popcll(m0 & lt);
  p1 = s_w[NW + w] + __popcll(m1 & lt);
  __syncthreads();
}

template <int RP>
__global__ __launch_bounds__(WG) void k_bwd(DevArgs a) {
  constexpr int KS = RP / 4, NM = RP / 16, LD = BwdLds<RP>::LD, MBW = bwd_mbw(RP);
  constexpr int KP = (RP * RP + WG - 1) / WG;
  const int wi = blockIdx.x;
  const int plan = a.hdr[H_PLAN], nitems = a.hdr[H_NFWD];
  const int4 item = a.fitem[wi];
  if (plan != (int)a.plan_fp || wi >= nitems) return;
  const int grp = item.x, gs = item.y, ge = item.z;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, c = lane & 15;
  const int q1 = a.q1, q2 = a.q2, q3 = a.q3, R1 = a.R1, R2 = a.R2, D = a.D, CHI = a.CHI;
  const int CHPb = a.CHPb, nred = a.NRED;
  const int t = grp / a.p2, i2 = grp - t * a.p2;

  extern __shared__ float smem[];
  float *sG2 = smem;
  float *sRed = sG2 + 2 * RP * LD;  // aliases sT
  float *sT = sRed;
  float *sGu = sRed + BwdLds<RP>::red_floats(nred);
  float *sG3 = sGu + (size_t)CHI * D;
  float *sdA3 = sG3 + (size_t)CHI * RP * q3;
  int *it_beg = (int *)(sdA3 + (size_t)CHI * RP * q3);  // [CHI+1] final-order positions
  int *it_i3 = it_beg + CHI + 1;                          // [CHI]
  int *it_pair = it_i3 + CHI;                             // [CHI]
  int *pr_it = it_pair + CHI;                             // [CHP+1]
  int *pr_i1 = pr_it + CHP + 1;                           // [CHP]
  int *s_w = pr_i1 + CHP;                                 // [2*NW]
  int *s_misc = s_w + 2 * NW;                             // [16]

  const size_t W1 = (size_t)q1 * R1, W3 = (size_t)R2 * q3;
  const size_t slice2 = (size_t)R1 * q2 * R2;
  const size_t g2base = (size_t)(t * a.p2 + i2) * slice2;
  const float *G1t = a.G1 + (size_t)t * a.p1 * W1;
  const float *G3t = a.G3 + (size_t)t * a.p3 * W3;
  float *part2 = a.part2 + (size_t)wi * slice2;

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

  int cur = gs, chunk = 0;
  while (cur < ge) {
    fetch_g2(0);
    // ---------------- chunk formation: whole items, <= CHI items, <= CHPb pairs;
    // the links of the chunk's positions are written on the way
    if (tid == 0) { s_misc[0] = 0; s_misc[1] = 0; s_misc[2] = ge; }
    __syncthreads();
    for (int base = cur; base < ge; base += WG) {
      const int nI0 = s_misc[0], nP0 = s_misc[1];
      const int s = base + tid;
      const bool v = s < ge;
      const int sc = v ? s : ge - 1, sp = max(sc - 1, 0);
      const int dA0 = a.s_dA[sc], dI0 = a.s_dI3[sc], pdA0 = a.s_dA[sp], pdI0 = a.s_dI3[sp];
      const int lA = a.s_posA[sc], lI = a.s_posI3[sc];
      const bool first = s == cur;
      const bool ist = v && (first || dA0 != pdA0 || dI0 != pdI0);
      const bool pst = v && (first || dA0 != pdA0);
      int ip, pp;
      block_prefix2(ist, pst, s_w, &s_misc[3], ip, pp);
      const int item_idx = nI0 + ip, pair_idx = nP0 + pp;  // index of an item / pair starting at s
      if ((ist && item_idx >= CHI) || (pst && pair_idx >= CHPb)) atomicMin(&s_misc[2], s);
      __syncthreads();
      const int ce = s_misc[2];
      if (ist && s < ce) {
        it_beg[item_idx] = s;
        it_i3[item_idx] = dI0 - t * a.p3;
        it_pair[item_idx] = pst ? pair_idx : pair_idx - 1;
      }
      if (pst && s < ce) { pr_it[pair_idx] = item_idx; pr_i1[pair_idx] = dA0 - t * a.p1; }
      if (v && s < ce) {
        a.link1[lA] = pst ? s : -1;
        a.link3[lI] = ist ? s : -1;
      }
      if (s == ce) { s_misc[5] = ip; s_misc[6] = pp; }
      __syncthreads();
      if (tid == 0) {
        if (ce < ge) { s_misc[0] = nI0 + s_misc[5]; s_misc[1] = nP0 + s_misc[6]; }
        else { s_misc[0] = nI0 + s_misc[3]; s_misc[1] = nP0 + s_misc[4]; }
      }
      __syncthreads();
      if (ce < ge) break;
    }
    const int nI = s_misc[0], nP = s_misc[1], ce = s_misc[2];
    if (tid == 0) { it_beg[nI] = ce; pr_it[nP] = nI; }
    __syncthreads();
    // ---------------- chunk data: G_u (run fragments), the items' G3 slices, A operands,
    // STAGE_U loads in flight per thread
    {
      const int total = nI * D;
      for (int base = tid; base < total; base += WG * STAGE_U) {
        float v[STAGE_U];
#pragma unroll
        for (int u = 0; u < STAGE_U; ++u) {
          const int i = min(base + u * WG, total - 1);
          const int it = i / D, d = i - it * D;
          v[u] = a.frag[(size_t)it_beg[it] * D + d];
        }
#pragma unroll
        for (int u = 0; u < STAGE_U; ++u) {
          const int i = base + u * WG;
          if (i < total) {
            const int it = i / D, d = i - it * D;
            const int b0 = it_beg[it], b1 = it_beg[it + 1];
            float acc = v[u];  // runs longer than a piece carry more fragments (rare)
            for (int p = (b0 / a.P + 1) * a.P; p < b1; p += a.P)
              acc += a.frag[(size_t)p * D + d];
            sGu[i] = acc;
          }
        }
      }
    }
    {
      const int per_item = RP * q3, total = nI * per_item;
      for (int base = tid; base < total; base += WG * STAGE_U) {
        float v[STAGE_U];
#pragma unroll
        for (int u = 0; u < STAGE_U; ++u) {
          const int i = min(base + u * WG, total - 1);
          const int it = i / per_item, rem = i - it * per_item;
          const int r2 = rem / q3;
          v[u] = G3t[(size_t)it_i3[it] * W3 + (r2 < R2 ? rem : 0)];
        }
#pragma unroll
        for (int u = 0; u < STAGE_U; ++u) {
          const int i = base + u * WG;
          if (i < total) {
            const int rem = i % per_item;
            sG3[i] = (rem / q3 < R2) ? v[u] : 0.f;
            sdA3[i] = 0.f;
          }
        }
      }
    }
    const int nmb = (nP * q1 + 15) / 16;
    float aT[MBW][KS];      // A1[row = 16mb + c][r1 = g*KS + ks]    (stage 1)
    float aG[MBW][4][NM];   // A1[row = 16mb + 4g + s][r1 = 16mr + c] (dG2)
    f4 dA1[MBW][NM];        // dG1^T[r1 = 16mr + 4g + v][row = c]
#pragma unroll
    for (int mbi = 0; mbi < MBW; ++mbi) {
      const int mb = w + mbi * NW;
      {
        const int row = mb * 16 + c;
        const int pr = row / q1, j1 = row - pr * q1;
        const bool ok = mb < nmb && pr < nP;
        const float *src = G1t + ((size_t)(ok ? pr_i1[pr] : 0) * q1 + j1) * R1;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int r1 = g * KS + ks;
          const float v = src[min(r1, R1 - 1)];
          aT[mbi][ks] = (ok && r1 < R1) ? v : 0.f;
        }
      }
#pragma unroll
      for (int sr = 0; sr < 4; ++sr) {
        const int row = mb * 16 + 4 * g + sr;
        const int pr = row / q1, j1 = row - pr * q1;
        const bool ok = mb < nmb && pr < nP;
        const float *src = G1t + ((size_t)(ok ? pr_i1[pr] : 0) * q1 + j1) * R1;
#pragma unroll
        for (int mr = 0; mr < NM; ++mr) {
          const int r1 = 16 * mr + c;
          const float v = src[min(r1, R1 - 1)];
          aG[mbi][sr][mr] = (ok && r1 < R1) ? v : 0.f;
        }
      }
#pragma unroll
      for (int mr = 0; mr < NM; ++mr) dA1[mbi][mr] = zero4();
    }
    store_g2(sG2);
    if (q2 > 1) fetch_g2(1);
    __syncthreads();

    for (int j2 = 0; j2 < q2; ++j2) {
      const float *buf = sG2 + (j2 & 1) * RP * LD;
      f4 gacc[NM][NM];  // dG2[r1 = 16mr + 4g + v][r2 = 16m2 + c]
#pragma unroll
      for (int mr = 0; mr < NM; ++mr)
#pragma unroll
        for (int m2 = 0; m2 < NM; ++m2) gacc[mr][m2] = zero4();
#pragma unroll
      for (int mbi = 0; mbi < MBW; ++mbi) {
        const int mb = w + mbi * NW;
        if (mb >= nmb) break;
        // stage 1: T[row = 16mb + 4g + v][r2 = 16m + c]
        f4 T[NM], dT[NM];
#pragma unroll
        for (int m = 0; m < NM; ++m) { T[m] = zero4(); dT[m] = zero4(); }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
          for (int m = 0; m < NM; ++m)
            T[m] = mfma4(aT[mbi][ks], buf[(16 * m + c) * LD + g * KS + ks], T[m]);
        // items whose pair owns rows 16mb + 4g .. +3
        const int rb = mb * 16 + 4 * g;
        const int plo = rb / q1;
        const int phi = min((rb + 3) / q1, nP - 1);
        const int ib = plo < nP ? pr_it[plo] : 0;
        const int ie = plo < nP ? pr_it[phi + 1] : 0;
        const int nk = wave_max(ie - ib);
        for (int kk = 0; kk < nk; ++kk) {
          const int it = ib + kk;
          const bool act = it < ie;
          const int itc = act ? it : 0;
          const int pr = act ? it_pair[itc] : -1;
          const float *g3 = sG3 + (size_t)itc * RP * q3;
          const float *gu = sGu + (size_t)itc * D;
          float *da3 = sdA3 + (size_t)itc * RP * q3;
          for (int j3 = 0; j3 < q3; ++j3) {
            float gv[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const int row = rb + v;
              const int j1 = row - (row / q1) * q1;
              const float x = gu[(j1 * q2 + j2) * q3 + j3];
              gv[v] = (act && row / q1 == pr) ? x : 0.f;
            }
#pragma unroll
            for (int m = 0; m < NM; ++m) {
              const int r2 = 16 * m + c;
              const float a3v = g3[r2 * q3 + j3];
              float sacc = 0.f;
#pragma unroll
              for (int v = 0; v < 4; ++v) {
                sacc += T[m][v] * gv[v];
                dT[m][v] += gv[v] * a3v;
              }
              if (act) da3[r2 * q3 + j3] += sacc;
            }
          }
        }
        // dG2 += A1^T dT   (K = the 16 rows; lane group g feeds rows 4g + s)
#pragma unroll
        for (int sr = 0; sr < 4; ++sr)
#pragma unroll
          for (int mr = 0; mr < NM; ++mr)
#pragma unroll
            for (int m2 = 0; m2 < NM; ++m2)
              gacc[mr][m2] = mfma4(aG[mbi][sr][mr], dT[m2][sr], gacc[mr][m2]);
        // dG1^T += G2_j2 dT^T  (K = r2; dT transposed through the wave's LDS tile)
        float *tt = sT + (size_t)w * 16 * LD;
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int v = 0; v < 4; ++v) tt[(4 * g + v) * LD + 16 * m + c] = dT[m][v];
        wave_lds_sync();
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int r2 = 16 * m + 4 * g + v;
            const float bT = tt[c * LD + r2];
#pragma unroll
            for (int mr = 0; mr < NM; ++mr)
              dA1[mbi][mr] = mfma4(buf[r2 * LD + 16 * mr + c], bT, dA1[mbi][mr]);
          }
        wave_lds_sync();
      }
      // reduce dG2 over the waves: wave w adds into slot w % nred, rounds in wave order,
      // then the slots are summed in slot order
      __syncthreads();  // the transpose tiles (aliased by the slots) are free
      for (int rr = 0; rr < NW / nred; ++rr) {
        if (w / nred == rr) {
          float *slot = sRed + (size_t)(w % nred) * RP * LD;
#pragma unroll
          for (int mr = 0; mr < NM; ++mr)
#pragma unroll
            for (int m2 = 0; m2 < NM; ++m2)
#pragma unroll
              for (int v = 0; v < 4; ++v) {
                const int idx = (16 * mr + 4 * g + v) * LD + 16 * m2 + c;
                slot[idx] = (rr == 0 ? 0.f : slot[idx]) + gacc[mr][m2][v];
              }
        }
        __syncthreads();
      }
      for (int i = tid; i < R1 * R2; i += WG) {
        const int r1 = i / R2, r2 = i - r1 * R2;
        float val = 0.f;
        for (int k = 0; k < nred; ++k) val += sRed[(size_t)k * RP * LD + r1 * LD + r2];
        const size_t off = ((size_t)r1 * q2 + j2) * R2 + r2;
        if (chunk == 0) part2[off] = val;
        else part2[off] += val;
      }
      if (j2 + 1 < q2) {
        store_g2(sG2 + ((j2 + 1) & 1) * RP * LD);
        if (j2 + 2 < q2) fetch_g2(j2 + 2);
      }
      __syncthreads();
    }
    // dG1 partial per pair, dG3 partial per item, at their first positions
#pragma unroll
    for (int mbi = 0; mbi < MBW; ++mbi) {
      const int mb = w + mbi * NW;
      if (mb >= nmb) break;
      const int row = mb * 16 + c;
      const int pr = row / q1, j1 = row - pr * q1;
      if (pr < nP) {
        float *dst = a.part1 + (size_t)it_beg[pr_it[pr]] * W1 + (size_t)j1 * R1;
#pragma unroll
        for (int mr = 0; mr < NM; ++mr)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int r1 = 16 * mr + 4 * g + v;
            if (r1 < R1) dst[r1] = dA1[mbi][mr][v];
          }
      }
    }
    for (int i = tid; i < nI * (int)W3; i += WG) {
      const int it = i / W3, rem = i - it * W3;
      const int r2 = rem / q3, j3 = rem - r2 * q3;
      a.part3[(size_t)it_beg[it] * W3 + rem] = sdA3[((size_t)it * RP + r2) * q3 + j3];
    }
    __syncthreads();
    cur = ce;
    ++chunk;
  }
}

template <int RP>
static hipError_t launch_bwd_t(const DevArgs &a, size_t lds, hipStream_t s) {
  static bool attr_set = false;  // dynamic LDS above 64 KiB is opt-in per kernel
  if (!attr_set) {
    (void)hipFuncSetAttribute((const void *)k_bwd<RP>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              160 * 1024);
    attr_set = true;
  }
  prof_begin(K_BWD, s);
  hipLaunchKernelGGL(k_bwd<RP>, dim3(items_max(a)), dim3(WG), lds, s, a);
  prof_end(K_BWD, s);
  return hipGetLastError();
}

hipError_t launch_bwd(const DevArgs &a, int RP, size_t lds, hipStream_t s) {
  switch (RP) {
    case 16: return launch_bwd_t<16>(a, lds, s);
    case 32: return launch_bwd_t<32>(a, lds, s);
    default: return launch_bwd_t<64>(a, lds, s);
  }
}

// ---------------------------------------------------------------- k_seg
// Blocks of 256 threads, three kinds of task:
//  * four waves = four core-1 slices (t, i1) or core-3 slices (t, i3): a slice walks
//    its segment of the (t,i1)- or (t,i3)-ordered element list; the link of each
//    position names the final-order position of a partial (or -1); the partials are
//    summed in segment order, eight loads in flight at a time, then SGD is applied;
//  * one block = one core-2 slice (t, i2): the dG2 partials of the group's work
//    items are summed in item order, then SGD;
//  * four waves = four 64-position pieces of the cache-hit region: a cache run (one
//    slot) is finished by the piece that holds its first position, which sums the
//    run's fragments (its first position, then every multiple of P inside the run).
__global__ __launch_bounds__(256) void k_seg(DevArgs a) {
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int nA = a.T * a.p1, nC = a.T * a.p3, G = a.T * a.p2;
  const int nb1 = (nA + nC + 3) / 4;
  if (a.hdr[H_PLAN] != (int)a.plan_fp) return;
  const int bid = blockIdx.x;
  if (bid < nb1) {
    const int task = bid * 4 + w;
    if (task >= nA + nC) return;
    const bool one = task < nA;
    const int seg = one ? task : task - nA;
    const int *hist = one ? a.histA : a.histI3;
    const int *link = one ? a.link1 : a.link3;
    const float *part = one ? a.part1 : a.part3;
    const int W = one ? a.q1 * a.R1 : a.R2 * a.q3;
    float *dst = one ? a.G1 + (size_t)seg * W : a.G3 + (size_t)seg * W;
    const int beg = hist[(size_t)seg * a.nblk], end = hist[(size_t)(seg + 1) * a.nblk];
    if (beg >= end) return;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};  // W <= 256
    const int c0c = min(lane, W - 1), c1c = min(lane + 64, W - 1), c2c = min(lane + 128, W - 1),
              c3c = min(lane + 192, W - 1);
    for (int s0 = beg; s0 < end; s0 += 64) {
      const int sl = min(s0 + lane, end - 1);
      const int lk = link[sl];
      unsigned long long m = __ballot(s0 + lane < end && lk >= 0);
      while (m) {
        int ps[8];
        int cnt = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          ps[k] = -1;
          if (m) {
            const int l = __ffsll((long long)m) - 1;
            m &= m - 1;
            ps[k] = __builtin_amdgcn_readlane(lk, l);
            ++cnt;
          }
        }
        float v[8][4];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float *row = part + (size_t)max(ps[k], 0) * W;
          v[k][0] = row[c0c];
          v[k][1] = row[c1c];
          v[k][2] = row[c2c];
          v[k][3] = row[c3c];
        }
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (k < cnt)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j] += v[k][j];
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = lane + 64 * j;
      if (col < W) dst[col] -= a.lr * acc[j];
    }
    return;
  }
  if (bid < nb1 + G) {
    const int g = bid - nb1;
    const int i0 = a.chunk_pre[g], i1 = a.chunk_pre[g + 1];
    if (i0 >= i1) return;
    const size_t slice2 = (size_t)a.R1 * a.q2 * a.R2;
    float *dst = a.G2 + (size_t)g * slice2;
    for (size_t e0 = tid; e0 < slice2; e0 += 256 * 4) {
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
      for (int it = i0; it < i1; ++it) {
        const float *src = a.part2 + (size_t)it * slice2;
        float v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = src[min(e0 + (size_t)u * 256, slice2 - 1)];
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[u] += v[u];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const size_t e = e0 + (size_t)u * 256;
        if (e < slice2) dst[e] -= a.lr * acc[u];
      }
    }
    return;
  }
  if (!a.has_cache) return;
  const int k = (bid - nb1 - G) * 4 + w;
  const int hb = a.hdr[H_HIT_BEG], he = a.hdr[H_HIT_END];
  const int lo = max(k * PIECE, hb), hi = min((k + 1) * PIECE, he);
  for (int s = lo; s < hi; ++s) {
    const int kA = a.s_dA[s], kB = a.s_dB[s];
    if (s > hb && a.s_dA[s - 1] == kA && a.s_dB[s - 1] == kB) continue;  // not a run start
    const int slot = (kB - a.T * a.p2) * HB + (kA - a.T * a.p1);
    for (int d = lane; d < a.D; d += 64) {
      float acc = a.frag[(size_t)s * a.D + d];
      for (int p = (s / a.P + 1) * a.P; p < he; p += a.P) {
        if (a.s_dA[p] != kA || a.s_dB[p] != kB) break;
        acc += a.frag[(size_t)p * a.D + d];
      }
      a.crows[(size_t)slot * a.D + d] -= a.lr * acc;
    }
  }
}

hipError_t launch_seg(const DevArgs &a, hipStream_t s) {
  const int nb1 = (a.T * a.p1 + a.T * a.p3 + 3) / 4;
  const int nbh = a.has_cache ? ((a.nnz + PIECE - 1) / PIECE + 3) / 4 : 0;
  prof_begin(K_SEG, s);
  hipLaunchKernelGGL(k_seg, dim3(nb1 + a.T * a.p2 + nbh), dim3(256), 0, s, a);
  prof_end(K_SEG, s);
  return hipGetLastError();
}

}  // namespace ttb
