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
// k_bwd: one workgroup per (table, i2) group.  The group is cut into chunks of at
// most CHP pairs and CHI items (distinct indices); per chunk and per column block
// j2 of G2 (staged in LDS): recompute T (MFMA), form dT and the dG3 partial per item
// (VALU), accumulate dG2 (MFMA, K = rows of (pair, j1)) and dG1 per pair (MFMA after
// an LDS transpose of dT).  dG2 is reduced across the 8 waves in a fixed order and
// applied in place (or summed over chunks in the workspace when a group needs more
// than one chunk).  The dG1 / dG3 partials go to the workspace at the position of
// their first element and are summed per slice by k_seg.
#include "tt_internal.h"
#include "tt_mfma.h"

namespace ttb {

template <int RP>
struct BwdLds {
  static constexpr int LD = RP + 4;
  static size_t floats(int CHI, int D, int q3) {
    return (size_t)2 * RP * LD      // G2 column block, double buffered
           + (size_t)RP * LD        // cross-wave dG2 reduction
           + (size_t)NW * 16 * LD   // per-wave dT transpose tile
           + (size_t)CHI * D        // G_u per item
           + (size_t)CHI * RP * q3; // dG3 partial per item
  }
  static size_t ints(int CHI) {
    return (size_t)(CHI + 1) + CHI + CHI + (CHP + 1) + CHP + 2 * (NW + 1) + 16;
  }
  static size_t bytes(int CHI, int D, int q3) { return floats(CHI, D, q3) * 4 + ints(CHI) * 4; }
};

size_t bwd_lds_bytes(int RP, int CHI, int D, int q3) {
  switch (RP) {
    case 16: return BwdLds<16>::bytes(CHI, D, q3);
    case 32: return BwdLds<32>::bytes(CHI, D, q3);
    default: return BwdLds<64>::bytes(CHI, D, q3);
  }
}

// block-wide exclusive prefix of a 0/1 flag (WG threads); returns the prefix and
// writes the block total to *total (LDS int, read after the call).
static __device__ __forceinline__ int block_prefix(bool f, int *s_w, int *total) {
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const unsigned long long m = __ballot(f);
  const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  if (lane == 0) s_w[w] = __popcll(m);
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int i = 0; i < NW; ++i) { const int v = s_w[i]; s_w[i] = run; run += v; }
    *total = run;
  }
  __syncthreads();
  const int r = s_w[w] + __popcll(m & lt);
  __syncthreads();
  return r;
}

template <int RP>
__global__ __launch_bounds__(WG) void k_bwd(DevArgs a) {
  constexpr int KS = RP / 4, NM = RP / 16, LD = BwdLds<RP>::LD, MBW = bwd_mbw(RP);
  const int grp = blockIdx.x;
  const int gs = a.grp_off[grp], ge = a.grp_off[grp + 1];
  if (gs >= ge) return;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, c = lane & 15;
  const int q1 = a.q1, q2 = a.q2, q3 = a.q3, R1 = a.R1, R2 = a.R2, D = a.D, CHI = a.CHI;
  const int CHPb = a.CHPb;
  const int t = grp / a.p2, i2 = grp % a.p2;

  extern __shared__ float smem[];
  float *sG2 = smem;
  float *sRed = sG2 + 2 * RP * LD;
  float *sT = sRed + RP * LD;
  float *sGu = sT + NW * 16 * LD;
  float *sdA3 = sGu + (size_t)CHI * D;
  int *it_beg = (int *)(sdA3 + (size_t)CHI * RP * q3);  // [CHI+1] absolute positions
  int *it_i3 = it_beg + CHI + 1;                          // [CHI]
  int *it_pair = it_i3 + CHI;                             // [CHI]
  int *pr_it = it_pair + CHI;                             // [CHP+1]
  int *pr_i1 = pr_it + CHP + 1;                           // [CHP]
  int *s_w = pr_i1 + CHP;                                 // [NW+1]
  int *s_w2 = s_w + NW + 1;                               // [NW+1]
  int *s_misc = s_w2 + NW + 1;                            // [16]

  const size_t W1 = (size_t)q1 * R1, W3 = (size_t)R2 * q3;
  const size_t slice2 = (size_t)R1 * q2 * R2;
  const size_t g2base = (size_t)(t * a.p2 + i2) * slice2;
  const float *G1t = a.G1 + (size_t)t * a.p1 * W1;
  const float *G3t = a.G3 + (size_t)t * a.p3 * W3;
  float *gacc_g = a.gacc + (size_t)grp * slice2;

  int cur = gs, chunk = 0;
  bool multi = false;
  while (cur < ge) {
    // ---------------- chunk formation: whole items, <= CHI items, <= CHP pairs
    if (tid == 0) { s_misc[0] = 0; s_misc[1] = 0; s_misc[2] = ge; }
    __syncthreads();
    for (int base = cur; base < ge; base += WG) {
      const int nI0 = s_misc[0], nP0 = s_misc[1];
      const int s = base + tid;
      const bool v = s < ge;
      int dA = -1, dI = -1, pdA = -1, pdI = -1;
      if (v) {
        dA = a.s_dA[s];
        dI = a.s_dI3[s];
        if (s > cur) { pdA = a.s_dA[s - 1]; pdI = a.s_dI3[s - 1]; }
      }
      const bool ist = v && (s == cur || dA != pdA || dI != pdI);
      const bool pst = v && (s == cur || dA != pdA);
      const int ip = block_prefix(ist, s_w, &s_misc[3]);
      const int pp = block_prefix(pst, s_w2, &s_misc[4]);
      const int item_idx = nI0 + ip, pair_idx = nP0 + pp;  // index of an item / pair starting at s
      if ((ist && item_idx >= CHI) || (pst && pair_idx >= CHPb)) atomicMin(&s_misc[2], s);
      __syncthreads();
      const int ce = s_misc[2];
      if (ist && s < ce) {
        it_beg[item_idx] = s;
        it_i3[item_idx] = dI - t * a.p3;
        it_pair[item_idx] = pst ? pair_idx : pair_idx - 1;
      }
      if (pst && s < ce) { pr_it[pair_idx] = item_idx; pr_i1[pair_idx] = dA - t * a.p1; }
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
    if (chunk == 0 && ce < ge) multi = true;
    __syncthreads();
    // G_u per item from the run fragments; clear the dG3 partials and the flags
    for (int i = tid; i < nI * D; i += WG) {
      const int it = i / D, d = i - it * D;
      const int b0 = it_beg[it], b1 = it_beg[it + 1];
      float acc = a.frag[(size_t)b0 * D + d];
      for (int p = (b0 / PIECE + 1) * PIECE; p < b1; p += PIECE) acc += a.frag[(size_t)p * D + d];
      sGu[i] = acc;
    }
    for (int i = tid; i < nI * RP * q3; i += WG) sdA3[i] = 0.f;
    for (int s = cur + tid; s < ce; s += WG) { a.flag1[s] = 0; a.flag3[s] = 0; }
    __threadfence_block();
    __syncthreads();
    for (int it = tid; it < nI; it += WG) a.flag3[it_beg[it]] = 1;
    for (int p = tid; p < nP; p += WG) a.flag1[it_beg[pr_it[p]]] = 1;

    const int nmb = (nP * q1 + 15) / 16;
    // A operands from the G1 rows of the wave's M-blocks
    float aT[MBW][KS];         // A1[row = 16mb + c][r1 = g*KS + ks]    (stage 1)
    float aG[MBW][4][NM];      // A1[row = 16mb + 4g + s][r1 = 16mr + c] (dG2)
    f4 dA1[MBW][NM];           // dG1^T[r1 = 16mr + 4g + v][row = c]
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
          aT[mbi][ks] = (ok && r1 < R1) ? src[r1] : 0.f;
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
          aG[mbi][sr][mr] = (ok && r1 < R1) ? src[r1] : 0.f;
        }
      }
#pragma unroll
      for (int mr = 0; mr < NM; ++mr) dA1[mbi][mr] = zero4();
    }

    for (int j2 = 0; j2 < q2; ++j2) {
      float *buf = sG2 + (j2 & 1) * RP * LD;
      for (int i = tid; i < RP * RP; i += WG) {
        const int r1 = i / RP, r2 = i - r1 * RP;
        buf[r2 * LD + r1] =
            (r1 < R1 && r2 < R2) ? a.G2[g2base + ((size_t)r1 * q2 + j2) * R2 + r2] : 0.f;
      }
      __syncthreads();
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
          const int pr = act ? it_pair[it] : -1;
          const int i3 = act ? it_i3[it] : 0;
          const float *a3 = G3t + (size_t)i3 * W3;
          const float *gu = sGu + (size_t)(act ? it : 0) * D;
          for (int j3 = 0; j3 < q3; ++j3) {
            float gv[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const int row = rb + v;
              const int j1 = row - (row / q1) * q1;
              gv[v] = (act && row / q1 == pr) ? gu[(j1 * q2 + j2) * q3 + j3] : 0.f;
            }
#pragma unroll
            for (int m = 0; m < NM; ++m) {
              const int r2 = 16 * m + c;
              const float a3v = (act && r2 < R2) ? a3[r2 * q3 + j3] : 0.f;
              float sacc = 0.f;
#pragma unroll
              for (int v = 0; v < 4; ++v) {
                sacc += T[m][v] * gv[v];
                dT[m][v] += gv[v] * a3v;
              }
              if (act) sdA3[((size_t)it * RP + r2) * q3 + j3] += sacc;
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
        // dG1^T += G2_j2 dT^T  (K = r2; dT transposed through LDS)
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
      // reduce dG2 over the waves in wave order
      for (int ww = 0; ww < NW; ++ww) {
        if (w == ww) {
#pragma unroll
          for (int mr = 0; mr < NM; ++mr)
#pragma unroll
            for (int m2 = 0; m2 < NM; ++m2)
#pragma unroll
              for (int v = 0; v < 4; ++v) {
                const int idx = (16 * mr + 4 * g + v) * LD + 16 * m2 + c;
                sRed[idx] = (ww == 0 ? 0.f : sRed[idx]) + gacc[mr][m2][v];
              }
        }
        __syncthreads();
      }
      for (int i = tid; i < R1 * R2; i += WG) {
        const int r1 = i / R2, r2 = i - r1 * R2;
        const float val = sRed[r1 * LD + r2];
        const size_t off = ((size_t)r1 * q2 + j2) * R2 + r2;
        if (!multi) a.G2[g2base + off] -= a.lr * val;
        else if (chunk == 0) gacc_g[off] = val;
        else gacc_g[off] += val;
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
  if (multi) {
    __threadfence_block();
    __syncthreads();
    for (size_t i = tid; i < slice2; i += WG) a.G2[g2base + i] -= a.lr * gacc_g[i];
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
  hipLaunchKernelGGL(k_bwd<RP>, dim3(a.T * a.p2), dim3(WG), lds, s, a);
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
// One wave per task: a core-1 slice (t, i1), a core-3 slice (t, i3), or a 64-position
// piece of the cache-hit region.  Core slices sum the partials of their segment of
// the (t,i1)- / (t,i3)-ordered element list in that order and apply SGD.  A cache run
// (one slot) is finished by the piece that holds its first position: it sums the run's
// fragments (its first position, then every 64-aligned position inside the run).
__global__ __launch_bounds__(256) void k_seg(DevArgs a) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int task = blockIdx.x * 4 + w;
  const int nA = a.T * a.p1, nC = a.T * a.p3;
  if (task < nA + nC) {
    const bool one = task < nA;
    const int seg = one ? task : task - nA;
    const int *hist = one ? a.histA : a.histI3;
    const int *order = one ? a.orderA : a.orderI3;
    const int *flag = one ? a.flag1 : a.flag3;
    const float *part = one ? a.part1 : a.part3;
    const int W = one ? a.q1 * a.R1 : a.R2 * a.q3;
    float *dst = one ? a.G1 + (size_t)seg * W : a.G3 + (size_t)seg * W;
    const int beg = hist[(size_t)seg * a.nblk], end = hist[(size_t)(seg + 1) * a.nblk];
    if (beg >= end) return;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};  // W <= 256
    bool any = false;
    for (int c0 = beg; c0 < end; c0 += 64) {
      const int s = c0 + lane;
      int pos = 0, f = 0;
      if (s < end) { pos = a.pos_of[order[s]]; f = flag[pos]; }
      unsigned long long m = __ballot(f != 0);
      while (m) {
        const int l = __ffsll((long long)m) - 1;
        m &= m - 1;
        const int ps = __shfl(pos, l);
        any = true;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = lane + 64 * j;
          if (col < W) acc[j] += part[(size_t)ps * W + col];
        }
      }
    }
    if (any) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = lane + 64 * j;
        if (col < W) dst[col] -= a.lr * acc[j];
      }
    }
    return;
  }
  if (!a.has_cache) return;
  const int k = task - nA - nC;
  const int hb = a.hdr[H_HIT_BEG], he = a.hdr[H_HIT_END];
  const int lo = max(k * PIECE, hb), hi = min((k + 1) * PIECE, he);
  for (int s = lo; s < hi; ++s) {
    const int kA = a.s_dA[s], kB = a.s_dB[s];
    if (s > hb && a.s_dA[s - 1] == kA && a.s_dB[s - 1] == kB) continue;  // not a run start
    const int slot = (kB - a.T * a.p2) * HB + (kA - a.T * a.p1);
    for (int d = lane; d < a.D; d += 64) {
      float acc = a.frag[(size_t)s * a.D + d];
      for (int p = (s / PIECE + 1) * PIECE; p < he; p += PIECE) {
        if (a.s_dA[p] != kA || a.s_dB[p] != kB) break;
        acc += a.frag[(size_t)p * a.D + d];
      }
      a.crows[(size_t)slot * a.D + d] -= a.lr * acc;
    }
  }
}

hipError_t launch_seg(const DevArgs &a, hipStream_t s) {
  const int tasks = a.T * a.p1 + a.T * a.p3 + (a.has_cache ? (a.nnz + PIECE - 1) / PIECE : 0);
  prof_begin(K_SEG, s);
  hipLaunchKernelGGL(k_seg, dim3((tasks + 3) / 4), dim3(256), 0, s, a);
  prof_end(K_SEG, s);
  return hipGetLastError();
}

}  // namespace ttb
