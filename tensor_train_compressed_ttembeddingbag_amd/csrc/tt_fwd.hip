// tt_fwd.hip -- forward TT contraction + bag pooling.
//
// "FBTT-Embedding" README, "Software Cache": a lookup rebuilds a row by two
// consecutive GEMMs; "TT-Rec" (MLSys 2021) abstract: lookups are batched into
// matrix multiplications.  With the row split i -> (i1,i2,i3):
//   stage 1  T[j1][j2][r2] = sum_r1 G1[i1][j1][r1] * G2[i2][r1][j2][r2]
//   stage 2  W[i][(j1 q2 + j2) q3 + j3] = sum_r2 T[j1][j2][r2] * G3[i3][r2][j3]
// and EmbeddingBag pooling out[b] += w_n * W[idx_n] (tensorflow/addons #2201: the
// gathered rows are never materialised in global memory).
//
// One workgroup takes one work item: the elements of one (table, i2) group that
// fall in one P-aligned piece of the grouping order (all of them share one G2
// slice).  The kernel is built around three dependent rounds of global loads
//   1. the work item (group, position range),
//   2. the item's elements and its G2 slice (the first JB column blocks),
//   3. the G1 rows of its distinct (i1, i2) pairs and the G3 slices of its
//      distinct indices,
// after which everything runs out of LDS and registers.  Without a cache the first
// workgroups also clear out (fwd_clear_out), so no separate kernel runs before.
// Stage 1 runs once per pair as a GEMM on the fp32 matrix cores,
//     T^T[r2][(pair, j1)] = sum_r1 G2[r1][j2][r2] * G1[i1(pair)][j1][r1],
// with 16 (pair, j1) rows per "M-block" in the MFMA column dimension and G2^T
// read from LDS as 16-byte vectors.  Stage 2 runs once per distinct index in VALU
// and leaves the item's rows W in LDS; a last pass adds w * W[item] into each
// element's bag with row-contiguous fp32 atomics.  Bits of out may depend on the
// order of the atomics.
#include "tt_device.h"
#include "tt_mfma.h"

namespace ttb {

// LDS carve of one forward workgroup (float words, then int words)
template <int RP>
struct FwdLds {
  static constexpr int LD = RP + 4;  // row pitch of G2^T [r2][r1]: conflict-free 16-byte reads
  // j3 pitch of the staged G3 slices [item][j3][r2]: with RP + 4 the sixteen lanes of a lane
  // group (four items x four j3 in the matrix-core stage 2) read sixteen different bank
  // quadruples instead of one
  static constexpr int GS = RP + 4;
  static constexpr int INTS = META_INTS;
  __host__ __device__ static size_t g2_floats(int JB) { return (size_t)JB * RP * LD; }
  __host__ __device__ static size_t g3_floats(int P, int q3) { return (size_t)P * q3 * GS; }
  __host__ __device__ static size_t w_floats(int P, int D, int sw) { return sw ? (size_t)P * D : 0; }
  static size_t bytes(int JB, int P, int q3, int D, int sw) {
    return (g2_floats(JB) + g3_floats(P, q3) + w_floats(P, D, sw)) * 4 + INTS * 4;
  }
};

// Clearing of out by the forward itself (no cache): blocks 0 .. nz-1 clear a slice each
// with device-coherent stores and then raise their flag (this call's epoch); every block
// checks all flags before its first atomic into out.  The clearing blocks are dispatched
// before any block that waits and never wait themselves before raising the flag.
__device__ __forceinline__ int fwd_zero_blocks(const DevArgs &a) {
  return min(FWD_ZERO_BLOCKS, (int)gridDim.x);
}
static __device__ void fwd_clear_out(const DevArgs &a) {
  const long long n = (long long)a.NB * a.D, nz = fwd_zero_blocks(a);
  const long long chunk = (n + nz - 1) / nz, lo = blockIdx.x * chunk, hi = min(n, lo + chunk);
  for (long long i = lo + threadIdx.x; i < hi; i += WG)
    __hip_atomic_store(a.Y + i, 0.f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
static __device__ void fwd_raise_flag(const DevArgs &a) {  // whole block
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this thread's clearing stores are done
  __syncthreads();
  if (threadIdx.x == 0)
    __hip_atomic_store(&a.fflag[blockIdx.x], (unsigned long long)a.epoch, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
// one poll of the clearing flags by the first wave (lane k: flag k); issued early, its
// answer is looked at when the block needs out, so a flag raised by then costs no wait
static __device__ unsigned long long fwd_poll_flags(const DevArgs &a) {
  const int lane = threadIdx.x;
  return (lane < 64 && lane < fwd_zero_blocks(a))
             ? __hip_atomic_load(&a.fflag[lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
             : (unsigned long long)a.epoch;
}
// first: an earlier poll's answer (fwd_poll_flags), taken as the first poll
static __device__ void fwd_wait_out(const DevArgs &a, unsigned long long first) {  // whole block
  __shared__ int s_ok;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int ok = 1;
    unsigned long long v = first;
    for (unsigned polls = 0;; ++polls) {
      if (polls >= a.sync_polls) {  // (a limit of 0 gives up before the first poll)
        ok = 0;
        if (lane == 0) set_status(a.status, TT_DEV_SYNC_TIMEOUT);
        break;
      }
      if (polls > 0) {
        __builtin_amdgcn_s_sleep(1);
        v = fwd_poll_flags(a);
      }
      if (__ballot(v != (unsigned long long)a.epoch) == 0ull) break;
    }
    if (lane == 0) s_ok = ok;
  }
  __syncthreads();
  (void)s_ok;
}

// DOT: instead of pooling, the gradient with respect to each element's per-sample weight,
// dL/dw_n = <grad_out[bag n], row n> (times 1 / bag length with mean pooling); rows in LDS.
// MF: stage 2 on the matrix cores (q1 = q3 = 4, rows kept in LDS, RP <= 32), chosen by the
// host when the work items are expected to be resident at once (see mf_stage2).
template <int RP, bool DOT, bool MF>
__device__ __forceinline__ void fwd_item(const DevArgs &a) {
  constexpr int KS = RP / 4;   // k-steps: lane group g covers r1 = g*KS + ks
  constexpr int NM = RP / 16;  // 16-row blocks of r2
  constexpr int LD = FwdLds<RP>::LD, GS = FwdLds<RP>::GS, LRP = log2_rp<RP>();
  extern __shared__ float4 smem4[];
  float *smem = (float *)smem4;
  const int q1 = a.q1, q2 = a.q2, q3 = a.q3, R1 = a.R1, R2 = a.R2, D = a.D;
  const int JB = a.JBf, P = a.P, SW = DOT ? 1 : a.fwd_sw;
  float *sG2 = smem;                                            // [JB][r2 < RP][LD]
  float *sG3 = sG2 + FwdLds<RP>::g2_floats(JB);                 // [item][j3][r2 < RP], pitch GS
  float *sW = sG3 + FwdLds<RP>::g3_floats(P, q3);               // [item][D]
  int *s_meta = (int *)(sW + FwdLds<RP>::w_floats(P, D, SW));  // [META_INTS]
  const WorkMeta &M = *(const WorkMeta *)s_meta;

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, c = lane & 15;
  const int wi = blockIdx.x;
  const bool clearer = a.fzero && wi < fwd_zero_blocks(a);
  // round 1: plan check and the work item's metadata (a stale plan leaves out untouched)
  const int plan = a.hdr[H_PLAN], nitems = a.hdr[H_NFWD];
  __shared__ int s_pl[NW];
  if (tid < META_INTS) s_meta[tid] = a.meta[(size_t)wi * META_INTS + tid];
  note_placement(s_pl);
  const bool stale = plan != (int)a.plan_fp;
  if (clearer && !stale) fwd_clear_out(a);
  if (stale || wi >= nitems) {
    if (clearer) fwd_raise_flag(a);
    if (stale && wi == 0 && tid == 0) set_status(a.status, DEV_STALE_PLAN);
    return;
  }
  lds_barrier();
  // the record's counts are the same for the whole workgroup: scalar registers
  const int grp = wave_uniform(M.grp), n_el = wave_uniform(M.n_el), nI = wave_uniform(M.nI);
  const int nP = wave_uniform(M.nP);
  // this wave's M-block (MBW = 1), by the slot the grouping gave it
  const int wp = wave_uniform(M.mb_fslot[placed_mblock<NW>(s_pl)]);
  const int t = wave_uniform(M.t);
  const float *G2g = a.G2 + (size_t)grp * R1 * q2 * R2;  // slice [r1][j2][r2]
  const size_t W3 = (size_t)R2 * q3;
  const float *G3t = a.G3 + (size_t)t * a.p3 * W3;

  // G2 columns [j0, j0 + nj) -> LDS as G2^T blocks (zero padding to RP x RP), in
  // batches of STAGE_U loads per thread
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
  const int nj0 = min(JB, q2);
  const int nmb = (nP * q1 + 15) >> 4;

  // round 2: the first G2 stage, the G3 slices of the item's indices -> LDS
  // [item][j3][r2 < RP], and the B operand of stage 1 (G1 rows of the wave's M-blocks,
  // kept for all j2).  The first batch of everything is issued before the first wait;
  // rows past the pairs read a valid row and are zeroed afterwards.
  const int per_item = RP * q3, total3 = nI * per_item;
  // element i = (item * RP + r2) * q3 + j3: contiguous in the global slice [r2][j3],
  // stored to LDS at (item * q3 + j3) * RP + r2
  auto load3 = [&](int base, float *v) {
#pragma unroll
    for (int u = 0; u < STAGE_U; ++u) {
      const int i = min(base + u * WG, total3 - 1);
      const int jr = fdiv(i, a.mq3), j3 = i - jr * q3, it = jr >> LRP, r2 = jr & (RP - 1);
      v[u] = G3t[M.it_i3[it] * (int)W3 + (r2 < R2 ? r2 : 0) * q3 + j3];
    }
  };
  auto store3 = [&](int base, const float *v) {
#pragma unroll
    for (int u = 0; u < STAGE_U; ++u) {
      const int i = base + u * WG;
      if (i < total3) {
        const int jr = fdiv(i, a.mq3), j3 = i - jr * q3, it = jr >> LRP, r2 = jr & (RP - 1);
        sG3[(it * q3 + j3) * GS + r2] = r2 < R2 ? v[u] : 0.f;
      }
    }
  };
  float bv[MBW][KS];
  const float *G1t = a.G1 + (size_t)t * a.p1 * q1 * R1;  // the table's core 1
  auto load_g1 = [&](bool vec) {
#pragma unroll
    for (int mbi = 0; mbi < MBW; ++mbi) {
      const int row = (wp + mbi * NW) * 16 + c;
      const int pr = row >> a.lq1, j1 = row & (q1 - 1);
      // a 32-bit offset inside the table (i1 < 2^13, q1 R1 <= 2^12)
      const float *src =
          G1t + __umul24((unsigned)M.pr_i1[min(pr, nP - 1)] * (unsigned)q1 + (unsigned)j1,
                         (unsigned)R1);
      if (vec) {
#pragma unroll
        for (int k4 = 0; k4 < KS / 4; ++k4) {
          const float4 x = *(const float4 *)&src[g * KS + 4 * k4];
          bv[mbi][4 * k4] = x.x; bv[mbi][4 * k4 + 1] = x.y;
          bv[mbi][4 * k4 + 2] = x.z; bv[mbi][4 * k4 + 3] = x.w;
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) bv[mbi][ks] = src[min(g * KS + ks, R1 - 1)];
      }
    }
  };
  if (q3 == 4 && R1 == RP && R2 == RP) {
    // 16-byte loads (ranks fill RP, q3 = 4): G2 along r2, one (r2, four j3) vector of an
    // item's G3 slice per lane; the LDS layouts stay those of the general path
    constexpr int SV = 2;
    const int n2 = nj0 * RP * RP / 4, n3 = nI * RP;
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
    auto st3 = [&](int i4, float4 x) {  // LDS [item][j3][r2]
      float *d = &sG3[(size_t)(i4 >> LRP) * 4 * GS + (i4 & (RP - 1))];
      d[0] = x.x; d[GS] = x.y; d[2 * GS] = x.z; d[3 * GS] = x.w;
    };
    float4 v2[SV], v3[SV];
#pragma unroll
    for (int u = 0; u < SV; ++u) {
      v2[u] = ld2(min(tid + u * WG, n2 - 1));
      v3[u] = ld3(min(tid + u * WG, n3 - 1));
    }
    load_g1(true);
#pragma unroll
    for (int u = 0; u < SV; ++u) {
      const int i4 = tid + u * WG;
      if (i4 < n2) st2(i4, v2[u]);
      if (i4 < n3) st3(i4, v3[u]);
    }
    for (int i4 = tid + SV * WG; i4 < n2; i4 += WG) st2(i4, ld2(i4));
    for (int i4 = tid + SV * WG; i4 < n3; i4 += WG) st3(i4, ld3(i4));
  } else {
    float v2[STAGE_U], v3[STAGE_U];
    load2(0, nj0, tid, v2);
    load3(tid, v3);
    load_g1(false);
    store2(nj0, tid, v2);
    stage_g2(0, nj0, tid + WG * STAGE_U);
    store3(tid, v3);
    for (int base = tid + WG * STAGE_U; base < total3; base += WG * STAGE_U) {
      float v[STAGE_U];
      load3(base, v);
      store3(base, v);
    }
  }
#pragma unroll
  for (int mbi = 0; mbi < MBW; ++mbi) {
    const int row = (wp + mbi * NW) * 16 + c;
    const bool ok = (wp + mbi * NW) < nmb && (row >> a.lq1) < nP;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const float v = keep(bv[mbi][ks]);
      bv[mbi][ks] = (ok && g * KS + ks < R1) ? v : 0.f;
    }
  }
  vmem_drain();
  if (clearer) fwd_raise_flag(a);  // (includes the barrier)
  else lds_barrier();

  if (a.fzero && !SW) fwd_wait_out(a, fwd_poll_flags(a));  // stage 2 adds into out directly
  // rows kept in LDS: the first poll of the clearing flags is in flight during the columns
  const unsigned long long fpoll = (a.fzero && SW) ? fwd_poll_flags(a) : 0ull;
  for (int j0 = 0; j0 < q2; j0 += JB) {
    if (j0 > 0) {  // next G2 stage (only when the slice does not fit at once)
      lds_barrier();
      stage_g2(j0, min(JB, q2 - j0), tid);
      vmem_drain();
      lds_barrier();
    }
    const int jend = min(q2, j0 + JB);
    for (int j2 = j0; j2 < jend; ++j2) {
      const float *buf = sG2 + (size_t)(j2 - j0) * RP * LD;
#pragma unroll
      for (int mbi = 0; mbi < MBW; ++mbi) {
        const int mb = wp + mbi * NW;
        if (mb >= nmb) break;
        f4 acc[NM];
#pragma unroll
        for (int m = 0; m < NM; ++m) acc[m] = zero4();
#pragma unroll
        for (int kq = 0; kq < KS / 4; ++kq) {
#pragma unroll
          for (int m = 0; m < NM; ++m) {
            const float4 av = *(const float4 *)&buf[(16 * m + c) * LD + g * KS + 4 * kq];
            acc[m] = mfma4(av.x, bv[mbi][4 * kq + 0], acc[m]);
            acc[m] = mfma4(av.y, bv[mbi][4 * kq + 1], acc[m]);
            acc[m] = mfma4(av.z, bv[mbi][4 * kq + 2], acc[m]);
            acc[m] = mfma4(av.w, bv[mbi][4 * kq + 3], acc[m]);
          }
        }
        if (MF) {
          // stage 2 on the matrix cores (q1 = q3 = 4, rows kept in LDS): the rows of the
          // M-block's items times their G3 slices, four items x four j3 per 16-column
          // block.  A = T straight from acc (instruction (m, v) takes r2 = 16m + 4g + v
          // as the k index of lane group g); B = G3 of item s = c / 4 at j3 = c % 4.
          // Lane (g, c) gets rows 4g .. 4g+3 of the M-block (its pair p0 + g, j1 = v) in
          // column c and keeps the columns of its own pair's items.
          const int p0 = mb * 4;  // mb < nmb, so p0 < nP
          const int it0 = M.pr_it[p0], it1 = M.pr_it[min(p0 + 4, nP)];
          const int myp = p0 + g;
          const int mib = myp < nP ? M.pr_it[myp] : 0, mie = myp < nP ? M.pr_it[myp + 1] : 0;
          const int s4 = c >> 2, jc = c & 3;
          for (int nb = it0; nb < it1; nb += 4) {
            const int it = nb + s4;
            const bool okit = it < it1;
            const float *g3p = sG3 + (size_t)(okit ? it : it0) * GS * 4 + jc * GS + 4 * g;
            f4 dW = zero4();
#pragma unroll
            for (int m = 0; m < NM; ++m) {
              float4 bq = *(const float4 *)&g3p[16 * m];
              if (!okit) bq = make_float4(0.f, 0.f, 0.f, 0.f);
              dW = mfma4(acc[m][0], bq.x, dW);
              dW = mfma4(acc[m][1], bq.y, dW);
              dW = mfma4(acc[m][2], bq.z, dW);
              dW = mfma4(acc[m][3], bq.w, dW);
            }
            if (okit && it >= mib && it < mie) {
              float *wr = sW + (size_t)it * D + j2 * 4 + jc;
#pragma unroll
              for (int v = 0; v < 4; ++v) wr[v * q2 * 4] = dW[v];
            }
          }
          continue;
        }
        // stage 2: lane (g, c) holds T^T[r2 = 16m + 4g + v][row c] of this j2
        const int row = mb * 16 + c;
        const int pr = row >> a.lq1, j1 = row & (q1 - 1);
        const bool okp = pr < nP;
        const int ib = okp ? M.pr_it[pr] : 0, ie = okp ? M.pr_it[pr + 1] : 0;
        const int nk = M.mbf[mb];
        const int col0 = (j1 * q2 + j2) * q3;
        for (int kk = 0; kk < nk; ++kk) {
          const int it = ib + kk;
          const bool act = it < ie;
          const float *g3 = sG3 + (size_t)(act ? it : 0) * GS * q3 + 4 * g;
          // four j3 at a time: independent sums, then lane group g keeps j3 = j30 + g
          for (int j30 = 0; j30 < q3; j30 += 4) {
            float sacc[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const int j3 = min(j30 + u, q3 - 1);
              float x = 0.f;
#pragma unroll
              for (int m = 0; m < NM; ++m) {
                const float4 gv = *(const float4 *)&g3[j3 * GS + 16 * m];
                x += acc[m][0] * gv.x + acc[m][1] * gv.y + acc[m][2] * gv.z + acc[m][3] * gv.w;
              }
              sacc[u] = x;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) sacc[u] = sum_lane_groups(sacc[u]);
            const float val = g == 0 ? sacc[0] : (g == 1 ? sacc[1] : (g == 2 ? sacc[2] : sacc[3]));
            const int j3 = j30 + g;
            if (act && j3 < q3) {
              if (SW) {
                sW[(size_t)it * D + col0 + j3] = val;
              } else {
                for (int k = M.it_beg[it]; k < M.it_beg[it + 1]; ++k) {
                  const int e = M.e_perm[k];
                  unsafeAtomicAdd(a.Y + (size_t)M.e_bag[e] * D + col0 + j3, M.e_w[e] * val);
                }
              }
            }
          }
        }
      }
    }
  }
  if (DOT) {  // dL/dw per element: one wave per element, row . grad_out[bag]
    lds_barrier();
    for (int e = w; e < n_el; e += NW) {
      const int it = M.e_it[e], b = M.e_bag[e];
      float acc = 0.f;
      for (int d = lane; d < D; d += 64) acc += sW[(size_t)it * D + d] * a.dY[(size_t)b * D + d];
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
      if (lane == 0) {
        float scale = 1.f;
        if (a.mean) {
          const long long len = a.off[b + 1] - a.off[b];
          scale = 1.f / (float)(len > 0 ? len : 1);
        }
        a.gw[a.srec[2 * (size_t)(M.s0 + e)].x] = acc * scale;  // element position n
      }
    }
    return;
  }
  if (!SW) return;
  // pooling: out[bag] += w * W[item], one row-contiguous pass per element
  if (a.fzero) fwd_wait_out(a, fpoll);  // (includes the barrier)
  else lds_barrier();
  for (int e = w; e < n_el; e += NW) {
    const int it = M.e_it[e];
    float *yrow = a.Y + (size_t)M.e_bag[e] * D;
    const float we = M.e_w[e];
    for (int d = lane; d < D; d += 64) unsafeAtomicAdd(yrow + d, we * sW[(size_t)it * D + d]);
  }
}

// The forward kernel.  Its flags carry this call's tag.  In a captured launch the tag
// counts the clearing forwards on the workspace: the last block to finish (counted in
// hdr[H_FCNT], which the grouping zeroes) moves that count on -- every block has read it
// by then -- and zeroes the block count for the next forward on the same grouping, so a
// replayed launch tags its flags afresh.
template <int RP, bool DOT, bool MF>
__global__ __launch_bounds__(WG) void k_fwd(DevArgs a) {
  if (a.fzero) a.epoch = launch_tag(a, a.hdr + H_FEPOCH);
  fwd_item<RP, DOT, MF>(a);
  if (a.fzero && a.devtag) {
    __syncthreads();  // every wave of the block has read the count
    if (threadIdx.x == 0 && atomicAdd(&a.hdr[H_FCNT], 1) + 1 == (int)gridDim.x) {
      a.hdr[H_FCNT] = 0;
      a.hdr[H_FEPOCH] = a.hdr[H_FEPOCH] + 1;
    }
  }
}

size_t fwd_lds_bytes(int RP, int JB, int P, int q3, int D, int sw) {
  switch (RP) {
    case 16: return FwdLds<16>::bytes(JB, P, q3, D, sw);
    case 32: return FwdLds<32>::bytes(JB, P, q3, D, sw);
    default: return FwdLds<64>::bytes(JB, P, q3, D, sw);
  }
}

// Stage 2 on the matrix cores is chosen when the shape allows it and the work items are
// expected to fit the device at once (two workgroups per CU; groups of the mean size
// nnz / groups cut into P-position items).  Such a launch is bound by each item's chain
// of dependent steps, which the matrix cores shorten; with more items it is bound by
// throughput, where the per-item VALU path does less work (both measured).  A wrong
// guess costs time only.
static bool mf_stage2(const DevArgs &a, int RP, bool dot) {
  if (RP > 32 || a.q1 != 4 || a.q3 != 4 || !(dot || a.fwd_sw) || a.nnz <= 0) return false;
  const long long G = (long long)a.T * a.p2;
  const long long per = (a.nnz + G - 1) / G;
  const long long items = G * ((per + a.P - 1) / a.P);
  return items <= 2LL * device_cus();
}

template <int RP, bool DOT, bool MF>
static hipError_t launch_fwd_k(const DevArgs &a, size_t lds, hipStream_t s) {
  static bool attr_set = false;  // dynamic LDS above 64 KiB is opt-in per kernel
  if (!attr_set) {
    (void)hipFuncSetAttribute((const void *)k_fwd<RP, DOT, MF>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, LDS_DYN_MAX);
    attr_set = true;
  }
  tt_launch(K_FWD, k_fwd<RP, DOT, MF>, dim3(items_max(a)), dim3(WG), lds, s,
            tag_for_launch(a, s));
  return hipGetLastError();
}

template <int RP, bool DOT>
static hipError_t launch_fwd_t(const DevArgs &a, size_t lds, hipStream_t s) {
  if (RP <= 32 && mf_stage2(a, RP, DOT)) return launch_fwd_k<RP, DOT, RP <= 32>(a, lds, s);
  return launch_fwd_k<RP, DOT, false>(a, lds, s);
}

hipError_t launch_wgrad(const DevArgs &a, int RP, size_t lds, hipStream_t s) {
  switch (RP) {
    case 16: return launch_fwd_t<16, true>(a, lds, s);
    case 32: return launch_fwd_t<32, true>(a, lds, s);
    default: return launch_fwd_t<64, true>(a, lds, s);
  }
}

hipError_t launch_fwd(const DevArgs &a, int RP, size_t lds, hipStream_t s) {
  switch (RP) {
    case 16: return launch_fwd_t<16, false>(a, lds, s);
    case 32: return launch_fwd_t<32, false>(a, lds, s);
    default: return launch_fwd_t<64, false>(a, lds, s);
  }
}

}  // namespace ttb
