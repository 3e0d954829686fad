// tt_mfma.h -- the fp32 matrix-core primitive used by the contraction kernels.
//
// v_mfma_f32_16x16x4_f32 (CDNA3/CDNA4 ISA): D(16x16) = A(16x4) * B(4x16) + C, full
// fp32.  Lane l of the wave (64 lanes) supplies A[l % 16][l / 16] and
// B[l / 16][l % 16]; it holds D[4*(l/16) + v][l % 16] for v = 0..3.
//
// Naming used throughout: lane = 16*g + c with g = l/16 (the "lane group") and
// c = l%16 (the "column").  Because a contraction is a plain sum, the k index of
// one instruction may stand for any set of four contraction indices as long as A
// and B use the same mapping; the kernels use that freedom to feed results of one
// MFMA (rows 4g+v held by lane group g) straight into the B operand of the next.
#pragma once
#include <hip/hip_runtime.h>

namespace ttb {

typedef float f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f4 mfma4(float a, float b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f4 zero4() {
  f4 z = {0.f, 0.f, 0.f, 0.f};
  return z;
}

// max over the 64 lanes of a wave
__device__ __forceinline__ int wave_max(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o));
  return v;
}

// Sum of x over the four lane groups (lanes l, l^16, l^32, l^48), returned to all
// four.  gfx950's permlane swaps exchange row halves of two registers in VALU:
// swapping x with itself and adding gives x + x[l^32], then x + x[l^16].
__device__ __forceinline__ float sum_lane_groups(float x) {
  const unsigned u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const unsigned uy = __float_as_uint(y);
  const auto b = __builtin_amdgcn_permlane16_swap(uy, uy, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Pins a loaded value on every lane of the wave.  Without it the compiler may sink a
// load whose result is used only under a per-lane condition into a divergent
// branch, where it gets a full wait of its own instead of overlapping the others.
__device__ __forceinline__ float keep(float v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Workgroup barrier that orders LDS accesses only.  __syncthreads() also makes the
// wave's global stores visible to the workgroup, which on this hardware means waiting for
// every store in flight to complete (a memory round trip per barrier); the contraction
// kernels' barriers guard LDS data alone, so they wait for LDS operations only and leave
// their global stores (partial sums read by a later kernel) in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Wait for every vector-memory operation of the wave (s_waitcnt vmcnt(0), the other
// counters left alone).  Staging loops whose LDS stores sit in divergent branches leave the
// compiler unsure whether their loads are done, so it puts a vmcnt(0) wait into the next
// loop that reuses those registers; that wait then also stalls on the loop's own global
// stores on every pass.  One wait after staging settles it once.
__device__ __forceinline__ void vmem_drain() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// LDS ordering between lanes of one wave (write by one lane, read by another).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// Placement of the M-blocks (16-row blocks) of a contraction workgroup on its waves.  An
// 8-wave workgroup puts two waves on each SIMD of its CU, but a work item has fewer
// M-blocks than waves (6 of 8 is typical), so with the identity map two SIMDs carry twice
// the matrix work of the other two -- in both workgroups that share a CU.  Each wave
// records where it runs (hardware register HW_ID: wave slot [3:0], SIMD [5:4]); after a
// barrier every wave derives the same map: M-blocks go round-robin over the SIMDs, the
// CU's first workgroup (it holds the lowest wave slots) starting at SIMD 0 and the second
// at SIMD 2, so that the two workgroups' extra M-blocks land on different SIMDs.  Any
// other placement (not two waves per SIMD) keeps the identity map.  Correctness does not
// depend on the map: it is a permutation of the waves.
__device__ __forceinline__ void note_placement(int *s_pl) {  // before a barrier
  if ((threadIdx.x & 63) == 0)
    s_pl[threadIdx.x >> 6] = (int)__builtin_amdgcn_s_getreg((5 << 11) | 4);  // HW_ID[5:0]
}
// the same value on every lane of the wave, held in a scalar register (values read from
// LDS or derived from threadIdx.x / 64 that the compiler cannot prove uniform otherwise)
__device__ __forceinline__ int wave_uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

template <int NWAVES>
__device__ __forceinline__ int placed_mblock(const int *s_pl) {  // after the barrier
  const int w = wave_uniform(threadIdx.x >> 6);
  const int my = wave_uniform((s_pl[w] >> 4) & 3);
  // waves per SIMD packed 8 bits each, the lowest wave slot on SIMD 0, and this wave's rank
  // among the waves of its SIMD (all uniform over the wave)
  unsigned per = 0u;
  int slot0 = 16, rank = 0;
#pragma unroll
  for (int v = 0; v < NWAVES; ++v) {
    const int x = wave_uniform(s_pl[v]), sm = (x >> 4) & 3;
    per += 1u << (8 * sm);
    if (sm == 0) slot0 = min(slot0, x & 15);
    rank += (v < w && sm == my) ? 1 : 0;
  }
  if (per != (unsigned)(NWAVES / 4) * 0x01010101u || NWAVES % 4) return w;
  const int rot = slot0 >= 2 ? 2 : 0;
  return rank * 4 + ((my - rot) & 3);
}

}  // namespace ttb
