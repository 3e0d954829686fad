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

// LDS ordering between lanes of one wave (write by one lane, read by another).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

}  // namespace ttb
