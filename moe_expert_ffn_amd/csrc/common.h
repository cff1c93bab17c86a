// Device helpers shared by the MoE expert-layer kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define MOE_DEV __device__ __forceinline__

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

namespace moe {

constexpr int kWave = 64;
constexpr int kXcds = 8;          // MI355X: 8 accelerator complex dies
constexpr int kMaxP = 8;

// bf16 is carried as raw 16-bit words; conversions are exact (widen) or
// round-to-nearest-even in hardware (narrow).
MOE_DEV float bf2f(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }
MOE_DEV uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }  // v_cvt_pk_bf16_f32

// Explicit address spaces: LDS (3) and global (1).  Without them a pointer
// that passes through a select or an array decays to a generic pointer and
// every access becomes a flat load that waits on both memory counters.
#define MOE_LDS __attribute__((address_space(3)))
#define MOE_GLB __attribute__((address_space(1)))
// Constant address space: loads of wave-uniform values that are not written
// during the kernel become scalar loads (counted by lgkmcnt, not vmcnt).
#define MOE_CONST __attribute__((address_space(4)))
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
MOE_DEV uint4 ldg16(const void* p) {
  const u32x4_t v = *(const MOE_GLB u32x4_t*)p;
  return make_uint4(v.x, v.y, v.z, v.w);
}
MOE_DEV void stg16(void* p, uint4 v) { *(MOE_GLB u32x4_t*)p = u32x4_t{v.x, v.y, v.z, v.w}; }
MOE_DEV uint4 lds_ld16(const MOE_LDS void* p) {
  const u32x4_t v = *(const MOE_LDS u32x4_t*)p;
  return make_uint4(v.x, v.y, v.z, v.w);
}
MOE_DEV void lds_st16(MOE_LDS void* p, uint4 v) { *(MOE_LDS u32x4_t*)p = u32x4_t{v.x, v.y, v.z, v.w}; }
MOE_DEV void lds_st8(MOE_LDS void* p, uint2 v) { *(MOE_LDS u32x2_t*)p = u32x2_t{v.x, v.y}; }

// OCP e4m3fn -> float, from the format's definition: sign, 4-bit exponent with
// bias 7, 3-bit mantissa, subnormals at exponent 0.  (S.1111.111 = NaN is never
// produced by the weight quantiser and decodes as 480 here.)
MOE_DEV float e4m3_to_f32(uint32_t c) {
  uint32_t ex = (c >> 3) & 0xfu, man = c & 7u;
  float mag = ex ? __uint_as_float(((ex + 120u) << 23) | (man << 20))
                 : (float)man * (1.0f / 512.0f);
  return (c & 0x80u) ? -mag : mag;
}

// Worker (CU partition) of a workgroup.  Workgroups of one dispatch are handed
// to the XCDs round-robin, so blockIdx % 8 is the XCD; worker r owns the XCDs
// x with x * P / 8 == r.  Correctness never depends on the mapping being
// physical: every worker always receives gridDim/ P workgroups.
MOE_DEV int worker_of_block(int P) { return (int)(blockIdx.x % kXcds) * P / kXcds; }

// Wave-wide inclusive prefix sum (64 lanes).
MOE_DEV int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int t = __shfl_up(v, off, 64);
    if (lane >= off) v += t;
  }
  return v;
}

MOE_DEV int wave_sum(int v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

MOE_DEV long long wave_sum64(long long v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Lanes of this wave holding the same value as this lane (value < 2^nbits).
MOE_DEV uint64_t wave_match(uint32_t v, int nbits, bool active) {
  uint64_t m = __ballot(active);
  for (int b = 0; b < nbits; ++b) {
    uint64_t bal = __ballot(active && ((v >> b) & 1u));
    m &= ((v >> b) & 1u) ? bal : ~bal;
  }
  return active ? m : 0ull;
}

MOE_DEV uint64_t lanemask_lt() {
  const int lane = threadIdx.x & 63;
  return lane ? (~0ull >> (64 - lane)) : 0ull;
}

}  // namespace moe
