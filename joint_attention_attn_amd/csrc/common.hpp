// Device-side vocabulary shared by the gfx950 kernels: vector types,
// bf16 packing and the RoPE pair rotation.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ja {

typedef __bf16 bf16;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

template <typename To, typename From>
__device__ __forceinline__ To bit_cast(const From &f) {
  static_assert(sizeof(To) == sizeof(From), "size mismatch");
  return __builtin_bit_cast(To, f);
}

// Two fp32 -> packed bf16x2 (round to nearest even; low half = a).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  return bit_cast<uint32_t>(__builtin_convertvector(v, bf16x2));
}

// The two bf16 of a packed word, widened exactly to fp32.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// RoPE of one adjacent pair (x, y) by the angle whose (cos, sin) is cs:
// (x c - y s, x s + y c) in fp32 with a fixed operation order, the y term
// rounded on its own and the x term fused onto it:
//   rx = fma(x, c, -fl(y s)),  ry = fma(x, s, fl(y c)).
// The result is later rounded to bf16 or e4m3, so the order is pinned down
// (no compiler contraction) to make those rounding decisions reproducible.
__device__ __forceinline__ void rope_pair_f32(float x, float y, float2 cs, float &rx,
                                              float &ry) {
#pragma clang fp contract(off)
  const float ys = y * cs.y;
  const float yc = y * cs.x;
  rx = __builtin_fmaf(x, cs.x, -ys);
  ry = __builtin_fmaf(x, cs.y, yc);
}

// The same rotation of a packed bf16 pair, rounded back to packed bf16.
__device__ __forceinline__ uint32_t rope_pair_bf16(uint32_t w, float2 cs) {
  float rx, ry;
  rope_pair_f32(bf16_lo(w), bf16_hi(w), cs, rx, ry);
  return pack_bf16x2(rx, ry);
}

// Rotate the 8 bf16 (4 pairs) of a 16-byte chunk with 4 consecutive table
// entries.
__device__ __forceinline__ u32x4 rope_chunk_bf16(u32x4 w, const float2 *cs) {
  const float4 t01 = reinterpret_cast<const float4 *>(cs)[0];
  const float4 t23 = reinterpret_cast<const float4 *>(cs)[1];
  u32x4 r;
  r.x = rope_pair_bf16(w.x, make_float2(t01.x, t01.y));
  r.y = rope_pair_bf16(w.y, make_float2(t01.z, t01.w));
  r.z = rope_pair_bf16(w.z, make_float2(t23.x, t23.y));
  r.w = rope_pair_bf16(w.w, make_float2(t23.z, t23.w));
  return r;
}

// ---- query/key RMS normalization ("Speed Up Image Generation with FLUX 3
// Image Klein on NVIDIA Blackwell GPUs", section "GEMM kernel optimization":
// query/key normalization next to RoPE in the QKV epilogue), applied in fp32
// before the rotation:  y_d = fl(fl(x_d * r) * g_d),
// r = 1 / sqrt(ss / D + eps) with IEEE fp32 square root and division.  The sum
// of squares ss has one fixed order wherever it is computed: chunk c of 8
// elements accumulates fma(x, x, s) over its elements from 0, then the chunk
// sums combine pairwise with partner c ^ k for k = 2, 4, ..., D/16, then
// k = 1 (a butterfly: every chunk ends with the same total).

// Sum of squares of the 8 bf16 of a 16-byte chunk, in element order.
__device__ __forceinline__ float chunk_sumsq(u32x4 w) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    s = __builtin_fmaf(bf16_lo(ws[e]), bf16_lo(ws[e]), s);
    s = __builtin_fmaf(bf16_hi(ws[e]), bf16_hi(ws[e]), s);
  }
  return s;
}

// Butterfly over the chunk sums when lane (i % CH) of each group of CH
// consecutive lanes holds chunk i % CH.
template <int CH>
__device__ __forceinline__ float chunk_sum_lanes(float s) {
#pragma unroll
  for (int k = 2; k < CH; k <<= 1) s = s + __shfl_xor(s, k);
  if constexpr (CH > 1) s = s + __shfl_xor(s, 1);
  return s;
}

// r = 1 / sqrt(ss / D + eps); D is a power of two, so ss / D is exact.
template <int D>
__device__ __forceinline__ float rms_scale(float ss, float eps) {
  return 1.f / __builtin_sqrtf(ss * (1.f / D) + eps);
}

// The 8 values of a chunk normalized: fl(fl(x * r) * g) with g the chunk's 8
// weights.
__device__ __forceinline__ void norm_chunk(u32x4 w, float r, const float *g, float (&y)[8]) {
#pragma clang fp contract(off)
  const float4 g0 = reinterpret_cast<const float4 *>(g)[0];
  const float4 g1 = reinterpret_cast<const float4 *>(g)[1];
  const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    y[2 * e] = (bf16_lo(ws[e]) * r) * gv[2 * e];
    y[2 * e + 1] = (bf16_hi(ws[e]) * r) * gv[2 * e + 1];
  }
}

// Normalize (if g) and rotate (if cs) a chunk, rounded to bf16.
__device__ __forceinline__ u32x4 norm_rope_chunk_bf16(u32x4 w, float r, const float *g,
                                                      const float2 *cs) {
  float y[8];
  norm_chunk(w, r, g, y);
  u32x4 o;
  uint32_t *op = reinterpret_cast<uint32_t *>(&o);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float rx = y[2 * e], ry = y[2 * e + 1];
    if (cs) rope_pair_f32(y[2 * e], y[2 * e + 1], cs[e], rx, ry);
    op[e] = pack_bf16x2(rx, ry);
  }
  return o;
}

// Key held by slot p (0..15) of a 16-key group in the P operand of the P.V
// MFMA: the S^T accumulator gives lane half hf = p / 8 the keys
// 4hf + {0..3} and 4hf + {8..11} of the group, in that order.  V^T rows store
// the keys of each group in this slot order so that one 16-byte read is the
// matching A operand.
__host__ __device__ constexpr int vt_key_of_slot(int p) {
  return 4 * (p / 8) + (p % 8 < 4 ? p % 8 : p % 8 + 4);
}

// FP8 forward: position of key r (0..63) of a tile inside a V^T row: the P' operand of
// lane half hf holds, in slot kb*16 + g*4 + i, key kb*32 + g*8 + hf*4 + i
// (the S^T accumulator order), so V^T keeps that key at hf*32 + slot.
__host__ __device__ constexpr int vt8_pos(int r) {
  return ((r >> 2) & 1) * 32 + (r >> 5) * 16 + ((r >> 3) & 3) * 4 + (r & 3);
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// vmcnt-only wait (gfx9 s_waitcnt encoding: vmcnt bits 3:0 and 15:14,
// expcnt and lgkmcnt at their maxima, i.e. not waited for).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt(0x0f70 | (N & 15) | ((N >> 4) << 14));
}

// Workgroup barrier with no memory fence: a fence would make the compiler
// wait for every load to LDS in flight, including the ones for later tiles.
// The visibility that matters is ordered by hand (each wave waits for its own
// loads of the next tile before the barrier); the empty asm statements keep
// the compiler from moving LDS accesses across it.
__device__ __forceinline__ void tile_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

// LDS destination of a buffer load to LDS
#define JA_LDS_PTR(p) ((__attribute__((address_space(3))) void *)(p))

}  // namespace ja
