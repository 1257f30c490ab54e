// Device-side vocabulary shared by the gfx950 kernels: vector types, bf16
// packing, and the Q/K prologue (RMS normalization and RoPE in fp64, one
// rounding to the operand format).
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

// ---- The Q/K prologue: the query/key RMS normalization and the RoPE
// rotation that the pages put in the epilogue of the QKV projection ("Speed
// Up Image Generation with FLUX 3 Image Klein on NVIDIA Blackwell GPUs",
// section "GEMM kernel optimization"), evaluated in fp64 and rounded ONCE to
// the operand format (bf16, or e4m3 after the scale):
//   y_d = x_d * r * g_d,  r = 1 / sqrt(sum(x^2) / D + eps)   (optional)
//   (y_2p, y_2p+1) -> (y_2p cos - y_2p+1 sin, y_2p sin + y_2p+1 cos)
// fp64 carries the exact products and, for bf16 inputs, the exact sum of
// squares, so the rounded result is the rounding of the exact value except
// in cases of probability ~2^-40.  The single rounding goes through fp32
// with round-to-odd, which keeps the second rounding (fp32 -> bf16 or e4m3,
// 24 against 8 or 4 significant bits) correct.

// fp64 -> fp32, rounded to odd: truncation toward zero, with the last bit
// set when the result is inexact.
__device__ __forceinline__ float f32_round_odd(double x) {
  const float f = (float)x;                       // to nearest even
  uint32_t u = __float_as_uint(f);
  if ((double)f != x && (u & 1u) == 0) {
    // the odd neighbour on x's side of f
    u += __builtin_fabs(x) > __builtin_fabs((double)f) ? 1 : -1;
  }
  return __uint_as_float(u);
}

// Two fp64 values -> packed bf16x2, each rounded once to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2_f64(double a, double b) {
  return pack_bf16x2(f32_round_odd(a), f32_round_odd(b));
}

// Rotation of one adjacent pair (x, y) by the angle whose (cos, sin) is cs,
// in fp64 (products and difference each rounded, as the formula reads).
__device__ __forceinline__ void rope_pair_f64(double x, double y, double2 cs, double &rx,
                                              double &ry) {
#pragma clang fp contract(off)
  rx = x * cs.x - y * cs.y;
  ry = x * cs.y + y * cs.x;
}

// Sum of squares of the 8 bf16 of a 16-byte chunk, in fp64 (exact: every
// square has 16 significant bits).
__device__ __forceinline__ double chunk_sumsq_f64(u32x4 w) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
  double s = 0.0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const double lo = bf16_lo(ws[e]), hi = bf16_hi(ws[e]);
    s = __builtin_fma(lo, lo, s);
    s = __builtin_fma(hi, hi, s);
  }
  return s;
}

// ---- Reductions over aligned groups of G = 2, 4, 8 or 16 consecutive lanes
//      with DPP row operations (no LDS traffic, no lane arithmetic).  Step 0
//      pairs lanes l and l^1, step 1 lanes l and l^2 (quad permutations),
//      step 2 mirrors each half row (l <-> 7-l within 8 lanes), step 3
//      mirrors each 16-lane row (l <-> 15-l); after steps 0..s every lane of
//      an aligned group of 2^(s+1) lanes holds the combination of the whole
//      group. ----
template <int STEP>
__device__ __forceinline__ uint32_t dpp_row_xchg(uint32_t v) {
  static_assert(STEP >= 0 && STEP < 4, "16-lane rows");
  constexpr int ctrl = STEP == 0 ? 0xB1 : STEP == 1 ? 0x4E : STEP == 2 ? 0x141 : 0x140;
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, ctrl, 0xf, 0xf, false);
}
template <int STEP>
__device__ __forceinline__ double dpp_row_xchg_f64(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint64_t lo = dpp_row_xchg<STEP>((uint32_t)u);
  const uint64_t hi = dpp_row_xchg<STEP>((uint32_t)(u >> 32));
  return __longlong_as_double((long long)((hi << 32) | lo));
}
template <int G>
__device__ __forceinline__ double group_sum_f64(double s) {
  static_assert(G == 1 || G == 2 || G == 4 || G == 8 || G == 16, "group size");
  if constexpr (G > 1) s += dpp_row_xchg_f64<0>(s);
  if constexpr (G > 2) s += dpp_row_xchg_f64<1>(s);
  if constexpr (G > 4) s += dpp_row_xchg_f64<2>(s);
  if constexpr (G > 8) s += dpp_row_xchg_f64<3>(s);
  return s;
}
template <int G>
__device__ __forceinline__ int group_max_i32(int v) {
  static_assert(G == 1 || G == 2 || G == 4 || G == 8 || G == 16, "group size");
  if constexpr (G > 1) v = max(v, (int)dpp_row_xchg<0>((uint32_t)v));
  if constexpr (G > 2) v = max(v, (int)dpp_row_xchg<1>((uint32_t)v));
  if constexpr (G > 4) v = max(v, (int)dpp_row_xchg<2>((uint32_t)v));
  if constexpr (G > 8) v = max(v, (int)dpp_row_xchg<3>((uint32_t)v));
  return v;
}
template <int G>
__device__ __forceinline__ uint32_t group_max_u32(uint32_t v) {
  static_assert(G == 1 || G == 2 || G == 4 || G == 8 || G == 16, "group size");
  if constexpr (G > 1) v = max(v, dpp_row_xchg<0>(v));
  if constexpr (G > 2) v = max(v, dpp_row_xchg<1>(v));
  if constexpr (G > 4) v = max(v, dpp_row_xchg<2>(v));
  if constexpr (G > 8) v = max(v, dpp_row_xchg<3>(v));
  return v;
}

// Sum over the chunks of a row when lane (i % CH) of each aligned group of
// CH consecutive lanes holds chunk i % CH (every lane gets the total).
template <int CH>
__device__ __forceinline__ double chunk_sum_lanes_f64(double s) {
  return group_sum_f64<CH>(s);
}

// max(m, |y|) for m >= 0 as one v_max_f64 with the abs modifier (fmax would
// first canonicalize both operands); a NaN y leaves m (IEEE maxNum).
__device__ __forceinline__ double max_abs_f64(double m, double y) {
  double r;
  asm("v_max_f64 %0, %1, |%2|" : "=v"(r) : "v"(m), "v"(y));
  return r;
}

// r = 1 / sqrt(ss / D + eps) in fp64.
template <int D>
__device__ __forceinline__ double rms_scale_f64(double ss, float eps) {
  return 1.0 / __builtin_sqrt(ss * (1.0 / D) + (double)eps);
}

// The prologue of one 16-byte chunk (elements d0 .. d0+7 of a head vector)
// in fp64: normalized with r and the chunk's 8 weights g (if g), rotated
// with the chunk's 4 table entries cs (if rope; held in registers).
__device__ __forceinline__ void prologue_chunk_f64_regs(u32x4 w, double r, const float *g,
                                                        bool rope, const double2 (&cs)[4],
                                                        double (&y)[8]) {
#pragma clang fp contract(off)
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    y[2 * e] = bf16_lo(ws[e]);
    y[2 * e + 1] = bf16_hi(ws[e]);
  }
  if (g) {
    const float4 g0 = reinterpret_cast<const float4 *>(g)[0];
    const float4 g1 = reinterpret_cast<const float4 *>(g)[1];
    const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = y[e] * r * (double)gv[e];
  }
  if (rope) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const double x0 = y[2 * e], x1 = y[2 * e + 1];
      rope_pair_f64(x0, x1, cs[e], y[2 * e], y[2 * e + 1]);
    }
  }
}

// The same with the chunk's 8 norm weights already in registers (used if
// norm).
__device__ __forceinline__ void prologue_chunk_f64_w(u32x4 w, double r, bool norm,
                                                     const float (&gv)[8], bool rope,
                                                     const double2 (&cs)[4], double (&y)[8]) {
#pragma clang fp contract(off)
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    y[2 * e] = bf16_lo(ws[e]);
    y[2 * e + 1] = bf16_hi(ws[e]);
  }
  if (norm) {
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = y[e] * r * (double)gv[e];
  }
  if (rope) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const double x0 = y[2 * e], x1 = y[2 * e + 1];
      rope_pair_f64(x0, x1, cs[e], y[2 * e], y[2 * e + 1]);
    }
  }
}

// The same with the chunk's 4 table entries read from cs (if cs).
__device__ __forceinline__ void prologue_chunk_f64(u32x4 w, double r, const float *g,
                                                   const double2 *cs, double (&y)[8]) {
#pragma clang fp contract(off)
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    y[2 * e] = bf16_lo(ws[e]);
    y[2 * e + 1] = bf16_hi(ws[e]);
  }
  if (g) {
    const float4 g0 = reinterpret_cast<const float4 *>(g)[0];
    const float4 g1 = reinterpret_cast<const float4 *>(g)[1];
    const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = y[e] * r * (double)gv[e];
  }
  if (cs) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const double2 t = cs[e];
      const double x0 = y[2 * e], x1 = y[2 * e + 1];
      rope_pair_f64(x0, x1, t, y[2 * e], y[2 * e + 1]);
    }
  }
}

// Eight fp64 values rounded once to bf16 (nearest even), packed.  The
// nearest fp32 value rounds to the same bf16 unless it lands exactly on a
// bf16 midpoint (low 16 bits 0x8000) without being the fp64 value itself;
// only then (about one element in 2^16) the round-to-odd path runs.
__device__ __forceinline__ u32x4 pack8_bf16_f64(const double (&y)[8]) {
  float f[8];
  bool tie = false;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    f[e] = (float)y[e];
    tie = tie || (__float_as_uint(f[e]) & 0xffffu) == 0x8000u;
  }
  if (tie) {
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = f32_round_odd(y[e]);
  }
  return u32x4{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
               pack_bf16x2(f[6], f[7])};
}

// The prologue of a chunk rounded to bf16 (the MFMA operand).
__device__ __forceinline__ u32x4 prologue_chunk_bf16(u32x4 w, double r, const float *g,
                                                     const double2 *cs) {
  double y[8];
  prologue_chunk_f64(w, r, g, cs, y);
  return pack8_bf16_f64(y);
}

// Key held by slot p (0..15) of a 16-key group in the P operand of the P.V
// MFMA: the S^T accumulator gives lane half hf = p / 8 the keys
// 4hf + {0..3} and 4hf + {8..11} of the group, in that order.  V^T rows store
// the keys of each group in this slot order so that one 16-byte read is the
// matching A operand.
__host__ __device__ constexpr int vt_key_of_slot(int p) {
  return 4 * (p / 8) + (p % 8 < 4 ? p % 8 : p % 8 + 4);
}
// BF16 path: keys per tile of the prepared V^T (one 64-byte row per
// head-dimension column and tile).
constexpr int kVtTile = 32;

// FP8 forward: position of key r (0..63) of a tile inside a V^T row: the P' operand of
// lane half hf holds, in slot kb*16 + g*4 + i, key kb*32 + g*8 + hf*4 + i
// (the S^T accumulator order), so V^T keeps that key at hf*32 + slot.
__host__ __device__ constexpr int vt8_pos(int r) {
  return ((r >> 2) & 1) * 32 + (r >> 5) * 16 + ((r >> 3) & 3) * 4 + (r & 3);
}

// Quotient of a 32-bit numerator by a runtime divisor d >= 1 through a
// precomputed multiplier (round-up method): q = (umulhi(n, m) + n) >> s with
// 2^(s-1) < d <= 2^s and m = 2^32 (2^s - d) / d + 1; the add is 64-bit, so
// every n < 2^32 divides exactly.
struct FastDiv {
  uint32_t d = 1, m = 1, s = 0;
};
inline FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  f.d = d;
  while ((1ull << f.s) < d) ++f.s;
  f.m = (uint32_t)(((1ull << 32) * ((1ull << f.s) - d)) / d + 1);
  return f;
}
__device__ __forceinline__ uint32_t fast_div(uint32_t n, const FastDiv &f) {
  return (uint32_t)(((uint64_t)__umulhi(n, f.m) + n) >> f.s);
}

// Batch row b, token s and head h of head vector `row` of a [B, S, H]
// sequence of vectors (row = (b S + s) H + h).
template <bool WIDE>
__device__ __forceinline__ void split_row(int64_t row, const FastDiv &fh, const FastDiv &fs,
                                          int64_t &b, int64_t &s, int &h) {
  if constexpr (WIDE) {
    h = (int)(row % fh.d);
    const int64_t t = row / fh.d;
    s = t % fs.d;
    b = t / fs.d;
  } else {
    const uint32_t r = (uint32_t)row;
    const uint32_t t = fast_div(r, fh);
    h = (int)(r - t * fh.d);
    const uint32_t bb = fast_div(t, fs);
    s = (int64_t)(t - bb * fs.d);
    b = bb;
  }
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
