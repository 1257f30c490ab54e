// RoPE + per-token FP8 (e4m3) quantization of Q, K and V for gfx950.
//
// The pages switch attention to FP8 Q/K and V (qk_dtype / v_dtype fp8,
// "Speed Up Image Generation with FLUX 3 Image Klein on NVIDIA Blackwell
// GPUs", section "Quantized and sparse attention").  Granularity and format
// here: one fp32 scale per (batch, token, head) head vector, codes in OCP
// e4m3 (v_cvt_pk_fp8_f32 produces OCP e4m3 on gfx950), round to nearest even,
// saturated at +-448.  V's scale is amax/448.  Q's and K's is the smallest
// power of two s with amax <= 448 s (an E8M0 exponent, which the fp8 matrix
// core applies exactly in Q K^T).
//
// The pass is HBM-bound (read bf16, write 1-byte codes): each head vector of
// D elements is handled by D/8 lanes with one 16-byte load each; its amax is
// reduced with lane exchanges inside that lane group.  A lane handles RPT
// head vectors and issues all their loads first, so that enough bytes are in
// flight to cover the HBM latency.
//
// Precision: Q and K go through the fp64 prologue (RMS norm, RoPE) of
// common.hpp; amax and the power-of-two scale come from those fp64 values,
// and the code is the e4m3 rounding of x * 2^-k taken once (round to odd to
// fp32, then to nearest even).  V's scale is the IEEE fp32 quotient
// amax / 448, and its code the e4m3 rounding of the exact quotient x / scale:
// the fp32 division is correctly rounded, an fma gives its exact remainder,
// and that decides the round-to-odd fp32 value that the e4m3 conversion
// rounds once more (correctly, with 24 against 4 significant bits).
#include "common.hpp"
#include "internal.hpp"

namespace ja {

namespace {

struct QuantArgs {
  const bf16 *x[3];
  int64_t sb[3], ss[3], sh[3];
  uint8_t *x8[3];
  float *scale[3];
  const double2 *rope;    // RoPE table [S][D/2] (cos, sin) in fp64
  const float *norm[2];   // Q / K RMS-norm weights [D], NULL = none
  float eps;
  int S, H;
  int64_t rows;  // B * S * H
  FastDiv fh, fs;  // division by H and by S
};

constexpr int RPT = 2;        // head vectors per lane

// Four fp32 values -> packed e4m3 (nearest even), saturated at +-448.
__device__ __forceinline__ uint32_t pack_e4m3x4(const float (&y)[4]) {
  float c[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) c[j] = fminf(fmaxf(y[j], -448.f), 448.f);
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], lo, true);
}

// Whether an fp32 value lies within `ulps` of an e4m3 rounding midpoint (or
// in e4m3's subnormal range, where the midpoints are spaced differently):
// there the e4m3 rounding of the value and of a value `ulps` away may differ.
// In the normal range a midpoint has a 1 in mantissa bit 19 and zeros below.
__device__ __forceinline__ bool near_e4m3_midpoint(float f, uint32_t ulps) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t low = u & 0xfffffu;
  const bool tiny = (u & 0x7fffffffu) < 0x3c800000u && (u & 0x7fffffffu) != 0u;  // 0 < |f| < 2^-6
  return tiny || (low + ulps - 0x80000u) <= 2u * ulps;
}

// x / scale rounded to odd in fp32, from the correctly rounded quotient and
// its exact remainder (x, scale > 0 finite fp32).
__device__ __forceinline__ float div_round_odd(float x, float scale) {
  const float q = x / scale;
  const float t = __builtin_fmaf(q, scale, -x);        // q scale - x, exact
  uint32_t u = __float_as_uint(q);
  if (t != 0.f && (u & 1u) == 0) {
    // the exact quotient lies beyond q (larger magnitude) when q scale falls
    // short of x in magnitude
    const bool up = x > 0.f ? t < 0.f : t > 0.f;
    u += up ? 1 : -1;
  }
  return __uint_as_float(u);
}

template <int D, bool WIDE>
__device__ __forceinline__ void quant_row(const QuantArgs &a, int t, int64_t row, int sub,
                                          u32x4 w) {
  constexpr int LPR = D / 8;  // lanes per head vector
  const bool live = row < a.rows;
  int64_t b, s;
  int h;
  split_row<WIDE>(live ? row : 0, a.fh, a.fs, b, s, h);
  float scale = 1.f;
  uint32_t packed[2];
  if (t < 2) {
    // Q, K: the fp64 prologue, amax and a power-of-two scale
    const float *g = a.norm[t];
    double rn = 0.0;
    if (g) rn = rms_scale_f64<D>(chunk_sum_lanes_f64<LPR>(chunk_sumsq_f64(w)), a.eps);
    double y[8];
    prologue_chunk_f64(w, rn, g ? g + sub * 8 : nullptr,
                       a.rope ? a.rope + s * (D / 2) + sub * 4 : nullptr, y);
    double amax = 0.0;
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = __builtin_fmax(amax, __builtin_fabs(y[e]));
#pragma unroll
    for (int off = 1; off < LPR; off <<= 1) amax = __builtin_fmax(amax, __shfl_xor(amax, off));
    // amax = m 2^E with m in [1, 2) and 448 = 1.75 2^8: s = 2^(E-8), or
    // 2^(E-7) when m > 1.75; at least 2^-126
    int k = 0;
    if (amax > 0.0) {
      const uint64_t ab = __double_as_longlong(amax);
      const int e2 = (int)(ab >> 52) - 1023;
      k = max(e2 - 8 + ((ab & 0xfffffffffffffull) > 0xc000000000000ull ? 1 : 0), -126);
      scale = __uint_as_float((uint32_t)(127 + k) << 23);
    }
    // codes of y 2^-k: the nearest fp32 value rounds to the same e4m3 unless
    // it is itself a midpoint (then round to odd from the fp64 value)
    float v[8];
    bool tie = false;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[e] = (float)__builtin_ldexp(y[e], -k);
      tie = tie || near_e4m3_midpoint(v[e], 0);
    }
    if (tie) {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = f32_round_odd(__builtin_ldexp(y[e], -k));
    }
    packed[0] = pack_e4m3x4({v[0], v[1], v[2], v[3]});
    packed[1] = pack_e4m3x4({v[4], v[5], v[6], v[7]});
  } else {
    // V: exact in fp32; scale = amax / 448
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
    float x[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = bf16_lo(ww[e]);
      x[2 * e + 1] = bf16_hi(ww[e]);
    }
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x[e]));
#pragma unroll
    for (int off = 1; off < LPR; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    if (amax > 0.f) scale = amax / 448.f;
    // x / scale through the reciprocal: within two fp32 ulps of the exact
    // quotient (two roundings of 2^-24), so its e4m3 rounding is the exact
    // one unless it sits within three ulps of a midpoint; only then the
    // correctly rounded division
    const float inv = 1.f / scale;
    float v[8];
    bool near = false;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      v[e] = x[e] * inv;
      near = near || near_e4m3_midpoint(v[e], 3);
    }
    if (near) {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = div_round_odd(x[e], scale);
    }
    packed[0] = pack_e4m3x4({v[0], v[1], v[2], v[3]});
    packed[1] = pack_e4m3x4({v[4], v[5], v[6], v[7]});
  }
  if (live) {
    *reinterpret_cast<u32x2 *>(a.x8[t] + row * D + sub * 8) = u32x2{packed[0], packed[1]};
    if (sub == 0) a.scale[t][(b * a.H + h) * a.S + s] = scale;
  }
}

// Workgroup of 256 lanes: RPT blocks of 256 / LPR consecutive head vectors.
// WIDE: more than 2^32 head vectors (64-bit index arithmetic).
template <int D, bool WIDE>
__global__ __launch_bounds__(256) void quant_rope_fp8_kernel(QuantArgs a) {
  constexpr int LPR = D / 8;
  constexpr int ROWS = 256 / LPR;
  const int t = blockIdx.y;   // 0 = Q, 1 = K, 2 = V
  const int sub = threadIdx.x % LPR;
  const int64_t row0 = (int64_t)blockIdx.x * ROWS * RPT + threadIdx.x / LPR;
  u32x4 w[RPT];
#pragma unroll
  for (int j = 0; j < RPT; ++j) {
    const int64_t row = row0 + j * ROWS;
    int64_t b, s;
    int h;
    split_row<WIDE>(row < a.rows ? row : 0, a.fh, a.fs, b, s, h);
    w[j] = *reinterpret_cast<const u32x4 *>(a.x[t] + b * a.sb[t] + s * a.ss[t] + h * a.sh[t] +
                                            sub * 8);
  }
#pragma unroll
  for (int j = 0; j < RPT; ++j) quant_row<D, WIDE>(a, t, row0 + j * ROWS, sub, w[j]);
}

template <int D>
void launch_quant(const QuantArgs &a, dim3 grid, hipStream_t st) {
  if (a.rows >= (1ll << 32))
    hipLaunchKernelGGL((quant_rope_fp8_kernel<D, true>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((quant_rope_fp8_kernel<D, false>), grid, dim3(256), 0, st, a);
}

}  // namespace

hipError_t launch_quant_rope_fp8(const AttnLayout &L, const void *q,
                                 const void *k, const void *v,
                                 const double *rope, void *q8, void *k8,
                                 void *v8, float *sq, float *sk, float *sv,
                                 hipStream_t st) {
  QuantArgs a;
  a.x[0] = static_cast<const bf16 *>(q);
  a.x[1] = static_cast<const bf16 *>(k);
  a.x[2] = static_cast<const bf16 *>(v);
  a.sb[0] = L.q_sb; a.ss[0] = L.q_ss; a.sh[0] = L.q_sh;
  a.sb[1] = L.k_sb; a.ss[1] = L.k_ss; a.sh[1] = L.k_sh;
  a.sb[2] = L.v_sb; a.ss[2] = L.v_ss; a.sh[2] = L.v_sh;
  a.x8[0] = static_cast<uint8_t *>(q8);
  a.x8[1] = static_cast<uint8_t *>(k8);
  a.x8[2] = static_cast<uint8_t *>(v8);
  a.scale[0] = sq;
  a.scale[1] = sk;
  a.scale[2] = sv;
  a.rope = reinterpret_cast<const double2 *>(rope);
  a.norm[0] = L.q_norm;
  a.norm[1] = L.k_norm;
  a.eps = L.norm_eps;
  a.S = L.S;
  a.H = L.H;
  a.rows = (int64_t)L.B * L.S * L.H;
  a.fh = make_fastdiv((uint32_t)L.H);
  a.fs = make_fastdiv((uint32_t)L.S);
  const int64_t rows_per_wg = (256 / (L.D / 8)) * RPT;
  const dim3 grid((unsigned)((a.rows + rows_per_wg - 1) / rows_per_wg), 3);
  if (L.D == 64)
    launch_quant<64>(a, grid, st);
  else
    launch_quant<128>(a, grid, st);
  return hipGetLastError();
}

}  // namespace ja
