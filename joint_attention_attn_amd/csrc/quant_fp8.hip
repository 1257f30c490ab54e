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
// Each head vector of D elements is handled by D/8 lanes with one 16-byte
// load each; its amax (V) or scale exponent (Q, K) is reduced over that lane
// group with DPP row exchanges.  A lane handles RPT head vectors and issues
// all their loads first, so that enough bytes are in flight to cover the HBM
// latency.  The fp64 prologue makes the pass issue-bound rather than
// HBM-bound, so the per-element work is kept to the fp64 rotation, one max,
// the scaling and a two-instruction boundary test.
//
// Precision: Q and K go through the fp64 prologue (RMS norm, RoPE) of
// common.hpp; amax and the power-of-two scale come from those fp64 values,
// and the code is the e4m3 rounding of x * 2^-k taken once (round to odd to
// fp32, then to nearest even).  V's scale is the IEEE fp32 quotient
// amax / 448, and its code the e4m3 rounding of the exact quotient x / scale:
// near a rounding boundary, the fp32 division is correctly rounded, an fma
// gives its exact remainder, and that decides the round-to-odd fp32 value
// that the e4m3 conversion rounds once more (correctly, with 24 against 4
// significant bits).
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

constexpr int RPT = 4;        // head vectors per lane

// Four fp32 values -> packed e4m3 (nearest even).  No clamp is needed: a Q/K
// value times 2^-k is at most 448 by the choice of k, and a V quotient
// exceeds 448 by at most a few fp32 ulps (the scale is the rounded
// amax / 448), which rounds to 448 (the rounding boundary above it is 464).
__device__ __forceinline__ uint32_t pack_e4m3x4(const float (&y)[4]) {
  int any;
  asm volatile("" : "=v"(any));      // the first conversion's upper half is overwritten
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], any, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], lo, true);
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

// a / 448 correctly rounded, for a bf16 value a > 0: the product with the
// rounded reciprocal, corrected once with its exact remainder (checked
// against IEEE division for every positive finite bf16 value).
__device__ __forceinline__ float div448(float a) {
  constexpr float r = 1.0f / 448.0f;
  const float q0 = a * r;
  const float rem = __builtin_fmaf(-q0, 448.0f, a);
  return __builtin_fmaf(rem, r, q0);
}

// Position of head vector `row` of a [B, S, H] order.
struct RowPos {
  int64_t b, s;
  int h;
};

// Q or K head vector (t = 0 or 1): the fp64 prologue, amax and a power-of-two
// scale; the chunk's codes and (lane 0 of the group) the scale are stored.
template <int D, bool WIDE, bool NORM, bool ROPE>
__device__ __forceinline__ void quant_qk_row(const QuantArgs &a, int t, int64_t row,
                                             const RowPos &p, int sub, u32x4 w,
                                             const double2 (&cs)[4]) {
  constexpr int LPR = D / 8;  // lanes per head vector
  const float *g = NORM ? a.norm[t] : nullptr;
  double rn = 0.0;
  if (NORM && g) rn = rms_scale_f64<D>(chunk_sum_lanes_f64<LPR>(chunk_sumsq_f64(w)), a.eps);
  double y[8];
  prologue_chunk_f64_regs(w, rn, NORM && g ? g + sub * 8 : nullptr, ROPE, cs, y);
  double amax = 0.0;
#pragma unroll
  for (int e = 0; e < 8; ++e) amax = max_abs_f64(amax, y[e]);
  // the scale's exponent k from amax = m 2^E (m in [1, 2), 448 = 1.75 2^8):
  // k = E - 8, or E - 7 when m > 1.75, at least -126.  k is monotone in
  // amax, so the head vector's k is the largest of its lanes' (a lane whose
  // elements are all zero proposes kNoScale).
  constexpr int kNoScale = -1024;
  int k = kNoScale;
  if (amax > 0.0) {
    const uint64_t ab = (uint64_t)__double_as_longlong(amax);
    const int e2 = (int)(ab >> 52) - 1023;
    k = max(e2 - 8 + ((ab & 0xfffffffffffffull) > 0xc000000000000ull ? 1 : 0), -126);
  }
  k = group_max_i32<LPR>(k);
  float scale = 1.f;
  if (k == kNoScale) k = 0;          // an all-zero head vector: scale 1
  else scale = __uint_as_float((uint32_t)(127 + k) << 23);
  // codes of y 2^-k: fp64 -> fp32 -> e4m3 gives the once-rounded code
  // unless the fp32 value is itself an e4m3 rounding boundary (a midpoint;
  // every such fp32 value has its low 16 bits zero); then round to odd
  float v[8];
  uint32_t low = 0xffffu;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    v[e] = (float)__builtin_ldexp(y[e], -k);
    low = min(low, __float_as_uint(v[e]) & 0xffffu);
  }
  if (low == 0u) {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = f32_round_odd(__builtin_ldexp(y[e], -k));
  }
  if (row < a.rows) {
    *reinterpret_cast<u32x2 *>(a.x8[t] + row * D + sub * 8) =
        u32x2{pack_e4m3x4({v[0], v[1], v[2], v[3]}), pack_e4m3x4({v[4], v[5], v[6], v[7]})};
    if (sub == 0) a.scale[t][(p.b * a.H + p.h) * a.S + p.s] = scale;
  }
}

// V head vector: exact in fp32; scale = amax / 448.
template <int D>
__device__ __forceinline__ void quant_v_row(const QuantArgs &a, int64_t row, const RowPos &p,
                                            int sub, u32x4 w) {
  constexpr int LPR = D / 8;
  const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
  float x[8];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[2 * e] = bf16_lo(ww[e]);
    x[2 * e + 1] = bf16_hi(ww[e]);
  }
  // amax on the magnitudes' bit patterns (ordered like the values), and
  // the lane's smallest nonzero magnitude (zero wraps to the maximum)
  uint32_t am = 0, mn = 0xffffffffu;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t m = __float_as_uint(x[e]) & 0x7fffffffu;
    am = max(am, m);
    mn = min(mn, m - 1u);
  }
  am = group_max_u32<LPR>(am);
  const float amax = __uint_as_float(am);
  const float scale = amax > 0.f ? div448(amax) : 1.f;
  // x / scale through the reciprocal (v_rcp_f32, within one ulp): the
  // product is within three fp32 ulps of the exact quotient, so its e4m3
  // rounding is the exact one unless it sits within four ulps of a midpoint
  // (low 20 mantissa bits within 4 of 0x80000), in e4m3's subnormal range
  // (0 < |x / scale| < 2^-6, where the midpoints lie elsewhere: tested on
  // the smallest nonzero |x| against 2^-5 scale, a superset), or the scale
  // is too small for the reciprocal; only then the correctly rounded
  // division
  const float inv = __builtin_amdgcn_rcpf(scale);
  float v[8];
  uint32_t dist = 0xffffffffu;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    v[e] = x[e] * inv;
    dist = min(dist, (__float_as_uint(v[e]) - 0x7fffcu) & 0xfffffu);
  }
  const bool tiny = mn + 1u < __float_as_uint(scale * 0x1p-5f) && mn != 0xffffffffu;
  const bool near = dist <= 8u || tiny || scale < 0x1p-125f;
  if (near) {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = div_round_odd(x[e], scale);
  }
  if (row < a.rows) {
    *reinterpret_cast<u32x2 *>(a.x8[2] + row * D + sub * 8) =
        u32x2{pack_e4m3x4({v[0], v[1], v[2], v[3]}), pack_e4m3x4({v[4], v[5], v[6], v[7]})};
    if (sub == 0) a.scale[2][(p.b * a.H + p.h) * a.S + p.s] = scale;
  }
}

// Workgroup of 256 lanes in 256 / LPR lane groups; lane group g handles the
// RPT consecutive head vectors RPT (blockIdx.x * 256 / LPR + g) + j.  When
// the head count is a multiple of RPT these are heads of one token, whose
// rotation table entries the lanes then load once for all of them.
// blockIdx.y: 0 = Q, 1 = K, 2 = V.  WIDE: more than 2^32 head vectors
// (64-bit index arithmetic); NORM: some RMS-norm weights; ROPE: a table.
template <int D, bool WIDE, bool NORM, bool ROPE>
__global__ __launch_bounds__(256) void quant_rope_fp8_kernel(QuantArgs a) {
  constexpr int LPR = D / 8;
  constexpr int GROUPS = 256 / LPR;
  const int t = blockIdx.y;
  const int sub = threadIdx.x % LPR;
  const int64_t row0 = ((int64_t)blockIdx.x * GROUPS + threadIdx.x / LPR) * RPT;
  // the RPT rows are heads h0 .. h0+RPT-1 of one token when H is a multiple
  // of RPT (rows = B S H then is a multiple of RPT too, so a group is whole)
  const bool shared = a.H % RPT == 0;
  u32x4 w[RPT];
  RowPos p[RPT];
  if (shared) {
    split_row<WIDE>(row0 < a.rows ? row0 : 0, a.fh, a.fs, p[0].b, p[0].s, p[0].h);
    const bf16 *src = a.x[t] + p[0].b * a.sb[t] + p[0].s * a.ss[t] + p[0].h * a.sh[t] + sub * 8;
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
      p[j] = RowPos{p[0].b, p[0].s, p[0].h + j};
      w[j] = *reinterpret_cast<const u32x4 *>(src + j * a.sh[t]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
      const int64_t row = row0 + j;
      split_row<WIDE>(row < a.rows ? row : 0, a.fh, a.fs, p[j].b, p[j].s, p[j].h);
      w[j] = *reinterpret_cast<const u32x4 *>(a.x[t] + p[j].b * a.sb[t] + p[j].s * a.ss[t] +
                                              p[j].h * a.sh[t] + sub * 8);
    }
  }
  if (t == 2) {
#pragma unroll
    for (int j = 0; j < RPT; ++j) quant_v_row<D>(a, row0 + j, p[j], sub, w[j]);
    return;
  }
  // the lane's 4 table entries (cos, sin) of its chunk, per row or shared
  double2 cs[4] = {};
  if (ROPE && shared) {
#pragma unroll
    for (int e = 0; e < 4; ++e) cs[e] = a.rope[p[0].s * (D / 2) + sub * 4 + e];
  }
#pragma unroll
  for (int j = 0; j < RPT; ++j) {
    if (ROPE && !shared) {
#pragma unroll
      for (int e = 0; e < 4; ++e) cs[e] = a.rope[p[j].s * (D / 2) + sub * 4 + e];
    }
    quant_qk_row<D, WIDE, NORM, ROPE>(a, t, row0 + j, p[j], sub, w[j], cs);
  }
}

template <int D, bool WIDE, bool NORM>
void launch_rope_q(const QuantArgs &a, dim3 grid, hipStream_t st) {
  if (a.rope)
    hipLaunchKernelGGL((quant_rope_fp8_kernel<D, WIDE, NORM, true>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((quant_rope_fp8_kernel<D, WIDE, NORM, false>), grid, dim3(256), 0, st, a);
}

template <int D, bool WIDE>
void launch_norm_q(const QuantArgs &a, dim3 grid, hipStream_t st) {
  if (a.norm[0] || a.norm[1])
    launch_rope_q<D, WIDE, true>(a, grid, st);
  else
    launch_rope_q<D, WIDE, false>(a, grid, st);
}

template <int D>
void launch_quant(const QuantArgs &a, dim3 grid, hipStream_t st) {
  if (a.rows >= (1ll << 32))
    launch_norm_q<D, true>(a, grid, st);
  else
    launch_norm_q<D, false>(a, grid, st);
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
