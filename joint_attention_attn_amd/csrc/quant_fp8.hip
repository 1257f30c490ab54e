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
// flight to cover the HBM latency.  The rotation uses the
// fixed fp32 operation order of rope_pair_f32 and x / scale is IEEE-rounded
// (for a power of two, the exact product x * 2^-k), so the codes are a fixed
// function of the inputs.
#include "common.hpp"
#include "internal.hpp"

namespace ja {

namespace {

struct QuantArgs {
  const bf16 *x[3];
  int64_t sb[3], ss[3], sh[3];
  uint8_t *x8[3];
  float *scale[3];
  const float2 *rope;
  const float *norm[2];   // Q / K RMS-norm weights [D], NULL = none
  float eps;
  int S, H;
  int64_t rows;  // B * S * H
};

constexpr int RPT = 2;        // head vectors per lane

template <int D>
__device__ __forceinline__ void quant_row(const QuantArgs &a, int t, int64_t row, int sub,
                                          u32x4 w) {
  constexpr int LPR = D / 8;  // lanes per head vector
  const bool live = row < a.rows;
  const int64_t rr = live ? row : 0;
  const int h = (int)(rr % a.H);
  const int64_t s = (rr / a.H) % a.S;
  const int64_t b = rr / ((int64_t)a.H * a.S);
  const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
  float r[8];
  const float *g = t < 2 ? a.norm[t] : nullptr;
  if (g) {
    // RMS norm (the LPR lanes of a vector hold its chunks in order), then RoPE
    const float rn = rms_scale<D>(chunk_sum_lanes<LPR>(chunk_sumsq(w)), a.eps);
    norm_chunk(w, rn, g + sub * 8, r);
    if (a.rope) {
      const float2 *cs = a.rope + s * (D / 2) + sub * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x0 = r[2 * e], x1 = r[2 * e + 1];
        rope_pair_f32(x0, x1, cs[e], r[2 * e], r[2 * e + 1]);
      }
    }
  } else if (a.rope && t < 2) {
    const float2 *cs = a.rope + s * (D / 2) + sub * 4;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      rope_pair_f32(bf16_lo(ww[e]), bf16_hi(ww[e]), cs[e], r[2 * e], r[2 * e + 1]);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      r[2 * e] = bf16_lo(ww[e]);
      r[2 * e + 1] = bf16_hi(ww[e]);
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(r[e]));
#pragma unroll
  for (int off = 1; off < LPR; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  float scale = 1.f, inv = 1.f;
  if (t < 2) {
    // amax = m 2^E with m in [1, 2) and 448 = 1.75 2^8: s = 2^(E-8), or
    // 2^(E-7) when m > 1.75; at least 2^-126 (subnormal amax included)
    const uint32_t ab = __float_as_uint(amax);
    const int k = max((int)(ab >> 23) - 135 + ((ab & 0x7fffffu) > 0x600000u ? 1 : 0), -126);
    if (amax > 0.f) {
      scale = __uint_as_float((uint32_t)(127 + k) << 23);
      inv = __uint_as_float((uint32_t)(127 - k) << 23);
    }
  } else if (amax > 0.f) {
    scale = amax / 448.f;
  }

  uint32_t packed[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    float y[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      y[j] = fminf(fmaxf(t < 2 ? r[4 * e + j] * inv : r[4 * e + j] / scale, -448.f), 448.f);
    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
    packed[e] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], lo, true);
  }
  if (live) {
    *reinterpret_cast<u32x2 *>(a.x8[t] + row * D + sub * 8) = u32x2{packed[0], packed[1]};
    if (sub == 0) a.scale[t][(b * a.H + h) * a.S + s] = scale;
  }
}

// Workgroup of 256 lanes: RPT blocks of 256 / LPR consecutive head vectors.
template <int D>
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
    const int64_t rr = row < a.rows ? row : 0;
    const int h = (int)(rr % a.H);
    const int64_t s = (rr / a.H) % a.S;
    const int64_t b = rr / ((int64_t)a.H * a.S);
    w[j] = *reinterpret_cast<const u32x4 *>(a.x[t] + b * a.sb[t] + s * a.ss[t] + h * a.sh[t] +
                                            sub * 8);
  }
#pragma unroll
  for (int j = 0; j < RPT; ++j) quant_row<D>(a, t, row0 + j * ROWS, sub, w[j]);
}

}  // namespace

hipError_t launch_quant_rope_fp8(const AttnLayout &L, const void *q,
                                 const void *k, const void *v,
                                 const float *rope, void *q8, void *k8,
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
  a.rope = reinterpret_cast<const float2 *>(rope);
  a.norm[0] = L.q_norm;
  a.norm[1] = L.k_norm;
  a.eps = L.norm_eps;
  a.S = L.S;
  a.H = L.H;
  a.rows = (int64_t)L.B * L.S * L.H;
  const int64_t rows_per_wg = (256 / (L.D / 8)) * RPT;
  const dim3 grid((unsigned)((a.rows + rows_per_wg - 1) / rows_per_wg), 3);
  if (L.D == 64)
    hipLaunchKernelGGL(quant_rope_fp8_kernel<64>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(quant_rope_fp8_kernel<128>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace ja
