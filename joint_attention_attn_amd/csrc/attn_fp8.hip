// FP8 joint-attention forward for gfx950 (Q, K, V in OCP e4m3 with one fp32
// scale per token and head, RoPE already applied by the quantize pass).
//
// FP8 attention is the pages' qk_dtype / v_dtype fp8 setting ("Speed Up Image
// Generation with FLUX 3 Image Klein on NVIDIA Blackwell GPUs", section
// "Quantized and sparse attention").  Both products run on
// v_mfma_f32_32x32x64_f8f6f4 with the same transposed orientation as the bf16
// kernel (a lane owns one query row):
//   S^T[key][q] = K8 . Q8^T, then s = acc * sk[key] * sq[q] * scale (fp32)
//   O^T[d][q]  += V8^T . P'^T
// V's scale is per key, i.e. on the reduction index of P.V, so it is folded
// into P before the e4m3 cast: P'[q][key] = P * sv[key] * 256 / sv_max, where
// sv_max is the largest V scale of the (batch, head).  P' then lies in
// [0, 256] and the epilogue multiplies by sv_max / 256.  The softmax
// normaliser sums the unquantized fp32 P.
#include "common.hpp"
#include "internal.hpp"

namespace ja {

namespace {

constexpr int BM = 128;
constexpr int BN = 64;
constexpr int VT8_STRIDE = BN + 16;  // bytes per transposed-V row in LDS

struct Fp8Args {
  const uint8_t *q, *k, *v;
  const float *sq, *sk, *sv;
  bf16 *o;
  float *lse;
  int64_t o_sb, o_ss, o_sh;
  int S, H;
  float scale_log2;
};

__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  // format 0 = fp8 e4m3 for both operands, no block scaling
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Position of key r (0..63) of a tile inside a transposed-V LDS row, chosen so
// that the 32 keys the P' operand of lane half hf carries are contiguous:
// key = kb*32 + g*8 + hf*4 + i  ->  hf*32 + kb*16 + g*4 + i.
__device__ __forceinline__ int vt8_pos(int r) {
  const int kb = r >> 5, g = (r >> 3) & 3, hf = (r >> 2) & 1, i = r & 3;
  return hf * 32 + kb * 16 + g * 4 + i;
}

template <int D>
__global__ __launch_bounds__(256) void attn_fwd_fp8_kernel(Fp8Args a) {
  constexpr int KCH = D / 16;  // 16-byte chunks per fp8 head vector
  __shared__ __attribute__((aligned(16))) uint8_t Ks[BN * D];
  __shared__ __attribute__((aligned(16))) uint8_t Vt[D * VT8_STRIDE];
  __shared__ __attribute__((aligned(16))) float sk_t[BN];
  __shared__ __attribute__((aligned(16))) float wv_t[BN];
  __shared__ float red[4];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int h = blockIdx.y, b = blockIdx.z;
  const int S = a.S;
  const int64_t bh = (int64_t)b * a.H + h;
  const int64_t row_stride = (int64_t)a.H * D;  // contiguous [B, S, H, D]

  // ---- largest V scale of this (b, h) ----
  float vmax = 0.f;
  for (int s = tid; s < S; s += 256) vmax = fmaxf(vmax, a.sv[bh * S + s]);
  for (int off = 32; off >= 1; off >>= 1) vmax = fmaxf(vmax, __shfl_xor(vmax, off));
  if (lane == 0) red[wave] = vmax;
  __syncthreads();
  const float sv_max = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float wv_mul = 256.f / sv_max;

  // ---- Q8 of this lane's query row ----
  const int qi = blockIdx.x * BM + wave * 32 + l32;
  const int qs = qi < S ? qi : S - 1;
  const uint8_t *qrow = a.q + ((int64_t)b * S + qs) * row_stride + (int64_t)h * D;
  i32x8 qreg[D / 64];
#pragma unroll
  for (int kk = 0; kk < D / 64; ++kk) {
    const i32x4 lo = *reinterpret_cast<const i32x4 *>(qrow + 64 * kk + 32 * hf);
    const i32x4 hi = *reinterpret_cast<const i32x4 *>(qrow + 64 * kk + 32 * hf + 16);
    qreg[kk] = i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    if (qi >= S) qreg[kk] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
  }
  const float qmul = a.sq[bh * S + qs] * a.scale_log2;

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const uint8_t *kbase = a.k + (int64_t)b * S * row_stride + (int64_t)h * D;
  const uint8_t *vbase = a.v + (int64_t)b * S * row_stride + (int64_t)h * D;

  for (int j0 = 0; j0 < S; j0 += BN) {
    for (int c = tid; c < BN * KCH; c += 256) {
      const int r = c / KCH, ch = c % KCH;
      const int key = j0 + r;
      u32x4 kw = {0, 0, 0, 0}, vw = {0, 0, 0, 0};
      if (key < S) {
        kw = *reinterpret_cast<const u32x4 *>(kbase + key * row_stride + ch * 16);
        vw = *reinterpret_cast<const u32x4 *>(vbase + key * row_stride + ch * 16);
      }
      *reinterpret_cast<u32x4 *>(Ks + r * D + ((ch ^ (r & (KCH - 1))) * 16)) = kw;
      const int pos = vt8_pos(r);
      const uint32_t vv[4] = {vw.x, vw.y, vw.z, vw.w};
#pragma unroll
      for (int e = 0; e < 16; ++e)
        Vt[(ch * 16 + e) * VT8_STRIDE + pos] = (uint8_t)(vv[e >> 2] >> (8 * (e & 3)));
    }
    if (tid < BN) {
      const int key = j0 + tid;
      const float skv = key < S ? a.sk[bh * S + key] : 0.f;
      const float svv = key < S ? a.sv[bh * S + key] : 0.f;
      sk_t[tid] = skv;
      wv_t[tid] = svv * wv_mul;
    }
    __syncthreads();

    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
      const int r = kb * 32 + l32;
#pragma unroll
      for (int kk = 0; kk < D / 64; ++kk) {
        const int c0 = 4 * kk + 2 * hf;
        const i32x4 lo = *reinterpret_cast<const i32x4 *>(Ks + r * D + ((c0 ^ (r & (KCH - 1))) * 16));
        const i32x4 hi = *reinterpret_cast<const i32x4 *>(Ks + r * D + (((c0 + 1) ^ (r & (KCH - 1))) * 16));
        const i32x8 kv = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        sacc[kb] = mfma_fp8(kv, qreg[kk], sacc[kb]);
      }
    }

    // t = acc * sk[key]; the row max of t * qmul is qmul * max(t) (qmul > 0)
    float tmax = -INFINITY;
    const bool tail = j0 + BN > S;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 skg = *reinterpret_cast<const float4 *>(&sk_t[kb * 32 + g * 8 + hf * 4]);
        const float skv[4] = {skg.x, skg.y, skg.z, skg.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float t = sacc[kb][4 * g + i] * skv[i];
          if (tail && j0 + kb * 32 + g * 8 + hf * 4 + i >= S) t = -INFINITY;
          sacc[kb][4 * g + i] = t;
          tmax = fmaxf(tmax, t);
        }
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax * qmul);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;

    // P = exp2(t * qmul - m); P' = P * w[key] -> e4m3; operand slot order is
    // kb*16 + g*4 + i, matching vt8_pos.
    uint32_t pw[8];
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 wg = *reinterpret_cast<const float4 *>(&wv_t[kb * 32 + g * 8 + hf * 4]);
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[i] = __builtin_amdgcn_exp2f(fmaf(sacc[kb][4 * g + i], qmul, -m_new));
          psum += p[i];
        }
        int w = __builtin_amdgcn_cvt_pk_fp8_f32(p[0] * wg.x, p[1] * wg.y, 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(p[2] * wg.z, p[3] * wg.w, w, true);
        pw[kb * 4 + g] = (uint32_t)w;
      }
    l_run = l_run * alpha + psum;
    const i32x8 pb = {(int)pw[0], (int)pw[1], (int)pw[2], (int)pw[3],
                      (int)pw[4], (int)pw[5], (int)pw[6], (int)pw[7]};
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
      const uint8_t *vrow = Vt + (db * 32 + l32) * VT8_STRIDE + 32 * hf;
      const i32x4 lo = *reinterpret_cast<const i32x4 *>(vrow);
      const i32x4 hi = *reinterpret_cast<const i32x4 *>(vrow + 16);
      const i32x8 va = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      oacc[db] = mfma_fp8(va, pb, oacc[db]);
    }
    __syncthreads();
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (qi < S) {
    const float inv = sv_max / (256.f * l_tot);
    bf16 *orow = a.o + b * a.o_sb + (int64_t)qi * a.o_ss + h * a.o_sh;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        const int d = db * 32 + 8 * grp + 4 * hf;
        u32x2 w;
        w.x = pack_bf16x2(oacc[db][4 * grp + 0] * inv, oacc[db][4 * grp + 1] * inv);
        w.y = pack_bf16x2(oacc[db][4 * grp + 2] * inv, oacc[db][4 * grp + 3] * inv);
        *reinterpret_cast<u32x2 *>(orow + d) = w;
      }
    if (a.lse && hf == 0) a.lse[bh * S + qi] = (m_run + __log2f(l_tot)) * kLn2;
  }
}

}  // namespace

int fwd_fp8_block_rows(int) { return BM; }

hipError_t launch_fwd_fp8(const AttnLayout &L, const void *q8, const void *k8,
                          const void *v8, const float *sq, const float *sk,
                          const float *sv, void *o, float *lse, hipStream_t st) {
  Fp8Args a;
  a.q = static_cast<const uint8_t *>(q8);
  a.k = static_cast<const uint8_t *>(k8);
  a.v = static_cast<const uint8_t *>(v8);
  a.sq = sq;
  a.sk = sk;
  a.sv = sv;
  a.o = static_cast<bf16 *>(o);
  a.lse = lse;
  a.o_sb = L.o_sb; a.o_ss = L.o_ss; a.o_sh = L.o_sh;
  a.S = L.S;
  a.H = L.H;
  a.scale_log2 = L.scale_log2;
  const dim3 grid((L.S + BM - 1) / BM, L.H, L.B);
  if (L.D == 64)
    hipLaunchKernelGGL(attn_fwd_fp8_kernel<64>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(attn_fwd_fp8_kernel<128>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace ja
