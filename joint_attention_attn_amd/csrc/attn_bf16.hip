// BF16 joint-attention forward for gfx950 with RoPE fused into the Q/K load.
//
// Joint attention ("Speed Up Image Generation with FLUX 3 Image Klein on
// NVIDIA Blackwell GPUs", section "FLUX 3 inference with TensorRT LLM
// VisualGen"): one dense softmax over the concatenated text / target / reference
// tokens.  RoPE is applied to Q and K before the product (same page, section
// "GEMM kernel optimization"); here it is applied in fp32 while Q and K are
// loaded and the rotated values are rounded to bf16 for the MFMA.
//
// Work decomposition: one workgroup per (128-query block, head, batch row),
// four wave64s of 32 query rows each.  Both products are computed transposed
// so that a lane owns one query row throughout:
//   S^T[key][q]  = K . Q^T      (v_mfma_f32_32x32x16_bf16, A = K from LDS,
//                                B = rotated Q kept in registers)
//   O^T[d][q]   += V^T . P^T    (A = V^T from LDS, B = P straight from the
//                                S^T accumulators)
// With that orientation the online-softmax state (running max m and sum l,
// fp32, exp2 domain) is per lane, the row max needs one cross-half exchange
// and the O rescale is one multiply per accumulator.
#include "common.hpp"
#include "internal.hpp"

namespace ja {

namespace {

constexpr int BM = 128;     // query rows per workgroup
constexpr int BN = 64;      // keys per K/V tile
constexpr int VT_PAD = 8;   // bf16 padding of each transposed-V row in LDS

struct FwdArgs {
  const bf16 *q, *k, *v;
  const float2 *rope;
  bf16 *o;
  float *lse;
  int64_t q_sb, q_ss, q_sh, k_sb, k_ss, k_sh, v_sb, v_ss, v_sh, o_sb, o_ss, o_sh;
  int S, H;
  float scale_log2;
};

template <int D>
__global__ __launch_bounds__(256) void attn_fwd_bf16_kernel(FwdArgs a) {
  constexpr int KCH = D / 8;              // 16-byte chunks per head vector
  constexpr int VT_STRIDE = BN + VT_PAD;  // bf16 per transposed-V row
  __shared__ __attribute__((aligned(16))) bf16 Ks[BN * D];
  __shared__ __attribute__((aligned(16))) bf16 Vt[D * VT_STRIDE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;
  const int h = blockIdx.y, b = blockIdx.z;
  const int S = a.S;

  // ---- Q rows of this lane: rotate, round to bf16, keep in registers ----
  const int qi = blockIdx.x * BM + wave * 32 + l32;
  const int qs = qi < S ? qi : S - 1;
  const bf16 *qrow = a.q + b * a.q_sb + (int64_t)qs * a.q_ss + h * a.q_sh;
  bf16x8 qreg[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    const int d0 = 16 * kk + 8 * hf;
    u32x4 w = *reinterpret_cast<const u32x4 *>(qrow + d0);
    if (a.rope) w = rope_chunk_bf16(w, a.rope + (int64_t)qs * (D / 2) + d0 / 2);
    if (qi >= S) w = u32x4{0, 0, 0, 0};
    qreg[kk] = bit_cast<bf16x8>(w);
  }

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const bf16 *kbase = a.k + b * a.k_sb + h * a.k_sh;
  const bf16 *vbase = a.v + b * a.v_sb + h * a.v_sh;

  for (int j0 = 0; j0 < S; j0 += BN) {
    // ---- stage K (rotated) and V^T of this tile in LDS ----
    for (int c = tid; c < BN * KCH; c += 256) {
      const int r = c / KCH, ch = c % KCH;
      const int key = j0 + r;
      u32x4 kw = {0, 0, 0, 0}, vw = {0, 0, 0, 0};
      if (key < S) {
        kw = *reinterpret_cast<const u32x4 *>(kbase + (int64_t)key * a.k_ss + ch * 8);
        if (a.rope) kw = rope_chunk_bf16(kw, a.rope + (int64_t)key * (D / 2) + ch * 4);
        vw = *reinterpret_cast<const u32x4 *>(vbase + (int64_t)key * a.v_ss + ch * 8);
      }
      // 16-byte chunks of a K row are XOR-swizzled by the row index so that
      // the 32 rows read by one MFMA operand load hit distinct banks.
      *reinterpret_cast<u32x4 *>(Ks + r * D + ((ch ^ (r & 7)) * 8)) = kw;
      uint16_t *vt = reinterpret_cast<uint16_t *>(Vt) + (ch * 8) * VT_STRIDE + r;
      const uint32_t vv[4] = {vw.x, vw.y, vw.z, vw.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vt[(2 * e) * VT_STRIDE] = (uint16_t)(vv[e] & 0xffffu);
        vt[(2 * e + 1) * VT_STRIDE] = (uint16_t)(vv[e] >> 16);
      }
    }
    __syncthreads();

    // ---- S^T = K . Q^T for this wave's 32 queries and the tile's 64 keys ----
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
      const int r = kb * 32 + l32;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const int ch = 2 * kk + hf;
        const bf16x8 kv = *reinterpret_cast<const bf16x8 *>(Ks + r * D + ((ch ^ (r & 7)) * 8));
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kv, qreg[kk], sacc[kb], 0, 0, 0);
      }
    }

    // ---- online softmax (exp2 domain); accumulator row i of block kb is
    //      key kb*32 + 8*(i/4) + 4*hf + i%4 ----
    float mloc = -INFINITY;
    const bool tail = j0 + BN > S;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float s = sacc[kb][i] * a.scale_log2;
        if (tail) {
          const int key = j0 + kb * 32 + 8 * (i / 4) + 4 * hf + (i % 4);
          if (key >= S) s = -INFINITY;
        }
        sacc[kb][i] = s;
        mloc = fmaxf(mloc, s);
      }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    const float m_new = fmaxf(m_run, mloc);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;

    bf16x8 pb[2][2];
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = __builtin_amdgcn_exp2f(sacc[kb][g * 8 + 2 * e] - m_new);
          const float p1 = __builtin_amdgcn_exp2f(sacc[kb][g * 8 + 2 * e + 1] - m_new);
          w[e] = pack_bf16x2(p0, p1);
          // the normaliser sums the same bf16-rounded P that feeds P.V
          psum += bf16_lo(w[e]) + bf16_hi(w[e]);
        }
        pb[kb][g] = bit_cast<bf16x8>(u32x4{w[0], w[1], w[2], w[3]});
      }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;

    // ---- O^T += V^T . P^T ; P operand slot j of half hf (block kb, group g)
    //      is key kb*32 + 16g + 4hf + (j<4 ? j : j+4) ----
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const uint16_t *vrow = reinterpret_cast<const uint16_t *>(Vt) + (db * 32 + l32) * VT_STRIDE;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const int base = kb * 32 + g * 16 + 4 * hf;
          const u32x2 lo = *reinterpret_cast<const u32x2 *>(vrow + base);
          const u32x2 hi = *reinterpret_cast<const u32x2 *>(vrow + base + 8);
          const bf16x8 va = bit_cast<bf16x8>(u32x4{lo.x, lo.y, hi.x, hi.y});
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[kb][g], oacc[db], 0, 0, 0);
        }
    }
    __syncthreads();
  }

  // ---- epilogue: O = acc / l, bf16; LSE in natural log ----
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (qi < S) {
    const float inv = 1.f / l_tot;
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
    if (a.lse && hf == 0)
      a.lse[((int64_t)b * a.H + h) * S + qi] = (m_run + __log2f(l_tot)) * kLn2;
  }
}

}  // namespace

int fwd_bf16_block_rows(int) { return BM; }

hipError_t launch_fwd_bf16(const AttnLayout &L, const void *q, const void *k,
                           const void *v, const float *rope, void *o,
                           float *lse, hipStream_t st) {
  FwdArgs a;
  a.q = static_cast<const bf16 *>(q);
  a.k = static_cast<const bf16 *>(k);
  a.v = static_cast<const bf16 *>(v);
  a.rope = reinterpret_cast<const float2 *>(rope);
  a.o = static_cast<bf16 *>(o);
  a.lse = lse;
  a.q_sb = L.q_sb; a.q_ss = L.q_ss; a.q_sh = L.q_sh;
  a.k_sb = L.k_sb; a.k_ss = L.k_ss; a.k_sh = L.k_sh;
  a.v_sb = L.v_sb; a.v_ss = L.v_ss; a.v_sh = L.v_sh;
  a.o_sb = L.o_sb; a.o_ss = L.o_ss; a.o_sh = L.o_sh;
  a.S = L.S;
  a.H = L.H;
  a.scale_log2 = L.scale_log2;
  const dim3 grid((L.S + BM - 1) / BM, L.H, L.B);
  if (L.D == 64)
    hipLaunchKernelGGL(attn_fwd_bf16_kernel<64>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(attn_fwd_bf16_kernel<128>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace ja
