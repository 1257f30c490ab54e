// K/V preparation pass of the BF16 forward: K rotated once per (batch, head)
// and V written transposed, both in the layouts that the attention kernel
// copies into LDS tile by tile without touching them.
//
// RoPE on K ("Speed Up Image Generation with FLUX 3 Image Klein on NVIDIA
// Blackwell GPUs", section "GEMM kernel optimization", where it is fused into
// the epilogue that produces Q and K): here it is fused into this pass's
// single load of K, with the same fp32 pair rotation and bf16 rounding as the
// Q load of the attention kernel.  Every workgroup of the attention kernel
// reads each K tile once, so rotating there would redo the rotation (and its
// table reads) once per query block.
//
// A workgroup covers 64 keys of HG heads of one batch row (HG = 4, 2 or 1,
// whichever divides the head count): the rotation table entries of a key are
// read once and applied to the key's rows in all HG heads.
//
// Layout of the prepared buffer, Kr then Vt (S_pad = S rounded up to 64
// keys; rows and columns past S are 0):
//   Kr [B*H][S_pad][D]  rotated K, one row per key;
//   Vt [B*H][D][S_pad]  V transposed, one row per head-dimension column; in
//                       every 16-key group the keys are stored in the order
//                       in which the attention kernel's P operand holds them
//                       (position p holds key vt_key_of_slot(p)).
#include "common.hpp"
#include "internal.hpp"

namespace ja {

namespace {

constexpr int PT = 256;       // threads per workgroup
constexpr int PK = 64;        // keys per workgroup

struct PrepArgs {
  const bf16 *k, *v;
  const float2 *rope;
  const float *kn;     // K RMS-norm weights [D], NULL = none
  float eps;
  bf16 *kr, *vt;
  int64_t k_sb, k_ss, k_sh, v_sb, v_ss, v_sh;
  int S, S_pad, H;
};

template <int D, bool ROPE, int HG>
__global__ __launch_bounds__(PT) void prep_kv_bf16_kernel(PrepArgs a) {
  constexpr int CH = D / 8;          // 16-byte chunks per row
  constexpr int VSTR = D + 8;        // bf16 per staged V row (16-byte pad)
  __shared__ __attribute__((aligned(16))) bf16 vs[HG * PK * VSTR];
  const int tid = threadIdx.x;
  const int nkb = a.S_pad / PK;
  const int k0 = (blockIdx.x % nkb) * PK;
  const int bg = blockIdx.x / nkb;               // (batch row, head group)
  const int ng = a.H / HG;
  const int b = bg / ng, h0 = (bg % ng) * HG;
  const int64_t bh0 = (int64_t)b * a.H + h0;

  // K: (normalize,) rotate and copy; V: stage row-major in LDS.  The CH
  // chunks of a row are CH consecutive lanes, so the norm's butterfly runs
  // inside each lane group (every lane takes part; rows past S are zeros).
  // All loads of a chunk position are issued before any of them is used.
#pragma unroll
  for (int idx = tid; idx < PK * CH; idx += PT) {
    const int r = idx / CH, c = idx % CH;
    const int key = k0 + r;
    u32x4 kw[HG], vw[HG];
#pragma unroll
    for (int g = 0; g < HG; ++g) {
      kw[g] = u32x4{0, 0, 0, 0};
      vw[g] = u32x4{0, 0, 0, 0};
      if (key < a.S) {
        kw[g] = *reinterpret_cast<const u32x4 *>(a.k + b * a.k_sb + (h0 + g) * a.k_sh +
                                                 (int64_t)key * a.k_ss + 8 * c);
        vw[g] = *reinterpret_cast<const u32x4 *>(a.v + b * a.v_sb + (h0 + g) * a.v_sh +
                                                 (int64_t)key * a.v_ss + 8 * c);
      }
    }
    float2 cs[4];
    const bool rot = ROPE && key < a.S;
    if (rot) {
      const float4 *t = reinterpret_cast<const float4 *>(a.rope + (int64_t)key * (D / 2) + 4 * c);
      const float4 t01 = t[0], t23 = t[1];
      cs[0] = make_float2(t01.x, t01.y);
      cs[1] = make_float2(t01.z, t01.w);
      cs[2] = make_float2(t23.x, t23.y);
      cs[3] = make_float2(t23.z, t23.w);
    }
#pragma unroll
    for (int g = 0; g < HG; ++g) {
      u32x4 x = kw[g];
      if (a.kn) {
        const float ss = chunk_sum_lanes<CH>(chunk_sumsq(x));
        x = norm_rope_chunk_bf16(x, rms_scale<D>(ss, a.eps), a.kn + 8 * c, rot ? cs : nullptr);
      } else if (rot) {
        x = u32x4{rope_pair_bf16(x.x, cs[0]), rope_pair_bf16(x.y, cs[1]),
                  rope_pair_bf16(x.z, cs[2]), rope_pair_bf16(x.w, cs[3])};
      }
      *reinterpret_cast<u32x4 *>(a.kr + ((bh0 + g) * a.S_pad + key) * D + 8 * c) = x;
      *reinterpret_cast<u32x4 *>(vs + (g * PK + r) * VSTR + 8 * c) = vw[g];
    }
  }
  __syncthreads();

  // V^T: rows d and d+1, 8 keys per 16-byte chunk, in P-slot order within
  // 16-key groups.  One 4-byte LDS read holds a key's values in both rows;
  // v_perm_b32 pairs the low halves (row d) and the high halves (row d+1).
#pragma unroll
  for (int idx = tid; idx < HG * (D / 2) * (PK / 8); idx += PT) {
    const int g = idx / ((D / 2) * (PK / 8));
    const int d = 2 * ((idx / (PK / 8)) % (D / 2)), j = idx % (PK / 8);
    const bf16 *vsg = vs + g * PK * VSTR;
    bf16 *vtb = a.vt + (bh0 + g) * D * a.S_pad;
    uint32_t w[4], x[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int p0 = 8 * j + 2 * e, p1 = p0 + 1;
      const int r0 = 16 * (p0 / 16) + vt_key_of_slot(p0 % 16);
      const int r1 = 16 * (p1 / 16) + vt_key_of_slot(p1 % 16);
      const uint32_t v0 = *reinterpret_cast<const uint32_t *>(vsg + r0 * VSTR + d);
      const uint32_t v1 = *reinterpret_cast<const uint32_t *>(vsg + r1 * VSTR + d);
      w[e] = __builtin_amdgcn_perm(v1, v0, 0x05040100u);    // row d:   key r0 | key r1
      x[e] = __builtin_amdgcn_perm(v1, v0, 0x07060302u);    // row d+1: key r0 | key r1
    }
    *reinterpret_cast<u32x4 *>(vtb + (int64_t)d * a.S_pad + k0 + 8 * j) = u32x4{w[0], w[1], w[2], w[3]};
    *reinterpret_cast<u32x4 *>(vtb + (int64_t)(d + 1) * a.S_pad + k0 + 8 * j) =
        u32x4{x[0], x[1], x[2], x[3]};
  }
}

template <int D, bool ROPE>
void launch_rope(const PrepArgs &a, dim3 grid, int hg, hipStream_t st) {
  if (hg == 4)
    hipLaunchKernelGGL((prep_kv_bf16_kernel<D, ROPE, 4>), grid, dim3(PT), 0, st, a);
  else if (hg == 2)
    hipLaunchKernelGGL((prep_kv_bf16_kernel<D, ROPE, 2>), grid, dim3(PT), 0, st, a);
  else
    hipLaunchKernelGGL((prep_kv_bf16_kernel<D, ROPE, 1>), grid, dim3(PT), 0, st, a);
}

template <int D>
void launch_group(const PrepArgs &a, dim3 grid, bool rope, int hg, hipStream_t st) {
  if (rope)
    launch_rope<D, true>(a, grid, hg, st);
  else
    launch_rope<D, false>(a, grid, hg, st);
}

}  // namespace

int prep_pad(int S) { return (S + PK - 1) / PK * PK; }

int64_t prep_kv_bytes(const AttnLayout &L) {
  return 2 * (int64_t)L.B * L.H * prep_pad(L.S) * L.D * 2;
}

hipError_t launch_prep_kv_bf16(const AttnLayout &L, const void *k, const void *v,
                               const float *rope, void *kv, hipStream_t st) {
  PrepArgs a;
  a.k = static_cast<const bf16 *>(k);
  a.v = static_cast<const bf16 *>(v);
  a.rope = reinterpret_cast<const float2 *>(rope);
  a.kn = L.k_norm;
  a.eps = L.norm_eps;
  a.kr = static_cast<bf16 *>(kv);
  a.vt = a.kr + (int64_t)L.B * L.H * prep_pad(L.S) * L.D;
  a.k_sb = L.k_sb; a.k_ss = L.k_ss; a.k_sh = L.k_sh;
  a.v_sb = L.v_sb; a.v_ss = L.v_ss; a.v_sh = L.v_sh;
  a.S = L.S;
  a.S_pad = prep_pad(L.S);
  a.H = L.H;
  const int hg = L.H % 4 == 0 ? 4 : L.H % 2 == 0 ? 2 : 1;
  const dim3 grid((unsigned)((int64_t)(a.S_pad / PK) * L.B * (L.H / hg)));
  if (L.D == 64)
    launch_group<64>(a, grid, rope != nullptr, hg, st);
  else
    launch_group<128>(a, grid, rope != nullptr, hg, st);
  return hipGetLastError();
}

}  // namespace ja
