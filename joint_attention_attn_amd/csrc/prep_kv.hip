// K/V preparation pass of the BF16 forward: K rotated once per (batch, head)
// and V written transposed, both in the layouts that the attention kernel
// copies into LDS tile by tile without touching them.
//
// RoPE on K ("Speed Up Image Generation with FLUX 3 Image Klein on NVIDIA
// Blackwell GPUs", section "GEMM kernel optimization", where it is fused into
// the epilogue that produces Q and K): here it is fused into this pass's
// single load of K, with the same fp64 rotation and single bf16 rounding as
// the Q load of the attention kernel.  Every workgroup of the attention kernel
// reads each K tile once, so rotating there would redo the rotation (and its
// table reads) once per query block.
//
// A workgroup covers 64 keys of HG heads of one batch row (HG = 2, or 1 for
// an odd head count): the rotation table entries of a key are read once and
// applied to the key's rows in both heads.  (Four heads share the table
// reads better but need 64 KB of LDS per workgroup, which leaves two
// workgroups per CU: too few loads in flight for this HBM-bound pass.)
//
// Layout of the prepared buffer, Kr then Vt (S_pad = S rounded up to 64
// keys; rows and columns past S are 0):
//   Kr [B*H][S_pad][D]  rotated K, one row per key;
//   Vt [B*H][S_pad/32][D][32]  V transposed in tiles of 32 keys: per tile
//                       one 64-byte row per head-dimension column, so that a
//                       tile of the attention kernel is one contiguous 8 KB
//                       (D = 128) block; in every 16-key group the keys are
//                       stored in the order in which the attention kernel's
//                       P operand holds them (position p holds key
//                       vt_key_of_slot(p)).
#include "common.hpp"
#include "internal.hpp"

namespace ja {

namespace {

constexpr int PT = 256;       // threads per workgroup
constexpr int PK = 64;        // keys per workgroup

struct PrepArgs {
  const bf16 *k, *v;
  const double2 *rope;  // RoPE table [S][D/2] (cos, sin) in fp64
  const float *kn;     // K RMS-norm weights [D], NULL = none
  float eps;
  bf16 *kr, *vt;
  int64_t k_sb, k_ss, k_sh, v_sb, v_ss, v_sh;
  int S, S_pad, H, B;
};

// Staged V row r keeps its 16-byte chunk c at c ^ vchunk_swz(r): the eight
// rows that a transpose read touches at once (keys 0, 4, 16, 20, 32, 36, 48,
// 52 plus a multiple of 2 or 8, see below) then sit in distinct bank groups.
template <int CH>
__device__ __forceinline__ int vchunk_swz(int r) {
  return (2 * (((r >> 2) & 1) | (((r >> 4) & 3) << 1))) & (CH - 1);
}

template <int D, bool ROPE, int HG>
__global__ __launch_bounds__(PT, 3) void prep_kv_bf16_kernel(PrepArgs a) {
  constexpr int CH = D / 8;          // 16-byte chunks per row
  constexpr int IT = PK * CH / PT;   // chunk positions per thread
  static_assert(PK * CH % PT == 0 && PT % CH == 0, "whole rows per pass");
  __shared__ __attribute__((aligned(16))) bf16 vs[HG * PK * D];
  const int tid = threadIdx.x;
  const int nkb = a.S_pad / PK;
  const int ng = a.H / HG;
  // XCD-aware order: workgroups go round-robin over the 8 XCDs, and XCD x
  // takes key blocks x, x + 8, ... with all (batch row, head group) pairs of
  // a key block back to back, so that the key block's rotation table rows
  // are fetched into that XCD's L2 once
  const int nbg = a.B * ng;                      // (batch row, head group) pairs
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int kb = (slot / nbg) * 8 + xcd;
  const int bg = slot % nbg;                     // (batch row, head group)
  if (kb >= nkb) return;
  const int k0 = kb * PK;
  const int b = bg / ng, h0 = (bg % ng) * HG;
  const int64_t bh0 = (int64_t)b * a.H + h0;

  // A thread holds chunk c of keys r0, r0 + PT/CH, ... (IT of them) in each
  // of the HG heads.  Every load of the workgroup's share of K, V and the
  // rotation table is issued before any of them is used: the pass is bound
  // by the bytes it keeps in flight, and stores in between would keep the
  // compiler from hoisting later loads above them.
  const int c = tid % CH, r0 = tid / CH;
  // the chunk's norm weights (the same for every key and head of the thread;
  // loaded first, so that waiting for them waits for nothing else)
  float gw[8];
  if (a.kn) {
    const float4 g0 = reinterpret_cast<const float4 *>(a.kn + 8 * c)[0];
    const float4 g1 = reinterpret_cast<const float4 *>(a.kn + 8 * c)[1];
    gw[0] = g0.x; gw[1] = g0.y; gw[2] = g0.z; gw[3] = g0.w;
    gw[4] = g1.x; gw[5] = g1.y; gw[6] = g1.z; gw[7] = g1.w;
  }
  // Loads are unconditional (a key past S reads key S-1; its V and its
  // rotated K are replaced by zeros), so the compiler keeps them together.
  // K and V are read once: non-temporal loads keep them from displacing
  // cache lines that are reused (the table; the prepared buffer, which the
  // forward reads right after).
  u32x4 kw[IT][HG], vw[IT][HG];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int ks = min(k0 + r0 + it * (PT / CH), a.S - 1);
#pragma unroll
    for (int g = 0; g < HG; ++g) {
      kw[it][g] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(
          a.k + b * a.k_sb + (h0 + g) * a.k_sh + (int64_t)ks * a.k_ss + 8 * c));
      vw[it][g] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(
          a.v + b * a.v_sb + (h0 + g) * a.v_sh + (int64_t)ks * a.v_ss + 8 * c));
    }
  }
  // the 4 table entries of each of the thread's keys (pairs 4c .. 4c+3)
  double2 cs[IT][4];
  if constexpr (ROPE) {
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int ks = min(k0 + r0 + it * (PT / CH), a.S - 1);
#pragma unroll
      for (int e = 0; e < 4; ++e) cs[it][e] = a.rope[(int64_t)ks * (D / 2) + 4 * c + e];
    }
  }
#pragma unroll
  for (int it = 0; it < IT; ++it)
    if (k0 + r0 + it * (PT / CH) >= a.S)
#pragma unroll
      for (int g = 0; g < HG; ++g) vw[it][g] = u32x4{0, 0, 0, 0};

  // V: staged row-major in LDS for the transpose below
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int r = r0 + it * (PT / CH);
#pragma unroll
    for (int g = 0; g < HG; ++g)
      *reinterpret_cast<u32x4 *>(vs + (g * PK + r) * D + 8 * (c ^ vchunk_swz<CH>(r))) = vw[it][g];
  }
  // K: (normalize,) rotate, round once, store.  The CH chunks of a row are
  // CH consecutive lanes, so the norm's butterfly runs inside each lane group
  // (every lane takes part; rows past S are zeros).
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int key = k0 + r0 + it * (PT / CH);
#pragma unroll
    for (int g = 0; g < HG; ++g) {
      u32x4 x = kw[it][g];
      if (a.kn || ROPE) {
        double rn = 0.0;
        if (a.kn) rn = rms_scale_f64<D>(chunk_sum_lanes_f64<CH>(chunk_sumsq_f64(x)), a.eps);
        double y[8];
        prologue_chunk_f64_w(x, rn, a.kn != nullptr, gw, ROPE, cs[it], y);
        x = pack8_bf16_f64(y);
      }
      if (key >= a.S) x = u32x4{0, 0, 0, 0};
      *reinterpret_cast<u32x4 *>(a.kr + ((bh0 + g) * a.S_pad + key) * D + 8 * c) = x;
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
    const bf16 *vsg = vs + g * PK * D;
    bf16 *vtb = a.vt + (bh0 + g) * D * a.S_pad;
    uint32_t w[4], x[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int p0 = 8 * j + 2 * e, p1 = p0 + 1;
      const int r0 = 16 * (p0 / 16) + vt_key_of_slot(p0 % 16);
      const int r1 = 16 * (p1 / 16) + vt_key_of_slot(p1 % 16);
      const uint32_t v0 = *reinterpret_cast<const uint32_t *>(
          vsg + r0 * D + 8 * ((d / 8) ^ vchunk_swz<CH>(r0)) + d % 8);
      const uint32_t v1 = *reinterpret_cast<const uint32_t *>(
          vsg + r1 * D + 8 * ((d / 8) ^ vchunk_swz<CH>(r1)) + d % 8);
      w[e] = __builtin_amdgcn_perm(v1, v0, 0x05040100u);    // row d:   key r0 | key r1
      x[e] = __builtin_amdgcn_perm(v1, v0, 0x07060302u);    // row d+1: key r0 | key r1
    }
    const int kk = k0 + 8 * j;           // first key of the chunk
    bf16 *vtt = vtb + (int64_t)(kk / kVtTile) * (D * kVtTile) + kk % kVtTile;
    *reinterpret_cast<u32x4 *>(vtt + d * kVtTile) = u32x4{w[0], w[1], w[2], w[3]};
    *reinterpret_cast<u32x4 *>(vtt + (d + 1) * kVtTile) = u32x4{x[0], x[1], x[2], x[3]};
  }
}

template <int D, bool ROPE>
void launch_rope(const PrepArgs &a, dim3 grid, int hg, hipStream_t st) {
  if (hg == 2)
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
                               const double *rope, void *kv, hipStream_t st) {
  PrepArgs a;
  a.k = static_cast<const bf16 *>(k);
  a.v = static_cast<const bf16 *>(v);
  a.rope = reinterpret_cast<const double2 *>(rope);
  a.kn = L.k_norm;
  a.eps = L.norm_eps;
  a.kr = static_cast<bf16 *>(kv);
  a.vt = a.kr + (int64_t)L.B * L.H * prep_pad(L.S) * L.D;
  a.k_sb = L.k_sb; a.k_ss = L.k_ss; a.k_sh = L.k_sh;
  a.v_sb = L.v_sb; a.v_ss = L.v_ss; a.v_sh = L.v_sh;
  a.S = L.S;
  a.S_pad = prep_pad(L.S);
  a.H = L.H;
  a.B = L.B;
  const int hg = L.H % 2 == 0 ? 2 : 1;
  // every XCD gets ceil(nkb / 8) key blocks (the excess workgroups exit)
  const int64_t nkb8 = (a.S_pad / PK + 7) / 8 * 8;
  const dim3 grid((unsigned)(nkb8 * L.B * (L.H / hg)));
  if (L.D == 64)
    launch_group<64>(a, grid, rope != nullptr, hg, st);
  else
    launch_group<128>(a, grid, rope != nullptr, hg, st);
  return hipGetLastError();
}

}  // namespace ja
