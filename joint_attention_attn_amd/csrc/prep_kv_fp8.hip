// K/V preparation of the FP8 forward: the e4m3 K and V of each (batch, head)
// in the layouts that the attention kernel copies into LDS tile by tile
// without touching them, and the per-key values its softmax needs.
//
// FP8 attention is the pages' qk_dtype / v_dtype fp8 setting ("Speed Up Image
// Generation with FLUX 3 Image Klein on NVIDIA Blackwell GPUs", section
// "Quantized and sparse attention"); the repair bias is the VC-Attention
// repair of the same section.
//
// Layout of the prepared buffer (S_pad = S rounded up to 64 keys, T = S_pad/64
// tiles; rows and keys past S are 0):
//   K8  [B*H][S_pad][D]   e4m3 keys, one row per key;
//   V8t [B*H][D][S_pad]   V transposed, one row per head-dimension column; in
//                         every 64-key tile key r sits at byte vt8_pos(r), the
//                         order in which the attention kernel's P' operand
//                         holds the keys;
//   info [B*H][T][256]    32-bit words per tile: bias[64] (fp32), inv[64]
//                         (fp32), ke[64] (int32), the softmax scale c in the
//                         exp2 domain (fp32), 63 zero words.
// Per key: bias = log2(sv) / c plus the repair bias (-inf for a repaired
// key); inv = 1 / sv; ke = the E8M0 exponent of sk, i.e. its fp32 exponent
// field.  Past the end: bias = -inf, inv = 0, ke = 127.  A K scale that is
// not a positive normal power of two, or a V scale that is not positive and
// finite, makes the key's bias NaN, which turns every row of the head into
// NaN in the forward.
#include "common.hpp"
#include "internal.hpp"

namespace ja {

namespace {

constexpr int PT = 256;       // threads per workgroup
constexpr int PK = 64;        // keys per workgroup (one attention tile)
constexpr int INFO_WORDS = 256;

struct Prep8Args {
  const uint8_t *k, *v;       // contiguous [B, S, H, D] e4m3
  const float *sk, *sv;       // [B, H, S]
  const float *kbias;         // [B, H, S] repair bias, NULL = none
  uint8_t *k8, *v8t;
  uint32_t *info;
  float c;
  int S, S_pad, H;
};

// Staged V row r keeps its 16-byte chunk c at c ^ vrow_swz(r): the 16 rows
// 4m + e (m = 0..15) that one transpose read touches then spread over the
// bank groups.
template <int CH>
__device__ __forceinline__ int vrow_swz(int r) { return (r >> 2) & (CH - 1); }

template <int D>
__global__ __launch_bounds__(PT) void prep_kv_fp8_kernel(Prep8Args a) {
  constexpr int CH = D / 16;          // 16-byte chunks per row
  __shared__ __attribute__((aligned(16))) uint8_t vs[PK * D];
  const int tid = threadIdx.x;
  const int nt = a.S_pad / PK;
  const int tile = blockIdx.x % nt;
  const int k0 = tile * PK;
  const int bh = blockIdx.x / nt;
  const int b = bh / a.H, h = bh % a.H;
  const int64_t row = (int64_t)a.H * D;
  const uint8_t *kb = a.k + (int64_t)b * a.S * row + (int64_t)h * D;
  const uint8_t *vb = a.v + (int64_t)b * a.S * row + (int64_t)h * D;
  uint8_t *krb = a.k8 + (int64_t)bh * a.S_pad * D;
  uint8_t *vtb = a.v8t + (int64_t)bh * D * a.S_pad;
  uint32_t *info = a.info + ((int64_t)bh * nt + tile) * INFO_WORDS;

  // K rows copied as they are; V rows staged in LDS
#pragma unroll
  for (int idx = tid; idx < PK * CH; idx += PT) {
    const int r = idx / CH, ch = idx % CH;
    const int key = k0 + r;
    u32x4 kw = {0, 0, 0, 0}, vw = {0, 0, 0, 0};
    if (key < a.S) {
      kw = *reinterpret_cast<const u32x4 *>(kb + key * row + 16 * ch);
      vw = *reinterpret_cast<const u32x4 *>(vb + key * row + 16 * ch);
    }
    *reinterpret_cast<u32x4 *>(krb + (int64_t)key * D + 16 * ch) = kw;
    *reinterpret_cast<u32x4 *>(vs + r * D + 16 * (ch ^ vrow_swz<CH>(r))) = vw;
  }

  // per-key values
  if (tid < PK) {
    const int key = k0 + tid;
    float bias = -INFINITY, inv = 0.f;
    int ke = 127;
    if (key < a.S) {
      const int64_t si = (int64_t)bh * a.S + key;
      const float skv = a.sk[si], svv = a.sv[si];
      const uint32_t u = __float_as_uint(skv);
      const uint32_t e = u >> 23;                 // includes the sign bit
      const bool ok = (u & 0x7fffffu) == 0 && e != 0 && e < 255 && svv > 0.f && svv < INFINITY;
      ke = ok ? (int)e : 127;
      inv = ok ? 1.f / svv : 0.f;
      bias = ok ? log2f(svv) / a.c : __builtin_nanf("");
      if (a.kbias) bias += a.kbias[si];
    }
    info[tid] = __float_as_uint(bias);
    info[PK + tid] = __float_as_uint(inv);
    info[2 * PK + tid] = (uint32_t)ke;
  } else if (tid < 2 * PK) {
    info[2 * PK + tid] = tid == PK ? __float_as_uint(a.c) : 0u;
  }
  __syncthreads();

  // V^T: each thread transposes a block of 4 keys x 4 columns (bytes) and
  // writes 4 bytes into each of 4 V^T rows; keys 4m..4m+3 are contiguous in
  // the P' order, at vt8_pos(4m)
#pragma unroll
  for (int idx = tid; idx < (PK / 4) * (D / 4); idx += PT) {
    const int m = idx % (PK / 4), dq = idx / (PK / 4);
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 4 * m + e;
      w[e] = *reinterpret_cast<const uint32_t *>(vs + r * D + 16 * ((dq / 4) ^ vrow_swz<CH>(r)) +
                                                 4 * (dq % 4));
    }
    // w[e] holds columns 4dq..+3 of key 4m+e; u[j] gets keys 4m..+3 of column 4dq+j
    const uint32_t t01l = __builtin_amdgcn_perm(w[1], w[0], 0x05010400u);
    const uint32_t t01h = __builtin_amdgcn_perm(w[1], w[0], 0x07030602u);
    const uint32_t t23l = __builtin_amdgcn_perm(w[3], w[2], 0x05010400u);
    const uint32_t t23h = __builtin_amdgcn_perm(w[3], w[2], 0x07030602u);
    const uint32_t u[4] = {__builtin_amdgcn_perm(t23l, t01l, 0x05040100u),
                           __builtin_amdgcn_perm(t23l, t01l, 0x07060302u),
                           __builtin_amdgcn_perm(t23h, t01h, 0x05040100u),
                           __builtin_amdgcn_perm(t23h, t01h, 0x07060302u)};
    const int pos = k0 + vt8_pos(4 * m);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<uint32_t *>(vtb + (int64_t)(4 * dq + j) * a.S_pad + pos) = u[j];
  }
}

}  // namespace

int prep8_pad(int S) { return (S + PK - 1) / PK * PK; }

int64_t prep_kv_fp8_bytes(const AttnLayout &L) {
  const int64_t sp = prep8_pad(L.S);
  return (int64_t)L.B * L.H * (2 * sp * L.D + (sp / PK) * INFO_WORDS * 4);
}

hipError_t launch_prep_kv_fp8(const AttnLayout &L, const void *k8, const void *v8,
                              const float *sk, const float *sv, const float *kbias, void *kv8,
                              hipStream_t st) {
  Prep8Args a;
  a.k = static_cast<const uint8_t *>(k8);
  a.v = static_cast<const uint8_t *>(v8);
  a.sk = sk;
  a.sv = sv;
  a.kbias = kbias;
  a.S = L.S;
  a.S_pad = prep8_pad(L.S);
  a.H = L.H;
  a.c = L.scale_log2;
  const int64_t kv = (int64_t)L.B * L.H * a.S_pad * L.D;
  a.k8 = static_cast<uint8_t *>(kv8);
  a.v8t = a.k8 + kv;
  a.info = reinterpret_cast<uint32_t *>(a.v8t + kv);
  const dim3 grid((unsigned)((int64_t)(a.S_pad / PK) * L.B * L.H));
  if (L.D == 64)
    hipLaunchKernelGGL(prep_kv_fp8_kernel<64>, grid, dim3(PT), 0, st, a);
  else
    hipLaunchKernelGGL(prep_kv_fp8_kernel<128>, grid, dim3(PT), 0, st, a);
  return hipGetLastError();
}

}  // namespace ja
