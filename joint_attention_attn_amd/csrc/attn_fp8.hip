// FP8 joint-attention forward for gfx950 (Q, K, V in OCP e4m3 with one fp32
// scale per token and head, RoPE already applied by the quantize pass).
//
// FP8 attention is the pages' qk_dtype / v_dtype fp8 setting ("Speed Up Image
// Generation with FLUX 3 Image Klein on NVIDIA Blackwell GPUs", section
// "Quantized and sparse attention").  Both products run on
// v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3 operands) in the transposed
// orientation of the bf16 kernel, so a lane owns one query row:
//   acc[key][q] = log2(sv[key]) / c + sk[key] sq[q] (K8 . Q8^T)[key][q]
//   O^T[d][q]  += V8^T . P'^T
// Q's and K's scales are powers of two (the quantizer's choice): the MFMA
// applies them exactly as E8M0 block scales.  V's scale is per key, i.e. on
// the reduction index of P.V, where no block scale reaches; it enters the
// exp2 argument through the accumulator's initial value instead, so that
// P' = exp2(c acc - ref) = P sv[key] with c the softmax scale in the exp2
// domain, and P'.V8 is P.V in true units.  The running max of c acc is
// refreshed whenever a row max grows by more than 3, and the reference sits
// 5 below it, so P' stays below 2^8, inside the e4m3 range.  The softmax
// normaliser sums the unquantized fp32 P' / sv[key] (a key with a small V
// scale has a small P', which can vanish in e4m3 while its probability is
// large, so the sum must not use the rounded P').  A key past the end or
// a repaired key starts at -inf.  Per score this leaves a max, an FMA, an
// exp2, the sum's FMA and half a conversion.
//
// Structure: one workgroup of four wave64s per (128-query block, head,
// batch row), three workgroups per CU (three waves per SIMD), XCD-aware
// placement, split of the last round.  A preparation pass (prep_kv_fp8.hip)
// writes each (batch, head)'s K, V^T and per-key values in the layouts of
// the LDS tiles; buffer loads to LDS copy 64-key tiles into a 3-stage ring
// two tiles ahead, with no staging registers and no vector work.  Each wave
// runs Q K^T, softmax and P.V of a tile in turn, and the three waves of a
// SIMD (from three workgroups) overlap one another's matrix and vector work.
//
// Block-sparse variant (the pages' general block-sparse attention kernel,
// section "Quantized and sparse attention", on a given mask of 128-query x
// 64-key blocks): the workgroup (one query block) compacts the list of key
// blocks its query block keeps into LDS and stages only those tiles (one
// 64-key tile is one key block).  Rows that keep no key get O = 0 and
// LSE = -inf.
#include <atomic>

#include "common.hpp"
#include "internal.hpp"

#define JA_INLINE __attribute__((always_inline))

namespace ja {

namespace {

constexpr int BN = 64;              // keys per K/V tile (the MFMA's K extent)

// Workgroup shape: four waves of 32 query rows (one 128-row query block),
// three workgroups per CU, so three waves per SIMD (at most 168 VGPRs each),
// each workgroup over its own 3-stage ring two tiles ahead.  The three
// workgroups of a CU keep their own barriers, so the waves of a SIMD drift
// apart and one's matrix work overlaps another's vector work; one twelve-wave
// workgroup sharing a 4-stage ring (each tile staged once per CU) keeps them
// in step and is 7 % slower at 16896 tokens, 12 % at 4608.  Software
// pipelining inside a wave (Q K^T of the next tile issued ahead of this
// tile's softmax) would keep two tiles of accumulators live, about 245
// VGPRs, and allow only two waves per SIMD.  The block-sparse variant has
// the same shape; its workgroup stages the key blocks its query block keeps.
template <bool SPARSE>
struct Cfg {
  static constexpr int NW = 4;                    // waves per workgroup
  static constexpr int NSTAGE = 3;                // K/V tiles in the LDS ring
  static constexpr int PREF = NSTAGE - 1;         // tiles issued ahead
  static constexpr int WG_PER_CU = 3;
  static constexpr int BM = 32 * NW;              // query rows per workgroup
  static constexpr int NT = 64 * NW;              // threads per workgroup
};
// Block-mask granularity of the block-sparse variant (a key block is a tile).
constexpr int kQueryBlock = 128;
static_assert(Cfg<true>::BM == kQueryBlock, "one query block per sparse workgroup");
// Longest sequence of the block-sparse variant (its key-block list lives in
// LDS, 4 bytes per key block).
constexpr int kSparseMaxSeq = 1 << 20;
constexpr int INFO_BYTES = 1024;    // per-key values of a tile (see prep_kv_fp8.hip)

// The running max m is refreshed when some row's max grows by more than
// kRescaleLog2 (exp2 domain); until then P' = exp2(u - m + kPOffset) stays
// below 2^(kRescaleLog2 + kPOffset) = 256, inside the e4m3 range, and the
// largest P' of a row sits in its top three binades.  (A threshold of 3
// rather than 2 takes 2 % off the time for 1.5e-3 more relative L2 error at
// 16896 tokens.)
constexpr float kRescaleLog2 = 3.f;
constexpr float kPOffset = 5.f;

constexpr int kBufferFlags = 0x00020000;

struct Fp8Args {
  const uint8_t *q;
  const float *sq;
  // prepared K [B*H][S_pad][D], V^T [B*H][D][S_pad], per-key values
  // [B*H][S_pad/64][1 KB] (prep_kv_fp8.hip)
  const uint8_t *k8, *v8t, *info;
  int S_pad;
  bf16 *o;
  float *lse;
  int64_t o_sb, o_ss, o_sh;
  int S, H, B, n_qblk;
  float scale_log2;
  int n_direct, parts;
  SplitWorkspace ws;
  // repair of the tokens with the largest quantization error (REPAIR
  // kernels only; their keys left the FP8 tiles through the preparation
  // pass's bias): kr / vr [B][H][n_pad][D] hold the repaired keys' exact
  // rotated K and V (bf16).
  const bf16 *kr, *vr;
  int n_rep, n_pad;
  // block-sparse variant: mask [B][H][nqb][nkb] (nonzero = keep)
  const uint8_t *mask;
  int nqb, nkb;
};

// Formats 0 = fp8 e4m3 for both operands; sa / sb are E8M0 exponents (127 =
// x1): lane (l32, hf) gives the scale of A row l32 and of B column l32 for
// the 32-element k-block hf, and k-block s is operand dwords 4s..4s+3 of
// every lane, of both lane halves (both checked on hardware).
__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}
// Unscaled (constant zero scale operands select the plain instruction).
__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// E8M0 exponent of a scale, which must be a positive normal power of two (its
// fp32 exponent field); anything else sets `bad`.
__device__ __forceinline__ int e8m0_of(float s, bool &bad) {
  const uint32_t u = __float_as_uint(s);
  const uint32_t e = u >> 23;                 // includes the sign bit
  bad = bad || (u & 0x7fffffu) != 0 || e == 0 || e >= 255;
  return (int)e;
}

__device__ __forceinline__ float half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  // a plain v_max_f32 (fmaxf would first canonicalize both swapped values)
  float m;
  asm("v_max_f32 %0, %1, %2" : "=v"(m) : "v"(__uint_as_float(r[0])), "v"(__uint_as_float(r[1])));
  return m;
}
__device__ __forceinline__ float half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// LDS ring: NSTAGE stages of [K tile | V^T tile | per-key values], each
// part a whole number of 1 KB loads (one wave's 64 lanes x 16 bytes).  A K
// row is D bytes whose 16-byte granules are XOR-swizzled (granule g of row r
// at g ^ ksw(r)), a V^T row the 64 keys of one head-dimension column with
// granule g at g ^ vswz8(d): the fragment reads of every 8 and every 16
// consecutive lanes then cover distinct banks (checked on the CPU against
// both the 32-bank and the 64-bank view of the LDS).
__host__ __device__ constexpr int vswz8(int d) { return (d / 4) % 4; }
template <int D>
__host__ __device__ constexpr int ksw(int r) {
  return D == 128 ? (r ^ (r >> 3)) & 7 : ((r >> 1) ^ (r >> 3)) & 3;
}

// The rows of the second 32-key block of a tile (r + 32) carry the swizzle
// of row r XOR a constant that flips only the granule bit of the 64-byte
// step kk, so a lane's reads of that block use the addresses of its reads of
// the first block with kk swapped, plus 32 rows.
template <int D>
__host__ __device__ constexpr int ksw_flip() { return ksw<D>(32) ^ ksw<D>(0); }
template <int D>
constexpr bool ksw_flip_uniform() {
  for (int r = 0; r < 32; ++r)
    if ((ksw<D>(r + 32) ^ ksw<D>(r)) != ksw_flip<D>()) return false;
  return ksw_flip<D>() % 4 == 0 && (ksw_flip<D>() >> 2) < D / 64 + (D == 64);
}
static_assert(ksw_flip_uniform<64>() && ksw_flip_uniform<128>(), "second key block swizzle");

template <int D, int NSTAGE>
struct Fp8Lds {
  static constexpr int CH = D / 16;                    // 16-byte granules per K row
  static constexpr int K_LOADS = BN * CH / 64;
  static constexpr int V_LOADS = D * (BN / 16) / 64;
  static constexpr int LOADS = K_LOADS + V_LOADS + 1;  // + per-key values
  static constexpr int KBYTES = K_LOADS * 1024;
  static constexpr int VBYTES = V_LOADS * 1024;
  static constexpr int STAGE = LOADS * 1024;
  static constexpr int BYTES = NSTAGE * STAGE;
  // block-sparse variant: per-wave counts, then the key-block list
  static constexpr int LIST_OFFSET = BYTES + 64;
  static constexpr int sparse_bytes(int nkb) { return LIST_OFFSET + 4 * nkb; }
  static_assert(BN * CH % 64 == 0 && D * (BN / 16) % 64 == 0, "whole loads");
};

template <int D, bool REPAIR, bool SPARSE>
__global__ __launch_bounds__(Cfg<SPARSE>::NT, Cfg<SPARSE>::WG_PER_CU)
void attn_fwd_fp8_kernel(Fp8Args a) {
  static_assert(!(REPAIR && SPARSE), "the repair pass is dense only");
  constexpr int NW = Cfg<SPARSE>::NW, NT = Cfg<SPARSE>::NT, BM = Cfg<SPARSE>::BM;
  constexpr int NSTAGE = Cfg<SPARSE>::NSTAGE, PREF = Cfg<SPARSE>::PREF;
  using L = Fp8Lds<D, NSTAGE>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem8[];
  // per-key values of stage 0: bias (fp32), then inv (fp32), then ke (int32)
  // and the softmax scale they were prepared for
  const float *info0 = reinterpret_cast<const float *>(smem8 + L::KBYTES + L::VBYTES);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave-uniform in a scalar register: the LDS destination of a buffer load
  // to LDS derives from it and must be uniform
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hf = lane >> 5;
  const int S = a.S;
  const int ntiles_all = (S + BN - 1) / BN;

  // ---- work item: XCD-aware placement of whole items, then the key-range
  //      parts of split items (see split.hip) ----
  int item, part = 0, unit = -1;
  if ((int)blockIdx.x < a.n_direct) {
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int per = a.n_direct >> 3, rem = a.n_direct & 7;
    item = xcd * per + min(xcd, rem) + slot;
  } else {
    unit = blockIdx.x - a.n_direct;
    part = unit % a.parts;
    item = a.n_direct + unit / a.parts;
  }
  const int qblk = item % a.n_qblk;
  const int bh32 = item / a.n_qblk;
  const int h = bh32 % a.H, b = bh32 / a.H;
  const int64_t bh = (int64_t)b * a.H + h;
  const int64_t row_stride = (int64_t)a.H * D;  // contiguous [B, S, H, D]

  // ---- block-sparse variant: the key blocks (= tiles) this query block
  //      keeps, compacted in ascending order into an LDS list; the dense
  //      kernel's tiles are 0 .. ntiles-1 ----
  uint32_t *blist = reinterpret_cast<uint32_t *>(smem8 + L::LIST_OFFSET);
  int ntiles = ntiles_all;
  if constexpr (SPARSE) {
    int *wcnt = reinterpret_cast<int *>(smem8 + L::BYTES);
    const uint8_t *mrow = a.mask + ((int64_t)bh * a.nqb + qblk) * a.nkb;
    int nact = 0;
    for (int base = 0; base < a.nkb; base += NT) {
      const int j = base + tid;
      const bool keep = j < a.nkb && mrow[j] != 0;
      const uint64_t bal = __builtin_amdgcn_ballot_w64(keep);
      if (lane == 0) wcnt[wave] = (int)__builtin_popcountll(bal);
      __syncthreads();
      int off = nact, tot = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const int cw = wcnt[w];
        off += w < wave ? cw : 0;
        tot += cw;
      }
      if (keep) blist[off + __builtin_popcountll(bal & ((1ull << lane) - 1))] = (uint32_t)j;
      nact += tot;
      __syncthreads();
    }
    ntiles = nact;
  }
  int t0 = 0, t1 = ntiles;
  if (unit >= 0) {
    t0 = (int)((int64_t)part * ntiles / a.parts);
    t1 = (int)((int64_t)(part + 1) * ntiles / a.parts);
  }
  // key tile of list position x
  auto tile_of = [&](int x) JA_INLINE -> int {
    if constexpr (SPARSE)
      return (int)__builtin_amdgcn_readfirstlane(blist[x]);
    else
      return x;
  };

  // ---- Q8 of this lane's query row ----
  const int qi = qblk * BM + wave * 32 + l32;
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
  // Q's scale enters Q K^T as an E8M0 block scale (the repair pass uses it
  // in the exp2 argument instead)
  bool bad = false;
  const float sqv = a.sq[bh * S + qs];
  const int qe = e8m0_of(sqv, bad);
  const float c = a.scale_log2;
  const float qmul = sqv * c;

  // ---- staging of a tile: K, V^T, per-key values (loads of 1 KB) ----
  const int span_k = a.S_pad * D, span_i = a.S_pad / BN * INFO_BYTES;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(a.k8 + bh * a.S_pad * D), 0, span_k, kBufferFlags);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(a.v8t + bh * D * a.S_pad), 0, span_k, kBufferFlags);
  const __amdgpu_buffer_rsrc_t irs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(a.info + bh * span_i), 0, span_i, kBufferFlags);
  // source offset of this lane in load j: K lanes fetch the granule that
  // the row's swizzle puts at their LDS position, V^T lanes likewise
  auto load_offset = [&](int j) JA_INLINE -> int {
    if (j < L::K_LOADS) {
      const int g = 64 * j + lane;
      const int r = g / L::CH;
      return r * D + 16 * ((g % L::CH) ^ ksw<D>(r));
    }
    if (j < L::K_LOADS + L::V_LOADS) {
      const int g = 64 * (j - L::K_LOADS) + lane;
      const int d = g / 4;
      return d * a.S_pad + 16 * ((g % 4) ^ vswz8(d));
    }
    return 16 * lane;
  };
  // Wave w issues K loads w + NW m (m < MK), then V loads K_LOADS + w + NW m
  // (m < MV); wave 0 also issues the per-key values.  Successive V loads of a
  // wave are 16 NW head-dimension rows apart with the same swizzle, so they
  // share one offset register and differ by a scalar offset.  (Scalar
  // variables: an array element as the builtin's offset operand makes the
  // host compilation drop the kernel's launch stub without a message.)
  constexpr int MK = L::K_LOADS / NW, MV = L::V_LOADS / NW;
  static_assert(L::K_LOADS % NW == 0 && L::V_LOADS % NW == 0 && MK <= 2, "load split");
  static_assert(vswz8(16 * NW) == 0, "V loads of a wave share the swizzle");
  const int koff0 = load_offset(wave);
  const int koff1 = MK > 1 ? load_offset(wave + NW) : 0;
  const int voff = load_offset(L::K_LOADS + wave);
  auto issue = [&](int t, int st) JA_INLINE {
    char *base = reinterpret_cast<char *>(smem8) + st * L::STAGE;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, JA_LDS_PTR(base + wave * 1024), 16, koff0,
                                             t * (BN * D), 0, 0);
    if constexpr (MK > 1)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, JA_LDS_PTR(base + (wave + NW) * 1024), 16,
                                               koff1, t * (BN * D), 0, 0);
#pragma unroll
    for (int m = 0; m < MV; ++m)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          vrs, JA_LDS_PTR(base + (L::K_LOADS + wave + NW * m) * 1024), 16, voff,
          t * BN + m * (16 * NW) * a.S_pad, 0, 0);
    if (wave == 0)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(irs, JA_LDS_PTR(base + (L::LOADS - 1) * 1024), 16,
                                               lane * 16, t * INFO_BYTES, 0, 0);
  };
  // wait until at most `AHEAD` later tiles' loads of this wave are in flight
  auto wait_tiles = [&]<int AHEAD>() JA_INLINE {
    if (wave == 0)
      wait_vmcnt<(MK + MV + 1) * AHEAD>();
    else
      wait_vmcnt<(MK + MV) * AHEAD>();
  };

  // ---- S^T = K8 . Q8^T for the 64 keys of a tile (two 32-key blocks), the
  //      K and Q scales applied as E8M0 block scales, each accumulator
  //      starting at its key's bias (element i of a lane is key
  //      kb*32 + 8(i/4) + 4hf + i%4): acc = sk sq K8.Q8 + log2(sv)/c ----
  // per-lane byte offsets of the fragment reads inside a stage, opaque to
  // the compiler: each read address is one add of the stage base, the rest
  // sits in the read's immediate offset.  kro[2j + half]: K granule
  // 4j + 2hf + half of row l32; vro[half]: V^T granule 2hf + half of row
  // l32; iro: this lane half's per-key values; ero: key l32's K exponent.
  int kro[D / 32], vro[2];
  {
    const int ks = ksw<D>(l32), vsw = vswz8(l32);
#pragma unroll
    for (int j = 0; j < D / 64; ++j)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        kro[2 * j + half] = l32 * D + 16 * ((4 * j + 2 * hf + half) ^ ks);
        asm volatile("" : "+v"(kro[2 * j + half]));
      }
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      vro[half] = L::KBYTES + l32 * BN + 16 * ((2 * hf + half) ^ vsw);
      asm volatile("" : "+v"(vro[half]));
    }
  }
  int iro = L::KBYTES + L::VBYTES + 16 * hf;
  int ero = L::KBYTES + L::VBYTES + 2 * BN * 4 + 4 * l32;
  asm volatile("" : "+v"(iro), "+v"(ero));
  constexpr int KFLIP = ksw_flip<D>() >> 2;
  // address of byte `off` of the stage that starts at byte sb (uniform)
  auto lds_at = [&](int sb, int off) JA_INLINE { return smem8 + sb + off; };

  // ---- S^T = K8 . Q8^T for the 64 keys of a tile (two 32-key blocks), the
  //      K and Q scales applied as E8M0 block scales, each accumulator
  //      starting at its key's bias (element i of a lane is key
  //      kb*32 + 8(i/4) + 4hf + i%4): acc = sk sq K8.Q8 + log2(sv)/c ----
  auto qk = [&](int sb, f32x16 (&sacc)[2]) JA_INLINE {
    const uint8_t *ib = lds_at(sb, iro);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 bg = *reinterpret_cast<const float4 *>(ib + 4 * (kb * 32 + g * 8));
        sacc[kb][4 * g] = bg.x;
        sacc[kb][4 * g + 1] = bg.y;
        sacc[kb][4 * g + 2] = bg.z;
        sacc[kb][4 * g + 3] = bg.w;
      }
      // A row l32 is key kb*32 + l32
      const int kex = *reinterpret_cast<const int *>(lds_at(sb, ero) + 4 * 32 * kb);
#pragma unroll
      for (int kk = 0; kk < D / 64; ++kk) {
        const int j = kb ? kk ^ KFLIP : kk;
        const i32x4 lo =
            *reinterpret_cast<const i32x4 *>(lds_at(sb, kro[2 * j]) + kb * 32 * D);
        const i32x4 hi =
            *reinterpret_cast<const i32x4 *>(lds_at(sb, kro[2 * j + 1]) + kb * 32 * D);
        sacc[kb] = mfma_fp8(i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w}, qreg[kk],
                            sacc[kb], kex, qe);
      }
    }
  };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  // ---- O^T += V8^T . P'^T: lane (l32, hf) reads the logical granules 2hf
  //      and 2hf+1 of V^T row db*32 + l32, whose swizzle is vswz8(l32) ----
  static_assert(vswz8(32) == 0, "V^T row blocks share the swizzle");
  auto pv = [&](const i32x8 &pb, int sb) JA_INLINE {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const i32x4 lo = *reinterpret_cast<const i32x4 *>(lds_at(sb, vro[0]) + db * 32 * BN);
      const i32x4 hi = *reinterpret_cast<const i32x4 *>(lds_at(sb, vro[1]) + db * 32 * BN);
      oacc[db] = mfma_fp8(i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w}, pb, oacc[db]);
    }
  };

  // ---- online softmax of one tile.  u = c acc = c score + log2(sv) is a
  //      key's score in the exp2 domain plus log2 of its V scale; m_run
  //      tracks the row max of u, and P' = exp2(u - m_run + kPOffset) is P
  //      times sv against the reference m_run - kPOffset, so P'.V8 is P.V in
  //      true units and the row sum adds P' / sv.  The tile's row max is
  //      taken first; when some row's max grew by more than the threshold,
  //      the wave moves the references of the rows that grew (rescaling
  //      their O and l), then computes P' once.  (Computing P' first against
  //      the old reference and again after a move costs a second exp2 pass
  //      in about a fifth of the tiles at 16896 tokens with outlier keys:
  //      one growing row of 32 is enough.)  m_run starts finite, so that a
  //      tile whose keys are all -inf leaves it (and O, l) unchanged. ----
  float m_run = -1e30f, l_run = 0.f;
  // P' of the tile against reference mref, and psum = sum of P' / sv over
  // the lane's keys (ig: 1/sv of those keys, element kb*4 + g of group g of
  // key block kb)
  auto exp_tile = [&](const f32x16 (&t)[2], float mref, const f32x4 (&ig)[8],
                      float &psum) JA_INLINE -> i32x8 {
    const float nref = kPOffset - mref;
    uint32_t pw[8];
    psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 iv = ig[kb * 4 + g];
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(t[kb][4 * g + i], c, nref));
        psum = __builtin_fmaf(p[0], iv.x, psum);
        psum = __builtin_fmaf(p[1], iv.y, psum);
        psum = __builtin_fmaf(p[2], iv.z, psum);
        psum = __builtin_fmaf(p[3], iv.w, psum);
        // the first conversion's upper half is overwritten by the second, so
        // it starts from any register value (no zeroing move)
        int any;
        asm volatile("" : "=v"(any));
        int w = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], any, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], w, true);
        pw[kb * 4 + g] = (uint32_t)w;
        // one group of four scores at a time, its sum included (left to the
        // scheduler, the 32 exp2 results wait for the sums past the P.V
        // products and overflow the register budget)
        asm volatile("" : "+v"(psum));
        __builtin_amdgcn_sched_barrier(0);
      }
    return bit_cast<i32x8>(pw);
  };
  auto softmax = [&](f32x16 (&sacc)[2], int sb) JA_INLINE -> i32x8 {
    // 1/sv of the lane's 32 keys, read while the max is taken
    f32x4 ig[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      ig[j] = *reinterpret_cast<const f32x4 *>(lds_at(sb, iro) + 4 * (BN + 8 * j));
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, sacc[kb][i]);
    const float mx = half_max(tmax) * c;      // c > 0
    const bool grow = mx > m_run + kRescaleLog2;
    // the reads complete here, above the branch
    asm volatile("" ::"v"(ig[0]), "v"(ig[1]), "v"(ig[2]), "v"(ig[3]), "v"(ig[4]), "v"(ig[5]),
                 "v"(ig[6]), "v"(ig[7]));
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float m_new = grow ? mx : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
    }
    float psum;
    const i32x8 pb = exp_tile(sacc, m_run, ig, psum);
    l_run += psum;
    return pb;
  };

  // ---- loop over the key tiles t0 .. t1-1 (local index i).  Tile i lives
  //      in stage i % NSTAGE.  Iteration i first issues the loads of tile
  //      i+3 into the stage of tile i-1, which every wave finished before the
  //      barrier that closed iteration i-1; then Q K^T, the softmax and P.V
  //      of tile i; before the barrier that closes it, each wave waits for
  //      its own loads of tile i+1 only. ----
  const int nt = t1 - t0;
  // a dense workgroup always has at least one tile; a sparse one may have none
  const bool any_tile = !SPARSE || nt > 0;
  if (any_tile) {
#pragma unroll
    for (int p = 0; p < PREF; ++p)
      if (p < nt) issue(tile_of(t0 + p), p);
    wait_vmcnt<0>();
    tile_barrier();
    // the per-key values were prepared for this softmax scale
    bad = bad || info0[3 * BN] != c;
  }
  f32x16 sacc[2];
  auto iteration = [&]<bool LAST>(int i) JA_INLINE {
    const bool ahead = i + PREF < nt;
    if (ahead) issue(tile_of(t0 + i + PREF), (i + PREF) % NSTAGE);
    // stage byte offset as one scalar (each address is then a single add)
    const int sb = __builtin_amdgcn_readfirstlane((i % NSTAGE) * L::STAGE);
    qk(sb, sacc);
    const i32x8 pb = softmax(sacc, sb);
    pv(pb, sb);
    if constexpr (!LAST) {
      if (ahead)
        wait_tiles.template operator()<PREF - 1>();
      else
        wait_vmcnt<0>();
      tile_barrier();
    } else if constexpr (REPAIR) {
      __syncthreads();        // the repair pass restages through the ring
    }
  };
  for (int i = 0; i + 1 < nt; ++i) iteration.template operator()<false>(i);
  if (any_tile) iteration.template operator()<true>(nt - 1);

  // ---- repaired keys: one more pass over them with their exact values, on
  //      bf16 MFMA (an e4m3 code times its scale is exact in this product:
  //      the codes are bf16-representable and the scale stays in the exp2
  //      argument), within the same online softmax: P against the reference
  //      m_run - kPOffset times the exact V, in the true units of the FP8
  //      accumulator.  Only one part of a split item runs it. ----
  if constexpr (REPAIR) {
    if (a.n_rep > 0 && (unit < 0 || unit % a.parts == 0)) {
      constexpr int KBS = D + 8;          // bf16 per staged K row (16-byte pad)
      constexpr int VBS = 32 + 8;         // bf16 per staged V^T row
      bf16 *kbuf = reinterpret_cast<bf16 *>(smem8);
      bf16 *vbuf = reinterpret_cast<bf16 *>(smem8 + 32 * KBS * 2);
      // Q codes in the bf16 operand layout: lane half hf holds d = 16kk + 8hf
      // + 0..7 (decoded for each 32-key block rather than held: the registers
      // are the O accumulators')
      // the row address is formed again from qi (kept opaque so that the
      // compiler does not hold the 64-bit address through the tile loop)
      int qr = qi < S ? qi : S - 1;
      asm volatile("" : "+v"(qr));
      const uint8_t *qrow_r = a.q + ((int64_t)b * S + qr) * row_stride + (int64_t)h * D;
      auto q_operand = [&](int kk) JA_INLINE -> bf16x8 {
        const u32x2 cw = *reinterpret_cast<const u32x2 *>(qrow_r + 16 * kk + 8 * hf);
        float f[8];
        f[0] = __builtin_amdgcn_cvt_f32_fp8((int)cw.x, 0);
        f[1] = __builtin_amdgcn_cvt_f32_fp8((int)cw.x, 1);
        f[2] = __builtin_amdgcn_cvt_f32_fp8((int)cw.x, 2);
        f[3] = __builtin_amdgcn_cvt_f32_fp8((int)cw.x, 3);
        f[4] = __builtin_amdgcn_cvt_f32_fp8((int)cw.y, 0);
        f[5] = __builtin_amdgcn_cvt_f32_fp8((int)cw.y, 1);
        f[6] = __builtin_amdgcn_cvt_f32_fp8((int)cw.y, 2);
        f[7] = __builtin_amdgcn_cvt_f32_fp8((int)cw.y, 3);
        u32x4 w = {pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                   pack_bf16x2(f[6], f[7])};
        if (qi >= S) w = u32x4{0, 0, 0, 0};
        return bit_cast<bf16x8>(w);
      };
      const bf16 *krb = a.kr + bh * a.n_pad * D;
      const bf16 *vrb = a.vr + bh * a.n_pad * D;
      for (int r0 = 0; r0 < a.n_pad; r0 += 32) {
        // stage 32 keys: K row-major, V transposed in the P operand's key order
        for (int task = tid; task < 32 * (D / 8); task += NT) {
          const int r = task / (D / 8), ch = task % (D / 8);
          *reinterpret_cast<u32x4 *>(kbuf + r * KBS + ch * 8) =
              *reinterpret_cast<const u32x4 *>(krb + (int64_t)(r0 + r) * D + ch * 8);
        }
        for (int task = tid; task < D * 4; task += NT) {
          const int vd = task % D, vc = task / D;
          uint32_t hv[8];
#pragma unroll
          for (int j = 0; j < 8; ++j)
            hv[j] = *reinterpret_cast<const uint16_t *>(
                vrb + (int64_t)(r0 + 16 * (vc >> 1) + vt_key_of_slot(8 * (vc & 1) + j)) * D + vd);
          *reinterpret_cast<u32x4 *>(vbuf + vd * VBS + 8 * vc) =
              u32x4{hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16), hv[4] | (hv[5] << 16),
                    hv[6] | (hv[7] << 16)};
        }
        __syncthreads();
        f32x16 st;
#pragma unroll
        for (int i = 0; i < 16; ++i) st[i] = 0.f;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
          const bf16x8 kv = *reinterpret_cast<const bf16x8 *>(kbuf + l32 * KBS + 16 * kk + 8 * hf);
          st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kv, q_operand(kk), st, 0, 0, 0);
        }
        // accumulator row i is key r0 + 8(i/4) + 4hf + i%4; rows past n are padding
        float tmax = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          if (r0 + 8 * (i / 4) + 4 * hf + (i % 4) >= a.n_rep) st[i] = -INFINITY;
          tmax = fmaxf(tmax, st[i]);
        }
        const float mx = half_max(tmax) * qmul;
        const bool grow = mx > m_run + kRescaleLog2;
        auto exp_rep = [&](float mref, bf16x8 (&pbr)[2]) JA_INLINE -> float {
          float ps = 0.f;
#pragma unroll
          for (int g = 0; g < 2; ++g) {
            uint32_t w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float nref = kPOffset - mref;
              const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(st[8 * g + 2 * e], qmul, nref));
              const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(st[8 * g + 2 * e + 1], qmul, nref));
              ps += p0 + p1;
              w[e] = pack_bf16x2(p0, p1);
            }
            pbr[g] = bit_cast<bf16x8>(u32x4{w[0], w[1], w[2], w[3]});
          }
          return ps;
        };
        bf16x8 pbr[2];
        float ps = exp_rep(m_run, pbr);
        if (__builtin_amdgcn_ballot_w64(grow)) {
          const float m_new = grow ? mx : m_run;
          const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
          m_run = m_new;
          l_run *= alpha;
#pragma unroll
          for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
          ps = exp_rep(m_new, pbr);
        }
        l_run += ps;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int g = 0; g < 2; ++g) {
            const bf16x8 va =
                *reinterpret_cast<const bf16x8 *>(vbuf + (32 * db + l32) * VBS + 16 * g + 8 * hf);
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pbr[g], oacc[db], 0, 0, 0);
          }
        __syncthreads();
      }
    }
  }

  // a Q or K scale that is not a positive normal power of two turns the rows
  // of its workgroup into NaN
  const bool bad_wg = __syncthreads_or(bad);
  const float o_mul = bad_wg ? __builtin_nanf("") : 1.f;
  const float l_tot = half_sum(l_run);
  const float ref = m_run - kPOffset;       // P was computed against ref
  if (unit >= 0) {
    // split part: unnormalised O in true units, reference (exp2 domain), sum
    const int row = wave * 32 + l32;
    float *orow = a.ws.o + ((int64_t)unit * BM + row) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp)
        *reinterpret_cast<float4 *>(orow + db * 32 + 8 * grp + 4 * hf) =
            make_float4(oacc[db][4 * grp] * o_mul, oacc[db][4 * grp + 1] * o_mul,
                        oacc[db][4 * grp + 2] * o_mul, oacc[db][4 * grp + 3] * o_mul);
    // a block-sparse row that saw no key in this part: row max -inf, so
    // that the merge treats it as empty
    const float mref = SPARSE && l_tot == 0.f ? -INFINITY : ref;
    if (hf == 0)
      *reinterpret_cast<float2 *>(a.ws.ml + ((int64_t)unit * BM + row) * 2) =
          make_float2(mref * o_mul, l_tot);
    return;
  }
  if (qi < S) {
    // a block-sparse row that keeps no key has l = 0 and O accumulators 0:
    // O = 0, LSE = -inf (NaN if poisoned)
    const float inv = SPARSE && l_tot == 0.f ? 0.f * o_mul : o_mul / l_tot;
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
    if (a.lse && hf == 0) a.lse[bh * S + qi] = (ref + __log2f(l_tot)) * kLn2 * o_mul;
  }
}

// Dynamic LDS of one instantiation; its limit is raised once per device (the
// attribute is set with the device current).
template <int D, bool REPAIR, bool SPARSE>
hipError_t launch_fp8_instance(const Fp8Args &a, dim3 grid, hipStream_t st) {
  using L = Fp8Lds<D, Cfg<SPARSE>::NSTAGE>;
  const int bytes = SPARSE ? L::sparse_bytes(a.nkb) : L::BYTES;
  constexpr int kMaxDevices = 64;
  static std::atomic<bool> done[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices || !done[dev].load(std::memory_order_acquire)) {
    e = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&attn_fwd_fp8_kernel<D, REPAIR, SPARSE>),
        hipFuncAttributeMaxDynamicSharedMemorySize,
        SPARSE ? L::sparse_bytes((kSparseMaxSeq + BN - 1) / BN) : L::BYTES);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < kMaxDevices) done[dev].store(true, std::memory_order_release);
  }
  hipLaunchKernelGGL((attn_fwd_fp8_kernel<D, REPAIR, SPARSE>), grid, dim3(Cfg<SPARSE>::NT),
                     bytes, st, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_fp8_dim(const Fp8Args &a, dim3 grid, bool repair, hipStream_t st) {
  if (a.mask) return launch_fp8_instance<D, false, true>(a, grid, st);
  return repair ? launch_fp8_instance<D, true, false>(a, grid, st)
                : launch_fp8_instance<D, false, false>(a, grid, st);
}

}  // namespace

int fwd_fp8_block_rows(bool sparse) { return sparse ? Cfg<true>::BM : Cfg<false>::BM; }

int fwd_fp8_sparse_max_seq() { return kSparseMaxSeq; }

SplitPlan plan_fwd_fp8(const AttnLayout &L, int n_cu, bool sparse) {
  const int bm = fwd_fp8_block_rows(sparse);
  const int wg = sparse ? Cfg<true>::WG_PER_CU : Cfg<false>::WG_PER_CU;
  const int n_items = ((L.S + bm - 1) / bm) * L.H * L.B;
  return plan_split(n_items, (L.S + BN - 1) / BN, n_cu * wg, bm, L.D);
}

hipError_t launch_fwd_fp8(const AttnLayout &L, const void *q8, const float *sq, const void *kv8,
                          const uint8_t *mask, void *o, float *lse, const SplitPlan &plan,
                          void *workspace, const Fp8Repair &repair, hipStream_t st) {
  Fp8Args a;
  a.q = static_cast<const uint8_t *>(q8);
  a.sq = sq;
  a.S_pad = prep8_pad(L.S);
  const int64_t kv = (int64_t)L.B * L.H * a.S_pad * L.D;
  a.k8 = static_cast<const uint8_t *>(kv8);
  a.v8t = a.k8 + kv;
  a.info = a.v8t + kv;
  a.o = static_cast<bf16 *>(o);
  a.lse = lse;
  a.o_sb = L.o_sb; a.o_ss = L.o_ss; a.o_sh = L.o_sh;
  a.S = L.S;
  a.H = L.H;
  a.B = L.B;
  const int bm = fwd_fp8_block_rows(mask != nullptr);
  a.n_qblk = (L.S + bm - 1) / bm;
  a.scale_log2 = L.scale_log2;
  a.n_direct = plan.n_direct;
  a.parts = plan.parts;
  a.ws = split_workspace(plan, workspace, bm, L.D);
  a.mask = mask;
  a.nqb = (L.S + kQueryBlock - 1) / kQueryBlock;
  a.nkb = (L.S + BN - 1) / BN;
  const dim3 grid((unsigned)(plan.n_direct + plan.n_units));
  const bool rep = repair.n_rep > 0 && mask == nullptr;
  a.kr = static_cast<const bf16 *>(repair.kr);
  a.vr = static_cast<const bf16 *>(repair.vr);
  a.n_rep = rep ? repair.n_rep : 0;
  a.n_pad = repair_pad(a.n_rep);
  const hipError_t e = L.D == 64 ? launch_fp8_dim<64>(a, grid, rep, st)
                                 : launch_fp8_dim<128>(a, grid, rep, st);
  if (e != hipSuccess || plan.n_units == 0) return e;
  return launch_merge_split(L, plan, a.ws, bm, 1.f, o, lse, st);
}

}  // namespace ja
