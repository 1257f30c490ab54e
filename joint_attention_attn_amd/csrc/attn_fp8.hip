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
// normaliser sums the unquantized fp32 P' / sv[key].  A key past the end or
// a repaired key starts at -inf.  Per score this leaves a max, an FMA, an
// exp2, the sum's FMA and half a conversion.
//
// Structure as in the bf16 kernel: one workgroup of twelve wave64s (three
// per SIMD) per (384-query block, head, batch row), XCD-aware placement,
// split of the last round.  A preparation pass (prep_kv_fp8.hip) writes each
// (batch, head)'s K, V^T and per-key values in the layouts of the LDS tiles;
// buffer loads to LDS copy 64-key tiles into a 4-stage ring three tiles
// ahead, with no staging registers and no vector work.  Each wave runs
// Q K^T, softmax and P.V of a tile in turn, and the three waves of a SIMD
// overlap one another's matrix and vector work.
#include <atomic>

#include "common.hpp"
#include "internal.hpp"

#define JA_INLINE __attribute__((always_inline))

namespace ja {

namespace {

// Waves per workgroup, 32 query rows each, three per SIMD (at most 168 VGPRs
// each).  Software pipelining inside a wave (Q K^T of the next tile issued
// ahead of this tile's softmax) would keep two tiles of accumulators live,
// about 245 VGPRs, and allow only two waves per SIMD, which is slower.
constexpr int NW = 12;
constexpr int BM = 32 * NW;         // query rows per workgroup
constexpr int BN = 64;              // keys per K/V tile (the MFMA's K extent)
constexpr int NT = 64 * NW;         // threads per workgroup
constexpr int NSTAGE = 4;           // K/V tiles in the LDS ring
constexpr int PREF = 3;             // tiles issued ahead
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
};

// Formats 0 = fp8 e4m3 for both operands; sa / sb are E8M0 exponents (127 =
// x1): lane (l32, hf) gives the scale of A row l32 and of B column l32 for
// the 32-element k-block hf (checked on hardware).
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
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// LDS ring: NSTAGE stages of [K tile | V^T tile | per-key values], each
// part a whole number of 1 KB loads (one wave's 64 lanes x 16 bytes).  A K
// row is D bytes plus a 16-byte pad, the pad lanes loading a dummy chunk.  A
// V^T row is the 64 keys of one head-dimension column, granule g stored at
// g ^ vswz(d) so that the fragment reads of 16 consecutive rows cover all 16
// bank groups.
__host__ __device__ constexpr int vswz8(int d) { return (d / 4) % 4; }

template <int D>
struct Fp8Lds {
  static constexpr int CH = D / 16;                    // 16-byte chunks per K row
  static constexpr int KSTR = D + 16;                  // bytes per K row
  static constexpr int K_LOADS = BN * (CH + 1) / 64;
  static constexpr int V_LOADS = D * (BN / 16) / 64;
  static constexpr int LOADS = K_LOADS + V_LOADS + 1;  // + per-key values
  static constexpr int KBYTES = K_LOADS * 1024;
  static constexpr int VBYTES = V_LOADS * 1024;
  static constexpr int STAGE = LOADS * 1024;
  static constexpr int BYTES = NSTAGE * STAGE;
  static_assert(BN * (CH + 1) % 64 == 0 && D * (BN / 16) % 64 == 0, "whole loads");
};

template <int D, bool REPAIR>
__global__ __launch_bounds__(NT, 1) void attn_fwd_fp8_kernel(Fp8Args a) {
  using L = Fp8Lds<D>;
  constexpr int KSTR = L::KSTR;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem8[];
  auto Kst = [&](int st) JA_INLINE { return smem8 + st * L::STAGE; };
  auto Vst = [&](int st) JA_INLINE { return smem8 + st * L::STAGE + L::KBYTES; };
  // per-key values of a stage: bias (fp32), then inv (fp32), then ke (int32)
  auto Ist = [&](int st) JA_INLINE {
    return reinterpret_cast<const float *>(smem8 + st * L::STAGE + L::KBYTES + L::VBYTES);
  };

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
  int item, t0, t1, unit = -1;
  if ((int)blockIdx.x < a.n_direct) {
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int per = a.n_direct >> 3, rem = a.n_direct & 7;
    item = xcd * per + min(xcd, rem) + slot;
    t0 = 0;
    t1 = ntiles_all;
  } else {
    unit = blockIdx.x - a.n_direct;
    const int part = unit % a.parts;
    item = a.n_direct + unit / a.parts;
    t0 = (int)((int64_t)part * ntiles_all / a.parts);
    t1 = (int)((int64_t)(part + 1) * ntiles_all / a.parts);
  }
  const int qblk = item % a.n_qblk;
  const int bh32 = item / a.n_qblk;
  const int h = bh32 % a.H, b = bh32 / a.H;
  const int64_t bh = (int64_t)b * a.H + h;
  const int64_t row_stride = (int64_t)a.H * D;  // contiguous [B, S, H, D]

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

  // ---- staging: wave w issues loads w, w + NW, w + 2 NW of each tile ----
  const int span_k = a.S_pad * D, span_i = a.S_pad / BN * INFO_BYTES;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(a.k8 + bh * a.S_pad * D), 0, span_k, kBufferFlags);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(a.v8t + bh * D * a.S_pad), 0, span_k, kBufferFlags);
  const __amdgpu_buffer_rsrc_t irs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t *>(a.info + bh * span_i), 0, span_i, kBufferFlags);
  // source offset of this lane in load j (K lanes that fall on a pad load a
  // dummy chunk; V^T lanes fetch the granule that the swizzle puts there)
  auto load_offset = [&](int j) JA_INLINE -> int {
    if (j < L::K_LOADS) {
      const int g = 64 * j + lane;
      const int r = g / (L::CH + 1), ch = g % (L::CH + 1);
      return ch < L::CH ? r * D + 16 * ch : 0;
    }
    if (j < L::K_LOADS + L::V_LOADS) {
      const int g = 64 * (j - L::K_LOADS) + lane;
      const int d = g / 4;
      return d * a.S_pad + 16 * ((g % 4) ^ vswz8(d));
    }
    return 16 * lane;
  };
  constexpr int JW = (L::LOADS + NW - 1) / NW;         // loads per wave, at most
  static_assert(JW <= 3, "loads per wave");
  // (scalar offsets: an array element as the builtin's offset operand makes
  // the host compilation drop the kernel's launch stub without a message)
  const int voff0 = load_offset(wave);
  const int voff1 = wave + NW < L::LOADS ? load_offset(wave + NW) : 0;
  const int voff2 = wave + 2 * NW < L::LOADS ? load_offset(wave + 2 * NW) : 0;
  const int nl = (L::LOADS - wave + NW - 1) / NW;      // loads of this wave per tile
  auto issue_one = [&](int j, int voff, int t, int st) JA_INLINE {
    char *dst = reinterpret_cast<char *>(smem8) + st * L::STAGE + j * 1024;
    if (j < L::K_LOADS)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, JA_LDS_PTR(dst), 16, voff, t * (BN * D), 0, 0);
    else if (j < L::K_LOADS + L::V_LOADS)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, JA_LDS_PTR(dst), 16, voff, t * BN, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(irs, JA_LDS_PTR(dst), 16, voff, t * INFO_BYTES, 0, 0);
  };
  // loads of key tile t into stage st (at D = 64 a tile has fewer loads than
  // the workgroup has waves; the last waves issue none)
  auto issue = [&](int t, int st) JA_INLINE {
    if (wave < L::LOADS) issue_one(wave, voff0, t, st);
    if (wave + NW < L::LOADS) issue_one(wave + NW, voff1, t, st);
    if (JW >= 3 && wave + 2 * NW < L::LOADS) issue_one(wave + 2 * NW, voff2, t, st);
  };
  // wait until at most `AHEAD` later tiles' loads of this wave are in flight
  auto wait_tiles = [&]<int AHEAD>() JA_INLINE {
    if constexpr (JW >= 3) {
      if (nl >= 3) { wait_vmcnt<3 * AHEAD>(); return; }
    }
    if (nl >= 2)
      wait_vmcnt<2 * AHEAD>();
    else
      wait_vmcnt<AHEAD>();
  };

  // ---- S^T = K8 . Q8^T for the 64 keys of a tile (two 32-key blocks), the
  //      K and Q scales applied as E8M0 block scales, each accumulator
  //      starting at its key's bias (element i of a lane is key
  //      kb*32 + 8(i/4) + 4hf + i%4): acc = sk sq K8.Q8 + log2(sv)/c ----
  auto qk = [&](int st, f32x16 (&sacc)[2]) JA_INLINE {
    const float *bias = Ist(st);
    const int *ke = reinterpret_cast<const int *>(Ist(st) + 2 * BN);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 bg = *reinterpret_cast<const float4 *>(bias + kb * 32 + g * 8 + hf * 4);
        sacc[kb][4 * g] = bg.x;
        sacc[kb][4 * g + 1] = bg.y;
        sacc[kb][4 * g + 2] = bg.z;
        sacc[kb][4 * g + 3] = bg.w;
      }
      const int kex = ke[kb * 32 + l32];            // A row l32 is key kb*32 + l32
      const uint8_t *krow = Kst(st) + (kb * 32 + l32) * KSTR + 32 * hf;
#pragma unroll
      for (int kk = 0; kk < D / 64; ++kk) {
        const i32x4 lo = *reinterpret_cast<const i32x4 *>(krow + 64 * kk);
        const i32x4 hi = *reinterpret_cast<const i32x4 *>(krow + 64 * kk + 16);
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
  const int vsw = vswz8(l32);
  auto pv = [&](const i32x8 &pb, int st) JA_INLINE {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const uint8_t *vrow = Vst(st) + (db * 32 + l32) * BN;
      const i32x4 lo = *reinterpret_cast<const i32x4 *>(vrow + 16 * ((2 * hf) ^ vsw));
      const i32x4 hi = *reinterpret_cast<const i32x4 *>(vrow + 16 * ((2 * hf + 1) ^ vsw));
      oacc[db] = mfma_fp8(i32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w}, pb, oacc[db]);
    }
  };

  // ---- online softmax of one tile.  u = c acc = c score + log2(sv) is a
  //      key's score in the exp2 domain plus log2 of its V scale; m_run
  //      tracks the row max of u, and P' = exp2(u - m_run + kPOffset) is P
  //      times sv against the reference m_run - kPOffset, so P'.V8 is P.V in
  //      true units and the row sum adds P' / sv.  As in the bf16 kernel, P'
  //      is first computed against the running max and only recomputed (with
  //      O and l rescaled) when some row max grew by more than the threshold.
  //      m_run starts finite, so that a tile whose keys are all -inf leaves
  //      it (and O, l) unchanged. ----
  float m_run = -1e30f, l_run = 0.f;
  auto exp_tile = [&](const f32x16 (&t)[2], float mref, int buf, float &psum) JA_INLINE -> i32x8 {
    const float nref = kPOffset - mref;
    uint32_t pw[8];
    psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 ig = *reinterpret_cast<const float4 *>(Ist(buf) + BN + kb * 32 + g * 8 + hf * 4);
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(t[kb][4 * g + i], c, nref));
        psum = __builtin_fmaf(p[0], ig.x, psum);
        psum = __builtin_fmaf(p[1], ig.y, psum);
        psum = __builtin_fmaf(p[2], ig.z, psum);
        psum = __builtin_fmaf(p[3], ig.w, psum);
        int w = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], w, true);
        pw[kb * 4 + g] = (uint32_t)w;
      }
    return bit_cast<i32x8>(pw);
  };
  auto softmax = [&](f32x16 (&sacc)[2], int buf) JA_INLINE -> i32x8 {
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, sacc[kb][i]);
    const float mx = half_max(tmax) * c;      // c > 0
    const bool grow = mx > m_run + kRescaleLog2;
    float psum;
    i32x8 pb = exp_tile(sacc, m_run, buf, psum);
    // the fast path's sum stays before the branch (sunk past it, its
    // reciprocal-scale reads would wait one by one)
    asm volatile("" ::"v"(psum));
    if (__builtin_amdgcn_ballot_w64(grow)) {
      asm volatile("" ::"v"(pb));
      const float m_new = grow ? mx : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
      pb = exp_tile(sacc, m_new, buf, psum);
    }
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
#pragma unroll
  for (int p = 0; p < PREF; ++p)
    if (p < nt) issue(t0 + p, p);
  wait_vmcnt<0>();
  tile_barrier();
  // the per-key values were prepared for this softmax scale
  bad = bad || Ist(0)[3 * BN] != c;
  f32x16 sacc[2];
  auto iteration = [&]<bool LAST>(int i) JA_INLINE {
    const bool ahead = i + PREF < nt;
    if (ahead) issue(t0 + i + PREF, (i + PREF) % NSTAGE);
    qk(i % NSTAGE, sacc);
    const i32x8 pb = softmax(sacc, i % NSTAGE);
    pv(pb, i % NSTAGE);
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
  iteration.template operator()<true>(nt - 1);

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
      // Q codes in the bf16 operand layout: lane half hf holds d = 16kk + 8hf + 0..7
      bf16x8 qb[D / 16];
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const u32x2 cw = *reinterpret_cast<const u32x2 *>(qrow + 16 * kk + 8 * hf);
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
        qb[kk] = bit_cast<bf16x8>(w);
      }
      const bf16 *krb = a.kr + bh * a.n_pad * D;
      const bf16 *vrb = a.vr + bh * a.n_pad * D;
      for (int r0 = 0; r0 < a.n_pad; r0 += 32) {
        // stage 32 keys: K row-major, V transposed in the P operand's key order
        if (tid < 32 * (D / 8)) {
          const int r = tid / (D / 8), ch = tid % (D / 8);
          *reinterpret_cast<u32x4 *>(kbuf + r * KBS + ch * 8) =
              *reinterpret_cast<const u32x4 *>(krb + (int64_t)(r0 + r) * D + ch * 8);
        }
        if (tid < D * 4) {
          const int vd = tid % D, vc = tid / D;
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
          st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kv, qb[kk], st, 0, 0, 0);
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
    if (hf == 0)
      *reinterpret_cast<float2 *>(a.ws.ml + ((int64_t)unit * BM + row) * 2) =
          make_float2(ref * o_mul, l_tot);
    return;
  }
  if (qi < S) {
    const float inv = o_mul / l_tot;
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
template <int D, bool REPAIR>
hipError_t launch_fp8_instance(const Fp8Args &a, dim3 grid, hipStream_t st) {
  constexpr int kMaxDevices = 64;
  static std::atomic<bool> done[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices || !done[dev].load(std::memory_order_acquire)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(&attn_fwd_fp8_kernel<D, REPAIR>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, Fp8Lds<D>::BYTES);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < kMaxDevices) done[dev].store(true, std::memory_order_release);
  }
  hipLaunchKernelGGL((attn_fwd_fp8_kernel<D, REPAIR>), grid, dim3(NT), Fp8Lds<D>::BYTES, st, a);
  return hipGetLastError();
}

}  // namespace

int fwd_fp8_block_rows(int) { return BM; }

SplitPlan plan_fwd_fp8(const AttnLayout &L, int n_cu) {
  const int n_items = ((L.S + BM - 1) / BM) * L.H * L.B;
  return plan_split(n_items, (L.S + BN - 1) / BN, n_cu, BM, L.D);
}

hipError_t launch_fwd_fp8(const AttnLayout &L, const void *q8, const float *sq, const void *kv8,
                          void *o, float *lse, const SplitPlan &plan, void *workspace,
                          const Fp8Repair &repair, hipStream_t st) {
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
  a.n_qblk = (L.S + BM - 1) / BM;
  a.scale_log2 = L.scale_log2;
  a.n_direct = plan.n_direct;
  a.parts = plan.parts;
  a.ws = split_workspace(plan, workspace, BM, L.D);
  const dim3 grid((unsigned)(plan.n_direct + plan.n_units));
  const bool rep = repair.n_rep > 0;
  a.kr = static_cast<const bf16 *>(repair.kr);
  a.vr = static_cast<const bf16 *>(repair.vr);
  a.n_rep = repair.n_rep;
  a.n_pad = repair_pad(repair.n_rep);
  hipError_t e;
  if (L.D == 64)
    e = rep ? launch_fp8_instance<64, true>(a, grid, st) : launch_fp8_instance<64, false>(a, grid, st);
  else
    e = rep ? launch_fp8_instance<128, true>(a, grid, st) : launch_fp8_instance<128, false>(a, grid, st);
  if (e != hipSuccess || plan.n_units == 0) return e;
  return launch_merge_split(L, plan, a.ws, BM, 1.f, o, lse, st);
}

}  // namespace ja
