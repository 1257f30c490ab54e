// BF16 joint-attention forward for gfx950 with RoPE fused into the Q/K load.
//
// Joint attention ("Speed Up Image Generation with FLUX 3 Image Klein on
// NVIDIA Blackwell GPUs", section "FLUX 3 inference with TensorRT LLM
// VisualGen"): one dense softmax over the concatenated text / target / reference
// tokens.  RoPE is applied to Q and K before the product (same page, section
// "GEMM kernel optimization"); here it is applied in fp32 while Q and K are
// loaded and the rotated values are rounded to bf16 for the MFMA.
//
// Work decomposition: one workgroup per (256-query block, head, batch row),
// eight wave64s of 32 query rows each.  Both products are computed transposed
// so that a lane owns one query row throughout:
//   S^T[key][q]  = K . Q^T      (v_mfma_f32_32x32x16_bf16, A = rotated K from
//                                LDS, B = rotated Q kept in registers)
//   O^T[d][q]   += V^T . P^T    (A = V^T read from row-major V in LDS with
//                                ds_read_b64_tr_b16, B = P straight from the
//                                S^T accumulators)
// With that orientation the online-softmax state (running max m and sum l,
// fp32) is per lane, the row max needs one cross-half exchange and the O
// rescale is one multiply per accumulator.
//
// K/V tiles of 64 keys are double-buffered in LDS: the next tile is loaded
// from global memory into registers while the current one is consumed, then
// K is rotated (fp32, rounded to bf16) and both are stored row-major to the
// other buffer; one barrier per tile.  Every K tile is rotated once per
// workgroup, shared by its 256 query rows.  V^T operands come from row-major V
// through ds_read_b64_tr_b16 (a 16-lane group reads 4 key rows x 16 columns
// and each lane receives one column's 4 keys).  Rows are padded (K by 16
// bytes, V by 32 bytes) so that the lanes served together hit distinct banks
// and every LDS address is a per-lane base plus a compile-time offset.
#include "common.hpp"
#include "internal.hpp"

namespace ja {

namespace {

constexpr int BM = 256;     // query rows per workgroup
constexpr int BN = 64;      // keys per K/V tile
constexpr int NT = 512;     // threads per workgroup (8 waves)

// Rescale the output accumulator only when the running row max grows by more
// than 2^8 in the exp2 domain; until then P may exceed 1 by up to 2^8, which
// fp32 and bf16 carry exactly as well as values below 1.
constexpr float kRescaleLog2 = 8.f;

// Buffer-resource word 3 for raw (unswizzled, unformatted 32-bit) buffer
// access on gfx950: out-of-range reads return zeros.
constexpr int kBufferFlags = 0x00020000;

struct FwdArgs {
  const bf16 *q, *k, *v;
  const float2 *rope;
  bf16 *o;
  float *lse;
  int64_t q_sb, q_ss, q_sh, k_sb, k_ss, k_sh, v_sb, v_ss, v_sh, o_sb, o_ss, o_sh;
  int S, H, B, n_qblk;
  float scale_log2;
};

// Max and sum of x over the two lanes l and l ^ 32 that share a query row.
// v_permlane32_swap hands each lane the other half's value in one of its two
// results and keeps its own in the other, so a symmetric combination of both
// results is the cross-half reduction.
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

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x2 lds_read_tr16(const bf16 *p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4 *)(p));
  return bit_cast<u32x2>(v);
}

template <int D>
struct Lds {
  static constexpr int KSTR = D + 8;        // bf16 per K row (16-byte pad)
  static constexpr int VSTR = D + 16;       // bf16 per V row (32-byte pad)
  static constexpr int KTILE = BN * KSTR;
  static constexpr int VTILE = BN * VSTR;
  static constexpr int BYTES = 2 * (KTILE + VTILE) * 2;
};

template <int D, bool ROPE>
__global__ __launch_bounds__(NT, 1) void attn_fwd_bf16_kernel(FwdArgs a) {
  constexpr int CH = D / 8;             // 16-byte chunks per head vector
  constexpr int ROWS_PER_PASS = NT / CH;
  constexpr int PASSES = BN / ROWS_PER_PASS;
  constexpr int KSTR = Lds<D>::KSTR, VSTR = Lds<D>::VSTR;
  extern __shared__ __attribute__((aligned(16))) bf16 smem[];
  auto Kbuf = [&](int buf) { return smem + buf * Lds<D>::KTILE; };
  auto Vbuf = [&](int buf) { return smem + 2 * Lds<D>::KTILE + buf * Lds<D>::VTILE; };

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;

  // XCD-aware placement: workgroups are dispatched round-robin over the 8
  // XCDs, so give each XCD a contiguous range of (q-block, head) work items;
  // the workgroups resident on one XCD then stream the same head's K/V
  // through that XCD's L2.
  const int nwg = gridDim.x;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int per = nwg >> 3, rem = nwg & 7;
  const int item = xcd * per + min(xcd, rem) + slot;
  const int qblk = item % a.n_qblk;
  const int bh = item / a.n_qblk;
  const int h = bh % a.H, b = bh / a.H;
  const int S = a.S;

  // ---- Q rows of this lane: rotate, round to bf16, keep in registers ----
  const int qi = qblk * BM + wave * 32 + l32;
  const int qs = qi < S ? qi : S - 1;
  const bf16 *qrow = a.q + b * a.q_sb + (int64_t)qs * a.q_ss + h * a.q_sh;
  bf16x8 qreg[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    const int d0 = 16 * kk + 8 * hf;
    u32x4 w = *reinterpret_cast<const u32x4 *>(qrow + d0);
    if constexpr (ROPE) w = rope_chunk_bf16(w, a.rope + (int64_t)qs * (D / 2) + d0 / 2);
    if (qi >= S) w = u32x4{0, 0, 0, 0};
    qreg[kk] = bit_cast<bf16x8>(w);
  }

  const bf16 *kbase = a.k + b * a.k_sb + h * a.k_sh;
  const bf16 *vbase = a.v + b * a.v_sb + h * a.v_sh;
  const int st_c = tid % CH;            // chunk this thread stages
  const int st_r = tid / CH;            // first row this thread stages

  // ---- staging: global -> registers through buffer resources, then
  //      registers -> LDS (K rotated on the way).  Each lane's byte offset
  //      inside a tile is fixed; the tile offset is a scalar.  The resource
  //      ends after row S-1, so rows past the end of the sequence read as
  //      zeros (their scores are masked, their P is 0). ----
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16 *>(kbase), 0, (int)(((int64_t)(S - 1) * a.k_ss + D) * 2), kBufferFlags);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16 *>(vbase), 0, (int)(((int64_t)(S - 1) * a.v_ss + D) * 2), kBufferFlags);
  const __amdgpu_buffer_rsrc_t trs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float2 *>(a.rope), 0, ROPE ? S * D * 4 : 0, kBufferFlags);
  int koff[PASSES], voff[PASSES], toff[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int r = st_r + p * ROWS_PER_PASS;
    koff[p] = (int)(r * a.k_ss * 2) + st_c * 16;
    voff[p] = (int)(r * a.v_ss * 2) + st_c * 16;
    toff[p] = r * D * 4 + st_c * 32;
  }
  const int ktile_bytes = (int)(BN * a.k_ss * 2), vtile_bytes = (int)(BN * a.v_ss * 2);
  u32x4 kreg[PASSES], vreg[PASSES];
  float4 treg[PASSES][2];
  auto load_k = [&](int t) {
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      kreg[p] = bit_cast<u32x4>(__builtin_amdgcn_raw_buffer_load_b128(krs, koff[p], t * ktile_bytes, 0));
      if constexpr (ROPE) {
        treg[p][0] = bit_cast<float4>(__builtin_amdgcn_raw_buffer_load_b128(trs, toff[p], t * BN * D * 4, 0));
        treg[p][1] = bit_cast<float4>(__builtin_amdgcn_raw_buffer_load_b128(trs, toff[p] + 16, t * BN * D * 4, 0));
      }
    }
  };
  auto load_v = [&](int t) {
#pragma unroll
    for (int p = 0; p < PASSES; ++p)
      vreg[p] = bit_cast<u32x4>(__builtin_amdgcn_raw_buffer_load_b128(vrs, voff[p], t * vtile_bytes, 0));
  };
  auto store_k = [&](int buf) {
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int r = st_r + p * ROWS_PER_PASS;
      u32x4 kw = kreg[p];
      if constexpr (ROPE) {
        kw.x = rope_pair_bf16(kw.x, make_float2(treg[p][0].x, treg[p][0].y));
        kw.y = rope_pair_bf16(kw.y, make_float2(treg[p][0].z, treg[p][0].w));
        kw.z = rope_pair_bf16(kw.z, make_float2(treg[p][1].x, treg[p][1].y));
        kw.w = rope_pair_bf16(kw.w, make_float2(treg[p][1].z, treg[p][1].w));
      }
      *reinterpret_cast<u32x4 *>(Kbuf(buf) + r * KSTR + st_c * 8) = kw;
    }
  };
  auto store_v = [&](int buf) {
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int r = st_r + p * ROWS_PER_PASS;
      *reinterpret_cast<u32x4 *>(Vbuf(buf) + r * VSTR + st_c * 8) = vreg[p];
    }
  };

  // ---- S^T = K . Q^T for this wave's 32 queries and the 64 keys of a tile ----
  auto qk = [&](int buf, f32x16 (&sacc)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[kb][i] = 0.f;
      const int r = kb * 32 + l32;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const bf16x8 kv =
            *reinterpret_cast<const bf16x8 *>(Kbuf(buf) + r * KSTR + (2 * kk + hf) * 8);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kv, qreg[kk], sacc[kb], 0, 0, 0);
      }
    }
  };

  // per-lane part of the transposed V read: lane i of its 16-lane group
  // addresses key row i / 4 and columns 4 (i % 4) .. +3 of a 4 x 16 block;
  // groups 1 and 3 take the upper 16 columns of each 32-column block and
  // lane half hf the keys 4 hf .. 4 hf + 3 of each group of 8.
  const int tr_i = lane & 15;
  const int tr_off = (4 * hf + (tr_i >> 2)) * VSTR + 16 * ((lane >> 4) & 1) + 4 * (tr_i & 3);

  // ---- O^T += V^T . P^T ; P operand slot j of half hf (block kb, group g)
  //      is key 16(2kb+g) + 4hf + (j<4 ? j : j+4) ----
  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[db][i] = 0.f;
  auto pv = [&](int buf, const bf16x8 (&pb)[2][2]) {
    const bf16 *vt = Vbuf(buf) + tr_off;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const bf16 *p0 = vt + 16 * (2 * kb + g) * VSTR + 32 * db;
          const u32x2 lo = lds_read_tr16(p0);
          const u32x2 hi = lds_read_tr16(p0 + 8 * VSTR);
          const bf16x8 va = bit_cast<bf16x8>(u32x4{lo.x, lo.y, hi.x, hi.y});
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[kb][g], oacc[db], 0, 0, 0);
        }
    }
  };

  float m_run = -INFINITY, l_run = 0.f;
  const float c = a.scale_log2;
  const float thresh = kRescaleLog2 / c;    // in raw score units
  const uint32_t ones_bf16x2 = 0x3f803f80u;

  // ---- online softmax of one tile (scores in sacc; accumulator row i of
  //      block kb is key kb*32 + 8*(i/4) + 4*hf + i%4).  P is first computed
  //      against the running max m_run: that is exact and bounded by 2^8
  //      unless some row's tile max exceeds m_run by the threshold, which is
  //      rare after the first tile.  Then the slow path rescales O and l and
  //      recomputes P against the new max. ----
  auto exp_tile = [&](const f32x16 (&sacc)[2], float mref, bf16x8 (&pb)[2][2]) -> float {
    const float mc = mref * c;
    float lt = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][g * 8 + 2 * e], c, -mc));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][g * 8 + 2 * e + 1], c, -mc));
          w[e] = pack_bf16x2(p0, p1);
          // the normaliser sums the same bf16-rounded P that feeds P.V
          lt = __builtin_amdgcn_fdot2_f32_bf16(bit_cast<bf16x2>(w[e]),
                                               bit_cast<bf16x2>(ones_bf16x2), lt, false);
        }
        pb[kb][g] = bit_cast<bf16x8>(u32x4{w[0], w[1], w[2], w[3]});
      }
    return lt;
  };
  auto softmax = [&]<bool TAIL>(f32x16 (&sacc)[2], int j0, bf16x8 (&pb)[2][2]) {
    if constexpr (TAIL) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (j0 + kb * 32 + 8 * (i / 4) + 4 * hf + (i % 4) >= S) sacc[kb][i] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
    mx = half_max(mx);
    const bool grow = mx > m_run + thresh;
    float lt = exp_tile(sacc, m_run, pb);
    if (__builtin_amdgcn_ballot_w64(grow)) {
      // keep the speculative P computed before the branch (it is the result
      // on the common path); here it is replaced
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int g = 0; g < 2; ++g) asm volatile("" ::"v"(pb[kb][g]));
      const float m_new = grow ? mx : m_run;
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
      lt = exp_tile(sacc, m_new, pb);
    }
    l_run += lt;
  };

  // ---- software pipeline over key tiles.  K tile x lives in K buffer x%2
  //      and V tile x in V buffer x%2.  Iteration t computes Q K^T of tile
  //      t+1 while it runs the softmax of tile t, then P.V of tile t while it
  //      rotates and stores K of tile t+2 and V of tile t+1 (both into the
  //      buffers freed by iteration t-1); one barrier per iteration. ----
  const int ntiles = (S + BN - 1) / BN;
  load_k(0);
  load_v(0);
  store_k(0);
  store_v(0);
  if (ntiles > 1) {
    load_k(1);
    store_k(1);
  }
  __syncthreads();
  f32x16 s_a[2], s_b[2];
  qk(0, s_a);

  // One pipeline step: softmax of tile t from `cur`, Q K^T of tile t+1 into
  // `nxt`.  NEXT: a tile t+1 exists (its Q K^T computed, its V staged); K2: a
  // tile t+2 exists (its K staged).  Only the last tile can be partial.
  auto iteration = [&]<bool NEXT, bool K2>(int t, f32x16 (&cur)[2], f32x16 (&nxt)[2]) {
    const int j0 = t * BN;
    if constexpr (K2) load_k(t + 2);
    if constexpr (NEXT) load_v(t + 1);
    if constexpr (NEXT) qk((t + 1) & 1, nxt);
    bf16x8 pb[2][2];
    softmax.template operator()<!NEXT>(cur, j0, pb);
    pv(t & 1, pb);
    if constexpr (K2) store_k(t & 1);
    if constexpr (NEXT) store_v((t + 1) & 1);
    __syncthreads();
  };
  int t = 0;
  for (; t + 2 < ntiles; ++t) {
    iteration.template operator()<true, true>(t, s_a, s_b);
    s_a[0] = s_b[0];
    s_a[1] = s_b[1];
  }
  if (t + 1 < ntiles) {
    iteration.template operator()<true, false>(t, s_a, s_b);
    iteration.template operator()<false, false>(t + 1, s_b, s_a);
  } else {
    iteration.template operator()<false, false>(t, s_a, s_b);
  }

  // ---- epilogue: O = acc / l, bf16; LSE in natural log ----
  const float l_tot = half_sum(l_run);
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
      a.lse[((int64_t)b * a.H + h) * S + qi] = (m_run * c + __log2f(l_tot)) * kLn2;
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
  a.B = L.B;
  a.n_qblk = (L.S + BM - 1) / BM;
  a.scale_log2 = L.scale_log2;
  const int64_t nwg = (int64_t)a.n_qblk * L.H * L.B;
  const dim3 grid((unsigned)nwg);
  const bool rope_on = rope != nullptr;
  if (L.D == 64) {
    auto kern = rope_on ? attn_fwd_bf16_kernel<64, true> : attn_fwd_bf16_kernel<64, false>;
    hipLaunchKernelGGL(kern, grid, dim3(NT), Lds<64>::BYTES, st, a);
  } else {
    static const hipError_t attr = []() {
      hipError_t e = hipFuncSetAttribute(
          reinterpret_cast<const void *>(&attn_fwd_bf16_kernel<128, true>),
          hipFuncAttributeMaxDynamicSharedMemorySize, Lds<128>::BYTES);
      if (e != hipSuccess) return e;
      return hipFuncSetAttribute(
          reinterpret_cast<const void *>(&attn_fwd_bf16_kernel<128, false>),
          hipFuncAttributeMaxDynamicSharedMemorySize, Lds<128>::BYTES);
    }();
    if (attr != hipSuccess) return attr;
    auto kern = rope_on ? attn_fwd_bf16_kernel<128, true> : attn_fwd_bf16_kernel<128, false>;
    hipLaunchKernelGGL(kern, grid, dim3(NT), Lds<128>::BYTES, st, a);
  }
  return hipGetLastError();
}

}  // namespace ja
