// BF16 joint-attention forward for gfx950 with RoPE fused into the Q/K load.
//
// Joint attention ("Speed Up Image Generation with FLUX 3 Image Klein on
// NVIDIA Blackwell GPUs", section "FLUX 3 inference with TensorRT LLM
// VisualGen"): one dense softmax over the concatenated text / target / reference
// tokens.  RoPE is applied to Q and K before the product (same page, section
// "GEMM kernel optimization"); here it is applied in fp32 while Q and K are
// loaded and the rotated values are rounded to bf16 for the MFMA.
//
// Work decomposition: one workgroup per (384-query block, head, batch row),
// twelve wave64s of 32 query rows each, three per SIMD.  Both products are
// computed transposed so that a lane owns one query row throughout:
//   S^T[key][q]  = K . Q^T      (v_mfma_f32_32x32x16_bf16, A = rotated K from
//                                LDS, B = rotated Q kept in registers)
//   O^T[d][q]   += V^T . P^T    (A = V^T from LDS, B = P straight from the S^T
//                                accumulators)
// With that orientation the online-softmax state (running max m and sum l,
// fp32) is per lane, the row max needs one cross-half exchange and the O
// rescale is one multiply per accumulator.
//
// K/V tiles of 32 keys are double-buffered in LDS.  K is staged row-major
// (rotated in fp32 and rounded to bf16 on the way); V is staged transposed
// (one row per head-dimension column, the keys of a row in the order in which
// the P operand holds them), so both MFMA operands are single 16-byte LDS
// reads.  Rows are padded so that the 16 lanes served together hit distinct
// banks.
//
// Each wave runs Q K^T, softmax and P.V of a tile in turn; the three waves of
// a SIMD overlap one another's MFMA, VALU and memory waits (a wave needs 160
// VGPRs this way, against more than 168 for a wave that also overlaps the
// next tile's Q K^T with its own softmax).  The next tiles' global loads are
// issued one iteration ahead; one barrier per tile.
//
// Block-sparse variant (the kernel half of the pages' sparse attention,
// section "Quantized and sparse attention": attention restricted to the
// blocks of a given block mask over 128-query x 64-key blocks).  A workgroup
// covers three query blocks; it first compacts, in LDS, the list of key
// blocks that any of the three keeps, with a 3-bit flag per entry, then
// stages only the tiles of that list.  A wave computes a staged tile only if
// its own query block keeps it (a wave-uniform branch); staging and the
// barrier are shared.  Query rows that keep no key get O = 0 and LSE = -inf.
#include "common.hpp"
#include "internal.hpp"

namespace ja {

namespace {

#ifndef JA_BF16_WAVES
#define JA_BF16_WAVES 12
#endif
#ifndef JA_BF16_STAGE_WAVES
#define JA_BF16_STAGE_WAVES JA_BF16_WAVES
#endif
#ifndef JA_BF16_RW
#define JA_BF16_RW 1
#endif
constexpr int NW = JA_BF16_WAVES;   // waves per workgroup
constexpr int RW = JA_BF16_RW;      // 32-row query blocks per wave
constexpr int BM = 32 * RW * NW;    // query rows per workgroup
constexpr int BN = 32;              // keys per K/V tile
constexpr int NT = 64 * NW;         // threads per workgroup
constexpr int NS = 64 * JA_BF16_STAGE_WAVES;   // threads that stage K/V tiles
// One workgroup per CU: 12 waves, three per SIMD, at most 168 VGPRs each.
// Latency is hidden by the three waves of a SIMD rather than by deeper
// software pipelining inside a wave (which needs more registers).
constexpr int WG_PER_CU = 1;

// Block-mask granularity of the block-sparse variant.
constexpr int kQueryBlock = 128;
constexpr int kKeyBlock = 64;
constexpr int KB_TILES = kKeyBlock / BN;              // key tiles per key block
constexpr int QB_PER_WG = BM / kQueryBlock;           // query blocks per workgroup
static_assert(BM % kQueryBlock == 0 && kKeyBlock % BN == 0, "mask blocks");
static_assert(QB_PER_WG <= 16, "query-block flags");
// Longest sequence of the block-sparse variant (its key-block list lives in
// LDS, 4 bytes per key block, and entries hold the key block in 16 bits).
constexpr int kSparseMaxSeq = 1 << 20;

// Rescale the output accumulator only when the running row max grows by more
// than 2^24 in the exp2 domain.  Until then P may exceed 1 by up to 2^24;
// fp32 and bf16 carry such values with the same relative precision as values
// below 1, and the sums stay far below the fp32 range.
constexpr float kRescaleLog2 = 24.f;

// Buffer-resource word 3 for raw (unswizzled, unformatted 32-bit) buffer
// access on gfx950: reads outside [0, num_records) return zeros (the check
// covers the scalar offset too).
constexpr int kBufferFlags = 0x00020000;

#define JA_INLINE __attribute__((always_inline))

struct FwdArgs {
  const bf16 *q, *k, *v;
  const float2 *rope;
  bf16 *o;
  float *lse;
  int64_t q_sb, q_ss, q_sh, k_sb, k_ss, k_sh, v_sb, v_ss, v_sh, o_sb, o_ss, o_sh;
  int S, H, B, n_qblk;
  float scale_log2;
  // Split of the last, partial round of workgroups over key ranges: the
  // first n_direct workgroups each own one (q-block, head, batch) item; the
  // remaining ones are `parts` workgroups per item, each over a contiguous
  // range of key tiles, writing unnormalised partial results to `ws`.
  int n_direct, parts;
  SplitWorkspace ws;
  // block-sparse variant: mask [B][H][nqb][nkb] (nonzero = keep)
  const uint8_t *mask;
  int nqb, nkb;
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

template <int D>
struct Lds {
  static constexpr int KSTR = D + 8;        // bf16 per K row (16-byte pad)
  static constexpr int VTSTR = BN + 8;      // bf16 per V^T row (16-byte pad)
  static constexpr int KTILE = BN * KSTR;
  static constexpr int VTILE = D * VTSTR;
  static constexpr int BYTES = 2 * (KTILE + VTILE) * 2;
  // block-sparse variant: per-wave counts, then the key-block list
  static constexpr int LIST_OFFSET = BYTES + 64;
  static constexpr int sparse_bytes(int nkb) { return LIST_OFFSET + 4 * nkb; }
};

// Position, inside a 16-key group of a V^T row, of key k: the P operand of
// lane half hf holds keys 4hf + {0..3} and 4hf + {8..11} of the group in its
// eight slots, so V^T stores them at 8hf + slot.
__host__ __device__ constexpr int vt_key_of_slot(int p) {
  return 4 * (p / 8) + (p % 8 < 4 ? p % 8 : p % 8 + 4);
}

template <int D, bool ROPE, bool SPARSE>
__global__ __launch_bounds__(NT, WG_PER_CU) void attn_fwd_bf16_kernel(FwdArgs a) {
  constexpr int CH = D / 8;                  // 16-byte chunks per K row
  constexpr int K_CHUNKS = BN * CH;          // 16-byte K chunks per tile
  constexpr int V_SLOTS = D * (BN / 8);      // 8-key V^T slots per tile
  constexpr int KP = (K_CHUNKS + NS - 1) / NS;   // K chunks per staging thread
  constexpr int VP = (V_SLOTS + NS - 1) / NS;    // V^T slots per staging thread
  static_assert(K_CHUNKS % NS == 0 || K_CHUNKS < NS, "staging layout");
  static_assert(V_SLOTS % NS == 0 || V_SLOTS < NS, "staging layout");
  static_assert(NS % D == 0, "V^T slot groups must be wave-uniform");
  constexpr int K_THREADS = K_CHUNKS < NS ? K_CHUNKS : NS;
  constexpr int V_THREADS = V_SLOTS < NS ? V_SLOTS : NS;
  constexpr int KSTR = Lds<D>::KSTR, VTSTR = Lds<D>::VTSTR;
  extern __shared__ __attribute__((aligned(16))) bf16 smem[];
  auto Kbuf = [&](int buf) JA_INLINE { return smem + buf * Lds<D>::KTILE; };
  auto Vbuf = [&](int buf) JA_INLINE { return smem + 2 * Lds<D>::KTILE + buf * Lds<D>::VTILE; };

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hf = lane >> 5;

  // XCD-aware placement: workgroups are dispatched round-robin over the 8
  // XCDs, so give each XCD a contiguous range of (q-block, head) work items;
  // the workgroups resident on one XCD then stream the same head's K/V
  // through that XCD's L2.
  const int S = a.S;
  const int ntiles_all = (S + BN - 1) / BN;
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
  const int bh = item / a.n_qblk;
  const int h = bh % a.H, b = bh / a.H;

  // ---- block-sparse variant: compact the key blocks kept by any of this
  //      workgroup's query blocks into an LDS list (ascending), entry =
  //      key block | (flags of the query blocks that keep it) << 16.  The
  //      workgroup's key tiles are then the tiles of the listed blocks that
  //      lie inside the sequence; the dense kernel's tiles are 0..ntiles-1. ----
  uint32_t *blist = reinterpret_cast<uint32_t *>(reinterpret_cast<char *>(smem) + Lds<D>::LIST_OFFSET);
  int ntiles = ntiles_all;
  if constexpr (SPARSE) {
    int *wcnt = reinterpret_cast<int *>(reinterpret_cast<char *>(smem) + Lds<D>::BYTES);
    const int qb0 = qblk * QB_PER_WG;
    const uint8_t *mrow = a.mask + ((int64_t)bh * a.nqb + qb0) * a.nkb;
    int nact = 0;
    for (int base = 0; base < a.nkb; base += NT) {
      const int j = base + tid;
      uint32_t flags = 0;
      if (j < a.nkb) {
#pragma unroll
        for (int r = 0; r < QB_PER_WG; ++r)
          if (qb0 + r < a.nqb && mrow[(int64_t)r * a.nkb + j] != 0) flags |= 1u << r;
      }
      const uint64_t bal = __builtin_amdgcn_ballot_w64(flags != 0);
      if (lane == 0) wcnt[wave] = (int)__builtin_popcountll(bal);
      __syncthreads();
      int off = nact, tot = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const int cw = wcnt[w];
        off += w < wave ? cw : 0;
        tot += cw;
      }
      if (flags) blist[off + __builtin_popcountll(bal & ((1ull << lane) - 1))] = (uint32_t)j | (flags << 16);
      nact += tot;
      __syncthreads();
    }
    ntiles = nact * KB_TILES;
    if (nact > 0) {
      // tiles of the last key block past the end of the sequence
      const int kb_last = (int)(blist[nact - 1] & 0xffffu);
      ntiles -= max(0, (kb_last + 1) * KB_TILES - ntiles_all);
    }
  }
  int t0 = 0, t1 = ntiles;
  if (unit >= 0) {
    t0 = (int)((int64_t)part * ntiles / a.parts);
    t1 = (int)((int64_t)(part + 1) * ntiles / a.parts);
  }
  // key tile of list position x, and whether this wave's query block keeps it
  const int my_qb = (wave * RW * 32) / kQueryBlock;
  auto tile_of = [&](int x) JA_INLINE -> int {
    if constexpr (SPARSE) {
      const uint32_t e = __builtin_amdgcn_readfirstlane(blist[x / KB_TILES]);
      return (int)(e & 0xffffu) * KB_TILES + x % KB_TILES;
    } else {
      return x;
    }
  };
  auto kept = [&](int x) JA_INLINE -> bool {
    if constexpr (SPARSE) {
      const uint32_t e = __builtin_amdgcn_readfirstlane(blist[x / KB_TILES]);
      return (e >> (16 + my_qb)) & 1u;
    } else {
      return true;
    }
  };

  // ---- Q rows of this lane (one per 32-row block): rotate, round to bf16,
  //      keep in registers ----
  int qi[RW];
  bf16x8 qreg[RW][D / 16];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    qi[r] = qblk * BM + (wave * RW + r) * 32 + l32;
    const int qs = qi[r] < S ? qi[r] : S - 1;
    const bf16 *qrow = a.q + b * a.q_sb + (int64_t)qs * a.q_ss + h * a.q_sh;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const int d0 = 16 * kk + 8 * hf;
      u32x4 w = *reinterpret_cast<const u32x4 *>(qrow + d0);
      if constexpr (ROPE) w = rope_chunk_bf16(w, a.rope + (int64_t)qs * (D / 2) + d0 / 2);
      if (qi[r] >= S) w = u32x4{0, 0, 0, 0};
      qreg[r][kk] = bit_cast<bf16x8>(w);
    }
  }

  // ---- staging: global -> registers through buffer resources, then
  //      registers -> LDS.  Per-lane offsets inside a tile are fixed; the
  //      tile offset is scalar.  Each resource ends after row S-1, so rows
  //      past the end of the sequence read as zeros (their scores are masked
  //      and their P is 0). ----
  const bf16 *kbase = a.k + b * a.k_sb + h * a.k_sh;
  const bf16 *vbase = a.v + b * a.v_sb + h * a.v_sh;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16 *>(kbase), 0, (int)(((int64_t)(S - 1) * a.k_ss + D) * 2), kBufferFlags);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16 *>(vbase), 0, (int)(((int64_t)(S - 1) * a.v_ss + D) * 2), kBufferFlags);
  const __amdgpu_buffer_rsrc_t trs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float2 *>(a.rope), 0, ROPE ? S * D * 4 : 0, kBufferFlags);

  // K: pass p of a staging thread stages chunk st_c of row st_r + p * (NS / CH)
  const int st_r = tid / CH, st_c = tid % CH;
  const int koff = (int)(st_r * a.k_ss * 2) + st_c * 16;
  const int toff = st_r * D * 4 + st_c * 32;
  const int ktile_bytes = (int)(BN * a.k_ss * 2);
  const int kpass_bytes = (int)((NS / CH) * a.k_ss * 2);
  // V^T: pass p of a thread stages column vd, slots 8 vc .. 8 vc + 7 with
  // vc = tid / D + p * (NS / D) (wave-uniform)
  const int vd = tid % D;
  const int vc0 = __builtin_amdgcn_readfirstlane(tid / D);
  const int vrow_bytes = (int)(a.v_ss * 2);
  u32x4 kreg[KP];
  float4 treg[KP][2];
  uint32_t vreg[VP][8];
  auto load_k = [&](int t) JA_INLINE {
    if (K_THREADS < NT && tid >= K_THREADS) return;
#pragma unroll
    for (int p = 0; p < KP; ++p) {
      kreg[p] = bit_cast<u32x4>(__builtin_amdgcn_raw_buffer_load_b128(
          krs, koff, t * ktile_bytes + p * kpass_bytes, 0));
      if constexpr (ROPE) {
        const int tt = (t * BN + p * (NS / CH)) * D * 4;
        treg[p][0] = bit_cast<float4>(__builtin_amdgcn_raw_buffer_load_b128(trs, toff, tt, 0));
        treg[p][1] = bit_cast<float4>(__builtin_amdgcn_raw_buffer_load_b128(trs, toff + 16, tt, 0));
      }
    }
  };
  auto load_v = [&](int t) JA_INLINE {
    if (V_THREADS < NT && tid >= V_THREADS) return;
#pragma unroll
    for (int p = 0; p < VP; ++p) {
      const int vc = vc0 + p * (NS / D);
      const int key0 = t * BN + 16 * (vc >> 1);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        vreg[p][j] = __builtin_amdgcn_raw_buffer_load_b16(
            vrs, vd * 2, (key0 + vt_key_of_slot(8 * (vc & 1) + j)) * vrow_bytes, 0);
    }
  };
  // The empty asm statements in the stores pin the use of the loaded
  // registers there: otherwise the compiler moves the rotation and packing
  // (and with them the wait for the loads) up to just after the previous
  // barrier, where every wave would wait for memory at the same moment.
  auto store_k = [&](int buf) JA_INLINE {
    if (K_THREADS < NT && tid >= K_THREADS) return;
#pragma unroll
    for (int p = 0; p < KP; ++p) {
      asm volatile("" : "+v"(kreg[p]));
      if constexpr (ROPE) {
        u32x4 c0 = bit_cast<u32x4>(treg[p][0]), c1 = bit_cast<u32x4>(treg[p][1]);
        asm volatile("" : "+v"(c0), "+v"(c1));
        treg[p][0] = bit_cast<float4>(c0);
        treg[p][1] = bit_cast<float4>(c1);
      }
      u32x4 kw = kreg[p];
      if constexpr (ROPE) {
        kw.x = rope_pair_bf16(kw.x, make_float2(treg[p][0].x, treg[p][0].y));
        kw.y = rope_pair_bf16(kw.y, make_float2(treg[p][0].z, treg[p][0].w));
        kw.z = rope_pair_bf16(kw.z, make_float2(treg[p][1].x, treg[p][1].y));
        kw.w = rope_pair_bf16(kw.w, make_float2(treg[p][1].z, treg[p][1].w));
      }
      *reinterpret_cast<u32x4 *>(Kbuf(buf) + (st_r + p * (NS / CH)) * KSTR + st_c * 8) = kw;
    }
  };
  auto store_v = [&](int buf) JA_INLINE {
    if (V_THREADS < NT && tid >= V_THREADS) return;
#pragma unroll
    for (int p = 0; p < VP; ++p) {
      const int vc = vc0 + p * (NS / D);
#pragma unroll
      for (int j = 0; j < 8; ++j) asm volatile("" : "+v"(vreg[p][j]));
      u32x4 w;
      w.x = vreg[p][0] | (vreg[p][1] << 16);
      w.y = vreg[p][2] | (vreg[p][3] << 16);
      w.z = vreg[p][4] | (vreg[p][5] << 16);
      w.w = vreg[p][6] | (vreg[p][7] << 16);
      *reinterpret_cast<u32x4 *>(Vbuf(buf) + vd * VTSTR + 8 * vc) = w;
    }
  };

  // ---- S^T = K . Q^T for this wave's 32 queries and the 32 keys of a tile,
  //      in two halves over the head dimension ----
  auto qk = [&]<int KK0, int KK1>(int buf, f32x16 (&sacc)[RW]) JA_INLINE {
    if constexpr (KK0 == 0) {
#pragma unroll
      for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[r][i] = 0.f;
    }
    const bf16 *krow = Kbuf(buf) + l32 * KSTR + 8 * hf;
#pragma unroll
    for (int kk = KK0; kk < KK1; ++kk) {
      const bf16x8 kv = *reinterpret_cast<const bf16x8 *>(krow + 16 * kk);
#pragma unroll
      for (int r = 0; r < RW; ++r)
        sacc[r] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kv, qreg[r][kk], sacc[r], 0, 0, 0);
    }
  };

  // ---- O^T += V^T . P^T ; P operand slot j of half hf (key group g) is key
  //      16g + 4hf + (j<4 ? j : j+4), which V^T stores at 16g + 8hf + j ----
  f32x16 oacc[RW][D / 32];
#pragma unroll
  for (int r = 0; r < RW; ++r)
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[r][db][i] = 0.f;
  auto pv = [&](const bf16x8 (&pb)[RW][2], int buf) JA_INLINE {
    const bf16 *vt = Vbuf(buf) + l32 * VTSTR + 8 * hf;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const bf16x8 va = *reinterpret_cast<const bf16x8 *>(vt + 32 * db * VTSTR + 16 * g);
#pragma unroll
        for (int r = 0; r < RW; ++r)
          oacc[r][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[r][g], oacc[r][db], 0, 0, 0);
      }
  };

  float m_run[RW], l_run[RW];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    m_run[r] = -INFINITY;
    l_run[r] = 0.f;
  }
  const float c = a.scale_log2;
  const float thresh = kRescaleLog2 / c;    // in raw score units
  const uint32_t ones_bf16x2 = 0x3f803f80u;

  // ---- online softmax of one tile (accumulator row i is key
  //      8*(i/4) + 4*hf + i%4).  P is first computed against the running max
  //      m_run: that is exact and bounded by 2^24 unless some row's tile max
  //      exceeds m_run by the threshold, which is rare after the first tile.
  //      Then the slow path rescales O and l and recomputes P against the new
  //      max. ----
  auto exp_tile = [&](const f32x16 &sacc, float mref, bf16x8 (&pb)[2]) JA_INLINE -> float {
    const float mc = mref * c;
    float lt = 0.f;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[g * 8 + 2 * e], c, -mc));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[g * 8 + 2 * e + 1], c, -mc));
        w[e] = pack_bf16x2(p0, p1);
        // the normaliser sums the same bf16-rounded P that feeds P.V
        lt = __builtin_amdgcn_fdot2_f32_bf16(bit_cast<bf16x2>(w[e]),
                                             bit_cast<bf16x2>(ones_bf16x2), lt, false);
      }
      pb[g] = bit_cast<bf16x8>(u32x4{w[0], w[1], w[2], w[3]});
    }
    return lt;
  };
  auto softmax = [&]<bool TAIL>(f32x16 (&sacc)[RW], int j0, bf16x8 (&pb)[RW][2]) JA_INLINE {
    float mx[RW], lt[RW];
    bool grow[RW], any = false;
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      if constexpr (TAIL) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (j0 + 8 * (i / 4) + 4 * hf + (i % 4) >= S) sacc[r][i] = -INFINITY;
      }
      mx[r] = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) mx[r] = fmaxf(mx[r], sacc[r][i]);
      mx[r] = half_max(mx[r]);
      grow[r] = mx[r] > m_run[r] + thresh;
      any = any || grow[r];
      lt[r] = exp_tile(sacc[r], m_run[r], pb[r]);
    }
    if (__builtin_amdgcn_ballot_w64(any)) {
      // keep the speculative P computed before the branch (it is the result
      // on the common path); here it is replaced
#pragma unroll
      for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int g = 0; g < 2; ++g) asm volatile("" ::"v"(pb[r][g]));
#pragma unroll
      for (int r = 0; r < RW; ++r) {
        const float m_new = grow[r] ? mx[r] : m_run[r];
        const float alpha = __builtin_amdgcn_exp2f((m_run[r] - m_new) * c);
        m_run[r] = m_new;
        l_run[r] *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[r][db][i] *= alpha;
        lt[r] = exp_tile(sacc[r], m_new, pb[r]);
      }
    }
#pragma unroll
    for (int r = 0; r < RW; ++r) l_run[r] += lt[r];
  };

  // ---- loop over the key tiles t0 .. t1-1 (local index i = t - t0).  Local
  //      tile i lives in K buffer i%2 and V buffer i%2.  Iteration i computes
  //      Q K^T, the softmax and P.V of tile i, then rotates and stores K and V
  //      of tile i+1 (into the buffers read by iteration i-1) and issues the
  //      global loads of tile i+2, which have a whole iteration to arrive; a
  //      barrier closes the iteration. ----
  const int nt = t1 - t0;
  // a dense workgroup always has at least one tile; a sparse one may have none
  const bool any_tile = !SPARSE || nt > 0;
  if (any_tile) {
    load_k(tile_of(t0));
    load_v(tile_of(t0));
    store_k(0);
    store_v(0);
    if (nt > 1) {
      load_k(tile_of(t0 + 1));
      load_v(tile_of(t0 + 1));
    }
    __syncthreads();
  }
  f32x16 sacc[RW];
  // NEXT: tile i+1 exists.  Only the last tile of the sequence can be partial
  // (masking a full tile changes nothing), and it is always the last of the
  // workgroup's tiles.
  auto iteration = [&]<bool NEXT>(int i) JA_INLINE {
    const int t = tile_of(t0 + i);
    if (kept(t0 + i)) {
      qk.template operator()<0, D / 16>(i & 1, sacc);
      bf16x8 pb[RW][2];
      softmax.template operator()<!NEXT>(sacc, t * BN, pb);
      pv(pb, i & 1);
    }
    if constexpr (NEXT) {
      store_k((i + 1) & 1);
      store_v((i + 1) & 1);
      if (i + 2 < nt) {
        const int t2 = tile_of(t0 + i + 2);
        load_k(t2);
        load_v(t2);
      }
    }
    __syncthreads();
  };
  for (int i = 0; i + 1 < nt; ++i) iteration.template operator()<true>(i);
  if (any_tile) iteration.template operator()<false>(nt - 1);

  // ---- a split part leaves O unnormalised, with its row max (raw score
  //      units) and row sum, for the merge kernel ----
  if (unit >= 0) {
#pragma unroll
    for (int r = 0; r < RW; ++r) {
      const float l_tot = half_sum(l_run[r]);
      const int row = (wave * RW + r) * 32 + l32;
      float *orow = a.ws.o + ((int64_t)unit * BM + row) * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int grp = 0; grp < 4; ++grp)
          *reinterpret_cast<float4 *>(orow + db * 32 + 8 * grp + 4 * hf) =
              make_float4(oacc[r][db][4 * grp], oacc[r][db][4 * grp + 1],
                          oacc[r][db][4 * grp + 2], oacc[r][db][4 * grp + 3]);
      if (hf == 0)
        *reinterpret_cast<float2 *>(a.ws.ml + ((int64_t)unit * BM + row) * 2) =
            make_float2(m_run[r], l_tot);
    }
    return;
  }

  // ---- epilogue: O = acc / l, bf16; LSE in natural log ----
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    const float l_tot = half_sum(l_run[r]);
    if (qi[r] < S) {
      // a row of the block-sparse variant that keeps no key has l = 0 (and
      // O accumulators 0): O = 0, LSE = -inf
      const float inv = SPARSE && l_tot == 0.f ? 0.f : 1.f / l_tot;
      bf16 *orow = a.o + b * a.o_sb + (int64_t)qi[r] * a.o_ss + h * a.o_sh;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int grp = 0; grp < 4; ++grp) {
          const int d = db * 32 + 8 * grp + 4 * hf;
          u32x2 w;
          w.x = pack_bf16x2(oacc[r][db][4 * grp + 0] * inv, oacc[r][db][4 * grp + 1] * inv);
          w.y = pack_bf16x2(oacc[r][db][4 * grp + 2] * inv, oacc[r][db][4 * grp + 3] * inv);
          *reinterpret_cast<u32x2 *>(orow + d) = w;
        }
      if (a.lse && hf == 0)
        a.lse[((int64_t)b * a.H + h) * S + qi[r]] = (m_run[r] * c + __log2f(l_tot)) * kLn2;
    }
  }
}

// Dynamic LDS of one instantiation; kernels that need more than the default
// limit get it raised once per process.
template <int D, bool ROPE, bool SPARSE>
hipError_t launch_instance(const FwdArgs &a, dim3 grid, hipStream_t st) {
  const int bytes = SPARSE ? Lds<D>::sparse_bytes(a.nkb) : Lds<D>::BYTES;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void *>(&attn_fwd_bf16_kernel<D, ROPE, SPARSE>),
      hipFuncAttributeMaxDynamicSharedMemorySize,
      SPARSE ? Lds<D>::sparse_bytes((kSparseMaxSeq + kKeyBlock - 1) / kKeyBlock) : Lds<D>::BYTES);
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, ROPE, SPARSE>), grid, dim3(NT), bytes, st, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_dim(const FwdArgs &a, dim3 grid, bool rope_on, hipStream_t st) {
  if (a.mask)
    return rope_on ? launch_instance<D, true, true>(a, grid, st)
                   : launch_instance<D, false, true>(a, grid, st);
  return rope_on ? launch_instance<D, true, false>(a, grid, st)
                 : launch_instance<D, false, false>(a, grid, st);
}

}  // namespace

int fwd_bf16_block_rows(int) { return BM; }

SplitPlan plan_fwd_bf16(const AttnLayout &L, int n_cu) {
  const int n_items = ((L.S + BM - 1) / BM) * L.H * L.B;
  return plan_split(n_items, (L.S + BN - 1) / BN, n_cu * WG_PER_CU, BM, L.D);
}

int fwd_bf16_sparse_max_seq() { return kSparseMaxSeq; }

hipError_t launch_fwd_bf16(const AttnLayout &L, const void *q, const void *k,
                           const void *v, const float *rope, const uint8_t *mask,
                           void *o, float *lse, const SplitPlan &plan, void *workspace,
                           hipStream_t st) {
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
  a.n_direct = plan.n_direct;
  a.parts = plan.parts;
  a.ws = split_workspace(plan, workspace, BM, L.D);
  a.mask = mask;
  a.nqb = (L.S + kQueryBlock - 1) / kQueryBlock;
  a.nkb = (L.S + kKeyBlock - 1) / kKeyBlock;
  const dim3 grid((unsigned)(plan.n_direct + plan.n_units));
  const hipError_t e = L.D == 64 ? launch_dim<64>(a, grid, rope != nullptr, st)
                                 : launch_dim<128>(a, grid, rope != nullptr, st);
  if (e != hipSuccess || plan.n_units == 0) return e;
  return launch_merge_split(L, plan, a.ws, BM, L.scale_log2, o, lse, st);
}

}  // namespace ja
