// BF16 joint-attention forward for gfx950 with RoPE fused into the Q/K load.
//
// Joint attention ("Speed Up Image Generation with FLUX 3 Image Klein on
// NVIDIA Blackwell GPUs", section "FLUX 3 inference with TensorRT LLM
// VisualGen"): one dense softmax over the concatenated text / target / reference
// tokens.  RoPE is applied to Q and K before the product (same page, section
// "GEMM kernel optimization"); here it is applied in fp64 while Q is loaded
// (K in the preparation pass) and the rotated values are rounded once to
// bf16 for the MFMA.
//
// Work decomposition: one workgroup per (512-query block, head, batch row),
// eight wave64s of 64 query rows each (two 32-row blocks), two per SIMD.
// The two blocks of a wave share every K and V^T fragment read from LDS,
// which halves the LDS bytes per MFMA flop against 32-row waves; under the
// chip's power limit that energy is what sets the clock.  Both products are
// computed transposed so that a lane owns one query row of each block
// throughout:
//   S^T[key][q]  = K . Q^T      (v_mfma_f32_32x32x16_bf16, A = rotated K from
//                                LDS, B = rotated Q kept in registers)
//   O^T[d][q]   += V^T . P^T    (A = V^T from LDS, B = P straight from the S^T
//                                accumulators)
// With that orientation the online-softmax state (running max m and sum l,
// fp32) is per lane, the row max needs one cross-half exchange and the O
// rescale is one multiply per accumulator.
//
// K and V arrive from the preparation pass (prep_kv.hip) as rotated K rows
// and as V^T rows whose keys are in the order in which the P operand holds
// them, so both MFMA operands are single 16-byte LDS reads.  Tiles of 32 keys
// go from HBM straight into an LDS ring (four stages; three for the
// block-sparse variant's smaller workgroups) with buffer loads to LDS: no
// registers, no VALU work, and the loads of a tile are issued a ring's depth
// minus one tiles ahead of its use.  A K tile is stored in fragment order
// (1 KB per 16-column step: lane l's 16 bytes of row l%32 at byte 16 l) and
// V^T rows are XOR-swizzled, so that the 16 lanes served together by a
// fragment read hit distinct banks.
//
// Each wave runs Q K^T, softmax and P.V of a tile in turn; the two waves of
// a SIMD overlap one another's MFMA, VALU and memory waits (a wave fits in
// 256 VGPRs this way: 128 for O, 64 for Q, 32 for S).  Inside Q K^T and P.V
// the LDS fragment reads run four fragments ahead.  One barrier per tile; it
// waits only for the loads of the next tile, never for the ones still in
// flight behind it.
//
// Block-sparse variant (the kernel half of the pages' sparse attention,
// section "Quantized and sparse attention": attention restricted to the
// blocks of a given block mask over 128-query x 64-key blocks).  A workgroup
// of four waves covers one query block, three such workgroups share a CU; it
// first compacts, in LDS, the list of key blocks its query block keeps, then
// stages only the tiles of that list.  (The code keeps a per-entry flag for
// each query block of a workgroup and a wave-uniform skip of tiles its own
// block does not keep, which a one-block workgroup never takes.)  Query rows
// that keep no key get O = 0 and LSE = -inf.
#include <atomic>

#include "common.hpp"
#include "internal.hpp"

namespace ja {

namespace {

constexpr int BN = 32;              // keys per K/V tile
static_assert(BN == kVtTile, "a V^T tile of the prepared buffer is one K/V tile");

// Block-mask granularity of the block-sparse variant.
constexpr int kQueryBlock = 128;
constexpr int kKeyBlock = 64;
constexpr int KB_TILES = kKeyBlock / BN;              // key tiles per key block

// Workgroup shapes.  Wide (the dense forward when its items fill the CUs):
// one workgroup of 8 waves of 64 rows per CU, two per SIMD at most 256
// VGPRs each, over a 4-stage ring; latency is hidden by the two waves of a
// SIMD rather than by software pipelining inside a wave (which needs more
// registers).  Small (the block-sparse variant, and the dense forward when
// the wide items would fill at most half of the CUs): one 128-row query block per
// workgroup of 4 waves of 32 rows, three workgroups per CU over 3-stage
// rings, so that a block-sparse workgroup stages only the key tiles its own
// query block keeps, and a short dense launch has four times as many items
// to spread over the CUs.
template <bool SMALL>
struct Cfg {
  static constexpr int RW = SMALL ? 1 : 2;            // 32-row query blocks per wave
  static constexpr int NW = SMALL ? 4 : 8;            // waves per workgroup
  static constexpr int NSTAGE = SMALL ? 3 : 4;        // K/V tiles in the LDS ring
  static constexpr int WG_PER_CU = SMALL ? 3 : 1;
  static constexpr int BM = 32 * RW * NW;             // query rows per workgroup
  static constexpr int NT = 64 * NW;                  // threads per workgroup
  static constexpr int QB_PER_WG = BM / kQueryBlock;  // query blocks per workgroup
  static_assert(BM % kQueryBlock == 0 && kKeyBlock % BN == 0, "mask blocks");
  static_assert(QB_PER_WG <= 16, "query-block flags");
};
// Longest sequence of the block-sparse variant (its key-block list lives in
// LDS, 4 bytes per key block, and entries hold the key block in 16 bits).
constexpr int kSparseMaxSeq = 1 << 20;

// Rescale the output accumulator only when the running row max grows by more
// than 2^48 in the exp2 domain.  Until then P may exceed 1 by up to 2^48;
// fp32 and bf16 carry such values with the same relative precision as values
// below 1.  The sums stay finite while S * 2^48 * max|V| < 2^128, i.e.
// max|V| < 2^60 at 2^20 keys.  (Rows of outlier tokens, whose scores spread
// over tens of units in the exp2 domain, move their max by more than 2^24
// now and then; at that threshold the slow path cost 2.4 % at 16896 tokens.)
constexpr float kRescaleLog2 = 48.f;

// LDS fragment reads in flight ahead of the MFMA that consumes them.
constexpr int kPrefetch = 4;

// Buffer-resource word 3 for raw (unswizzled, unformatted 32-bit) buffer
// access on gfx950: reads outside [0, num_records) return zeros (the check
// covers the scalar offset too).
constexpr int kBufferFlags = 0x00020000;

#define JA_INLINE __attribute__((always_inline))

struct FwdArgs {
  const bf16 *q;
  const float *qn;          // Q RMS-norm weights [D], NULL = none
  float eps;
  const bf16 *kr, *vt;      // prepared K and V^T (prep_kv.hip), S_pad keys
  const double2 *rope;      // RoPE table [S][D/2] (cos, sin) in fp64
  // the coordinate table of the same positions, [kCoordTableN][D/4] (cos,
  // sin), and the positions [S][2] (both NULL = per-token table only)
  const double2 *ctab;
  const int32_t *pos;
  bf16 *o;
  float *lse;
  int64_t q_sb, q_ss, q_sh, o_sb, o_ss, o_sh;
  int S, S_pad, H, B, n_qblk;
  float scale_log2;
  // Split of the last, partial round of workgroups over key ranges: the
  // first n_direct workgroups each own one (q-block, head, batch) item; the
  // remaining ones are `parts` workgroups per item, each over a contiguous
  // range of key tiles, writing unnormalised partial results to `ws`.
  int n_direct, parts;
  int qgroup;               // work-item order (item_coords)
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

// LDS ring: NSTAGE stages of [K tile | V^T tile].  The K tile is stored in
// the order in which the Q K^T fragment reads consume it: for each 16-column
// block kk of the head dimension, 1 KB holding, at position 16 lane, the
// 8 bf16 that `lane` reads (key lane % 32, columns 16 kk + 8 (lane / 32) ..
// + 7).  A fragment read is then one 1 KB block read contiguously by the
// wave's lanes (conflict-free, immediate offsets), and the tile is whole
// 1 KB loads without padding.  A V^T row is the 32 keys of one
// head-dimension column, 64 bytes, granule g stored at g ^ vswz.
// Granule position of V^T row d's granule g is g ^ vswz(d): the 16 rows read
// together by a fragment read then cover all 16 bank groups of 16 bytes.
__host__ __device__ constexpr int vswz(int d) { return (d / 4) % 4; }

template <int D, int NSTAGE>
struct Lds {
  static constexpr int CH = D / 8;                    // 16-byte chunks per K row
  static constexpr int K_LOADS = D / 16;              // K part: one 1 KB block per kk
  static constexpr int V_LOADS = D * (BN / 8) / 64;   // V^T part: 4 granules per row
  static constexpr int LOADS = K_LOADS + V_LOADS;     // 1 KB loads per tile
  static constexpr int KBYTES = K_LOADS * 1024;
  static constexpr int STAGE = LOADS * 1024;
  static constexpr int BYTES = NSTAGE * STAGE;
  // block-sparse variant: per-wave counts, then the key-block list
  static constexpr int LIST_OFFSET = BYTES + 64;
  static constexpr int sparse_bytes(int nkb) { return LIST_OFFSET + 4 * nkb; }
};


template <int D, bool ROPE, bool SPARSE, bool SMALL>
__global__ __launch_bounds__(Cfg<SMALL>::NT, Cfg<SMALL>::WG_PER_CU)
void attn_fwd_bf16_kernel(FwdArgs a) {
  static_assert(SMALL || !SPARSE, "the block-sparse variant has the small shape");
  constexpr int RW = Cfg<SMALL>::RW, NW = Cfg<SMALL>::NW, NT = Cfg<SMALL>::NT,
                BM = Cfg<SMALL>::BM;
  constexpr int NSTAGE = Cfg<SMALL>::NSTAGE, QB_PER_WG = Cfg<SMALL>::QB_PER_WG;
  using L = Lds<D, NSTAGE>;
  constexpr int LOADS = L::LOADS, K_LOADS = L::K_LOADS;
  constexpr int JW = (LOADS + NW - 1) / NW;           // tile loads per wave, at most
  static_assert(JW <= 5, "at most five tile loads per wave");
  extern __shared__ __attribute__((aligned(16))) bf16 smem[];
  auto Kst = [&](int st) JA_INLINE { return smem + st * (L::STAGE / 2); };
  auto Vst = [&](int st) JA_INLINE {
    return smem + st * (L::STAGE / 2) + L::KBYTES / 2;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  int qblk, bh;
  item_coords(item, a.n_qblk, a.B * a.H, a.qgroup, bh, qblk);
  const int h = bh % a.H, b = bh / a.H;

  // ---- block-sparse variant: compact the key blocks kept by any of this
  //      workgroup's query blocks into an LDS list (ascending), entry =
  //      key block | (flags of the query blocks that keep it) << 16.  The
  //      workgroup's key tiles are then the tiles of the listed blocks that
  //      lie inside the sequence; the dense kernel's tiles are 0..ntiles-1. ----
  uint32_t *blist = reinterpret_cast<uint32_t *>(reinterpret_cast<char *>(smem) + L::LIST_OFFSET);
  int ntiles = ntiles_all;
  if constexpr (SPARSE) {
    int *wcnt = reinterpret_cast<int *>(reinterpret_cast<char *>(smem) + L::BYTES);
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

  // ---- Q rows of this lane (one per 32-row block): normalize (optional),
  //      rotate, round to bf16, keep in registers ----
  int qi[RW];
  bf16x8 qreg[RW][D / 16];
#pragma unroll
  for (int r = 0; r < RW; ++r) {
    qi[r] = qblk * BM + (wave * RW + r) * 32 + l32;
    const int qs = qi[r] < S ? qi[r] : S - 1;
    const bf16 *qrow = a.q + b * a.q_sb + (int64_t)qs * a.q_ss + h * a.q_sh;
    // lane half hf holds chunks c = 2 kk + hf of the row
    constexpr int NK = D / 16;
    u32x4 w[NK];
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) w[kk] = *reinterpret_cast<const u32x4 *>(qrow + 16 * kk + 8 * hf);
    // RMS norm scale (fp64: the lane half holds half the row's chunks)
    double rn = 0.0;
    if (a.qn) {
      double ss = 0.0;
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) ss += chunk_sumsq_f64(w[kk]);
      rn = rms_scale_f64<D>(ss + __shfl_xor(ss, 32), a.eps);
    }
    // (cos, sin) of the row's pairs: pairs below D/4 turn by the token's
    // grid row, the others by its column.  When every lane of the wave has
    // both coordinates inside the coordinate table, read them there (the
    // same values bit for bit; a 512-row block of an image spans a few grid
    // rows, so most of its reads hit lines another row already brought into
    // the vector L1), else from the token's row of the per-token table.
    const double2 *row_cs = nullptr, *col_cs = nullptr;
    if (ROPE) {
      row_cs = a.rope + (int64_t)qs * (D / 2);
      col_cs = row_cs + D / 4;
      if (a.ctab) {
        const int32_t pr = a.pos[2 * (int64_t)qs], pc = a.pos[2 * (int64_t)qs + 1];
        const bool inside = (uint32_t)pr < (uint32_t)kCoordTableN &&
                            (uint32_t)pc < (uint32_t)kCoordTableN;
        if (__builtin_amdgcn_ballot_w64(!inside) == 0) {
          row_cs = a.ctab + pr * (D / 4);
          col_cs = a.ctab + pc * (D / 4);
        }
      }
    }
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      const int d0 = 16 * kk + 8 * hf;
      u32x4 x = w[kk];
      if (ROPE || a.qn)
        x = prologue_chunk_bf16(x, rn, a.qn ? a.qn + d0 : nullptr,
                                !ROPE ? nullptr
                                : kk < D / 32 ? row_cs + d0 / 2 : col_cs + (d0 / 2 - D / 4));
      if (qi[r] >= S) x = u32x4{0, 0, 0, 0};
      qreg[r][kk] = bit_cast<bf16x8>(x);
    }
  }

  // ---- tile loads: load j (0 <= j < LOADS) of a tile fills LDS bytes
  //      [j KB, (j+1) KB) of its stage, lane i the 16 bytes at 16 i.  Loads
  //      below K_LOADS carry the K tile's column block kk = j: lane i the
  //      chunk 2 j + i / 32 of key i % 32.  The others carry V^T rows, 16
  //      per load: row
  //      d = 16 (j - K_LOADS) + i / 4, position i % 4 holding granule
  //      (i % 4) ^ vswz(d) of the row.  Wave w issues loads w, w + NW, ...
  //      The lane offsets are fixed (scalars: an array element as the
  //      builtin's offset operand makes the host compilation drop the
  //      kernel's launch stub); the tile offset is scalar. ----
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16 *>(a.kr + (int64_t)bh * a.S_pad * D), 0, a.S_pad * D * 2, kBufferFlags);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16 *>(a.vt + (int64_t)bh * D * a.S_pad), 0, a.S_pad * D * 2, kBufferFlags);
  auto load_offset = [&](int j) JA_INLINE -> int {
    if (j < K_LOADS) return ((lane % 32) * D + 8 * (2 * j + lane / 32)) * 2;
    const int d = 16 * (j - K_LOADS) + lane / 4;
    return (d * BN + 8 * ((lane % 4) ^ vswz(d))) * 2;
  };
  auto voff_of = [&](int m) JA_INLINE -> int {
    return wave + m * NW < LOADS ? load_offset(wave + m * NW) : 0;
  };
  const int voff0 = voff_of(0), voff1 = voff_of(1), voff2 = voff_of(2), voff3 = voff_of(3),
            voff4 = voff_of(4);
  const int nl = (LOADS - wave + NW - 1) / NW;         // loads of this wave per tile
  auto issue_one = [&](int j, int voff, int t, int st) JA_INLINE {
    char *dst = reinterpret_cast<char *>(smem) + st * L::STAGE + j * 1024;
    if (j < K_LOADS)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, JA_LDS_PTR(dst), 16, voff, t * (BN * D * 2), 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, JA_LDS_PTR(dst), 16, voff, t * (BN * D * 2), 0, 0);
  };
  // loads of key tile t into stage st
  auto issue = [&](int t, int st) JA_INLINE {
    if (0 < nl) issue_one(wave, voff0, t, st);
    if (JW > 1 && 1 < nl) issue_one(wave + NW, voff1, t, st);
    if (JW > 2 && 2 < nl) issue_one(wave + 2 * NW, voff2, t, st);
    if (JW > 3 && 3 < nl) issue_one(wave + 3 * NW, voff3, t, st);
    if (JW > 4 && 4 < nl) issue_one(wave + 4 * NW, voff4, t, st);
  };
  // wait until at most `ahead` later tiles' loads of this wave are in flight
  auto wait_tiles = [&]<int AHEAD>() JA_INLINE {
    if (JW > 4 && nl == 5)
      wait_vmcnt<5 * AHEAD>();
    else if (JW > 3 && nl == 4)
      wait_vmcnt<4 * AHEAD>();
    else if (JW > 2 && nl == 3)
      wait_vmcnt<3 * AHEAD>();
    else if (JW > 1 && nl == 2)
      wait_vmcnt<2 * AHEAD>();
    else
      wait_vmcnt<AHEAD>();
  };

  // ---- S^T = K . Q^T for this wave's 32 queries and the 32 keys of a tile.
  //      The K fragments are read kPrefetch steps ahead of their MFMA (left
  //      to itself the compiler reuses one register and every MFMA waits a
  //      full LDS latency); the scheduling barriers keep that order. ----
  auto qk = [&]<int KK0, int KK1>(int buf, f32x16 (&sacc)[RW]) JA_INLINE {
    if constexpr (KK0 == 0) {
#pragma unroll
      for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[r][i] = 0.f;
    }
    const bf16 *krow = Kst(buf) + 8 * lane;
    bf16x8 kf[kPrefetch];
#pragma unroll
    for (int j = 0; j < kPrefetch && KK0 + j < KK1; ++j)
      kf[j] = *reinterpret_cast<const bf16x8 *>(krow + 512 * (KK0 + j));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = KK0; kk < KK1; ++kk) {
#pragma unroll
      for (int r = 0; r < RW; ++r)
        sacc[r] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[(kk - KK0) % kPrefetch], qreg[r][kk],
                                                          sacc[r], 0, 0, 0);
      if (kk + kPrefetch < KK1)
        kf[(kk - KK0) % kPrefetch] = *reinterpret_cast<const bf16x8 *>(krow + 512 * (kk + kPrefetch));
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- O^T += V^T . P^T ; P operand slot j of half hf (key group g) is key
  //      16g + 4hf + (j<4 ? j : j+4), which V^T stores in logical granule
  //      2g + hf of its row.  Step st covers head-dimension block st/2 and key
  //      group st%2; its V^T fragment is read kPrefetch steps ahead, as in
  //      Q K^T.  Row l32 of every 32-row block has the same swizzle, so the
  //      two granules of a lane sit at two fixed offsets. ----
  f32x16 oacc[RW][D / 32];
#pragma unroll
  for (int r = 0; r < RW; ++r)
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[r][db][i] = 0.f;
  auto pv = [&](const bf16x8 (&pb)[RW][2], int buf) JA_INLINE {
    const int vy = hf ^ vswz(l32);
    const bf16 *vt0 = Vst(buf) + l32 * BN + 8 * vy;          // key group 0
    const bf16 *vt1 = Vst(buf) + l32 * BN + 8 * (vy ^ 2);    // key group 1
    constexpr int NV = 2 * (D / 32);
    auto vaddr = [&](int st) JA_INLINE { return (st % 2 ? vt1 : vt0) + 32 * BN * (st / 2); };
    bf16x8 vf[kPrefetch];
#pragma unroll
    for (int j = 0; j < kPrefetch && j < NV; ++j) vf[j] = *reinterpret_cast<const bf16x8 *>(vaddr(j));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int st = 0; st < NV; ++st) {
#pragma unroll
      for (int r = 0; r < RW; ++r)
        oacc[r][st / 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[st % kPrefetch], pb[r][st % 2],
                                                                  oacc[r][st / 2], 0, 0, 0);
      if (st + kPrefetch < NV) vf[st % kPrefetch] = *reinterpret_cast<const bf16x8 *>(vaddr(st + kPrefetch));
      __builtin_amdgcn_sched_barrier(0);
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
  //      8*(i/4) + 4*hf + i%4).  The tile's row maxima come first; P is then
  //      computed against the running max m_run, which is exact and bounded
  //      by 2^48 unless some row's tile max exceeds m_run by the threshold
  //      (rare after the first tile).  Only then are O and l rescaled and
  //      m_run moved to the new max, before P is computed.  Taking the max
  //      first keeps S alone alive up to the decision, not S and a
  //      speculative P. ----
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
    float mx[RW];
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
    }
    if (__builtin_amdgcn_ballot_w64(any)) {
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
      }
    }
#pragma unroll
    for (int r = 0; r < RW; ++r) l_run[r] += exp_tile(sacc[r], m_run[r], pb[r]);
  };

  // ---- loop over the workgroup's tiles (local index i, list position
  //      t0 + i).  Tile i lives in stage i % NSTAGE.  Iteration i first issues
  //      the loads of tile i + NSTAGE - 1 into the stage that iteration i - 1
  //      read, then computes Q K^T, the softmax and P.V of tile i; before the
  //      barrier that closes it, each wave waits for its own loads of tile
  //      i + 1 only. ----
  const int nt = t1 - t0;
  // a dense workgroup always has at least one tile; a sparse one may have none
  const bool any_tile = !SPARSE || nt > 0;
  if (any_tile) {
#pragma unroll
    for (int p = 0; p < NSTAGE - 1; ++p)
      if (p < nt) issue(tile_of(t0 + p), p);
    wait_vmcnt<0>();
    tile_barrier();
  }
  f32x16 sacc[RW];
  // NEXT: tile i+1 exists.  Only the last tile of the sequence can be partial
  // (masking a full tile changes nothing), and it is always the last of the
  // workgroup's tiles.
  auto iteration = [&]<bool NEXT>(int i) JA_INLINE {
    const int x = t0 + i;
    const bool ahead = i + NSTAGE - 1 < nt;
    if (ahead) issue(tile_of(x + NSTAGE - 1), (i + NSTAGE - 1) % NSTAGE);
    if (kept(x)) {
      const int t = tile_of(x);
      qk.template operator()<0, D / 16>(i % NSTAGE, sacc);
      bf16x8 pb[RW][2];
      softmax.template operator()<!NEXT>(sacc, t * BN, pb);
      pv(pb, i % NSTAGE);
    }
    if constexpr (NEXT) {
      if (ahead)
        wait_tiles.template operator()<NSTAGE - 2>();
      else
        wait_vmcnt<0>();
      tile_barrier();
    }
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

// Dynamic LDS of one instantiation; its limit is raised once per device (the
// attribute is set with the device current).
template <int D, bool ROPE, bool SPARSE, bool SMALL>
hipError_t launch_instance(const FwdArgs &a, dim3 grid, hipStream_t st) {
  using L = Lds<D, Cfg<SMALL>::NSTAGE>;
  const int bytes = SPARSE ? L::sparse_bytes(a.nkb) : L::BYTES;
  constexpr int kMaxDevices = 64;
  static std::atomic<bool> done[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices || !done[dev].load(std::memory_order_acquire)) {
    e = hipFuncSetAttribute(
        reinterpret_cast<const void *>(&attn_fwd_bf16_kernel<D, ROPE, SPARSE, SMALL>),
        hipFuncAttributeMaxDynamicSharedMemorySize,
        SPARSE ? L::sparse_bytes((kSparseMaxSeq + kKeyBlock - 1) / kKeyBlock) : L::BYTES);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < kMaxDevices) done[dev].store(true, std::memory_order_release);
  }
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, ROPE, SPARSE, SMALL>), grid, dim3(Cfg<SMALL>::NT),
                     bytes, st, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_dim(const FwdArgs &a, dim3 grid, bool rope_on, bool small, hipStream_t st) {
  if (a.mask)
    return rope_on ? launch_instance<D, true, true, true>(a, grid, st)
                   : launch_instance<D, false, true, true>(a, grid, st);
  if (small)
    return rope_on ? launch_instance<D, true, false, true>(a, grid, st)
                   : launch_instance<D, false, false, true>(a, grid, st);
  return rope_on ? launch_instance<D, true, false, false>(a, grid, st)
                 : launch_instance<D, false, false, false>(a, grid, st);
}

}  // namespace

int fwd_bf16_block_rows(bool small) { return small ? Cfg<true>::BM : Cfg<false>::BM; }

SplitPlan plan_fwd_bf16(const AttnLayout &L, int n_cu, bool sparse) {
  // The dense forward takes the small shape when the wide items would leave
  // at least half of the CUs idle.  (Between half and one round the wide
  // shape stays ahead: at 16896 tokens and 6 heads, 198 wide items, it is
  // 5 % faster than 792 small ones; at 3 heads the small shape is 30 %
  // faster.)
  const int64_t wide_items = (int64_t)((L.S + Cfg<false>::BM - 1) / Cfg<false>::BM) * L.H * L.B;
  const bool small = sparse || 2 * wide_items <= n_cu;
  const int bm = fwd_bf16_block_rows(small);
  const int wg = small ? Cfg<true>::WG_PER_CU : Cfg<false>::WG_PER_CU;
  const int n_items = ((L.S + bm - 1) / bm) * L.H * L.B;
  SplitPlan p = plan_split(n_items, (L.S + BN - 1) / BN, n_cu * wg, bm, L.D);
  p.small = small;
  // dense: the query blocks of a head run together on the CUs of one XCD
  p.qgroup = sparse ? 0 : (n_cu >= 8 ? n_cu / 8 * wg : 1);
  return p;
}

int fwd_bf16_sparse_max_seq() { return kSparseMaxSeq; }

hipError_t launch_fwd_bf16(const AttnLayout &L, const void *q, const void *kv,
                           const double *rope, const double *ctab, const int32_t *pos,
                           const uint8_t *mask, void *o, float *lse, const SplitPlan &plan,
                           void *workspace, hipStream_t st) {
  // kv: prepared K | prepared V^T (prep_kv.hip)
  const int64_t prep_elems = (int64_t)L.B * L.H * prep_pad(L.S) * L.D;
  const bf16 *kr = static_cast<const bf16 *>(kv);
  const bf16 *vt = kr + prep_elems;
  FwdArgs a;
  a.q = static_cast<const bf16 *>(q);
  a.qn = L.q_norm;
  a.eps = L.norm_eps;
  a.kr = kr;
  a.vt = vt;
  a.rope = reinterpret_cast<const double2 *>(rope);
  a.ctab = rope && pos ? reinterpret_cast<const double2 *>(ctab) : nullptr;
  a.pos = a.ctab ? pos : nullptr;
  a.o = static_cast<bf16 *>(o);
  a.lse = lse;
  a.q_sb = L.q_sb; a.q_ss = L.q_ss; a.q_sh = L.q_sh;
  a.o_sb = L.o_sb; a.o_ss = L.o_ss; a.o_sh = L.o_sh;
  a.S = L.S;
  a.S_pad = prep_pad(L.S);
  a.H = L.H;
  a.B = L.B;
  const bool small = mask != nullptr || plan.small;
  const int bm = fwd_bf16_block_rows(small);
  a.n_qblk = (L.S + bm - 1) / bm;
  a.scale_log2 = L.scale_log2;
  a.n_direct = plan.n_direct;
  a.parts = plan.parts;
  a.qgroup = plan.qgroup;
  a.ws = split_workspace(plan, workspace, bm, L.D);
  a.mask = mask;
  a.nqb = (L.S + kQueryBlock - 1) / kQueryBlock;
  a.nkb = (L.S + kKeyBlock - 1) / kKeyBlock;
  const dim3 grid((unsigned)(plan.n_direct + plan.n_units));
  const hipError_t e = L.D == 64 ? launch_dim<64>(a, grid, rope != nullptr, small, st)
                                 : launch_dim<128>(a, grid, rope != nullptr, small, st);
  if (e != hipSuccess || plan.n_units == 0) return e;
  return launch_merge_split(L, plan, a.ws, bm, L.scale_log2, o, lse, st);
}

}  // namespace ja
