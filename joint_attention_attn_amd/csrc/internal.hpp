// Host-side launch interface between the C ABI (api.cpp) and the kernels.
// Arguments here are already validated.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ja {

struct AttnLayout {
  int32_t B, S, H, D;
  int64_t q_sb, q_ss, q_sh;
  int64_t k_sb, k_ss, k_sh;
  int64_t v_sb, v_ss, v_sh;
  int64_t o_sb, o_ss, o_sh;
  float scale_log2;  // softmax scale * log2(e): scores live in the exp2 domain
  // query/key RMS normalization weights [D] (NULL = none) and its epsilon
  const float *q_norm = nullptr, *k_norm = nullptr;
  float norm_eps = 1e-6f;
};

// RoPE table: (cos, sin) in fp64 per (token, pair), [S][D/2][2] doubles.
// ctab (NULL = not built): the coordinate table, (cos, sin) of c * w_k for
// every grid coordinate c < kCoordTableN and k < D/4, [kCoordTableN][D/4][2]
// doubles.  A token's entry for pair p < D/4 equals ctab[row][p], for
// p >= D/4 ctab[col][p - D/4], bit for bit (the same product and sincos).
constexpr int kCoordTableN = 1024;
inline int64_t coord_table_bytes(int D) { return (int64_t)kCoordTableN * (D / 4) * 16; }
hipError_t launch_rope_table_2d(const int32_t *pos, int S, int D, float theta,
                                double *table, double *ctab, hipStream_t st);

// Split of the last partial round of workgroups over key ranges.  A forward
// launch has n_items (query block, head, batch row) work items for `slots`
// co-resident workgroups.  When the last round would leave more than half of
// the slots idle, its items are cut into `parts` key ranges each; those
// workgroups write unnormalised partial results that a merge pass combines.
struct SplitPlan {
  int n_direct = 0;     // items computed by one workgroup each
  int parts = 1;        // key ranges per split item
  int n_units = 0;      // workgroups over key ranges (split items x parts)
  int64_t ws_bytes = 0; // workspace the split needs
  int qgroup = 0;       // work-item order, see item_coords
  bool small = false;   // bf16 dense forward: the 128-row workgroup shape
};

// (batch x head, query block) of work item `item`.  qgroup = 0: head-major.
// qgroup = G > 0: the first floor(n_qblk / G) * G query blocks of every
// head, head-major, then the remaining blocks of every head.  With G the
// CUs of one XCD and the forward's XCD-aware placement, a round of an XCD's
// workgroups then covers G blocks of one head, which stream the same K/V
// through that XCD's L2 together, and the leftover blocks gather in the
// last round (the one the split cuts into key ranges).
__host__ __device__ inline void item_coords(int item, int n_qblk, int n_bh, int qgroup, int &bh,
                                            int &qblk) {
  const int full_blocks = qgroup > 0 ? n_qblk / qgroup * qgroup : 0;
  const int full_items = n_bh * full_blocks;
  if (item < full_items) {
    bh = item / full_blocks;
    qblk = item % full_blocks;
  } else {
    const int j = item - full_items, rest = n_qblk - full_blocks;
    bh = j / rest;
    qblk = full_blocks + j % rest;
  }
}
// Partial results of the split workgroups: O rows [n_units][block_rows][D]
// (fp32, unnormalised) and (row max, row sum) [n_units][block_rows][2]; the
// row max times the merge's m_scale is in the exp2 domain.
struct SplitWorkspace {
  float *o = nullptr;
  float *ml = nullptr;
};
SplitPlan plan_split(int n_items, int ntiles, int slots, int block_rows, int D);
SplitWorkspace split_workspace(const SplitPlan &plan, void *ws, int block_rows, int D);
hipError_t launch_merge_split(const AttnLayout &L, const SplitPlan &plan,
                              const SplitWorkspace &ws, int block_rows, float m_scale,
                              void *o, float *lse, hipStream_t st);

// K/V preparation of the BF16 forward (prep_kv.hip): one buffer of
// prep_kv_bytes(L) holding rotated K [B*H][S_pad][D], then V^T [B*H][D][S_pad],
// S_pad = prep_pad(S).
int prep_pad(int S);
int64_t prep_kv_bytes(const AttnLayout &L);
hipError_t launch_prep_kv_bf16(const AttnLayout &L, const void *k, const void *v,
                               const double *rope, void *kv, hipStream_t st);

SplitPlan plan_fwd_bf16(const AttnLayout &L, int n_cu, bool sparse);
// kv: the prepared K/V buffer; rope: the RoPE table (NULL = no RoPE); ctab,
// pos: the coordinate table of the same positions and the positions (both
// NULL when the table came without them); mask: NULL = dense, else the block
// mask of the block-sparse variant, uint8 [B][H][ceil(S/128)][ceil(S/64)]
// (nonzero = keep).  workspace: the split's partial results (plan.ws_bytes).
hipError_t launch_fwd_bf16(const AttnLayout &L, const void *q, const void *kv,
                           const double *rope, const double *ctab, const int32_t *pos,
                           const uint8_t *mask, void *o, float *lse, const SplitPlan &plan,
                           void *workspace, hipStream_t st);
int fwd_bf16_sparse_max_seq();   // longest sequence of the block-sparse variant

hipError_t launch_quant_rope_fp8(const AttnLayout &L, const void *q,
                                 const void *k, const void *v,
                                 const double *rope, void *q8, void *k8,
                                 void *v8, float *sq, float *sk, float *sv,
                                 hipStream_t st);

// Repaired keys of the FP8 forward (see repair_fp8.hip); n_rep = 0: none.
// Their bias reaches the forward through the K/V preparation.
struct Fp8Repair {
  int n_rep = 0;
  const void *kr = nullptr, *vr = nullptr;
};
int repair_pad(int n);          // repaired keys rounded up to whole 32-key tiles
int repair_max_seq();           // longest sequence the selection handles
hipError_t launch_repair_plan(const AttnLayout &L, const void *k, const void *v,
                              const double *rope, const void *k8, const void *v8,
                              const float *sk, const float *sv, int n, int32_t *idx,
                              void *kr, void *vr, float *kbias, hipStream_t st);

// K/V preparation of the FP8 forward (prep_kv_fp8.hip): one buffer of
// prep_kv_fp8_bytes(L) holding K [B*H][S_pad][D], V^T [B*H][D][S_pad] and the
// per-key values [B*H][S_pad/64][1 KB], S_pad = prep8_pad(S); kbias: the
// repair bias, NULL = none.
int prep8_pad(int S);
int64_t prep_kv_fp8_bytes(const AttnLayout &L);
hipError_t launch_prep_kv_fp8(const AttnLayout &L, const void *k8, const void *v8,
                              const float *sk, const float *sv, const float *kbias, void *kv8,
                              hipStream_t st);

SplitPlan plan_fwd_fp8(const AttnLayout &L, int n_cu, bool sparse);
// mask: NULL = dense, else the block mask of the block-sparse variant (no
// repair then), uint8 [B][H][ceil(S/128)][ceil(S/64)].
hipError_t launch_fwd_fp8(const AttnLayout &L, const void *q8, const float *sq, const void *kv8,
                          const uint8_t *mask, void *o, float *lse, const SplitPlan &plan,
                          void *workspace, const Fp8Repair &repair, hipStream_t st);
int fwd_fp8_sparse_max_seq();    // longest sequence of the block-sparse variant

// Query rows per workgroup of each forward kernel (the grid's x extent is
// ceil(S / rows)).
int fwd_bf16_block_rows(bool small);
int fwd_fp8_block_rows(bool sparse);

}  // namespace ja
