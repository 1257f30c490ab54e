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
};

hipError_t launch_rope_table_2d(const int32_t *pos, int S, int D, float theta,
                                float *table, hipStream_t st);

hipError_t launch_fwd_bf16(const AttnLayout &L, const void *q, const void *k,
                           const void *v, const float *rope, void *o,
                           float *lse, hipStream_t st);

hipError_t launch_quant_rope_fp8(const AttnLayout &L, const void *q,
                                 const void *k, const void *v,
                                 const float *rope, void *q8, void *k8,
                                 void *v8, float *sq, float *sk, float *sv,
                                 hipStream_t st);

hipError_t launch_fwd_fp8(const AttnLayout &L, const void *q8, const void *k8,
                          const void *v8, const float *sq, const float *sk,
                          const float *sv, void *o, float *lse, hipStream_t st);

// Query rows per workgroup of each forward kernel (the grid's x extent is
// ceil(S / rows)).
int fwd_bf16_block_rows(int D);
int fwd_fp8_block_rows(int D);

}  // namespace ja
