// C ABI of libjoint_attn.so: argument validation, status codes and launch.
// Every check runs on the host before anything is enqueued, so an invalid
// call never touches the device.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "../../include/joint_attn.h"
#include "internal.hpp"

namespace {

thread_local char g_last_error[256] = "";

ja_status hip_status(hipError_t e) {
  if (e == hipSuccess) return JA_OK;
  std::snprintf(g_last_error, sizeof g_last_error, "%s: %s", hipGetErrorName(e),
                hipGetErrorString(e));
  return JA_ERR_HIP;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool shape_ok(const ja_params *p) {
  return p->batch >= 1 && p->seq_len >= 1 && p->heads >= 1;
}

bool dim_supported(int d) { return d == 64 || d == 128; }

// Strides of a bf16 tensor: multiples of 8 elements (16-byte vector access)
// and non-negative.
bool strides_ok(int64_t sb, int64_t ss, int64_t sh) {
  return sb >= 0 && ss >= 0 && sh >= 0 && sb % 8 == 0 && ss % 8 == 0 && sh % 8 == 0;
}

// Grid limits: the forward kernels launch one workgroup per
// (query block, head, batch row) on a 1-D grid indexed with 32-bit ints.
bool grid_ok(const ja_params *p, int block_rows) {
  const int64_t nx = ((int64_t)p->seq_len + block_rows - 1) / block_rows;
  return nx * p->heads * p->batch <= 0x7fffffffLL && p->heads <= 65535 &&
         p->batch <= 65535;
}

ja::AttnLayout layout(const ja_params *p) {
  ja::AttnLayout L;
  L.B = p->batch; L.S = p->seq_len; L.H = p->heads; L.D = p->head_dim;
  L.q_sb = p->q_sb; L.q_ss = p->q_ss; L.q_sh = p->q_sh;
  L.k_sb = p->k_sb; L.k_ss = p->k_ss; L.k_sh = p->k_sh;
  L.v_sb = p->v_sb; L.v_ss = p->v_ss; L.v_sh = p->v_sh;
  L.o_sb = p->o_sb; L.o_ss = p->o_ss; L.o_sh = p->o_sh;
  const float scale = p->softmax_scale != 0.f ? p->softmax_scale
                                              : 1.f / std::sqrt((float)p->head_dim);
  L.scale_log2 = scale * 1.4426950408889634f;
  L.q_norm = p->q_norm;
  L.k_norm = p->k_norm;
  L.norm_eps = p->norm_eps != 0.f ? p->norm_eps : 1e-6f;
  return L;
}

// Common checks of the Q/K/V/O description.  `qkv_strided` is false for the
// FP8 forward, whose inputs are contiguous by contract.
ja_status check_params(const ja_params *p, bool qkv_strided, int block_rows) {
  if (!p) return JA_ERR_INVALID_ARG;
  if (!shape_ok(p)) return JA_ERR_INVALID_ARG;
  if (!dim_supported(p->head_dim)) return JA_ERR_UNSUPPORTED;
  if (!std::isfinite(p->softmax_scale) || p->softmax_scale < 0.f) return JA_ERR_INVALID_ARG;
  if (!std::isfinite(p->norm_eps) || p->norm_eps < 0.f) return JA_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(p->q_norm) & 15u) || (reinterpret_cast<uintptr_t>(p->k_norm) & 15u))
    return JA_ERR_INVALID_ARG;
  if (qkv_strided &&
      (!strides_ok(p->q_sb, p->q_ss, p->q_sh) || !strides_ok(p->k_sb, p->k_ss, p->k_sh) ||
       !strides_ok(p->v_sb, p->v_ss, p->v_sh)))
    return JA_ERR_INVALID_ARG;
  if (block_rows > 0) {
    if (!strides_ok(p->o_sb, p->o_ss, p->o_sh)) return JA_ERR_INVALID_ARG;
    if (!grid_ok(p, block_rows)) return JA_ERR_UNSUPPORTED;
  }
  return JA_OK;
}

// Compute units of the current device (cached per device id).
int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev < 0 || dev >= 64) {
    int n = 0;
    return hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess ? n : 0;
  }
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Checks of joint_attn_fwd_bf16 that do not involve device pointers.
ja_status check_fwd_bf16(const ja_params *p) {
  // the block-sparse forward has the smaller workgroups, hence the larger grid
  const ja_status st = check_params(p, true, ja::fwd_bf16_block_rows(true));
  if (st != JA_OK) return st;
  // the prepared K and V^T of one (batch, head) are addressed with 32-bit
  // byte offsets; the preparation pass has one workgroup per 64 keys and head
  const int64_t s_pad = ((int64_t)p->seq_len + 63) / 64 * 64;
  if (s_pad * p->head_dim * 2 > 0x7fffffffLL ||
      s_pad / 64 * p->batch * p->heads > 0x7fffffffLL)
    return JA_ERR_UNSUPPORTED;
  return JA_OK;
}

// Checks of joint_attn_fwd_fp8 that do not involve device pointers.
ja_status check_fwd_fp8(const ja_params *p) {
  const ja_status st = check_params(p, false, ja::fwd_fp8_block_rows(p ? p->head_dim : 0));
  if (st != JA_OK) return st;
  // the prepared K and V^T of one (batch, head) are addressed with 32-bit
  // byte offsets; the preparation pass has one workgroup per 64 keys and head
  const int64_t s_pad = ((int64_t)p->seq_len + 63) / 64 * 64;
  if (s_pad * p->head_dim > 0x7fffffffLL || s_pad / 64 * p->batch * p->heads > 0x7fffffffLL)
    return JA_ERR_UNSUPPORTED;
  return JA_OK;
}

}  // namespace

extern "C" {

const char *joint_attn_status_string(ja_status s) {
  switch (s) {
    case JA_OK: return "JA_OK";
    case JA_ERR_INVALID_ARG: return "JA_ERR_INVALID_ARG: invalid argument";
    case JA_ERR_UNSUPPORTED: return "JA_ERR_UNSUPPORTED: unsupported shape";
    case JA_ERR_HIP: return "JA_ERR_HIP: HIP runtime error";
  }
  return "unknown ja_status";
}

const char *joint_attn_last_error(void) { return g_last_error; }

ja_status joint_attn_rope_table_2d(const int32_t *pos, int32_t seq_len,
                                   int32_t head_dim, float theta, float *table,
                                   void *stream) {
  if (!pos || !table || seq_len < 1) return JA_ERR_INVALID_ARG;
  if (!(theta > 0.f) || !std::isfinite(theta)) return JA_ERR_INVALID_ARG;
  if (!dim_supported(head_dim)) return JA_ERR_UNSUPPORTED;
  if (!aligned16(table) || (reinterpret_cast<uintptr_t>(pos) & 3u)) return JA_ERR_INVALID_ARG;
  if ((int64_t)seq_len * (head_dim / 2) > 0x7fffffffLL * 256) return JA_ERR_UNSUPPORTED;
  return hip_status(ja::launch_rope_table_2d(pos, seq_len, head_dim, theta, table,
                                             static_cast<hipStream_t>(stream)));
}

size_t joint_attn_prep_kv_bf16_bytes(const ja_params *p) {
  if (!p || check_fwd_bf16(p) != JA_OK) return 0;
  return (size_t)ja::prep_kv_bytes(layout(p));
}

ja_status joint_attn_prep_kv_bf16(const ja_params *p, const void *k, const void *v,
                                  const float *rope, void *kv, size_t kv_bytes, void *stream) {
  if (!p || !k || !v || !kv) return JA_ERR_INVALID_ARG;
  const ja_status st = check_fwd_bf16(p);
  if (st != JA_OK) return st;
  if (!aligned16(k) || !aligned16(v) || !aligned16(kv) || (rope && !aligned16(rope)))
    return JA_ERR_INVALID_ARG;
  const ja::AttnLayout L = layout(p);
  if (kv_bytes < (size_t)ja::prep_kv_bytes(L)) return JA_ERR_INVALID_ARG;
  return hip_status(ja::launch_prep_kv_bf16(L, k, v, rope, kv, static_cast<hipStream_t>(stream)));
}

size_t joint_attn_fwd_bf16_workspace_bytes(const ja_params *p) {
  if (!p || check_fwd_bf16(p) != JA_OK) return 0;
  const ja::AttnLayout L = layout(p);
  const int n_cu = device_cu_count();
  return (size_t)std::max(ja::plan_fwd_bf16(L, n_cu, false).ws_bytes,
                          ja::plan_fwd_bf16(L, n_cu, true).ws_bytes);
}

// Shared checks and launch of the dense and block-sparse BF16 forwards.
static ja_status fwd_bf16_call(const ja_params *p, const void *q, const void *kv, size_t kv_bytes,
                        const float *rope, const uint8_t *mask, void *o, float *lse,
                        void *workspace, size_t workspace_bytes, void *stream) {
  if (!p || !q || !kv || !o) return JA_ERR_INVALID_ARG;
  const ja_status st = check_fwd_bf16(p);
  if (st != JA_OK) return st;
  if (!aligned16(q) || !aligned16(kv) || !aligned16(o) || (rope && !aligned16(rope)) ||
      (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) || (workspace && !aligned16(workspace)))
    return JA_ERR_INVALID_ARG;
  if (o == q || o == kv) return JA_ERR_INVALID_ARG;
  const ja::AttnLayout L = layout(p);
  if (kv_bytes < (size_t)ja::prep_kv_bytes(L)) return JA_ERR_INVALID_ARG;
  ja::SplitPlan plan = ja::plan_fwd_bf16(L, device_cu_count(), mask != nullptr);
  if (plan.n_units > 0 && (!workspace || workspace_bytes < (size_t)plan.ws_bytes))
    plan = ja::SplitPlan{plan.n_direct + plan.n_units / plan.parts, 1, 0, 0};
  return hip_status(ja::launch_fwd_bf16(L, q, kv, rope, mask, o, lse, plan, workspace,
                                        static_cast<hipStream_t>(stream)));
}

ja_status joint_attn_fwd_bf16(const ja_params *p, const void *q, const void *kv,
                              size_t kv_bytes, const float *rope, void *o, float *lse,
                              void *workspace, size_t workspace_bytes, void *stream) {
  return fwd_bf16_call(p, q, kv, kv_bytes, rope, nullptr, o, lse, workspace, workspace_bytes,
                       stream);
}

ja_status joint_attn_fwd_bf16_block_sparse(const ja_params *p, const void *q, const void *kv,
                                           size_t kv_bytes, const float *rope,
                                           const uint8_t *block_mask, void *o, float *lse,
                                           void *workspace, size_t workspace_bytes,
                                           void *stream) {
  if (!block_mask) return JA_ERR_INVALID_ARG;
  if (p && p->seq_len > ja::fwd_bf16_sparse_max_seq()) return JA_ERR_UNSUPPORTED;
  return fwd_bf16_call(p, q, kv, kv_bytes, rope, block_mask, o, lse, workspace,
                       workspace_bytes, stream);
}

ja_status joint_attn_quant_rope_fp8(const ja_params *p, const void *q,
                                    const void *k, const void *v,
                                    const float *rope, void *q8, void *k8,
                                    void *v8, float *sq, float *sk, float *sv,
                                    void *stream) {
  if (!p || !q || !k || !v || !q8 || !k8 || !v8 || !sq || !sk || !sv)
    return JA_ERR_INVALID_ARG;
  const ja_status st = check_params(p, true, 0);
  if (st != JA_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(q8) ||
      !aligned16(k8) || !aligned16(v8) || (rope && !aligned16(rope)) ||
      (reinterpret_cast<uintptr_t>(sq) & 3u) || (reinterpret_cast<uintptr_t>(sk) & 3u) ||
      (reinterpret_cast<uintptr_t>(sv) & 3u))
    return JA_ERR_INVALID_ARG;
  const int64_t threads = (int64_t)p->batch * p->seq_len * p->heads * (p->head_dim / 8);
  if ((threads + 255) / 256 > 0x7fffffffLL) return JA_ERR_UNSUPPORTED;
  return hip_status(ja::launch_quant_rope_fp8(layout(p), q, k, v, rope, q8, k8, v8,
                                              sq, sk, sv,
                                              static_cast<hipStream_t>(stream)));
}

size_t joint_attn_fwd_fp8_workspace_bytes(const ja_params *p) {
  if (!p || check_fwd_fp8(p) != JA_OK) return 0;
  return (size_t)ja::plan_fwd_fp8(layout(p), device_cu_count()).ws_bytes;
}

ja_status joint_attn_fp8_repair_plan(const ja_params *p, const void *k, const void *v,
                                     const float *rope, const void *k8, const void *v8,
                                     const float *sk, const float *sv, int32_t n_rep,
                                     int32_t *idx, void *kr, void *vr, float *kbias,
                                     void *stream) {
  if (!p || !k || !v || !k8 || !v8 || !sk || !sv || !kbias || !kr || !vr)
    return JA_ERR_INVALID_ARG;
  const ja_status st = check_params(p, true, 0);
  if (st != JA_OK) return st;
  if (n_rep < 0 || n_rep > p->seq_len || (n_rep > 0 && !idx)) return JA_ERR_INVALID_ARG;
  if (p->seq_len > ja::repair_max_seq()) return JA_ERR_UNSUPPORTED;
  if ((int64_t)p->batch * p->heads > 0x7fffffffLL) return JA_ERR_UNSUPPORTED;
  if (!aligned16(k) || !aligned16(v) || !aligned16(k8) || !aligned16(v8) || !aligned16(kr) ||
      !aligned16(vr) || (rope && !aligned16(rope)) ||
      (reinterpret_cast<uintptr_t>(sk) & 3u) || (reinterpret_cast<uintptr_t>(sv) & 3u) ||
      (reinterpret_cast<uintptr_t>(kbias) & 3u) || (idx && (reinterpret_cast<uintptr_t>(idx) & 3u)))
    return JA_ERR_INVALID_ARG;
  const int64_t threads = (int64_t)p->batch * p->seq_len * p->heads * (p->head_dim / 8);
  if ((threads + 255) / 256 > 0x7fffffffLL) return JA_ERR_UNSUPPORTED;
  return hip_status(ja::launch_repair_plan(layout(p), k, v, rope, k8, v8, sk, sv, n_rep, idx,
                                           kr, vr, kbias, static_cast<hipStream_t>(stream)));
}

// Repair bias of joint_attn_prep_kv_fp8 (NULL without repair); false: invalid.
static bool repair_bias(const ja_params *p, const ja_fp8_repair *repair, const float **kbias) {
  *kbias = nullptr;
  if (!repair) return true;
  if (repair->n_rep < 0 || repair->n_rep > p->seq_len) return false;
  if (repair->n_rep == 0) return true;
  if (!repair->kbias || (reinterpret_cast<uintptr_t>(repair->kbias) & 3u)) return false;
  *kbias = repair->kbias;
  return true;
}

size_t joint_attn_prep_kv_fp8_bytes(const ja_params *p) {
  if (!p || check_fwd_fp8(p) != JA_OK) return 0;
  return (size_t)ja::prep_kv_fp8_bytes(layout(p));
}

ja_status joint_attn_prep_kv_fp8(const ja_params *p, const void *k8, const void *v8,
                                 const float *sk, const float *sv, const ja_fp8_repair *repair,
                                 void *kv8, size_t kv8_bytes, void *stream) {
  if (!p || !k8 || !v8 || !sk || !sv || !kv8) return JA_ERR_INVALID_ARG;
  const ja_status st = check_fwd_fp8(p);
  if (st != JA_OK) return st;
  const float *kbias;
  if (!repair_bias(p, repair, &kbias)) return JA_ERR_INVALID_ARG;
  if (!aligned16(k8) || !aligned16(v8) || !aligned16(kv8) ||
      (reinterpret_cast<uintptr_t>(sk) & 3u) || (reinterpret_cast<uintptr_t>(sv) & 3u))
    return JA_ERR_INVALID_ARG;
  const ja::AttnLayout L = layout(p);
  if (kv8_bytes < (size_t)ja::prep_kv_fp8_bytes(L)) return JA_ERR_INVALID_ARG;
  return hip_status(ja::launch_prep_kv_fp8(L, k8, v8, sk, sv, kbias, kv8,
                                           static_cast<hipStream_t>(stream)));
}

ja_status joint_attn_fwd_fp8(const ja_params *p, const void *q8, const float *sq,
                             const void *kv8, size_t kv8_bytes, const ja_fp8_repair *repair,
                             void *o, float *lse, void *workspace, size_t workspace_bytes,
                             void *stream) {
  if (!p || !q8 || !sq || !kv8 || !o) return JA_ERR_INVALID_ARG;
  const ja_status st = check_fwd_fp8(p);
  if (st != JA_OK) return st;
  ja::Fp8Repair rp;
  if (repair && repair->n_rep > 0) {
    if (repair->n_rep > p->seq_len || !repair->kr || !repair->vr || !aligned16(repair->kr) ||
        !aligned16(repair->vr))
      return JA_ERR_INVALID_ARG;
    rp.n_rep = repair->n_rep;
    rp.kr = repair->kr;
    rp.vr = repair->vr;
  } else if (repair && repair->n_rep < 0) {
    return JA_ERR_INVALID_ARG;
  }
  if (!aligned16(q8) || !aligned16(kv8) || !aligned16(o) ||
      (reinterpret_cast<uintptr_t>(sq) & 3u) || (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) ||
      (workspace && !aligned16(workspace)))
    return JA_ERR_INVALID_ARG;
  if (o == q8 || o == kv8) return JA_ERR_INVALID_ARG;
  const ja::AttnLayout L = layout(p);
  if (kv8_bytes < (size_t)ja::prep_kv_fp8_bytes(L)) return JA_ERR_INVALID_ARG;
  ja::SplitPlan plan = ja::plan_fwd_fp8(L, device_cu_count());
  if (plan.n_units > 0 && (!workspace || workspace_bytes < (size_t)plan.ws_bytes))
    plan = ja::SplitPlan{plan.n_direct + plan.n_units / plan.parts, 1, 0, 0};
  return hip_status(ja::launch_fwd_fp8(L, q8, sq, kv8, o, lse, plan, workspace, rp,
                                       static_cast<hipStream_t>(stream)));
}

}  // extern "C"
