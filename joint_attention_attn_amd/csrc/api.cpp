// C ABI of libjoint_attn.so: argument validation, workspace layout, status
// codes and launch.  Every check runs on the host before anything is
// enqueued, so an invalid call never touches the device.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/joint_attn.h"
#include "internal.hpp"

namespace {

thread_local char g_last_error[256] = "";

// Record what was wrong with a call and return its status.
ja_status fail(ja_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return s;
}

ja_status hip_status(hipError_t e) {
  if (e == hipSuccess) return JA_OK;
  return fail(JA_ERR_HIP, "%s: %s", hipGetErrorName(e), hipGetErrorString(e));
}

#define JA_TRY(expr)                         \
  do {                                       \
    const ja_status st_ = (expr);            \
    if (st_ != JA_OK) return st_;            \
  } while (0)

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
int64_t align256(int64_t n) { return (n + 255) / 256 * 256; }
char *byte_ptr(void *p, int64_t off) { return static_cast<char *>(p) + off; }

bool dim_supported(int d) { return d == 64 || d == 128; }

// Strides of a bf16 tensor: multiples of 8 elements (16-byte vector access)
// and non-negative.
bool strides_ok(int64_t sb, int64_t ss, int64_t sh) {
  return sb >= 0 && ss >= 0 && sh >= 0 && sb % 8 == 0 && ss % 8 == 0 && sh % 8 == 0;
}

// ---- RoPE: where the table comes from ----
// the call must build the table itself (positions given, no table)
bool rope_build(const ja_params *p) { return p->rope_table == nullptr && p->pos != nullptr; }
int64_t rope_bytes(const ja_params *p) { return (int64_t)p->seq_len * p->head_dim * 8; }
float rope_theta(const ja_params *p) { return p->rope_theta != 0.f ? p->rope_theta : 10000.f; }

// Checks of the shape, scale, RoPE and norm fields shared by every call.
ja_status check_common(const ja_params *p) {
  if (!p) return fail(JA_ERR_INVALID_ARG, "p is NULL");
  if (p->batch < 1 || p->seq_len < 1 || p->heads < 1)
    return fail(JA_ERR_INVALID_ARG, "batch, seq_len and heads must be >= 1");
  if (!dim_supported(p->head_dim))
    return fail(JA_ERR_UNSUPPORTED, "head_dim %d is not 64 or 128", p->head_dim);
  if (p->heads > 65535 || p->batch > 65535)
    return fail(JA_ERR_UNSUPPORTED, "batch and heads are limited to 65535");
  if (!std::isfinite(p->softmax_scale) || p->softmax_scale < 0.f)
    return fail(JA_ERR_INVALID_ARG, "softmax_scale must be finite and >= 0");
  if (!std::isfinite(p->norm_eps) || p->norm_eps < 0.f)
    return fail(JA_ERR_INVALID_ARG, "norm_eps must be finite and >= 0");
  if (!aligned16(p->q_norm) || !aligned16(p->k_norm))
    return fail(JA_ERR_INVALID_ARG, "q_norm and k_norm must be 16-byte aligned");
  if (!std::isfinite(p->rope_theta) || p->rope_theta < 0.f)
    return fail(JA_ERR_INVALID_ARG, "rope_theta must be finite and >= 0");
  if (!aligned4(p->pos)) return fail(JA_ERR_INVALID_ARG, "pos must be 4-byte aligned");
  if (p->rope_table) {
    if (!aligned16(p->rope_table))
      return fail(JA_ERR_INVALID_ARG, "rope_table must be 16-byte aligned");
    if (p->rope_table_bytes < (size_t)rope_bytes(p))
      return fail(JA_ERR_INVALID_ARG,
                  "rope_table_bytes %zu is less than seq_len * head_dim * 8 = %lld",
                  p->rope_table_bytes, (long long)rope_bytes(p));
  }
  if ((p->flags & ~JA_FLAG_NO_SPLIT) != 0) return fail(JA_ERR_INVALID_ARG, "unknown flags");
  return JA_OK;
}

ja_status check_bf16_strides(const ja_params *p, bool q, bool kv, bool o) {
  if (q && !strides_ok(p->q_sb, p->q_ss, p->q_sh))
    return fail(JA_ERR_INVALID_ARG, "Q strides must be non-negative multiples of 8");
  if (kv && (!strides_ok(p->k_sb, p->k_ss, p->k_sh) || !strides_ok(p->v_sb, p->v_ss, p->v_sh)))
    return fail(JA_ERR_INVALID_ARG, "K and V strides must be non-negative multiples of 8");
  if (o && !strides_ok(p->o_sb, p->o_ss, p->o_sh))
    return fail(JA_ERR_INVALID_ARG, "O strides must be non-negative multiples of 8");
  return JA_OK;
}

// Grid of a forward: one workgroup per (query block, head, batch row) on a
// 1-D grid indexed with 32-bit ints.
ja_status check_grid(const ja_params *p, int block_rows) {
  const int64_t nx = ((int64_t)p->seq_len + block_rows - 1) / block_rows;
  if (nx * p->heads * p->batch > 0x7fffffffLL)
    return fail(JA_ERR_UNSUPPORTED, "too many work items for one launch");
  return JA_OK;
}

// Lane-per-chunk passes (quantizer, repair): their 1-D grid of 256-thread
// workgroups.
ja_status check_vector_grid(const ja_params *p) {
  const int64_t threads = (int64_t)p->batch * p->seq_len * p->heads * (p->head_dim / 8);
  if ((threads + 255) / 256 > 0x7fffffffLL)
    return fail(JA_ERR_UNSUPPORTED, "too many head vectors for one launch");
  return JA_OK;
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

// Split plan of a forward, or no split when the flags say so.
ja::SplitPlan no_split(const ja::SplitPlan &plan) {
  if (plan.n_units == 0) return plan;
  ja::SplitPlan p = plan;
  p.n_direct = plan.n_direct + plan.n_units / plan.parts;
  p.parts = 1;
  p.n_units = 0;
  p.ws_bytes = 0;
  return p;
}
ja::SplitPlan plan_bf16(const ja_params *p, bool sparse) {
  const ja::SplitPlan plan = ja::plan_fwd_bf16(layout(p), device_cu_count(), sparse);
  return (p->flags & JA_FLAG_NO_SPLIT) ? no_split(plan) : plan;
}
ja::SplitPlan plan_fp8(const ja_params *p, bool sparse) {
  const ja::SplitPlan plan = ja::plan_fwd_fp8(layout(p), device_cu_count(), sparse);
  return (p->flags & JA_FLAG_NO_SPLIT) ? no_split(plan) : plan;
}
// Workspace of the split for either FP8 forward (dense or block-sparse).
int64_t fp8_split_bytes(const ja_params *p) {
  return std::max(plan_fp8(p, false).ws_bytes, plan_fp8(p, true).ws_bytes);
}

// ---- BF16 path ----

// Checks of the BF16 forwards that do not involve device pointers.
ja_status check_bf16(const ja_params *p, bool q, bool kv) {
  JA_TRY(check_common(p));
  JA_TRY(check_bf16_strides(p, q, kv, q));
  // the block-sparse forward has the smaller workgroups, hence the larger grid
  JA_TRY(check_grid(p, ja::fwd_bf16_block_rows(true)));
  // the prepared K and V^T of one (batch, head) are addressed with 32-bit
  // byte offsets; the preparation pass has one workgroup per 64 keys and head
  const int64_t s_pad = ((int64_t)p->seq_len + 63) / 64 * 64;
  if (s_pad * p->head_dim * 2 > 0x7fffffffLL || s_pad / 64 * p->batch * p->heads > 0x7fffffffLL)
    return fail(JA_ERR_UNSUPPORTED, "sequence too long for the prepared K/V layout");
  return JA_OK;
}

// Prepared K/V of the BF16 path: rotated K and V^T, then (when the call
// builds them from pos) the RoPE table and the coordinate table.
int64_t prep_kv_bf16_core(const ja_params *p) { return align256(ja::prep_kv_bytes(layout(p))); }
int64_t prep_kv_bf16_total(const ja_params *p) {
  return prep_kv_bf16_core(p) +
         (rope_build(p) ? align256(rope_bytes(p)) + align256(ja::coord_table_bytes(p->head_dim))
                        : 0);
}
// Table a BF16 call on prepared K/V rotates Q with (NULL = no RoPE).
const double *prepared_table(const ja_params *p, const void *kv) {
  if (p->rope_table) return p->rope_table;
  if (p->pos) return reinterpret_cast<const double *>(
      static_cast<const char *>(kv) + prep_kv_bf16_core(p));
  return nullptr;
}
// The coordinate table built beside it (NULL with a caller's table).
const double *prepared_coord_table(const ja_params *p, const void *kv) {
  if (!rope_build(p)) return nullptr;
  return reinterpret_cast<const double *>(static_cast<const char *>(kv) + prep_kv_bf16_core(p) +
                                          align256(rope_bytes(p)));
}

ja_status launch_table(const ja_params *p, double *table, double *ctab, hipStream_t st) {
  return hip_status(ja::launch_rope_table_2d(p->pos, p->seq_len, p->head_dim, rope_theta(p),
                                             table, ctab, st));
}

ja_status prep_bf16(const ja_params *p, const void *k, const void *v, void *kv, hipStream_t st) {
  const double *table = p->rope_table;
  if (rope_build(p)) {
    double *built = reinterpret_cast<double *>(byte_ptr(kv, prep_kv_bf16_core(p)));
    double *ctab = reinterpret_cast<double *>(
        byte_ptr(kv, prep_kv_bf16_core(p) + align256(rope_bytes(p))));
    JA_TRY(launch_table(p, built, ctab, st));
    table = built;
  }
  return hip_status(ja::launch_prep_kv_bf16(layout(p), k, v, table, kv, st));
}

ja_status fwd_bf16_launch(const ja_params *p, const void *q, const void *kv,
                          const uint8_t *mask, void *o, float *lse, void *ws,
                          size_t ws_bytes, hipStream_t st) {
  ja::SplitPlan plan = plan_bf16(p, mask != nullptr);
  if (plan.n_units > 0 && (size_t)plan.ws_bytes > ws_bytes)
    return fail(JA_ERR_INVALID_ARG, "workspace of %zu bytes is less than the %lld needed",
                ws_bytes, (long long)plan.ws_bytes);
  const double *ctab = prepared_coord_table(p, kv);
  return hip_status(ja::launch_fwd_bf16(layout(p), q, kv, prepared_table(p, kv), ctab,
                                        ctab ? p->pos : nullptr, mask, o, lse, plan, ws, st));
}

ja_status check_sparse(const ja_params *p, const uint8_t *mask, int max_seq) {
  if (!mask) return fail(JA_ERR_INVALID_ARG, "block_mask is NULL");
  if (p && p->seq_len > max_seq)
    return fail(JA_ERR_UNSUPPORTED, "the block-sparse forward takes at most %d tokens", max_seq);
  return JA_OK;
}

// Checks and launch of the one-call BF16 forwards (dense, or block-sparse
// with a mask).
ja_status fwd_bf16_call(const ja_params *p, const void *q, const void *k, const void *v,
                        const uint8_t *mask, void *o, float *lse, void *ws, size_t ws_bytes,
                        void *stream) {
  JA_TRY(check_bf16(p, true, true));
  if (!q || !k || !v || !o) return fail(JA_ERR_INVALID_ARG, "q, k, v and o must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned4(lse) ||
      !aligned16(ws))
    return fail(JA_ERR_INVALID_ARG, "misaligned pointer (16 bytes; lse 4 bytes)");
  if (o == q || o == k || o == v || o == ws) return fail(JA_ERR_INVALID_ARG, "o aliases an input");
  const int64_t kv_bytes = prep_kv_bf16_total(p);
  const ja::SplitPlan plan = plan_bf16(p, mask != nullptr);
  const int64_t need = kv_bytes + plan.ws_bytes;
  if (!ws || ws_bytes < (size_t)need)
    return fail(JA_ERR_INVALID_ARG, "workspace of %zu bytes is less than the %lld needed",
                ws_bytes, (long long)need);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  JA_TRY(prep_bf16(p, k, v, ws, st));
  return fwd_bf16_launch(p, q, ws, mask, o, lse, byte_ptr(ws, kv_bytes), ws_bytes - kv_bytes, st);
}

// Checks and launch of the BF16 forwards on prepared K/V.
ja_status fwd_bf16_prepared_call(const ja_params *p, const void *q, const void *kv,
                                 size_t kv_bytes, const uint8_t *mask, void *o, float *lse,
                                 void *ws, size_t ws_bytes, void *stream) {
  JA_TRY(check_bf16(p, true, false));
  if (!q || !kv || !o) return fail(JA_ERR_INVALID_ARG, "q, kv and o must be non-NULL");
  if (!aligned16(q) || !aligned16(kv) || !aligned16(o) || !aligned4(lse) || !aligned16(ws))
    return fail(JA_ERR_INVALID_ARG, "misaligned pointer (16 bytes; lse 4 bytes)");
  if (o == q || o == kv) return fail(JA_ERR_INVALID_ARG, "o aliases an input");
  if (kv_bytes < (size_t)prep_kv_bf16_total(p))
    return fail(JA_ERR_INVALID_ARG, "kv_bytes %zu is less than joint_attn_prep_kv_bf16_bytes",
                kv_bytes);
  return fwd_bf16_launch(p, q, kv, mask, o, lse, ws, ws ? ws_bytes : 0,
                         static_cast<hipStream_t>(stream));
}

// ---- FP8 path ----

ja_status check_fp8(const ja_params *p) {
  JA_TRY(check_common(p));
  JA_TRY(check_bf16_strides(p, false, false, true));
  // the block-sparse forward has the smaller workgroups, hence the larger grid
  JA_TRY(check_grid(p, ja::fwd_fp8_block_rows(true)));
  // the prepared K and V^T of one (batch, head) are addressed with 32-bit
  // byte offsets; the preparation pass has one workgroup per 64 keys and head
  const int64_t s_pad = ((int64_t)p->seq_len + 63) / 64 * 64;
  if (s_pad * p->head_dim > 0x7fffffffLL || s_pad / 64 * p->batch * p->heads > 0x7fffffffLL)
    return fail(JA_ERR_UNSUPPORTED, "sequence too long for the prepared K/V layout");
  return JA_OK;
}

// Repair bias of the FP8 preparation (NULL without repair).
ja_status repair_bias(const ja_params *p, const ja_fp8_repair *repair, const float **kbias) {
  *kbias = nullptr;
  if (!repair || repair->n_rep == 0) return JA_OK;
  if (repair->n_rep < 0 || repair->n_rep > p->seq_len)
    return fail(JA_ERR_INVALID_ARG, "repair->n_rep must be in [0, seq_len]");
  if (!repair->kbias || !aligned4(repair->kbias))
    return fail(JA_ERR_INVALID_ARG, "repair->kbias must be a 4-byte aligned pointer");
  *kbias = repair->kbias;
  return JA_OK;
}

ja_status prep_fp8(const ja_params *p, const void *k8, const void *v8, const float *sk,
                   const float *sv, const float *kbias, void *kv8, hipStream_t st) {
  return hip_status(ja::launch_prep_kv_fp8(layout(p), k8, v8, sk, sv, kbias, kv8, st));
}

ja_status fwd_fp8_launch(const ja_params *p, const void *q8, const float *sq, const void *kv8,
                         const uint8_t *mask, const ja::Fp8Repair &rp, void *o, float *lse,
                         void *ws, size_t ws_bytes, hipStream_t st) {
  const ja::SplitPlan plan = plan_fp8(p, mask != nullptr);
  if (plan.n_units > 0 && (size_t)plan.ws_bytes > ws_bytes)
    return fail(JA_ERR_INVALID_ARG, "workspace of %zu bytes is less than the %lld needed",
                ws_bytes, (long long)plan.ws_bytes);
  return hip_status(ja::launch_fwd_fp8(layout(p), q8, sq, kv8, mask, o, lse, plan, ws, rp, st));
}

// Checks and launch of the one-call FP8 forwards (dense, or block-sparse
// with a mask).
ja_status fwd_fp8_call(const ja_params *p, const void *q8, const void *k8, const void *v8,
                       const float *sq, const float *sk, const float *sv, const uint8_t *mask,
                       void *o, float *lse, void *ws, size_t ws_bytes, void *stream) {
  JA_TRY(check_fp8(p));
  if (!q8 || !k8 || !v8 || !sq || !sk || !sv || !o)
    return fail(JA_ERR_INVALID_ARG, "every tensor pointer must be non-NULL");
  if (!aligned16(q8) || !aligned16(k8) || !aligned16(v8) || !aligned16(o) || !aligned4(sq) ||
      !aligned4(sk) || !aligned4(sv) || !aligned4(lse) || !aligned16(ws))
    return fail(JA_ERR_INVALID_ARG, "misaligned pointer (16 bytes; scales, lse 4 bytes)");
  if (o == q8 || o == k8 || o == v8 || o == ws)
    return fail(JA_ERR_INVALID_ARG, "o aliases an input");
  const int64_t kv_bytes = align256(ja::prep_kv_fp8_bytes(layout(p)));
  const int64_t need = kv_bytes + plan_fp8(p, mask != nullptr).ws_bytes;
  if (!ws || ws_bytes < (size_t)need)
    return fail(JA_ERR_INVALID_ARG, "workspace of %zu bytes is less than the %lld needed",
                ws_bytes, (long long)need);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  JA_TRY(prep_fp8(p, k8, v8, sk, sv, nullptr, ws, st));
  return fwd_fp8_launch(p, q8, sq, ws, mask, ja::Fp8Repair{}, o, lse, byte_ptr(ws, kv_bytes),
                        ws_bytes - kv_bytes, st);
}

// Checks and launch of the FP8 forwards on prepared K/V.
ja_status fwd_fp8_prepared_call(const ja_params *p, const void *q8, const float *sq,
                                const void *kv8, size_t kv8_bytes, const ja_fp8_repair *repair,
                                const uint8_t *mask, void *o, float *lse, void *ws,
                                size_t ws_bytes, void *stream) {
  JA_TRY(check_fp8(p));
  if (!q8 || !sq || !kv8 || !o) return fail(JA_ERR_INVALID_ARG, "q8, sq, kv8 and o must be non-NULL");
  ja::Fp8Repair rp;
  if (repair && repair->n_rep != 0) {
    if (repair->n_rep < 0 || repair->n_rep > p->seq_len)
      return fail(JA_ERR_INVALID_ARG, "repair->n_rep must be in [0, seq_len]");
    if (!repair->kr || !repair->vr || !aligned16(repair->kr) || !aligned16(repair->vr))
      return fail(JA_ERR_INVALID_ARG, "repair->kr and repair->vr must be 16-byte aligned pointers");
    rp.n_rep = repair->n_rep;
    rp.kr = repair->kr;
    rp.vr = repair->vr;
  }
  if (!aligned16(q8) || !aligned16(kv8) || !aligned16(o) || !aligned4(sq) || !aligned4(lse) ||
      !aligned16(ws))
    return fail(JA_ERR_INVALID_ARG, "misaligned pointer (16 bytes; sq, lse 4 bytes)");
  if (o == q8 || o == kv8) return fail(JA_ERR_INVALID_ARG, "o aliases an input");
  if (kv8_bytes < (size_t)ja::prep_kv_fp8_bytes(layout(p)))
    return fail(JA_ERR_INVALID_ARG, "kv8_bytes %zu is less than joint_attn_prep_kv_fp8_bytes",
                kv8_bytes);
  return fwd_fp8_launch(p, q8, sq, kv8, mask, rp, o, lse, ws, ws ? ws_bytes : 0,
                        static_cast<hipStream_t>(stream));
}

// ---- scratch of joint_attn_fwd_bf16_prepared_noalloc ----
// A static device array (each device the library runs on holds its own copy
// until the process ends).  In host code `scratch` only names the symbol:
// its device address comes from hipGetSymbolAddress, looked up once per
// device with that device current.
__device__ __align__(256) unsigned char scratch[JA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;
void *g_scratch_ptr[kMaxScratchDevices];
std::mutex g_scratch_mutex;

// Device address of the current device's scratch array.
ja_status scratch_address(void **out) {
  int dev = 0;
  JA_TRY(hip_status(hipGetDevice(&dev)));
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(JA_ERR_UNSUPPORTED, "device %d is past the %d devices the scratch table holds",
                dev, kMaxScratchDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    JA_TRY(hip_status(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch))));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return JA_OK;
}

}  // namespace

extern "C" {

const char *joint_attn_status_string(ja_status s) {
  // a C caller may pass any int; read it as one (an out-of-range value of
  // the enum type is not a valid C++ value)
  int code;
  std::memcpy(&code, &s, sizeof code);
  switch (code) {
    case JA_OK: return "JA_OK";
    case JA_ERR_INVALID_ARG: return "JA_ERR_INVALID_ARG: invalid argument";
    case JA_ERR_UNSUPPORTED: return "JA_ERR_UNSUPPORTED: unsupported shape";
    case JA_ERR_HIP: return "JA_ERR_HIP: HIP runtime error";
  }
  return "unknown ja_status";
}

const char *joint_attn_last_error(void) { return g_last_error; }

ja_status joint_attn_rope_table_2d(const int32_t *pos, int32_t seq_len, int32_t head_dim,
                                   float theta, double *table, void *stream) {
  if (!pos || !table) return fail(JA_ERR_INVALID_ARG, "pos and table must be non-NULL");
  if (seq_len < 1) return fail(JA_ERR_INVALID_ARG, "seq_len must be >= 1");
  if (!(theta > 0.f) || !std::isfinite(theta))
    return fail(JA_ERR_INVALID_ARG, "theta must be finite and > 0");
  if (!dim_supported(head_dim))
    return fail(JA_ERR_UNSUPPORTED, "head_dim %d is not 64 or 128", head_dim);
  if (!aligned16(table) || !aligned4(pos))
    return fail(JA_ERR_INVALID_ARG, "table must be 16-byte and pos 4-byte aligned");
  if ((int64_t)seq_len * (head_dim / 2) > 0x7fffffffLL * 256)
    return fail(JA_ERR_UNSUPPORTED, "table too large for one launch");
  return hip_status(ja::launch_rope_table_2d(pos, seq_len, head_dim, theta, table, nullptr,
                                             static_cast<hipStream_t>(stream)));
}

// ---- BF16 path ----

size_t joint_attn_prep_kv_bf16_bytes(const ja_params *p) {
  if (check_bf16(p, false, true) != JA_OK) return 0;
  return (size_t)prep_kv_bf16_total(p);
}

ja_status joint_attn_prep_kv_bf16(const ja_params *p, const void *k, const void *v, void *kv,
                                  size_t kv_bytes, void *stream) {
  JA_TRY(check_bf16(p, false, true));
  if (!k || !v || !kv) return fail(JA_ERR_INVALID_ARG, "k, v and kv must be non-NULL");
  if (!aligned16(k) || !aligned16(v) || !aligned16(kv))
    return fail(JA_ERR_INVALID_ARG, "k, v and kv must be 16-byte aligned");
  if (kv_bytes < (size_t)prep_kv_bf16_total(p))
    return fail(JA_ERR_INVALID_ARG, "kv_bytes %zu is less than joint_attn_prep_kv_bf16_bytes",
                kv_bytes);
  return prep_bf16(p, k, v, kv, static_cast<hipStream_t>(stream));
}

size_t joint_attn_fwd_bf16_prepared_workspace_bytes(const ja_params *p) {
  if (check_bf16(p, true, false) != JA_OK) return 0;
  // the dense and the block-sparse forwards plan different splits
  return (size_t)std::max(plan_bf16(p, false).ws_bytes, plan_bf16(p, true).ws_bytes);
}

size_t joint_attn_fwd_bf16_workspace_bytes(const ja_params *p) {
  if (check_bf16(p, true, true) != JA_OK) return 0;
  return (size_t)prep_kv_bf16_total(p) + joint_attn_fwd_bf16_prepared_workspace_bytes(p);
}

ja_status joint_attn_fwd_bf16(const ja_params *p, const void *q, const void *k, const void *v,
                              void *o, float *lse, void *workspace, size_t workspace_bytes,
                              void *stream) {
  return fwd_bf16_call(p, q, k, v, nullptr, o, lse, workspace, workspace_bytes, stream);
}

ja_status joint_attn_fwd_bf16_block_sparse(const ja_params *p, const void *q, const void *k,
                                           const void *v, const uint8_t *block_mask, void *o,
                                           float *lse, void *workspace, size_t workspace_bytes,
                                           void *stream) {
  JA_TRY(check_sparse(p, block_mask, ja::fwd_bf16_sparse_max_seq()));
  return fwd_bf16_call(p, q, k, v, block_mask, o, lse, workspace, workspace_bytes, stream);
}

ja_status joint_attn_fwd_bf16_prepared(const ja_params *p, const void *q, const void *kv,
                                       size_t kv_bytes, void *o, float *lse, void *workspace,
                                       size_t workspace_bytes, void *stream) {
  return fwd_bf16_prepared_call(p, q, kv, kv_bytes, nullptr, o, lse, workspace, workspace_bytes,
                                stream);
}

ja_status joint_attn_fwd_bf16_prepared_noalloc(const ja_params *p, const void *q,
                                               const void *kv, size_t kv_bytes, void *o,
                                               float *lse, void *stream) {
  JA_TRY(check_bf16(p, true, false));
  const ja::SplitPlan plan = plan_bf16(p, false);
  if ((size_t)plan.ws_bytes > JA_NOALLOC_SCRATCH_BYTES)
    return fail(JA_ERR_UNSUPPORTED,
                "the split needs %lld bytes of scratch, more than the %zu of the static array",
                (long long)plan.ws_bytes, (size_t)JA_NOALLOC_SCRATCH_BYTES);
  void *ws = nullptr;
  if (plan.n_units > 0) JA_TRY(scratch_address(&ws));
  return fwd_bf16_prepared_call(p, q, kv, kv_bytes, nullptr, o, lse, ws,
                                ws ? JA_NOALLOC_SCRATCH_BYTES : 0, stream);
}

ja_status joint_attn_fwd_bf16_block_sparse_prepared(const ja_params *p, const void *q,
                                                    const void *kv, size_t kv_bytes,
                                                    const uint8_t *block_mask, void *o,
                                                    float *lse, void *workspace,
                                                    size_t workspace_bytes, void *stream) {
  JA_TRY(check_sparse(p, block_mask, ja::fwd_bf16_sparse_max_seq()));
  return fwd_bf16_prepared_call(p, q, kv, kv_bytes, block_mask, o, lse, workspace,
                                workspace_bytes, stream);
}

// ---- FP8 path ----

size_t joint_attn_quant_rope_fp8_workspace_bytes(const ja_params *p) {
  if (check_common(p) != JA_OK) return 0;
  return rope_build(p) ? (size_t)rope_bytes(p) : 0;
}

ja_status joint_attn_quant_rope_fp8(const ja_params *p, const void *q, const void *k,
                                    const void *v, void *q8, void *k8, void *v8, float *sq,
                                    float *sk, float *sv, void *workspace,
                                    size_t workspace_bytes, void *stream) {
  JA_TRY(check_common(p));
  JA_TRY(check_bf16_strides(p, true, true, false));
  JA_TRY(check_vector_grid(p));
  if (!q || !k || !v || !q8 || !k8 || !v8 || !sq || !sk || !sv)
    return fail(JA_ERR_INVALID_ARG, "every tensor pointer must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(q8) || !aligned16(k8) ||
      !aligned16(v8) || !aligned4(sq) || !aligned4(sk) || !aligned4(sv) || !aligned16(workspace))
    return fail(JA_ERR_INVALID_ARG, "misaligned pointer (16 bytes; scales 4 bytes)");
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const double *table = p->rope_table;
  if (rope_build(p)) {
    if (!workspace || workspace_bytes < (size_t)rope_bytes(p))
      return fail(JA_ERR_INVALID_ARG, "workspace of %zu bytes is less than the %lld needed",
                  workspace_bytes, (long long)rope_bytes(p));
    JA_TRY(launch_table(p, static_cast<double *>(workspace), nullptr, st));
    table = static_cast<const double *>(workspace);
  }
  return hip_status(ja::launch_quant_rope_fp8(layout(p), q, k, v, table, q8, k8, v8, sq, sk, sv,
                                              st));
}

int32_t joint_attn_fp8_repair_count(double budget, int32_t seq_len) {
  if (!(budget >= 0.0 && budget <= 1.0) || seq_len < 1) {
    fail(JA_ERR_INVALID_ARG, "budget must be in [0, 1] and seq_len >= 1");
    return -1;
  }
  return (int32_t)std::ceil(budget * (double)seq_len);
}

size_t joint_attn_fp8_repair_plan_workspace_bytes(const ja_params *p) {
  return joint_attn_quant_rope_fp8_workspace_bytes(p);
}

ja_status joint_attn_fp8_repair_plan(const ja_params *p, const void *k, const void *v,
                                     const void *k8, const void *v8, const float *sk,
                                     const float *sv, int32_t n_rep, int32_t *idx, void *kr,
                                     void *vr, float *kbias, void *workspace,
                                     size_t workspace_bytes, void *stream) {
  JA_TRY(check_common(p));
  JA_TRY(check_bf16_strides(p, false, true, false));
  JA_TRY(check_vector_grid(p));
  if (!k || !v || !k8 || !v8 || !sk || !sv || !kbias || !kr || !vr)
    return fail(JA_ERR_INVALID_ARG, "every tensor pointer must be non-NULL");
  if (n_rep < 0 || n_rep > p->seq_len || (n_rep > 0 && !idx))
    return fail(JA_ERR_INVALID_ARG, "n_rep must be in [0, seq_len] and idx non-NULL if n_rep > 0");
  if (p->seq_len > ja::repair_max_seq())
    return fail(JA_ERR_UNSUPPORTED, "the repair selection takes at most %d tokens",
                ja::repair_max_seq());
  if (!aligned16(k) || !aligned16(v) || !aligned16(k8) || !aligned16(v8) || !aligned16(kr) ||
      !aligned16(vr) || !aligned4(sk) || !aligned4(sv) || !aligned4(kbias) || !aligned4(idx) ||
      !aligned16(workspace))
    return fail(JA_ERR_INVALID_ARG, "misaligned pointer (16 bytes; scales, idx, kbias 4 bytes)");
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const double *table = p->rope_table;
  if (rope_build(p)) {
    if (!workspace || workspace_bytes < (size_t)rope_bytes(p))
      return fail(JA_ERR_INVALID_ARG, "workspace of %zu bytes is less than the %lld needed",
                  workspace_bytes, (long long)rope_bytes(p));
    JA_TRY(launch_table(p, static_cast<double *>(workspace), nullptr, st));
    table = static_cast<const double *>(workspace);
  }
  return hip_status(ja::launch_repair_plan(layout(p), k, v, table, k8, v8, sk, sv, n_rep, idx,
                                           kr, vr, kbias, st));
}

size_t joint_attn_prep_kv_fp8_bytes(const ja_params *p) {
  if (check_fp8(p) != JA_OK) return 0;
  return (size_t)ja::prep_kv_fp8_bytes(layout(p));
}

ja_status joint_attn_prep_kv_fp8(const ja_params *p, const void *k8, const void *v8,
                                 const float *sk, const float *sv, const ja_fp8_repair *repair,
                                 void *kv8, size_t kv8_bytes, void *stream) {
  JA_TRY(check_fp8(p));
  if (!k8 || !v8 || !sk || !sv || !kv8)
    return fail(JA_ERR_INVALID_ARG, "k8, v8, sk, sv and kv8 must be non-NULL");
  const float *kbias;
  JA_TRY(repair_bias(p, repair, &kbias));
  if (!aligned16(k8) || !aligned16(v8) || !aligned16(kv8) || !aligned4(sk) || !aligned4(sv))
    return fail(JA_ERR_INVALID_ARG, "misaligned pointer (16 bytes; scales 4 bytes)");
  if (kv8_bytes < (size_t)ja::prep_kv_fp8_bytes(layout(p)))
    return fail(JA_ERR_INVALID_ARG, "kv8_bytes %zu is less than joint_attn_prep_kv_fp8_bytes",
                kv8_bytes);
  return prep_fp8(p, k8, v8, sk, sv, kbias, kv8, static_cast<hipStream_t>(stream));
}

size_t joint_attn_fwd_fp8_prepared_workspace_bytes(const ja_params *p) {
  if (check_fp8(p) != JA_OK) return 0;
  return (size_t)fp8_split_bytes(p);
}

ja_status joint_attn_fwd_fp8_prepared(const ja_params *p, const void *q8, const float *sq,
                                      const void *kv8, size_t kv8_bytes,
                                      const ja_fp8_repair *repair, void *o, float *lse,
                                      void *workspace, size_t workspace_bytes, void *stream) {
  return fwd_fp8_prepared_call(p, q8, sq, kv8, kv8_bytes, repair, nullptr, o, lse, workspace,
                               workspace_bytes, stream);
}

ja_status joint_attn_fwd_fp8_block_sparse_prepared(const ja_params *p, const void *q8,
                                                   const float *sq, const void *kv8,
                                                   size_t kv8_bytes, const uint8_t *block_mask,
                                                   void *o, float *lse, void *workspace,
                                                   size_t workspace_bytes, void *stream) {
  JA_TRY(check_sparse(p, block_mask, ja::fwd_fp8_sparse_max_seq()));
  return fwd_fp8_prepared_call(p, q8, sq, kv8, kv8_bytes, nullptr, block_mask, o, lse, workspace,
                               workspace_bytes, stream);
}

size_t joint_attn_fwd_fp8_workspace_bytes(const ja_params *p) {
  if (check_fp8(p) != JA_OK) return 0;
  return (size_t)align256(ja::prep_kv_fp8_bytes(layout(p))) + (size_t)fp8_split_bytes(p);
}

ja_status joint_attn_fwd_fp8(const ja_params *p, const void *q8, const void *k8, const void *v8,
                             const float *sq, const float *sk, const float *sv, void *o,
                             float *lse, void *workspace, size_t workspace_bytes, void *stream) {
  return fwd_fp8_call(p, q8, k8, v8, sq, sk, sv, nullptr, o, lse, workspace, workspace_bytes,
                      stream);
}

ja_status joint_attn_fwd_fp8_block_sparse(const ja_params *p, const void *q8, const void *k8,
                                          const void *v8, const float *sq, const float *sk,
                                          const float *sv, const uint8_t *block_mask, void *o,
                                          float *lse, void *workspace, size_t workspace_bytes,
                                          void *stream) {
  JA_TRY(check_sparse(p, block_mask, ja::fwd_fp8_sparse_max_seq()));
  return fwd_fp8_call(p, q8, k8, v8, sq, sk, sv, block_mask, o, lse, workspace, workspace_bytes,
                      stream);
}

}  // extern "C"
