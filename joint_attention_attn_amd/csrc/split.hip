// Key-range split of the last partial round of a forward launch, and the
// merge of its partial results.
//
// A forward launch runs one workgroup per (query block, head, batch row)
// item on `slots` co-resident workgroups, so it takes ceil(items / slots)
// rounds; when the last round holds few items most of the chip idles through
// it.  Those items are instead each computed by `parts` workgroups over
// contiguous key ranges.  Softmax attention over a union of key sets is
// recovered exactly from the parts: with per-part row max m_j, row sum l_j
// and unnormalised output O_j (all against m_j),
//   m = max_j m_j,  l = sum_j l_j 2^{(m_j - m) c},  O = sum_j O_j 2^{(m_j - m) c} / l,
// which is the same rescaling the online softmax applies between tiles.
#include "common.hpp"
#include "internal.hpp"

namespace ja {

namespace {

constexpr int kMaxParts = 16;
constexpr int kMinTilesPerPart = 4;

struct MergeArgs {
  SplitWorkspace ws;
  bf16 *o;
  float *lse;
  int64_t o_sb, o_ss, o_sh;
  int S, H, B, n_qblk, block_rows, n_direct, parts, n_split, qgroup;
  float scale_log2;   // factor from stored row maxima to the exp2 domain
};

// One thread per (split item, row, 8-column chunk).
template <int D>
__global__ __launch_bounds__(256) void merge_split_kernel(MergeArgs m) {
  constexpr int CH = D / 8;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= (int64_t)m.n_split * m.block_rows * CH) return;
  const int ch = (int)(gid % CH);
  const int64_t rr = gid / CH;
  const int row = (int)(rr % m.block_rows);
  const int sidx = (int)(rr / m.block_rows);
  const int item = m.n_direct + sidx;
  int qblk, bh;
  item_coords(item, m.n_qblk, m.B * m.H, m.qgroup, bh, qblk);
  const int h = bh % m.H, b = bh / m.H;
  const int qi = qblk * m.block_rows + row;
  if (qi >= m.S) return;
  const float c = m.scale_log2;
  const int64_t unit0 = (int64_t)sidx * m.parts;
  bf16 *orow = m.o + b * m.o_sb + (int64_t)qi * m.o_ss + h * m.o_sh + ch * 8;
  float *lse = m.lse ? m.lse + ((int64_t)b * m.H + h) * m.S + qi : nullptr;
  float mx = -INFINITY;
  bool poisoned = false;
  for (int j = 0; j < m.parts; ++j) {
    const float mj = m.ws.ml[((unit0 + j) * m.block_rows + row) * 2];
    poisoned = poisoned || mj != mj;
    mx = fmaxf(mx, mj);
  }
  if (poisoned) {
    // a part that met an invalid input (the FP8 forward's NaN poisoning)
    // writes a NaN row maximum: the merged row is NaN too, not empty
    const uint32_t qnan = 0x7fc07fc0u;   // two bf16 quiet NaNs
    *reinterpret_cast<u32x4 *>(orow) = u32x4{qnan, qnan, qnan, qnan};
    if (lse && ch == 0) *lse = __builtin_nanf("");
    return;
  }
  float l = 0.f, acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // a row that no part saw a key for (block-sparse rows that keep no key
  // block) has every part at max -inf and sum 0: O = 0, LSE = -inf
  const bool empty = mx == -INFINITY;
  for (int j = 0; j < m.parts && !empty; ++j) {
    const int64_t r = (unit0 + j) * m.block_rows + row;
    const float2 ml = *reinterpret_cast<const float2 *>(m.ws.ml + r * 2);
    const float w = __builtin_amdgcn_exp2f((ml.x - mx) * c);
    l += ml.y * w;
    const float4 *src = reinterpret_cast<const float4 *>(m.ws.o + r * D + ch * 8);
    const float4 x0 = src[0], x1 = src[1];
    acc[0] += w * x0.x; acc[1] += w * x0.y; acc[2] += w * x0.z; acc[3] += w * x0.w;
    acc[4] += w * x1.x; acc[5] += w * x1.y; acc[6] += w * x1.z; acc[7] += w * x1.w;
  }
  const float inv = empty ? 0.f : 1.f / l;
  u32x4 out;
  out.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  out.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
  out.z = pack_bf16x2(acc[4] * inv, acc[5] * inv);
  out.w = pack_bf16x2(acc[6] * inv, acc[7] * inv);
  *reinterpret_cast<u32x4 *>(orow) = out;
  if (lse && ch == 0) *lse = empty ? -INFINITY : (mx * c + __log2f(l)) * kLn2;
}

}  // namespace

SplitPlan plan_split(int n_items, int ntiles, int slots, int block_rows, int D) {
  SplitPlan p;
  p.n_direct = n_items;
  if (slots <= 0) return p;
  const int full = n_items / slots, rem = n_items % slots;
  if (full == 0 || rem == 0 || 2 * rem > slots) return p;
  int k = slots / rem;
  k = k < kMaxParts ? k : kMaxParts;
  k = k < ntiles / kMinTilesPerPart ? k : ntiles / kMinTilesPerPart;
  if (k < 2) return p;
  p.n_direct = n_items - rem;
  p.parts = k;
  p.n_units = rem * k;
  p.ws_bytes = (int64_t)p.n_units * block_rows * (D + 2) * 4;
  return p;
}

SplitWorkspace split_workspace(const SplitPlan &plan, void *ws, int block_rows, int D) {
  SplitWorkspace w;
  if (plan.n_units == 0 || !ws) return w;
  w.o = static_cast<float *>(ws);
  w.ml = w.o + (int64_t)plan.n_units * block_rows * D;
  return w;
}

hipError_t launch_merge_split(const AttnLayout &L, const SplitPlan &plan,
                              const SplitWorkspace &ws, int block_rows, float m_scale,
                              void *o, float *lse, hipStream_t st) {
  MergeArgs m;
  m.ws = ws;
  m.o = static_cast<bf16 *>(o);
  m.lse = lse;
  m.o_sb = L.o_sb; m.o_ss = L.o_ss; m.o_sh = L.o_sh;
  m.S = L.S;
  m.H = L.H;
  m.B = L.B;
  m.n_qblk = (L.S + block_rows - 1) / block_rows;
  m.qgroup = plan.qgroup;
  m.block_rows = block_rows;
  m.n_direct = plan.n_direct;
  m.parts = plan.parts;
  m.n_split = plan.n_units / plan.parts;
  m.scale_log2 = m_scale;
  const int64_t threads = (int64_t)m.n_split * block_rows * (L.D / 8);
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (L.D == 64)
    hipLaunchKernelGGL(merge_split_kernel<64>, grid, dim3(256), 0, st, m);
  else
    hipLaunchKernelGGL(merge_split_kernel<128>, grid, dim3(256), 0, st, m);
  return hipGetLastError();
}

}  // namespace ja
