// Repair set of the FP8 path: the tokens with the largest quantization error.
//
// In the pages' VC-Attention FP8 setting, a budget (vc_repair_budget) sets
// what share of the tokens gets corrected: those whose quantization hurt
// most ("Speed Up Image Generation with FLUX 3 Image Klein on NVIDIA
// Blackwell GPUs", section "Quantized and sparse attention").  Here, per
// (batch, head):
//   e[token] = max_d |k - k^| + max_d |v - v^|   (k the rotated key that was
//              quantized, from the fp64 prologue; k^ = value(code) * scale,
//              exact in fp64; the differences, maxima and sum in fp64, the
//              sum then rounded to fp32, the precision in which tokens are
//              ranked)
//   the n tokens with the largest e are repaired (ties to the lower index);
//   their keys and values then enter the FP8 forward at bf16-path precision:
//   the K/V preparation masks them out of the FP8 tiles (kbias = -inf in their
//   score's initial value) and the forward attends them once more from kr / vr
//   (the rotated key rounded once to bf16, the bf16 value).
//
// Two kernels:
//   repair_err_kernel     one lane group per (b, token, head) vector, as in the
//                         quantizer; writes e into kbias [B][H][S].
//   repair_select_kernel  one workgroup per (b, h): finds the n-th largest e by
//                         a radix select over its fp32 pattern, four 8-bit
//                         digits (e >= 0, so the patterns order like the
//                         values), ranks ties by index with block scans,
//                         writes the ascending index list and kbias = 0 /
//                         -inf, then gathers kr / vr.
#include "common.hpp"
#include "internal.hpp"

namespace ja {

namespace {

constexpr int SEL_NT = 1024;   // threads of the selection workgroup

struct ErrArgs {
  const bf16 *k, *v;
  int64_t k_sb, k_ss, k_sh, v_sb, v_ss, v_sh;
  const double2 *rope;          // RoPE table [S][D/2] (cos, sin) in fp64
  const float *kn;              // K RMS-norm weights [D], NULL = none
  float eps;
  const uint8_t *k8, *v8;
  const float *sk, *sv;
  float *err;                   // [B][H][S]
  int S, H;
  int64_t rows;                 // B * S * H
  FastDiv fh, fs;               // division by H and by S
};

// Max over the 8 elements of a chunk of |x - value(code) * scale| in fp64
// (value(code) * scale is exact there).
__device__ __forceinline__ double chunk_error(const double (&x)[8], u32x2 codes, float scale) {
  double e = 0.0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t w = i < 4 ? codes.x : codes.y;
    float dq;
    switch (i & 3) {
      case 0: dq = __builtin_amdgcn_cvt_f32_fp8((int)w, 0); break;
      case 1: dq = __builtin_amdgcn_cvt_f32_fp8((int)w, 1); break;
      case 2: dq = __builtin_amdgcn_cvt_f32_fp8((int)w, 2); break;
      default: dq = __builtin_amdgcn_cvt_f32_fp8((int)w, 3); break;
    }
    e = __builtin_fmax(e, __builtin_fabs(x[i] - (double)dq * (double)scale));
  }
  return e;
}

template <int D, bool WIDE>
__global__ __launch_bounds__(256) void repair_err_kernel(ErrArgs a) {
  constexpr int LPR = D / 8;  // lanes per head vector
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gid / LPR;
  const int sub = (int)(gid % LPR);
  const bool live = row < a.rows;
  int64_t b, s;
  int h;
  split_row<WIDE>(live ? row : 0, a.fh, a.fs, b, s, h);
  const int64_t sidx = (b * a.H + h) * a.S + s;

  // the key as the quantizer saw it: normalized, then rotated (fp64)
  double x[8];
  const u32x4 kw = *reinterpret_cast<const u32x4 *>(a.k + b * a.k_sb + s * a.k_ss + h * a.k_sh + sub * 8);
  double rn = 0.0;
  if (a.kn) rn = rms_scale_f64<D>(chunk_sum_lanes_f64<LPR>(chunk_sumsq_f64(kw)), a.eps);
  prologue_chunk_f64(kw, rn, a.kn ? a.kn + sub * 8 : nullptr,
                     a.rope ? a.rope + s * (D / 2) + sub * 4 : nullptr, x);
  const int64_t c8 = row * D + sub * 8;   // contiguous [B, S, H, D] codes
  double ek = chunk_error(x, *reinterpret_cast<const u32x2 *>(a.k8 + (live ? c8 : 0)), a.sk[sidx]);

  const u32x4 vw = *reinterpret_cast<const u32x4 *>(a.v + b * a.v_sb + s * a.v_ss + h * a.v_sh + sub * 8);
  prologue_chunk_f64(vw, 0.0, nullptr, nullptr, x);
  double ev = chunk_error(x, *reinterpret_cast<const u32x2 *>(a.v8 + (live ? c8 : 0)), a.sv[sidx]);
#pragma unroll
  for (int off = 1; off < LPR; off <<= 1) {
    ek = __builtin_fmax(ek, __shfl_xor(ek, off));
    ev = __builtin_fmax(ev, __shfl_xor(ev, off));
  }
  if (live && sub == 0) a.err[sidx] = (float)(ek + ev);
}

struct SelArgs {
  float *kbias;                 // in: e; out: 0 / -inf
  int32_t *idx;                 // [B][H][n]
  const bf16 *k, *v;
  int64_t k_sb, k_ss, k_sh, v_sb, v_ss, v_sh;
  const double2 *rope;          // RoPE table [S][D/2] (cos, sin) in fp64
  const float *kn;              // K RMS-norm weights [D], NULL = none
  float eps;
  bf16 *kr, *vr;                // [B][H][n_pad][D]
  int S, H, n, n_pad;
};

// Sum of x over the workgroup (every thread gets it).
__device__ __forceinline__ int block_sum(int x, int *red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = x;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int w = 0; w < SEL_NT / 64; ++w) t += red[w];
  return t;
}

// Exclusive prefix sum of x over the threads of the workgroup in thread order.
__device__ __forceinline__ int block_exclusive_scan(int x, int *red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  __syncthreads();
  if (lane == 63) red[wave] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += red[w];
  return before + incl - x;
}

template <int D>
__global__ __launch_bounds__(SEL_NT) void repair_select_kernel(SelArgs a) {
  extern __shared__ uint32_t ekey[];        // [S] fp32 patterns of e
  __shared__ int red[SEL_NT / 64];
  __shared__ int hist[256];                 // radix-select histogram
  __shared__ int sel_digit[2];              // chosen digit, rank within it
  const int tid = threadIdx.x;
  const int h = blockIdx.x % a.H, b = blockIdx.x / a.H;
  const int64_t bh = (int64_t)b * a.H + h;
  float *row = a.kbias + bh * a.S;
  const int S = a.S, n = a.n;
  for (int s = tid; s < S; s += SEL_NT) ekey[s] = __float_as_uint(row[s]);
  __syncthreads();

  // contiguous chunk of tokens of this thread (index order for the scans)
  const int per = (S + SEL_NT - 1) / SEL_NT;
  const int s0 = min(S, tid * per), s1 = min(S, s0 + per);

  // n-th largest pattern, by a radix select over four 8-bit digits from the
  // top: each pass histograms the next digit of the patterns that match the
  // digits fixed so far, and keeps the digit whose bin holds the target rank
  // (counted from the largest)
  uint32_t thr = 0;
  if (n > 0) {
    uint32_t mask = 0;
    int rank = n;       // rank of the target among the patterns matching thr
    for (int shift = 24; shift >= 0; shift -= 8) {
      if (tid < 256) hist[tid] = 0;
      __syncthreads();
      for (int s = s0; s < s1; ++s) {
        const uint32_t key = ekey[s];
        if ((key & mask) == thr) atomicAdd(&hist[(key >> shift) & 255u], 1);
      }
      __syncthreads();
      if (tid < 64) {
        // lane l holds bins 255-4l, ..., 252-4l (descending); counts above
        // each bin by an inclusive scan over the lanes
        int c[4], tot = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          c[j] = hist[255 - 4 * tid - j];
          tot += c[j];
        }
        int incl = tot;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const int y = __shfl_up(incl, off);
          if (tid >= off) incl += y;
        }
        int above = incl - tot;   // patterns in the bins above this lane's
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (above < rank && rank <= above + c[j]) {
            sel_digit[0] = 255 - 4 * tid - j;
            sel_digit[1] = rank - above;
          }
          above += c[j];
        }
      }
      __syncthreads();
      thr |= (uint32_t)sel_digit[0] << shift;
      rank = sel_digit[1];
      mask |= 255u << shift;
    }
  }
  int gt = 0, eq = 0;
  for (int s = s0; s < s1; ++s) {
    gt += ekey[s] > thr;
    eq += ekey[s] == thr;
  }
  const int need = n > 0 ? n - block_sum(gt, red) : 0;   // ties to take
  int tie_rank = block_exclusive_scan(eq, red);
  int nsel = 0;
  for (int s = s0; s < s1; ++s) {
    const bool sel = n > 0 && (ekey[s] > thr || (ekey[s] == thr && tie_rank++ < need));
    nsel += sel;
  }
  int pos = block_exclusive_scan(nsel, red);
  tie_rank = block_exclusive_scan(eq, red);
  for (int s = s0; s < s1; ++s) {
    const bool sel = n > 0 && (ekey[s] > thr || (ekey[s] == thr && tie_rank++ < need));
    if (sel) a.idx[bh * n + pos++] = s;
    row[s] = sel ? -INFINITY : 0.f;
  }
  __threadfence_block();
  __syncthreads();

  // gather the exact rotated keys and values of the repaired tokens
  constexpr int CH = D / 8;
  for (int task = tid; task < a.n_pad * CH; task += SEL_NT) {
    const int i = task / CH, c = task % CH;
    u32x4 kw = {0, 0, 0, 0}, vw = {0, 0, 0, 0};
    if (i < n) {
      const int64_t s = a.idx[bh * n + i];
      kw = *reinterpret_cast<const u32x4 *>(a.k + b * a.k_sb + s * a.k_ss + h * a.k_sh + c * 8);
      vw = *reinterpret_cast<const u32x4 *>(a.v + b * a.v_sb + s * a.v_ss + h * a.v_sh + c * 8);
    }
    // the CH chunks of a key are CH consecutive lanes (SEL_NT % CH == 0)
    const int64_t s = i < n ? a.idx[bh * n + i] : 0;
    double rn = 0.0;
    if (a.kn) rn = rms_scale_f64<D>(chunk_sum_lanes_f64<CH>(chunk_sumsq_f64(kw)), a.eps);
    if (i < n && (a.kn || a.rope))
      kw = prologue_chunk_bf16(kw, rn, a.kn ? a.kn + c * 8 : nullptr,
                               a.rope ? a.rope + s * (D / 2) + c * 4 : nullptr);
    const int64_t o = (bh * a.n_pad + i) * D + c * 8;
    *reinterpret_cast<u32x4 *>(a.kr + o) = kw;
    *reinterpret_cast<u32x4 *>(a.vr + o) = vw;
  }
}

}  // namespace

int repair_pad(int n) { return (n + 31) / 32 * 32; }

int repair_max_seq() { return 160 * 1024 / 4 - 1024; }

hipError_t launch_repair_plan(const AttnLayout &L, const void *k, const void *v,
                              const double *rope, const void *k8, const void *v8,
                              const float *sk, const float *sv, int n, int32_t *idx,
                              void *kr, void *vr, float *kbias, hipStream_t st) {
  ErrArgs e;
  e.k = static_cast<const bf16 *>(k);
  e.v = static_cast<const bf16 *>(v);
  e.k_sb = L.k_sb; e.k_ss = L.k_ss; e.k_sh = L.k_sh;
  e.v_sb = L.v_sb; e.v_ss = L.v_ss; e.v_sh = L.v_sh;
  e.rope = reinterpret_cast<const double2 *>(rope);
  e.kn = L.k_norm;
  e.eps = L.norm_eps;
  e.k8 = static_cast<const uint8_t *>(k8);
  e.v8 = static_cast<const uint8_t *>(v8);
  e.sk = sk;
  e.sv = sv;
  e.err = kbias;
  e.S = L.S;
  e.H = L.H;
  e.rows = (int64_t)L.B * L.S * L.H;
  e.fh = make_fastdiv((uint32_t)L.H);
  e.fs = make_fastdiv((uint32_t)L.S);
  const int64_t threads = e.rows * (L.D / 8);
  const dim3 grid((unsigned)((threads + 255) / 256));
  const bool wide = e.rows >= (1ll << 32);
  void (*err_kernel)(ErrArgs) = L.D == 64 ? (wide ? repair_err_kernel<64, true> : repair_err_kernel<64, false>)
                                          : (wide ? repair_err_kernel<128, true> : repair_err_kernel<128, false>);
  hipLaunchKernelGGL(err_kernel, grid, dim3(256), 0, st, e);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  SelArgs a;
  a.kbias = kbias;
  a.idx = idx;
  a.k = e.k;
  a.v = e.v;
  a.k_sb = L.k_sb; a.k_ss = L.k_ss; a.k_sh = L.k_sh;
  a.v_sb = L.v_sb; a.v_ss = L.v_ss; a.v_sh = L.v_sh;
  a.rope = e.rope;
  a.kn = L.k_norm;
  a.eps = L.norm_eps;
  a.kr = static_cast<bf16 *>(kr);
  a.vr = static_cast<bf16 *>(vr);
  a.S = L.S;
  a.H = L.H;
  a.n = n;
  a.n_pad = repair_pad(n);
  const size_t lds = (size_t)L.S * 4;
  auto sel = L.D == 64 ? repair_select_kernel<64> : repair_select_kernel<128>;
  if (lds > 64 * 1024) {
    err = hipFuncSetAttribute(reinterpret_cast<const void *>(sel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(sel, dim3((unsigned)(L.B * L.H)), dim3(SEL_NT), lds, st, a);
  return hipGetLastError();
}

}  // namespace ja
