// Microbenchmark of the bf16 forward's per-tile instruction chain on gfx950,
// without HBM traffic: what rate the chip sustains for the same mix of
// matrix, vector and LDS work under its power limit.
//
// One workgroup of 12 wave64s per CU (three waves per SIMD, as in the bf16
// forward); each wave runs NTILE iterations of one 32-key tile for 32 query
// rows at D = 128:
//   Q K^T : 8 x v_mfma_f32_32x32x16_bf16, A = K fragments, B = Q (registers)
//   softmax-shaped vector work on the 16 scores per lane: row max (with the
//           cross-half exchange), 16 FMAs, 16 exp2, the row sum, 8 packs to
//           bf16 (the fast path of the forward's softmax)
//   P.V   : 8 x v_mfma_f32_32x32x16_bf16, A = V^T fragments, B = P
// Variants: K/V fragments from registers or from LDS (16 x ds_read_b128 per
// tile, three stages of pseudo-random bf16 cycled tile by tile, so operands
// change as they do on real data); with or without a workgroup barrier per
// tile; and MFMA only (no vector work).
//
// Reported per variant: TFLOP/s over the launch (HIP events), the mean
// shader clock of the waves (clock64 against the 100 MHz wall clock), and
// the MFMA utilisation at that clock (rate / (1024 SIMDs x clock x 1024 flop
// per cycle)).  Every LDS address stays inside the workgroup's array, and every
// loop has a fixed trip count.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <vector>

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 12;
constexpr int kThreads = 64 * kWaves;
constexpr int kKBytes = 32 * 272;        // K tile: 32 rows of 128 bf16 + a 16-byte pad
constexpr int kStage = kKBytes + 8192;   // + V^T tile: 128 rows of 32 keys
constexpr int kNStage = 3;

__device__ __forceinline__ unsigned pack2(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
}

// bf16 pair with random sign and mantissa, magnitude in [0.5, 2)
__device__ __forceinline__ unsigned rand_pair(unsigned i) {
  unsigned x = i * 2654435761u;
  x ^= x >> 15;
  x *= 2246822519u;
  x ^= x >> 13;
  return (x & 0x807f807fu) | 0x3f003f00u | ((x >> 7) & 0x00800080u);
}

template <bool LDS, bool BARRIER, bool SOFTMAX>
__global__ __launch_bounds__(kThreads, 1) void chain_kernel(float *out, long long *clk, int ntile) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[kNStage * kStage];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < kNStage * kStage / 16; i += kThreads) {
    const unsigned b = 4u * (unsigned)(i + 4096 * blockIdx.x);
    reinterpret_cast<u32x4 *>(lds)[i] = u32x4{rand_pair(b), rand_pair(b + 1), rand_pair(b + 2), rand_pair(b + 3)};
  }
  __syncthreads();
  bf16x8 q[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const unsigned b = 4u * (unsigned)(tid * 8 + k) + 977u;
    q[k] = __builtin_bit_cast(bf16x8, u32x4{rand_pair(b), rand_pair(b + 1), rand_pair(b + 2), rand_pair(b + 3)});
  }
  f32x16 o[4];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[d][i] = 0.f;
  float m = -1e30f, l = 0.f;
  // K rows of 272 bytes (the forward's padded rows); V^T rows of 64 bytes
  // with 16-byte granule g of row d at g ^ ((d / 4) % 4), the forward's
  // swizzle (d % 32 is lane % 32 for every fragment of a lane)
  const int koff = (lane & 31) * 272 + (lane >> 5) * 16;
  const int vswz = ((lane & 31) >> 2) & 3;
  auto voff = [&](int k) { return kKBytes + ((lane & 31) + 32 * (k & 3)) * 64 + 16 * ((2 * (k >> 2) + (lane >> 5)) ^ vswz); };
  const long long w0 = wall_clock64(), c0 = clock64();
  for (int t = 0; t < ntile; ++t) {
    const int st = (t % kNStage) * kStage;
    bf16x8 kf[8], vf[8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      kf[k] = LDS ? *reinterpret_cast<const bf16x8 *>(lds + st + koff + 32 * k) : q[k ^ 1];
    f32x16 s;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[k], q[k], s, 0, 0, 0);
    bf16x8 pb[2];
    if (SOFTMAX) {
      float mx = s[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mn = fmaxf(m, mx * 0.18f);
      float ps = 0.f;
      unsigned pk[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * i], 0.18f, -mn));
        const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * i + 1], 0.18f, -mn));
        ps += e0 + e1;
        pk[i] = pack2(e0, e1);
      }
      m = mn;
      l += ps;
      pb[0] = __builtin_bit_cast(bf16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});
      pb[1] = __builtin_bit_cast(bf16x8, u32x4{pk[4], pk[5], pk[6], pk[7]});
    } else {
      pb[0] = (t & 1) ? q[2] : q[0];
      pb[1] = (t & 1) ? q[3] : q[1];
      l += s[0];
    }
#pragma unroll
    for (int k = 0; k < 8; ++k)
      vf[k] = LDS ? *reinterpret_cast<const bf16x8 *>(lds + st + voff(k))
                  : q[k ^ 2];
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
        o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[2 * d + kk], pb[kk], o[d], 0, 0, 0);
    if (BARRIER) __syncthreads();
  }
  const long long c1 = clock64(), w1 = wall_clock64();
  float acc = l;
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc += o[d][i];
  out[(int64_t)blockIdx.x * kThreads + tid] = acc;
  if (lane == 0) {
    long long *r = clk + 3 * ((int64_t)blockIdx.x * kWaves + wave);
    r[0] = c1 - c0;
    r[1] = w0;
    r[2] = w1;
  }
}

bool check(hipError_t e, const char *what) {
  if (e != hipSuccess) fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
  return e == hipSuccess;
}

template <bool LDS, bool BARRIER, bool SOFTMAX>
bool run(const char *name, int nblk, int ntile, float *out, long long *clk, double wall_mhz) {
  auto launch = [&] {
    hipLaunchKernelGGL((chain_kernel<LDS, BARRIER, SOFTMAX>), dim3(nblk), dim3(kThreads), 0, 0, out, clk, ntile);
    return hipGetLastError();
  };
  if (!check(launch(), "launch") || !check(hipDeviceSynchronize(), "sync")) return false;
  hipEvent_t e0, e1;
  if (!check(hipEventCreate(&e0), "event") || !check(hipEventCreate(&e1), "event")) return false;
  float ms = 0.f;
  if (!check(hipEventRecord(e0, 0), "record") || !check(launch(), "launch") ||
      !check(hipEventRecord(e1, 0), "record") || !check(hipEventSynchronize(e1), "sync") ||
      !check(hipEventElapsedTime(&ms, e0, e1), "elapsed"))
    return false;
  std::vector<long long> r((size_t)nblk * kWaves * 3);
  if (!check(hipMemcpy(r.data(), clk, r.size() * sizeof(long long), hipMemcpyDeviceToHost), "copy"))
    return false;
  double cyc = 0.0, wall = 0.0;
  for (size_t i = 0; i < r.size(); i += 3) {
    cyc += (double)r[i];
    wall += (double)(r[i + 2] - r[i + 1]);
  }
  const double ghz = cyc / (wall / wall_mhz) / 1e3;
  const double flops = (double)nblk * kWaves * ntile * 16 * 32768.0;
  const double tflops = flops / ms / 1e9;
  const double util = tflops * 1e12 / (1024.0 * ghz * 1e9 * 1024.0);
  printf("%-34s %7.0f TFLOP/s  shader clock %.2f GHz  MFMA utilisation %5.1f %%  (%.3f ms)\n", name,
         tflops, ghz, 100.0 * util, ms);
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  return true;
}

}  // namespace

int main() {
  int cus = 0, wclk = 0;
  if (!check(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0), "attr") ||
      !check(hipDeviceGetAttribute(&wclk, hipDeviceAttributeWallClockRate, 0), "attr"))
    return 1;
  const int nblk = cus, ntile = 4096;
  const double wall_mhz = wclk / 1000.0;
  printf("%d CUs, wall clock %.0f MHz; %d workgroups of %d waves, %d tiles per wave\n", cus, wall_mhz, nblk,
         kWaves, ntile);
  float *out = nullptr;
  long long *clk = nullptr;
  if (!check(hipMalloc(&out, (size_t)nblk * kThreads * sizeof(float)), "malloc") ||
      !check(hipMalloc(&clk, (size_t)nblk * kWaves * 3 * sizeof(long long)), "malloc"))
    return 1;
  const bool ok = run<false, false, false>("MFMA only, operands in registers", nblk, ntile, out, clk, wall_mhz) &&
                  run<true, false, false>("MFMA only, K/V from LDS", nblk, ntile, out, clk, wall_mhz) &&
                  run<false, false, true>("chain, operands in registers", nblk, ntile, out, clk, wall_mhz) &&
                  run<true, false, true>("chain, K/V from LDS", nblk, ntile, out, clk, wall_mhz) &&
                  run<true, true, true>("chain, K/V from LDS, barrier per tile", nblk, ntile, out, clk, wall_mhz);
  (void)hipFree(out);
  (void)hipFree(clk);
  return ok ? 0 : 1;
}
