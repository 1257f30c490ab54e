// Microbenchmark of the bf16 forward's per-tile instruction chain on gfx950,
// without HBM traffic: what rate the chip sustains for the same mix of
// matrix, vector and LDS work under its power limit.
//
// One workgroup of NW wave64s per CU; each wave holds NB 32-row query blocks
// and runs NTILE iterations of one 32-key tile at D = 128:
//   Q K^T : 8 x v_mfma_f32_32x32x16_bf16 per block, A = K fragments (each
//           fragment read once and used by all NB blocks), B = Q (registers)
//   softmax-shaped vector work on the 16 scores per lane and block: row max
//           (with the cross-half exchange), 16 FMAs, 16 exp2, the row sum,
//           8 packs to bf16 (the fast path of the forward's softmax)
//   P.V   : 8 x v_mfma_f32_32x32x16_bf16 per block, A = V^T fragments (shared
//           by the blocks), B = P
// Shapes: 12 waves x 1 block (three waves of 32 rows per SIMD) and 8 waves x
// 2 blocks (two waves of 64 rows per SIMD, the bf16 forward's shape, which
// reads half the LDS bytes per MFMA flop).  Variants: K/V fragments from
// registers or from LDS (16 x ds_read_b128 per tile, three stages of
// pseudo-random bf16 cycled tile by tile, so operands change as they do on
// real data); with or without a workgroup barrier per tile; and MFMA only
// (no vector work).
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

constexpr int kMaxThreads = 64 * 12;
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

template <int NW, int NB, bool LDS, bool BARRIER, bool SOFTMAX>
__global__ __launch_bounds__(64 * NW, 1) void chain_kernel(float *out, long long *clk, int ntile) {
  constexpr int kThreads = 64 * NW;
  __shared__ __attribute__((aligned(16))) unsigned char lds[kNStage * kStage];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < kNStage * kStage / 16; i += kThreads) {
    const unsigned b = 4u * (unsigned)(i + 4096 * blockIdx.x);
    reinterpret_cast<u32x4 *>(lds)[i] = u32x4{rand_pair(b), rand_pair(b + 1), rand_pair(b + 2), rand_pair(b + 3)};
  }
  __syncthreads();
  bf16x8 q[NB][8];
#pragma unroll
  for (int r = 0; r < NB; ++r)
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const unsigned b = 4u * (unsigned)((tid * NB + r) * 8 + k) + 977u;
      q[r][k] = __builtin_bit_cast(bf16x8, u32x4{rand_pair(b), rand_pair(b + 1), rand_pair(b + 2), rand_pair(b + 3)});
    }
  f32x16 o[NB][4];
#pragma unroll
  for (int r = 0; r < NB; ++r)
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[r][d][i] = 0.f;
  float m[NB], l[NB];
#pragma unroll
  for (int r = 0; r < NB; ++r) {
    m[r] = -1e30f;
    l[r] = 0.f;
  }
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
      kf[k] = LDS ? *reinterpret_cast<const bf16x8 *>(lds + st + koff + 32 * k) : q[0][k ^ 1];
    f32x16 s[NB];
#pragma unroll
    for (int r = 0; r < NB; ++r)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[r][i] = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int r = 0; r < NB; ++r) s[r] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[k], q[r][k], s[r], 0, 0, 0);
    bf16x8 pb[NB][2];
#pragma unroll
    for (int r = 0; r < NB; ++r) {
      if (SOFTMAX) {
        float mx = s[r][0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[r][i]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mn = fmaxf(m[r], mx * 0.18f);
        float ps = 0.f;
        unsigned pk[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r][2 * i], 0.18f, -mn));
          const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r][2 * i + 1], 0.18f, -mn));
          ps += e0 + e1;
          pk[i] = pack2(e0, e1);
        }
        m[r] = mn;
        l[r] += ps;
        pb[r][0] = __builtin_bit_cast(bf16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});
        pb[r][1] = __builtin_bit_cast(bf16x8, u32x4{pk[4], pk[5], pk[6], pk[7]});
      } else {
        pb[r][0] = (t & 1) ? q[r][2] : q[r][0];
        pb[r][1] = (t & 1) ? q[r][3] : q[r][1];
        l[r] += s[r][0];
      }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k)
      vf[k] = LDS ? *reinterpret_cast<const bf16x8 *>(lds + st + voff(k)) : q[0][k ^ 2];
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int r = 0; r < NB; ++r)
          o[r][d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[2 * d + kk], pb[r][kk], o[r][d], 0, 0, 0);
    if (BARRIER) __syncthreads();
  }
  const long long c1 = clock64(), w1 = wall_clock64();
  float acc = 0.f;
#pragma unroll
  for (int r = 0; r < NB; ++r) {
    acc += l[r];
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc += o[r][d][i];
  }
  out[(int64_t)blockIdx.x * kMaxThreads + tid] = acc;
  if (lane == 0) {
    long long *r = clk + 3 * ((int64_t)blockIdx.x * 12 + wave);
    r[0] = c1 - c0;
    r[1] = w0;
    r[2] = w1;
  }
}

bool check(hipError_t e, const char *what) {
  if (e != hipSuccess) fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
  return e == hipSuccess;
}

template <int NW, int NB, bool LDS, bool BARRIER, bool SOFTMAX>
bool run(const char *name, int nblk, int ntile, float *out, long long *clk, double wall_mhz) {
  auto launch = [&] {
    hipLaunchKernelGGL((chain_kernel<NW, NB, LDS, BARRIER, SOFTMAX>), dim3(nblk), dim3(64 * NW), 0, 0, out, clk,
                       ntile);
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
  std::vector<long long> r((size_t)nblk * 12 * 3);
  if (!check(hipMemcpy(r.data(), clk, r.size() * sizeof(long long), hipMemcpyDeviceToHost), "copy"))
    return false;
  double cyc = 0.0, wall = 0.0;
  for (int b = 0; b < nblk; ++b)
    for (int w = 0; w < NW; ++w) {
      const long long *x = r.data() + 3 * ((size_t)b * 12 + w);
      cyc += (double)x[0];
      wall += (double)(x[2] - x[1]);
    }
  const double ghz = cyc / (wall / wall_mhz) / 1e3;
  const double flops = (double)nblk * NW * NB * ntile * 16 * 32768.0;
  const double tflops = flops / ms / 1e9;
  const double util = tflops * 1e12 / (1024.0 * ghz * 1e9 * 1024.0);
  printf("%-44s %7.0f TFLOP/s  shader clock %.2f GHz  MFMA utilisation %5.1f %%  (%.3f ms)\n", name,
         tflops, ghz, 100.0 * util, ms);
  fflush(stdout);
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
  printf("%d CUs, wall clock %.0f MHz; %d workgroups, 4096 tiles per 32-row block (3072 for 64-row waves)\n",
         cus, wall_mhz, nblk);
  float *out = nullptr;
  long long *clk = nullptr;
  if (!check(hipMalloc(&out, (size_t)nblk * kMaxThreads * sizeof(float)), "malloc") ||
      !check(hipMalloc(&clk, (size_t)nblk * 12 * 3 * sizeof(long long)), "malloc"))
    return 1;
  // the 64-row shape runs 3072 tiles per wave: the same flops per CU
  const bool ok =
      run<12, 1, false, false, false>("12x32 rows: MFMA only, operands in registers", nblk, ntile, out, clk, wall_mhz) &&
      run<12, 1, true, false, false>("12x32 rows: MFMA only, K/V from LDS", nblk, ntile, out, clk, wall_mhz) &&
      run<12, 1, false, false, true>("12x32 rows: chain, operands in registers", nblk, ntile, out, clk, wall_mhz) &&
      run<12, 1, true, false, true>("12x32 rows: chain, K/V from LDS", nblk, ntile, out, clk, wall_mhz) &&
      run<12, 1, true, true, true>("12x32 rows: chain, LDS, barrier per tile", nblk, ntile, out, clk, wall_mhz) &&
      run<8, 2, true, false, false>("8x64 rows: MFMA only, K/V from LDS", nblk, 3 * ntile / 4, out, clk, wall_mhz) &&
      run<8, 2, true, false, true>("8x64 rows: chain, K/V from LDS", nblk, 3 * ntile / 4, out, clk, wall_mhz) &&
      run<8, 2, true, true, true>("8x64 rows: chain, LDS, barrier per tile", nblk, 3 * ntile / 4, out, clk, wall_mhz) &&
      run<12, 1, true, true, true>("12x32 rows: chain, LDS, barrier (again)", nblk, ntile, out, clk, wall_mhz) &&
      run<8, 2, true, true, true>("8x64 rows: chain, LDS, barrier (again)", nblk, 3 * ntile / 4, out, clk, wall_mhz);
  (void)hipFree(out);
  (void)hipFree(clk);
  return ok ? 0 : 1;
}
