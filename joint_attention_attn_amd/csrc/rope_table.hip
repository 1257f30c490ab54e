// 2D-axial RoPE table: (cos, sin) of every pair angle of every token.
//
// RoPE sits in the QKV projection epilogue of the DiT ("Speed Up Image
// Generation with FLUX 3 Image Klein on NVIDIA Blackwell GPUs", section "GEMM
// kernel optimization"); the image tokens carry a 2-D latent-grid position.
// Pair p < D/4 turns by the token's row, pair p >= D/4 by its column, with
// frequency w_k = theta^(-4k/D) (k = p mod D/4): the 1-D rotary embedding of
// dimension D/2 on each axis.  Angles, cos and sin are evaluated in fp64 and
// rounded once to fp32.  The table is small ([S][D/2] float2) and is built
// once per forward pass.
#include "common.hpp"
#include "internal.hpp"

namespace ja {

// The D/4 frequencies are computed once per workgroup (fp64 pow is the most
// expensive step); every entry then takes one fp64 product and one sincos
// (a shared argument reduction for the cosine and the sine).
__global__ __launch_bounds__(256) void rope_table_2d_kernel(
    const int32_t *__restrict__ pos, int S, int D, double theta,
    float2 *__restrict__ table) {
  __shared__ double freq[32];                 // D/4 <= 32
  const int half = D / 2, quarter = D / 4;
  if ((int)threadIdx.x < quarter) freq[threadIdx.x] = pow(theta, (double)(-4 * (int)threadIdx.x) / (double)D);
  __syncthreads();
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)S * half) return;
  const int p = (int)(idx % half);
  const int64_t s = idx / half;
  const int axis = p / quarter;
  const int k = p - axis * quarter;
  const double ang = (double)pos[2 * s + axis] * freq[k];
  double sn, cs;
  sincos(ang, &sn, &cs);
  table[idx] = make_float2((float)cs, (float)sn);
}

hipError_t launch_rope_table_2d(const int32_t *pos, int S, int D, float theta,
                                float *table, hipStream_t st) {
  const int64_t n = (int64_t)S * (D / 2);
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(rope_table_2d_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     st, pos, S, D, (double)theta,
                     reinterpret_cast<float2 *>(table));
  return hipGetLastError();
}

}  // namespace ja
