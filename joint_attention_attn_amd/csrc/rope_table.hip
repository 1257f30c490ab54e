// 2D-axial RoPE table: (cos, sin) of every pair angle of every token.
//
// RoPE sits in the QKV projection epilogue of the DiT ("Speed Up Image
// Generation with FLUX 3 Image Klein on NVIDIA Blackwell GPUs", section "GEMM
// kernel optimization"); the image tokens carry a 2-D latent-grid position.
// Pair p < D/4 turns by the token's row, pair p >= D/4 by its column, with
// frequency w_k = theta^(-4k/D) (k = p mod D/4): the 1-D rotary embedding of
// dimension D/2 on each axis.  Angles, cos and sin are evaluated and kept in
// fp64, the precision in which the kernels rotate Q and K.  The table
// ([S][D/2] double2, 16 bytes per pair) is built once per forward pass.
#include "common.hpp"
#include "internal.hpp"

namespace ja {

// The D/4 frequencies are computed once per workgroup (fp64 pow is the most
// expensive step); every entry then takes one fp64 product and one sincos
// (a shared argument reduction for the cosine and the sine).  The threads
// past the per-token table fill the coordinate table (ctab), where the
// coordinate c takes the place of the token's position.
__global__ __launch_bounds__(256) void rope_table_2d_kernel(
    const int32_t *__restrict__ pos, int S, int D, double theta,
    double2 *__restrict__ table, double2 *__restrict__ ctab) {
  __shared__ double freq[32];                 // D/4 <= 32
  const int half = D / 2, quarter = D / 4;
  if ((int)threadIdx.x < quarter) freq[threadIdx.x] = pow(theta, (double)(-4 * (int)threadIdx.x) / (double)D);
  __syncthreads();
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n_tok = (int64_t)S * half;
  int32_t coord;
  int k;
  if (idx < n_tok) {
    const int p = (int)(idx % half);
    const int64_t s = idx / half;
    const int axis = p / quarter;
    k = p - axis * quarter;
    coord = pos[2 * s + axis];
  } else {
    const int64_t j = idx - n_tok;
    if (!ctab || j >= (int64_t)kCoordTableN * quarter) return;
    k = (int)(j % quarter);
    coord = (int32_t)(j / quarter);
  }
  const double ang = (double)coord * freq[k];
  double sn, cs;
  sincos(ang, &sn, &cs);
  if (idx < n_tok)
    table[idx] = make_double2(cs, sn);
  else
    ctab[idx - n_tok] = make_double2(cs, sn);
}

hipError_t launch_rope_table_2d(const int32_t *pos, int S, int D, float theta,
                                double *table, double *ctab, hipStream_t st) {
  const int64_t n = (int64_t)S * (D / 2) + (ctab ? (int64_t)kCoordTableN * (D / 4) : 0);
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(rope_table_2d_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     st, pos, S, D, (double)theta,
                     reinterpret_cast<double2 *>(table), reinterpret_cast<double2 *>(ctab));
  return hipGetLastError();
}

}  // namespace ja
