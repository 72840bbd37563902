// Channel means of Q and K for the 8-bit sparse branch (the smoothing below);
// the int8 K, its per-block scales and the per-key bias are formed by the h/z
// kernel from the same K rows it reads for phi(K).
//
// SLA2 article (mcffsbgs.com), quantisation-aware paragraph: Q and K enter the
// sparse branch in 8 bits with a scale that is restored after the product.
// Before quantising, both are smoothed by their channel means over the N
// tokens of the head (q̄, k̄):
//     q.k = (q - q̄).(k - k̄) + q̄.(k - k̄) + q.k̄ .
// The last term is the same for every key of a query and cancels in the
// softmax; the middle one is a per-key bias b = q̄.(k - k̄) kept in float32;
// the first is the int8 product. Subtracting the means takes the common
// offset out of the absmax scales, which otherwise costs most of the int8
// resolution on inputs with a large shared component.
//
// k_qk_mean: grid (B*H, 2), the channel means of Q (z = 0) and K (z = 1) from
//   the float64 block means of the pooling kernel, weighted by the valid
//   tokens of each block. It runs before the h/z kernel, which needs them.
#include "sla_internal.h"
#include "dev_common.h"

namespace sla {
namespace {

__global__ __launch_bounds__(1024) void k_qk_mean(const double* __restrict__ raw,
                                                  float* __restrict__ qkmean, int N, int d,
                                                  int Nb, int BH) {
  __shared__ double part[1024];
  const int tid = threadIdx.x;
  const int bh = blockIdx.x, z = blockIdx.y;
  const int RG = 1024 / d, c = tid % d, rg = tid / d;
  const double* src = raw + ((size_t)z * BH + bh) * Nb * d;
  // 8 block means in flight per thread (rows past Nb re-read a valid row, weight 0)
  double s = 0.0;
  for (int j0 = rg; j0 < Nb; j0 += 8 * RG) {
    double v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = src[(size_t)min(j0 + u * RG, Nb - 1) * d + c];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = j0 + u * RG;
      if (j < Nb) s += (double)min(kBlock, N - j * kBlock) * v[u];
    }
  }
  part[tid] = s;
  __syncthreads();
  if (tid < d) {
    double t = 0.0;
    for (int u = 0; u < RG; ++u) t += part[u * d + tid];
    qkmean[((size_t)z * BH + bh) * d + tid] = (float)(t / (double)N);
  }
}

}  // namespace

hipError_t launch_qk_mean(const Dims& D, const Work& w, hipStream_t s) {
  if (!D.quant || !D.bf16) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_qk_mean, dim3(D.BH, 2), dim3(1024), 0, s, w.pooled_raw, w.qkmean, D.N, D.d,
                     D.Nb, D.BH);
  return hipGetLastError();
}

}  // namespace sla
