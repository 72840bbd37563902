// K1: router projection and 64-token mean pooling of Q and K.
//
// SLA paper summary (aipaper.cc), section 4 step 1 and Eq. 1: pool(.) averages
// along the sequence inside each block; SLA2 article (mcffsbgs.com), router
// paragraph: two learned projection matrices act on Q and K first. Pooling is
// linear, so pool(X proj) = pool(X) proj: this kernel pools first (N*d adds)
// and projects the Nb block means (Nb*d*d multiply-adds) instead of projecting
// all N tokens. Everything is accumulated in float64 so that the ranking that
// follows is decided in the same precision as the float64 definition.
//
// Grid (ceil(Nb/8), B*H, 2): z = 0 pools Q with proj_q, z = 1 pools K with
// proj_k. 256 threads read 8 consecutive blocks (512 tokens, contiguous in
// HBM) with 16-byte loads; the block means go through LDS to the projection.
#include "sla_internal.h"
#include "dev_common.h"

namespace sla {
namespace {

constexpr int kG = 8;  // blocks per workgroup

template <typename T>
__device__ __forceinline__ void load_chunk(const T* p, double* out);

template <>
__device__ __forceinline__ void load_chunk<uint16_t>(const uint16_t* p, double* out) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    out[2 * e] = (double)bf_lo(w[e]);
    out[2 * e + 1] = (double)bf_hi(w[e]);
  }
}

template <>
__device__ __forceinline__ void load_chunk<float>(const float* p, double* out) {
  const float4 v = *reinterpret_cast<const float4*>(p);
  out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
}

template <typename T>
__global__ __launch_bounds__(256) void k_pool_proj(const T* __restrict__ Q, const T* __restrict__ K,
                                                   const float* __restrict__ proj_q,
                                                   const float* __restrict__ proj_k, int proj_hs,
                                                   double* __restrict__ pq, double* __restrict__ pk,
                                                   int H, int N, int d, int Nb) {
  constexpr int E = 16 / sizeof(T);             // elements per 16-byte chunk
  __shared__ double part[4096 / sizeof(T)];     // row groups x d partial sums
  __shared__ double mean[kG * 128];

  const int tid = threadIdx.x;
  const bool isk = blockIdx.z != 0;
  const int bh = blockIdx.y;
  const T* X = (isk ? K : Q) + (size_t)bh * N * d;
  const float* P = (isk ? proj_k : proj_q) + (size_t)(bh % H) * proj_hs;
  double* out = (isk ? pk : pq) + (size_t)bh * Nb * d;

  const int C = d / E;        // chunks per row
  const int RG = 256 / C;     // row groups
  const int c = tid % C, rg = tid / C;
  const int blk0 = blockIdx.x * kG;

  for (int g = 0; g < kG; ++g) {
    const int blk = blk0 + g;
    if (blk >= Nb) break;
    double acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.0;
    for (int r = rg; r < kBlock; r += RG) {
      const int t = blk * kBlock + r;
      if (t < N) {
        double v[E];
        load_chunk<T>(X + (size_t)t * d + c * E, v);
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] += v[e];
      }
    }
#pragma unroll
    for (int e = 0; e < E; ++e) part[rg * d + c * E + e] = acc[e];
    __syncthreads();
    if (tid < d) {
      double s = 0.0;
      for (int u = 0; u < RG; ++u) s += part[u * d + tid];
      const int cnt = min(kBlock, N - blk * kBlock);
      mean[g * d + tid] = s / (double)cnt;
    }
    __syncthreads();
  }

  // projection of the block means: out[blk][col] = sum_k mean[blk][k] * P[k][col]
  const int col = tid % d, g0 = tid / d, ng = 256 / d;
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  for (int k = 0; k < d; ++k) {
    const double p = (double)P[k * d + col];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int g = g0 + u * ng;
      if (g < kG) acc[u] += mean[g * d + k] * p;
    }
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int g = g0 + u * ng;
    if (g < kG && blk0 + g < Nb) out[(size_t)(blk0 + g) * d + col] = acc[u];
  }
}

}  // namespace

hipError_t launch_pool_proj(const Dims& D, const void* Q, const void* K, const float* proj_q,
                            const float* proj_k, int proj_hs, double* pq, double* pk,
                            hipStream_t s) {
  dim3 grid((D.Nb + kG - 1) / kG, D.BH, 2);
  if (D.bf16)
    hipLaunchKernelGGL(k_pool_proj<uint16_t>, grid, dim3(256), 0, s, (const uint16_t*)Q,
                       (const uint16_t*)K, proj_q, proj_k, proj_hs, pq, pk, D.H, D.N, D.d, D.Nb);
  else
    hipLaunchKernelGGL(k_pool_proj<float>, grid, dim3(256), 0, s, (const float*)Q,
                       (const float*)K, proj_q, proj_k, proj_hs, pq, pk, D.H, D.N, D.d, D.Nb);
  return hipGetLastError();
}

}  // namespace sla
