// K1: router projection and 64-token mean pooling of Q and K.
//
// SLA paper summary (aipaper.cc), section 4 step 1 and Eq. 1: pool(.) averages
// along the sequence inside each block; SLA2 article (mcffsbgs.com), router
// paragraph: two learned projection matrices act on Q and K first. Pooling is
// linear, so pool(X proj) = pool(X) proj: the block means are formed first
// (N*d adds, a pure stream over Q and K) and only the Nb means are projected
// (Nb*d*d multiply-adds). Everything is accumulated in float64 so that the
// ranking that follows is decided in the same precision as the float64
// definition.
//
// k_pool_sum: grid (ceil(Nb/2), B*H, 2), z = 0 for Q and 1 for K; each
//   workgroup sums 2 blocks with every 16-byte load of a thread issued before
//   the first add; the means go to raw[z][bh][block][d] (the 8-bit sparse
//   branch also takes its per-head channel means of Q and K from them).
// k_pool_proj: grid (ceil(Nb/64), B*H, 2); float64 MFMA 16x16x4 against the
//   head's router matrix (f32 [in][out], staged in LDS), 16 block means per wave.
#include "sla_internal.h"
#include "dev_common.h"

namespace sla {
namespace {

constexpr int kG = 2;      // blocks per summing workgroup
constexpr int kPR = 64;    // block means per projecting workgroup (16 per wave)

template <typename T>
__device__ __forceinline__ void add_chunk(const uint4& v, double* acc);

template <>
__device__ __forceinline__ void add_chunk<uint16_t>(const uint4& v, double* acc) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    acc[2 * e] += (double)bf_lo(w[e]);
    acc[2 * e + 1] += (double)bf_hi(w[e]);
  }
}

template <>
__device__ __forceinline__ void add_chunk<float>(const uint4& v, double* acc) {
  acc[0] += (double)__uint_as_float(v.x);
  acc[1] += (double)__uint_as_float(v.y);
  acc[2] += (double)__uint_as_float(v.z);
  acc[3] += (double)__uint_as_float(v.w);
}

template <typename T>
__global__ __launch_bounds__(256) void k_pool_sum(const T* __restrict__ Q, const T* __restrict__ K,
                                                  double* __restrict__ raw, int N, int d, int Nb,
                                                  int BH) {
  constexpr int E = 16 / sizeof(T);           // elements per 16-byte chunk
  __shared__ double part[kG][4096 / sizeof(T)];  // row groups x d partial sums per block
  const int tid = threadIdx.x;
  const int z = blockIdx.z, bh = blockIdx.y;
  const T* X = (z ? K : Q) + (size_t)bh * N * d;
  const int C = d / E, RG = 256 / C, RPT = kBlock / RG;  // rows per thread per block
  const int c = tid % C, rg = tid / C;
  const int blk0 = blockIdx.x * kG;
  uint4 v[kG][8];  // at most 8 rows per thread (f32, d = 128)
#pragma unroll
  for (int b = 0; b < kG; ++b)
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int t = (blk0 + b) * kBlock + rg + RG * u;
      v[b][u] = (u < RPT && blk0 + b < Nb && t < N)
                    ? *reinterpret_cast<const uint4*>(X + (size_t)t * d + c * E)
                    : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
  for (int b = 0; b < kG; ++b) {
    double acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = 0.0;
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (u < RPT) add_chunk<T>(v[b][u], acc);
#pragma unroll
    for (int e = 0; e < E; ++e) part[b][rg * d + c * E + e] = acc[e];
  }
  __syncthreads();
  for (int o = tid; o < kG * d; o += 256) {
    const int b = o / d, col = o % d, blk = blk0 + b;
    if (blk >= Nb) continue;
    double sum = 0.0;
    for (int u = 0; u < RG; ++u) sum += part[b][u * d + col];
    const int cnt = min(kBlock, N - blk * kBlock);
    raw[(((size_t)z * BH + bh) * Nb + blk) * d + col] = sum / (double)cnt;
  }
}

// pooled[row][col] = sum_k raw[row][k] * P[k][col] on float64 MFMA 16x16x4:
// wave w of a workgroup owns 16 consecutive block means; the head's router
// matrix (f32 [in][out]) is staged once in LDS and widened to f64 per operand.
__global__ __launch_bounds__(256) void k_pool_proj(const double* __restrict__ raw,
                                                   const float* __restrict__ proj_q,
                                                   const float* __restrict__ proj_k, int proj_hs,
                                                   double* __restrict__ pq, double* __restrict__ pk,
                                                   int H, int d, int Nb, int BH) {
  __shared__ __attribute__((aligned(16))) float P[128 * 128];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int z = blockIdx.z, bh = blockIdx.y;
  const float* Pg = (z ? proj_k : proj_q) + (size_t)(bh % H) * proj_hs;
  for (int x = tid * 4; x < d * d; x += 1024)
    *reinterpret_cast<float4*>(&P[x]) = *reinterpret_cast<const float4*>(Pg + x);
  __syncthreads();
  const int r0 = blockIdx.x * kPR + 16 * wave;     // first of the wave's 16 rows
  const int row = min(r0 + l16, Nb - 1);           // rows past Nb are never stored
  const double* src = raw + (((size_t)z * BH + bh) * Nb + row) * d;
  typedef double f64x4 __attribute__((__vector_size__(4 * sizeof(double))));
  f64x4 acc[8];
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) acc[ct] = f64x4{0.0, 0.0, 0.0, 0.0};
  const int nct = d / 16;
  for (int ks = 0; ks < d / 4; ++ks) {
    const double a = src[4 * ks + g];              // A[row l16][k = 4ks + g]
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      if (ct < nct) {
        const double b = (double)P[(4 * ks + g) * d + 16 * ct + l16];  // B[k][col]
        acc[ct] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, acc[ct], 0, 0, 0);
      }
    }
  }
  double* out = (z ? pk : pq) + ((size_t)bh * Nb) * d;
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) {
    if (ct >= nct) continue;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = r0 + g + 4 * e;                // f64 16x16 layout: D[g + 4e][l16]
      if (r < Nb) out[(size_t)r * d + 16 * ct + l16] = acc[ct][e];
    }
  }
}

}  // namespace

hipError_t launch_pool_sum(const Dims& D, const void* Q, const void* K, double* raw,
                           hipStream_t s) {
  dim3 g1((D.Nb + kG - 1) / kG, D.BH, 2);
  if (D.bf16)
    hipLaunchKernelGGL(k_pool_sum<uint16_t>, g1, dim3(256), 0, s, (const uint16_t*)Q,
                       (const uint16_t*)K, raw, D.N, D.d, D.Nb, D.BH);
  else
    hipLaunchKernelGGL(k_pool_sum<float>, g1, dim3(256), 0, s, (const float*)Q, (const float*)K,
                       raw, D.N, D.d, D.Nb, D.BH);
  return hipGetLastError();
}

hipError_t launch_pool_proj(const Dims& D, const void* Q, const void* K, const float* proj_q,
                            const float* proj_k, int proj_hs, double* raw, double* pq, double* pk,
                            hipStream_t s) {
  hipError_t e = launch_pool_sum(D, Q, K, raw, s);
  if (e != hipSuccess) return e;
  dim3 g2((D.Nb + kPR - 1) / kPR, D.BH, 2);
  hipLaunchKernelGGL(k_pool_proj, g2, dim3(256), 0, s, raw, proj_q, proj_k, proj_hs, pq, pk, D.H,
                     D.d, D.Nb, D.BH);
  return hipGetLastError();
}

}  // namespace sla
