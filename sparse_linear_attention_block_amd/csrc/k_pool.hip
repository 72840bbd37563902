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
// k_pool_proj: grid (ceil(Nb/64), B*H, 2 * d/64); float64 MFMA 16x16x4
//   against the head's router matrix (f32 [in][out]), 64 block means and a
//   64-column slice of the matrix (staged in LDS) per workgroup.
#include "sla_internal.h"
#include "dev_common.h"

namespace sla {
namespace {

constexpr int kG = 2;      // blocks per summing workgroup

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

template <typename T, int d>
__global__ __launch_bounds__(256) void k_pool_sum(const T* __restrict__ Q, const T* __restrict__ K,
                                                  double* __restrict__ raw, int N, int Nb, int BH) {
  constexpr int E = 16 / sizeof(T);           // elements per 16-byte chunk
  constexpr int C = d / E, RG = 256 / C, RPT = kBlock / RG;  // rows per thread per block
  // partial sums per block: row group rg, feature c E + e at rg (d + 16) + e C + c, so
  // that the lanes of a row group write one e of consecutive c side by side and
  // consecutive row groups fall 128 bytes apart in the banks
  constexpr int PS = d + 16;
  __shared__ double part[kG][RG * PS];
  const int tid = threadIdx.x;
  const int z = blockIdx.z, bh = blockIdx.y;
  const T* X = (z ? K : Q) + (size_t)bh * N * d;
  const int c = tid % C, rg = tid / C;
  const int blk0 = blockIdx.x * kG;
  uint4 v[kG][8];  // at most 8 rows per thread (f32, d = 128)
  // every load is issued (rows past N re-read row N - 1) and masked afterwards,
  // so that no branch separates them and one memory latency covers them all
#pragma unroll
  for (int b = 0; b < kG; ++b)
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (u >= RPT) break;  // uniform
      const int t = (blk0 + b) * kBlock + rg + RG * u;
      v[b][u] = *reinterpret_cast<const uint4*>(X + (size_t)min(t, N - 1) * d + c * E);
    }
#pragma unroll
  for (int b = 0; b < kG; ++b)
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int t = (blk0 + b) * kBlock + rg + RG * u;
      if (u >= RPT || t >= N) v[b][u] = make_uint4(0, 0, 0, 0);
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
    for (int e = 0; e < E; ++e) part[b][rg * PS + e * C + c] = acc[e];
  }
  __syncthreads();
  for (int o = tid; o < kG * d; o += 256) {
    // consecutive threads read consecutive positions l = e C + c of feature c E + e
    const int b = o / d, l = o % d, col = (l % C) * E + l / C, blk = blk0 + b;
    if (blk >= Nb) continue;
    double sum = 0.0;
    for (int u = 0; u < RG; ++u) sum += part[b][u * PS + l];
    const int cnt = min(kBlock, N - blk * kBlock);
    raw[(((size_t)z * BH + bh) * Nb + blk) * d + col] = sum / (double)cnt;
  }
}

// pooled[row][col] = sum_k raw[row][k] * P[k][col] on float64 MFMA 16x16x4.
// A workgroup owns 64 block means (wave w rows 16w .. 16w+15) and 64 output
// columns: the router matrix's 64-column slice (f32, all D rows) is staged once
// in LDS with its rows padded to 80 floats, so the four k groups of a B
// fragment (rows 4ks + g) fall 16 banks apart; each wave reads its own means
// straight from global memory (all loads issued before the first product)
// and runs four independent MFMA chains, one per 16-column tile.
template <int D>
__global__ __launch_bounds__(256) void k_pool_proj(const double* __restrict__ raw,
                                                   const float* __restrict__ proj_q,
                                                   const float* __restrict__ proj_k, int proj_hs,
                                                   double* __restrict__ pq, double* __restrict__ pk,
                                                   int H, int Nb, int BH) {
  constexpr int KS = D / 4;        // k steps
  constexpr int CW = 64;           // output columns per workgroup
  constexpr int PS = CW + 16;      // LDS row stride of the slice (floats)
  __shared__ float ps[D * PS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int z = blockIdx.z & 1, c0 = (blockIdx.z >> 1) * CW, bh = blockIdx.y;
  const float* Pg = (z ? proj_k : proj_q) + (size_t)(bh % H) * proj_hs;
  // the slice: D rows x 64 columns as float4, 16 per row
  for (int x = tid; x < D * CW / 4; x += 256) {
    const int r = x / (CW / 4), c4 = x % (CW / 4);
    *reinterpret_cast<float4*>(&ps[r * PS + 4 * c4]) =
        *reinterpret_cast<const float4*>(Pg + (size_t)r * D + c0 + 4 * c4);
  }
  const int r0 = blockIdx.x * 64 + 16 * wave;
  const int row = min(r0 + l16, Nb - 1);           // rows past Nb are never stored
  const double* src = raw + (((size_t)z * BH + bh) * Nb + row) * D;
  double a[KS];                                    // A[row l16][k = 4ks + g]
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) a[ks] = src[4 * ks + g];
  __syncthreads();
  typedef double f64x4 __attribute__((__vector_size__(4 * sizeof(double))));
  f64x4 acc[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) acc[ct] = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
      acc[ct] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[ks], (double)ps[(4 * ks + g) * PS + 16 * ct + l16],
                                                     acc[ct], 0, 0, 0);
  double* out = (z ? pk : pq) + ((size_t)bh * Nb) * D;
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = r0 + g + 4 * e;                // f64 16x16 layout: D[g + 4e][l16]
      if (r < Nb) out[(size_t)r * D + c0 + 16 * ct + l16] = acc[ct][e];
    }
}

}  // namespace

hipError_t launch_pool_sum(const Dims& D, const void* Q, const void* K, double* raw,
                           hipStream_t s) {
  dim3 g1((D.Nb + kG - 1) / kG, D.BH, 2);
  if (D.bf16 && D.d == 128)
    hipLaunchKernelGGL((k_pool_sum<uint16_t, 128>), g1, dim3(256), 0, s, (const uint16_t*)Q,
                       (const uint16_t*)K, raw, D.N, D.Nb, D.BH);
  else if (D.bf16)
    hipLaunchKernelGGL((k_pool_sum<uint16_t, 64>), g1, dim3(256), 0, s, (const uint16_t*)Q,
                       (const uint16_t*)K, raw, D.N, D.Nb, D.BH);
  else if (D.d == 128)
    hipLaunchKernelGGL((k_pool_sum<float, 128>), g1, dim3(256), 0, s, (const float*)Q,
                       (const float*)K, raw, D.N, D.Nb, D.BH);
  else
    hipLaunchKernelGGL((k_pool_sum<float, 64>), g1, dim3(256), 0, s, (const float*)Q,
                       (const float*)K, raw, D.N, D.Nb, D.BH);
  return hipGetLastError();
}

hipError_t launch_pool_proj(const Dims& D, const float* proj_q, const float* proj_k, int proj_hs,
                            const double* raw, double* pq, double* pk, hipStream_t s) {
  dim3 g2((D.Nb + 63) / 64, D.BH, 2 * (D.d / 64));  // z: (column slice, Q or K)
  if (D.d == 128)
    hipLaunchKernelGGL(k_pool_proj<128>, g2, dim3(256), 0, s, raw, proj_q, proj_k, proj_hs, pq, pk,
                       D.H, D.Nb, D.BH);
  else
    hipLaunchKernelGGL(k_pool_proj<64>, g2, dim3(256), 0, s, raw, proj_q, proj_k, proj_hs, pq, pk,
                       D.H, D.Nb, D.BH);
  return hipGetLastError();
}

}  // namespace sla
