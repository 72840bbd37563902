// Inputs of the 8-bit sparse branch that depend on K: int8 K with per-block
// scales and the per-key bias of the Q smoothing.
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
//   tokens of each block.
// k_quant_k: grid (Nb, B*H), one 64-token key block per workgroup: K - k̄ in
//   float32, absmax over the block (scale absmax / 127, 1 for an all-zero
//   block), codes round-half-even and clamped to +-127, the bias b per key
//   (stored multiplied by log2(e) / sqrt(d), the unit of the sparse kernel's
//   scores).
//   Rows past N are zero with bias 0. The bytes of a row are stored in the
//   k-slot order of the sparse kernel's int8 16x16x64 product: k step s
//   (64 bytes), lane group g, byte e holds feature 32 (2s + e / 8) + 8g + e % 8,
//   so that the query operand of that product is built from the same 16-byte
//   bf16 loads as the operand of its bf16 linear-branch product.
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

template <int D>
__device__ __forceinline__ float kBiasScale() {
  return 1.4426950408889634f / (D == 128 ? 11.313708498984761f : 8.0f);
}

template <int D>
__global__ __launch_bounds__(256) void k_quant_k(const uint16_t* __restrict__ K,
                                                 const float* __restrict__ qkmean,
                                                 int8_t* __restrict__ k8, float* __restrict__ ksc,
                                                 float* __restrict__ kb, int N, int Nb, int BH) {
  constexpr int CPT = D / 32;  // 16-byte bf16 chunks per thread
  __shared__ float wmax[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = blockIdx.x, bh = blockIdx.y;
  const int r = tid >> 2, qt = tid & 3;  // token r of the block; chunks qt + 4m
  const int t = j * kBlock + r;
  const bool valid = t < N;
  const float* qm = qkmean + (size_t)bh * D;
  const float* km = qkmean + ((size_t)BH + bh) * D;
  float ksm[CPT][8];
  float bias = 0.f, am = 0.f;
#pragma unroll
  for (int m = 0; m < CPT; ++m) {
    const int f0 = 8 * (qt + 4 * m);
    const uint4 w = *reinterpret_cast<const uint4*>(K + ((size_t)bh * N + min(t, N - 1)) * D + f0);
    const uint32_t wv[4] = {w.x, w.y, w.z, w.w};
    const float4 k0 = *reinterpret_cast<const float4*>(km + f0);
    const float4 k1 = *reinterpret_cast<const float4*>(km + f0 + 4);
    const float4 q0 = *reinterpret_cast<const float4*>(qm + f0);
    const float4 q1 = *reinterpret_cast<const float4*>(qm + f0 + 4);
    const float kmv[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
    const float qmv[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = (e & 1) ? bf_hi(wv[e >> 1]) : bf_lo(wv[e >> 1]);
      ksm[m][e] = valid ? x - kmv[e] : 0.f;
      bias = fmaf(qmv[e], ksm[m][e], bias);
      am = fmaxf(am, fabsf(ksm[m][e]));
    }
  }
  bias += __shfl_xor(bias, 1);
  bias += __shfl_xor(bias, 2);
  // stored in the sparse kernel's log2 score units: b * log2(e) / sqrt(d)
  if (qt == 0) kb[((size_t)bh * Nb + j) * kBlock + r] = valid ? bias * kBiasScale<D>() : 0.f;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) am = fmaxf(am, __shfl_xor(am, o));
  if (lane == 0) wmax[wave] = am;
  __syncthreads();
  am = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const float inv = am > 0.f ? 127.0f / am : 1.0f;
  if (tid == 0) ksc[(size_t)bh * Nb + j] = am > 0.f ? am / 127.0f : 1.0f;
  int8_t* dst = k8 + (((size_t)bh * Nb + j) * kBlock + r) * D;
#pragma unroll
  for (int m = 0; m < CPT; ++m) {
    uint32_t o[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int c0 = q_i8(ksm[m][4 * hh], inv), c1 = q_i8(ksm[m][4 * hh + 1], inv);
      const int c2 = q_i8(ksm[m][4 * hh + 2], inv), c3 = q_i8(ksm[m][4 * hh + 3], inv);
      o[hh] = (uint32_t)(c0 & 0xff) | ((uint32_t)(c1 & 0xff) << 8) | ((uint32_t)(c2 & 0xff) << 16) |
              ((uint32_t)(c3 & 0xff) << 24);
    }
    // chunk qt + 4m holds features 32m + 8qt .. +7: k step m / 2, lane group qt, half m % 2
    *reinterpret_cast<uint2*>(dst + 64 * (m >> 1) + 16 * qt + 8 * (m & 1)) = make_uint2(o[0], o[1]);
  }
}

}  // namespace

hipError_t launch_quant_k(const Dims& D, const void* K, const Work& w, hipStream_t s) {
  if (!D.quant || !D.bf16) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_qk_mean, dim3(D.BH, 2), dim3(1024), 0, s, w.pooled_raw, w.qkmean, D.N, D.d,
                     D.Nb, D.BH);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (D.d == 128)
    hipLaunchKernelGGL(k_quant_k<128>, dim3(D.Nb, D.BH), dim3(256), 0, s, (const uint16_t*)K,
                       w.qkmean, w.k8, w.ks, w.kb, D.N, D.Nb, D.BH);
  else
    hipLaunchKernelGGL(k_quant_k<64>, dim3(D.Nb, D.BH), dim3(256), 0, s, (const uint16_t*)K,
                       w.qkmean, w.k8, w.ks, w.kb, D.N, D.Nb, D.BH);
  return hipGetLastError();
}

}  // namespace sla
