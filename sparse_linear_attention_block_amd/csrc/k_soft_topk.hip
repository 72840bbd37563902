// SoftTop-k of the compressed attention map: the differentiable stand-in for
// Eq. 2's top-k in SLA2's first training stage (SLA2 article, the two-stage
// training paragraphs, stage 1: a sigmoid with a temperature; SLA2 cross-paper
// synthesis, §3: a per-row threshold lambda_i found by binary search so that
// the row meets its budget). For a row of logits s:
//   Pc = softmax(s),  M[j] = sigmoid((Pc[j] - lambda) / tau),  sum_j M[j] = k.
//
// One wave per row, four rows per workgroup. Lane l holds columns l + 64 e
// (e < E, E the smallest instantiated width with 64 E >= cols) in registers for
// the whole search, so the row is read from HBM once and written once. Pc is
// formed from the float64 logits (max and differences in float64, the
// exponential and everything after it in float32). The bracket starts 60 tau
// beyond the row's extremes (every term saturates to 1 or 0 in float32) and is
// halved until its float32 midpoint stops moving. Each row sum is reduced
// across the wave in a fixed order that leaves the same value in every lane,
// so every lane makes the same decision and the search stays uniform.
#include "sla_internal.h"
#include "dev_common.h"

namespace sla {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

// sigmoid(x) from y = -x log2(e): 1 / (1 + 2^y). For very negative x the
// exponential overflows to +inf, whose reciprocal is the exact 0.
__device__ __forceinline__ float sigmoid_l2(float y) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(y));
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}

__device__ __forceinline__ float lane_value(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Sum over the wave, the same value in every lane. Within each row of 16
// lanes the partial sums meet through DPP moves (quad permutations for lane
// distances 1 and 2, then the half-row and row mirrors for 4 and 8), which
// leave every lane of a row holding the same bits (each step adds two values
// that both partners hold, and addition commutes); the four row sums are then
// read from lanes 0, 16, 32 and 48 and added in that order.
__device__ __forceinline__ float wave_sum_uniform(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v += dpp<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v += dpp<0x141>(v);  // row_half_mirror
  v += dpp<0x140>(v);  // row_mirror
  const float t = ((lane_value(v, 0) + lane_value(v, 16)) + lane_value(v, 32)) + lane_value(v, 48);
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(t)));
}

template <int E>
__global__ __launch_bounds__(256) void k_soft_topk(const double* __restrict__ lg, int rows, int cols,
                                                   float k, float tau, float* __restrict__ out,
                                                   float* __restrict__ lam) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;  // wave-uniform
  const double* src = lg + (size_t)row * cols;
  float* dst = out + (size_t)row * cols;
  double s[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = lane + 64 * e;
    s[e] = j < cols ? src[j] : -INFINITY;
  }
  double m = s[0];
#pragma unroll
  for (int e = 1; e < E; ++e) m = fmax(m, s[e]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmax(m, __shfl_xor(m, o));
  float p[E];
  float z = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    // columns past the row have s = -inf: their exponential is 0
    p[e] = __builtin_amdgcn_exp2f((float)(s[e] - m) * kLog2e);
    z += p[e];
  }
  const float iz = 1.0f / wave_sum_uniform(z);
  float pmin = INFINITY, pmax = -INFINITY;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    p[e] *= iz;
    if (lane + 64 * e < cols) {
      pmin = fminf(pmin, p[e]);
      pmax = fmaxf(pmax, p[e]);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    pmin = fminf(pmin, __shfl_xor(pmin, o));
    pmax = fmaxf(pmax, __shfl_xor(pmax, o));
  }
  // columns past the row become -inf: their sigmoid is exactly 0, so the
  // search needs no per-column test
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (lane + 64 * e >= cols) p[e] = -INFINITY;
  if (!(k > 0.f) || k >= (float)cols) {  // the whole row is out, or in
    const float v = k > 0.f ? 1.0f : 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (lane + 64 * e < cols) dst[lane + 64 * e] = v;
    if (lam && lane == 0) lam[row] = k > 0.f ? -INFINITY : INFINITY;
    return;
  }
  const float c = -kLog2e / tau;  // sigmoid((p - mid) / tau) = sigmoid_l2((p - mid) c)
  float lo = pmin - 60.0f * tau, hi = pmax + 60.0f * tau;
  for (int n = 0; n < 256; ++n) {  // ends when the midpoint stops moving, or after 256 halvings
    const float mid = 0.5f * (lo + hi);
    if (!(mid > lo && mid < hi)) break;
    float sp = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) sp += sigmoid_l2((p[e] - mid) * c);
    if (wave_sum_uniform(sp) > k)
      lo = mid;
    else
      hi = mid;
  }
  const float l = 0.5f * (lo + hi);
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (lane + 64 * e < cols) dst[lane + 64 * e] = sigmoid_l2((p[e] - l) * c);
  if (lam && lane == 0) lam[row] = l;
}

}  // namespace

hipError_t launch_soft_topk(const double* logits, int rows, int cols, float k, float tau, float* out,
                            float* lambda, hipStream_t s) {
  const dim3 grid((rows + 3) / 4), block(256);
#define SLA_SOFT_TOPK(EE)                                                                     \
  hipLaunchKernelGGL(k_soft_topk<EE>, grid, block, 0, s, logits, rows, cols, k, tau, out, lambda)
  // columns per lane: the smallest instantiated width that holds the row
  // (padding lanes still evaluate, so the widths are spaced finely)
  const int need = (cols + 63) / 64;
  if (need <= 1)
    SLA_SOFT_TOPK(1);
  else if (need <= 2)
    SLA_SOFT_TOPK(2);
  else if (need <= 4)
    SLA_SOFT_TOPK(4);
  else if (need <= 6)
    SLA_SOFT_TOPK(6);
  else if (need <= 8)
    SLA_SOFT_TOPK(8);
  else if (need <= 12)
    SLA_SOFT_TOPK(12);
  else if (need <= 16)
    SLA_SOFT_TOPK(16);
  else if (need <= 20)
    SLA_SOFT_TOPK(20);
  else if (need <= 24)
    SLA_SOFT_TOPK(24);
  else if (need <= 32)
    SLA_SOFT_TOPK(32);
  else if (need <= 48)
    SLA_SOFT_TOPK(48);
  else if (need <= 64)
    SLA_SOFT_TOPK(64);
  else
    return hipErrorInvalidValue;
#undef SLA_SOFT_TOPK
  return hipGetLastError();
}

}  // namespace sla
