// K4: per-query-block sums of the linear-attention state over marginal blocks.
//
// SLA paper summary (aipaper.cc), Eq. 3: H_i = sum over j with Mc[i, j] = 0 of
// phi(K_j)^T V_j and Z_i = sum of rowsum(phi(K_j)^T) over the same j. For all
// query blocks of one (batch, head) at once this is one matrix product
//     Hx[i][n] = sum_j M01[i][j] * hx[j][n],   M01[i][j] = (Mc[i][j] == 0),
// with n running over the d*d entries of h_j^T and the d entries of z_j. The
// 0/1 matrix is exact in bf16, so the product runs on MFMA 16x16x32 (bf16 in,
// f32 accumulate) and costs 2*Nb*Nb*(d*d + d) flops per head instead of a
// gather of (n_h + n_l) d x d blocks per query block from cache.
//
// The kernel computes the transpose Hx^T = hx^T M01^T: the hx operand has 4
// consecutive key blocks per 8-byte word (written so by K3), which is the k
// layout the MFMA A operand needs; the mask tile is turned into bf16 0/1 once
// per workgroup in LDS and read as the B operand; each lane then holds 4
// consecutive n of one query block and stores them as one 8-byte word.
//
// Workgroup tile: 256 n x 128 query blocks, 4 waves of 64 n x 128 i each,
// k steps of 32 key blocks, LDS double-buffered mask tiles.
#include "sla_internal.h"
#include "dev_common.h"

namespace sla {
namespace {

constexpr int kTN = 256;  // n per workgroup
constexpr int kTI = 128;  // query blocks per workgroup
constexpr int kMS = 40;   // LDS row stride of the mask tile (bf16 elements)

__global__ __launch_bounds__(256) void k_linear_bf16(const int8_t* __restrict__ mask,
                                                     const uint16_t* __restrict__ hx,
                                                     uint16_t* __restrict__ Hx, int Nb, int Nbp,
                                                     int NN) {
  __shared__ __attribute__((aligned(16))) uint16_t ms[2][kTI][kMS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int bh = blockIdx.z;
  const int i0 = blockIdx.y * kTI;
  const int n0 = blockIdx.x * kTN + wave * 64;
  const int Nb4 = Nbp / 4;
  const int8_t* mrow = mask + (size_t)bh * Nb * Nb;
  const uint16_t* hb = hx + (size_t)bh * Nb4 * NN * 4;

  // staging assignment: row si, 16 key blocks starting at 16*sh
  const int si = tid >> 1, sh = tid & 1;
  auto stage = [&](int s, int buf) {
    const int i = i0 + si;
    uint32_t w[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int j0 = 32 * s + 16 * sh + 2 * e;
      uint32_t lo = 0, hi = 0;
      if (i < Nb && j0 < Nb && mrow[(size_t)i * Nb + j0] == 0) lo = 0x3f80u;
      if (i < Nb && j0 + 1 < Nb && mrow[(size_t)i * Nb + j0 + 1] == 0) hi = 0x3f80u;
      w[e] = lo | (hi << 16);
    }
    uint4* dst = reinterpret_cast<uint4*>(&ms[buf][si][16 * sh]);
    dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
    dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
  };

  f32x4 acc[4][8];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int S = Nbp / 32;
  for (int s = 0; s < S; ++s) {
    stage(s, s & 1);
    __syncthreads();
    uint4 a[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int n = n0 + 16 * mt + l16;
      if (n < NN) {
        const int q = 8 * s + 2 * g;
        const uint2 lo = *reinterpret_cast<const uint2*>(hb + ((size_t)q * NN + n) * 4);
        const uint2 hi = *reinterpret_cast<const uint2*>(hb + ((size_t)(q + 1) * NN + n) * 4);
        a[mt] = make_uint4(lo.x, lo.y, hi.x, hi.y);
      } else {
        a[mt] = make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const uint4 b = *reinterpret_cast<const uint4*>(&ms[s & 1][16 * nt + l16][8 * g]);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) acc[mt][nt] = mfma_bf16(a[mt], b, acc[mt][nt]);
    }
  }
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) {
    const int i = i0 + 16 * nt + l16;
    if (i >= Nb) continue;
    uint16_t* orow = Hx + ((size_t)bh * Nb + i) * NN;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int n = n0 + 16 * mt + 4 * g;
      if (n < NN) {
        uint2 w;
        w.x = pack_bf2(acc[mt][nt][0], acc[mt][nt][1]);
        w.y = pack_bf2(acc[mt][nt][2], acc[mt][nt][3]);
        *reinterpret_cast<uint2*>(orow + n) = w;
      }
    }
  }
}

// ---------------------------------------------------------------- f32 path
__global__ __launch_bounds__(256) void k_linear_f32(const int8_t* __restrict__ mask,
                                                    const float* __restrict__ hx,
                                                    float* __restrict__ Hx, int Nb, int NN) {
  const int n = blockIdx.x * 256 + threadIdx.x;
  const int i = blockIdx.y, bh = blockIdx.z;
  if (n >= NN) return;
  const int8_t* mrow = mask + ((size_t)bh * Nb + i) * Nb;
  const float* hb = hx + (size_t)bh * Nb * NN;
  float s = 0.f;
  for (int j = 0; j < Nb; ++j)
    if (mrow[j] == 0) s += hb[(size_t)j * NN + n];
  Hx[((size_t)bh * Nb + i) * NN + n] = s;
}

}  // namespace

hipError_t launch_linear(const Dims& D, const int8_t* mask, const Work& w, hipStream_t s) {
  if (D.bf16) {
    dim3 grid((D.NN + kTN - 1) / kTN, (D.Nb + kTI - 1) / kTI, D.BH);
    hipLaunchKernelGGL(k_linear_bf16, grid, dim3(256), 0, s, mask, (const uint16_t*)w.hx,
                       (uint16_t*)w.Hx, D.Nb, D.Nbp, D.NN);
  } else {
    dim3 grid((D.NN + 255) / 256, D.Nb, D.BH);
    hipLaunchKernelGGL(k_linear_f32, grid, dim3(256), 0, s, mask, (const float*)w.hx,
                       (float*)w.Hx, D.Nb, D.NN);
  }
  return hipGetLastError();
}

}  // namespace sla
