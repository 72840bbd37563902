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
// layout the MFMA A operand needs; the mask is first turned into a bf16 0/1
// indicator (k_indicator) in a layout the GEMM copies straight into LDS and
// reads as the B operand; each lane then holds 4 consecutive n of one query
// block and stores them as one 8-byte word.
#include "sla_internal.h"
#include "dev_common.h"

namespace sla {
namespace {

constexpr int kTN = 256;  // n per workgroup
constexpr int kTI = 128;  // query blocks per workgroup
constexpr int kOS = kTN + 8;  // row stride of the staged output (bf16)

// The marginal indicator M01[i][j] = (Mc[i][j] == 0) as bf16 0/1, one
// [Nb128][32] slab per 32-key step; chunk q (keys 8q..8q+7 of the step) of row
// i sits at chunk position q ^ ((i >> 1) & 3), so that 8 lanes reading 8
// consecutive rows of the slab hit distinct LDS banks. Rows >= Nb and keys >=
// Nb are 0.
__global__ __launch_bounds__(256) void k_indicator(const int8_t* __restrict__ mask,
                                                   uint16_t* __restrict__ ind, int Nb, int Nbp,
                                                   int Nb128) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  const int s = blockIdx.y, bh = blockIdx.z;
  const int q = t & 3, i = t >> 2;
  if (i >= Nb128) return;
  uint32_t w[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    uint32_t v = 0;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int j = 32 * s + 8 * q + 2 * e + hh;
      if (i < Nb && j < Nb && mask[((size_t)bh * Nb + i) * Nb + j] == 0) v |= 0x3f80u << (16 * hh);
    }
    w[e] = v;
  }
  uint16_t* dst = ind + (((size_t)bh * (Nbp / 32) + s) * Nb128 + i) * 32 + 8 * (q ^ ((i >> 1) & 3));
  *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
}

// Hx^T = hx^T M01^T for one (batch, head): workgroup tile 256 n x 128 query
// blocks, wave w owns n0 + 64w .. +63 against all 128 rows, k steps of 32 key
// blocks. The hx operand (4 key blocks per 8-byte word, as written by the h/z
// kernel) goes straight from global memory to registers one step ahead; the
// indicator slab of a step arrives in LDS by direct asynchronous copies,
// double-buffered, one LDS barrier per step. The finished tile is staged in LDS
// in two halves and written as contiguous 16-byte stores along each row.
// Workgroups are remapped so that the row tiles of one n range run back to back
// on one XCD and share hx in L2.
__global__ __launch_bounds__(256, 2) void k_linear_bf16(const uint16_t* __restrict__ ind,
                                                        const uint16_t* __restrict__ hx,
                                                        uint16_t* __restrict__ Hx, int Nb, int Nbp,
                                                        int Nb128, int NN, int ntn, int nti) {
  __shared__ __attribute__((aligned(16))) uint16_t bA[kTI * 32];
  __shared__ __attribute__((aligned(16))) uint16_t bB[kTI * 32];
  __shared__ __attribute__((aligned(16))) uint16_t ost[64 * kOS];  // half the output tile
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int it = id % nti;
  const int rest = id / nti;
  const int nt = rest % ntn, bh = rest / ntn;
  const int i0 = it * kTI;
  const int n0 = nt * kTN + wave * 64;
  const int S = Nbp / 32, Nb4 = Nbp / 4;
  const uint16_t* indb = ind + ((size_t)bh * S * Nb128 + i0) * 32;
  const uint16_t* hb = hx + (size_t)bh * Nb4 * NN * 4;

  auto issue = [&](int s, uint16_t* dst) {  // 8 KB slab: two 16-byte copies per lane
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int G = 64 * (4 * u + wave) + lane;
      load_lds16(indb + (size_t)s * Nb128 * 32 + (size_t)G * 8, dst + 512 * (4 * u + wave));
    }
  };
  auto loadA = [&](int s, uint4* a) {
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
  };

  f32x4 acc[4][8];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int n2 = 0; n2 < 8; ++n2) acc[mt][n2] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto step = [&](int s, const uint16_t* cur, uint16_t* nxt, const uint4* a, uint4* an) {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // slab s and operand s have landed
    lds_barrier();
    if (s + 1 < S) {
      issue(s + 1, nxt);
      loadA(s + 1, an);
    }
#pragma unroll
    for (int n2 = 0; n2 < 8; ++n2) {
      const int row = 16 * n2 + l16;
      const uint4 b = *reinterpret_cast<const uint4*>(cur + row * 32 + 8 * (g ^ ((row >> 1) & 3)));
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) acc[mt][n2] = mfma_bf16(a[mt], b, acc[mt][n2]);
    }
  };
  uint4 aA[4], aB[4];
  issue(0, bA);
  loadA(0, aA);
  for (int s = 0; s < S; s += 2) {
    step(s, bA, bB, aA, aB);
    if (s + 1 < S) step(s + 1, bB, bA, aB, aA);
  }
  // the output tile goes out in two halves of 64 query blocks, staged in LDS so
  // that every row segment of 256 columns is written as contiguous 16-byte stores
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if (half) __syncthreads();  // the first half has been copied out
#pragma unroll
    for (int n4 = 0; n4 < 4; ++n4) {
      const int n2 = 4 * half + n4;
      const int il = 16 * n4 + l16;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        uint2 w;
        w.x = pack_bf2(acc[mt][n2][0], acc[mt][n2][1]);
        w.y = pack_bf2(acc[mt][n2][2], acc[mt][n2][3]);
        *reinterpret_cast<uint2*>(ost + il * kOS + 64 * wave + 16 * mt + 4 * g) = w;
      }
    }
    __syncthreads();
    const int nbase = nt * kTN;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int x = 256 * u + tid;          // 64 rows x 32 chunks of 16 bytes
      const int row = x >> 5, ch = x & 31;
      const int i = i0 + 64 * half + row, n = nbase + 8 * ch;
      if (i < Nb && n < NN)
        *reinterpret_cast<uint4*>(Hx + ((size_t)bh * Nb + i) * NN + n) =
            *reinterpret_cast<const uint4*>(ost + row * kOS + 8 * ch);
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

hipError_t launch_indicator(const Dims& D, const int8_t* mask, const Work& w, hipStream_t s) {
  dim3 grid(D.Nb128 * 4 / 256, D.Nbp / 32, D.BH);
  hipLaunchKernelGGL(k_indicator, grid, dim3(256), 0, s, mask, w.ind, D.Nb, D.Nbp, D.Nb128);
  return hipGetLastError();
}

hipError_t launch_linear(const Dims& D, const int8_t* mask, const Work& w, hipStream_t s) {
  if (D.bf16) {
    const int ntn = (D.NN + kTN - 1) / kTN, nti = D.Nb128 / kTI;
    hipLaunchKernelGGL(k_linear_bf16, dim3(D.BH * ntn * nti), dim3(256), 0, s,
                       (const uint16_t*)w.ind, (const uint16_t*)w.hx, (uint16_t*)w.Hx, D.Nb,
                       D.Nbp, D.Nb128, D.NN, ntn, nti);
  } else {
    dim3 grid((D.NN + 255) / 256, D.Nb, D.BH);
    hipLaunchKernelGGL(k_linear_f32, grid, dim3(256), 0, s, mask, (const float*)w.hx,
                       (float*)w.Hx, D.Nb, D.NN);
  }
  return hipGetLastError();
}

}  // namespace sla
