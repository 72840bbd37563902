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
// The product runs per workgroup over a 64-column slice of hx and up to 512
// query blocks, so hx is read from memory once. The 0/1 matrix travels as
// bits, one 32-bit word per (32-key step, query block), and each lane expands
// its word into the bf16 B operand of the MFMA with two integer operations per
// register; the hx operand (4 consecutive key blocks per 8-byte word, written
// so by K3) is the A operand.
#include <type_traits>

#include "sla_internal.h"
#include "dev_common.h"

namespace sla {
namespace {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kTN = 64;    // hx columns per workgroup
constexpr int kRows = 128; // query blocks per wave (4 waves per workgroup)

// The marginal indicator M01[i][j] = (Mc[i][j] == 0) as bits. Word W(s, i)
// covers keys 32s .. 32s+31 of query block i: for lane group g and e < 4,
// bit 4g + e is key 32s + 8g + 2e and bit 16 + 4g + e is key 32s + 8g + 2e + 1
// (the two bf16 halves of register e of that lane group's B operand). The word
// sits at [bh][s][i / 128][i % 16][(i / 16) % 8], so that a lane reads the
// words of its 8 query tiles as 32 contiguous bytes. Rows >= Nb and keys >= Nb
// are 0.
__global__ __launch_bounds__(256) void k_indicator(const int8_t* __restrict__ mask,
                                                   uint32_t* __restrict__ ind, int Nb, int Nbp,
                                                   int Nb128) {
  // one wave per query block, two k steps per iteration: lane L takes key
  // 32 (s + L / 32) + k(L % 32) with k(16 hi + 4 g + e) = 8 g + 2 e + hi, so the
  // wave's ballot is the two words W(s), W(s + 1) in their bit layout
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int bh = blockIdx.y;
  const int S = Nbp / 32, NI = Nb128 / 128;
  if (i >= Nb128) return;  // wave-uniform
  const int L = lane & 31, k = 8 * ((L >> 2) & 3) + 2 * (L & 3) + (L >> 4);
  const int8_t* row = mask + ((size_t)bh * Nb + min(i, Nb - 1)) * Nb;
  uint32_t* dst = ind + ((size_t)bh * S * NI + i / 128) * 128 + (i % 16) * 8 + (i / 16) % 8;
  // eight step pairs per round, every load of a round issued before the first ballot
  for (int s0 = 0; s0 < S; s0 += 16) {
    int8_t m[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) m[u] = row[min(32 * (s0 + 2 * u + (lane >> 5)) + k, Nb - 1)];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int s = s0 + 2 * u;
      if (s >= S) break;  // uniform
      const int j = 32 * (s + (lane >> 5)) + k;
      const uint64_t w = __ballot(i < Nb && j < Nb && m[u] == 0);
      if (lane == 0) dst[(size_t)s * NI * 128] = (uint32_t)w;
      if (lane == 32 && s + 1 < S) dst[(size_t)(s + 1) * NI * 128] = (uint32_t)(w >> 32);
    }
  }
}

// Hx^T = hx^T M01^T for one (batch, head): workgroup tile 64 columns n x 512
// query blocks, wave w owns query blocks 128 w .. +127 of the tile against all
// 64 columns (4 x 8 MFMA tiles), k steps of 32 key blocks. hx comes from memory
// exactly once, so its latency is that of HBM: the 4 KB hx slab of a k step
// arrives in LDS by direct copies kRing - 1 steps ahead (a ring of kRing
// slots, one barrier per step); each wave reads its A operands from there. The
// slots are distinct LDS objects picked at compile time (the loop is unrolled
// by kRing), so the compiler sees that reads of one slot do not alias the
// copies into another and does not wait for those copies. The indicator words
// of each wave travel in the same slot. With no operand held in registers
// across steps, three workgroups fit on a CU.
// Each lane
// holds 4 consecutive n of one query block per MFMA tile and stores them as
// one 8-byte word; the wave fills whole 128-byte row segments. Workgroups are
// remapped so that the column slices of one head run back to back on one XCD.
constexpr int kRing = 6;              // hx slabs in flight or in use (a multiple of 3)
constexpr int kSeg = 1024 + 128;      // bytes per wave segment of a slab (padded)
constexpr int kOSt = 128 + 16;       // bytes per staged output row (64 bf16, padded)
static_assert(32 * kOSt <= 4 * kSeg + 4 * 512, "a 32-row output stage fits in one ring slot");
constexpr int kSlab = 4 * kSeg + 4 * 512;  // one k step: 8 groups of 4 key blocks x 64 n x
                                           // 8 bytes, then 128 indicator words per wave

__global__ __launch_bounds__(256, 3) void k_linear_bf16(const uint32_t* __restrict__ ind,
                                                        const uint16_t* __restrict__ hx,
                                                        uint16_t* __restrict__ Hx, int Nb, int Nbp,
                                                        int Nb128, int NN, int ntn, int nit) {
  __shared__ __attribute__((aligned(16))) uint8_t slab0[kSlab];
  __shared__ __attribute__((aligned(16))) uint8_t slab1[kSlab];
  __shared__ __attribute__((aligned(16))) uint8_t slab2[kSlab];
  __shared__ __attribute__((aligned(16))) uint8_t slab3[kSlab];
  __shared__ __attribute__((aligned(16))) uint8_t slab4[kSlab];
  __shared__ __attribute__((aligned(16))) uint8_t slab5[kSlab];
  uint8_t* const slabs[kRing] = {slab0, slab1, slab2, slab3, slab4, slab5};
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int it = id % nit;
  const int rest = id / nit;
  const int nt = rest % ntn, bh = rest / ntn;
  const int ig = 4 * it + wave;          // the wave's group of 128 query blocks
  const bool live = ig * kRows < Nb;     // wave-uniform; idle waves still take the barriers
  const int NI = Nb128 / kRows;
  const int S = Nbp / 32, Nb4 = Nbp / 4;
  const int n0 = nt * kTN;
  // buffer resources over this head's hx and indicator words: the per-lane
  // byte offsets are fixed, the k step moves the scalar offset only
  const __amdgpu_buffer_rsrc_t hrs = make_rsrc(hx + (size_t)bh * Nb4 * NN * 4, Nb4 * NN * 8);
  const __amdgpu_buffer_rsrc_t wrs = make_rsrc(ind + (size_t)bh * S * NI * kRows, S * NI * kRows * 4);
  // slab copy: wave w brings groups 2w (lanes 0-31) and 2w + 1 (lanes 32-63) of
  // 4 key blocks, 16 bytes (two columns) per lane, into its segment
  const uint32_t coff = ((uint32_t)(2 * wave + (lane >> 5)) * NN + n0 + 2 * (lane & 31)) * 8u;
  // indicator copy: lanes 0-31 of a wave bring its 128 words (lanes 32-63 idle)
  const uint32_t woff = (uint32_t)(min(ig, NI - 1) * kRows + 4 * (lane & 31)) * 4u;
  // The slab of k step t (clamped) into a ring slot: two copies per wave.
  auto copy = [&](int t, uint8_t* slot) {
    const int tc = min(t, S - 1);
    load_lds16_buf(hrs, coff, tc * 64 * NN, slot + wave * kSeg);
    if (lane < 32) load_lds16_buf(wrs, woff, tc * NI * kRows * 4, slot + 4 * kSeg + wave * 512);
  };

  f32x4 acc[4][8];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int n2 = 0; n2 < 8; ++n2) acc[mt][n2] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int sh = 4 * g;
  // A operand of lane (l16, g), tile mt: group 2g (low 8 bytes) and 2g + 1 (high)
  // at column 16 mt + l16, both in the segment of wave g
  const int aoff = g * kSeg + l16 * 8;
  // One k step s at ring position P = s % kRing: copy(s + kRing - 1), two
  // vector-memory operations per wave, so when step s starts only the two of
  // step s - 1 may still be in flight and everything step s reads has landed.
  auto step = [&](int s, auto Pc) {
    constexpr int P = decltype(Pc)::value;
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(2));
    lds_barrier();  // every wave's copies of slab s have landed; the slot of step s - 1 is free
    copy(s + kRing - 1, slabs[(P + kRing - 1) % kRing]);
    if (live) {
      const uint8_t* slab = slabs[P] + aoff;
      const uint4* w = reinterpret_cast<const uint4*>(slabs[P] + 4 * kSeg + wave * 512 + l16 * 32);
      uint4 a[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const uint2 lo = *reinterpret_cast<const uint2*>(slab + 128 * mt);
        const uint2 hi = *reinterpret_cast<const uint2*>(slab + 512 + 128 * mt);
        a[mt] = make_uint4(lo.x, lo.y, hi.x, hi.y);
      }
      const uint4 w0 = w[0], w1 = w[1];
      const uint32_t wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
      for (int n2 = 0; n2 < 8; ++n2) {
        // register e of the B operand: bf16 1.0 (0x3f80) in the halves whose bits are set
        const uint32_t W = wv[n2] >> sh;
        const uint4 b = make_uint4((W & 0x00010001u) * 0x3f80u, (W & 0x00020002u) * 0x1fc0u,
                                   (W & 0x00040004u) * 0x0fe0u, (W & 0x00080008u) * 0x07f0u);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc[mt][n2] = mfma_bf16(a[mt], b, acc[mt][n2]);
      }
    }
  };
  // prologue: slabs 0 .. kRing - 2
#pragma unroll
  for (int t = 0; t + 1 < kRing; ++t) copy(t, slabs[t]);
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using I4 = std::integral_constant<int, 4>;
  using I5 = std::integral_constant<int, 5>;
  // unrolled by kRing: full rounds carry no condition (so the wait counts stay
  // exact), the last steps follow
  int s = 0;
  for (; s + kRing <= S; s += kRing) {
    step(s, I0{});
    step(s + 1, I1{});
    step(s + 2, I2{});
    step(s + 3, I3{});
    step(s + 4, I4{});
    step(s + 5, I5{});
  }
  if (s < S) step(s, I0{});
  if (s + 1 < S) step(s + 1, I1{});
  if (s + 2 < S) step(s + 2, I2{});
  if (s + 3 < S) step(s + 3, I3{});
  if (s + 4 < S) step(s + 4, I4{});
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // the clamped copies past the end land before exit

  // The tile goes out through LDS in four quarters of 32 query blocks per wave,
  // so that every store is 16 bytes of a whole 128-byte row segment. Wave w
  // stages in ring slot w, which is free once every wave is past its last step
  // and the last copies have landed.
  __syncthreads();
  uint8_t* stage = wave == 0 ? slab0 : wave == 1 ? slab1 : wave == 2 ? slab2 : slab3;
  if (live) {
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
#pragma unroll
      for (int n4 = 0; n4 < 2; ++n4) {
        const int n2 = 2 * qq + n4;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          *reinterpret_cast<uint2*>(stage + (16 * n4 + l16) * kOSt + (16 * mt + 4 * g) * 2) =
              make_uint2(pack_bf2(acc[mt][n2][0], acc[mt][n2][1]), pack_bf2(acc[mt][n2][2], acc[mt][n2][3]));
      }
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);  // a wave reads back only its own rows
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int row = 8 * u + (lane >> 3), ch = lane & 7;
        const int i = ig * kRows + 32 * qq + row;
        const uint4 v = *reinterpret_cast<const uint4*>(stage + row * kOSt + 16 * ch);
        if (i < Nb) *reinterpret_cast<uint4*>(Hx + ((size_t)bh * Nb + i) * NN + n0 + 8 * ch) = v;
      }
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);  // reads done before the next quarter overwrites
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
  dim3 grid(D.Nb128 / 4, D.BH);  // one wave per query block (rows past Nb get zeros)
  hipLaunchKernelGGL(k_indicator, grid, dim3(256), 0, s, mask, w.ind, D.Nb, D.Nbp, D.Nb128);
  return hipGetLastError();
}

hipError_t launch_linear(const Dims& D, const int8_t* mask, const Work& w, hipStream_t s) {
  if (D.bf16) {
    // d (d + 1) is a multiple of 64 for the supported d, so column slices are whole
    if (D.NN % kTN != 0) return hipErrorInvalidValue;
    const int ntn = D.NN / kTN, nit = (D.Nb128 / kRows + 3) / 4;
    hipLaunchKernelGGL(k_linear_bf16, dim3(D.BH * ntn * nit), dim3(256), 0, s,
                       (const uint32_t*)w.ind, (const uint16_t*)w.hx, (uint16_t*)w.Hx, D.Nb,
                       D.Nbp, D.Nb128, D.NN, ntn, nit);
  } else {
    dim3 grid((D.NN + 255) / 256, D.Nb, D.BH);
    hipLaunchKernelGGL(k_linear_f32, grid, dim3(256), 0, s, mask, (const float*)w.hx,
                       (float*)w.Hx, D.Nb, D.NN);
  }
  return hipGetLastError();
}

}  // namespace sla
