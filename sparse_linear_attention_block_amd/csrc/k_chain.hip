// K4, second form: the marginal sums H_i, Z_i by a chain of updates along the
// query blocks instead of one indicator product per head.
//
// SLA paper summary (aipaper.cc), Eq. 3: H_i = sum over j with Mc[i, j] = 0 of
// h_j (and Z_i of z_j). The SLA explainer (intelliparadigm.com), section 2.3,
// points at cheaper forms of these per-row sums for very sparse masks (a
// lookup table of the positions that matter instead of a dense pass). Here the
// rows of one head are walked in order and each row's sum is taken from the
// previous row's: H_i = H_{i-1} + sum of h_j over the blocks that became
// marginal - sum over those that stopped being marginal. Neighbouring query
// blocks attend to nearly the same blocks, so a row changes in few places (25
// blocks on average at the Wan2.1-1.3B shape against 512 in the row, 41 of 1182
// at the 14B shape). The chain restarts at the first row of each of 16
// segments from the head's total minus the row's excluded blocks, so 16 waves
// walk their segments at once.
//
// k_chain_lists writes, per row, the blocks to add (from the front of the row's
// list) and to subtract (from the back); k_chain runs one workgroup per
// (64-column slice of h_j^T | z_j, head): the slice of every key block stays in
// LDS (Nb x 64 bf16, so Nb <= 1216), each wave keeps its column's running sum
// in float32 (one column per lane) and stores every row of its segment.
#include "sla_internal.h"
#include "dev_common.h"

namespace sla {
namespace {

constexpr int kChainWaves = 16;   // segments (and waves) per workgroup
constexpr int kChainCols = 64;    // h_j^T | z_j columns per workgroup, one per lane

// Row i of head bh: with p the row before it, add = {j : Mc[i][j] == 0 and
// Mc[p][j] != 0}, sub = {j : Mc[i][j] != 0 and Mc[p][j] == 0}; at the first row
// of a segment (i % S == 0) add is empty and sub is every block with
// Mc[i][j] != 0 (taken from the head's total). The two sets are disjoint, so
// both fit in one row of Nb entries: add ascending from the front, sub
// ascending from the back, a sub entry with bit 15 set. cnt = n_add | n_sub << 16.
__global__ __launch_bounds__(64) void k_chain_lists(const int8_t* __restrict__ mask, uint16_t* __restrict__ lists,
                                                    uint32_t* __restrict__ cnt, int Nb, int S) {
  const int i = blockIdx.x, bh = blockIdx.y, lane = threadIdx.x;
  const int8_t* cur = mask + ((size_t)bh * Nb + i) * Nb;
  const bool start = i % S == 0;
  const int8_t* prv = start ? cur : cur - Nb;
  uint16_t* out = lists + ((size_t)bh * Nb + i) * Nb;
  const uint64_t below = (1ull << lane) - 1ull;
  int na = 0, ns = 0;
  for (int c = 0; c < Nb; c += 64) {
    const int j = c + lane;
    const bool in = j < Nb;
    const int8_t m = in ? cur[j] : (int8_t)0;
    const int8_t p = in ? prv[j] : (int8_t)0;
    const bool add = in && !start && m == 0 && p != 0;
    const bool sub = in && m != 0 && (start || p == 0);
    const uint64_t ba = __ballot(add), bs = __ballot(sub);
    if (add) out[na + __popcll(ba & below)] = (uint16_t)j;
    if (sub) out[Nb - 1 - (ns + __popcll(bs & below))] = (uint16_t)(j | 0x8000);
    na += __popcll(ba);
    ns += __popcll(bs);
  }
  if (lane == 0) cnt[(size_t)bh * Nb + i] = (uint32_t)na | ((uint32_t)ns << 16);
}

// Dynamic LDS: the slice [Nbp + 1][64] bf16 (the last row all zero), then
// kChainWaves x 64 float partials.
template <int D>
__global__ __launch_bounds__(kChainWaves * 64) void k_chain(const uint16_t* __restrict__ hx,
                                                           const uint16_t* __restrict__ lists,
                                                           const uint32_t* __restrict__ cnt,
                                                           uint16_t* __restrict__ Hx, int Nb, int Nbp, int S) {
  constexpr int NN = D * D + D;
  extern __shared__ __attribute__((aligned(16))) uint16_t sl[];
  float* part = reinterpret_cast<float*>(sl + (size_t)(Nbp + 1) * kChainCols);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c0 = blockIdx.x * kChainCols, bh = blockIdx.y;
  // the slice, block-major: hx keeps four key blocks per 8-byte word of a column
  const uint16_t* src = hx + (size_t)bh * (Nbp / 4) * NN * 4 + (size_t)(c0 + lane) * 4;
  for (int q = wave; q < Nbp / 4; q += kChainWaves) {
    const uint2 w = *reinterpret_cast<const uint2*>(src + (size_t)q * NN * 4);
    sl[(4 * q + 0) * kChainCols + lane] = (uint16_t)(w.x & 0xffffu);
    sl[(4 * q + 1) * kChainCols + lane] = (uint16_t)(w.x >> 16);
    sl[(4 * q + 2) * kChainCols + lane] = (uint16_t)(w.y & 0xffffu);
    sl[(4 * q + 3) * kChainCols + lane] = (uint16_t)(w.y >> 16);
  }
  if (wave == 0) sl[Nbp * kChainCols + lane] = 0;  // the zero row that pads entry groups
  __syncthreads();
  // the head's total, summed in a fixed order (wave partials, then the waves)
  float t = 0.f;
  for (int j = wave; j < Nb; j += kChainWaves) t += bf2f(sl[j * kChainCols + lane]);
  part[wave * kChainCols + lane] = t;
  __syncthreads();
  float h = 0.f;
#pragma unroll
  for (int w = 0; w < kChainWaves; ++w) h += part[w * kChainCols + lane];
  // the wave's segment of rows. A row's entries travel one per lane (adds
  // first, then subtracts; past the row's count, the zero row), fetched a row
  // ahead; each is broadcast from its lane and names the key block whose slice
  // row is added (bit 15 clear) or subtracted. Four entries at a time go to
  // four partial sums, so four LDS reads are in flight.
  const int i0 = wave * S, i1 = min(Nb, i0 + S);
  auto fetch = [&](int i, int k0, uint32_t c) -> int {
    const int na = (int)(c & 0xffffu), n = na + (int)(c >> 16);
    const int k = k0 + lane;
    const uint16_t* L = lists + ((size_t)bh * Nb + min(i, Nb - 1)) * Nb;
    return k < n ? (int)L[k < na ? k : Nb - 1 - (k - na)] : Nbp;
  };
  auto term = [&](int e, int k) {
    const int j = __builtin_amdgcn_readlane(e, k);
    const float sg = (j & 0x8000) ? -1.0f : 1.0f;
    return sg * bf2f(sl[(j & 0x7fff) * kChainCols + lane]);
  };
  uint32_t cn = i0 < i1 ? cnt[(size_t)bh * Nb + i0] : 0u;
  int en = i0 < i1 ? fetch(i0, 0, __builtin_amdgcn_readfirstlane(cn)) : 0;
  for (int i = i0; i < i1; ++i) {
    const uint32_t c = __builtin_amdgcn_readfirstlane(cn);
    int e = en;
    if (i + 1 < i1) {  // the next row's count and first entries
      cn = cnt[(size_t)bh * Nb + i + 1];
      en = fetch(i + 1, 0, __builtin_amdgcn_readfirstlane(cn));
    }
    const int n = (int)(c & 0xffffu) + (int)(c >> 16);
    float p0 = 0.f, p1 = 0.f, p2 = 0.f, p3 = 0.f;
    for (int k0 = 0; k0 < n; k0 += 64) {
      if (k0 > 0) e = fetch(i, k0, c);
      const int m = min(64, n - k0);
      for (int k = 0; k < m; k += 4) {
        p0 += term(e, k);
        p1 += term(e, k + 1);
        p2 += term(e, k + 2);
        p3 += term(e, k + 3);
      }
    }
    h += (p0 + p1) + (p2 + p3);
    Hx[((size_t)bh * Nb + i) * NN + c0 + lane] = (uint16_t)f2bf(h);
  }
}

}  // namespace

size_t chain_lds_bytes(int Nbp) {
  return (size_t)(Nbp + 1) * kChainCols * 2 + (size_t)kChainWaves * kChainCols * 4;
}

hipError_t launch_chain(const Dims& D, const int8_t* mask, const Work& w, hipStream_t s) {
  if (!D.bf16 || D.NN % kChainCols != 0) return hipErrorInvalidValue;
  const int S = (D.Nb + kChainWaves - 1) / kChainWaves;
  hipLaunchKernelGGL(k_chain_lists, dim3(D.Nb, D.BH), dim3(64), 0, s, mask, w.chain_lists, w.chain_cnt, D.Nb, S);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds = chain_lds_bytes(D.Nbp);
  const dim3 grid(D.NN / kChainCols, D.BH);
  if (D.d == 128) {
    e = hipFuncSetAttribute((const void*)k_chain<128>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_chain<128>, grid, dim3(kChainWaves * 64), lds, s, (const uint16_t*)w.hx,
                       w.chain_lists, w.chain_cnt, (uint16_t*)w.Hx, D.Nb, D.Nbp, S);
  } else {
    e = hipFuncSetAttribute((const void*)k_chain<64>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_chain<64>, grid, dim3(kChainWaves * 64), lds, s, (const uint16_t*)w.hx,
                       w.chain_lists, w.chain_cnt, (uint16_t*)w.Hx, D.Nb, D.Nbp, S);
  }
  return hipGetLastError();
}

}  // namespace sla
