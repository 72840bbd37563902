// K2: compressed scores and three-way block classification.
//
// SLA paper summary (aipaper.cc), section 4, Eq. 1 (Pc = softmax of the pooled
// logits, scaled by 1/sqrt(d)) and Eq. 2 (Mc = 1 for the top kh% of each row,
// -1 for the bottom kl%, 0 otherwise). Softmax is monotone in each row, so the
// ranking is taken on the logits themselves and Pc is never materialised. The
// order is the float64 logit, descending, with the lower block index first
// among equal logits; the mask is exactly that order's head and tail.
//
// k_logits_est: float32 estimates a of the logits of a 64 x 64 tile on bf16
//   MFMA 16x16x32 from a two-term split of each float64 pooled value
//   (x = hi + lo + r, hi = bf16(x), lo = bf16(x - hi), |r| <= 2^-16 |x|; the
//   three products hi.hi + hi.lo + lo.hi accumulated in float32). The tiles of
//   the first column also write the norms of their pooled queries, those of
//   the first row the largest norm of their 64 pooled keys. Every a is within
//   eps = kBandKappa |q| max_j |k_j| / sqrt(d) of the float64 logit: the
//   dropped terms are at most 3.1 2^-16 sum_c |q_c k_c|, the float32 sums
//   (3 d products) at most 3 d 2^-24 of the same, and sum_c |q_c k_c| <=
//   |q| |k| (Cauchy-Schwarz); kBandKappa carries a margin over that sum.
// k_classify_band: one wave per row. The n_h-th largest estimate A_h is
//   located in a value interval [lo, hi] no wider than eps by 256-bin
//   histograms over the row's range (LDS atomics), each level refining the bin
//   that holds the rank. Order statistics move by at most eps when every
//   element moves by at most eps, so a block with a > hi + 2 eps is critical,
//   one with a < lo - 2 eps is not, and only the band [lo - 2 eps, hi + 2 eps]
//   is undecided (one to three blocks per row on the Wan-shaped workloads).
//   The band's blocks get their float64 logits from the pooled vectors (one
//   wave-wide dot product each, summed in a fixed butterfly order, divided by
//   sqrt(d)) and are ranked exactly among themselves. The tail n_l is found
//   the same way around the n_l-th smallest estimate, among the blocks that
//   are not critical. No Nb x Nb float64 matrix is stored.
// k_logits: the float64 logits themselves on float64 MFMA 16x16x4, written only
//   when the caller asks for them (debug output); the mask never reads them.
#include "sla_internal.h"
#include "dev_common.h"

namespace sla {
namespace {

// Bound on |a - logit| per unit of |q| max_j |k_j| / sqrt(d): the derivation in
// the header gives 3.1 2^-16 + 3 d 2^-24 <= 7.2e-5 at d <= 128 (plus float32
// roundings of the scale and of the norms, below 1e-6 relative); 1e-4 leaves a
// margin. kBandAbs covers products that underflow float32.
constexpr float kBandKappa = 1.0e-4f;
constexpr float kBandAbs = 1.0e-30f;

// Lane exchanges inside a row of 16 lanes by DPP (plain VALU operations, no
// LDS round trip): quad_perm [1,0,3,2] and [2,3,0,1] swap lanes l ^ 1 and
// l ^ 2, row_half_mirror reverses each 8 lanes, row_mirror each 16; after the
// four, every lane of a row has combined all 16. The four rows are then read
// with v_readlane and combined in a fixed order.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(dpp_i<CTRL>(__float_as_int(v)));
}
template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
  const int2 w = __builtin_bit_cast(int2, v);
  return __builtin_bit_cast(double, make_int2(dpp_i<CTRL>(w.x), dpp_i<CTRL>(w.y)));
}
__device__ __forceinline__ float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ double readlane_d(double v, int l) {
  const int2 w = __builtin_bit_cast(int2, v);
  return __builtin_bit_cast(double, make_int2(__builtin_amdgcn_readlane(w.x, l), __builtin_amdgcn_readlane(w.y, l)));
}
__device__ __forceinline__ float wave_min(float v) {
  v = fminf(v, dpp_f<kDppXor1>(v));
  v = fminf(v, dpp_f<kDppXor2>(v));
  v = fminf(v, dpp_f<kDppHalfMirror>(v));
  v = fminf(v, dpp_f<kDppMirror>(v));
  return fminf(fminf(readlane_f(v, 0), readlane_f(v, 16)), fminf(readlane_f(v, 32), readlane_f(v, 48)));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v));
  v = fmaxf(v, dpp_f<kDppXor2>(v));
  v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f<kDppMirror>(v));
  return fmaxf(fmaxf(readlane_f(v, 0), readlane_f(v, 16)), fmaxf(readlane_f(v, 32), readlane_f(v, 48)));
}
// float64 sum over the wave in a fixed order (the same value in every lane, and
// bit-equal sums for bit-equal inputs)
__device__ __forceinline__ double wave_sum_d(double v) {
  v += dpp_d<kDppXor1>(v);
  v += dpp_d<kDppXor2>(v);
  v += dpp_d<kDppHalfMirror>(v);
  v += dpp_d<kDppMirror>(v);
  return (readlane_d(v, 0) + readlane_d(v, 16)) + (readlane_d(v, 32) + readlane_d(v, 48));
}
// inclusive prefix sum over the 64 lanes: Hillis-Steele shifts inside each
// row (row_shr 1, 2, 4, 8), then row_bcast 15 into rows 1 and 3 and row_bcast
// 31 into rows 2 and 3
__device__ __forceinline__ int wave_scan_incl(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);
  return v;
}

template <int D>
__global__ __launch_bounds__(256) void k_logits(const double* __restrict__ pq,
                                                const double* __restrict__ pk,
                                                double* __restrict__ lg, int Nb) {
  constexpr int KS = D / 4;   // k steps of the 16x16x4 product
  constexpr int PS = D + 4;   // padded LDS row stride (doubles)
  __shared__ __attribute__((aligned(16))) double kt[64 * PS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int j0 = blockIdx.x * 64, i0 = blockIdx.y * 64, bh = blockIdx.z;
  const double* Pk = pk + ((size_t)bh * Nb + j0) * D;
  // key rows past Nb re-read row Nb - 1 (their columns are never stored); all
  // loads are issued before the first LDS write
  constexpr int NL = 64 * D / 2 / 256;
  double2 kv[NL];
#pragma unroll
  for (int u = 0; u < NL; ++u) {
    const int x = 256 * u + tid, row = x / (D / 2), c2 = x % (D / 2);
    kv[u] = reinterpret_cast<const double2*>(Pk + (size_t)min(row, Nb - 1 - j0) * D)[c2];
  }
#pragma unroll
  for (int u = 0; u < NL; ++u) {
    const int x = 256 * u + tid, row = x / (D / 2), c2 = x % (D / 2);
    *reinterpret_cast<double2*>(&kt[row * PS + 2 * c2]) = kv[u];
  }
  const int ir = min(i0 + 16 * wave + l16, Nb - 1);  // rows past Nb are never stored
  const double* qrow = pq + ((size_t)bh * Nb + ir) * D;
  double a[KS];                                       // A[row l16][k = 4ks + g]
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) a[ks] = qrow[4 * ks + g];
  __syncthreads();
  typedef double f64x4 __attribute__((__vector_size__(4 * sizeof(double))));
  f64x4 acc[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) acc[ct] = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
      acc[ct] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[ks], kt[(16 * ct + l16) * PS + 4 * ks + g],
                                                     acc[ct], 0, 0, 0);
  const double sd = sqrt((double)D);
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    const int j = j0 + 16 * ct + l16;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int i = i0 + 16 * wave + g + 4 * e;       // f64 16x16 layout: D[g + 4e][l16]
      if (i < Nb && j < Nb) lg[((size_t)bh * Nb + i) * Nb + j] = acc[ct][e] / sd;
    }
  }
}

// hi = bf16(x), lo = bf16(x - hi) for two float64 values, packed as bf16 pairs
// (x - hi is exact in float64: hi is x rounded to 8 bits)
__device__ __forceinline__ void split_pair(double x0, double x1, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf2((float)x0, (float)x1);
  lo = pack_bf2((float)(x0 - (double)bf_lo(hi)), (float)(x1 - (double)bf_hi(hi)));
}

// The two-term split of the pooled vectors, once per call: hilo holds
// [q hi, q lo, k hi, k lo], each [BH, Nb, d] bf16. Workgroup: 64 rows of one
// (batch, head) of pooled queries (z = 0) or keys (z = 1), kSplitRows rows per
// wave, a row's features spread over the lanes (F = d / 64 per lane). Queries
// also write their norms, keys the largest norm of the 64 rows. Each row's norm
// is a chain of cross-lane sums, so the rows go to many waves (the grid is a few
// hundred workgroups): 4 rows per wave instead of 16 take ~2 us off its 8.7 us
// at the 1.3B shape.
constexpr int kSplitRows = 4;
constexpr int kSplitWaves = 64 / kSplitRows;
template <int D>
__global__ __launch_bounds__(64 * kSplitWaves) void k_split(const double* __restrict__ pq, const double* __restrict__ pk,
                                               uint16_t* __restrict__ hilo, float* __restrict__ qnorm,
                                               float* __restrict__ knmax, int Nb, int nt, int BH) {
  constexpr int F = D / 64;
  __shared__ float wmax[kSplitWaves];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x, bh = blockIdx.y, z = blockIdx.z;
  const size_t plane = (size_t)BH * Nb * D;
  const double* src = (z ? pk : pq) + (size_t)bh * Nb * D;
  uint16_t* hi = hilo + (2 * z) * plane + (size_t)bh * Nb * D;
  uint16_t* lo = hi + plane;
  double x[kSplitRows][F];
#pragma unroll
  for (int u = 0; u < kSplitRows; ++u) {
    const int r = min(64 * t + kSplitRows * wave + u, Nb - 1);
#pragma unroll
    for (int f = 0; f < F; ++f) x[u][f] = src[(size_t)r * D + F * lane + f];
  }
  float mx = 0.f;
#pragma unroll
  for (int u = 0; u < kSplitRows; ++u) {
    const int r = 64 * t + kSplitRows * wave + u;
    double sq = 0.0;
#pragma unroll
    for (int f = 0; f < F; ++f) sq = fma(x[u][f], x[u][f], sq);
    const float nrm = (float)sqrt(wave_sum_d(sq));
    if (r < Nb) {
      if constexpr (F == 2) {
        uint32_t h, l;
        split_pair(x[u][0], x[u][1], h, l);
        reinterpret_cast<uint32_t*>(hi + (size_t)r * D)[lane] = h;
        reinterpret_cast<uint32_t*>(lo + (size_t)r * D)[lane] = l;
      } else {
        const float xf = (float)x[u][0];
        const uint32_t h = f2bf(xf);
        hi[(size_t)r * D + lane] = (uint16_t)h;
        lo[(size_t)r * D + lane] = (uint16_t)f2bf((float)(x[u][0] - (double)bf2f(h)));
      }
      if (z == 0 && lane == 0) qnorm[(size_t)bh * Nb + r] = nrm;
      mx = fmaxf(mx, nrm);
    }
  }
  if (z == 1) {
    if (lane == 0) wmax[wave] = mx;
    __syncthreads();
    if (threadIdx.x == 0) {
      float m = wmax[0];
      for (int w = 1; w < kSplitWaves; ++w) m = fmaxf(m, wmax[w]);
      knmax[(size_t)bh * nt + t] = m;
    }
  }
}

// Workgroup: 64 pooled keys x 128 pooled queries of one (batch, head), on a
// 1-D grid whose workgroups are remapped so that each XCD walks whole heads (a
// head's split vectors, 4 Nb d bf16, then stay in that XCD's L2). The key tile
// (hi and lo rows) is staged in LDS with rows padded to d + 8, so that 16 lanes
// reading 16 rows at one 16-byte chunk hit distinct banks; each wave keeps the
// A operands of its 32 queries (two groups of 16: row l16, features
// 32 ks + 8 g .. +7) in registers and forms its 32 x 64 tile with three
// products per k step.
template <int D>
__global__ __launch_bounds__(256) void k_logits_est(const uint16_t* __restrict__ hilo, float* __restrict__ est,
                                                    int Nb, int BH, int nt, int nq) {
  constexpr int KS = D / 32;        // k steps of the 16x16x32 product
  constexpr int CH = D / 8;         // 16-byte chunks per row
  constexpr int RS = D + 8;         // LDS row stride (bf16)
  constexpr int NU = 64 * CH / 256;  // chunks per thread and array
  __shared__ __attribute__((aligned(16))) uint16_t khi[64 * RS];
  __shared__ __attribute__((aligned(16))) uint16_t klo[64 * RS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = id / (nq * nt), tq = id / nt % nq, tk = id % nt;
  const int j0 = tk * 64, i0 = tq * 128 + 32 * wave;
  const size_t plane = (size_t)BH * Nb * D, hoff = (size_t)bh * Nb * D;
  const uint16_t* qh = hilo + hoff;
  const uint16_t* ql = qh + plane;
  const uint16_t* kh = ql + plane;
  const uint16_t* kl = kh + plane;
  // all loads first: the key tile (chunk x = 256 u + tid is row x / CH; rows past
  // Nb re-read row Nb - 1 and are never stored), then the wave's queries
  uint4 kv[2][NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int x = 256 * u + tid, r = x / CH, c = x % CH;
    const size_t o = (size_t)min(j0 + r, Nb - 1) * D + 8 * c;
    kv[0][u] = *reinterpret_cast<const uint4*>(kh + o);
    kv[1][u] = *reinterpret_cast<const uint4*>(kl + o);
  }
  uint4 ahi[2][KS], alo[2][KS];
#pragma unroll
  for (int qg = 0; qg < 2; ++qg) {
    const size_t o = (size_t)min(i0 + 16 * qg + l16, Nb - 1) * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      ahi[qg][ks] = *reinterpret_cast<const uint4*>(qh + o + 32 * ks);
      alo[qg][ks] = *reinterpret_cast<const uint4*>(ql + o + 32 * ks);
    }
  }
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int x = 256 * u + tid, r = x / CH, c = x % CH;
    *reinterpret_cast<uint4*>(&khi[r * RS + 8 * c]) = kv[0][u];
    *reinterpret_cast<uint4*>(&klo[r * RS + 8 * c]) = kv[1][u];
  }
  __syncthreads();
  f32x4 acc[2][4];
#pragma unroll
  for (int qg = 0; qg < 2; ++qg)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) acc[qg][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const int off = (16 * ct + l16) * RS + 32 * ks + 8 * g;
      const uint4 bh16 = *reinterpret_cast<const uint4*>(&khi[off]);
      const uint4 bl16 = *reinterpret_cast<const uint4*>(&klo[off]);
#pragma unroll
      for (int qg = 0; qg < 2; ++qg) {
        acc[qg][ct] = mfma_bf16(alo[qg][ks], bh16, acc[qg][ct]);
        acc[qg][ct] = mfma_bf16(ahi[qg][ks], bl16, acc[qg][ct]);
        acc[qg][ct] = mfma_bf16(ahi[qg][ks], bh16, acc[qg][ct]);
      }
    }
  const float isd = 1.0f / sqrtf((float)D);
#pragma unroll
  for (int qg = 0; qg < 2; ++qg)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const int j = j0 + 16 * ct + l16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = i0 + 16 * qg + 4 * g + r;  // D[4 g + r][l16]
        if (i < Nb && j < Nb) est[((size_t)bh * Nb + i) * Nb + j] = acc[qg][ct][r] * isd;
      }
    }
}

// The bin of a 256-bin histogram h (a wave's LDS slice) where the running count
// from the top (from_top) or from the bottom reaches need; before: the count of
// the bins passed over.
__device__ void find_bin(const uint32_t* h, bool from_top, int need, int& bin, int& before) {
  const int lane = threadIdx.x & 63;
  int c[4], tot = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int o = 4 * lane + q;  // lane l owns the order positions 4l .. 4l+3
    c[q] = (int)h[from_top ? 255 - o : o];
    tot += c[q];
  }
  const int incl = wave_scan_incl(tot);
  const int excl = incl - tot;
  const uint64_t hit = __ballot(excl < need && incl >= need);
  const int hl = __ffsll((unsigned long long)hit) - 1;
  int bef = excl, dg = 0;
  bool found = false;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (!found && bef + c[q] >= need) {
      dg = from_top ? 255 - (4 * lane + q) : 4 * lane + q;
      found = true;
    } else if (!found) {
      bef += c[q];
    }
  }
  bin = __builtin_amdgcn_readlane(dg, hl);
  before = __builtin_amdgcn_readlane(bef, hl);
}

// A value interval [lo, hi] that holds the rank-th largest (from_top) or
// smallest estimate of the row (1 <= rank <= number of valid elements): the
// elements are cut into 256 bins of equal width over the range of a cell (at
// first the whole row), the cell becomes the bin that holds the rank, and the
// rank is counted inside it, until the cell's range is at most tol wide or
// four levels are done. Bins are a monotone function of the value, so equal
// values share a bin and a higher bin never holds a smaller value. Once a cell
// holds at most 64 elements they move to one per lane (through tmp, the
// wave's 64 floats of LDS), so the later levels cost one value per lane
// instead of a sweep over the row.
template <int kMaxE>
__device__ void locate(const float (&a)[kMaxE], int E, uint64_t cell, int rank, bool from_top, float tol,
                       uint32_t* __restrict__ hist, float* __restrict__ tmp, float& lo, float& hi) {
  const int lane = threadIdx.x & 63;
  const uint64_t below = (1ull << lane) - 1ull;
  bool packed = false, xin = false;
  float x = 0.f;
  for (int level = 0;; ++level) {
    float mn = INFINITY, mx = -INFINITY;
    if (packed) {
      if (xin) mn = mx = x;
    } else {
#pragma unroll
      for (int e = 0; e < kMaxE; ++e) {
        if ((cell >> e) & 1ull) {
          mn = fminf(mn, a[e]);
          mx = fmaxf(mx, a[e]);
        }
      }
    }
    lo = wave_min(mn);
    hi = wave_max(mx);
    const float w = hi - lo;
    if (level == 4 || !(w > tol)) return;
    const float sc = 256.0f / w;
#pragma unroll
    for (int q = 0; q < 4; ++q) hist[64 * q + lane] = 0u;
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    if (packed) {
      if (xin) atomicAdd(&hist[min(255, (int)((x - lo) * sc))], 1u);
    } else {
#pragma unroll
      for (int e = 0; e < kMaxE; ++e) {
        if ((cell >> e) & 1ull) atomicAdd(&hist[min(255, (int)((a[e] - lo) * sc))], 1u);
      }
    }
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    int bin, before;
    find_bin(hist, from_top, rank, bin, before);
    rank -= before;
    if (packed) {
      xin = xin && min(255, (int)((x - lo) * sc)) == bin;
      continue;
    }
    uint64_t nc = 0ull;
    int cnt = 0;
#pragma unroll
    for (int e = 0; e < kMaxE; ++e) {
      const bool in = ((cell >> e) & 1ull) && min(255, (int)((a[e] - lo) * sc)) == bin;
      if (in) nc |= 1ull << e;
      cnt += __popcll(__ballot(in));
    }
    cell = nc;
    if (cnt <= 64) {  // one element of the new cell per lane
      int pos = 0;
#pragma unroll
      for (int e = 0; e < kMaxE; ++e) {
        const bool in = (nc >> e) & 1ull;
        const uint64_t b = __ballot(in);
        if (in) tmp[pos + __popcll(b & below)] = a[e];
        pos += __popcll(b);
      }
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      xin = lane < cnt;
      x = xin ? tmp[lane] : 0.f;
      packed = true;
    }
  }
}

// One band of a wave's row. [lo, hi] holds the n-th largest (TOP) or smallest
// estimate; among the elements of `avail`, those beyond [lo - eps2, hi + eps2]
// on the selected side are selected at once and those inside it are the
// candidates: if they are more than the rank still needs, they are ranked by
// their float64 logits (TOP: logit descending, index ascending; else logit
// ascending, index descending) and the first ones selected. wide: the bound
// decides nothing (every element is a candidate). Returns the selection as a
// per-lane bit mask over the lane's elements.
template <bool TOP, int kMaxE>
__device__ uint64_t band_select(const float (&a)[kMaxE], int E, uint64_t avail, float lo, float hi, float eps2,
                                bool wide, int n, int D, const double* __restrict__ qrow,
                                const double* __restrict__ pkh, uint16_t* __restrict__ lst) {
  const int lane = threadIdx.x & 63;
  const uint64_t below = (1ull << lane) - 1ull;
  const float blo = lo - eps2, bhi = hi + eps2;
  uint64_t sel = 0ull;
  int c_in = 0, m = 0;
#pragma unroll
  for (int e = 0; e < kMaxE; ++e) {
    const bool ok = (avail >> e) & 1ull;
    const bool in = ok && !wide && (TOP ? a[e] > bhi : a[e] < blo);
    const bool cand = ok && !in && (wide || (TOP ? a[e] >= blo : a[e] <= bhi));
    const uint64_t bc = __ballot(cand);
    if (in) sel |= 1ull << e;
    if (cand) lst[m + __popcll(bc & below)] = (uint16_t)(lane + 64 * e);
    c_in += __popcll(__ballot(in));
    m += __popcll(bc);
  }
  const int need = max(0, min(n - c_in, m));
  if (need == 0) return sel;
  const bool all = need == m;
  double q0 = 0.0, q1 = 0.0;
  if (!all) {
    q0 = qrow[lane];
    if (D > 64) q1 = qrow[lane + 64];
  }
  const double sd = sqrt((double)D);
  // lane c receives the float64 logit of candidate base + c, four candidates'
  // loads in flight at a time
  auto exact = [&](int base) -> double {
    double mine = 0.0;
    const int cnt = min(64, m - base);
    for (int c0 = 0; c0 < cnt; c0 += 4) {
      double v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const double* kr = pkh + (size_t)lst[base + min(c0 + u, cnt - 1)] * D;
        v[u] = q0 * kr[lane];
        if (D > 64) v[u] = fma(q1, kr[lane + 64], v[u]);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const double t = wave_sum_d(v[u]) / sd;
        if (lane == c0 + u) mine = t;
      }
    }
    return mine;
  };
  for (int a0 = 0; a0 < m; a0 += 64) {
    const int cnt_a = min(64, m - a0);
    const int ja = lane < cnt_a ? (int)lst[a0 + lane] : 0;
    bool pick = lane < cnt_a;
    if (!all) {
      const double ea = exact(a0);
      int rank = 0;
      for (int b0 = 0; b0 < m; b0 += 64) {
        const double eb = b0 == a0 ? ea : exact(b0);
        const int jb = lane < min(64, m - b0) ? (int)lst[b0 + lane] : 0;
        const int cnt = min(64, m - b0);
        for (int k = 0; k < cnt; ++k) {
          const double ek = readlane_d(eb, k);
          const int jk = __builtin_amdgcn_readlane(jb, k);
          rank += TOP ? (ek > ea || (ek == ea && jk < ja)) : (ek < ea || (ek == ea && jk > ja));
        }
      }
      pick = pick && rank < need;
    }
    // hand each picked candidate to the lane that owns its element
    const uint64_t picked = __ballot(pick);
    for (int k = 0; k < cnt_a; ++k) {
      const int jk = __builtin_amdgcn_readlane(ja, k);
      if (((picked >> k) & 1ull) && (jk & 63) == lane) sel |= 1ull << (jk >> 6);
    }
  }
  return sel;
}

// One wave per row of the [rows, Nb] estimates (rows = B*H*Nb).
template <int kMaxE>
__global__ __launch_bounds__(256) void k_classify_band(const float* __restrict__ est,
                                                       const float* __restrict__ qnorm,
                                                       const float* __restrict__ knmax,
                                                       const double* __restrict__ pq,
                                                       const double* __restrict__ pk, int8_t* __restrict__ mask,
                                                       int Nb, int nt, int D, int n_h, int n_l, int rows) {
  __shared__ uint32_t hist[4][256];
  __shared__ float tmp[4][64];             // a located cell, one element per lane
  __shared__ uint16_t lst[4][64 * kMaxE];  // a band's candidates, per wave
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + wave;
  if (row >= rows) return;  // whole wave; the kernel has no barrier
  const int bh = row / Nb;
  const int E = (Nb + 63) >> 6;
  const float* arow = est + (size_t)row * Nb;
  float a[kMaxE];
#pragma unroll
  for (int e = 0; e < kMaxE; ++e) a[e] = arow[min(lane + 64 * e, Nb - 1)];
  const float kmax = wave_max(lane < nt ? knmax[(size_t)bh * nt + lane] : 0.0f);
  uint64_t valid = 0ull;
#pragma unroll
  for (int e = 0; e < kMaxE; ++e)
    if (e < E && lane + 64 * e < Nb) valid |= 1ull << e;
  const float eps = kBandKappa * qnorm[row] * kmax / sqrtf((float)D) + kBandAbs;
  const bool wide = !(eps <= 1e30f);  // the bound overflowed float32: it decides nothing
  const double* qrow = pq + (size_t)row * D;
  const double* pkh = pk + (size_t)bh * Nb * D;
  uint64_t top = 0ull, bot = 0ull;
  if (n_h > 0) {
    float lo = 0.f, hi = 0.f;
    if (!wide) locate<kMaxE>(a, E, valid, n_h, true, eps, hist[wave], tmp[wave], lo, hi);
    top = band_select<true, kMaxE>(a, E, valid, lo, hi, 2.0f * eps, wide, n_h, D, qrow, pkh, lst[wave]);
  }
  if (n_l > 0) {
    const uint64_t rest = valid & ~top;
    float lo = 0.f, hi = 0.f;
    if (!wide) locate<kMaxE>(a, E, rest, n_l, false, eps, hist[wave], tmp[wave], lo, hi);
    bot = band_select<false, kMaxE>(a, E, rest, lo, hi, 2.0f * eps, wide, n_l, D, qrow, pkh, lst[wave]);
  }
  int8_t* mrow = mask + (size_t)row * Nb;
#pragma unroll
  for (int e = 0; e < kMaxE; ++e) {
    const int j = lane + 64 * e;
    if (j < Nb) mrow[j] = ((top >> e) & 1ull) ? (int8_t)1 : ((bot >> e) & 1ull) ? (int8_t)-1 : (int8_t)0;
  }
}

}  // namespace

hipError_t launch_select(const Dims& D, const double* pq, const double* pk, int8_t* mask,
                         uint16_t* hilo, float* est, float* norms, double* dbg_lg, hipStream_t s) {
  const int nt = (D.Nb + 63) / 64, nq = (D.Nb + 127) / 128;
  float* qn = norms;
  float* kn = norms + (size_t)D.BH * D.Nb;  // [BH, nt]
  const dim3 gs(nt, D.BH, 2), ge((unsigned)(nt * nq * D.BH));
  if (D.d == 128) {
    hipLaunchKernelGGL(k_split<128>, gs, dim3(64 * kSplitWaves), 0, s, pq, pk, hilo, qn, kn, D.Nb, nt, D.BH);
    hipLaunchKernelGGL(k_logits_est<128>, ge, dim3(256), 0, s, hilo, est, D.Nb, D.BH, nt, nq);
  } else {
    hipLaunchKernelGGL(k_split<64>, gs, dim3(64 * kSplitWaves), 0, s, pq, pk, hilo, qn, kn, D.Nb, nt, D.BH);
    hipLaunchKernelGGL(k_logits_est<64>, ge, dim3(256), 0, s, hilo, est, D.Nb, D.BH, nt, nq);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int rows = D.BH * D.Nb;
  const int E = (D.Nb + 63) / 64;
  // the row's elements in registers, every loop over them unrolled in full
  auto kern = E <= 2    ? k_classify_band<2>
              : E <= 4  ? k_classify_band<4>
              : E <= 8  ? k_classify_band<8>
              : E <= 12 ? k_classify_band<12>
              : E <= 16 ? k_classify_band<16>
              : E <= 20 ? k_classify_band<20>
              : E <= 24 ? k_classify_band<24>
              : E <= 32 ? k_classify_band<32>
              : E <= 48 ? k_classify_band<48>
                        : k_classify_band<64>;
  hipLaunchKernelGGL(kern, dim3((rows + 3) / 4), dim3(256), 0, s, est, qn, kn, pq, pk, mask, D.Nb, nt, D.d,
                     D.n_h, D.n_l, rows);
  e = hipGetLastError();
  if (e != hipSuccess || !dbg_lg) return e;
  dim3 g2(nt, nt, D.BH);
  if (D.d == 128)
    hipLaunchKernelGGL(k_logits<128>, g2, dim3(256), 0, s, pq, pk, dbg_lg, D.Nb);
  else
    hipLaunchKernelGGL(k_logits<64>, g2, dim3(256), 0, s, pq, pk, dbg_lg, D.Nb);
  return hipGetLastError();
}

}  // namespace sla
