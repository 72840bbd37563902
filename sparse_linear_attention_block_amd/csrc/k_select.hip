// K2: compressed scores and three-way block classification.
//
// SLA paper summary (aipaper.cc), section 4, Eq. 1 (Pc = softmax of the pooled
// logits, scaled by 1/sqrt(d)) and Eq. 2 (Mc = 1 for the top kh% of each row,
// -1 for the bottom kl%, 0 otherwise). Softmax is monotone in each row, so the
// ranking is taken on the logits themselves and Pc is never materialised.
//
// k_logits: the float64 logits of one (batch, head) as a GEMM on float64 MFMA
//   16x16x4, one 64 x 64 tile per workgroup: the 64 pooled keys of the tile are
//   staged once in LDS (padded rows), each wave keeps its 16 pooled queries in
//   registers. The logits go to HBM ([B*H, Nb, Nb] float64).
// k_classify: one wave per row finds the two class boundaries without sorting:
//  * every logit is rounded to float32 and mapped to an order-preserving
//    uint32 key (round-to-nearest is monotone, so key order never contradicts
//    float64 order);
//  * a radix select (top byte by a ballot search, then three 8-bit passes over
//    per-wave LDS histograms) finds the n_h-th largest key T and the n_l-th
//    smallest key L, both searches in the same sweeps;
//  * keys strictly above T are critical, strictly below L negligible; the few
//    elements whose key equals T (or L) are ordered exactly by their float64
//    logit and then by block index (lower index first), which reproduces the
//    total order (logit descending, index ascending) without approximation.
#include "sla_internal.h"
#include "dev_common.h"

namespace sla {
namespace {

__device__ __forceinline__ uint32_t order_key(double s) {
  float f = (float)s;
  if (f == 0.0f) f = 0.0f;  // -0 and +0 are the same logit
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int wave_count(bool p) {
  return __popcll(__ballot(p));
}

// The kt-th largest key T and the kb-th smallest key L of a wave's row
// (1 <= kt, kb <= number of valid keys), found together so that the two
// searches' latencies overlap: the top byte of each by a bitwise search with
// wave ballots, then three 8-bit radix passes, each a pair of 256-bin
// histograms in the wave's own LDS slice of the keys that match the digits
// found so far, scanned across lanes to find the bin where the running count
// reaches the rank. Equal keys are counted with their multiplicity, so T is the
// value v with #(keys above v) < kt <= #(keys at or above v), and L likewise
// from below.
template <int kMaxE>
__device__ void radix_select2(const uint32_t* key, int E, int Nb, int kt, int kb,
                              uint32_t* __restrict__ hist, uint32_t& T, uint32_t& L) {
  const int lane = threadIdx.x & 63;
  // #keys >= lo and #keys <= hi in one sweep (the top byte comes first: logits of
  // one row share few top bytes, which would serialise a first radix pass)
  auto count2 = [&](uint32_t lo, uint32_t hi, int& ct, int& cb) {
    ct = 0;
    cb = 0;
#pragma unroll
    for (int e = 0; e < kMaxE; ++e) {
      if (e >= E) break;
      const bool valid = lane + 64 * e < Nb;
      ct += __popcll(__ballot(valid && key[e] >= lo));
      cb += __popcll(__ballot(valid && key[e] <= hi));
    }
  };
  uint32_t tbt = 0, tbb = 255;
  int nt = kt, nb = kb;
  for (int bit = 7; bit >= 0; --bit) {
    const uint32_t ct_cand = tbt | (1u << bit), cb_cand = tbb & ~(1u << bit);
    int ct, cb;
    count2(ct_cand << 24, (cb_cand << 24) | 0xffffffu, ct, cb);
    if (ct >= nt) tbt = ct_cand;
    if (cb >= nb) tbb = cb_cand;
  }
  {
    int ct, cb;
    count2(tbt < 255 ? (tbt + 1) << 24 : 0xffffffffu, tbb > 0 ? (tbb << 24) - 1u : 0u, ct, cb);
    if (tbt < 255) nt -= ct;
    if (tbb > 0) nb -= cb;
  }
  uint32_t pt = tbt << 24, pb = tbb << 24, pmask = 0xff000000u;
  uint32_t* ht = hist;
  uint32_t* hb = hist + 256;
  // the bin where the running count from the top (or the bottom) reaches need
  auto find = [&](const uint32_t* h, bool from_top, int need, int& digit, int& before) {
    int c[4], tot = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int o = 4 * lane + q;  // lane l owns the order positions 4l .. 4l+3
      c[q] = (int)h[from_top ? 255 - o : o];
      tot += c[q];
    }
    int incl = tot;  // inclusive scan over lanes
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(incl, off);
      if (lane >= off) incl += v;
    }
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
    digit = __shfl(dg, hl);
    before = __shfl(bef, hl);
  };
  for (int pass = 1; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      ht[64 * q + lane] = 0u;
      hb[64 * q + lane] = 0u;
    }
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
#pragma unroll
    for (int e = 0; e < kMaxE; ++e) {
      if (e >= E) break;
      if (lane + 64 * e >= Nb) continue;
      const uint32_t bin = (key[e] >> shift) & 255u;
      if ((key[e] & pmask) == pt) atomicAdd(&ht[bin], 1u);
      if ((key[e] & pmask) == pb) atomicAdd(&hb[bin], 1u);
    }
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    int dt, bt, db, bb;
    find(ht, true, nt, dt, bt);
    find(hb, false, nb, db, bb);
    nt -= bt;
    nb -= bb;
    pt |= (uint32_t)dt << shift;
    pb |= (uint32_t)db << shift;
    pmask |= 0xffu << shift;
  }
  T = pt;
  L = pb;
}

// One wave classifies one row of Nb float64 logits (Nb <= 64 * kMaxE).
template <int kMaxE>
__device__ void classify_row(const double* __restrict__ lg, int Nb, int n_h, int n_l,
                             int8_t* __restrict__ mrow, uint32_t* __restrict__ hist) {
  const int lane = threadIdx.x & 63;
  const int E = (Nb + 63) >> 6;
  uint32_t key[kMaxE];
  double v[kMaxE];
  // all loads first (slots past Nb re-read the last logit), then the keys
#pragma unroll
  for (int e = 0; e < kMaxE; ++e) v[e] = lg[min(lane + 64 * e, Nb - 1)];
#pragma unroll
  for (int e = 0; e < kMaxE; ++e) {
    const int j = lane + 64 * e;
    key[e] = (e < E && j < Nb) ? order_key(v[e]) : 0u;
  }
  // T: the n_h-th largest key; L: the n_l-th smallest key (a side with no
  // blocks is searched at rank 1 and then ignored)
  uint32_t T, L;
  radix_select2<kMaxE>(key, E, Nb, max(n_h, 1), max(n_l, 1), hist, T, L);
  if (n_h == 0) T = 0u;
  if (n_l == 0) L = 0xffffffffu;
  // sizes of the strict parts and of the tie groups at the two boundaries, in one sweep
  int ge1 = 0, ge0 = 0, le1 = 0, le0 = 0;
#pragma unroll
  for (int e = 0; e < kMaxE; ++e) {
    if (e >= E) break;
    const bool valid = lane + 64 * e < Nb;
    ge1 += wave_count(valid && T != 0xffffffffu && key[e] >= T + 1);
    ge0 += wave_count(valid && key[e] >= T);
    le1 += wave_count(valid && L != 0u && key[e] <= L - 1);
    le0 += wave_count(valid && key[e] <= L);
  }
  const int gt_h = n_h > 0 ? ge1 : 0;
  const int need_h = n_h > 0 ? n_h - gt_h : 0;
  const int grp_h = n_h > 0 ? ge0 - gt_h : 0;
  const int lt_l = n_l > 0 ? le1 : 0;
  const int need_l = n_l > 0 ? n_l - lt_l : 0;
  const int grp_l = n_l > 0 ? le0 - lt_l : 0;

#pragma unroll
  for (int e = 0; e < kMaxE; ++e) {
    if (e >= E) break;
    const int j = lane + 64 * e;
    if (j >= Nb) continue;
    int8_t m = 0;
    if (n_h > 0 && key[e] > T) {
      m = 1;
    } else if (n_h > 0 && key[e] == T) {
      if (grp_h == need_h) {
        m = 1;
      } else {  // rank inside the tie group by (float64 logit desc, index asc)
        const double sj = lg[j];
        int rank = 0;
        for (int k = 0; k < Nb; ++k) {
          const double sk = lg[k];
          if (order_key(sk) == T && (sk > sj || (sk == sj && k < j))) ++rank;
        }
        if (rank < need_h) m = 1;
      }
    }
    if (m == 0 && n_l > 0) {
      if (key[e] < L) {
        m = -1;
      } else if (key[e] == L) {
        if (grp_l == need_l) {
          m = -1;
        } else {  // the tail of the tie group: smallest logit, then highest index
          const double sj = lg[j];
          int rank = 0;
          for (int k = 0; k < Nb; ++k) {
            const double sk = lg[k];
            if (order_key(sk) == L && (sk < sj || (sk == sj && k > j))) ++rank;
          }
          if (rank < need_l) m = -1;
        }
      }
    }
    mrow[j] = m;
  }
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

// one wave per row of the [rows, Nb] logits
template <int kMaxE>
__global__ __launch_bounds__(256) void k_classify(const double* __restrict__ lg,
                                                  int8_t* __restrict__ mask, int Nb, int n_h,
                                                  int n_l, int rows) {
  __shared__ uint32_t hist[4][512];  // two histograms per wave
  const int wave = threadIdx.x >> 6;
  const int row = blockIdx.x * 4 + wave;
  if (row >= rows) return;  // whole wave; the kernel has no barrier
  classify_row<kMaxE>(lg + (size_t)row * Nb, Nb, n_h, n_l, mask + (size_t)row * Nb, hist[wave]);
}

}  // namespace

hipError_t launch_select(const Dims& D, const double* pq, const double* pk, int8_t* mask,
                         double* lg, hipStream_t s) {
  const int nt = (D.Nb + 63) / 64;
  dim3 g1(nt, nt, D.BH);
  if (D.d == 128)
    hipLaunchKernelGGL(k_logits<128>, g1, dim3(256), 0, s, pq, pk, lg, D.Nb);
  else
    hipLaunchKernelGGL(k_logits<64>, g1, dim3(256), 0, s, pq, pk, lg, D.Nb);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int rows = D.BH * D.Nb;
  const int E = (D.Nb + 63) / 64;
  auto kern = E <= 8 ? k_classify<8> : E <= 16 ? k_classify<16> : E <= 32 ? k_classify<32> : k_classify<64>;
  hipLaunchKernelGGL(kern, dim3((rows + 3) / 4), dim3(256), 0, s, lg, mask, D.Nb, D.n_h, D.n_l, rows);
  return hipGetLastError();
}

}  // namespace sla
