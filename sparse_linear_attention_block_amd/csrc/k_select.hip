// K2: compressed scores and three-way block classification.
//
// SLA paper summary (aipaper.cc), section 4, Eq. 1 (Pc = softmax of the pooled
// logits, scaled by 1/sqrt(d)) and Eq. 2 (Mc = 1 for the top kh% of each row,
// -1 for the bottom kl%, 0 otherwise). Softmax is monotone in each row, so the
// ranking is taken on the logits themselves and Pc is never materialised.
//
// One workgroup owns R query-block rows of one (batch, head). Phase 1 forms
// the R x Nb float64 logits in LDS (k-bar rows stream from L2). Phase 2 gives
// each row to one wave, which finds the two class boundaries without sorting:
//  * every logit is rounded to float32 and mapped to an order-preserving
//    uint32 key (round-to-nearest is monotone, so key order never contradicts
//    float64 order);
//  * a 32-step bitwise search over the key finds the n_h-th largest key T and
//    the n_l-th smallest key L, counting with wave ballots;
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

// One wave classifies one row of Nb logits held in LDS (Nb <= 64 * kMaxE).
template <int kMaxE>
__device__ void classify_row(const double* __restrict__ lg, int Nb, int n_h, int n_l,
                             int8_t* __restrict__ mrow) {
  const int lane = threadIdx.x & 63;
  const int E = (Nb + 63) >> 6;
  uint32_t key[kMaxE];
#pragma unroll
  for (int e = 0; e < kMaxE; ++e) {
    const int j = lane + 64 * e;
    key[e] = (e < E && j < Nb) ? order_key(lg[j]) : 0u;
  }
  // counts over valid elements only: invalid slots carry key 0 and are masked
  auto cnt_ge = [&](uint32_t t) {
    int c = 0;
#pragma unroll
    for (int e = 0; e < kMaxE; ++e) {
      if (e >= E) break;
      const int j = lane + 64 * e;
      c += wave_count(j < Nb && key[e] >= t);
    }
    return c;
  };
  auto cnt_le = [&](uint32_t t) {
    int c = 0;
#pragma unroll
    for (int e = 0; e < kMaxE; ++e) {
      if (e >= E) break;
      const int j = lane + 64 * e;
      c += wave_count(j < Nb && key[e] <= t);
    }
    return c;
  };

  // T: largest key with at least n_h keys >= T; L: smallest key with at least n_l keys <= L
  uint32_t T = 0, L = 0xffffffffu;
  if (n_h > 0) {
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = T | (1u << bit);
      if (cnt_ge(cand) >= n_h) T = cand;
    }
  }
  if (n_l > 0) {
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = L & ~(1u << bit);
      if (cnt_le(cand) >= n_l) L = cand;
    }
  }
  // sizes of the strict parts and of the tie groups at the two boundaries
  const int gt_h = (n_h > 0 && T != 0xffffffffu) ? cnt_ge(T + 1) : 0;
  const int need_h = n_h > 0 ? n_h - gt_h : 0;
  const int grp_h = n_h > 0 ? cnt_ge(T) - gt_h : 0;
  const int lt_l = (n_l > 0 && L != 0u) ? cnt_le(L - 1) : 0;
  const int need_l = n_l > 0 ? n_l - lt_l : 0;
  const int grp_l = n_l > 0 ? cnt_le(L) - lt_l : 0;

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

template <int kMaxE>
__global__ __launch_bounds__(256) void k_select(const double* __restrict__ pq,
                                                const double* __restrict__ pk,
                                                int8_t* __restrict__ mask,
                                                double* __restrict__ dbg_logits, int Nb, int d,
                                                int n_h, int n_l, int R) {
  extern __shared__ double lds[];
  double* qs = lds;            // [8][d], rows past the workgroup's R are zero
  double* lg = lds + 8 * d;    // [R][Nb]
  const int tid = threadIdx.x;
  const int bh = blockIdx.y;
  const int i0 = blockIdx.x * R;
  const int nr = min(R, Nb - i0);
  const double* Pq = pq + ((size_t)bh * Nb + i0) * d;
  const double* Pk = pk + (size_t)bh * Nb * d;
  for (int x = tid; x < 8 * d; x += 256) qs[x] = x < nr * d ? Pq[x] : 0.0;  // rows past nr: 0
  __syncthreads();
  const double sd = sqrt((double)d);
  // one key row per thread; its d values arrive in batches of 16 double2
  // loads issued back to back, so each batch costs one memory latency
  for (int j = tid; j < Nb; j += 256) {
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    const double2* kr = reinterpret_cast<const double2*>(Pk + (size_t)j * d);
    for (int cb = 0; cb < d / 2; cb += 16) {
      double2 kv[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) kv[u] = kr[cb + u];
#pragma unroll
      for (int u = 0; u < 16; ++u)
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const double2 qv = *reinterpret_cast<const double2*>(&qs[r * d + 2 * (cb + u)]);
          acc[r] = fma(qv.x, kv[u].x, acc[r]);
          acc[r] = fma(qv.y, kv[u].y, acc[r]);
        }
    }
#pragma unroll
    for (int r = 0; r < 8; ++r)
      if (r < nr) lg[r * Nb + j] = acc[r] / sd;
  }
  __syncthreads();
  if (dbg_logits) {
    double* out = dbg_logits + ((size_t)bh * Nb + i0) * Nb;
    for (int x = tid; x < nr * Nb; x += 256) out[x] = lg[x];
  }
  const int wave = tid >> 6;
  for (int r = wave; r < nr; r += 4)
    classify_row<kMaxE>(lg + (size_t)r * Nb, Nb, n_h, n_l, mask + ((size_t)bh * Nb + i0 + r) * Nb);
}

}  // namespace

hipError_t launch_select(const Dims& D, const double* pq, const double* pk, int8_t* mask,
                         double* dbg_logits, hipStream_t s) {
  // R rows per workgroup, bounded by LDS (logits + pooled queries in float64)
  int R = 8;  // the logits loop always computes 8 rows; fewer are kept when LDS is short
  while (R > 1 && (size_t)8 * D.d * sizeof(double) + (size_t)R * D.Nb * sizeof(double) > 64 * 1024) R >>= 1;
  const size_t lds = ((size_t)8 * D.d + (size_t)R * D.Nb) * sizeof(double);
  dim3 grid((D.Nb + R - 1) / R, D.BH);
  const int E = (D.Nb + 63) / 64;
  auto kern = E <= 8 ? k_select<8> : E <= 16 ? k_select<16> : E <= 32 ? k_select<32> : k_select<64>;
  hipLaunchKernelGGL(kern, grid, dim3(256), lds, s, pq, pk, mask, dbg_logits, D.Nb, D.d,
                     D.n_h, D.n_l, R);
  return hipGetLastError();
}

}  // namespace sla
