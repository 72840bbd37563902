// K5: block-sparse softmax attention over the critical blocks, the linear
// branch output and the SLA2 mix, one workgroup per query block.
//
// Sparse branch: SLA paper summary (aipaper.cc), section 4 step 3, first
// bullet, and SLA explainer (intelliparadigm.com), section 2.2 items 2-3:
// FlashAttention restricted to the blocks with Mc = 1, online softmax, the N x N
// score matrix is never stored; negligible blocks are skipped. The softmax is
// normalised over the critical keys only (SLA2 article, the scale-mismatch
// paragraph). Linear branch: Eq. 3, O_l = phi(Q_i) H_i / (phi(Q_i) Z_i) with
// H_i, Z_i summed by K4. Mix: O = alpha_h O_s + (1 - alpha_h) O_l (SLA2
// article, mixing-ratio paragraph).
//
// bf16 path. The critical list of the row is compacted from the mask into LDS
// with wave ballots (the lookup table of the SLA explainer, section 2.3, built
// on chip per query block). Each of the 4 waves owns 16 queries. Per critical
// key tile (64 keys) the workgroup stages K (row-major) and V^T (from K3) in
// LDS, double-buffered with register prefetch of the next tile, then:
//   S^T = K Q^T    MFMA 16x16x32: K rows as A, the wave's Q (registers) as B;
//                  each lane gets 4 consecutive keys of one query;
//   online softmax in the exp2 domain, row max over the 4 lane groups;
//   O^T += V^T P^T MFMA 16x16x32: P^T never leaves registers - the 8 k slots
//                  of a lane are its keys {4g..4g+3, 16+4g..16+4g+3} and the
//                  V^T operand is read from LDS in the same key order.
// Epilogue: O_s = acc / l; phi(Q) from the Q registers (softmax over the d
// features in f32, rounded to bf16); num^T = H_i^T phi(Q)^T on MFMA with H_i^T
// read straight from K4's output; den = phi(Q) . Z_i; O_l = num / den;
// O = alpha O_s + (1 - alpha) O_l, rows past N not written.
// Workgroups are remapped so that each XCD walks a contiguous range of
// (batch, head, query block): neighbouring query blocks share most critical
// key tiles, which then come from the XCD's L2.
//
// f32 path: 4 threads per query, plain FMA, one key at a time.
#include "sla_internal.h"
#include "dev_common.h"

namespace sla {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ int xcd_remap(int L, int T) {
  const int q = T >> 3, rm = T & 7;
  const int x = L & 7, pos = L >> 3;
  return x * q + min(x, rm) + pos;
}

// Compacts the indices j with mrow[j] == value, ascending, into list; returns the count.
__device__ int compact_row(const int8_t* __restrict__ mrow, int Nb, int8_t value,
                           uint16_t* list, int* wsum) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int total = 0;
  for (int base = 0; base < Nb; base += 256) {
    const int j = base + tid;
    const bool f = (j < Nb) && (mrow[j] == value);
    const uint64_t bal = __ballot(f);
    const int before = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wsum[wave] = __popcll(bal);
    __syncthreads();
    int off = total;
    for (int w = 0; w < wave; ++w) off += wsum[w];
    if (f) list[off + before] = (uint16_t)j;
    total += wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
  }
  return total;
}

template <int D>
struct FaCfg {
  static constexpr int KS = D + 8;   // K tile row stride (elements), 16-byte aligned rows
  static constexpr int VS = 64 + 4;  // V^T tile row stride (elements), 8-byte aligned rows
  static constexpr int NN = D * D + D;
  static constexpr int KCH = kBlock * D / 8 / 256;  // 16-byte K chunks per thread
  static constexpr int VCH = D * kBlock / 8 / 256;  // 16-byte V^T chunks per thread
};

template <int D>
__global__ __launch_bounds__(256, 2) void k_sparse_bf16(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ vt, const int8_t* __restrict__ mask,
    const uint16_t* __restrict__ Hx, const float* __restrict__ alpha, uint16_t* __restrict__ O,
    float* __restrict__ dbg_os, float* __restrict__ dbg_ol, int H, int N, int Nb) {
  using C = FaCfg<D>;
  constexpr int KS = C::KS, VS = C::VS, NN = C::NN, KCH = C::KCH, VCH = C::VCH;
  constexpr int KSTEPS = D / 32;
  constexpr int FT = D / 16;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][kBlock][KS];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][D][VS];
  __shared__ uint16_t list[kMaxNb];
  __shared__ int wsum[4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int T = gridDim.x;
  const int id = xcd_remap(blockIdx.x, T);
  const int bh = id / Nb, i = id - bh * Nb;
  const int h = bh % H;

  const int8_t* mrow = mask + ((size_t)bh * Nb + i) * Nb;
  const int ncrit = compact_row(mrow, Nb, (int8_t)1, list, wsum);

  // the wave's 16 queries as MFMA B operands: Q[t][32ks + 8g .. +7]
  const int tq = i * kBlock + wave * 16 + l16;
  const bool qvalid = tq < N;
  const uint16_t* qrow = Q + ((size_t)bh * N + (qvalid ? tq : 0)) * D;
  uint4 qr[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks)
    qr[ks] = qvalid ? *reinterpret_cast<const uint4*>(qrow + 32 * ks + 8 * g)
                    : make_uint4(0, 0, 0, 0);

  const uint16_t* Kb = K + (size_t)bh * N * D;
  const uint16_t* Vb = vt + (size_t)bh * Nb * D * kBlock;
  uint4 kreg[KCH], vreg[VCH];
  auto load_tile = [&](int j) {
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
      const int x = tid + 256 * u;
      const int key = x / (D / 8), ch = x % (D / 8);
      const int t = j * kBlock + key;
      kreg[u] = t < N ? *reinterpret_cast<const uint4*>(Kb + (size_t)t * D + ch * 8)
                      : make_uint4(0, 0, 0, 0);
    }
    const uint16_t* vsrc = Vb + (size_t)j * D * kBlock;
#pragma unroll
    for (int u = 0; u < VCH; ++u) {
      const int x = tid + 256 * u;
      vreg[u] = *reinterpret_cast<const uint4*>(vsrc + (size_t)x * 8);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
      const int x = tid + 256 * u;
      const int key = x / (D / 8), ch = x % (D / 8);
      *reinterpret_cast<uint4*>(&Ks[buf][key][ch * 8]) = kreg[u];
    }
#pragma unroll
    for (int u = 0; u < VCH; ++u) {
      const int x = tid + 256 * u;
      const int c = x / 8, ch = x % 8;
      uint2* dst = reinterpret_cast<uint2*>(&Vs[buf][c][ch * 8]);
      dst[0] = make_uint2(vreg[u].x, vreg[u].y);
      dst[1] = make_uint2(vreg[u].z, vreg[u].w);
    }
  };

  const float sc = kLog2e / sqrtf((float)D);
  f32x4 acc[FT];
#pragma unroll
  for (int ft = 0; ft < FT; ++ft) acc[ft] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_part = 0.f;

  if (ncrit > 0) {
    load_tile(list[0]);
    store_tile(0);
  }
  __syncthreads();
  for (int c = 0; c < ncrit; ++c) {
    const int buf = c & 1;
    const int j = list[c];
    if (c + 1 < ncrit) load_tile(list[c + 1]);
    // S^T tile: 64 keys x 16 queries
    f32x4 s[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      s[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        const uint4 a = *reinterpret_cast<const uint4*>(&Ks[buf][16 * kt + l16][32 * ks + 8 * g]);
        s[kt] = mfma_bf16(a, qr[ks], s[kt]);
      }
    }
    const bool ragged = (j + 1) * kBlock > N;
    float tmax = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float x = s[kt][r] * sc;
        if (ragged && j * kBlock + 16 * kt + 4 * g + r >= N) x = -INFINITY;
        s[kt][r] = x;
        tmax = fmaxf(tmax, x);
      }
    tmax = group4_max(tmax);
    const float m_new = fmaxf(m_run, tmax);
    const float corr = exp2f(m_run - m_new);
    m_run = m_new;
    float lsum = 0.f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = exp2f(s[kt][r] - m_new);
        s[kt][r] = p;
        lsum += p;
      }
    l_part = l_part * corr + lsum;
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) acc[ft] *= corr;
    uint4 pb[2];
#pragma unroll
    for (int u = 0; u < 2; ++u)
      pb[u] = make_uint4(pack_bf2(s[2 * u][0], s[2 * u][1]), pack_bf2(s[2 * u][2], s[2 * u][3]),
                         pack_bf2(s[2 * u + 1][0], s[2 * u + 1][1]),
                         pack_bf2(s[2 * u + 1][2], s[2 * u + 1][3]));
#pragma unroll
    for (int ft = 0; ft < FT; ++ft)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const uint2 lo = *reinterpret_cast<const uint2*>(&Vs[buf][16 * ft + l16][32 * u + 4 * g]);
        const uint2 hi =
            *reinterpret_cast<const uint2*>(&Vs[buf][16 * ft + l16][32 * u + 16 + 4 * g]);
        acc[ft] = mfma_bf16(make_uint4(lo.x, lo.y, hi.x, hi.y), pb[u], acc[ft]);
      }
    if (c + 1 < ncrit) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: sparse output, linear branch, mix
  const float l = group4_sum(l_part);
  const float inv_l = (ncrit > 0 && l > 0.f) ? 1.0f / l : 0.f;

  // phi(Q): softmax over the D features of the lane's query, lane holds 8*KSTEPS of them
  float qf[KSTEPS * 8];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    const uint32_t w[4] = {qr[ks].x, qr[ks].y, qr[ks].z, qr[ks].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qf[ks * 8 + 2 * e] = bf_lo(w[e]);
      qf[ks * 8 + 2 * e + 1] = bf_hi(w[e]);
    }
  }
  float qm = -INFINITY;
#pragma unroll
  for (int e = 0; e < KSTEPS * 8; ++e) qm = fmaxf(qm, qf[e]);
  qm = group4_max(qm);
  float qsum = 0.f;
#pragma unroll
  for (int e = 0; e < KSTEPS * 8; ++e) {
    qf[e] = __expf(qf[e] - qm);
    qsum += qf[e];
  }
  const float qinv = 1.0f / group4_sum(qsum);
  const uint16_t* Hrow = Hx + ((size_t)bh * Nb + i) * NN;
  uint4 fq[KSTEPS];
  float den_part = 0.f;
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = pack_bf2(qf[ks * 8 + 2 * e] * qinv, qf[ks * 8 + 2 * e + 1] * qinv);
    fq[ks] = make_uint4(w[0], w[1], w[2], w[3]);
    const uint4 z = *reinterpret_cast<const uint4*>(Hrow + D * D + 32 * ks + 8 * g);
    const uint32_t zw[4] = {z.x, z.y, z.z, z.w};
#pragma unroll
    for (int e = 0; e < 4; ++e)
      den_part += bf_lo(w[e]) * bf_lo(zw[e]) + bf_hi(w[e]) * bf_hi(zw[e]);
  }
  const float den = group4_sum(den_part);
  const float inv_den = den > 0.f ? 1.0f / den : 0.f;
  const float al = alpha[h];
  const size_t orow = ((size_t)bh * N + tq) * D;
#pragma unroll
  for (int ft = 0; ft < FT; ++ft) {
    f32x4 nm = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const uint4 a =
          *reinterpret_cast<const uint4*>(Hrow + (size_t)(16 * ft + l16) * D + 32 * ks + 8 * g);
      nm = mfma_bf16(a, fq[ks], nm);
    }
    float os[4], ol[4], o[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      os[r] = acc[ft][r] * inv_l;
      ol[r] = nm[r] * inv_den;
      o[r] = al * os[r] + (1.0f - al) * ol[r];
    }
    if (qvalid) {
      const int c0 = 16 * ft + 4 * g;
      *reinterpret_cast<uint2*>(O + orow + c0) =
          make_uint2(pack_bf2(o[0], o[1]), pack_bf2(o[2], o[3]));
      if (dbg_os) *reinterpret_cast<float4*>(dbg_os + orow + c0) = make_float4(os[0], os[1], os[2], os[3]);
      if (dbg_ol) *reinterpret_cast<float4*>(dbg_ol + orow + c0) = make_float4(ol[0], ol[1], ol[2], ol[3]);
    }
  }
}

// ---------------------------------------------------------------- f32 path
template <int D>
__global__ __launch_bounds__(256) void k_sparse_f32(const float* __restrict__ Q,
                                                    const float* __restrict__ K,
                                                    const float* __restrict__ V,
                                                    const int8_t* __restrict__ mask,
                                                    const float* __restrict__ Hx,
                                                    const float* __restrict__ alpha,
                                                    float* __restrict__ O,
                                                    float* __restrict__ dbg_os,
                                                    float* __restrict__ dbg_ol, int H, int N,
                                                    int Nb) {
  constexpr int P = D / 4;  // features per thread
  constexpr int NN = D * D + D;
  __shared__ float Ks[kBlock][D];
  __shared__ float Vs[kBlock][D];
  __shared__ uint16_t list[kMaxNb];
  __shared__ int wsum[4];
  const int tid = threadIdx.x;
  const int bh = blockIdx.y, i = blockIdx.x, h = bh % H;
  const int row = tid >> 2, part = tid & 3;
  const int t = i * kBlock + row;
  const bool valid = t < N;
  const int8_t* mrow = mask + ((size_t)bh * Nb + i) * Nb;
  const int ncrit = compact_row(mrow, Nb, (int8_t)1, list, wsum);

  float q[P], acc[P];
  const float* qp = Q + ((size_t)bh * N + (valid ? t : 0)) * D + part * P;
#pragma unroll
  for (int e = 0; e < P; ++e) {
    q[e] = valid ? qp[e] : 0.f;
    acc[e] = 0.f;
  }
  const float scale = 1.0f / sqrtf((float)D);
  float m = -INFINITY, l = 0.f;
  for (int c = 0; c < ncrit; ++c) {
    const int j = list[c];
    __syncthreads();
    for (int x = tid; x < kBlock * D; x += 256) {
      const int key = x / D;
      const int tk = j * kBlock + key;
      Ks[key][x % D] = tk < N ? K[((size_t)bh * N + tk) * D + x % D] : 0.f;
      Vs[key][x % D] = tk < N ? V[((size_t)bh * N + tk) * D + x % D] : 0.f;
    }
    __syncthreads();
    const int nk = min(kBlock, N - j * kBlock);
    for (int key = 0; key < nk; ++key) {
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < P; ++e) s = fmaf(q[e], Ks[key][part * P + e], s);
      s += __shfl_xor(s, 1);
      s += __shfl_xor(s, 2);
      s *= scale;
      const float mn = fmaxf(m, s);
      const float corr = expf(m - mn);
      const float p = expf(s - mn);
      l = l * corr + p;
#pragma unroll
      for (int e = 0; e < P; ++e) acc[e] = fmaf(p, Vs[key][part * P + e], acc[e] * corr);
      m = mn;
    }
  }
  // linear branch
  float qm = -INFINITY;
#pragma unroll
  for (int e = 0; e < P; ++e) qm = fmaxf(qm, q[e]);
  qm = fmaxf(qm, __shfl_xor(qm, 1));
  qm = fmaxf(qm, __shfl_xor(qm, 2));
  float f[P], fs = 0.f;
#pragma unroll
  for (int e = 0; e < P; ++e) {
    f[e] = expf(q[e] - qm);
    fs += f[e];
  }
  fs += __shfl_xor(fs, 1);
  fs += __shfl_xor(fs, 2);
  const float finv = 1.0f / fs;
#pragma unroll
  for (int e = 0; e < P; ++e) f[e] *= finv;
  const float* Hrow = Hx + ((size_t)bh * Nb + i) * NN;
  float den = 0.f;
#pragma unroll
  for (int e = 0; e < P; ++e) den = fmaf(f[e], Hrow[D * D + part * P + e], den);
  den += __shfl_xor(den, 1);
  den += __shfl_xor(den, 2);
  float num[P];
#pragma unroll
  for (int e = 0; e < P; ++e) num[e] = 0.f;
  const int lane = tid & 63;
  for (int r = 0; r < D; ++r) {
    const int src = (lane & ~3) | (r / P);
    float fr = 0.f;
#pragma unroll
    for (int e = 0; e < P; ++e)
      if (e == r % P) fr = f[e];
    fr = __shfl(fr, src);
#pragma unroll
    for (int e = 0; e < P; ++e) num[e] = fmaf(fr, Hrow[(size_t)(part * P + e) * D + r], num[e]);
  }
  if (!valid) return;
  const float inv_l = (ncrit > 0 && l > 0.f) ? 1.0f / l : 0.f;
  const float inv_den = den > 0.f ? 1.0f / den : 0.f;
  const float al = alpha[h];
  const size_t orow = ((size_t)bh * N + t) * D + part * P;
#pragma unroll
  for (int e = 0; e < P; ++e) {
    const float os = acc[e] * inv_l, ol = num[e] * inv_den;
    O[orow + e] = al * os + (1.0f - al) * ol;
    if (dbg_os) dbg_os[orow + e] = os;
    if (dbg_ol) dbg_ol[orow + e] = ol;
  }
}

}  // namespace

hipError_t launch_sparse(const Dims& D, const void* Q, const void* K, const int8_t* mask,
                         const float* alpha, const Work& w, void* O, float* dbg_os,
                         float* dbg_ol, hipStream_t s) {
  if (D.bf16) {
    const int T = D.BH * D.Nb;
    if (D.d == 128)
      hipLaunchKernelGGL(k_sparse_bf16<128>, dim3(T), dim3(256), 0, s, (const uint16_t*)Q,
                         (const uint16_t*)K, w.vt, mask, (const uint16_t*)w.Hx, alpha,
                         (uint16_t*)O, dbg_os, dbg_ol, D.H, D.N, D.Nb);
    else
      hipLaunchKernelGGL(k_sparse_bf16<64>, dim3(T), dim3(256), 0, s, (const uint16_t*)Q,
                         (const uint16_t*)K, w.vt, mask, (const uint16_t*)w.Hx, alpha,
                         (uint16_t*)O, dbg_os, dbg_ol, D.H, D.N, D.Nb);
  } else {
    // the f32 path reads V directly; vt is not formed
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_sparse_f32(const Dims& D, const void* Q, const void* K, const void* V,
                             const int8_t* mask, const float* alpha, const Work& w, void* O,
                             float* dbg_os, float* dbg_ol, hipStream_t s) {
  dim3 grid(D.Nb, D.BH);
  if (D.d == 128)
    hipLaunchKernelGGL(k_sparse_f32<128>, grid, dim3(256), 0, s, (const float*)Q,
                       (const float*)K, (const float*)V, mask, (const float*)w.Hx, alpha,
                       (float*)O, dbg_os, dbg_ol, D.H, D.N, D.Nb);
  else
    hipLaunchKernelGGL(k_sparse_f32<64>, grid, dim3(256), 0, s, (const float*)Q,
                       (const float*)K, (const float*)V, mask, (const float*)w.Hx, alpha,
                       (float*)O, dbg_os, dbg_ol, D.H, D.N, D.Nb);
  return hipGetLastError();
}

}  // namespace sla
