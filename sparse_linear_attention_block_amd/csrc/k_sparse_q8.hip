// K5 with the 8-bit sparse branch: int8 Q.K^T and OCP fp8 e4m3 P.V.
//
// SLA2 article (mcffsbgs.com), quantisation-aware paragraph: the sparse branch
// computes with Q, K, P and V in 8 bits, each with a scale that is restored
// after the product; the linear branch stays in 16 bits. Everything else is
// the bf16 kernel's arithmetic (SLA paper summary, section 4 step 3 and Eq. 3;
// SLA2 article, scale-mismatch and mixing-ratio paragraphs).
//
// Scales and smoothing: Q and K are smoothed by their channel means over the
// head's tokens (q.k splits into (q - q̄).(k - k̄), a per-key float32 bias
// q̄.(k - k̄) and a per-query constant that cancels in the softmax; see
// k_quant.hip). K8 and its per-block absmax/127 scales and the bias come from
// the K quantisation kernel; the workgroup quantises its own 64 queries (one
// absmax/127 scale for the block) into registers, so Q8 never reaches HBM.
// V8^T carries one absmax/448 scale per block (written by the h/z kernel).
// P is quantised per query row over the 128 keys that one fp8 product
// contracts: P' = P~ * s_V(key block) (the V scale is folded into P, since
// the two tiles of one product may come from blocks with different V scales),
// s_P = 2^ceil(log2(rowmax(P') / 448)) (a power of two, so the largest code
// lies in (224, 448]), P8 = e4m3(P' / s_P), and acc += s_P * (V8^T P8) with
// s_P applied by the fp8 product as its E8M0 block scale.
// The softmax denominator l sums the unquantised P~.
//
// One workgroup of 4 waves per query block; wave w owns queries 16w .. 16w+15
// against all 64 keys of each tile, and tiles go in pairs (128 keys, one
// 16x16x128 fp8 product per feature tile). Per pair:
//   S^T = K8 Q8^T  int8 MFMA 16x16x64 to int32, the keys (LDS, row-swizzled)
//                  as A, the wave's queries (registers) as B; a lane gets keys
//                  16kt + 4g + r (kt, r = 0..3) of query l16 from each tile;
//   dequantise (s_Q s_K / sqrt(d)) and add the key bias, online softmax
//                  against a lazily raised reference max as in the bf16 kernel;
//   O^T += V8^T P8^T  fp8 MFMA 16x16x128: a lane group's 32 k slots are its
//                  16 keys of each tile, the order the h/z kernel wrote V8^T in.
// Both tiles of a pair (K8, V8^T and the key bias) arrive by direct global->LDS copies,
// double-buffered one pair ahead, one barrier per pair. A pair with one tile
// (odd critical count) takes zeros for the missing operands.
#include <type_traits>

#include "sla_internal.h"
#include "dev_common.h"

namespace sla {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

template <int D>
struct Q8Cfg {
  static constexpr int C8 = D / 16;          // 16-byte chunks per int8 K row
  static constexpr int KT = kBlock * D;      // bytes of one K8 tile (and of one V8^T tile)
  static constexpr int PAIR = 4 * KT + 512;  // K8 of two tiles, V8^T of two tiles, two key biases
  static constexpr int CPL = KT / 16 / 256;  // 16-byte copies per lane per tile operand
  static constexpr int KS8 = D / 64;         // int8 k steps of the score product
  static constexpr int KS = D / 32;          // bf16 k steps of the linear-branch product
  static constexpr int FT = D / 16;          // feature tiles of O
  static constexpr int NN = D * D + D;
  static constexpr int OS = D + 8;           // row stride of the staged output (bf16)
};

// Position of 16-byte chunk ch of int8 K row r in LDS is ch ^ ksw(r): the 16
// rows one MFMA lane group reads at one chunk then fall on distinct banks.
template <int D>
__device__ __forceinline__ int ksw(int r) {
  return D == 128 ? ((r >> 1) & 7) : (r & 3);
}

template <int D>
__global__ __launch_bounds__(256, 2) void k_sparse_q8(
    const uint16_t* __restrict__ Q, const float* __restrict__ qkmean,
    const int8_t* __restrict__ k8, const float* __restrict__ ksc, const float* __restrict__ kbias,
    const uint8_t* __restrict__ v8t, const float* __restrict__ vsc,
    const int8_t* __restrict__ mask, const uint16_t* __restrict__ Hx,
    const float* __restrict__ alpha, int elu, uint16_t* __restrict__ O, float* __restrict__ dbg_os,
    float* __restrict__ dbg_ol, int H, int N, int Nb) {
  using Cf = Q8Cfg<D>;
  constexpr int C8 = Cf::C8, KT = Cf::KT, PAIR = Cf::PAIR, CPL = Cf::CPL, KS8 = Cf::KS8;
  constexpr int KS = Cf::KS, FT = Cf::FT, NN = Cf::NN, OS = Cf::OS, C = D / 8;
  constexpr float TAU = 8.0f;  // a stale reference max may lag the pair max by 2^8 at most
  __shared__ __attribute__((aligned(16))) uint8_t bufA[PAIR];
  __shared__ __attribute__((aligned(16))) uint8_t bufB[PAIR];
  __shared__ uint16_t list[kMaxNb];
  __shared__ int wsum[4 * kMaskPre];
  __shared__ float qmax[4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = id / Nb, i = id - bh * Nb;
  const int h = bh % H;
  const int qrow = 16 * wave + l16;                // the lane's query within the block
  const int tq = min(i * kBlock + qrow, N - 1);    // rows past N are never stored

  // the mask row first; then the lane's query, features 32ks + 8g .. +7 (the
  // bf16 B operand layout), and the channel means of Q for the same features
  const int8_t* mrow = mask + ((size_t)bh * Nb + i) * Nb;
  int8_t mv[kMaskPre];
  mask_load(mrow, Nb, mv);
  uint4 qr[KS];
  float4 qmv[KS][2];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qr[ks] = *reinterpret_cast<const uint4*>(Q + ((size_t)bh * N + tq) * D + 32 * ks + 8 * g);
    qmv[ks][0] = *reinterpret_cast<const float4*>(qkmean + (size_t)bh * D + 32 * ks + 8 * g);
    qmv[ks][1] = *reinterpret_cast<const float4*>(qkmean + (size_t)bh * D + 32 * ks + 8 * g + 4);
  }

  const int ncrit = compact_loaded(mv, mrow, Nb, (int8_t)1, list, wsum);
  const int npair = (ncrit + 1) >> 1;

  const int8_t* Kb = k8 + (size_t)bh * Nb * KT;
  const uint8_t* Vb = v8t + (size_t)bh * Nb * KT;
  const float* Bb = kbias + (size_t)bh * Nb * kBlock;
  const float* ks_b = ksc + (size_t)bh * Nb;
  const float* vs_b = vsc + (size_t)bh * Nb;
  int koff[CPL];
#pragma unroll
  for (int u = 0; u < CPL; ++u) {
    const int G = 64 * (4 * u + wave) + lane;  // LDS chunk: row G / C8, position G % C8
    const int r = G / C8, pos = G % C8;
    koff[u] = r * D + 16 * (pos ^ ksw<D>(r));
  }
  // K8 rows past N are zero in memory (their scores are masked below). Copies go
  // through buffer resources over this head's K8, V8^T and key biases; the tile
  // offset (wave-uniform) is the scalar offset.
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(Kb, Nb * KT);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(Vb, Nb * KT);
  const __amdgpu_buffer_rsrc_t brs = make_rsrc(Bb, Nb * kBlock * 4);
  auto issue = [&](int p, uint8_t* dst) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int c = 2 * p + t;
      if (c >= ncrit) break;
      const int j = __builtin_amdgcn_readfirstlane((int)list[c]);
#pragma unroll
      for (int u = 0; u < CPL; ++u) {
        load_lds16_buf(krs, koff[u], j * KT, dst + t * KT + 1024 * (4 * u + wave));
        load_lds16_buf(vrs, 16 * (64 * (4 * u + wave) + lane), j * KT,
                       dst + (2 + t) * KT + 1024 * (4 * u + wave));
      }
      if (wave == 0 && lane < 16)  // the 64 key biases: 256 bytes
        load_lds16_buf(brs, 16 * lane, j * kBlock * 4, dst + 4 * KT + 256 * t);
    }
  };
  if (npair > 0) issue(0, bufA);

  // ---- Q8: this block's queries minus the channel means, one absmax/127 scale
  float qsm[KS][8];
  float qa = 0.f;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const uint32_t w4[4] = {qr[ks].x, qr[ks].y, qr[ks].z, qr[ks].w};
    const float mv[8] = {qmv[ks][0].x, qmv[ks][0].y, qmv[ks][0].z, qmv[ks][0].w,
                         qmv[ks][1].x, qmv[ks][1].y, qmv[ks][1].z, qmv[ks][1].w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      qsm[ks][e] = ((e & 1) ? bf_hi(w4[e >> 1]) : bf_lo(w4[e >> 1])) - mv[e];
      qa = fmaxf(qa, fabsf(qsm[ks][e]));
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) qa = fmaxf(qa, __shfl_xor(qa, o));
  if (lane == 0) qmax[wave] = qa;
  lds_barrier();  // (the copies of the first pair stay in flight)
  qa = fmaxf(fmaxf(qmax[0], qmax[1]), fmaxf(qmax[2], qmax[3]));
  const float qinv8 = qa > 0.f ? 127.0f / qa : 1.0f;
  const float qscale = qa > 0.f ? qa / 127.0f : 1.0f;
  // int8 B operand of k step ks8: features 32(2 ks8) + 8g .. +7, then 32(2 ks8 + 1) + 8g .. +7
  uint4 qr8[KS8];
#pragma unroll
  for (int ks8 = 0; ks8 < KS8; ++ks8) {
    uint32_t w[4];
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) {
      const float* x = &qsm[2 * ks8 + (hh >> 1)][4 * (hh & 1)];
      const int c0 = q_i8(x[0], qinv8), c1 = q_i8(x[1], qinv8);
      const int c2 = q_i8(x[2], qinv8), c3 = q_i8(x[3], qinv8);
      w[hh] = (uint32_t)(c0 & 0xff) | ((uint32_t)(c1 & 0xff) << 8) |
              ((uint32_t)(c2 & 0xff) << 16) | ((uint32_t)(c3 & 0xff) << 24);
    }
    qr8[ks8] = make_uint4(w[0], w[1], w[2], w[3]);
  }

  const float sc = kLog2e / sqrtf((float)D);
  const float sq = qscale * sc;
  f32x4 acc[FT];
#pragma unroll
  for (int ft = 0; ft < FT; ++ft) acc[ft] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mref = -INFINITY, lp = 0.f;

  // FAST: both tiles present and no key past N (every pair but possibly the
  // last and the one holding the ragged block), so no score needs masking
  auto step = [&](auto fast_c, int p, int j0, int j1, const uint8_t* cur, uint8_t* nxt)
                  __attribute__((always_inline)) {
    constexpr bool FAST = decltype(fast_c)::value;
    const bool has1 = FAST || 2 * p + 1 < ncrit;
    const float su0 = sq * ks_b[j0], su1 = sq * ks_b[j1];
    const float sv0 = vs_b[j0], sv1 = has1 ? vs_b[j1] : 1.f;
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // this wave's copies of pair p have landed
    lds_barrier();  // all copies of pair p are in LDS; every wave is done with pair p-1
    if (p + 1 < npair) issue(p + 1, nxt);
    // The integer products accumulate onto the bit image of the float 1.5 * 2^23:
    // with |n| <= 127^2 D < 2^22 the sum's bits read as the float 1.5 * 2^23 + n
    // exactly, so no conversion is needed; fma(that, su, bias) then carries the
    // tile constant C_t = 1.5 * 2^23 * su_t (rounded once, at the magnitude of
    // C_t, an error below 1e-4 of the int8 codes' own rounding error), which is
    // taken out of the tile maximum and added to the exponent offset.
    constexpr int kMagic = 0x4B400000;
    constexpr float kMagicF = 12582912.0f;
    i32x4 s[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) s[t][kt] = i32x4{kMagic, kMagic, kMagic, kMagic};
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (t == 1 && !has1) break;
#pragma unroll
      for (int ks = 0; ks < KS8; ++ks)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          const int row = 16 * kt + l16;
          const uint4 a = *reinterpret_cast<const uint4*>(cur + t * KT + row * D +
                                                          16 * ((4 * ks + g) ^ ksw<D>(row)));
          s[t][kt] = mfma_i8(a, qr8[ks], s[t][kt]);
        }
    }
    // dequantised scores plus key bias (stored already in the log2 domain); keys
    // past N and a missing tile take no part
    float sf[2][4][4];
    float tmax[2] = {-INFINITY, -INFINITY};
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int j = t ? j1 : j0;
      const bool live = t == 0 || has1;
      const bool rag = (j + 1) * kBlock > N;
      const float su = t ? su1 : su0;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const float4 b4 = live ? *reinterpret_cast<const float4*>(cur + 4 * KT + 256 * t + 4 * (16 * kt + 4 * g))
                               : make_float4(0.f, 0.f, 0.f, 0.f);
        const float bv[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v = fmaf(__int_as_float(s[t][kt][r]), su, bv[r]);
          if constexpr (FAST) {
            sf[t][kt][r] = v;
          } else {
            const bool out = !live || (rag && j * kBlock + 16 * kt + 4 * g + r >= N);
            sf[t][kt][r] = out ? -INFINITY : v;
          }
        }
      }
      // three-input max chain over the tile's 16 scores
      float m = fmaxf(fmaxf(sf[t][0][0], sf[t][0][1]), sf[t][0][2]);
#pragma unroll
      for (int x = 3; x + 1 < 16; x += 2)
        m = fmaxf(fmaxf(m, sf[t][x >> 2][x & 3]), sf[t][(x + 1) >> 2][(x + 1) & 3]);
      tmax[t] = fmaxf(m, sf[t][3][3]) - kMagicF * su;  // -inf stays -inf
    }
    // the rest of the pair; called on both sides of the (rare) reference raise,
    // so that the common path keeps the accumulators where the products left them
    auto finish = [&]() __attribute__((always_inline)) {
      const float meff = mref == -INFINITY ? 0.0f : mref;  // no valid key yet: every p is 0
      // P' = P~ s_V with P~ = 2^(s - meff). Its row scale over the pair is the
      // power of two s_P = 2^E, E = ceil(log2 rowmax(P') - log2 448), so that the
      // largest fp8 input lies in (224, 448]; the fp8 product applies it as the
      // E8M0 block scale of its B operand. With meff an integer, meff + E =
      // ceil(Mq - log2 448) and the codes 2^(s + log2 s_V - meff - E) are those
      // of the scores alone. The fp8 input of a key of tile t is 2^(s - off_t),
      // off_t = meff - log2 s_V(t) + E, and the tile's share of l (the
      // unquantised P~) is 2^(off_t - meff) times the sum of those inputs.
      const float lsv0 = __log2f(sv0), lsv1 = has1 ? __log2f(sv1) : 0.f;
      const float Mq = group4_max(fmaxf(tmax[0] + lsv0, tmax[1] + lsv1));
      constexpr float kLog2_448 = 8.807354922057604f;
      const float E = fminf(fmaxf(ceilf(Mq - meff - kLog2_448), -127.f), 127.f);
      const float off0 = (meff - lsv0 + E) + kMagicF * su0, off1 = (meff - lsv1 + E) + kMagicF * su1;
      float ssum[2] = {0.f, 0.f};
      i32x8 pb;
  #pragma unroll
      for (int t = 0; t < 2; ++t) {
        const float off = t ? off1 : off0;
  #pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          float e[4];
  #pragma unroll
          for (int r = 0; r < 4; ++r) {
            e[r] = __builtin_amdgcn_exp2f(sf[t][kt][r] - off);
            ssum[t] += e[r];
          }
          pb[4 * t + kt] = (int)pack_e4m3x4_nosat(e[0], e[1], e[2], e[3]);
        }
      }
      lp += ssum[0] * __builtin_amdgcn_exp2f(E - lsv0) + ssum[1] * __builtin_amdgcn_exp2f(E - lsv1);
      const int sb = (int)E + 127;
  #pragma unroll
      for (int ft = 0; ft < FT; ++ft) {
        const int c = 16 * ft + l16;
        const int off = c * 64 + 16 * (g ^ ((c >> 1) & 3));
        const uint4 v0 = *reinterpret_cast<const uint4*>(cur + 2 * KT + off);
        const uint4 v1 = has1 ? *reinterpret_cast<const uint4*>(cur + 3 * KT + off) : make_uint4(0, 0, 0, 0);
        const i32x8 a = {(int)v0.x, (int)v0.y, (int)v0.z, (int)v0.w,
                         (int)v1.x, (int)v1.y, (int)v1.z, (int)v1.w};
        acc[ft] = mfma_fp8_sb(a, pb, acc[ft], sb);
      }
    };
    const float lmax = fmaxf(tmax[0], tmax[1]);
    if (__ballot(lmax > mref + TAU)) {
      const float tm = group4_max(lmax);
      // an integer reference: the fp8 codes below then depend on the scores
      // alone, not on when the reference was raised
      const float nref = tm > mref + TAU ? ceilf(tm) : mref;
      const float fac = nref == mref ? 1.0f : __builtin_amdgcn_exp2f(mref - nref);
      mref = nref;
      lp *= fac;
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) acc[ft] *= fac;
      finish();
    } else {
      finish();
    }
  };
  auto run = [&](int p, const uint8_t* cur, uint8_t* nxt) __attribute__((always_inline)) {
    const int j0 = __builtin_amdgcn_readfirstlane((int)list[2 * p]);
    if (2 * p + 1 < ncrit) {
      const int j1 = __builtin_amdgcn_readfirstlane((int)list[2 * p + 1]);
      if ((max(j0, j1) + 1) * kBlock <= N) {
        step(std::true_type{}, p, j0, j1, cur, nxt);
        return;
      }
      step(std::false_type{}, p, j0, j1, cur, nxt);
    } else {
      step(std::false_type{}, p, j0, j0, cur, nxt);
    }
  };
  for (int p = 0; p < npair; p += 2) {
    run(p, bufA, bufB);
    if (p + 1 < npair) run(p + 1, bufB, bufA);
  }

  const float lw = group4_sum(lp);
  const float inv_l = lw > 0.f ? 1.0f / lw : 0.f;

  // ---- linear branch for the wave's 16 queries from bf16 Q: phi(Q), den = phi(Q).Z_i,
  // num^T = H_i^T phi(Q)^T
  const uint16_t* Hrow = Hx + ((size_t)bh * Nb + i) * NN;
  float zf[KS * 8];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const uint4 z = *reinterpret_cast<const uint4*>(Hrow + D * D + 32 * ks + 8 * g);
    const uint32_t zw[4] = {z.x, z.y, z.z, z.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      zf[ks * 8 + 2 * e] = bf_lo(zw[e]);
      zf[ks * 8 + 2 * e + 1] = bf_hi(zw[e]);
    }
  }
  uint4 fq[KS];
  float inv_den;
  {
    float qf[KS * 8];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint32_t w4[4] = {qr[ks].x, qr[ks].y, qr[ks].z, qr[ks].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qf[ks * 8 + 2 * e] = bf_lo(w4[e]);
        qf[ks * 8 + 2 * e + 1] = bf_hi(w4[e]);
      }
    }
    if (elu) {  // uniform: phi = elu + 1, elementwise
#pragma unroll
      for (int e = 0; e < KS * 8; ++e) qf[e] = elu1(qf[e]);
    } else {
      float qm = -INFINITY;
#pragma unroll
      for (int e = 0; e < KS * 8; ++e) qm = fmaxf(qm, qf[e]);
      qm = group4_max(qm) * kLog2e;
      // e = exp(q - max q); phi(Q) = e / sum(e), but the sum cancels between the
      // numerator phi(Q) H_i and the denominator phi(Q) Z_i, so e enters both unscaled
#pragma unroll
      for (int e = 0; e < KS * 8; ++e) qf[e] = __builtin_amdgcn_exp2f(fmaf(qf[e], kLog2e, -qm));
    }
    float dp = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint32_t w4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        w4[e] = pack_bf2(qf[ks * 8 + 2 * e], qf[ks * 8 + 2 * e + 1]);
        dp += bf_lo(w4[e]) * zf[ks * 8 + 2 * e] + bf_hi(w4[e]) * zf[ks * 8 + 2 * e + 1];
      }
      fq[ks] = make_uint4(w4[0], w4[1], w4[2], w4[3]);
    }
    const float den = group4_sum(dp);
    inv_den = den > 0.f ? 1.0f / den : 0.f;
  }
  const float al = alpha[h];
  __syncthreads();  // every wave is done with the pair buffers
  uint16_t* ost = reinterpret_cast<uint16_t*>(bufA);  // staged output tile [64][OS]
#pragma unroll
  for (int ft = 0; ft < FT; ++ft) {
    f32x4 nm = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint4 a = *reinterpret_cast<const uint4*>(Hrow + (size_t)(16 * ft + l16) * D + 32 * ks + 8 * g);
      nm = mfma_bf16(a, fq[ks], nm);
    }
    float os[4], ol[4], o[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      os[r] = acc[ft][r] * inv_l;
      ol[r] = nm[r] * inv_den;
      o[r] = al * os[r] + (1.0f - al) * ol[r];
    }
    *reinterpret_cast<uint2*>(ost + qrow * OS + 16 * ft + 4 * g) =
        make_uint2(pack_bf2(o[0], o[1]), pack_bf2(o[2], o[3]));
    const int t = i * kBlock + qrow;
    if (t < N && (dbg_os || dbg_ol)) {
      const size_t off = ((size_t)bh * N + t) * D + 16 * ft + 4 * g;
      if (dbg_os) *reinterpret_cast<float4*>(dbg_os + off) = make_float4(os[0], os[1], os[2], os[3]);
      if (dbg_ol) *reinterpret_cast<float4*>(dbg_ol + off) = make_float4(ol[0], ol[1], ol[2], ol[3]);
    }
  }
  __syncthreads();
  const int nrow = min(kBlock, N - i * kBlock);
  uint16_t* Ob = O + ((size_t)bh * N + (size_t)i * kBlock) * D;
  for (int x = tid; x < nrow * C; x += 256) {
    const int row = x / C, ch = x % C;
    *reinterpret_cast<uint4*>(Ob + (size_t)row * D + ch * 8) =
        *reinterpret_cast<const uint4*>(ost + row * OS + ch * 8);
  }
}

}  // namespace

hipError_t launch_sparse_q8(const Dims& D, const void* Q, const int8_t* mask, const float* alpha,
                            const Work& w, void* O, float* dbg_os, float* dbg_ol, hipStream_t s) {
  if (!D.quant || !D.bf16) return hipErrorInvalidValue;
  const int T = D.BH * D.Nb;
  if (D.d == 128)
    hipLaunchKernelGGL(k_sparse_q8<128>, dim3(T), dim3(256), 0, s, (const uint16_t*)Q, w.qkmean,
                       w.k8, w.ks, w.kb, w.v8t, w.vs, mask, (const uint16_t*)w.Hx, alpha,
                       D.elu ? 1 : 0, (uint16_t*)O, dbg_os, dbg_ol, D.H, D.N, D.Nb);
  else
    hipLaunchKernelGGL(k_sparse_q8<64>, dim3(T), dim3(256), 0, s, (const uint16_t*)Q, w.qkmean,
                       w.k8, w.ks, w.kb, w.v8t, w.vs, mask, (const uint16_t*)w.Hx, alpha,
                       D.elu ? 1 : 0, (uint16_t*)O, dbg_os, dbg_ol, D.H, D.N, D.Nb);
  return hipGetLastError();
}

}  // namespace sla
