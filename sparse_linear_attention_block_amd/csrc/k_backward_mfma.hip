// Backward pass of SLA2 on MFMA for bf16 inputs and a fixed block mask: dQ,
// dK, dV and dalpha of sum(O * dO), O = alpha O_s + (1 - alpha) O_l.
//
// The algebra is that of the float32 kernels in k_backward.hip (SLA explainer,
// intelliparadigm.com, section 2.3: the FlashAttention backward over the
// blocks with Mc = 1 for the sparse path, the chain rule through phi(Q),
// phi(K) and V for the linear path), arranged for the matrix cores:
//  * the forward sparse kernel (k_sparse.hip) runs first with the given mask
//    and writes O_s (float32) and the log2 normaliser lse2 of every query, so
//    that P = exp2(s log2(e) / sqrt(d) - lse2);
//  * k_bwdq_mfma, one workgroup per query block, 4 waves x 16 queries:
//    D_t = alpha dO . O_s; for every 32-key step of the block's critical
//    tiles (K and V rows copied to LDS as in the forward),
//      S^T = K Q^T, dP^T = V dO^T (16x16x32 bf16, queries as the B operand),
//      P = exp2(S^T log2(e) / sqrt(d) - lse2), dS^T = P (alpha dP^T - D_t),
//      dQ^T += K^T dS^T (K^T by transposed LDS reads, dS^T from registers);
//    then the linear branch with H_i^T in LDS: u = phi(q), num^T = H_i^T u^T,
//    den = u . Z_i, dnum = (1 - alpha) dO / den, dden = -(dO_l . O_l) / den,
//    du^T = H_i dnum^T + Z_i dden (H_i by transposed reads), dQ += J_phi^T du;
//    dH_i = u^T dnum and dZ_i = u^T dden over the block's 64 queries (u and
//    dnum rows in LDS, both operands by transposed reads), stored in bf16; the
//    block's dalpha partial;
//  * dh_j = sum over the query blocks i with Mc[i, j] = 0 of dH_i is the
//    forward's indicator product (k_linear.hip) on the transposed mask;
//  * k_bwdkv_mfma, one workgroup per key block, 4 waves x 16 keys: the linear
//    branch with dh_j^T in LDS (dV = phi(K) dh_j, dw^T = dh_j V^T + dz_j,
//    dK = J_phi^T dw), then for every 32-query step of the query blocks that
//    hold the key block as critical (the transposed mask row), S = Q K^T and
//    dP = dO V^T (Q and dO rows in LDS, keys as the B operand), P and dS from
//    lse2 and D_t, dV^T += dO^T (alpha P), dK^T += Q^T dS / sqrt(d).
// The SLA fusion O = O_s + O_l W (SLA paper summary, section 4, step 4) takes
// the same kernels with alpha = 1 for the sparse side, dO_l = dO W^T on MFMA
// (W packed once into A-operand fragments), O_l of every row stored in bf16 by
// k_bwdq_mfma, and dW = O_l^T dO formed by k_bwd_dw_mfma over chunks of rows
// (O_l and dO rows in LDS, both operands by transposed reads), the chunk parts
// summed in float64 by k_bwd_dw_part and k_bwd_dw_fin.
// Every product takes bf16 operands and accumulates in float32.
#include "sla_internal.h"
#include "dev_common.h"

namespace sla {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

template <int D>
struct BwCfg {
  static constexpr int NT = 256;              // 4 waves, 16 queries or keys each
  static constexpr int NW = 4;
  static constexpr int C = D / 8;             // 16-byte chunks per row
  static constexpr int HT = 32 * D;           // elements of 32 rows
  static constexpr int INSTR = HT / 8 / NT;   // 16-byte copies per lane per tensor and step
  static constexpr int KS = D / 32;           // 32-feature k steps
  static constexpr int FT = D / 16;           // 16-feature tiles
  static constexpr int HPARTS = D / 64;       // 64-row parts of a d x d tile (one step buffer each)
  static constexpr int HINSTR = 64 * D / 8 / NT;
  static constexpr int NN = D * D + D;
};

__device__ __forceinline__ float wsum64(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Row r, 16-byte chunk c of a row-major tile in LDS whose chunks are
// XOR-swizzled by the row (row_swz, the layout of the forward's K rows), as an element offset.
template <int D>
__device__ __forceinline__ int swz(int r, int c) {
  constexpr int C = D / 8;
  return (r * C + (c ^ row_swz<D>(r))) * 8;
}

// Per-lane element offsets of the copies of 32 rows (row r, chunk sch of the
// global rows lands at LDS chunk r C + sch ^ row_swz(r)), the same for every step.
template <int D>
__device__ __forceinline__ void row_offsets(int wave, int lane, int (&koff)[BwCfg<D>::INSTR]) {
  constexpr int C = D / 8;
#pragma unroll
  for (int u = 0; u < BwCfg<D>::INSTR; ++u) {
    const int G = 64 * (BwCfg<D>::NW * u + wave) + lane;
    const int r = G / C, sch = G % C;
    koff[u] = r * D + (sch ^ row_swz<D>(r)) * 8;
  }
}

// Rows row0 .. row0 + 31 of two [N, D] tensors (buffer resources ar, br) into
// dst and dst + HT; rows past N re-read row N - 1.
template <int D>
__device__ __forceinline__ void copy_rows(__amdgpu_buffer_rsrc_t ar, __amdgpu_buffer_rsrc_t br,
                                          const int (&koff)[BwCfg<D>::INSTR], int row0, int N, uint16_t* dst,
                                          int wave) {
  using Cf = BwCfg<D>;
  const int sk = row0 * D * 2;
  if (row0 + 32 > N) {
    const int over = row0 - (N - 1);
#pragma unroll
    for (int u = 0; u < Cf::INSTR; ++u) {
      const int off = koff[u] - max(0, koff[u] / D + over) * D;
      load_lds16_buf(ar, 2 * off, sk, dst + 512 * (Cf::NW * u + wave));
      load_lds16_buf(br, 2 * off, sk, dst + Cf::HT + 512 * (Cf::NW * u + wave));
    }
  } else {
#pragma unroll
    for (int u = 0; u < Cf::INSTR; ++u) {
      load_lds16_buf(ar, 2 * koff[u], sk, dst + 512 * (Cf::NW * u + wave));
      load_lds16_buf(br, 2 * koff[u], sk, dst + Cf::HT + 512 * (Cf::NW * u + wave));
    }
  }
}

// Part `part` (64 rows) of a d x d tile stored row-major (c-major H^T) at src
// into dst, swizzled like the K rows; part 0 also brings the d values that
// follow the tile (Z) into zbuf.
template <int D>
__device__ __forceinline__ void copy_tile_part(const uint16_t* src, int part, uint16_t* dst, uint16_t* zbuf,
                                               int wave, int lane) {
  using Cf = BwCfg<D>;
  constexpr int C = Cf::C;
#pragma unroll
  for (int u = 0; u < Cf::HINSTR; ++u) {
    const int G = 64 * (Cf::NW * u + wave) + lane;
    const int r = G / C, sch = G % C;
    load_lds16(src + (part * 64 + r) * D + (sch ^ row_swz<D>(r)) * 8, dst + 512 * (Cf::NW * u + wave));
  }
  if (part == 0 && wave == 0 && lane < C) load_lds16(src + D * D + 8 * lane, zbuf);
}

__device__ __forceinline__ void unpack4(uint2 w, float (&f)[4]) {
  f[0] = bf_lo(w.x);
  f[1] = bf_hi(w.x);
  f[2] = bf_lo(w.y);
  f[3] = bf_hi(w.y);
}

// phi of one token in two layouts: acc[ft][e] = phi(x)[16 ft + 4 g + e] (the
// float32 accumulator layout) and bop[ks] = bf16 phi(x)[32 ks + 8 g .. +7] (the
// B operand of a product over the features); x is given in both layouts.
// Softmax over the features (normalised) or elu + 1.
template <int D, bool ELU>
__device__ __forceinline__ void phi_two_layouts(const float (&xa)[BwCfg<D>::FT][4], const uint4 (&xb)[BwCfg<D>::KS],
                                                float (&acc)[BwCfg<D>::FT][4], uint4 (&bop)[BwCfg<D>::KS]) {
  using Cf = BwCfg<D>;
  if constexpr (ELU) {
#pragma unroll
    for (int ft = 0; ft < Cf::FT; ++ft)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[ft][e] = elu1(xa[ft][e]);
#pragma unroll
    for (int ks = 0; ks < Cf::KS; ++ks) {
      const uint32_t w4[4] = {xb[ks].x, xb[ks].y, xb[ks].z, xb[ks].w};
      uint32_t o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = pack_bf2(elu1(bf_lo(w4[e])), elu1(bf_hi(w4[e])));
      bop[ks] = make_uint4(o[0], o[1], o[2], o[3]);
    }
  } else {
    float m = -INFINITY;
#pragma unroll
    for (int ft = 0; ft < Cf::FT; ++ft)
#pragma unroll
      for (int e = 0; e < 4; ++e) m = fmaxf(m, xa[ft][e]);
    m = group4_max(m) * kLog2e;
    float s = 0.f;
#pragma unroll
    for (int ft = 0; ft < Cf::FT; ++ft)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[ft][e] = __builtin_amdgcn_exp2f(fmaf(xa[ft][e], kLog2e, -m));
        s += acc[ft][e];
      }
    const float inv = 1.0f / group4_sum(s);
#pragma unroll
    for (int ft = 0; ft < Cf::FT; ++ft)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[ft][e] *= inv;
#pragma unroll
    for (int ks = 0; ks < Cf::KS; ++ks) {
      const uint32_t w4[4] = {xb[ks].x, xb[ks].y, xb[ks].z, xb[ks].w};
      uint32_t o[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        o[e] = pack_bf2(__builtin_amdgcn_exp2f(fmaf(bf_lo(w4[e]), kLog2e, -m)) * inv,
                        __builtin_amdgcn_exp2f(fmaf(bf_hi(w4[e]), kLog2e, -m)) * inv);
      bop[ks] = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
}

// J_phi^T g for one token in the accumulator layout (phi = u, input x)
template <int D, bool ELU>
__device__ __forceinline__ void phi_vjp(const float (&x)[BwCfg<D>::FT][4], const float (&u)[BwCfg<D>::FT][4],
                                        const float (&gin)[BwCfg<D>::FT][4], float (&out)[BwCfg<D>::FT][4]) {
  using Cf = BwCfg<D>;
  if constexpr (ELU) {
#pragma unroll
    for (int ft = 0; ft < Cf::FT; ++ft)
#pragma unroll
      for (int e = 0; e < 4; ++e) out[ft][e] = gin[ft][e] * (x[ft][e] > 0.f ? 1.0f : u[ft][e]);
  } else {
    float d = 0.f;
#pragma unroll
    for (int ft = 0; ft < Cf::FT; ++ft)
#pragma unroll
      for (int e = 0; e < 4; ++e) d = fmaf(u[ft][e], gin[ft][e], d);
    d = group4_sum(d);
#pragma unroll
    for (int ft = 0; ft < Cf::FT; ++ft)
#pragma unroll
      for (int e = 0; e < 4; ++e) out[ft][e] = u[ft][e] * (gin[ft][e] - d);
  }
}

template <int D, bool ELU, bool PROJ>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_bwdq_mfma(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const int8_t* __restrict__ mask, const uint16_t* __restrict__ Hx,
    const uint16_t* __restrict__ Os, const float* __restrict__ lse2, const float* __restrict__ alpha,
    const uint16_t* __restrict__ wq, int wq_hs, float* __restrict__ dQ, float* __restrict__ Dt,
    uint16_t* __restrict__ dH, float* __restrict__ dal, uint16_t* __restrict__ Ol, int H, int N, int Nb) {
  using Cf = BwCfg<D>;
  constexpr int NT = Cf::NT, HT = Cf::HT, INSTR = Cf::INSTR, KS = Cf::KS, FT = Cf::FT;
  constexpr int HPARTS = Cf::HPARTS, NN = Cf::NN;
  __shared__ __attribute__((aligned(16))) uint16_t bufA[2 * HT];
  __shared__ __attribute__((aligned(16))) uint16_t bufB[2 * HT];
  __shared__ __attribute__((aligned(16))) uint16_t zbuf[D];
  __shared__ float ddn[kBlock];
  __shared__ float red[4];
  __shared__ int wsum[4 * kMaskPre];
  extern __shared__ __attribute__((aligned(16))) uint16_t list[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = id / Nb, i = id - bh * Nb, h = bh % H;
  const int8_t* mrow = mask + ((size_t)bh * Nb + i) * Nb;
  int8_t mv[kMaskPre];
  mask_load<NT>(mrow, Nb, mv);
  const int tq = i * kBlock + 16 * wave + l16;  // the lane's query (an MFMA column)
  const bool qv = tq < N;
  const size_t qrow = ((size_t)bh * N + min(tq, N - 1)) * D;
  uint4 qr[KS], gr[KS];  // B operands: features 32 ks + 8 g .. +7
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qr[ks] = *reinterpret_cast<const uint4*>(Q + qrow + 32 * ks + 8 * g);
    gr[ks] = *reinterpret_cast<const uint4*>(dO + qrow + 32 * ks + 8 * g);
  }
  uint2 qa2[FT], ga2[FT], os2[FT], ol2[FT];  // accumulator layout: features 16 ft + 4 g .. +3
  const size_t oplane = (size_t)(gridDim.x / Nb) * N * D;  // O_s lo after the hi plane
#pragma unroll
  for (int ft = 0; ft < FT; ++ft) {
    qa2[ft] = *reinterpret_cast<const uint2*>(Q + qrow + 16 * ft + 4 * g);
    ga2[ft] = *reinterpret_cast<const uint2*>(dO + qrow + 16 * ft + 4 * g);
    os2[ft] = *reinterpret_cast<const uint2*>(Os + qrow + 16 * ft + 4 * g);
    ol2[ft] = *reinterpret_cast<const uint2*>(Os + oplane + qrow + 16 * ft + 4 * g);
  }
  const float l2 = lse2[((size_t)bh * Nb + i) * kBlock + 16 * wave + l16];
  const float al = PROJ ? 1.0f : alpha[h];  // the SLA fusion weighs O_s by 1
  const int ncrit = compact_loaded<NT>(mv, mrow, Nb, (int8_t)1, list, wsum);
  float qf[FT][4], gf[FT][4];
#pragma unroll
  for (int ft = 0; ft < FT; ++ft) {
    unpack4(qa2[ft], qf[ft]);
    unpack4(ga2[ft], gf[ft]);
  }
  float dos = 0.f;  // dO . O_s
#pragma unroll
  for (int ft = 0; ft < FT; ++ft) {
    float of[4], lf[4];
    unpack4(os2[ft], of);
    unpack4(ol2[ft], lf);
#pragma unroll
    for (int r = 0; r < 4; ++r) of[r] += lf[r];
    dos = fmaf(gf[ft][0], of[0], fmaf(gf[ft][1], of[1], fmaf(gf[ft][2], of[2], fmaf(gf[ft][3], of[3], dos))));
  }
  dos = qv ? group4_sum(dos) : 0.f;
  const float Dq = al * dos;

  // ---- sparse branch
  const uint16_t* Kb = K + (size_t)bh * N * D;
  const uint16_t* Vb = V + (size_t)bh * N * D;
  int koff[INSTR];
  row_offsets<D>(wave, lane, koff);
  const int vxb = vt_base<D>(g, l16);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(Kb, N * D * 2);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(Vb, N * D * 2);
  const float sc = kLog2e / sqrtf((float)D);
  f32x4 dq[FT];
#pragma unroll
  for (int ft = 0; ft < FT; ++ft) dq[ft] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nstep = 2 * ncrit;  // step s: keys 32 (s & 1) .. +31 of critical tile s >> 1
  auto step = [&](int s, const uint16_t* cur, uint16_t* nxt) {
    const int j = __builtin_amdgcn_readfirstlane((int)list[s >> 1]);
    const int hh = s & 1;
    const int jn = __builtin_amdgcn_readfirstlane((int)list[min((s + 1) >> 1, ncrit - 1)]);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    lds_barrier();
    uint4 ka[KS][2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
        ka[ks][kt] = *reinterpret_cast<const uint4*>(cur + swz<D>(16 * kt + l16, 4 * ks + g));
    __builtin_amdgcn_sched_barrier(0);
    if (s + 1 < nstep) copy_rows<D>(krs, vrs, koff, jn * kBlock + 32 * ((s + 1) & 1), N, nxt, wave);
    __builtin_amdgcn_sched_barrier(0);
    f32x4 sv[2], dp[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) sv[kt] = dp[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) sv[kt] = mfma_bf16(ka[ks][kt], qr[ks], sv[kt]);
    __builtin_amdgcn_sched_barrier(0);  // one operand set in registers at a time
    uint4 vb[KS][2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
        vb[ks][kt] = *reinterpret_cast<const uint4*>(cur + HT + swz<D>(16 * kt + l16, 4 * ks + g));
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) dp[kt] = mfma_bf16(vb[ks][kt], gr[ks], dp[kt]);
    __builtin_amdgcn_sched_barrier(0);
    uint4 kt_[FT];
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) kt_[ft] = vt_frag<D>(cur, vxb, ft);
    if (j * kBlock + 32 * hh + 32 > N) {  // ragged last block: keys past N take no part
      const int kbase = j * kBlock + 32 * hh + 4 * g;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) sv[kt][r] = kbase + 16 * kt + r >= N ? -INFINITY : sv[kt][r];
    }
    float ds[2][4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sv[kt][r], sc, -l2));
        ds[kt][r] = p * fmaf(al, dp[kt][r], -Dq);
      }
    const uint4 dsb = make_uint4(pack_bf2(ds[0][0], ds[0][1]), pack_bf2(ds[0][2], ds[0][3]),
                                 pack_bf2(ds[1][0], ds[1][1]), pack_bf2(ds[1][2], ds[1][3]));
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) dq[ft] = mfma_bf16(kt_[ft], dsb, dq[ft]);
  };
  if (nstep > 0) copy_rows<D>(krs, vrs, koff, (int)list[0] * kBlock, N, bufA, wave);
  for (int s = 0; s < nstep; s += 2) {  // nstep is even
    step(s, bufA, bufB);
    step(s + 1, bufB, bufA);
  }

  // ---- linear branch: H_i^T (rows n) in parts of 64 rows into bufA / bufB, Z_i into zbuf
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  lds_barrier();  // every wave is done with the step buffers
  const uint16_t* Hrow = Hx + ((size_t)bh * Nb + i) * NN;
  copy_tile_part<D>(Hrow, 0, bufA, zbuf, wave, lane);
  if constexpr (HPARTS == 2) copy_tile_part<D>(Hrow, 1, bufB, zbuf, wave, lane);
  float u[FT][4];
  uint4 fq[KS];
  phi_two_layouts<D, ELU>(qf, qr, u, fq);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  lds_barrier();
  auto hpart = [&](int ks) -> const uint16_t* { return (ks < KS / HPARTS ? bufA : bufB) + 32 * (ks % (KS / HPARTS)) * D; };
  // num^T = H_i^T u^T (A: rows n of H_i^T); den = u . Z_i (Z_i as row 0 of an A operand)
  f32x4 nm[FT];
#pragma unroll
  for (int ft = 0; ft < FT; ++ft) {
    nm[ft] = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint16_t* hb = ft < FT / HPARTS ? bufA : bufB;
    const int hr = 16 * (ft % (FT / HPARTS)) + l16;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      nm[ft] = mfma_bf16(*reinterpret_cast<const uint4*>(hb + swz<D>(hr, 4 * ks + g)), fq[ks], nm[ft]);
  }
  float den;
  {
    f32x4 dacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint4 z = *reinterpret_cast<const uint4*>(zbuf + 32 * ks + 8 * g);
      dacc = mfma_bf16(l16 == 0 ? z : make_uint4(0u, 0u, 0u, 0u), fq[ks], dacc);
    }
    den = __shfl(dacc[0], l16);  // row 0 of the product, from lane group 0
  }
  const float inv_den = den > 0.f ? 1.0f / den : 0.f;
  // dO_l: (1 - alpha) dO, or dO W^T for the SLA fusion (A: W's rows c from the
  // packed fragments, B: dO with the features 32 ks + 8 g .. +7)
  float glf[FT][4];
  if constexpr (PROJ) {
    const uint4* wf = reinterpret_cast<const uint4*>(wq + (size_t)h * wq_hs) + lane;
#pragma unroll
    for (int ct = 0; ct < FT; ++ct) {
      f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) a = mfma_bf16(wf[(ct * KS + ks) * 64], gr[ks], a);
#pragma unroll
      for (int e = 0; e < 4; ++e) glf[ct][e] = a[e];
    }
  } else {
#pragma unroll
    for (int ft = 0; ft < FT; ++ft)
#pragma unroll
      for (int e = 0; e < 4; ++e) glf[ft][e] = (1.0f - al) * gf[ft][e];
  }
  float dnm[FT][4], olf[FT][4];
  float dop = 0.f, dol = 0.f;
#pragma unroll
  for (int ft = 0; ft < FT; ++ft)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float ol = nm[ft][e] * inv_den;
      const float gl = glf[ft][e];
      olf[ft][e] = qv ? ol : 0.f;
      dnm[ft][e] = qv ? gl * inv_den : 0.f;
      dop = fmaf(gl, ol, dop);
      dol = fmaf(gf[ft][e], ol, dol);
    }
  const float dden = qv ? -group4_sum(dop) * inv_den : 0.f;
  const float dool = group4_sum(dol);
  // du^T = H_i dnum^T + Z_i dden: A = H_i by transposed reads of the rows n,
  // B = dnum^T with the k slots {4g..4g+3, 16+4g..16+4g+3} of each 32-feature step
  uint4 nb[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    nb[ks] = make_uint4(pack_bf2(dnm[2 * ks][0], dnm[2 * ks][1]), pack_bf2(dnm[2 * ks][2], dnm[2 * ks][3]),
                        pack_bf2(dnm[2 * ks + 1][0], dnm[2 * ks + 1][1]),
                        pack_bf2(dnm[2 * ks + 1][2], dnm[2 * ks + 1][3]));
  float du[FT][4];
#pragma unroll
  for (int rt = 0; rt < FT; ++rt) {
    f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) a = mfma_bf16(vt_frag<D>(hpart(ks), vxb, rt), nb[ks], a);
#pragma unroll
    for (int e = 0; e < 4; ++e) du[rt][e] = fmaf(bf2f(zbuf[16 * rt + 4 * g + e]), dden, a[e]);
  }
  float dql[FT][4];
  phi_vjp<D, ELU>(qf, u, du, dql);
  const float isd = 1.0f / sqrtf((float)D);
  if (qv) {
#pragma unroll
    for (int ft = 0; ft < FT; ++ft)
      *reinterpret_cast<float4*>(dQ + qrow + 16 * ft + 4 * g) =
          make_float4(fmaf(dq[ft][0], isd, dql[ft][0]), fmaf(dq[ft][1], isd, dql[ft][1]),
                      fmaf(dq[ft][2], isd, dql[ft][2]), fmaf(dq[ft][3], isd, dql[ft][3]));
  }
  if (g == 0) Dt[((size_t)bh * Nb + i) * kBlock + 16 * wave + l16] = Dq;

  // ---- dH_i = u^T dnum and dZ_i = u^T dden over the block's queries (zero past N)
  lds_barrier();  // every wave has read H_i^T: the buffers take the u and dnum rows
  {
    const int row = 16 * wave + l16;
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) {
      const int o = swz<D>(row, 2 * ft + (g >> 1)) + 4 * (g & 1);
      *reinterpret_cast<uint2*>(bufA + o) =
          qv ? make_uint2(pack_bf2(u[ft][0], u[ft][1]), pack_bf2(u[ft][2], u[ft][3])) : make_uint2(0u, 0u);
      *reinterpret_cast<uint2*>(bufB + o) =
          make_uint2(pack_bf2(dnm[ft][0], dnm[ft][1]), pack_bf2(dnm[ft][2], dnm[ft][3]));
    }
    if (g == 0) ddn[row] = dden;
  }
  if constexpr (!PROJ) {
    float da = (qv && g == 0) ? dos - dool : 0.f;  // this query's dO . (O_s - O_l)
    da = wsum64(da);
    if (lane == 0) red[wave] = da;
  }
  lds_barrier();
  if (!PROJ && tid == 0) dal[(size_t)bh * Nb + i] = (red[0] + red[1]) + (red[2] + red[3]);
  // D[r][n] = sum_q u[q][r] dnum[q][n]: A = u^T, B = dnum, both by transposed
  // reads of the staged rows; lane (l16 = n, g) holds r = 16 rt + 4 g .. +3,
  // four consecutive entries of dH_i^T's row n
  uint4 ua[FT][2];
#pragma unroll
  for (int rt = 0; rt < FT; ++rt)
#pragma unroll
    for (int kq = 0; kq < 2; ++kq) ua[rt][kq] = vt_frag<D>(bufA + 32 * kq * D, vxb, rt);
  uint16_t* dHrow = dH + ((size_t)bh * Nb + i) * NN;
  constexpr int NTW = FT / 4;  // n tiles per wave
#pragma unroll
  for (int x = 0; x < NTW; ++x) {
    const int nt = NTW * wave + x;
    uint4 nbq[2];
#pragma unroll
    for (int kq = 0; kq < 2; ++kq) nbq[kq] = vt_frag<D>(bufB + 32 * kq * D, vxb, nt);
#pragma unroll
    for (int rt = 0; rt < FT; ++rt) {
      f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kq = 0; kq < 2; ++kq) a = mfma_bf16(ua[rt][kq], nbq[kq], a);
      *reinterpret_cast<uint2*>(dHrow + (16 * nt + l16) * D + 16 * rt + 4 * g) =
          make_uint2(pack_bf2(a[0], a[1]), pack_bf2(a[2], a[3]));
    }
  }
  if (wave == 0) {  // dZ_i: B has dden in column 0
    uint4 bz[2];
#pragma unroll
    for (int kq = 0; kq < 2; ++kq) {
      const int q0 = 32 * kq + 4 * g;
      bz[kq] = l16 == 0 ? make_uint4(pack_bf2(ddn[q0], ddn[q0 + 1]), pack_bf2(ddn[q0 + 2], ddn[q0 + 3]),
                                     pack_bf2(ddn[q0 + 16], ddn[q0 + 17]), pack_bf2(ddn[q0 + 18], ddn[q0 + 19]))
                        : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int rt = 0; rt < FT; ++rt) {
      f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kq = 0; kq < 2; ++kq) a = mfma_bf16(ua[rt][kq], bz[kq], a);
      if (l16 == 0)
        *reinterpret_cast<uint2*>(dHrow + D * D + 16 * rt + 4 * g) = make_uint2(pack_bf2(a[0], a[1]), pack_bf2(a[2], a[3]));
    }
  }
  if constexpr (PROJ) {
    // O_l of the block's rows in bf16 for dW = O_l^T dO (k_bwd_dw_mfma), staged in
    // bufA and stored as whole rows; each wave reads back only its own 16 rows
    lds_barrier();  // every wave has read the u and dnum rows
    const int row = 16 * wave + l16;
#pragma unroll
    for (int ft = 0; ft < FT; ++ft)
      *reinterpret_cast<uint2*>(bufA + swz<D>(row, 2 * ft + (g >> 1)) + 4 * (g & 1)) =
          make_uint2(pack_bf2(olf[ft][0], olf[ft][1]), pack_bf2(olf[ft][2], olf[ft][3]));
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    constexpr int C = D / 8;
    uint16_t* orow = Ol + ((size_t)bh * N + (size_t)i * kBlock + 16 * wave) * D;
    const int nr = min(16, N - (i * kBlock + 16 * wave));
#pragma unroll
    for (int x0 = 0; x0 < 16 * C; x0 += 64) {
      const int r = (x0 + lane) / C, ch = (x0 + lane) % C;
      if (r < nr)
        *reinterpret_cast<uint4*>(orow + (size_t)r * D + ch * 8) =
            *reinterpret_cast<const uint4*>(bufA + swz<D>(16 * wave + r, ch));
    }
  }
}

// dW = O_l^T dO over one chunk of rows (SLA fusion, bf16 inputs): the rows of
// the (batch, head) pairs whose output map is W hw (head hw's own, or every
// pair when W is shared), in the order (pair, token), are cut into steps of 32
// and the steps into `chunks` consecutive chunks; workgroup (chunk r, W hw)
// writes its chunk's part of dW in float32 (bf16 products, float32
// accumulation over at most a few thousand rows); the parts are summed in
// float64 in a fixed order by k_bwd_dw_part / k_bwd_dw_fin. Each step's O_l and
// dO rows go through LDS (row-major, chunks swizzled by the row), the next
// step's rows loaded into registers meanwhile; D[n][c] = sum_t dO[t][n] O_l[t][c]
// with A = dO^T and B = O_l by transposed reads, so lane (l16 = c, g) holds
// n = 16 nt + 4 g .. +3 of row c of dW. Wave w owns the c tiles FT/4 w .. +FT/4-1.
template <int D>
__global__ __launch_bounds__(256) void k_bwd_dw_mfma(const uint16_t* __restrict__ Ol, const uint16_t* __restrict__ dO,
                                                     float* __restrict__ part, int B, int H, int N, int per_head,
                                                     int chunks) {
  constexpr int C = D / 8, FT = D / 16, CTW = FT / 4, CPT = 32 * C / 256;
  __shared__ __attribute__((aligned(16))) uint16_t tl[2][32 * D];  // O_l rows of a step
  __shared__ __attribute__((aligned(16))) uint16_t tg[2][32 * D];  // dO rows of a step
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int r = blockIdx.x, hw = blockIdx.y;
  const int nseg = per_head ? B : B * H;  // (batch, head) pairs of W hw, N rows each
  const long long R = (long long)nseg * N;
  const int steps = (int)((R + 31) / 32);
  const int per = (steps + chunks - 1) / chunks;
  const int s0 = min(steps, r * per), s1 = min(steps, s0 + per);
  // the current step's first row as (pair, token), advanced by 32 rows per step
  int sg = (int)(32LL * s0 / N), tb = (int)(32LL * s0 % N);
  uint4 rl[CPT], rg[CPT];
  auto load = [&]() {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int G = 256 * u + tid, rw = G / C, ch = G % C;
      int t = tb + rw, seg = sg;
      while (t >= N) {  // at most once when N >= 32
        t -= N;
        ++seg;
      }
      if (seg < nseg) {
        const size_t bh = per_head ? (size_t)seg * H + hw : (size_t)seg;
        const size_t off = (bh * N + t) * D + ch * 8;
        rl[u] = *reinterpret_cast<const uint4*>(Ol + off);
        rg[u] = *reinterpret_cast<const uint4*>(dO + off);
      } else {
        rl[u] = make_uint4(0u, 0u, 0u, 0u);
        rg[u] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
  };
  auto advance = [&]() {
    tb += 32;
    while (tb >= N) {
      tb -= N;
      ++sg;
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int G = 256 * u + tid, rw = G / C, ch = G % C;
      *reinterpret_cast<uint4*>(&tl[buf][swz<D>(rw, ch)]) = rl[u];
      *reinterpret_cast<uint4*>(&tg[buf][swz<D>(rw, ch)]) = rg[u];
    }
  };
  f32x4 acc[CTW][FT];
#pragma unroll
  for (int c = 0; c < CTW; ++c)
#pragma unroll
    for (int nt = 0; nt < FT; ++nt) acc[c][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int vxb = vt_base<D>(g, l16);
  if (s0 < s1) {
    load();
    stash(0);
  }
  __syncthreads();
  for (int s = s0; s < s1; ++s) {
    const int buf = (s - s0) & 1;
    if (s + 1 < s1) {
      advance();
      load();
    }
    uint4 ob[CTW];
#pragma unroll
    for (int c = 0; c < CTW; ++c) ob[c] = vt_frag<D>(tl[buf], vxb, CTW * wave + c);
#pragma unroll
    for (int nt = 0; nt < FT; ++nt) {
      const uint4 a = vt_frag<D>(tg[buf], vxb, nt);
#pragma unroll
      for (int c = 0; c < CTW; ++c) acc[c][nt] = mfma_bf16(a, ob[c], acc[c][nt]);
    }
    if (s + 1 < s1) stash(buf ^ 1);  // the other buffer was last read before the previous barrier
    __syncthreads();
  }
  float* out = part + ((size_t)hw * chunks + r) * D * D;
#pragma unroll
  for (int c = 0; c < CTW; ++c)
#pragma unroll
    for (int nt = 0; nt < FT; ++nt)
      *reinterpret_cast<float4*>(out + (size_t)(16 * (CTW * wave + c) + l16) * D + 16 * nt + 4 * g) =
          make_float4(acc[c][nt][0], acc[c][nt][1], acc[c][nt][2], acc[c][nt][3]);
}

template <int D, bool ELU>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_bwdkv_mfma(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const int8_t* __restrict__ maskT, const float* __restrict__ lse2,
    const float* __restrict__ Dt, const uint16_t* __restrict__ dh, const float* __restrict__ alpha,
    const int* __restrict__ order, const int* __restrict__ hdr, const int2* __restrict__ info,
    const int2* __restrict__ tab, float* __restrict__ part, int slots, float* __restrict__ dK,
    float* __restrict__ dV, int H, int N, int Nb) {
  using Cf = BwCfg<D>;
  constexpr int NT = Cf::NT, HT = Cf::HT, INSTR = Cf::INSTR, KS = Cf::KS, FT = Cf::FT;
  constexpr int HPARTS = Cf::HPARTS, NN = Cf::NN;
  __shared__ __attribute__((aligned(16))) uint16_t bufA[2 * HT];
  __shared__ __attribute__((aligned(16))) uint16_t bufB[2 * HT];
  __shared__ __attribute__((aligned(16))) float lsA[64];  // lse2 then D_t of the step's 32 queries
  __shared__ __attribute__((aligned(16))) float lsB[64];
  __shared__ __attribute__((aligned(16))) uint16_t zbuf[D];
  __shared__ int wsum[4 * kMaskPre];
  extern __shared__ __attribute__((aligned(16))) uint16_t list[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, g = lane >> 4;
  // workgroups 0 .. slots-1: the extra chunks (chunk >= 1) of the key blocks cut
  // into several; then chunk 0 of every key block, in order of falling critical
  // count (the longest first)
  int id, chunk;
  if ((int)blockIdx.x < slots) {
    if ((int)blockIdx.x >= hdr[1]) return;  // whole workgroup: no extra chunk here
    const int2 t = tab[blockIdx.x];
    id = t.x;
    chunk = t.y;
  } else {
    id = order[blockIdx.x - slots];
    chunk = 0;
  }
  const int2 inf = info[id];  // chunks of this key block, its first partial slot
  const int bh = id / Nb, j = id - bh * Nb, h = bh % H;
  const int8_t* mrow = maskT + ((size_t)bh * Nb + j) * Nb;
  int8_t mv[kMaskPre];
  mask_load<NT>(mrow, Nb, mv);
  const int tk = j * kBlock + 16 * wave + l16;  // the lane's key (an MFMA column)
  const bool kv = tk < N;
  const size_t krow = ((size_t)bh * N + min(tk, N - 1)) * D;
  uint4 kr[KS], vr[KS], vn[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    kr[ks] = *reinterpret_cast<const uint4*>(K + krow + 32 * ks + 8 * g);
    vr[ks] = *reinterpret_cast<const uint4*>(V + krow + 32 * ks + 8 * g);
    // v in the k-slot order {4g..4g+3, 16+4g..16+4g+3} of each 32-feature step
    const uint2 a = *reinterpret_cast<const uint2*>(V + krow + 32 * ks + 4 * g);
    const uint2 b = *reinterpret_cast<const uint2*>(V + krow + 32 * ks + 16 + 4 * g);
    vn[ks] = make_uint4(a.x, a.y, b.x, b.y);
  }
  uint2 ka2[FT];
#pragma unroll
  for (int ft = 0; ft < FT; ++ft) ka2[ft] = *reinterpret_cast<const uint2*>(K + krow + 16 * ft + 4 * g);
  const float al = alpha ? alpha[h] : 1.0f;  // the SLA fusion (no alpha) weighs O_s by 1
  const int ncol = compact_loaded<NT>(mv, mrow, Nb, (int8_t)1, list, wsum);
  const int vxb = vt_base<D>(g, l16);

  f32x4 dv[FT], dk[FT];
  if (chunk == 0) {  // uniform
  // ---- linear branch: dh_j^T (rows n) in parts of 64 rows into bufA / bufB, dz_j into zbuf
  const uint16_t* Hrow = dh + ((size_t)bh * Nb + j) * NN;
  copy_tile_part<D>(Hrow, 0, bufA, zbuf, wave, lane);
  if constexpr (HPARTS == 2) copy_tile_part<D>(Hrow, 1, bufB, zbuf, wave, lane);
  float kf[FT][4];
#pragma unroll
  for (int ft = 0; ft < FT; ++ft) unpack4(ka2[ft], kf[ft]);
  float w[FT][4];
  uint4 wf[KS];
  phi_two_layouts<D, ELU>(kf, kr, w, wf);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  lds_barrier();
  auto hpart = [&](int ks) -> const uint16_t* { return (ks < KS / HPARTS ? bufA : bufB) + 32 * (ks % (KS / HPARTS)) * D; };
  // dV^T = dh_j^T phi(K)^T (A: rows n of dh_j^T); dw^T = dh_j V^T (A by transposed reads) + dz_j
  float dw[FT][4];
#pragma unroll
  for (int ft = 0; ft < FT; ++ft) {
    dv[ft] = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint16_t* hb = ft < FT / HPARTS ? bufA : bufB;
    const int hr = 16 * (ft % (FT / HPARTS)) + l16;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      dv[ft] = mfma_bf16(*reinterpret_cast<const uint4*>(hb + swz<D>(hr, 4 * ks + g)), wf[ks], dv[ft]);
    f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) a = mfma_bf16(vt_frag<D>(hpart(ks), vxb, ft), vn[ks], a);
#pragma unroll
    for (int e = 0; e < 4; ++e) dw[ft][e] = a[e] + bf2f(zbuf[16 * ft + 4 * g + e]);
  }
  {
    float dkl[FT][4];
    phi_vjp<D, ELU>(kf, w, dw, dkl);
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) dk[ft] = f32x4{dkl[ft][0], dkl[ft][1], dkl[ft][2], dkl[ft][3]};
  }
  lds_barrier();  // every wave has read dh_j: the buffers take the query rows
  } else {
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) dv[ft] = dk[ft] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // ---- sparse branch over the query blocks that hold this key block as critical
  const uint16_t* Qb = Q + (size_t)bh * N * D;
  const uint16_t* Gb = dO + (size_t)bh * N * D;
  int koff[INSTR];
  row_offsets<D>(wave, lane, koff);
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(Qb, N * D * 2);
  const __amdgpu_buffer_rsrc_t grs = make_rsrc(Gb, N * D * 2);
  const float sc = kLog2e / sqrtf((float)D), isd = 1.0f / sqrtf((float)D);
  const float* Lh = lse2 + (size_t)bh * Nb * kBlock;
  const float* Dh = Dt + (size_t)bh * Nb * kBlock;
  // this chunk's part of the critical list: entries c0 .. c1 - 1
  const int c0 = (int)((long long)chunk * ncol / inf.x), c1 = (int)((long long)(chunk + 1) * ncol / inf.x);
  const int nstep = 2 * (c1 - c0);  // step s: queries 32 (s & 1) .. +31 of listed query block c0 + s / 2
  auto copy = [&](int s, uint16_t* dst, float* ls) {
    const int iq = __builtin_amdgcn_readfirstlane((int)list[c0 + (s >> 1)]);
    const int q0 = iq * kBlock + 32 * (s & 1);
    copy_rows<D>(qrs, grs, koff, q0, N, dst, wave);
    if (wave == 0 && lane < 8) load_lds16(Lh + q0 + 4 * lane, ls);
    if (wave == 1 && lane < 8) load_lds16(Dh + q0 + 4 * lane, ls + 32);
  };
  auto step = [&](int s, const uint16_t* cur, uint16_t* nxt, const float* lc, float* ln) {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    lds_barrier();
    uint4 qa[KS][2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
        qa[ks][qt] = *reinterpret_cast<const uint4*>(cur + swz<D>(16 * qt + l16, 4 * ks + g));
    __builtin_amdgcn_sched_barrier(0);
    if (s + 1 < nstep) copy(s + 1, nxt, ln);
    __builtin_amdgcn_sched_barrier(0);
    f32x4 sv[2], dp[2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) sv[qt] = dp[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) sv[qt] = mfma_bf16(qa[ks][qt], kr[ks], sv[qt]);
    // one operand set in registers at a time (the phases are kept apart so that
    // two waves fit on a SIMD)
    __builtin_amdgcn_sched_barrier(0);
    uint4 ga[KS][2];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
        ga[ks][qt] = *reinterpret_cast<const uint4*>(cur + HT + swz<D>(16 * qt + l16, 4 * ks + g));
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) dp[qt] = mfma_bf16(ga[ks][qt], vr[ks], dp[qt]);
    __builtin_amdgcn_sched_barrier(0);
    uint4 gtr[FT];
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) gtr[ft] = vt_frag<D>(cur + HT, vxb, ft);
    // lse2 and D_t of queries 16 qt + 4 g .. +3 (rows past N: lse2 = +inf, so P = 0)
    float p[2][4], ds[2][4];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const float4 L = *reinterpret_cast<const float4*>(lc + 16 * qt + 4 * g);
      const float4 Dd = *reinterpret_cast<const float4*>(lc + 32 + 16 * qt + 4 * g);
      const float Lr[4] = {L.x, L.y, L.z, L.w}, Dr[4] = {Dd.x, Dd.y, Dd.z, Dd.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float pr = __builtin_amdgcn_exp2f(fmaf(sv[qt][r], sc, -Lr[r]));
        p[qt][r] = al * pr;
        ds[qt][r] = pr * fmaf(al, dp[qt][r], -Dr[r]) * isd;
      }
    }
    const uint4 pb = make_uint4(pack_bf2(p[0][0], p[0][1]), pack_bf2(p[0][2], p[0][3]), pack_bf2(p[1][0], p[1][1]),
                                pack_bf2(p[1][2], p[1][3]));
    const uint4 db = make_uint4(pack_bf2(ds[0][0], ds[0][1]), pack_bf2(ds[0][2], ds[0][3]),
                                pack_bf2(ds[1][0], ds[1][1]), pack_bf2(ds[1][2], ds[1][3]));
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) dv[ft] = mfma_bf16(gtr[ft], pb, dv[ft]);
    __builtin_amdgcn_sched_barrier(0);
    uint4 qtr[FT];
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) qtr[ft] = vt_frag<D>(cur, vxb, ft);
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) dk[ft] = mfma_bf16(qtr[ft], db, dk[ft]);
  };
  if (nstep > 0) copy(0, bufA, lsA);
  for (int s = 0; s < nstep; s += 2) {  // nstep is even
    step(s, bufA, bufB, lsA, lsB);
    step(s + 1, bufB, bufA, lsB, lsA);
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  if (chunk == 0) {
    if (kv) {
#pragma unroll
      for (int ft = 0; ft < FT; ++ft) {
        *reinterpret_cast<float4*>(dK + krow + 16 * ft + 4 * g) = make_float4(dk[ft][0], dk[ft][1], dk[ft][2], dk[ft][3]);
        *reinterpret_cast<float4*>(dV + krow + 16 * ft + 4 * g) = make_float4(dv[ft][0], dv[ft][1], dv[ft][2], dv[ft][3]);
      }
    }
  } else {  // this chunk's part, added to chunk 0's by k_kv_reduce in chunk order
    float* pk = part + ((size_t)(inf.y + chunk - 1) * 2) * kBlock * D + (size_t)(16 * wave + l16) * D;
    float* pv = pk + kBlock * D;
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) {
      *reinterpret_cast<float4*>(pk + 16 * ft + 4 * g) = make_float4(dk[ft][0], dk[ft][1], dk[ft][2], dk[ft][3]);
      *reinterpret_cast<float4*>(pv + 16 * ft + 4 * g) = make_float4(dv[ft][0], dv[ft][1], dv[ft][2], dv[ft][3]);
    }
  }
}

// Block-wide exclusive scan of one int per thread (1024 threads); returns the
// exclusive prefix and leaves the total in *tot.
__device__ int block_scan_1024(int v, int* sh, int* tot) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o);
    if (lane >= o) incl += u;
  }
  if (lane == 63) sh[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    int w = lane < 16 ? sh[lane] : 0, wi = w;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const int u = __shfl_up(wi, o);
      if (lane >= o) wi += u;
    }
    if (lane < 16) sh[16 + lane] = wi - w;  // exclusive prefix of the wave sums
    if (lane == 15) sh[32] = wi;
  }
  __syncthreads();
  const int ex = sh[16 + wave] + incl - v;
  *tot = sh[32];
  __syncthreads();  // sh is reused by the next call
  return ex;
}

// The dK/dV work of key block j (its c_j critical query blocks, two 32-query
// steps each) cut into nch_j = ceil(c_j / ch) chunks of consecutive list
// entries, ch = max(kKvChunk, ceil(sum_j c_j / slots)) so that the extra chunks
// (nch_j - 1 per key block) fit the partial slots. Everything depends on the
// counts only, not on the launch order, so the chunks and the order of their
// sums are the same on every call. One workgroup: hdr = {ch, extra chunks,
// split key blocks}; info[j] = {nch_j, first slot}; tab[slot] = {j, chunk};
// list = the split key blocks in index order.
__global__ __launch_bounds__(1024) void k_kv_split(const int* __restrict__ cnt, int rows, int slots,
                                                   int* __restrict__ hdr, int2* __restrict__ info,
                                                   int2* __restrict__ tab, int* __restrict__ list) {
  __shared__ int sh[40];
  __shared__ long long ssum[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  long long t = 0;
  for (int r = tid; r < rows; r += 1024) t += cnt[r];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) t += __shfl_xor(t, o);
  if (lane == 0) ssum[wave] = t;
  __syncthreads();
  long long S = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) S += ssum[w];
  const long long need = (S + slots - 1) / slots;
  const int ch = (int)(need > kKvChunk ? need : kKvChunk);
  // each thread a contiguous range of key blocks, so the scans follow the index order
  const int per = (rows + 1023) / 1024, r0 = min(rows, tid * per), r1 = min(rows, r0 + per);
  int ext = 0, nsp = 0;
  for (int r = r0; r < r1; ++r) {
    const int n = max(1, (cnt[r] + ch - 1) / ch);
    ext += n - 1;
    nsp += n > 1;
  }
  int text, tsp;
  int slot = block_scan_1024(ext, sh, &text);
  int pos = block_scan_1024(nsp, sh, &tsp);
  for (int r = r0; r < r1; ++r) {
    const int n = max(1, (cnt[r] + ch - 1) / ch);
    info[r] = make_int2(n, slot);
    for (int k = 1; k < n; ++k) tab[slot + k - 1] = make_int2(r, k);
    if (n > 1) list[pos++] = r;
    slot += n - 1;
  }
  if (tid == 0) {
    hdr[0] = ch;
    hdr[1] = text;
    hdr[2] = tsp;
  }
}

// dK, dV of the key blocks cut into several chunks: chunk 0's values (written by
// k_bwdkv_mfma) plus the parts of chunks 1 .. nch - 1, added in chunk order.
// Workgroup (m, y) takes slice y of kKvRedY of split key block list[m]; rows past
// N are not touched; each thread's words are loaded chunk by chunk, all of them
// in flight before the adds.
template <int D>
__global__ __launch_bounds__(256) void k_kv_reduce(const int* __restrict__ hdr, const int2* __restrict__ info,
                                                   const int* __restrict__ list, const float* __restrict__ part,
                                                   float* __restrict__ dK, float* __restrict__ dV, int N, int Nb) {
  if ((int)blockIdx.x >= hdr[2]) return;
  const int id = list[blockIdx.x];
  const int2 inf = info[id];
  const int bh = id / Nb, j = id - bh * Nb;
  constexpr int Q4 = kBlock * D / 4;        // float4 words of one key block's dK (or dV)
  constexpr int PER = 2 * Q4 / kKvRedY / 256;  // words per thread
  float4 acc[PER];
  float* out[PER];
  bool live[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int x = (blockIdx.y * PER + u) * 256 + threadIdx.x;
    const int which = x / Q4, e = x % Q4, key = j * kBlock + (4 * e) / D;
    live[u] = key < N;
    out[u] = (which ? dV : dK) + ((size_t)bh * N + min(key, N - 1)) * D + (4 * e) % D;
    acc[u] = live[u] ? *reinterpret_cast<const float4*>(out[u]) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  for (int k = 1; k < inf.x; ++k) {
    float4 p[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int x = (blockIdx.y * PER + u) * 256 + threadIdx.x;
      p[u] = *reinterpret_cast<const float4*>(part + ((size_t)(inf.y + k - 1) * 2) * kBlock * D + 4 * x);
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      acc[u].x += p[u].x;
      acc[u].y += p[u].y;
      acc[u].z += p[u].z;
      acc[u].w += p[u].w;
    }
  }
#pragma unroll
  for (int u = 0; u < PER; ++u)
    if (live[u]) *reinterpret_cast<float4*>(out[u]) = acc[u];
}

// maskT[bh][j][i] = mask[bh][i][j], 64 x 64 tiles through LDS
__global__ __launch_bounds__(256) void k_mask_t(const int8_t* __restrict__ mask, int8_t* __restrict__ maskT,
                                                int Nb) {
  __shared__ int8_t t[64][65];
  const int bh = blockIdx.z, i0 = blockIdx.y * 64, j0 = blockIdx.x * 64;
  for (int x = threadIdx.x; x < 64 * 64; x += 256) {
    const int r = x / 64, c = x % 64, i = i0 + r, j = j0 + c;
    t[r][c] = (i < Nb && j < Nb) ? mask[((size_t)bh * Nb + i) * Nb + j] : (int8_t)0;
  }
  __syncthreads();
  for (int x = threadIdx.x; x < 64 * 64; x += 256) {
    const int r = x / 64, c = x % 64, j = j0 + r, i = i0 + c;
    if (i < Nb && j < Nb) maskT[((size_t)bh * Nb + j) * Nb + i] = t[c][r];
  }
}

// dH (bf16 [BH, Nb, NN]) into the layout of hx that the indicator product reads
// ([BH, Nbp / 4, NN, 4]: four consecutive blocks per 8-byte word), zero past Nb.
// A thread moves four consecutive n of four consecutive blocks: four 8-byte
// loads, four 8-byte stores (NN is a multiple of 4).
__global__ __launch_bounds__(256) void k_dh_interleave(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst,
                                                       int Nb, int Nbp, int NN) {
  const int bh = blockIdx.y;
  const int N4 = NN / 4;
  const size_t x = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (x >= (size_t)(Nbp / 4) * N4) return;
  const int q = (int)(x / N4), n = 4 * (int)(x % N4);
  uint2 v[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int i = 4 * q + k;
    v[k] = i < Nb ? *reinterpret_cast<const uint2*>(src + ((size_t)bh * Nb + i) * NN + n) : make_uint2(0u, 0u);
  }
  // v[k] holds blocks 4q + k at n .. n + 3 as (n, n+1 | n+2, n+3); word e of the output is
  // (block 4q, 4q+1 | 4q+2, 4q+3) at n + e
  uint2* out = reinterpret_cast<uint2*>(dst + (((size_t)bh * (Nbp / 4) + q) * NN + n) * 4);
  auto lo16 = [](uint32_t w) { return w & 0xffffu; };
  auto hi16 = [](uint32_t w) { return w >> 16; };
  out[0] = make_uint2(lo16(v[0].x) | (lo16(v[1].x) << 16), lo16(v[2].x) | (lo16(v[3].x) << 16));
  out[1] = make_uint2(hi16(v[0].x) | (hi16(v[1].x) << 16), hi16(v[2].x) | (hi16(v[3].x) << 16));
  out[2] = make_uint2(lo16(v[0].y) | (lo16(v[1].y) << 16), lo16(v[2].y) | (lo16(v[3].y) << 16));
  out[3] = make_uint2(hi16(v[0].y) | (hi16(v[1].y) << 16), hi16(v[2].y) | (hi16(v[3].y) << 16));
}

// cnt[row] = number of critical entries of row `row` of the transposed mask
// (the query blocks that take key block row % Nb as critical); one wave per row
__global__ __launch_bounds__(256) void k_col_count(const int8_t* __restrict__ maskT, int* __restrict__ cnt,
                                                   int Nb, int rows) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= rows) return;  // whole wave
  const int8_t* m = maskT + (size_t)row * Nb;
  int c = 0;
  for (int x0 = 0; x0 < Nb; x0 += 64) c += __popcll(__ballot(x0 + lane < Nb && m[x0 + lane] == 1));
  if (lane == 0) cnt[row] = c;
}

// order = the rows sorted by falling count (a counting sort over 0 .. Nb in one
// workgroup; rows of equal count in any order), so that the key blocks with the
// most critical query blocks start first
__global__ __launch_bounds__(1024) void k_lpt_order(const int* __restrict__ cnt, int* __restrict__ order, int Nb,
                                                    int rows) {
  __shared__ int bins[kMaxNb + 1];
  const int tid = threadIdx.x;
  for (int x = tid; x <= Nb; x += 1024) bins[x] = 0;
  __syncthreads();
  for (int r = tid; r < rows; r += 1024) atomicAdd(&bins[cnt[r]], 1);
  __syncthreads();
  if (tid < 64) {  // exclusive scan from the highest count down, 64 lanes over contiguous ranges
    const int per = (Nb + 1 + 63) / 64;
    const int hi = Nb - per * tid, lo = max(hi - per, -1);  // bins hi .. lo + 1
    int sum = 0;
    for (int c = hi; c > lo; --c) sum += bins[c];
    int incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o);
      if (tid >= o) incl += v;
    }
    int run = incl - sum;
    for (int c = hi; c > lo; --c) {
      const int n = bins[c];
      bins[c] = run;
      run += n;
    }
  }
  __syncthreads();
  for (int r = tid; r < rows; r += 1024) order[atomicAdd(&bins[cnt[r]], 1)] = r;
}

// W ([in c][out n], float32, one matrix or one per head) as bf16 A-operand
// fragments of dO_l^T = W dO^T: fragment (ct, ks) of lane (l16, g) holds
// W[16 ct + l16][32 ks + 8 g .. +7]; [Hs][FT][KS][64] uint4
template <int D>
__global__ __launch_bounds__(256) void k_pack_w(const float* __restrict__ W, uint16_t* __restrict__ wq) {
  constexpr int FT = D / 16, KS = D / 32;
  const float* Wh = W + (size_t)blockIdx.x * D * D;
  uint4* out = reinterpret_cast<uint4*>(wq + (size_t)blockIdx.x * D * D);
  for (int x = threadIdx.x; x < FT * KS * 64; x += 256) {
    const int lane = x & 63, ks = (x >> 6) % KS, ct = (x >> 6) / KS;
    const float* src = Wh + (size_t)(16 * ct + (lane & 15)) * D + 32 * ks + 8 * (lane >> 4);
    out[x] = make_uint4(pack_bf2(src[0], src[1]), pack_bf2(src[2], src[3]), pack_bf2(src[4], src[5]),
                        pack_bf2(src[6], src[7]));
  }
}

template <int D, bool ELU, bool PROJ>
hipError_t launch_mfma_t(const Dims& Dm, const void* Q, const void* K, const void* V, const int8_t* mask,
                         const float* alpha, const float* proj_o, const void* dO, const Work& w, const BwdWork& bw,
                         float* dQ, float* dK, float* dV, hipStream_t s) {
  const size_t lbytes = ((size_t)2 * Dm.Nb + 15) / 16 * 16;
  const dim3 grid(Dm.BH * Dm.Nb);
  uint16_t* dH = reinterpret_cast<uint16_t*>(bw.dHx);
  hipError_t e;
  if constexpr (PROJ) {
    hipLaunchKernelGGL(k_pack_w<D>, dim3(Dm.proj_hs ? Dm.H : 1), dim3(256), 0, s, proj_o, bw.wq);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((k_bwdq_mfma<D, ELU, PROJ>), grid, dim3(256), lbytes, s, (const uint16_t*)Q,
                     (const uint16_t*)K, (const uint16_t*)V, (const uint16_t*)dO, mask, (const uint16_t*)w.Hx, bw.Os,
                     bw.lse, alpha, (const uint16_t*)bw.wq, Dm.proj_hs, dQ, bw.dt, dH, bw.dal, bw.Ol, Dm.H, Dm.N,
                     Dm.Nb);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nt = (Dm.Nb + 63) / 64;
  hipLaunchKernelGGL(k_mask_t, dim3(nt, nt, Dm.BH), dim3(256), 0, s, mask, bw.maskT, Dm.Nb);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // dh_j = sum_i M01[i][j] dH_i: the indicator product of the forward on the transposed mask,
  // with dH in the place of hx and dh written over H_i (no longer needed)
  e = launch_indicator(Dm, bw.maskT, w, s);
  if (e != hipSuccess) return e;
  const size_t per = (size_t)(Dm.Nbp / 4) * (Dm.NN / 4);
  hipLaunchKernelGGL(k_dh_interleave, dim3((unsigned)((per + 255) / 256), Dm.BH), dim3(256), 0, s, dH,
                     (uint16_t*)w.hx, Dm.Nb, Dm.Nbp, Dm.NN);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_linear(Dm, bw.maskT, w, s);
  if (e != hipSuccess) return e;
  const int rows = Dm.BH * Dm.Nb;
  hipLaunchKernelGGL(k_col_count, dim3((rows + 3) / 4), dim3(256), 0, s, bw.maskT, bw.kvcnt, Dm.Nb, rows);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_lpt_order, dim3(1), dim3(1024), 0, s, bw.kvcnt, bw.kvorder, Dm.Nb, rows);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int slots = kv_slots(rows);
  hipLaunchKernelGGL(k_kv_split, dim3(1), dim3(1024), 0, s, bw.kvcnt, rows, slots, bw.kvhdr,
                     reinterpret_cast<int2*>(bw.kvinfo), reinterpret_cast<int2*>(bw.kvtab), bw.kvlist);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_bwdkv_mfma<D, ELU>), dim3(slots + rows), dim3(256), lbytes, s, (const uint16_t*)Q,
                     (const uint16_t*)K, (const uint16_t*)V, (const uint16_t*)dO, bw.maskT, bw.lse, bw.dt,
                     (const uint16_t*)w.Hx, PROJ ? nullptr : alpha, bw.kvorder, bw.kvhdr,
                     reinterpret_cast<const int2*>(bw.kvinfo), reinterpret_cast<const int2*>(bw.kvtab), bw.kvpart,
                     slots, dK, dV, Dm.H, Dm.N, Dm.Nb);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_kv_reduce<D>, dim3(slots, kKvRedY), dim3(256), 0, s, bw.kvhdr,
                     reinterpret_cast<const int2*>(bw.kvinfo), bw.kvlist, bw.kvpart, dK, dV, Dm.N, Dm.Nb);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_backward_mfma(const Dims& D, const void* Q, const void* K, const void* V, const int8_t* mask,
                                const float* alpha, const float* proj_o, const void* dO, const Work& w,
                                const BwdWork& bw, float* dQ, float* dK, float* dV, bool recompute,
                                hipStream_t s) {
  if (!D.bf16) return hipErrorInvalidValue;
  if (recompute) {
    // O_s and lse2 from the forward sparse kernel with this mask (O itself is not stored, so
    // the SLA2 mix runs with any alpha: the SLA fusion passes a workspace array in its place)
    hipError_t e = launch_sparse(D, Q, K, V, mask, proj_o ? bw.dal : alpha, nullptr, w, nullptr, nullptr, nullptr,
                                 s, bw.lse, bw.Os);
    if (e != hipSuccess) return e;
  }
  const bool p = proj_o != nullptr;
  if (D.d == 128) {
    if (p)
      return D.elu ? launch_mfma_t<128, true, true>(D, Q, K, V, mask, alpha, proj_o, dO, w, bw, dQ, dK, dV, s)
                   : launch_mfma_t<128, false, true>(D, Q, K, V, mask, alpha, proj_o, dO, w, bw, dQ, dK, dV, s);
    return D.elu ? launch_mfma_t<128, true, false>(D, Q, K, V, mask, alpha, proj_o, dO, w, bw, dQ, dK, dV, s)
                 : launch_mfma_t<128, false, false>(D, Q, K, V, mask, alpha, proj_o, dO, w, bw, dQ, dK, dV, s);
  }
  if (p)
    return D.elu ? launch_mfma_t<64, true, true>(D, Q, K, V, mask, alpha, proj_o, dO, w, bw, dQ, dK, dV, s)
                 : launch_mfma_t<64, false, true>(D, Q, K, V, mask, alpha, proj_o, dO, w, bw, dQ, dK, dV, s);
  return D.elu ? launch_mfma_t<64, true, false>(D, Q, K, V, mask, alpha, proj_o, dO, w, bw, dQ, dK, dV, s)
               : launch_mfma_t<64, false, false>(D, Q, K, V, mask, alpha, proj_o, dO, w, bw, dQ, dK, dV, s);
}

hipError_t launch_dw_mfma(const Dims& D, const BwdWork& bw, const void* dO, hipStream_t s) {
  const int hs = D.proj_hs ? D.H : 1;
  const dim3 grid(dw_chunks(hs), hs);
  if (D.d == 128)
    hipLaunchKernelGGL(k_bwd_dw_mfma<128>, grid, dim3(256), 0, s, bw.Ol, (const uint16_t*)dO, bw.dWg, D.B, D.H, D.N,
                       D.proj_hs ? 1 : 0, dw_chunks(hs));
  else
    hipLaunchKernelGGL(k_bwd_dw_mfma<64>, grid, dim3(256), 0, s, bw.Ol, (const uint16_t*)dO, bw.dWg, D.B, D.H, D.N,
                       D.proj_hs ? 1 : 0, dw_chunks(hs));
  return hipGetLastError();
}

}  // namespace sla
