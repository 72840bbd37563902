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
// on chip per query block). One workgroup of 4 waves owns a query block; the
// waves split the 64 keys of a tile into two halves and the 64 queries into
// two halves. Tiles arrive by direct global->LDS copies (no register
// staging), double-buffered one tile ahead, one barrier per tile. Per tile:
//   S^T = K Q^T    MFMA 16x16x32, the wave's 32 keys as A (row-swizzled LDS),
//                  its 32 queries (registers) as B; a lane gets 4 keys of one
//                  query per 16-key tile;
//   online softmax per wave against a reference max that is only raised
//                  when some score exceeds it by more than 2^8: the common
//                  path needs no cross-lane reduction and no rescale (exact:
//                  softmax does not depend on the reference); the row sums
//                  of P come from one more MFMA per query tile with an A
//                  operand whose row 0 is all ones;
//   O^T += V^T P^T MFMA 16x16x32 with P^T straight from registers: a lane's 8
//                  k slots are its keys {4g..4g+3, 16+4g..16+4g+3}, and the h/z
//                  kernel stored V^T in that key order.
// All K fragments of a tile are read before its first product and the V^T
// fragments right after the last one, so their LDS latency overlaps. While the
// last tile is processed, H_i^T (from K4's output, rows swizzled like K) is
// copied into the idle tile buffer and Z_i into the spent critical list.
// The two key halves are combined through LDS (max-rescaled partial sums);
// each wave then finishes all features of one 16-query tile (so phi is formed
// once per query): O_s = acc / l, phi(Q) (softmax over the features in f32,
// left unnormalised because the normalisation cancels in O_l, rounded to
// bf16), num^T = H_i^T phi(Q)^T and den = phi(Q).Z_i on MFMA (Z_i as row 0 of
// an A operand), O = alpha O_s + (1 - alpha) O_l, staged in LDS and written
// as full rows.
// Workgroups are remapped so that each XCD walks a contiguous range of
// (batch, head, query block): neighbouring query blocks share most critical
// key tiles, which then come from the XCD's L2.
//
// f32 path: 4 threads per query, plain FMA, one key at a time.
#include <type_traits>

#include "sla_internal.h"
#include "dev_common.h"

namespace sla {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

template <int D>
struct FaCfg {
  static constexpr int C = D / 8;                  // 16-byte chunks per K row
  static constexpr int TILE = kBlock * D;          // elements of one K (or V^T) tile
  static constexpr int INSTR = TILE / 8 / 256;     // 16-byte async copies per lane per operand
  static constexpr int NN = D * D + D;
  static constexpr int KSTEPS = D / 32;
  static constexpr int FT = D / 16;                // feature tiles of O
  static constexpr int OS = D + 8;                 // LDS row stride of the staged output
  static constexpr int HINSTR = D * D / 8 / 256;   // 16-byte copies per lane of H_i^T
};

// Workgroup: 4 waves, one query block (64 queries). Wave w takes key half
// kh = w & 1 (keys 32kh .. 32kh+31 of every critical tile) and query half
// qh = w >> 1 (queries 32qh .. 32qh+31), so every product is a full-rate
// 16x16x32 MFMA (the P.V product contracts over the wave's 32 keys). Each wave
// keeps its own reference maximum per query; the two key halves are combined
// once at the end like the partial results of a split softmax.
template <int D>
__global__ __launch_bounds__(256, 2) void k_sparse_bf16(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ vt, const int8_t* __restrict__ mask,
    const uint16_t* __restrict__ Hx, const float* __restrict__ alpha, uint16_t* __restrict__ O,
    float* __restrict__ dbg_os, float* __restrict__ dbg_ol, int H, int N, int Nb) {
  using Cf = FaCfg<D>;
  constexpr int C = Cf::C, TILE = Cf::TILE, INSTR = Cf::INSTR, NN = Cf::NN;
  constexpr int KSTEPS = Cf::KSTEPS, FT = Cf::FT, OS = Cf::OS, HINSTR = Cf::HINSTR;
  constexpr float TAU = 8.0f;  // a stale reference max may lag the tile max by 2^8 at most
  // Two tile buffers (K then V^T each) as distinct LDS objects, so that reads of
  // one provably do not alias the asynchronous copies into the other.
  __shared__ __attribute__((aligned(16))) uint16_t bufA[2 * TILE];
  __shared__ __attribute__((aligned(16))) uint16_t bufB[2 * TILE];
  __shared__ __attribute__((aligned(16))) uint16_t list[kMaxNb];  // critical list, then Z_i
  __shared__ float xm[4][2][16];
  __shared__ float xl[4][2][16];
  __shared__ int wsum[4 * kMaskPre];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar LDS addresses
  const int l16 = lane & 15, g = lane >> 4;
  const int kh = wave & 1, qh = wave >> 1;
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = id / Nb, i = id - bh * Nb;
  const int h = bh % H;

  // the mask row first, then the wave's 32 queries as MFMA B operands:
  // Q[t][32ks + 8g .. +7] (they land while the critical list is compacted)
  const int8_t* mrow = mask + ((size_t)bh * Nb + i) * Nb;
  int8_t mv[kMaskPre];
  mask_load(mrow, Nb, mv);
  uint4 qr[2][KSTEPS];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int t = min(i * kBlock + 32 * qh + 16 * qt + l16, N - 1);  // rows past N are never stored
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
      qr[qt][ks] = *reinterpret_cast<const uint4*>(Q + ((size_t)bh * N + t) * D + 32 * ks + 8 * g);
  }

  const int ncrit = compact_loaded(mv, mrow, Nb, (int8_t)1, list, wsum);

  const uint16_t* Kb = K + (size_t)bh * N * D;
  const uint16_t* Vb = vt + (size_t)bh * Nb * TILE;
  // K rows land in LDS with their 16-byte chunks XOR-swizzled by the row
  // index (16 lanes reading 16 rows at one column hit distinct banks); the
  // V^T tile is copied as laid out by the h/z kernel. The per-lane source
  // offsets within a tile are the same for every tile.
  int koff[INSTR];
#pragma unroll
  for (int u = 0; u < INSTR; ++u) {
    const int G = 64 * (4 * u + wave) + lane;
    const int r = G / C, sch = G % C;
    koff[u] = r * D + (sch ^ (r & (C - 1))) * 8;
  }
  // Copies go through buffer resources over this head's K rows and V^T tiles:
  // the per-lane byte offsets stay in registers and the tile offset j * TILE
  // (wave-uniform) is the scalar offset, so issuing a tile costs no vector
  // instruction.
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(Kb, N * D * 2);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(Vb, Nb * TILE * 2);
  auto issue = [&](int jv, uint16_t* dst) {
    const int j = __builtin_amdgcn_readfirstlane(jv);
    const int soff = j * TILE * 2;
    if ((j + 1) * kBlock > N) {  // ragged block: rows past N re-read row N-1 (masked below)
      const int over = j * kBlock - (N - 1);
#pragma unroll
      for (int u = 0; u < INSTR; ++u) {
        const int off = koff[u] - max(0, koff[u] / D + over) * D;
        load_lds16_buf(krs, 2 * off, soff, dst + 512 * (4 * u + wave));
        load_lds16_buf(vrs, (64 * (4 * u + wave) + lane) * 16, soff, dst + TILE + 512 * (4 * u + wave));
      }
    } else {
#pragma unroll
      for (int u = 0; u < INSTR; ++u) {
        load_lds16_buf(krs, 2 * koff[u], soff, dst + 512 * (4 * u + wave));
        load_lds16_buf(vrs, (64 * (4 * u + wave) + lane) * 16, soff, dst + TILE + 512 * (4 * u + wave));
      }
    }
  };
  // H_i^T (d x d, rows swizzled like the K tiles) into a free tile buffer, and
  // Z_i into the critical-list area, for the epilogue
  const uint16_t* Hrow = Hx + ((size_t)bh * Nb + i) * NN;
  uint16_t* zbuf = list;
  auto issueH = [&](uint16_t* dst) {
#pragma unroll
    for (int u = 0; u < HINSTR; ++u) {
      const int G = 64 * (4 * u + wave) + lane;
      const int r = G / C, sch = G % C;
      load_lds16(Hrow + r * D + (sch ^ (r & (C - 1))) * 8, dst + 512 * (4 * u + wave));
    }
    if (wave == 0 && lane < C) load_lds16(Hrow + D * D + 8 * lane, zbuf);
  };

  const float sc = kLog2e / sqrtf((float)D);
  f32x4 acc[FT][2];
#pragma unroll
  for (int ft = 0; ft < FT; ++ft) acc[ft][0] = acc[ft][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mref[2] = {-INFINITY, -INFINITY};
  // Row sums of P come out of the MFMA unit: an A operand whose row 0 is all
  // ones gives sum_k P[k][q] in row 0 of the product (lane group 0, register 0)
  // and is rescaled together with acc.
  f32x4 accl[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  const uint32_t one2 = l16 == 0 ? 0x3f803f80u : 0u;  // two bf16 ones in row 0
  const uint4 ones = make_uint4(one2, one2, one2, one2);

  // one tile: wait for it, start the copy of the next one into the other
  // buffer, S^T, online softmax against the wave's reference max, O^T += V^T P^T
  auto step = [&](int c, const uint16_t* cur, uint16_t* nxt) {
    const int j = __builtin_amdgcn_readfirstlane((int)list[c]);
    const int jn = list[min(c + 1, ncrit - 1)];  // read before the K fragments queue behind it
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // this wave's copies of tile c have landed
    lds_barrier();  // all copies of tile c are in LDS; every wave is done with tile c-1
    // all K fragments of the tile first (their LDS latency overlaps the issue of
    // the next tile's copies), then the products
    uint4 ka[KSTEPS][2];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const int row = 32 * kh + 16 * kt + l16;
        ka[ks][kt] = *reinterpret_cast<const uint4*>(cur + (row * C + ((4 * ks + g) ^ (row & (C - 1)))) * 8);
      }
    __builtin_amdgcn_sched_barrier(0);
    if (c + 1 < ncrit)
      issue(jn, nxt);
    else
      issueH(nxt);  // every wave has read list[c]: the list area is free
    __builtin_amdgcn_sched_barrier(0);
    f32x4 s[2][2];  // [key tile][query tile]
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) s[kt][0] = s[kt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) s[kt][qt] = mfma_bf16(ka[ks][kt], qr[qt][ks], s[kt][qt]);
    // the V^T fragments of the tile load while the softmax runs
    const uint16_t* vtile = cur + TILE + kh * D * 32;
    uint4 va[FT];
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) {
      const int c = 16 * ft + l16;
      va[ft] = *reinterpret_cast<const uint4*>(vtile + c * 32 + 8 * (g ^ ((c >> 1) & 3)));
    }
    __builtin_amdgcn_sched_barrier(0);
    if ((j + 1) * kBlock > N) {  // ragged last block: keys past N take no part
      const int kbase = j * kBlock + 32 * kh + 4 * g;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool out = kbase + 16 * kt + r >= N;
#pragma unroll
          for (int qt = 0; qt < 2; ++qt) s[kt][qt][r] = out ? -INFINITY : s[kt][qt][r];
        }
    }
    // Reference max: raised only when some score exceeds it by more than 2^8
    // (rare after the first tile); the 4 lane groups of a query then agree on
    // the new value through a cross-group max, and acc / l are rescaled.
    float lmax[2];
    bool raise = false;
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      lmax[qt] = fmaxf(fmaxf(fmaxf(s[0][qt][0], s[0][qt][1]), fmaxf(s[0][qt][2], s[0][qt][3])),
                       fmaxf(fmaxf(s[1][qt][0], s[1][qt][1]), fmaxf(s[1][qt][2], s[1][qt][3]))) * sc;
      raise |= lmax[qt] > mref[qt] + TAU;
    }
    if (__ballot(raise)) {
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        const float tm = group4_max(lmax[qt]);
        const float nref = tm > mref[qt] + TAU ? tm : mref[qt];
        const float fac = nref == mref[qt] ? 1.0f : __builtin_amdgcn_exp2f(mref[qt] - nref);
        mref[qt] = nref;
        accl[qt] *= fac;
#pragma unroll
        for (int ft = 0; ft < FT; ++ft) acc[ft][qt] *= fac;
      }
    }
    uint4 pb[2];
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const float meff = mref[qt] == -INFINITY ? 0.0f : mref[qt];  // no valid key yet: every p is 0
      float p[2][4];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) p[kt][r] = __builtin_amdgcn_exp2f(fmaf(s[kt][qt][r], sc, -meff));
      pb[qt] = make_uint4(pack_bf2(p[0][0], p[0][1]), pack_bf2(p[0][2], p[0][3]),
                          pack_bf2(p[1][0], p[1][1]), pack_bf2(p[1][2], p[1][3]));
    }
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) {
      acc[ft][0] = mfma_bf16(va[ft], pb[0], acc[ft][0]);
      acc[ft][1] = mfma_bf16(va[ft], pb[1], acc[ft][1]);
    }
    accl[0] = mfma_bf16(ones, pb[0], accl[0]);
    accl[1] = mfma_bf16(ones, pb[1], accl[1]);
  };
  if (ncrit > 0)
    issue(list[0], bufA);
  else
    issueH(bufA);
  for (int c = 0; c < ncrit; c += 2) {
    step(c, bufA, bufB);
    if (c + 1 < ncrit) step(c + 1, bufB, bufA);
  }

  // ---- combine the two key halves: wave (kh, qh) finishes every feature of
  // query tile kh of its query half, so each query's phi(Q) is formed once
  float lw[2];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) lw[qt] = __shfl(accl[qt][0], l16);  // from lane group 0
  // the last tile's buffer takes the exchange and then the staged output; H_i^T
  // arrived in the other one (bufA when there was no tile)
  uint16_t* xbuf = (ncrit & 1) ? bufA : bufB;
  const uint16_t* hbuf = (ncrit & 1) ? bufB : bufA;
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // this wave's copies of H_i^T and Z_i
  __syncthreads();  // every wave is done with the tile buffers; H_i^T and Z_i have landed
  float* ex = reinterpret_cast<float*>(xbuf);  // [wave][FT][64 lanes][4]
  // The query tile is chosen with compile-time indices (a runtime index would
  // send the accumulator array through scratch memory): wave kh sends its
  // partial sums of query tile 1 - kh and keeps those of query tile kh.
  auto send = [&](auto KH) {
    constexpr int qs = 1 - decltype(KH)::value;
#pragma unroll
    for (int ft = 0; ft < FT; ++ft)
      *reinterpret_cast<f32x4*>(ex + ((wave * FT + ft) * 64 + lane) * 4) = acc[ft][qs];
  };
  if (kh == 0) send(std::integral_constant<int, 0>{}); else send(std::integral_constant<int, 1>{});
  if (g == 0) {
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      xm[wave][qt][l16] = mref[qt];
      xl[wave][qt][l16] = lw[qt];
    }
  }
  __syncthreads();
  // own (this wave's partial sums), oth (the partner's) and their max-rescale
  // weights w0, w1; O_s = (w0 own + w1 oth) / l
  const int partner = wave ^ 1;
  f32x4 own[FT], oth[FT];
  float w0, w1, inv_l;
  uint4 qk[KSTEPS];  // the query tile's Q fragments
  auto keep = [&](auto KH) {
    constexpr int qt = decltype(KH)::value;
    const float m0 = mref[qt], m1 = xm[partner][qt][l16];
    const float M = fmaxf(m0, m1);
    w0 = m0 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m0 - M);
    w1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - M);
    const float l = w0 * lw[qt] + w1 * xl[partner][qt][l16];
    inv_l = l > 0.f ? 1.0f / l : 0.f;
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) {
      own[ft] = acc[ft][qt];
      oth[ft] = *reinterpret_cast<const f32x4*>(ex + ((partner * FT + ft) * 64 + lane) * 4);
    }
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) qk[ks] = qr[qt][ks];
  };
  if (kh == 0) keep(std::integral_constant<int, 0>{}); else keep(std::integral_constant<int, 1>{});

  // ---- linear branch for the wave's 16 queries: phi(Q); den = phi(Q).Z_i and
  // num^T = H_i^T phi(Q)^T on MFMA
  float qf[KSTEPS * 8];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    const uint32_t w4[4] = {qk[ks].x, qk[ks].y, qk[ks].z, qk[ks].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qf[ks * 8 + 2 * e] = bf_lo(w4[e]);
      qf[ks * 8 + 2 * e + 1] = bf_hi(w4[e]);
    }
  }
  float qm = -INFINITY;
#pragma unroll
  for (int e = 0; e < KSTEPS * 8; ++e) qm = fmaxf(qm, qf[e]);
  qm = group4_max(qm) * kLog2e;
  // e = exp(q - max q); phi(Q) = e / sum(e), but the sum cancels between the
  // numerator phi(Q) H_i and the denominator phi(Q) Z_i, so e enters both unscaled
  uint4 fq[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    uint32_t w4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w4[e] = pack_bf2(__builtin_amdgcn_exp2f(fmaf(qf[ks * 8 + 2 * e], kLog2e, -qm)),
                       __builtin_amdgcn_exp2f(fmaf(qf[ks * 8 + 2 * e + 1], kLog2e, -qm)));
    fq[ks] = make_uint4(w4[0], w4[1], w4[2], w4[3]);
  }
  // den: an A operand whose row 0 is Z_i gives phi(Q).Z_i in row 0 of the product
  f32x4 dacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    const uint4 z = *reinterpret_cast<const uint4*>(zbuf + 32 * ks + 8 * g);
    dacc = mfma_bf16(l16 == 0 ? z : make_uint4(0u, 0u, 0u, 0u), fq[ks], dacc);
  }
  const float den = __shfl(dacc[0], l16);  // from lane group 0
  const float inv_den = den > 0.f ? 1.0f / den : 0.f;
  const float al = alpha[h];
  const float cs0 = al * inv_l * w0, cs1 = al * inv_l * w1, cl = (1.0f - al) * inv_den;
  __syncthreads();  // every wave has read the exchange area: it becomes the output stage
  uint16_t* ost = xbuf;  // staged output tile [64][OS]
  const int q = 32 * qh + 16 * kh + l16;
  const int t = i * kBlock + q;
  const bool dbg = (dbg_os || dbg_ol) && t < N;
#pragma unroll
  for (int ft = 0; ft < FT; ++ft) {
    f32x4 nm = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const int hr = 16 * ft + l16;
      const uint4 a = *reinterpret_cast<const uint4*>(hbuf + (hr * C + ((4 * ks + g) ^ (hr & (C - 1)))) * 8);
      nm = mfma_bf16(a, fq[ks], nm);
    }
    float o[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) o[r] = fmaf(own[ft][r], cs0, fmaf(oth[ft][r], cs1, nm[r] * cl));
    *reinterpret_cast<uint2*>(ost + q * OS + 16 * ft + 4 * g) =
        make_uint2(pack_bf2(o[0], o[1]), pack_bf2(o[2], o[3]));
    if (dbg) {
      const size_t off = ((size_t)bh * N + t) * D + 16 * ft + 4 * g;
      float os[4], ol[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        os[r] = (own[ft][r] * w0 + oth[ft][r] * w1) * inv_l;
        ol[r] = nm[r] * inv_den;
      }
      if (dbg_os) *reinterpret_cast<float4*>(dbg_os + off) = make_float4(os[0], os[1], os[2], os[3]);
      if (dbg_ol) *reinterpret_cast<float4*>(dbg_ol + off) = make_float4(ol[0], ol[1], ol[2], ol[3]);
    }
  }
  __syncthreads();
  // full-row 16-byte stores of the staged tile
  const int nrow = min(kBlock, N - i * kBlock);
  uint16_t* Ob = O + ((size_t)bh * N + (size_t)i * kBlock) * D;
  for (int x = tid; x < nrow * C; x += 256) {
    const int row = x / C, ch = x % C;
    *reinterpret_cast<uint4*>(Ob + (size_t)row * D + ch * 8) =
        *reinterpret_cast<const uint4*>(ost + row * OS + ch * 8);
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
