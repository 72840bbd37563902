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
// on chip per query block). One workgroup of 4 waves owns a query block; wave
// w owns queries 16w .. 16w+15 against every key, so its online softmax needs
// no partner. The keys of a critical tile are taken 32 at a time (a step):
// the K rows and V rows of a step arrive by direct global->LDS copies (no
// register staging) into one of two 16 KB buffers, one step ahead, one barrier
// per step. Per step:
//   S^T = K Q^T    MFMA 16x16x32, the step's 32 keys as A (row-swizzled LDS),
//                  the wave's 16 queries (registers) as B; a lane gets 4 keys
//                  of one query per 16-key tile;
//   online softmax against a reference max that is only raised when some
//                  score exceeds it by more than 2^8: the common path needs no
//                  cross-lane reduction and no rescale (exact: softmax does
//                  not depend on the reference); the row sums of P come from
//                  one more MFMA with an A operand whose row 0 is all ones;
//   O^T += V^T P^T MFMA 16x16x32 with P^T straight from registers: a lane's 8
//                  k slots are its keys {4g..4g+3, 16+4g..16+4g+3}; the V^T
//                  operand comes from the V rows in LDS through gfx950's
//                  transposed LDS reads (ds_read_b64_tr_b16), in that key order.
// All K fragments of a step are read before the next step's copies are issued
// and before its first product, and the V^T fragments right after the last
// one, so their LDS latency overlaps. Each wave owns two 16-query groups (two
// waves per query block), so every fragment it reads from LDS feeds two
// products. During the last step the first half of
// H_i^T (from K4's output, rows swizzled like K) is copied into the idle buffer
// and Z_i into the spent critical list; the second half follows into the other
// buffer while phi(Q) is formed. Each wave then finishes its 16 queries:
// O_s = acc / l, phi(Q) (softmax over the features in f32, left unnormalised
// because the normalisation cancels in O_l, rounded to bf16), num^T =
// H_i^T phi(Q)^T and den = phi(Q).Z_i on MFMA (Z_i as row 0 of an A operand),
// O = alpha O_s + (1 - alpha) O_l, staged in LDS and written as full rows.
// The SLA fusion O = O_s + Proj(O_l) (SLA paper summary, section 4, step 4)
// is a second epilogue product: num^T, rounded to bf16, is already in the k-slot
// order of a B operand (each lane holds features {4g..4g+3, 16+4g..16+4g+3} of
// every 32-feature step), and Proj^T comes as A-operand fragments packed once
// per call in that same feature order (k_pack_proj), read straight from L2;
// (num Proj)^T has num^T's layout, so the mix and the stores are unchanged.
// With phi = elu + 1 (SLA paper summary, Eq. 3's symbol list) phi(Q) is taken
// elementwise instead of the softmax over the features.
// Workgroups are remapped so that each XCD walks a contiguous range of
// (batch, head, query block): neighbouring query blocks share most critical
// key tiles, which then come from the XCD's L2.
//
// f32 path: 4 threads per query, plain FMA, one key at a time.
#include <stdlib.h>

#include <type_traits>

#include "sla_internal.h"
#include "dev_common.h"

namespace sla {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

template <int D, int NW>
struct FaCfg {
  static constexpr int NT = 64 * NW;               // threads of a workgroup
  static constexpr int QG = 4 / NW;                // 16-query groups a wave owns
  static constexpr int C = D / 8;                  // 16-byte chunks per K row
  static constexpr int HT = 32 * D;                // elements of one half tile (32 keys) of K or of V^T
  static constexpr int INSTR = HT / 8 / NT;        // 16-byte async copies per lane per operand and step
  static constexpr int NN = D * D + D;
  static constexpr int KSTEPS = D / 32;
  static constexpr int FT = D / 16;                // feature tiles of O
  static constexpr int OS = D + 8;                 // LDS row stride of the staged output
  static constexpr int HROWS = 2 * HT / D;         // rows of H_i^T one step buffer holds (64)
  static constexpr int HPARTS = D / HROWS;         // buffers H_i^T takes (2 at d = 128, 1 at d = 64)
  static constexpr int HINSTR = HROWS * D / 8 / NT;  // 16-byte copies per lane of one part
};

// Workgroup: NW waves, one query block (64 queries). Wave w owns the QG = 4/NW
// groups of 16 queries 16 QG w .. 16 QG w + 16 QG - 1 against every key, so
// its softmax needs no partner; every K and V^T fragment a wave reads from LDS
// feeds the products of all its query groups, so two groups per wave (NW = 2)
// halve the LDS bytes per flop of one group per wave (NW = 4). The keys of a
// critical tile are taken 32 at a time (a step), so that each product is a
// full-rate 16x16x32 MFMA (P.V contracts over the step's 32 keys) and the step
// buffers are 16 KB. The critical list lives in dynamic LDS of
// max(2 Nb, 2 D) bytes.
// LSE: also write each query's log2 softmax normaliser and O_s as two bf16 planes
// hi + lo (for the backward pass; a separate instance so that the plain forward
// pays nothing).
template <int D, int NW, bool PROJ, bool ELU, bool LSE>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW == 2 ? 2 : 3, NW == 2 ? 2 : 3)))
void k_sparse_bf16(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const int8_t* __restrict__ mask,
    const uint16_t* __restrict__ Hx, const float* __restrict__ alpha,
    const uint16_t* __restrict__ wo, int wo_hs, uint16_t* __restrict__ O,
    float* __restrict__ dbg_os, float* __restrict__ dbg_ol, float* __restrict__ lse_out,
    uint16_t* __restrict__ os_out, uint16_t* __restrict__ os_lo, int H, int N, int Nb) {
  using Cf = FaCfg<D, NW>;
  constexpr int NT = Cf::NT, QG = Cf::QG;
  constexpr int C = Cf::C, HT = Cf::HT, INSTR = Cf::INSTR, NN = Cf::NN;
  constexpr int KSTEPS = Cf::KSTEPS, FT = Cf::FT, OS = Cf::OS;
  constexpr int HROWS = Cf::HROWS, HPARTS = Cf::HPARTS, HINSTR = Cf::HINSTR;
  constexpr float TAU = 8.0f;  // a stale reference max may lag the step max by 2^8 at most
  // Two step buffers (32 K rows, then the matching 32 columns of V^T) as
  // distinct LDS objects, so that reads of one provably do not alias the
  // asynchronous copies into the other.
  __shared__ __attribute__((aligned(16))) uint16_t bufA[2 * HT];
  __shared__ __attribute__((aligned(16))) uint16_t bufB[2 * HT];
  extern __shared__ __attribute__((aligned(16))) uint16_t list[];  // critical list, then Z_i
  __shared__ int wsum[NW * kMaskPre];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar LDS addresses
  const int l16 = lane & 15, g = lane >> 4;
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = id / Nb, i = id - bh * Nb;
  const int h = bh % H;

  // the mask row first, then the wave's queries as MFMA B operands:
  // Q[t][32ks + 8g .. +7] (they land while the critical list is compacted)
  const int8_t* mrow = mask + ((size_t)bh * Nb + i) * Nb;
  int8_t mv[kMaskPre];
  mask_load<NT>(mrow, Nb, mv);
  uint4 qr[QG][KSTEPS];
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    const int t = min(i * kBlock + 16 * (QG * wave + qg) + l16, N - 1);  // rows past N are never stored
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
      qr[qg][ks] = *reinterpret_cast<const uint4*>(Q + ((size_t)bh * N + t) * D + 32 * ks + 8 * g);
  }

  const int ncrit = compact_loaded<NT>(mv, mrow, Nb, (int8_t)1, list, wsum);
  const int nstep = 2 * ncrit;  // step s: keys 32 (s & 1) .. +31 of critical tile s >> 1

  const uint16_t* Kb = K + (size_t)bh * N * D;
  const uint16_t* Vb = V + (size_t)bh * N * D;
  // K and V rows land in LDS with their 16-byte chunks XOR-swizzled by the row
  // index (16 lanes reading 16 rows at one chunk hit distinct banks, and a
  // transposed read of 32 bytes from each of 16 V rows takes the two cycles
  // its 512 bytes need). The per-lane source offsets within a half tile are the
  // same for every step and for K and V.
  int koff[INSTR];
#pragma unroll
  for (int u = 0; u < INSTR; ++u) {
    const int G = 64 * (NW * u + wave) + lane;
    const int r = G / C, sch = G % C;
    koff[u] = r * D + (sch ^ row_swz<D>(r)) * 8;
  }
  const int vxb = vt_base<D>(g, l16);
  // Copies go through buffer resources over this head's K and V rows: the
  // per-lane byte offsets stay in registers and the step's offset
  // (wave-uniform) is the scalar offset.
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(Kb, N * D * 2);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(Vb, N * D * 2);
  auto issue = [&](auto RAGc, int j, int hh, uint16_t* dst) {
    constexpr bool RAG = decltype(RAGc)::value;
    const int row0 = j * kBlock + 32 * hh;
    const int sk = row0 * D * 2;
    if constexpr (RAG) {  // ragged: rows past N re-read row N-1 (their P is 0)
      const int over = row0 - (N - 1);
#pragma unroll
      for (int u = 0; u < INSTR; ++u) {
        const int off = koff[u] - max(0, koff[u] / D + over) * D;
        load_lds16_buf(krs, 2 * off, sk, dst + 512 * (NW * u + wave));
        load_lds16_buf(vrs, 2 * off, sk, dst + HT + 512 * (NW * u + wave));
      }
    } else {
#pragma unroll
      for (int u = 0; u < INSTR; ++u) {
        load_lds16_buf(krs, 2 * koff[u], sk, dst + 512 * (NW * u + wave));
        load_lds16_buf(vrs, 2 * koff[u], sk, dst + HT + 512 * (NW * u + wave));
      }
    }
  };
  // H_i^T (d x d, rows swizzled like the K rows) in parts of HROWS rows, one
  // step buffer each, and Z_i into the critical-list area, for the epilogue
  const uint16_t* Hrow = Hx + ((size_t)bh * Nb + i) * NN;
  uint16_t* zbuf = list;
  auto issueH = [&](int part, uint16_t* dst) {
#pragma unroll
    for (int u = 0; u < HINSTR; ++u) {
      const int G = 64 * (NW * u + wave) + lane;
      const int r = G / C, sch = G % C;
      load_lds16(Hrow + (part * HROWS + r) * D + (sch ^ row_swz<D>(r)) * 8, dst + 512 * (NW * u + wave));
    }
    if (part == 0 && wave == 0 && lane < C) load_lds16(Hrow + D * D + 8 * lane, zbuf);
  };

  const float sc = kLog2e / sqrtf((float)D);
  f32x4 acc[QG][FT];
#pragma unroll
  for (int qg = 0; qg < QG; ++qg)
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) acc[qg][ft] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mref[QG];
  // Row sums of P come out of the MFMA unit: an A operand whose row 0 is all
  // ones gives sum_k P[k][q] in row 0 of the product (lane group 0, register 0)
  // and is rescaled together with acc.
  f32x4 accl[QG];
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    mref[qg] = -INFINITY;
    accl[qg] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const uint32_t one2 = l16 == 0 ? 0x3f803f80u : 0u;  // two bf16 ones in row 0
  const uint4 ones = make_uint4(one2, one2, one2, one2);

  // one step: wait for its half tile, start the copy of the next one into the
  // other buffer, S^T, online softmax against each group's reference max,
  // O^T += V^T P^T
  auto step = [&](int s, const uint16_t* cur, uint16_t* nxt) {
    const int j = __builtin_amdgcn_readfirstlane((int)list[s >> 1]);
    const int hh = s & 1;
    const int jn = list[min((s + 1) >> 1, ncrit - 1)];  // read before the K fragments queue behind it
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));  // this wave's copies of step s have landed
    lds_barrier();  // all copies of step s are in LDS; every wave is done with step s-1
    // all K fragments of the step first (their LDS latency overlaps the issue of
    // the next step's copies), then the products
    uint4 ka[KSTEPS][2];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const int row = 16 * kt + l16;
        ka[ks][kt] = *reinterpret_cast<const uint4*>(cur + (row * C + ((4 * ks + g) ^ row_swz<D>(row))) * 8);
      }
    __builtin_amdgcn_sched_barrier(0);
    // S^T products; the copies of the next step are issued between them, so
    // that a copy waiting for the memory pipeline holds up no product
    f32x4 sv[QG][2];  // [query group][key tile]
    auto sprod = [&]() {
#pragma unroll
      for (int qg = 0; qg < QG; ++qg) sv[qg][0] = sv[qg][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int qg = 0; qg < QG; ++qg) sv[qg][kt] = mfma_bf16(ka[ks][kt], qr[qg][ks], sv[qg][kt]);
    };
    auto spread = [&]() {
#pragma unroll
      for (int u = 0; u < 2 * INSTR; ++u) {
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * KSTEPS * QG / (2 * INSTR), 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
    };
    if (s + 1 < nstep) {
      const int jnu = __builtin_amdgcn_readfirstlane(jn);
      const int hn = (s + 1) & 1;
      if (jnu * kBlock + 32 * hn + 32 > N) {
        issue(std::true_type{}, jnu, hn, nxt);
        sprod();
        spread();
      } else {
        issue(std::false_type{}, jnu, hn, nxt);
        sprod();
        spread();
      }
    } else {
      issueH(0, nxt);  // every wave has read list[s >> 1]: the list area is free
      sprod();
    }
    __builtin_amdgcn_sched_barrier(0);
    // the V^T fragments of the step (transposed reads of the V rows) load
    // while the softmax runs
    const uint16_t* vtile = cur + HT;
    uint4 va[FT];
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) va[ft] = vt_frag<D>(vtile, vxb, ft);
    __builtin_amdgcn_sched_barrier(0);
    if (j * kBlock + 32 * hh + 32 > N) {  // ragged last block: keys past N take no part
      const int kbase = j * kBlock + 32 * hh + 4 * g;
#pragma unroll
      for (int qg = 0; qg < QG; ++qg)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) sv[qg][kt][r] = kbase + 16 * kt + r >= N ? -INFINITY : sv[qg][kt][r];
    }
    // Reference max: raised only when some score exceeds it by more than 2^8
    // (rare after the first step); the 4 lane groups of a query then agree on
    // the new value through a cross-group max, and acc / l are rescaled.
    float lmax[QG];
    bool raise = false;
#pragma unroll
    for (int qg = 0; qg < QG; ++qg) {
      lmax[qg] = fmaxf(fmaxf(fmaxf(sv[qg][0][0], sv[qg][0][1]), fmaxf(sv[qg][0][2], sv[qg][0][3])),
                       fmaxf(fmaxf(sv[qg][1][0], sv[qg][1][1]), fmaxf(sv[qg][1][2], sv[qg][1][3]))) * sc;
      raise = raise || lmax[qg] > mref[qg] + TAU;
    }
    if (__ballot(raise)) {
#pragma unroll
      for (int qg = 0; qg < QG; ++qg) {
        const float tm = group4_max(lmax[qg]);
        const float nref = tm > mref[qg] + TAU ? tm : mref[qg];
        const float fac = nref == mref[qg] ? 1.0f : __builtin_amdgcn_exp2f(mref[qg] - nref);
        mref[qg] = nref;
        accl[qg] *= fac;
#pragma unroll
        for (int ft = 0; ft < FT; ++ft) acc[qg][ft] *= fac;
      }
    }
    uint4 pb[QG];
#pragma unroll
    for (int qg = 0; qg < QG; ++qg) {
      const float meff = mref[qg] == -INFINITY ? 0.0f : mref[qg];  // no valid key yet: every p is 0
      float p[2][4];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) p[kt][r] = __builtin_amdgcn_exp2f(fmaf(sv[qg][kt][r], sc, -meff));
      pb[qg] = make_uint4(pack_bf2(p[0][0], p[0][1]), pack_bf2(p[0][2], p[0][3]),
                          pack_bf2(p[1][0], p[1][1]), pack_bf2(p[1][2], p[1][3]));
    }
#pragma unroll
    for (int ft = 0; ft < FT; ++ft)
#pragma unroll
      for (int qg = 0; qg < QG; ++qg) acc[qg][ft] = mfma_bf16(va[ft], pb[qg], acc[qg][ft]);
#pragma unroll
    for (int qg = 0; qg < QG; ++qg) accl[qg] = mfma_bf16(ones, pb[qg], accl[qg]);
  };
  if (nstep > 0) {
    const int j0 = __builtin_amdgcn_readfirstlane((int)list[0]);
    if (j0 * kBlock + 32 > N)
      issue(std::true_type{}, j0, 0, bufA);
    else
      issue(std::false_type{}, j0, 0, bufA);
  }
  else
    issueH(0, bufA);
  for (int s = 0; s < nstep; s += 2) {  // nstep is even
    step(s, bufA, bufB);
    step(s + 1, bufB, bufA);
  }

  // ---- epilogue: O_s = acc / l; phi(Q) of the wave's queries; den =
  // phi(Q).Z_i and num^T = H_i^T phi(Q)^T on MFMA; the mix; full-row stores.
  // H_i^T part 0 went into bufA during the last step (in the prologue when
  // there was no step); part 1 (d = 128) follows into bufB.
  float inv_l[QG];
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    const float lw = __shfl(accl[qg][0], l16);  // from lane group 0
    inv_l[qg] = lw > 0.f ? 1.0f / lw : 0.f;
    if (LSE && g == 0) {  // log2 of the softmax normaliser: P = exp2(s log2(e) / sqrt(d) - lse2)
      const int tq = 16 * (QG * wave + qg) + l16;
      const float meff = mref[qg] == -INFINITY ? 0.0f : mref[qg];
      lse_out[((size_t)bh * Nb + i) * kBlock + tq] =
          (lw > 0.f && i * kBlock + tq < N) ? meff + __log2f(lw) : INFINITY;
    }
  }
  if constexpr (HPARTS == 2) {
    lds_barrier();  // every wave is done with bufB
    issueH(1, bufB);
  }
  uint4 fq[QG][KSTEPS];
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    float qf[KSTEPS * 8];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const uint32_t w4[4] = {qr[qg][ks].x, qr[qg][ks].y, qr[qg][ks].z, qr[qg][ks].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qf[ks * 8 + 2 * e] = bf_lo(w4[e]);
        qf[ks * 8 + 2 * e + 1] = bf_hi(w4[e]);
      }
    }
    if constexpr (ELU) {  // phi = elu + 1, elementwise
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        uint32_t w4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) w4[e] = pack_bf2(elu1(qf[ks * 8 + 2 * e]), elu1(qf[ks * 8 + 2 * e + 1]));
        fq[qg][ks] = make_uint4(w4[0], w4[1], w4[2], w4[3]);
      }
    } else {
      float qm = -INFINITY;
#pragma unroll
      for (int e = 0; e < KSTEPS * 8; ++e) qm = fmaxf(qm, qf[e]);
      qm = group4_max(qm) * kLog2e;
      // e = exp(q - max q); phi(Q) = e / sum(e), but the sum cancels between the
      // numerator phi(Q) H_i and the denominator phi(Q) Z_i, so e enters both unscaled
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        uint32_t w4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          w4[e] = pack_bf2(__builtin_amdgcn_exp2f(fmaf(qf[ks * 8 + 2 * e], kLog2e, -qm)),
                           __builtin_amdgcn_exp2f(fmaf(qf[ks * 8 + 2 * e + 1], kLog2e, -qm)));
        fq[qg][ks] = make_uint4(w4[0], w4[1], w4[2], w4[3]);
      }
    }
  }
  // part 0 of H_i^T and Z_i have landed (part 1's copies, issued after them, may not)
  if constexpr (HPARTS == 2)
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(HINSTR));
  else
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  lds_barrier();
  // den: an A operand whose row 0 is Z_i gives phi(Q).Z_i in row 0 of the product
  float inv_den[QG];
  {
    f32x4 dacc[QG];
#pragma unroll
    for (int qg = 0; qg < QG; ++qg) dacc[qg] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const uint4 z = *reinterpret_cast<const uint4*>(zbuf + 32 * ks + 8 * g);
      const uint4 za = l16 == 0 ? z : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
      for (int qg = 0; qg < QG; ++qg) dacc[qg] = mfma_bf16(za, fq[qg][ks], dacc[qg]);
    }
#pragma unroll
    for (int qg = 0; qg < QG; ++qg) {
      const float den = __shfl(dacc[qg][0], l16);  // from lane group 0
      inv_den[qg] = den > 0.f ? 1.0f / den : 0.f;
    }
  }
  f32x4 nm[QG][FT];
  auto numpart = [&](auto PART, const uint16_t* hb) {
    constexpr int part = decltype(PART)::value;
#pragma unroll
    for (int f = 0; f < FT / HPARTS; ++f) {
      const int ft = part * (FT / HPARTS) + f;
#pragma unroll
      for (int qg = 0; qg < QG; ++qg) nm[qg][ft] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        const int hr = 16 * f + l16;  // row within the part
        const uint4 a = *reinterpret_cast<const uint4*>(hb + (hr * C + ((4 * ks + g) ^ row_swz<D>(hr))) * 8);
#pragma unroll
        for (int qg = 0; qg < QG; ++qg) nm[qg][ft] = mfma_bf16(a, fq[qg][ks], nm[qg][ft]);
      }
    }
  };
  numpart(std::integral_constant<int, 0>{}, bufA);
  if constexpr (HPARTS == 2) {
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    lds_barrier();
    numpart(std::integral_constant<int, 1>{}, bufB);
  }
  float cs[QG], cl[QG];
  if constexpr (PROJ) {
    // Proj(O_l) = O_l W. B operand: num^T rounded to bf16, its k slots the
    // features {4g..4g+3, 16+4g..16+4g+3} of each 32-feature step; A operand:
    // W^T in the same feature order (k_pack_proj), one fragment set per output
    // tile, the next tile's fragments in flight while the current one multiplies.
    uint4 nb[QG][KSTEPS];
#pragma unroll
    for (int qg = 0; qg < QG; ++qg)
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks)
        nb[qg][ks] = make_uint4(pack_bf2(nm[qg][2 * ks][0], nm[qg][2 * ks][1]),
                                pack_bf2(nm[qg][2 * ks][2], nm[qg][2 * ks][3]),
                                pack_bf2(nm[qg][2 * ks + 1][0], nm[qg][2 * ks + 1][1]),
                                pack_bf2(nm[qg][2 * ks + 1][2], nm[qg][2 * ks + 1][3]));
    const uint4* wf = reinterpret_cast<const uint4*>(wo + (size_t)h * wo_hs) + lane;
    uint4 wa[2][KSTEPS];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) wa[0][ks] = wf[ks * 64];
#pragma unroll
    for (int nt = 0; nt < FT; ++nt) {
      if (nt + 1 < FT) {
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) wa[(nt + 1) & 1][ks] = wf[((nt + 1) * KSTEPS + ks) * 64];
      }
#pragma unroll
      for (int qg = 0; qg < QG; ++qg) {
        nm[qg][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ++ks) nm[qg][nt] = mfma_bf16(wa[nt & 1][ks], nb[qg][ks], nm[qg][nt]);
      }
    }
#pragma unroll
    for (int qg = 0; qg < QG; ++qg) {
      cs[qg] = inv_l[qg];  // O = O_s + Proj(O_l)
      cl[qg] = inv_den[qg];
    }
  } else {
    const float al = alpha[h];
#pragma unroll
    for (int qg = 0; qg < QG; ++qg) {
      cs[qg] = al * inv_l[qg];
      cl[qg] = (1.0f - al) * inv_den[qg];
    }
  }
  lds_barrier();  // every wave has read H_i^T: the buffers become the output stage
  // the waves' 16 QG rows each, NW / 2 waves per buffer; each wave writes back its own rows
  constexpr int WPB = NW / 2;
  uint16_t* ost = ((wave / WPB) ? bufB : bufA) + (wave % WPB) * 16 * QG * OS;
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    const int t = i * kBlock + 16 * (QG * wave + qg) + l16;
    const bool dbg = (dbg_os || dbg_ol) && t < N;
#pragma unroll
    for (int ft = 0; ft < FT; ++ft) {
      float o[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) o[r] = fmaf(acc[qg][ft][r], cs[qg], nm[qg][ft][r] * cl[qg]);
      *reinterpret_cast<uint2*>(ost + (16 * qg + l16) * OS + 16 * ft + 4 * g) =
          make_uint2(pack_bf2(o[0], o[1]), pack_bf2(o[2], o[3]));
      if (dbg) {
        const size_t off = ((size_t)bh * N + t) * D + 16 * ft + 4 * g;
        const float il = inv_l[qg], id_ = inv_den[qg];
        if (dbg_os)
          *reinterpret_cast<float4*>(dbg_os + off) =
              make_float4(acc[qg][ft][0] * il, acc[qg][ft][1] * il, acc[qg][ft][2] * il, acc[qg][ft][3] * il);
        if (dbg_ol)
          *reinterpret_cast<float4*>(dbg_ol + off) =
              make_float4(nm[qg][ft][0] * id_, nm[qg][ft][1] * id_, nm[qg][ft][2] * id_, nm[qg][ft][3] * id_);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);  // a wave reads back only its own rows
  // full-row 16-byte stores of the wave's staged rows
  const int nrow = O ? min(16 * QG, N - (i * kBlock + 16 * QG * wave)) : 0;
  uint16_t* Ob = O + ((size_t)bh * N + (size_t)i * kBlock + 16 * QG * wave) * D;
#pragma unroll
  for (int x0 = 0; x0 < 16 * QG * C; x0 += 64) {
    const int x = x0 + lane;
    const int row = x / C, ch = x % C;
    if (row < nrow)
      *reinterpret_cast<uint4*>(Ob + (size_t)row * D + ch * 8) =
          *reinterpret_cast<const uint4*>(ost + row * OS + ch * 8);
  }
  if constexpr (LSE) {
    // O_s of the same rows as hi = bf16(O_s) and lo = bf16(O_s - hi) (relative
    // error 2^-17), each plane through the same stage and stored as full rows (a
    // wave's LDS operations run in order, so each read above precedes the next writes)
    const int nr = min(16 * QG, N - (i * kBlock + 16 * QG * wave));
#pragma unroll
    for (int part = 0; part < 2; ++part) {
#pragma unroll
      for (int qg = 0; qg < QG; ++qg) {
        const float il = inv_l[qg];
#pragma unroll
        for (int ft = 0; ft < FT; ++ft) {
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float x = acc[qg][ft][r] * il;
            v[r] = part == 0 ? x : x - bf_lo(pack_bf2(x, 0.f));
          }
          *reinterpret_cast<uint2*>(ost + (16 * qg + l16) * OS + 16 * ft + 4 * g) =
              make_uint2(pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]));
        }
      }
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      uint16_t* Sb = (part == 0 ? os_out : os_lo) + ((size_t)bh * N + (size_t)i * kBlock + 16 * QG * wave) * D;
#pragma unroll
      for (int x0 = 0; x0 < 16 * QG * C; x0 += 64) {
        const int x = x0 + lane;
        const int row = x / C, ch = x % C;
        if (row < nr)
          *reinterpret_cast<uint4*>(Sb + (size_t)row * D + ch * 8) =
              *reinterpret_cast<const uint4*>(ost + row * OS + ch * 8);
      }
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
                                                    const float* __restrict__ proj_o,
                                                    int proj_hs, int elu,
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
  // linear branch: phi(q) (softmax over the features, or elu + 1 elementwise)
  float f[P];
  if (elu) {
#pragma unroll
    for (int e = 0; e < P; ++e) f[e] = q[e] > 0.f ? q[e] + 1.0f : expf(q[e]);
  } else {
    float qm = -INFINITY;
#pragma unroll
    for (int e = 0; e < P; ++e) qm = fmaxf(qm, q[e]);
    qm = fmaxf(qm, __shfl_xor(qm, 1));
    qm = fmaxf(qm, __shfl_xor(qm, 2));
    float fs = 0.f;
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
  }
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
  if (proj_o) {  // uniform: SLA fusion, num <- num W (the division by den commutes with it)
    const float* W = proj_o + (size_t)h * proj_hs;
    float pr[P];
#pragma unroll
    for (int e = 0; e < P; ++e) pr[e] = 0.f;
    for (int r = 0; r < D; ++r) {
      const int src = (lane & ~3) | (r / P);
      float nr = 0.f;
#pragma unroll
      for (int e = 0; e < P; ++e)
        if (e == r % P) nr = num[e];
      nr = __shfl(nr, src);
#pragma unroll
      for (int e = 0; e < P; ++e) pr[e] = fmaf(nr, W[(size_t)r * D + part * P + e], pr[e]);
    }
#pragma unroll
    for (int e = 0; e < P; ++e) num[e] = pr[e];
  }
  if (!valid) return;
  const float inv_l = (ncrit > 0 && l > 0.f) ? 1.0f / l : 0.f;
  const float inv_den = den > 0.f ? 1.0f / den : 0.f;
  const float al = proj_o ? 1.0f : alpha[h];
  const float bl = proj_o ? 1.0f : 1.0f - al;
  const size_t orow = ((size_t)bh * N + t) * D + part * P;
#pragma unroll
  for (int e = 0; e < P; ++e) {
    const float os = acc[e] * inv_l, ol = num[e] * inv_den;
    O[orow + e] = al * os + bl * ol;
    if (dbg_os) dbg_os[orow + e] = os;
    if (dbg_ol) dbg_ol[orow + e] = ol;
  }
}

// The SLA output map W ([in][out] float32, one [D][D] matrix per workgroup)
// as bf16 A-operand fragments of the epilogue product (num W)^T = W^T num^T:
// entry ((nt * D/32 + ks) * 64 + lane) holds, for output feature
// n = 16 nt + lane % 16 and g = lane / 16, the 8 values W[c][n] with
// c = 32 ks + 16 (j / 4) + 4 g + j % 4, j = 0..7 (the k-slot order of num^T).
template <int D>
__global__ __launch_bounds__(256) void k_pack_proj(const float* __restrict__ W,
                                                   uint16_t* __restrict__ wo) {
  constexpr int FT = D / 16, KS = D / 32;
  const float* Wh = W + (size_t)blockIdx.x * D * D;
  uint4* out = reinterpret_cast<uint4*>(wo + (size_t)blockIdx.x * D * D);
  for (int x = threadIdx.x; x < FT * KS * 64; x += 256) {
    const int lane = x & 63, ks = (x >> 6) % KS, nt = (x >> 6) / KS;
    const int n = 16 * nt + (lane & 15), g = lane >> 4;
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = Wh[(size_t)(32 * ks + 16 * (j >> 2) + 4 * g + (j & 3)) * D + n];
    out[x] = make_uint4(pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]), pack_bf2(v[4], v[5]),
                        pack_bf2(v[6], v[7]));
  }
}

// waves per workgroup of the bf16 sparse kernel (2: two 16-query groups per
// wave; 4: one); SLA_SPARSE_WAVES in the environment overrides it for timing
int sparse_waves() {
  static int nw = [] {
    const char* e = getenv("SLA_SPARSE_WAVES");
    return (e && atoi(e) == 4) ? 4 : 2;
  }();
  return nw;
}

template <int D, int NW, bool PROJ, bool ELU>
hipError_t launch_bf16(const Dims& D_, const void* Q, const void* K, const void* V, const int8_t* mask,
                       const float* alpha, const Work& w, void* O, float* dbg_os, float* dbg_ol,
                       float* lse_out, uint16_t* os_out, hipStream_t s) {
  // dynamic LDS: the critical list (2 Nb bytes), later Z_i (2 D bytes)
  const size_t lbytes = ((size_t)2 * (D_.Nb > D ? D_.Nb : D) + 15) / 16 * 16;
  if constexpr (!PROJ || NW == 2) {  // the SLA fusion's saving forward: two-wave layout only
    if (lse_out) {
      if (!os_out) return hipErrorInvalidValue;
      hipLaunchKernelGGL((k_sparse_bf16<D, NW, PROJ, ELU, true>), dim3(D_.BH * D_.Nb), dim3(64 * NW), lbytes, s,
                         (const uint16_t*)Q, (const uint16_t*)K, (const uint16_t*)V, mask, (const uint16_t*)w.Hx,
                         alpha, w.wo, D_.proj_hs, (uint16_t*)O, dbg_os, dbg_ol, lse_out, os_out,
                         os_out + (size_t)D_.BH * D_.N * D, D_.H, D_.N, D_.Nb);
      return hipGetLastError();
    }
  }
  if (lse_out || os_out) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_sparse_bf16<D, NW, PROJ, ELU, false>), dim3(D_.BH * D_.Nb), dim3(64 * NW), lbytes, s,
                     (const uint16_t*)Q, (const uint16_t*)K, (const uint16_t*)V, mask, (const uint16_t*)w.Hx, alpha,
                     w.wo, D_.proj_hs, (uint16_t*)O, dbg_os, dbg_ol, nullptr, nullptr, nullptr, D_.H, D_.N, D_.Nb);
  return hipGetLastError();
}

template <int D, int NW>
hipError_t launch_bf16_nw(const Dims& D_, const void* Q, const void* K, const void* V, const int8_t* mask,
                          const float* alpha, bool proj, const Work& w, void* O, float* dbg_os,
                          float* dbg_ol, float* lse_out, uint16_t* os_out, hipStream_t s) {
  if (proj)
    return D_.elu ? launch_bf16<D, NW, true, true>(D_, Q, K, V, mask, alpha, w, O, dbg_os, dbg_ol, lse_out, os_out, s)
                  : launch_bf16<D, NW, true, false>(D_, Q, K, V, mask, alpha, w, O, dbg_os, dbg_ol, lse_out, os_out, s);
  return D_.elu ? launch_bf16<D, NW, false, true>(D_, Q, K, V, mask, alpha, w, O, dbg_os, dbg_ol, lse_out, os_out, s)
                : launch_bf16<D, NW, false, false>(D_, Q, K, V, mask, alpha, w, O, dbg_os, dbg_ol, lse_out, os_out, s);
}

template <int D>
hipError_t launch_bf16_d(const Dims& D_, const void* Q, const void* K, const void* V, const int8_t* mask,
                         const float* alpha, bool proj, const Work& w, void* O, float* dbg_os,
                         float* dbg_ol, float* lse_out, uint16_t* os_out, hipStream_t s) {
  if (sparse_waves() == 4)
    return launch_bf16_nw<D, 4>(D_, Q, K, V, mask, alpha, proj, w, O, dbg_os, dbg_ol, lse_out, os_out, s);
  return launch_bf16_nw<D, 2>(D_, Q, K, V, mask, alpha, proj, w, O, dbg_os, dbg_ol, lse_out, os_out, s);
}

}  // namespace

hipError_t launch_pack_proj(const Dims& D, const float* proj_o, const Work& w, hipStream_t s) {
  if (!D.bf16 || !proj_o) return hipErrorInvalidValue;
  const int hs = D.proj_hs ? D.H : 1;
  if (D.d == 128)
    hipLaunchKernelGGL(k_pack_proj<128>, dim3(hs), dim3(256), 0, s, proj_o, w.wo);
  else
    hipLaunchKernelGGL(k_pack_proj<64>, dim3(hs), dim3(256), 0, s, proj_o, w.wo);
  return hipGetLastError();
}

hipError_t launch_sparse(const Dims& D, const void* Q, const void* K, const void* V, const int8_t* mask,
                         const float* alpha, const float* proj_o, const Work& w, void* O,
                         float* dbg_os, float* dbg_ol, hipStream_t s, float* lse_out, uint16_t* os_out) {
  if (!D.bf16) return hipErrorInvalidValue;
  if (D.d == 128)
    return launch_bf16_d<128>(D, Q, K, V, mask, alpha, proj_o != nullptr, w, O, dbg_os, dbg_ol, lse_out, os_out, s);
  return launch_bf16_d<64>(D, Q, K, V, mask, alpha, proj_o != nullptr, w, O, dbg_os, dbg_ol, lse_out, os_out, s);
}

hipError_t launch_sparse_f32(const Dims& D, const void* Q, const void* K, const void* V,
                             const int8_t* mask, const float* alpha, const float* proj_o,
                             const Work& w, void* O, float* dbg_os, float* dbg_ol, hipStream_t s) {
  dim3 grid(D.Nb, D.BH);
  const int elu = D.elu ? 1 : 0;
  if (D.d == 128)
    hipLaunchKernelGGL(k_sparse_f32<128>, grid, dim3(256), 0, s, (const float*)Q,
                       (const float*)K, (const float*)V, mask, (const float*)w.Hx, alpha, proj_o,
                       D.proj_hs, elu, (float*)O, dbg_os, dbg_ol, D.H, D.N, D.Nb);
  else
    hipLaunchKernelGGL(k_sparse_f32<64>, grid, dim3(256), 0, s, (const float*)Q,
                       (const float*)K, (const float*)V, mask, (const float*)w.Hx, alpha, proj_o,
                       D.proj_hs, elu, (float*)O, dbg_os, dbg_ol, D.H, D.N, D.Nb);
  return hipGetLastError();
}

}  // namespace sla
