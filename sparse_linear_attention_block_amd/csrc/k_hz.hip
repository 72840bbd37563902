// K3: per-key-block linear-attention state.
//
// SLA explainer (intelliparadigm.com), section 1.2 "key implementation trick":
// h_j = phi(K_j)^T V_j (d x d) and z_j = rowsum(phi(K_j)^T) (d) are formed once
// per key block so that a query block only has to add them up (SLA paper
// summary, Eq. 3). phi is the softmax over the d features of each key token
// (SLA explainer, section 3.2; SLA paper summary, Table 2), or elu + 1 taken
// elementwise (Eq. 3's symbol list; Table 2's "SLA (elu+1)" row).
//
// bf16 path, one workgroup (8 waves for d = 128, 4 for d = 64) per 2
// consecutive key blocks of one (batch, head), two workgroups per CU:
//  1. each block's K and V rows stream in with 16-byte loads (two tokens per
//     lane), phi(K) is formed in float32 (row max / sum through LDS) and
//     rounded to bf16, and phi(K)^T and V^T are written to LDS with the
//     token index contiguous, two tokens per 32-bit word;
//  2. MFMA 16x16x32 (bf16 in, f32 accumulate) forms h_j^T[c][r] =
//     sum_t V[t][c] phi(K)[t][r] for the 2 blocks at once, so every lane holds
//     the same (c, r) of both and writes them as one 4-byte word, one half of
//     the 8-byte word of the output layout hx[bh][j/4][c*d + r][j%4] (the
//     linear-branch GEMM's k operand, 4 consecutive key blocks, contiguous);
//     the workgroups of the two halves run on one XCD, so the halves meet in
//     its L2;
//  3. z_j[r] (from the same bf16 phi values) goes to column d*d + r.
//  (A V^T copy for the sparse kernel can still be written through `vt`; the
//  bf16 sparse kernel now reads the V rows themselves, so it is passed NULL.)
// Tokens past N and blocks past Nb are zero in LDS, so they add nothing.
// 8-bit sparse branch: from the K rows already in registers the same pass forms
// K - mean(K), its int8 codes with one absmax scale per block and the per-key
// bias mean(Q).(K - mean(K)) (see k_quant.hip for the smoothing), and V^T in
// e4m3 with one absmax scale per block; the block maxima and the bias sums
// share the first phase's barriers, so the 8-bit outputs cost no extra pass
// over K.
//
// f32 path: one workgroup per key block, plain FMA loops, hx[bh][j][c*d + r].
#include "sla_internal.h"
#include "dev_common.h"

namespace sla {
namespace {

template <int D>
struct HzCfg {
  static constexpr int NT = D == 128 ? 512 : 256;  // threads per workgroup
  static constexpr int NW = NT / 64;               // waves
  static constexpr int NCG = NT / 32;              // chunk groups (32 token pairs each)
  static constexpr int TS = 72;            // LDS row stride in tokens (144 B, 16-B aligned)
  static constexpr int CHUNKS = D / 8;     // 16-byte chunks per token row
  static constexpr int CPT = CHUNKS / NCG; // chunks per thread
  static constexpr int NN = D * D + D;
};
constexpr int JB = 2;  // key blocks per workgroup: half of a group of 4

template <int D>
__device__ __forceinline__ float kBiasScale() {
  return 1.4426950408889634f / (D == 128 ? 11.313708498984761f : 8.0f);
}

template <int D>
__global__ __launch_bounds__(HzCfg<D>::NT, 2) void k_hz_bf16(const uint16_t* __restrict__ K,
                                                 const uint16_t* __restrict__ V,
                                                 uint16_t* __restrict__ hx,
                                                 uint16_t* __restrict__ vt, int N, int Nb,
                                                 int Nb4, uint8_t* __restrict__ v8t,
                                                 float* __restrict__ vsc,
                                                 const float* __restrict__ qkmean,
                                                 int8_t* __restrict__ k8, float* __restrict__ ksc,
                                                 float* __restrict__ kb, int BH, int elu) {
  using C = HzCfg<D>;
  constexpr int TS = C::TS, CPT = C::CPT, NN = C::NN, NT = C::NT, NW = C::NW, NCG = C::NCG;
  __shared__ __attribute__((aligned(16))) uint16_t kT[JB][D][TS];
  __shared__ __attribute__((aligned(16))) uint16_t vT[JB][D][TS];
  __shared__ float red[NCG][64];
  __shared__ float tstat[64];
  // 8-bit sparse branch only: the wave maxima of |K - mean(K)| and of |V|
  __shared__ float kam[NW];
  __shared__ float vmax[JB][NW];
  const bool quant = v8t != nullptr;  // uniform

  const int tid = threadIdx.x;
  // workgroups remapped so that the two halves of a group of 4 key blocks run
  // on one XCD: their 4-byte halves of each 8-byte hx word meet in its L2
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = id / (2 * Nb4);
  const int jq = (id >> 1) % Nb4;   // group of 4 key blocks
  const int half = id & 1;          // this workgroup's blocks: 4 jq + 2 half + jj, jj < JB
  const int tp = tid & 31;          // token pair
  const int cg = tid >> 5;          // chunk group
  const uint16_t* Kb = K + (size_t)bh * N * D;
  const uint16_t* Vb = V + (size_t)bh * N * D;

  // K and V rows of block jj+1 are loaded while block jj is processed
  uint4 kr[2][2][CPT], vr[2][2][CPT];  // [register set][token of the pair][chunk]
  bool valid[2][2];
  auto load_block = [&](int jj, int set) {
    const int j = 4 * jq + JB * half + jj;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int t = j * kBlock + 2 * tp + u;
      valid[set][u] = (j < Nb) && (t < N);
#pragma unroll
      for (int q = 0; q < CPT; ++q) {
        const int ch = cg * CPT + q;
        if (valid[set][u]) {
          kr[set][u][q] = *reinterpret_cast<const uint4*>(Kb + (size_t)t * D + ch * 8);
          vr[set][u][q] = *reinterpret_cast<const uint4*>(Vb + (size_t)t * D + ch * 8);
        } else {
          kr[set][u][q] = make_uint4(0, 0, 0, 0);
          vr[set][u][q] = make_uint4(0, 0, 0, 0);
        }
      }
    }
  };
  load_block(0, 0);
#pragma unroll
  for (int jj = 0; jj < JB; ++jj) {
    const int cs = jj & 1;
    if (jj + 1 < JB) load_block(jj + 1, cs ^ 1);
    // phi(K) row statistics: max then sum of exp over the D features
    float x[2][CPT * 8];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int q = 0; q < CPT; ++q) {
        const uint32_t w[4] = {kr[cs][u][q].x, kr[cs][u][q].y, kr[cs][u][q].z, kr[cs][u][q].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[u][q * 8 + 2 * e] = bf_lo(w[e]);
          x[u][q * 8 + 2 * e + 1] = bf_hi(w[e]);
        }
      }
    // row maxima: lanes l and l + 32 of a wave hold the same two tokens (chunk
    // groups 2w, 2w + 1), so one exchange leaves one partial per wave in red[w]
    const int wv = tid >> 6;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      float m = -INFINITY;
#pragma unroll
      for (int e = 0; e < CPT * 8; ++e) m = fmaxf(m, x[u][e]);
      m = fmaxf(m, __shfl_xor(m, 32));
      if ((tid & 32) == 0) red[wv][2 * tp + u] = m;
    }
    const int j = 4 * jq + JB * half + jj;
    // 8-bit sparse branch: K - mean(K) of the thread's two tokens, their bias
    // partials mean(Q).(k - mean(K)) over its features, and |K - mean(K)|, |V|
    // maxima (the block absmax scales), all at the barrier that follows
    float ks[2][CPT * 8];
    if (quant) {
      const float* qm = qkmean + (size_t)bh * D;
      const float* km = qkmean + ((size_t)BH + bh) * D;
      float bsum[2] = {0.f, 0.f};
      float am = 0.f, av = 0.f;
#pragma unroll
      for (int q = 0; q < CPT; ++q) {
        const int f0 = (cg * CPT + q) * 8;
        const float4 k0 = *reinterpret_cast<const float4*>(km + f0);
        const float4 k1 = *reinterpret_cast<const float4*>(km + f0 + 4);
        const float4 q0 = *reinterpret_cast<const float4*>(qm + f0);
        const float4 q1 = *reinterpret_cast<const float4*>(qm + f0 + 4);
        const float kmv[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
        const float qmv[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const uint32_t vw[4] = {vr[cs][u][q].x, vr[cs][u][q].y, vr[cs][u][q].z, vr[cs][u][q].w};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float kx = valid[cs][u] ? x[u][q * 8 + e] - kmv[e] : 0.f;
            ks[u][q * 8 + e] = kx;
            bsum[u] = fmaf(qmv[e], kx, bsum[u]);
            am = fmaxf(am, fabsf(kx));
            av = fmaxf(av, fabsf((e & 1) ? bf_hi(vw[e >> 1]) : bf_lo(vw[e >> 1])));
          }
        }
      }
      // bias partials, one per wave after the same exchange, in red[NW + w]
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const float b = bsum[u] + __shfl_xor(bsum[u], 32);
        if ((tid & 32) == 0) red[NW + wv][2 * tp + u] = b;
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        am = fmaxf(am, __shfl_xor(am, o));
        av = fmaxf(av, __shfl_xor(av, o));
      }
      if ((tid & 63) == 0) {
        kam[tid >> 6] = am;
        vmax[jj][tid >> 6] = av;
      }
    }
    __syncthreads();
    if (tid < 64) {
      float m = red[0][tid];
#pragma unroll
      for (int g = 1; g < NW; ++g) m = fmaxf(m, red[g][tid]);
      tstat[tid] = m;
      if (quant && j < Nb) {
        // the key bias, stored in the sparse kernel's log2 score units; 0 past N
        float b = 0.f;
#pragma unroll
        for (int g = 0; g < NW; ++g) b += red[NW + g][tid];
        kb[((size_t)bh * Nb + j) * kBlock + tid] = j * kBlock + tid < N ? b * kBiasScale<D>() : 0.f;
      }
    }
    if (quant && j < Nb) {
      // int8 codes of K - mean(K) with the block's absmax scale (absmax / 127; 1
      // for an all-zero block), round-half-even, clamped to +-127; rows past N
      // are zero. The bytes of a row go in the k-slot order of the sparse
      // kernel's int8 16x16x64 product: chunk ch = qt + 4m (features 8ch .. +7)
      // at 64 (m / 2) + 16 qt + 8 (m % 2).
      float amk = kam[0];
#pragma unroll
      for (int w = 1; w < NW; ++w) amk = fmaxf(amk, kam[w]);
      const float inv = amk > 0.f ? 127.0f / amk : 1.0f;
      if (tid == 0) ksc[(size_t)bh * Nb + j] = amk > 0.f ? amk / 127.0f : 1.0f;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        int8_t* dst = k8 + (((size_t)bh * Nb + j) * kBlock + 2 * tp + u) * D;
#pragma unroll
        for (int q = 0; q < CPT; ++q) {
          const int ch = cg * CPT + q, qt = ch & 3, m = ch >> 2;
          uint32_t o[2];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const float* v4 = &ks[u][q * 8 + 4 * hh];
            o[hh] = (uint32_t)(q_i8(v4[0], inv) & 0xff) | ((uint32_t)(q_i8(v4[1], inv) & 0xff) << 8) |
                    ((uint32_t)(q_i8(v4[2], inv) & 0xff) << 16) | ((uint32_t)(q_i8(v4[3], inv) & 0xff) << 24);
          }
          *reinterpret_cast<uint2*>(dst + 64 * (m >> 1) + 16 * qt + 8 * (m & 1)) = make_uint2(o[0], o[1]);
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const float m = tstat[2 * tp + u];
      float s = 0.f;
      if (elu) {  // uniform
#pragma unroll
        for (int e = 0; e < CPT * 8; ++e) x[u][e] = elu1(x[u][e]);
      } else {
#pragma unroll
        for (int e = 0; e < CPT * 8; ++e) {
          x[u][e] = __expf(x[u][e] - m);
          s += x[u][e];
        }
      }
      red[cg][2 * tp + u] = s;
    }
    __syncthreads();
    if (tid < 64) {
      float s = 0.f;
#pragma unroll
      for (int g = 0; g < NCG; ++g) s += red[g][tid];
      tstat[tid] = 1.0f / s;
    }
    __syncthreads();
    // the softmax is normalised per token; elu + 1 is not
    const float inv0 = valid[cs][0] ? (elu ? 1.0f : tstat[2 * tp]) : 0.f;
    const float inv1 = valid[cs][1] ? (elu ? 1.0f : tstat[2 * tp + 1]) : 0.f;
    // transposed stores: word (token 2tp, token 2tp+1) of each feature
#pragma unroll
    for (int q = 0; q < CPT; ++q) {
      const int f0 = (cg * CPT + q) * 8;
      const uint32_t v0[4] = {vr[cs][0][q].x, vr[cs][0][q].y, vr[cs][0][q].z, vr[cs][0][q].w};
      const uint32_t v1[4] = {vr[cs][1][q].x, vr[cs][1][q].y, vr[cs][1][q].z, vr[cs][1][q].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t kw = pack_bf2(x[0][q * 8 + e] * inv0, x[1][q * 8 + e] * inv1);
        *reinterpret_cast<uint32_t*>(&kT[jj][f0 + e][2 * tp]) = kw;
        const uint32_t a = (e & 1) ? (v0[e >> 1] >> 16) : (v0[e >> 1] & 0xffffu);
        const uint32_t b = (e & 1) ? (v1[e >> 1] >> 16) : (v1[e >> 1] & 0xffffu);
        *reinterpret_cast<uint32_t*>(&vT[jj][f0 + e][2 * tp]) = a | (b << 16);
      }
    }
    // red/tstat are reused by the next block only after this barrier
    __syncthreads();
  }

  // ---- h_j^T[c][r] for the 4 blocks, MFMA 16x16x32
  const int lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  constexpr int CT = D / 16;            // c tiles
  constexpr int CT_PER_WAVE = CT / NW;  // 1 (D=128, 8 waves; D=64, 4 waves)
  uint16_t* hxg = hx + ((size_t)bh * Nb4 + jq) * NN * 4;
  for (int cti = 0; cti < CT_PER_WAVE; ++cti) {
    const int ct = wave * CT_PER_WAVE + cti;
    uint4 a[JB][2];
#pragma unroll
    for (int jj = 0; jj < JB; ++jj)
#pragma unroll
      for (int u = 0; u < 2; ++u)
        a[jj][u] = *reinterpret_cast<const uint4*>(&vT[jj][16 * ct + l16][32 * u + 8 * g]);
    for (int rh = 0; rh < D / 64; ++rh) {
      f32x4 acc[4][JB];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int jj = 0; jj < JB; ++jj) acc[rt][jj] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const int r = 16 * (4 * rh + rt) + l16;
#pragma unroll
        for (int jj = 0; jj < JB; ++jj)
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const uint4 b = *reinterpret_cast<const uint4*>(&kT[jj][r][32 * u + 8 * g]);
            acc[rt][jj] = mfma_bf16(a[jj][u], b, acc[rt][jj]);
          }
      }
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const int r = 16 * (4 * rh + rt) + l16;
#pragma unroll
        for (int reg = 0; reg < 4; ++reg) {
          const int c = 16 * ct + 4 * g + reg;
          *reinterpret_cast<uint32_t*>(hxg + ((size_t)c * D + r) * 4 + JB * half) =
              pack_bf2(acc[rt][0][reg], acc[rt][1][reg]);
        }
      }
    }
  }
  // ---- z_j[r] = sum_t phi(K)[t][r] over the same bf16 values
  if (tid < D) {
    float z[JB];
#pragma unroll
    for (int jj = 0; jj < JB; ++jj) {
      float s = 0.f;
#pragma unroll
      for (int t8 = 0; t8 < 8; ++t8) {
        const uint4 w = *reinterpret_cast<const uint4*>(&kT[jj][tid][8 * t8]);
        s += bf_lo(w.x) + bf_hi(w.x) + bf_lo(w.y) + bf_hi(w.y) + bf_lo(w.z) + bf_hi(w.z) +
             bf_lo(w.w) + bf_hi(w.w);
      }
      z[jj] = s;
    }
    *reinterpret_cast<uint32_t*>(hxg + ((size_t)D * D + tid) * 4 + JB * half) = pack_bf2(z[0], z[1]);
  }
  // ---- V^T tiles for the sparse kernel, in the order its LDS copy wants:
  // vt[bh][j][kh][c][32] holds the 32 keys 32kh .. 32kh+31 of feature c as four
  // 16-byte chunks; chunk q carries keys {4q..4q+3, 16+4q..16+4q+3} (the k
  // slots of one MFMA lane group) and sits at position q ^ ((c >> 1) & 3), so
  // that 8 lanes reading 8 consecutive rows touch distinct LDS banks.
  // (the 8-bit sparse branch reads V8^T below instead: then vt is NULL)
  for (int jj = 0; jj < JB && vt != nullptr; ++jj) {
    const int j = 4 * jq + JB * half + jj;
    if (j >= Nb) break;
    uint16_t* dst = vt + ((size_t)bh * Nb + j) * D * kBlock;
    for (int x = tid; x < D * 8; x += NT) {
      const int khh = x / (D * 4), rem = x % (D * 4), c = rem >> 2, q = rem & 3;
      const uint2 lo = *reinterpret_cast<const uint2*>(&vT[jj][c][32 * khh + 4 * q]);
      const uint2 hi = *reinterpret_cast<const uint2*>(&vT[jj][c][32 * khh + 16 + 4 * q]);
      *reinterpret_cast<uint4*>(dst + ((size_t)khh * D + c) * 32 + 8 * (q ^ ((c >> 1) & 3))) =
          make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
  }
  if (v8t == nullptr) return;  // uniform: no 8-bit copy of V wanted
  // ---- 8-bit sparse branch: V^T of each block in OCP e4m3 with one absmax
  // scale per block (absmax / 448; an all-zero block gets scale 1). Row c of a
  // block holds four 16-byte chunks; chunk g carries keys 16kt + 4g + r in the
  // order (kt, r), the k slots one lane group of the 8-bit sparse kernel's
  // 16x16x128 product takes from one tile, and sits at position
  // g ^ ((c >> 1) & 3) against LDS bank conflicts.
  // (the block absmax of |V| was reduced in the first phase)
  const int cq = tid >> 2, gq = tid & 3;  // rows cq, cq + NT/4, ... of chunk gq
  float am[JB];
#pragma unroll
  for (int jj = 0; jj < JB; ++jj) {
    am[jj] = vmax[jj][0];
#pragma unroll
    for (int w = 1; w < NW; ++w) am[jj] = fmaxf(am[jj], vmax[jj][w]);
  }
#pragma unroll
  for (int jj = 0; jj < JB; ++jj) {
    const int j = 4 * jq + JB * half + jj;
    if (j >= Nb) break;
    const float inv = am[jj] > 0.f ? 448.0f / am[jj] : 1.0f;
    if (tid == 0) vsc[(size_t)bh * Nb + j] = am[jj] > 0.f ? am[jj] / 448.0f : 1.0f;
    uint8_t* dst = v8t + ((size_t)bh * Nb + j) * D * kBlock;
    for (int c = cq; c < D; c += NT / 4) {
      uint32_t o[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const uint2 w = *reinterpret_cast<const uint2*>(&vT[jj][c][16 * kt + 4 * gq]);
        o[kt] = pack_e4m3x4(bf_lo(w.x) * inv, bf_hi(w.x) * inv, bf_lo(w.y) * inv, bf_hi(w.y) * inv);
      }
      *reinterpret_cast<uint4*>(dst + (size_t)c * 64 + 16 * (gq ^ ((c >> 1) & 3))) =
          make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
}

// ---------------------------------------------------------------- f32 path
__global__ __launch_bounds__(256) void k_hz_f32(const float* __restrict__ K,
                                                const float* __restrict__ V,
                                                float* __restrict__ hx, int N, int d, int Nb,
                                                int elu) {
  extern __shared__ float sm[];
  float* phk = sm;               // [64][d]
  float* vs = sm + kBlock * d;   // [64][d]
  const int tid = threadIdx.x;
  const int bh = blockIdx.y, j = blockIdx.x;
  const int NN = d * d + d;
  const float* Kb = K + ((size_t)bh * N + (size_t)j * kBlock) * d;
  const float* Vb = V + ((size_t)bh * N + (size_t)j * kBlock) * d;
  const int nt = min(kBlock, N - j * kBlock);
  for (int x = tid; x < kBlock * d; x += 256) {
    const int t = x / d;
    phk[x] = t < nt ? Kb[x] : 0.f;
    vs[x] = t < nt ? Vb[x] : 0.f;
  }
  __syncthreads();
  if (tid < kBlock) {
    float* row = phk + tid * d;
    if (tid < nt && elu) {
      for (int c = 0; c < d; ++c) row[c] = row[c] > 0.f ? row[c] + 1.0f : expf(row[c]);
    } else if (tid < nt) {
      float m = -INFINITY;
      for (int c = 0; c < d; ++c) m = fmaxf(m, row[c]);
      float s = 0.f;
      for (int c = 0; c < d; ++c) {
        row[c] = expf(row[c] - m);
        s += row[c];
      }
      const float inv = 1.0f / s;
      for (int c = 0; c < d; ++c) row[c] *= inv;
    }
  }
  __syncthreads();
  float* out = hx + ((size_t)bh * Nb + j) * NN;
  for (int x = tid; x < d * d; x += 256) {
    const int c = x / d, r = x % d;
    float s = 0.f;
    for (int t = 0; t < kBlock; ++t) s = fmaf(vs[t * d + c], phk[t * d + r], s);
    out[x] = s;  // x = c*d + r
  }
  for (int r = tid; r < d; r += 256) {
    float s = 0.f;
    for (int t = 0; t < kBlock; ++t) s += phk[t * d + r];
    out[d * d + r] = s;
  }
}

}  // namespace

hipError_t launch_hz(const Dims& D, const void* K, const void* V, const Work& w, hipStream_t s) {
  if (D.bf16) {
    dim3 grid(D.Nbp / 4 * 2 * D.BH);
    if (D.d == 128)
      hipLaunchKernelGGL(k_hz_bf16<128>, grid, dim3(HzCfg<128>::NT), 0, s, (const uint16_t*)K,
                         (const uint16_t*)V, (uint16_t*)w.hx, nullptr, D.N, D.Nb, D.Nbp / 4,
                         D.quant ? w.v8t : nullptr, w.vs, w.qkmean, w.k8, w.ks, w.kb, D.BH, D.elu ? 1 : 0);
    else
      hipLaunchKernelGGL(k_hz_bf16<64>, grid, dim3(HzCfg<64>::NT), 0, s, (const uint16_t*)K,
                         (const uint16_t*)V, (uint16_t*)w.hx, nullptr, D.N, D.Nb, D.Nbp / 4,
                         D.quant ? w.v8t : nullptr, w.vs, w.qkmean, w.k8, w.ks, w.kb, D.BH, D.elu ? 1 : 0);
  } else {
    dim3 grid(D.Nb, D.BH);
    const size_t lds = 2 * kBlock * D.d * sizeof(float);
    hipLaunchKernelGGL(k_hz_f32, grid, dim3(256), lds, s, (const float*)K, (const float*)V,
                       (float*)w.hx, D.N, D.d, D.Nb, D.elu ? 1 : 0);
  }
  return hipGetLastError();
}

}  // namespace sla
