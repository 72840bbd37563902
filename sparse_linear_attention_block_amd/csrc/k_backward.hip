// Backward pass of SLA2 for a fixed block mask: dQ, dK, dV and dalpha of
// sum(O * dO), with O = alpha O_s + (1 - alpha) O_l.
//
// SLA explainer (intelliparadigm.com), section 2.3: the sparse path takes the
// FlashAttention backward over the blocks with Mc = 1 only, the linear path
// the chain rule through phi(Q), phi(K) and V with per-block accumulation.
// Written out, per head, with dO_s = alpha dO and dO_l = (1 - alpha) dO:
//  sparse (query t, its critical keys s; P = exp(S - lse_t), S = q.k / sqrt(d)):
//    D_t = dO_s[t] . O_s[t],  dS = P (dO_s[t] . v_s - D_t),
//    dq_t += sum_s dS k_s / sqrt(d),  dk_s += sum_t dS q_t / sqrt(d),
//    dv_s += sum_t P dO_s[t];
//  linear (query t in block i, u = phi(q_t), num = u H_i, den = u . Z_i):
//    dnum = dO_l[t] / den,  dden = -(dO_l[t] . O_l[t]) / den,
//    du = H_i dnum + Z_i dden,  dH_i += u^T dnum,  dZ_i += u dden;
//    dh_j = sum over query blocks i with Mc[i, j] = 0 of dH_i (dz_j likewise),
//    taken as the head's total minus the blocks with Mc != 0;
//    key s in block j, w = phi(k_s): dw = dh_j v_s + dz_j, dv_s += w dh_j;
//  feature map: softmax over the features, dx = phi (dphi - dphi . phi); or
//  elu + 1 elementwise, dx = dphi * (1 if x > 0 else exp(x));
//  dalpha_h = sum over the head of dO . (O_s - O_l).
// The SLA fusion O = O_s + O_l W (SLA paper summary, section 4, step 4):
// dO_s = dO, dO_l = dO W^T, and dW = sum over tokens of O_l^T dO, formed per
// query block (k_bwd_q) and summed in a fixed order (k_bwd_dw_part and
// k_bwd_dw_fin); no dalpha.
//
// fp32 arithmetic throughout (bf16 or f32 inputs), eight threads per query or
// key token, each holding d/8 features (with four, a thread's state filled
// 256 VGPRs and one wave ran per SIMD); a token's dot products are summed
// across its 8 lanes with DPP moves; the per-key exponentials use the
// hardware base-2 exponential (__expf, a few ulp). H_i and Z_i come from the forward's own h/z and marginal-sum
// kernels. k_bwd_q (one workgroup per query block) recomputes the sparse
// forward for its log-sum-exp and O_s, then produces dQ, dH_i / dZ_i and the
// block's dalpha partial; k_bwd_htot sums dH_i per head; k_bwd_kv (one
// workgroup per key block) produces dK and dV; k_bwd_alpha sums the partials
// per head in a fixed order.
#include "sla_internal.h"
#include "dev_common.h"

namespace sla {
namespace {

constexpr int kTpt = 8;              // threads per query / key token
constexpr int kThreads = kBlock * kTpt;  // one 64-token block per workgroup

template <typename T>
__device__ __forceinline__ float ldf(const T* p);
template <>
__device__ __forceinline__ float ldf<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float ldf<uint16_t>(const uint16_t* p) { return bf2f(*p); }

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}

// Sum and max over the kTpt = 8 threads of a token (8 consecutive lanes),
// with DPP moves instead of LDS permutes: partners at lane distance 1 and 2
// (quad permutations), then the other quad of the 8 (half-row mirror). Every
// step combines two values both partners hold, so all 8 lanes end with the
// same bits.
static_assert(kTpt == 8, "the DPP reductions span 8 lanes");
__device__ __forceinline__ float sum4(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v += dpp<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v += dpp<0x141>(v);  // row_half_mirror
  return v;
}
__device__ __forceinline__ float max4(float v) {
  v = fmaxf(v, dpp<0xB1>(v));
  v = fmaxf(v, dpp<0x4E>(v));
  v = fmaxf(v, dpp<0x141>(v));
  return v;
}

// value r of a token group's d features (thread k of the group holds
// features k P .. k P + P - 1 in x[])
template <int P>
__device__ __forceinline__ float group_get(const float (&x)[P], int r, int lane) {
  float v = 0.f;
#pragma unroll
  for (int e = 0; e < P; ++e)
    if (e == r % P) v = x[e];
  return __shfl(v, (lane & ~(kTpt - 1)) | (r / P));
}

// softmax over the d features held by a token group
template <int P>
__device__ __forceinline__ void feature_softmax(const float (&x)[P], float (&f)[P]) {
  float m = -INFINITY;
#pragma unroll
  for (int e = 0; e < P; ++e) m = fmaxf(m, x[e]);
  m = max4(m);
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < P; ++e) {
    f[e] = expf(x[e] - m);
    s += f[e];
  }
  const float inv = 1.0f / sum4(s);
#pragma unroll
  for (int e = 0; e < P; ++e) f[e] *= inv;
}

// elu + 1 of a thread's features and its derivative (1 above zero, exp(x) at or below)
template <int P>
__device__ __forceinline__ void feature_elu1(const float (&x)[P], float (&f)[P]) {
#pragma unroll
  for (int e = 0; e < P; ++e) f[e] = x[e] > 0.f ? x[e] + 1.0f : expf(x[e]);
}

// The block indices j of a mask row with mrow[j] == value, in ascending order,
// into list (for workgroups of kThreads); returns their number.
__device__ int compact_row_wg(const int8_t* __restrict__ mrow, int Nb, int8_t value, uint16_t* list,
                              int* wsum) {
  constexpr int NW = kThreads / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int total = 0;
  for (int base = 0; base < Nb; base += kThreads) {
    const int j = base + tid;
    const bool f = (j < Nb) && (mrow[j] == value);
    const uint64_t bal = __ballot(f);
    const int before = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wsum[wave] = __popcll(bal);
    __syncthreads();
    int off = total;
    for (int w = 0; w < wave; ++w) off += wsum[w];
    if (f) list[off + before] = (uint16_t)j;
    for (int w = 0; w < NW; ++w) total += wsum[w];
    __syncthreads();
  }
  return total;
}

// The 64 keys of block j (f32, zero past N) into Ks / Vs.
template <typename T, int D>
__device__ __forceinline__ void stage_kv(const T* Kb, const T* Vb, int j, int N, float (*Ks)[D],
                                         float (*Vs)[D]) {
  for (int x = threadIdx.x; x < kBlock * D; x += kThreads) {
    const int key = x / D, c = x % D, tk = j * kBlock + key;
    Ks[key][c] = tk < N ? ldf<T>(Kb + (size_t)tk * D + c) : 0.f;
    Vs[key][c] = tk < N ? ldf<T>(Vb + (size_t)tk * D + c) : 0.f;
  }
}

template <typename T, int D, bool ELU, bool PROJ>
__global__ __launch_bounds__(kThreads) void k_bwd_q(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const int8_t* __restrict__ mask, const T* __restrict__ Hx, const float* __restrict__ alpha,
    const float* __restrict__ proj_o, int proj_hs,
    const T* __restrict__ dO, float* __restrict__ dQ, float* __restrict__ lse_out,
    float* __restrict__ dt_out, float* __restrict__ dHx, float* __restrict__ dal, float* __restrict__ dWp,
    int H, int N, int Nb) {
  constexpr int P = D / kTpt;
  constexpr int NN = D * D + D;
  __shared__ float Ks[kBlock][D];  // key tiles; then phi(Q) of the block
  __shared__ float Vs[kBlock][D];  // value tiles; then dnum of the block
  __shared__ float dd[kBlock];     // dden of the block
  __shared__ uint16_t list[kMaxNb];
  __shared__ int wsum[kThreads / 64];
  __shared__ float red[kThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int bh = blockIdx.y, i = blockIdx.x, h = bh % H;
  const int row = tid / kTpt, part = tid % kTpt;
  const int t = i * kBlock + row;
  const bool valid = t < N;
  const size_t base = (size_t)bh * N * D;
  const int ncrit = compact_row_wg(mask + ((size_t)bh * Nb + i) * Nb, Nb, (int8_t)1, list, wsum);
  float q[P], g[P];
#pragma unroll
  for (int e = 0; e < P; ++e) {
    q[e] = valid ? ldf<T>(Q + base + (size_t)t * D + part * P + e) : 0.f;
    g[e] = valid ? ldf<T>(dO + base + (size_t)t * D + part * P + e) : 0.f;
  }
  const float al = PROJ ? 1.0f : alpha[h];  // the SLA fusion weighs O_s by 1
  const float scale = 1.0f / sqrtf((float)D);
  const T* Kb = K + base;
  const T* Vb = V + base;

  // sparse forward again: log-sum-exp and O_s of the query
  float m = -INFINITY, l = 0.f, acc[P];
#pragma unroll
  for (int e = 0; e < P; ++e) acc[e] = 0.f;
  for (int c = 0; c < ncrit; ++c) {
    const int j = list[c];
    __syncthreads();
    stage_kv<T, D>(Kb, Vb, j, N, Ks, Vs);
    __syncthreads();
    const int nk = min(kBlock, N - j * kBlock);
    for (int key = 0; key < nk; ++key) {
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < P; ++e) s = fmaf(q[e], Ks[key][part * P + e], s);
      s = sum4(s) * scale;
      const float mn = fmaxf(m, s);
      const float corr = __expf(m - mn), p = __expf(s - mn);
      l = l * corr + p;
#pragma unroll
      for (int e = 0; e < P; ++e) acc[e] = fmaf(p, Vs[key][part * P + e], acc[e] * corr);
      m = mn;
    }
  }
  const bool has_crit = ncrit > 0 && l > 0.f;
  const float inv_l = has_crit ? 1.0f / l : 0.f;
  const float lse = has_crit ? m + logf(l) : INFINITY;  // no critical key: every P is 0
  float os[P], gs[P];
  float dtp = 0.f;
#pragma unroll
  for (int e = 0; e < P; ++e) {
    os[e] = acc[e] * inv_l;
    gs[e] = al * g[e];
    dtp = fmaf(gs[e], os[e], dtp);
  }
  const float Dt = sum4(dtp);

  // sparse dq: dS = P (dO_s . v - D_t), dq += dS k / sqrt(d)
  float dq[P];
#pragma unroll
  for (int e = 0; e < P; ++e) dq[e] = 0.f;
  for (int c = 0; c < ncrit; ++c) {
    const int j = list[c];
    __syncthreads();
    stage_kv<T, D>(Kb, Vb, j, N, Ks, Vs);
    __syncthreads();
    const int nk = min(kBlock, N - j * kBlock);
    for (int key = 0; key < nk; ++key) {
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int e = 0; e < P; ++e) {
        s = fmaf(q[e], Ks[key][part * P + e], s);
        dp = fmaf(gs[e], Vs[key][part * P + e], dp);
      }
      s = sum4(s) * scale;
      dp = sum4(dp);
      const float ds = __expf(s - lse) * (dp - Dt) * scale;
#pragma unroll
      for (int e = 0; e < P; ++e) dq[e] = fmaf(ds, Ks[key][part * P + e], dq[e]);
    }
  }

  // linear branch: u = phi(q), num = u H_i, den = u . Z_i (H_i^T stored c-major: Hrow[n D + r] = H_i[r][n])
  const T* Hrow = Hx + ((size_t)bh * Nb + i) * NN;
  float u[P];
  if constexpr (ELU)
    feature_elu1<P>(q, u);
  else
    feature_softmax<P>(q, u);
  float den = 0.f;
#pragma unroll
  for (int e = 0; e < P; ++e) den = fmaf(u[e], ldf<T>(Hrow + D * D + part * P + e), den);
  den = sum4(den);
  float num[P];
#pragma unroll
  for (int e = 0; e < P; ++e) num[e] = 0.f;
  for (int r = 0; r < D; ++r) {
    const float ur = group_get<P>(u, r, lane);
#pragma unroll
    for (int e = 0; e < P; ++e) num[e] = fmaf(ur, ldf<T>(Hrow + (size_t)(part * P + e) * D + r), num[e]);
  }
  const float inv_den = den > 0.f ? 1.0f / den : 0.f;
  // dO_l: (1 - alpha) dO, or dO W^T for the SLA fusion (W [in][out]: dO_l[c] = sum_n W[c][n] dO[n])
  float gl[P];
  if constexpr (PROJ) {
    const float* W = proj_o + (size_t)h * proj_hs;
#pragma unroll
    for (int e = 0; e < P; ++e) gl[e] = 0.f;
    for (int n = 0; n < D; ++n) {
      const float gn = group_get<P>(g, n, lane);
#pragma unroll
      for (int e = 0; e < P; ++e) gl[e] = fmaf(W[(size_t)(part * P + e) * D + n], gn, gl[e]);
    }
  } else {
#pragma unroll
    for (int e = 0; e < P; ++e) gl[e] = (1.0f - al) * g[e];
  }
  float ol[P], dnum[P];
  float dop = 0.f, dap = 0.f;
#pragma unroll
  for (int e = 0; e < P; ++e) {
    ol[e] = num[e] * inv_den;
    dnum[e] = gl[e] * inv_den;
    dop = fmaf(gl[e], ol[e], dop);
    dap = fmaf(g[e], os[e] - ol[e], dap);
  }
  const float dden = -sum4(dop) * inv_den;
  // du[r] = sum_n H_i[r][n] dnum[n] + Z_i[r] dden, for the thread's features r
  float du[P];
#pragma unroll
  for (int e = 0; e < P; ++e) du[e] = ldf<T>(Hrow + D * D + part * P + e) * dden;
  for (int n = 0; n < D; ++n) {
    const float dn = group_get<P>(dnum, n, lane);
#pragma unroll
    for (int e = 0; e < P; ++e) du[e] = fmaf(ldf<T>(Hrow + (size_t)n * D + part * P + e), dn, du[e]);
  }
  if constexpr (ELU) {
#pragma unroll
    for (int e = 0; e < P; ++e) dq[e] = fmaf(du[e], q[e] > 0.f ? 1.0f : u[e], dq[e]);
  } else {
    float dup = 0.f;
#pragma unroll
    for (int e = 0; e < P; ++e) dup = fmaf(du[e], u[e], dup);
    dup = sum4(dup);
#pragma unroll
    for (int e = 0; e < P; ++e) dq[e] = fmaf(u[e], du[e] - dup, dq[e]);
  }

  if (valid) {
#pragma unroll
    for (int e = 0; e < P; ++e) dQ[base + (size_t)t * D + part * P + e] = dq[e];
  }
  const size_t tok = ((size_t)bh * Nb + i) * kBlock + row;
  if (part == 0) {
    lse_out[tok] = lse;
    dt_out[tok] = Dt;
  }

  // dalpha partial of the block (rows past N hold zeros)
  float da = valid ? dap : 0.f;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) da += __shfl_xor(da, o);
  __syncthreads();  // the key tiles are no longer needed
  if (lane == 0) red[tid >> 6] = da;
  // dH_i and dZ_i: phi(Q) and dnum of the block's queries (zero past N) in LDS
#pragma unroll
  for (int e = 0; e < P; ++e) {
    Ks[row][part * P + e] = valid ? u[e] : 0.f;
    Vs[row][part * P + e] = valid ? dnum[e] : 0.f;
  }
  if (part == 0) dd[row] = valid ? dden : 0.f;
  __syncthreads();
  if (!PROJ && tid == 0) {
    float sdal = 0.f;
    for (int wv = 0; wv < kThreads / 64; ++wv) sdal += red[wv];
    dal[(size_t)bh * Nb + i] = sdal;
  }
  float* out = dHx + ((size_t)bh * Nb + i) * NN;
  for (int x = tid; x < NN; x += kThreads) {
    float s = 0.f;
    if (x < D * D) {
      const int n = x / D, r = x % D;  // dH_i[r][n], stored like H_i
      for (int tq = 0; tq < kBlock; ++tq) s = fmaf(Ks[tq][r], Vs[tq][n], s);
    } else {
      const int r = x - D * D;
      for (int tq = 0; tq < kBlock; ++tq) s = fmaf(Ks[tq][r], dd[tq], s);
    }
    out[x] = s;
  }
  if constexpr (PROJ) {
    // the block's part of dW = O_l^T dO: O_l and dO of its queries (zero past N) in LDS
    __syncthreads();
#pragma unroll
    for (int e = 0; e < P; ++e) {
      Ks[row][part * P + e] = valid ? ol[e] : 0.f;
      Vs[row][part * P + e] = valid ? g[e] : 0.f;
    }
    __syncthreads();
    float* wout = dWp + ((size_t)bh * Nb + i) * D * D;
    for (int x = tid; x < D * D; x += kThreads) {
      const int c = x / D, n = x % D;  // dW[c][n], W indexed [in][out]
      float s = 0.f;
      for (int tq = 0; tq < kBlock; ++tq) s = fmaf(Ks[tq][c], Vs[tq][n], s);
      wout[x] = s;
    }
  }
}

// dW = sum of the parts, in float64 and a fixed order: the parts of each W
// (float32 inputs: one per query block, in the order (batch, head, query
// block), over the batches and blocks, and over the heads when W is shared;
// bf16 inputs: the dW product's row chunks, in row order) are cut into
// kDwSplit consecutive ranges; k_bwd_dw_part sums each range (a thread owns
// four consecutive entries of W, read as 16-byte words, eight parts' words in
// flight before they are added in part order; 1024 consecutive entries per
// workgroup, so every part is read as whole rows), k_bwd_dw_fin the kDwSplit
// range sums in range order.
template <int D>
__global__ __launch_bounds__(256) void k_bwd_dw_part(const float* __restrict__ dWp, double* __restrict__ dWs,
                                                     int B, int H, int Nb, int per_head, int chunks) {
  const int x = 4 * (blockIdx.x * 256 + threadIdx.x), r = blockIdx.y, hw = blockIdx.z;
  if (x >= D * D) return;
  // parts summed into this W: `chunks` contiguous ones (bf16), else the query blocks'
  const int P = chunks > 0 ? chunks : per_head ? B * Nb : B * H * Nb;
  const int per = (P + kDwSplit - 1) / kDwSplit;
  const int p0 = r * per, p1 = min(P, p0 + per);
  // part q: chunk q of W hw; or (batch, head, block) = (q / (H Nb), q / Nb % H, q % Nb)
  // for a shared W, (q / Nb, hw, q % Nb) for head hw's own
  auto part = [&](int q) -> size_t {
    if (chunks > 0) return (size_t)hw * chunks + q;
    return per_head ? ((size_t)(q / Nb) * H + hw) * Nb + q % Nb : (size_t)q;
  };
  double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
  constexpr int U = 8;
  for (int q0 = p0; q0 < p1; q0 += U) {
    float4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      v[u] = q0 + u < p1 ? *reinterpret_cast<const float4*>(dWp + part(q0 + u) * D * D + x)
                         : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (q0 + u < p1) {
        s0 += (double)v[u].x;
        s1 += (double)v[u].y;
        s2 += (double)v[u].z;
        s3 += (double)v[u].w;
      }
    }
  }
  double* out = dWs + ((size_t)hw * kDwSplit + r) * D * D + x;
  out[0] = s0;
  out[1] = s1;
  out[2] = s2;
  out[3] = s3;
}
template <int D>
__global__ __launch_bounds__(256) void k_bwd_dw_fin(const double* __restrict__ dWs, float* __restrict__ dW) {
  const int x = blockIdx.x * 256 + threadIdx.x, hw = blockIdx.y;
  if (x >= D * D) return;
  double s = 0.0;
  for (int r = 0; r < kDwSplit; ++r) s += dWs[((size_t)hw * kDwSplit + r) * D * D + x];
  dW[(size_t)hw * D * D + x] = (float)s;
}

template <int D>
hipError_t launch_dw(const Dims& Dm, const BwdWork& bw, const void* dO, float* dW, hipStream_t s) {
  const int hs = Dm.proj_hs ? Dm.H : 1;
  if (Dm.bf16) {  // the row-chunk parts of the dW product (k_backward_mfma.hip)
    const hipError_t e = launch_dw_mfma(Dm, bw, dO, s);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_bwd_dw_part<D>, dim3((D * D / 4 + 255) / 256, kDwSplit, hs), dim3(256), 0, s,
                     Dm.bf16 ? bw.dWg : bw.dWp, bw.dWs, Dm.B, Dm.H, Dm.Nb, Dm.proj_hs ? 1 : 0,
                     Dm.bf16 ? dw_chunks(hs) : 0);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_bwd_dw_fin<D>, dim3((D * D + 255) / 256, hs), dim3(256), 0, s, bw.dWs, dW);
  return hipGetLastError();
}

// dH_tot[bh][x] = sum over the head's query blocks of dHx[bh][i][x]
template <int D>
__global__ __launch_bounds__(256) void k_bwd_htot(const float* __restrict__ dHx, float* __restrict__ dHtot,
                                                  int Nb) {
  constexpr int NN = D * D + D;
  const int x = blockIdx.x * 256 + threadIdx.x, bh = blockIdx.y;
  if (x >= NN) return;
  double s = 0.0;
  for (int i = 0; i < Nb; ++i) s += (double)dHx[((size_t)bh * Nb + i) * NN + x];
  dHtot[(size_t)bh * NN + x] = (float)s;
}

template <typename T, int D, bool ELU>
__global__ __launch_bounds__(kThreads) void k_bwd_kv(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
    const int8_t* __restrict__ mask, const float* __restrict__ alpha, const T* __restrict__ dO,
    const float* __restrict__ lse_in, const float* __restrict__ dt_in, const float* __restrict__ dHx,
    const float* __restrict__ dHtot, float* __restrict__ dK, float* __restrict__ dV, int H, int N,
    int Nb) {
  constexpr int P = D / kTpt;
  constexpr int NN = D * D + D;
  __shared__ float sm[NN > 2 * kBlock * D + 2 * kBlock ? NN : 2 * kBlock * D + 2 * kBlock];
  const int tid = threadIdx.x, lane = tid & 63;
  const int bh = blockIdx.y, j = blockIdx.x, h = bh % H;
  const int row = tid / kTpt, part = tid % kTpt;
  const int s = j * kBlock + row;
  const bool valid = s < N;
  const size_t base = (size_t)bh * N * D;
  float kk[P], vv[P];
#pragma unroll
  for (int e = 0; e < P; ++e) {
    kk[e] = valid ? ldf<T>(K + base + (size_t)s * D + part * P + e) : 0.f;
    vv[e] = valid ? ldf<T>(V + base + (size_t)s * D + part * P + e) : 0.f;
  }
  const float al = alpha ? alpha[h] : 1.0f;  // the SLA fusion (no alpha) weighs O_s by 1
  const float scale = 1.0f / sqrtf((float)D);
  float dk[P], dv[P];
#pragma unroll
  for (int e = 0; e < P; ++e) dk[e] = dv[e] = 0.f;

  // linear branch: dh_j = dH_tot - sum of dH_i over the query blocks with Mc[i, j] != 0
  float* DH = sm;  // [NN]: dh_j stored like H (DH[n D + r] = dh_j[r][n]), then dz_j
  for (int x = tid; x < NN; x += kThreads) DH[x] = dHtot[(size_t)bh * NN + x];
  for (int i = 0; i < Nb; ++i) {
    if (mask[((size_t)bh * Nb + i) * Nb + j] == 0) continue;  // uniform
    const float* src = dHx + ((size_t)bh * Nb + i) * NN;
    for (int x = tid; x < NN; x += kThreads) DH[x] -= src[x];  // each thread owns its x
  }
  __syncthreads();
  float w[P];
  if constexpr (ELU)
    feature_elu1<P>(kk, w);
  else
    feature_softmax<P>(kk, w);
  // dw[r] = sum_n dh_j[r][n] v[n] + dz_j[r]; dv[n] += sum_r w[r] dh_j[r][n]
  float dw[P];
#pragma unroll
  for (int e = 0; e < P; ++e) dw[e] = DH[D * D + part * P + e];
  for (int n = 0; n < D; ++n) {
    const float vn = group_get<P>(vv, n, lane);
#pragma unroll
    for (int e = 0; e < P; ++e) dw[e] = fmaf(DH[n * D + part * P + e], vn, dw[e]);
  }
  for (int r = 0; r < D; ++r) {
    const float wr = group_get<P>(w, r, lane);
#pragma unroll
    for (int e = 0; e < P; ++e) dv[e] = fmaf(wr, DH[(part * P + e) * D + r], dv[e]);
  }
  if constexpr (ELU) {
#pragma unroll
    for (int e = 0; e < P; ++e) dk[e] = dw[e] * (kk[e] > 0.f ? 1.0f : w[e]);
  } else {
    float dwp = 0.f;
#pragma unroll
    for (int e = 0; e < P; ++e) dwp = fmaf(dw[e], w[e], dwp);
    dwp = sum4(dwp);
#pragma unroll
    for (int e = 0; e < P; ++e) dk[e] = w[e] * (dw[e] - dwp);
  }

  // sparse branch over the query blocks that hold key block j as critical
  float (*Qs)[D] = reinterpret_cast<float (*)[D]>(sm);
  float (*Gs)[D] = reinterpret_cast<float (*)[D]>(sm + kBlock * D);
  float* Ls = sm + 2 * kBlock * D;
  float* Ds = Ls + kBlock;
  for (int i = 0; i < Nb; ++i) {
    if (mask[((size_t)bh * Nb + i) * Nb + j] != 1) continue;  // uniform
    __syncthreads();
    for (int x = tid; x < kBlock * D; x += kThreads) {
      const int tq = x / D, c = x % D, tt = i * kBlock + tq;
      Qs[tq][c] = tt < N ? ldf<T>(Q + base + (size_t)tt * D + c) : 0.f;
      Gs[tq][c] = tt < N ? al * ldf<T>(dO + base + (size_t)tt * D + c) : 0.f;
    }
    if (tid < kBlock) {
      Ls[tid] = lse_in[((size_t)bh * Nb + i) * kBlock + tid];
      Ds[tid] = dt_in[((size_t)bh * Nb + i) * kBlock + tid];
    }
    __syncthreads();
    const int nq = min(kBlock, N - i * kBlock);
    for (int tq = 0; tq < nq; ++tq) {
      float sc = 0.f, dp = 0.f;
#pragma unroll
      for (int e = 0; e < P; ++e) {
        sc = fmaf(kk[e], Qs[tq][part * P + e], sc);
        dp = fmaf(vv[e], Gs[tq][part * P + e], dp);
      }
      sc = sum4(sc) * scale;
      dp = sum4(dp);
      const float p = __expf(sc - Ls[tq]);
      const float ds = p * (dp - Ds[tq]) * scale;
#pragma unroll
      for (int e = 0; e < P; ++e) {
        dv[e] = fmaf(p, Gs[tq][part * P + e], dv[e]);
        dk[e] = fmaf(ds, Qs[tq][part * P + e], dk[e]);
      }
    }
  }
  if (valid) {
#pragma unroll
    for (int e = 0; e < P; ++e) {
      dK[base + (size_t)s * D + part * P + e] = dk[e];
      dV[base + (size_t)s * D + part * P + e] = dv[e];
    }
  }
}

// dalpha[h] = sum over batches and query blocks of the partials, in that order
// one wave per head: lane l sums the partials i = l (mod 64) of every batch in
// order, then the lanes combine in a fixed butterfly (the same bits in every lane)
__global__ __launch_bounds__(64) void k_bwd_alpha(const float* __restrict__ dal, float* __restrict__ dalpha,
                                                  int B, int H, int Nb) {
  const int h = blockIdx.x, lane = threadIdx.x;
  double s = 0.0;
  for (int b = 0; b < B; ++b)
    for (int i = lane; i < Nb; i += 64) s += (double)dal[((size_t)b * H + h) * Nb + i];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
  if (lane == 0) dalpha[h] = (float)s;
}

template <typename T, int D, bool ELU, bool PROJ>
hipError_t launch_bwd_t(const Dims& Dm, const void* Q, const void* K, const void* V, const int8_t* mask,
                        const float* alpha, const float* proj_o, const void* dO, const Work& w,
                        const BwdWork& bw, float* dQ, float* dK, float* dV, float* dalpha, float* dproj_o,
                        hipStream_t s) {
  constexpr int NN = D * D + D;
  const dim3 grid(Dm.Nb, Dm.BH);
  hipLaunchKernelGGL((k_bwd_q<T, D, ELU, PROJ>), grid, dim3(kThreads), 0, s, (const T*)Q, (const T*)K,
                     (const T*)V, mask, (const T*)w.Hx, alpha, proj_o, Dm.proj_hs, (const T*)dO, dQ, bw.lse,
                     bw.dt, bw.dHx, bw.dal, bw.dWp, Dm.H, Dm.N, Dm.Nb);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_bwd_htot<D>, dim3((NN + 255) / 256, Dm.BH), dim3(256), 0, s, bw.dHx, bw.dHtot, Dm.Nb);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_bwd_kv<T, D, ELU>), grid, dim3(kThreads), 0, s, (const T*)Q, (const T*)K, (const T*)V,
                     mask, PROJ ? nullptr : alpha, (const T*)dO, bw.lse, bw.dt, bw.dHx, bw.dHtot, dK, dV, Dm.H,
                     Dm.N, Dm.Nb);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (PROJ) {
    e = launch_dw<D>(Dm, bw, dO, dproj_o, s);
    if (e != hipSuccess) return e;
  } else {
    hipLaunchKernelGGL(k_bwd_alpha, dim3(Dm.H), dim3(64), 0, s, bw.dal, dalpha, Dm.B, Dm.H, Dm.Nb);
  }
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_bwd_td(const Dims& Dm, const void* Q, const void* K, const void* V, const int8_t* mask,
                         const float* alpha, const float* proj_o, const void* dO, const Work& w,
                         const BwdWork& bw, float* dQ, float* dK, float* dV, float* dalpha, float* dproj_o,
                         hipStream_t s) {
  if (proj_o)
    return Dm.elu ? launch_bwd_t<T, D, true, true>(Dm, Q, K, V, mask, alpha, proj_o, dO, w, bw, dQ, dK, dV,
                                                   dalpha, dproj_o, s)
                  : launch_bwd_t<T, D, false, true>(Dm, Q, K, V, mask, alpha, proj_o, dO, w, bw, dQ, dK, dV,
                                                    dalpha, dproj_o, s);
  return Dm.elu ? launch_bwd_t<T, D, true, false>(Dm, Q, K, V, mask, alpha, proj_o, dO, w, bw, dQ, dK, dV,
                                                  dalpha, dproj_o, s)
                : launch_bwd_t<T, D, false, false>(Dm, Q, K, V, mask, alpha, proj_o, dO, w, bw, dQ, dK, dV,
                                                   dalpha, dproj_o, s);
}

}  // namespace

hipError_t launch_backward(const Dims& D, const void* Q, const void* K, const void* V, const int8_t* mask,
                           const float* alpha, const float* proj_o, const void* dO, const Work& w,
                           const BwdWork& bw, float* dQ, float* dK, float* dV, float* dalpha, float* dproj_o,
                           bool recompute, hipStream_t s) {
  if (D.bf16) {  // bf16 inputs: the MFMA kernels (k_backward_mfma.hip)
    hipError_t e = launch_backward_mfma(D, Q, K, V, mask, alpha, proj_o, dO, w, bw, dQ, dK, dV, recompute, s);
    if (e != hipSuccess) return e;
    if (proj_o) {
      e = D.d == 128 ? launch_dw<128>(D, bw, dO, dproj_o, s) : launch_dw<64>(D, bw, dO, dproj_o, s);
      if (e != hipSuccess) return e;
    } else {
      hipLaunchKernelGGL(k_bwd_alpha, dim3(D.H), dim3(64), 0, s, bw.dal, dalpha, D.B, D.H, D.Nb);
    }
    return hipGetLastError();
  }
  return D.d == 128 ? launch_bwd_td<float, 128>(D, Q, K, V, mask, alpha, proj_o, dO, w, bw, dQ, dK, dV, dalpha,
                                                dproj_o, s)
                    : launch_bwd_td<float, 64>(D, Q, K, V, mask, alpha, proj_o, dO, w, bw, dQ, dK, dV, dalpha,
                                               dproj_o, s);
}

}  // namespace sla
