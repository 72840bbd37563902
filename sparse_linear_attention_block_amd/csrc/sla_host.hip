// Host side of the C ABI declared in include/sla.h: argument validation,
// block counts, workspace carving, the launch order of the forward pass's
// kernels on the caller's stream (SLA2 and SLA formulations), and the
// SoftTop-k entry point. No device memory is allocated here and no call
// synchronises.
#include <float.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "sla_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Validates the problem and derives its sizes; SLA_OK or an error code.
int make_dims(const sla_problem* p, sla::Dims* D) {
  if (!p) return fail(SLA_ERR_ARG, "problem is NULL");
  if (p->B < 1 || p->H < 1 || p->N < 1)
    return fail(SLA_ERR_ARG, "B, H and N must be >= 1 (got %d, %d, %d)", p->B, p->H, p->N);
  if (p->dtype != SLA_F32 && p->dtype != SLA_BF16)
    return fail(SLA_ERR_ARG, "unknown dtype %d", p->dtype);
  if (p->quant != SLA_QUANT_NONE && p->quant != SLA_QUANT_I8QK_F8PV)
    return fail(SLA_ERR_ARG, "unknown quant mode %d", p->quant);
  if (p->phi != SLA_PHI_SOFTMAX && p->phi != SLA_PHI_ELU1)
    return fail(SLA_ERR_ARG, "unknown feature map %d", p->phi);
  if (!(p->kh >= 0.0 && p->kh <= 1.0) || !(p->kl >= 0.0 && p->kl <= 1.0))
    return fail(SLA_ERR_ARG, "kh and kl must lie in [0, 1] (got %g, %g)", p->kh, p->kl);
  if (p->d != 64 && p->d != 128) return fail(SLA_ERR_UNSUPPORTED, "head dim %d not built", p->d);
  if (p->proj_head_stride != 0 && p->proj_head_stride != p->d * p->d)
    return fail(SLA_ERR_ARG, "proj_head_stride must be 0 or d*d");
  if ((long long)p->B * p->H > 65535)
    return fail(SLA_ERR_UNSUPPORTED, "B*H = %lld exceeds 65535", (long long)p->B * p->H);
  const int Nb = (p->N + sla::kBlock - 1) / sla::kBlock;
  if (Nb > sla::kMaxNb) return fail(SLA_ERR_UNSUPPORTED, "N = %d exceeds %d tokens", p->N, sla::kMaxNb * sla::kBlock);
  int n_h = p->kh <= 0.0 ? 0 : (int)floor(p->kh * Nb + 1e-9);
  if (p->kh > 0.0 && n_h < 1) n_h = 1;
  if (n_h > Nb) n_h = Nb;
  const int n_l = (int)floor(p->kl * Nb + 1e-9);
  if (n_h + n_l > Nb)
    return fail(SLA_ERR_ARG, "kh and kl select %d + %d > %d blocks per row", n_h, n_l, Nb);
  if (p->quant == SLA_QUANT_I8QK_F8PV && p->dtype != SLA_BF16)
    return fail(SLA_ERR_UNSUPPORTED, "the 8-bit sparse branch needs bf16 inputs");
  if (p->linear_sums != SLA_LINEAR_GEMM && p->linear_sums != SLA_LINEAR_CHAIN)
    return fail(SLA_ERR_ARG, "unknown linear_sums %d", p->linear_sums);
  if (p->linear_sums == SLA_LINEAR_CHAIN && (p->dtype != SLA_BF16 || (Nb + 31) / 32 * 32 > sla::kChainMaxNbp))
    return fail(SLA_ERR_UNSUPPORTED, "the chain form of the marginal sums is built for bf16 and Nb <= %d",
                sla::kChainMaxNbp);
  D->B = p->B;
  D->H = p->H;
  D->N = p->N;
  D->d = p->d;
  D->BH = p->B * p->H;
  D->Nb = Nb;
  D->n_h = n_h;
  D->n_l = n_l;
  D->Nbp = (Nb + 31) / 32 * 32;
  D->Nb128 = (Nb + 127) / 128 * 128;
  D->NN = p->d * p->d + p->d;
  D->bf16 = p->dtype == SLA_BF16;
  D->quant = p->quant == SLA_QUANT_I8QK_F8PV;
  D->elu = p->phi == SLA_PHI_ELU1;
  D->proj_hs = p->proj_head_stride;
  D->chain = p->linear_sums == SLA_LINEAR_CHAIN;
  return SLA_OK;
}

}  // namespace

namespace sla {

size_t carve(const Dims& D, void* base, Work* w) {
  size_t off = 0;
  char* b = (char*)base;
  auto take = [&](size_t bytes) -> void* {
    void* p = b ? (void*)(b + off) : nullptr;
    off += align256(bytes);
    return p;
  };
  const size_t BH = (size_t)D.BH;
  Work x = {};
  x.pooled_q = (double*)take(BH * D.Nb * D.d * sizeof(double));
  x.pooled_k = (double*)take(BH * D.Nb * D.d * sizeof(double));
  x.pooled_raw = (double*)take(2 * BH * D.Nb * D.d * sizeof(double));
  x.hilo = (uint16_t*)take(4 * BH * D.Nb * D.d * sizeof(uint16_t));
  x.est = (float*)take(BH * D.Nb * D.Nb * sizeof(float));
  x.norms = (float*)take(BH * (D.Nb + (D.Nb + 63) / 64) * sizeof(float));
  if (D.bf16) {
    x.hx = take(BH * (D.Nbp / 4) * D.NN * 4 * sizeof(uint16_t));
    x.Hx = take(BH * D.Nb * D.NN * sizeof(uint16_t));
    x.ind = (uint32_t*)take(BH * (D.Nbp / 32) * D.Nb128 * sizeof(uint32_t));
    x.wo = (uint16_t*)take((size_t)(D.proj_hs ? D.H : 1) * D.d * D.d * sizeof(uint16_t));
    if (D.chain) {
      x.chain_lists = (uint16_t*)take(BH * D.Nb * D.Nb * sizeof(uint16_t));
      x.chain_cnt = (uint32_t*)take(BH * D.Nb * sizeof(uint32_t));
    }
  } else {
    x.hx = take(BH * D.Nb * D.NN * sizeof(float));
    x.Hx = take(BH * D.Nb * D.NN * sizeof(float));
  }
  if (D.quant) {
    x.qkmean = (float*)take(2 * BH * D.d * sizeof(float));
    x.k8 = (int8_t*)take(BH * D.Nb * kBlock * D.d);
    x.ks = (float*)take(BH * D.Nb * sizeof(float));
    x.kb = (float*)take(BH * D.Nb * kBlock * sizeof(float));
    x.v8t = (uint8_t*)take(BH * D.Nb * D.d * kBlock);
    x.vs = (float*)take(BH * D.Nb * sizeof(float));
  }
  if (w) *w = x;
  return off;
}

size_t carve_bwd(const Dims& D, bool proj, void* base, Work* w, BwdWork* bw) {
  size_t off = carve(D, base, w);
  char* b = (char*)base;
  auto take = [&](size_t bytes) -> void* {
    void* p = b ? (void*)(b + off) : nullptr;
    off += align256(bytes);
    return p;
  };
  const size_t BH = (size_t)D.BH, T = BH * D.Nb * kBlock;
  BwdWork x = {};
  x.lse = (float*)take(T * sizeof(float));
  x.dt = (float*)take(T * sizeof(float));
  x.dHx = (float*)take(BH * D.Nb * D.NN * sizeof(float));
  x.dHtot = (float*)take(BH * D.NN * sizeof(float));
  x.dal = (float*)take(BH * D.Nb * sizeof(float));
  if (D.bf16) {  // the MFMA path (SLA2; carved for both formulations so that the SLA fusion only adds dW)
    x.Os = (uint16_t*)take(2 * BH * D.N * D.d * sizeof(uint16_t));
    x.maskT = (int8_t*)take(BH * D.Nb * D.Nb);
    x.kvcnt = (int*)take(BH * D.Nb * sizeof(int));
    x.kvorder = (int*)take(BH * D.Nb * sizeof(int));
    const int slots = kv_slots((int)(BH * D.Nb));
    x.kvhdr = (int*)take(4 * sizeof(int));
    x.kvinfo = (int*)take(2 * BH * D.Nb * sizeof(int));
    x.kvtab = (int*)take(2 * (size_t)slots * sizeof(int));
    x.kvlist = (int*)take((size_t)slots * sizeof(int));
    x.kvpart = (float*)take((size_t)slots * 2 * kBlock * D.d * sizeof(float));
  }
  if (proj) {
    const int hs = D.proj_hs ? D.H : 1;
    if (D.bf16) {
      x.Ol = (uint16_t*)take(BH * D.N * D.d * sizeof(uint16_t));
      x.dWg = (float*)take((size_t)hs * dw_chunks(hs) * D.d * D.d * sizeof(float));
    } else {
      x.dWp = (float*)take(BH * D.Nb * D.d * D.d * sizeof(float));
    }
    x.dWs = (double*)take((size_t)hs * kDwSplit * D.d * D.d * sizeof(double));
    if (D.bf16) x.wq = (uint16_t*)take((size_t)(D.proj_hs ? D.H : 1) * D.d * D.d * sizeof(uint16_t));
  }
  if (bw) *bw = x;
  return off;
}

}  // namespace sla

extern "C" {

int sla_version(void) { return (1 << 16) | 2; }

const char* sla_status_str(int status) {
  switch (status) {
    case SLA_OK: return "SLA_OK";
    case SLA_ERR_ARG: return "SLA_ERR_ARG: invalid argument";
    case SLA_ERR_UNSUPPORTED: return "SLA_ERR_UNSUPPORTED: valid request outside what is built";
    case SLA_ERR_WORKSPACE: return "SLA_ERR_WORKSPACE: workspace missing, misaligned or too small";
    case SLA_ERR_HIP: return "SLA_ERR_HIP: HIP runtime error";
    default: return "unknown sla status";
  }
}

const char* sla_last_error(void) { return g_err; }

int sla_block_counts(const sla_problem* p, int32_t* nb, int32_t* n_h, int32_t* n_l) {
  sla::Dims D;
  sla_problem q;
  if (!p) return fail(SLA_ERR_ARG, "problem is NULL");
  // counts do not depend on what is built: validate with a buildable stand-in
  q = *p;
  q.quant = SLA_QUANT_NONE;
  if (q.d != 64 && q.d != 128) q.d = 64;
  q.proj_head_stride = 0;
  q.phi = SLA_PHI_SOFTMAX;
  q.linear_sums = SLA_LINEAR_GEMM;
  const int rc = make_dims(&q, &D);
  if (rc != SLA_OK) return rc;
  if (nb) *nb = D.Nb;
  if (n_h) *n_h = D.n_h;
  if (n_l) *n_l = D.n_l;
  g_err[0] = 0;
  return SLA_OK;
}

int sla_workspace_bytes(const sla_problem* p, size_t* bytes) {
  sla::Dims D;
  const int rc = make_dims(p, &D);
  if (rc != SLA_OK) return rc;
  if (!bytes) return fail(SLA_ERR_ARG, "bytes is NULL");
  *bytes = sla::carve(D, nullptr, nullptr);
  g_err[0] = 0;
  return SLA_OK;
}

}  // extern "C"

static int make_bwd_dims(const sla_problem* p, sla::Dims* D);

namespace {

// Both formulations: proj_o == NULL is SLA2 (O = alpha O_s + (1 - alpha) O_l),
// otherwise SLA (O = O_s + O_l proj_o). save: the workspace is the backward
// pass's, and the pass leaves there what the backward would otherwise recompute
// (h/z and H_i, Z_i in the forward regions; O_s and each query's log-sum-exp in
// the backward regions).
int run_forward(const sla_problem* p, const void* Q, const void* K, const void* V,
                const float* proj_q, const float* proj_k, const float* alpha, const float* proj_o,
                const int8_t* mask_in, void* O, int8_t* mask_out, void* workspace,
                size_t workspace_bytes, void* stream, const sla_debug* dbg, bool save = false) {
  sla::Dims D;
  int rc = save ? make_bwd_dims(p, &D) : make_dims(p, &D);
  if (rc != SLA_OK) return rc;
  if (save && !D.bf16) return fail(SLA_ERR_UNSUPPORTED, "the saving forward pass is built for bf16 inputs");
  const bool sla1 = proj_o != nullptr;
  if (!Q || !K || !V || !O) return fail(SLA_ERR_ARG, "Q, K, V and O must not be NULL");
  if (!sla1 && !alpha) return fail(SLA_ERR_ARG, "alpha must not be NULL");
  if (sla1 && D.quant)
    return fail(SLA_ERR_UNSUPPORTED, "the SLA output projection is built without the 8-bit sparse branch");
  if ((proj_q == nullptr) != (proj_k == nullptr))
    return fail(SLA_ERR_ARG, "proj_q and proj_k must both be given or both be NULL");
  if (!mask_in && !mask_out) return fail(SLA_ERR_ARG, "mask_out may be NULL only when mask_in is given");
  if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16))
    return fail(SLA_ERR_ARG, "Q, K, V and O must be 16-byte aligned");
  if ((proj_q && !aligned(proj_q, 4)) || (proj_k && !aligned(proj_k, 4)) || (alpha && !aligned(alpha, 4)) ||
      (proj_o && !aligned(proj_o, 4)))
    return fail(SLA_ERR_ARG, "proj_q, proj_k, proj_o and alpha must be 4-byte aligned");
  if (dbg && ((dbg->pooled_q && !aligned(dbg->pooled_q, 8)) || (dbg->pooled_k && !aligned(dbg->pooled_k, 8)) ||
              (dbg->logits && !aligned(dbg->logits, 8)) || (dbg->o_s && !aligned(dbg->o_s, 16)) ||
              (dbg->o_l && !aligned(dbg->o_l, 16))))
    return fail(SLA_ERR_ARG, "debug buffers must be aligned (8 bytes float64, 16 bytes float32)");
  const size_t need = save ? sla::carve_bwd(D, sla1, nullptr, nullptr, nullptr) : sla::carve(D, nullptr, nullptr);
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < need)
    return fail(SLA_ERR_WORKSPACE, "workspace needs %zu bytes at 256-byte alignment (got %zu at %p)",
                need, workspace_bytes, workspace);
  sla::Work w;
  sla::BwdWork bw = {};
  if (save)
    sla::carve_bwd(D, sla1, workspace, &w, &bw);
  else
    sla::carve(D, workspace, &w);
  hipStream_t s = (hipStream_t)stream;
  const int proj_hs = p->proj_head_stride;
  (void)hipGetLastError();  // a stale error from earlier work is not ours to report

#define SLA_LAUNCH(call, what)                                                            \
  do {                                                                                    \
    hipError_t e_ = (call);                                                               \
    if (e_ != hipSuccess) return fail(SLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e_)); \
  } while (0)

  auto mark = [&](int k) -> hipError_t {
    if (dbg && dbg->events[k]) return hipEventRecord((hipEvent_t)dbg->events[k], s);
    return hipSuccess;
  };
  const int8_t* mask = mask_in;
  SLA_LAUNCH(mark(0), "event record");
  if (!mask_in) {
    // without a router the block means themselves are compared
    const double* pq = w.pooled_raw;
    const double* pk = w.pooled_raw + (size_t)D.BH * D.Nb * D.d;
    SLA_LAUNCH(sla::launch_pool_sum(D, Q, K, w.pooled_raw, s), "pool kernel");
    if (proj_q) {
      SLA_LAUNCH(sla::launch_pool_proj(D, proj_q, proj_k, proj_hs, w.pooled_raw, w.pooled_q, w.pooled_k, s),
                 "pool/proj kernel");
      pq = w.pooled_q;
      pk = w.pooled_k;
    }
    SLA_LAUNCH(mark(1), "event record");
    SLA_LAUNCH(sla::launch_select(D, pq, pk, mask_out, w.hilo, w.est, w.norms, dbg ? dbg->logits : nullptr, s),
               "score/select kernel");
    SLA_LAUNCH(mark(2), "event record");
    if (dbg && dbg->pooled_q)
      SLA_LAUNCH(hipMemcpyAsync(dbg->pooled_q, pq, (size_t)D.BH * D.Nb * D.d * sizeof(double),
                                hipMemcpyDeviceToDevice, s), "debug copy");
    if (dbg && dbg->pooled_k)
      SLA_LAUNCH(hipMemcpyAsync(dbg->pooled_k, pk, (size_t)D.BH * D.Nb * D.d * sizeof(double),
                                hipMemcpyDeviceToDevice, s), "debug copy");
    mask = mask_out;
  } else {
    // the 8-bit branch smooths Q and K with their channel means, taken from the block means
    if (D.quant) SLA_LAUNCH(sla::launch_pool_sum(D, Q, K, w.pooled_raw, s), "pool kernel");
    SLA_LAUNCH(mark(1), "event record");
    SLA_LAUNCH(mark(2), "event record");
  }
  if (D.quant) SLA_LAUNCH(sla::launch_qk_mean(D, w, s), "channel-mean kernel");
  SLA_LAUNCH(sla::launch_hz(D, K, V, w, s), "h/z kernel");
  SLA_LAUNCH(mark(3), "event record");
  if (D.chain) {
    SLA_LAUNCH(sla::launch_chain(D, mask, w, s), "chain kernels");
  } else {
    if (D.bf16) SLA_LAUNCH(sla::launch_indicator(D, mask, w, s), "indicator kernel");
    SLA_LAUNCH(sla::launch_linear(D, mask, w, s), "linear kernel");
  }
  SLA_LAUNCH(mark(4), "event record");
  float* dos = dbg ? dbg->o_s : nullptr;
  float* dol = dbg ? dbg->o_l : nullptr;
  if (sla1 && D.bf16) SLA_LAUNCH(sla::launch_pack_proj(D, proj_o, w, s), "projection packing kernel");
  if (D.quant)
    SLA_LAUNCH(sla::launch_sparse_q8(D, Q, mask, alpha, w, O, dos, dol, s), "8-bit sparse kernel");
  else if (D.bf16 && save)
    SLA_LAUNCH(sla::launch_sparse(D, Q, K, V, mask, alpha, proj_o, w, O, nullptr, nullptr, s, bw.lse, bw.Os),
               "sparse kernel");
  else if (D.bf16)
    SLA_LAUNCH(sla::launch_sparse(D, Q, K, V, mask, alpha, proj_o, w, O, dos, dol, s), "sparse kernel");
  else
    SLA_LAUNCH(sla::launch_sparse_f32(D, Q, K, V, mask, alpha, proj_o, w, O, dos, dol, s), "sparse kernel");
  SLA_LAUNCH(mark(5), "event record");
#undef SLA_LAUNCH
  g_err[0] = 0;
  return SLA_OK;
}

}  // namespace

extern "C" {

int sla_forward_debug(const sla_problem* p, const void* Q, const void* K, const void* V,
                      const float* proj_q, const float* proj_k, const float* alpha,
                      const int8_t* mask_in, void* O, int8_t* mask_out, void* workspace,
                      size_t workspace_bytes, void* stream, const sla_debug* dbg) {
  return run_forward(p, Q, K, V, proj_q, proj_k, alpha, nullptr, mask_in, O, mask_out, workspace,
                     workspace_bytes, stream, dbg);
}

int sla_forward(const sla_problem* p, const void* Q, const void* K, const void* V,
                const float* proj_q, const float* proj_k, const float* alpha,
                const int8_t* mask_in, void* O, int8_t* mask_out, void* workspace,
                size_t workspace_bytes, void* stream) {
  return run_forward(p, Q, K, V, proj_q, proj_k, alpha, nullptr, mask_in, O, mask_out, workspace,
                     workspace_bytes, stream, nullptr);
}

int sla1_forward_debug(const sla_problem* p, const void* Q, const void* K, const void* V,
                       const float* proj_q, const float* proj_k, const float* proj_o,
                       const int8_t* mask_in, void* O, int8_t* mask_out, void* workspace,
                       size_t workspace_bytes, void* stream, const sla_debug* dbg) {
  if (!proj_o) return fail(SLA_ERR_ARG, "proj_o must not be NULL");
  return run_forward(p, Q, K, V, proj_q, proj_k, nullptr, proj_o, mask_in, O, mask_out, workspace,
                     workspace_bytes, stream, dbg);
}

int sla1_forward(const sla_problem* p, const void* Q, const void* K, const void* V,
                 const float* proj_q, const float* proj_k, const float* proj_o,
                 const int8_t* mask_in, void* O, int8_t* mask_out, void* workspace,
                 size_t workspace_bytes, void* stream) {
  return sla1_forward_debug(p, Q, K, V, proj_q, proj_k, proj_o, mask_in, O, mask_out, workspace,
                            workspace_bytes, stream, nullptr);
}

int sla_forward_train(const sla_problem* p, const void* Q, const void* K, const void* V,
                      const float* proj_q, const float* proj_k, const float* alpha,
                      const int8_t* mask_in, void* O, int8_t* mask_out, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return run_forward(p, Q, K, V, proj_q, proj_k, alpha, nullptr, mask_in, O, mask_out, workspace,
                     workspace_bytes, stream, nullptr, true);
}

int sla1_forward_train(const sla_problem* p, const void* Q, const void* K, const void* V,
                       const float* proj_q, const float* proj_k, const float* proj_o,
                       const int8_t* mask_in, void* O, int8_t* mask_out, void* workspace,
                       size_t workspace_bytes, void* stream) {
  if (!proj_o) return fail(SLA_ERR_ARG, "proj_o must not be NULL");
  return run_forward(p, Q, K, V, proj_q, proj_k, nullptr, proj_o, mask_in, O, mask_out, workspace,
                     workspace_bytes, stream, nullptr, true);
}

}  // extern "C"

// ---- the allocation-free forward pass
//
// Scratch of sla_forward_noalloc: one file-scope device array per GPU (every
// device that loads this library holds its own copy until the process ends).
// Host code never passes the array's name to a kernel (on the host it is only a
// stand-in symbol); it resolves the device address once per device with
// hipGetSymbolAddress and uses that.
static __device__ __align__(256) unsigned char scratch[SLA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address, resolved on its first use on that
// device (with the device current); nullptr on failure (g_err set).
void* scratch_ptr(int* status) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *status = fail(SLA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *status = fail(SLA_ERR_UNSUPPORTED, "device %d is beyond the %d devices the scratch table holds", dev,
                   kMaxDevices);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      *status = fail(SLA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int sla_forward_noalloc(const sla_problem* p, const void* Q, const void* K, const void* V,
                        const float* proj_q, const float* proj_k, const float* alpha,
                        const int8_t* mask_in, void* O, int8_t* mask_out, void* stream) {
  sla::Dims D;
  const int rc = make_dims(p, &D);
  if (rc != SLA_OK) return rc;
  const size_t need = sla::carve(D, nullptr, nullptr);
  if (need > (size_t)SLA_NOALLOC_SCRATCH_BYTES)
    return fail(SLA_ERR_WORKSPACE,
                "this problem needs %zu bytes of scratch; sla_forward_noalloc holds %zu (use sla_forward "
                "with a workspace)", need, (size_t)SLA_NOALLOC_SCRATCH_BYTES);
  int status = SLA_OK;
  void* ws = scratch_ptr(&status);
  if (!ws) return status;
  return run_forward(p, Q, K, V, proj_q, proj_k, alpha, nullptr, mask_in, O, mask_out, ws,
                     (size_t)SLA_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}

int sla_soft_topk(const double* logits, int32_t rows, int32_t cols, double k, double tau, float* out,
                  float* lambda, void* stream) {
  if (!logits || !out) return fail(SLA_ERR_ARG, "logits and out must not be NULL");
  if (!aligned(logits, 8) || !aligned(out, 4) || (lambda && !aligned(lambda, 4)))
    return fail(SLA_ERR_ARG, "logits must be 8-byte aligned, out and lambda 4-byte aligned");
  if (rows < 1 || cols < 1 || cols > sla::kMaxNb)
    return fail(SLA_ERR_ARG, "rows must be >= 1 and cols in [1, %d] (got %d, %d)", sla::kMaxNb, rows, cols);
  if (!(k >= 0.0 && k <= (double)cols)) return fail(SLA_ERR_ARG, "k must lie in [0, cols] (got %g)", k);
  if (!(tau >= 1e-20 && tau <= 1e20)) return fail(SLA_ERR_ARG, "tau must lie in [1e-20, 1e20] (got %g)", tau);
  // the kernel searches in float32: a budget strictly inside (0, cols) stays
  // strictly inside when rounded, so only k = 0 and k = cols take the edge cases
  float kf = (float)k;
  if (k > 0.0 && k < (double)cols) {
    if (!(kf > 0.f)) kf = FLT_MIN;
    if (kf >= (float)cols) kf = nextafterf((float)cols, 0.f);
  }
  (void)hipGetLastError();  // a stale error from earlier work is not ours to report
  const hipError_t e = sla::launch_soft_topk(logits, rows, cols, kf, (float)tau, out, lambda,
                                             (hipStream_t)stream);
  if (e != hipSuccess) return fail(SLA_ERR_HIP, "soft top-k kernel: %s", hipGetErrorString(e));
  g_err[0] = 0;
  return SLA_OK;
}

// Validation shared by the backward entry points; SLA_OK or an error code.
static int make_bwd_dims(const sla_problem* p, sla::Dims* D) {
  const int rc = make_dims(p, D);
  if (rc != SLA_OK) return rc;
  if (D->quant) return fail(SLA_ERR_UNSUPPORTED, "the backward pass is built without the 8-bit branch");
  return SLA_OK;
}

int sla_backward_workspace_bytes(const sla_problem* p, size_t* bytes) {
  sla::Dims D;
  const int rc = make_bwd_dims(p, &D);
  if (rc != SLA_OK) return rc;
  if (!bytes) return fail(SLA_ERR_ARG, "bytes is NULL");
  *bytes = sla::carve_bwd(D, false, nullptr, nullptr, nullptr);
  g_err[0] = 0;
  return SLA_OK;
}

int sla1_backward_workspace_bytes(const sla_problem* p, size_t* bytes) {
  sla::Dims D;
  const int rc = make_bwd_dims(p, &D);
  if (rc != SLA_OK) return rc;
  if (!bytes) return fail(SLA_ERR_ARG, "bytes is NULL");
  *bytes = sla::carve_bwd(D, true, nullptr, nullptr, nullptr);
  g_err[0] = 0;
  return SLA_OK;
}

}  // extern "C"

namespace {

// Both formulations: proj_o == NULL is SLA2 (dalpha), otherwise SLA (dproj_o).
// saved: the workspace holds what the saving forward pass left there, so the
// forward is not run again.
int run_backward(const sla_problem* p, const void* Q, const void* K, const void* V, const float* alpha,
                 const float* proj_o, const int8_t* mask, const void* dO, float* dQ, float* dK, float* dV,
                 float* dalpha, float* dproj_o, void* workspace, size_t workspace_bytes, void* stream,
                 bool saved = false) {
  sla::Dims D;
  const int rc = make_bwd_dims(p, &D);
  if (rc != SLA_OK) return rc;
  if (saved && !D.bf16) return fail(SLA_ERR_UNSUPPORTED, "the backward from saved state is built for bf16 inputs");
  const bool sla1 = proj_o != nullptr;
  if (!Q || !K || !V || !mask || !dO || !dQ || !dK || !dV)
    return fail(SLA_ERR_ARG, "Q, K, V, mask, dO, dQ, dK and dV must not be NULL");
  if (!sla1 && (!alpha || !dalpha)) return fail(SLA_ERR_ARG, "alpha and dalpha must not be NULL");
  if (sla1 && !dproj_o) return fail(SLA_ERR_ARG, "dproj_o must not be NULL");
  if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(dO, 16) || !aligned(dQ, 16) ||
      !aligned(dK, 16) || !aligned(dV, 16) || (alpha && !aligned(alpha, 4)) || (dalpha && !aligned(dalpha, 4)) ||
      (proj_o && !aligned(proj_o, 4)) || (dproj_o && !aligned(dproj_o, 4)))
    return fail(SLA_ERR_ARG, "tensors must be 16-byte aligned, alpha, proj_o and their gradients 4-byte aligned");
  const size_t need = sla::carve_bwd(D, sla1, nullptr, nullptr, nullptr);
  if (!workspace || !aligned(workspace, 256) || workspace_bytes < need)
    return fail(SLA_ERR_WORKSPACE, "workspace needs %zu bytes at 256-byte alignment (got %zu at %p)",
                need, workspace_bytes, workspace);
  sla::Work w;
  sla::BwdWork bw;
  sla::carve_bwd(D, sla1, workspace, &w, &bw);
  hipStream_t s = (hipStream_t)stream;
  (void)hipGetLastError();  // a stale error from earlier work is not ours to report
#define SLA_LAUNCH(call, what)                                                            \
  do {                                                                                    \
    hipError_t e_ = (call);                                                               \
    if (e_ != hipSuccess) return fail(SLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e_)); \
  } while (0)
  if (!saved) {
    // the linear branch's per-query-block state H_i, Z_i, as in the forward pass
    SLA_LAUNCH(sla::launch_hz(D, K, V, w, s), "h/z kernel");
    if (D.chain) {
      SLA_LAUNCH(sla::launch_chain(D, mask, w, s), "chain kernels");
    } else {
      if (D.bf16) SLA_LAUNCH(sla::launch_indicator(D, mask, w, s), "indicator kernel");
      SLA_LAUNCH(sla::launch_linear(D, mask, w, s), "linear kernel");
    }
  }
  SLA_LAUNCH(sla::launch_backward(D, Q, K, V, mask, sla1 ? nullptr : alpha, proj_o, dO, w, bw, dQ, dK, dV,
                                  dalpha, dproj_o, !saved, s),
             "backward kernels");
#undef SLA_LAUNCH
  g_err[0] = 0;
  return SLA_OK;
}

}  // namespace

extern "C" {

int sla_backward(const sla_problem* p, const void* Q, const void* K, const void* V, const float* alpha,
                 const int8_t* mask, const void* dO, float* dQ, float* dK, float* dV, float* dalpha,
                 void* workspace, size_t workspace_bytes, void* stream) {
  return run_backward(p, Q, K, V, alpha, nullptr, mask, dO, dQ, dK, dV, dalpha, nullptr, workspace,
                      workspace_bytes, stream);
}

int sla1_backward(const sla_problem* p, const void* Q, const void* K, const void* V, const float* proj_o,
                  const int8_t* mask, const void* dO, float* dQ, float* dK, float* dV, float* dproj_o,
                  void* workspace, size_t workspace_bytes, void* stream) {
  if (!proj_o) return fail(SLA_ERR_ARG, "proj_o must not be NULL");
  return run_backward(p, Q, K, V, nullptr, proj_o, mask, dO, dQ, dK, dV, nullptr, dproj_o, workspace,
                      workspace_bytes, stream);
}

int sla_backward_saved(const sla_problem* p, const void* Q, const void* K, const void* V, const float* alpha,
                       const int8_t* mask, const void* dO, float* dQ, float* dK, float* dV, float* dalpha,
                       void* workspace, size_t workspace_bytes, void* stream) {
  return run_backward(p, Q, K, V, alpha, nullptr, mask, dO, dQ, dK, dV, dalpha, nullptr, workspace,
                      workspace_bytes, stream, true);
}

int sla1_backward_saved(const sla_problem* p, const void* Q, const void* K, const void* V, const float* proj_o,
                        const int8_t* mask, const void* dO, float* dQ, float* dK, float* dV, float* dproj_o,
                        void* workspace, size_t workspace_bytes, void* stream) {
  if (!proj_o) return fail(SLA_ERR_ARG, "proj_o must not be NULL");
  return run_backward(p, Q, K, V, nullptr, proj_o, mask, dO, dQ, dK, dV, nullptr, dproj_o, workspace,
                      workspace_bytes, stream, true);
}

}  // extern "C"
