// Internal declarations shared by the host dispatcher and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "sla.h"

namespace sla {

constexpr int kBlock = 64;        // tokens per query / key block
constexpr int kMaxNb = 4096;      // largest block count the selection kernel handles

// Sizes derived from an sla_problem.
struct Dims {
  int B, H, N, d, BH, Nb;
  int n_h, n_l;
  int Nbp;          // Nb rounded up to a multiple of 32 (K extent of the linear GEMM)
  int Nb128;        // Nb rounded up to a multiple of 128 (row tiles of the linear GEMM)
  int NN;           // d*d + d: one h_j (stored transposed, c-major) followed by z_j
  bool bf16;
  bool quant;
  bool elu;         // feature map elu(x) + 1 instead of the softmax over the features
  int proj_hs;      // head stride of proj_q / proj_k / proj_o in elements: 0 or d*d
};

// Device workspace regions, carved from the caller's buffer.
struct Work {
  double* pooled_q;   // [BH, Nb, d]
  double* pooled_k;   // [BH, Nb, d]
  double* pooled_raw; // [2, BH, Nb, d] block means before the router projection
  double* logits;     // [BH, Nb, Nb] pooled logits pool(Q) pool(K)^T / sqrt(d)
  void* hx;           // bf16: [BH, Nbp/4, NN, 4] (four key blocks interleaved per column)
                      // f32:  [BH, Nb, NN]
  void* Hx;           // [BH, Nb, NN] per query block: H_i^T (c-major) then Z_i; bf16 or f32
  uint32_t* ind;      // bf16 only: [BH, Nbp/32, Nb128/128, 16, 8] marginal indicator (Mc == 0)
                      // as bits, one 32-bit word per (32-key step, query block) (k_linear.hip)
  uint16_t* vt;       // bf16 without quant: [BH, Nb, d, 64] V^T of every key block (zero past N)
  float* qkmean;      // quant only: [2, BH, d] channel means of Q and K over the N tokens
  int8_t* k8;         // quant only: [BH, Nb*64, d] int8 of K - mean(K), zero rows past N;
                      // bytes of each row in the score product's k-slot order (k_quant.hip)
  float* ks;          // quant only: [BH, Nb] per-block scales of k8
  float* kb;          // quant only: [BH, Nb*64] per-key bias mean(Q).(K - mean(K)) * log2(e)/sqrt(d), 0 past N
  uint8_t* v8t;       // quant only: [BH, Nb, d, 4, 16] fp8 e4m3 V^T (see the h/z kernel)
  float* vs;          // quant only: [BH, Nb] per-block scales of V
  uint16_t* wo;       // bf16 only: [Hs, d/16, d/32, 64, 8] the SLA output map Proj in bf16 MFMA
                      // A-operand fragments (Hs = H if it is per head, else 1; k_sparse.hip)
};

size_t carve(const Dims& D, void* base, Work* w);  // returns bytes needed (base may be NULL)

// Backward-pass regions, carved after the forward's (k_backward.hip).
struct BwdWork {
  float* lse;    // [BH, Nb*64] log-sum-exp of each query's critical scores (+inf if none)
  float* dt;     // [BH, Nb*64] dO_s . O_s of each query
  float* dHx;    // [BH, Nb, NN] dH_i (stored like H_i^T) then dZ_i, per query block
  float* dHtot;  // [BH, NN] their sum over the head's query blocks
  float* dal;    // [BH, Nb] partial dalpha of each query block
};
size_t carve_bwd(const Dims& D, void* base, Work* w, BwdWork* bw);  // forward + backward bytes

// ---- launchers (each enqueues one or more kernels on `s`, returns hipError_t)
hipError_t launch_pool_sum(const Dims& D, const void* Q, const void* K, double* raw,
                           hipStream_t s);
// the router projection of the block means launch_pool_sum wrote to raw
hipError_t launch_pool_proj(const Dims& D, const float* proj_q, const float* proj_k, int proj_hs,
                            const double* raw, double* pq, double* pk, hipStream_t s);
hipError_t launch_qk_mean(const Dims& D, const Work& w, hipStream_t s);
hipError_t launch_sparse_q8(const Dims& D, const void* Q, const int8_t* mask, const float* alpha,
                            const Work& w, void* O, float* dbg_os, float* dbg_ol, hipStream_t s);
hipError_t launch_select(const Dims& D, const double* pq, const double* pk, int8_t* mask,
                         double* lg, hipStream_t s);  // lg: [BH, Nb, Nb] float64 logits (written)
hipError_t launch_hz(const Dims& D, const void* K, const void* V, const Work& w, hipStream_t s);
hipError_t launch_indicator(const Dims& D, const int8_t* mask, const Work& w, hipStream_t s);
hipError_t launch_linear(const Dims& D, const int8_t* mask, const Work& w, hipStream_t s);
// proj_o == NULL: the SLA2 mix with alpha; else O = O_s + O_l proj_o (alpha unused; the
// bf16 kernel reads the fragments that launch_pack_proj wrote to w.wo)
hipError_t launch_pack_proj(const Dims& D, const float* proj_o, const Work& w, hipStream_t s);
hipError_t launch_sparse(const Dims& D, const void* Q, const void* K, const int8_t* mask,
                         const float* alpha, const float* proj_o, const Work& w, void* O,
                         float* dbg_os, float* dbg_ol, hipStream_t s);
hipError_t launch_sparse_f32(const Dims& D, const void* Q, const void* K, const void* V,
                             const int8_t* mask, const float* alpha, const float* proj_o,
                             const Work& w, void* O, float* dbg_os, float* dbg_ol, hipStream_t s);

hipError_t launch_backward(const Dims& D, const void* Q, const void* K, const void* V, const int8_t* mask,
                           const float* alpha, const void* dO, const Work& w, const BwdWork& bw, float* dQ,
                           float* dK, float* dV, float* dalpha, hipStream_t s);
// SoftTop-k rows of a float64 logit matrix (k_soft_topk.hip); cols <= 4096
hipError_t launch_soft_topk(const double* logits, int rows, int cols, float k, float tau, float* out,
                            float* lambda, hipStream_t s);

}  // namespace sla
