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
  bool chain;       // marginal sums by the row-to-row chain (k_chain.hip) instead of the GEMM
};

// Device workspace regions, carved from the caller's buffer.
struct Work {
  double* pooled_q;   // [BH, Nb, d]
  double* pooled_k;   // [BH, Nb, d]
  double* pooled_raw; // [2, BH, Nb, d] block means before the router projection
  uint16_t* hilo;     // [4, BH, Nb, d] bf16 two-term split of the pooled queries (hi, lo), then keys
  float* est;         // [BH, Nb, Nb] float32 estimates of the pooled logits
                      // pool(Q) pool(K)^T / sqrt(d) (k_select.hip)
  float* norms;       // [BH, Nb] norms of the pooled queries, then [BH, ceil(Nb / 64)] the
                      // largest norm of each 64 pooled keys
  void* hx;           // bf16: [BH, Nbp/4, NN, 4] (four key blocks interleaved per column)
                      // f32:  [BH, Nb, NN]
  void* Hx;           // [BH, Nb, NN] per query block: H_i^T (c-major) then Z_i; bf16 or f32
  uint32_t* ind;      // bf16 only: [BH, Nbp/32, Nb128/128, 16, 8] marginal indicator (Mc == 0)
                      // as bits, one 32-bit word per (32-key step, query block) (k_linear.hip)
  float* qkmean;      // quant only: [2, BH, d] channel means of Q and K over the N tokens
  int8_t* k8;         // quant only: [BH, Nb*64, d] int8 of K - mean(K), zero rows past N;
                      // bytes of each row in the score product's k-slot order (k_quant.hip)
  float* ks;          // quant only: [BH, Nb] per-block scales of k8
  float* kb;          // quant only: [BH, Nb*64] per-key bias mean(Q).(K - mean(K)) * log2(e)/sqrt(d), 0 past N
  uint8_t* v8t;       // quant only: [BH, Nb, d, 4, 16] fp8 e4m3 V^T (see the h/z kernel)
  float* vs;          // quant only: [BH, Nb] per-block scales of V
  uint16_t* wo;       // bf16 only: [Hs, d/16, d/32, 64, 8] the SLA output map Proj in bf16 MFMA
                      // A-operand fragments (Hs = H if it is per head, else 1; k_sparse.hip)
  uint16_t* chain_lists;  // chain only: [BH, Nb, Nb] per row, the blocks to add (front) and subtract (back)
  uint32_t* chain_cnt;    // chain only: [BH, Nb] their counts, n_add | n_sub << 16
};

size_t carve(const Dims& D, void* base, Work* w);  // returns bytes needed (base may be NULL)

// Backward-pass regions, carved after the forward's (k_backward.hip).
struct BwdWork {
  float* lse;    // [BH, Nb*64] log-sum-exp of each query's critical scores (+inf if none)
  float* dt;     // [BH, Nb*64] dO_s . O_s of each query
  float* dHx;    // [BH, Nb, NN] dH_i (stored like H_i^T) then dZ_i, per query block
  float* dHtot;  // [BH, NN] their sum over the head's query blocks
  float* dal;    // [BH, Nb] partial dalpha of each query block
  float* dWp;    // SLA fusion, float32 inputs: [BH, Nb, d, d] each query block's part of dW = O_l^T dO
  uint16_t* Ol;  // SLA fusion, bf16 inputs: [BH, N, d] O_l in bf16 (the dQ kernel's, for dW)
  float* dWg;    // SLA fusion, bf16 inputs: [Hs, kDwChunks / Hs, d, d] dW over consecutive row chunks
  double* dWs;   // SLA fusion only: [Hs, kDwSplit, d, d] sums of consecutive ranges of those parts
  uint16_t* Os;  // bf16 only: [2, BH, N, d] O_s as bf16 hi, then bf16 lo = O_s - hi (the sparse
                 // kernel's LSE instance)
  int8_t* maskT; // bf16 only: [BH, Nb, Nb] the transposed mask
  uint16_t* wq;  // bf16 SLA fusion only: [Hs, d, d] the output map as bf16 A-operand fragments
  int* kvcnt;    // bf16 only: [BH * Nb] critical query blocks per key block
  int* kvorder;  // bf16 only: [BH * Nb] key blocks by falling count (the dK/dV launch order)
  // bf16 only: the dK/dV work of a key block cut into chunks of its critical list (k_kv_split)
  int* kvhdr;    // [4]: chunk length, extra chunks, split key blocks
  int* kvinfo;   // [BH * Nb][2]: chunks of the key block, its first partial slot
  int* kvtab;    // [kv_slots][2]: key block and chunk (>= 1) of each extra chunk
  int* kvlist;   // [kv_slots]: the key blocks cut into more than one chunk
  float* kvpart; // [kv_slots][2][64][d]: dK and dV of each extra chunk
};
// ranges the SLA fusion's dW parts are summed in before the ranges are added
constexpr int kDwSplit = 32;
// partial slots of the chunked dK/dV work (one per extra chunk) and the shortest chunk
inline int kv_slots(int rows) { return rows / 4 > 0 ? rows / 4 : 1; }
constexpr int kKvChunk = 64;
constexpr int kKvRedY = 8;  // slices of a key block in the ordered sum of its chunk parts
// row chunks of the bf16 dW product (over all W matrices together)
constexpr int kDwChunks = 512;
inline int dw_chunks(int hs) { return kDwChunks / hs > 0 ? kDwChunks / hs : 1; }
// forward + backward bytes; proj: the SLA fusion's dW parts are included
size_t carve_bwd(const Dims& D, bool proj, void* base, Work* w, BwdWork* bw);

// ---- launchers (each enqueues one or more kernels on `s`, returns hipError_t)
hipError_t launch_pool_sum(const Dims& D, const void* Q, const void* K, double* raw,
                           hipStream_t s);
// the router projection of the block means launch_pool_sum wrote to raw
hipError_t launch_pool_proj(const Dims& D, const float* proj_q, const float* proj_k, int proj_hs,
                            const double* raw, double* pq, double* pk, hipStream_t s);
hipError_t launch_qk_mean(const Dims& D, const Work& w, hipStream_t s);
hipError_t launch_sparse_q8(const Dims& D, const void* Q, const int8_t* mask, const float* alpha,
                            const Work& w, void* O, float* dbg_os, float* dbg_ol, hipStream_t s);
// the mask from the pooled vectors; dbg_lg (may be NULL): [BH, Nb, Nb] float64 logits, written
hipError_t launch_select(const Dims& D, const double* pq, const double* pk, int8_t* mask,
                         uint16_t* hilo, float* est, float* norms, double* dbg_lg, hipStream_t s);
hipError_t launch_hz(const Dims& D, const void* K, const void* V, const Work& w, hipStream_t s);
hipError_t launch_indicator(const Dims& D, const int8_t* mask, const Work& w, hipStream_t s);
hipError_t launch_linear(const Dims& D, const int8_t* mask, const Work& w, hipStream_t s);
// the chain form of the marginal sums (bf16, Nbp <= kChainMaxNbp), and its LDS bytes per workgroup
constexpr int kChainMaxNbp = 1216;
size_t chain_lds_bytes(int Nbp);
hipError_t launch_chain(const Dims& D, const int8_t* mask, const Work& w, hipStream_t s);
// proj_o == NULL: the SLA2 mix with alpha; else O = O_s + O_l proj_o (alpha unused; the
// bf16 kernel reads the fragments that launch_pack_proj wrote to w.wo)
hipError_t launch_pack_proj(const Dims& D, const float* proj_o, const Work& w, hipStream_t s);
// O may be NULL (nothing stored); lse_out (may be NULL): [BH, Nb*64] log2 of each query's softmax
// normaliser over its critical keys, P = exp2(s log2(e) / sqrt(d) - lse2) (+inf past N or with no
// critical key)
hipError_t launch_sparse(const Dims& D, const void* Q, const void* K, const void* V, const int8_t* mask,
                         const float* alpha, const float* proj_o, const Work& w, void* O,
                         float* dbg_os, float* dbg_ol, hipStream_t s, float* lse_out = nullptr,
                         uint16_t* os_out = nullptr);
hipError_t launch_sparse_f32(const Dims& D, const void* Q, const void* K, const void* V,
                             const int8_t* mask, const float* alpha, const float* proj_o,
                             const Work& w, void* O, float* dbg_os, float* dbg_ol, hipStream_t s);

// proj_o == NULL: SLA2 (dalpha written, dproj_o unused); else the SLA fusion (dproj_o
// written, alpha and dalpha unused)
// bf16 inputs: the MFMA kernels of k_backward_mfma.hip; writes dQ, dK, dV and the per-block
// dalpha partials (bw.dal; SLA2) or dW parts (bw.dWp; proj_o given); uses bw.lse / bw.dt as
// lse2 / D_t and bw.dHx as bf16 dH. recompute: first run the sparse forward for bw.Os and
// bw.lse; otherwise they hold what a saving forward pass left there (bf16 only)
hipError_t launch_backward_mfma(const Dims& D, const void* Q, const void* K, const void* V, const int8_t* mask,
                                const float* alpha, const float* proj_o, const void* dO, const Work& w,
                                const BwdWork& bw, float* dQ, float* dK, float* dV, bool recompute,
                                hipStream_t s);
// bf16 SLA fusion: dW over row chunks of O_l (bw.Ol) and dO into bw.dWg, one part per chunk
hipError_t launch_dw_mfma(const Dims& D, const BwdWork& bw, const void* dO, hipStream_t s);
hipError_t launch_backward(const Dims& D, const void* Q, const void* K, const void* V, const int8_t* mask,
                           const float* alpha, const float* proj_o, const void* dO, const Work& w,
                           const BwdWork& bw, float* dQ, float* dK, float* dV, float* dalpha, float* dproj_o,
                           bool recompute, hipStream_t s);
// SoftTop-k rows of a float64 logit matrix (k_soft_topk.hip); cols <= 4096
hipError_t launch_soft_topk(const double* logits, int rows, int cols, float k, float tau, float* out,
                            float* lambda, hipStream_t s);

}  // namespace sla
