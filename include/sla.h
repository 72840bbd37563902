/*
 * sla.h - C ABI of the MI355X (gfx950) forward pass of SLA / SLA2
 * sparse-linear attention.
 *
 * The method (SLA paper summary on aipaper.cc, section 4, Eq. 1-3 and Fig. 4;
 * SLA2 article on mcffsbgs.com, the learned-router and mixing paragraphs):
 * for every (batch, head), queries and keys are cut into 64-token blocks; a
 * router projects Q and K with two learned d x d matrices and mean-pools each
 * block; the compressed map Pc = softmax(pool(Q) pool(K)^T / sqrt(d)) ranks,
 * per query block, the key blocks into critical (top kh), negligible
 * (bottom kl) and marginal (the rest); critical blocks get exact block-sparse
 * softmax attention O_s, marginal blocks get linear attention
 * O_l = phi(Q_i) H_i / (phi(Q_i) Z_i) with H_i, Z_i the sums of
 * phi(K_j)^T V_j and rowsum(phi(K_j)^T) over marginal j (phi = softmax over
 * the features), negligible blocks are skipped, and
 * O = alpha_h * O_s + (1 - alpha_h) * O_l.
 * The SLA formulation (SLA paper summary, section 4, step 4 and the
 * final-output formula) fuses the branches as O = O_s + Proj(O_l) with a
 * learned d x d linear map instead (sla1_forward), and the linear branch may
 * use phi = ELU + 1 instead of the softmax (Eq. 3's symbol list and Table 2;
 * sla_problem.phi, for either formulation).
 *
 * Conventions shared by every entry point:
 *  - Q, K, V, O are [B, H, N, d] contiguous, row-major, 16-byte aligned
 *    device buffers of `dtype`. Self-attention: queries and keys share N.
 *  - Nb = ceil(N / 64). The last block may be ragged; its missing tokens
 *    take no part in pooling, attention or sums, and are never written.
 *  - Block mask values: 1 critical, 0 marginal, -1 negligible (Eq. 2 of the
 *    SLA paper summary). Layout [B, H, Nb, Nb] int8, row = query block.
 *  - Counts per query-block row: n_h = 0 if kh == 0, else
 *    max(1, floor(kh*Nb + 1e-9)); n_l = floor(kl*Nb + 1e-9); n_h + n_l <= Nb.
 *    Ranking order: larger compressed logit first, lower block index first
 *    among equal logits; critical = head n_h, negligible = tail n_l.
 *    Logits are formed and ranked in float64.
 *  - All device work is enqueued on `stream` (a hipStream_t, NULL = the
 *    default stream); calls return after enqueue and never synchronise.
 *  - The library allocates no device memory and keeps no state between calls:
 *    the caller owns every buffer, including the workspace sized by
 *    sla_workspace_bytes(). Calls are reentrant if their workspaces differ.
 *    The one exception is sla_forward_noalloc, whose scratch is a fixed array
 *    that the library holds on each GPU (see its declaration).
 *  - Argument errors are reported before anything is enqueued, with outputs
 *    untouched. No C++ exception crosses this interface.
 */
#ifndef SLA_H
#define SLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SLA_OK = 0,
  SLA_ERR_ARG = -1,          /* bad pointer, size, fraction, alignment        */
  SLA_ERR_UNSUPPORTED = -2,  /* valid request outside what is built           */
  SLA_ERR_WORKSPACE = -3,    /* workspace missing, misaligned or too small    */
  SLA_ERR_HIP = -4           /* a HIP runtime call or a launch failed         */
} sla_status;

typedef enum { SLA_F32 = 0, SLA_BF16 = 1 } sla_dtype;

typedef enum {
  SLA_QUANT_NONE = 0,
  /* 8-bit sparse branch (SLA2 article, quantisation-aware paragraph): Q and
   * K minus their channel means over the N tokens as int8 (the Q mean enters
   * as an exact per-key float32 bias, the K mean cancels in the softmax) and
   * V as fp8 e4m3, each with one absmax scale per 64-token block; P as fp8
   * e4m3 with one power-of-two scale per query row and pair of 64-key tiles
   * (the largest code of the row in (224, 448]).
   * Requires dtype == SLA_BF16. The linear branch stays bf16; the mask is
   * decided from the unquantised inputs. */
  SLA_QUANT_I8QK_F8PV = 1
} sla_quant;

/* Feature map phi of the linear branch, applied to every query and key token
 * of the un-projected Q and K. */
typedef enum {
  SLA_PHI_SOFTMAX = 0,  /* softmax over the d features of the token             */
  SLA_PHI_ELU1 = 1      /* elementwise elu(x) + 1: x + 1 for x > 0, exp(x) else */
} sla_phi;

/* How the per-query-block marginal sums H_i, Z_i of the linear branch are
 * formed (the result is the same up to float32 rounding order). */
typedef enum {
  SLA_LINEAR_GEMM = 0,   /* one 0/1-indicator matrix product per head on MFMA      */
  SLA_LINEAR_CHAIN = 1   /* each row from the previous one: add the blocks that
                          * became marginal, subtract those that stopped being so
                          * (SLA explainer, section 2.3, on sparse per-row sums);
                          * bf16 only, Nb <= 1216 (SLA_ERR_UNSUPPORTED otherwise) */
} sla_linear_sums;

typedef struct {
  int32_t B, H, N, d;         /* d in {64, 128}                                  */
  int32_t dtype;              /* sla_dtype of Q, K, V, O                         */
  int32_t quant;              /* sla_quant                                       */
  int32_t proj_head_stride;   /* 0: proj_q/proj_k (and proj_o) are one [d, d]    */
                              /* matrix for all heads; d*d: they are [H, d, d]   */
  int32_t phi;                /* sla_phi                                         */
  double  kh, kl;             /* critical / negligible fractions in [0, 1]       */
  int32_t linear_sums;        /* sla_linear_sums (0, the default, is the GEMM)   */
} sla_problem;

/* Debug outputs of sla_forward_debug. Every pointer is a device buffer or NULL.
 * pooled_q, pooled_k: [B, H, Nb, d] float64, the router-projected block means
 *                     (Eq. 1's pool(Q), pool(K)); the plain block means when
 *                     the router matrices are NULL;
 * logits:             [B, H, Nb, Nb] float64, pool(Q) pool(K)^T / sqrt(d);
 * o_s, o_l:           [B, H, N, d] float32, the sparse and linear branch outputs
 *                     before the mix (for sla1_forward_debug, o_l is Proj(O_l)).
 *                     pooled_q/pooled_k/logits are only written when the mask
 *                     is computed (mask_in == NULL).
 * events:             caller-owned hipEvent_t handles (or NULL), recorded on
 *                     `stream`: events[0] before the pooling kernel and
 *                     events[k] after kernel k = 1 pooling, 2 scores/selection,
 *                     3 h/z, 4 marginal sums, 5 sparse attention + mix. With
 *                     mask_in, events 0-2 are recorded back to back. */
typedef struct {
  double* pooled_q;
  double* pooled_k;
  double* logits;
  float*  o_s;
  float*  o_l;
  void*   events[6];
} sla_debug;

/* Block counts of a problem (host only, no device work).
 * Out: *nb = Nb, *n_h and *n_l as defined above (each pointer may be NULL).
 * Returns SLA_OK, or SLA_ERR_ARG for a NULL problem, non-positive sizes,
 * fractions outside [0, 1] or n_h + n_l > Nb. */
int sla_block_counts(const sla_problem* p, int32_t* nb, int32_t* n_h, int32_t* n_l);

/* Device workspace that sla_forward needs for `p` (host only, no device work).
 * Out: *bytes. The workspace must be 256-byte aligned. Returns SLA_OK or the
 * validation error sla_forward would return for `p`. */
int sla_workspace_bytes(const sla_problem* p, size_t* bytes);

/* The SLA2 forward pass.
 *  Q, K, V   device, dtype, [B, H, N, d].
 *  proj_q,   device float32 router matrices indexed [in, out], one [d, d] or
 *  proj_k    [H, d, d] (see proj_head_stride). Both NULL: no router projection,
 *            the compressed map pools Q and K themselves (as SLA does); one
 *            NULL and the other not is SLA_ERR_ARG.
 *  alpha     device float32 [H], the per-head mixing ratio.
 *  mask_in   NULL, or a device int8 [B, H, Nb, Nb] block mask with values in
 *            {1, 0, -1} that replaces the router, pooling and classification;
 *            any such mask is valid and rows may hold any number of each class.
 *  O         device, dtype, [B, H, N, d] output.
 *  mask_out  device int8 [B, H, Nb, Nb]: the computed block mask. May be NULL
 *            only when mask_in is given (then nothing is written there).
 *  workspace device scratch of at least sla_workspace_bytes(p) bytes.
 * An empty critical set gives O_s = 0 for that query block, an empty marginal
 * set gives O_l = 0. Returns SLA_OK once all work is enqueued; SLA_ERR_ARG,
 * SLA_ERR_UNSUPPORTED or SLA_ERR_WORKSPACE before any enqueue; SLA_ERR_HIP if
 * a launch fails (sla_last_error() has the HIP message). Device faults surface
 * at the caller's next synchronisation of `stream`. */
int sla_forward(const sla_problem* p,
                const void* Q, const void* K, const void* V,
                const float* proj_q, const float* proj_k, const float* alpha,
                const int8_t* mask_in,
                void* O, int8_t* mask_out,
                void* workspace, size_t workspace_bytes,
                void* stream);

/* sla_forward plus the debug outputs of `dbg` (which may be NULL). */
int sla_forward_debug(const sla_problem* p,
                      const void* Q, const void* K, const void* V,
                      const float* proj_q, const float* proj_k, const float* alpha,
                      const int8_t* mask_in,
                      void* O, int8_t* mask_out,
                      void* workspace, size_t workspace_bytes,
                      void* stream, const sla_debug* dbg);

/* The SLA forward pass: as sla_forward, but the branches are fused as
 * O = O_s + Proj(O_l), Proj(x) = x proj_o (SLA paper summary, section 4,
 * step 4; SLA explainer, section 2.1 on the projection of its Eq. 6).
 *  proj_o    device float32, indexed [in, out], one [d, d] or [H, d, d] (see
 *            proj_head_stride); required. No bias term.
 * Every other argument is as for sla_forward; there is no alpha. Requires
 * quant == SLA_QUANT_NONE (SLA_ERR_UNSUPPORTED otherwise). The workspace size
 * is sla_workspace_bytes(p), as for sla_forward. */
int sla1_forward(const sla_problem* p,
                 const void* Q, const void* K, const void* V,
                 const float* proj_q, const float* proj_k, const float* proj_o,
                 const int8_t* mask_in,
                 void* O, int8_t* mask_out,
                 void* workspace, size_t workspace_bytes,
                 void* stream);

/* sla1_forward plus the debug outputs of `dbg` (which may be NULL); o_l then
 * receives Proj(O_l), the linear branch's term of the sum. */
int sla1_forward_debug(const sla_problem* p,
                       const void* Q, const void* K, const void* V,
                       const float* proj_q, const float* proj_k, const float* proj_o,
                       const int8_t* mask_in,
                       void* O, int8_t* mask_out,
                       void* workspace, size_t workspace_bytes,
                       void* stream, const sla_debug* dbg);

/* Bytes of device scratch that sla_forward_noalloc holds per GPU (160 MiB). */
#define SLA_NOALLOC_SCRATCH_BYTES (160u * 1024u * 1024u)

/* sla_forward without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation). Every argument is as for sla_forward. The
 * intermediate buffers live in a scratch array of SLA_NOALLOC_SCRATCH_BYTES
 * that the library holds on every GPU it is loaded on, until the process ends;
 * the current device's copy is used (the stream must belong to that device).
 * No device memory is allocated or freed by this call. Problems whose
 * workspace (sla_workspace_bytes) exceeds the scratch return SLA_ERR_WORKSPACE
 * before any work. All calls on one GPU share its scratch and it keeps the
 * last call's contents: calls that overlap on one GPU (two streams, or two
 * host threads) race and must be serialised by the caller. */
int sla_forward_noalloc(const sla_problem* p,
                        const void* Q, const void* K, const void* V,
                        const float* proj_q, const float* proj_k, const float* alpha,
                        const int8_t* mask_in,
                        void* O, int8_t* mask_out,
                        void* stream);

/* Workspace that sla_backward needs for `p` (host only, no device work).
 * Returns SLA_OK or the validation error sla_backward would return. */
int sla_backward_workspace_bytes(const sla_problem* p, size_t* bytes);

/* The SLA2 backward pass for a fixed block mask: the gradients of
 * sum(O * dO) with O = alpha O_s + (1 - alpha) O_l (SLA explainer, section 2.3:
 * the FlashAttention backward over the critical blocks and the chain rule
 * through phi(Q), phi(K) and V for the marginal ones, accumulated per block).
 *  Q, K, V   device, dtype, [B, H, N, d]: the forward pass's inputs.
 *  alpha     device float32 [H].
 *  mask      device int8 [B, H, Nb, Nb]: the forward pass's block mask (the
 *            mask is piecewise constant in Q and K: no gradient flows through
 *            the router, the pooling or the ranking, so proj_q / proj_k get none).
 *  dO        device, dtype, [B, H, N, d]: the gradient of the output.
 *  dQ, dK,   device float32 [B, H, N, d] outputs (rows past N untouched).
 *  dV
 *  dalpha    device float32 [H] output, summed over the batch.
 *  workspace device scratch of at least sla_backward_workspace_bytes(p) bytes.
 * Arithmetic: with bf16 inputs every product runs on bf16 matrix cores with
 * float32 accumulation (P, dS, phi and the linear-branch gradients rounded to
 * bf16); with float32 inputs, float32 throughout. Either feature map
 * (p->phi). Requires quant == SLA_QUANT_NONE (SLA_ERR_UNSUPPORTED otherwise).
 * Errors as for sla_forward. */
int sla_backward(const sla_problem* p,
                 const void* Q, const void* K, const void* V, const float* alpha,
                 const int8_t* mask, const void* dO,
                 float* dQ, float* dK, float* dV, float* dalpha,
                 void* workspace, size_t workspace_bytes,
                 void* stream);

/* Workspace that sla1_backward needs for `p` (host only, no device work): that
 * of sla_backward plus the parts of dproj_o before their float64 sum (bf16
 * inputs: O_l in bf16 and 512 d x d float32 parts, over consecutive row chunks,
 * with proj_o once in bf16; float32 inputs: one d x d float32 part per query
 * block) and 32 d x d float64 range sums per output map. */
int sla1_backward_workspace_bytes(const sla_problem* p, size_t* bytes);

/* The backward pass of the SLA formulation O = O_s + O_l proj_o (SLA paper
 * summary, section 4, step 4 and its final-output formula) for a fixed block
 * mask: dO_s = dO, dO_l = dO proj_o^T, and
 *  dproj_o   device float32 output of proj_o's shape ([d, d], or [H, d, d]
 *            with proj_head_stride = d*d): the sum over tokens of O_l^T dO,
 *            over the batch, and over the heads when proj_o is shared.
 *  proj_o    device float32 [d, d] or [H, d, d], indexed [in, out]; required.
 * Every other argument is as for sla_backward (there is no alpha or dalpha).
 * The router matrices get no gradient (the mask is held fixed). */
int sla1_backward(const sla_problem* p,
                  const void* Q, const void* K, const void* V, const float* proj_o,
                  const int8_t* mask, const void* dO,
                  float* dQ, float* dK, float* dV, float* dproj_o,
                  void* workspace, size_t workspace_bytes,
                  void* stream);

/* The training pair: a forward pass that keeps what the backward pass needs,
 * and a backward pass that takes it instead of running the forward again. The
 * sparse path's backward follows FlashAttention's (SLA explainer, section 2.3),
 * which takes the softmax normaliser that its forward saved; here the forward
 * also keeps O_s (for D_t = dO_s . O_s) and the linear branch's h_j, z_j, H_i
 * and Z_i.
 *
 * sla_forward_train / sla1_forward_train: as sla_forward / sla1_forward (same
 * arguments, same O and mask), with a workspace of at least
 * sla_backward_workspace_bytes(p) (sla1: sla1_backward_workspace_bytes(p))
 * bytes; on completion it holds, besides the forward's intermediates, O_s as
 * float32 and each query's log2 softmax normaliser over its critical keys.
 * Requires dtype == SLA_BF16 and quant == SLA_QUANT_NONE
 * (SLA_ERR_UNSUPPORTED otherwise).
 *
 * sla_backward_saved / sla1_backward_saved: as sla_backward / sla1_backward
 * (same arguments and outputs), reading that state from `workspace` instead of
 * recomputing it. The caller passes the workspace the forward_train call
 * filled, unmodified since, and the same Q, K, V, alpha (sla1: proj_o), mask
 * (mask_in, or the mask_out that call wrote) and the same B, H, N, d,
 * proj_head_stride, phi and linear_sums; the library cannot check that the
 * workspace holds that state, and anything else gives undefined gradients
 * (the reads stay inside the workspace). The results equal those of
 * sla_backward / sla1_backward for the same inputs. Requires dtype ==
 * SLA_BF16. The workspace may be reused for the next forward_train once the
 * backward has completed on `stream`. */
int sla_forward_train(const sla_problem* p,
                      const void* Q, const void* K, const void* V,
                      const float* proj_q, const float* proj_k, const float* alpha,
                      const int8_t* mask_in,
                      void* O, int8_t* mask_out,
                      void* workspace, size_t workspace_bytes,
                      void* stream);
int sla1_forward_train(const sla_problem* p,
                       const void* Q, const void* K, const void* V,
                       const float* proj_q, const float* proj_k, const float* proj_o,
                       const int8_t* mask_in,
                       void* O, int8_t* mask_out,
                       void* workspace, size_t workspace_bytes,
                       void* stream);
int sla_backward_saved(const sla_problem* p,
                       const void* Q, const void* K, const void* V, const float* alpha,
                       const int8_t* mask, const void* dO,
                       float* dQ, float* dK, float* dV, float* dalpha,
                       void* workspace, size_t workspace_bytes,
                       void* stream);
int sla1_backward_saved(const sla_problem* p,
                        const void* Q, const void* K, const void* V, const float* proj_o,
                        const int8_t* mask, const void* dO,
                        float* dQ, float* dK, float* dV, float* dproj_o,
                        void* workspace, size_t workspace_bytes,
                        void* stream);

/* SoftTop-k of the compressed attention map, the differentiable stand-in for
 * Eq. 2's top-k in SLA2's first training stage (SLA2 article, the two-stage
 * training paragraphs, stage 1: a sigmoid with a temperature; SLA2
 * cross-paper synthesis, section 3: a per-row threshold found by binary
 * search so that each row meets its budget). For each row of logits s:
 *   Pc = softmax(s),  out[j] = sigmoid((Pc[j] - lambda) / tau),
 *   lambda such that sum_j out[j] = k.
 *  logits  device float64 [rows, cols], row-major (for instance the logits
 *          of sla_forward_debug: rows = B*H*Nb, cols = Nb).
 *  k       the row budget in [0, cols]; n_h makes tau -> 0 the critical set.
 *  tau     temperature in Pc units, in [1e-20, 1e20].
 *  out     device float32 [rows, cols].
 *  lambda  device float32 [rows] or NULL: the thresholds (+inf where k = 0,
 *          -inf where k = cols, whose rows are all 0 or all 1).
 * Pc and the search are float32 (max and differences of the logits in
 * float64); the search halves a bracket on which the row sum crosses k until
 * its midpoint stops moving. Returns SLA_OK once enqueued; SLA_ERR_ARG (NULL
 * or misaligned pointers, rows < 1, cols outside [1, 4096], k or tau out of
 * range) before any work; SLA_ERR_HIP if the launch fails. */
int sla_soft_topk(const double* logits, int32_t rows, int32_t cols, double k, double tau,
                  float* out, float* lambda, void* stream);

/* Static text of a status code. */
const char* sla_status_str(int status);

/* Detail of the last non-OK return on the calling thread ("" if none). */
const char* sla_last_error(void);

/* Interface version: (major << 16) | minor (1.2 added sla_problem.linear_sums). */
int sla_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SLA_H */
