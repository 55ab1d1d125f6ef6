/*
 * kda.h — C ABI of libkda, Kimi Delta Attention (KDA) on AMD Instinct MI355X
 * (gfx950).
 *
 * What is computed
 * ----------------
 * One independent chain per (batch b, head h).  Row-vector convention: q_t and
 * k_t are rows of length dk, v_t a row of length dv, the state S is dk x dv.
 * For t = 0 .. T-1:
 *
 *     S'   = Diag(alpha_t) S              decay first, one gate per key channel
 *     r    = k_t S'                       read the state at the key
 *     u    = beta_t (v_t - r)             the delta
 *     S    = S' + k_t^T u                 write
 *     o_t  = q_t S                        read after the write, no normaliser
 *
 * i.e. S_t = (I - beta_t k_t^T k_t) Diag(alpha_t) S_{t-1} + beta_t k_t^T v_t.
 *
 * Sources, by page title and section:
 *   - "From GPT-2 to Kimi K3, Explained" (marvinlee.cn), section "DeltaNet
 *     (Fast Weight Programmers)": the read / delta / write / read step with a
 *     per-token write strength beta and no denominator;
 *   - same page, section "DeltaNet (Parallelizing Linear Transformers with
 *     Delta Rule)": the sequential prefill writes before it reads, the
 *     Householder reparameterisation, and the chunkwise form with a
 *     triangular (UT) transform that these kernels generalise;
 *   - same page, section "Gated Delta Net": a gate in [0,1] decays the old
 *     state before the precise write; 1 is plain DeltaNet, 0 clears memory;
 *   - same page, section "KDA/Kimi Linear", and "Kimi Delta Attention (KDA):
 *     что это за механизм внимания" (ai-flip.ru), section "Как KDA развивает
 *     идею Gated DeltaNet": the gate becomes one value per channel, a diagonal
 *     gate matrix.
 * Readings where the pages are silent: the gate scales the key dimension (the
 * rows of S) and acts before the read-back; the output reads the state after
 * the write; q and k are used exactly as given (no scaling, no feature map)
 * unless a *_logits call maps them; a missing initial state is zero.
 *
 * Conventions common to every entry point
 * ---------------------------------------
 *   - Every array argument is a DEVICE pointer owned by the caller, contiguous,
 *     row-major, and 16-byte aligned.  The library allocates nothing and keeps
 *     no mutable global state; calls are asynchronous on `stream` (an opaque
 *     hipStream_t; NULL means the null stream) and reentrant.
 *   - q, k, v and o have the element type `dt`; the states and beta (or its
 *     logit) are always float32.  The gate is float32 alpha per key channel
 *     (kda_prefill_chunked, kda_decode_step), a logit of type `dt` per key
 *     channel (the *_logits calls) or float32 per token and head (the
 *     kda_gdn_* calls).
 *   - Arguments are validated on the host before any launch; a failed
 *     validation returns a negative status and launches nothing.  A launch
 *     failure returns KDA_ERR_HIP.  Faults inside a kernel surface at the
 *     caller's next synchronisation.  No C++ exception crosses this ABI.
 *   - Supported sizes: dk, dv in {16, 32, 64, 128}.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t kda_status;

enum {
  KDA_OK = 0,
  KDA_ERR_NULL = -1,        /* a required pointer is NULL                          */
  KDA_ERR_SHAPE = -2,       /* a size is out of range (B, H, N < 1; T < 0)         */
  KDA_ERR_UNSUPPORTED = -3, /* dk, dv, C, dtype or q/k map not supported            */
  KDA_ERR_ALIGN = -4,       /* a pointer is not 16-byte aligned                    */
  KDA_ERR_ALIAS = -5,       /* an output overlaps an input it may not overlap      */
  KDA_ERR_WORKSPACE = -6,   /* workspace missing or smaller than the query says    */
  KDA_ERR_DEVICE = -7,      /* current device is not gfx950                        */
  KDA_ERR_HIP = -8,         /* a HIP runtime call or kernel launch failed          */
  KDA_ERR_SCRATCH = -9      /* sizes need more than the fixed device scratch of    */
                            /* kda_prefill_chunked_noalloc                         */
};

typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

/* Feature map the *_logits entry points apply to q and k, per token and head:
 *   KDA_QK_AS_GIVEN  q, k used as given
 *   KDA_QK_L2        x / max(||x||_2, 1e-12) over the head dimension
 *   KDA_QK_SILU_L2   the same after silu(x) = x * sigmoid(x); the SiLU
 *                    output is rounded to the I/O type before the norm
 * (the DeltaNet module on "22580: от GPT-2 до Kimi K3, объяснение", section
 * "DeltaNet, или Fast Weight Programmers", normalises silu(q) and silu(k)). */
typedef enum { KDA_QK_AS_GIVEN = 0, KDA_QK_L2 = 1, KDA_QK_SILU_L2 = 2 } kda_qk_map;

/*
 * kda_prefill_workspace_bytes — bytes of device workspace kda_prefill_chunked
 * needs for these sizes, or (size_t)-1 when the sizes are not supported.
 *
 * The library picks one of two paths from the sizes alone (the same choice in
 * this query and in the call):
 *   - few chains (B*H <= 128, when the chunk kernels fit on chip for these
 *     dk, dv, C, dt): a chunk-parallel kernel first writes one record per
 *     chunk to the workspace (the state-free chunk quantities W, Q.E,
 *     (K.E')^T, P, the chunk decay and Y diag(beta) V), then a scan kernel
 *     walks the chunks in order.  Long sequences go in segments of whole
 *     chunks (records of one segment at a time, at most 192 MiB unless one
 *     chunk of every chain is larger), with the fp32 state carried between
 *     segments.  With
 *       rec    = round_up((3*C*dk + C*C + C*dv) * sizeof(dt) + 4*dk, 256)
 *       nc     = ceil(T / C)
 *       runs   = floor(256 / (B*H))   (1 from 256 chains up)
 *       segmax = max(1, floor(192 MiB / (B*H*rec))), less its remainder
 *                mod runs when it exceeds runs
 *       nseg   = ceil(nc / segmax),  segch = ceil(nc / nseg), and when
 *                nseg > 1 rounded up to a multiple of runs (at most segmax)
 *     the workspace is B*H*segch*rec bytes, plus B*H*dk*dv*4 bytes of
 *     carried state when nseg > 1 (0 bytes when T = 0);
 *   - otherwise one fused kernel per (chain, value-column slab) keeps every
 *     intermediate on chip, and the query returns 0.
 */
size_t kda_prefill_workspace_bytes(int B, int T, int H, int dk, int dv, int C,
                                   kda_dtype dt);

/*
 * kda_prefill_chunked — KDA over a whole sequence for B x H chains, chunk by
 * chunk ("From GPT-2 to Kimi K3, Explained", section "DeltaNet (Parallelizing
 * Linear Transformers with Delta Rule)", generalised to the per-channel gate
 * of section "KDA/Kimi Linear").
 *
 *   q, k   [B, T, H, dk]  dt        queries and keys (used as given)
 *   v      [B, T, H, dv]  dt        values
 *   alpha  [B, T, H, dk]  float32   per-channel forget gate, expected in [0, 1]
 *   beta   [B, T, H]      float32   per-token write strength, expected in [0, 1]
 *   S0     [B, H, dk, dv] float32   initial state, or NULL for zeros
 *   o      [B, T, H, dv]  dt        output o_t = q_t S_t (written)
 *   S_T    [B, H, dk, dv] float32   final state (written), or NULL to skip;
 *                                   may be equal to S0 (in place) but may not
 *                                   overlap it otherwise
 *   C                               chunk length in {16, 32, 64, 128}; a
 *                                   performance knob only: the result does not
 *                                   depend on C beyond rounding.  C = 128 runs
 *                                   as two 64-token chunks (a 128-row chunk's
 *                                   tiles do not fit one CU's LDS), so its
 *                                   workspace and results are those of C = 64.
 *                                   With float32 q/k/v/o at dk = 128, C = 64
 *                                   (and so C = 128) is KDA_ERR_UNSUPPORTED:
 *                                   the fp32 tiles of a 64-token chunk do not
 *                                   fit beside each other; C = 16 and 32 run
 *   workspace, workspace_bytes      caller-owned device scratch of at least
 *                                   kda_prefill_workspace_bytes(...) bytes,
 *                                   16-byte aligned, overlapping no other
 *                                   argument (may be NULL when the query
 *                                   returns 0).  Its contents are overwritten
 *                                   and carry nothing between calls; two
 *                                   calls in flight at once need two
 *                                   workspaces.
 *
 * Any T >= 0 is accepted; a tail shorter than C is handled as identity
 * padding (gate 1, strength 0), and T = 0 copies S0 (or zeros) to S_T.
 * o may not overlap any input.  Errors: KDA_ERR_NULL, KDA_ERR_SHAPE,
 * KDA_ERR_UNSUPPORTED, KDA_ERR_ALIGN, KDA_ERR_ALIAS, KDA_ERR_WORKSPACE (NULL
 * or smaller than the query when one is needed), KDA_ERR_DEVICE, KDA_ERR_HIP.
 */
kda_status kda_prefill_chunked(const void* q, const void* k, const void* v,
                               const float* alpha, const float* beta,
                               const float* S0, void* o, float* S_T,
                               int B, int T, int H, int dk, int dv, int C,
                               kda_dtype dt, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * kda_prefill_chunked_noalloc — kda_prefill_chunked for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  It takes no workspace; it allocates
 * nothing and calls no allocating routine.
 *
 * Where kda_prefill_chunked needs a workspace (the chunk-record path), this
 * call uses a device array inside the library instead: 64 MiB, one copy per
 * GPU, held until the process ends.  It splits the sequence into more
 * segments than kda_prefill_chunked may use, so that one segment's records
 * plus the carried state (B*H*dk*dv*4 bytes) fit that array.  The results
 * are bit-identical to kda_prefill_chunked's for the same arguments.
 *
 * Every call on a GPU shares that GPU's array.  Nothing in it needs clearing
 * between calls, but calls that overlap in time on one GPU (two streams, two
 * threads) race on it and must not be issued.
 *
 * Arguments, layouts and the other errors are those of kda_prefill_chunked,
 * without workspace and workspace_bytes.  KDA_ERR_SCRATCH: the sizes need
 * more than the array holds (only when one chunk of every chain plus the
 * carried state exceeds 64 MiB, which no size the chunk-record path accepts
 * reaches at dk, dv <= 128).
 */
kda_status kda_prefill_chunked_noalloc(const void* q, const void* k, const void* v,
                                       const float* alpha, const float* beta,
                                       const float* S0, void* o, float* S_T,
                                       int B, int T, int H, int dk, int dv, int C,
                                       kda_dtype dt, void* stream);

/*
 * kda_prefill_chunked_logits — kda_prefill_chunked with the input prologue
 * fused into its kernels: the caller passes raw projections and every
 * transform below runs on chip, in fp32, as each chunk is loaded.
 *
 *   q, k   [B, T, H, dk]  dt        raw queries and keys, mapped by qk_map
 *   v      [B, T, H, dv]  dt        values
 *   g      [B, T, H, dk]  dt        gate logits: alpha = exp(-softplus(g))
 *                                   = 1 / (1 + e^g), in (0, 1) for every
 *                                   real g (+inf gives 0, -inf gives 1)
 *   b      [B, T, H]      float32   write-strength logits: beta = sigmoid(b)
 *   qk_map                          KDA_QK_AS_GIVEN, KDA_QK_L2 or
 *                                   KDA_QK_SILU_L2 (see kda_qk_map)
 *   all other arguments as kda_prefill_chunked, including the workspace
 *   (kda_prefill_workspace_bytes gives its size; the records are the same)
 *
 * The result equals kda_prefill_chunked on alpha = exp(-softplus(g)), beta =
 * sigmoid(b) and the mapped q, k, up to rounding.  The gate is read at the
 * I/O type's width (bf16: 2 bytes instead of 4 per key channel and token).
 * Sources: the module on "22580: от GPT-2 до Kimi K3, объяснение", section
 * "DeltaNet, или Fast Weight Programmers" (SiLU, L2 norm, sigmoid strength);
 * the gate must lie in [0, 1] ("From GPT-2 to Kimi K3, Explained", section
 * "Gated Delta Net"), which exp(-softplus(g)) guarantees.
 * Errors: as kda_prefill_chunked; an unknown qk_map is KDA_ERR_UNSUPPORTED.
 */
kda_status kda_prefill_chunked_logits(const void* q, const void* k, const void* v,
                                      const void* g, const float* b, const float* S0,
                                      void* o, float* S_T, int B, int T, int H, int dk,
                                      int dv, int C, kda_dtype dt, kda_qk_map qk_map,
                                      void* workspace, size_t workspace_bytes,
                                      void* stream);

/*
 * kda_gdn_prefill_chunked — the same chunked prefill with one forget gate
 * per token and head instead of one per key channel: Gated DeltaNet, the
 * rule KDA refines ("From GPT-2 to Kimi K3, Explained", sections "Gated
 * Delta Net" and "KDA/Kimi Linear"), or, with a = NULL, DeltaNet (gate 1,
 * section "DeltaNet (Fast Weight Programmers)").
 *
 *   a      [B, T, H]      float32   gate per token and head, expected in
 *                                   [0, 1], or NULL for a = 1
 *   all other arguments, the workspace query and the errors as
 *   kda_prefill_chunked
 *
 * The result equals kda_prefill_chunked with alpha[b,t,h,:] = a[b,t,h] on
 * every channel, up to rounding.  The gate costs 4 bytes per token and head
 * (0 with NULL) instead of 4*dk.
 */
kda_status kda_gdn_prefill_chunked(const void* q, const void* k, const void* v,
                                   const float* a, const float* beta, const float* S0,
                                   void* o, float* S_T, int B, int T, int H, int dk, int dv,
                                   int C, kda_dtype dt, void* workspace,
                                   size_t workspace_bytes, void* stream);

/*
 * kda_decode_step — one recurrence step for N sequences x H heads (the same
 * step as one token of the prefill; the pages' decode path calls the layer
 * with t = 1 and the cached state, "From GPT-2 to Kimi K3, Explained",
 * sections "Linear Attention" and "DeltaNet (Fast Weight Programmers)").
 *
 *   q, k   [N, H, dk]      dt
 *   v      [N, H, dv]      dt
 *   alpha  [N, H, dk]      float32
 *   beta   [N, H]          float32
 *   S_in   [N, H, dk, dv]  float32  state before the step
 *   o      [N, H, dv]      dt       output (written); may not overlap inputs
 *   S_out  [N, H, dk, dv]  float32  state after the step (written); may be
 *                                   equal to S_in (in place) but may not
 *                                   overlap it otherwise
 *
 * Errors: as kda_prefill_chunked (no workspace).
 */
kda_status kda_decode_step(const void* q, const void* k, const void* v,
                           const float* alpha, const float* beta,
                           const float* S_in, void* o, float* S_out,
                           int N, int H, int dk, int dv, kda_dtype dt,
                           void* stream);

/*
 * kda_decode_step_logits — kda_decode_step with the input prologue of
 * kda_prefill_chunked_logits fused in: q, k [N, H, dk] raw (mapped by
 * qk_map), g [N, H, dk] gate logits of type dt, b [N, H] float32
 * write-strength logits; all other arguments as kda_decode_step.  One call
 * is exactly one token of kda_prefill_chunked_logits.
 * Errors: as kda_decode_step; an unknown qk_map is KDA_ERR_UNSUPPORTED.
 */
kda_status kda_decode_step_logits(const void* q, const void* k, const void* v,
                                  const void* g, const float* b, const float* S_in,
                                  void* o, float* S_out, int N, int H, int dk, int dv,
                                  kda_dtype dt, kda_qk_map qk_map, void* stream);

/*
 * kda_gdn_decode_step — one Gated DeltaNet step (kda_decode_step with the
 * gate a [N, H] float32 the same on every key channel, or NULL for DeltaNet);
 * exactly one token of kda_gdn_prefill_chunked.  Errors: as kda_decode_step.
 */
kda_status kda_gdn_decode_step(const void* q, const void* k, const void* v, const float* a,
                               const float* beta, const float* S_in, void* o, float* S_out,
                               int N, int H, int dk, int dv, kda_dtype dt, void* stream);

/*
 * kda_decode_step_backward — the adjoint of kda_decode_step: given the
 * gradients of a loss L with respect to the step's output and new state,
 * the gradients with respect to every input of the step.  Applied backwards
 * over a sequence's tokens (with the state before each token), it gives the
 * exact gradient of a prefill or of a run of decode steps.  The forward step
 * is that of "From GPT-2 to Kimi K3, Explained", sections "DeltaNet (Fast
 * Weight Programmers)" and "KDA/Kimi Linear"; the adjoint is its chain rule:
 * with S' = Diag(alpha) S_in, r = k S', u = beta (v - r) and
 * G = dS_new + q^T dO,
 *     dq = (S' + k^T u) dO^T        dk = G u^T - beta S' (k G)^T
 *     dv = beta k G                 dbeta = (k G) . (v - r)
 *     dalpha = rowsum((G - beta k^T (k G)) * S_in)
 *     dS = Diag(alpha) (G - beta k^T (k G))
 *
 *   q, k, v, alpha, beta, S_in   the step's inputs, as kda_decode_step
 *   dO      [N, H, dv]      dt        dL/do
 *   dS_new  [N, H, dk, dv]  float32   dL/dS after the step
 *   dq, dk  [N, H, dk]      dt        written
 *   dv      [N, H, dv]      dt        written
 *   dalpha  [N, H, dk]      float32   written
 *   dbeta   [N, H]          float32   written
 *   dS      [N, H, dk, dv]  float32   dL/dS_in (written); may be equal to
 *                                     dS_new (in place) but may not overlap
 *                                     it otherwise
 *
 * Every pointer is required.  No output may overlap an input or another
 * output (dS == dS_new aside).  Errors: KDA_ERR_NULL, KDA_ERR_SHAPE,
 * KDA_ERR_UNSUPPORTED, KDA_ERR_ALIGN, KDA_ERR_ALIAS, KDA_ERR_DEVICE,
 * KDA_ERR_HIP.
 */
kda_status kda_decode_step_backward(const void* q, const void* k, const void* v,
                                    const float* alpha, const float* beta, const float* S_in,
                                    const void* dO, const float* dS_new, void* dq, void* dk,
                                    void* dv, float* dalpha, float* dbeta, float* dS, int N,
                                    int H, int dk_, int dv_, kda_dtype dt, void* stream);

/*
 * kda_prefill_backward_workspace_bytes — device workspace, in bytes, that
 * kda_prefill_backward needs for these sizes: the state of every sequence
 * and head stored once every 16 tokens, B * H * ceil(T / 16) * dk * dv * 4
 * bytes, and every token's write and read per value column, 2 * B * T * H *
 * dv * 4 bytes (320 MiB at B = 1, T = 4096, H = 16, dk = dv = 128).
 * (size_t)-1 for sizes the call does not accept.
 */
size_t kda_prefill_backward_workspace_bytes(int B, int T, int H, int dk, int dv);

/*
 * kda_prefill_backward — the gradients of a loss L through a whole
 * kda_prefill_chunked call: given dL/do for every token and dL/dS_T for
 * the final state, the gradients with respect to q, k, v, alpha, beta and
 * the initial state.  It is kda_decode_step_backward applied from the last
 * token to the first, each time at the state before that token, with the
 * state gradient carried from token to token (the chain rule of the
 * recurrence of "From GPT-2 to Kimi K3, Explained", sections "DeltaNet
 * (Fast Weight Programmers)" and "KDA/Kimi Linear").  The states are
 * recomputed from S0: one forward pass stores them every 16 tokens in the
 * workspace, with each token's write and read, and each 16-token piece's
 * states are rebuilt from them before its backward.
 *
 *   q, k, v, alpha, beta, S0   the prefill's inputs, as kda_prefill_chunked
 *                              (S0 may be NULL: zeros)
 *   dO      [B, T, H, dv]  dt       dL/do
 *   dS_T    [B, H, dk, dv] float32  dL/dS_T, or NULL (zeros)
 *   dq, dk  [B, T, H, dk]  float32  written
 *   dv      [B, T, H, dv]  float32  written
 *   dalpha  [B, T, H, dk]  float32  written
 *   dbeta   [B, T, H]      float32  written
 *   dS0     [B, H, dk, dv] float32  dL/dS0, written unless NULL; may be
 *                                   equal to dS_T (in place) but may not
 *                                   overlap it otherwise
 *   workspace, workspace_bytes      at least
 *                                   kda_prefill_backward_workspace_bytes
 *
 * Gradients are float32 whatever dt is; dq, dk, dalpha and dbeta are sums
 * over value-column slabs taken with float atomics, so their last bits may
 * differ from run to run.  T = 0 writes dS0 = dS_T (or zeros).  No output
 * or the workspace may overlap an input or another output (dS0 == dS_T
 * aside).  Errors: KDA_ERR_NULL, KDA_ERR_SHAPE, KDA_ERR_UNSUPPORTED,
 * KDA_ERR_ALIGN, KDA_ERR_ALIAS, KDA_ERR_WORKSPACE, KDA_ERR_DEVICE,
 * KDA_ERR_HIP.
 */
kda_status kda_prefill_backward(const void* q, const void* k, const void* v,
                                const float* alpha, const float* beta, const float* S0,
                                const void* dO, const float* dS_T, float* dq, float* dk,
                                float* dv, float* dalpha, float* dbeta, float* dS0, int B,
                                int T, int H, int dk_, int dv_, kda_dtype dt, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * kda_prefill_backward_chunked_workspace_bytes — device workspace, in bytes,
 * that kda_prefill_backward_chunked needs: the forward's split-path records
 * (kda_prefill_workspace_bytes at C = 64 with the split path), the state and
 * the state gradient at every 64-token chunk boundary
 * (2 * B * H * ceil(T / 64) * dk * dv * 4 bytes), one
 * 15 KiB record per 16 tokens of every sequence and head, and, per 64-token
 * chunk, the states at its four 16-token blocks and their writes (bf16:
 * 4 * dk * dv * 2 + 64 * dv * 2 bytes) that the gradient pass rebuilds
 * (about 404 MiB at B = 1, H = 16, T = 4096).  (size_t)-1 for
 * sizes the call does not accept (dk or dv other than 128).
 */
size_t kda_prefill_backward_chunked_workspace_bytes(int B, int T, int H, int dk, int dv);

/*
 * kda_prefill_backward_chunked — the gradients of kda_prefill_backward in
 * chunk form on the matrix cores, for bf16 I/O at dk = dv = 128: the chunk
 * algebra of "From GPT-2 to Kimi K3, Explained", section "DeltaNet
 * (Parallelizing Linear Transformers with Delta Rule)", with the per-channel
 * decay of section "KDA/Kimi Linear", differentiated.  The state gradient
 * runs backwards over 16-token sub-chunks through their WY factors; every
 * other gradient is local to a sub-chunk given its start state (from a
 * forward pass that stores the state every 64 tokens) and its end state
 * gradient, with the pairwise decays taken exactly as running products of
 * alpha (closed gates, alpha = 0, included).  Operands are bf16 with fp32
 * accumulation, so the results carry bf16-level rounding (relative error
 * around 3e-3, against the fp32 rounding of kda_prefill_backward); every
 * element is written once, with no atomics, so repeated calls agree bit
 * for bit.
 *
 * Arguments, layouts, T = 0, dS0 == dS_T and the errors are those of
 * kda_prefill_backward, with the workspace of
 * kda_prefill_backward_chunked_workspace_bytes; dt must be KDA_BF16 and
 * dk = dv = 128 (else KDA_ERR_UNSUPPORTED).
 *
 * Streams: when B * H * dv / 16 <= 128 the state-gradient half runs on a
 * second stream of the library's own (one per device, default priority,
 * created on the first such call and kept until the process ends), forked
 * from `stream` by an event at the start of the call and joined back into it
 * before the last kernel, so all of the call's work is ordered on `stream`
 * as usual.  Calls from several host threads are serialised while they
 * enqueue.  A call made while `stream` is being captured into a graph, or
 * one for which the second stream cannot be created, runs in order on
 * `stream` alone (same results, bit for bit).
 */
kda_status kda_prefill_backward_chunked(const void* q, const void* k, const void* v,
                                        const float* alpha, const float* beta, const float* S0,
                                        const void* dO, const float* dS_T, float* dq, float* dk,
                                        float* dv, float* dalpha, float* dbeta, float* dS0,
                                        int B, int T, int H, int dk_, int dv_, kda_dtype dt,
                                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * kda_gdn_decode_step_backward — kda_decode_step_backward for Gated
 * DeltaNet and DeltaNet (the step of kda_gdn_decode_step): the gate a [N, H]
 * float32 is one value per head, or NULL (gate 1).  Its gradient da [N, H]
 * float32 is the sum over the key channels of the per-channel one; da is
 * written when both a and da are given, and ignored otherwise.  Every other
 * argument and the errors are those of kda_decode_step_backward.
 */
kda_status kda_gdn_decode_step_backward(const void* q, const void* k, const void* v,
                                        const float* a, const float* beta, const float* S_in,
                                        const void* dO, const float* dS_new, void* dq, void* dk,
                                        void* dv, float* da, float* dbeta, float* dS, int N,
                                        int H, int dk_, int dv_, kda_dtype dt, void* stream);

/*
 * kda_gdn_prefill_backward — kda_prefill_backward for Gated DeltaNet and
 * DeltaNet (the recurrence of kda_gdn_prefill_chunked): the gate a [B, T, H]
 * float32 is one value per token and head, the same on every key channel,
 * or NULL for DeltaNet (gate 1).  Its gradient da [B, T, H] float32 is the
 * sum over the key channels of the per-channel one; da is written when both
 * a and da are given, and ignored otherwise.  Every other argument, the
 * workspace and the errors are those of kda_prefill_backward.
 */
kda_status kda_gdn_prefill_backward(const void* q, const void* k, const void* v, const float* a,
                                    const float* beta, const float* S0, const void* dO,
                                    const float* dS_T, float* dq, float* dk, float* dv,
                                    float* da, float* dbeta, float* dS0, int B, int T, int H,
                                    int dk_, int dv_, kda_dtype dt, void* workspace,
                                    size_t workspace_bytes, void* stream);

/*
 * kda_prologue_forward — the input prologue of kda_prefill_chunked_logits on
 * its own, for training from raw projections: per row (one token of one
 * head) alpha = 1 / (1 + e^g) per key channel, beta = sigmoid(b), and q, k
 * mapped by qk_map, written out as the inputs of kda_prefill_chunked and
 * kda_prefill_backward.  The gate form keeps every logit inside (0, 1) as
 * "From GPT-2 to Kimi K3, Explained", section "Gated Delta Net", requires;
 * SiLU, the L2 map and the sigmoid follow "22580: от GPT-2 до Kimi K3,
 * объяснение", section "DeltaNet, или Fast Weight Programmers".
 *
 *   q, k, g   [rows, dk]  dt       raw queries, keys and gate logits
 *   b         [rows]      float32  raw write-strength logits
 *   q_hat, k_hat [rows, dk] dt     mapped queries and keys (written)
 *   alpha     [rows, dk]  float32  written
 *   beta      [rows]      float32  written
 *
 * rows = B*T*H for [B,T,H,dk] arrays (any row-major leading shape).
 * rows = 0 does nothing.  Errors: KDA_ERR_NULL, KDA_ERR_SHAPE (rows < 0),
 * KDA_ERR_UNSUPPORTED (dk, dt or qk_map), KDA_ERR_ALIGN, KDA_ERR_ALIAS (an
 * output overlapping an input or another output), KDA_ERR_DEVICE,
 * KDA_ERR_HIP.
 */
kda_status kda_prologue_forward(const void* q, const void* k, const void* g, const float* b,
                                void* q_hat, void* k_hat, float* alpha, float* beta, int rows,
                                int dk, kda_dtype dt, kda_qk_map qk_map, void* stream);

/*
 * kda_prologue_backward — the adjoint of kda_prologue_forward: from the
 * gradients with respect to its outputs (as kda_prefill_backward returns
 * them) to those with respect to the raw inputs.  The chain rule of the
 * forward maps:
 *     dg = -dalpha alpha (1 - alpha),   db = dbeta beta (1 - beta)
 *     L2 map, y = x / max(||x||, 1e-12):
 *         dx = (dy - y (y . dy)) / ||x||   (dy / 1e-12 on the floor)
 *     SiLU:  dq = dx sigmoid(q) (1 + q (1 - sigmoid(q)))
 *
 *   q, k, g, b                 the raw inputs, as kda_prologue_forward
 *   dq_hat, dk_hat, dalpha [rows, dk], dbeta [rows]   float32
 *   dq, dk, dg [rows, dk], db [rows]                  float32, written
 *
 * Errors: as kda_prologue_forward.
 */
kda_status kda_prologue_backward(const void* q, const void* k, const void* g, const float* b,
                                 const float* dq_hat, const float* dk_hat, const float* dalpha,
                                 const float* dbeta, float* dq, float* dk, float* dg, float* db,
                                 int rows, int dk_, kda_dtype dt, kda_qk_map qk_map,
                                 void* stream);

/* kda_status_string — static, human-readable text for a status code. */
const char* kda_status_string(kda_status s);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
