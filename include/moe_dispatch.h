/*
 * moe_dispatch.h -- C ABI of the dropless Mixture-of-Experts layer hot path
 * for AMD Instinct MI355X (gfx950).
 *
 * The layer (token-choice top-K routing, SwiGLU experts):
 *   z      = x Wg^T (+ b)                          router logits, [T,E]
 *   S_t    = TopK(z_t), w_t = softmax over z_t[S_t] (renormalised top-K weights)
 *   a, b   = x_t W_gate[e]^T, x_t W_up[e]^T        per assignment (t, e in S_t)
 *   y      = SiLU(a) * b,  SiLU(u) = u * sigmoid(u)
 *   out_t  = sum_k w_{t,k} * y_{t,k} W_down[e_k]^T
 * with the backward pass of L = <dY, out>, recomputing SiLU from the saved
 * pre-activations.
 *
 * Sources:
 *   MoEBlaze reading notes (papercache.org), sec. 2.1 (gating network:
 *     TopK(softmax(W_g x)), W_g in R^{E x d}), sec. 2.3 (weighted output
 *     aggregation), sec. 4.1 and Figure 2 (the index structures), sec. 5.2
 *     Algorithm 1 (fused SwiGLU MoE training: forward stores A, B, Y_swi;
 *     backward recomputes SiLU(A)).
 *   "MoEBlaze: Breaking the Memory Wall for Efficient MoE Training on Modern
 *     GPUs" (paper-graph-ui analysis page): "Memory-Efficient Token Routing:
 *     Forward Pass / Backward Pass", "Dispatch Data Structures:
 *     Specification and Roles", "Dispatch Data Structure Construction: The
 *     Atomic-Free Three-Step Algorithm", "Fused SwiGLU Kernel with
 *     Activation Checkpoint".
 *   "SonicMoE: Accelerating MoE with IO and Tile-aware Optimizations"
 *     (paper-graph-ui analysis page), sec. 3.4.1 (dS = <dA', A>, dA = s*dA').
 *   "Dropless MoE, in depth" (aicassindra.com), "A reference implementation"
 *     (renormalised top-K weights; counts stay on the device).
 *
 * Conventions for every entry point
 *   - Pointers are DEVICE pointers unless marked "host".  The caller owns all
 *     memory, including the workspace; the library never allocates, frees or
 *     keeps a pointer after the call returns.
 *   - Every call only enqueues work on `stream` (a hipStream_t; NULL = the
 *     default stream).  No device-to-host copy, no synchronisation, and no
 *     launch size depends on the routing, so a call sequence can be captured
 *     into a HIP graph.  Results are valid once the stream has completed.
 *   - Layouts are row-major.  Activations x, dY, out, dX: [T,d].  Router
 *     weight Wg: [E,d].  Expert weights in [out,in] layout per expert:
 *     W_gate, W_up: [E,h,d]; W_down: [E,d,h].  Weight gradients are fp32 in
 *     the same layouts.  Activations and expert weights use moe_shape.dtype
 *     (bf16 or fp32); router logits and top-K weights are fp32; index arrays
 *     are int32.
 *   - Return value: a moe_status.  Arguments are validated on the host
 *     before anything is enqueued; on MOE_ERR_INVALID_ARG, _UNSUPPORTED or
 *     _WORKSPACE nothing has been enqueued.  MOE_ERR_HIP reports a failed
 *     launch (hipGetLastError after the enqueue).
 *   - Workspaces hold no state between calls; size them with
 *     moe_workspace_bytes, which depends on the shape only (never on the
 *     routing, so skewed routing cannot exhaust it).
 *   - One workspace may serve moe_expert_fwd, moe_combine and
 *     moe_expert_bwd of the same shape (their layouts share a prefix and no
 *     call reads what an earlier one left there), sized as the largest of
 *     MOE_WS_EXPERT_FWD, MOE_WS_COMBINE and MOE_WS_EXPERT_BWD(_H, _LEAN).  Calls
 *     that share a workspace must not overlap in time (enqueue them on one
 *     stream, or order their streams).
 *   - Device error words (int32, in the workspace): bytes 0-3 belong to
 *     moe_combine, bytes 4-7 to moe_expert_bwd.  Each call clears its own at
 *     its start and leaves the other's, so after a forward and a backward
 *     through a shared workspace both are readable.  A word is nonzero when
 *     a bounded wait of that call's ordered fold ran out (moe_set_spin_limit):
 *     the call still returns MOE_OK, because it only enqueues work and the
 *     wait happens later on the device, but its output (out or dx) is then
 *     NOT valid.  A caller must read the word after the stream completes
 *     before trusting out / dx.
 *   - Supported shapes: 1 <= K <= min(E, 32), E <= 1024, T*K < 2^31,
 *     d and h multiples of 128, and under 2 GiB each for x [T,d], one
 *     expert's weight matrix [h,d] and T rows of the saved pre-activations
 *     [T, 2h] (2h -> h for the plain experts) in the activation dtype (the
 *     kernels address them with 32-bit offsets); otherwise
 *     MOE_ERR_UNSUPPORTED.  (Multiples of 128, where multiples of 8 would
 *     satisfy the 16-byte row alignment: the expert GEMM tiles are 128 or
 *     256 wide and have no masked column tail for d; h is masked per
 *     128-column block.)  Device pointers 16-byte aligned.
 */
#ifndef MOE_DISPATCH_H
#define MOE_DISPATCH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,   /* null required pointer, bad size, K > E, misaligned pointer */
  MOE_ERR_UNSUPPORTED = 2,   /* shape or dtype outside what the kernels cover */
  MOE_ERR_WORKSPACE = 3,     /* workspace smaller than moe_workspace_bytes */
  MOE_ERR_HIP = 4            /* a kernel launch failed */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Expert feed-forward kind.
 *   MOE_ACT_SWIGLU: gated, y = SiLU(x W_gate^T) * (x W_up^T) (MoEBlaze
 *     analysis page, "Fused SwiGLU Kernel with Activation Checkpoint").
 *   MOE_ACT_SILU / MOE_ACT_RELU: the plain two-layer expert
 *     E_i(x) = W_2 sigma(W_1 x) of the MoEBlaze reading notes (sec. 2.2),
 *     sigma = SiLU or ReLU.  W_1 is passed as w_gate; there is no w_up (pass
 *     NULL) and no dw_up; the saved pre-activation h_ab holds a = x W_1^T
 *     only ([T*K, h] instead of [T*K, 2h]). */
typedef enum { MOE_ACT_SWIGLU = 0, MOE_ACT_SILU = 1, MOE_ACT_RELU = 2 } moe_act;

/* host struct: T tokens, model dim d, E experts, top-K, expert hidden h */
typedef struct {
  int32_t T, d, E, K, h;
  int32_t dtype; /* moe_dtype of activations and expert weights */
  int32_t act;   /* moe_act; 0 (SwiGLU) for a zero-initialised struct */
} moe_shape;

typedef enum {
  MOE_WS_INDEX = 0,       /* moe_build_index */
  MOE_WS_EXPERT_FWD = 1,  /* moe_expert_fwd */
  MOE_WS_COMBINE = 2,     /* moe_combine */
  MOE_WS_EXPERT_BWD = 3,  /* moe_expert_bwd with the saved y_swi */
  MOE_WS_EXPERT_BWD_H = 4, /* moe_expert_bwd with y_swi == NULL (H-only saving):
                              MOE_WS_EXPERT_BWD plus a [T*K, h] dtype buffer */
  MOE_WS_COMBINE_STAGED = 5, /* moe_combine_staged: holds a [T*K, d] dtype buffer */
  MOE_WS_INDEX_DENSE = 6,    /* moe_build_index_dense: two [E, T] int32 maps */
  MOE_WS_EXPERT_BWD_LEAN = 7 /* moe_expert_bwd with dh given (and a_prime given under
                                H-only saving): MOE_WS_EXPERT_BWD without its
                                [T*K, 2h] (plain experts: [T*K, h]) dtype dH buffer */
} moe_workspace_kind;

/* Bytes of device workspace the call of kind `which` needs for shape *s
 * (host pointer).  Returns 0 for an invalid shape or kind. */
size_t moe_workspace_bytes(const moe_shape* s, int which);

/* Router (MoEBlaze reading notes sec. 2.1; Dropless MoE in depth, "A reference
 * implementation").
 *   x != NULL: logits[T,E] (fp32, output) = x Wg^T (+ bias), fp32 accumulation.
 *   x == NULL: logits[T,E] is an INPUT (routing from given logits); wg and
 *              bias are ignored.
 *   topk_ids[T,K] (int32, output): the K largest logits of each token, in
 *     descending order; ties go to the lower expert id.  This array is the
 *     token_expert_indices structure of the index.
 *   topk_w[T,K] (fp32, output): softmax of the chosen K logits, i.e. the
 *     softmax probabilities renormalised over the chosen experts.
 *   bias[E] (fp32, nullable): fixed per-expert logit offset.
 * The selection and the weights are computed from the fp32 logits as written,
 * so routing from x and routing from the logits it wrote give the same ids
 * and weights bit for bit. */
int moe_route_topk(const moe_shape* s, const void* x, const void* wg, const float* bias, float* logits,
                   int32_t* topk_ids, float* topk_w, void* stream);

/* Routing index by counting sort, without a global sort or atomics
 * (MoEBlaze analysis page, "Dispatch Data Structures" and "Dispatch Data
 * Structure Construction"; MoEBlaze reading notes sec. 4.1, Figure 2).
 *   topk_ids[T*K]: input (token_expert_indices).  Every entry must lie in
 *     [0, E) and a token's K entries must be distinct, as moe_route_topk
 *     writes them; the ids live on the device and are not checked, and other
 *     values give undefined results.
 *   offsets[E+1] (output): expert_token_offsets, offsets[E] = T*K.
 *   expert_token_indices[T*K] (output): token ids grouped by ascending
 *     expert, ascending token id within an expert.
 *   token_index_map[T*K] (output): entry t*K+k is the position of
 *     (t, topk_ids[t,k]) in expert_token_indices.
 * Bit-exact and deterministic.  ws: MOE_WS_INDEX workspace. */
int moe_build_index(const moe_shape* s, const int32_t* topk_ids, int32_t* offsets, int32_t* expert_token_indices,
                    int32_t* token_index_map, void* ws, size_t ws_bytes, void* stream);

/* moe_build_index without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture that must not
 * allocate, tight serving loops, harnesses that forbid hipMalloc).  Same
 * arguments (minus ws), outputs and errors as moe_build_index; the index
 * workspace lives in a static device array of the library, one per GPU,
 * MOE_NOALLOC_INDEX_MAX_BYTES long (about 0.14 * T * E bytes are needed:
 * e.g. T = 32768 with E = 1024), held until the process ends.  A shape whose
 * MOE_WS_INDEX workspace is larger returns MOE_ERR_WORKSPACE before anything
 * is enqueued.  The call allocates nothing (no hipMalloc, no library
 * allocation); its first call on a device looks up that device's copy of the
 * array.  Every call on a GPU shares that GPU's array: calls that overlap in
 * time on one GPU (other streams, other threads) race and give undefined
 * results; calls ordered on one stream are fine. */
#define MOE_NOALLOC_INDEX_MAX_BYTES (8u << 20)
int moe_build_index_noalloc(const moe_shape* s, const int32_t* topk_ids, int32_t* offsets,
                            int32_t* expert_token_indices, int32_t* token_index_map, void* stream);

/* The same routing index, built by MoEBlaze's three steps taken literally
 * (MoEBlaze analysis page, "Dispatch Data Structure Construction: The
 * Atomic-Free Three-Step Algorithm"): a dense token-expert map [E][T]
 * (token id or -1), one workgroup per expert to count its column, an
 * exclusive scan of the lengths, one workgroup per expert for the tile-level
 * scan that gives each entry its position (the location map), and a final
 * conflict-free scatter.  Same arguments, outputs and errors as
 * moe_build_index, and the same arrays bit for bit; the workspace
 * (MOE_WS_INDEX_DENSE) grows as T*E.  An alternate backend for comparison. */
int moe_build_index_dense(const moe_shape* s, const int32_t* topk_ids, int32_t* offsets,
                          int32_t* expert_token_indices, int32_t* token_index_map, void* ws, size_t ws_bytes,
                          void* stream);

/* Gate/up grouped GEMM with the SwiGLU epilogue, gathering x rows in place
 * through expert_token_indices (MoEBlaze analysis page, "Fused SwiGLU Kernel
 * with Activation Checkpoint"; reading notes Algorithm 1 forward).  For each
 * position p of expert e (offsets[e] <= p < offsets[e+1]), t = eti[p]:
 *   h_ab[p, 0:h]  = a = x[t] W_gate[e]^T     (rounded to dtype)
 *   h_ab[p, h:2h] = b = x[t] W_up[e]^T       (rounded to dtype)
 *   y_swi[p, :]   = SiLU(a) * b, from the unrounded fp32 a and b.
 * h_ab: [T*K, 2h], y_swi: [T*K, h], both dtype, outputs (h_ab, and y_swi
 * unless the backward takes the H-only path, are saved for the backward).
 * h_ab may be NULL for a forward that no moe_expert_bwd follows: then
 * nothing is stored but y_swi, which moe_combine reads.  No permuted copy of
 * x is made.  ws: MOE_WS_EXPERT_FWD. */
int moe_expert_fwd(const moe_shape* s, const void* x, const int32_t* offsets, const int32_t* expert_token_indices,
                   const void* w_gate, const void* w_up, void* h_ab, void* y_swi, void* ws, size_t ws_bytes,
                   void* stream);

/* Down-projection grouped GEMM whose epilogue does the weighted combine
 * through the reverse index (MoEBlaze analysis page, "On-the-Fly Output
 * Aggregation"; reading notes sec. 2.3):
 *   out[t] = sum_k topk_w[t,k] * y_swi[token_index_map[t*K+k]] W_down[e_k]^T.
 * No float atomics and no [T*K, d] buffer: each output row block receives its
 * K contributions in ascending expert order through integer turn counters,
 * accumulating in an fp32 [T,d] workspace; deterministic.
 * out: [T,d] dtype, output.  ws: MOE_WS_COMBINE. */
int moe_combine(const moe_shape* s, const void* y_swi, const void* w_down, const int32_t* offsets,
                const int32_t* expert_token_indices, const int32_t* token_index_map, const int32_t* topk_ids,
                const float* topk_w, void* out, void* ws, size_t ws_bytes, void* stream);

/* Staged-Y combine: an ABLATION of moe_combine, not part of the product path
 * (SonicMoE analysis page, sec. 3.4.1 on the temporary Y, sec. 3.4.2
 * "Expert aggregation kernels: gather-and-sum", Figure 17 left: the down
 * projection stores Y = y_swi W_down^T for every assignment contiguously,
 * then an aggregation kernel gathers each token's K rows and sums).  It
 * computes the same out[t] = sum_k topk_w[t,k] * Y[token_index_map[t*K+k]]
 * as moe_combine, but materialises Y: a [T*K, d] buffer in the activation
 * dtype inside the workspace (MOE_WS_COMBINE_STAGED).  The sum runs in slot
 * order k = 0..K-1 in fp32; Y is rounded to the activation dtype before it,
 * so results differ from moe_combine by that rounding.  Deterministic, no
 * atomics.  Same arguments and errors as moe_combine. */
int moe_combine_staged(const moe_shape* s, const void* y_swi, const void* w_down, const int32_t* offsets,
                       const int32_t* expert_token_indices, const int32_t* token_index_map,
                       const int32_t* topk_ids, const float* topk_w, void* out, void* ws, size_t ws_bytes,
                       void* stream);

/* Backward of L = <dout, out> (reading notes Algorithm 1 backward; MoEBlaze
 * analysis page "Backward Pass" and "Fused SwiGLU Kernel"; SonicMoE analysis
 * page sec. 3.4.1).  Per position p (expert e, token t, weight w):
 *   dA' = dout[t] W_down[e]            dS = <dA', y_swi[p]>
 *   sigma = sigmoid(a), recomputed from the saved a; dy = w * dA'
 *   da = dy * b * (sigma + a*sigma*(1-sigma)),   db = dy * a * sigma
 *   dw_down[e] += (w dout[t])^T y_swi[p];  dw_gate[e] += da^T x[t];
 *   dw_up[e] += db^T x[t];  dx[t] += da W_gate[e] + db W_up[e]
 *   router: dz[t,S_k] = w_k (dS_k - sum_j w_j dS_j), zero elsewhere;
 *           dwg[e] = sum_t dz[t,e] x[t];  dx[t] += sum_k dz[t,S_k] Wg[S_k].
 * Inputs: dout, x [T,d]; wg [E,d]; weights; routing arrays; h_ab, y_swi from
 * moe_expert_fwd.  Outputs (every element written; experts with no rows get
 * exact zeros): dx [T,d] dtype, dwg [E,d] fp32, dw_gate/dw_up [E,h,d] fp32,
 * dw_down [E,d,h] fp32, ds [T,K] fp32 (nullable: the router score
 * gradient dL/dw).  The bias, if any, gets no gradient.  dx is assembled by
 * the same ordered, atomic-free fold as moe_combine.  ws: MOE_WS_EXPERT_BWD.
 *
 * H-only saving (SonicMoE analysis page sec. 3.4.1, the minimal cached set
 * of the memory-efficient backward): y_swi == NULL.  The forward's y_swi is
 * then only a forward transient (moe_combine reads it; the caller may free
 * it before the backward).  The dH kernel recomputes y = SiLU(a) * b from the
 * saved bf16 a and b, uses it for dS = <dA', y>, and writes A' = w * y in
 * the activation dtype into the workspace, where dW_down reads it as its
 * right-hand operand (dw_down[e] += dout[t]^T A'[p]).
 *   a_prime [T*K, h] dtype (nullable; H-only only): where A' is written.
 *     The forward's y_swi buffer, dead once moe_combine has read it, is the
 *     intended one.  With a_prime == NULL, A' lives in the workspace, which
 *     must then be MOE_WS_EXPERT_BWD_H; with a_prime given, MOE_WS_EXPERT_BWD
 *     suffices.  It is overwritten, must not overlap any other argument, and
 *     must be NULL when y_swi is passed (MOE_ERR_INVALID_ARG otherwise).
 *   dh [T*K, 2h] dtype (nullable; [T*K, h] for the plain experts): where the
 *     gradient of the pre-activations, dH = [da | db], is written (the same
 *     layout as h_ab), for the dW_gate/dW_up and dX GEMMs that read it.  NULL:
 *     the workspace holds it (MOE_WS_EXPERT_BWD or _H).  Given, the workspace
 *     needs only MOE_WS_EXPERT_BWD_LEAN, and under H-only saving a_prime must
 *     be given too (MOE_ERR_INVALID_ARG otherwise).  dh may be h_ab itself:
 *     the saved H is then overwritten by its own gradient, which the backward
 *     allows because each element of H is read (once, by the dH kernel)
 *     before the gradient element at the same place is written, and nothing
 *     after the dH kernel reads H.  That saves the [T*K, 2h] buffer; the
 *     saved H is gone after the call.  Otherwise dh must not overlap any
 *     other argument (dh equal to y_swi, a_prime, dout, x or dx is
 *     MOE_ERR_INVALID_ARG). */
int moe_expert_bwd(const moe_shape* s, const void* dout, const void* x, const void* wg, const void* w_gate,
                   const void* w_up, const void* w_down, const int32_t* topk_ids, const float* topk_w,
                   const int32_t* offsets, const int32_t* expert_token_indices, const int32_t* token_index_map,
                   const void* h_ab, const void* y_swi, void* a_prime, void* dh, void* dx, float* dwg,
                   float* dw_gate, float* dw_up, float* dw_down, float* ds, void* ws, size_t ws_bytes,
                   void* stream);

/* Static string for a moe_status value (host). */
const char* moe_status_string(int code);

/* Bound on the polls of one wait in the ordered combine (default 1<<20,
 * about a second); a wait that runs out sets the calling entry's workspace
 * error word and proceeds, so every kernel always finishes, but that call's
 * output is then invalid (see the error words above).  polls <= 0 only
 * reads the value.  Returns the previous value.  Thread-safe; a call reads
 * the limit once, when it enqueues its kernels. */
int moe_set_spin_limit(int polls);

/* Per-kernel timing (profiling aid).  While enabled, each internal kernel
 * launch is bracketed by HIP events on its stream; moe_timing_read
 * synchronises on those events and returns up to `cap` (name, milliseconds)
 * records in launch order (host arrays), then clears them.  Off by default. */
int moe_timing_enable(int on);
int moe_timing_read(const char** names, float* ms, int cap);

#ifdef __cplusplus
}
#endif
#endif /* MOE_DISPATCH_H */
