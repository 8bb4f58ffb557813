/*
 * rope_attn.h -- exact softmax attention with rotary position embedding and
 * learnable per-band log-frequencies, forward and backward, on AMD gfx950.
 *
 * What is computed (every entry point shares these conventions):
 *
 *   theta_m     = base^(-2m/D),  theta_hat_m = exp(alpha_m) * theta_m,
 *                 m = 0 .. D/2-1  (LeRoPE, "Central mechanism"; alpha = 0 is
 *                 standard RoPE, "Key design choices", initialisation)
 *   rotation    the pair (x[2m], x[2m+1]) of query and key row p is turned
 *               counter-clockwise by p * theta_hat_m (LeRoPE, "Problem
 *               statement": queries and keys are rotated in 2-D frequency
 *               bands; values are not rotated), positions p = 0 .. N-1
 *   scores      S = Q~ K~^T / sqrt(D), causal mask keeps key j <= query i
 *   forward     O = softmax(S) V, LSE_i = log sum_j exp(S_ij)   (natural log)
 *               ("RoPE attention can be trained in almost-linear time",
 *               "Problem definition"; s(x) in "Methodology", item 1)
 *   backward    the vector-Jacobian product for the upstream gradient dO:
 *               beta = dO V^T, dS = P o (beta - D_i) with D_i = sum_c dO O,
 *               i.e. gamma = diag(s) beta - s s^T beta (same page,
 *               "Methodology", items 1 and 2, gamma_1 and gamma_2), returned
 *               as dQ, dK (un-rotated frame), dV, and
 *   d alpha     dalpha_m = theta_hat_m * sum over batch, heads and positions
 *               p of p * (x[2m] g[2m+1] - x[2m+1] g[2m]) for (x, g) = (q, dQ)
 *               and (k, dK): one alpha vector is shared by every head and
 *               layer (LeRoPE, "Key design choices", parameter sharing), so
 *               its gradient sums over all of them.  It equals theta_hat_m
 *               times the slope of the surrogate of LeRoPE, "Theoretical
 *               analysis".
 *
 * Layout: Q, K, V, dO, O, dQ, dK, dV are contiguous [B][H][N][D] with D
 * fastest; LSE is [B][H][N]; alpha and dalpha are [D/2] float32 shared by all
 * (b, h).  Q, K, V, dO are stored as float32 (dtype ROPE_ATTN_FP32) or
 * bfloat16 (ROPE_ATTN_BF16); every output is float32.
 *
 * Pointers: all tensor pointers are device pointers (hipMalloc'd or
 * equivalent), 16-byte aligned.  The caller owns every buffer; the library
 * allocates nothing and keeps no state between calls.  `stream` is a
 * hipStream_t (NULL = the default stream); all work is enqueued on it
 * asynchronously and nothing is synchronised on the host.  Inputs are read
 * only.  Outputs are overwritten, dalpha included (not accumulated).
 *
 * Errors: every entry point validates its arguments before launching
 * anything and returns ROPE_ATTN_OK or a negative status; no exception or
 * abort crosses this boundary.  A launch failure reported by the HIP runtime
 * returns ROPE_ATTN_ERR_HIP.
 *
 * Numerics: with bf16 inputs, products run on fp16 matrix-core operands with
 * float32 accumulation, except the leading causal corner (query rows below
 * 128 per started 8192 positions; one 128-row block with block lists), whose
 * products use split fp16 operands (hi + lo, three products per
 * contraction, about 22-bit operands) with float32 accumulation.  Calls with
 * fp32 inputs run in float32 throughout.
 *
 * Input domain of the bf16 path (fp16 operands):
 *  - dO: any finite magnitude.  The backward is linear in dO, so each head's
 *    dO is scaled by a power of two (exact) that puts its largest entry in
 *    [4, 8) before the fp16 conversion, and the scale is undone in dQ, dK,
 *    dV and dalpha.  Gradients of 1e-30 or 1e30 get the same relative
 *    accuracy as gradients of 1.
 *  - Q, K, V: entries of the rotated Q~ * log2(e) * scale, of K~ and of V
 *    must lie within fp16's finite range, |x| <= 65504 (for K and V about
 *    |x| < 4.6e4, since the rotation mixes pairs).  The PREP stage sets
 *    ROPE_ATTN_FLAG_FP16_RANGE in the workspace when an entry does not
 *    (that operand became +-inf and the outputs are not meaningful); read it
 *    with rope_attn_workspace_flags.  Entries below 6.1e-5 in magnitude keep
 *    fp16's absolute precision (2^-24) but lose relative precision.
 *  - accuracy: the error of each output row is a small fraction of that
 *    row's own size (measured max |err_row| <= 1.3e-2 * rms(row), typically
 *    2e-3 to 8e-3, for scores up to 26 in log2 units).  Normalised by the
 *    whole tensor's RMS instead, the error grows with the tensor's
 *    peak-to-RMS ratio max|x| / rms(x), so max |err| <= 2e-2 * rms(x) holds
 *    for outputs whose largest entries are within ROPE_ATTN_PEAK_RATIO_MAX
 *    times their RMS (typical workloads: 3 to 16); inputs with a few rows
 *    far above the rest (gradient ratios of 30 to 60) reach 3e-2 there.
 *
 * bwd_rope_apply_amd/examples/rope_attn_example.cpp is a plain C++ caller of
 * these entry points (one problem from a file, forward and backward).
 */
#ifndef ROPE_ATTN_H
#define ROPE_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { ROPE_ATTN_FP32 = 0, ROPE_ATTN_BF16 = 1 } rope_attn_dtype;

typedef enum {
  ROPE_ATTN_OK = 0,
  ROPE_ATTN_ERR_NULL = -1,      /* a required pointer is NULL */
  ROPE_ATTN_ERR_SHAPE = -2,     /* B, H, N < 1, D not 64 or 128, or sizes overflow */
  ROPE_ATTN_ERR_DTYPE = -3,     /* dtype not a rope_attn_dtype */
  ROPE_ATTN_ERR_ALIGN = -4,     /* a pointer is not 16-byte aligned */
  ROPE_ATTN_ERR_WORKSPACE = -5, /* workspace smaller than the *_workspace_bytes(_min) query */
  ROPE_ATTN_ERR_HIP = -6,       /* the HIP runtime reported a launch error */
  ROPE_ATTN_ERR_ARG = -7        /* base not finite and > 0, or causal not 0/1 */
} rope_attn_status;

/* Workspace (device memory, 256-byte aligned recommended) needed by
 * rope_attn_fwd for these arguments; 0 on invalid arguments. */
size_t rope_attn_fwd_workspace_bytes(int B, int H, int N, int D, int dtype, int causal);

/* Forward.  q, k, v: [B,H,N,D] inputs of `dtype`; o: [B,H,N,D] float32
 * output; lse: [B,H,N] float32 output (natural log, scale included).
 * alpha: [D/2] float32 device pointer, or NULL for alpha = 0 (standard
 * RoPE).  base: RoPE base b > 0.  causal: 1 = keys j <= i, 0 = all keys. */
int rope_attn_fwd(const void* q, const void* k, const void* v, float* o, float* lse, int B, int H,
                  int N, int D, int dtype, double base, const float* alpha, int causal,
                  void* workspace, size_t workspace_bytes, void* stream);

/* Workspace for rope_attn_bwd; 0 on invalid arguments.  With bf16 inputs and
 * D = 128 it includes the dS panels: the dK/dV pass stores dS = P o (dP - D_i) in fp16
 * there (about B*H*N^2 bytes under the causal mask, 2*B*H*N^2 without it)
 * and dQ is then one product dS K~ instead of a pass that recomputes the
 * scores and dP.  The panels are included when they take at most 16 GiB;
 * block-list calls do not use them.  A workspace of at least
 * rope_attn_bwd_workspace_bytes_min but smaller than this selects the
 * recomputing dQ pass; the two agree within the bf16 tolerance (the same dS
 * values, summed in another order). */
size_t rope_attn_bwd_workspace_bytes(int B, int H, int N, int D, int dtype, int causal);

/* The smallest workspace rope_attn_bwd accepts (no dS panels); equal to
 * rope_attn_bwd_workspace_bytes for fp32 inputs, for D = 64 (where
 * recomputing the scores is the faster dQ pass) and when the panels would
 * exceed 16 GiB; 0 on invalid arguments. */
size_t rope_attn_bwd_workspace_bytes_min(int B, int H, int N, int D, int dtype, int causal);

/* Backward.  q, k, v, dO: [B,H,N,D] of `dtype`; o, lse: the forward's float32
 * outputs for the same q, k, v, base, alpha, causal.  dq, dk, dv: [B,H,N,D]
 * float32 outputs (un-rotated frame).  dalpha: [D/2] float32 output, or
 * NULL to skip it. */
int rope_attn_bwd(const void* q, const void* k, const void* v, const float* o, const void* dO,
                  const float* lse, float* dq, float* dk, float* dv, float* dalpha, int B, int H,
                  int N, int D, int dtype, double base, const float* alpha, int causal,
                  void* workspace, size_t workspace_bytes, void* stream);

/* Staged forms of the two passes, for callers that time or interleave the
 * phases.  `stages` is a bitwise OR of rope_attn_stage values; calling every
 * stage in increasing order, on one stream with one workspace and the same
 * arguments, is exactly rope_attn_fwd / rope_attn_bwd (which call these with
 * ROPE_ATTN_STAGE_ALL).  A stage reads what the earlier stages left in the
 * workspace, so the workspace must not be modified in between.
 *   PREP    frequency table; fp16 operand planes (bf16 inputs); D_i (bwd)
 *   EXACT   the float32 path: the whole problem (fp32 inputs); nothing
 *           with bf16 inputs (their leading causal corner runs in MAIN and
 *           in DQ)
 *   MAIN    forward matrix-core pass (bf16 inputs), the leading causal
 *           corner's split-operand rows included
 *   DKDV    dK, dV matrix-core pass (bf16 inputs); with the dS panels it
 *           also writes dS into the workspace
 *   DQ      dQ matrix-core pass (bf16 inputs), and the leading causal
 *           corner's dQ rows and its shares of dK and dV, which it adds to
 *           what DKDV wrote; with the dS panels it also reads the dS that
 *           DKDV left.  DKDV must have run first
 *   DALPHA  fixed-order reduction of the d alpha partials
 *   PREP_GRAD  (backward only, in place of PREP) the dO plane and D_i only:
 *           the frequency table and the Q~, K~, V planes are taken from the
 *           workspace as the forward's PREP stage left them.  The caller
 *           guarantees that this workspace buffer was last passed to
 *           rope_attn_fwd / rope_attn_fwd_stages with PREP for the same q, k,
 *           v, B, H, N, D, dtype, base, alpha and causal, and was not
 *           modified since (the forward's regions are a prefix of the
 *           backward's layout, so one buffer of rope_attn_bwd_workspace_bytes
 *           serves both calls).  Violating this gives wrong results; it is
 *           not detected. */
typedef enum {
  ROPE_ATTN_STAGE_PREP = 1,
  ROPE_ATTN_STAGE_EXACT = 2,
  ROPE_ATTN_STAGE_MAIN = 4,
  ROPE_ATTN_STAGE_DKDV = 8,
  ROPE_ATTN_STAGE_DQ = 16,
  ROPE_ATTN_STAGE_DALPHA = 32,
  ROPE_ATTN_STAGE_ALL = 63,
  ROPE_ATTN_STAGE_PREP_GRAD = 64
} rope_attn_stage;

int rope_attn_fwd_stages(unsigned stages, const void* q, const void* k, const void* v, float* o,
                         float* lse, int B, int H, int N, int D, int dtype, double base,
                         const float* alpha, int causal, void* workspace, size_t workspace_bytes,
                         void* stream);

int rope_attn_bwd_stages(unsigned stages, const void* q, const void* k, const void* v,
                         const float* o, const void* dO, const float* lse, float* dq, float* dk,
                         float* dv, float* dalpha, int B, int H, int N, int D, int dtype,
                         double base, const float* alpha, int causal, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Frequency-schedule options (a zero-initialised struct, or a NULL pointer,
 * means the defaults, i.e. exactly rope_attn_fwd / rope_attn_bwd):
 *   unrotated_pairs  the slowest `unrotated_pairs` bands m >= D/2 -
 *           unrotated_pairs pass through unrotated (partial RoPE: their
 *           effective rate is 0, so alpha has no effect there and dalpha is
 *           0).  LeRoPE ("Experimental setup", baselines) compares against
 *           p-RoPE, which removes the rotation from the slowest 25% of the
 *           bands: unrotated_pairs = D/8.  Range [0, D/2].
 *   scale   softmax scale on q.k; 0 = 1/sqrt(D).  Context-extension schemes
 *           that LeRoPE is combined with (its "Extrapolation" result) act
 *           through per-band offsets, which are alpha, and such a scale.
 *           Finite and > 0 when nonzero.
 *   pos_offset  position of row 0, shared by queries and keys (rows sit at
 *           pos_offset .. pos_offset + N - 1).  Outputs depend on positions
 *           only through their differences (LeRoPE, "Problem statement":
 *           relative position through the rotation), so this tests large
 *           absolute angles; dalpha uses positions relative to row 0, which
 *           equals the absolute-position form because the per-band wedge
 *           sums of the query and key gradients cancel.  >= 0 with
 *           pos_offset + N <= 2^30.
 * Invalid options return ROPE_ATTN_ERR_ARG before any launch. */
typedef struct {
  int unrotated_pairs;
  float scale;
  int pos_offset;
  /* Block-list attention: exact attention in which each query block of 128
   * rows sees its own (diagonal) key block plus the key blocks its list
   * names, and no other key (Multipole Semantic Attention, "Retrieval-
   * augmented approximation": the exact part, over retrieved block pairs and
   * the local block diagonal).  Lists are CSR over the B*H*ceil(N/128)
   * query blocks in [b][h][query block] order: the list of query block r is
   * block_idx[block_ptr[r] .. block_ptr[r+1]-1], so block_ptr has
   * B*H*ceil(N/128)+1 entries.  Both are DEVICE pointers to int32, read on
   * the call's stream by the PREP stage, which turns them into a visibility
   * bitmask in the workspace; the caller keeps them valid until then.
   * block_ptr == NULL means dense attention (the default).  Entries of
   * block_ptr are clamped to [0, block_nnz]; key blocks outside
   * [0, ceil(N/128)), and under the causal mask blocks after the query's
   * own, are ignored; duplicates are harmless.  O and LSE are over exactly
   * the visible keys, so partial results over disjoint key sets merge
   * through their LSEs.  Requires N <= 65536 (ERR_SHAPE otherwise),
   * block_nnz >= 0 and block_idx non-NULL when block_nnz > 0 (ERR_ARG),
   * 4-byte aligned pointers (ERR_ALIGN).  The bf16 path's cost scales with
   * the listed blocks; the fp32 path tests every key. */
  const int* block_ptr;
  const int* block_idx;
  int block_nnz;
} rope_attn_options;

/* The staged forward and backward with options (opts may be NULL).  A
 * backward run with PREP_GRAD must use the same options as the forward that
 * filled the workspace. */
int rope_attn_fwd_ex(unsigned stages, const rope_attn_options* opts, const void* q, const void* k,
                     const void* v, float* o, float* lse, int B, int H, int N, int D, int dtype,
                     double base, const float* alpha, int causal, void* workspace,
                     size_t workspace_bytes, void* stream);

int rope_attn_bwd_ex(unsigned stages, const rope_attn_options* opts, const void* q, const void* k,
                     const void* v, const float* o, const void* dO, const float* lse, float* dq,
                     float* dk, float* dv, float* dalpha, int B, int H, int N, int D, int dtype,
                     double base, const float* alpha, int causal, void* workspace,
                     size_t workspace_bytes, void* stream);

/* Range flags that the PREP stage leaves at the start of the workspace
 * (cleared by every PREP, kept by the other stages and by PREP_GRAD). */
#define ROPE_ATTN_FLAG_FP16_RANGE 1u /* an entry of Q~ (scaled), K~ or V exceeded 65504 */

/* The largest peak-to-RMS ratio of an output tensor (O, dQ, dK, dV) at
 * which the bf16 path is specified to meet max |err| <= 2e-2 * rms. */
#define ROPE_ATTN_PEAK_RATIO_MAX 20

/* Copies the range flags of `workspace` (as the last PREP stage on it left
 * them) into *flags on the host.  Enqueues a 4-byte device-to-host copy on
 * `stream` and synchronises that stream, so it waits for every call enqueued
 * before it.  Returns ROPE_ATTN_ERR_NULL, _ALIGN (workspace not 16-byte
 * aligned), _WORKSPACE (workspace_bytes < 4) or _HIP on failure. */
int rope_attn_workspace_flags(const void* workspace, size_t workspace_bytes, unsigned* flags,
                              void* stream);

/* The forward (rope_attn_fwd) for callers that cannot allocate device
 * memory or pass a workspace: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Its workspace is a file-scope
 * device array of ROPE_ATTN_NOALLOC_SCRATCH_BYTES held by every GPU the
 * library runs on until the process ends; the call allocates nothing and
 * looks up this GPU's copy of the array once (on the first call on the
 * device).  Arguments, outputs and results are exactly rope_attn_fwd's.
 * Returns ROPE_ATTN_ERR_WORKSPACE when the problem needs more than the array
 * holds (rope_attn_fwd_workspace_bytes > ROPE_ATTN_NOALLOC_SCRATCH_BYTES, for
 * example B*H*N*D above about 1e7 at N = 2048), ROPE_ATTN_ERR_HIP when the
 * array's address cannot be obtained, and rope_attn_fwd's other statuses.
 * Calls on one GPU share its array: calls that overlap in time on one GPU
 * (on different streams, or from several threads without ordering) race and
 * give wrong results; calls ordered on one stream are safe. */
#define ROPE_ATTN_NOALLOC_SCRATCH_BYTES (64u << 20)
int rope_attn_fwd_noalloc(const void* q, const void* k, const void* v, float* o, float* lse, int B,
                          int H, int N, int D, int dtype, double base, const float* alpha,
                          int causal, void* stream);

/* Static, NUL-terminated description of a status code. */
const char* rope_attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* ROPE_ATTN_H */
