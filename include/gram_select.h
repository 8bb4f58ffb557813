/* Gram-threshold token selection on AMD MI355X (gfx950): C ABI.
 *
 * "Cascade token selection for transformer attention acceleration":
 *   - the selection rule (Problem statement, ADA's Gram threshold): token i
 *     of a sequence is a representative when the largest cosine between it
 *     and any earlier token j < i is below 1 - tau^2, where
 *     cos(i, j) = <x_i, x_j> / (|x_i| |x_j|);
 *   - the cascade (Methodology, steps 1-3): inherit the previous layer's set
 *     R; keep the members whose largest cosine to earlier members of R is
 *     below the threshold (the r x r Gram product); add the tokens outside R
 *     whose largest cosine to earlier kept members is below it (the
 *     (T - r) x r cross product).  Every representative of the full rule on
 *     the same tokens is kept (Contributions, Proposition 4).
 *
 * Readings where the page is open: the cosine is signed; "below" is strict;
 * "earlier" is the sequence order; a token with no earlier token (and, in
 * the cascade, none in the set it is compared with) has maximum -inf and is
 * a representative; a zero token has cosine 0 with every token.
 *
 * Conventions: x is a DEVICE pointer to a contiguous [B][T][d] array
 * (gram_cascade: [T][d]) of bfloat16 (GRAM_BF16) or float16 (GRAM_FP16),
 * 16-byte aligned, d a multiple of 64 in [64, 65536], T >= 1, B >= 1,
 * T * d <= 2^31, B * T <= 2^31.  Products of the stored values are exact in
 * the float32 accumulator of the matrix cores; norms are float32 sums of
 * exact squares.  All other pointers are device pointers, 4-byte aligned
 * (rep and prev: any alignment).  Outputs are overwritten:
 *   max_cos [B][T] float32: the maximum the decision used (-inf when empty);
 *   rep     [B][T] uint8:   1 for a representative, else 0;
 *   count   [B] int32 (NULL: not written): the number of representatives.
 * Work is enqueued on `stream` (a hipStream_t, NULL = the default stream);
 * the call returns without synchronising.  The workspace (device memory of
 * at least *_workspace_bytes, 256-byte aligned) is owned by the caller; two
 * calls may not share one concurrently.  Status codes are those of
 * rope_attn.h: ROPE_ATTN_ERR_* is returned before any launch for a NULL
 * pointer, a bad shape or dtype, a misaligned pointer, a workspace that is
 * too small or a tau that is not finite and >= 0; ROPE_ATTN_ERR_HIP if a
 * launch fails. */
#ifndef GRAM_SELECT_H
#define GRAM_SELECT_H

#include <stddef.h>

#include "rope_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { GRAM_BF16 = 1, GRAM_FP16 = 2 } gram_dtype;

/* Bytes of workspace gram_select needs (0 for an invalid shape). */
size_t gram_select_workspace_bytes(int B, int T, int d);

/* The selection rule on each of B sequences: the causal T x T Gram product
 * of the normalised tokens, reduced to a running maximum per token. */
int gram_select(const void* x, int B, int T, int d, int dtype, float tau, float* max_cos,
                unsigned char* rep, int* count, void* workspace, size_t workspace_bytes,
                void* stream);

/* gram_select split at kernel boundaries, so a caller can time the Gram
 * product alone (each stage reads what the earlier ones left in the same
 * workspace): PREP resets the maxima and the count and computes the inverse
 * norms; GRAM runs the causal Gram product with its running maximum; DECIDE
 * writes max_cos, rep and count. */
typedef enum {
  GRAM_STAGE_PREP = 1,
  GRAM_STAGE_GRAM = 2,
  GRAM_STAGE_DECIDE = 4,
  GRAM_STAGE_ALL = 7
} gram_stage;

int gram_select_stages(unsigned stages, const void* x, int B, int T, int d, int dtype, float tau,
                       float* max_cos, unsigned char* rep, int* count, void* workspace,
                       size_t workspace_bytes, void* stream);

/* Bytes of workspace gram_cascade needs (0 for an invalid shape). */
size_t gram_cascade_workspace_bytes(int T, int d);

/* One cascade step on one sequence: prev [T] uint8 flags the inherited set R
 * (nonzero = member).  max_cos holds, for members of R, the maximum over
 * earlier members; for the others, the maximum over earlier kept members.
 * rep flags the updated set; the kept members are rep & prev. */
int gram_cascade(const void* x, int T, int d, int dtype, float tau, const unsigned char* prev,
                 float* max_cos, unsigned char* rep, int* count, void* workspace,
                 size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GRAM_SELECT_H */
