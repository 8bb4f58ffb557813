// Shared device helpers and launch parameter blocks for the RoPE attention
// kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ra {

typedef _Float16 half_t;
typedef __attribute__((ext_vector_type(8))) _Float16 half8;
typedef __attribute__((ext_vector_type(2))) _Float16 half2v;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;

// Causal corner: query rows [0, corner) of every head, and the keys they
// see, are computed with split fp16 operands (x = hi + lo, three products per
// contraction, ~22-bit operands) when the inputs are bf16.  Those rows
// average few keys, so their outputs and gradients are the largest entries
// of each tensor, and plain fp16 rounding there would dominate the error
// relative to the tensor's RMS; the effect grows with N (the typical row
// averages more keys), so the corner grows with it: 128 rows per 8192
// positions, at least 128.
constexpr int CORNER_UNIT = 128;
__host__ __device__ inline int corner_rows(int N) {
  const int units = (N + 8191) / 8192;
  return CORNER_UNIT * (units < 1 ? 1 : units);
}

// Backward row scalars in 32-row groups: [-LSE * log2(e) x 32 | -D x 32] per
// group (negated: they seed the dK/dV products' accumulators), one spare
// group after the last; rows >= N hold (-inf, 0) so that their
// P = exp2(S - LSE2) is exactly 0.
__host__ __device__ inline int rs_groups(int N) { return (N + 31) / 32 + 1; }

// Block-list attention: query and key blocks of BLK rows; a visibility
// bitmask row [W words] per (bh, query block), bit kb set when the query
// block attends key block kb (its own block always).  Up to MAX_BLOCKS
// blocks per head (N <= 65536).
constexpr int BLK = 128;
constexpr int MAX_BLOCKS = 512;
__host__ __device__ inline int n_blocks(int N) { return (N + BLK - 1) / BLK; }
__host__ __device__ inline int mask_words(int N) { return (n_blocks(N) + 31) / 32; }

// dS panels (bf16 backward with a large enough workspace): the dK/dV pass
// stores dS of every head in fp16, one panel per PANEL-query block; the dQ
// pass reads them as the left operand of dQ~ = dS K~.  Under the causal mask
// panel b holds keys 0 .. PANEL (b + 1) - 1 (the rest are masked), otherwise
// every key up to PANEL n_panels(N).  A panel is blocked by 32 keys x 32
// queries, 2 KiB per block, blocks ordered [key block][query block]; inside
// a block, element (key k, query q) sits at half (q / 16) 512 + k 16 + q % 16.
// One wave's dK/dV step (32 keys x 32 queries) is then one contiguous block,
// stored by two fully coalesced 1 KiB instructions, and 32 keys of a panel
// are one contiguous 16 KiB tile.  Offsets are in halfs from the head's
// first panel.
constexpr int PANEL = 256;
__host__ __device__ inline int n_panels(int N) { return (N + PANEL - 1) / PANEL; }
__host__ __device__ inline int panel_rows(int b, int N, int causal) {
  return causal ? PANEL * (b + 1) : PANEL * n_panels(N);
}
__host__ __device__ inline size_t panel_off(int b, int N, int causal) {
  return causal ? (size_t)PANEL * PANEL * ((size_t)b * (b + 1) / 2)
                : (size_t)b * PANEL * ((size_t)PANEL * n_panels(N));
}
__host__ __device__ inline size_t panel_head(int N, int causal) {
  return panel_off(n_panels(N), N, causal);
}

// The fp16 operand planes in the workspace carry PLANE_PAD_ROWS zero rows
// after their last head, so a streamed tile that starts below N never reads
// past the plane: the tile copies need no per-row clamp.  Rows at or past N
// of a head read the next head's rows (or the zero pad); every use of them
// is masked or multiplied by an exact zero, and all of them are finite.
constexpr int PLANE_PAD_ROWS = 64;

// Per-head power-of-two scaling of the upstream gradient (bf16 inputs).  The
// backward is linear in dO, so each head's dO is multiplied by
// s = 2^(2 - floor(log2 max|dO|)) before its fp16 conversion (its largest
// entry lands in [4, 8)), D_i is taken from the scaled values, and 1 / s is
// applied where dQ, dK and dV leave the accumulators.  Multiplying by a
// power of two is exact, so gradients of any magnitude an fp32 or bf16
// tensor holds keep fp16's full precision instead of falling into its
// subnormals (below 6.1e-5) or overflowing it (above 65504).  The head's
// maximum comes from AMAX_SLOTS partial maxima per head.
constexpr int AMAX_SLOTS = 32;

// Range flags (one word at the start of every workspace), set by the PREP
// stage: an entry of the rotated, scaled Q~, of K~ or of V lay outside
// fp16's finite range, so that operand became +-inf.
constexpr unsigned FLAG_FP16_RANGE = 1u;

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// ------------------------------------------------------------------ params
struct TableParams {
  float2* cs;           // [N][D/2] (cos, sin) of (p + pos0) * theta_hat_m
  double* theta_hat;    // [D/2]; 0 for the unrotated bands m >= rot
  const float* alpha;   // [D/2] or null (all zero)
  double base;
  int N, D;
  int rot;              // bands m < rot are rotated (partial RoPE), D/2 = all
  int pos0;             // position of row 0
  unsigned* flags;      // range flags, cleared here (the first kernel of PREP), or null
};

struct AbsmaxParams {
  const void* x;        // [BH][N][D] bf16
  float* amax;          // [BH][AMAX_SLOTS] partial maxima of |x|
  int BH, N, D;
};

struct PrepParams {
  const void* q; const void* k; const void* v; const void* dO;  // [B,H,N,D] inputs
  const float* o;        // [B,H,N,D] forward output (for D = rowsum(dO*O)), or null
  const float2* cs;      // [N][D/2]
  half_t* qh; half_t* kh; half_t* vh; half_t* doh;  // fp16 operand planes, any may be null
  half_t* qlo; half_t* klo;  // [BH][rlo][D] low parts x - fp16(x) of rows < rlo, or null
  int rlo;
  float* drow;           // [B,H,N] or null
  const float* lse;      // [B,H,N] forward LSE (natural log), with rs
  float* rs;             // [BH][rs_groups(N)][64] row scalars, or null
  float qscale;          // factor folded into the rotated Q plane
  const float* amax;     // [BH][AMAX_SLOTS] partial maxima of |dO| (scales the dO plane), or null
  float* dsc;            // [BH] written: 1 / (the head's dO scale), when amax is set
  unsigned* flags;       // range flags (FLAG_FP16_RANGE), or null
  int bf16;              // input storage: 1 = bf16, 0 = fp32
  int BH, N, D;
};

struct BlockMaskParams {
  const int* ptr;       // [rows + 1] CSR offsets into idx (device)
  const int* idx;       // [nnz] key-block indices (device)
  int nnz;
  uint32_t* mask;       // [rows][W] output
  int rows, nb, W;      // rows = BH * nb
  int causal;
};

// Exact fp32 path (one query or key row per 4-lane group).
struct SimtParams {
  const void* q; const void* k; const void* v; const void* dO;
  const float* o; const float* lse; const float* drow;
  const float2* cs;
  float* out_o; float* out_lse;        // forward outputs
  float* dq;                            // [B,H,N,D] un-rotated dQ
  float* dk; float* dv;                 // final dK, dV (when final != 0)
  float* dk_part; float* dv_part;       // [BH][rows][D] rotated-frame partials (final == 0)
  float* dalpha_part;                   // [slots][D/2]
  int slot0;                            // first dalpha slot of this launch
  const uint32_t* bmask;                // block visibility [BH][nb][W], or null (all visible)
  int nb, W;
  int bf16;
  int BH, N, D;
  int rows;        // query rows (fwd, dq) or key rows (dkdv) handled: [0, rows)
  int qend;        // dkdv: contributions from query rows [.., qend)
  int causal;
  int final_;      // dkdv: 1 = write dK/dV, 0 = write rotated partials
  float scale;
};

// qh holds Q~ * log2(e) / sqrt(D), so scores come out in log2 units.
struct MfmaParams {
  const half_t* qh; const half_t* kh; const half_t* vh; const half_t* doh;
  const half_t* qlo; const half_t* klo;   // [BH][corner][D] low parts (corner kernels)
  const void* q; const void* k;        // original inputs (for the d alpha wedge)
  const float2* cs;
  const float* lse; const float* drow;
  const float* rs;                     // [BH][rs_groups(N)][64] row scalars (dK/dV)
  float* o; float* out_lse;
  float* dq; float* dk; float* dv;
  half_t* dsp;                      // dS panels [BH][panel_head] (dK/dV writes, dQ reads), or null
  const float* dsc;                 // [BH] 1 / (dO scale) of each head (backward), or null (1)
  float* dalpha_part;
  int slot0;
  const uint32_t* bmask;           // block visibility [BH][nb][W], or null (causal triangle / all)
  int nb, W;
  int bf16;
  int B, H, N, D;
  int corner;      // rows [0, corner) are done by the corner's split-operand workgroups
  int corner_at;   // dQ launch: grid position of its corner workgroups (set by the launcher)
  int causal;
  float scale;
};

struct DalphaParams {
  const float* part;     // [slots][D/2]
  const double* theta_hat;
  float* dalpha;         // [D/2]
  int slots, D;
};

// ------------------------------------------------------------------ launchers
void launch_table(const TableParams& p, hipStream_t s);
void launch_prep(const PrepParams& p, hipStream_t s);
void launch_absmax(const AbsmaxParams& p, hipStream_t s);
void launch_block_mask(const BlockMaskParams& p, hipStream_t s);
void launch_simt_fwd(const SimtParams& p, hipStream_t s);
void launch_simt_dq(const SimtParams& p, hipStream_t s);
void launch_simt_dkdv(const SimtParams& p, hipStream_t s);
int simt_slots(int BH, int rows);       // dalpha slots used by one simt dq/dkdv launch
// the fp32 path on the matrix cores (dense attention; the same slots as simt)
void launch_f32_fwd(const SimtParams& p, hipStream_t s);
void launch_f32_dq(const SimtParams& p, hipStream_t s);
void launch_f32_dkdv(const SimtParams& p, hipStream_t s);
void launch_fwd_mfma(const MfmaParams& p, hipStream_t s);
void launch_dq_mfma(const MfmaParams& p, hipStream_t s);
void launch_dkdv_mfma(const MfmaParams& p, hipStream_t s);
int dq_mfma_slots(const MfmaParams& p);   // either dQ kernel (p.dsp selects)
int dkdv_mfma_slots(const MfmaParams& p);
void launch_dalpha_reduce(const DalphaParams& p, hipStream_t s);

// ------------------------------------------------------------------ device helpers
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// Load 4 consecutive input elements (bf16 or fp32 storage) as floats.
__device__ __forceinline__ void load4(const void* base, size_t idx, int bf16, float* x) {
  if (bf16) {
    uint2 u = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(base) + idx);
    x[0] = __uint_as_float(u.x << 16);
    x[1] = __uint_as_float(u.x & 0xffff0000u);
    x[2] = __uint_as_float(u.y << 16);
    x[3] = __uint_as_float(u.y & 0xffff0000u);
  } else {
    float4 f = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + idx);
    x[0] = f.x; x[1] = f.y; x[2] = f.z; x[3] = f.w;
  }
}

// The factor that undoes a head's dO scaling in the backward epilogues.
__device__ __forceinline__ float dscale_inv(const float* dsc, int bh) { return dsc ? dsc[bh] : 1.f; }

// Whether key `key` is visible to query row `row` under a block mask (null:
// all blocks visible; the causal mask is separate).
__device__ __forceinline__ bool block_visible(const uint32_t* bm, int nb, int W, int bh, int row,
                                              int key) {
  if (!bm) return true;
  const int kb = key / BLK;
  return (bm[((size_t)bh * nb + row / BLK) * W + (kb >> 5)] >> (kb & 31)) & 1u;
}

// Turn the pair (x0, x1) by +phi given (cos phi, sin phi).
__device__ __forceinline__ void rot(float c, float s, float& x0, float& x1) {
  float a = x0 * c - x1 * s;
  float b = x0 * s + x1 * c;
  x0 = a; x1 = b;
}
// Turn the pair by -phi (transpose rotation, the chain rule of rot).
__device__ __forceinline__ void unrot(float c, float s, float& g0, float& g1) {
  float a = g0 * c + g1 * s;
  float b = -g0 * s + g1 * c;
  g0 = a; g1 = b;
}

}  // namespace ra
