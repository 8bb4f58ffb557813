// C ABI: argument validation, workspace layout and the launch sequence of
// the forward and backward passes.
#include <math.h>
#include <stdint.h>

#include "common.h"
#include "rope_attn.h"

namespace {

using namespace ra;

constexpr size_t ALIGN = 256;

size_t up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

struct Shape {
  int B, H, N, D, dtype, causal;
  int blocks;  // block-list attention requested
  size_t bh() const { return (size_t)B * H; }
  size_t elems() const { return bh() * N * D; }
  bool bf16() const { return dtype == ROPE_ATTN_BF16; }
  // split-operand corner rows: bf16 causal only.  With block lists every row
  // averages at most its listed blocks, so the first block suffices.
  int corner() const { return (bf16() && causal) ? (blocks ? BLK : corner_rows(N)) : 0; }
  // block visibility bitmask (any call that may use block lists)
  bool mask_ok() const { return N <= MAX_BLOCKS * BLK; }
  // dS panels for the backward's dQ product (bf16, D = 128, up to
  // PANEL_MAX_BYTES).  Their traffic is 2 bytes per (query, key) pair at any
  // D, while the recomputation they replace scales with D: at D = 64 the
  // recomputing dQ pass is faster (measured on MI355X), so it is kept there.
  size_t panel_bytes() const { return 2 * bh() * panel_head(N, causal); }
  bool panels_ok() const { return bf16() && D == 128 && panel_bytes() <= PANEL_MAX_BYTES; }
  static constexpr size_t PANEL_MAX_BYTES = (size_t)16 << 30;
};

int check_shape(const Shape& s) {
  if (s.dtype != ROPE_ATTN_FP32 && s.dtype != ROPE_ATTN_BF16) return ROPE_ATTN_ERR_DTYPE;
  if (s.B < 1 || s.H < 1 || s.N < 1) return ROPE_ATTN_ERR_SHAPE;
  if (s.D != 64 && s.D != 128) return ROPE_ATTN_ERR_SHAPE;
  if (s.causal != 0 && s.causal != 1) return ROPE_ATTN_ERR_ARG;
  // keep every index of the kernels inside int / 2^40-element ranges
  if (s.N > (1 << 24) || s.bh() > (1u << 24) || s.elems() > ((size_t)1 << 40)) return ROPE_ATTN_ERR_SHAPE;
  if ((size_t)s.N * (s.D / 2) > (size_t)INT32_MAX) return ROPE_ATTN_ERR_SHAPE;
  return ROPE_ATTN_OK;
}

bool misaligned(const void* p) { return ((uintptr_t)p & 15u) != 0; }

bool misaligned_4(const void* p) { return ((uintptr_t)p & 3u) != 0; }

// Options with their defaults resolved.
struct Opts {
  int rot;      // rotated bands (D/2 - unrotated_pairs)
  float scale;  // softmax scale
  int pos0;     // position of row 0
  const int* bptr;  // block lists (CSR over BH x n_blocks query blocks), or null
  const int* bidx;
  int bnnz;
};

int resolve(const rope_attn_options* o, const Shape& s, Opts& r) {
  r.rot = s.D / 2;
  r.scale = 1.0f / sqrtf((float)s.D);
  r.pos0 = 0;
  r.bptr = nullptr;
  r.bidx = nullptr;
  r.bnnz = 0;
  if (!o) return ROPE_ATTN_OK;
  if (o->block_ptr) {
    if (!s.mask_ok()) return ROPE_ATTN_ERR_SHAPE;
    if (o->block_nnz < 0 || (o->block_nnz > 0 && !o->block_idx)) return ROPE_ATTN_ERR_ARG;
    if (misaligned_4(o->block_ptr) || misaligned_4(o->block_idx)) return ROPE_ATTN_ERR_ALIGN;
    r.bptr = o->block_ptr;
    r.bidx = o->block_idx;
    r.bnnz = o->block_nnz;
  }
  if (o->unrotated_pairs < 0 || o->unrotated_pairs > s.D / 2) return ROPE_ATTN_ERR_ARG;
  if (!(o->scale == 0.0f || (isfinite(o->scale) && o->scale > 0.0f))) return ROPE_ATTN_ERR_ARG;
  if (o->pos_offset < 0 || (long)o->pos_offset + s.N > (1L << 30)) return ROPE_ATTN_ERR_ARG;
  r.rot = s.D / 2 - o->unrotated_pairs;
  if (o->scale != 0.0f) r.scale = o->scale;
  r.pos0 = o->pos_offset;
  return ROPE_ATTN_OK;
}

// Workspace regions, in order.  Sizes are 0 for regions a call does not use.
// The forward's regions (table, operand planes, corner low parts) come first
// and are laid out identically by both passes, so a backward run on the
// forward's workspace can reuse them (ROPE_ATTN_STAGE_PREP_GRAD).
// The dS panels come last, so the layouts with and without them agree on
// every other region.
struct Layout {
  size_t flags, theta, cs, qh, kh, vh, qlo, klo, bmask, amax, dsc, doh, drow, rs, part, dsp;
  int slots;
  size_t total() const {
    return flags + theta + cs + qh + kh + vh + qlo + klo + bmask + amax + dsc + doh + drow + rs +
           part + dsp;
  }
};

MfmaParams mfma_base(const Shape& s, float scale) {
  MfmaParams m = {};
  m.B = s.B; m.H = s.H; m.N = s.N; m.D = s.D;
  m.corner = s.corner();
  m.causal = s.causal;
  m.bf16 = s.bf16();
  m.scale = scale;
  return m;
}

// dQ/dK/dV/dalpha partial-sum slots of the MFMA path for one corner choice
// and dQ kernel (panels or recomputation)
int mfma_slots(const Shape& s, bool panels) {
  MfmaParams m = mfma_base(s, 1.0f);
  if (panels) m.dsp = reinterpret_cast<half_t*>(ALIGN);  // only selects the dQ kernel's grid
  return dq_mfma_slots(m) + dkdv_mfma_slots(m);   // the corner's slots are the dQ launch's
}

// Region sizes do not depend on whether a call passes block lists (the
// workspace queries take no options): corner regions are sized for the
// larger, dense corner, and the slot count is the largest over the modes.
// `panels` adds the backward's dS panels (only when s.panels_ok()).
Layout layout(Shape s, bool bwd, bool panels = false) {
  Layout L = {};
  s.blocks = 0;
  L.flags = ALIGN;   // range flags: offset 0 of every layout
  L.theta = up(sizeof(double) * (s.D / 2));
  L.cs = up(sizeof(float2) * (size_t)s.N * (s.D / 2));
  // fp16 planes: every head's rows, then PLANE_PAD_ROWS zero rows
  const size_t h16 = up(2 * (s.elems() + (size_t)PLANE_PAD_ROWS * s.D));
  if (s.bf16()) {
    L.qh = L.kh = L.vh = h16;
    if (bwd) L.doh = h16;
    if (s.corner()) L.qlo = L.klo = up(2 * s.bh() * s.corner() * s.D);
  }
  if (s.mask_ok()) L.bmask = up(sizeof(uint32_t) * s.bh() * n_blocks(s.N) * mask_words(s.N));
  if (bwd) {
    if (s.bf16()) {
      L.amax = up(sizeof(float) * s.bh() * AMAX_SLOTS);
      L.dsc = up(sizeof(float) * s.bh());
    }
    L.drow = up(sizeof(float) * s.bh() * s.N);
    if (s.bf16()) L.rs = up(sizeof(float) * s.bh() * rs_groups(s.N) * 64);
    if (s.bf16()) {
      Shape sb = s;
      sb.blocks = 1;
      L.slots = max(mfma_slots(s, false), mfma_slots(s, true));
      if (s.mask_ok()) L.slots = max(L.slots, mfma_slots(sb, false));
    } else {
      L.slots = 2 * simt_slots((int)s.bh(), s.N);
    }
    L.part = up(sizeof(float) * (size_t)L.slots * (s.D / 2));
    if (panels && s.panels_ok()) L.dsp = up(s.panel_bytes());
  }
  return L;
}

struct Carve {
  char* p;
  template <class T>
  T* take(size_t bytes) {
    if (!bytes) return nullptr;
    T* r = reinterpret_cast<T*>(p);
    p += bytes;
    return r;
  }
};

int check_common(const Shape& s, double base, void* ws, size_t ws_bytes, bool bwd) {
  int st = check_shape(s);
  if (st) return st;
  if (!(base > 0.0) || !isfinite(base)) return ROPE_ATTN_ERR_ARG;
  if (!ws) return ROPE_ATTN_ERR_NULL;
  if (misaligned(ws)) return ROPE_ATTN_ERR_ALIGN;
  if (ws_bytes < layout(s, bwd).total()) return ROPE_ATTN_ERR_WORKSPACE;
  return ROPE_ATTN_OK;
}

void tables(const Shape& s, const Opts& op, double base, const float* alpha, double* theta,
            float2* cs, unsigned* flags, hipStream_t st) {
  TableParams t = {};
  t.cs = cs; t.theta_hat = theta; t.alpha = alpha; t.base = base; t.N = s.N; t.D = s.D;
  t.rot = op.rot; t.pos0 = op.pos0; t.flags = flags;
  launch_table(t, st);
}

void block_mask(const Shape& s, const Opts& op, uint32_t* mask, hipStream_t st) {
  BlockMaskParams bp = {};
  bp.ptr = op.bptr; bp.idx = op.bidx; bp.nnz = op.bnnz; bp.mask = mask;
  bp.nb = n_blocks(s.N); bp.W = mask_words(s.N); bp.rows = (int)s.bh() * bp.nb;
  bp.causal = s.causal;
  launch_block_mask(bp, st);
}

void set_blocks(MfmaParams& m, const Shape& s, const Opts& op, const uint32_t* mask) {
  m.bmask = op.bptr ? mask : nullptr;
  m.nb = n_blocks(s.N);
  m.W = mask_words(s.N);
}

int finish() {
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? ROPE_ATTN_OK : ROPE_ATTN_ERR_HIP;
}

}  // namespace

extern "C" {

size_t rope_attn_fwd_workspace_bytes(int B, int H, int N, int D, int dtype, int causal) {
  const Shape s{B, H, N, D, dtype, causal};
  if (check_shape(s)) return 0;
  return layout(s, false).total();
}

size_t rope_attn_bwd_workspace_bytes(int B, int H, int N, int D, int dtype, int causal) {
  const Shape s{B, H, N, D, dtype, causal};
  if (check_shape(s)) return 0;
  return layout(s, true, true).total();
}

size_t rope_attn_bwd_workspace_bytes_min(int B, int H, int N, int D, int dtype, int causal) {
  const Shape s{B, H, N, D, dtype, causal};
  if (check_shape(s)) return 0;
  return layout(s, true, false).total();
}

int rope_attn_fwd_ex(unsigned stages, const rope_attn_options* opts, const void* q, const void* k,
                     const void* v, float* o, float* lse, int B, int H, int N, int D, int dtype,
                     double base, const float* alpha, int causal, void* workspace,
                     size_t workspace_bytes, void* stream) {
  Shape s{B, H, N, D, dtype, causal, 0};
  if (!q || !k || !v || !o || !lse) return ROPE_ATTN_ERR_NULL;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o) || misaligned(lse) ||
      misaligned(alpha))
    return ROPE_ATTN_ERR_ALIGN;
  int st = check_shape(s);
  if (st) return st;
  Opts op;
  st = resolve(opts, s, op);
  if (st) return st;
  s.blocks = op.bptr != nullptr;
  st = check_common(s, base, workspace, workspace_bytes, false);
  if (st) return st;

  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  const Layout L = layout(s, false);
  Carve c{reinterpret_cast<char*>(workspace)};
  unsigned* flags = c.take<unsigned>(L.flags);
  double* theta = c.take<double>(L.theta);
  float2* cs = c.take<float2>(L.cs);
  half_t* qh = c.take<half_t>(L.qh);
  half_t* kh = c.take<half_t>(L.kh);
  half_t* vh = c.take<half_t>(L.vh);
  half_t* qlo = c.take<half_t>(L.qlo);
  half_t* klo = c.take<half_t>(L.klo);
  uint32_t* bmask = c.take<uint32_t>(L.bmask);

  if (stages & ROPE_ATTN_STAGE_PREP) {
    tables(s, op, base, alpha, theta, cs, flags, hs);
    if (op.bptr) block_mask(s, op, bmask, hs);
    if (s.bf16()) {
      PrepParams pp = {};
      pp.q = q; pp.k = k; pp.v = v; pp.cs = cs; pp.qh = qh; pp.kh = kh; pp.vh = vh;
      pp.flags = flags;
      pp.qlo = qlo; pp.klo = klo; pp.rlo = s.corner();
      pp.bf16 = 1; pp.BH = (int)s.bh(); pp.N = N; pp.D = D;
      pp.qscale = LOG2E * op.scale;
      launch_prep(pp, hs);
    }
  }
  MfmaParams mp = mfma_base(s, op.scale);
  mp.qh = qh; mp.kh = kh; mp.vh = vh; mp.qlo = qlo; mp.klo = klo; mp.o = o; mp.out_lse = lse;
  set_blocks(mp, s, op, bmask);
  if (stages & ROPE_ATTN_STAGE_EXACT) {
    if (!s.bf16()) {
      SimtParams sp = {};
      sp.q = q; sp.k = k; sp.v = v; sp.cs = cs; sp.out_o = o; sp.out_lse = lse;
      sp.bf16 = 0; sp.BH = (int)s.bh(); sp.N = N; sp.D = D; sp.causal = causal;
      sp.scale = op.scale;
      sp.rows = N;
      sp.bmask = mp.bmask; sp.nb = mp.nb; sp.W = mp.W;
      if (sp.bmask) launch_simt_fwd(sp, hs);   // block lists: the vector path
      else launch_f32_fwd(sp, hs);
    }
    // bf16: the corner's split-operand rows run in the MAIN launch
  }
  if ((stages & ROPE_ATTN_STAGE_MAIN) && s.bf16()) launch_fwd_mfma(mp, hs);
  return finish();
}

int rope_attn_fwd(const void* q, const void* k, const void* v, float* o, float* lse, int B, int H,
                  int N, int D, int dtype, double base, const float* alpha, int causal,
                  void* workspace, size_t workspace_bytes, void* stream) {
  return rope_attn_fwd_ex(ROPE_ATTN_STAGE_ALL, nullptr, q, k, v, o, lse, B, H, N, D, dtype, base,
                          alpha, causal, workspace, workspace_bytes, stream);
}

int rope_attn_fwd_stages(unsigned stages, const void* q, const void* k, const void* v, float* o,
                         float* lse, int B, int H, int N, int D, int dtype, double base,
                         const float* alpha, int causal, void* workspace, size_t workspace_bytes,
                         void* stream) {
  return rope_attn_fwd_ex(stages, nullptr, q, k, v, o, lse, B, H, N, D, dtype, base, alpha, causal,
                          workspace, workspace_bytes, stream);
}

int rope_attn_bwd_ex(unsigned stages, const rope_attn_options* opts, const void* q, const void* k,
                     const void* v, const float* o, const void* dO, const float* lse, float* dq,
                     float* dk, float* dv, float* dalpha, int B, int H, int N, int D, int dtype,
                     double base, const float* alpha, int causal, void* workspace,
                     size_t workspace_bytes, void* stream) {
  Shape s{B, H, N, D, dtype, causal, 0};
  if (!q || !k || !v || !o || !dO || !lse || !dq || !dk || !dv) return ROPE_ATTN_ERR_NULL;
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o) || misaligned(dO) ||
      misaligned(lse) || misaligned(dq) || misaligned(dk) || misaligned(dv) || misaligned(alpha) ||
      misaligned(dalpha))
    return ROPE_ATTN_ERR_ALIGN;
  int st = check_shape(s);
  if (st) return st;
  Opts op;
  st = resolve(opts, s, op);
  if (st) return st;
  s.blocks = op.bptr != nullptr;
  st = check_common(s, base, workspace, workspace_bytes, true);
  if (st) return st;

  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  // dQ as a product over dS panels when the workspace holds them (dense
  // attention), else by recomputing the scores
  const Layout Lp = layout(s, true, true);
  const bool panels = !op.bptr && Lp.dsp && workspace_bytes >= Lp.total();
  const Layout L = panels ? Lp : layout(s, true, false);
  Carve c{reinterpret_cast<char*>(workspace)};
  unsigned* flags = c.take<unsigned>(L.flags);
  double* theta = c.take<double>(L.theta);
  float2* cs = c.take<float2>(L.cs);
  half_t* qh = c.take<half_t>(L.qh);
  half_t* kh = c.take<half_t>(L.kh);
  half_t* vh = c.take<half_t>(L.vh);
  half_t* qlo = c.take<half_t>(L.qlo);
  half_t* klo = c.take<half_t>(L.klo);
  uint32_t* bmask = c.take<uint32_t>(L.bmask);
  float* amax = c.take<float>(L.amax);
  float* dsc = c.take<float>(L.dsc);
  half_t* doh = c.take<half_t>(L.doh);
  float* drow = c.take<float>(L.drow);
  float* rs = c.take<float>(L.rs);
  float* part = c.take<float>(L.part);
  half_t* dsp = c.take<half_t>(L.dsp);

  // d alpha partial slots: [exact dQ rows | exact dK rows | dQ launch | dK/dV launch]; the
  // dQ launch of the bf16 path also runs the corner (its dQ rows, and its share of dK, dV)
  const int BHi = (int)s.bh();
  MfmaParams mp = mfma_base(s, op.scale);
  mp.dsp = dsp;
  const int n_exact_dq = s.bf16() ? 0 : simt_slots(BHi, N);
  const int n_exact_dk = s.bf16() ? 0 : simt_slots(BHi, N);
  const int n_dq = s.bf16() ? dq_mfma_slots(mp) : 0;
  const int n_dk = s.bf16() ? dkdv_mfma_slots(mp) : 0;

  if (stages & (ROPE_ATTN_STAGE_PREP | ROPE_ATTN_STAGE_PREP_GRAD)) {
    // PREP_GRAD alone: the table and the Q~, K~, V planes are the forward's
    const bool full = (stages & ROPE_ATTN_STAGE_PREP) != 0;
    if (full) tables(s, op, base, alpha, theta, cs, flags, hs);
    if (full && op.bptr) block_mask(s, op, bmask, hs);
    if (s.bf16()) {  // per-head maxima of |dO| for its power-of-two scale
      AbsmaxParams ap = {};
      ap.x = dO; ap.amax = amax; ap.BH = BHi; ap.N = N; ap.D = D;
      launch_absmax(ap, hs);
    }
    PrepParams pp = {};
    pp.q = q; pp.k = k; pp.v = v; pp.dO = dO; pp.o = o; pp.cs = cs;
    pp.qh = full ? qh : nullptr; pp.kh = full ? kh : nullptr; pp.vh = full ? vh : nullptr;
    pp.doh = doh; pp.drow = drow;
    pp.lse = lse; pp.rs = rs;
    pp.qlo = full ? qlo : nullptr; pp.klo = full ? klo : nullptr; pp.rlo = s.corner();
    pp.bf16 = s.bf16(); pp.BH = BHi; pp.N = N; pp.D = D;
    pp.qscale = LOG2E * op.scale;
    pp.amax = amax; pp.dsc = dsc;
    pp.flags = full ? flags : nullptr;
    launch_prep(pp, hs);
  }
  mp.dsc = dsc;
  mp.qh = qh; mp.kh = kh; mp.vh = vh; mp.doh = doh; mp.qlo = qlo; mp.klo = klo; mp.q = q; mp.k = k;
  mp.cs = cs; mp.lse = lse; mp.drow = drow; mp.rs = rs; mp.dq = dq; mp.dk = dk; mp.dv = dv;
  set_blocks(mp, s, op, bmask);
  mp.dalpha_part = part;
  if (stages & ROPE_ATTN_STAGE_EXACT) {
    if (!s.bf16()) {
      SimtParams sp = {};
      sp.q = q; sp.k = k; sp.v = v; sp.dO = dO; sp.o = o; sp.lse = lse; sp.drow = drow; sp.cs = cs;
      sp.dq = dq; sp.dk = dk; sp.dv = dv; sp.dalpha_part = part;
      sp.bf16 = 0; sp.BH = BHi; sp.N = N; sp.D = D; sp.causal = causal;
      sp.scale = op.scale;
      sp.rows = N; sp.qend = N; sp.final_ = 1;
      sp.bmask = mp.bmask; sp.nb = mp.nb; sp.W = mp.W;
      sp.slot0 = 0;
      if (sp.bmask) launch_simt_dq(sp, hs);   // block lists: the vector path
      else launch_f32_dq(sp, hs);
      sp.slot0 = n_exact_dq;
      if (sp.bmask) launch_simt_dkdv(sp, hs);
      else launch_f32_dkdv(sp, hs);
    }
    // bf16: the corner runs in the dQ launch (DQ stage)
  }
  // dK/dV first: with panels it writes the dS that the dQ product reads
  if ((stages & ROPE_ATTN_STAGE_DKDV) && s.bf16()) {
    mp.slot0 = n_exact_dq + n_exact_dk + n_dq;
    launch_dkdv_mfma(mp, hs);
  }
  if ((stages & ROPE_ATTN_STAGE_DQ) && s.bf16()) {
    mp.slot0 = n_exact_dq + n_exact_dk;
    launch_dq_mfma(mp, hs);
  }
  if ((stages & ROPE_ATTN_STAGE_DALPHA) && dalpha) {
    DalphaParams dp = {};
    dp.part = part; dp.theta_hat = theta; dp.dalpha = dalpha;
    dp.slots = n_exact_dq + n_exact_dk + n_dq + n_dk; dp.D = D;
    launch_dalpha_reduce(dp, hs);
  }
  return finish();
}

int rope_attn_bwd(const void* q, const void* k, const void* v, const float* o, const void* dO,
                  const float* lse, float* dq, float* dk, float* dv, float* dalpha, int B, int H,
                  int N, int D, int dtype, double base, const float* alpha, int causal,
                  void* workspace, size_t workspace_bytes, void* stream) {
  return rope_attn_bwd_ex(ROPE_ATTN_STAGE_ALL, nullptr, q, k, v, o, dO, lse, dq, dk, dv, dalpha, B,
                          H, N, D, dtype, base, alpha, causal, workspace, workspace_bytes, stream);
}

int rope_attn_bwd_stages(unsigned stages, const void* q, const void* k, const void* v,
                         const float* o, const void* dO, const float* lse, float* dq, float* dk,
                         float* dv, float* dalpha, int B, int H, int N, int D, int dtype,
                         double base, const float* alpha, int causal, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return rope_attn_bwd_ex(stages, nullptr, q, k, v, o, dO, lse, dq, dk, dv, dalpha, B, H, N, D,
                          dtype, base, alpha, causal, workspace, workspace_bytes, stream);
}

int rope_attn_workspace_flags(const void* workspace, size_t workspace_bytes, unsigned* flags,
                              void* stream) {
  if (!workspace || !flags) return ROPE_ATTN_ERR_NULL;
  if (misaligned(workspace)) return ROPE_ATTN_ERR_ALIGN;
  if (workspace_bytes < sizeof(unsigned)) return ROPE_ATTN_ERR_WORKSPACE;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  unsigned v = 0;
  if (hipMemcpyAsync(&v, workspace, sizeof(unsigned), hipMemcpyDeviceToHost, hs) != hipSuccess)
    return ROPE_ATTN_ERR_HIP;
  if (hipStreamSynchronize(hs) != hipSuccess) return ROPE_ATTN_ERR_HIP;
  *flags = v;
  return ROPE_ATTN_OK;
}

const char* rope_attn_status_string(int status) {
  switch (status) {
    case ROPE_ATTN_OK: return "ok";
    case ROPE_ATTN_ERR_NULL: return "a required pointer is NULL";
    case ROPE_ATTN_ERR_SHAPE: return "invalid shape: need B, H, N >= 1 and D in {64, 128}";
    case ROPE_ATTN_ERR_DTYPE: return "dtype must be ROPE_ATTN_FP32 or ROPE_ATTN_BF16";
    case ROPE_ATTN_ERR_ALIGN: return "pointers must be 16-byte aligned";
    case ROPE_ATTN_ERR_WORKSPACE: return "workspace smaller than the *_workspace_bytes(_min) query";
    case ROPE_ATTN_ERR_HIP: return "HIP runtime reported a launch error";
    case ROPE_ATTN_ERR_ARG:
      return "base must be finite and > 0, causal 0 or 1; options: unrotated_pairs in [0, D/2], "
             "scale 0 (default) or finite > 0, pos_offset >= 0 with pos_offset + N <= 2^30";
    default: return "unknown status";
  }
}

}  // extern "C"
