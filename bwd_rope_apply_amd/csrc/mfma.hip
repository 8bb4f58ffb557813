// MFMA kernels for exact RoPE attention on gfx950: forward, dQ and dK/dV.
//
// Operands are the fp16 planes written by the prep pass (Q~, K~ rotated,
// V, dO converted); products accumulate in fp32 with
// v_mfma_f32_32x32x16_f16.  fp16 rather than bf16 operands: the two run at
// the same MFMA rate on gfx950, and the 3 extra mantissa bits are what keeps
// the error of P, dS, Q~ and K~ rounding within 2e-2 of each output's RMS.
//
// Fragment convention of v_mfma_f32_32x32x16_f16 (lane l, l32 = l % 32,
// g = l / 32):  A[m][k]: lane (m, g) holds k = 8g..8g+7 of a 16-wide k step;
// B[k][n]: lane (n, g) holds the same k; C[m][n]: lane (n, g) holds rows
// 8(r/4) + 4g + r%4 in register r.  Every score tile is computed transposed
// (keys along m, queries along n) so all per-query scalars (row max, row
// sum, LSE, D) live in one lane.  The A rows of the key operand are read in
// the order perm(m) (bits 2 and 3 swapped), which makes register r of a
// score block hold key 16(r/8) + 8g + r%8: the 8 keys a lane needs as the
// B operand of the next product are then contiguous.
//
// What each product computes ("RoPE attention can be trained in
// almost-linear time", Methodology 1 and 2): the normalised softmax s(x),
// the weighted sum with V, beta = dO V^T, gamma = diag(s) beta - s s^T beta
// = P o (dP - D), and the gradient back through the scores.
#include "common.h"

namespace ra {

namespace {

// Tiling (compile-time; the defaults are the measured best on MI355X):
//   *_WPS   waves per SIMD the register budget is sized for (2 lets one
//           wave's softmax VALU work overlap the other wave's MFMAs)
//   *_BN    rows of the streamed operand per loop step (multiple of 32)
//   FWD_NB  32-row query blocks per forward wave
#ifndef RA_FWD_NB
#define RA_FWD_NB 1
#endif
#ifndef RA_FWD_WPS
#define RA_FWD_WPS 2
#endif
#ifndef RA_FWD_SEED
#define RA_FWD_SEED 0      // 1: fold the running max into the score accumulators
#endif
#ifndef RA_DQ_BN
#define RA_DQ_BN 64
#endif
#ifndef RA_DQ_WPS
#define RA_DQ_WPS 1
#endif
#ifndef RA_DKDV_BN
#define RA_DKDV_BN 64
#endif
#ifndef RA_DKDV_WPS
#define RA_DKDV_WPS 1
#endif

constexpr int BN = 64;     // keys per forward loop step
constexpr int BM = 128;    // stationary rows per dq / dkdv workgroup (4 waves x 32)

__device__ __forceinline__ int perm(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// LDS tile layout ([BN][D + 8] fp16): logical row L (bits b5..b0) is stored
// at physical row sig(L) = (b5 b4 b2 | b1 b0 b3).  With the 16-byte row pad
// (4 banks), the natural fragment reads (8 lanes on rows perm(l32)) and the
// transposed reads (16 lanes on 4 rows x 32 bytes) both touch 32 distinct
// banks, and every read of a lane is one base address plus immediates.
__device__ __forceinline__ int sig(int L) {
  return (L & 48) | ((L & 4) << 1) | ((L & 3) << 1) | ((L >> 3) & 1);
}

__device__ __forceinline__ f32x16 mfma(half8 a, half8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Block index -> (head, tile).  Workgroups are dispatched round-robin over
// the 8 XCDs; when the head count allows, each XCD gets a fixed set of heads
// so that their K/V (or Q/dO) tiles stay in that XCD's L2.  Tiles are issued
// heaviest first (most causal work).
__device__ __forceinline__ void map_block(int idx, int BH, int ntiles, bool heavy_high, int& bh,
                                          int& t) {
  int k;
  if ((BH & 7) == 0) {
    const int hpx = BH >> 3;
    const int x = idx & 7, s = idx >> 3;
    bh = x * hpx + s % hpx;
    k = s / hpx;
  } else {
    bh = idx % BH;
    k = idx / BH;
  }
  t = heavy_high ? ntiles - 1 - k : k;
}

// Register copy of one streamed [BN][D] fp16 tile: every thread holds NCH
// 16-byte chunks (row = chunk / (D/8)).  Rows at or past N are clamped to
// N - 1: they are masked downstream, so they only need to be finite.
template <int D, int ROWS = BN>
struct TileRegs {
  static constexpr int CPR = D / 8;
  static constexpr int NCH = ROWS * CPR / 256;
  half8 x[NCH];
  __device__ __forceinline__ void load(const half_t* src, int r0, int N) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int ch = threadIdx.x + 256 * i;
      const int row = min(r0 + ch / CPR, N - 1);
      x[i] = *reinterpret_cast<const half8*>(src + (size_t)row * D + (ch % CPR) * 8);
    }
  }
  __device__ __forceinline__ void store(half_t* dst) const {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int ch = threadIdx.x + 256 * i;
      *reinterpret_cast<half8*>(dst + sig(ch / CPR) * (D + 8) + (ch % CPR) * 8) = x[i];
    }
  }
};

template <int D>
__device__ __forceinline__ void load_frag_rows(half8* f, const half_t* src, int row, int N, int g) {
  // B-operand fragment of one row: k steps t -> columns 16t + 8g .. +8
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    half8 x = {};
    if (row < N) x = *reinterpret_cast<const half8*>(src + (size_t)row * D + 16 * t + 8 * g);
    f[t] = x;
  }
}

// Two 32-key score blocks (keys along m, this lane's query along n), the
// accumulators seeded with `seed` (a per-query offset folded into the product).
template <int D, int NMB = 2>
__device__ __forceinline__ void scores(f32x16* s, const half_t* lds, const half8* bf, int l32,
                                       int g, float seed = 0.f) {
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) {
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = seed;
    const half_t* row = lds + sig(32 * mb + perm(l32)) * (D + 8) + 8 * g;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) acc = mfma(*reinterpret_cast<const half8*>(row + 16 * t), bf[t], acc);
    s[mb] = acc;
  }
}

// Pack register values of NMB score blocks into the 2 NMB 16-key B-operand
// fragments (k step t holds keys 16t + 8g + e).
template <int NMB = 2>
__device__ __forceinline__ void to_frags(const f32x16* s, half8* f) {
#pragma unroll
  for (int t = 0; t < 2 * NMB; ++t) {
#pragma unroll
    for (int e = 0; e < 8; ++e) f[t][e] = (half_t)s[t >> 1][8 * (t & 1) + e];
  }
}

typedef __attribute__((ext_vector_type(4))) short s16x4;

__device__ __forceinline__ s16x4 ds_read_tr(const half_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}

// A-operand fragment of X^T for k step t and column block cb, X a [BN][D]
// tile in LDS (two transposed reads).
template <int D>
__device__ __forceinline__ half8 tr_frag(const half_t* lds, int t, int cb, int lane) {
  // logical rows 16t + 8g + 4h + e, e = s16 >> 2 (h = 0, 1), columns
  // 32cb + 16 b + 4 (s16 & 3): physical row 16t + 8h + sig(8g + e)
  constexpr int LD = D + 8;
  const int s16 = lane & 15, g = lane >> 5, b = (lane >> 4) & 1;
  const half_t* p = lds + (sig(8 * g + (s16 >> 2)) + 16 * t) * LD + 32 * cb + 16 * b + 4 * (s16 & 3);
  const s16x4 lo = ds_read_tr(p), hi = ds_read_tr(p + 8 * LD);
  typedef __attribute__((ext_vector_type(8))) short s16x8;
  const s16x8 both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(half8, both);
}

// acc[cb] += X^T(columns 32cb.., rows = 16-wide k steps) * frag, with X a
// [BN][D + 8] tile in LDS.  ds_read_b64_tr_b16 transposes a 4 x 16 block per
// 16-lane group (lane j receives element j of the 4 rows that lanes
// 4e + j/4 point at), so lane s of a group points at row s/4, columns
// 4 (s % 4) .. +3 of its block, and two reads give the 8 k-values (rows
// 16t + 8g + 0..7) of column 32cb + l32.
template <int D, int NT = 4>
__device__ __forceinline__ void accumulate_tr(f32x16* acc, const half_t* lds, const half8* f, int lane) {
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb) {
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[cb] = mfma(tr_frag<D>(lds, t, cb, lane), f[t], acc[cb]);
  }
}

// Position-weighted wedge partial of one row's gradient (already in the
// un-rotated frame) summed over the workgroup into one [D/2] slot.
// w[cb*8 + rq*2 + h] is pair m = 16cb + 4rq + 2g + h.
template <int D>
__device__ __forceinline__ void store_dalpha(float* w, float* red, float* slot, int g) {
  constexpr int NW = D / 4;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    float x = w[i];
    x += __shfl_xor(x, 1, 64);
    x += __shfl_xor(x, 2, 64);
    x += __shfl_xor(x, 4, 64);
    x += __shfl_xor(x, 8, 64);
    x += __shfl_xor(x, 16, 64);
    if ((lane & 31) == 0) {
      const int cb = i >> 3, rq = (i >> 1) & 3, h = i & 1;
      red[wave * (D / 2) + 16 * cb + 4 * rq + 2 * g + h] = x;
    }
  }
  __syncthreads();
  for (int m = threadIdx.x; m < D / 2; m += 256)
    slot[m] = (red[m] + red[D / 2 + m]) + (red[D + m] + red[3 * D / 2 + m]);
}

// Un-rotate one lane's gradient registers (row `row`, columns
// 32cb + 8rq + 4g + 0..3), add the wedge partials and store float4s.
template <int D>
__device__ __forceinline__ void finish_rows(f32x16* acc, float scale, const float* part_row,
                                            const float2* cs_row, const void* x_in, size_t x_off,
                                            int bf16, float* out, float pos, float* w, int g) {
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb) {
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      const int c = 32 * cb + 8 * rq + 4 * g;
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = acc[cb][4 * rq + e] * scale;
      if (part_row) {
        const float4 pr = *reinterpret_cast<const float4*>(part_row + c);
        v[0] += pr.x; v[1] += pr.y; v[2] += pr.z; v[3] += pr.w;
      }
      const float2 t0 = cs_row[c / 2], t1 = cs_row[c / 2 + 1];
      unrot(t0.x, t0.y, v[0], v[1]);
      unrot(t1.x, t1.y, v[2], v[3]);
      float x[4];
      load4(x_in, x_off + c, bf16, x);
      w[cb * 8 + rq * 2 + 0] = pos * (x[0] * v[1] - x[1] * v[0]);
      w[cb * 8 + rq * 2 + 1] = pos * (x[2] * v[3] - x[3] * v[2]);
      *reinterpret_cast<float4*>(out + c) = make_float4(v[0], v[1], v[2], v[3]);
    }
  }
}

// One 64-key step of the forward for one wave owning NB blocks of 32 query
// rows: scores, online softmax, O += P V.  Every K~ and V fragment read from
// LDS feeds NB products.  Q~ carries the factor log2(e)/sqrt(D), so scores
// are in log2 units.  m is the reference maximum the running sum l and O
// are relative to; it is seeded into the score accumulators (so they hold
// S - m) and only moved when a score exceeds it by more than 2^RESCALE_SLACK,
// which keeps every P below 2^8 (exact in the arithmetic, since O and l
// share the reference) and makes the O rescale rare.  MASK hides keys after
// klim[nb] (causal diagonal, ragged tail).
constexpr float RESCALE_SLACK = 8.f;

template <int D, int NB, bool MASK>
__device__ __forceinline__ void fwd_tile(f32x16 (*o)[D / 32], float* m, float* l,
                                         const half_t* Ks, const half_t* Vs,
                                         const half8 (*qf)[D / 16], int k0, const int* klim,
                                         int lane) {
  const int l32 = lane & 31, g = lane >> 5;
  f32x16 s[NB][2];
  float base[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) base[nb] = m[nb] == -INFINITY ? 0.f : m[nb];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[nb][mb][r] = RA_FWD_SEED ? -base[nb] : 0.f;
    }
    const half_t* row = Ks + sig(32 * mb + perm(l32)) * (D + 8) + 8 * g;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      const half8 a = *reinterpret_cast<const half8*>(row + 16 * t);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) s[nb][mb] = mfma(a, qf[nb][t], s[nb][mb]);
    }
  }
  half8 pf[NB][4];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    float mx = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = RA_FWD_SEED ? s[nb][mb][r] : s[nb][mb][r] - base[nb];
        if (MASK) {
          const int key = k0 + 32 * mb + 16 * (r >> 3) + 8 * g + (r & 7);
          x = key > klim[nb] ? -INFINITY : x;
        }
        s[nb][mb][r] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const bool upd = (m[nb] == -INFINITY) ? (mx != -INFINITY) : (mx > RESCALE_SLACK);
    if (__any(upd)) {  // rare: move the reference maximum
      const float shift = upd ? mx : 0.f;
      const float mn = upd ? base[nb] + mx : m[nb];
      const float alpha = upd ? exp2_fast(m[nb] - mn) : 1.f;
      l[nb] *= alpha;
      m[nb] = mn;
#pragma unroll
      for (int cb = 0; cb < D / 32; ++cb) o[nb][cb] *= alpha;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[nb][mb][r] -= shift;
      }
    }
    float ls = 0.f;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pr = exp2_fast(s[nb][mb][r]);
        s[nb][mb][r] = pr;
        ls += pr;
      }
    }
    l[nb] += ls;
    to_frags(s[nb], pf[nb]);
  }
  // O^T[c][q] += V^T[c][key] P^T[key][q]: V^T fragments by transposed reads
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const half8 a = tr_frag<D>(Vs, t, cb, lane);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) o[nb][cb] = mfma(a, pf[nb][t], o[nb][cb]);
    }
  }
}

// One step of dQ for one wave over 32 NMB keys: P = exp2(S' - LSE2) with
// the LSE seeded into the score accumulators, dP - D with D seeded into the
// dP accumulators (dP = dO V^T), dS = P o (dP - D), dQ~ += dS K~.
template <int D, int NMB, bool MASK>
__device__ __forceinline__ void dq_tile(f32x16* acc, const half_t* Ks, const half_t* Vs,
                                        const half8* qf, const half8* df, int k0, int klim,
                                        float lse2, float dr, int lane) {
  const int l32 = lane & 31, g = lane >> 5;
  f32x16 s[NMB], dp[NMB];
  scores<D, NMB>(s, Ks, qf, l32, g, -lse2);
  scores<D, NMB>(dp, Vs, df, l32, g, -dr);
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float pr = exp2_fast(s[mb][r]);
      if (MASK) {
        const int key = k0 + 32 * mb + 16 * (r >> 3) + 8 * g + (r & 7);
        pr = key > klim ? 0.f : pr;
      }
      s[mb][r] = pr * dp[mb][r];
    }
  }
  half8 sf[2 * NMB];
  to_frags<NMB>(s, sf);
  accumulate_tr<D, 2 * NMB>(acc, Ks, sf, lane);
}

// One step of dK, dV for one wave over 32 NMB queries (this lane's key
// along n): P = exp(S - LSE), dV += P^T dO, dP = dO V^T, dS = P o (dP - D),
// dK~ += dS^T Q~.  MASK hides queries before this lane's key.
template <int D, int NMB, bool MASK>
__device__ __forceinline__ void dkdv_tile(f32x16* dk, f32x16* dv, const half_t* Qs,
                                          const half_t* Ds, const float* lses, const float* drs,
                                          const half8* kf, const half8* vf, int r0, int key,
                                          int lane) {
  const int l32 = lane & 31, g = lane >> 5;
  f32x16 s[NMB], dp[NMB];
  scores<D, NMB>(s, Qs, kf, l32, g);   // queries along m, this lane's key along n
  scores<D, NMB>(dp, Ds, vf, l32, g);
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int ql = 32 * mb + 16 * h + 8 * g;
      const float4 la = *reinterpret_cast<const float4*>(lses + ql);
      const float4 lb = *reinterpret_cast<const float4*>(lses + ql + 4);
      const float4 da = *reinterpret_cast<const float4*>(drs + ql);
      const float4 db = *reinterpret_cast<const float4*>(drs + ql + 4);
      const float lv8[8] = {la.x, la.y, la.z, la.w, lb.x, lb.y, lb.z, lb.w};
      const float dv8[8] = {da.x, da.y, da.z, da.w, db.x, db.y, db.z, db.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int r = 8 * h + e;
        float pr = exp2_fast(s[mb][r] - lv8[e]);
        if (MASK) pr = key > r0 + ql + e ? 0.f : pr;
        s[mb][r] = pr;
        dp[mb][r] = pr * (dp[mb][r] - dv8[e]);
      }
    }
  }
  half8 pf[2 * NMB], sf[2 * NMB];
  to_frags<NMB>(s, pf);
  to_frags<NMB>(dp, sf);
  accumulate_tr<D, 2 * NMB>(dv, Ds, pf, lane);
  accumulate_tr<D, 2 * NMB>(dk, Qs, sf, lane);
}

// ------------------------------------------------------------------ forward
// Workgroup = 256 query rows of one head (4 waves x 64 rows, two 32-row
// blocks per wave); the loop streams 64-key tiles of K~ and V through
// double-buffered LDS, the next tile's global loads in flight while the
// current tile is computed.  Rows below the exact corner are skipped.
constexpr int FWD_NB = RA_FWD_NB;
constexpr int FWD_BM = 4 * 32 * FWD_NB;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, RA_FWD_WPS) void fwd_kernel(MfmaParams p) {
  constexpr int DT = D / 16, CB = D / 32, TILE = BN * (D + 8), NB = FWD_NB;
  __shared__ __attribute__((aligned(16))) half_t Ks[2 * TILE];
  __shared__ __attribute__((aligned(16))) half_t Vs[2 * TILE];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, l32 = lane & 31, g = lane >> 5;
  const int BH = p.B * p.H;
  const int ntiles = (p.N + FWD_BM - 1) / FWD_BM;
  int bh, t;
  map_block(blockIdx.x, BH, ntiles, true, bh, t);
  const int q0 = t * FWD_BM, wrow0 = q0 + 32 * NB * w;
  const size_t head = (size_t)bh * p.N * D;
  const half_t* kh = p.kh + head;
  const half_t* vh = p.vh + head;
  // waves whose rows all lie in the exact corner (or past N) only help load
  const bool active = wrow0 + 32 * NB > p.corner && wrow0 < p.N;

  half8 qf[NB][DT];
  int qrow[NB], klim[NB];
  f32x16 o[NB][CB];
  float m[NB], l[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    qrow[nb] = wrow0 + 32 * nb + l32;
    klim[nb] = CAUSAL ? min(qrow[nb], p.N - 1) : p.N - 1;
    load_frag_rows<D>(qf[nb], p.qh + head, qrow[nb], p.N, g);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) o[nb][cb] = f32x16{};
    m[nb] = -INFINITY;
    l[nb] = 0.f;
  }
  const int nk = (p.N + BN - 1) / BN;
  const int n_kt = CAUSAL ? min(nk, (q0 + FWD_BM + BN - 1) / BN) : nk;
  const int wlast = wrow0 + 32 * NB - 1;

  TileRegs<D> kr, vr;
  kr.load(kh, 0, p.N);
  vr.load(vh, 0, p.N);
  kr.store(Ks);
  vr.store(Vs);
  __syncthreads();
  for (int kt = 0; kt < n_kt; ++kt) {
    const int k0 = kt * BN;
    const int cur = (kt & 1) * TILE, nxt = TILE - cur;
    const bool more = kt + 1 < n_kt;
    if (more) {
      kr.load(kh, k0 + BN, p.N);
      vr.load(vh, k0 + BN, p.N);
    }
    if (active && !(CAUSAL && k0 > wlast)) {  // skip tiles wholly above this wave's rows
      if ((CAUSAL && k0 + BN - 1 > wrow0) || (k0 + BN > p.N))
        fwd_tile<D, NB, true>(o, m, l, Ks + cur, Vs + cur, qf, k0, klim, lane);
      else
        fwd_tile<D, NB, false>(o, m, l, Ks + cur, Vs + cur, qf, k0, klim, lane);
    }
    if (more) {
      kr.store(Ks + nxt);
      vr.store(Vs + nxt);
    }
    __syncthreads();
  }

#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const float lt = l[nb] + __shfl_xor(l[nb], 32, 64);
    const int row = qrow[nb];
    if (active && row >= p.corner && row < p.N) {
      const float inv = 1.f / lt;
      float* orow = p.o + head + (size_t)row * D;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int c = 32 * cb + 8 * rq + 4 * g;
          *reinterpret_cast<float4*>(orow + c) =
              make_float4(o[nb][cb][4 * rq] * inv, o[nb][cb][4 * rq + 1] * inv,
                          o[nb][cb][4 * rq + 2] * inv, o[nb][cb][4 * rq + 3] * inv);
        }
      }
      if (g == 0) p.out_lse[(size_t)bh * p.N + row] = (m[nb] + __log2f(lt)) * LN2;
    }
  }
}

// ------------------------------------------------------------------ dQ
// Workgroup = 128 query rows; streams KB-key tiles of K~ and V.  The K~
// tile serves both the score product (natural reads) and dQ~ += dS K~
// (transposed reads).
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, RA_DQ_WPS) void dq_kernel(MfmaParams p) {
  constexpr int KB = RA_DQ_BN, NMB = KB / 32;
  constexpr int DT = D / 16, CB = D / 32, TILE = KB * (D + 8);
  __shared__ __attribute__((aligned(16))) half_t Ks[2 * TILE];
  __shared__ __attribute__((aligned(16))) half_t Vs[2 * TILE];
  __shared__ float red[4 * (D / 2)];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, l32 = lane & 31, g = lane >> 5;
  const int BH = p.B * p.H;
  const int ntiles = (p.N + BM - 1) / BM, t0 = p.corner / BM;
  int bh, t;
  map_block(blockIdx.x, BH, ntiles - t0, true, bh, t);
  const int slot = p.slot0 + blockIdx.x;
  t += t0;
  const int q0 = t * BM, wrow0 = q0 + 32 * w, qrow = wrow0 + l32;
  const size_t head = (size_t)bh * p.N * D;
  const half_t* kh = p.kh + head;
  const half_t* vh = p.vh + head;

  half8 qf[DT], df[DT];
  load_frag_rows<D>(qf, p.qh + head, qrow, p.N, g);
  load_frag_rows<D>(df, p.doh + head, qrow, p.N, g);
  const bool row_ok = qrow < p.N;
  const float lse2 = row_ok ? p.lse[(size_t)bh * p.N + qrow] * LOG2E : 0.f;
  const float dr = row_ok ? p.drow[(size_t)bh * p.N + qrow] : 0.f;
  f32x16 acc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) acc[cb] = f32x16{};
  const int nk = (p.N + KB - 1) / KB;
  const int n_kt = CAUSAL ? min(nk, (q0 + BM + KB - 1) / KB) : nk;

  TileRegs<D, KB> kr, vr;
  kr.load(kh, 0, p.N);
  vr.load(vh, 0, p.N);
  kr.store(Ks);
  vr.store(Vs);
  __syncthreads();
  for (int kt = 0; kt < n_kt; ++kt) {
    const int k0 = kt * KB;
    const int cur = (kt & 1) * TILE, nxt = TILE - cur;
    const bool more = kt + 1 < n_kt;
    if (more) {
      kr.load(kh, k0 + KB, p.N);
      vr.load(vh, k0 + KB, p.N);
    }
    if (!(CAUSAL && k0 > wrow0 + 31)) {
      const int klim = CAUSAL ? min(qrow, p.N - 1) : p.N - 1;
      if ((CAUSAL && k0 + KB - 1 > wrow0) || (k0 + KB > p.N))
        dq_tile<D, NMB, true>(acc, Ks + cur, Vs + cur, qf, df, k0, klim, lse2, dr, lane);
      else
        dq_tile<D, NMB, false>(acc, Ks + cur, Vs + cur, qf, df, k0, klim, lse2, dr, lane);
    }
    if (more) {
      kr.store(Ks + nxt);
      vr.store(Vs + nxt);
    }
    __syncthreads();
  }

  float wv[D / 4];
#pragma unroll
  for (int i = 0; i < D / 4; ++i) wv[i] = 0.f;
  if (row_ok)
    finish_rows<D>(acc, p.scale, nullptr, p.cs + (size_t)qrow * (D / 2), p.q,
                   head + (size_t)qrow * D, p.bf16, p.dq + head + (size_t)qrow * D, (float)qrow, wv,
                   g);
  store_dalpha<D>(wv, red, p.dalpha_part + (size_t)slot * (D / 2), g);
}

// ------------------------------------------------------------------ dK, dV
// Workgroup = 128 keys of one head (4 waves x 32 keys); streams QB-row
// tiles of Q~ and dO (plus their LSE and D values).  Q~ serves the score
// product and dK~ += dS^T Q~; dO serves dP = dO V^T and dV += P^T dO.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, RA_DKDV_WPS) void dkdv_kernel(MfmaParams p) {
  constexpr int QB = RA_DKDV_BN, NMB = QB / 32;
  constexpr int DT = D / 16, CB = D / 32, TILE = QB * (D + 8);
  __shared__ __attribute__((aligned(16))) half_t Qs[2 * TILE];
  __shared__ __attribute__((aligned(16))) half_t Ds[2 * TILE];
  __shared__ __attribute__((aligned(16))) float lses[2 * QB];
  __shared__ __attribute__((aligned(16))) float drs[2 * QB];
  __shared__ float red[4 * (D / 2)];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, l32 = lane & 31, g = lane >> 5;
  const int BH = p.B * p.H;
  const int ntiles = (p.N + BM - 1) / BM;
  int bh, t;
  // key tile t has the N - 128 t query rows after it under the causal
  // mask: low tiles are the heavy ones
  map_block(blockIdx.x, BH, ntiles, false, bh, t);
  const int slot = p.slot0 + blockIdx.x;
  const int k0 = t * BM, wkey0 = k0 + 32 * w, key = wkey0 + l32;
  const size_t head = (size_t)bh * p.N * D;
  const half_t* qh = p.qh + head;
  const half_t* doh = p.doh + head;
  const float* lse_h = p.lse + (size_t)bh * p.N;
  const float* dr_h = p.drow + (size_t)bh * p.N;

  half8 kf[DT], vf[DT];
  load_frag_rows<D>(kf, p.kh + head, key, p.N, g);
  load_frag_rows<D>(vf, p.vh + head, key, p.N, g);
  f32x16 dk[CB], dv[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) { dk[cb] = f32x16{}; dv[cb] = f32x16{}; }
  int qs0 = CAUSAL ? k0 : 0;
  if (qs0 < p.corner) qs0 = p.corner;  // pairs with query rows < corner: exact path
  const int n_it = qs0 < p.N ? (p.N - qs0 + QB - 1) / QB : 0;

  TileRegs<D, QB> qr, dr;
  float lv = INFINITY, dvv = 0.f;   // row scalars held by threads < QB
  auto load_rows = [&](int r0) {
    qr.load(qh, r0, p.N);
    dr.load(doh, r0, p.N);
    if (threadIdx.x < QB) {
      const int row = r0 + threadIdx.x;
      const bool ok = row < p.N;
      lv = ok ? lse_h[ok ? row : 0] * LOG2E : INFINITY;
      dvv = ok ? dr_h[ok ? row : 0] : 0.f;
    }
  };
  auto store_rows = [&](int buf) {
    qr.store(Qs + buf * TILE);
    dr.store(Ds + buf * TILE);
    if (threadIdx.x < QB) {
      lses[buf * QB + threadIdx.x] = lv;
      drs[buf * QB + threadIdx.x] = dvv;
    }
  };
  if (n_it > 0) {
    load_rows(qs0);
    store_rows(0);
  }
  __syncthreads();
  for (int it = 0; it < n_it; ++it) {
    const int r0 = qs0 + it * QB;
    const int cur = it & 1;
    const bool more = it + 1 < n_it;
    if (more) load_rows(r0 + QB);
    if (!(CAUSAL && wkey0 > r0 + QB - 1)) {  // skip tiles wholly before this wave's keys
      const half_t* qt = Qs + cur * TILE;
      const half_t* dt = Ds + cur * TILE;
      if (CAUSAL && wkey0 + 31 > r0)
        dkdv_tile<D, NMB, true>(dk, dv, qt, dt, lses + cur * QB, drs + cur * QB, kf, vf, r0, key, lane);
      else
        dkdv_tile<D, NMB, false>(dk, dv, qt, dt, lses + cur * QB, drs + cur * QB, kf, vf, r0, key, lane);
    }
    if (more) store_rows(cur ^ 1);
    __syncthreads();
  }

  float wv[D / 4];
#pragma unroll
  for (int i = 0; i < D / 4; ++i) wv[i] = 0.f;
  if (key < p.N) {
    const bool has_part = p.dk_part && key < p.corner;
    const float* dkp = has_part ? p.dk_part + ((size_t)bh * p.corner + key) * D : nullptr;
    const float* dvp = has_part ? p.dv_part + ((size_t)bh * p.corner + key) * D : nullptr;
    // Q~ carries log2(e)/sqrt(D): dK~ = dS^T Q~ / sqrt(D) = ln 2 * (dS^T Q~')
    finish_rows<D>(dk, LN2, dkp, p.cs + (size_t)key * (D / 2), p.k, head + (size_t)key * D,
                   p.bf16, p.dk + head + (size_t)key * D, (float)key, wv, g);
    float* dvrow = p.dv + head + (size_t)key * D;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int c = 32 * cb + 8 * rq + 4 * g;
        float4 v = make_float4(dv[cb][4 * rq], dv[cb][4 * rq + 1], dv[cb][4 * rq + 2], dv[cb][4 * rq + 3]);
        if (dvp) {
          const float4 pr = *reinterpret_cast<const float4*>(dvp + c);
          v.x += pr.x; v.y += pr.y; v.z += pr.z; v.w += pr.w;
        }
        *reinterpret_cast<float4*>(dvrow + c) = v;
      }
    }
  }
  store_dalpha<D>(wv, red, p.dalpha_part + (size_t)slot * (D / 2), g);
}

int fwd_blocks(const MfmaParams& p) {
  const int ntiles = (p.N + BM - 1) / BM;
  return p.B * p.H * (ntiles - p.corner / BM);
}
int dkdv_blocks(const MfmaParams& p) { return p.B * p.H * ((p.N + BM - 1) / BM); }

}  // namespace

int dq_mfma_slots(const MfmaParams& p) { return fwd_blocks(p); }
int dkdv_mfma_slots(const MfmaParams& p) { return dkdv_blocks(p); }

#define RA_LAUNCH(KERNEL, BLOCKS)                                                               \
  do {                                                                                         \
    const dim3 grid((unsigned)(BLOCKS)), block(256);                                           \
    if (p.D == 64) {                                                                           \
      if (p.causal) hipLaunchKernelGGL((KERNEL<64, true>), grid, block, 0, s, p);              \
      else hipLaunchKernelGGL((KERNEL<64, false>), grid, block, 0, s, p);                      \
    } else {                                                                                   \
      if (p.causal) hipLaunchKernelGGL((KERNEL<128, true>), grid, block, 0, s, p);             \
      else hipLaunchKernelGGL((KERNEL<128, false>), grid, block, 0, s, p);                     \
    }                                                                                          \
  } while (0)

void launch_fwd_mfma(const MfmaParams& p, hipStream_t s) {
  const int nb = p.B * p.H * ((p.N + FWD_BM - 1) / FWD_BM);
  if (nb > 0) RA_LAUNCH(fwd_kernel, nb);
}
void launch_dq_mfma(const MfmaParams& p, hipStream_t s) {
  const int nb = fwd_blocks(p);
  if (nb > 0) RA_LAUNCH(dq_kernel, nb);
}
void launch_dkdv_mfma(const MfmaParams& p, hipStream_t s) {
  const int nb = dkdv_blocks(p);
  if (nb > 0) RA_LAUNCH(dkdv_kernel, nb);
}

}  // namespace ra
