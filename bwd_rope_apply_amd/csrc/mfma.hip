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

constexpr int BN = 64;     // keys (fwd, dq) or queries (dkdv) per loop step
constexpr int BM = 128;    // stationary rows per workgroup (4 waves x 32)

__device__ __forceinline__ int perm(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
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
template <int D>
struct TileRegs {
  static constexpr int CPR = D / 8;
  static constexpr int NCH = BN * CPR / 256;
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
      *reinterpret_cast<half8*>(dst + (ch / CPR) * (D + 8) + (ch % CPR) * 8) = x[i];
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

// Two 32-key score blocks (keys along m, this lane's query along n).
template <int D>
__device__ __forceinline__ void scores(f32x16* s, const half_t* lds, const half8* bf, int l32,
                                       int g) {
  constexpr int LD = D + 8;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    f32x16 acc = {};
    const half_t* row = lds + (32 * mb + perm(l32)) * LD + 8 * g;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) acc = mfma(*reinterpret_cast<const half8*>(row + 16 * t), bf[t], acc);
    s[mb] = acc;
  }
}

// Pack register values of two score blocks into the four 16-key B-operand
// fragments (k step t holds keys 16t + 8g + e).
__device__ __forceinline__ void to_frags(const f32x16* s, half8* f) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
#pragma unroll
    for (int e = 0; e < 8; ++e) f[t][e] = (half_t)s[t >> 1][8 * (t & 1) + e];
  }
}

typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(2))) short s16x2;

__device__ __forceinline__ s16x4 ds_read_tr(const half_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}

// acc[cb] += X^T(columns 32cb.., rows = 16-wide k steps) * frag, with X the
// natural [BN][D + 8] tile in LDS.  ds_read_b64_tr_b16 transposes a 4 x 16
// block per 16-lane group (lane j receives element j of the 4 rows that
// lanes 4e + j/4 point at), so lane s of a group points at row s/4, columns
// 4 (s % 4) .. +3 of its block, and two reads give the 8 k-values (rows
// 16t + 8g + 0..7) of column 32cb + l32.
template <int D>
__device__ __forceinline__ void accumulate_tr(f32x16* acc, const half_t* lds, const half8* f, int lane) {
  constexpr int LD = D + 8;
  const int s16 = lane & 15, g = lane >> 5;
  const half_t* base = lds + (8 * g + (s16 >> 2)) * LD + 16 * ((lane >> 4) & 1) + 4 * (s16 & 3);
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const half_t* p = base + 16 * t * LD + 32 * cb;
      const s16x4 lo = ds_read_tr(p), hi = ds_read_tr(p + 4 * LD);
      typedef __attribute__((ext_vector_type(8))) short s16x8;
      const s16x8 both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      const half8 a = __builtin_bit_cast(half8, both);
      acc[cb] = mfma(a, f[t], acc[cb]);
    }
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

// One 64-key step of the forward for one wave: scores, online softmax
// (running max m and sum l per query, in log2 units), O += P V.  MASK hides
// keys after klim (causal diagonal, ragged tail).
template <int D, bool MASK>
__device__ __forceinline__ void fwd_tile(f32x16* o, float& m, float& l, const half_t* Ks,
                                         const half_t* Vs, const half8* qf, int k0, int klim,
                                         float c2, int lane) {
  const int l32 = lane & 31, g = lane >> 5;
  f32x16 s[2];
  scores<D>(s, Ks, qf, l32, g);
  float mx = -INFINITY;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float x = s[mb][r] * c2;
      if (MASK) {
        const int key = k0 + 32 * mb + 16 * (r >> 3) + 8 * g + (r & 7);
        x = key > klim ? -INFINITY : x;
      }
      s[mb][r] = x;
      mx = fmaxf(mx, x);
    }
  }
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  const float mn = fmaxf(m, mx);
  const float ms = (mn == -INFINITY) ? 0.f : mn;
  const float alpha = exp2_fast(m - ms);
  float ls = 0.f;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float pr = exp2_fast(s[mb][r] - ms);
      s[mb][r] = pr;
      ls += pr;
    }
  }
  l = l * alpha + ls;
  m = mn;
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb) o[cb] *= alpha;
  half8 pf[4];
  to_frags(s, pf);
  accumulate_tr<D>(o, Vs, pf, lane);
}

// One 64-key step of dQ for one wave: recompute P from the LSE,
// dP = dO V^T, dS = P o (dP - D), dQ~ += dS K~.
template <int D, bool MASK>
__device__ __forceinline__ void dq_tile(f32x16* acc, const half_t* Ks, const half_t* Vs,
                                        const half8* qf, const half8* df, int k0, int klim,
                                        float c2, float lse2, float dr, int lane) {
  const int l32 = lane & 31, g = lane >> 5;
  f32x16 s[2], dp[2];
  scores<D>(s, Ks, qf, l32, g);
  scores<D>(dp, Vs, df, l32, g);
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float pr = exp2_fast(s[mb][r] * c2 - lse2);
      if (MASK) {
        const int key = k0 + 32 * mb + 16 * (r >> 3) + 8 * g + (r & 7);
        pr = key > klim ? 0.f : pr;
      }
      s[mb][r] = pr * (dp[mb][r] - dr);
    }
  }
  half8 sf[4];
  to_frags(s, sf);
  accumulate_tr<D>(acc, Ks, sf, lane);
}

// One 64-query step of dK, dV for one wave (this lane's key along n):
// P = exp(S - LSE), dV += P^T dO, dP = dO V^T, dS = P o (dP - D),
// dK~ += dS^T Q~.  MASK hides queries before this lane's key.
template <int D, bool MASK>
__device__ __forceinline__ void dkdv_tile(f32x16* dk, f32x16* dv, const half_t* Qs,
                                          const half_t* Ds, const float* lses, const float* drs,
                                          const half8* kf, const half8* vf, int r0, int key,
                                          float c2, int lane) {
  const int l32 = lane & 31, g = lane >> 5;
  f32x16 s[2], dp[2];
  scores<D>(s, Qs, kf, l32, g);
  scores<D>(dp, Ds, vf, l32, g);
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
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
        float pr = exp2_fast(s[mb][r] * c2 - lv8[e]);
        if (MASK) pr = key > r0 + ql + e ? 0.f : pr;
        s[mb][r] = pr;
        dp[mb][r] = pr * (dp[mb][r] - dv8[e]);
      }
    }
  }
  half8 pf[4], sf[4];
  to_frags(s, pf);
  to_frags(dp, sf);
  accumulate_tr<D>(dv, Ds, pf, lane);
  accumulate_tr<D>(dk, Qs, sf, lane);
}

// ------------------------------------------------------------------ forward
// Workgroup = 128 query rows of one head (4 waves x 32 rows); the loop
// streams 64-key tiles of K~ and V through double-buffered LDS, the next
// tile's global loads in flight while the current tile is computed.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void fwd_kernel(MfmaParams p) {
  constexpr int DT = D / 16, CB = D / 32, LD = D + 8, TILE = BN * LD;
  __shared__ __attribute__((aligned(16))) half_t Ks[2 * TILE];
  __shared__ __attribute__((aligned(16))) half_t Vs[2 * TILE];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, l32 = lane & 31, g = lane >> 5;
  const int BH = p.B * p.H;
  const int ntiles = (p.N + BM - 1) / BM, t0 = p.corner / BM;
  int bh, t;
  map_block(blockIdx.x, BH, ntiles - t0, true, bh, t);
  t += t0;
  const int q0 = t * BM, wrow0 = q0 + 32 * w, qrow = wrow0 + l32;
  const size_t head = (size_t)bh * p.N * D;
  const half_t* kh = p.kh + head;
  const half_t* vh = p.vh + head;

  half8 qf[DT];
  load_frag_rows<D>(qf, p.qh + head, qrow, p.N, g);
  f32x16 o[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) o[cb] = f32x16{};
  float m = -INFINITY, l = 0.f;
  const float c2 = p.scale * LOG2E;
  const int nk = (p.N + BN - 1) / BN;
  const int n_kt = CAUSAL ? min(nk, (q0 + BM + BN - 1) / BN) : nk;

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
    if (!(CAUSAL && k0 > wrow0 + 31)) {  // skip tiles wholly above this wave's rows
      const int klim = CAUSAL ? min(qrow, p.N - 1) : p.N - 1;  // last visible key
      if ((CAUSAL && k0 + BN - 1 > wrow0) || (k0 + BN > p.N))
        fwd_tile<D, true>(o, m, l, Ks + cur, Vs + cur, qf, k0, klim, c2, lane);
      else
        fwd_tile<D, false>(o, m, l, Ks + cur, Vs + cur, qf, k0, klim, c2, lane);
    }
    if (more) {
      kr.store(Ks + nxt);
      vr.store(Vs + nxt);
    }
    __syncthreads();
  }

  const float lt = l + __shfl_xor(l, 32, 64);
  if (qrow < p.N) {
    const float inv = 1.f / lt;
    float* orow = p.o + head + (size_t)qrow * D;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int c = 32 * cb + 8 * rq + 4 * g;
        *reinterpret_cast<float4*>(orow + c) =
            make_float4(o[cb][4 * rq] * inv, o[cb][4 * rq + 1] * inv, o[cb][4 * rq + 2] * inv,
                        o[cb][4 * rq + 3] * inv);
      }
    }
    if (g == 0) p.out_lse[(size_t)bh * p.N + qrow] = (m + __log2f(lt)) * LN2;
  }
}

// ------------------------------------------------------------------ dQ
// Workgroup = 128 query rows; streams 64-key tiles of K~ and V.  The K~
// tile serves both the score product (natural reads) and dQ~ += dS K~
// (transposed reads).
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void dq_kernel(MfmaParams p) {
  constexpr int DT = D / 16, CB = D / 32, LD = D + 8, TILE = BN * LD;
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
  const float c2 = p.scale * LOG2E;
  const int nk = (p.N + BN - 1) / BN;
  const int n_kt = CAUSAL ? min(nk, (q0 + BM + BN - 1) / BN) : nk;

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
    if (!(CAUSAL && k0 > wrow0 + 31)) {
      const int klim = CAUSAL ? min(qrow, p.N - 1) : p.N - 1;
      if ((CAUSAL && k0 + BN - 1 > wrow0) || (k0 + BN > p.N))
        dq_tile<D, true>(acc, Ks + cur, Vs + cur, qf, df, k0, klim, c2, lse2, dr, lane);
      else
        dq_tile<D, false>(acc, Ks + cur, Vs + cur, qf, df, k0, klim, c2, lse2, dr, lane);
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
// Workgroup = 128 keys of one head (4 waves x 32 keys); streams 64-row
// tiles of Q~ and dO (plus their LSE and D values).  Q~ serves the score
// product and dK~ += dS^T Q~; dO serves dP = dO V^T and dV += P^T dO.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void dkdv_kernel(MfmaParams p) {
  constexpr int DT = D / 16, CB = D / 32, LD = D + 8, TILE = BN * LD;
  __shared__ __attribute__((aligned(16))) half_t Qs[2 * TILE];
  __shared__ __attribute__((aligned(16))) half_t Ds[2 * TILE];
  __shared__ __attribute__((aligned(16))) float lses[2 * BN];
  __shared__ __attribute__((aligned(16))) float drs[2 * BN];
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
  const float c2 = p.scale * LOG2E;
  int qs0 = CAUSAL ? k0 : 0;
  if (qs0 < p.corner) qs0 = p.corner;  // pairs with query rows < corner: exact path
  const int n_it = qs0 < p.N ? (p.N - qs0 + BN - 1) / BN : 0;

  TileRegs<D> qr, dr;
  float lv = INFINITY, dvv = 0.f;   // row scalars held by threads < BN
  auto load_rows = [&](int r0) {
    qr.load(qh, r0, p.N);
    dr.load(doh, r0, p.N);
    if (threadIdx.x < BN) {
      const int row = r0 + threadIdx.x;
      const bool ok = row < p.N;
      lv = ok ? lse_h[ok ? row : 0] * LOG2E : INFINITY;
      dvv = ok ? dr_h[ok ? row : 0] : 0.f;
    }
  };
  auto store_rows = [&](int buf) {
    qr.store(Qs + buf * TILE);
    dr.store(Ds + buf * TILE);
    if (threadIdx.x < BN) {
      lses[buf * BN + threadIdx.x] = lv;
      drs[buf * BN + threadIdx.x] = dvv;
    }
  };
  if (n_it > 0) {
    load_rows(qs0);
    store_rows(0);
  }
  __syncthreads();
  for (int it = 0; it < n_it; ++it) {
    const int r0 = qs0 + it * BN;
    const int cur = it & 1;
    const bool more = it + 1 < n_it;
    if (more) load_rows(r0 + BN);
    if (!(CAUSAL && wkey0 > r0 + BN - 1)) {  // skip tiles wholly before this wave's keys
      const half_t* qt = Qs + cur * TILE;
      const half_t* dt = Ds + cur * TILE;
      if (CAUSAL && wkey0 + 31 > r0)
        dkdv_tile<D, true>(dk, dv, qt, dt, lses + cur * BN, drs + cur * BN, kf, vf, r0, key, c2, lane);
      else
        dkdv_tile<D, false>(dk, dv, qt, dt, lses + cur * BN, drs + cur * BN, kf, vf, r0, key, c2, lane);
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
    finish_rows<D>(dk, p.scale, dkp, p.cs + (size_t)key * (D / 2), p.k, head + (size_t)key * D,
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
  const int nb = fwd_blocks(p);
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
