// Causal corner with split fp16 operands (bf16 inputs): query rows
// [0, corner) and the keys they see.  Every rotated operand is x = hi + lo
// (hi = fp16(x), lo = fp16(x - hi), ~22 bits), and each product is
// hi*hi + hi*lo + lo*hi on v_mfma_f32_32x32x16_f16 (V and dO are exact in
// fp16 -- dO after its per-head power-of-two scale -- so their products need
// only P or dS split).  The rows in the corner average few keys, so they
// carry the largest entries of O, dQ, dK and dV; computing them to ~fp32
// accuracy keeps the whole tensors within 2e-2 of their RMS.
//
// What is computed is the same as in mfma.hip ("RoPE attention can be
// trained in almost-linear time", Methodology 1 and 2): s(x), O = P V,
// beta = dO V^T, dS = P o (beta - D), and the gradients through the scores.
//
// The backward's corner parts run as the first workgroups of the dQ
// launch, so their latency-bound chains overlap the dQ product instead of
// taking a launch of their own: dQ of the corner rows, and the corner's
// share of dK and dV for keys < corner, which is added to the dK, dV that
// the dK/dV pass (all later queries of those keys) wrote before.  Their LDS
// comes from the launch's pool (corner_bwd_smem bytes).
#pragma once

#include "tile.h"

namespace ra {
namespace {

// Loads one streamed [ROWS][D] tile of the hi plane, the lo plane (rows <
// nlo) and a third exact plane into LDS.
// At most two tiles' registers are live at once (the backward's corner
// bodies run inside another launch's register budget).
template <int D, int ROWS>
__device__ __forceinline__ void stage3(half_t* a, const half_t* sa, half_t* b, const half_t* sb,
                                       half_t* c, const half_t* sc, int r0, int N, int nlo) {
  TileRegs<D, ROWS> ra_, rb_;
  ra_.load(sa, r0, N);
  rb_.load(sb, r0, nlo);
  ra_.store(a);
  ra_.load(sc, r0, N);
  rb_.store(b);
  ra_.store(c);
}

// The backward's corner steps: 32 rows of the streamed operand each (one
// 32 x 32 score block per wave), which keeps every corner body within the
// dQ launch's register budget.
constexpr int CBN = 32;

__host__ __device__ constexpr int corner_tile_halfs(int D, int rows) { return rows * (D + 8); }

// LDS bytes of any backward corner body: three tiles, two row-scalar
// vectors, the d alpha reduction buffer and (dQ part) the rows' dO.
__host__ __device__ constexpr size_t corner_bwd_smem(int D) {
  return 3 * (size_t)corner_tile_halfs(D, CBN) * 2 + 2 * CBN * 4 + 4 * (D / 2) * 4 +
         (size_t)BM * (D + 8) * 2;
}

// Workgroups of each backward corner part: one per 128 corner rows of a head.
__host__ __device__ inline int corner_blocks(const MfmaParams& p) {
  return p.B * p.H * ((p.corner + BM - 1) / BM);
}

// ------------------------------------------------------------------ forward
// LDS bytes of the forward's corner body: three 32-row tiles.
__host__ __device__ constexpr size_t corner_fwd_smem(int D) {
  return 3 * (size_t)corner_tile_halfs(D, CBN) * 2;
}

// Column blocks (32 columns) per pass of the corner's forward.
constexpr int CORNER_FWD_CBP = 1;

// Step counts of the corner bodies.  Every step of a body holds two
// barriers, so the idle waves of an 8-wave workgroup (corner_fwd_idle,
// corner_bwd_idle) take their counts from these same functions.
// Key steps of the forward and dQ bodies for the 128-row query block at q0:
__device__ __forceinline__ int corner_q_steps(const MfmaParams& p, int q0) {
  return q0 < p.N ? min((p.N + CBN - 1) / CBN, (q0 + BM + CBN - 1) / CBN) : 0;
}
// Query steps of the dK, dV share bodies for the key block at k0 (the query
// rows below the corner, from k0 on):
__device__ __forceinline__ int corner_kv_steps(const MfmaParams& p, int k0) {
  const int nlo = min(p.N, p.corner);
  return k0 < nlo ? (nlo - k0 + CBN - 1) / CBN : 0;
}

// O and LSE of query rows [128 t, 128 t + 128) below the corner (corner
// workgroup `bid`), run as the last workgroups of the forward launch.  O is
// built 32 columns at a time, each pass streaming the keys again (the
// scores and the softmax statistics come out bit-identical in every pass),
// so that the body fits the forward's register budget.
template <int D>
__device__ __forceinline__ void corner_fwd(const MfmaParams& p, int bid, char* smem) {
  constexpr int DT = D / 16, CB = D / 32, TILE = corner_tile_halfs(D, CBN);
  constexpr int CBP = CORNER_FWD_CBP;
  half_t* Kh = reinterpret_cast<half_t*>(smem);
  half_t* Kl = Kh + TILE;
  half_t* Vs = Kl + TILE;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, l32 = lane & 31, g = lane >> 5;
  const int BH = p.B * p.H;
  const int bh = bid % BH, t = bid / BH;
  const int q0 = t * BM, wrow0 = q0 + 32 * w, qrow = wrow0 + l32;
  if (q0 >= p.N) return;  // whole workgroup
  const int nlo = min(p.N, p.corner);
  const size_t head = (size_t)bh * p.N * D, lhead = (size_t)bh * p.corner * D;

  half8 qf[DT], ql[DT];
  load_frag_rows<D>(qf, p.qh + head, qrow, p.N, g);
  load_frag_rows<D>(ql, p.qlo + lhead, qrow, nlo, g);
  const int klim = min(qrow, p.N - 1);
  const int n_kt = corner_q_steps(p, q0);
  const bool row_ok = qrow < p.N && qrow < p.corner;
  float* orow = p.o + head + (size_t)qrow * D;
#pragma unroll 1
  for (int cb0 = 0; cb0 < CB; cb0 += CBP) {
    f32x16 o[CBP];
#pragma unroll
    for (int c = 0; c < CBP; ++c) o[c] = f32x16{};
    float m = -INFINITY, l = 0.f;
    for (int kt = 0; kt < n_kt; ++kt) {
      const int k0 = kt * CBN;
      __syncthreads();
      stage3<D, CBN>(Kh, p.kh + head, Kl, p.klo + lhead, Vs, p.vh + head, k0, p.N, nlo);
      __syncthreads();
      if (k0 > wrow0 + 31) continue;
      f32x16 s[1];
      scores<D, 1>(s, Kh, qf, l32, g);
      scores_add<D, 1>(s, Kl, qf, l32, g);
      scores_add<D, 1>(s, Kh, ql, l32, g);
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + 16 * (r >> 3) + 8 * g + (r & 7);
        const float x = key > klim ? -INFINITY : s[0][r];   // log2 units
        s[0][r] = x;
        mx = fmaxf(mx, x);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mn = fmaxf(m, mx);
      const float ms = mn == -INFINITY ? 0.f : mn;
      const float alpha = exp2_fast(m - ms);
      float ls = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pr = exp2_fast(s[0][r] - ms);
        s[0][r] = pr;
        ls += pr;
      }
      l = l * alpha + ls;
      m = mn;
#pragma unroll
      for (int c = 0; c < CBP; ++c) o[c] *= alpha;
      half8 ph[2], pl[2];
      to_frags_split<1>(s, ph, pl);
#pragma unroll
      for (int c = 0; c < CBP; ++c) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const half8 a = tr_frag<D>(Vs, tt, cb0 + c, lane);
          o[c] = mfma(a, ph[tt], o[c]);
          o[c] = mfma(a, pl[tt], o[c]);
        }
      }
    }
    const float lt = l + __shfl_xor(l, 32, 64);
    if (row_ok) {
      const float inv = 1.f / lt;
#pragma unroll
      for (int c = 0; c < CBP; ++c) {
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int col = 32 * (cb0 + c) + 8 * rq + 4 * g;
          *reinterpret_cast<float4*>(orow + col) =
              make_float4(o[c][4 * rq] * inv, o[c][4 * rq + 1] * inv, o[c][4 * rq + 2] * inv,
                          o[c][4 * rq + 3] * inv);
        }
      }
      if (cb0 == 0 && g == 0) p.out_lse[(size_t)bh * p.N + qrow] = (m + __log2f(lt)) * LN2;
    }
  }
}

// The waves past the first four of a corner workgroup in a launch of 8-wave
// workgroups: they take part in corner_fwd's barriers (two per key step,
// per column pass) and do nothing else.
template <int D>
__device__ __forceinline__ void corner_fwd_idle(const MfmaParams& p, int bid) {
  constexpr int CB = D / 32, CBP = CORNER_FWD_CBP;
  const int q0 = (bid / (p.B * p.H)) * BM;
  if (q0 >= p.N) return;  // whole workgroup
  const int n_kt = corner_q_steps(p, q0);
#pragma unroll 1
  for (int cb0 = 0; cb0 < CB; cb0 += CBP) {
    for (int kt = 0; kt < n_kt; ++kt) {
      __syncthreads();
      __syncthreads();
    }
  }
}

// ------------------------------------------------------------------ dQ
// dQ of query rows [128 t, 128 t + 128) below the corner (d alpha slot `slot`).
template <int D>
__device__ __forceinline__ void corner_dq(const MfmaParams& p, int bid, int slot, char* smem) {
  constexpr int DT = D / 16, CB = D / 32, TILE = corner_tile_halfs(D, CBN);
  half_t* Kh = reinterpret_cast<half_t*>(smem);
  half_t* Kl = Kh + TILE;
  half_t* Vs = Kl + TILE;
  float* red = reinterpret_cast<float*>(Vs + TILE) + 2 * CBN;
  half_t* Dq = reinterpret_cast<half_t*>(red + 4 * (D / 2));   // the rows' dO, [BM][D + 8]
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, l32 = lane & 31, g = lane >> 5;
  const int BH = p.B * p.H;
  const int bh = bid % BH, t = bid / BH;
  const int q0 = t * BM, wrow0 = q0 + 32 * w, qrow = wrow0 + l32;
  const int nlo = min(p.N, p.corner);
  const size_t head = (size_t)bh * p.N * D, lhead = (size_t)bh * p.corner * D;
  const bool row_ok = qrow < nlo;

  half8 qf[DT], ql[DT];
  load_frag_rows<D>(qf, p.qh + head, qrow, p.N, g);
  load_frag_rows<D>(ql, p.qlo + lhead, qrow, nlo, g);
  // dO of the workgroup's rows stays in LDS (read where dP needs it), which
  // keeps this body within the launch's registers
  for (int ch = threadIdx.x; ch < BM * (D / 8); ch += 256) {
    const int r = ch / (D / 8), c8 = ch % (D / 8);
    const int row = min(q0 + r, p.N - 1);
    *reinterpret_cast<half8*>(Dq + r * (D + 8) + c8 * 8) =
        *reinterpret_cast<const half8*>(p.doh + head + (size_t)row * D + c8 * 8);
  }
  const half_t* drow_lds = Dq + (32 * w + l32) * (D + 8) + 8 * g;
  const float lse2 = row_ok ? p.lse[(size_t)bh * p.N + qrow] * LOG2E : 0.f;
  const float dr = row_ok ? p.drow[(size_t)bh * p.N + qrow] : 0.f;
  f32x16 acc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) acc[cb] = f32x16{};
  const int klim = min(qrow, p.N - 1);
  const int n_kt = corner_q_steps(p, q0);
  for (int kt = 0; kt < n_kt; ++kt) {
    const int k0 = kt * CBN;
    __syncthreads();
    stage3<D, CBN>(Kh, p.kh + head, Kl, p.klo + lhead, Vs, p.vh + head, k0, p.N, nlo);
    __syncthreads();
    if (k0 > wrow0 + 31) continue;
    f32x16 s[1], dp[1];
    scores<D, 1>(s, Kh, qf, l32, g, -lse2);
    scores_add<D, 1>(s, Kl, qf, l32, g);
    scores_add<D, 1>(s, Kh, ql, l32, g);
    {
      half8 df[DT];
#pragma unroll
      for (int tt = 0; tt < DT; ++tt) df[tt] = *reinterpret_cast<const half8*>(drow_lds + 16 * tt);
      scores<D, 1>(dp, Vs, df, l32, g, -dr);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = k0 + 16 * (r >> 3) + 8 * g + (r & 7);
      const float pr = key > klim ? 0.f : exp2_fast(s[0][r]);
      s[0][r] = pr * dp[0][r];
    }
    half8 sh[2], sl[2];
    to_frags_split<1>(s, sh, sl);
    accumulate_tr<D, 2>(acc, Kh, sh, lane);
    accumulate_tr<D, 2>(acc, Kh, sl, lane);
    accumulate_tr<D, 2>(acc, Kl, sh, lane);
  }
  float wv[D / 4];
#pragma unroll
  for (int i = 0; i < D / 4; ++i) wv[i] = 0.f;
  if (row_ok)
    finish_rows<D>(acc, p.scale * dscale_inv(p.dsc, bh), nullptr, p.cs + (size_t)qrow * (D / 2),
                   p.q, head + (size_t)qrow * D, p.bf16, p.dq + head + (size_t)qrow * D,
                   (float)qrow, wv, g);
  store_dalpha<D>(wv, red, p.dalpha_part + (size_t)slot * (D / 2), g);
}

// ------------------------------------------------------------------ dK, dV
// Keys [128 t, 128 t + 128) below the corner against query rows [key,
// corner): their share of dV (DK false) or of dK (DK true), un-rotated and
// with the dO scale undone, added to the rows the dK/dV pass wrote (it
// covers every query at or past the corner).  The dK part's slot takes the
// d alpha part of its contribution; the dV part's slot is zero.  Split in
// two workgroups so that each fits the launch's register budget.
template <int D, bool DK>
__device__ __forceinline__ void corner_kv(const MfmaParams& p, int bid, int slot, char* smem) {
  constexpr int DT = D / 16, CB = D / 32, TILE = corner_tile_halfs(D, CBN);
  half_t* Qh = reinterpret_cast<half_t*>(smem);
  half_t* Ql = Qh + TILE;
  half_t* Ds = Ql + TILE;
  float* lses = reinterpret_cast<float*>(Ds + TILE);
  float* drs = lses + CBN;
  float* red = drs + CBN;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, l32 = lane & 31, g = lane >> 5;
  const int BH = p.B * p.H;
  const int bh = bid % BH, t = bid / BH;
  const int k0 = t * BM, wkey0 = k0 + 32 * w, key = wkey0 + l32;
  const int nlo = min(p.N, p.corner);
  const size_t head = (size_t)bh * p.N * D, lhead = (size_t)bh * p.corner * D;

  half8 kf[DT], kl[DT], vf[DK ? DT : 1];
  load_frag_rows<D>(kf, p.kh + head, key, p.N, g);
  load_frag_rows<D>(kl, p.klo + lhead, key, nlo, g);
  if constexpr (DK) load_frag_rows<D>(vf, p.vh + head, key, p.N, g);
  f32x16 acc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) acc[cb] = f32x16{};
  const int n_st = corner_kv_steps(p, k0);
  for (int st = 0; st < n_st; ++st) {
    const int r0 = k0 + st * CBN;
    __syncthreads();
    stage3<D, CBN>(Qh, p.qh + head, Ql, p.qlo + lhead, Ds, p.doh + head, r0, p.N, nlo);
    if (threadIdx.x < CBN) {
      const int row = r0 + threadIdx.x;
      const bool ok = row < nlo;   // query rows past the corner are not part of it
      lses[threadIdx.x] = ok ? p.lse[(size_t)bh * p.N + row] * LOG2E : INFINITY;
      drs[threadIdx.x] = ok ? p.drow[(size_t)bh * p.N + row] : 0.f;
    }
    __syncthreads();
    if (wkey0 > r0 + CBN - 1) continue;
    f32x16 s[1];
    scores<D, 1>(s, Qh, kf, l32, g);
    scores_add<D, 1>(s, Ql, kf, l32, g);
    scores_add<D, 1>(s, Qh, kl, l32, g);
    if constexpr (!DK) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qo = 16 * (r >> 3) + 8 * g + (r & 7);
        const float pr = exp2_fast(s[0][r] - lses[qo]);
        s[0][r] = key > r0 + qo ? 0.f : pr;
      }
      half8 ph[2], pl[2];
      to_frags_split<1>(s, ph, pl);
      accumulate_tr<D, 2>(acc, Ds, ph, lane);
      accumulate_tr<D, 2>(acc, Ds, pl, lane);
    } else {
      f32x16 dp[1];
      scores<D, 1>(dp, Ds, vf, l32, g);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qo = 16 * (r >> 3) + 8 * g + (r & 7);
        float pr = exp2_fast(s[0][r] - lses[qo]);
        pr = key > r0 + qo ? 0.f : pr;
        dp[0][r] = pr * (dp[0][r] - drs[qo]);
      }
      half8 sh[2], sl[2];
      to_frags_split<1>(dp, sh, sl);
      accumulate_tr<D, 2>(acc, Qh, sh, lane);
      accumulate_tr<D, 2>(acc, Qh, sl, lane);
      accumulate_tr<D, 2>(acc, Ql, sh, lane);
    }
  }
  float wv[D / 4];
#pragma unroll
  for (int i = 0; i < D / 4; ++i) wv[i] = 0.f;
  if (key < nlo) {
    const float dinv = dscale_inv(p.dsc, bh);
    if constexpr (DK) {
      // Q~ carries log2(e)/sqrt(D): dK~ = ln 2 * (dS^T Q~')
      finish_rows<D, true>(acc, LN2 * dinv, nullptr, p.cs + (size_t)key * (D / 2), p.k,
                           head + (size_t)key * D, p.bf16, p.dk + head + (size_t)key * D,
                           (float)key, wv, g);
    } else {
      float* dvrow = p.dv + head + (size_t)key * D;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int c = 32 * cb + 8 * rq + 4 * g;
          float4 v = *reinterpret_cast<const float4*>(dvrow + c);
          v.x += acc[cb][4 * rq] * dinv;
          v.y += acc[cb][4 * rq + 1] * dinv;
          v.z += acc[cb][4 * rq + 2] * dinv;
          v.w += acc[cb][4 * rq + 3] * dinv;
          *reinterpret_cast<float4*>(dvrow + c) = v;
        }
      }
    }
  }
  store_dalpha<D>(wv, red, p.dalpha_part + (size_t)slot * (D / 2), g);
}

// The waves past the first four of a corner workgroup in a dQ launch of
// 8-wave workgroups: they take part in the corner body's barriers and do
// nothing else.  corner_dq has two per 32-key step, corner_kv two per
// 32-row query step, and each one more in its d alpha reduction.
template <int D>
__device__ __forceinline__ void corner_bwd_idle(const MfmaParams& p, int bid) {
  const int n = corner_blocks(p), BH = p.B * p.H;
  const int steps = bid < n ? corner_q_steps(p, (bid / BH) * BM)
                            : corner_kv_steps(p, ((bid - (bid < 2 * n ? n : 2 * n)) / BH) * BM);
  for (int i = 0; i < 2 * steps + 1; ++i) __syncthreads();
}

// The corner workgroups of a dQ launch: [0, n) take dQ rows, [n, 2 n) the
// dV shares and [2 n, 3 n) the dK shares (n = corner_blocks); slots follow
// the workgroup index.
template <int D>
__device__ __forceinline__ void corner_bwd(const MfmaParams& p, int bid, char* smem) {
  const int n = corner_blocks(p);
  if (bid < n) corner_dq<D>(p, bid, p.slot0 + bid, smem);
  else if (bid < 2 * n) corner_kv<D, false>(p, bid - n, p.slot0 + bid, smem);
  else corner_kv<D, true>(p, bid - 2 * n, p.slot0 + bid, smem);
}

}  // namespace
}  // namespace ra
