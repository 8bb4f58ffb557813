// Causal corner with split fp16 operands (bf16 inputs): query rows
// [0, corner) and the keys they see.  Every rotated operand is x = hi + lo
// (hi = fp16(x), lo = fp16(x - hi), ~22 bits), and each product is
// hi*hi + hi*lo + lo*hi on v_mfma_f32_32x32x16_f16 (V and dO come from bf16
// inputs and are exact in fp16, so their products need only P or dS split).
// The rows in the corner average few keys, so they carry the largest
// entries of O, dQ, dK and dV; computing them to ~fp32 accuracy keeps the
// whole tensors within 2e-2 of their RMS.
//
// What is computed is the same as in mfma.hip ("RoPE attention can be
// trained in almost-linear time", Methodology 1 and 2): s(x), O = P V,
// beta = dO V^T, dS = P o (beta - D), and the gradients through the scores.
// The key side writes rotated-frame partial sums of dK~ and dV that the
// main dK/dV pass adds before un-rotating.
#include "tile.h"

namespace ra {

namespace {

// Loads one streamed [BN][D] tile of the hi plane, the lo plane (rows < nlo)
// and, optionally, a third exact plane into LDS.
template <int D>
__device__ __forceinline__ void stage3(half_t* a, const half_t* sa, half_t* b, const half_t* sb,
                                       half_t* c, const half_t* sc, int r0, int N, int nlo) {
  TileRegs<D> ra_, rb_, rc_;
  ra_.load(sa, r0, N);
  rb_.load(sb, r0, nlo);
  rc_.load(sc, r0, N);
  ra_.store(a);
  rb_.store(b);
  rc_.store(c);
}

// ------------------------------------------------------------------ forward
template <int D>
__global__ __launch_bounds__(256) void corner_fwd_kernel(MfmaParams p) {
  constexpr int DT = D / 16, CB = D / 32, TILE = BN * (D + 8);
  __shared__ __attribute__((aligned(16))) half_t Kh[TILE];
  __shared__ __attribute__((aligned(16))) half_t Kl[TILE];
  __shared__ __attribute__((aligned(16))) half_t Vs[TILE];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, l32 = lane & 31, g = lane >> 5;
  const int BH = p.B * p.H;
  const int bh = blockIdx.x % BH, t = blockIdx.x / BH;
  const int q0 = t * BM, wrow0 = q0 + 32 * w, qrow = wrow0 + l32;
  if (q0 >= p.N) return;  // whole workgroup
  const int nlo = min(p.N, p.corner);
  const size_t head = (size_t)bh * p.N * D, lhead = (size_t)bh * p.corner * D;

  half8 qf[DT], ql[DT];
  load_frag_rows<D>(qf, p.qh + head, qrow, p.N, g);
  load_frag_rows<D>(ql, p.qlo + lhead, qrow, nlo, g);
  f32x16 o[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) o[cb] = f32x16{};
  float m = -INFINITY, l = 0.f;
  const int klim = min(qrow, p.N - 1);
  const int n_kt = min((p.N + BN - 1) / BN, (q0 + BM + BN - 1) / BN);
  for (int kt = 0; kt < n_kt; ++kt) {
    const int k0 = kt * BN;
    __syncthreads();
    stage3<D>(Kh, p.kh + head, Kl, p.klo + lhead, Vs, p.vh + head, k0, p.N, nlo);
    __syncthreads();
    if (k0 > wrow0 + 31) continue;
    f32x16 s[2];
    scores<D>(s, Kh, qf, l32, g);
    scores_add<D>(s, Kl, qf, l32, g);
    scores_add<D>(s, Kh, ql, l32, g);
    float mx = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + 32 * mb + 16 * (r >> 3) + 8 * g + (r & 7);
        const float x = key > klim ? -INFINITY : s[mb][r];   // log2 units
        s[mb][r] = x;
        mx = fmaxf(mx, x);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mn = fmaxf(m, mx);
    const float ms = mn == -INFINITY ? 0.f : mn;
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
    for (int cb = 0; cb < CB; ++cb) o[cb] *= alpha;
    half8 ph[4], pl[4];
    to_frags_split(s, ph, pl);
    accumulate_tr<D>(o, Vs, ph, lane);
    accumulate_tr<D>(o, Vs, pl, lane);
  }
  const float lt = l + __shfl_xor(l, 32, 64);
  if (qrow < p.N && qrow < p.corner) {
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
// Workgroup bid of the dQ part (its own d alpha slot).
template <int D>
__device__ __forceinline__ void corner_dq(const MfmaParams& p, int bid) {
  constexpr int DT = D / 16, CB = D / 32, TILE = BN * (D + 8);
  __shared__ __attribute__((aligned(16))) half_t Kh[TILE];
  __shared__ __attribute__((aligned(16))) half_t Kl[TILE];
  __shared__ __attribute__((aligned(16))) half_t Vs[TILE];
  __shared__ float red[4 * (D / 2)];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, l32 = lane & 31, g = lane >> 5;
  const int BH = p.B * p.H;
  const int bh = bid % BH, t = bid / BH;
  const int q0 = t * BM, wrow0 = q0 + 32 * w, qrow = wrow0 + l32;
  const int slot = p.slot0 + bid;
  const int nlo = min(p.N, p.corner);
  const size_t head = (size_t)bh * p.N * D, lhead = (size_t)bh * p.corner * D;
  const bool row_ok = qrow < nlo;

  half8 qf[DT], ql[DT], df[DT];
  load_frag_rows<D>(qf, p.qh + head, qrow, p.N, g);
  load_frag_rows<D>(ql, p.qlo + lhead, qrow, nlo, g);
  load_frag_rows<D>(df, p.doh + head, qrow, p.N, g);
  const float lse2 = row_ok ? p.lse[(size_t)bh * p.N + qrow] * LOG2E : 0.f;
  const float dr = row_ok ? p.drow[(size_t)bh * p.N + qrow] : 0.f;
  f32x16 acc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) acc[cb] = f32x16{};
  const int klim = min(qrow, p.N - 1);
  const int n_kt = q0 < p.N ? min((p.N + BN - 1) / BN, (q0 + BM + BN - 1) / BN) : 0;
  for (int kt = 0; kt < n_kt; ++kt) {
    const int k0 = kt * BN;
    __syncthreads();
    stage3<D>(Kh, p.kh + head, Kl, p.klo + lhead, Vs, p.vh + head, k0, p.N, nlo);
    __syncthreads();
    if (k0 > wrow0 + 31) continue;
    f32x16 s[2], dp[2];
    scores<D>(s, Kh, qf, l32, g, -lse2);
    scores_add<D>(s, Kl, qf, l32, g);
    scores_add<D>(s, Kh, ql, l32, g);
    scores<D>(dp, Vs, df, l32, g, -dr);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + 32 * mb + 16 * (r >> 3) + 8 * g + (r & 7);
        const float pr = key > klim ? 0.f : exp2_fast(s[mb][r]);
        s[mb][r] = pr * dp[mb][r];
      }
    }
    half8 sh[4], sl[4];
    to_frags_split(s, sh, sl);
    accumulate_tr<D>(acc, Kh, sh, lane);
    accumulate_tr<D>(acc, Kh, sl, lane);
    accumulate_tr<D>(acc, Kl, sh, lane);
  }
  float wv[D / 4];
#pragma unroll
  for (int i = 0; i < D / 4; ++i) wv[i] = 0.f;
  if (row_ok)
    finish_rows<D>(acc, p.scale * dscale_inv(p.dsc, bh), nullptr, p.cs + (size_t)qrow * (D / 2), p.q,
                   head + (size_t)qrow * D, p.bf16, p.dq + head + (size_t)qrow * D, (float)qrow, wv,
                   g);
  store_dalpha<D>(wv, red, p.dalpha_part + (size_t)slot * (D / 2), g);
}

// ------------------------------------------------------------------ dK, dV
// Keys [0, corner) against query rows [key, corner): rotated-frame partial
// sums of dK~ (final scale) and dV, completed by the main dK/dV pass.
template <int D>
__device__ __forceinline__ void corner_dkdv(const MfmaParams& p, int bid) {
  constexpr int DT = D / 16, CB = D / 32, TILE = BN * (D + 8);
  __shared__ __attribute__((aligned(16))) half_t Qh[TILE];
  __shared__ __attribute__((aligned(16))) half_t Ql[TILE];
  __shared__ __attribute__((aligned(16))) half_t Ds[TILE];
  __shared__ __attribute__((aligned(16))) float lses[BN];
  __shared__ __attribute__((aligned(16))) float drs[BN];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, l32 = lane & 31, g = lane >> 5;
  const int BH = p.B * p.H;
  const int bh = bid % BH, t = bid / BH;
  const int k0 = t * BM, wkey0 = k0 + 32 * w, key = wkey0 + l32;
  const int nlo = min(p.N, p.corner);
  if (k0 >= nlo) return;  // whole workgroup
  const size_t head = (size_t)bh * p.N * D, lhead = (size_t)bh * p.corner * D;

  half8 kf[DT], kl[DT], vf[DT];
  load_frag_rows<D>(kf, p.kh + head, key, p.N, g);
  load_frag_rows<D>(kl, p.klo + lhead, key, nlo, g);
  load_frag_rows<D>(vf, p.vh + head, key, p.N, g);
  f32x16 dk[CB], dv[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) { dk[cb] = f32x16{}; dv[cb] = f32x16{}; }
  for (int r0 = k0; r0 < nlo; r0 += BN) {
    __syncthreads();
    stage3<D>(Qh, p.qh + head, Ql, p.qlo + lhead, Ds, p.doh + head, r0, p.N, nlo);
    if (threadIdx.x < BN) {
      const int row = r0 + threadIdx.x;
      const bool ok = row < nlo;   // query rows past the corner are not part of it
      lses[threadIdx.x] = ok ? p.lse[(size_t)bh * p.N + row] * LOG2E : INFINITY;
      drs[threadIdx.x] = ok ? p.drow[(size_t)bh * p.N + row] : 0.f;
    }
    __syncthreads();
    if (wkey0 > r0 + BN - 1) continue;
    f32x16 s[2], dp[2];
    scores<D>(s, Qh, kf, l32, g);
    scores_add<D>(s, Ql, kf, l32, g);
    scores_add<D>(s, Qh, kl, l32, g);
    scores<D>(dp, Ds, vf, l32, g);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int ql = 32 * mb + 16 * h + 8 * g;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = 8 * h + e;
          float pr = exp2_fast(s[mb][r] - lses[ql + e]);
          pr = key > r0 + ql + e ? 0.f : pr;
          s[mb][r] = pr;
          dp[mb][r] = pr * (dp[mb][r] - drs[ql + e]);
        }
      }
    }
    half8 ph[4], pl[4], sh[4], sl[4];
    to_frags_split(s, ph, pl);
    to_frags_split(dp, sh, sl);
    accumulate_tr<D>(dv, Ds, ph, lane);
    accumulate_tr<D>(dv, Ds, pl, lane);
    accumulate_tr<D>(dk, Qh, sh, lane);
    accumulate_tr<D>(dk, Qh, sl, lane);
    accumulate_tr<D>(dk, Ql, sh, lane);
  }
  if (key < nlo) {
    // Q~ carries log2(e)/sqrt(D): dK~ = ln 2 * (dS^T Q~'); the dO scale is undone here
    const float dinv = dscale_inv(p.dsc, bh), kf2 = LN2 * dinv;
    float* dkp = p.dk_part + ((size_t)bh * p.corner + key) * D;
    float* dvp = p.dv_part + ((size_t)bh * p.corner + key) * D;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int c = 32 * cb + 8 * rq + 4 * g;
        *reinterpret_cast<float4*>(dkp + c) =
            make_float4(dk[cb][4 * rq] * kf2, dk[cb][4 * rq + 1] * kf2, dk[cb][4 * rq + 2] * kf2,
                        dk[cb][4 * rq + 3] * kf2);
        *reinterpret_cast<float4*>(dvp + c) =
            make_float4(dv[cb][4 * rq] * dinv, dv[cb][4 * rq + 1] * dinv, dv[cb][4 * rq + 2] * dinv,
                        dv[cb][4 * rq + 3] * dinv);
      }
    }
  }
}

int corner_blocks(const MfmaParams& p) { return p.B * p.H * ((p.corner + BM - 1) / BM); }

// The two backward parts are independent (dQ rows < corner; dK~, dV partials
// of keys < corner), and each has few workgroups of latency-bound work, so
// they share one launch: workgroups [0, ndq) take dQ, the rest dK/dV.
template <int D>
__global__ __launch_bounds__(256) void corner_bwd_kernel(MfmaParams p, int ndq) {
  if ((int)blockIdx.x < ndq) corner_dq<D>(p, blockIdx.x);
  else corner_dkdv<D>(p, blockIdx.x - ndq);
}

}  // namespace

int corner_dq_slots(const MfmaParams& p) { return corner_blocks(p); }

void launch_corner_fwd(const MfmaParams& p, hipStream_t s) {
  const dim3 grid((unsigned)corner_blocks(p)), block(256);
  if (p.D == 64) hipLaunchKernelGGL(corner_fwd_kernel<64>, grid, block, 0, s, p);
  else hipLaunchKernelGGL(corner_fwd_kernel<128>, grid, block, 0, s, p);
}
void launch_corner_bwd(const MfmaParams& p, hipStream_t s) {
  const int n = corner_blocks(p);
  if (n <= 0) return;
  const dim3 grid((unsigned)(2 * n)), block(256);
  if (p.D == 64) hipLaunchKernelGGL(corner_bwd_kernel<64>, grid, block, 0, s, p, n);
  else hipLaunchKernelGGL(corner_bwd_kernel<128>, grid, block, 0, s, p, n);
}

}  // namespace ra
