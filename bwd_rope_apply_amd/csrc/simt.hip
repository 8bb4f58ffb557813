// Exact fp32 path on the vector ALUs: plain fused multiply-adds, one row per
// group of four lanes (each lane owns D/4 consecutive columns, so every
// rotation pair stays inside one lane).  It serves fp32 calls with block
// lists; dense fp32 calls take the matrix-core path (f32mfma.hip).
//
// Forward: S = Q~ K~^T / sqrt(D) with the causal mask j <= i, the
// normalised softmax s(x), O = P V and the row log-sum-exp ("RoPE attention
// can be trained in almost-linear time", Problem definition).  Backward:
// beta = dO V^T, dS = P o (beta - D_i) = (diag(s) - s s^T) beta (same page,
// Methodology 1 and 2, gamma_1 and gamma_2); dQ~ = dS K~ / sqrt(D),
// dK~ = dS^T Q~ / sqrt(D), dV = P^T dO, then the transpose rotation.
#include "common.h"

namespace ra {

namespace {

constexpr int ROWS_PER_WG = 64;   // 256 lanes, 4 per row
constexpr int TK = 32;            // staged rows per LDS tile

template <int D>
struct Lane {
  static constexpr int DL = D / 4;   // columns owned by one lane
};

__device__ __forceinline__ float group_sum(float x) {
  x += __shfl_xor(x, 1, 64);
  x += __shfl_xor(x, 2, 64);
  return x;
}

// Load DL consecutive elements [c0, c0+DL) of an input row as floats.
template <int DL>
__device__ __forceinline__ void load_row(const void* base, size_t off, int bf16, float* x) {
#pragma unroll
  for (int c = 0; c < DL; c += 4) load4(base, off + c, bf16, x + c);
}

template <int DL>
__device__ __forceinline__ void rotate_row(const float2* cs_row, int c0, float* x) {
#pragma unroll
  for (int c = 0; c < DL; c += 2) {
    float2 t = cs_row[(c0 + c) / 2];
    rot(t.x, t.y, x[c], x[c + 1]);
  }
}

// Cooperative staging of TK rows [r0, r0+TK) of one head into LDS as fp32,
// rotated when cs != null.  Rows outside [0, N) are zero.
template <int D>
__device__ __forceinline__ void stage(float (*dst)[D], const void* src, size_t head_off, int r0,
                                      int N, int bf16, const float2* cs) {
  constexpr int CH = D / 4;  // float4 chunks per row
  for (int t = threadIdx.x; t < TK * CH; t += 256) {
    const int r = t / CH, c = (t % CH) * 4;
    const int row = r0 + r;
    float x[4] = {0.f, 0.f, 0.f, 0.f};
    if (row >= 0 && row < N) {
      load4(src, head_off + (size_t)row * D + c, bf16, x);
      if (cs) {
        const float2* t2 = cs + (size_t)row * (D / 2) + c / 2;
        rot(t2[0].x, t2[0].y, x[0], x[1]);
        rot(t2[1].x, t2[1].y, x[2], x[3]);
      }
    }
    *reinterpret_cast<float4*>(&dst[r][c]) = make_float4(x[0], x[1], x[2], x[3]);
  }
}

// Sum the position-weighted wedge partials w[D/8 per lane] over the 64 rows
// of the workgroup and write one [D/2] slot.
template <int D>
__device__ __forceinline__ void store_dalpha_slot(float* w, float* slot) {
  constexpr int NP = D / 8;   // pairs per lane
  __shared__ float red[4][D / 2];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, j = threadIdx.x & 3;
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    float x = w[i];
    x += __shfl_xor(x, 4, 64);
    x += __shfl_xor(x, 8, 64);
    x += __shfl_xor(x, 16, 64);
    x += __shfl_xor(x, 32, 64);
    if (lane < 4) red[wave][j * NP + i] = x;
  }
  __syncthreads();
  for (int m = threadIdx.x; m < D / 2; m += 256)
    slot[m] = (red[0][m] + red[1][m]) + (red[2][m] + red[3][m]);
}

template <int D>
__global__ __launch_bounds__(256) void simt_fwd_kernel(SimtParams p) {
  constexpr int DL = Lane<D>::DL;
  __shared__ float ks[TK][D];
  __shared__ float vs[TK][D];
  const int bh = blockIdx.y;
  const int g = threadIdx.x >> 2, j = threadIdx.x & 3;
  const int i = blockIdx.x * ROWS_PER_WG + g;
  const int c0 = j * DL;
  const size_t head = (size_t)bh * p.N * D;
  const bool row_ok = i < p.rows && i < p.N;
  float qv[DL], acc[DL];
#pragma unroll
  for (int c = 0; c < DL; ++c) { qv[c] = 0.f; acc[c] = 0.f; }
  if (row_ok) {
    load_row<DL>(p.q, head + (size_t)i * D + c0, p.bf16, qv);
    rotate_row<DL>(p.cs + (size_t)i * (D / 2), c0, qv);
  }
  float m = -INFINITY, l = 0.f;
  const int last_row = min(p.rows, (int)(blockIdx.x + 1) * ROWS_PER_WG) - 1;
  const int kend = p.causal ? min(p.N, last_row + 1) : p.N;
  for (int kt = 0; kt < kend; kt += TK) {
    __syncthreads();
    stage<D>(ks, p.k, head, kt, p.N, p.bf16, p.cs);
    stage<D>(vs, p.v, head, kt, p.N, p.bf16, nullptr);
    __syncthreads();
    for (int jj = 0; jj < TK; ++jj) {
      const int key = kt + jj;
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < DL; ++c) s += qv[c] * ks[jj][c0 + c];
      s = group_sum(s) * p.scale;
      const bool ok = row_ok && key < kend && (!p.causal || key <= i) &&
                      block_visible(p.bmask, p.nb, p.W, bh, i, key);
      if (ok) {
        const float mn = fmaxf(m, s);
        const float a = expf(m - mn);
        const float pr = expf(s - mn);
        l = l * a + pr;
#pragma unroll
        for (int c = 0; c < DL; ++c) acc[c] = acc[c] * a + pr * vs[jj][c0 + c];
        m = mn;
      }
    }
  }
  if (row_ok) {
    const float inv = 1.f / l;
    float* o = p.out_o + head + (size_t)i * D + c0;
#pragma unroll
    for (int c = 0; c < DL; c += 4)
      *reinterpret_cast<float4*>(o + c) =
          make_float4(acc[c] * inv, acc[c + 1] * inv, acc[c + 2] * inv, acc[c + 3] * inv);
    if (j == 0) p.out_lse[(size_t)bh * p.N + i] = m + logf(l);
  }
}

template <int D>
__global__ __launch_bounds__(256) void simt_dq_kernel(SimtParams p) {
  constexpr int DL = Lane<D>::DL;
  __shared__ float ks[TK][D];
  __shared__ float vs[TK][D];
  const int bh = blockIdx.y;
  const int g = threadIdx.x >> 2, j = threadIdx.x & 3;
  const int i = blockIdx.x * ROWS_PER_WG + g;
  const int c0 = j * DL;
  const size_t head = (size_t)bh * p.N * D;
  const bool row_ok = i < p.rows && i < p.N;
  float qv[DL], dov[DL], acc[DL];
  float lse = 0.f, drow = 0.f;
#pragma unroll
  for (int c = 0; c < DL; ++c) { qv[c] = 0.f; dov[c] = 0.f; acc[c] = 0.f; }
  if (row_ok) {
    load_row<DL>(p.q, head + (size_t)i * D + c0, p.bf16, qv);
    rotate_row<DL>(p.cs + (size_t)i * (D / 2), c0, qv);
    load_row<DL>(p.dO, head + (size_t)i * D + c0, p.bf16, dov);
    lse = p.lse[(size_t)bh * p.N + i];
    drow = p.drow[(size_t)bh * p.N + i];
  }
  const int last_row = min(p.rows, (int)(blockIdx.x + 1) * ROWS_PER_WG) - 1;
  const int kend = p.causal ? min(p.N, last_row + 1) : p.N;
  for (int kt = 0; kt < kend; kt += TK) {
    __syncthreads();
    stage<D>(ks, p.k, head, kt, p.N, p.bf16, p.cs);
    stage<D>(vs, p.v, head, kt, p.N, p.bf16, nullptr);
    __syncthreads();
    for (int jj = 0; jj < TK; ++jj) {
      const int key = kt + jj;
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int c = 0; c < DL; ++c) {
        s += qv[c] * ks[jj][c0 + c];
        dp += dov[c] * vs[jj][c0 + c];
      }
      s = group_sum(s) * p.scale;
      dp = group_sum(dp);
      const bool ok = row_ok && key < kend && (!p.causal || key <= i) &&
                      block_visible(p.bmask, p.nb, p.W, bh, i, key);
      const float pr = ok ? expf(s - lse) : 0.f;
      const float ds = pr * (dp - drow);
#pragma unroll
      for (int c = 0; c < DL; ++c) acc[c] += ds * ks[jj][c0 + c];
    }
  }
  float w[DL / 2];
#pragma unroll
  for (int c = 0; c < DL / 2; ++c) w[c] = 0.f;
  if (row_ok) {
    const float2* cs = p.cs + (size_t)i * (D / 2);
    float qo[DL];
    load_row<DL>(p.q, head + (size_t)i * D + c0, p.bf16, qo);
#pragma unroll
    for (int c = 0; c < DL; c += 2) {
      float g0 = acc[c] * p.scale, g1 = acc[c + 1] * p.scale;
      float2 t = cs[(c0 + c) / 2];
      unrot(t.x, t.y, g0, g1);
      acc[c] = g0; acc[c + 1] = g1;
      w[c / 2] = (float)i * (qo[c] * g1 - qo[c + 1] * g0);
    }
    float* dq = p.dq + head + (size_t)i * D + c0;
#pragma unroll
    for (int c = 0; c < DL; c += 4)
      *reinterpret_cast<float4*>(dq + c) = make_float4(acc[c], acc[c + 1], acc[c + 2], acc[c + 3]);
  }
  const int slot = p.slot0 + bh * gridDim.x + blockIdx.x;
  store_dalpha_slot<D>(w, p.dalpha_part + (size_t)slot * (D / 2));
}

template <int D>
__global__ __launch_bounds__(256) void simt_dkdv_kernel(SimtParams p) {
  constexpr int DL = Lane<D>::DL;
  __shared__ float qs[TK][D];
  __shared__ float dos[TK][D];
  __shared__ float lses[TK], drs[TK];
  const int bh = blockIdx.y;
  const int g = threadIdx.x >> 2, j = threadIdx.x & 3;
  const int key = blockIdx.x * ROWS_PER_WG + g;
  const int c0 = j * DL;
  const size_t head = (size_t)bh * p.N * D;
  const bool key_ok = key < p.rows && key < p.N;
  float kv[DL], vv[DL], dk[DL], dv[DL];
#pragma unroll
  for (int c = 0; c < DL; ++c) { kv[c] = 0.f; vv[c] = 0.f; dk[c] = 0.f; dv[c] = 0.f; }
  if (key_ok) {
    load_row<DL>(p.k, head + (size_t)key * D + c0, p.bf16, kv);
    rotate_row<DL>(p.cs + (size_t)key * (D / 2), c0, kv);
    load_row<DL>(p.v, head + (size_t)key * D + c0, p.bf16, vv);
  }
  const int first_key = blockIdx.x * ROWS_PER_WG;
  const int q0 = p.causal ? first_key : 0;
  for (int it = q0; it < p.qend; it += TK) {
    __syncthreads();
    stage<D>(qs, p.q, head, it, p.N, p.bf16, p.cs);
    stage<D>(dos, p.dO, head, it, p.N, p.bf16, nullptr);
    if (threadIdx.x < TK) {
      const int row = it + threadIdx.x;
      const bool ok = row < p.N;
      lses[threadIdx.x] = ok ? p.lse[(size_t)bh * p.N + row] : 0.f;
      drs[threadIdx.x] = ok ? p.drow[(size_t)bh * p.N + row] : 0.f;
    }
    __syncthreads();
    for (int ii = 0; ii < TK; ++ii) {
      const int row = it + ii;
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int c = 0; c < DL; ++c) {
        s += qs[ii][c0 + c] * kv[c];
        dp += dos[ii][c0 + c] * vv[c];
      }
      s = group_sum(s) * p.scale;
      dp = group_sum(dp);
      const bool ok = key_ok && row < p.qend && (!p.causal || row >= key) &&
                      block_visible(p.bmask, p.nb, p.W, bh, row, key);
      const float pr = ok ? expf(s - lses[ii]) : 0.f;
      const float ds = pr * (dp - drs[ii]);
#pragma unroll
      for (int c = 0; c < DL; ++c) {
        dv[c] += pr * dos[ii][c0 + c];
        dk[c] += ds * qs[ii][c0 + c];
      }
    }
  }
  if (!p.final_) {
    if (key_ok) {
      float* dkp = p.dk_part + ((size_t)bh * p.rows + key) * D + c0;
      float* dvp = p.dv_part + ((size_t)bh * p.rows + key) * D + c0;
#pragma unroll
      for (int c = 0; c < DL; c += 4) {
        *reinterpret_cast<float4*>(dkp + c) = make_float4(dk[c] * p.scale, dk[c + 1] * p.scale,
                                                          dk[c + 2] * p.scale, dk[c + 3] * p.scale);
        *reinterpret_cast<float4*>(dvp + c) = make_float4(dv[c], dv[c + 1], dv[c + 2], dv[c + 3]);
      }
    }
    return;
  }
  float w[DL / 2];
#pragma unroll
  for (int c = 0; c < DL / 2; ++c) w[c] = 0.f;
  if (key_ok) {
    const float2* cs = p.cs + (size_t)key * (D / 2);
    float ko[DL];
    load_row<DL>(p.k, head + (size_t)key * D + c0, p.bf16, ko);
#pragma unroll
    for (int c = 0; c < DL; c += 2) {
      float g0 = dk[c] * p.scale, g1 = dk[c + 1] * p.scale;
      float2 t = cs[(c0 + c) / 2];
      unrot(t.x, t.y, g0, g1);
      dk[c] = g0; dk[c + 1] = g1;
      w[c / 2] = (float)key * (ko[c] * g1 - ko[c + 1] * g0);
    }
    float* dkp = p.dk + head + (size_t)key * D + c0;
    float* dvp = p.dv + head + (size_t)key * D + c0;
#pragma unroll
    for (int c = 0; c < DL; c += 4) {
      *reinterpret_cast<float4*>(dkp + c) = make_float4(dk[c], dk[c + 1], dk[c + 2], dk[c + 3]);
      *reinterpret_cast<float4*>(dvp + c) = make_float4(dv[c], dv[c + 1], dv[c + 2], dv[c + 3]);
    }
  }
  const int slot = p.slot0 + bh * gridDim.x + blockIdx.x;
  store_dalpha_slot<D>(w, p.dalpha_part + (size_t)slot * (D / 2));
}

dim3 simt_grid(const SimtParams& p) {
  return dim3((unsigned)((p.rows + ROWS_PER_WG - 1) / ROWS_PER_WG), (unsigned)p.BH);
}

}  // namespace

int simt_slots(int BH, int rows) { return BH * ((rows + ROWS_PER_WG - 1) / ROWS_PER_WG); }

void launch_simt_fwd(const SimtParams& p, hipStream_t s) {
  if (p.D == 64) hipLaunchKernelGGL(simt_fwd_kernel<64>, simt_grid(p), dim3(256), 0, s, p);
  else hipLaunchKernelGGL(simt_fwd_kernel<128>, simt_grid(p), dim3(256), 0, s, p);
}
void launch_simt_dq(const SimtParams& p, hipStream_t s) {
  if (p.D == 64) hipLaunchKernelGGL(simt_dq_kernel<64>, simt_grid(p), dim3(256), 0, s, p);
  else hipLaunchKernelGGL(simt_dq_kernel<128>, simt_grid(p), dim3(256), 0, s, p);
}
void launch_simt_dkdv(const SimtParams& p, hipStream_t s) {
  if (p.D == 64) hipLaunchKernelGGL(simt_dkdv_kernel<64>, simt_grid(p), dim3(256), 0, s, p);
  else hipLaunchKernelGGL(simt_dkdv_kernel<128>, simt_grid(p), dim3(256), 0, s, p);
}

}  // namespace ra
