// The float32 path on the matrix cores: every product of the forward and the
// backward on v_mfma_f32_32x32x2f32 (fp32 operands, fp32 accumulation).  It
// serves calls with fp32 inputs and dense (causal or full) attention; block
// lists take the vector-ALU path in simt.hip.
//
// Forward: S = Q~ K~^T * scale with the causal mask j <= i, the softmax s(x),
// O = P V and the row log-sum-exp ("RoPE attention can be trained in
// almost-linear time", Problem definition).  Backward: beta = dO V^T,
// dS = P o (beta - D_i) = (diag(s) - s s^T) beta (same page, Methodology 1
// and 2), dQ~ = dS K~ * scale, dK~ = dS^T Q~ * scale, dV = P^T dO, then the
// transpose rotation; d alpha from the un-rotated gradients ("LeRoPE",
// Theoretical analysis).
//
// Fragment convention of v_mfma_f32_32x32x2f32 (lane l, l32 = l % 32,
// g = l / 32): A[m][k]: lane (m, g) holds k = g; B[k][n]: lane (n, g) holds
// k = g; C[m][n]: lane (n, g) holds row 8(r/4) + 4g + r%4 in register r.
// Products are accumulated over k steps kk of two (element 2 kk + g).  The
// rows of a score product's A operand are read in the order pi(m) =
// 8(m/8) + 2(m%4) + (m/4)%2, so register r of lane (n, g) holds the score
// of row 2r + g: exactly the B operand element of k step r of the next
// product, with no data movement between lanes.  Tiles are fp32 in LDS,
// [32][D + 4], staged (and rotated) from the inputs; each workgroup is two
// waves of 32 rows (or keys), the same 64-row blocks as the vector path, so
// the d alpha partial slots are the same.
#include "tile.h"

namespace ra {

namespace {

constexpr int FW = 64;   // rows (keys) per workgroup: two waves x 32
constexpr int FT = 32;   // rows per streamed tile

__device__ __forceinline__ f32x16 mfma32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Row order of a score product's A operand (see above).
__device__ __forceinline__ int pi32(int m) { return (m & ~7) | ((m & 3) << 1) | ((m >> 2) & 1); }

// Rows [r0, r0 + FT) of one head into an LDS tile [FT][LD] as fp32,
// rotated when cs != null; rows outside [0, N) are zero.  128 threads.
template <int D, int LD>
__device__ __forceinline__ void stage_f32(float* dst, const void* src, size_t head_off, int r0,
                                          int N, int bf16, const float2* cs) {
  constexpr int CH = D / 4;
  for (int t = threadIdx.x; t < FT * CH; t += 128) {
    const int r = t / CH, c = (t % CH) * 4;
    const int row = r0 + r;
    float x[4] = {0.f, 0.f, 0.f, 0.f};
    if (row < N) {
      load4(src, head_off + (size_t)row * D + c, bf16, x);
      if (cs) {
        const float2* t2 = cs + (size_t)row * (D / 2) + c / 2;
        rot(t2[0].x, t2[0].y, x[0], x[1]);
        rot(t2[1].x, t2[1].y, x[2], x[3]);
      }
    }
    *reinterpret_cast<float4*>(dst + r * LD + c) = make_float4(x[0], x[1], x[2], x[3]);
  }
}

// This lane's B-operand elements of one row: f[kk] = x~[2 kk + g] (rotated
// when cs != null), zeros for a row at or past N.
template <int D>
__device__ __forceinline__ void row_frags(float* f, const void* src, size_t head_off, int row,
                                          int N, int bf16, const float2* cs, int g) {
#pragma unroll
  for (int c = 0; c < D; c += 4) {
    float x[4] = {0.f, 0.f, 0.f, 0.f};
    if (row < N) {
      load4(src, head_off + (size_t)row * D + c, bf16, x);
      if (cs) {
        const float2* t2 = cs + (size_t)row * (D / 2) + c / 2;
        rot(t2[0].x, t2[0].y, x[0], x[1]);
        rot(t2[1].x, t2[1].y, x[2], x[3]);
      }
    }
    f[c / 2] = x[g];
    f[c / 2 + 1] = x[2 + g];
  }
}

// S^T-style product over D: acc[r] += sum_d A[pi(l32)][d] * f[d/2] with A a
// tile in LDS (row stride LD) and f this lane's B elements.
template <int D, int LD>
__device__ __forceinline__ f32x16 score32(const float* tile, const float* f, int l32, int g) {
  f32x16 acc = {};
  const float* arow = tile + pi32(l32) * LD + g;
#pragma unroll
  for (int kk = 0; kk < D / 2; ++kk) acc = mfma32(arow[2 * kk], f[kk], acc);
  return acc;
}

// acc[cb] += X^T[32 cb + l32][rows] * b[rows], rows = 2 kk + g of a tile X in
// LDS and b the 16 B elements (k step kk in b[kk]).
template <int D, int LD>
__device__ __forceinline__ void accumulate_t32(f32x16* acc, const float* tile, const f32x16& b,
                                               int l32, int g) {
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb) {
    const float* col = tile + g * LD + 32 * cb + l32;
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) acc[cb] = mfma32(col[2 * kk * LD], b[kk], acc[cb]);
  }
}

// The wedge partials of a two-wave workgroup (finish_rows' layout) summed
// into one [D/2] slot.
template <int D>
__device__ __forceinline__ void store_dalpha2(float* w, float* red, float* slot, int g) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < D / 4; ++i) {
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
  for (int m = threadIdx.x; m < D / 2; m += 128) slot[m] = red[m] + red[D / 2 + m];
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(128) void f32_fwd_kernel(SimtParams p) {
  constexpr int LD = D + 4, CB = D / 32;
  __shared__ __attribute__((aligned(16))) float ks[FT * LD];
  __shared__ __attribute__((aligned(16))) float vs[FT * LD];
  const int bh = blockIdx.y;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, l32 = lane & 31, g = lane >> 5;
  const int r0 = blockIdx.x * FW, q = r0 + 32 * w + l32;   // this lane's query
  const size_t head = (size_t)bh * p.N * D;
  float qf[D / 2];
  row_frags<D>(qf, p.q, head, q, p.N, p.bf16, p.cs, g);
  f32x16 o[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) o[cb] = f32x16{};
  float m = -INFINITY, l = 0.f;
  const int kend = CAUSAL ? min(p.N, r0 + FW) : p.N;
  for (int k0 = 0; k0 < kend; k0 += FT) {
    __syncthreads();
    stage_f32<D, LD>(ks, p.k, head, k0, p.N, p.bf16, p.cs);
    stage_f32<D, LD>(vs, p.v, head, k0, p.N, p.bf16, nullptr);
    __syncthreads();
    f32x16 s = score32<D, LD>(ks, qf, l32, g);   // register r: key k0 + 2r + g
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = k0 + 2 * r + g;
      const bool ok = key < p.N && (!CAUSAL || key <= q);
      const float x = ok ? s[r] * p.scale : -INFINITY;
      s[r] = x;
      mx = fmaxf(mx, x);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mn = fmaxf(m, mx);
    const float a = m == -INFINITY ? 0.f : expf(m - mn);
    l *= a;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) o[cb] *= a;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float pr = s[r] == -INFINITY ? 0.f : expf(s[r] - mn);
      s[r] = pr;
      l += pr;
    }
    m = mn;
    accumulate_t32<D, LD>(o, vs, s, l32, g);   // O^T += V^T P^T
  }
  l += __shfl_xor(l, 32, 64);
  if (q < p.N) {
    const float inv = 1.f / l;
    float* orow = p.out_o + head + (size_t)q * D;
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
    if (g == 0) p.out_lse[(size_t)bh * p.N + q] = m + logf(l);
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(128) void f32_dq_kernel(SimtParams p) {
  constexpr int LD = D + 4, CB = D / 32;
  __shared__ __attribute__((aligned(16))) float ks[FT * LD];
  __shared__ __attribute__((aligned(16))) float vs[FT * LD];
  __shared__ float red[2 * (D / 2)];
  const int bh = blockIdx.y;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, l32 = lane & 31, g = lane >> 5;
  const int r0 = blockIdx.x * FW, q = r0 + 32 * w + l32;
  const size_t head = (size_t)bh * p.N * D;
  float qf[D / 2], df[D / 2];
  row_frags<D>(qf, p.q, head, q, p.N, p.bf16, p.cs, g);
  row_frags<D>(df, p.dO, head, q, p.N, p.bf16, nullptr, g);
  const bool q_ok = q < p.N;
  const float lse = q_ok ? p.lse[(size_t)bh * p.N + q] : 0.f;
  const float drow = q_ok ? p.drow[(size_t)bh * p.N + q] : 0.f;
  f32x16 acc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) acc[cb] = f32x16{};
  const int kend = CAUSAL ? min(p.N, r0 + FW) : p.N;
  for (int k0 = 0; k0 < kend; k0 += FT) {
    __syncthreads();
    stage_f32<D, LD>(ks, p.k, head, k0, p.N, p.bf16, p.cs);
    stage_f32<D, LD>(vs, p.v, head, k0, p.N, p.bf16, nullptr);
    __syncthreads();
    f32x16 s = score32<D, LD>(ks, qf, l32, g);    // S^T: register r, key k0 + 2r + g
    const f32x16 dp = score32<D, LD>(vs, df, l32, g);   // (dO V^T)^T
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = k0 + 2 * r + g;
      const bool ok = q_ok && key < p.N && (!CAUSAL || key <= q);
      const float pr = ok ? expf(s[r] * p.scale - lse) : 0.f;
      s[r] = pr * (dp[r] - drow);   // dS^T
    }
    accumulate_t32<D, LD>(acc, ks, s, l32, g);   // dQ~^T += K~^T dS^T
  }
  float wv[D / 4];
#pragma unroll
  for (int i = 0; i < D / 4; ++i) wv[i] = 0.f;
  if (q_ok)
    finish_rows<D>(acc, p.scale, nullptr, p.cs + (size_t)q * (D / 2), p.q, head + (size_t)q * D,
                   p.bf16, p.dq + head + (size_t)q * D, (float)q, wv, g);
  const int slot = p.slot0 + bh * gridDim.x + blockIdx.x;
  store_dalpha2<D>(wv, red, p.dalpha_part + (size_t)slot * (D / 2), g);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(128) void f32_dkdv_kernel(SimtParams p) {
  constexpr int LD = D + 4, CB = D / 32;
  __shared__ __attribute__((aligned(16))) float qs[FT * LD];
  __shared__ __attribute__((aligned(16))) float dos[FT * LD];
  __shared__ __attribute__((aligned(16))) float vst[FW * LD];   // this workgroup's V rows
  __shared__ float lses[FT], drs[FT];
  __shared__ float red[2 * (D / 2)];
  const int bh = blockIdx.y;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, l32 = lane & 31, g = lane >> 5;
  const int k0 = blockIdx.x * FW, key = k0 + 32 * w + l32;   // this lane's key
  const size_t head = (size_t)bh * p.N * D;
  const bool key_ok = key < p.N;
  float kf[D / 2];
  row_frags<D>(kf, p.k, head, key, p.N, p.bf16, p.cs, g);
  stage_f32<D, LD>(vst, p.v, head, k0, p.N, p.bf16, nullptr);
  stage_f32<D, LD>(vst + FT * LD, p.v, head, k0 + FT, p.N, p.bf16, nullptr);
  const float* vrow = vst + (32 * w + l32) * LD + g;   // B elements of dP: V[key][2 kk + g]
  f32x16 dk[CB], dv[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) { dk[cb] = f32x16{}; dv[cb] = f32x16{}; }
  const int qstart = CAUSAL ? k0 : 0;
  for (int r0 = qstart; r0 < p.N; r0 += FT) {
    __syncthreads();
    stage_f32<D, LD>(qs, p.q, head, r0, p.N, p.bf16, p.cs);
    stage_f32<D, LD>(dos, p.dO, head, r0, p.N, p.bf16, nullptr);
    if (threadIdx.x < FT) {
      const int row = r0 + threadIdx.x;
      const bool ok = row < p.N;
      lses[threadIdx.x] = ok ? p.lse[(size_t)bh * p.N + row] : 0.f;
      drs[threadIdx.x] = ok ? p.drow[(size_t)bh * p.N + row] : 0.f;
    }
    __syncthreads();
    f32x16 s = score32<D, LD>(qs, kf, l32, g);   // S: register r, query r0 + 2r + g
    f32x16 dp = {};
    {
      const float* arow = dos + pi32(l32) * LD + g;
#pragma unroll
      for (int kk = 0; kk < D / 2; ++kk) dp = mfma32(arow[2 * kk], vrow[2 * kk], dp);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i = 2 * r + g, row = r0 + i;
      const bool ok = key_ok && row < p.N && (!CAUSAL || row >= key);
      const float pr = ok ? expf(s[r] * p.scale - lses[i]) : 0.f;
      s[r] = pr;
      dp[r] = pr * (dp[r] - drs[i]);   // dS
    }
    accumulate_t32<D, LD>(dv, dos, s, l32, g);   // dV^T += dO^T P
    accumulate_t32<D, LD>(dk, qs, dp, l32, g);   // dK~^T += Q~^T dS
  }
  float wv[D / 4];
#pragma unroll
  for (int i = 0; i < D / 4; ++i) wv[i] = 0.f;
  if (key_ok) {
    finish_rows<D>(dk, p.scale, nullptr, p.cs + (size_t)key * (D / 2), p.k, head + (size_t)key * D,
                   p.bf16, p.dk + head + (size_t)key * D, (float)key, wv, g);
    float* dvrow = p.dv + head + (size_t)key * D;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int c = 32 * cb + 8 * rq + 4 * g;
        *reinterpret_cast<float4*>(dvrow + c) =
            make_float4(dv[cb][4 * rq], dv[cb][4 * rq + 1], dv[cb][4 * rq + 2], dv[cb][4 * rq + 3]);
      }
    }
  }
  const int slot = p.slot0 + bh * gridDim.x + blockIdx.x;
  store_dalpha2<D>(wv, red, p.dalpha_part + (size_t)slot * (D / 2), g);
}

dim3 f32_grid(const SimtParams& p) {
  return dim3((unsigned)((p.N + FW - 1) / FW), (unsigned)p.BH);
}

#define RA_F32_LAUNCH(KERNEL)                                                                  \
  do {                                                                                         \
    if (p.D == 64) {                                                                           \
      if (p.causal) hipLaunchKernelGGL((KERNEL<64, true>), f32_grid(p), dim3(128), 0, s, p);   \
      else hipLaunchKernelGGL((KERNEL<64, false>), f32_grid(p), dim3(128), 0, s, p);           \
    } else {                                                                                   \
      if (p.causal) hipLaunchKernelGGL((KERNEL<128, true>), f32_grid(p), dim3(128), 0, s, p);  \
      else hipLaunchKernelGGL((KERNEL<128, false>), f32_grid(p), dim3(128), 0, s, p);          \
    }                                                                                          \
  } while (0)

}  // namespace

void launch_f32_fwd(const SimtParams& p, hipStream_t s) { RA_F32_LAUNCH(f32_fwd_kernel); }
void launch_f32_dq(const SimtParams& p, hipStream_t s) { RA_F32_LAUNCH(f32_dq_kernel); }
void launch_f32_dkdv(const SimtParams& p, hipStream_t s) { RA_F32_LAUNCH(f32_dkdv_kernel); }

}  // namespace ra
