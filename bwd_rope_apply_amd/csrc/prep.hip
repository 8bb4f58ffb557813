// Frequency table, operand preparation and the final d alpha reduction.
//
// Frequencies: theta_m = b^(-2m/D), theta_hat_m = exp(alpha_m) theta_m
// (LeRoPE, "Central mechanism"; alpha = 0 is standard RoPE).  The angle
// p * theta_hat_m reaches ~6.5e4 rad at N = 32768, where a float product is
// already off by ~4e-3 rad, so the table is evaluated in double and rounded
// once to float.
#include "common.h"

namespace ra {

__global__ void table_kernel(TableParams p) {
  const int half = p.D / 2;
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long)p.N * half) return;
  const int m = (int)(idx % half);
  const int pos = (int)(idx / half);
  const double a = p.alpha ? (double)p.alpha[m] : 0.0;
  // unrotated bands (partial RoPE) have rate 0: angle 0, and a zero alpha
  // gradient through the theta_hat factor
  const double th = m < p.rot ? exp(a) * pow(p.base, -2.0 * (double)m / (double)p.D) : 0.0;
  if (pos == 0) p.theta_hat[m] = th;
  double s, c;
  sincos((double)(pos + p.pos0) * th, &s, &c);
  p.cs[idx] = make_float2((float)c, (float)s);
}

void launch_table(const TableParams& p, hipStream_t s) {
  const long n = (long)p.N * (p.D / 2);
  hipLaunchKernelGGL(table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p);
}

// One thread per 8 consecutive elements of a row.  Q and K are rotated
// (pairs (2m, 2m+1) turned by +p theta_hat_m), V and dO converted; every
// output plane is fp16.  D_i = sum_c dO_ic O_ic is the gamma_2 row scalar of
// "RoPE attention can be trained in almost-linear time" (Methodology 2).
__device__ __forceinline__ void load8(const void* base, size_t idx, int bf16, float* x) {
  load4(base, idx, bf16, x);
  load4(base, idx + 4, bf16, x + 4);
}

__device__ __forceinline__ void store8h(half_t* dst, const float* x) {
  half8 h;
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = (half_t)x[i];
  *reinterpret_cast<half8*>(dst) = h;
}

// x - fp16(x), the low part of a split fp16 operand
__device__ __forceinline__ void store8lo(half_t* dst, const float* x) {
  half8 h;
#pragma unroll
  for (int i = 0; i < 8; ++i) h[i] = (half_t)(x[i] - (float)(half_t)x[i]);
  *reinterpret_cast<half8*>(dst) = h;
}

__global__ void prep_kernel(PrepParams p) {
  const int cpr = p.D / 8;                        // chunks per row (8 or 16)
  const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long total = (long)p.BH * p.N * cpr;
  const bool live = gid < total;
  const long row = live ? gid / cpr : 0;          // bh * N + pos
  const int chunk = (int)(gid % cpr);
  const int pos = (int)(row % p.N);
  const size_t e0 = (size_t)row * p.D + (size_t)chunk * 8;
  float x[8];
  if (live) {
    const float2* cs = p.cs + (size_t)pos * (p.D / 2) + chunk * 4;
    if (p.qh) {
      load8(p.q, e0, p.bf16, x);
#pragma unroll
      for (int i = 0; i < 4; ++i) rot(cs[i].x, cs[i].y, x[2 * i], x[2 * i + 1]);
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] *= p.qscale;
      store8h(p.qh + e0, x);
      if (p.qlo && pos < p.rlo)
        store8lo(p.qlo + ((size_t)(row / p.N) * p.rlo + pos) * p.D + chunk * 8, x);
    }
    if (p.kh) {
      load8(p.k, e0, p.bf16, x);
#pragma unroll
      for (int i = 0; i < 4; ++i) rot(cs[i].x, cs[i].y, x[2 * i], x[2 * i + 1]);
      store8h(p.kh + e0, x);
      if (p.klo && pos < p.rlo)
        store8lo(p.klo + ((size_t)(row / p.N) * p.rlo + pos) * p.D + chunk * 8, x);
    }
    if (p.vh) {
      load8(p.v, e0, p.bf16, x);
      store8h(p.vh + e0, x);
    }
  }
  if (p.doh || p.drow) {
    float acc = 0.f;
    if (live) {
      load8(p.dO, e0, p.bf16, x);
      if (p.doh) store8h(p.doh + e0, x);
      if (p.drow) {
        const float4* o4 = reinterpret_cast<const float4*>(p.o + e0);
        float4 a = o4[0], b = o4[1];
        acc = x[0] * a.x + x[1] * a.y + x[2] * a.z + x[3] * a.w +
              x[4] * b.x + x[5] * b.y + x[6] * b.z + x[7] * b.w;
      }
    }
    if (p.drow) {
      // the cpr lanes of a row are consecutive and aligned inside the wave
      for (int off = 1; off < cpr; off <<= 1) acc += __shfl_xor(acc, off, 64);
      if (live && chunk == 0) {
        p.drow[row] = acc;
        if (p.rs) {
          const int G = rs_groups(p.N);
          float* rsh = p.rs + (size_t)(row / p.N) * G * 64;
          rsh[(pos >> 5) * 64 + (pos & 31)] = p.lse[row] * LOG2E;
          rsh[(pos >> 5) * 64 + 32 + (pos & 31)] = acc;
          if (pos == p.N - 1) {  // pad rows up to the end of the spare group
            for (int r = p.N; r < 32 * G; ++r) {
              rsh[(r >> 5) * 64 + (r & 31)] = INFINITY;
              rsh[(r >> 5) * 64 + 32 + (r & 31)] = 0.f;
            }
          }
        }
      }
    }
  }
}

void launch_prep(const PrepParams& p, hipStream_t s) {
  const long total = (long)p.BH * p.N * (p.D / 8);
  hipLaunchKernelGGL(prep_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, p);
}

// Block visibility rows from a CSR list, one wave per (bh, query block):
// lanes take the list's entries in turn and OR their bits into an LDS row;
// the own block always; entries out of range are skipped and duplicates
// merge; under the causal mask no block after the own one.  Offsets are
// clamped to [0, nnz], so no read leaves the list.
__global__ __launch_bounds__(64) void block_mask_kernel(BlockMaskParams p) {
  __shared__ uint32_t w[MAX_BLOCKS / 32];
  const int r = blockIdx.x, lane = threadIdx.x;
  const int qb = r % p.nb;
  if (lane < MAX_BLOCKS / 32) w[lane] = lane == (qb >> 5) ? 1u << (qb & 31) : 0u;
  __syncthreads();
  const int e0 = min(max(p.ptr[r], 0), p.nnz);
  const int e1 = min(max(p.ptr[r + 1], e0), p.nnz);
  for (int e = e0 + lane; e < e1; e += 64) {
    const int kb = p.idx[e];
    if (kb >= 0 && kb < p.nb && (!p.causal || kb <= qb)) atomicOr(&w[kb >> 5], 1u << (kb & 31));
  }
  __syncthreads();
  if (lane < p.W) p.mask[(size_t)r * p.W + lane] = w[lane];
}

void launch_block_mask(const BlockMaskParams& p, hipStream_t s) {
  if (p.rows > 0) hipLaunchKernelGGL(block_mask_kernel, dim3((unsigned)p.rows), dim3(64), 0, s, p);
}

// d alpha_m = theta_hat_m * sum over slots of the position-weighted wedge
// partials, summed in double in a fixed order (deterministic).
__global__ void dalpha_kernel(DalphaParams p) {
  const int m = blockIdx.x;
  const int half = p.D / 2;
  __shared__ double red[256];
  double acc = 0.0;
  for (int s = threadIdx.x; s < p.slots; s += 256) acc += (double)p.part[(size_t)s * half + m];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) p.dalpha[m] = (float)(p.theta_hat[m] * red[0]);
}

void launch_dalpha_reduce(const DalphaParams& p, hipStream_t s) {
  hipLaunchKernelGGL(dalpha_kernel, dim3(p.D / 2), dim3(256), 0, s, p);
}

}  // namespace ra
