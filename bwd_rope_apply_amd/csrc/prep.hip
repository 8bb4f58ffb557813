// Frequency table, operand preparation and the final d alpha reduction.
//
// Frequencies: theta_m = b^(-2m/D), theta_hat_m = exp(alpha_m) theta_m
// (LeRoPE, "Central mechanism"; alpha = 0 is standard RoPE).  The angle
// p * theta_hat_m reaches ~6.5e4 rad at N = 32768, where a float product is
// already off by ~4e-3 rad, so the table is evaluated in double and rounded
// once to float.
#include "common.h"

namespace ra {

// Each thread takes one band m over a run of TABLE_RUN consecutive
// positions: theta_hat_m and the run's first angle are evaluated directly,
// and each later position turns the previous (cos, sin) by theta_hat_m
// (angle addition, in double: the error grows by a few units of 2^-53 a
// step, far below the float rounding).  Consecutive threads take
// consecutive bands, so each position's row is stored contiguously.
constexpr int TABLE_RUN = 8;

__global__ void table_kernel(TableParams p) {
  const int half = p.D / 2;
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const int runs = (p.N + TABLE_RUN - 1) / TABLE_RUN;
  if (idx >= (long)runs * half) return;
  const int m = (int)(idx % half);
  const int pos0 = (int)(idx / half) * TABLE_RUN;
  const double a = p.alpha ? (double)p.alpha[m] : 0.0;
  // unrotated bands (partial RoPE) have rate 0: angle 0, and a zero alpha
  // gradient through the theta_hat factor
  const double th = m < p.rot ? exp(a) * pow(p.base, -2.0 * (double)m / (double)p.D) : 0.0;
  if (pos0 == 0) p.theta_hat[m] = th;
  if (idx == 0 && p.flags) *p.flags = 0u;
  double s, c, sd, cd;
  sincos((double)(pos0 + p.pos0) * th, &s, &c);
  sincos(th, &sd, &cd);
  const int n = min(TABLE_RUN, p.N - pos0);
  for (int i = 0; i < n; ++i) {
    p.cs[(size_t)(pos0 + i) * half + m] = make_float2((float)c, (float)s);
    const double cn = c * cd - s * sd;
    s = s * cd + c * sd;
    c = cn;
  }
}

void launch_table(const TableParams& p, hipStream_t s) {
  const long n = (long)((p.N + TABLE_RUN - 1) / TABLE_RUN) * (p.D / 2);
  hipLaunchKernelGGL(table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p);
}

// One thread per 8 consecutive elements of a row.  Q and K are rotated
// (pairs (2m, 2m+1) turned by +p theta_hat_m), V and dO converted; every
// output plane is fp16.  D_i = sum_c dO_ic O_ic is the gamma_2 row scalar of
// "RoPE attention can be trained in almost-linear time" (Methodology 2).
// The pass is bound by HBM: every input of a thread is loaded (one 16-byte
// load per bf16 chunk) before anything is stored, so all its loads are in
// flight together.
// 8 consecutive input elements as stored (bf16: one uint4; fp32: two), and
// their float values; loading and converting are separate steps so that a
// thread's loads are all issued before the first conversion waits
struct Raw8 {
  uint4 a, b;
};
template <bool BF16>
__device__ __forceinline__ Raw8 load8(const void* base, size_t idx) {
  Raw8 r;
  if constexpr (BF16) {
    r.a = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + idx);
    r.b = r.a;
  } else {
    const uint4* f = reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(base) + idx);
    r.a = f[0];
    r.b = f[1];
  }
  return r;
}
template <bool BF16>
__device__ __forceinline__ void unpack8(const Raw8& r, float* x) {
  if constexpr (BF16) {
    const uint32_t w[4] = {r.a.x, r.a.y, r.a.z, r.a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
    const uint32_t w[8] = {r.a.x, r.a.y, r.a.z, r.a.w, r.b.x, r.b.y, r.b.z, r.b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = __uint_as_float(w[i]);
  }
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

// Partial maxima of |dO| (bf16), AMAX_SLOTS per head: block (slot, bh)
// takes every AMAX_SLOTS-th 256-chunk group of the head.  Grid (AMAX_SLOTS,
// heads mod 4096, heads / 4096).
__global__ __launch_bounds__(256) void absmax_kernel(AbsmaxParams p) {
  __shared__ float red[4];
  const int bh = (int)blockIdx.z * 4096 + (int)blockIdx.y;   // heads over y and z (y < 4096)
  if (bh >= p.BH) return;
  const size_t chunks = (size_t)p.N * p.D / 8;
  const uint4* src = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(p.x) +
                                                    (size_t)bh * p.N * p.D);
  uint32_t mx = 0;   // max of |x| as bf16 bit patterns (the order of non-negative floats)
  constexpr size_t STRIDE = (size_t)AMAX_SLOTS * 256;
  constexpr int U = 4;   // loads in flight per thread
  for (size_t c0 = (size_t)blockIdx.x * 256 + threadIdx.x; c0 < chunks; c0 += STRIDE * U) {
    uint4 u[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const size_t c = c0 + STRIDE * j;
      u[j] = c < chunks ? src[c] : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const uint32_t w[4] = {u[j].x, u[j].y, u[j].z, u[j].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        mx = max(mx, w[i] & 0x7fffu);
        mx = max(mx, (w[i] >> 16) & 0x7fffu);
      }
    }
  }
  float f = __uint_as_float(mx << 16);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) f = fmaxf(f, __shfl_xor(f, off, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = f;
  __syncthreads();
  if (threadIdx.x == 0)
    p.amax[(size_t)bh * AMAX_SLOTS + blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

void launch_absmax(const AbsmaxParams& p, hipStream_t s) {
  const dim3 grid(AMAX_SLOTS, (unsigned)(p.BH < 4096 ? p.BH : 4096), (unsigned)((p.BH + 4095) / 4096));
  hipLaunchKernelGGL(absmax_kernel, grid, dim3(256), 0, s, p);
}

// The head's dO scale s = 2^(2 - floor(log2 max)), clamped to [2^-126, 2^126]
// (1 for a head whose dO is all zero or not finite), from its partial maxima.
__device__ __forceinline__ float dO_scale(const float* amax) {
  float mx = 0.f;
#pragma unroll
  for (int i = 0; i < AMAX_SLOTS; ++i) mx = fmaxf(mx, amax[i]);
  if (!(mx > 0.f) || !(mx <= 3.0e38f)) return 1.f;
  const int e = (int)((__float_as_uint(mx) >> 23) & 0xffu);   // biased exponent (0: subnormal)
  const int sh = min(126, max(-126, 129 - max(e, 1)));        // 2 - (e - 127)
  return __uint_as_float((uint32_t)(sh + 127) << 23);
}

// BF16: the input storage (compile time, so that no branch separates a
// load from its use and every load of a thread issues before the first wait)
// Grid: x over the chunks of one head (N * D / 8 < 2^28), y and z over the
// heads (bh = 4096 z + y): the head is a scalar and the position and chunk
// are shifts, so no thread divides.
constexpr int PREP_HEADS_Y = 4096;

template <bool BF16>
__global__ void prep_kernel(PrepParams p) {
  const int cshift = p.D == 128 ? 4 : 3;          // chunks per row: 16 or 8
  const int cpr = 1 << cshift;
  const int bh = (int)blockIdx.z * PREP_HEADS_Y + (int)blockIdx.y;
  const int lin = (int)blockIdx.x * 256 + (int)threadIdx.x;   // chunk within the head
  const bool live = bh < p.BH && lin < (p.N << cshift);
  const int pos = live ? lin >> cshift : 0;
  const int chunk = lin & (cpr - 1);
  const size_t row = (size_t)bh * p.N + pos;      // bh * N + pos
  const size_t e0 = row * p.D + (size_t)chunk * 8;
  // this head's dO scale (a power of two; 1 without amax)
  const float dsc = (p.amax && bh < p.BH) ? dO_scale(p.amax + (size_t)bh * AMAX_SLOTS) : 1.f;
  if (p.amax && p.dsc && lin == 0 && bh < p.BH) p.dsc[bh] = 1.f / dsc;
  float xq[8], xk[8], xv[8], xd[8];
  Raw8 rq = {}, rk = {}, rv = {}, rd = {};
  float4 oa = {}, ob = {};
  float2 cs[4] = {};
  if (live) {
    if (p.qh) rq = load8<BF16>(p.q, e0);
    if (p.kh) rk = load8<BF16>(p.k, e0);
    if (p.vh) rv = load8<BF16>(p.v, e0);
    if (p.doh || p.drow) rd = load8<BF16>(p.dO, e0);
    if (p.drow) {
      const float4* o4 = reinterpret_cast<const float4*>(p.o + e0);
      oa = o4[0];
      ob = o4[1];
    }
    if (p.qh || p.kh) {
      const float4* c4 = reinterpret_cast<const float4*>(p.cs + (size_t)pos * (p.D / 2) + chunk * 4);
      const float4 c01 = c4[0], c23 = c4[1];
      cs[0] = make_float2(c01.x, c01.y); cs[1] = make_float2(c01.z, c01.w);
      cs[2] = make_float2(c23.x, c23.y); cs[3] = make_float2(c23.z, c23.w);
    }
    unpack8<BF16>(rq, xq);
    unpack8<BF16>(rk, xk);
    unpack8<BF16>(rv, xv);
    unpack8<BF16>(rd, xd);
    // all arithmetic before the first store: a wait for a load issued
    // before a store also waits for that store
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      rot(cs[i].x, cs[i].y, xq[2 * i], xq[2 * i + 1]);
      rot(cs[i].x, cs[i].y, xk[2 * i], xk[2 * i + 1]);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      xq[i] *= p.qscale;
      xd[i] *= dsc;
    }
    if (p.flags) {
      // an operand entry fp16 cannot hold (it would become +-inf)
      bool out = false;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (p.qh) out |= !(fabsf(xq[i]) <= 65504.f);
        if (p.kh) out |= !(fabsf(xk[i]) <= 65504.f);
        if (p.vh) out |= !(fabsf(xv[i]) <= 65504.f);
      }
      if (__any(out) && (threadIdx.x & 63) == __builtin_amdgcn_readfirstlane(threadIdx.x & 63))
        atomicOr(p.flags, FLAG_FP16_RANGE);
    }
    if (p.qh) store8h(p.qh + e0, xq);
    if (p.kh) store8h(p.kh + e0, xk);
    if (p.vh) store8h(p.vh + e0, xv);
    if (pos < p.rlo) {
      const size_t lo = ((size_t)bh * p.rlo + pos) * p.D + chunk * 8;
      if (p.qh && p.qlo) store8lo(p.qlo + lo, xq);
      if (p.kh && p.klo) store8lo(p.klo + lo, xk);
    }
  }
  // the planes' zero pad rows after the last head (PLANE_PAD_ROWS x D)
  if (bh == 0 && lin < PLANE_PAD_ROWS * cpr) {
    const size_t e = (size_t)p.BH * p.N * p.D + (size_t)lin * 8;
    const half8 z = {};
    if (p.qh) *reinterpret_cast<half8*>(p.qh + e) = z;
    if (p.kh) *reinterpret_cast<half8*>(p.kh + e) = z;
    if (p.vh) *reinterpret_cast<half8*>(p.vh + e) = z;
    if (p.doh) *reinterpret_cast<half8*>(p.doh + e) = z;
  }
  if (p.doh || p.drow) {
    float acc = 0.f;
    if (live) {
      if (p.doh) store8h(p.doh + e0, xd);
      if (p.drow)
        acc = xd[0] * oa.x + xd[1] * oa.y + xd[2] * oa.z + xd[3] * oa.w +
              xd[4] * ob.x + xd[5] * ob.y + xd[6] * ob.z + xd[7] * ob.w;
    }
    if (p.drow) {
      // the cpr lanes of a row are consecutive and aligned inside the wave
      for (int off = 1; off < cpr; off <<= 1) acc += __shfl_xor(acc, off, 64);
      if (live && chunk == 0) {
        p.drow[row] = acc;
        if (p.rs) {
          const int G = rs_groups(p.N);
          float* rsh = p.rs + (size_t)bh * G * 64;
          rsh[(pos >> 5) * 64 + (pos & 31)] = -(p.lse[row] * LOG2E);
          rsh[(pos >> 5) * 64 + 32 + (pos & 31)] = -acc;
          if (pos == p.N - 1) {  // pad rows up to the end of the spare group
            for (int r = p.N; r < 32 * G; ++r) {
              rsh[(r >> 5) * 64 + (r & 31)] = -INFINITY;
              rsh[(r >> 5) * 64 + 32 + (r & 31)] = 0.f;
            }
          }
        }
      }
    }
  }
}

void launch_prep(const PrepParams& p, hipStream_t s) {
  // every chunk of every row, and at least the planes' pad chunks
  const int per_head = max(p.N * (p.D / 8), PLANE_PAD_ROWS * (p.D / 8));
  const int hy = min(p.BH, PREP_HEADS_Y);
  const dim3 grid((unsigned)((per_head + 255) / 256), (unsigned)hy,
                  (unsigned)((p.BH + PREP_HEADS_Y - 1) / PREP_HEADS_Y)),
      block(256);
  if (p.bf16) hipLaunchKernelGGL(prep_kernel<true>, grid, block, 0, s, p);
  else hipLaunchKernelGGL(prep_kernel<false>, grid, block, 0, s, p);
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
  // eight independent partial sums per thread, so its loads are all in
  // flight at once; they combine in a fixed order (deterministic)
  constexpr int U = 8;
  double acc[U] = {};
  for (int s0 = threadIdx.x; s0 < p.slots; s0 += 256 * U) {
    float x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = s0 + 256 * u;
      x[u] = s < p.slots ? p.part[(size_t)s * half + m] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc[u] += (double)x[u];
  }
  double a = 0.0;
#pragma unroll
  for (int u = 0; u < U; ++u) a += acc[u];
  red[threadIdx.x] = a;
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
