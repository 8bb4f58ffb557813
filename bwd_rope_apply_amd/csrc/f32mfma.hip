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
// [32][D + 4], staged (and rotated) from the inputs; each workgroup owns 64
// rows (or keys) as two waves of 32, the same 64-row blocks as the vector
// path, so the d alpha partial slots are the same.  Small launches give a
// workgroup 2 or 4 such pairs of waves, each over part of the streamed
// range (see GroupSteps below).
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
// rotated when cs != null; rows outside [0, N) are zero.  128 threads, tid
// in [0, 128).
template <int D, int LD>
__device__ __forceinline__ void stage_f32(float* dst, const void* src, size_t head_off, int r0,
                                          int N, int bf16, const float2* cs, int tid) {
  constexpr int CH = D / 4;
  for (int t = tid; t < FT * CH; t += 128) {
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

// The wedge partials of the first two waves of a workgroup (finish_rows'
// layout) summed into one [D/2] slot; every thread of the workgroup calls
// it (one barrier), waves past the first two hold no partials.
template <int D>
__device__ __forceinline__ void store_dalpha2(float* w, float* red, float* slot, int g) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (wave < 2) {
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
  }
  __syncthreads();
  for (int m = threadIdx.x; m < D / 2; m += 128) slot[m] = red[m] + red[D / 2 + m];
}

// G: groups of 128 threads per workgroup.  Launches too small to fill the
// GPU (tiny problems are bound by each workgroup's chain of steps) split the
// streamed range (keys in the forward and dQ, queries in dK/dV) between G
// groups on the same rows; each group stages its own tiles, every thread
// runs the same number of steps (a group past its own range only keeps the
// barriers), and groups 1 .. G-1 hand their partial results to group 0
// through the staging tiles, which adds them in that order.

// This group's steps of a range of n: [first, first + count), count <= h.
struct GroupSteps {
  int h, first, count;
  __device__ GroupSteps(int n, int G, int grp) {
    h = (n + G - 1) / G;
    first = grp * h;
    count = max(0, min(n - first, h));
  }
};

// Hands over NV floats a lane (x[0 .. NV)) from each group past the first
// to group 0 through buf ((G - 1) x 128 x NV floats); merge(x, j) runs in
// group 0 for j = 1 .. G-1 in order.  Every thread calls it (two barriers).
template <int G, int NV, typename Put, typename Merge>
__device__ __forceinline__ void hand_over(float* buf, int grp, int tid, Put put, Merge merge) {
  __syncthreads();   // every group is done with the staging tiles
  if (grp > 0) {
    float x[NV];
    put(x);
#pragma unroll
    for (int v = 0; v < NV; ++v) buf[((grp - 1) * NV + v) * 128 + tid] = x[v];
  }
  __syncthreads();
  if (grp == 0) {
    for (int j = 1; j < G; ++j) {
      float x[NV];
#pragma unroll
      for (int v = 0; v < NV; ++v) x[v] = buf[((j - 1) * NV + v) * 128 + tid];
      merge(x, j);
    }
  }
}

template <int D, bool CAUSAL, int G>
__global__ __launch_bounds__(128 * G) void f32_fwd_kernel(SimtParams p) {
  constexpr int LD = D + 4, CB = D / 32, TSZ = FT * LD;
  static_assert(G == 1 || 2 * G * TSZ >= (G - 1) * 128 * (16 * CB + 2), "hand-over fits the tiles");
  __shared__ __attribute__((aligned(16))) float pool[G * 2 * TSZ];
  const int bh = blockIdx.y;
  const int grp = threadIdx.x >> 7, tid = threadIdx.x & 127;
  const int lane = threadIdx.x & 63, w = tid >> 6, l32 = lane & 31, g = lane >> 5;
  float* ks = pool + grp * 2 * TSZ;
  float* vs = ks + TSZ;
  const int r0 = blockIdx.x * FW, q = r0 + 32 * w + l32;   // this lane's query
  const size_t head = (size_t)bh * p.N * D;
  float qf[D / 2];
  row_frags<D>(qf, p.q, head, q, p.N, p.bf16, p.cs, g);
  f32x16 o[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) o[cb] = f32x16{};
  float m = -INFINITY, l = 0.f;
  const int kend = CAUSAL ? min(p.N, r0 + FW) : p.N;
  const GroupSteps st((kend + FT - 1) / FT, G, grp);
  for (int i = 0; i < st.h; ++i) {
    const int k0 = (st.first + i) * FT;
    const bool mine = i < st.count;
    __syncthreads();
    if (mine) {
      stage_f32<D, LD>(ks, p.k, head, k0, p.N, p.bf16, p.cs, tid);
      stage_f32<D, LD>(vs, p.v, head, k0, p.N, p.bf16, nullptr, tid);
    }
    __syncthreads();
    if (!mine) continue;
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
  if constexpr (G > 1) {
    // partial softmax states (each row's max is the same in both of its
    // lanes; a group that saw no key of a row has m = -inf, O = l = 0)
    hand_over<G, 16 * CB + 2>(pool, grp, tid,
        [&](float* x) {
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) x[16 * cb + r] = o[cb][r];
          }
          x[16 * CB] = m;
          x[16 * CB + 1] = l;
        },
        [&](const float* x, int) {
          const float mj = x[16 * CB], mn = fmaxf(m, mj);
          const float a0 = m == -INFINITY ? 0.f : expf(m - mn);
          const float aj = mj == -INFINITY ? 0.f : expf(mj - mn);
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) o[cb][r] = o[cb][r] * a0 + x[16 * cb + r] * aj;
          }
          l = l * a0 + x[16 * CB + 1] * aj;
          m = mn;
        });
  }
  l += __shfl_xor(l, 32, 64);
  if (grp == 0 && q < p.N) {
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

template <int D, bool CAUSAL, int G>
__global__ __launch_bounds__(128 * G) void f32_dq_kernel(SimtParams p) {
  constexpr int LD = D + 4, CB = D / 32, TSZ = FT * LD;
  static_assert(G == 1 || 2 * G * TSZ >= (G - 1) * 128 * (16 * CB), "hand-over fits the tiles");
  __shared__ __attribute__((aligned(16))) float pool[G * 2 * TSZ];
  __shared__ float red[2 * (D / 2)];
  const int bh = blockIdx.y;
  const int grp = threadIdx.x >> 7, tid = threadIdx.x & 127;
  const int lane = threadIdx.x & 63, w = tid >> 6, l32 = lane & 31, g = lane >> 5;
  float* ks = pool + grp * 2 * TSZ;
  float* vs = ks + TSZ;
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
  const GroupSteps st((kend + FT - 1) / FT, G, grp);
  for (int i = 0; i < st.h; ++i) {
    const int k0 = (st.first + i) * FT;
    const bool mine = i < st.count;
    __syncthreads();
    if (mine) {
      stage_f32<D, LD>(ks, p.k, head, k0, p.N, p.bf16, p.cs, tid);
      stage_f32<D, LD>(vs, p.v, head, k0, p.N, p.bf16, nullptr, tid);
    }
    __syncthreads();
    if (!mine) continue;
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
  if constexpr (G > 1) {
    hand_over<G, 16 * CB>(pool, grp, tid,
        [&](float* x) {
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) x[16 * cb + r] = acc[cb][r];
          }
        },
        [&](const float* x, int) {
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[cb][r] += x[16 * cb + r];
          }
        });
  }
  float wv[D / 4];
#pragma unroll
  for (int i = 0; i < D / 4; ++i) wv[i] = 0.f;
  if (grp == 0 && q_ok)
    finish_rows<D>(acc, p.scale, nullptr, p.cs + (size_t)q * (D / 2), p.q, head + (size_t)q * D,
                   p.bf16, p.dq + head + (size_t)q * D, (float)q, wv, g);
  const int slot = p.slot0 + bh * gridDim.x + blockIdx.x;
  store_dalpha2<D>(wv, red, p.dalpha_part + (size_t)slot * (D / 2), g);
}

template <int D, bool CAUSAL, int G>
__global__ __launch_bounds__(128 * G) void f32_dkdv_kernel(SimtParams p) {
  constexpr int LD = D + 4, CB = D / 32, TSZ = FT * LD;
  // the hand-over goes dK then dV, 16 CB floats a lane each
  static_assert(G == 1 || 2 * G * TSZ >= (G - 1) * 128 * (16 * CB), "hand-over fits the tiles");
  __shared__ __attribute__((aligned(16))) float pool[G * 2 * TSZ];
  __shared__ __attribute__((aligned(16))) float vst[FW * LD];   // this workgroup's V rows
  __shared__ float lsg[G][2][FT];   // each group's row scalars: LSE, D
  __shared__ float red[2 * (D / 2)];
  const int bh = blockIdx.y;
  const int grp = threadIdx.x >> 7, tid = threadIdx.x & 127;
  const int lane = threadIdx.x & 63, w = tid >> 6, l32 = lane & 31, g = lane >> 5;
  float* qs = pool + grp * 2 * TSZ;
  float* dos = qs + TSZ;
  float* lses = lsg[grp][0];
  float* drs = lsg[grp][1];
  const int k0 = blockIdx.x * FW, key = k0 + 32 * w + l32;   // this lane's key
  const size_t head = (size_t)bh * p.N * D;
  const bool key_ok = key < p.N;
  float kf[D / 2];
  row_frags<D>(kf, p.k, head, key, p.N, p.bf16, p.cs, g);
  if (grp == 0) {   // published by the first step's barrier
    stage_f32<D, LD>(vst, p.v, head, k0, p.N, p.bf16, nullptr, tid);
    stage_f32<D, LD>(vst + FT * LD, p.v, head, k0 + FT, p.N, p.bf16, nullptr, tid);
  }
  const float* vrow = vst + (32 * w + l32) * LD + g;   // B elements of dP: V[key][2 kk + g]
  f32x16 dk[CB], dv[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) { dk[cb] = f32x16{}; dv[cb] = f32x16{}; }
  const int qstart = CAUSAL ? k0 : 0;
  const GroupSteps st(qstart < p.N ? (p.N - qstart + FT - 1) / FT : 0, G, grp);
  for (int i = 0; i < st.h; ++i) {
    const int r0 = qstart + (st.first + i) * FT;
    const bool mine = i < st.count;
    __syncthreads();
    if (mine) {
      stage_f32<D, LD>(qs, p.q, head, r0, p.N, p.bf16, p.cs, tid);
      stage_f32<D, LD>(dos, p.dO, head, r0, p.N, p.bf16, nullptr, tid);
      if (tid < FT) {
        const int row = r0 + tid;
        const bool ok = row < p.N;
        lses[tid] = ok ? p.lse[(size_t)bh * p.N + row] : 0.f;
        drs[tid] = ok ? p.drow[(size_t)bh * p.N + row] : 0.f;
      }
    }
    __syncthreads();
    if (!mine) continue;
    f32x16 s = score32<D, LD>(qs, kf, l32, g);   // S: register r, query r0 + 2r + g
    f32x16 dp = {};
    {
      const float* arow = dos + pi32(l32) * LD + g;
#pragma unroll
      for (int kk = 0; kk < D / 2; ++kk) dp = mfma32(arow[2 * kk], vrow[2 * kk], dp);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int i2 = 2 * r + g, row = r0 + i2;
      const bool ok = key_ok && row < p.N && (!CAUSAL || row >= key);
      const float pr = ok ? expf(s[r] * p.scale - lses[i2]) : 0.f;
      s[r] = pr;
      dp[r] = pr * (dp[r] - drs[i2]);   // dS
    }
    accumulate_t32<D, LD>(dv, dos, s, l32, g);   // dV^T += dO^T P
    accumulate_t32<D, LD>(dk, qs, dp, l32, g);   // dK~^T += Q~^T dS
  }
  if constexpr (G > 1) {
    auto put = [](const f32x16* a) {
      return [a](float* x) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) x[16 * cb + r] = a[cb][r];
        }
      };
    };
    auto add = [](f32x16* a) {
      return [a](const float* x, int) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) a[cb][r] += x[16 * cb + r];
        }
      };
    };
    hand_over<G, 16 * CB>(pool, grp, tid, put(dk), add(dk));
    hand_over<G, 16 * CB>(pool, grp, tid, put(dv), add(dv));
  }
  float wv[D / 4];
#pragma unroll
  for (int i = 0; i < D / 4; ++i) wv[i] = 0.f;
  if (grp == 0 && key_ok) {
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

// Groups per workgroup: 4 (D = 64 only: the tiles of four groups fit the
// LDS beside dK/dV's V rows) for launches of at most 64 workgroups, 2 for at
// most 256, else 1.
int f32_groups(const SimtParams& p) {
  const long nwg = (long)((p.N + FW - 1) / FW) * p.BH;
  if (nwg <= 64 && p.D == 64) return 4;
  return nwg <= 256 ? 2 : 1;
}

#define RA_F32_LAUNCH_DG(KERNEL, DD, G)                                                       \
  do {                                                                                        \
    if (p.causal) hipLaunchKernelGGL((KERNEL<DD, true, G>), grid, dim3(128 * (G)), 0, s, p);  \
    else hipLaunchKernelGGL((KERNEL<DD, false, G>), grid, dim3(128 * (G)), 0, s, p);          \
  } while (0)
#define RA_F32_LAUNCH(KERNEL)                                              \
  do {                                                                     \
    const dim3 grid = f32_grid(p);                                         \
    const int groups = f32_groups(p);                                      \
    if (p.D == 64) {                                                       \
      if (groups == 4) RA_F32_LAUNCH_DG(KERNEL, 64, 4);                    \
      else if (groups == 2) RA_F32_LAUNCH_DG(KERNEL, 64, 2);               \
      else RA_F32_LAUNCH_DG(KERNEL, 64, 1);                                \
    } else {                                                               \
      if (groups == 2) RA_F32_LAUNCH_DG(KERNEL, 128, 2);                   \
      else RA_F32_LAUNCH_DG(KERNEL, 128, 1);                               \
    }                                                                      \
  } while (0)

}  // namespace

void launch_f32_fwd(const SimtParams& p, hipStream_t s) { RA_F32_LAUNCH(f32_fwd_kernel); }
void launch_f32_dq(const SimtParams& p, hipStream_t s) { RA_F32_LAUNCH(f32_dq_kernel); }
void launch_f32_dkdv(const SimtParams& p, hipStream_t s) { RA_F32_LAUNCH(f32_dkdv_kernel); }

}  // namespace ra
