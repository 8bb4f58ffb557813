// Causal corner of the forward with split fp16 operands (bf16 inputs): query
// rows [0, corner) against the keys they see, every rotated operand and P
// split into hi + lo fp16 parts (about 22 bits; see corner.h, which also
// holds the backward's corner parts).  s(x) and O = P V as in mfma.hip ("RoPE
// attention can be trained in almost-linear time", Methodology 1).
#include "corner.h"

namespace ra {

namespace {

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
    stage3<D, BN>(Kh, p.kh + head, Kl, p.klo + lhead, Vs, p.vh + head, k0, p.N, nlo);
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

}  // namespace

void launch_corner_fwd(const MfmaParams& p, hipStream_t s) {
  const dim3 grid((unsigned)corner_blocks(p)), block(256);
  if (p.D == 64) hipLaunchKernelGGL(corner_fwd_kernel<64>, grid, block, 0, s, p);
  else hipLaunchKernelGGL(corner_fwd_kernel<128>, grid, block, 0, s, p);
}
}  // namespace ra
