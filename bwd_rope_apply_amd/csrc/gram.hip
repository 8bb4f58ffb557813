// Gram-threshold token selection ("Cascade token selection for transformer
// attention acceleration"): the causal Gram product of the tokens on the
// matrix cores with a running-maximum epilogue, the threshold decision, and
// the cascade's compaction, member check and cross check.
//
// Cosines are formed as <x_i, x_j> * inv_i * inv_j: the stored bf16 / fp16
// values enter the matrix cores unrounded (their products are exact in the
// float32 accumulator), and the inverse norms (float32 sums of exact
// squares) scale the result in the epilogue.
#include <limits.h>

#include <algorithm>
#include <math.h>
#include <stdint.h>

#include "gram_select.h"
#include "tile.h"

namespace ra {
namespace {

constexpr int KC = 64;             // features per LDS stage
constexpr int RSB = (KC + 8) * 2;  // LDS bytes per tile row (16-byte pad)

// Tile shape of the Gram kernel: KT keys x QT queries per workgroup, WK x WQ
// waves (each a (KT / WK) x (QT / WQ) block of 32 x 32 products).
template <int KT_, int QT_, int WK_, int WQ_>
struct Tiles {
  static constexpr int KT = KT_, QT = QT_, WK = WK_, WQ = WQ_;
  static constexpr int NW = WK * WQ, NT = 64 * NW;
  static constexpr int KBYTES = KT * RSB, QBYTES = QT * RSB, STAGE = KBYTES + QBYTES;
  static constexpr int NBK = KBYTES / 1024, NBQ = QBYTES / 1024;  // 1-KiB copy blocks per operand
  static constexpr int PWK = (NBK + NW - 1) / NW, PWQ = (NBQ + NW - 1) / NW;
  static constexpr int MB = KT / WK / 32, NB = QT / WQ / 32;      // 32 x 32 blocks per wave
  static constexpr int KM = KT / QT;  // a key tile spans KM query tiles (triangle walk)
  static constexpr int WG_PER_CU = 2 * STAGE <= 80 * 1024 ? 2 : 1;
  static_assert(KBYTES % 1024 == 0 && QBYTES % 1024 == 0, "tiles are whole copy blocks");
  static_assert(KT % QT == 0, "the triangle walk needs key tiles that are whole query tiles");
  // tiles of the query tiles q < a in the triangle walk: query tile q meets
  // the key tiles that start before its end, ceil((q + 1) / KM) of them
  static __host__ __device__ long long tri_before(long long a) {
    const long long u = a / KM, v = a % KM;
    return KM * u * (u + 1) / 2 + v * (u + 1);
  }
};
// 128 x 128 (2 workgroups per CU): fine-grained, for short sequences and
// the cascade's data-dependent lists; 256 x 256 (1 per CU): 1.5x the
// operand reuse per copied byte and per LDS read, for long sequences
typedef Tiles<128, 128, 2, 2> SmallTiles;
typedef Tiles<256, 256, 4, 2> LargeTiles;

constexpr int MAX_SPLITS = 16;     // feature-axis splits of a tile, at most
constexpr int ENC_NEG_INF = (int)(0xff800000u ^ 0x7fffffffu);

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// float <-> int with the same order (so an integer atomic max is a float max)
__device__ __forceinline__ int enc(float f) {
  const int i = __float_as_int(f);
  return i >= 0 ? i : i ^ 0x7fffffff;
}
__device__ __forceinline__ float dec(int k) { return __int_as_float(k >= 0 ? k : k ^ 0x7fffffff); }

struct GramParams {
  const void* x;                // [B][T][d] bf16 or fp16
  const float* inv;             // [B][T] inverse norms (0 for a zero token)
  const int* qidx;              // query tokens, ascending (null: 0..T-1)
  const int* kidx;              // key tokens, ascending (null: 0..T-1)
  const int* qn;                // device count of qidx (null: T)
  const int* kn;                // device count of kidx (null: T)
  const unsigned char* kvalid;  // per-token key mask (null: every key)
  int* mkey;                    // [B][T] running maximum, order-preserving int
  int B, T, d;
  int tri;                      // queries and keys are one list: lower-triangle tiles
  int tiles;                    // tiles per sequence in the grid (an upper bound)
  int splits;                   // feature-axis splits per tile (1: unsplit)
  int sub_first;                // >= 0: ids are the 4 quarter tiles of large-tile triangle
                                // ids sub_first, sub_first + 1, ... (sub_tiles per sequence)
  int sub_tiles;
  float* part;                  // split partial products (splits > 1)
  int contiguous;               // hand each XCD a contiguous run of tiles (every id is real work)
};

template <bool BF16>
struct Frag;
template <>
struct Frag<true> {
  typedef bf16x8 T;
  static __device__ __forceinline__ f32x16 mma(T a, T b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <>
struct Frag<false> {
  typedef half8 T;
  static __device__ __forceinline__ f32x16 mma(T a, T b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

// Tile decode shared by the Gram kernel and the split reduction: work id ->
// (sequence, tile slot b * tiles + tile, query and key tile, split, with
// `splits` ids per tile); false when the id is past the real work or the
// tile holds no key before any of its queries.
template <class C>
__device__ __forceinline__ bool decode_tile(const GramParams& p, int id, int splits, int& b, int& slot,
                                            int& q0, int& k0, int& split, int& nq, int& nk) {
  nq = p.qn ? *p.qn : p.T;
  nk = p.kn ? *p.kn : p.T;
  int qt, kt;
  if constexpr (LargeTiles::KT == 2 * C::KT && LargeTiles::QT == 2 * C::QT) {
    if (p.sub_first >= 0) {
      // quarter (id % 4) of large triangle tile sub_first + id / 4
      typedef LargeTiles L;
      const int big = p.sub_first + id / 4, quarter = id % 4;
      b = big / p.sub_tiles;
      const int tid = big - b * p.sub_tiles;
      int lo = 0, hi = (p.T + L::QT - 1) / L::QT;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (L::tri_before(mid) <= tid) lo = mid;
        else hi = mid;
      }
      qt = 2 * lo + (quarter >> 1);
      kt = 2 * (tid - (int)L::tri_before(lo)) + (quarter & 1);
      split = 0;
      slot = id;
      if (qt * C::QT >= nq || kt * C::KT >= nk) return false;
      q0 = qt * C::QT;
      k0 = kt * C::KT;
      return k0 < min(q0 + C::QT, nq) - 1;  // identity lists (the full selection)
    }
  }
  const int per_seq = p.tiles * splits;
  b = id / per_seq;
  const int within = id - b * per_seq;
  const int tid = within / splits;
  split = within - tid * splits;
  slot = b * p.tiles + tid;
  if (p.tri) {
    // the largest qt with tri_before(qt) <= tid
    int lo = 0, hi = (p.T + C::QT - 1) / C::QT;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (C::tri_before(mid) <= tid) lo = mid;
      else hi = mid;
    }
    qt = lo;
    kt = tid - (int)C::tri_before(qt);
    if (qt * C::QT >= nq) return false;
  } else {
    const int ntk = (nk + C::KT - 1) / C::KT, ntq = (nq + C::QT - 1) / C::QT;
    if (tid >= ntk * ntq) return false;
    qt = tid / ntk;
    kt = tid - qt * ntk;
  }
  q0 = qt * C::QT;
  k0 = kt * C::KT;
  const int qlast = min(q0 + C::QT, nq) - 1;
  const int tq = p.qidx ? p.qidx[qlast] : qlast;
  const int tk = p.kidx ? p.kidx[k0] : k0;
  return tk < tq;
}

// token, inverse norm and mask of the tile's keys and queries, into LDS
// (keys not in the list or not valid get INT_MAX, which no query exceeds)
template <class C>
__device__ __forceinline__ void tile_rows(const GramParams& p, size_t seq, int q0, int k0, int nq,
                                          int nk, int* kpos, int* qpos, float* kinv, float* qinv) {
  for (int t = threadIdx.x; t < C::KT + C::QT; t += C::NT) {
    if (t < C::KT) {
      const int i = k0 + t;
      int tok = INT_MAX;
      float iv = 0.f;
      if (i < nk) {
        const int tk = p.kidx ? p.kidx[i] : i;
        iv = p.inv[seq + tk];
        tok = (p.kvalid && !p.kvalid[tk]) ? INT_MAX : tk;
      }
      kpos[t] = tok;
      kinv[t] = iv;
    } else {
      const int r = t - C::KT, i = q0 + r;
      int tok = -1;
      float iv = 0.f;
      if (i < nq) {
        tok = p.qidx ? p.qidx[i] : i;
        iv = p.inv[seq + tok];
      }
      qpos[r] = tok;
      qinv[r] = iv;
    }
  }
}

// Each query's column of the products scaled to cosines, masked to keys
// before the query, reduced to its maximum and merged into the global
// maximum with an integer atomic max (exact and order-independent).
template <class C>
__device__ __forceinline__ void tile_max(const f32x16 (&acc)[C::MB][C::NB], const GramParams& p,
                                         size_t seq, const int* kpos, const int* qpos,
                                         const float* kinv, const float* qinv, int w) {
  const int lane = threadIdx.x & 63, l32 = lane & 31, g = lane >> 5;
  const int kh = w / C::WQ, qh = w % C::WQ;
#pragma unroll
  for (int n = 0; n < C::NB; ++n) {
    const int ql_ = qh * (C::QT / C::WQ) + n * 32 + l32;
    const int qtok = qpos[ql_];
    float mx = -INFINITY;
#pragma unroll
    for (int m = 0; m < C::MB; ++m)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kl_ = kh * (C::KT / C::WK) + m * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
        const float v = acc[m][n][r] * kinv[kl_];
        if (kpos[kl_] < qtok) mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    if (g == 0 && qtok >= 0 && mx > -INFINITY) atomicMax(p.mkey + seq + qtok, enc(mx * qinv[ql_]));
  }
}

// Workgroup = a KT-key x QT-query tile (keys along the MFMA's m, so a lane
// holds one query's column).  The feature axis is streamed in 64-wide
// stages through double-buffered LDS by direct global->LDS copies; each
// tile row carries a 16-byte pad, so the 32 rows a 128-bit fragment read
// touches fall on distinct banks.  With SPLIT the workgroup covers one of
// p.splits contiguous ranges of the stages and stores its partial products
// (in the accumulators' own lane layout) for gram_reduce_kernel; otherwise
// it finishes the tile itself.
template <bool BF16, class C, bool SPLIT>
__global__ __launch_bounds__(C::NT, C::WG_PER_CU) void gram_max_kernel(GramParams p) {
  typedef typename Frag<BF16>::T vec;
  constexpr int KT = C::KT, QT = C::QT, WK = C::WK, WQ = C::WQ, NW = C::NW;
  constexpr int KBYTES = C::KBYTES, STAGE = C::STAGE, NBK = C::NBK, NBQ = C::NBQ;
  constexpr int PWK = C::PWK, PWQ = C::PWQ, MB = C::MB, NB = C::NB;
  __shared__ __attribute__((aligned(16))) char lds[2 * STAGE];  // [stage][keys | queries]
  __shared__ int kpos[KT], qpos[QT];
  __shared__ float kinv[KT], qinv[QT];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, l32 = lane & 31, g = lane >> 5;
  // work id: the hardware deals workgroups to the 8 XCDs in turn.  When
  // every id is real work, each XCD gets a contiguous run of tiles, so tiles
  // that share rows share its L2; when only a prefix of the ids is real (the
  // cascade's grids are sized for the worst case), ids stay dealt in turn so
  // the real ones spread over all XCDs.
  int id = blockIdx.x;
  if (p.contiguous) {
    const int nblk = gridDim.x, xcd = blockIdx.x & 7, jx = blockIdx.x >> 3;
    const int per = nblk >> 3, rem = nblk & 7;
    id = xcd < rem ? xcd * (per + 1) + jx : rem * (per + 1) + (xcd - rem) * per + jx;
  }
  int b, slot, q0, k0, split, nq, nk;
  if (!decode_tile<C>(p, id, SPLIT ? p.splits : 1, b, slot, q0, k0, split, nq, nk)) return;
  const size_t seq = (size_t)b * p.T;
  if (!SPLIT) tile_rows<C>(p, seq, q0, k0, nq, nk, kpos, qpos, kinv, qinv);

  // per-lane copy offsets (bytes from the start of the sequence's first
  // feature stage): copy block w + NW i of an operand tile, 16 bytes a lane;
  // the pad chunk of a row re-reads the row's first chunk (never used)
  const int wave = __builtin_amdgcn_readfirstlane(w);
  auto offset = [&](int blk, int r0, int n, const int* idx, int rows) -> uint32_t {
    const int o = blk * 1024 + 16 * lane;
    const int row = min(o / RSB, rows - 1), within = o % RSB;
    const uint32_t col = within < 2 * KC ? (uint32_t)within : 0u;
    const int li = min(r0 + row, n - 1);
    const int tok = idx ? idx[li] : li;
    return (uint32_t)tok * (uint32_t)(2 * p.d) + col;
  };
  uint32_t offk[PWK], offq[PWQ];
#pragma unroll
  for (int i = 0; i < PWK; ++i) offk[i] = offset(w + NW * i, k0, nk, p.kidx, KT);
#pragma unroll
  for (int i = 0; i < PWQ; ++i) offq[i] = offset(w + NW * i, q0, nq, p.qidx, QT);
  const char* xs = reinterpret_cast<const char*>(p.x) + seq * (size_t)p.d * 2;
  auto issue = [&](int c, int stage) {
    const char* base = xs + (size_t)c * (2 * KC);
    char* dst = lds + stage * STAGE;
#pragma unroll
    for (int i = 0; i < PWK; ++i)
      if (wave + NW * i < NBK) lds_copy16(base, offk[i], dst + (wave + NW * i) * 1024);
#pragma unroll
    for (int i = 0; i < PWQ; ++i)
      if (wave + NW * i < NBQ) lds_copy16(base, offq[i], dst + KBYTES + (wave + NW * i) * 1024);
  };

  const int kh = w / WQ, qh = w % WQ;
  f32x16 acc[MB][NB];
#pragma unroll
  for (int a = 0; a < MB; ++a)
#pragma unroll
    for (int c = 0; c < NB; ++c) acc[a][c] = f32x16{};
  const int nc = p.d / KC;
  const int c0 = SPLIT ? split * nc / p.splits : 0, c1 = SPLIT ? (split + 1) * nc / p.splits : nc;
  issue(c0, 0);
  wait_lds_copies();
  __syncthreads();
  for (int c = c0; c < c1; ++c) {
    const int cur = (c - c0) & 1;
    if (c + 1 < c1) issue(c + 1, cur ^ 1);
    __builtin_amdgcn_sched_barrier(0);  // keep the next stage's copies ahead of the products
    const char* kl = lds + cur * STAGE + (kh * (KT / WK) + l32) * RSB + 16 * g;
    const char* ql = lds + cur * STAGE + KBYTES + (qh * (QT / WQ) + l32) * RSB + 16 * g;
#pragma unroll
    for (int s = 0; s < KC / 16; ++s) {
      vec a[MB], bq[NB];
#pragma unroll
      for (int m = 0; m < MB; ++m) a[m] = *reinterpret_cast<const vec*>(kl + m * 32 * RSB + 32 * s);
#pragma unroll
      for (int n = 0; n < NB; ++n) bq[n] = *reinterpret_cast<const vec*>(ql + n * 32 * RSB + 32 * s);
#pragma unroll
      for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int n = 0; n < NB; ++n) acc[m][n] = Frag<BF16>::mma(a[m], bq[n], acc[m][n]);
    }
    wait_lds_copies();
    __syncthreads();
  }

  if (SPLIT) {
    // partial products of this split, [tile slot][wave][split][block][reg/4][lane][4]
    float4* dst = reinterpret_cast<float4*>(p.part) +
                  (((size_t)slot * NW + w) * p.splits + split) * (size_t)(MB * NB * 4 * 64) + lane;
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
      for (int n = 0; n < NB; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          dst[((m * NB + n) * 4 + r) * 64] =
              make_float4(acc[m][n][4 * r], acc[m][n][4 * r + 1], acc[m][n][4 * r + 2], acc[m][n][4 * r + 3]);
    return;
  }
  tile_max<C>(acc, p, seq, kpos, qpos, kinv, qinv, w);
}

// Sum of a split tile's partial products in split order (deterministic),
// then the unsplit epilogue, element-wise: one thread per 4 accumulator
// registers (4 consecutive keys of one query) of one tile slot, so the
// partial reads of every split are in flight at once and spread over the
// chip; each thread merges its 4 keys' maximum into its query's.
template <class C>
__global__ __launch_bounds__(256) void gram_reduce_kernel(GramParams p, int slots) {
  constexpr int MB = C::MB, NB = C::NB, NW = C::NW;
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  const int lane = (int)(gid & 63);
  long long rest = gid >> 6;
  const int r4 = (int)(rest % 4);
  rest /= 4;
  const int n = (int)(rest % NB);
  rest /= NB;
  const int m = (int)(rest % MB);
  rest /= MB;
  const int w = (int)(rest % NW);
  const long long sl = rest / NW;
  if (sl >= slots) return;
  int b, slot, q0, k0, split, nq, nk;
  if (!decode_tile<C>(p, (int)sl, 1, b, slot, q0, k0, split, nq, nk)) return;
  const size_t seq = (size_t)b * p.T;
  const float4* src = reinterpret_cast<const float4*>(p.part) +
                      ((size_t)slot * NW + w) * p.splits * (size_t)(MB * NB * 4 * 64) +
                      ((m * NB + n) * 4 + r4) * 64 + lane;
  float4 u[MAX_SPLITS];
#pragma unroll
  for (int s = 0; s < MAX_SPLITS; ++s)  // all loads first, then the sum in split order
    if (s < p.splits) u[s] = src[(size_t)s * (MB * NB * 4 * 64)];
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int s = 0; s < MAX_SPLITS; ++s)
    if (s < p.splits) {
      v.x += u[s].x;
      v.y += u[s].y;
      v.z += u[s].z;
      v.w += u[s].w;
    }
  const int l32 = lane & 31, g = lane >> 5, kh = w / C::WQ, qh = w % C::WQ;
  const int qi = q0 + qh * (C::QT / C::WQ) + n * 32 + l32;
  if (qi >= nq) return;
  const int qtok = p.qidx ? p.qidx[qi] : qi;
  const float vv[4] = {v.x, v.y, v.z, v.w};
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int ki = k0 + kh * (C::KT / C::WK) + m * 32 + 8 * r4 + 4 * g + j;
    if (ki < nk) {
      const int tk = p.kidx ? p.kidx[ki] : ki;
      if (tk < qtok && !(p.kvalid && !p.kvalid[tk])) mx = fmaxf(mx, vv[j] * p.inv[seq + tk]);
    }
  }
  if (mx > -INFINITY) atomicMax(p.mkey + seq + qtok, enc(mx * p.inv[seq + qtok]));
}

// inverse norms, one wave per token: float32 sum of exact squares
template <bool BF16>
// (with mkey set: also resets the row's running maximum, and the first row
// of each sequence of T resets that sequence's count)
__global__ __launch_bounds__(256) void gram_norm_kernel(const void* x, float* inv, int rows, int d,
                                                        int* mkey, int* count, int T) {
  const int lane = threadIdx.x & 63, row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  if (mkey && lane == 0) {
    mkey[row] = ENC_NEG_INF;
    if (count && row % T == 0) count[row / T] = 0;
  }
  const uint4* xr = reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(x) + (size_t)row * d * 2);
  float s = 0.f;
  for (int c = lane; c < d / 8; c += 64) {
    const uint4 u = xr[c];
    const uint32_t wv[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      float lo, hi;
      if (BF16) {
        lo = __uint_as_float(wv[h] << 16);
        hi = __uint_as_float(wv[h] & 0xffff0000u);
      } else {
        lo = (float)__builtin_bit_cast(_Float16, (uint16_t)(wv[h] & 0xffffu));
        hi = (float)__builtin_bit_cast(_Float16, (uint16_t)(wv[h] >> 16));
      }
      s = fmaf(lo, lo, s);
      s = fmaf(hi, hi, s);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o, 64);
  if (lane == 0) inv[row] = s > 0.f ? 1.0f / sqrtf(s) : 0.f;
}

// decisions of the selection rule; blockIdx.y = sequence
__global__ __launch_bounds__(256) void gram_flags_kernel(const int* mkey, float thr, float* max_cos,
                                                          unsigned char* rep, int* count, int T) {
  __shared__ int part[4];
  const int t = blockIdx.x * 256 + threadIdx.x, b = blockIdx.y;
  int r = 0;
  if (t < T) {
    const size_t i = (size_t)b * T + t;
    const float m = dec(mkey[i]);
    r = m < thr;
    max_cos[i] = m;
    rep[i] = (unsigned char)r;
  }
  if (!count) return;
  const int wsum = __popcll(__ballot(r));
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = wsum;
  __syncthreads();
  if (threadIdx.x == 0) {
    const int c = part[0] + part[1] + part[2] + part[3];
    if (c) atomicAdd(count + b, c);
  }
}

// cascade step 1: the inherited members R and the other tokens N as
// ascending token lists (one workgroup of 1024 threads), counts in cnt[0..1];
// also resets the running maxima, the validity flags and the count
__global__ __launch_bounds__(1024) void gram_compact_kernel(const unsigned char* prev, int T, int* idxR,
                                                             int* idxN, int* cnt, int* mkey,
                                                             unsigned char* valid, int* count) {
  __shared__ int wr[16], wn[16];
  __shared__ int base[2];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (threadIdx.x == 0) base[0] = base[1] = 0;
  __syncthreads();
  for (int t0 = 0; t0 < T; t0 += 1024) {
    const int t = t0 + (int)threadIdx.x;
    const bool in = t < T && prev[t] != 0, out = t < T && prev[t] == 0;
    const unsigned long long br = __ballot(in), bn = __ballot(out);
    const int pr = __builtin_amdgcn_mbcnt_hi((uint32_t)(br >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)br, 0u));
    const int pn = __builtin_amdgcn_mbcnt_hi((uint32_t)(bn >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bn, 0u));
    if (lane == 0) {
      wr[w] = __popcll(br);
      wn[w] = __popcll(bn);
    }
    __syncthreads();
    int orr = base[0], on = base[1];
    for (int v = 0; v < w; ++v) {
      orr += wr[v];
      on += wn[v];
    }
    if (in) idxR[orr + pr] = t;
    if (out) idxN[on + pn] = t;
    if (t < T) {
      mkey[t] = ENC_NEG_INF;
      valid[t] = 0;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      int sr = 0, sn = 0;
      for (int v = 0; v < 16; ++v) {
        sr += wr[v];
        sn += wn[v];
      }
      base[0] += sr;
      base[1] += sn;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    cnt[0] = base[0];
    cnt[1] = base[1];
    if (count) *count = 0;
  }
}

// cascade step 2a: members whose maximum over earlier members is below the threshold
__global__ void gram_valid_kernel(const int* idxR, const int* cnt, const int* mkey, float thr,
                                  unsigned char* valid) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= cnt[0]) return;
  const int t = idxR[j];
  valid[t] = dec(mkey[t]) < thr;
}

// cascade step 3: the updated set
__global__ __launch_bounds__(256) void gram_final_kernel(const unsigned char* prev, const unsigned char* valid,
                                                          const int* mkey, float thr, float* max_cos,
                                                          unsigned char* rep, int* count, int T) {
  __shared__ int part[4];
  const int t = blockIdx.x * 256 + threadIdx.x;
  int r = 0;
  if (t < T) {
    const float m = dec(mkey[t]);
    r = prev[t] ? (int)valid[t] : (int)(m < thr);
    max_cos[t] = m;
    rep[t] = (unsigned char)r;
  }
  if (!count) return;
  const int wsum = __popcll(__ballot(r));
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = wsum;
  __syncthreads();
  if (threadIdx.x == 0) {
    const int c = part[0] + part[1] + part[2] + part[3];
    if (c) atomicAdd(count, c);
  }
}

// `slots` = B * tiles work units; with splits > 1 each is split along the
// features and finished by gram_reduce_kernel from the partials in `part`
template <class C>
void launch_gram_max(GramParams p, int slots, int splits, float* part, int bf16, hipStream_t s) {
  if (slots <= 0) return;
  if (splits > 1) {
    p.splits = splits;
    p.part = part;
    const dim3 grid((unsigned)(slots * splits));
    if (bf16) hipLaunchKernelGGL((gram_max_kernel<true, C, true>), grid, dim3(C::NT), 0, s, p);
    else hipLaunchKernelGGL((gram_max_kernel<false, C, true>), grid, dim3(C::NT), 0, s, p);
    const long long threads = (long long)slots * C::KT * C::QT / 4;
    hipLaunchKernelGGL((gram_reduce_kernel<C>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, p,
                       slots);
  } else {
    p.splits = 1;
    if (bf16) hipLaunchKernelGGL((gram_max_kernel<true, C, false>), dim3((unsigned)slots), dim3(C::NT), 0, s, p);
    else hipLaunchKernelGGL((gram_max_kernel<false, C, false>), dim3((unsigned)slots), dim3(C::NT), 0, s, p);
  }
}

void launch_norms(const void* x, float* inv, int rows, int d, int bf16, hipStream_t s, int* mkey = nullptr,
                  int* count = nullptr, int T = 1) {
  const dim3 grid((unsigned)((rows + 3) / 4));
  if (bf16) hipLaunchKernelGGL(gram_norm_kernel<true>, grid, dim3(256), 0, s, x, inv, rows, d, mkey, count, T);
  else hipLaunchKernelGGL(gram_norm_kernel<false>, grid, dim3(256), 0, s, x, inv, rows, d, mkey, count, T);
}

}  // namespace
}  // namespace ra

namespace {

using namespace ra;

constexpr size_t GALIGN = 256;
size_t gup(size_t x) { return (x + GALIGN - 1) / GALIGN * GALIGN; }

template <class C>
long long tri_tiles(int T) { return C::tri_before((T + C::QT - 1) / C::QT); }

// cross-product tiles for any split T = r + (T - r): at most
// ceil((T - r) / QT) query tiles times ceil(r / KT) key tiles
template <class C>
long long rect_tiles(int T) {
  long long best = 0;
  const long long nq = (T + C::QT - 1) / C::QT;
  for (long long a = 0; a <= nq; ++a) {  // a query tiles hold at least (a - 1) QT + 1 tokens
    const long long rest = T - ((a > 0 ? (a - 1) * C::QT + 1 : 0));
    const long long b = rest > 0 ? (rest + C::KT - 1) / C::KT : 0;
    if (a * b > best) best = a * b;
  }
  return best;
}

// compute units of the current device (cached per device; 256 when the
// runtime cannot say, e.g. with no device, which only sizes work splits)
int cu_count() {
  static int cached[64];
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (dev >= 0 && dev < 64 && cached[dev] > 0) return cached[dev];
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  if (dev >= 0 && dev < 64) cached[dev] = n;
  return n;
}

// Large tiles when their rounds of resident workgroups, each about 1.6 times
// as long as a round of small tiles (measured on long sequences), finish
// first; short sequences keep small tiles.
bool use_large_tiles(int B, int T) {
  const long long cus = cu_count();
  const long long small = (B * tri_tiles<SmallTiles>(T) + SmallTiles::WG_PER_CU * cus - 1) /
                          (SmallTiles::WG_PER_CU * cus);
  const long long large = (B * tri_tiles<LargeTiles>(T) + LargeTiles::WG_PER_CU * cus - 1) /
                          (LargeTiles::WG_PER_CU * cus);
  return 16 * large < 10 * small;
}

// Fewer tiles than resident workgroups (short sequences): split each tile's
// feature axis into up to (resident workgroups / tiles) ranges of at least
// four stages, so the chip fills; the partial products are summed in a fixed
// order afterwards.
template <class C>
int choose_splits(long long slots, int d) {
  const long long resident = (long long)C::WG_PER_CU * cu_count();
  if (slots <= 0 || slots >= resident) return 1;
  const long long s = std::min<long long>(std::min<long long>(resident / slots, (d / KC) / 4), MAX_SPLITS);
  return (int)std::max<long long>(1, s);
}

template <class C>
size_t part_bytes(long long slots, int d) {
  const int s = choose_splits<C>(slots, d);
  return s > 1 ? (size_t)slots * s * C::KT * C::QT * sizeof(float) : 0;
}

int check_tokens(int B, int T, int d) {
  if (B < 1 || T < 1 || d < 64 || d > 65536 || d % 64) return ROPE_ATTN_ERR_SHAPE;
  if (T > (1 << 20) || (long long)T * d > (1LL << 31) || (long long)B * T > (1LL << 31))
    return ROPE_ATTN_ERR_SHAPE;
  if ((long long)B * tri_tiles<SmallTiles>(T) > INT_MAX) return ROPE_ATTN_ERR_SHAPE;
  return ROPE_ATTN_OK;
}

bool mis16(const void* q) { return ((uintptr_t)q & 15u) != 0; }
bool mis4(const void* q) { return ((uintptr_t)q & 3u) != 0; }

float gram_threshold(float tau) { return (float)(1.0 - (double)tau * (double)tau); }

size_t select_part_bytes(int B, int T, int d) {
  return use_large_tiles(B, T) ? part_bytes<LargeTiles>(B * tri_tiles<LargeTiles>(T), d)
                               : part_bytes<SmallTiles>(B * tri_tiles<SmallTiles>(T), d);
}

size_t select_bytes(int B, int T, int d) {
  const size_t n = (size_t)B * T;
  // inverse norms, running maxima, split partial products
  return gup(4 * n) + gup(4 * n) + gup(select_part_bytes(B, T, d));
}

size_t cascade_part_bytes(int T, int d) {
  return std::max(part_bytes<SmallTiles>(tri_tiles<SmallTiles>(T), d),
                  part_bytes<SmallTiles>(rect_tiles<SmallTiles>(T), d));
}

size_t cascade_bytes(int T, int d) {
  const size_t n = (size_t)T;
  return gup(4 * n) + gup(4 * n) + gup(4 * n) + gup(4 * n) + gup(2 * 4) + gup(n) +
         gup(cascade_part_bytes(T, d));
}

int gram_finish() { return hipGetLastError() == hipSuccess ? ROPE_ATTN_OK : ROPE_ATTN_ERR_HIP; }

}  // namespace

extern "C" {

size_t gram_select_workspace_bytes(int B, int T, int d) {
  if (check_tokens(B, T, d)) return 0;
  return select_bytes(B, T, d);
}

size_t gram_cascade_workspace_bytes(int T, int d) {
  if (check_tokens(1, T, d)) return 0;
  return cascade_bytes(T, d);
}

int gram_select(const void* x, int B, int T, int d, int dtype, float tau, float* max_cos,
                unsigned char* rep, int* count, void* workspace, size_t workspace_bytes, void* stream) {
  return gram_select_stages(GRAM_STAGE_ALL, x, B, T, d, dtype, tau, max_cos, rep, count, workspace,
                            workspace_bytes, stream);
}

int gram_select_stages(unsigned stages, const void* x, int B, int T, int d, int dtype, float tau,
                       float* max_cos, unsigned char* rep, int* count, void* workspace,
                       size_t workspace_bytes, void* stream) {
  if (!x || !max_cos || !rep || !workspace) return ROPE_ATTN_ERR_NULL;
  if (dtype != GRAM_BF16 && dtype != GRAM_FP16) return ROPE_ATTN_ERR_DTYPE;
  int st = check_tokens(B, T, d);
  if (st) return st;
  if (!(isfinite(tau) && tau >= 0.0f)) return ROPE_ATTN_ERR_ARG;
  if (mis16(x) || mis4(max_cos) || mis4(count) || ((uintptr_t)workspace & (GALIGN - 1)))
    return ROPE_ATTN_ERR_ALIGN;
  if (workspace_bytes < select_bytes(B, T, d)) return ROPE_ATTN_ERR_WORKSPACE;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  const size_t n = (size_t)B * T;
  char* ws = reinterpret_cast<char*>(workspace);
  float* inv = reinterpret_cast<float*>(ws);
  int* mkey = reinterpret_cast<int*>(ws + gup(4 * n));
  float* part = reinterpret_cast<float*>(ws + 2 * gup(4 * n));
  const int bf16 = dtype == GRAM_BF16;

  if (stages & GRAM_STAGE_PREP) {
    launch_norms(x, inv, (int)n, d, bf16, hs, mkey, count, T);
  }
  if (stages & GRAM_STAGE_GRAM) {
    GramParams p = {};
    p.x = x; p.inv = inv; p.mkey = mkey; p.B = B; p.T = T; p.d = d; p.tri = 1;
    p.contiguous = 1;
    p.sub_first = -1;
    if (use_large_tiles(B, T)) {
      // whole rounds of resident large tiles; the large tiles left over for a
      // last, mostly idle round run as four small tiles each instead
      p.tiles = (int)tri_tiles<LargeTiles>(T);
      const int slots = B * p.tiles;
      const int resident = LargeTiles::WG_PER_CU * cu_count();
      int full = slots / resident * resident;
      // quarters of the leftover tiles fill at most one round of small tiles
      if (full == 0 || 2 * (slots - full) > resident) full = slots;
      launch_gram_max<LargeTiles>(p, full, 1, part, bf16, hs);
      if (full < slots) {
        GramParams q = p;
        q.sub_first = full;
        q.sub_tiles = p.tiles;
        q.contiguous = 0;
        launch_gram_max<SmallTiles>(q, 4 * (slots - full), 1, part, bf16, hs);
      }
    } else {
      p.tiles = (int)tri_tiles<SmallTiles>(T);
      const int slots = B * p.tiles;
      launch_gram_max<SmallTiles>(p, slots, choose_splits<SmallTiles>(slots, d), part, bf16, hs);
    }
  }
  if (stages & GRAM_STAGE_DECIDE)
    hipLaunchKernelGGL(gram_flags_kernel, dim3((unsigned)((T + 255) / 256), (unsigned)B), dim3(256), 0,
                       hs, mkey, gram_threshold(tau), max_cos, rep, count, T);
  return gram_finish();
}

int gram_cascade(const void* x, int T, int d, int dtype, float tau, const unsigned char* prev,
                 float* max_cos, unsigned char* rep, int* count, void* workspace, size_t workspace_bytes,
                 void* stream) {
  if (!x || !prev || !max_cos || !rep || !workspace) return ROPE_ATTN_ERR_NULL;
  if (dtype != GRAM_BF16 && dtype != GRAM_FP16) return ROPE_ATTN_ERR_DTYPE;
  int st = check_tokens(1, T, d);
  if (st) return st;
  if (!(isfinite(tau) && tau >= 0.0f)) return ROPE_ATTN_ERR_ARG;
  if (mis16(x) || mis4(max_cos) || mis4(count) || ((uintptr_t)workspace & (GALIGN - 1)))
    return ROPE_ATTN_ERR_ALIGN;
  if (workspace_bytes < cascade_bytes(T, d)) return ROPE_ATTN_ERR_WORKSPACE;
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  const size_t n = (size_t)T;
  char* ws = reinterpret_cast<char*>(workspace);
  float* inv = reinterpret_cast<float*>(ws);
  int* mkey = reinterpret_cast<int*>(ws + gup(4 * n));
  int* idxR = reinterpret_cast<int*>(ws + 2 * gup(4 * n));
  int* idxN = reinterpret_cast<int*>(ws + 3 * gup(4 * n));
  int* cnt = reinterpret_cast<int*>(ws + 4 * gup(4 * n));
  unsigned char* valid = reinterpret_cast<unsigned char*>(ws + 4 * gup(4 * n) + gup(8));
  float* part = reinterpret_cast<float*>(ws + 4 * gup(4 * n) + gup(8) + gup(n));
  const int bf16 = dtype == GRAM_BF16;
  const float thr = gram_threshold(tau);

  hipLaunchKernelGGL(gram_compact_kernel, dim3(1), dim3(1024), 0, hs, prev, T, idxR, idxN, cnt, mkey, valid,
                     count);
  launch_norms(x, inv, T, d, bf16, hs);
  GramParams p = {};
  p.x = x; p.inv = inv; p.mkey = mkey; p.B = 1; p.T = T; p.d = d;
  p.sub_first = -1;
  // the r x r product among the inherited members
  p.qidx = p.kidx = idxR;
  p.qn = p.kn = cnt;
  p.tri = 1;
  p.tiles = (int)tri_tiles<SmallTiles>(T);
  launch_gram_max<SmallTiles>(p, p.tiles, choose_splits<SmallTiles>(p.tiles, d), part, bf16, hs);
  hipLaunchKernelGGL(gram_valid_kernel, dim3((unsigned)((T + 255) / 256)), dim3(256), 0, hs, idxR, cnt, mkey,
                     thr, valid);
  // the (T - r) x r product between the other tokens and the valid members
  p.qidx = idxN;
  p.qn = cnt + 1;
  p.kvalid = valid;
  p.tri = 0;
  p.tiles = (int)rect_tiles<SmallTiles>(T);
  launch_gram_max<SmallTiles>(p, p.tiles, choose_splits<SmallTiles>(p.tiles, d), part, bf16, hs);
  hipLaunchKernelGGL(gram_final_kernel, dim3((unsigned)((T + 255) / 256)), dim3(256), 0, hs, prev, valid,
                     mkey, thr, max_cos, rep, count, T);
  return gram_finish();
}

}  // extern "C"
