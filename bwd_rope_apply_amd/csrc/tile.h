// Device building blocks shared by the MFMA kernels (gfx950, wave64):
// fragment layouts, LDS tile layout, score products, transposed reads,
// epilogues.
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
#pragma once

#include <type_traits>

#include "common.h"

namespace ra {
namespace {

constexpr int BN = 64;     // rows of a streamed tile per loop step (default)
constexpr int BM = 128;    // stationary rows per workgroup (4 waves x 32)

__device__ __forceinline__ int perm(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// LDS tile layout ([BN][D + 8] fp16): logical row L (bits b5..b0) is stored
// at physical row sig(L) = (b5 b4 b2 | b1 b0 b3).  With the 16-byte row pad
// (4 banks), the natural fragment reads (8 lanes on rows perm(l32)) and the
// transposed reads (16 lanes on 4 rows x 32 bytes) both touch 32 distinct
// banks, and every read of a lane is one base address plus immediates.
__device__ __forceinline__ int sig(int L) {
  return (L & 48) | ((L & 4) << 1) | ((L & 3) << 1) | ((L >> 3) & 1);
}

__device__ __forceinline__ f32x16 mfma(half8 a, half8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Block index -> (head, tile).  Workgroups are dispatched round-robin over
// the 8 XCDs; when the head count allows, each XCD gets a fixed set of heads
// so that their K/V (or Q/dO) tiles stay in that XCD's L2.  Tiles are issued
// heaviest first (most causal work).  An XCD with more than `group` heads
// works through them `group` at a time (heaviest first within each group),
// so that fewer heads' streamed tiles compete for its L2 at once (measured
// at 4 x 32 x 4096 with groups of 4: dK/dV -2.5%, dQ from panels -5.6%
// against all 16 heads interleaved; groups of 2 made the forward and the
// dQ product slower at 1 x 32 x 8192 and left dK/dV unchanged).
__host__ __device__ __forceinline__ void map_block(int idx, int BH, int ntiles, bool heavy_high,
                                                   int& bh, int& t, int group = 4) {
  int k;
  if ((BH & 7) == 0) {
    const int hpx = BH >> 3;
    const int x = idx & 7, s = idx >> 3;
    if (hpx > group && hpx % group == 0) {
      const int per = group * ntiles, grp = s / per, within = s % per;
      bh = x * hpx + grp * group + within % group;
      k = within / group;
    } else {
      bh = x * hpx + s % hpx;
      k = s / hpx;
    }
  } else {
    bh = idx % BH;
    k = idx / BH;
  }
  t = heavy_high ? ntiles - 1 - k : k;
}

// Register copy of one streamed [BN][D] fp16 tile: every thread holds NCH
// 16-byte chunks (row = chunk / (D/8)).  Rows at or past N are clamped to
// N - 1: they are masked downstream, so they only need to be finite.
template <int D, int ROWS = BN>
struct TileRegs {
  static constexpr int CPR = D / 8;
  static constexpr int NCH = ROWS * CPR / 256;
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
      *reinterpret_cast<half8*>(dst + sig(ch / CPR) * (D + 8) + (ch % CPR) * 8) = x[i];
    }
  }
};

__device__ __forceinline__ int sig_inv(int P) {
  return (P & 48) | ((P & 1) << 3) | ((P >> 1) & 7);
}

// Direct global -> LDS copy of one streamed [ROWS][D] fp16 tile into the
// sig() layout, without passing through registers (global_load_lds_dwordx4:
// each wave instruction writes 1 KiB of LDS, lane i at byte 16 i).  A tile
// buffer is a whole number of 1 KiB blocks (ALLOC halfs), block b issued by
// wave b % 4; a lane whose 16-byte slot falls in a row pad or past the tile
// loads a dummy chunk (row 0), so every lane of an issued block loads and no
// per-lane branch is needed.  Each lane's byte offset from the tile's first
// row is computed once; a step adds the tile's row base in scalar registers.
// Rows past the head's last row are read as they are (the next head's rows
// or the plane's zero pad, see PLANE_PAD_ROWS); the tiles' consumers mask
// them.  Callers wait for the copies (wait_lds_copies) before the barrier
// that publishes the tile.
// One lane-wise 16-byte (or 4-byte) global -> LDS copy: lane i writes LDS
// bytes [lds + size i, lds + size (i + 1)) from gbase + voff (gbase and lds
// uniform).  It is the same global_load_lds instruction the compiler's
// builtin emits, written out so that the compiler does not treat it as a
// pending LDS write: otherwise it waits for every copy in flight (the next
// tile's included) before each LDS read of the current tile, which leaves
// the double buffer nothing to overlap.  Callers wait for the copies
// explicitly (wait_lds_copies) before the barrier that publishes a tile.
// M0 carries the LDS address; the s_nop covers the wait states between the
// scalar writes of M0 / the base and the copy's reads of them.
__device__ __forceinline__ void lds_copy16(const void* gbase, uint32_t voff, const void* lds) {
  const uint32_t m0v = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds;
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 4\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(gbase), "s"(m0v)
      : "memory", "m0");
}
// The same copy with the non-temporal hint, for data read once (streamed
// past the caches rather than kept in them).
__device__ __forceinline__ void lds_copy16_nt(const void* gbase, uint32_t voff, const void* lds) {
  const uint32_t m0v = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds;
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 4\n\t"
      "global_load_lds_dwordx4 %0, %1 nt"
      :
      : "v"(voff), "s"(gbase), "s"(m0v)
      : "memory", "m0");
}
__device__ __forceinline__ void lds_copy4(const void* gbase, uint32_t voff, const void* lds) {
  const uint32_t m0v = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)lds;
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 4\n\t"
      "global_load_lds_dword %0, %1"
      :
      : "v"(voff), "s"(gbase), "s"(m0v)
      : "memory", "m0");
}

template <int D, int ROWS>
struct TileDMA {
  static_assert(ROWS <= PLANE_PAD_ROWS, "a tile starting below N must end inside the padded plane");
  static constexpr int RB = (D + 8) * 2;                 // bytes per physical row
  static constexpr int BYTES = ROWS * RB;
  static constexpr int NBLK = (BYTES + 1023) / 1024;
  static constexpr int PER_WAVE = (NBLK + 3) / 4;
  static constexpr int ALLOC = NBLK * 512;               // halfs per tile buffer
  uint32_t off[PER_WAVE];   // byte offset of this lane's chunk from row r0 (row * 2D + col)
  int wave;                 // wave index (uniform)
  __device__ __forceinline__ void init(int lane, int w) {
    wave = __builtin_amdgcn_readfirstlane(w);
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int o = (w + 4 * i) * 1024 + 16 * lane;
      const int pr = o / RB, within = o % RB;
      const bool real = o < BYTES && within < 2 * D;
      off[i] = real ? (uint32_t)(sig_inv(pr) * D * 2 + within) : 0u;
    }
  }
  // block wave + 4 i exists for every wave in the full rounds i < NBLK / 4
  __device__ __forceinline__ bool issued(int i) const { return i < NBLK / 4 || wave + 4 * i < NBLK; }
  // copy instructions this wave issues per load (uniform)
  __device__ __forceinline__ int count() const { return NBLK / 4 + (wave < NBLK % 4 ? 1 : 0); }
  // src is the head's rows in a padded plane and r0 < N, so the tile ends
  // inside the plane.  Byte offsets from src fit 32 bits (r0 is a multiple
  // of ROWS below N <= 2^24, and 2 D <= 256),
  // so the address is a scalar base plus one zero-extended 32-bit lane
  // offset: the scalar-base form.
  __device__ __forceinline__ void load(half_t* tile, const half_t* src, int r0) const {
    const char* base = reinterpret_cast<const char*>(src);
    const uint32_t rb = (uint32_t)r0 * (uint32_t)(2 * D);
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      if (issued(i)) lds_copy16(base, rb + off[i], tile + (wave + 4 * i) * 512);
    }
  }
};

// Row offsets of the steps of a tile walk: dense (base + i STEP) or over a
// block list in LDS (list[i / SPB] BLK + (i % SPB) STEP).  In block-list
// mode the entry of step i + 2 is read from LDS during step i and made a
// scalar after the step's closing wait, so no step stalls on an LDS read
// before issuing its copies.
template <int STEP, bool BL>
struct Walk {
  static constexpr int SPB = BLK / STEP;
  const short* list;
  int base, n;
  int cur, next, raw;
  __device__ __forceinline__ int at(int i) const {
    if constexpr (BL) return __builtin_amdgcn_readfirstlane(list[i / SPB]) * BLK + (i % SPB) * STEP;
    else return base + i * STEP;
  }
  __device__ __forceinline__ void init(const short* l, int b, int count) {
    list = l; base = b; n = count; raw = 0;
    cur = count > 0 ? at(0) : 0;
    next = count > 1 ? at(1) : 0;
  }
  // during step i (i < n)
  __device__ __forceinline__ void prefetch(int i) {
    if constexpr (BL) raw = list[min(i + 2, n - 1) / SPB];
  }
  // after step i's closing wait
  __device__ __forceinline__ void advance(int i) {
    cur = next;
    if constexpr (BL) next = __builtin_amdgcn_readfirstlane(raw) * BLK + ((i + 2) % SPB) * STEP;
    else next = base + (i + 2) * STEP;
  }
};

// Block lists for block-list attention.  One wave lists the set bits of a
// visibility row [ceil(nb / 32) words] in ascending order, 64 candidate
// blocks per ballot; the count is returned to every lane.
__device__ __forceinline__ int row_blocks(const uint32_t* row, int nb, short* list, int lane) {
  int n = 0;
  for (int b0 = 0; b0 < nb; b0 += 64) {
    const int b = b0 + lane;
    const bool bit = b < nb && ((row[b >> 5] >> (b & 31)) & 1u);
    const unsigned long long m = __ballot(bit);
    const int before = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    if (bit) list[n + before] = (short)b;
    n += __popcll(m);
  }
  return n;
}

// Query blocks qb >= qb0 whose visibility row has bit kb, ascending, for a
// workgroup of NT threads: each thread tests some rows, wave ballots land in
// `col` (MAX_BLOCKS / 32 words of LDS), then wave 0 lists the set bits.
// Every thread calls it; the count is returned to all.
template <int NT>
__device__ __forceinline__ int column_blocks(const uint32_t* bm, int nb, int W, int bh, int kb,
                                             int qb0, uint32_t* col, short* list, int* count) {
  for (int base = 0; base < nb; base += NT) {
    const int qb = base + (int)threadIdx.x;
    bool bit = false;
    if (qb < nb && qb >= qb0)
      bit = (bm[((size_t)bh * nb + qb) * W + (kb >> 5)] >> (kb & 31)) & 1u;
    const unsigned long long b = __ballot(bit);
    if ((threadIdx.x & 63) == 0 && base + (int)threadIdx.x < MAX_BLOCKS) {
      const int w0 = (base + (int)threadIdx.x) >> 5;
      col[w0] = (uint32_t)b;
      if (w0 + 1 < MAX_BLOCKS / 32) col[w0 + 1] = (uint32_t)(b >> 32);
    }
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    const int c = row_blocks(col, nb, list, (int)threadIdx.x);
    if (threadIdx.x == 0) *count = c;
  }
  __syncthreads();
  return *count;
}

__device__ __forceinline__ void wait_lds_copies() { __builtin_amdgcn_s_waitcnt(0); }

// Wait until at most N (0..63) vector memory operations of this wave are
// outstanding, ignoring the other counters.  On gfx9 loads, stores and
// global -> LDS copies share this counter and retire from it in issue
// order, so everything older than the N most recent has completed.
template <int N>
__device__ __forceinline__ void wait_vm_const() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// The lane index, computed where it is used (two VALU instructions that the
// compiler cannot hoist): under register pressure this is cheaper than
// keeping it live across a loop, which the compiler may do by spilling it.
__device__ __forceinline__ uint32_t lane_here() {
  uint32_t x;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(x));
  return x;
}

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

// Two 32-key score blocks (keys along m, this lane's query along n), the
// accumulators seeded with `seed` (a per-query offset folded into the product).
template <int D, int NMB = 2>
__device__ __forceinline__ void scores(f32x16* s, const half_t* lds, const half8* bf, int l32,
                                       int g, float seed = 0.f) {
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) {
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = seed;
    const half_t* row = lds + sig(32 * mb + perm(l32)) * (D + 8) + 8 * g;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) acc = mfma(*reinterpret_cast<const half8*>(row + 16 * t), bf[t], acc);
    s[mb] = acc;
  }
}

// s[mb] += the same products (for split-operand sums).
template <int D, int NMB = 2>
__device__ __forceinline__ void scores_add(f32x16* s, const half_t* lds, const half8* bf, int l32,
                                           int g) {
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) {
    const half_t* row = lds + sig(32 * mb + perm(l32)) * (D + 8) + 8 * g;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) s[mb] = mfma(*reinterpret_cast<const half8*>(row + 16 * t), bf[t], s[mb]);
  }
}

// Split-fp16 fragments: hi = fp16(x), lo = fp16(x - hi).
template <int NMB = 2>
__device__ __forceinline__ void to_frags_split(const f32x16* s, half8* hi, half8* lo) {
#pragma unroll
  for (int t = 0; t < 2 * NMB; ++t) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = s[t >> 1][8 * (t & 1) + e];
      const half_t h = (half_t)x;
      hi[t][e] = h;
      lo[t][e] = (half_t)(x - (float)h);
    }
  }
}

// Pack register values of NMB score blocks into the 2 NMB 16-key B-operand
// fragments (k step t holds keys 16t + 8g + e).
template <int NMB = 2>
__device__ __forceinline__ void to_frags(const f32x16* s, half8* f) {
#pragma unroll
  for (int t = 0; t < 2 * NMB; ++t) {
#pragma unroll
    for (int e = 0; e < 8; ++e) f[t][e] = (half_t)s[t >> 1][8 * (t & 1) + e];
  }
}

typedef __attribute__((ext_vector_type(4))) short s16x4;

__device__ __forceinline__ s16x4 ds_read_tr(const half_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}

// Two transposed reads, at p and p + HI halfs, as one 8-value fragment.
template <int HI>
__device__ __forceinline__ half8 tr_pair(const half_t* p) {
  const s16x4 lo = ds_read_tr(p), hi = ds_read_tr(p + HI);
  typedef __attribute__((ext_vector_type(8))) short s16x8;
  const s16x8 both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(half8, both);
}

// This lane's part of the address of tr_frag's reads (halfs from the tile):
// the rest, 16 t (D + 8) + 32 cb, is the same for every lane.
template <int D>
__device__ __forceinline__ int tr_lane_offset(int lane) {
  const int s16 = lane & 15, g = lane >> 5, b = (lane >> 4) & 1;
  return sig(8 * g + (s16 >> 2)) * (D + 8) + 16 * b + 4 * (s16 & 3);
}

// A-operand fragment of X^T for k step t and column block cb, X a [BN][D]
// tile in LDS (two transposed reads).
template <int D>
__device__ __forceinline__ half8 tr_frag(const half_t* lds, int t, int cb, int lane) {
  // logical rows 16t + 8g + 4h + e, e = s16 >> 2 (h = 0, 1), columns
  // 32cb + 16 b + 4 (s16 & 3): physical row 16t + 8h + sig(8g + e)
  constexpr int LD = D + 8;
  return tr_pair<8 * LD>(lds + tr_lane_offset<D>(lane) + 16 * t * LD + 32 * cb);
}

// acc[cb] += X^T(columns 32cb.., rows = 16-wide k steps) * frag, with X a
// [BN][D + 8] tile in LDS.  ds_read_b64_tr_b16 transposes a 4 x 16 block per
// 16-lane group (lane j receives element j of the 4 rows that lanes
// 4e + j/4 point at), so lane s of a group points at row s/4, columns
// 4 (s % 4) .. +3 of its block, and two reads give the 8 k-values (rows
// 16t + 8g + 0..7) of column 32cb + l32.
template <int D, int NT = 4>
__device__ __forceinline__ void accumulate_tr(f32x16* acc, const half_t* lds, const half8* f, int lane) {
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb) {
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[cb] = mfma(tr_frag<D>(lds, t, cb, lane), f[t], acc[cb]);
  }
}

// Position-weighted wedge partial of one row's gradient (already in the
// un-rotated frame) summed over the NW waves of the workgroup into one
// [D/2] slot (red holds NW x D/2 floats).  w[cb*8 + rq*2 + h] is pair
// m = 16cb + 4rq + 2g + h.
template <int D, int NW = 4>
__device__ __forceinline__ void store_dalpha(float* w, float* red, float* slot, int g) {
  constexpr int NP = D / 4;   // wedge partials per lane
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < NP; ++i) {
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
  for (int m = threadIdx.x; m < D / 2; m += 64 * NW) {
    float x = (red[m] + red[D / 2 + m]) + (red[D + m] + red[3 * D / 2 + m]);
#pragma unroll
    for (int v = 4; v < NW; v += 4)
      x += (red[v * (D / 2) + m] + red[(v + 1) * (D / 2) + m]) +
           (red[(v + 2) * (D / 2) + m] + red[(v + 3) * (D / 2) + m]);
    slot[m] = x;
  }
}

// Un-rotate one lane's gradient registers (row `row`, columns
// 32cb + 8rq + 4g + 0..3), add the wedge partials and store float4s (ADD:
// add them to what `out` holds, a gradient another pass already wrote; the
// wedge partials are those of this contribution alone).
template <int D, bool ADD = false>
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
      if constexpr (ADD) {
        const float4 o = *reinterpret_cast<const float4*>(out + c);
        v[0] += o.x; v[1] += o.y; v[2] += o.z; v[3] += o.w;
      }
      *reinterpret_cast<float4*>(out + c) = make_float4(v[0], v[1], v[2], v[3]);
    }
  }
}

}  // namespace
}  // namespace ra
