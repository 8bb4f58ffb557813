// MFMA kernels for exact RoPE attention on gfx950: forward, dQ and dK/dV.
//
// Operands are the fp16 planes written by the prep pass (Q~, K~ rotated,
// V, dO converted); products accumulate in fp32 with
// v_mfma_f32_32x32x16_f16.  fp16 rather than bf16 operands: the two run at
// the same MFMA rate on gfx950, and the 3 extra mantissa bits are what keeps
// the error of P, dS, Q~ and K~ rounding within 2e-2 of each output's RMS.
//
// Fragment conventions and the LDS tile layout are described in tile.h.
//
// What each product computes ("RoPE attention can be trained in
// almost-linear time", Methodology 1 and 2): the normalised softmax s(x),
// the weighted sum with V, beta = dO V^T, gamma = diag(s) beta - s s^T beta
// = P o (dP - D), and the gradient back through the scores.
#include "corner.h"

namespace ra {

namespace {

// Tiling (the measured best on MI355X):
//   *_WPS   waves per SIMD the register budget is sized for (more waves
//           let one wave's softmax VALU work overlap another's MFMAs; the
//           512 VGPRs of a SIMD lane are shared among them)
//   *_BN    rows of the streamed operand per product (multiple of 32)
//   FWD_NB  32-row query blocks per forward wave
//   FWD_MB  32-key blocks per forward step (1: 32-key tiles, whose smaller
//           registers and LDS allow 3 waves per SIMD)
//   DQ_SUB  DQ_BN-key products per copied tile in the recomputing dQ
//           (one barrier per tile)
constexpr int FWD_NB = 1;
constexpr int FWD_WPS = 3;
constexpr int FWD_MB = 1;
constexpr int DQ_BN = 32;
constexpr int DQ_SUB = 2;
constexpr int DQ_WPS = 2;
constexpr int DKDV_BN = 32;
constexpr int DKDV_WPS = 2;

// One step of the forward (MB blocks of 32 keys) for one wave owning NB
// blocks of 32 query rows: scores, online softmax, O += P V.  Every K~ and
// V fragment read from LDS feeds NB products.  Q~ carries the factor
// log2(e)/sqrt(D), so scores are in log2 units.  m is the reference
// maximum the running sum l and O are relative to.  The common step takes
// P = exp2(S - m) with the reference as it stands and checks the sum of
// each lane's fp16 P: at most LAZY_LIMIT (2^15) bounds every P, so all fit
// fp16 and nothing else is needed (O and l share the reference, so any
// reference is exact in the arithmetic; a P past fp16's range makes the sum
// +inf).  A step that fails the check (a row's first
// step, m = -inf, or a score far above the reference) recomputes its
// scores and moves the reference to the row maximum, rescaling O and l.
// MASK hides keys after klim[nb] (causal diagonal, ragged tail).
constexpr float LAZY_LIMIT = 32768.f;   // 2^15: every P <= this fits fp16

// seed: the accumulators' starting values per row block (null: zero)
template <int D, int NB, int MB>
__device__ __forceinline__ void fwd_scores(f32x16 (*s)[MB], const half_t* Ks,
                                           const half8 (*qf)[D / 16], int l32, int g,
                                           const f32x16* seed = nullptr) {
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) s[nb][mb] = seed ? seed[nb] : f32x16{};
    const half_t* row = Ks + sig(32 * mb + perm(l32)) * (D + 8) + 8 * g;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      const half8 a = *reinterpret_cast<const half8*>(row + 16 * t);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) s[nb][mb] = mfma(a, qf[nb][t], s[nb][mb]);
    }
  }
}

// negm: at D = 64 (SEEDED), -m of each row in all 16 registers of a block,
// the score products' starting value, so that they come out as S - m; at
// D = 128 the registers are short (three waves per SIMD), and the step
// subtracts m from the scores instead.
template <int D, int NB, bool MASK, int MB = 2>
__device__ __forceinline__ void fwd_tile(f32x16 (*o)[D / 32], float* m, float* l, f32x16* negm,
                                         const half_t* Ks, const half_t* Vs,
                                         const half8 (*qf)[D / 16], int k0, const int* klim,
                                         int lane) {
  constexpr bool SEEDED = D == 64;
  const int l32 = lane & 31, g = lane >> 5;
  // the scheduler's LDS-read / MFMA interleaving strategy: more fragment
  // reads stay ahead of the products
  __builtin_amdgcn_iglp_opt(0);
  f32x16 s[NB][MB];
  fwd_scores<D, NB, MB>(s, Ks, qf, l32, g, SEEDED ? negm : nullptr);
  // scores minus the reference, masked keys at -inf
  auto relative = [&](int nb, float ref) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = s[nb][mb][r] - ref;
        if (MASK) {
          const int key = k0 + 32 * mb + 16 * (r >> 3) + 8 * g + (r & 7);
          x = key > klim[nb] ? -INFINITY : x;
        }
        s[nb][mb][r] = x;
      }
    }
  };
  auto exps = [&](int nb) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[nb][mb][r] = exp2_fast(s[nb][mb][r]);
    }
  };
  // the step's fp16 weights, and their sum in fp32 (two interleaved chains of
  // v_dot2 against (1, 1)): a weight past fp16's range makes the sum +inf
  half8 pf[NB][2 * MB];
  auto weights = [&](int nb) {
    to_frags<MB>(s[nb], pf[nb]);
    float a = 0.f, b = 0.f;
#pragma unroll
    for (int t = 0; t < 2 * MB; ++t) {
#pragma unroll
      for (int e = 0; e < 8; e += 4) {
        a = __builtin_amdgcn_fdot2(half2v{pf[nb][t][e], pf[nb][t][e + 1]}, half2v{1.0f16, 1.0f16}, a,
                                   false);
        b = __builtin_amdgcn_fdot2(half2v{pf[nb][t][e + 2], pf[nb][t][e + 3]},
                                   half2v{1.0f16, 1.0f16}, b, false);
      }
    }
    return a + b;
  };
  float ls[NB];
  bool exact = false;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    if (!SEEDED || MASK) relative(nb, SEEDED ? 0.f : m[nb]);   // seeded: the mask only
    exps(nb);
    ls[nb] = weights(nb);
    // NaN (m = -inf) and +inf (a weight past fp16) fail the test too
    exact |= m[nb] == -INFINITY || !(ls[nb] <= LAZY_LIMIT);
  }
  if (__any(exact)) {  // rare: the scores again, and the reference to the row maximum
    // seeded: the fragments are read again rather than kept live through the
    // exps, which leaves the registers the seed blocks take
    if constexpr (SEEDED) asm volatile("" ::: "memory");
    fwd_scores<D, NB, MB>(s, Ks, qf, l32, g);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      relative(nb, 0.f);
      float mx = -INFINITY;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[nb][mb][r]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      // a row with no visible key yet keeps m = -inf (its P are 0)
      const float mn = fmaxf(m[nb], mx);
      const float alpha = m[nb] == -INFINITY ? 0.f : exp2_fast(m[nb] - mn);
      l[nb] *= alpha;
#pragma unroll
      for (int cb = 0; cb < D / 32; ++cb) o[nb][cb] *= alpha;
      m[nb] = mn;
      if constexpr (SEEDED) {
#pragma unroll
        for (int r = 0; r < 16; ++r) negm[nb][r] = -mn;
      }
      const float ref = mn == -INFINITY ? 0.f : mn;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[nb][mb][r] -= ref;
      }
      exps(nb);
      ls[nb] = weights(nb);
    }
  }
  // l sums the fp16 weights that the PV product uses: it is O's normaliser
  // (a row whose weight sits on one key then keeps that key's value, the
  // weight's rounding cancelling) and the LSE's sum
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) l[nb] += ls[nb];
  // O^T[c][q] += V^T[c][key] P^T[key][q]: V^T fragments by transposed reads
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb) {
#pragma unroll
    for (int t = 0; t < 2 * MB; ++t) {
      const half8 a = tr_frag<D>(Vs, t, cb, lane);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) o[nb][cb] = mfma(a, pf[nb][t], o[nb][cb]);
    }
  }
}

// One step of dQ for one wave over 32 NMB keys: P = exp2(S' - LSE2) with
// the LSE seeded into the score accumulators, dP - D with D seeded into the
// dP accumulators (dP = dO V^T), dS = P o (dP - D), dQ~ += dS K~.
template <int D, int NMB, bool MASK>
__device__ __forceinline__ void dq_tile(f32x16* acc, const half_t* Ks, const half_t* Vs,
                                        const half8* qf, const half8* df, int k0, int klim,
                                        float lse2, float dr, int lane) {
  const int l32 = lane & 31, g = lane >> 5;
  f32x16 s[NMB], dp[NMB];
  scores<D, NMB>(s, Ks, qf, l32, g, -lse2);
  // P first: it needs only the scores, so its exps can issue between the
  // dP products
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float pr = exp2_fast(s[mb][r]);
      if (MASK) {
        const int key = k0 + 32 * mb + 16 * (r >> 3) + 8 * g + (r & 7);
        pr = key > klim ? 0.f : pr;
      }
      s[mb][r] = pr;
    }
  }
  scores<D, NMB>(dp, Vs, df, l32, g, -dr);
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s[mb][r] *= dp[mb][r];
  }
  half8 sf[2 * NMB];
  to_frags<NMB>(s, sf);
  accumulate_tr<D, 2 * NMB>(acc, Ks, sf, lane);
}

// One step of dK, dV for one wave over 32 NMB queries (this lane's key
// along n): P = exp(S - LSE), dV += P^T dO, dP = dO V^T, dS = P o (dP - D),
// dK~ += dS^T Q~.  MASK hides queries before this lane's key.  rsc holds
// the step's row scalars, 32-row groups of [-LSE * log2(e) | -D]: they seed
// the score and dP accumulators (each accumulator row is one query), so
// the products come out as S - LSE and dP - D.  vrow points at this lane's
// V row in the stationary LDS tile.  DS also hands out the fp16 dS row of
// this lane's key (its 32 NMB queries, 8 per 16-byte chunk) in ds_out,
// zeros for a key at or past N.
template <int D, int NMB, bool MASK, bool DS = false>
__device__ __forceinline__ void dkdv_tile(f32x16* dk, f32x16* dv, const half_t* Qs,
                                          const half_t* Ds, const float* rsc, const half8* kf,
                                          const half_t* vrow, int r0, int key, int lane,
                                          half8* ds_out = nullptr, bool key_ok = true) {
  const int l32 = lane & 31, g = lane >> 5;
  // the scheduler's LDS-read / MFMA interleaving strategy: about 8 fragment
  // reads stay ahead of the products instead of 1-2
  __builtin_amdgcn_iglp_opt(0);
  f32x16 s[NMB], dp[NMB];
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float* lr = rsc + 64 * mb + 16 * h + 8 * g;
      const float4 la = *reinterpret_cast<const float4*>(lr);
      const float4 lb = *reinterpret_cast<const float4*>(lr + 4);
      const float4 da = *reinterpret_cast<const float4*>(lr + 32);
      const float4 db = *reinterpret_cast<const float4*>(lr + 36);
      const float lv8[8] = {la.x, la.y, la.z, la.w, lb.x, lb.y, lb.z, lb.w};
      const float dv8[8] = {da.x, da.y, da.z, da.w, db.x, db.y, db.z, db.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        s[mb][8 * h + e] = lv8[e];
        dp[mb][8 * h + e] = dv8[e];
      }
    }
  }
  scores_add<D, NMB>(s, Qs, kf, l32, g);   // queries along m, this lane's key along n
  // P first: it needs only the scores, so its exps can issue between the
  // dP products below
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float pr = exp2_fast(s[mb][r]);
      if (MASK) pr = key > r0 + 32 * mb + 16 * (r >> 3) + 8 * g + (r & 7) ? 0.f : pr;
      s[mb][r] = pr;
    }
  }
  {
    half8 vl[D / 16];
#pragma unroll
    for (int t = 0; t < D / 16; ++t) vl[t] = *reinterpret_cast<const half8*>(vrow + 16 * t);
    scores_add<D, NMB>(dp, Ds, vl, l32, g);
  }
#pragma unroll
  for (int mb = 0; mb < NMB; ++mb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) dp[mb][r] = s[mb][r] * dp[mb][r];
  }
  half8 pf[2 * NMB], sf[2 * NMB];
  to_frags<NMB>(s, pf);
  to_frags<NMB>(dp, sf);
  if constexpr (DS) {
#pragma unroll
    for (int t = 0; t < 2 * NMB; ++t) ds_out[t] = key_ok ? sf[t] : half8{};
  }
  accumulate_tr<D, 2 * NMB>(dv, Ds, pf, lane);
  accumulate_tr<D, 2 * NMB>(dk, Qs, sf, lane);
}

// ------------------------------------------------------------------ forward
// Workgroup = 128 FWD_NB query rows of one head (4 waves x 32 FWD_NB rows);
// the loop streams FBN-key tiles of K~ and V through double-buffered LDS,
// the next tile's copies in flight while the current tile is computed.
// Rows below the exact corner are skipped.
// G: key groups.  G = 2 (launches too small to give every CU two
// workgroups) splits each workgroup's key range between two groups of 4
// waves on the same 128 queries, each streaming its own tiles; the second
// group's O, m and l are merged into the first's through LDS at the end.
constexpr int FWD_BM = 4 * 32 * FWD_NB;
constexpr int FBN = 32 * FWD_MB;   // keys per forward step

template <int D, bool CAUSAL, bool BL, int G = 1>
__global__ __launch_bounds__(256 * G, FWD_WPS) void fwd_kernel(MfmaParams p) {
  static_assert(G == 1 || (G == 2 && !BL && FWD_NB == 1), "key groups: dense attention, 32-row waves");
  constexpr int DT = D / 16, CB = D / 32, TILE = TileDMA<D, FBN>::ALLOC, NB = FWD_NB;
  constexpr size_t MAIN = G * 4 * (size_t)TILE * sizeof(half_t);
  // G = 2 hands group 1's O (D/2 floats a lane), m and l over through the tiles
  static_assert(G == 1 || MAIN >= 4 * 64 * (D / 2 + 2) * sizeof(float), "hand-over fits the tiles");
  // the main tiles, or a corner workgroup's tiles (the launch's last ones)
  __shared__ __attribute__((aligned(16))) char pool[MAIN > corner_fwd_smem(D) ? MAIN : corner_fwd_smem(D)];
  __shared__ short blist[BL ? MAX_BLOCKS : 1];   // block-list mode: the key blocks, ascending
  __shared__ int bcount;
  const int BH = p.B * p.H;
  const int ntiles = (p.N + FWD_BM - 1) / FWD_BM, t0 = p.corner / FWD_BM;
  if ((int)blockIdx.x >= BH * (ntiles - t0)) {   // the corner's split-operand rows
    if (p.corner > 0) {
      if (G > 1 && threadIdx.x >= 256) corner_fwd_idle<D>(p, (int)blockIdx.x - BH * (ntiles - t0));
      else corner_fwd<D>(p, (int)blockIdx.x - BH * (ntiles - t0), pool);
    }
    return;
  }

  const int lane = threadIdx.x & 63, wg = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = wg >> 2, w = wg & 3;   // key group, wave within it
  const int l32 = lane & 31, g = lane >> 5;
  half_t* Ks = reinterpret_cast<half_t*>(pool) + grp * 4 * TILE;
  half_t* Vs = Ks + 2 * TILE;
  int bh, t;
  map_block(blockIdx.x, BH, ntiles - t0, true, bh, t);
  t += t0;
  const int q0 = t * FWD_BM, wrow0 = q0 + 32 * NB * w;
  const size_t head = (size_t)bh * p.N * D;
  const half_t* kh = p.kh + head;
  const half_t* vh = p.vh + head;
  // waves whose rows all lie in the exact corner (or past N) only help load
  const bool active = wrow0 + 32 * NB > p.corner && wrow0 < p.N;

  half8 qf[NB][DT];
  int qrow[NB], klim[NB];
  f32x16 o[NB][CB];
  f32x16 negm[NB];   // -m (D = 64 seeds the score products with it)
  float m[NB], l[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    qrow[nb] = wrow0 + 32 * nb + l32;
    klim[nb] = CAUSAL ? min(qrow[nb], p.N - 1) : p.N - 1;
    load_frag_rows<D>(qf[nb], p.qh + head, qrow[nb], p.N, g);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) o[nb][cb] = f32x16{};
    m[nb] = -INFINITY;
    l[nb] = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) negm[nb][r] = INFINITY;
  }
  const int wlast = wrow0 + 32 * NB - 1;
  // steps before `split` need no mask for any wave (the workgroup's diagonal
  // and the ragged tail come after); the loop is peeled there so each loop
  // carries a single inlined tile body.  Block-list mode walks the listed
  // key blocks (two steps each; the own block, masked, is the last under the
  // causal mask, and a ragged last block is the last in any case, cut to
  // the steps that start below N).
  int n_kt, split;
  if constexpr (BL) {
    static_assert(FWD_BM == BLK && BLK % FBN == 0, "one query block per workgroup");
    if (w == 0) {
      const int c = row_blocks(p.bmask + ((size_t)bh * p.nb + t) * p.W, p.nb, blist, lane);
      if (lane == 0) bcount = c;
    }
    __syncthreads();
    const int last = blist[bcount - 1];
    const int rows = min(BLK, p.N - last * BLK), steps = (rows + FBN - 1) / FBN;
    n_kt = BLK / FBN * (bcount - 1) + steps;
    split = ((CAUSAL && last == t) || rows < BLK) ? n_kt - steps : n_kt;
  } else {
    const int nk = (p.N + FBN - 1) / FBN;
    n_kt = CAUSAL ? min(nk, (q0 + FWD_BM + FBN - 1) / FBN) : nk;
    split = min(n_kt, min(CAUSAL ? q0 / FBN : nk, p.N / FBN));
  }
  // this group's steps: [0, h) for group 0, [h, n_kt) for group 1; every
  // wave runs h steps (a group past its own count only keeps the barriers)
  const int h = G == 1 ? n_kt : (n_kt + 1) / 2;
  const int g_first = grp ? h : 0, n_g = grp ? n_kt - h : h;
  const int unmasked = G == 1 ? split : min(max(split - g_first, 0), n_g);
  Walk<FBN, BL> walk;
  walk.init(blist, g_first * FBN, n_g);

  TileDMA<D, FBN> dma;
  dma.init(lane, w);
  if (G == 1 || n_g > 0) {
    dma.load(Ks, kh, walk.cur);
    dma.load(Vs, vh, walk.cur);
  }
  wait_lds_copies();
  __syncthreads();
  auto step = [&](int kt, auto masked) {
    if (G > 1 && kt >= n_g) {
      __syncthreads();
      return;
    }
    const int k0 = walk.cur;
    const int cur = (kt & 1) * TILE, nxt = TILE - cur;
    if (kt + 1 < n_g) {
      dma.load(Ks + nxt, kh, walk.next);
      dma.load(Vs + nxt, vh, walk.next);
    }
    walk.prefetch(kt);
    __builtin_amdgcn_sched_barrier(0);  // keep the next tile's copies ahead of the compute
    if (active && !(CAUSAL && k0 > wlast))  // skip tiles wholly above this wave's rows
      fwd_tile<D, NB, decltype(masked)::value, FWD_MB>(o, m, l, negm, Ks + cur, Vs + cur, qf, k0, klim,
                                                       lane);
    wait_lds_copies();
    __syncthreads();
    walk.advance(kt);
  };
  int kt = 0;
  for (; kt < unmasked; ++kt) step(kt, std::false_type{});
  for (; kt < h; ++kt) step(kt, std::true_type{});

  if constexpr (G == 2) {   // group 1's partial softmax merged into group 0's
    float* const xf = reinterpret_cast<float*>(pool) + w * (64 * (D / 2 + 2));
    if (grp == 1) {
#pragma unroll
      for (int j = 0; j < 4 * CB; ++j)
        *reinterpret_cast<float4*>(xf + 4 * (64 * j + lane)) =
            make_float4(o[0][j >> 2][4 * (j & 3)], o[0][j >> 2][4 * (j & 3) + 1],
                        o[0][j >> 2][4 * (j & 3) + 2], o[0][j >> 2][4 * (j & 3) + 3]);
      xf[64 * (D / 2) + lane] = m[0];
      xf[64 * (D / 2 + 1) + lane] = l[0];
    }
    __syncthreads();
    if (grp == 0) {
      // both groups hold each row's reference in both of its lanes; a group
      // that saw no key of a row has m = -inf and O = l = 0 there
      const float m1 = xf[64 * (D / 2) + lane], l1 = xf[64 * (D / 2 + 1) + lane];
      const float mn = fmaxf(m[0], m1);
      const float a0 = m[0] == -INFINITY ? 0.f : exp2_fast(m[0] - mn);
      const float a1 = m1 == -INFINITY ? 0.f : exp2_fast(m1 - mn);
#pragma unroll
      for (int j = 0; j < 4 * CB; ++j) {
        const float4 x = *reinterpret_cast<const float4*>(xf + 4 * (64 * j + lane));
        f32x16& r = o[0][j >> 2];
        const int e = 4 * (j & 3);
        r[e] = r[e] * a0 + x.x * a1;
        r[e + 1] = r[e + 1] * a0 + x.y * a1;
        r[e + 2] = r[e + 2] * a0 + x.z * a1;
        r[e + 3] = r[e + 3] * a0 + x.w * a1;
      }
      l[0] = l[0] * a0 + l1 * a1;
      m[0] = mn;
    }
  }

#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const float lt = l[nb] + __shfl_xor(l[nb], 32, 64);
    const int row = qrow[nb];
    if (grp == 0 && active && row >= p.corner && row < p.N) {
      const float inv = 1.f / lt;
      float* orow = p.o + head + (size_t)row * D;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int c = 32 * cb + 8 * rq + 4 * g;
          *reinterpret_cast<float4*>(orow + c) =
              make_float4(o[nb][cb][4 * rq] * inv, o[nb][cb][4 * rq + 1] * inv,
                          o[nb][cb][4 * rq + 2] * inv, o[nb][cb][4 * rq + 3] * inv);
        }
      }
      if (g == 0) p.out_lse[(size_t)bh * p.N + row] = (m[nb] + __log2f(lt)) * LN2;
    }
  }
}

// ------------------------------------------------------------------ dQ
// Workgroup = 128 query rows; streams KB-key tiles of K~ and V.  The K~
// tile serves both the score product (natural reads) and dQ~ += dS K~
// (transposed reads).
// At D = 64 the operands and accumulators take half the registers: three
// waves per SIMD fit (measured at 1 x 8 x 32768 x 64: 1.493 vs 1.557 ms with two).
template <int D, bool CAUSAL, bool BL>
__global__ __launch_bounds__(256, (D == 64 ? 3 : DQ_WPS)) void dq_kernel(MfmaParams p) {
  constexpr int SB = DQ_BN, NMB = SB / 32, KB = SB * DQ_SUB;
  constexpr int DT = D / 16, CB = D / 32, TILE = TileDMA<D, KB>::ALLOC;
  constexpr size_t MAIN = 4 * (size_t)TILE * sizeof(half_t);
  // the main tiles, or a corner workgroup's tiles (the launch's first ones)
  __shared__ __attribute__((aligned(16))) char pool[MAIN > corner_bwd_smem(D) ? MAIN : corner_bwd_smem(D)];
  __shared__ short blist[BL ? MAX_BLOCKS : 1];
  __shared__ int bcount;
  __shared__ float red[4 * (D / 2)];
  const int ncorner = p.corner ? 3 * corner_blocks(p) : 0;
  const int bx = (int)blockIdx.x;
  if (bx >= p.corner_at && bx < p.corner_at + ncorner) {
    corner_bwd<D>(p, bx - p.corner_at, pool);
    return;
  }
  const int mb = bx < p.corner_at ? bx : bx - ncorner;   // this workgroup's dQ tile
  half_t* Ks = reinterpret_cast<half_t*>(pool);
  half_t* Vs = Ks + 2 * TILE;

  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const int BH = p.B * p.H;
  const int ntiles = (p.N + BM - 1) / BM, t0 = p.corner / BM;
  int bh, t;
  map_block(mb, BH, ntiles - t0, true, bh, t);
  const int slot = p.slot0 + ncorner + mb;
  t += t0;
  const int q0 = t * BM, wrow0 = q0 + 32 * w, qrow = wrow0 + l32;
  const size_t head = (size_t)bh * p.N * D;
  const half_t* kh = p.kh + head;
  const half_t* vh = p.vh + head;

  half8 qf[DT], df[DT];
  load_frag_rows<D>(qf, p.qh + head, qrow, p.N, g);
  load_frag_rows<D>(df, p.doh + head, qrow, p.N, g);
  const bool row_ok = qrow < p.N;
  const float lse2 = row_ok ? p.lse[(size_t)bh * p.N + qrow] * LOG2E : 0.f;
  const float dr = row_ok ? p.drow[(size_t)bh * p.N + qrow] : 0.f;
  f32x16 acc[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) acc[cb] = f32x16{};
  // unmasked steps first, then the diagonal and ragged tail (peeled loops,
  // one inlined tile body each); block-list mode walks the listed key blocks
  constexpr int SPB = BLK / KB;   // steps per block
  int n_kt, split;
  if constexpr (BL) {
    static_assert(BM == BLK && BLK % KB == 0, "one query block per workgroup");
    if (w == 0) {
      const int c = row_blocks(p.bmask + ((size_t)bh * p.nb + t) * p.W, p.nb, blist, lane);
      if (lane == 0) bcount = c;
    }
    __syncthreads();
    const int last = blist[bcount - 1];
    const int rows = min(BLK, p.N - last * BLK), steps = (rows + KB - 1) / KB;
    n_kt = SPB * (bcount - 1) + steps;
    split = ((CAUSAL && last == t) || rows < BLK) ? n_kt - steps : n_kt;
  } else {
    const int nk = (p.N + KB - 1) / KB;
    n_kt = CAUSAL ? min(nk, (q0 + BM + KB - 1) / KB) : nk;
    split = min(n_kt, min(CAUSAL ? q0 / KB : nk, p.N / KB));
  }
  Walk<KB, BL> walk;
  walk.init(blist, 0, n_kt);

  TileDMA<D, KB> dma;
  dma.init(lane, w);
  dma.load(Ks, kh, walk.cur);
  dma.load(Vs, vh, walk.cur);
  wait_lds_copies();
  __syncthreads();
  const int klim = CAUSAL ? min(qrow, p.N - 1) : p.N - 1;
  auto step = [&](int kt, auto masked) {
    const int k0 = walk.cur;
    const int cur = (kt & 1) * TILE, nxt = TILE - cur;
    if (kt + 1 < n_kt) {
      dma.load(Ks + nxt, kh, walk.next);
      dma.load(Vs + nxt, vh, walk.next);
    }
    walk.prefetch(kt);
    __builtin_amdgcn_sched_barrier(0);  // keep the next tile's copies ahead of the compute
#pragma unroll
    for (int sub = 0; sub < DQ_SUB; ++sub) {
      // rows SB sub .. of the tile: the row layout keeps each 32-row half whole
      const int ks = k0 + SB * sub;
      if (!(CAUSAL && ks > wrow0 + 31))
        dq_tile<D, NMB, decltype(masked)::value>(acc, Ks + cur + SB * sub * (D + 8),
                                                 Vs + cur + SB * sub * (D + 8), qf, df, ks, klim,
                                                 lse2, dr, lane);
    }
    wait_lds_copies();
    __syncthreads();
    walk.advance(kt);
  };
  int kt = 0;
  for (; kt < split; ++kt) step(kt, std::false_type{});
  for (; kt < n_kt; ++kt) step(kt, std::true_type{});

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
// Workgroup = 128 keys of one head (4 waves x 32 keys); streams QB-row
// tiles of Q~ and dO plus their row scalars.  Q~ serves the score product
// and dK~ += dS^T Q~; dO serves dP = dO V^T and dV += P^T dO.  The
// workgroup's V rows stay in LDS (natural layout) and feed dP.  DS also
// writes dS into the panels for the dQ product (zeros for the pairs of
// a step that a wave skips as wholly masked, which that product reads).
// G: query groups.  G = 2 (launches too small to give every CU two
// workgroups) splits each workgroup's query range between two groups of 4
// waves on the same 128 keys, each streaming its own tiles; the second
// group's dK, dV are added to the first's through LDS at the end (a fixed
// order), so the per-workgroup chain of steps is half as long.
template <int D, bool CAUSAL, bool BL, bool DS, int G = 1>
__global__ __launch_bounds__(256 * G, DKDV_WPS) void dkdv_kernel(MfmaParams p) {
  static_assert(G == 1 || (G == 2 && !BL), "query groups: dense attention only");
  constexpr int QB = DKDV_BN, NMB = QB / 32;
  constexpr int DT = D / 16, CB = D / 32, TILE = TileDMA<D, QB>::ALLOC;
  // each group's double-buffered Q~ and dO tiles; G = 2 also reuses them
  // for the dK, dV hand-over (4 waves x 64 lanes x D/2 floats)
  static_assert(G == 1 || 2 * G * 2 * TILE * 2 >= 4 * 64 * (D / 2) * 4, "hand-over fits the tiles");
  __shared__ __attribute__((aligned(16))) half_t tiles[G * 2 * 2 * TILE];
  __shared__ __attribute__((aligned(16))) half_t Vst[BM * (D + 8)];
  __shared__ __attribute__((aligned(16))) float rsl[G * 2 * 2 * QB];
  __shared__ float red[4 * G * (D / 2)];
  __shared__ short blist[BL ? MAX_BLOCKS : 1];   // block-list mode: the query blocks, ascending
  __shared__ uint32_t bcol[BL ? MAX_BLOCKS / 32 : 1];
  __shared__ int bcount;

  // the wave index as a scalar: per-wave skips and panel addresses stay uniform
  const int lane = threadIdx.x & 63, wg = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = wg >> 2, w = wg & 3;   // query group, wave within it
  const int l32 = lane & 31, g = lane >> 5;
  half_t* const Qs = tiles + grp * 4 * TILE;
  half_t* const Ds = Qs + 2 * TILE;
  float* const rsg = rsl + grp * 2 * 2 * QB;
  const int BH = p.B * p.H;
  const int ntiles = (p.N + BM - 1) / BM;
  int bh, t;
  // key tile t has the N - 128 t query rows after it under the causal
  // mask: low tiles are the heavy ones
  map_block(blockIdx.x, BH, ntiles, false, bh, t);
  const int slot = p.slot0 + blockIdx.x;
  const int k0 = t * BM, wkey0 = k0 + 32 * w, key = wkey0 + l32;
  const size_t head = (size_t)bh * p.N * D;
  const half_t* qh = p.qh + head;
  const half_t* doh = p.doh + head;
  const float* rs_h = p.rs + (size_t)bh * rs_groups(p.N) * 64;

  half8 kf[DT];
  load_frag_rows<D>(kf, p.kh + head, key, p.N, g);
  // rows k0 .. k0 + 127 of V, padded rows; lane reads row 32 w + l32
  for (int ch = threadIdx.x; ch < BM * (D / 8); ch += 256 * G) {
    const int r = ch / (D / 8), c8 = ch % (D / 8);
    const int row = min(k0 + r, p.N - 1);
    *reinterpret_cast<half8*>(Vst + r * (D + 8) + c8 * 8) =
        *reinterpret_cast<const half8*>(p.vh + head + (size_t)row * D + c8 * 8);
  }
  const half_t* vrow = Vst + (32 * w + l32) * (D + 8) + 8 * g;
  f32x16 dk[CB], dv[CB];
#pragma unroll
  for (int cb = 0; cb < CB; ++cb) { dk[cb] = f32x16{}; dv[cb] = f32x16{}; }
  int qs0 = CAUSAL ? k0 : 0;
  if (qs0 < p.corner) qs0 = p.corner;  // pairs with query rows < corner: exact path
  // block-list mode: the query blocks that attend this key block (the own
  // block first, masked, under the causal mask; rows < corner excluded; a
  // ragged last block cut to the steps that start below N, as the row
  // scalars end there)
  constexpr int SPB = BLK / QB;
  int n_it;
  if constexpr (BL) {
    static_assert(BM == BLK && BLK % QB == 0, "one key block per workgroup");
    const int cnt = column_blocks<256 * G>(p.bmask, p.nb, p.W, bh, t, qs0 / BLK, bcol, blist, &bcount);
    n_it = 0;
    if (cnt > 0) {
      const int rows = min(BLK, p.N - blist[cnt - 1] * BLK);
      n_it = SPB * (cnt - 1) + (rows + QB - 1) / QB;
    }
  } else {
    n_it = qs0 < p.N ? (p.N - qs0 + QB - 1) / QB : 0;
  }
  // this group's steps: [0, h) for group 0, [h, n_it) for group 1
  const int h = G == 1 ? n_it : (n_it + 1) / 2;
  const int g_first = grp ? h : 0, n_g = grp ? n_it - h : h;
  Walk<QB, BL> walk;
  walk.init(blist, qs0 + g_first * QB, n_g);

  TileDMA<D, QB> dma;
  dma.init(lane, w);
  // one step's tiles; wave j < NMB also copies the row scalars of 32-row
  // group j (lane i -> float i; qs0 is a multiple of 32)
  auto load_rows = [&](int r0, int buf) {
    dma.load(Qs + buf * TILE, qh, r0);
    dma.load(Ds + buf * TILE, doh, r0);
    if (dma.wave < NMB)
      lds_copy4(rs_h + ((r0 >> 5) + dma.wave) * 64, 4u * lane_here(), rsg + buf * 2 * QB + dma.wave * 64);
  };
  if (n_g > 0) load_rows(walk.cur, 0);
  wait_lds_copies();
  __syncthreads();
  // the first steps cross the workgroup's diagonal (masked), the rest need
  // no mask: peeled loops, one inlined tile body each (with G = 2 the second
  // group runs its first steps through the masked body too, which is exact)
  int n_masked;
  if constexpr (BL)
    n_masked = (CAUSAL && n_it > 0 && blist[0] == t) ? min(n_it, SPB) : 0;
  else
    n_masked = (CAUSAL && qs0 <= k0 + BM - 2) ? min(n_it, (k0 + BM - 2 - qs0) / QB + 1) : 0;
  // dS panels: a scalar base per step (the block of this wave's 32 keys and
  // the step's 32 queries) plus this lane's byte offset in it (its key's
  // 16-query rows, 8 g columns; chunk t adds a 1 KiB half).  A step's dS is
  // stored at the start of the next step (non-temporal: the dQ pass reads
  // it once), so the stores have a whole step to complete before the step's
  // closing wait, which covers them too.
  const char* const ds_head =
      DS ? reinterpret_cast<const char*>(p.dsp + (size_t)bh * panel_head(p.N, CAUSAL)) : nullptr;
  const uint32_t ds_lane = 2u * (16u * l32 + 8u * g);
  // keys at or past N store zeros; under the causal mask every pair of such
  // a key is masked (every query is below N), so dS is already 0 there
  const bool key_ok = CAUSAL || key < p.N;
  half8 ds_pend[2 * NMB];
  const char* ds_base = nullptr;   // the pending step's row base (uniform), or null
  auto flush_ds = [&]() {
    if constexpr (DS) {
      if (ds_base) {
#pragma unroll
        for (int t = 0; t < 2 * NMB; ++t)
          __builtin_nontemporal_store(
              ds_pend[t], reinterpret_cast<half8*>(const_cast<char*>(ds_base) + ds_lane + 1024 * t));
      }
    }
  };
  auto step = [&](int it, auto masked) {
    if (G > 1 && it >= n_g) {   // this group is done: keep the barriers in step
      __syncthreads();
      return;
    }
    const int r0 = walk.cur;
    const int cur = it & 1;
    if (it + 1 < n_g) load_rows(walk.next, cur ^ 1);
    walk.prefetch(it);
    flush_ds();
    __builtin_amdgcn_sched_barrier(0);  // keep the next tile's copies ahead of the compute
    if constexpr (DS)
      ds_base = ds_head + 2 * (panel_off(r0 / PANEL, p.N, CAUSAL) + (size_t)wkey0 * PANEL +
                               (size_t)(r0 % PANEL) * 32);
    if (!(CAUSAL && wkey0 > r0 + QB - 1)) {  // skip tiles wholly before this wave's keys
      dkdv_tile<D, NMB, decltype(masked)::value, DS>(dk, dv, Qs + cur * TILE, Ds + cur * TILE,
                                                     rsg + cur * 2 * QB, kf, vrow, r0, key, lane,
                                                     ds_pend, key_ok);
    } else if constexpr (DS) {
#pragma unroll
      for (int t = 0; t < 2 * NMB; ++t) ds_pend[t] = half8{};
    }
    wait_lds_copies();
    __syncthreads();
    walk.advance(it);
  };
  int it = 0;
  for (; it < n_masked; ++it) step(it, std::true_type{});
  for (; it < h; ++it) step(it, std::false_type{});
  flush_ds();
  if constexpr (G == 2) {   // group 1's dK, dV added to group 0's (then group 1 idles)
    float* const xf = reinterpret_cast<float*>(tiles) + w * (64 * 64);
    auto hand_over = [&](f32x16* acc) {
      __syncthreads();
      if (grp == 1) {
#pragma unroll
        for (int j = 0; j < 4 * CB; ++j)
          *reinterpret_cast<float4*>(xf + 4 * (64 * j + lane)) =
              make_float4(acc[j >> 2][4 * (j & 3)], acc[j >> 2][4 * (j & 3) + 1],
                          acc[j >> 2][4 * (j & 3) + 2], acc[j >> 2][4 * (j & 3) + 3]);
      }
      __syncthreads();
      if (grp == 0) {
#pragma unroll
        for (int j = 0; j < 4 * CB; ++j) {
          const float4 x = *reinterpret_cast<const float4*>(xf + 4 * (64 * j + lane));
          acc[j >> 2][4 * (j & 3)] += x.x;
          acc[j >> 2][4 * (j & 3) + 1] += x.y;
          acc[j >> 2][4 * (j & 3) + 2] += x.z;
          acc[j >> 2][4 * (j & 3) + 3] += x.w;
        }
      }
    };
    hand_over(dk);
    hand_over(dv);
  }

  float wv[D / 4];
#pragma unroll
  for (int i = 0; i < D / 4; ++i) wv[i] = 0.f;
  if (grp == 0 && key < p.N) {
    // Q~ carries log2(e)/sqrt(D): dK~ = dS^T Q~ / sqrt(D) = ln 2 * (dS^T Q~'); the
    // dO scale is undone here.  Keys below the corner get the corner's share
    // (queries below it) added by the dQ launch.
    const float dinv = dscale_inv(p.dsc, bh);
    finish_rows<D>(dk, LN2 * dinv, nullptr, p.cs + (size_t)key * (D / 2), p.k, head + (size_t)key * D,
                   p.bf16, p.dk + head + (size_t)key * D, (float)key, wv, g);
    float* dvrow = p.dv + head + (size_t)key * D;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int c = 32 * cb + 8 * rq + 4 * g;
        *reinterpret_cast<float4*>(dvrow + c) =
            make_float4(dv[cb][4 * rq] * dinv, dv[cb][4 * rq + 1] * dinv,
                        dv[cb][4 * rq + 2] * dinv, dv[cb][4 * rq + 3] * dinv);
      }
    }
  }
  store_dalpha<D, 4 * G>(wv, red, p.dalpha_part + (size_t)slot * (D / 2), g);
}

// ------------------------------------------------------------------ dQ from the dS panels
// B fragments (8 keys of one query per lane, as the score registers give
// it) from a 32-key panel tile in LDS: query block c (32 queries), k step
// ts at lane offset + 1024 c + 256 ts, two transposed reads 64 halfs apart.
// In each 16-lane group the 16 lanes point at 4 keys x 16 queries of the
// block's half b (4 consecutive queries each, 128 contiguous bytes: no bank
// conflict) and the transposing read hands lane j query j's 4 keys.
__device__ __forceinline__ int panel_lane_offset(int lane) {
  const int s16 = lane & 15, b = (lane >> 4) & 1, g = lane >> 5;
  return b * 512 + (8 * g + (s16 >> 2)) * 16 + 4 * (s16 & 3);
}

// dQ~ = dS K~ over the panels the dK/dV pass wrote: a plain product, no
// score recomputation.  Workgroup = the PANEL (256) query rows of one panel,
// 4 waves x 64 rows; streams 32-key tiles of the panel (16 KiB, contiguous,
// copied as is) and of K~ through a ring of DQP_STAGES LDS buffers, so that
// DQP_STAGES - 1 tiles are in flight while one is computed (the panel is
// read once from HBM, and the copies in flight cover its latency; it is
// streamed with the non-temporal hint).  Both operands are read transposed:
// the panel gives the B fragments (8 keys of one query per lane), K~
// columns the A fragments, and each K~ fragment feeds the wave's two 32-row
// blocks.  Pairs after a query's diagonal hold zeros in the panel; a wave
// skips tiles wholly after its rows.  Waves whose rows lie in the exact
// corner only help load.
constexpr int DQP_KB = 32;
constexpr int DQP_TS = DQP_KB * PANEL;   // halfs per panel tile (16 KiB)
constexpr int DQP_STAGES = 3;

// NJ: 32-row query blocks per wave, 2 (a whole panel per workgroup) or 1 (half
// a panel, for launches too small to fill the GPU otherwise).
// G: key groups.  G = 2 (half panels, launches still too small to give
// every CU two workgroups) splits each workgroup's key tiles between two
// groups of 4 waves on the same query rows, each with its own ring; the
// second group's dQ~ is added to the first's through LDS at the end.
template <int D, bool CAUSAL, int NJ, int G = 1>
__global__ __launch_bounds__(256 * G, DQ_WPS) void dq_panel_kernel(MfmaParams p) {
  static_assert(G == 1 || (G == 2 && NJ == 1), "key groups: half panels");
  constexpr int CB = D / 32, TK = TileDMA<D, DQP_KB>::ALLOC, TS = DQP_TS * NJ / 2;
  constexpr int NS = DQP_STAGES;
  static_assert(TS * 2 == NJ * 8 * 1024, "2 NJ 1 KiB copies per wave per panel tile");
  constexpr size_t RING = (size_t)NS * (TK + TS) * sizeof(half_t), MAIN = G * RING;
  static_assert(G == 1 || MAIN >= 4 * 64 * NJ * (D / 2) * sizeof(float), "hand-over fits the rings");
  // the rings, or a corner workgroup's tiles (the launch's last ones)
  __shared__ __attribute__((aligned(16))) char pool[MAIN > corner_bwd_smem(D) ? MAIN : corner_bwd_smem(D)];
  __shared__ float red[4 * G * (D / 2)];
  const int ncorner = p.corner ? 3 * corner_blocks(p) : 0;
  const int bx = (int)blockIdx.x;
  if (bx >= p.corner_at && bx < p.corner_at + ncorner) {
    if (G > 1 && threadIdx.x >= 256) corner_bwd_idle<D>(p, bx - p.corner_at);
    else corner_bwd<D>(p, bx - p.corner_at, pool);
    return;
  }
  const int mb = bx < p.corner_at ? bx : bx - ncorner;   // this workgroup's panel (half)

  const int lane = threadIdx.x & 63, wg = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = wg >> 2, w = wg & 3;   // key group, wave within it
  const int l32 = lane & 31, g = lane >> 5;
  half_t* Ks = reinterpret_cast<half_t*>(pool + grp * RING);
  half_t* Ss = Ks + NS * TK;
  const int BH = p.B * p.H;
  const int np = n_panels(p.N), t0 = p.corner / PANEL;
  int bh, u;
  map_block(mb, BH, (np - t0) * (2 / NJ), true, bh, u);
  const int slot = p.slot0 + ncorner + mb;
  const int t = u / (2 / NJ) + t0, hb = NJ == 1 ? (u & 1) : 0;   // panel, half
  const int q0 = t * PANEL + 128 * hb, wrow0 = q0 + 32 * NJ * w;
  const size_t head = (size_t)bh * p.N * D;
  const half_t* kh = p.kh + head;
  const half_t* panel = p.dsp + (size_t)bh * panel_head(p.N, CAUSAL) + panel_off(t, p.N, CAUSAL);
  const bool active = wrow0 + 32 * NJ > p.corner && wrow0 < p.N;
  // keys of this panel below N, in whole tiles (the panel rows are a
  // multiple of the tile; a ragged last tile holds zeros past N)
  const int nkeys = min(panel_rows(t, p.N, CAUSAL), (p.N + DQP_KB - 1) / DQP_KB * DQP_KB);
  const int n_kt_all = nkeys / DQP_KB;
  // this group's tiles: [0, h) for group 0, [h, n_kt_all) for group 1, as
  // steps 0 .. n_kt - 1 from kt0; every wave runs h steps (a group past its
  // own count only keeps the barriers)
  const int h = G == 1 ? n_kt_all : (n_kt_all + 1) / 2;
  const int kt0 = grp ? h : 0, n_kt = grp ? n_kt_all - h : h;

  f32x16 acc[NJ][CB];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[j][cb] = f32x16{};
  }
  TileDMA<D, DQP_KB> dmk;
  dmk.init(lane, w);
  const int wave = w;
  // this lane's fragment offsets in a ring slot (its wave's NJ query blocks)
  const int pf_lane = 1024 * NJ * w + panel_lane_offset(lane), tr_lane = tr_lane_offset<D>(lane);
  // Copies this wave issues per tile: KLO or KLO + 1 for K~, 2 NJ for the panel.
  // Every outstanding vector memory operation of the loop is such a copy, so
  // "tile i landed" is "at most (copies per tile) x (tiles issued after i)
  // outstanding".  In the steady state NS - 2 tiles stay in flight; the last
  // steps wait for everything.
  constexpr int KLO = TileDMA<D, DQP_KB>::NBLK / 4;
  constexpr int PC = 2 * NJ;   // panel copies per wave per tile
  static_assert((KLO + 1 + PC) * (NS - 2) < 64, "vmcnt range");
  const bool khi = dmk.count() > KLO;
  auto wait_landed = [&](bool steady) {
    if (!steady) wait_vm_const<0>();
    else if (khi) wait_vm_const<(KLO + 1 + PC) * (NS - 2)>();
    else wait_vm_const<(KLO + PC) * (NS - 2)>();
  };
  auto load = [&](int kt) {
    const int b = kt % NS;
    dmk.load(Ks + b * TK, kh, (kt0 + kt) * DQP_KB);
    // the panel tile (this half's query blocks): 1 KiB blocks wave + 4 i,
    // lane l at byte 16 l
    const uint32_t tb = (uint32_t)(kt0 + kt) * (uint32_t)(2 * DQP_TS) + 8192u * (uint32_t)hb;
#pragma unroll
    for (int i = 0; i < PC; ++i)
      lds_copy16_nt(panel, tb + 1024u * (wave + 4 * i) + 16u * lane, Ss + b * TS + (wave + 4 * i) * 512);
  };
#pragma unroll
  for (int i = 0; i < NS - 1; ++i) {
    if (i < n_kt) load(i);
  }
  wait_landed(n_kt >= NS - 1);   // tile 0
  __syncthreads();
  for (int kt = 0; kt < h; ++kt) {
    if (G > 1 && kt >= n_kt) {   // this group is done (its copies all landed)
      __syncthreads();
      continue;
    }
    const int k0 = (kt0 + kt) * DQP_KB;
    // ring slot offsets as opaque scalars: the fragment addresses are then one
    // add each, not offsets the compiler derives from kt per read
    const int slot = __builtin_amdgcn_readfirstlane(kt % NS);
    const int ck = slot * TK, cs = slot * TS;
    // into the buffer every wave finished reading before the last barrier
    if (kt + NS - 1 < n_kt) load(kt + NS - 1);
    __builtin_amdgcn_sched_barrier(0);  // keep the next tiles' copies ahead of the compute
    if (active && !(CAUSAL && k0 > wrow0 + 32 * NJ - 1)) {
      // every fragment of the step first (one address add per operand, the
      // rest in the reads' offsets), then the products
      const half_t* pb = Ss + cs + pf_lane;
      const half_t* kb = Ks + ck + tr_lane;
      half8 bf[DQP_KB / 16][NJ], af[DQP_KB / 16][CB];
#pragma unroll
      for (int ts = 0; ts < DQP_KB / 16; ++ts) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) bf[ts][j] = tr_pair<64>(pb + 1024 * j + 256 * ts);
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) af[ts][cb] = tr_pair<8 * (D + 8)>(kb + 16 * ts * (D + 8) + 32 * cb);
      }
#pragma unroll
      for (int ts = 0; ts < DQP_KB / 16; ++ts) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) {
#pragma unroll
          for (int j = 0; j < NJ; ++j) acc[j][cb] = mfma(af[ts][cb], bf[ts][j], acc[j][cb]);
        }
      }
    }
    wait_landed(kt + NS - 1 < n_kt);   // tile kt + 1
    __syncthreads();
  }
  if constexpr (G == 2) {   // group 1's dQ~ added to group 0's (then group 1 idles)
    float* const xf = reinterpret_cast<float*>(pool) + w * (64 * (D / 2));
    if (grp == 1) {
#pragma unroll
      for (int j = 0; j < 4 * CB; ++j)
        *reinterpret_cast<float4*>(xf + 4 * (64 * j + lane)) =
            make_float4(acc[0][j >> 2][4 * (j & 3)], acc[0][j >> 2][4 * (j & 3) + 1],
                        acc[0][j >> 2][4 * (j & 3) + 2], acc[0][j >> 2][4 * (j & 3) + 3]);
    }
    __syncthreads();
    if (grp == 0) {
#pragma unroll
      for (int j = 0; j < 4 * CB; ++j) {
        const float4 x = *reinterpret_cast<const float4*>(xf + 4 * (64 * j + lane));
        f32x16& r = acc[0][j >> 2];
        const int e = 4 * (j & 3);
        r[e] += x.x;
        r[e + 1] += x.y;
        r[e + 2] += x.z;
        r[e + 3] += x.w;
      }
    }
  }

  float wv[D / 4], wj[D / 4];
#pragma unroll
  for (int i = 0; i < D / 4; ++i) wv[i] = 0.f;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int qrow = wrow0 + 32 * j + l32;
    if (grp == 0 && active && qrow >= p.corner && qrow < p.N) {
      finish_rows<D>(acc[j], p.scale * dscale_inv(p.dsc, bh), nullptr, p.cs + (size_t)qrow * (D / 2), p.q,
                     head + (size_t)qrow * D, p.bf16, p.dq + head + (size_t)qrow * D, (float)qrow,
                     wj, g);
#pragma unroll
      for (int i = 0; i < D / 4; ++i) wv[i] += wj[i];
    }
  }
  store_dalpha<D, 4 * G>(wv, red, p.dalpha_part + (size_t)slot * (D / 2), g);
}

int fwd_blocks(const MfmaParams& p) {  // dQ workgroups: 128-row tiles past the corner
  const int tiles = (p.N + BM - 1) / BM - p.corner / BM;
  return tiles > 0 ? p.B * p.H * tiles : 0;
}
int dkdv_blocks(const MfmaParams& p) { return p.B * p.H * ((p.N + BM - 1) / BM); }
// The dQ product takes half a panel per workgroup when whole panels would
// leave the GPU short of workgroups (fewer than two per CU of a 256-CU part).
constexpr int DQP_HALF_BELOW = 512;
bool dq_panel_half(const MfmaParams& p) {
  const int np = n_panels(p.N) - p.corner / PANEL;
  return (long)p.B * p.H * np < DQP_HALF_BELOW;
}
int dq_panel_blocks(const MfmaParams& p) {  // panels (halves) past the corner
  const int np = n_panels(p.N) - p.corner / PANEL;
  return np > 0 ? p.B * p.H * np * (dq_panel_half(p) ? 2 : 1) : 0;
}
// Half-panel launches of fewer workgroups than this also split each
// workgroup's key tiles between two wave groups.
constexpr int DQP_SPLIT_BELOW = 512;

}  // namespace

// dQ launch: the corner workgroups (dQ rows and dK, dV shares below the
// corner) first, then the dQ product's
int dq_corner_blocks(const MfmaParams& p) { return p.corner ? 3 * corner_blocks(p) : 0; }
int dq_mfma_slots(const MfmaParams& p) {
  return dq_corner_blocks(p) + (p.dsp ? dq_panel_blocks(p) : fwd_blocks(p));
}
int dkdv_mfma_slots(const MfmaParams& p) { return dkdv_blocks(p); }

#define RA_LAUNCH1(KERNEL, ...)                                                                 \
  do {                                                                                         \
    if (p.D == 64) {                                                                           \
      if (p.causal) hipLaunchKernelGGL((KERNEL<64, true, ##__VA_ARGS__>), grid, block, 0, s, p); \
      else hipLaunchKernelGGL((KERNEL<64, false, ##__VA_ARGS__>), grid, block, 0, s, p);       \
    } else {                                                                                   \
      if (p.causal) hipLaunchKernelGGL((KERNEL<128, true, ##__VA_ARGS__>), grid, block, 0, s, p); \
      else hipLaunchKernelGGL((KERNEL<128, false, ##__VA_ARGS__>), grid, block, 0, s, p);      \
    }                                                                                          \
  } while (0)
#define RA_LAUNCH(KERNEL, BLOCKS)                                                               \
  do {                                                                                         \
    const dim3 grid((unsigned)(BLOCKS)), block(256);                                           \
    if (p.bmask) RA_LAUNCH1(KERNEL, true);                                                     \
    else RA_LAUNCH1(KERNEL, false);                                                            \
  } while (0)

// The forward launch: the row tiles past the corner, heaviest first, then
// the corner's split-operand workgroups (beside the lightest tiles).
// Dense forward launches of fewer main workgroups than this (two per CU of
// a 256-CU part) split each workgroup's keys between two wave groups.
constexpr int FWD_SPLIT_BELOW = 512;
void launch_fwd_mfma(const MfmaParams& p, hipStream_t s) {
  const int nmain = p.B * p.H * max(0, (p.N + FWD_BM - 1) / FWD_BM - p.corner / FWD_BM);
  const int nb = nmain + (p.corner ? corner_blocks(p) : 0);
  if (nb <= 0) return;
  if (!p.bmask && nmain < FWD_SPLIT_BELOW) {
    const dim3 grid((unsigned)nb), block(512);
    if (p.D == 64) {
      if (p.causal) hipLaunchKernelGGL((fwd_kernel<64, true, false, 2>), grid, block, 0, s, p);
      else hipLaunchKernelGGL((fwd_kernel<64, false, false, 2>), grid, block, 0, s, p);
    } else {
      if (p.causal) hipLaunchKernelGGL((fwd_kernel<128, true, false, 2>), grid, block, 0, s, p);
      else hipLaunchKernelGGL((fwd_kernel<128, false, false, 2>), grid, block, 0, s, p);
    }
    return;
  }
  RA_LAUNCH(fwd_kernel, nb);
}
// The corner workgroups (latency-bound chains of a few to a few tens of
// steps) come last in the dQ launch's grid: the grid issues the heaviest dQ
// tiles first, and corner workgroups at its front would hold those back and
// lengthen the launch; at its end they run beside the lightest tiles
// (measured: at the front +22 us, in the middle +11 us, at the end +0 at
// 1 x 32 x 8192 x 128).
void launch_dq_mfma(const MfmaParams& p_in, hipStream_t s) {
  MfmaParams p = p_in;
  if (p.dsp) {  // dense attention with the dS panels written by the dK/dV pass (D = 128)
    p.corner_at = dq_panel_blocks(p);
    const int nb = dq_corner_blocks(p) + dq_panel_blocks(p);
    const dim3 grid((unsigned)nb), block(256);
    if (nb <= 0) return;
    if (dq_panel_half(p) && dq_panel_blocks(p) < DQP_SPLIT_BELOW) {
      const dim3 block2(512);
      if (p.causal) hipLaunchKernelGGL((dq_panel_kernel<128, true, 1, 2>), grid, block2, 0, s, p);
      else hipLaunchKernelGGL((dq_panel_kernel<128, false, 1, 2>), grid, block2, 0, s, p);
    } else if (dq_panel_half(p)) {
      if (p.causal) hipLaunchKernelGGL((dq_panel_kernel<128, true, 1>), grid, block, 0, s, p);
      else hipLaunchKernelGGL((dq_panel_kernel<128, false, 1>), grid, block, 0, s, p);
    } else {
      if (p.causal) hipLaunchKernelGGL((dq_panel_kernel<128, true, 2>), grid, block, 0, s, p);
      else hipLaunchKernelGGL((dq_panel_kernel<128, false, 2>), grid, block, 0, s, p);
    }
    return;
  }
  p.corner_at = fwd_blocks(p);
  const int nb = dq_corner_blocks(p) + fwd_blocks(p);
  if (nb > 0) RA_LAUNCH(dq_kernel, nb);
}
// Dense dK/dV launches of fewer workgroups than this (two per CU of a 256-CU
// part) split each workgroup's queries between two wave groups.
constexpr int DKDV_SPLIT_BELOW = 512;
void launch_dkdv_mfma(const MfmaParams& p, hipStream_t s) {
  const int nb = dkdv_blocks(p);
  if (nb <= 0) return;
  const dim3 grid((unsigned)nb), block(256);
  if (p.bmask) {
    RA_LAUNCH1(dkdv_kernel, true, false);
  } else if (nb < DKDV_SPLIT_BELOW) {
    const dim3 block2(512);
    if (p.dsp) {  // D = 128 only (the library sets panels for no other D)
      if (p.causal) hipLaunchKernelGGL((dkdv_kernel<128, true, false, true, 2>), grid, block2, 0, s, p);
      else hipLaunchKernelGGL((dkdv_kernel<128, false, false, true, 2>), grid, block2, 0, s, p);
    } else if (p.D == 64) {
      if (p.causal) hipLaunchKernelGGL((dkdv_kernel<64, true, false, false, 2>), grid, block2, 0, s, p);
      else hipLaunchKernelGGL((dkdv_kernel<64, false, false, false, 2>), grid, block2, 0, s, p);
    } else {
      if (p.causal) hipLaunchKernelGGL((dkdv_kernel<128, true, false, false, 2>), grid, block2, 0, s, p);
      else hipLaunchKernelGGL((dkdv_kernel<128, false, false, false, 2>), grid, block2, 0, s, p);
    }
  } else if (p.dsp) {  // D = 128 only (the library sets panels for no other D)
    if (p.causal) hipLaunchKernelGGL((dkdv_kernel<128, true, false, true>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((dkdv_kernel<128, false, false, true>), grid, block, 0, s, p);
  } else {
    RA_LAUNCH1(dkdv_kernel, false, false);
  }
}

}  // namespace ra
