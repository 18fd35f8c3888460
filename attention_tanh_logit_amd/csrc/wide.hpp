// 16-bit kernels (bf16; fp16 in the second build of these sources) for head
// dim 512: forward, and dk/dv, which hands dU to the dq kernel through the
// workspace, on the fast path's tiles and fragments.  With a bias (Sk % 8 ==
// 0), each quarter's owner reads the bias of its own pairs from global memory
// and dk/dv writes their dbias, so no slice repeats that work.
//
// A workgroup is 8 waves: two row (or key) groups x four column slices of
// 128.  A wave keeps only its slice of the fixed operand (Q columns in the
// forward, K and V columns in dk/dv) and of the output accumulators, so that
// two waves fit a SIMD.  Each wave contracts its 128 columns into a partial
// logit block (MaxText commit quoted on "Support logits soft-capping in the
// Pallas-Triton attention VJP": head_dim above 256 accumulated in chunks).
// The four partials of a group are reduce-scattered through LDS: each wave
// sums one quarter of the block's elements, in slice order, and computes the
// probabilities (and in dk/dv the dU) of that quarter only; the quarters,
// rounded to 16 bits as the P V, dO^T P and Q^T dU products take them, are
// then gathered through LDS so that every wave holds the whole fragments.
// The transcendental and elementwise work of a tile is thus done once per
// group, not once per slice.  Streamed tiles (K/V in the forward, Q/dO in
// dk/dv; 32 rows of 1 KiB) go HBM -> LDS by buffer DMA, double-buffered,
// swizzled per row as on the fast path (the swizzles permute 16-byte slots
// inside 128-column groups, so a slice is a plain column offset).  LDS:
// 4 x 32 KiB of tiles + 24 KiB of partials + the gathered fragments (and in
// the forward the row extremes and sums) = 156-158 KiB, one workgroup per CU.
#pragma once

#include "fast.hpp"

namespace ATL_NS {

// ============================================================== forward (D = 512)

// One workgroup = 64 query rows of one head; wave w = 4 rg + sl holds rows
// q0 + 32 rg .. + 31 and columns 128 sl .. + 127 of Q (as Q^T fragments)
// and of O.  Per 32-key tile: partial S^T = K Q^T over the slice's columns,
// reduce-scattered across the row group; wave sl takes the capped logits,
// masking and probabilities of its quarter (keys acc_row(h, 4 sl) + 0..3 of
// each lane's query) under the online softmax (running maximum, its extreme
// exchanged between the quarters through LDS, or for caps with
// 2 c log2(e) <= 120 a fixed reference maximum; see fwd_fast_kernel), keeps
// the row sum of its quarter, and after the gather O^T += V^T P^T over the
// slice's columns.  The quarters' row sums are added once, at the end.
// DROP: dropout as in fwd_fast_kernel; a lane's quarter is four keys of its
// query, half of a Philox4x32-10 evaluation (the other half belongs to
// another wave's quarter), so each lane evaluates once per key block.
template <bool CAP, bool FIXM, bool DROP, bool BIAS>
__global__ __launch_bounds__(512, 1) void fwd512_kernel(FwdParams p) {
  static_assert(CAP || !FIXM, "a fixed reference maximum needs bounded logits");
  constexpr int D = 512, NT = 512, BM = 64, BN = 32;
  constexpr int NCW = 8;   // 16-column contraction steps per slice
  constexpr int NOB = 4;   // 32-column output blocks per slice

  __shared__ __attribute__((aligned(16))) bf16 sK0[BN * D];
  __shared__ __attribute__((aligned(16))) bf16 sK1[BN * D];
  __shared__ __attribute__((aligned(16))) bf16 sV0[BN * D];
  __shared__ __attribute__((aligned(16))) bf16 sV1[BN * D];
  // partials for the reduce-scatter: [rg][quarter][the three other slices][lane]
  __shared__ __attribute__((aligned(16))) f32x4 sX[2 * 4 * 3 * 64];
  // the gathered P fragments: [rg][key half][lane]
  __shared__ __attribute__((aligned(16))) bf16x8 sP[2 * 2 * 64];
  // the quarters' logit extremes (per key tile), then their row sums: [rg][slice][lane]
  __shared__ float sE[2 * 4 * 64];

  int qt, hq, b;
  {
    int x, grp;
    xcd_order(gridDim.x, gridDim.y * gridDim.z, x, grp);
    qt = p.reverse ? gridDim.x - 1 - x : x;
    hq = grp % gridDim.y;
    b = grp / gridDim.y;
  }
  const int hk = hq / p.G;
  const int Sq = p.mask.Sq, Sk = p.mask.Sk;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int n = lane & 31;
  const int h = lane >> 5;
  const int rg = w >> 2;
  const int sl = w & 3;
  const int colofs = 128 * sl;
  const int q0 = qt * BM;
  const int i = q0 + rg * 32 + n;
  const LogitK lk(p.sl2, p.xc, p.bc, p.cl2, CAP);
  const FragOfs<D, false> fo(lane);

  const bf16* kbase = reinterpret_cast<const bf16*>(p.k) + koff(p, b, 0, hk, D);
  const bf16* vbase = reinterpret_cast<const bf16*>(p.v) + koff(p, b, 0, hk, D);
  const long kstride = p.kts;

  int lo_i = 0, hi_i = 0;
  if (i < Sq) keys_of(p.mask, b, i, lo_i, hi_i);
  const int ilast = min(q0 + BM, Sq) - 1;
  int lo_first, hi_first, lo_last, hi_last;
  keys_of(p.mask, b, q0, lo_first, hi_first);
  keys_of(p.mask, b, ilast, lo_last, hi_last);
  const bool dchk = dense_row(p.mask, b);
  const bool rows_full = (q0 + BM <= Sq) && !dchk;
  // BIAS: this lane's query row of the bias (Sk % 8 == 0 on this path, so a
  // run of four keys starting below Sk lies wholly inside the row)
  const bf16* brow = nullptr;
  if constexpr (BIAS)
    brow = reinterpret_cast<const bf16*>(p.bias) + b * p.bias_bs + hq * p.bias_hs + (long)min(i, Sq - 1) * Sk;

  bf16x8 qf[NCW];
  {
    const bf16* qrow =
        reinterpret_cast<const bf16*>(p.q) + qoff(p, b, min(i, Sq - 1), hq, D) + colofs;
#pragma unroll
    for (int c = 0; c < NCW; ++c) qf[c] = *reinterpret_cast<const bf16x8*>(qrow + 16 * c + 8 * h);
  }

  const bool has_sink = p.sink_mode != 0;
  const float sink2 = p.sink_mode == 2 ? p.sink[hq] * kLog2e : 0.0f;
  float m = FIXM ? lk.c2 : (has_sink ? sink2 : -INFINITY);
  const float kfix = -0.5f / lk.c2;
  float lsum = 0.0f;
  f32x16 oacc[NOB];
#pragma unroll
  for (int ob = 0; ob < NOB; ++ob) oacc[ob] = f32x16{};

  const int kbeg = (lo_first / BN) * BN;
  const int ntiles = hi_last > kbeg ? (hi_last - kbeg + BN - 1) / BN : 0;
  if (ntiles > 0) {
    load_tile<BN, D, NT, true>(sK0, kbase, kstride, kbeg, Sk);
    load_tile<BN, D, NT, false>(sV0, vbase, kstride, kbeg, Sk);
  }
  wait_loads();
  __syncthreads();

  auto step = [&](const bf16* tK, const bf16* tV, bf16* wK, bf16* wV, int t) {
    const int k0 = kbeg + t * BN;
    if (t + 1 < ntiles) {
      load_tile<BN, D, NT, true>(wK, kbase, kstride, k0 + BN, Sk);
      load_tile<BN, D, NT, false>(wV, vbase, kstride, k0 + BN, Sk);
    }
    f32x16 s = f32x16{};
#pragma unroll
    for (int c = 0; c < NCW; ++c) mma(s, fo.frag(tK, 0, 8 * sl + c), qf[c]);
    // reduce-scatter: quarter x (elements 4x .. 4x + 3, keys acc_row(h, 4x) + 0..3)
    // goes to slice x; each wave sums its own quarter in slice order
    f32x4 own = f32x4{};
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const f32x4 v = {s[4 * x], s[4 * x + 1], s[4 * x + 2], s[4 * x + 3]};
      if (x != sl) sX[((rg * 4 + x) * 3 + (sl < x ? sl : sl - 1)) * 64 + lane] = v;
      else own = v;
    }
    __syncthreads();
    f32x4 lq = f32x4{};
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      if (y == sl) lq += own;
      else lq += sX[((rg * 4 + sl) * 3 + (y < sl ? y : y - 1)) * 64 + lane];
    }
    // logits of the quarter: CAP keeps r = 1/(1+2^y) (masked: +inf), else y (masked: -inf)
    float ext = CAP ? INFINITY : -INFINITY;
    bf16x4 bq = {};
    if constexpr (BIAS) {
      const int key0 = k0 + acc_row(h, 4 * sl);
      if (key0 < Sk) bq = *reinterpret_cast<const bf16x4*>(brow + key0);
    }
    auto logits = [&](auto masked) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float y = lq[e] * lk.a;
        if constexpr (BIAS) y = fmaf((float)bq[e], lk.bb, y);
        float v;
        if constexpr (FIXM) v = __builtin_amdgcn_rcpf(fmaf(fast_exp2(y), kfix, kfix));
        else if constexpr (CAP) v = __builtin_amdgcn_rcpf(1.0f + fast_exp2(y));
        else v = y;
        if constexpr (decltype(masked)::value) {
          const int key = k0 + acc_row(h, 4 * sl + e);
          v = (key >= lo_i && key < hi_i && dense_ok(p.mask, dchk, b, i, key)) ? v : ((CAP && !FIXM) ? INFINITY : -INFINITY);
        }
        lq[e] = v;
        if constexpr (!FIXM) ext = CAP ? fminf(ext, v) : fmaxf(ext, v);
      }
    };
    if (rows_full && k0 >= lo_last && k0 + BN <= hi_first) logits(bool_c<false>{});
    else logits(bool_c<true>{});
    float base = 0.0f;
    if constexpr (!FIXM) {
      // the row's extreme over the four quarters
      ext = CAP ? fminf(ext, xor32(ext)) : fmaxf(ext, xor32(ext));
      sE[(rg * 4 + sl) * 64 + lane] = ext;
      __syncthreads();
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        const float o = sE[(rg * 4 + y) * 64 + lane];
        ext = CAP ? fminf(ext, o) : fmaxf(ext, o);
      }
      const float mx = CAP ? fmaf(ext, -2.0f * lk.c2, lk.c2) : ext;
      const bool grow = mx > m + 8.0f;
      if (__any(grow)) {
        const float m_new = grow ? mx : m;
        const float alpha = (m == -INFINITY) ? 0.0f : fast_exp2(m - m_new);
        lsum *= alpha;
#pragma unroll
        for (int ob = 0; ob < NOB; ++ob) oacc[ob] *= alpha;
        m = m_new;
      }
      base = (m == -INFINITY) ? 0.0f : m;
    }
    bf16x4 pq;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pq[e] = (bf16)(FIXM  ? fast_exp2(lq[e])
                     : CAP ? fast_exp2(fmaf(lq[e], -2.0f * lk.c2, lk.c2 - base))
                           : fast_exp2(lq[e] - base));
    }
    // the quarter's share of the row sum (of the rounded probabilities, before dropout)
    lsum = sum_bf16x4(pq, lsum);
    if constexpr (DROP) {
      const unsigned kp = keep4(p.drop, i, k0 + acc_row(h, 4 * sl), b * p.Hq + hq);
#pragma unroll
      for (int e = 0; e < 4; ++e) pq[e] = ((kp >> e) & 1u) ? pq[e] : (bf16)0.0f;
    }
    // gather the quarters: quarter sl is elements 4 (sl % 2) .. + 3 of P fragment sl / 2
    reinterpret_cast<bf16x4*>(&sP[(rg * 2 + (sl >> 1)) * 64 + lane])[sl & 1] = pq;
    __syncthreads();
    bf16x8 pf[2];
    pf[0] = sP[(rg * 2) * 64 + lane];
    pf[1] = sP[(rg * 2 + 1) * 64 + lane];
    bf16x8 tv[NOB][2];
#pragma unroll
    for (int ob = 0; ob < NOB; ++ob) {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) tv[ob][sb] = fo.frag_tr(tV + colofs, 16 * sb, ob);
    }
#pragma unroll
    for (int ob = 0; ob < NOB; ++ob) {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) mma(oacc[ob], tv[ob][sb], pf[sb]);
    }
    wait_loads();
    __syncthreads();
  };
  for (int t = 0; t < ntiles; t += 2) {
    step(sK0, sV0, sK1, sV1, t);
    if (t + 1 < ntiles) step(sK1, sV1, sK0, sV0, t + 1);
  }

  // the row sum over the four quarters, in slice order, and the two key halves
  sE[(rg * 4 + sl) * 64 + lane] = lsum;
  __syncthreads();
  float lrow = 0.0f;
#pragma unroll
  for (int y = 0; y < 4; ++y) lrow += sE[(rg * 4 + y) * 64 + lane];
  float ltot = lrow + xor32(lrow);
  float oscale = 1.0f;
  if constexpr (FIXM) {
    if (has_sink && sink2 > m) {
      oscale = fast_exp2(m - sink2);
      ltot *= oscale;
      m = sink2;
    }
  }
  if (has_sink) ltot += fast_exp2(sink2 - m);
  const float inv = ltot > 0.0f ? (DROP ? p.drop.scale : 1.0f) * oscale / ltot : 0.0f;
  if (i < Sq) {
    const long orow_off = qoff(p, b, i, hq, D) + colofs;
    bf16* orow = reinterpret_cast<bf16*>(p.out) + orow_off;
    bf16* lorow = reinterpret_cast<bf16*>(p.out_lo) + orow_off;
#pragma unroll
    for (int ob = 0; ob < NOB; ++ob) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        float vals[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) vals[e] = oacc[ob][8 * hf + e] * inv;
        store8<bf16>(orow + ob * 32 + 16 * hf + 8 * h, vals);
        if (p.out_lo) store8_lo(lorow + ob * 32 + 16 * hf + 8 * h, vals);
      }
    }
    if (h == 0 && sl == 0) p.lse[((long)b * p.Hq + hq) * Sq + i] = ltot > 0.0f ? (m + __log2f(ltot)) * kLn2 : -INFINITY;
  }
}

// ============================================================== dk, dv (D = 512)

// One workgroup = 32 keys of one KV head; wave w = 4 kg + sl holds keys
// k0 + 16 kg .. + 15 and columns 128 sl .. + 127.  Per 32-query item (one
// query head): partial S = Q K^T and dP = dO V^T over the slice's columns on
// v_mfma_f32_16x16x32_bf16 (lane: key r, queries 16 qb + 4g + e).  The
// partials are reduce-scattered across the group: wave sl sums, in slice
// order, only the quarter qb = sl / 2, e = 2 (sl % 2) .. + 1 of each lane's
// eight (key, query) pairs and takes P and dU = P (dP - delta) (1 - t^2) / 4
// for that quarter alone; the four quarters, packed to 16 bits, are then
// gathered through LDS so that every wave of the group holds all of P and
// dU.  Then dV^T += dO^T P and dK^T += Q^T dU over the slice's columns with
// Q^T, dO^T from transposing reads.  Slice 0 writes the dU block halves for
// dq.  DROP: dropout, the keep decisions shared in quads of lanes as in
// dkdv16_kernel (each wave evaluates those of its quarter).
template <bool CAP, bool DROP, bool BIAS>
__global__ __launch_bounds__(512, 1) void dkdv512_kernel(BwdParams p) {
  constexpr int D = 512, NT = 512, BNK = 32, BMQ = 32;
  constexpr int NCW = 4;   // 32-column contraction steps per slice
  constexpr int NOB = 8;   // 16-column output blocks per slice

  __shared__ __attribute__((aligned(16))) bf16 sQ0[BMQ * D];
  __shared__ __attribute__((aligned(16))) bf16 sQ1[BMQ * D];
  __shared__ __attribute__((aligned(16))) bf16 sO0[BMQ * D];
  __shared__ __attribute__((aligned(16))) bf16 sO1[BMQ * D];
  // partials for the reduce-scatter: [kg][quarter][the three other slices][lane],
  // each (S, S, dP, dP) of the quarter's two pairs
  __shared__ __attribute__((aligned(16))) f32x4 sX[2 * 4 * 3 * 64];
  // the gathered P and dU fragments: [kg][P, dU][lane]
  __shared__ __attribute__((aligned(16))) bf16x8 sPU[2 * 2 * 64];

  int kb, hk, b, split;
  {
    int grp;
    xcd_order(gridDim.x, gridDim.y * gridDim.z, kb, grp);
    const int y = grp % gridDim.y;   // the splits of one KV head are adjacent
    hk = y / p.hsplit;
    split = y % p.hsplit;
    b = grp / gridDim.y;
  }
  const int GS = p.G / p.hsplit;
  const int Sq = p.mask.Sq, Sk = p.mask.Sk;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int kg = w >> 2;
  const int sl = w & 3;
  const int colofs = 128 * sl;
  const int r = lane & 15;
  const int g = lane >> 4;
  const int qbw = sl >> 1;       // this wave's quarter: query block qbw,
  const int ew = 2 * (sl & 1);   // pairs e = ew, ew + 1
  const int k0 = kb * BNK;
  const int kw = k0 + 16 * kg;
  const int j = kw + r;
  const int jc = min(j, Sk - 1);
  const long qstride = p.qts;
  const LogitK lk(p.sl2, p.xc, p.bc, p.cl2, CAP);
  const Frag16Ofs<D> fo(lane);

  // this wave's columns of its keys' K and V rows (B operand of S, dP)
  bf16x8 kf[NCW], vf[NCW];
  {
    const long off = koff(p, b, jc, hk, D) + colofs;
    const bf16* krow = reinterpret_cast<const bf16*>(p.k) + off;
    const bf16* vrow = reinterpret_cast<const bf16*>(p.v) + off;
#pragma unroll
    for (int c = 0; c < NCW; ++c) {
      kf[c] = *reinterpret_cast<const bf16x8*>(krow + 8 * c + 32 * g);
      vf[c] = *reinterpret_cast<const bf16x8*>(vrow + 8 * c + 32 * g);
    }
  }

  int lo_j = 0, hi_j = 0;
  if (j < Sk) queries_of(p.mask, b, j, lo_j, hi_j);
  const int jlast = min(k0 + BNK, Sk) - 1;
  int lo_first, hi_first, lo_last, hi_last;
  queries_of(p.mask, b, k0, lo_first, hi_first);
  queries_of(p.mask, b, jlast, lo_last, hi_last);
  const bool dchk = dense_row(p.mask, b);
  const bool keys_full = (k0 + BNK <= Sk) && !dchk;
  const int qbeg = (lo_first / BMQ) * BMQ;
  const int nqt = hi_last > qbeg ? (hi_last - qbeg + BMQ - 1) / BMQ : 0;
  const int nitems = GS * nqt;

  f32x4 kacc[NOB], vacc[NOB];
#pragma unroll
  for (int ob = 0; ob < NOB; ++ob) { kacc[ob] = f32x4{}; vacc[ob] = f32x4{}; }

  auto head_of = [&](int it) { return hk * p.G + split * GS + it % GS; };
  auto q0_of = [&](int it) { return qbeg + (nqt - 1 - it / GS) * BMQ; };
  auto fetch = [&](int it, bf16* nQ, bf16* nO) {
    const long hoff = qoff(p, b, 0, head_of(it), D);
    const int q0 = q0_of(it);
    load_tile<BMQ, D, NT, false, true>(nQ, reinterpret_cast<const bf16*>(p.q) + hoff, qstride, q0, Sq);
    load_tile<BMQ, D, NT, false, true>(nO, reinterpret_cast<const bf16*>(p.dout) + hoff, qstride, q0, Sq);
  };
  // lse and delta of this lane's queries of the wave's quarter of item it
  // (16 qbw + 4g + ew + t), raw
  float nl[2], nd[2];
  auto get_stats = [&](int it) {
    const long row = ((long)b * p.Hq + head_of(it)) * Sq;
    const int q0 = q0_of(it);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int q = q0 + 16 * qbw + 4 * g + ew + t;
      const long li = row + min(q, Sq - 1);
      nl[t] = q < Sq ? p.lse[li] : -INFINITY;
      nd[t] = p.delta[li];
    }
  };

  if (nitems > 0) {
    fetch(0, sQ0, sO0);
    get_stats(0);
  }
  wait_loads();
  __syncthreads();

  auto step = [&](const bf16* tQ, const bf16* tO, bf16* nQ, bf16* nO, int it) {
    const bool more = it + 1 < nitems;
    const int hq = head_of(it);
    const int q0 = q0_of(it);
    // this item's stats (log2 units, folded with the cap's constant), then
    // the next item's loads
    float lc[2], md[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      lc[t] = nl[t] != -INFINITY ? (CAP ? p.cl2 : 0.0f) - nl[t] * kLog2e : -INFINITY;
      md[t] = -nd[t];
    }
    if (more) {
      fetch(it + 1, nQ, nO);
      get_stats(it + 1);
    }

    // partial S and dP over this slice's columns
    f32x4 acc[4] = {f32x4{}, f32x4{}, f32x4{}, f32x4{}};   // S qb 0, 1; dP qb 0, 1
#pragma unroll
    for (int c = 0; c < NCW; ++c) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        mma16(acc[qb], fo.frag(tQ, 16 * qb, 4 * sl + c), kf[c]);
        mma16(acc[2 + qb], fo.frag(tO, 16 * qb, 4 * sl + c), vf[c]);
      }
    }
    ATL_READ_AHEAD(8, 1, 4 * NCW);

    // reduce-scatter: quarter x (query block x / 2, pairs 2 (x % 2) .. + 1)
    // goes to slice x; each wave sums its own quarter in slice order
    f32x4 own = f32x4{};
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int qb = x >> 1, e = 2 * (x & 1);
      const f32x4 v = {acc[qb][e], acc[qb][e + 1], acc[2 + qb][e], acc[2 + qb][e + 1]};
      if (x != sl) sX[((kg * 4 + x) * 3 + (sl < x ? sl : sl - 1)) * 64 + lane] = v;
      else own = v;
    }
    __syncthreads();
    f32x4 tot = f32x4{};
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      if (y == sl) tot += own;
      else tot += sX[((kg * 4 + sl) * 3 + (y < sl ? y : y - 1)) * 64 + lane];
    }

    // dropout: bit t keeps (query q0 + 16 qbw + 4g + ew + t, key j)
    unsigned kq = 0;
    if constexpr (DROP) {
      const int t = r & 3;
      const int w4 = (int)keep4(p.drop, q0 + 16 * qbw + 4 * g + t, j & ~3, b * p.Hq + hq);
      int n0, n1;
      if (ew == 0) {
        n0 = __builtin_amdgcn_update_dpp(0, w4, 0x00, 0xF, 0xF, false);
        n1 = __builtin_amdgcn_update_dpp(0, w4, 0x55, 0xF, 0xF, false);
      } else {
        n0 = __builtin_amdgcn_update_dpp(0, w4, 0xAA, 0xF, 0xF, false);
        n1 = __builtin_amdgcn_update_dpp(0, w4, 0xFF, 0xF, 0xF, false);
      }
      kq = (unsigned)(((n0 >> t) & 1) | (((n1 >> t) & 1) << 1));
    }
    float pq[2], uq[2];
    // BIAS: the bias of this wave's two pairs, and where their dbias goes
    float bv[2] = {0.0f, 0.0f};
    const long brow0 = (long)b * p.bias_bs + hq * p.bias_hs + jc;
    if constexpr (BIAS) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int qi = q0 + 16 * qbw + 4 * g + ew + t;
        bv[t] = (float)reinterpret_cast<const bf16*>(p.bias)[brow0 + (long)min(qi, Sq - 1) * Sk];
      }
    }
    auto grads = [&](auto masked) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        float l = lc[t];
        if constexpr (decltype(masked)::value) {
          const int qi = q0 + 16 * qbw + 4 * g + ew + t;
          l = (qi >= lo_j && qi < hi_j && dense_ok(p.mask, dchk, b, qi, j)) ? l : -INFINITY;
        }
        float gg;
        const float pv = prob_fast<CAP, BIAS>(tot[t], bv[t], lk, l, gg);
        if constexpr (DROP) {
          // m dP - delta with m = keep / (1 - p); md = -delta
          const float mk = ((kq >> t) & 1u) ? p.drop.scale : 0.0f;
          pq[t] = pv * mk;
          uq[t] = pv * fmaf(mk, tot[2 + t], md[t]) * gg;
        } else {
          pq[t] = pv;
          uq[t] = pv * (tot[2 + t] + md[t]) * gg;
        }
      }
    };
    if (keys_full && q0 >= lo_last && q0 + BMQ <= hi_first) grads(bool_c<false>{});
    else grads(bool_c<true>{});
    // dbias of this wave's pairs that the visibility range covers (the pairs
    // outside it were zeroed by the fill pass); a pair the dense mask drops
    // inside the range has P = 0 and writes 0
    if constexpr (BIAS) {
      if (p.dbias && j < Sk) {
        bf16* drow = reinterpret_cast<bf16*>(p.dbias) + ((long)b * p.Hq + hq) * Sq * Sk + j;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int qi = q0 + 16 * qbw + 4 * g + ew + t;
          if (qi < Sq && qi >= lo_j && qi < hi_j) drow[(long)qi * Sk] = (bf16)(uq[t] * kGrad4<CAP>);
        }
      }
    }
    // gather the quarters: element 4 qbw + ew + t of the lane's fragments
    {
      bf16x2 pp, uu;
      pp[0] = (bf16)pq[0];
      pp[1] = (bf16)pq[1];
      uu[0] = (bf16)uq[0];
      uu[1] = (bf16)uq[1];
      reinterpret_cast<bf16x2*>(&sPU[(kg * 2) * 64 + lane])[2 * qbw + (ew >> 1)] = pp;
      reinterpret_cast<bf16x2*>(&sPU[(kg * 2 + 1) * 64 + lane])[2 * qbw + (ew >> 1)] = uu;
    }
    __syncthreads();
    const bf16x8 pf = sPU[(kg * 2) * 64 + lane];
    const bf16x8 uf = sPU[(kg * 2 + 1) * 64 + lane];
    // this key group's half of the dU block (32-key block k0, query block q0)
    if (p.du && sl == 0) {
      bf16* blk = reinterpret_cast<bf16*>(p.du) +
                  ((((long)b * p.Hq + hq) * p.nkb32 + (k0 >> 5)) * p.nqb32 + (q0 >> 5)) * 1024 + kg * 512 + lane * 8;
      __builtin_nontemporal_store(uf, reinterpret_cast<bf16x8*>(blk));
    }

    // dV^T += dO^T P, dK^T += Q^T dU over this slice's columns, transposing
    // reads two column blocks ahead of their MFMAs
    constexpr int TRA = 2;
    bf16x8 tro[TRA + 1], trq[TRA + 1];
#pragma unroll
    for (int a = 0; a < TRA; ++a) {
      tro[a] = fo.frag_tr(tO + colofs, 0, a);
      trq[a] = fo.frag_tr(tQ + colofs, 0, a);
    }
#pragma unroll
    for (int ob = 0; ob < NOB; ++ob) {
      if (ob + TRA < NOB) {
        tro[(ob + TRA) % (TRA + 1)] = fo.frag_tr(tO + colofs, 0, ob + TRA);
        trq[(ob + TRA) % (TRA + 1)] = fo.frag_tr(tQ + colofs, 0, ob + TRA);
      }
      mma16(vacc[ob], tro[ob % (TRA + 1)], pf);
      mma16(kacc[ob], trq[ob % (TRA + 1)], uf);
    }

    wait_loads();
    __syncthreads();
  };
  for (int it = 0; it < nitems; it += 2) {
    step(sQ0, sO0, sQ1, sO1, it);
    if (it + 1 < nitems) step(sQ1, sO1, sQ0, sO0, it + 1);
  }

  if (j < Sk && p.hsplit > 1) {
    const long nel = (long)gridDim.z * Sk * p.Hkv * D;
    const long off = (((long)b * Sk + j) * p.Hkv + hk) * D;
    float* kp = p.dkv_part + (long)split * nel + off;
    float* vp = p.dkv_part + (long)(p.hsplit + split) * nel + off;
#pragma unroll
    for (int ob = 0; ob < NOB; ++ob) {
      *reinterpret_cast<f32x4*>(kp + colofs + 16 * ob + 4 * g) = kacc[ob];
      *reinterpret_cast<f32x4*>(vp + colofs + 16 * ob + 4 * g) = vacc[ob];
    }
  } else if (j < Sk) {
    const long off = koff(p, b, j, hk, D);
    bf16* krow = reinterpret_cast<bf16*>(p.dk) + off;
    bf16* vrow = reinterpret_cast<bf16*>(p.dv) + off;
    const float ks = p.scale * kGrad4<CAP>;
#pragma unroll
    for (int ob = 0; ob < NOB; ++ob) {
      bf16x4 kv, vv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kv[e] = (bf16)(kacc[ob][e] * ks);
        vv[e] = (bf16)vacc[ob][e];
      }
      *reinterpret_cast<bf16x4*>(krow + colofs + 16 * ob + 4 * g) = kv;
      *reinterpret_cast<bf16x4*>(vrow + colofs + 16 * ob + 4 * g) = vv;
    }
  }
}

}  // namespace ATL_NS
