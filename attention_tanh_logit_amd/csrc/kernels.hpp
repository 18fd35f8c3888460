// gfx950 kernels of the soft-capped attention forward and backward.
//
// Forward (one workgroup per batch row, query head and tile of 32*NQG
// queries): S^T = K Q^T on MFMA, the scale / bias / tanh cap / mask in
// registers, an online softmax whose running maximum and sum start from the
// sink logit (so the sink joins each row's normaliser exactly once), and
// O^T += V^T P^T on MFMA.  Key tiles outside the visible range are never
// visited; the mask is evaluated only on tiles that are partly visible.
//
// Backward, two kernels after a row pre-pass (delta_i = <dO_i, O_i>):
//  * dq:   one workgroup per query tile, looping over its visible key tiles:
//          recompute S^T, P^T = exp(s - lse), dP^T = V dO^T,
//          dU^T = P^T (dP^T - delta) (1 - t^2), dQ^T += K^T dU^T;
//  * dkdv: one workgroup per KV head and key tile, looping over the query
//          heads of its GQA group and their visible query tiles:
//          recompute S, P, dP, dU the same way, dV^T += dO^T P,
//          dK^T += Q^T dU, and write dbias = dU on the visible pairs.
// The 1 - tanh^2 factor is formed from the unmasked logit before the mask is
// applied, and dU (the gradient with respect to the pre-cap logit u) feeds
// dq, dk and dbias alike ("Support logits soft-capping in the Pallas-Triton
// attention VJP", PR description).
//
// Head dimensions that do not fit LDS in one piece are staged in chunks of
// DC columns; a wave owns a slice of DO output columns.  The D/DO waves that
// share the same queries or keys split the logits' contraction over the head
// dimension between them and sum their partial products through LDS, where
// LDS has room for the partials; otherwise each computes the whole logits.
#pragma once

#include "common.hpp"

namespace ATL_NS {

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* bias;
  long bias_bs, bias_hs;   // bias element strides over batch rows and query heads (0: broadcast)
  void* out;
  float* lse;
  // bf16 only, nullable: out_lo = bf16(O - bf16(O)) of the fp32 output O, so
  // that out + out_lo carries O to about 16 bits and the backward's
  // delta = <dO, O> does not inherit the rounding of out
  void* out_lo;
  long qbs, qts, kbs, kts;   // element strides: batch row and token, q side and k side
  Dropout drop;
  Mask mask;
  int Hq, Hkv, G;
  float sl2;    // scale * log2(e)            (no cap)
  float xc;     // scale / softcap            (cap)
  float bc;     // 1 / softcap                (cap)
  float cl2;    // softcap * log2(e)          (cap)
  const float* sink;  // [Hq] or null
  int sink_mode;      // 0 none, 1 off-by-one, 2 learnable
  int reverse;        // visit query tiles from the last (heaviest under causal masks)
};

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* bias;
  long bias_bs, bias_hs;   // bias element strides over batch rows and query heads (0: broadcast)
  const void* dout;
  const float* lse;    // [B,Hq,Sq] natural log
  const float* delta;  // [B,Hq,Sq]
  void* dq;
  void* dk;
  void* dv;
  void* dbias;
  // 0: dbias is [B, Hq, Sq, Sk].  > 0 (a bias broadcast over heads, on the
  // 16-key dk/dv kernel): dbias is [B, dbias_np, Sq, Sk] with dbias_np =
  // grid.y = Hkv * hsplit, each workgroup column's sum over its query heads
  int dbias_np;
  // dU^T in 32-key x 32-query blocks (bf16), written by the dk/dv kernel and
  // read by the dq kernel; null when dq recomputes the probabilities itself
  void* du;
  int nkb32, nqb32;  // blocks along keys and along queries
  long qbs, qts, kbs, kts;   // element strides: batch row and token, q side and k side
  Dropout drop;
  Mask mask;
  int Hq, Hkv, G;
  float scale;
  float sl2, xc, bc, cl2;
  int reverse;
  // bf16 dk/dv kernels: the GQA group's query heads split over hsplit
  // workgroups per key block (grid.y = Hkv * hsplit); with hsplit > 1 each
  // writes unscaled fp32 partial dK, dV to dkv_part ([2][hsplit][B, Sk, Hkv, D])
  // and dkv_reduce_kernel sums them in a fixed order
  int hsplit;
  float* dkv_part;
};

// Element offset of (batch row b, token t, head h) in a q-side tensor (q, out,
// out_lo, dout, dq) or a k-side one (k, v, dk, dv): batch and token strides
// come from the layout (BSHD or SBHD), heads and columns are contiguous.
template <class P>
__device__ __forceinline__ long qoff(const P& p, int b, long t, int h, int D) {
  return b * p.qbs + t * p.qts + (long)h * D;
}
template <class P>
__device__ __forceinline__ long koff(const P& p, int b, long t, int h, int D) {
  return b * p.kbs + t * p.kts + (long)h * D;
}

template <typename T> struct Pad { static constexpr int v = 16 / sizeof(T); };

// logits in log2 units from the raw product x and the bias value b
template <typename T, bool CAP, bool BIAS>
__device__ __forceinline__ float logit2(float x, float b, float sl2, float xc, float bc, float cl2, float& f) {
  if constexpr (CAP) {
    float a = x * xc;
    if constexpr (BIAS) a = fmaf(b, bc, a);
    const float t = cap_tanh(a, (T*)nullptr);
    f = fmaf(-t, t, 1.0f);
    return t * cl2;
  } else {
    f = 1.0f;
    float a = x * sl2;
    if constexpr (BIAS) a = fmaf(b, kLog2e, a);
    return a;
  }
}

// Sum of partial accumulators over the NSL waves of one row (or key) group,
// each of which holds the contraction over its own share of the head
// dimension.  Every wave of the group gets the same total, added in slice
// order, so the waves agree bit for bit.  Wave w of the group at slice sl
// writes red[w], so red holds NW * NA * 4 KiB; the caller puts a barrier
// between two uses.
template <int NSL, int NA>
__device__ __forceinline__ void slice_sum(float* red, int w, int sl, f32x16 (&acc)[NA]) {
  const int lane = threadIdx.x & 63;
  float4* r4 = reinterpret_cast<float4*>(red);
#pragma unroll
  for (int a = 0; a < NA; ++a) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      r4[((w * NA + a) * 4 + q) * 64 + lane] = make_float4(acc[a][4 * q], acc[a][4 * q + 1], acc[a][4 * q + 2], acc[a][4 * q + 3]);
  }
  __syncthreads();
  const int g0 = w - sl;
#pragma unroll
  for (int a = 0; a < NA; ++a) acc[a] = f32x16{};
#pragma unroll
  for (int s = 0; s < NSL; ++s) {
#pragma unroll
    for (int a = 0; a < NA; ++a) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 v = r4[(((g0 + s) * NA + a) * 4 + q) * 64 + lane];
        acc[a][4 * q] += v.x;
        acc[a][4 * q + 1] += v.y;
        acc[a][4 * q + 2] += v.z;
        acc[a][4 * q + 3] += v.w;
      }
    }
  }
}

// LDS budget of a workgroup, leaving a little for the compiler's own layout
constexpr int kLdsBudget = 158 * 1024;

// ============================================================== forward

template <typename T, int D, int DO, int NQG, int BN, int DC, bool CAP, bool BIAS>
__global__ __launch_bounds__(64 * NQG * (D / DO)) void fwd_kernel(FwdParams p) {
  constexpr int NSL = D / DO;
  constexpr int NW = NQG * NSL;
  constexpr int NT = 64 * NW;
  constexpr int BM = 32 * NQG;
  constexpr int NKB = BN / 32;
  constexpr int NOB = DO / 32;
  constexpr int NCH = D / DC;
  constexpr bool ONE = (NCH == 1);
  constexpr int QS = DC + Pad<T>::v;
  constexpr int KS = DC + Pad<T>::v;
  constexpr int VS = BN + Pad<T>::v;
  static_assert(D % DO == 0 && D % DC == 0 && DO % 32 == 0 && DC % 32 == 0 && BN % 32 == 0, "tile shape");
  static_assert(ONE || DO % DC == 0, "a chunk must not straddle two slices");
  using F = typename Frag<T>::type;

  // fp32 with several column slices: each V^T stage holds one chunk per
  // slice (chunk k of every slice's columns), so that all slices have P V
  // work in every stage instead of taking turns on the chunks
  constexpr bool VPAIR = sizeof(T) == 4 && !ONE && NSL > 1;
  constexpr int VST = (VPAIR ? NSL : 1) * DC * VS;   // V^T staging elements
  // the slices of a row group split each chunk's contraction for S
  // (fp32 only: with bf16 the partial sums cost the forward more than the
  // MFMA work they save)
  constexpr bool SPLIT = sizeof(T) == 4 && !ONE && NSL > 1 && (DC / 16) % NSL == 0 &&
                         (BM * QS + BN * KS + VST) * (int)sizeof(T) + NW * NKB * 4096 <= kLdsBudget;
  constexpr int CPW = SPLIT ? DC / 16 / NSL : DC / 16;   // 16-column steps per wave and chunk
  constexpr int RED = SPLIT ? NW * NKB * 4096 : 0;
  // with the head dimension in chunks, all chunks of the Q tile stay in LDS
  // for the whole key sweep where they fit (instead of being staged again
  // for every key tile)
  constexpr bool QRES = !ONE && (NCH * BM * QS + BN * KS + VST) * (int)sizeof(T) + RED <= 150 * 1024;
  __shared__ __attribute__((aligned(16))) T sQ[(QRES ? NCH : 1) * BM * QS];
  __shared__ __attribute__((aligned(16))) T sK[BN * KS];
  __shared__ __attribute__((aligned(16))) T sV[VST];
  __shared__ __attribute__((aligned(16))) float sRed[SPLIT ? NW * NKB * 1024 : 4];

  // XCD-aware, longest-first numbering: the query tiles of a head share its K/V
  // stream through one XCD's L2
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
  const int w = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int n = lane & 31;
  const int h = lane >> 5;
  const int qg = w / NSL;
  const int sl = w % NSL;
  const int q0 = qt * BM;
  const int i = q0 + qg * 32 + n;

  const T* qbase = reinterpret_cast<const T*>(p.q) + qoff(p, b, 0, hq, D);
  const T* kbase = reinterpret_cast<const T*>(p.k) + koff(p, b, 0, hk, D);
  const T* vbase = reinterpret_cast<const T*>(p.v) + koff(p, b, 0, hk, D);
  const long qstride = p.qts;
  const long kstride = p.kts;

  // visible key range of this lane's query and of the whole tile
  int lo_i = 0, hi_i = 0;
  if (i < Sq) keys_of(p.mask, b, i, lo_i, hi_i);
  const int ilast = min(q0 + BM, Sq) - 1;
  int lo_first, hi_first, lo_last, hi_last;
  keys_of(p.mask, b, q0, lo_first, hi_first);
  keys_of(p.mask, b, ilast, lo_last, hi_last);
  const bool dchk = dense_row(p.mask, b);
  const bool rows_full = (q0 + BM <= Sq) && !dchk;

  const T* brow = nullptr;
  if constexpr (BIAS) brow = reinterpret_cast<const T*>(p.bias) + b * p.bias_bs + hq * p.bias_hs + (long)min(i, Sq - 1) * Sk;

  const bool has_sink = p.sink_mode != 0;
  const float sink2 = p.sink_mode == 2 ? p.sink[hq] * kLog2e : 0.0f;
  float m = has_sink ? sink2 : -INFINITY;
  float lsum = 0.0f;
  f32x16 oacc[NOB];
#pragma unroll
  for (int ob = 0; ob < NOB; ++ob) oacc[ob] = f32x16{};

  const int kbeg = (lo_first / BN) * BN;

  // ---- scale, bias, cap, mask; online softmax of one key tile (S -> P fragments)
  auto softmax = [&](int k0, bool full, f32x16* sacc, F (*pf)[2]) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      float bv[16];
      if constexpr (BIAS) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int j0 = k0 + kb * 32 + 16 * hf + 8 * h;
          if (i < Sq && j0 + 8 <= Sk && (Sk & 7) == 0) {
            load8(brow + j0, bv + 8 * hf);
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) bv[8 * hf + e] = (i < Sq && j0 + e < Sk) ? to_f32(brow[j0 + e]) : 0.0f;
          }
        }
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        float f;
        float s2 = logit2<T, CAP, BIAS>(sacc[kb][j], BIAS ? bv[j] : 0.0f, p.sl2, p.xc, p.bc, p.cl2, f);
        if (!full) {
          const int key = k0 + kb * 32 + acc_row(h, j);
          if (key < lo_i || key >= hi_i || !dense_ok(p.mask, dchk, b, i, key)) s2 = -INFINITY;
        }
        sacc[kb][j] = s2;
        mx = fmaxf(mx, s2);
      }
    }
    mx = fmaxf(mx, xor32(mx));
    const float m_new = fmaxf(m, mx);
    const float base = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = fast_exp2(m - base);
    float ps = 0.0f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float pv = fast_exp2(sacc[kb][j] - base);
        sacc[kb][j] = pv;
        ps += pv;
      }
      if (p.drop.on) {
        // the row sum (lse) is that of the undropped softmax; V sees the kept
        // probabilities, scaled by 1 / (1 - p) in the epilogue
        // registers 8 m + e: keys k0 + 32 kb + 16 m + 8 h + e, the eight keys of one evaluation
        const uint32_t th16 = p.drop.thresh << 16;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          uint32_t c[4];
          draw8(p.drop, i, k0 + kb * 32 + acc_row(h, 8 * m), b * p.Hq + hq, c);
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (!kept(c, e, th16)) sacc[kb][8 * m + e] = 0.0f;
        }
      }
      pf[kb][0] = to_frag(sacc[kb], 0, (T*)nullptr);
      pf[kb][1] = to_frag(sacc[kb], 8, (T*)nullptr);
    }
    lsum = lsum * alpha + ps;
    m = m_new;
#pragma unroll
    for (int ob = 0; ob < NOB; ++ob) oacc[ob] *= alpha;
  };

  if constexpr (ONE) {
  stage_rows<T, BM, DC, QS, false, NT>(sQ, qbase, qstride, q0, Sq, 0);
  for (int k0 = kbeg; k0 < hi_last; k0 += BN) {
    const bool full = rows_full && k0 >= lo_last && k0 + BN <= hi_first;
    // ---- S^T = K Q^T over the head dimension
    f32x16 sacc[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) sacc[kb] = f32x16{};
    __syncthreads();
    stage_rows<T, BN, DC, KS, true, NT>(sK, kbase, kstride, k0, Sk, 0);
    stage_rows_t<T, BN, DC, VS, true, NT>(sV, vbase, kstride, k0, Sk, 0);
    __syncthreads();
#pragma unroll
    for (int cc = 0; cc < DC / 16; ++cc) {
      const F bq = lds_frag<T>(sQ + (qg * 32 + n) * QS + cc * 16 + 8 * h);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const F ak = lds_frag<T>(sK + (kb * 32 + n) * KS + cc * 16 + 8 * h);
        mma(sacc[kb], ak, bq);
      }
    }
    F pf[NKB][2];
    softmax(k0, full, sacc, pf);
    // ---- O^T += V^T P^T over this wave's slice of the head dimension
#pragma unroll
    for (int ob = 0; ob < NOB; ++ob) {
      const int db = sl * NOB + ob;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
          const F av = lds_frag<T>(sV + (db * 32 + n) * VS + kb * 32 + 16 * sb + 8 * h);
          mma(oacc[ob], av, pf[kb][sb]);
        }
      }
    }
  }
  } else {
  // Head dimension in NCH chunks: per key tile, the chunks of K and Q (for S)
  // and then of V^T (for O) pass through LDS stage by stage; each stage's
  // global loads are issued into registers while the previous stage's MFMAs
  // run.
  const int ntile = hi_last > kbeg ? (hi_last - kbeg + BN - 1) / BN : 0;
  RowChunks<T, BN, DC, NT> rk;
  RowChunks<T, BM, DC, NT> rq;
  constexpr int NVS = VPAIR ? NSL : 1;       // V^T chunks per stage
  constexpr int CPS = DO / DC;               // chunks per slice
  constexpr int NVSTAGE = VPAIR ? CPS : NCH; // V^T stages per key tile
  RowPairChunks<T, BN, DC, NT> rvt[NVS];
  auto load_s = [&](int t, int c) {
    rk.load(kbase, kstride, kbeg + t * BN, Sk, c * DC);
    if constexpr (!QRES) rq.load(qbase, qstride, q0, Sq, c * DC);
  };
  if constexpr (QRES) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) stage_rows<T, BM, DC, QS, false, NT>(sQ + c * BM * QS, qbase, qstride, q0, Sq, c * DC);
  }
  // V^T stage c: chunk c, or (VPAIR) chunk c of every slice, slice s2's in rvt[s2]
  auto load_v = [&](int t, int c) {
#pragma unroll
    for (int s2 = 0; s2 < NVS; ++s2) rvt[s2].load(vbase, kstride, kbeg + t * BN, Sk, ((VPAIR ? s2 * CPS : 0) + c) * DC);
  };
  if (ntile > 0) load_s(0, 0);
  for (int t = 0; t < ntile; ++t) {
    const int k0 = kbeg + t * BN;
    const bool full = rows_full && k0 >= lo_last && k0 + BN <= hi_first;
    f32x16 sacc[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) sacc[kb] = f32x16{};
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      __syncthreads();
      rk.template store<KS, true>(sK);
      if constexpr (!QRES) rq.template store<QS, false>(sQ);
      __syncthreads();
      if (c + 1 < NCH) load_s(t, c + 1);
      else load_v(t, 0);
      const T* tQ = sQ + (QRES ? c * BM * QS : 0);
#pragma unroll
      for (int ci = 0; ci < CPW; ++ci) {
        const int cc = SPLIT ? ci * NSL + sl : ci;
        const F bq = lds_frag<T>(tQ + (qg * 32 + n) * QS + cc * 16 + 8 * h);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const F ak = lds_frag<T>(sK + (kb * 32 + n) * KS + cc * 16 + 8 * h);
          mma(sacc[kb], ak, bq);
        }
      }
    }
    if constexpr (SPLIT) slice_sum<NSL, NKB>(sRed, w, sl, sacc);
    F pf[NKB][2];
    softmax(k0, full, sacc, pf);
    // ---- O^T += V^T P^T over this wave's slice of the head dimension
#pragma unroll
    for (int c = 0; c < NVSTAGE; ++c) {
      __syncthreads();
#pragma unroll
      for (int s2 = 0; s2 < NVS; ++s2) rvt[s2].template store<VS, true>(sV + s2 * DC * VS);
      __syncthreads();
      if (c + 1 < NVSTAGE) load_v(t, c + 1);
      else if (t + 1 < ntile) load_s(t + 1, 0);
      // VPAIR: this slice's chunk c sits at sV + sl DC VS; else chunk c
      // belongs to slice c / CPS, at its column block (c % CPS) DC / 32
      const T* tV = sV + (VPAIR ? sl * DC * VS : 0);
      if (VPAIR || sl == c / CPS) {
#pragma unroll
        for (int db = 0; db < DC / 32; ++db) {
          const int ob = (VPAIR ? c : c % CPS) * (DC / 32) + db;
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
            for (int sb = 0; sb < 2; ++sb) {
              const F av = lds_frag<T>(tV + (db * 32 + n) * VS + kb * 32 + 16 * sb + 8 * h);
              mma(oacc[ob], av, pf[kb][sb]);
            }
          }
        }
      }
    }
  }
  }

  // ---- epilogue: normalise (the sink joins the sum once) and write
  float ltot = lsum + xor32(lsum);
  if (has_sink) ltot += fast_exp2(sink2 - m);
  const float inv = ltot > 0.0f ? (p.drop.on ? p.drop.scale : 1.0f) / ltot : 0.0f;
  if (i < Sq) {
    T* orow = reinterpret_cast<T*>(p.out) + qoff(p, b, i, hq, D);
    T* lorow = reinterpret_cast<T*>(p.out_lo) + qoff(p, b, i, hq, D);
#pragma unroll
    for (int ob = 0; ob < NOB; ++ob) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        float vals[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) vals[e] = oacc[ob][8 * hf + e] * inv;
        store8<T>(orow + sl * DO + ob * 32 + 16 * hf + 8 * h, vals);
        if constexpr (sizeof(T) == 2) {
          if (p.out_lo) store8_lo(lorow + sl * DO + ob * 32 + 16 * hf + 8 * h, vals);
        }
      }
    }
    if (sl == 0 && h == 0) {
      p.lse[((long)b * p.Hq + hq) * Sq + i] = ltot > 0.0f ? (m + __log2f(ltot)) * kLn2 : -INFINITY;
    }
  }
}

// ============================================================== backward: dq

// DU (fp32): dQ from the dU blocks the dk/dv kernel wrote (32 x 32 fp32 per
// (key block, query block), row-major [query][key]) instead of recomputing S,
// dP and the gradients: Q, dO and V are not read, and K^T comes from global
// memory without LDS.
template <typename T, int D, int DO, int NQG, int BN, int DC, bool CAP, bool BIAS, bool DU = false>
__global__ __launch_bounds__(64 * NQG * (D / DO)) void dq_kernel(BwdParams p) {
  constexpr int NSL = D / DO;
  constexpr int NW = NQG * NSL;
  constexpr int NT = 64 * NW;
  constexpr int BM = 32 * NQG;
  constexpr int NKB = BN / 32;
  constexpr int NOB = DO / 32;
  constexpr int NCH = D / DC;
  constexpr bool ONE = (NCH == 1);
  constexpr int RS = DC + Pad<T>::v;
  constexpr int TS = BN + Pad<T>::v;
  static_assert(ONE || DO % DC == 0, "a chunk must not straddle two slices");
  static_assert(!DU || sizeof(T) == 4, "dU blocks of the generic kernels are fp32");
  using F = typename Frag<T>::type;

  __shared__ __attribute__((aligned(16))) T sQ[DU ? 4 : BM * RS];
  __shared__ __attribute__((aligned(16))) T sO[DU ? 4 : BM * RS];   // dO
  __shared__ __attribute__((aligned(16))) T sK[DU ? 4 : BN * RS];
  __shared__ __attribute__((aligned(16))) T sV[DU ? 4 : BN * RS];
  __shared__ __attribute__((aligned(16))) T sKt[DU ? 4 : DC * TS];
  // the slices of a row group split each chunk's contraction for S and dP
  constexpr bool SPLIT = !DU && !ONE && NSL > 1 && (DC / 16) % NSL == 0 &&
                         (2 * BM * RS + 2 * BN * RS + DC * TS) * (int)sizeof(T) + NW * 2 * NKB * 4096 <= kLdsBudget;
  constexpr int CPW = SPLIT ? DC / 16 / NSL : DC / 16;
  __shared__ __attribute__((aligned(16))) float sRed[SPLIT ? NW * 2 * NKB * 1024 : 4];

  // XCD-aware, longest-first numbering: the query tiles of a head share its K/V
  // stream through one XCD's L2
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
  const int w = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int n = lane & 31;
  const int h = lane >> 5;
  const int qg = w / NSL;
  const int sl = w % NSL;
  const int q0 = qt * BM;
  const int i = q0 + qg * 32 + n;

  const T* qbase = reinterpret_cast<const T*>(p.q) + qoff(p, b, 0, hq, D);
  const T* obase = reinterpret_cast<const T*>(p.dout) + qoff(p, b, 0, hq, D);
  const T* kbase = reinterpret_cast<const T*>(p.k) + koff(p, b, 0, hk, D);
  const T* vbase = reinterpret_cast<const T*>(p.v) + koff(p, b, 0, hk, D);
  const long qstride = p.qts;
  const long kstride = p.kts;

  int lo_i = 0, hi_i = 0;
  if (i < Sq) keys_of(p.mask, b, i, lo_i, hi_i);
  const int ilast = min(q0 + BM, Sq) - 1;
  int lo_first, hi_first, lo_last, hi_last;
  keys_of(p.mask, b, q0, lo_first, hi_first);
  keys_of(p.mask, b, ilast, lo_last, hi_last);
  const bool dchk = dense_row(p.mask, b);
  const bool rows_full = (q0 + BM <= Sq) && !dchk;

  const long row = ((long)b * p.Hq + hq) * Sq + min(i, Sq - 1);
  const float lse_i = p.lse[row];
  // a row with no visible key and no sink has lse = -inf: its P is zero
  const float lse2 = (i < Sq && lse_i != -INFINITY) ? lse_i * kLog2e : INFINITY;
  const float delta_i = (i < Sq) ? p.delta[row] : 0.0f;
  const T* brow = nullptr;
  if constexpr (BIAS) brow = reinterpret_cast<const T*>(p.bias) + b * p.bias_bs + hq * p.bias_hs + (long)min(i, Sq - 1) * Sk;

  f32x16 qacc[NOB];
#pragma unroll
  for (int ob = 0; ob < NOB; ++ob) qacc[ob] = f32x16{};

  const int kbeg = (lo_first / BN) * BN;

  // ---- dU^T = P^T (dP^T - delta) (1 - t^2) of one key tile, as fragments
  auto grads = [&](int k0, bool full, f32x16* sacc, const f32x16* dpacc, F (*uf)[2]) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      float bv[16];
      if constexpr (BIAS) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int j0 = k0 + kb * 32 + 16 * hf + 8 * h;
          if (i < Sq && j0 + 8 <= Sk && (Sk & 7) == 0) {
            load8(brow + j0, bv + 8 * hf);
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) bv[8 * hf + e] = (i < Sq && j0 + e < Sk) ? to_f32(brow[j0 + e]) : 0.0f;
          }
        }
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        float f;
        const float s2 = logit2<T, CAP, BIAS>(sacc[kb][j], BIAS ? bv[j] : 0.0f, p.sl2, p.xc, p.bc, p.cl2, f);
        float pv = fast_exp2(s2 - lse2);
        if (!full) {
          const int key = k0 + kb * 32 + acc_row(h, j);
          if (key < lo_i || key >= hi_i || !dense_ok(p.mask, dchk, b, i, key)) pv = 0.0f;
        }
        float dp = dpacc[kb][j];
        if (p.drop.on) {
          // dP reaches the softmax through the kept, rescaled probabilities
          const int key = k0 + kb * 32 + acc_row(h, j);
          const unsigned kp = keep4(p.drop, i, key & ~3, b * p.Hq + hq);
          dp = ((kp >> (key & 3)) & 1u) ? dp * p.drop.scale : 0.0f;
        }
        sacc[kb][j] = pv * (dp - delta_i) * f;
      }
      uf[kb][0] = to_frag(sacc[kb], 0, (T*)nullptr);
      uf[kb][1] = to_frag(sacc[kb], 8, (T*)nullptr);
    }
  };

  // DU: a 32-key block is read when some query of this wave's 32-row group
  // sees one of its keys (a wave vote over the lanes' own queries); dk/dv
  // wrote every such block.  Any other block holds no visible pair of the
  // group and was not necessarily written, so it counts as zero; a query that
  // sees no key contributes nothing, wherever keys_of puts its empty interval.
  // Lane (query n, half h) takes keys 16 sb + 8 h .. + 7 of the block's row n:
  // the contraction order of the fp32 MFMA fragments (element s at key
  // 16 sb + 8 h + s).
  const int qw = q0 + qg * 32;
  int ilo = 0, ihi = 0;
  if constexpr (DU) {
    if (qw + n < Sq) keys_of(p.mask, b, qw + n, ilo, ihi);
  }
  auto load_du = [&](int k0, F (*uf)[2]) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const int kb32 = k0 + kb * 32;
      if (kb32 < Sk && __any(ilo < ihi && ilo < kb32 + 32 && ihi > kb32)) {
        const float* blk = reinterpret_cast<const float*>(p.du) +
                           ((((long)b * p.Hq + hq) * p.nkb32 + (kb32 >> 5)) * p.nqb32 + (qw >> 5)) * 1024 + n * 32 +
                           8 * h;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
          const f32x4 lo = *reinterpret_cast<const f32x4*>(blk + 16 * sb);
          const f32x4 hi = *reinterpret_cast<const f32x4*>(blk + 16 * sb + 4);
          F f;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            f[e] = lo[e];
            f[4 + e] = hi[e];
          }
          uf[kb][sb] = f;
        }
      } else {
        uf[kb][0] = F{};
        uf[kb][1] = F{};
      }
    }
  };

  if constexpr (DU) {
  // dQ^T += K^T dU^T from the dU blocks.  Each wave reads the K^T operands of
  // its own output columns straight from global memory -- lane (n, half h)
  // takes column swp(n) of each 32-column block (the order staged transposes
  // would give, which puts the accumulator rows in acc_row order) and keys
  // 16 sb + 8 h + s, s = 0..7, each load a 128-byte run of one key row --
  // so no LDS and no barrier: the slices of a row group never wait for each
  // other.
  const int ntile = hi_last > kbeg ? (hi_last - kbeg + BN - 1) / BN : 0;
  const T* kcol = kbase + sl * DO + swp(n);
  for (int t = 0; t < ntile; ++t) {
    const int k0 = kbeg + t * BN;
    F uf[NKB][2];
    load_du(k0, uf);
#pragma unroll
    for (int ob = 0; ob < NOB; ++ob) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
          F ak;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int key = k0 + kb * 32 + 16 * sb + 8 * h + e;
            ak[e] = key < Sk ? kcol[(long)key * kstride + ob * 32] : 0.0f;
          }
          mma(qacc[ob], ak, uf[kb][sb]);
        }
      }
    }
  }
  } else if constexpr (ONE) {
  stage_rows<T, BM, DC, RS, false, NT>(sQ, qbase, qstride, q0, Sq, 0);
  stage_rows<T, BM, DC, RS, false, NT>(sO, obase, qstride, q0, Sq, 0);
  for (int k0 = kbeg; k0 < hi_last; k0 += BN) {
    const bool full = rows_full && k0 >= lo_last && k0 + BN <= hi_first;
    f32x16 sacc[NKB], dpacc[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) { sacc[kb] = f32x16{}; dpacc[kb] = f32x16{}; }
    __syncthreads();
    stage_rows<T, BN, DC, RS, true, NT>(sK, kbase, kstride, k0, Sk, 0);
    stage_rows<T, BN, DC, RS, true, NT>(sV, vbase, kstride, k0, Sk, 0);
    stage_rows_t<T, BN, DC, TS, true, NT>(sKt, kbase, kstride, k0, Sk, 0);
    __syncthreads();
#pragma unroll
    for (int cc = 0; cc < DC / 16; ++cc) {
      const F bq = lds_frag<T>(sQ + (qg * 32 + n) * RS + cc * 16 + 8 * h);
      const F bo = lds_frag<T>(sO + (qg * 32 + n) * RS + cc * 16 + 8 * h);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const F ak = lds_frag<T>(sK + (kb * 32 + n) * RS + cc * 16 + 8 * h);
        mma(sacc[kb], ak, bq);
        const F av = lds_frag<T>(sV + (kb * 32 + n) * RS + cc * 16 + 8 * h);
        mma(dpacc[kb], av, bo);
      }
    }
    F uf[NKB][2];
    grads(k0, full, sacc, dpacc, uf);
    // ---- dQ^T += K^T dU^T over this wave's slice
#pragma unroll
    for (int ob = 0; ob < NOB; ++ob) {
      const int db = sl * NOB + ob;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
          const F ak = lds_frag<T>(sKt + (db * 32 + n) * TS + kb * 32 + 16 * sb + 8 * h);
          mma(qacc[ob], ak, uf[kb][sb]);
        }
      }
    }
  }
  } else {
  // Head dimension in NCH chunks: per key tile, the chunks of K, V, Q, dO
  // (for S and dP) and then of K^T (for dQ) pass through LDS stage by stage;
  // each stage's global loads are issued into registers while the previous
  // stage's MFMAs run.
  const int ntile = hi_last > kbeg ? (hi_last - kbeg + BN - 1) / BN : 0;
  RowChunks<T, BN, DC, NT> rk, rv;
  RowChunks<T, BM, DC, NT> rq, ro;
  RowPairChunks<T, BN, DC, NT> rkt;
  auto load_s = [&](int t, int c) {
    const int k0 = kbeg + t * BN;
    rk.load(kbase, kstride, k0, Sk, c * DC);
    rv.load(vbase, kstride, k0, Sk, c * DC);
    rq.load(qbase, qstride, q0, Sq, c * DC);
    ro.load(obase, qstride, q0, Sq, c * DC);
  };
  auto load_t = [&](int t, int c) { rkt.load(kbase, kstride, kbeg + t * BN, Sk, c * DC); };
  if (ntile > 0) load_s(0, 0);
  for (int t = 0; t < ntile; ++t) {
    const int k0 = kbeg + t * BN;
    const bool full = rows_full && k0 >= lo_last && k0 + BN <= hi_first;
    f32x16 sacc[NKB], dpacc[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) { sacc[kb] = f32x16{}; dpacc[kb] = f32x16{}; }
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      __syncthreads();
      rk.template store<RS, true>(sK);
      rv.template store<RS, true>(sV);
      rq.template store<RS, false>(sQ);
      ro.template store<RS, false>(sO);
      __syncthreads();
      if (c + 1 < NCH) load_s(t, c + 1);
      else load_t(t, 0);
#pragma unroll
      for (int ci = 0; ci < CPW; ++ci) {
        const int cc = SPLIT ? ci * NSL + sl : ci;
        const F bq = lds_frag<T>(sQ + (qg * 32 + n) * RS + cc * 16 + 8 * h);
        const F bo = lds_frag<T>(sO + (qg * 32 + n) * RS + cc * 16 + 8 * h);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const F ak = lds_frag<T>(sK + (kb * 32 + n) * RS + cc * 16 + 8 * h);
          mma(sacc[kb], ak, bq);
          const F av = lds_frag<T>(sV + (kb * 32 + n) * RS + cc * 16 + 8 * h);
          mma(dpacc[kb], av, bo);
        }
      }
    }
    if constexpr (SPLIT) {
      f32x16 sd[2 * NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) { sd[kb] = sacc[kb]; sd[NKB + kb] = dpacc[kb]; }
      slice_sum<NSL, 2 * NKB>(sRed, w, sl, sd);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) { sacc[kb] = sd[kb]; dpacc[kb] = sd[NKB + kb]; }
    }
    F uf[NKB][2];
    grads(k0, full, sacc, dpacc, uf);
    // ---- dQ^T += K^T dU^T over this wave's slice
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      __syncthreads();
      rkt.template store<TS, true>(sKt);
      __syncthreads();
      if (c + 1 < NCH) load_t(t, c + 1);
      else if (t + 1 < ntile) load_s(t + 1, 0);
      // chunk c belongs to slice c / (DO / DC), at its column block (c % (DO / DC)) DC / 32
      constexpr int CPS = DO / DC;
      if (sl == c / CPS) {
#pragma unroll
        for (int db = 0; db < DC / 32; ++db) {
          const int ob = (c % CPS) * (DC / 32) + db;
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
            for (int sb = 0; sb < 2; ++sb) {
              const F ak = lds_frag<T>(sKt + (db * 32 + n) * TS + kb * 32 + 16 * sb + 8 * h);
              mma(qacc[ob], ak, uf[kb][sb]);
            }
          }
        }
      }
    }
  }
  }

  if (i < Sq) {
    T* drow = reinterpret_cast<T*>(p.dq) + qoff(p, b, i, hq, D);
#pragma unroll
    for (int ob = 0; ob < NOB; ++ob) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        float vals[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) vals[e] = qacc[ob][8 * hf + e] * p.scale;
        store8<T>(drow + sl * DO + ob * 32 + 16 * hf + 8 * h, vals);
      }
    }
  }
}

// ============================================================== backward: dk, dv, dbias

template <typename T, int D, int DO, int NKG, int DC, bool CAP, bool BIAS>
__global__ __launch_bounds__(64 * NKG * (D / DO)) void dkdv_kernel(BwdParams p) {
  constexpr int NSL = D / DO;
  constexpr int NW = NKG * NSL;
  constexpr int NT = 64 * NW;
  constexpr int BNK = 32 * NKG;
  constexpr int BMQ = 32;
  constexpr int NOB = DO / 32;
  constexpr int NCH = D / DC;
  constexpr bool ONE = (NCH == 1);
  constexpr int RS = DC + Pad<T>::v;
  constexpr int TS = BMQ + Pad<T>::v;
  static_assert(ONE || DO % DC == 0, "a chunk must not straddle two slices");
  using F = typename Frag<T>::type;

  // the slices of a key group split each chunk's contraction for S and dP
  constexpr bool SPLIT = !ONE && NSL > 1 && (DC / 16) % NSL == 0 &&
                         (2 * BNK * RS + 2 * BMQ * RS + 2 * DC * TS) * (int)sizeof(T) + NW * 2 * 4096 <= kLdsBudget;
  constexpr int CPW = SPLIT ? DC / 16 / NSL : DC / 16;
  constexpr int RED = SPLIT ? NW * 2 * 4096 : 0;
  // bf16 with split logits: a wave needs only its share of the columns of K
  // and V (NCH * CPW fragments of each, 4 registers apiece), which it keeps
  // in registers for the whole sweep instead of staging K and V per item
  constexpr bool KVREG = SPLIT && sizeof(T) == 2;
  // fp32 with one chunk per slice (D = 256, 512): every slice reads the Q^T
  // and dO^T operands of its own columns straight from global memory (each
  // load a 128-byte run of one query row, mostly L2 hits after the S/dP
  // stages) instead of staging them.  Staged one chunk at a time (where all
  // do not fit, D = 512) each chunk stage would fall to the one slice owning
  // its columns, the other SIMDs waiting at the stage barriers; kept all in
  // LDS (D = 256) they would hold 74 KiB and one workgroup per CU.
  constexpr bool TDIRECT = !ONE && sizeof(T) == 4 && DO == DC;
  // Otherwise, with the head dimension in chunks and LDS to spare, the Q^T
  // and dO^T chunks of an item all stay in LDS: staged with Q and dO (the
  // same global lines, loaded back to back) instead of read again for the
  // gradient stages.  (Keeping the key block's K and V chunks in LDS
  // instead, where only one of the two fits, was slower.)
  constexpr bool QTALL = !TDIRECT && !ONE &&
                         (2 * BNK * RS + 2 * BMQ * RS + 2 * NCH * DC * TS) * (int)sizeof(T) + RED <= 150 * 1024;
  __shared__ __attribute__((aligned(16))) T sK[BNK * RS];
  __shared__ __attribute__((aligned(16))) T sV[BNK * RS];
  __shared__ __attribute__((aligned(16))) T sQ[BMQ * RS];
  __shared__ __attribute__((aligned(16))) T sO[BMQ * RS];
  __shared__ __attribute__((aligned(16))) T sQt[TDIRECT ? 4 : (QTALL ? NCH : 1) * DC * TS];
  __shared__ __attribute__((aligned(16))) T sOt[TDIRECT ? 4 : (QTALL ? NCH : 1) * DC * TS];
  __shared__ __attribute__((aligned(16))) float sL[BMQ];
  __shared__ __attribute__((aligned(16))) float sDl[BMQ];
  __shared__ __attribute__((aligned(16))) float sRed[SPLIT ? NW * 2 * 1024 : 4];

  // XCD-aware numbering: neighbouring key blocks of a KV head, which see mostly
  // the same query tiles, run on one XCD and share them through its L2
  int kt, hk, b;
  {
    int grp;
    xcd_order(gridDim.x, gridDim.y * gridDim.z, kt, grp);
    hk = grp % gridDim.y;
    b = grp / gridDim.y;
  }
  const int Sq = p.mask.Sq, Sk = p.mask.Sk;
  const int w = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int n = lane & 31;
  const int h = lane >> 5;
  const int kg = w / NSL;
  const int sl = w % NSL;
  const int k0 = kt * BNK;
  const int j = k0 + kg * 32 + n;

  const T* kbase = reinterpret_cast<const T*>(p.k) + koff(p, b, 0, hk, D);
  const T* vbase = reinterpret_cast<const T*>(p.v) + koff(p, b, 0, hk, D);
  const long qstride = p.qts;
  const long kstride = p.kts;

  // queries that see this lane's key, and the query range of the whole tile
  int lo_j = 0, hi_j = 0;
  if (j < Sk) queries_of(p.mask, b, j, lo_j, hi_j);
  const int jlast = min(k0 + BNK, Sk) - 1;
  int lo_first, hi_first, lo_last, hi_last;
  queries_of(p.mask, b, k0, lo_first, hi_first);
  queries_of(p.mask, b, jlast, lo_last, hi_last);
  const bool dchk = dense_row(p.mask, b);
  const bool keys_full = (k0 + BNK <= Sk) && !dchk;

  f32x16 kacc[NOB], vacc[NOB];
#pragma unroll
  for (int ob = 0; ob < NOB; ++ob) { kacc[ob] = f32x16{}; vacc[ob] = f32x16{}; }

  if constexpr (ONE) {
    stage_rows<T, BNK, DC, RS, false, NT>(sK, kbase, kstride, k0, Sk, 0);
    stage_rows<T, BNK, DC, RS, false, NT>(sV, vbase, kstride, k0, Sk, 0);
  }

  const int qbeg = (lo_first / BMQ) * BMQ;

  // fp32 dU hand-off (p.du): this key group's 32 x 32 block of the item,
  // row-major [query][key] so that the dq kernel's lanes read whole runs of
  // keys; nullptr for 16-bit elements, without the hand-off, or for a key
  // group past the last key.  Every lane stores its own key's column, so each
  // store instruction writes 32 consecutive floats of two query rows.
  auto du_block = [&](int hq, int q0) -> float* {
    if constexpr (sizeof(T) == 4) {
      const int kb32 = k0 + kg * 32;
      if (!p.du || kb32 >= Sk) return nullptr;
      return reinterpret_cast<float*>(p.du) +
             ((((long)b * p.Hq + hq) * p.nkb32 + (kb32 >> 5)) * p.nqb32 + (q0 >> 5)) * 1024;
    } else {
      return nullptr;
    }
  };
  // ---- P, dU of one (query head, 32-query tile) item from S and dP
  // (lane: key j; register r: query q0 + acc_row(h, r)), as operand fragments
  auto grads = [&](int hq, int q0, bool full, f32x16& sacc, f32x16& dpacc, F* pf, F* uf) {
    // Explicit wait states between the last MFMA of the S / dP chains and
    // the reads of their results: on the branch that skips the visibility
    // test (a fully visible item) the compiler left about 8 after a 16-pass
    // fp32 MFMA, and that instantiation (fp32, D = 64, no cap, no bias)
    // read stale dP values under dropout (dk off by 0.2; exact with these).
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    const long lrow = ((long)b * p.Hq + hq) * Sq;
    const T* bbase = nullptr;
    T* dbbase = nullptr;
    if constexpr (BIAS) {
      bbase = reinterpret_cast<const T*>(p.bias) + b * p.bias_bs + hq * p.bias_hs;
      if (p.dbias) dbbase = reinterpret_cast<T*>(p.dbias) + lrow * Sk;
    }
    float* ublk = du_block(hq, q0);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qi = q0 + acc_row(h, r);
      float bvv = 0.0f;
      if constexpr (BIAS) bvv = (qi < Sq && j < Sk) ? to_f32(bbase[(long)qi * Sk + j]) : 0.0f;
      float f;
      const float s2 = logit2<T, CAP, BIAS>(sacc[r], bvv, p.sl2, p.xc, p.bc, p.cl2, f);
      float pv = fast_exp2(s2 - sL[acc_row(h, r)]);
      bool vis = true;
      if (!full) vis = (qi >= lo_j && qi < hi_j);
      // a pair the dense mask removes inside the range gets P = 0 and a dbias of 0
      if (!vis || (!full && !dense_ok(p.mask, dchk, b, qi, j))) pv = 0.0f;
      float dp = dpacc[r], pd = pv;
      if (p.drop.on) {
        // V and dP see the kept probabilities, scaled by 1 / (1 - p)
        const unsigned kp = keep4(p.drop, qi, j & ~3, b * p.Hq + hq);
        const float kd = ((kp >> (j & 3)) & 1u) ? p.drop.scale : 0.0f;
        dp *= kd;
        pd *= kd;
      }
      const float du = pv * (dp - sDl[acc_row(h, r)]) * f;
      sacc[r] = pd;
      dpacc[r] = du;
      if constexpr (BIAS) {
        if (dbbase && sl == 0 && vis && qi < Sq && j < Sk) dbbase[(long)qi * Sk + j] = (T)du;
      }
      if constexpr (sizeof(T) == 4) {
        if (ublk && sl == 0) __builtin_nontemporal_store(du, ublk + acc_row(h, r) * 32 + n);
      }
    }
    pf[0] = to_frag(sacc, 0, (T*)nullptr);
    pf[1] = to_frag(sacc, 8, (T*)nullptr);
    uf[0] = to_frag(dpacc, 0, (T*)nullptr);
    uf[1] = to_frag(dpacc, 8, (T*)nullptr);
  };
  // SPLIT over four slices: the partial S and dP are reduce-scattered over the
  // key group's slices instead of summed by each (slice_sum): slice sl adds up,
  // in slice order (the same totals, bit for bit), only accumulator registers
  // 4 sl .. 4 sl + 3 of each lane -- query rows acc_row(h, 4 sl) + 0..3 of its
  // key -- and takes P and dU of those alone; the quarters (fp32, before the
  // operand rounding) are then gathered back, so every slice holds the whole
  // operand fragments and the elementwise work is done once per key group.
  // sRed: [kg][quarter][the three other slices][S, dP][lane] float4 partials,
  // then [kg][P, dU][quarter][lane] float4 gathered values (NW * 8 KiB).
  auto grads_rs = [&](int hq, int q0, bool full, f32x16& sacc, f32x16& dpacc, F* pf, F* uf) {
    // the same explicit wait states after the S / dP MFMAs as in grads
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    float4* r4 = reinterpret_cast<float4*>(sRed);
    float4* g4 = r4 + NKG * 4 * 3 * 2 * 64;
    float4 os = make_float4(0.0f, 0.0f, 0.0f, 0.0f), od = os;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const float4 vs = make_float4(sacc[4 * x], sacc[4 * x + 1], sacc[4 * x + 2], sacc[4 * x + 3]);
      const float4 vd = make_float4(dpacc[4 * x], dpacc[4 * x + 1], dpacc[4 * x + 2], dpacc[4 * x + 3]);
      if (x != sl) {
        const int base = ((kg * 4 + x) * 3 + (sl < x ? sl : sl - 1)) * 2;
        r4[base * 64 + lane] = vs;
        r4[(base + 1) * 64 + lane] = vd;
      } else {
        os = vs;
        od = vd;
      }
    }
    __syncthreads();
    float ts[4] = {0.0f, 0.0f, 0.0f, 0.0f}, td[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      float4 vs, vd;
      if (y == sl) {
        vs = os;
        vd = od;
      } else {
        const int base = ((kg * 4 + sl) * 3 + (y < sl ? y : y - 1)) * 2;
        vs = r4[base * 64 + lane];
        vd = r4[(base + 1) * 64 + lane];
      }
      ts[0] += vs.x; ts[1] += vs.y; ts[2] += vs.z; ts[3] += vs.w;
      td[0] += vd.x; td[1] += vd.y; td[2] += vd.z; td[3] += vd.w;
    }
    const long lrow = ((long)b * p.Hq + hq) * Sq;
    const T* bbase = nullptr;
    T* dbbase = nullptr;
    if constexpr (BIAS) {
      bbase = reinterpret_cast<const T*>(p.bias) + b * p.bias_bs + hq * p.bias_hs;
      if (p.dbias) dbbase = reinterpret_cast<T*>(p.dbias) + lrow * Sk;
    }
    float* ublk = du_block(hq, q0);
    float ps[4], us[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 16 * (sl >> 1) + 8 * h + 4 * (sl & 1) + e;   // acc_row(h, 4 sl + e)
      const int qi = q0 + row;
      float bvv = 0.0f;
      if constexpr (BIAS) bvv = (qi < Sq && j < Sk) ? to_f32(bbase[(long)qi * Sk + j]) : 0.0f;
      float f;
      const float s2 = logit2<T, CAP, BIAS>(ts[e], bvv, p.sl2, p.xc, p.bc, p.cl2, f);
      float pv = fast_exp2(s2 - sL[row]);
      bool vis = true;
      if (!full) vis = (qi >= lo_j && qi < hi_j);
      if (!vis || (!full && !dense_ok(p.mask, dchk, b, qi, j))) pv = 0.0f;
      float dp = td[e], pd = pv;
      if (p.drop.on) {
        const unsigned kp = keep4(p.drop, qi, j & ~3, b * p.Hq + hq);
        const float kd = ((kp >> (j & 3)) & 1u) ? p.drop.scale : 0.0f;
        dp *= kd;
        pd *= kd;
      }
      const float du = pv * (dp - sDl[row]) * f;
      ps[e] = pd;
      us[e] = du;
      if constexpr (BIAS) {
        if (dbbase && vis && qi < Sq && j < Sk) dbbase[(long)qi * Sk + j] = (T)du;
      }
      if constexpr (sizeof(T) == 4) {
        if (ublk) __builtin_nontemporal_store(du, ublk + row * 32 + n);
      }
    }
    g4[((kg * 2) * 4 + sl) * 64 + lane] = make_float4(ps[0], ps[1], ps[2], ps[3]);
    g4[((kg * 2 + 1) * 4 + sl) * 64 + lane] = make_float4(us[0], us[1], us[2], us[3]);
    __syncthreads();
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const float4 a = g4[((kg * 2) * 4 + x) * 64 + lane];
      const float4 c = g4[((kg * 2 + 1) * 4 + x) * 64 + lane];
      sacc[4 * x] = a.x; sacc[4 * x + 1] = a.y; sacc[4 * x + 2] = a.z; sacc[4 * x + 3] = a.w;
      dpacc[4 * x] = c.x; dpacc[4 * x + 1] = c.y; dpacc[4 * x + 2] = c.z; dpacc[4 * x + 3] = c.w;
    }
    pf[0] = to_frag(sacc, 0, (T*)nullptr);
    pf[1] = to_frag(sacc, 8, (T*)nullptr);
    uf[0] = to_frag(dpacc, 0, (T*)nullptr);
    uf[1] = to_frag(dpacc, 8, (T*)nullptr);
  };
  // lse (log2 units; +inf on rows past the end) and delta of the item's queries
  auto put_stats = [&](int i, float l, float dl) {
    if (threadIdx.x < BMQ) {
      sL[threadIdx.x] = (i < Sq && l != -INFINITY) ? l * kLog2e : INFINITY;
      sDl[threadIdx.x] = i < Sq ? dl : 0.0f;
    }
  };
  auto get_stats = [&](int hq, int q0, float& l, float& dl) {
    l = -INFINITY;
    dl = 0.0f;
    const int qi = q0 + (int)threadIdx.x;
    if (threadIdx.x < BMQ && qi < Sq) {
      const long lrow = ((long)b * p.Hq + hq) * Sq;
      l = p.lse[lrow + qi];
      dl = p.delta[lrow + qi];
    }
  };

  if constexpr (ONE) {
  for (int g = 0; g < p.G; ++g) {
    const int hq = hk * p.G + g;
    const T* qbase = reinterpret_cast<const T*>(p.q) + qoff(p, b, 0, hq, D);
    const T* obase = reinterpret_cast<const T*>(p.dout) + qoff(p, b, 0, hq, D);
    for (int q0 = qbeg; q0 < hi_last; q0 += BMQ) {
      const bool full = keys_full && q0 >= lo_last && q0 + BMQ <= hi_first;
      f32x16 sacc = f32x16{}, dpacc = f32x16{};
      __syncthreads();
      stage_rows<T, BMQ, DC, RS, true, NT>(sQ, qbase, qstride, q0, Sq, 0);
      stage_rows<T, BMQ, DC, RS, true, NT>(sO, obase, qstride, q0, Sq, 0);
      stage_rows_t<T, BMQ, DC, TS, true, NT>(sQt, qbase, qstride, q0, Sq, 0);
      stage_rows_t<T, BMQ, DC, TS, true, NT>(sOt, obase, qstride, q0, Sq, 0);
      {
        float l, dl;
        get_stats(hq, q0, l, dl);
        put_stats(q0 + (int)threadIdx.x, l, dl);
      }
      __syncthreads();
#pragma unroll
      for (int cc = 0; cc < DC / 16; ++cc) {
        const F aq = lds_frag<T>(sQ + n * RS + cc * 16 + 8 * h);
        const F bk = lds_frag<T>(sK + (kg * 32 + n) * RS + cc * 16 + 8 * h);
        mma(sacc, aq, bk);
        const F ao = lds_frag<T>(sO + n * RS + cc * 16 + 8 * h);
        const F bv = lds_frag<T>(sV + (kg * 32 + n) * RS + cc * 16 + 8 * h);
        mma(dpacc, ao, bv);
      }
      F pf[2], uf[2];
      grads(hq, q0, full, sacc, dpacc, pf, uf);
      // ---- dV^T += dO^T P,  dK^T += Q^T dU  over this wave's slice
#pragma unroll
      for (int ob = 0; ob < NOB; ++ob) {
        const int db = sl * NOB + ob;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
          const F ao = lds_frag<T>(sOt + (db * 32 + n) * TS + 16 * sb + 8 * h);
          mma(vacc[ob], ao, pf[sb]);
          const F aq = lds_frag<T>(sQt + (db * 32 + n) * TS + 16 * sb + 8 * h);
          mma(kacc[ob], aq, uf[sb]);
        }
      }
    }
  }
  } else {
  // Head dimension in NCH chunks: every chunk of Q, dO, K, V (for S and dP)
  // and then of Q^T, dO^T (for dV, dK) passes through LDS, one stage after
  // the other; each stage's global loads are issued into registers while the
  // previous stage's MFMAs run, across the items of the (query head,
  // 32-query tile) sweep.
  const int nqt = hi_last > qbeg ? (hi_last - qbeg + BMQ - 1) / BMQ : 0;
  const int nitems = p.G * nqt;
  auto head_of = [&](int it) { return hk * p.G + it / nqt; };
  auto q0_of = [&](int it) { return qbeg + (it % nqt) * BMQ; };
  auto qb_of = [&](int hq) { return reinterpret_cast<const T*>(p.q) + qoff(p, b, 0, hq, D); };
  auto ob_of = [&](int hq) { return reinterpret_cast<const T*>(p.dout) + qoff(p, b, 0, hq, D); };
  RowChunks<T, BMQ, DC, NT> rq, ro;
  RowChunks<T, BNK, DC, NT> rk, rv;
  RowPairChunks<T, BMQ, DC, NT> rqt, rot;
  float nl = -INFINITY, ndl = 0.0f;
  auto load_s = [&](int it, int c) {   // stage c of S / dP
    const int hq = head_of(it), q0 = q0_of(it);
    rq.load(qb_of(hq), qstride, q0, Sq, c * DC);
    ro.load(ob_of(hq), qstride, q0, Sq, c * DC);
    if constexpr (QTALL) {
      rqt.load(qb_of(hq), qstride, q0, Sq, c * DC);
      rot.load(ob_of(hq), qstride, q0, Sq, c * DC);
    }
    if constexpr (!KVREG) {
      rk.load(kbase, kstride, k0, Sk, c * DC);
      rv.load(vbase, kstride, k0, Sk, c * DC);
    }
    if (c == 0) get_stats(hq, q0, nl, ndl);
  };
  auto load_t = [&](int it, int c) {   // stage c of dV / dK
    const int hq = head_of(it), q0 = q0_of(it);
    rqt.load(qb_of(hq), qstride, q0, Sq, c * DC);
    rot.load(ob_of(hq), qstride, q0, Sq, c * DC);
  };
  F kf[KVREG ? NCH * CPW : 1], vf[KVREG ? NCH * CPW : 1];
  if constexpr (KVREG) {
    // lane (n, h) holds K, V row j, columns c DC + (ci NSL + sl) 16 + 8 h .. + 8
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
#pragma unroll
      for (int ci = 0; ci < CPW; ++ci) {
        const long off = (long)j * kstride + c * DC + (ci * NSL + sl) * 16 + 8 * h;
        kf[c * CPW + ci] = j < Sk ? *reinterpret_cast<const F*>(kbase + off) : F{};
        vf[c * CPW + ci] = j < Sk ? *reinterpret_cast<const F*>(vbase + off) : F{};
      }
    }
  }
  if (nitems > 0) load_s(0, 0);
  for (int it = 0; it < nitems; ++it) {
    const int hq = head_of(it), q0 = q0_of(it);
    const bool full = keys_full && q0 >= lo_last && q0 + BMQ <= hi_first;
    f32x16 sacc = f32x16{}, dpacc = f32x16{};
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      __syncthreads();
      rq.template store<RS, true>(sQ);
      ro.template store<RS, true>(sO);
      if constexpr (!KVREG) {
        rk.template store<RS, false>(sK);
        rv.template store<RS, false>(sV);
      }
      if constexpr (QTALL) {
        rqt.template store<TS, true>(sQt + c * DC * TS);
        rot.template store<TS, true>(sOt + c * DC * TS);
      }
      if (c == 0) put_stats(q0 + (int)threadIdx.x, nl, ndl);
      __syncthreads();
      if (c + 1 < NCH) {
        load_s(it, c + 1);
      } else if constexpr (QTALL || TDIRECT) {
        if (it + 1 < nitems) load_s(it + 1, 0);
      } else {
        load_t(it, 0);
      }
#pragma unroll
      for (int ci = 0; ci < CPW; ++ci) {
        const int cc = SPLIT ? ci * NSL + sl : ci;
        const F aq = lds_frag<T>(sQ + n * RS + cc * 16 + 8 * h);
        const F bk = KVREG ? kf[KVREG ? c * CPW + ci : 0] : lds_frag<T>(sK + (kg * 32 + n) * RS + cc * 16 + 8 * h);
        mma(sacc, aq, bk);
        const F ao = lds_frag<T>(sO + n * RS + cc * 16 + 8 * h);
        const F bv = KVREG ? vf[KVREG ? c * CPW + ci : 0] : lds_frag<T>(sV + (kg * 32 + n) * RS + cc * 16 + 8 * h);
        mma(dpacc, ao, bv);
      }
    }
    F pf[2], uf[2];
    if constexpr (SPLIT && NSL == 4) {
      grads_rs(hq, q0, full, sacc, dpacc, pf, uf);
    } else {
      if constexpr (SPLIT) {
        f32x16 sd[2] = {sacc, dpacc};
        slice_sum<NSL, 2>(sRed, w, sl, sd);
        sacc = sd[0];
        dpacc = sd[1];
      }
      grads(hq, q0, full, sacc, dpacc, pf, uf);
    }
    // ---- dV^T += dO^T P,  dK^T += Q^T dU  over this wave's slice
    if constexpr (TDIRECT) {
      // lane (n, half h) takes column swp(n) of block db (the staged
      // transposes store column c at row swp(c), which puts the accumulator
      // rows in acc_row order) and queries 16 sb + 8 h + s, s = 0..7
      const T* qg = qb_of(hq) + sl * DO + swp(n);
      const T* og = ob_of(hq) + sl * DO + swp(n);
#pragma unroll
      for (int db = 0; db < NOB; ++db) {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
          F ao, aq;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int qi = q0 + 16 * sb + 8 * h + e;
            const long off = (long)min(qi, Sq - 1) * qstride + db * 32;
            ao[e] = qi < Sq ? og[off] : 0.0f;
            aq[e] = qi < Sq ? qg[off] : 0.0f;
          }
          mma(vacc[db], ao, pf[sb]);
          mma(kacc[db], aq, uf[sb]);
        }
      }
    } else
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      if constexpr (!QTALL) {
        __syncthreads();
        rqt.template store<TS, true>(sQt);
        rot.template store<TS, true>(sOt);
        __syncthreads();
        if (c + 1 < NCH) load_t(it, c + 1);
        else if (it + 1 < nitems) load_s(it + 1, 0);
      }
      const T* tQt = sQt + (QTALL ? c * DC * TS : 0);
      const T* tOt = sOt + (QTALL ? c * DC * TS : 0);
      // chunk c belongs to slice c / (DO / DC), at its column block (c % (DO / DC)) DC / 32
      constexpr int CPS = DO / DC;
      if (sl == c / CPS) {
#pragma unroll
        for (int db = 0; db < DC / 32; ++db) {
          const int ob = (c % CPS) * (DC / 32) + db;
#pragma unroll
          for (int sb = 0; sb < 2; ++sb) {
            const F ao = lds_frag<T>(tOt + (db * 32 + n) * TS + 16 * sb + 8 * h);
            mma(vacc[ob], ao, pf[sb]);
            const F aq = lds_frag<T>(tQt + (db * 32 + n) * TS + 16 * sb + 8 * h);
            mma(kacc[ob], aq, uf[sb]);
          }
        }
      }
    }
  }
  }

  if (j < Sk) {
    T* krow = reinterpret_cast<T*>(p.dk) + koff(p, b, j, hk, D);
    T* vrow = reinterpret_cast<T*>(p.dv) + koff(p, b, j, hk, D);
#pragma unroll
    for (int ob = 0; ob < NOB; ++ob) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        float kv[8], vv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          kv[e] = kacc[ob][8 * hf + e] * p.scale;
          vv[e] = vacc[ob][8 * hf + e];
        }
        const int d = sl * DO + ob * 32 + 16 * hf + 8 * h;
        store8<T>(krow + d, kv);
        store8<T>(vrow + d, vv);
      }
    }
  }
}

// ============================================================== small kernels

// delta_i = <dO_i, O_i> per row; per-block partial sums of the sink gradient
// -sum_i exp(sigma - lse_i) delta_i (summed in a fixed order afterwards).
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const T* out, const T* out_lo, const T* dout, const float* lse, float* delta,
                                                      float* dsink_part, const float* sink, int sink_mode, int Sq,
                                                      int Hq, int rows_per_block, long qbs, long qts) {
  constexpr int LPR = D / 8;            // lanes per row, 8 elements each
  constexpr int RPP = 256 / LPR;        // rows per pass
  const int hq = blockIdx.y;
  const int b = blockIdx.z;
  const int r0 = blockIdx.x * rows_per_block;
  const int t = threadIdx.x;
  const int sub = t % LPR;
  const int rr = t / LPR;
  float part = 0.0f;
  const float sig = (sink_mode == 2) ? sink[hq] : 0.0f;
  for (int base = 0; base < rows_per_block; base += RPP) {
    const int i = r0 + base + rr;
    float s = 0.0f;
    if (base + rr < rows_per_block && i < Sq) {
      const long off = b * qbs + i * qts + (long)hq * D + sub * 8;
      float a[8], c[8];
      load8(out + off, a);
      load8(dout + off, c);
      if (out_lo) {
        float lo[8];
        load8(out_lo + off, lo);
#pragma unroll
        for (int e = 0; e < 8; ++e) s = fmaf(lo[e], c[e], s);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) s = fmaf(a[e], c[e], s);
    }
#pragma unroll
    for (int o = LPR / 2; o >= 1; o >>= 1) s += __shfl_xor(s, o, 64);
    if (sub == 0 && base + rr < rows_per_block && i < Sq) {
      const long li = ((long)b * Hq + hq) * Sq + i;
      delta[li] = s;
      if (sink_mode == 2) {
        const float l = lse[li];
        part -= (l == -INFINITY) ? 0.0f : expf(sig - l) * s;
      }
    }
  }
  if (sink_mode != 2) return;
  __shared__ float red[256];
  red[t] = part;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (t < s) red[t] += red[t + s];
    __syncthreads();
  }
  if (t == 0) dsink_part[((long)hq * gridDim.z + b) * gridDim.x + blockIdx.x] = red[0];
}

// The gradient of a bias broadcast over batch rows (bcast & 1) and/or query
// heads (bcast & 2): the full [B, Hq, Sq*Sk] gradient summed over those
// dimensions, in fp32 and in a fixed order, into out [Bb, Hb, Sq*Sk].
template <typename T>
__global__ __launch_bounds__(256) void dbias_reduce_kernel(const T* full, T* out, int B, int Hq, long SS, int bcast) {
  const int Hb = (bcast & 2) ? 1 : Hq;
  const int Bb = (bcast & 1) ? 1 : B;
  const long x = (long)blockIdx.x * 256 + threadIdx.x;
  if (x >= (long)Bb * Hb * SS) return;
  const long e = x % SS;
  const int hb = (int)((x / SS) % Hb);
  const int bb = (int)(x / SS / Hb);
  const int b0 = (bcast & 1) ? 0 : bb, b1 = (bcast & 1) ? B : bb + 1;
  const int h0 = (bcast & 2) ? 0 : hb, h1 = (bcast & 2) ? Hq : hb + 1;
  float s = 0.0f;
  for (int b = b0; b < b1; ++b)
    for (int h = h0; h < h1; ++h) s += to_f32(full[((long)b * Hq + h) * SS + e]);
  out[x] = (T)s;
}

// The same with 8 consecutive elements per thread, as 16-byte loads and
// stores (8 elements never straddle two [Sq, Sk] slabs when SS % 8 == 0;
// both buffers 16-byte aligned): the reduction streams at the HBM rate
// instead of issuing one 2-byte load per slab and element.
template <typename T>
__global__ __launch_bounds__(256) void dbias_reduce8_kernel(const T* full, T* out, int B, int Hq, long SS, int bcast) {
  const int Hb = (bcast & 2) ? 1 : Hq;
  const int Bb = (bcast & 1) ? 1 : B;
  const long SS8 = SS / 8;
  const long x = (long)blockIdx.x * 256 + threadIdx.x;
  if (x >= (long)Bb * Hb * SS8) return;
  const long e = (x % SS8) * 8;
  const int hb = (int)((x / SS8) % Hb);
  const int bb = (int)(x / SS8 / Hb);
  const int b0 = (bcast & 1) ? 0 : bb, b1 = (bcast & 1) ? B : bb + 1;
  const int h0 = (bcast & 2) ? 0 : hb, h1 = (bcast & 2) ? Hq : hb + 1;
  float s[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  for (int b = b0; b < b1; ++b)
    for (int h = h0; h < h1; ++h) {
      float v[8];
      load8(full + ((long)b * Hq + h) * SS + e, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) s[i] += v[i];
    }
  store8<T>(out + x * 8, s);
}

// Head-summed dbias slabs of the 16-bit dk/dv kernel ([B][np][Sq][Sk], one
// per KV head and head split) into the caller's dbias ([B or 1][1][Sq][Sk]).
// The dk/dv workgroups of a block of BNK keys write the rows
// [qbeg, qbeg + nqt BMQ) of its columns, which the same visibility bounds
// give here; every other row of those columns sees none of the block's keys,
// is left unwritten in the slabs, and is zero in the result.  8 consecutive
// keys per thread (Sk % 8 == 0 on this path).
template <typename T, int BNK, int BMQ>
__global__ __launch_bounds__(256) void dbias_reduce_part_kernel(const T* slabs, T* out, int B, int np, int bcast,
                                                                Mask m, bool vec_out) {
  const int Sq = m.Sq, Sk = m.Sk;
  const int nc = Sk / 8;
  const int Bb = (bcast & 1) ? 1 : B;
  const long x = (long)blockIdx.x * 256 + threadIdx.x;
  if (x >= (long)Bb * Sq * nc) return;
  const int bb = (int)(x / ((long)Sq * nc));
  const long rem = x % ((long)Sq * nc);
  const int i = (int)(rem / nc);
  const int j = (int)(rem % nc) * 8;
  const int k0 = (j / BNK) * BNK;
  const int jlast = min(k0 + BNK, Sk) - 1;
  const long SS = (long)Sq * Sk;
  float s[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
  const int b0 = (bcast & 1) ? 0 : bb, b1 = (bcast & 1) ? B : bb + 1;
  for (int b = b0; b < b1; ++b) {
    int lo_first, hi_first, lo_last, hi_last;
    queries_of(m, b, k0, lo_first, hi_first);
    queries_of(m, b, jlast, lo_last, hi_last);
    const int qbeg = (lo_first / BMQ) * BMQ;
    const int nqt = hi_last > qbeg ? (hi_last - qbeg + BMQ - 1) / BMQ : 0;
    if (i < qbeg || i >= qbeg + nqt * BMQ) continue;
    const T* src = slabs + (long)b * np * SS + (long)i * Sk + j;
    for (int h = 0; h < np; ++h) {
      float v[8];
      load8(src + h * SS, v);
#pragma unroll
      for (int e = 0; e < 8; ++e) s[e] += v[e];
    }
  }
  T* dst = out + ((long)bb * Sq + i) * Sk + j;
  if (vec_out) {
    store8<T>(dst, s);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) dst[e] = (T)s[e];
  }
}

// dbias = 0 on every pair that no query-key visibility covers (the dkdv
// kernel writes the visible pairs).  One block per (row group, head, batch).
template <typename T>
__global__ __launch_bounds__(256) void dbias_fill_kernel(T* dbias, Mask mask, int Hq, int rows_per_block) {
  const int hq = blockIdx.y;
  const int b = blockIdx.z;
  const int Sq = mask.Sq, Sk = mask.Sk;
  const int r0 = blockIdx.x * rows_per_block;
  for (int rr = 0; rr < rows_per_block; ++rr) {
    const int i = r0 + rr;
    if (i >= Sq) break;
    int lo, hi;
    keys_of(mask, b, i, lo, hi);
    T* row = dbias + (((long)b * Hq + hq) * Sq + i) * Sk;
    for (int j = threadIdx.x; j < Sk; j += 256) {
      if (j < lo || j >= hi) row[j] = (T)0.0f;
    }
  }
}

}  // namespace ATL_NS
