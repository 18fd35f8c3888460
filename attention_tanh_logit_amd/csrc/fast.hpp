// Pipelined bf16 kernels for head dims 64 and 128.
//
// Same arithmetic and masking as the kernels in kernels.hpp, arranged for
// gfx950 throughput:
//  * operands that stay fixed for a workgroup's whole loop (Q in the forward
//    and dq, K and V in dk/dv) live in registers as MFMA fragments;
//  * streamed tiles go straight from HBM into LDS with global_load_lds
//    (no registers held across the loop), issued one tile ahead into a
//    double-buffered LDS tile; one barrier per tile separates producers and
//    consumers and the HBM latency hides behind the current tile's MFMAs;
//  * every tile is stored once, row-major with 16-byte column slots XOR-
//    swizzled per row, and read both ways: plain 16-byte fragment reads for
//    one contraction and ds_read_b64_tr_b16 transposing reads for the other
//    (no transposed copies in LDS), both free of bank conflicts;
//  * loads are branch-free: rows past the end repeat the last row, whose
//    pairs the mask removes (their probabilities are exactly 0), and the mask
//    itself is evaluated only on tiles that are partly visible, chosen once
//    per tile rather than per element;
//  * the output accumulator is rescaled only when some row's running
//    maximum grows by more than 2^8 (probabilities stay bounded by 256 in
//    between, well inside fp32 and bf16 range).
//
// The cap in log2 units: with e = 2^(A*qk + Bb*bias), A = 2*log2(e)*scale/c,
// Bb = 2*log2(e)/c and r = 1/(1 + e), tanh(u/c) = 1 - 2r, so the capped logit
// is s2 = c*log2(e) - 2*c*log2(e)*r and the chain factor 1 - tanh^2 = 4r(1-r).
#pragma once

#include <type_traits>

#include "kernels.hpp"

namespace atl {

typedef short v4i16 __attribute__((ext_vector_type(4)));

// swap the two bits of a 2-bit index
__device__ __forceinline__ int swp2(int a) { return ((a & 1) << 1) | ((a >> 1) & 1); }

// ---------------------------------------------------------------- swizzled tiles
//
// Tile element (R, col) of a D-wide bf16 tile sits at R*D + 8*(col/8 ^ f(R)) +
// col%8 with f(R) = 2*(R%4) + (R/4)%2.  Eight consecutive rows then map one
// logical 16-byte slot to eight different bank groups (plain fragment reads),
// and four consecutive rows map a 32-byte column pair to eight different bank
// groups (transposing reads).
__device__ __forceinline__ int swz_f(int R) { return 2 * (R & 3) + ((R >> 2) & 1); }
template <int D>
__device__ __forceinline__ int sw_idx(int R, int col) {
  return R * D + (((col >> 3) ^ swz_f(R)) << 3) + (col & 7);
}

// Direct HBM -> LDS load of a ROWS x D tile.  global_load_lds writes lane i's
// 16 bytes at the instruction's LDS base + 16*i, so each wave instruction fills
// one contiguous KiB: lane chunk p is tile row R = p/(D/8), physical slot
// s = p%(D/8), and so takes logical column chunk s ^ f(R) of global row
// (PERM ? swp(R) : R); rows at or beyond nvalid repeat row nvalid-1.
template <int ROWS, int D, int NT, bool PERM>
__device__ __forceinline__ void load_tile(bf16* lds, const bf16* g, long gstride, int row0, int nvalid) {
  constexpr int CPR = D / 8;
  constexpr int N = ROWS * CPR / NT;
  static_assert((ROWS * CPR) % NT == 0, "tile must split evenly over the threads");
  const int w = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int u = 0; u < N; ++u) {
    const int pw = u * NT + w * 64;
    const int p = pw + lane;
    const int R = p / CPR;
    const int s = p % CPR;
    const int grow = min(row0 + (PERM ? swp(R) : R), nvalid - 1);
    const bf16* src = g + (long)grow * gstride + 8 * (s ^ swz_f(R));
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(lds + pw * 8), 16, 0, 0);
  }
}

__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ v4i16 ds_tr16(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(const_cast<bf16*>(p)));
}

// Plain A/B fragment: lane r + 32g holds tile row R, columns col0 + 8g .. +8.
template <int D>
__device__ __forceinline__ bf16x8 frag(const bf16* tile, int R, int col) {
  return *reinterpret_cast<const bf16x8*>(tile + sw_idx<D>(R, col));
}

// A fragment of X^T from the swizzled tile X: lane r + 32g receives
// X[row0 + 8g + i][col0 + swp(r)] for i = 0..7 (COLPERM) or ...[col0 + r].
// With ROWPERM the tile's rows are stored through swp (tile row swp(k) holds
// logical row k) and the fragment still walks logical rows row0 + 8g + i.
// ds_read_b64_tr_b16 hands lane j of each 16-lane group element j&3 of the
// 4-element chunk read by lane (j>>2) + 4e, for e = 0..3; choosing each
// source lane's row and column group accordingly yields the fragment.
template <int D, bool COLPERM, bool ROWPERM>
__device__ __forceinline__ bf16x8 frag_tr(const bf16* tile, int row0, int col0, int lane) {
  const int G = lane >> 4;
  const int s = lane & 15;
  const int R = row0 + (ROWPERM ? 4 : 8) * (G >> 1) + (s >> 2);
  const int c = col0 + 16 * (G & 1) + 4 * (COLPERM ? swp2(s & 3) : (s & 3));
  const v4i16 a = ds_tr16(tile + sw_idx<D>(R, c));
  const v4i16 b = ds_tr16(tile + sw_idx<D>(R + (ROWPERM ? 8 : 4), c));
  bf16x8 r;
  __builtin_memcpy(&r, &a, 8);
  __builtin_memcpy(reinterpret_cast<char*>(&r) + 8, &b, 8);
  return r;
}

// Log2-unit logit constants of the bf16 fast path (see the header comment).
struct LogitK {
  float a;    // multiplies q.k:   2*log2e*scale/c (cap) or scale*log2e
  float bb;   // multiplies bias:  2*log2e/c (cap) or log2e
  float c2;   // c*log2e (cap)
  __device__ __forceinline__ LogitK(float sl2, float xc, float bc, float cl2, bool cap) {
    a = cap ? xc * (2.0f * kLog2e) : sl2;
    bb = cap ? bc * (2.0f * kLog2e) : kLog2e;
    c2 = cl2;
  }
};

// s2 = capped logit in log2 units; f = d s / d u (1 - tanh^2; 1 without a cap)
template <bool CAP, bool BIAS, bool WANT_F>
__device__ __forceinline__ float logit_fast(float x, float bias, const LogitK& k, float& f) {
  float y = x * k.a;
  if constexpr (BIAS) y = fmaf(bias, k.bb, y);
  if constexpr (CAP) {
    const float r = __builtin_amdgcn_rcpf(1.0f + fast_exp2(y));
    if constexpr (WANT_F) f = 4.0f * r * (1.0f - r);
    return fmaf(r, -2.0f * k.c2, k.c2);
  } else {
    if constexpr (WANT_F) f = 1.0f;
    return y;
  }
}

template <bool B> using bool_c = std::integral_constant<bool, B>;

// ============================================================== forward

template <int D, bool CAP, bool BIAS>
__global__ __launch_bounds__(256, 2) void fwd_fast_kernel(FwdParams p) {
  constexpr int NT = 256;
  constexpr int BM = 128;
  constexpr int BN = 64;
  constexpr int NKB = BN / 32;
  constexpr int NOB = D / 32;
  constexpr int NCC = D / 16;

  __shared__ __attribute__((aligned(16))) bf16 sK[2][BN * D];
  __shared__ __attribute__((aligned(16))) bf16 sV[2][BN * D];

  const int qt = p.reverse ? (gridDim.x - 1 - blockIdx.x) : blockIdx.x;
  const int hq = blockIdx.y;
  const int b = blockIdx.z;
  const int hk = hq / p.G;
  const int Sq = p.mask.Sq, Sk = p.mask.Sk;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int n = lane & 31;
  const int h = lane >> 5;
  const int q0 = qt * BM;
  const int i = q0 + w * 32 + n;
  const LogitK lk(p.sl2, p.xc, p.bc, p.cl2, CAP);

  const bf16* kbase = reinterpret_cast<const bf16*>(p.k) + ((long)b * Sk * p.Hkv + hk) * D;
  const bf16* vbase = reinterpret_cast<const bf16*>(p.v) + ((long)b * Sk * p.Hkv + hk) * D;
  const long kstride = (long)p.Hkv * D;

  int lo_i = 0, hi_i = 0;
  if (i < Sq) keys_of(p.mask, b, i, lo_i, hi_i);
  const int ilast = min(q0 + BM, Sq) - 1;
  int lo_first, hi_first, lo_last, hi_last;
  keys_of(p.mask, b, q0, lo_first, hi_first);
  keys_of(p.mask, b, ilast, lo_last, hi_last);
  const bool rows_full = (q0 + BM <= Sq);

  // Q^T fragments of this wave's 32 queries stay in registers
  bf16x8 qf[NCC];
  {
    const bf16* qrow = reinterpret_cast<const bf16*>(p.q) + (((long)b * Sq + min(i, Sq - 1)) * p.Hq + hq) * D;
#pragma unroll
    for (int cc = 0; cc < NCC; ++cc) qf[cc] = *reinterpret_cast<const bf16x8*>(qrow + 16 * cc + 8 * h);
  }
  const bf16* brow = nullptr;
  if constexpr (BIAS) brow = reinterpret_cast<const bf16*>(p.bias) + (((long)b * p.Hq + hq) * Sq + min(i, Sq - 1)) * Sk;

  const bool has_sink = p.sink_mode != 0;
  const float sink2 = p.sink_mode == 2 ? p.sink[hq] * kLog2e : 0.0f;
  float m = has_sink ? sink2 : -INFINITY;
  float lsum = 0.0f;
  f32x16 oacc[NOB];
#pragma unroll
  for (int ob = 0; ob < NOB; ++ob) oacc[ob] = f32x16{};

  const int kbeg = (lo_first / BN) * BN;
  if (kbeg < hi_last) {
    load_tile<BN, D, NT, true>(sK[0], kbase, kstride, kbeg, Sk);
    load_tile<BN, D, NT, false>(sV[0], vbase, kstride, kbeg, Sk);
  }
  wait_loads();
  __syncthreads();

  int buf = 0;
  for (int k0 = kbeg; k0 < hi_last; k0 += BN, buf ^= 1) {
    if (k0 + BN < hi_last) {
      load_tile<BN, D, NT, true>(sK[buf ^ 1], kbase, kstride, k0 + BN, Sk);
      load_tile<BN, D, NT, false>(sV[buf ^ 1], vbase, kstride, k0 + BN, Sk);
    }
    const bf16* tK = sK[buf];
    const bf16* tV = sV[buf];

    // ---- S^T = K Q^T (tile row kb*32 + r holds key kb*32 + swp(r))
    f32x16 sacc[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) sacc[kb] = f32x16{};
#pragma unroll
    for (int cc = 0; cc < NCC; ++cc) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) mma(sacc[kb], frag<D>(tK, kb * 32 + n, 16 * cc + 8 * h), qf[cc]);
    }

    // ---- logits (log2 units), mask on partly visible tiles, running max
    float mx = -INFINITY;
    auto logits = [&](auto masked) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        float bv[16];
        if constexpr (BIAS) {
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) load8(brow + min(k0 + kb * 32 + 16 * hf + 8 * h, Sk - 8), bv + 8 * hf);
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          float f;
          float s2 = logit_fast<CAP, BIAS, false>(sacc[kb][j], BIAS ? bv[j] : 0.0f, lk, f);
          if constexpr (decltype(masked)::value) {
            const int key = k0 + kb * 32 + acc_row(h, j);
            s2 = (key >= lo_i && key < hi_i) ? s2 : -INFINITY;
          }
          sacc[kb][j] = s2;
          mx = fmaxf(mx, s2);
        }
      }
    };
    if (rows_full && k0 >= lo_last && k0 + BN <= hi_first) logits(bool_c<false>{});
    else logits(bool_c<true>{});
    mx = fmaxf(mx, xor32(mx));

    // ---- lazy rescale: move the reference maximum only when it grew by > 8
    const bool grow = mx > m + 8.0f;
    if (__any(grow)) {
      const float m_new = grow ? mx : m;
      const float alpha = (m == -INFINITY) ? 0.0f : fast_exp2(m - m_new);
      lsum *= alpha;
#pragma unroll
      for (int ob = 0; ob < NOB; ++ob) oacc[ob] *= alpha;
      m = m_new;
    }
    const float base = (m == -INFINITY) ? 0.0f : m;

    // ---- probabilities -> bf16 fragments
    bf16x8 pf[NKB][2];
    float ps = 0.0f;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float pv = fast_exp2(sacc[kb][j] - base);
        sacc[kb][j] = pv;
        ps += pv;
      }
      pf[kb][0] = to_frag(sacc[kb], 0, (bf16*)nullptr);
      pf[kb][1] = to_frag(sacc[kb], 8, (bf16*)nullptr);
    }
    lsum += ps;

    // ---- O^T += V^T P^T (V^T fragments by transposing LDS reads)
#pragma unroll
    for (int ob = 0; ob < NOB; ++ob) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb)
          mma(oacc[ob], frag_tr<D, true, false>(tV, kb * 32 + 16 * sb, ob * 32, lane), pf[kb][sb]);
      }
    }

    wait_loads();
    __syncthreads();
  }

  // ---- epilogue
  float ltot = lsum + xor32(lsum);
  if (has_sink) ltot += fast_exp2(sink2 - m);
  const float inv = ltot > 0.0f ? 1.0f / ltot : 0.0f;
  if (i < Sq) {
    bf16* orow = reinterpret_cast<bf16*>(p.out) + (((long)b * Sq + i) * p.Hq + hq) * D;
#pragma unroll
    for (int ob = 0; ob < NOB; ++ob) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        float vals[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) vals[e] = oacc[ob][8 * hf + e] * inv;
        store8<bf16>(orow + ob * 32 + 16 * hf + 8 * h, vals);
      }
    }
    if (h == 0) p.lse[((long)b * p.Hq + hq) * Sq + i] = ltot > 0.0f ? (m + __log2f(ltot)) * kLn2 : -INFINITY;
  }
}

// ============================================================== backward: dk, dv, dbias

// One workgroup = 4 waves = 128 keys of one KV head; K^T and V^T fragments of
// each wave's 32 keys stay in registers, dK^T / dV^T accumulate in registers
// over the GQA group's query heads and their visible 32-query tiles, which
// stream through a double-buffered LDS tile (rows stored through swp).
template <int D, bool CAP, bool BIAS>
__global__ __launch_bounds__(256, D > 64 ? 1 : 2) void dkdv_fast_kernel(BwdParams p) {
  constexpr int NT = 256;
  constexpr int BNK = 128;
  constexpr int BMQ = 32;
  constexpr int NOB = D / 32;
  constexpr int NCC = D / 16;

  __shared__ __attribute__((aligned(16))) bf16 sQ[2][BMQ * D];
  __shared__ __attribute__((aligned(16))) bf16 sO[2][BMQ * D];
  __shared__ __attribute__((aligned(16))) float sL[2][BMQ];
  __shared__ __attribute__((aligned(16))) float sDl[2][BMQ];

  const int hk = blockIdx.y;
  const int b = blockIdx.z;
  const int Sq = p.mask.Sq, Sk = p.mask.Sk;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int n = lane & 31;
  const int h = lane >> 5;
  const int k0 = blockIdx.x * BNK;
  const int j = k0 + w * 32 + n;
  const int jc = min(j, Sk - 1);
  const long qstride = (long)p.Hq * D;
  const LogitK lk(p.sl2, p.xc, p.bc, p.cl2, CAP);

  bf16x8 kf[NCC], vf[NCC];
  {
    const long off = (((long)b * Sk + jc) * p.Hkv + hk) * D;
    const bf16* krow = reinterpret_cast<const bf16*>(p.k) + off;
    const bf16* vrow = reinterpret_cast<const bf16*>(p.v) + off;
#pragma unroll
    for (int cc = 0; cc < NCC; ++cc) {
      kf[cc] = *reinterpret_cast<const bf16x8*>(krow + 16 * cc + 8 * h);
      vf[cc] = *reinterpret_cast<const bf16x8*>(vrow + 16 * cc + 8 * h);
    }
  }

  int lo_j = 0, hi_j = 0;
  if (j < Sk) queries_of(p.mask, b, j, lo_j, hi_j);
  const int jlast = min(k0 + BNK, Sk) - 1;
  int lo_first, hi_first, lo_last, hi_last;
  queries_of(p.mask, b, k0, lo_first, hi_first);
  queries_of(p.mask, b, jlast, lo_last, hi_last);
  const bool keys_full = (k0 + BNK <= Sk);
  const int qbeg = (lo_first / BMQ) * BMQ;
  const int nqt = hi_last > qbeg ? (hi_last - qbeg + BMQ - 1) / BMQ : 0;
  const int nitems = p.G * nqt;

  f32x16 kacc[NOB], vacc[NOB];
#pragma unroll
  for (int ob = 0; ob < NOB; ++ob) { kacc[ob] = f32x16{}; vacc[ob] = f32x16{}; }

  // item it = (query head it / nqt of the group, query tile it % nqt); its
  // Q and dO tiles go straight to LDS, its lse and delta (one row per thread
  // of the first 32) through registers, written to LDS after the current
  // item's work so the load latency overlaps it.
  float nl = 0.0f, nd = 0.0f;
  int nq = 0;
  auto fetch = [&](int it, int bf) {
    const int hq = hk * p.G + it / nqt;
    const int q0 = qbeg + (it % nqt) * BMQ;
    const long hoff = ((long)b * Sq * p.Hq + hq) * D;
    load_tile<BMQ, D, NT, true>(sQ[bf], reinterpret_cast<const bf16*>(p.q) + hoff, qstride, q0, Sq);
    load_tile<BMQ, D, NT, true>(sO[bf], reinterpret_cast<const bf16*>(p.dout) + hoff, qstride, q0, Sq);
    if (threadIdx.x < BMQ) {
      nq = q0 + threadIdx.x;
      const long li = ((long)b * p.Hq + hq) * Sq + min(nq, Sq - 1);
      nl = p.lse[li];
      nd = p.delta[li];
    }
  };
  auto put_stats = [&](int bf) {
    if (threadIdx.x < BMQ) {
      // a query past the end, or one that sees nothing, contributes P = 0
      sL[bf][threadIdx.x] = (nq < Sq && nl != -INFINITY) ? nl * kLog2e : INFINITY;
      sDl[bf][threadIdx.x] = nd;
    }
  };
  if (nitems > 0) {
    fetch(0, 0);
    put_stats(0);
  }
  wait_loads();
  __syncthreads();

  int buf = 0;
  for (int it = 0; it < nitems; ++it, buf ^= 1) {
    const bool more = it + 1 < nitems;
    if (more) fetch(it + 1, buf ^ 1);
    const int hq = hk * p.G + it / nqt;
    const int q0 = qbeg + (it % nqt) * BMQ;
    const bf16* tQ = sQ[buf];
    const bf16* tO = sO[buf];

    // ---- S = Q K^T, dP = dO V^T (rows: queries through swp; columns: this wave's keys)
    f32x16 sacc = f32x16{}, dpacc = f32x16{};
#pragma unroll
    for (int cc = 0; cc < NCC; ++cc) {
      mma(sacc, frag<D>(tQ, n, 16 * cc + 8 * h), kf[cc]);
      mma(dpacc, frag<D>(tO, n, 16 * cc + 8 * h), vf[cc]);
    }

    // ---- P and dU = P (dP - delta) (1 - t^2); register r <-> query q0 + acc_row(h, r)
    float lv[16], dl[16];
    {
      const f32x4* L4 = reinterpret_cast<const f32x4*>(sL[buf]);
      const f32x4* D4 = reinterpret_cast<const f32x4*>(sDl[buf]);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          const f32x4 a = L4[(16 * hf + 8 * h) / 4 + x];
          const f32x4 c = D4[(16 * hf + 8 * h) / 4 + x];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            lv[8 * hf + 4 * x + e] = a[e];
            dl[8 * hf + 4 * x + e] = c[e];
          }
        }
      }
    }
    const bf16* bcol = nullptr;
    bf16* dbcol = nullptr;
    if constexpr (BIAS) {
      const long boff = (((long)b * p.Hq + hq) * Sq) * Sk + jc;
      bcol = reinterpret_cast<const bf16*>(p.bias) + boff;
      if (p.dbias) dbcol = reinterpret_cast<bf16*>(p.dbias) + boff;
    }
    auto grads = [&](auto masked) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qi = q0 + acc_row(h, r);
        float bvv = 0.0f;
        if constexpr (BIAS) bvv = (float)bcol[(long)min(qi, Sq - 1) * Sk];
        float f;
        const float s2 = logit_fast<CAP, BIAS, true>(sacc[r], bvv, lk, f);
        float pv = fast_exp2(s2 - lv[r]);
        if constexpr (decltype(masked)::value) pv = (qi >= lo_j && qi < hi_j) ? pv : 0.0f;
        const float du = pv * (dpacc[r] - dl[r]) * f;
        sacc[r] = pv;
        dpacc[r] = du;
        if constexpr (BIAS) {
          const bool vis = decltype(masked)::value ? (qi >= lo_j && qi < hi_j) : true;
          if (dbcol && vis) dbcol[(long)qi * Sk] = (bf16)du;
        }
      }
    };
    if (keys_full && q0 >= lo_last && q0 + BMQ <= hi_first) grads(bool_c<false>{});
    else grads(bool_c<true>{});
    bf16x8 pf[2], uf[2];
    pf[0] = to_frag(sacc, 0, (bf16*)nullptr);
    pf[1] = to_frag(sacc, 8, (bf16*)nullptr);
    uf[0] = to_frag(dpacc, 0, (bf16*)nullptr);
    uf[1] = to_frag(dpacc, 8, (bf16*)nullptr);

    // ---- dV^T += dO^T P,  dK^T += Q^T dU
#pragma unroll
    for (int ob = 0; ob < NOB; ++ob) {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        mma(vacc[ob], frag_tr<D, true, true>(tO, 16 * sb, ob * 32, lane), pf[sb]);
        mma(kacc[ob], frag_tr<D, true, true>(tQ, 16 * sb, ob * 32, lane), uf[sb]);
      }
    }

    if (more) put_stats(buf ^ 1);
    wait_loads();
    __syncthreads();
  }

  if (j < Sk) {
    const long off = (((long)b * Sk + j) * p.Hkv + hk) * D;
    bf16* krow = reinterpret_cast<bf16*>(p.dk) + off;
    bf16* vrow = reinterpret_cast<bf16*>(p.dv) + off;
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
        const int d = ob * 32 + 16 * hf + 8 * h;
        store8<bf16>(krow + d, kv);
        store8<bf16>(vrow + d, vv);
      }
    }
  }
}

// ============================================================== backward: dq

// One workgroup = 4 waves = 128 queries of one query head; Q^T and dO^T
// fragments stay in registers, dQ^T accumulates in registers, K and V tiles
// of 32 keys stream through a double-buffered LDS tile (rows stored through
// swp; K^T fragments for dQ come from the same tile by transposing reads).
template <int D, bool CAP, bool BIAS>
__global__ __launch_bounds__(256, 2) void dq_fast_kernel(BwdParams p) {
  constexpr int NT = 256;
  constexpr int BM = 128;
  constexpr int BN = 32;
  constexpr int NOB = D / 32;
  constexpr int NCC = D / 16;

  __shared__ __attribute__((aligned(16))) bf16 sK[2][BN * D];
  __shared__ __attribute__((aligned(16))) bf16 sV[2][BN * D];

  const int qt = p.reverse ? (gridDim.x - 1 - blockIdx.x) : blockIdx.x;
  const int hq = blockIdx.y;
  const int b = blockIdx.z;
  const int hk = hq / p.G;
  const int Sq = p.mask.Sq, Sk = p.mask.Sk;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int n = lane & 31;
  const int h = lane >> 5;
  const int q0 = qt * BM;
  const int i = q0 + w * 32 + n;
  const LogitK lk(p.sl2, p.xc, p.bc, p.cl2, CAP);

  const bf16* kbase = reinterpret_cast<const bf16*>(p.k) + ((long)b * Sk * p.Hkv + hk) * D;
  const bf16* vbase = reinterpret_cast<const bf16*>(p.v) + ((long)b * Sk * p.Hkv + hk) * D;
  const long kstride = (long)p.Hkv * D;

  int lo_i = 0, hi_i = 0;
  if (i < Sq) keys_of(p.mask, b, i, lo_i, hi_i);
  const int ilast = min(q0 + BM, Sq) - 1;
  int lo_first, hi_first, lo_last, hi_last;
  keys_of(p.mask, b, q0, lo_first, hi_first);
  keys_of(p.mask, b, ilast, lo_last, hi_last);
  const bool rows_full = (q0 + BM <= Sq);

  const long row = ((long)b * p.Hq + hq) * Sq + min(i, Sq - 1);
  const float lse_i = p.lse[row];
  const float lse2 = (i < Sq && lse_i != -INFINITY) ? lse_i * kLog2e : INFINITY;
  const float delta_i = p.delta[row];

  bf16x8 qf[NCC], of[NCC];
  {
    const long off = (((long)b * Sq + min(i, Sq - 1)) * p.Hq + hq) * D;
    const bf16* qrow = reinterpret_cast<const bf16*>(p.q) + off;
    const bf16* orow = reinterpret_cast<const bf16*>(p.dout) + off;
#pragma unroll
    for (int cc = 0; cc < NCC; ++cc) {
      qf[cc] = *reinterpret_cast<const bf16x8*>(qrow + 16 * cc + 8 * h);
      of[cc] = *reinterpret_cast<const bf16x8*>(orow + 16 * cc + 8 * h);
    }
  }
  const bf16* brow = nullptr;
  if constexpr (BIAS) brow = reinterpret_cast<const bf16*>(p.bias) + row * Sk;

  f32x16 qacc[NOB];
#pragma unroll
  for (int ob = 0; ob < NOB; ++ob) qacc[ob] = f32x16{};

  const int kbeg = (lo_first / BN) * BN;
  if (kbeg < hi_last) {
    load_tile<BN, D, NT, true>(sK[0], kbase, kstride, kbeg, Sk);
    load_tile<BN, D, NT, true>(sV[0], vbase, kstride, kbeg, Sk);
  }
  wait_loads();
  __syncthreads();

  int buf = 0;
  for (int k0 = kbeg; k0 < hi_last; k0 += BN, buf ^= 1) {
    if (k0 + BN < hi_last) {
      load_tile<BN, D, NT, true>(sK[buf ^ 1], kbase, kstride, k0 + BN, Sk);
      load_tile<BN, D, NT, true>(sV[buf ^ 1], vbase, kstride, k0 + BN, Sk);
    }
    const bf16* tK = sK[buf];
    const bf16* tV = sV[buf];

    // ---- S^T = K Q^T, dP^T = V dO^T
    f32x16 sacc = f32x16{}, dpacc = f32x16{};
#pragma unroll
    for (int cc = 0; cc < NCC; ++cc) {
      mma(sacc, frag<D>(tK, n, 16 * cc + 8 * h), qf[cc]);
      mma(dpacc, frag<D>(tV, n, 16 * cc + 8 * h), of[cc]);
    }

    // ---- dU^T = P^T (dP^T - delta) (1 - t^2)
    float bv[16];
    if constexpr (BIAS) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) load8(brow + min(k0 + 16 * hf + 8 * h, Sk - 8), bv + 8 * hf);
    }
    auto grads = [&](auto masked) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float f;
        const float s2 = logit_fast<CAP, BIAS, true>(sacc[r], BIAS ? bv[r] : 0.0f, lk, f);
        float pv = fast_exp2(s2 - lse2);
        if constexpr (decltype(masked)::value) {
          const int key = k0 + acc_row(h, r);
          pv = (key >= lo_i && key < hi_i) ? pv : 0.0f;
        }
        sacc[r] = pv * (dpacc[r] - delta_i) * f;
      }
    };
    if (rows_full && k0 >= lo_last && k0 + BN <= hi_first) grads(bool_c<false>{});
    else grads(bool_c<true>{});
    bf16x8 uf[2];
    uf[0] = to_frag(sacc, 0, (bf16*)nullptr);
    uf[1] = to_frag(sacc, 8, (bf16*)nullptr);

    // ---- dQ^T += K^T dU^T (K^T fragments by transposing reads of the K tile)
#pragma unroll
    for (int ob = 0; ob < NOB; ++ob) {
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) mma(qacc[ob], frag_tr<D, true, true>(tK, 16 * sb, ob * 32, lane), uf[sb]);
    }

    wait_loads();
    __syncthreads();
  }

  if (i < Sq) {
    bf16* drow = reinterpret_cast<bf16*>(p.dq) + (((long)b * Sq + i) * p.Hq + hq) * D;
#pragma unroll
    for (int ob = 0; ob < NOB; ++ob) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        float vals[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) vals[e] = qacc[ob][8 * hf + e] * p.scale;
        store8<bf16>(drow + ob * 32 + 16 * hf + 8 * h, vals);
      }
    }
  }
}

}  // namespace atl
