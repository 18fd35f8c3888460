// Device building blocks shared by the gfx950 attention kernels: MFMA
// fragments, LDS tile staging, the soft-cap arithmetic and the visibility
// ranges of packed / causal / windowed rows.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

// The kernels live in namespace ATL_NS (atl).  The fp16 unit compiles the
// same sources a second time with ATL_FAST_F16 set and ATL_NS renamed: there
// the 16-bit element type `bf16` is IEEE fp16 (_Float16), with the fp16 MFMA
// and dot instructions, so that fp16 inputs run the same kernels.
#ifndef ATL_NS
#define ATL_NS atl
#endif
#ifndef ATL_FAST_F16
#define ATL_FAST_F16 0
#endif

namespace ATL_NS {

#if ATL_FAST_F16
typedef _Float16 bf16;
typedef _Float16 bf16x8 __attribute__((ext_vector_type(8)));
#else
typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
#endif
// the 16-bit element type has fp16's exponent range (2^-24 .. 65504)
constexpr bool kNarrow16 = ATL_FAST_F16 != 0;
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------- fragments
//
// Every contraction runs on 32x32 MFMA blocks.  A lane l = r + 32g (r < 32,
// g in {0,1}) holds, for each group of 16 contraction indices, the 8
// consecutive indices 8g..8g+7 of row r (A operand) or column r (B operand).
// bf16 feeds them to one v_mfma_f32_32x32x16_bf16; fp32 feeds them one index
// at a time to eight v_mfma_f32_32x32x2_f32 (index 8g+s in step s), which is
// the same pairing of A and B elements, so one fragment layout serves both.
//
// The accumulator layout of a 32x32 block: lane r + 32h, register j holds
// row 8(j/4) + 4h + (j%4), column r.  Operand rows are read through the bit
// swap `swp` (bits 2 and 3 of the row index exchanged), which turns that into
// row 16(j/8) + 8h + (j%8): register j of a lane then walks 8 consecutive
// rows twice, which is exactly the index order the next contraction's B
// fragment wants (registers 8s..8s+7 = indices 16s + 8g + 0..7), so
// probabilities and gradients feed the next MFMA with no lane shuffles.

template <typename T> struct Frag;
template <> struct Frag<bf16> { using type = bf16x8; };
template <> struct Frag<float> { using type = f32x8; };

__device__ __forceinline__ void mma(f32x16& c, const bf16x8& a, const bf16x8& b) {
#if ATL_FAST_F16
  c = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
#else
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
#endif
}
__device__ __forceinline__ void mma(f32x16& c, const f32x8& a, const f32x8& b) {
#pragma unroll
  for (int s = 0; s < 8; ++s) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[s], b[s], c, 0, 0, 0);
}

__host__ __device__ constexpr int swp(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// logical row (after the swp-permuted operand read) of accumulator register j
__device__ __forceinline__ int acc_row(int h, int j) { return 16 * (j >> 3) + 8 * h + (j & 7); }

template <typename T>
__device__ __forceinline__ typename Frag<T>::type lds_frag(const T* p);
template <>
__device__ __forceinline__ bf16x8 lds_frag<bf16>(const bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }

template <>
__device__ __forceinline__ f32x8 lds_frag<float>(const float* p) {
  f32x4 a = *reinterpret_cast<const f32x4*>(p);
  f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  f32x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
  r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
  return r;
}

// 8 fp32 accumulator values -> an operand fragment (round to nearest even)
__device__ __forceinline__ bf16x8 to_frag(const f32x16& c, int base, bf16*) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (bf16)c[base + i];
  return r;
}
__device__ __forceinline__ f32x8 to_frag(const f32x16& c, int base, float*) {
  f32x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = c[base + i];
  return r;
}

// ---------------------------------------------------------------- scalar helpers

__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// tanh for the soft-cap.  The 16-bit paths use 1 - 2/(1 + e^{2x}) (one
// exp2, one reciprocal; exact limits +-1 at overflow/underflow, absolute
// error a few fp32 ulps, far below bf16 or fp16 rounding).  The fp32 path keeps the device
// library's tanhf, which stays accurate to a few ulps relative near 0.
__device__ __forceinline__ float cap_tanh(float x, bf16*) {
  float e = fast_exp2(x * (2.0f * kLog2e));
  return 1.0f - 2.0f * __builtin_amdgcn_rcpf(1.0f + e);
}
__device__ __forceinline__ float cap_tanh(float x, float*) { return tanhf(x); }

template <typename T> __device__ __forceinline__ void store8(T* p, const float* v);
template <> __device__ __forceinline__ void store8<bf16>(bf16* p, const float* v) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (bf16)v[i];
  *reinterpret_cast<bf16x8*>(p) = r;
}
template <> __device__ __forceinline__ void store8<float>(float* p, const float* v) {
  f32x4 a, b;
#pragma unroll
  for (int i = 0; i < 4; ++i) { a[i] = v[i]; b[i] = v[4 + i]; }
  reinterpret_cast<f32x4*>(p)[0] = a;
  reinterpret_cast<f32x4*>(p)[1] = b;
}

// The part of 8 fp32 values that their bf16 rounding drops, v - bf16(v),
// itself rounded to bf16 (together the two carry v to about 16 bits)
__device__ __forceinline__ void store8_lo(bf16* p, const float* v) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (bf16)(v[i] - (float)(bf16)v[i]);
  *reinterpret_cast<bf16x8*>(p) = r;
}


// 8 consecutive values from global memory into fp32 (16-byte aligned for bf16,
// 32-byte for fp32)
__device__ __forceinline__ void load8(const bf16* p, float* v) {
  bf16x8 r = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (float)r[i];
}
__device__ __forceinline__ void load8(const float* p, float* v) {
  f32x4 a = reinterpret_cast<const f32x4*>(p)[0];
  f32x4 b = reinterpret_cast<const f32x4*>(p)[1];
#pragma unroll
  for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
}

// ---------------------------------------------------------------- LDS staging
//
// All threads of the workgroup take part.  Rows at or beyond `nvalid` are
// written as zeros so that masked-out keys or queries can never inject
// non-finite values into a contraction.

// lds[(PERM ? swp(r) : r) * LDS_STRIDE + c] = g[(row0 + r) * gstride + col0 + c]
template <typename T, int ROWS, int COLS, int LDS_STRIDE, bool PERM, int NT>
__device__ __forceinline__ void stage_rows(T* lds, const T* g, long gstride, int row0, int nvalid, int col0) {
  constexpr int VEC = 16 / sizeof(T);
  constexpr int CPR = COLS / VEC;
  constexpr int TOTAL = ROWS * CPR;
  static_assert(COLS % VEC == 0, "tile width must be a multiple of 16 bytes");
  const int tid = threadIdx.x;
#pragma unroll
  for (int idx0 = 0; idx0 < TOTAL; idx0 += NT) {
    const int idx = idx0 + tid;
    if (TOTAL % NT == 0 || idx < TOTAL) {
      const int r = idx / CPR;
      const int c = (idx % CPR) * VEC;
      uint4 val = {0u, 0u, 0u, 0u};
      if (row0 + r < nvalid) val = *reinterpret_cast<const uint4*>(g + (long)(row0 + r) * gstride + col0 + c);
      const int lr = PERM ? swp(r) : r;
      *reinterpret_cast<uint4*>(lds + lr * LDS_STRIDE + c) = val;
    }
  }
}

// Transposed: lds[(PERM ? swp(c) : c) * LDS_STRIDE + r] = g[(row0 + r) * gstride + col0 + c].
// Each thread takes two adjacent rows and one 16-byte column chunk and writes
// packed (row r, row r+1) pairs, so consecutive lanes write consecutive words.
template <typename T, int ROWS, int COLS, int LDS_STRIDE, bool PERM, int NT>
__device__ __forceinline__ void stage_rows_t(T* lds, const T* g, long gstride, int row0, int nvalid, int col0) {
  constexpr int VEC = 16 / sizeof(T);
  constexpr int RP = ROWS / 2;
  constexpr int TOTAL = RP * (COLS / VEC);
  static_assert(ROWS % 2 == 0 && COLS % VEC == 0, "bad transposed tile");
  const int tid = threadIdx.x;
#pragma unroll
  for (int idx0 = 0; idx0 < TOTAL; idx0 += NT) {
    const int idx = idx0 + tid;
    if (TOTAL % NT == 0 || idx < TOTAL) {
      const int rp = idx % RP;
      const int c0 = (idx / RP) * VEC;
      const int r = 2 * rp;
      T a[VEC], b[VEC];
      uint4 va = {0u, 0u, 0u, 0u}, vb = {0u, 0u, 0u, 0u};
      if (row0 + r < nvalid) va = *reinterpret_cast<const uint4*>(g + (long)(row0 + r) * gstride + col0 + c0);
      if (row0 + r + 1 < nvalid) vb = *reinterpret_cast<const uint4*>(g + (long)(row0 + r + 1) * gstride + col0 + c0);
      __builtin_memcpy(a, &va, 16);
      __builtin_memcpy(b, &vb, 16);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const int lc = PERM ? swp(c0 + e) : (c0 + e);
        T pair[2] = {a[e], b[e]};
        if constexpr (sizeof(T) == 2) {
          uint32_t w;
          __builtin_memcpy(&w, pair, 4);
          *reinterpret_cast<uint32_t*>(lds + lc * LDS_STRIDE + r) = w;
        } else {
          f32x2 w;
          __builtin_memcpy(&w, pair, 8);
          *reinterpret_cast<f32x2*>(lds + lc * LDS_STRIDE + r) = w;
        }
      }
    }
  }
}

// The same two stagings split in two: load() brings the tile's 16-byte
// chunks into registers, store() writes them to LDS, so that the global
// loads of the next tile can be in flight while the current one is in use.
template <typename T, int ROWS, int COLS, int NT>
struct RowChunks {
  static constexpr int VEC = 16 / sizeof(T);
  static constexpr int CPR = COLS / VEC;
  static constexpr int TOTAL = ROWS * CPR;
  static constexpr int N = (TOTAL + NT - 1) / NT;
  static_assert(COLS % VEC == 0, "tile width must be a multiple of 16 bytes");
  uint4 v[N];
  __device__ __forceinline__ void load(const T* g, long gstride, int row0, int nvalid, int col0) {
#pragma unroll
    for (int u = 0; u < N; ++u) {
      const int idx = u * NT + (int)threadIdx.x;
      v[u] = uint4{0u, 0u, 0u, 0u};
      if (TOTAL % NT == 0 || idx < TOTAL) {
        const int r = idx / CPR;
        const int c = (idx % CPR) * VEC;
        if (row0 + r < nvalid) v[u] = *reinterpret_cast<const uint4*>(g + (long)(row0 + r) * gstride + col0 + c);
      }
    }
  }
  template <int LDS_STRIDE, bool PERM>
  __device__ __forceinline__ void store(T* lds) const {
#pragma unroll
    for (int u = 0; u < N; ++u) {
      const int idx = u * NT + (int)threadIdx.x;
      if (TOTAL % NT == 0 || idx < TOTAL) {
        const int r = idx / CPR;
        const int c = (idx % CPR) * VEC;
        *reinterpret_cast<uint4*>(lds + (PERM ? swp(r) : r) * LDS_STRIDE + c) = v[u];
      }
    }
  }
};

template <typename T, int ROWS, int COLS, int NT>
struct RowPairChunks {
  static constexpr int VEC = 16 / sizeof(T);
  static constexpr int RP = ROWS / 2;
  static constexpr int TOTAL = RP * (COLS / VEC);
  static constexpr int N = (TOTAL + NT - 1) / NT;
  static_assert(ROWS % 2 == 0 && COLS % VEC == 0, "bad transposed tile");
  uint4 a[N], b[N];
  __device__ __forceinline__ void load(const T* g, long gstride, int row0, int nvalid, int col0) {
#pragma unroll
    for (int u = 0; u < N; ++u) {
      const int idx = u * NT + (int)threadIdx.x;
      a[u] = uint4{0u, 0u, 0u, 0u};
      b[u] = uint4{0u, 0u, 0u, 0u};
      if (TOTAL % NT == 0 || idx < TOTAL) {
        const int r = 2 * (idx % RP);
        const int c0 = (idx / RP) * VEC;
        if (row0 + r < nvalid) a[u] = *reinterpret_cast<const uint4*>(g + (long)(row0 + r) * gstride + col0 + c0);
        if (row0 + r + 1 < nvalid) b[u] = *reinterpret_cast<const uint4*>(g + (long)(row0 + r + 1) * gstride + col0 + c0);
      }
    }
  }
  // lds[(PERM ? swp(c) : c) * LDS_STRIDE + r] = tile[r][c]
  template <int LDS_STRIDE, bool PERM>
  __device__ __forceinline__ void store(T* lds) const {
#pragma unroll
    for (int u = 0; u < N; ++u) {
      const int idx = u * NT + (int)threadIdx.x;
      if (TOTAL % NT == 0 || idx < TOTAL) {
        const int r = 2 * (idx % RP);
        const int c0 = (idx / RP) * VEC;
        T x[VEC], y[VEC];
        __builtin_memcpy(x, &a[u], 16);
        __builtin_memcpy(y, &b[u], 16);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const int lc = PERM ? swp(c0 + e) : (c0 + e);
          T pair[2] = {x[e], y[e]};
          if constexpr (sizeof(T) == 2) {
            uint32_t w;
            __builtin_memcpy(&w, pair, 4);
            *reinterpret_cast<uint32_t*>(lds + lc * LDS_STRIDE + r) = w;
          } else {
            f32x2 w;
            __builtin_memcpy(&w, pair, 8);
            *reinterpret_cast<f32x2*>(lds + lc * LDS_STRIDE + r) = w;
          }
        }
      }
    }
  }
};

// Workgroup numbering for the 8 XCDs (each with its own L2), which receive
// workgroups round-robin by linear id.  A grid of ntile x ngroup workgroups
// (a group = one head, or one KV head, of one batch row) is renumbered so
// that XCD x works on groups x*ngroup/8 .. (x+1)*ngroup/8 - 1 only -- their
// tiles share K/V (or Q/dO) through that XCD's L2 -- and hands them out tile
// index by tile index across those groups, so that tile 0 (the longest
// under a causal mask) of every group is dispatched before any tile 1, and
// so on: longest first over the whole XCD, which keeps the tail short.
__device__ __forceinline__ void xcd_order(int ntile, int ngroup, int& tile, int& group) {
  const int L = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  if (ngroup % 8 == 0) {
    const int gpx = ngroup / 8;
    const int t = L / 8;
    tile = t / gpx;
    group = (L % 8) * gpx + t % gpx;
  } else {
    tile = L % ntile;
    group = L / ntile;
  }
}

// ---------------------------------------------------------------- visibility
//
// The keys a query sees and the queries a key is seen by are each one
// contiguous range, cut down by the causal flag and the window from bounds
// prepared per token: q_lo / q_hi (first visible key and one past the last,
// per query: packed segment runs, k_start) and k_lo / k_hi (first query that
// sees the key and one past the last, per key); absent arrays do not
// restrict.  All range ends are non-decreasing in the token index.  A dense
// boolean mask, where given, removes further pairs inside those ranges,
// unless its batch row is marked exact (the ranges, prepared from the mask
// itself, then hold exactly its visible pairs).

struct Mask {
  const int* q_lo;     // [B * Sq] or null
  const int* q_hi;
  const int* k_lo;     // [B * Sk] or null
  const int* k_hi;
  const unsigned char* dense;   // [B, Sq, Sk] or null: nonzero = visible
  const int* exact;    // [B] or null: 1 where the bounds already say all the dense mask says
  int Sq, Sk;
  int causal, window;
};

// keys visible to query i of batch row b: [lo, hi)
__device__ __forceinline__ void keys_of(const Mask& m, int b, int i, int& lo, int& hi) {
  lo = 0;
  hi = m.Sk;
  if (m.q_lo) lo = max(m.q_lo[(long)b * m.Sq + i], 0);
  if (m.q_hi) hi = min(m.q_hi[(long)b * m.Sq + i], m.Sk);
  if (m.causal) hi = min(hi, i + 1);
  if (m.window > 0) {
    lo = max(lo, i - m.window + 1);
    if (!m.causal) hi = min(hi, i + m.window);
  }
  lo = min(lo, m.Sk);  // keeps both ends non-decreasing in i and within [0, Sk]
  hi = max(hi, lo);
}

// queries that see key j of batch row b: [lo, hi)
__device__ __forceinline__ void queries_of(const Mask& m, int b, int j, int& lo, int& hi) {
  lo = 0;
  hi = m.Sq;
  if (m.k_lo) lo = max(m.k_lo[(long)b * m.Sk + j], 0);
  if (m.k_hi) hi = min(m.k_hi[(long)b * m.Sk + j], m.Sq);
  if (m.causal) lo = max(lo, j);
  if (m.window > 0) {
    hi = min(hi, j + m.window);
    if (!m.causal) lo = max(lo, j - m.window + 1);
  }
  lo = min(lo, m.Sq);  // keeps both ends non-decreasing in j and within [0, Sq]
  hi = max(hi, lo);
}

// whether batch row b needs the dense mask read pair by pair: it has one and
// the bounds above do not already describe it exactly
__device__ __forceinline__ bool dense_row(const Mask& m, int b) {
  return m.dense != nullptr && !(m.exact != nullptr && m.exact[b] != 0);
}

// the dense mask at (query i, key j) of batch row b, where chk = dense_row(m,
// b) (true otherwise); only called for pairs inside the ranges above, so
// i < Sq and j < Sk
__device__ __forceinline__ bool dense_ok(const Mask& m, bool chk, int b, int i, int j) {
  return !chk || m.dense[((long)b * m.Sq + i) * m.Sk + j] != 0;
}

// ---------------------------------------------------------------- dropout
//
// Keep decisions from the counter-based generator Philox4x32-10 (Salmon,
// Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC
// 2011): ten rounds over a four-word counter and a two-word key; each round
// forms the full 64-bit products of words 0 and 2 with 0xD2511F53 and
// 0xCD9E8D57 and crosses their halves with words 1 and 3 and the key, which
// grows by 0x9E3779B9 and 0xBB67AE85 between rounds.  One evaluation decides
// eight pairs: pair (query i, key j) of batch row b, query head h takes the
// 16-bit half j % 8 (low half of word (j % 8) / 2 for even j % 8, high half
// for odd) of the output at counter (j / 8, i, b * Hq + h, offset) under key
// (seed low, seed high), and is kept iff that half is at least thresh =
// floor(p 2^16).  The drop probability is thus p' = thresh / 2^16, and kept
// probabilities are scaled by 1 / (1 - p'), which keeps the expectation exact.
struct Dropout {
  int on;
  uint32_t thresh, seed_lo, seed_hi, offset;   // thresh < 2^16
  float scale;   // 1 / (1 - thresh / 2^16)
};

__device__ __forceinline__ void philox4x32_10(uint32_t c[4], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    // one 32x32 -> 64-bit multiply each (v_mad_u64_u32) for both halves
    const uint64_t p0 = (uint64_t)0xD2511F53u * c[0], p1 = (uint64_t)0xCD9E8D57u * c[2];
    const uint32_t lo0 = (uint32_t)p0, hi0 = (uint32_t)(p0 >> 32);
    const uint32_t lo1 = (uint32_t)p1, hi1 = (uint32_t)(p1 >> 32);
    const uint32_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
  }
}

// the Philox output c[4] that decides keys j8 .. j8 + 7 (j8 a multiple of 8) at query i
__device__ __forceinline__ void draw8(const Dropout& d, int i, int j8, int bh, uint32_t c[4]) {
  c[0] = (uint32_t)j8 >> 3;
  c[1] = (uint32_t)i;
  c[2] = (uint32_t)bh;
  c[3] = d.offset;
  philox4x32_10(c, d.seed_lo, d.seed_hi);
}

// decision e (0..7) of a draw: 16-bit half e is at least thresh, compared as
// the word (odd e) or the word shifted up by 16 (even e) against th16 = thresh << 16
__device__ __forceinline__ bool kept(const uint32_t c[4], int e, uint32_t th16) {
  const uint32_t w = c[e >> 1];
  return ((e & 1) ? w : (w << 16)) >= th16;
}

// the eight keep decisions of keys j8 .. j8 + 7 (j8 a multiple of 8), bit e for key j8 + e
__device__ __forceinline__ unsigned keep8(const Dropout& d, int i, int j8, int bh) {
  uint32_t c[4];
  draw8(d, i, j8, bh, c);
  const uint32_t th16 = d.thresh << 16;
  unsigned r = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) r |= (kept(c, e, th16) ? 1u : 0u) << e;
  return r;
}

// the four keep decisions of keys j4 .. j4 + 3 (j4 a multiple of 4), bit e for key j4 + e:
// half of one evaluation, for kernels whose lanes hold no more of its keys
__device__ __forceinline__ unsigned keep4(const Dropout& d, int i, int j4, int bh) {
  uint32_t c[4];
  draw8(d, i, j4 & ~7, bh, c);
  const uint32_t th16 = d.thresh << 16;
  const bool up = (j4 & 4) != 0;
  const uint32_t w[2] = {up ? c[2] : c[0], up ? c[3] : c[1]};
  return ((w[0] << 16) >= th16 ? 1u : 0u) | (w[0] >= th16 ? 2u : 0u) | ((w[1] << 16) >= th16 ? 4u : 0u) |
         (w[1] >= th16 ? 8u : 0u);
}

// x of lane l ^ 4 (both lanes in one row of 16): DPP row_shl:4 reads lane l + 4,
// row_shr:4 lane l - 4
__device__ __forceinline__ int from_lane_xor4(int x, int lane) {
  const int up = __builtin_amdgcn_update_dpp(0, x, 0x104, 0xF, 0xF, false);
  const int dn = __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);
  return (lane & 4) ? dn : up;
}

// shuffle with the partner lane l ^ 32 (the other half of a 32x32 column)
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

}  // namespace ATL_NS
