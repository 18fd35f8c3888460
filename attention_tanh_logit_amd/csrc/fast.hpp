// Pipelined kernels for 16-bit elements (bf16; fp16 in the second build of
// these sources) at head dims 64, 128 and 256, and the dq kernel that reads
// the dU blocks (also at head dim 512, after the kernels of wide.hpp).
//
// Same arithmetic and masking as the kernels in kernels.hpp, arranged for
// gfx950 throughput:
//  * operands that stay fixed for a workgroup's whole loop (Q in the forward
//    and dq, K and V in dk/dv) live in registers as MFMA fragments;
//  * streamed tiles go straight from HBM into LDS with buffer loads
//    (no registers held across the loop), issued one tile ahead into a
//    double-buffered LDS tile; one barrier per tile separates producers and
//    consumers and the HBM latency hides behind the current tile's MFMAs;
//  * every tile is stored once, row-major with 16-byte column slots XOR-
//    swizzled per row, and read both ways: plain 16-byte fragment reads for
//    one contraction and ds_read_b64_tr_b16 transposing reads for the other
//    (no transposed copies in LDS), both free of bank conflicts;
//  * loads are branch-free: the buffer resource's range check returns zeros
//    for rows past the end of a head's rows, whose pairs the mask removes
//    (their probabilities are exactly 0), and the mask itself is evaluated
//    only on tiles that are partly visible, chosen once per tile rather than
//    per element;
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

namespace ATL_NS {

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));

// swap the two bits of a 2-bit index
__device__ __forceinline__ int swp2(int a) { return ((a & 1) << 1) | ((a >> 1) & 1); }

// ---------------------------------------------------------------- swizzled tiles
//
// gfx950 LDS has 64 four-byte banks (256 bytes); a 16-byte read is serviced
// 16 lanes at a time and an 8-byte read 32 lanes at a time, each group
// conflict-free only if it touches distinct banks.  Tile element (R, col) of
// a D-wide bf16 tile sits at R*D + 8*(col/8 ^ f(R)) + col%8, with f chosen so
// that 16 consecutive rows put one logical 16-byte slot into 16 different bank
// slots (plain fragment reads) and 4 consecutive rows x 64 bytes of columns
// cover 32 different 8-byte bank pairs (transposing reads):
//   D = 128 (256-byte rows):     f(R) = 4*(R%4) + (R/4)%4
//   D = 64  (two rows per 256):  f(R) = 4*((R/2)%2) + (R/4)%4
// Both have period 16 in R, so row offsets that are multiples of 16 are
// plain constants.
template <int D>
__device__ __forceinline__ int swz_f(int R) {
  return D >= 128 ? 4 * (R & 3) + ((R >> 2) & 3) : 4 * ((R >> 1) & 1) + ((R >> 2) & 3);
}
template <int D>
__device__ __forceinline__ int sw_idx(int R, int col) {
  return R * D + (((col >> 3) ^ swz_f<D>(R)) << 3) + (col & 7);
}

// Buffer resource (V#) over rows row0 .. nvalid-1 of a row-strided bf16
// tensor: base at row row0, range (nvalid - row0) rows.  Buffer reads whose
// offset lies past the range return zeros, so a tile that runs past the last
// row needs no clamping.  Word 3 is the gfx9 raw-buffer format word.  Tile
// offsets stay below 2^31 bytes (the host only picks these kernels then).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const bf16* g, long gstride, int row0, int nvalid) {
  const long bytes = (long)max(nvalid - row0, 0) * gstride * 2;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(g + (long)row0 * gstride), 0,
                                           (int)min(bytes, 0x7fffffffL), 0x00020000);
}

// One 16-byte buffer read straight into LDS: lane i's bytes land at the LDS
// base + 16*i.  A buffer (not global) load so that the LDS DMA counts in
// vmcnt alone and LDS reads issued meanwhile can still be waited for one at
// a time.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, int voff_bytes, bf16* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds, 16, voff_bytes, 0,
                                           0, 0);
}
// the same with the non-temporal cache policy: for the dU blocks, which the
// dk/dv kernel writes once (non-temporal stores) and the dq kernel reads once;
// streaming both ways moves dU at about 5.3 TB/s instead of 4.5
__device__ __forceinline__ void dma16_nt(__amdgpu_buffer_rsrc_t rsrc, int voff_bytes, bf16* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void*)lds, 16, voff_bytes, 0,
                                           0, 2);
}

// Direct HBM -> LDS load of a ROWS x D tile.  Each wave instruction fills one
// contiguous KiB: lane chunk p is tile row R = p/(D/8), physical slot
// s = p%(D/8), and so takes logical column chunk s ^ f(R) of global row
// row0 + (PERM ? swp(R) : R); rows at or beyond nvalid read as zeros.
// Row swizzle of tiles read by 16x16x32 fragments (D = 128): f(R) =
// 2*(R%8) + (R/8)%2.  Plain fragment reads (16 lanes: 16 consecutive rows,
// one logical slot) need f one-to-one on 16 rows; the transposing reads of
// such fragments (32 lanes: 8 consecutive rows x one aligned 32-byte slot
// pair) need f/2 one-to-one on 8 consecutive rows.  Period 16.
__device__ __forceinline__ int swz16(int R) { return 2 * (R & 7) + ((R >> 3) & 1); }

template <int ROWS, int D, int NT, bool PERM, bool SW16 = false>
__device__ __forceinline__ void load_tile(bf16* lds, const bf16* g, long gstride, int row0, int nvalid) {
  constexpr int CPR = D / 8;
  constexpr int N = ROWS * CPR / NT;
  static_assert((ROWS * CPR) % NT == 0, "tile must split evenly over the threads");
  const int w = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const auto rsrc = rows_rsrc(g, gstride, row0, nvalid);
#pragma unroll
  for (int u = 0; u < N; ++u) {
    const int pw = u * NT + w * 64;
    const int p = pw + lane;
    const int R = p / CPR;
    const int s = p % CPR;
    dma16(rsrc, 2 * ((PERM ? swp(R) : R) * (int)gstride + 8 * (s ^ (SW16 ? swz16(R) : swz_f<D>(R)))), lds + pw * 8);
  }
}

__device__ __forceinline__ void wait_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ v4i16 ds_tr16(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(const_cast<bf16*>(p)));
}

// Per-lane fragment offsets of a swizzled tile.  With f(R) = 4*fa(R) + fb(R)
// (fa, fb two-bit fields), XOR-ing a compile-time slot offset with f
// separates into XORs on independent bit fields, so a read at a compile-time
// (row, column block) is a per-lane base, one XOR with a constant and a
// constant add -- a few registers instead of one per read.
//
// Plain fragment of contraction step cc at tile rows row0 + 0..31 (lane
// r + 32g: row r, columns 16cc + 8g .. +8): slot 2cc + g ^ f(r).
// Transposing fragment of output column block ob at rows row0 + ...: lane
// r + 32g receives X[row0 + 8g + i][32ob + swp(r)], i = 0..7 (with ROWPERM
// the tile's rows are stored through swp and the fragment still walks
// logical rows row0 + 8g + i).  ds_read_b64_tr_b16 hands lane j of each
// 16-lane group element j&3 of the 4-element chunk read by lane (j>>2) + 4e,
// e = 0..3; each source lane's row and column group are chosen accordingly.
// Hides an integer's known bits from the optimiser.  LDS offsets built from
// it stay additions, which fold into the ds instruction's immediate offset
// field (a buffer's base address included), instead of becoming disjoint ORs
// that need one register per (buffer, fragment) pair.
__device__ __forceinline__ int opaque(int x) {
  asm("" : "+v"(x));
  return x;
}

template <int D, bool ROWPERM>
struct FragOfs {
  static constexpr int NCC = D / 16;
  static constexpr int NOB = D / 32;
  int pbase;    // plain: row offset + the slot bits that do not move with cc
  int pxor;     // plain: 16 * (f(r) >> 1), XOR-ed with 16 * cc
  int tbase[2]; // transposing reads: everything but the column block
  int txor;     // transposing reads: 32 * (slot-block bits of f), XOR-ed with 32 * ob
  __device__ __forceinline__ explicit FragOfs(int lane) {
    const int n = lane & 31, h = lane >> 5;
    const int fn = swz_f<D>(n);
    pbase = opaque(n * D + 8 * ((h ^ fn) & 1));
    pxor = opaque(16 * (fn >> 1));
    const int G = lane >> 4, s = lane & 15;
    const int R = (ROWPERM ? 4 : 8) * (G >> 1) + (s >> 2);
    const int R2 = R + (ROWPERM ? 8 : 4);
    const int c = 16 * (G & 1) + 4 * swp2(s & 3);   // column inside a 32-column block
    // slot (4 ob + c/8) ^ f(R) = 4 (ob ^ (f >> 2)) + ((c/8) ^ (f & 3)); f >> 2 agrees for R and R2
    tbase[0] = opaque(R * D + 8 * (((c >> 3) ^ swz_f<D>(R)) & 3) + (c & 7));
    tbase[1] = opaque(R2 * D + 8 * (((c >> 3) ^ swz_f<D>(R2)) & 3) + (c & 7));
    txor = opaque(32 * (swz_f<D>(R) >> 2));
  }
  __device__ __forceinline__ bf16x8 frag(const bf16* tile, int row0, int cc) const {
    return *reinterpret_cast<const bf16x8*>(tile + row0 * D + pbase + ((16 * cc) ^ pxor));
  }
  __device__ __forceinline__ bf16x8 frag_tr(const bf16* tile, int row0, int ob) const {
    const int x = (32 * ob) ^ txor;
    const v4i16 a = ds_tr16(tile + row0 * D + tbase[0] + x);
    const v4i16 b = ds_tr16(tile + row0 * D + tbase[1] + x);
    bf16x8 r;
    __builtin_memcpy(&r, &a, 8);
    __builtin_memcpy(reinterpret_cast<char*>(&r) + 8, &b, 8);
    return r;
  }
};

// Per-lane fragment offsets for v_mfma_f32_16x16x32_bf16 operands from a
// D = 128 tile stored with swz16.  Lane r + 16g:
//  * frag(row0, c): row row0 + r, 16-byte chunk (c % 4) + 4g + 16 (c / 4)
//    (the A or B operand of a product that contracts over the columns;
//    lanes 16 apart take chunks 64 bytes apart, which measured free of bank
//    conflicts where adjacent chunks (columns 32c + 8g) conflicted two ways;
//    the swizzle permutes chunks inside 128-column groups only);
//  * frag_tr(row0, ob): X[row0 + sigma(g, i)][16 ob + r], i = 0..7, with
//    sigma(g, i) = 4g + i for i < 4 and 16 + 4g + i - 4 after, which is the
//    query order in which a 16x16 accumulator pair (rows 16qb + 4g + e) hands
//    its values to the next product.  Two ds_read_b64_tr_b16: source lane
//    s + 16g points at row 4g + s/4 (+16), columns 16 ob + 4(s%4) .. + 3.
template <int D>
struct Frag16Ofs {
  static_assert(D == 128 || D == 256 || D == 512, "laid out for 256-, 512- or 1024-byte rows");
  int pbase, pxor, tbase, txor;
  __device__ __forceinline__ explicit Frag16Ofs(int lane) {
    const int r = lane & 15, g = lane >> 4;
    const int fr = swz16(r);
    // slot (c + 4g) ^ f = 4 (g ^ (f >> 2)) + (c ^ (f & 3))
    pbase = opaque(r * D + 32 * (g ^ (fr >> 2)));
    pxor = opaque(8 * (fr & 3));
    const int R1 = 4 * g + (r >> 2);
    const int f = swz16(R1);
    // slot (2 ob + (r%4)/2) ^ f = ((2 ob) ^ (f & 14)) + (((r%4)/2 ^ f) & 1)
    tbase = opaque(R1 * D + 8 * ((((r & 3) >> 1) ^ f) & 1) + 4 * (r & 1));
    txor = opaque(8 * (f & 14));
  }
  __device__ __forceinline__ bf16x8 frag(const bf16* tile, int row0, int c) const {
    return *reinterpret_cast<const bf16x8*>(tile + row0 * D + pbase + ((8 * (c & 3)) ^ pxor) + 128 * (c >> 2));
  }
  __device__ __forceinline__ bf16x8 frag_tr(const bf16* tile, int row0, int ob) const {
    const bf16* a = tile + row0 * D + tbase + ((16 * ob) ^ txor);
    const v4i16 x = ds_tr16(a);
    const v4i16 y = ds_tr16(a + 16 * D);
    bf16x8 r;
    __builtin_memcpy(&r, &x, 8);
    __builtin_memcpy(reinterpret_cast<char*>(&r) + 8, &y, 8);
    return r;
  }
};

__device__ __forceinline__ void mma16(f32x4& c, const bf16x8& a, const bf16x8& b) {
#if ATL_FAST_F16
  c = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
#else
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
#endif
}

// Two 16x16 accumulators (query blocks 2kc, 2kc+1) -> one operand fragment
// whose 8 contraction indices are the queries sigma(g, 0..7).
__device__ __forceinline__ bf16x8 pack8(const f32x4& a, const f32x4& b) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r[e] = (bf16)a[e];
    r[4 + e] = (bf16)b[e];
  }
  return r;
}

// Sum of the 8 bf16 values of a fragment, added to acc in fp32 (v_dot2 with
// (1, 1)): the forward's row sums are taken over exactly the rounded
// probabilities its P V products use, so that each output row is normalised
// by its own numerator's weights (an fp32 sum would scale the row by the
// rounding of its largest probability, up to 2^-9).
typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float sum_bf16x8(const bf16x8& f, float acc) {
  const bf16x2 one = {(bf16)1.0f, (bf16)1.0f};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
#if ATL_FAST_F16
    acc = __builtin_amdgcn_fdot2(bf16x2{f[2 * e], f[2 * e + 1]}, one, acc, false);
#else
    acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{f[2 * e], f[2 * e + 1]}, one, acc, false);
#endif
  }
  return acc;
}

// The same for 4 values.
__device__ __forceinline__ float sum_bf16x4(const bf16x4& f, float acc) {
  const bf16x2 one = {(bf16)1.0f, (bf16)1.0f};
#pragma unroll
  for (int e = 0; e < 2; ++e) {
#if ATL_FAST_F16
    acc = __builtin_amdgcn_fdot2(bf16x2{f[2 * e], f[2 * e + 1]}, one, acc, false);
#else
    acc = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{f[2 * e], f[2 * e + 1]}, one, acc, false);
#endif
  }
  return acc;
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

// Backward probability P = 2^(s2 - lse2) with Lc = (cap ? c2 : 0) - lse2
// folded into one fma, and g = (1 - tanh^2)/4 = r(1 - r) (1 without a cap);
// the gradients carry the factor 4 in their final scale (kGrad4).
template <bool CAP, bool BIAS>
__device__ __forceinline__ float prob_fast(float x, float bias, const LogitK& k, float Lc, float& g) {
  float y = x * k.a;
  if constexpr (BIAS) y = fmaf(bias, k.bb, y);
  if constexpr (CAP) {
    const float r = __builtin_amdgcn_rcpf(1.0f + fast_exp2(y));
    g = fmaf(-r, r, r);
    return fast_exp2(fmaf(r, -2.0f * k.c2, Lc));
  } else {
    g = 1.0f;
    return fast_exp2(y + Lc);
  }
}
template <bool CAP> constexpr float kGrad4 = CAP ? 4.0f : 1.0f;

template <bool B> using bool_c = std::integral_constant<bool, B>;

// Per-thread plan of a direct tile load: this thread's 16-byte chunk u sits
// NT/(D/8) rows below chunk u-1 (a multiple of 16 rows, where swp and the
// swizzle repeat), so one byte offset off0 relative to the tile's first row
// serves every chunk; rows past the end read as zeros through the buffer range.
template <int ROWS, int D, int NT, bool PERM>
struct TilePlan {
  static constexpr int CPR = D / 8;
  static constexpr int N = ROWS * CPR / NT;
  static constexpr int RSTEP = NT / CPR;
  static_assert((ROWS * CPR) % NT == 0 && RSTEP % 16 == 0, "tile must split evenly over the threads");
  int off0;
  int ustep;   // bytes between consecutive chunks of one thread
  __device__ __forceinline__ explicit TilePlan(long gstride) {
    const int p = threadIdx.x;
    const int R = p / CPR, s = p % CPR;
    off0 = 2 * ((PERM ? swp(R) : R) * (int)gstride + 8 * (s ^ swz_f<D>(R)));
    ustep = 2 * RSTEP * (int)gstride;
  }
  __device__ __forceinline__ void issue(bf16* lds, const bf16* g, long gstride, int row0, int nvalid) const {
    const int w = threadIdx.x >> 6;
    const auto rsrc = rows_rsrc(g, gstride, row0, nvalid);
#pragma unroll
    for (int u = 0; u < N; ++u) dma16(rsrc, off0 + u * ustep, lds + (u * NT + w * 64) * 8);
  }
};

// Scheduling hint for a block of NMFMA MFMAs that each consume PER LDS reads:
// AHEAD reads are issued up front and every MFMA is followed by the next PER
// reads, so that reads stay in flight instead of each one being waited for
// right before its MFMA.  (A macro: the hint must sit in the caller's own
// scheduling region.)
#define ATL_READ_AHEAD(AHEAD, PER, NMFMA)                        \
  do {                                                           \
    __builtin_amdgcn_sched_group_barrier(0x100, (AHEAD), 0);     \
    _Pragma("unroll") for (int x_ = 0; x_ < (NMFMA); ++x_) {     \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);         \
      __builtin_amdgcn_sched_group_barrier(0x100, (PER), 0);     \
    }                                                            \
  } while (0)


// ============================================================== forward

// With PIPE the loop is software-pipelined over key tiles: while the softmax
// of tile t runs on the VALU, the MFMAs of S_{t+1} = K_{t+1} Q^T are already
// in flight (they sit in the same straight-line block, so the scheduler
// interleaves them).  K tiles are then fetched two tiles ahead and V tiles
// one ahead; two LDS buffers of each suffice.  The pipelined form holds two
// score tiles, which fits the register file at D = 64 but not at D = 128.
//
// Capped logits are tracked through r = 1/(1 + 2^y) (s2 = c2 - 2 c2 r is
// decreasing in r): the row maximum is c2 - 2 c2 min(r), and the probability
// 2^(s2 - m) = 2^(fma(r, -2 c2, c2 - m)) needs no separate subtraction.
//
// FIXM (capped logits with 2 c2 <= 120): a capped logit never exceeds c2, so
// the reference maximum stays at c2 for the whole row -- no running maximum,
// no rescaling -- and 2^(s2 - c2) = 2^(-2 c2 r) lies in [2^-120, 1], inside the
// normal range of fp32 and bf16.  The reciprocal then produces -2 c2 r
// directly: 1 / fma(e, k, k) with k = -1/(2 c2) equals -2 c2 / (1 + e).
//
// D = 256: the output columns split over NSL = 2 waves per 32-row group (8
// waves, 128 rows); both compute the row's logits and probabilities, each
// accumulates its 128 columns of O, so O fits the register file beside the
// whole row of Q^T fragments.
//
// DROP: dropout on the probabilities.  A lane's 16 logits of a 32-key block
// are two runs of 8 consecutive keys of its query, so one Philox4x32-10
// evaluation gives the keep decisions of a run; the row sum (and lse) takes
// the undropped probabilities, P.V the kept ones, and the epilogue scales O
// by 1 / (1 - p').
template <int D, bool CAP, bool BIAS, bool FIXM, bool DROP>
__global__ __launch_bounds__(D > 128 ? 512 : 256, D > 128 ? 1 : 2) void fwd_fast_kernel(FwdParams p) {
  static_assert(CAP || !FIXM, "a fixed reference maximum needs bounded logits");
  constexpr int NSL = D > 128 ? 2 : 1;     // column slices of O per row group
  constexpr int NT = 256 * NSL;
  constexpr int BM = 128;
  constexpr int BN = D > 128 ? 32 : 64;  // D = 256: one 32-key block per tile (registers)
  constexpr bool PIPE = D <= 64;
  constexpr bool ROWPERM_TR = false;  // V rows in key order
  constexpr int NKB = BN / 32;
  constexpr int NOB = D / 32 / NSL;     // this wave's output column blocks
  constexpr int NCC = D / 16;

  // two LDS buffers per tile as distinct objects: the compiler can then see
  // that reading one never aliases the DMA filling the other
  __shared__ __attribute__((aligned(16))) bf16 sK0[BN * D];
  __shared__ __attribute__((aligned(16))) bf16 sK1[BN * D];
  __shared__ __attribute__((aligned(16))) bf16 sV0[BN * D];
  __shared__ __attribute__((aligned(16))) bf16 sV1[BN * D];

  // each XCD takes whole heads (with the heads of a GQA group adjacent, whole
  // K/V streams); with `reverse` the longest query tiles go first
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
  const int rg = w / NSL;               // row group
  const int sl = w % NSL;               // output column slice: columns 32 NOB sl ..
  const int q0 = qt * BM;
  const int i = q0 + rg * 32 + n;
  const LogitK lk(p.sl2, p.xc, p.bc, p.cl2, CAP);
  const FragOfs<D, ROWPERM_TR> fo(lane);
  // the swizzle permutes 16-byte slots inside 128-column groups only, so a
  // slice's V^T fragments are those of column block ob at a column offset
  const int colofs = 32 * NOB * sl;

  const bf16* kbase = reinterpret_cast<const bf16*>(p.k) + koff(p, b, 0, hk, D);
  const bf16* vbase = reinterpret_cast<const bf16*>(p.v) + koff(p, b, 0, hk, D);
  const long kstride = p.kts;
  const TilePlan<BN, D, NT, true> kplan(kstride);
  const TilePlan<BN, D, NT, false> vplan(kstride);

  int lo_i = 0, hi_i = 0;
  if (i < Sq) keys_of(p.mask, b, i, lo_i, hi_i);
  const int ilast = min(q0 + BM, Sq) - 1;
  int lo_first, hi_first, lo_last, hi_last;
  keys_of(p.mask, b, q0, lo_first, hi_first);
  keys_of(p.mask, b, ilast, lo_last, hi_last);
  const bool dchk = dense_row(p.mask, b);
  const bool rows_full = (q0 + BM <= Sq) && !dchk;

  // Q^T fragments of this wave's 32 queries stay in registers
  bf16x8 qf[NCC];
  {
    const bf16* qrow = reinterpret_cast<const bf16*>(p.q) + qoff(p, b, min(i, Sq - 1), hq, D);
#pragma unroll
    for (int cc = 0; cc < NCC; ++cc) qf[cc] = *reinterpret_cast<const bf16x8*>(qrow + 16 * cc + 8 * h);
  }
  const bf16* brow = nullptr;
  if constexpr (BIAS) brow = reinterpret_cast<const bf16*>(p.bias) + b * p.bias_bs + hq * p.bias_hs + (long)min(i, Sq - 1) * Sk;

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

  // S^T = K Q^T of the tile in LDS (tile row kb*32 + r holds key kb*32 + swp(r))
  auto qk = [&](const bf16* tK, f32x16* s) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16{};
    // key block by key block, so that the logits of block 0 can run while
    // the MFMAs of block 1 do
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int cc = 0; cc < NCC; ++cc) mma(s[kb], fo.frag(tK, kb * 32, cc), qf[cc]);
    }
  };

  f32x16 scur[NKB];
  if (ntiles > 0) {
    kplan.issue(sK0, kbase, kstride, kbeg, Sk);
    vplan.issue(sV0, vbase, kstride, kbeg, Sk);
    if (PIPE && ntiles > 1) kplan.issue(sK1, kbase, kstride, kbeg + BN, Sk);
  }
  wait_loads();
  __syncthreads();
  if (PIPE && ntiles > 0) qk(sK0, scur);

  // tile t: PIPE: softmax of scur (tile t) while S of tile t+1 comes from
  // tK, DMA K_{t+2} -> wK; otherwise S of tile t from tK, DMA K_{t+1} -> wK.
  // Both: PV from tV, DMA V_{t+1} -> wV.
  auto step = [&](const bf16* tK, const bf16* tV, bf16* wK, bf16* wV, int t) {
    const int k0 = kbeg + t * BN;
    if (t + (PIPE ? 2 : 1) < ntiles) kplan.issue(wK, kbase, kstride, k0 + (PIPE ? 2 : 1) * BN, Sk);
    if (t + 1 < ntiles) vplan.issue(wV, vbase, kstride, k0 + BN, Sk);
    const bool next = t + 1 < ntiles;

    {
      f32x16 snext[NKB];
      if constexpr (PIPE) {
        if (next) qk(tK, snext);
      } else {
        qk(tK, scur);
      }
      // logits: CAP keeps r = 1/(1+2^y) (masked: +inf), else y (masked: -inf)
      float ext = CAP ? INFINITY : -INFINITY;
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
          float y = scur[kb][j] * lk.a;
          if constexpr (BIAS) y = fmaf(bv[j], lk.bb, y);
          float v;
          if constexpr (FIXM) v = __builtin_amdgcn_rcpf(fmaf(fast_exp2(y), kfix, kfix));
          else if constexpr (CAP) v = __builtin_amdgcn_rcpf(1.0f + fast_exp2(y));
          else v = y;
          if constexpr (decltype(masked)::value) {
            const int key = k0 + kb * 32 + acc_row(h, j);
            v = (key >= lo_i && key < hi_i && dense_ok(p.mask, dchk, b, i, key)) ? v : ((CAP && !FIXM) ? INFINITY : -INFINITY);
          }
          scur[kb][j] = v;
          if constexpr (!FIXM) ext = CAP ? fminf(ext, v) : fmaxf(ext, v);
        }
      }
      };
      if (rows_full && k0 >= lo_last && k0 + BN <= hi_first) logits(bool_c<false>{});
      else logits(bool_c<true>{});
      float base = 0.0f;
      if constexpr (!FIXM) {
        ext = CAP ? fminf(ext, xor32(ext)) : fmaxf(ext, xor32(ext));
        const float mx = CAP ? fmaf(ext, -2.0f * lk.c2, lk.c2) : ext;

        // lazy rescale: move the reference maximum only when it grew by > 8
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

      // probabilities of key block kb, then O^T += V^T P^T for that block
      // (V^T fragments by transposing LDS reads): the exponentials of block
      // kb + 1 can run while the MFMAs of block kb do
      float ps = 0.0f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float pv = FIXM  ? fast_exp2(scur[kb][j])
                           : CAP ? fast_exp2(fmaf(scur[kb][j], -2.0f * lk.c2, lk.c2 - base))
                                 : fast_exp2(scur[kb][j] - base);
          scur[kb][j] = pv;
        }
        bf16x8 pf[2];
        pf[0] = to_frag(scur[kb], 0, (bf16*)nullptr);
        pf[1] = to_frag(scur[kb], 8, (bf16*)nullptr);
        ps = sum_bf16x8(pf[1], sum_bf16x8(pf[0], ps));
        if constexpr (DROP) {
          // registers 8 m + e hold keys k0 + 32 kb + acc_row(h, 8 m + e) = k0 + 32 kb + 16 m + 8 h + e,
          // e = 0..7: the eight keys of one Philox evaluation
          const uint32_t th16 = p.drop.thresh << 16;
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            uint32_t c[4];
            draw8(p.drop, i, k0 + kb * 32 + acc_row(h, 8 * m), b * p.Hq + hq, c);
#pragma unroll
            for (int e = 0; e < 8; ++e) scur[kb][8 * m + e] = kept(c, e, th16) ? scur[kb][8 * m + e] : 0.0f;
          }
          pf[0] = to_frag(scur[kb], 0, (bf16*)nullptr);
          pf[1] = to_frag(scur[kb], 8, (bf16*)nullptr);
        }
        // V^T fragments of column block ob + 2 requested before the MFMAs of block ob
        {
          constexpr int TA = D > 128 ? 1 : 2;
          bf16x8 tv[TA + 1][2];
#pragma unroll
          for (int a2 = 0; a2 < TA; ++a2) {
#pragma unroll
            for (int sb = 0; sb < 2; ++sb) tv[a2][sb] = fo.frag_tr(tV + colofs, kb * 32 + 16 * sb, a2);
          }
#pragma unroll
          for (int ob = 0; ob < NOB; ++ob) {
            if (ob + TA < NOB) {
#pragma unroll
              for (int sb = 0; sb < 2; ++sb)
                tv[(ob + TA) % (TA + 1)][sb] = fo.frag_tr(tV + colofs, kb * 32 + 16 * sb, ob + TA);
            }
#pragma unroll
            for (int sb = 0; sb < 2; ++sb) mma(oacc[ob], tv[ob % (TA + 1)][sb], pf[sb]);
          }
        }
      }
      lsum += ps;
      if constexpr (PIPE) {
        // unconditional: after the last tile scur is not read again, and a
        // select per element would cost a VALU instruction per pair
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) scur[kb] = snext[kb];
      }
    }

    wait_loads();
    __syncthreads();
  };
  for (int t = 0; t < ntiles; t += 2) {
    if constexpr (PIPE) {
      step(sK1, sV0, sK0, sV1, t);
      if (t + 1 < ntiles) step(sK0, sV1, sK1, sV0, t + 1);
    } else {
      step(sK0, sV0, sK1, sV1, t);
      if (t + 1 < ntiles) step(sK1, sV1, sK0, sV0, t + 1);
    }
  }

  // ---- epilogue
  float ltot = lsum + xor32(lsum);
  float oscale = 1.0f;
  if constexpr (FIXM) {
    // the sink logit is not capped: move the reference to it if it is larger
    if (has_sink && sink2 > m) {
      oscale = fast_exp2(m - sink2);
      ltot *= oscale;
      m = sink2;
    }
  }
  if (has_sink) ltot += fast_exp2(sink2 - m);
  const float inv = ltot > 0.0f ? (DROP ? p.drop.scale : 1.0f) * oscale / ltot : 0.0f;
  if (i < Sq) {
    bf16* orow = reinterpret_cast<bf16*>(p.out) + qoff(p, b, i, hq, D);
    bf16* lorow = reinterpret_cast<bf16*>(p.out_lo) + qoff(p, b, i, hq, D);
#pragma unroll
    for (int ob = 0; ob < NOB; ++ob) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        float vals[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) vals[e] = oacc[ob][8 * hf + e] * inv;
        store8<bf16>(orow + colofs + ob * 32 + 16 * hf + 8 * h, vals);
        if (p.out_lo) store8_lo(lorow + colofs + ob * 32 + 16 * hf + 8 * h, vals);
      }
    }
    if (h == 0 && sl == 0) p.lse[((long)b * p.Hq + hq) * Sq + i] = ltot > 0.0f ? (m + __log2f(ltot)) * kLn2 : -INFINITY;
  }
}

// ============================================================== backward: dk, dv, dbias

// D = 64.  One workgroup = 4 waves = 128 keys of one KV head; the K^T
// fragments of each wave's 32 keys stay in registers and the workgroup's V
// rows stay in LDS (keeping the wave under 256 registers with both
// accumulators), dK^T / dV^T accumulate in registers over the GQA group's
// query heads and their visible 32-query tiles, which stream through a
// double-buffered LDS tile (rows stored through swp).  (D = 128 runs
// dkdv16_kernel.)
//
// DROP: dropout, with the keep decisions shared in quads of lanes (keys 4m ..
// 4m + 3) as in dkdv16_kernel: per run of four consecutive queries of a
// lane, lane t evaluates Philox4x32-10 for query t of the run, and the two
// quads of one eight-key evaluation split the runs between them.
template <int D, bool CAP, bool BIAS, bool DROP>
__global__ __launch_bounds__(256, 2) void dkdv_fast_kernel(BwdParams p) {
  static_assert(D == 64, "32-key waves at D = 64 only");
  constexpr int NT = 256;
  constexpr int BNK = 128;
  constexpr int BMQ = 32;
  constexpr int NOB = D / 32;
  constexpr int NCC = D / 16;

  __shared__ __attribute__((aligned(16))) bf16 sVr[BNK * D];
  __shared__ __attribute__((aligned(16))) bf16 sQ0[BMQ * D];
  __shared__ __attribute__((aligned(16))) bf16 sQ1[BMQ * D];
  __shared__ __attribute__((aligned(16))) bf16 sO0[BMQ * D];
  __shared__ __attribute__((aligned(16))) bf16 sO1[BMQ * D];
  __shared__ __attribute__((aligned(16))) float sL0[BMQ];
  __shared__ __attribute__((aligned(16))) float sL1[BMQ];
  __shared__ __attribute__((aligned(16))) float sD0[BMQ];
  __shared__ __attribute__((aligned(16))) float sD1[BMQ];

  // each XCD takes whole (batch row, KV head) groups, key block 0 (the
  // longest under a causal mask) first; all key blocks of a group sweep the
  // same query tiles (from the last one backwards, in step) through one L2
  int kb, hk, b, split;
  {
    int grp;
    xcd_order(gridDim.x, gridDim.y * gridDim.z, kb, grp);
    const int y = grp % gridDim.y;   // the splits of one KV head are adjacent
    hk = y / p.hsplit;
    split = y % p.hsplit;
    b = grp / gridDim.y;
  }
  const int GS = p.G / p.hsplit;     // query heads of this workgroup
  const int Sq = p.mask.Sq, Sk = p.mask.Sk;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int n = lane & 31;
  const int h = lane >> 5;
  const int k0 = kb * BNK;
  const int j = k0 + w * 32 + n;
  const int jc = min(j, Sk - 1);
  const long qstride = p.qts;
  const LogitK lk(p.sl2, p.xc, p.bc, p.cl2, CAP);
  const FragOfs<D, true> fo(lane);

  bf16x8 kf[NCC];
  {
    const bf16* krow = reinterpret_cast<const bf16*>(p.k) + koff(p, b, jc, hk, D);
#pragma unroll
    for (int cc = 0; cc < NCC; ++cc) kf[cc] = *reinterpret_cast<const bf16x8*>(krow + 16 * cc + 8 * h);
  }
  load_tile<BNK, D, NT, false>(sVr, reinterpret_cast<const bf16*>(p.v) + koff(p, b, 0, hk, D),
                               p.kts, k0, Sk);

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

  f32x16 kacc[NOB], vacc[NOB];
#pragma unroll
  for (int ob = 0; ob < NOB; ++ob) { kacc[ob] = f32x16{}; vacc[ob] = f32x16{}; }

  // item it = (query tile nqt - 1 - it / G counted from the end, query head
  // it % G of the group); its Q and dO tiles go straight to LDS, its lse and
  // delta (one row per thread of the first 32) through registers, written to
  // LDS after the current item's work so the load latency overlaps it.
  float nl = 0.0f, nd = 0.0f;
  int nq = 0;
  auto fetch = [&](int it, bf16* nQ, bf16* nO) {
    const int hq = hk * p.G + split * GS + it % GS;
    const int q0 = qbeg + (nqt - 1 - it / GS) * BMQ;
    const long hoff = qoff(p, b, 0, hq, D);
    load_tile<BMQ, D, NT, true>(nQ, reinterpret_cast<const bf16*>(p.q) + hoff, qstride, q0, Sq);
    load_tile<BMQ, D, NT, true>(nO, reinterpret_cast<const bf16*>(p.dout) + hoff, qstride, q0, Sq);
    if (threadIdx.x < BMQ) {
      nq = q0 + threadIdx.x;
      const long li = ((long)b * p.Hq + hq) * Sq + min(nq, Sq - 1);
      nl = p.lse[li];
      nd = p.delta[li];
    }
  };
  auto put_stats = [&](float* nL, float* nD) {
    if (threadIdx.x < BMQ) {
      // a query past the end, or one that sees nothing, contributes P = 0
      nL[threadIdx.x] = (nq < Sq && nl != -INFINITY) ? (CAP ? p.cl2 : 0.0f) - nl * kLog2e : -INFINITY;
      nD[threadIdx.x] = -nd;
    }
  };
  if (nitems > 0) {
    fetch(0, sQ0, sO0);
    put_stats(sL0, sD0);
  }
  wait_loads();
  __syncthreads();

  auto step = [&](const bf16* tQ, const bf16* tO, const float* tL, const float* tD, bf16* nQ, bf16* nO, float* nL,
                  float* nD, int it) {
    const bool more = it + 1 < nitems;
    if (more) fetch(it + 1, nQ, nO);
    const int hq = hk * p.G + split * GS + it % GS;
    const int q0 = qbeg + (nqt - 1 - it / GS) * BMQ;

    // ---- S = Q K^T, dP - delta = dO V^T - delta (rows: queries through swp;
    // columns: this wave's keys).  Per query the LDS stats hold
    // Lc = (cap ? c2 : 0) - lse2 and -delta; register r <-> query
    // q0 + acc_row(h, r), whose stats sit in f32x4 number
    // 4*(r/8) + 2h + (r/4)%2, element r%4.  The dP accumulator starts from
    // the -delta of its rows.
    const f32x4* L4 = reinterpret_cast<const f32x4*>(tL);
    const f32x4* D4 = reinterpret_cast<const f32x4*>(tD);
    f32x16 sacc = f32x16{}, dpacc;
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      const f32x4 nd4 = D4[4 * (e4 >> 1) + 2 * h + (e4 & 1)];
#pragma unroll
      for (int e = 0; e < 4; ++e) dpacc[4 * e4 + e] = nd4[e];
    }
#pragma unroll
    for (int cc = 0; cc < NCC; ++cc) {
      mma(sacc, fo.frag(tQ, 0, cc), kf[cc]);
      mma(dpacc, fo.frag(tO, 0, cc), fo.frag(sVr, w * 32, cc));
    }

    // ---- P and dU/4 = P (dP - delta) (1 - t^2)/4
    const bf16* bcol = nullptr;
    bf16* dbcol = nullptr;
    if constexpr (BIAS) {
      bcol = reinterpret_cast<const bf16*>(p.bias) + b * p.bias_bs + hq * p.bias_hs + jc;
      if (p.dbias) dbcol = reinterpret_cast<bf16*>(p.dbias) + (((long)b * p.Hq + hq) * Sq) * Sk + jc;
    }
    auto grads = [&](auto masked) {
      // dropout: bit r of kq keeps (query q0 + acc_row(h, r), key j); run u =
      // registers 4u .. 4u + 3 = queries q0 + acc_row(h, 4u) + 0..3
      unsigned kq = 0;
      if constexpr (DROP) {
        const int t = n & 3;
        // lanes n and n ^ 4 hold the two halves of the eight keys j & ~7 of one
        // evaluation: this lane evaluates runs 2 hf and 2 hf + 1 (hf = its half),
        // keeps its own four decisions and hands the other four to its partner
        const int hf = (n >> 2) & 1;
        int own[2], give = 0;
#pragma unroll
        for (int v = 0; v < 2; ++v) {
          const int u = 2 * hf + v;
          const unsigned k8 = keep8(p.drop, q0 + acc_row(h, 4 * u) + t, j & ~7, b * p.Hq + hq);
          own[v] = (int)((k8 >> (4 * hf)) & 15u);
          give |= (int)((k8 >> (4 - 4 * hf)) & 15u) << (4 * v);
        }
        const int got = from_lane_xor4(give, n);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int w4 = ((u >> 1) == hf) ? own[u & 1] : ((got >> (4 * (u & 1))) & 15);
          const int n0 = __builtin_amdgcn_update_dpp(0, w4, 0x00, 0xF, 0xF, false);
          const int n1 = __builtin_amdgcn_update_dpp(0, w4, 0x55, 0xF, 0xF, false);
          const int n2 = __builtin_amdgcn_update_dpp(0, w4, 0xAA, 0xF, 0xF, false);
          const int n3 = __builtin_amdgcn_update_dpp(0, w4, 0xFF, 0xF, 0xF, false);
          kq |= (unsigned)(((n0 >> t) & 1) | (((n1 >> t) & 1) << 1) | (((n2 >> t) & 1) << 2) |
                           (((n3 >> t) & 1) << 3)) << (4 * u);
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qi = q0 + acc_row(h, r);
        const int si = 4 * (r >> 3) + 2 * h + ((r >> 2) & 1);   // f32x4 of this query's stats
        float lc = L4[si][r & 3];
        // a masked pair gets Lc = -inf, hence P = 0, without a branch
        if constexpr (decltype(masked)::value) lc = (qi >= lo_j && qi < hi_j && dense_ok(p.mask, dchk, b, qi, j)) ? lc : -INFINITY;
        float bvv = 0.0f;
        if constexpr (BIAS) bvv = (float)bcol[(long)min(qi, Sq - 1) * Sk];
        float g;
        const float pv = prob_fast<CAP, BIAS>(sacc[r], bvv, lk, lc, g);
        float du, pd;
        if constexpr (DROP) {
          // m dP - delta = m (dP - delta) + (1 - m)(-delta), m = keep / (1 - p)
          const float mk = ((kq >> r) & 1u) ? p.drop.scale : 0.0f;
          du = pv * fmaf(mk, dpacc[r], (1.0f - mk) * D4[si][r & 3]) * g;
          pd = pv * mk;
        } else {
          du = pv * dpacc[r] * g;
          pd = pv;
        }
        sacc[r] = pd;
        dpacc[r] = du;
        if constexpr (BIAS) {
          const bool vis = decltype(masked)::value ? (qi >= lo_j && qi < hi_j) : true;
          if (dbcol && vis) dbcol[(long)qi * Sk] = (bf16)(du * kGrad4<CAP>);
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
    // dU^T of this (32-key, 32-query) block for the dq kernel, as the
    // fragments stand: element (key n, query 16sb + 8h + e) at
    // sb*512 + (n + 32h)*8 + e; one contiguous KiB per store instruction
    if (p.du && k0 + 32 * w < Sk) {
      bf16* blk = reinterpret_cast<bf16*>(p.du) +
                  ((((long)b * p.Hq + hq) * p.nkb32 + (k0 >> 5) + w) * p.nqb32 + (q0 >> 5)) * 1024 + lane * 8;
      __builtin_nontemporal_store(uf[0], reinterpret_cast<bf16x8*>(blk));
      __builtin_nontemporal_store(uf[1], reinterpret_cast<bf16x8*>(blk + 512));
    }

    // ---- dV^T += dO^T P,  dK^T += Q^T dU
    // The transposing reads keep their source order through scheduling, so
    // the fragments of column block ob + 1 are requested before the MFMAs of
    // block ob: eight reads stay in flight behind four MFMAs.
    bf16x8 tr_o[2][2], tr_q[2][2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      tr_o[0][sb] = fo.frag_tr(tO, 16 * sb, 0);
      tr_q[0][sb] = fo.frag_tr(tQ, 16 * sb, 0);
    }
#pragma unroll
    for (int ob = 0; ob < NOB; ++ob) {
      const int c = ob & 1;
      if (ob + 1 < NOB) {
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
          tr_o[c ^ 1][sb] = fo.frag_tr(tO, 16 * sb, ob + 1);
          tr_q[c ^ 1][sb] = fo.frag_tr(tQ, 16 * sb, ob + 1);
        }
      }
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        mma(vacc[ob], tr_o[c][sb], pf[sb]);
        mma(kacc[ob], tr_q[c][sb], uf[sb]);
      }
    }

    if (more) put_stats(nL, nD);
    wait_loads();
    __syncthreads();
  };
  for (int it = 0; it < nitems; it += 2) {
    step(sQ0, sO0, sL0, sD0, sQ1, sO1, sL1, sD1, it);
    if (it + 1 < nitems) step(sQ1, sO1, sL1, sD1, sQ0, sO0, sL0, sD0, it + 1);
  }

  if (j < Sk && p.hsplit > 1) {
    // unscaled fp32 partials of this split
    const long nel = (long)gridDim.z * Sk * p.Hkv * D;
    const long off = (((long)b * Sk + j) * p.Hkv + hk) * D;
    float* kp = p.dkv_part + (long)split * nel + off;
    float* vp = p.dkv_part + (long)(p.hsplit + split) * nel + off;
#pragma unroll
    for (int ob = 0; ob < NOB; ++ob) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int d = ob * 32 + 16 * hf + 8 * h;
#pragma unroll
        for (int e4 = 0; e4 < 2; ++e4) {
          f32x4 kv, vv;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            kv[e] = kacc[ob][8 * hf + 4 * e4 + e];
            vv[e] = vacc[ob][8 * hf + 4 * e4 + e];
          }
          *reinterpret_cast<f32x4*>(kp + d + 4 * e4) = kv;
          *reinterpret_cast<f32x4*>(vp + d + 4 * e4) = vv;
        }
      }
    }
  } else if (j < Sk) {
    const long off = koff(p, b, j, hk, D);
    bf16* krow = reinterpret_cast<bf16*>(p.dk) + off;
    bf16* vrow = reinterpret_cast<bf16*>(p.dv) + off;
#pragma unroll
    for (int ob = 0; ob < NOB; ++ob) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        float kv[8], vv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          kv[e] = kacc[ob][8 * hf + e] * (p.scale * kGrad4<CAP>);
          vv[e] = vacc[ob][8 * hf + e];
        }
        const int d = ob * 32 + 16 * hf + 8 * h;
        store8<bf16>(krow + d, kv);
        store8<bf16>(vrow + d, vv);
      }
    }
  }
}

// ============================================================== backward: dk, dv with 16-key waves

// D = 128.  One workgroup = 4 waves = 64 keys of one KV head, 16 keys per
// wave on v_mfma_f32_16x16x32_bf16: the wave's K and V rows stay in
// registers as fragments (16 registers each) and dK^T, dV^T take 64, so a
// wave needs well under 256 registers and two run per SIMD, each hiding the
// other's exponentials and LDS latency behind its MFMAs.  Per 32-query item:
//   S = Q K^T and dP - delta = dO V^T in 16x16 blocks (lane: key r, queries
//   16qb + 4g + e), P and dU/4 in place, then dV^T += dO^T P and
//   dK^T += Q^T dU with the accumulator pair of each quantity as the B
//   operand directly (contraction order sigma) and dO^T, Q^T fragments from
//   transposing reads of the same row-major tiles.
// The dU hand-off block (32 keys x 32 queries, 2 KiB) takes the two waves of
// a 32-key pair as its halves: half kh = w % 2, then chunk lane' = key
// kappa + 16 g' holding dU(16 kh + kappa, queries sigma(g', 0..7)).
//
// DROP: dropout.  The lanes of a quad (keys 4m .. 4m + 3, one lane each)
// hold the same four queries; lane t takes the decisions of query t of the
// four at keys 4m .. 4m + 3, and the quad exchanges them (DPP broadcasts).
// One Philox4x32-10 evaluation decides eight keys, held by two quads (lanes
// r and r ^ 4): with two or four query blocks per wave they split the blocks
// and swap halves, so a pair costs an eighth of an evaluation as in the
// forward (a quarter with one block per wave, at D = 256).  dV takes the kept
// probabilities times 1 / (1 - p), and dS = P (m dP - delta) with m = keep /
// (1 - p).
//
// PART (with BIAS, a bias broadcast over heads): dbias summed over the
// workgroup's query heads in LDS, one slab per workgroup column
// (p.dbias_np > 0), written only on the query rows the items cover.
template <int D, bool CAP, bool BIAS, int NW, int BMQ, bool DROP, bool PART>
__global__ __launch_bounds__(64 * NW, 8 / NW) void dkdv16_kernel(BwdParams p) {
  static_assert(BIAS || !PART, "head-summed dbias needs a bias");
  // D = 256: waves w and w + 1 share 16 keys and split dK^T, dV^T by columns
  // (and the query blocks of S, dP and dU between them: see QSPLIT)
  constexpr int NSL = D > 128 ? 2 : 1;
  constexpr int NT = 64 * NW;
  constexpr int BNK = 16 * NW / NSL;
  constexpr int NQB = BMQ / 16;
  constexpr int NKC = BMQ / 32;
  constexpr int NC = D / 32;
  constexpr int NOB = D / 16 / NSL;     // this wave's 16-column blocks

  __shared__ __attribute__((aligned(16))) bf16 sQ0[BMQ * D];
  __shared__ __attribute__((aligned(16))) bf16 sQ1[BMQ * D];
  __shared__ __attribute__((aligned(16))) bf16 sO0[BMQ * D];
  __shared__ __attribute__((aligned(16))) bf16 sO1[BMQ * D];
  __shared__ __attribute__((aligned(16))) float sL0[BMQ];
  __shared__ __attribute__((aligned(16))) float sL1[BMQ];
  __shared__ __attribute__((aligned(16))) float sD0[BMQ];
  __shared__ __attribute__((aligned(16))) float sD1[BMQ];
  // with a bias: the item's bias tile (BMQ queries x BNK keys) loaded with
  // the Q/dO tiles, and its dbias tile gathered here and written out as whole
  // rows during the next item; 16-byte chunks swizzled per row (bsw)
  constexpr int BT = BIAS ? BMQ * BNK : 8;
  // D = 256: the two waves of a key group each take half of an item's query
  // blocks for S, dP and the gradients, then swap their P and dU values
  // through LDS (both need all of them for their column slices of dV, dK)
  constexpr bool QSPLIT = NSL == 2;
  constexpr int QPW = NQB / NSL;          // query blocks per wave
  __shared__ __attribute__((aligned(16))) bf16 sX[QSPLIT ? NW * 64 * 8 * QPW : 8];
  __shared__ __attribute__((aligned(16))) bf16 sB0[BT];
  __shared__ __attribute__((aligned(16))) bf16 sB1[BT];
  __shared__ __attribute__((aligned(16))) bf16 sG0[BT];
  __shared__ __attribute__((aligned(16))) bf16 sG1[BT];
  // a bias broadcast over heads (p.dbias_np > 0): the dbias tile summed over
  // the workgroup's query heads of one query tile, in fp32, one buffer per
  // query tile in turn (written out during the next tile's first item)
  constexpr int BA = PART ? BT : 4;
  __shared__ __attribute__((aligned(16))) float sA0[BA];
  __shared__ __attribute__((aligned(16))) float sA1[BA];

  // XCD-aware, longest-first numbering and a lockstep query sweep, as in
  // the 32-key kernel
  int kb, hk, b, split;
  {
    int grp;
    xcd_order(gridDim.x, gridDim.y * gridDim.z, kb, grp);
    const int y = grp % gridDim.y;   // the splits of one KV head are adjacent
    hk = y / p.hsplit;
    split = y % p.hsplit;
    b = grp / gridDim.y;
  }
  const int GS = p.G / p.hsplit;     // query heads of this workgroup
  const int Sq = p.mask.Sq, Sk = p.mask.Sk;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6 ;
  const int kgi = w / NSL;              // key group
  const int sl = w % NSL;               // column slice: columns 16 NOB sl ..
  const int colofs = 16 * NOB * sl;
  const int r = lane & 15;
  const int g = lane >> 4;
  const int k0 = kb * BNK;
  const int kw = k0 + 16 * kgi;
  const int j = kw + r;
  const int jc = min(j, Sk - 1);
  const long qstride = p.qts;
  const LogitK lk(p.sl2, p.xc, p.bc, p.cl2, CAP);
  const Frag16Ofs<D> fo(lane);

  // K and V fragments of this wave's keys: lane r + 16g holds columns
  // 8(c + 4g) .. + 7 of key kw + r (the B operand of S = Q K^T, dP = dO V^T)
  bf16x8 kf[NC], vf[NC];
  {
    const long off = koff(p, b, jc, hk, D);
    const bf16* krow = reinterpret_cast<const bf16*>(p.k) + off;
    const bf16* vrow = reinterpret_cast<const bf16*>(p.v) + off;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      kf[c] = *reinterpret_cast<const bf16x8*>(krow + 8 * (c & 3) + 32 * g + 128 * (c >> 2));
      vf[c] = *reinterpret_cast<const bf16x8*>(vrow + 8 * (c & 3) + 32 * g + 128 * (c >> 2));
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

  float nl = 0.0f, nd = 0.0f;
  int nq = 0;
  auto fetch = [&](int it, bf16* nQ, bf16* nO) {
    const int hq = hk * p.G + split * GS + it % GS;
    const int q0 = qbeg + (nqt - 1 - it / GS) * BMQ;
    const long hoff = qoff(p, b, 0, hq, D);
    load_tile<BMQ, D, NT, false, true>(nQ, reinterpret_cast<const bf16*>(p.q) + hoff, qstride, q0, Sq);
    load_tile<BMQ, D, NT, false, true>(nO, reinterpret_cast<const bf16*>(p.dout) + hoff, qstride, q0, Sq);
    if (threadIdx.x < BMQ) {
      nq = q0 + threadIdx.x;
      const long li = ((long)b * p.Hq + hq) * Sq + min(nq, Sq - 1);
      nl = p.lse[li];
      nd = p.delta[li];
    }
  };
  auto put_stats = [&](float* nL, float* nD) {
    if (threadIdx.x < BMQ) {
      nL[threadIdx.x] = (nq < Sq && nl != -INFINITY) ? (CAP ? p.cl2 : 0.0f) - nl * kLog2e : -INFINITY;
      nD[threadIdx.x] = -nd;
    }
  };
  // bias tiles: rows R = queries q0 + R, 16-byte chunk c (keys k0 + 8c ..) in
  // slot c ^ bsw(R), so that the four row groups of a wave (rows 4 apart)
  // read disjoint banks
  constexpr int BCPR = BNK / 8;
  auto bsw = [](int R) { return 2 * ((R >> 2) & (BCPR / 2 - 1)); };
  auto bias_tile = [&](int it, bf16* nB) {
    if constexpr (BIAS) {
      const int hq = hk * p.G + split * GS + it % GS;
      const int q0 = qbeg + (nqt - 1 - it / GS) * BMQ;
      const bf16* g0 = reinterpret_cast<const bf16*>(p.bias) + b * p.bias_bs + hq * p.bias_hs + k0;
      const auto rsrc = rows_rsrc(g0, Sk, q0, Sq);
      const int past = (int)min((long)max(Sq - q0, 0) * Sk * 2, 0x7fffffffL);   // first byte past the range
      const int w64 = threadIdx.x >> 6;
#pragma unroll
      for (int u = 0; u < (BMQ * BCPR + NT - 1) / NT; ++u) {
        const int pw = u * NT + w64 * 64;
        if (pw < BMQ * BCPR) {
          const int pc = pw + lane;
          const int R = pc / BCPR, c = pc % BCPR;
          const int kc = 8 * (c ^ bsw(R));   // the chunk's first key in the tile (Sk % 8 == 0)
          // a chunk of keys past Sk reads as zeros (an offset past the buffer's
          // range, as rows past Sq do): the range holds whole rows from key k0
          // on, so those keys would otherwise read the next row, and past the
          // last row the bytes after the bias, which need not be finite
          dma16(rsrc, k0 + kc < Sk ? 2 * (R * Sk + kc) : past, nB + pw * 8);
        }
      }
    }
  };
  // the dbias tile of item it, gathered in tG, to global memory as whole rows
  // (partial mode: the sum over the query tile's heads, after its last head)
  auto store_dbias = [&](int it, const bf16* tG) {
    if constexpr (BIAS) {
      if (!p.dbias) return;
      const int q0 = qbeg + (nqt - 1 - it / GS) * BMQ;
      if constexpr (PART) {
        if (it % GS != GS - 1) return;
        const float* tA = ((it / GS) & 1) ? sA1 : sA0;
        bf16* g0 = reinterpret_cast<bf16*>(p.dbias) + (((long)b * p.dbias_np + hk * p.hsplit + split) * Sq) * Sk + k0;
#pragma unroll
        for (int u = 0; u < (BMQ * BCPR + NT - 1) / NT; ++u) {
          const int pc = u * NT + threadIdx.x;
          if (pc < BMQ * BCPR) {
            const int R = pc / BCPR, c = pc % BCPR;
            if (q0 + R < Sq && k0 + 8 * c < Sk) {
              const float* src = tA + R * BNK + 8 * (c ^ bsw(R));
              float vals[8];
#pragma unroll
              for (int e = 0; e < 8; ++e) vals[e] = src[e];
              store8<bf16>(g0 + (long)(q0 + R) * Sk + 8 * c, vals);
            }
          }
        }
        return;
      }
      const int hq = hk * p.G + split * GS + it % GS;
      bf16* g0 = reinterpret_cast<bf16*>(p.dbias) + (((long)b * p.Hq + hq) * Sq) * Sk + k0;
#pragma unroll
      for (int u = 0; u < (BMQ * BCPR + NT - 1) / NT; ++u) {
        const int pc = u * NT + threadIdx.x;
        if (pc < BMQ * BCPR) {
          const int R = pc / BCPR, c = pc % BCPR;
          if (q0 + R < Sq && k0 + 8 * c < Sk)
            *reinterpret_cast<bf16x8*>(g0 + (long)(q0 + R) * Sk + 8 * c) =
                *reinterpret_cast<const bf16x8*>(tG + R * BNK + 8 * (c ^ bsw(R)));
        }
      }
    }
  };
  // element (row R, key column cidx) of a swizzled bias tile
  auto bidx = [&](int R, int cidx) { return R * BNK + 8 * ((cidx >> 3) ^ bsw(R)) + (cidx & 7); };

  if (nitems > 0) {
    fetch(0, sQ0, sO0);
    bias_tile(0, sB0);
    put_stats(sL0, sD0);
  }
  wait_loads();
  __syncthreads();

  auto step = [&](const bf16* tQ, const bf16* tO, const float* tL, const float* tD, bf16* nQ, bf16* nO, float* nL,
                  float* nD, const bf16* tB, bf16* nB, bf16* tG, const bf16* pG, int it) {
    const bool more = it + 1 < nitems;
    if (more) {
      fetch(it + 1, nQ, nO);
      bias_tile(it + 1, nB);
    }
    if (it > 0) store_dbias(it - 1, pG);
    const int hq = hk * p.G + split * GS + it % GS;
    const int q0 = qbeg + (nqt - 1 - it / GS) * BMQ;

    // S and dP - delta; the stats of queries 16qb + 4g .. + 3 are one f32x4
    const f32x4* L4 = reinterpret_cast<const f32x4*>(tL);
    const f32x4* D4 = reinterpret_cast<const f32x4*>(tD);
    // this wave's query blocks: all of them, or (QSPLIT) qb = sl QPW + i
    constexpr int NQL = QSPLIT ? QPW : NQB;
    const int qb0 = QSPLIT ? sl * QPW : 0;
    f32x4 sacc[NQL], dpacc[NQL];
#pragma unroll
    for (int i = 0; i < NQL; ++i) {
      sacc[i] = f32x4{};
      dpacc[i] = D4[4 * (qb0 + i) + g];
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
#pragma unroll
      for (int i = 0; i < NQL; ++i) {
        mma16(sacc[i], fo.frag(tQ, 16 * (qb0 + i), c), kf[c]);
        mma16(dpacc[i], fo.frag(tO, 16 * (qb0 + i), c), vf[c]);
      }
    }
    // keep fragment reads in flight ahead of their MFMAs
    ATL_READ_AHEAD(8, 1, 2 * NC * NQL);

    const int bcol = 16 * kgi + r;      // this lane's key column in the bias tiles
    auto grads = [&](auto masked) {
      // DROP: lanes r and r ^ 4 hold the two halves of the eight keys j & ~7 of
      // one evaluation; with an even number of items, at each even item i lane
      // r evaluates item i + (its half) and hands its partner the partner's
      // half, which gives both lanes the decisions of items i and i + 1
      int w4n = 0;
#pragma unroll
      for (int i = 0; i < NQL; ++i) {
        const int qb = qb0 + i;
        const f32x4 l4 = L4[4 * qb + g];
        unsigned kq = 0xFu;   // bit e: keep (query q0 + 16 qb + 4g + e, key j)
        f32x4 md4{};          // -delta of those queries
        if constexpr (DROP) {
          const int t = r & 3;
          int w4;   // the decisions of query q0 + 16 qb + 4g + t at keys (j & ~3) + 0..3
          if constexpr (NQL % 2 == 0) {
            if (i % 2 == 0) {
              const int hf = (r >> 2) & 1;
              const unsigned k8 = keep8(p.drop, q0 + 16 * (qb + hf) + 4 * g + t, j & ~7, b * p.Hq + hq);
              const int own = (int)((k8 >> (4 * hf)) & 15u);
              const int got = from_lane_xor4((int)((k8 >> (4 - 4 * hf)) & 15u), r);
              w4 = hf ? got : own;
              w4n = hf ? own : got;
            } else {
              w4 = w4n;
            }
          } else {
            w4 = (int)keep4(p.drop, q0 + 16 * qb + 4 * g + t, j & ~3, b * p.Hq + hq);
          }
          const int n0 = __builtin_amdgcn_update_dpp(0, w4, 0x00, 0xF, 0xF, false);
          const int n1 = __builtin_amdgcn_update_dpp(0, w4, 0x55, 0xF, 0xF, false);
          const int n2 = __builtin_amdgcn_update_dpp(0, w4, 0xAA, 0xF, 0xF, false);
          const int n3 = __builtin_amdgcn_update_dpp(0, w4, 0xFF, 0xF, 0xF, false);
          kq = ((n0 >> t) & 1) | (((n1 >> t) & 1) << 1) | (((n2 >> t) & 1) << 2) | (((n3 >> t) & 1) << 3);
          md4 = D4[4 * qb + g];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int qi = q0 + 16 * qb + 4 * g + e;
          float lc = l4[e];
          if constexpr (decltype(masked)::value) lc = (qi >= lo_j && qi < hi_j && dense_ok(p.mask, dchk, b, qi, j)) ? lc : -INFINITY;
          float bvv = 0.0f;
          if constexpr (BIAS) bvv = (float)tB[bidx(16 * qb + 4 * g + e, bcol)];
          float gg;
          const float pv = prob_fast<CAP, BIAS>(sacc[i][e], bvv, lk, lc, gg);
          float du, pd;
          if constexpr (DROP) {
            // dP - delta sits on top of -delta (md4): m dP - delta = m (dP - delta) + (1 - m)(-delta)
            const float mk = ((kq >> e) & 1u) ? p.drop.scale : 0.0f;
            du = pv * fmaf(mk, dpacc[i][e], (1.0f - mk) * md4[e]) * gg;
            pd = pv * mk;
          } else {
            du = pv * dpacc[i][e] * gg;
            pd = pv;
          }
          sacc[i][e] = pd;
          dpacc[i][e] = du;
          // masked pairs have P = 0 and are written as zeros; each query block
          // by the one wave that computed it
          if constexpr (BIAS) {
            if (QSPLIT || sl == 0) {
              const int x = bidx(16 * qb + 4 * g + e, bcol);
              if constexpr (PART) {
                float* tA = ((it / GS) & 1) ? sA1 : sA0;
                tA[x] = (it % GS == 0 ? 0.0f : tA[x]) + du * kGrad4<CAP>;
              } else {
                tG[x] = (bf16)(du * kGrad4<CAP>);
              }
            }
          }
        }
      }
    };
    if (keys_full && q0 >= lo_last && q0 + BMQ <= hi_first) grads(bool_c<false>{});
    else grads(bool_c<true>{});
    bf16x8 pf[NKC], uf[NKC];
    if constexpr (QSPLIT) {
      static_assert(QPW == 1 && NKC == 1, "query split laid out for 32-query items");
      // lane's P and dU of its query block (bf16) out, the partner's in
      bf16x8 mine;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        mine[e] = (bf16)sacc[0][e];
        mine[4 + e] = (bf16)dpacc[0][e];
      }
      *reinterpret_cast<bf16x8*>(sX + (w * 64 + lane) * 8) = mine;
      __syncthreads();
      const bf16x8 other = *reinterpret_cast<const bf16x8*>(sX + ((w ^ 1) * 64 + lane) * 8);
      const bf16x8 lo = sl == 0 ? mine : other, hi = sl == 0 ? other : mine;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pf[0][e] = lo[e];
        pf[0][4 + e] = hi[e];
        uf[0][e] = lo[4 + e];
        uf[0][4 + e] = hi[4 + e];
      }
    } else {
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        pf[kc] = pack8(sacc[2 * kc], sacc[2 * kc + 1]);
        uf[kc] = pack8(dpacc[2 * kc], dpacc[2 * kc + 1]);
      }
    }
    // this wave's half of the dU block (32-key block of the pair, query block q0/32 + kc)
    if (p.du && sl == 0 && k0 + 16 * (kgi & ~1) < Sk) {
      bf16* blk = reinterpret_cast<bf16*>(p.du) +
                  ((((long)b * p.Hq + hq) * p.nkb32 + (kw >> 5)) * p.nqb32 + (q0 >> 5)) * 1024 + (kgi & 1) * 512 +
                  lane * 8;
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        // a ragged last item may end before its second 32-query block
        if (kc == 0 || q0 + 32 * kc < Sq)
          __builtin_nontemporal_store(uf[kc], reinterpret_cast<bf16x8*>(blk + kc * 1024));
      }
    }

    // dV^T += dO^T P, dK^T += Q^T dU (rows: columns 16 ob + 4g + e; lane's key r)
    // transposing reads keep their order through scheduling: request the
    // fragments of column block ob + TRA before the MFMAs of block ob
    constexpr int TRA = 2;
    bf16x8 tro[TRA + 1][NKC], trq[TRA + 1][NKC];
#pragma unroll
    for (int a = 0; a < TRA; ++a) {
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        tro[a][kc] = fo.frag_tr(tO + colofs, 32 * kc, a);
        trq[a][kc] = fo.frag_tr(tQ + colofs, 32 * kc, a);
      }
    }
#pragma unroll
    for (int ob = 0; ob < NOB; ++ob) {
      if (ob + TRA < NOB) {
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
          tro[(ob + TRA) % (TRA + 1)][kc] = fo.frag_tr(tO + colofs, 32 * kc, ob + TRA);
          trq[(ob + TRA) % (TRA + 1)][kc] = fo.frag_tr(tQ + colofs, 32 * kc, ob + TRA);
        }
      }
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        mma16(vacc[ob], tro[ob % (TRA + 1)][kc], pf[kc]);
        mma16(kacc[ob], trq[ob % (TRA + 1)][kc], uf[kc]);
      }
    }

    if (more) put_stats(nL, nD);
    wait_loads();
    __syncthreads();
  };
  for (int it = 0; it < nitems; it += 2) {
    step(sQ0, sO0, sL0, sD0, sQ1, sO1, sL1, sD1, sB0, sB1, sG0, sG1, it);
    if (it + 1 < nitems) step(sQ1, sO1, sL1, sD1, sQ0, sO0, sL0, sD0, sB1, sB0, sG1, sG0, it + 1);
  }
  if (nitems > 0) store_dbias(nitems - 1, ((nitems - 1) & 1) ? sG1 : sG0);

  if (j < Sk && p.hsplit > 1) {
    // unscaled fp32 partials of this split
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

  // dbias of this key block: the items wrote whole tiles over the query rows
  // [qbeg, qbeg + nqt BMQ); every other row sees none of the block's keys
  // (the visible query range of a key moves monotonically with the key), so
  // its dbias is zero.  Written here rather than by a separate pass, so that
  // these stores stream out while other workgroups compute.  (PART: left
  // unwritten in the slabs; the slab reduction recomputes the covered rows
  // and writes the zeros of the others into the result.)
  if constexpr (BIAS && !PART) {
    if (p.dbias) {
      const int z_lo = min(qbeg, Sq);
      const int z_hi = max(z_lo, min(qbeg + nqt * BMQ, Sq));
      const int nz = z_lo + (Sq - z_hi);
      const bf16x8 zero = {};
      for (int hh = 0; hh < GS; ++hh) {
        const int hq = hk * p.G + split * GS + hh;
        bf16* g0 = reinterpret_cast<bf16*>(p.dbias) + (((long)b * p.Hq + hq) * Sq) * Sk + k0;
        for (int u = threadIdx.x; u < nz * BCPR; u += NT) {
          const int R = u / BCPR, c = u % BCPR;
          const int i = R < z_lo ? R : z_hi + (R - z_lo);
          if (k0 + 8 * c < Sk) *reinterpret_cast<bf16x8*>(g0 + (long)i * Sk + 8 * c) = zero;
        }
      }
    }
  }
}

// ============================================================== backward: split reduction

// dk = kscale * sum of the dK partials, dv = sum of the dV partials, over the
// hsplit query-head splits in a fixed order (deterministic); 4 elements per
// thread, nel = B * Sk * Hkv * D (a multiple of 4).
// The partials are [B, Sk, Hkv, D] contiguous; dk and dv have the k-side
// layout's strides (kbs, kts; hd = Hkv * D elements per token).
template <typename T>
__global__ __launch_bounds__(256) void dkv_reduce_kernel(const float* part, int hsplit, long nel, float kscale, T* dk,
                                                        T* dv, int Sk, long hd, long kbs, long kts) {
  static_assert(std::is_same<T, bf16>::value, "bf16 outputs");
  const long i = 4 * ((long)blockIdx.x * 256 + threadIdx.x);
  if (i >= nel) return;
  f32x4 sk = f32x4{}, sv = f32x4{};
  for (int s = 0; s < hsplit; ++s) {
    sk += *reinterpret_cast<const f32x4*>(part + (long)s * nel + i);
    sv += *reinterpret_cast<const f32x4*>(part + (long)(hsplit + s) * nel + i);
  }
  bf16x4 ok, ov;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    ok[e] = (bf16)(sk[e] * kscale);
    ov[e] = (bf16)sv[e];
  }
  // 4 consecutive elements share a token (hd is a multiple of 4)
  const long tok = i / hd;
  const long o = (tok / Sk) * kbs + (tok % Sk) * kts + i % hd;
  *reinterpret_cast<bf16x4*>(dk + o) = ok;
  *reinterpret_cast<bf16x4*>(dv + o) = ov;
}

// ============================================================== backward: dq from dU

// A dU^T block of the workspace in LDS: 128 chunks of 16 bytes, chunk c
// (c = 64 sb + 32 h + key n, holding queries 16 sb + 8 h .. + 7) stored in
// slot c ^ (4 * ((c >> 5) & 3)), which makes the gather below conflict-free.
__device__ __forceinline__ int du_slot(int c) { return c ^ (((c >> 5) & 3) << 2); }

// B fragment of dQ^T += K^T dU^T for keys 16 sb .. 16 sb + 15 of the block:
// lane n + 32 g receives dU(key 16 sb + 8 g + i, query n), i = 0..7, from two
// transposing reads.  ds_read_b64_tr_b16 hands lane j of each 16-lane group
// element j % 4 of the 4-element chunk read by lane j / 4 + 4 e, e = 0..3, so
// source lane s points at key 16 sb + 8 g + 4 t + s / 4 and the four queries
// starting at 16 (G % 2) + 4 (s % 4) (G = lane / 16, t = which read).
__device__ __forceinline__ bf16x8 du_frag(const bf16* blk, int lane, int sb) {
  const int G = lane >> 4, s = lane & 15;
  const int c0 = (G & 1) * 64 + ((s & 3) >> 1) * 32 + 8 * (G >> 1) + (s >> 2) + 16 * sb;
  const v4i16 a = ds_tr16(blk + du_slot(c0) * 8 + 4 * (s & 1));
  const v4i16 b = ds_tr16(blk + du_slot(c0 + 4) * 8 + 4 * (s & 1));
  bf16x8 r;
  __builtin_memcpy(&r, &a, 8);
  __builtin_memcpy(reinterpret_cast<char*>(&r) + 8, &b, 8);
  return r;
}

// The same fragment from a block written by 16-key waves (D = 128): chunk c
// = 64 sb + kappa + 16 g' (key 16 sb + kappa, queries sigma(g', 0..7): the
// first 8 bytes queries 4g' .. + 3, the last 8 bytes 16 + 4g' .. + 3) sits in
// slot c ^ (4 * ((c >> 4) & 3)).  Source lane s of group G reads key
// 8 (G/2) + 4t + s/4 at the four queries 4 (4 (G%2) + s%4) .. + 3.
__device__ __forceinline__ int du_slot16(int c) { return c ^ (((c >> 4) & 3) << 2); }
__device__ __forceinline__ bf16x8 du_frag16(const bf16* blk, int lane, int sb) {
  const int G = lane >> 4, s = lane & 15;
  const int c0 = 64 * sb + 8 * (G >> 1) + (s >> 2) + 16 * (s & 3);
  const v4i16 a = ds_tr16(blk + du_slot16(c0) * 8 + 4 * (G & 1));
  const v4i16 b = ds_tr16(blk + du_slot16(c0 + 4) * 8 + 4 * (G & 1));
  bf16x8 r;
  __builtin_memcpy(&r, &a, 8);
  __builtin_memcpy(reinterpret_cast<char*>(&r) + 8, &b, 8);
  return r;
}

// dQ from the dU^T blocks the dk/dv kernel left in the workspace.  One
// workgroup = 4 waves = 128 queries of one query head; per 32-key block that
// some query of the wave sees, dQ^T += K^T dU^T on the MFMAs, with K^T from
// the shared key tile and dU^T from the wave's own 2 KiB block, both through
// transposing LDS reads.  No exponentials and no masks: the dk/dv kernel
// stored masked pairs as zeros, and it wrote every block that holds a
// visible pair (blocks no query of the wave sees are skipped, never read).
// With NSL > 1 (D = 512) the output columns split over NSL waves per 32-query
// group: they share the group's dU blocks (loaded by the first of them) and
// each accumulates D / NSL columns of dQ.
template <int D, bool CAP, int BN, int NST, int NSL = 1>
__global__ __launch_bounds__(256 * NSL, NSL > 1 ? 1 : (NST >= 3 ? 3 : 2)) void dq_du_kernel(BwdParams p) {
  constexpr int NT = 256 * NSL;
  constexpr int BM = 128;
  constexpr int NKB = BN / 32;
  constexpr int NOB = D / 32 / NSL;
  constexpr bool DU16 = D >= 128;   // blocks written by 16-key dk/dv waves
  static_assert(NST == 2 || NST == 3, "two or three tile stages");
  static_assert(NSL == 1 || NST == 2, "uneven load counts per thread need full waits");

  // NST stages of (K tile, this workgroup's dU blocks), distinct objects so
  // that the compiler sees a read of one never alias the DMA into another
  __shared__ __attribute__((aligned(16))) bf16 sK0[BN * D];
  __shared__ __attribute__((aligned(16))) bf16 sK1[BN * D];
  __shared__ __attribute__((aligned(16))) bf16 sK2[NST > 2 ? BN * D : 8];
  __shared__ __attribute__((aligned(16))) bf16 sU0[4 * NKB * 1024];
  __shared__ __attribute__((aligned(16))) bf16 sU1[4 * NKB * 1024];
  __shared__ __attribute__((aligned(16))) bf16 sU2[NST > 2 ? 4 * NKB * 1024 : 8];

  // XCD-aware, longest-first numbering as in the other kernels
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
  const int w = (threadIdx.x >> 6) / NSL;   // 32-query group
  const int sl = (threadIdx.x >> 6) % NSL;  // column slice
  const int n = lane & 31;
  const int h = lane >> 5;
  const int q0 = qt * BM;
  const int qw = q0 + 32 * w;        // this wave's first query
  const int i = qw + n;
  const FragOfs<D, true> fo(lane);

  const bf16* kbase = reinterpret_cast<const bf16*>(p.k) + koff(p, b, 0, hk, D);
  const long kstride = p.kts;

  const int ilast = min(q0 + BM, Sq) - 1;
  int lo_first, hi_first, lo_last, hi_last;
  keys_of(p.mask, b, q0, lo_first, hi_first);
  keys_of(p.mask, b, ilast, lo_last, hi_last);
  // this lane's query's visible keys [ilo, ihi) (empty past Sq)
  int ilo = 0, ihi = 0;
  if (i < Sq) keys_of(p.mask, b, i, ilo, ihi);
  const bf16* ublocks = reinterpret_cast<const bf16*>(p.du) +
                        (((long)b * p.Hq + hq) * p.nkb32 * p.nqb32 + (qw >> 5)) * 1024;
  const long ukstride = (long)p.nqb32 * 1024;   // elements between key blocks

  f32x16 qacc[NOB];
#pragma unroll
  for (int ob = 0; ob < NOB; ++ob) qacc[ob] = f32x16{};

  // a 32-key block is read when some query of the wave sees one of its keys
  // (a wave vote, so the same on every lane).  dk/dv wrote every such block:
  // the queries that see a key are an interval whose bounds never decrease
  // with the key, so the query tiles dk/dv covers for a key block hold them.
  // A query that sees no key contributes nothing, wherever keys_of puts its
  // empty interval (with k_start it can lie beyond the query's own position).
  auto visible = [&](int kb32) {
    return kb32 < Sk && __any(ilo < ihi && ilo < kb32 + 32 && ihi > kb32);
  };
  // the tile's K rows (all waves) and this wave's dU^T blocks; every thread
  // issues the same number of loads per tile (a block no query of the wave
  // sees is read through an empty range, which fills zeros and touches no
  // memory), so the loads of a later tile can be left in flight by count
  auto fetch = [&](int k0, bf16* tK, bf16* tU) {
    load_tile<BN, D, NT, true>(tK, kbase, kstride, k0, Sk);
    if (sl != 0) return;
#pragma unroll
    for (int kk = 0; kk < NKB; ++kk) {
      const bool vis = visible(k0 + 32 * kk);
      const bf16* blk = ublocks + (vis ? (long)((k0 >> 5) + kk) * ukstride : 0);
      const auto rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(blk), 0, vis ? 2048 : 0, 0x00020000);
#pragma unroll
      for (int u = 0; u < 2; ++u)
        dma16_nt(rsrc, 16 * (DU16 ? du_slot16(64 * u + lane) : du_slot(64 * u + lane)),
              tU + (w * NKB + kk) * 1024 + 64 * u * 8);
    }
  };

  const int kbeg = (lo_first / BN) * BN;
  const int nt = hi_last > kbeg ? (hi_last - kbeg + BN - 1) / BN : 0;
  if (nt > 0) fetch(kbeg, sK0, sU0);
  if (NST > 2 && nt > 1) fetch(kbeg + BN, sK1, sU1);
  if (NST > 2 && nt > 1) {
    // tile 0 landed, tile 1 may stay in flight
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(BN * D / 8 / NT + 2 * NKB) : "memory");
  } else {
    wait_loads();
  }
  __syncthreads();

  // tile t from (tK, tU); tile t + NST - 1 into (nK, nU), the buffers of tile t - 1
  auto step = [&](const bf16* tK, const bf16* tU, bf16* nK, bf16* nU, int t) __attribute__((always_inline)) {
    const int k0 = kbeg + t * BN;
    const bool issued = t + NST - 1 < nt;
    if (issued) fetch(kbeg + (t + NST - 1) * BN, nK, nU);
#pragma unroll
    for (int kk = 0; kk < NKB; ++kk) {
      if (visible(k0 + 32 * kk)) {
        const bf16* blk = tU + (w * NKB + kk) * 1024;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
          const bf16x8 uf = DU16 ? du_frag16(blk, lane, sb) : du_frag(blk, lane, sb);
#pragma unroll
          for (int ob = 0; ob < NOB; ++ob) mma(qacc[ob], fo.frag_tr(tK, 32 * kk + 16 * sb, sl * NOB + ob), uf);
        }
      }
    }
    // tile t + 1 landed; with three stages tile t + 2 may stay in flight
    if (NST > 2 && issued) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(BN * D / 8 / NT + 2 * NKB) : "memory");
    else wait_loads();
    __syncthreads();
  };
  if constexpr (NST == 2) {
    for (int t = 0; t < nt; t += 2) {
      step(sK0, sU0, sK1, sU1, t);
      if (t + 1 < nt) step(sK1, sU1, sK0, sU0, t + 1);
    }
  } else {
    for (int t = 0; t < nt; t += 3) {
      step(sK0, sU0, sK2, sU2, t);
      if (t + 1 < nt) step(sK1, sU1, sK0, sU0, t + 1);
      if (t + 2 < nt) step(sK2, sU2, sK1, sU1, t + 2);
    }
  }

  if (i < Sq) {
    bf16* drow = reinterpret_cast<bf16*>(p.dq) + qoff(p, b, i, hq, D);
#pragma unroll
    for (int ob = 0; ob < NOB; ++ob) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        float vals[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) vals[e] = qacc[ob][8 * hf + e] * (p.scale * kGrad4<CAP>);
        store8<bf16>(drow + (sl * NOB + ob) * 32 + 16 * hf + 8 * h, vals);
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
  constexpr bool ROWPERM_TR = true;   // K rows stored through swp
  constexpr int NOB = D / 32;
  constexpr int NCC = D / 16;

  // two LDS buffers per tile as distinct objects: the compiler can then see
  // that reading one never aliases the DMA filling the other
  __shared__ __attribute__((aligned(16))) bf16 sK0[BN * D];
  __shared__ __attribute__((aligned(16))) bf16 sK1[BN * D];
  __shared__ __attribute__((aligned(16))) bf16 sV0[BN * D];
  __shared__ __attribute__((aligned(16))) bf16 sV1[BN * D];

  // each XCD takes whole heads (with the heads of a GQA group adjacent, whole
  // K/V streams); with `reverse` the longest query tiles go first
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
  const int q0 = qt * BM;
  const int i = q0 + w * 32 + n;
  const LogitK lk(p.sl2, p.xc, p.bc, p.cl2, CAP);
  const FragOfs<D, ROWPERM_TR> fo(lane);

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

  const long row = ((long)b * p.Hq + hq) * Sq + min(i, Sq - 1);
  const float lse_i = p.lse[row];
  // Lc = (cap ? c2 : 0) - lse2; a query past the end or seeing nothing gets P = 0
  const float lc_i = (i < Sq && lse_i != -INFINITY) ? (CAP ? p.cl2 : 0.0f) - lse_i * kLog2e : -INFINITY;
  const float delta_i = p.delta[row];

  bf16x8 qf[NCC], of[NCC];
  {
    const long off = qoff(p, b, min(i, Sq - 1), hq, D);
    const bf16* qrow = reinterpret_cast<const bf16*>(p.q) + off;
    const bf16* orow = reinterpret_cast<const bf16*>(p.dout) + off;
#pragma unroll
    for (int cc = 0; cc < NCC; ++cc) {
      qf[cc] = *reinterpret_cast<const bf16x8*>(qrow + 16 * cc + 8 * h);
      of[cc] = *reinterpret_cast<const bf16x8*>(orow + 16 * cc + 8 * h);
    }
  }
  const bf16* brow = nullptr;
  if constexpr (BIAS) brow = reinterpret_cast<const bf16*>(p.bias) + b * p.bias_bs + hq * p.bias_hs + (long)min(i, Sq - 1) * Sk;

  f32x16 qacc[NOB];
#pragma unroll
  for (int ob = 0; ob < NOB; ++ob) qacc[ob] = f32x16{};

  const int kbeg = (lo_first / BN) * BN;
  if (kbeg < hi_last) {
    load_tile<BN, D, NT, true>(sK0, kbase, kstride, kbeg, Sk);
    load_tile<BN, D, NT, true>(sV0, vbase, kstride, kbeg, Sk);
  }
  wait_loads();
  __syncthreads();

  auto step = [&](const bf16* tK, const bf16* tV, bf16* nK, bf16* nV, int k0) {
    if (k0 + BN < hi_last) {
      load_tile<BN, D, NT, true>(nK, kbase, kstride, k0 + BN, Sk);
      load_tile<BN, D, NT, true>(nV, vbase, kstride, k0 + BN, Sk);
    }

    // ---- S^T = K Q^T, dP^T = V dO^T
    f32x16 sacc = f32x16{}, dpacc = f32x16{};
#pragma unroll
    for (int cc = 0; cc < NCC; ++cc) {
      mma(sacc, fo.frag(tK, 0, cc), qf[cc]);
      mma(dpacc, fo.frag(tV, 0, cc), of[cc]);
    }

    // ---- dU^T/4 = P^T (dP^T - delta) (1 - t^2)/4
    float bv[16];
    if constexpr (BIAS) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) load8(brow + min(k0 + 16 * hf + 8 * h, Sk - 8), bv + 8 * hf);
    }
    auto grads = [&](auto masked) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float g;
        float pv = prob_fast<CAP, BIAS>(sacc[r], BIAS ? bv[r] : 0.0f, lk, lc_i, g);
        if constexpr (decltype(masked)::value) {
          const int key = k0 + acc_row(h, r);
          pv = (key >= lo_i && key < hi_i && dense_ok(p.mask, dchk, b, i, key)) ? pv : 0.0f;
        }
        sacc[r] = pv * (dpacc[r] - delta_i) * g;
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
      for (int sb = 0; sb < 2; ++sb) mma(qacc[ob], fo.frag_tr(tK, 16 * sb, ob), uf[sb]);
    }

    wait_loads();
    __syncthreads();
  };
  for (int k0 = kbeg; k0 < hi_last; k0 += 2 * BN) {
    step(sK0, sV0, sK1, sV1, k0);
    if (k0 + BN < hi_last) step(sK1, sV1, sK0, sV0, k0 + BN);
  }

  if (i < Sq) {
    bf16* drow = reinterpret_cast<bf16*>(p.dq) + qoff(p, b, i, hq, D);
#pragma unroll
    for (int ob = 0; ob < NOB; ++ob) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        float vals[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) vals[e] = qacc[ob][8 * hf + e] * (p.scale * kGrad4<CAP>);
        store8<bf16>(drow + ob * 32 + 16 * hf + 8 * h, vals);
      }
    }
  }
}

}  // namespace ATL_NS
