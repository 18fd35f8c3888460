// C ABI of the soft-capped attention library: argument validation (fail
// closed: a requested cap or sink is never dropped), workspace layout and the
// launch sequence on the caller's stream.
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <climits>
#include <cstdio>
#include <mutex>
#include <string>

#include "attn_softcap.h"
#include "dispatch.hpp"

namespace atl {

// dsink[h] = sum of its partials, in a fixed order (deterministic)
__global__ __launch_bounds__(256) void dsink_final_kernel(const float* part, float* dsink, int nper) {
  const int hq = blockIdx.x;
  __shared__ float red[256];
  float s = 0.0f;
  for (int x = threadIdx.x; x < nper; x += 256) s += part[(long)hq * nper + x];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int st = 128; st > 0; st >>= 1) {
    if ((int)threadIdx.x < st) red[threadIdx.x] += red[threadIdx.x + st];
    __syncthreads();
  }
  if (threadIdx.x == 0) dsink[hq] = red[0];
}

// Per-token run [start, end) of packed segment ids: the maximal stretch of
// equal adjacent ids around the token.  One workgroup per batch row sweeps
// the row in chunks of 1024 tokens with a running maximum of run starts
// (forwards) and a running minimum of run ends (backwards), so that the runs
// of any id sequence are consistent (j lies in t's run iff t lies in j's);
// for ids that do not decrease along the row they are exactly the tokens of
// equal id.
__device__ __forceinline__ int wave_scan_max(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x = max(x, y);
  }
  return x;
}

__global__ __launch_bounds__(1024) void seg_from_ids_kernel(const int* ids, int* seg_lo, int* seg_hi, int S) {
  __shared__ int wtot[16];
  const int b = blockIdx.x;
  const int* row = ids + (long)b * S;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  // starts: inclusive prefix maximum of the boundary positions
  int carry = 0;
  for (int c0 = 0; c0 < S; c0 += 1024) {
    const int t = c0 + tid;
    int f = 0;
    if (t < S) f = (t == 0 || row[t] != row[t - 1]) ? t : 0;
    f = wave_scan_max(f);
    if (lane == 63) wtot[w] = f;
    __syncthreads();
    int pre = carry;
    for (int x = 0; x < w; ++x) pre = max(pre, wtot[x]);
    const int st = max(f, pre);
    if (t < S) seg_lo[(long)b * S + t] = st;
    int last = carry;
    for (int x = 0; x < 16; ++x) last = max(last, wtot[x]);
    __syncthreads();
    carry = last;
  }
  // ends: suffix minimum of the run ends, as a prefix maximum over -end
  // walking the row from its end
  carry = -S;
  for (int c0 = 0; c0 < S; c0 += 1024) {
    const int t = S - 1 - (c0 + tid);
    int f = -S;
    if (t >= 0) f = (t + 1 == S || row[t + 1] != row[t]) ? -(t + 1) : -S;
    f = wave_scan_max(f);
    if (lane == 63) wtot[w] = f;
    __syncthreads();
    int pre = carry;
    for (int x = 0; x < w; ++x) pre = max(pre, wtot[x]);
    const int en = -max(f, pre);
    if (t >= 0) seg_hi[(long)b * S + t] = en;
    int last = carry;
    for (int x = 0; x < 16; ++x) last = max(last, wtot[x]);
    __syncthreads();
    carry = last;
  }
}

// Per-token run from cumulative sequence lengths (THD layout, one row):
// [cu[s], cu[s+1]) for the sequence s holding the token; tokens before cu[0]
// form one run [0, cu[0]) and tokens at or past cu[nseq] one run
// [cu[nseq], T), so that the runs stay consistent for such inputs too
// (cu non-decreasing is required; the binary search assumes it).
__global__ __launch_bounds__(256) void seg_from_cu_kernel(const int* cu, int nseq, int* seg_lo, int* seg_hi, int T) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= T) return;
  int lo = 0, hi = nseq + 1;
  while (lo < hi) {  // first index with cu[x] > t
    const int mid = (lo + hi) >> 1;
    if (cu[mid] <= t) lo = mid + 1; else hi = mid;
  }
  int a, e;
  if (lo == 0) {
    a = 0;
    e = cu[0];
  } else if (lo > nseq) {
    a = cu[nseq];
    e = T;
  } else {
    a = cu[lo - 1];
    e = cu[lo];
  }
  seg_lo[t] = max(min(a, t), 0);
  seg_hi[t] = max(min(e, T), t + 1);
}

// k_start (first visible key per query, non-decreasing along a row): q_lo =
// its running maximum along the row (so that the bounds stay non-decreasing
// for any input; equal to k_start where it does not decrease), raised to the
// segment-run start where segments are given.  One workgroup per batch row.
__global__ __launch_bounds__(1024) void kstart_lo_kernel(const int* k_start, const int* seg_lo, int* q_lo, int Sq) {
  __shared__ int wtot[16];
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int carry = INT_MIN;
  for (int c0 = 0; c0 < Sq; c0 += 1024) {
    const int t = c0 + tid;
    int f = INT_MIN;
    if (t < Sq) f = k_start[(long)b * Sq + t];
    f = wave_scan_max(f);
    if (lane == 63) wtot[w] = f;
    __syncthreads();
    int pre = carry;
    for (int x = 0; x < w; ++x) pre = max(pre, wtot[x]);
    int lo = max(f, pre);
    if (t < Sq) {
      if (seg_lo) lo = max(lo, seg_lo[(long)b * Sq + t]);
      q_lo[(long)b * Sq + t] = lo;
    }
    int last = carry;
    for (int x = 0; x < 16; ++x) last = max(last, wtot[x]);
    __syncthreads();
    carry = last;
  }
}

// With k_start: the queries that see key j end at the first query whose
// (non-decreasing) q_lo passes j, cut to the segment run's end.
__global__ __launch_bounds__(256) void kstart_hi_kernel(const int* q_lo, const int* seg_hi, int* k_hi, int Sq, int Sk) {
  const int b = blockIdx.y;
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= Sk) return;
  const int* row = q_lo + (long)b * Sq;
  int lo = 0, hi = Sq;
  while (lo < hi) {  // first query with q_lo > j
    const int mid = (lo + hi) >> 1;
    if (row[mid] <= j) lo = mid + 1; else hi = mid;
  }
  if (seg_hi) lo = min(lo, seg_hi[(long)b * Sk + j]);
  k_hi[(long)b * Sk + j] = lo;
}

// Dense mask, first pass: per query row, the first visible key a, one past
// the last e (a = Sk, e = 0 for a row that sees none) and whether the row's
// visible keys are all of [a, e).  One wave per row; rows are read 16 bytes
// per lane when Sk is a multiple of 16 (the mask is 16-byte aligned), else a
// byte per lane.
__device__ __forceinline__ unsigned nonzero_bytes(unsigned w) {
  // bit 7 of each byte set iff that byte is nonzero
  return (((w & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | w) & 0x80808080u;
}
__global__ __launch_bounds__(256) void dense_rows_kernel(const unsigned char* mask, int Sq, int Sk, int* ra, int* re,
                                                         int* rc) {
  const int b = blockIdx.y;
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (i >= Sq) return;
  const unsigned char* row = mask + ((long)b * Sq + i) * Sk;
  int first = INT_MAX, last = -1, cnt = 0;
  if ((Sk & 15) == 0) {
    const uint4* row16 = reinterpret_cast<const uint4*>(row);
    for (int c = lane; c < Sk / 16; c += 64) {
      const uint4 v = row16[c];
      const unsigned wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const unsigned m = nonzero_bytes(wd[q]);
        if (m) {
          const int j0 = 16 * c + 4 * q;
          first = min(first, j0 + (__builtin_ctz(m) >> 3));
          last = max(last, j0 + ((31 - __builtin_clz(m)) >> 3));
          cnt += __builtin_popcount(m);
        }
      }
    }
  } else {
    for (int j = lane; j < Sk; j += 64) {
      if (row[j]) {
        first = min(first, j);
        last = max(last, j);
        ++cnt;
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    first = min(first, __shfl_xor(first, o, 64));
    last = max(last, __shfl_xor(last, o, 64));
    cnt += __shfl_xor(cnt, o, 64);
  }
  if (lane == 0) {
    const long t = (long)b * Sq + i;
    ra[t] = cnt ? first : Sk;
    re[t] = cnt ? last + 1 : 0;
    rc[t] = (cnt == 0 || cnt == last + 1 - first) ? 1 : 0;
  }
}

// Dense mask, second pass (one workgroup per batch row): non-decreasing
// envelopes A_i = min over rows i' >= i of a_i' and E_i = max over rows
// i' <= i of e_i', cut by the bounds of segments / k_start (lo_in, hi_in,
// nullable) into q_lo, q_hi.  The batch row is exact when every row's final
// range [q_lo, q_hi) is empty or lies inside its own [a, e) with all of
// [a, e) visible: the ranges then say everything the mask says.
__global__ __launch_bounds__(1024) void dense_bounds_kernel(const int* ra, const int* re, const int* rc,
                                                            const int* lo_in, const int* hi_in, int* q_lo, int* q_hi,
                                                            int* exact, int Sq, int Sk) {
  __shared__ int wtot[16];
  const int b = blockIdx.x;
  const long base = (long)b * Sq;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  // A: running maximum of -a from the last row backwards
  int carry = INT_MIN;
  for (int c0 = ((Sq - 1) / 1024) * 1024; c0 >= 0; c0 -= 1024) {
    const int t = c0 + 1023 - tid;
    int f = INT_MIN;
    if (t < Sq) f = -ra[base + t];
    f = wave_scan_max(f);
    if (lane == 63) wtot[w] = f;
    __syncthreads();
    int pre = carry;
    for (int x = 0; x < w; ++x) pre = max(pre, wtot[x]);
    if (t < Sq) q_lo[base + t] = -max(f, pre);
    int lastv = carry;
    for (int x = 0; x < 16; ++x) lastv = max(lastv, wtot[x]);
    __syncthreads();
    carry = lastv;
  }
  // E: running maximum of e; then the final ranges and their exactness
  carry = INT_MIN;
  int ok = 1;
  for (int c0 = 0; c0 < Sq; c0 += 1024) {
    const int t = c0 + tid;
    int f = INT_MIN;
    if (t < Sq) f = re[base + t];
    f = wave_scan_max(f);
    if (lane == 63) wtot[w] = f;
    __syncthreads();
    int pre = carry;
    for (int x = 0; x < w; ++x) pre = max(pre, wtot[x]);
    if (t < Sq) {
      int lo = q_lo[base + t];   // A_t, written by this workgroup above
      int hi = max(f, pre);      // E_t
      if (lo_in) lo = max(lo, lo_in[base + t]);
      hi = min(hi, hi_in ? hi_in[base + t] : Sk);
      q_lo[base + t] = lo;
      q_hi[base + t] = hi;
      ok &= rc[base + t] != 0 && (lo >= hi || (lo >= ra[base + t] && hi <= re[base + t]));
    }
    int lastv = carry;
    for (int x = 0; x < 16; ++x) lastv = max(lastv, wtot[x]);
    __syncthreads();
    carry = lastv;
  }
  ok = __syncthreads_and(ok);
  if (tid == 0) exact[b] = ok;
}

// Per key, the queries whose (non-decreasing) ranges [q_lo, q_hi) hold it:
// from the first query with q_hi > j to the first with q_lo > j.
__global__ __launch_bounds__(256) void rows_to_keys_kernel(const int* q_lo, const int* q_hi, int* k_lo, int* k_hi,
                                                           int Sq, int Sk) {
  const int b = blockIdx.y;
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= Sk) return;
  const int* rl = q_lo + (long)b * Sq;
  const int* rh = q_hi + (long)b * Sq;
  int lo = 0, hi = Sq;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (rh[mid] <= j) lo = mid + 1; else hi = mid;
  }
  const int first = lo;
  lo = first;
  hi = Sq;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (rl[mid] <= j) lo = mid + 1; else hi = mid;
  }
  k_lo[(long)b * Sk + j] = first;
  k_hi[(long)b * Sk + j] = lo;
}

// Scratch of attn_bwd_noalloc: the backward's workspace (segment runs,
// delta, sink-gradient partials, split partials, dU blocks when they fit) for
// callers that cannot allocate.  One copy per GPU the library runs on, held
// until the process ends; host code reaches it only through the address that
// hipGetSymbolAddress returns for the current device.
constexpr size_t kScratchBytes = (size_t)128 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

}  // namespace atl

// The fp16 unit's entry points (its argument structs have the layout of ours)
namespace atl_f16_bridge {
hipError_t fwd(int D, bool cap, bool bias, const void* p, const void* l);
hipError_t dq(int D, bool cap, bool bias, const void* p, const void* l);
hipError_t dkdv(int D, bool cap, bool bias, const void* p, const void* l);
hipError_t pre(int D, const void* out, const void* out_lo, const void* dout, const float* lse, float* delta,
               float* part, const float* sink, int sink_mode, int Hq, int rpb, const void* l);
hipError_t dbias_fill(void* dbias, const void* m, int Hq, int rpb, const void* l);
hipError_t dbias_reduce(const void* full, void* out, int Hq, int bcast, const void* part, int D, const void* l);
}  // namespace atl_f16_bridge

using namespace atl;

namespace {

hipError_t f16_fwd(int D, bool c, bool b, const FwdParams& p, const Launch& l) {
  return atl_f16_bridge::fwd(D, c, b, &p, &l);
}
hipError_t f16_dq(int D, bool c, bool b, const BwdParams& p, const Launch& l) {
  return atl_f16_bridge::dq(D, c, b, &p, &l);
}
hipError_t f16_dkdv(int D, bool c, bool b, const BwdParams& p, const Launch& l) {
  return atl_f16_bridge::dkdv(D, c, b, &p, &l);
}
hipError_t f16_pre(int D, const void* out, const void* out_lo, const void* dout, const float* lse, float* delta,
                   float* part, const float* sink, int sink_mode, int Hq, int rpb, const Launch& l) {
  return atl_f16_bridge::pre(D, out, out_lo, dout, lse, delta, part, sink, sink_mode, Hq, rpb, &l);
}
hipError_t f16_fill(void* dbias, const Mask& m, int Hq, int rpb, const Launch& l) {
  return atl_f16_bridge::dbias_fill(dbias, &m, Hq, rpb, &l);
}
hipError_t f16_reduce(const void* full, void* out, int Hq, int bcast, const Mask* part, int D, const Launch& l) {
  return atl_f16_bridge::dbias_reduce(full, out, Hq, bcast, part, D, &l);
}
const TypeOps& ops_fp16() {
  static const TypeOps o = {f16_fwd, f16_dq, f16_dkdv, f16_pre, f16_fill, f16_reduce};
  return o;
}

thread_local std::string g_err;

attn_status fail(attn_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

constexpr size_t kAlign = 256;
constexpr int kPreRows = 64;      // rows per block of the backward pre-pass
constexpr int kFillRows = 4;      // rows per block of the dbias zero fill

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool has_segments(const attn_args* a) { return a->segment_ids != nullptr || a->cu_seqlens != nullptr; }

// The kernels move rows 16 bytes at a time (vector loads, LDS DMA).
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// bf16 and fp16 run the same kernels (the 16-bit fast paths)
bool is16(const attn_args* a) { return a->dtype == ATTN_BF16 || a->dtype == ATTN_FP16; }

// Element strides of the q side and the k side for the layout
struct Strides {
  long qbs, qts, kbs, kts;
};
Strides strides_of(const attn_args* a) {
  const long qh = (long)a->Hq * a->D, kh = (long)a->Hkv * a->D;
  if (a->layout == ATTN_LAYOUT_SBHD) return {qh, qh * a->B, kh, kh * a->B};
  return {qh * a->Sq, qh, kh * a->Sk, kh};
}
long max_token_stride(const attn_args* a) {
  const Strides t = strides_of(a);
  return t.qts > t.kts ? t.qts : t.kts;
}

// The 16-bit dk/dv kernels that write dU blocks (fast.hpp D = 64 .. 256,
// wide.hpp D = 512 without a bias), with or without dropout; the generic
// kernels write none.
bool du_supported(const attn_args* a) {
  return a->dtype == ATTN_FP32 || fast_ok(is16(a), a->D, max_token_stride(a), a->Sk, a->bias != nullptr) ||
         wide_ok(is16(a), a->D, max_token_stride(a), a->Sk, a->bias != nullptr);
}

attn_status validate(const attn_args* a) {
  if (!a) return fail(ATTN_INVALID_ARGUMENT, "args is NULL");
  if (a->dtype != ATTN_BF16 && a->dtype != ATTN_FP32 && a->dtype != ATTN_FP16)
    return fail(ATTN_INVALID_ARGUMENT, "dtype must be ATTN_BF16, ATTN_FP16 or ATTN_FP32");
  if (a->B < 0 || a->Sq < 0 || a->Sk < 0) return fail(ATTN_INVALID_ARGUMENT, "B, Sq and Sk must be >= 0");
  if (a->Hq < 1 || a->Hkv < 1) return fail(ATTN_INVALID_ARGUMENT, "Hq and Hkv must be >= 1");
  if (a->Hq % a->Hkv != 0) return fail(ATTN_INVALID_ARGUMENT, "Hq must be a multiple of Hkv (GQA groups)");
  if (a->D != 64 && a->D != 128 && a->D != 256 && a->D != 512)
    return fail(ATTN_UNSUPPORTED, "head dim D must be 64, 128, 256 or 512");
  if (!(a->softcap >= 0.0f) || !std::isfinite(a->softcap))
    return fail(ATTN_INVALID_ARGUMENT, "softcap must be finite and >= 0 (0 turns the cap off)");
  if (!(a->scale >= 0.0f) || !std::isfinite(a->scale))
    return fail(ATTN_INVALID_ARGUMENT, "scale must be finite and >= 0 (0 means 1/sqrt(D))");
  if (a->sink_mode != ATTN_SINK_NONE && a->sink_mode != ATTN_SINK_OFF_BY_ONE && a->sink_mode != ATTN_SINK_LEARNABLE)
    return fail(ATTN_INVALID_ARGUMENT, "sink_mode must be NONE, OFF_BY_ONE or LEARNABLE");
  if (a->sink_mode == ATTN_SINK_LEARNABLE && !a->sink)
    return fail(ATTN_INVALID_ARGUMENT, "LEARNABLE sink needs the sink logits [Hq]");
  if (a->sink_mode != ATTN_SINK_LEARNABLE && a->sink)
    return fail(ATTN_INVALID_ARGUMENT, "sink logits given but sink_mode is not LEARNABLE");
  if (a->segment_ids && a->cu_seqlens) return fail(ATTN_INVALID_ARGUMENT, "give segment_ids or cu_seqlens, not both");
  if (a->cu_seqlens) {
    if (a->B != 1) return fail(ATTN_INVALID_ARGUMENT, "cu_seqlens (THD layout) needs B == 1");
    if (a->nseq < 1) return fail(ATTN_INVALID_ARGUMENT, "cu_seqlens needs nseq >= 1");
  }
  if (has_segments(a) && a->Sq != a->Sk) return fail(ATTN_INVALID_ARGUMENT, "packed segments need Sq == Sk");
  if (a->mask && ((uintptr_t)a->mask & 15) != 0) return fail(ATTN_INVALID_ARGUMENT, "mask must be 16-byte aligned");
  if (!(a->dropout_p >= 0.0f && a->dropout_p < 1.0f))
    return fail(ATTN_INVALID_ARGUMENT, "dropout_p must be in [0, 1)");
  if (a->layout != ATTN_LAYOUT_BSHD && a->layout != ATTN_LAYOUT_SBHD)
    return fail(ATTN_INVALID_ARGUMENT, "layout must be ATTN_LAYOUT_BSHD or ATTN_LAYOUT_SBHD");
  if (a->layout == ATTN_LAYOUT_SBHD && a->cu_seqlens && a->B != 1)
    return fail(ATTN_INVALID_ARGUMENT, "cu_seqlens needs B == 1");
  if (a->bias_bcast < 0 || a->bias_bcast > 3)
    return fail(ATTN_INVALID_ARGUMENT, "bias_bcast must be a combination of ATTN_BIAS_BCAST_BATCH and _HEADS");
  if (a->bias_bcast && !a->bias) return fail(ATTN_INVALID_ARGUMENT, "bias_bcast given without a bias");
  if (a->causal && a->Sq != a->Sk) return fail(ATTN_UNSUPPORTED, "causal masking needs Sq == Sk");
  const long long maxi = 2147483647LL;
  if ((long long)a->B * a->Sq > maxi || (long long)a->B * a->Sk > maxi)
    return fail(ATTN_UNSUPPORTED, "B*S must fit in int32");
  if (a->dq_mode != ATTN_DQ_AUTO && a->dq_mode != ATTN_DQ_DU_BLOCKS && a->dq_mode != ATTN_DQ_RECOMPUTE)
    return fail(ATTN_INVALID_ARGUMENT, "dq_mode must be ATTN_DQ_AUTO, ATTN_DQ_DU_BLOCKS or ATTN_DQ_RECOMPUTE");
  if (a->dq_mode == ATTN_DQ_DU_BLOCKS && !du_supported(a))
    return fail(ATTN_UNSUPPORTED, "ATTN_DQ_DU_BLOCKS needs fp32, or bf16 / fp16 with D = 64, 128, 256 or 512 (with a "
                                  "bias, Sk % 8 == 0)");
  if ((long long)a->B * a->Sq > 0 && a->Sk == 0) return fail(ATTN_UNSUPPORTED, "Sk == 0 with Sq > 0");
  const size_t elems = (size_t)a->B * (a->Sq + a->Sk);
  if (elems != 0 && (!a->q || !a->k || !a->v)) return fail(ATTN_INVALID_ARGUMENT, "q, k and v must not be NULL");
  if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->bias))
    return fail(ATTN_INVALID_ARGUMENT, "q, k, v and bias must be 16-byte aligned");
  return ATTN_OK;
}

// Per-token visibility bounds in the workspace: the segment runs (two
// [B*Sq] arrays), with k_start q_lo [B*Sq] and k_hi [B*Sk], and with a dense
// mask the per-row scan (three [B*Sq] arrays), the final q_lo, q_hi [B*Sq],
// k_lo, k_hi [B*Sk] and one exactness flag per batch row.
size_t seg_bytes(const attn_args* a) {
  const size_t nq = align_up((size_t)a->B * a->Sq * sizeof(int)), nk = align_up((size_t)a->B * a->Sk * sizeof(int));
  size_t n = has_segments(a) ? 2 * nq : 0;
  if (a->k_start) n += nq + nk;
  if (a->mask) n += 5 * nq + 2 * nk + align_up((size_t)a->B * sizeof(int));
  return n;
}

size_t pre_blocks(const attn_args* a) { return ((size_t)a->Sq + kPreRows - 1) / kPreRows; }

size_t fwd_ws(const attn_args* a) { return seg_bytes(a); }

// The bf16 kernels for head dims 64/128/256/512 can hand dU from the dk/dv
// kernel to the dq kernel through the workspace (bf16, 32-key x 32-query
// blocks), so that dq needs neither exponentials nor a second pass over the
// logits.  The buffer holds every block of [B, Hq, Sq, Sk]; ATTN_DQ_AUTO
// takes it for D >= 128 while it stays within kDuAutoBytes, else dq
// recomputes (at D = 64 the round trip of 2 bytes per pair costs more than
// recomputing 4 * 64 flop of it: measured 1.15 against 1.10 ms per step on
// B=1, Hq=64, Hkv=8, S=4096 with a learnable sink).
constexpr size_t kDuAutoBytes = (size_t)16 << 30;

size_t elem_bytes(const attn_args* a) { return a->dtype == ATTN_FP32 ? 4 : 2; }

// 32 x 32 blocks of dU in the element type (fp32 for the fp32 path)
size_t du_raw_bytes(const attn_args* a) {
  return (size_t)a->B * a->Hq * (((size_t)a->Sk + 31) / 32) * (((size_t)a->Sq + 31) / 32) * 1024 * elem_bytes(a);
}

bool du_path(const attn_args* a) {
  if (!du_supported(a) || a->dq_mode == ATTN_DQ_RECOMPUTE) return false;
  // at D = 64 recomputing is faster, except with dropout (whose recomputing
  // dq kernel is the generic one)
  return a->dq_mode == ATTN_DQ_DU_BLOCKS ||
         ((a->D >= 128 || a->dropout_p > 0.0f) && du_raw_bytes(a) <= kDuAutoBytes);
}

// With a bias, the bf16 dk/dv kernel of D = 128 and 256 writes the whole of
// dbias, the zeros of the masked pairs included; elsewhere the pre-pass
// writes those zeros and the dk/dv kernel the visible pairs.
bool dkdv_writes_dbias_zeros(const attn_args* a) {
  return a->bias != nullptr && (a->D == 128 || a->D == 256) &&
         fast_ok(is16(a), a->D, max_token_stride(a), a->Sk, true);
}

// Query-head splits of the bf16 dk/dv kernels (both take 128 keys per
// workgroup): the smallest divisor of G that gives at least 1024 workgroups
// (four per CU), so that a small batch with a wide GQA group does not leave
// the GPU to a few long workgroups; 1 when there are enough already.
int head_split(const attn_args* a) {
  const bool bf = is16(a), bias = a->bias != nullptr;
  const bool wide = wide_ok(bf, a->D, max_token_stride(a), a->Sk, bias);
  if (!fast_ok(bf, a->D, max_token_stride(a), a->Sk, bias) && !wide) return 1;
  const int bnk = wide ? 32 : 128;   // keys per dk/dv workgroup (as counted here)
  const long wgs = (long)((a->Sk + bnk - 1) / bnk) * a->Hkv * a->B;
  const int G = a->Hq / a->Hkv;
  int hs = 1;
  for (int s = 2; s <= G && wgs * hs < 1024; ++s)
    if (G % s == 0) hs = s;
  return hs;
}

size_t dkv_part_bytes(const attn_args* a) {
  const int hs = head_split(a);
  return hs > 1 ? (size_t)2 * hs * a->B * a->Sk * a->Hkv * a->D * sizeof(float) : 0;
}


// A bias broadcast over heads on the 16-key dk/dv kernel: each workgroup
// column (KV head and query-head split) sums its heads' dbias tiles in LDS
// and writes one [Sq, Sk] slab per batch row; 0 otherwise.
int dbias_partials(const attn_args* a) {
  return a->bias && (a->bias_bcast & ATTN_BIAS_BCAST_HEADS) && dkdv_writes_dbias_zeros(a) ? a->Hkv * head_split(a)
                                                                                             : 0;
}

// A broadcast bias: the kernels write the full [B, Hq, Sq, Sk] dbias (or the
// [B, partials, Sq, Sk] slabs above) here, reduced into the caller's dbias
// afterwards.
size_t dbias_full_bytes(const attn_args* a) {
  if (!a->bias || !a->bias_bcast) return 0;
  const int np = dbias_partials(a);
  return align_up((size_t)a->B * (np > 0 ? np : a->Hq) * a->Sq * a->Sk * elem_bytes(a));
}

size_t bwd_ws(const attn_args* a) {
  size_t s = seg_bytes(a) + dbias_full_bytes(a);
  s += align_up((size_t)a->B * a->Hq * a->Sq * sizeof(float));  // delta
  if (a->sink_mode == ATTN_SINK_LEARNABLE) s += align_up((size_t)a->Hq * a->B * pre_blocks(a) * sizeof(float));
  if (du_path(a)) s += align_up(du_raw_bytes(a));
  s += align_up(dkv_part_bytes(a));
  return s;
}

const TypeOps& ops(const attn_args* a) {
  return a->dtype == ATTN_BF16 ? ops_bf16() : a->dtype == ATTN_FP16 ? ops_fp16() : ops_f32();
}

// Lays the bounds out in the workspace (advancing ws) and, with launch,
// computes them on stream s.
hipError_t prep_bounds(const attn_args* a, char*& ws, Mask& m, hipStream_t s, bool launch) {
  m.q_lo = m.q_hi = m.k_lo = m.k_hi = nullptr;
  const size_t nq = align_up((size_t)a->B * a->Sq * sizeof(int)), nk = align_up((size_t)a->B * a->Sk * sizeof(int));
  int* seg_lo = nullptr;
  int* seg_hi = nullptr;
  if (has_segments(a)) {
    seg_lo = reinterpret_cast<int*>(ws);
    seg_hi = reinterpret_cast<int*>(ws + nq);
    ws += 2 * nq;
    if (launch) {
      if (a->segment_ids) seg_from_ids_kernel<<<a->B, 1024, 0, s>>>(a->segment_ids, seg_lo, seg_hi, a->Sq);
      else seg_from_cu_kernel<<<(a->Sq + 255) / 256, 256, 0, s>>>(a->cu_seqlens, a->nseq, seg_lo, seg_hi, a->Sq);
    }
    m.q_lo = m.k_lo = seg_lo;
    m.q_hi = m.k_hi = seg_hi;
  }
  if (a->k_start) {
    int* q_lo = reinterpret_cast<int*>(ws);
    int* k_hi = reinterpret_cast<int*>(ws + nq);
    ws += nq + nk;
    if (launch) {
      kstart_lo_kernel<<<a->B, 1024, 0, s>>>(a->k_start, seg_lo, q_lo, a->Sq);
      if (a->Sk > 0) kstart_hi_kernel<<<dim3((a->Sk + 255) / 256, a->B), 256, 0, s>>>(q_lo, seg_hi, k_hi, a->Sq, a->Sk);
    }
    m.q_lo = q_lo;
    m.k_hi = k_hi;
  }
  if (a->mask) {
    // ranges from the mask itself, cut by the bounds above; where they say
    // all the mask says, the kernels skip its per-pair reads
    int* ra = reinterpret_cast<int*>(ws);
    int* re = reinterpret_cast<int*>(ws + nq);
    int* rc = reinterpret_cast<int*>(ws + 2 * nq);
    int* q_lo = reinterpret_cast<int*>(ws + 3 * nq);
    int* q_hi = reinterpret_cast<int*>(ws + 4 * nq);
    int* k_lo = reinterpret_cast<int*>(ws + 5 * nq);
    int* k_hi = reinterpret_cast<int*>(ws + 5 * nq + nk);
    int* exact = reinterpret_cast<int*>(ws + 5 * nq + 2 * nk);
    ws += 5 * nq + 2 * nk + align_up((size_t)a->B * sizeof(int));
    if (launch && a->Sq > 0) {
      dense_rows_kernel<<<dim3((a->Sq + 3) / 4, a->B), 256, 0, s>>>(a->mask, a->Sq, a->Sk, ra, re, rc);
      dense_bounds_kernel<<<a->B, 1024, 0, s>>>(ra, re, rc, m.q_lo, m.q_hi, q_lo, q_hi, exact, a->Sq, a->Sk);
      rows_to_keys_kernel<<<dim3((a->Sk + 255) / 256, a->B), 256, 0, s>>>(q_lo, q_hi, k_lo, k_hi, a->Sq, a->Sk);
    }
    m.q_lo = q_lo;
    m.q_hi = q_hi;
    m.k_lo = k_lo;
    m.k_hi = k_hi;
    m.exact = exact;
  }
  return launch ? hipGetLastError() : hipSuccess;
}

// Element strides of the bias over batch rows and query heads (0 where broadcast)
void bias_strides(const attn_args* a, long& bs, long& hs) {
  const long SS = (long)a->Sq * a->Sk;
  hs = (a->bias_bcast & ATTN_BIAS_BCAST_HEADS) ? 0 : SS;
  bs = (a->bias_bcast & ATTN_BIAS_BCAST_BATCH) ? 0 : ((a->bias_bcast & ATTN_BIAS_BCAST_HEADS) ? 1 : a->Hq) * SS;
}

Dropout dropout_of(const attn_args* a) {
  Dropout d;
  d.on = a->dropout_p > 0.0f;
  const double t = std::floor((double)a->dropout_p * 65536.0);
  d.thresh = (uint32_t)(t > 65535.0 ? 65535.0 : t);
  d.seed_lo = (uint32_t)(a->dropout_seed & 0xFFFFFFFFu);
  d.seed_hi = (uint32_t)(a->dropout_seed >> 32);
  d.offset = (uint32_t)(a->dropout_offset & 0xFFFFFFFFu);
  d.scale = (float)(65536.0 / (65536.0 - (double)d.thresh));
  return d;
}

Mask base_mask(const attn_args* a) {
  Mask m;
  m.q_lo = m.q_hi = m.k_lo = m.k_hi = nullptr;
  m.dense = a->mask;
  m.exact = nullptr;
  m.Sq = a->Sq;
  m.Sk = a->Sk;
  m.causal = a->causal ? 1 : 0;
  m.window = a->window > 0 ? a->window : 0;
  return m;
}

void fill_consts(const attn_args* a, float& scale, float& sl2, float& xc, float& bc, float& cl2) {
  scale = a->scale > 0.0f ? a->scale : 1.0f / std::sqrt((float)a->D);
  sl2 = scale * kLog2e;
  if (a->softcap > 0.0f) {
    xc = scale / a->softcap;
    bc = 1.0f / a->softcap;
    cl2 = a->softcap * kLog2e;
  } else {
    xc = bc = cl2 = 0.0f;
  }
}

attn_status hip_fail(hipError_t e, const char* what) {
  return fail(ATTN_HIP_ERROR, std::string(what) + ": " + hipGetErrorString(e));
}

// Device address of `scratch` on the stream's device (which must be the
// current device), looked up once per device.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

attn_status scratch_for(void* stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (stream) {
    int sdev = -1;
    e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev);
    if (e != hipSuccess) return hip_fail(e, "hipStreamGetDevice");
    if (sdev != dev) return fail(ATTN_INVALID_ARGUMENT, "the stream must belong to the current device");
  }
  if (dev < 0 || dev >= kMaxDevices) return fail(ATTN_UNSUPPORTED, "device index beyond 63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ATTN_OK;
}

}  // namespace

extern "C" {

attn_status attn_validate(const attn_args* a) {
  g_err.clear();
  return validate(a);
}

size_t attn_fwd_workspace_size(const attn_args* a) {
  if (validate(a) != ATTN_OK) return (size_t)-1;
  return fwd_ws(a);
}

size_t attn_bwd_workspace_size(const attn_args* a) {
  if (validate(a) != ATTN_OK) return (size_t)-1;
  return bwd_ws(a);
}

const char* attn_last_error(void) { return g_err.c_str(); }

attn_status attn_fwd(const attn_args* a, void* out, float* lse, void* out_lo, void* workspace,
                     size_t workspace_bytes, void* stream) {
  g_err.clear();
  attn_status st = validate(a);
  if (st != ATTN_OK) return st;
  const size_t need = fwd_ws(a);
  if (workspace_bytes < need || (need && !workspace))
    return fail(ATTN_INVALID_ARGUMENT, "workspace smaller than attn_fwd_workspace_size");
  if (((uintptr_t)workspace & 255) != 0) return fail(ATTN_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  if ((size_t)a->B * a->Sq * a->Hq == 0) return ATTN_OK;
  if (!out || !lse) return fail(ATTN_INVALID_ARGUMENT, "out and lse must not be NULL");
  if (!aligned16(out) || !aligned16(out_lo)) return fail(ATTN_INVALID_ARGUMENT, "out and out_lo must be 16-byte aligned");
  if (out_lo && a->dtype == ATTN_FP32) return fail(ATTN_INVALID_ARGUMENT, "out_lo is for bf16 and fp16 outputs only");
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  FwdParams p;
  p.q = a->q;
  p.k = a->k;
  p.v = a->v;
  p.bias = a->bias;
  bias_strides(a, p.bias_bs, p.bias_hs);
  p.out = out;
  p.lse = lse;
  p.out_lo = out_lo;
  const Strides st_ = strides_of(a);
  p.qbs = st_.qbs;
  p.qts = st_.qts;
  p.kbs = st_.kbs;
  p.kts = st_.kts;
  p.mask = base_mask(a);
  p.drop = dropout_of(a);
  hipError_t e = prep_bounds(a, ws, p.mask, s, true);
  if (e != hipSuccess) return hip_fail(e, "segment preparation launch");
  p.Hq = a->Hq;
  p.Hkv = a->Hkv;
  p.G = a->Hq / a->Hkv;
  float scale;
  fill_consts(a, scale, p.sl2, p.xc, p.bc, p.cl2);
  p.sink = a->sink;
  p.sink_mode = a->sink_mode;
  p.reverse = a->causal ? 1 : 0;
  const Launch l{a->B, a->Sq, a->Sk, s, st_.qbs, st_.qts, st_.kbs, st_.kts};
  e = ops(a).fwd(a->D, a->softcap > 0.0f, a->bias != nullptr, p, l);
  if (e != hipSuccess) return hip_fail(e, "forward kernel launch");
  return ATTN_OK;
}

// The three backward phases share one workspace: segment runs, delta and
// the sink-gradient partials are written by the pre-pass and read by the
// dq and dk/dv kernels.
enum { kPhasePre = 1, kPhaseDq = 2, kPhaseDkdv = 4 };

static attn_status bwd_impl(const attn_args* a, const void* out, const void* out_lo, const float* lse, const void* dout, void* dq,
                            void* dk, void* dv, void* dbias, float* dsink, void* workspace, size_t workspace_bytes,
                            void* stream, int phases) {
  g_err.clear();
  attn_status st = validate(a);
  if (st != ATTN_OK) return st;
  if (dbias && !a->bias) return fail(ATTN_INVALID_ARGUMENT, "dbias requested without a bias");
  if (phases & kPhasePre) {
    if (a->sink_mode == ATTN_SINK_LEARNABLE && !dsink)
      return fail(ATTN_INVALID_ARGUMENT, "LEARNABLE sink needs dsink [Hq] for its gradient");
    if (a->sink_mode != ATTN_SINK_LEARNABLE && dsink)
      return fail(ATTN_INVALID_ARGUMENT, "dsink given but the sink is not LEARNABLE");
  }
  const size_t need = bwd_ws(a);
  if (workspace_bytes < need || (need && !workspace))
    return fail(ATTN_INVALID_ARGUMENT, "workspace smaller than attn_bwd_workspace_size");
  if (((uintptr_t)workspace & 255) != 0) return fail(ATTN_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  if ((size_t)a->B * (a->Sq + a->Sk) == 0) return ATTN_OK;
  if (!lse || !dout) return fail(ATTN_INVALID_ARGUMENT, "lse and dout must not be NULL");
  if ((phases & kPhasePre) && !out) return fail(ATTN_INVALID_ARGUMENT, "out must not be NULL");
  if ((phases & kPhaseDq) && !dq) return fail(ATTN_INVALID_ARGUMENT, "dq must not be NULL");
  if ((phases & kPhaseDkdv) && (!dk || !dv)) return fail(ATTN_INVALID_ARGUMENT, "dk and dv must not be NULL");
  if (!aligned16(out) || !aligned16(out_lo) || !aligned16(dout) || !aligned16(dq) || !aligned16(dk) ||
      !aligned16(dv) || !aligned16(dbias))
    return fail(ATTN_INVALID_ARGUMENT, "out, out_lo, dout, dq, dk, dv and dbias must be 16-byte aligned");
  if (out_lo && a->dtype == ATTN_FP32) return fail(ATTN_INVALID_ARGUMENT, "out_lo is for bf16 and fp16 outputs only");
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  BwdParams p;
  p.q = a->q;
  p.k = a->k;
  p.v = a->v;
  p.bias = a->bias;
  bias_strides(a, p.bias_bs, p.bias_hs);
  p.dout = dout;
  p.lse = lse;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.dbias = dbias;
  const Strides st_ = strides_of(a);
  p.qbs = st_.qbs;
  p.qts = st_.qts;
  p.kbs = st_.kbs;
  p.kts = st_.kts;
  p.mask = base_mask(a);
  p.drop = dropout_of(a);
  hipError_t e = hipSuccess;
  // the pre-pass computes the bounds; the other phases find them in the workspace
  e = prep_bounds(a, ws, p.mask, s, (phases & kPhasePre) != 0);
  if (e != hipSuccess) return hip_fail(e, "segment preparation launch");
  // with a broadcast bias the kernels write the full gradient to the workspace
  void* dbias_user = dbias;
  if (dbias && a->bias_bcast) {
    dbias = ws;
    p.dbias = ws;
  }
  ws += dbias_full_bytes(a);
  p.dbias_np = dbias ? dbias_partials(a) : 0;
  float* delta = reinterpret_cast<float*>(ws);
  ws += align_up((size_t)a->B * a->Hq * a->Sq * sizeof(float));
  float* part = nullptr;
  if (a->sink_mode == ATTN_SINK_LEARNABLE) {
    part = reinterpret_cast<float*>(ws);
    ws += align_up((size_t)a->Hq * a->B * pre_blocks(a) * sizeof(float));
  }
  p.du = nullptr;
  p.nkb32 = (a->Sk + 31) / 32;
  p.nqb32 = (a->Sq + 31) / 32;
  if (du_path(a)) {
    p.du = ws;
    ws += align_up(du_raw_bytes(a));
  }
  p.hsplit = head_split(a);
  p.dkv_part = p.hsplit > 1 ? reinterpret_cast<float*>(ws) : nullptr;
  p.delta = delta;
  p.Hq = a->Hq;
  p.Hkv = a->Hkv;
  p.G = a->Hq / a->Hkv;
  fill_consts(a, p.scale, p.sl2, p.xc, p.bc, p.cl2);
  p.reverse = a->causal ? 1 : 0;
  const Launch l{a->B, a->Sq, a->Sk, s, st_.qbs, st_.qts, st_.kbs, st_.kts};
  const TypeOps& o = ops(a);
  const bool cap = a->softcap > 0.0f, bias = a->bias != nullptr;
  if (phases & kPhasePre) {
    if (a->Sq > 0) {
      e = o.pre(a->D, out, out_lo, dout, lse, delta, part, a->sink, a->sink_mode, a->Hq, kPreRows, l);
      if (e != hipSuccess) return hip_fail(e, "backward pre-pass launch");
    }
    if (part) {
      dsink_final_kernel<<<a->Hq, 256, 0, s>>>(part, dsink, (int)(a->B * pre_blocks(a)));
      e = hipGetLastError();
      if (e != hipSuccess) return hip_fail(e, "sink gradient launch");
    }
    if (dbias && a->Sq > 0 && a->Sk > 0 && !dkdv_writes_dbias_zeros(a)) {
      e = o.dbias_fill(dbias, p.mask, a->Hq, kFillRows, l);
      if (e != hipSuccess) return hip_fail(e, "dbias fill launch");
    }
  }
  // dk/dv before dq: on the dU path the dq kernel reads what dk/dv wrote
  if ((phases & kPhaseDkdv) && a->Sk > 0) {
    e = o.dkdv(a->D, cap, bias, p, l);
    if (e != hipSuccess) return hip_fail(e, "dk/dv kernel launch");
    if (dbias_user && a->bias_bcast && a->Sq > 0) {
      e = p.dbias_np > 0 ? o.dbias_reduce(dbias, dbias_user, p.dbias_np, a->bias_bcast, &p.mask, a->D, l)
                         : o.dbias_reduce(dbias, dbias_user, a->Hq, a->bias_bcast, nullptr, a->D, l);
      if (e != hipSuccess) return hip_fail(e, "dbias reduction launch");
    }
  }
  if ((phases & kPhaseDq) && a->Sq > 0) {
    e = o.dq(a->D, cap, bias, p, l);
    if (e != hipSuccess) return hip_fail(e, "dq kernel launch");
  }
  return ATTN_OK;
}

attn_status attn_bwd(const attn_args* a, const void* out, const void* out_lo, const float* lse, const void* dout,
                     void* dq, void* dk, void* dv, void* dbias, float* dsink, void* workspace, size_t workspace_bytes,
                     void* stream) {
  return bwd_impl(a, out, out_lo, lse, dout, dq, dk, dv, dbias, dsink, workspace, workspace_bytes, stream,
                  kPhasePre | kPhaseDq | kPhaseDkdv);
}

attn_status attn_bwd_pre(const attn_args* a, const void* out, const void* out_lo, const float* lse,
                         const void* dout, void* dbias, float* dsink, void* workspace, size_t workspace_bytes,
                         void* stream) {
  return bwd_impl(a, out, out_lo, lse, dout, nullptr, nullptr, nullptr, dbias, dsink, workspace, workspace_bytes,
                  stream, kPhasePre);
}

attn_status attn_bwd_dq(const attn_args* a, const float* lse, const void* dout, void* dq, void* workspace,
                        size_t workspace_bytes, void* stream) {
  return bwd_impl(a, nullptr, nullptr, lse, dout, dq, nullptr, nullptr, nullptr, nullptr, workspace, workspace_bytes,
                  stream, kPhaseDq);
}

attn_status attn_bwd_dkdv(const attn_args* a, const float* lse, const void* dout, void* dk, void* dv, void* dbias,
                          void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_impl(a, nullptr, nullptr, lse, dout, nullptr, dk, dv, dbias, nullptr, workspace, workspace_bytes,
                  stream, kPhaseDkdv);
}

attn_status attn_bwd_noalloc(const attn_args* a, const void* out, const void* out_lo, const float* lse,
                             const void* dout, void* dq, void* dk, void* dv, void* dbias, float* dsink,
                             void* stream) {
  g_err.clear();
  attn_status st = validate(a);
  if (st != ATTN_OK) return st;
  attn_args r = *a;
  if (r.dq_mode == ATTN_DQ_AUTO) {
    // attn_bwd's choice, as long as the workspace then fits the scratch
    r.dq_mode = du_path(&r) ? ATTN_DQ_DU_BLOCKS : ATTN_DQ_RECOMPUTE;
    if (r.dq_mode == ATTN_DQ_DU_BLOCKS && bwd_ws(&r) > kScratchBytes) r.dq_mode = ATTN_DQ_RECOMPUTE;
  }
  const size_t need = bwd_ws(&r);
  if (need > kScratchBytes)
    return fail(ATTN_UNSUPPORTED, "attn_bwd_noalloc: this problem needs " + std::to_string(need) +
                                      " bytes of scratch, more than its " + std::to_string(kScratchBytes) +
                                      " (use attn_bwd with a workspace)");
  if ((size_t)r.B * (r.Sq + r.Sk) == 0) return bwd_impl(&r, out, out_lo, lse, dout, dq, dk, dv, dbias, dsink,
                                                         nullptr, 0, stream, kPhasePre | kPhaseDq | kPhaseDkdv);
  void* ws = nullptr;
  st = scratch_for(stream, &ws);
  if (st != ATTN_OK) return st;
  return bwd_impl(&r, out, out_lo, lse, dout, dq, dk, dv, dbias, dsink, ws, kScratchBytes, stream,
                  kPhasePre | kPhaseDq | kPhaseDkdv);
}

}  // extern "C"
