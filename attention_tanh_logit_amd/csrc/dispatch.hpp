// Tile shapes per (element type, head dim) and the launch wrappers.
//
// The shapes keep every workgroup's LDS tiles under the 160 KiB of a gfx950
// CU and every wave's fp32 accumulators at or under 128 registers:
//   DO  output columns owned by one wave (D/DO waves share a row group),
//   NQG query groups of 32 per workgroup (forward, dq),
//   NKG key groups of 32 per workgroup (dkdv),
//   BN  keys per forward / dq tile,
//   DC  head-dim columns staged in LDS at a time (DC == D: no chunking).
#pragma once

#include <type_traits>

#include "wide.hpp"

namespace ATL_NS {

template <typename T, int D> struct FwdCfg;
template <typename T, int D> struct DqCfg;
template <typename T, int D> struct DkdvCfg;

#define ATL_FWD(T, D_, DO_, NQG_, BN_, DC_) \
  template <> struct FwdCfg<T, D_> { static constexpr int DO = DO_, NQG = NQG_, BN = BN_, DC = DC_; };
#define ATL_DQ(T, D_, DO_, NQG_, BN_, DC_) \
  template <> struct DqCfg<T, D_> { static constexpr int DO = DO_, NQG = NQG_, BN = BN_, DC = DC_; };
#define ATL_DKDV(T, D_, DO_, NKG_, DC_) \
  template <> struct DkdvCfg<T, D_> { static constexpr int DO = DO_, NKG = NKG_, DC = DC_; };

//          T      D    DO  NQG  BN   DC
ATL_FWD(bf16, 64, 64, 4, 64, 64)
ATL_FWD(bf16, 128, 128, 4, 64, 128)
ATL_FWD(bf16, 256, 256, 2, 32, 256)
ATL_FWD(bf16, 512, 128, 2, 64, 128)
ATL_FWD(float, 64, 64, 4, 32, 64)
ATL_FWD(float, 128, 128, 2, 32, 128)
ATL_FWD(float, 256, 256, 4, 64, 64)
ATL_FWD(float, 512, 256, 4, 32, 64)

ATL_DQ(bf16, 64, 64, 4, 64, 64)
ATL_DQ(bf16, 128, 128, 4, 32, 128)
ATL_DQ(bf16, 256, 256, 2, 32, 256)
ATL_DQ(bf16, 512, 256, 2, 64, 128)
ATL_DQ(float, 64, 64, 4, 32, 64)
ATL_DQ(float, 128, 128, 2, 32, 128)
ATL_DQ(float, 256, 128, 4, 32, 64)
ATL_DQ(float, 512, 256, 2, 32, 128)

//           T      D   DO NKG  DC
ATL_DKDV(bf16, 64, 64, 4, 64)
ATL_DKDV(bf16, 128, 128, 4, 128)
ATL_DKDV(bf16, 256, 128, 2, 256)
ATL_DKDV(bf16, 512, 128, 1, 128)
ATL_DKDV(float, 64, 64, 4, 64)
ATL_DKDV(float, 128, 128, 2, 128)
ATL_DKDV(float, 256, 64, 1, 64)
ATL_DKDV(float, 512, 128, 1, 128)

// fp32 dq from the dU blocks: only K^T passes through LDS, so the rows per
// workgroup trade against K^T reuse differently than when recomputing
template <int D> struct DqDuCfg;
#define ATL_DQU(D_, DO_, NQG_, BN_, DC_) \
  template <> struct DqDuCfg<D_> { static constexpr int DO = DO_, NQG = NQG_, BN = BN_, DC = DC_; };
//      D    DO  NQG  BN   DC
ATL_DQU(64, 64, 4, 32, 64)
ATL_DQU(128, 128, 2, 32, 128)
ATL_DQU(256, 64, 2, 32, 64)
ATL_DQU(512, 64, 1, 32, 64)

#undef ATL_FWD
#undef ATL_DQ
#undef ATL_DKDV
#undef ATL_DQU

struct Launch {
  int B, Sq, Sk;
  hipStream_t stream;
  long qbs, qts, kbs, kts;   // element strides of batch rows and tokens, q side and k side
};

template <typename T, int D> constexpr int fwd_rows() { return 32 * FwdCfg<T, D>::NQG; }
template <typename T, int D> constexpr int dq_rows() { return 32 * DqCfg<T, D>::NQG; }
template <typename T, int D> constexpr int dkdv_keys() { return 32 * DkdvCfg<T, D>::NKG; }

// bf16 with D <= 256 takes the pipelined kernels of fast.hpp (with dropout
// too: dq then reads the dk/dv kernel's dU blocks, or runs the generic
// kernel when asked to recompute)
template <typename T, int D> constexpr bool use_fast() {
  return std::is_same<T, bf16>::value && (D == 64 || D == 128 || D == 256);
}

// The fast kernels address a streamed tile through a buffer resource with
// 32-bit byte offsets: 128 rows of the widest token stride (tstride,
// elements) must stay below 2^31 bytes.  The fast path reads bias rows 8
// keys at a time.
inline bool fast_ok(bool bf16_input, int D, long tstride, int Sk, bool bias) {
  return bf16_input && (D == 64 || D == 128 || D == 256) && 128L * tstride * 2 < (1L << 31) &&
         (!bias || (Sk % 8 == 0 && Sk >= 8));
}
// bf16 with D = 512 takes the kernels of wide.hpp (same 32-bit buffer
// offsets as the fast kernels; with a bias, Sk % 8 == 0 as on the fast path)
inline bool wide_ok(bool bf16_input, int D, long tstride, int Sk, bool bias) {
  return bf16_input && D == 512 && 128L * tstride * 2 < (1L << 31) && (!bias || (Sk % 8 == 0 && Sk >= 8));
}
template <typename T, int D, bool BIAS> constexpr bool use_wide() {
  return std::is_same<T, bf16>::value && D == 512;
}

template <int D, class Params>
bool fast_fits(const Params& p, const Launch& l, bool bias) {
  return fast_ok(true, D, p.qts > p.kts ? p.qts : p.kts, l.Sk, bias);
}


template <typename T, int D, bool CAP, bool BIAS>
hipError_t launch_fwd(const FwdParams& p, const Launch& l) {
  if constexpr (use_fast<T, D>()) {
    if (fast_fits<D>(p, l, BIAS)) {
      constexpr int NT = D > 128 ? 512 : 256;
      const dim3 grid((l.Sq + 127) / 128, p.Hq, l.B);
      // capped logits with 2 c log2(e) <= 120 keep a fixed reference maximum
      // (not with fp16 elements: probabilities relative to the cap would
      // leave fp16's exponent range)
      const bool fixm = CAP && p.cl2 <= 60.0f && !kNarrow16;
      if (p.drop.on) {
        if (fixm) fwd_fast_kernel<D, CAP, BIAS, CAP, true><<<grid, NT, 0, l.stream>>>(p);
        else fwd_fast_kernel<D, CAP, BIAS, false, true><<<grid, NT, 0, l.stream>>>(p);
      } else {
        if (fixm) fwd_fast_kernel<D, CAP, BIAS, CAP, false><<<grid, NT, 0, l.stream>>>(p);
        else fwd_fast_kernel<D, CAP, BIAS, false, false><<<grid, NT, 0, l.stream>>>(p);
      }
      return hipGetLastError();
    }
  }
  if constexpr (use_wide<T, D, BIAS>()) {
    if (wide_ok(true, D, p.qts > p.kts ? p.qts : p.kts, l.Sk, BIAS)) {
      const dim3 grid((l.Sq + 63) / 64, p.Hq, l.B);
      const bool fixm = CAP && p.cl2 <= 60.0f && !kNarrow16;
      if (p.drop.on) {
        if (fixm) fwd512_kernel<CAP, CAP, true, BIAS><<<grid, 512, 0, l.stream>>>(p);
        else fwd512_kernel<CAP, false, true, BIAS><<<grid, 512, 0, l.stream>>>(p);
      } else {
        if (fixm) fwd512_kernel<CAP, CAP, false, BIAS><<<grid, 512, 0, l.stream>>>(p);
        else fwd512_kernel<CAP, false, false, BIAS><<<grid, 512, 0, l.stream>>>(p);
      }
      return hipGetLastError();
    }
  }
  using C = FwdCfg<T, D>;
  constexpr int BM = 32 * C::NQG;
  const dim3 grid((l.Sq + BM - 1) / BM, p.Hq, l.B);
  const dim3 block(64 * C::NQG * (D / C::DO));
  fwd_kernel<T, D, C::DO, C::NQG, C::BN, C::DC, CAP, BIAS><<<grid, block, 0, l.stream>>>(p);
  return hipGetLastError();
}

template <typename T, int D, bool CAP, bool BIAS>
hipError_t launch_dq(const BwdParams& p, const Launch& l) {
  if constexpr (use_fast<T, D>()) {
    if (fast_fits<D>(p, l, BIAS)) {
      const dim3 grid((l.Sq + 127) / 128, p.Hq, l.B);
      // 32-key tiles, two stages, four workgroups per CU (measured against
      // 64-key tiles and against three stages); the dU blocks carry any
      // dropout already
      if (p.du) {
        dq_du_kernel<D, CAP, 32, 2><<<grid, 256, 0, l.stream>>>(p);
        return hipGetLastError();
      }
      // the recomputing dq kernel holds whole Q and dO rows: D <= 128 only
      if constexpr (D <= 128) {
        if (!p.drop.on) {
          dq_fast_kernel<D, CAP, BIAS><<<grid, 256, 0, l.stream>>>(p);
          return hipGetLastError();
        }
      }
    }
  }
  if constexpr (std::is_same<T, bf16>::value && D == 512) {
    // the dU blocks exist only where the wide dk/dv kernel wrote them
    if (p.du) {
      const dim3 grid((l.Sq + 127) / 128, p.Hq, l.B);
      dq_du_kernel<D, CAP, 32, 2, 2><<<grid, 512, 0, l.stream>>>(p);
      return hipGetLastError();
    }
  }
  if constexpr (std::is_same<T, float>::value) {
    // fp32 dU blocks from the generic dk/dv kernel (cap, bias and dropout are
    // in them already)
    if (p.du) {
      using U = DqDuCfg<D>;
      constexpr int BMU = 32 * U::NQG;
      const dim3 grid((l.Sq + BMU - 1) / BMU, p.Hq, l.B);
      dq_kernel<T, D, U::DO, U::NQG, U::BN, U::DC, false, false, true>
          <<<grid, dim3(64 * U::NQG * (D / U::DO)), 0, l.stream>>>(p);
      return hipGetLastError();
    }
  }
  using C = DqCfg<T, D>;
  constexpr int BM = 32 * C::NQG;
  const dim3 grid((l.Sq + BM - 1) / BM, p.Hq, l.B);
  const dim3 block(64 * C::NQG * (D / C::DO));
  dq_kernel<T, D, C::DO, C::NQG, C::BN, C::DC, CAP, BIAS><<<grid, block, 0, l.stream>>>(p);
  return hipGetLastError();
}

// dk/dv tiles of dkdv16_kernel (D = 128 / 256): keys per workgroup and queries
// per item (8 waves x 16 keys, 64-query items -- measured best of 4/8 waves x
// 32/64 queries; at D = 256 two waves per 16 keys and 32-query items; with a
// bias, 32-query items: the bias and dbias tiles take registers).  The
// reduction of head-summed dbias slabs recomputes the rows they wrote from
// the same two numbers.
template <int D> constexpr int dkdv16_keys() { return D > 128 ? 64 : 128; }
template <int D, bool BIAS> constexpr int dkdv16_queries() { return (D > 128 || BIAS) ? 32 : 64; }

template <typename T>
hipError_t launch_reduce_part(const void* slabs, void* out, int np, int bcast, const Mask& m, int D,
                              const Launch& l) {
  if constexpr (std::is_same<T, float>::value) {
    return hipErrorInvalidValue;   // head-summed slabs come from the 16-bit kernels only
  } else {
    if (l.Sk % 8 != 0 || (D != 128 && D != 256)) return hipErrorInvalidValue;
    const long n = (long)((bcast & 1) ? 1 : l.B) * l.Sq * (l.Sk / 8);
    const unsigned blocks = (unsigned)((n + 255) / 256);
    const bool vec = ((uintptr_t)out & 15) == 0;
    const T* s = static_cast<const T*>(slabs);
    T* o = static_cast<T*>(out);
    if (D == 128)
      dbias_reduce_part_kernel<T, dkdv16_keys<128>(), dkdv16_queries<128, true>()><<<blocks, 256, 0, l.stream>>>(
          s, o, l.B, np, bcast, m, vec);
    else
      dbias_reduce_part_kernel<T, dkdv16_keys<256>(), dkdv16_queries<256, true>()><<<blocks, 256, 0, l.stream>>>(
          s, o, l.B, np, bcast, m, vec);
    return hipGetLastError();
  }
}

template <typename T, int D, bool CAP, bool BIAS>
hipError_t launch_dkdv(const BwdParams& p, const Launch& l) {
  if constexpr (use_fast<T, D>()) {
    if (fast_fits<D>(p, l, BIAS)) {
      if constexpr (D >= 128) {
        constexpr int NW = 8, BMQ = dkdv16_queries<D, BIAS>(), BNK = dkdv16_keys<D>();
        const dim3 grid((l.Sk + BNK - 1) / BNK, p.Hkv * p.hsplit, l.B);
        const bool part = BIAS && p.dbias_np > 0;
        if (part) {
          if (p.drop.on) dkdv16_kernel<D, CAP, BIAS, NW, BMQ, true, BIAS><<<grid, 64 * NW, 0, l.stream>>>(p);
          else dkdv16_kernel<D, CAP, BIAS, NW, BMQ, false, BIAS><<<grid, 64 * NW, 0, l.stream>>>(p);
        } else {
          if (p.drop.on) dkdv16_kernel<D, CAP, BIAS, NW, BMQ, true, false><<<grid, 64 * NW, 0, l.stream>>>(p);
          else dkdv16_kernel<D, CAP, BIAS, NW, BMQ, false, false><<<grid, 64 * NW, 0, l.stream>>>(p);
        }
      } else {
        const dim3 grid((l.Sk + 127) / 128, p.Hkv * p.hsplit, l.B);
        if (p.drop.on) dkdv_fast_kernel<D, CAP, BIAS, true><<<grid, 256, 0, l.stream>>>(p);
        else dkdv_fast_kernel<D, CAP, BIAS, false><<<grid, 256, 0, l.stream>>>(p);
      }
      if (p.hsplit > 1) {
        const long nel = (long)l.B * l.Sk * p.Hkv * D;
        const float kscale = p.scale * (CAP ? 4.0f : 1.0f);
        dkv_reduce_kernel<bf16><<<(unsigned)((nel / 4 + 255) / 256), 256, 0, l.stream>>>(
            p.dkv_part, p.hsplit, nel, kscale, reinterpret_cast<bf16*>(p.dk), reinterpret_cast<bf16*>(p.dv), l.Sk,
            (long)p.Hkv * D, p.kbs, p.kts);
      }
      return hipGetLastError();
    }
  }
  if constexpr (use_wide<T, D, BIAS>()) {
    if (wide_ok(true, D, p.qts > p.kts ? p.qts : p.kts, l.Sk, BIAS)) {
      const dim3 grid((l.Sk + 31) / 32, p.Hkv * p.hsplit, l.B);
      if (p.drop.on) dkdv512_kernel<CAP, true, BIAS><<<grid, 512, 0, l.stream>>>(p);
      else dkdv512_kernel<CAP, false, BIAS><<<grid, 512, 0, l.stream>>>(p);
      if (p.hsplit > 1) {
        const long nel = (long)l.B * l.Sk * p.Hkv * D;
        const float kscale = p.scale * (CAP ? 4.0f : 1.0f);
        dkv_reduce_kernel<bf16><<<(unsigned)((nel / 4 + 255) / 256), 256, 0, l.stream>>>(
            p.dkv_part, p.hsplit, nel, kscale, reinterpret_cast<bf16*>(p.dk), reinterpret_cast<bf16*>(p.dv), l.Sk,
            (long)p.Hkv * D, p.kbs, p.kts);
      }
      return hipGetLastError();
    }
  }
  using C = DkdvCfg<T, D>;
  constexpr int BNK = 32 * C::NKG;
  const dim3 grid((l.Sk + BNK - 1) / BNK, p.Hkv, l.B);
  const dim3 block(64 * C::NKG * (D / C::DO));
  dkdv_kernel<T, D, C::DO, C::NKG, C::DC, CAP, BIAS><<<grid, block, 0, l.stream>>>(p);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_pre(const T* out, const T* out_lo, const T* dout, const float* lse, float* delta, float* dsink_part,
                      const float* sink, int sink_mode, int Hq, int rows_per_block, const Launch& l) {
  const dim3 grid((l.Sq + rows_per_block - 1) / rows_per_block, Hq, l.B);
  bwd_pre_kernel<T, D><<<grid, 256, 0, l.stream>>>(out, out_lo, dout, lse, delta, dsink_part, sink, sink_mode, l.Sq, Hq,
                                                   rows_per_block, l.qbs, l.qts);
  return hipGetLastError();
}

// Entry points of one element type (defined in attn_bf16.hip / attn_f32.hip).
struct TypeOps {
  hipError_t (*fwd)(int D, bool cap, bool bias, const FwdParams&, const Launch&);
  hipError_t (*dq)(int D, bool cap, bool bias, const BwdParams&, const Launch&);
  hipError_t (*dkdv)(int D, bool cap, bool bias, const BwdParams&, const Launch&);
  hipError_t (*pre)(int D, const void* out, const void* out_lo, const void* dout, const float* lse, float* delta,
                    float* dsink_part,
                    const float* sink, int sink_mode, int Hq, int rows_per_block, const Launch&);
  hipError_t (*dbias_fill)(void* dbias, const Mask&, int Hq, int rows_per_block, const Launch&);
  // part: the mask when `full` holds the head-summed slabs of the 16-bit dk/dv
  // kernel (Hq = their number per batch row), else nullptr
  hipError_t (*dbias_reduce)(const void* full, void* out, int Hq, int bcast, const Mask* part, int D,
                             const Launch&);
};

const TypeOps& ops_bf16();
const TypeOps& ops_f16();
const TypeOps& ops_f32();

}  // namespace ATL_NS

// Instantiates the TypeOps of one element type.
#define ATL_DEFINE_TYPE_OPS(T, NAME)                                                                        \
  namespace ATL_NS {                                                                                           \
  namespace {                                                                                               \
  template <int D>                                                                                          \
  hipError_t fwd_d(bool cap, bool bias, const FwdParams& p, const Launch& l) {                              \
    if (cap) return bias ? launch_fwd<T, D, true, true>(p, l) : launch_fwd<T, D, true, false>(p, l);         \
    return bias ? launch_fwd<T, D, false, true>(p, l) : launch_fwd<T, D, false, false>(p, l);                \
  }                                                                                                         \
  template <int D>                                                                                          \
  hipError_t dq_d(bool cap, bool bias, const BwdParams& p, const Launch& l) {                               \
    if (cap) return bias ? launch_dq<T, D, true, true>(p, l) : launch_dq<T, D, true, false>(p, l);           \
    return bias ? launch_dq<T, D, false, true>(p, l) : launch_dq<T, D, false, false>(p, l);                  \
  }                                                                                                         \
  template <int D>                                                                                          \
  hipError_t dkdv_d(bool cap, bool bias, const BwdParams& p, const Launch& l) {                             \
    if (cap) return bias ? launch_dkdv<T, D, true, true>(p, l) : launch_dkdv<T, D, true, false>(p, l);       \
    return bias ? launch_dkdv<T, D, false, true>(p, l) : launch_dkdv<T, D, false, false>(p, l);              \
  }                                                                                                         \
  hipError_t fwd_any(int D, bool cap, bool bias, const FwdParams& p, const Launch& l) {                     \
    switch (D) {                                                                                            \
      case 64: return fwd_d<64>(cap, bias, p, l);                                                           \
      case 128: return fwd_d<128>(cap, bias, p, l);                                                         \
      case 256: return fwd_d<256>(cap, bias, p, l);                                                         \
      case 512: return fwd_d<512>(cap, bias, p, l);                                                         \
    }                                                                                                       \
    return hipErrorInvalidValue;                                                                            \
  }                                                                                                         \
  hipError_t dq_any(int D, bool cap, bool bias, const BwdParams& p, const Launch& l) {                      \
    switch (D) {                                                                                            \
      case 64: return dq_d<64>(cap, bias, p, l);                                                            \
      case 128: return dq_d<128>(cap, bias, p, l);                                                          \
      case 256: return dq_d<256>(cap, bias, p, l);                                                          \
      case 512: return dq_d<512>(cap, bias, p, l);                                                          \
    }                                                                                                       \
    return hipErrorInvalidValue;                                                                            \
  }                                                                                                         \
  hipError_t dkdv_any(int D, bool cap, bool bias, const BwdParams& p, const Launch& l) {                    \
    switch (D) {                                                                                            \
      case 64: return dkdv_d<64>(cap, bias, p, l);                                                          \
      case 128: return dkdv_d<128>(cap, bias, p, l);                                                        \
      case 256: return dkdv_d<256>(cap, bias, p, l);                                                        \
      case 512: return dkdv_d<512>(cap, bias, p, l);                                                        \
    }                                                                                                       \
    return hipErrorInvalidValue;                                                                            \
  }                                                                                                         \
  hipError_t pre_any(int D, const void* out, const void* out_lo, const void* dout, const float* lse,        \
                     float* delta, float* part, const float* sink, int sink_mode, int Hq, int rpb,          \
                     const Launch& l) {                                                                     \
    const T* o = static_cast<const T*>(out);                                                                \
    const T* lo = static_cast<const T*>(out_lo);                                                            \
    const T* g = static_cast<const T*>(dout);                                                               \
    switch (D) {                                                                                            \
      case 64: return launch_pre<T, 64>(o, lo, g, lse, delta, part, sink, sink_mode, Hq, rpb, l);               \
      case 128: return launch_pre<T, 128>(o, lo, g, lse, delta, part, sink, sink_mode, Hq, rpb, l);             \
      case 256: return launch_pre<T, 256>(o, lo, g, lse, delta, part, sink, sink_mode, Hq, rpb, l);             \
      case 512: return launch_pre<T, 512>(o, lo, g, lse, delta, part, sink, sink_mode, Hq, rpb, l);             \
    }                                                                                                       \
    return hipErrorInvalidValue;                                                                            \
  }                                                                                                         \
  hipError_t fill_any(void* dbias, const Mask& m, int Hq, int rpb, const Launch& l) {                       \
    const dim3 grid((l.Sq + rpb - 1) / rpb, Hq, l.B);                                                       \
    dbias_fill_kernel<T><<<grid, 256, 0, l.stream>>>(static_cast<T*>(dbias), m, Hq, rpb);                    \
    return hipGetLastError();                                                                               \
  }                                                                                                         \
  hipError_t reduce_any(const void* full, void* out, int Hq, int bcast, const Mask* part, int D,            \
                        const Launch& l) {                                                                  \
    if (part) return launch_reduce_part<T>(full, out, Hq, bcast, *part, D, l);                              \
    const long SS = (long)l.Sq * l.Sk;                                                                      \
    const long n = (long)((bcast & 1) ? 1 : l.B) * ((bcast & 2) ? 1 : Hq) * SS;                             \
    if (SS % 8 == 0 && ((uintptr_t)full & 15) == 0 && ((uintptr_t)out & 15) == 0) {                         \
      dbias_reduce8_kernel<T><<<(unsigned)((n / 8 + 255) / 256), 256, 0, l.stream>>>(                       \
          static_cast<const T*>(full), static_cast<T*>(out), l.B, Hq, SS, bcast);                           \
      return hipGetLastError();                                                                             \
    }                                                                                                       \
    dbias_reduce_kernel<T><<<(unsigned)((n + 255) / 256), 256, 0, l.stream>>>(                              \
        static_cast<const T*>(full), static_cast<T*>(out), l.B, Hq, SS, bcast);                             \
    return hipGetLastError();                                                                               \
  }                                                                                                         \
  }                                                                                                         \
  const TypeOps& NAME() {                                                                                   \
    static const TypeOps o = {fwd_any, dq_any, dkdv_any, pre_any, fill_any, reduce_any};                   \
    return o;                                                                                               \
  }                                                                                                         \
  }
