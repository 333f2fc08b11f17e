// gfx950 kernels of the STEPQuant packed-state decode step.
//
// Method: summary pages of "STEPQuant: When and Where Errors Matter in
// Delta-Rule Recurrent State Quantization" -- ai.info AI summary ("Key
// Contributions" item 4, "Methodology in Plain English"), ai-papers.net
// ("STEPQuantの仕組み"), ai-trend.me ("방법", "핵심 용어: Gated Delta Rule").
//
// One workgroup per (request, head) tile M (D x D, row = key channel,
// column = value channel).  Lane l of row group g owns value columns 2l and
// 2l+1 for the RPL key rows of its group, so the five column reductions of the
// step (u = M~^T k, w = M~^T q, the clip-free maximum and the two sums of the
// least-squares column fit) run inside a lane and are combined across the NG
// groups through LDS; the single row reduction (row RMS, refit mode only) goes
// through a padded LDS transpose private to the group's wave.  Per-row
// coefficients are
// computed once per tile by the first D threads and read back as LDS
// broadcasts.  The path is rank-1 update plus matrix-vector work on a
// bit-packed stream, so it uses no MFMA.
//
// Scales follow the layout's mode (kMode template parameter): 1 calibrated
// row-scale constants r^_i from the layout table (ai-papers.net
// "STEPQuantの仕組み": the row scale comes from the row's average size and
// its impact; ai-feeds.com key modules 2-3: scale factors from calibration
// statistics), 0 row scales refitted from the updated row's RMS at every step,
// 2 the uniform INT-b baseline with one absmax scale per tile (ai.info "Main
// Findings").
//
// Two bodies:
//  * uniform heads (every row of the head has the same width -- always the
//    case for the per-head gate): codes stay in registers, field offsets are
//    compile-time constants (bfe / alignbit to unpack, an alignbit chain to
//    pack), one template instance per (D, width);
//  * mixed heads (per-key-row widths of the per-key-channel gate, pivot rows
//    among integer rows): the tile's words are staged in LDS, fields are read
//    at run-time bit offsets and written back with LDS atomic OR.
#include <type_traits>
#include <utility>

#include "stepq_internal.hpp"

namespace stepq {
namespace {

// Adding 1.5 * 2^23 to |x| < 2^22 leaves round-half-even(x) in the low
// mantissa bits: the float's value is magic + rne(x) and its low bits are the
// two's-complement code.
constexpr float kMagic = 12582912.0f;
constexpr float kScaleMin = 6.103515625e-05f;  // 2^-14
constexpr float kScaleMax = 65504.0f;
constexpr float kFactorMin = 5.421010862427522e-20f;   // 2^-64

template <int D, int kRPL = (D == 128) ? 32 : 16>
struct Geo {
  static constexpr int RPL = kRPL;                    // key rows per lane
  static constexpr int NG = D / RPL;                  // row groups
  static constexpr int LPG = D / 2;                   // lanes per group (2 columns each)
  static constexpr int NT = NG * LPG;                 // working threads
  static constexpr int BS = NT < 64 ? 64 : NT;        // block size, whole waves
  static constexpr int STR = LPG + 2;                 // row-partial stride (bank spread)
  // the lanes that finish the row reduction: LPR lanes per row, NR rows per lane
  static constexpr int LPR = LPG >= RPL ? LPG / RPL : 1;
  static constexpr int NR = LPG >= RPL ? 1 : RPL / LPG;
  static constexpr int CH = LPG / LPR;                // partials each finishing lane sums
};

// The mixed-width path runs 16 rows per lane at every D (twice the waves of
// the uniform path at D = 128), which halves its registers per lane.
template <int D>
using GeoM = Geo<D, 16>;

// A per-row value is uniform across a row group.  When a group fills a whole
// wave (D = 128) it is moved to a scalar register and branches on it are
// scalar; smaller D packs several groups into one wave, so the lane keeps its
// own copy.
template <int D>
__device__ __forceinline__ int group_uniform(int x) {
  if constexpr (Geo<D>::LPG >= 64) {
    return __builtin_amdgcn_readfirstlane(x);
  } else {
    return x;
  }
}

__device__ __forceinline__ float half_to_float(uint32_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h & 0xffffu)));
}
__device__ __forceinline__ uint32_t float_to_half(float x) {
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<_Float16>(x)));
}
__device__ __forceinline__ uint32_t fbits(float x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ float bitsf(uint32_t x) { return __builtin_bit_cast(float, x); }

// LDS ordering among the lanes of one wave (row partials, per-row scales).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

template <int CTRL, int ROW_MASK = 0xf, int BANK_MASK = 0xf>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROW_MASK,
                                                               BANK_MASK, false));
}

// Sum over the 64 lanes of a wave, returned in every lane: DPP within quads,
// half-rows and rows, then row broadcasts towards lane 63.
__device__ __forceinline__ float wave_sum(float x) {
  x += dpp<0xb1>(x);           // quad_perm [1,0,3,2]
  x += dpp<0x4e>(x);           // quad_perm [2,3,0,1]
  x += dpp<0x141>(x);          // row_half_mirror
  x += dpp<0x140>(x);          // row_mirror: every lane holds its row's sum
  x += dpp<0x142, 0xa>(x);     // row_bcast:15 into rows 1 and 3
  x += dpp<0x143, 0xc>(x);     // row_bcast:31 into rows 2 and 3
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

// Maximum over the 64 lanes of a wave, returned in every lane (same DPP
// pattern as wave_sum).
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp<0xb1>(x));
  x = fmaxf(x, dpp<0x4e>(x));
  x = fmaxf(x, dpp<0x141>(x));
  x = fmaxf(x, dpp<0x140>(x));
  x = fmaxf(x, dpp<0x142, 0xa>(x));
  x = fmaxf(x, dpp<0x143, 0xc>(x));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

// n / d for normal, finite operands of moderate range: reciprocal estimate
// and one residual correction (the quotient is the correctly rounded one
// except in rare near-halfway cases, where it is one ulp off).
__device__ __forceinline__ float quotient(float n, float d) {
  const float r = __builtin_amdgcn_rcpf(d);
  const float q = n * r;
  return fmaf(fmaf(-d, q, n), r, q);
}

// Row refit: r = RMS / sqrt(w), 1 for a zero row, clamped to the binary16
// normal range (ai.info "Methodology in Plain English": grows with the row's
// magnitude, shrinks with its impact weight).
__device__ __forceinline__ float row_scale(float ss, float inv_d_omega) {
  float r = ss > 0.f ? __builtin_amdgcn_sqrtf(ss * inv_d_omega) : 1.0f;
  return fminf(fmaxf(r, kScaleMin), kScaleMax);
}

// ------------------------------------------------------------ uniform fields
// Field r of a lane's word array: row r occupies bits [r*B, r*B + B).
template <int B, int R, int NW>
__device__ __forceinline__ int field_get(const uint32_t (&w)[NW]) {
  constexpr int p = R * B, k = p / 32, s = p % 32;
  if constexpr (s + B <= 32) {
    return __builtin_amdgcn_sbfe(static_cast<int>(w[k]), s, B);
  } else {
    return __builtin_amdgcn_sbfe(static_cast<int>(__builtin_amdgcn_alignbit(w[k + 1], w[k], s)), 0, B);
  }
}

// Appends field r (its low B bits) to the lane's output words.  alignbit
// shifts the word right and inserts the new bits at the top, so after the last
// field of a word every field sits at its own offset and older bits have left
// through the bottom.  A field crossing a word boundary is inserted in both
// words: its low part tops off the first, all of it seeds the second.
template <int B, int R, int NW>
__device__ __forceinline__ void field_put(uint32_t (&w)[NW], uint32_t f) {
  constexpr int p = R * B, k = p / 32, s = p % 32;
  if constexpr (s + B <= 32) {
    w[k] = __builtin_amdgcn_alignbit(f, w[k], B);
  } else {
    w[k] = __builtin_amdgcn_alignbit(f, w[k], 32 - s);
    w[k + 1] = __builtin_amdgcn_alignbit(f, w[k + 1], B);
  }
}

template <int N, typename F, int... I>
__device__ __forceinline__ void unroll_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void unroll(F&& f) {
  unroll_impl<N>(f, std::make_integer_sequence<int, N>{});
}

// ------------------------------------------------------------ shared memory
template <int D>
struct __align__(16) SmemU {
  using G = Geo<D>;
  float4 coefA[D];                          // per row {kappa, lambda, alpha, gamma};
                                            // a group's slice is reused for its column maxima
  float4 colA[G::NG][G::LPG];               // column partials: (u, w), later (N, Dn)
  float rowbuf[G::NG][G::RPL][G::STR];      // row partials; a group's head holds {1/r, U} per row
  float qk[4];
  float red[4];                             // per-wave tile maxima (uniform tile scale)
};

// Shared memory of the readout-only kernel: coefficients, column partials and
// q.k only (a quarter of SmemU), so more workgroups share a CU.
template <int D>
struct __align__(16) SmemR {
  using G = Geo<D>;
  float4 coefA[D];
  float4 colA[G::NG][G::LPG];
  float qk[4];
};

template <int D>
__device__ __forceinline__ float2* colB_of(SmemU<D>& sm, int g) {
  return reinterpret_cast<float2*>(&sm.coefA[g * Geo<D>::RPL]);
}
template <int D>
__device__ __forceinline__ float2* coefB_of(SmemU<D>& sm, int g) {
  return reinterpret_cast<float2*>(&sm.rowbuf[g][0][0]);
}

// Finishing the row reduction: returns the sum of row rr's partials; the
// calling lane is the row's owner when part == 0.
template <int D, class G = Geo<D>>
__device__ __forceinline__ float row_total(const float (*rb)[G::STR], int rr, int part) {
  const float* p = &rb[rr][part * G::CH];
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int m = 0; m < G::CH; m += 4) {
    const float2 x = *reinterpret_cast<const float2*>(p + m);
    const float2 y = *reinterpret_cast<const float2*>(p + m + 2);
    s0 += x.x + x.y;
    s1 += y.x + y.y;
  }
  float s = s0 + s1;
  if constexpr (G::LPR >= 2) s += __shfl_xor(s, 1, 64);
  if constexpr (G::LPR >= 4) s += __shfl_xor(s, 2, 64);
  return s;
}

// Common tail of decode and pack for an integer head of width B.
// Refit mode: P holds Y = M' / y_i for this lane's rows x 2 columns (y_i = r^_i,
// the row's stored scale, in decode -- coefA[i].w -- and 1 in pack) and rowbuf
// the row partials of Y^2; the row scales are refitted, rounded to binary16
// and stored first, and everything after uses the stored value.
// Calibrated mode: P holds z / f_j = M' / (r^_i f_j), with a positive factor
// f_j per column (fa, fb for the lane's two columns; 1 in pack), and coefB
// holds {1, w r^^2} per row (written before the caller's last block barrier).
// A positive per-column factor changes neither the clip-free codes (the
// column maximum carries it too) nor the least-squares denominator; the
// numerator is multiplied by it at the end.  Then clip-free
// column maxima, codes, least-squares column scales; packs and stores codes
// and column scales.  Rule (ai.info "Methodology in Plain English",
// ai-papers.net "STEPQuantの仕組み"): r^_i = binary16(RMS_i / sqrt(w_i))
// (refit) or the constant r^_i (calibrated); c0_j = max_i |M'_ij| / (r^_i qmax);
// q = rne(M' / (r^_i c0_j)) in binary32; c_j = sum_i w_i r^_i q M' /
// sum_i w_i r^_i^2 q^2 (c0_j = 1 when the column is zero, the only case with a
// zero denominator: the row attaining the maximum is coded at +-qmax).
template <int D, int B, bool kScaled, bool kCal>
__device__ __forceinline__ void requant_int(SmemU<D>& sm, float (&P)[Geo<D>::RPL][2],
                                            uint32_t* tw, uint16_t* sc, const RowInfo (&ri)[Geo<D>::NR],
                                            bool worker, int g, int l, float fa = 1.0f, float fb = 1.0f) {
  using G = Geo<D>;
  constexpr int RPL = G::RPL, NWL = RPL * B / 32;
  constexpr float QMAX = static_cast<float>((1 << (B - 1)) - 1);
  const int c0 = 2 * l;
  float2* coefB = coefB_of<D>(sm, g);

  if constexpr (!kCal) {
  wave_sync();
  // --- row reduction -> r, 1/r, U = w r^2, stored r^
  if constexpr (G::NR == 1) {
    const int rr = l / G::LPR, part = l % G::LPR;
    const float ss = row_total<D>(sm.rowbuf[g], rr, part);
    wave_sync();
    if (worker && part == 0) {
      const float y = kScaled ? sm.coefA[g * RPL + rr].w : 1.0f;
      const uint32_t rb = float_to_half(row_scale(ss * y * y, ri[0].inv_d_omega));
      const float rh = half_to_float(rb);
      sc[g * RPL + rr] = static_cast<uint16_t>(rb);
      coefB[rr] = make_float2(quotient(y, rh), ri[0].omega * rh * rh);
    }
  } else {
    float ss[G::NR];
#pragma unroll
    for (int m = 0; m < G::NR; ++m) ss[m] = row_total<D>(sm.rowbuf[g], l * G::NR + m, 0);
    wave_sync();
#pragma unroll
    for (int m = 0; m < G::NR; ++m) {
      if (worker) {
        const float y = kScaled ? sm.coefA[g * RPL + l * G::NR + m].w : 1.0f;
        const uint32_t rb = float_to_half(row_scale(ss[m] * y * y, ri[m].inv_d_omega));
        const float rh = half_to_float(rb);
        sc[g * RPL + l * G::NR + m] = static_cast<uint16_t>(rb);
        coefB[l * G::NR + m] = make_float2(quotient(y, rh), ri[m].omega * rh * rh);
      }
    }
  }
  wave_sync();
  }   // !kCal

  // --- z = M' / r^ (refit: Y (y / r^); calibrated: Y itself) and the clip-free column maxima
  float mxa = 0.f, mxb = 0.f;
#pragma unroll
  for (int r = 0; r < RPL; ++r) {
    float za = P[r][0], zb = P[r][1];
    if constexpr (!kCal) {
      const float ir = coefB[r].x;
      za *= ir;
      zb *= ir;
    }
    mxa = fmaxf(mxa, fabsf(za));
    mxb = fmaxf(mxb, fabsf(zb));
    P[r][0] = za;
    P[r][1] = zb;
  }
  if (worker) colB_of<D>(sm, g)[l] = make_float2(mxa, mxb);
  __syncthreads();
#pragma unroll
  for (int gg = 0; gg < G::NG; ++gg) {
    const float2 m = colB_of<D>(sm, gg)[l];
    mxa = fmaxf(mxa, m.x);
    mxb = fmaxf(mxb, m.y);
  }
  const float sa = mxa > 0.f ? quotient(QMAX, mxa) : 1.0f, sb = mxb > 0.f ? quotient(QMAX, mxb) : 1.0f;

  // --- codes, least-squares sums, packing
  uint32_t oa[NWL], ob[NWL];
#pragma unroll
  for (int w = 0; w < NWL; ++w) { oa[w] = 0u; ob[w] = 0u; }
  float Na = 0.f, Nb = 0.f, Da = 0.f, Db = 0.f;
  unroll<RPL>([&](auto RC) {
    constexpr int r = decltype(RC)::value;
    const float U = coefB[r].y;
    const float za = P[r][0], zb = P[r][1];
    const float ea = fmaf(za, sa, kMagic), eb = fmaf(zb, sb, kMagic);
    const float qa = ea - kMagic, qb = eb - kMagic;
    const float ta = U * qa, tb = U * qb;
    Na = fmaf(ta, za, Na);
    Nb = fmaf(tb, zb, Nb);
    Da = fmaf(ta, qa, Da);
    Db = fmaf(tb, qb, Db);
    field_put<B, r>(oa, fbits(ea));
    field_put<B, r>(ob, fbits(eb));
  });
  if (worker) {
#pragma unroll
    for (int w = 0; w < NWL; ++w)
      *reinterpret_cast<uint2*>((tw + g * NWL * D + w * D) + static_cast<uint32_t>(c0)) = make_uint2(oa[w], ob[w]);
    sm.colA[g][l] = make_float4(Na, Nb, Da, Db);
  }
  __syncthreads();
  if (worker && g == 0) {
    Na = Nb = Da = Db = 0.f;
#pragma unroll
    for (int gg = 0; gg < G::NG; ++gg) {
      const float4 x = sm.colA[gg][l];
      Na += x.x; Nb += x.y; Da += x.z; Db += x.w;
    }
    // the least-squares scale is only stored as binary16: a reciprocal estimate suffices
    Na *= fa;
    Nb *= fb;
    float ca = Da > 0.f ? Na * __builtin_amdgcn_rcpf(Da) : 1.0f, cb = Db > 0.f ? Nb * __builtin_amdgcn_rcpf(Db) : 1.0f;
    ca = fminf(fmaxf(ca, kScaleMin), kScaleMax);
    cb = fminf(fmaxf(cb, kScaleMin), kScaleMax);
    *reinterpret_cast<uint32_t*>(sc + D + c0) = float_to_half(ca) | (float_to_half(cb) << 16);
  }
}

// Uniform INT-b tail of decode and pack (one absmax scale per tile, the
// baseline of ai.info "Main Findings"): P holds M' / y (y = the tile's old
// scale times its decay a in decode, 1 in pack).  s' = binary32(max |M'| / qmax) (1 for a zero
// tile), codes q = rne(M' / s'); packs and stores the codes and s' (the first
// two binary16 entries of the head's scale table hold s' as binary32).
template <int D, int B>
__device__ __forceinline__ void requant_tile(SmemU<D>& sm, float (&P)[Geo<D>::RPL][2], uint32_t* tw, uint16_t* sc,
                                             float y, bool worker, int g, int l) {
  using G = Geo<D>;
  constexpr int RPL = G::RPL, NWL = RPL * B / 32, NW = G::BS / 64;
  constexpr float QMAX = static_cast<float>((1 << (B - 1)) - 1);
  float mx = 0.f;
#pragma unroll
  for (int r = 0; r < RPL; ++r) mx = fmaxf(mx, fmaxf(fabsf(P[r][0]), fabsf(P[r][1])));
  mx = wave_max(mx);
  if ((threadIdx.x & 63) == 0) sm.red[threadIdx.x >> 6] = mx;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < NW; ++w) mx = fmaxf(mx, sm.red[w]);
  const float mxm = mx * y;                              // max |M'|
  const float sn = mxm > 0.f ? mxm / QMAX : 1.0f;
  const float f = y / sn;                                // Y f = M' / s'
  uint32_t oa[NWL], ob[NWL];
#pragma unroll
  for (int w = 0; w < NWL; ++w) { oa[w] = 0u; ob[w] = 0u; }
  unroll<RPL>([&](auto RC) {
    constexpr int r = decltype(RC)::value;
    field_put<B, r>(oa, fbits(fmaf(P[r][0], f, kMagic)));
    field_put<B, r>(ob, fbits(fmaf(P[r][1], f, kMagic)));
  });
  if (worker) {
#pragma unroll
    for (int w = 0; w < NWL; ++w)
      *reinterpret_cast<uint2*>((tw + g * NWL * D + w * D) + static_cast<uint32_t>(2 * l)) = make_uint2(oa[w], ob[w]);
  }
  if (threadIdx.x == 0) *reinterpret_cast<uint32_t*>(sc) = fbits(sn);
}

// Stores M' of a pivot (B = 16: binary16, saturated) or zero-loss (B = 32:
// binary32) head.
template <int D, int B>
__device__ __forceinline__ void store_float_rows(const float (&P)[Geo<D>::RPL][2], uint32_t* tw,
                                                 bool worker, int g, int l) {
  constexpr int RPL = Geo<D>::RPL, NWL = RPL * B / 32;
  if constexpr (B == 32) {
    // binary32 rows: word r of the lane's columns is row r itself.  The base
    // pointer is passed through an empty asm so the store addresses are not
    // shared with the loads of the same rows (which would keep 32 64-bit
    // addresses live across the whole tile).
    uint32_t* tws = tw + g * NWL * D;
    if constexpr (Geo<D>::LPG >= 64) asm volatile("" : "+s"(tws));   // g is wave-uniform here
    if (worker) {
#pragma unroll
      for (int r = 0; r < RPL; ++r)
        *reinterpret_cast<float2*>((tws + r * D) + static_cast<uint32_t>(2 * l)) = make_float2(P[r][0], P[r][1]);
    }
  } else {
    uint32_t oa[NWL], ob[NWL];
#pragma unroll
    for (int w = 0; w < NWL; ++w) { oa[w] = 0u; ob[w] = 0u; }
    unroll<RPL>([&](auto RC) {
      constexpr int r = decltype(RC)::value;
      field_put<16, r>(oa, float_to_half(fminf(fmaxf(P[r][0], -kScaleMax), kScaleMax)));
      field_put<16, r>(ob, float_to_half(fminf(fmaxf(P[r][1], -kScaleMax), kScaleMax)));
    });
    if (worker) {
#pragma unroll
      for (int w = 0; w < NWL; ++w)
        *reinterpret_cast<uint2*>((tw + g * NWL * D + w * D) + static_cast<uint32_t>(2 * l)) = make_uint2(oa[w], ob[w]);
    }
  }
}

// Value of field r of a uniform head: the integer code (B <= 8), or the stored
// binary16 / binary32 value.
template <int B, int R, int NW>
__device__ __forceinline__ float field_value(const uint32_t (&w)[NW]) {
  if constexpr (B <= 8) {
    return static_cast<float>(field_get<B, R>(w));
  } else if constexpr (B == 16) {
    constexpr int p = R * 16;
    return half_to_float(w[p / 32] >> (p % 32));
  } else {
    return bitsf(w[R]);
  }
}

// ------------------------------------------------------------ decode, uniform head
// Gated Delta rule (ai-trend.me "핵심 용어: Gated Delta Rule"; ai.info
// "Methodology in Plain English"): M~ = a M, u = M~^T k,
// M' = M~ + beta k (v - u)^T, o = M'^T q = w + beta (q.k)(v - u) with
// w = M~^T q accumulated in the same sweep as u.  For integer rows
// M_ij = r^_i c^_j code_ij, so u_j = a c^_j sum_i (k_i r^_i) code_ij.  The
// calibrated and tile-scale modes carry the update as
// Y' = M' / (r^_i f_j) = code_ij + (beta k_i / r^_i)(d_j / f_j), f_j = a c^_j:
// one fma per element.  The refit mode carries
// Y = M' / r^_i = (a c^_j) code_ij + (beta k_i / r^_i) d_j (one product and one
// fma), which keeps the row scale factored out of the squares
// (sum_j M'^2 = r^_i^2 sum_j Y^2) and of z = M' / r_i = Y (r^_i / r_i).
// Binary16 / binary32 heads use the refit form with r^_i = c^_j = 1.
// kRowGate (D = 128 only): one retention a_i per key channel (KDA), folded
// into the per-row coefficients k_i a_i r^_i and q_i a_i r^_i of phase 1;
// phase 2 then carries Y' = a_i code + (beta k_i / r^_i)(d_j / f_j) with
// f_j = c^_j (refit: Y = (a_i code) c^_j + (beta k_i / r^_i) d_j).  a_i is
// kept in the padding column of the group's row-partial buffer.
// kReadout: stop after the readout (the split-phase first half: o without
// touching the pool).  A.o == nullptr: the update without the readout store.
template <int D, int B, int kMode, bool kReadout, bool kRowGate, typename SM>
__device__ __forceinline__ void decode_uniform(SM& sm, const Tables& T, const StepArgs& A, int tile,
                                               int h, uint32_t* tw, uint16_t* sc) {
  using G = Geo<D>;
  constexpr int RPL = G::RPL, LPG = G::LPG, NWL = RPL * B / 32;
  constexpr bool kInt = B <= 8;
  constexpr bool kCal = kMode == 1, kTileScale = kMode == 2;
  static_assert(!kRowGate || D == 128, "the per-row gate of the uniform body needs one row group per wave");
  const int tid = threadIdx.x;
  const bool worker = (G::NT == G::BS) || tid < G::NT;
  const int g = group_uniform<D>(worker ? tid / LPG : 0);
  const int l = worker ? tid % LPG : 0;
  const int c0 = 2 * l;

  uint32_t wa[B == 32 ? 1 : NWL], wb[B == 32 ? 1 : NWL];
  float P[RPL][2];
  if constexpr (B == 32) {   // binary32 rows: word r of the lane's columns is row r itself
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
      const float2 x = *reinterpret_cast<const float2*>((tw + g * NWL * D + r * D) + static_cast<uint32_t>(c0));
      P[r][0] = x.x;
      P[r][1] = x.y;
    }
  } else {
#pragma unroll
    for (int w = 0; w < NWL; ++w) {
      const uint2 x = *reinterpret_cast<const uint2*>((tw + g * NWL * D + w * D) + static_cast<uint32_t>(c0));
      wa[w] = x.x;
      wb[w] = x.y;
    }
  }
  float cha = 1.0f, chb = 1.0f, s_tile = 1.0f;
  if constexpr (kInt && kTileScale) {
    s_tile = bitsf(*reinterpret_cast<const uint32_t*>(sc));
  } else if constexpr (kInt) {
    const uint32_t chw = *reinterpret_cast<const uint32_t*>(sc + D + c0);
    cha = half_to_float(chw);
    chb = half_to_float(chw >> 16);
  }
  const float2 vv = *reinterpret_cast<const float2*>((A.v + static_cast<size_t>(tile) * D) + static_cast<uint32_t>(c0));
  const float beta = A.beta[tile];
  const float a = kRowGate ? 1.0f : A.gate[tile];     // per-row gates sit in the row coefficients
  const float acha = a * cha, achb = a * chb;
  RowInfo ri[G::NR];
  if constexpr (kInt && kMode == 0) {
#pragma unroll
    for (int m = 0; m < G::NR; ++m)
      ri[m] = T.rows[h * D + g * RPL + (G::NR == 1 ? l / G::LPR : l * G::NR + m)];
  }

  float pqk = 0.f;
  if (tid < D) {
    const float ki = (A.k + static_cast<size_t>(tile) * D)[static_cast<uint32_t>(tid)];
    const float qi = (A.q + static_cast<size_t>(tile) * D)[static_cast<uint32_t>(tid)];
    float rh = 1.0f;
    if constexpr (kInt && kTileScale) {
      rh = s_tile;
    } else if constexpr (kInt && kCal) {
      const RowInfo rw = T.rows[h * D + tid];
      rh = rw.rhat;
      if constexpr (!kReadout) coefB_of<D>(sm, tid / RPL)[tid % RPL] = make_float2(1.0f, rw.u_weight);
    } else if constexpr (kInt) {
      rh = half_to_float(sc[tid]);
    }
    const float eps = kInt ? beta * ki * __builtin_amdgcn_rcpf(rh) : beta * ki;
    if constexpr (kRowGate) {
      const float ai = (A.gate + static_cast<size_t>(tile) * D)[static_cast<uint32_t>(tid)];
      sm.coefA[tid] = make_float4(ki * rh * ai, qi * rh * ai, eps, rh);
      if constexpr (!kReadout) sm.rowbuf[tid / RPL][tid % RPL][LPG] = ai;
    } else {
      sm.coefA[tid] = make_float4(ki * rh, qi * rh, eps, rh);
    }
    pqk = qi * ki;
  }
  pqk = wave_sum(pqk);
  if ((tid & 63) == 0 && tid < D) sm.qk[tid >> 6] = pqk;
  __syncthreads();

  // --- phase 1: codes -> values, column sums of k and q weighted rows
  float Ua = 0.f, Ub = 0.f, Wa = 0.f, Wb = 0.f;
  unroll<RPL>([&](auto RC) {
    constexpr int r = decltype(RC)::value;
    const float4 c = sm.coefA[g * RPL + r];
    float pa, pb;
    if constexpr (B == 32) {
      pa = P[r][0];
      pb = P[r][1];
    } else {
      pa = field_value<B, r>(wa);
      pb = field_value<B, r>(wb);
    }
    Ua = fmaf(c.x, pa, Ua);
    Ub = fmaf(c.x, pb, Ub);
    Wa = fmaf(c.y, pa, Wa);
    Wb = fmaf(c.y, pb, Wb);
    P[r][0] = pa;
    P[r][1] = pb;
  });
  if (worker) sm.colA[g][l] = make_float4(Ua, Ub, Wa, Wb);
  __syncthreads();
  Ua = Ub = 0.f;
#pragma unroll
  for (int gg = 0; gg < G::NG; ++gg) {
    const float4 x = sm.colA[gg][l];
    Ua += x.x; Ub += x.y;
  }
  const float da = vv.x - acha * Ua, db = vv.y - achb * Ub;
  if (worker && g == 0 && A.o != nullptr) {
    float qk = 0.f;
#pragma unroll
    for (int w = 0; w < (D + 63) / 64; ++w) qk += sm.qk[w];
    Wa = Wb = 0.f;
#pragma unroll
    for (int gg = 0; gg < G::NG; ++gg) {
      const float4 x = sm.colA[gg][l];
      Wa += x.z; Wb += x.w;
    }
    const float bq = beta * qk;
    *reinterpret_cast<float2*>((A.o + static_cast<size_t>(tile) * D) + static_cast<uint32_t>(c0)) =
        make_float2(fmaf(bq, da, acha * Wa), fmaf(bq, db, achb * Wb));
  }
  if constexpr (!kReadout) {
  if constexpr (kInt && kMode != 0) {
    // --- phase 2, calibrated and tile-scale modes: Y' = M' / (r^_i f_j) with
    // f_j = a c^_j, i.e. Y' = code + eps_i (d_j / f_j), one fma per element.
    // A decayed scale below 2^-64 (a vanishing gate) is raised to 2^-64 and
    // the codes are scaled by a c^_j / f_j first, so d_j / f_j stays finite.
    const float fa = fmaxf(acha, kFactorMin), fb = fmaxf(achb, kFactorMin);
    if (acha < kFactorMin || achb < kFactorMin) {
      const float ga = acha / fa, gb = achb / fb;
#pragma unroll
      for (int r = 0; r < RPL; ++r) {
        P[r][0] *= ga;
        P[r][1] *= gb;
      }
    }
    const float dpa = quotient(da, fa), dpb = quotient(db, fb);
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
      const float eps = sm.coefA[g * RPL + r].z;
      if constexpr (kRowGate) {
        const float ai = sm.rowbuf[g][r][LPG];
        P[r][0] = fmaf(eps, dpa, ai * P[r][0]);
        P[r][1] = fmaf(eps, dpb, ai * P[r][1]);
      } else {
        P[r][0] = fmaf(eps, dpa, P[r][0]);
        P[r][1] = fmaf(eps, dpb, P[r][1]);
      }
    }
    if constexpr (kTileScale) {
      requant_tile<D, B>(sm, P, tw, sc, s_tile * fa, worker, g, l);   // c^ = 1: f is the tile's a
    } else {
      requant_int<D, B, true, true>(sm, P, tw, sc, ri, worker, g, l, fa, fb);
    }
  } else {
  // --- phase 2: Y = M' / r^ = (a c^) code + eps d, squared row partials (refit mode)
#pragma unroll
  for (int r = 0; r < RPL; ++r) {
    const float eps = sm.coefA[g * RPL + r].z;
    float pa = P[r][0], pb = P[r][1];
    if constexpr (kRowGate) {
      const float ai = sm.rowbuf[g][r][LPG];
      pa *= ai;
      pb *= ai;
    }
    const float ya = fmaf(pa, acha, eps * da);
    const float yb = fmaf(pb, achb, eps * db);
    if constexpr (kInt && kMode == 0) {
      if (worker) sm.rowbuf[g][r][l] = fmaf(yb, yb, ya * ya);
    }
    P[r][0] = ya;
    P[r][1] = yb;
  }
  if constexpr (kInt) {
    requant_int<D, B, true, false>(sm, P, tw, sc, ri, worker, g, l);
  } else {
    store_float_rows<D, B>(P, tw, worker, g, l);
  }
  }
  }   // !kReadout
}

template <int D, int kMode, bool kReadout, bool kRowGate>
__device__ __forceinline__ void decode_uniform_tile(const Tables& T, const StepArgs& A);

template <int D, int kMode, bool kRowGate = false>
__global__ __launch_bounds__(Geo<D>::BS) __attribute__((amdgpu_waves_per_eu(4)))
void k_decode_uniform(const Tables T, const StepArgs A) {
  decode_uniform_tile<D, kMode, false, kRowGate>(T, A);
}

// The readout-only half of the split-phase schedule: phase 1 and o (6 waves
// per SIMD; 5 with per-row gates, which need a few more registers).
template <int D, int kMode, bool kRowGate = false>
__global__ __launch_bounds__(Geo<D>::BS) __attribute__((amdgpu_waves_per_eu(kRowGate ? 5 : 6)))
void k_readout_uniform(const Tables T, const StepArgs A) {
  decode_uniform_tile<D, kMode, true, kRowGate>(T, A);
}

template <int D, int kMode, bool kReadout, bool kRowGate>
__device__ __forceinline__ void decode_uniform_tile(const Tables& T, const StepArgs& A) {
  using SM = typename std::conditional<kReadout, SmemR<D>, SmemU<D>>::type;
  __shared__ SM sm;
  const int tile = blockIdx.x;
  const int b = tile / T.H, h = tile - b * T.H;
  const int slot = A.slot_ids[b];
  if (slot < 0 || slot >= A.num_slots) {
    if (A.o != nullptr)
      for (int j = threadIdx.x; j < D; j += blockDim.x) A.o[static_cast<size_t>(tile) * D + j] = __builtin_nanf("");
    return;
  }
  uint32_t* tw = reinterpret_cast<uint32_t*>(A.pool + static_cast<size_t>(slot) * T.slot_bytes) + T.head_woff[h];
  uint16_t* sc = A.scales + (static_cast<size_t>(slot) * T.H + h) * 2 * D;
  switch (T.head_bits[h]) {
    case 2: decode_uniform<D, 2, kMode, kReadout, kRowGate, SM>(sm, T, A, tile, h, tw, sc); break;
    case 4: decode_uniform<D, 4, kMode, kReadout, kRowGate, SM>(sm, T, A, tile, h, tw, sc); break;
    case 6: decode_uniform<D, 6, kMode, kReadout, kRowGate, SM>(sm, T, A, tile, h, tw, sc); break;
    case 8: decode_uniform<D, 8, kMode, kReadout, kRowGate, SM>(sm, T, A, tile, h, tw, sc); break;
    case 16: decode_uniform<D, 16, kMode, kReadout, kRowGate, SM>(sm, T, A, tile, h, tw, sc); break;
    case 32: decode_uniform<D, 32, kMode, kReadout, kRowGate, SM>(sm, T, A, tile, h, tw, sc); break;
    default: break;
  }
}

// ------------------------------------------------------------ pack / unpack, uniform head
template <int D, int B, int kMode>
__device__ __forceinline__ void pack_uniform(SmemU<D>& sm, const Tables& T, const PackArgs& A, int tile, int h,
                                             uint32_t* tw, uint16_t* sc) {
  using G = Geo<D>;
  constexpr int RPL = G::RPL, LPG = G::LPG;
  const int tid = threadIdx.x;
  const bool worker = (G::NT == G::BS) || tid < G::NT;
  const int g = group_uniform<D>(worker ? tid / LPG : 0);
  const int l = worker ? tid % LPG : 0;
  const int c0 = 2 * l;
  const float* st = A.state + static_cast<size_t>(tile) * D * D;
  float P[RPL][2];
#pragma unroll
  for (int r = 0; r < RPL; ++r) {
    const float2 x = *reinterpret_cast<const float2*>((st + (g * RPL + r) * D) + static_cast<uint32_t>(c0));
    P[r][0] = x.x;
    P[r][1] = x.y;
  }
  if constexpr (B <= 8 && kMode == 2) {
    for (int j = 2 + tid; j < 2 * D; j += blockDim.x) sc[j] = 0;   // only the tile scale is live
    requant_tile<D, B>(sm, P, tw, sc, 1.0f, worker, g, l);
  } else if constexpr (B <= 8 && kMode == 1) {
    // calibrated row scales: z = M' / r^ with a correctly rounded reciprocal;
    // the constant r^ goes into the scale table for unpack
    if (tid < D) {
      const RowInfo rw = T.rows[h * D + tid];
      sm.coefA[tid] = make_float4(quotient(1.0f, rw.rhat), 0.f, 0.f, 0.f);
      coefB_of<D>(sm, tid / RPL)[tid % RPL] = make_float2(1.0f, rw.u_weight);
      sc[tid] = static_cast<uint16_t>(float_to_half(rw.rhat));
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
      const float ir = sm.coefA[g * RPL + r].x;
      P[r][0] *= ir;
      P[r][1] *= ir;
    }
    RowInfo ri[G::NR];
    requant_int<D, B, false, true>(sm, P, tw, sc, ri, worker, g, l);
  } else if constexpr (B <= 8) {
    RowInfo ri[G::NR];
#pragma unroll
    for (int m = 0; m < G::NR; ++m)
      ri[m] = T.rows[h * D + g * RPL + (G::NR == 1 ? l / G::LPR : l * G::NR + m)];
#pragma unroll
    for (int r = 0; r < RPL; ++r)
      if (worker) sm.rowbuf[g][r][l] = fmaf(P[r][1], P[r][1], P[r][0] * P[r][0]);
    requant_int<D, B, false, false>(sm, P, tw, sc, ri, worker, g, l);
  } else {
    store_float_rows<D, B>(P, tw, worker, g, l);
    // scale entries no integer row uses are written as 0
    for (int j = tid; j < 2 * D; j += blockDim.x) sc[j] = 0;
  }
}

template <int D, int kMode>
__global__ __launch_bounds__(Geo<D>::BS) void k_pack_uniform(const Tables T, const PackArgs A) {
  __shared__ SmemU<D> sm;
  const int tile = blockIdx.x;
  const int b = tile / T.H, h = tile - b * T.H;
  const int slot = A.slot_ids[b];
  if (slot < 0 || slot >= A.num_slots) return;
  uint32_t* tw = reinterpret_cast<uint32_t*>(A.pool + static_cast<size_t>(slot) * T.slot_bytes) + T.head_woff[h];
  uint16_t* sc = A.scales + (static_cast<size_t>(slot) * T.H + h) * 2 * D;
  switch (T.head_bits[h]) {
    case 2: pack_uniform<D, 2, kMode>(sm, T, A, tile, h, tw, sc); break;
    case 4: pack_uniform<D, 4, kMode>(sm, T, A, tile, h, tw, sc); break;
    case 6: pack_uniform<D, 6, kMode>(sm, T, A, tile, h, tw, sc); break;
    case 8: pack_uniform<D, 8, kMode>(sm, T, A, tile, h, tw, sc); break;
    case 16: pack_uniform<D, 16, kMode>(sm, T, A, tile, h, tw, sc); break;
    case 32: pack_uniform<D, 32, kMode>(sm, T, A, tile, h, tw, sc); break;
    default: break;
  }
}

// Reconstruction: binary32((r^_i * c^_j) * code_ij); the scale product of two
// binary16 values is exact in binary32.
template <int D, int B, bool kTileScale>
__device__ __forceinline__ void unpack_uniform(const PackArgs& A, int tile, const uint32_t* tw, const uint16_t* sc) {
  using G = Geo<D>;
  constexpr int RPL = G::RPL, LPG = G::LPG, NWL = RPL * B / 32;
  const int tid = threadIdx.x;
  const bool worker = (G::NT == G::BS) || tid < G::NT;
  if (!worker) return;
  const int g = group_uniform<D>(tid / LPG), l = tid % LPG, c0 = 2 * l;
  uint32_t wa[NWL], wb[NWL];
#pragma unroll
  for (int w = 0; w < NWL; ++w) {
    const uint2 x = *reinterpret_cast<const uint2*>((tw + g * NWL * D + w * D) + static_cast<uint32_t>(c0));
    wa[w] = x.x;
    wb[w] = x.y;
  }
  float cha = 1.f, chb = 1.f, s_tile = 1.f;
  if constexpr (B <= 8 && kTileScale) {
    s_tile = bitsf(*reinterpret_cast<const uint32_t*>(sc));
  } else if constexpr (B <= 8) {
    const uint32_t chw = *reinterpret_cast<const uint32_t*>(sc + D + c0);
    cha = half_to_float(chw);
    chb = half_to_float(chw >> 16);
  }
  float* st = A.state_out + static_cast<size_t>(tile) * D * D;
  unroll<RPL>([&](auto RC) {
    constexpr int r = decltype(RC)::value;
    float xa = field_value<B, r>(wa), xb = field_value<B, r>(wb);
    if constexpr (B <= 8) {
      const float rh = kTileScale ? s_tile : half_to_float(sc[g * RPL + r]);
      xa = (rh * cha) * xa;
      xb = (rh * chb) * xb;
    }
    *reinterpret_cast<float2*>((st + (g * RPL + r) * D) + static_cast<uint32_t>(c0)) = make_float2(xa, xb);
  });
}

template <int D, bool kTileScale>
__global__ __launch_bounds__(Geo<D>::BS) void k_unpack_uniform(const Tables T, const PackArgs A) {
  const int tile = blockIdx.x;
  const int b = tile / T.H, h = tile - b * T.H;
  const int slot = A.slot_ids[b];
  if (slot < 0 || slot >= A.num_slots) {
    for (int e = threadIdx.x; e < D * D; e += blockDim.x)
      A.state_out[static_cast<size_t>(tile) * D * D + e] = __builtin_nanf("");
    return;
  }
  const uint32_t* tw =
      reinterpret_cast<const uint32_t*>(A.pool + static_cast<size_t>(slot) * T.slot_bytes) + T.head_woff[h];
  const uint16_t* sc = A.scales + (static_cast<size_t>(slot) * T.H + h) * 2 * D;
  switch (T.head_bits[h]) {
    case 2: unpack_uniform<D, 2, kTileScale>(A, tile, tw, sc); break;
    case 4: unpack_uniform<D, 4, kTileScale>(A, tile, tw, sc); break;
    case 6: unpack_uniform<D, 6, kTileScale>(A, tile, tw, sc); break;
    case 8: unpack_uniform<D, 8, kTileScale>(A, tile, tw, sc); break;
    case 16: unpack_uniform<D, 16, kTileScale>(A, tile, tw, sc); break;
    case 32: unpack_uniform<D, 32, kTileScale>(A, tile, tw, sc); break;
    default: break;
  }
}

// ------------------------------------------------------------ mixed heads
// Per-key-row widths (the KDA unit is the key row: ai.info "Future
// Directions", ai-papers.net "STEPQuantの仕組み") and pivot rows among integer
// rows.  The tile is staged in LDS; a field of row i in column j is read at
// bit bitoff_i of the column string and written back with atomic OR.
// kRows: the refit mode's row-partial buffer (absent in the other modes,
// which leaves room for more workgroups per CU).
template <int D, bool kRows = true>
struct __align__(16) SmemG {
  using G = GeoM<D>;
  float4 coefA[D];                          // {k_i, q_i, a_i * (r^_i or 1), beta k_i}
  float4 coefB[D];                          // {1 / (r^_i qmax_i), w_i r^_i^2, qmax_i, 1 / r^_i}; 0 for non-integer rows
  int2 rinfo[D];                            // {bitoff_i, bits_i}
  float4 colA[G::NG][G::LPG];
  float2 colB[G::NG][G::LPG];
  float rowbuf[kRows ? G::NG : 1][kRows ? G::RPL : 1][kRows ? G::STR : 1];
  float qk[4];
  float red[G::BS / 64];                    // per-wave tile maxima (uniform tile scale)
};

// The fields of one row in the lane's two adjacent columns c0, c0+1: one
// 64-bit LDS read per word row (conflict-free across the wave).
__device__ __forceinline__ uint2 staged_pair(const uint32_t* stage, int D, int bitoff, int bits, int c0) {
  const int k = bitoff >> 5, s = bitoff & 31;
  const uint2 lo = *reinterpret_cast<const uint2*>(stage + k * D + c0);
  const uint2 hi = *reinterpret_cast<const uint2*>(stage + (k + 1) * D + c0);
  const uint32_t m = bits == 32 ? 0xffffffffu : ((1u << bits) - 1u);
  return make_uint2(__builtin_amdgcn_alignbit(hi.x, lo.x, s) & m, __builtin_amdgcn_alignbit(hi.y, lo.y, s) & m);
}

// OR-in the fields fa, fb (already masked to bits) of one row in columns c0,
// c0+1: one 64-bit LDS atomic OR per word row touched (OR is bitwise, so the
// pair of 32-bit words takes it as one 64-bit value).
__device__ __forceinline__ void staged_put_pair(uint32_t* stage, int D, int bitoff, int bits, int c0, uint32_t fa,
                                                uint32_t fb) {
  const int k = bitoff >> 5, s = bitoff & 31;
  const unsigned long long lo = static_cast<unsigned long long>(fa << s) |
                                (static_cast<unsigned long long>(fb << s) << 32);
  atomicOr(reinterpret_cast<unsigned long long*>(stage + k * D + c0), lo);
  if (s + bits > 32) {
    const unsigned long long hi = static_cast<unsigned long long>(fa >> (32 - s)) |
                                  (static_cast<unsigned long long>(fb >> (32 - s)) << 32);
    atomicOr(reinterpret_cast<unsigned long long*>(stage + (k + 1) * D + c0), hi);
  }
}

// Value of a staged field: integer code (sign-extended, still to be scaled),
// binary16 or binary32.  The sign extension of a run-time-width field is
// written as (f ^ h) - h, h = 2^(bits-1): clang 22 for gfx950 follows a
// run-time-width signed bitfield extract with an unsigned int-to-float
// conversion, which turns negative codes into values near 2^32.
__device__ __forceinline__ float staged_value(uint32_t f, int bits) {
  if (bits <= 8) {
    const uint32_t h = 1u << (bits - 1);
    return static_cast<float>(static_cast<int>(f ^ h) - static_cast<int>(h));
  }
  if (bits == 16) return half_to_float(f);
  return bitsf(f);
}

__device__ __forceinline__ int tile_words_of(const Tables& T, int h) { return T.head_words[h]; }

// Per-row coefficients of the calibrated mode: {1 / (r^ qmax), w r^^2, qmax,
// 1 / r^} for integer rows, zeros otherwise.
__device__ __forceinline__ float4 calibrated_coef(const RowInfo& ri) {
  if (ri.bits > 8) return make_float4(0.f, 0.f, 0.f, 0.f);
  const float qm = static_cast<float>((1 << (ri.bits - 1)) - 1);
  return make_float4(1.0f / (ri.rhat * qm), ri.u_weight, qm, 1.0f / ri.rhat);
}

// Value of a staged field of width bits without branching on the width (the
// width is wave-uniform at D = 128 and per lane below): the integer code
// (sign-extended, still to be scaled), the binary16 or the binary32 value.
__device__ __forceinline__ float staged_value_sel(uint32_t f, int bits) {
  const uint32_t h = bits <= 8 ? (1u << (bits - 1)) : 0u;
  const float vi = static_cast<float>(static_cast<int>(f ^ h) - static_cast<int>(h));
  const float vh = half_to_float(f);
  const float vf = bitsf(f);
  return bits <= 8 ? vi : (bits == 16 ? vh : vf);
}

// Common tail of decode and pack for a mixed head: M' in P, stage zeroed
// (ordered by a barrier before this call's first block barrier).  Refit mode:
// squared row partials of integer rows in rowbuf; the row scales are refitted,
// rounded to binary16 and stored here, and the codes and the fit use the
// stored value.  Calibrated mode: coefB already holds calibrated_coef of
// every row.
template <int D, bool kCal, typename SM>
__device__ __forceinline__ void requant_mixed(SM& sm, uint32_t* stage, const Tables& T, int h,
                                              float (&P)[GeoM<D>::RPL][2], uint32_t* tw, uint16_t* sc, int TW,
                                              bool has_int, bool worker, int g, int l) {
  using G = GeoM<D>;
  constexpr int RPL = G::RPL;
  const int tid = threadIdx.x;
  const int c0 = 2 * l;
  if constexpr (!kCal) {
  wave_sync();
  float ss[G::NR];
#pragma unroll
  for (int m = 0; m < G::NR; ++m)
    ss[m] = row_total<D, GeoM<D>>(sm.rowbuf[g], G::NR == 1 ? l / G::LPR : l * G::NR + m, G::NR == 1 ? l % G::LPR : 0);
  if (worker && (G::NR > 1 || l % G::LPR == 0)) {
#pragma unroll
    for (int m = 0; m < G::NR; ++m) {
      const int i = g * RPL + (G::NR == 1 ? l / G::LPR : l * G::NR + m);
      const RowInfo ri = T.rows[h * D + i];
      if (ri.bits <= 8) {
        const float qm = static_cast<float>((1 << (ri.bits - 1)) - 1);
        const uint32_t rb = float_to_half(row_scale(ss[m], ri.inv_d_omega));
        const float rh = half_to_float(rb);
        sc[i] = static_cast<uint16_t>(rb);
        sm.coefB[i] = make_float4(1.0f / (rh * qm), ri.omega * rh * rh, qm, 1.0f / rh);
      } else {
        sm.coefB[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
  }
  wave_sync();
  }   // !kCal
  // column maxima of |M'| / (r qmax) over integer rows = c0 (the coefficient is
  // 0 on other rows, which therefore add nothing)
  float mxa = 0.f, mxb = 0.f;
#pragma unroll
  for (int r = 0; r < RPL; ++r) {
    const float ir = sm.coefB[g * RPL + r].x;
    mxa = fmaxf(mxa, fabsf(P[r][0] * ir));
    mxb = fmaxf(mxb, fabsf(P[r][1] * ir));
  }
  if (worker) sm.colB[g][l] = make_float2(mxa, mxb);
  __syncthreads();
#pragma unroll
  for (int gg = 0; gg < G::NG; ++gg) {
    const float2 m = sm.colB[gg][l];
    mxa = fmaxf(mxa, m.x);
    mxb = fmaxf(mxb, m.y);
  }
  const float c0a = mxa > 0.f ? mxa : 1.0f, c0b = mxb > 0.f ? mxb : 1.0f;
  const float sa = 1.0f / c0a, sb = 1.0f / c0b;
  // codes and least-squares sums without branching on the row width: the
  // coefficients of non-integer rows are 0, so their z, t and sums vanish
  float Na = 0.f, Nb = 0.f, Da = 0.f, Db = 0.f;
  const RowInfo* rrow = T.rows + h * D + g * RPL;
#pragma unroll
  for (int r = 0; r < RPL; ++r) {
    const int i = g * RPL + r;
    const int bitoff = group_uniform<D>(rrow[r].bitoff);
    const int bits = group_uniform<D>(rrow[r].bits);
    const float4 cb = sm.coefB[i];
    const float za = P[r][0] * cb.w, zb = P[r][1] * cb.w;     // M' / r
    const float ya = fmaf(za, sa, kMagic), yb = fmaf(zb, sb, kMagic);
    const float qa = ya - kMagic, qb = yb - kMagic;
    const float ta = cb.y * qa, tb = cb.y * qb;
    Na = fmaf(ta, za, Na);
    Nb = fmaf(tb, zb, Nb);
    Da = fmaf(ta, qa, Da);
    Db = fmaf(tb, qb, Db);
    const uint32_t mask = bits >= 32 ? 0xffffffffu : ((1u << bits) - 1u);
    const uint32_t fa = bits <= 8 ? (fbits(ya) & mask)
                      : (bits == 16 ? float_to_half(fminf(fmaxf(P[r][0], -kScaleMax), kScaleMax)) : fbits(P[r][0]));
    const uint32_t fb = bits <= 8 ? (fbits(yb) & mask)
                      : (bits == 16 ? float_to_half(fminf(fmaxf(P[r][1], -kScaleMax), kScaleMax)) : fbits(P[r][1]));
    if (worker) staged_put_pair(stage, D, bitoff, bits, c0, fa, fb);
  }
  if (worker) sm.colA[g][l] = make_float4(Na, Nb, Da, Db);
  __syncthreads();
  for (int e = tid * 4; e < TW; e += G::BS * 4)
    *reinterpret_cast<uint4*>(tw + e) = *reinterpret_cast<const uint4*>(stage + e);
  if (has_int && worker && g == 0) {
    Na = Nb = Da = Db = 0.f;
#pragma unroll
    for (int gg = 0; gg < G::NG; ++gg) {
      const float4 x = sm.colA[gg][l];
      Na += x.x; Nb += x.y; Da += x.z; Db += x.w;
    }
    float ca = Da > 0.f ? Na / Da : c0a, cb = Db > 0.f ? Nb / Db : c0b;
    ca = fminf(fmaxf(ca, kScaleMin), kScaleMax);
    cb = fminf(fmaxf(cb, kScaleMin), kScaleMax);
    *reinterpret_cast<uint32_t*>(sc + D + c0) = float_to_half(ca) | (float_to_half(cb) << 16);
  }
}

// Uniform INT-b tail of a mixed-path head (every row the same integer width):
// M' in P, stage zeroed.  s' = binary32(max |M'| / qmax) (1 for a zero tile),
// codes q = rne(M' / s'), staged, copied out, s' stored.
template <int D, typename SM>
__device__ __forceinline__ void requant_tile_mixed(SM& sm, uint32_t* stage, float (&P)[GeoM<D>::RPL][2],
                                                   uint32_t* tw, uint16_t* sc, int TW, bool worker, int g, int l) {
  using G = GeoM<D>;
  constexpr int RPL = G::RPL, NW = G::BS / 64;
  const int tid = threadIdx.x;
  const int c0 = 2 * l;
  const int bits = group_uniform<D>(sm.rinfo[0].y);
  const float qm = static_cast<float>((1 << (bits - 1)) - 1);
  float mx = 0.f;
#pragma unroll
  for (int r = 0; r < RPL; ++r) mx = fmaxf(mx, fmaxf(fabsf(P[r][0]), fabsf(P[r][1])));
  mx = wave_max(mx);
  if ((tid & 63) == 0) sm.red[tid >> 6] = mx;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < NW; ++w) mx = fmaxf(mx, sm.red[w]);
  const float sn = mx > 0.f ? mx / qm : 1.0f;
  const float f = 1.0f / sn;
  const uint32_t mask = (1u << bits) - 1u;
#pragma unroll
  for (int r = 0; r < RPL; ++r) {
    const int bitoff = group_uniform<D>(sm.rinfo[g * RPL + r].x);
    if (worker) {
      staged_put_pair(stage, D, bitoff, bits, c0, fbits(fmaf(P[r][0], f, kMagic)) & mask,
                      fbits(fmaf(P[r][1], f, kMagic)) & mask);
    }
  }
  __syncthreads();
  for (int e = tid * 4; e < TW; e += G::BS * 4)
    *reinterpret_cast<uint4*>(tw + e) = *reinterpret_cast<const uint4*>(stage + e);
  if (tid == 0) *reinterpret_cast<uint32_t*>(sc) = fbits(sn);
}

template <int D, int kMode, bool kReadout>
__global__ __launch_bounds__(GeoM<D>::BS)
void k_decode_mixed(const Tables T, const StepArgs A) {
  constexpr bool kCal = kMode == 1, kTileScale = kMode == 2;
  using G = GeoM<D>;
  constexpr int RPL = G::RPL, LPG = G::LPG;
  __shared__ SmemG<D, kMode == 0> sm;
  extern __shared__ __align__(16) uint32_t stage[];
  const int tile = blockIdx.x;
  const int b = tile / T.H, h = tile - b * T.H;
  const int slot = A.slot_ids[b];
  const int tid = threadIdx.x;
  if (slot < 0 || slot >= A.num_slots) {
    if (A.o != nullptr)
      for (int j = tid; j < D; j += blockDim.x) A.o[static_cast<size_t>(tile) * D + j] = __builtin_nanf("");
    return;
  }
  const bool worker = (G::NT == G::BS) || tid < G::NT;
  const int g = group_uniform<D>(worker ? tid / LPG : 0);
  const int l = worker ? tid % LPG : 0;
  const int c0 = 2 * l;
  uint32_t* tw = reinterpret_cast<uint32_t*>(A.pool + static_cast<size_t>(slot) * T.slot_bytes) + T.head_woff[h];
  uint16_t* sc = A.scales + (static_cast<size_t>(slot) * T.H + h) * 2 * D;
  const bool has_int = (T.head_flags[h] & kHeadHasInt) != 0;
  const int TW = tile_words_of(T, h);

  for (int e = tid * 4; e < TW; e += G::BS * 4)
    *reinterpret_cast<uint4*>(stage + e) = *reinterpret_cast<const uint4*>(tw + e);
  for (int e = TW + tid; e < TW + D; e += G::BS) stage[e] = 0u;   // guard word row
  float cha = 1.f, chb = 1.f, s_tile = 1.f;
  if (kTileScale) {
    s_tile = bitsf(*reinterpret_cast<const uint32_t*>(sc));
  } else if (has_int) {
    const uint32_t chw = *reinterpret_cast<const uint32_t*>(sc + D + c0);
    cha = half_to_float(chw);
    chb = half_to_float(chw >> 16);
  }
  const float2 vv = *reinterpret_cast<const float2*>((A.v + static_cast<size_t>(tile) * D) + static_cast<uint32_t>(c0));
  const float beta = A.beta[tile];
  float pqk = 0.f;
  if (tid < D) {
    const RowInfo ri = T.rows[h * D + tid];
    const float ki = (A.k + static_cast<size_t>(tile) * D)[static_cast<uint32_t>(tid)];
    const float qi = (A.q + static_cast<size_t>(tile) * D)[static_cast<uint32_t>(tid)];
    const float a = T.gate_mode == 0 ? A.gate[tile] : A.gate[static_cast<size_t>(tile) * D + tid];
    const float rh = kTileScale ? s_tile : (kCal ? ri.rhat : half_to_float(sc[tid]));
    const float alpha = ri.bits <= 8 ? rh * a : a;
    sm.coefA[tid] = make_float4(ki, qi, alpha, beta * ki);
    if constexpr (kCal) sm.coefB[tid] = calibrated_coef(ri);
    sm.rinfo[tid] = make_int2(ri.bitoff, ri.bits);
    pqk = qi * ki;
  }
  pqk = wave_sum(pqk);
  if ((tid & 63) == 0 && tid < D) sm.qk[tid >> 6] = pqk;
  __syncthreads();

  float P[RPL][2];
  float Ua = 0.f, Ub = 0.f, Wa = 0.f, Wb = 0.f;
  const RowInfo* rrow = T.rows + h * D + g * RPL;     // scalar loads when a group fills a wave
  // all rows' fields first (no branch between the LDS reads), then the values
  uint32_t fra[RPL], frb[RPL];
#pragma unroll
  for (int r = 0; r < RPL; ++r) {
    const uint2 fp = staged_pair(stage, D, group_uniform<D>(rrow[r].bitoff), group_uniform<D>(rrow[r].bits), c0);
    fra[r] = fp.x;
    frb[r] = fp.y;
  }
#pragma unroll
  for (int r = 0; r < RPL; ++r) {
    const int i = g * RPL + r;
    const int bits = group_uniform<D>(rrow[r].bits);
    const float4 c = sm.coefA[i];
    const float ma = staged_value_sel(fra[r], bits) * (bits <= 8 ? c.z * cha : c.z);
    const float mb = staged_value_sel(frb[r], bits) * (bits <= 8 ? c.z * chb : c.z);
    Ua = fmaf(c.x, ma, Ua);
    Ub = fmaf(c.x, mb, Ub);
    Wa = fmaf(c.y, ma, Wa);
    Wb = fmaf(c.y, mb, Wb);
    P[r][0] = ma;
    P[r][1] = mb;
  }
  if (worker) sm.colA[g][l] = make_float4(Ua, Ub, Wa, Wb);
  __syncthreads();
  for (int e = tid; e < TW; e += G::BS) stage[e] = 0u;   // staged words now become the output
  float qk = 0.f;
#pragma unroll
  for (int w = 0; w < (D + 63) / 64; ++w) qk += sm.qk[w];
  Ua = Ub = Wa = Wb = 0.f;
#pragma unroll
  for (int gg = 0; gg < G::NG; ++gg) {
    const float4 x = sm.colA[gg][l];
    Ua += x.x; Ub += x.y; Wa += x.z; Wb += x.w;
  }
  const float da = vv.x - Ua, db = vv.y - Ub;
  if (worker && g == 0 && A.o != nullptr) {
    const float bq = beta * qk;
    *reinterpret_cast<float2*>((A.o + static_cast<size_t>(tile) * D) + static_cast<uint32_t>(c0)) = make_float2(fmaf(bq, da, Wa), fmaf(bq, db, Wb));
  }
  if constexpr (kReadout) return;
#pragma unroll
  for (int r = 0; r < RPL; ++r) {
    const int i = g * RPL + r;
    const int bits = group_uniform<D>(rrow[r].bits);
    const float gam = sm.coefA[i].w;
    const float ma = fmaf(gam, da, P[r][0]), mb = fmaf(gam, db, P[r][1]);
    if constexpr (kMode == 0) {
      if (worker) sm.rowbuf[g][r][l] = bits <= 8 ? fmaf(mb, mb, ma * ma) : 0.f;
    }
    P[r][0] = ma;
    P[r][1] = mb;
  }
  if constexpr (kTileScale) {
    requant_tile_mixed<D>(sm, stage, P, tw, sc, TW, worker, g, l);
  } else {
    requant_mixed<D, kCal>(sm, stage, T, h, P, tw, sc, TW, has_int, worker, g, l);
  }
}

template <int D, int kMode>
__global__ __launch_bounds__(GeoM<D>::BS)
void k_pack_mixed(const Tables T, const PackArgs A) {
  constexpr bool kCal = kMode == 1, kTileScale = kMode == 2;
  using G = GeoM<D>;
  constexpr int RPL = G::RPL, LPG = G::LPG;
  __shared__ SmemG<D, kMode == 0> sm;
  extern __shared__ __align__(16) uint32_t stage[];
  const int tile = blockIdx.x;
  const int b = tile / T.H, h = tile - b * T.H;
  const int slot = A.slot_ids[b];
  const int tid = threadIdx.x;
  if (slot < 0 || slot >= A.num_slots) return;
  const bool worker = (G::NT == G::BS) || tid < G::NT;
  const int g = group_uniform<D>(worker ? tid / LPG : 0);
  const int l = worker ? tid % LPG : 0;
  const int c0 = 2 * l;
  uint32_t* tw = reinterpret_cast<uint32_t*>(A.pool + static_cast<size_t>(slot) * T.slot_bytes) + T.head_woff[h];
  uint16_t* sc = A.scales + (static_cast<size_t>(slot) * T.H + h) * 2 * D;
  const bool has_int = (T.head_flags[h] & kHeadHasInt) != 0;
  const int TW = tile_words_of(T, h);
  for (int e = tid; e < TW; e += G::BS) stage[e] = 0u;
  if (tid < D) {
    const RowInfo ri = T.rows[h * D + tid];
    sm.rinfo[tid] = make_int2(ri.bitoff, ri.bits);
    if (ri.bits > 8 || kTileScale) sc[tid] = 0;        // unused row-scale entries
    if (!has_int || kTileScale) sc[D + tid] = 0;       // unused column-scale entries
    if constexpr (kCal) {
      sm.coefB[tid] = calibrated_coef(ri);
      if (ri.bits <= 8) sc[tid] = static_cast<uint16_t>(float_to_half(ri.rhat));
    }
  }
  const float* st = A.state + static_cast<size_t>(tile) * D * D;
  float P[RPL][2];
#pragma unroll
  for (int r = 0; r < RPL; ++r) {
    const float2 x = *reinterpret_cast<const float2*>((st + (g * RPL + r) * D) + static_cast<uint32_t>(c0));
    P[r][0] = x.x;
    P[r][1] = x.y;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < RPL; ++r) {
    const int bits = group_uniform<D>(sm.rinfo[g * RPL + r].y);
    if constexpr (kMode == 0) {
      if (worker) sm.rowbuf[g][r][l] = bits <= 8 ? fmaf(P[r][1], P[r][1], P[r][0] * P[r][0]) : 0.f;
    }
  }
  if constexpr (kTileScale) {
    requant_tile_mixed<D>(sm, stage, P, tw, sc, TW, worker, g, l);
  } else {
    requant_mixed<D, kCal>(sm, stage, T, h, P, tw, sc, TW, has_int, worker, g, l);
  }
}

template <int D, bool kTileScale>
__global__ __launch_bounds__(GeoM<D>::BS) void k_unpack_mixed(const Tables T, const PackArgs A) {
  using G = GeoM<D>;
  constexpr int RPL = G::RPL, LPG = G::LPG;
  __shared__ int2 rinfo[D];
  __shared__ float rhat[D];
  extern __shared__ __align__(16) uint32_t stage[];
  const int tile = blockIdx.x;
  const int b = tile / T.H, h = tile - b * T.H;
  const int slot = A.slot_ids[b];
  const int tid = threadIdx.x;
  if (slot < 0 || slot >= A.num_slots) {
    for (int e = tid; e < D * D; e += blockDim.x) A.state_out[static_cast<size_t>(tile) * D * D + e] = __builtin_nanf("");
    return;
  }
  const bool worker = (G::NT == G::BS) || tid < G::NT;
  const int g = group_uniform<D>(worker ? tid / LPG : 0);
  const int l = worker ? tid % LPG : 0;
  const int c0 = 2 * l;
  const uint32_t* tw =
      reinterpret_cast<const uint32_t*>(A.pool + static_cast<size_t>(slot) * T.slot_bytes) + T.head_woff[h];
  const uint16_t* sc = A.scales + (static_cast<size_t>(slot) * T.H + h) * 2 * D;
  const int TW = tile_words_of(T, h);
  for (int e = tid * 4; e < TW; e += G::BS * 4)
    *reinterpret_cast<uint4*>(stage + e) = *reinterpret_cast<const uint4*>(tw + e);
  for (int e = TW + tid; e < TW + D; e += G::BS) stage[e] = 0u;
  if (tid < D) {
    const RowInfo ri = T.rows[h * D + tid];
    rinfo[tid] = make_int2(ri.bitoff, ri.bits);
    rhat[tid] = kTileScale ? bitsf(*reinterpret_cast<const uint32_t*>(sc)) : half_to_float(sc[tid]);
  }
  const uint32_t chw = *reinterpret_cast<const uint32_t*>(sc + D + c0);
  const float cha = kTileScale ? 1.f : half_to_float(chw), chb = kTileScale ? 1.f : half_to_float(chw >> 16);
  __syncthreads();
  if (!worker) return;
  float* st = A.state_out + static_cast<size_t>(tile) * D * D;
#pragma unroll
  for (int r = 0; r < RPL; ++r) {
    const int i = g * RPL + r;
    const int bitoff = group_uniform<D>(rinfo[i].x);
    const int bits = group_uniform<D>(rinfo[i].y);
    const uint2 fp = staged_pair(stage, D, bitoff, bits, c0);
    float xa = staged_value(fp.x, bits);
    float xb = staged_value(fp.y, bits);
    if (bits <= 8) {
      const float rh = rhat[i];
      xa = (rh * cha) * xa;
      xb = (rh * chb) * xb;
    }
    *reinterpret_cast<float2*>(st + static_cast<uint32_t>(i * D + c0)) = make_float2(xa, xb);
  }
}

size_t mixed_stage_bytes(const Tables& t) {
  return static_cast<size_t>(t.max_tile_words + t.D) * sizeof(uint32_t);
}

// ------------------------------------------------------------ mixed head, D = 128
// At D = 128 each wave takes four blocks of 8 stored rows (a head stores its
// rows by ascending width, so most blocks hold one width); the rows' widths,
// the blocks' first bits and kinds are wave-uniform, held in scalar
// registers, and a stored row's inputs (k, q, the gate, its scales) are those
// of the key row stored there.  Same rule and storage as k_decode_mixed
// (ai.info "Methodology in Plain English"; ai-papers.net "STEPQuantの仕組み"),
// calibrated (kMode 1) or refitted (kMode 0) row scales, with
// f_j = max(c^_j, 2^-64) and every row carried in units of f_j:
//   integer rows: x_ij = code_ij, later Y'_ij = M'_ij / (r^_i f_j)
//                 = a_i x_ij + (beta k_i / r^_i)(d_j / f_j);
//   float rows:   x_ij = h_ij / f_j, later M'_ij / f_j = a_i x_ij + beta k_i (d_j / f_j);
//   u_j = f_j sum_i kappa_i x_ij (kappa = k a r^ or k a), w_j alike with q_i;
//   codes: c0_j = f_j max_int |Y'_ij| / qmax_i, q = rne(Y' f_j / c0_j) in
//   binary32; the least-squares scale c_j = f_j sum w q Y' / sum w q^2 with
//   w = omega r^^2 (0 on float rows).
// Every pass runs block by block: a block of one integer width at
// compile-time field offsets, any other block row by row at run-time offsets
// with the integer-row arithmetic, the few float rows fixed up in
// scalar-branched code (their coefficients in the integer passes are 0).
// Packing: each lane appends its rows' fields to one running word per column
// (alignbit by the row's width; a block of one width first packs its own
// aligned words) and ORs every finished word into the staged tile, which is
// then copied out; a block's words shared with the blocks stored next to it
// are joined by the ORs.
// Refit mode: r^_i is the stored row scale; after the update the row sums
// S_i = sum_j (f_j Y'_ij)^2 = sum_j M'_ij^2 / r^_i^2 are reduced across the
// wave's lanes in registers (lane_row_sums), lane pair 2i, 2i+1 refits
// r'_i = r^_i sqrt(S_i / (D w_i)) (1 for a zero row), stores binary16 r^'_i and
// publishes rho_i = r^_i / r^'_i; rows are then carried as M' / (r^'_i f_j) and
// quantised exactly as in the calibrated mode with r^'_i in place of r^_i.
template <int NG>
struct __align__(16) SmemK {
  static constexpr int D = 128, LPG = 64;
  float4 coefA[D];          // {k a r^ | 0, q a r^ | 0, a, beta k / r^ | beta k} (integer | float row)
  float4 coefB[D];          // {omega r^^2 | 0, 1 / qmax | 0, 0 | k a, 0 | q a}
  float4 colA[NG][LPG];     // column partials (u, w), later (N, Dn)
  float2 colB[NG][LPG];     // column maxima of |Y'| / qmax
  int32_t rowid[D];         // key row held at each storage position (refit: its row scale's slot)
  float qk[2];
};

// Threads per workgroup of k_decode_rows: four waves of 32 stored rows each.
constexpr int kRowsBlock = 256;

// Running words of a lane's two columns: fields are appended LSB-first and
// each finished dword is ORed into the staged tile (row k, columns c0, c0+1).
// alignbit(f, w, n) is w shifted right by n with the low n bits of f on top.
// Only the top `fill` bits of a running word are live: older bits below them
// leave through the bottom as fields arrive, and finish() drops them.
struct RowPacker {
  uint32_t a, b;
  int fill;   // bits already in the running word (wave-uniform)
  int k;      // its dword row (wave-uniform)
  __device__ __forceinline__ void flush(uint32_t* stage, int c0) {
    atomicOr(reinterpret_cast<unsigned long long*>(stage + k * 128 + c0),
             static_cast<unsigned long long>(a) | (static_cast<unsigned long long>(b) << 32));
  }
  // bits in 2..32, wave-uniform
  __device__ __forceinline__ void put(uint32_t* stage, int c0, int bits, uint32_t fa, uint32_t fb) {
    if (bits == 32) {
      if (fill == 0) {
        a = fa;
        b = fb;
        flush(stage, c0);
        a = b = 0u;
      } else {
        a = __builtin_amdgcn_alignbit(fa, a, 32 - fill);
        b = __builtin_amdgcn_alignbit(fb, b, 32 - fill);
        flush(stage, c0);
        a = fa;         // the whole field seeds the next word
        b = fb;
      }
      ++k;
    } else if (fill + bits < 32) {
      a = __builtin_amdgcn_alignbit(fa, a, bits);
      b = __builtin_amdgcn_alignbit(fb, b, bits);
      fill += bits;
    } else if (fill + bits == 32) {
      a = __builtin_amdgcn_alignbit(fa, a, bits);
      b = __builtin_amdgcn_alignbit(fb, b, bits);
      flush(stage, c0);
      a = b = 0u;
      fill = 0;
      ++k;
    } else {
      // the field crosses the word: its low part tops off this word, and the
      // whole field seeds the next one (its low part leaves through the
      // bottom as later fields arrive)
      const int part = 32 - fill;
      a = __builtin_amdgcn_alignbit(fa, a, part);
      b = __builtin_amdgcn_alignbit(fb, b, part);
      flush(stage, c0);
      a = __builtin_amdgcn_alignbit(fa, 0u, bits);
      b = __builtin_amdgcn_alignbit(fb, 0u, bits);
      fill = bits - part;
      ++k;
    }
  }
  // bits in 2..8: one test.  A field that fills the word exactly takes the
  // crossing path: the copy of it seeding the next word leaves through the
  // bottom as later fields arrive, or is dropped when the last word is
  // shifted into place.
  __device__ __forceinline__ void put_int(uint32_t* stage, int c0, int bits, uint32_t fa, uint32_t fb) {
    if (fill + bits < 32) {
      a = __builtin_amdgcn_alignbit(fa, a, bits);
      b = __builtin_amdgcn_alignbit(fb, b, bits);
      fill += bits;
    } else {
      const int part = 32 - fill;
      a = __builtin_amdgcn_alignbit(fa, a, part);
      b = __builtin_amdgcn_alignbit(fb, b, part);
      flush(stage, c0);
      a = __builtin_amdgcn_alignbit(fa, 0u, bits);
      b = __builtin_amdgcn_alignbit(fb, 0u, bits);
      fill = bits - part;
      ++k;
    }
  }
  __device__ __forceinline__ void finish(uint32_t* stage, int c0) {
    if (fill > 0) {
      a = __builtin_amdgcn_alignbit(0u, a, 32 - fill);
      b = __builtin_amdgcn_alignbit(0u, b, 32 - fill);
      flush(stage, c0);
    }
  }
};

// Sign-extended integer code of a field at bit 0 of x (width bits, wave-
// uniform; a float row's field gives a finite value that is not used).  The
// empty asm keeps the signed conversion: without it clang 22 for gfx950
// follows the signed extract with an unsigned int-to-float conversion.
__device__ __forceinline__ float code_value(uint32_t x, int bits) {
  int v = __builtin_amdgcn_sbfe(static_cast<int>(x), 0, bits);
  asm volatile("" : "+v"(v));
  return static_cast<float>(v);
}

// The two staged dwords holding a row's field (bit offset bo, wave-uniform)
// in the lane's two columns: {lo.a, lo.b, hi.a, hi.b}.
__device__ __forceinline__ uint4 staged_words(const uint32_t* stage, int c0, int bo) {
  const int k = bo >> 5;
  const uint2 lo = *reinterpret_cast<const uint2*>(stage + k * 128 + c0);
  const uint2 hi = *reinterpret_cast<const uint2*>(stage + (k + 1) * 128 + c0);
  return make_uint4(lo.x, lo.y, hi.x, hi.y);
}

// The field at bit offset bo of those words, shifted to bit 0.
__device__ __forceinline__ uint2 field_of(const uint4& w, int bo) {
  const int s = bo & 31;
  return make_uint2(__builtin_amdgcn_alignbit(w.z, w.x, s), __builtin_amdgcn_alignbit(w.w, w.y, s));
}

__device__ __forceinline__ uint2 staged_fields(const uint32_t* stage, int c0, int bo) {
  return field_of(staged_words(stage, c0, bo), bo);
}

// Width shared by the 8 stored rows of sub-block sb of a group (0: mixed, or
// a float row among them).
__device__ __forceinline__ int sub_kind(uint32_t kinds, int sb) {
  return static_cast<int>((kinds >> (8 * sb)) & 255u);
}

// Phase 1 of k_decode_rows over sub-block SB of a wave (its rows 8 SB ..
// 8 SB + 7, coefficients at cA[0 .. 7]) when its rows share the integer width
// B: the 8 B bits of each of the lane's two columns start at bit bs of the
// column strings.  They are read
// as two or three staged dwords and shifted down to bit 0 (alignbit by the
// wave-uniform bs & 31); the fields then sit at compile-time offsets.  The
// reads stay inside the staged tile and its guard word row: the sub-block
// ends inside the tile, so its last dword row read is at most the tile's
// word-row count.
template <int B, int SB, int RPL>
__device__ __forceinline__ void rows_fields_uniform(const uint32_t* stage, int c0, int bs, const float4* cA,
                                                    float (&P)[RPL][2], float& Ua, float& Ub, float& Wa,
                                                    float& Wb) {
  const uint32_t* base = stage + (bs >> 5) * 128 + c0;
  const int s = bs & 31;
  const uint2 w0 = *reinterpret_cast<const uint2*>(base);
  const uint2 w1 = *reinterpret_cast<const uint2*>(base + 128);
  uint32_t wa[2] = {__builtin_amdgcn_alignbit(w1.x, w0.x, s), 0u};
  uint32_t wb[2] = {__builtin_amdgcn_alignbit(w1.y, w0.y, s), 0u};
  if constexpr (8 * B > 32) {
    const uint2 w2 = *reinterpret_cast<const uint2*>(base + 256);
    wa[1] = __builtin_amdgcn_alignbit(w2.x, w1.x, s);
    wb[1] = __builtin_amdgcn_alignbit(w2.y, w1.y, s);
  }
  unroll<8>([&](auto I) {
    constexpr int i = decltype(I)::value, r = 8 * SB + i;
    const float4 c = cA[i];
    P[r][0] = static_cast<float>(field_get<B, i>(wa));
    P[r][1] = static_cast<float>(field_get<B, i>(wb));
    Ua = fmaf(c.x, P[r][0], Ua);
    Ub = fmaf(c.x, P[r][1], Ub);
    Wa = fmaf(c.y, P[r][0], Wa);
    Wb = fmaf(c.y, P[r][1], Wb);
  });
}

// Codes, least-squares sums and packing of sub-block SB (coefficients at
// cB[0 .. 7]) when its rows share the integer width B: the same per-row
// arithmetic as the run-time path, the fields packed at compile-time offsets
// into the sub-block's own aligned words (field_put), which then join the
// running words with one append of 32 and one of the remaining 16 bits at
// most.  A partly filled word holds its
// fields at the top (alignbit inserts there), hence the shift by 16.
template <int B, int SB, int RPL>
__device__ __forceinline__ void rows_pack_uniform(RowPacker& pk, uint32_t* stage, int c0, const float4* cB,
                                                  const float (&P)[RPL][2], float sa, float sb, float magic,
                                                  float& Na, float& Nb, float& Da, float& Db) {
  uint32_t oa[2] = {0u, 0u}, ob[2] = {0u, 0u};
  unroll<8>([&](auto I) {
    constexpr int i = decltype(I)::value, r = 8 * SB + i;
    const float w = cB[i].x;
    const float ya = P[r][0], yb = P[r][1];
    const float ma = fmaf(ya, sa, magic), mb = fmaf(yb, sb, magic);
    const float qa = ma - kMagic, qb = mb - kMagic;
    const float ta = w * qa, tb = w * qb;
    Na = fmaf(ta, ya, Na);
    Nb = fmaf(tb, yb, Nb);
    Da = fmaf(ta, qa, Da);
    Db = fmaf(tb, qb, Db);
    field_put<B, i>(oa, fbits(ma));
    field_put<B, i>(ob, fbits(mb));
  });
  if constexpr (B == 2) {
    pk.put(stage, c0, 16, oa[0] >> 16, ob[0] >> 16);
  } else {
    pk.put(stage, c0, 32, oa[0], ob[0]);
    if constexpr (B == 6) pk.put(stage, c0, 16, oa[1] >> 16, ob[1] >> 16);
    if constexpr (B == 8) pk.put(stage, c0, 32, oa[1], ob[1]);
  }
}

// The layout's group table is immutable, so it is read through the constant
// address space: uniform reads of it become scalar loads.
using ConstGroups = const __attribute__((address_space(4))) GroupInfo*;

__device__ __forceinline__ float2 swap32(float x, float y) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, y),
                                                  false, false);
  return make_float2(__builtin_bit_cast(float, static_cast<unsigned>(r[0])),
                     __builtin_bit_cast(float, static_cast<unsigned>(r[1])));
}
__device__ __forceinline__ float2 swap16(float x, float y) {
  const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, y),
                                                  false, false);
  return make_float2(__builtin_bit_cast(float, static_cast<unsigned>(r[0])),
                     __builtin_bit_cast(float, static_cast<unsigned>(r[1])));
}

// Sums of 32 per-lane values v[r] (one per row) over the 64 lanes of a wave,
// with the rows spread over the lanes: in lane l, the sum of row l >> 1.
// Each stage pairs row r with row r + h and lanes across one lane bit: one
// half of the lanes keeps the sum of row r, the other the sum of row r + h
// (bits 5 and 4: permlane swaps, one swap and one add per pair; bits 3, 2 and
// 1: DPP row_ror:8, row_half_mirror and quad_perm [2,3,0,1], two adds and a
// select per pair); a last DPP add joins the two lanes of each row.  The first
// stage is the caller's (row_pair_stage, as each pair of rows r, r + 16 is
// formed), which keeps 16 values live instead of 32.
__device__ __forceinline__ float row_pair_stage(float vr, float vr16) {
  const float2 x = swap32(vr, vr16);
  return x.x + x.y;
}
__device__ __forceinline__ float lane_row_sums(const float (&s1)[16], int lane) {
  float s2[8], s3[4], s4[2];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const float2 x = swap16(s1[r], s1[r + 8]);
    s2[r] = x.x + x.y;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const float a = s2[r] + dpp<0x128>(s2[r]), b = s2[r + 4] + dpp<0x128>(s2[r + 4]);   // row_ror:8
    s3[r] = (lane & 8) ? b : a;
  }
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const float a = s3[r] + dpp<0x141>(s3[r]), b = s3[r + 2] + dpp<0x141>(s3[r + 2]);   // row_half_mirror
    s4[r] = (lane & 4) ? b : a;
  }
  const float a = s4[0] + dpp<0x4e>(s4[0]), b = s4[1] + dpp<0x4e>(s4[1]);               // quad_perm [2,3,0,1]
  const float s5 = (lane & 2) ? b : a;
  return s5 + dpp<0xb1>(s5);                                                            // quad_perm [1,0,3,2]
}

template <int kMode, bool kReadout>
__global__ __launch_bounds__(kRowsBlock) __attribute__((amdgpu_waves_per_eu(4)))
void k_decode_rows(const Tables T, const StepArgs A) {
  constexpr int D = 128, NG = kRowsBlock / 64, RPL = D / NG;
  constexpr bool kRefit = kMode == 0;
  static_assert(kMode == 0 || kMode == 1, "mixed heads carry calibrated or refitted row scales");
  __shared__ SmemK<NG> sm;
  extern __shared__ __align__(16) uint32_t stage[];
  const int tile = blockIdx.x;
  const int b = tile / T.H, h = tile - b * T.H;
  const int slot = A.slot_ids[b];
  const int tid = threadIdx.x;
  if (slot < 0 || slot >= A.num_slots) {
    if (A.o != nullptr)
      for (int j = tid; j < D; j += blockDim.x) A.o[static_cast<size_t>(tile) * D + j] = __builtin_nanf("");
    return;
  }
  // Row group (four blocks) of this wave.  The host deals a head's blocks
  // so that its groups carry similar work; the group-to-wave map also turns
  // with the tile, so that what difference remains does not land on the same
  // SIMD every time.
  const int g = __builtin_amdgcn_readfirstlane(((tid >> 6) + tile) & (NG - 1));
  const int l = tid & 63;
  const int c0 = 2 * l;
  uint32_t* tw = reinterpret_cast<uint32_t*>(A.pool + static_cast<size_t>(slot) * T.slot_bytes) + T.head_woff[h];
  uint16_t* sc = A.scales + (static_cast<size_t>(slot) * T.H + h) * 2 * D;
  const bool has_int = (T.head_flags[h] & kHeadHasInt) != 0;
  const int TW = tile_words_of(T, h);

  // Every load of the prologue is issued before the first wait: the staged
  // words as direct global -> LDS copies (16 B a lane into consecutive LDS,
  // no register round trip), then the column scales, v, beta and the rows'
  // inputs into registers.  The tile arrives in about one memory round trip
  // instead of one per copy-loop iteration and per dependent load.
  {
    const int wave = tid >> 6, lane = tid & 63;
    for (int e = wave * 256; e < TW; e += kRowsBlock * 4)   // 1 KB a wave per copy
      if (e + lane * 4 < TW)
        __builtin_amdgcn_global_load_lds(tw + e + lane * 4, stage + e, 16, 0, 0);
  }
  asm volatile("" ::: "memory");   // the loads below stay behind the copies
  uint32_t chw = 0x3c003c00u;   // binary16 1.0, 1.0
  if (has_int) chw = *reinterpret_cast<const uint32_t*>(sc + D + c0);
  const float2 vv = *reinterpret_cast<const float2*>((A.v + static_cast<size_t>(tile) * D) + static_cast<uint32_t>(c0));
  const float beta = A.beta[tile];
  // thread tid < D sets up key row tid, stored at position ri.pos: its
  // coefficients go to that position's slot (no load waits on another)
  RowInfo ri{};
  float ki = 0.f, qi = 0.f, a = 0.f;
  if (tid < D) {
    ri = T.rows[h * D + tid];
    ki = (A.k + static_cast<size_t>(tile) * D)[static_cast<uint32_t>(tid)];
    qi = (A.q + static_cast<size_t>(tile) * D)[static_cast<uint32_t>(tid)];
    a = T.gate_mode == 0 ? A.gate[tile] : A.gate[static_cast<size_t>(tile) * D + tid];
  }
  for (int e = TW + tid; e < TW + D; e += kRowsBlock) stage[e] = 0u;   // guard word row
  const float cha = half_to_float(chw), chb = half_to_float(chw >> 16);
  const float fa = fmaxf(cha, kFactorMin), fb = fmaxf(chb, kFactorMin);
  float pqk = 0.f;
  if (tid < D) {
    const int p = ri.pos;
    if constexpr (kRefit) sm.rowid[p] = tid;
    if (ri.bits <= 8) {
      const float rh = kRefit ? half_to_float(sc[tid]) : ri.rhat;   // refit: the stored row scale
      const float irh = kRefit ? quotient(1.0f, rh) : ri.inv_rhat;
      const float ar = a * rh;
      sm.coefA[p] = make_float4(ki * ar, qi * ar, a, beta * ki * irh);
      // refit: {w, 1 / qmax, r^, 1 / (D w)} until the row scale is refitted
      sm.coefB[p] = kRefit ? make_float4(ri.omega, ri.inv_qmax, rh, ri.inv_d_omega)
                           : make_float4(ri.u_weight, ri.inv_qmax, 0.f, 0.f);
    } else {
      sm.coefA[p] = make_float4(0.f, 0.f, a, beta * ki);
      sm.coefB[p] = make_float4(0.f, 0.f, ki * a, qi * a);
    }
    pqk = qi * ki;
  }
  pqk = wave_sum(pqk);
  if ((tid & 63) == 0 && tid < D) sm.qk[tid >> 6] = pqk;
  __syncthreads();

  // The wave's rows: four sub-blocks of 8 stored rows, their widths one byte
  // a row (four rows a dword) in scalar registers, their bit offsets, kinds
  // and indices, from the layout's group table (one batch of scalar loads).
  // Held packed, 32 rows take 8 scalar registers instead of 32.  The per-row
  // coefficients are LDS broadcasts from a per-sub-block base.
  const ConstGroups cgrp = (ConstGroups)(T.groups + h * NG + g);
  uint32_t wb[RPL / 4];
#pragma unroll
  for (int i = 0; i < RPL / 4; ++i) {
    wb[i] = cgrp->widths[i];
    asm volatile("" : "+s"(wb[i]));   // keep the packed form: no per-row copies stay live
  }
  const uint32_t offs01 = cgrp->offs[0], offs23 = cgrp->offs[1], kinds = cgrp->kinds, ids = cgrp->ids;
  auto row_bits = [&](int r) { return static_cast<int>((wb[r >> 2] >> (8 * (r & 3))) & 255u); };
  auto sub_bit = [&](int j) { return static_cast<int>(((j < 2 ? offs01 : offs23) >> (16 * (j & 1))) & 0xffffu); };
  auto sub_id = [&](int j) { return static_cast<int>((ids >> (8 * j)) & 255u); };
  const bool has_float = (cgrp->flags & kGroupHasFloat) != 0;
  const float4* cAs[RPL / 8];
  const float4* cBs[RPL / 8];
#pragma unroll
  for (int j = 0; j < RPL / 8; ++j) {
    cAs[j] = &sm.coefA[8 * sub_id(j)];
    cBs[j] = &sm.coefB[8 * sub_id(j)];
  }
  auto cA = [&](int r) -> const float4& { return cAs[r >> 3][r & 7]; };
  auto cB = [&](int r) -> const float4& { return cBs[r >> 3][r & 7]; };

  // --- phase 1: fields -> values, column sums of the k- and q-weighted rows,
  // sub-block by sub-block: one integer width at compile-time offsets, else
  // row by row at run-time offsets (each row's words read while the row
  // before it converts)
  float P[RPL][2];
  float Ua = 0.f, Ub = 0.f, Wa = 0.f, Wb = 0.f;
  unroll<RPL / 8>([&](auto SBc) {
    constexpr int sb = decltype(SBc)::value;
    const int bs = sub_bit(sb);
    switch (sub_kind(kinds, sb)) {
      case 6: rows_fields_uniform<6, sb>(stage, c0, bs, cAs[sb], P, Ua, Ub, Wa, Wb); break;
      case 4: rows_fields_uniform<4, sb>(stage, c0, bs, cAs[sb], P, Ua, Ub, Wa, Wb); break;
      case 8: rows_fields_uniform<8, sb>(stage, c0, bs, cAs[sb], P, Ua, Ub, Wa, Wb); break;
      case 2: rows_fields_uniform<2, sb>(stage, c0, bs, cAs[sb], P, Ua, Ub, Wa, Wb); break;
      default: {
        int bo = bs;
        uint4 w_row = staged_words(stage, c0, bs);
#pragma unroll
        for (int r = 8 * sb; r < 8 * sb + 8; ++r) {
          const int bits = row_bits(r);
          const uint4 w_cur = w_row;
          const int bo_cur = bo;
          bo += bits;
          if (r + 1 < 8 * sb + 8) w_row = staged_words(stage, c0, bo);
          const uint2 f = field_of(w_cur, bo_cur);
          const float4 c = cA(r);
          P[r][0] = code_value(f.x, bits);
          P[r][1] = code_value(f.y, bits);
          Ua = fmaf(c.x, P[r][0], Ua);
          Ub = fmaf(c.x, P[r][1], Ub);
          Wa = fmaf(c.y, P[r][0], Wa);
          Wb = fmaf(c.y, P[r][1], Wb);
        }
      }
    }
  });
  if (has_float) {
    const float ifa = quotient(1.0f, fa), ifb = quotient(1.0f, fb);
    int bf = 0;
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
      if ((r & 7) == 0) bf = sub_bit(r >> 3);
      const int bits = row_bits(r);
      const int bor = bf;
      bf += bits;
      if (bits > 8) {
        const uint2 f = staged_fields(stage, c0, bor);
        const float4 c = cB(r);
        P[r][0] = (bits == 16 ? half_to_float(f.x) : bitsf(f.x)) * ifa;
        P[r][1] = (bits == 16 ? half_to_float(f.y) : bitsf(f.y)) * ifb;
        Ua = fmaf(c.z, P[r][0], Ua);
        Ub = fmaf(c.z, P[r][1], Ub);
        Wa = fmaf(c.w, P[r][0], Wa);
        Wb = fmaf(c.w, P[r][1], Wb);
      }
    }
  }
  sm.colA[g][l] = make_float4(Ua, Ub, Wa, Wb);
  __syncthreads();
  for (int e = tid * 4; e < TW; e += kRowsBlock * 4)           // staged words now become the output
    *reinterpret_cast<uint4*>(stage + e) = make_uint4(0u, 0u, 0u, 0u);
  const float qk = sm.qk[0] + sm.qk[1];
  Ua = Ub = Wa = Wb = 0.f;
#pragma unroll
  for (int gg = 0; gg < NG; ++gg) {
    const float4 x = sm.colA[gg][l];
    Ua += x.x; Ub += x.y; Wa += x.z; Wb += x.w;
  }
  Ua *= fa; Ub *= fb; Wa *= fa; Wb *= fb;
  const float da = vv.x - Ua, db = vv.y - Ub;
  if (g == 0 && A.o != nullptr) {
    const float bq = beta * qk;
    *reinterpret_cast<float2*>((A.o + static_cast<size_t>(tile) * D) + static_cast<uint32_t>(c0)) =
        make_float2(fmaf(bq, da, Wa), fmaf(bq, db, Wb));
  }
  if constexpr (kReadout) return;

  // --- phase 2: every row in units of f_j (a column scale below 2^-64
  // rescales the integer rows' codes by c^_j / f_j first)
  if (cha < kFactorMin || chb < kFactorMin) {
    const float ga = cha / fa, gb = chb / fb;
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
      if (row_bits(r) <= 8) {
        P[r][0] *= ga;
        P[r][1] *= gb;
      }
    }
  }
  const float dpa = quotient(da, fa), dpb = quotient(db, fb);
  float mxa = 0.f, mxb = 0.f;
  if constexpr (kRefit) {
    // Y' and the row sums of M'^2 / r^^2 = sum_j (f_j Y'_ij)^2, reduced in
    // registers; the lane pair of row i refits its scale (integer rows) and
    // publishes {w r^'^2, 1 / qmax, rho = r^ / r^', 0} (float rows: rho = 1)
    const float fa2 = fa * fa, fb2 = fb * fb;
    float s1[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float part[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int rr = r + 16 * u;
        const float4 c = cA(rr);
        P[rr][0] = fmaf(c.w, dpa, c.z * P[rr][0]);
        P[rr][1] = fmaf(c.w, dpb, c.z * P[rr][1]);
        part[u] = fmaf(P[rr][0] * fa2, P[rr][0], (P[rr][1] * fb2) * P[rr][1]);
      }
      s1[r] = row_pair_stage(part[0], part[1]);
    }
    const float S = lane_row_sums(s1, l);
    if ((l & 1) == 0) {
      const int rl = l >> 1, j = rl >> 3;   // the lane pair's row: row rl & 7 of sub-block j
      const int i = 8 * (j == 0 ? sub_id(0) : j == 1 ? sub_id(1) : j == 2 ? sub_id(2) : sub_id(3)) + (rl & 7);
      const float4 cb = sm.coefB[i];
      if (cb.y > 0.f) {              // integer row: cb = {w, 1 / qmax, r^, 1 / (D w)}
        const uint32_t rb = float_to_half(row_scale(S * cb.z * cb.z, cb.w));
        const float rn = half_to_float(rb);
        sc[sm.rowid[i]] = static_cast<uint16_t>(rb);
        sm.coefB[i] = make_float4(cb.x * rn * rn, cb.y, quotient(cb.z, rn), 0.f);
      } else {
        sm.coefB[i].z = 1.0f;
      }
    }
    wave_sync();
#pragma unroll
    for (int sb = 0; sb < RPL / 8; ++sb) {
      if (sub_kind(kinds, sb) != 0) {
        float ua = 0.f, ub = 0.f;
#pragma unroll
        for (int r = 8 * sb; r < 8 * sb + 8; ++r) {
          const float rho = cB(r).z;
          P[r][0] *= rho;
          P[r][1] *= rho;
          ua = fmaxf(ua, fabsf(P[r][0]));
          ub = fmaxf(ub, fabsf(P[r][1]));
        }
        const float iq = cBs[sb][0].y;
        mxa = fmaxf(mxa, ua * iq);
        mxb = fmaxf(mxb, ub * iq);
      } else {
#pragma unroll
        for (int r = 8 * sb; r < 8 * sb + 8; ++r) {
          const float4 cb = cB(r);
          P[r][0] *= cb.z;
          P[r][1] *= cb.z;
          mxa = fmaxf(mxa, fabsf(P[r][0]) * cb.y);
          mxb = fmaxf(mxb, fabsf(P[r][1]) * cb.y);
        }
      }
    }
  } else {
    // a sub-block of one integer width takes the maximum of |Y'| and scales
    // it by the shared 1 / qmax once (rounding is monotone, so the result is
    // the maximum of the scaled values); a mixed one scales row by row
#pragma unroll
    for (int sb = 0; sb < RPL / 8; ++sb) {
      if (sub_kind(kinds, sb) != 0) {
        float ua = 0.f, ub = 0.f;
#pragma unroll
        for (int r = 8 * sb; r < 8 * sb + 8; ++r) {
          const float4 c = cA(r);
          P[r][0] = fmaf(c.w, dpa, c.z * P[r][0]);
          P[r][1] = fmaf(c.w, dpb, c.z * P[r][1]);
          ua = fmaxf(ua, fabsf(P[r][0]));
          ub = fmaxf(ub, fabsf(P[r][1]));
        }
        const float iq = cBs[sb][0].y;
        mxa = fmaxf(mxa, ua * iq);
        mxb = fmaxf(mxb, ub * iq);
      } else {
#pragma unroll
        for (int r = 8 * sb; r < 8 * sb + 8; ++r) {
          const float4 c = cA(r);
          const float iq = cB(r).y;     // 0 on float rows
          P[r][0] = fmaf(c.w, dpa, c.z * P[r][0]);
          P[r][1] = fmaf(c.w, dpb, c.z * P[r][1]);
          mxa = fmaxf(mxa, fabsf(P[r][0]) * iq);
          mxb = fmaxf(mxb, fabsf(P[r][1]) * iq);
        }
      }
    }
  }
  sm.colB[g][l] = make_float2(mxa, mxb);
  __syncthreads();
#pragma unroll
  for (int gg = 0; gg < NG; ++gg) {
    const float2 m = sm.colB[gg][l];
    mxa = fmaxf(mxa, m.x);
    mxb = fmaxf(mxb, m.y);
  }
  const float sa = mxa > 0.f ? quotient(1.0f, mxa) : 1.0f, sb = mxb > 0.f ? quotient(1.0f, mxb) : 1.0f;

  // --- codes, least-squares sums (weight 0 on float rows), packing
  // The least-squares sums of a row are taken before its packing branches
  // (the empty asm): left to the compiler, they sink past all of them and
  // keep every row's codes and weight live until the end.  The rounding
  // constant sits in a scalar register so both columns' roundings are one
  // fma each, and the next row's weight is read while this row packs.
  RowPacker pk;
  float Na = 0.f, Nb = 0.f, Da = 0.f, Db = 0.f;
  float magic;
  asm("s_mov_b32 %0, %1" : "=s"(magic) : "i"(__builtin_bit_cast(int, kMagic)));
  unroll<RPL / 8>([&](auto KBc) {
    constexpr int kb = decltype(KBc)::value;
    // each sub-block starts its own running words at its first bit; the words
    // it shares with the sub-blocks stored next to it are joined by the ORs
    const int bs = sub_bit(kb);
    pk.a = pk.b = 0u;
    pk.fill = bs & 31;
    pk.k = bs >> 5;
    switch (sub_kind(kinds, kb)) {
      case 6: rows_pack_uniform<6, kb>(pk, stage, c0, cBs[kb], P, sa, sb, magic, Na, Nb, Da, Db); break;
      case 4: rows_pack_uniform<4, kb>(pk, stage, c0, cBs[kb], P, sa, sb, magic, Na, Nb, Da, Db); break;
      case 8: rows_pack_uniform<8, kb>(pk, stage, c0, cBs[kb], P, sa, sb, magic, Na, Nb, Da, Db); break;
      case 2: rows_pack_uniform<2, kb>(pk, stage, c0, cBs[kb], P, sa, sb, magic, Na, Nb, Da, Db); break;
      default: {
        float w_next = cB(8 * kb).x;
#pragma unroll
        for (int r = 8 * kb; r < 8 * kb + 8; ++r) {
          const int bits = row_bits(r);
          const float w = w_next;
          if (r + 1 < 8 * kb + 8) w_next = cB(r + 1).x;
          const float ya = P[r][0], yb = P[r][1];
          const float ma = fmaf(ya, sa, magic), mb = fmaf(yb, sb, magic);
          const float qa = ma - kMagic, qb = mb - kMagic;
          const float ta = w * qa, tb = w * qb;
          Na = fmaf(ta, ya, Na);
          Nb = fmaf(tb, yb, Nb);
          Da = fmaf(ta, qa, Da);
          Db = fmaf(tb, qb, Db);
          asm volatile("" : "+v"(Na), "+v"(Nb), "+v"(Da), "+v"(Db));
          if (bits > 8) {          // float row: M' = f_j (M' / f_j)
            const float xa = ya * fa, xb = yb * fb;
            uint32_t ea, eb;
            if (bits == 16) {
              ea = float_to_half(fminf(fmaxf(xa, -kScaleMax), kScaleMax));
              eb = float_to_half(fminf(fmaxf(xb, -kScaleMax), kScaleMax));
            } else {
              ea = fbits(xa);
              eb = fbits(xb);
            }
            pk.put(stage, c0, bits, ea, eb);
          } else {
            pk.put_int(stage, c0, bits, fbits(ma), fbits(mb));
          }
        }
      }
    }
    pk.finish(stage, c0);
  });
  sm.colA[g][l] = make_float4(Na, Nb, Da, Db);
  __syncthreads();
  for (int e = tid * 4; e < TW; e += kRowsBlock * 4)
    *reinterpret_cast<uint4*>(tw + e) = *reinterpret_cast<const uint4*>(stage + e);
  if (has_int && g == 0) {
    Na = Nb = Da = Db = 0.f;
#pragma unroll
    for (int gg = 0; gg < NG; ++gg) {
      const float4 x = sm.colA[gg][l];
      Na += x.x; Nb += x.y; Da += x.z; Db += x.w;
    }
    // a zero column (the only case with a zero denominator) keeps the scale 1;
    // the scale is only stored as binary16: a reciprocal estimate suffices
    float ca = Da > 0.f ? (fa * Na) * __builtin_amdgcn_rcpf(Da) : 1.0f;
    float cb = Db > 0.f ? (fb * Nb) * __builtin_amdgcn_rcpf(Db) : 1.0f;
    ca = fminf(fmaxf(ca, kScaleMin), kScaleMax);
    cb = fminf(fmaxf(cb, kScaleMin), kScaleMax);
    *reinterpret_cast<uint32_t*>(sc + D + c0) = float_to_half(ca) | (float_to_half(cb) << 16);
  }
}

template <int D, bool kReadout>
hipError_t decode_for(const Tables& t, const StepArgs& a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.batch) * t.H), block(Geo<D>::BS), blockm(GeoM<D>::BS);
  const size_t dyn = mixed_stage_bytes(t);
  switch (t.gate_mode * 3 + t.row_mode) {
    case 0:
      if (kReadout) hipLaunchKernelGGL((k_readout_uniform<D, 0>), grid, block, 0, s, t, a);
      else hipLaunchKernelGGL((k_decode_uniform<D, 0>), grid, block, 0, s, t, a);
      break;
    case 1:
      if (kReadout) hipLaunchKernelGGL((k_readout_uniform<D, 1>), grid, block, 0, s, t, a);
      else hipLaunchKernelGGL((k_decode_uniform<D, 1>), grid, block, 0, s, t, a);
      break;
    case 2:
      if (kReadout) hipLaunchKernelGGL((k_readout_uniform<D, 2>), grid, block, 0, s, t, a);
      else hipLaunchKernelGGL((k_decode_uniform<D, 2>), grid, block, 0, s, t, a);
      break;
    case 3:
      if (D == 128 && t.all_uniform) {
        if (kReadout) hipLaunchKernelGGL((k_readout_uniform<128, 0, true>), grid, block, 0, s, t, a);
        else hipLaunchKernelGGL((k_decode_uniform<128, 0, true>), grid, block, 0, s, t, a);
      } else if constexpr (D == 128) {
        hipLaunchKernelGGL((k_decode_rows<0, kReadout>), grid, dim3(kRowsBlock), dyn, s, t, a);
      } else {
        hipLaunchKernelGGL((k_decode_mixed<D, 0, kReadout>), grid, blockm, dyn, s, t, a);
      }
      break;
    case 4:
      if (D == 128 && t.all_uniform) {
        if (kReadout) hipLaunchKernelGGL((k_readout_uniform<128, 1, true>), grid, block, 0, s, t, a);
        else hipLaunchKernelGGL((k_decode_uniform<128, 1, true>), grid, block, 0, s, t, a);
      } else if constexpr (D == 128) {
        hipLaunchKernelGGL((k_decode_rows<1, kReadout>), grid, dim3(kRowsBlock), dyn, s, t, a);
      } else {
        hipLaunchKernelGGL((k_decode_mixed<D, 1, kReadout>), grid, blockm, dyn, s, t, a);
      }
      break;
    case 5:
      if (D == 128 && t.all_uniform) {
        if (kReadout) hipLaunchKernelGGL((k_readout_uniform<128, 2, true>), grid, block, 0, s, t, a);
        else hipLaunchKernelGGL((k_decode_uniform<128, 2, true>), grid, block, 0, s, t, a);
      } else {
        hipLaunchKernelGGL((k_decode_mixed<D, 2, kReadout>), grid, blockm, dyn, s, t, a);
      }
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D>
hipError_t pack_for(const Tables& t, const PackArgs& a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.batch) * t.H), block(Geo<D>::BS), blockm(GeoM<D>::BS);
  const size_t dyn = mixed_stage_bytes(t);
  switch (t.gate_mode * 3 + t.row_mode) {
    case 0: hipLaunchKernelGGL((k_pack_uniform<D, 0>), grid, block, 0, s, t, a); break;
    case 1: hipLaunchKernelGGL((k_pack_uniform<D, 1>), grid, block, 0, s, t, a); break;
    case 2: hipLaunchKernelGGL((k_pack_uniform<D, 2>), grid, block, 0, s, t, a); break;
    case 3: hipLaunchKernelGGL((k_pack_mixed<D, 0>), grid, blockm, dyn, s, t, a); break;
    case 4: hipLaunchKernelGGL((k_pack_mixed<D, 1>), grid, blockm, dyn, s, t, a); break;
    case 5: hipLaunchKernelGGL((k_pack_mixed<D, 2>), grid, blockm, dyn, s, t, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D>
hipError_t unpack_for(const Tables& t, const PackArgs& a, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(a.batch) * t.H), block(Geo<D>::BS), blockm(GeoM<D>::BS);
  const bool ts = t.row_mode == 2;
  if (t.gate_mode == 0) {
    if (ts) hipLaunchKernelGGL((k_unpack_uniform<D, true>), grid, block, 0, s, t, a);
    else hipLaunchKernelGGL((k_unpack_uniform<D, false>), grid, block, 0, s, t, a);
  } else {
    if (ts) hipLaunchKernelGGL((k_unpack_mixed<D, true>), grid, blockm, mixed_stage_bytes(t), s, t, a);
    else hipLaunchKernelGGL((k_unpack_mixed<D, false>), grid, blockm, mixed_stage_bytes(t), s, t, a);
  }
  return hipGetLastError();
}

}  // namespace

size_t mixed_lds_bytes(int D, int max_tile_words) {
  const size_t dyn = static_cast<size_t>(max_tile_words + D) * sizeof(uint32_t);
  switch (D) {
    case 16: return sizeof(SmemG<16>) + dyn;
    case 32: return sizeof(SmemG<32>) + dyn;
    case 64: return sizeof(SmemG<64>) + dyn;
    case 128: return sizeof(SmemG<128>) + dyn;
    default: return 0;
  }
}

hipError_t launch_decode_step(const Tables& t, const StepArgs& a, hipStream_t s) {
  switch (t.D) {
    case 16: return decode_for<16, false>(t, a, s);
    case 32: return decode_for<32, false>(t, a, s);
    case 64: return decode_for<64, false>(t, a, s);
    case 128: return decode_for<128, false>(t, a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_readout(const Tables& t, const StepArgs& a, hipStream_t s) {
  switch (t.D) {
    case 16: return decode_for<16, true>(t, a, s);
    case 32: return decode_for<32, true>(t, a, s);
    case 64: return decode_for<64, true>(t, a, s);
    case 128: return decode_for<128, true>(t, a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_pack(const Tables& t, const PackArgs& a, hipStream_t s) {
  switch (t.D) {
    case 16: return pack_for<16>(t, a, s);
    case 32: return pack_for<32>(t, a, s);
    case 64: return pack_for<64>(t, a, s);
    case 128: return pack_for<128>(t, a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_unpack(const Tables& t, const PackArgs& a, hipStream_t s) {
  switch (t.D) {
    case 16: return unpack_for<16>(t, a, s);
    case 32: return unpack_for<32>(t, a, s);
    case 64: return unpack_for<64>(t, a, s);
    case 128: return unpack_for<128>(t, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace stepq
