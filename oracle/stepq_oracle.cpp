// STEPQuant packed-state decode step -- CPU ORACLE.
//
// TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
// baseline leg of the benchmark may load this library.  The product path (the
// HIP library) never links, loads or calls it, and this file shares no code,
// header, table or constant generator with the HIP path.
//
// It is deliberately plain and slow: float64 arithmetic, one element at a
// time, a bit-by-bit codec, OpenMP only across independent (request, head)
// tiles.  Sources (summary pages of "STEPQuant: When and Where Errors Matter
// in Delta-Rule Recurrent State Quantization"):
//   [AIINFO-METH] ai.info AI summary, section "Methodology in Plain English"
//   [AIINFO-KC]   ai.info AI summary, section "Key Contributions"
//   [AIINFO-MF]   ai.info AI summary, section "Main Findings"
//   [JA-MECH]     ai-papers.net article, section "STEPQuantの仕組み"
//   [KO-METH]     ai-trend.me review, sections "방법" and "핵심 용어"
//   [ZH-METH]     ai-feeds.com summary, section "方法" (key modules 1-3)
// Where the pages leave a step open, the concrete rule used here is the one
// written next to each function; the HIP path implements the same rule.
//
// Storage format (both paths implement it independently from this description):
//   tile = one (request, head) state M, D x D, row i = key channel, column j =
//   value channel.  Each row i has a width b_i: 2/4/6/8 = symmetric two's-
//   complement integer code, 16 = IEEE binary16 pivot, 32 = IEEE binary32
//   (zero-loss).  Column j's fields are concatenated LSB-first into one bit
//   string, the rows in storage order: ascending width, rows of one width in
//   ascending row order (a head whose rows share one width keeps plain row
//   order); the string is zero-padded to W = ceil(sum_i b_i / 32) dwords;
//   dword w of column j is tile word w*D + j.  Tiles of a slot follow head
//   order; a slot is padded to 256 bytes.  Scale table per (slot, head): D
//   binary16 row scales then D binary16 column scales.
//
// Two readings of the row scale are supported (a layout property):
//   calibrated (row magnitudes given): r_i is a per-row constant set offline
//     from the row's calibrated average magnitude and its impact weight
//     ([JA-MECH]: the row scale comes from the row's average size and its
//     influence on the output error; [ZH-METH] modules 2-3: the dual-axis scale
//     factors are optimised from calibration statistics); only the column
//     scales are refitted at every step.
//   refit (no row magnitudes): r_i is recomputed from the current row's RMS at
//     every step.

#include <omp.h>

#include <cfloat>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

namespace {

// ------------------------------------------------------------------ binary16
// IEEE 754 binary16, round to nearest even, from a float64 value in one
// rounding.  Overflow gives +-inf (callers that need saturation clamp first).
uint16_t half_from_double(double x) {
  uint16_t sign = std::signbit(x) ? 0x8000u : 0u;
  double a = std::fabs(x);
  if (std::isnan(x)) return 0x7E00u;
  if (a >= 65520.0) return sign | 0x7C00u;              // rounds past the largest finite
  if (a >= std::ldexp(1.0, -14)) {                        // normal range
    int e;
    double m = std::frexp(a, &e);                         // a = m * 2^e, m in [0.5, 1)
    double n = std::nearbyint(std::ldexp(m, 11));         // 11 significant bits
    if (n >= 2048.0) { n = 1024.0; e += 1; }
    int field = (e - 1) + 15;
    if (field >= 31) return sign | 0x7C00u;
    uint16_t mant = (uint16_t)((int)n - 1024);
    return sign | (uint16_t)(field << 10) | mant;
  }
  double n = std::nearbyint(std::ldexp(a, 24));          // subnormal: units of 2^-24
  return sign | (uint16_t)n;                              // n == 1024 encodes 2^-14 correctly
}

double double_from_half(uint16_t h) {
  int sign = (h >> 15) & 1;
  int field = (h >> 10) & 31;
  int mant = h & 1023;
  double v;
  if (field == 0) v = std::ldexp((double)mant, -24);
  else if (field == 31) v = mant ? NAN : INFINITY;
  else v = std::ldexp((double)(1024 + mant), field - 25);
  return sign ? -v : v;
}

uint32_t bits_of_float(float f) { uint32_t u; std::memcpy(&u, &f, 4); return u; }
float float_of_bits(uint32_t u) { float f; std::memcpy(&f, &u, 4); return f; }

constexpr double kScaleMin = 6.103515625e-05;  // 2^-14, smallest normal binary16
constexpr double kScaleMax = 65504.0;          // largest finite binary16

// ------------------------------------------------------------------ layout
struct Layout {
  int H = 0, D = 0, gate_mode = 0;
  std::vector<int> row_bits;          // [H*D]
  std::vector<double> omega;          // [H*D]
  int row_mode = 0;                   // 0 refit from the row RMS, 1 calibrated constant
  std::vector<double> rcal;           // [H*D] calibrated r^_i (binary16 value), mode 1
  std::vector<int64_t> row_bitoff;    // [H*D] bit offset of the row in its column string
  std::vector<int64_t> head_words;    // words of one tile of head h (W_h * D)
  std::vector<int64_t> head_word_off; // word offset of head h's tile inside a slot
  int64_t slot_bytes = 0;
};

bool width_ok(int b) { return b == 2 || b == 4 || b == 6 || b == 8 || b == 16 || b == 32; }

// Returns 0 on success, 1 on an invalid description.
// row_mag == nullptr selects the refit reading; otherwise row_mag[h*D + i] is
// the calibrated magnitude of row i of head h (positive, finite) and
//   r^_i = fp16(clamp(row_mag_i / sqrt(w_i), 2^-14, 65504)).
int build_layout(int H, int D, int gate_mode, const uint8_t* unit_bits, const float* omega,
                 const float* row_mag, Layout* L) {
  if (H < 1 || !(D == 16 || D == 32 || D == 64 || D == 128)) return 1;
  if (gate_mode != 0 && gate_mode != 1) return 1;
  L->H = H; L->D = D; L->gate_mode = gate_mode;
  L->row_bits.assign((size_t)H * D, 0);
  L->omega.assign((size_t)H * D, 1.0);
  L->row_bitoff.assign((size_t)H * D, 0);
  L->row_mode = row_mag ? 1 : 0;
  L->rcal.assign((size_t)H * D, 0.0);
  L->head_words.assign(H, 0);
  L->head_word_off.assign(H, 0);
  int64_t off = 0;
  for (int h = 0; h < H; ++h) {
    for (int i = 0; i < D; ++i) {
      int b = gate_mode == 0 ? unit_bits[h] : unit_bits[(size_t)h * D + i];
      if (!width_ok(b)) return 1;
      L->row_bits[(size_t)h * D + i] = b;
      if (omega) {
        double w = omega[(size_t)h * D + i];
        if (!(w > 0.0) || !std::isfinite(w)) return 1;
        L->omega[(size_t)h * D + i] = w;
      }
      if (row_mag) {
        double m = row_mag[(size_t)h * D + i];
        if (!(m > 0.0) || !std::isfinite(m) || !omega) return 1;
        double r = m / std::sqrt(L->omega[(size_t)h * D + i]);
        r = r < kScaleMin ? kScaleMin : (r > kScaleMax ? kScaleMax : r);
        L->rcal[(size_t)h * D + i] = double_from_half(half_from_double(r));
      }
    }
    // fields in storage order: every row of width 2, then 4, 6, 8, 16, 32,
    // each width's rows in ascending row order; a row starts after the widths
    // of the rows stored before it
    int64_t bit = 0;
    for (int b : {2, 4, 6, 8, 16, 32}) {
      for (int i = 0; i < D; ++i) {
        if (L->row_bits[(size_t)h * D + i] != b) continue;
        L->row_bitoff[(size_t)h * D + i] = bit;
        bit += b;
      }
    }
    int64_t W = (bit + 31) / 32;
    L->head_words[h] = W * D;
    L->head_word_off[h] = off;
    off += W * D;
  }
  L->slot_bytes = ((off * 4 + 255) / 256) * 256;
  return 0;
}

// ------------------------------------------------------------------ codec
// Column j's bit string, read / written one bit at a time.
uint32_t read_field(const uint32_t* words, int D, int j, int64_t bitpos, int b) {
  uint64_t v = 0;
  for (int p = 0; p < b; ++p) {
    int64_t bit = bitpos + p;
    uint32_t w = words[(bit >> 5) * D + j];
    v |= (uint64_t)((w >> (bit & 31)) & 1u) << p;
  }
  return (uint32_t)v;
}

void write_field(uint32_t* words, int D, int j, int64_t bitpos, int b, uint32_t value) {
  for (int p = 0; p < b; ++p) {
    int64_t bit = bitpos + p;
    uint32_t& w = words[(bit >> 5) * D + j];
    uint32_t m = 1u << (bit & 31);
    if ((value >> p) & 1u) w |= m; else w &= ~m;
  }
}

int32_t sign_extend(uint32_t field, int b) {
  int64_t v = field & ((1ull << b) - 1);
  if (v >= (1ll << (b - 1))) v -= (1ll << b);
  return (int32_t)v;
}

int qmax_of(int b) { return (1 << (b - 1)) - 1; }

// ------------------------------------------------------------------ reconstruct
// [JA-MECH], [AIINFO-KC] item 3: every stored element is the product of its
// key-row scale, its value-column scale and its integer code; FP16 pivots
// [AIINFO-KC] item 2 and zero-loss rows hold the value itself.
// The products r_i * c_j * q are exact in float64.
void reconstruct(const Layout& L, int h, const uint32_t* words, const uint16_t* rhat,
                 const uint16_t* chat, double* M) {
  const int D = L.D;
  for (int i = 0; i < D; ++i) {
    int b = L.row_bits[(size_t)h * D + i];
    int64_t pos = L.row_bitoff[(size_t)h * D + i];
    for (int j = 0; j < D; ++j) {
      uint32_t f = read_field(words, D, j, pos, b);
      double m;
      if (b == 32) m = (double)float_of_bits(f);
      else if (b == 16) m = double_from_half((uint16_t)f);
      else m = double_from_half(rhat[i]) * double_from_half(chat[j]) * (double)sign_extend(f, b);
      M[(size_t)i * D + j] = m;
    }
  }
}

// Diagnostics of one requantisation, exposed for the property tests.
struct QuantDiag {
  double* r = nullptr;     // [D] row scale before binary16 rounding (0 for non-integer rows)
  double* c0 = nullptr;    // [D] clip-free column scale
  double* c = nullptr;     // [D] least-squares column scale before binary16 rounding
  int32_t* codes = nullptr;// [D*D] integer codes (0 for pivot / zero-loss rows)
};

// ------------------------------------------------------------------ column fit
// Step (e) of the rule below: for fixed codes q, the impact-weighted
// least-squares column scale of the stored reconstruction r^_i c q_ij,
//   c_j = argmin_c sum_i w_i (M'_ij - r^_i c q_ij)^2
//       = sum_i w_i r^_i q_ij M'_ij / sum_i w_i r^_i^2 q_ij^2
// over integer rows (c0_j when the denominator is 0), clamped and rounded to
// binary16 ([AIINFO-METH]: the value-column scales are chosen to make the
// impact-weighted error of what is stored as small as possible).  rhat holds
// the stored (binary16) row scales as float64 values.
void fit_columns(const Layout& L, int h, const double* Mp, const double* rhat, const double* c0,
                 const int32_t* code, bool any_int, uint16_t* chat, double* c_out) {
  const int D = L.D;
  const int* bits = &L.row_bits[(size_t)h * D];
  const double* om = &L.omega[(size_t)h * D];
  for (int j = 0; j < D; ++j) {
    double num = 0.0, den = 0.0;
    for (int i = 0; i < D; ++i) {
      if (bits[i] > 8) continue;
      double q = code[(size_t)i * D + j];
      num += om[i] * rhat[i] * q * Mp[(size_t)i * D + j];
      den += om[i] * rhat[i] * rhat[i] * q * q;
    }
    double cj = den > 0.0 ? num / den : c0[j];
    if (c_out) c_out[j] = cj;
    cj = cj < kScaleMin ? kScaleMin : (cj > kScaleMax ? kScaleMax : cj);
    chat[j] = any_int ? half_from_double(cj) : 0;
  }
}

// ------------------------------------------------------------------ requantise
// Key-row-aware dual-axis fitting and quantised writeback of an updated
// state M' (float64), [AIINFO-METH], [JA-MECH], [KO-METH], [ZH-METH] module 2-3.
// Concrete rule (the pages give words, not formulas):
//  (a) pivot rows -> binary16 of M', saturated to +-65504; zero-loss rows ->
//      binary32 of M'.
//  (b) integer rows i, refit reading: rho_i = sqrt(mean_j M'_ij^2);
//      r_i = rho_i / sqrt(w_i) (grows with the row's magnitude, shrinks with
//      its impact weight); a zero row gets r_i = 1; r_i clamped to
//      [2^-14, 65504]; stored r^_i = fp16(r_i).  Calibrated reading: r^_i is
//      the layout's constant (same formula with the calibrated magnitude in
//      place of rho_i), so an on-grid state requantises to itself.  Every
//      later step uses the stored r^_i, the row scale the pool reconstructs
//      with.
//  (c) clip-free column scale c0_j = max_i |M'_ij| / (r^_i * qmax_i) over
//      integer rows (1 if that maximum is 0).
//  (d) code q_ij = clamp(rne(M'_ij / (r^_i * c0_j)), -qmax_i, qmax_i): the
//      point of the grid r^_i c0_j {-qmax_i .. qmax_i} nearest to M'_ij,
//      round half to even of the float64 quotient.  c0_j is not rounded.
//  (e) impact-weighted least-squares column scale for the fixed codes:
//      c_j = argmin_c sum_i w_i (M'_ij - r^_i c q_ij)^2
//          = sum_i w_i r^_i q_ij M'_ij / sum_i w_i r^_i^2 q_ij^2
//      (c0_j if the denominator is 0); stored c^_j = fp16(clamp(c_j)).
//  Scale entries that no integer row uses are written as 0.
void requantize(const Layout& L, int h, const double* Mp, uint32_t* words, uint16_t* rhat,
                uint16_t* chat, QuantDiag* dg) {
  const int D = L.D;
  const int* bits = &L.row_bits[(size_t)h * D];
  const double* om = &L.omega[(size_t)h * D];
  const int64_t* off = &L.row_bitoff[(size_t)h * D];
  std::memset(words, 0, sizeof(uint32_t) * (size_t)L.head_words[h]);

  std::vector<double> r(D, 0.0), rh(D, 0.0), c0(D, 1.0);
  bool any_int = false;
  for (int i = 0; i < D; ++i) {
    int b = bits[i];
    if (b == 32) {
      for (int j = 0; j < D; ++j) write_field(words, D, j, off[i], 32, bits_of_float((float)Mp[(size_t)i * D + j]));
      rhat[i] = 0;
    } else if (b == 16) {
      for (int j = 0; j < D; ++j) {
        double x = Mp[(size_t)i * D + j];
        x = x > kScaleMax ? kScaleMax : (x < -kScaleMax ? -kScaleMax : x);
        write_field(words, D, j, off[i], 16, half_from_double(x));
      }
      rhat[i] = 0;
    } else {
      any_int = true;
      double ri;
      if (L.row_mode == 1) {
        ri = L.rcal[(size_t)h * D + i];
      } else {
        double ss = 0.0;
        for (int j = 0; j < D; ++j) ss += Mp[(size_t)i * D + j] * Mp[(size_t)i * D + j];
        double rho = std::sqrt(ss / D);
        ri = rho == 0.0 ? 1.0 : rho / std::sqrt(om[i]);
        ri = ri < kScaleMin ? kScaleMin : (ri > kScaleMax ? kScaleMax : ri);
      }
      r[i] = ri;
      rhat[i] = half_from_double(ri);
      rh[i] = double_from_half(rhat[i]);
    }
  }
  for (int j = 0; j < D; ++j) {
    double mx = 0.0;
    for (int i = 0; i < D; ++i) {
      int b = bits[i];
      if (b > 8) continue;
      double t = std::fabs(Mp[(size_t)i * D + j]) / (rh[i] * qmax_of(b));
      if (t > mx) mx = t;
    }
    c0[j] = mx > 0.0 ? mx : 1.0;
  }
  std::vector<int32_t> code((size_t)D * D, 0);
  for (int i = 0; i < D; ++i) {
    int b = bits[i];
    if (b > 8) continue;
    int qm = qmax_of(b);
    for (int j = 0; j < D; ++j) {
      double y = Mp[(size_t)i * D + j] / (rh[i] * c0[j]);
      double n = std::nearbyint(y);          // round half to even (default rounding mode)
      int32_t q = (int32_t)n;
      if (q > qm) q = qm;
      if (q < -qm) q = -qm;
      code[(size_t)i * D + j] = q;
      write_field(words, D, j, off[i], b, (uint32_t)q & ((1u << b) - 1u));
    }
  }
  fit_columns(L, h, Mp, rh.data(), c0.data(), code.data(), any_int, chat, dg ? dg->c : nullptr);
  if (dg) {
    if (dg->r) for (int i = 0; i < D; ++i) dg->r[i] = r[i];
    if (dg->c0) for (int j = 0; j < D; ++j) dg->c0[j] = c0[j];
    if (dg->codes) for (size_t e = 0; e < (size_t)D * D; ++e) dg->codes[e] = code[e];
  }
}

// ------------------------------------------------------------------ one step
// Gated Delta rule, [KO-METH] "Gated Delta Rule" glossary entry and
// [AIINFO-METH]: the retention gate decays the old state, then a correction
// writes along the current key.  In the key-row orientation used here
// (M = S^T of the d_v x d_k form  S' = S Diag(a) (I - beta k k^T) + beta v k^T):
//   M~ = Diag(a) M                  (a_i = a for a per-head gate)
//   u  = M~^T k
//   M' = M~ + beta k (v - u)^T      (= (I - beta k k^T) M~ + beta k v^T)
//   o  = M'^T q                     read from the updated state before it is
//                                   requantised ([AIINFO-KC] item 4: rebuild,
//                                   update and readout in one pass, refit and
//                                   writeback after it).
void step_tile(const Layout& L, int h, const float* q, const float* k, const float* v, float beta,
               const float* gate_rows, const uint32_t* words_in, const uint16_t* rhat_in,
               const uint16_t* chat_in, uint32_t* words_out, uint16_t* rhat_out,
               uint16_t* chat_out, float* o, double* Mp_out) {
  const int D = L.D;
  std::vector<double> M((size_t)D * D), Mp((size_t)D * D), u(D, 0.0);
  reconstruct(L, h, words_in, rhat_in, chat_in, M.data());
  for (int i = 0; i < D; ++i)
    for (int j = 0; j < D; ++j) M[(size_t)i * D + j] *= (double)gate_rows[i];
  for (int j = 0; j < D; ++j) {
    double s = 0.0;
    for (int i = 0; i < D; ++i) s += (double)k[i] * M[(size_t)i * D + j];
    u[j] = s;
  }
  for (int i = 0; i < D; ++i)
    for (int j = 0; j < D; ++j)
      Mp[(size_t)i * D + j] = M[(size_t)i * D + j] + (double)beta * (double)k[i] * ((double)v[j] - u[j]);
  for (int j = 0; j < D; ++j) {
    double s = 0.0;
    for (int i = 0; i < D; ++i) s += (double)q[i] * Mp[(size_t)i * D + j];
    o[j] = (float)s;
  }
  if (Mp_out) std::memcpy(Mp_out, Mp.data(), sizeof(double) * (size_t)D * D);
  requantize(L, h, Mp.data(), words_out, rhat_out, chat_out, nullptr);
}

struct PoolView {
  const Layout* L;
  uint8_t* pool;
  uint16_t* scales;
  uint32_t* tile(int slot, int h) const {
    return reinterpret_cast<uint32_t*>(pool + (size_t)slot * L->slot_bytes) + L->head_word_off[h];
  }
  uint16_t* rhat(int slot, int h) const { return scales + ((size_t)slot * L->H + h) * 2 * L->D; }
  uint16_t* chat(int slot, int h) const { return rhat(slot, h) + L->D; }
};

}  // namespace

// ====================================================================== C ABI
extern "C" {

int ora_layout_check(int H, int D, int gate_mode, const uint8_t* unit_bits, const float* omega,
                     const float* row_mag) {
  Layout L;
  return build_layout(H, D, gate_mode, unit_bits, omega, row_mag, &L);
}

int64_t ora_slot_bytes(int H, int D, int gate_mode, const uint8_t* unit_bits) {
  Layout L;
  if (build_layout(H, D, gate_mode, unit_bits, nullptr, nullptr, &L)) return -1;
  return L.slot_bytes;
}

int64_t ora_head_word_offset(int H, int D, int gate_mode, const uint8_t* unit_bits, int h) {
  Layout L;
  if (build_layout(H, D, gate_mode, unit_bits, nullptr, nullptr, &L) || h < 0 || h > H) return -1;
  return h == H ? L.head_word_off[H - 1] + L.head_words[H - 1] : L.head_word_off[h];
}

uint16_t ora_half_from_double(double x) { return half_from_double(x); }
double ora_double_from_half(uint16_t h) { return double_from_half(h); }

// Codec of one tile's bit strings with the rows in the order given (row i of
// fields and row_bits is the i-th row stored): fields[i*D + j] (low b_i bits)
// <-> words[W*D].
void ora_encode_fields(int D, const int32_t* row_bits, const uint32_t* fields, uint32_t* words,
                       int64_t nwords) {
  std::memset(words, 0, sizeof(uint32_t) * (size_t)nwords);
  int64_t pos = 0;
  for (int i = 0; i < D; ++i) {
    int b = row_bits[i];
    for (int j = 0; j < D; ++j) {
      uint32_t f = b == 32 ? fields[(size_t)i * D + j] : fields[(size_t)i * D + j] & ((1u << b) - 1u);
      write_field(words, D, j, pos, b, f);
    }
    pos += b;
  }
}

void ora_decode_fields(int D, const int32_t* row_bits, const uint32_t* words, uint32_t* fields) {
  int64_t pos = 0;
  for (int i = 0; i < D; ++i) {
    int b = row_bits[i];
    for (int j = 0; j < D; ++j) fields[(size_t)i * D + j] = read_field(words, D, j, pos, b);
    pos += b;
  }
}

// Fields of one tile of head h, by original row: fields[i*D + j] <-> words,
// at the layout's bit offsets.
int ora_tile_decode(int H, int D, int gate_mode, const uint8_t* unit_bits, int h, const uint32_t* words,
                    uint32_t* fields) {
  Layout L;
  if (build_layout(H, D, gate_mode, unit_bits, nullptr, nullptr, &L) || h < 0 || h >= H) return 1;
  for (int i = 0; i < D; ++i) {
    int b = L.row_bits[(size_t)h * D + i];
    for (int j = 0; j < D; ++j)
      fields[(size_t)i * D + j] = read_field(words, D, j, L.row_bitoff[(size_t)h * D + i], b);
  }
  return 0;
}

int ora_tile_encode(int H, int D, int gate_mode, const uint8_t* unit_bits, int h, const uint32_t* fields,
                    uint32_t* words) {
  Layout L;
  if (build_layout(H, D, gate_mode, unit_bits, nullptr, nullptr, &L) || h < 0 || h >= H) return 1;
  std::memset(words, 0, sizeof(uint32_t) * (size_t)L.head_words[h]);
  for (int i = 0; i < D; ++i) {
    int b = L.row_bits[(size_t)h * D + i];
    for (int j = 0; j < D; ++j) {
      uint32_t f = b == 32 ? fields[(size_t)i * D + j] : fields[(size_t)i * D + j] & ((1u << b) - 1u);
      write_field(words, D, j, L.row_bitoff[(size_t)h * D + i], b, f);
    }
  }
  return 0;
}

// Requantise one tile of head h from a float64 state; diagnostics optional.
int ora_quantize_tile(int H, int D, int gate_mode, const uint8_t* unit_bits, const float* omega,
                      const float* row_mag, int h, const double* Mp, uint32_t* words, uint16_t* rhat, uint16_t* chat,
                      double* r, double* c0, double* c, int32_t* codes) {
  Layout L;
  if (build_layout(H, D, gate_mode, unit_bits, omega, row_mag, &L)) return 1;
  QuantDiag dg;
  dg.r = r; dg.c0 = c0; dg.c = c; dg.codes = codes;
  requantize(L, h, Mp, words, rhat, chat, &dg);
  return 0;
}

// Column scales of one tile for codes given by the caller (e.g. codes that
// differ from the oracle's own by a rounding tie): r and c0 come from M' by
// the same rule as in requantize, the fit uses the given codes.
int ora_fit_columns_for_codes(int H, int D, int gate_mode, const uint8_t* unit_bits,
                              const float* omega, const float* row_mag, int h, const double* Mp, const int32_t* codes,
                              uint16_t* chat) {
  Layout L;
  if (build_layout(H, D, gate_mode, unit_bits, omega, row_mag, &L)) return 1;
  std::vector<uint32_t> words((size_t)L.head_words[h]);
  std::vector<uint16_t> rh(D), ch(D);
  std::vector<double> r(D), c0(D), rhd(D);
  QuantDiag dg;
  dg.r = r.data(); dg.c0 = c0.data();
  requantize(L, h, Mp, words.data(), rh.data(), ch.data(), &dg);
  bool any_int = false;
  for (int i = 0; i < D; ++i) {
    any_int = any_int || L.row_bits[(size_t)h * D + i] <= 8;
    rhd[i] = double_from_half(rh[i]);
  }
  fit_columns(L, h, Mp, rhd.data(), c0.data(), codes, any_int, chat, nullptr);
  return 0;
}

// Reconstruct one tile of head h in float64.
int ora_reconstruct_tile(int H, int D, int gate_mode, const uint8_t* unit_bits, int h,
                         const uint32_t* words, const uint16_t* rhat, const uint16_t* chat,
                         double* M) {
  Layout L;
  if (build_layout(H, D, gate_mode, unit_bits, nullptr, nullptr, &L)) return 1;
  reconstruct(L, h, words, rhat, chat, M);
  return 0;
}

// Pool-level entry points (same argument meaning as the library's):
//   state [B][H][D][D] f32, pool [num_slots * slot_bytes], scales [num_slots][H][2D] half.
int ora_pack(int H, int D, int gate_mode, const uint8_t* unit_bits, const float* omega,
             const float* row_mag, int B,
             const int32_t* slot_ids, const float* state, uint8_t* pool, uint16_t* scales) {
  Layout L;
  if (build_layout(H, D, gate_mode, unit_bits, omega, row_mag, &L)) return 1;
  PoolView P{&L, pool, scales};
  const int64_t n = (int64_t)B * H;
#pragma omp parallel for schedule(dynamic)
  for (int64_t t = 0; t < n; ++t) {
    int b = (int)(t / H), h = (int)(t % H);
    int slot = slot_ids[b];
    std::vector<double> M((size_t)D * D);
    const float* s = state + (size_t)t * D * D;
    for (size_t e = 0; e < (size_t)D * D; ++e) M[e] = s[e];
    requantize(L, h, M.data(), P.tile(slot, h), P.rhat(slot, h), P.chat(slot, h), nullptr);
  }
  return 0;
}

// Unpack: binary32 state = binary32((r^_i * c^_j) * q_ij) for integer rows (the
// product is exact in float64, so this is a single rounding), the binary16 or
// binary32 value for pivot / zero-loss rows.
int ora_unpack(int H, int D, int gate_mode, const uint8_t* unit_bits, int B,
               const int32_t* slot_ids, const uint8_t* pool, const uint16_t* scales, float* state) {
  Layout L;
  if (build_layout(H, D, gate_mode, unit_bits, nullptr, nullptr, &L)) return 1;
  PoolView P{&L, const_cast<uint8_t*>(pool), const_cast<uint16_t*>(scales)};
  const int64_t n = (int64_t)B * H;
#pragma omp parallel for schedule(dynamic)
  for (int64_t t = 0; t < n; ++t) {
    int b = (int)(t / H), h = (int)(t % H);
    int slot = slot_ids[b];
    std::vector<double> M((size_t)D * D);
    reconstruct(L, h, P.tile(slot, h), P.rhat(slot, h), P.chat(slot, h), M.data());
    float* s = state + (size_t)t * D * D;
    for (size_t e = 0; e < (size_t)D * D; ++e) s[e] = (float)M[e];
  }
  return 0;
}

// One decode step over a list of tiles (tile = b*H + h); tiles == nullptr means
// all B*H tiles.  Reads pool_in/scales_in, writes pool_out/scales_out (these may
// alias the inputs: tiles are independent) and o [B][H][D].
int ora_step(int H, int D, int gate_mode, const uint8_t* unit_bits, const float* omega,
             const float* row_mag, int B,
             const int32_t* slot_ids, const float* q, const float* k, const float* v,
             const float* beta, const float* gate, const uint8_t* pool_in,
             const uint16_t* scales_in, uint8_t* pool_out, uint16_t* scales_out, float* o,
             const int32_t* tiles, int64_t ntiles) {
  Layout L;
  if (build_layout(H, D, gate_mode, unit_bits, omega, row_mag, &L)) return 1;
  PoolView Pin{&L, const_cast<uint8_t*>(pool_in), const_cast<uint16_t*>(scales_in)};
  PoolView Pout{&L, pool_out, scales_out};
  const int64_t n = tiles ? ntiles : (int64_t)B * H;
#pragma omp parallel for schedule(dynamic)
  for (int64_t x = 0; x < n; ++x) {
    int64_t t = tiles ? tiles[x] : x;
    int b = (int)(t / H), h = (int)(t % H);
    int slot = slot_ids[b];
    std::vector<float> a(D);
    for (int i = 0; i < D; ++i) a[i] = gate_mode == 0 ? gate[t] : gate[(size_t)t * D + i];
    std::vector<uint32_t> w((size_t)L.head_words[h]);
    std::vector<uint16_t> rh(D), ch(D);
    step_tile(L, h, q + (size_t)t * D, k + (size_t)t * D, v + (size_t)t * D, beta[t], a.data(),
              Pin.tile(slot, h), Pin.rhat(slot, h), Pin.chat(slot, h), w.data(), rh.data(),
              ch.data(), o + (size_t)t * D, nullptr);
    std::memcpy(Pout.tile(slot, h), w.data(), sizeof(uint32_t) * w.size());
    std::memcpy(Pout.rhat(slot, h), rh.data(), sizeof(uint16_t) * D);
    std::memcpy(Pout.chat(slot, h), ch.data(), sizeof(uint16_t) * D);
  }
  return 0;
}

// One step of a single tile with the float64 updated state M' returned
// (before requantisation), for the invariant and error-recursion tests.
int ora_step_tile_diag(int H, int D, int gate_mode, const uint8_t* unit_bits, const float* omega,
                       const float* row_mag, int h, const float* q, const float* k, const float* v, float beta,
                       const float* gate_rows, const uint32_t* words_in, const uint16_t* rhat_in,
                       const uint16_t* chat_in, uint32_t* words_out, uint16_t* rhat_out,
                       uint16_t* chat_out, float* o, double* Mp) {
  Layout L;
  if (build_layout(H, D, gate_mode, unit_bits, omega, row_mag, &L)) return 1;
  step_tile(L, h, q, k, v, beta, gate_rows, words_in, rhat_in, chat_in, words_out, rhat_out,
            chat_out, o, Mp);
  return 0;
}

// Uniform INT-b state with one absmax scale per tile: the comparison baseline
// of [AIINFO-MF] ("Uniform quantization degrades sharply").  State per tile:
// codes [D*D] int32 and one binary32 scale s; value = s * q.  Requantisation:
// s' = binary32(max|M'| / qmax) (1 if zero), q = clamp(rne(M' / s')), the grid
// point of the stored scale nearest to M' (float64 quotient).
int ora_uniform_step(int B, int H, int D, int gate_mode, int bits, const float* q, const float* k,
                     const float* v, const float* beta, const float* gate, int32_t* codes,
                     float* scale, float* o) {
  if (bits < 2 || bits > 16) return 1;
  const int qm = qmax_of(bits);
  const int64_t n = (int64_t)B * H;
#pragma omp parallel for schedule(dynamic)
  for (int64_t t = 0; t < n; ++t) {
    int32_t* c = codes + (size_t)t * D * D;
    std::vector<double> M((size_t)D * D), u(D, 0.0);
    for (int i = 0; i < D; ++i) {
      double a = gate_mode == 0 ? gate[t] : gate[(size_t)t * D + i];
      for (int j = 0; j < D; ++j) M[(size_t)i * D + j] = a * (double)scale[t] * c[(size_t)i * D + j];
    }
    const float* kk = k + (size_t)t * D;
    const float* qq = q + (size_t)t * D;
    const float* vv = v + (size_t)t * D;
    for (int j = 0; j < D; ++j)
      for (int i = 0; i < D; ++i) u[j] += (double)kk[i] * M[(size_t)i * D + j];
    double mx = 0.0;
    for (int i = 0; i < D; ++i)
      for (int j = 0; j < D; ++j) {
        double& m = M[(size_t)i * D + j];
        m += (double)beta[t] * kk[i] * ((double)vv[j] - u[j]);
        mx = std::fmax(mx, std::fabs(m));
      }
    for (int j = 0; j < D; ++j) {
      double s = 0.0;
      for (int i = 0; i < D; ++i) s += (double)qq[i] * M[(size_t)i * D + j];
      o[(size_t)t * D + j] = (float)s;
    }
    float s32 = mx > 0.0 ? (float)(mx / qm) : 1.0f;
    scale[t] = s32;
    for (size_t e = 0; e < (size_t)D * D; ++e) {
      int32_t x = (int32_t)std::nearbyint(M[e] / (double)s32);
      c[e] = x > qm ? qm : (x < -qm ? -qm : x);
    }
  }
  return 0;
}

// Initial uniform INT-b encoding of a binary32 state (same rule as above).
int ora_uniform_pack(int B, int H, int D, int bits, const float* state, int32_t* codes,
                     float* scale) {
  if (bits < 2 || bits > 16) return 1;
  const int qm = qmax_of(bits);
  const int64_t n = (int64_t)B * H;
#pragma omp parallel for schedule(dynamic)
  for (int64_t t = 0; t < n; ++t) {
    const float* s = state + (size_t)t * D * D;
    double mx = 0.0;
    for (size_t e = 0; e < (size_t)D * D; ++e) mx = std::fmax(mx, std::fabs((double)s[e]));
    float s32 = mx > 0.0 ? (float)(mx / qm) : 1.0f;
    scale[t] = s32;
    for (size_t e = 0; e < (size_t)D * D; ++e) {
      int32_t x = (int32_t)std::nearbyint((double)s[e] / (double)s32);
      codes[(size_t)t * D * D + e] = x > qm ? qm : (x < -qm ? -qm : x);
    }
  }
  return 0;
}

int ora_num_threads() { return omp_get_max_threads(); }

}  // extern "C"
