// Host side of libstepq.so: layout handle, argument checks, launches.
// The storage layout and the step are described in include/stepq.h.
#include "../../include/stepq.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <new>
#include <vector>

#include "stepq_internal.hpp"

struct stepq_layout {
  stepq::Tables tables{};
  int32_t* d_ints = nullptr;           // head_woff | head_bits | head_flags | head_words
  stepq::RowInfo* d_rows = nullptr;
  stepq::GroupInfo* d_groups = nullptr;   // D = 128 only
  size_t slot_bytes = 0;
  size_t scale_bytes = 0;
  int device = 0;
};

namespace {

bool width_ok(int b) { return b == 2 || b == 4 || b == 6 || b == 8 || b == 16 || b == 32; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Calibrated row scale: m / sqrt(w) in double, clamped to the binary16 normal
// range [2^-14, 65504] and rounded to 11 significant bits (round half to even),
// i.e. the binary16 value r^ held in a float.
float calibrated_row_scale(float m, float w) {
  double r = static_cast<double>(m) / std::sqrt(static_cast<double>(w));
  r = std::fmin(std::fmax(r, 6.103515625e-05), 65504.0);
  int e = 0;
  const double f = std::frexp(r, &e);                       // r = f * 2^e, f in [0.5, 1)
  return static_cast<float>(std::ldexp(std::nearbyint(std::ldexp(f, 11)), e - 11));
}

stepq_status check_common(const stepq_layout* l, int32_t batch, const int32_t* slot_ids, int32_t num_slots) {
  if (!l || batch < 0 || num_slots < 1) return STEPQ_ERR_INVALID_ARG;
  if (batch > 0 && (!slot_ids || !aligned(slot_ids, 4))) return STEPQ_ERR_INVALID_ARG;
  if (static_cast<int64_t>(batch) * l->tables.H > 0x7fffffffLL) return STEPQ_ERR_UNSUPPORTED;
  return STEPQ_OK;
}

stepq_status from_hip(hipError_t e) { return e == hipSuccess ? STEPQ_OK : STEPQ_ERR_HIP; }

// The layout's tables are device memory of the device current at creation;
// work for them is only launched while that device is current.
stepq_status check_device(const stepq_layout* l) {
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return STEPQ_ERR_HIP;
  return cur == l->device ? STEPQ_OK : STEPQ_ERR_INVALID_ARG;
}

}  // namespace

extern "C" {

stepq_status stepq_layout_create(const stepq_layout_desc* d, stepq_layout** out) {
  if (!d || !out || !d->unit_bits || !d->row_impact) return STEPQ_ERR_INVALID_ARG;
  if (d->row_scale_mode != STEPQ_ROW_SCALES_REFIT && d->row_scale_mode != STEPQ_ROW_SCALES_CALIBRATED &&
      d->row_scale_mode != STEPQ_UNIFORM_TILE_SCALE)
    return STEPQ_ERR_INVALID_ARG;
  const bool tile_scale = d->row_scale_mode == STEPQ_UNIFORM_TILE_SCALE;
  const bool calibrated = d->row_scale_mode == STEPQ_ROW_SCALES_CALIBRATED;
  if (calibrated && !d->row_magnitude) return STEPQ_ERR_INVALID_ARG;
  const int H = d->num_heads, D = d->d_k;
  if (H < 1 || d->d_k < 1 || d->d_v < 1) return STEPQ_ERR_INVALID_ARG;
  if (d->gate_mode != 0 && d->gate_mode != 1) return STEPQ_ERR_INVALID_ARG;
  if (d->d_k != d->d_v) return STEPQ_ERR_UNSUPPORTED;
  if (!(D == 16 || D == 32 || D == 64 || D == 128)) return STEPQ_ERR_UNSUPPORTED;
  if (H > (1 << 20)) return STEPQ_ERR_UNSUPPORTED;

  std::vector<int32_t> woff(H), hbits(H), hflags(H), hwords(H);
  std::vector<stepq::RowInfo> rows(static_cast<size_t>(H) * D);
  std::vector<int32_t> row_of(static_cast<size_t>(H) * D);   // storage position -> key row (host only)
  int64_t off = 0;
  int32_t max_words = 0;
  bool all_uniform = true;
  for (int h = 0; h < H; ++h) {
    int first = -1;
    bool uniform = true, has_int = false;
    for (int i = 0; i < D; ++i) {
      const int b = d->gate_mode == 0 ? d->unit_bits[h] : d->unit_bits[static_cast<size_t>(h) * D + i];
      if (!width_ok(b)) return STEPQ_ERR_INVALID_ARG;
      const float w = d->row_impact[static_cast<size_t>(h) * D + i];
      if (!(w > 0.0f) || !std::isfinite(w)) return STEPQ_ERR_INVALID_ARG;
      if (first < 0) first = b;
      uniform = uniform && b == first;
      if (tile_scale && (b > 8 || b != first)) return STEPQ_ERR_INVALID_ARG;
      has_int = has_int || b <= 8;
      stepq::RowInfo& r = rows[static_cast<size_t>(h) * D + i];
      r.bitoff = 0;      // set below, once the head's row widths are known
      r.bits = static_cast<uint16_t>(b);
      r.omega = w;
      r.inv_d_omega = static_cast<float>(1.0 / (static_cast<double>(D) * static_cast<double>(w)));
      r.rhat = 0.0f;
      r.u_weight = 0.0f;
      r.inv_rhat = 0.0f;
      r.inv_qmax = b <= 8 ? static_cast<float>(1.0 / ((1 << (b - 1)) - 1)) : 0.0f;
      if (calibrated) {
        const float m = d->row_magnitude[static_cast<size_t>(h) * D + i];
        if (!(m > 0.0f) || !std::isfinite(m)) return STEPQ_ERR_INVALID_ARG;
        if (b <= 8) {
          r.rhat = calibrated_row_scale(m, w);
          r.u_weight = static_cast<float>(static_cast<double>(w) * r.rhat * r.rhat);
          r.inv_rhat = static_cast<float>(1.0 / static_cast<double>(r.rhat));
        }
      }
    }
    // Fields in storage order: ascending width, rows of one width in ascending
    // row order; the column's bit string is padded to dwords.
    int64_t bit = 0;
    int pos = 0;
    for (int b : {2, 4, 6, 8, 16, 32}) {
      for (int i = 0; i < D; ++i) {
        stepq::RowInfo& r = rows[static_cast<size_t>(h) * D + i];
        if (r.bits != b) continue;
        r.bitoff = static_cast<int32_t>(bit);
        r.pos = static_cast<uint16_t>(pos);
        row_of[static_cast<size_t>(h) * D + pos++] = i;
        bit += b;
      }
    }
    const int64_t words = ((bit + 31) / 32) * D;
    if (off + words > 0x7fffffffLL) return STEPQ_ERR_UNSUPPORTED;
    woff[h] = static_cast<int32_t>(off);
    hwords[h] = static_cast<int32_t>(words);
    hbits[h] = uniform ? first : 0;
    all_uniform = all_uniform && uniform;
    hflags[h] = has_int ? stepq::kHeadHasInt : 0;
    max_words = words > max_words ? static_cast<int32_t>(words) : max_words;
    off += words;
  }
  stepq_layout* l = new (std::nothrow) stepq_layout;
  if (!l) return STEPQ_ERR_NO_MEMORY;
  if (hipGetDevice(&l->device) != hipSuccess) {
    delete l;
    return STEPQ_ERR_HIP;
  }
  // The mixed-head body stages a whole tile (+ one guard word row) in LDS.
  if (d->gate_mode == 1) {
    int lds_max = 0;
    if (hipDeviceGetAttribute(&lds_max, hipDeviceAttributeMaxSharedMemoryPerBlock, l->device) != hipSuccess) {
      delete l;
      return STEPQ_ERR_HIP;
    }
    if (stepq::mixed_lds_bytes(D, max_words) > static_cast<size_t>(lds_max)) {
      delete l;
      return STEPQ_ERR_UNSUPPORTED;
    }
  }
  if (hipMalloc(reinterpret_cast<void**>(&l->d_ints), sizeof(int32_t) * 4 * H) != hipSuccess) {
    delete l;
    return STEPQ_ERR_NO_MEMORY;
  }
  if (hipMalloc(reinterpret_cast<void**>(&l->d_rows), sizeof(stepq::RowInfo) * rows.size()) != hipSuccess) {
    (void)hipFree(l->d_ints);
    delete l;
    return STEPQ_ERR_NO_MEMORY;
  }
  // At D = 128: the head's 16 sub-blocks of 8 stored rows dealt out to its 4
  // waves, dearest first, each to the least loaded wave with room (a sub-block
  // of one integer width costs 2, a mixed one 3 plus 1 per float row), then
  // each wave's sub-blocks in storage order.
  std::vector<stepq::GroupInfo> groups;
  if (D == 128) {
    groups.resize(static_cast<size_t>(H) * 4);
    for (int h = 0; h < H; ++h) {
      const stepq::RowInfo* hr = &rows[static_cast<size_t>(h) * D];
      const int32_t* ro = &row_of[static_cast<size_t>(h) * D];
      int kind[16], cost[16], order[16];
      for (int sb = 0; sb < 16; ++sb) {
        const int b0 = hr[ro[8 * sb]].bits;
        bool same = b0 <= 8;
        int nfloat = 0;
        for (int p = 8 * sb; p < 8 * sb + 8; ++p) {
          same = same && hr[ro[p]].bits == b0;
          nfloat += hr[ro[p]].bits > 8 ? 1 : 0;
        }
        kind[sb] = same ? b0 : 0;
        cost[sb] = same ? 2 : 3 + nfloat;
        order[sb] = sb;
      }
      for (int a = 1; a < 16; ++a)       // by cost, dearest first; ties by index
        for (int b = a; b > 0 && (cost[order[b]] > cost[order[b - 1]] ||
                                  (cost[order[b]] == cost[order[b - 1]] && order[b] < order[b - 1]));
             --b) {
          const int t = order[b];
          order[b] = order[b - 1];
          order[b - 1] = t;
        }
      int load[4] = {0, 0, 0, 0}, cnt[4] = {0, 0, 0, 0}, member[4][4];
      for (int a = 0; a < 16; ++a) {
        int w = -1;
        for (int c = 0; c < 4; ++c)
          if (cnt[c] < 4 && (w < 0 || load[c] < load[w])) w = c;
        member[w][cnt[w]++] = order[a];
        load[w] += cost[order[a]];
      }
      for (int w = 0; w < 4; ++w) {
        std::sort(member[w], member[w] + 4);
        stepq::GroupInfo& gi = groups[static_cast<size_t>(h) * 4 + w];
        std::memset(&gi, 0, sizeof(gi));
        for (int j = 0; j < 4; ++j) {
          const int sb = member[w][j];
          gi.ids |= static_cast<uint32_t>(sb) << (8 * j);
          gi.kinds |= static_cast<uint32_t>(kind[sb]) << (8 * j);
          gi.offs[j / 2] |= static_cast<uint32_t>(hr[ro[8 * sb]].bitoff) << (16 * (j % 2));
          for (int i = 0; i < 8; ++i) {
            const int r = 8 * j + i, b = hr[ro[8 * sb + i]].bits;
            gi.widths[r / 4] |= static_cast<uint32_t>(b) << (8 * (r % 4));
            if (b > 8) gi.flags |= stepq::kGroupHasFloat;
          }
        }
      }
    }
    if (hipMalloc(reinterpret_cast<void**>(&l->d_groups), sizeof(stepq::GroupInfo) * groups.size()) != hipSuccess) {
      (void)hipFree(l->d_ints);
      (void)hipFree(l->d_rows);
      delete l;
      return STEPQ_ERR_NO_MEMORY;
    }
    if (hipMemcpy(l->d_groups, groups.data(), sizeof(stepq::GroupInfo) * groups.size(), hipMemcpyHostToDevice) !=
        hipSuccess) {
      (void)hipFree(l->d_ints);
      (void)hipFree(l->d_rows);
      (void)hipFree(l->d_groups);
      delete l;
      return STEPQ_ERR_HIP;
    }
  }
  std::vector<int32_t> ints;
  ints.insert(ints.end(), woff.begin(), woff.end());
  ints.insert(ints.end(), hbits.begin(), hbits.end());
  ints.insert(ints.end(), hflags.begin(), hflags.end());
  ints.insert(ints.end(), hwords.begin(), hwords.end());
  if (hipMemcpy(l->d_ints, ints.data(), sizeof(int32_t) * ints.size(), hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(l->d_rows, rows.data(), sizeof(stepq::RowInfo) * rows.size(), hipMemcpyHostToDevice) != hipSuccess) {
    (void)hipFree(l->d_ints);
    (void)hipFree(l->d_rows);
    (void)hipFree(l->d_groups);
    delete l;
    return STEPQ_ERR_HIP;
  }
  stepq::Tables& t = l->tables;
  t.groups = l->d_groups;
  t.head_woff = l->d_ints;
  t.head_bits = l->d_ints + H;
  t.head_flags = l->d_ints + 2 * H;
  t.head_words = l->d_ints + 3 * H;
  t.rows = l->d_rows;
  t.H = H;
  t.D = D;
  t.gate_mode = d->gate_mode;
  t.row_mode = tile_scale ? 2 : (calibrated ? 1 : 0);
  t.max_tile_words = max_words;
  t.all_uniform = all_uniform ? 1 : 0;
  l->slot_bytes = static_cast<size_t>(((off * 4 + 255) / 256) * 256);
  l->scale_bytes = static_cast<size_t>(H) * 2 * D * sizeof(uint16_t);
  t.slot_bytes = static_cast<int64_t>(l->slot_bytes);
  *out = l;
  return STEPQ_OK;
}

void stepq_layout_destroy(stepq_layout* l) {
  if (!l) return;
  (void)hipFree(l->d_ints);
  (void)hipFree(l->d_rows);
  (void)hipFree(l->d_groups);
  delete l;
}

size_t stepq_slot_pool_bytes(const stepq_layout* l) { return l ? l->slot_bytes : 0; }

size_t stepq_slot_scale_bytes(const stepq_layout* l) { return l ? l->scale_bytes : 0; }

stepq_status stepq_pack(const stepq_layout* l, int32_t batch, const int32_t* slot_ids, int32_t num_slots,
                        const float* state, void* pool, void* scales, void* stream) {
  stepq_status st = check_common(l, batch, slot_ids, num_slots);
  if (st != STEPQ_OK) return st;
  if (batch == 0) return STEPQ_OK;
  if (!state || !pool || !scales || !aligned(state, 16) || !aligned(pool, 16) || !aligned(scales, 16))
    return STEPQ_ERR_INVALID_ARG;
  if ((st = check_device(l)) != STEPQ_OK) return st;
  stepq::PackArgs a{slot_ids, batch, num_slots, state, nullptr, static_cast<uint8_t*>(pool),
                    static_cast<uint16_t*>(scales)};
  return from_hip(stepq::launch_pack(l->tables, a, static_cast<hipStream_t>(stream)));
}

stepq_status stepq_unpack(const stepq_layout* l, int32_t batch, const int32_t* slot_ids, int32_t num_slots,
                          const void* pool, const void* scales, float* state, void* stream) {
  stepq_status st = check_common(l, batch, slot_ids, num_slots);
  if (st != STEPQ_OK) return st;
  if (batch == 0) return STEPQ_OK;
  if (!state || !pool || !scales || !aligned(state, 16) || !aligned(pool, 16) || !aligned(scales, 16))
    return STEPQ_ERR_INVALID_ARG;
  if ((st = check_device(l)) != STEPQ_OK) return st;
  stepq::PackArgs a{slot_ids, batch, num_slots, nullptr, state,
                    const_cast<uint8_t*>(static_cast<const uint8_t*>(pool)),
                    const_cast<uint16_t*>(static_cast<const uint16_t*>(scales))};
  return from_hip(stepq::launch_unpack(l->tables, a, static_cast<hipStream_t>(stream)));
}

stepq_status stepq_decode_step(const stepq_layout* l, int32_t batch, const int32_t* slot_ids, int32_t num_slots,
                               const float* q, const float* k, const float* v, const float* beta,
                               const float* gate, void* pool, void* scales, float* o, void* stream) {
  stepq_status st = check_common(l, batch, slot_ids, num_slots);
  if (st != STEPQ_OK) return st;
  if (batch == 0) return STEPQ_OK;
  const void* ptrs[] = {q, k, v, beta, gate, pool, scales};
  for (const void* p : ptrs)
    if (!p || !aligned(p, 16)) return STEPQ_ERR_INVALID_ARG;
  if (o && !aligned(o, 16)) return STEPQ_ERR_INVALID_ARG;
  if ((st = check_device(l)) != STEPQ_OK) return st;
  stepq::StepArgs a{slot_ids, batch, num_slots, q, k, v, beta, gate,
                    static_cast<uint8_t*>(pool), static_cast<uint16_t*>(scales), o};
  return from_hip(stepq::launch_decode_step(l->tables, a, static_cast<hipStream_t>(stream)));
}

stepq_status stepq_readout(const stepq_layout* l, int32_t batch, const int32_t* slot_ids, int32_t num_slots,
                           const float* q, const float* k, const float* v, const float* beta, const float* gate,
                           const void* pool, const void* scales, float* o, void* stream) {
  stepq_status st = check_common(l, batch, slot_ids, num_slots);
  if (st != STEPQ_OK) return st;
  if (batch == 0) return STEPQ_OK;
  const void* ptrs[] = {q, k, v, beta, gate, pool, scales, o};
  for (const void* p : ptrs)
    if (!p || !aligned(p, 16)) return STEPQ_ERR_INVALID_ARG;
  if ((st = check_device(l)) != STEPQ_OK) return st;
  stepq::StepArgs a{slot_ids, batch, num_slots, q, k, v, beta, gate,
                    const_cast<uint8_t*>(static_cast<const uint8_t*>(pool)),
                    const_cast<uint16_t*>(static_cast<const uint16_t*>(scales)), o};
  return from_hip(stepq::launch_readout(l->tables, a, static_cast<hipStream_t>(stream)));
}

const char* stepq_status_string(stepq_status s) {
  switch (s) {
    case STEPQ_OK: return "ok";
    case STEPQ_ERR_INVALID_ARG: return "invalid argument";
    case STEPQ_ERR_UNSUPPORTED: return "unsupported configuration";
    case STEPQ_ERR_HIP: return "HIP runtime error";
    case STEPQ_ERR_NO_MEMORY: return "out of device memory";
    default: return "unknown status";
  }
}

}  // extern "C"
