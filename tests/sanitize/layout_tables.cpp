// Host check of the layout tables that stepq_layout_create builds, run under
// the address and undefined-behaviour sanitizers on a machine without a GPU.
//
// The library's host side is compiled into this program (its source is
// included, so the layout handle's tables are visible), the kernel launchers
// come from launch_stub.cpp, and the five HIP runtime calls layout creation
// makes are replaced below by host-memory stand-ins: the "device" tables are
// then ordinary host arrays that this program reads back.  Every property is
// recomputed here from the layout description alone:
//   - storage order: a head's rows by ascending width, rows of one width in
//     ascending row order; each row's bit offset is the sum of the widths
//     stored before it, and its position is its rank in that order;
//   - head word counts and offsets, and the slot size;
//   - at D = 128, the group table: the 4 waves' blocks of 8 stored rows cover
//     the head's 16 blocks exactly once, in ascending order within a wave;
//     each block's first bit, kind (shared integer width, else 0) and the
//     widths of its rows match the storage order; the float flag is set
//     exactly when a wave holds a binary16 or binary32 row; and each block
//     sits in the wave the dealing rule names: blocks taken dearest first
//     (cost 2 for a block of one width, 3 plus 1 per float row otherwise;
//     ties by block index), each to the least-loaded wave that holds fewer
//     than 4 (ties to the lower wave).
//
// Input (argv[1]): a text file "H D gate_mode calibrated" followed by the
// unit widths (H or H*D of them).  Prints one summary line; exits non-zero at
// the first violated property.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../quantized_recurrent_state_packed_amd/csrc/stepq_api.cpp"

extern "C" {
hipError_t hipGetDevice(int* d) {
  *d = 0;
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t, int) {
  *v = 160 * 1024;
  return hipSuccess;
}
hipError_t hipMalloc(void** p, size_t n) {
  *p = std::malloc(n == 0 ? 1 : n);
  return *p ? hipSuccess : hipErrorOutOfMemory;
}
hipError_t hipMemcpy(void* dst, const void* src, size_t n, hipMemcpyKind) {
  std::memcpy(dst, src, n);
  return hipSuccess;
}
hipError_t hipFree(void* p) {
  std::free(p);
  return hipSuccess;
}
}

namespace {

int fail(const char* what, int h, int x) {
  std::fprintf(stderr, "FAIL: %s (head %d, at %d)\n", what, h, x);
  return 1;
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 2) return 2;
  FILE* f = std::fopen(argv[1], "r");
  if (!f) return 2;
  int H = 0, D = 0, gate = 0, cal = 0;
  if (std::fscanf(f, "%d %d %d %d", &H, &D, &gate, &cal) != 4) return 2;
  const int n_units = gate == 0 ? H : H * D;
  std::vector<uint8_t> ub(n_units);
  for (int u = 0; u < n_units; ++u) {
    int b = 0;
    if (std::fscanf(f, "%d", &b) != 1) return 2;
    ub[u] = static_cast<uint8_t>(b);
  }
  std::fclose(f);
  std::vector<float> omega(static_cast<size_t>(H) * D), mag(static_cast<size_t>(H) * D);
  for (size_t i = 0; i < omega.size(); ++i) {
    omega[i] = 0.5f + 0.001f * static_cast<float>(i % 997);
    mag[i] = 0.25f + 0.002f * static_cast<float>(i % 499);
  }
  stepq_layout_desc d{};
  d.num_heads = H;
  d.d_k = D;
  d.d_v = D;
  d.gate_mode = gate;
  d.unit_bits = ub.data();
  d.row_impact = omega.data();
  d.row_scale_mode = cal ? STEPQ_ROW_SCALES_CALIBRATED : STEPQ_ROW_SCALES_REFIT;
  d.row_magnitude = cal ? mag.data() : nullptr;
  stepq_layout* l = nullptr;
  if (stepq_layout_create(&d, &l) != STEPQ_OK) return fail("layout creation", -1, 0);
  const stepq::Tables& t = l->tables;

  int64_t off = 0, blocks_of_one_width = 0, blocks = 0;
  for (int h = 0; h < H; ++h) {
    std::vector<int> bits(D), order;
    for (int i = 0; i < D; ++i) bits[i] = gate == 0 ? ub[h] : ub[static_cast<size_t>(h) * D + i];
    for (int b : {2, 4, 6, 8, 16, 32})
      for (int i = 0; i < D; ++i)
        if (bits[i] == b) order.push_back(i);
    if (static_cast<int>(order.size()) != D) return fail("row widths", h, 0);
    std::vector<int64_t> start(D);
    int64_t bit = 0;
    for (int p = 0; p < D; ++p) {
      const stepq::RowInfo& r = t.rows[static_cast<size_t>(h) * D + order[p]];
      if (r.bitoff != bit) return fail("row bit offset", h, p);
      if (r.pos != p) return fail("row storage position", h, p);
      if (r.bits != bits[order[p]]) return fail("row width", h, p);
      start[p] = bit;
      bit += bits[order[p]];
    }
    const int64_t words = (bit + 31) / 32 * D;
    if (t.head_words[h] != words || t.head_woff[h] != off) return fail("head words", h, 0);
    off += words;
    if (D != 128) continue;
    // the dealing rule, from its statement
    int cost[16], want[16];
    for (int sb = 0; sb < 16; ++sb) {
      bool one = bits[order[8 * sb]] <= 8;
      int nfloat = 0;
      for (int i = 0; i < 8; ++i) {
        one = one && bits[order[8 * sb + i]] == bits[order[8 * sb]];
        nfloat += bits[order[8 * sb + i]] > 8 ? 1 : 0;
      }
      cost[sb] = one ? 2 : 3 + nfloat;
    }
    {
      bool taken[16] = {false};
      int wl[4] = {0}, wc[4] = {0};
      for (int n = 0; n < 16; ++n) {
        int best = -1;
        for (int sb = 0; sb < 16; ++sb)
          if (!taken[sb] && (best < 0 || cost[sb] > cost[best])) best = sb;
        taken[best] = true;
        int w = -1;
        for (int c = 0; c < 4; ++c)
          if (wc[c] < 4 && (w < 0 || wl[c] < wl[w])) w = c;
        want[best] = w;
        wl[w] += cost[best];
        wc[w]++;
      }
    }
    int cover[16] = {0};
    for (int w = 0; w < 4; ++w) {
      const stepq::GroupInfo& gi = t.groups[h * 4 + w];
      bool has_float = false;
      int prev = -1;
      for (int j = 0; j < 4; ++j) {
        const int sb = static_cast<int>((gi.ids >> (8 * j)) & 255u);
        if (sb < 0 || sb >= 16 || sb <= prev) return fail("block index order", h, w * 4 + j);
        prev = sb;
        cover[sb]++;
        const int b0 = bits[order[8 * sb]];
        bool same = b0 <= 8;
        int nfloat = 0;
        for (int i = 0; i < 8; ++i) {
          const int b = bits[order[8 * sb + i]];
          const int r = 8 * j + i;
          if (static_cast<int>((gi.widths[r / 4] >> (8 * (r % 4))) & 255u) != b) return fail("group widths", h, r);
          same = same && b == b0;
          nfloat += b > 8 ? 1 : 0;
        }
        has_float = has_float || nfloat > 0;
        const int kind = static_cast<int>((gi.kinds >> (8 * j)) & 255u);
        if (kind != (same ? b0 : 0)) return fail("block kind", h, sb);
        const int64_t first = (gi.offs[j / 2] >> (16 * (j % 2))) & 0xffffu;
        if (first != start[8 * sb]) return fail("block first bit", h, sb);
        if (want[sb] != w) return fail("block dealt to another wave than the rule's", h, sb);
        blocks_of_one_width += same ? 1 : 0;
        blocks += 1;
      }
      if (((gi.flags & stepq::kGroupHasFloat) != 0) != has_float) return fail("float flag", h, w);
    }
    for (int sb = 0; sb < 16; ++sb)
      if (cover[sb] != 1) return fail("blocks covered once", h, sb);
  }
  if (static_cast<int64_t>(stepq_slot_pool_bytes(l)) != (off * 4 + 255) / 256 * 256) return fail("slot bytes", -1, 0);
  std::printf("ok H=%d D=%d gate=%d: %lld of %lld blocks of one width\n", H, D, gate,
              static_cast<long long>(blocks_of_one_width), static_cast<long long>(blocks));
  stepq_layout_destroy(l);
  return 0;
}
