// Internal declarations shared by the host API (stepq_api.cpp) and the
// gfx950 kernels (stepq_kernels.hip).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace stepq {

// One (head, key row) entry of the layout's device table, indexed by key row.
// A head stores its rows by ascending width, rows of one width in ascending
// row order; pos is the row's place in that order.
struct alignas(16) RowInfo {
  int32_t bitoff;      // bit offset of the row's field inside its column string
  uint16_t bits;       // field width: 2/4/6/8 integer code, 16 binary16, 32 binary32
  uint16_t pos;        // storage position of the row within its head (0 .. D-1)
  float omega;         // row-impact weight w_i
  float inv_d_omega;   // 1 / (D * w_i): r_i^2 = (sum_j M'_ij^2) / (D w_i) (refit mode)
  float rhat;          // calibrated mode: constant row scale r^_i (a binary16 value)
  float u_weight;      // calibrated mode: w_i r^_i^2, the row's least-squares weight
  float inv_rhat;      // calibrated mode: 1 / r^_i, rounded once (0 on other rows)
  float inv_qmax;      // integer rows: 1 / qmax_i (0 on binary16 / binary32 rows)
};

// The rows one wave handles at D = 128: four sub-blocks of 8 stored rows
// (sub-block s of a head holds storage positions 8s .. 8s+7).  The host deals
// a head's 16 sub-blocks out to its 4 waves so that each wave gets a similar
// share of the dearer ones (mixed widths, float rows).  Row r = 8j + i of the
// wave is row i of its sub-block j.
struct alignas(16) GroupInfo {
  uint32_t widths[8];  // the widths of the wave's 32 rows, one byte a row, four rows a dword
  uint32_t offs[2];    // bit offsets of sub-blocks 0, 1 | 2, 3 in the column strings (16 bits each)
  uint32_t kinds;      // byte j: the integer width (2/4/6/8) shared by sub-block j's rows,
                       // 0 if they differ or hold floats
  uint32_t ids;        // byte j: the head's sub-block index s of sub-block j
  int32_t flags;       // GroupFlags
  int32_t pad[3];
};

enum GroupFlags : int32_t {
  kGroupHasFloat = 1,  // a binary16 or binary32 row among the group's rows
};

enum HeadFlags : int32_t {
  kHeadHasInt = 1,     // at least one integer row (column scales are live)
};

// Immutable layout tables, passed to every kernel by value.
struct Tables {
  const int32_t* head_woff;   // [H] 32-bit word offset of head h's tile inside a slot
  const int32_t* head_bits;   // [H] width shared by all rows of head h, 0 if mixed
  const int32_t* head_flags;  // [H] HeadFlags
  const int32_t* head_words;  // [H] 32-bit words of one tile of head h
  const RowInfo* rows;        // [H*D] by key row
  const GroupInfo* groups;    // [H*4] at D = 128, null otherwise
  int32_t H;
  int32_t D;
  int32_t gate_mode;
  int32_t row_mode;           // 0: row scales refitted every step; 1: calibrated constants
  int32_t max_tile_words;     // largest tile, in 32-bit words
  int32_t all_uniform;        // 1: every head has one width for all its rows
  int64_t slot_bytes;
};

struct StepArgs {
  const int32_t* slot_ids;
  int32_t batch;
  int32_t num_slots;
  const float* q;
  const float* k;
  const float* v;
  const float* beta;
  const float* gate;
  uint8_t* pool;
  uint16_t* scales;
  float* o;                    // nullptr: no readout store
};

struct PackArgs {
  const int32_t* slot_ids;
  int32_t batch;
  int32_t num_slots;
  const float* state;          // pack: input [batch][H][D][D]
  float* state_out;            // unpack: output [batch][H][D][D]
  uint8_t* pool;
  uint16_t* scales;
};

// LDS bytes one block of the mixed-head kernels needs (static + staging).
size_t mixed_lds_bytes(int D, int max_tile_words);

// Launchers (stepq_kernels.hip).  Each returns the launch's hipError_t.
hipError_t launch_decode_step(const Tables& t, const StepArgs& a, hipStream_t s);
hipError_t launch_readout(const Tables& t, const StepArgs& a, hipStream_t s);   // o only, pool untouched
hipError_t launch_pack(const Tables& t, const PackArgs& a, hipStream_t s);
hipError_t launch_unpack(const Tables& t, const PackArgs& a, hipStream_t s);

}  // namespace stepq
