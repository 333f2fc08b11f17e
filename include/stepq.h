/*
 * stepq.h -- C ABI of libstepq.so: STEPQuant packed recurrent-state decode
 * step on AMD Instinct MI355X (gfx950).
 *
 * Method source: the summary pages of "STEPQuant: When and Where Errors
 * Matter in Delta-Rule Recurrent State Quantization" (ai.info AI summary,
 * sections "Key Contributions" and "Methodology in Plain English";
 * ai-papers.net article, section "STEPQuantの仕組み"; ai-trend.me review,
 * sections "방법" and "핵심 용어").
 *
 * Conventions used by every entry point
 *   - A tile is the recurrent state of one (request, head): a D x D float
 *     matrix M with row i = key channel and column j = value channel
 *     (D = d_k = d_v in {16, 32, 64, 128}).
 *   - Pool: caller-owned device bytes, num_slots slots of
 *     stepq_slot_pool_bytes() bytes each.  A slot holds the H tiles of one
 *     request in head order.  Inside a tile, row i of column j is a field of
 *     b_i bits (2/4/6/8: two's-complement integer code, 16: binary16 pivot,
 *     32: binary32); column j's fields are concatenated least-significant bit
 *     first in storage order (ascending width, rows of one width in ascending
 *     row order, so a head of one width keeps plain row order) and
 *     zero-padded to W = ceil(sum_i b_i / 32) dwords; dword w of column j is
 *     the tile's 32-bit word w*D + j.
 *   - Scales: caller-owned device bytes, num_slots * stepq_slot_scale_bytes();
 *     per (slot, head): D binary16 key-row scales r^ followed by D binary16
 *     value-column scales c^.  Integer rows hold r^_i * c^_j * code_ij.
 *     Entries no integer row uses are written as 0.
 *   - slot_ids: device int32 [batch]; request b uses slot slot_ids[b].  Ids
 *     must be distinct within one call.  A tile whose id lies outside
 *     [0, num_slots) is skipped: its pool bytes are not touched and its
 *     outputs (o, or the unpacked state) are written as NaN.
 *   - Device pointers must be 16-byte aligned (pool and scales: 256 bytes
 *     suffices for every slot); all arrays are dense and row-major.
 *   - stream: a hipStream_t passed as void*; NULL means the default stream.
 *     Calls enqueue work and return without synchronising; a fault during
 *     execution surfaces at the caller's next synchronisation.
 *   - Ownership: the caller owns every device buffer.  The library owns only
 *     the layout handle and its small device tables.  pack, unpack and
 *     decode_step never allocate, copy between host and device, or sync.
 *   - Errors: argument checks run before any launch and return
 *     STEPQ_ERR_INVALID_ARG / STEPQ_ERR_UNSUPPORTED without side effects; a
 *     failed launch returns STEPQ_ERR_HIP.  No exceptions cross the ABI.
 *   - A layout handle is immutable after creation and may be used from
 *     several threads and streams at once on disjoint slots.
 *   - Device: a layout's tables live on the HIP device that was current at
 *     stepq_layout_create.  A call with batch > 0 made while another device
 *     is current returns STEPQ_ERR_INVALID_ARG (checked after the pointer
 *     checks, before any launch).
 */
#ifndef STEPQ_H
#define STEPQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  STEPQ_OK = 0,
  STEPQ_ERR_INVALID_ARG = 1,  /* null / misaligned pointer, bad size or width */
  STEPQ_ERR_UNSUPPORTED = 2,  /* well-formed but outside what the library supports */
  STEPQ_ERR_HIP = 3,          /* a HIP runtime call or a launch failed */
  STEPQ_ERR_NO_MEMORY = 4     /* device allocation of the layout tables failed */
} stepq_status;

typedef struct stepq_layout stepq_layout; /* opaque */

/* Row-scale readings.  The pages set a key row's scale from its average
 * magnitude and its impact on the output error (ai-papers.net,
 * "STEPQuantの仕組み"), with the dual-axis scale factors optimised from
 * calibration statistics (ai-feeds.com, key modules 2-3). */
typedef enum {
  STEPQ_ROW_SCALES_REFIT = 0,      /* r_i = RMS_j(M'_ij) / sqrt(w_i), recomputed from
                                      the updated state at every step (1 for a zero
                                      row); stored as binary16 in the scale table.
                                      Re-deriving r from an already quantised row
                                      moves codes at every step: over long low-bit
                                      runs with outlier channels the state drifts
                                      and can diverge (binary16 pivots saturate).
                                      Opt in explicitly; the calibrated mode is the
                                      one to serve with. */
  STEPQ_ROW_SCALES_CALIBRATED = 1, /* r_i = m_i / sqrt(w_i) from the calibrated row
                                      magnitude m_i: a per-row constant of the
                                      layout; only column scales are refitted */
  STEPQ_UNIFORM_TILE_SCALE = 2     /* comparison baseline, not STEPQuant: uniform INT-b
                                      with one absmax scale per tile (ai.info "Main
                                      Findings"), s = binary32(max|M'| / qmax) (1 for a
                                      zero tile), code = rne(M' / s) in binary32, value
                                      = s * code.  Every row of a head must carry the
                                      same integer width (2/4/6/8).  The first two
                                      binary16 entries of the head's scale-table entry
                                      hold s as binary32 (low half first); the rest
                                      are 0 */
} stepq_row_scale_mode;

/* Offline configuration: the bit allocation, the calibrated row-impact
 * weights and (calibrated mode) row magnitudes come from an offline step and
 * are fixed for all requests (ai-papers.net, "STEPQuantの仕組み"; ai-trend.me,
 * "방법"). */
typedef struct {
  int32_t num_heads;        /* H >= 1 */
  int32_t d_k;              /* key channels per head: 16, 32, 64 or 128 */
  int32_t d_v;              /* value channels per head: must equal d_k */
  int32_t gate_mode;        /* 0: one retention per (request, head) (gated DeltaNet);
                               1: one retention per key channel (KDA).  The unit of
                               bit allocation is the head (0) or the key row (1). */
  const uint8_t *unit_bits; /* host; [H] (mode 0) or [H*d_k] (mode 1); each in
                               {2,4,6,8} (integer code), 16 (FP16 pivot) or
                               32 (binary32, zero-loss) */
  const float *row_impact;  /* host; [H*d_k]; row-impact weight w > 0, finite
                               (expected squared weight of a key row's error in
                               the readout, ai.info "Methodology in Plain English") */
  int32_t row_scale_mode;   /* stepq_row_scale_mode */
  const float *row_magnitude; /* host; [H*d_k]; calibrated mode only (NULL otherwise):
                               the row's calibrated RMS magnitude m > 0, finite */
} stepq_layout_desc;

/* Validates desc, derives the pool layout and uploads its tables to the
 * current HIP device.  The only entry point that allocates (device memory
 * for the tables, freed by stepq_layout_destroy).  *out is set only on
 * STEPQ_OK.  STEPQ_ERR_UNSUPPORTED: d_k outside {16, 32, 64, 128}, d_v != d_k,
 * more than 2^20 heads, a slot of 2^31 words or more, or, under the
 * per-key-channel gate, a head whose tile (staged whole in LDS
 * with one guard word row by the decode step) does not fit the device's
 * shared memory per workgroup together with the kernel's own. */
stepq_status stepq_layout_create(const stepq_layout_desc *desc, stepq_layout **out);

/* Frees the handle and its device tables.  NULL is accepted.  The caller
 * must not destroy a layout that queued work still uses. */
void stepq_layout_destroy(stepq_layout *layout);

/* Bytes of one pool slot (all H tiles of a request), a multiple of 256.
 * Returns 0 for a NULL handle. */
size_t stepq_slot_pool_bytes(const stepq_layout *layout);

/* Bytes of one slot's scale-table entry: H * 2 * D * 2 (both modes; in
 * calibrated mode the decode step reads and rewrites only the column half).
 * 0 for NULL. */
size_t stepq_slot_scale_bytes(const stepq_layout *layout);

/* Admission of FP32 states into the packed pool (requantisation of a state,
 * as after every decode step).  state: device float [batch][H][D][D], read
 * only.  Writes the slots' codes / pivots / binary32 rows and scales.
 * Method: key-row-aware dual-axis fitting and quantised writeback (ai.info
 * "Methodology in Plain English"; ai-papers.net "STEPQuantの仕組み"):
 * per integer row the row scale of the layout's row-scale mode, clamped to
 * [2^-14, 65504] and rounded to binary16, r^_i; every later step uses r^_i:
 * clip-free column scale c0_j = max_i |M_ij| / (r^_i qmax_i) (1 for a zero
 * column), codes q = round-half-even(M / (r^_i c0_j)) (decided in binary32:
 * a value within a few binary32 ulps of a rounding tie may take the other
 * neighbour), and the stored column scale is the impact-weighted
 * least-squares fit sum_i w_i r^_i q_ij M_ij / sum_i w_i r^_i^2 q_ij^2.
 * Pivot rows are stored as binary16 saturated to +-65504.  In calibrated mode
 * the row-scale entries of the scale table receive the constant r^_i.
 * batch = 0 is a no-op. */
stepq_status stepq_pack(const stepq_layout *layout, int32_t batch, const int32_t *slot_ids,
                        int32_t num_slots, const float *state, void *pool, void *scales,
                        void *stream);

/* Reconstruction of FP32 states from the packed pool: integer rows give
 * binary32((r^_i * c^_j) * code_ij) (the scale product is exact, so this is
 * one rounding), pivot and binary32 rows give their value (ai-papers.net,
 * "STEPQuantの仕組み").  state: device float [batch][H][D][D], written. */
stepq_status stepq_unpack(const stepq_layout *layout, int32_t batch, const int32_t *slot_ids,
                          int32_t num_slots, const void *pool, const void *scales,
                          float *state, void *stream);

/* One fused decode step for batch*H tiles, updating pool and scales in place
 * (ai.info "Key Contributions" item 4 and "Methodology in Plain English";
 * ai-trend.me "핵심 용어: Gated Delta Rule"):
 *   M~ = Diag(a) M            reconstructed state, decayed by the gate
 *   u  = M~^T k;  M' = M~ + beta k (v - u)^T
 *   o  = M'^T q               readout of the updated state (before requantisation)
 *   then M' is requantised into the slot exactly as stepq_pack does.
 * Reconstruction uses the stored r^ (refit mode) or the layout's constant r^
 * (calibrated mode; the stored row-scale entries are then neither read nor
 * written).
 * q, k: device float [batch][H][D] (q and k are used as given; the callers
 * L2-normalise them).  v: [batch][H][D].  beta: [batch][H].  gate: linear
 * retention a in (0, 1], [batch][H] (mode 0) or [batch][H][D] (mode 1).
 * o: device float [batch][H][D], written; NULL skips the readout store (the
 * second half of the split-phase schedule below). */
stepq_status stepq_decode_step(const stepq_layout *layout, int32_t batch,
                               const int32_t *slot_ids, int32_t num_slots, const float *q,
                               const float *k, const float *v, const float *beta,
                               const float *gate, void *pool, void *scales, float *o,
                               void *stream);

/* Readout of the decode step without the state update: o = M'^T q of the
 * step stepq_decode_step would take with the same arguments (bit-identical
 * to its o), computed from the column sums u = M~^T k and w = M~^T q of the
 * reconstructed state as o = w + beta (q.k)(v - u); pool and scales are only
 * read.  The pages overlap the scale refit and packed writeback with the rest
 * of the model's computation (ai.info "Key Contributions" item 4 and
 * "Methodology in Plain English"): a split-phase schedule calls
 * stepq_readout, lets the consumer of o proceed, and runs
 * stepq_decode_step(..., o = NULL) on another stream ordered after the
 * readout (it overwrites the state the readout reads).  Arguments as for
 * stepq_decode_step; o must not be NULL. */
stepq_status stepq_readout(const stepq_layout *layout, int32_t batch, const int32_t *slot_ids,
                           int32_t num_slots, const float *q, const float *k, const float *v,
                           const float *beta, const float *gate, const void *pool,
                           const void *scales, float *o, void *stream);

/* Static text for a status code; never NULL. */
const char *stepq_status_string(stepq_status status);

#ifdef __cplusplus
}
#endif

#endif /* STEPQ_H */
