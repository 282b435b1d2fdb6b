/*
 * ecw.h -- entropy-coded weights, decoded inside a batch-1 GEMV on MI355X (gfx950).
 *
 * Plain C ABI.  No C++ types, exceptions or HIP headers cross it.  Every buffer is
 * owned by the caller and the library calls no device allocator.  Device state that
 * outlives a call: the arrival tickets in a caller's dec_gemv workspace (zero
 * between completed calls, see dec_gemv_workspace_size) and the per-GPU scratch
 * array of the allocation-free entry point dec_gemv_noalloc.
 *
 * The operation: a weight matrix W [rows][cols] is stored as independent rANS
 * tiles of 64 rows x tile_cols columns, 32-bit states and 16-bit payload words
 * (EntroPack page, Sections 3.6 and C.3).  dec_gemv decodes the tiles in parallel,
 * rebuilds each weight in registers and multiplies it into y = W x straight away,
 * without writing a weight tensor to memory (MINE page, Section 4.1 "Fused mvm";
 * EntroPack page, Section D names the fusion as the missing step).  Weights per
 * symbol, table size M and tile width are the per-tensor tuning axes of the MINE
 * page (Section 4.2).
 *
 * Status convention: every entry point returns ECW_OK or an error code and, on
 * error, launches nothing and writes no output; ecw_last_error() gives a message
 * (thread-local).  dec_gemv / dec_materialize are asynchronous on the given stream:
 * ECW_OK means "enqueued"; a device fault shows at the caller's next
 * synchronisation.  Calls are reentrant; concurrent calls on different streams are
 * allowed when they use different workspaces.
 */
#ifndef ECW_H
#define ECW_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ECW_ABI_VERSION 3u
#define ECW_PAIR_DIGITS 16
#define ECW_MAX_TUPLES 4096
#define ECW_MAX_TABLES 17
#define ECW_MAX_ALPHABET 256
/* device scratch of dec_gemv_noalloc, per GPU: arrival tickets, then partial sums */
#define ECW_NOALLOC_TICKET_BYTES (64u << 10)
#define ECW_NOALLOC_PARTIAL_BYTES ((8u << 20) - (64u << 10))

typedef struct ihipStream_t* ecw_stream; /* same type as hipStream_t; NULL = default */

typedef enum {
  ECW_OK = 0,
  ECW_E_INVALID_ARG = 1,     /* null pointer, bad size, misaligned buffer, bad dtype */
  ECW_E_UNSUPPORTED = 2,     /* legal coding the library does not implement */
  ECW_E_CORRUPT = 3,         /* blob fails validation */
  ECW_E_BUFFER_TOO_SMALL = 4,
  ECW_E_HIP = 5              /* the HIP runtime refused a launch */
} ecw_status;

typedef enum {
  ECW_P_INT_CODES = 1,       /* signed b-bit integer codes, k per symbol, fp16 row scale */
  ECW_P_BF16_EXP = 2,        /* BF16: 8-bit exponent coded, sign+mantissa byte raw     */
  ECW_P_FP8_E4M3 = 3,        /* OCP E4M3 bytes coded, fp16 row scale                   */
  ECW_P_E8_LATTICE = 4       /* E8 lattice fields, 17 coset-conditioned tables          */
} ecw_payload;

typedef enum {
  ECW_DT_F16 = 1, ECW_DT_BF16 = 2, ECW_DT_F32 = 3, ECW_DT_I8 = 4, ECW_DT_FP8_E4M3 = 5
} ecw_dtype;

/* One coding of one tensor (one point of the per-tensor tuning space). */
typedef struct {
  uint32_t payload;            /* ecw_payload */
  uint32_t rows, cols;         /* N (outputs) x K (inputs); W is row-major [N][K] */
  uint32_t weights_per_symbol; /* k: INT 1|2|4 with code_bits*k <= 8, or 4 with
                                  4-bit codes over stored tuples; BF16 1|2; FP8 1;
                                  E8 8 (BF16 k = 2 and INT quads of 4-bit codes:
                                  cols a multiple of 32 (quads: 64), tile_cols at
                                  most 2048) */
  uint32_t code_bits;          /* INT only: 2, 3 or 4; else 0 */
  uint32_t log2_m;             /* table size M = 2^log2_m, 8..13 */
  uint32_t tile_rows;          /* must be 64 (one wave64 lane per row) */
  uint32_t tile_cols;          /* columns per tile: multiple of 64 (and of 8k);
                                  E8: any multiple of 8 (whole 8-weight blocks) */
  uint32_t recon_dtype;        /* E8 only: ECW_DT_I8 (2v) or ECW_DT_FP8_E4M3 (v); else 0 */
  uint32_t stored_tuples;      /* INT, code_bits 4, k 4 only: t, the 4-tuples of codes
                                  the table stores, 1 .. min(M, ECW_MAX_TUPLES); else 0 */
} ecw_coding;

/* Frequency tables of a coding (host POD).  Table 0 serves every payload except
 * E8, where table 0 codes the coset and table 1 + 8c + j codes field j (z1..z7, then
 * m = floor(z8/2)) given coset c (EntroPack page, Sections 3.3 and A.3).
 * BF16 pairs (k = 2; MINE page, Section 4.1 "Escapes" and Section 4.2 "Tuning t"):
 * a symbol is two 4-bit digits (even column low) into pair_values, the 16 exponents
 * the table codes.  enc_build_tables stores 0 and the 15 most frequent nonzero
 * exponents (ties to the smaller), ascending; pair_values[0] must be 0.  An exponent
 * e != 0 has the first digit d >= 1 with pair_values[d] == e; a weight whose
 * exponent has no digit is escaped: coded as digit 0 with raw byte 0 (+0.0), its
 * bits kept in the tile's correction stream (one 4-byte record).
 * INT quads (code_bits 4, k = 4; the same passages): a symbol is one of the stored
 * 4-tuples of codes (digit q + 8 of column 4j + i at bits 4i..4i+3).
 * enc_build_tables stores the stored_tuples most frequent tuples (ties to the
 * smaller, the zero tuple 0x8888 always kept in place of the last), ascending.  A
 * tuple outside the table is coded as the stored tuple reached by setting the
 * fewest of its codes to 0 (the first such position set in (count, mask) order);
 * each nonzero code so set is escaped, its record holding the code as a bf16
 * number. */
typedef struct {
  uint32_t n_tables;
  uint32_t alphabet[ECW_MAX_TABLES];          /* symbols in use per table (<= 256)   */
  int32_t value_offset[ECW_MAX_TABLES];       /* field value = symbol + value_offset */
  uint16_t freq[ECW_MAX_TABLES][ECW_MAX_ALPHABET];   /* f > 0 iff count > 0; sum = M */
  uint64_t count[ECW_MAX_TABLES][ECW_MAX_ALPHABET];  /* histogram the freqs come from */
  uint8_t pair_values[ECW_PAIR_DIGITS];        /* BF16 pairs: exponent of each digit */
  uint64_t escapes;                            /* pairs / quads: weights escaped (output) */
  /* INT quads: the stored tuples (ascending; symbol i = tuples[i]), their
   * frequencies and the histogram of the tuples they code, n_tuples of each */
  uint32_t n_tuples;
  uint16_t tuples[ECW_MAX_TUPLES];
  uint16_t tuple_freq[ECW_MAX_TUPLES];
  uint64_t tuple_count[ECW_MAX_TUPLES];
} ecw_tables;

/* Validated, device-ready view of one blob (host POD, filled by dec_prepare). */
typedef struct {
  ecw_coding coding;
  uint32_t n_tables, n_row_groups, n_slices, n_tiles;
  uint32_t steps_full, steps_last;   /* symbols per lane in a full / the last slice */
  uint32_t lut_entry_bytes;
  uint32_t waves_per_block;          /* launch shape; dec_prepare sets a default and */
  uint32_t tiles_per_wave;           /* the caller may change it (autotuning)        */
  uint32_t streams_per_wave;         /* 1, or 2: each wave decodes the tiles of two
                                        adjacent row groups at the same slices in
                                        lockstep, sharing the activation reads
                                        (fused GEMV of INT and FP8 payloads, INT
                                        quads with fp16 activations only; BF16, E8
                                        and the decode-only calls use 1) */
  uint32_t row_groups_per_block;     /* >= 1: a block decodes this many row-group
                                        units (streams_per_wave adjacent row groups
                                        each) one after the other, staging the decode
                                        table and activations once */
  uint64_t blob_bytes;
  /* byte ledger of the stored representation */
  uint64_t bytes_words, bytes_raw, bytes_tile_meta, bytes_tables, bytes_scales;
  const void* device_blob;           /* the caller's device copy of the blob */
  uint64_t off_tables, off_lut, off_states, off_offsets, off_words, off_raw, off_scales;
} ecw_tensor;

/* Histogram + frequency normalisation of the logical tensor `w`.
 *   c: coding; w: host, row-major [rows][cols], element type by payload:
 *      INT: int8 codes in [-2^(b-1), 2^(b-1)); BF16: uint16 bit patterns;
 *      FP8: uint8 e4m3fn bytes; E8: int8 doubled coordinates 2v, each block of 8
 *      columns all even or all odd with sum(v) even.
 *   out: filled.  Frequencies minimise the cross-entropy size bound (MINE page,
 *   Section 4.2, "Compressed Size Prediction"); ties go to the smaller symbol.
 * Errors: INVALID_ARG (nulls, bad coding, values out of range), UNSUPPORTED (more
 * distinct symbols than M slots, alphabet > 256). */
ecw_status enc_build_tables(const ecw_coding* c, const void* w, ecw_tables* out);

/* Encode `w` into a self-describing blob (format version 2, little-endian): the
 * symbols of each tile of 64 rows x tile_cols columns are rANS-coded as one
 * independent stream per tile with 32-bit states and 16-bit words, and the blob
 * stores what the EntroPack page lists as the stored representation (Section 3.6:
 * payload words, offsets, terminal states, tables, row scales, layout; Section C.3:
 * per tile the terminal states and a 32-bit payload offset, plus a final boundary
 * offset).  rANS itself is the asymmetric numeral system of the MINE page's Section 3
 * (Background).
 *   t: tables from enc_build_tables for the same w (or any tables with f > 0 for
 *      every occurring symbol); row_scales: host fp16 [rows] (NULL for BF16).
 *   Two-call protocol: blob == NULL -> *blob_bytes = required size, ECW_OK;
 *   otherwise *blob_bytes is the capacity (BUFFER_TOO_SMALL if short) and is set
 *   to the bytes written.
 * Tiles are rANS-coded independently on up to hardware_concurrency host threads. */
ecw_status enc_encode(const ecw_coding* c, const ecw_tables* t, const void* w,
                      const uint16_t* row_scales, void* blob, size_t* blob_bytes);

/* Lattice quantisation for the E8 payload (EntroPack page, Section 3.2: blocks of
 * eight row-normalised weights are quantised to E8 lattice points).  For each of
 * n_blocks blocks of 8 doubles in u (host, [n_blocks][8]) writes the nearest point
 * of E8 = D8 u (D8 + 1/2) as doubled coordinates 2v (host int8 [n_blocks][8]), the
 * logical tensor enc_encode takes for ECW_P_E8_LATTICE.  The nearest point follows
 * Conway and Sloane's decoder: each coordinate rounded half to even; for D8, when
 * the rounded sum is odd, the coordinate with the largest rounding error (lowest
 * index among equals) is rounded the other way; D8 + 1/2 the same on u - 1/2; the
 * closer of the two by squared distance, the integer coset on a tie.
 * Errors: INVALID_ARG (NULL with n_blocks > 0, non-finite input), UNSUPPORTED (a
 * doubled coordinate outside [-127, 127]); nothing is written on error. */
ecw_status enc_e8_nearest(const double* u, size_t n_blocks, int8_t* v2);

/* Validate a blob and describe it.  The checks follow the loader gates of the
 * quantized-artifacts page (sections 0x05A "Parse Before Allocation": checked
 * integer arithmetic before any size is trusted; 0x05B "Container Gates": versions,
 * out-of-bounds, overlapping or misaligned intervals, lengths inconsistent with
 * dtype and shape; 0x05C "Semantic Gates": shapes, layout version and the coding's
 * own invariants).  Nothing is allocated.
 *   host_blob / blob_bytes: the blob in host memory (read only during the call).
 *   device_blob: the same bytes already copied to device memory, 256-byte aligned
 *   (may be NULL for host-only inspection; dec_gemv then refuses the tensor).
 * Checks, before anything is used: magic, version, checked 64-bit section
 * arithmetic, section bounds and overlap, table sums (sum f = M), the decode table
 * against the frequencies, monotone tile offsets, start states in [2^16, 2^32).
 * Errors: INVALID_ARG, CORRUPT, UNSUPPORTED. */
ecw_status dec_prepare(const void* host_blob, size_t blob_bytes, const void* device_blob,
                       ecw_tensor* out);

/* Bytes of device workspace dec_gemv needs for this tensor, launch shape and batch
 * (0 when each row group fits one block).  The workspace is this library's addition
 * to the plain call dec_gemv(stream, tensor, x, y, batch): a short row group split
 * over several blocks (to keep every CU busy) needs a place for its partial sums and
 * a counter for the last block to finish them in a fixed order, and the library does
 * not allocate.  dec_gemv_noalloc is that plain call, with a library-held scratch.
 * The workspace holds the per-block partial sums of row groups that span several
 * blocks and one arrival ticket per row group: the block that arrives last adds the
 * partials in block order, inside the same kernel.  The workspace must be
 * zero-filled before its first use (from a nonzero ticket the wrong block finishes
 * the row group, and its y is wrong or left unwritten, with ECW_OK); every
 * call that completes leaves its tickets at zero again, so later calls and graph
 * replays need no re-initialisation.  One tensor's tickets sit at the start of its
 * workspace for every launch shape; in a group (dec_gemv_group) they move with the
 * other members' launch shapes, so a group workspace is zero-filled again when a
 * member's launch shape changes.  Calls that overlap in time must not share a
 * workspace. */
ecw_status dec_gemv_workspace_size(const ecw_tensor* t, int batch, size_t* bytes);

/* Fused decode + matrix-vector product: y[b][r] = sum_c W[r][c] * x[b][c].
 *   x: device [batch][cols], ECW_DT_F16 or ECW_DT_BF16, 16-byte aligned.
 *   y: device fp32 [batch][rows], overwritten, 16-byte aligned.
 *   batch: 1..4.  workspace: device, >= dec_gemv_workspace_size bytes (NULL if 0).
 * Weight reconstruction (never stored): INT q * scale_r; BF16 the exact bf16 value;
 * FP8 e4m3(q) * scale_r; E8 (2v) * scale_r / 2 or e4m3(v) * scale_r.  Accumulation
 * in fp32; per-row sums are reduced in a fixed order (deterministic).
 * Errors: INVALID_ARG, UNSUPPORTED, HIP. */
ecw_status dec_gemv(ecw_stream stream, const ecw_tensor* t, const void* x, int x_dtype,
                    float* y, int batch, void* workspace, size_t workspace_bytes);

/* dec_gemv without a workspace argument and without any allocation, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same operation, kernels, launch shape,
 * bits and errors as dec_gemv; the arrival tickets and partial sums of row groups
 * that span several blocks live in a file-scope device array of the library, one
 * copy per GPU (held until the process ends): ECW_NOALLOC_TICKET_BYTES of tickets
 * (one u32 per row group) and ECW_NOALLOC_PARTIAL_BYTES of partial sums.  A launch
 * that needs more returns ECW_E_UNSUPPORTED before launching anything (choose a
 * launch shape with fewer blocks per row group, or use dec_gemv).  The first call
 * on a device that needs the array also enqueues a small kernel clearing its ticket
 * region on `stream`.  Every call on one GPU shares that GPU's array: calls that
 * overlap in time on one GPU (different streams without ordering, concurrent graph
 * replays) race and give wrong sums; calls ordered on one stream are safe.
 * Errors: INVALID_ARG, UNSUPPORTED, HIP. */
ecw_status dec_gemv_noalloc(ecw_stream stream, const ecw_tensor* t, const void* x, int x_dtype,
                            float* y, int batch);

/* Grouped launch: several tensors that read the same activations, decoded and
 * multiplied in one kernel launch (MINE page, Section 4.2 "Launch": sections with
 * the same input dimension and quantisation share a launch, e.g. q/k/v and
 * gate/up).  t[0..n): 1 <= n <= 8 tensors with the same payload, code width, codes
 * per symbol, reconstruction dtype, cols and waves_per_block (each keeps its own
 * table size, stored tuples, tile width and tiles per wave); y[i]: device fp32 [batch][t[i]->coding.rows].  x, batch, workspace as for
 * dec_gemv; the workspace size comes from dec_gemv_group_workspace_size.  Results
 * are bit-identical to separate dec_gemv calls with the same launch shapes.
 * Errors: INVALID_ARG, UNSUPPORTED, HIP. */
ecw_status dec_gemv_group_workspace_size(const ecw_tensor* const* t, int n, int batch, size_t* bytes);
ecw_status dec_gemv_group(ecw_stream stream, const ecw_tensor* const* t, int n, const void* x,
                          int x_dtype, float* const* y, int batch, void* workspace,
                          size_t workspace_bytes);

/* Geometry of the one kernel dec_gemv_group launches for these tensors at this
 * batch and activation type, from their launch shapes: grid and block size in
 * threads (grid_threads = 0 when no member has work) and the dynamic LDS bytes per
 * block.  These are the values a profiler's dispatch record shows, so profiles can
 * be matched to launches (two launches with the same kernel and grid differ in
 * LDS); nothing is launched.  Host-only: callable without a GPU.
 * Errors: INVALID_ARG (NULL pointers, n outside 1..8, batch outside 1..4, x_dtype
 * not F16/BF16, a bad launch shape or members with different waves per block). */
ecw_status dec_gemv_group_geometry(const ecw_tensor* const* t, int n, int batch, int x_dtype,
                                   uint32_t* grid_threads, uint32_t* block_threads, size_t* lds_bytes);

/* Launch-shape autotuning for one tensor (MINE page, Section 4.2: per-tensor
 * tuning of the kernel configuration by measured time).  For each candidate shape
 * shapes[4i..4i+3] = (waves_per_block, tiles_per_wave, streams_per_wave,
 * row_groups_per_block), the fused GEMV is captured `reps` times into a HIP graph on `stream` and replayed; us_out[i] receives
 * the mean microseconds per call, or -1 when the shape is not launchable (e.g. it
 * needs more than 160 KiB of LDS).  x, y, batch as for dec_gemv; the workspace must
 * hold the largest dec_gemv_workspace_size over the candidates.  On return t's
 * launch shape is the fastest candidate.  Host-blocking (synchronises the stream);
 * not itself capturable.  Errors: INVALID_ARG (bad arguments, no launchable
 * candidate or a NULL stream, which cannot be captured), HIP. */
ecw_status dec_tune_launch(ecw_stream stream, ecw_tensor* t, const void* x, int x_dtype, float* y,
                           int batch, void* workspace, size_t workspace_bytes,
                           const uint32_t* shapes, int n_shapes, int reps, float* us_out);

/* Time a grouped launch as tuned: `reps` dec_gemv_group calls with the tensors'
 * current launch shapes are captured into a HIP graph on `stream` (not the NULL
 * stream) and replayed once after a warm-up replay; *us_out = microseconds per call.
 * Arguments otherwise as dec_gemv_group.  Host-blocking.  Errors: INVALID_ARG, HIP,
 * and whatever dec_gemv_group returns for the group. */
ecw_status dec_time_group(ecw_stream stream, const ecw_tensor* const* t, int n, const void* x, int x_dtype,
                          float* const* y, int batch, void* workspace, size_t workspace_bytes, int reps,
                          float* us_out);

/* Roofline probes (measurement hooks; asynchronous on `stream`, time them with events).
 * ecw_probe_stream_read: reads `bytes` (multiple of 16, 16-byte aligned) of device
 *   memory `buf` once with `blocks` blocks of 256 threads (grid-stride, 16-byte loads)
 *   and writes one word per thread to `sink` (device, blocks x 256 u32): the
 *   achievable HBM streaming-read rate the decode is compared against.
 * ecw_probe_lds_lookup: every lane of `blocks` blocks of `waves_per_block` waves runs
 *   `steps` dependent lookups into an LDS table of 2^log2_m entries of entry_bytes
 *   (4, 8, 12 or 16; at most 160 KiB) bytes, the access pattern of the decode's table
 *   reads; writes one word
 *   per thread to `sink` (device, blocks x waves x 64 u32).
 * Errors: INVALID_ARG, HIP. */
ecw_status ecw_probe_stream_read(ecw_stream stream, const void* buf, size_t bytes, uint32_t* sink,
                                 uint32_t blocks);
ecw_status ecw_probe_lds_lookup(ecw_stream stream, uint32_t log2_m, uint32_t entry_bytes, uint32_t steps,
                                uint32_t blocks, uint32_t waves_per_block, uint32_t* sink);
/* ecw_probe_tile_stream: `waves` waves, `waves_per_block` per block, each read their
 *   own contiguous kib_per_wave KiB of `buf` (16-byte aligned; bytes must cover
 *   waves x kib_per_wave KiB) as 1 KiB wave-wide loads (16 bytes per lane) with
 *   `inflight` (1, 2 or 4) loads in flight, in the decode's block order: the read
 *   pattern of the decode's word and raw-byte planes, one stream per tile.  Writes
 *   one word per lane to `sink` (device, waves x 64 u32). */
ecw_status ecw_probe_tile_stream(ecw_stream stream, const void* buf, size_t bytes, uint32_t kib_per_wave,
                                 uint32_t waves, uint32_t waves_per_block, uint32_t inflight, uint32_t* sink);
/* ecw_probe_clock: `blocks` one-wave blocks each keep a dependent FMA chain busy for
 *   duration_us (by the constant-rate real-time counter, whose rate in kHz goes to
 *   *wall_clock_khz) and write [shader-clock cycles, real-time ticks] elapsed, two u64
 *   per block, to `sink` (device).  cycles / ticks * rate = the shader clock; launched
 *   on a second stream beside a kernel, the clock that kernel runs at (the issue peak
 *   of the VALU roofline is priced at it). */
ecw_status ecw_probe_clock(ecw_stream stream, uint32_t duration_us, uint32_t blocks, uint64_t* sink,
                           uint32_t* wall_clock_khz);

/* Test hook: the same decode core, writing what dec_gemv keeps in registers, so the
 * GPU decode can be held to the parity levels of the quantized-artifacts page
 * (section 0x09B "Pack/Unpack Parity": decoded codes equal the stored codes
 * elementwise; 0x09C "Reference Reconstruction": reconstruction against a slow,
 * explicit decoder) and to the rANS end-of-tile invariant (EntroPack page, Section
 * C.3: each tile ends on its final boundary offset).
 *   symbols: nullable device uint16 [rows][symbols per row] (symbol indices; INT
 *          quads: the index of the stored tuple the symbol codes);
 *   w_out: nullable device [rows][cols] in the logical dtype (INT int8 codes, BF16
 *          uint16 bits, FP8 uint8 bytes, E8 int8 2v or uint8 e4m3 per recon_dtype),
 *          escaped weights (BF16 pairs, INT quads) restored from the correction
 *          streams;
 *   tile_status: nullable device uint32 [n_tiles], 0 when the tile ended with every
 *          active state back at 2^16 and exactly its words read, else nonzero.
 * Errors: INVALID_ARG, UNSUPPORTED, HIP. */
ecw_status dec_materialize(ecw_stream stream, const ecw_tensor* t, uint16_t* symbols,
                           void* w_out, uint32_t* tile_status);

/* Dequantising decode for products with more than four activation rows (prefill):
 * the weights are decoded once into a dense matrix that a library GEMM then reads
 * (MINE page, Section 4.2: the dequant kernel that materialises a layer; EntroPack
 * page, Section 3.7).  Writes the real weight values W_val [rows][cols], row-major,
 * rounded to nearest even into out_dtype (ECW_DT_F16 or ECW_DT_BF16): INT code *
 * row scale, BF16 the bf16 value (escaped weights included), FP8 the E4M3 value *
 * row scale, E8 v * row scale (INT8 route) or e4m3(v) * row scale (FP8 route); every
 * such value is exact in fp32 before the rounding.
 *   w_out: device, rows x cols x 2 bytes, 16-byte aligned (caller-owned).
 * Asynchronous on `stream`, stores are row-contiguous 64-byte segments.
 * Errors: INVALID_ARG (bad tensor, dtype or buffer), UNSUPPORTED (cols not a
 * multiple of 8, tables too large for LDS), HIP. */
ecw_status dec_dequantize(ecw_stream stream, const ecw_tensor* t, void* w_out, int out_dtype);

const char* ecw_last_error(void);
uint32_t ecw_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* ECW_H */
