/*
 * libkvtc -- KVTC-style transform coding of transformer KV caches on AMD
 * Instinct MI355X (gfx950), behind a plain C ABI.
 *
 * The method (cited by page title and section):
 *  - "KVTC: The Open-Source KV Cache Codec That Treats LLM Memory Like Media",
 *    "How the Pipeline Works": the cache is split into sink tokens, a
 *    compressed middle and a recent window; the middle goes through RoPE undo
 *    -> PCA transform -> bit allocation -> quantization -> entropy coding, and
 *    each section carries scales, zero points and bit widths
 *    (CompressedSection).  "Bit Budget Is Not Fair": uneven allocation.
 *    "rANS Makes the Last Mile Smaller": rANS over the quantised data.
 *  - "Codec-Gauge: Learning Compression-Friendly Gauges for Transformer KV
 *    Caches", "Problem Statement and Overview": K_l, V_l in R^{B x H x T x d},
 *    the frame Z = G X, B_c = C(Z), Z^ = D(B_c), X^ = G^-1 Z^; "Compression
 *    Conditions": PCA/KLT as the uncentered second-moment eigenbasis and the
 *    Hadamard control.
 *  - "TTAS-X2: Extreme KV Cache Compression for Large Language Models", 2.1
 *    (K: 4-bit scalar, per-head scale) and 2.2 (V: per-vector RMS
 *    normalisation, Hadamard transform): the WHT path.
 *
 * Conventions for every entry point:
 *  - Tensors are contiguous [layers, kv_heads, tokens, head_dim] in the cache
 *    dtype (bf16 or fp32), little-endian, in device memory.
 *  - Every device pointer passed to encode or decode must be 16-byte aligned
 *    (allocations from hipMalloc or PyTorch are); otherwise the call returns
 *    KVTC_ERR_INVALID_ARG.
 *  - The caller owns every buffer (device memory from any allocator, e.g.
 *    PyTorch).  The library never allocates device memory: plan memory and
 *    workspaces are passed in, sized by the *_size queries.  The one
 *    exception is the fixed per-device array of kvtc_decode_noalloc.
 *  - Calls return a kvtc_status; no exception crosses the ABI.  Argument
 *    errors are reported synchronously and nothing is enqueued.  Errors found
 *    on the device (corrupt container, non-finite input, capacity) are
 *    written to a status word inside the workspace; read it with
 *    kvtc_result() after synchronising the stream.
 *  - Encode and decode are asynchronous on the caller's stream and never
 *    synchronise with the host.
 *  - A plan is immutable after kvtc_plan() and may be shared by concurrent
 *    calls on different streams; each concurrent call needs its own
 *    workspace.
 */
#ifndef KVTC_H
#define KVTC_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVTC_OK = 0,
  KVTC_ERR_INVALID_ARG = 1, /* bad pointer, size or configuration value */
  KVTC_ERR_UNSUPPORTED = 2, /* valid configuration this build does not run */
  KVTC_ERR_CAPACITY = 3,    /* output or workspace too small */
  KVTC_ERR_CORRUPT = 4,     /* container fails a header, table or stream check */
  KVTC_ERR_NONFINITE = 5,   /* NaN or Inf in the coded middle region */
  KVTC_ERR_HIP = 6          /* a HIP runtime call failed */
} kvtc_status;

enum { KVTC_FP32 = 0, KVTC_BF16 = 1 };
enum { KVTC_PCA = 0, KVTC_WHT = 1 };
enum { KVTC_ROPE_HALF = 0, KVTC_ROPE_INTERLEAVED = 1 };

/* Codec configuration.  It is echoed into every container header, and a
 * decoder accepts only containers written under an identical configuration.
 *
 *  layers, kv_heads, head_dim  cache shape; head_dim 64 or 128
 *  dtype            KVTC_BF16 / KVTC_FP32: cache dtype and operand precision
 *                   of the projection (basis and un-rotated keys are rounded
 *                   to it before the contraction)
 *  transform        KVTC_PCA: supplied orthogonal basis per layer and K/V
 *                   (per head with basis_per_head); KVTC_WHT: per-token RMS
 *                   normalisation then the orthonormal Walsh-Hadamard
 *                   transform in Sylvester order
 *  sink_tokens, recent_tokens   raw regions at the front and back
 *  bits_k, bits_v   PCA: average bits per component, budget floor(bits*D)
 *                   per token, spread by greedy marginal allocation; WHT:
 *                   floor(bits) bits for every component (keys use one
 *                   symmetric scale per section, values a min/max range per
 *                   component)
 *  max_bits         1..8 bits per component
 *  rope_keys        1: keys carry RoPE and are un-rotated before coding and
 *                   re-rotated after decoding
 *  rope_style       KVTC_ROPE_HALF (pairs j, j+D/2) or KVTC_ROPE_INTERLEAVED
 *  rope_theta       base; the angle of pair j at position t is
 *                   t * theta^(-2j/D) in fp64, cos/sin rounded to fp32
 *  rans_scale_bits  frequency precision, 8..12 (M = 2^bits)
 *  rans_lanes       interleaved rANS states per stream, 16 or 32
 *  chunk_tokens     tokens of a section's chunk: one container record with
 *                   a frequency table per coded component; at most 32
 *                   tiles, and a multiple of 1024 when longer than 1024
 *  tile_tokens      tokens per packed tile = one rANS stream; divides
 *                   chunk_tokens (and 1024 when the chunk is longer)
 *  basis_per_head   0: basis [L,2,D,D]; 1: [L,2,H,D,D]
 *  wht_keys         WHT path: 1 = keys are normalised and transformed too,
 *                   0 = keys are quantised directly
 *  max_tokens       largest T any call on the plan may use (sizes the RoPE
 *                   table)
 *  alloc_scope      PCA path: 0 = each section spends its own budget
 *                   (floor(bits D) bits per token); 1 = one budget, the
 *                   sum of those, over all sections of the cache (of each
 *                   sequence of a paged batch), spent by the same greedy
 *                   marginal rule over every component at once, lowest
 *                   (section, component) first on ties ("KVTC: The
 *                   Open-Source KV Cache Codec That Treats LLM Memory Like
 *                   Media", Bit Budget Is Not Fair, and That Is the Point:
 *                   the budget moves toward the sections that need it).
 *                   Needs n_sections * head_dim <= 2^20.
 */
typedef struct kvtc_config {
  int32_t layers, kv_heads, head_dim;
  int32_t dtype;
  int32_t transform;
  int32_t sink_tokens, recent_tokens;
  float bits_k, bits_v;
  int32_t max_bits;
  int32_t rope_keys;
  int32_t rope_style;
  double rope_theta;
  int32_t rans_scale_bits;
  int32_t rans_lanes;
  int32_t chunk_tokens;
  int32_t tile_tokens;
  int32_t basis_per_head;
  int32_t wht_keys;
  int32_t max_tokens;
  int32_t alloc_scope;
} kvtc_config;

typedef struct kvtc_plan_s* kvtc_plan_t;

/* Human-readable name of a status code (static storage). */
const char* kvtc_status_str(kvtc_status s);

/* Device bytes kvtc_plan() needs for this configuration (basis copies in the
 * operand precision and the RoPE cos/sin table). */
kvtc_status kvtc_plan_mem_size(const kvtc_config* cfg, size_t* bytes);

/* Validate cfg and build a plan ("The Tradeoff Is Real": the PCA basis is a
 * calibrated input).
 *  basis_dev   device fp32 [L,2,D,D] (or [L,2,H,D,D]); column i (stride 1
 *              within a row of D) is component i, components in descending
 *              variance order; NULL for KVTC_WHT.  Read during this call only.
 *  plan_mem    device buffer of plan_mem_bytes >= kvtc_plan_mem_size();
 *              owned by the caller, must outlive the plan.
 *  stream      used for the uploads; the call synchronises it once.
 *  out         receives the plan handle (host object).
 * Errors: INVALID_ARG (config or pointers), UNSUPPORTED, CAPACITY (plan_mem
 * too small), NONFINITE (non-finite basis entry), HIP. */
kvtc_status kvtc_plan(const kvtc_config* cfg, const float* basis_dev, void* plan_mem,
                      size_t plan_mem_bytes, hipStream_t stream, kvtc_plan_t* out);

/* Release the host-side plan object (plan memory stays the caller's). */
kvtc_status kvtc_plan_destroy(kvtc_plan_t plan);

/* 64-bit FNV-1a fingerprint of the operand-precision basis, as stored in
 * container headers. */
kvtc_status kvtc_plan_fingerprint(kvtc_plan_t plan, uint64_t* fp);

/* Workspace bytes for an encode or decode of T tokens, and the worst-case
 * container size (the capacity an encode output needs to be sure to fit). */
kvtc_status kvtc_workspace_size(kvtc_plan_t plan, int32_t T, size_t* ws_bytes,
                                size_t* max_container_bytes);

/* Encode one cache of T tokens (T <= max_tokens) into a container at `out`
 * (device, `cap` bytes): the steps of "KVTC: The Open-Source KV Cache Codec
 * That Treats LLM Memory Like Media", How the Pipeline Works (regions, RoPE
 * undo, PCA or Hadamard transform, bit allocation, quantisation, entropy
 * coding), each section carrying its widths, zero points and scales as in
 * its CompressedSection.  k, v: device [L,H,T,D] in the cache dtype.  ws:
 * device workspace of ws_bytes >= kvtc_workspace_size().  Asynchronous; the
 * container size and the device status (OK, NONFINITE, CAPACITY) are read
 * with kvtc_result() after the stream has been synchronised.  The container
 * is deterministic: the same inputs give the same bytes.
 *
 * Container (version 3, little-endian): a 256-byte header (config echo, T,
 * region offsets, total bytes, basis fingerprint, and at bytes 200..215 the
 * checksum of everything before the records); per section u8 widths[D],
 * f32 zero[D], f32 scale[D] (and per-token RMS on the Hadamard path); the
 * raw sink and recent windows; a directory of 32-byte entries (u64 offset,
 * u32 size, u32 mode, u64 x 2 checksum of the record); the chunk records.
 * Checksums ("Quantum-Aware Tensor Compression", QATC transport: an
 * aggregate checksum over bounded chunks) are A = sum w_j and
 * B = sum (j + 1) w_j modulo 2^61 - 1 over the range's 32-bit words, the
 * header's own field counting as zero. */
kvtc_status kvtc_encode(kvtc_plan_t plan, const void* k, const void* v, int32_t T, void* out,
                        size_t cap, void* ws, size_t ws_bytes, hipStream_t stream);

/* Decode a container of T tokens (the T it was encoded with; the header is
 * checked against it on the device) from `in` (device, in_bytes) into k_out,
 * v_out (device [L,H,T,D] in out_dtype, KVTC_BF16 or KVTC_FP32: RNE cast):
 * the inverse steps of the same pipeline (entropy decode, dequantise,
 * inverse transform, RoPE re-applied), which "returns the same native tensor
 * bytes" for the raw windows ("Compress the most expensive bytes in AI", KV
 * & tensor mode).  Sink and recent windows are restored bit-exactly
 * (converted when out_dtype differs from the cache dtype).  The header, the
 * checksum of the fixed part and every record's checksum are verified; a
 * damaged or truncated container (QATC: rejected before restore) sets
 * KVTC_ERR_CORRUPT in the workspace status and leaves the outputs
 * undefined.  Asynchronous. */
kvtc_status kvtc_decode(kvtc_plan_t plan, const void* in, size_t in_bytes, int32_t T,
                        void* k_out, void* v_out, int32_t out_dtype, void* ws, size_t ws_bytes,
                        hipStream_t stream);

/* ---- decode without allocation ----------------------------------------- */

/* Bytes of the fixed device array kvtc_decode_noalloc works in. */
#define KVTC_NOALLOC_SCRATCH_BYTES ((int64_t)128 << 20)

/* For callers that cannot allocate device memory or hand in a workspace:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  kvtc_decode with its workspace replaced by a fixed array inside
 * the library: KVTC_NOALLOC_SCRATCH_BYTES of device memory per device, held
 * from the code object's load on that device until the process ends.  The
 * decoder needs a 256-aligned status block of 8448 bytes, 16 KiB of
 * partial checksums and its packed tiles there (about 71 MB for 32 layers x 8 KV heads x 4096 tokens x
 * head_dim 128 at 2 bits per component); a call that needs more returns
 * KVTC_ERR_CAPACITY and enqueues nothing.  The call allocates nothing:
 * no hipMalloc, hipFree, event or library allocation.
 *
 * Arguments, outputs and device checks are those of kvtc_decode.  When
 * status_dev (device, 4-byte aligned) is not NULL, the decode's status word
 * is copied there after the last kernel: 0, or bit KVTC_ERR_CORRUPT set for a
 * damaged container.
 *
 * Every call on a device works in that device's one array, which keeps the
 * last call's contents (each call clears what it reads back).  Calls that
 * overlap in time on one device -- different streams or host threads --
 * race: the caller serialises them (one stream does). */
kvtc_status kvtc_decode_noalloc(kvtc_plan_t plan, const void* in, size_t in_bytes, int32_t T,
                                void* k_out, void* v_out, int32_t out_dtype, uint32_t* status_dev,
                                hipStream_t stream);

/* ---- paged ragged batches ---------------------------------------------- */

/* A batch of n_seqs independent sequences whose K and V live in page pools
 * [layers, pool_pages, kv_heads, 16, head_dim] (cache dtype): token t of
 * sequence z is row t % 16 of page page_table[z * max_pages + t / 16].  Each
 * sequence is coded on its own, exactly as kvtc_encode codes a contiguous
 * cache of its length (regions, sections and chunks are per sequence, as in
 * "KVTC: The Open-Source KV Cache Codec That Treats LLM Memory Like Media",
 * "How the Pipeline Works"); the batch container holds the sequence
 * containers in order:
 *   bytes 0..63: "KVTB", u32 version 1, u32 n_seqs, u32 header bytes,
 *                u64 total bytes, zeros;
 *   then per sequence u64 offset, u64 size of its container;
 *   sequence containers start 256-byte aligned, gaps are zero.
 * Every phase is one launch over the whole batch.  Supported for the bf16,
 * head_dim 128, PCA configurations with tile_tokens % 64 == 0 (otherwise
 * KVTC_ERR_UNSUPPORTED).
 *
 * seq_lens_host and seq_lens_dev hold the same n_seqs lengths (host copy for
 * sizing the launches, device copy for the kernels); page_table and
 * seq_lens_dev are device int32 arrays (4-byte aligned).  The device checks
 * the lengths against the host's (sum and maximum) and every page index
 * against pool_pages; a mismatch sets KVTC_ERR_INVALID_ARG in the status and
 * codes nothing.  Page pools must not overlap the container or workspace. */

/* Workspace and worst-case container bytes of a batch. */
kvtc_status kvtc_workspace_size_paged(kvtc_plan_t plan, int32_t n_seqs, const int32_t* seq_lens_host,
                                      size_t* ws_bytes, size_t* max_container_bytes);

/* Encode a paged batch into `out` (device, cap bytes).  Asynchronous; read
 * the total size and status with kvtc_result(). */
kvtc_status kvtc_encode_paged(kvtc_plan_t plan, const void* k_pool, const void* v_pool, int32_t pool_pages,
                              const int32_t* page_table, int32_t max_pages, const int32_t* seq_lens_dev,
                              const int32_t* seq_lens_host, int32_t n_seqs, void* out, size_t cap, void* ws,
                              size_t ws_bytes, hipStream_t stream);

/* Decode a batch container into the pages of k_pool and v_pool (cache dtype)
 * named by the page table; only the pages of the sequences' tokens are
 * written.  Asynchronous; a damaged container sets KVTC_ERR_CORRUPT. */
kvtc_status kvtc_decode_paged(kvtc_plan_t plan, const void* in, size_t in_bytes, void* k_pool, void* v_pool,
                              int32_t pool_pages, const int32_t* page_table, int32_t max_pages,
                              const int32_t* seq_lens_dev, const int32_t* seq_lens_host, int32_t n_seqs, void* ws,
                              size_t ws_bytes, hipStream_t stream);

/* After synchronising the stream of the last encode/decode that used ws:
 * the container size of that encode (0 after a decode) and the status the
 * device recorded.  Blocking device-to-host copy of 16 bytes. */
kvtc_status kvtc_result(kvtc_plan_t plan, const void* ws, uint64_t* container_bytes,
                        int32_t* device_status);

/* After synchronising the stream of the last encode that used ws: how many
 * quantisation codes that encode re-computed exactly because the MFMA
 * coefficient lay within its error bound of a rounding boundary. */
kvtc_status kvtc_encode_counters(kvtc_plan_t plan, const void* ws, uint64_t* exact_recomputed);

/* ---- profiling -------------------------------------------------------- */

/* When on, kvtc_encode and kvtc_decode record a HIP event on the caller's
 * stream before their first kernel and after each phase (one phase = one
 * kernel launch of the path, except "copy_raw", "assemble" and
 * "dec_check", which also clear or set the status word).  Events are created
 * on first use.  A plan is then no longer safe to share between concurrent
 * calls. */
kvtc_status kvtc_profile_enable(kvtc_plan_t plan, int32_t on);

/* Per-phase milliseconds of the last profiled encode or decode on this plan,
 * in launch order: up to max_n entries into ms[] and names[] (static
 * strings), the count to *n.  Synchronises on the last event. */
kvtc_status kvtc_profile_read(kvtc_plan_t plan, int32_t max_n, float* ms, const char** names,
                              int32_t* n);

/* ---- stage entry points for parity tests (same kernels as the path) ---- */

/* Per-section statistics left in ws by the last kvtc_encode: host arrays of
 * n_sections*D floats each (mean, variance, min, max of the coefficients). */
kvtc_status kvtc_test_section_stats(kvtc_plan_t plan, const void* ws, int32_t T, float* mu,
                                    float* var, float* cmin, float* cmax);

/* Encoder coefficients of sections [sec_begin, sec_end) of a cache: device
 * fp32 out [n, T_mid, D]; r_out device fp32 [n, T_mid] (WHT path) or NULL. */
kvtc_status kvtc_test_coeffs(kvtc_plan_t plan, const void* k, const void* v, int32_t T,
                             int32_t sec_begin, int32_t sec_end, float* out, float* r_out,
                             hipStream_t stream);

/* Frequency tables with the record encoder's normaliser ("KVTC: The
 * Open-Source KV Cache Codec That Treats LLM Memory Like Media", rANS Makes
 * the Last Mile Smaller): n tables, counts u32 [n][16] with alphabet[i]
 * (1..16) meaningful entries each -> freq u16 [n][16] summing to
 * 2^scale_bits (entries past the alphabet are 0).  Present symbols get
 * max(1, round-half-up(count M / N)); a shortfall goes to the most frequent
 * symbol, an excess is taken one unit at a time from the largest frequency
 * above 1 (lowest symbol on ties).  All pointers are device memory. */
kvtc_status kvtc_test_freq_tables(const uint32_t* counts, const int32_t* alphabet, int32_t n,
                                  int32_t scale_bits, uint16_t* freq, hipStream_t stream);

/* The packed tiles of one section as the last kvtc_encode (or kvtc_decode)
 * that used ws left them in the workspace: *blocks work blocks of
 * *slot_bytes bytes each (the tiles of a block back to back, each tile the
 * channel-major rows of its codes, "Compress the most expensive bytes in
 * AI", KV & tensor mode).  With out = NULL only the sizes are returned;
 * otherwise out (device, out_bytes >= blocks * slot_bytes) receives them
 * (asynchronous on `stream`). */
kvtc_status kvtc_test_packed_tiles(kvtc_plan_t plan, const void* ws, int32_t T, int32_t section,
                                   void* out, size_t out_bytes, int32_t* blocks, size_t* slot_bytes,
                                   hipStream_t stream);

/* Stage hook, RoPE undo ("KVTC: The Open-Source KV Cache Codec That Treats
 * LLM Memory Like Media", Why RoPE Has to Be Reversed First): the middle
 * keys of k (device [L,H,T,D] bf16) with the rotation removed and rounded to
 * bf16, as the encoder's first pass computes them, into out (device,
 * [L,H,T_mid,D] bf16, out_bytes >= L H T_mid D 2).  ws: a workspace of
 * kvtc_workspace_size() bytes.  Only the bf16 head_dim-128 PCA path with
 * RoPE keys runs this as a pass of its own (elsewhere it is fused):
 * KVTC_ERR_UNSUPPORTED otherwise. */
kvtc_status kvtc_test_rope(kvtc_plan_t plan, const void* k, int32_t T, void* ws, size_t ws_bytes, void* out,
                           size_t out_bytes, hipStream_t stream);

/* Stage hook, bit allocation and side information (same page, Bit Budget Is
 * Not Fair; How the Pipeline Works: widths, scales and zero points per
 * section): from per-component statistics stats (host, [n_sections][D][4]
 * f32: mean, variance, min, max) to the section records written to side_out
 * (device, >= n_sections 9 D bytes: u8 widths[D], f32 zero[D], f32
 * scale[D] per section) by the allocation kernels of the plan's scope.  ws:
 * a workspace of kvtc_workspace_size(T) bytes (T fixes T_mid, which decides
 * the empty-middle case). */
kvtc_status kvtc_test_alloc(kvtc_plan_t plan, int32_t T, const float* stats, void* ws, size_t ws_bytes,
                            void* side_out, size_t side_bytes, hipStream_t stream);

/* Stage hook, the encoder up to quantisation and packing (same page, How the
 * Pipeline Works: RoPE undo -> transform -> bit allocation -> quantization):
 * the encode passes before entropy coding.  The section records go to out
 * (device, cap >= the raw-window offset of the layout) at their container
 * offsets, the packed tiles stay in ws (read them with
 * kvtc_test_packed_tiles). */
kvtc_status kvtc_test_quant_pack(kvtc_plan_t plan, const void* k, const void* v, int32_t T, void* out, size_t cap,
                                 void* ws, size_t ws_bytes, hipStream_t stream);

/* Stage hook, dequantisation and inverse projection ("Codec-Gauge", Problem
 * Statement and Overview: Z^ = D(B_c), X^ = G^-1 Z^; RoPE re-applied to
 * keys): the decode transform alone, from the packed tiles in ws (as
 * kvtc_test_quant_pack or a record decode left them) and the section records
 * of in (device, in_bytes >= the raw-window offset) into the middle rows of
 * k_out, v_out (device [L,H,T,D] in out_dtype); other rows are untouched. */
kvtc_status kvtc_test_dequant_project(kvtc_plan_t plan, const void* in, size_t in_bytes, int32_t T, void* ws,
                                      size_t ws_bytes, void* k_out, void* v_out, int32_t out_dtype,
                                      hipStream_t stream);

/* ---- scalar quantisers on gauge coordinates ------------------------------ */

/* "Codec-Gauge: Learning Compression-Friendly Gauges for Transformer KV
 * Caches", Compression Conditions: the gauge coordinates Z = G X also feed
 * two scalar quantisers with one bit setting per cache type.  The plan's
 * basis is the gauge (component i is column i of B = G^T: a grouped
 * block-diagonal gauge, PCA/KLT or the identity); the plan's transform must
 * be KVTC_PCA.  Every token of [0, T) is coded (no raw windows); keys are
 * un-rotated first when the plan's keys carry RoPE.
 *
 *  KVTC_SQ_BLOCK  block-uniform: one range per block of `tile` tokens x
 *                 `group` channels, keys and values alike (group = head_dim
 *                 gives one range per T_b x d_l block)
 *  KVTC_SQ_KIVI   KIVI-style: keys one range per channel over `tile`
 *                 tokens, values one range per token over `group` channels
 *
 * A range over coefficients c has zero = min c and scale = (max c - min c) /
 * (2^b - 1) (fp64, rounded once to fp32); rcp = 1 / scale in fp32, or 0 when
 * scale is 0 or the reciprocal overflows.  A code is
 * clamp(rint((c - zero) * rcp), 0, 2^b - 1) in fp32; decoding takes
 * fma(code, scale, zero) rounded to bf16, applies X = B c and re-applies
 * RoPE.  The coefficients come from bf16 MFMA products with fp32
 * accumulation; a code whose pre-rounding value lies within the
 * accumulation error of a rounding boundary is re-computed from the exact
 * coefficient.
 *
 * Layout, sections u = (l 2 + s) H + h in order (s 0 keys, 1 values):
 *  codes   per section T head_dim b_s / 8 bytes: token-major rows of
 *          head_dim b_s bits, channel i at bits [i b, i b + b) of its row,
 *          least significant bit first;
 *  ranges  per section ceil(T / te) (head_dim / ce) fp32 (zero, scale)
 *          pairs, index (t / te) (head_dim / ce) + i / ce, where (te, ce) is
 *          (tile, group) for block-uniform, (tile, 1) for KIVI keys and
 *          (1, group) for KIVI values.
 *
 * Supported: bf16 head_dim-128 plans with tile dividing 64 (otherwise
 * KVTC_ERR_UNSUPPORTED).  group must divide head_dim, tile >= 1, bits 1..8
 * (otherwise KVTC_ERR_INVALID_ARG). */
enum { KVTC_SQ_BLOCK = 1, KVTC_SQ_KIVI = 2 };

typedef struct kvtc_sq_config {
  int32_t kind;    /* KVTC_SQ_BLOCK or KVTC_SQ_KIVI */
  int32_t group;   /* channels per range (see above) */
  int32_t tile;    /* tokens per range, T_b (see above) */
  int32_t bits_k;  /* bits per key coefficient, 1..8 */
  int32_t bits_v;  /* bits per value coefficient, 1..8 */
} kvtc_sq_config;

/* Code bytes and (zero, scale) pairs of a call over T tokens (host only). */
kvtc_status kvtc_sq_sizes(kvtc_plan_t plan, const kvtc_sq_config* q, int32_t T, size_t* code_bytes,
                          size_t* range_pairs);

/* Quantise k, v (device [L,H,T,D] bf16) into codes (device, code_cap bytes)
 * and ranges (device, range_cap pairs of fp32), laid out as above.  When
 * status_dev (device, 4-byte aligned) is not NULL it is cleared and then
 * gets bit KVTC_ERR_NONFINITE if a coefficient is NaN or infinite (codes
 * and ranges are then undefined).  Asynchronous on `stream`. */
kvtc_status kvtc_sq_encode(kvtc_plan_t plan, const kvtc_sq_config* q, const void* k, const void* v, int32_t T,
                           void* codes, size_t code_cap, float* ranges, size_t range_cap, uint32_t* status_dev,
                           hipStream_t stream);

/* Reconstruct k_out, v_out (device [L,H,T,D] in out_dtype, KVTC_BF16 or
 * KVTC_FP32 with a round-to-nearest-even cast) from codes (code_bytes) and
 * ranges (range_pairs) written by kvtc_sq_encode under the same plan, sq
 * configuration and T.  Asynchronous on `stream`. */
kvtc_status kvtc_sq_decode(kvtc_plan_t plan, const kvtc_sq_config* q, const void* codes, size_t code_bytes,
                           const float* ranges, size_t range_pairs, int32_t T, void* k_out, void* v_out,
                           int32_t out_dtype, hipStream_t stream);

/* ---- TTAS-X2 value path: two-level product quantisation ------------------ */

/* "TTAS-X2: Extreme KV Cache Compression for Large Language Models", 2.2 V
 * Compression: every value vector x (value sections only) is RMS-normalised,
 * r = sqrt(sum x^2 / D), and Hadamard-transformed, y = WHT(x / r) (the
 * orthonormal Sylvester transform); y is split into D / sub_dim subvectors,
 * each coded by two-level product quantisation -- the nearest of k1
 * centroids, then the nearest of k2 centroids to the fp32 residual -- and
 * per (layer, head) and block of block_tokens tokens the `outliers`
 * coefficients with the largest |y - y^| (then the lowest index) are kept
 * exactly; 3 Experiments: K1 = 256, K2 = 64..512, 32..256 outliers per
 * head.  The keys' 4-bit scalar path of 2.1 is kvtc_encode with the WHT
 * transform and wht_keys = 0.
 *
 * Definitions: r in fp64 rounded to fp32; the transform in fp64, rounded
 * once; centroids are held in bf16 (the given fp32 codebooks are rounded to
 * nearest even); the nearest centroid minimises sum_j (y_j - c_j)^2 in fp64
 * summed in channel order, lowest index on ties; y^ = c1 + c2 in fp32;
 * decoding puts the outliers back into y^ and returns WHT(y^) r.  The
 * encoder's scores come from bf16 MFMA products of y split into two bf16
 * parts; a choice whose two best scores lie within their error bound is
 * re-decided by the exact distances, so the indices are the exact ones.
 *
 * Codebooks (device, fp32, 16-byte aligned, owned by the caller): cb1
 * [L][D / sub_dim][k1][sub_dim], cb2 [L][D / sub_dim][k2][sub_dim], per
 * layer and subspace (shared by the layer's heads).
 *
 * Layout, value sections (l, h) = l H + h in order:
 *  codes     [L H][T][row_words] u32: per token the level-1 indices of
 *            log2(k1) bits, then the level-2 indices of log2(k2) bits, in
 *            subspace order, least significant bit first, zero-padded;
 *  rms       [L H][T] fp32;
 *  outliers  [L H][blocks][outliers] slots of two u32: index t D + j within
 *            the section (t the token, j the channel) and the fp32 bits of
 *            y; index-ascending within a block, unused slots
 *            (0xFFFFFFFF, 0); blocks = ceil(T / block_tokens).
 *
 * Supported: bf16 head_dim-128 plans with sub_dim 8, k1 and k2 in
 * {32, ..., 512}, outliers <= 256, block_tokens a multiple of 64 with
 * (block_tokens / 64) outliers <= 4096 (otherwise KVTC_ERR_UNSUPPORTED).
 * sub_dim must divide head_dim, k1 and k2 be powers of two in [2, 512],
 * outliers >= 0 and block_tokens >= 1 (otherwise KVTC_ERR_INVALID_ARG). */
typedef struct kvtc_pq_config {
  int32_t sub_dim;       /* channels per subvector */
  int32_t k1, k2;        /* centroids per subspace, levels 1 and 2 */
  int32_t outliers;      /* budget per (layer, head) and block */
  int32_t block_tokens;  /* tokens per outlier block */
} kvtc_pq_config;

/* Bytes of codes, outlier slots and workspace bytes of a call over T tokens
 * (host only).  rms holds L H T floats. */
kvtc_status kvtc_pq_sizes(kvtc_plan_t plan, const kvtc_pq_config* q, int32_t T, size_t* code_bytes,
                          size_t* outlier_slots, size_t* ws_bytes);

/* Encode the values v (device [L,H,T,D] bf16) into codes (code_cap bytes),
 * rms (rms_cap floats) and outliers (outlier_cap slots), all device.  ws:
 * device workspace of kvtc_pq_sizes() bytes.  When status_dev (device,
 * 4-byte aligned) is not NULL it is cleared and then gets bit
 * KVTC_ERR_NONFINITE for a NaN or infinite value (the outputs are then
 * undefined).  Asynchronous on `stream`. */
kvtc_status kvtc_pq_encode(kvtc_plan_t plan, const kvtc_pq_config* q, const float* cb1, const float* cb2,
                           const void* v, int32_t T, uint32_t* codes, size_t code_cap, float* rms, size_t rms_cap,
                           uint32_t* outliers, size_t outlier_cap, void* ws, size_t ws_bytes, uint32_t* status_dev,
                           hipStream_t stream);

/* Reconstruct the values into v_out (device [L,H,T,D] in out_dtype,
 * KVTC_BF16 or KVTC_FP32) from what kvtc_pq_encode wrote under the same
 * plan, configuration, codebooks and T.  An outlier index outside its block
 * sets bit KVTC_ERR_CORRUPT in status_dev (cleared first; may be NULL) and
 * is ignored.  Asynchronous on `stream`. */
kvtc_status kvtc_pq_decode(kvtc_plan_t plan, const kvtc_pq_config* q, const float* cb1, const float* cb2,
                           const uint32_t* codes, size_t code_bytes, const float* rms, const uint32_t* outliers,
                           size_t outlier_slots, int32_t T, void* v_out, int32_t out_dtype, void* ws, size_t ws_bytes,
                           uint32_t* status_dev, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* KVTC_H */
