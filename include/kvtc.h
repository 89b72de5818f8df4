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
 *    workspaces are passed in, sized by the *_size queries.
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
 *  chunk_tokens     tokens of a section sharing one frequency table
 *  tile_tokens      tokens per packed tile = one rANS stream; divides
 *                   chunk_tokens
 *  basis_per_head   0: basis [L,2,D,D]; 1: [L,2,H,D,D]
 *  wht_keys         WHT path: 1 = keys are normalised and transformed too,
 *                   0 = keys are quantised directly
 *  max_tokens       largest T any call on the plan may use (sizes the RoPE
 *                   table)
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
 * (device, `cap` bytes).  k, v: device [L,H,T,D] in the cache dtype.  ws:
 * device workspace of ws_bytes >= kvtc_workspace_size().  Asynchronous; the
 * container size and the device status (OK, NONFINITE, CAPACITY) are read
 * with kvtc_result() after the stream has been synchronised.  The container
 * is deterministic: the same inputs give the same bytes. */
kvtc_status kvtc_encode(kvtc_plan_t plan, const void* k, const void* v, int32_t T, void* out,
                        size_t cap, void* ws, size_t ws_bytes, hipStream_t stream);

/* Decode a container of T tokens (the T it was encoded with; the header is
 * checked against it on the device) from `in` (device, in_bytes) into k_out,
 * v_out (device [L,H,T,D] in out_dtype, KVTC_BF16 or KVTC_FP32: RNE cast).
 * Sink and recent windows are restored bit-exactly (converted when out_dtype
 * differs from the cache dtype).  Asynchronous; a corrupt container sets
 * KVTC_ERR_CORRUPT in the workspace status and leaves the outputs undefined. */
kvtc_status kvtc_decode(kvtc_plan_t plan, const void* in, size_t in_bytes, int32_t T,
                        void* k_out, void* v_out, int32_t out_dtype, void* ws, size_t ws_bytes,
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

/* One interleaved rANS stream with the device coder: encode N bytes `sym`
 * with table `freq` (u16[256], sums to 2^scale_bits) into states u32[lanes]
 * and words u16[words_cap] (emission order), word count to *nwords (device
 * int64).  All pointers are device memory.  N must be below 2^30
 * (KVTC_ERR_INVALID_ARG otherwise); a words_cap above 2^30 acts as 2^30. */
kvtc_status kvtc_test_rans_encode(const uint8_t* sym, int64_t N, const uint16_t* freq,
                                  int32_t scale_bits, int32_t lanes, uint32_t* states,
                                  uint16_t* words, int64_t words_cap, int64_t* nwords,
                                  hipStream_t stream);

/* Decode one stream; status (device int32) gets KVTC_OK or KVTC_ERR_CORRUPT. */
kvtc_status kvtc_test_rans_decode(const uint32_t* states, const uint16_t* words,
                                  int64_t nwords, const uint16_t* freq, int32_t scale_bits,
                                  int32_t lanes, int64_t N, uint8_t* sym, int32_t* status,
                                  hipStream_t stream);

/* Frequency table of a byte histogram with the device normaliser:
 * counts u32[256] -> freq u16[256] (device). */
kvtc_status kvtc_test_freq_table(const uint32_t* counts, int32_t scale_bits, uint16_t* freq,
                                 hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* KVTC_H */
