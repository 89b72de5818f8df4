/*
 * KVTC reference oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, single-threaded C implementation of KVTC-style transform
 * coding of transformer KV caches.  It exists to check the HIP library and
 * nothing else: only the tests, the smoke entry point and the benchmark's
 * CPU-baseline leg may load it.  It shares no code, header, table or
 * constant generator with the HIP library under tensor_compression_amd/.
 *
 * Sources (cited by page title and section):
 *  [KVTC]  "KVTC: The Open-Source KV Cache Codec That Treats LLM Memory Like
 *          Media" (repo explainer of OnlyTerp/kvtc): sections "How the
 *          Pipeline Works", "Why RoPE Has to Be Reversed First", "Bit Budget
 *          Is Not Fair, and That Is the Point", "rANS Makes the Last Mile
 *          Smaller", "The Tradeoff Is Real".
 *  [CG]    "Codec-Gauge: Learning Compression-Friendly Gauges for Transformer
 *          KV Caches": "Problem Statement and Overview" (cache notation, the
 *          Z=GX / C / D / G^-1 frame), "Compression Conditions" (uncentered
 *          second-moment PCA/KLT, Hadamard control, KIVI-style ranges),
 *          "Evaluation Design" (NRMSE, measured bits/value, sanity rows).
 *  [TTAS]  "TTAS-X2: Extreme KV Cache Compression for Large Language Models":
 *          2.1 K Compression (4-bit scalar, per-head scale), 2.2 V Compression
 *          (per-vector RMS normalisation, Hadamard transform), 4 Memory
 *          Analysis.
 *  [AT1]   "Compress the most expensive bytes in AI" (AT-1 Memory), "KV &
 *          tensor mode": token-major to channel-major reordering.
 *
 * Where the pages leave a step open, the oracle follows one stated reading;
 * every reading is listed in the design notes of the repository.
 */
#ifndef KVTC_ORACLE_H
#define KVTC_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_FP32 = 0, ORC_BF16 = 1 };
enum { ORC_PCA = 0, ORC_WHT = 1 };
enum { ORC_ROPE_HALF = 0, ORC_ROPE_INTERLEAVED = 1 };

enum {
  ORC_OK = 0,
  ORC_ERR_INVALID_ARG = 1,
  ORC_ERR_UNSUPPORTED = 2,
  ORC_ERR_CAPACITY = 3,
  ORC_ERR_CORRUPT = 4,
  ORC_ERR_NONFINITE = 5
};

typedef struct {
  int32_t layers, kv_heads, head_dim;
  int32_t dtype;          /* ORC_FP32 / ORC_BF16: cache dtype = operand precision */
  int32_t transform;      /* ORC_PCA / ORC_WHT */
  int32_t sink_tokens, recent_tokens;
  float bits_k, bits_v;   /* average bits per component */
  int32_t max_bits;       /* 1..8 */
  int32_t rope_keys;      /* 1: keys carry RoPE and are un-rotated first */
  int32_t rope_style;     /* ORC_ROPE_HALF / ORC_ROPE_INTERLEAVED */
  double rope_theta;
  int32_t rans_scale_bits;/* 8..15 */
  int32_t rans_lanes;     /* 1..64 */
  int32_t chunk_tokens;   /* tokens sharing one frequency table */
  int32_t tile_tokens;    /* tokens per packed tile = one rANS stream */
  int32_t basis_per_head; /* 0: basis [L,2,D,D]; 1: [L,2,H,D,D] */
  int32_t wht_keys;       /* WHT path: 1 = keys get RMS+WHT too */
  int32_t alloc_scope;    /* PCA path: 0 = one budget per section; 1 = one budget over all sections */
} orc_config;

/* ---- numeric primitives ---------------------------------------------- */
uint16_t orc_f32_to_bf16(float f);
float orc_bf16_to_f32(uint16_t h);
void orc_rope_table(int32_t T, int32_t D, double theta, float* cos_out, float* sin_out);
void orc_rope_inverse(const float* y, float* x, int32_t D, int32_t style,
                      const float* cos_row, const float* sin_row);
void orc_rope_forward(const float* x, float* y, int32_t D, int32_t style,
                      const float* cos_row, const float* sin_row);
void orc_project(const float* x, const float* Bp, int32_t D, float* c);
void orc_unproject(const float* chat, const float* Bp, int32_t D, float* x);
float orc_rms(const float* x, int32_t D);
void orc_wht(const float* x, int32_t D, float* y);

/* ---- statistics, allocation, quantiser ------------------------------- */
void orc_stats(const float* c, int64_t N, int32_t D, float* mu, float* var,
               float* cmin, float* cmax);
int32_t orc_budget(float bits, int32_t D);
void orc_alloc_greedy(const float* var, int32_t D, int32_t budget, int32_t max_bits,
                      uint8_t* bits);
double orc_alloc_dp(const float* var, int32_t D, int32_t budget, int32_t max_bits,
                    uint8_t* bits);
void orc_alloc_greedy_heap(const float* var, int64_t n, int64_t budget, int32_t max_bits,
                           uint8_t* bits);
void orc_checksum(const uint8_t* data, int64_t n_bytes, int64_t skip_from, int64_t skip_to,
                  uint64_t* a_out, uint64_t* b_out);
double orc_distortion(const float* var, const uint8_t* bits, int32_t D);
void orc_side_info(const uint8_t* bits, const float* mu, const float* cmin,
                   const float* cmax, int32_t D, float* zero, float* scale, float* rcp);
void orc_quantize(const float* c, int64_t N, int32_t D, const uint8_t* bits,
                  const float* zero, const float* rcp, uint8_t* q, float* vpre);
void orc_quantize_sym(const float* c, int64_t N, int32_t D, int32_t b, float rcp,
                      uint8_t* q, float* vpre);

/* ---- packing and entropy coding -------------------------------------- */
int64_t orc_packed_bytes(const uint8_t* bits, int32_t D, int64_t ntok);
void orc_pack(const uint8_t* q, int64_t ntok, int32_t D, const uint8_t* bits, uint8_t* out);
void orc_unpack(const uint8_t* in, int64_t ntok, int32_t D, const uint8_t* bits, uint8_t* q);
void orc_freq_normalize(const uint32_t* counts, int32_t n_sym, int32_t scale_bits, uint16_t* freq);
int64_t orc_rans_encode_seq(int64_t N, const uint8_t* sym, const uint8_t* lane, const int32_t* tab,
                            const int32_t* n_sym, const uint16_t* freqs, int32_t scale_bits,
                            int32_t lanes, uint32_t* states, uint16_t* words, int64_t words_cap);
int orc_rans_decode_seq(int64_t N, const uint8_t* lane, const int32_t* tab, const int32_t* n_sym,
                        const uint16_t* freqs, int32_t scale_bits, int32_t lanes,
                        const uint32_t* states, const uint16_t* words, int64_t nwords,
                        uint8_t* sym);
int64_t orc_rans_encode(const uint8_t* sym, int64_t N, const uint16_t* freq,
                        int32_t scale_bits, int32_t lanes, uint32_t* states,
                        uint16_t* words, int64_t words_cap);
int orc_rans_decode(const uint32_t* states, const uint16_t* words, int64_t nwords,
                    const uint16_t* freq, int32_t scale_bits, int32_t lanes,
                    int64_t N, uint8_t* sym);
/* Entropy-coding classes of a component of width b: symbol bits (the top
 * min(b, 4) bits of codes of width >= 2) and raw bits (the rest). */
int32_t orc_sym_bits(int32_t b);
int32_t orc_raw_bits(int32_t b);
/* One chunk record from its codes q[n][D]; *mode = 0 coded, 1 packed.
 * Returns the size (multiple of 16) or -1 when cap is too small. */
int64_t orc_chunk_encode(const orc_config* cfg, const uint8_t* bits, const uint8_t* q, int32_t n,
                         uint8_t* rec, int64_t cap, int32_t* mode);
int orc_chunk_decode(const orc_config* cfg, const uint8_t* bits, const uint8_t* rec, int64_t size,
                     int32_t mode, int32_t n, uint8_t* q);

/* ---- container ------------------------------------------------------- */
int orc_check_config(const orc_config* cfg);
uint64_t orc_fnv1a64(uint64_t h, const uint8_t* bytes, int64_t n);
uint64_t orc_fingerprint(const orc_config* cfg, const float* basis);
int64_t orc_max_container_bytes(const orc_config* cfg, int32_t T);
int orc_encode(const orc_config* cfg, const void* k, const void* v, int32_t T,
               const float* basis, uint8_t* out, int64_t cap, int64_t* out_bytes);
int orc_decode(const orc_config* cfg, const float* basis, const uint8_t* in,
               int64_t in_bytes, void* k_out, void* v_out, int32_t out_dtype);
/* Decode only sections [sec_begin, sec_end) of a container: the middle rows
 * of each, after forward RoPE on keys and before the output cast, as
 * [nsec, T_mid, D] fp32 (sampled cross-decode at full size). */
int orc_decode_sections(const orc_config* cfg, const float* basis, const uint8_t* in,
                        int64_t in_bytes, int32_t sec_begin, int32_t sec_end,
                        float* mid_out);
/* Quantisation codes of section u read back from a container (rANS decode
 * and unpacking only): q_out [T_mid, D]. */
int orc_section_codes(const orc_config* cfg, const float* basis, const uint8_t* in,
                      int64_t in_bytes, int32_t section, uint8_t* q_out);
/* Rows t0..t1 of section u as the encoder sees them: keys un-rotated, all rows
 * rounded to the operand precision.  x_out [t1-t0, D] fp32.  Used for basis
 * calibration (the basis is an input of the method, fitted offline). */
int orc_section_rows(const orc_config* cfg, const void* k, const void* v, int32_t T,
                     int32_t section, int32_t t0, int32_t t1, float* x_out);
/* Coefficients of one section's middle rows, as the encoder computes them.
 * c_out [T_mid, D] fp32; r_out [T_mid] (WHT path, may be NULL). */
int orc_section_coeffs(const orc_config* cfg, const void* k, const void* v, int32_t T,
                       const float* basis, int32_t section, float* c_out, float* r_out);

/* ---- scalar quantisers on gauge coordinates --------------------------- */
/* ("Codec-Gauge: Learning Compression-Friendly Gauges for Transformer KV
 * Caches", Compression Conditions: block-uniform uses one range per
 * T_b x d_l block; the KIVI-style path uses per-channel key and per-token
 * value ranges; both at a fixed bit setting.)  Every token of the cache is
 * coded; keys are un-rotated first and rotated back on decode. */
#define ORC_SQ_BLOCK 1
#define ORC_SQ_KIVI 2
typedef struct {
  int32_t kind;    /* ORC_SQ_BLOCK or ORC_SQ_KIVI */
  int32_t group;   /* channels per range (d_l); divides head_dim */
  int32_t tile;    /* tokens per range block (T_b) */
  int32_t bits_k, bits_v;  /* code widths, 1..8 */
} orc_sq_config;
int orc_sq_check(const orc_config* c, const orc_sq_config* q);
int64_t orc_sq_code_bytes(const orc_config* c, const orc_sq_config* q, int32_t T);
int64_t orc_sq_range_pairs(const orc_config* c, const orc_sq_config* q, int32_t T);
int orc_sq_encode(const orc_config* c, const orc_sq_config* q, const void* k, const void* v, int32_t T,
                  const float* basis, uint8_t* codes, float* ranges);
int orc_sq_decode(const orc_config* c, const orc_sq_config* q, const uint8_t* codes, const float* ranges,
                  int32_t T, const float* basis, float* k_out, float* v_out);

/* ---- TTAS-X2 value path: two-level product quantisation ---------------- */
/* ("TTAS-X2: Extreme KV Cache Compression for Large Language Models", 2.2 V
 * Compression: per-vector RMS normalisation, Hadamard transform, two-level
 * product quantisation with K1 = 256 and K2 = 64..512 centroids, a fixed
 * budget of outliers per head; 3 Experiments: the budget and K2 per layer.)
 * Value sections only.  Each value vector x: r = rms(x), y = WHT(x / r);
 * y is split into head_dim / sub_dim subvectors; level 1 takes the nearest
 * of k1 centroids, level 2 the nearest of k2 centroids to the level-1
 * residual; per (layer, head) and block of block_tokens tokens the
 * `outliers` coefficients with the largest |y - y^| are stored exactly. */
typedef struct {
  int32_t sub_dim;       /* channels per subvector; divides head_dim */
  int32_t k1, k2;        /* centroids per subspace, powers of two in [2, 512] */
  int32_t outliers;      /* budget per (layer, head) and block, >= 0 */
  int32_t block_tokens;  /* tokens per outlier block, >= 1 */
} orc_pq_config;
int orc_pq_check(const orc_config* c, const orc_pq_config* q);
int32_t orc_pq_row_words(const orc_config* c, const orc_pq_config* q);
int64_t orc_pq_outlier_slots(const orc_config* c, const orc_pq_config* q, int32_t T);
/* Nearest of k centroids cb[k][d] (entries rounded to bf16) to y[d]: the
 * smallest sum_j (y_j - c_j)^2 in fp64, summed in j order; ties go to the
 * lowest index. */
int32_t orc_pq_nearest(const float* y, const float* cb, int32_t k, int32_t d);
/* v: [L,H,T,D] in the cache dtype; cb1 [L][M][k1][d], cb2 [L][M][k2][d]
 * fp32 (rounded to bf16 on use).  codes [L][H][T][row_words] u32, rms
 * [L][H][T] f32, outliers [L][H][blocks][outliers][2] u32 (index t D + j
 * within the section, fp32 bits of y), index-ascending per block, unused
 * slots (0xFFFFFFFF, 0). */
int orc_pq_encode(const orc_config* c, const orc_pq_config* q, const void* v, int32_t T, const float* cb1,
                  const float* cb2, uint32_t* codes, float* rms, uint32_t* outliers);
int orc_pq_decode(const orc_config* c, const orc_pq_config* q, const uint32_t* codes, const float* rms,
                  const uint32_t* outliers, int32_t T, const float* cb1, const float* cb2, float* v_out);

#ifdef __cplusplus
}
#endif
#endif
