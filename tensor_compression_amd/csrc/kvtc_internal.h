// Internal declarations of libkvtc: container and workspace layouts, kernel
// parameter blocks and the launch functions implemented by the .hip files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvtc.h"

namespace kvtc {

constexpr uint32_t kRansL = 1u << 16;  // lower end of the normalised rANS state interval
constexpr int kHeaderBytes = 256;
constexpr int kDirEntry = 32;  // u64 offset, u32 size, u32 record mode, u64 x 2 record checksum
constexpr int kContainerVersion = 3;
constexpr int kCsumField = 200;     // header bytes [200, 216): checksum of the fixed part
constexpr int kCsumParts = 1024;    // workgroups (partial sums) of a fixed-part checksum
constexpr int kBlkTokens = 1024;  // tokens of a transform work block (at most)
constexpr int kMaxTilesPerRec = 32;

// Two token granularities split a section's middle:
//  * chunks (config.chunk_tokens): the container's records, each with its own
//    frequency tables, stream word counts and directory entry;
//  * work blocks of at most kBlkTokens tokens: the unit the transform kernels
//    (statistics, quantise-and-pack, decode transform) take per workgroup and
//    the unit of the packed buffer in the workspace.  A chunk is a whole
//    number of blocks and a block a whole number of tiles.

// Where each part of a container sits for a given T (all offsets in bytes
// from the container start).  Only the chunk records have data-dependent
// sizes; everything before chunks_off is fixed by the configuration and T.
struct Layout {
  int32_t T, s0, mid_begin, mid_end, T_mid, W_eff;
  int32_t n_sections;
  int32_t blk_tokens, blks_per_sec, n_blks, tiles_per_blk;             // work blocks
  int32_t rec_tokens, recs_per_sec, n_recs, tiles_per_rec, blks_per_rec;  // chunk records
  int32_t n_r_sections;
  int32_t budget_k, budget_v;
  int32_t sec_bits_max;  // largest width sum of one section (its budget, or all components at max_bits)
  int64_t total_budget;  // the budget of all sections together (one-budget allocation)
  int64_t side_off, r_off, side_bytes, raw_off, raw_bytes, dir_off, chunks_off;
};

// Workspace carve-up (byte offsets from the workspace start).
struct WsLayout {
  int64_t status;      // u32 status, u32 exact re-computations, u64 container bytes
  int64_t part_sum;    // f64 [n_sections][blocks][D]
  int64_t part_sq;     // f64 [n_sections][blocks][D]
  int64_t part_min;    // f32 [n_sections][blocks][D]
  int64_t part_max;    // f32 [n_sections][blocks][D]
  int64_t sec_stats;   // f32x4 [n_sections][D]: mean, variance, min, max
  int64_t side_rcp;    // f32 [n_sections][D]
  int64_t side_zero;   // f32 [n_sections][D]
  int64_t side_bits;   // u8  [n_sections][D]
  int64_t packed;      // [n_blks][packed_slot] packed tiles of each work block
  int64_t packed_slot;
  int64_t rec;         // [n_recs][rec_slot] encoder record slots
  int64_t rec_slot;
  int64_t tile_words_max;  // words capacity of one tile stream in a slot
  int64_t tile_raw_max;    // bytes of one tile's raw rows in a slot
  int64_t rec_size;    // u32 [n_recs]
  int64_t rec_mode;    // u32 [n_recs]: 0 coded, 1 packed
  int64_t rec_pos;     // u64 [n_recs]
  int64_t kprime;      // bf16 [L][H][T_mid][D]: mid-region keys with RoPE removed (head_dim 128 bf16 path)
  int64_t fixed;       // paged batch: staging of the container's fixed part [chunks_off]
  int64_t csum;        // u64 x 2 [kCsumParts]: partial checksums of the fixed part
  int64_t total;
};

#define KVTC_HD __host__ __device__

KVTC_HD inline int64_t align16(int64_t x) { return (x + 15) & ~(int64_t)15; }
KVTC_HD inline int64_t align256(int64_t x) { return (x + 255) & ~(int64_t)255; }

KVTC_HD inline int32_t floor_bits(float b) { return (int32_t)floorf(b); }

// Work-block size of a configuration: the chunk itself when it has at most
// kBlkTokens tokens, otherwise kBlkTokens (the configuration check makes a
// longer chunk a multiple of it).
KVTC_HD inline int32_t blk_tokens_of(const kvtc_config& c) {
  return c.chunk_tokens <= kBlkTokens ? c.chunk_tokens : kBlkTokens;
}

// Entropy-coding classes of a component of width b ("rANS Makes the Last Mile
// Smaller"): codes of width >= 2 are coded one symbol per token, the symbol
// being the top min(b, 4) bits with a frequency table per (chunk,
// component); 1-bit codes and the low b - 4 bits of wider codes are raw.
KVTC_HD inline int32_t sym_bits_of(int32_t b) { return b >= 2 ? (b < 4 ? b : 4) : 0; }
KVTC_HD inline int32_t raw_bits_of(int32_t b) { return b == 1 ? 1 : (b >= 5 ? b - 4 : 0); }

KVTC_HD inline bool section_has_r(const kvtc_config& c, int s) {
  return c.transform == KVTC_WHT && (s == 1 || c.wht_keys);
}

// Region split ("How the Pipeline Works": sink tokens at the front, a
// compressed middle, a recent window kept at full fidelity) and the fixed
// part of the container.
KVTC_HD inline Layout make_layout(const kvtc_config& c, int32_t T) {
  Layout lo{};
  lo.T = T;
  lo.s0 = c.sink_tokens < T ? c.sink_tokens : T;
  lo.mid_begin = lo.s0;
  int32_t e = T - c.recent_tokens;
  lo.mid_end = e > lo.s0 ? e : lo.s0;
  lo.T_mid = lo.mid_end - lo.mid_begin;
  lo.W_eff = T - lo.mid_end;
  lo.n_sections = c.layers * 2 * c.kv_heads;
  lo.blk_tokens = blk_tokens_of(c);
  lo.blks_per_sec = lo.T_mid > 0 ? (lo.T_mid + lo.blk_tokens - 1) / lo.blk_tokens : 0;
  lo.n_blks = lo.n_sections * lo.blks_per_sec;
  lo.tiles_per_blk = lo.blk_tokens / c.tile_tokens;
  lo.rec_tokens = c.chunk_tokens;
  lo.recs_per_sec = lo.T_mid > 0 ? (lo.T_mid + c.chunk_tokens - 1) / c.chunk_tokens : 0;
  lo.n_recs = lo.n_sections * lo.recs_per_sec;
  lo.tiles_per_rec = c.chunk_tokens / c.tile_tokens;
  lo.blks_per_rec = c.chunk_tokens / lo.blk_tokens;
  lo.n_r_sections = 0;
  for (int s = 0; s < 2; ++s)
    if (section_has_r(c, s)) lo.n_r_sections += c.layers * c.kv_heads;
  int64_t eb = c.dtype == KVTC_BF16 ? 2 : 4;
  int64_t D = c.head_dim;
  lo.side_off = kHeaderBytes;
  lo.r_off = lo.side_off + (int64_t)lo.n_sections * 9 * D;
  lo.side_bytes = align16((int64_t)lo.n_sections * 9 * D + (int64_t)lo.n_r_sections * lo.T_mid * 4);
  lo.raw_off = lo.side_off + lo.side_bytes;
  lo.raw_bytes = align16(2 * (int64_t)c.layers * c.kv_heads * (lo.s0 + lo.W_eff) * D * eb);
  lo.dir_off = lo.raw_off + lo.raw_bytes;
  lo.chunks_off = lo.dir_off + (int64_t)lo.n_recs * kDirEntry;
  if (c.transform == KVTC_PCA) {
    lo.budget_k = (int32_t)floorf(c.bits_k * (float)c.head_dim);
    lo.budget_v = (int32_t)floorf(c.bits_v * (float)c.head_dim);
  } else {
    lo.budget_k = floor_bits(c.bits_k) * c.head_dim;
    lo.budget_v = floor_bits(c.bits_v) * c.head_dim;
  }
  lo.total_budget = (int64_t)c.layers * c.kv_heads * ((int64_t)lo.budget_k + lo.budget_v);
  lo.sec_bits_max = lo.budget_k > lo.budget_v ? lo.budget_k : lo.budget_v;
  if (c.alloc_scope == 1) {
    const int64_t cap = (int64_t)c.head_dim * c.max_bits;
    lo.sec_bits_max = (int32_t)(lo.total_budget < cap ? lo.total_budget : cap);
  }
  return lo;
}

// Packed bytes of a tile of ntok tokens at most: ntok budget / 8 plus one
// padding word per nonzero-width component row.
KVTC_HD inline int64_t max_tile_bytes(const kvtc_config& c, int32_t ntok, int32_t budget) {
  int32_t nz = budget < c.head_dim ? budget : c.head_dim;
  return ((int64_t)ntok * budget + 7) / 8 + 4 * (int64_t)nz;
}

// Status block at the start of every workspace: the status word (error
// bits), the exact re-computation count and the container size in its first
// 16 bytes, then kCountSlots counters on lines of their own that workgroups
// add their re-computation counts to (spread so that the adds do not queue
// on one line); the count is word 1 plus the slots.
constexpr int kCountSlots = 64;
constexpr int64_t kCountOff = 256;
constexpr int64_t kCountStride = 128;
constexpr int64_t kStatusBlockBytes = kCountOff + kCountSlots * kCountStride;
constexpr int64_t kGlobalThrOff = 16;  // u64 threshold key of the one-budget allocation

// Bytes of a record slot's table area: 16 u16 entries per component.
KVTC_HD inline int64_t slot_table_bytes(const kvtc_config& c) { return 32 * (int64_t)c.head_dim; }

// `paged`: the workspace of one sequence of a paged batch, which also stages
// the fixed part of its container (everything before chunks_off).
KVTC_HD inline WsLayout make_ws_layout(const kvtc_config& c, const Layout& lo, bool paged = false) {
  WsLayout w{};
  int64_t D = c.head_dim;
  int64_t nsc = (int64_t)lo.n_sections * (lo.blks_per_sec > 0 ? lo.blks_per_sec : 1);
  auto take = [](int64_t& at, int64_t bytes) {
    int64_t o = at;
    at += (bytes + 255) & ~(int64_t)255;
    return o;
  };
  int64_t at = 0;
  w.status = take(at, kStatusBlockBytes);
  w.part_sum = take(at, nsc * D * 8);
  w.part_sq = take(at, nsc * D * 8);
  w.part_min = take(at, nsc * D * 4);
  w.part_max = take(at, nsc * D * 4);
  w.sec_stats = take(at, (int64_t)lo.n_sections * D * 16);
  w.side_rcp = take(at, (int64_t)lo.n_sections * D * 4);
  w.side_zero = take(at, (int64_t)lo.n_sections * D * 4);
  w.side_bits = take(at, (int64_t)lo.n_sections * D);
  int64_t tile_max = max_tile_bytes(c, c.tile_tokens, lo.sec_bits_max);
  w.packed_slot = align16(tile_max * lo.tiles_per_blk);
  w.packed = take(at, (int64_t)lo.n_blks * w.packed_slot);
  // A tile stream whose words outgrow its packed size cannot make the record
  // smaller than the packed form, so the record falls back to it; the word
  // capacity (rounded so that every piece of a slot stays 16-byte aligned)
  // only has to hold streams that can still win.
  w.tile_words_max = ((tile_max / 2 + 2 * (int64_t)c.rans_lanes + 8 + 7) & ~(int64_t)7);
  w.tile_raw_max = align16(tile_max);
  w.rec_slot = align16(slot_table_bytes(c) + 4 * (int64_t)lo.tiles_per_rec) +
               (int64_t)lo.tiles_per_rec * (4 * c.rans_lanes + 2 * w.tile_words_max + w.tile_raw_max);
  const bool fast128 = c.head_dim == 128 && c.dtype == KVTC_BF16 && c.transform == KVTC_PCA &&
                       c.tile_tokens % 64 == 0 && c.rope_keys;
  const int64_t kprime_bytes = fast128 ? (int64_t)c.layers * c.kv_heads * lo.T_mid * D * 2 : 0;
  const int64_t rec_bytes = (int64_t)lo.n_recs * w.rec_slot;
  w.kprime = take(at, kprime_bytes);
  // the record slots are written by the rANS encoder, after the last reader
  // of the un-rotated keys (the quantiser): they share its memory when it is
  // large enough
  w.rec = (kprime_bytes > 0 && rec_bytes <= kprime_bytes) ? w.kprime : take(at, rec_bytes);
  w.rec_size = take(at, (int64_t)lo.n_recs * 4);
  w.rec_mode = take(at, (int64_t)lo.n_recs * 4);
  w.rec_pos = take(at, (int64_t)lo.n_recs * 8 + 8);
  w.fixed = take(at, paged ? lo.chunks_off : 0);
  w.csum = take(at, (int64_t)kCsumParts * 16);
  w.total = at;
  return w;
}


struct PlanImpl {
  kvtc_config cfg;
  uint8_t* mem;          // plan memory (device)
  void* basis_t;         // operand precision, component-major: [n_basis][i][j] = B[j][i]
  void* basis;           // operand precision, channel-major:   [n_basis][j][i]
  float2* rope;          // [max_tokens][D/2] (cos, sin)
  int32_t n_basis;
  uint64_t fingerprint;
  float max_col_norm;  // largest column norm of the operand-precision basis
  size_t mem_bytes;
  // profiling (kvtc_profile_*)
  int32_t prof_on;
  int32_t prof_n;  // events recorded by the last call
  hipEvent_t prof_ev[24];
  const char* prof_name[24];
  int32_t prof_created;
};

// Everything a kernel needs about one call, passed by value.
struct Params {
  // shape / config
  int32_t L, H, D, dtype, transform, rope_keys, rope_style, max_bits;
  int32_t sb, lanes, blk_tokens, tile_tokens, basis_per_head, wht_keys;
  int32_t budget_k, budget_v;
  int32_t sec_bits_max, alloc_scope;
  int64_t total_budget;
  int32_t T, s0, mid_begin, mid_end, T_mid, W_eff, n_sections, blks_per_sec, n_blks,
      tiles_per_blk;
  int32_t rec_tokens, recs_per_sec, n_recs, tiles_per_rec, blks_per_rec;
  int32_t bits_k_uniform, bits_v_uniform;
  float mfma_err;  // bound factor: |c_mfma - c_exact| <= mfma_err * ||x||_2
  int64_t side_off, r_off, raw_off, raw_bytes, dir_off, chunks_off;
  // plan
  const void* basis_t;
  const void* basis;
  const float2* rope;
  // tensors
  const void* k;
  const void* v;
  void* k_out;
  void* v_out;
  int32_t out_dtype;
  // container
  uint8_t* out;      // encode output
  const uint8_t* in; // decode input
  int64_t cap;       // encode capacity / decode input bytes
  // workspace
  uint8_t* ws;
  WsLayout w;
  // paged batch (n_seqs > 0): blockIdx.z selects a sequence; at_seq() turns
  // the batch parameters into that sequence's
  kvtc_config cfg;
  int32_t n_seqs;
  int32_t pool_pages;           // pages in each pool [L, pool_pages, H, 16, D]
  int32_t max_pages;            // length of a page-table row
  const int32_t* page_table;    // [n_seqs][max_pages]
  const int32_t* page_row;      // this sequence's row (null: contiguous cache)
  struct SeqInfo* seqs;         // [n_seqs], in the batch workspace
  uint8_t* out_final;           // where this sequence's records go (encode)
};

constexpr int kPageTokens = 16;

// One call of the scalar quantisers on gauge coordinates (kernels_sq.hip).
// Every token of [0, T) is coded.  A range is a block of te tokens x ce
// channels of one section: block-uniform (tile, group), KIVI keys (tile, 1),
// KIVI values (1, group).  Index [s]: the section kind, 0 keys, 1 values.
struct SqParams {
  int32_t L, H, T, basis_per_head, rope_keys, rope_style, out_dtype;
  int32_t bits[2], te[2], ce[2];
  int64_t code_bytes[2];  // bytes of one section's codes
  int64_t n_ranges[2];    // (zero, scale) pairs of one section
  float mfma_err;         // |c_mfma - c_exact| <= mfma_err * ||x||_2
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* basis_t;  // component-major [n_basis][i][j] = B[j][i], bf16
  const uint16_t* basis;    // channel-major   [n_basis][j][i], bf16
  const float2* rope;
  uint8_t* codes;
  float* ranges;
  void* k_out;
  void* v_out;
  uint32_t* status;  // device word or null
};

// Per-sequence placement of a paged batch, written on the device.
struct SeqInfo {
  int32_t T;        // tokens of the sequence
  int32_t pad;
  int64_t ws_off;   // its workspace, from the batch workspace start
  int64_t out_off;  // its container, from the batch container start
  int64_t cap;      // decode: bytes of its container
};

// Batch workspace: a status block in the contiguous-call format (status bits,
// exact re-computations, total bytes), the SeqInfo table, then one workspace
// per sequence.
KVTC_HD inline int64_t batch_seqinfo_off() { return 256; }
KVTC_HD inline int64_t batch_ws_head(int32_t n_seqs) {
  return align256(batch_seqinfo_off() + (int64_t)n_seqs * (int64_t)sizeof(SeqInfo));
}
// Batch container: "KVTB", version, n_seqs, header bytes, u64 total, then
// u64 offset and u64 size per sequence; sequence containers start 256-byte
// aligned and are each what kvtc_encode writes for that sequence alone.
constexpr int kBatchFixedBytes = 64;
KVTC_HD inline int64_t batch_header_bytes(int32_t n_seqs) {
  return align256(kBatchFixedBytes + 16 * (int64_t)n_seqs);
}

// This sequence's parameters (identity for a contiguous call).
__device__ inline Params at_seq(const Params& p0, int z) {
  if (p0.n_seqs == 0) return p0;
  Params p = p0;
  const SeqInfo si = p0.seqs[z];
  const Layout lo = make_layout(p0.cfg, si.T);
  p.T = lo.T; p.s0 = lo.s0; p.mid_begin = lo.mid_begin; p.mid_end = lo.mid_end;
  p.T_mid = lo.T_mid; p.W_eff = lo.W_eff; p.blks_per_sec = lo.blks_per_sec; p.n_blks = lo.n_blks;
  p.recs_per_sec = lo.recs_per_sec; p.n_recs = lo.n_recs;
  p.side_off = lo.side_off; p.r_off = lo.r_off; p.raw_off = lo.raw_off; p.raw_bytes = lo.raw_bytes;
  p.dir_off = lo.dir_off; p.chunks_off = lo.chunks_off;
  p.w = make_ws_layout(p0.cfg, lo, true);
  p.ws = p0.ws + si.ws_off;
  p.out = p.ws + p.w.fixed;  // the fixed part is staged until the sequence is placed
  p.out_final = p0.out + si.out_off;
  p.in = p0.in + si.out_off;
  p.cap = si.cap;
  p.page_row = p0.page_table + (int64_t)z * p0.max_pages;
  return p;
}

// gridDim.z of a launch: one slice per sequence of a paged batch.
inline unsigned seq_grid(const Params& p) { return p.n_seqs > 0 ? (unsigned)p.n_seqs : 1u; }

// Element offset of the row (layer l, head h, token pos) of K or V: the
// contiguous [L, H, T, D] cache, or a pool [L, P, H, 16, D] through the page
// table.
__device__ inline int64_t cache_row(const Params& p, int l, int h, int pos) {
  if (p.page_row == nullptr) return (((int64_t)l * p.H + h) * p.T + pos) * p.D;
  const int64_t page = p.page_row[pos >> 4];
  return (((((int64_t)l * p.pool_pages + page) * p.H + h) << 4) + (pos & 15)) * p.D;
}

// host helpers (kvtc_api.hip)
int64_t max_container_bytes(const kvtc_config& c, const Layout& lo);
Params make_params(const PlanImpl& p, const Layout& lo, const WsLayout& w);
void build_header(const PlanImpl& p, const Layout& lo, uint8_t* hdr);

// launches (kernels_*.hip); each returns hipSuccess or the launch error
hipError_t launch_copy_raw(const Params& p, int to_container, hipStream_t s);
hipError_t launch_enc_transform(const Params& p, int mode, hipStream_t s);  // 0 stats, 1 quant
hipError_t launch_enc_alloc(const Params& p, hipStream_t s);
hipError_t launch_quant128(const Params& p, hipStream_t s);  // head_dim 128 bf16 PCA, tile % 64 == 0
hipError_t launch_rans_encode_chunks(const Params& p, hipStream_t s, bool with_raw = false);
hipError_t launch_assemble(const Params& p, const uint8_t* hdr, hipStream_t s);
hipError_t launch_dec_check(const Params& p, const uint8_t* hdr, hipStream_t s);
// checksum of the fixed part: written into the header (encode = 1) or
// checked against it (encode = 0)
hipError_t launch_csum(const Params& p, int encode, hipStream_t s);
// stage hooks: allocation and side information from the statistics in the
// workspace; RoPE undo of the middle keys into the workspace (bf16 head_dim
// 128 path)
hipError_t launch_alloc_from_stats(const Params& p, hipStream_t s);
hipError_t launch_unrope(const Params& p, hipStream_t s);
hipError_t launch_rans_decode_chunks(const Params& p, hipStream_t s, bool with_raw = false);
hipError_t launch_dec_transform(const Params& p, hipStream_t s);
hipError_t launch_coeffs(const Params& p, int sec_begin, int sec_end, float* out, float* r_out,
                         hipStream_t s);
hipError_t launch_seq_setup(const Params& p, const int32_t* seq_lens, int64_t sum_t, int32_t max_t, int64_t ws_bytes,
                            int mode, hipStream_t s);  // mode 0 encode, 1 decode
hipError_t launch_batch_place(const Params& p, hipStream_t s);
hipError_t launch_batch_finish(const Params& p, hipStream_t s);
hipError_t launch_test_freq_tables(const uint32_t* counts, const int32_t* alpha, int n, int sb, uint16_t* freq,
                                   hipStream_t s);
// One call of the TTAS-X2 value path (kernels_pq.hip): value sections
// (layer l, head h) = l H + h, head_dim 128, subvectors of 8 channels.
struct PqParams {
  int32_t L, H, T;
  int32_t k1, k2, b1, b2;  // centroids per subspace and their index bits
  int32_t B, bt;           // outliers per (section, block), tokens per block
  int32_t rw;              // u32 words of a token's code row
  int32_t nspan, nblk;     // 64-token spans and outlier blocks per section
  int32_t out_dtype;
  const float* cb1;  // [L][16][k1][8] fp32 (caller's)
  const float* cb2;  // [L][16][k2][8]
  uint16_t* cb1h;    // workspace: the codebooks in bf16
  uint16_t* cb2h;
  float* cn2;        // workspace: [L][16][k1 + k2] squared norms of the bf16 centroids
  float* cmax;       // workspace: [L][16][2] largest centroid norm per level
  uint4* cand;       // workspace: [L H][nspan][B] candidates (|err| bits, index, y bits, 0)
  const uint16_t* v;
  uint32_t* codes;        // [L H][T][rw]
  float* rms;             // [L H][T]
  uint32_t* outl;         // [L H][nblk][B][2]
  void* v_out;
  uint32_t* status;       // device word or null
};
hipError_t launch_pq_encode(const PqParams& q, hipStream_t s);
hipError_t launch_pq_decode(const PqParams& q, hipStream_t s);

// scalar quantisers (head_dim 128, bf16): encode clears *status first
hipError_t launch_sq_encode(const SqParams& q, hipStream_t s);
hipError_t launch_sq_decode(const SqParams& q, hipStream_t s);
hipError_t launch_prep_basis(const float* src, void* basis_t, void* basis, int n_basis, int D,
                             int dtype, int32_t* bad, hipStream_t s);

// ---------------------------------------------------------------------------
// device helpers shared by the kernels
// ---------------------------------------------------------------------------

// Bytes of one packed tile of `ntok` tokens: a row of ceil(ntok*b/32) words
// per component with b > 0.
__device__ inline int32_t tile_row_words(int32_t ntok, int32_t b) { return (ntok * b + 31) >> 5; }

__device__ inline float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

__device__ inline uint16_t f32_to_bf16(float f) {
  __bf16 b = (__bf16)f;  // round to nearest even (v_cvt_pk_bf16_f32)
  return __builtin_bit_cast(uint16_t, b);
}

__device__ inline float round_bf16(float f) { return bf16_to_f32(f32_to_bf16(f)); }

// A decoder's output rows: 16 bytes stored with the non-temporal cache policy
// (nothing in the codec reads them again, and they then do not fill the
// caches with dirty lines that the next launch would have to write back)
typedef uint32_t u32x4_out __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_out16(void* dst, uint4 v) {
  __builtin_nontemporal_store(__builtin_bit_cast(u32x4_out, v), reinterpret_cast<u32x4_out*>(dst));
}
__device__ __forceinline__ void store_out16(void* dst, float4 v) { store_out16(dst, __builtin_bit_cast(uint4, v)); }

// ---- integrity checksum ("Quantum-Aware Tensor Compression", QATC
// transport: an aggregate checksum; damaged payloads are refused before
// restore).  Over the little-endian 32-bit words w_j of a range:
// A = sum w_j and B = sum (j + 1) w_j, both modulo the prime 2^61 - 1.
constexpr uint64_t kCsumP = (1ull << 61) - 1;

__device__ __forceinline__ uint64_t mod61(uint64_t x) {  // x < 2^64 -> [0, P)
  x = (x & kCsumP) + (x >> 61);
  return x >= kCsumP ? x - kCsumP : x;
}

__device__ __forceinline__ uint64_t mulmod61(uint64_t a, uint64_t b) {  // a, b < 2^61
  const uint64_t lo = a * b, hi = __umul64hi(a, b);
  // a b = hi 2^64 + lo = (8 hi) 2^61 + lo, and 2^61 = 1 (mod P)
  return mod61((lo & kCsumP) + (lo >> 61) + (hi << 3));
}

// Adds word w at index j of the range to a thread's partial sums.
__device__ __forceinline__ void csum_add(uint64_t& A, uint64_t& B, uint64_t j, uint32_t w) {
  A = mod61(A + w);
  B = mod61(B + mulmod61(j + 1, w));
}

// Sum of the partials of a whole workgroup (at most 16 waves) in thread 0;
// `sh` holds 32 u64 of LDS.  Every thread of the workgroup must call it.
__device__ inline void csum_block_reduce(uint64_t& A, uint64_t& B, uint64_t* sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    A = mod61(A + __shfl_xor(A, o, 64));
    B = mod61(B + __shfl_xor(B, o, 64));
  }
  if (lane == 0) { sh[wave] = A; sh[16 + wave] = B; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int k = 1; k < (int)((blockDim.x + 63) >> 6); ++k) {
      A = mod61(A + sh[k]);
      B = mod61(B + sh[16 + k]);
    }
  }
  __syncthreads();
}

__device__ inline void set_status(uint8_t* ws, const WsLayout& w, uint32_t code) {
  atomicOr(reinterpret_cast<uint32_t*>(ws + w.status), 1u << code);
}

__device__ inline uint32_t get_status(const uint8_t* ws, const WsLayout& w) {
  return __atomic_load_n(reinterpret_cast<const uint32_t*>(ws + w.status), __ATOMIC_RELAXED);
}

// Workgroup barrier for LDS traffic only: waits for this wave's LDS
// operations, not for its global loads and stores (which a plain
// __syncthreads also drains, so prefetches in flight would stall it).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Encode of a contiguous cache: the first workgroup of the first pass over
// the middle clears the status word and the count slots (no workgroup of that
// pass reads or sets them).
__device__ inline void clear_status_block(const Params& p) {
  if (threadIdx.x < 4) reinterpret_cast<uint32_t*>(p.ws + p.w.status)[threadIdx.x] = 0u;
  if (threadIdx.x < kCountSlots)
    *reinterpret_cast<uint32_t*>(p.ws + p.w.status + kCountOff + kCountStride * threadIdx.x) = 0u;
}

// The counter slot of a workgroup (x, y).
__device__ inline uint32_t* count_slot(uint8_t* ws, const WsLayout& w) {
  const uint32_t i = (blockIdx.x + blockIdx.y * gridDim.x) % kCountSlots;
  return reinterpret_cast<uint32_t*>(ws + w.status + kCountOff + kCountStride * i);
}

// ---- raw sink / recent regions ------------------------------------------------
// to_container = 1: cache -> container (+ zero the side and raw padding);
// 0: container -> output tensors in out_dtype.
// Raw regions as contiguous runs: for every (tensor, region, layer x head) the
// n_region rows are consecutive both in the cache ([L,H,T,D]) and in the
// container ([L,H,n_region,D] per tensor and region).  A workgroup per run;
// each thread moves up to eight 16-byte units (rows are whole 16-byte units
// for head_dim 64 and 128), all loads issued before the stores.
// One run by the calling workgroup (any size; the rANS decoder's extra
// workgroups also use it).  first: clears the status block (encode,
// contiguous cache).
__device__ inline void copy_raw_run(const Params& p, int run, int to_container, bool first) {
  const int nth = (int)blockDim.x;
  const int e = p.dtype == KVTC_BF16 ? 2 : 4;
  const int row_units = p.D * e / 16;
  const int LH = p.L * p.H;
  const int s = run / (2 * LH), region = (run / LH) & 1, lh = run % LH;
  const int n_region = region == 0 ? p.s0 : p.W_eff;
  const int units = n_region * row_units;
  if (to_container && first && run == 0) {
    if (threadIdx.x < 4) reinterpret_cast<uint32_t*>(p.ws + p.w.status)[threadIdx.x] = 0u;
    if (threadIdx.x < kCountSlots)
      *reinterpret_cast<uint32_t*>(p.ws + p.w.status + kCountOff + kCountStride * threadIdx.x) = 0u;
  }
  if (!to_container && (get_status(p.ws, p.w) & (1u << KVTC_ERR_CORRUPT))) return;
  const int64_t row_bytes = (int64_t)p.D * e;
  const int64_t per_tensor = (int64_t)LH * (p.s0 + p.W_eff) * row_bytes;
  const int64_t cbase = (int64_t)s * per_tensor + (region == 0 ? 0 : (int64_t)LH * p.s0 * row_bytes) +
                        (int64_t)lh * n_region * row_bytes;
  const int pos0 = region == 0 ? 0 : p.mid_end;
  // first element of unit i of the run in the cache
  auto telem = [&](int i) {
    const int row = i / row_units, ui = i - row * row_units;
    return cache_row(p, lh / p.H, lh % p.H, pos0 + row) + (int64_t)ui * (16 / e);
  };
  for (int i0 = 0; i0 < units; i0 += 8 * nth) {
    uint4 v[8];
    if (to_container) {
      const uint8_t* src = reinterpret_cast<const uint8_t*>(s ? p.v : p.k);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int i = i0 + k * nth + (int)threadIdx.x;
        if (i < units) v[k] = *reinterpret_cast<const uint4*>(src + telem(i) * e);
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int i = i0 + k * nth + (int)threadIdx.x;
        if (i < units) *reinterpret_cast<uint4*>(p.out + p.raw_off + cbase + (int64_t)i * 16) = v[k];
      }
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int i = i0 + k * nth + (int)threadIdx.x;
        if (i < units) v[k] = *reinterpret_cast<const uint4*>(p.in + p.raw_off + cbase + (int64_t)i * 16);
      }
      void* dst = s ? p.v_out : p.k_out;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int i = i0 + k * nth + (int)threadIdx.x;
        if (i >= units) continue;
        const uint4 w = v[k];
        const int64_t te = telem(i);
        if (p.out_dtype == p.dtype) {
          *reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(dst) + te * e) = w;
        } else if (p.dtype == KVTC_BF16) {  // bf16 -> fp32: exact widening of 8 values
          uint4* d = reinterpret_cast<uint4*>(reinterpret_cast<float*>(dst) + te);
          d[0] = make_uint4(w.x << 16, w.x & 0xffff0000u, w.y << 16, w.y & 0xffff0000u);
          d[1] = make_uint4(w.z << 16, w.z & 0xffff0000u, w.w << 16, w.w & 0xffff0000u);
        } else {  // fp32 -> bf16 (RNE) of 4 values
          const uint32_t lo = (uint32_t)f32_to_bf16(__uint_as_float(w.x)) | ((uint32_t)f32_to_bf16(__uint_as_float(w.y)) << 16);
          const uint32_t hi = (uint32_t)f32_to_bf16(__uint_as_float(w.z)) | ((uint32_t)f32_to_bf16(__uint_as_float(w.w)) << 16);
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(dst) + te) = make_uint2(lo, hi);
        }
      }
    }
  }
  if (to_container && run == 0 && threadIdx.x < 64) {
    // zero padding: the gap between the side records (and r area) and
    // raw_off, and the raw area's tail; each is shorter than 16 bytes
    int64_t r_used = 0;
    if (p.transform == KVTC_WHT) r_used = (int64_t)(p.wht_keys ? 2 : 1) * p.L * p.H * p.T_mid * 4;
    const int64_t a0 = p.r_off + r_used, a1 = p.raw_off;
    const int64_t b0 = p.raw_off + 2 * (int64_t)LH * (p.s0 + p.W_eff) * p.D * e, b1 = p.raw_off + p.raw_bytes;
    const int64_t na = a1 - a0, nb = b1 - b0;
    for (int64_t k = threadIdx.x; k < na + nb; k += 64) p.out[k < na ? a0 + k : b0 + (k - na)] = 0;
  }
}

// ---------------------------------------------------------------------------
// fp64 Walsh-Hadamard butterflies over 16-lane rows and exactly rounded
// quotients (the RMS / Hadamard value paths)
// ---------------------------------------------------------------------------

// Lane i of every 16-lane row takes v from lane i ^ O, O = 1, 2, 4, 8:
// DPP quad permutations for 1 and 2, a swizzle for 4, a row rotation for 8.
template <int O>
__device__ __forceinline__ uint32_t xor16_u32(uint32_t v) {
  if constexpr (O == 1) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
  else if constexpr (O == 2) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);
  else if constexpr (O == 4) return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, (4 << 10) | 0x1F);
  else return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, false);
}
template <int O>
__device__ __forceinline__ double xor16(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint64_t lo = xor16_u32<O>((uint32_t)u), hi = xor16_u32<O>((uint32_t)(u >> 32));
  return __longlong_as_double((long long)(lo | (hi << 32)));
}

// One fp64 butterfly stage across lanes: the lane with bit O of q set keeps
// (partner - own), the other (own + partner); fma by +-1 rounds each once.
template <int O>
__device__ __forceinline__ void wht_lane_stage(double (&y)[8], int q) {
  const double sg = (q & O) ? -1.0 : 1.0;
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] = __fma_rn(sg, y[e], xor16<O>(y[e]));
}

// Butterflies over the 128 channels of a token (the orthonormal transform
// without its 1 / sqrt(128)): bits 0-2 of the channel index in a lane's
// registers, bits 3-6 across its 16-lane row (lane q holds channels
// 8 q .. 8 q + 7).  Every sum is one fp64 rounding, stage by stage.
__device__ __forceinline__ void wht_fp64(double (&y)[8], int q) {
#pragma unroll
  for (int st = 1; st < 8; st <<= 1)
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (!(e & st)) {
        const double a = y[e], b = y[e + st];
        y[e] = a + b;
        y[e + st] = a - b;
      }
  wht_lane_stage<1>(y, q);
  wht_lane_stage<2>(y, q);
  wht_lane_stage<4>(y, q);
  wht_lane_stage<8>(y, q);
}

// True when z (an fp64 value within 2 of its units in the last place of a
// real number u) cannot be trusted to round to fp32 as u does: z lies within
// 8 fp64 units of an fp32 rounding midpoint of its binade, or below the fp32
// normal range, where that grid changes.  Zero is exact.
__device__ __forceinline__ bool f32_round_unsure(double z) {
  const uint32_t lo = (uint32_t)__double_as_longlong(z);
  const bool mid = ((lo + 8u - 0x10000000u) & 0x1FFFFFFFu) <= 16u;
  return mid || (fabs(z) < 0x1p-125 && z != 0.0);
}

// c = (float)(y / rs), the fp64 quotient rounded to fp32, for 8 values:
// from the product with irs = 1 / rs (within 2 fp64 units of the quotient),
// with the division itself only where that product cannot decide the
// rounding (behind a wave-level branch).
__device__ __forceinline__ void quot_f32(const double (&y)[8], double rs, double irs, float (&c)[8]) {
  uint32_t unsure = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const double w = y[e] * irs;
    c[e] = (float)w;
    unsure |= f32_round_unsure(w) ? 1u << e : 0u;
  }
  if (__builtin_amdgcn_ballot_w64(unsure != 0)) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (unsure & (1u << e)) c[e] = (float)__ddiv_rn(y[e], rs);
  }
}

// xn = (float)(x / rt), the correctly rounded fp32 quotient, for 8 values:
// from the fp64 product with 1 / rt (within 2 fp64 units of the quotient),
// with the division itself only where that product cannot decide the
// rounding (behind a wave-level branch).
__device__ __forceinline__ void div_f32(const float (&x)[8], float rt, float (&xn)[8]) {
  const double inv = __ddiv_rn(1.0, (double)rt);
  uint32_t unsure = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const double z = (double)x[e] * inv;
    xn[e] = (float)z;
    unsure |= f32_round_unsure(z) ? 1u << e : 0u;
  }
  if (__builtin_amdgcn_ballot_w64(unsure != 0)) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (unsure & (1u << e)) xn[e] = __fdiv_rn(x[e], rt);
  }
}

}  // namespace kvtc
