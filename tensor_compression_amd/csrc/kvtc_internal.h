// Internal declarations of libkvtc: container and workspace layouts, kernel
// parameter blocks and the launch functions implemented by the .hip files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvtc.h"

namespace kvtc {

constexpr uint32_t kRansL = 1u << 16;  // lower end of the normalised rANS state interval
constexpr int kHeaderBytes = 256;
constexpr int kDirEntry = 16;  // u64 offset, u32 size, u32 reserved

// Where each part of a container sits for a given T (all offsets in bytes
// from the container start).  Only the chunk records have data-dependent
// sizes; everything before chunks_off is fixed by the configuration and T.
struct Layout {
  int32_t T, s0, mid_begin, mid_end, T_mid, W_eff;
  int32_t n_sections, chunks_per_sec, n_chunks, tiles_per_chunk;
  int32_t n_r_sections;
  int32_t budget_k, budget_v;
  int64_t side_off, r_off, side_bytes, raw_off, raw_bytes, dir_off, chunks_off;
};

// Workspace carve-up (byte offsets from the workspace start).
struct WsLayout {
  int64_t status;      // u32 status, u32 exact re-computations, u64 container bytes
  int64_t part_sum;    // f64 [n_sections][chunks][D]
  int64_t part_sq;     // f64 [n_sections][chunks][D]
  int64_t part_min;    // f32 [n_sections][chunks][D]
  int64_t part_max;    // f32 [n_sections][chunks][D]
  int64_t sec_stats;   // f32x4 [n_sections][D]: mean, variance, min, max
  int64_t side_rcp;    // f32 [n_sections][D]
  int64_t side_zero;   // f32 [n_sections][D]
  int64_t side_bits;   // u8  [n_sections][D]
  int64_t packed;      // [n_chunks][packed_slot] packed tiles of each chunk
  int64_t packed_slot;
  int64_t rec;         // [n_chunks][rec_slot] encoder record slots
  int64_t rec_slot;
  int64_t tile_words_max;  // words capacity of one tile stream in a slot
  int64_t rec_size;    // u32 [n_chunks]
  int64_t rec_pos;     // u64 [n_chunks]
  int64_t kprime;      // bf16 [L][H][T_mid][D]: mid-region keys with RoPE removed (head_dim 128 bf16 path)
  int64_t total;
};

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
  int32_t sb, lanes, chunk_tokens, tile_tokens, basis_per_head, wht_keys;
  int32_t budget_k, budget_v;
  int32_t T, s0, mid_begin, mid_end, T_mid, W_eff, n_sections, chunks_per_sec, n_chunks,
      tiles_per_chunk;
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
};

// host helpers (kvtc_api.hip)
Layout make_layout(const kvtc_config& c, int32_t T);
WsLayout make_ws_layout(const kvtc_config& c, const Layout& lo);
int64_t max_container_bytes(const kvtc_config& c, const Layout& lo);
Params make_params(const PlanImpl& p, const Layout& lo, const WsLayout& w);
void build_header(const PlanImpl& p, const Layout& lo, uint8_t* hdr);

// launches (kernels_*.hip); each returns hipSuccess or the launch error
hipError_t launch_copy_raw(const Params& p, int to_container, hipStream_t s);
hipError_t launch_enc_transform(const Params& p, int mode, hipStream_t s);  // 0 stats, 1 quant
hipError_t launch_enc_alloc(const Params& p, hipStream_t s);
hipError_t launch_quant128(const Params& p, hipStream_t s);  // head_dim 128 bf16 PCA, tile % 64 == 0
hipError_t launch_rans_encode_chunks(const Params& p, hipStream_t s);
hipError_t launch_assemble(const Params& p, const uint8_t* hdr, hipStream_t s);
hipError_t launch_dec_check(const Params& p, const uint8_t* hdr, hipStream_t s);
hipError_t launch_rans_decode_chunks(const Params& p, hipStream_t s);
hipError_t launch_dec_transform(const Params& p, hipStream_t s);
hipError_t launch_coeffs(const Params& p, int sec_begin, int sec_end, float* out, float* r_out,
                         hipStream_t s);
hipError_t launch_test_rans_encode(const uint8_t* sym, int64_t N, const uint16_t* freq, int sb,
                                   int lanes, uint32_t* states, uint16_t* words, int64_t cap,
                                   int64_t* nwords, hipStream_t s);
hipError_t launch_test_rans_decode(const uint32_t* states, const uint16_t* words, int64_t nwords,
                                   const uint16_t* freq, int sb, int lanes, int64_t N,
                                   uint8_t* sym, int32_t* status, hipStream_t s);
hipError_t launch_test_freq(const uint32_t* counts, int sb, uint16_t* freq, hipStream_t s);
hipError_t launch_prep_basis(const float* src, void* basis_t, void* basis, int n_basis, int D,
                             int dtype, int32_t* bad, hipStream_t s);

// ---------------------------------------------------------------------------
// device helpers shared by the kernels
// ---------------------------------------------------------------------------

__host__ __device__ inline int64_t align16(int64_t x) { return (x + 15) & ~(int64_t)15; }

// Bytes of one packed tile of `ntok` tokens: a row of ceil(ntok*b/32) words
// per component with b > 0.
__device__ inline int32_t tile_row_words(int32_t ntok, int32_t b) { return (ntok * b + 31) >> 5; }

__device__ inline float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

__device__ inline uint16_t f32_to_bf16(float f) {
  __bf16 b = (__bf16)f;  // round to nearest even (v_cvt_pk_bf16_f32)
  return __builtin_bit_cast(uint16_t, b);
}

__device__ inline float round_bf16(float f) { return bf16_to_f32(f32_to_bf16(f)); }

__device__ inline void set_status(uint8_t* ws, const WsLayout& w, uint32_t code) {
  atomicOr(reinterpret_cast<uint32_t*>(ws + w.status), 1u << code);
}

__device__ inline uint32_t get_status(const uint8_t* ws, const WsLayout& w) {
  return __atomic_load_n(reinterpret_cast<const uint32_t*>(ws + w.status), __ATOMIC_RELAXED);
}

}  // namespace kvtc
