// Decode-side transform: unpack the channel-major tiles written by the rANS
// decoder, dequantise (c^ = fma(q, scale, zero), or (q - 2^(b-1)) scale for
// the symmetric key quantiser), undo the transform (X^ = B C^ on MFMA, or
// the orthonormal WHT times the stored RMS), re-apply RoPE to keys and store
// in the output dtype (Codec-Gauge "Problem Statement and Overview":
// Z^ = D(B_c), X^ = G^-1 Z^).
#include <type_traits>

#include <string.h>

#include "kvtc_internal.h"

namespace kvtc {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t extract_bits(const uint32_t* row, uint32_t bitpos, uint32_t nbits) {
  const uint32_t w = bitpos >> 5, sh = bitpos & 31;
  uint64_t v = (uint64_t)row[w] | ((uint64_t)row[w + 1] << 32);
  return (uint32_t)(v >> sh) & ((nbits >= 32) ? 0xffffffffu : ((1u << nbits) - 1u));
}

__device__ __forceinline__ void store_out(void* dst, int out_dtype, int64_t idx, float v) {
  if (out_dtype == KVTC_BF16) reinterpret_cast<uint16_t*>(dst)[idx] = f32_to_bf16(v);
  else reinterpret_cast<float*>(dst)[idx] = v;
}

// ---- PCA path ----------------------------------------------------------------
// Workgroup per chunk, 4 waves.  Per packed tile: stage the tile bytes in
// LDS, dequantise 64 tokens at a time into a bf16 (or fp32) token-major LDS
// tile, then each wave runs one 16-token MFMA block: lane (g, r) supplies
// token r and the component run [g D/4, (g+1) D/4) as the K slice; the
// basis rows (channel nb*16 + r, same component run) are register-resident.
// The result lane holds channel nb*16 + r of tokens 4g .. 4g+3, so RoPE
// pairs (j, j + D/2) are (nb, nb + D/32) in the same lane.

template <int D, int DT>
struct DecGeo {
  static constexpr int NB = D / 16;
  static constexpr int KPL = D / 4;                       // components per lane
  static constexpr int CS = DT == KVTC_BF16 ? D + 8 : D + 4;  // padded LDS row stride (elements)
};

template <int D, int DT>
__global__ __launch_bounds__(256) void k_dec_pca(const Params p) {
  constexpr int NB = DecGeo<D, DT>::NB, KPL = DecGeo<D, DT>::KPL, CS = DecGeo<D, DT>::CS;
  const int u = blockIdx.y, ch = blockIdx.x;
  const int h = u % p.H, s = (u / p.H) & 1, l = u / (2 * p.H);
  const int t0 = ch * p.blk_tokens;
  const int n = min(p.blk_tokens, p.T_mid - t0);
  if (n <= 0) return;
  if (get_status(p.ws, p.w) & (1u << KVTC_ERR_CORRUPT)) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, r = lane & 15;
  const bool rope = (s == 0) && p.rope_keys;
  void* dst = s ? p.v_out : p.k_out;
  const int64_t lh_row0 = ((int64_t)l * p.H + h) * p.T;

  __shared__ uint32_t s_bits[D], s_roww[D + 1];
  __shared__ float s_zero[D], s_scale[D];
  extern __shared__ uint32_t dyn[];
  const uint8_t* rec = p.in + p.side_off + (int64_t)u * 9 * D;
  if (tid < D) {
    s_bits[tid] = rec[tid];
    s_zero[tid] = reinterpret_cast<const float*>(rec + D)[tid];
    s_scale[tid] = reinterpret_cast<const float*>(rec + 5 * D)[tid];
  }
  __syncthreads();
  // dyn: [chat tile 64 x CS][out staging 4 x 16 x D][packed tile]
  using ctype = typename std::conditional<DT == KVTC_BF16, uint16_t, float>::type;
  ctype* chat = reinterpret_cast<ctype*>(dyn);
  const int chat_bytes = 64 * CS * (int)sizeof(ctype);
  const int ob = p.out_dtype == KVTC_BF16 ? 2 : 4;
  uint8_t* ostage = reinterpret_cast<uint8_t*>(dyn) + chat_bytes + wave * 16 * D * ob;
  uint32_t* ptile = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(dyn) + chat_bytes + 4 * 16 * D * ob);

  // register-resident basis rows: B[j = nb*16 + r][i = g*KPL + k]
  const int64_t bi = (p.basis_per_head ? ((int64_t)(l * 2 + s) * p.H + h) : (int64_t)(l * 2 + s)) * D * D;
  uint4 bq[DT == KVTC_BF16 ? NB : 1][DT == KVTC_BF16 ? KPL / 8 : 1];
  float bf[DT == KVTC_FP32 ? NB : 1][DT == KVTC_FP32 ? KPL : 1];
  if constexpr (DT == KVTC_BF16) {
    const uint16_t* B = reinterpret_cast<const uint16_t*>(p.basis) + bi;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int kb = 0; kb < KPL / 8; ++kb)
        bq[nb][kb] = *reinterpret_cast<const uint4*>(B + (int64_t)(nb * 16 + r) * D + g * KPL + kb * 8);
  } else {
    const float* B = reinterpret_cast<const float*>(p.basis) + bi;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int k = 0; k < KPL; ++k) bf[nb][k] = B[(int64_t)(nb * 16 + r) * D + g * KPL + k];
  }

  // bytes of a full tile: every tile but the section's last starts at t * full
  __shared__ uint32_t s_full;
  if (tid < 64) {
    uint32_t v0 = 0;
    for (int i = lane; i < D; i += 64) v0 += (uint32_t)((p.tile_tokens * (int)s_bits[i] + 31) >> 5);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v0 += __shfl_xor(v0, o, 64);
    if (lane == 0) s_full = v0;
  }
  __syncthreads();
  const uint32_t* slot = reinterpret_cast<const uint32_t*>(p.ws + p.w.packed + (int64_t)(u * p.blks_per_sec + ch) * p.w.packed_slot);
  // dequantisation role: fixed component per thread
  const int di = tid % D;
  const uint32_t db = s_bits[di];
  const float dz = s_zero[di], dsc = s_scale[di];
  const int ntiles = (n + p.tile_tokens - 1) / p.tile_tokens;
  for (int tl = 0; tl < ntiles; ++tl) {
    const int ta = tl * p.tile_tokens;
    const int nt = min(p.tile_tokens, n - ta);
    if (tid < 64) {
      uint32_t w0 = 0, w1 = 0;
      const int i0 = 2 * lane, i1 = 2 * lane + 1;
      if (i0 < D) w0 = (uint32_t)((nt * (int)s_bits[i0] + 31) >> 5);
      if (i1 < D) w1 = (uint32_t)((nt * (int)s_bits[i1] + 31) >> 5);
      uint32_t x = w0 + w1;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        uint32_t y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
      }
      const uint32_t ex = x - (w0 + w1);
      if (i0 < D) s_roww[i0] = ex;
      if (i1 < D) s_roww[i1] = ex + w0;
      if (lane == 63) s_roww[D] = x;
    }
    __syncthreads();
    const uint32_t tw = s_roww[D];
    const uint32_t* src = slot + (int64_t)tl * s_full;
    for (uint32_t i = tid; i < tw; i += blockDim.x) ptile[i] = src[i];
    if (tid == 0) ptile[tw] = 0;  // extraction reads one word past a row
    __syncthreads();
    const uint32_t myrow = s_roww[di];
    for (int sb0 = 0; sb0 < nt; sb0 += 64) {
      const int ns = min(64, nt - sb0);
      // dequantise 64 tokens: thread (component di, token groups of 4)
      for (int tg = tid / D; tg < 16; tg += 256 / D) {
        const int tk = sb0 + 4 * tg;
        float v[4];
        uint32_t codes = 0;
        if (db > 0 && tk < nt) codes = extract_bits(ptile + myrow, (uint32_t)tk * db, 4 * db);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t q = db > 0 ? (codes >> (e * db)) & ((1u << db) - 1u) : 0u;
          v[e] = __fmaf_rn((float)q, dsc, dz);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if constexpr (DT == KVTC_BF16) chat[(4 * tg + e) * CS + di] = f32_to_bf16(v[e]);
          else chat[(4 * tg + e) * CS + di] = v[e];
        }
      }
      __syncthreads();
      // MFMA: wave w takes tokens [16 w, 16 w + 16) of the 64
      const int blk0 = 16 * wave;
      if (blk0 < ns) {
        f32x4_t acc[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if constexpr (DT == KVTC_BF16) {
#pragma unroll
          for (int kb = 0; kb < KPL / 8; ++kb) {
            uint4 a = *reinterpret_cast<const uint4*>(chat + (blk0 + r) * CS + g * KPL + kb * 8);
            bf16x8_t av = __builtin_bit_cast(bf16x8_t, a);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
              acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8_t, bq[nb][kb]), acc[nb], 0, 0, 0);
          }
        } else {
#pragma unroll
          for (int k = 0; k < KPL; ++k) {
            float av = chat[(blk0 + r) * CS + g * KPL + k];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
              acc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bf[nb][k], acc[nb], 0, 0, 0);
          }
        }
        // RoPE forward on keys, then the output cast into the staging tile
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int tk = blk0 + 4 * g + e;  // token within the 64
          const int pos = p.mid_begin + t0 + ta + sb0 + tk;
          float x[NB];
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) x[nb] = acc[nb][e];
          if (rope && sb0 + tk < nt) {
            const float2* rr = p.rope + (int64_t)pos * (D / 2);
            if (p.rope_style == KVTC_ROPE_HALF) {
#pragma unroll
              for (int nb = 0; nb < NB / 2; ++nb) {
                float2 cs = rr[nb * 16 + r];
                float xa = x[nb], xb = x[nb + NB / 2];
                float xb_s = __fmul_rn(xb, cs.y), xb_c = __fmul_rn(xb, cs.x);
                x[nb] = __fmaf_rn(xa, cs.x, -xb_s);
                x[nb + NB / 2] = __fmaf_rn(xa, cs.y, xb_c);
              }
            } else {
#pragma unroll
              for (int nb = 0; nb < NB; ++nb) {
                float other = __shfl_xor(x[nb], 1, 64);
                float2 cs = rr[(nb * 16 + r) >> 1];
                const bool first = (r & 1) == 0;
                float xa = first ? x[nb] : other, xb = first ? other : x[nb];
                float xb_s = __fmul_rn(xb, cs.y), xb_c = __fmul_rn(xb, cs.x);
                x[nb] = first ? __fmaf_rn(xa, cs.x, -xb_s) : __fmaf_rn(xa, cs.y, xb_c);
              }
            }
          }
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            const int jj = (4 * g + e) * D + nb * 16 + r;
            if (p.out_dtype == KVTC_BF16) reinterpret_cast<uint16_t*>(ostage)[jj] = f32_to_bf16(x[nb]);
            else reinterpret_cast<float*>(ostage)[jj] = x[nb];
          }
        }
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __builtin_amdgcn_wave_barrier();
        // coalesced store of the wave's 16 rows
        const int row_u4 = D * ob / 16;
        for (int idx = lane; idx < 16 * row_u4; idx += 64) {
          const int rr2 = idx / row_u4, cc = idx % row_u4;
          const int tk = blk0 + rr2;
          if (tk < ns) {
            const int pos = p.mid_begin + t0 + ta + sb0 + tk;
            uint8_t* drow = reinterpret_cast<uint8_t*>(dst) + ((lh_row0 + pos) * D) * ob;
            reinterpret_cast<uint4*>(drow)[cc] = reinterpret_cast<const uint4*>(ostage + rr2 * D * ob)[cc];
          }
        }
      }
      __syncthreads();
    }
  }
}

// ---- WHT path ------------------------------------------------------------------
// 16 lanes per token; lane q holds components 8q .. 8q+7.

__global__ __launch_bounds__(256) void k_dec_wht(const Params p) {
  constexpr int D = 128;
  const int u = blockIdx.y, ch = blockIdx.x;
  const int h = u % p.H, s = (u / p.H) & 1, l = u / (2 * p.H);
  const int t0 = ch * p.blk_tokens;
  const int n = min(p.blk_tokens, p.T_mid - t0);
  if (n <= 0) return;
  if (get_status(p.ws, p.w) & (1u << KVTC_ERR_CORRUPT)) return;
  const int tid = threadIdx.x, q = tid & 15, grp = tid >> 4;
  const bool rope = (s == 0) && p.rope_keys;
  const bool transform = (s == 1) || p.wht_keys;
  const bool sym = s == 0;
  void* dst = s ? p.v_out : p.k_out;
  const int64_t lh_row0 = ((int64_t)l * p.H + h) * p.T;
  const uint8_t* rec = p.in + p.side_off + (int64_t)u * 9 * D;
  const uint32_t b = rec[0];
  float zr[8], sc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    zr[e] = reinterpret_cast<const float*>(rec + D)[8 * q + e];
    sc[e] = reinterpret_cast<const float*>(rec + 5 * D)[8 * q + e];
  }
  const int64_t r_index = !transform ? -1 : (p.wht_keys ? (int64_t)u : (int64_t)l * p.H + h);
  const float* rarea = reinterpret_cast<const float*>(p.in + p.r_off);
  const uint32_t* slot = reinterpret_cast<const uint32_t*>(p.ws + p.w.packed + (int64_t)(u * p.blks_per_sec + ch) * p.w.packed_slot);
  const uint32_t full_row = (uint32_t)((p.tile_tokens * (int)b + 31) >> 5);
  const int ntiles = (n + p.tile_tokens - 1) / p.tile_tokens;
  for (int tl = 0; tl < ntiles; ++tl) {
    const int ta = tl * p.tile_tokens;
    const int nt = min(p.tile_tokens, n - ta);
    const uint32_t row_words = (uint32_t)((nt * (int)b + 31) >> 5);
    const uint32_t* tile = slot + (int64_t)tl * full_row * D;
    for (int tb = grp; tb < nt; tb += 16) {
      const int tok = ta + tb;
      const int pos = p.mid_begin + t0 + tok;
      float c[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = 8 * q + e;
        const uint32_t* row = tile + (int64_t)i * row_words;
        const uint32_t bitpos = (uint32_t)tb * b;
        const uint32_t w = bitpos >> 5, sh = bitpos & 31;
        uint64_t v = (uint64_t)row[w];
        if (sh + b > 32) v |= (uint64_t)row[w + 1] << 32;
        const uint32_t code = (uint32_t)(v >> sh) & ((1u << b) - 1u);
        if (sym) c[e] = __fmul_rn((float)((int)code - (1 << (b - 1))), sc[e]);
        else c[e] = __fmaf_rn((float)code, sc[e], zr[e]);
      }
      float x[8];
      if (transform) {
        double y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = (double)c[e];
        wht_fp64(y, q);  // channel strides 1, 2, 4 in the lane, then 8 .. 64 across the row
        const double rs = __dsqrt_rn((double)D);
        const float rt = rarea[r_index * p.T_mid + t0 + tok];
        quot_f32(y, rs, __ddiv_rn(1.0, rs), x);  // y / sqrt(D), exactly rounded
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = __fmul_rn(x[e], rt);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = c[e];
      }
      if (rope) {
        const float2* rr = p.rope + (int64_t)pos * (D / 2);
        if (p.rope_style == KVTC_ROPE_HALF) {
          float pr[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) pr[e] = __shfl_xor(x[e], 8, 16);
          const bool lower = q < 8;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            float2 cs = rr[8 * (q & 7) + e];
            float xa = lower ? x[e] : pr[e], xb = lower ? pr[e] : x[e];
            float xb_s = __fmul_rn(xb, cs.y), xb_c = __fmul_rn(xb, cs.x);
            x[e] = lower ? __fmaf_rn(xa, cs.x, -xb_s) : __fmaf_rn(xa, cs.y, xb_c);
          }
        } else {
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            float2 cs = rr[4 * q + m];
            float xa = x[2 * m], xb = x[2 * m + 1];
            float xb_s = __fmul_rn(xb, cs.y), xb_c = __fmul_rn(xb, cs.x);
            x[2 * m] = __fmaf_rn(xa, cs.x, -xb_s);
            x[2 * m + 1] = __fmaf_rn(xa, cs.y, xb_c);
          }
        }
      }
      const int64_t base = (lh_row0 + pos) * D + 8 * q;
      if (p.out_dtype == KVTC_BF16) {
        uint4 o;
        o.x = (uint32_t)f32_to_bf16(x[0]) | ((uint32_t)f32_to_bf16(x[1]) << 16);
        o.y = (uint32_t)f32_to_bf16(x[2]) | ((uint32_t)f32_to_bf16(x[3]) << 16);
        o.z = (uint32_t)f32_to_bf16(x[4]) | ((uint32_t)f32_to_bf16(x[5]) << 16);
        o.w = (uint32_t)f32_to_bf16(x[6]) | ((uint32_t)f32_to_bf16(x[7]) << 16);
        store_out16(reinterpret_cast<uint16_t*>(dst) + base, o);
      } else {
        float* d = reinterpret_cast<float*>(dst) + base;
        store_out16(d, make_float4(x[0], x[1], x[2], x[3]));
        store_out16(d + 4, make_float4(x[4], x[5], x[6], x[7]));
      }
    }
  }
}

// ---- head_dim 128, bf16 cache: the bandwidth-oriented decode pass -------------
// A workgroup (four waves) per chunk; the chunk's packed tiles are staged in
// LDS one at a time and decoded in 64-token sub-tiles, all four waves on the
// same sub-tile.  The workgroup prologue reads the section's side
// information, orders the components with codes (b > 0) by bit width (the
// contraction runs over this order) and folds the b = 0 components, whose
// value is their zero point, into a per-channel constant that seeds the
// accumulators.
//
// Dequantisation (all 256 threads): lane = token, one component octet per
// wave at a time, so the width and constants of each component are
// wave-uniform; the eight bf16 values of the octet go to LDS as one 16-byte
// MFMA operand, laid out [K slice][16-token group][lane group][token].
//
// MFMA: D^T = B^T C^T with the basis rows (permuted channel order) in
// registers.  Wave w takes the channel half hf = w & 1 (channel runs hf and
// hf + 2 of 32, so both members of every RoPE pair) and the 16-token groups
// 2 (w >> 1), +1 of the sub-tile; the result lane holds eight consecutive
// channels of one token per run and leaves with 16-byte stores.

constexpr int kBS = 136;  // LDS row stride (bf16) of the staged basis

struct DecKInfo {  // per component in the sorted order
  uint32_t b, idx;
  float scale, zero;
};

typedef __attribute__((address_space(3))) const uint32_t lds_word_t;
typedef __attribute__((address_space(3))) const uint8_t lds_byte_t;

__device__ __forceinline__ uint32_t lds_u32(const uint32_t* base, uint32_t byte_off) {
  return *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(base) + byte_off);
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Decoded rows are stored non-temporally (the cache policy's nt bit): nothing
// in the codec reads them again, and streaming them past the caches keeps
// the packed tiles that later workgroups read in the memory-side cache.
constexpr int kNtStore = 2;
// The packed tiles are read here for the last time: their direct-to-LDS
// loads carry the same policy.
constexpr int kNtLoad = 2;

// two fp32 values rounded to bf16 (nearest even) in one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

// Words of the LDS tile buffer: the packed tile and four zero words past it.
__host__ __device__ inline int dec_tile_words(const Params& p) {
  const int32_t bmax = p.sec_bits_max;
  return (int)(((int64_t)p.tile_tokens * bmax + 31) / 32) + 4;
}

// The section's coded components by width: KB K slices of 32 (entries past
// the coded components are zero).  KBMAX = 3 serves sections with at most 96
// coded components, KBMAX = 4 the rest; each instantiation leaves the other's
// sections alone.  PG: the output is a paged pool (bf16) addressed through
// the page table; lanes past the section store to a scratch row of the
// workspace.  OB: output bytes per element.
template <int KB, int KBMAX, int OB, bool PG>
__device__ __forceinline__ void dec_chunk128(const Params& p, int u, int ch, const uint4 (&A)[4][KBMAX],
                                             uint4* cq, uint32_t* tb, uint4* s_kw, const DecKInfo* s_ki,
                                             const uint8_t* s_rank, const uint32_t* s_b, const float* s_const,
                                             uint32_t fw, uint4* stage, bool pf0) {
  constexpr int D = 128;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = wave & 1, th = wave >> 1;
  const int h = u % p.H, s = (u / p.H) & 1, l = u / (2 * p.H);
  const int t0 = ch * p.blk_tokens;
  const int n = min(p.blk_tokens, p.T_mid - t0);
  const bool rope = (s == 0) && p.rope_keys;
  const bool half_style = p.rope_style == KVTC_ROPE_HALF;
  const int64_t lh_row0 = ((int64_t)l * p.H + h) * p.T;
  // the (layer, head) slab of the output as a buffer resource: stores of
  // tokens past the section get an offset at the slab end and are dropped by
  // the range check, so every store instruction is issued unconditionally
  uint8_t* obase = reinterpret_cast<uint8_t*>(s ? p.v_out : p.k_out);
  uint8_t* slab = obase + (PG ? 0 : lh_row0 * D * OB);
  const int32_t slab_bytes = PG ? 0 : p.T * D * OB;
  uint8_t* const dummy = p.ws + p.w.fixed;  // PG: scratch row for tokens past the section
  const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(slab, 0, slab_bytes, 0x00020000);
  // the RoPE table as a buffer resource (one offset register per load)
  const __amdgpu_buffer_rsrc_t rrsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float2*>(p.rope), 0, rope ? p.T * 512 : 0, 0x00020000);
  const uint32_t* slot = reinterpret_cast<const uint32_t*>(p.ws + p.w.packed + (int64_t)(u * p.blks_per_sec + ch) * p.w.packed_slot);

  // widths of this wave's octets (sorted positions 8 c8 .. +7, c8 = 4 j8 +
  // wave), one byte each: the single width of the octet, 0 when it holds no
  // coded component, 0xff when its widths differ.  Widths ascend along the
  // sorted order with the uncoded entries last, so the first and last entry
  // decide.
  uint32_t oct_w = 0u;
#pragma unroll
  for (int j8 = 0; j8 < KB; ++j8) {
    const int c8 = 4 * j8 + wave;
    const uint32_t bf = __builtin_amdgcn_readfirstlane(s_ki[8 * c8].b);
    const uint32_t bl = __builtin_amdgcn_readfirstlane(s_ki[8 * c8 + 7].b);
    oct_w |= (bf == bl ? bf : 0xffu) << (8 * j8);
  }
  // Two tile buffers: the next tile is loaded straight into the other one
  // (no registers) once the current tile's last dequantisation is done, and
  // waited for at its start.
  // (tile 0 in the second buffer: it may have been loaded during the set-up,
  // pf0)
  uint32_t* const tb2 = reinterpret_cast<uint32_t*>(stage + 64 * 17);
  bool pf = pf0;  // the current tile's 16-byte words were loaded ahead
  auto tile_words = [&](int ntok) -> uint32_t {
    uint32_t w = ((uint32_t)(ntok * (int)s_b[2 * lane] + 31) >> 5) + ((uint32_t)(ntok * (int)s_b[2 * lane + 1] + 31) >> 5);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) w += __shfl_xor(w, o, 64);
    return w;
  };
  for (int ta = 0; ta < n; ta += p.tile_tokens) {
    const int nt = min(p.tile_tokens, n - ta);
    uint32_t* const tbc = ((ta / p.tile_tokens) & 1) ? tb : tb2;
    lds_barrier();  // the previous tile's buffer and operands are consumed
    // row offsets of this tile (natural order, scanned), stored by sorted
    // position together with the width and the dequantisation constants;
    // components without codes keep all-zero entries
    uint32_t tw;
    {
      const uint32_t b0 = s_b[2 * lane], b1 = s_b[2 * lane + 1];
      const uint32_t w0 = (uint32_t)(nt * (int)b0 + 31) >> 5, w1 = (uint32_t)(nt * (int)b1 + 31) >> 5;
      uint32_t x = w0 + w1;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
      }
      tw = __shfl(x, 63, 64);
      if (wave == 0) {
        const uint32_t ex = x - (w0 + w1);
        const uint32_t r0 = s_rank[2 * lane], r1 = s_rank[2 * lane + 1];
        const DecKInfo i0 = s_ki[r0], i1 = s_ki[r1];
        s_kw[r0] = b0 ? make_uint4(b0, 4u * ex, __float_as_uint(i0.scale), __float_as_uint(i0.zero)) : make_uint4(0, 0, 0, 0);
        s_kw[r1] = b1 ? make_uint4(b1, 4u * (ex + w0), __float_as_uint(i1.scale), __float_as_uint(i1.zero)) : make_uint4(0, 0, 0, 0);
      }
    }
    // stage the packed tile (tile stride fw words in the slot; tw is a
    // multiple of 4 when the tile is full, whose slots are 16-byte aligned)
    {
      const uint32_t* src = slot + (int64_t)(ta / p.tile_tokens) * fw;
      const bool al = ((reinterpret_cast<uintptr_t>(src) & 15u) == 0);
      const uint32_t n4 = al ? tw >> 2 : 0u;
      if (pf) {
        __builtin_amdgcn_s_waitcnt(0);  // this wave's direct loads of the tile have landed
      } else {
        for (uint32_t i = tid; i < n4; i += 256) reinterpret_cast<uint4*>(tbc)[i] = reinterpret_cast<const uint4*>(src)[i];
      }
      for (uint32_t i = 4 * n4 + tid; i < tw; i += 256) tbc[i] = src[i];
      if (tid < 4) tbc[tw + tid] = 0u;
    }
    pf = false;
    lds_barrier();

    lds_byte_t* const tb3 = (lds_byte_t*)tbc;  // the tile buffer in the LDS address space
    for (int sub = 0; sub * 64 < nt; ++sub) {
      // RoPE table entries of this wave's two 16-token groups, in flight
      // during the dequantisation (a row is 64 pairs of cos, sin: 512 bytes;
      // half style: pairs 32 hf + 8 g + 2 x, +1; interleaved: pairs
      // 16 pp + 4 g + 2 (x & 1), +1 with pp = hf + 2 (x >> 1))
      float4 cs[2][4];
      if (rope) {
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          const int pos = p.mid_begin + t0 + ta + sub * 64 + (2 * th + k2) * 16 + r;
          const int32_t crow = min(pos, p.T - 1) * 512;
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const int pr = half_style ? 32 * hf + 8 * g + 2 * x : 16 * (hf + 2 * (x >> 1)) + 4 * g + 2 * (x & 1);
            cs[k2][x] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rrsrc, crow + 8 * pr, 0, 0));
          }
        }
      }
      // ---- dequantise: lane = token sub*64 + lane of the tile, octets w, w+4, ...
      // One wave-uniform branch per octet on its width class (one width,
      // mixed widths, no coded component); inside an octet every component
      // is branch-free (entries past the coded components are all zero and
      // yield 0), so its table and code-word reads are issued together.
#pragma unroll 1
      for (int j8 = 0; j8 < KB; ++j8) {
        const int c8 = 4 * j8 + wave;
        const uint32_t bf = (oct_w >> (8 * j8)) & 0xffu;
        uint32_t w4[4] = {0u, 0u, 0u, 0u};
        if (bf != 0xffu && bf != 0u) {
          // one width: the lane's bit position and word offset are shared by
          // the eight rows; per code one add, one or two LDS words, extract,
          // convert, fma (offsets and constants stay in vector registers)
          const uint32_t bpos = __umul24((uint32_t)lane, bf);
          const lds_byte_t* const lb = tb3 + 8u * bf * (uint32_t)sub + ((bpos >> 5) << 2);
          uint32_t x[8];
          float sc[8], zr[8];
          if ((bf & (bf - 1u)) == 0u) {  // 1, 2, 4, 8 bits: a code never straddles two words
#pragma unroll
            for (int z = 0; z < 8; ++z) {
              const uint4 ki = s_kw[8 * c8 + z];
              x[z] = *(const lds_word_t*)(lb + ki.y);
              sc[z] = __uint_as_float(ki.z);
              zr[z] = __uint_as_float(ki.w);
            }
#pragma unroll
            for (int z = 0; z < 8; ++z) x[z] = __builtin_amdgcn_ubfe(x[z], bpos & 31u, bf);
          } else {
            uint32_t hi[8];
#pragma unroll
            for (int z = 0; z < 8; ++z) {
              const uint4 ki = s_kw[8 * c8 + z];
              const lds_word_t* wp = (const lds_word_t*)(lb + ki.y);
              x[z] = wp[0];
              hi[z] = wp[1];
              sc[z] = __uint_as_float(ki.z);
              zr[z] = __uint_as_float(ki.w);
            }
#pragma unroll
            for (int z = 0; z < 8; ++z) x[z] = __builtin_amdgcn_ubfe(__builtin_amdgcn_alignbit(hi[z], x[z], bpos), 0u, bf);
          }
#pragma unroll
          for (int q2 = 0; q2 < 4; ++q2)
            w4[q2] = pk_bf16(__fmaf_rn((float)x[2 * q2], sc[2 * q2], zr[2 * q2]),
                             __fmaf_rn((float)x[2 * q2 + 1], sc[2 * q2 + 1], zr[2 * q2 + 1]));
        } else if (bf == 0xffu) {
          // mixed widths: per row width, offsets and constants (wave-uniform),
          // then all eight code-word pairs in flight before any is used
          uint32_t bw[8], bp[8], lo[8], hi[8];
          float sc[8], zr[8];
#pragma unroll
          for (int z = 0; z < 8; ++z) {
            const uint4 ki = s_kw[8 * c8 + z];
            bw[z] = __builtin_amdgcn_readfirstlane(ki.x);
            const uint32_t seg = __builtin_amdgcn_readfirstlane(ki.y) + 8u * bw[z] * (uint32_t)sub;
            sc[z] = __uint_as_float(__builtin_amdgcn_readfirstlane(ki.z));
            zr[z] = __uint_as_float(ki.w);  // uniform; the fma takes it from a vector register
            bp[z] = __umul24((uint32_t)lane, bw[z]);
            // the row segment's first word (uniform LDS address) plus this lane's word
            const lds_word_t* wp = (const lds_word_t*)(tb3 + seg) + (bp[z] >> 5);
            lo[z] = wp[0];
            hi[z] = wp[1];
          }
#pragma unroll
          for (int q2 = 0; q2 < 4; ++q2) {
            float v[2];
#pragma unroll
            for (int z2 = 0; z2 < 2; ++z2) {
              const int z = 2 * q2 + z2;
              const uint32_t q = __builtin_amdgcn_ubfe(__builtin_amdgcn_alignbit(hi[z], lo[z], bp[z]), 0u, bw[z]);
              v[z2] = __fmaf_rn((float)q, sc[z], zr[z]);
            }
            w4[q2] = pk_bf16(v[0], v[1]);
          }
        }
        // operand slot [kb = c8 / 4][kk = lane / 16][g = c8 % 4][r = lane % 16]
        cq[((c8 >> 2) * 4 + (lane >> 4)) * 64 + (c8 & 3) * 16 + (lane & 15)] = make_uint4(w4[0], w4[1], w4[2], w4[3]);
      }
      lds_barrier();
      if ((sub + 1) * 64 >= nt && ta + p.tile_tokens < n) {
        // the other buffer held the previous tile, consumed before this one
        // started: the next tile's 16-byte words go there directly
        const uint32_t* nsrc = slot + (int64_t)(ta / p.tile_tokens + 1) * fw;
        if ((reinterpret_cast<uintptr_t>(nsrc) & 15u) == 0) {
          const uint32_t n4n = tile_words(min(p.tile_tokens, n - ta - p.tile_tokens)) >> 2;
          uint32_t* const tbn = tbc == tb ? tb2 : tb;
          for (uint32_t c = (uint32_t)wave; c * 64 < n4n; c += 4)
            if (c * 64 + (uint32_t)lane < n4n)
              __builtin_amdgcn_global_load_lds(
                  (const void __attribute__((address_space(1)))*)(nsrc + 4 * (c * 64 + lane)),
                  (void __attribute__((address_space(3)))*)(tbn + 256 * c), 16, 0, kNtLoad);
          pf = true;
        }
      }
      // ---- MFMA, RoPE, store: this wave's two 16-token groups
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        // one group at a time (bounds the registers in flight)
        __builtin_amdgcn_sched_barrier(0);
        const int kk = 2 * th + k2;
        const int tok = sub * 64 + kk * 16 + r;  // tile-relative
        const bool valid = tok < nt;
        const int pos = p.mid_begin + t0 + ta + tok;
        // RoPE table entries of this lane's eight pairs (token clamped into the cache)
        // accumulator seeds: channel 32 pp + 8 g + 4 a + e of tile mi = (pp, a)
        f32x4_t acc[4];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
          const int pp = hf + 2 * (mi >> 1), a = mi & 1;
          const float4 c4 = *reinterpret_cast<const float4*>(&s_const[32 * pp + 8 * g + 4 * a]);
          acc[mi] = f32x4_t{c4.x, c4.y, c4.z, c4.w};
        }
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const uint4 bq = cq[(kb * 4 + kk) * 64 + lane];
          const bf16x8_t bop = __builtin_bit_cast(bf16x8_t, bq);
#pragma unroll
          for (int mi = 0; mi < 4; ++mi)
            acc[mi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, A[mi][kb]), bop, acc[mi], 0, 0, 0);
        }
        if (rope) {
          if (half_style) {
            // pair j = 32 hf + 8 g + 4 a + e: x_a = acc[a][e], x_b = acc[2 + a][e]
#pragma unroll
            for (int a = 0; a < 2; ++a) {
              const float4 c01 = cs[k2][2 * a], c23 = cs[k2][2 * a + 1];
              const float cc[4] = {c01.x, c01.z, c23.x, c23.z}, ss[4] = {c01.y, c01.w, c23.y, c23.w};
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const float xa = acc[a][e], xb = acc[2 + a][e];
                acc[a][e] = __fmaf_rn(xa, cc[e], -__fmul_rn(xb, ss[e]));
                acc[2 + a][e] = __fmaf_rn(xa, ss[e], __fmul_rn(xb, cc[e]));
              }
            }
          } else {
            // pairs (e, e + 1) of tile (pp, a): index 16 pp + 4 g + 2 a + e / 2
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) {
              const float4 c4 = cs[k2][mi];
              const float cc[2] = {c4.x, c4.z}, ss[2] = {c4.y, c4.w};
#pragma unroll
              for (int e2 = 0; e2 < 2; ++e2) {
                const float xa = acc[mi][2 * e2], xb = acc[mi][2 * e2 + 1];
                acc[mi][2 * e2] = __fmaf_rn(xa, cc[e2], -__fmul_rn(xb, ss[e2]));
                acc[mi][2 * e2 + 1] = __fmaf_rn(xa, ss[e2], __fmul_rn(xb, cc[e2]));
              }
            }
          }
        }
        if constexpr (OB == 2) {
          // bf16 rows go through LDS (row = 16 units of 16 bytes, stride 17
          // units against bank conflicts): this
          // wave's two 64-byte runs per token now, whole rows below
#pragma unroll
          for (int pq = 0; pq < 2; ++pq) {
            const int pp = hf + 2 * pq;
            const f32x4_t x0 = acc[2 * pq], x1 = acc[2 * pq + 1];
            stage[(kk * 16 + r) * 17 + 4 * pp + g] =
                make_uint4(pk_bf16(x0[0], x0[1]), pk_bf16(x0[2], x0[3]), pk_bf16(x1[0], x1[1]), pk_bf16(x1[2], x1[3]));
          }
        } else {
          const int32_t vo = valid ? (int32_t)(((int64_t)pos * D) * OB) : slab_bytes;
#pragma unroll
          for (int pq = 0; pq < 2; ++pq) {
            const int pp = hf + 2 * pq;
            const f32x4_t x0 = acc[2 * pq], x1 = acc[2 * pq + 1];
            const int c0 = 32 * pp + 8 * g;
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, x0), orsrc, vo + 4 * c0, 0, kNtStore);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, x1), orsrc, vo + 4 * c0 + 16, 0, kNtStore);
          }
        }
      }
      if constexpr (OB == 2) {
        lds_barrier();  // the sub-tile's rows are complete in LDS
        // whole rows: wave w stores tokens 16 w .. 16 w + 15, four rows per
        // instruction (lane = row l / 16, unit l % 16)
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const int rr = 16 * wave + 4 * it + (lane >> 4), un = lane & 15;
          const uint4 v = stage[rr * 17 + un];
          const int tok = sub * 64 + rr;
          const bool valid = tok < nt;
          const int pos = p.mid_begin + t0 + ta + tok;
          if constexpr (PG) {
            const int64_t page = p.page_row[min(pos, p.T - 1) >> 4];
            uint8_t* rowp = valid ? obase + ((((page + (int64_t)l * p.pool_pages) * p.H + h) << 4) + (pos & 15)) * D * 2
                                  : dummy;
            store_out16(rowp + 16 * un, v);
          } else {
            const int32_t vo = valid ? (int32_t)((int64_t)pos * D * 2) : slab_bytes;
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), orsrc, vo + 16 * un, 0, kNtStore);
          }
        }
      }
      lds_barrier();  // the operands of this sub-tile are consumed
    }
  }
}

template <int KBMAX, bool PG>
__global__ __launch_bounds__(256, 3) void k_dec_pca128(const Params p0) {
  const Params p = at_seq(p0, blockIdx.z);
  constexpr int D = 128;
  const int u = blockIdx.y, ch = blockIdx.x;
  if (ch >= p.blks_per_sec) return;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = u % p.H, s = (u / p.H) & 1, l = u / (2 * p.H);
  if (min(p.blk_tokens, p.T_mid - ch * p.blk_tokens) <= 0) return;

  __shared__ DecKInfo s_ki[D];
  __shared__ uint4 s_kw[D];          // sorted order: {b, row byte offset in the tile, scale, zero}
  __shared__ uint8_t s_rank[D];      // natural component -> sorted position
  __shared__ __attribute__((aligned(16))) float s_const[D];
  __shared__ __attribute__((aligned(16))) float s_zr[D];  // bf16-rounded zero points, sorted order
  __shared__ uint32_t s_b[D];
  __shared__ int32_t s_misc[4];      // [1] corrupt flag, [2] full tile words
  // dynamic: [MFMA operands of the sub-tile: KBMAX x 4 KB][tile buffer][bf16
  // output rows of the sub-tile: 64 x 272 bytes], the staged basis (prologue)
  // overlaying them
  extern __shared__ __attribute__((aligned(16))) uint32_t dlds[];
  uint4* cq = reinterpret_cast<uint4*>(dlds);
  uint32_t* tb = dlds + KBMAX * 4 * 64 * 4;
  uint4* stage = reinterpret_cast<uint4*>(tb + ((dec_tile_words(p) + 3) & ~3));  // 64 rows x 17 units

  if (tid == 0) s_misc[1] = (int32_t)((get_status(p.ws, p.w) >> KVTC_ERR_CORRUPT) & 1u);
  const uint8_t* rec = p.in + p.side_off + (int64_t)u * 9 * D;
  if (tid < D) s_b[tid] = min((uint32_t)rec[tid], 8u);
  __syncthreads();
  if (s_misc[1]) return;
  // coded components (every wave counts them): the variant for this section
  const int nnz = (int)(__popcll(__ballot(s_b[lane] != 0u)) + __popcll(__ballot(s_b[lane + 64] != 0u)));
  const int KB = (nnz + 31) >> 5;
  if ((KBMAX == 3) != (KB <= 3)) return;
  // the basis rows (channel-major, operand precision) in flight during the sort
  const int64_t bidx = (p.basis_per_head ? ((int64_t)(l * 2 + s) * p.H + h) : (int64_t)(l * 2 + s)) * D * D;
  const uint16_t* bsrc = reinterpret_cast<const uint16_t*>(p.basis) + bidx;
  uint4 brow8[8];
#pragma unroll
  for (int it = 0; it < 8; ++it)
    brow8[it] = *reinterpret_cast<const uint4*>(bsrc + (it * 16 + (tid >> 4)) * D + (tid & 15) * 8);
  if (wave == 0) {
    // counting sort of the components by width, b = 0 last
    const uint32_t b0 = s_b[2 * lane], b1 = s_b[2 * lane + 1];
    const uint32_t k0 = b0 ? b0 : 9u, k1 = b1 ? b1 : 9u;
    const uint64_t lt = (1ull << lane) - 1ull;
    uint32_t base = 0, r0 = 0, r1 = 0;
    for (uint32_t v = 1; v <= 9; ++v) {
      const uint64_t m0 = __ballot(k0 == v), m1 = __ballot(k1 == v);
      const uint32_t before = base + __popcll(m0 & lt) + __popcll(m1 & lt);
      if (k0 == v) r0 = before;
      if (k1 == v) r1 = before + (k0 == v ? 1u : 0u);
      base += __popcll(m0) + __popcll(m1);
    }
    s_rank[2 * lane] = (uint8_t)r0;
    s_rank[2 * lane + 1] = (uint8_t)r1;
    const float* zr = reinterpret_cast<const float*>(rec + D);
    const float* sc = reinterpret_cast<const float*>(rec + 5 * D);
    s_ki[r0] = DecKInfo{b0, (uint32_t)(2 * lane), sc[2 * lane], zr[2 * lane]};
    s_ki[r1] = DecKInfo{b1, (uint32_t)(2 * lane + 1), sc[2 * lane + 1], zr[2 * lane + 1]};
    s_zr[r0] = round_bf16(zr[2 * lane]);
    s_zr[r1] = round_bf16(zr[2 * lane + 1]);
    uint32_t fw = ((uint32_t)(p.tile_tokens * (int)b0 + 31) >> 5) + ((uint32_t)(p.tile_tokens * (int)b1 + 31) >> 5);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) fw += __shfl_xor(fw, o, 64);
    if (lane == 0) s_misc[2] = (int32_t)fw;
  }
  __syncthreads();
  // the chunk's first packed tile straight into the second tile buffer
  // (past the staged basis) while the set-up goes on
  bool pf0 = false;
  {
    uint32_t* const tb2 = reinterpret_cast<uint32_t*>(stage + 64 * 17);
    const uint32_t* slot0 =
        reinterpret_cast<const uint32_t*>(p.ws + p.w.packed + (int64_t)(u * p.blks_per_sec + ch) * p.w.packed_slot);
    const bool clear = reinterpret_cast<uint8_t*>(tb2) - reinterpret_cast<uint8_t*>(dlds) >= 128 * kBS * 2;
    if (clear && (reinterpret_cast<uintptr_t>(slot0) & 15u) == 0) {
      const int nt0 = min(p.tile_tokens, min(p.blk_tokens, p.T_mid - ch * p.blk_tokens));
      uint32_t w = ((uint32_t)(nt0 * (int)s_b[2 * lane] + 31) >> 5) + ((uint32_t)(nt0 * (int)s_b[2 * lane + 1] + 31) >> 5);
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) w += __shfl_xor(w, o, 64);
      const uint32_t n4 = w >> 2;
      for (uint32_t c = (uint32_t)wave; c * 64 < n4; c += 4)
        if (c * 64 + (uint32_t)lane < n4)
          __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)(slot0 + 4 * (c * 64 + lane)),
                                           (void __attribute__((address_space(3)))*)(tb2 + 256 * c), 16, 0, kNtLoad);
      pf0 = true;
    }
  }
  // stage the basis with its columns in sorted component order:
  // bst[channel][sorted position]
  uint16_t* bst = reinterpret_cast<uint16_t*>(dlds);
  {
    uint32_t rk[8];
#pragma unroll
    for (int z = 0; z < 8; ++z) rk[z] = s_rank[(tid & 15) * 8 + z];
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      uint16_t* brow = bst + (it * 16 + (tid >> 4)) * kBS;
      const uint32_t w[4] = {brow8[it].x, brow8[it].y, brow8[it].z, brow8[it].w};
#pragma unroll
      for (int z = 0; z < 8; ++z) brow[rk[z]] = (uint16_t)(w[z >> 1] >> (16 * (z & 1)));
    }
  }
  __syncthreads();
  if (tid >= 128) {
    // constant of the b = 0 components (sorted positions nnz .. D-1):
    // sum_i B[j][i] bf16(zero_i), fp64 (four partial sums), one rounding;
    // eight basis entries and zero points per step from 16-byte LDS reads
    const int j = tid - 128;
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    for (int k8 = nnz & ~7; k8 < D; k8 += 8) {
      const uint4 bw = *reinterpret_cast<const uint4*>(&bst[j * kBS + k8]);
      const float4 z0 = *reinterpret_cast<const float4*>(&s_zr[k8]);
      const float4 z1 = *reinterpret_cast<const float4*>(&s_zr[k8 + 4]);
      const uint32_t bv[4] = {bw.x, bw.y, bw.z, bw.w};
      const float zv[8] = {z0.x, z0.y, z0.z, z0.w, z1.x, z1.y, z1.z, z1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float bf = __uint_as_float((e & 1) ? (bv[e >> 1] & 0xffff0000u) : (bv[e >> 1] << 16));
        const double t = (double)bf * (double)zv[e];
        acc[e & 3] += (k8 + e >= nnz) ? t : 0.0;
      }
    }
    s_const[j] = (float)((acc[0] + acc[1]) + (acc[2] + acc[3]));
  }
  // this wave's basis operand fragments A[mi][kb]: lane (g, r) holds channel
  // 32 pp + 8 (r >> 2) + 4 a + (r & 3), pp = hf + 2 (mi >> 1), a = mi & 1,
  // hf = wave & 1, of the sorted components 32 kb + 8 g .. +7.  Positions past
  // the coded components multiply dequantised zeros (the basis is finite).
  uint4 A[4][KBMAX];
  {
    const int hf = wave & 1;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const int pp = hf + 2 * (mi >> 1), a = mi & 1;
      const uint16_t* brow = bst + (32 * pp + 8 * (r >> 2) + 4 * a + (r & 3)) * kBS;
#pragma unroll
      for (int kb = 0; kb < KBMAX; ++kb) A[mi][kb] = *reinterpret_cast<const uint4*>(brow + 32 * kb + 8 * g);
    }
  }
  __syncthreads();  // the staged basis area becomes the operand and tile buffers
  const uint32_t fw = (uint32_t)s_misc[2];

#define KVTC_DEC_CHUNK(KBV, OBV) dec_chunk128<KBV, KBMAX, OBV, PG>(p, u, ch, A, cq, tb, s_kw, s_ki, s_rank, s_b, s_const, fw, stage, pf0)
  if constexpr (PG) {  // pools hold the cache dtype: bf16
    if constexpr (KBMAX == 4) {
      KVTC_DEC_CHUNK(4, 2);
    } else {
      switch (KB) {
        case 0: KVTC_DEC_CHUNK(0, 2); break;
        case 1: KVTC_DEC_CHUNK(1, 2); break;
        case 2: KVTC_DEC_CHUNK(2, 2); break;
        default: KVTC_DEC_CHUNK(3, 2); break;
      }
    }
  } else if constexpr (KBMAX == 4) {
    if (p.out_dtype == KVTC_BF16) KVTC_DEC_CHUNK(4, 2);
    else KVTC_DEC_CHUNK(4, 4);
  } else if (p.out_dtype == KVTC_BF16) {
    switch (KB) {
      case 0: KVTC_DEC_CHUNK(0, 2); break;
      case 1: KVTC_DEC_CHUNK(1, 2); break;
      case 2: KVTC_DEC_CHUNK(2, 2); break;
      default: KVTC_DEC_CHUNK(3, 2); break;
    }
  } else {
    switch (KB) {
      case 0: KVTC_DEC_CHUNK(0, 4); break;
      case 1: KVTC_DEC_CHUNK(1, 4); break;
      case 2: KVTC_DEC_CHUNK(2, 4); break;
      default: KVTC_DEC_CHUNK(3, 4); break;
    }
  }
#undef KVTC_DEC_CHUNK
}

hipError_t launch_dec_transform(const Params& p, hipStream_t s) {
  dim3 grid(p.blks_per_sec, p.n_sections), block(256);
  if (p.transform == KVTC_WHT) {
    hipLaunchKernelGGL(k_dec_wht, grid, block, 0, s, p);
    return hipGetLastError();
  }
  const int ob = p.out_dtype == KVTC_BF16 ? 2 : 4;
  const int32_t bmax = p.sec_bits_max;
  const int32_t nz = bmax < p.D ? bmax : p.D;
  const size_t tile_words = (size_t)(((int64_t)p.tile_tokens * bmax + 31) / 32 + nz) + 4;
  if (p.D == 128 && p.dtype == KVTC_BF16 && p.tile_tokens % 64 == 0 &&
      (p.n_seqs > 0 || (int64_t)p.T * 128 * ob < (1ll << 31))) {
    // dynamic LDS: operands + tile buffer, at least the staged basis
    // two tile buffers around the row staging
    const size_t tbytes = (size_t)((dec_tile_words(p) + 3) & ~3) * 4 * 2 + (size_t)64 * 17 * 16, bbytes = (size_t)128 * kBS * 2;
    size_t lds3 = (size_t)3 * 4 * 64 * 16 + tbytes, lds4 = (size_t)4 * 4 * 64 * 16 + tbytes;
    if (lds3 < bbytes) lds3 = bbytes;
    if (lds4 < bbytes) lds4 = bbytes;
    if (lds4 <= 140 * 1024) {
      dim3 g4(p.blks_per_sec, p.n_sections, seq_grid(p));
      if (p.n_seqs > 0) {
        if (ob != 2) return hipErrorInvalidValue;
        (void)hipFuncSetAttribute((const void*)k_dec_pca128<3, true>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds3);
        (void)hipFuncSetAttribute((const void*)k_dec_pca128<4, true>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds4);
        hipLaunchKernelGGL((k_dec_pca128<3, true>), g4, block, lds3, s, p);
        hipLaunchKernelGGL((k_dec_pca128<4, true>), g4, block, lds4, s, p);
        return hipGetLastError();
      }
      (void)hipFuncSetAttribute((const void*)k_dec_pca128<3, false>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds3);
      (void)hipFuncSetAttribute((const void*)k_dec_pca128<4, false>, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds4);
      hipLaunchKernelGGL((k_dec_pca128<3, false>), g4, block, lds3, s, p);
      hipLaunchKernelGGL((k_dec_pca128<4, false>), g4, block, lds4, s, p);
      return hipGetLastError();
    }
  }
  if (p.D == 128 && p.dtype == KVTC_BF16) {
    size_t lds = 64 * (128 + 8) * 2 + 4 * 16 * 128 * ob + tile_words * 4;
    hipLaunchKernelGGL((k_dec_pca<128, KVTC_BF16>), grid, block, lds, s, p);
  } else if (p.D == 64 && p.dtype == KVTC_BF16) {
    size_t lds = 64 * (64 + 8) * 2 + 4 * 16 * 64 * ob + tile_words * 4;
    hipLaunchKernelGGL((k_dec_pca<64, KVTC_BF16>), grid, block, lds, s, p);
  } else if (p.D == 64 && p.dtype == KVTC_FP32) {
    size_t lds = 64 * (64 + 4) * 4 + 4 * 16 * 64 * ob + tile_words * 4;
    hipLaunchKernelGGL((k_dec_pca<64, KVTC_FP32>), grid, block, lds, s, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kvtc
