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
  const int t0 = ch * p.chunk_tokens;
  const int n = min(p.chunk_tokens, p.T_mid - t0);
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
  const uint32_t* slot = reinterpret_cast<const uint32_t*>(p.ws + p.w.packed + (int64_t)(u * p.chunks_per_sec + ch) * p.w.packed_slot);
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
  const int t0 = ch * p.chunk_tokens;
  const int n = min(p.chunk_tokens, p.T_mid - t0);
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
  const uint32_t* slot = reinterpret_cast<const uint32_t*>(p.ws + p.w.packed + (int64_t)(u * p.chunks_per_sec + ch) * p.w.packed_slot);
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
#pragma unroll
        for (int st = 1; st < 8; st <<= 1)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (!(e & st)) {
              double a = y[e], bb = y[e + st];
              y[e] = a + bb;
              y[e + st] = a - bb;
            }
#pragma unroll
        for (int o = 1; o < 16; o <<= 1)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            double other = __shfl_xor(y[e], o, 16);
            y[e] = (q & o) ? other - y[e] : y[e] + other;
          }
        const double rs = __dsqrt_rn((double)D);
        const float rt = rarea[r_index * p.T_mid + t0 + tok];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = __fmul_rn((float)__ddiv_rn(y[e], rs), rt);
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
        *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(dst) + base) = o;
      } else {
        float* d = reinterpret_cast<float*>(dst) + base;
        *reinterpret_cast<float4*>(d) = make_float4(x[0], x[1], x[2], x[3]);
        *reinterpret_cast<float4*>(d + 4) = make_float4(x[4], x[5], x[6], x[7]);
      }
    }
  }
}

// ---- head_dim 128, bf16 cache: the bandwidth-oriented decode pass -------------
// Workgroup per chunk, 4 waves, 64-token sub-tiles.  Dequantisation: wave w
// takes components [32w, 32w+32) with lane = token, so the bit width, scale
// and zero point are wave-uniform; the codes come from the packed tile in
// LDS (double-buffered: the next tile's bytes are loaded into registers while
// the current one is decoded).  MFMA: wave w owns output channels
// {16w .. 16w+15} and {64+16w .. 64+16w+15} -- both members of every
// half-split RoPE pair -- with the basis rows in registers and the token rows
// of c^ read from LDS.  Results go through an LDS tile to 16-byte stores.

constexpr int kCS = 136;  // LDS row stride (bf16) of the c^ and output tiles

__global__ __launch_bounds__(256) void k_dec128(const Params p) {
  constexpr int D = 128;
  const int u = blockIdx.y, ch = blockIdx.x;
  const int h = u % p.H, s = (u / p.H) & 1, l = u / (2 * p.H);
  const int t0 = ch * p.chunk_tokens;
  const int n = min(p.chunk_tokens, p.T_mid - t0);
  if (n <= 0) return;
  if (get_status(p.ws, p.w) & (1u << KVTC_ERR_CORRUPT)) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, r = lane & 15;
  const bool rope = (s == 0) && p.rope_keys;
  uint8_t* dst = reinterpret_cast<uint8_t*>(s ? p.v_out : p.k_out);
  const int ob = p.out_dtype == KVTC_BF16 ? 2 : 4;
  const int64_t lh_row0 = ((int64_t)l * p.H + h) * p.T;

  __shared__ uint32_t s_bits[D], s_roww[D + 1];
  __shared__ float s_zero[D], s_scale[D];
  __shared__ __attribute__((aligned(16))) uint16_t C[64 * kCS];
  extern __shared__ __attribute__((aligned(16))) uint32_t dyn[];
  // dyn: [output tile 64 x 128 x ob (+pad)][packed tile buffers x 2]
  uint8_t* O = reinterpret_cast<uint8_t*>(dyn);
  const int orow = D * ob + 16;  // padded output row bytes
  uint32_t* pk[2];
  pk[0] = reinterpret_cast<uint32_t*>(O + 64 * orow);
  const uint8_t* rec = p.in + p.side_off + (int64_t)u * 9 * D;
  if (tid < D) {
    s_bits[tid] = rec[tid];
    s_zero[tid] = reinterpret_cast<const float*>(rec + D)[tid];
    s_scale[tid] = reinterpret_cast<const float*>(rec + 5 * D)[tid];
  }
  __syncthreads();
  uint32_t full_words = 0;
  for (int i = 0; i < D; ++i) full_words += (uint32_t)((p.tile_tokens * (int)s_bits[i] + 31) >> 5);
  pk[1] = pk[0] + full_words + 4;
  const uint32_t* slot = reinterpret_cast<const uint32_t*>(
      p.ws + p.w.packed + (int64_t)(u * p.chunks_per_sec + ch) * p.w.packed_slot);
  const int ntiles = (n + p.tile_tokens - 1) / p.tile_tokens;

  // basis rows j = 16(w + 4m) + r, components 32kb + 8g .. +7
  const int64_t bi = (p.basis_per_head ? ((int64_t)(l * 2 + s) * p.H + h) : (int64_t)(l * 2 + s)) * D * D;
  const uint16_t* B = reinterpret_cast<const uint16_t*>(p.basis) + bi;
  uint4 bq[2][4];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      bq[m][kb] = *reinterpret_cast<const uint4*>(B + (int64_t)((wave + 4 * m) * 16 + r) * D + kb * 32 + 8 * g);

  // packed tile prefetch: up to 36 words per thread (8-bit budget, 256 tokens)
  constexpr int kPF = 36;
  uint32_t pf[kPF];
  auto fetch_tile = [&](int tl) {
    const int nt = min(p.tile_tokens, n - tl * p.tile_tokens);
    uint32_t tw = 0;
    for (int i = 0; i < D; ++i) tw += (uint32_t)((nt * (int)s_bits[i] + 31) >> 5);
    const uint32_t* srcw = slot + (int64_t)tl * full_words;
#pragma unroll
    for (int k = 0; k < kPF; ++k) {
      const uint32_t i = tid + 256 * k;
      pf[k] = i < tw ? srcw[i] : 0u;
    }
    return tw;
  };
  auto commit_tile = [&](int buf, uint32_t tw) {
#pragma unroll
    for (int k = 0; k < kPF; ++k) {
      const uint32_t i = tid + 256 * k;
      if (i <= tw) pk[buf][i] = i < tw ? pf[k] : 0u;  // one zero word past the end
    }
  };

  uint32_t tw_cur = fetch_tile(0);
  commit_tile(0, tw_cur);
  for (int tl = 0; tl < ntiles; ++tl) {
    const int buf = tl & 1;
    const int ta = tl * p.tile_tokens;
    const int nt = min(p.tile_tokens, n - ta);
    uint32_t tw_next = 0;
    if (tl + 1 < ntiles) tw_next = fetch_tile(tl + 1);
    // row offsets of this tile
    if (tid < 64) {
      const uint32_t w0 = (uint32_t)((nt * (int)s_bits[2 * lane] + 31) >> 5);
      const uint32_t w1 = (uint32_t)((nt * (int)s_bits[2 * lane + 1] + 31) >> 5);
      uint32_t x = w0 + w1;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
      }
      s_roww[2 * lane] = x - (w0 + w1);
      s_roww[2 * lane + 1] = x - w1;
    }
    __syncthreads();
    const uint32_t* P = pk[buf];
    for (int sb0 = 0; sb0 < nt; sb0 += 64) {
      const int ns = min(64, nt - sb0);
      // ---- dequantise: wave w, components [32w, 32w+32), lane = token
      {
        const int tt = sb0 + lane;  // token within the tile
        const bool valid = lane < ns;
#pragma unroll 4
        for (int c2 = 0; c2 < 32; c2 += 2) {
          uint32_t packed2 = 0;
#pragma unroll
          for (int z = 0; z < 2; ++z) {
            const int i = wave * 32 + c2 + z;
            const uint32_t b = s_bits[i];
            uint32_t q = 0;
            if (b && valid) {
              const uint32_t pos = (uint32_t)tt * b;
              const uint32_t* rw = P + s_roww[i] + (pos >> 5);
              const uint64_t v = (uint64_t)rw[0] | ((uint64_t)rw[1] << 32);
              q = (uint32_t)(v >> (pos & 31)) & ((1u << b) - 1u);
            }
            const float c = __fmaf_rn((float)q, s_scale[i], s_zero[i]);
            packed2 |= (uint32_t)f32_to_bf16(c) << (16 * z);
          }
          *reinterpret_cast<uint32_t*>(&C[lane * kCS + wave * 32 + c2]) = packed2;
        }
      }
      __syncthreads();
      // ---- inverse projection
      f32x4_t acc[4][2];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        acc[kk][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        acc[kk][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const uint4 a = *reinterpret_cast<const uint4*>(&C[(kk * 16 + r) * kCS + kb * 32 + 8 * g]);
          const bf16x8_t av = __builtin_bit_cast(bf16x8_t, a);
#pragma unroll
          for (int m = 0; m < 2; ++m)
            acc[kk][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8_t, bq[m][kb]),
                                                                 acc[kk][m], 0, 0, 0);
        }
      }
      // ---- RoPE on keys, output cast, into the output tile
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int tk = kk * 16 + 4 * g + e;  // token within the sub-tile
          float x0 = acc[kk][0][e], x1 = acc[kk][1][e];
          if (rope && tk < ns) {
            const int pos = p.mid_begin + t0 + ta + sb0 + tk;
            const float2* rr = p.rope + (int64_t)pos * (D / 2);
            if (p.rope_style == KVTC_ROPE_HALF) {
              const float2 cs = rr[wave * 16 + r];  // pair (j, j + 64), j = 16w + r
              const float xb_s = __fmul_rn(x1, cs.y), xb_c = __fmul_rn(x1, cs.x);
              const float y0 = __fmaf_rn(x0, cs.x, -xb_s);
              const float y1 = __fmaf_rn(x0, cs.y, xb_c);
              x0 = y0;
              x1 = y1;
            } else {
              const bool first = (r & 1) == 0;
              const float o0 = __shfl_xor(x0, 1, 64), o1 = __shfl_xor(x1, 1, 64);
              const float2 c0 = rr[(wave * 16 + r) >> 1], c1 = rr[(64 + wave * 16 + r) >> 1];
              const float a0 = first ? x0 : o0, b0 = first ? o0 : x0;
              const float a1 = first ? x1 : o1, b1 = first ? o1 : x1;
              x0 = first ? __fmaf_rn(a0, c0.x, -__fmul_rn(b0, c0.y)) : __fmaf_rn(a0, c0.y, __fmul_rn(b0, c0.x));
              x1 = first ? __fmaf_rn(a1, c1.x, -__fmul_rn(b1, c1.y)) : __fmaf_rn(a1, c1.y, __fmul_rn(b1, c1.x));
            }
          }
          uint8_t* orow_p = O + tk * orow;
          const int j0 = wave * 16 + r, j1 = 64 + wave * 16 + r;
          if (ob == 2) {
            reinterpret_cast<uint16_t*>(orow_p)[j0] = f32_to_bf16(x0);
            reinterpret_cast<uint16_t*>(orow_p)[j1] = f32_to_bf16(x1);
          } else {
            reinterpret_cast<float*>(orow_p)[j0] = x0;
            reinterpret_cast<float*>(orow_p)[j1] = x1;
          }
        }
      }
      __syncthreads();
      // ---- coalesced stores: row bytes D * ob, 16 B per thread per step
      {
        const int per_row = D * ob / 16;
        for (int idx = tid; idx < ns * per_row; idx += 256) {
          const int tk = idx / per_row, cc = idx % per_row;
          const int pos = p.mid_begin + t0 + ta + sb0 + tk;
          uint8_t* drow = dst + (lh_row0 + pos) * (int64_t)D * ob;
          reinterpret_cast<uint4*>(drow)[cc] = *reinterpret_cast<const uint4*>(O + tk * orow + 16 * cc);
        }
      }
    }
    if (tl + 1 < ntiles) {
      commit_tile(buf ^ 1, tw_next);
      __syncthreads();
    }
  }
}

hipError_t launch_dec_transform(const Params& p, hipStream_t s) {
  dim3 grid(p.chunks_per_sec, p.n_sections), block(256);
  if (p.transform == KVTC_WHT) {
    hipLaunchKernelGGL(k_dec_wht, grid, block, 0, s, p);
    return hipGetLastError();
  }
  const int ob = p.out_dtype == KVTC_BF16 ? 2 : 4;
  const int32_t bmax = p.budget_k > p.budget_v ? p.budget_k : p.budget_v;
  const int32_t nz = bmax < p.D ? bmax : p.D;
  const size_t tile_words = (size_t)(((int64_t)p.tile_tokens * bmax + 31) / 32 + nz) + 4;
  if (p.D == 128 && p.dtype == KVTC_BF16 && tile_words <= 36 * 256) {
    const size_t lds = 64 * (size_t)(128 * ob + 16) + 2 * (tile_words + 4) * 4;
    (void)hipFuncSetAttribute((const void*)k_dec128, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL(k_dec128, grid, block, lds, s, p);
    return hipGetLastError();
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
