// Encode-side kernels: raw windows, the RoPE-undo + MFMA projection with
// per-component statistics, greedy bit allocation with side information,
// and the fused quantise-and-pack pass.
//
// Projection layout (gfx950 v_mfma_f32_16x16x32_bf16, wave64): a wave
// projects 16 tokens at a time.  Lane l = 16 g + r holds token r of the
// block; its K-slice is the channel run [g D/8, (g+1) D/8) of the first
// half and the matching run of the second half, so both members of every
// half-split RoPE pair (j, j + D/2) sit in the same lane.  The basis of the
// section is register-resident as B operands (component nb*16 + r, same
// channel permutation).  The result lane l holds the coefficients of
// component nb*16 + r for tokens 4g .. 4g+3 of the block: four consecutive
// codes of one component, which is what channel-major packing wants.
#include <string.h>

#include <type_traits>

#include "kvtc_internal.h"

namespace kvtc {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int D>
struct Geo {
  static constexpr int HALF = D / 2;
  static constexpr int PER = D / 8;  // channels per lane per half
  static constexpr int NB = D / 16;  // 16-component output blocks
  static constexpr int NKB = D / 32; // bf16 K blocks of 8 channels per lane
};

// channel of the e-th element of K-run position k (0 <= k < D/4) of lane group g
template <int D>
__device__ __forceinline__ int lane_channel(int g, int k) {
  constexpr int PER = Geo<D>::PER;
  return k < PER ? g * PER + k : Geo<D>::HALF + g * PER + (k - PER);
}

__device__ __forceinline__ void unpack_bf16x8(uint4 a, float* o) {
  o[0] = __uint_as_float(a.x << 16); o[1] = __uint_as_float(a.x & 0xffff0000u);
  o[2] = __uint_as_float(a.y << 16); o[3] = __uint_as_float(a.y & 0xffff0000u);
  o[4] = __uint_as_float(a.z << 16); o[5] = __uint_as_float(a.z & 0xffff0000u);
  o[6] = __uint_as_float(a.w << 16); o[7] = __uint_as_float(a.w & 0xffff0000u);
}

__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  return (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
}

// Load the lane's channel runs of one cache row (lo: first half, hi: second).
template <int D, int DT>
__device__ __forceinline__ void load_runs(const void* src, int64_t row, int g, bool valid,
                                          float* lo, float* hi) {
  constexpr int PER = Geo<D>::PER, HALF = Geo<D>::HALF;
  if (DT == KVTC_BF16) {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(src) + row;
#pragma unroll
    for (int q = 0; q < PER / 8; ++q) {
      uint4 a = make_uint4(0, 0, 0, 0), b = make_uint4(0, 0, 0, 0);
      if (valid) {
        a = *reinterpret_cast<const uint4*>(p + g * PER + q * 8);
        b = *reinterpret_cast<const uint4*>(p + HALF + g * PER + q * 8);
      }
      unpack_bf16x8(a, lo + q * 8);
      unpack_bf16x8(b, hi + q * 8);
    }
  } else {
    const float* p = reinterpret_cast<const float*>(src) + row;
#pragma unroll
    for (int q = 0; q < PER / 4; ++q) {
      float4 a = make_float4(0, 0, 0, 0), b = make_float4(0, 0, 0, 0);
      if (valid) {
        a = *reinterpret_cast<const float4*>(p + g * PER + q * 4);
        b = *reinterpret_cast<const float4*>(p + HALF + g * PER + q * 4);
      }
      lo[q * 4 + 0] = a.x; lo[q * 4 + 1] = a.y; lo[q * 4 + 2] = a.z; lo[q * 4 + 3] = a.w;
      hi[q * 4 + 0] = b.x; hi[q * 4 + 1] = b.y; hi[q * 4 + 2] = b.z; hi[q * 4 + 3] = b.w;
    }
  }
}

// Undo RoPE in place ("Why RoPE Has to Be Reversed First"):
//   x_a = fma(y_a, c, y_b s),  x_b = fma(y_b, c, -(y_a s)).
template <int D>
__device__ __forceinline__ void rope_inverse_runs(const float2* rope_row, int g, int style,
                                                  float* lo, float* hi) {
  constexpr int PER = Geo<D>::PER, HALF = Geo<D>::HALF;
  if (style == KVTC_ROPE_HALF) {
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      float2 cs = rope_row[g * PER + e];
      float ya = lo[e], yb = hi[e];
      float yb_s = __fmul_rn(yb, cs.y), ya_s = __fmul_rn(ya, cs.y);
      lo[e] = __fmaf_rn(ya, cs.x, yb_s);
      hi[e] = __fmaf_rn(yb, cs.x, -ya_s);
    }
  } else {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      float* v = half ? hi : lo;
      int base = (half ? HALF : 0) + g * PER;
#pragma unroll
      for (int m = 0; m < PER / 2; ++m) {
        float2 cs = rope_row[(base >> 1) + m];
        float ya = v[2 * m], yb = v[2 * m + 1];
        float yb_s = __fmul_rn(yb, cs.y), ya_s = __fmul_rn(ya, cs.y);
        v[2 * m] = __fmaf_rn(ya, cs.x, yb_s);
        v[2 * m + 1] = __fmaf_rn(yb, cs.x, -ya_s);
      }
    }
  }
}

// Register-resident basis operands of one section.
template <int D, int DT>
struct BasisRegs;

template <int D>
struct BasisRegs<D, KVTC_BF16> {
  uint4 b[Geo<D>::NB][Geo<D>::NKB];
  __device__ __forceinline__ void load(const uint16_t* bt, int g, int r) {
    constexpr int PER = Geo<D>::PER, HALF = Geo<D>::HALF, NKB = Geo<D>::NKB;
#pragma unroll
    for (int nb = 0; nb < Geo<D>::NB; ++nb)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        int ch = kb < NKB / 2 ? g * PER + kb * 8 : HALF + g * PER + (kb - NKB / 2) * 8;
        b[nb][kb] = *reinterpret_cast<const uint4*>(bt + (int64_t)(nb * 16 + r) * D + ch);
      }
  }
};

template <int D>
struct BasisRegs<D, KVTC_FP32> {
  float b[Geo<D>::NB][D / 4];
  __device__ __forceinline__ void load(const float* bt, int g, int r) {
#pragma unroll
    for (int nb = 0; nb < Geo<D>::NB; ++nb)
#pragma unroll
      for (int k = 0; k < D / 4; ++k) b[nb][k] = bt[(int64_t)(nb * 16 + r) * D + lane_channel<D>(g, k)];
  }
};

// c[token 4g+e][component nb*16+r] = acc[nb][e]
template <int D, int DT>
__device__ __forceinline__ void project_block(const BasisRegs<D, DT>& B, const float* lo,
                                              const float* hi, f32x4_t* acc) {
  constexpr int NB = Geo<D>::NB;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if constexpr (DT == KVTC_BF16) {
    constexpr int NKB = Geo<D>::NKB, PER = Geo<D>::PER;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      const float* src = kb < NKB / 2 ? lo + kb * 8 : hi + (kb - NKB / 2) * 8;
      uint4 a;
      a.x = pack2_bf16(src[0], src[1]); a.y = pack2_bf16(src[2], src[3]);
      a.z = pack2_bf16(src[4], src[5]); a.w = pack2_bf16(src[6], src[7]);
      bf16x8_t av = __builtin_bit_cast(bf16x8_t, a);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8_t, B.b[nb][kb]),
                                                          acc[nb], 0, 0, 0);
    }
    (void)PER;
  } else {
    constexpr int PER = Geo<D>::PER;
#pragma unroll
    for (int k = 0; k < D / 4; ++k) {
      float av = k < PER ? lo[k] : hi[k - PER];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, B.b[nb][k], acc[nb], 0, 0, 0);
    }
  }
}

__device__ __forceinline__ int64_t basis_index(const Params& p, int l, int s, int h) {
  return p.basis_per_head ? ((int64_t)(l * 2 + s) * p.H + h) : (int64_t)(l * 2 + s);
}

// exclusive prefix sum over the lanes of one wave
__device__ __forceinline__ uint32_t wave_excl_scan(uint32_t v, uint32_t* total) {
  const int lane = threadIdx.x & 63;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  *total = __shfl(x, 63, 64);
  return x - v;
}

// ---------------------------------------------------------------------------
// raw windows: [sink K][recent K][sink V][recent V], each [L,H,n,D], copied
// bit-exactly ("How the Pipeline Works": they stay in high fidelity)
// ---------------------------------------------------------------------------

// The raw sink and recent runs (copy_raw_run), one workgroup per run.
// Encode: the first workgroup also clears the status word and the count slots.
__global__ __launch_bounds__(256) void k_copy_raw(const Params p0, int to_container) {
  const Params p = at_seq(p0, blockIdx.z);
  copy_raw_run(p, blockIdx.x, to_container, p0.n_seqs == 0);
}

hipError_t launch_copy_raw(const Params& p, int to_container, hipStream_t s) {
  const int e = p.dtype == KVTC_BF16 ? 2 : 4;
  if ((p.D * e) % 16) return hipErrorInvalidValue;
  const int64_t runs = 4 * (int64_t)p.L * p.H;
  if (runs > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_copy_raw, dim3((unsigned)runs, 1, seq_grid(p)), dim3(256), 0, s, p, to_container);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// projection passes over the middle region of every section
//   mode 0: statistics per (section, chunk, component)
//   mode 1: quantise and pack into channel-major tiles
//   mode 2: write the coefficients (parity hook)
// ---------------------------------------------------------------------------

struct SideLds {
  float zero[128];
  float rcp[128];
  uint32_t bits[128];
  uint32_t row_w[129];  // word offset of each component's row in the current tile
};

template <int D, int DT, int MODE>
__global__ __launch_bounds__(256) void k_enc_pca(const Params p, int sec0, float* coef_out) {
  constexpr int NB = Geo<D>::NB, PER = Geo<D>::PER;
  if (MODE == 0 && p.n_seqs == 0 && blockIdx.x == 0 && blockIdx.y == 0) clear_status_block(p);
  const int u = blockIdx.y + sec0, ch = blockIdx.x;
  const int h = u % p.H, s = (u / p.H) & 1, l = u / (2 * p.H);
  const int t0 = ch * p.blk_tokens;
  const int n = min(p.blk_tokens, p.T_mid - t0);
  if (n <= 0) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, r = lane & 15;
  const void* src = s ? p.v : p.k;
  const bool rope = (s == 0) && p.rope_keys;
  const int64_t lh_row0 = ((int64_t)l * p.H + h) * p.T;

  BasisRegs<D, DT> B;
  {
    const int64_t bi = basis_index(p, l, s, h) * D * D;
    if constexpr (DT == KVTC_BF16)
      B.load(reinterpret_cast<const uint16_t*>(p.basis_t) + bi, g, r);
    else
      B.load(reinterpret_cast<const float*>(p.basis_t) + bi, g, r);
  }

  float lo[PER], hi[PER];
  f32x4_t acc[NB];

  if constexpr (MODE == 0) {
    double sum[NB], sq[NB];
    float mn[NB], mx[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) { sum[nb] = 0.0; sq[nb] = 0.0; mn[nb] = INFINITY; mx[nb] = -INFINITY; }
    for (int blk = wave; blk * 16 < n; blk += 4) {
      const int tok = blk * 16 + r;
      const bool valid = tok < n;
      const int pos = p.mid_begin + t0 + tok;
      load_runs<D, DT>(src, (lh_row0 + pos) * D, g, valid, lo, hi);
      if (rope && valid) {
        rope_inverse_runs<D>(p.rope + (int64_t)pos * Geo<D>::HALF, g, p.rope_style, lo, hi);
        if (DT == KVTC_BF16) {
#pragma unroll
          for (int e2 = 0; e2 < PER; ++e2) { lo[e2] = round_bf16(lo[e2]); hi[e2] = round_bf16(hi[e2]); }
        }
      }
      project_block<D, DT>(B, lo, hi, acc);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (blk * 16 + 4 * g + e < n) {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            float c = acc[nb][e];
            sum[nb] += (double)c;
            sq[nb] = __fma_rn((double)c, (double)c, sq[nb]);
            mn[nb] = fminf(mn[nb], c);
            mx[nb] = fmaxf(mx[nb], c);
          }
        }
      }
    }
    // combine the four lane groups, then the four waves, in a fixed order
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int o = 16; o <= 32; o <<= 1) {
        sum[nb] += __shfl_xor(sum[nb], o, 64);
        sq[nb] += __shfl_xor(sq[nb], o, 64);
        mn[nb] = fminf(mn[nb], __shfl_xor(mn[nb], o, 64));
        mx[nb] = fmaxf(mx[nb], __shfl_xor(mx[nb], o, 64));
      }
    }
    __shared__ double s_sum[4][D], s_sq[4][D];
    __shared__ float s_mn[4][D], s_mx[4][D];
    if (g == 0) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        int i = nb * 16 + r;
        s_sum[wave][i] = sum[nb]; s_sq[wave][i] = sq[nb]; s_mn[wave][i] = mn[nb]; s_mx[wave][i] = mx[nb];
      }
    }
    __syncthreads();
    if (threadIdx.x < D) {
      int i = threadIdx.x;
      double a = s_sum[0][i], b = s_sq[0][i];
      float c = s_mn[0][i], d = s_mx[0][i];
      for (int w2 = 1; w2 < 4; ++w2) {
        a += s_sum[w2][i]; b += s_sq[w2][i];
        c = fminf(c, s_mn[w2][i]); d = fmaxf(d, s_mx[w2][i]);
      }
      int64_t idx = ((int64_t)u * p.blks_per_sec + ch) * D + i;
      reinterpret_cast<double*>(p.ws + p.w.part_sum)[idx] = a;
      reinterpret_cast<double*>(p.ws + p.w.part_sq)[idx] = b;
      reinterpret_cast<float*>(p.ws + p.w.part_min)[idx] = c;
      reinterpret_cast<float*>(p.ws + p.w.part_max)[idx] = d;
    }
  } else if constexpr (MODE == 1) {
    if (get_status(p.ws, p.w) & (1u << KVTC_ERR_NONFINITE)) return;
    __shared__ SideLds sd;
    // dynamic LDS: [basis copy D x D][staged rows 4 x 16 x D][tile buffer]
    using otype = typename std::conditional<DT == KVTC_BF16, uint16_t, float>::type;
    extern __shared__ uint32_t dynlds[];
    otype* bt_lds = reinterpret_cast<otype*>(dynlds);
    otype* xs = bt_lds + D * D;
    uint32_t* tilebuf = reinterpret_cast<uint32_t*>(xs + 4 * 16 * D);
    {
      const otype* bsrc = reinterpret_cast<const otype*>(p.basis_t) + basis_index(p, l, s, h) * D * D;
      const int n4 = D * D * (int)sizeof(otype) / 16;
      for (int i = threadIdx.x; i < n4; i += blockDim.x)
        reinterpret_cast<uint4*>(bt_lds)[i] = reinterpret_cast<const uint4*>(bsrc)[i];
    }
    if (threadIdx.x < D) {
      int i = threadIdx.x;
      int64_t si = (int64_t)u * D + i;
      sd.zero[i] = reinterpret_cast<const float*>(p.ws + p.w.side_zero)[si];
      sd.rcp[i] = reinterpret_cast<const float*>(p.ws + p.w.side_rcp)[si];
      sd.bits[i] = p.ws[p.w.side_bits + si];
    }
    __syncthreads();
    // per-lane side information of the components this lane produces
    float zr[NB], rc[NB], qmax[NB];
    uint32_t bl[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      int i = nb * 16 + r;
      zr[nb] = sd.zero[i]; rc[nb] = sd.rcp[i]; bl[nb] = sd.bits[i];
      qmax[nb] = (float)((1u << bl[nb]) - 1u);
    }
    // bytes of a full tile (all but possibly the last tile of the section)
    uint32_t full_words;
    {
      uint32_t v0 = 0;
      if (threadIdx.x < 64) {
        for (int i = lane; i < D; i += 64) v0 += (uint32_t)((p.tile_tokens * (int)sd.bits[i] + 31) >> 5);
      }
      __shared__ uint32_t s_full;
      if (threadIdx.x < 64) {
        uint32_t tot;
        wave_excl_scan(v0, &tot);
        if (lane == 0) s_full = tot;
      }
      __syncthreads();
      full_words = s_full;
    }
    uint32_t* slot = reinterpret_cast<uint32_t*>(p.ws + p.w.packed + (int64_t)(u * p.blks_per_sec + ch) * p.w.packed_slot);
    const int ntiles = (n + p.tile_tokens - 1) / p.tile_tokens;
    for (int tl = 0; tl < ntiles; ++tl) {
      const int ta = tl * p.tile_tokens;
      const int nt = min(p.tile_tokens, n - ta);
      // row offsets of this tile
      if (threadIdx.x < 64) {
        uint32_t w0 = 0, w1 = 0;
        int i0 = 2 * lane, i1 = 2 * lane + 1;
        if (i0 < D) w0 = (uint32_t)((nt * (int)sd.bits[i0] + 31) >> 5);
        if (i1 < D) w1 = (uint32_t)((nt * (int)sd.bits[i1] + 31) >> 5);
        uint32_t tot;
        uint32_t ex = wave_excl_scan(w0 + w1, &tot);
        if (i0 < D) sd.row_w[i0] = ex;
        if (i1 < D) sd.row_w[i1] = ex + w0;
        if (lane == 0) sd.row_w[D] = tot;
      }
      __syncthreads();
      const uint32_t tw = sd.row_w[D];
      for (uint32_t i = threadIdx.x; i < tw; i += blockDim.x) tilebuf[i] = 0;
      __syncthreads();
      const int nblk = (nt + 15) / 16;
      for (int blk = wave; blk < nblk; blk += 4) {
        const int tok = ta + blk * 16 + r;
        const bool valid = blk * 16 + r < nt;
        const int pos = p.mid_begin + t0 + tok;
        load_runs<D, DT>(src, (lh_row0 + pos) * D, g, valid, lo, hi);
        if (rope && valid) {
          rope_inverse_runs<D>(p.rope + (int64_t)pos * Geo<D>::HALF, g, p.rope_style, lo, hi);
          if (DT == KVTC_BF16) {
#pragma unroll
            for (int e2 = 0; e2 < PER; ++e2) { lo[e2] = round_bf16(lo[e2]); hi[e2] = round_bf16(hi[e2]); }
          }
        }
        project_block<D, DT>(B, lo, hi, acc);
        const int tt = blk * 16 + 4 * g;  // first token of this lane's four within the tile
        // stage this lane's channels of token r (operand precision) for the
        // exact recomputation below
        {
          otype* xr = xs + (wave * 16 + r) * D;
#pragma unroll
          for (int e2 = 0; e2 < PER; ++e2) {
            if constexpr (DT == KVTC_BF16) {
              xr[g * PER + e2] = f32_to_bf16(lo[e2]);
              xr[Geo<D>::HALF + g * PER + e2] = f32_to_bf16(hi[e2]);
            } else {
              xr[g * PER + e2] = lo[e2];
              xr[Geo<D>::HALF + g * PER + e2] = hi[e2];
            }
          }
        }
        // |c_mfma - c_exact| <= mfma_err * ||x||_2 (fp32 accumulation of the D
        // exact products; Cauchy-Schwarz with unit-norm basis columns scaled
        // by the plan's largest column norm)
        float n2 = 0.f;
#pragma unroll
        for (int e2 = 0; e2 < PER; ++e2) n2 = __fmaf_rn(lo[e2], lo[e2], __fmaf_rn(hi[e2], hi[e2], n2));
        n2 += __shfl_xor(n2, 16, 64);
        n2 += __shfl_xor(n2, 32, 64);
        float ecm[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) ecm[e] = p.mfma_err * __fsqrt_rn(__shfl(n2, 4 * g + e, 64));
        uint32_t qv[NB];
        uint32_t flags = 0;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          qv[nb] = 0;
          const uint32_t b = bl[nb];
          if (b == 0) continue;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            // v = (c - zero) * rcp, rounded half to even, clamped to [0, 2^b - 1]
            const float v = __fmul_rn(__fsub_rn(acc[nb][e], zr[nb]), rc[nb]);
            const float rv = __builtin_rintf(v);
            const float q = fminf(fmaxf(rv, 0.0f), qmax[nb]);
            if (tt + e < nt) {
              qv[nb] |= (uint32_t)q << (8 * e);
              // within the error of v of a rounding boundary: recompute exactly
              const float ev = __fmaf_rn(ecm[e], rc[nb], 3.0f * 0x1p-23f * fmaxf(fabsf(v), 1.0f));
              if (fabsf(fabsf(__fsub_rn(v, rv)) - 0.5f) < ev) flags |= 1u << (nb * 4 + e);
            }
          }
        }
        __builtin_amdgcn_wave_barrier();
        uint64_t pend = __ballot(flags != 0);
        while (pend) {
          const int L = __ffsll((unsigned long long)pend) - 1;
          const uint32_t fl = __shfl(flags, L, 64);
          const int bit = __ffs(fl) - 1;
          const int nbx = bit >> 2, ex = bit & 3;
          const int tx = 4 * (L >> 4) + ex;   // token within the block
          const int ix = nbx * 16 + (L & 15); // component
          // exact products summed in fp64 over the wave in a fixed order
          const otype* xrow = xs + (wave * 16 + tx) * D;
          const otype* brow = bt_lds + ix * D;
          double part = 0.0;
#pragma unroll
          for (int c2 = lane; c2 < D; c2 += 64) {
            float xv, bv;
            if constexpr (DT == KVTC_BF16) { xv = bf16_to_f32(xrow[c2]); bv = bf16_to_f32(brow[c2]); }
            else { xv = xrow[c2]; bv = brow[c2]; }
            part = __fma_rn((double)xv, (double)bv, part);
          }
#pragma unroll
          for (int o = 32; o > 0; o >>= 1) part += __shfl_xor(part, o, 64);
          if (lane == L) {
            const float cex = (float)part;
            const float v = __fmul_rn(__fsub_rn(cex, sd.zero[ix]), sd.rcp[ix]);
            const float q = fminf(fmaxf(__builtin_rintf(v), 0.0f), (float)((1u << sd.bits[ix]) - 1u));
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
              if (nb == nbx) qv[nb] = (qv[nb] & ~(0xffu << (8 * ex))) | ((uint32_t)q << (8 * ex));
            flags &= ~(1u << bit);
          }
          pend = __ballot(flags != 0);
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const uint32_t b = bl[nb];
          if (b == 0 || tt >= nt) continue;
          const uint32_t word = (qv[nb] & 0xffu) | (((qv[nb] >> 8) & 0xffu) << b) |
                                (((qv[nb] >> 16) & 0xffu) << (2 * b)) | ((qv[nb] >> 24) << (3 * b));
          const uint32_t bitpos = (uint32_t)tt * b;
          const uint32_t wi = sd.row_w[nb * 16 + r] + (bitpos >> 5), sh = bitpos & 31;
          atomicOr(&tilebuf[wi], word << sh);
          // bits past the 32-bit boundary; codes of tokens past the tile end are
          // zero, so a nonzero spill always lands inside this row
          const uint32_t spill = sh + 4 * b > 32 ? word >> (32 - sh) : 0u;
          if (spill) atomicOr(&tilebuf[wi + 1], spill);
        }
        __builtin_amdgcn_wave_barrier();
      }
      __syncthreads();
      uint32_t* dst = slot + (int64_t)tl * full_words;
      for (uint32_t i = threadIdx.x; i < tw; i += blockDim.x) dst[i] = tilebuf[i];
      __syncthreads();
    }
  } else {
    // mode 2: coefficients [section - sec0][T_mid][D]
    for (int blk = wave; blk * 16 < n; blk += 4) {
      const int tok = blk * 16 + r;
      const bool valid = tok < n;
      const int pos = p.mid_begin + t0 + tok;
      load_runs<D, DT>(src, (lh_row0 + pos) * D, g, valid, lo, hi);
      if (rope && valid) {
        rope_inverse_runs<D>(p.rope + (int64_t)pos * Geo<D>::HALF, g, p.rope_style, lo, hi);
        if (DT == KVTC_BF16) {
#pragma unroll
          for (int e2 = 0; e2 < PER; ++e2) { lo[e2] = round_bf16(lo[e2]); hi[e2] = round_bf16(hi[e2]); }
        }
      }
      project_block<D, DT>(B, lo, hi, acc);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        int tk = blk * 16 + 4 * g + e;
        if (tk < n) {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            coef_out[((int64_t)(u - sec0) * p.T_mid + t0 + tk) * D + nb * 16 + r] = acc[nb][e];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// WHT path: per-token RMS normalisation and the orthonormal Walsh-Hadamard
// transform in Sylvester order (TTAS-X2 2.2; the Hadamard control of
// Codec-Gauge).  16 lanes per token, lane q holds channels 8q .. 8q+7; the
// butterflies run in fp64, where every partial sum of bf16-rounded inputs is
// exact, so the coefficients are the exactly rounded transform.
// ---------------------------------------------------------------------------

template <int MODE>
__global__ __launch_bounds__(256) void k_enc_wht(const Params p, int sec0, float* coef_out, float* r_out) {
  constexpr int D = 128;
  if (MODE == 0 && p.n_seqs == 0 && blockIdx.x == 0 && blockIdx.y == 0) clear_status_block(p);
  const int u = blockIdx.y + sec0, ch = blockIdx.x;
  const int h = u % p.H, s = (u / p.H) & 1, l = u / (2 * p.H);
  const int t0 = ch * p.blk_tokens;
  const int n = min(p.blk_tokens, p.T_mid - t0);
  if (n <= 0) return;
  const int lane = threadIdx.x & 63, q = lane & 15, grp = threadIdx.x >> 4;  // 16 tokens per pass
  const void* src = s ? p.v : p.k;
  const bool rope = (s == 0) && p.rope_keys;
  const bool transform = (s == 1) || p.wht_keys;
  const int64_t lh_row0 = ((int64_t)l * p.H + h) * p.T;
  const int64_t r_index = !transform ? -1 : (p.wht_keys ? (int64_t)u : (int64_t)l * p.H + h);

  double sum[8], sq[8];
  float mn[8], mx[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) { sum[e] = 0; sq[e] = 0; mn[e] = INFINITY; mx[e] = -INFINITY; }

  __shared__ SideLds sd;
  extern __shared__ uint32_t tilebuf[];
  float zr[8], rc[8], qmax[8];
  uint32_t bl = 0;
  const bool sym = (s == 0);
  if constexpr (MODE == 1) {
    if (get_status(p.ws, p.w) & (1u << KVTC_ERR_NONFINITE)) return;
    if (threadIdx.x < D) {
      int64_t si = (int64_t)u * D + threadIdx.x;
      sd.zero[threadIdx.x] = reinterpret_cast<const float*>(p.ws + p.w.side_zero)[si];
      sd.rcp[threadIdx.x] = reinterpret_cast<const float*>(p.ws + p.w.side_rcp)[si];
      sd.bits[threadIdx.x] = p.ws[p.w.side_bits + si];
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      int i = 8 * q + e;
      zr[e] = sd.zero[i]; rc[e] = sd.rcp[i];
    }
    bl = sd.bits[0];  // uniform width on this path
#pragma unroll
    for (int e = 0; e < 8; ++e) qmax[e] = (float)((1u << bl) - 1u);
  }
  const uint32_t row_words_full = (uint32_t)((p.tile_tokens * (int)bl + 31) >> 5);
  const int ntiles = (n + p.tile_tokens - 1) / p.tile_tokens;
  uint32_t* slot = MODE == 1 ? reinterpret_cast<uint32_t*>(p.ws + p.w.packed + (int64_t)(u * p.blks_per_sec + ch) * p.w.packed_slot) : nullptr;

  for (int tl = 0; tl < ntiles; ++tl) {
    const int ta = tl * p.tile_tokens;
    const int nt = min(p.tile_tokens, n - ta);
    const uint32_t row_words = (uint32_t)((nt * (int)bl + 31) >> 5);
    if constexpr (MODE == 1) {
      for (uint32_t i = threadIdx.x; i < row_words * D; i += blockDim.x) tilebuf[i] = 0;
      __syncthreads();
    }
    for (int tb = grp; tb < nt; tb += 16) {
      const int tok = ta + tb;
      const int pos = p.mid_begin + t0 + tok;
      const uint16_t* rowp = nullptr;
      float x[8];
      if (p.dtype == KVTC_BF16) {
        rowp = reinterpret_cast<const uint16_t*>(src) + (lh_row0 + pos) * D;
        unpack_bf16x8(*reinterpret_cast<const uint4*>(rowp + 8 * q), x);
      } else {
        const float* fp = reinterpret_cast<const float*>(src) + (lh_row0 + pos) * D + 8 * q;
        float4 a = *reinterpret_cast<const float4*>(fp), b = *reinterpret_cast<const float4*>(fp + 4);
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
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
            float ya = lower ? x[e] : pr[e], yb = lower ? pr[e] : x[e];
            float yb_s = __fmul_rn(yb, cs.y), ya_s = __fmul_rn(ya, cs.y);
            x[e] = lower ? __fmaf_rn(ya, cs.x, yb_s) : __fmaf_rn(yb, cs.x, -ya_s);
          }
        } else {
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            float2 cs = rr[4 * q + m];
            float ya = x[2 * m], yb = x[2 * m + 1];
            float yb_s = __fmul_rn(yb, cs.y), ya_s = __fmul_rn(ya, cs.y);
            x[2 * m] = __fmaf_rn(ya, cs.x, yb_s);
            x[2 * m + 1] = __fmaf_rn(yb, cs.x, -ya_s);
          }
        }
        if (p.dtype == KVTC_BF16) {
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = round_bf16(x[e]);
        }
      }
      float c[8];
      if (transform) {
        static_assert((D & (D - 1)) == 0, "sum / D is a power-of-two scaling");
        double ss = 0.0;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = __fma_rn((double)x[e], (double)x[e], ss);
        ss += xor16<1>(ss);
        ss += xor16<2>(ss);
        ss += xor16<4>(ss);
        ss += xor16<8>(ss);
        const float rt = (float)__dsqrt_rn(ss * (1.0 / D));
        double y[8];
        float xn[8];
        div_f32(x, rt, xn);  // x / r, exactly rounded
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = rt == 0.0f ? 0.0 : (double)xn[e];
        wht_fp64(y, q);  // channel strides 1, 2, 4 in the lane, then 8 .. 64 across the row
        const double rs = __dsqrt_rn((double)D);
        quot_f32(y, rs, __ddiv_rn(1.0, rs), c);  // y / sqrt(D), exactly rounded
        if (q == 0) {
          if (MODE == 0) reinterpret_cast<float*>(p.out + p.r_off)[r_index * p.T_mid + t0 + tok] = rt;
          if (MODE == 2 && r_out) r_out[(int64_t)(u - sec0) * p.T_mid + t0 + tok] = rt;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) c[e] = x[e];
      }
      if constexpr (MODE == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          sum[e] += (double)c[e];
          sq[e] = __fma_rn((double)c[e], (double)c[e], sq[e]);
          mn[e] = fminf(mn[e], c[e]);
          mx[e] = fmaxf(mx[e], c[e]);
        }
      } else if constexpr (MODE == 1) {
        if (bl > 0) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            uint32_t qi;
            if (sym) {
              // symmetric: clamp(rint(c * rcp), -Q, Q) + 2^(b-1)
              const float Q = (float)((1 << (bl - 1)) - 1);
              float v = __fmul_rn(c[e], rc[e]);
              float qq = fminf(fmaxf(__builtin_rintf(v), -Q), Q);
              qi = (uint32_t)((int)qq + (1 << (bl - 1)));
            } else {
              float v = __fmul_rn(__fsub_rn(c[e], zr[e]), rc[e]);
              qi = (uint32_t)fminf(fmaxf(__builtin_rintf(v), 0.0f), qmax[e]);
            }
            const int i = 8 * q + e;
            const uint32_t bitpos = (uint32_t)tb * bl;
            const uint32_t wi = (uint32_t)i * row_words + (bitpos >> 5), sh = bitpos & 31;
            atomicOr(&tilebuf[wi], qi << sh);
            if (sh + bl > 32) atomicOr(&tilebuf[wi + 1], qi >> (32 - sh));
          }
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) coef_out[((int64_t)(u - sec0) * p.T_mid + t0 + tok) * D + 8 * q + e] = c[e];
      }
    }
    if constexpr (MODE == 1) {
      __syncthreads();
      uint32_t* dst = slot + (int64_t)tl * row_words_full * D;
      for (uint32_t i = threadIdx.x; i < row_words * D; i += blockDim.x) dst[i] = tilebuf[i];
      __syncthreads();
    }
  }
  if constexpr (MODE == 0) {
    // reduce the 16 token groups of the block: lanes with equal q in the
    // 16 groups (4 per wave, 4 waves), fixed order
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int o = 16; o <= 32; o <<= 1) {
        sum[e] += __shfl_xor(sum[e], o, 64);
        sq[e] += __shfl_xor(sq[e], o, 64);
        mn[e] = fminf(mn[e], __shfl_xor(mn[e], o, 64));
        mx[e] = fmaxf(mx[e], __shfl_xor(mx[e], o, 64));
      }
    __shared__ double s_sum[4][D], s_sq[4][D];
    __shared__ float s_mn[4][D], s_mx[4][D];
    const int wave = threadIdx.x >> 6;
    if ((lane >> 4) == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        int i = 8 * q + e;
        s_sum[wave][i] = sum[e]; s_sq[wave][i] = sq[e]; s_mn[wave][i] = mn[e]; s_mx[wave][i] = mx[e];
      }
    }
    __syncthreads();
    if (threadIdx.x < D) {
      int i = threadIdx.x;
      double a = s_sum[0][i], b = s_sq[0][i];
      float c = s_mn[0][i], d = s_mx[0][i];
      for (int w2 = 1; w2 < 4; ++w2) {
        a += s_sum[w2][i]; b += s_sq[w2][i];
        c = fminf(c, s_mn[w2][i]); d = fmaxf(d, s_mx[w2][i]);
      }
      int64_t idx = ((int64_t)u * p.blks_per_sec + ch) * D + i;
      reinterpret_cast<double*>(p.ws + p.w.part_sum)[idx] = a;
      reinterpret_cast<double*>(p.ws + p.w.part_sq)[idx] = b;
      reinterpret_cast<float*>(p.ws + p.w.part_min)[idx] = c;
      reinterpret_cast<float*>(p.ws + p.w.part_max)[idx] = d;
    }
  }
}

// ---------------------------------------------------------------------------
// head_dim 128, bf16 cache: RoPE removed from the mid-region keys ahead of the
// projection passes (Codec-Gauge "Problem Statement and Overview"; KVTC
// undoes the rotation before the transform).  x_a = fma(y_a, c, fp32(y_b s)),
// x_b = fma(y_b, c, -fp32(y_a s)), rounded to bf16, into a copy laid out
// [layer][head][mid token][channel] in the workspace.  A workgroup takes 16
// positions of one layer: their table rows are read once into LDS with
// coalesced loads and applied to every head.  Lane q of a row's 8 lanes holds
// channels [8q, 8q+8) and [64+8q, 64+8q+8), which contain both members of
// each of its RoPE pairs in either pairing style.
// ---------------------------------------------------------------------------

// LDS image of a table row: pair j at float offset 18 (j / 8) + 2 (j % 8), so
// the 8 lanes of a row read 8 distinct bank pairs in either pairing style.
__device__ __forceinline__ int cs_at(int t, int j) { return t * 144 + 18 * (j >> 3) + 2 * (j & 7); }

__global__ __launch_bounds__(256) void k_unrope128(const Params p0) {
  const Params p = at_seq(p0, blockIdx.z);
  if (p0.n_seqs == 0 && blockIdx.x == 0 && blockIdx.y == 0) clear_status_block(p);
  constexpr int D = 128;
  const int l = blockIdx.y, t0 = blockIdx.x * 16;
  const int nt = min(16, p.T_mid - t0);
  if (nt <= 0) return;
  const int tid = threadIdx.x;
  __shared__ __attribute__((aligned(16))) float cs[16 * 144];
  {
    const float2* srow = p.rope + (int64_t)(p.mid_begin + t0) * 64;
    for (int i = tid; i < nt * 64; i += 256)
      *reinterpret_cast<float2*>(cs + cs_at(i >> 6, i & 63)) = srow[i];
  }
  __syncthreads();
  const int q = tid & 7;
  const bool half = p.rope_style == KVTC_ROPE_HALF;
  const uint16_t* kin = reinterpret_cast<const uint16_t*>(p.k);
  uint16_t* kout = reinterpret_cast<uint16_t*>(p.ws + p.w.kprime);
  const int rows = p.H * nt;
  // row ri = (token t = ri / H, head h = ri % H): the lanes of a wave share a
  // token (table reads broadcast); each thread loads four rows before using them
  for (int ri0 = tid >> 3; ri0 < rows; ri0 += 4 * 32) {
    uint4 a[4], b[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int ri = min(ri0 + 32 * k, rows - 1);
      const int t = ri / p.H, h = ri % p.H;
      const uint16_t* in = kin + cache_row(p, l, h, p.mid_begin + t0 + t);
      a[k] = *reinterpret_cast<const uint4*>(in + 8 * q);
      b[k] = *reinterpret_cast<const uint4*>(in + 64 + 8 * q);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int ri = ri0 + 32 * k;
      if (ri >= rows) break;
      const int t = ri / p.H, h = ri % p.H;
      float ya[8], yb[8];
      unpack_bf16x8(a[k], ya);
      unpack_bf16x8(b[k], yb);
      if (half) {
        // pair j = 8q + e: (channel j, channel j + 64)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float2 c = *reinterpret_cast<const float2*>(cs + cs_at(t, 8 * q + e));
          const float xa = __fmaf_rn(ya[e], c.x, __fmul_rn(yb[e], c.y));
          const float xb = __fmaf_rn(yb[e], c.x, -__fmul_rn(ya[e], c.y));
          ya[e] = xa;
          yb[e] = xb;
        }
      } else {
        // pairs (2m, 2m + 1): m = 4q + e/2 in the low run, 32 + 4q + e/2 in the high run
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const float2 cl = *reinterpret_cast<const float2*>(cs + cs_at(t, 4 * q + m));
          const float2 ch = *reinterpret_cast<const float2*>(cs + cs_at(t, 32 + 4 * q + m));
          const float a0 = ya[2 * m], a1 = ya[2 * m + 1], b0 = yb[2 * m], b1 = yb[2 * m + 1];
          ya[2 * m] = __fmaf_rn(a0, cl.x, __fmul_rn(a1, cl.y));
          ya[2 * m + 1] = __fmaf_rn(a1, cl.x, -__fmul_rn(a0, cl.y));
          yb[2 * m] = __fmaf_rn(b0, ch.x, __fmul_rn(b1, ch.y));
          yb[2 * m + 1] = __fmaf_rn(b1, ch.x, -__fmul_rn(b0, ch.y));
        }
      }
      uint16_t* o = kout + (((int64_t)l * p.H + h) * p.T_mid + t0 + t) * D;
      *reinterpret_cast<uint4*>(o + 8 * q) =
          make_uint4(pack2_bf16(ya[0], ya[1]), pack2_bf16(ya[2], ya[3]), pack2_bf16(ya[4], ya[5]), pack2_bf16(ya[6], ya[7]));
      *reinterpret_cast<uint4*>(o + 64 + 8 * q) =
          make_uint4(pack2_bf16(yb[0], yb[1]), pack2_bf16(yb[2], yb[3]), pack2_bf16(yb[4], yb[5]), pack2_bf16(yb[6], yb[7]));
    }
  }
}

// ---------------------------------------------------------------------------
// head_dim 128, bf16 cache: the bandwidth-oriented projection pass.
//
// A workgroup (4 waves) walks its chunk in 64-token sub-tiles.  Staging:
// thread (token tid/4, quarter tid%4) loads the channel runs [16q, 16q+16)
// and [64+16q, 64+16q+16) of its token -- both members of every RoPE pair --
// undoes RoPE, rounds to bf16 and writes the row into a double-buffered LDS
// tile; the loads of the next sub-tile are issued before the MFMA phase of
// the current one.  MFMA: wave w owns components [32w, 32w+32) (its basis
// rows, 32 VGPRs, stay in registers) and reads the token rows from LDS with
// the K slice of lane group g = channels 32kb + 8g .. +7.  The result lane
// (g, r) holds component (2w+m)*16 + r of tokens 16kk + 4g .. +3.
// ---------------------------------------------------------------------------

constexpr int kXS = 136;  // LDS row stride (bf16) of staged tokens: 16-B aligned, 4-bank shift

template <int MODE>
__global__ __launch_bounds__(256, MODE == 0 ? 3 : 1) void k_enc128(const Params p0, int sec0, float* coef_out) {
  const Params p = at_seq(p0, blockIdx.z);
  if (MODE == 0 && p0.n_seqs == 0 && !p.rope_keys && blockIdx.x == 0 && blockIdx.y == 0) clear_status_block(p);
  constexpr int D = 128;
  // the statistics pass walks the sections backwards: the RoPE pass has just
  // written the last layers' keys, and the quantiser, which walks forwards,
  // then starts on the rows read last; both find more of them in the
  // memory-side cache
  const int u = (MODE == 0 ? (int)gridDim.y - 1 - (int)blockIdx.y : (int)blockIdx.y) + sec0, ch = blockIdx.x;
  const int h = u % p.H, s = (u / p.H) & 1, l = u / (2 * p.H);
  const int t0 = ch * p.blk_tokens;
  const int n = min(p.blk_tokens, p.T_mid - t0);
  if (n <= 0) return;
  if (MODE == 1 && (get_status(p.ws, p.w) & (1u << KVTC_ERR_NONFINITE))) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, r = lane & 15;
  const int st_t = tid >> 2, st_q = tid & 3;
  // keys with RoPE come from the workspace copy with the rotation removed
  // (k_unrope128), except for the coefficient export, which has no workspace
  const bool pre = MODE != 2 && s == 0 && p.rope_keys;
  const uint16_t* src = pre ? reinterpret_cast<const uint16_t*>(p.ws + p.w.kprime)
                            : reinterpret_cast<const uint16_t*>(s ? p.v : p.k);
  // only the coefficient export rotates in place (the passes read un-rotated keys)
  const bool rope = MODE == 2 && !pre && (s == 0) && p.rope_keys;
  const int64_t lh_row0 = ((int64_t)l * p.H + h) * (pre ? p.T_mid : p.T);
  const int pos_base = pre ? 0 : p.mid_begin;
  const int64_t bi = basis_index(p, l, s, h) * D * D;
  const uint16_t* bt = reinterpret_cast<const uint16_t*>(p.basis_t) + bi;

  __shared__ __attribute__((aligned(16))) uint16_t X[2][64 * kXS];
  __shared__ SideLds sd;
  extern __shared__ uint32_t tilebuf[];

  uint4 bq[2][4];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      bq[m][kb] = *reinterpret_cast<const uint4*>(bt + (int64_t)((2 * wave + m) * 16 + r) * D + kb * 32 + 8 * g);

  // per-lane statistics / side information of the lane's two components
  double sum[2] = {0.0, 0.0}, sq[2] = {0.0, 0.0};
  float mn[2] = {INFINITY, INFINITY}, mx[2] = {-INFINITY, -INFINITY};
  float zr[2] = {0.f, 0.f}, rc[2] = {0.f, 0.f}, qmax[2] = {0.f, 0.f};
  uint32_t bl[2] = {0u, 0u};
  uint32_t full_words = 0;
  uint32_t* slot = nullptr;
  if constexpr (MODE == 1) {
    if (tid < D) {
      const int64_t si = (int64_t)u * D + tid;
      sd.zero[tid] = reinterpret_cast<const float*>(p.ws + p.w.side_zero)[si];
      sd.rcp[tid] = reinterpret_cast<const float*>(p.ws + p.w.side_rcp)[si];
      sd.bits[tid] = p.ws[p.w.side_bits + si];
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int i = (2 * wave + m) * 16 + r;
      zr[m] = sd.zero[i]; rc[m] = sd.rcp[i]; bl[m] = sd.bits[i];
      qmax[m] = (float)((1u << bl[m]) - 1u);
    }
    for (int i = 0; i < D; ++i) full_words += (uint32_t)((p.tile_tokens * (int)sd.bits[i] + 31) >> 5);
    slot = reinterpret_cast<uint32_t*>(p.ws + p.w.packed + (int64_t)(u * p.blks_per_sec + ch) * p.w.packed_slot);
  }

  // ---- staging registers and helpers
  float4 cs[8];
  auto load_sub = [&](int sub, uint4 (&y)[4]) {
    const int tok = sub * 64 + st_t;
    const bool valid = tok < n;
    const int pos = p.mid_begin + t0 + tok;
    y[0] = y[1] = y[2] = y[3] = make_uint4(0, 0, 0, 0);
    if (valid) {
      const uint16_t* row = src + (pre ? (lh_row0 + pos_base + t0 + tok) * D : cache_row(p, l, h, pos));
      y[0] = *reinterpret_cast<const uint4*>(row + 16 * st_q);
      y[1] = *reinterpret_cast<const uint4*>(row + 16 * st_q + 8);
      y[2] = *reinterpret_cast<const uint4*>(row + 64 + 16 * st_q);
      y[3] = *reinterpret_cast<const uint4*>(row + 64 + 16 * st_q + 8);
    }
    if (rope && valid) {
      if (p.rope_style == KVTC_ROPE_HALF) {  // pairs [16q, 16q+16)
        const float4* cr = reinterpret_cast<const float4*>(p.rope + (int64_t)pos * 64 + 16 * st_q);
#pragma unroll
        for (int k = 0; k < 8; ++k) cs[k] = cr[k];
      } else {  // interleaved: pairs [8q, 8q+8) and [32+8q, 32+8q+8)
        const float4* cl = reinterpret_cast<const float4*>(p.rope + (int64_t)pos * 64 + 8 * st_q);
        const float4* ch2 = reinterpret_cast<const float4*>(p.rope + (int64_t)pos * 64 + 32 + 8 * st_q);
#pragma unroll
        for (int k = 0; k < 4; ++k) { cs[k] = cl[k]; cs[4 + k] = ch2[k]; }
      }
    }
  };
  auto stage_sub = [&](int buf, const uint4 (&y)[4]) {
    uint16_t* xr = &X[buf][st_t * kXS];
    if (!rope) {  // the loaded bf16 words as they are
      *reinterpret_cast<uint4*>(xr + 16 * st_q) = y[0];
      *reinterpret_cast<uint4*>(xr + 16 * st_q + 8) = y[1];
      *reinterpret_cast<uint4*>(xr + 64 + 16 * st_q) = y[2];
      *reinterpret_cast<uint4*>(xr + 64 + 16 * st_q + 8) = y[3];
      return;
    }
    float lo[16], hi[16];
    unpack_bf16x8(y[0], lo); unpack_bf16x8(y[1], lo + 8);
    unpack_bf16x8(y[2], hi); unpack_bf16x8(y[3], hi + 8);
    uint4 o[4];
    if (rope) {
      if (p.rope_style == KVTC_ROPE_HALF) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float c = (e & 1) ? cs[e >> 1].z : cs[e >> 1].x;
          const float sn = (e & 1) ? cs[e >> 1].w : cs[e >> 1].y;
          const float ya = lo[e], yb = hi[e];
          lo[e] = __fmaf_rn(ya, c, __fmul_rn(yb, sn));
          hi[e] = __fmaf_rn(yb, c, -__fmul_rn(ya, sn));
        }
      } else {
#pragma unroll
        for (int m = 0; m < 8; ++m) {
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            float* v = half ? hi : lo;
            const float4 q4 = cs[4 * half + (m >> 1)];
            const float c = (m & 1) ? q4.z : q4.x;
            const float sn = (m & 1) ? q4.w : q4.y;
            const float ya = v[2 * m], yb = v[2 * m + 1];
            v[2 * m] = __fmaf_rn(ya, c, __fmul_rn(yb, sn));
            v[2 * m + 1] = __fmaf_rn(yb, c, -__fmul_rn(ya, sn));
          }
        }
      }
    }
    o[0] = make_uint4(pack2_bf16(lo[0], lo[1]), pack2_bf16(lo[2], lo[3]), pack2_bf16(lo[4], lo[5]), pack2_bf16(lo[6], lo[7]));
    o[1] = make_uint4(pack2_bf16(lo[8], lo[9]), pack2_bf16(lo[10], lo[11]), pack2_bf16(lo[12], lo[13]), pack2_bf16(lo[14], lo[15]));
    o[2] = make_uint4(pack2_bf16(hi[0], hi[1]), pack2_bf16(hi[2], hi[3]), pack2_bf16(hi[4], hi[5]), pack2_bf16(hi[6], hi[7]));
    o[3] = make_uint4(pack2_bf16(hi[8], hi[9]), pack2_bf16(hi[10], hi[11]), pack2_bf16(hi[12], hi[13]), pack2_bf16(hi[14], hi[15]));
    *reinterpret_cast<uint4*>(xr + 16 * st_q) = o[0];
    *reinterpret_cast<uint4*>(xr + 16 * st_q + 8) = o[1];
    *reinterpret_cast<uint4*>(xr + 64 + 16 * st_q) = o[2];
    *reinterpret_cast<uint4*>(xr + 64 + 16 * st_q + 8) = o[3];
  };

  const int nsub = (n + 63) / 64;
  const int subs_per_tile = p.tile_tokens / 64 > 0 ? p.tile_tokens / 64 : 1;
  uint32_t refined = 0;  // codes re-computed exactly (wave-uniform count)
  // the loop body after staging (sub-tile sub in X[sub & 1])
  auto body = [&](int sub) {
    const int buf = sub & 1;
    // packed-tile bookkeeping (tile_tokens is a multiple of 64 on this path)
    const int tl = (sub * 64) / p.tile_tokens;
    const int ta = tl * p.tile_tokens;
    const int nt = min(p.tile_tokens, n - ta);
    if constexpr (MODE == 1) {
      if (sub % subs_per_tile == 0) {
        if (tid < 64) {
          uint32_t w0 = (uint32_t)((nt * (int)sd.bits[2 * lane] + 31) >> 5);
          uint32_t w1 = (uint32_t)((nt * (int)sd.bits[2 * lane + 1] + 31) >> 5);
          uint32_t tot;
          uint32_t ex = wave_excl_scan(w0 + w1, &tot);
          sd.row_w[2 * lane] = ex;
          sd.row_w[2 * lane + 1] = ex + w0;
          if (lane == 0) sd.row_w[D] = tot;
        }
        __syncthreads();
        for (uint32_t i = tid; i < sd.row_w[D]; i += 256) tilebuf[i] = 0;
      }
    }
    // the staged rows are complete (an LDS-only barrier: the next sub-tile's
    // loads stay in flight)
    if constexpr (MODE == 1) __syncthreads();
    else lds_barrier();
    // the 16-token groups kk of the sub-tile: tokens 16 kk + r as A rows
    auto project = [&](int kk, f32x4_t (&a2)[2]) {
      a2[0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      a2[1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const uint4 a = *reinterpret_cast<const uint4*>(&X[buf][(kk * 16 + r) * kXS + kb * 32 + 8 * g]);
        const bf16x8_t av = __builtin_bit_cast(bf16x8_t, a);
#pragma unroll
        for (int m = 0; m < 2; ++m)
          a2[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8_t, bq[m][kb]), a2[m], 0, 0, 0);
      }
    };
    if constexpr (MODE == 0) {
      // each group is folded into the statistics right after its products
      // (eight accumulator registers live, not 32), in the same order
      // min / max as med3 against -inf / +inf: one instruction each (finite
      // coefficients; non-finite inputs are caught by the fp64 sums)
      auto accumulate = [&](float c, int m) {
        sum[m] += (double)c;
        sq[m] = __fma_rn((double)c, (double)c, sq[m]);
        mn[m] = __builtin_amdgcn_fmed3f(c, mn[m], -INFINITY);
        mx[m] = __builtin_amdgcn_fmed3f(c, mx[m], INFINITY);
      };
      const bool full_sub = sub * 64 + 64 <= n;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        f32x4_t a2[2];
        project(kk, a2);
        if (full_sub) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int m = 0; m < 2; ++m) accumulate(a2[m][e], m);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (sub * 64 + kk * 16 + 4 * g + e < n) {
#pragma unroll
              for (int m = 0; m < 2; ++m) accumulate(a2[m][e], m);
            }
        }
      }
      return;
    }
    f32x4_t acc[4][2];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) project(kk, acc[kk]);
    if constexpr (MODE == 2) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int tk = sub * 64 + kk * 16 + 4 * g + e;
          if (tk < n) {
#pragma unroll
            for (int m = 0; m < 2; ++m)
              coef_out[((int64_t)(u - sec0) * p.T_mid + t0 + tk) * D + (2 * wave + m) * 16 + r] = acc[kk][m][e];
          }
        }
    } else {
      // quantise; values within their error of a rounding boundary are
      // recomputed exactly from the staged row (fp64 sum of exact products)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int tt = sub * 64 + kk * 16 + 4 * g - ta;  // first of the lane's 4 tokens, tile-relative
        // token norms for the coefficient error bound
        float ecm[4];
        {
          float n2 = 0.f;
          const uint16_t* xr = &X[buf][(kk * 16 + r) * kXS];
#pragma unroll
          for (int c8 = 0; c8 < 4; ++c8) {
            const uint4 a = *reinterpret_cast<const uint4*>(xr + c8 * 32 + 8 * g);
            float f[8];
            unpack_bf16x8(a, f);
#pragma unroll
            for (int z = 0; z < 8; ++z) n2 = __fmaf_rn(f[z], f[z], n2);
          }
          n2 += __shfl_xor(n2, 16, 64);
          n2 += __shfl_xor(n2, 32, 64);
#pragma unroll
          for (int e = 0; e < 4; ++e) ecm[e] = p.mfma_err * __fsqrt_rn(__shfl(n2, 4 * g + e, 64));
        }
        uint32_t qv[2] = {0u, 0u};
        uint32_t flags = 0;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          if (bl[m] == 0) continue;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float v = __fmul_rn(__fsub_rn(acc[kk][m][e], zr[m]), rc[m]);
            const float rv = __builtin_rintf(v);
            const float q = fminf(fmaxf(rv, 0.0f), qmax[m]);
            if (tt + e < nt) {
              qv[m] |= (uint32_t)q << (8 * e);
              const float ev = __fmaf_rn(ecm[e], rc[m], 3.0f * 0x1p-23f * fmaxf(fabsf(v), 1.0f));
              if (fabsf(fabsf(__fsub_rn(v, rv)) - 0.5f) < ev) flags |= 1u << (m * 4 + e);
            }
          }
        }
        uint64_t pend = __ballot(flags != 0);
        while (pend) {
          const int L = __ffsll((unsigned long long)pend) - 1;
          const uint32_t fl = __shfl(flags, L, 64);
          const int bit = __ffs(fl) - 1;
          const int mx_ = bit >> 2, ex = bit & 3;
          ++refined;
          const int tx = kk * 16 + 4 * (L >> 4) + ex;     // token within the sub-tile
          const int ix = (2 * wave + mx_) * 16 + (L & 15);  // component
          const uint32_t xw = *reinterpret_cast<const uint32_t*>(&X[buf][tx * kXS + 2 * lane]);
          const uint32_t bw = *reinterpret_cast<const uint32_t*>(bt + (int64_t)ix * D + 2 * lane);
          double part = __fma_rn((double)__uint_as_float(xw << 16), (double)__uint_as_float(bw << 16),
                                 (double)__uint_as_float(xw & 0xffff0000u) *
                                     (double)__uint_as_float(bw & 0xffff0000u));
#pragma unroll
          for (int o = 32; o > 0; o >>= 1) part += __shfl_xor(part, o, 64);
          if (lane == L) {
            const float cex = (float)part;
            const float v = __fmul_rn(__fsub_rn(cex, sd.zero[ix]), sd.rcp[ix]);
            const float q = fminf(fmaxf(__builtin_rintf(v), 0.0f), (float)((1u << sd.bits[ix]) - 1u));
#pragma unroll
            for (int m = 0; m < 2; ++m)
              if (m == mx_) qv[m] = (qv[m] & ~(0xffu << (8 * ex))) | ((uint32_t)q << (8 * ex));
            flags &= ~(1u << bit);
          }
          pend = __ballot(flags != 0);
        }
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const uint32_t b = bl[m];
          if (b == 0 || tt >= nt) continue;
          const uint32_t word = (qv[m] & 0xffu) | (((qv[m] >> 8) & 0xffu) << b) |
                                (((qv[m] >> 16) & 0xffu) << (2 * b)) | ((qv[m] >> 24) << (3 * b));
          const uint32_t bitpos = (uint32_t)tt * b;
          const uint32_t wi = sd.row_w[(2 * wave + m) * 16 + r] + (bitpos >> 5), sh = bitpos & 31;
          atomicOr(&tilebuf[wi], word << sh);
          const uint32_t spill = sh + 4 * b > 32 ? word >> (32 - sh) : 0u;
          if (spill) atomicOr(&tilebuf[wi + 1], spill);
        }
      }
      // flush a finished packed tile
      if ((sub % subs_per_tile) == subs_per_tile - 1 || sub == nsub - 1) {
        __syncthreads();
        uint32_t* dst = slot + (int64_t)tl * full_words;
        for (uint32_t i = tid; i < sd.row_w[D]; i += 256) dst[i] = tilebuf[i];
        __syncthreads();
      }
    }
  };
  uint4 yA[4], yB[4];
  if constexpr (MODE == 0) {
    // rows two sub-tiles ahead in flight: the sub-tile after next is loaded
    // into the registers just staged
    load_sub(0, yA);
    if (1 < nsub) load_sub(1, yB);
    for (int sub = 0; sub < nsub; sub += 2) {
      stage_sub(0, yA);
      if (sub + 2 < nsub) load_sub(sub + 2, yA);
      body(sub);
      if (sub + 1 < nsub) {
        stage_sub(1, yB);
        if (sub + 3 < nsub) load_sub(sub + 3, yB);
        body(sub + 1);
      }
    }
  } else {
    load_sub(0, yA);
    for (int sub = 0; sub < nsub; ++sub) {
      stage_sub(sub & 1, yA);
      if (sub + 1 < nsub) load_sub(sub + 1, yA);
      body(sub);
    }
  }
  if (MODE == 1 && lane == 0 && refined) atomicAdd(count_slot(p.ws, p.w), refined);
  if constexpr (MODE == 0) {
#pragma unroll
    for (int m = 0; m < 2; ++m) {
#pragma unroll
      for (int o = 16; o <= 32; o <<= 1) {
        sum[m] += __shfl_xor(sum[m], o, 64);
        sq[m] += __shfl_xor(sq[m], o, 64);
        mn[m] = fminf(mn[m], __shfl_xor(mn[m], o, 64));
        mx[m] = fmaxf(mx[m], __shfl_xor(mx[m], o, 64));
      }
      if (g == 0) {
        const int64_t idx = ((int64_t)u * p.blks_per_sec + ch) * D + (2 * wave + m) * 16 + r;
        reinterpret_cast<double*>(p.ws + p.w.part_sum)[idx] = sum[m];
        reinterpret_cast<double*>(p.ws + p.w.part_sq)[idx] = sq[m];
        reinterpret_cast<float*>(p.ws + p.w.part_min)[idx] = mn[m];
        reinterpret_cast<float*>(p.ws + p.w.part_max)[idx] = mx[m];
      }
    }
  }
}

static size_t quant_lds_bytes(const Params& p, size_t tile) {
  if (p.transform == KVTC_WHT) return tile;
  const size_t os = p.dtype == KVTC_BF16 ? 2 : 4;
  return (size_t)p.D * p.D * os + 4 * 16 * (size_t)p.D * os + tile;
}

static size_t tile_lds_bytes(const Params& p) {
  int32_t bmax = p.sec_bits_max;
  if (p.transform == KVTC_WHT) {
    int32_t b = p.bits_k_uniform > p.bits_v_uniform ? p.bits_k_uniform : p.bits_v_uniform;
    return (size_t)((p.tile_tokens * b + 31) / 32) * p.D * 4;
  }
  int32_t nz = bmax < p.D ? bmax : p.D;
  return (size_t)(((int64_t)p.tile_tokens * bmax + 31) / 32 + nz) * 4;
}

hipError_t launch_enc_transform(const Params& p, int mode, hipStream_t s) {
  dim3 grid(p.blks_per_sec, p.n_sections, seq_grid(p)), block(256);
  size_t lds = mode == 1 ? quant_lds_bytes(p, tile_lds_bytes(p)) : 0;
  if (p.transform == KVTC_WHT) {
    if (mode == 0) hipLaunchKernelGGL(k_enc_wht<0>, grid, block, 0, s, p, 0, (float*)nullptr, (float*)nullptr);
    else hipLaunchKernelGGL(k_enc_wht<1>, grid, block, lds, s, p, 0, (float*)nullptr, (float*)nullptr);
    return hipGetLastError();
  }
  if (p.D == 128 && p.dtype == KVTC_BF16 && (p.tile_tokens % 64) == 0) {
    if (mode == 0) {
      if (p.rope_keys) hipLaunchKernelGGL(k_unrope128, dim3((p.T_mid + 15) / 16, p.L, seq_grid(p)), dim3(256), 0, s, p);
      hipLaunchKernelGGL(k_enc128<0>, grid, block, 0, s, p, 0, (float*)nullptr);
    } else {
      return launch_quant128(p, s);
    }
    return hipGetLastError();
  }
#define KVTC_LAUNCH_PCA(D_, DT_)                                                              \
  if (p.D == D_ && p.dtype == DT_) {                                                          \
    if (mode == 0) {                                                                          \
      hipLaunchKernelGGL((k_enc_pca<D_, DT_, 0>), grid, block, 0, s, p, 0, (float*)nullptr);  \
    } else {                                                                                  \
      (void)hipFuncSetAttribute((const void*)k_enc_pca<D_, DT_, 1>,                          \
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);       \
      hipLaunchKernelGGL((k_enc_pca<D_, DT_, 1>), grid, block, lds, s, p, 0, (float*)nullptr); \
    }                                                                                         \
    return hipGetLastError();                                                                 \
  }
  KVTC_LAUNCH_PCA(128, KVTC_BF16)
  KVTC_LAUNCH_PCA(64, KVTC_BF16)
  KVTC_LAUNCH_PCA(64, KVTC_FP32)
#undef KVTC_LAUNCH_PCA
  return hipErrorInvalidValue;
}

hipError_t launch_coeffs(const Params& p, int sec_begin, int sec_end, float* out, float* r_out,
                         hipStream_t s) {
  dim3 grid(p.blks_per_sec, sec_end - sec_begin), block(256);
  if (p.transform == KVTC_WHT) {
    hipLaunchKernelGGL(k_enc_wht<2>, grid, block, 0, s, p, sec_begin, out, r_out);
    return hipGetLastError();
  }
  if (p.D == 128 && p.dtype == KVTC_BF16 && (p.tile_tokens % 64) == 0)
    hipLaunchKernelGGL(k_enc128<2>, grid, block, 0, s, p, sec_begin, out);
  else if (p.D == 128 && p.dtype == KVTC_BF16)
    hipLaunchKernelGGL((k_enc_pca<128, KVTC_BF16, 2>), grid, block, 0, s, p, sec_begin, out);
  else if (p.D == 64 && p.dtype == KVTC_BF16)
    hipLaunchKernelGGL((k_enc_pca<64, KVTC_BF16, 2>), grid, block, 0, s, p, sec_begin, out);
  else if (p.D == 64 && p.dtype == KVTC_FP32)
    hipLaunchKernelGGL((k_enc_pca<64, KVTC_FP32, 2>), grid, block, 0, s, p, sec_begin, out);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// allocation and side information, one workgroup (D threads) per section
// ("Bit Budget Is Not Fair": uneven widths; CompressedSection: scales, zero
// points, bit widths)
// ---------------------------------------------------------------------------

// Exact ordering key of var * 4^-k: (extended exponent, 24-bit significand),
// then the component index reversed so that lower indices win ties.
__device__ __forceinline__ uint64_t alloc_key(float var, int k, int i) {
  uint32_t bits = __float_as_uint(var);
  int32_t ex = (int32_t)(bits >> 23);
  uint32_t man = bits & 0x7fffffu;
  if (ex == 0) {  // subnormal: normalise the significand
    int sh = __clz(man) - 8;
    man = (man << sh) & 0x7fffffu;
    ex = 1 - sh;
  }
  uint64_t e2 = (uint64_t)(ex - 2 * k + 256);  // > 0 for every fp32 value and k <= 8
  return (((e2 << 23) | man) << 8) | (uint64_t)(255 - i);
}

// Ordering key of var * 4^-k for the one-budget allocation over all
// sections: (extended exponent, significand, then the (section, component)
// index reversed in 20 bits so that lower indices win ties), 53 bits.
__device__ __forceinline__ void var_exp_man(float var, int32_t& ex, uint32_t& man) {
  const uint32_t bits = __float_as_uint(var);
  ex = (int32_t)(bits >> 23);
  man = bits & 0x7fffffu;
  if (ex == 0) {  // subnormal: normalise the significand
    const int sh = __clz(man) - 8;
    man = (man << sh) & 0x7fffffu;
    ex = 1 - sh;
  }
}
constexpr int kGKeyLow = 43;  // bits below the exponent field: 23 significand + 20 index
__device__ __forceinline__ uint64_t global_key(int32_t ex, uint32_t man, int k, int64_t idx) {
  const uint64_t e2 = (uint64_t)(ex - 2 * k + 256);  // in [220, 510]
  return (e2 << kGKeyLow) | ((uint64_t)man << 20) | (uint64_t)(0xfffffu - (uint32_t)idx);
}

// One wave per section; lane l holds components l and l + 64 (head_dim 128).
// MODE 0: statistics, the section's own greedy widths and side information.
// MODE 1 (one budget over all sections): statistics only, for k_alloc_global.
// MODE 2: statistics, widths from the global threshold key, side information.
// MODE 3 / 4: as 0 / 2 from statistics already in the workspace (the
// allocation stage hook).
template <int MODE>
__global__ __launch_bounds__(64) void k_enc_alloc(const Params p0) {
  constexpr bool FROM_STATS = MODE >= 3;
  constexpr bool GLOBAL_W = MODE == 2 || MODE == 4;
  const Params p = at_seq(p0, blockIdx.z);
  const int u = blockIdx.x;
  const int D = p.D;
  const int lane = threadIdx.x;
  const int NC = D / 64;  // components per lane
  const int s = (u / p.H) & 1;
  uint8_t* rec = p.out + p.side_off + (int64_t)u * 9 * D;
  const int64_t N = p.T_mid;
  float mu[2] = {0.f, 0.f}, var[2] = {0.f, 0.f}, mn[2] = {0.f, 0.f}, mx[2] = {0.f, 0.f};
  bool nonfinite = false;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int i = lane + 64 * c;
    if (FROM_STATS) {
      if (c < NC) {
        const float4 st4 = reinterpret_cast<const float4*>(p.ws + p.w.sec_stats)[(int64_t)u * D + i];
        mu[c] = st4.x; var[c] = st4.y; mn[c] = st4.z; mx[c] = st4.w;
      }
      continue;
    }
    if (c < NC && N > 0) {
      double a = 0.0, b = 0.0;
      float lo = INFINITY, hi = -INFINITY;
      // the chunks' partials, eight chunks' loads in flight at a time
      for (int c0 = 0; c0 < p.blks_per_sec; c0 += 8) {
        double pa[8], pb[8];
        float pl[8], ph[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int ch = min(c0 + k, p.blks_per_sec - 1);
          const int64_t idx = ((int64_t)u * p.blks_per_sec + ch) * D + i;
          pa[k] = reinterpret_cast<const double*>(p.ws + p.w.part_sum)[idx];
          pb[k] = reinterpret_cast<const double*>(p.ws + p.w.part_sq)[idx];
          pl[k] = reinterpret_cast<const float*>(p.ws + p.w.part_min)[idx];
          ph[k] = reinterpret_cast<const float*>(p.ws + p.w.part_max)[idx];
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          if (c0 + k < p.blks_per_sec) {
            a += pa[k];
            b += pb[k];
            lo = fminf(lo, pl[k]);
            hi = fmaxf(hi, ph[k]);
          }
        }
      }
      nonfinite |= !isfinite(a) || !isfinite(b);
      const double m = a / (double)N;
      double vv = (b - a * m) / (double)N;
      if (vv < 0.0) vv = 0.0;
      mu[c] = (float)m;
      var[c] = (lo != hi) ? (float)vv : 0.0f;
      mn[c] = lo;
      mx[c] = hi;
    }
  }
  if (__ballot(nonfinite) && lane == 0) set_status(p.ws, p.w, KVTC_ERR_NONFINITE);
  if (MODE == 1) {
#pragma unroll
    for (int c = 0; c < 2; ++c)
      if (c < NC)
        reinterpret_cast<float4*>(p.ws + p.w.sec_stats)[(int64_t)u * D + lane + 64 * c] =
            make_float4(mu[c], var[c], mn[c], mx[c]);
    return;
  }
  // ---- bit widths ----
  uint32_t bits[2] = {0u, 0u};
  if (GLOBAL_W) {
    // every k whose key reaches the threshold (keys fall as k grows)
    const uint64_t thr = *reinterpret_cast<const uint64_t*>(p.ws + p.w.status + kGlobalThrOff);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      if (c >= NC || !(var[c] > 0.0f)) continue;
      int32_t ex;
      uint32_t man;
      var_exp_man(var[c], ex, man);
      const int64_t idx = (int64_t)u * D + lane + 64 * c;
      for (int k = 0; k < p.max_bits; ++k) bits[c] += global_key(ex, man, k, idx) >= thr ? 1u : 0u;
    }
  } else if (p.transform == KVTC_PCA) {
    const int budget = s == 0 ? p.budget_k : p.budget_v;
    // greedy marginal allocation == the `budget` largest var_i 4^-k (k < max_bits),
    // ranked by exact value then lowest index: find the budget-th largest key
    // by a bitwise search over the 41-bit keys.  The keys are formed once
    // (0 for no candidate, below every real key) and counted with ballots.
    uint64_t key[2][8];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int k = 0; k < 8; ++k)
        key[c][k] = (c < NC && var[c] > 0.0f && k < p.max_bits) ? alloc_key(var[c], k, lane + 64 * c) : 0ull;
    auto count_ge = [&](uint64_t thr) -> int {
      int cnt = 0;
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int k = 0; k < 8; ++k) cnt += (int)__popcll(__ballot(key[c][k] >= thr));
      return cnt;
    };
    uint64_t thr = 1;  // every real candidate key is >= 1
    if (count_ge(1) > budget) {
      uint64_t t = 0;
      for (int bit = 40; bit >= 0; --bit) {
        const uint64_t c2 = t | (1ull << bit);
        if (count_ge(c2) >= budget) t = c2;
      }
      thr = t;
    }
    if (budget > 0)
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int k = 0; k < 8; ++k) bits[c] += key[c][k] >= thr ? 1u : 0u;
  } else {
    bits[0] = bits[1] = (uint32_t)(s == 0 ? p.bits_k_uniform : p.bits_v_uniform);
  }
  // ---- side information ----
  const bool sym = p.transform == KVTC_WHT && s == 0;
  float amax = 0.f;
  if (sym) {
#pragma unroll
    for (int c = 0; c < 2; ++c)
      if (c < NC && N > 0) amax = fmaxf(amax, fmaxf(fabsf(mn[c]), fabsf(mx[c])));
    for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
  }
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    if (c >= NC) continue;
    const int i = lane + 64 * c;
    uint32_t b = bits[c];
    float zero = 0.f, scale = 0.f, rcp = 0.f;
    if (sym) {
      const int Q = (1 << (b - 1)) - 1;
      scale = (float)__ddiv_rn((double)amax, (double)Q);
      rcp = scale > 0.f ? __fdiv_rn(1.0f, scale) : 0.f;
      if (!(scale > 0.f) || isinf(rcp)) { scale = 0.f; rcp = 0.f; }
    } else if (b == 0) {
      zero = mu[c];
    } else {
      zero = mn[c];
      scale = (float)__ddiv_rn((double)mx[c] - (double)mn[c], (double)((1u << b) - 1u));
      rcp = scale > 0.f ? __fdiv_rn(1.0f, scale) : 0.f;
      if (!(scale > 0.f) || isinf(rcp)) { scale = 0.f; rcp = 0.f; }
    }
    if (N == 0) { b = 0; zero = 0.f; scale = 0.f; rcp = 0.f; }
    rec[i] = (uint8_t)b;
    reinterpret_cast<float*>(rec + D)[i] = zero;
    reinterpret_cast<float*>(rec + 5 * (int64_t)D)[i] = scale;
    const int64_t si = (int64_t)u * D + i;
    reinterpret_cast<float*>(p.ws + p.w.side_zero)[si] = zero;
    reinterpret_cast<float*>(p.ws + p.w.side_rcp)[si] = rcp;
    p.ws[p.w.side_bits + si] = (uint8_t)b;
    reinterpret_cast<float4*>(p.ws + p.w.sec_stats)[si] = make_float4(mu[c], var[c], mn[c], mx[c]);
  }
}

// One budget over all sections of a cache (of each sequence of a batch): the
// greedy marginal allocation over every component at once takes exactly the
// total_budget largest keys var * 4^-k (k < max_bits), so the widths follow
// from the total_budget-th largest key.  One workgroup finds that key by a
// most-significant-digit-first radix selection: the exponent field from a
// histogram of the variances' exponents (each variance contributes the
// exponents e - 2k of its keys), then the 43 low bits in four digits over the
// keys in the chosen exponent (at most one per component).
constexpr int kGDigits = 4;
__device__ __forceinline__ int gdigit_shift(int d) { return d < 3 ? 32 - 11 * d : 0; }
__device__ __forceinline__ int gdigit_bits(int d) { return d < 3 ? 11 : 10; }

__global__ __launch_bounds__(1024) void k_alloc_global(const Params p0) {
  const Params p = at_seq(p0, blockIdx.z);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t n = (int64_t)p.n_sections * p.D;
  const float4* st = reinterpret_cast<const float4*>(p.ws + p.w.sec_stats);
  uint64_t* thr_out = reinterpret_cast<uint64_t*>(p.ws + p.w.status + kGlobalThrOff);
  const int64_t B = p.T_mid > 0 ? p.total_budget : 0;
  const int mb = p.max_bits;
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t wsum[16];
  __shared__ int64_t s_total;
  __shared__ int32_t s_sel;
  __shared__ int64_t s_need;
  // -- exponents of the variances (fp32 exponent + 32, subnormals included)
  for (int i = tid; i < 2048; i += blockDim.x) hist[i] = 0u;
  if (tid == 0) s_total = 0;
  __syncthreads();
  uint32_t cand = 0;
  for (int64_t i = tid; i < n; i += blockDim.x) {
    const float v = st[i].y;
    if (!(v > 0.0f)) continue;
    int32_t ex;
    uint32_t man;
    var_exp_man(v, ex, man);
    atomicAdd(&hist[ex + 32], 1u);
    cand += (uint32_t)mb;
  }
  for (int o = 32; o > 0; o >>= 1) cand += __shfl_xor(cand, o, 64);
  if (lane == 0) atomicAdd((unsigned long long*)&s_total, (unsigned long long)cand);
  __syncthreads();
  if (B <= 0 || s_total <= B) {  // nothing to spend, or every candidate fits
    if (tid == 0) *thr_out = B <= 0 ? ~0ull : 1ull;
    return;
  }
  // -- the exponent field E = e - 2k + 256 of the B-th largest key: thread
  // t evaluates count(E >= t) over the exponent histogram
  {
    const int t = tid;  // candidate E values 0 .. 1023
    int64_t cnt = 0;
    for (int e = 0; e < 320; ++e) {
      const uint32_t h = hist[e];
      if (!h) continue;
      const int32_t top = (e - 32) + 256;  // E of k = 0
      // k in [0, mb) with top - 2k >= t
      const int32_t kk = top >= t ? (top - t) / 2 + 1 : 0;
      cnt += (int64_t)h * (kk < mb ? kk : mb);
    }
    // the largest t with count(E >= t) >= B; count(E >= t + 1) < B then
    const bool ok = cnt >= B;
    const uint64_t bl = __ballot(ok);
    // counts fall as t grows, so the largest qualifying t is the last set lane
    if (lane == 0) wsum[wave] = bl ? (uint32_t)(63 - __clzll(bl)) + 1u : 0u;
    __syncthreads();
    if (tid == 0) {
      int best = -1;
      for (int w = 0; w < (int)(blockDim.x >> 6); ++w)
        if (wsum[w]) best = 64 * w + (int)wsum[w] - 1;
      s_sel = best;
    }
    __syncthreads();
  }
  const int32_t Et = s_sel;
  // keys above the chosen exponent, and what is still needed inside it
  if (tid == 0) s_need = 0;
  __syncthreads();
  {
    int64_t above = 0;
    for (int e = tid; e < 320; e += blockDim.x) {
      const uint32_t h = hist[e];
      const int32_t top = (e - 32) + 256;
      const int32_t kk = top >= Et + 1 ? (top - Et - 1) / 2 + 1 : 0;
      above += (int64_t)h * (kk < mb ? kk : mb);
    }
    for (int o = 32; o > 0; o >>= 1) above += __shfl_xor(above, o, 64);
    if (lane == 0) atomicAdd((unsigned long long*)&s_need, (unsigned long long)above);
  }
  __syncthreads();
  int64_t need = B - s_need;  // 1 <= need <= keys with E == Et
  uint64_t prefix = 0;        // low bits chosen so far (above the current digit)
  for (int d = 0; d < kGDigits; ++d) {
    const int sh = gdigit_shift(d), nb = gdigit_bits(d);
    for (int i = tid; i < 2048; i += blockDim.x) hist[i] = 0u;
    __syncthreads();
    for (int64_t i = tid; i < n; i += blockDim.x) {
      const float v = st[i].y;
      if (!(v > 0.0f)) continue;
      int32_t ex;
      uint32_t man;
      var_exp_man(v, ex, man);
      const int32_t diff = ex + 256 - Et;  // = 2k for the key in the chosen exponent
      if (diff < 0 || (diff & 1) || diff / 2 >= mb) continue;
      const uint64_t low = global_key(ex, man, diff / 2, i) & ((1ull << kGKeyLow) - 1ull);
      if ((low >> (sh + nb)) != prefix) continue;
      atomicAdd(&hist[(low >> sh) & ((1u << nb) - 1u)], 1u);
    }
    __syncthreads();
    // suffix sums over the digit's bins (two per thread, high bins first)
    const int nbins = 1 << nb;
    const int b0 = nbins - 1 - 2 * tid;  // this thread's higher bin
    uint32_t c0 = 0, c1 = 0;
    if (2 * tid < nbins) {
      c0 = hist[b0];
      c1 = b0 - 1 >= 0 ? hist[b0 - 1] : 0u;
    }
    uint32_t x = c0 + c1;  // inclusive scan in descending bin order
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    uint32_t before = 0;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    const uint32_t incl = before + x;          // keys in bins >= b0 - 1
    const uint32_t excl = incl - c0 - c1;      // keys in bins > b0
    if (2 * tid < nbins) {
      if (excl < need && excl + c0 >= need) { s_sel = b0; s_need = need - excl; }
      else if (excl + c0 < need && incl >= need) { s_sel = b0 - 1; s_need = need - excl - c0; }
    }
    __syncthreads();
    prefix = (prefix << nb) | (uint64_t)s_sel;
    need = s_need;
    __syncthreads();
  }
  if (tid == 0) *thr_out = ((uint64_t)Et << kGKeyLow) | prefix;
}

hipError_t launch_alloc_from_stats(const Params& p, hipStream_t s) {
  if (p.alloc_scope == 1 && p.transform == KVTC_PCA) {
    hipLaunchKernelGGL(k_alloc_global, dim3(1, 1, seq_grid(p)), dim3(1024), 0, s, p);
    hipLaunchKernelGGL(k_enc_alloc<4>, dim3(p.n_sections, 1, seq_grid(p)), dim3(64), 0, s, p);
  } else {
    hipLaunchKernelGGL(k_enc_alloc<3>, dim3(p.n_sections, 1, seq_grid(p)), dim3(64), 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_unrope(const Params& p, hipStream_t s) {
  if (!(p.D == 128 && p.dtype == KVTC_BF16 && p.transform == KVTC_PCA && p.rope_keys && (p.tile_tokens % 64) == 0))
    return hipErrorInvalidValue;
  if (p.T_mid > 0) hipLaunchKernelGGL(k_unrope128, dim3((p.T_mid + 15) / 16, p.L, seq_grid(p)), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_enc_alloc(const Params& p, hipStream_t s) {
  if (p.alloc_scope == 1 && p.transform == KVTC_PCA) {
    hipLaunchKernelGGL(k_enc_alloc<1>, dim3(p.n_sections, 1, seq_grid(p)), dim3(64), 0, s, p);
    hipLaunchKernelGGL(k_alloc_global, dim3(1, 1, seq_grid(p)), dim3(1024), 0, s, p);
    hipLaunchKernelGGL(k_enc_alloc<2>, dim3(p.n_sections, 1, seq_grid(p)), dim3(64), 0, s, p);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_enc_alloc<0>, dim3(p.n_sections, 1, seq_grid(p)), dim3(64), 0, s, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// plan: basis rounded to the operand precision, in both layouts
// ---------------------------------------------------------------------------

__global__ void k_prep_basis(const float* src, void* bt, void* b, int64_t n_basis, int D, int dtype,
                             int32_t* bad) {
  const int64_t total = n_basis * D * D;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    int64_t m = idx / ((int64_t)D * D), rem = idx % ((int64_t)D * D);
    int j = (int)(rem / D), i = (int)(rem % D);  // src[m][j][i]: row j = channel, col i = component
    float v = src[idx];
    if (!isfinite(v)) atomicOr(bad, 1);
    int64_t tpos = m * D * D + (int64_t)i * D + j;
    if (dtype == KVTC_BF16) {
      uint16_t hv = f32_to_bf16(v);
      reinterpret_cast<uint16_t*>(b)[idx] = hv;
      reinterpret_cast<uint16_t*>(bt)[tpos] = hv;
    } else {
      reinterpret_cast<float*>(b)[idx] = v;
      reinterpret_cast<float*>(bt)[tpos] = v;
    }
  }
}

hipError_t launch_prep_basis(const float* src, void* basis_t, void* basis, int n_basis, int D,
                             int dtype, int32_t* bad, hipStream_t s) {
  int64_t total = (int64_t)n_basis * D * D;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(k_prep_basis, dim3((unsigned)blocks), dim3(256), 0, s, src, basis_t, basis,
                     (int64_t)n_basis, D, dtype, bad);
  return hipGetLastError();
}

}  // namespace kvtc
