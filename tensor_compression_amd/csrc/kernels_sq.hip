// Scalar quantisers on gauge coordinates ("Codec-Gauge: Learning
// Compression-Friendly Gauges for Transformer KV Caches", Compression
// Conditions): the backend sees Z = G X, with the plan's basis as the gauge
// (Problem Statement and Overview), and quantises every coefficient of a
// section with the same b bits against an affine (zero = min, step) range.
// The block-uniform quantiser takes one range per block of T_b tokens x a
// run of channels; the KIVI-style quantiser takes ranges per channel over
// T_b tokens for keys and per token over a run of g channels for values.
// Decoding dequantises, applies X^ = G^T Z^ and re-applies RoPE to keys.
//
// Layout of a call over T tokens (all tokens coded, no raw windows):
//  * sections u = (l 2 + s) H + h in order; a section of kind s holds
//    T D b_s / 8 code bytes and ceil(T / te) (D / ce) ranges;
//  * codes: token-major rows of D b bits, channel i at bits [i b, i b + b)
//    of the row, least significant bit first; a row is 4 b whole words;
//  * ranges: (zero, scale) fp32 pairs, index (t / te) (D / ce) + i / ce.
//
// Work decomposition (head_dim 128, bf16): a workgroup of four waves per
// (64-token span, section).  Ranges never straddle a span (te divides 64),
// so every span is independent.
//  encode: stage the rows in LDS (keys un-rotated and rounded to bf16) ->
//    v_mfma_f32_16x16x32_bf16 projection with the section's basis rows in
//    registers -> fp32 coefficient tile in LDS -> range minima and maxima
//    (per token and channel run, then over the te tokens) -> zero, step and
//    reciprocal per range -> quantise 32 channels of a token per lane ->
//    bit-pack in LDS -> coalesced row stores.  A value whose fp32 pre-rounding
//    value v lies within its error bound of a rounding boundary is recomputed
//    exactly (fp64 sum of the exact bf16 products) before rounding.
//  decode: stage the span's code rows and ranges in LDS -> dequantise
//    (fma(q, scale, zero), rounded to bf16) into token-major operand rows ->
//    MFMA with the channel-major basis rows in registers -> RoPE -> output
//    rows through LDS -> coalesced stores in the output dtype.
#include "kvtc_internal.h"

namespace kvtc {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kSpan = 64;   // tokens per span
constexpr int kXS = 136;    // bf16 row stride of staged rows (16-B aligned, 4-bank shift)
constexpr int kCS = 132;    // fp32 row stride of the coefficient / output tile

__device__ __forceinline__ void unpack8(uint4 a, float* o) {
  o[0] = __uint_as_float(a.x << 16); o[1] = __uint_as_float(a.x & 0xffff0000u);
  o[2] = __uint_as_float(a.y << 16); o[3] = __uint_as_float(a.y & 0xffff0000u);
  o[4] = __uint_as_float(a.z << 16); o[5] = __uint_as_float(a.z & 0xffff0000u);
  o[6] = __uint_as_float(a.w << 16); o[7] = __uint_as_float(a.w & 0xffff0000u);
}

__device__ __forceinline__ uint32_t pk2(float a, float b) {
  return (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
}

__device__ __forceinline__ bool finite(float x) { return fabsf(x) <= 3.402823466e38f; }

// Offset of section u's block among sections whose sizes depend only on
// their kind: x0 per key section, x1 per value section.
__device__ __forceinline__ int64_t sec_off(int u, int H, int64_t x0, int64_t x1) {
  const int h = u % H, s = (u / H) & 1, l = u / (2 * H);
  return (int64_t)l * H * (x0 + x1) + (s ? (int64_t)H * x0 : 0) + (int64_t)h * (s ? x1 : x0);
}

__device__ __forceinline__ int64_t basis_of(const SqParams& q, int l, int s, int h) {
  return q.basis_per_head ? ((int64_t)(l * 2 + s) * q.H + h) : (int64_t)(l * 2 + s);
}

// Range of a span: zero = min, step = (max - min) / (2^b - 1) in fp64 rounded
// once to fp32, reciprocal 1 / step in fp32; an empty or unusable step
// (0, subnormal reciprocal overflow) gives step 0 and reciprocal 0.
__device__ __forceinline__ void make_range(float mn, float mx, int b, float* zero, float* scale, float* rcp) {
  float sc = (float)__ddiv_rn(__dadd_rn((double)mx, -(double)mn), (double)((1u << b) - 1u));
  float r = sc > 0.0f ? __fdiv_rn(1.0f, sc) : 0.0f;
  if (!(sc > 0.0f) || !finite(r)) {
    sc = 0.0f;
    r = 0.0f;
  }
  *zero = mn;
  *scale = sc;
  *rcp = r;
}

}  // namespace

// Dynamic LDS of the encoder: the span's range table (zero, reciprocal).
__host__ __device__ inline int sq_span_ranges(int te, int ce) { return (kSpan / te) * (128 / ce); }

__global__ void k_sq_clear(uint32_t* status) {
  if (threadIdx.x == 0) *status = 0u;
}

// Quantise and pack the 32 channels [32 w, 32 w + 32) of token t = lane of
// the span (wave w): codes clamp(rint((c - zero) rcp)) into B whole words at
// word (t 4 + w) B.  A coarse test per value flags the lane when some
// pre-rounding value v may lie within its error bound of a rounding
// boundary (the bound taken at its largest, |v| <= 2^B); such lanes find
// their values one by one, and each is recomputed from the exact
// coefficient (one wave-wide fp64 dot product of the staged row and the
// basis row).
template <int B>
__device__ __forceinline__ void quant_pack(const SqParams& q, const float* C, const uint16_t* X, const uint16_t* bt,
                                           const float2* R, const float* nrm, uint32_t* out, int n, int lte, int lce,
                                           int lncg) {
  constexpr int D = 128;
  constexpr float QM = (float)((1u << B) - 1u);
  constexpr uint32_t MASK = (1u << B) - 1u;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, t = lane;
  const bool valid = t < n;
  const int rrow = (t >> lte) << lncg;
  const float ecm = valid ? q.mfma_err * nrm[t] : 0.0f;
  const float slack = 3.0f * 0x1p-23f * (QM + 1.0f);
  uint32_t w[B];
#pragma unroll
  for (int i = 0; i < B; ++i) w[i] = 0u;
  float worst = -1.0f;  // max over values of |v - rint(v)| - (1/2 - bound)
  if (valid) {
#pragma unroll
    for (int k4 = 0; k4 < 8; ++k4) {
      const float4 v4 = *reinterpret_cast<const float4*>(&C[t * kCS + 32 * wave + 4 * k4]);
      const float cv[4] = {v4.x, v4.y, v4.z, v4.w};
      float2 zr[4];
      if (lce >= 2) {
        zr[0] = zr[1] = zr[2] = zr[3] = R[rrow + ((32 * wave + 4 * k4) >> lce)];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) zr[e] = R[rrow + ((32 * wave + 4 * k4 + e) >> lce)];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c = 4 * k4 + e;
        const float v = __fmul_rn(__fsub_rn(cv[e], zr[e].x), zr[e].y);
        const float rv = __builtin_rintf(v);
        const uint32_t code = (uint32_t)__builtin_amdgcn_fmed3f(rv, 0.0f, QM);
        const float hth = 0.5f - __fmaf_rn(ecm, zr[e].y, slack);
        worst = fmaxf(worst, fabsf(__fsub_rn(v, rv)) - hth);
        const int bit = c * B;
        w[bit >> 5] |= code << (bit & 31);
        if ((bit & 31) + B > 32) w[(bit >> 5) + 1] |= code >> (32 - (bit & 31));
      }
    }
  }
  // the lanes that may hold a near-boundary value list them precisely
  uint32_t flags = 0u;
  if (worst >= 0.0f) {
    for (int c = 0; c < 32; ++c) {
      const float cvv = C[t * kCS + 32 * wave + c];
      const float2 zr = R[rrow + ((32 * wave + c) >> lce)];
      const float v = __fmul_rn(__fsub_rn(cvv, zr.x), zr.y);
      const float hth = 0.5f - __fmaf_rn(ecm, zr.y, slack);
      if (fabsf(__fsub_rn(v, __builtin_rintf(v))) >= hth) flags |= 1u << c;
    }
  }
  uint64_t pend = __ballot(flags != 0u);
  while (pend) {
    const int L = __ffsll((unsigned long long)pend) - 1;
    const uint32_t fl = __shfl(flags, L, 64);
    const int c = __ffs(fl) - 1;
    const int i = 32 * wave + c;
    const uint32_t xw = *reinterpret_cast<const uint32_t*>(&X[L * kXS + 2 * lane]);
    const uint32_t bw = *reinterpret_cast<const uint32_t*>(bt + (int64_t)i * D + 2 * lane);
    double part = __fma_rn((double)__uint_as_float(xw << 16), (double)__uint_as_float(bw << 16),
                           (double)__uint_as_float(xw & 0xffff0000u) * (double)__uint_as_float(bw & 0xffff0000u));
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) part += __shfl_xor(part, o, 64);
    if (lane == L) {
      const float2 zr = R[rrow + (i >> lce)];
      const float v = __fmul_rn(__fsub_rn((float)part, zr.x), zr.y);
      const uint32_t code = (uint32_t)__builtin_amdgcn_fmed3f(__builtin_rintf(v), 0.0f, QM);
      const int bit = c * B, wi = bit >> 5, sh = bit & 31;
#pragma unroll
      for (int k = 0; k < B; ++k) {
        if (k == wi) w[k] = (w[k] & ~(MASK << sh)) | (code << sh);
        if (sh + B > 32 && k == wi + 1) w[k] = (w[k] & ~(MASK >> (32 - sh))) | (code >> (32 - sh));
      }
      flags &= ~(1u << c);
    }
    pend = __ballot(flags != 0u);
  }
  if (valid) {  // the lane's B words of its token's row, in the widest aligned stores
    uint32_t* dst = out + (t * 4 + wave) * B;
    if constexpr (B % 4 == 0) {
#pragma unroll
      for (int k = 0; k < B; k += 4) *reinterpret_cast<uint4*>(dst + k) = make_uint4(w[k], w[k + 1], w[k + 2], w[k + 3]);
    } else if constexpr (B % 2 == 0) {
#pragma unroll
      for (int k = 0; k < B; k += 2) *reinterpret_cast<uint2*>(dst + k) = make_uint2(w[k], w[k + 1]);
    } else {
#pragma unroll
      for (int k = 0; k < B; ++k) dst[k] = w[k];
    }
  }
}

__global__ __launch_bounds__(256) void k_sq_enc128(const SqParams q) {
  constexpr int D = 128;
  const int u = blockIdx.y;
  const int H = q.H, h = u % H, s = (u / H) & 1, l = u / (2 * H);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, r = lane & 15;
  const int b = q.bits[s], te = q.te[s], ce = q.ce[s];
  // te and ce are powers of two (divisors of 64 and 128)
  const int lte = __ffs(te) - 1, lce = __ffs(ce) - 1;
  const int ncg = D >> lce;             // channel runs per token
  const int lncg = 7 - lce;
  const int nrs = (kSpan >> lte) << lncg;  // ranges of a full span

  __shared__ __attribute__((aligned(16))) uint16_t X[kSpan * kXS];
  __shared__ __attribute__((aligned(16))) float C[kSpan * kCS];
  __shared__ float nrm[kSpan];
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];
  float2* const R = reinterpret_cast<float2*>(dyn);  // (zero, rcp) per range

  const uint16_t* bt = q.basis_t + basis_of(q, l, s, h) * D * D;

  // ---- stage: thread (token tid / 4, quarter tid % 4) holds channel runs
  // [16 q, 16 q + 16) and [64 + 16 q, +16): both members of every RoPE pair
  const int st_t = tid >> 2, st_q = tid & 3;
  const bool rope = s == 0 && q.rope_keys;
  uint4 y[4];
  float4 cs[8];
  auto load_rows = [&](int ts, int ns) {
    const bool valid = st_t < ns;
    const int pos = ts + st_t;
    y[0] = y[1] = y[2] = y[3] = make_uint4(0, 0, 0, 0);
    if (valid) {
      const uint16_t* row = (s ? q.v : q.k) + (((int64_t)l * H + h) * q.T + pos) * D;
      y[0] = *reinterpret_cast<const uint4*>(row + 16 * st_q);
      y[1] = *reinterpret_cast<const uint4*>(row + 16 * st_q + 8);
      y[2] = *reinterpret_cast<const uint4*>(row + 64 + 16 * st_q);
      y[3] = *reinterpret_cast<const uint4*>(row + 64 + 16 * st_q + 8);
      if (rope) {
        if (q.rope_style == KVTC_ROPE_HALF) {  // pairs [16 q, 16 q + 16)
          const float4* cr = reinterpret_cast<const float4*>(q.rope + (int64_t)pos * 64 + 16 * st_q);
#pragma unroll
          for (int k = 0; k < 8; ++k) cs[k] = cr[k];
        } else {  // interleaved: pairs [8 q, 8 q + 8) and [32 + 8 q, +8)
          const float4* c0 = reinterpret_cast<const float4*>(q.rope + (int64_t)pos * 64 + 8 * st_q);
          const float4* c1 = reinterpret_cast<const float4*>(q.rope + (int64_t)pos * 64 + 32 + 8 * st_q);
#pragma unroll
          for (int k = 0; k < 4; ++k) { cs[k] = c0[k]; cs[4 + k] = c1[k]; }
        }
      }
    }
  };
  const int t0 = blockIdx.x * kSpan;
  const int n = min(kSpan, q.T - t0);
  load_rows(t0, n);
  // B operands: component (2 wave + m) 16 + r, channels 32 kb + 8 g .. +7,
  // requested after the rows so that waiting for the rows does not wait for them
  uint4 bq[2][4];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      bq[m][kb] = *reinterpret_cast<const uint4*>(bt + (int64_t)((2 * wave + m) * 16 + r) * D + kb * 32 + 8 * g);
  {
    const bool valid = st_t < n;
    float lo[16], hi[16];
    unpack8(y[0], lo); unpack8(y[1], lo + 8);
    unpack8(y[2], hi); unpack8(y[3], hi + 8);
    if (rope && valid) {
      // x_a = y_a c + y_b s, x_b = y_b c - y_a s (one fma each)
      if (q.rope_style == KVTC_ROPE_HALF) {
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
    uint4 o[4];
    o[0] = make_uint4(pk2(lo[0], lo[1]), pk2(lo[2], lo[3]), pk2(lo[4], lo[5]), pk2(lo[6], lo[7]));
    o[1] = make_uint4(pk2(lo[8], lo[9]), pk2(lo[10], lo[11]), pk2(lo[12], lo[13]), pk2(lo[14], lo[15]));
    o[2] = make_uint4(pk2(hi[0], hi[1]), pk2(hi[2], hi[3]), pk2(hi[4], hi[5]), pk2(hi[6], hi[7]));
    o[3] = make_uint4(pk2(hi[8], hi[9]), pk2(hi[10], hi[11]), pk2(hi[12], hi[13]), pk2(hi[14], hi[15]));
    uint16_t* xr = &X[st_t * kXS];
    *reinterpret_cast<uint4*>(xr + 16 * st_q) = o[0];
    *reinterpret_cast<uint4*>(xr + 16 * st_q + 8) = o[1];
    *reinterpret_cast<uint4*>(xr + 64 + 16 * st_q) = o[2];
    *reinterpret_cast<uint4*>(xr + 64 + 16 * st_q + 8) = o[3];
    // squared norm of the staged (rounded) row for the coefficient error bound
    float n2 = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float f[8];
      unpack8(o[k], f);
#pragma unroll
      for (int z = 0; z < 8; ++z) n2 = __fmaf_rn(f[z], f[z], n2);
    }
    n2 += __shfl_xor(n2, 1, 64);
    n2 += __shfl_xor(n2, 2, 64);
    if (st_q == 0) nrm[st_t] = __fsqrt_rn(n2);
  }
  __syncthreads();

  // ---- projection: lane (g, r) of wave w holds component (2 w + m) 16 + r
  // of tokens 16 kk + 4 g .. +3
  {
    f32x4_t acc[4][2];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      acc[kk][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      acc[kk][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const uint4 a = *reinterpret_cast<const uint4*>(&X[(kk * 16 + r) * kXS + kb * 32 + 8 * g]);
        const bf16x8_t av = __builtin_bit_cast(bf16x8_t, a);
#pragma unroll
        for (int m = 0; m < 2; ++m)
          acc[kk][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8_t, bq[m][kb]), acc[kk][m], 0, 0, 0);
      }
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) C[(kk * 16 + 4 * g + e) * kCS + (2 * wave + m) * 16 + r] = acc[kk][m][e];
  }
  __syncthreads();

  // ---- ranges
  bool bad = false;
  {
    const int64_t rbase = sec_off(u, H, q.n_ranges[0], q.n_ranges[1]) + (int64_t)(t0 >> lte) * ncg;
    if (ce > 1) {
      // lane = token, wave = channel runs wave, wave + 4, ...: the run's
      // extremes, then across the te tokens of a range with lane shuffles
      for (int cg = wave; cg < ncg; cg += 4) {
        const int t = lane;
        const float* c = &C[t * kCS + cg * ce];
        float mn = INFINITY, mx = -INFINITY;
        if (ce >= 4) {
          for (int j = 0; j < ce; j += 4) {
            const float4 v = *reinterpret_cast<const float4*>(c + j);
            mn = fminf(fminf(mn, v.x), fminf(v.y, fminf(v.z, v.w)));
            mx = fmaxf(fmaxf(mx, v.x), fmaxf(v.y, fmaxf(v.z, v.w)));
            bad |= !(finite(v.x) && finite(v.y) && finite(v.z) && finite(v.w));
          }
        } else {
          for (int j = 0; j < ce; ++j) {
            mn = fminf(mn, c[j]);
            mx = fmaxf(mx, c[j]);
            bad |= !finite(c[j]);
          }
        }
        if (t >= n) {  // tokens past the span take no part
          mn = INFINITY;
          mx = -INFINITY;
          bad = false;
        }
        for (int o = 1; o < te; o <<= 1) {
          mn = fminf(mn, __shfl_xor(mn, o, 64));
          mx = fmaxf(mx, __shfl_xor(mx, o, 64));
        }
        if ((t & (te - 1)) == 0) {
          const int it = ((t >> lte) << lncg) + cg;
          float zero = 0.f, scale = 0.f, rcp = 0.f;
          if (t < n) {
            make_range(mn, mx, b, &zero, &scale, &rcp);
            *reinterpret_cast<float2*>(q.ranges + 2 * (rbase + it)) = make_float2(zero, scale);
          }
          R[it] = make_float2(zero, rcp);
        }
      }
    } else {
      // one channel a range: a column scan of te tokens, four loads in flight
      for (int it = tid; it < nrs; it += 256) {
        const int cg = it & (ncg - 1), tj = it >> lncg;
        const int ta = tj * te, tb = min(ta + te, n);
        float mn = INFINITY, mx = -INFINITY;
        int t = ta;
        for (; t + 4 <= tb; t += 4) {
          const float c0 = C[t * kCS + cg], c1 = C[(t + 1) * kCS + cg];
          const float c2 = C[(t + 2) * kCS + cg], c3 = C[(t + 3) * kCS + cg];
          mn = fminf(fminf(mn, c0), fminf(c1, fminf(c2, c3)));
          mx = fmaxf(fmaxf(mx, c0), fmaxf(c1, fmaxf(c2, c3)));
          bad |= !(finite(c0) && finite(c1) && finite(c2) && finite(c3));
        }
        for (; t < tb; ++t) {
          const float c = C[t * kCS + cg];
          mn = fminf(mn, c);
          mx = fmaxf(mx, c);
          bad |= !finite(c);
        }
        float zero = 0.f, scale = 0.f, rcp = 0.f;
        if (ta < n) {
          make_range(mn, mx, b, &zero, &scale, &rcp);
          *reinterpret_cast<float2*>(q.ranges + 2 * (rbase + it)) = make_float2(zero, scale);
        }
        R[it] = make_float2(zero, rcp);
      }
    }
  }
  if (bad && q.status) atomicOr(q.status, 1u << KVTC_ERR_NONFINITE);
  __syncthreads();  // the range table is complete

  // ---- quantise and pack: lane = token, wave = channel quarter [32 w, 32 w + 32)
  // the span's rows go straight to the output (16-byte aligned: a section's
  // rows are 16 b bytes each)
  uint32_t* const out = reinterpret_cast<uint32_t*>(q.codes + sec_off(u, H, q.code_bytes[0], q.code_bytes[1]) +
                                                    (int64_t)t0 * 16 * b);
  switch (b) {
    case 1: quant_pack<1>(q, C, X, bt, R, nrm, out, n, lte, lce, lncg); break;
    case 2: quant_pack<2>(q, C, X, bt, R, nrm, out, n, lte, lce, lncg); break;
    case 3: quant_pack<3>(q, C, X, bt, R, nrm, out, n, lte, lce, lncg); break;
    case 4: quant_pack<4>(q, C, X, bt, R, nrm, out, n, lte, lce, lncg); break;
    case 5: quant_pack<5>(q, C, X, bt, R, nrm, out, n, lte, lce, lncg); break;
    case 6: quant_pack<6>(q, C, X, bt, R, nrm, out, n, lte, lce, lncg); break;
    case 7: quant_pack<7>(q, C, X, bt, R, nrm, out, n, lte, lce, lncg); break;
    default: quant_pack<8>(q, C, X, bt, R, nrm, out, n, lte, lce, lncg); break;
  }
}

// Dynamic LDS of the decoder: the span's code rows plus four zero words,
// then its range table (zero, scale).
__host__ __device__ inline int sq_dec_code_bytes(int b) { return ((kSpan * 4 * b + 4) * 4 + 15) & ~15; }

__global__ __launch_bounds__(256) void k_sq_dec128(const SqParams q) {
  constexpr int D = 128;
  const int u = blockIdx.y, t0 = blockIdx.x * kSpan;
  const int n = min(kSpan, q.T - t0);
  const int H = q.H, h = u % H, s = (u / H) & 1, l = u / (2 * H);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, r = lane & 15;
  const int b = q.bits[s], te = q.te[s], ce = q.ce[s];
  const int lte = __ffs(te) - 1, lce = __ffs(ce) - 1;
  const int ncg = D >> lce;
  const int nrv = ((n + te - 1) >> lte) * ncg;

  // operand rows (bf16), later the output rows (fp32)
  __shared__ __attribute__((aligned(16))) float OS[kSpan * kCS];
  uint16_t* const CH = reinterpret_cast<uint16_t*>(OS);
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];
  uint32_t* const PK = reinterpret_cast<uint32_t*>(dyn);
  float2* const R = reinterpret_cast<float2*>(dyn + sq_dec_code_bytes(b));

  const uint16_t* bc = q.basis + basis_of(q, l, s, h) * D * D;

  {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(q.codes + sec_off(u, H, q.code_bytes[0], q.code_bytes[1]) +
                                                            (int64_t)t0 * 16 * b);
    const int nw = n * 4 * b;
    for (int i = tid; i < nw + 4; i += 256) PK[i] = i < nw ? src[i] : 0u;
    const float2* rs = reinterpret_cast<const float2*>(q.ranges) + sec_off(u, H, q.n_ranges[0], q.n_ranges[1]) +
                       (int64_t)(t0 >> lte) * ncg;
    for (int i = tid; i < nrv; i += 256) R[i] = rs[i];
  }
  // A operands: channel 16 (wave + 4 nbi) + r, components 32 kb + 8 g .. +7,
  // requested after the codes so that they arrive during the dequantisation
  uint4 A[2][4];
#pragma unroll
  for (int nbi = 0; nbi < 2; ++nbi)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      A[nbi][kb] = *reinterpret_cast<const uint4*>(bc + (int64_t)(16 * (wave + 4 * nbi) + r) * D + kb * 32 + 8 * g);
  __syncthreads();

  // ---- dequantise: item = (token, component octet), lanes on consecutive tokens
  const uint32_t mask = (1u << b) - 1u;
  for (int it = tid; it < kSpan * 16; it += 256) {
    const int t = it & (kSpan - 1), o = it >> 6;
    uint4 w4 = make_uint4(0, 0, 0, 0);
    if (t < n) {
      const uint32_t P = (uint32_t)(t * 128 + 8 * o) * (uint32_t)b;
      const uint32_t W = P >> 5, sh = P & 31u;
      uint64_t v64 = ((uint64_t)PK[W + 1] << 32 | PK[W]) >> sh;
      if (sh) v64 |= (uint64_t)PK[W + 2] << (64 - sh);
      const float2* rr = R + (t >> lte) * ncg;
      float x[8];
#pragma unroll
      for (int z = 0; z < 8; ++z) {
        const uint32_t code = (uint32_t)(v64 >> (z * b)) & mask;
        const float2 zs = rr[(8 * o + z) >> lce];
        x[z] = __fmaf_rn((float)code, zs.y, zs.x);
      }
      w4 = make_uint4(pk2(x[0], x[1]), pk2(x[2], x[3]), pk2(x[4], x[5]), pk2(x[6], x[7]));
    }
    *reinterpret_cast<uint4*>(&CH[t * kXS + 8 * o]) = w4;
  }
  __syncthreads();

  // ---- inverse projection: lane (g, r) holds channels 16 (wave + 4 nbi) + 4 g .. +3
  // of token 16 kk + r
  f32x4_t acc[4][2];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    acc[kk][0] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    acc[kk][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const uint4 bv = *reinterpret_cast<const uint4*>(&CH[(kk * 16 + r) * kXS + kb * 32 + 8 * g]);
      const bf16x8_t bop = __builtin_bit_cast(bf16x8_t, bv);
#pragma unroll
      for (int nbi = 0; nbi < 2; ++nbi)
        acc[kk][nbi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, A[nbi][kb]), bop, acc[kk][nbi], 0, 0, 0);
    }
  }
  if (s == 0 && q.rope_keys) {
    // y_a = x_a c - x_b s, y_b = x_a s + x_b c (one fma each)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int pos = min(t0 + kk * 16 + r, q.T - 1);
      const float4* row = reinterpret_cast<const float4*>(q.rope + (int64_t)pos * 64);
      if (q.rope_style == KVTC_ROPE_HALF) {
        // pair j = 16 wave + 4 g + e: x_a = acc[kk][0][e], x_b = acc[kk][1][e]
        const float4 c01 = row[(16 * wave + 4 * g) / 2], c23 = row[(16 * wave + 4 * g) / 2 + 1];
        const float cc[4] = {c01.x, c01.z, c23.x, c23.z}, ss[4] = {c01.y, c01.w, c23.y, c23.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float xa = acc[kk][0][e], xb = acc[kk][1][e];
          acc[kk][0][e] = __fmaf_rn(xa, cc[e], -__fmul_rn(xb, ss[e]));
          acc[kk][1][e] = __fmaf_rn(xa, ss[e], __fmul_rn(xb, cc[e]));
        }
      } else {
        // pairs (4 g + 2 e2, +1) of channel block wave + 4 nbi: index 8 nb + 2 g + e2
#pragma unroll
        for (int nbi = 0; nbi < 2; ++nbi) {
          const float4 c4 = row[(8 * (wave + 4 * nbi) + 2 * g) / 2];
          const float cc[2] = {c4.x, c4.z}, ss[2] = {c4.y, c4.w};
#pragma unroll
          for (int e2 = 0; e2 < 2; ++e2) {
            const float xa = acc[kk][nbi][2 * e2], xb = acc[kk][nbi][2 * e2 + 1];
            acc[kk][nbi][2 * e2] = __fmaf_rn(xa, cc[e2], -__fmul_rn(xb, ss[e2]));
            acc[kk][nbi][2 * e2 + 1] = __fmaf_rn(xa, ss[e2], __fmul_rn(xb, cc[e2]));
          }
        }
      }
    }
  }
  __syncthreads();  // every wave has read its operand rows
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
#pragma unroll
    for (int nbi = 0; nbi < 2; ++nbi)
      *reinterpret_cast<float4*>(&OS[(kk * 16 + r) * kCS + 16 * (wave + 4 * nbi) + 4 * g]) =
          make_float4(acc[kk][nbi][0], acc[kk][nbi][1], acc[kk][nbi][2], acc[kk][nbi][3]);
  __syncthreads();

  // ---- rows out, 16 bytes per lane
  uint8_t* out = reinterpret_cast<uint8_t*>(s ? q.v_out : q.k_out);
  if (q.out_dtype == KVTC_FP32) {
    float* o = reinterpret_cast<float*>(out) + (((int64_t)l * H + h) * q.T + t0) * D;
    for (int it = tid; it < n * 32; it += 256) {
      const int t = it >> 5, un = it & 31;
      store_out16(o + (int64_t)t * D + 4 * un, *reinterpret_cast<const float4*>(&OS[t * kCS + 4 * un]));
    }
  } else {
    uint16_t* o = reinterpret_cast<uint16_t*>(out) + (((int64_t)l * H + h) * q.T + t0) * D;
    for (int it = tid; it < n * 16; it += 256) {
      const int t = it >> 4, un = it & 15;
      const float4 a = *reinterpret_cast<const float4*>(&OS[t * kCS + 8 * un]);
      const float4 c = *reinterpret_cast<const float4*>(&OS[t * kCS + 8 * un + 4]);
      store_out16(o + (int64_t)t * D + 8 * un, make_uint4(pk2(a.x, a.y), pk2(a.z, a.w), pk2(c.x, c.y), pk2(c.z, c.w)));
    }
  }
}

static int max2(int a, int b) { return a > b ? a : b; }

hipError_t launch_sq_encode(const SqParams& q, hipStream_t s) {
  if (q.status) {
    k_sq_clear<<<1, 64, 0, s>>>(q.status);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (q.T == 0) return hipSuccess;
  int lds = 0;
  for (int k = 0; k < 2; ++k)
    lds = max2(lds, 8 * sq_span_ranges(q.te[k], q.ce[k]));
  (void)hipFuncSetAttribute((const void*)k_sq_enc128, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  const dim3 grid((unsigned)((q.T + kSpan - 1) / kSpan), (unsigned)(q.L * 2 * q.H));
  k_sq_enc128<<<grid, 256, lds, s>>>(q);
  return hipGetLastError();
}

hipError_t launch_sq_decode(const SqParams& q, hipStream_t s) {
  if (q.T == 0) return hipSuccess;
  int lds = 0;
  for (int k = 0; k < 2; ++k)
    lds = max2(lds, sq_dec_code_bytes(q.bits[k]) + 8 * sq_span_ranges(q.te[k], q.ce[k]));
  (void)hipFuncSetAttribute((const void*)k_sq_dec128, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  const dim3 grid((unsigned)((q.T + kSpan - 1) / kSpan), (unsigned)(q.L * 2 * q.H));
  k_sq_dec128<<<grid, 256, lds, s>>>(q);
  return hipGetLastError();
}

}  // namespace kvtc
