// TTAS-X2 value path ("TTAS-X2: Extreme KV Cache Compression for Large
// Language Models", 2.2 V Compression): per-vector RMS normalisation, the
// Hadamard transform, two-level product quantisation (K1 and K2 centroids
// per subspace of 8 channels) and a fixed budget of outliers per head and
// block of tokens, stored exactly.
//
// Definitions (shared with the oracle, stated here on their own):
//  * r = sqrt(sum x^2 / D) (fp64, rounded once), y = WHT(x / r): the
//    orthonormal Sylvester transform, fp64 butterflies, one rounding;
//  * centroids are held in bf16; the nearest centroid minimises
//    sum_j (y_j - c_j)^2 in fp64 summed in channel order, lowest index on
//    ties; level 2 codes the fp32 residual e = y - c1;
//  * y^ = c1 + c2 (fp32); per (layer, head) and block of `bt` tokens the B
//    coefficients with the largest |y - y^| (then the lowest index t D + j)
//    are kept as (index, y), index-ascending;
//  * decode: y^ with the outliers put back, x^ = WHT(y^) r.
//
// Kernels (head_dim 128, bf16 cache, one workgroup of four waves per
// (64-token span, value section) unless noted):
//  k_pq_prep   per (layer, subspace): bf16 codebooks, centroid squared
//              norms, largest norm per level.
//  k_pq_enc    stage + RMS + WHT (fp64 butterflies, 16 lanes a token) ->
//              level 1: v_mfma_f32_32x32x16_bf16 scores ||c||^2 - 2 y.c for 32
//              centroids x 32 tokens at a time (a wave takes one subspace
//              and both 32-token groups of the span), y split into bf16 hi + lo
//              halves of K, running best / second-best per token with the index
//              packed into the score's low bits; a token whose best two
//              scores lie within the score error bound is decided again by
//              one wave-wide exact fp64 scan -> residual -> level 2 alike ->
//              code rows -> y - y^ -> the span's B largest errors by a
//              radix select over distinct 44-bit keys -> candidates.
//  k_pq_merge  per (section, block): the B largest of the block's span
//              candidates (radix select over 63-bit keys), index-ascending.
//  k_pq_dec    gather y^, put the block's outliers back, WHT, times r, store.
#include "kvtc_internal.h"

namespace kvtc {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int D = 128;
constexpr int SD = 8;        // channels per subvector
constexpr int NS = D / SD;   // subspaces
constexpr int kSpan = 64;
constexpr int kYS = 132;     // fp32 row stride of the coefficient tile
constexpr int kMaxRow = 9;   // code row words: 16 (9 + 9) bits

__device__ __forceinline__ bool finite_f(float x) { return fabsf(x) <= 3.402823466e38f; }

__device__ __forceinline__ void unpack8(uint4 a, float* o) {
  o[0] = __uint_as_float(a.x << 16); o[1] = __uint_as_float(a.x & 0xffff0000u);
  o[2] = __uint_as_float(a.y << 16); o[3] = __uint_as_float(a.y & 0xffff0000u);
  o[4] = __uint_as_float(a.z << 16); o[5] = __uint_as_float(a.z & 0xffff0000u);
  o[6] = __uint_as_float(a.w << 16); o[7] = __uint_as_float(a.w & 0xffff0000u);
}

// Row of the 32 x 32 MFMA result in accumulator i of a lane in half hf (the
// column is lane % 32).
__device__ __forceinline__ int acc_row(int i, int hf) { return 8 * (i >> 2) + 4 * hf + (i & 3); }

// The orthonormal WHT butterflies of a 16-lane group (lane q holds channels
// 8 q .. 8 q + 7), in fp64, unscaled.
// y = WHT(x / r) of 16 tokens at a time: lane q = lane % 16 of a 16-lane
// group holds channels 8 q .. 8 q + 7.  Returns r.  Each x / r (an fp32
// quotient) and each y / sqrt(D) (an fp64 quotient, then fp32) is first
// taken from one fp64 product with the reciprocal, which is within 2 fp64
// units of the quotient; where that cannot decide the fp32 rounding the
// division is done outright, so every result is the correctly rounded one.
__device__ __forceinline__ float rms_wht(const float (&x)[8], int q, float (&c)[8]) {
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
  div_f32(x, rt, xn);
#pragma unroll
  for (int e = 0; e < 8; ++e) y[e] = rt == 0.0f ? 0.0 : (double)xn[e];
  wht_fp64(y, q);
  const double rs = __dsqrt_rn((double)D);
  quot_f32(y, rs, __ddiv_rn(1.0, rs), c);
  return rt;
}

// Minimum and median of packed keys.  The keys are built with integer
// operations, so the compiler would quiet each one before a float min; a
// key is a NaN only when its score is, and then it is already quiet.
__device__ __forceinline__ float key_min(float a, float b) {
  float d;
  asm("v_min_f32 %0, %1, %2" : "=v"(d) : "v"(a), "v"(b));
  return d;
}
__device__ __forceinline__ float key_med3(float a, float b, float c) {
  float d;
  asm("v_med3_f32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
  return d;
}

// Best and second-best packed keys (score with the candidate index in its
// low 9 bits) over k centroids for tokens g 32 + lane % 32 (g = 0, 1) in
// subspace s; both lane halves end with the same pairs, and with the norm
// of each token's subvector.  The subvector is y (c1 == null) or the level-1
// residual y - c1 (c1: the level-1 codebook of the subspace, idx1 its
// chosen rows), formed in registers and split into bf16 high and low parts.
// One 32 x 32 x 16 MFMA per block of 32 centroids and token group gives
// ||c||^2 - 2 y.c outright: K = the subvector's 8 channels twice, -2 y's
// high part from the lower lane half and its low part from the upper half
// against the centroid's 8 values in both, and ||c||^2 as the accumulator's
// input.  The next block's operands are loaded during this block's scores,
// which run in four independent min chains per group.
__device__ __forceinline__ void search64(const float* Y, int s, const uint16_t* c1, const uint16_t* idx1,
                                         const uint16_t* cbh, const float* cn2, int k, float (&best)[2],
                                         float (&second)[2], float (&norm)[2]) {
  const int lane = threadIdx.x & 63, n32 = lane & 31, hf = lane >> 5;
  bf16x8_t bop[2];
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int tok = g * 32 + n32;
    const float4 a = *reinterpret_cast<const float4*>(&Y[tok * kYS + s * SD]);
    const float4 b = *reinterpret_cast<const float4*>(&Y[tok * kYS + s * SD + 4]);
    float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    if (c1) {
      float cv[8];
      unpack8(*reinterpret_cast<const uint4*>(c1 + (uint32_t)idx1[tok * NS + s] * SD), cv);
#pragma unroll
      for (int j = 0; j < SD; ++j) v[j] = __fsub_rn(v[j], cv[j]);
    }
    uint32_t w[8];
    float n2 = 0.f;
#pragma unroll
    for (int j = 0; j < SD; ++j) {
      const float m2 = -2.0f * v[j];  // exact
      const uint32_t h = (uint32_t)f32_to_bf16(m2);
      w[j] = hf ? (uint32_t)f32_to_bf16(__fsub_rn(m2, __uint_as_float(h << 16))) : h;
      n2 = __fmaf_rn(v[j], v[j], n2);
    }
    norm[g] = __fsqrt_rn(n2);
    bop[g] = __builtin_bit_cast(bf16x8_t, make_uint4(w[0] | (w[1] << 16), w[2] | (w[3] << 16), w[4] | (w[5] << 16),
                                                     w[6] | (w[7] << 16)));
  }
  float b1[2][4], b2[2][4];
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int c = 0; c < 4; ++c) b1[g][c] = b2[g][c] = INFINITY;
  const int nb = k >> 5;
  const uint4 an = *reinterpret_cast<const uint4*>(cbh + n32 * SD);
  // accumulator input: output row i of a lane is centroid 8 (i / 4) + 4 (lane / 32) + i % 4
  auto load_cn = [&](int blk) {
    f32x16_t c;
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const float4 v4 = *reinterpret_cast<const float4*>(cn2 + blk * 32 + 8 * r4 + 4 * hf);
      c[4 * r4] = v4.x;
      c[4 * r4 + 1] = v4.y;
      c[4 * r4 + 2] = v4.z;
      c[4 * r4 + 3] = v4.w;
    }
    return c;
  };
  // the score bits kept above the index, from a scalar register so that one
  // and-or per key packs it
  uint32_t kmask;
  asm volatile("s_mov_b32 %0, 0xfffffe00" : "=s"(kmask));
  // the next block's operands are loaded once both products have read this block's
  uint4 a = an;
  f32x16_t cn = load_cn(0);
  for (int blk = 0; blk < nb; ++blk) {
    f32x16_t acc[2];
    acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), bop[0], cn, 0, 0, 0);
    acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), bop[1], cn, 0, 0, 0);
    if (blk + 1 < nb) {
      a = *reinterpret_cast<const uint4*>(cbh + ((blk + 1) * 32 + n32) * SD);
      cn = load_cn(blk + 1);
    }
    const uint32_t base = (uint32_t)(blk * 32 + 4 * hf);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      uint32_t idx = base | (uint32_t)(8 * (i >> 2) + (i & 3));  // disjoint bits
      asm("" : "+v"(idx));  // one index per row, shared by both groups' and-or
      const int c = i & 3;
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const float key = __uint_as_float((__float_as_uint(acc[g][i]) & kmask) | idx);
        b2[g][c] = key_med3(b1[g][c], b2[g][c], key);
        b1[g][c] = key_min(b1[g][c], key);
      }
    }
  }
  // the four chains, then the other lane half
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    float x1 = b1[g][0], x2 = b2[g][0];
#pragma unroll
    for (int c = 1; c < 4; ++c) {
      x2 = fminf(fmaxf(x1, b1[g][c]), fminf(x2, b2[g][c]));
      x1 = fminf(x1, b1[g][c]);
    }
    const float o1 = __shfl_xor(x1, 32, 64), o2 = __shfl_xor(x2, 32, 64);
    second[g] = fminf(fmaxf(x1, o1), fminf(x2, o2));
    best[g] = fminf(x1, o1);
  }
}

// The exact nearest of k bf16 centroids to the wave-uniform subvector ys:
// fp64 squared distances summed in channel order, lowest index on ties.
__device__ __forceinline__ int exact_nearest(const float (&ys)[SD], const uint16_t* cbh, int k) {
  const int lane = threadIdx.x & 63;
  double bd = INFINITY;
  int bi = 0x7fffffff;
  for (int c = lane; c < k; c += 64) {
    float cv[8];
    unpack8(*reinterpret_cast<const uint4*>(cbh + c * SD), cv);
    double acc = 0.0;
#pragma unroll
    for (int j = 0; j < SD; ++j) {
      const double e = __dsub_rn((double)ys[j], (double)cv[j]);
      acc = __dadd_rn(acc, __dmul_rn(e, e));
    }
    if (acc < bd) {
      bd = acc;
      bi = c;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const double od = __shfl_xor(bd, o, 64);
    const int oi = __shfl_xor(bi, o, 64);
    if (od < bd || (od == bd && oi < bi)) {
      bd = od;
      bi = oi;
    }
  }
  // no candidate compares below +inf only for a non-finite subvector (the
  // call reports it): any valid index keeps the codebook reads in range
  return bi < k ? bi : 0;
}

// One radix pass of a block-wide selection (256 threads): among the keys
// that match `prefix` on `pmask`, the digit d of bits [sh, sh + w) holding
// the need-th largest, and how many of the keys with that digit are still
// needed.  each(f) calls f(key) on every key the thread holds.  HIST holds
// 2048 words of LDS, SM 8.
template <class EachFn>
__device__ void radix_pass(EachFn each, int sh, int w, uint64_t prefix, uint64_t pmask, uint32_t need,
                           uint32_t* HIST, uint32_t* SM, uint32_t& digit, uint32_t& need_out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t dmask = (1u << w) - 1u;
  for (int i = tid; i < 2048; i += 256) HIST[i] = 0u;
  __syncthreads();
  each([&](uint64_t kk) {
    if ((kk & pmask) == prefix) atomicAdd(&HIST[(uint32_t)(kk >> sh) & dmask], 1u);
  });
  __syncthreads();
  uint32_t c[8], loc = 0;
#pragma unroll
  for (int z = 0; z < 8; ++z) {
    c[z] = HIST[8 * tid + z];
    loc += c[z];
  }
  // counts in the bins above this thread's: a suffix sum over the threads
  uint32_t x = loc;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_down(x, o, 64);
    if (lane + o < 64) x += y;
  }
  if (lane == 0) SM[wave] = x;
  __syncthreads();
  uint32_t above = x - loc;
  for (int w2 = wave + 1; w2 < 4; ++w2) above += SM[w2];
  __syncthreads();
  if (above < need && above + loc >= need) {
    uint32_t run = above;
    for (int z = 7; z >= 0; --z) {
      if (run + c[z] >= need) {
        SM[4] = (uint32_t)(8 * tid + z);
        SM[5] = need - run;
        break;
      }
      run += c[z];
    }
  }
  __syncthreads();
  digit = SM[4];
  need_out = SM[5];
  __syncthreads();
}

// The B-th largest of the distinct keys each(f) visits that lie below bit
// `top` and match `prefix` on `pmask`, 11 bits per pass from the top.
template <class EachFn>
__device__ uint64_t radix_kth(EachFn each, int top, uint32_t B, uint32_t* HIST, uint32_t* SM,
                              uint64_t prefix = 0, uint64_t pmask = 0) {
  uint32_t need = B;
  for (; top > 0; top -= 11) {
    const int w = top < 11 ? top : 11, sh = top - w;
    uint32_t d;
    radix_pass(each, sh, w, prefix, pmask, need, HIST, SM, d, need);
    prefix |= (uint64_t)d << sh;
    pmask |= (uint64_t)((1u << w) - 1u) << sh;
  }
  return prefix;
}

}  // namespace

__global__ __launch_bounds__(256) void k_pq_prep(const PqParams q) {
  const int ls = blockIdx.x;  // layer * 16 + subspace
  const int tid = threadIdx.x;
  __shared__ uint32_t smax[2];
  if (tid < 2) smax[tid] = 0u;
  if (ls == 0 && tid == 0 && q.status) *q.status = 0u;
  __syncthreads();
  const int kk = q.k1 + q.k2;
  for (int c = tid; c < kk; c += 256) {
    const int lv = c < q.k1 ? 0 : 1, i = lv ? c - q.k1 : c, k = lv ? q.k2 : q.k1;
    const float* src = (lv ? q.cb2 : q.cb1) + ((int64_t)ls * k + i) * SD;
    const float4 f0 = reinterpret_cast<const float4*>(src)[0], f1 = reinterpret_cast<const float4*>(src)[1];
    const float f[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
    uint32_t h[8];
    double n2 = 0.0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      h[e] = (uint32_t)f32_to_bf16(f[e]);
      const double cv = (double)__uint_as_float(h[e] << 16);
      n2 = __fma_rn(cv, cv, n2);
    }
    uint16_t* dst = (lv ? q.cb2h : q.cb1h) + ((int64_t)ls * k + i) * SD;
    *reinterpret_cast<uint4*>(dst) = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                                                h[6] | (h[7] << 16));
    q.cn2[(int64_t)ls * kk + c] = (float)n2;
    atomicMax(&smax[lv], __float_as_uint(__fmul_rn((float)__dsqrt_rn(n2), 1.0f + 0x1p-20f)));
  }
  __syncthreads();
  if (tid < 2) q.cmax[ls * 2 + tid] = __uint_as_float(smax[tid]);
}

__global__ __launch_bounds__(256, 3) void k_pq_enc(const PqParams q) {
  const int sec = blockIdx.y, span = blockIdx.x;
  const int l = sec / q.H;
  const int t0 = span * kSpan, n = min(kSpan, q.T - t0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hf = lane >> 5, n32 = lane & 31;

  // 50 KB of LDS (three workgroups a CU): the span's coefficients, the chosen
  // indices, the radix histogram (first the code rows) and the short list
  __shared__ __attribute__((aligned(16))) float Y[kSpan * kYS];
  __shared__ uint16_t I1[kSpan * NS], I2[kSpan * NS];
  __shared__ __attribute__((aligned(16))) uint32_t HIST[2048];
  __shared__ __attribute__((aligned(16))) uint64_t LIST[512];
  __shared__ uint32_t SM[8];
  uint32_t* const ROW = HIST;  // the code rows, before the selection

  // ---- stage, RMS, WHT: 16 lanes a token, 16 tokens a pass
  {
    const int q16 = lane & 15, grp = tid >> 4;
    bool bad = false;
    uint4 raw[4];
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {  // every row of the span in flight at once
      const int tok = pass * 16 + grp;
      raw[pass] = tok < n ? *reinterpret_cast<const uint4*>(q.v + ((int64_t)sec * q.T + t0 + tok) * D + 8 * q16)
                          : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
      const int tok = pass * 16 + grp;
      const bool valid = tok < n;
      float x[8];
      unpack8(raw[pass], x);
#pragma unroll
      for (int e = 0; e < 8; ++e) bad |= !finite_f(x[e]);
      float c[8];
      const float rt = rms_wht(x, q16, c);
      if (valid && q16 == 0) q.rms[(int64_t)sec * q.T + t0 + tok] = rt;
      float* yr = &Y[tok * kYS + 8 * q16];
      *reinterpret_cast<float4*>(yr) = make_float4(c[0], c[1], c[2], c[3]);
      *reinterpret_cast<float4*>(yr + 4) = make_float4(c[4], c[5], c[6], c[7]);
    }
    if (bad && q.status) atomicOr(q.status, 1u << KVTC_ERR_NONFINITE);
  }
  __syncthreads();

  const int64_t ls0 = (int64_t)l * NS;  // first (layer, subspace) row of the tables
  // ---- levels 1 and 2: a wave takes subspaces wave, wave + 4, ... with both token groups
  for (int level = 0; level < 2; ++level) {
    const int k = level ? q.k2 : q.k1;
    uint16_t* const I = level ? I2 : I1;
    for (int it = 0; it < 4; ++it) {
      const int s = wave + 4 * it;
      const int64_t ls = ls0 + s;
      const uint16_t* cbh = (level ? q.cb2h : q.cb1h) + ls * k * SD;
      const uint16_t* c1 = level ? q.cb1h + ls * q.k1 * SD : nullptr;
      const float* cn2 = q.cn2 + ls * (q.k1 + q.k2) + (level ? q.k1 : 0);
      const float cm = q.cmax[ls * 2 + level];
      float best[2], second[2], norm[2];
      search64(Y, s, c1, I1, cbh, cn2, k, best, second, norm);
#pragma unroll
      for (int g2 = 0; g2 < 2; ++g2) {
        const int tok = g2 * 32 + n32;
        const float thr = 0x1p-13f * (norm[g2] * cm + cm * cm) + 0x1p-12f * (fabsf(best[g2]) + fabsf(second[g2]));
        const bool owner = hf == 0 && tok < n;
        // every token gets an index (tokens past the span keep a valid one)
        if (hf == 0) I[tok * NS + s] = (uint16_t)(__float_as_uint(best[g2]) & 0x1FFu & (uint32_t)(k - 1));
        // near ties: decided again exactly, one wave-wide scan each
        uint64_t pend = __ballot(owner && !(__fsub_rn(second[g2], best[g2]) > thr));
        while (pend) {
          const int L = __ffsll((unsigned long long)pend) - 1;
          const int tk = g2 * 32 + (L & 31);
          float ys[SD];
#pragma unroll
          for (int j = 0; j < SD; ++j) ys[j] = Y[tk * kYS + s * SD + j];
          if (level) {
            float cv[8];
            unpack8(*reinterpret_cast<const uint4*>(c1 + ((uint32_t)I1[tk * NS + s] & (q.k1 - 1)) * SD), cv);
#pragma unroll
            for (int j = 0; j < SD; ++j) ys[j] = __fsub_rn(ys[j], cv[j]);
          }
          const int bi = exact_nearest(ys, cbh, k);
          if (lane == L) I[tk * NS + s] = (uint16_t)bi;
          pend &= pend - 1;
        }
      }
    }
    __syncthreads();
  }

  // ---- code rows: level-1 fields, then level-2 fields
  for (int i = tid; i < kSpan * q.rw; i += 256) ROW[i] = 0u;
  __syncthreads();
  for (int it = tid; it < kSpan * NS; it += 256) {
    const int tok = it >> 4, s = it & 15;
    if (tok >= n) continue;
    const uint32_t i1 = I1[tok * NS + s] & (q.k1 - 1), i2 = I2[tok * NS + s] & (q.k2 - 1);
    const int bits[2] = {s * q.b1, NS * q.b1 + s * q.b2};
    const uint32_t vals[2] = {i1, i2}, nbs[2] = {(uint32_t)q.b1, (uint32_t)q.b2};
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const int w = bits[f] >> 5, sh = bits[f] & 31;
      atomicOr(&ROW[tok * q.rw + w], vals[f] << sh);
      if (sh + (int)nbs[f] > 32) atomicOr(&ROW[tok * q.rw + w + 1], vals[f] >> (32 - sh));
    }
  }
  __syncthreads();
  {
    uint32_t* dst = q.codes + ((int64_t)sec * q.T + t0) * q.rw;
    for (int i = tid; i < n * q.rw; i += 256) dst[i] = ROW[i];
  }
  if (q.B == 0) return;
  __syncthreads();  // the rows are read; HIST reuses their memory

  // ---- the span's B largest |y - y^|, then the lowest index: distinct
  // 44-bit keys (|y - y^| bits << 13) | (8191 - e), e = 128 token + channel.
  // Thread tid holds the keys of channel tid % 128 for tokens 2 i + tid / 128
  // (i < 32).  Slots past the span's last token hold |y - y^| = 0 and an
  // index past every real one, so their keys lie below all real keys: they
  // are never among the B largest while there are more than B real keys.
  constexpr int kSel = kSpan / 2;
  const int nel = n * D;
  const uint32_t B = (uint32_t)q.B;
  uint32_t mag[kSel];
  {
    const int j = tid & 127, s = j >> 3, jj = j & 7;
    const uint16_t* c1 = q.cb1h + (ls0 + s) * q.k1 * SD + jj;
    const uint16_t* c2 = q.cb2h + (ls0 + s) * q.k2 * SD + jj;
#pragma unroll
    for (int i = 0; i < kSel; ++i) {
      const int tok = 2 * i + (tid >> 7);  // every token of the span has indices, so reads stay in bounds
      const uint32_t i1 = I1[tok * NS + s] & (q.k1 - 1), i2 = I2[tok * NS + s] & (q.k2 - 1);
      const float yh = __fadd_rn(__uint_as_float((uint32_t)c1[i1 * SD] << 16), __uint_as_float((uint32_t)c2[i2 * SD] << 16));
      const uint32_t m = __float_as_uint(__fsub_rn(Y[tok * kYS + j], yh)) & 0x7fffffffu;
      mag[i] = tok < n ? m : 0u;
    }
  }
  // the key of element e = 128 token + channel (e < nel), from LDS and the
  // codebooks: for the rare walks that need every key in full
  auto key_of = [&](int e) -> uint64_t {
    const int tok = e >> 7, j = e & 127, s = j >> 3, jj = j & 7;
    const uint32_t i1 = I1[tok * NS + s] & (q.k1 - 1), i2 = I2[tok * NS + s] & (q.k2 - 1);
    const float c1v = __uint_as_float((uint32_t)q.cb1h[((ls0 + s) * q.k1 + i1) * SD + jj] << 16);
    const float c2v = __uint_as_float((uint32_t)q.cb2h[((ls0 + s) * q.k2 + i2) * SD + jj] << 16);
    const float dv = __fsub_rn(Y[tok * kYS + j], __fadd_rn(c1v, c2v));
    return ((uint64_t)(__float_as_uint(dv) & 0x7fffffffu) << 13) | (uint64_t)(8191 - e);
  };
  auto each_full = [&](auto f) {
    for (int e = tid; e < nel; e += 256) f(key_of(e));
  };
  uint4* cand = q.cand + ((int64_t)sec * q.nspan + span) * q.B;
  auto put = [&](uint64_t kk, uint32_t slot) {
    const int e = 8191 - (int)(kk & 8191u);
    const int tok = e >> 7, j = e & 127;
    if (slot < B)
      cand[slot] = make_uint4((uint32_t)(kk >> 13), (uint32_t)((t0 + tok) * D + j), __float_as_uint(Y[tok * kYS + j]), 0u);
  };
  if ((uint32_t)nel <= B) {
    each_full([&](uint64_t kk) { put(kk, (uint32_t)(8191 - (int)(kk & 8191u))); });
    return;
  }
  // the top 11 bits over every slot (bits 30..20 of |y - y^|; the index
  // bits play no part); keys above the threshold digit are selected
  // outright, those on it go to a short list for the remaining passes
  uint32_t d0, need;
  radix_pass(
      [&](auto f) {
#pragma unroll
        for (int i = 0; i < kSel; ++i) f((uint64_t)mag[i] << 13);
      },
      33, 11, 0, 0, B, HIST, SM, d0, need);
  const uint32_t on_digit = HIST[d0];
  constexpr uint32_t kList = 512;
  if (tid == 0) { SM[6] = 0u; SM[7] = 0u; }
  __syncthreads();
  if (on_digit <= kList) {
#pragma unroll
    for (int i = 0; i < kSel; ++i) {
      const uint32_t dg = mag[i] >> 20;
      if (dg >= d0) {
        const uint64_t kk = ((uint64_t)mag[i] << 13) | (uint64_t)(8191 - (tid + 256 * i));
        if (dg > d0) put(kk, atomicAdd(&SM[6], 1u));
        else LIST[atomicAdd(&SM[7], 1u)] = kk;
      }
    }
    __syncthreads();
    const int nl = (int)SM[7];
    auto each_list = [&](auto f) {
      for (int e = tid; e < nl; e += 256) f(LIST[e]);
    };
    const uint64_t tau = radix_kth(each_list, 33, need, HIST, SM, (uint64_t)d0 << 33, (uint64_t)0x7FF << 33);
    for (int e = tid; e < nl; e += 256)
      if (LIST[e] >= tau) put(LIST[e], atomicAdd(&SM[6], 1u));
  } else {
    // many equal top digits (e.g. an all-zero error): the remaining passes over every key
    const uint64_t tau = radix_kth(each_full, 33, need, HIST, SM, (uint64_t)d0 << 33, (uint64_t)0x7FF << 33);
    each_full([&](uint64_t kk) {
      if (kk >= tau) put(kk, atomicAdd(&SM[6], 1u));
    });
  }
}

__global__ __launch_bounds__(256) void k_pq_merge(const PqParams q) {
  const int sec = blockIdx.y, blk = blockIdx.x;
  const int tid = threadIdx.x;
  const int spb = q.bt / kSpan;  // spans per block
  const int sp0 = blk * spb, sp1 = min(q.nspan, sp0 + spb);
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];
  __shared__ uint32_t HIST[2048];
  __shared__ uint32_t SM[8];
  __shared__ uint32_t OI[256], OY[256];
  // candidates of the block's spans, back to back: key (63 bits) and y
  uint64_t* const CK = reinterpret_cast<uint64_t*>(dyn);
  int nc = 0;
  for (int sp = sp0; sp < sp1; ++sp) {
    const int nsp = min(kSpan, q.T - sp * kSpan);
    const int cnt = min(q.B, nsp * D);
    const uint4* src = q.cand + ((int64_t)sec * q.nspan + sp) * q.B;
    for (int i = tid; i < cnt; i += 256) {
      const uint4 c = src[i];
      CK[nc + i] = ((uint64_t)c.x << 32) | (uint64_t)(0xFFFFFFFFu - c.y);
    }
    nc += cnt;
  }
  uint32_t* const CY = reinterpret_cast<uint32_t*>(CK + nc);
  nc = 0;
  for (int sp = sp0; sp < sp1; ++sp) {
    const int nsp = min(kSpan, q.T - sp * kSpan);
    const int cnt = min(q.B, nsp * D);
    const uint4* src = q.cand + ((int64_t)sec * q.nspan + sp) * q.B;
    for (int i = tid; i < cnt; i += 256) CY[nc + i] = src[i].z;
    nc += cnt;
  }
  __syncthreads();
  const uint32_t B = (uint32_t)q.B;
  uint64_t tau = 0;
  auto each_cand = [&](auto f) {
    for (int e = tid; e < nc; e += 256) f(CK[e]);
  };
  if ((uint32_t)nc > B) tau = radix_kth(each_cand, 63, B, HIST, SM);
  if (tid == 0) SM[6] = 0u;
  __syncthreads();
  for (int e = tid; e < nc; e += 256) {
    if ((uint32_t)nc <= B || CK[e] >= tau) {
      const uint32_t slot = atomicAdd(&SM[6], 1u);
      if (slot < B) {
        OI[slot] = 0xFFFFFFFFu - (uint32_t)CK[e];
        OY[slot] = CY[e];
      }
    }
  }
  __syncthreads();
  const uint32_t nsel = min(SM[6], B);
  uint32_t* out = q.outl + (((int64_t)sec * q.nblk + blk) * q.B) * 2;
  for (uint32_t a = tid; a < B; a += 256) {
    if (a < nsel) {
      // index-ascending: the rank among the selected (indices are distinct)
      const uint32_t idx = OI[a];
      uint32_t rank = 0;
      for (uint32_t b = 0; b < nsel; ++b) rank += OI[b] < idx ? 1u : 0u;
      out[2 * rank] = idx;
      out[2 * rank + 1] = OY[a];
    } else {
      out[2 * a] = 0xFFFFFFFFu;
      out[2 * a + 1] = 0u;
    }
  }
}

__global__ __launch_bounds__(256) void k_pq_dec(const PqParams q) {
  const int sec = blockIdx.y, span = blockIdx.x;
  const int l = sec / q.H;
  const int t0 = span * kSpan, n = min(kSpan, q.T - t0);
  const int tid = threadIdx.x, lane = tid & 63;
  __shared__ __attribute__((aligned(16))) float Y[kSpan * kYS];
  __shared__ uint32_t ROW[kSpan * kMaxRow];
  {
    const uint32_t* src = q.codes + ((int64_t)sec * q.T + t0) * q.rw;
    for (int i = tid; i < n * q.rw; i += 256) ROW[i] = src[i];
  }
  __syncthreads();
  const int64_t ls0 = (int64_t)l * NS;
  for (int it = tid; it < kSpan * NS; it += 256) {
    const int tok = it >> 4, s = it & 15;
    if (tok >= n) continue;
    uint32_t f[2];
    const int bits[2] = {s * q.b1, NS * q.b1 + s * q.b2}, nbs[2] = {q.b1, q.b2};
#pragma unroll
    for (int z = 0; z < 2; ++z) {
      const int w = bits[z] >> 5, sh = bits[z] & 31;
      uint64_t v = ROW[tok * q.rw + w];
      if (sh + nbs[z] > 32) v |= (uint64_t)ROW[tok * q.rw + w + 1] << 32;
      f[z] = (uint32_t)(v >> sh) & ((1u << nbs[z]) - 1u);
    }
    float c1[8], c2[8];
    unpack8(*reinterpret_cast<const uint4*>(q.cb1h + ((ls0 + s) * q.k1 + f[0]) * SD), c1);
    unpack8(*reinterpret_cast<const uint4*>(q.cb2h + ((ls0 + s) * q.k2 + f[1]) * SD), c2);
    float* yr = &Y[tok * kYS + s * SD];
    *reinterpret_cast<float4*>(yr) =
        make_float4(__fadd_rn(c1[0], c2[0]), __fadd_rn(c1[1], c2[1]), __fadd_rn(c1[2], c2[2]), __fadd_rn(c1[3], c2[3]));
    *reinterpret_cast<float4*>(yr + 4) =
        make_float4(__fadd_rn(c1[4], c2[4]), __fadd_rn(c1[5], c2[5]), __fadd_rn(c1[6], c2[6]), __fadd_rn(c1[7], c2[7]));
  }
  __syncthreads();
  // the block's outliers inside this span replace their coefficients
  if (q.B > 0) {
    const int blk = t0 / q.bt;
    const int64_t lo = (int64_t)blk * q.bt * D, hi = (int64_t)min(q.T, (blk + 1) * q.bt) * D;
    const uint32_t* o = q.outl + (((int64_t)sec * q.nblk + blk) * q.B) * 2;
    for (int a = tid; a < q.B; a += 256) {
      const uint32_t idx = o[2 * a];
      if (idx == 0xFFFFFFFFu) continue;
      if ((int64_t)idx < lo || (int64_t)idx >= hi) {
        if (q.status) atomicOr(q.status, 1u << KVTC_ERR_CORRUPT);
        continue;
      }
      const int64_t rel = (int64_t)idx - (int64_t)t0 * D;
      if (rel >= 0 && rel < (int64_t)n * D) Y[(rel >> 7) * kYS + (rel & 127)] = __uint_as_float(o[2 * a + 1]);
    }
  }
  __syncthreads();
  // inverse transform (the orthonormal WHT is its own inverse), times r
  const int q16 = lane & 15, grp = tid >> 4;
  const double rs = __dsqrt_rn((double)D), irs = __ddiv_rn(1.0, rs);
  for (int pass = 0; pass < 4; ++pass) {
    const int tok = pass * 16 + grp;
    double y[8];
    const float* yr = &Y[tok * kYS + 8 * q16];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = (double)yr[e];
    wht_fp64(y, q16);
    if (tok >= n) continue;
    const float rt = q.rms[(int64_t)sec * q.T + t0 + tok];
    float o[8];
    quot_f32(y, rs, irs, o);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = __fmul_rn(o[e], rt);
    const int64_t row = ((int64_t)sec * q.T + t0 + tok) * D + 8 * q16;
    if (q.out_dtype == KVTC_FP32) {
      float* dst = reinterpret_cast<float*>(q.v_out) + row;
      store_out16(dst, make_float4(o[0], o[1], o[2], o[3]));
      store_out16(dst + 4, make_float4(o[4], o[5], o[6], o[7]));
    } else {
      uint32_t h[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) h[e] = (uint32_t)f32_to_bf16(o[e]);
      store_out16(reinterpret_cast<uint16_t*>(q.v_out) + row,
                  make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)));
    }
  }
}

hipError_t launch_pq_encode(const PqParams& q, hipStream_t s) {
  hipLaunchKernelGGL(k_pq_prep, dim3((unsigned)(q.L * NS)), dim3(256), 0, s, q);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || q.T == 0) return e;
  hipLaunchKernelGGL(k_pq_enc, dim3((unsigned)q.nspan, (unsigned)(q.L * q.H)), dim3(256), 0, s, q);
  e = hipGetLastError();
  if (e != hipSuccess || q.B == 0) return e;
  const int spb = q.bt / kSpan;
  const size_t lds = (size_t)spb * q.B * 12;
  (void)hipFuncSetAttribute((const void*)k_pq_merge, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  hipLaunchKernelGGL(k_pq_merge, dim3((unsigned)q.nblk, (unsigned)(q.L * q.H)), dim3(256), lds, s, q);
  return hipGetLastError();
}

hipError_t launch_pq_decode(const PqParams& q, hipStream_t s) {
  hipLaunchKernelGGL(k_pq_prep, dim3((unsigned)(q.L * NS)), dim3(256), 0, s, q);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || q.T == 0) return e;
  hipLaunchKernelGGL(k_pq_dec, dim3((unsigned)q.nspan, (unsigned)(q.L * q.H)), dim3(256), 0, s, q);
  return hipGetLastError();
}

}  // namespace kvtc
