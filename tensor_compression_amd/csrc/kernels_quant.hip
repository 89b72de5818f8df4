// Quantise-and-pack pass, head_dim 128, bf16 cache, PCA transform
// (KVTC "Quantization and bit allocation"; Codec-Gauge "Problem Statement
// and Overview": B_c = Q(Z_c), channel-major packing of the codes).
//
// Workgroup = eight packed tiles of one section, one wave per tile.  Only the
// components with codes (b > 0) are projected: they are ordered by width and
// their basis columns are staged in LDS as MFMA B fragments of 16 components.
// A wave walks its tile in 16-token groups with the token rows loaded
// straight from global memory as MFMA A operands (lane (g, r) of group kk
// holds token 16 kk + r, channels 32 kb + 8 g .. +7; the next two groups'
// rows are in flight meanwhile).  For each 16-component tile the result lane
// (g, r) holds tokens 16 kk + 4 g .. +3 of component 16 m + r, i.e. four
// consecutive codes of one channel-major row.
//
// Quantisation: v = (c - zero) * rcp, clamped to [0, 2^b - 1] and rounded to
// nearest even by adding 2^23, whose float bits then carry the code.  The
// four codes of a lane fold into one 4b-bit piece that is OR-ed into the
// wave's LDS segment buffer (the sub-tile's slice of every row); the buffer
// is copied to the packed tile after every 64 tokens.  A code is recomputed
// on the spot from the exact dot product (fp64 sum of the exact bf16
// products, over the four lanes that hold the token) when v lies within the
// coefficient's error bound of a rounding boundary: |c_mfma - c| <= mfma_err ||x||_2 (fp32 accumulation of
// the exact products; Cauchy-Schwarz), with ||x||_2 from a bf16 dot product
// of the token with itself, taken 1% high.
#include <string.h>

#include <type_traits>

#include "kvtc_internal.h"

namespace kvtc {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

struct QInfo {     // per component, sorted order (b > 0 first, by width)
  uint32_t idx;    // natural component index
  uint32_t b;      // width
  float zero, rcp;
  float thr;       // 0.5 minus the rounding error of v
  uint32_t kb;     // 0x4B000000 (1 + 2^b + 2^2b + 2^3b) mod 2^32
  uint32_t seg;    // word offset of the component's slice in the segment buffer
  uint32_t pad;    // fp32 bits of mfma_err * rcp: error of v per unit token norm
};

constexpr int kQWaves = 8;  // one packed tile per wave
// Per-wave queue of codes to recompute exactly.  The hot loop only notes, in a
// scalar bitmask, which 16 x 16 steps of a 16-token group had a code within
// its error bound of a rounding boundary; after the group those steps are
// redone and their codes queued (one step adds at most 256 entries, and the
// queue is drained once it holds kQDrain or more).
constexpr int kQDrain = 64;
constexpr int kQCap = kQDrain + 256;

__global__ __launch_bounds__(64 * kQWaves, 4) void k_quant128(const Params p0) {
  const Params p = at_seq(p0, blockIdx.z);
  constexpr int D = 128;
  const int u = blockIdx.y;
  const int h = u % p.H, s = (u / p.H) & 1, l = u / (2 * p.H);
  if (get_status(p.ws, p.w) & (1u << KVTC_ERR_NONFINITE)) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, r = lane & 15;

  __shared__ QInfo s_q[D];
  __shared__ uint8_t s_rank[D];
  __shared__ uint32_t s_bs[D];          // widths in sorted order
  __shared__ uint32_t s_row[kQWaves][D];  // per wave: row offset (words) in its tile, sorted order
  __shared__ uint8_t s_wmap[2048 + 64];   // segment-buffer word -> sorted component
  __shared__ int32_t s_misc[4];           // nnz, segment words, full tile words
  __shared__ uint32_t s_queue[kQWaves][kQCap];  // (sub-tile token << 16) | (sorted component << 8) | code
  extern __shared__ __attribute__((aligned(16))) uint32_t dq[];  // [B fragments][segment buffers]

  const int64_t si0 = (int64_t)u * D;
  if (wave == 0) {
    // order the components by width, b = 0 last
    const uint32_t b0 = p.ws[p.w.side_bits + si0 + 2 * lane], b1 = p.ws[p.w.side_bits + si0 + 2 * lane + 1];
    const uint32_t k0 = b0 ? b0 : 9u, k1 = b1 ? b1 : 9u;
    const uint64_t lt = (1ull << lane) - 1ull;
    uint32_t base = 0, r0 = 0, r1 = 0, nnz = 0;
    for (uint32_t v = 1; v <= 9; ++v) {
      const uint64_t m0 = __ballot(k0 == v), m1 = __ballot(k1 == v);
      const uint32_t before = base + __popcll(m0 & lt) + __popcll(m1 & lt);
      if (k0 == v) r0 = before;
      if (k1 == v) r1 = before + (k0 == v ? 1u : 0u);
      base += __popcll(m0) + __popcll(m1);
      if (v == 8) nnz = base;
    }
    s_rank[2 * lane] = (uint8_t)r0;
    s_rank[2 * lane + 1] = (uint8_t)r1;
    s_bs[r0] = b0;
    s_bs[r1] = b1;
    uint32_t fw = ((uint32_t)(p.tile_tokens * (int)b0 + 31) >> 5) + ((uint32_t)(p.tile_tokens * (int)b1 + 31) >> 5);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) fw += __shfl_xor(fw, o, 64);
    __builtin_amdgcn_wave_barrier();
    // segment offsets: exclusive scan of 2 b over the sorted order
    const uint32_t sb0 = s_bs[2 * lane], sb1 = s_bs[2 * lane + 1];
    uint32_t x = 2 * (sb0 + sb1);
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    const uint32_t segw = __shfl(x, 63, 64);
    const uint32_t seg0 = x - 2 * (sb0 + sb1), seg1 = seg0 + 2 * sb0;
    const float* zr = reinterpret_cast<const float*>(p.ws + p.w.side_zero) + si0;
    const float* rc = reinterpret_cast<const float*>(p.ws + p.w.side_rcp) + si0;
    auto info = [&](uint32_t i, uint32_t b, uint32_t seg) {
      QInfo q;
      q.idx = i; q.b = b; q.zero = zr[i]; q.rcp = rc[i];
      // error of v: (coefficient bound per unit token norm) * rcp, and the
      // rounding term of v itself (subtracted from 0.5 in thr)
      q.thr = 0.5f - 3.0f * 0x1p-23f * (float)(1u << b);
      q.pad = __float_as_uint(p.mfma_err * q.rcp);
      q.kb = 0x4B000000u * (1u + (1u << b) + (1u << (2 * b)) + (1u << (3 * b)));
      q.seg = seg;
      return q;
    };
    s_q[r0] = info(2 * lane, b0, 0);
    s_q[r1] = info(2 * lane + 1, b1, 0);
    __builtin_amdgcn_wave_barrier();
    s_q[2 * lane].seg = seg0;
    s_q[2 * lane + 1].seg = seg1;
    // word -> component map of the segment buffer
    for (uint32_t w = 0; w < 2 * sb0; ++w) s_wmap[seg0 + w] = (uint8_t)(2 * lane);
    for (uint32_t w = 0; w < 2 * sb1; ++w) s_wmap[seg1 + w] = (uint8_t)(2 * lane + 1);
    if (lane == 0) { s_misc[0] = (int32_t)nnz; s_misc[1] = (int32_t)segw; s_misc[2] = (int32_t)fw; }
  }
  __syncthreads();
  const int nnz = s_misc[0];
  const int NT = (nnz + 15) >> 4;
  const uint32_t segw = (uint32_t)s_misc[1], fw = (uint32_t)s_misc[2];
  if (nnz == 0) return;  // no codes: every tile is empty
  uint4* sB = reinterpret_cast<uint4*>(dq);
  const int segstride = ((int)segw + 4 + 3) & ~3;  // words per wave, 16-byte aligned
  uint32_t* segbuf = dq + NT * 4 * 64 * 4 + wave * segstride;
  // B fragments [m][kb][lane]: lane (g, r) holds channels 32 kb + 8 g .. +7 of
  // the basis column of sorted component 16 m + r
  {
    const int64_t bidx = (p.basis_per_head ? ((int64_t)(l * 2 + s) * p.H + h) : (int64_t)(l * 2 + s)) * D * D;
    const uint16_t* bt = reinterpret_cast<const uint16_t*>(p.basis_t) + bidx;
    for (int f = wave; f < NT * 4; f += kQWaves) {
      const int m = f >> 2, kb = f & 3, k = 16 * m + r;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (k < nnz) v = *reinterpret_cast<const uint4*>(bt + (int64_t)s_q[k].idx * D + 32 * kb + 8 * g);
      sB[f * 64 + lane] = v;
    }
  }
  __syncthreads();

  // token rows: keys with RoPE come from the workspace copy with the rotation removed
  const bool pre = s == 0 && p.rope_keys;
  const uint16_t* src = pre ? reinterpret_cast<const uint16_t*>(p.ws + p.w.kprime)
                            : reinterpret_cast<const uint16_t*>(s ? p.v : p.k);
  uint32_t refined = 0;
  // this wave's tile: the f-th tile of the section
  const int f = blockIdx.x * kQWaves + wave;
  const int ch = f / p.tiles_per_chunk, tl = f % p.tiles_per_chunk;
  const int t0 = ch * p.chunk_tokens;
  const int n = min(p.chunk_tokens, p.T_mid - t0);
  const int ta = tl * p.tile_tokens;
  if (ch < p.chunks_per_sec && ta < n) {
    const int nt = min(p.tile_tokens, n - ta);
    const int64_t row0 = ((int64_t)l * p.H + h) * (pre ? p.T_mid : p.T) + (pre ? 0 : p.mid_begin) + t0 + ta;
    uint32_t* tile = reinterpret_cast<uint32_t*>(p.ws + p.w.packed + (int64_t)(u * p.chunks_per_sec + ch) * p.w.packed_slot) +
                     (int64_t)tl * fw;
    // row offsets of this tile (natural order scan), by sorted position
    {
      const uint32_t b0 = s_bs[s_rank[2 * lane]], b1 = s_bs[s_rank[2 * lane + 1]];
      const uint32_t w0 = (uint32_t)(nt * (int)b0 + 31) >> 5, w1 = (uint32_t)(nt * (int)b1 + 31) >> 5;
      uint32_t x = w0 + w1;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
      }
      const uint32_t ex = x - (w0 + w1);
      s_row[wave][s_rank[2 * lane]] = ex;
      s_row[wave][s_rank[2 * lane + 1]] = ex + w0;
    }
    // A operands of a 16-token group: lane (g, r) holds token 16 kk + r (rows
    // past the tile repeat its last token), channels 32 kb + 8 g .. +7
    auto load_group = [&](int sub, int kk, uint4 (&a)[4]) {
      const int tok = min(sub * 64 + kk * 16 + r, nt - 1);
      const uint16_t* rowp = src + (pre ? (row0 + tok) * D : cache_row(p, l, h, p.mid_begin + t0 + ta + tok));
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) a[kb] = *reinterpret_cast<const uint4*>(rowp + 32 * kb + 8 * g);
    };
    // four group buffers: group kk of a sub-tile lives in Ab[kk]; the loads of
    // group kk + 2 are issued while group kk is projected
    uint4 Ab[4][4];
    load_group(0, 0, Ab[0]);
    load_group(0, 1, Ab[1]);
    // Exact re-computation of the queued codes, one per lane: the fp64 sum of
    // the 128 exact bf16 products (four independent partial sums), rounded to
    // fp32 once, then the code; a changed code is XOR-ed into the segment
    // buffer over the provisional one.
    uint32_t* queue = s_queue[wave];
    int qn = 0;
    auto drain = [&](int sub) {
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
      for (int q0 = 0; q0 < qn; q0 += 64) {
        if (q0 + lane < qn) {
          const uint32_t ent = queue[q0 + lane];
          const int t = (int)(ent >> 16), k = (int)((ent >> 8) & 0xffu);
          const uint32_t old = ent & 0xffu;
          const QInfo qk = s_q[k];
          const int tt = sub * 64 + t;  // tile-relative token
          const uint16_t* rowp = src + (pre ? (row0 + tt) * D : cache_row(p, l, h, p.mid_begin + t0 + ta + tt));
          const int mk = k >> 4, rk = k & 15;
          double part[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll 1
          for (int kb = 0; kb < 4; ++kb) {
#pragma unroll 1
            for (int gq = 0; gq < 4; ++gq) {
              // channels 32 kb + 8 gq .. +7: the token row and the component's basis fragment
              const uint4 xv = *reinterpret_cast<const uint4*>(rowp + 32 * kb + 8 * gq);
              const uint4 bv = sB[(mk * 4 + kb) * 64 + 16 * gq + rk];
              const uint32_t aw[4] = {xv.x, xv.y, xv.z, xv.w}, bw[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
              for (int z = 0; z < 4; ++z) {
                part[z] += (double)__fmul_rn(__uint_as_float(aw[z] << 16), __uint_as_float(bw[z] << 16));
                part[z] += (double)__fmul_rn(__uint_as_float(aw[z] & 0xffff0000u), __uint_as_float(bw[z] & 0xffff0000u));
              }
            }
          }
          const double cex = (part[0] + part[1]) + (part[2] + part[3]);
          const float v = __fmul_rn(__fsub_rn((float)cex, qk.zero), qk.rcp);
          const uint32_t code = __float_as_uint(__fadd_rn(__builtin_amdgcn_fmed3f(v, 0.0f, (float)((1u << qk.b) - 1u)),
                                                          0x1p23f)) & 0xffu;
          const uint64_t dx = (uint64_t)(code ^ old) << ((t * qk.b) & 31);
          const uint32_t wi = qk.seg + (((uint32_t)t * qk.b) >> 5);
          if (dx) {
            atomicXor(&segbuf[wi], (uint32_t)dx);
            if (dx >> 32) atomicXor(&segbuf[wi + 1], (uint32_t)(dx >> 32));
          }
        }
      }
      refined += (uint32_t)qn;
      qn = 0;
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
    };
    // The 16 x 16 (token x component) steps of one 16-token group: project,
    // quantise, queue the codes within their error bound of a rounding
    // boundary, OR the provisional codes into segbuf.  FULL: the tile has
    // every token (no tail masking).
    auto group = [&](auto full_tag, const uint4 (&A)[4], const float (&tn)[4], int kk, int tb0, int sub) {
      constexpr bool FULL = decltype(full_tag)::value;
      for (int m = 0; m < NT; ++m) {
        uint4 Bm[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) Bm[kb] = sB[(m * 4 + kb) * 64 + lane];
        const QInfo qi = s_q[16 * m + r];
        const uint32_t b = qi.b;
        const float qmax = (float)((1u << b) - 1u);
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, A[kb]),
                                                        __builtin_bit_cast(bf16x8_t, Bm[kb]), acc, 0, 0, 0);
        uint32_t uq[4];
        uint64_t near[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // components without codes (b = 0, rcp = 0, qmax = 0) give v = 0 and
          // code 0, so only the token tail needs masking
          const float v = __fmul_rn(__fsub_rn(acc[e], qi.zero), qi.rcp);
          const float vc = (FULL || tb0 + e < nt) ? __builtin_amdgcn_fmed3f(v, 0.0f, qmax) : 0.0f;
          const float sv = __fadd_rn(vc, 0x1p23f);  // rint(vc), nearest even, in the low bits
          uq[e] = __float_as_uint(sv);
          const float d = __fsub_rn(vc, __fsub_rn(sv, 0x1p23f));
          near[e] = __ballot(fabsf(d) > __fmaf_rn(-__uint_as_float(qi.pad), tn[e], qi.thr));
        }
        if (near[0] | near[1] | near[2] | near[3]) {
          // queue them: (sub-tile token, sorted component, provisional code)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (near[e]) {
              const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(near[e] >> 32),
                                                               __builtin_amdgcn_mbcnt_lo((uint32_t)near[e], 0u));
              if ((near[e] >> lane) & 1ull)
                queue[qn + below] = ((uint32_t)((tb0 & 63) + e) << 16) | ((uint32_t)(16 * m + r) << 8) | (uq[e] & 0xffu);
              qn += (int)__popcll(near[e]);
            }
          }
        }
        // four codes -> one 4b-bit piece (the exponent bits cancel in kb)
        const uint32_t piece = uq[0] + (uq[1] << b) + (uq[2] << (2 * b)) + (uq[3] << (3 * b)) - qi.kb;
        if (piece != 0u) {
          const uint32_t bitoff = (uint32_t)(kk * 16 + 4 * g) * b;
          const uint32_t wi = qi.seg + (bitoff >> 5), sh = bitoff & 31;
          atomicOr(&segbuf[wi], piece << sh);
          if (sh + 4 * b > 32) atomicOr(&segbuf[wi + 1], piece >> (32 - sh));
        }
        if (qn >= kQDrain) drain(sub);
      }
    };
    const bool full = nt == p.tile_tokens;
    for (int sub = 0; sub * 64 < nt; ++sub) {
      for (uint32_t w = lane; w < segw + 4; w += 64) segbuf[w] = 0u;
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        // group kk + 2 of this sub-tile or of the next (the loads of groups
        // past the tile are clamped to its last token and never used)
        load_group(sub + ((kk + 2) >> 2), (kk + 2) & 3, Ab[(kk + 2) & 3]);
        const uint4 (&A)[4] = Ab[kk];
        // norm bound of the token of output element (row 4 g + e of the group)
        float tn[4];
        {
          float n2 = 0.f;
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            const uint32_t w4[4] = {A[kb].x, A[kb].y, A[kb].z, A[kb].w};
#pragma unroll
            for (int z = 0; z < 4; ++z) {
              const bf16x2_t h2 = __builtin_bit_cast(bf16x2_t, w4[z]);
              n2 = __builtin_amdgcn_fdot2_f32_bf16(h2, h2, n2, false);
            }
          }
          n2 += __shfl_xor(n2, 16, 64);
          n2 += __shfl_xor(n2, 32, 64);
#pragma unroll
          for (int e = 0; e < 4; ++e) tn[e] = 1.01f * __fsqrt_rn(__shfl(n2, 4 * g + e, 64));
        }
        const int tb0 = sub * 64 + kk * 16 + 4 * g;  // tile-relative token of element 0
        if (full) group(std::true_type{}, A, tn, kk, tb0, sub);
        else group(std::false_type{}, A, tn, kk, tb0, sub);
      }
      if (qn > 0) drain(sub);
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
      // segment buffer -> the rows of the packed tile
      for (uint32_t w = lane; w < segw; w += 64) {
        const uint32_t k = s_wmap[w];
        const QInfo& qk = s_q[k];
        const uint32_t idx = w - qk.seg;
        const int32_t rw = (int32_t)((nt * (int)qk.b + 31) >> 5) - (int32_t)(2 * qk.b * sub);
        if ((int32_t)idx < rw) tile[s_row[wave][k] + 2 * qk.b * sub + idx] = segbuf[w];
      }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
    }
  }
  if (lane == 0 && refined) atomicAdd(reinterpret_cast<uint32_t*>(p.ws + p.w.status) + 1, refined);
}

hipError_t launch_quant128(const Params& p, hipStream_t s) {
  const int32_t bmax = p.budget_k > p.budget_v ? p.budget_k : p.budget_v;
  // segment buffer: 64 tokens of every row, 2 b words per component
  const int segw = 2 * (bmax < 8 * p.D ? bmax : 8 * p.D);
  if (segw > 2048) return hipErrorInvalidValue;
  const int segstride = (segw + 4 + 3) & ~3;
  const size_t lds = (size_t)8 * 4 * 64 * 16 + (size_t)kQWaves * segstride * 4;
  const int tiles = p.chunks_per_sec * p.tiles_per_chunk;
  (void)hipFuncSetAttribute((const void*)k_quant128, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  hipLaunchKernelGGL(k_quant128, dim3((tiles + kQWaves - 1) / kQWaves, p.n_sections, seq_grid(p)), dim3(64 * kQWaves), lds, s, p);
  return hipGetLastError();
}

}  // namespace kvtc
