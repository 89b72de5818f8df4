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
// from the exact dot product (fp64 sum of the exact bf16 products) when v
// lies within the coefficient's error bound of a rounding boundary:
// |c_mfma - c| <= mfma_err ||x||_2 (fp32 accumulation of the exact products;
// Cauchy-Schwarz), with ||x||_2 from a bf16 dot product of the token with
// itself, taken 1% high.
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

// The lane index, formed anew at each use: lane-derived addresses are then
// recomputed where they are needed instead of held in registers across the
// projection loop.
__device__ __forceinline__ int fresh_lane() {
  int x;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(x));
  return x;
}
// Per-wave queue of codes to recompute exactly.  The hot loop only sets, per
// lane, one bit for every code of its pair that lies within its error bound
// of a rounding boundary; after every 64 tokens (once they are in the packed
// tile) the flagged codes are queued, and the queue is worked off at the end
// of the tile, or when it fills up, with all its loads in flight together.
constexpr int kQCap = 128;
// fl * 2 + (|d| > bnd): the compare's lane mask is the carry-in of one
// add-with-carry (false for a NaN d, like the C comparison)
__device__ __forceinline__ uint32_t shift_in_flag(uint32_t fl, float d, float bnd) {
  uint32_t r;
  asm("v_cmp_gt_f32_e64 vcc, |%1|, %2\n\tv_addc_co_u32_e32 %0, vcc, %3, %3, vcc" : "=v"(r) : "v"(d), "v"(bnd), "v"(fl) : "vcc");
  return r;
}

__global__ __launch_bounds__(64 * kQWaves, 4) void k_quant128(const Params p0) {
  const Params p = at_seq(p0, blockIdx.z);
  constexpr int D = 128;
  const int u = blockIdx.y;
  const int h = u % p.H, s = (u / p.H) & 1, l = u / (2 * p.H);
  if (get_status(p.ws, p.w) & (1u << KVTC_ERR_NONFINITE)) return;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, r = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in scalar registers

  __shared__ QInfo s_q[D];
  __shared__ float4 s_hf[D];            // hot loop: rcp, -zero rcp, 2^b - 1, margin
  __shared__ uint4 s_hu[D];             // hot loop: b, kb, seg, pad
  __shared__ uint8_t s_rank[D];
  __shared__ uint32_t s_bs[D];          // widths in sorted order
  __shared__ uint32_t s_row[kQWaves][D];  // per wave: row offset (words) in its tile, sorted order
  __shared__ uint8_t s_wmap[2048 + 64];   // segment-buffer word -> sorted component
  __shared__ int32_t s_misc[4];           // nnz, segment words, full tile words
  __shared__ uint32_t s_flags[kQWaves][4][64];    // per wave: flags of the sub-tile's pairs and halves
  __shared__ uint32_t s_queue[kQWaves][kQCap];  // (tile token << 16) | (sorted component << 8)
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
#pragma unroll
    for (int z = 0; z < 2; ++z) {
      // the hot loop forms v as one fma, c rcp + (-zero rcp); against the
      // two roundings of (c - zero) rcp that adds the rounding of -zero rcp
      // and of the fma to the margin to the rounding boundary
      const QInfo& q = s_q[2 * lane + z];
      const float nzr = __fmul_rn(-q.zero, q.rcp);
      const float thr = q.thr - 0x1p-23f * fabsf(nzr);
      s_hf[2 * lane + z] = make_float4(q.rcp, nzr, (float)((1u << q.b) - 1u), thr);
      s_hu[2 * lane + z] = make_uint4(q.b, q.kb, z ? seg1 : seg0, q.pad);
    }
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
  const int ch = f / p.tiles_per_blk, tl = f % p.tiles_per_blk;
  const int t0 = ch * p.blk_tokens;
  const int n = min(p.blk_tokens, p.T_mid - t0);
  const int ta = tl * p.tile_tokens;
  if (ch < p.blks_per_sec && ta < n) {
    const int nt = min(p.tile_tokens, n - ta);
    const int64_t row0 = ((int64_t)l * p.H + h) * (pre ? p.T_mid : p.T) + (pre ? 0 : p.mid_begin) + t0 + ta;
    uint32_t* tile = reinterpret_cast<uint32_t*>(p.ws + p.w.packed + (int64_t)(u * p.blks_per_sec + ch) * p.w.packed_slot) +
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
    // A operands of a 32-token pair, two 16-row halves h: row 4 i + e of half
    // h holds token 8 i + 4 h + e, so that result lane (g, r) holds tokens
    // 8 g .. 8 g + 7 of one component, eight consecutive codes of one row.
    // Lane (g, r) loads rows r of both halves, channels 32 kb + 8 g .. +7
    // (rows past the tile repeat its last token).
    auto load_pair = [&](int pr, uint4 (&a)[2][4]) {
      const int ln = fresh_lane(), g = ln >> 4, r = ln & 15;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int tok = min(pr * 32 + 8 * (r >> 2) + 4 * hh + (r & 3), nt - 1);
        const uint16_t* rowp = src + (pre ? (row0 + tok) * D : cache_row(p, l, h, p.mid_begin + t0 + ta + tok));
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) a[hh][kb] = *reinterpret_cast<const uint4*>(rowp + 32 * kb + 8 * g);
      }
    };
    // two pair buffers: pair P + 1 is in flight while pair P is projected
    uint4 Ab[2][2][4];
    load_pair(0, Ab[0]);
    // Exact re-computation of the queued codes, 16 Z at a time: four lanes per
    // code each take 32 channels of the token row (four 16-byte loads; the
    // loads of all 16 Z codes, and of the packed words that hold their
    // provisional values, are issued together) and the matching basis
    // fragments, sum the exact bf16 products in fp64 and reduce across the
    // four; the sum is rounded to fp32 once and quantised, and a changed code
    // is XOR-ed into the packed tile over the provisional one.
    uint32_t* queue = s_queue[wave];
    auto drain = [&](auto z_tag, int qn) {
      constexpr int Z = decltype(z_tag)::value;
      const int lane = fresh_lane();
      // the packed words are stored before they are read back
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_wave_barrier();
      const int j = lane & 3;
      for (int q0 = 0; q0 < qn; q0 += 16 * Z) {
        uint32_t ent[Z], wd[Z][2];
        uint4 xv[Z][4];
#pragma unroll
        for (int z = 0; z < Z; ++z) {
          const int qe = q0 + 16 * z + (lane >> 2);
          ent[z] = queue[qe < qn ? qe : q0];
          const int t = (int)(ent[z] >> 16), k = (int)((ent[z] >> 8) & 0xffu);  // tile-relative token
          const uint16_t* rowp = src + (pre ? (row0 + t) * D : cache_row(p, l, h, p.mid_begin + t0 + ta + t));
#pragma unroll
          for (int q = 0; q < 4; ++q) xv[z][q] = *reinterpret_cast<const uint4*>(rowp + 32 * j + 8 * q);
          // the one or two packed words of the code (the second read only
          // when the code crosses into it)
          const uint32_t b = s_bs[k], bitpos = (uint32_t)t * b;
          uint32_t* wp = tile + s_row[wave][k] + (bitpos >> 5);
          wd[z][0] = __hip_atomic_load(wp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          wd[z][1] = __hip_atomic_load(wp + ((bitpos & 31) + b > 32 ? 1 : 0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int z = 0; z < Z; ++z) {
          const int k = (int)((ent[z] >> 8) & 0xffu);
          double part[2] = {0.0, 0.0};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            // channels 32 j + 8 q .. +7 of the component's basis column
            const uint4 bv = sB[((k >> 4) * 4 + j) * 64 + 16 * q + (k & 15)];
            const uint32_t aw[4] = {xv[z][q].x, xv[z][q].y, xv[z][q].z, xv[z][q].w};
            const uint32_t bw[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
            for (int y = 0; y < 4; ++y) {
              part[0] += (double)__fmul_rn(__uint_as_float(aw[y] << 16), __uint_as_float(bw[y] << 16));
              part[1] += (double)__fmul_rn(__uint_as_float(aw[y] & 0xffff0000u), __uint_as_float(bw[y] & 0xffff0000u));
            }
          }
          double cex = part[0] + part[1];
          cex += __shfl_xor(cex, 1, 64);
          cex += __shfl_xor(cex, 2, 64);
          if (j == 0 && q0 + 16 * z + (lane >> 2) < qn) {
            const QInfo qk = s_q[k];
            const int t = (int)(ent[z] >> 16);
            const float v = __fmul_rn(__fsub_rn((float)cex, qk.zero), qk.rcp);
            const uint32_t code = __float_as_uint(__fadd_rn(__builtin_amdgcn_fmed3f(v, 0.0f, (float)((1u << qk.b) - 1u)),
                                                            0x1p23f)) & 0xffu;
            const uint32_t bitpos = (uint32_t)t * qk.b, sh = bitpos & 31;
            const uint64_t cur = (uint64_t)wd[z][0] | ((uint64_t)wd[z][1] << 32);
            const uint32_t old = (uint32_t)(cur >> sh) & ((1u << qk.b) - 1u);
            const uint64_t dx = (uint64_t)(code ^ old) << sh;
            uint32_t* wp = tile + s_row[wave][k] + (bitpos >> 5);
            if (dx) {
              atomicXor(wp, (uint32_t)dx);
              if (dx >> 32) atomicXor(wp + 1, (uint32_t)(dx >> 32));
            }
          }
        }
      }
      refined += (uint32_t)qn;
    };
    // The 32 x 16 (token x component) steps of one pair: project, quantise,
    // OR the provisional codes into segbuf and shift into fl[h] one flag per
    // code (step m, element e at bit 4 (NT - 1 - m) + 3 - e) for the codes
    // within their error bound of a rounding boundary.  No LDS access here
    // depends on the data, so every wait on LDS stays exact.  FULL: the tile
    // has every token (no tail masking).
    auto pair = [&](auto full_tag, const uint4 (&A)[2][4], float tnmax, int P, int tb0, uint32_t (&fl)[2]) {
      constexpr bool FULL = decltype(full_tag)::value;
      const int lane = fresh_lane(), g = lane >> 4, r = lane & 15;
      for (int m = 0; m < NT; ++m) {
        uint4 Bm[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) Bm[kb] = sB[(m * 4 + kb) * 64 + lane];
        const float4 qf = s_hf[16 * m + r];  // rcp, -zero rcp, 2^b - 1, margin
        const uint4 qu = s_hu[16 * m + r];   // b, kb, seg, pad
        const uint32_t b = qu.x;
        f32x4_t acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int hh = 0; hh < 2; ++hh)
            acc[hh] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, A[hh][kb]),
                                                              __builtin_bit_cast(bf16x8_t, Bm[kb]), acc[hh], 0, 0, 0);
        // bound on |v - v_exact| away from the rounding boundary
        const float bnd = __fmaf_rn(-__uint_as_float(qu.w), tnmax, qf.w);
        uint32_t pc[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          uint32_t uq[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            // components without codes (b = 0, rcp = 0, qmax = 0) give v = 0
            // and code 0, so only the token tail needs masking
            const float v = __fmaf_rn(acc[hh][e], qf.x, qf.y);
            const bool in = FULL || tb0 + 4 * hh + e < nt;
            const float vc = in ? __builtin_amdgcn_fmed3f(v, 0.0f, qf.z) : 0.0f;
            const float sv = __fadd_rn(vc, 0x1p23f);  // rint(vc), nearest even, in the low bits
            uq[e] = __float_as_uint(sv);
            const float d = __fsub_rn(vc, __fsub_rn(sv, 0x1p23f));
            if constexpr (FULL) {
              fl[hh] = shift_in_flag(fl[hh], d, bnd);
            } else {
              const bool nr = in && fabsf(d) > bnd;
              fl[hh] = fl[hh] + fl[hh] + (nr ? 1u : 0u);
            }
          }
          // four codes -> one 4b-bit piece (the exponent bits cancel in kb)
          pc[hh] = uq[0] + (uq[1] << b) + (uq[2] << (2 * b)) + (uq[3] << (3 * b)) - qu.y;
        }
        // eight codes (8b bits) at bit (32 P + 8 g) b of the component's row
        const uint64_t piece = (uint64_t)pc[0] | ((uint64_t)pc[1] << (4 * b));
        const uint32_t bitoff = __umul24((uint32_t)(32 * P + 8 * g), b), sh = bitoff & 31;
        const uint32_t wi = qu.z + (bitoff >> 5);
        const uint64_t w01 = piece << sh;
        const uint32_t w2 = (uint32_t)(((piece >> 32) << sh) >> 32);
        atomicOr(&segbuf[wi], (uint32_t)w01);
        atomicOr(&segbuf[wi + 1], (uint32_t)(w01 >> 32));
        atomicOr(&segbuf[wi + 2], w2);
      }
    };
    const bool full = nt == p.tile_tokens;
    int qn = 0;  // queued codes
    for (int sub = 0; sub * 64 < nt; ++sub) {
      for (uint32_t w = fresh_lane(); w < segw + 4; w += 64) segbuf[w] = 0u;
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int P = 0; P < 2; ++P) {
        // the next pair (of this sub-tile or the next; loads past the tile
        // are clamped to its last token and never used)
        load_pair(2 * sub + P + 1, Ab[P ^ 1]);
        const uint4 (&A)[2][4] = Ab[P];
        // bound on the norms of the pair's 32 tokens: the sum over the four
        // channel quarters of the largest partial norm of each, 1% high
        float tnmax;
        {
          float n2[2] = {0.f, 0.f};
#pragma unroll
          for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
              const uint32_t w4[4] = {A[hh][kb].x, A[hh][kb].y, A[hh][kb].z, A[hh][kb].w};
#pragma unroll
              for (int z = 0; z < 4; ++z) {
                const bf16x2_t h2 = __builtin_bit_cast(bf16x2_t, w4[z]);
                n2[hh] = __builtin_amdgcn_fdot2_f32_bf16(h2, h2, n2[hh], false);
              }
            }
          // non-negative floats order as their bit patterns
          uint32_t mx = max(__float_as_uint(n2[0]), __float_as_uint(n2[1]));
#pragma unroll
          for (int o = 1; o < 16; o <<= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, o, 64));
          const float s01 = __uint_as_float(__builtin_amdgcn_readlane(mx, 0)) +
                            __uint_as_float(__builtin_amdgcn_readlane(mx, 16));
          const float s23 = __uint_as_float(__builtin_amdgcn_readlane(mx, 32)) +
                            __uint_as_float(__builtin_amdgcn_readlane(mx, 48));
          tnmax = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(1.01f * __fsqrt_rn(s01 + s23))));
        }
        const int tb0 = sub * 64 + 32 * P + 8 * g;  // tile-relative token of element (0, 0)
        uint32_t fl[2] = {0u, 0u};
        if (full) pair(std::true_type{}, A, tnmax, P, tb0, fl);
        else pair(std::false_type{}, A, tnmax, P, tb0, fl);
        const int ln = fresh_lane();
        s_flags[wave][2 * P][ln] = fl[0];
        s_flags[wave][2 * P + 1][ln] = fl[1];
      }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
      // segment buffer -> the rows of the packed tile
      for (uint32_t w = fresh_lane(); w < segw; w += 64) {
        const uint32_t k = s_wmap[w];
        const QInfo& qk = s_q[k];
        const uint32_t idx = w - qk.seg;
        const int32_t rw = (int32_t)((nt * (int)qk.b + 31) >> 5) - (int32_t)(2 * qk.b * sub);
        if ((int32_t)idx < rw) tile[s_row[wave][k] + 2 * qk.b * sub + idx] = segbuf[w];
      }
      // queue every flagged code of the sub-tile (all lanes at once, at the
      // offsets of a wave-wide scan of their counts); a full queue is worked
      // off first
      const int lane = fresh_lane(), g = lane >> 4, r = lane & 15;
      uint32_t fl[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) fl[q] = s_flags[wave][q][lane];
      for (;;) {
        const uint32_t cnt = __popc(fl[0]) + __popc(fl[1]) + __popc(fl[2]) + __popc(fl[3]);
        uint32_t incl = cnt;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const uint32_t y = (uint32_t)__shfl_up((int)incl, o, 64);
          if (lane >= o) incl += y;
        }
        const int total = (int)__builtin_amdgcn_readlane(incl, 63);
        if (total == 0) break;
        if (qn > 0 && qn + total > kQCap) {
          drain(std::integral_constant<int, 1>{}, qn);  // the next pair's loads hold registers
          qn = 0;
        }
        const int room = kQCap - qn;
        int idx = (int)(incl - cnt);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          while (fl[q] != 0u && idx < room) {
            const uint32_t bit = (uint32_t)__builtin_ctz(fl[q]);
            fl[q] &= fl[q] - 1u;
            const uint32_t m = (uint32_t)(NT - 1) - (bit >> 2), e = 3u - (bit & 3u);
            const uint32_t t = (uint32_t)(sub * 64 + 32 * (q >> 1) + 8 * g + 4 * (q & 1)) + e;
            queue[qn + idx] = (t << 16) | ((16u * m + (uint32_t)r) << 8);
            ++idx;
          }
        }
        if (total <= room) {
          qn += total;
          break;
        }
        drain(std::integral_constant<int, 1>{}, kQCap);
        qn = 0;
      }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
    }
    if (qn > 0) drain(std::integral_constant<int, 2>{}, qn);
  }
  // one count per workgroup, into the workgroup's slot
  __shared__ uint32_t s_refined;
  if (tid == 0) s_refined = 0u;
  __syncthreads();
  if (lane == 0 && refined) atomicAdd(&s_refined, refined);
  __syncthreads();
  if (tid == 0 && s_refined) atomicAdd(count_slot(p.ws, p.w), s_refined);
}

hipError_t launch_quant128(const Params& p, hipStream_t s) {
  const int32_t bmax = p.sec_bits_max;
  // segment buffer: 64 tokens of every row, 2 b words per component
  const int segw = 2 * (bmax < 8 * p.D ? bmax : 8 * p.D);
  if (segw > 2048) return hipErrorInvalidValue;
  const int segstride = (segw + 4 + 3) & ~3;
  const size_t lds = (size_t)8 * 4 * 64 * 16 + (size_t)kQWaves * segstride * 4;
  const int tiles = p.blks_per_sec * p.tiles_per_blk;
  (void)hipFuncSetAttribute((const void*)k_quant128, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  hipLaunchKernelGGL(k_quant128, dim3((tiles + kQWaves - 1) / kQWaves, p.n_sections, seq_grid(p)), dim3(64 * kQWaves), lds, s, p);
  return hipGetLastError();
}

}  // namespace kvtc
