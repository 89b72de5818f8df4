// Entropy coding ("rANS Makes the Last Mile Smaller"): per-chunk byte
// histograms and 2^sb frequency tables, interleaved rANS streams with
// `lanes` states each (one stream per packed tile, 64/lanes streams per
// wave64), the prefix sum over record sizes, container assembly, and the
// decoder with a slot lookup table in LDS.
//
// Stream format (one tile of P bytes): symbol i belongs to lane i % lanes
// and step i / lanes; states live in [2^16, 2^32) and renormalise with
// 16-bit words.  The encoder walks the steps backwards and, inside a step,
// the lanes in descending order, storing words in emission order; the
// decoder walks forward, lanes ascending, consuming words from the end.
#include <string.h>

#include <type_traits>

#include "kvtc_internal.h"

namespace kvtc {

struct alignas(16) EncSym {  // one 16-byte LDS read per lookup
  uint32_t f;
  uint32_t cum;
  double rcp;     // 1/f rounded to fp64; quotient = trunc(fma(x, rcp, 2^-20))
};

// Raw buffer resource over [base, base + bytes) with wave-uniform fields, so
// the compiler keeps it in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(void* base, int32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a), hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* b = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(b, 0, __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// ---- frequency table ------------------------------------------------------

// Lane-local best of (value desc, symbol asc) across the wave.
__device__ __forceinline__ void wave_argmax(uint64_t& v, int& s) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint64_t ov = __shfl_xor(v, o, 64);
    int os = __shfl_xor(s, o, 64);
    if (ov > v || (ov == v && os < s)) { v = ov; s = os; }
  }
}

__device__ __forceinline__ uint64_t wave_sum64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Counts -> frequencies summing to M = 2^sb (one wave; lane holds symbols
// 4*lane .. 4*lane+3).  Each present symbol gets max(1, round(n M / N)); a
// shortfall goes to the most frequent symbol, an excess is taken one unit at
// a time from the largest frequency (lowest symbol on ties).  The excess loop
// is evaluated in closed form: every frequency above a level tau is lowered
// to tau, then the r lowest symbols at tau lose one more unit.
__device__ void wave_freq_normalize(const uint32_t* counts, int sb, uint32_t* freq) {
  const int lane = threadIdx.x & 63;
  const uint64_t M = 1ull << sb;
  uint32_t n[4];
  uint64_t f[4];
  uint64_t N = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) { n[k] = counts[4 * lane + k]; N += n[k]; }
  N = wave_sum64(N);
  if (N == 0) {
#pragma unroll
    for (int k = 0; k < 4; ++k) freq[4 * lane + k] = 0;
    return;
  }
  uint64_t local = 0;
  // floor((n 2M + N) / 2N): the quotient from one fp64 reciprocal of the
  // common divisor (numerator < 2^53, so exact in fp64), off by at most one
  // and corrected in integers
  const uint64_t div = 2 * N;
  const double inv = 1.0 / (double)div;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    if (n[k] == 0) f[k] = 0;
    else {
      const uint64_t a = (uint64_t)n[k] * (2 * M) + N;
      uint64_t r = (uint64_t)((double)a * inv);
      if (r * div > a) --r;
      else if ((r + 1) * div <= a) ++r;
      f[k] = r < 1 ? 1 : r;
    }
    local += f[k];
  }
  const int64_t d = (int64_t)M - (int64_t)wave_sum64(local);
  if (d > 0) {
    uint64_t bv = 0;
    int bs = 1 << 30;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if ((uint64_t)n[k] > bv || ((uint64_t)n[k] == bv && 4 * lane + k < bs)) { bv = n[k]; bs = 4 * lane + k; }
    wave_argmax(bv, bs);
#pragma unroll
    for (int k = 0; k < 4; ++k) if (4 * lane + k == bs) f[k] += (uint64_t)d;
  } else if (d < 0) {
    const uint64_t R = (uint64_t)(-d);
    // smallest tau >= 1 with E(tau) = sum max(0, f - tau) <= R
    // (f <= 2^13, so E <= 2^21 sums in 32 bits)
    uint32_t lo = 1, hi = (uint32_t)M;  // E(M) = 0 <= R
    while (lo < hi) {
      const uint32_t mid = (lo + hi) >> 1;
      uint32_t e = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) e += (uint32_t)f[k] > mid ? (uint32_t)f[k] - mid : 0u;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) e += (uint32_t)__shfl_xor((int)e, o, 64);
      if (e <= R) hi = mid; else lo = mid + 1;
    }
    const uint64_t tau = lo;
    uint64_t e = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) e += f[k] > tau ? f[k] - tau : 0;
    e = wave_sum64(e);
    uint64_t rem = R - e;
    // symbols at level tau after lowering, in ascending symbol order
    uint32_t at[4], cnt = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) { at[k] = f[k] >= tau ? 1u : 0u; cnt += at[k]; }
    uint32_t x = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      uint32_t y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    uint32_t before = x - cnt;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (f[k] > tau) f[k] = tau;
      if (at[k]) {
        if (before < rem) f[k] -= 1;
        before += 1;
      }
    }
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) freq[4 * lane + k] = (uint32_t)f[k];
}

// Build the encoder table (wave 0 computes, the block shares it).
__device__ void build_enc_table(const uint32_t* freq, EncSym* tab) {
  const int lane = threadIdx.x & 63;
  uint32_t f[4], s = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) { f[k] = freq[4 * lane + k]; s += f[k]; }
  uint32_t x = s;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  uint32_t cum = x - s;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    EncSym e;
    e.f = f[k];
    e.cum = cum;
    e.rcp = f[k] ? __ddiv_rn(1.0, (double)f[k]) : 0.0;
    tab[4 * lane + k] = e;
    cum += f[k];
  }
}

// ---- stream coder ---------------------------------------------------------

// Encode one stream per `lanes`-lane group of the wave.  sym: the tile's
// bytes (any address space); words: output (emission order).  Returns the
// word count (uniform within the group) or -1 when the capacity is exceeded.
__device__ __forceinline__ int64_t rans_encode_stream(const uint8_t* sbase, int32_t sbytes, int32_t soff, int32_t Nt,
                                                      bool valid, int steps_max, const EncSym* tab, int sb, int lanes,
                                                      uint8_t* wbase, int32_t wbytes, int32_t woff, int32_t wcap,
                                                      uint32_t* state_out) {
  // Symbols come from sbase + soff + i and words go to wbase + woff + 2 at,
  // both through buffer resources whose range check turns the accesses of
  // lanes without work into no-ops, so every step issues exactly one load
  // and one store (the waits for the prefetched symbols then never cover an
  // unknown number of stores).  The symbol of step k is loaded PF steps
  // ahead into slot k % PF of a register ring that is consumed in place.
  const __amdgpu_buffer_rsrc_t srsrc = uniform_rsrc(const_cast<uint8_t*>(sbase), sbytes);
  const __amdgpu_buffer_rsrc_t wrsrc = uniform_rsrc(wbase, wbytes);
  const int lane = threadIdx.x & 63;
  const int j = lane % lanes, grp = lane / lanes;
  // this group's lanes as halves of the 64-bit lane mask
  const uint64_t gm = ((lanes == 64) ? ~0ull : ((1ull << lanes) - 1ull)) << (grp * lanes);
  const uint32_t gm_lo = (uint32_t)gm, gm_hi = (uint32_t)(gm >> 32);
  const uint32_t M = 1u << sb;
  uint32_t x = kRansL;
  int32_t nw = 0;
  constexpr int PF = 8;
  auto fetch = [&](int k) -> uint32_t {
    const int32_t i = k * lanes + j;
    return __builtin_amdgcn_raw_buffer_load_b8(srsrc, (valid && k >= 0 && i < Nt) ? soff + i : sbytes, 0, 0);
  };
  // the same for a step below kfull (every lane of a present tile has a symbol)
  auto fetch_full = [&](int k) -> uint32_t {
    return __builtin_amdgcn_raw_buffer_load_b8(srsrc, (valid && k >= 0) ? soff + k * lanes + j : sbytes, 0, 0);
  };
  // Steps are padded up to a multiple of PF (the padding steps hold no
  // symbol for any lane) so that the unrolled body has no branch: a branch
  // would make the ring registers merge across it and wait on their loads.
  const int kt = (__builtin_amdgcn_readfirstlane(steps_max) + PF - 1) / PF * PF;
  uint32_t ring[PF];
#pragma unroll
  for (int d = 0; d < PF; ++d) ring[d] = fetch(kt - 1 - d);
  // the table entry of the next step is read a step ahead (ring slot d + 1
  // holds the next step's symbol, slot 0 the next block's after its refill)
  // table entries as one 16-byte LDS read (its offset field takes the table's base)
  auto entry = [&](uint32_t sym) -> EncSym {
    const uint4 q = reinterpret_cast<const uint4*>(tab)[sym];
    EncSym e;
    e.f = q.x;
    e.cum = q.y;
    e.rcp = __hiloint2double((int)q.w, (int)q.z);
    return e;
  };
  EncSym en = entry(ring[0]);
  // Blocks of PF steps from the last step down.  Steps below kfull have a
  // symbol for every lane of a present tile, so their blocks skip the
  // per-lane step masks (lanes of an absent tile never emit, and their state
  // is not stored).
  int kfull = valid ? Nt / lanes : kt;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) kfull = min(kfull, __shfl_xor(kfull, o, 64));
  kfull = __builtin_amdgcn_readfirstlane(kfull);
  auto block = [&](auto masked_tag, int k0) {
    constexpr bool MASKED = decltype(masked_tag)::value;
#pragma unroll
    for (int d = 0; d < PF; ++d) {
      const int k = k0 - d;
      {
        const int32_t i = k * lanes + j;
        const bool active = MASKED ? (valid && i < Nt) : valid;
        const EncSym e = en;
        // refill after the last use so the load can reuse the same register
        ring[d] = MASKED ? fetch(k - PF) : fetch_full(k - PF);
        en = entry(ring[(d + 1) % PF]);
        // renormalise while x >= f 2^(32 - sb): one 16-bit word at most
        const bool emit = active && (x >> (32 - sb)) >= e.f;
        const uint64_t bl = __ballot(emit);
        const uint32_t mlo = (uint32_t)bl & gm_lo, mhi = (uint32_t)(bl >> 32) & gm_hi;
        const int32_t cnt = (int32_t)(__popc(mlo) + __popc(mhi));
        // words are written in emission order, higher lanes first
        const int32_t below = (int32_t)__builtin_amdgcn_mbcnt_hi(mhi, __builtin_amdgcn_mbcnt_lo(mlo, 0u));
        const int32_t at = nw + cnt - 1 - below;
        const bool fits = at < wcap;
        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(x & 0xffffu), wrsrc, (emit && fits) ? woff + 2 * at : wbytes, 0, 0);
        if (emit) x >>= 16;
        nw += cnt;
        // x = floor(x / f) * M + (x mod f) + cum, via an exact fp64 quotient
        const uint32_t q = (uint32_t)__fma_rn((double)x, e.rcp, 0x1p-20);
        // q < 2^(32 - sb) <= 2^24 and M - f < 2^12: a 24-bit product
        const uint32_t xn = x + e.cum + __umul24(q, M - e.f);
        x = MASKED ? (active ? xn : x) : xn;
        // keep the steps in order so that each ring register is refilled in place
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  int k0 = kt - 1;
  for (; k0 >= 0 && k0 >= kfull; k0 -= PF) block(std::true_type{}, k0);
  for (; k0 >= 0; k0 -= PF) block(std::false_type{}, k0);
  if (valid) state_out[j] = x;
  // every word of the group went below its final count nw, so one went past
  // the capacity exactly when nw exceeds it (those stores were dropped)
  return nw > wcap ? -1 : nw;
}

// Decoder tables from the cumulative frequencies (cum[256] = 2^sb): the
// symbol of every slot (one byte each) and, per symbol, f | cum << 16.  Every
// present symbol marks the first slot of its range; since symbols ascend
// with their ranges, the symbol of a slot is the running maximum of the marks
// up to it.  Each thread takes a run of whole words, and the maxima of the
// earlier runs come from a block scan, so no step depends on the data.
// Called by every thread of the block (it synchronises the block).
__device__ __forceinline__ void build_dec_tables(const uint32_t* cum, int sb, uint8_t* sym_of, uint32_t* fc) {
  const int tid = threadIdx.x, nt = blockDim.x, lane = tid & 63, wave = tid >> 6;
  for (int s = tid; s < 256; s += nt) fc[s] = (cum[s + 1] - cum[s]) | (cum[s] << 16);
  const int nw = (1 << sb) >> 2;  // words of the slot table
  uint32_t* w = reinterpret_cast<uint32_t*>(sym_of);
  for (int i = tid; i < nw; i += nt) w[i] = 0u;
  __syncthreads();
  for (int s = tid; s < 256; s += nt)
    if (cum[s + 1] > cum[s]) sym_of[cum[s]] = (uint8_t)s;
  __syncthreads();
  const int per = (nw + nt - 1) / nt;
  const int w0 = min(nw, tid * per), w1 = min(nw, w0 + per);
  uint32_t m = 0;
  for (int i = w0; i < w1; ++i) {
    const uint32_t v = w[i];
    m = max(m, max(max(v & 0xffu, (v >> 8) & 0xffu), max((v >> 16) & 0xffu, v >> 24)));
  }
  // the maximum over the runs before this thread's
  uint32_t inc = m;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(inc, o, 64);
    if (lane >= o) inc = max(inc, y);
  }
  __shared__ uint32_t s_wmax[16];
  if (lane == 63) s_wmax[wave] = inc;
  __syncthreads();
  uint32_t run = __shfl_up(inc, 1, 64);
  if (lane == 0) run = 0u;
  for (int v2 = 0; v2 < wave; ++v2) run = max(run, s_wmax[v2]);
  for (int i = w0; i < w1; ++i) {
    const uint32_t v = w[i];
    uint32_t o4 = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      run = max(run, (v >> (8 * b)) & 0xffu);
      o4 |= run << (8 * b);
    }
    w[i] = o4;
  }
}

constexpr int kRing = 512;  // words of a stream's LDS ring
constexpr int kUnit = 256;  // words per refill

// Decode one interleaved stream: this lane runs state j = lane % LANES of
// its group of LANES lanes; symbol i belongs to state i % LANES.  The stream's
// 16-bit words (global memory, 4-byte aligned) are consumed from the end; a
// ring of kRing words in LDS holds the next ones, refilled kUnit words at a
// time from registers loaded one refill ahead, so no step waits on global
// memory.  Returns false (for any lane) if the stream is not one the encoder
// can have written.
template <int LANES>
__device__ __forceinline__ bool rans_decode_ring(const uint32_t* states, const uint16_t* words, int32_t nw,
                                                 int32_t Nt, bool valid, int steps_max, const uint8_t* sym_of,
                                                 const uint32_t* fc, int sb, uint16_t* ring, uint8_t* obase,
                                                 int32_t out_off, int32_t out_end) {
  const __amdgpu_buffer_rsrc_t orsrc = uniform_rsrc(obase, out_end);
  const int lane = threadIdx.x & 63;
  const int j = lane % LANES, grp = lane / LANES;
  // this group's lanes as halves of the 64-bit lane mask
  const uint64_t gm = (LANES == 64 ? ~0ull : ((1ull << LANES) - 1ull)) << (grp * LANES);
  const uint32_t gm_lo = (uint32_t)gm, gm_hi = (uint32_t)(gm >> 32);
  const uint32_t mask = (1u << sb) - 1u;
  const uint32_t* wd = reinterpret_cast<const uint32_t*>(words);  // word pairs
  uint32_t* ring32 = reinterpret_cast<uint32_t*>(ring);
  uint32_t x = valid ? states[j] : kRansL;
  const bool bad0 = valid && x < kRansL;
  int32_t ptr = nw;
  // committed words [clo, nw) (clo a multiple of 8), pending words [plo, clo)
  int32_t clo = max(0, (nw - kRing + 7) & ~7);
  if (valid) {
    for (int32_t q = clo / 2 + j; 2 * q < nw; q += LANES)
      ring32[q & (kRing / 2 - 1)] = (2 * q + 1 < nw) ? wd[q] : (uint32_t)words[2 * q];
  }
  int32_t plo = max(0, clo - kUnit);
  constexpr int PER = kUnit / 2 / LANES;
  uint32_t pend[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int32_t q = plo / 2 + j + LANES * k;
    pend[k] = (valid && q < clo / 2) ? wd[q] : 0u;
  }
  __builtin_amdgcn_wave_barrier();
  // Every step is branch-free apart from the (group-uniform) refill: a
  // corrupt stream may read wrong ring words, which the final state and
  // word-count checks then reject.
  //
  // Main phase: steps at which every valid lane of the wave decodes a
  // symbol (no per-lane masks; lanes of an absent tile compute values that
  // are never used and store past the output's range, where the stores are
  // dropped).  The refill test runs once per four steps: a group takes at
  // most LANES words a step, so the ring cannot run short between tests.
  int kfull = valid ? Nt / LANES : steps_max;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) kfull = min(kfull, __shfl_xor(kfull, o, 64));
  kfull = __builtin_amdgcn_readfirstlane(min(kfull, steps_max));
  const int steps_u = __builtin_amdgcn_readfirstlane(steps_max);
  int32_t voff = valid ? out_off + j : out_end;
  int k = 0;
  for (; k + 4 <= kfull; k += 4) {
    if (valid && clo > 0 && ptr - clo <= kUnit) {
#pragma unroll
      for (int q2 = 0; q2 < PER; ++q2) {
        const int32_t q = plo / 2 + j + LANES * q2;
        if (q < clo / 2) ring32[q & (kRing / 2 - 1)] = pend[q2];
      }
      clo = plo;
      plo = max(0, clo - kUnit);
#pragma unroll
      for (int q2 = 0; q2 < PER; ++q2) {
        const int32_t q = plo / 2 + j + LANES * q2;
        pend[q2] = q < clo / 2 ? wd[q] : 0u;
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t slot = x & mask;
      const uint32_t sym = sym_of[slot];
      const uint32_t e = fc[sym];
      x = __umul24(e & 0xffffu, x >> sb) + slot - (e >> 16);
      __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sym, orsrc, voff, 0, 0);
      voff += LANES;
      const bool need = x < kRansL;
      const uint64_t bl = __ballot(need);
      const uint32_t mlo = (uint32_t)bl & gm_lo, mhi = (uint32_t)(bl >> 32) & gm_hi;
      const uint32_t rank = __builtin_amdgcn_mbcnt_hi(mhi, __builtin_amdgcn_mbcnt_lo(mlo, 0u));
      const uint32_t w = ring[(uint32_t)(ptr - 1 - (int32_t)rank) & (kRing - 1)];
      x = need ? ((x << 16) | w) : x;
      ptr -= (int32_t)(__popc(mlo) + __popc(mhi));
    }
  }
  // the remaining steps, masked per lane
  for (; k < steps_u; ++k) {
    if (valid && clo > 0 && ptr - clo <= kUnit) {
      // the ring slots of [plo, clo) held words >= clo + kUnit >= ptr: consumed
#pragma unroll
      for (int q2 = 0; q2 < PER; ++q2) {
        const int32_t q = plo / 2 + j + LANES * q2;
        if (q < clo / 2) ring32[q & (kRing / 2 - 1)] = pend[q2];
      }
      clo = plo;
      plo = max(0, clo - kUnit);
#pragma unroll
      for (int q2 = 0; q2 < PER; ++q2) {
        const int32_t q = plo / 2 + j + LANES * q2;
        pend[q2] = q < clo / 2 ? wd[q] : 0u;
      }
    }
    const int32_t i = k * LANES + j;
    const bool active = valid && i < Nt;
    const uint32_t slot = x & mask;
    const uint32_t sym = sym_of[slot];
    const uint32_t e = fc[sym];
    const uint32_t xn = __umul24(e & 0xffffu, x >> sb) + slot - (e >> 16);
    x = active ? xn : x;
    // lanes past the stream store out of the resource's range (dropped)
    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)sym, orsrc, active ? out_off + i : out_end, 0, 0);
    const bool need = active && x < kRansL;
    const uint64_t bl = __ballot(need);
    const uint32_t mlo = (uint32_t)bl & gm_lo, mhi = (uint32_t)(bl >> 32) & gm_hi;
    const uint32_t rank = __builtin_amdgcn_mbcnt_hi(mhi, __builtin_amdgcn_mbcnt_lo(mlo, 0u));
    const uint32_t w = ring[(uint32_t)(ptr - 1 - (int32_t)rank) & (kRing - 1)];
    x = need ? ((x << 16) | w) : x;
    ptr -= (int32_t)(__popc(mlo) + __popc(mhi));
  }
  return !(bad0 || (valid && (x != kRansL || ptr != 0)));
}

// ---- per-chunk encoder ------------------------------------------------------

// record slot of chunk c: [freq u16 x256][nwords u32 x tiles][tile t: states, words]
__device__ __forceinline__ int64_t slot_states_off(const Params& p, int t) {
  // 16-byte aligned: 4 lanes and 2 tile_words_max + 4 are multiples of 16
  return ((512 + 4 * (int64_t)p.tiles_per_chunk + 15) & ~(int64_t)15) +
         (int64_t)t * (4 * p.lanes + 2 * p.w.tile_words_max + 4);
}

// raw_runs > 0 (contiguous cache): workgroups past the chunks copy the raw
// sink and recent runs into the container, on the bandwidth this
// latency-bound pass leaves idle.
__global__ void k_rans_enc_chunks(const Params p0, int raw_runs) {
  const Params p = at_seq(p0, blockIdx.z);
  const int c = blockIdx.x;
  if (c >= p.n_chunks) {
    if (c - p.n_chunks < raw_runs) copy_raw_run(p, c - p.n_chunks, 1, false);
    return;
  }
  const int u = c / p.chunks_per_sec, ch = c % p.chunks_per_sec;
  const int D = p.D;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (get_status(p.ws, p.w) & (1u << KVTC_ERR_NONFINITE)) return;
  __shared__ uint32_t hist[256];
  __shared__ uint32_t freq[256];
  __shared__ EncSym tab[256];
  __shared__ uint8_t bits[256];
  __shared__ int64_t s_P[2];
  for (int i = threadIdx.x; i < D; i += blockDim.x) bits[i] = p.ws[p.w.side_bits + (int64_t)u * D + i];
  __syncthreads();
  const int n = min(p.chunk_tokens, p.T_mid - ch * p.chunk_tokens);
  const int ntiles = (n + p.tile_tokens - 1) / p.tile_tokens;
  const int n_last = n - (ntiles - 1) * p.tile_tokens;
  if (wave == 0) {  // packed bytes of a full and of the last tile
    int64_t pf = 0, pl = 0;
    for (int i = lane; i < D; i += 64) {
      pf += 4 * (int64_t)((p.tile_tokens * (int)bits[i] + 31) >> 5);
      pl += 4 * (int64_t)((n_last * (int)bits[i] + 31) >> 5);
    }
    pf = (int64_t)wave_sum64((uint64_t)pf);
    pl = (int64_t)wave_sum64((uint64_t)pl);
    if (lane == 0) { s_P[0] = pf; s_P[1] = pl; }
  }
  __syncthreads();
  const int64_t P_full = s_P[0], P_last = s_P[1];
  const int64_t P = (ntiles - 1) * P_full + P_last;
  uint32_t* rec_size = reinterpret_cast<uint32_t*>(p.ws + p.w.rec_size);
  if (P == 0) {
    if (threadIdx.x == 0) rec_size[c] = 0;
    return;
  }
  const uint8_t* packed = p.ws + p.w.packed + (int64_t)c * p.w.packed_slot;
  // histogram of the chunk's bytes (P is a multiple of 4), in eight
  // interleaved copies (bin b of copy c at 8 b + c, lane l counts into copy
  // l % 8) so that lanes hitting a popular byte value spread over banks
  __shared__ uint32_t hist8[256 * 8];
  for (int i = threadIdx.x; i < 256 * 8; i += blockDim.x) hist8[i] = 0;
  __syncthreads();
  {
    // 16-byte loads, eight in flight per thread before their bytes are
    // counted (the slot is 16-byte aligned; a tail of 4-byte words follows)
    const uint32_t cpy = lane & 7;
    auto count = [&](uint32_t wv) {
      atomicAdd(&hist8[8 * (wv & 0xff) + cpy], 1u);
      atomicAdd(&hist8[8 * ((wv >> 8) & 0xff) + cpy], 1u);
      atomicAdd(&hist8[8 * ((wv >> 16) & 0xff) + cpy], 1u);
      atomicAdd(&hist8[8 * (wv >> 24) + cpy], 1u);
    };
    const int64_t n16 = P / 16;
    const uint4* p16 = reinterpret_cast<const uint4*>(packed);
    for (int64_t i0 = 0; i0 < n16; i0 += 8 * (int64_t)blockDim.x) {
      uint4 v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int64_t i = i0 + k * (int64_t)blockDim.x + threadIdx.x;
        v[k] = i < n16 ? p16[i] : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (i0 + k * (int64_t)blockDim.x + threadIdx.x < n16) {
          count(v[k].x);
          count(v[k].y);
          count(v[k].z);
          count(v[k].w);
        }
      }
    }
    for (int64_t i = 4 * n16 + threadIdx.x; i < P / 4; i += blockDim.x)
      count(reinterpret_cast<const uint32_t*>(packed)[i]);
  }
  __syncthreads();
  for (int b = threadIdx.x; b < 256; b += blockDim.x) {
    uint32_t sum = 0;
#pragma unroll
    for (int c2 = 0; c2 < 8; ++c2) sum += hist8[8 * b + c2];
    hist[b] = sum;
  }
  __syncthreads();
  if (wave == 0) {
    wave_freq_normalize(hist, p.sb, freq);
    __builtin_amdgcn_wave_barrier();
    build_enc_table(freq, tab);
  }
  __syncthreads();
  uint8_t* slot = p.ws + p.w.rec + (int64_t)c * p.w.rec_slot;
  for (int i = threadIdx.x; i < 256; i += blockDim.x) reinterpret_cast<uint16_t*>(slot)[i] = (uint16_t)freq[i];
  // streams: 64/lanes per wave
  const int spw = 64 / p.lanes;
  const int t = wave * spw + lane / p.lanes;
  const bool valid = t < ntiles;
  const int64_t Nt = valid ? (t == ntiles - 1 ? P_last : P_full) : 0;
  const int steps = (int)((Nt + p.lanes - 1) / p.lanes);
  int steps_max = steps;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) steps_max = max(steps_max, __shfl_xor(steps_max, o, 64));
  const int tt = valid ? t : 0;
  uint32_t* states = reinterpret_cast<uint32_t*>(slot + slot_states_off(p, tt));
  const int64_t nw = rans_encode_stream(packed, (int32_t)P, (int32_t)(tt * P_full), (int32_t)Nt, valid, steps_max, tab,
                                        p.sb, p.lanes, slot, (int32_t)p.w.rec_slot,
                                        (int32_t)(slot_states_off(p, tt) + 4 * p.lanes), p.w.tile_words_max, states);
  __shared__ int32_t s_nw[64];
  if (valid && (lane % p.lanes) == 0) {
    s_nw[t] = (int32_t)nw;
    reinterpret_cast<uint32_t*>(slot + 512)[t] = (uint32_t)(nw < 0 ? 0 : nw);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int64_t size = 512 + 4 * (int64_t)ntiles;
    bool over = false;
    for (int k = 0; k < ntiles; ++k) {
      if (s_nw[k] < 0) over = true;
      int64_t w = s_nw[k] < 0 ? 0 : s_nw[k];
      size += 4 * (int64_t)p.lanes + 2 * w + ((w & 1) ? 2 : 0);
    }
    if (over) set_status(p.ws, p.w, KVTC_ERR_CAPACITY);
    rec_size[c] = (uint32_t)align16(size);
  }
}

hipError_t launch_rans_encode_chunks(const Params& p, hipStream_t s, bool with_raw) {
  int streams = p.tiles_per_chunk;
  int waves = (streams * p.lanes + 63) / 64;
  if (waves < 1) waves = 1;
  const int raw_runs = with_raw && p.n_seqs == 0 ? 4 * p.L * p.H : 0;
  hipLaunchKernelGGL(k_rans_enc_chunks, dim3(p.n_chunks + raw_runs, 1, seq_grid(p)), dim3(64 * waves), 0, s, p, raw_runs);
  return hipGetLastError();
}

// ---- prefix sum, directory, header and record copy -------------------------

struct HeaderBytes {
  uint8_t b[kHeaderBytes];
};

// Header word i: the plan's template with the fields that depend on T taken
// from this call's (or this sequence's) layout.
__device__ inline uint32_t header_word(const Params& p, const HeaderBytes& hdr, int i) {
  auto lo32 = [](int64_t v) { return (uint32_t)v; };
  auto hi32 = [](int64_t v) { return (uint32_t)((uint64_t)v >> 32); };
  switch (i) {
    case 24: return (uint32_t)p.T;
    case 25: return (uint32_t)p.s0;
    case 26: return (uint32_t)p.mid_begin;
    case 27: return (uint32_t)p.mid_end;
    case 29: return (uint32_t)p.chunks_per_sec;
    case 30: return lo32(p.side_off);
    case 31: return hi32(p.side_off);
    case 32: return lo32(p.raw_off - p.side_off);
    case 33: return hi32(p.raw_off - p.side_off);
    case 34: return lo32(p.raw_off);
    case 35: return hi32(p.raw_off);
    case 36: return lo32(p.raw_bytes);
    case 37: return hi32(p.raw_bytes);
    case 38: return lo32(p.dir_off);
    case 39: return hi32(p.dir_off);
    case 40: return lo32(p.chunks_off);
    case 41: return hi32(p.chunks_off);
    default:
      return (uint32_t)hdr.b[4 * i] | ((uint32_t)hdr.b[4 * i + 1] << 8) | ((uint32_t)hdr.b[4 * i + 2] << 16) |
             ((uint32_t)hdr.b[4 * i + 3] << 24);
  }
}

__global__ __launch_bounds__(1024) void k_scan(const Params p0, HeaderBytes hdr) {
  const Params p = at_seq(p0, blockIdx.z);
  __shared__ uint64_t s_part[1024];
  const uint32_t* rec_size = reinterpret_cast<const uint32_t*>(p.ws + p.w.rec_size);
  uint64_t* rec_pos = reinterpret_cast<uint64_t*>(p.ws + p.w.rec_pos);
  const int64_t n = p.n_chunks;
  const int tid = threadIdx.x;
  const int64_t per = (n + 1023) / 1024;
  const int64_t a = tid * per, b = min(n, a + per);
  uint64_t local = 0;
  for (int64_t i = a; i < b; ++i) local += rec_size[i];
  // inclusive scan: within each wave by shuffles, then over the 16 wave totals
  const int lane = tid & 63, wave = tid >> 6;
  uint64_t incl = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint64_t v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  __shared__ uint64_t s_wave[16];
  if (lane == 63) s_wave[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    uint64_t w = lane < 16 ? s_wave[lane] : 0;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const uint64_t v = __shfl_up(w, o, 64);
      if (lane >= o) w += v;
    }
    if (lane < 16) s_wave[lane] = w;  // inclusive wave totals
  }
  __syncthreads();
  incl += wave > 0 ? s_wave[wave - 1] : 0;
  s_part[tid] = incl;
  uint64_t run = incl - local;
  for (int64_t i = a; i < b; ++i) {
    rec_pos[i] = run;
    uint8_t* d = p.out + p.dir_off + i * kDirEntry;
    uint64_t off = (uint64_t)p.chunks_off + run;
    *reinterpret_cast<uint64_t*>(d) = off;
    *reinterpret_cast<uint32_t*>(d + 8) = rec_size[i];
    *reinterpret_cast<uint32_t*>(d + 12) = 0;
    run += rec_size[i];
  }
  __syncthreads();
  const uint64_t total = (uint64_t)p.chunks_off + s_part[1023];
  if (tid < kHeaderBytes / 4) {
    uint32_t wv = header_word(p, hdr, tid);
    if (tid == 42) wv = (uint32_t)total;
    if (tid == 43) wv = (uint32_t)(total >> 32);
    reinterpret_cast<uint32_t*>(p.out)[tid] = wv;
  }
  if (tid == 0) {
    uint64_t* st = reinterpret_cast<uint64_t*>(p.ws + p.w.status);
    if (total > (uint64_t)p.cap) {
      set_status(p.ws, p.w, KVTC_ERR_CAPACITY);
      st[1] = 0;
    } else {
      st[1] = (get_status(p.ws, p.w) & ((1u << KVTC_ERR_NONFINITE) | (1u << KVTC_ERR_CAPACITY))) ? 0 : total;
    }
  }
}

// scan = 1 (a contiguous call with chunks): each workgroup sums the sizes of
// the records before its own (at most a few KB, cached) instead of reading
// k_scan's offsets, writes its directory entry, and the last one writes the
// header, the container size and the status word, as k_scan does.
__global__ __launch_bounds__(256) void k_copy_records(const Params p0, HeaderBytes hdr, int scan) {
  const Params p = at_seq(p0, blockIdx.z);
  const int c = blockIdx.x;
  if (c >= p.n_chunks) return;
  const uint32_t* rec_size = reinterpret_cast<const uint32_t*>(p.ws + p.w.rec_size);
  const uint32_t size = rec_size[c];
  uint64_t pos;
  if (scan) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    uint64_t part = 0;
    for (int i = tid; i < c; i += 256) part += rec_size[i];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) part += __shfl_xor(part, o, 64);
    __shared__ uint64_t s_part[4];
    if (lane == 0) s_part[wave] = part;
    __syncthreads();
    pos = (s_part[0] + s_part[1]) + (s_part[2] + s_part[3]);
    if (tid == 0) {
      reinterpret_cast<uint64_t*>(p.ws + p.w.rec_pos)[c] = pos;
      uint8_t* d = p.out + p.dir_off + (int64_t)c * kDirEntry;
      *reinterpret_cast<uint64_t*>(d) = (uint64_t)p.chunks_off + pos;
      *reinterpret_cast<uint32_t*>(d + 8) = size;
      *reinterpret_cast<uint32_t*>(d + 12) = 0;
    }
    if (c == p.n_chunks - 1) {
      const uint64_t total = (uint64_t)p.chunks_off + pos + size;
      if (tid < kHeaderBytes / 4) {
        uint32_t wv = header_word(p, hdr, tid);
        if (tid == 42) wv = (uint32_t)total;
        if (tid == 43) wv = (uint32_t)(total >> 32);
        reinterpret_cast<uint32_t*>(p.out)[tid] = wv;
      }
      if (tid == 0) {
        uint64_t* st = reinterpret_cast<uint64_t*>(p.ws + p.w.status);
        if (total > (uint64_t)p.cap) {
          set_status(p.ws, p.w, KVTC_ERR_CAPACITY);
          st[1] = 0;
        } else {
          st[1] = (get_status(p.ws, p.w) & ((1u << KVTC_ERR_NONFINITE) | (1u << KVTC_ERR_CAPACITY))) ? 0 : total;
        }
      }
    }
    // a record that does not fit is not copied (the last workgroup reports
    // the capacity error)
    if ((uint64_t)p.chunks_off + pos + size > (uint64_t)p.cap) return;
  } else {
    pos = reinterpret_cast<const uint64_t*>(p.ws + p.w.rec_pos)[c];
  }
  if (get_status(p.ws, p.w) & ((1u << KVTC_ERR_CAPACITY) | (1u << KVTC_ERR_NONFINITE))) return;
  if (size == 0) return;
  const uint8_t* slot = p.ws + p.w.rec + (int64_t)c * p.w.rec_slot;
  uint8_t* dst = p.out_final + p.chunks_off + pos;  // 16-byte aligned record
  const int ch = c % p.chunks_per_sec;
  const int n = min(p.chunk_tokens, p.T_mid - ch * p.chunk_tokens);
  const int ntiles = (n + p.tile_tokens - 1) / p.tile_tokens;
  const uint32_t* nwv = reinterpret_cast<const uint32_t*>(slot + 512);
  const int tid = threadIdx.x;
  // dword copy of n_dw dwords; the last one keeps only its low half when
  // `half_last` (an odd word count padded with zeros)
  auto copy_dw = [&](const uint32_t* src, uint32_t* d, int n_dw, bool half_last) {
    for (int i0 = 0; i0 < n_dw; i0 += 4 * 256) {
      uint32_t v[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int i = i0 + k * 256 + tid;
        v[k] = i < n_dw ? src[i] : 0u;
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int i = i0 + k * 256 + tid;
        if (i < n_dw) d[i] = (half_last && i == n_dw - 1) ? (v[k] & 0xffffu) : v[k];
      }
    }
  };
  // table and word counts
  copy_dw(reinterpret_cast<const uint32_t*>(slot), reinterpret_cast<uint32_t*>(dst), 128 + ntiles, false);
  int64_t at = 512 + 4 * (int64_t)ntiles;
  for (int t = 0; t < ntiles; ++t) {
    const uint32_t nw = nwv[t];
    const int n_dw = p.lanes + (int)((nw + 1) >> 1);  // states, words, zero pad to 4 bytes
    copy_dw(reinterpret_cast<const uint32_t*>(slot + slot_states_off(p, t)), reinterpret_cast<uint32_t*>(dst + at),
            n_dw, (nw & 1) != 0);
    at += 4 * (int64_t)n_dw;
  }
  for (int64_t i = at + tid; i < size; i += 256) dst[i] = 0;
}

hipError_t launch_assemble(const Params& p, const uint8_t* hdr, hipStream_t s) {
  HeaderBytes h;
  memcpy(h.b, hdr, kHeaderBytes);
  if (p.n_seqs == 0 && p.n_chunks > 0) {
    // one launch: offsets, directory, header and records
    hipLaunchKernelGGL(k_copy_records, dim3(p.n_chunks), dim3(256), 0, s, p, h, 1);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_scan, dim3(1, 1, seq_grid(p)), dim3(1024), 0, s, p, h);
  if (p.n_seqs > 0) {
    // place the sequences, then move each one's staged fixed part and records
    const hipError_t e = launch_batch_place(p, s);
    if (e != hipSuccess) return e;
  }
  if (p.n_chunks > 0) hipLaunchKernelGGL(k_copy_records, dim3(p.n_chunks, 1, seq_grid(p)), dim3(256), 0, s, p, h, 0);
  return hipGetLastError();
}

// ---- decoder ----------------------------------------------------------------

__global__ void k_dec_check(const Params p0, HeaderBytes hdr) {
  const Params p = at_seq(p0, blockIdx.z);
  const int tid = threadIdx.x;
  __shared__ int s_bad;
  if (tid == 0) s_bad = 0;
  __syncthreads();
  if (p.cap < p.chunks_off || p.cap < kHeaderBytes) {
    if (tid == 0) s_bad = 1;
  } else if (tid < kHeaderBytes / 4 && tid != 42 && tid != 43) {
    const uint32_t want = header_word(p, hdr, tid);
    if (reinterpret_cast<const uint32_t*>(p.in)[tid] != want) atomicOr(&s_bad, 1);
  }
  __syncthreads();
  if (tid == 0) {
    uint32_t* st = reinterpret_cast<uint32_t*>(p.ws + p.w.status);
    uint32_t code = 0;
    if (!s_bad) {
      uint64_t total = *reinterpret_cast<const uint64_t*>(p.in + 168);
      if (total < (uint64_t)p.chunks_off || total > (uint64_t)p.cap) s_bad = 1;
    }
    if (s_bad) code = 1u << KVTC_ERR_CORRUPT;
    st[0] = code; st[1] = 0; st[2] = 0; st[3] = 0;
  }
}

hipError_t launch_dec_check(const Params& p, const uint8_t* hdr, hipStream_t s) {
  HeaderBytes h;
  memcpy(h.b, hdr, kHeaderBytes);
  hipLaunchKernelGGL(k_dec_check, dim3(1, 1, seq_grid(p)), dim3(64), 0, s, p, h);
  return hipGetLastError();
}

// raw_runs > 0 (contiguous cache): workgroups past the chunks copy the raw
// sink and recent runs of the container to the outputs, which costs the
// bandwidth this latency-bound pass leaves idle.
__global__ void k_rans_dec_chunks(const Params p0, int raw_runs) {
  const Params p = at_seq(p0, blockIdx.z);
  const int c = blockIdx.x;
  if (c >= p.n_chunks) {
    if (c - p.n_chunks < raw_runs) copy_raw_run(p, c - p.n_chunks, 0, false);
    return;
  }
  const int u = c / p.chunks_per_sec, ch = c % p.chunks_per_sec;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (get_status(p.ws, p.w) & (1u << KVTC_ERR_CORRUPT)) return;
  // the decode tables at fixed LDS addresses (their base folds into the
  // instructions' offsets); the word rings in dynamic LDS
  __shared__ uint32_t fc[256];
  __shared__ uint32_t s_sym[1024];  // one byte per slot, 2^sb <= 4096 slots
  uint8_t* sym_of = reinterpret_cast<uint8_t*>(s_sym);
  extern __shared__ uint32_t lds[];
  uint16_t* rings = reinterpret_cast<uint16_t*>(lds);                     // kRing words per tile
  __shared__ int64_t s_info[4];
  __shared__ uint32_t s_cum[257];
  __shared__ int s_ok;
  __shared__ int32_t s_toff[17];
  const int n = min(p.chunk_tokens, p.T_mid - ch * p.chunk_tokens);
  const int ntiles = (n + p.tile_tokens - 1) / p.tile_tokens;
  const int n_last = n - (ntiles - 1) * p.tile_tokens;
  const uint8_t* dir = p.in + p.dir_off + (int64_t)c * kDirEntry;
  const uint64_t off = *reinterpret_cast<const uint64_t*>(dir);
  const uint32_t size = *reinterpret_cast<const uint32_t*>(dir + 8);
  const uint32_t resv = *reinterpret_cast<const uint32_t*>(dir + 12);
  const uint64_t total = *reinterpret_cast<const uint64_t*>(p.in + 168);
  const uint8_t* rec = p.in + off;
  if (wave == 0) {
    // the section's widths: each no more than max_bits (and the uniform
    // width on the WHT path), their sum within the budget; the packed tile
    // sizes follow from them
    const uint8_t* bits = p.in + p.side_off + (int64_t)u * 9 * p.D;
    const int s = (u / p.H) & 1;
    bool okl = true;
    int sum = 0;
    int64_t Pf = 0, Pl = 0;
    for (int i = lane; i < p.D; i += 64) {
      const int b = bits[i];
      if (b > p.max_bits) okl = false;
      if (p.transform == KVTC_WHT && b != (s == 0 ? p.bits_k_uniform : p.bits_v_uniform)) okl = false;
      sum += b;
      Pf += 4 * (int64_t)((p.tile_tokens * b + 31) >> 5);
      Pl += 4 * (int64_t)((n_last * b + 31) >> 5);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      sum += __shfl_xor(sum, o, 64);
      Pf += __shfl_xor(Pf, o, 64);
      Pl += __shfl_xor(Pl, o, 64);
    }
    bool ok = __ballot(!okl) == 0ull;
    if (p.transform == KVTC_PCA && sum > (s == 0 ? p.budget_k : p.budget_v)) ok = false;
    const int64_t P = ok ? (ntiles - 1) * Pf + Pl : 0;
    if (ok && resv != 0) ok = false;
    if (ok && P == 0 && size != 0) ok = false;
    if (ok && P > 0 &&
        (off < (uint64_t)p.chunks_off || (off & 15) || off > total || size > total - off ||
         size < 512 + 4 * (uint32_t)ntiles))
      ok = false;
    // stream offsets inside the record (a prefix sum over its tiles)
    int64_t piece = 0;
    if (ok && P > 0 && lane < ntiles) {
      const uint32_t nw = reinterpret_cast<const uint32_t*>(rec + 512)[lane];
      piece = 4 * (int64_t)p.lanes + 2 * (int64_t)nw + ((nw & 1) ? 2 : 0);
    }
    int64_t xs = piece;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int64_t y = __shfl_up(xs, o, 64);
      if (lane >= o) xs += y;
    }
    const int64_t base = 512 + 4 * (int64_t)ntiles;
    if (ok && P > 0 && align16(base + __shfl(xs, 63, 64)) != (int64_t)size) ok = false;
    if (lane < ntiles) s_toff[lane] = (int32_t)(base + xs - piece);
    if (lane == 0) {
      s_ok = ok ? 1 : 0;
      s_info[0] = Pf; s_info[1] = Pl; s_info[2] = P;
    }
  }
  __syncthreads();
  if (!s_ok) { if (threadIdx.x == 0) set_status(p.ws, p.w, KVTC_ERR_CORRUPT); return; }
  const int64_t P_full = s_info[0], P_last = s_info[1], P = s_info[2];
  if (P == 0) return;
  // frequency table -> cumulative -> slot lookup table
  if (wave == 0) {
    const uint16_t* fq = reinterpret_cast<const uint16_t*>(rec);
    uint32_t f[4], s = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) { f[k] = fq[4 * lane + k]; s += f[k]; }
    uint32_t x = s;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      uint32_t y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    uint32_t cum = x - s;
#pragma unroll
    for (int k = 0; k < 4; ++k) { s_cum[4 * lane + k] = cum; cum += f[k]; }
    if (lane == 63) s_cum[256] = cum;
  }
  __syncthreads();
  if (s_cum[256] != (1u << p.sb)) {
    if (threadIdx.x == 0) set_status(p.ws, p.w, KVTC_ERR_CORRUPT);
    return;
  }
  build_dec_tables(s_cum, p.sb, sym_of, fc);
  __syncthreads();
  const int spw = 64 / p.lanes;
  const int t = wave * spw + lane / p.lanes;
  const bool valid = t < ntiles;
  const int tt = valid ? t : 0;
  const int32_t Nt = valid ? (int32_t)(t == ntiles - 1 ? P_last : P_full) : 0;
  const int steps = (Nt + p.lanes - 1) / p.lanes;
  int steps_max = steps;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) steps_max = max(steps_max, __shfl_xor(steps_max, o, 64));
  uint8_t* slot = p.ws + p.w.packed + (int64_t)c * p.w.packed_slot;
  const int32_t nw = (int32_t)reinterpret_cast<const uint32_t*>(rec + 512)[tt];
  const uint32_t* states = reinterpret_cast<const uint32_t*>(rec + s_toff[tt]);
  const uint16_t* words = reinterpret_cast<const uint16_t*>(rec + s_toff[tt] + 4 * p.lanes);
  uint16_t* ring = rings + tt * kRing;
  const int32_t oo = (int32_t)(tt * P_full);
  const bool ok = p.lanes == 16
      ? rans_decode_ring<16>(states, words, nw, Nt, valid, steps_max, sym_of, fc, p.sb, ring, slot, oo, (int32_t)P)
      : rans_decode_ring<32>(states, words, nw, Nt, valid, steps_max, sym_of, fc, p.sb, ring, slot, oo, (int32_t)P);
  if (__ballot(!ok)) {
    if (lane == 0) set_status(p.ws, p.w, KVTC_ERR_CORRUPT);
  }
}

hipError_t launch_rans_decode_chunks(const Params& p, hipStream_t s, bool with_raw) {
  int streams = p.tiles_per_chunk;
  int waves = (streams * p.lanes + 63) / 64;
  if (waves < 1) waves = 1;
  // dynamic LDS: one word ring per tile (the symbol tables are static)
  const size_t lds = (size_t)p.tiles_per_chunk * kRing * 2;
  const int raw_runs = with_raw && p.n_seqs == 0 ? 4 * p.L * p.H : 0;
  hipLaunchKernelGGL(k_rans_dec_chunks, dim3(p.n_chunks + raw_runs, 1, seq_grid(p)), dim3(64 * waves), lds, s, p, raw_runs);
  return hipGetLastError();
}

// ---- single-stream parity hooks ---------------------------------------------

__global__ void k_test_rans_encode(const uint8_t* sym, int64_t N, const uint16_t* freq, int sb,
                                   int lanes, uint32_t* states, uint16_t* words, int64_t cap,
                                   int64_t* nwords) {
  __shared__ uint32_t f32v[256];
  __shared__ EncSym tab[256];
  for (int i = threadIdx.x; i < 256; i += blockDim.x) f32v[i] = freq[i];
  __syncthreads();
  build_enc_table(f32v, tab);
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const bool valid = lane < lanes;  // one stream in the first lane group
  const int steps = (int)((N + lanes - 1) / lanes);
  int64_t nw = rans_encode_stream(sym, (int32_t)N, 0, (int32_t)N, valid, steps, tab, sb, lanes,
                                  reinterpret_cast<uint8_t*>(words), (int32_t)(2 * cap), 0, (int32_t)cap, states);
  if (lane == 0) *nwords = nw;
}

hipError_t launch_test_rans_encode(const uint8_t* sym, int64_t N, const uint16_t* freq, int sb,
                                   int lanes, uint32_t* states, uint16_t* words, int64_t cap,
                                   int64_t* nwords, hipStream_t s) {
  hipLaunchKernelGGL(k_test_rans_encode, dim3(1), dim3(64), 0, s, sym, N, freq, sb, lanes, states,
                     words, cap, nwords);
  return hipGetLastError();
}

__global__ void k_test_rans_decode(const uint32_t* states, const uint16_t* words, int64_t nwords,
                                   const uint16_t* freq, int sb, int lanes, int64_t N, uint8_t* sym,
                                   int32_t* status) {
  extern __shared__ uint32_t lut[];
  __shared__ uint32_t s_cum[257];
  const int lane = threadIdx.x & 63;
  uint32_t f[4], s = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) { f[k] = freq[4 * lane + k]; s += f[k]; }
  uint32_t x = s;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  uint32_t cum = x - s;
#pragma unroll
  for (int k = 0; k < 4; ++k) { s_cum[4 * lane + k] = cum; cum += f[k]; }
  if (lane == 63) s_cum[256] = cum;
  __syncthreads();
  if (N > 0 && s_cum[256] != (1u << sb)) {
    if (lane == 0) *status = KVTC_ERR_CORRUPT;
    return;
  }
  uint32_t* fc = lut;
  uint8_t* sym_of = reinterpret_cast<uint8_t*>(lut + 256);
  build_dec_tables(s_cum, sb, sym_of, fc);
  __syncthreads();
  const bool valid = lane < lanes;
  const int steps = (int)((N + lanes - 1) / lanes);
  uint16_t* ring = reinterpret_cast<uint16_t*>(sym_of + (1 << sb));
  const bool ok = lanes == 16 ? rans_decode_ring<16>(states, words, (int32_t)nwords, (int32_t)N, valid, steps, sym_of, fc, sb, ring, sym, 0, (int32_t)N)
                              : rans_decode_ring<32>(states, words, (int32_t)nwords, (int32_t)N, valid, steps, sym_of, fc, sb, ring, sym, 0, (int32_t)N);
  if (__ballot(!ok) != 0ull) {
    if (lane == 0) *status = KVTC_ERR_CORRUPT;
  } else if (lane == 0) {
    *status = KVTC_OK;
  }
}

hipError_t launch_test_rans_decode(const uint32_t* states, const uint16_t* words, int64_t nwords,
                                   const uint16_t* freq, int sb, int lanes, int64_t N,
                                   uint8_t* sym, int32_t* status, hipStream_t s) {
  hipLaunchKernelGGL(k_test_rans_decode, dim3(1), dim3(64), 1024 + (size_t)(1u << sb) + kRing * 2, s, states, words,
                     nwords, freq, sb, lanes, N, sym, status);
  return hipGetLastError();
}

__global__ void k_test_freq(const uint32_t* counts, int sb, uint16_t* freq) {
  __shared__ uint32_t c[256], f[256];
  for (int i = threadIdx.x; i < 256; i += blockDim.x) c[i] = counts[i];
  __syncthreads();
  wave_freq_normalize(c, sb, f);
  __syncthreads();
  for (int i = threadIdx.x; i < 256; i += blockDim.x) freq[i] = (uint16_t)f[i];
}

hipError_t launch_test_freq(const uint32_t* counts, int sb, uint16_t* freq, hipStream_t s) {
  hipLaunchKernelGGL(k_test_freq, dim3(1), dim3(64), 0, s, counts, sb, freq);
  return hipGetLastError();
}

}  // namespace kvtc
