// Entropy coding ("KVTC: The Open-Source KV Cache Codec That Treats LLM
// Memory Like Media", rANS Makes the Last Mile Smaller): every chunk of a
// section is one record.  A component of width b >= 2 contributes one symbol
// per token -- the top min(b, 4) bits of its code -- coded with that
// component's own frequency table over the chunk; 1-bit codes and the low
// b - 4 bits of wider codes are stored raw.  Each tile of the chunk is one
// interleaved rANS stream of `lanes` 32-bit states: its symbol sequence runs
// over the coded components in index order, tokens in order within a
// component, and the k-th symbol of a component belongs to lane k % lanes.
// The decoder walks that sequence forwards, lanes ascending within a step,
// consuming 16-bit words from the end; the encoder walks it backwards and
// stores words in emission order.  A record that would not be smaller than
// the chunk's packed rows is stored as those rows instead ("Compress the
// most expensive bytes in AI", KV & tensor mode: never worse than plain).
//
// Record (coded): per coded component its 2^min(b,4) u16 frequencies (sum
// 2^sb), padded to 4 bytes; u32 word count per tile; per tile the lane
// states, the words (a zero u16 after an odd count) and the raw rows (per
// component with raw bits r, ceil(m r / 32) words, LSB-first); zero padding
// to 16 bytes.  Record (packed): the packed tiles back to back, padded to 16.
//
// Kernels: the record encoder (one workgroup per chunk: histograms, tables,
// streams, raw rows, record size and mode), the record assembly (prefix sum
// of record sizes, directory, header, compaction), the container check and
// the record decoder (one workgroup per chunk: tables, streams and raw rows
// back into packed tiles for the decode transform).
#include <string.h>

#include <algorithm>

#include "kvtc_internal.h"

namespace kvtc {

struct alignas(16) EncSym {  // one 16-byte LDS read per lookup
  uint32_t f;
  uint32_t cum;
  double rcp;  // 1/f rounded to fp64; quotient = trunc(fma(x, rcp, 2^-20))
};

// Raw buffer resource over [base, base + bytes) with wave-uniform fields, so
// the compiler keeps it in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(void* base, int32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a), hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* b = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(b, 0, __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

// ---- frequency tables of small alphabets ------------------------------------

// Counts of an alphabet of A <= 16 symbols -> frequencies summing to
// M = 2^sb (one thread per table): each present symbol gets
// max(1, round-half-up(n M / N)); a shortfall goes to the most frequent
// symbol (lowest on ties), an excess is taken one unit at a time from the
// largest frequency above 1 (lowest symbol on ties).  All zero when N = 0.
__device__ void normalize_small(const uint32_t* cnt, int A, int sb, uint32_t* f) {
  // a chunk has at most 32 tiles of 256 tokens, so n 2M + N < 2^27 and the
  // rounding division is exact in 32 bits
  uint32_t N = 0;
  for (int s = 0; s < A; ++s) N += cnt[s];
  if (N == 0) {
    for (int s = 0; s < A; ++s) f[s] = 0;
    return;
  }
  const uint32_t M = 1u << sb;
  int32_t sum = 0;
  int best = 0;
  for (int s = 0; s < A; ++s) {
    uint32_t r = 0;
    if (cnt[s]) {
      r = (cnt[s] * (2 * M) + N) / (2 * N);
      if (r < 1) r = 1;
    }
    f[s] = r;
    sum += (int32_t)r;
    if (cnt[s] > cnt[best]) best = s;
  }
  int32_t d = (int32_t)M - sum;
  if (d > 0) f[best] += (uint32_t)d;
  while (d < 0) {
    int bi = -1;
    for (int s = 0; s < A; ++s)
      if (f[s] > 1 && (bi < 0 || f[s] > f[bi])) bi = s;
    f[bi] -= 1;
    ++d;
  }
}

// ---- record geometry --------------------------------------------------------

constexpr int kMaxD = 128;

// What every workgroup of a chunk needs about its section's widths, in LDS.
struct RecGeo {
  uint8_t b[kMaxD];            // widths
  uint16_t roff[2][kMaxD];     // word offset of a component's row in a full [0] / the last [1] tile
  uint16_t raoff[2][kMaxD];    // word offset of its raw row in a tile's raw rows
  uint16_t toff[kMaxD];        // offset (u16 entries) of a coded component's table
  uint8_t coded[kMaxD];        // coded components (width >= 2), ascending
  uint8_t raw1[kMaxD];         // 1-bit components, ascending
  int32_t nc, n1;
  int32_t n, ntiles, n_last;   // tokens of the chunk, its tiles, tokens of the last tile
  int32_t pf, pl;              // packed bytes of a full / the last tile
  int32_t rf, rl;              // raw-row bytes of a full / the last tile
  int32_t tb;                  // table bytes of the record (4-aligned)
  int32_t tu;                  // table bytes before the padding
  int32_t sum_b;
  int64_t P;                   // packed bytes of the chunk
};

// Exclusive prefix over the components (lane l holds 2l and 2l + 1, so the
// order is the index order): the offsets of both and the total.
__device__ __forceinline__ void wave_scan2(uint32_t v0, uint32_t v1, uint32_t& e0, uint32_t& e1, uint32_t& total) {
  const int lane = threadIdx.x & 63;
  uint32_t x = v0 + v1;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  total = __shfl(x, 63, 64);
  e0 = x - v0 - v1;
  e1 = e0 + v0;
}

// Geometry of chunk cr of a section with widths `bits`; wave 0 of the block
// calls it and the caller synchronises.  D <= 128.
__device__ void rec_setup(const Params& p, int cr, const uint8_t* bits, RecGeo& g) {
  const int lane = threadIdx.x & 63;
  const int D = p.D;
  const int n = min(p.rec_tokens, p.T_mid - cr * p.rec_tokens);
  const int ntiles = (n + p.tile_tokens - 1) / p.tile_tokens;
  const int nl = n - (ntiles - 1) * p.tile_tokens;
  const int i0 = 2 * lane, i1 = 2 * lane + 1;
  const uint32_t b0 = i0 < D ? bits[i0] : 0u, b1 = i1 < D ? bits[i1] : 0u;
  const uint32_t h0 = (uint32_t)sym_bits_of((int)b0), h1 = (uint32_t)sym_bits_of((int)b1);
  const uint32_t r0 = (uint32_t)raw_bits_of((int)b0), r1 = (uint32_t)raw_bits_of((int)b1);
  const uint32_t T = (uint32_t)p.tile_tokens, L = (uint32_t)nl;
  uint32_t e0, e1, tot;
  wave_scan2((T * b0 + 31) >> 5, (T * b1 + 31) >> 5, e0, e1, tot);
  if (i0 < D) g.roff[0][i0] = (uint16_t)e0;
  if (i1 < D) g.roff[0][i1] = (uint16_t)e1;
  if (lane == 0) g.pf = 4 * (int32_t)tot;
  wave_scan2((L * b0 + 31) >> 5, (L * b1 + 31) >> 5, e0, e1, tot);
  if (i0 < D) g.roff[1][i0] = (uint16_t)e0;
  if (i1 < D) g.roff[1][i1] = (uint16_t)e1;
  if (lane == 0) g.pl = 4 * (int32_t)tot;
  wave_scan2((T * r0 + 31) >> 5, (T * r1 + 31) >> 5, e0, e1, tot);
  if (i0 < D) g.raoff[0][i0] = (uint16_t)e0;
  if (i1 < D) g.raoff[0][i1] = (uint16_t)e1;
  if (lane == 0) g.rf = 4 * (int32_t)tot;
  wave_scan2((L * r0 + 31) >> 5, (L * r1 + 31) >> 5, e0, e1, tot);
  if (i0 < D) g.raoff[1][i0] = (uint16_t)e0;
  if (i1 < D) g.raoff[1][i1] = (uint16_t)e1;
  if (lane == 0) g.rl = 4 * (int32_t)tot;
  wave_scan2(h0 ? 1u << h0 : 0u, h1 ? 1u << h1 : 0u, e0, e1, tot);
  if (i0 < D) g.toff[i0] = (uint16_t)e0;
  if (i1 < D) g.toff[i1] = (uint16_t)e1;
  if (lane == 0) {
    g.tu = (int32_t)(2 * tot);
    g.tb = (int32_t)((2 * tot + 3) & ~3u);
  }
  wave_scan2(h0 ? 1u : 0u, h1 ? 1u : 0u, e0, e1, tot);
  if (h0) g.coded[e0] = (uint8_t)i0;
  if (h1) g.coded[e1] = (uint8_t)i1;
  if (lane == 0) g.nc = (int32_t)tot;
  wave_scan2(b0 == 1 ? 1u : 0u, b1 == 1 ? 1u : 0u, e0, e1, tot);
  if (b0 == 1) g.raw1[e0] = (uint8_t)i0;
  if (b1 == 1) g.raw1[e1] = (uint8_t)i1;
  if (lane == 0) g.n1 = (int32_t)tot;
  wave_scan2(b0, b1, e0, e1, tot);
  if (lane == 0) g.sum_b = (int32_t)tot;
  if (i0 < D) g.b[i0] = (uint8_t)b0;
  if (i1 < D) g.b[i1] = (uint8_t)b1;
  if (lane == 0) {
    g.n = n;
    g.ntiles = ntiles;
    g.n_last = nl;
    g.P = (int64_t)(ntiles - 1) * g.pf + g.pl;
  }
}

// Packed tile t of chunk cr of section u in the workspace (work-block slots;
// every tile before a section's last is full).
__device__ __forceinline__ uint8_t* packed_tile(const Params& p, int u, int cr, int t, int32_t pf) {
  const int blk = cr * p.blks_per_rec + t / p.tiles_per_blk;
  const int ti = t % p.tiles_per_blk;
  return p.ws + p.w.packed + ((int64_t)u * p.blks_per_sec + blk) * p.w.packed_slot + (int64_t)ti * pf;
}

// Record slot of chunk r and the pieces of tile t inside it: lane states,
// words (capacity tile_words_max) and raw rows (capacity tile_raw_max).
__device__ __forceinline__ uint8_t* rec_slot(const Params& p, int r) { return p.ws + p.w.rec + (int64_t)r * p.w.rec_slot; }
__device__ __forceinline__ int64_t slot_counts_off(const Params& p) { return slot_table_bytes(p.cfg); }
__device__ __forceinline__ int64_t slot_tile_off(const Params& p, int t) {
  return align16(slot_table_bytes(p.cfg) + 4 * (int64_t)p.tiles_per_rec) +
         (int64_t)t * (4 * p.lanes + 2 * p.w.tile_words_max + p.w.tile_raw_max);
}
__device__ __forceinline__ int64_t slot_raw_off(const Params& p, int t) {
  return slot_tile_off(p, t) + 4 * p.lanes + 2 * p.w.tile_words_max;
}

__device__ __forceinline__ uint32_t funnel(uint32_t lo, uint32_t hi, uint32_t sh) {
  return (uint32_t)((((uint64_t)hi << 32) | lo) >> sh);
}

// ---- record encoder ---------------------------------------------------------

constexpr int kHistCopies = 4;  // histogram copies per component in the record encoder
constexpr int kRowWords = 66;  // a staged component row of a 256-token tile (<= 64 words), zero-padded
constexpr int kRawWords = 34;  // a raw row of a 256-token tile (<= 32 words), zero-padded

// raw_runs > 0 (contiguous cache): workgroups past the chunks copy the raw
// sink and recent runs into the container, on the bandwidth this
// latency-bound pass leaves idle.
// STEPS = tile_tokens / LANES when the launch fixes it (0: from the tile at
// run time).  With a fixed step count the loops unroll and every memory
// operation of a component is issued unconditionally, so the wait for the
// next component's prefetched row does not also wait for the stores issued
// after it (loads and stores retire in order on one counter).
template <int LANES, int STEPS>
__global__ __launch_bounds__(1024) void k_rans_enc_recs(const Params p0, int raw_runs) {
  constexpr int SPW = 64 / LANES;  // streams per wave
  constexpr int NQ = 64 / LANES + 1;  // staged row words per lane
  const Params p = at_seq(p0, blockIdx.z);
  const int r = blockIdx.x;
  if (r >= p.n_recs) {
    if (r - p.n_recs < raw_runs) copy_raw_run(p, r - p.n_recs, 1, false);
    return;
  }
  const int u = r / p.recs_per_sec, cr = r % p.recs_per_sec;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (get_status(p.ws, p.w) & (1u << KVTC_ERR_NONFINITE)) return;
  __shared__ RecGeo g;
  // histograms (kHistCopies per component, picked by lane, so that fewer
  // lanes add to one bin at once), later the encoder tables in the same LDS
  __shared__ __align__(16) uint32_t histtab[kMaxD * kHistCopies * 17];
  static_assert(sizeof(histtab) >= kMaxD * 16 * sizeof(EncSym), "tables fit in the histogram space");
  uint32_t* const hist = histtab;
  EncSym* const tab = reinterpret_cast<EncSym*>(histtab);
  __shared__ uint32_t rowbuf[kMaxTilesPerRec][2][kRowWords];
  __shared__ uint32_t rawrow[kMaxTilesPerRec][kRawWords];  // a component's raw row being assembled
  __shared__ int32_t s_nw[kMaxTilesPerRec];
  if (wave == 0) rec_setup(p, cr, p.ws + p.w.side_bits + (int64_t)u * p.D, g);
  for (int i = tid; i < kMaxD * kHistCopies * 17; i += blockDim.x) hist[i] = 0;
  __syncthreads();
  uint32_t* rec_size = reinterpret_cast<uint32_t*>(p.ws + p.w.rec_size);
  uint32_t* rec_mode = reinterpret_cast<uint32_t*>(p.ws + p.w.rec_mode);
  if (g.P == 0) {
    if (tid == 0) { rec_size[r] = 0; rec_mode[r] = 0; }
    return;
  }
  const int nc = g.nc, ntiles = g.ntiles;
  uint8_t* slot = rec_slot(p, r);
  // -- streams: lane group grp of the wave codes tile t
  const int grp = lane / LANES, j = lane % LANES;
  const int t = wave * SPW + grp;
  const bool valid = t < ntiles;
  const bool last = valid && t == ntiles - 1;
  const int m = !valid ? 0 : (last ? g.n_last : p.tile_tokens);
  const int tt = valid ? t : 0;
  const bool has_stream = wave * SPW < ntiles;  // wave-uniform
  const uint32_t* tbase = reinterpret_cast<const uint32_t*>(packed_tile(p, u, cr, tt, g.pf));
  uint32_t* rb = &rowbuf[tt][0][0];
  int steps_max = (m + LANES - 1) / LANES;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) steps_max = max(steps_max, __shfl_xor(steps_max, o, 64));
  steps_max = STEPS > 0 ? STEPS : __builtin_amdgcn_readfirstlane(steps_max);
  // the record's packed tiles through one buffer resource: its work blocks
  // are consecutive slots, and a lane's tile starts at tile_at
  const int32_t prec_bytes = (int32_t)((int64_t)p.blks_per_rec * p.w.packed_slot);
  const __amdgpu_buffer_rsrc_t prsrc = uniform_rsrc(packed_tile(p, u, cr, 0, g.pf), prec_bytes);
  const int32_t tile_at = (int32_t)((int64_t)(tt / p.tiles_per_blk) * p.w.packed_slot + (int64_t)(tt % p.tiles_per_blk) * g.pf);
  // the row of component i of this tile: NQ words per lane into registers
  // (lanes past the row load zeros), then into this stream's LDS row buffer.
  // Two register sets alternate between even and odd components, so a row
  // is loaded two components before its use and the load's latency hides
  // behind a whole component.
  uint32_t pre0[NQ], pre1[NQ];
  auto row_load = [&](uint32_t(&pr)[NQ], int i) {
    const int W = (m * (int)g.b[i] + 31) >> 5;
    const int32_t at = tile_at + 4 * (int32_t)g.roff[last][i];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int w = j + q * LANES;
      pr[q] = __builtin_amdgcn_raw_buffer_load_b32(prsrc, (valid && w < W) ? at + 4 * w : prec_bytes, 0, 0);
    }
  };
  auto row_store = [&](const uint32_t(&pr)[NQ], int which) {
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int w = j + q * LANES;
      if (valid && w < kRowWords) rb[which * kRowWords + w] = pr[q];
    }
  };
  // -- histograms: each stream counts its tile's symbols component by
  // component from the staged rows
  if (has_stream && nc > 0) {
    auto hist_component = [&](int ci, uint32_t(&pr)[NQ]) {
      const int i = g.coded[ci];
      const uint32_t b = g.b[i], rr = b - (uint32_t)sym_bits_of((int)b);
      row_store(pr, ci & 1);  // its buffer was last read two components ago
      if (ci + 2 < nc) row_load(pr, g.coded[ci + 2]);
      __builtin_amdgcn_wave_barrier();
      const uint32_t* rw = rb + (ci & 1) * kRowWords;
      uint32_t* hc = hist + (ci * kHistCopies + (lane & (kHistCopies - 1))) * 17;
      if constexpr (LANES == 32 && STEPS > 0) {
        // token k = 32 s + j sits at word s b + (j b >> 5) of the row, at the
        // lane's constant shift (j b) & 31: every word of the component first
        const uint32_t jb = (uint32_t)j * b, sh = jb & 31u, mask = (1u << b) - 1u;
        const uint32_t* rwl = rw + (jb >> 5);
        uint32_t lo[STEPS], hi[STEPS];
#pragma unroll
        for (int s = 0; s < STEPS; ++s) {
          lo[s] = rwl[s * b];
          hi[s] = rwl[s * b + 1];
        }
        // the lane's STEPS <= 8 symbols counted in 4-bit fields (symbol y at
        // bits 4y), widened to bytes (B0: even symbols 0-6, B1: odd 1-7, B2:
        // even 8-14, B3: odd 9-15) and summed over each 16-lane row by DPP
        // adds (at most 128 a byte); then lane k of a row adds the row's count
        // of symbol k to the first histogram copy
        static_assert(STEPS <= 8, "4-bit per-lane counts");
        uint64_t nib = 0;
#pragma unroll
        for (int s = 0; s < STEPS; ++s) {
          const uint32_t code = __builtin_amdgcn_alignbit(hi[s], lo[s], sh) & mask;
          if (valid && s * LANES + j < m) nib += 1ull << (4u * (code >> rr));
        }
        const uint32_t A = 1u << (b - rr);  // symbols: 4, 8 or 16
        auto row_sum = [](uint32_t v) {
          v += (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);   // lane ^ 1
          v += (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);   // lane ^ 2
          v += (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false);  // 7 - lane % 8
          v += (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false);  // 15 - lane % 16
          return v;
        };
        const uint32_t nlo = (uint32_t)nib, nhi = (uint32_t)(nib >> 32);
        const uint32_t B0 = row_sum(nlo & 0x0F0F0F0Fu), B1 = row_sum((nlo >> 4) & 0x0F0F0F0Fu);
        uint32_t B2 = 0u, B3 = 0u;
        if (A > 8u) {
          B2 = row_sum(nhi & 0x0F0F0F0Fu);
          B3 = row_sum((nhi >> 4) & 0x0F0F0F0Fu);
        }
        const uint32_t k = (uint32_t)j & 15u;
        const uint32_t reg = k < 8u ? ((k & 1u) ? B1 : B0) : ((k & 1u) ? B3 : B2);
        const uint32_t cnt = (reg >> (8u * ((k >> 1) & 3u))) & 0xFFu;
        if (valid && k < A && cnt) atomicAdd(&hist[ci * kHistCopies * 17 + k], cnt);
        return;
      }
#pragma unroll
      for (int s = 0; s < (STEPS > 0 ? STEPS : steps_max); ++s) {
        const int k = s * LANES + j;
        if (valid && k < m) {
          const uint32_t bp = (uint32_t)k * b;
          const uint32_t code = funnel(rw[bp >> 5], rw[(bp >> 5) + 1], bp & 31) & ((1u << b) - 1u);
          atomicAdd(&hc[code >> rr], 1u);
        }
      }
    };
    row_load(pre0, g.coded[0]);
    if (nc > 1) row_load(pre1, g.coded[1]);
    for (int ci = 0; ci < nc; ci += 2) {
      hist_component(ci, pre0);
      if (ci + 1 < nc) hist_component(ci + 1, pre1);
    }
  }
  __syncthreads();
  // -- tables: the histogram copies summed into the first, then one thread
  // per coded component normalises its counts into the record's table; the
  // encoder tables overwrite the histograms once every count has been read
  for (int idx = tid; idx < nc * 16; idx += blockDim.x) {
    uint32_t* hc = hist + (idx >> 4) * kHistCopies * 17 + (idx & 15);
    uint32_t sum = 0;
#pragma unroll
    for (int c = 0; c < kHistCopies; ++c) sum += hc[c * 17];
    hc[0] = sum;
  }
  __syncthreads();
  for (int ci = tid; ci < nc; ci += blockDim.x) {
    const int i = g.coded[ci];
    const int A = 1 << sym_bits_of((int)g.b[i]);
    uint32_t f[16];
    normalize_small(hist + ci * kHistCopies * 17, A, p.sb, f);
    uint16_t* ft = reinterpret_cast<uint16_t*>(slot) + g.toff[i];
    for (int s = 0; s < A; ++s) ft[s] = (uint16_t)f[s];
  }
  __syncthreads();
  for (int ci = tid; ci < nc; ci += blockDim.x) {
    const int i = g.coded[ci];
    const int A = 1 << sym_bits_of((int)g.b[i]);
    const uint16_t* ft = reinterpret_cast<const uint16_t*>(slot) + g.toff[i];
    uint32_t cum = 0;
    for (int s = 0; s < A; ++s) {
      const uint32_t fs = ft[s];
      EncSym e;
      e.f = fs;
      e.cum = cum;
      e.rcp = fs ? __ddiv_rn(1.0, (double)fs) : 0.0;
      tab[ci * 16 + s] = e;
      cum += fs;
    }
  }
  if (tid == 0 && g.tu < g.tb) *reinterpret_cast<uint16_t*>(slot + g.tu) = 0;  // padding to 4 bytes
  __syncthreads();
  int32_t nw = 0;
  if (has_stream) {
    const int64_t toff = slot_tile_off(p, tt);
    uint32_t* states = reinterpret_cast<uint32_t*>(slot + toff);
    const int32_t woff = (int32_t)(toff + 4 * LANES);
    const int32_t wcap = (int32_t)p.w.tile_words_max;
    const __amdgpu_buffer_rsrc_t wrsrc = uniform_rsrc(slot, (int32_t)p.w.rec_slot);
    uint32_t* rawdst = reinterpret_cast<uint32_t*>(slot + slot_raw_off(p, tt));
    const uint64_t gm = ((1ull << LANES) - 1ull) << (grp * LANES);
    const uint32_t gm_lo = (uint32_t)gm, gm_hi = (uint32_t)(gm >> 32);
    const uint32_t sbm = 32u - (uint32_t)p.sb, Mv = 1u << p.sb;
    uint32_t x = kRansL;
    uint32_t* rrow = &rawrow[tt][0];
    if (valid)
      for (int w = j; w < kRawWords; w += LANES) rrow[w] = 0u;
    auto enc_component = [&](int ci, uint32_t(&pr)[NQ]) {
      const int i = g.coded[ci];
      const uint32_t b = g.b[i], rr = b - (uint32_t)sym_bits_of((int)b);
      const uint32_t mask = (1u << b) - 1u, rmask = (1u << rr) - 1u;
      row_store(pr, ci & 1);  // its buffer was last read two components ago
      if (ci >= 2) row_load(pr, g.coded[ci - 2]);
      __builtin_amdgcn_wave_barrier();
      const uint32_t* rw = rb + (ci & 1) * kRowWords;
      const uint4* tc = reinterpret_cast<const uint4*>(tab + ci * 16);
      if constexpr (LANES == 32 && STEPS > 0 && STEPS % 4 == 0) {
        // token k = 32 s + j: its code at word s b + (j b >> 5) of the row and
        // its raw bits at word s rr + (j rr >> 5) of the raw row, each at the
        // lane's constant shift; a step's words for the ring are placed by a
        // ballot over the wave split into its two streams (lanes 0-31, 32-63)
        const uint32_t jb = (uint32_t)j * b, shb = jb & 31u;
        const uint32_t jr = (uint32_t)j * rr, shr = jr & 31u;
        const uint32_t* rwl = rw + (jb >> 5);
        uint32_t* rrl = rrow + (jr >> 5);
        const bool upper = grp != 0;
#pragma unroll
        for (int s0 = STEPS - 1; s0 >= 0; s0 -= 4) {
          uint32_t lo[4], hi[4], code[4];
          uint4 ent[4];
          bool act[4];
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            lo[d] = rwl[(s0 - d) * b];
            hi[d] = rwl[(s0 - d) * b + 1];
          }
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            act[d] = valid && (s0 - d) * LANES + j < m;
            code[d] = __builtin_amdgcn_alignbit(hi[d], lo[d], shb) & mask;
            ent[d] = tc[code[d] >> rr];
          }
          if (rr == 3) {  // the low bits into the raw row (a 3-bit field may straddle a word)
#pragma unroll
            for (int d = 0; d < 4; ++d) {
              const uint32_t v = act[d] ? (code[d] & rmask) : 0u;
              uint32_t* wp = rrl + (s0 - d) * rr;
              atomicOr(wp, v << shr);
              if (shr > 29) atomicOr(wp + 1, v >> (32 - shr));
            }
          } else if (rr) {
            // rr = 1, 2, 4: a raw word holds the fields of an aligned run of
            // 32 / rr lanes of one step; the run ORs them across lanes (quad
            // swaps, half-row and row mirrors, then row 0's total into row 1)
            // and one lane of the run stores the word
            const bool leader = rr == 1 ? j == 31 : (j & ((32u / rr) - 1u)) == 0u;
#pragma unroll
            for (int d = 0; d < 4; ++d) {
              uint32_t v = (act[d] ? (code[d] & rmask) : 0u) << shr;
              v |= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);  // lane ^ 1
              v |= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);  // lane ^ 2
              v |= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false);  // 7 - lane % 8
              if (rr <= 2u) v |= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false);  // 15 - lane % 16
              if (rr == 1u) v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);  // lane 15 into the next row
              if (valid && leader) rrl[(s0 - d) * rr] = v;
            }
          }
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            const uint32_t f = ent[d].x, cum = ent[d].y;
            const double rcp = __hiloint2double((int)ent[d].w, (int)ent[d].z);
            // renormalise while x >= f 2^(32 - sb): one 16-bit word at most
            const bool emit = act[d] && (x >> sbm) >= f;
            const uint64_t bl = __ballot(emit);
            const uint32_t blo = (uint32_t)bl, bhi = (uint32_t)(bl >> 32);
            const uint32_t nlo = (uint32_t)__popc(blo), nhi = (uint32_t)__popc(bhi);
            const int32_t cnt = (int32_t)(upper ? nhi : nlo);
            // words are written in emission order, higher lanes first
            const int32_t below =
                (int32_t)__builtin_amdgcn_mbcnt_hi(bhi, __builtin_amdgcn_mbcnt_lo(blo, 0u)) - (upper ? (int32_t)nlo : 0);
            const int32_t at = nw + cnt - 1 - below;
            if (emit && at < wcap)
              __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(x & 0xffffu), wrsrc, woff + 2 * at, 0, 0);
            const uint32_t xe = emit ? (x >> 16) : x;
            nw += cnt;
            // x = floor(x / f) M + (x mod f) + cum, via an exact fp64 quotient
            const uint32_t qq = (uint32_t)__fma_rn((double)xe, rcp, 0x1p-20);
            const uint32_t xn = xe + cum + __umul24(qq, Mv - f);
            x = act[d] ? xn : x;
          }
        }
      } else {
      // bit positions of token k = s LANES + j in the packed row and in the raw row
      const uint32_t jb = (uint32_t)j * b, jr = (uint32_t)j * rr;
      const uint32_t sb_step = (uint32_t)LANES * b, sr_step = (uint32_t)LANES * rr;
      // steps from the last down, four at a time: the symbols and their table
      // entries do not depend on the state, so they are all read first
#pragma unroll
      for (int s0 = (STEPS > 0 ? STEPS : steps_max) - 1; s0 >= 0; s0 -= 4) {
        uint4 ent[4];
        bool act[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const int st = s0 - d;
          const int k = st * LANES + j;
          act[d] = valid && st >= 0 && k < m;
          const uint32_t bp = act[d] ? jb + (uint32_t)st * sb_step : 0u;
          const uint32_t code = funnel(rw[bp >> 5], rw[(bp >> 5) + 1], bp & 31) & mask;
          ent[d] = tc[code >> rr];
          if (rr) {  // the low bits into the raw row (no field straddles a word unless rr = 3)
            const uint32_t bq = act[d] ? jr + (uint32_t)st * sr_step : 0u;
            const uint32_t lo = act[d] ? (code & rmask) : 0u;
            atomicOr(&rrow[bq >> 5], lo << (bq & 31));
            if (rr == 3) atomicOr(&rrow[(bq >> 5) + 1], (uint32_t)(((uint64_t)lo << (bq & 31)) >> 32));
          }
        }
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const bool active = act[d];
          const uint32_t f = ent[d].x, cum = ent[d].y;
          const double rcp = __hiloint2double((int)ent[d].w, (int)ent[d].z);
          // renormalise while x >= f 2^(32 - sb): one 16-bit word at most
          const bool emit = active && (x >> sbm) >= f;
          const uint64_t bl = __ballot(emit);
          const uint32_t mlo = (uint32_t)bl & gm_lo, mhi = (uint32_t)(bl >> 32) & gm_hi;
          const int32_t cnt = (int32_t)(__popc(mlo) + __popc(mhi));
          // words are written in emission order, higher lanes first
          const int32_t below = (int32_t)__builtin_amdgcn_mbcnt_hi(mhi, __builtin_amdgcn_mbcnt_lo(mlo, 0u));
          const int32_t at = nw + cnt - 1 - below;
          __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(x & 0xffffu), wrsrc,
                                                (emit && at < wcap) ? woff + 2 * at : (int32_t)p.w.rec_slot, 0, 0);
          const uint32_t xe = emit ? (x >> 16) : x;
          nw += cnt;
          // x = floor(x / f) M + (x mod f) + cum, via an exact fp64 quotient
          const uint32_t qq = (uint32_t)__fma_rn((double)xe, rcp, 0x1p-20);
          const uint32_t xn = xe + cum + __umul24(qq, Mv - f);
          x = active ? xn : x;
        }
      }
      }  // generic steps
      // the component's raw row to the slot; the buffer is cleared for the next
      if (rr) {
        __builtin_amdgcn_wave_barrier();
        const int Wr = (m * (int)rr + 31) >> 5;
        const int32_t at = (int32_t)(slot_raw_off(p, tt) + 4 * (int64_t)g.raoff[last][i]);
#pragma unroll
        for (int q = 0; q < (kRawWords + LANES - 1) / LANES; ++q) {
          const int w = j + q * LANES;
          const uint32_t v = w < kRawWords ? rrow[w] : 0u;
          __builtin_amdgcn_raw_buffer_store_b32(v, wrsrc, (valid && w < Wr) ? at + 4 * w : (int32_t)p.w.rec_slot, 0, 0);
          if (valid && w < kRawWords) rrow[w] = 0u;
        }
      }
    };
    if (nc > 0) row_load(pre0, g.coded[nc - 1]);
    if (nc > 1) row_load(pre1, g.coded[nc - 2]);
    for (int ci = nc - 1; ci >= 0; ci -= 2) {
      enc_component(ci, pre0);
      if (ci >= 1) enc_component(ci - 1, pre1);
    }
    if (valid) states[j] = x;
    // 1-bit components: the packed row is the raw row
    if (valid) {
      for (int q = 0; q < g.n1; ++q) {
        const int i = g.raw1[q];
        const uint32_t* src = tbase + g.roff[last][i];
        uint32_t* dst = rawdst + g.raoff[last][i];
        for (int w = j; w < ((m + 31) >> 5); w += LANES) dst[w] = src[w];
      }
    }
    // every word of the stream went below its final count, so one went past
    // the capacity exactly when the count exceeds it (those stores were
    // dropped, and the record falls back to the packed form)
    if (nw > wcap) nw = -1;
  }
  if (valid && j == 0) s_nw[t] = nw;
  __syncthreads();
  if (tid == 0) {
    bool fall_back = false;
    int64_t size = g.tb + 4 * (int64_t)ntiles;
    for (int k = 0; k < ntiles; ++k) {
      const int32_t w = s_nw[k];
      if (w < 0) fall_back = true;
      const int64_t wk = w < 0 ? 0 : w;
      reinterpret_cast<uint32_t*>(slot + slot_counts_off(p))[k] = (uint32_t)wk;
      size += 4 * (int64_t)LANES + 2 * wk + ((wk & 1) ? 2 : 0) + (k == ntiles - 1 ? g.rl : g.rf);
    }
    size = align16(size);
    const int64_t packed = align16(g.P);
    if (fall_back || size >= packed) {
      rec_size[r] = (uint32_t)packed;
      rec_mode[r] = 1;
    } else {
      rec_size[r] = (uint32_t)size;
      rec_mode[r] = 0;
    }
  }
}

hipError_t launch_rans_encode_chunks(const Params& p, hipStream_t s, bool with_raw) {
  int waves = (p.tiles_per_rec * p.lanes + 63) / 64;
  if (waves < 1) waves = 1;
  const int raw_runs = with_raw && p.n_seqs == 0 ? 4 * p.L * p.H : 0;
  const dim3 grid(p.n_recs + raw_runs, 1, seq_grid(p)), block(64 * waves);
  const int steps = p.tile_tokens / p.lanes;
  if (p.lanes == 16) {
    if (steps == 16) hipLaunchKernelGGL((k_rans_enc_recs<16, 16>), grid, block, 0, s, p, raw_runs);
    else if (steps == 8) hipLaunchKernelGGL((k_rans_enc_recs<16, 8>), grid, block, 0, s, p, raw_runs);
    else hipLaunchKernelGGL((k_rans_enc_recs<16, 0>), grid, block, 0, s, p, raw_runs);
  } else {
    if (steps == 8) hipLaunchKernelGGL((k_rans_enc_recs<32, 8>), grid, block, 0, s, p, raw_runs);
    else if (steps == 4) hipLaunchKernelGGL((k_rans_enc_recs<32, 4>), grid, block, 0, s, p, raw_runs);
    else hipLaunchKernelGGL((k_rans_enc_recs<32, 0>), grid, block, 0, s, p, raw_runs);
  }
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
    case 29: return (uint32_t)p.recs_per_sec;
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

// The header, the container size and the status, once the total is known.
__device__ inline void finish_container(const Params& p, const HeaderBytes& hdr, uint64_t total, int tid) {
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

__device__ inline void write_dir(const Params& p, int r, uint64_t pos, uint32_t size, uint32_t mode) {
  reinterpret_cast<uint64_t*>(p.ws + p.w.rec_pos)[r] = pos;
  uint8_t* d = p.out + p.dir_off + (int64_t)r * kDirEntry;
  *reinterpret_cast<uint64_t*>(d) = (uint64_t)p.chunks_off + pos;
  *reinterpret_cast<uint32_t*>(d + 8) = size;
  *reinterpret_cast<uint32_t*>(d + 12) = mode;
}

// One workgroup: exclusive prefix of the record sizes, directory, header.
__global__ __launch_bounds__(1024) void k_scan(const Params p0, HeaderBytes hdr) {
  const Params p = at_seq(p0, blockIdx.z);
  const uint32_t* rec_size = reinterpret_cast<const uint32_t*>(p.ws + p.w.rec_size);
  const uint32_t* rec_mode = reinterpret_cast<const uint32_t*>(p.ws + p.w.rec_mode);
  const int64_t n = p.n_recs;
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
  uint64_t run = incl - local;
  for (int64_t i = a; i < b; ++i) {
    write_dir(p, (int)i, run, rec_size[i], reinterpret_cast<const uint32_t*>(rec_mode)[i]);
    run += rec_size[i];
  }
  __shared__ uint64_t s_total;
  if (tid == 1023) s_total = incl;
  __syncthreads();
  finish_container(p, hdr, (uint64_t)p.chunks_off + s_total, tid);
}

// Copy of record r into the container, one wave per tile piece (the waves'
// copies overlap).  scan = 1 (a contiguous call with few records): each
// workgroup sums the sizes of the records before its own, writes its
// directory entry, and the last one writes the header, the container size and
// the status word, as k_scan does.
constexpr int kCopyWaves = 16;

// at least 8 waves per SIMD (64 VGPRs): two 16-wave workgroups share a CU, so
// the 512 records of a 32-layer, 8-head cache are copied in one round
__global__ __launch_bounds__(64 * kCopyWaves, 8) void k_copy_records(const Params p0, HeaderBytes hdr, int scan) {
  const Params p = at_seq(p0, blockIdx.z);
  const int r = blockIdx.x;
  if (r >= p.n_recs) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t* rec_size = reinterpret_cast<const uint32_t*>(p.ws + p.w.rec_size);
  const uint32_t size = rec_size[r];
  const uint32_t mode = reinterpret_cast<const uint32_t*>(p.ws + p.w.rec_mode)[r];
  __shared__ uint64_t s_part[kCopyWaves];
  __shared__ int64_t s_at[kMaxTilesPerRec + 1];
  __shared__ RecGeo g;
  uint64_t pos;
  if (scan) {
    uint64_t part = 0;
    for (int i = tid; i < r; i += 64 * kCopyWaves) part += rec_size[i];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) part += __shfl_xor(part, o, 64);
    if (lane == 0) s_part[wave] = part;
    __syncthreads();
    pos = 0;
    for (int k = 0; k < kCopyWaves; ++k) pos += s_part[k];
    if (tid == 0) write_dir(p, r, pos, size, mode);
    if (r == p.n_recs - 1) finish_container(p, hdr, (uint64_t)p.chunks_off + pos + size, tid);
    // a record that does not fit is not copied (the last workgroup reports
    // the capacity error)
    if ((uint64_t)p.chunks_off + pos + size > (uint64_t)p.cap) return;
  } else {
    pos = reinterpret_cast<const uint64_t*>(p.ws + p.w.rec_pos)[r];
  }
  if (get_status(p.ws, p.w) & ((1u << KVTC_ERR_CAPACITY) | (1u << KVTC_ERR_NONFINITE))) return;
  if (size == 0) {  // an empty record: the checksum of no words
    if (tid < 2) reinterpret_cast<uint64_t*>(p.out_final + p.dir_off + (int64_t)r * kDirEntry + 16)[tid] = 0;
    return;
  }
  const int u = r / p.recs_per_sec, cr = r % p.recs_per_sec;
  if (wave == 0) rec_setup(p, cr, p.ws + p.w.side_bits + (int64_t)u * p.D, g);
  __syncthreads();
  const int ntiles = g.ntiles;
  const uint8_t* slot = rec_slot(p, r);
  const uint32_t* nwv = reinterpret_cast<const uint32_t*>(slot + slot_counts_off(p));
  if (wave == 0) {  // where each tile's piece starts in the record
    int64_t piece = 0;
    if (lane < ntiles) {
      const int64_t pt = lane == ntiles - 1 ? g.pl : g.pf;
      if (mode == 1) {
        piece = pt;
      } else {
        const uint32_t nw = nwv[lane];
        piece = 4 * (int64_t)p.lanes + 2 * (int64_t)nw + ((nw & 1) ? 2 : 0) + (lane == ntiles - 1 ? g.rl : g.rf);
      }
    }
    int64_t xs = piece;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int64_t y = __shfl_up(xs, o, 64);
      if (lane >= o) xs += y;
    }
    const int64_t base = mode == 1 ? 0 : g.tb + 4 * (int64_t)ntiles;
    if (lane < ntiles) s_at[lane] = base + xs - piece;
    if (lane == ntiles - 1) s_at[ntiles] = base + xs;
  }
  __syncthreads();
  uint8_t* dst = p.out_final + p.chunks_off + pos;  // 16-byte aligned record
  // the record's checksum, summed over the words as they are copied (the
  // zero padding adds nothing)
  uint64_t ca = 0, cb = 0;
  // one wave copies n_dw dwords, eight in flight per lane; the last keeps only
  // its low half when `half_last` (an odd word count padded with zeros)
  auto copy_dw = [&](const uint32_t* src, uint32_t* d, int n_dw, bool half_last) {
    const uint64_t j0 = (uint64_t)(reinterpret_cast<uint8_t*>(d) - dst) >> 2;  // record word index of d[0]
    for (int i0 = 0; i0 < n_dw; i0 += 8 * 64) {
      uint32_t v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int i = i0 + k * 64 + lane;
        v[k] = i < n_dw ? src[i] : 0u;
      }
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int i = i0 + k * 64 + lane;
        if (i < n_dw) {
          const uint32_t w = (half_last && i == n_dw - 1) ? (v[k] & 0xffffu) : v[k];
          d[i] = w;
          csum_add(ca, cb, j0 + (uint64_t)i, w);
        }
      }
    }
  };
  for (int t = wave; t < ntiles; t += kCopyWaves) {
    uint8_t* d = dst + s_at[t];
    if (mode == 1) {
      const int32_t pt = t == ntiles - 1 ? g.pl : g.pf;
      copy_dw(reinterpret_cast<const uint32_t*>(packed_tile(p, u, cr, t, g.pf)), reinterpret_cast<uint32_t*>(d),
              pt / 4, false);
    } else {
      const uint32_t nw = nwv[t];
      const int n_dw = p.lanes + (int)((nw + 1) >> 1);  // states, words, zero pad to 4 bytes
      copy_dw(reinterpret_cast<const uint32_t*>(slot + slot_tile_off(p, t)), reinterpret_cast<uint32_t*>(d), n_dw,
              (nw & 1) != 0);
      const int32_t rbytes = t == ntiles - 1 ? g.rl : g.rf;
      copy_dw(reinterpret_cast<const uint32_t*>(slot + slot_raw_off(p, t)), reinterpret_cast<uint32_t*>(d + 4 * n_dw),
              rbytes / 4, false);
    }
  }
  if (mode == 0 && wave == kCopyWaves - 1) {  // tables and word counts
    copy_dw(reinterpret_cast<const uint32_t*>(slot), reinterpret_cast<uint32_t*>(dst), g.tb / 4, false);
    copy_dw(nwv, reinterpret_cast<uint32_t*>(dst + g.tb), ntiles, false);
  }
  for (int64_t i = s_at[ntiles] + tid; i < size; i += 64 * kCopyWaves) dst[i] = 0;
  __shared__ uint64_t s_cs[32];
  csum_block_reduce(ca, cb, s_cs);
  if (tid == 0) {
    uint64_t* d = reinterpret_cast<uint64_t*>(p.out_final + p.dir_off + (int64_t)r * kDirEntry + 16);
    d[0] = ca;
    d[1] = cb;
  }
}

// ---- checksum of the fixed part ----------------------------------------------

// Partial checksums of the words [0, chunks_off / 4) of a container (the
// header's checksum field counts as zero), one contiguous range per
// workgroup; k_csum_final sums them.
constexpr int kCsumThreads = 256;

__global__ __launch_bounds__(kCsumThreads) void k_csum_part(const Params p0, int encode) {
  const Params p = at_seq(p0, blockIdx.z);
  const uint32_t* w32 = reinterpret_cast<const uint32_t*>(encode ? p.out_final : p.in);
  // 16-byte units (chunks_off is a multiple of 16), four in flight per thread
  const int64_t nq = p.chunks_off / 16;
  const int64_t per = (nq + kCsumParts - 1) / kCsumParts;
  const int64_t a = (int64_t)blockIdx.x * per, b = min(nq, a + per);
  const uint4* q4 = reinterpret_cast<const uint4*>(w32);
  uint64_t A = 0, B = 0;
  if (!encode && (uint64_t)p.cap < (uint64_t)p.chunks_off) {
    // a truncated container: k_dec_check reports it, nothing is read
  } else {
    for (int64_t q0 = a + threadIdx.x; q0 < b; q0 += 4 * kCsumThreads) {
      uint4 v[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int64_t q = q0 + k * kCsumThreads;
        v[k] = q < b ? q4[q] : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int64_t q = q0 + k * kCsumThreads;
        if (q >= b) continue;
        const uint32_t e[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int64_t j = 4 * q + c;
          const bool field = j >= kCsumField / 4 && j < kCsumField / 4 + 4;
          csum_add(A, B, (uint64_t)j, field ? 0u : e[c]);
        }
      }
    }
  }
  __shared__ uint64_t s_cs[32];
  csum_block_reduce(A, B, s_cs);
  if (threadIdx.x == 0) {
    uint64_t* out = reinterpret_cast<uint64_t*>(p.ws + p.w.csum) + 2 * blockIdx.x;
    out[0] = A;
    out[1] = B;
  }
}

// Encode: the sum of the partials into the header's checksum field.
// Decode: the sum against that field; a mismatch marks the container corrupt.
__global__ __launch_bounds__(kCsumThreads) void k_csum_final(const Params p0, int encode) {
  const Params p = at_seq(p0, blockIdx.z);
  const uint64_t* part = reinterpret_cast<const uint64_t*>(p.ws + p.w.csum);
  uint64_t A = 0, B = 0;
  for (int k = threadIdx.x; k < kCsumParts; k += kCsumThreads) {
    A = mod61(A + part[2 * k]);
    B = mod61(B + part[2 * k + 1]);
  }
  __shared__ uint64_t s_cs[32];
  csum_block_reduce(A, B, s_cs);
  if (threadIdx.x != 0) return;
  if (encode) {
    if (get_status(p.ws, p.w) & ((1u << KVTC_ERR_CAPACITY) | (1u << KVTC_ERR_NONFINITE))) return;
    uint64_t* f = reinterpret_cast<uint64_t*>(p.out_final + kCsumField);
    f[0] = A;
    f[1] = B;
  } else {
    if ((uint64_t)p.cap < (uint64_t)p.chunks_off) return;
    const uint64_t* f = reinterpret_cast<const uint64_t*>(p.in + kCsumField);
    if (f[0] != A || f[1] != B) set_status(p.ws, p.w, KVTC_ERR_CORRUPT);
  }
}

hipError_t launch_csum(const Params& p, int encode, hipStream_t s) {
  hipLaunchKernelGGL(k_csum_part, dim3(kCsumParts, 1, seq_grid(p)), dim3(kCsumThreads), 0, s, p, encode);
  hipLaunchKernelGGL(k_csum_final, dim3(1, 1, seq_grid(p)), dim3(kCsumThreads), 0, s, p, encode);
  return hipGetLastError();
}

hipError_t launch_assemble(const Params& p, const uint8_t* hdr, hipStream_t s) {
  HeaderBytes h;
  memcpy(h.b, hdr, kHeaderBytes);
  if (p.n_seqs == 0 && p.n_recs > 0 && p.n_recs <= 2048) {
    // one launch: offsets (each workgroup sums at most 2047 sizes), directory,
    // header and records
    hipLaunchKernelGGL(k_copy_records, dim3(p.n_recs), dim3(64 * kCopyWaves), 0, s, p, h, 1);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_scan, dim3(1, 1, seq_grid(p)), dim3(1024), 0, s, p, h);
  if (p.n_seqs > 0) {
    // place the sequences, then move each one's staged fixed part and records
    const hipError_t e = launch_batch_place(p, s);
    if (e != hipSuccess) return e;
  }
  if (p.n_recs > 0)
    hipLaunchKernelGGL(k_copy_records, dim3(p.n_recs, 1, seq_grid(p)), dim3(64 * kCopyWaves), 0, s, p, h, 0);
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
  } else if (tid < kHeaderBytes / 4 && tid != 42 && tid != 43 && (tid < kCsumField / 4 || tid >= kCsumField / 4 + 4)) {
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

constexpr int kRing = 512;  // words of a stream's LDS ring
constexpr int kUnit = 256;  // words per refill

template <bool B>
struct BoolTag {
  static constexpr bool value = B;
};

// Decoder slot table of one component: entry s describes the symbol whose
// cumulative range holds slot s -- its frequency f (bits 16..28), the symbol
// (bits 12..15) and s minus the range's start (bits 0..11) -- so that one
// LDS read per step gives x <- f (x >> sb) + offset and the symbol.
__device__ __forceinline__ uint32_t slot_entry(uint32_t f, uint32_t sy, uint32_t off) {
  return (f << 16) | (sy << 12) | off;
}

// Fills tab[0, M) from a component's cumulative frequencies cm[0..16]
// (entries past the alphabet hold M; cm is non-decreasing and ends at M), 8
// consecutive slots per thread: the last symbol whose range starts at or
// before the first slot (binary search), then a walk over the run.
__device__ __forceinline__ void build_slot_table(const uint32_t* cm, uint32_t M, uint32_t* tab, uint32_t tid,
                                                 uint32_t nthreads) {
  for (uint32_t s0 = tid * 8u; s0 < M; s0 += nthreads * 8u) {
    uint32_t sy = 0;
    sy += cm[sy + 8] <= s0 ? 8u : 0u;
    sy += cm[sy + 4] <= s0 ? 4u : 0u;
    sy += cm[sy + 2] <= s0 ? 2u : 0u;
    sy += cm[sy + 1] <= s0 ? 1u : 0u;
    uint32_t c0 = cm[sy], c1 = cm[sy + 1];
    uint32_t e[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const uint32_t sl = s0 + (uint32_t)q;
      while (c1 <= sl) {
        ++sy;
        c0 = c1;
        c1 = cm[sy + 1];
      }
      e[q] = slot_entry(c1 - c0, sy, sl - c0);
    }
    uint4* dst = reinterpret_cast<uint4*>(tab + s0);
    dst[0] = make_uint4(e[0], e[1], e[2], e[3]);
    dst[1] = make_uint4(e[4], e[5], e[6], e[7]);
  }
}

// raw_runs > 0 (contiguous cache): workgroups past the chunks copy the raw
// sink and recent runs of the container to the outputs, which costs the
// bandwidth this latency-bound pass leaves idle.
//
// The workgroup walks the coded components in lockstep: while its streams
// decode component ci with ci's slot table, every thread helps build the
// table of ci + 1 in the other buffer, and a barrier ends the component.
// BIG: workgroups of more than 768 threads (more than 24 tiles per record);
// otherwise two workgroups of up to 12 waves share a CU: six waves per SIMD,
// which caps the registers at 80.
template <int LANES, int STEPS, bool BIG>
__global__ __launch_bounds__(BIG ? 1024 : 768, BIG ? 4 : 6) void k_rans_dec_recs(const Params p0, int raw_runs) {
  constexpr int SPW = 64 / LANES;
  constexpr int NR = 32 / LANES + 1;  // staged raw-row words per lane
  const Params p = at_seq(p0, blockIdx.z);
  const int r = blockIdx.x;
  if (r >= p.n_recs) {
    if (r - p.n_recs < raw_runs) copy_raw_run(p, r - p.n_recs, 0, false);
    return;
  }
  const int u = r / p.recs_per_sec, cr = r % p.recs_per_sec;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (get_status(p.ws, p.w) & (1u << KVTC_ERR_CORRUPT)) return;
  __shared__ RecGeo g;
  __shared__ uint32_t cumt[kMaxD * 17];
  __shared__ int32_t s_toff[kMaxTilesPerRec];
  __shared__ int s_ok;
  __shared__ uint32_t outbuf[kMaxTilesPerRec][kRowWords];
  __shared__ uint32_t rawbuf[kMaxTilesPerRec][2][kRawWords];
  // dynamic: one word ring per tile (kRing u16), then two slot tables of 2^sb u32
  extern __shared__ __align__(16) uint8_t dyn[];
  uint16_t* rings = reinterpret_cast<uint16_t*>(dyn);
  uint32_t* stab = reinterpret_cast<uint32_t*>(dyn + (size_t)p.tiles_per_rec * kRing * 2);
  if (wave == 0) rec_setup(p, cr, p.in + p.side_off + (int64_t)u * 9 * p.D, g);
  __syncthreads();
  const uint8_t* dir = p.in + p.dir_off + (int64_t)r * kDirEntry;
  const uint64_t off = *reinterpret_cast<const uint64_t*>(dir);
  const uint32_t size = *reinterpret_cast<const uint32_t*>(dir + 8);
  const uint32_t mode = *reinterpret_cast<const uint32_t*>(dir + 12);
  const uint64_t total = *reinterpret_cast<const uint64_t*>(p.in + 168);
  const uint8_t* rec = p.in + off;
  const int ntiles = g.ntiles, nc = g.nc;
  if (wave == 0) {
    // the section's widths: each no more than max_bits (and the uniform width
    // on the WHT path), their sum within the budget; then the directory entry
    // against the record's geometry
    const int s = (u / p.H) & 1;
    bool okl = true;
    for (int i = lane; i < p.D; i += 64) {
      const int b = g.b[i];
      if (b > p.max_bits) okl = false;
      if (p.transform == KVTC_WHT && b != (s == 0 ? p.bits_k_uniform : p.bits_v_uniform)) okl = false;
    }
    bool ok = __ballot(!okl) == 0ull;
    if (p.transform == KVTC_PCA && g.sum_b > (p.alloc_scope == 1 ? p.sec_bits_max : (s == 0 ? p.budget_k : p.budget_v)))
      ok = false;
    if (ok && mode > 1) ok = false;
    if (ok && g.P == 0 && (size != 0 || mode != 0)) ok = false;
    if (ok && g.P > 0 && (off < (uint64_t)p.chunks_off || (off & 15) || off > total || size > total - off)) ok = false;
    if (ok && g.P > 0 && mode == 1 && (int64_t)size != align16(g.P)) ok = false;
    if (ok && g.P > 0 && mode == 0 && size < (uint32_t)(g.tb + 4 * ntiles)) ok = false;
    // stream pieces inside a coded record (a prefix sum over its tiles)
    int64_t piece = 0;
    if (ok && g.P > 0 && mode == 0 && lane < ntiles) {
      const uint32_t nw = reinterpret_cast<const uint32_t*>(rec + g.tb)[lane];
      piece = 4 * (int64_t)LANES + 2 * (int64_t)nw + ((nw & 1) ? 2 : 0) + (lane == ntiles - 1 ? g.rl : g.rf);
    }
    int64_t xs = piece;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int64_t y = __shfl_up(xs, o, 64);
      if (lane >= o) xs += y;
    }
    const int64_t base = g.tb + 4 * (int64_t)ntiles;
    if (ok && g.P > 0 && mode == 0 && align16(base + __shfl(xs, 63, 64)) != (int64_t)size) ok = false;
    if (lane < ntiles) s_toff[lane] = (int32_t)(base + xs - piece);
    if (lane == 0) s_ok = ok ? 1 : 0;
  }
  __syncthreads();
  if (!s_ok) {
    if (tid == 0) set_status(p.ws, p.w, KVTC_ERR_CORRUPT);
    return;
  }
  // The record against its directory checksum (its range was checked
  // above).  Threads add 16-byte units [q0, q1) of the record to their
  // partial sums -- at once on the short paths, after the decode on the coded
  // path -- and the block total is compared; a mismatch marks the container
  // corrupt (the decode of a damaged record stays in bounds).
  const uint4* r4 = reinterpret_cast<const uint4*>(rec);
  const uint32_t nq = size / 16;
  uint64_t csA = 0, csB = 0;
  auto csum_units = [&](uint32_t q0, uint32_t q1, uint32_t t, uint32_t nt) {
    for (uint32_t q = q0 + t; q < q1; q += nt) {
      const uint4 v = r4[q];
      const uint64_t j = 4ull * q;
      csum_add(csA, csB, j, v.x);
      csum_add(csA, csB, j + 1, v.y);
      csum_add(csA, csB, j + 2, v.z);
      csum_add(csA, csB, j + 3, v.w);
    }
  };
  auto verify_record = [&]() {
    __shared__ uint64_t s_cs[32];
    csum_block_reduce(csA, csB, s_cs);
    if (tid == 0) {
      const uint64_t* d = reinterpret_cast<const uint64_t*>(dir + 16);
      if (d[0] != csA || d[1] != csB) set_status(p.ws, p.w, KVTC_ERR_CORRUPT);
    }
  };
  if (g.P == 0) {
    csum_units(0, nq, tid, blockDim.x);
    verify_record();
    return;
  }
  if (mode == 1) {  // the packed rows themselves
    int64_t at = 0;
    for (int t = 0; t < ntiles; ++t) {
      const int32_t pt = t == ntiles - 1 ? g.pl : g.pf;
      const uint32_t* src = reinterpret_cast<const uint32_t*>(rec + at);
      uint32_t* dst = reinterpret_cast<uint32_t*>(packed_tile(p, u, cr, t, g.pf));
      for (int i = tid; i < pt / 4; i += blockDim.x) dst[i] = src[i];
      at += pt;
    }
    csum_units(0, nq, tid, blockDim.x);
    verify_record();
    return;
  }
  // tables -> cumulative frequencies (entries past the alphabet hold M, so
  // every search stops inside the alphabet); each table must sum to M
  const uint32_t M = 1u << p.sb;
  for (int ci = tid; ci < nc; ci += blockDim.x) {
    const int i = g.coded[ci];
    const int A = 1 << sym_bits_of((int)g.b[i]);
    const uint16_t* ft = reinterpret_cast<const uint16_t*>(rec) + g.toff[i];
    uint32_t c = 0;
    for (int s = 0; s < 16; ++s) {
      cumt[ci * 17 + s] = s < A ? c : M;
      if (s < A) c += ft[s];
    }
    cumt[ci * 17 + 16] = M;
    if (c != M) atomicOr(&s_ok, 2);
  }
  __syncthreads();
  if (s_ok != 1) {
    if (tid == 0) set_status(p.ws, p.w, KVTC_ERR_CORRUPT);
    return;
  }
  // waves past the streams' (when the launch adds them) build the slot
  // tables of the components ahead while the streams decode; without them
  // every thread builds
  const int stream_waves = (p.tiles_per_rec * LANES + 63) / 64;
  const bool builders = (int)(blockDim.x >> 6) > stream_waves;
  const uint32_t btid = builders ? (uint32_t)(tid - 64 * stream_waves) : (uint32_t)tid;
  const uint32_t bthreads = builders ? blockDim.x - 64u * stream_waves : blockDim.x;
  const bool builds = !builders || wave >= stream_waves;
  if (nc > 0) build_slot_table(cumt, M, stab, tid, blockDim.x);
  const int grp = lane / LANES, j = lane % LANES;
  const int t = wave * SPW + grp;
  const bool valid = t < ntiles;
  const bool last = valid && t == ntiles - 1;
  const int m = !valid ? 0 : (last ? g.n_last : p.tile_tokens);
  const int tt = valid ? t : 0;
  const bool has_stream = wave * SPW < ntiles;  // wave-uniform
  uint32_t* tbase = reinterpret_cast<uint32_t*>(packed_tile(p, u, cr, tt, g.pf));
  const uint8_t* piece = rec + s_toff[tt];
  const uint32_t nw = reinterpret_cast<const uint32_t*>(rec + g.tb)[tt];
  const uint32_t* raws = reinterpret_cast<const uint32_t*>(piece + 4 * LANES + 2 * (int64_t)nw + ((nw & 1) ? 2 : 0));
  // the record (raw rows) and its packed tiles (the rows this kernel
  // writes) through buffer resources, so that lanes past a row load zeros and
  // drop their stores without a branch
  const __amdgpu_buffer_rsrc_t rrsrc = uniform_rsrc(const_cast<uint8_t*>(rec), (int32_t)size);
  const int32_t raws_at = (int32_t)(reinterpret_cast<const uint8_t*>(raws) - rec);
  const int32_t prec_bytes = (int32_t)((int64_t)p.blks_per_rec * p.w.packed_slot);
  const __amdgpu_buffer_rsrc_t prsrc = uniform_rsrc(packed_tile(p, u, cr, 0, g.pf), prec_bytes);
  const int32_t tile_at = (int32_t)((int64_t)(tt / p.tiles_per_blk) * p.w.packed_slot + (int64_t)(tt % p.tiles_per_blk) * g.pf);
  // 1-bit components: the raw row is the packed row; eight words per lane
  // in flight at a time
  if (valid && g.n1 > 0) {
    const int W1 = (m + 31) >> 5;
    const int n1w = g.n1 * W1;
    for (int q0 = 0; q0 < n1w; q0 += 8 * LANES) {
      uint32_t v[8];
      int32_t dat[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int e = q0 + q * LANES + j;
        const int c1 = e / W1, w = e - c1 * W1;
        const int i = e < n1w ? g.raw1[c1] : 0;
        v[q] = __builtin_amdgcn_raw_buffer_load_b32(rrsrc, e < n1w ? raws_at + 4 * ((int32_t)g.raoff[last][i] + w) : (int32_t)size, 0, 0);
        dat[q] = e < n1w ? tile_at + 4 * ((int32_t)g.roff[last][i] + w) : prec_bytes;
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) __builtin_amdgcn_raw_buffer_store_b32(v[q], prsrc, dat[q], 0, 0);
    }
  }
  // -- streams
  const uint64_t gm = ((1ull << LANES) - 1ull) << (grp * LANES);
  const uint32_t gm_lo = (uint32_t)gm, gm_hi = (uint32_t)(gm >> 32);
  const uint32_t* states = reinterpret_cast<const uint32_t*>(piece);
  const uint16_t* words = reinterpret_cast<const uint16_t*>(piece + 4 * LANES);
  const uint32_t* wd = reinterpret_cast<const uint32_t*>(words);  // word pairs (4-byte aligned)
  uint16_t* ring = rings + tt * kRing;
  uint32_t* ring32 = reinterpret_cast<uint32_t*>(ring);
  uint32_t x = valid ? states[j] : kRansL;
  const bool bad0 = valid && x < kRansL;
  const int32_t nwi = valid ? (int32_t)nw : 0;
  int32_t ptr = nwi;
  // committed words [clo, nw) (clo a multiple of 8), pending words [plo, clo)
  int32_t clo = max(0, (nwi - kRing + 7) & ~7);
  if (valid) {
    for (int32_t q = clo / 2 + j; 2 * q < nwi; q += LANES)
      ring32[q & (kRing / 2 - 1)] = (2 * q + 1 < nwi) ? wd[q] : (uint32_t)words[2 * q];
  }
  int32_t plo = max(0, clo - kUnit);
  constexpr int PER = kUnit / 2 / LANES;
  uint32_t pend[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int32_t q = plo / 2 + j + LANES * k;
    pend[k] = (valid && q < clo / 2) ? wd[q] : 0u;
  }
  int steps_max = (m + LANES - 1) / LANES;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) steps_max = max(steps_max, __shfl_xor(steps_max, o, 64));
  steps_max = STEPS > 0 ? STEPS : __builtin_amdgcn_readfirstlane(steps_max);
  // every step of both of the wave's streams codes a token (full tiles):
  // the step loop then carries no activity masks
  const bool wave_full = STEPS > 0 && __all(valid && m == STEPS * LANES);
  uint32_t* ob = &outbuf[tt][0];
  uint32_t* rbb = &rawbuf[tt][0][0];
  if (valid)
    for (int w = j; w < kRowWords; w += LANES) ob[w] = 0u;
  // the raw row of component i of this tile: registers, then LDS.  Two
  // register sets alternate between even and odd components, so a row is
  // loaded two components before its use and the load's latency hides
  // behind a whole component.
  uint32_t rpre0[NR], rpre1[NR];
  auto raw_load = [&](uint32_t(&rp)[NR], int i) {
    const uint32_t rr = (uint32_t)raw_bits_of((int)g.b[i]);
    const int Wr = rr ? (m * (int)rr + 31) >> 5 : 0;
    const int32_t at = raws_at + 4 * (int32_t)g.raoff[last][i];
#pragma unroll
    for (int q = 0; q < NR; ++q) {
      const int w = j + q * LANES;
      rp[q] = __builtin_amdgcn_raw_buffer_load_b32(rrsrc, (valid && w < Wr) ? at + 4 * w : (int32_t)size, 0, 0);
    }
  };
  auto raw_store = [&](const uint32_t(&rp)[NR], int which) {
#pragma unroll
    for (int q = 0; q < NR; ++q) {
      const int w = j + q * LANES;
      if (valid && w < kRawWords) rbb[which * kRawWords + w] = rp[q];
    }
  };
  if (has_stream) {
    if (nc > 0) raw_load(rpre0, g.coded[0]);
    if (nc > 1) raw_load(rpre1, g.coded[1]);
  }
  __syncthreads();  // slot table 0 and the rings are complete
  const uint32_t sb = (uint32_t)p.sb;
  // one component of both streams: STEPS (or steps_max) steps, the codes
  // OR-ed into the LDS row buffer at bit (k b) of token k = s LANES + j
  auto decode_component = [&](auto full_tag, auto straddle_tag, const uint32_t* tab, uint32_t b, uint32_t rr,
                              const uint32_t* rw) {
    constexpr bool FULL = decltype(full_tag)::value;
    constexpr bool STRADDLES = decltype(straddle_tag)::value;  // widths 3, 5, 6, 7: a code may cross a word
    // bit position of token k = s LANES + j: j b + s LANES b; with 32 lanes a
    // step is b whole words, so the shift is the same at every step
    const uint32_t jb = (uint32_t)j * b, jr = (uint32_t)j * rr;
    const uint32_t sh0 = jb & 31u;
    // the raw low bits of every step do not depend on the state: read first
    constexpr int NS = STEPS > 0 ? STEPS : 16;
    uint32_t rlow[NS];
    {
      const uint32_t rmask = (1u << rr) - 1u;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        if (s >= (STEPS > 0 ? STEPS : steps_max)) break;
        const uint32_t bq = jr + (uint32_t)(s * LANES) * rr;
        rlow[s] = rr ? (funnel(rw[bq >> 5], rw[(bq >> 5) + 1], bq & 31u) & rmask) : 0u;
      }
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (s >= (STEPS > 0 ? STEPS : steps_max)) break;
      const bool active = FULL || (valid && s * LANES + j < m);
      const uint32_t e = tab[x & (M - 1u)];
      const uint32_t xn = __umul24(e >> 16, x >> sb) + (e & 0xfffu);
      x = active ? xn : x;
      const bool need = active && x < kRansL;
      const uint64_t bl = __builtin_amdgcn_ballot_w64(need);
      const uint32_t mlo = (uint32_t)bl & gm_lo, mhi = (uint32_t)(bl >> 32) & gm_hi;
      const uint32_t rank = __builtin_amdgcn_mbcnt_hi(mhi, __builtin_amdgcn_mbcnt_lo(mlo, 0u));
      const uint32_t wnext = ring[(uint32_t)(ptr - 1 - (int32_t)rank) & (kRing - 1)];
      x = need ? ((x << 16) | wnext) : x;
      ptr -= (int32_t)(__popc(mlo) + __popc(mhi));
      uint32_t code = (((e >> 12) & 15u) << rr) | rlow[s];
      if (!FULL) code = active ? code : 0u;
      const uint32_t bp = jb + (uint32_t)(s * LANES) * b;
      const uint32_t sh = LANES == 32 ? sh0 : (bp & 31u);
      uint32_t* ow = LANES == 32 ? ob + (jb >> 5) + s * b : ob + (bp >> 5);
      const uint64_t c64 = (uint64_t)code << sh;  // the high word holds what crosses into the next word
      if constexpr (!STRADDLES) {
        // widths 2, 4, 8: a word holds the codes of an aligned run of 32 / b
        // lanes of one step, so the run ORs its codes across lanes and its
        // first lane stores the word (no atomics on the state's critical path)
        uint32_t v = (uint32_t)c64;
        v |= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);  // lane ^ 1
        v |= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);  // lane ^ 2
        if (b <= 4u) v |= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false);  // 7 - lane % 8
        if (b <= 2u) v |= (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false);  // 15 - lane % 16
        if (valid && (j & ((32u / b) - 1u)) == 0u) *ow = v;
      } else {
        atomicOr(ow, (uint32_t)c64);
        const uint32_t hi = (uint32_t)(c64 >> 32);
        if (hi) atomicOr(ow + 1, hi);  // only lanes whose code crosses the word
      }
    }
  };
  auto component = [&](int ci, uint32_t(&rp)[NR]) {
    if (ci + 1 < nc && builds) build_slot_table(cumt + (ci + 1) * 17, M, stab + ((ci + 1) & 1) * M, btid, bthreads);
    if (has_stream) {
      const int i = g.coded[ci];
      const uint32_t b = __builtin_amdgcn_readfirstlane((uint32_t)g.b[i]);
      const uint32_t rr = b - (uint32_t)sym_bits_of((int)b);
      // this component's raw row to LDS (its buffer was last read two
      // components ago), then the row of ci + 2 into the same registers
      raw_store(rp, ci & 1);
      if (ci + 2 < nc) raw_load(rp, g.coded[ci + 2]);
      // A component takes at most tile_tokens <= kUnit words, so one refill test
      // per component keeps the ring ahead: after a refill at least kUnit
      // committed words remain unread.
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
      __builtin_amdgcn_wave_barrier();
      const uint32_t* tab = stab + (ci & 1) * M;
      const uint32_t* rw = rbb + (ci & 1) * kRawWords;
      const bool straddles = (b & (b - 1u)) != 0u;
      if (wave_full) {
        if (straddles) decode_component(BoolTag<true>{}, BoolTag<true>{}, tab, b, rr, rw);
        else decode_component(BoolTag<true>{}, BoolTag<false>{}, tab, b, rr, rw);
      } else {
        if (straddles) decode_component(BoolTag<false>{}, BoolTag<true>{}, tab, b, rr, rw);
        else decode_component(BoolTag<false>{}, BoolTag<false>{}, tab, b, rr, rw);
      }
      // the component's packed row is flushed and the buffer cleared
      __builtin_amdgcn_wave_barrier();
      const int W = (m * (int)b + 31) >> 5;
      const int32_t at = tile_at + 4 * (int32_t)g.roff[last][i];
#pragma unroll
      for (int q = 0; q < (kRowWords + LANES - 1) / LANES; ++q) {
        const int w = j + q * LANES;
        const uint32_t v = w < kRowWords ? ob[w] : 0u;
        __builtin_amdgcn_raw_buffer_store_b32(v, prsrc, (valid && w < W) ? at + 4 * w : prec_bytes, 0, 0);
        if (valid && w < kRowWords) ob[w] = 0u;
      }
    }
    __syncthreads();  // table ci + 1 is complete; table ci may be rebuilt
  };
  for (int ci = 0; ci < nc; ci += 2) {
    component(ci, rpre0);
    if (ci + 1 < nc) component(ci + 1, rpre1);
  }
  const bool ok = !(bad0 || (valid && (x != kRansL || ptr != 0)));
  if (has_stream && __ballot(!ok)) {
    if (lane == 0) set_status(p.ws, p.w, KVTC_ERR_CORRUPT);
  }
  // the record's checksum by the table-building waves (by every thread
  // when the launch has none); the streams meet them in the reduction
  if (builds) csum_units(0, nq, btid, bthreads);
  verify_record();
}

hipError_t launch_rans_decode_chunks(const Params& p, hipStream_t s, bool with_raw) {
  int waves = (p.tiles_per_rec * p.lanes + 63) / 64;
  if (waves < 1) waves = 1;
  // plus table-building waves, half as many as the streams' (within 16)
  waves += std::min(std::max(waves / 2, 1), 16 - waves);
  // one word ring per tile, then two slot tables
  const size_t lds = (size_t)p.tiles_per_rec * kRing * 2 + 2 * ((size_t)4 << p.sb);
  const int raw_runs = with_raw && p.n_seqs == 0 ? 4 * p.L * p.H : 0;
  const dim3 grid(p.n_recs + raw_runs, 1, seq_grid(p)), block(64 * waves);
  const int steps = p.tile_tokens / p.lanes;
  if (64 * waves > 768) {
    if (p.lanes == 16) hipLaunchKernelGGL((k_rans_dec_recs<16, 0, true>), grid, block, lds, s, p, raw_runs);
    else hipLaunchKernelGGL((k_rans_dec_recs<32, 0, true>), grid, block, lds, s, p, raw_runs);
  } else if (p.lanes == 16) {
    if (steps == 16) hipLaunchKernelGGL((k_rans_dec_recs<16, 16, false>), grid, block, lds, s, p, raw_runs);
    else if (steps == 8) hipLaunchKernelGGL((k_rans_dec_recs<16, 8, false>), grid, block, lds, s, p, raw_runs);
    else hipLaunchKernelGGL((k_rans_dec_recs<16, 0, false>), grid, block, lds, s, p, raw_runs);
  } else {
    if (steps == 8) hipLaunchKernelGGL((k_rans_dec_recs<32, 8, false>), grid, block, lds, s, p, raw_runs);
    else if (steps == 4) hipLaunchKernelGGL((k_rans_dec_recs<32, 4, false>), grid, block, lds, s, p, raw_runs);
    else hipLaunchKernelGGL((k_rans_dec_recs<32, 0, false>), grid, block, lds, s, p, raw_runs);
  }
  return hipGetLastError();
}

// ---- parity hooks -----------------------------------------------------------

// n tables of up to 16 counts each (stride 16) -> frequencies with the
// record encoder's normaliser.
__global__ void k_test_freq_tables(const uint32_t* counts, const int32_t* alpha, int n, int sb, uint16_t* freq) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  uint32_t c[16], f[16];
  int A = alpha[i];
  A = A < 1 ? 1 : (A > 16 ? 16 : A);
  for (int s = 0; s < 16; ++s) c[s] = s < A ? counts[16 * i + s] : 0u;
  normalize_small(c, A, sb, f);
  for (int s = 0; s < 16; ++s) freq[16 * i + s] = s < A ? (uint16_t)f[s] : 0;
}

hipError_t launch_test_freq_tables(const uint32_t* counts, const int32_t* alpha, int n, int sb, uint16_t* freq,
                                   hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_test_freq_tables, dim3((n + 63) / 64), dim3(64), 0, s, counts, alpha, n, sb, freq);
  return hipGetLastError();
}

}  // namespace kvtc
