// C ABI of libkvtc: configuration checks, plans, workspace sizing and the
// launch sequences of encode and decode.  Kernels live in kernels_*.hip.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <new>

#include "kvtc_internal.h"

using namespace kvtc;

#define HIP_TRY(x)                         \
  do {                                     \
    hipError_t e_ = (x);                   \
    if (e_ != hipSuccess) return KVTC_ERR_HIP; \
  } while (0)

namespace kvtc {

// Worst-case container: the fixed part plus every record at its packed size
// (a record never exceeds the packed form of its chunk, rounded to 16 bytes).
int64_t max_container_bytes(const kvtc_config& c, const Layout& lo) {
  int64_t total = lo.chunks_off;
  if (lo.recs_per_sec == 0) return total;
  for (int s = 0; s < 2; ++s) {
    int32_t budget = c.alloc_scope == 1 ? lo.sec_bits_max : (s == 0 ? lo.budget_k : lo.budget_v);
    int64_t per_rec[2] = {0, 0};
    for (int which = 0; which < 2; ++which) {
      int32_t n = which == 0 ? lo.rec_tokens : lo.T_mid - (lo.recs_per_sec - 1) * lo.rec_tokens;
      int64_t P = 0;
      for (int32_t a = 0; a < n; a += c.tile_tokens) {
        int32_t m = n - a < c.tile_tokens ? n - a : c.tile_tokens;
        P += max_tile_bytes(c, m, budget);
      }
      per_rec[which] = align16(P);
    }
    int64_t secs = (int64_t)c.layers * c.kv_heads;
    total += secs * ((lo.recs_per_sec - 1) * per_rec[0] + per_rec[1]);
  }
  return total;
}

Params make_params(const PlanImpl& pl, const Layout& lo, const WsLayout& w) {
  const kvtc_config& c = pl.cfg;
  Params p{};
  p.L = c.layers; p.H = c.kv_heads; p.D = c.head_dim; p.dtype = c.dtype;
  p.transform = c.transform; p.rope_keys = c.rope_keys; p.rope_style = c.rope_style;
  p.max_bits = c.max_bits; p.sb = c.rans_scale_bits; p.lanes = c.rans_lanes;
  p.blk_tokens = lo.blk_tokens; p.tile_tokens = c.tile_tokens;
  p.rec_tokens = lo.rec_tokens; p.recs_per_sec = lo.recs_per_sec; p.n_recs = lo.n_recs;
  p.tiles_per_rec = lo.tiles_per_rec; p.blks_per_rec = lo.blks_per_rec;
  p.basis_per_head = c.basis_per_head; p.wht_keys = c.wht_keys;
  p.budget_k = lo.budget_k; p.budget_v = lo.budget_v;
  p.sec_bits_max = lo.sec_bits_max; p.alloc_scope = c.alloc_scope; p.total_budget = lo.total_budget;
  p.T = lo.T; p.s0 = lo.s0; p.mid_begin = lo.mid_begin; p.mid_end = lo.mid_end;
  p.T_mid = lo.T_mid; p.W_eff = lo.W_eff; p.n_sections = lo.n_sections;
  p.blks_per_sec = lo.blks_per_sec; p.n_blks = lo.n_blks;
  p.tiles_per_blk = lo.tiles_per_blk;
  p.bits_k_uniform = floor_bits(c.bits_k); p.bits_v_uniform = floor_bits(c.bits_v);
  p.side_off = lo.side_off; p.r_off = lo.r_off; p.raw_off = lo.raw_off;
  p.raw_bytes = lo.raw_bytes; p.dir_off = lo.dir_off; p.chunks_off = lo.chunks_off;
  p.basis_t = pl.basis_t; p.basis = pl.basis; p.rope = pl.rope;
  // fp32 MFMA accumulation of D exact bf16 products (four chained 32-deep
  // steps) has measured up to 9.2 * 2^-24 * sum|x_j B_ji|; 24 (bf16) and 64
  // (fp32 operands, whose products round too) leave margin, and
  // sum|x_j B_ji| <= ||x||_2 ||B_i||_2 bounds the sum by the token norm
  p.mfma_err = (c.dtype == KVTC_BF16 ? 24.0f : 64.0f) * 0x1p-24f * pl.max_col_norm;
  p.w = w;
  p.cfg = c;
  return p;
}

static void put32(uint8_t* p, uint32_t v) { memcpy(p, &v, 4); }
static void put64(uint8_t* p, uint64_t v) { memcpy(p, &v, 8); }

// Fixed 256-byte header (all fields little-endian); the total size at byte
// 168 is filled in on the device once the chunk sizes are known.
void build_header(const PlanImpl& pl, const Layout& lo, uint8_t* h) {
  const kvtc_config& c = pl.cfg;
  memset(h, 0, kHeaderBytes);
  memcpy(h, "KVTC", 4);
  put32(h + 4, kContainerVersion);
  put32(h + 8, kHeaderBytes);
  put32(h + 16, c.layers); put32(h + 20, c.kv_heads); put32(h + 24, c.head_dim);
  put32(h + 28, c.dtype); put32(h + 32, c.transform);
  put32(h + 36, c.sink_tokens); put32(h + 40, c.recent_tokens);
  memcpy(h + 44, &c.bits_k, 4); memcpy(h + 48, &c.bits_v, 4);
  put32(h + 52, c.max_bits); put32(h + 56, c.rope_keys); put32(h + 60, c.rope_style);
  memcpy(h + 64, &c.rope_theta, 8);
  put32(h + 72, c.rans_scale_bits); put32(h + 76, c.rans_lanes);
  put32(h + 80, c.chunk_tokens); put32(h + 84, c.tile_tokens);
  put32(h + 88, c.basis_per_head); put32(h + 92, c.wht_keys);
  put32(h + 96, lo.T); put32(h + 100, lo.s0); put32(h + 104, lo.mid_begin);
  put32(h + 108, lo.mid_end); put32(h + 112, lo.n_sections); put32(h + 116, lo.recs_per_sec);
  put64(h + 120, lo.side_off); put64(h + 128, lo.side_bytes); put64(h + 136, lo.raw_off);
  put64(h + 144, lo.raw_bytes); put64(h + 152, lo.dir_off); put64(h + 160, lo.chunks_off);
  put64(h + 176, pl.fingerprint);
  put32(h + 184, lo.budget_k); put32(h + 188, lo.budget_v);
  put32(h + 192, c.alloc_scope);
}

}  // namespace kvtc

// ---------------------------------------------------------------------------

static kvtc_status check_config(const kvtc_config* c) {
  if (!c) return KVTC_ERR_INVALID_ARG;
  if (c->layers < 1 || c->kv_heads < 1 || c->max_tokens < 1) return KVTC_ERR_INVALID_ARG;
  if (c->head_dim != 64 && c->head_dim != 128) return KVTC_ERR_UNSUPPORTED;
  if (c->dtype != KVTC_BF16 && c->dtype != KVTC_FP32) return KVTC_ERR_INVALID_ARG;
  if (c->transform != KVTC_PCA && c->transform != KVTC_WHT) return KVTC_ERR_INVALID_ARG;
  if (c->transform == KVTC_PCA && c->dtype == KVTC_FP32 && c->head_dim != 64)
    return KVTC_ERR_UNSUPPORTED;  // fp32 MFMA operands: the basis is register-resident
  if (c->transform == KVTC_WHT && c->head_dim != 128)
    return KVTC_ERR_UNSUPPORTED;  // the WHT kernels run 16 lanes x 8 components per token
  if (c->sink_tokens < 0 || c->recent_tokens < 0) return KVTC_ERR_INVALID_ARG;
  if (c->max_bits < 1 || c->max_bits > 8) return KVTC_ERR_INVALID_ARG;
  if (!(c->bits_k >= 0.0f) || !(c->bits_v >= 0.0f)) return KVTC_ERR_INVALID_ARG;
  if (c->bits_k > (float)c->max_bits || c->bits_v > (float)c->max_bits) return KVTC_ERR_INVALID_ARG;
  if (c->transform == KVTC_WHT && (c->bits_k < 2.0f || c->bits_v < 1.0f)) return KVTC_ERR_INVALID_ARG;
  if (c->rope_style != KVTC_ROPE_HALF && c->rope_style != KVTC_ROPE_INTERLEAVED)
    return KVTC_ERR_INVALID_ARG;
  if (c->rope_keys != 0 && c->rope_keys != 1) return KVTC_ERR_INVALID_ARG;
  if (c->rope_keys && !(c->rope_theta > 1.0)) return KVTC_ERR_INVALID_ARG;
  if (c->rans_scale_bits < 8 || c->rans_scale_bits > 12) return KVTC_ERR_UNSUPPORTED;
  if (c->rans_lanes != 16 && c->rans_lanes != 32) return KVTC_ERR_UNSUPPORTED;
  if (c->tile_tokens < 16 || c->tile_tokens > 256 || (c->tile_tokens % 16)) return KVTC_ERR_UNSUPPORTED;
  if (c->chunk_tokens < c->tile_tokens || (c->chunk_tokens % c->tile_tokens)) return KVTC_ERR_INVALID_ARG;
  // longer chunks split into work blocks of kBlkTokens tokens, whole tiles each
  if (c->chunk_tokens > kBlkTokens && ((c->chunk_tokens % kBlkTokens) || (kBlkTokens % c->tile_tokens)))
    return KVTC_ERR_UNSUPPORTED;
  if (c->chunk_tokens / c->tile_tokens > kMaxTilesPerRec) return KVTC_ERR_UNSUPPORTED;
  if (c->basis_per_head != 0 && c->basis_per_head != 1) return KVTC_ERR_INVALID_ARG;
  if (c->wht_keys != 0 && c->wht_keys != 1) return KVTC_ERR_INVALID_ARG;
  if (c->alloc_scope != 0 && c->alloc_scope != 1) return KVTC_ERR_INVALID_ARG;
  if (c->alloc_scope == 1 && c->transform != KVTC_PCA) return KVTC_ERR_INVALID_ARG;
  // one-budget keys carry the (section, component) index in 20 bits
  if (c->alloc_scope == 1 && (int64_t)c->layers * 2 * c->kv_heads * c->head_dim > (1 << 20))
    return KVTC_ERR_UNSUPPORTED;
  return KVTC_OK;
}

static size_t plan_layout(const kvtc_config& c, size_t* off_bt, size_t* off_b, size_t* off_rope) {
  size_t eb = c.dtype == KVTC_BF16 ? 2 : 4;
  size_t nb = c.transform == KVTC_PCA
                  ? (size_t)c.layers * 2 * (c.basis_per_head ? c.kv_heads : 1)
                  : 0;
  size_t bbytes = nb * c.head_dim * c.head_dim * eb;
  size_t at = 0;
  *off_bt = at; at += (bbytes + 255) & ~(size_t)255;
  *off_b = at; at += (bbytes + 255) & ~(size_t)255;
  *off_rope = at; at += (size_t)c.max_tokens * (c.head_dim / 2) * sizeof(float2);
  at = (at + 255) & ~(size_t)255;
  return at + 256;  // flag word used while the plan is built
}

// Phase markers for kvtc_profile_*: event i is recorded before phase i's
// launch, the last one after the final phase.
struct ProfScope {
  PlanImpl* pl;
  hipStream_t s;
  explicit ProfScope(PlanImpl* p, hipStream_t st) : pl(p), s(st) {
    if (pl && pl->prof_on) {
      pl->prof_n = 0;
      (void)hipEventRecord(pl->prof_ev[0], s);
      pl->prof_n = 1;
    }
  }
  void phase(const char* name) {
    if (!pl || !pl->prof_on || pl->prof_n >= 24) return;
    pl->prof_name[pl->prof_n - 1] = name;
    (void)hipEventRecord(pl->prof_ev[pl->prof_n], s);
    pl->prof_n += 1;
  }
};

extern "C" {

kvtc_status kvtc_profile_enable(kvtc_plan_t plan, int32_t on) {
  if (!plan) return KVTC_ERR_INVALID_ARG;
  PlanImpl* p = (PlanImpl*)plan;
  if (on && !p->prof_created) {
    for (int i = 0; i < 24; ++i)
      if (hipEventCreate(&p->prof_ev[i]) != hipSuccess) return KVTC_ERR_HIP;
    p->prof_created = 1;
  }
  p->prof_on = on ? 1 : 0;
  p->prof_n = 0;
  return KVTC_OK;
}

kvtc_status kvtc_profile_read(kvtc_plan_t plan, int32_t max_n, float* ms, const char** names,
                              int32_t* n) {
  if (!plan || !n) return KVTC_ERR_INVALID_ARG;
  PlanImpl* p = (PlanImpl*)plan;
  int32_t cnt = p->prof_n > 1 ? p->prof_n - 1 : 0;
  if (cnt > 0 && hipEventSynchronize(p->prof_ev[cnt]) != hipSuccess) return KVTC_ERR_HIP;
  for (int32_t i = 0; i < cnt && i < max_n; ++i) {
    float t = 0.f;
    if (hipEventElapsedTime(&t, p->prof_ev[i], p->prof_ev[i + 1]) != hipSuccess) return KVTC_ERR_HIP;
    if (ms) ms[i] = t;
    if (names) names[i] = p->prof_name[i];
  }
  *n = cnt;
  return KVTC_OK;
}

const char* kvtc_status_str(kvtc_status s) {
  switch (s) {
    case KVTC_OK: return "KVTC_OK";
    case KVTC_ERR_INVALID_ARG: return "KVTC_ERR_INVALID_ARG";
    case KVTC_ERR_UNSUPPORTED: return "KVTC_ERR_UNSUPPORTED";
    case KVTC_ERR_CAPACITY: return "KVTC_ERR_CAPACITY";
    case KVTC_ERR_CORRUPT: return "KVTC_ERR_CORRUPT";
    case KVTC_ERR_NONFINITE: return "KVTC_ERR_NONFINITE";
    case KVTC_ERR_HIP: return "KVTC_ERR_HIP";
  }
  return "KVTC_ERR_UNKNOWN";
}

kvtc_status kvtc_plan_mem_size(const kvtc_config* cfg, size_t* bytes) {
  kvtc_status st = check_config(cfg);
  if (st != KVTC_OK) return st;
  if (!bytes) return KVTC_ERR_INVALID_ARG;
  size_t a, b, r;
  *bytes = plan_layout(*cfg, &a, &b, &r);
  return KVTC_OK;
}

kvtc_status kvtc_plan(const kvtc_config* cfg, const float* basis_dev, void* plan_mem,
                      size_t plan_mem_bytes, hipStream_t stream, kvtc_plan_t* out) {
  kvtc_status st = check_config(cfg);
  if (st != KVTC_OK) return st;
  if (!out || !plan_mem) return KVTC_ERR_INVALID_ARG;
  if (cfg->transform == KVTC_PCA && !basis_dev) return KVTC_ERR_INVALID_ARG;
  size_t off_bt, off_b, off_rope;
  size_t need = plan_layout(*cfg, &off_bt, &off_b, &off_rope);
  if (plan_mem_bytes < need) return KVTC_ERR_CAPACITY;
  PlanImpl* p = new (std::nothrow) PlanImpl();
  if (!p) return KVTC_ERR_HIP;
  p->cfg = *cfg;
  p->mem = (uint8_t*)plan_mem;
  p->basis_t = p->mem + off_bt;
  p->basis = p->mem + off_b;
  p->rope = (float2*)(p->mem + off_rope);
  p->mem_bytes = need;
  p->n_basis = cfg->transform == KVTC_PCA
                   ? cfg->layers * 2 * (cfg->basis_per_head ? cfg->kv_heads : 1)
                   : 0;
  const int D = cfg->head_dim;
  // RoPE table: angle t * theta^(-2j/D) in fp64, cos/sin from the C library,
  // rounded to fp32 ("Why RoPE Has to Be Reversed First").
  size_t nrope = (size_t)cfg->max_tokens * (D / 2);
  float2* tab = (float2*)malloc(nrope * sizeof(float2));
  if (!tab) { delete p; return KVTC_ERR_HIP; }
  double* inv = (double*)malloc(sizeof(double) * (D / 2));
  for (int j = 0; j < D / 2; ++j) inv[j] = pow(cfg->rope_theta, -2.0 * (double)j / (double)D);
  for (int32_t t = 0; t < cfg->max_tokens; ++t)
    for (int j = 0; j < D / 2; ++j) {
      double a = (double)t * inv[j];
      tab[(size_t)t * (D / 2) + j] = make_float2((float)cos(a), (float)sin(a));
    }
  free(inv);
  hipError_t e = hipMemcpyAsync(p->rope, tab, nrope * sizeof(float2), hipMemcpyHostToDevice, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  free(tab);
  if (e != hipSuccess) { delete p; return KVTC_ERR_HIP; }
  p->fingerprint = 0xcbf29ce484222325ull;
  p->max_col_norm = 1.0f;
  if (cfg->transform == KVTC_PCA) {
    // operand-precision basis in both layouts; non-finite entries raise a
    // flag word kept at the end of plan memory
    int32_t* flag = (int32_t*)(p->mem + need - 256);
    e = hipMemsetAsync(flag, 0, 4, stream);
    if (e == hipSuccess)
      e = launch_prep_basis(basis_dev, p->basis_t, p->basis, p->n_basis, D, cfg->dtype, flag, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    int32_t nonfinite = 0;
    if (e == hipSuccess) e = hipMemcpy(&nonfinite, flag, 4, hipMemcpyDeviceToHost);
    if (e != hipSuccess) { delete p; return KVTC_ERR_HIP; }
    if (nonfinite) { delete p; return KVTC_ERR_NONFINITE; }
    // fingerprint: FNV-1a over the operand-precision basis bytes, row-major
    size_t eb = cfg->dtype == KVTC_BF16 ? 2 : 4;
    size_t nbytes = (size_t)p->n_basis * D * D * eb;
    uint8_t* hb = (uint8_t*)malloc(nbytes);
    if (!hb) { delete p; return KVTC_ERR_HIP; }
    e = hipMemcpy(hb, p->basis, nbytes, hipMemcpyDeviceToHost);
    if (e != hipSuccess) { free(hb); delete p; return KVTC_ERR_HIP; }
    uint64_t h = 0xcbf29ce484222325ull;
    for (size_t i = 0; i < nbytes; ++i) { h ^= hb[i]; h *= 0x100000001b3ull; }
    // largest column (component) norm, for the coefficient error bound
    double mx = 0.0;
    for (int m = 0; m < p->n_basis; ++m)
      for (int i = 0; i < D; ++i) {
        double acc = 0.0;
        for (int j = 0; j < D; ++j) {
          size_t idx = ((size_t)m * D + j) * D + i;
          double v;
          if (cfg->dtype == KVTC_BF16) {
            uint16_t b16;
            memcpy(&b16, hb + 2 * idx, 2);
            uint32_t u32 = (uint32_t)b16 << 16;
            float f;
            memcpy(&f, &u32, 4);
            v = f;
          } else {
            float f;
            memcpy(&f, hb + 4 * idx, 4);
            v = f;
          }
          acc += v * v;
        }
        if (acc > mx) mx = acc;
      }
    free(hb);
    p->fingerprint = h;
    p->max_col_norm = (float)(sqrt(mx) * (1.0 + 1e-6));
  }
  *out = (kvtc_plan_t)p;
  return KVTC_OK;
}

kvtc_status kvtc_plan_destroy(kvtc_plan_t plan) {
  if (!plan) return KVTC_ERR_INVALID_ARG;
  PlanImpl* p = (PlanImpl*)plan;
  if (p->prof_created)
    for (int i = 0; i < 24; ++i) (void)hipEventDestroy(p->prof_ev[i]);
  delete p;
  return KVTC_OK;
}

kvtc_status kvtc_plan_fingerprint(kvtc_plan_t plan, uint64_t* fp) {
  if (!plan || !fp) return KVTC_ERR_INVALID_ARG;
  *fp = ((PlanImpl*)plan)->fingerprint;
  return KVTC_OK;
}

kvtc_status kvtc_workspace_size(kvtc_plan_t plan, int32_t T, size_t* ws_bytes,
                                size_t* max_container) {
  if (!plan) return KVTC_ERR_INVALID_ARG;
  PlanImpl* p = (PlanImpl*)plan;
  if (T < 0 || T > p->cfg.max_tokens) return KVTC_ERR_INVALID_ARG;
  Layout lo = make_layout(p->cfg, T);
  WsLayout w = make_ws_layout(p->cfg, lo);
  if (ws_bytes) *ws_bytes = (size_t)w.total;
  if (max_container) *max_container = (size_t)max_container_bytes(p->cfg, lo);
  return KVTC_OK;
}

// Kernels move 16-byte units of every buffer.
static bool misaligned(const void* ptr) { return ((uintptr_t)ptr & 15u) != 0; }

kvtc_status kvtc_encode(kvtc_plan_t plan, const void* k, const void* v, int32_t T, void* out,
                        size_t cap, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!plan || !out || !ws) return KVTC_ERR_INVALID_ARG;
  PlanImpl* pl = (PlanImpl*)plan;
  if (T < 0 || T > pl->cfg.max_tokens) return KVTC_ERR_INVALID_ARG;
  if (T > 0 && (!k || !v)) return KVTC_ERR_INVALID_ARG;
  if (misaligned(k) || misaligned(v) || misaligned(out) || misaligned(ws)) return KVTC_ERR_INVALID_ARG;
  Layout lo = make_layout(pl->cfg, T);
  WsLayout w = make_ws_layout(pl->cfg, lo);
  if ((int64_t)ws_bytes < w.total) return KVTC_ERR_CAPACITY;
  if ((int64_t)cap < lo.chunks_off) return KVTC_ERR_CAPACITY;
  Params p = make_params(*pl, lo, w);
  p.k = k; p.v = v; p.out = (uint8_t*)out; p.out_final = p.out; p.cap = (int64_t)cap; p.ws = (uint8_t*)ws;
  uint8_t hdr[kHeaderBytes];
  build_header(*pl, lo, hdr);
  ProfScope prof(pl, stream);
  if (lo.n_blks > 0) {
    // the first pass clears the status block; the raw runs are copied by
    // extra workgroups of the rANS encoder
    HIP_TRY(launch_enc_transform(p, 0, stream));
    prof.phase("enc_stats");
  } else {
    HIP_TRY(launch_copy_raw(p, 1, stream));  // also clears the status block
    prof.phase("copy_raw");
  }
  HIP_TRY(launch_enc_alloc(p, stream));
  prof.phase("enc_alloc");
  if (lo.n_blks > 0) {
    HIP_TRY(launch_enc_transform(p, 1, stream));
    prof.phase("enc_quant_pack");
    HIP_TRY(launch_rans_encode_chunks(p, stream, true));
    prof.phase("rans_encode");
  }
  HIP_TRY(launch_assemble(p, hdr, stream));
  prof.phase("assemble");
  HIP_TRY(launch_csum(p, 1, stream));
  prof.phase("enc_checksum");
  return KVTC_OK;
}

// Checks shared by the decode entry points (all but the workspace).
static kvtc_status decode_args(const PlanImpl* pl, const void* in, int32_t T, const void* k_out,
                               const void* v_out, int32_t out_dtype) {
  if (T < 0 || T > pl->cfg.max_tokens) return KVTC_ERR_INVALID_ARG;
  if (T > 0 && (!k_out || !v_out)) return KVTC_ERR_INVALID_ARG;
  if (out_dtype != KVTC_BF16 && out_dtype != KVTC_FP32) return KVTC_ERR_INVALID_ARG;
  if (misaligned(in) || misaligned(k_out) || misaligned(v_out)) return KVTC_ERR_INVALID_ARG;
  return KVTC_OK;
}

// The decode launch sequence on a workspace laid out as `w`.
static kvtc_status decode_launch(PlanImpl* pl, const Layout& lo, const WsLayout& w, const void* in,
                                 size_t in_bytes, void* k_out, void* v_out, int32_t out_dtype, uint8_t* ws,
                                 hipStream_t stream, bool profile) {
  Params p = make_params(*pl, lo, w);
  p.in = (const uint8_t*)in; p.cap = (int64_t)in_bytes; p.ws = ws;
  p.k_out = k_out; p.v_out = v_out; p.out_dtype = out_dtype;
  uint8_t hdr[kHeaderBytes];
  build_header(*pl, lo, hdr);
  ProfScope prof(profile ? pl : nullptr, stream);
  HIP_TRY(launch_dec_check(p, hdr, stream));  // clears, then sets the status word
  prof.phase("dec_check");
  HIP_TRY(launch_csum(p, 0, stream));
  prof.phase("dec_checksum");
  if (lo.n_blks > 0) {
    // the raw runs are copied by extra workgroups of the rANS decoder
    HIP_TRY(launch_rans_decode_chunks(p, stream, true));
    prof.phase("rans_decode");
    HIP_TRY(launch_dec_transform(p, stream));
    prof.phase("dec_transform");
  } else {
    HIP_TRY(launch_copy_raw(p, 0, stream));
    prof.phase("copy_raw_out");
  }
  return KVTC_OK;
}

kvtc_status kvtc_decode(kvtc_plan_t plan, const void* in, size_t in_bytes, int32_t T,
                        void* k_out, void* v_out, int32_t out_dtype, void* ws, size_t ws_bytes,
                        hipStream_t stream) {
  if (!plan || !in || !ws) return KVTC_ERR_INVALID_ARG;
  PlanImpl* pl = (PlanImpl*)plan;
  const kvtc_status st = decode_args(pl, in, T, k_out, v_out, out_dtype);
  if (st != KVTC_OK) return st;
  if (misaligned(ws)) return KVTC_ERR_INVALID_ARG;
  Layout lo = make_layout(pl->cfg, T);
  WsLayout w = make_ws_layout(pl->cfg, lo);
  if ((int64_t)ws_bytes < w.total) return KVTC_ERR_CAPACITY;
  return decode_launch(pl, lo, w, in, in_bytes, k_out, v_out, out_dtype, (uint8_t*)ws, stream, true);
}

// ---- decode into a fixed device array ------------------------------------------

// The decoder's only workspace is the status block, the partial checksums
// of the fixed part and the packed tiles; the
// variant below keeps both in this array (one copy per device, alive until
// the process ends) instead of a caller's workspace.
constexpr int64_t kScratchBytes = KVTC_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static uint8_t* g_scratch_at[kMaxDevices];  // device address of `scratch`, per device

// The device address of the current device's copy of `scratch`, looked up on
// the first call on that device.
static kvtc_status scratch_of_current_device(uint8_t** at) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return KVTC_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return KVTC_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_at[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return KVTC_ERR_HIP;
    g_scratch_at[dev] = (uint8_t*)ptr;
  }
  *at = g_scratch_at[dev];
  return KVTC_OK;
}

// The decoder's workspace inside the scratch array: the status block, the
// partial checksums, then the packed tiles; every other region is unused by
// the decode kernels and points at the status block.
static WsLayout decode_scratch_layout(const kvtc_config& c, const Layout& lo) {
  const WsLayout full = make_ws_layout(c, lo);
  WsLayout w{};
  w.packed_slot = full.packed_slot;
  w.tile_words_max = full.tile_words_max;
  w.tile_raw_max = full.tile_raw_max;
  w.rec_slot = full.rec_slot;
  w.status = 0;
  w.csum = align256(kStatusBlockBytes);
  w.packed = w.csum + align256((int64_t)kCsumParts * 16);
  w.total = w.packed + align256((int64_t)lo.n_blks * w.packed_slot);
  return w;
}

kvtc_status kvtc_decode_noalloc(kvtc_plan_t plan, const void* in, size_t in_bytes, int32_t T, void* k_out,
                                void* v_out, int32_t out_dtype, uint32_t* status_dev, hipStream_t stream) {
  if (!plan || !in) return KVTC_ERR_INVALID_ARG;
  PlanImpl* pl = (PlanImpl*)plan;
  const kvtc_status st = decode_args(pl, in, T, k_out, v_out, out_dtype);
  if (st != KVTC_OK) return st;
  if ((uintptr_t)status_dev & 3u) return KVTC_ERR_INVALID_ARG;
  Layout lo = make_layout(pl->cfg, T);
  WsLayout w = decode_scratch_layout(pl->cfg, lo);
  if (w.total > kScratchBytes) return KVTC_ERR_CAPACITY;
  uint8_t* ws = nullptr;
  const kvtc_status sst = scratch_of_current_device(&ws);
  if (sst != KVTC_OK) return sst;
  const kvtc_status lst = decode_launch(pl, lo, w, in, in_bytes, k_out, v_out, out_dtype, ws, stream, false);
  if (lst != KVTC_OK) return lst;
  if (status_dev) HIP_TRY(hipMemcpyAsync(status_dev, ws + w.status, 4, hipMemcpyDeviceToDevice, stream));
  return KVTC_OK;
}

// ---- paged ragged batches ----------------------------------------------------

// Host-side sizes of a batch from the host copy of the lengths; false when a
// length is out of range.  `lo_max` is the layout of the longest sequence,
// which bounds every launch grid.
static bool batch_sizes(const PlanImpl& pl, int32_t n_seqs, const int32_t* lens, int64_t* ws_total,
                        int64_t* cont_total, int64_t* sum_t, int32_t* max_t) {
  int64_t ws = batch_ws_head(n_seqs), cont = batch_header_bytes(n_seqs), st = 0;
  int32_t mt = 0;
  for (int32_t z = 0; z < n_seqs; ++z) {
    const int32_t T = lens[z];
    if (T < 0 || T > pl.cfg.max_tokens) return false;
    const Layout lo = make_layout(pl.cfg, T);
    ws += align256(make_ws_layout(pl.cfg, lo, true).total);
    cont += align256(max_container_bytes(pl.cfg, lo));
    st += T;
    if (T > mt) mt = T;
  }
  if (ws_total) *ws_total = ws;
  if (cont_total) *cont_total = cont;
  if (sum_t) *sum_t = st;
  if (max_t) *max_t = mt;
  return true;
}

// The paged path runs on the bf16 head_dim-128 PCA kernels.
static bool paged_supported(const kvtc_config& c) {
  return c.head_dim == 128 && c.dtype == KVTC_BF16 && c.transform == KVTC_PCA && c.tile_tokens % 64 == 0;
}

kvtc_status kvtc_workspace_size_paged(kvtc_plan_t plan, int32_t n_seqs, const int32_t* seq_lens_host,
                                      size_t* ws_bytes, size_t* max_container) {
  if (!plan || n_seqs < 1 || n_seqs > 65535 || !seq_lens_host) return KVTC_ERR_INVALID_ARG;
  PlanImpl* pl = (PlanImpl*)plan;
  if (!paged_supported(pl->cfg)) return KVTC_ERR_UNSUPPORTED;
  int64_t ws = 0, cont = 0;
  if (!batch_sizes(*pl, n_seqs, seq_lens_host, &ws, &cont, nullptr, nullptr)) return KVTC_ERR_INVALID_ARG;
  if (ws_bytes) *ws_bytes = (size_t)ws;
  if (max_container) *max_container = (size_t)cont;
  return KVTC_OK;
}

// Batch parameters: the layout of the longest sequence (grids) plus the pool,
// page table and sequence table.
static kvtc_status paged_params(PlanImpl* pl, int32_t pool_pages, const int32_t* page_table, int32_t max_pages,
                                const int32_t* seq_lens_dev, const int32_t* seq_lens_host, int32_t n_seqs,
                                void* ws, size_t ws_bytes, Params* out_p, int64_t* sum_t, int32_t* max_t) {
  if (n_seqs < 1 || n_seqs > 65535 || !seq_lens_host || !seq_lens_dev || !page_table || !ws)
    return KVTC_ERR_INVALID_ARG;
  if (pool_pages < 1 || max_pages < 1) return KVTC_ERR_INVALID_ARG;
  if (!paged_supported(pl->cfg)) return KVTC_ERR_UNSUPPORTED;
  if (misaligned(ws) || ((uintptr_t)page_table & 3u) || ((uintptr_t)seq_lens_dev & 3u)) return KVTC_ERR_INVALID_ARG;
  int64_t ws_total = 0;
  if (!batch_sizes(*pl, n_seqs, seq_lens_host, &ws_total, nullptr, sum_t, max_t)) return KVTC_ERR_INVALID_ARG;
  for (int32_t z = 0; z < n_seqs; ++z)
    if ((seq_lens_host[z] + kPageTokens - 1) / kPageTokens > max_pages) return KVTC_ERR_INVALID_ARG;
  if ((int64_t)ws_bytes < ws_total) return KVTC_ERR_CAPACITY;
  const Layout lo = make_layout(pl->cfg, *max_t);
  Params p = make_params(*pl, lo, make_ws_layout(pl->cfg, lo, true));
  p.ws = (uint8_t*)ws;
  p.n_seqs = n_seqs;
  p.pool_pages = pool_pages;
  p.max_pages = max_pages;
  p.page_table = page_table;
  p.seqs = reinterpret_cast<SeqInfo*>((uint8_t*)ws + batch_seqinfo_off());
  *out_p = p;
  return KVTC_OK;
}

kvtc_status kvtc_encode_paged(kvtc_plan_t plan, const void* k_pool, const void* v_pool, int32_t pool_pages,
                              const int32_t* page_table, int32_t max_pages, const int32_t* seq_lens_dev,
                              const int32_t* seq_lens_host, int32_t n_seqs, void* out, size_t cap, void* ws,
                              size_t ws_bytes, hipStream_t stream) {
  if (!plan || !k_pool || !v_pool || !out) return KVTC_ERR_INVALID_ARG;
  if (misaligned(k_pool) || misaligned(v_pool) || misaligned(out)) return KVTC_ERR_INVALID_ARG;
  PlanImpl* pl = (PlanImpl*)plan;
  Params p;
  int64_t sum_t = 0;
  int32_t max_t = 0;
  kvtc_status st = paged_params(pl, pool_pages, page_table, max_pages, seq_lens_dev, seq_lens_host, n_seqs, ws,
                                ws_bytes, &p, &sum_t, &max_t);
  if (st != KVTC_OK) return st;
  if ((int64_t)cap < batch_header_bytes(n_seqs)) return KVTC_ERR_CAPACITY;
  p.k = k_pool; p.v = v_pool; p.out = (uint8_t*)out; p.cap = (int64_t)cap;
  uint8_t hdr[kHeaderBytes];
  build_header(*pl, make_layout(pl->cfg, max_t), hdr);  // T-dependent fields are set per sequence
  ProfScope prof(pl, stream);
  HIP_TRY(launch_seq_setup(p, seq_lens_dev, sum_t, max_t, (int64_t)ws_bytes, 0, stream));
  HIP_TRY(launch_copy_raw(p, 1, stream));
  prof.phase("copy_raw");
  if (p.n_blks > 0) {
    HIP_TRY(launch_enc_transform(p, 0, stream));
    prof.phase("enc_stats");
  }
  HIP_TRY(launch_enc_alloc(p, stream));
  prof.phase("enc_alloc");
  if (p.n_blks > 0) {
    HIP_TRY(launch_enc_transform(p, 1, stream));
    prof.phase("enc_quant_pack");
    HIP_TRY(launch_rans_encode_chunks(p, stream));
    prof.phase("rans_encode");
  }
  HIP_TRY(launch_assemble(p, hdr, stream));
  HIP_TRY(launch_csum(p, 1, stream));
  HIP_TRY(launch_batch_finish(p, stream));
  prof.phase("assemble");
  return KVTC_OK;
}

kvtc_status kvtc_decode_paged(kvtc_plan_t plan, const void* in, size_t in_bytes, void* k_pool, void* v_pool,
                              int32_t pool_pages, const int32_t* page_table, int32_t max_pages,
                              const int32_t* seq_lens_dev, const int32_t* seq_lens_host, int32_t n_seqs, void* ws,
                              size_t ws_bytes, hipStream_t stream) {
  if (!plan || !in || !k_pool || !v_pool) return KVTC_ERR_INVALID_ARG;
  if (misaligned(in) || misaligned(k_pool) || misaligned(v_pool)) return KVTC_ERR_INVALID_ARG;
  PlanImpl* pl = (PlanImpl*)plan;
  Params p;
  int64_t sum_t = 0;
  int32_t max_t = 0;
  kvtc_status st = paged_params(pl, pool_pages, page_table, max_pages, seq_lens_dev, seq_lens_host, n_seqs, ws,
                                ws_bytes, &p, &sum_t, &max_t);
  if (st != KVTC_OK) return st;
  p.in = (const uint8_t*)in; p.cap = (int64_t)in_bytes;
  p.k_out = k_pool; p.v_out = v_pool; p.out_dtype = pl->cfg.dtype;
  uint8_t hdr[kHeaderBytes];
  build_header(*pl, make_layout(pl->cfg, max_t), hdr);
  ProfScope prof(pl, stream);
  HIP_TRY(launch_seq_setup(p, seq_lens_dev, sum_t, max_t, (int64_t)ws_bytes, 1, stream));
  HIP_TRY(launch_dec_check(p, hdr, stream));
  HIP_TRY(launch_csum(p, 0, stream));
  prof.phase("dec_check");
  if (p.n_blks > 0) {
    HIP_TRY(launch_rans_decode_chunks(p, stream));
    prof.phase("rans_decode");
    HIP_TRY(launch_dec_transform(p, stream));
    prof.phase("dec_transform");
  }
  HIP_TRY(launch_copy_raw(p, 0, stream));
  HIP_TRY(launch_batch_finish(p, stream));
  prof.phase("copy_raw_out");
  return KVTC_OK;
}

kvtc_status kvtc_result(kvtc_plan_t plan, const void* ws, uint64_t* container_bytes,
                        int32_t* device_status) {
  if (!plan || !ws) return KVTC_ERR_INVALID_ARG;
  uint32_t buf[4];
  if (hipMemcpy(buf, ws, 16, hipMemcpyDeviceToHost) != hipSuccess) return KVTC_ERR_HIP;
  uint32_t bits = buf[0];
  int32_t st = KVTC_OK;
  if (bits & (1u << KVTC_ERR_INVALID_ARG)) st = KVTC_ERR_INVALID_ARG;
  else if (bits & (1u << KVTC_ERR_NONFINITE)) st = KVTC_ERR_NONFINITE;
  else if (bits & (1u << KVTC_ERR_CORRUPT)) st = KVTC_ERR_CORRUPT;
  else if (bits & (1u << KVTC_ERR_CAPACITY)) st = KVTC_ERR_CAPACITY;
  else if (bits) st = KVTC_ERR_HIP;
  if (device_status) *device_status = st;
  if (container_bytes) {
    uint64_t n;
    memcpy(&n, &buf[2], 8);
    *container_bytes = n;
  }
  return KVTC_OK;
}

kvtc_status kvtc_encode_counters(kvtc_plan_t plan, const void* ws, uint64_t* exact_recomputed) {
  if (!plan || !ws || !exact_recomputed) return KVTC_ERR_INVALID_ARG;
  static_assert(kStatusBlockBytes % 4 == 0, "status block in words");
  uint32_t buf[kStatusBlockBytes / 4];
  if (hipMemcpy(buf, ws, sizeof(buf), hipMemcpyDeviceToHost) != hipSuccess) return KVTC_ERR_HIP;
  uint64_t n = buf[1];
  for (int i = 0; i < kCountSlots; ++i) n += buf[(kCountOff + kCountStride * i) / 4];
  *exact_recomputed = n;
  return KVTC_OK;
}

kvtc_status kvtc_test_section_stats(kvtc_plan_t plan, const void* ws, int32_t T, float* mu,
                                    float* var, float* cmin, float* cmax) {
  if (!plan || !ws || !mu || !var || !cmin || !cmax) return KVTC_ERR_INVALID_ARG;
  PlanImpl* pl = (PlanImpl*)plan;
  if (T < 0 || T > pl->cfg.max_tokens) return KVTC_ERR_INVALID_ARG;
  Layout lo = make_layout(pl->cfg, T);
  WsLayout w = make_ws_layout(pl->cfg, lo);
  size_t n = (size_t)lo.n_sections * pl->cfg.head_dim;
  float* h = (float*)malloc(n * 16);
  if (!h) return KVTC_ERR_HIP;
  if (hipMemcpy(h, (const uint8_t*)ws + w.sec_stats, n * 16, hipMemcpyDeviceToHost) != hipSuccess) {
    free(h);
    return KVTC_ERR_HIP;
  }
  for (size_t i = 0; i < n; ++i) {
    mu[i] = h[4 * i]; var[i] = h[4 * i + 1]; cmin[i] = h[4 * i + 2]; cmax[i] = h[4 * i + 3];
  }
  free(h);
  return KVTC_OK;
}

kvtc_status kvtc_test_coeffs(kvtc_plan_t plan, const void* k, const void* v, int32_t T,
                             int32_t sec_begin, int32_t sec_end, float* out, float* r_out,
                             hipStream_t stream) {
  if (!plan || !k || !v || !out) return KVTC_ERR_INVALID_ARG;
  PlanImpl* pl = (PlanImpl*)plan;
  if (T < 0 || T > pl->cfg.max_tokens) return KVTC_ERR_INVALID_ARG;
  Layout lo = make_layout(pl->cfg, T);
  if (sec_begin < 0 || sec_end > lo.n_sections || sec_begin > sec_end) return KVTC_ERR_INVALID_ARG;
  WsLayout w = make_ws_layout(pl->cfg, lo);
  Params p = make_params(*pl, lo, w);
  p.k = k; p.v = v;
  if (lo.T_mid == 0 || sec_end == sec_begin) return KVTC_OK;
  HIP_TRY(launch_coeffs(p, sec_begin, sec_end, out, r_out, stream));
  return KVTC_OK;
}

kvtc_status kvtc_test_freq_tables(const uint32_t* counts, const int32_t* alphabet, int32_t n,
                                  int32_t scale_bits, uint16_t* freq, hipStream_t stream) {
  if (n < 0 || (n > 0 && (!counts || !alphabet || !freq))) return KVTC_ERR_INVALID_ARG;
  if (scale_bits < 8 || scale_bits > 12) return KVTC_ERR_UNSUPPORTED;
  HIP_TRY(launch_test_freq_tables(counts, alphabet, n, scale_bits, freq, stream));
  return KVTC_OK;
}

kvtc_status kvtc_test_packed_tiles(kvtc_plan_t plan, const void* ws, int32_t T, int32_t section,
                                   void* out, size_t out_bytes, int32_t* blocks, size_t* slot_bytes,
                                   hipStream_t stream) {
  if (!plan || !ws) return KVTC_ERR_INVALID_ARG;
  PlanImpl* pl = (PlanImpl*)plan;
  if (T < 0 || T > pl->cfg.max_tokens) return KVTC_ERR_INVALID_ARG;
  Layout lo = make_layout(pl->cfg, T);
  if (section < 0 || section >= lo.n_sections) return KVTC_ERR_INVALID_ARG;
  WsLayout w = make_ws_layout(pl->cfg, lo);
  if (blocks) *blocks = lo.blks_per_sec;
  if (slot_bytes) *slot_bytes = (size_t)w.packed_slot;
  const size_t n = (size_t)lo.blks_per_sec * (size_t)w.packed_slot;
  if (!out || n == 0) return KVTC_OK;
  if (out_bytes < n) return KVTC_ERR_CAPACITY;
  HIP_TRY(hipMemcpyAsync(out, (const uint8_t*)ws + w.packed + (int64_t)section * lo.blks_per_sec * w.packed_slot, n,
                         hipMemcpyDeviceToDevice, stream));
  return KVTC_OK;
}

kvtc_status kvtc_test_rope(kvtc_plan_t plan, const void* k, int32_t T, void* ws, size_t ws_bytes, void* out,
                           size_t out_bytes, hipStream_t stream) {
  if (!plan || !k || !ws || !out) return KVTC_ERR_INVALID_ARG;
  PlanImpl* pl = (PlanImpl*)plan;
  if (T < 0 || T > pl->cfg.max_tokens) return KVTC_ERR_INVALID_ARG;
  const kvtc_config& c = pl->cfg;
  if (!(c.head_dim == 128 && c.dtype == KVTC_BF16 && c.transform == KVTC_PCA && c.rope_keys && c.tile_tokens % 64 == 0))
    return KVTC_ERR_UNSUPPORTED;
  Layout lo = make_layout(c, T);
  WsLayout w = make_ws_layout(c, lo);
  if ((int64_t)ws_bytes < w.total) return KVTC_ERR_CAPACITY;
  const size_t n = (size_t)c.layers * c.kv_heads * lo.T_mid * c.head_dim * 2;
  if (out_bytes < n) return KVTC_ERR_CAPACITY;
  Params p = make_params(*pl, lo, w);
  p.k = k; p.ws = (uint8_t*)ws;
  HIP_TRY(launch_unrope(p, stream));
  if (n) HIP_TRY(hipMemcpyAsync(out, (const uint8_t*)ws + w.kprime, n, hipMemcpyDeviceToDevice, stream));
  return KVTC_OK;
}

kvtc_status kvtc_test_alloc(kvtc_plan_t plan, int32_t T, const float* stats, void* ws, size_t ws_bytes,
                            void* side_out, size_t side_bytes, hipStream_t stream) {
  if (!plan || !stats || !ws || !side_out) return KVTC_ERR_INVALID_ARG;
  PlanImpl* pl = (PlanImpl*)plan;
  if (T < 0 || T > pl->cfg.max_tokens) return KVTC_ERR_INVALID_ARG;
  Layout lo = make_layout(pl->cfg, T);
  WsLayout w = make_ws_layout(pl->cfg, lo);
  if ((int64_t)ws_bytes < w.total) return KVTC_ERR_CAPACITY;
  const size_t n = (size_t)lo.n_sections * pl->cfg.head_dim;
  if (side_bytes < n * 9) return KVTC_ERR_CAPACITY;
  HIP_TRY(hipMemcpyAsync((uint8_t*)ws + w.sec_stats, stats, n * 16, hipMemcpyHostToDevice, stream));
  Params p = make_params(*pl, lo, w);
  p.ws = (uint8_t*)ws;
  p.out = (uint8_t*)side_out - lo.side_off;  // the section records land at side_out
  HIP_TRY(launch_alloc_from_stats(p, stream));
  return KVTC_OK;
}

kvtc_status kvtc_test_quant_pack(kvtc_plan_t plan, const void* k, const void* v, int32_t T, void* out, size_t cap,
                                 void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!plan || !k || !v || !out || !ws) return KVTC_ERR_INVALID_ARG;
  PlanImpl* pl = (PlanImpl*)plan;
  if (T < 0 || T > pl->cfg.max_tokens) return KVTC_ERR_INVALID_ARG;
  if (misaligned(k) || misaligned(v) || misaligned(out) || misaligned(ws)) return KVTC_ERR_INVALID_ARG;
  Layout lo = make_layout(pl->cfg, T);
  WsLayout w = make_ws_layout(pl->cfg, lo);
  if ((int64_t)ws_bytes < w.total || (int64_t)cap < lo.raw_off) return KVTC_ERR_CAPACITY;
  Params p = make_params(*pl, lo, w);
  p.k = k; p.v = v; p.out = (uint8_t*)out; p.out_final = p.out; p.cap = (int64_t)cap; p.ws = (uint8_t*)ws;
  if (lo.n_blks == 0) return KVTC_OK;
  HIP_TRY(launch_enc_transform(p, 0, stream));
  HIP_TRY(launch_enc_alloc(p, stream));
  HIP_TRY(launch_enc_transform(p, 1, stream));
  return KVTC_OK;
}

kvtc_status kvtc_test_dequant_project(kvtc_plan_t plan, const void* in, size_t in_bytes, int32_t T, void* ws,
                                      size_t ws_bytes, void* k_out, void* v_out, int32_t out_dtype,
                                      hipStream_t stream) {
  if (!plan || !in || !ws || !k_out || !v_out) return KVTC_ERR_INVALID_ARG;
  PlanImpl* pl = (PlanImpl*)plan;
  const kvtc_status st = decode_args(pl, in, T, k_out, v_out, out_dtype);
  if (st != KVTC_OK) return st;
  Layout lo = make_layout(pl->cfg, T);
  WsLayout w = make_ws_layout(pl->cfg, lo);
  if ((int64_t)ws_bytes < w.total || (int64_t)in_bytes < lo.raw_off) return KVTC_ERR_CAPACITY;
  Params p = make_params(*pl, lo, w);
  p.in = (const uint8_t*)in; p.cap = (int64_t)in_bytes; p.ws = (uint8_t*)ws;
  p.k_out = k_out; p.v_out = v_out; p.out_dtype = out_dtype;
  if (lo.n_blks == 0) return KVTC_OK;
  HIP_TRY(launch_dec_transform(p, stream));
  return KVTC_OK;
}

// ---- scalar quantisers on gauge coordinates --------------------------------

static kvtc_status sq_params(const PlanImpl* pl, const kvtc_sq_config* q, int32_t T, SqParams* sp) {
  if (!q) return KVTC_ERR_INVALID_ARG;
  const kvtc_config& c = pl->cfg;
  if (c.transform != KVTC_PCA) return KVTC_ERR_INVALID_ARG;
  if (q->kind != KVTC_SQ_BLOCK && q->kind != KVTC_SQ_KIVI) return KVTC_ERR_INVALID_ARG;
  if (q->group < 1 || c.head_dim % q->group) return KVTC_ERR_INVALID_ARG;
  if (q->tile < 1) return KVTC_ERR_INVALID_ARG;
  if (q->bits_k < 1 || q->bits_k > 8 || q->bits_v < 1 || q->bits_v > 8) return KVTC_ERR_INVALID_ARG;
  if (T < 0 || T > c.max_tokens) return KVTC_ERR_INVALID_ARG;
  // the kernels run 64-token spans of head_dim 128 bf16 rows on MFMA; a
  // range may not straddle a span
  if (c.head_dim != 128 || c.dtype != KVTC_BF16 || (64 % q->tile)) return KVTC_ERR_UNSUPPORTED;
  SqParams p{};
  p.L = c.layers; p.H = c.kv_heads; p.T = T;
  p.basis_per_head = c.basis_per_head; p.rope_keys = c.rope_keys; p.rope_style = c.rope_style;
  p.bits[0] = q->bits_k; p.bits[1] = q->bits_v;
  const bool block = q->kind == KVTC_SQ_BLOCK;
  p.te[0] = q->tile; p.ce[0] = block ? q->group : 1;          // keys
  p.te[1] = block ? q->tile : 1; p.ce[1] = q->group;          // values
  for (int s = 0; s < 2; ++s) {
    p.code_bytes[s] = (int64_t)T * c.head_dim * p.bits[s] / 8;
    p.n_ranges[s] = ((int64_t)T + p.te[s] - 1) / p.te[s] * (c.head_dim / p.ce[s]);
  }
  p.mfma_err = 24.0f * 0x1p-24f * pl->max_col_norm;  // as for the codec's projection
  p.basis_t = (const uint16_t*)pl->basis_t;
  p.basis = (const uint16_t*)pl->basis;
  p.rope = pl->rope;
  *sp = p;
  return KVTC_OK;
}

kvtc_status kvtc_sq_sizes(kvtc_plan_t plan, const kvtc_sq_config* q, int32_t T, size_t* code_bytes,
                          size_t* range_pairs) {
  if (!plan || !code_bytes || !range_pairs) return KVTC_ERR_INVALID_ARG;
  SqParams p;
  const kvtc_status st = sq_params((const PlanImpl*)plan, q, T, &p);
  if (st != KVTC_OK) return st;
  const int64_t LH = (int64_t)p.L * p.H;
  *code_bytes = (size_t)(LH * (p.code_bytes[0] + p.code_bytes[1]));
  *range_pairs = (size_t)(LH * (p.n_ranges[0] + p.n_ranges[1]));
  return KVTC_OK;
}

kvtc_status kvtc_sq_encode(kvtc_plan_t plan, const kvtc_sq_config* q, const void* k, const void* v, int32_t T,
                           void* codes, size_t code_cap, float* ranges, size_t range_cap, uint32_t* status_dev,
                           hipStream_t stream) {
  if (!plan) return KVTC_ERR_INVALID_ARG;
  SqParams p;
  const kvtc_status st = sq_params((const PlanImpl*)plan, q, T, &p);
  if (st != KVTC_OK) return st;
  if (T > 0 && (!k || !v || !codes || !ranges)) return KVTC_ERR_INVALID_ARG;
  if (misaligned(k) || misaligned(v) || misaligned(codes) || misaligned(ranges) || ((uintptr_t)status_dev & 3u))
    return KVTC_ERR_INVALID_ARG;
  const int64_t LH = (int64_t)p.L * p.H;
  if ((int64_t)code_cap < LH * (p.code_bytes[0] + p.code_bytes[1]) ||
      (int64_t)range_cap < LH * (p.n_ranges[0] + p.n_ranges[1]))
    return KVTC_ERR_CAPACITY;
  p.k = (const uint16_t*)k; p.v = (const uint16_t*)v;
  p.codes = (uint8_t*)codes; p.ranges = ranges; p.status = status_dev;
  HIP_TRY(launch_sq_encode(p, stream));
  return KVTC_OK;
}

kvtc_status kvtc_sq_decode(kvtc_plan_t plan, const kvtc_sq_config* q, const void* codes, size_t code_bytes,
                           const float* ranges, size_t range_pairs, int32_t T, void* k_out, void* v_out,
                           int32_t out_dtype, hipStream_t stream) {
  if (!plan) return KVTC_ERR_INVALID_ARG;
  SqParams p;
  const kvtc_status st = sq_params((const PlanImpl*)plan, q, T, &p);
  if (st != KVTC_OK) return st;
  if (out_dtype != KVTC_BF16 && out_dtype != KVTC_FP32) return KVTC_ERR_INVALID_ARG;
  if (T > 0 && (!codes || !ranges || !k_out || !v_out)) return KVTC_ERR_INVALID_ARG;
  if (misaligned(codes) || misaligned(ranges) || misaligned(k_out) || misaligned(v_out)) return KVTC_ERR_INVALID_ARG;
  const int64_t LH = (int64_t)p.L * p.H;
  if ((int64_t)code_bytes < LH * (p.code_bytes[0] + p.code_bytes[1]) ||
      (int64_t)range_pairs < LH * (p.n_ranges[0] + p.n_ranges[1]))
    return KVTC_ERR_CAPACITY;
  p.codes = (uint8_t*)codes; p.ranges = (float*)ranges;
  p.k_out = k_out; p.v_out = v_out; p.out_dtype = out_dtype;
  HIP_TRY(launch_sq_decode(p, stream));
  return KVTC_OK;
}

// ---- TTAS-X2 value path -------------------------------------------------------

static bool pq_pow2(int32_t k) { return k >= 2 && k <= 512 && (k & (k - 1)) == 0; }

static int32_t pq_log2(int32_t k) {
  int32_t b = 0;
  while ((1 << b) < k) ++b;
  return b;
}

// Checks, parameters and the workspace layout of a call; ws_at == null only sizes it.
static kvtc_status pq_params(const PlanImpl* pl, const kvtc_pq_config* q, int32_t T, uint8_t* ws_at,
                             PqParams* pp, int64_t* ws_need) {
  if (!q) return KVTC_ERR_INVALID_ARG;
  const kvtc_config& c = pl->cfg;
  if (q->sub_dim < 1 || c.head_dim % q->sub_dim) return KVTC_ERR_INVALID_ARG;
  if (!pq_pow2(q->k1) || !pq_pow2(q->k2) || q->outliers < 0 || q->block_tokens < 1) return KVTC_ERR_INVALID_ARG;
  if (T < 0 || T > c.max_tokens) return KVTC_ERR_INVALID_ARG;
  // the kernels: head_dim 128 bf16 rows, 8-channel subvectors on 32 x 32 x 8
  // MFMA blocks of 32 centroids, 64-token spans inside a block, at most 4096
  // candidates per block merge
  if (c.head_dim != 128 || c.dtype != KVTC_BF16 || q->sub_dim != 8 || q->k1 < 32 || q->k2 < 32 ||
      q->outliers > 256 || (q->block_tokens % 64) || (int64_t)(q->block_tokens / 64) * q->outliers > 4096)
    return KVTC_ERR_UNSUPPORTED;
  PqParams p{};
  p.L = c.layers; p.H = c.kv_heads; p.T = T;
  p.k1 = q->k1; p.k2 = q->k2; p.b1 = pq_log2(q->k1); p.b2 = pq_log2(q->k2);
  p.B = q->outliers; p.bt = q->block_tokens;
  p.rw = (16 * (p.b1 + p.b2) + 31) / 32;
  p.nspan = (T + 63) / 64;
  p.nblk = (T + q->block_tokens - 1) / q->block_tokens;
  int64_t at = 0;
  auto take = [&](int64_t bytes) { const int64_t o = at; at += align256(bytes); return o; };
  const int64_t o1 = take((int64_t)c.layers * 16 * p.k1 * 8 * 2);
  const int64_t o2 = take((int64_t)c.layers * 16 * p.k2 * 8 * 2);
  const int64_t o3 = take((int64_t)c.layers * 16 * (p.k1 + p.k2) * 4);
  const int64_t o4 = take((int64_t)c.layers * 16 * 2 * 4);
  const int64_t o5 = take((int64_t)c.layers * c.kv_heads * p.nspan * p.B * 16);
  *ws_need = at;
  if (ws_at) {
    p.cb1h = (uint16_t*)(ws_at + o1);
    p.cb2h = (uint16_t*)(ws_at + o2);
    p.cn2 = (float*)(ws_at + o3);
    p.cmax = (float*)(ws_at + o4);
    p.cand = (uint4*)(ws_at + o5);
  }
  *pp = p;
  return KVTC_OK;
}

kvtc_status kvtc_pq_sizes(kvtc_plan_t plan, const kvtc_pq_config* q, int32_t T, size_t* code_bytes,
                          size_t* outlier_slots, size_t* ws_bytes) {
  if (!plan || !code_bytes || !outlier_slots || !ws_bytes) return KVTC_ERR_INVALID_ARG;
  PqParams p;
  int64_t ws = 0;
  const kvtc_status st = pq_params((const PlanImpl*)plan, q, T, nullptr, &p, &ws);
  if (st != KVTC_OK) return st;
  *code_bytes = (size_t)((int64_t)p.L * p.H * T * p.rw * 4);
  *outlier_slots = (size_t)((int64_t)p.L * p.H * p.nblk * p.B);
  *ws_bytes = (size_t)ws;
  return KVTC_OK;
}

kvtc_status kvtc_pq_encode(kvtc_plan_t plan, const kvtc_pq_config* q, const float* cb1, const float* cb2,
                           const void* v, int32_t T, uint32_t* codes, size_t code_cap, float* rms, size_t rms_cap,
                           uint32_t* outliers, size_t outlier_cap, void* ws, size_t ws_bytes, uint32_t* status_dev,
                           hipStream_t stream) {
  if (!plan || !ws) return KVTC_ERR_INVALID_ARG;
  PqParams p;
  int64_t need = 0;
  const kvtc_status st = pq_params((const PlanImpl*)plan, q, T, (uint8_t*)ws, &p, &need);
  if (st != KVTC_OK) return st;
  if (!cb1 || !cb2 || (T > 0 && (!v || !codes || !rms)) || (T > 0 && p.B > 0 && !outliers)) return KVTC_ERR_INVALID_ARG;
  if (misaligned(cb1) || misaligned(cb2) || misaligned(v) || misaligned(codes) || misaligned(rms) ||
      misaligned(outliers) || misaligned(ws) || ((uintptr_t)status_dev & 3u))
    return KVTC_ERR_INVALID_ARG;
  const int64_t LH = (int64_t)p.L * p.H;
  if ((int64_t)ws_bytes < need || (int64_t)code_cap < LH * T * p.rw * 4 || (int64_t)rms_cap < LH * T ||
      (int64_t)outlier_cap < LH * p.nblk * p.B)
    return KVTC_ERR_CAPACITY;
  p.cb1 = cb1; p.cb2 = cb2; p.v = (const uint16_t*)v;
  p.codes = codes; p.rms = rms; p.outl = outliers; p.status = status_dev;
  HIP_TRY(launch_pq_encode(p, stream));
  return KVTC_OK;
}

kvtc_status kvtc_pq_decode(kvtc_plan_t plan, const kvtc_pq_config* q, const float* cb1, const float* cb2,
                           const uint32_t* codes, size_t code_bytes, const float* rms, const uint32_t* outliers,
                           size_t outlier_slots, int32_t T, void* v_out, int32_t out_dtype, void* ws, size_t ws_bytes,
                           uint32_t* status_dev, hipStream_t stream) {
  if (!plan || !ws) return KVTC_ERR_INVALID_ARG;
  PqParams p;
  int64_t need = 0;
  const kvtc_status st = pq_params((const PlanImpl*)plan, q, T, (uint8_t*)ws, &p, &need);
  if (st != KVTC_OK) return st;
  if (out_dtype != KVTC_BF16 && out_dtype != KVTC_FP32) return KVTC_ERR_INVALID_ARG;
  if (!cb1 || !cb2 || (T > 0 && (!codes || !rms || !v_out)) || (T > 0 && p.B > 0 && !outliers))
    return KVTC_ERR_INVALID_ARG;
  if (misaligned(cb1) || misaligned(cb2) || misaligned(codes) || misaligned(rms) || misaligned(outliers) ||
      misaligned(v_out) || misaligned(ws) || ((uintptr_t)status_dev & 3u))
    return KVTC_ERR_INVALID_ARG;
  const int64_t LH = (int64_t)p.L * p.H;
  if ((int64_t)ws_bytes < need || (int64_t)code_bytes < LH * T * p.rw * 4 || (int64_t)outlier_slots < LH * p.nblk * p.B)
    return KVTC_ERR_CAPACITY;
  p.cb1 = cb1; p.cb2 = cb2; p.codes = (uint32_t*)codes; p.rms = (float*)rms; p.outl = (uint32_t*)outliers;
  p.v_out = v_out; p.out_dtype = out_dtype; p.status = status_dev;
  HIP_TRY(launch_pq_decode(p, stream));
  return KVTC_OK;
}

}  // extern "C"
