/*
 * KVTC reference oracle -- TEST INFRASTRUCTURE ONLY (see kvtc_oracle.h).
 *
 * Plain single-threaded C11.  Floating point follows IEEE-754 with
 * round-to-nearest-even; the file is compiled with -ffp-contract=off so the
 * only fused multiply-adds are the explicit fmaf() calls written below.
 * Sums that the method defines as "exact, then rounded once" are taken in
 * fp64, sequentially, in index order.
 */
#include "kvtc_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#define ORC_RANS_L 65536u /* lower bound of the normalised rANS state interval */

/* ===================================================================== */
/* bf16 <-> fp32                                                          */
/* ===================================================================== */

/* Round-to-nearest-even fp32 -> bf16 (the operand precision of a bf16 cache).
 * NaN stays NaN (quietened); overflow rounds to infinity as IEEE requires. */
uint16_t orc_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
  uint32_t upper = u >> 16;
  uint32_t lower = u & 0xffffu;
  if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) upper += 1u;
  return (uint16_t)upper;
}

float orc_bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static float round_p(float x, int32_t dtype) {
  return dtype == ORC_BF16 ? orc_bf16_to_f32(orc_f32_to_bf16(x)) : x;
}

static float load_elem(const void* base, int32_t dtype, int64_t idx) {
  if (dtype == ORC_BF16) return orc_bf16_to_f32(((const uint16_t*)base)[idx]);
  return ((const float*)base)[idx];
}

static void store_elem(void* base, int32_t dtype, int64_t idx, float v) {
  if (dtype == ORC_BF16)
    ((uint16_t*)base)[idx] = orc_f32_to_bf16(v);
  else
    ((float*)base)[idx] = v;
}

/* ===================================================================== */
/* RoPE ([KVTC] "Why RoPE Has to Be Reversed First"; apply_rope_inverse in */
/* "How the Pipeline Works")                                               */
/* ===================================================================== */

/* Angle of pair j at position t is t * theta^(-2j/D), taken in fp64; the
 * cosine and sine come from the C library in fp64 and are rounded to fp32. */
void orc_rope_table(int32_t T, int32_t D, double theta, float* cos_out, float* sin_out) {
  int32_t h = D / 2;
  for (int32_t t = 0; t < T; ++t) {
    for (int32_t j = 0; j < h; ++j) {
      double inv = pow(theta, -2.0 * (double)j / (double)D);
      double a = (double)t * inv;
      cos_out[(int64_t)t * h + j] = (float)cos(a);
      sin_out[(int64_t)t * h + j] = (float)sin(a);
    }
  }
}

static void rope_pair(int32_t j, int32_t D, int32_t style, int32_t* a, int32_t* b) {
  if (style == ORC_ROPE_INTERLEAVED) {
    *a = 2 * j;
    *b = 2 * j + 1;
  } else {
    *a = j;
    *b = j + D / 2;
  }
}

/* Undo the rotation: (x_a, x_b) = R(-angle) (y_a, y_b).
 * x_a = y_a c + y_b s,  x_b = y_b c - y_a s, each with one explicit fma. */
void orc_rope_inverse(const float* y, float* x, int32_t D, int32_t style,
                      const float* cos_row, const float* sin_row) {
  for (int32_t j = 0; j < D / 2; ++j) {
    int32_t a, b;
    rope_pair(j, D, style, &a, &b);
    float c = cos_row[j], s = sin_row[j];
    float yb_s = y[b] * s;
    float ya_s = y[a] * s;
    x[a] = fmaf(y[a], c, yb_s);
    x[b] = fmaf(y[b], c, -ya_s);
  }
}

/* Re-apply the rotation: (y_a, y_b) = R(angle) (x_a, x_b). */
void orc_rope_forward(const float* x, float* y, int32_t D, int32_t style,
                      const float* cos_row, const float* sin_row) {
  for (int32_t j = 0; j < D / 2; ++j) {
    int32_t a, b;
    rope_pair(j, D, style, &a, &b);
    float c = cos_row[j], s = sin_row[j];
    float xb_s = x[b] * s;
    float xb_c = x[b] * c;
    y[a] = fmaf(x[a], c, -xb_s);
    y[b] = fmaf(x[a], s, xb_c);
  }
}

/* ===================================================================== */
/* Orthogonal transform ([KVTC] pca_transform; [CG] Z = G X, X^ = G^-1 Z^) */
/* ===================================================================== */

/* c_i = sum_j x_j B[j][i]: column i of B is component i.  Products and the
 * sum are taken in fp64 (exact products for bf16 and fp32 operands) and the
 * result is rounded to fp32 once. */
void orc_project(const float* x, const float* Bp, int32_t D, float* c) {
  for (int32_t i = 0; i < D; ++i) {
    double acc = 0.0;
    for (int32_t j = 0; j < D; ++j) acc += (double)x[j] * (double)Bp[(int64_t)j * D + i];
    c[i] = (float)acc;
  }
}

/* x_j = sum_i B[j][i] chat_i (B orthogonal, so B^-1 = B^T). */
void orc_unproject(const float* chat, const float* Bp, int32_t D, float* x) {
  for (int32_t j = 0; j < D; ++j) {
    double acc = 0.0;
    for (int32_t i = 0; i < D; ++i) acc += (double)Bp[(int64_t)j * D + i] * (double)chat[i];
    x[j] = (float)acc;
  }
}

/* Per-vector RMS ([TTAS] 2.2): sqrt(sum x^2 / D) in fp64, rounded to fp32. */
float orc_rms(const float* x, int32_t D) {
  double acc = 0.0;
  for (int32_t j = 0; j < D; ++j) acc += (double)x[j] * (double)x[j];
  return (float)sqrt(acc / (double)D);
}

/* Orthonormal Walsh-Hadamard transform in Sylvester (natural) order
 * ([TTAS] 2.2 "Hadamard transform to spread energy"; [CG] Hadamard control):
 * H[i][j] = (-1)^popcount(i & j); y = H x / sqrt(D), sum in fp64, one
 * rounding.  H/sqrt(D) is symmetric and orthogonal, so it is its own inverse. */
void orc_wht(const float* x, int32_t D, float* y) {
  double rs = sqrt((double)D);
  for (int32_t i = 0; i < D; ++i) {
    double acc = 0.0;
    for (int32_t j = 0; j < D; ++j) {
      int neg = __builtin_popcount((unsigned)(i & j)) & 1;
      acc += neg ? -(double)x[j] : (double)x[j];
    }
    y[i] = (float)(acc / rs);
  }
}

/* ===================================================================== */
/* Statistics and bit allocation ([KVTC] "Bit Budget Is Not Fair")         */
/* ===================================================================== */

/* Per component over N coefficient rows c[N][D]: mean and variance (two
 * passes in fp64, population variance), minimum and maximum.  A component
 * whose minimum equals its maximum has variance 0. */
void orc_stats(const float* c, int64_t N, int32_t D, float* mu, float* var,
               float* cmin, float* cmax) {
  for (int32_t i = 0; i < D; ++i) {
    double s = 0.0;
    float mn = INFINITY, mx = -INFINITY;
    for (int64_t t = 0; t < N; ++t) {
      float v = c[t * D + i];
      s += (double)v;
      if (v < mn) mn = v;
      if (v > mx) mx = v;
    }
    double m = N > 0 ? s / (double)N : 0.0;
    double ss = 0.0;
    for (int64_t t = 0; t < N; ++t) {
      double d = (double)c[t * D + i] - m;
      ss += d * d;
    }
    mu[i] = (float)m;
    var[i] = (N > 0 && mx != mn) ? (float)(ss / (double)N) : 0.0f;
    cmin[i] = N > 0 ? mn : 0.0f;
    cmax[i] = N > 0 ? mx : 0.0f;
  }
}

/* Total bits per token: floor(bits * D), with the product taken in fp32. */
int32_t orc_budget(float bits, int32_t D) {
  float p = bits * (float)D;
  return (int32_t)floorf(p);
}

/* Greedy marginal allocation: spend the budget one bit at a time on the
 * component whose modelled distortion var * 4^-b falls the most, i.e. the
 * largest var_i * 4^-b_i (an exact comparison: the scaling by a power of two
 * is exact in fp64), lowest index first on ties.  Components at max_bits or
 * with zero variance are not candidates; allocation stops when none is left. */
void orc_alloc_greedy(const float* var, int32_t D, int32_t budget, int32_t max_bits,
                      uint8_t* bits) {
  for (int32_t i = 0; i < D; ++i) bits[i] = 0;
  for (int32_t step = 0; step < budget; ++step) {
    int32_t best = -1;
    double best_v = 0.0;
    for (int32_t i = 0; i < D; ++i) {
      if (bits[i] >= max_bits || !(var[i] > 0.0f)) continue;
      double v = ldexp((double)var[i], -2 * (int)bits[i]);
      if (best < 0 || v > best_v) {
        best = i;
        best_v = v;
      }
    }
    if (best < 0) break;
    bits[best] += 1;
  }
}

double orc_distortion(const float* var, const uint8_t* bits, int32_t D) {
  double d = 0.0;
  for (int32_t i = 0; i < D; ++i) d += ldexp((double)var[i], -2 * (int)bits[i]);
  return d;
}

/* The "dynamic programming" allocation: minimise sum_i var_i 4^-b_i subject
 * to sum_i b_i <= budget and 0 <= b_i <= max_bits, by a table over
 * (component, bits spent).  Used only to check the greedy allocation. */
double orc_alloc_dp(const float* var, int32_t D, int32_t budget, int32_t max_bits,
                    uint8_t* bits) {
  int32_t B = budget;
  double* cost = (double*)malloc(sizeof(double) * (size_t)(D + 1) * (size_t)(B + 1));
  int32_t* choice = (int32_t*)malloc(sizeof(int32_t) * (size_t)(D + 1) * (size_t)(B + 1));
  for (int32_t b = 0; b <= B; ++b) cost[b] = 0.0;
  for (int32_t i = 1; i <= D; ++i) {
    for (int32_t b = 0; b <= B; ++b) {
      double best = INFINITY;
      int32_t bc = 0;
      for (int32_t k = 0; k <= max_bits && k <= b; ++k) {
        double v = ldexp((double)var[i - 1], -2 * k) + cost[(size_t)(i - 1) * (B + 1) + (b - k)];
        if (v < best) {
          best = v;
          bc = k;
        }
      }
      cost[(size_t)i * (B + 1) + b] = best;
      choice[(size_t)i * (B + 1) + b] = bc;
    }
  }
  double result = cost[(size_t)D * (B + 1) + B];
  int32_t b = B;
  for (int32_t i = D; i >= 1; --i) {
    int32_t k = choice[(size_t)i * (B + 1) + b];
    bits[i - 1] = (uint8_t)k;
    b -= k;
  }
  free(cost);
  free(choice);
  return result;
}

/* Scale and zero point per component ([KVTC] CompressedSection "scales,
 * zero points, bit widths"; [CG] KIVI-style min/max ranges):
 *   b >= 1: zero = min, scale = (max - min) / (2^b - 1), rcp = 1 / scale;
 *   b == 0: zero = mean, scale = rcp = 0 (the component decodes to its mean).
 * A zero range, or a reciprocal that overflows, gives scale = rcp = 0. */
void orc_side_info(const uint8_t* bits, const float* mu, const float* cmin,
                   const float* cmax, int32_t D, float* zero, float* scale, float* rcp) {
  for (int32_t i = 0; i < D; ++i) {
    if (bits[i] == 0) {
      zero[i] = mu[i];
      scale[i] = 0.0f;
      rcp[i] = 0.0f;
      continue;
    }
    zero[i] = cmin[i];
    double levels = (double)((1u << bits[i]) - 1u);
    float sc = (float)(((double)cmax[i] - (double)cmin[i]) / levels);
    float r = sc > 0.0f ? 1.0f / sc : 0.0f;
    if (!(sc > 0.0f) || isinf(r)) {
      sc = 0.0f;
      r = 0.0f;
    }
    scale[i] = sc;
    rcp[i] = r;
  }
}

/* Affine quantiser: v = (c - zero) * rcp in fp32 (two roundings, no fma),
 * q = clamp(round-half-even(v), 0, 2^b - 1).  vpre (optional) receives v. */
void orc_quantize(const float* c, int64_t N, int32_t D, const uint8_t* bits,
                  const float* zero, const float* rcp, uint8_t* q, float* vpre) {
  for (int64_t t = 0; t < N; ++t) {
    for (int32_t i = 0; i < D; ++i) {
      float d = c[t * D + i] - zero[i];
      float v = d * rcp[i];
      float r = nearbyintf(v);
      float hi = (float)((1u << bits[i]) - 1u);
      if (r < 0.0f) r = 0.0f;
      if (r > hi) r = hi;
      q[t * D + i] = (uint8_t)r;
      if (vpre) vpre[t * D + i] = v;
    }
  }
}

/* Symmetric scalar quantiser with one scale per section ([TTAS] 2.1: 4-bit
 * scalar with a per-head scale): v = c * rcp, q = clamp(rint(v), -Q, Q) + 2^(b-1)
 * with Q = 2^(b-1) - 1. */
void orc_quantize_sym(const float* c, int64_t N, int32_t D, int32_t b, float rcp,
                      uint8_t* q, float* vpre) {
  float Q = (float)((1 << (b - 1)) - 1);
  int32_t off = 1 << (b - 1);
  for (int64_t t = 0; t < N; ++t) {
    for (int32_t i = 0; i < D; ++i) {
      float v = c[t * D + i] * rcp;
      float r = nearbyintf(v);
      if (r < -Q) r = -Q;
      if (r > Q) r = Q;
      q[t * D + i] = (uint8_t)((int32_t)r + off);
      if (vpre) vpre[t * D + i] = v;
    }
  }
}

/* ===================================================================== */
/* Bit packing: channel-major rows ([AT1] token-major -> channel-major)    */
/* ===================================================================== */

int64_t orc_packed_bytes(const uint8_t* bits, int32_t D, int64_t ntok) {
  int64_t total = 0;
  for (int32_t i = 0; i < D; ++i) {
    if (bits[i] == 0) continue;
    total += 4 * ((ntok * bits[i] + 31) / 32);
  }
  return total;
}

/* For each component i with b_i > 0, in index order, one row: code of token
 * k sits at bits [k b_i, (k+1) b_i) of the row, least significant bit first,
 * in little-endian 32-bit words; each row is zero-padded to a whole word. */
void orc_pack(const uint8_t* q, int64_t ntok, int32_t D, const uint8_t* bits, uint8_t* out) {
  int64_t pos = 0;
  for (int32_t i = 0; i < D; ++i) {
    int32_t b = bits[i];
    if (b == 0) continue;
    int64_t nbytes = 4 * ((ntok * b + 31) / 32);
    memset(out + pos, 0, (size_t)nbytes);
    for (int64_t k = 0; k < ntok; ++k) {
      uint32_t code = q[k * D + i];
      for (int32_t bit = 0; bit < b; ++bit) {
        if ((code >> bit) & 1u) {
          int64_t gb = k * b + bit; /* bit index within the row */
          int64_t word = gb / 32, inword = gb % 32;
          int64_t byte = word * 4 + inword / 8; /* little-endian word */
          out[pos + byte] |= (uint8_t)(1u << (inword % 8));
        }
      }
    }
    pos += nbytes;
  }
}

void orc_unpack(const uint8_t* in, int64_t ntok, int32_t D, const uint8_t* bits, uint8_t* q) {
  int64_t pos = 0;
  for (int32_t i = 0; i < D; ++i) {
    int32_t b = bits[i];
    if (b == 0) {
      for (int64_t k = 0; k < ntok; ++k) q[k * D + i] = 0;
      continue;
    }
    int64_t nbytes = 4 * ((ntok * b + 31) / 32);
    for (int64_t k = 0; k < ntok; ++k) {
      uint32_t code = 0;
      for (int32_t bit = 0; bit < b; ++bit) {
        int64_t gb = k * b + bit;
        int64_t word = gb / 32, inword = gb % 32;
        int64_t byte = word * 4 + inword / 8;
        if ((in[pos + byte] >> (inword % 8)) & 1u) code |= 1u << bit;
      }
      q[k * D + i] = (uint8_t)code;
    }
    pos += nbytes;
  }
}

/* ===================================================================== */
/* rANS ([KVTC] "rANS Makes the Last Mile Smaller"; rans_encode)           */
/* ===================================================================== */

/* Frequencies summing to M = 2^scale_bits from byte counts: each present
 * symbol gets max(1, round-half-up(n_s M / N)); a positive remainder goes to
 * the most frequent symbol, an excess is removed one unit at a time from the
 * symbol with the largest frequency above 1 (lowest symbol on ties). */
void orc_freq_normalize(const uint32_t* counts, int32_t scale_bits, uint16_t* freq) {
  uint64_t N = 0;
  for (int s = 0; s < 256; ++s) N += counts[s];
  int64_t M = (int64_t)1 << scale_bits;
  if (N == 0) {
    for (int s = 0; s < 256; ++s) freq[s] = 0;
    return;
  }
  int64_t f[256];
  int64_t sum = 0;
  for (int s = 0; s < 256; ++s) {
    if (counts[s] == 0) {
      f[s] = 0;
    } else {
      int64_t r = (int64_t)(((uint64_t)counts[s] * (uint64_t)(2 * M) + N) / (2 * N));
      f[s] = r < 1 ? 1 : r;
    }
    sum += f[s];
  }
  int64_t d = M - sum;
  if (d > 0) {
    int best = 0;
    for (int s = 1; s < 256; ++s)
      if (counts[s] > counts[best]) best = s;
    f[best] += d;
  }
  while (d < 0) {
    int best = -1;
    for (int s = 0; s < 256; ++s)
      if (f[s] > 1 && (best < 0 || f[s] > f[best])) best = s;
    f[best] -= 1;
    d += 1;
  }
  for (int s = 0; s < 256; ++s) freq[s] = (uint16_t)f[s];
}

/* Interleaved rANS with `lanes` 32-bit states (state interval [2^16, 2^32),
 * 16-bit renormalisation words).  Symbol i belongs to lane i mod lanes and
 * step i / lanes.  Encoding walks the steps backwards and, inside a step,
 * the lanes in descending order; words are stored in the order they are
 * emitted.  The decoder walks the steps forwards and the lanes in ascending
 * order, consuming the words from the last one to the first.  Returns the
 * number of words, or -1 when words_cap is too small or a symbol has
 * frequency 0. */
int64_t orc_rans_encode(const uint8_t* sym, int64_t N, const uint16_t* freq,
                        int32_t scale_bits, int32_t lanes, uint32_t* states,
                        uint16_t* words, int64_t words_cap) {
  uint32_t cum[257];
  cum[0] = 0;
  for (int s = 0; s < 256; ++s) cum[s + 1] = cum[s] + freq[s];
  for (int32_t j = 0; j < lanes; ++j) states[j] = ORC_RANS_L;
  int64_t steps = (N + lanes - 1) / lanes;
  int64_t n = 0;
  for (int64_t k = steps - 1; k >= 0; --k) {
    for (int32_t j = lanes - 1; j >= 0; --j) {
      int64_t i = k * lanes + j;
      if (i >= N) continue;
      uint32_t s = sym[i];
      uint32_t f = freq[s];
      if (f == 0) return -1;
      uint32_t x = states[j];
      if ((uint64_t)x >= ((uint64_t)f << (32 - scale_bits))) {
        if (n >= words_cap) return -1;
        words[n++] = (uint16_t)(x & 0xffffu);
        x >>= 16;
      }
      x = ((x / f) << scale_bits) + (x % f) + cum[s];
      states[j] = x;
    }
  }
  return n;
}

/* Inverse of orc_rans_encode.  Returns ORC_OK, or ORC_ERR_CORRUPT when the
 * table is invalid, the words run out or are left over, or a final state
 * differs from the initial state 2^16. */
int orc_rans_decode(const uint32_t* states, const uint16_t* words, int64_t nwords,
                    const uint16_t* freq, int32_t scale_bits, int32_t lanes,
                    int64_t N, uint8_t* sym) {
  uint32_t M = 1u << scale_bits;
  uint32_t cum[257];
  cum[0] = 0;
  for (int s = 0; s < 256; ++s) cum[s + 1] = cum[s] + freq[s];
  if (N > 0 && cum[256] != M) return ORC_ERR_CORRUPT;
  uint32_t x[64];
  for (int32_t j = 0; j < lanes; ++j) {
    x[j] = states[j];
    if (x[j] < ORC_RANS_L) return ORC_ERR_CORRUPT;
  }
  int64_t ptr = nwords; /* words are consumed from the last one backwards */
  int64_t steps = (N + lanes - 1) / lanes;
  for (int64_t k = 0; k < steps; ++k) {
    for (int32_t j = 0; j < lanes; ++j) {
      int64_t i = k * lanes + j;
      if (i >= N) break;
      uint32_t slot = x[j] & (M - 1);
      int s = 0;
      while (!(slot < cum[s + 1])) ++s; /* the symbol whose range holds slot */
      sym[i] = (uint8_t)s;
      x[j] = freq[s] * (x[j] >> scale_bits) + slot - cum[s];
      if (x[j] < ORC_RANS_L) {
        if (ptr <= 0) return ORC_ERR_CORRUPT;
        x[j] = (x[j] << 16) | words[--ptr];
        if (x[j] < ORC_RANS_L) return ORC_ERR_CORRUPT;
      }
    }
  }
  if (ptr != 0) return ORC_ERR_CORRUPT;
  for (int32_t j = 0; j < lanes; ++j)
    if (x[j] != ORC_RANS_L) return ORC_ERR_CORRUPT;
  return ORC_OK;
}

/* ===================================================================== */
/* Container ([KVTC] CompressedSection: data, scales, zero points, bit     */
/* widths, metadata; chunked transport with ordered lengths as on the QATQ */
/* page).  All fields little-endian.                                       */
/* ===================================================================== */

#define HDR_BYTES 256
#define SEC_REC(D) (9 * (int64_t)(D))
#define DIR_ENTRY 16

typedef struct {
  int32_t T, s0, mid_begin, mid_end, T_mid, W_eff;
  int32_t n_sections, chunks_per_sec, n_r_sections;
  int64_t side_off, side_bytes, r_off, raw_off, raw_bytes, dir_off, chunks_off;
  int32_t budget_k, budget_v;
} layout_t;

static int64_t align16(int64_t x) { return (x + 15) & ~(int64_t)15; }

int orc_check_config(const orc_config* c) {
  if (c->layers < 1 || c->kv_heads < 1) return ORC_ERR_INVALID_ARG;
  if (c->head_dim < 16 || c->head_dim > 256 || (c->head_dim % 16) != 0) return ORC_ERR_INVALID_ARG;
  if (c->dtype != ORC_FP32 && c->dtype != ORC_BF16) return ORC_ERR_INVALID_ARG;
  if (c->transform != ORC_PCA && c->transform != ORC_WHT) return ORC_ERR_INVALID_ARG;
  if (c->transform == ORC_WHT && (c->head_dim & (c->head_dim - 1))) return ORC_ERR_INVALID_ARG;
  if (c->sink_tokens < 0 || c->recent_tokens < 0) return ORC_ERR_INVALID_ARG;
  if (c->max_bits < 1 || c->max_bits > 8) return ORC_ERR_INVALID_ARG;
  if (!(c->bits_k >= 0.0f) || !(c->bits_v >= 0.0f)) return ORC_ERR_INVALID_ARG;
  if (c->bits_k > (float)c->max_bits || c->bits_v > (float)c->max_bits) return ORC_ERR_INVALID_ARG;
  if (c->transform == ORC_WHT) {
    if (c->bits_k < 2.0f || c->bits_v < 1.0f) return ORC_ERR_INVALID_ARG;
  }
  if (c->rope_style != ORC_ROPE_HALF && c->rope_style != ORC_ROPE_INTERLEAVED) return ORC_ERR_INVALID_ARG;
  if (c->rope_keys && !(c->rope_theta > 1.0)) return ORC_ERR_INVALID_ARG;
  if (c->rans_scale_bits < 8 || c->rans_scale_bits > 15) return ORC_ERR_INVALID_ARG;
  if (c->rans_lanes < 1 || c->rans_lanes > 64) return ORC_ERR_INVALID_ARG;
  if (c->tile_tokens < 1 || c->chunk_tokens < c->tile_tokens) return ORC_ERR_INVALID_ARG;
  if (c->chunk_tokens % c->tile_tokens) return ORC_ERR_INVALID_ARG;
  return ORC_OK;
}

static int32_t uniform_bits(float bits) { return (int32_t)floorf(bits); }

/* Sections that carry per-token RMS values (WHT path). */
static int section_has_r(const orc_config* c, int32_t s) {
  if (c->transform != ORC_WHT) return 0;
  return s == 1 || c->wht_keys;
}

static void make_layout(const orc_config* c, int32_t T, layout_t* lo) {
  lo->T = T;
  lo->s0 = c->sink_tokens < T ? c->sink_tokens : T;
  lo->mid_begin = lo->s0;
  int32_t e = T - c->recent_tokens;
  lo->mid_end = e > lo->s0 ? e : lo->s0;
  lo->T_mid = lo->mid_end - lo->mid_begin;
  lo->W_eff = T - lo->mid_end;
  lo->n_sections = c->layers * 2 * c->kv_heads;
  lo->chunks_per_sec = lo->T_mid > 0 ? (lo->T_mid + c->chunk_tokens - 1) / c->chunk_tokens : 0;
  lo->n_r_sections = 0;
  for (int32_t s = 0; s < 2; ++s)
    if (section_has_r(c, s)) lo->n_r_sections += c->layers * c->kv_heads;
  int64_t e_bytes = c->dtype == ORC_BF16 ? 2 : 4;
  lo->side_off = HDR_BYTES;
  lo->r_off = lo->side_off + (int64_t)lo->n_sections * SEC_REC(c->head_dim);
  lo->side_bytes = align16((int64_t)lo->n_sections * SEC_REC(c->head_dim) +
                           (int64_t)lo->n_r_sections * lo->T_mid * 4);
  lo->raw_off = lo->side_off + lo->side_bytes;
  lo->raw_bytes = align16(2 * (int64_t)c->layers * c->kv_heads * (lo->s0 + lo->W_eff) *
                          c->head_dim * e_bytes);
  lo->dir_off = lo->raw_off + lo->raw_bytes;
  lo->chunks_off = lo->dir_off + (int64_t)lo->n_sections * lo->chunks_per_sec * DIR_ENTRY;
  if (c->transform == ORC_PCA) {
    lo->budget_k = orc_budget(c->bits_k, c->head_dim);
    lo->budget_v = orc_budget(c->bits_v, c->head_dim);
  } else {
    lo->budget_k = uniform_bits(c->bits_k) * c->head_dim;
    lo->budget_v = uniform_bits(c->bits_v) * c->head_dim;
  }
}

/* r-area index of section u, or -1 */
static int64_t r_index(const orc_config* c, int32_t u) {
  int32_t H = c->kv_heads;
  int32_t h = u % H, s = (u / H) % 2, l = u / (2 * H);
  if (!section_has_r(c, s)) return -1;
  if (c->wht_keys) return u;
  return (int64_t)l * H + h; /* only value sections carry r */
}

static void put32(uint8_t* p, uint32_t v) { memcpy(p, &v, 4); }
static void put64(uint8_t* p, uint64_t v) { memcpy(p, &v, 8); }
static uint32_t get32(const uint8_t* p) { uint32_t v; memcpy(&v, p, 4); return v; }
static uint64_t get64(const uint8_t* p) { uint64_t v; memcpy(&v, p, 8); return v; }

static const float* basis_of(const orc_config* c, const float* basis, int32_t l, int32_t s, int32_t h) {
  int64_t DD = (int64_t)c->head_dim * c->head_dim;
  if (c->basis_per_head) return basis + (((int64_t)l * 2 + s) * c->kv_heads + h) * DD;
  return basis + ((int64_t)l * 2 + s) * DD;
}

/* 64-bit FNV-1a over the operand-precision basis bytes (bf16: 2 bytes,
 * fp32: 4 bytes per entry, little-endian), in storage order. */
uint64_t orc_fingerprint(const orc_config* c, const float* basis) {
  uint64_t h = 0xcbf29ce484222325ull;
  if (c->transform != ORC_PCA || basis == NULL) return h;
  int64_t n = (int64_t)c->layers * 2 * (c->basis_per_head ? c->kv_heads : 1) *
              c->head_dim * c->head_dim;
  for (int64_t i = 0; i < n; ++i) {
    uint8_t b[4];
    int nb;
    if (c->dtype == ORC_BF16) {
      uint16_t v = orc_f32_to_bf16(basis[i]);
      memcpy(b, &v, 2);
      nb = 2;
    } else {
      memcpy(b, &basis[i], 4);
      nb = 4;
    }
    for (int k = 0; k < nb; ++k) {
      h ^= b[k];
      h *= 0x100000001b3ull;
    }
  }
  return h;
}

static int64_t max_words(int64_t P, int32_t lanes, int32_t sb) {
  /* each symbol adds at most sb bits of state, each word removes 16 */
  return (P * (sb + 1)) / 16 + 2 * (int64_t)lanes + 2;
}

static int64_t max_record(const orc_config* c, int32_t ntok, int32_t budget) {
  int32_t D = c->head_dim;
  int32_t ntiles = (ntok + c->tile_tokens - 1) / c->tile_tokens;
  int32_t nz = budget < D ? budget : D; /* components with >= 1 bit */
  int64_t rec = 512 + 4 * (int64_t)ntiles;
  for (int32_t t = 0; t < ntiles; ++t) {
    int32_t n = ntok - t * c->tile_tokens;
    if (n > c->tile_tokens) n = c->tile_tokens;
    int64_t P = ((int64_t)n * budget + 7) / 8 + 4 * (int64_t)nz;
    rec += 4 * (int64_t)c->rans_lanes + 2 * max_words(P, c->rans_lanes, c->rans_scale_bits) + 2;
  }
  return align16(rec);
}

int64_t orc_max_container_bytes(const orc_config* c, int32_t T) {
  if (orc_check_config(c) != ORC_OK || T < 0) return -1;
  layout_t lo;
  make_layout(c, T, &lo);
  int64_t total = lo.chunks_off;
  for (int32_t u = 0; u < lo.n_sections; ++u) {
    int32_t s = (u / c->kv_heads) % 2;
    int32_t budget = s == 0 ? lo.budget_k : lo.budget_v;
    for (int32_t ch = 0; ch < lo.chunks_per_sec; ++ch) {
      int32_t n = lo.T_mid - ch * c->chunk_tokens;
      if (n > c->chunk_tokens) n = c->chunk_tokens;
      total += max_record(c, n, budget);
    }
  }
  return total;
}

/* Middle-region rows of section u, un-rotated (keys) and rounded to the
 * operand precision: x[T_mid][D]. Returns ORC_ERR_NONFINITE on NaN/Inf. */
static int gather_section(const orc_config* c, const void* k, const void* v, const layout_t* lo,
                          int32_t u, const float* cos_t, const float* sin_t, float* x) {
  int32_t D = c->head_dim, H = c->kv_heads;
  int32_t h = u % H, s = (u / H) % 2, l = u / (2 * H);
  const void* src = s == 0 ? k : v;
  float* y = (float*)malloc(sizeof(float) * D);
  for (int32_t t = 0; t < lo->T_mid; ++t) {
    int32_t pos = lo->mid_begin + t;
    int64_t base = (((int64_t)l * H + h) * lo->T + pos) * D;
    for (int32_t j = 0; j < D; ++j) {
      y[j] = load_elem(src, c->dtype, base + j);
      if (!isfinite(y[j])) {
        free(y);
        return ORC_ERR_NONFINITE;
      }
    }
    float* xr = x + (int64_t)t * D;
    if (s == 0 && c->rope_keys) {
      orc_rope_inverse(y, xr, D, c->rope_style, cos_t + (int64_t)pos * (D / 2),
                       sin_t + (int64_t)pos * (D / 2));
      for (int32_t j = 0; j < D; ++j) xr[j] = round_p(xr[j], c->dtype);
    } else {
      for (int32_t j = 0; j < D; ++j) xr[j] = y[j];
    }
  }
  free(y);
  return ORC_OK;
}

/* Coefficients c[T_mid][D] of section u from gathered rows x; r[T_mid] on the
 * WHT path (NULL-safe). */
static void transform_section(const orc_config* c, const float* basis, int32_t u,
                              int32_t T_mid, const float* x, float* coef, float* r) {
  int32_t D = c->head_dim, H = c->kv_heads;
  int32_t h = u % H, s = (u / H) % 2, l = u / (2 * H);
  if (c->transform == ORC_PCA) {
    const float* B = basis_of(c, basis, l, s, h);
    float* Bp = (float*)malloc(sizeof(float) * D * D);
    for (int64_t i = 0; i < (int64_t)D * D; ++i) Bp[i] = round_p(B[i], c->dtype);
    for (int32_t t = 0; t < T_mid; ++t) orc_project(x + (int64_t)t * D, Bp, D, coef + (int64_t)t * D);
    free(Bp);
    return;
  }
  if (!section_has_r(c, s)) { /* keys quantised directly ([TTAS] 2.1: no Hadamard) */
    memcpy(coef, x, sizeof(float) * (size_t)T_mid * D);
    return;
  }
  float* xn = (float*)malloc(sizeof(float) * D);
  for (int32_t t = 0; t < T_mid; ++t) {
    const float* xr = x + (int64_t)t * D;
    float rt = orc_rms(xr, D);
    if (r) r[t] = rt;
    for (int32_t j = 0; j < D; ++j) xn[j] = rt == 0.0f ? 0.0f : xr[j] / rt;
    orc_wht(xn, D, coef + (int64_t)t * D);
  }
  free(xn);
}

static void write_header(const orc_config* c, const layout_t* lo, uint64_t fp,
                         int64_t total, uint8_t* out) {
  memset(out, 0, HDR_BYTES);
  memcpy(out + 0, "KVTC", 4);
  put32(out + 4, 1);
  put32(out + 8, HDR_BYTES);
  put32(out + 12, 0);
  put32(out + 16, (uint32_t)c->layers);
  put32(out + 20, (uint32_t)c->kv_heads);
  put32(out + 24, (uint32_t)c->head_dim);
  put32(out + 28, (uint32_t)c->dtype);
  put32(out + 32, (uint32_t)c->transform);
  put32(out + 36, (uint32_t)c->sink_tokens);
  put32(out + 40, (uint32_t)c->recent_tokens);
  memcpy(out + 44, &c->bits_k, 4);
  memcpy(out + 48, &c->bits_v, 4);
  put32(out + 52, (uint32_t)c->max_bits);
  put32(out + 56, (uint32_t)c->rope_keys);
  put32(out + 60, (uint32_t)c->rope_style);
  memcpy(out + 64, &c->rope_theta, 8);
  put32(out + 72, (uint32_t)c->rans_scale_bits);
  put32(out + 76, (uint32_t)c->rans_lanes);
  put32(out + 80, (uint32_t)c->chunk_tokens);
  put32(out + 84, (uint32_t)c->tile_tokens);
  put32(out + 88, (uint32_t)c->basis_per_head);
  put32(out + 92, (uint32_t)c->wht_keys);
  put32(out + 96, (uint32_t)lo->T);
  put32(out + 100, (uint32_t)lo->s0);
  put32(out + 104, (uint32_t)lo->mid_begin);
  put32(out + 108, (uint32_t)lo->mid_end);
  put32(out + 112, (uint32_t)lo->n_sections);
  put32(out + 116, (uint32_t)lo->chunks_per_sec);
  put64(out + 120, (uint64_t)lo->side_off);
  put64(out + 128, (uint64_t)lo->side_bytes);
  put64(out + 136, (uint64_t)lo->raw_off);
  put64(out + 144, (uint64_t)lo->raw_bytes);
  put64(out + 152, (uint64_t)lo->dir_off);
  put64(out + 160, (uint64_t)lo->chunks_off);
  put64(out + 168, (uint64_t)total);
  put64(out + 176, fp);
  put32(out + 184, (uint32_t)lo->budget_k);
  put32(out + 188, (uint32_t)lo->budget_v);
}

/* Copy the sink and recent windows bit-exactly ([KVTC] "How the Pipeline
 * Works": sink tokens and the recent window stay in high fidelity). */
static void copy_raw(const orc_config* c, const layout_t* lo, const void* k, const void* v,
                     uint8_t* raw, int to_container) {
  int64_t e = c->dtype == ORC_BF16 ? 2 : 4;
  int64_t D = c->head_dim;
  int64_t pos = 0;
  for (int s = 0; s < 2; ++s) {
    uint8_t* t = (uint8_t*)(s == 0 ? k : v);
    for (int region = 0; region < 2; ++region) {
      int32_t t0 = region == 0 ? 0 : lo->mid_end;
      int32_t n = region == 0 ? lo->s0 : lo->W_eff;
      for (int32_t l = 0; l < c->layers; ++l)
        for (int32_t h = 0; h < c->kv_heads; ++h)
          for (int32_t tt = 0; tt < n; ++tt) {
            int64_t off = ((((int64_t)l * c->kv_heads + h) * lo->T) + t0 + tt) * D * e;
            if (to_container)
              memcpy(raw + pos, t + off, (size_t)(D * e));
            else
              memcpy(t + off, raw + pos, (size_t)(D * e));
            pos += D * e;
          }
    }
  }
}

typedef struct {
  uint8_t bits[256];
  float zero[256], scale[256], rcp[256];
} side_t;

/* Allocation and side information of one section from its coefficients. */
static void section_side(const orc_config* c, const layout_t* lo, int32_t u,
                         const float* coef, side_t* si) {
  int32_t D = c->head_dim, s = (u / c->kv_heads) % 2;
  int32_t N = lo->T_mid;
  float mu[256], var[256], mn[256], mx[256];
  orc_stats(coef, N, D, mu, var, mn, mx);
  if (c->transform == ORC_PCA) {
    orc_alloc_greedy(var, D, s == 0 ? lo->budget_k : lo->budget_v, c->max_bits, si->bits);
    orc_side_info(si->bits, mu, mn, mx, D, si->zero, si->scale, si->rcp);
    return;
  }
  if (s == 1) { /* values: uniform width, per-component range */
    for (int32_t i = 0; i < D; ++i) si->bits[i] = (uint8_t)uniform_bits(c->bits_v);
    orc_side_info(si->bits, mu, mn, mx, D, si->zero, si->scale, si->rcp);
    return;
  }
  /* keys: uniform width, one symmetric scale per section (per head) */
  int32_t b = uniform_bits(c->bits_k);
  float amax = 0.0f;
  for (int32_t i = 0; i < D; ++i) {
    float a = fabsf(mn[i]) > fabsf(mx[i]) ? fabsf(mn[i]) : fabsf(mx[i]);
    if (a > amax) amax = a;
  }
  int32_t Q = (1 << (b - 1)) - 1;
  float sc = (float)((double)amax / (double)Q);
  float r = sc > 0.0f ? 1.0f / sc : 0.0f;
  if (!(sc > 0.0f) || isinf(r)) {
    sc = 0.0f;
    r = 0.0f;
  }
  for (int32_t i = 0; i < D; ++i) {
    si->bits[i] = (uint8_t)b;
    si->zero[i] = 0.0f;
    si->scale[i] = sc;
    si->rcp[i] = r;
  }
}

static int sym_section(const orc_config* c, int32_t u) {
  return c->transform == ORC_WHT && ((u / c->kv_heads) % 2) == 0;
}

int orc_section_rows(const orc_config* c, const void* k, const void* v, int32_t T,
                     int32_t u, int32_t t0, int32_t t1, float* x_out) {
  int st = orc_check_config(c);
  if (st != ORC_OK) return st;
  if (u < 0 || u >= c->layers * 2 * c->kv_heads || t0 < 0 || t1 > T || t0 > t1)
    return ORC_ERR_INVALID_ARG;
  int32_t D = c->head_dim, H = c->kv_heads;
  int32_t h = u % H, s = (u / H) % 2, l = u / (2 * H);
  const void* src = s == 0 ? k : v;
  float cos_r[128], sin_r[128], y[256];
  for (int32_t t = t0; t < t1; ++t) {
    int64_t base = (((int64_t)l * H + h) * T + t) * D;
    for (int32_t j = 0; j < D; ++j) y[j] = load_elem(src, c->dtype, base + j);
    float* xr = x_out + (int64_t)(t - t0) * D;
    if (s == 0 && c->rope_keys) {
      for (int32_t j = 0; j < D / 2; ++j) {
        double a = (double)t * pow(c->rope_theta, -2.0 * (double)j / (double)D);
        cos_r[j] = (float)cos(a);
        sin_r[j] = (float)sin(a);
      }
      orc_rope_inverse(y, xr, D, c->rope_style, cos_r, sin_r);
      for (int32_t j = 0; j < D; ++j) xr[j] = round_p(xr[j], c->dtype);
    } else {
      for (int32_t j = 0; j < D; ++j) xr[j] = y[j];
    }
  }
  return ORC_OK;
}

int orc_section_coeffs(const orc_config* c, const void* k, const void* v, int32_t T,
                       const float* basis, int32_t u, float* c_out, float* r_out) {
  int st = orc_check_config(c);
  if (st != ORC_OK) return st;
  layout_t lo;
  make_layout(c, T, &lo);
  if (u < 0 || u >= lo.n_sections) return ORC_ERR_INVALID_ARG;
  int32_t D = c->head_dim;
  float* cos_t = (float*)malloc(sizeof(float) * ((size_t)T * D / 2 + 1));
  float* sin_t = (float*)malloc(sizeof(float) * ((size_t)T * D / 2 + 1));
  orc_rope_table(T, D, c->rope_theta, cos_t, sin_t);
  float* x = (float*)malloc(sizeof(float) * ((size_t)lo.T_mid * D + 1));
  st = gather_section(c, k, v, &lo, u, cos_t, sin_t, x);
  if (st == ORC_OK) transform_section(c, basis, u, lo.T_mid, x, c_out, r_out);
  free(x);
  free(cos_t);
  free(sin_t);
  return st;
}

/* Encode: regions, RoPE undo, transform, allocation, quantisation, packing,
 * rANS ([KVTC] "How the Pipeline Works": RoPE undo -> PCA transform -> bit
 * allocation -> quantization -> entropy coding). */
int orc_encode(const orc_config* c, const void* k, const void* v, int32_t T,
               const float* basis, uint8_t* out, int64_t cap, int64_t* out_bytes) {
  int st = orc_check_config(c);
  if (st != ORC_OK) return st;
  if (T < 0 || (c->transform == ORC_PCA && basis == NULL)) return ORC_ERR_INVALID_ARG;
  layout_t lo;
  make_layout(c, T, &lo);
  int32_t D = c->head_dim, L = c->layers, H = c->kv_heads;
  (void)L; (void)H;
  if (cap < lo.chunks_off) return ORC_ERR_CAPACITY;
  memset(out, 0, (size_t)lo.chunks_off);
  float* cos_t = (float*)malloc(sizeof(float) * ((size_t)T * D / 2 + 1));
  float* sin_t = (float*)malloc(sizeof(float) * ((size_t)T * D / 2 + 1));
  orc_rope_table(T, D, c->rope_theta, cos_t, sin_t);
  float* x = (float*)malloc(sizeof(float) * ((size_t)lo.T_mid * D + 1));
  float* coef = (float*)malloc(sizeof(float) * ((size_t)lo.T_mid * D + 1));
  float* r = (float*)malloc(sizeof(float) * ((size_t)lo.T_mid + 1));
  uint8_t* q = (uint8_t*)malloc((size_t)c->chunk_tokens * D + 1);
  uint8_t* packed = (uint8_t*)malloc((size_t)c->chunk_tokens * D + 64 * (size_t)D + 1);
  int64_t wcap = max_words((int64_t)c->tile_tokens * D + 4 * D, c->rans_lanes, c->rans_scale_bits);
  uint16_t* words = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)wcap);
  int64_t pos = lo.chunks_off;
  side_t si;
  for (int32_t u = 0; u < lo.n_sections && st == ORC_OK; ++u) {
    st = gather_section(c, k, v, &lo, u, cos_t, sin_t, x);
    if (st != ORC_OK) break;
    if (lo.T_mid == 0) continue;
    transform_section(c, basis, u, lo.T_mid, x, coef, r);
    section_side(c, &lo, u, coef, &si);
    /* section record */
    uint8_t* rec = out + lo.side_off + (int64_t)u * SEC_REC(D);
    memcpy(rec, si.bits, (size_t)D);
    memcpy(rec + D, si.zero, sizeof(float) * D);
    memcpy(rec + 5 * (int64_t)D, si.scale, sizeof(float) * D);
    int64_t ri = r_index(c, u);
    if (ri >= 0) memcpy(out + lo.r_off + ri * lo.T_mid * 4, r, sizeof(float) * (size_t)lo.T_mid);
    for (int32_t ch = 0; ch < lo.chunks_per_sec; ++ch) {
      int32_t t0 = ch * c->chunk_tokens;
      int32_t n = lo.T_mid - t0 < c->chunk_tokens ? lo.T_mid - t0 : c->chunk_tokens;
      if (sym_section(c, u))
        orc_quantize_sym(coef + (int64_t)t0 * D, n, D, si.bits[0], si.rcp[0], q, NULL);
      else
        orc_quantize(coef + (int64_t)t0 * D, n, D, si.bits, si.zero, si.rcp, q, NULL);
      int32_t ntiles = (n + c->tile_tokens - 1) / c->tile_tokens;
      int64_t tile_off[1024 + 1];
      if (ntiles > 1024) { st = ORC_ERR_UNSUPPORTED; break; }
      tile_off[0] = 0;
      for (int32_t tl = 0; tl < ntiles; ++tl) {
        int32_t a = tl * c->tile_tokens;
        int32_t m = n - a < c->tile_tokens ? n - a : c->tile_tokens;
        orc_pack(q + (int64_t)a * D, m, D, si.bits, packed + tile_off[tl]);
        tile_off[tl + 1] = tile_off[tl] + orc_packed_bytes(si.bits, D, m);
      }
      int64_t P = tile_off[ntiles];
      int64_t dir = lo.dir_off + ((int64_t)u * lo.chunks_per_sec + ch) * DIR_ENTRY;
      if (P == 0) { /* every component at 0 bits: empty record */
        if (cap < lo.chunks_off) { st = ORC_ERR_CAPACITY; break; }
        put64(out + dir, (uint64_t)pos);
        put32(out + dir + 8, 0);
        put32(out + dir + 12, 0);
        continue;
      }
      uint32_t counts[256] = {0};
      for (int64_t b = 0; b < P; ++b) counts[packed[b]]++;
      uint16_t freq[256];
      orc_freq_normalize(counts, c->rans_scale_bits, freq);
      int64_t start = pos;
      int64_t p = pos + 512 + 4 * (int64_t)ntiles;
      if (p > cap) { st = ORC_ERR_CAPACITY; break; }
      memcpy(out + pos, freq, 512);
      for (int32_t tl = 0; tl < ntiles && st == ORC_OK; ++tl) {
        uint32_t states[64];
        int64_t nw = orc_rans_encode(packed + tile_off[tl], tile_off[tl + 1] - tile_off[tl], freq,
                                     c->rans_scale_bits, c->rans_lanes, states, words, wcap);
        if (nw < 0) { st = ORC_ERR_CAPACITY; break; }
        int64_t need = 4 * (int64_t)c->rans_lanes + 2 * nw + (nw & 1 ? 2 : 0);
        if (p + need > cap) { st = ORC_ERR_CAPACITY; break; }
        put32(out + pos + 512 + 4 * (int64_t)tl, (uint32_t)nw);
        memcpy(out + p, states, 4 * (size_t)c->rans_lanes);
        memcpy(out + p + 4 * (int64_t)c->rans_lanes, words, 2 * (size_t)nw);
        if (nw & 1) memset(out + p + 4 * (int64_t)c->rans_lanes + 2 * nw, 0, 2);
        p += need;
      }
      if (st != ORC_OK) break;
      int64_t end = align16(p);
      if (end > cap) { st = ORC_ERR_CAPACITY; break; }
      memset(out + p, 0, (size_t)(end - p));
      put64(out + dir, (uint64_t)start);
      put32(out + dir + 8, (uint32_t)(end - start));
      put32(out + dir + 12, 0);
      pos = end;
    }
  }
  if (st == ORC_OK) {
    copy_raw(c, &lo, k, v, out + lo.raw_off, 1);
    write_header(c, &lo, orc_fingerprint(c, basis), pos, out);
    *out_bytes = pos;
  }
  free(x); free(coef); free(r); free(q); free(packed); free(words);
  free(cos_t); free(sin_t);
  return st;
}

/* ---- decode ---------------------------------------------------------- */

static int parse_header(const orc_config* c, const float* basis, const uint8_t* in,
                        int64_t n, layout_t* lo) {
  if (n < HDR_BYTES) return ORC_ERR_CORRUPT;
  if (memcmp(in, "KVTC", 4) != 0 || get32(in + 4) != 1 || get32(in + 8) != HDR_BYTES)
    return ORC_ERR_CORRUPT;
  orc_config h;
  memset(&h, 0, sizeof h);
  h.layers = (int32_t)get32(in + 16);
  h.kv_heads = (int32_t)get32(in + 20);
  h.head_dim = (int32_t)get32(in + 24);
  h.dtype = (int32_t)get32(in + 28);
  h.transform = (int32_t)get32(in + 32);
  h.sink_tokens = (int32_t)get32(in + 36);
  h.recent_tokens = (int32_t)get32(in + 40);
  memcpy(&h.bits_k, in + 44, 4);
  memcpy(&h.bits_v, in + 48, 4);
  h.max_bits = (int32_t)get32(in + 52);
  h.rope_keys = (int32_t)get32(in + 56);
  h.rope_style = (int32_t)get32(in + 60);
  memcpy(&h.rope_theta, in + 64, 8);
  h.rans_scale_bits = (int32_t)get32(in + 72);
  h.rans_lanes = (int32_t)get32(in + 76);
  h.chunk_tokens = (int32_t)get32(in + 80);
  h.tile_tokens = (int32_t)get32(in + 84);
  h.basis_per_head = (int32_t)get32(in + 88);
  h.wht_keys = (int32_t)get32(in + 92);
  if (h.layers != c->layers || h.kv_heads != c->kv_heads || h.head_dim != c->head_dim ||
      h.dtype != c->dtype || h.transform != c->transform || h.sink_tokens != c->sink_tokens ||
      h.recent_tokens != c->recent_tokens || memcmp(&h.bits_k, &c->bits_k, 4) ||
      memcmp(&h.bits_v, &c->bits_v, 4) || h.max_bits != c->max_bits ||
      h.rope_keys != c->rope_keys || h.rope_style != c->rope_style ||
      memcmp(&h.rope_theta, &c->rope_theta, 8) || h.rans_scale_bits != c->rans_scale_bits ||
      h.rans_lanes != c->rans_lanes || h.chunk_tokens != c->chunk_tokens ||
      h.tile_tokens != c->tile_tokens || h.basis_per_head != c->basis_per_head ||
      h.wht_keys != c->wht_keys)
    return ORC_ERR_CORRUPT;
  int32_t T = (int32_t)get32(in + 96);
  if (T < 0) return ORC_ERR_CORRUPT;
  make_layout(c, T, lo);
  if ((int32_t)get32(in + 100) != lo->s0 || (int32_t)get32(in + 104) != lo->mid_begin ||
      (int32_t)get32(in + 108) != lo->mid_end || (int32_t)get32(in + 112) != lo->n_sections ||
      (int32_t)get32(in + 116) != lo->chunks_per_sec ||
      get64(in + 120) != (uint64_t)lo->side_off || get64(in + 128) != (uint64_t)lo->side_bytes ||
      get64(in + 136) != (uint64_t)lo->raw_off || get64(in + 144) != (uint64_t)lo->raw_bytes ||
      get64(in + 152) != (uint64_t)lo->dir_off || get64(in + 160) != (uint64_t)lo->chunks_off ||
      (int32_t)get32(in + 184) != lo->budget_k || (int32_t)get32(in + 188) != lo->budget_v)
    return ORC_ERR_CORRUPT;
  uint64_t total = get64(in + 168);
  if (total > (uint64_t)n || total < (uint64_t)lo->chunks_off) return ORC_ERR_CORRUPT;
  if (get64(in + 176) != orc_fingerprint(c, basis)) return ORC_ERR_CORRUPT;
  return ORC_OK;
}

/* Decode the codes of chunk ch of section u into q[n][D]. */
static int decode_chunk_codes(const orc_config* c, const layout_t* lo, const uint8_t* in,
                              int64_t total, int32_t u, int32_t ch, const uint8_t* bits,
                              uint8_t* q, uint8_t* packed, uint8_t* syms) {
  int32_t D = c->head_dim;
  int32_t t0 = ch * c->chunk_tokens;
  int32_t n = lo->T_mid - t0 < c->chunk_tokens ? lo->T_mid - t0 : c->chunk_tokens;
  int32_t ntiles = (n + c->tile_tokens - 1) / c->tile_tokens;
  int64_t dir = lo->dir_off + ((int64_t)u * lo->chunks_per_sec + ch) * DIR_ENTRY;
  uint64_t off = get64(in + dir);
  uint32_t size = get32(in + dir + 8);
  if (get32(in + dir + 12) != 0) return ORC_ERR_CORRUPT;
  int64_t P = 0;
  for (int32_t tl = 0; tl < ntiles; ++tl) {
    int32_t m = n - tl * c->tile_tokens < c->tile_tokens ? n - tl * c->tile_tokens : c->tile_tokens;
    P += orc_packed_bytes(bits, D, m);
  }
  if (P == 0) {
    if (size != 0) return ORC_ERR_CORRUPT;
    for (int64_t i = 0; i < (int64_t)n * D; ++i) q[i] = 0;
    return ORC_OK;
  }
  if (off < (uint64_t)lo->chunks_off || (off & 15) || off + size > (uint64_t)total) return ORC_ERR_CORRUPT;
  const uint8_t* rec = in + off;
  if (size < 512 + 4 * (uint32_t)ntiles) return ORC_ERR_CORRUPT;
  uint16_t freq[256];
  memcpy(freq, rec, 512);
  int64_t p = 512 + 4 * (int64_t)ntiles;
  int64_t done = 0;
  for (int32_t tl = 0; tl < ntiles; ++tl) {
    int32_t a = tl * c->tile_tokens;
    int32_t m = n - a < c->tile_tokens ? n - a : c->tile_tokens;
    int64_t Pt = orc_packed_bytes(bits, D, m);
    uint32_t nw = get32(rec + 512 + 4 * (int64_t)tl);
    int64_t need = 4 * (int64_t)c->rans_lanes + 2 * (int64_t)nw + (nw & 1 ? 2 : 0);
    if (p + need > (int64_t)size) return ORC_ERR_CORRUPT;
    uint32_t states[64];
    memcpy(states, rec + p, 4 * (size_t)c->rans_lanes);
    uint16_t* w = (uint16_t*)malloc(sizeof(uint16_t) * ((size_t)nw + 1));
    memcpy(w, rec + p + 4 * (int64_t)c->rans_lanes, 2 * (size_t)nw);
    int st = orc_rans_decode(states, w, nw, freq, c->rans_scale_bits, c->rans_lanes, Pt, syms);
    free(w);
    if (st != ORC_OK) return st;
    memcpy(packed + done, syms, (size_t)Pt);
    orc_unpack(packed + done, m, D, bits, q + (int64_t)a * D);
    done += Pt;
    p += need;
  }
  if (align16(p) != (int64_t)size) return ORC_ERR_CORRUPT;
  return ORC_OK;
}

/* Reconstruct the middle rows of section u (before RoPE and the output
 * cast): xo[T_mid][D] fp32. */
static int decode_section_mid(const orc_config* c, const float* basis, const layout_t* lo,
                              const uint8_t* in, int64_t total, int32_t u, float* xo) {
  int32_t D = c->head_dim, H = c->kv_heads;
  int32_t h = u % H, s = (u / H) % 2, l = u / (2 * H);
  const uint8_t* rec = in + lo->side_off + (int64_t)u * SEC_REC(D);
  uint8_t bits[256];
  float zero[256], scale[256];
  memcpy(bits, rec, (size_t)D);
  memcpy(zero, rec + D, sizeof(float) * D);
  memcpy(scale, rec + 5 * (int64_t)D, sizeof(float) * D);
  for (int32_t i = 0; i < D; ++i)
    if (bits[i] > c->max_bits) return ORC_ERR_CORRUPT;
  const float* rarea = NULL;
  int64_t ri = r_index(c, u);
  if (ri >= 0) rarea = (const float*)(in + lo->r_off + ri * lo->T_mid * 4);
  float* Bp = NULL;
  if (c->transform == ORC_PCA) {
    const float* B = basis_of(c, basis, l, s, h);
    Bp = (float*)malloc(sizeof(float) * D * D);
    for (int64_t i = 0; i < (int64_t)D * D; ++i) Bp[i] = round_p(B[i], c->dtype);
  }
  uint8_t* q = (uint8_t*)malloc((size_t)c->chunk_tokens * D + 1);
  uint8_t* packed = (uint8_t*)malloc((size_t)c->chunk_tokens * D + 64 * (size_t)D + 1);
  uint8_t* syms = (uint8_t*)malloc((size_t)c->tile_tokens * D + 64 * (size_t)D + 1);
  float chat[256], tmp[256];
  int st = ORC_OK;
  int sym = sym_section(c, u);
  int32_t off = sym ? 1 << (bits[0] - 1) : 0;
  for (int32_t ch = 0; ch < lo->chunks_per_sec && st == ORC_OK; ++ch) {
    int32_t t0 = ch * c->chunk_tokens;
    int32_t n = lo->T_mid - t0 < c->chunk_tokens ? lo->T_mid - t0 : c->chunk_tokens;
    st = decode_chunk_codes(c, lo, in, total, u, ch, bits, q, packed, syms);
    if (st != ORC_OK) break;
    for (int32_t t = 0; t < n; ++t) {
      const uint8_t* qr = q + (int64_t)t * D;
      for (int32_t i = 0; i < D; ++i) {
        if (sym)
          chat[i] = (float)((int32_t)qr[i] - off) * scale[i];
        else
          chat[i] = fmaf((float)qr[i], scale[i], zero[i]);
      }
      float* xr = xo + (int64_t)(t0 + t) * D;
      if (c->transform == ORC_PCA) {
        for (int32_t i = 0; i < D; ++i) chat[i] = round_p(chat[i], c->dtype);
        orc_unproject(chat, Bp, D, xr);
      } else if (rarea) {
        float rt;
        memcpy(&rt, &rarea[t0 + t], 4);
        orc_wht(chat, D, tmp);
        for (int32_t j = 0; j < D; ++j) xr[j] = tmp[j] * rt;
      } else {
        for (int32_t j = 0; j < D; ++j) xr[j] = chat[j];
      }
    }
  }
  free(q); free(packed); free(syms); free(Bp);
  return st;
}

int orc_decode(const orc_config* c, const float* basis, const uint8_t* in, int64_t n,
               void* k_out, void* v_out, int32_t out_dtype) {
  int st = orc_check_config(c);
  if (st != ORC_OK) return st;
  if (out_dtype != ORC_FP32 && out_dtype != ORC_BF16) return ORC_ERR_INVALID_ARG;
  layout_t lo;
  st = parse_header(c, basis, in, n, &lo);
  if (st != ORC_OK) return st;
  int64_t total = (int64_t)get64(in + 168);
  int32_t D = c->head_dim, H = c->kv_heads, T = lo.T;
  float* cos_t = (float*)malloc(sizeof(float) * ((size_t)T * D / 2 + 1));
  float* sin_t = (float*)malloc(sizeof(float) * ((size_t)T * D / 2 + 1));
  orc_rope_table(T, D, c->rope_theta, cos_t, sin_t);
  float* xo = (float*)malloc(sizeof(float) * ((size_t)lo.T_mid * D + 1));
  float y[256];
  for (int32_t u = 0; u < lo.n_sections && st == ORC_OK; ++u) {
    if (lo.T_mid == 0) break;
    st = decode_section_mid(c, basis, &lo, in, total, u, xo);
    if (st != ORC_OK) break;
    int32_t h = u % H, s = (u / H) % 2, l = u / (2 * H);
    void* dst = s == 0 ? k_out : v_out;
    for (int32_t t = 0; t < lo.T_mid; ++t) {
      int32_t pos = lo.mid_begin + t;
      const float* xr = xo + (int64_t)t * D;
      if (s == 0 && c->rope_keys)
        orc_rope_forward(xr, y, D, c->rope_style, cos_t + (int64_t)pos * (D / 2),
                         sin_t + (int64_t)pos * (D / 2));
      else
        memcpy(y, xr, sizeof(float) * D);
      int64_t base = (((int64_t)l * H + h) * T + pos) * D;
      for (int32_t j = 0; j < D; ++j) store_elem(dst, out_dtype, base + j, y[j]);
    }
  }
  if (st == ORC_OK) {
    /* raw windows: bit-exact in the cache dtype, converted if out_dtype differs */
    if (out_dtype == c->dtype) {
      copy_raw(c, &lo, k_out, v_out, (uint8_t*)(in + lo.raw_off), 0);
    } else {
      int64_t e = c->dtype == ORC_BF16 ? 2 : 4;
      int64_t cnt = 2 * (int64_t)c->layers * H * (lo.s0 + lo.W_eff) * D;
      uint8_t* tmpk = (uint8_t*)malloc((size_t)((int64_t)c->layers * H * T * D * e + 1));
      uint8_t* tmpv = (uint8_t*)malloc((size_t)((int64_t)c->layers * H * T * D * e + 1));
      copy_raw(c, &lo, tmpk, tmpv, (uint8_t*)(in + lo.raw_off), 0);
      for (int s = 0; s < 2; ++s) {
        uint8_t* tsrc = s == 0 ? tmpk : tmpv;
        void* dst = s == 0 ? k_out : v_out;
        for (int region = 0; region < 2; ++region) {
          int32_t t0 = region == 0 ? 0 : lo.mid_end;
          int32_t m = region == 0 ? lo.s0 : lo.W_eff;
          for (int32_t l = 0; l < c->layers; ++l)
            for (int32_t h = 0; h < H; ++h)
              for (int32_t tt = 0; tt < m; ++tt)
                for (int32_t j = 0; j < D; ++j) {
                  int64_t idx = (((int64_t)l * H + h) * T + t0 + tt) * D + j;
                  store_elem(dst, out_dtype, idx, load_elem(tsrc, c->dtype, idx));
                }
        }
      }
      (void)cnt;
      free(tmpk);
      free(tmpv);
    }
  }
  free(xo); free(cos_t); free(sin_t);
  return st;
}

int orc_decode_sections(const orc_config* c, const float* basis, const uint8_t* in,
                        int64_t n, int32_t sec_begin, int32_t sec_end, float* mid_out) {
  int st = orc_check_config(c);
  if (st != ORC_OK) return st;
  layout_t lo;
  st = parse_header(c, basis, in, n, &lo);
  if (st != ORC_OK) return st;
  if (sec_begin < 0 || sec_end > lo.n_sections || sec_begin > sec_end) return ORC_ERR_INVALID_ARG;
  int64_t total = (int64_t)get64(in + 168);
  int32_t D = c->head_dim, H = c->kv_heads, T = lo.T;
  float* cos_t = (float*)malloc(sizeof(float) * ((size_t)T * D / 2 + 1));
  float* sin_t = (float*)malloc(sizeof(float) * ((size_t)T * D / 2 + 1));
  orc_rope_table(T, D, c->rope_theta, cos_t, sin_t);
  for (int32_t u = sec_begin; u < sec_end && st == ORC_OK; ++u) {
    float* xo = mid_out + (int64_t)(u - sec_begin) * lo.T_mid * D;
    st = decode_section_mid(c, basis, &lo, in, total, u, xo);
    if (st != ORC_OK || !(((u / H) % 2) == 0 && c->rope_keys)) continue;
    float y[256];
    for (int32_t t = 0; t < lo.T_mid; ++t) {
      int32_t pos = lo.mid_begin + t;
      float* xr = xo + (int64_t)t * D;
      orc_rope_forward(xr, y, D, c->rope_style, cos_t + (int64_t)pos * (D / 2),
                       sin_t + (int64_t)pos * (D / 2));
      memcpy(xr, y, sizeof(float) * D);
    }
  }
  free(cos_t);
  free(sin_t);
  return st;
}

int orc_section_codes(const orc_config* c, const float* basis, const uint8_t* in, int64_t n,
                      int32_t u, uint8_t* q_out) {
  int st = orc_check_config(c);
  if (st != ORC_OK) return st;
  layout_t lo;
  st = parse_header(c, basis, in, n, &lo);
  if (st != ORC_OK) return st;
  if (u < 0 || u >= lo.n_sections) return ORC_ERR_INVALID_ARG;
  int32_t D = c->head_dim;
  int64_t total = (int64_t)get64(in + 168);
  const uint8_t* rec = in + lo.side_off + (int64_t)u * SEC_REC(D);
  uint8_t bits[256];
  memcpy(bits, rec, (size_t)D);
  for (int32_t i = 0; i < D; ++i)
    if (bits[i] > c->max_bits) return ORC_ERR_CORRUPT;
  uint8_t* packed = (uint8_t*)malloc((size_t)c->chunk_tokens * D + 64 * (size_t)D + 1);
  uint8_t* syms = (uint8_t*)malloc((size_t)c->tile_tokens * D + 64 * (size_t)D + 1);
  for (int32_t ch = 0; ch < lo.chunks_per_sec && st == ORC_OK; ++ch)
    st = decode_chunk_codes(c, &lo, in, total, u, ch, bits,
                            q_out + (int64_t)ch * c->chunk_tokens * D, packed, syms);
  free(packed);
  free(syms);
  return st;
}
