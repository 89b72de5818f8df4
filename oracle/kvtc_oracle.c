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

/* little-endian field access (the host is little-endian) */
static void put32(uint8_t* p, uint32_t v) { memcpy(p, &v, 4); }
static void put64(uint8_t* p, uint64_t v) { memcpy(p, &v, 8); }
static uint32_t get32(const uint8_t* p) { uint32_t v; memcpy(&v, p, 4); return v; }
static uint64_t get64(const uint8_t* p) { uint64_t v; memcpy(&v, p, 8); return v; }

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
 * ([TTAS] 2.2: values pass through a Hadamard transform before quantisation;
 * [CG] Hadamard control):
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

/* The same greedy allocation over n components of any number of sections
 * (one budget over all of them, "Bit Budget Is Not Fair": the budget moves
 * toward the hard parts), with a binary max-heap holding each candidate's
 * next marginal gain var * 4^-b (exact in fp64); ties go to the lowest index
 * as in orc_alloc_greedy, which it equals on every input. */
static int gain_before(const double* g, const int64_t* id, int64_t a, int64_t b) {
  return g[a] > g[b] || (g[a] == g[b] && id[a] < id[b]);
}

static void gain_sift_down(double* g, int64_t* id, int64_t m, int64_t at) {
  for (;;) {
    int64_t l = 2 * at + 1, r = l + 1, top = at;
    if (l < m && gain_before(g, id, l, top)) top = l;
    if (r < m && gain_before(g, id, r, top)) top = r;
    if (top == at) return;
    double tg = g[at]; g[at] = g[top]; g[top] = tg;
    int64_t ti = id[at]; id[at] = id[top]; id[top] = ti;
    at = top;
  }
}

void orc_alloc_greedy_heap(const float* var, int64_t n, int64_t budget, int32_t max_bits,
                           uint8_t* bits) {
  double* g = (double*)malloc(sizeof(double) * (size_t)(n + 1));
  int64_t* id = (int64_t*)malloc(sizeof(int64_t) * (size_t)(n + 1));
  int64_t m = 0;
  for (int64_t i = 0; i < n; ++i) {
    bits[i] = 0;
    if (max_bits > 0 && var[i] > 0.0f) {
      g[m] = (double)var[i];
      id[m] = i;
      ++m;
    }
  }
  for (int64_t at = m / 2 - 1; at >= 0; --at) gain_sift_down(g, id, m, at);
  for (int64_t step = 0; step < budget && m > 0; ++step) {
    int64_t i = id[0];
    bits[i] += 1;
    if (bits[i] >= max_bits) { /* no further gain: drop the candidate */
      --m;
      g[0] = g[m];
      id[0] = id[m];
    } else {
      g[0] = ldexp((double)var[i], -2 * (int)bits[i]);
    }
    gain_sift_down(g, id, m, 0);
  }
  free(g);
  free(id);
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

/* Frequencies summing to M = 2^scale_bits from the counts of an alphabet of
 * n_sym symbols: each present symbol gets max(1, round-half-up(n_s M / N));
 * a positive remainder goes to the most frequent symbol (lowest symbol on
 * ties), an excess is removed one unit at a time from the symbol with the
 * largest frequency above 1 (lowest symbol on ties).  All zero when N = 0. */
void orc_freq_normalize(const uint32_t* counts, int32_t n_sym, int32_t scale_bits, uint16_t* freq) {
  uint64_t N = 0;
  for (int s = 0; s < n_sym; ++s) N += counts[s];
  int64_t M = (int64_t)1 << scale_bits;
  if (N == 0) {
    for (int s = 0; s < n_sym; ++s) freq[s] = 0;
    return;
  }
  int64_t f[256];
  int64_t sum = 0;
  for (int s = 0; s < n_sym; ++s) {
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
    for (int s = 1; s < n_sym; ++s)
      if (counts[s] > counts[best]) best = s;
    f[best] += d;
  }
  while (d < 0) {
    int best = -1;
    for (int s = 0; s < n_sym; ++s)
      if (f[s] > 1 && (best < 0 || f[s] > f[best])) best = s;
    f[best] -= 1;
    d += 1;
  }
  for (int s = 0; s < n_sym; ++s) freq[s] = (uint16_t)f[s];
}

/* Interleaved rANS over a sequence of N symbols given in decoding order
 * (Duda's range variant of ANS; interleaving after Giesen).  Symbol p is
 * coded by state lane[p] (of `lanes` 32-bit states in [2^16, 2^32), 16-bit
 * renormalisation words) with the frequency table that starts at
 * freqs[tab[p]] and has n_sym[p] entries summing to M = 2^scale_bits.
 *
 * Encoding walks the sequence from the last symbol to the first.  Before a
 * symbol of frequency f is coded, a state x >= f 2^(32 - scale_bits) emits
 * its low 16 bits as one word and shifts them out; then
 * x = floor(x / f) M + (x mod f) + cum, cum being the sum of the
 * frequencies of the smaller symbols.  Words are stored in emission order.
 * Decoding walks the sequence forwards: slot = x mod M selects the symbol
 * whose cumulative range holds it, x = f floor(x / M) + slot - cum, and a
 * state below 2^16 takes the last unread word as its new low 16 bits.
 *
 * Returns the number of words, or -1 when words_cap is too small or a
 * symbol has frequency 0. */
int64_t orc_rans_encode_seq(int64_t N, const uint8_t* sym, const uint8_t* lane, const int32_t* tab,
                            const int32_t* n_sym, const uint16_t* freqs, int32_t scale_bits,
                            int32_t lanes, uint32_t* states, uint16_t* words, int64_t words_cap) {
  for (int32_t j = 0; j < lanes; ++j) states[j] = ORC_RANS_L;
  int64_t n = 0;
  for (int64_t p = N - 1; p >= 0; --p) {
    const uint16_t* fr = freqs + tab[p];
    uint32_t s = sym[p];
    if ((int32_t)s >= n_sym[p]) return -1;
    uint32_t f = fr[s];
    if (f == 0) return -1;
    uint32_t cum = 0;
    for (uint32_t k = 0; k < s; ++k) cum += fr[k];
    uint32_t x = states[lane[p]];
    if ((uint64_t)x >= ((uint64_t)f << (32 - scale_bits))) {
      if (n >= words_cap) return -1;
      words[n++] = (uint16_t)(x & 0xffffu);
      x >>= 16;
    }
    x = ((x / f) << scale_bits) + (x % f) + cum;
    states[lane[p]] = x;
  }
  return n;
}

/* Inverse of orc_rans_encode_seq.  Returns ORC_OK, or ORC_ERR_CORRUPT when a
 * table does not sum to M, the words run out or are left over, or a final
 * state differs from the initial state 2^16. */
int orc_rans_decode_seq(int64_t N, const uint8_t* lane, const int32_t* tab, const int32_t* n_sym,
                        const uint16_t* freqs, int32_t scale_bits, int32_t lanes,
                        const uint32_t* states, const uint16_t* words, int64_t nwords,
                        uint8_t* sym) {
  uint32_t M = 1u << scale_bits;
  uint32_t x[64];
  for (int32_t j = 0; j < lanes; ++j) {
    x[j] = states[j];
    if (x[j] < ORC_RANS_L) return ORC_ERR_CORRUPT;
  }
  int64_t ptr = nwords; /* words are consumed from the last one backwards */
  for (int64_t p = 0; p < N; ++p) {
    const uint16_t* fr = freqs + tab[p];
    uint32_t total = 0;
    for (int32_t k = 0; k < n_sym[p]; ++k) total += fr[k];
    if (total != M) return ORC_ERR_CORRUPT;
    uint32_t j = lane[p];
    uint32_t slot = x[j] & (M - 1);
    uint32_t cum = 0;
    int s = 0;
    while (!(slot < cum + fr[s])) cum += fr[s++]; /* the symbol whose range holds slot */
    sym[p] = (uint8_t)s;
    x[j] = fr[s] * (x[j] >> scale_bits) + slot - cum;
    if (x[j] < ORC_RANS_L) {
      if (ptr <= 0) return ORC_ERR_CORRUPT;
      x[j] = (x[j] << 16) | words[--ptr];
      if (x[j] < ORC_RANS_L) return ORC_ERR_CORRUPT;
    }
  }
  if (ptr != 0) return ORC_ERR_CORRUPT;
  for (int32_t j = 0; j < lanes; ++j)
    if (x[j] != ORC_RANS_L) return ORC_ERR_CORRUPT;
  return ORC_OK;
}

/* One stream of N byte symbols with a single 256-entry table, symbol i on
 * lane i mod lanes: the sequence coder with uniform lanes and table. */
static void single_table_seq(int64_t N, int32_t lanes, uint8_t* lane, int32_t* tab, int32_t* n_sym) {
  for (int64_t i = 0; i < N; ++i) {
    lane[i] = (uint8_t)(i % lanes);
    tab[i] = 0;
    n_sym[i] = 256;
  }
}

int64_t orc_rans_encode(const uint8_t* sym, int64_t N, const uint16_t* freq,
                        int32_t scale_bits, int32_t lanes, uint32_t* states,
                        uint16_t* words, int64_t words_cap) {
  uint8_t* lane = (uint8_t*)malloc((size_t)N + 1);
  int32_t* tab = (int32_t*)malloc(sizeof(int32_t) * ((size_t)N + 1));
  int32_t* ns = (int32_t*)malloc(sizeof(int32_t) * ((size_t)N + 1));
  single_table_seq(N, lanes, lane, tab, ns);
  int64_t n = orc_rans_encode_seq(N, sym, lane, tab, ns, freq, scale_bits, lanes, states, words, words_cap);
  free(lane); free(tab); free(ns);
  return n;
}

int orc_rans_decode(const uint32_t* states, const uint16_t* words, int64_t nwords,
                    const uint16_t* freq, int32_t scale_bits, int32_t lanes,
                    int64_t N, uint8_t* sym) {
  uint8_t* lane = (uint8_t*)malloc((size_t)N + 1);
  int32_t* tab = (int32_t*)malloc(sizeof(int32_t) * ((size_t)N + 1));
  int32_t* ns = (int32_t*)malloc(sizeof(int32_t) * ((size_t)N + 1));
  single_table_seq(N, lanes, lane, tab, ns);
  int st = orc_rans_decode_seq(N, lane, tab, ns, freq, scale_bits, lanes, states, words, nwords, sym);
  free(lane); free(tab); free(ns);
  return st;
}

/* ===================================================================== */
/* Chunk records: what the entropy coder models ([KVTC] "rANS Makes the    */
/* Last Mile Smaller": codes that occur more often should cost less)       */
/* ===================================================================== */

/* A component of width b >= 2 contributes one symbol per token: the top
 * min(b, 4) bits of its code, coded with that component's own frequency
 * table over the chunk (2^min(b,4) entries).  The remaining low bits of a
 * wider code (b - 4 of them when b >= 5) and the whole code of a 1-bit
 * component are stored as raw bits. */
int32_t orc_sym_bits(int32_t b) { return b >= 2 ? (b < 4 ? b : 4) : 0; }
int32_t orc_raw_bits(int32_t b) { return b == 1 ? 1 : (b >= 5 ? b - 4 : 0); }

/* Bytes of a record's frequency tables (u16 each), padded to 4 bytes. */
static int64_t table_bytes(const uint8_t* bits, int32_t D) {
  int64_t n = 0;
  for (int32_t i = 0; i < D; ++i)
    if (orc_sym_bits(bits[i]) > 0) n += (int64_t)1 << orc_sym_bits(bits[i]);
  return (2 * n + 3) & ~(int64_t)3;
}

/* Bytes of a tile's raw rows: per component with raw bits r > 0, in index
 * order, ceil(m r / 32) little-endian words, bits LSB-first. */
static int64_t raw_row_bytes(const uint8_t* bits, int32_t D, int64_t m) {
  int64_t n = 0;
  for (int32_t i = 0; i < D; ++i) {
    int32_t r = orc_raw_bits(bits[i]);
    if (r > 0) n += 4 * ((m * r + 31) / 32);
  }
  return n;
}

/* Symbols of one tile of m tokens (codes q[m][D]) in decoding order: the
 * components with symbol bits in index order, and within a component the
 * tokens in order; the k-th symbol of a component goes to lane k mod lanes
 * and uses that component's table (tab_off[i] into the record's tables). */
static int64_t tile_sequence(const uint8_t* q, int32_t m, int32_t D, const uint8_t* bits, int32_t lanes,
                             const int32_t* tab_off, uint8_t* sym, uint8_t* lane, int32_t* tab,
                             int32_t* n_sym) {
  int64_t p = 0;
  for (int32_t i = 0; i < D; ++i) {
    int32_t h = orc_sym_bits(bits[i]);
    if (h == 0) continue;
    int32_t r = bits[i] - h;
    for (int32_t k = 0; k < m; ++k) {
      if (sym) sym[p] = (uint8_t)(q[(int64_t)k * D + i] >> r);
      lane[p] = (uint8_t)(k % lanes);
      tab[p] = tab_off[i];
      n_sym[p] = 1 << h;
      ++p;
    }
  }
  return p;
}

static void put_bits(uint8_t* row, int64_t at, uint32_t v, int32_t nb) {
  for (int32_t bit = 0; bit < nb; ++bit)
    if ((v >> bit) & 1u) row[(at + bit) / 8] |= (uint8_t)(1u << ((at + bit) % 8));
}

static uint32_t get_bits(const uint8_t* row, int64_t at, int32_t nb) {
  uint32_t v = 0;
  for (int32_t bit = 0; bit < nb; ++bit)
    if ((row[(at + bit) / 8] >> ((at + bit) % 8)) & 1u) v |= 1u << bit;
  return v;
}

static int64_t seq_words_cap(int64_t nsym, int32_t lanes, int32_t sb) {
  /* each symbol adds at most sb bits of state, each word removes 16 */
  return (nsym * (sb + 1)) / 16 + 2 * (int64_t)lanes + 2;
}

/* Packed size of a chunk of n tokens: its tiles' packed rows back to back. */
static int64_t chunk_packed_bytes(const orc_config* c, const uint8_t* bits, int32_t n) {
  int64_t P = 0;
  for (int32_t a = 0; a < n; a += c->tile_tokens) {
    int32_t m = n - a < c->tile_tokens ? n - a : c->tile_tokens;
    P += orc_packed_bytes(bits, c->head_dim, m);
  }
  return P;
}

/* Encode the record of one chunk (codes q[n][D] of widths bits[D]).
 *
 * Coded record (mode 0):
 *   tables: for each component with symbol bits h > 0, in index order, 2^h
 *           u16 frequencies of its symbols over the chunk (sum 2^sb), then
 *           zero padding to 4 bytes;
 *   u32 word count of each tile's stream;
 *   per tile (tile_tokens tokens, the last one shorter): u32 final state of
 *           each lane (lane 0 first), the stream's u16 words in emission
 *           order (a zero u16 after an odd count), then its raw rows;
 *   zero padding to 16 bytes.
 * Packed record (mode 1): the packed tiles back to back, zero padding to 16
 * bytes.  The packed form is written when the coded record would not be
 * smaller (the never-worse rule of the AT-1 Memory page, "KV & tensor
 * mode": keep the smaller of the coded and the plain form).  A chunk whose
 * components all have width 0 has an empty record.
 *
 * Returns the record size (a multiple of 16), or -1 when cap is too small. */
int64_t orc_chunk_encode(const orc_config* c, const uint8_t* bits, const uint8_t* q, int32_t n,
                         uint8_t* rec, int64_t cap, int32_t* mode) {
  int32_t D = c->head_dim, lanes = c->rans_lanes, sb = c->rans_scale_bits;
  int32_t ntiles = (n + c->tile_tokens - 1) / c->tile_tokens;
  int64_t P = chunk_packed_bytes(c, bits, n);
  *mode = 0;
  if (P == 0) return 0;
  /* packed form, kept in case it wins */
  int64_t Pa = (P + 15) & ~(int64_t)15;
  uint8_t* packed = (uint8_t*)calloc((size_t)Pa, 1);
  int64_t at = 0;
  for (int32_t t = 0; t < ntiles; ++t) {
    int32_t a = t * c->tile_tokens, m = n - a < c->tile_tokens ? n - a : c->tile_tokens;
    orc_pack(q + (int64_t)a * D, m, D, bits, packed + at);
    at += orc_packed_bytes(bits, D, m);
  }
  /* coded form */
  int32_t tab_off[256];
  int64_t ntab = 0;
  for (int32_t i = 0; i < D; ++i) {
    tab_off[i] = (int32_t)ntab;
    int32_t h = orc_sym_bits(bits[i]);
    if (h > 0) ntab += (int64_t)1 << h;
  }
  int64_t tb = table_bytes(bits, D);
  int64_t cap_coded = tb + 4 * (int64_t)ntiles;
  for (int32_t t = 0; t < ntiles; ++t) {
    int32_t a = t * c->tile_tokens, m = n - a < c->tile_tokens ? n - a : c->tile_tokens;
    int64_t nsym = (int64_t)m * (ntab > 0 ? D : 0);
    cap_coded += 4 * (int64_t)lanes + 2 * seq_words_cap(nsym, lanes, sb) + 2 + raw_row_bytes(bits, D, m);
  }
  uint8_t* buf = (uint8_t*)calloc((size_t)cap_coded + 16, 1);
  uint16_t* freqs = (uint16_t*)buf; /* the tables sit at the start of the record */
  for (int32_t i = 0; i < D; ++i) {
    int32_t h = orc_sym_bits(bits[i]);
    if (h == 0) continue;
    uint32_t counts[16] = {0};
    for (int32_t k = 0; k < n; ++k) counts[q[(int64_t)k * D + i] >> (bits[i] - h)]++;
    orc_freq_normalize(counts, 1 << h, sb, freqs + tab_off[i]);
  }
  int64_t p = tb + 4 * (int64_t)ntiles;
  int64_t maxsym = (int64_t)c->tile_tokens * D;
  uint8_t* sym = (uint8_t*)malloc((size_t)maxsym + 1);
  uint8_t* lane = (uint8_t*)malloc((size_t)maxsym + 1);
  int32_t* tab = (int32_t*)malloc(sizeof(int32_t) * ((size_t)maxsym + 1));
  int32_t* ns = (int32_t*)malloc(sizeof(int32_t) * ((size_t)maxsym + 1));
  uint16_t* words = (uint16_t*)malloc(sizeof(uint16_t) * ((size_t)seq_words_cap(maxsym, lanes, sb) + 1));
  int ok = 1;
  for (int32_t t = 0; t < ntiles && ok; ++t) {
    int32_t a = t * c->tile_tokens, m = n - a < c->tile_tokens ? n - a : c->tile_tokens;
    const uint8_t* qt = q + (int64_t)a * D;
    int64_t N = tile_sequence(qt, m, D, bits, lanes, tab_off, sym, lane, tab, ns);
    uint32_t states[64];
    int64_t nw = orc_rans_encode_seq(N, sym, lane, tab, ns, freqs, sb, lanes, states, words,
                                     seq_words_cap(N, lanes, sb));
    if (nw < 0) { ok = 0; break; }
    put32(buf + tb + 4 * (int64_t)t, (uint32_t)nw);
    memcpy(buf + p, states, 4 * (size_t)lanes);
    p += 4 * (int64_t)lanes;
    memcpy(buf + p, words, 2 * (size_t)nw);
    p += 2 * nw + ((nw & 1) ? 2 : 0);
    for (int32_t i = 0; i < D; ++i) {
      int32_t r = orc_raw_bits(bits[i]);
      if (r == 0) continue;
      for (int32_t k = 0; k < m; ++k)
        put_bits(buf + p, (int64_t)k * r, qt[(int64_t)k * D + i] & ((1u << r) - 1u), r);
      p += 4 * (((int64_t)m * r + 31) / 32);
    }
  }
  int64_t size;
  int64_t coded = (p + 15) & ~(int64_t)15;
  if (ok && coded < Pa) {
    size = coded;
    if (size <= cap) memcpy(rec, buf, (size_t)size);
  } else {
    size = Pa;
    *mode = 1;
    if (size <= cap) memcpy(rec, packed, (size_t)size);
  }
  free(buf); free(packed); free(sym); free(lane); free(tab); free(ns); free(words);
  return size <= cap ? size : -1;
}

/* Decode one chunk record (mode 0 coded, 1 packed) of n tokens into codes
 * q[n][D].  Returns ORC_OK or ORC_ERR_CORRUPT (sizes, tables, streams). */
int orc_chunk_decode(const orc_config* c, const uint8_t* bits, const uint8_t* rec, int64_t size,
                     int32_t mode, int32_t n, uint8_t* q) {
  int32_t D = c->head_dim, lanes = c->rans_lanes, sb = c->rans_scale_bits;
  int32_t ntiles = (n + c->tile_tokens - 1) / c->tile_tokens;
  int64_t P = chunk_packed_bytes(c, bits, n);
  if (P == 0) {
    if (size != 0 || mode != 0) return ORC_ERR_CORRUPT;
    memset(q, 0, (size_t)n * D);
    return ORC_OK;
  }
  if (mode == 1) {
    if (size != ((P + 15) & ~(int64_t)15)) return ORC_ERR_CORRUPT;
    int64_t at = 0;
    for (int32_t t = 0; t < ntiles; ++t) {
      int32_t a = t * c->tile_tokens, m = n - a < c->tile_tokens ? n - a : c->tile_tokens;
      orc_unpack(rec + at, m, D, bits, q + (int64_t)a * D);
      at += orc_packed_bytes(bits, D, m);
    }
    return ORC_OK;
  }
  if (mode != 0) return ORC_ERR_CORRUPT;
  int32_t tab_off[256];
  int64_t ntab = 0;
  for (int32_t i = 0; i < D; ++i) {
    tab_off[i] = (int32_t)ntab;
    int32_t h = orc_sym_bits(bits[i]);
    if (h > 0) ntab += (int64_t)1 << h;
  }
  int64_t tb = table_bytes(bits, D);
  if (size < tb + 4 * (int64_t)ntiles) return ORC_ERR_CORRUPT;
  const uint16_t* freqs = (const uint16_t*)rec; /* little-endian host */
  int64_t p = tb + 4 * (int64_t)ntiles;
  int64_t maxsym = (int64_t)c->tile_tokens * D;
  uint8_t* sym = (uint8_t*)malloc((size_t)maxsym + 1);
  uint8_t* lane = (uint8_t*)malloc((size_t)maxsym + 1);
  int32_t* tab = (int32_t*)malloc(sizeof(int32_t) * ((size_t)maxsym + 1));
  int32_t* ns = (int32_t*)malloc(sizeof(int32_t) * ((size_t)maxsym + 1));
  int st = ORC_OK;
  for (int32_t t = 0; t < ntiles && st == ORC_OK; ++t) {
    int32_t a = t * c->tile_tokens, m = n - a < c->tile_tokens ? n - a : c->tile_tokens;
    uint8_t* qt = q + (int64_t)a * D;
    uint32_t nw = get32(rec + tb + 4 * (int64_t)t);
    int64_t need = 4 * (int64_t)lanes + 2 * (int64_t)nw + ((nw & 1) ? 2 : 0);
    if (p + need > size) { st = ORC_ERR_CORRUPT; break; }
    int64_t N = tile_sequence(NULL, m, D, bits, lanes, tab_off, NULL, lane, tab, ns);
    uint32_t states[64];
    memcpy(states, rec + p, 4 * (size_t)lanes);
    uint16_t* w = (uint16_t*)malloc(sizeof(uint16_t) * ((size_t)nw + 1));
    memcpy(w, rec + p + 4 * (int64_t)lanes, 2 * (size_t)nw);
    st = orc_rans_decode_seq(N, lane, tab, ns, freqs, sb, lanes, states, w, nw, sym);
    free(w);
    if (st != ORC_OK) break;
    p += need;
    int64_t rb = raw_row_bytes(bits, D, m);
    if (p + rb > size) { st = ORC_ERR_CORRUPT; break; }
    /* symbols back into codes, then the raw bits */
    int64_t s_at = 0;
    for (int32_t i = 0; i < D; ++i) {
      int32_t h = orc_sym_bits(bits[i]);
      for (int32_t k = 0; k < m; ++k) qt[(int64_t)k * D + i] = h > 0 ? (uint8_t)(sym[s_at + k] << (bits[i] - h)) : 0;
      if (h > 0) s_at += m;
    }
    for (int32_t i = 0; i < D; ++i) {
      int32_t r = orc_raw_bits(bits[i]);
      if (r == 0) continue;
      for (int32_t k = 0; k < m; ++k) qt[(int64_t)k * D + i] |= (uint8_t)get_bits(rec + p, (int64_t)k * r, r);
      p += 4 * (((int64_t)m * r + 31) / 32);
    }
  }
  free(sym); free(lane); free(tab); free(ns);
  if (st == ORC_OK && ((p + 15) & ~(int64_t)15) != size) st = ORC_ERR_CORRUPT;
  return st;
}

/* ===================================================================== */
/* Container ([KVTC] CompressedSection: data, scales, zero points, bit     */
/* widths, metadata; chunked transport with ordered lengths as on the QATQ */
/* page).  All fields little-endian.                                       */
/* ===================================================================== */

#define HDR_BYTES 256
#define SEC_REC(D) (9 * (int64_t)(D))
#define DIR_ENTRY 32
#define CSUM_FIELD 200 /* header bytes [200, 216): checksum of the fixed part */

typedef struct {
  int32_t T, s0, mid_begin, mid_end, T_mid, W_eff;
  int32_t n_sections, chunks_per_sec, n_r_sections;
  int64_t side_off, side_bytes, r_off, raw_off, raw_bytes, dir_off, chunks_off;
  int32_t budget_k, budget_v;
} layout_t;

static int64_t align16(int64_t x) { return (x + 15) & ~(int64_t)15; }

/* Integrity checksum of a byte range whose length is a multiple of 4
 * ("Quantum-Aware Tensor Compression", QATC transport: bounded chunks with an
 * aggregate checksum, and a damaged or truncated payload is refused before
 * restore).  Over the little-endian 32-bit words w_0 .. w_{n-1}, with the
 * prime P = 2^61 - 1: A = sum w_j mod P and B = sum (j + 1) w_j mod P -- the
 * plain and the position-weighted sum of Fletcher's construction, taken
 * modulo a prime so that every change of one or two words is caught.  Words
 * in [skip_from, skip_to) count as zero (the field that holds the result). */
#define CSUM_P ((uint64_t)0x1fffffffffffffffull)

void orc_checksum(const uint8_t* data, int64_t n_bytes, int64_t skip_from, int64_t skip_to,
                  uint64_t* a_out, uint64_t* b_out) {
  unsigned __int128 A = 0, B = 0;
  for (int64_t j = 0; j < n_bytes / 4; ++j) {
    uint64_t w = (uint64_t)data[4 * j] | ((uint64_t)data[4 * j + 1] << 8) |
                 ((uint64_t)data[4 * j + 2] << 16) | ((uint64_t)data[4 * j + 3] << 24);
    if (4 * j >= skip_from && 4 * j < skip_to) w = 0;
    A = (A + w) % CSUM_P;
    B = (B + (unsigned __int128)(j + 1) * w) % CSUM_P;
  }
  *a_out = (uint64_t)A;
  *b_out = (uint64_t)B;
}

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
  if (c->alloc_scope != 0 && c->alloc_scope != 1) return ORC_ERR_INVALID_ARG;
  if (c->alloc_scope == 1 && c->transform != ORC_PCA) return ORC_ERR_INVALID_ARG;
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

/* The largest width sum one section of kind s (0 keys, 1 values) can have:
 * its own budget, or with one budget over all sections every component at
 * max_bits (within the total). */
static int32_t sec_bits_max(const orc_config* c, const layout_t* lo, int32_t s) {
  if (c->alloc_scope == 0) return s == 0 ? lo->budget_k : lo->budget_v;
  int64_t total = (int64_t)c->layers * c->kv_heads * ((int64_t)lo->budget_k + lo->budget_v);
  int64_t cap = (int64_t)c->head_dim * c->max_bits;
  return (int32_t)(total < cap ? total : cap);
}

/* r-area index of section u, or -1 */
static int64_t r_index(const orc_config* c, int32_t u) {
  int32_t H = c->kv_heads;
  int32_t h = u % H, s = (u / H) % 2, l = u / (2 * H);
  if (!section_has_r(c, s)) return -1;
  if (c->wht_keys) return u;
  return (int64_t)l * H + h; /* only value sections carry r */
}


static const float* basis_of(const orc_config* c, const float* basis, int32_t l, int32_t s, int32_t h) {
  int64_t DD = (int64_t)c->head_dim * c->head_dim;
  if (c->basis_per_head) return basis + (((int64_t)l * 2 + s) * c->kv_heads + h) * DD;
  return basis + ((int64_t)l * 2 + s) * DD;
}

/* 64-bit FNV-1a (offset basis 0xcbf29ce484222325, prime 2^40 + 0x1b3):
 * for each byte, XOR it in, then multiply by the prime modulo 2^64.  `h`
 * carries a running hash (start with the offset basis). */
uint64_t orc_fnv1a64(uint64_t h, const uint8_t* bytes, int64_t n) {
  for (int64_t i = 0; i < n; ++i) {
    h ^= bytes[i];
    h *= 0x100000001b3ull;
  }
  return h;
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
    h = orc_fnv1a64(h, b, nb);
  }
  return h;
}

/* Largest record of a chunk of ntok tokens: never above its packed size
 * (records fall back to the packed form), which is at most ntok budget / 8
 * bytes plus a padding word per component row of each tile. */
static int64_t max_record(const orc_config* c, int32_t ntok, int32_t budget) {
  int32_t D = c->head_dim;
  int32_t ntiles = (ntok + c->tile_tokens - 1) / c->tile_tokens;
  int32_t nz = budget < D ? budget : D; /* components with >= 1 bit */
  int64_t P = 0;
  for (int32_t t = 0; t < ntiles; ++t) {
    int32_t n = ntok - t * c->tile_tokens;
    if (n > c->tile_tokens) n = c->tile_tokens;
    P += ((int64_t)n * budget + 7) / 8 + 4 * (int64_t)nz;
  }
  return align16(P);
}

int64_t orc_max_container_bytes(const orc_config* c, int32_t T) {
  if (orc_check_config(c) != ORC_OK || T < 0) return -1;
  layout_t lo;
  make_layout(c, T, &lo);
  int64_t total = lo.chunks_off;
  for (int32_t u = 0; u < lo.n_sections; ++u) {
    int32_t s = (u / c->kv_heads) % 2;
    int32_t budget = sec_bits_max(c, &lo, s);
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
  put32(out + 4, 3);
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
  put32(out + 192, (uint32_t)c->alloc_scope);
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
                         const float* coef, const uint8_t* bits_given, side_t* si) {
  int32_t D = c->head_dim, s = (u / c->kv_heads) % 2;
  int32_t N = lo->T_mid;
  float mu[256], var[256], mn[256], mx[256];
  orc_stats(coef, N, D, mu, var, mn, mx);
  if (c->transform == ORC_PCA) {
    if (bits_given)
      memcpy(si->bits, bits_given, (size_t)D);
    else
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
  int64_t pos = lo.chunks_off;
  side_t si;
  /* one budget over all sections: the variances of every section first,
   * then the greedy allocation over all of their components at once */
  uint8_t* bits_all = NULL;
  if (c->alloc_scope == 1 && lo.T_mid > 0) {
    float* var_all = (float*)calloc((size_t)lo.n_sections * D, sizeof(float));
    bits_all = (uint8_t*)malloc((size_t)lo.n_sections * D);
    int64_t budget = 0;
    for (int32_t u = 0; u < lo.n_sections && st == ORC_OK; ++u) {
      st = gather_section(c, k, v, &lo, u, cos_t, sin_t, x);
      if (st != ORC_OK) break;
      transform_section(c, basis, u, lo.T_mid, x, coef, r);
      float mu[256], mn[256], mx[256];
      orc_stats(coef, lo.T_mid, D, mu, var_all + (int64_t)u * D, mn, mx);
      budget += ((u / H) % 2) == 0 ? lo.budget_k : lo.budget_v;
    }
    if (st == ORC_OK) orc_alloc_greedy_heap(var_all, (int64_t)lo.n_sections * D, budget, c->max_bits, bits_all);
    free(var_all);
  }
  for (int32_t u = 0; u < lo.n_sections && st == ORC_OK; ++u) {
    st = gather_section(c, k, v, &lo, u, cos_t, sin_t, x);
    if (st != ORC_OK) break;
    if (lo.T_mid == 0) continue;
    transform_section(c, basis, u, lo.T_mid, x, coef, r);
    section_side(c, &lo, u, coef, bits_all ? bits_all + (int64_t)u * D : NULL, &si);
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
      int32_t mode = 0;
      int64_t size = orc_chunk_encode(c, si.bits, q, n, out + pos, cap - pos, &mode);
      if (size < 0) { st = ORC_ERR_CAPACITY; break; }
      int64_t dir = lo.dir_off + ((int64_t)u * lo.chunks_per_sec + ch) * DIR_ENTRY;
      put64(out + dir, (uint64_t)pos);
      put32(out + dir + 8, (uint32_t)size);
      put32(out + dir + 12, (uint32_t)mode);
      uint64_t ca, cb;
      orc_checksum(out + pos, size, 0, 0, &ca, &cb);
      put64(out + dir + 16, ca);
      put64(out + dir + 24, cb);
      pos += size;
    }
  }
  if (st == ORC_OK) {
    copy_raw(c, &lo, k, v, out + lo.raw_off, 1);
    write_header(c, &lo, orc_fingerprint(c, basis), pos, out);
    /* last: the checksum of everything before the records */
    uint64_t fa, fb;
    orc_checksum(out, lo.chunks_off, CSUM_FIELD, CSUM_FIELD + 16, &fa, &fb);
    put64(out + CSUM_FIELD, fa);
    put64(out + CSUM_FIELD + 8, fb);
    *out_bytes = pos;
  }
  free(x); free(coef); free(r); free(q);
  free(cos_t); free(sin_t);
  free(bits_all);
  return st;
}

/* ---- decode ---------------------------------------------------------- */

static int parse_header(const orc_config* c, const float* basis, const uint8_t* in,
                        int64_t n, layout_t* lo) {
  if (n < HDR_BYTES) return ORC_ERR_CORRUPT;
  if (memcmp(in, "KVTC", 4) != 0 || get32(in + 4) != 3 || get32(in + 8) != HDR_BYTES)
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
  h.alloc_scope = (int32_t)get32(in + 192);
  if (h.layers != c->layers || h.kv_heads != c->kv_heads || h.head_dim != c->head_dim ||
      h.dtype != c->dtype || h.transform != c->transform || h.sink_tokens != c->sink_tokens ||
      h.recent_tokens != c->recent_tokens || memcmp(&h.bits_k, &c->bits_k, 4) ||
      memcmp(&h.bits_v, &c->bits_v, 4) || h.max_bits != c->max_bits ||
      h.rope_keys != c->rope_keys || h.rope_style != c->rope_style ||
      memcmp(&h.rope_theta, &c->rope_theta, 8) || h.rans_scale_bits != c->rans_scale_bits ||
      h.rans_lanes != c->rans_lanes || h.chunk_tokens != c->chunk_tokens ||
      h.tile_tokens != c->tile_tokens || h.basis_per_head != c->basis_per_head ||
      h.wht_keys != c->wht_keys || h.alloc_scope != c->alloc_scope)
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
  uint64_t fa, fb;
  orc_checksum(in, lo->chunks_off, CSUM_FIELD, CSUM_FIELD + 16, &fa, &fb);
  if (fa != get64(in + CSUM_FIELD) || fb != get64(in + CSUM_FIELD + 8)) return ORC_ERR_CORRUPT;
  return ORC_OK;
}

/* Decode the codes of chunk ch of section u into q[n][D]. */
static int decode_chunk_codes(const orc_config* c, const layout_t* lo, const uint8_t* in,
                              int64_t total, int32_t u, int32_t ch, const uint8_t* bits,
                              uint8_t* q) {
  int32_t t0 = ch * c->chunk_tokens;
  int32_t n = lo->T_mid - t0 < c->chunk_tokens ? lo->T_mid - t0 : c->chunk_tokens;
  int64_t dir = lo->dir_off + ((int64_t)u * lo->chunks_per_sec + ch) * DIR_ENTRY;
  uint64_t off = get64(in + dir);
  uint32_t size = get32(in + dir + 8);
  uint32_t mode = get32(in + dir + 12);
  if (mode > 1) return ORC_ERR_CORRUPT;
  if (size > 0 && (off < (uint64_t)lo->chunks_off || (off & 15) || off > (uint64_t)total ||
                   size > (uint64_t)total - off))
    return ORC_ERR_CORRUPT;
  uint64_t ca, cb;
  orc_checksum(size > 0 ? in + off : in, size, 0, 0, &ca, &cb);
  if (ca != get64(in + dir + 16) || cb != get64(in + dir + 24)) return ORC_ERR_CORRUPT;
  return orc_chunk_decode(c, bits, size > 0 ? in + off : in, size, (int32_t)mode, n, q);
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
  float chat[256], tmp[256];
  int st = ORC_OK;
  int sym = sym_section(c, u);
  int32_t off = sym ? 1 << (bits[0] - 1) : 0;
  for (int32_t ch = 0; ch < lo->chunks_per_sec && st == ORC_OK; ++ch) {
    int32_t t0 = ch * c->chunk_tokens;
    int32_t n = lo->T_mid - t0 < c->chunk_tokens ? lo->T_mid - t0 : c->chunk_tokens;
    st = decode_chunk_codes(c, lo, in, total, u, ch, bits, q);
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
  free(q); free(Bp);
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
  for (int32_t ch = 0; ch < lo.chunks_per_sec && st == ORC_OK; ++ch)
    st = decode_chunk_codes(c, &lo, in, total, u, ch, bits, q_out + (int64_t)ch * c->chunk_tokens * D);
  return st;
}

/* ===================================================================== */
/* Scalar quantisers on gauge coordinates ("Codec-Gauge", Compression     */
/* Conditions: block-uniform ranges per T_b x d_l block; KIVI-style        */
/* per-channel key and per-token value ranges; the same bit settings).    */
/* ===================================================================== */

int orc_sq_check(const orc_config* c, const orc_sq_config* q) {
  int st = orc_check_config(c);
  if (st != ORC_OK) return st;
  if (c->transform != ORC_PCA) return ORC_ERR_INVALID_ARG;
  if (q->kind != ORC_SQ_BLOCK && q->kind != ORC_SQ_KIVI) return ORC_ERR_INVALID_ARG;
  if (q->group < 1 || c->head_dim % q->group) return ORC_ERR_INVALID_ARG;
  if (q->tile < 1) return ORC_ERR_INVALID_ARG;
  if (q->bits_k < 1 || q->bits_k > 8 || q->bits_v < 1 || q->bits_v > 8) return ORC_ERR_INVALID_ARG;
  return ORC_OK;
}

/* Code bytes and (zero, scale) pairs of one section of kind s (0 keys,
 * 1 values) over T tokens. */
static int64_t sq_sec_codes(const orc_config* c, const orc_sq_config* q, int32_t T, int32_t s) {
  return (int64_t)T * c->head_dim * (s == 0 ? q->bits_k : q->bits_v) / 8;
}

static int64_t sq_sec_ranges(const orc_config* c, const orc_sq_config* q, int32_t T, int32_t s) {
  int64_t nt = ((int64_t)T + q->tile - 1) / q->tile, D = c->head_dim, g = q->group;
  if (q->kind == ORC_SQ_BLOCK) return nt * (D / g);
  return s == 0 ? nt * D : (int64_t)T * (D / g);
}

/* Offset of section u = (l 2 + s) H + h among sections whose sizes depend
 * only on s. */
static int64_t sq_sec_off(const orc_config* c, int32_t u, int64_t x0, int64_t x1) {
  int32_t H = c->kv_heads, h = u % H, s = (u / H) % 2, l = u / (2 * H);
  return (int64_t)l * H * (x0 + x1) + (s ? (int64_t)H * x0 : 0) + (int64_t)h * (s ? x1 : x0);
}

int64_t orc_sq_code_bytes(const orc_config* c, const orc_sq_config* q, int32_t T) {
  if (orc_sq_check(c, q) != ORC_OK || T < 0) return -1;
  return (int64_t)c->layers * c->kv_heads * (sq_sec_codes(c, q, T, 0) + sq_sec_codes(c, q, T, 1));
}

int64_t orc_sq_range_pairs(const orc_config* c, const orc_sq_config* q, int32_t T) {
  if (orc_sq_check(c, q) != ORC_OK || T < 0) return -1;
  return (int64_t)c->layers * c->kv_heads * (sq_sec_ranges(c, q, T, 0) + sq_sec_ranges(c, q, T, 1));
}

/* The range index (within its section) of coefficient (t, i) of kind s. */
static int64_t sq_range_of(const orc_config* c, const orc_sq_config* q, int32_t s, int32_t t, int32_t i) {
  int32_t D = c->head_dim, g = q->group;
  int64_t ti = t / q->tile;
  if (q->kind == ORC_SQ_BLOCK) return ti * (D / g) + i / g;
  return s == 0 ? ti * D + i : (int64_t)t * (D / g) + i / g;
}

/* zero = min, scale = (max - min) / (2^b - 1) in fp64 rounded once, rcp =
 * 1 / scale (0 for an empty step), as for a component's side information. */
static void sq_range(float mn, float mx, int32_t b, float* zero, float* scale, float* rcp) {
  float sc = (float)(((double)mx - (double)mn) / (double)((1u << b) - 1u));
  float r = sc > 0.0f ? 1.0f / sc : 0.0f;
  if (!(sc > 0.0f) || isinf(r)) {
    sc = 0.0f;
    r = 0.0f;
  }
  *zero = mn;
  *scale = sc;
  *rcp = r;
}

int orc_sq_encode(const orc_config* c, const orc_sq_config* q, const void* k, const void* v, int32_t T,
                  const float* basis, uint8_t* codes, float* ranges) {
  int st = orc_sq_check(c, q);
  if (st != ORC_OK) return st;
  if (T < 0 || !basis) return ORC_ERR_INVALID_ARG;
  int32_t D = c->head_dim, H = c->kv_heads, n_sec = c->layers * 2 * H;
  int64_t cb0 = sq_sec_codes(c, q, T, 0), cb1 = sq_sec_codes(c, q, T, 1);
  int64_t nr0 = sq_sec_ranges(c, q, T, 0), nr1 = sq_sec_ranges(c, q, T, 1);
  float* x = (float*)malloc(sizeof(float) * ((size_t)T * D + 1));
  float* coef = (float*)malloc(sizeof(float) * ((size_t)T * D + 1));
  float* Bp = (float*)malloc(sizeof(float) * (size_t)D * D);
  float* mn = (float*)malloc(sizeof(float) * (size_t)(nr0 > nr1 ? nr0 : nr1) + 4);
  float* mx = (float*)malloc(sizeof(float) * (size_t)(nr0 > nr1 ? nr0 : nr1) + 4);
  for (int32_t u = 0; u < n_sec && st == ORC_OK; ++u) {
    int32_t h = u % H, s = (u / H) % 2, l = u / (2 * H);
    int32_t b = s == 0 ? q->bits_k : q->bits_v;
    int64_t nr = s == 0 ? nr0 : nr1;
    st = orc_section_rows(c, k, v, T, u, 0, T, x);
    if (st != ORC_OK) break;
    const float* B = basis_of(c, basis, l, s, h);
    for (int64_t a = 0; a < (int64_t)D * D; ++a) Bp[a] = round_p(B[a], c->dtype);
    for (int32_t t = 0; t < T; ++t) orc_project(x + (int64_t)t * D, Bp, D, coef + (int64_t)t * D);
    /* ranges: min and max of each range's coefficients */
    for (int64_t r = 0; r < nr; ++r) {
      mn[r] = INFINITY;
      mx[r] = -INFINITY;
    }
    for (int32_t t = 0; t < T; ++t)
      for (int32_t i = 0; i < D; ++i) {
        float cv = coef[(int64_t)t * D + i];
        if (!isfinite(cv)) st = ORC_ERR_NONFINITE;
        int64_t r = sq_range_of(c, q, s, t, i);
        if (cv < mn[r]) mn[r] = cv;
        if (cv > mx[r]) mx[r] = cv;
      }
    if (st != ORC_OK) break;
    float* rg = ranges + 2 * sq_sec_off(c, u, nr0, nr1);
    for (int64_t r = 0; r < nr; ++r) {
      float z, sc, rc;
      sq_range(mn[r], mx[r], b, &z, &sc, &rc);
      rg[2 * r] = z;
      rg[2 * r + 1] = sc;
    }
    /* codes: v = (c - zero) * rcp in fp32, q = clamp(rint(v), 0, 2^b - 1),
     * token rows of D b bits, channel i at bits [i b, i b + b), LSB-first */
    uint8_t* cs = codes + sq_sec_off(c, u, cb0, cb1);
    memset(cs, 0, (size_t)(s == 0 ? cb0 : cb1));
    for (int32_t t = 0; t < T; ++t)
      for (int32_t i = 0; i < D; ++i) {
        int64_t r = sq_range_of(c, q, s, t, i);
        float z, sc, rc;
        sq_range(mn[r], mx[r], b, &z, &sc, &rc);
        float d = coef[(int64_t)t * D + i] - z;
        float vv = d * rc;
        float rq = nearbyintf(vv);
        float hi = (float)((1u << b) - 1u);
        if (rq < 0.0f) rq = 0.0f;
        if (rq > hi) rq = hi;
        uint32_t code = (uint32_t)rq;
        int64_t bit = ((int64_t)t * D + i) * b;
        for (int32_t e = 0; e < b; ++e)
          if ((code >> e) & 1u) cs[(bit + e) >> 3] |= (uint8_t)(1u << ((bit + e) & 7));
      }
  }
  free(x); free(coef); free(Bp); free(mn); free(mx);
  return st;
}

int orc_sq_decode(const orc_config* c, const orc_sq_config* q, const uint8_t* codes, const float* ranges,
                  int32_t T, const float* basis, float* k_out, float* v_out) {
  int st = orc_sq_check(c, q);
  if (st != ORC_OK) return st;
  if (T < 0 || !basis) return ORC_ERR_INVALID_ARG;
  int32_t D = c->head_dim, H = c->kv_heads, n_sec = c->layers * 2 * H;
  int64_t cb0 = sq_sec_codes(c, q, T, 0), cb1 = sq_sec_codes(c, q, T, 1);
  int64_t nr0 = sq_sec_ranges(c, q, T, 0), nr1 = sq_sec_ranges(c, q, T, 1);
  float* Bp = (float*)malloc(sizeof(float) * (size_t)D * D);
  float* cos_t = (float*)malloc(sizeof(float) * ((size_t)T * D / 2 + 1));
  float* sin_t = (float*)malloc(sizeof(float) * ((size_t)T * D / 2 + 1));
  orc_rope_table(T, D, c->rope_theta, cos_t, sin_t);
  float chat[256], xr[256], y[256];
  for (int32_t u = 0; u < n_sec; ++u) {
    int32_t h = u % H, s = (u / H) % 2, l = u / (2 * H);
    int32_t b = s == 0 ? q->bits_k : q->bits_v;
    const float* B = basis_of(c, basis, l, s, h);
    for (int64_t a = 0; a < (int64_t)D * D; ++a) Bp[a] = round_p(B[a], c->dtype);
    const float* rg = ranges + 2 * sq_sec_off(c, u, nr0, nr1);
    const uint8_t* cs = codes + sq_sec_off(c, u, cb0, cb1);
    float* out = s == 0 ? k_out : v_out;
    for (int32_t t = 0; t < T; ++t) {
      for (int32_t i = 0; i < D; ++i) {
        int64_t bit = ((int64_t)t * D + i) * b;
        uint32_t code = 0;
        for (int32_t e = 0; e < b; ++e) code |= (uint32_t)((cs[(bit + e) >> 3] >> ((bit + e) & 7)) & 1u) << e;
        int64_t r = sq_range_of(c, q, s, t, i);
        chat[i] = round_p(fmaf((float)code, rg[2 * r + 1], rg[2 * r]), c->dtype);
      }
      orc_unproject(chat, Bp, D, xr);
      if (s == 0 && c->rope_keys) {
        orc_rope_forward(xr, y, D, c->rope_style, cos_t + (int64_t)t * (D / 2), sin_t + (int64_t)t * (D / 2));
      } else {
        memcpy(y, xr, sizeof(float) * D);
      }
      memcpy(out + (((int64_t)l * H + h) * T + t) * D, y, sizeof(float) * D);
    }
  }
  free(Bp); free(cos_t); free(sin_t);
  return ORC_OK;
}

/* ===================================================================== */
/* TTAS-X2 value path ([TTAS] 2.2 V Compression: RMS normalisation per     */
/* vector, Hadamard transform, two-level product quantisation with         */
/* K1 = 256 and K2 = 64..512, fixed-budget outliers per head).             */
/* ===================================================================== */

static int pq_pow2_in(int32_t k, int32_t lo, int32_t hi) { return k >= lo && k <= hi && (k & (k - 1)) == 0; }

static int32_t pq_log2(int32_t k) {
  int32_t b = 0;
  while ((1 << b) < k) ++b;
  return b;
}

int orc_pq_check(const orc_config* c, const orc_pq_config* q) {
  int st = orc_check_config(c);
  if (st != ORC_OK) return st;
  if (!q || (c->head_dim & (c->head_dim - 1))) return ORC_ERR_INVALID_ARG; /* the WHT needs 2^n */
  if (q->sub_dim < 1 || c->head_dim % q->sub_dim) return ORC_ERR_INVALID_ARG;
  if (!pq_pow2_in(q->k1, 2, 512) || !pq_pow2_in(q->k2, 2, 512)) return ORC_ERR_INVALID_ARG;
  if (q->outliers < 0 || q->block_tokens < 1) return ORC_ERR_INVALID_ARG;
  return ORC_OK;
}

/* A token's row: the M level-1 indices of log2(k1) bits, then the M level-2
 * indices of log2(k2) bits, least significant bit first, padded to 32. */
int32_t orc_pq_row_words(const orc_config* c, const orc_pq_config* q) {
  if (orc_pq_check(c, q) != ORC_OK) return -1;
  int32_t M = c->head_dim / q->sub_dim;
  return (M * (pq_log2(q->k1) + pq_log2(q->k2)) + 31) / 32;
}

int64_t orc_pq_outlier_slots(const orc_config* c, const orc_pq_config* q, int32_t T) {
  if (orc_pq_check(c, q) != ORC_OK || T < 0) return -1;
  int64_t nblk = ((int64_t)T + q->block_tokens - 1) / q->block_tokens;
  return (int64_t)c->layers * c->kv_heads * nblk * q->outliers;
}

/* The nearest of k centroids (already bf16-valued) to y: fp64 squared
 * distance summed in channel order, lowest index on ties. */
static int32_t pq_nearest_r(const float* y, const float* cb, int32_t k, int32_t d) {
  int32_t best = 0;
  double bd = INFINITY;
  for (int32_t i = 0; i < k; ++i) {
    double acc = 0.0;
    for (int32_t j = 0; j < d; ++j) {
      double e = (double)y[j] - (double)cb[(int64_t)i * d + j];
      acc += e * e;
    }
    if (acc < bd) {
      bd = acc;
      best = i;
    }
  }
  return best;
}

int32_t orc_pq_nearest(const float* y, const float* cb, int32_t k, int32_t d) {
  float* r = (float*)malloc(sizeof(float) * (size_t)k * d);
  for (int64_t a = 0; a < (int64_t)k * d; ++a) r[a] = orc_bf16_to_f32(orc_f32_to_bf16(cb[a]));
  int32_t i = pq_nearest_r(y, r, k, d);
  free(r);
  return i;
}

static void pq_put(uint32_t* row, int64_t bit, int32_t nb, uint32_t v) {
  for (int32_t e = 0; e < nb; ++e)
    if ((v >> e) & 1u) row[(bit + e) >> 5] |= 1u << ((bit + e) & 31);
}

static uint32_t pq_get(const uint32_t* row, int64_t bit, int32_t nb) {
  uint32_t v = 0;
  for (int32_t e = 0; e < nb; ++e) v |= ((row[(bit + e) >> 5] >> ((bit + e) & 31)) & 1u) << e;
  return v;
}

/* The layer's codebooks with every entry rounded to bf16. */
static void pq_round_codebooks(const orc_config* c, const orc_pq_config* q, int32_t l, const float* cb1,
                               const float* cb2, float* c1, float* c2) {
  int32_t M = c->head_dim / q->sub_dim, d = q->sub_dim;
  int64_t n1 = (int64_t)M * q->k1 * d, n2 = (int64_t)M * q->k2 * d;
  for (int64_t a = 0; a < n1; ++a) c1[a] = orc_bf16_to_f32(orc_f32_to_bf16(cb1[(int64_t)l * n1 + a]));
  for (int64_t a = 0; a < n2; ++a) c2[a] = orc_bf16_to_f32(orc_f32_to_bf16(cb2[(int64_t)l * n2 + a]));
}

typedef struct {
  float mag;
  uint32_t idx;
} pq_cand;

/* |y - y^| descending, then the lower index first. */
static int pq_cmp_mag(const void* a, const void* b) {
  const pq_cand* x = (const pq_cand*)a;
  const pq_cand* y = (const pq_cand*)b;
  if (x->mag != y->mag) return x->mag > y->mag ? -1 : 1;
  return x->idx < y->idx ? -1 : (x->idx > y->idx);
}

static int pq_cmp_idx(const void* a, const void* b) {
  const pq_cand* x = (const pq_cand*)a;
  const pq_cand* y = (const pq_cand*)b;
  return x->idx < y->idx ? -1 : (x->idx > y->idx);
}

int orc_pq_encode(const orc_config* c, const orc_pq_config* q, const void* v, int32_t T, const float* cb1,
                  const float* cb2, uint32_t* codes, float* rms, uint32_t* outliers) {
  int st = orc_pq_check(c, q);
  if (st != ORC_OK) return st;
  if (T < 0) return ORC_ERR_INVALID_ARG;
  if (T == 0) return ORC_OK;
  if (!v || !cb1 || !cb2 || !codes || !rms || (q->outliers > 0 && !outliers)) return ORC_ERR_INVALID_ARG;
  const int32_t D = c->head_dim, H = c->kv_heads, d = q->sub_dim, M = D / d;
  const int32_t b1 = pq_log2(q->k1), b2 = pq_log2(q->k2), rw = orc_pq_row_words(c, q);
  const int32_t B = q->outliers, bt = q->block_tokens;
  const int32_t nblk = (T + bt - 1) / bt;
  float* c1 = (float*)malloc(sizeof(float) * (size_t)M * q->k1 * d);
  float* c2 = (float*)malloc(sizeof(float) * (size_t)M * q->k2 * d);
  float* y = (float*)malloc(sizeof(float) * (size_t)T * D);
  float* del = (float*)malloc(sizeof(float) * (size_t)T * D);
  pq_cand* cand = (pq_cand*)malloc(sizeof(pq_cand) * ((size_t)(bt < T ? bt : T) * D + 1));
  float x[256], xn[256], e[256];
  for (int32_t l = 0; l < c->layers && st == ORC_OK; ++l) {
    pq_round_codebooks(c, q, l, cb1, cb2, c1, c2);
    for (int32_t h = 0; h < H && st == ORC_OK; ++h) {
      const int64_t sec = (int64_t)l * H + h;
      for (int32_t t = 0; t < T; ++t) {
        for (int32_t j = 0; j < D; ++j) {
          x[j] = load_elem(v, c->dtype, (sec * T + t) * D + j);
          if (!isfinite(x[j])) st = ORC_ERR_NONFINITE;
        }
        if (st != ORC_OK) break;
        /* RMS normalisation and the orthonormal Hadamard transform */
        float r = orc_rms(x, D);
        rms[sec * T + t] = r;
        for (int32_t j = 0; j < D; ++j) xn[j] = r == 0.0f ? 0.0f : x[j] / r;
        float* yt = y + (int64_t)t * D;
        orc_wht(xn, D, yt);
        uint32_t* row = codes + (sec * T + t) * rw;
        memset(row, 0, sizeof(uint32_t) * (size_t)rw);
        for (int32_t s = 0; s < M; ++s) {
          const float* ys = yt + s * d;
          const float* cs1 = c1 + (int64_t)s * q->k1 * d;
          const float* cs2 = c2 + (int64_t)s * q->k2 * d;
          /* level 1, then level 2 on the fp32 residual */
          int32_t i1 = pq_nearest_r(ys, cs1, q->k1, d);
          for (int32_t j = 0; j < d; ++j) e[j] = ys[j] - cs1[(int64_t)i1 * d + j];
          int32_t i2 = pq_nearest_r(e, cs2, q->k2, d);
          for (int32_t j = 0; j < d; ++j) {
            float yh = cs1[(int64_t)i1 * d + j] + cs2[(int64_t)i2 * d + j];
            del[(int64_t)t * D + s * d + j] = ys[j] - yh;
          }
          pq_put(row, (int64_t)s * b1, b1, (uint32_t)i1);
          pq_put(row, (int64_t)M * b1 + (int64_t)s * b2, b2, (uint32_t)i2);
        }
      }
      if (st != ORC_OK || B == 0) continue;
      /* per block: the B coefficients with the largest |y - y^|, kept exactly */
      for (int32_t k = 0; k < nblk; ++k) {
        int32_t ta = k * bt, tb = ta + bt < T ? ta + bt : T;
        int64_t n = (int64_t)(tb - ta) * D;
        for (int64_t a = 0; a < n; ++a) {
          cand[a].idx = (uint32_t)((int64_t)ta * D + a);
          cand[a].mag = fabsf(del[(int64_t)ta * D + a]);
        }
        qsort(cand, (size_t)n, sizeof(pq_cand), pq_cmp_mag);
        int64_t nsel = n < B ? n : B;
        qsort(cand, (size_t)nsel, sizeof(pq_cand), pq_cmp_idx);
        uint32_t* o = outliers + ((sec * nblk + k) * B) * 2;
        for (int64_t a = 0; a < B; ++a) {
          if (a < nsel) {
            uint32_t bits;
            memcpy(&bits, &y[cand[a].idx], 4);
            o[2 * a] = cand[a].idx;
            o[2 * a + 1] = bits;
          } else {
            o[2 * a] = 0xFFFFFFFFu;
            o[2 * a + 1] = 0u;
          }
        }
      }
    }
  }
  free(c1); free(c2); free(y); free(del); free(cand);
  return st;
}

int orc_pq_decode(const orc_config* c, const orc_pq_config* q, const uint32_t* codes, const float* rms,
                  const uint32_t* outliers, int32_t T, const float* cb1, const float* cb2, float* v_out) {
  int st = orc_pq_check(c, q);
  if (st != ORC_OK) return st;
  if (T < 0) return ORC_ERR_INVALID_ARG;
  if (T == 0) return ORC_OK;
  if (!codes || !rms || !cb1 || !cb2 || !v_out || (q->outliers > 0 && !outliers)) return ORC_ERR_INVALID_ARG;
  const int32_t D = c->head_dim, H = c->kv_heads, d = q->sub_dim, M = D / d;
  const int32_t b1 = pq_log2(q->k1), b2 = pq_log2(q->k2), rw = orc_pq_row_words(c, q);
  const int32_t B = q->outliers, bt = q->block_tokens;
  const int32_t nblk = (T + bt - 1) / bt;
  float* c1 = (float*)malloc(sizeof(float) * (size_t)M * q->k1 * d);
  float* c2 = (float*)malloc(sizeof(float) * (size_t)M * q->k2 * d);
  float* yh = (float*)malloc(sizeof(float) * ((size_t)(bt < T ? bt : T) * D + 1));
  float tmp[256];
  for (int32_t l = 0; l < c->layers && st == ORC_OK; ++l) {
    pq_round_codebooks(c, q, l, cb1, cb2, c1, c2);
    for (int32_t h = 0; h < H && st == ORC_OK; ++h) {
      const int64_t sec = (int64_t)l * H + h;
      for (int32_t k = 0; k < nblk && st == ORC_OK; ++k) {
        int32_t ta = k * bt, tb = ta + bt < T ? ta + bt : T;
        for (int32_t t = ta; t < tb; ++t) {
          const uint32_t* row = codes + (sec * T + t) * rw;
          for (int32_t s = 0; s < M; ++s) {
            uint32_t i1 = pq_get(row, (int64_t)s * b1, b1);
            uint32_t i2 = pq_get(row, (int64_t)M * b1 + (int64_t)s * b2, b2);
            for (int32_t j = 0; j < d; ++j)
              yh[(int64_t)(t - ta) * D + s * d + j] =
                  c1[((int64_t)s * q->k1 + i1) * d + j] + c2[((int64_t)s * q->k2 + i2) * d + j];
          }
        }
        /* the block's outliers replace their coefficients */
        const uint32_t* o = B > 0 ? outliers + ((sec * nblk + k) * B) * 2 : NULL;
        for (int32_t a = 0; a < B; ++a) {
          uint32_t idx = o[2 * a];
          if (idx == 0xFFFFFFFFu) continue;
          if ((int64_t)idx < (int64_t)ta * D || (int64_t)idx >= (int64_t)tb * D) {
            st = ORC_ERR_CORRUPT;
            break;
          }
          memcpy(&yh[idx - (int64_t)ta * D], &o[2 * a + 1], 4);
        }
        if (st != ORC_OK) break;
        /* inverse transform (the orthonormal WHT is its own inverse), times r */
        for (int32_t t = ta; t < tb; ++t) {
          float r = rms[sec * T + t];
          orc_wht(yh + (int64_t)(t - ta) * D, D, tmp);
          for (int32_t j = 0; j < D; ++j) v_out[(sec * T + t) * D + j] = tmp[j] * r;
        }
      }
    }
  }
  free(c1); free(c2); free(yh);
  return st;
}
