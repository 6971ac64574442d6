/*
 * csk_oracle.c - plain CPU oracle for hybrid compressed attention (CSA + HCA).
 *
 * TEST INFRASTRUCTURE ONLY: the reference the GPU library is checked
 * against. Only tests, the smoke check and the benchmark's CPU-baseline leg
 * may load it. Written for a reader to check against the pages by eye:
 * plain loops, double arithmetic, one rounding at the end. Built with
 * -ffp-contract=off so that every fused multiply-add is an explicit fmaf().
 *
 * Page keys ([P1]..[P4]) are listed in csk_oracle.h.
 */
#include "csk_oracle.h"

#include <float.h>
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int csk_ref_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------------------------ RoPE */

/* [P4]: only the last d_rope dims carry rotary position. Pairs are
 * interleaved (channel D-d_rope+2j with D-d_rope+2j+1); pair j turns by
 * pos * base^(-2j/d_rope). Angle and rotation in double. */
void csk_ref_rope(double* x, int D, int d_rope, double pos, double base) {
  for (int j = 0; j < d_rope / 2; ++j) {
    double theta = pow(base, -2.0 * (double)j / (double)d_rope);
    double ang = pos * theta;
    double c = cos(ang), s = sin(ang);
    int i0 = D - d_rope + 2 * j;
    double x0 = x[i0], x1 = x[i0 + 1];
    x[i0] = x0 * c - x1 * s;
    x[i0 + 1] = x0 * s + x1 * c;
  }
}

/* ------------------------------------------------------------ compression */

/* Softmax over a set of logits applied channel-wise ("Hadamard" sum):
 * out = sum_r exp(L_r - max L) * V_r / sum_r exp(L_r - max L).
 * [P1] «CSA…» step 1 (weights through softmax together with learned
 * positional biases, records summed with these weights) and exercise 2
 * (softmax over 2m elements, Hadamard summation). */
static double softmax_pool(const double* L, const double* V, int n) {
  double mx = -INFINITY;
  for (int r = 0; r < n; ++r)
    if (L[r] > mx) mx = L[r];
  double num = 0.0, den = 0.0;
  for (int r = 0; r < n; ++r) {
    double e = exp(L[r] - mx);
    num += e * V[r];
    den += e;
  }
  return num / den;
}

static int check_compress_args(int B, int S, int D, int m, int d_rope) {
  if (B < 0 || S < 0 || D <= 0 || m <= 0) return -1;
  if (d_rope < 0 || d_rope > D || (d_rope & 1)) return -1;
  return 0;
}

/* CSA: entry i pools the a-series over tokens [m*i, m*i+m) together with
 * the b-series over the previous block [m*(i-1), m*i), i.e. 2m sources with
 * stride m, so neighbouring entries share sources and the length shrinks
 * exactly m-fold ([P1] «CSA…» step 1; [P4]: every 2m tokens with stride m).
 * Entry 0 has no previous block: its softmax runs over the m a-slots only.
 * A trailing partial block produces no entry. */
int csk_ref_csa_compress(const float* ca, const float* za, const float* cb, const float* zb,
                         const float* bias_a, const float* bias_b, int B, int S, int D, int m,
                         int d_rope, double rope_base, const int32_t* entry_pos, double* out) {
  if (check_compress_args(B, S, D, m, d_rope)) return -1;
  const int N = S / m;
#pragma omp parallel for collapse(2) schedule(static)
  for (int b = 0; b < B; ++b) {
    for (int i = 0; i < N; ++i) {
      double* L = (double*)malloc(sizeof(double) * 2 * (size_t)m);
      double* V = (double*)malloc(sizeof(double) * 2 * (size_t)m);
      double* row = out + ((size_t)b * N + i) * D;
      for (int c = 0; c < D; ++c) {
        int n = 0;
        for (int r = 0; r < m; ++r) {
          size_t src = ((size_t)b * S + (size_t)m * i + r) * D + c;
          L[n] = (double)za[src] + (double)bias_a[(size_t)r * D + c];
          V[n] = (double)ca[src];
          ++n;
        }
        if (i >= 1) {
          for (int r = 0; r < m; ++r) {
            size_t src = ((size_t)b * S + (size_t)m * (i - 1) + r) * D + c;
            L[n] = (double)zb[src] + (double)bias_b[(size_t)r * D + c];
            V[n] = (double)cb[src];
            ++n;
          }
        }
        row[c] = softmax_pool(L, V, n);
      }
      double pos = entry_pos ? (double)entry_pos[(size_t)b * N + i] : (double)m * i;
      if (d_rope > 0) csk_ref_rope(row, D, d_rope, pos, rope_base);
      free(L);
      free(V);
    }
  }
  return 0;
}

/* HCA: the same pooling over one non-overlapping block of m tokens
 * ([P1] «HCA…»: compression m' = 128, no window overlap). */
int csk_ref_hca_compress(const float* c, const float* z, const float* bias, int B, int S, int D,
                         int m, int d_rope, double rope_base, const int32_t* entry_pos, double* out) {
  if (check_compress_args(B, S, D, m, d_rope)) return -1;
  const int N = S / m;
#pragma omp parallel for collapse(2) schedule(static)
  for (int b = 0; b < B; ++b) {
    for (int i = 0; i < N; ++i) {
      double* L = (double*)malloc(sizeof(double) * (size_t)m);
      double* V = (double*)malloc(sizeof(double) * (size_t)m);
      double* row = out + ((size_t)b * N + i) * D;
      for (int ch = 0; ch < D; ++ch) {
        for (int r = 0; r < m; ++r) {
          size_t src = ((size_t)b * S + (size_t)m * i + r) * D + ch;
          L[r] = (double)z[src] + (double)bias[(size_t)r * D + ch];
          V[r] = (double)c[src];
        }
        row[ch] = softmax_pool(L, V, m);
      }
      double pos = entry_pos ? (double)entry_pos[(size_t)b * N + i] : (double)m * i;
      if (d_rope > 0) csk_ref_rope(row, D, d_rope, pos, rope_base);
      free(L);
      free(V);
    }
  }
  return 0;
}

/* --------------------------------------------------------------- rounding */

/* Nearest bf16 (8 significant bits, exponent range of fp32), ties to even,
 * rounded once from the double value. */
static uint16_t round_one_bf16(double x) {
  if (isnan(x)) return 0x7fc0;
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  double a = fabs(x);
  if (a == 0.0) return sign;
  if (isinf(a)) return sign | 0x7f80;
  int e;
  frexp(a, &e);          /* a = f * 2^e, f in [0.5, 1) */
  int E = e - 1;          /* floor(log2 a) */
  if (E < -126) E = -126; /* subnormal range: fixed quantum 2^-133 */
  double quantum = ldexp(1.0, E - 7);
  double v = nearbyint(a / quantum) * quantum; /* default mode: ties to even */
  if (v >= ldexp(1.0, 128)) return sign | 0x7f80;
  float fv = (float)v; /* exact: v has at most 8 significant bits */
  uint32_t u;
  memcpy(&u, &fv, 4);
  return sign | (uint16_t)((u >> 16) & 0x7fff);
}

void csk_ref_round_bf16(const double* x, uint16_t* y, int64_t n) {
  for (int64_t i = 0; i < n; ++i) y[i] = round_one_bf16(x[i]);
}

void csk_ref_round_f32(const double* x, float* y, int64_t n) {
  for (int64_t i = 0; i < n; ++i) y[i] = (float)x[i];
}

/* ------------------------------------------------------------------ MXFP4 */

/* E2M1 magnitudes by 3-bit code; bit 3 of a code is the sign. */
static const double kE2M1[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

/* One 1x32 tile ([P1] «FP4 с учётом квантования»: MXFP4, E2M1, 1x32 tiles).
 * The shared scale is the power of two 2^s with s = floor(log2 amax) - 2
 * (2 = exponent of the largest E2M1 magnitude, 6 = 1.5 * 2^2), clamped to
 * the E8M0 range and stored as s + 127; an all-zero tile stores 127. Each
 * element becomes the E2M1 value nearest to x / 2^s, ties to the code with
 * an even mantissa bit, magnitudes past 6 saturating to 6. A result of zero
 * is always the +0 code. */
static void encode_tile(const float* x, uint8_t* codes, uint8_t* scale) {
  double amax = 0.0;
  for (int i = 0; i < 32; ++i)
    if (fabs((double)x[i]) > amax) amax = fabs((double)x[i]);
  if (amax == 0.0) {
    *scale = 127;
    memset(codes, 0, 16);
    return;
  }
  int e;
  frexp(amax, &e);
  int s = (e - 1) - 2;
  if (s < -127) s = -127;
  if (s > 127) s = 127;
  *scale = (uint8_t)(s + 127);
  uint8_t c4[32];
  for (int i = 0; i < 32; ++i) {
    double y = fabs((double)x[i]) * ldexp(1.0, -s);
    int best = 0;
    double bestd = fabs(y - kE2M1[0]);
    for (int c = 1; c < 8; ++c) {
      double d = fabs(y - kE2M1[c]);
      if (d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) == 1)) {
        best = c;
        bestd = d;
      }
    }
    c4[i] = (uint8_t)((best != 0 && x[i] < 0.0f) ? (best | 8) : best);
  }
  for (int j = 0; j < 16; ++j) codes[j] = (uint8_t)(c4[2 * j] | (c4[2 * j + 1] << 4));
}

int csk_ref_mxfp4_encode(const float* x, int64_t rows, int cols, uint8_t* codes, uint8_t* scales) {
  if (rows < 0 || cols <= 0 || cols % 32) return -1;
  const int tiles = cols / 32;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r)
    for (int t = 0; t < tiles; ++t)
      encode_tile(x + r * cols + 32 * t, codes + r * (cols / 2) + 16 * t, scales + r * tiles + t);
  return 0;
}

static double decode_code(uint8_t code) {
  double v = kE2M1[code & 7];
  return (code & 8) ? -v : v;
}

int csk_ref_mxfp4_decode(const uint8_t* codes, const uint8_t* scales, int64_t rows, int cols,
                         float* x) {
  if (rows < 0 || cols <= 0 || cols % 32) return -1;
  for (int64_t r = 0; r < rows; ++r)
    for (int i = 0; i < cols; ++i) {
      uint8_t byte = codes[r * (cols / 2) + i / 2];
      uint8_t code = (i & 1) ? (byte >> 4) : (byte & 15);
      int s = (int)scales[r * (cols / 32) + i / 32] - 127;
      x[r * cols + i] = (float)ldexp(decode_code(code), s);
    }
  return 0;
}

/* ---------------------------------------------------------------- indexer */

/* Round the exact value N * 2^e2 (N an integer) to the nearest float, ties
 * to even, in one step. Returns 0 and writes *out, or -1 if the value would
 * need more than 127 bits of N (never for in-range inputs). */
static float exact_to_f32(__int128 N, int e2) {
  if (N == 0) return 0.0f;
  int neg = N < 0;
  unsigned __int128 u = neg ? (unsigned __int128)(-N) : (unsigned __int128)N;
  int nb = 0;
  for (unsigned __int128 t = u; t; t >>= 1) ++nb;
  /* exponent of the last kept bit: 24 significant bits, but never below
   * the fp32 subnormal quantum 2^-149 */
  int lsb = e2 + nb - 24;
  if (lsb < -149) lsb = -149;
  int sh = lsb - e2;
  unsigned __int128 q = u;
  if (sh > 0) {
    unsigned __int128 rem = u & ((((unsigned __int128)1) << sh) - 1);
    unsigned __int128 half = ((unsigned __int128)1) << (sh - 1);
    q = u >> sh;
    if (rem > half || (rem == half && (q & 1))) q += 1;
  } else {
    lsb = e2;
  }
  double v = ldexp((double)q, lsb); /* q < 2^25: exact */
  if (v >= ldexp(1.0, 128)) v = INFINITY;
  return (float)(neg ? -v : v); /* exact: already on the fp32 grid */
}

/* Exact q.k of two MXFP4 vectors of length dI, rounded once to fp32. Within
 * a 32-tile the element products (2a)(2b) are integers, so the tile sum P_g
 * is an integer with |P_g| <= 32*144; the vector sum is
 * sum_g P_g * 2^(sq_g + sk_g - 2*127 - 2), formed exactly in 128-bit
 * integers. */
static int mxfp4_dot_f32(const uint8_t* qc, const uint8_t* qs, const uint8_t* kc,
                         const uint8_t* ks, int dI, float* out) {
  const int tiles = dI / 32;
  int64_t P[64];
  int E[64];
  int emin = 1 << 30;
  for (int g = 0; g < tiles; ++g) {
    int64_t acc = 0;
    for (int i = 0; i < 32; ++i) {
      int e = 32 * g + i;
      uint8_t a = (e & 1) ? (qc[e / 2] >> 4) : (qc[e / 2] & 15);
      uint8_t b = (e & 1) ? (kc[e / 2] >> 4) : (kc[e / 2] & 15);
      int64_t ia = (int64_t)(2.0 * decode_code(a)); /* 2 * E2M1 value is an integer */
      int64_t ib = (int64_t)(2.0 * decode_code(b));
      acc += ia * ib;
    }
    P[g] = acc;
    E[g] = ((int)qs[g] - 127) + ((int)ks[g] - 127) - 2;
    if (acc != 0 && E[g] < emin) emin = E[g];
  }
  __int128 total = 0;
  for (int g = 0; g < tiles; ++g) {
    if (P[g] == 0) continue;
    int sh = E[g] - emin;
    if (sh > 100) return -1;
    total += ((__int128)P[g]) << sh;
  }
  *out = exact_to_f32(total, emin == (1 << 30) ? 0 : emin);
  return 0;
}

/* I[t,s] = sum_h w[t,h] * ReLU(q[t,h] . k[s]) ([P1] «CSA…» step 2: the
 * lightning indexer scores I_{t,s} with ReLU; [P3]: ReLU-scored multi-head
 * dot product). The head sum is a fp32 fused multiply-add chain over h in
 * ascending order starting from +0; the fp32 path forms q.k as a fused
 * multiply-add chain over the channels in ascending order starting from +0.
 * Entry s is visible to a query at position p when its last source token
 * m*(s+1)-1 is <= p, and s < n_entries[b]. */
int csk_ref_indexer_scores(const float* qf, const uint8_t* qc, const uint8_t* qs, const float* w,
                           const float* kf, const uint8_t* kc, const uint8_t* ks,
                           const int32_t* q_pos, const int32_t* n_entries, int B, int T, int HI,
                           int dI, int Nmax, int m, int dtype, const int32_t* rows, int n_rows,
                           float* scores, int32_t* n_vis) {
  if (B <= 0 || T <= 0 || HI <= 0 || dI <= 0 || Nmax < 0 || m <= 0 || n_rows < 0) return -1;
  if (dtype != 0 && dtype != 2) return -1;
  if (dtype == 2 && (dI % 32 || dI > 2048)) return -1;
  int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int r = 0; r < n_rows; ++r) {
    int b = rows[2 * r], t = rows[2 * r + 1];
    float* out = scores + (size_t)r * Nmax;
    for (int s = 0; s < Nmax; ++s) out[s] = -INFINITY;
    if (b < 0 || b >= B || t < 0 || t >= T) {
      n_vis[r] = 0;
#pragma omp atomic write
      err = -1;
      continue;
    }
    int64_t p = q_pos[(size_t)b * T + t];
    int64_t nv = (p + 1) / m;
    if (p < 0) nv = 0;
    if (nv > n_entries[b]) nv = n_entries[b];
    if (nv > Nmax) nv = Nmax;
    n_vis[r] = (int32_t)nv;
    for (int s = 0; s < nv; ++s) {
      float acc = 0.0f;
      for (int h = 0; h < HI; ++h) {
        float d = 0.0f;
        size_t qrow = ((size_t)b * T + t) * HI + h;
        size_t krow = (size_t)b * Nmax + s;
        if (dtype == 0) {
          for (int i = 0; i < dI; ++i) d = fmaf(qf[qrow * dI + i], kf[krow * dI + i], d);
        } else {
          if (mxfp4_dot_f32(qc + qrow * (dI / 2), qs + qrow * (dI / 32), kc + krow * (dI / 2),
                            ks + krow * (dI / 32), dI, &d)) {
#pragma omp atomic write
            err = -2;
          }
        }
        float relu = d > 0.0f ? d : 0.0f;
        acc = fmaf(w[qrow], relu, acc);
      }
      out[s] = acc;
    }
  }
  return err;
}

/* ---------------------------------------------------------- FP8 KV entries */

/* [P2] (FP8 storage finding) and [P1] «Почему это так сильно экономит»,
 * item 1: KV entries are stored in FP8 except the RoPE dims, which stay in
 * BF16. The pages fix no scale granularity; the reading here: the D_nope =
 * D - d_rope non-RoPE dims are OCP E4M3 values (sign, 4 exponent bits with
 * bias 7, 3 mantissa bits; exponent 0 is subnormal, m * 2^-9; the all-ones
 * code is NaN and never produced) with one power-of-two scale byte (2^(byte
 * - 127)) per 32 consecutive dims, chosen so that the block's largest
 * magnitude lands in [128, 256): s = floor(log2 amax) - 7, clamped to
 * [-126, 127]; an all-zero block gets byte 127. Codes are the nearest E4M3
 * value of x / 2^s, ties to the even mantissa; zero (and anything that
 * rounds to it) is the +0 code. Entry bytes: [D_nope codes][d_rope bf16
 * values][D_nope/32 scale bytes], padded with zeros to a multiple of 16. */
static double e4m3_value(int code) {
  const int e = (code >> 3) & 15, mnt = code & 7;
  const double mag = e == 0 ? ldexp((double)mnt, -9) : ldexp(1.0 + mnt / 8.0, e - 7);
  return (code & 0x80) ? -mag : mag;
}

/* Nearest non-negative E4M3 code of y in [0, 448]: the plain definition,
 * a search over the 127 finite codes (their values in `val`); ties go to the
 * code whose mantissa (its low bit) is even. */
static int e4m3_code_abs(double y, const double* val) {
  int best = 0;
  double bd = INFINITY;
  for (int c = 0; c < 127; ++c) {
    const double d = fabs(val[c] - y);
    if (d < bd || (d == bd && (c & 1) == 0)) {
      best = c;
      bd = d;
    }
  }
  return best;
}

int csk_ref_fp8kv_entry_bytes(int D, int d_rope) {
  const int dn = D - d_rope;
  const int raw = dn + 2 * d_rope + dn / 32;
  return (raw + 15) / 16 * 16;
}

int csk_ref_fp8kv_encode(const float* x, int64_t rows, int D, int d_rope, uint8_t* out) {
  const int dn = D - d_rope;
  if (D <= 0 || d_rope < 0 || d_rope > D || (d_rope & 1) || dn % 32 || rows < 0) return -1;
  const int ES = csk_ref_fp8kv_entry_bytes(D, d_rope);
  double val[127];
  for (int c = 0; c < 127; ++c) val[c] = e4m3_value(c);
  /* entries are independent: one per iteration, any thread */
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    const float* xr = x + r * D;
    uint8_t* o = out + r * ES;
    memset(o, 0, (size_t)ES);
    for (int g = 0; g < dn / 32; ++g) {
      double amax = 0.0;
      for (int i = 0; i < 32; ++i) amax = fmax(amax, fabs((double)xr[32 * g + i]));
      int s = 0, byte = 127;
      if (amax > 0.0) {
        int e;
        frexp(amax, &e);  /* amax = f * 2^e, f in [0.5, 1): floor(log2 amax) = e - 1 */
        s = e - 1 - 7;
        if (s < -126) s = -126;
        if (s > 127) s = 127;
        byte = s + 127;
      }
      o[dn + 2 * d_rope + g] = (uint8_t)byte;
      for (int i = 0; i < 32; ++i) {
        const double v = (double)xr[32 * g + i];
        const int c = amax > 0.0 ? e4m3_code_abs(ldexp(fabs(v), -s), val) : 0;
        o[32 * g + i] = (uint8_t)((v < 0.0 && c != 0) ? (c | 0x80) : c);
      }
    }
    for (int j = 0; j < d_rope; ++j) {
      const uint16_t h = round_one_bf16((double)xr[dn + j]);
      o[dn + 2 * j] = (uint8_t)(h & 0xff);
      o[dn + 2 * j + 1] = (uint8_t)(h >> 8);
    }
  }
  return 0;
}

int csk_ref_fp8kv_decode(const uint8_t* in, int64_t rows, int D, int d_rope, float* x) {
  const int dn = D - d_rope;
  if (D <= 0 || d_rope < 0 || d_rope > D || (d_rope & 1) || dn % 32 || rows < 0) return -1;
  const int ES = csk_ref_fp8kv_entry_bytes(D, d_rope);
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    const uint8_t* e = in + r * ES;
    float* xr = x + r * D;
    for (int i = 0; i < dn; ++i)
      xr[i] = (float)ldexp(e4m3_value(e[i]), (int)e[dn + 2 * d_rope + i / 32] - 127);
    for (int j = 0; j < d_rope; ++j) {
      const uint32_t u = ((uint32_t)e[dn + 2 * j] | ((uint32_t)e[dn + 2 * j + 1] << 8)) << 16;
      memcpy(&xr[dn + j], &u, 4);
    }
  }
  return 0;
}

/* BF16 indexer scores ([P1] «FP4 с учётом квантования»: the scores that the
 * top-k selects from are kept in BF16, which the page credits with a faster
 * top-k at a small loss of recall): every fp32 score is rounded once to the
 * nearest bf16, ties to even, and stored back as the float of that bf16. */
void csk_ref_scores_bf16(float* scores, int64_t n) {
  for (int64_t i = 0; i < n; ++i) {
    const uint32_t u = (uint32_t)round_one_bf16((double)scores[i]) << 16;
    memcpy(&scores[i], &u, 4);
  }
}

/* ------------------------------------------------------------------ top-k */

typedef struct {
  float score;
  int32_t s;
} cand_t;

/* score descending, then index ascending */
static int cmp_rank(const void* pa, const void* pb) {
  const cand_t* a = (const cand_t*)pa;
  const cand_t* b = (const cand_t*)pb;
  if (a->score > b->score) return -1;
  if (a->score < b->score) return 1;
  return (a->s > b->s) - (a->s < b->s);
}

static int cmp_index(const void* pa, const void* pb) {
  const cand_t* a = (const cand_t*)pa;
  const cand_t* b = (const cand_t*)pb;
  return (a->s > b->s) - (a->s < b->s);
}

/* [P1] «CSA…» step 2: the indexer picks the top-k compressed blocks per
 * query. Selection by full sort; ties go to the lower index. */
int csk_ref_topk(const float* scores, const int32_t* n_vis, int n_rows, int Nmax, int k,
                 int32_t* idx, float* out_scores) {
  if (n_rows < 0 || Nmax < 0 || k <= 0) return -1;
#pragma omp parallel for schedule(dynamic, 1)
  for (int r = 0; r < n_rows; ++r) {
    int n = n_vis[r];
    if (n > Nmax) n = Nmax;
    if (n < 0) n = 0;
    cand_t* c = (cand_t*)malloc(sizeof(cand_t) * (size_t)(n > 0 ? n : 1));
    for (int s = 0; s < n; ++s) {
      c[s].score = scores[(size_t)r * Nmax + s];
      c[s].s = s;
    }
    qsort(c, (size_t)n, sizeof(cand_t), cmp_rank);
    int sel = n < k ? n : k;
    qsort(c, (size_t)sel, sizeof(cand_t), cmp_index);
    for (int j = 0; j < k; ++j) {
      idx[(size_t)r * k + j] = j < sel ? c[j].s : -1;
      out_scores[(size_t)r * k + j] = j < sel ? c[j].score : -INFINITY;
    }
    free(c);
  }
  return 0;
}

/* -------------------------------------------------------------- attention */

/* One softmax over the candidate set plus the sink for one (row, head):
 * logits l_j = scale * (q~ . K_j); the sink adds exp(sink - M) to the
 * denominator and nothing to the numerator; out = sum_j p_j K_j[0:dv],
 * lse = M + log Z. Each entry is both key and value for every head
 * ([P1] «CSA…» step 3, MQA). With no candidate and no sink the output is 0
 * and lse is -inf. */
static void attend_one(const double* qr, const float* const* K, int nc, const float* sink_h,
                       int D, int dv, double scale, double* out, double* lse) {
  double* l = (double*)malloc(sizeof(double) * (size_t)(nc > 0 ? nc : 1));
  double M = -INFINITY;
  for (int j = 0; j < nc; ++j) {
    double dot = 0.0;
    for (int c = 0; c < D; ++c) dot += qr[c] * (double)K[j][c];
    l[j] = scale * dot;
    if (l[j] > M) M = l[j];
  }
  if (sink_h && (double)*sink_h > M) M = (double)*sink_h;
  for (int c = 0; c < dv; ++c) out[c] = 0.0;
  if (M == -INFINITY) {
    *lse = -INFINITY;
    free(l);
    return;
  }
  double Z = sink_h ? exp((double)*sink_h - M) : 0.0;
  for (int j = 0; j < nc; ++j) {
    double p = exp(l[j] - M);
    Z += p;
    for (int c = 0; c < dv; ++c) out[c] += p * (double)K[j][c];
  }
  for (int c = 0; c < dv; ++c) out[c] /= Z;
  *lse = M + log(Z);
  free(l);
}

static int check_attn_args(int B, int T, int H, int D, int dv, int d_rope, int W, int S_w,
                           int n_rows) {
  if (B <= 0 || T <= 0 || H <= 0 || D <= 0 || dv <= 0 || dv > D || n_rows < 0) return -1;
  if (d_rope < 0 || d_rope > D || (d_rope & 1) || W < 0 || S_w < 0) return -1;
  return 0;
}

/* Window candidates: the uncompressed tokens at positions
 * [max(0, p - W + 1), p] that the window buffer holds ([P1] «HCA…»: a
 * sliding window of 128 uncompressed tokens; [P4]: SWA branch). */
static int add_window(const float* kv_w, const int32_t* w_pos0, int S_w, int W, int b, int D,
                      int64_t p, const float** K, int nc) {
  if (W <= 0) return nc;
  int64_t lo = p - W + 1;
  if (lo < 0) lo = 0;
  for (int r = 0; r < S_w; ++r) {
    int64_t pos = (int64_t)w_pos0[b] + r;
    if (pos >= lo && pos <= p) K[nc++] = kv_w + ((size_t)b * S_w + r) * D;
  }
  return nc;
}

int csk_ref_sparse_attn(const float* q, const int32_t* q_pos, const float* kv_c, int Nmax,
                        const int32_t* idx, int k, const float* kv_w, const int32_t* w_pos0,
                        int S_w, int W, const float* sink, int B, int T, int H, int D, int dv,
                        int d_rope, double rope_base, double scale, const int32_t* rows,
                        int n_rows, double* out, double* lse) {
  if (check_attn_args(B, T, H, D, dv, d_rope, W, S_w, n_rows) || k < 0 || Nmax < 0) return -1;
  int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int r = 0; r < n_rows; ++r) {
    int b = rows[2 * r], t = rows[2 * r + 1];
    if (b < 0 || b >= B || t < 0 || t >= T) {
#pragma omp atomic write
      err = -1;
      continue;
    }
    int64_t p = q_pos[(size_t)b * T + t];
    const float** K = (const float**)malloc(sizeof(float*) * (size_t)(k + S_w + 1));
    int nc = 0;
    for (int j = 0; j < k; ++j) {
      int32_t i = idx[((size_t)b * T + t) * k + j];
      if (i < 0 || i >= Nmax) continue;
      K[nc++] = kv_c + ((size_t)b * Nmax + i) * D;
    }
    nc = add_window(kv_w, w_pos0, S_w, W, b, D, p, K, nc);
    double* qr = (double*)malloc(sizeof(double) * (size_t)D);
    for (int h = 0; h < H; ++h) {
      const float* qh = q + (((size_t)b * T + t) * H + h) * D;
      for (int c = 0; c < D; ++c) qr[c] = (double)qh[c];
      csk_ref_rope(qr, D, d_rope, (double)p, rope_base);
      attend_one(qr, K, nc, sink ? sink + h : NULL, D, dv, scale,
                 out + ((size_t)r * H + h) * dv, lse + (size_t)r * H + h);
    }
    free(qr);
    free(K);
  }
  return err;
}

int csk_ref_dense_attn(const float* q, const int32_t* q_pos, const float* kv_c, int Nmax,
                       const int32_t* n_entries, int m, const float* kv_w, const int32_t* w_pos0,
                       int S_w, int W, const float* sink, int B, int T, int H, int D, int dv,
                       int d_rope, double rope_base, double scale, const int32_t* rows,
                       int n_rows, double* out, double* lse) {
  if (check_attn_args(B, T, H, D, dv, d_rope, W, S_w, n_rows) || m <= 0 || Nmax < 0) return -1;
  int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int r = 0; r < n_rows; ++r) {
    int b = rows[2 * r], t = rows[2 * r + 1];
    if (b < 0 || b >= B || t < 0 || t >= T) {
#pragma omp atomic write
      err = -1;
      continue;
    }
    int64_t p = q_pos[(size_t)b * T + t];
    int ne = n_entries[b] < Nmax ? n_entries[b] : Nmax;
    const float** K = (const float**)malloc(sizeof(float*) * (size_t)(ne + S_w + 1));
    int nc = 0;
    for (int i = 0; i < ne; ++i)
      if ((int64_t)m * (i + 1) - 1 <= p) K[nc++] = kv_c + ((size_t)b * Nmax + i) * D;
    nc = add_window(kv_w, w_pos0, S_w, W, b, D, p, K, nc);
    double* qr = (double*)malloc(sizeof(double) * (size_t)D);
    for (int h = 0; h < H; ++h) {
      const float* qh = q + (((size_t)b * T + t) * H + h) * D;
      for (int c = 0; c < D; ++c) qr[c] = (double)qh[c];
      csk_ref_rope(qr, D, d_rope, (double)p, rope_base);
      attend_one(qr, K, nc, sink ? sink + h : NULL, D, dv, scale,
                 out + ((size_t)r * H + h) * dv, lse + (size_t)r * H + h);
    }
    free(qr);
    free(K);
  }
  return err;
}

/* ------------------------------------------ grouped output projection */

/* [P1] «CSA: сжать в 4 раза и выбрать top-k», step 4: the heads' outputs
 * are not projected to the hidden size in one matrix; they are split into
 * g groups, each group is projected to an intermediate width (1024 in the
 * pages' model), and the groups' intermediates together are projected to
 * the hidden state. Here: row r's outputs o[r] = [head 0 | head 1 | ...]
 * (H*dv values); group i holds heads i*H/g .. (i+1)*H/g - 1, i.e. the K1 =
 * (H/g)*dv values o[r][i*K1 .. (i+1)*K1); u[r][i*dg + n] = sum_k
 * o[r][i*K1 + k] * w1[i][n][k]; y[r][c] = sum_j u[r][j] * w2[c][j]. Weights
 * are [out, in] (each output feature's inputs contiguous). Reading: the
 * intermediate is an activation of a bf16 model, rounded once to bf16
 * before the second projection; y is returned in double. */
int csk_ref_grouped_out_proj(const float* o, const float* w1, const float* w2, int R, int H, int dv,
                             int g, int dg, int d, float* u_out, double* y) {
  if (R < 0 || H <= 0 || dv <= 0 || g <= 0 || H % g || dg <= 0 || d <= 0) return -1;
  const int K1 = H / g * dv, K2 = g * dg;
#pragma omp parallel for schedule(static)
  for (int r = 0; r < R; ++r) {
    const float* orow = o + (size_t)r * H * dv;
    float* u = (float*)malloc(sizeof(float) * (size_t)K2);
    for (int i = 0; i < g; ++i) {
      for (int n = 0; n < dg; ++n) {
        const float* wrow = w1 + ((size_t)i * dg + n) * K1;
        double acc = 0.0;
        for (int k = 0; k < K1; ++k) acc += (double)orow[(size_t)i * K1 + k] * (double)wrow[k];
        const uint32_t bits = (uint32_t)round_one_bf16(acc) << 16;
        memcpy(&u[i * dg + n], &bits, 4);
      }
    }
    for (int c = 0; c < d; ++c) {
      const float* wrow = w2 + (size_t)c * K2;
      double acc = 0.0;
      for (int j = 0; j < K2; ++j) acc += (double)u[j] * (double)wrow[j];
      y[(size_t)r * d + c] = acc;
    }
    if (u_out) memcpy(u_out + (size_t)r * K2, u, sizeof(float) * (size_t)K2);
    free(u);
  }
  return 0;
}

/* ----------------------------------------------------- QK RMSNorm */

/* [P1] «Muon и борьба с нестабильностью»: queries and KV entries can be
 * normalised directly with RMSNorm; [P4]: QK norms for stability. Reading:
 * the norm runs over all D values of a vector (RoPE dims included, before
 * the rotation), y = x * gamma / sqrt(mean(x^2) + eps), gamma a learned
 * per-dim scale. */
static void rmsnorm_row(double* v, const float* gamma, int D, double eps) {
  double ss = 0.0;
  for (int c = 0; c < D; ++c) ss += v[c] * v[c];
  const double inv = 1.0 / sqrt(ss / D + eps);
  for (int c = 0; c < D; ++c) v[c] = v[c] * inv * (double)gamma[c];
}

int csk_ref_rmsnorm(const float* x, const float* gamma, int64_t rows, int D, double eps, double* y) {
  if (rows < 0 || D <= 0 || !(eps >= 0.0)) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    double* v = y + r * D;
    for (int c = 0; c < D; ++c) v[c] = (double)x[r * D + c];
    rmsnorm_row(v, gamma, D, eps);
  }
  return 0;
}

/* ------------------------------------- projection, then compression */

/* [P1] «CSA…» step 1: the two KV series and the two weight series are
 * computed from the hidden states; here by learned projections
 * (series s = X W_s^T, W_s [D, hidden], [out, in]). CSA (csa = 1): w holds
 * W_ca, W_za, W_cb, W_zb and the entries pool as csk_ref_csa_compress; HCA
 * (csa = 0): w holds W_c, W_z and the entries pool as
 * csk_ref_hca_compress. Then, when gamma is given, each entry is
 * RMS-normalised ([P1] «Muon…»), and its last d_rope dims are rotated at
 * the entry's position. Everything in double, from the exact products. */
int csk_ref_project_compress(const float* x, const float* w, const float* bias_a, const float* bias_b,
                             const float* gamma, double eps, int csa, int B, int S, int hidden, int D,
                             int m, int d_rope, double rope_base, const int32_t* entry_pos, double* out) {
  if (check_compress_args(B, S, D, m, d_rope) || hidden <= 0 || !(eps >= 0.0)) return -1;
  const int NS = csa ? 4 : 2, N = S / m;
  /* the projected series, [NS][B][S][D] */
  double* ser = (double*)malloc(sizeof(double) * (size_t)NS * B * S * D);
  if (!ser) return -1;
#pragma omp parallel for collapse(2) schedule(static)
  for (int b = 0; b < B; ++b)
    for (int t = 0; t < S; ++t)
      for (int s = 0; s < NS; ++s)
        for (int c = 0; c < D; ++c) {
          const float* xr = x + ((size_t)b * S + t) * hidden;
          const float* wr = w + ((size_t)s * D + c) * hidden;
          double acc = 0.0;
          for (int k = 0; k < hidden; ++k) acc += (double)xr[k] * (double)wr[k];
          ser[(((size_t)s * B + b) * S + t) * D + c] = acc;
        }
#define SER(s, b, t, c) ser[(((size_t)(s) * B + (b)) * S + (t)) * D + (c)]
#pragma omp parallel for collapse(2) schedule(static)
  for (int b = 0; b < B; ++b) {
    for (int i = 0; i < N; ++i) {
      double* L = (double*)malloc(sizeof(double) * 2 * (size_t)m);
      double* V = (double*)malloc(sizeof(double) * 2 * (size_t)m);
      double* row = out + ((size_t)b * N + i) * D;
      for (int c = 0; c < D; ++c) {
        int n = 0;
        for (int r = 0; r < m; ++r) {
          const int t = m * i + r;
          L[n] = SER(1, b, t, c) + (double)bias_a[(size_t)r * D + c];
          V[n] = SER(0, b, t, c);
          ++n;
        }
        if (csa && i >= 1) {
          for (int r = 0; r < m; ++r) {
            const int t = m * (i - 1) + r;
            L[n] = SER(3, b, t, c) + (double)bias_b[(size_t)r * D + c];
            V[n] = SER(2, b, t, c);
            ++n;
          }
        }
        row[c] = softmax_pool(L, V, n);
      }
      if (gamma) rmsnorm_row(row, gamma, D, eps);
      double pos = entry_pos ? (double)entry_pos[(size_t)b * N + i] : (double)m * i;
      if (d_rope > 0) csk_ref_rope(row, D, d_rope, pos, rope_base);
      free(L);
      free(V);
    }
  }
#undef SER
  free(ser);
  return 0;
}
