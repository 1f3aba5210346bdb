/*
 * kvq_oracle.c -- TEST INFRASTRUCTURE ONLY (see kvq_oracle.h).
 *
 * Plain sequential C.  Floating-point contract of the encoder (the part the
 * GPU must reproduce bit for bit): IEEE fp32, round to nearest even, no fused
 * multiply-add (built with -ffp-contract=off), correctly rounded sqrtf and
 * division.  Reconstruction and attention are computed in fp64 from the plain
 * definitions (explicit Hadamard matrix, explicit S^T product, two-pass
 * softmax over materialised keys and values).
 *
 * Packed record layout (the pages print none; this is the reading used):
 *   bits in {1,2,4}: code i occupies bits [i*b, i*b+b) of the record, bytes
 *                    little-endian, i.e. byte (i*b)/8, shift (i*b)%8.
 *   bits == 3:       a 2-bit plane (low two bits of every code, laid out as
 *                    for b=2, d/4 bytes) followed by a 1-bit plane (the high
 *                    bit of every code, laid out as for b=1, d/8 bytes).
 *   sign bits:       bit k of the sketch at byte k/8, shift k%8.
 * These per-slot records are what orc_encode / orc_decode exchange.  A cache
 * side stores them per slot, or (value side at d = 128) in token groups whose
 * bit positions orc_vgroup_code_bit / orc_vgroup_sign_bit define.
 */
#include "kvq_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Number formats                                                            */
/* ------------------------------------------------------------------------ */

static uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float bits_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* IEEE binary16, round to nearest, ties to even; overflow gives infinity. */
uint16_t orc_f32_to_f16(float f) {
  uint32_t x = f32_bits(f);
  uint16_t sign = (uint16_t)((x >> 16) & 0x8000u);
  uint32_t a = x & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return (uint16_t)(sign | 0x7E00u);         /* NaN */
  if (a >= 0x477FF000u) return (uint16_t)(sign | 0x7C00u);        /* >= 65520 -> inf */
  int e = (int)(a >> 23);                                         /* biased fp32 exponent */
  uint32_t mant = a & 0x7FFFFFu;
  if (e >= 113) {                                                 /* normal binary16 */
    uint32_t h = ((uint32_t)(e - 112) << 10) | (mant >> 13);
    uint32_t rest = mant & 0x1FFFu;
    if (rest > 0x1000u || (rest == 0x1000u && (h & 1u))) h += 1u; /* carry may bump exponent */
    return (uint16_t)(sign | h);
  }
  /* subnormal binary16 (or zero): value = m * 2^(e-150); unit = 2^-24 */
  if (e == 0) return sign;                                        /* fp32 subnormal: < 2^-126 */
  uint32_t m = mant | 0x800000u;
  int s = 126 - e;                                                /* q = m >> s */
  if (s > 24) return sign;                                        /* < 2^-25 rounds to 0 */
  uint32_t q = m >> s;
  uint32_t rem = m & ((1u << s) - 1u);
  uint32_t half = 1u << (s - 1);
  if (rem > half || (rem == half && (q & 1u))) q += 1u;
  return (uint16_t)(sign | q);
}

/* bfloat16 = upper half of binary32, round to nearest, ties to even. */
uint16_t orc_f32_to_bf16(float f) {
  uint32_t x = f32_bits(f);
  if ((x & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((x >> 16) | 0x40u);
  uint32_t lsb = (x >> 16) & 1u;
  x += 0x7FFFu + lsb;
  return (uint16_t)(x >> 16);
}

float orc_bf16_to_f32(uint16_t h) { return bits_f32((uint32_t)h << 16); }

double orc_f16_to_f64(uint16_t h) {
  int e = (h >> 10) & 0x1F;
  int mnt = h & 0x3FF;
  double s = (h & 0x8000) ? -1.0 : 1.0;
  if (e == 0x1F) return mnt ? NAN : s * INFINITY;
  if (e == 0) return s * ldexp((double)mnt, -24);
  return s * ldexp((double)(mnt + 1024), e - 25);
}

/* ------------------------------------------------------------------------ */
/* Codebook: Lloyd-Max on f(t) ~ (1 - t^2)^((d-3)/2) over [-1, 1]            */
/* [KPP] "Codebook design"; [DA] "Theoretical framework" (a coordinate of a  */
/* uniform point on S^{d-1} has (1+t)/2 ~ Beta((d-1)/2, (d-1)/2)).           */
/* ------------------------------------------------------------------------ */

#define GL_N 20
static double gl_x[GL_N], gl_w[GL_N];
static pthread_once_t gl_once = PTHREAD_ONCE_INIT;

/* Gauss-Legendre nodes on [-1,1] by Newton iteration on P_n. */
static void gl_init(void) {
  const int n = GL_N;
  for (int i = 0; i < n; ++i) {
    double z = cos(M_PI * (i + 0.75) / (n + 0.5)), pp = 0.0;
    for (int it = 0; it < 100; ++it) {
      double p1 = 1.0, p2 = 0.0;
      for (int j = 1; j <= n; ++j) {
        double p3 = p2;
        p2 = p1;
        p1 = ((2.0 * j - 1.0) * z * p2 - (j - 1.0) * p3) / j;
      }
      pp = n * (z * p1 - p2) / (z * z - 1.0);
      double z1 = z;
      z = z1 - p1 / pp;
      if (fabs(z - z1) < 1e-16) break;
    }
    gl_x[i] = z;
    gl_w[i] = 2.0 / ((1.0 - z * z) * pp * pp);
  }
}

/* Integrals over [a,b] of w(t) and t*w(t), w(t) = (1-t^2)^alpha, by composite
 * Gauss-Legendre on 64 equal sub-intervals. */
static void cell_integrals(double a, double b, double alpha, double *mass, double *moment) {
  const int ns = 64;
  double h = (b - a) / ns, m0 = 0.0, m1 = 0.0;
  for (int s = 0; s < ns; ++s) {
    double lo = a + s * h, mid = lo + 0.5 * h;
    for (int i = 0; i < GL_N; ++i) {
      double t = mid + 0.5 * h * gl_x[i];
      double w = pow(1.0 - t * t, alpha) * gl_w[i] * 0.5 * h;
      m0 += w;
      m1 += t * w;
    }
  }
  *mass = m0;
  *moment = m1;
}

int orc_codebook(int d, int bits, double *pos_c64, float *centroid, float *threshold) {
  if (d < 3 || bits < 1 || bits > 8) return -1;
  pthread_once(&gl_once, gl_init);
  const int K = 1 << bits, K2 = K / 2;
  const double alpha = 0.5 * (d - 3);
  double *c = (double *)malloc(sizeof(double) * K2);
  double *t = (double *)malloc(sizeof(double) * (K2 + 1));
  /* start: equally spaced in (0, s), s = min(0.9, 3/sqrt(d)); the fixed point
   * is unique for this log-concave density, so the start only sets speed. */
  double span = fmin(0.9, 3.0 / sqrt((double)d));
  for (int i = 0; i < K2; ++i) c[i] = span * (i + 0.5) / K2;
  int it = 0, quiet = 0;
  for (it = 1; it <= 200000; ++it) {
    t[0] = 0.0;
    t[K2] = 1.0;
    for (int i = 1; i < K2; ++i) t[i] = 0.5 * (c[i - 1] + c[i]);
    double dd = 0.0, cmax = 0.0;
    for (int i = 0; i < K2; ++i) {
      double P, M;
      cell_integrals(t[i], t[i + 1], alpha, &P, &M);
      double cn = M / P;                 /* centroid = conditional mean of the cell */
      dd = fmax(dd, fabs(cn - c[i]));
      cmax = fmax(cmax, fabs(cn));
      c[i] = cn;
    }
    if (dd <= 4.0 * 2.220446049250313e-16 * cmax) break;
    quiet = (dd < 1e-13 * cmax) ? quiet + 1 : 0; /* at the rounding-noise floor */
    if (quiet >= 64) break;
  }
  /* Stored levels: the fp32 level rounded to the nearest binary16 (ties to
   * even), held as fp32.  Thresholds: fp32 of the fp64 midpoint of two
   * stored levels, so bucketize returns the nearest stored level. */
  double s16[256];
  for (int i = 0; i < K2; ++i) {
    if (pos_c64) pos_c64[i] = c[i];
    s16[i] = orc_f16_to_f64(orc_f32_to_f16((float)c[i]));
    float f = (float)s16[i];
    centroid[K2 + i] = f;
    centroid[K2 - 1 - i] = -f;
  }
  threshold[K2 - 1] = 0.0f;
  for (int i = 0; i + 1 < K2; ++i) {
    float f = (float)(0.5 * (s16[i] + s16[i + 1]));
    threshold[K2 + i] = f;
    threshold[K2 - 2 - i] = -f;
  }
  free(c);
  free(t);
  return it;
}

/* ------------------------------------------------------------------------ */
/* Encoder pieces                                                            */
/* ------------------------------------------------------------------------ */

/* y <- H y, Sylvester order, stages h = 1, 2, 4, ... (ascending); each pair
 * (y_i, y_{i+h}) with (i & h) == 0 becomes (y_i + y_{i+h}, y_i - y_{i+h}).
 * [DA] "Quantization schemes": WHT applied before scalar quantisation. */
void orc_wht_f32(float *y, int d) {
  for (int h = 1; h < d; h <<= 1)
    for (int i = 0; i < d; ++i)
      if ((i & h) == 0) {
        float a = y[i], b = y[i + h];
        y[i] = a + b;
        y[i + h] = a - b;
      }
}

/* Squares rounded to fp32, then summed by adjacent pairs, level by level:
 * z_i <- z_{2i} + z_{2i+1} until one value remains. */
float orc_sumsq_f32(const float *y, int d) {
  float z[4096];
  for (int i = 0; i < d; ++i) z[i] = y[i] * y[i];
  for (int n = d; n > 1; n >>= 1)
    for (int i = 0; i < n / 2; ++i) z[i] = z[2 * i] + z[2 * i + 1];
  return z[0];
}

/* [KPP] "Fast codebook lookup": bucketize against the sorted thresholds; the
 * code is the count of thresholds strictly below u (a tie goes to the lower
 * cell), which equals the index of the nearest centroid. */
int orc_bucketize(float u, const float *threshold, int nthr) {
  int c = 0;
  for (int t = 0; t < nthr; ++t) c += (threshold[t] < u) ? 1 : 0;
  return c;
}

static void put_code(uint8_t *rec, int d, int bits, int i, int code) {
  if (bits == 3) {
    rec[(2 * i) / 8] |= (uint8_t)((code & 3) << ((2 * i) % 8));
    rec[d / 4 + i / 8] |= (uint8_t)(((code >> 2) & 1) << (i % 8));
  } else {
    rec[(i * bits) / 8] |= (uint8_t)(code << ((i * bits) % 8));
  }
}

static int get_code(const uint8_t *rec, int d, int bits, int i) {
  if (bits == 3) {
    int lo = (rec[(2 * i) / 8] >> ((2 * i) % 8)) & 3;
    int hi = (rec[d / 4 + i / 8] >> (i % 8)) & 1;
    return lo | (hi << 2);
  }
  return (rec[(i * bits) / 8] >> ((i * bits) % 8)) & ((1 << bits) - 1);
}

/* Token-group storage of the value side at d = 128 (the library's format; the
 * pages fix none).  R = 16 b bytes per slot.
 * Codes: slots 4q .. 4q+3 share bytes [4q R, 4q R + 4R).  Piece n = c / 8
 * (coordinates 8n .. 8n+7) starts at 4q R + 4 b n.  With r = slot % 4 and
 * j = c % 8, bit i of the code of (slot, c) is at
 *   b = 4: byte 2j + r/2 of the piece, bit 4 (r%2) + i
 *   b = 3: P = the 6-bit pair field u = 2j + r/2, bit pb = 3 (r%2) + i of P;
 *          u < 12: byte u, bit 2 + pb; u >= 12: byte 4 (pb/2) + u - 12, bit pb%2
 *   b = 2: byte j, bit 2r + i
 *   b = 1: byte j/2, bit 4 (j%2) + r
 * Sign bits: slots 8o .. 8o+7 share bytes [128 o, 128 o + 128); the sign of
 * (slot, sketch row k) is bit slot % 8 of byte 128 o + k. */
void orc_vgroup_code_bit(int bits, size_t slot, int c, int i, size_t *byte, int *bit) {
  const size_t rec = (size_t)16 * bits;
  const size_t piece = (slot / 4) * 4 * rec + (size_t)(c / 8) * (size_t)(4 * bits);
  const int r = (int)(slot % 4), j = c % 8;
  if (bits == 4) {
    *byte = piece + (size_t)(2 * j + r / 2);
    *bit = 4 * (r % 2) + i;
  } else if (bits == 3) {
    const int u = 2 * j + r / 2, pb = 3 * (r % 2) + i;
    if (u < 12) {
      *byte = piece + (size_t)u;
      *bit = 2 + pb;
    } else {
      *byte = piece + (size_t)(4 * (pb / 2) + u - 12);
      *bit = pb % 2;
    }
  } else if (bits == 2) {
    *byte = piece + (size_t)j;
    *bit = 2 * r + i;
  } else {
    *byte = piece + (size_t)(j / 2);
    *bit = 4 * (j % 2) + r;
  }
}

void orc_vgroup_sign_bit(size_t slot, int k, size_t *byte, int *bit) {
  *byte = (slot / 8) * 128 + (size_t)k;
  *bit = (int)(slot % 8);
}

static void set_bit(uint8_t *p, size_t byte, int bit, int v) {
  p[byte] = (uint8_t)((p[byte] & ~(1u << bit)) | ((unsigned)(v & 1) << bit));
}

void orc_load_record(const uint8_t *codes, const uint8_t *signs, int grouped, size_t slot,
                     int d, int bits, int qjl, int m, uint8_t *rec, uint8_t *sg) {
  const size_t cb = (size_t)d * bits / 8, sbytes = (size_t)m / 8;
  if (!grouped) {
    memcpy(rec, codes + slot * cb, cb);
    if (qjl) memcpy(sg, signs + slot * sbytes, sbytes);
    return;
  }
  memset(rec, 0, cb);
  for (int c = 0; c < d; ++c) {
    int code = 0;
    for (int i = 0; i < bits; ++i) {
      size_t by;
      int bt;
      orc_vgroup_code_bit(bits, slot, c, i, &by, &bt);
      code |= ((codes[by] >> bt) & 1) << i;
    }
    put_code(rec, d, bits, c, code);
  }
  if (!qjl) return;
  memset(sg, 0, sbytes);
  for (int k = 0; k < m; ++k) {
    size_t by;
    int bt;
    orc_vgroup_sign_bit(slot, k, &by, &bt);
    sg[k / 8] |= (uint8_t)(((signs[by] >> bt) & 1) << (k % 8));
  }
}

/* Store one slot's record (per-slot layout in rec / sg) into either storage. */
static void store_record(uint8_t *codes, uint8_t *signs, int grouped, size_t slot, int d,
                         int bits, int qjl, int m, const uint8_t *rec, const uint8_t *sg) {
  const size_t cb = (size_t)d * bits / 8, sbytes = (size_t)m / 8;
  if (!grouped) {
    memcpy(codes + slot * cb, rec, cb);
    if (qjl) memcpy(signs + slot * sbytes, sg, sbytes);
    return;
  }
  for (int c = 0; c < d; ++c) {
    const int code = get_code(rec, d, bits, c);
    for (int i = 0; i < bits; ++i) {
      size_t by;
      int bt;
      orc_vgroup_code_bit(bits, slot, c, i, &by, &bt);
      set_bit(codes, by, bt, code >> i);
    }
  }
  if (!qjl) return;
  for (int k = 0; k < m; ++k) {
    size_t by;
    int bt;
    orc_vgroup_sign_bit(slot, k, &by, &bt);
    set_bit(signs, by, bt, sg[k / 8] >> (k % 8));
  }
}

/* Forward rotation y = R x in fp32 (kinds: see the header).  WHT and
 * randomized Hadamard: sign flips (exact) then the butterflies above.  Dense:
 * y_i = fma chain over j ascending from 0 ([KPP] "Rotation invariance
 * guarantee": Q is a rotation in SO(d); the order of the chain is this
 * library's reading, the pages give none). */
static void rotate_fwd(float *y, const float *x, int d, int rotate, const void *rparam) {
  if (rotate == 3) {
    const float *Q = (const float *)rparam;
    for (int i = 0; i < d; ++i) {
      float acc = 0.0f;
      for (int j = 0; j < d; ++j) acc = fmaf(Q[(size_t)i * d + j], x[j], acc);
      y[i] = acc;
    }
    return;
  }
  for (int i = 0; i < d; ++i) y[i] = x[i];
  if (rotate == 2) {
    const uint32_t *w = (const uint32_t *)rparam;
    for (int i = 0; i < d; ++i)
      if ((w[i / 32] >> (i % 32)) & 1u) y[i] = -y[i];
  }
  if (rotate == 1 || rotate == 2) orc_wht_f32(y, d);
}

/* [DA] "Quantization schemes" / "Problem statement": rotate, scalar Lloyd-Max
 * quantise the direction, keep the norm; QJL modes add the 1-bit sketch
 * sign(S r) of the scalar residual r and its norm ([DA] Contribution 1).
 *  1. y = R x (rotate_fwd; y = x when rotate == 0)
 *  2. nu = sqrtf(pairwise sum of y_i^2); rcp = 1/nu (0 when nu == 0)
 *  3. u_i = y_i * rcp; code_i = bucketize(u_i)
 *  4. stored norm = f16(nu * s), s = fp32(1/sqrt(d)) for the Hadamard kinds
 *     (||Hx|| = sqrt(d) ||x||) else 1, so the stored value is ||x|| (||y||
 *     for the dense rotation, equal up to rounding)
 *  5. QJL: r_i = u_i - C[code_i]; rnorm = f16(sqrtf(pairwise sum r_i^2));
 *     r~ = bf16(r); sign_k = [sum_i S_ki r~_i >= 0] with the sum taken in fp64,
 *     sequentially over ascending i (every product is exact in fp64). */
void orc_encode(const float *x, int d, int rotate, const void *rparam, int bits,
                const float *centroid, const float *threshold,
                int qjl, const uint16_t *S, int m,
                uint8_t *codes, uint8_t *signs, uint16_t *norm, uint16_t *rnorm) {
  float y[4096], u[4096], r[4096];
  uint16_t rt[4096];
  int code[4096];
  const int nthr = (1 << bits) - 1;
  rotate_fwd(y, x, d, rotate, rparam);
  float nu = sqrtf(orc_sumsq_f32(y, d));
  float rcp = (nu == 0.0f) ? 0.0f : 1.0f / nu;
  float s = (rotate == 1 || rotate == 2) ? (float)(1.0 / sqrt((double)d)) : 1.0f;
  *norm = orc_f32_to_f16(nu * s);
  memset(codes, 0, (size_t)(d * bits / 8));
  for (int i = 0; i < d; ++i) {
    u[i] = y[i] * rcp;
    code[i] = orc_bucketize(u[i], threshold, nthr);
    put_code(codes, d, bits, i, code[i]);
  }
  if (!qjl) return;
  for (int i = 0; i < d; ++i) r[i] = u[i] - centroid[code[i]];
  *rnorm = orc_f32_to_f16(sqrtf(orc_sumsq_f32(r, d)));
  for (int i = 0; i < d; ++i) rt[i] = orc_f32_to_bf16(r[i]);
  memset(signs, 0, (size_t)(m / 8));
  for (int k = 0; k < m; ++k) {
    double acc = 0.0;
    for (int i = 0; i < d; ++i)
      acc += (double)orc_bf16_to_f32(S[(size_t)k * d + i]) * (double)orc_bf16_to_f32(rt[i]);
    if (acc >= 0.0) signs[k / 8] |= (uint8_t)(1u << (k % 8));
  }
}

/* Reconstruction, fp64, plain definition:
 *   x^ = n^ R^T (C[code] + sqrt(pi/2)/m * rho * S^T (2 sigma - 1))
 * with R^T = H/sqrt(d) (WHT), D H/sqrt(d) (randomized Hadamard), Q^T (dense)
 * or I (no rotation); no sketch term when qjl == 0.  sqrt(pi/2)/m is the
 * scale that makes the sketch estimate unbiased ([DA] Contribution 1). */
void orc_decode(const uint8_t *codes, const uint8_t *signs, uint16_t norm, uint16_t rnorm,
                int d, int rotate, const void *rparam, int bits, const float *centroid,
                int qjl, const uint16_t *S, int m, double *xhat) {
  double t[4096];
  for (int i = 0; i < d; ++i) t[i] = (double)centroid[get_code(codes, d, bits, i)];
  if (qjl) {
    double coef = sqrt(M_PI / 2.0) / m * orc_f16_to_f64(rnorm);
    for (int i = 0; i < d; ++i) {
      double acc = 0.0;
      for (int k = 0; k < m; ++k) {
        double sg = ((signs[k / 8] >> (k % 8)) & 1) ? 1.0 : -1.0;
        acc += (double)orc_bf16_to_f32(S[(size_t)k * d + i]) * sg;
      }
      t[i] += coef * acc;
    }
  }
  double nh = orc_f16_to_f64(norm);
  if (!rotate) {
    for (int i = 0; i < d; ++i) xhat[i] = nh * t[i];
    return;
  }
  if (rotate == 3) {
    const float *Q = (const float *)rparam;
    for (int i = 0; i < d; ++i) {
      double acc = 0.0;
      for (int j = 0; j < d; ++j) acc += (double)Q[(size_t)j * d + i] * t[j];
      xhat[i] = nh * acc;
    }
    return;
  }
  double sc = nh / sqrt((double)d);
  for (int i = 0; i < d; ++i) {
    double acc = 0.0;
    for (int j = 0; j < d; ++j) acc += (__builtin_popcount((unsigned)(i & j)) & 1) ? -t[j] : t[j];
    xhat[i] = sc * acc;
    if (rotate == 2 && ((((const uint32_t *)rparam)[i / 32] >> (i % 32)) & 1u)) xhat[i] = -xhat[i];
  }
}

/* ------------------------------------------------------------------------ */
/* Batched drivers (independent (b,h) units spread over threads)             */
/* ------------------------------------------------------------------------ */

typedef struct {
  void (*fn)(void *ctx, int unit);
  void *ctx;
  int n;
  int next;
  pthread_mutex_t mu;
} pool_t;

static void *pool_worker(void *arg) {
  pool_t *p = (pool_t *)arg;
  for (;;) {
    pthread_mutex_lock(&p->mu);
    int u = p->next++;
    pthread_mutex_unlock(&p->mu);
    if (u >= p->n) return NULL;
    p->fn(p->ctx, u);
  }
}

static void run_units(void (*fn)(void *, int), void *ctx, int n, int nthreads) {
  pool_t p;
  p.fn = fn; p.ctx = ctx; p.n = n; p.next = 0;
  pthread_mutex_init(&p.mu, NULL);
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (nthreads == 1 || n <= 1) {
    pool_worker(&p);
  } else {
    pthread_t th[256];
    for (int i = 0; i < nthreads; ++i) pthread_create(&th[i], NULL, pool_worker, &p);
    for (int i = 0; i < nthreads; ++i) pthread_join(th[i], NULL);
  }
  pthread_mutex_destroy(&p.mu);
}

typedef struct {
  const void *src; int dtype, H, T, d; long long sb, sh, st; int t0, cap;
  int rotate; const void *rparam; int bits; const float *C, *Th; int qjl; const uint16_t *S; int m;
  uint8_t *codes, *signs; uint16_t *norm, *rnorm; int grouped;
} qctx_t;

static void quantize_unit(void *vc, int unit) {
  qctx_t *c = (qctx_t *)vc;
  int b = unit / c->H, h = unit % c->H;
  float x[4096];
  uint8_t rec[2048], sg[512];
  for (int t = 0; t < c->T; ++t) {
    long long off = b * c->sb + h * c->sh + t * c->st;
    for (int i = 0; i < c->d; ++i)
      x[i] = c->dtype == 0 ? ((const float *)c->src)[off + i]
                           : orc_bf16_to_f32(((const uint16_t *)c->src)[off + i]);
    size_t slot = ((size_t)unit * c->cap) + (size_t)(c->t0 + t);
    orc_encode(x, c->d, c->rotate, c->rparam, c->bits, c->C, c->Th, c->qjl, c->S, c->m, rec,
               c->qjl ? sg : NULL, c->norm + slot, c->qjl ? c->rnorm + slot : NULL);
    store_record(c->codes, c->signs, c->grouped, slot, c->d, c->bits, c->qjl, c->m, rec, sg);
  }
}

void orc_quantize_cache(const void *src, int dtype, int B, int H, int T, int d,
                        long long sb, long long sh, long long st, int t0, int cap,
                        int rotate, const void *rparam, int bits, const float *centroid,
                        const float *threshold, int qjl, const uint16_t *S, int m,
                        uint8_t *codes, uint8_t *signs, uint16_t *norm, uint16_t *rnorm,
                        int grouped, int nthreads) {
  qctx_t c = {src, dtype, H, T, d, sb, sh, st, t0, cap, rotate, rparam, bits, centroid, threshold,
              qjl, S, m, codes, signs, norm, rnorm, grouped};
  run_units(quantize_unit, &c, B * H, nthreads);
}

typedef struct {
  const uint8_t *codes, *signs; const uint16_t *norm, *rnorm;
  int H, cap, t0, T, d, rotate; const void *rparam; int bits; const float *C; int qjl;
  const uint16_t *S; int m; int grouped;
  double *out;
} dctx_t;

static void dequantize_unit(void *vc, int unit) {
  dctx_t *c = (dctx_t *)vc;
  uint8_t rec[2048], sg[512];
  for (int t = 0; t < c->T; ++t) {
    size_t slot = (size_t)unit * c->cap + (size_t)(c->t0 + t);
    orc_load_record(c->codes, c->signs, c->grouped, slot, c->d, c->bits, c->qjl, c->m, rec, sg);
    orc_decode(rec, c->qjl ? sg : NULL, c->norm[slot], c->qjl ? c->rnorm[slot] : 0, c->d,
               c->rotate, c->rparam, c->bits, c->C, c->qjl, c->S, c->m,
               c->out + ((size_t)unit * c->T + t) * c->d);
  }
}

void orc_dequantize_cache(const uint8_t *codes, const uint8_t *signs,
                          const uint16_t *norm, const uint16_t *rnorm,
                          int B, int H, int cap, int t0, int T, int d,
                          int rotate, const void *rparam, int bits, const float *centroid,
                          int qjl, const uint16_t *S, int m, int grouped, double *out,
                          int nthreads) {
  dctx_t c = {codes, signs, norm, rnorm, H, cap, t0, T, d, rotate, rparam, bits, centroid, qjl,
              S, m, grouped, out};
  run_units(dequantize_unit, &c, B * H, nthreads);
}

/* ------------------------------------------------------------------------ */
/* Attention over the reconstructed cache                                    */
/* [HQ] 2.1: score s_j = q.k_j / sqrt(d), softmax over the cached tokens;    */
/* [HQ] 2.2: output = sum_j p_j v_j.  [GEO] "Why the KV cache is the pain    */
/* point": one decode step reads every cached token.                         */
/* ------------------------------------------------------------------------ */

typedef struct {
  const orc_side *k, *v; const uint16_t *S; int m;
  int Hkv, cap, d; const void *q; int q_dtype; int Hq; int n_ctx;
  double *out; const int *units;
} actx_t;

static void side_decode(const orc_side *sd, size_t slot, int d, const uint16_t *S, int m,
                        double *x) {
  uint8_t rec[2048], sg[512];
  orc_load_record(sd->codes, sd->signs, sd->grouped, slot, d, sd->bits, sd->qjl, m, rec, sg);
  orc_decode(rec, sd->qjl ? sg : NULL, sd->norm[slot], sd->qjl ? sd->rnorm[slot] : 0, d,
             sd->rotate, sd->rparam, sd->bits, sd->centroid, sd->qjl, S, m, x);
}

/* Plain attention over explicit fp64 keys and values (n tokens, row-major):
 * s_j = q.K_j / sqrt(d); two passes: max, then p_j = exp(s_j - max),
 * out = sum_j p_j V_j / sum_j p_j. */
void orc_attention_dense(const double *q, const double *K, const double *V, int n, int d,
                         double *out) {
  double *s = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  double smax = -INFINITY;
  for (int j = 0; j < n; ++j) {
    double acc = 0.0;
    for (int i = 0; i < d; ++i) acc += q[i] * K[(size_t)j * d + i];
    s[j] = acc / sqrt((double)d);
    if (s[j] > smax) smax = s[j];
  }
  double L = 0.0;
  for (int i = 0; i < d; ++i) out[i] = 0.0;
  for (int j = 0; j < n; ++j) {
    double p = exp(s[j] - smax);
    L += p;
    for (int i = 0; i < d; ++i) out[i] += p * V[(size_t)j * d + i];
  }
  for (int i = 0; i < d; ++i) out[i] /= L;
  free(s);
}

static void attention_unit(void *vc, int idx) {
  actx_t *c = (actx_t *)vc;
  int row = c->units ? c->units[idx] : idx;      /* row = b*Hq + hq */
  int b = row / c->Hq, hq = row % c->Hq;
  int G = c->Hq / c->Hkv, hkv = hq / G;          /* G query heads share one KV head */
  int d = c->d, n = c->n_ctx;
  double q[4096];
  for (int i = 0; i < d; ++i) {
    size_t off = (size_t)row * d + i;
    q[i] = c->q_dtype == 0 ? (double)((const float *)c->q)[off]
                           : (double)orc_bf16_to_f32(((const uint16_t *)c->q)[off]);
  }
  double *K = (double *)malloc(sizeof(double) * (size_t)n * d);
  double *V = (double *)malloc(sizeof(double) * (size_t)n * d);
  size_t base = ((size_t)b * c->Hkv + hkv) * c->cap;
  for (int j = 0; j < n; ++j) {
    side_decode(c->k, base + j, d, c->S, c->m, K + (size_t)j * d);
    side_decode(c->v, base + j, d, c->S, c->m, V + (size_t)j * d);
  }
  orc_attention_dense(q, K, V, n, d, c->out + (size_t)row * d);
  free(K);
  free(V);
}

void orc_attention(const orc_side *k, const orc_side *v, const uint16_t *S, int m,
                   int B, int Hkv, int cap, int d, const void *q, int q_dtype, int Hq,
                   int n_ctx, double *out, const int *unit_list, int n_units, int nthreads) {
  actx_t c = {k, v, S, m, Hkv, cap, d, q, q_dtype, Hq, n_ctx, out, unit_list};
  int n = unit_list ? n_units : B * Hq;
  run_units(attention_unit, &c, n, nthreads);
}
