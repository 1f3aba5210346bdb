/*
 * kvq_oracle.h -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, sequential CPU reference of the KQV KV-cache codec and of
 * attention over the reconstructed cache.  Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may load it.  It shares no code,
 * header, table or constant generator with the product library (libkvq).
 *
 * Sources (web pages; cited by title and section):
 *  [DA]  "Statistical Inference and Quality Measures of KV Cache
 *        Quantisations Inspired by TurboQuant" (P. D'Alberto), gist.science
 *        technical summary: sections "Theoretical framework" (sphere
 *        marginal), "Quantization schemes" (KV / KQV / QKQV), "Contribution 1"
 *        (QJL sketch, its unbiasedness and variance).
 *  [HQ]  "HeadQ" explanation, gist.science: section 2.1 (score q.k/sqrt(d),
 *        softmax-null key shift), section 2.2 (value readout is linear).
 *  [GEO] "Your KV cache is not a bit problem but a geometry problem":
 *        "Why the KV cache is the pain point" (decode reads the whole cache
 *        per generated token), "Systems tax" (per-token append).
 *  [KPP] "KVQuant++" forum thread (zingnex.cn): "Codebook design: the true
 *        sphere marginal" f(t) ~ (1-t^2)^((d-3)/2), "Fast codebook lookup"
 *        (bucketize), "Entropy coding" (QR or Hadamard random rotation),
 *        "Rotation invariance guarantee" (QR rotation in SO(d)),
 *        "Rate-distortion performance" (MSE bound).
 *
 * Readings where the pages are silent are listed in the repository's design
 * notes; each function below states the one it implements.
 */
#ifndef KVQ_ORACLE_H
#define KVQ_ORACLE_H
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Lloyd-Max codebook on the sphere-marginal density ([KPP] codebook design,
 * [DA] theoretical framework).  Writes K = 2^bits fp32 centroids (ascending),
 * K-1 fp32 thresholds (midpoints), and the K/2 positive fp64 centroids.
 * Returns the number of Lloyd iterations, or -1 on bad arguments. */
int orc_codebook(int d, int bits, double *pos_c64, float *centroid, float *threshold);

/* Number formats (IEEE 754 binary16 / bfloat16, round to nearest even). */
uint16_t orc_f32_to_f16(float x);
uint16_t orc_f32_to_bf16(float x);
float orc_bf16_to_f32(uint16_t h);
double orc_f16_to_f64(uint16_t h);

/* fp32 in-place Sylvester Walsh-Hadamard butterfly (unnormalised). */
void orc_wht_f32(float *y, int d);
/* fp32 adjacent-pair pairwise sum of squares. */
float orc_sumsq_f32(const float *y, int d);
/* Bucketize: number of thresholds strictly below u. */
int orc_bucketize(float u, const float *threshold, int nthr);

/* Rotation kinds ("rotate" arguments below):
 *   0 none; 1 WHT y = H x; 2 randomized Hadamard y = H (D x), rparam = sign
 *   words (uint32, bit i set: x_i negated); 3 dense y = Q x, rparam = Q
 *   (fp32, d x d, row-major). */

/* Encode one d-vector (fp32).  rotate, rparam: rotation (above).  bits: code
 * width.  qjl: also write m sign bits of S.bf16(r) and the fp16 residual
 * norm.  S: m x d bf16 bit patterns, row-major.  Packed layout: see the .c
 * file. */
void orc_encode(const float *x, int d, int rotate, const void *rparam, int bits,
                const float *centroid, const float *threshold,
                int qjl, const uint16_t *S, int m,
                uint8_t *codes, uint8_t *signs, uint16_t *norm, uint16_t *rnorm);

/* Reconstruct one vector in fp64 from its record. */
void orc_decode(const uint8_t *codes, const uint8_t *signs, uint16_t norm, uint16_t rnorm,
                int d, int rotate, const void *rparam, int bits, const float *centroid,
                int qjl, const uint16_t *S, int m, double *xhat);

/* Storage of a cache side's records.  grouped == 0: slot s holds its own
 * record at bytes [s R, s R + R) (R = record bytes) and its sign record at
 * [s m/8, (s+1) m/8).  grouped == 1 (value side at d = 128, cap a multiple of
 * 16): the codes and sign bits of neighbouring slots share bytes; the bit
 * positions are given by orc_vgroup_code_bit / orc_vgroup_sign_bit. */
void orc_vgroup_code_bit(int bits, size_t slot, int c, int i, size_t *byte, int *bit);
void orc_vgroup_sign_bit(size_t slot, int k, size_t *byte, int *bit);

/* Record of one slot in the per-slot layout, from either storage. */
void orc_load_record(const uint8_t *codes, const uint8_t *signs, int grouped, size_t slot,
                     int d, int bits, int qjl, int m, uint8_t *rec, uint8_t *sg);

/* Quantize-on-write of T tokens into a cache laid out [B][H][cap][record].
 * src: fp32 (dtype 0) or bf16 bit patterns (dtype 1), element (b,h,t,i) at
 * b*sb + h*sh + t*st + i (in elements).  Tokens go to cache slots t0..t0+T-1.
 * signs / rnorm may be NULL when qjl == 0.  nthreads >= 1. */
void orc_quantize_cache(const void *src, int dtype, int B, int H, int T, int d,
                        long long sb, long long sh, long long st, int t0, int cap,
                        int rotate, const void *rparam, int bits, const float *centroid,
                        const float *threshold,
                        int qjl, const uint16_t *S, int m,
                        uint8_t *codes, uint8_t *signs, uint16_t *norm, uint16_t *rnorm,
                        int grouped, int nthreads);

/* Dequantize cache slots t0..t0+T-1 of every (b,h) into out [B][H][T][d] fp64. */
void orc_dequantize_cache(const uint8_t *codes, const uint8_t *signs,
                          const uint16_t *norm, const uint16_t *rnorm,
                          int B, int H, int cap, int t0, int T, int d,
                          int rotate, const void *rparam, int bits, const float *centroid,
                          int qjl, const uint16_t *S, int m, int grouped, double *out,
                          int nthreads);

/* Plain attention over explicit fp64 keys K [n][d] and values V [n][d]. */
void orc_attention_dense(const double *q, const double *K, const double *V, int n, int d,
                         double *out);

/* One side of a cache (K or V), as seen by orc_attention. */
typedef struct {
  const uint8_t *codes, *signs;
  const uint16_t *norm, *rnorm;
  int rotate, bits, qjl;
  const float *centroid;
  const void *rparam;
  int grouped;
} orc_side;

/* Decode attention over the reconstructed cache, fp64, plain definition:
 * o[b][hq] = sum_j softmax_j(q.k^_j / sqrt(d)) v^_j over the first n_ctx slots,
 * KV head of query head hq is hq / (Hq/Hkv).  q: fp32 (0) or bf16 (1),
 * [B][Hq][d] contiguous.  out: [B][Hq][d] fp64.  If unit_list is non-NULL only
 * the listed (b*Hq + hq) rows are computed. */
void orc_attention(const orc_side *k, const orc_side *v, const uint16_t *S, int m,
                   int B, int Hkv, int cap, int d, const void *q, int q_dtype, int Hq,
                   int n_ctx, double *out, const int *unit_list, int n_units, int nthreads);

#ifdef __cplusplus
}
#endif
#endif
