/*
 * kvq.h -- C ABI of libkvq: KQV KV-cache quantisation and decode attention
 * over the compressed cache, for AMD Instinct MI355X (gfx950).
 *
 * The method (sources are web pages, cited by title and section):
 *  - D'Alberto, "Statistical Inference and Quality Measures of KV Cache
 *    Quantisations Inspired by TurboQuant" (gist.science technical summary),
 *    "Quantization schemes": three schemes at a budget of n bits/coordinate
 *      KV   : scalar Lloyd-Max on K and V, no rotation, no sketch
 *      KQV  : Walsh-Hadamard transform (WHT) on both; K n-bit scalar;
 *             V (n-1)-bit scalar + 1-bit QJL sketch of the residual
 *      QKQV : WHT on both; K and V each (n-1)-bit scalar + 1-bit QJL sketch
 *    "Theoretical framework": a coordinate of a uniform point on S^{d-1}
 *    follows Beta((d-1)/2,(d-1)/2) on (1+t)/2; "Contribution 1": the sign
 *    sketch is unbiased with variance (pi/2)||r||^2/d.
 *  - "KVQuant++" forum thread (zingnex.cn): "Codebook design" -- the codebook
 *    is fitted to f(t) ~ (1-t^2)^((d-3)/2); "Fast codebook lookup" --
 *    bucketize against sorted thresholds; "Deployment and usage" --
 *    construct(head_dim, num_bits) / compress / decompress.
 *  - "Your KV cache is not a bit problem but a geometry problem": "Why the
 *    KV cache is the pain point" -- every generated token reads the whole
 *    cache; "Systems tax" -- per-token quantisation appends along the token
 *    axis and nothing else moves.
 *  - "HeadQ" explanation (gist.science), 2.1 score q.k/sqrt(d) and softmax;
 *    2.2 the value readout is linear in the values.
 *
 * Conventions for every entry point
 *  - Returns kvq_status; never throws; never synchronises a stream.
 *  - Device pointers are caller-owned (allocate with torch / hipMalloc).  The
 *    library allocates no device memory and keeps no pointer after return;
 *    its only device storage is the fixed scratch array that
 *    kvq_decode_attention_noalloc uses.
 *  - All validation happens on the host before any launch: a call that fails
 *    validation launches nothing.  A failed launch returns KVQ_ERR_HIP.
 *    Asynchronous device faults surface at the caller's next synchronisation.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *  - Entry points are reentrant; calls that write the same cache region
 *    concurrently on different streams race.
 *  - Inputs must be finite; NaN/Inf inputs give unspecified codes.  A norm
 *    that overflows binary16 is stored as +Inf.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVQ_OK = 0,
  KVQ_ERR_NULL = 1,       /* a required pointer is NULL */
  KVQ_ERR_ALIGN = 2,      /* a pointer or stride breaks the 16-byte alignment rule */
  KVQ_ERR_DIM = 3,        /* head dimension not in {8, 16, 32, 64, 128, 256} */
  KVQ_ERR_BITS = 4,       /* bit width out of range for the scheme */
  KVQ_ERR_SCHEME = 5,     /* unknown scheme */
  KVQ_ERR_CAPACITY = 6,   /* t0 + T or n_ctx exceeds the cache capacity */
  KVQ_ERR_WORKSPACE = 7,  /* workspace missing or too small */
  KVQ_ERR_DTYPE = 8,      /* unknown element type */
  KVQ_ERR_HEADS = 9,      /* q_heads not a supported multiple of kv_heads */
  KVQ_ERR_RANGE = 10,     /* a size is zero/negative or a count overflows */
  KVQ_ERR_HIP = 11        /* the HIP runtime reported an error on launch */
} kvq_status;

typedef enum { KVQ_SCHEME_KV = 0, KVQ_SCHEME_KQV = 1, KVQ_SCHEME_QKQV = 2 } kvq_scheme;
typedef enum { KVQ_F32 = 0, KVQ_BF16 = 1 } kvq_dtype;

/* Rotation of the rotated schemes (KQV, QKQV); the KV scheme has none.
 * "KVQuant++" thread, "Entropy coding" (a random QR or Hadamard rotation makes
 * the coordinates near-Gaussian), "Rotation invariance guarantee" (the QR
 * rotation is kept in SO(d), determinant +1) and "Rate-distortion
 * performance" (either rotation stays under the MSE bound).
 *   KVQ_ROT_WHT : y = H x, H the Sylvester Walsh-Hadamard matrix (default)
 *   KVQ_ROT_RHT : y = H D x, D = diag(+-1) (randomized Hadamard)
 *   KVQ_ROT_QR  : y = Q x, Q in SO(d), fp32 */
typedef enum { KVQ_ROT_WHT = 0, KVQ_ROT_RHT = 1, KVQ_ROT_QR = 2 } kvq_rotation;

/* Scalar codebook for one (d, bits): 2^bits ascending fp32 centroids and the
 * 2^bits - 1 midpoint thresholds (unused entries are zero).  Host POD; it is
 * copied by value into kernel arguments. */
typedef struct {
  int32_t d, bits;
  float centroid[16];
  float threshold[15];
} kvq_codebook;

/* Lloyd-Max codebook on the sphere-marginal density f(t) ~ (1-t^2)^((d-3)/2)
 * over [-1, 1] ("KVQuant++" thread, "Codebook design"; D'Alberto summary,
 * "Theoretical framework"; Lloyd-Max: "Quantization schemes").  Host only.
 * Iterated in fp64 to its fixed point (unique: the density is log-concave),
 * then rounded once to fp32; the table is exactly symmetric and the middle
 * threshold is 0.  d in [3, 4096], bits in [1, 4].
 * Errors: KVQ_ERR_NULL (out NULL), KVQ_ERR_DIM, KVQ_ERR_BITS. */
kvq_status kvq_codebook_init(int d, int bits, kvq_codebook *out);

/* Gaussian sketch S (m x d, row-major, bfloat16 bit patterns) for the 1-bit
 * QJL residual sketch (D'Alberto summary, "Problem statement" and
 * "Contribution 1").  Host only; fills a caller-owned host buffer of m*d
 * uint16.  Generator: SplitMix64 counter stream from `seed`, 53-bit uniforms,
 * Box-Muller in fp64, rounded to fp32 then to bf16 (nearest even).
 * Errors: KVQ_ERR_NULL, KVQ_ERR_RANGE (m or d < 1). */
kvq_status kvq_sketch_init(uint64_t seed, int m, int d, uint16_t *S_bf16_host);

/* A compressed cache: caller-owned device buffers plus codec parameters.
 * Buffer shapes (record per (batch b, KV head h, slot t), slot-major):
 *   k_codes [B][Hkv][cap][d*kb/8]  k_norm  [B][Hkv][cap] binary16
 *   k_signs [B][Hkv][cap][m/8]     k_rnorm [B][Hkv][cap] binary16  (K sketch only)
 *   v_codes [B][Hkv][cap][d*vb/8]  v_norm  [B][Hkv][cap] binary16
 *   v_signs [B][Hkv][cap][m/8]     v_rnorm [B][Hkv][cap] binary16  (V sketch only)
 * kb, vb = per-side code widths of the scheme (see kvq_cache_init); m = d.
 * Code layout inside a record: widths 1, 2, 4 -- code i at bit offset i*w,
 * little-endian bytes; width 3 -- a 2-bit plane of the low bits (d/4 bytes)
 * followed by a 1-bit plane of the high bits (d/8 bytes).  Sign bit k at byte
 * k/8, bit k%8; bit = 1 means the sketch row is >= 0.  The stored norm is
 * ||x|| (||y|| for KVQ_ROT_QR); the residual norm is ||r|| of the rotated unit
 * direction.  Pointers not used by the scheme must be NULL.  All pointers 16-B
 * aligned.  The rotation fields are set by kvq_cache_set_rotation.
 * At d = 128 the value side is stored in token groups instead (same buffer
 * sizes; cap must be a multiple of 16): the codes of slots 4q .. 4q+3 share
 * bytes [4q R, 4q R + 4R) (R = d*vb/8), piece n (coordinates 8n .. 8n+7) at
 * byte 4 vb n, holding for coordinate 8n+j and slot 4q+r:
 *   vb 4: byte 2j + r/2, bits 4 (r%2) .. +3
 *   vb 3: the 6-bit field u = 2j + r/2 = code(4q + 2(r/2)) | code(+1) << 3;
 *         u < 12: bits 2..7 of byte u; u >= 12: its bit pairs (0,1), (2,3),
 *         (4,5) in bits 0, 1 of bytes u-12, u-8, u-4
 *   vb 2: byte j, bits 2r .. 2r+1;   vb 1: byte j/2, bit 4 (j%2) + r
 * and the sign bits of slots 8o .. 8o+7 share bytes [128 o, 128 o + 128):
 * bit e of byte 128 o + k = sign of slot 8o + e at sketch row k. */
typedef struct {
  int32_t scheme, n_bits, d, m, batch, kv_heads, capacity;
  int32_t k_bits, v_bits, k_qjl, v_qjl, rotate;  /* derived by kvq_cache_init */
  kvq_codebook cb_k, cb_v;                       /* host copies, by value */
  const uint16_t *S;                             /* device, m*d bf16, NULL if no sketch */
  uint8_t *k_codes, *k_signs, *v_codes, *v_signs;
  uint16_t *k_norm, *k_rnorm, *v_norm, *v_rnorm;
  int32_t rot_kind;                              /* kvq_rotation (rotated schemes) */
  uint32_t rot_signs[8];                         /* RHT: bit i%32 of word i/32 = negate x_i */
  const float *rot_Q;                            /* QR: device, d*d fp32 row-major, else NULL */
} kvq_cache;

/* Fill the scalar fields and codebooks of `c` for a scheme at n_bits per
 * coordinate (KV: n in 1..4; KQV, QKQV: n in 2..4); leaves the pointers
 * NULL and the rotation at KVQ_ROT_WHT.  Errors: KVQ_ERR_NULL,
 * KVQ_ERR_SCHEME, KVQ_ERR_BITS, KVQ_ERR_DIM, KVQ_ERR_RANGE (also: d = 128
 * with a capacity that is not a multiple of 16). */
kvq_status kvq_cache_init(kvq_cache *c, int scheme, int n_bits, int d, int batch,
                          int kv_heads, int capacity);

/* Choose the rotation of a rotated-scheme cache (before anything is written
 * to it; codes written under one rotation do not decode under another).
 * kind KVQ_ROT_WHT: signs and Q ignored.  KVQ_ROT_RHT: signs = host array of
 * d bits (d/32 words, at least one; bits at and beyond d must be 0).
 * KVQ_ROT_QR: Q = device pointer to d*d fp32 (row-major, 16-B aligned),
 * which must stay valid while the cache is used; its orthogonality is the
 * caller's (see kvq_rotation_qr).
 * Errors: KVQ_ERR_NULL, KVQ_ERR_SCHEME (KV scheme, or unknown kind),
 * KVQ_ERR_ALIGN, KVQ_ERR_RANGE (sign bits beyond d). */
kvq_status kvq_cache_set_rotation(kvq_cache *c, int kind, const uint32_t *signs,
                                  const float *Q_device);

/* Random diagonal of KVQ_ROT_RHT: bit i = SplitMix64 stream from `seed`, one
 * draw per coordinate, its top bit.  Host; out = 8 words (bits at and beyond
 * d are 0).  Errors: KVQ_ERR_NULL, KVQ_ERR_DIM (d not a supported head
 * dimension). */
kvq_status kvq_rotation_signs(uint64_t seed, int d, uint32_t out[8]);

/* Random rotation of KVQ_ROT_QR, Haar-distributed on SO(d) ("Rotation
 * invariance guarantee"): a d x d standard Gaussian matrix (SplitMix64,
 * Box-Muller, fp64) factored by Householder QR in fp64; Q is scaled column by
 * column by sign(R_kk) (Haar on O(d)) and its first column is negated when
 * det Q = -1; the result is rounded to fp32, row-major.  Host; Q_host holds
 * d*d floats.  Errors: KVQ_ERR_NULL, KVQ_ERR_DIM. */
kvq_status kvq_rotation_qr(uint64_t seed, int d, float *Q_host);

/* Byte sizes of the eight buffers, in the order k_codes, k_signs, k_norm,
 * k_rnorm, v_codes, v_signs, v_norm, v_rnorm (0 = buffer unused).
 * Errors: as kvq_cache_init. */
kvq_status kvq_cache_layout(int scheme, int n_bits, int d, int batch, int kv_heads,
                            int capacity, size_t bytes_out[8]);

/* Quantize-on-write of T new tokens of K (resp. V) into slots t0..t0+T-1 of
 * every (b, h) ("Systems tax": per-token append along the token axis).
 * src element (b, h, t, i) is at src + (b*stride_b + h*stride_h + t*stride_t
 * + i) elements of `dtype` (fp32 or bf16); strides are in elements, rows must
 * be 16-B aligned.  Per vector: y = R x (rotated schemes: the cache's
 * rotation, see kvq_rotation; y = x for KV), nu = ||y||,
 * u = y/nu, code_i = #{thresholds < u_i} (bucketize), norm = ||x|| in fp16;
 * sketch sides add r = u - C[code], ||r|| in fp16 and sign(S bf16(r)).
 * fp32 arithmetic in a fixed order (ascending butterfly stages, adjacent-pair
 * sums, correctly rounded sqrt and division, no contraction) so codes and
 * sign bits are reproducible bit for bit.
 * Errors: KVQ_ERR_NULL, KVQ_ERR_ALIGN, KVQ_ERR_DTYPE, KVQ_ERR_CAPACITY,
 * KVQ_ERR_RANGE, KVQ_ERR_HIP. */
kvq_status kvq_quantize_k(const kvq_cache *c, const void *src, int dtype, int t0, int T,
                          int64_t stride_b, int64_t stride_h, int64_t stride_t, void *stream);
kvq_status kvq_quantize_v(const kvq_cache *c, const void *src, int dtype, int t0, int T,
                          int64_t stride_b, int64_t stride_h, int64_t stride_t, void *stream);

/* Reconstruct slots t0..t0+T-1 of one side (which: 0 = K, 1 = V) into out
 * [B][Hkv][T][d] fp32 (device):
 *   x^ = ||x|| R^T (C[code] + sqrt(pi/2)/m ||r|| S^T (2 sigma - 1))
 * with R^T = H/sqrt(d) (WHT), D H/sqrt(d) (randomized Hadamard), Q^T (dense),
 * I (KV scheme); no sketch term for scalar-only sides.
 * ("KVQuant++" thread, "Deployment and usage": decompress.)
 * Errors: KVQ_ERR_NULL, KVQ_ERR_ALIGN, KVQ_ERR_CAPACITY, KVQ_ERR_RANGE, KVQ_ERR_HIP. */
kvq_status kvq_dequantize(const kvq_cache *c, int which, int t0, int T, float *out, void *stream);

/* One decode step over the first n_ctx slots ("Why the KV cache is the pain
 * point": every generated token reads the whole cache):
 *   out[b][hq] = sum_j softmax_j(q[b][hq] . k^_j / sqrt(d)) v^_j
 * with KV head hq / (q_heads / kv_heads) (grouped-query attention; q_heads a
 * multiple of kv_heads with ratio 1, 2, 4 or a multiple of 4), no mask.
 * q: [B][q_heads][d] fp32 or bf16 (device, contiguous); out: [B][q_heads][d]
 * fp32 (device).  splits: number of token splits per (b, KV head); 0 picks
 * one for the GPU.  A split holds at most 1280 tokens when four or more query
 * heads share a KV head (2560 for two, 5120 for one): fewer splits than that
 * allows, or more than 8192, give KVQ_ERR_RANGE.  Each split covers
 * ceil(n_ctx / splits) tokens rounded up to a multiple of 64, so trailing
 * splits may be empty.  workspace: device scratch of kvq_decode_workspace
 * bytes (contents on entry do not matter).  Three kernels run on the stream:
 * query preparation, the split scan, the split merge.
 * Keys are scored in rotated space (q is rotated once instead of each key);
 * values and the V sketch term are accumulated in rotated and sketch space and
 * mapped back with one S^T product and one WHT per query head.
 * Errors: KVQ_ERR_NULL, KVQ_ERR_ALIGN, KVQ_ERR_DTYPE, KVQ_ERR_HEADS,
 * KVQ_ERR_CAPACITY, KVQ_ERR_RANGE, KVQ_ERR_WORKSPACE, KVQ_ERR_HIP. */
kvq_status kvq_decode_attention(const kvq_cache *c, const void *q, int q_dtype, int q_heads,
                                int n_ctx, int splits, float *out, void *workspace,
                                size_t workspace_bytes, void *stream);

/* One decode step over compressed slots t_begin..t_end-1 plus n_win tokens
 * the caller keeps at full precision ("Your KV cache is not a bit problem but
 * a geometry problem", sections "Systems tax" and "What we should do": a
 * window of the most recent tokens stays unquantized; "Frontier": attention
 * sink tokens likewise).  The softmax runs over the union of both sets:
 *   out[b][hq] = sum_{j in cache} p_j v^_j + sum_{j in window} p_j v_j,
 *   p = softmax over all (q . k / sqrt(d)), exact k, v for window tokens.
 * wk, wv: [B][kv_heads][n_win][d] of w_dtype (fp32 or bf16), device,
 * contiguous, 16-B aligned; the window tokens' order does not matter.
 * 0 <= t_begin <= t_end <= capacity, 0 <= n_win <= 4096, and at least one
 * token in all (t_end - t_begin + n_win >= 1); wk and wv may be null when
 * n_win == 0.  Other arguments as kvq_decode_attention; size the workspace
 * with kvq_decode_workspace(c, q_heads, t_end - t_begin, splits, ...).
 * Errors: as kvq_decode_attention. */
kvq_status kvq_decode_attention_window(const kvq_cache *c, const void *q, int q_dtype,
                                       int q_heads, int t_begin, int t_end, const void *wk,
                                       const void *wv, int w_dtype, int n_win, int splits,
                                       float *out, void *workspace, size_t workspace_bytes,
                                       void *stream);

/* kvq_decode_attention for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the workspace comes from a fixed device array inside the
 * library, KVQ_NOALLOC_SCRATCH_BYTES bytes on each GPU it runs on (held until
 * the process ends; its address is looked up once per device on the first
 * call).  The call allocates nothing; the caller still passes q and out.
 * Arguments and results as kvq_decode_attention, on the current device (the
 * stream must belong to it).  Nothing in the array needs to start at zero.
 * Every call on one GPU shares that GPU's array: calls that overlap on one GPU
 * (different streams, or host threads) race and give undefined results.
 * Errors: as kvq_decode_attention; KVQ_ERR_WORKSPACE when the call needs more
 * than KVQ_NOALLOC_SCRATCH_BYTES of workspace (kvq_decode_workspace tells);
 * KVQ_ERR_HIP when the array's device address cannot be obtained. */
#define KVQ_NOALLOC_SCRATCH_BYTES (64u << 20)
kvq_status kvq_decode_attention_noalloc(const kvq_cache *c, const void *q, int q_dtype,
                                        int q_heads, int n_ctx, int splits, float *out,
                                        void *stream);

/* Decode stages for kvq_decode_attention_stages (bit mask). */
enum {
  KVQ_STAGE_PREP = 1,   /* query preparation q' = R q (and S q'); window partial */
  KVQ_STAGE_SCAN = 2,   /* split scan over the compressed slots -> split partials */
  KVQ_STAGE_MERGE = 4,  /* merge of the split partials -> out */
  KVQ_STAGE_ALL = 7
};

/* kvq_decode_attention run stage by stage: the same arguments plus `stages`,
 * a non-empty mask of KVQ_STAGE_*; only the selected stages are launched, in
 * the order prep, scan, merge.  The stages communicate through the workspace,
 * so calls with PREP, then SCAN, then MERGE on one stream (same arguments and
 * workspace) give exactly the result of one kvq_decode_attention call, which
 * equals stages = KVQ_STAGE_ALL.  For callers that time or overlap the stages
 * separately.  At d = 128 with a Hadamard rotation or none and no key sketch
 * the scan prepares q' in its own prologue: there PREP launches only the
 * window kernel (nothing without a window) and SCAN reads q itself, so q must
 * stay unchanged until SCAN has run.
 * Errors: as kvq_decode_attention; KVQ_ERR_RANGE for a bad mask. */
kvq_status kvq_decode_attention_stages(const kvq_cache *c, const void *q, int q_dtype,
                                       int q_heads, int n_ctx, int splits, int stages, float *out,
                                       void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes kvq_decode_attention (or kvq_decode_attention_window over
 * n_ctx compressed slots) needs for these arguments; n_ctx may be 0 here. */
kvq_status kvq_decode_workspace(const kvq_cache *c, int q_heads, int n_ctx, int splits,
                                size_t *bytes);

/* The split count kvq_decode_attention uses when splits == 0.  At d = 128 it
 * follows the current device's compute-unit count (one round of resident scan
 * blocks; 256 CUs assumed where no device answers), so a workspace sized with
 * splits == 0 on one device may be too small on a larger one (the call then
 * returns KVQ_ERR_WORKSPACE).  0 for invalid arguments. */
int kvq_decode_auto_splits(const kvq_cache *c, int q_heads, int n_ctx);

/* Multi-query (chunked-prefill) attention over the compressed cache ("Your
 * KV cache is not a bit problem but a geometry problem", "Systems tax": a
 * prompt chunk is quantised into the cache along the token axis, then its
 * queries attend over the cache):
 *   out[b][i][hq] = sum_{t < T_i} softmax_t(q[b][i][hq] . k^_t / sqrt(d)) v^_t
 * with T_i = n_ctx, or min(n_ctx, q_pos0 + i + 1) when causal (query token i
 * sits at absolute position q_pos0 + i; its own token must already be in the
 * cache).  q: [B][n_q][q_heads][d] fp32 or bf16 (device, contiguous); out:
 * [B][n_q][q_heads][d] fp32 (device); q_heads any multiple of kv_heads.
 * Same decoded-vector semantics as kvq_decode_attention (rotated-space
 * scoring, sketch-space value term, one S^T product per row).  workspace:
 * kvq_prefill_workspace bytes.  1 <= n_ctx <= capacity, n_q >= 1,
 * q_pos0 >= 0, causal in {0, 1}.
 * Errors: KVQ_ERR_NULL, KVQ_ERR_ALIGN, KVQ_ERR_DTYPE, KVQ_ERR_HEADS,
 * KVQ_ERR_CAPACITY, KVQ_ERR_RANGE, KVQ_ERR_WORKSPACE, KVQ_ERR_HIP. */
kvq_status kvq_prefill_attention(const kvq_cache *c, const void *q, int q_dtype, int q_heads,
                                 int n_q, int q_pos0, int causal, int n_ctx, float *out,
                                 void *workspace, size_t workspace_bytes, void *stream);

/* kvq_prefill_attention with a full-precision window ("Your KV cache is not a
 * bit problem but a geometry problem", "Systems tax" and "What we should do":
 * recent tokens kept unquantized; its frontier section: attention sinks).
 * Query token i (position q_pos0 + i) attends over the compressed slots
 * [t_begin, t_end) -- only slots <= q_pos0 + i when causal -- together with
 * all n_win window tokens wk, wv [B][kv_heads][n_win][d] (w_dtype KVQ_F32 or
 * KVQ_BF16, 16-B aligned; caller-owned, read only): the window holds tokens
 * that precede the chunk (sinks, the most recent tokens before it), so every
 * query of the chunk sees all of them.  One softmax over the union.
 * 0 <= t_begin <= t_end <= capacity, 0 <= n_win <= 4096,
 * t_end - t_begin + n_win >= 1; wk / wv may be null when n_win == 0.  Other
 * arguments, workspace and errors as kvq_prefill_attention. */
kvq_status kvq_prefill_attention_window(const kvq_cache *c, const void *q, int q_dtype,
                                        int q_heads, int n_q, int q_pos0, int causal, int t_begin,
                                        int t_end, const void *wk, const void *wv, int w_dtype,
                                        int n_win, float *out, void *workspace,
                                        size_t workspace_bytes, void *stream);

/* Workspace bytes kvq_prefill_attention (and kvq_prefill_attention_window)
 * needs: 4 * B * q_heads * n_q * (d * (1 + [K sketched]) + S * (2 + 2 d) +
 * 2 + d), S the token splits the library uses for this shape (more when the
 * rows alone do not fill the GPU; at most 64). */
kvq_status kvq_prefill_workspace(const kvq_cache *c, int q_heads, int n_q, size_t *bytes);

/* Static text for a status code. */
const char *kvq_status_str(kvq_status s);

/* Library version string. */
const char *kvq_version(void);

/* Measurement aid, not part of the codec: one streaming read of `bytes`
 * (a multiple of 16) of device memory at buf (16-B aligned), grid-stride,
 * non-temporal 16-byte loads; out: 4 device words that the kernel may write
 * (its result is meaningless).  Timing it gives the read bandwidth the device
 * reaches with the simplest access pattern, the practical ceiling for the
 * decode scan.  Errors: KVQ_ERR_NULL, KVQ_ERR_ALIGN, KVQ_ERR_RANGE, KVQ_ERR_HIP. */
kvq_status kvq_probe_stream_read(const void *buf, size_t bytes, uint32_t *out, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* KVQ_H */
