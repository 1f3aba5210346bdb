// kvq_internal.hpp -- declarations shared by the libkvq translation units.
// Host-side argument blocks and the per-head-dimension launch dispatchers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kvq.h"

namespace kvq {

// Vector-unit scan (d < 128): the logits and weights of one decode split stay
// in LDS, 2 floats per (token, query head of the block), so a split holds at
// most kScanWbufFloats / (2 GT) tokens.
constexpr int kScanWbufFloats = 10240;
inline int scan_tokens_max(int gt) { return kScanWbufFloats / (2 * gt); }

// Target block count of the automatic decode split choice (vector-unit scan).
constexpr long long kScanBlocks = 4096;
// Matrix-core scan: resident blocks per CU (the key-sketch variants need more
// registers and fit two), and the CU count assumed where no device answers.
constexpr int kScanBlocksPerCu = 3, kScanBlocksPerCuSketch = 2, kCusFallback = 256;

// Rotation applied by the codec (kernel template / argument code):
// none, Walsh-Hadamard, randomized Hadamard (signs, then WHT), dense Q.
enum { RK_NONE = 0, RK_WHT = 1, RK_RHT = 2, RK_QR = 3 };

// Quantize-on-write launch description (one side of the cache).
struct QuantArgs {
  const void *src;
  long long sb, sh, st;      // element strides of the source
  int B, H, T, t0, cap;
  int tiles_per_bh, total_tiles;
  float scale;               // stored norm = ||y|| * scale (1/sqrt(d) for the Hadamard kinds)
  float cent[16];
  float thr[15];
  const uint16_t *S;         // m x d bf16 (sketch sides)
  uint8_t *codes, *signs;
  uint16_t *norm, *rnorm;
  uint32_t rsign[8];         // RK_RHT: coordinate i negated when bit i is set
  const float *Q;            // RK_QR: d x d row-major
};

struct DequantArgs {
  const uint8_t *codes, *signs;
  const uint16_t *norm, *rnorm;
  const uint16_t *S;
  float *out;
  int H, cap, t0, T;
  float cent[16];
  float coef;                // sqrt(pi/2)/m
  float oscale;              // 1/sqrt(d) for the Hadamard kinds, else 1
  uint32_t rsign[8];         // RK_RHT
  const float *Q;            // RK_QR
  int vg;                    // token-group storage (value side at d = 128)
};

struct PrepArgs {
  const void *q;             // [B][Hq][d]
  float *qt;                 // rotated, scaled query [B][Hkv][HG][d][GT]
  float *sqt;                // S q' (K sketch only), same layout
  const uint16_t *S;
  int rows;                  // B * Hq
  int Hq, Hkv, G, GT, HG;    // G = Hq / Hkv query heads per KV head, GT per block, HG = G / GT
  float qscale;              // log2(e)/d (Hadamard kinds) or log2(e)/sqrt(d)
  uint32_t rsign[8];         // RK_RHT
  const float *Q;            // RK_QR
  int nq;                    // > 0: multi-query layout (rows (b, i, hq) of [B][nq][Hq][d];
                             // output [B][Hkv][nq * G][d], row i * G + g)
};

struct DecodeArgs {
  const uint8_t *kc, *ks, *vc, *vs;
  const uint16_t *kn, *kr, *vn, *vr;
  const float *qt, *sqt;      // prepared queries, layout of PrepArgs::qt
  float *part;               // [B][Hq][splits][2 + 2d]
  const uint16_t *S;         // sketch (merge: S^T a)
  float *out;                // [B][Hq][d]
  float kcent[16], vcent[16];
  float kcoef;               // sqrt(pi/2)/m (K sketch)
  float vcoef;               // sqrt(pi/2)/m (V sketch)
  float oscale;              // 1/sqrt(d) for the Hadamard kinds, else 1
  int rk;                    // rotation kind (RK_*), undone in the merge
  uint32_t rsign[8];         // RK_RHT
  const float *Q;            // RK_QR
  const float *wpart;        // full-precision window partial [B][Hq][2 + d] or null
  // the query itself ([B][Hq][d], bf16 when q_bf16) when the matrix-core scan
  // prepares q' = R q qscale in its prologue (Hadamard kinds or none, no key
  // sketch); null: q' is read from qt
  const void *qsrc;
  int q_bf16;
  float qscale;
  int t0;                    // first cache slot of the scanned range
  int Hkv, Hq, Gtot, HG, cap, n_ctx, splits, tps;
};

// Multi-query (chunked-prefill) attention over the compressed cache: nq query
// tokens x G heads per KV head attend to cache slots [0, n_ctx), causally to
// slot q_pos0 + i for query token i when `causal`.
struct PrefillArgs {
  const uint8_t *kc, *ks, *vc, *vs;
  const uint16_t *kn, *kr, *vn, *vr;
  const float *qt, *sqt;     // prepared queries [B][Hkv][NR][d], NR = nq * G (row i * G + g)
  float *part;               // [B][Hkv][NR][splits][2 + 2d]: M (base 2), L, o', a
  float kcent[16], vcent[16];
  float kcoef;               // sqrt(pi/2)/m (K sketch)
  int Hkv, G, cap, nq, q_pos0, n_ctx, causal;
  int t0;                    // first compressed slot (slots [t0, n_ctx) are read)
  int splits, tps;           // token splits per row tile, tokens per split (multiple of 64),
                             // counted from t0 rounded down to 16
};

// Finish of a multi-query call, one block per output row: o = R^T (o' + c S^T a).
struct FinishArgs {
  const float *part;         // as PrefillArgs::part (merged here)
  const uint16_t *S;
  float *out;                // [B][nq][Hq][d]
  float vcoef, oscale;
  int rk;
  uint32_t rsign[8];
  const float *Q;
  int Hkv, Hq, G, nq;
  int rows;                  // B * Hkv * nq * G
  int splits;
  const float *wpart;        // full-precision window partial per output row, or null
};

// Full-precision window (sinks and recent tokens): exact partial softmax sums
// per query row, merged with the compressed cache's splits.
#define KVQ_WINDOW_MAX 4096  // window tokens per (batch, KV head): LDS logits of one block
struct WindowArgs {
  const void *q;             // [B][Hq][d], q_dtype
  const void *wk, *wv;       // [B][Hkv][n_win][d], w_dtype
  float *wpart;              // [rows][2 + d]: max (base 2), sum, unnormalised o
  int Hq, Hkv, n_win;
  int nq;                    // query tokens per batch row (q is [B][nq][Hq][d]; 1 for decode)
  float qscale;              // log2(e)/sqrt(d)
};


// Dispatchers: one translation unit per head dimension.
template <int D> hipError_t launch_quantize(const QuantArgs &a, int bits, int rk, bool qjl,
                                            bool bf16, bool vg, hipStream_t s);
template <int D> hipError_t launch_dequantize(const DequantArgs &a, int bits, int rk, bool qjl,
                                              int n_vec, hipStream_t s);
template <int D> hipError_t launch_prep(const PrepArgs &a, int rk, bool kqjl, bool bf16,
                                        hipStream_t s);
// decode stages (bit mask): query preparation (and the full-precision window),
// the split scan, the merge
enum { STAGE_PREP = 1, STAGE_SCAN = 2, STAGE_MERGE = 4 };
template <int D> hipError_t launch_decode(const DecodeArgs &a, int kb, bool kq, int vb, bool vq,
                                          int gt, int B, int stages, hipStream_t s);
template <int D> hipError_t launch_window(const WindowArgs &a, bool q_bf16, bool w_bf16, int rows,
                                          hipStream_t s);
template <int D> hipError_t launch_prefill(const PrefillArgs &a, int kb, bool kq, int vb, bool vq,
                                           int B, hipStream_t s);
template <int D> hipError_t launch_finish(const FinishArgs &a, bool vq, int rows, hipStream_t s);

}  // namespace kvq
