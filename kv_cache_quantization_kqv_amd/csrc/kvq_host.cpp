// kvq_host.cpp -- host half of libkvq: codebook construction, sketch
// generation, cache layout, argument validation and the extern "C" entry
// points that launch the gfx950 kernels.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <type_traits>
#include <vector>

#include "kvq_internal.hpp"

namespace {

// ---------------------------------------------------------------------------
// Codebook: Lloyd-Max on f(t) ~ (1 - t^2)^((d-3)/2) over [-1, 1].
// ("KVQuant++" thread, "Codebook design"; D'Alberto summary, "Theoretical
// framework".)  With t = sin(theta) the weight becomes cos^(d-2)(theta), whose
// integral from 0 follows the Wallis reduction
//   W_n(x) = cos^(n-1)(x) sin(x) / n + (n-1)/n * W_(n-2)(x),  W_0 = x, W_1 = sin x,
// and the first moment has the antiderivative -(1 - t^2)^((d-1)/2) / (d-1).
// Only the positive half is iterated; the table is mirrored, so it is exactly
// symmetric and the middle threshold is 0.
// ---------------------------------------------------------------------------
double wallis(int n, double x) {
  double s = std::sin(x), c = std::cos(x);
  double w = (n & 1) ? s : x;
  double cp = (n & 1) ? 1.0 : c;  // cos^(k-1) for the next k
  for (int k = (n & 1) ? 3 : 2; k <= n; k += 2) {
    w = cp * s / k + (double)(k - 1) / k * w;
    cp *= c * c;
  }
  return w;
}

double cell_mass(int d, double a, double b) {
  return wallis(d - 2, std::asin(b)) - wallis(d - 2, std::asin(a));
}

double cell_moment(int d, double a, double b) {
  double e = 0.5 * (d - 1);
  return (std::pow(1.0 - a * a, e) - std::pow(1.0 - b * b, e)) / (d - 1);
}

void lloyd_max_positive(int d, int half, double *c) {
  for (int i = 0; i < half; ++i) c[i] = std::fmin(0.95, 2.0 * (i + 0.5) / (half * std::sqrt((double)d)));
  double edge[9];
  int still = 0;
  for (int it = 0; it < 400000; ++it) {
    edge[0] = 0.0;
    edge[half] = 1.0;
    for (int i = 1; i < half; ++i) edge[i] = 0.5 * (c[i - 1] + c[i]);
    double delta = 0.0, top = 0.0;
    for (int i = 0; i < half; ++i) {
      double nc = cell_moment(d, edge[i], edge[i + 1]) / cell_mass(d, edge[i], edge[i + 1]);
      delta = std::fmax(delta, std::fabs(nc - c[i]));
      top = std::fmax(top, std::fabs(nc));
      c[i] = nc;
    }
    if (delta <= 4.0 * 2.220446049250313e-16 * top) break;
    still = delta < 1e-13 * top ? still + 1 : 0;
    if (still >= 64) break;
  }
}

// ---------------------------------------------------------------------------
// Sketch generator: SplitMix64 (Steele, Lea & Flood 2014) counter stream,
// 53-bit uniforms in (0, 1], Box-Muller pairs in fp64, fp32 then bf16 RNE.
// ---------------------------------------------------------------------------
uint64_t splitmix64(uint64_t &state) {
  uint64_t z = (state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

uint16_t to_bf16(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Haar-random rotation in SO(d) ("KVQuant++" thread, "Rotation invariance
// guarantee"): Householder QR of a standard Gaussian matrix G = Q R in fp64
// (Golub & Van Loan, Householder QR), Q times diag(sign R_kk) (Haar on O(d)),
// the first column negated when det Q = -1 (each reflector has determinant -1),
// rounded to fp32.  Q_out row-major.  False if G is numerically singular.
bool haar_so(uint64_t seed, int d, float *Q_out) {
  const int n = d;
  std::vector<double> Ab((size_t)n * n), Vb((size_t)n * n), Qb((size_t)n * n);
  double *A = Ab.data(), *V = Vb.data(), *Qd = Qb.data();
  uint64_t state = seed;
  const double two_pi = 6.283185307179586476925286766559;
  for (int i = 0; i < n * n; i += 2) {
    double u1 = (double)((splitmix64(state) >> 11) + 1) * 0x1.0p-53;
    double u2 = (double)((splitmix64(state) >> 11) + 1) * 0x1.0p-53;
    double r = std::sqrt(-2.0 * std::log(u1));
    A[i] = r * std::cos(two_pi * u2);
    if (i + 1 < n * n) A[i + 1] = r * std::sin(two_pi * u2);
  }
  int det_sign = 1;
  double rdiag_sign[128];
  for (int k = 0; k < n; ++k) {
    // reflector v (stored in V[k][k..n-1]) mapping A[k..n-1][k] onto -sign(a_kk) ||.|| e_k
    double norm = 0.0;
    for (int i = k; i < n; ++i) norm += A[i * n + k] * A[i * n + k];
    norm = std::sqrt(norm);
    if (!(norm > 0.0)) return false;
    const double akk = A[k * n + k];
    const double alpha = akk >= 0.0 ? -norm : norm;
    double vnorm2 = 0.0;
    for (int i = k; i < n; ++i) {
      V[k * n + i] = A[i * n + k] - (i == k ? alpha : 0.0);
      vnorm2 += V[k * n + i] * V[k * n + i];
    }
    if (vnorm2 > 0.0) {
      det_sign = -det_sign;
      for (int j = k; j < n; ++j) {
        double dot = 0.0;
        for (int i = k; i < n; ++i) dot += V[k * n + i] * A[i * n + j];
        const double f = 2.0 * dot / vnorm2;
        for (int i = k; i < n; ++i) A[i * n + j] -= f * V[k * n + i];
      }
    }
    rdiag_sign[k] = A[k * n + k] >= 0.0 ? 1.0 : -1.0;
    // remember the reflector's squared norm in A's (now zero) subdiagonal slot
    A[k * n + k] = vnorm2;
  }
  // Q = H_0 H_1 ... H_{n-1}: apply the reflectors in reverse to the identity
  for (int i = 0; i < n * n; ++i) Qd[i] = 0.0;
  for (int i = 0; i < n; ++i) Qd[i * n + i] = 1.0;
  for (int k = n - 1; k >= 0; --k) {
    const double vnorm2 = A[k * n + k];
    if (!(vnorm2 > 0.0)) continue;
    for (int j = 0; j < n; ++j) {
      double dot = 0.0;
      for (int i = k; i < n; ++i) dot += V[k * n + i] * Qd[i * n + j];
      const double f = 2.0 * dot / vnorm2;
      for (int i = k; i < n; ++i) Qd[i * n + j] -= f * V[k * n + i];
    }
  }
  for (int k = 0; k < n; ++k) {
    if (rdiag_sign[k] < 0.0) {
      det_sign = -det_sign;
      for (int i = 0; i < n; ++i) Qd[i * n + k] = -Qd[i * n + k];
    }
  }
  if (det_sign < 0)
    for (int i = 0; i < n; ++i) Qd[i * n] = -Qd[i * n];
  for (int i = 0; i < n * n; ++i) Q_out[i] = (float)Qd[i];
  return true;
}

struct Sides {
  int kb, vb, kq, vq, rot;
};

kvq_status scheme_sides(int scheme, int n, Sides *s) {
  switch (scheme) {
    case KVQ_SCHEME_KV:
      if (n < 1 || n > 4) return KVQ_ERR_BITS;
      *s = {n, n, 0, 0, 0};
      return KVQ_OK;
    case KVQ_SCHEME_KQV:
      if (n < 2 || n > 4) return KVQ_ERR_BITS;
      *s = {n, n - 1, 0, 1, 1};
      return KVQ_OK;
    case KVQ_SCHEME_QKQV:
      if (n < 2 || n > 4) return KVQ_ERR_BITS;
      *s = {n - 1, n - 1, 1, 1, 1};
      return KVQ_OK;
    default:
      return KVQ_ERR_SCHEME;
  }
}

bool supported_dim(int d) { return d == 8 || d == 16 || d == 32 || d == 64 || d == 128 || d == 256; }

// The encoder's table bucketize needs a symmetric threshold table with a zero
// middle threshold, and at most one threshold in every cell of the prefix
// (sign, exponent, MB mantissa bits; MB = 2 for 4-bit codes, else 1) of u:
// positive thresholds with distinct prefixes, the smallest one above the
// prefix-0 cell (which holds the zero threshold).
bool codebook_usable(const kvq_codebook &cb) {
  const int K = 1 << cb.bits, half = K / 2;
  const int shift = 23 - (cb.bits >= 4 ? 2 : 1);
  // the cell table serves codes of 3 and 4 bits at d >= 16; compares (which
  // need only the symmetry) serve the others
  const bool cells = cb.bits > 2 && cb.d >= 16;
  if (cb.threshold[half - 1] != 0.0f) return false;
  for (int k = 0; k + 1 < half; ++k) {
    const float p = cb.threshold[half + k];
    if (!(p > 0.0f) || p >= 2.0f || cb.threshold[half - 2 - k] != -p) return false;
    if (!cells) continue;
    if (k == 0) {
      uint32_t a;
      std::memcpy(&a, &p, 4);
      if ((a >> shift) == 0) return false;
    }
    if (k > 0) {
      uint32_t a, b;
      const float q = cb.threshold[half + k - 1];
      std::memcpy(&a, &q, 4);
      std::memcpy(&b, &p, 4);
      if ((a >> shift) == (b >> shift) || !(p > q)) return false;
    }
  }
  for (int i = 0; i < half; ++i)
    if (cb.centroid[half + i] != -cb.centroid[half - 1 - i]) return false;
  return true;
}

// Sign words of the randomized Hadamard rotation: no bits at or beyond d.
bool signs_fit(const uint32_t *w, int d) {
  for (int k = 0; k < 8; ++k) {
    const int lo = 32 * k;
    const uint32_t allowed = d >= lo + 32 ? 0xFFFFFFFFu : (d <= lo ? 0u : ((1u << (d - lo)) - 1u));
    if (w[k] & ~allowed) return false;
  }
  return true;
}

// Rotation kind of the codec (RK_*).
int rot_code(const kvq_cache *c) { return c->rotate ? kvq::RK_WHT + c->rot_kind : kvq::RK_NONE; }
bool hadamard_kind(int rk) { return rk == kvq::RK_WHT || rk == kvq::RK_RHT; }

// Structural checks shared by every device entry point.
// The value side at d = 128 is stored in token groups (kvq_vgroup.hpp).
bool vgrouped(const kvq_cache *c) { return c->d == 128; }

kvq_status check_cache(const kvq_cache *c) {
  if (!c) return KVQ_ERR_NULL;
  Sides s;
  kvq_status st = scheme_sides(c->scheme, c->n_bits, &s);
  if (st != KVQ_OK) return st;
  if (!supported_dim(c->d)) return KVQ_ERR_DIM;
  if (c->m != c->d) return KVQ_ERR_DIM;
  if (c->k_bits != s.kb || c->v_bits != s.vb || c->k_qjl != s.kq || c->v_qjl != s.vq ||
      c->rotate != s.rot)
    return KVQ_ERR_SCHEME;
  if (c->cb_k.d != c->d || c->cb_k.bits != s.kb || c->cb_v.d != c->d || c->cb_v.bits != s.vb)
    return KVQ_ERR_BITS;
  if (!codebook_usable(c->cb_k) || !codebook_usable(c->cb_v)) return KVQ_ERR_BITS;
  if (c->batch < 1 || c->kv_heads < 1 || c->capacity < 1) return KVQ_ERR_RANGE;
  // value groups (d = 128) must not straddle two units
  if (vgrouped(c) && c->capacity % 16) return KVQ_ERR_RANGE;
  if ((long long)c->batch * c->kv_heads * c->capacity > (1ll << 40)) return KVQ_ERR_RANGE;
  if (!c->k_codes || !c->k_norm || !c->v_codes || !c->v_norm) return KVQ_ERR_NULL;
  if (s.kq && (!c->k_signs || !c->k_rnorm)) return KVQ_ERR_NULL;
  if (s.vq && (!c->v_signs || !c->v_rnorm)) return KVQ_ERR_NULL;
  if ((s.kq || s.vq) && !c->S) return KVQ_ERR_NULL;
  if (c->rot_kind < KVQ_ROT_WHT || c->rot_kind > KVQ_ROT_QR) return KVQ_ERR_SCHEME;
  if (!s.rot && c->rot_kind != KVQ_ROT_WHT) return KVQ_ERR_SCHEME;
  if (c->rot_kind == KVQ_ROT_QR && !c->rot_Q) return KVQ_ERR_NULL;
  if (c->rot_kind == KVQ_ROT_RHT && !signs_fit(c->rot_signs, c->d)) return KVQ_ERR_RANGE;
  const void *ptrs[] = {c->k_codes, c->k_norm, c->v_codes, c->v_norm, c->k_signs, c->k_rnorm,
                        c->v_signs, c->v_rnorm, c->S,
                        c->rot_kind == KVQ_ROT_QR ? (const void *)c->rot_Q : nullptr};
  for (const void *p : ptrs)
    if (p && !aligned16(p)) return KVQ_ERR_ALIGN;
  return KVQ_OK;
}

kvq_status hip_status(hipError_t e) { return e == hipSuccess ? KVQ_OK : KVQ_ERR_HIP; }

template <typename F>
hipError_t by_dim(int d, F &&f) {
  switch (d) {
    case 8: return f(std::integral_constant<int, 8>{});
    case 16: return f(std::integral_constant<int, 16>{});
    case 32: return f(std::integral_constant<int, 32>{});
    case 64: return f(std::integral_constant<int, 64>{});
    case 256: return f(std::integral_constant<int, 256>{});
    default: return f(std::integral_constant<int, 128>{});
  }
}

const float kLog2e = 1.4426950408889634f;

kvq_status quantize_side(const kvq_cache *c, int side, const void *src, int dtype, int t0, int T,
                         int64_t sb, int64_t sh, int64_t st, void *stream) {
  kvq_status s = check_cache(c);
  if (s != KVQ_OK) return s;
  if (!src) return KVQ_ERR_NULL;
  if (dtype != KVQ_F32 && dtype != KVQ_BF16) return KVQ_ERR_DTYPE;
  if (T < 1 || t0 < 0) return KVQ_ERR_RANGE;
  if ((long long)t0 + T > c->capacity) return KVQ_ERR_CAPACITY;
  const int esz = dtype == KVQ_F32 ? 4 : 2;
  if (!aligned16(src) || ((sb * esz) & 15) || ((sh * esz) & 15) || ((st * esz) & 15))
    return KVQ_ERR_ALIGN;
  kvq::QuantArgs a;
  std::memset(&a, 0, sizeof(a));
  a.src = src;
  a.sb = sb; a.sh = sh; a.st = st;
  a.B = c->batch; a.H = c->kv_heads; a.T = T; a.t0 = t0; a.cap = c->capacity;
  const int rk = rot_code(c);
  // tokens per quantize tile (64 / lanes per vector; one lane per vector for
  // the dense rotation, a lane pair at d = 256)
  const int vt = rk == kvq::RK_QR ? (c->d > 128 ? 32 : 64)
                                  : (c->d <= 64 ? 64 : (c->d == 128 ? 32 : 16));
  // tiles are aligned to vt slots: the first starts at t0 - t0 % vt
  a.tiles_per_bh = (t0 % vt + T + vt - 1) / vt;
  long long tiles = (long long)a.tiles_per_bh * a.B * a.H;
  if (tiles > (1ll << 31) - 1) return KVQ_ERR_RANGE;
  a.total_tiles = (int)tiles;
  a.scale = hadamard_kind(rk) ? (float)(1.0 / std::sqrt((double)c->d)) : 1.0f;
  for (int k = 0; k < 8; ++k) a.rsign[k] = c->rot_signs[k];
  a.Q = c->rot_Q;
  const kvq_codebook &cb = side == 0 ? c->cb_k : c->cb_v;
  for (int i = 0; i < 16; ++i) a.cent[i] = cb.centroid[i];
  for (int i = 0; i < 15; ++i) a.thr[i] = cb.threshold[i];
  a.S = c->S;
  const bool qjl = side == 0 ? c->k_qjl : c->v_qjl;
  a.codes = side == 0 ? c->k_codes : c->v_codes;
  a.signs = side == 0 ? c->k_signs : c->v_signs;
  a.norm = side == 0 ? c->k_norm : c->v_norm;
  a.rnorm = side == 0 ? c->k_rnorm : c->v_rnorm;
  const int bits = side == 0 ? c->k_bits : c->v_bits;
  hipStream_t hs = (hipStream_t)stream;
  return hip_status(by_dim(c->d, [&](auto D) {
    return kvq::launch_quantize<decltype(D)::value>(a, bits, rk, qjl, dtype == KVQ_BF16,
                                                    side == 1 && vgrouped(c), hs);
  }));
}

int heads_per_block(int G) { return G >= 4 ? 4 : G; }

// Token splits of a multi-query call: enough blocks to fill the GPU (about
// 1024) when the rows alone do not, at least 256 slots per split.
int prefill_splits(const kvq_cache *c, int q_heads, int n_q) {
  const long long NR = (long long)n_q * (q_heads / c->kv_heads);
  const long long blocks = (NR + 63) / 64 * c->kv_heads * c->batch;
  long long sp = (1024 + blocks - 1) / blocks;
  const long long cap_sp = (c->capacity + 255) / 256;
  if (sp > cap_sp) sp = cap_sp;
  if (sp > 64) sp = 64;
  return sp < 1 ? 1 : (int)sp;
}

bool supported_group(int G) { return G == 1 || G == 2 || G == 4 || (G > 4 && G % 4 == 0); }

// The matrix-core scan (head dimension 128) streams any number of tokens per
// split; the vector-unit scan keeps a split's logits in LDS.
bool scan_mfma(const kvq_cache *c) { return c->d == 128; }

// Fewest splits that keep every split's logits in LDS (vector-unit scan).
long long min_splits(const kvq_cache *c, int q_heads, int n_ctx) {
  if (scan_mfma(c)) return 1;
  const int tmax = kvq::scan_tokens_max(heads_per_block(q_heads / c->kv_heads));
  return ((long long)n_ctx + tmax - 1) / tmax;
}

// Compute units of the current device (looked up once per device; the
// fallback where the runtime has no device, e.g. for host-only calls).
int device_cus() {
  static std::mutex mu;
  static std::vector<int> known;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return kvq::kCusFallback;
  std::lock_guard<std::mutex> lock(mu);
  if ((int)known.size() > dev && known[dev] > 0) return known[dev];
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus < 1)
    return kvq::kCusFallback;
  if ((int)known.size() <= dev) known.resize(dev + 1, 0);
  known[dev] = cus;
  return cus;
}

// Vector-unit scan: about kvq::kScanBlocks blocks, the split length rounded up
// to whole 256-token rounds (at least 256) and within the LDS logit buffer.
// Matrix-core scan (workers take interleaved 64-token chunks): one round of
// resident blocks (every CU at the scan's occupancy), so no block waits for a
// second round and the fewest split partials are written; at most one chunk
// per worker (4 per split).
int auto_splits(const kvq_cache *c, int q_heads, int n_ctx) {
  const int G = q_heads / c->kv_heads;
  const int HG = G / heads_per_block(G);
  const long long units = (long long)c->batch * c->kv_heads * HG;
  const long long target =
      scan_mfma(c) ? (long long)device_cus() *
                         (c->k_qjl ? kvq::kScanBlocksPerCuSketch : kvq::kScanBlocksPerCu)
                   : kvq::kScanBlocks;
  const long long want = (target + units - 1) / units;
  if (n_ctx <= 0) return 1;
  if (scan_mfma(c)) {
    const long long chunks = ((long long)n_ctx + 15 + 63) / 64;
    const long long most = (chunks + 3) / 4;
    const long long s = want < most ? want : most;
    return s < 1 ? 1 : (int)s;
  }
  long long tps = ((long long)n_ctx + want - 1) / want;
  tps = tps < 256 ? 256 : (tps + 255) / 256 * 256;
  if (!scan_mfma(c)) {
    const long long tmax = kvq::scan_tokens_max(heads_per_block(G));
    if (tps > tmax) tps = tmax;
  }
  const long long s = ((long long)n_ctx + tps - 1) / tps;
  return s < 1 ? 1 : (int)s;
}

// Tokens per split for a split count: whole 64-token value tiles (trailing
// splits may be empty; they contribute nothing to the merge).
int split_tokens(int n_ctx, int splits) {
  const int t = (n_ctx + splits - 1) / splits;
  return (t + 63) / 64 * 64;
}

}  // namespace

// ---------------------------------------------------------------------------
// Fixed device scratch for kvq_decode_attention_noalloc: a file-scope device
// array (each GPU the library runs on holds its own copy until the process
// ends).  Host code never passes the array's name to a kernel: the device
// address is looked up once per device with hipGetSymbolAddress and cached.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[KVQ_NOALLOC_SCRATCH_BYTES];

// Streaming-read probe (kvq_probe_stream_read): every thread reads 16-byte
// words in a grid-stride sweep with non-temporal loads (the pattern that comes
// closest to the HBM peak), folds them with XOR and writes one word per block
// only when the fold hits an unlikely value (the loads stay live).
constexpr int kStreamReadBlocks = 2048;
typedef unsigned int probe_u32x4 __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void stream_read_kernel(const probe_u32x4 *__restrict__ p,
                                                          size_t n16, uint32_t *out) {
  const size_t stride = (size_t)gridDim.x * 256;
  uint32_t acc = 0u;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) {
    const probe_u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) out[blockIdx.x & 3] = acc;
}

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (nullptr on failure).
void *scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

const char *kvq_version(void) { return "libkvq 0.1 (gfx950)"; }

kvq_status kvq_probe_stream_read(const void *buf, size_t bytes, uint32_t *out, void *stream) {
  if (!buf || !out) return KVQ_ERR_NULL;
  if (!aligned16(buf) || !aligned16(out)) return KVQ_ERR_ALIGN;
  if (bytes < 16 || bytes % 16) return KVQ_ERR_RANGE;
  hipLaunchKernelGGL(stream_read_kernel, dim3(kStreamReadBlocks), dim3(256), 0, (hipStream_t)stream,
                     (const probe_u32x4 *)buf, bytes / 16, out);
  return hip_status(hipGetLastError());
}

const char *kvq_status_str(kvq_status s) {
  switch (s) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_NULL: return "null pointer";
    case KVQ_ERR_ALIGN: return "misaligned pointer or stride (16-byte rule)";
    case KVQ_ERR_DIM: return "unsupported head dimension";
    case KVQ_ERR_BITS: return "bit width out of range for the scheme";
    case KVQ_ERR_SCHEME: return "unknown or inconsistent scheme";
    case KVQ_ERR_CAPACITY: return "token range exceeds cache capacity";
    case KVQ_ERR_WORKSPACE: return "workspace missing or too small";
    case KVQ_ERR_DTYPE: return "unsupported element type";
    case KVQ_ERR_HEADS: return "unsupported query/KV head ratio";
    case KVQ_ERR_RANGE: return "size out of range";
    case KVQ_ERR_HIP: return "HIP launch error";
  }
  return "unknown status";
}

kvq_status kvq_codebook_init(int d, int bits, kvq_codebook *out) {
  if (!out) return KVQ_ERR_NULL;
  if (d < 3 || d > 4096) return KVQ_ERR_DIM;
  if (bits < 1 || bits > 4) return KVQ_ERR_BITS;
  std::memset(out, 0, sizeof(*out));
  out->d = d;
  out->bits = bits;
  const int K = 1 << bits, half = K / 2;
  double c[8];
  lloyd_max_positive(d, half, c);
  // levels are binary16 values (the fp32 level rounded to nearest even), so
  // the matrix-core decode contracts with them exactly; the thresholds are
  // the midpoints of the stored levels (bucketize = nearest stored level)
  double c16[8];
  for (int i = 0; i < half; ++i) c16[i] = (double)(float)(_Float16)(float)c[i];
  for (int i = 0; i < half; ++i) {
    out->centroid[half + i] = (float)c16[i];
    out->centroid[half - 1 - i] = -(float)c16[i];
  }
  out->threshold[half - 1] = 0.0f;
  for (int i = 0; i + 1 < half; ++i) {
    float t = (float)(0.5 * (c16[i] + c16[i + 1]));
    out->threshold[half + i] = t;
    out->threshold[half - 2 - i] = -t;
  }
  return KVQ_OK;
}

kvq_status kvq_sketch_init(uint64_t seed, int m, int d, uint16_t *S) {
  if (!S) return KVQ_ERR_NULL;
  if (m < 1 || d < 1) return KVQ_ERR_RANGE;
  uint64_t state = seed;
  const size_t n = (size_t)m * d;
  const double two_pi = 6.283185307179586476925286766559;
  for (size_t i = 0; i < n; i += 2) {
    double u1 = (double)((splitmix64(state) >> 11) + 1) * 0x1.0p-53;
    double u2 = (double)((splitmix64(state) >> 11) + 1) * 0x1.0p-53;
    double r = std::sqrt(-2.0 * std::log(u1));
    S[i] = to_bf16((float)(r * std::cos(two_pi * u2)));
    if (i + 1 < n) S[i + 1] = to_bf16((float)(r * std::sin(two_pi * u2)));
  }
  return KVQ_OK;
}

kvq_status kvq_cache_init(kvq_cache *c, int scheme, int n_bits, int d, int batch, int kv_heads,
                          int capacity) {
  if (!c) return KVQ_ERR_NULL;
  Sides s;
  kvq_status st = scheme_sides(scheme, n_bits, &s);
  if (st != KVQ_OK) return st;
  if (!supported_dim(d)) return KVQ_ERR_DIM;
  if (batch < 1 || kv_heads < 1 || capacity < 1) return KVQ_ERR_RANGE;
  if (d == 128 && capacity % 16) return KVQ_ERR_RANGE;   // value token groups
  std::memset(c, 0, sizeof(*c));
  c->scheme = scheme; c->n_bits = n_bits; c->d = d; c->m = d;
  c->batch = batch; c->kv_heads = kv_heads; c->capacity = capacity;
  c->k_bits = s.kb; c->v_bits = s.vb; c->k_qjl = s.kq; c->v_qjl = s.vq; c->rotate = s.rot;
  st = kvq_codebook_init(d, s.kb, &c->cb_k);
  if (st != KVQ_OK) return st;
  return kvq_codebook_init(d, s.vb, &c->cb_v);
}

kvq_status kvq_cache_set_rotation(kvq_cache *c, int kind, const uint32_t *signs,
                                  const float *Q_device) {
  if (!c) return KVQ_ERR_NULL;
  if (kind < KVQ_ROT_WHT || kind > KVQ_ROT_QR) return KVQ_ERR_SCHEME;
  if (!c->rotate && kind != KVQ_ROT_WHT) return KVQ_ERR_SCHEME;
  uint32_t w[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
  if (kind == KVQ_ROT_RHT) {
    if (!signs) return KVQ_ERR_NULL;
    const int nw = (c->d + 31) / 32;
    for (int k = 0; k < nw && k < 8; ++k) w[k] = signs[k];
    if (!signs_fit(w, c->d)) return KVQ_ERR_RANGE;
  }
  if (kind == KVQ_ROT_QR) {
    if (!Q_device) return KVQ_ERR_NULL;
    if (!aligned16(Q_device)) return KVQ_ERR_ALIGN;
  }
  c->rot_kind = kind;
  for (int k = 0; k < 8; ++k) c->rot_signs[k] = w[k];
  c->rot_Q = kind == KVQ_ROT_QR ? Q_device : nullptr;
  return KVQ_OK;
}

kvq_status kvq_rotation_signs(uint64_t seed, int d, uint32_t out[8]) {
  if (!out) return KVQ_ERR_NULL;
  if (!supported_dim(d)) return KVQ_ERR_DIM;
  uint64_t state = seed;
  for (int k = 0; k < 8; ++k) out[k] = 0u;
  for (int i = 0; i < d; ++i)
    if (splitmix64(state) >> 63) out[i >> 5] |= 1u << (i & 31);
  return KVQ_OK;
}

kvq_status kvq_rotation_qr(uint64_t seed, int d, float *Q) {
  if (!Q) return KVQ_ERR_NULL;
  if (!supported_dim(d)) return KVQ_ERR_DIM;
  return haar_so(seed, d, Q) ? KVQ_OK : KVQ_ERR_RANGE;
}

kvq_status kvq_cache_layout(int scheme, int n_bits, int d, int batch, int kv_heads, int capacity,
                            size_t bytes_out[8]) {
  if (!bytes_out) return KVQ_ERR_NULL;
  Sides s;
  kvq_status st = scheme_sides(scheme, n_bits, &s);
  if (st != KVQ_OK) return st;
  if (!supported_dim(d)) return KVQ_ERR_DIM;
  if (batch < 1 || kv_heads < 1 || capacity < 1) return KVQ_ERR_RANGE;
  size_t rec = (size_t)batch * kv_heads * capacity;
  bytes_out[0] = rec * d * s.kb / 8;
  bytes_out[1] = s.kq ? rec * d / 8 : 0;
  bytes_out[2] = rec * 2;
  bytes_out[3] = s.kq ? rec * 2 : 0;
  bytes_out[4] = rec * d * s.vb / 8;
  bytes_out[5] = s.vq ? rec * d / 8 : 0;
  bytes_out[6] = rec * 2;
  bytes_out[7] = s.vq ? rec * 2 : 0;
  return KVQ_OK;
}

kvq_status kvq_quantize_k(const kvq_cache *c, const void *src, int dtype, int t0, int T,
                          int64_t stride_b, int64_t stride_h, int64_t stride_t, void *stream) {
  return quantize_side(c, 0, src, dtype, t0, T, stride_b, stride_h, stride_t, stream);
}

kvq_status kvq_quantize_v(const kvq_cache *c, const void *src, int dtype, int t0, int T,
                          int64_t stride_b, int64_t stride_h, int64_t stride_t, void *stream) {
  return quantize_side(c, 1, src, dtype, t0, T, stride_b, stride_h, stride_t, stream);
}

kvq_status kvq_dequantize(const kvq_cache *c, int which, int t0, int T, float *out, void *stream) {
  kvq_status s = check_cache(c);
  if (s != KVQ_OK) return s;
  if (!out) return KVQ_ERR_NULL;
  if (!aligned16(out)) return KVQ_ERR_ALIGN;
  if (which != 0 && which != 1) return KVQ_ERR_RANGE;
  if (T < 1 || t0 < 0) return KVQ_ERR_RANGE;
  if ((long long)t0 + T > c->capacity) return KVQ_ERR_CAPACITY;
  long long nvec = (long long)c->batch * c->kv_heads * T;
  if (nvec > (1ll << 31) - 1) return KVQ_ERR_RANGE;
  kvq::DequantArgs a;
  std::memset(&a, 0, sizeof(a));
  const bool k = which == 0;
  a.codes = k ? c->k_codes : c->v_codes;
  a.signs = k ? c->k_signs : c->v_signs;
  a.norm = k ? c->k_norm : c->v_norm;
  a.rnorm = k ? c->k_rnorm : c->v_rnorm;
  a.S = c->S;
  a.out = out;
  a.H = c->kv_heads; a.cap = c->capacity; a.t0 = t0; a.T = T;
  a.vg = !k && vgrouped(c);
  const kvq_codebook &cb = k ? c->cb_k : c->cb_v;
  for (int i = 0; i < 16; ++i) a.cent[i] = cb.centroid[i];
  a.coef = (float)(std::sqrt(std::acos(-1.0) / 2.0) / c->m);
  const int rk = rot_code(c);
  a.oscale = hadamard_kind(rk) ? (float)(1.0 / std::sqrt((double)c->d)) : 1.0f;
  for (int r = 0; r < 8; ++r) a.rsign[r] = c->rot_signs[r];
  a.Q = c->rot_Q;
  const int bits = k ? c->k_bits : c->v_bits;
  const bool qjl = k ? c->k_qjl : c->v_qjl;
  hipStream_t hs = (hipStream_t)stream;
  return hip_status(by_dim(c->d, [&](auto D) {
    return kvq::launch_dequantize<decltype(D)::value>(a, bits, rk, qjl, (int)nvec, hs);
  }));
}

int kvq_decode_auto_splits(const kvq_cache *c, int q_heads, int n_ctx) {
  if (check_cache(c) != KVQ_OK || q_heads < 1 || n_ctx < 1 || q_heads % c->kv_heads) return 0;
  if (!supported_group(q_heads / c->kv_heads)) return 0;
  return auto_splits(c, q_heads, n_ctx);
}

kvq_status kvq_decode_workspace(const kvq_cache *c, int q_heads, int n_ctx, int splits,
                                size_t *bytes) {
  kvq_status s = check_cache(c);
  if (s != KVQ_OK) return s;
  if (!bytes) return KVQ_ERR_NULL;
  if (q_heads < 1 || q_heads % c->kv_heads) return KVQ_ERR_HEADS;
  if (!supported_group(q_heads / c->kv_heads)) return KVQ_ERR_HEADS;
  if (n_ctx < 0) return KVQ_ERR_RANGE;
  if (n_ctx > c->capacity) return KVQ_ERR_CAPACITY;
  if (splits < 0 || splits > 8192) return KVQ_ERR_RANGE;
  if (splits == 0) splits = auto_splits(c, q_heads, n_ctx);
  if (splits < min_splits(c, q_heads, n_ctx)) return KVQ_ERR_RANGE;
  const size_t rows = (size_t)c->batch * q_heads, d = (size_t)c->d;
  *bytes = sizeof(float) * (rows * d * 2 + rows * (size_t)splits * (2 + 2 * d) + rows * (2 + d));
  return KVQ_OK;
}

namespace {

// One decode step over cache slots [t_begin, t_end) plus n_win full-precision
// window tokens (both entry points).
kvq_status decode_impl(const kvq_cache *c, const void *q, int q_dtype, int q_heads, int t_begin,
                       int t_end, const void *wk, const void *wv, int w_dtype, int n_win,
                       int splits, float *out, void *workspace, size_t workspace_bytes,
                       void *stream, int stages = KVQ_STAGE_ALL) {
  if (stages < 1 || stages > KVQ_STAGE_ALL) return KVQ_ERR_RANGE;
  kvq_status s = check_cache(c);
  if (s != KVQ_OK) return s;
  if (!q || !out) return KVQ_ERR_NULL;
  if (q_dtype != KVQ_F32 && q_dtype != KVQ_BF16) return KVQ_ERR_DTYPE;
  if (!aligned16(q) || !aligned16(out)) return KVQ_ERR_ALIGN;
  if (t_begin < 0 || t_end < t_begin || n_win < 0 || n_win > KVQ_WINDOW_MAX)
    return KVQ_ERR_RANGE;
  if (t_end > c->capacity) return KVQ_ERR_CAPACITY;
  if (t_end - t_begin + n_win < 1) return KVQ_ERR_RANGE;
  // the matrix-core scan addresses a unit's records with 32-bit byte offsets,
  // up to the end of the 64-slot chunk holding slot t_end - 1 (and one block
  // past it)
  if (scan_mfma(c) && ((uint64_t)t_end + 128) * 64u >= (1ull << 32)) return KVQ_ERR_RANGE;
  if (n_win > 0) {
    if (!wk || !wv) return KVQ_ERR_NULL;
    if (w_dtype != KVQ_F32 && w_dtype != KVQ_BF16) return KVQ_ERR_DTYPE;
    if (!aligned16(wk) || !aligned16(wv)) return KVQ_ERR_ALIGN;
  }
  const int n_ctx = t_end - t_begin;
  size_t need = 0;
  s = kvq_decode_workspace(c, q_heads, n_ctx, splits, &need);
  if (s != KVQ_OK) return s;
  if (!workspace || workspace_bytes < need) return KVQ_ERR_WORKSPACE;
  if (!aligned16(workspace)) return KVQ_ERR_ALIGN;
  if (splits == 0) splits = auto_splits(c, q_heads, n_ctx);
  const int d = c->d;
  const int G = q_heads / c->kv_heads;
  const int gt = heads_per_block(G);
  const int rows = c->batch * q_heads;
  float *ws = (float *)workspace;
  float *qt = ws;
  float *sqt = ws + (size_t)rows * d;
  float *part = ws + (size_t)rows * d * 2;
  float *wpart = part + (size_t)rows * splits * (2 + 2 * (size_t)d);
  hipStream_t hs = (hipStream_t)stream;

  kvq::PrepArgs p;
  std::memset(&p, 0, sizeof(p));       // nq = 0: decode layout
  p.q = q; p.qt = qt; p.sqt = sqt; p.S = c->S; p.rows = rows;
  p.Hq = q_heads; p.Hkv = c->kv_heads; p.G = G; p.GT = gt; p.HG = G / gt;
  const int rk = rot_code(c);
  p.qscale = hadamard_kind(rk) ? (float)(kLog2e / d) : (float)(kLog2e / std::sqrt((double)d));
  for (int k = 0; k < 8; ++k) p.rsign[k] = c->rot_signs[k];
  p.Q = c->rot_Q;
  // the matrix-core scan prepares q' itself (Hadamard kinds or none, no key
  // sketch): no query-preparation launch
  const bool scan_preps = scan_mfma(c) && !c->k_qjl && rk != kvq::RK_QR;
  hipError_t e = hipSuccess;
  if ((stages & KVQ_STAGE_PREP) && !scan_preps) {
    e = by_dim(d, [&](auto D) {
      return kvq::launch_prep<decltype(D)::value>(p, rk, c->k_qjl != 0, q_dtype == KVQ_BF16, hs);
    });
    if (e != hipSuccess) return KVQ_ERR_HIP;
  }

  if (n_win > 0 && (stages & KVQ_STAGE_PREP)) {
    kvq::WindowArgs w;
    std::memset(&w, 0, sizeof(w));
    w.q = q; w.wk = wk; w.wv = wv; w.wpart = wpart;
    w.Hq = q_heads; w.Hkv = c->kv_heads; w.n_win = n_win; w.nq = 1;
    w.qscale = (float)(kLog2e / std::sqrt((double)d));
    e = by_dim(d, [&](auto D) {
      return kvq::launch_window<decltype(D)::value>(w, q_dtype == KVQ_BF16, w_dtype == KVQ_BF16,
                                                    rows, hs);
    });
    if (e != hipSuccess) return KVQ_ERR_HIP;
  }

  kvq::DecodeArgs a;
  std::memset(&a, 0, sizeof(a));
  a.kc = c->k_codes; a.ks = c->k_signs; a.vc = c->v_codes; a.vs = c->v_signs;
  a.kn = c->k_norm; a.kr = c->k_rnorm; a.vn = c->v_norm; a.vr = c->v_rnorm;
  a.qt = qt; a.sqt = sqt; a.part = part; a.S = c->S; a.out = out;
  a.wpart = n_win > 0 ? wpart : nullptr;
  if (scan_preps) {
    a.qsrc = q;
    a.q_bf16 = q_dtype == KVQ_BF16;
    a.qscale = p.qscale;
  }
  a.t0 = t_begin;
  a.vcoef = (float)(std::sqrt(std::acos(-1.0) / 2.0) / c->m);
  a.oscale = hadamard_kind(rk) ? (float)(1.0 / std::sqrt((double)d)) : 1.0f;
  a.rk = rk;
  for (int k = 0; k < 8; ++k) a.rsign[k] = c->rot_signs[k];
  a.Q = c->rot_Q;
  for (int i = 0; i < 16; ++i) {
    a.kcent[i] = c->cb_k.centroid[i];
    a.vcent[i] = c->cb_v.centroid[i];
  }
  a.kcoef = (float)(std::sqrt(std::acos(-1.0) / 2.0) / c->m);
  a.Hkv = c->kv_heads; a.Hq = q_heads; a.Gtot = G; a.HG = G / gt; a.cap = c->capacity;
  a.n_ctx = n_ctx; a.splits = splits;
  // the matrix-core scan splits the slots from t_begin rounded down to 16
  const int lead = scan_mfma(c) ? (t_begin & 15) : 0;
  a.tps = n_ctx > 0 ? split_tokens(n_ctx + lead, splits) : 0;
  e = by_dim(d, [&](auto D) {
    return kvq::launch_decode<decltype(D)::value>(a, c->k_bits, c->k_qjl != 0, c->v_bits,
                                                  c->v_qjl != 0, gt, c->batch,
                                                  stages & (kvq::STAGE_SCAN | kvq::STAGE_MERGE), hs);
  });
  return hip_status(e);
}

}  // namespace

kvq_status kvq_decode_attention(const kvq_cache *c, const void *q, int q_dtype, int q_heads,
                                int n_ctx, int splits, float *out, void *workspace,
                                size_t workspace_bytes, void *stream) {
  if (n_ctx < 1) return c ? KVQ_ERR_RANGE : KVQ_ERR_NULL;
  return decode_impl(c, q, q_dtype, q_heads, 0, n_ctx, nullptr, nullptr, KVQ_F32, 0, splits,
                     out, workspace, workspace_bytes, stream);
}

kvq_status kvq_decode_attention_noalloc(const kvq_cache *c, const void *q, int q_dtype,
                                        int q_heads, int n_ctx, int splits, float *out,
                                        void *stream) {
  if (n_ctx < 1) return c ? KVQ_ERR_RANGE : KVQ_ERR_NULL;
  size_t need = 0;
  kvq_status s = kvq_decode_workspace(c, q_heads, n_ctx, splits, &need);
  if (s != KVQ_OK) return s;
  if (need > (size_t)KVQ_NOALLOC_SCRATCH_BYTES) return KVQ_ERR_WORKSPACE;
  void *ws = scratch_address();
  if (!ws) return KVQ_ERR_HIP;
  return decode_impl(c, q, q_dtype, q_heads, 0, n_ctx, nullptr, nullptr, KVQ_F32, 0, splits, out,
                     ws, (size_t)KVQ_NOALLOC_SCRATCH_BYTES, stream);
}

kvq_status kvq_decode_attention_stages(const kvq_cache *c, const void *q, int q_dtype,
                                       int q_heads, int n_ctx, int splits, int stages, float *out,
                                       void *workspace, size_t workspace_bytes, void *stream) {
  if (n_ctx < 1) return c ? KVQ_ERR_RANGE : KVQ_ERR_NULL;
  return decode_impl(c, q, q_dtype, q_heads, 0, n_ctx, nullptr, nullptr, KVQ_F32, 0, splits,
                     out, workspace, workspace_bytes, stream, stages);
}

kvq_status kvq_decode_attention_window(const kvq_cache *c, const void *q, int q_dtype,
                                       int q_heads, int t_begin, int t_end, const void *wk,
                                       const void *wv, int w_dtype, int n_win, int splits,
                                       float *out, void *workspace, size_t workspace_bytes,
                                       void *stream) {
  return decode_impl(c, q, q_dtype, q_heads, t_begin, t_end, wk, wv, w_dtype, n_win, splits, out,
                     workspace, workspace_bytes, stream);
}

kvq_status kvq_prefill_workspace(const kvq_cache *c, int q_heads, int n_q, size_t *bytes) {
  kvq_status s = check_cache(c);
  if (s != KVQ_OK) return s;
  if (!bytes) return KVQ_ERR_NULL;
  if (q_heads < 1 || q_heads % c->kv_heads) return KVQ_ERR_HEADS;
  if (n_q < 1) return KVQ_ERR_RANGE;
  const size_t rows = (size_t)c->batch * q_heads * n_q;
  if (rows > ((size_t)1 << 31) - 1) return KVQ_ERR_RANGE;
  const size_t S = (size_t)prefill_splits(c, q_heads, n_q);
  // prepared q' (and S q'), then per row and token split (M, L, o', a), then
  // the full-precision window's partial (M, L, o) per row
  *bytes = sizeof(float) * rows * ((size_t)c->d * (1 + (c->k_qjl ? 1 : 0)) + S * (2 + 2 * (size_t)c->d) +
                                   2 + (size_t)c->d);
  return KVQ_OK;
}

}  // extern "C"

namespace {

// Multi-query attention over slots [t_begin, t_end) plus n_win full-precision
// window tokens (both entry points).
kvq_status prefill_impl(const kvq_cache *c, const void *q, int q_dtype, int q_heads, int n_q,
                        int q_pos0, int causal, int t_begin, int t_end, const void *wk,
                        const void *wv, int w_dtype, int n_win, float *out, void *workspace,
                        size_t workspace_bytes, void *stream) {
  kvq_status s = check_cache(c);
  if (s != KVQ_OK) return s;
  if (!q || !out) return KVQ_ERR_NULL;
  if (q_dtype != KVQ_F32 && q_dtype != KVQ_BF16) return KVQ_ERR_DTYPE;
  if (!aligned16(q) || !aligned16(out)) return KVQ_ERR_ALIGN;
  if (causal != 0 && causal != 1) return KVQ_ERR_RANGE;
  if (n_q < 1 || q_pos0 < 0 || t_begin < 0 || t_end < t_begin) return KVQ_ERR_RANGE;
  if (n_win < 0 || n_win > KVQ_WINDOW_MAX || t_end - t_begin + n_win < 1) return KVQ_ERR_RANGE;
  if (t_end > c->capacity) return KVQ_ERR_CAPACITY;
  if (n_win > 0) {
    if (!wk || !wv) return KVQ_ERR_NULL;
    if (w_dtype != KVQ_F32 && w_dtype != KVQ_BF16) return KVQ_ERR_DTYPE;
    if (!aligned16(wk) || !aligned16(wv)) return KVQ_ERR_ALIGN;
  }
  const int n_ctx = t_end;
  size_t need = 0;
  s = kvq_prefill_workspace(c, q_heads, n_q, &need);
  if (s != KVQ_OK) return s;
  if (!workspace || workspace_bytes < need) return KVQ_ERR_WORKSPACE;
  if (!aligned16(workspace)) return KVQ_ERR_ALIGN;
  const int d = c->d;
  const int G = q_heads / c->kv_heads;
  const size_t rows = (size_t)c->batch * q_heads * n_q;
  float *qt = (float *)workspace;
  float *sqt = qt + rows * d;
  float *part = sqt + (c->k_qjl ? rows * d : 0);
  const size_t smax = (size_t)prefill_splits(c, q_heads, n_q);
  float *wpart = part + rows * smax * (2 + 2 * (size_t)d);
  hipStream_t hs = (hipStream_t)stream;
  const int rk = rot_code(c);

  kvq::PrepArgs p;
  std::memset(&p, 0, sizeof(p));
  p.q = q; p.qt = qt; p.sqt = sqt; p.S = c->S; p.rows = (int)rows;
  p.Hq = q_heads; p.Hkv = c->kv_heads; p.G = G; p.GT = 1; p.HG = G;
  p.nq = n_q;
  p.qscale = hadamard_kind(rk) ? (float)(kLog2e / d) : (float)(kLog2e / std::sqrt((double)d));
  for (int k = 0; k < 8; ++k) p.rsign[k] = c->rot_signs[k];
  p.Q = c->rot_Q;
  hipError_t e = by_dim(d, [&](auto D) {
    return kvq::launch_prep<decltype(D)::value>(p, rk, c->k_qjl != 0, q_dtype == KVQ_BF16, hs);
  });
  if (e != hipSuccess) return KVQ_ERR_HIP;

  if (n_win > 0) {
    kvq::WindowArgs w;
    std::memset(&w, 0, sizeof(w));
    w.q = q; w.wk = wk; w.wv = wv; w.wpart = wpart;
    w.Hq = q_heads; w.Hkv = c->kv_heads; w.n_win = n_win; w.nq = n_q;
    w.qscale = (float)(kLog2e / std::sqrt((double)d));
    e = by_dim(d, [&](auto D) {
      return kvq::launch_window<decltype(D)::value>(w, q_dtype == KVQ_BF16, w_dtype == KVQ_BF16,
                                                    (int)rows, hs);
    });
    if (e != hipSuccess) return KVQ_ERR_HIP;
  }

  kvq::PrefillArgs a;
  std::memset(&a, 0, sizeof(a));
  a.kc = c->k_codes; a.ks = c->k_signs; a.vc = c->v_codes; a.vs = c->v_signs;
  a.kn = c->k_norm; a.kr = c->k_rnorm; a.vn = c->v_norm; a.vr = c->v_rnorm;
  a.qt = qt; a.sqt = sqt; a.part = part;
  for (int i = 0; i < 16; ++i) {
    a.kcent[i] = c->cb_k.centroid[i];
    a.vcent[i] = c->cb_v.centroid[i];
  }
  a.kcoef = (float)(std::sqrt(std::acos(-1.0) / 2.0) / c->m);
  a.Hkv = c->kv_heads; a.G = G; a.cap = c->capacity; a.nq = n_q; a.q_pos0 = q_pos0;
  a.n_ctx = n_ctx; a.causal = causal; a.t0 = t_begin;
  {
    // the slots [t_begin rounded down to 16, t_end) in splits of whole 64-slot tiles
    const int span = t_end - (t_begin & ~15);
    const int per = (span + (int)smax - 1) / (int)smax;
    a.tps = span > 0 ? (per + 63) / 64 * 64 : 64;
    a.splits = span > 0 ? (span + a.tps - 1) / a.tps : 1;
  }
  e = by_dim(d, [&](auto D) {
    return kvq::launch_prefill<decltype(D)::value>(a, c->k_bits, c->k_qjl != 0, c->v_bits,
                                                   c->v_qjl != 0, c->batch, hs);
  });
  if (e != hipSuccess) return KVQ_ERR_HIP;

  kvq::FinishArgs f;
  std::memset(&f, 0, sizeof(f));
  f.part = part; f.S = c->S; f.out = out;
  f.vcoef = (float)(std::sqrt(std::acos(-1.0) / 2.0) / c->m);
  f.oscale = hadamard_kind(rk) ? (float)(1.0 / std::sqrt((double)d)) : 1.0f;
  f.rk = rk;
  for (int k = 0; k < 8; ++k) f.rsign[k] = c->rot_signs[k];
  f.Q = c->rot_Q;
  f.Hkv = c->kv_heads; f.Hq = q_heads; f.G = G; f.nq = n_q; f.rows = (int)rows;
  f.splits = a.splits;
  f.wpart = n_win > 0 ? wpart : nullptr;
  e = by_dim(d, [&](auto D) {
    return kvq::launch_finish<decltype(D)::value>(f, c->v_qjl != 0, (int)rows, hs);
  });
  return hip_status(e);
}

}  // namespace

extern "C" {

kvq_status kvq_prefill_attention(const kvq_cache *c, const void *q, int q_dtype, int q_heads,
                                 int n_q, int q_pos0, int causal, int n_ctx, float *out,
                                 void *workspace, size_t workspace_bytes, void *stream) {
  if (n_ctx < 1) return c ? KVQ_ERR_RANGE : KVQ_ERR_NULL;
  return prefill_impl(c, q, q_dtype, q_heads, n_q, q_pos0, causal, 0, n_ctx, nullptr, nullptr,
                      KVQ_F32, 0, out, workspace, workspace_bytes, stream);
}

kvq_status kvq_prefill_attention_window(const kvq_cache *c, const void *q, int q_dtype,
                                        int q_heads, int n_q, int q_pos0, int causal, int t_begin,
                                        int t_end, const void *wk, const void *wv, int w_dtype,
                                        int n_win, float *out, void *workspace,
                                        size_t workspace_bytes, void *stream) {
  return prefill_impl(c, q, q_dtype, q_heads, n_q, q_pos0, causal, t_begin, t_end, wk, wv, w_dtype,
                      n_win, out, workspace, workspace_bytes, stream);
}

}  // extern "C"
