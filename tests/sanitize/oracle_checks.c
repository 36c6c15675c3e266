/*
 * The CPU oracle run under AddressSanitizer and UndefinedBehaviorSanitizer
 * (built with gcc, on its own, with no HIP code): every oracle function on
 * seeded inputs with ragged sizes, each result checked against a property the
 * definition fixes, so that the sanitizers watch the same code paths the
 * tests use.  Exits non-zero on a failed check; the sanitizers abort on any
 * memory error or undefined behaviour.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double oracle_f16_to_f64(uint16_t h);
void oracle_f16_decode(const uint16_t* h, int64_t n, double* out);
int oracle_quantize_q8_act(const float* x, int64_t ldx, int n_tok, int64_t K, int8_t* xq, float* xd);
void oracle_qgemv_q8_0(const uint8_t* w, int64_t N, int64_t K, const int8_t* xq, int64_t ldxq,
                       const float* xd, int64_t ldxd, int n_tok, const float* residual, int64_t ldr,
                       float* y, int64_t ldy, double* shadow, double* absterm, const int64_t* rows,
                       int64_t n_rows);
void oracle_rope_posvec(float* x, int n_tok, int n_heads, int head_dim, int64_t ld_tok,
                        int64_t ld_head, const int32_t* pos, double theta, int n_rot);
void oracle_attn_decode_one(const float* q, const uint16_t* k, const uint16_t* v, int64_t ld_tok,
                            int64_t ld_head, int ctx_len, int H_q, int H_kv, int D, double scale,
                            float* out);
void oracle_attn_decode_one_f64(const float* q, const double* k, const double* v, int64_t ld_tok,
                                int64_t ld_head, int ctx_len, int H_q, int H_kv, int D,
                                double scale, float* out);
void oracle_rmsnorm(const float* x, int64_t ldx, int n_tok, int64_t D, const float* gamma,
                    double eps, float* y, int64_t ldy);
void oracle_swiglu(const float* g, const float* u, int64_t n, float* y);

static int failures = 0;
#define CHECK(c)                                                   \
  do {                                                             \
    if (!(c)) {                                                    \
      fprintf(stderr, "line %d: check failed: %s\n", __LINE__, #c); \
      ++failures;                                                  \
    }                                                              \
  } while (0)

static uint64_t state = 88172645463325252ull;
static uint32_t next_u32(void) { /* xorshift64 */
  state ^= state << 13;
  state ^= state >> 7;
  state ^= state << 17;
  return (uint32_t)(state >> 32);
}
static float uniform(float lo, float hi) { return lo + (hi - lo) * (float)(next_u32() >> 8) / 16777216.0f; }

/* fp16 bits of a value exactly representable in fp16 (small integers here) */
static uint16_t f16_of_int(int v) {
  if (v == 0) return 0;
  uint16_t s = v < 0 ? 0x8000 : 0;
  unsigned a = (unsigned)(v < 0 ? -v : v);
  int e = 0;
  while ((a >> e) > 1) ++e;
  unsigned mant = (e <= 10 ? a << (10 - e) : a >> (e - 10)) & 0x3ff;
  return (uint16_t)(s | ((e + 15) << 10) | mant);
}

static void f16(void) {
  double* out = malloc(sizeof(double) * 65536);
  uint16_t* h = malloc(sizeof(uint16_t) * 65536);
  for (int i = 0; i < 65536; ++i) h[i] = (uint16_t)i;
  oracle_f16_decode(h, 65536, out);
  CHECK(out[0x3C00] == 1.0 && out[0xC000] == -2.0 && out[0x0001] == ldexp(1.0, -24));
  CHECK(isinf(out[0x7C00]) && isnan(out[0x7E00]));
  for (int v = -2048; v <= 2048; ++v) CHECK(oracle_f16_to_f64(f16_of_int(v)) == (double)v);
  free(out);
  free(h);
}

static void quantize_and_gemv(void) {
  const int n_tok = 3, K = 96, ldx = 100, N = 7, nb = K / 32;
  float* x = malloc(sizeof(float) * n_tok * ldx);
  int8_t* xq = malloc((size_t)n_tok * K);
  float* xd = malloc(sizeof(float) * n_tok * nb);
  for (int i = 0; i < n_tok * ldx; ++i) x[i] = uniform(-3.0f, 3.0f);
  for (int i = 0; i < 32; ++i) x[ldx + 32 + i] = 0.0f; /* a zero block */
  CHECK(oracle_quantize_q8_act(x, ldx, n_tok, K, xq, xd) == 0);
  for (int t = 0; t < n_tok; ++t)
    for (int k = 0; k < K; ++k) {
      const float d = xd[t * nb + k / 32];
      const int q = xq[t * K + k];
      CHECK(q >= -127 && q <= 127);
      CHECK(fabs((double)x[t * ldx + k] - (double)q * d) <= 0.5 * d * (1 + 1e-6) + 1e-30);
    }
  CHECK(xd[nb + 1] == 0.0f);
  CHECK(oracle_quantize_q8_act(x, ldx, n_tok, 48, xq, xd) == -1);
  x[5] = NAN;
  CHECK(oracle_quantize_q8_act(x, ldx, n_tok, K, xq, xd) == -1);
  x[5] = 0.5f;
  CHECK(oracle_quantize_q8_act(x, ldx, n_tok, K, xq, xd) == 0);

  uint8_t* w = malloc((size_t)N * nb * 34);
  for (int n = 0; n < N; ++n)
    for (int b = 0; b < nb; ++b) {
      uint8_t* blk = w + ((size_t)n * nb + b) * 34;
      const uint16_t h = f16_of_int((int)(next_u32() % 7) + 1); /* scales 1..7 */
      blk[0] = (uint8_t)(h & 0xff);
      blk[1] = (uint8_t)(h >> 8);
      for (int i = 0; i < 32; ++i) blk[2 + i] = (uint8_t)(int8_t)((int)(next_u32() % 255) - 127);
    }
  float* res = malloc(sizeof(float) * n_tok * 8);
  for (int i = 0; i < n_tok * 8; ++i) res[i] = uniform(-1.0f, 1.0f);
  float* y = malloc(sizeof(float) * n_tok * 8);
  double* sh = malloc(sizeof(double) * n_tok * 8);
  double* ab = malloc(sizeof(double) * n_tok * 8);
  oracle_qgemv_q8_0(w, N, K, xq, K, xd, nb, n_tok, res, 8, y, 8, sh, ab, NULL, 0);
  for (int t = 0; t < n_tok; ++t)
    for (int n = 0; n < N; ++n) {
      double exact = 0.0; /* sum over blocks of d_w d_x isum, in fp64 */
      for (int b = 0; b < nb; ++b) {
        const uint8_t* blk = w + ((size_t)n * nb + b) * 34;
        long isum = 0;
        for (int i = 0; i < 32; ++i) isum += (long)(int8_t)blk[2 + i] * xq[t * K + b * 32 + i];
        exact += oracle_f16_to_f64((uint16_t)(blk[0] | (blk[1] << 8))) * xd[t * nb + b] * (double)isum;
      }
      CHECK(fabs((double)y[t * 8 + n] - res[t * 8 + n] - exact) <= 1e-5 * (ab[t * 8 + n] + fabs(res[t * 8 + n])) + 1e-30);
    }
  const int64_t rows[2] = {6, 2};
  float y2[2 * 3];
  oracle_qgemv_q8_0(w, N, K, xq, K, xd, nb, n_tok, NULL, 0, y2, 2, NULL, NULL, rows, 2);
  /* listed rows: the same sums as the full product (no residual there) */
  float y3[3 * 8];
  oracle_qgemv_q8_0(w, N, K, xq, K, xd, nb, n_tok, NULL, 0, y3, 8, NULL, NULL, NULL, 0);
  for (int t = 0; t < n_tok; ++t) CHECK(y2[t * 2 + 0] == y3[t * 8 + 6] && y2[t * 2 + 1] == y3[t * 8 + 2]);
  free(x); free(xq); free(xd); free(w); free(res); free(y); free(sh); free(ab);
}

static void rope(void) {
  const int n_tok = 3, H = 5, hd = 128;
  const int64_t ld_head = 130, ld_tok = H * ld_head;
  float* x = malloc(sizeof(float) * n_tok * ld_tok);
  float* x0 = malloc(sizeof(float) * n_tok * ld_tok);
  for (int i = 0; i < n_tok * ld_tok; ++i) x0[i] = x[i] = uniform(-2.0f, 2.0f);
  const int32_t zero[3] = {0, 0, 0};
  oracle_rope_posvec(x, n_tok, H, hd, ld_tok, ld_head, zero, 1e6, hd);
  CHECK(memcmp(x, x0, sizeof(float) * n_tok * ld_tok) == 0);
  const int32_t pos[3] = {1, 1000, 123456};
  for (int n_rot = 64; n_rot <= hd; n_rot += 64) {
    memcpy(x, x0, sizeof(float) * n_tok * ld_tok);
    oracle_rope_posvec(x, n_tok, H, hd, ld_tok, ld_head, pos, 1e6, n_rot);
    const int off = hd - n_rot, half = n_rot / 2;
    for (int t = 0; t < n_tok; ++t)
      for (int h = 0; h < H; ++h) {
        const float* a = x0 + t * ld_tok + h * ld_head;
        const float* b = x + t * ld_tok + h * ld_head;
        for (int i = 0; i < off; ++i) CHECK(a[i] == b[i]);
        for (int i = 0; i < half; ++i) {
          const double n0 = hypot(a[off + i], a[off + i + half]), n1 = hypot(b[off + i], b[off + i + half]);
          CHECK(fabs(n0 - n1) <= 1e-6 * (n0 + 1e-30));
        }
      }
  }
  free(x);
  free(x0);
}

static void attention(void) {
  const int H_q = 8, H_kv = 2, D = 128, ctx = 37;
  const int64_t ld_head = D + 8, ld_tok = H_kv * ld_head;
  uint16_t* k = malloc(sizeof(uint16_t) * ctx * ld_tok);
  uint16_t* v = malloc(sizeof(uint16_t) * ctx * ld_tok);
  double* kd = malloc(sizeof(double) * ctx * ld_tok);
  double* vd = malloc(sizeof(double) * ctx * ld_tok);
  float q[8 * 128], out[8 * 128], out2[8 * 128];
  for (int i = 0; i < H_q * D; ++i) q[i] = uniform(-0.5f, 0.5f);
  for (int i = 0; i < ctx * ld_tok; ++i) {
    k[i] = f16_of_int((int)(next_u32() % 9) - 4);
    v[i] = f16_of_int((int)(next_u32() % 9) - 4);
    kd[i] = oracle_f16_to_f64(k[i]);
    vd[i] = oracle_f16_to_f64(v[i]);
  }
  /* one key: the output is that key's value row */
  oracle_attn_decode_one(q, k, v, ld_tok, ld_head, 1, H_q, H_kv, D, 0.088, out);
  for (int h = 0; h < H_q; ++h)
    for (int d = 0; d < D; ++d) CHECK(out[h * D + d] == (float)vd[(h / 4) * ld_head + d]);
  /* the fp64 route equals the fp16 route on exactly representable values */
  oracle_attn_decode_one(q, k, v, ld_tok, ld_head, ctx, H_q, H_kv, D, 0.088, out);
  oracle_attn_decode_one_f64(q, kd, vd, ld_tok, ld_head, ctx, H_q, H_kv, D, 0.088, out2);
  CHECK(memcmp(out, out2, sizeof(out)) == 0);
  /* equal scores: the mean of the values */
  oracle_attn_decode_one(q, k, v, ld_tok, ld_head, ctx, H_q, H_kv, D, 0.0, out);
  for (int h = 0; h < H_q; ++h)
    for (int d = 0; d < D; ++d) {
      double m = 0.0;
      for (int j = 0; j < ctx; ++j) m += vd[j * ld_tok + (h / 4) * ld_head + d];
      CHECK(fabs(out[h * D + d] - m / ctx) <= 1e-6);
    }
  free(k); free(v); free(kd); free(vd);
}

static void norm_and_swiglu(void) {
  const int n_tok = 2, D = 160;
  float x[2 * 170], g[160], y[2 * 160];
  for (int i = 0; i < 2 * 170; ++i) x[i] = 0.75f;
  for (int i = 0; i < D; ++i) g[i] = (float)(i % 5) - 2.0f;
  oracle_rmsnorm(x, 170, n_tok, D, g, 1e-6, y, 160);
  for (int t = 0; t < n_tok; ++t)
    for (int i = 0; i < D; ++i) CHECK(fabs(y[t * 160 + i] - 0.75 / sqrt(0.5625 + 1e-6) * g[i]) <= 1e-6);
  float gg[5] = {0.0f, 1.0f, -1.0f, 20.0f, -20.0f}, uu[5] = {3.0f, 2.0f, 2.0f, 1.0f, 1.0f}, s[5];
  oracle_swiglu(gg, uu, 5, s);
  CHECK(s[0] == 0.0f);
  for (int i = 1; i < 5; ++i) CHECK(fabs(s[i] - gg[i] / (1.0 + exp(-gg[i])) * uu[i]) <= 1e-6 * (1 + fabs(s[i])));
}

int main(void) {
  f16();
  quantize_and_gemv();
  rope();
  attention();
  norm_and_swiglu();
  if (failures) {
    fprintf(stderr, "%d failed checks\n", failures);
    return 1;
  }
  printf("oracle checks passed\n");
  return 0;
}
