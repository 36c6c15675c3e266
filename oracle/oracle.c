/*
 * oracle.c -- plain, slow CPU reference for the exact multi-sequence decode step.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call
 * this file: only the test suite, the package smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or helper with the
 * HIP kernels; the two sides meet only on the seeded inputs.
 *
 * Every function is the plain definition of the operation, written with loops
 * in the order the definition reads, with no blocking, fusion or reordering.
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off -fopenmp (OpenMP is used only
 * across independent outputs, so the arithmetic of each output is unchanged).
 *
 * Sources (web pages, cited by title and section):
 *  [P1] "feat(qwen4exp): exact 4-slot concurrent serving" -- "How it stays exact":
 *       a batched row must use the same arithmetic as a single row.
 *  [P4] "#1209 Speed up concurrent generation, fix QFUSE, and improve prefill
 *       monitoring" -- "What changed and why", item 2: an activation quantizer
 *       must follow the consuming quantizer's division and rounding convention.
 *  [P5] ds4 pull request 604 (single-GPU fused session batching) --
 *       "Commit walkthrough / CUDA kernels": narrow-batch q8_0 matmul (each
 *       32-weight block read once and dotted against every token), pos-vector
 *       RoPE (token t equals a single-token launch at pos[t]), multi-sequence
 *       decode attention (one query per sequence over its own cache);
 *       "2. Single-GPU decode batches don't scale": the fused step structure.
 *
 * The pages print no formulas.  Where they are silent, the readings used here
 * are: q8_0 block = fp16 scale followed by 32 int8 weights (34 bytes); an
 * activation block is 32 int8 codes with an fp32 scale d = amax/127; block dot
 * = d_w * d_x * sum(int8*int8) accumulated in fp32; RoPE pairs dimension i with
 * i + n_rot/2 and rotates the last n_rot dimensions of a head; attention is
 * softmax(scale * q.k) v in fp64 over keys [0, ctx_len).
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>

#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Thread count of the oracle's later parallel loops (timing only; the
 * arithmetic of every output does not depend on it). */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
  omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* IEEE binary16 -> double, decoded from its fields (exact). */
double oracle_f16_to_f64(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 31;
  int m = h & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24);                 /* subnormal: m * 2^-14 / 2^10 */
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + m), e - 25);     /* (1 + m/2^10) * 2^(e-15) */
  return sign ? -v : v;
}

/* Decode n half-precision values (used by tests to pin the decoder). */
void oracle_f16_decode(const uint16_t* h, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_f16_to_f64(h[i]);
}

/*
 * Activation quantization, per token t and per block b of 32 values [P4 item 2,
 * P5 CUDA kernels]:
 *   amax = max |x_i|;  d = amax / 127 (fp32 IEEE division);
 *   q_i  = round_half_away(x_i / d) (fp32 division, C roundf), clamped to
 *          [-127, 127]; when d == 0 every q_i is 0.
 * Outputs: xq[t*K + k] int8 codes, xd[t*(K/32) + b] fp32 scales.
 * Returns 0, or -1 when K is not a multiple of 32 or an input is not finite.
 */
int oracle_quantize_q8_act(const float* x, int64_t ldx, int n_tok, int64_t K,
                           int8_t* xq, float* xd) {
  if (K % 32 != 0) return -1;
  int64_t nb = K / 32;
  for (int t = 0; t < n_tok; ++t) {
    for (int64_t b = 0; b < nb; ++b) {
      const float* xb = x + (int64_t)t * ldx + b * 32;
      float amax = 0.0f;
      for (int i = 0; i < 32; ++i) {
        if (!isfinite(xb[i])) return -1;
        float a = fabsf(xb[i]);
        if (a > amax) amax = a;
      }
      float d = amax / 127.0f;
      xd[(int64_t)t * nb + b] = d;
      for (int i = 0; i < 32; ++i) {
        int q = 0;
        if (d != 0.0f) {
          float r = roundf(xb[i] / d);
          if (r > 127.0f) r = 127.0f;
          if (r < -127.0f) r = -127.0f;
          q = (int)r;
        }
        xq[(int64_t)t * K + b * 32 + i] = (int8_t)q;
      }
    }
  }
  return 0;
}

/*
 * q4_0 KV rows, the Q4 cache type of the Q4/Q8 and Q8/Q4 attention cases of
 * "feat(qwen36): complete concurrent serving implementation with speculation",
 * "Validation".  The pages name the type only; the reading used here is the
 * 4-bit analogue of the q8_0 rows above, per row and block b of 32 values:
 *   amax = max |x_i|;  d = amax / 7 (fp32 IEEE division);
 *   c_i  = round_half_away(x_i / d) (fp32 division, C roundf), clamped to
 *          [-8, 7]; when d == 0 every c_i is 0;
 *   stored nibble n_i = c_i + 8, two per byte: byte j of the block holds
 *   n_{2j} in its low and n_{2j+1} in its high four bits.
 * Outputs: packed[r*(D/2) + b*16 + j], d_out[r*(D/32) + b] (fp32; the cache
 * stores it rounded to fp16).  Value of a stored element: fp16(d) * (n - 8).
 * Returns 0, or -1 when D is not a multiple of 32 or an input is not finite.
 */
int oracle_quantize_kv_q4_0(const float* x, int64_t n_rows, int64_t D, uint8_t* packed,
                            float* d_out) {
  if (D % 32 != 0) return -1;
  int64_t nb = D / 32;
  for (int64_t r = 0; r < n_rows; ++r) {
    for (int64_t b = 0; b < nb; ++b) {
      const float* xb = x + r * D + b * 32;
      float amax = 0.0f;
      for (int i = 0; i < 32; ++i) {
        if (!isfinite(xb[i])) return -1;
        float a = fabsf(xb[i]);
        if (a > amax) amax = a;
      }
      float d = amax / 7.0f;
      d_out[r * nb + b] = d;
      int nib[32];
      for (int i = 0; i < 32; ++i) {
        int c = 0;
        if (d != 0.0f) {
          float q = roundf(xb[i] / d);
          if (q > 7.0f) q = 7.0f;
          if (q < -8.0f) q = -8.0f;
          c = (int)q;
        }
        nib[i] = c + 8;
      }
      for (int j = 0; j < 16; ++j)
        packed[r * (D / 2) + b * 16 + j] = (uint8_t)(nib[2 * j] | (nib[2 * j + 1] << 4));
    }
  }
  return 0;
}

/*
 * q8_0 matrix-vector product for n_tok token rows [P5 CUDA kernels: narrow-batch
 * q8_0 matmul].  W holds N rows of K/32 blocks, each block 34 bytes: an fp16
 * scale d_w (little-endian) then 32 int8 weights.  For token t and row n:
 *   isum_b = sum_i w[n,b,i] * xq[t,b,i]                (exact, int32)
 *   s_b    = fl32( fl32(d_w[n,b] * d_x[t,b]) * (float)isum_b )
 *   y      = s_0 + s_1 + ... in fp32, left to right in block order
 *   y      = residual[t,n] + y  when a residual is given.
 * rows == NULL computes all N rows into y[t*ldy + n]; otherwise the n_rows
 * listed rows are computed into y[t*ldy + i] for the i-th listed row.
 * shadow (optional) receives sum_b s_b in fp64; absterm (optional) receives
 * sum_b |s_b| (the magnitude the fp32 rounding error scales with); both use
 * the same indexing as y.
 */
void oracle_qgemv_q8_0(const uint8_t* w, int64_t N, int64_t K,
                       const int8_t* xq, int64_t ldxq, const float* xd, int64_t ldxd,
                       int n_tok, const float* residual, int64_t ldr,
                       float* y, int64_t ldy, double* shadow, double* absterm,
                       const int64_t* rows, int64_t n_rows) {
  int64_t nb = K / 32;
  int64_t count = rows ? n_rows : N;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) {
    int64_t n = rows ? rows[i] : i;
    for (int t = 0; t < n_tok; ++t) {
      float acc = 0.0f;
      double sh = 0.0, ab = 0.0;
      for (int64_t b = 0; b < nb; ++b) {
        const uint8_t* blk = w + (n * nb + b) * 34;
        uint16_t hbits = (uint16_t)(blk[0] | (blk[1] << 8));
        float dw = (float)oracle_f16_to_f64(hbits);
        const int8_t* wq = (const int8_t*)(blk + 2);
        const int8_t* aq = xq + (int64_t)t * ldxq + b * 32;
        int32_t isum = 0;
        for (int k = 0; k < 32; ++k) isum += (int32_t)wq[k] * (int32_t)aq[k];
        float scale = dw * xd[(int64_t)t * ldxd + b];
        float s = scale * (float)isum;
        acc = acc + s;
        sh += (double)s;
        ab += fabs((double)s);
      }
      if (residual) acc = residual[(int64_t)t * ldr + n] + acc;
      y[(int64_t)t * ldy + i] = acc;
      if (shadow) shadow[(int64_t)t * ldy + i] = sh;
      if (absterm) absterm[(int64_t)t * ldy + i] = ab;
    }
  }
}

/*
 * Rotary position embedding with one position per token [P5 CUDA kernels:
 * pos-vector RoPE].  x is [n_tok][n_heads][head_dim] fp32 (token stride ld_tok,
 * head stride ld_head), rotated in place.  The last n_rot dimensions of each
 * head are rotated; with off = head_dim - n_rot and h = n_rot/2, pair
 * (off+i, off+i+h) for i < h is rotated by the angle
 *   a = pos[t] * theta^(-2i/n_rot)
 *   x'[off+i]   = x[off+i] cos a - x[off+i+h] sin a
 *   x'[off+i+h] = x[off+i] sin a + x[off+i+h] cos a
 * in fp64, and the results are rounded to fp32.
 */
void oracle_rope_posvec(float* x, int n_tok, int n_heads, int head_dim,
                        int64_t ld_tok, int64_t ld_head, const int32_t* pos,
                        double theta, int n_rot) {
  int off = head_dim - n_rot;
  int half = n_rot / 2;
  for (int t = 0; t < n_tok; ++t) {
    for (int hd = 0; hd < n_heads; ++hd) {
      float* v = x + (int64_t)t * ld_tok + (int64_t)hd * ld_head + off;
      for (int i = 0; i < half; ++i) {
        double inv_freq = pow(theta, -2.0 * (double)i / (double)n_rot);
        double a = (double)pos[t] * inv_freq;
        double c = cos(a), s = sin(a);
        double x0 = v[i], x1 = v[i + half];
        v[i] = (float)(x0 * c - x1 * s);
        v[i + half] = (float)(x0 * s + x1 * c);
      }
    }
  }
}

/*
 * Decode attention for ONE sequence [P5 CUDA kernels: multi-sequence decode
 * attention; the multi-sequence result is this function applied to each
 * sequence independently].  q is [H_q][D] fp32; the cache holds fp16 keys and
 * values, element (j, g, d) at k[j*ld_tok + g*ld_head + d].  Query head h reads
 * KV head g = h / (H_q/H_kv).  Over keys j in [0, ctx_len), in fp64:
 *   z_j = scale * sum_d q[h,d] k[j,g,d];  p_j = exp(z_j - max z) / sum exp(.)
 *   out[h,d] = sum_j p_j v[j,g,d]        rounded to fp32.
 */
void oracle_attn_decode_one(const float* q, const uint16_t* k, const uint16_t* v,
                            int64_t ld_tok, int64_t ld_head, int ctx_len,
                            int H_q, int H_kv, int D, double scale, float* out) {
  int G = H_q / H_kv;
#pragma omp parallel for schedule(static)
  for (int h = 0; h < H_q; ++h) {
    int g = h / G;
    double zmax = -INFINITY;
    /* first pass: the maximum score */
    for (int j = 0; j < ctx_len; ++j) {
      const uint16_t* kj = k + (int64_t)j * ld_tok + (int64_t)g * ld_head;
      double z = 0.0;
      for (int d = 0; d < D; ++d) z += (double)q[h * D + d] * oracle_f16_to_f64(kj[d]);
      z *= scale;
      if (z > zmax) zmax = z;
    }
    /* second pass: weights and the weighted sum of values */
    double denom = 0.0;
    double acc[1024];
    for (int d = 0; d < D; ++d) acc[d] = 0.0;
    for (int j = 0; j < ctx_len; ++j) {
      const uint16_t* kj = k + (int64_t)j * ld_tok + (int64_t)g * ld_head;
      const uint16_t* vj = v + (int64_t)j * ld_tok + (int64_t)g * ld_head;
      double z = 0.0;
      for (int d = 0; d < D; ++d) z += (double)q[h * D + d] * oracle_f16_to_f64(kj[d]);
      z *= scale;
      double p = exp(z - zmax);
      denom += p;
      for (int d = 0; d < D; ++d) acc[d] += p * oracle_f16_to_f64(vj[d]);
    }
    for (int d = 0; d < D; ++d) out[h * D + d] = (float)(acc[d] / denom);
  }
}

/*
 * The same decode attention over keys and values given as fp64 numbers (the
 * dequantized d * c of a q8_0 cache, "#1209 Speed up concurrent generation,
 * fix QFUSE, and improve prefill monitoring", "What changed and why": int8
 * KV), element (j, g, d) at k[j*ld_tok + g*ld_head + d].
 */
void oracle_attn_decode_one_f64(const float* q, const double* k, const double* v,
                                int64_t ld_tok, int64_t ld_head, int ctx_len,
                                int H_q, int H_kv, int D, double scale, float* out) {
  int G = H_q / H_kv;
#pragma omp parallel for schedule(static)
  for (int h = 0; h < H_q; ++h) {
    int g = h / G;
    double zmax = -INFINITY;
    for (int j = 0; j < ctx_len; ++j) {
      const double* kj = k + (int64_t)j * ld_tok + (int64_t)g * ld_head;
      double z = 0.0;
      for (int d = 0; d < D; ++d) z += (double)q[h * D + d] * kj[d];
      z *= scale;
      if (z > zmax) zmax = z;
    }
    double denom = 0.0;
    double acc[1024];
    for (int d = 0; d < D; ++d) acc[d] = 0.0;
    for (int j = 0; j < ctx_len; ++j) {
      const double* kj = k + (int64_t)j * ld_tok + (int64_t)g * ld_head;
      const double* vj = v + (int64_t)j * ld_tok + (int64_t)g * ld_head;
      double z = 0.0;
      for (int d = 0; d < D; ++d) z += (double)q[h * D + d] * kj[d];
      z *= scale;
      double p = exp(z - zmax);
      denom += p;
      for (int d = 0; d < D; ++d) acc[d] += p * vj[d];
    }
    for (int d = 0; d < D; ++d) out[h * D + d] = (float)(acc[d] / denom);
  }
}

/*
 * RMS normalization of n_tok rows of length D (fp64, rounded to fp32):
 *   y = x / sqrt(mean(x^2) + eps) * gamma.
 * The step structure (normalize, project, attend, feed-forward, output head)
 * follows [P5 "2. Single-GPU decode batches don't scale" and "Graph driver"];
 * the normalization itself is the plain RMSNorm reading.
 */
void oracle_rmsnorm(const float* x, int64_t ldx, int n_tok, int64_t D,
                    const float* gamma, double eps, float* y, int64_t ldy) {
  for (int t = 0; t < n_tok; ++t) {
    const float* xr = x + (int64_t)t * ldx;
    double ss = 0.0;
    for (int64_t i = 0; i < D; ++i) ss += (double)xr[i] * (double)xr[i];
    double r = 1.0 / sqrt(ss / (double)D + eps);
    for (int64_t i = 0; i < D; ++i)
      y[(int64_t)t * ldy + i] = (float)((double)xr[i] * r * (double)gamma[i]);
  }
}

/* SwiGLU gate: y = silu(g) * u = g / (1 + exp(-g)) * u, fp64 rounded to fp32. */
void oracle_swiglu(const float* g, const float* u, int64_t n, float* y) {
  for (int64_t i = 0; i < n; ++i) {
    double gv = g[i];
    y[i] = (float)(gv / (1.0 + exp(-gv)) * (double)u[i]);
  }
}
