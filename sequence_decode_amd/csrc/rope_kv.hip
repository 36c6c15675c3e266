// rope_kv.hip -- pos-vector RoPE and the per-sequence KV-cache append.
//
// RoPE with one position per token: ds4 pull request 604, "Commit walkthrough
// / CUDA kernels" (decode tokens of different sequences sit at arbitrary
// positions; the per-element math is that of the single-token kernel, so token
// t equals a single-token launch at pos[t] bitwise).  Here every element's
// result depends on (x pair, pos[t], i, theta, n_rot) only, so the property
// holds by construction.  The angle pos * theta^(-2i/n_rot) and its sine and
// cosine are taken in fp64: at positions near 32K an fp32 angle would already
// be off by ~1e-3 rad.  The rotation itself is four fp32 products and two
// sums, unfused.
//
// KV append: ds4 pull request 604, "2. Single-GPU decode batches don't scale"
// (the append runs per sequence with the single-token helpers); each sequence
// writes its own row ctx_len - 1.
#include <math.h>

#include "device_math.hpp"
#include "internal.hpp"

namespace sd {

namespace {

// Grid (n_tok * n_heads); threads loop over the n_rot/2 pairs of one head.
__global__ __launch_bounds__(128) void k_rope_posvec(float* x, int n_heads, int head_dim,
                                                     int64_t ld_tok, int64_t ld_head,
                                                     const int32_t* __restrict__ pos,
                                                     double theta, int n_rot) {
  const int t = blockIdx.x / n_heads;
  const int h = blockIdx.x - t * n_heads;
  const int half = n_rot / 2;
  const int p = pos[t];
  float* v = x + (int64_t)t * ld_tok + (int64_t)h * ld_head + (head_dim - n_rot);
  for (int i = threadIdx.x; i < half; i += blockDim.x) {
    float c, s, y0, y1;
    rope_angle(p, i, n_rot, theta, &c, &s);
    rope_rotate(v[i], v[i + half], c, s, &y0, &y1);
    v[i] = y0;
    v[i + half] = y1;
  }
}

// Grid (n_seq, H_kv); one thread per element pair of a head.
__global__ __launch_bounds__(128) void k_kv_append(const float* __restrict__ k_new,
                                                   const float* __restrict__ v_new,
                                                   int64_t ld_new, SeqArgs seqs, int H_kv, int D) {
  const int s = blockIdx.x;
  const int g = blockIdx.y;
  const SeqArg& a = seqs.s[s];
  const int64_t row = seq_row(a, a.ctx_len - 1) * a.ld_tok + (int64_t)g * a.ld_head;
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    const int64_t src = (int64_t)s * ld_new + (int64_t)g * D + d;
    a.k_w[row + d] = f32_to_f16_bits(k_new[src]);
    a.v_w[row + d] = f32_to_f16_bits(v_new[src]);
  }
}

// q8_0 block of 32 consecutive values held by 32 consecutive lanes: lane d
// stores its code, and the block's first lane stores fp16(d) (nearest even).
// The scale d = amax / 127 and the codes follow the library's q8 convention.
__device__ __forceinline__ void put_q8_0(float x, int d, int8_t* codes, uint16_t* scales) {
  const float amax = group_max<32>(fabsf(x));
  const float dd = q8_scale(amax);
  codes[d] = (int8_t)q8_code(x, dd);
  if ((d & 31) == 0) scales[d >> 5] = f32_to_f16_bits(dd);
}

// One element of a q4_0 block: lane d of an aligned group of 32 holds x; the
// block's scale d = amax / 7 and the code c = clamp(round-half-away(x / d),
// -8, 7) (0 when d = 0) are those of the library's q4_0 convention; the even
// lane of each pair stores the byte of nibbles c + 8 (its own in the low four
// bits), the block's first lane stores fp16(d) (nearest even).
__device__ __forceinline__ void put_q4_0(float x, int d, uint8_t* packed, uint16_t* scales) {
  const float amax = group_max<32>(fabsf(x));
  const float dd = fdiv(amax, 7.0f);
  int c = 0;
  if (dd != 0.0f) c = (int)fminf(fmaxf(roundf(fdiv(x, dd)), -8.0f), 7.0f);
  const int n = c + 8;
  const int odd = __shfl_xor(n, 1);  // the partner dim's nibble (lane d ^ 1)
  if ((d & 1) == 0) packed[d >> 1] = (uint8_t)(n | (odd << 4));
  if ((d & 31) == 0) scales[d >> 5] = f32_to_f16_bits(dd);
}

// The quantized row of (row r, head g) of a cache, K or V: q4_0 nibble pairs
// at half the element offset, else q8_0 codes at the element offset.
__device__ __forceinline__ void put_quant(float x, int d, bool q4, int8_t* codes, int64_t r, int g,
                                          const SeqArg& a, uint16_t* scales) {
  if (q4)
    put_q4_0(x, d, reinterpret_cast<uint8_t*>(codes) + r * (a.ld_tok >> 1) + (int64_t)g * (a.ld_head >> 1),
             scales);
  else
    put_q8_0(x, d, codes + r * a.ld_tok + (int64_t)g * a.ld_head, scales);
}

// Grid (n_seq, H_kv), 128 threads; D % 32 == 0, so every block of 32 dims is
// one aligned group of 32 lanes.
__global__ __launch_bounds__(128) void k_kv_append_q8(const float* __restrict__ k_new,
                                                      const float* __restrict__ v_new,
                                                      int64_t ld_new, SeqArgs seqs, int H_kv, int D) {
  const int s = blockIdx.x;
  const int g = blockIdx.y;
  const SeqArg& a = seqs.s[s];
  const int64_t r = seq_row(a, a.ctx_len - 1);
  const int64_t srow = r * (a.ld_tok >> 5) + (int64_t)g * (a.ld_head >> 5);
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    const int64_t src = (int64_t)s * ld_new + (int64_t)g * D + d;
    put_quant(k_new[src], d, a.k4, a.kq, r, g, a, a.kd + srow);
    put_quant(v_new[src], d, a.v4, a.vq, r, g, a, a.vd + srow);
  }
}

// Fused step helper.  Workgroup (t, h) for h < n_heads rotates query head h of
// token row t in place; for n_heads <= h < n_heads + n_kv it rotates key head
// g = h - n_heads and writes it, with value head g, into the cache row of the
// row's position.  Only the last n_rot dims of a head rotate (the same pairs
// and angles as k_rope_posvec); the others pass through.
//
// The angles depend on the positions alone, which every layer of a step shares:
// with tab_mode 1 the kernel takes them from rope_angle and workgroup h = 0
// keeps them in cs_tab ([row][pair] as (cos, sin)); with tab_mode 2 it reads
// them back from there (the first layer writes, the later ones read).  The
// stored values are the fp32 results themselves, so every mode rotates with
// the same bits.
__global__ __launch_bounds__(64) void k_rope_kv_step(float* qkv, int64_t ld_qkv, int n_heads,
                                                     int n_kv, int head_dim, int n_rot,
                                                     const int32_t* __restrict__ pos,
                                                     double theta, SeqArgs seqs,
                                                     float2* cs_tab, int tab_mode) {
  const int t = blockIdx.x;
  const int h = blockIdx.y;
  const int off = head_dim - n_rot;
  const int half = n_rot / 2;
  const int p = pos[t];
  float* row = qkv + (int64_t)t * ld_qkv;
  auto angle = [&](int i, float* c, float* s) {
    if (tab_mode == 2) {
      const float2 cs = cs_tab[(int64_t)t * half + i];
      *c = cs.x;
      *s = cs.y;
      return;
    }
    rope_angle(p, i, n_rot, theta, c, s);
    if (tab_mode == 1 && h == 0) cs_tab[(int64_t)t * half + i] = make_float2(*c, *s);
  };
  if (h < n_heads) {
    float* v = row + (int64_t)h * head_dim + off;
    for (int i = threadIdx.x; i < half; i += blockDim.x) {
      float c, s, y0, y1;
      angle(i, &c, &s);
      rope_rotate(v[i], v[i + half], c, s, &y0, &y1);
      v[i] = y0;
      v[i + half] = y1;
    }
  } else {
    const int g = h - n_heads;
    const float* kh = row + (int64_t)(n_heads + g) * head_dim;
    const float* vh = row + (int64_t)(n_heads + n_kv + g) * head_dim;
    int sq = 0;
#pragma unroll
    for (int i = 1; i < SD_MAX_SEQS; ++i)
      if (i < seqs.n_seq && t >= seqs.s[i].row0) sq = i;
    const SeqArg& a = seqs.s[sq];
    const int64_t crow = seq_row(a, a.ctx_len - a.n_new + (t - a.row0));
    const int64_t dst = crow * a.ld_tok + (int64_t)g * a.ld_head;
    if (a.q8) {
      // rotated key head staged in LDS, then both heads quantized by 32-lane blocks
      __shared__ float s_k[kAttnHeadDim];
      for (int i = threadIdx.x; i < half; i += blockDim.x) {
        float c, s, y0, y1;
        angle(i, &c, &s);
        rope_rotate(kh[off + i], kh[off + i + half], c, s, &y0, &y1);
        s_k[off + i] = y0;
        s_k[off + i + half] = y1;
      }
      for (int d = threadIdx.x; d < off; d += blockDim.x) s_k[d] = kh[d];
      __syncthreads();
      const int64_t sdst = crow * (a.ld_tok >> 5) + (int64_t)g * (a.ld_head >> 5);
      for (int d = threadIdx.x; d < head_dim; d += blockDim.x) {
        put_quant(s_k[d], d, a.k4, a.kq, crow, g, a, a.kd + sdst);
        put_quant(vh[d], d, a.v4, a.vq, crow, g, a, a.vd + sdst);
      }
      return;
    }
    for (int i = threadIdx.x; i < half; i += blockDim.x) {
      float c, s, y0, y1;
      angle(i, &c, &s);
      rope_rotate(kh[off + i], kh[off + i + half], c, s, &y0, &y1);
      a.k_w[dst + off + i] = f32_to_f16_bits(y0);
      a.k_w[dst + off + i + half] = f32_to_f16_bits(y1);
    }
    for (int d = threadIdx.x; d < off; d += blockDim.x) a.k_w[dst + d] = f32_to_f16_bits(kh[d]);
    for (int d = threadIdx.x; d < head_dim; d += blockDim.x) a.v_w[dst + d] = f32_to_f16_bits(vh[d]);
  }
}

}  // namespace

hipError_t launch_rope_posvec(float* x, int n_tok, int n_heads, int head_dim, int64_t ld_tok,
                              int64_t ld_head, const int32_t* pos, double theta, int n_rot,
                              hipStream_t st) {
  const int threads = n_rot / 2 < 128 ? ((n_rot / 2 + 63) / 64) * 64 : 128;
  hipLaunchKernelGGL(k_rope_posvec, dim3(n_tok * n_heads), dim3(threads), 0, st, x, n_heads,
                     head_dim, ld_tok, ld_head, pos, theta, n_rot);
  return hipGetLastError();
}

hipError_t launch_kv_append(const float* k_new, const float* v_new, int64_t ld_new,
                            const SeqArgs& seqs, int H_kv, int D, hipStream_t st) {
  if (seqs.s[0].q8)
    hipLaunchKernelGGL(k_kv_append_q8, dim3(seqs.n_seq, H_kv), dim3(128), 0, st, k_new, v_new,
                       ld_new, seqs, H_kv, D);
  else
    hipLaunchKernelGGL(k_kv_append, dim3(seqs.n_seq, H_kv), dim3(128), 0, st, k_new, v_new, ld_new,
                       seqs, H_kv, D);
  return hipGetLastError();
}

hipError_t launch_rope_kv_step(float* qkv, int64_t ld_qkv, int rows, int n_heads, int n_kv,
                               int head_dim, int n_rot, const int32_t* pos, double theta,
                               const SeqArgs& seqs, float* cs_tab, int tab_mode, hipStream_t st) {
  hipLaunchKernelGGL(k_rope_kv_step, dim3(rows, n_heads + n_kv), dim3(64), 0, st, qkv,
                     ld_qkv, n_heads, n_kv, head_dim, n_rot, pos, theta, seqs,
                     reinterpret_cast<float2*>(cs_tab), tab_mode);
  return hipGetLastError();
}

}  // namespace sd
