// attn.hip -- multi-sequence grouped-query decode attention.
//
// What it computes: ds4 pull request 604, "Commit walkthrough / CUDA kernels"
// (one query token per sequence, each attending to its own cache; the
// per-sequence views travel by value in the kernel arguments, at most four),
// in one launch for all sequences ("2. Single-GPU decode batches don't
// scale").  The layout here is CDNA4's own:
//
// * Work unit = (sequence, KV head, chunk of SD_ATTN_CHUNK keys).  The chunk
//   size is fixed, so how a sequence is split depends on its own length only;
//   the grid is the sum of all sequences' units, which fills 256 CUs even for
//   four sequences (a sequence-per-workgroup split would give 32 units).
// * A workgroup loads each key and value row of its chunk once for the four
//   query heads that share the KV head; every load is issued before any
//   arithmetic.  Scores come from MFMA (fp16 keys as stored, the fp32 query as
//   an exact fp16 hi + lo pair), the weighted value sum from v_fma_mix (fp16
//   values straight into fp32 FMAs).
// * Each wave keeps its own softmax partial over its 64 keys, and the four
//   merge in wave order: partial (m, l, o[128]) per head and chunk.
// * A second kernel merges the partials of each (sequence, head) with fixed
//   reduction shapes.  Every sum has a fixed shape, so a sequence's output bits do not
//   depend on the other sequences in the call.
#include <math.h>

#include "device_math.hpp"
#include "internal.hpp"

namespace sd {

namespace {

constexpr int C = kAttnChunk;
constexpr int HD = kAttnHeadDim;
constexpr int PF = kAttnPartialFloats;

__device__ __forceinline__ void unpack8(const u32x4a& k, float* f) {
  f[0] = f16_bits_to_f32(k.x);
  f[1] = f16_bits_to_f32(k.x >> 16);
  f[2] = f16_bits_to_f32(k.y);
  f[3] = f16_bits_to_f32(k.y >> 16);
  f[4] = f16_bits_to_f32(k.z);
  f[5] = f16_bits_to_f32(k.z >> 16);
  f[6] = f16_bits_to_f32(k.w);
  f[7] = f16_bits_to_f32(k.w >> 16);
}

__device__ __forceinline__ int find_seq(const SeqArgs& a, int u) {
  int s = 0;
#pragma unroll
  for (int i = 1; i < SD_MAX_SEQS; ++i)
    if (i < a.n_seq && u >= a.s[i].unit_begin) s = i;
  return s;
}

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float cross_row_max(float v) {
  auto p = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, v),
                                            __builtin_bit_cast(uint32_t, v), false, false);
  v = fmaxf(__builtin_bit_cast(float, (uint32_t)p[0]), __builtin_bit_cast(float, (uint32_t)p[1]));
  auto q = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, v),
                                            __builtin_bit_cast(uint32_t, v), false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)q[0]), __builtin_bit_cast(float, (uint32_t)q[1]));
}

// One workgroup = (sequence, KV head g, chunk of C keys); wave w owns keys
// w*64 .. w*64+63 of the chunk.
//  * Scores by MFMA (v_mfma_f32_16x16x32_f16): A = 16 keys x 32 dims of K (fp16
//    as stored), B = 32 dims x 16 columns of q^T (the 4 heads of the group, the
//    other 12 columns zero).  q is fp32; it enters as q_hi + q_lo (two fp16
//    parts, q - q_hi - q_lo ~ 2^-22 |q|), so each fp16 x fp16 product is exact
//    and the score keeps fp32 accuracy.
//  * Each wave forms its own softmax partial (max, sum of weights, weighted
//    value sum) over its 64 keys; the weighted values use v_fma_mix (fp16 V
//    straight into fp32 FMAs).  The 4 wave partials merge in wave order.
__global__ __launch_bounds__(256) void k_attn_chunk(const float* __restrict__ q, int64_t ld_q,
                                                    SeqArgs seqs, int H_q, float scale,
                                                    float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) float s_p[4][64][kAttnGroup];  // [wave][key][head]
  __shared__ float s_m[4][kAttnGroup], s_l[4][kAttnGroup];
  __shared__ float s_o[4][kAttnGroup * HD];

  const int s = find_seq(seqs, blockIdx.x);
  const SeqArg& A = seqs.s[s];
  const int local = blockIdx.x - A.unit_begin;
  const int g = local / A.n_chunks;
  const int c = local - g * A.n_chunks;
  const int j0 = c * C;
  const int nk = min(C, A.ctx_len - j0);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 15;   // MFMA column / row-in-tile index
  const int kg = lane >> 4;    // MFMA k-group (8 of the 32 dims)

  // ---- K tiles (A operands), issued first: tile t = keys wave*64 + 16t + col
  const uint16_t* kbase = A.k + (int64_t)g * A.ld_head;
  u32x4a ka[4][4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int jl = wave * 64 + 16 * t + col;
    const uint16_t* kr = kbase + (int64_t)(j0 + jl) * A.ld_tok + 8 * kg;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      ka[t][kk] = u32x4a{0u, 0u, 0u, 0u};
      if (jl < nk) ka[t][kk] = *reinterpret_cast<const u32x4a*>(kr + 32 * kk);
    }
  }
  // ---- V rows for the weighted sum: lane = 16 * kslot + dg, key wave*64 + 4*step + kslot
  const int kslot = lane >> 4;
  const int dg = lane & 15;
  const uint16_t* vbase = A.v + (int64_t)g * A.ld_head + 8 * dg;
  u32x4a vv[16];
#pragma unroll
  for (int step = 0; step < 16; ++step) {
    const int jl = wave * 64 + step * 4 + kslot;
    vv[step] = u32x4a{0u, 0u, 0u, 0u};
    if (jl < nk) vv[step] = *reinterpret_cast<const u32x4a*>(vbase + (int64_t)(j0 + jl) * A.ld_tok);
  }
  // ---- q^T (B operands) as fp16 hi + lo: column col = head of the group (< 4)
  h8 bhi[4], blo[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      bhi[kk][j] = (_Float16)0.0f;
      blo[kk][j] = (_Float16)0.0f;
    }
    if (col < kAttnGroup) {
      const f32x4* qp = reinterpret_cast<const f32x4*>(
          q + (int64_t)s * ld_q + (int64_t)(g * kAttnGroup + col) * HD + 32 * kk + 8 * kg);
      const f32x4 a = qp[0], b = qp[1];
      const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const _Float16 hi = (_Float16)x[j];
        bhi[kk][j] = hi;
        blo[kk][j] = (_Float16)fsub(x[j], (float)hi);
      }
    }
  }
  // ---- scores: D[key][head] per 16-key tile; lane holds keys 16t + 4*kg + r of head col
  float z[4][4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    f32x4v acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const h8 av = __builtin_bit_cast(h8, ka[t][kk]);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bhi[kk], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, blo[kk], acc, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int jl = wave * 64 + 16 * t + 4 * kg + r;
      z[t][r] = jl < nk ? fmul(acc[r], scale) : -INFINITY;
    }
  }
  // ---- this wave's softmax partial, per head (lanes with col < 4 carry heads)
  float mw = -INFINITY;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) mw = fmaxf(mw, z[t][r]);
  mw = cross_row_max(mw);
  float lw = 0.0f;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float pz = z[t][r] == -INFINITY ? 0.0f : expf(fsub(z[t][r], mw));
      lw = fadd(lw, pz);
      if (col < kAttnGroup) s_p[wave][16 * t + 4 * kg + r][col] = pz;
    }
  lw = cross_row_sum_fixed(lw);
  if (lane < kAttnGroup) {
    s_m[wave][lane] = mw;
    s_l[wave][lane] = lw;
  }
  __syncthreads();

  // ---- weighted values of this wave's keys
  float o[kAttnGroup][8];
#pragma unroll
  for (int hh = 0; hh < kAttnGroup; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[hh][e] = 0.0f;
#pragma unroll
  for (int step = 0; step < 16; ++step) {
    const int kl = step * 4 + kslot;
    if (wave * 64 + kl < nk) {
      float vf[8];
      unpack8(vv[step], vf);
      const f32x4 pw = *reinterpret_cast<const f32x4*>(&s_p[wave][kl][0]);
      const float pr[4] = {pw.x, pw.y, pw.z, pw.w};
#pragma unroll
      for (int hh = 0; hh < kAttnGroup; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[hh][e] = ffma(pr[hh], vf[e], o[hh][e]);
    }
  }
#pragma unroll
  for (int hh = 0; hh < kAttnGroup; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[hh][e] = cross_row_sum_fixed(o[hh][e]);
  if (kslot == 0)
#pragma unroll
    for (int hh = 0; hh < kAttnGroup; ++hh)
#pragma unroll
      for (int e = 0; e < 8; ++e) s_o[wave][hh * HD + 8 * dg + e] = o[hh][e];
  __syncthreads();

  // ---- merge the four wave partials in wave order
  for (int idx = tid; idx < kAttnGroup * HD; idx += 256) {
    const int hh = idx / HD;
    const int d = idx - hh * HD;
    const float M = fmaxf(fmaxf(s_m[0][hh], s_m[1][hh]), fmaxf(s_m[2][hh], s_m[3][hh]));
    float O = 0.0f, L = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float e = s_m[w][hh] == -INFINITY ? 0.0f : expf(fsub(s_m[w][hh], M));
      O = fadd(O, fmul(s_o[w][idx], e));
      L = fadd(L, fmul(s_l[w][hh], e));
    }
    const int h = g * kAttnGroup + hh;
    float* dst = part + ((int64_t)A.partial_begin + (int64_t)h * A.n_chunks + c) * PF;
    dst[4 + d] = O;
    if (d == 0) {
      dst[0] = M;
      dst[1] = L;
    }
  }
}

// Grid (n_seq * H_q), 256 threads.  Merges the chunk partials of one
// (sequence, head): M = max_c m_c; w_c = exp(m_c - M); L = sum_c l_c w_c by a
// fixed tree over chunk index; O[d] = sum_c o_c[d] w_c with chunks split into
// two interleaved halves (threads 0..127 take even chunks, 128..255 odd ones,
// each in chunk order) that are then added.  Every shape depends only on the
// sequence's chunk count.  Optionally also emits the q8 blocks of the output
// row (the quantized input of the output projection).
constexpr int kMaxChunks = SD_MAX_CTX / SD_ATTN_CHUNK;

__global__ __launch_bounds__(256) void k_attn_combine(SeqArgs seqs, int H_q,
                                                      const float* __restrict__ part,
                                                      float* __restrict__ out, int8_t* oq, float* od) {
  __shared__ float s_w[kMaxChunks];
  __shared__ float s_red[256];
  __shared__ float s_o[HD];
  const int s = blockIdx.x / H_q;
  const int h = blockIdx.x - s * H_q;
  const int tid = threadIdx.x;
  const SeqArg& A = seqs.s[s];
  const int nc = A.n_chunks;
  const float* base = part + ((int64_t)A.partial_begin + (int64_t)h * nc) * PF;

  // maximum of the chunk maxima (exact, order-free)
  float mx = -INFINITY;
  for (int c = tid; c < nc; c += 256) mx = fmaxf(mx, base[(int64_t)c * PF]);
  mx = group_max<64>(mx);
  if ((tid & 63) == 0) s_red[tid >> 6] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  __syncthreads();
  // weights, and L by a fixed tree: thread partials over c = tid, tid+256, ...
  float lp = 0.0f;
  for (int c = tid; c < nc; c += 256) {
    const float w = expf(fsub(base[(int64_t)c * PF], M));
    s_w[c] = w;
    lp = fadd(lp, fmul(base[(int64_t)c * PF + 1], w));
  }
  lp = wave_sum_fixed(lp);
  if ((tid & 63) == 0) s_red[tid >> 6] = lp;
  __syncthreads();
  const float L = fadd(fadd(s_red[0], s_red[1]), fadd(s_red[2], s_red[3]));
  // values: two interleaved halves of the chunks, each in chunk order
  const int d = tid & (HD - 1);
  const int half = tid >> 7;
  float O = 0.0f;
  {
    int c = half;
    for (; c + 6 < nc; c += 8) {
      const float a0 = base[(int64_t)c * PF + 4 + d];
      const float a1 = base[(int64_t)(c + 2) * PF + 4 + d];
      const float a2 = base[(int64_t)(c + 4) * PF + 4 + d];
      const float a3 = base[(int64_t)(c + 6) * PF + 4 + d];
      O = fadd(O, fmul(a0, s_w[c]));
      O = fadd(O, fmul(a1, s_w[c + 2]));
      O = fadd(O, fmul(a2, s_w[c + 4]));
      O = fadd(O, fmul(a3, s_w[c + 6]));
    }
    for (; c < nc; c += 2) O = fadd(O, fmul(base[(int64_t)c * PF + 4 + d], s_w[c]));
  }
  if (half == 1) s_o[d] = O;
  __syncthreads();
  if (half == 0) {
    const float v = fdiv(fadd(O, s_o[d]), L);
    const int64_t idx = ((int64_t)s * H_q + h) * HD + d;
    out[idx] = v;
    if (oq) {
      const float amax = group_max<32>(fabsf(v));
      const float dd = q8_scale(amax);
      oq[idx] = (int8_t)q8_code(v, dd);
      if ((d & 31) == 0) od[idx >> 5] = dd;
    }
  }
}

}  // namespace

size_t attn_layout(SeqArgs* a, int H_q, int H_kv) {
  int units = 0, parts = 0;
  for (int s = 0; s < a->n_seq; ++s) {
    SeqArg& x = a->s[s];
    x.n_chunks = (x.ctx_len + C - 1) / C;
    x.unit_begin = units;
    x.partial_begin = parts;
    units += x.n_chunks * (H_q / kAttnGroup);
    parts += x.n_chunks * H_q;
  }
  (void)H_kv;
  return (size_t)parts * PF;
}

hipError_t launch_attn(const float* q, int64_t ld_q, const SeqArgs& seqs, int H_q, int H_kv,
                       float scale, float* out, float* partials, int8_t* oq, float* od,
                       hipStream_t st) {
  int units = 0;
  for (int s = 0; s < seqs.n_seq; ++s) units += seqs.s[s].n_chunks * H_kv;
  hipLaunchKernelGGL(k_attn_chunk, dim3(units), dim3(256), 0, st, q, ld_q, seqs, H_q, scale, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_attn_combine, dim3(seqs.n_seq * H_q), dim3(256), 0, st, seqs, H_q, partials,
                     out, oq, od);
  return hipGetLastError();
}

}  // namespace sd
