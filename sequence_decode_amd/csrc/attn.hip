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
//   query heads that share the KV head.  Lane = 16 * key_slot + dim_group: a
//   wave reads four 256-byte key rows per instruction (16 B per lane), and each
//   lane keeps its 8 query dims of the 4 heads in registers.  fp16 K/V enter
//   fp32 FMAs directly (v_fma_mix), with no conversion pass.
// * Two passes over the chunk (scores, then values) with the chunk maximum in
//   between, so no running rescale; partial (m, l, o[128]) per head and chunk.
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

__global__ __launch_bounds__(256) void k_attn_chunk(const float* __restrict__ q, int64_t ld_q,
                                                    SeqArgs seqs, int H_q, float scale,
                                                    float* __restrict__ part) {
  __shared__ f32x4 s_z[C];            // scores, then weights: [key][head of the group]
  __shared__ float s_red[2][4][4];    // [max|sum][wave][head]
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
  const int kslot = lane >> 4;
  const int dg = lane & 15;

  // query dims 8*dg .. 8*dg+7 of the four heads of group g
  float qv[kAttnGroup][8];
#pragma unroll
  for (int hh = 0; hh < kAttnGroup; ++hh) {
    const f32x4* qp = reinterpret_cast<const f32x4*>(q + (int64_t)s * ld_q +
                                                     (int64_t)(g * kAttnGroup + hh) * HD + 8 * dg);
    const f32x4 a = qp[0], b = qp[1];
    qv[hh][0] = a.x; qv[hh][1] = a.y; qv[hh][2] = a.z; qv[hh][3] = a.w;
    qv[hh][4] = b.x; qv[hh][5] = b.y; qv[hh][6] = b.z; qv[hh][7] = b.w;
  }
  const uint16_t* kbase = A.k + (int64_t)g * A.ld_head + 8 * dg;
  const uint16_t* vbase = A.v + (int64_t)g * A.ld_head + 8 * dg;
  constexpr int STEPS = C / 16;  // keys of one lane: wave * 64 + step * 4 + kslot

  // All key and value rows of this lane are requested before any arithmetic, so
  // the workgroup waits for one memory latency rather than one per step.
  u32x4a kk[STEPS], vv[STEPS];
#pragma unroll
  for (int step = 0; step < STEPS; ++step) {
    const int jl = wave * 64 + step * 4 + kslot;
    kk[step] = u32x4a{0u, 0u, 0u, 0u};
    if (jl < nk) kk[step] = *reinterpret_cast<const u32x4a*>(kbase + (int64_t)(j0 + jl) * A.ld_tok);
  }
#pragma unroll
  for (int step = 0; step < STEPS; ++step) {
    const int jl = wave * 64 + step * 4 + kslot;
    vv[step] = u32x4a{0u, 0u, 0u, 0u};
    if (jl < nk) vv[step] = *reinterpret_cast<const u32x4a*>(vbase + (int64_t)(j0 + jl) * A.ld_tok);
  }

  // ---- pass 1: scores
#pragma unroll
  for (int step = 0; step < STEPS; ++step) {
    const int jl = wave * 64 + step * 4 + kslot;
    const bool valid = jl < nk;
    float kf[8];
    unpack8(kk[step], kf);
    float pz[kAttnGroup];
#pragma unroll
    for (int hh = 0; hh < kAttnGroup; ++hh) {
      float acc = fmul(qv[hh][0], kf[0]);
#pragma unroll
      for (int e = 1; e < 8; ++e) acc = ffma(qv[hh][e], kf[e], acc);
      pz[hh] = acc;
    }
#pragma unroll
    for (int hh = 0; hh < kAttnGroup; ++hh) pz[hh] = row16_sum_fixed(pz[hh]);
    if (dg == 0) {
      f32x4 z;
      z.x = valid ? fmul(pz[0], scale) : -INFINITY;
      z.y = valid ? fmul(pz[1], scale) : -INFINITY;
      z.z = valid ? fmul(pz[2], scale) : -INFINITY;
      z.w = valid ? fmul(pz[3], scale) : -INFINITY;
      s_z[jl] = z;
    }
  }
  __syncthreads();

  // ---- chunk maximum and weights (thread tid owns key tid)
  f32x4 z = s_z[tid];
  float mx[4] = {z.x, z.y, z.z, z.w};
#pragma unroll
  for (int hh = 0; hh < 4; ++hh) mx[hh] = group_max<64>(mx[hh]);
  if (lane == 0)
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) s_red[0][wave][hh] = mx[hh];
  __syncthreads();
  float m[4], p[4], l[4];
#pragma unroll
  for (int hh = 0; hh < 4; ++hh) {
    m[hh] = fmaxf(fmaxf(s_red[0][0][hh], s_red[0][1][hh]), fmaxf(s_red[0][2][hh], s_red[0][3][hh]));
  }
  p[0] = expf(fsub(z.x, m[0]));
  p[1] = expf(fsub(z.y, m[1]));
  p[2] = expf(fsub(z.z, m[2]));
  p[3] = expf(fsub(z.w, m[3]));
#pragma unroll
  for (int hh = 0; hh < 4; ++hh) l[hh] = wave_sum_fixed(p[hh]);
  if (lane == 0)
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) s_red[1][wave][hh] = l[hh];
  {
    f32x4 pw;
    pw.x = p[0]; pw.y = p[1]; pw.z = p[2]; pw.w = p[3];
    s_z[tid] = pw;
  }
  __syncthreads();

  // ---- pass 2: weighted values
  float o[kAttnGroup][8];
#pragma unroll
  for (int hh = 0; hh < kAttnGroup; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[hh][e] = 0.0f;
#pragma unroll
  for (int step = 0; step < STEPS; ++step) {
    const int jl = wave * 64 + step * 4 + kslot;
    if (jl < nk) {
      float vf[8];
      unpack8(vv[step], vf);
      const f32x4 pw = s_z[jl];
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

  for (int idx = tid; idx < kAttnGroup * HD; idx += 256) {
    const int hh = idx / HD;
    const int d = idx - hh * HD;
    const float v = fadd(fadd(s_o[0][idx], s_o[1][idx]), fadd(s_o[2][idx], s_o[3][idx]));
    const int h = g * kAttnGroup + hh;
    float* dst = part + ((int64_t)A.partial_begin + (int64_t)h * A.n_chunks + c) * PF;
    dst[4 + d] = v;
    if (d == 0) {
      dst[0] = m[hh];
      dst[1] = fadd(fadd(s_red[1][0][hh], s_red[1][1][hh]), fadd(s_red[1][2][hh], s_red[1][3][hh]));
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
