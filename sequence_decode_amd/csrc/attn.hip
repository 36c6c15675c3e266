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
//   arithmetic.  Scores and the weighted value sum both come from MFMA (fp16
//   keys and values as stored, the fp32 query and the fp32 weights as exact
//   fp16 hi + lo pairs, fp32 accumulation).
// * Each wave keeps its own softmax partial over its 64 keys, and the four
//   merge in wave order: partial (m, l, o[128]) per head and chunk.
// * A sequence may bring up to four query tokens, its newest positions (the
//   packed verification of proposed tokens in "feat(qwen36): complete
//   concurrent serving implementation with speculation"): token i at position
//   p_i sees keys 0..p_i.  The four heads of a group times up to four tokens are
//   the 16 columns of the MFMA tiles, and each column keeps its own key limit
//   and its own chunk count ceil((p_i + 1) / SD_ATTN_CHUNK), so token i gets
//   bitwise what a one-token call over p_i + 1 keys gives.
// * Caches: plain (position j in row j), ring (row j % capacity, with a
//   sliding window), or paged (a per-sequence block table into a shared pool,
//   "feat(qwen36): complete concurrent serving implementation with
//   speculation", "Summary").  Which rows hold the keys does not enter any
//   sum, so the three give the same bits for the same keys.
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

__device__ __forceinline__ int find_seq(const SeqArgs& a, int u) {
  int s = 0;
#pragma unroll
  for (int i = 1; i < SD_MAX_SEQS; ++i)
    if (i < a.n_seq && u >= a.s[i].unit_begin) s = i;
  return s;
}

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef short s4 __attribute__((ext_vector_type(4)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr;
typedef __attribute__((address_space(3))) s4* lds_s4_ptr;

__device__ __forceinline__ float cross_row_max(float v) {
  auto p = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, v),
                                            __builtin_bit_cast(uint32_t, v), false, false);
  v = fmaxf(__builtin_bit_cast(float, (uint32_t)p[0]), __builtin_bit_cast(float, (uint32_t)p[1]));
  auto q = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, v),
                                            __builtin_bit_cast(uint32_t, v), false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)q[0]), __builtin_bit_cast(float, (uint32_t)q[1]));
}

// fp32 x as the fp16 pair (hi, lo) with hi + lo = x to about 2^-22 |x|.
__device__ __forceinline__ void split_f16(float x, _Float16& hi, _Float16& lo) {
  hi = (_Float16)x;
  lo = (_Float16)fsub(x, (float)hi);
}

// Byte layout of one wave's V rows in LDS: row r (64 keys, 256 B each) keeps
// its eight 32-byte segments at positions seg ^ vswz(r).  The permutation makes
// the transposed reads below conflict-free: the 32 lanes of a half-wave read
// eight rows whose swizzles differ, so their 32-byte pieces land on disjoint
// banks.
constexpr int kRowBytes = HD * 2;
constexpr int kWaveKeys = 64;
constexpr int kWaveVBytes = kWaveKeys * kRowBytes;
__device__ __forceinline__ int vswz(int r) { return (r & 3) | ((r >> 1) & 4); }

// One workgroup = (sequence, KV head g, chunk of C keys); wave w owns keys
// 64w .. 64w+63 of the chunk.  Both contractions run on v_mfma_f32_16x16x32_f16
// with the four query heads of the group as the first 4 of 16 columns:
//  * scores S^T = K q^T: A = 16 keys x 32 dims of K (fp16 as stored), B = q^T as
//    the exact fp16 pair hi + lo of the fp32 query.  Tile t = (key block b =
//    t/2, half = t%2) puts key 32b + 8(m/4) + 4 half + m%4 in row m, so that a
//    lane's score slots are already the key slots of the P^T operand below.
//  * the chunk's softmax uses one maximum per head, shared by the four waves
//    through LDS, so the wave partials add without rescaling.
//  * weighted values O^T = V^T P^T: A = 16 dims x 32 keys of V^T, read from the
//    LDS copy of the wave's V rows with ds_read_b64_tr_b16 (each 16-lane group
//    gathers 4 keys x 4 dims per read), B = the weights as fp16 hi + lo.
// The four wave partials are added in wave order.  Keys past the end of the
// sequence get weight 0; their V rows are clamped to the last key, so every
// product that enters a sum is finite.
__global__ __launch_bounds__(256) void k_attn_chunk(const float* __restrict__ q, int64_t ld_q,
                                                    SeqArgs seqs, int H_q, float scale,
                                                    float* __restrict__ part) {
  __shared__ __attribute__((aligned(1024))) uint8_t s_v[4 * kWaveVBytes];  // V rows, then O partials
  __shared__ float s_m[4][16], s_l[4][16];  // per wave and MFMA column (token, head)

  const int s = find_seq(seqs, blockIdx.x);
  const SeqArg& A = seqs.s[s];
  const int local = blockIdx.x - A.unit_begin;
  const int g = local / A.n_chunks;
  const int ci = local - g * A.n_chunks;  // chunk of this unit, counted from c0
  const int c = A.c0 + ci;                // absolute chunk: positions c*C .. c*C + C-1
  const int j0 = c * C;
  const int nk = min(C, A.ctx_len - j0);  // keys of the chunk below ctx_len
  const int jlo = max(0, A.lo0 - j0);     // keys of the chunk below any query's window
  // ring caches: row of chunk key jl (jlo <= jl < nk) runs on from that of jlo
  // and wraps once at the ring's end (the keys in use span at most the ring)
  auto krow = [&](int prow0, int jl) {
    const int r = prow0 + (jl - jlo);
    return r >= A.ring_cap ? r - A.ring_cap : r;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int col = lane & 15;  // MFMA row (A loads) / column (B, D)
  const int kg = lane >> 4;   // MFMA k-group
  const int wk = wave * kWaveKeys;
  // MFMA column col = 4 * (burst token) + (head in the group); token tk sits at
  // position p = ctx_len - T + tk and sees the keys from max(0, p - window + 1)
  // (or 0) up to p
  const int T = A.n_new;
  const int tk = col >> 2;
  const int hh = col & (kAttnGroup - 1);
  const bool colv = tk < T;
  const int p_col = A.ctx_len - T + tk;
  const int nk_col = colv ? min(C, p_col + 1 - j0) : 0;
  const int jlo_col = A.window ? max(0, p_col - A.window + 1) - j0 : 0;

  // ---- K (score A operands): tile t, row col -> key wk + 32b + 8(col/4) + 4half + col%4
  const int jk = wk + 8 * (col >> 2) + (col & 3);
  const uint16_t* kb = A.k + (int64_t)g * A.ld_head + 8 * kg;
  // plain caches: row = position, so tile t's rows are a fixed stride apart.
  // Keys outside jlo .. nk-1 read the nearest key in use: their scores are
  // replaced by -inf below, so what they load does not matter (it is finite).
  const bool lin = A.ring_cap == 0;
  // plain and paged caches: the wave's 64 positions j0 + wk + x are the 64
  // consecutive rows jrow + wk + x (a block holds a multiple of 64 positions and
  // chunks start at multiples of C); jlast is the row of the chunk's last key.
  // A wave wholly past the end loads no K and reads V from jlast only.
  int64_t jrow = j0, jlast = j0 + nk - 1;
  if (A.btab) {
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    jlast = seq_row(A, j0 + nk - 1);
    jrow = wv * kWaveKeys < nk ? seq_row(A, j0 + wv * kWaveKeys) - wv * kWaveKeys : jlast;
  }
  u32x4a ka[4][4];
  if (__builtin_expect(lin, 1)) {
    // plain / paged cache: tile t's rows a fixed stride apart; keys past the end
    // load zeros, keys below a window are real rows (masked below)
    const uint16_t* kr = kb + (jrow + jk) * A.ld_tok;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int dj = 32 * (t >> 1) + 4 * (t & 1);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        ka[t][kk] = u32x4a{0u, 0u, 0u, 0u};
        if (jk + dj < nk) ka[t][kk] = *reinterpret_cast<const u32x4a*>(kr + dj * A.ld_tok + 32 * kk);
      }
    }
  } else {
    // ring: keys outside jlo .. nk-1 read the nearest key in use (their scores
    // are replaced by -inf below)
    const int prow0 = (j0 + jlo) % A.ring_cap;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int jl = jk + 32 * (t >> 1) + 4 * (t & 1);
      const uint16_t* kr = kb + (int64_t)krow(prow0, min(max(jl, jlo), nk - 1)) * A.ld_tok;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) ka[t][kk] = *reinterpret_cast<const u32x4a*>(kr + 32 * kk);
    }
  }
  // ---- q (score B operands): column col = (token tk, head g*4 + hh), dims 32kk + 8kg ..
  f32x4 qv[4][2];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    qv[kk][0] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    qv[kk][1] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    if (colv) {
      const f32x4* qp = reinterpret_cast<const f32x4*>(
          q + (int64_t)(A.row0 + tk) * ld_q + (int64_t)(g * kAttnGroup + hh) * HD + 32 * kk + 8 * kg);
      qv[kk][0] = qp[0];
      qv[kk][1] = qp[1];
    }
  }
  // ---- V rows of this wave -> LDS by DMA: instruction i fills rows 4i .. 4i+3;
  // lane l writes row 4i + l/16 at 16-byte position l%16, which holds the row's
  // 16-byte piece (l%16) ^ 2 vswz(row).
  uint8_t* vw = s_v + wave * kWaveVBytes;
  {
    // keys past the end read the last key, and in a ring keys below jlo read
    // key jlo (their weight is 0); a plain cache's keys below a window are
    // real rows and read as they are
    const uint16_t* vbase = A.v + (int64_t)g * A.ld_head;
    const int jv = wk + (lane >> 4);
    if (__builtin_expect(lin, 1)) {
      const uint8_t* v0 = reinterpret_cast<const uint8_t*>(vbase + (jrow + jv) * A.ld_tok);
      const uint8_t* vlast = reinterpret_cast<const uint8_t*>(vbase + jlast * A.ld_tok);
      const int64_t step4 = 4 * A.ld_tok * 2;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = 4 * i + (lane >> 4);
        const int piece = (lane & 15) ^ (2 * vswz(r));
        const uint8_t* row = jv + 4 * i < nk ? v0 + i * step4 : vlast;
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(row + 16 * piece), (lds_ptr)(vw + i * 1024), 16, 0, 0);
      }
    } else {
      const int prow0 = (j0 + jlo) % A.ring_cap;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = 4 * i + (lane >> 4);
        const int piece = (lane & 15) ^ (2 * vswz(r));
        const int jl = min(max(jv + 4 * i, jlo), nk - 1);
        const uint8_t* row = reinterpret_cast<const uint8_t*>(vbase + (int64_t)krow(prow0, jl) * A.ld_tok);
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(row + 16 * piece), (lds_ptr)(vw + i * 1024), 16, 0, 0);
      }
    }
  }

  // ---- scores
  h8 bhi[4], blo[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const float x[8] = {qv[kk][0].x, qv[kk][0].y, qv[kk][0].z, qv[kk][0].w,
                        qv[kk][1].x, qv[kk][1].y, qv[kk][1].z, qv[kk][1].w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      _Float16 hi, lo;
      split_f16(x[j], hi, lo);
      bhi[kk][j] = hi;
      blo[kk][j] = lo;
    }
  }
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
    // D slot r of this lane = row 4kg + r = key wk + 32(t/2) + 8kg + 4(t%2) + r, head col
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int jl = wk + 32 * (t >> 1) + 8 * kg + 4 * (t & 1) + r;
      z[t][r] = (jl < nk_col && jl >= jlo_col) ? fmul(acc[r], scale) : -INFINITY;
    }
  }
  // ---- the chunk maximum per column, shared by the four waves
  {
    float mw = -INFINITY;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) mw = fmaxf(mw, z[t][r]);
    mw = cross_row_max(mw);
    if (lane < 16) s_m[wave][lane] = mw;
  }
  __syncthreads();
  const float M = fmaxf(fmaxf(s_m[0][col], s_m[1][col]), fmaxf(s_m[2][col], s_m[3][col]));
  // ---- weights, their sum, and the P^T operands (block b: slot j = tile 2b + j/4, slot j%4)
  h8 phi[2], plo[2];
  float lw = 0.0f;
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float pz = z[t][r] == -INFINITY ? 0.0f : expf(fsub(z[t][r], M));
      lw = fadd(lw, pz);
      _Float16 hi, lo;
      split_f16(pz, hi, lo);
      phi[t >> 1][4 * (t & 1) + r] = hi;
      plo[t >> 1][4 * (t & 1) + r] = lo;
    }
  lw = cross_row_sum_fixed(lw);
  if (lane < 16) s_l[wave][lane] = lw;

  // ---- weighted values: this wave's V rows have landed in LDS
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  // lane (col, kg) reads row 32b + 8kg + 4h + col/4, dims 16dt + 4(col%4) .. +3
  const int vg = vswz(8 * kg + (col >> 2));
  const int rbase = (8 * kg + (col >> 2)) * kRowBytes + 8 * (col & 3);
  f32x4v o[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    o[dt] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
    const int a0 = rbase + ((dt ^ vg) << 5);
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const s4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s4_ptr)((__attribute__((address_space(3))) uint8_t*)vw + a0 + b * 32 * kRowBytes));
      const s4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s4_ptr)((__attribute__((address_space(3))) uint8_t*)vw + a0 + b * 32 * kRowBytes + 4 * kRowBytes));
      const h8 av = __builtin_bit_cast(h8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, phi[b], o[dt], 0, 0, 0);
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, plo[b], o[dt], 0, 0, 0);
    }
  }
  // D slot r of lane (col, kg) = dim 16dt + 4kg + r of column col; the wave's
  // own V region (now read) takes its partial O[column][dim]
  float* so = reinterpret_cast<float*>(vw);
  if (colv)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
      *reinterpret_cast<f32x4*>(so + col * HD + 16 * dt + 4 * kg) =
          f32x4{o[dt][0], o[dt][1], o[dt][2], o[dt][3]};
  __syncthreads();

  // ---- sum of the four wave partials, in wave order, for each column whose
  // token reaches this chunk
  for (int idx = tid; idx < T * kAttnGroup * HD; idx += 256) {
    const int cc = idx / HD;
    const int d = idx - cc * HD;
    const int t2 = cc >> 2;
    const int p2 = A.ctx_len - T + t2;
    if (j0 > p2) continue;  // chunk past this token's position
    if (A.window && j0 + C <= p2 - A.window + 1) continue;  // chunk before its window
    float O = 0.0f, L = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      O = fadd(O, reinterpret_cast<const float*>(s_v + w * kWaveVBytes)[idx]);
      L = fadd(L, s_l[w][cc]);
    }
    const float Mh = fmaxf(fmaxf(s_m[0][cc], s_m[1][cc]), fmaxf(s_m[2][cc], s_m[3][cc]));
    const int h = g * kAttnGroup + (cc & (kAttnGroup - 1));
    float* dst = part + ((int64_t)A.partial_begin + ((int64_t)t2 * H_q + h) * A.n_chunks + ci) * PF;
    dst[4 + d] = O;
    if (d == 0) {
      dst[0] = Mh;
      dst[1] = L;
    }
  }
}

// Grid (query rows * H_q), 256 threads.  Merges the chunk partials of one
// (sequence, token, head) -- its chunks are those up to the token's position: M = max_c m_c; w_c = exp(m_c - M); L = sum_c l_c w_c by a
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
  const int row = blockIdx.x / H_q;
  const int h = blockIdx.x - row * H_q;
  const int tid = threadIdx.x;
  int s = 0;
#pragma unroll
  for (int i = 1; i < SD_MAX_SEQS; ++i)
    if (i < seqs.n_seq && row >= seqs.s[i].row0) s = i;
  const SeqArg& A = seqs.s[s];
  const int t = row - A.row0;
  const int p = A.ctx_len - A.n_new + t;
  const int lo = A.window ? max(0, p - A.window + 1) : 0;
  const int nc = p / C - lo / C + 1;  // this token's chunks: those of positions lo..p
  const float* base =
      part + ((int64_t)A.partial_begin + ((int64_t)t * H_q + h) * A.n_chunks + (lo / C - A.c0)) * PF;

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
    const int64_t idx = ((int64_t)row * H_q + h) * HD + d;
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
  int units = 0, parts = 0, rows = 0;
  for (int s = 0; s < a->n_seq; ++s) {
    SeqArg& x = a->s[s];
    x.lo0 = x.window ? (x.ctx_len - x.n_new - x.window + 1 > 0 ? x.ctx_len - x.n_new - x.window + 1 : 0) : 0;
    x.c0 = x.lo0 / C;
    x.n_chunks = (x.ctx_len - 1) / C - x.c0 + 1;
    x.unit_begin = units;
    x.partial_begin = parts;
    x.row0 = rows;
    units += x.n_chunks * (H_q / kAttnGroup);
    parts += x.n_chunks * H_q * x.n_new;
    rows += x.n_new;
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
  int rows = 0;
  for (int s = 0; s < seqs.n_seq; ++s) rows += seqs.s[s].n_new;
  hipLaunchKernelGGL(k_attn_combine, dim3(rows * H_q), dim3(256), 0, st, seqs, H_q, partials,
                     out, oq, od);
  return hipGetLastError();
}

}  // namespace sd
