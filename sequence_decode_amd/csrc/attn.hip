// attn.hip -- multi-sequence grouped-query decode attention.
//
// What it computes: ds4 pull request 604, "Commit walkthrough / CUDA kernels"
// (one query token per sequence, each attending to its own cache; the
// per-sequence views travel by value in the kernel arguments, at most four),
// in one launch for all sequences ("2. Single-GPU decode batches don't
// scale").  The layout here is CDNA4's own:
//
// * Work unit = (sequence, KV head, chunk).  Chunks sit on a grid fixed in
//   absolute positions: 64 keys below position 2048, 256 keys beyond, so how
//   a token's keys are split depends on its position alone.  The grid is the
//   sum of all sequences' units.  One CU streams only about 1/256 of the
//   chip's HBM rate, so a short context must spread over many CUs: 2050 keys
//   make 33 chunks x 8 KV heads = 264 workgroups of 32 KB each (with 256-key
//   chunks: 72 of 128 KB, on 72 CUs); long contexts keep 256-key chunks, whose
//   partials cost 3% of the cache bytes instead of 12%.
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
//   and its own chunks (those of positions 0..p_i), so token i gets bitwise
//   what a one-token call over p_i + 1 keys gives.
// * Caches: plain (position j in row j), ring (row j % capacity, with a
//   sliding window), or paged (a per-sequence block table into a shared pool,
//   "feat(qwen36): complete concurrent serving implementation with
//   speculation", "Summary").  Which rows hold the keys does not enter any
//   sum, so the three give the same bits for the same keys.
// * A second kernel merges the partials of each (sequence, head) with fixed
//   reduction shapes.  Every sum has a fixed shape, so a sequence's output bits do not
//   depend on the other sequences in the call.
#include <math.h>

#include <mutex>
#include <type_traits>

#include "device_math.hpp"
#include "internal.hpp"

namespace sd {

namespace {

constexpr int HD = kAttnHeadDim;
constexpr int PF = kAttnPartialFloats;

// Sequence of workgroup b: 256-key units first (every sequence's, from
// large_begin), then the 64-key ones (from small_begin).
__device__ __forceinline__ int find_seq(const SeqArgs& a, int b, bool large) {
  int s = 0;
#pragma unroll
  for (int i = 1; i < SD_MAX_SEQS; ++i)
    if (i < a.n_seq && b >= (large ? a.s[i].large_begin : a.s[i].small_begin)) s = i;
  return s;
}

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef short s4 __attribute__((ext_vector_type(4)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr;
typedef __attribute__((address_space(3))) s4* lds_s4_ptr;

// Cache policy of the V DMAs: non-temporal (nt).  In a decode step a layer's
// cache is read once between the rest of the model's bytes (several GB), so
// the 256 MB Infinity Cache never serves it again; with nt the four ragged
// contexts' step runs about 1.5% faster.  (K stays on the default policy: nt
// there gained nothing more.)
constexpr int kVCpol = 2;

__device__ __forceinline__ float cross_row_max(float v) {
  auto p = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, v),
                                            __builtin_bit_cast(uint32_t, v), false, false);
  v = fmaxf(__builtin_bit_cast(float, (uint32_t)p[0]), __builtin_bit_cast(float, (uint32_t)p[1]));
  auto q = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, v),
                                            __builtin_bit_cast(uint32_t, v), false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)q[0]), __builtin_bit_cast(float, (uint32_t)q[1]));
}

// fp32 x as the fp16 pair (hi, lo) with hi + lo = x to about 2^-22 |x|.
// (x - hi is exact in fp32, so the fused form rounds it only once, to fp16.)
__device__ __forceinline__ void split_f16(float x, _Float16& hi, _Float16& lo) {
  hi = (_Float16)x;
  lo = (_Float16)__builtin_fmaf(-1.0f, (float)hi, x);
}

// exp(x) for x <= 0 as 2^(x log2 e) on the hardware exp2 (about 1e-6 relative
// over the weights that matter; weights below 2^-126 flush to 0).  One fixed
// instruction sequence, so a weight's bits depend on x alone.
__device__ __forceinline__ float exp_w(float x) {
  return __builtin_amdgcn_exp2f(fmul(x, 1.44269504088896341f));
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

// q8_0 caches: a wave's 64 code rows (128 bytes each) sit in LDS with their
// eight 16-byte segments at positions seg ^ vswz8(r); the transposed byte reads
// below then touch 16 distinct rows per half-wave at distinct bank offsets.
constexpr int kRowBytes8 = HD;
constexpr int kWaveVBytes8 = kWaveKeys * kRowBytes8;
__device__ __forceinline__ int vswz8(int r) { return (r & 7) ^ ((r >> 3) & 1); }

typedef uint32_t u32x2a __attribute__((ext_vector_type(2), aligned(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i32x2* lds_i32x2_ptr;

// Eight int8 codes (bytes of w0, then w1) as eight exact fp16 values: byte c
// becomes the fp16 with bits 0x6400 | (c ^ 0x80), i.e. 1152 + c, minus 1152.
__device__ __forceinline__ h8 codes_to_h8(uint32_t w0, uint32_t w1) {
  const uint32_t a0 = w0 ^ 0x80808080u, a1 = w1 ^ 0x80808080u;
  const h2 bias = {(_Float16)1152.0f, (_Float16)1152.0f};
  const h2 e0 = __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, a0, 0x04010400u)) - bias;
  const h2 e1 = __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, a0, 0x04030402u)) - bias;
  const h2 e2 = __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, a1, 0x04010400u)) - bias;
  const h2 e3 = __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, a1, 0x04030402u)) - bias;
  return h8{e0.x, e0.y, e1.x, e1.y, e2.x, e2.y, e3.x, e3.y};
}

// q4_0 caches: a 32-bit word of eight nibbles (dims 2j and 2j + 1 in byte j,
// the even dim low) as its bytes in dim order: {n0, n1, n2, n3}, {n4 .. n7}.
__device__ __forceinline__ void nibbles_to_bytes(uint32_t w, uint32_t& b0, uint32_t& b1) {
  const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
  b0 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
  b1 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
}

// Eight q4_0 nibbles n as the exact fp16 values n - 8: bits 0x6400 | n is
// 1024 + n, minus 1032.
__device__ __forceinline__ h8 nibbles_to_h8(uint32_t w) {
  uint32_t b0, b1;
  nibbles_to_bytes(w, b0, b1);
  const h2 bias = {(_Float16)1032.0f, (_Float16)1032.0f};
  const h2 e0 = __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, b0, 0x04010400u)) - bias;
  const h2 e1 = __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, b0, 0x04030402u)) - bias;
  const h2 e2 = __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, b1, 0x04010400u)) - bias;
  const h2 e3 = __builtin_bit_cast(h2, __builtin_amdgcn_perm(0x64646464u, b1, 0x04030402u)) - bias;
  return h8{e0.x, e0.y, e1.x, e1.y, e2.x, e2.y, e3.x, e3.y};
}

// Eight nibbles as the int8 codes n - 8 (per byte: n + 0x78 stays below 0x100,
// and flipping its top bit gives n - 8 in two's complement).
__device__ __forceinline__ void nibbles_to_codes(uint32_t w, uint32_t& c0, uint32_t& c1) {
  uint32_t b0, b1;
  nibbles_to_bytes(w, b0, b1);
  c0 = (b0 + 0x78787878u) ^ 0x80808080u;
  c1 = (b1 + 0x78787878u) ^ 0x80808080u;
}

// One workgroup = (sequence, KV head g, chunk); wave w owns keys 64w .. 64w+63
// of the chunk (a chunk of at most 64 keys is one wave's).  Both contractions run on v_mfma_f32_16x16x32_f16
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
// q8_0 caches (Q8): the codes enter the same MFMAs as exact fp16 values.  One
// MFMA's 32 dims are one q8_0 block, so each block's partial score is its own
// accumulation, scaled by the key's block scale and added in block order.  The
// value scales fold into the weights: the B operand of dim tile dt is the
// fp32 product p_j * d_j[dt/2] as fp16 hi + lo.  V^T comes from the codes in
// LDS by ds_read_b64_tr_b8 (each 16-lane group gathers 8 keys x 16 dims).
// q4_0 keys (K4) enter the same MFMAs through nibbles_to_h8 (lane (col, kg)
// loads the 4 bytes of dims 8kg .. 8kg+7 of each block); q4_0 values (V4) are
// loaded into registers and written to the wave's LDS region as the int8 codes
// n - 8 in the q8_0 layout, so the value contraction is that of q8_0 caches.
// The four wave partials are added in wave order.  Keys past the end of the
// sequence get weight 0; their V rows (and scales) are clamped to the last key,
// so every product that enters a sum is finite.
template <bool Q8, bool K4 = false, bool V4 = false>
__global__ __launch_bounds__(256) void k_attn_chunk(const float* __restrict__ q, int64_t ld_q,
                                                    SeqArgs seqs, int H_q, float scale,
                                                    float* __restrict__ part) {
  constexpr int kVB = Q8 ? kWaveVBytes8 : kWaveVBytes / 2;  // LDS bytes of a wave's V rows (then O partial)
  static_assert(16 * HD * 4 <= kVB, "a wave's O partial fits its V region");
  __shared__ __attribute__((aligned(1024))) uint8_t s_v[4 * kVB];  // V rows, then O partials
  __shared__ __attribute__((aligned(16))) uint32_t s_sc[Q8 ? 4 * 64 * 4 : 1];  // per wave and key: K, V scales
  __shared__ float s_m[4][16], s_l[4][16];  // per wave and MFMA column (token, head)

  // The grid holds every sequence's 256-key units first (the long-running
  // ones start first), then its 64-key units; within each, head group by head
  // group (a head group: seqs.hpw query heads of one KV head; seqs.vg groups
  // share each KV head).
  const bool large = (int)blockIdx.x < seqs.large_total;
  const int s = find_seq(seqs, blockIdx.x, large);
  const SeqArg& A = seqs.s[s];
  const int n_su = (A.ns + A.pk - 1) / A.pk;  // 64-key units per head group
  const int n_lu = A.n_chunks - A.ns;         // 256-key units per head group
  int hg, u;  // head group, and unit within it (64-key units first)
  if (large) {
    const int local = blockIdx.x - A.large_begin;
    hg = local / n_lu;
    u = n_su + (local - hg * n_lu);
  } else {
    const int local = blockIdx.x - A.small_begin;
    hg = local / n_su;
    u = local - hg * n_su;
  }
  const int hpw = seqs.hpw;    // query heads of the group (columns 4 tk + hh, hh < hpw)
  const int g = hg / seqs.vg;  // its KV head
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // The chunk of this wave.  Units 0 .. n_su-1 hold the chunks of the 64-key
  // grid, A.pk of them per unit (4: one per wave; 1: wave 0's alone), the units
  // after them one chunk each.  A chunk with at most 64 keys below ctx_len is
  // one wave's ("small"): that wave keeps its softmax partial to itself (no
  // barrier, no cross-wave sums) and the waves without a chunk leave at once.
  // Which unit or wave computes a chunk changes no bits of its partial.
  const bool packed = u < n_su && A.pk == 4;
  const int ci = u < n_su ? u * A.pk + (packed ? wave : 0) : A.ns + (u - n_su);  // counted from c0
  const int c = A.c0 + ci;                // absolute chunk: positions j0 .. j0 + csz - 1
  const int j0 = attn_chunk_begin(c);
  const int csz = attn_chunk_size(c);
  const int nk = min(csz, A.ctx_len - j0);  // keys of the chunk below ctx_len
  const bool small = packed || nk <= kWaveKeys;
  if (packed ? ci >= A.ns : small && wave != 0) return;
  // a small chunk's wave alone in its workgroup takes the next wave's V region
  // too and loads all its V rows at once
  const bool alone = small && !packed;
  // The rest is compiled twice: for small chunks and for four-wave ones, so
  // neither path carries the other's branches.
  auto body = [&](auto small_c) {
    constexpr bool SMALL = decltype(small_c)::value;
    const int jlo = max(0, A.lo0 - j0);     // keys of the chunk below any query's window
    // ring caches: row of chunk key jl (jlo <= jl < nk) runs on from that of jlo
    // and wraps once at the ring's end (the keys in use span at most the ring)
    auto krow = [&](int prow0, int jl) {
      const int r = prow0 + (jl - jlo);
      return r >= A.ring_cap ? r - A.ring_cap : r;
    };

    const int lane = tid & 63;
    const int col = lane & 15;  // MFMA row (A loads) / column (B, D)
    const int kg = lane >> 4;   // MFMA k-group
    const int wk = SMALL ? 0 : wave * kWaveKeys;  // first key of the wave within the chunk
    // MFMA column col = 4 * (burst token) + (head in the group); token tk sits at
    // position p = ctx_len - T + tk and sees the keys from max(0, p - window + 1)
    // (or 0) up to p
    const int T = A.n_new;
    const int tk = col >> 2;
    const int hh = col & (kAttnGroup - 1);
    const bool colv = tk < T && hh < hpw;
    const int p_col = A.ctx_len - T + tk;
    const int nk_col = colv ? min(csz, p_col + 1 - j0) : 0;
    const int jlo_col = A.window ? max(0, p_col - A.window + 1) - j0 : 0;

    // ---- K (score A operands): tile t, row col -> key wk + 32b + 8(col/4) + 4half + col%4
    const int jk = wk + 8 * (col >> 2) + (col & 3);
    const bool lin = A.ring_cap == 0;
    // plain and paged caches: the wave's 64 positions j0 + wk + x are the 64
    // consecutive rows jrow + wk + x (a block holds a multiple of 64 positions and
    // chunks start at multiples of 64); jlast is the row of the chunk's last key.
    // A wave wholly past the end loads no K and reads V from jlast only.
    int64_t jrow = j0, jlast = j0 + nk - 1;
    if (A.btab) {
      jlast = seq_row(A, j0 + nk - 1);
      jrow = wk < nk ? seq_row(A, j0 + wk) - wk : jlast;
    }
    // cache row of chunk key jl, clamped into the keys in use (V rows, scales)
    auto vrow = [&](int jl) -> int64_t {
      if (__builtin_expect(lin, 1)) return jl < nk ? jrow + jl : jlast;
      return krow((j0 + jlo) % A.ring_cap, min(max(jl, jlo), nk - 1));
    };
    uint8_t* vw = s_v + wave * kVB;
    // q4_0 values: lane l loads the 64 nibble bytes of the wave's key l (to LDS
    // as codes before the value contraction), issued first
    u32x4a v4r[4];
    if constexpr (V4) {
      const uint8_t* vr = reinterpret_cast<const uint8_t*>(A.vq) + (int64_t)g * (A.ld_head >> 1) +
                          vrow(wk + lane) * (A.ld_tok >> 1);
#pragma unroll
      for (int i = 0; i < 4; ++i) v4r[i] = *reinterpret_cast<const u32x4a*>(vr + 16 * i);
    }
    if constexpr (Q8 && !V4) {
      // ---- V code rows of this wave -> LDS by DMA, issued first (the scores
      // wait for every load of the wave): instruction i fills rows
      // 8i .. 8i+7; lane l writes row 8i + l/8 at 16-byte position l%8, which
      // holds the row's segment (l%8) ^ vswz8(row)
      const int8_t* vbase = A.vq + (int64_t)g * A.ld_head;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = 8 * i + (lane >> 3);
        const int seg = (lane & 7) ^ vswz8(r);
        const int8_t* row = vbase + vrow(wk + r) * A.ld_tok;
        __builtin_amdgcn_global_load_lds(static_cast<const void*>(row + 16 * seg), (lds_ptr)(vw + i * 1024), 16, 0, kVCpol);
      }
    }
    u32x4a ka[4][4];   // fp16 caches: 8 dims per (tile, block)
    u32x2a kc[4][4];   // q8_0 caches: 8 codes per (tile, block)
    if constexpr (!Q8) {
      const uint16_t* kb = A.k + (int64_t)g * A.ld_head + 8 * kg;
      if (__builtin_expect(lin, 1)) {
        // plain / paged cache: keys past the end read the last key, keys below a
        // window are real rows (both masked below)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int jl = jk + 32 * (t >> 1) + 4 * (t & 1);
          const uint16_t* kr = kb + (jl < nk ? jrow + jl : jlast) * A.ld_tok;
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) ka[t][kk] = *reinterpret_cast<const u32x4a*>(kr + 32 * kk);
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
    } else if constexpr (K4) {
      // q4_0 keys: the 4 bytes of dims 8kg .. 8kg+7 of block kk (in kc[t][kk].x)
      const uint8_t* kb = reinterpret_cast<const uint8_t*>(A.kq) + (int64_t)g * (A.ld_head >> 1) + 4 * kg;
      const int64_t kst = A.ld_tok >> 1;
      if (__builtin_expect(lin, 1)) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int jl = jk + 32 * (t >> 1) + 4 * (t & 1);
          const uint8_t* kr = kb + (jl < nk ? jrow + jl : jlast) * kst;
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) kc[t][kk] = u32x2a{*reinterpret_cast<const uint32_t*>(kr + 16 * kk), 0u};
        }
      } else {
        const int prow0 = (j0 + jlo) % A.ring_cap;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int jl = jk + 32 * (t >> 1) + 4 * (t & 1);
          const uint8_t* kr = kb + (int64_t)krow(prow0, min(max(jl, jlo), nk - 1)) * kst;
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) kc[t][kk] = u32x2a{*reinterpret_cast<const uint32_t*>(kr + 16 * kk), 0u};
        }
      }
    } else {
      const int8_t* kb = A.kq + (int64_t)g * A.ld_head + 8 * kg;
      if (__builtin_expect(lin, 1)) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int jl = jk + 32 * (t >> 1) + 4 * (t & 1);
          const int8_t* kr = kb + (jl < nk ? jrow + jl : jlast) * A.ld_tok;
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) kc[t][kk] = *reinterpret_cast<const u32x2a*>(kr + 32 * kk);
        }
      } else {
        const int prow0 = (j0 + jlo) % A.ring_cap;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int jl = jk + 32 * (t >> 1) + 4 * (t & 1);
          const int8_t* kr = kb + (int64_t)krow(prow0, min(max(jl, jlo), nk - 1)) * A.ld_tok;
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) kc[t][kk] = *reinterpret_cast<const u32x2a*>(kr + 32 * kk);
        }
      }
    }
    // ---- q8_0 scales: lane (col, kg) fetches the K and V scales of key
    // 8kg + col%8 + 32(col/8) of the wave (the 16 lanes of a group cover the 16
    // keys whose scores and weights the group holds); they go to LDS below
    u32x2a ksc = {0u, 0u}, vsc = {0u, 0u};
    if constexpr (Q8) {
      const int kw = 8 * kg + (col & 7) + 32 * (col >> 3);
      const int64_t so = vrow(wk + kw) * (A.ld_tok >> 5) + (int64_t)g * (A.ld_head >> 5);
      ksc = *reinterpret_cast<const u32x2a*>(A.kd + so);
      vsc = *reinterpret_cast<const u32x2a*>(A.vd + so);
    }
    // ---- q (score B operands): column col = (token tk, head hg*hpw + hh), dims 32kk + 8kg ..
    // (a column past the sequence's tokens or the group's heads reads its last
    // token or head: all its keys are masked and its partial is not stored)
    f32x4 qv[4][2];
    {
      const f32x4* qp = reinterpret_cast<const f32x4*>(
          q + (int64_t)(A.row0 + min(tk, T - 1)) * ld_q + (int64_t)(hg * hpw + min(hh, hpw - 1)) * HD + 8 * kg);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        qv[kk][0] = qp[8 * kk];
        qv[kk][1] = qp[8 * kk + 1];
      }
    }
    // fp16: the wave's V rows go to LDS in two halves of 32 rows (8 KiB), the
    // second after the first has been read
    auto dma_v = [&](int h, uint8_t* dst) {
      const uint16_t* vbase = A.v + (int64_t)g * A.ld_head;
      const int jv = wk + (lane >> 4);
      if (__builtin_expect(lin, 1)) {
        const uint8_t* v0 = reinterpret_cast<const uint8_t*>(vbase + (jrow + jv) * A.ld_tok);
        const uint8_t* vlast = reinterpret_cast<const uint8_t*>(vbase + jlast * A.ld_tok);
        const int64_t step4 = 4 * A.ld_tok * 2;
#pragma unroll
        for (int ii = 0; ii < 8; ++ii) {
          const int i = 8 * h + ii;
          const int r = 4 * i + (lane >> 4);
          const int piece = (lane & 15) ^ (2 * vswz(r));
          const uint8_t* row = jv + 4 * i < nk ? v0 + i * step4 : vlast;
          __builtin_amdgcn_global_load_lds(static_cast<const void*>(row + 16 * piece), (lds_ptr)(dst + ii * 1024), 16, 0, kVCpol);
        }
      } else {
        const int prow0 = (j0 + jlo) % A.ring_cap;
#pragma unroll
        for (int ii = 0; ii < 8; ++ii) {
          const int i = 8 * h + ii;
          const int r = 4 * i + (lane >> 4);
          const int piece = (lane & 15) ^ (2 * vswz(r));
          const int jl = min(max(jv + 4 * i, jlo), nk - 1);
          const uint8_t* row = reinterpret_cast<const uint8_t*>(vbase + (int64_t)krow(prow0, jl) * A.ld_tok);
          __builtin_amdgcn_global_load_lds(static_cast<const void*>(row + 16 * piece), (lds_ptr)(dst + ii * 1024), 16, 0, kVCpol);
        }
      }
    };
    if constexpr (!Q8) {
      dma_v(0, vw);
      if (SMALL && alone) dma_v(1, vw + kVB);
    }
    if constexpr (Q8) {
      // every load is in flight before the first use of a loaded value: the pins
      // keep the compiler from moving arithmetic (and its waits) between the issues
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) asm volatile("" : "+v"(qv[kk][0]), "+v"(qv[kk][1]));
      // the scales, 16 bytes per key (K then V), in the wave's own region; only
      // this wave reads them back, after its own write
      uint32_t* sw = s_sc + wave * 256;
      const int kw = 8 * kg + (col & 7) + 32 * (col >> 3);
      *reinterpret_cast<u32x4a*>(sw + 4 * kw) = u32x4a{ksc.x, ksc.y, vsc.x, vsc.y};
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
      if constexpr (!Q8) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const h8 av = __builtin_bit_cast(h8, ka[t][kk]);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bhi[kk], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, blo[kk], acc, 0, 0, 0);
        }
      } else {
        // block kk's partial score, times the key's block-kk scale, in block order
        const uint32_t* sw = s_sc + wave * 256;
        f32x4v dk[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const h8 av = K4 ? nibbles_to_h8(kc[t][kk].x) : codes_to_h8(kc[t][kk].x, kc[t][kk].y);
          dk[kk] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bhi[kk], f32x4v{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
          dk[kk] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, blo[kk], dk[kk], 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int kw = 32 * (t >> 1) + 8 * kg + 4 * (t & 1) + r;
          // (the four fp16 scales as one h4: taking halves of the two dwords
          // separately made this compiler fold both dwords into the first)
          const h4 sk = __builtin_bit_cast(h4, *reinterpret_cast<const u32x2a*>(sw + 4 * kw));
          float a = __builtin_fmaf(dk[0][r], (float)sk[0], 0.0f);
          a = __builtin_fmaf(dk[1][r], (float)sk[1], a);
          a = __builtin_fmaf(dk[2][r], (float)sk[2], a);
          acc[r] = __builtin_fmaf(dk[3][r], (float)sk[3], a);
        }
      }
      // D slot r of this lane = row 4kg + r = key wk + 32(t/2) + 8kg + 4(t%2) + r, head col
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int jl = wk + 32 * (t >> 1) + 8 * kg + 4 * (t & 1) + r;
        z[t][r] = (jl < nk_col && jl >= jlo_col) ? fmul(acc[r], scale) : -INFINITY;
      }
    }
    // ---- the chunk maximum per column, shared by the four waves
    float M;
    {
      float mw = -INFINITY;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) mw = fmaxf(mw, z[t][r]);
      mw = cross_row_max(mw);
      if constexpr (SMALL) {
        M = mw;
      } else {
        if (lane < 16) s_m[wave][lane] = mw;
        __syncthreads();
        M = fmaxf(fmaxf(s_m[0][col], s_m[1][col]), fmaxf(s_m[2][col], s_m[3][col]));
      }
    }
    // ---- weights, their sum, and the P^T operands (block b: slot j = tile 2b + j/4, slot j%4)
    h8 phi[2], plo[2];
    float pw[4][4];
    float lw = 0.0f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float pz = z[t][r] == -INFINITY ? 0.0f : exp_w(fsub(z[t][r], M));
        lw = fadd(lw, pz);
        pw[t][r] = pz;
        if constexpr (!Q8) {
          _Float16 hi, lo;
          split_f16(pz, hi, lo);
          phi[t >> 1][4 * (t & 1) + r] = hi;
          plo[t >> 1][4 * (t & 1) + r] = lo;
        }
      }
    lw = cross_row_sum_fixed(lw);
    if (!SMALL && lane < 16) s_l[wave][lane] = lw;

    // ---- weighted values: this wave's V rows have landed in LDS
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if constexpr (V4) {
      // lane l's key: its 128 codes n - 8 as eight 16-byte segments, segment q
      // at 16-byte position q ^ vswz8(l) of row l (the q8_0 DMA layout)
      const uint32_t nb[16] = {v4r[0].x, v4r[0].y, v4r[0].z, v4r[0].w, v4r[1].x, v4r[1].y, v4r[1].z, v4r[1].w,
                               v4r[2].x, v4r[2].y, v4r[2].z, v4r[2].w, v4r[3].x, v4r[3].y, v4r[3].z, v4r[3].w};
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        uint32_t c0, c1, c2, c3;
        nibbles_to_codes(nb[2 * q], c0, c1);
        nibbles_to_codes(nb[2 * q + 1], c2, c3);
        *reinterpret_cast<u32x4a*>(vw + lane * kRowBytes8 + 16 * (q ^ vswz8(lane))) = u32x4a{c0, c1, c2, c3};
      }
      // every lane's codes are in LDS before the transposed reads below
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
    f32x4v o[8];
    if constexpr (!Q8) {
      // lane (col, kg) reads row 32b + 8kg + 4h + col/4, dims 16dt + 4(col%4) .. +3
      const int vg = vswz(8 * kg + (col >> 2));
      const int rbase = (8 * kg + (col >> 2)) * kRowBytes + 8 * (col & 3);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        if (b == 1 && !(SMALL && alone)) {
          // every read of the first half has returned before its rows are replaced
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
          dma_v(1, vw);
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        const int hb = SMALL && alone && b == 1 ? kVB : 0;  // where the second half sits
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          const int a0 = hb + rbase + ((dt ^ vg) << 5);
          const s4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s4_ptr)((__attribute__((address_space(3))) uint8_t*)vw + a0));
          const s4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s4_ptr)((__attribute__((address_space(3))) uint8_t*)vw + a0 + 4 * kRowBytes));
          const h8 av = __builtin_bit_cast(h8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
          o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, phi[b], o[dt], 0, 0, 0);
          o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, plo[b], o[dt], 0, 0, 0);
        }
      }
    } else {
      // lane (col, kg) of step b reads code row 32b + 8kg + col/2, bytes 16dt +
      // 8(col%2) .. +7: the transposed read hands lane (m, kg) the codes of keys
      // 32b + 8kg + 0..7 at dim 16dt + m
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};
      const uint32_t* sw = s_sc + wave * 256;
      const int sg = (col >> 1) ^ (kg & 1);  // vswz8 of the rows this lane reads
      u32x2a sv[2][8];  // V scales of keys 32b + 8kg + j
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int j = 0; j < 8; ++j) sv[b][j] = *reinterpret_cast<const u32x2a*>(sw + 4 * (32 * b + 8 * kg + j) + 2);
      // The weights p * d are about d times smaller than p, so their fp16 hi + lo
      // pair would lose bits to fp16's subnormal range.  Each column scales them
      // by 2^k, k = 29 - (fp16 exponent of the largest |d| among the keys it
      // weights in this wave), so p * d * 2^k < 2^15, and scales its partial back
      // by 2^-k (both exact).  k depends only on keys the column attends to.
      float up, down;
      {
        typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
        u16x2 mb = {0, 0};
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const u16x2 x = __builtin_elementwise_max(__builtin_bit_cast(u16x2, sv[b][j].x & 0x7fff7fffu),
                                                      __builtin_bit_cast(u16x2, sv[b][j].y & 0x7fff7fffu));
            if (pw[2 * b + (j >> 2)][j & 3] > 0.0f) mb = __builtin_elementwise_max(mb, x);
          }
        const float mf = cross_row_max((float)(mb.x > mb.y ? mb.x : mb.y));
        const int kx = 29 - ((int)mf >> 10);
        up = __builtin_bit_cast(float, (uint32_t)(kx + 127) << 23);
        down = __builtin_bit_cast(float, (uint32_t)(127 - kx) << 23);
      }
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) pw[t][r] = fmul(pw[t][r], up);
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const int rb = (32 * b + 8 * kg + (col >> 1)) * kRowBytes8 + 8 * (col & 1);
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          h8 whi, wlo;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const h4 sp = __builtin_bit_cast(h4, sv[b][j]);
            const float w = __builtin_fmaf(pw[2 * b + (j >> 2)][j & 3], (float)sp[bb], 0.0f);
            _Float16 hi, lo;
            split_f16(w, hi, lo);
            whi[j] = hi;
            wlo[j] = lo;
          }
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int dt = 2 * bb + e;
            const i32x2 cv = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (lds_i32x2_ptr)((__attribute__((address_space(3))) uint8_t*)vw + rb + 16 * (dt ^ sg)));
            const h8 av = codes_to_h8((uint32_t)cv.x, (uint32_t)cv.y);
            o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, whi, o[dt], 0, 0, 0);
            o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, wlo, o[dt], 0, 0, 0);
          }
        }
      }
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[dt][r] = fmul(o[dt][r], down);
    }
    // D slot r of lane (col, kg) = dim 16dt + 4kg + r of column col
    if constexpr (SMALL) {
      // a small chunk: the wave's partial is the chunk's, for each column whose
      // token reaches the chunk.  0 + o is what the four-wave sum below gives when
      // the other waves hold no key of the column (as in a verify call whose
      // later tokens make the same chunk a four-wave one), so the bits agree.
      const int p2 = A.ctx_len - T + tk;
      if (colv && j0 <= p2 && !(A.window && j0 + csz <= p2 - A.window + 1)) {
        const int h = hg * hpw + hh;
        float* dst = part + ((int64_t)A.partial_begin + ((int64_t)tk * H_q + h) * A.n_chunks + ci) * PF;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
          *reinterpret_cast<f32x4*>(dst + 4 + 16 * dt + 4 * kg) =
              f32x4{fadd(0.0f, o[dt][0]), fadd(0.0f, o[dt][1]), fadd(0.0f, o[dt][2]), fadd(0.0f, o[dt][3])};
        if (kg == 0) {
          dst[0] = M;
          dst[1] = lw;
        }
      }
      return;
    }
    // every lane of the wave is done reading the wave's V region before it takes
    // the partial (LDS reads of one wave complete in order); the wave's own V
    // region (now read) takes its partial O[column][dim]
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
      if ((cc & (kAttnGroup - 1)) >= hpw) continue;  // no head of the group
      if (j0 > p2) continue;  // chunk past this token's position
      if (A.window && j0 + csz <= p2 - A.window + 1) continue;  // chunk before its window
      float O = 0.0f, L = 0.0f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        O = fadd(O, reinterpret_cast<const float*>(s_v + w * kVB)[idx]);
        L = fadd(L, s_l[w][cc]);
      }
      const float Mh = fmaxf(fmaxf(s_m[0][cc], s_m[1][cc]), fmaxf(s_m[2][cc], s_m[3][cc]));
      const int h = hg * hpw + (cc & (kAttnGroup - 1));
      float* dst = part + ((int64_t)A.partial_begin + ((int64_t)t2 * H_q + h) * A.n_chunks + ci) * PF;
      dst[4 + d] = O;
      if (d == 0) {
        dst[0] = Mh;
        dst[1] = L;
      }
    }
  };
  if (small)
    body(std::true_type{});
  else
    body(std::false_type{});
}

// Grid (query rows * H_q), 256 threads.  Merges the chunk partials of one
// (sequence, token, head) -- its chunks are those up to the token's position: M = max_c m_c; w_c = exp(m_c - M); L = sum_c l_c w_c by a
// fixed tree over chunk index; O[d] = sum_c o_c[d] w_c with chunks split into
// eight interleaved groups (group j takes chunks j, j+8, ..., in chunk order)
// that are then added by a fixed tree.  Every shape depends only on the
// sequence's chunk count.  Optionally also emits the q8 blocks of the output
// row (the quantized input of the output projection).
constexpr int kMaxChunks = kAttnMaxChunks;
constexpr int kFastLoads = 20;  // value loads per thread on the one-pass path: up to 160 chunks

// The combine's one-pass merge for nc <= 8 * NL chunks: every load is issued
// up front, (m, l) of chunk tid and the values of chunks j, j + 8, ..., j + 8(NL-1)
// (thread (j, dims d4..d4+3)), so the merge waits for memory once.  Loads past
// the last chunk read chunk nc - 1 and are never used, so the sums are those
// of the general path term for term, whatever NL.  Leaves the eight group sums
// in s_o and returns L.
template <int NL>
__device__ __forceinline__ float merge_one_pass(const float* __restrict__ base, int nc, int tid,
                                                float* s_w, float* s_red, float* s_o) {
  const int j = tid >> 5;
  const int d4 = (tid & 31) * 4;
  const float* mlp = base + (int64_t)min(tid, nc - 1) * PF;
  const float m_c = mlp[0], l_c = mlp[1];
  f32x4 a[NL];
#pragma unroll
  for (int i = 0; i < NL; ++i)
    a[i] = *reinterpret_cast<const f32x4*>(base + (int64_t)min(j + 8 * i, nc - 1) * PF + 4 + d4);
  float mx = group_max<64>(tid < nc ? m_c : -INFINITY);
  if ((tid & 63) == 0) s_red[tid >> 6] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  __syncthreads();
  float lp = 0.0f;
  if (tid < nc) {
    const float w = expf(fsub(m_c, M));
    s_w[tid] = w;
    lp = fadd(lp, fmul(l_c, w));
  }
  lp = wave_sum_fixed(lp);
  if ((tid & 63) == 0) s_red[tid >> 6] = lp;
  __syncthreads();
  const float L = fadd(fadd(s_red[0], s_red[1]), fadd(s_red[2], s_red[3]));
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    if (j + 8 * i < nc) {
      const float w = s_w[j + 8 * i];
      acc.x = fadd(acc.x, fmul(a[i].x, w));
      acc.y = fadd(acc.y, fmul(a[i].y, w));
      acc.z = fadd(acc.z, fmul(a[i].z, w));
      acc.w = fadd(acc.w, fmul(a[i].w, w));
    }
  }
  *reinterpret_cast<f32x4*>(s_o + j * HD + d4) = acc;
  __syncthreads();
  return L;
}

__global__ __launch_bounds__(256) void k_attn_combine(SeqArgs seqs, int H_q,
                                                      const float* __restrict__ part,
                                                      float* __restrict__ out, int8_t* oq, float* od) {
  __shared__ float s_w[kMaxChunks];
  __shared__ float s_red[256];
  __shared__ __attribute__((aligned(16))) float s_o[8 * HD];
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
  const int nc = attn_chunks(lo, p);  // this token's chunks: those of positions lo..p
  const float* base = part + ((int64_t)A.partial_begin + ((int64_t)t * H_q + h) * A.n_chunks +
                              (attn_chunk_of(lo) - A.c0)) * PF;

  float L;
  const int j = tid >> 5;         // chunk group of the value sums
  const int d4 = (tid & 31) * 4;  // dims d4 .. d4+3
  if (nc <= 8 * kFastLoads) {
    // up to 160 chunks (34816 keys from position 0): one pass, with as many
    // value loads per thread as the token's chunk count needs
    if (nc <= 40)
      L = merge_one_pass<5>(base, nc, tid, s_w, s_red, s_o);
    else if (nc <= 80)
      L = merge_one_pass<10>(base, nc, tid, s_w, s_red, s_o);
    else if (nc <= 128)
      L = merge_one_pass<16>(base, nc, tid, s_w, s_red, s_o);
    else
      L = merge_one_pass<kFastLoads>(base, nc, tid, s_w, s_red, s_o);
  } else {
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
    L = fadd(fadd(s_red[0], s_red[1]), fadd(s_red[2], s_red[3]));
    // values: eight interleaved groups of chunks (group j: chunks j, j+8, ...),
    // each summed in chunk order by 32 threads of 4 dims (one 16-byte load per
    // chunk, 16 chunks in flight), then the groups added by a fixed tree
    {
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
      int c = j;
      for (; c + 8 * 15 < nc; c += 8 * 16) {
        f32x4 a[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) a[i] = *reinterpret_cast<const f32x4*>(base + (int64_t)(c + 8 * i) * PF + 4 + d4);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float w = s_w[c + 8 * i];
          acc.x = fadd(acc.x, fmul(a[i].x, w));
          acc.y = fadd(acc.y, fmul(a[i].y, w));
          acc.z = fadd(acc.z, fmul(a[i].z, w));
          acc.w = fadd(acc.w, fmul(a[i].w, w));
        }
      }
      for (; c < nc; c += 8) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(base + (int64_t)c * PF + 4 + d4);
        const float w = s_w[c];
        acc.x = fadd(acc.x, fmul(a.x, w));
        acc.y = fadd(acc.y, fmul(a.y, w));
        acc.z = fadd(acc.z, fmul(a.z, w));
        acc.w = fadd(acc.w, fmul(a.w, w));
      }
      *reinterpret_cast<f32x4*>(s_o + j * HD + d4) = acc;
    }
    __syncthreads();
  }
  if (tid < HD) {
    const int d = tid;
    const float* g8 = s_o + d;
    const float O = fadd(fadd(fadd(g8[0], g8[HD]), fadd(g8[2 * HD], g8[3 * HD])),
                         fadd(fadd(g8[4 * HD], g8[5 * HD]), fadd(g8[6 * HD], g8[7 * HD])));
    const float v = fdiv(O, L);
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
  // head groups: the largest divisor of the group size H_q / H_kv that fills at
  // most the 4 head columns of a workgroup (four: one group per KV head)
  const int G = H_q / H_kv;
  a->hpw = G >= 4 && G % 4 == 0 ? 4 : (G % 3 == 0 ? 3 : (G % 2 == 0 ? 2 : 1));
  a->vg = G / a->hpw;
  const int n_hg = H_q / a->hpw;
  int parts = 0, rows = 0;
  int64_t small_keys = 0, large_keys = 0;
  for (int s = 0; s < a->n_seq; ++s) {
    SeqArg& x = a->s[s];
    x.lo0 = x.window ? (x.ctx_len - x.n_new - x.window + 1 > 0 ? x.ctx_len - x.n_new - x.window + 1 : 0) : 0;
    x.c0 = attn_chunk_of(x.lo0);
    x.n_chunks = attn_chunks(x.lo0, x.ctx_len - 1);
    const int c_end = x.c0 + x.n_chunks;  // chunks c0 .. c_end - 1
    x.ns = (c_end < kAttnSmallChunks ? c_end : kAttnSmallChunks) - x.c0;
    if (x.ns < 0) x.ns = 0;
    small_keys += (int64_t)x.ns * kAttnSmallChunk;
    large_keys += x.ctx_len > kAttnSmallSpan ? x.ctx_len - kAttnSmallSpan : 0;
  }
  // One 64-key chunk per workgroup spreads a short context over the CUs (one
  // 2050-key sequence: 264 workgroups, 9.4 us against 12.4 us with four per
  // workgroup).  Once the call has more such chunks than the chip has CUs, or
  // most of its keys sit in 256-key chunks, four per workgroup (one per wave)
  // do better (graph-timed, us, one vs four per workgroup: {2050, 3072} 14.9
  // vs 13.8; four 2050s 16.5 vs 15.0; one 32768-key sequence 34.7 vs 32.6).
  const int pk = small_keys / kAttnSmallChunk * n_hg > kAttnSpreadUnits || large_keys > small_keys ? 4 : 1;
  for (int s = 0; s < a->n_seq; ++s) {
    SeqArg& x = a->s[s];
    x.pk = pk;
    x.partial_begin = parts;
    x.row0 = rows;
    parts += x.n_chunks * H_q * x.n_new;
    rows += x.n_new;
  }
  // workgroups: every sequence's 256-key units, then every sequence's 64-key units
  int units = 0;
  for (int s = 0; s < a->n_seq; ++s) {
    SeqArg& x = a->s[s];
    x.large_begin = units;
    units += (x.n_chunks - x.ns) * n_hg;
  }
  a->large_total = units;
  for (int s = 0; s < a->n_seq; ++s) {
    SeqArg& x = a->s[s];
    x.small_begin = units;
    units += (x.ns + pk - 1) / pk * n_hg;
  }
  a->units_total = units;
  return (size_t)parts * PF;
}

hipError_t launch_attn(const float* q, int64_t ld_q, const SeqArgs& seqs, int H_q, int H_kv,
                       float scale, float* out, float* partials, int8_t* oq, float* od,
                       hipStream_t st) {
  const int units = seqs.units_total;
  (void)H_kv;
  if (seqs.s[0].q8 && seqs.s[0].k4 && seqs.s[0].v4)
    hipLaunchKernelGGL((k_attn_chunk<true, true, true>), dim3(units), dim3(256), 0, st, q, ld_q, seqs, H_q,
                       scale, partials);
  else if (seqs.s[0].q8 && seqs.s[0].k4)
    hipLaunchKernelGGL((k_attn_chunk<true, true, false>), dim3(units), dim3(256), 0, st, q, ld_q, seqs, H_q,
                       scale, partials);
  else if (seqs.s[0].q8 && seqs.s[0].v4)
    hipLaunchKernelGGL((k_attn_chunk<true, false, true>), dim3(units), dim3(256), 0, st, q, ld_q, seqs, H_q,
                       scale, partials);
  else if (seqs.s[0].q8)
    hipLaunchKernelGGL(k_attn_chunk<true>, dim3(units), dim3(256), 0, st, q, ld_q, seqs, H_q, scale,
                       partials);
  else
    hipLaunchKernelGGL(k_attn_chunk<false>, dim3(units), dim3(256), 0, st, q, ld_q, seqs, H_q, scale,
                       partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  int rows = 0;
  for (int s = 0; s < seqs.n_seq; ++s) rows += seqs.s[s].n_new;
  hipLaunchKernelGGL(k_attn_combine, dim3(rows * H_q), dim3(256), 0, st, seqs, H_q, partials,
                     out, oq, od);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Scratch of the allocation-free attention entry point: the chunk partials
// live in this file-scope device array instead of a caller's workspace.  Each
// GPU the library runs on holds its own copy until the process ends.  Host
// code never passes `scratch` itself (on the host that name is a stand-in, not
// a device address): attn_scratch() looks up the device address once per
// device, with that device current, and every launch takes that pointer.
namespace {
static __device__ __align__(256) float scratch[kAttnScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
}  // namespace

hipError_t attn_scratch(float** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
  *ptr = static_cast<float*>(g_scratch_ptr[dev]);
  return hipSuccess;
}

}  // namespace sd
