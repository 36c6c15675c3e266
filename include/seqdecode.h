/*
 * seqdecode.h -- C ABI of the exact, batch-invariant multi-sequence decode step
 * for AMD Instinct MI355X (gfx950).
 *
 * Every entry point enqueues HIP kernels on the caller's stream and returns
 * without synchronizing.  Pointers are DEVICE pointers unless marked [host].
 * The caller owns every buffer; the library allocates no device memory and
 * keeps no device state between calls, so concurrent calls on different
 * streams are independent.  The one exception is
 * sd_decode_attn_multiseq_noalloc, whose partials live in a file-scope device
 * array that every call on a GPU shares (calls of it that overlap on one GPU
 * race).  Its only process state is each kernel's raised LDS limit, set once on
 * a kernel's first launch under std::call_once (safe when several host threads
 * make their first calls at once), and that array's device address, looked up
 * once per device the same way.
 *
 * Errors: arguments are validated on the host before any HIP call.  On failure
 * a negative sd_status is returned, nothing is launched and no output is
 * written.  SD_EHIP reports a launch error from the HIP runtime.
 *
 * Batch invariance: for every entry point, the bits of the output for token
 * (or sequence) t depend only on t's own inputs, never on how many other rows
 * are in the call or where t sits among them.  This is the property the
 * "feat(qwen4exp): exact 4-slot concurrent serving" page demands in "How it
 * stays exact" (a batch uses the same kernels and arithmetic as a single row),
 * and that ds4 pull request 604 does not reach ("Correctness notes and
 * limitations": its fused pass differs from serial decode by reduction order).
 *
 * Page citations below name the page and the section on it.
 */
#ifndef SEQDECODE_H
#define SEQDECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* sd_stream_t; /* a hipStream_t; NULL = legacy default stream */

typedef enum sd_status {
  SD_OK = 0,
  SD_EINVAL = -1,       /* a size, count or pointer is out of range or NULL */
  SD_EUNSUPPORTED = -2, /* a shape this build does not implement */
  SD_EALIGN = -3,       /* a pointer or stride breaks the stated alignment */
  SD_EWORKSPACE = -4,   /* the workspace is smaller than the query returned */
  SD_EHIP = -5          /* the HIP runtime rejected a launch */
} sd_status;

/* Human-readable name of a status code (static string; never NULL). */
const char* sd_status_string(int status);

/* ABI revision of this header; bumps on any signature change. */
#define SD_ABI_VERSION 10
int sd_abi_version(void);

/* Largest batch of token rows a GEMV call takes (speculative-verify width, see
 * "#1209 Speed up concurrent generation, fix QFUSE, and improve prefill
 * monitoring", "What changed and why" item 1: 8/12/16-row capacities). */
#define SD_MAX_TOKENS 16
/* Largest number of sequences one attention call takes: ds4 pull request 604,
 * "Commit walkthrough / CUDA kernels" (per-sequence views passed by value,
 * max 4); "feat(qwen4exp): exact 4-slot concurrent serving", "What" (more than
 * four is refused). */
#define SD_MAX_SEQS 4
/* Attention chunks (the units of the split over keys), fixed in absolute
 * positions so that a token's split depends on its own position only:
 * positions below SD_ATTN_SMALL_SPAN in chunks of SD_ATTN_SMALL_CHUNK keys
 * (a short context still spreads over the whole GPU), later positions in
 * chunks of SD_ATTN_CHUNK keys. */
#define SD_ATTN_CHUNK 256
#define SD_ATTN_SMALL_CHUNK 64
#define SD_ATTN_SMALL_SPAN 2048
/* Most keys one attention token attends to (the span from its lowest key to
 * its own position). */
#define SD_MAX_CTX (2048 * SD_ATTN_CHUNK)

/* ------------------------------------------------------------------ q8 data
 * q8_0 weight matrix: N rows, each of K/32 consecutive 34-byte blocks; a block
 * is a little-endian fp16 scale d_w followed by 32 int8 weights (the 32-weight
 * block of ds4 pull request 604, "Commit walkthrough / CUDA kernels").
 * q8 activations: per token, K int8 codes (row stride K) and K/32 fp32 block
 * scales (row stride K/32).
 */

/*
 * sd_quantize_q8_act -- fp32 rows -> q8 activation blocks.
 * For each token t < n_tok and block b < K/32: amax = max|x|, d = amax/127 in
 * fp32 (IEEE division), code = roundf(x/d) (fp32 division, ties away from
 * zero) clamped to [-127, 127]; all codes 0 when d == 0.  This is the division
 * and rounding convention every fused producer in this library also uses (the
 * QFUSE lesson of "#1209 ...", "What changed and why" item 2).
 *   x   [n_tok][ldx] fp32, 4-byte aligned; ldx >= K.
 *   xq  [n_tok][K] int8, 16-byte aligned.   xd [n_tok][K/32] fp32.
 * Requires 1 <= n_tok <= SD_MAX_TOKENS, K > 0, K % 32 == 0.  Inputs must be
 * finite (non-finite inputs give unspecified codes).
 */
int sd_quantize_q8_act(const float* x, int64_t ldx, int n_tok, int64_t K,
                       int8_t* xq, float* xd, sd_stream_t stream);

/*
 * sd_qgemv_q8_0_batch -- narrow-batch q8_0 matrix-vector product (ds4 pull
 * request 604, "Commit walkthrough / CUDA kernels": each 32-weight block is
 * read once and dotted against every token row).
 *   y[t][n] = (residual ? residual[t][n] : 0) + sum_b s_b,
 *   s_b = fl32(fl32(d_w[n][b] * xd[t][b]) * (float) sum_i w[n][b][i]*xq[t][b*32+i])
 * The block sums are exact int32; the fp32 sum over b uses one fixed order
 * that depends on K only, so y[t] is bitwise the same for any n_tok and any
 * row order.
 *   w         N*(K/32)*34 bytes, 16-byte aligned.
 *   xq, xd    q8 activations of n_tok tokens (layout above); xq 16-byte aligned.
 *   residual  NULL or [n_tok][ldy] fp32; may equal y (in-place accumulate).
 *   y         [n_tok][ldy] fp32, ldy >= N.
 * Requires 1 <= N <= 2^30, K % 256 == 0 (rows then start 16-byte aligned),
 * K <= 2^24, 1 <= n_tok <= SD_MAX_TOKENS; otherwise SD_EUNSUPPORTED /
 * SD_EINVAL.
 */
int sd_qgemv_q8_0_batch(const void* w, int64_t N, int64_t K,
                        const int8_t* xq, const float* xd, int n_tok,
                        const float* residual, float* y, int64_t ldy,
                        sd_stream_t stream);

/*
 * sd_qgemv_q8_0_batch_path -- sd_qgemv_q8_0_batch with the kernel chosen by
 * the caller, for the wide verify batches of "#1209 Speed up concurrent
 * generation, fix QFUSE, and improve prefill monitoring", "What changed and
 * why" item 1 (several proposed tokens per sequence checked together, with
 * 8/12/16-row capacities).
 *   path  SD_GEMV_AUTO   the kernel sd_qgemv_q8_0_batch uses (the narrow
 *                        kernel up to 8 tokens and K <= 16384, else MFMA);
 *         SD_GEMV_NARROW v_dot4 kernels (one lane per block pair);
 *         SD_GEMV_MFMA   matrix-core kernel (v_mfma_i32_16x16x32_i8 on tiles
 *                        of 16 rows x 16 tokens).
 * All paths compute the same cells in the same fixed order, so y is bitwise
 * identical whichever path runs, for any n_tok.  Other arguments, layouts and
 * errors as sd_qgemv_q8_0_batch; an unknown path gives SD_EINVAL.
 */
#define SD_GEMV_AUTO 0
#define SD_GEMV_NARROW 1
#define SD_GEMV_MFMA 2
int sd_qgemv_q8_0_batch_path(const void* w, int64_t N, int64_t K,
                             const int8_t* xq, const float* xd, int n_tok,
                             const float* residual, float* y, int64_t ldy,
                             int path, sd_stream_t stream);

/* ------------------------------------------------------------------ RoPE
 * sd_rope_posvec -- rotary embedding with one position per token (ds4 pull
 * request 604, "Commit walkthrough / CUDA kernels": pos-vector RoPE; token t
 * gives bitwise what a single-token call at pos[t] gives).
 * In place on x[t][h][:] (token stride ld_tok, head stride ld_head, in
 * elements).  The last n_rot dimensions of each head are rotated: with
 * off = head_dim - n_rot and half = n_rot/2, the pair (off+i, off+i+half) turns
 * by pos[t] * theta^(-2i/n_rot).  Angle, sine and cosine are computed in fp64
 * and rounded to fp32; the rotation is fp32.
 *   pos [n_tok] int32 >= 0 (device).
 * Requires 1 <= n_tok <= 4096, n_heads >= 1, n_rot even, 2 <= n_rot <= head_dim
 * <= 512, theta > 0.
 */
int sd_rope_posvec(float* x, int n_tok, int n_heads, int head_dim,
                   int64_t ld_tok, int64_t ld_head, const int32_t* pos,
                   double theta, int n_rot, sd_stream_t stream);

/* --------------------------------------------------- per-sequence KV views
 * Cache element types.  SD_KV_F16: fp16 keys and values (bit patterns).
 * SD_KV_Q8_0: the "int8 KV" / "Q8" caches of "#1209 Speed up concurrent
 * generation, fix QFUSE, and improve prefill monitoring" ("What changed and
 * why": resident int8 KV) and "feat(qwen36): complete concurrent serving
 * implementation with speculation" ("Validation": Q8 attention cases), in
 * q8_0 blocks: each run of 32 consecutive dims of a (row, head) is 32 int8
 * codes c with one fp16 scale d, value d * c.  Codes and scales live in two
 * planes: codes at the element offsets of an fp16 cache, scales at the same
 * offsets divided by 32.  Quantization of a new row (the append and the step)
 * takes, per block, d = amax / 127 in fp32, c = clamp(round-half-away(x / d),
 * -127, 127) (0 when d = 0), and stores fp16(d) rounded to nearest even.
 * SD_KV_Q4_0, SD_KV_Q4_Q8, SD_KV_Q8_Q4: the Q4 type and the mixed Q4/Q8 and
 * Q8/Q4 caches of the same "Validation" (K type / V type).  A q4_0 block is 32
 * four-bit codes with one fp16 scale d, value d * (n - 8) for the stored
 * nibble n; the nibbles of dims 2j and 2j + 1 of a block share byte j (the
 * even dim in the low four bits), so a row's codes take half the bytes of its
 * dims: codes at the element offsets of an fp16 cache divided by 2, scales (as
 * for q8_0) divided by 32.  Quantization takes d = amax / 7 in fp32 and
 * c = clamp(round-half-away(x / d), -8, 7) (0 when d = 0), stores n = c + 8
 * and fp16(d) rounded to nearest even.
 */
#define SD_KV_F16 0
#define SD_KV_Q8_0 1
#define SD_KV_Q4_0 2  /* K and V q4_0 */
#define SD_KV_Q4_Q8 3 /* K q4_0, V q8_0 */
#define SD_KV_Q8_Q4 4 /* K q8_0, V q4_0 */

/*
 * One sequence's key and value caches, element (row r, head g, dim d) at
 * base[r*ld_tok + g*ld_head + d] (elements).  The struct
 * array is [host] memory; kernels receive the views by value in their
 * arguments (ds4 pull request 604, "Commit walkthrough / CUDA kernels", whose
 * sequences each attend to their own KV ring).  ctx_len is one past the
 * newest position (the current token sits at ctx_len - 1).
 *   window  0: a token at position p attends to positions 0..p; else to the
 *           last `window` positions max(0, p - window + 1)..p.
 *   ring    0: position j lives in row j (ctx_len <= capacity);
 *           1: the cache is a ring, position j in row j % capacity (needs
 *           window >= 1 and room for every position still attended to).
 *   kv_type SD_KV_F16: k and v hold fp16 bits and k_q8 .. v_d are unused;
 *           the quantized types: k and v are unused, codes in k_q8 / v_q8
 *           (16-byte aligned; q4_0 nibbles at half the byte offsets), scales
 *           in k_d / v_d (8-byte aligned); D % 32 == 0 and ld_tok, ld_head
 *           multiples of 32 (of 128 for attention).
 *   block_table  NULL, or a paged cache ("feat(qwen36): complete concurrent
 *           serving implementation with speculation", "Summary": a shared
 *           paged KV pool with per-sequence block tables): k and v are a pool
 *           of capacity rows in blocks of block_size rows, and position j
 *           lives in row block_table[j / block_size] * block_size
 *           + j % block_size.  block_table is [device] int32, 4-byte aligned,
 *           with an entry for every block up to position ctx_len - 1 (entries
 *           of blocks wholly below a window may hold anything); block_size is
 *           64, 128 or 256 and divides capacity; an entry outside
 *           0 .. capacity / block_size - 1 is clamped into it, so no access
 *           leaves the pool.  ctx_len is not bounded by capacity (blocks may
 *           be shared).  Not combined with ring.  The table is read by the
 *           kernels on the stream: it must stay valid until they are done.
 * Zero-initialised trailing fields give the plain layout.
 */
typedef struct sd_seqview {
  uint16_t* k;
  uint16_t* v;
  int32_t ctx_len;
  int32_t capacity;
  int64_t ld_tok;
  int64_t ld_head;
  int32_t window;
  int32_t ring;
  const int32_t* block_table;
  int32_t block_size;
  int32_t kv_type;      /* SD_KV_F16 (k, v) or a quantized type (k_q8, v_q8, k_d, v_d) */
  int8_t* k_q8;         /* q8_0 codes [capacity][H_kv][D] at ld_tok, ld_head (bytes), or
                           q4_0 nibble pairs [capacity][H_kv][D/2] at ld_tok/2, ld_head/2 */
  int8_t* v_q8;
  uint16_t* k_d;        /* fp16 scales: block b of (r, g) at r*(ld_tok/32) + g*(ld_head/32) + b */
  uint16_t* v_d;
} sd_seqview;

/*
 * sd_kv_append_f16 -- write the current token's key and value rows.
 * For sequence s: the row of position ctx_len_s - 1 of views[s] (row
 * (ctx_len_s - 1) % capacity for a ring, the block table's row for a paged
 * view) receives fp16(k_new[s]) and
 * fp16(v_new[s]) (round to nearest even); no other row is touched (ds4 pull
 * request 604, "2. Single-GPU decode batches don't scale": the append runs per
 * sequence).
 *   k_new, v_new  [n_seq][H_kv][D] fp32 at sequence stride ld_new (elements).
 *   views         [host] n_seq views; 4-byte aligned bases, even strides.
 * Requires 1 <= n_seq <= SD_MAX_SEQS, ctx_len >= 1, ctx_len <= capacity
 * for a plain view, D even, every view SD_KV_F16.
 */
int sd_kv_append_f16(const float* k_new, const float* v_new, int64_t ld_new,
                     const sd_seqview* views, int n_seq, int H_kv, int D,
                     sd_stream_t stream);

/*
 * sd_kv_append_q8_0 -- the same append into quantized views: the row of
 * position ctx_len_s - 1 receives the blocks of k_new[s] and v_new[s] in the
 * view's K and V types (codes and fp16 scales, quantized as stated above); no
 * other row is touched.  Requires what sd_kv_append_f16 does, with every view
 * of one quantized kv_type (SD_KV_Q8_0, SD_KV_Q4_0, SD_KV_Q4_Q8 or
 * SD_KV_Q8_Q4) and D % 32 == 0; k_new, v_new finite.
 */
int sd_kv_append_q8_0(const float* k_new, const float* v_new, int64_t ld_new,
                      const sd_seqview* views, int n_seq, int H_kv, int D,
                      sd_stream_t stream);

/*
 * sd_decode_attn_workspace_bytes -- workspace size sd_decode_attn_multiseq
 * needs for these views (0 on invalid arguments).
 */
size_t sd_decode_attn_workspace_bytes(const sd_seqview* views, int n_seq, int H_q, int D);

/*
 * sd_decode_attn_multiseq -- one query token per sequence over that sequence's
 * own cache, all sequences in one launch (ds4 pull request 604, "Commit
 * walkthrough / CUDA kernels": multi-sequence decode attention).
 * For sequence s and query head h (KV head g = h / (H_q/H_kv)):
 *   out[s][h] = sum_j softmax_j(scale * q[s][h] . k_j) v_j,  j < ctx_len_s.
 * fp32 throughout (a softmax partial per chunk of the fixed position grid of
 * SD_ATTN_SMALL_CHUNK / SD_ATTN_CHUNK keys, merged with fixed reduction
 * shapes), so a sequence's bits do not depend on the others.
 *   q    [n_seq][H_q][D] fp32 at sequence stride ld_q (elements), 16-byte aligned.
 *   out  [n_seq][H_q][D] fp32 contiguous, 16-byte aligned.
 *   ws   workspace of at least sd_decode_attn_workspace_bytes(), 16-byte aligned.
 *   views [host]: 16-byte aligned bases, ld_tok and ld_head multiples of 8.
 * Requires 1 <= n_seq <= SD_MAX_SEQS, D == 128, H_q % H_kv == 0 (any number G
 * of query heads per KV head: a workgroup takes a head group, the hpw query
 * heads of one KV head with hpw the largest divisor of G up to 4, so for G of
 * 8, 16, 5, ... each of a KV head's G / hpw groups reads its keys and values),
 * ctx_len >= 1 and, for a plain view, ctx_len <= capacity; a ring needs
 * window >= 1 and min(ctx_len, window + n_new - 1) <= capacity (n_new = 1
 * here).  The keys attended to span at most SD_MAX_CTX positions (else
 * SD_EUNSUPPORTED).  Windows: token at p sees max(0, p - window + 1)..p; the
 * chunks are aligned to absolute positions, so a windowed result is the same
 * in a ring as in a plain cache holding the same rows.  A paged view (see
 * sd_seqview) gives the same bits as a plain cache holding the same keys.
 * Quantized views: keys and values are the dequantized d * c of q8_0 and
 * d * (n - 8) of q4_0 blocks (exact in fp32); all views of one call share one
 * kv_type (else SD_EUNSUPPORTED).
 */
int sd_decode_attn_multiseq(const float* q, int64_t ld_q, const sd_seqview* views,
                            int n_seq, int H_q, int H_kv, int D, float scale,
                            float* out, void* ws, size_t ws_bytes, sd_stream_t stream);

/*
 * sd_decode_attn_multiseq_noalloc -- sd_decode_attn_multiseq without a
 * workspace argument, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  The chunk partials go to a scratch array of
 * SD_ATTN_SCRATCH_BYTES that the library holds in static device memory, one
 * per GPU, until the process ends; the call itself allocates nothing.
 * Arguments, results (bitwise those of sd_decode_attn_multiseq) and errors are
 * those of sd_decode_attn_multiseq, plus SD_EWORKSPACE when
 * sd_decode_attn_workspace_bytes() for these views exceeds
 * SD_ATTN_SCRATCH_BYTES (checked before any HIP call; e.g. 32 query heads fit
 * 992 chunk partials per head summed over the sequences and their tokens).  Every call on
 * one GPU shares that GPU's array and leaves its partials there: calls that
 * overlap on one GPU (on different streams, or from several host threads
 * without ordering) race and give undefined results.  The first call on a
 * device looks up the array's address on it (SD_EHIP if that fails).
 */
#define SD_ATTN_SCRATCH_BYTES (16u << 20)
int sd_decode_attn_multiseq_noalloc(const float* q, int64_t ld_q, const sd_seqview* views,
                                    int n_seq, int H_q, int H_kv, int D, float scale,
                                    float* out, sd_stream_t stream);

/*
 * sd_decode_attn_verify -- several query tokens per sequence: the newest
 * n_new[s] positions of sequence s, each attending causally (the packed
 * multi-sequence verification of proposed tokens, "feat(qwen36): complete
 * concurrent serving implementation with speculation").  The tokens' own K/V
 * rows are already in the cache, so ctx_len_s counts them.  Token i of
 * sequence s (position p = ctx_len_s - n_new[s] + i) gives
 *   out[r][h] = sum_j softmax_j(scale * q[r][h] . k_j) v_j,  j <= p,
 * with r = (n_new[0] + .. + n_new[s-1]) + i the packed row.  Each token's
 * reduction has the shape of a one-token call over p + 1 keys, so its bits are
 * those of sd_decode_attn_multiseq with ctx_len = p + 1, whatever the other
 * tokens and sequences are.
 *   q    [rows][H_q][D] fp32 at row stride ld_q, packed as above, 16-byte aligned.
 *   out  [rows][H_q][D] fp32 contiguous, 16-byte aligned.
 *   n_new [host] n_seq entries, 1 <= n_new[s] <= SD_ATTN_MAX_NEW, <= ctx_len_s.
 *   ws   at least sd_decode_attn_verify_workspace_bytes().
 * Other requirements and errors as sd_decode_attn_multiseq, which is this call
 * with every n_new[s] = 1.
 */
#define SD_ATTN_MAX_NEW 4
size_t sd_decode_attn_verify_workspace_bytes(const sd_seqview* views, const int32_t* n_new,
                                             int n_seq, int H_q, int D);
int sd_decode_attn_verify(const float* q, int64_t ld_q, const sd_seqview* views,
                          const int32_t* n_new, int n_seq, int H_q, int H_kv, int D,
                          float scale, float* out, void* ws, size_t ws_bytes,
                          sd_stream_t stream);

/* ------------------------------------------------------------ step glue
 * Pieces of the fused decode step (ds4 pull request 604, "2. Single-GPU
 * decode batches don't scale" and "Commit walkthrough / Graph driver").
 */

/*
 * sd_rmsnorm_q8 -- y = x / sqrt(mean(x^2) + eps) * gamma per row (fp32, fixed
 * reduction order), quantized to q8 activation blocks exactly as
 * sd_quantize_q8_act would quantize y.
 *   x [n_tok][ldx] fp32; gamma [D] fp32; xq [n_tok][D]; xd [n_tok][D/32];
 *   y NULL or [n_tok][D] fp32 (the normalized row before quantization).
 * Requires 1 <= n_tok <= SD_MAX_TOKENS, D % 32 == 0, 32 <= D <= 32768.
 */
int sd_rmsnorm_q8(const float* x, int64_t ldx, int n_tok, int64_t D, const float* gamma,
                  float eps, int8_t* xq, float* xd, float* y, sd_stream_t stream);

/*
 * sd_swiglu_q8 -- m = silu(g) * u with g = gu[t][0..F), u = gu[t][F..2F),
 * silu(g) = g / (1 + exp(-g)) in fp32, quantized to q8 blocks (as above).
 *   gu [n_tok][ldgu] fp32, ldgu >= 2F; xq [n_tok][F]; xd [n_tok][F/32];
 *   y NULL or [n_tok][F] fp32.
 * Requires 1 <= n_tok <= SD_MAX_TOKENS, F % 32 == 0.
 */
int sd_swiglu_q8(const float* gu, int64_t ldgu, int n_tok, int64_t F,
                 int8_t* xq, float* xd, float* y, sd_stream_t stream);

/*
 * sd_qgemv_q8_0_swiglu_q8 -- the FFN's gate|up projection and its SwiGLU in
 * one launch (ds4 pull request 604, "Commit walkthrough / Graph driver": the
 * FFN runs on the whole batch; the quantizer fused into its producer keeps
 * the consumer's convention, as "#1209 Speed up concurrent generation, fix
 * QFUSE, and improve prefill monitoring", "What changed and why" item 2,
 * requires).  Bitwise equal to sd_qgemv_q8_0_batch(w, 2F, K, ...) into gu
 * followed by sd_swiglu_q8(gu, 2F, n_tok, F, xq_out, xd_out, NULL); gu is
 * never written.
 *   w       q8_0 [2F][K]: F gate rows, then F up rows (as sd_qgemv_q8_0_batch).
 *   xq, xd  q8 activations of n_tok tokens (as sd_qgemv_q8_0_batch).
 *   xq_out  [n_tok][F] int8; xd_out [n_tok][F/32] fp32.  Neither may overlap
 *           xq or xd: workgroups still read the activations while others write.
 * Requires 1 <= n_tok <= 8, K % 256 == 0, K <= 4096, F % 32 == 0,
 * 32 <= F <= 2^29; otherwise SD_EINVAL / SD_EUNSUPPORTED and nothing runs.
 */
int sd_qgemv_q8_0_swiglu_q8(const void* w, int64_t F, int64_t K, const int8_t* xq,
                            const float* xd, int n_tok, int8_t* xq_out, float* xd_out,
                            sd_stream_t stream);

/*
 * sd_embed_f16 -- x[t][:] = fp32(table[tokens[t]][:]) (exact widening).
 *   table [V][H] fp16 bits; tokens [n_tok] int32 in [0, V) (device; out-of-range
 *   ids are clamped to V-1); x [n_tok][H] fp32.
 */
int sd_embed_f16(const uint16_t* table, int64_t V, int64_t H, const int32_t* tokens,
                 int n_tok, float* x, sd_stream_t stream);

/* Workspace bytes sd_argmax_rows needs (0 on invalid arguments). */
size_t sd_argmax_workspace_bytes(int n_tok, int64_t V);

/*
 * sd_argmax_rows -- greedy next token per row: the lowest index among equal
 * maxima of logits[t][0..V).  NaN never wins.  (Selection is exact, so the
 * result does not depend on how the row is split across workgroups.)
 *   logits [n_tok][ld] fp32; out [n_tok] int32; ws >= sd_argmax_workspace_bytes.
 */
int sd_argmax_rows(const float* logits, int64_t ld, int n_tok, int64_t V, int32_t* out,
                   void* ws, size_t ws_bytes, sd_stream_t stream);

/* ------------------------------------------------------------ measurement
 * sd_hbm_stream_read -- reads every byte of buf once (16-byte non-temporal
 * loads, the cache policy of the GEMV's weight stream) and writes nothing
 * but, in a case no real buffer hits, a word of sink.  Not part of the decode
 * step: the plain streaming read that the GEMV and attention kernels'
 * bandwidth is compared with, timed by the caller.
 *   buf   16-byte aligned device buffer of bytes bytes (bytes % 16 == 0, >= 16).
 *   sink  64 uint32 of device memory (contents unspecified afterwards).
 */
int sd_hbm_stream_read(const void* buf, size_t bytes, uint32_t* sink, sd_stream_t stream);

/* ------------------------------------------------------- the decode step */

/* One decoder layer's weights (device pointers). */
typedef struct sd_layer_weights {
  const void* w_qkv;      /* q8_0 [(H_q + 2 H_kv) D][hidden]: q rows, k rows, v rows */
  const void* w_o;        /* q8_0 [hidden][H_q D] */
  const void* w_gate_up;  /* q8_0 [2 ffn][hidden]: gate rows, then up rows */
  const void* w_down;     /* q8_0 [hidden][ffn] */
  const float* attn_norm; /* [hidden] */
  const float* ffn_norm;  /* [hidden] */
} sd_layer_weights;

/* A dense decoder model (shapes and pointers). */
typedef struct sd_model {
  int32_t n_layers, hidden, n_heads, n_kv_heads, head_dim, ffn, vocab;
  float rms_eps;
  double rope_theta;
  const uint16_t* tok_embd;        /* fp16 bits [vocab][hidden] */
  const float* out_norm;           /* [hidden] */
  const void* w_lm_head;           /* q8_0 [vocab][hidden] */
  const sd_layer_weights* layers;  /* [host] n_layers entries */
  int32_t n_rot;                   /* rotated dims: the last n_rot of each head (0 = head_dim) */
  int32_t window;                  /* attention window in positions (0 = the whole context) */
} sd_model;

/* One sequence's state for a step: caches [n_layers][capacity][H_kv][D] fp16. */
typedef struct sd_step_seq {
  uint16_t* k_cache;
  uint16_t* v_cache;
  int32_t capacity;
  int32_t pos;        /* position of this sequence's first token in the step */
  int32_t n_new;      /* its tokens in the step, 1..SD_ATTN_MAX_NEW (0 counts as 1):
                         positions pos .. pos + n_new - 1, ctx_len = pos + n_new */
  int32_t ring;       /* 1: the caches are rings of capacity positions (needs a model
                         window); position j in row j % capacity */
  const int32_t* block_table;  /* NULL, or [device] block table of a paged cache: the caches
                                  are pools [n_layers][capacity][H_kv][D] in blocks of
                                  block_size rows (64, 128 or 256), as in sd_seqview */
  int32_t block_size;
  int32_t kv_type;    /* SD_KV_F16 (k_cache, v_cache) or a quantized type: codes
                         k_q8 / v_q8 [n_layers][capacity][H_kv][D] int8 (q8_0) or
                         [n_layers][capacity][H_kv][D/2] nibble pairs (q4_0), and
                         scales k_d / v_d [n_layers][capacity][H_kv][D/32] fp16; all
                         sequences of a step share one kv_type */
  int8_t* k_q8;
  int8_t* v_q8;
  uint16_t* k_d;
  uint16_t* v_d;
} sd_step_seq;

/* Inputs and outputs of one step.  Token rows are packed by sequence:
 * sequence s owns rows n_new[0] + .. + n_new[s-1] onward; rows = the sum. */
typedef struct sd_step_io {
  int32_t n_seq;
  const sd_step_seq* seqs;   /* [host] n_seq entries */
  const int32_t* tokens;     /* [rows] input tokens */
  const int32_t* positions;  /* [rows] seqs[s].pos + i for row i of sequence s */
  float* logits;             /* [rows][vocab] */
  int32_t* next_tokens;      /* [rows] greedy argmax of logits */
  void* ws;                  /* workspace, 256-byte aligned */
  size_t ws_bytes;
} sd_step_io;

/* Workspace bytes sd_decode_step needs for `rows` token rows (the sum of n_new;
 * n_seq for one-token steps, at most SD_MAX_TOKENS) whose contexts are at most
 * max_ctx keys (0 on invalid arguments). */
size_t sd_decode_step_workspace_bytes(const sd_model* m, int rows, int max_ctx);

/*
 * sd_decode_step -- one batched decode step for n_seq sequences: embedding,
 * n_layers x (rmsnorm, QKV projection, pos-vector RoPE, KV append, multi-
 * sequence attention, O projection + residual, rmsnorm, gate/up projection,
 * SwiGLU, down projection + residual), final rmsnorm, LM head, argmax.  The
 * projections run once for all token rows (ds4 pull request 604, "2.
 * Single-GPU decode batches don't scale").  A sequence may bring up to
 * SD_ATTN_MAX_NEW tokens (a verify step for proposed tokens, "feat(qwen36):
 * complete concurrent serving implementation with speculation"); they attend
 * causally.  Every row's logits and token are bitwise those of one-token steps
 * of that sequence alone, run one after another over the same tokens.
 * Requires 1 <= n_seq <= SD_MAX_SEQS, rows <= SD_MAX_TOKENS, head_dim == 128,
 * n_heads % n_kv_heads == 0, hidden % 256 == 0, ffn % 256 == 0,
 * n_heads*head_dim % 256 == 0, 0 <= pos and, for plain caches,
 * pos + n_new <= capacity (rings and paged pools as in sd_seqview).
 */
int sd_decode_step(const sd_model* m, const sd_step_io* io, sd_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SEQDECODE_H */
