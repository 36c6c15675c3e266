// Host-side checks of the C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code (device code is not
// instrumented) and run on the CPU: every call here is rejected by the host
// validation or is a size query, so no kernel is launched and no device
// pointer is dereferenced.  Exits non-zero on the first unexpected result;
// the sanitizers abort on any memory error or undefined behaviour.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>

#include "seqdecode.h"

namespace {

int failures = 0;

void expect(long long got, long long want, const char* what, int line) {
  if (got != want) {
    std::fprintf(stderr, "line %d: %s returned %lld, expected %lld\n", line, what, got, want);
    ++failures;
  }
}
#define EXPECT(call, want) expect((long long)(call), (long long)(want), #call, __LINE__)

void* const FAKE = reinterpret_cast<void*>(0x10000);  // never dereferenced
void* const ODD = reinterpret_cast<void*>(0x10002);
template <class T>
T* fk() { return static_cast<T*>(FAKE); }
template <class T>
T* od() { return static_cast<T*>(ODD); }

sd_seqview view(int ctx, int cap, int64_t ld_tok = 1024, int64_t ld_head = 128) {
  sd_seqview v{};
  v.k = fk<uint16_t>();
  v.v = fk<uint16_t>();
  v.ctx_len = ctx;
  v.capacity = cap;
  v.ld_tok = ld_tok;
  v.ld_head = ld_head;
  return v;
}

void gemv_and_glue() {
  EXPECT(sd_qgemv_q8_0_batch(nullptr, 64, 256, fk<int8_t>(), fk<float>(), 1, nullptr, fk<float>(), 64, nullptr), SD_EINVAL);
  EXPECT(sd_qgemv_q8_0_batch(FAKE, 64, 256, fk<int8_t>(), fk<float>(), 0, nullptr, fk<float>(), 64, nullptr), SD_EINVAL);
  EXPECT(sd_qgemv_q8_0_batch(FAKE, 64, 256, fk<int8_t>(), fk<float>(), 17, nullptr, fk<float>(), 64, nullptr), SD_EINVAL);
  EXPECT(sd_qgemv_q8_0_batch(FAKE, 64, 128, fk<int8_t>(), fk<float>(), 1, nullptr, fk<float>(), 64, nullptr), SD_EUNSUPPORTED);
  EXPECT(sd_qgemv_q8_0_batch(FAKE, 64, 4000, fk<int8_t>(), fk<float>(), 1, nullptr, fk<float>(), 64, nullptr), SD_EUNSUPPORTED);
  EXPECT(sd_qgemv_q8_0_batch(FAKE, 64, 256, fk<int8_t>(), fk<float>(), 1, nullptr, fk<float>(), 63, nullptr), SD_EINVAL);
  EXPECT(sd_qgemv_q8_0_batch(ODD, 64, 256, fk<int8_t>(), fk<float>(), 1, nullptr, fk<float>(), 64, nullptr), SD_EALIGN);
  EXPECT(sd_qgemv_q8_0_batch(FAKE, 64, 256, od<int8_t>(), fk<float>(), 1, nullptr, fk<float>(), 64, nullptr), SD_EALIGN);
  EXPECT(sd_qgemv_q8_0_batch(FAKE, 0, 14336, fk<int8_t>(), fk<float>(), 16, nullptr, fk<float>(), 64, nullptr), SD_EINVAL);
  EXPECT(sd_qgemv_q8_0_batch(FAKE, (int64_t)1 << 40, 256, fk<int8_t>(), fk<float>(), 1, nullptr, fk<float>(), (int64_t)1 << 40, nullptr), SD_EINVAL);
  for (int path : {-1, 3, 99})
    EXPECT(sd_qgemv_q8_0_batch_path(FAKE, 64, 256, fk<int8_t>(), fk<float>(), 1, nullptr, fk<float>(), 64, path, nullptr), SD_EINVAL);
  EXPECT(sd_qgemv_q8_0_swiglu_q8(FAKE, 48, 256, fk<int8_t>(), fk<float>(), 1, fk<int8_t>(), fk<float>(), nullptr), SD_EUNSUPPORTED);
  EXPECT(sd_qgemv_q8_0_swiglu_q8(FAKE, 64, 4096, fk<int8_t>(), fk<float>(), 9, fk<int8_t>(), fk<float>(), nullptr), SD_EUNSUPPORTED);
  EXPECT(sd_quantize_q8_act(fk<float>(), 64, 1, 48, fk<int8_t>(), fk<float>(), nullptr), SD_EUNSUPPORTED);
  EXPECT(sd_quantize_q8_act(fk<float>(), 64, 17, 64, fk<int8_t>(), fk<float>(), nullptr), SD_EINVAL);
  EXPECT(sd_rope_posvec(fk<float>(), 4, 32, 128, 4096, 128, fk<int32_t>(), 1e6, 127, nullptr), SD_EINVAL);
  EXPECT(sd_rope_posvec(fk<float>(), 4, 32, 128, 4096, 128, fk<int32_t>(), -1.0, 128, nullptr), SD_EINVAL);
  EXPECT(sd_rope_posvec(od<float>(), 4, 32, 128, 4096, 128, fk<int32_t>(), 1e6, 128, nullptr), SD_EALIGN);
  EXPECT(sd_rmsnorm_q8(fk<float>(), 100, 1, 100, fk<float>(), 1e-6f, fk<int8_t>(), fk<float>(), nullptr, nullptr), SD_EUNSUPPORTED);
  EXPECT(sd_rmsnorm_q8(fk<float>(), 128, 1, 128, fk<float>(), -1.0f, fk<int8_t>(), fk<float>(), nullptr, nullptr), SD_EINVAL);
  EXPECT(sd_swiglu_q8(fk<float>(), 100, 1, 64, fk<int8_t>(), fk<float>(), nullptr, nullptr), SD_EINVAL);
  EXPECT(sd_argmax_workspace_bytes(4, 151936), 4 * 19 * 8);
  EXPECT(sd_argmax_rows(fk<float>(), 151936, 4, 151936, fk<int32_t>(), FAKE, 4 * 19 * 8 - 1, nullptr), SD_EWORKSPACE);
  EXPECT(sd_argmax_rows(fk<float>(), 10, 1, 11, fk<int32_t>(), FAKE, 64, nullptr), SD_EINVAL);
  EXPECT(sd_embed_f16(fk<uint16_t>(), 0, 16, fk<int32_t>(), 1, fk<float>(), nullptr), SD_EINVAL);
  EXPECT(sd_hbm_stream_read(nullptr, 64, fk<uint32_t>(), nullptr), SD_EINVAL);
  EXPECT(sd_hbm_stream_read(FAKE, 40, fk<uint32_t>(), nullptr), SD_EINVAL);
  for (int code = -6; code <= 1; ++code)
    if (!sd_status_string(code)) ++failures;
}

void attention() {
  sd_seqview v5[5] = {view(10, 16), view(10, 16), view(10, 16), view(10, 16), view(10, 16)};
  EXPECT(sd_decode_attn_multiseq(fk<float>(), 4096, v5, 5, 32, 8, 128, 0.088f, fk<float>(), FAKE, 1 << 20, nullptr), SD_EINVAL);
  sd_seqview v1[1] = {view(10, 16)};
  EXPECT(sd_decode_attn_multiseq(fk<float>(), 4096, v1, 1, 32, 8, 64, 0.088f, fk<float>(), FAKE, 1 << 20, nullptr), SD_EUNSUPPORTED);
  EXPECT(sd_decode_attn_multiseq(fk<float>(), 4096, v1, 1, 30, 8, 128, 0.088f, fk<float>(), FAKE, 1 << 20, nullptr), SD_EINVAL);
  const size_t need = sd_decode_attn_workspace_bytes(v1, 1, 32, 128);
  EXPECT(need, 1 * 32 * 132 * 4);
  EXPECT(sd_decode_attn_multiseq(fk<float>(), 4096, v1, 1, 32, 8, 128, 0.088f, fk<float>(), FAKE, need - 4, nullptr), SD_EWORKSPACE);
  sd_seqview over[1] = {view(17, 16)};
  EXPECT(sd_decode_attn_multiseq(fk<float>(), 4096, over, 1, 32, 8, 128, 0.088f, fk<float>(), FAKE, 1 << 20, nullptr), SD_EINVAL);
  sd_seqview mis[1] = {view(10, 16)};
  mis[0].k = od<uint16_t>();
  EXPECT(sd_decode_attn_multiseq(fk<float>(), 4096, mis, 1, 32, 8, 128, 0.088f, fk<float>(), FAKE, 1 << 20, nullptr), SD_EALIGN);
  // the maximum span and one key past it
  sd_seqview big[1] = {view(SD_MAX_CTX, SD_MAX_CTX)};
  if (sd_decode_attn_workspace_bytes(big, 1, 32, 128) == 0) ++failures;
  big[0].ctx_len = SD_MAX_CTX + 1;
  big[0].capacity = SD_MAX_CTX + 1;
  EXPECT(sd_decode_attn_workspace_bytes(big, 1, 32, 128), 0);
  // windows, rings, paged views, q8 views
  sd_seqview ring[1] = {view(5000, 300)};
  ring[0].window = 256;
  ring[0].ring = 1;
  EXPECT(sd_decode_attn_workspace_bytes(ring, 1, 32, 128), 2 * 32 * 132 * 4);
  ring[0].capacity = 200;
  EXPECT(sd_decode_attn_workspace_bytes(ring, 1, 32, 128), 0);
  sd_seqview paged[1] = {view(5000, 1024)};
  paged[0].block_table = fk<int32_t>();
  paged[0].block_size = 64;
  EXPECT(sd_decode_attn_workspace_bytes(paged, 1, 32, 128), (32 + 12) * 32 * 132 * 4);
  paged[0].block_size = 48;
  EXPECT(sd_decode_attn_workspace_bytes(paged, 1, 32, 128), 0);
  sd_seqview q8[1] = {view(100, 128)};
  q8[0].k = nullptr;
  q8[0].v = nullptr;
  q8[0].kv_type = SD_KV_Q8_0;
  q8[0].k_q8 = fk<int8_t>();
  q8[0].v_q8 = fk<int8_t>();
  q8[0].k_d = fk<uint16_t>();
  q8[0].v_d = fk<uint16_t>();
  EXPECT(sd_decode_attn_workspace_bytes(q8, 1, 32, 128), 2 * 32 * 132 * 4);
  q8[0].k_d = reinterpret_cast<uint16_t*>(0x10004);
  EXPECT(sd_decode_attn_multiseq(fk<float>(), 4096, q8, 1, 32, 8, 128, 0.088f, fk<float>(), FAKE, 1 << 30, nullptr), SD_EALIGN);
  // verify bursts
  sd_seqview v2[2] = {view(258, 300), view(3, 16)};
  int32_t nn[2] = {4, 3};
  EXPECT(sd_decode_attn_verify_workspace_bytes(v2, nn, 2, 32, 128), (5 * 4 + 1 * 3) * 32 * 132 * 4);
  int32_t bad[2] = {4, 4};  // more tokens than keys
  EXPECT(sd_decode_attn_verify_workspace_bytes(v2, bad, 2, 32, 128), 0);
  // the allocation-free entry refuses partials beyond its scratch array
  sd_seqview huge[4] = {view(65536, 65536), view(65536, 65536), view(65536, 65536), view(65536, 65536)};
  EXPECT(sd_decode_attn_multiseq_noalloc(fk<float>(), 4096, huge, 4, 32, 8, 128, 0.088f, fk<float>(), nullptr), SD_EWORKSPACE);
  // random views: the size query must never misbehave (sanitizers watch it)
  std::mt19937 rng(12345);
  for (int it = 0; it < 20000; ++it) {
    sd_seqview vs[4];
    int32_t news[4];
    const int n = 1 + (int)(rng() % 4);
    for (int s = 0; s < n; ++s) {
      const int ctx = (int)(rng() % 70000) - 2;
      vs[s] = view(ctx, (int)(rng() % 70000) - 2);
      vs[s].window = (int)(rng() % 5000) - 1;
      vs[s].ring = (int)(rng() % 3);
      if (rng() % 3 == 0) {
        vs[s].block_table = fk<int32_t>();
        vs[s].block_size = 64 << (rng() % 3);
      }
      news[s] = (int)(rng() % 6);
    }
    const size_t a = sd_decode_attn_workspace_bytes(vs, n, 32, 128);
    const size_t b = sd_decode_attn_verify_workspace_bytes(vs, news, n, 32, 128);
    if (a > ((size_t)1 << 40) || b > ((size_t)1 << 40)) ++failures;
  }
}

void step() {
  sd_layer_weights lw{FAKE, FAKE, FAKE, FAKE, fk<float>(), fk<float>()};
  sd_model m{};
  m.n_layers = 1;
  m.hidden = 4096;
  m.n_heads = 32;
  m.n_kv_heads = 8;
  m.head_dim = 128;
  m.ffn = 14336;
  m.vocab = 1000;
  m.rms_eps = 1e-6f;
  m.rope_theta = 1e6;
  m.tok_embd = fk<uint16_t>();
  m.out_norm = fk<float>();
  m.w_lm_head = FAKE;
  m.layers = &lw;
  const size_t need = sd_decode_step_workspace_bytes(&m, 4, 32768);
  if (need == 0) ++failures;
  EXPECT(sd_decode_step_workspace_bytes(&m, 17, 32768), 0);
  sd_model bad = m;
  bad.head_dim = 64;
  EXPECT(sd_decode_step_workspace_bytes(&bad, 1, 16), 0);
  sd_step_seq sq{};
  sq.k_cache = fk<uint16_t>();
  sq.v_cache = fk<uint16_t>();
  sq.capacity = 16;
  sq.pos = 16;  // pos == capacity
  sd_step_io io{};
  io.n_seq = 1;
  io.seqs = &sq;
  io.tokens = fk<int32_t>();
  io.positions = fk<int32_t>();
  io.logits = fk<float>();
  io.next_tokens = fk<int32_t>();
  io.ws = reinterpret_cast<void*>(0x100000);
  io.ws_bytes = (size_t)1 << 30;
  EXPECT(sd_decode_step(&m, &io, nullptr), SD_EINVAL);
  EXPECT(sd_decode_step(&bad, &io, nullptr), SD_EUNSUPPORTED);
  sq.pos = 3;
  sq.n_new = 5;
  EXPECT(sd_decode_step(&m, &io, nullptr), SD_EINVAL);
  sq.n_new = 4;
  io.ws_bytes = 16;
  EXPECT(sd_decode_step(&m, &io, nullptr), SD_EWORKSPACE);
  std::mt19937 rng(777);
  for (int it = 0; it < 20000; ++it) {
    sd_model r = m;
    r.n_layers = 1 + (int)(rng() % 3);
    r.hidden = (int)(rng() % 40000) - 10;
    r.ffn = (int)(rng() % 40000) - 10;
    r.n_kv_heads = (int)(rng() % 20) - 1;
    r.n_heads = 4 * r.n_kv_heads + (int)(rng() % 2);
    r.vocab = (int)(rng() % 300000) - 5;
    r.n_rot = (int)(rng() % 140) - 4;
    r.window = (int)(rng() % 5000) - 2;
    sd_layer_weights lws[3] = {lw, lw, lw};
    r.layers = lws;
    const size_t b = sd_decode_step_workspace_bytes(&r, 1 + (int)(rng() % 18) - 1, (int)(rng() % 600000) - 5);
    if (b > ((size_t)1 << 44)) ++failures;
  }
}

}  // namespace

int main() {
  if (sd_abi_version() != SD_ABI_VERSION) ++failures;
  gemv_and_glue();
  attention();
  step();
  if (failures) {
    std::fprintf(stderr, "%d unexpected results\n", failures);
    return 1;
  }
  std::printf("abi checks passed\n");
  return 0;
}
