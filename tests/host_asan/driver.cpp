// Host-only driver of the C-ABI library built with the sanitizers: calls every
// entry point with valid arguments (the launchers are test doubles that record
// the argument block) and with invalid ones, and checks the statuses and the
// sizes the host code derived. Exit status 0 = every check passed; a sanitizer
// finding aborts the run. Device pointers are fake aligned addresses that the
// host code never dereferences.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <string>

#include "llama_attn.h"
#include "stub_launchers.hpp"

static int g_fail = 0;
#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      std::fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond); \
      ++g_fail;                                                       \
    }                                                                 \
  } while (0)

static void* fake(uintptr_t off = 0) { return reinterpret_cast<void*>(uintptr_t(1) << 20 | off); }

int main() {
  using la::g_stub;
  const int B = 2, S = 300, Hq = 32, Hkv = 8, D = 128;
  const int64_t qs[3] = {(int64_t)S * Hq * D, Hq * D, D};
  const int64_t ks[3] = {(int64_t)S * Hkv * D, Hkv * D, D};
  const int32_t* cu = reinterpret_cast<const int32_t*>(fake(0x100));

  // rope_qk / rope_qk_backward
  CHECK(rope_qk(fake(), fake(), qs, qs, fake(), fake(), ks, ks, LA_BF16, B, S, Hq, Hkv, D, nullptr,
                500000.0, 0, nullptr) == LA_OK);
  CHECK(g_stub.rope == 1 && g_stub.rope_q.H == Hq && g_stub.rope_k.H == Hkv);
  // theta_0 / 2 pi and theta_{D/2-1} / 2 pi
  CHECK(std::fabs(g_stub.angles.theta_rev[0] - 1.0 / (2 * M_PI)) < 1e-15);
  CHECK(std::fabs(g_stub.angles.theta_rev[D / 2 - 1] -
                  std::pow(500000.0, -(double)(D - 2) / D) / (2 * M_PI)) < 1e-15);
  CHECK(rope_qk_backward(fake(), fake(), qs, qs, nullptr, nullptr, nullptr, nullptr, LA_BF16, B, S, Hq, 0, D,
                         nullptr, 500000.0, 1, nullptr) == LA_OK);
  CHECK(g_stub.angles.theta_rev[0] < 0 && g_stub.angles.half == 1);
  CHECK(rope_qk(fake(), fake(), qs, qs, nullptr, nullptr, nullptr, nullptr, LA_BF16, B, S, Hq, 0, D, nullptr,
                -1.0, 0, nullptr) == LA_ERR_INVALID_ARG);
  CHECK(rope_qk(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, LA_BF16, B, S, Hq, Hkv,
                D, nullptr, 500000.0, 0, nullptr) == LA_ERR_INVALID_ARG);

  // gqa_prefill: 256 / g tokens per workgroup
  CHECK(gqa_prefill(fake(), fake(), fake(), fake(), nullptr, LA_BF16, B, S, Hq, Hkv, D, qs, ks, ks, qs, cu, 3,
                    0.f, nullptr) == LA_OK);
  CHECK(g_stub.pre.n_qtiles == (S + 63) / 64 && g_stub.G == 4 && g_stub.pre.q_off == 0);
  CHECK(std::fabs(g_stub.pre.scale - 1.f / std::sqrt(128.f)) < 1e-7f && g_stub.pre.rope_q == 0);
  // token stride too large for a 64-row tile's 32-bit byte offsets
  const int64_t big[3] = {(int64_t)1 << 40, (int64_t)1 << 25, D};
  CHECK(gqa_prefill(fake(), fake(), fake(), fake(), nullptr, LA_BF16, B, S, Hq, Hkv, D, qs, big, ks, qs, cu, 3,
                    0.f, nullptr) == LA_ERR_INVALID_ARG);
  CHECK(gqa_prefill(fake(), fake(), fake(), fake(), nullptr, LA_BF16, B, S, Hq, Hkv, D, qs, ks, big, qs, cu, 3,
                    0.f, nullptr) == LA_ERR_INVALID_ARG);
  // in-kernel query RoPE, chunked prefill: queries at positions S - Sq ..
  CHECK(gqa_prefill_rope(fake(), fake(), fake(), fake(), nullptr, LA_BF16, B, S, Hq, Hkv, D, qs, ks, ks, qs,
                         cu, 3, 0.f, nullptr, 500000.0, 0, nullptr) == LA_OK);
  CHECK(g_stub.pre.rope_q == 1 && g_stub.pre.theta_rev[0] > 0);
  CHECK(gqa_prefill_chunk(fake(), fake(), fake(), fake(), nullptr, LA_BF16, B, 40, S, Hq, Hkv, D, qs, ks, ks,
                          qs, cu, 3, 0.f, nullptr, 0.0, 0, nullptr) == LA_OK);
  CHECK(g_stub.pre.q_off == S - 40 && g_stub.pre.Sq == 40 && g_stub.pre.rope_q == 0);
  CHECK(gqa_prefill_chunk(fake(), fake(), fake(), fake(), nullptr, LA_BF16, B, S + 1, S, Hq, Hkv, D, qs, ks,
                          ks, qs, cu, 3, 0.f, nullptr, 0.0, 0, nullptr) == LA_ERR_INVALID_ARG);
  // split key ranges: merge launched after the prefill
  const int merges = g_stub.merge;
  CHECK(gqa_prefill_split(fake(), fake(), fake(), fake(), nullptr, LA_BF16, B, 40, S, Hq, Hkv, D, qs, ks, ks,
                          qs, cu, 3, 0.f, nullptr, 0.0, 0, 2, 3, (float*)fake(), (float*)fake(), nullptr) == LA_OK);
  CHECK(g_stub.merge == merges + 1 && g_stub.pre.split_tiles == 2 && g_stub.pre.max_splits == 3);
  CHECK(gqa_prefill_split(fake(), fake(), fake(), fake(), nullptr, LA_BF16, B, 40, S, Hq, Hkv, D, qs, ks, ks,
                          qs, cu, 3, 0.f, nullptr, 0.0, 0, 2, 2, (float*)fake(), (float*)fake(), nullptr) ==
        LA_ERR_INVALID_ARG);
  // ring step: first writes, later merges
  CHECK(gqa_prefill_ring_step(fake(), fake(), fake(), (float*)fake(), (float*)fake(), LA_BF16, B, 64, 128, 64,
                              0, Hq, Hkv, D, qs, ks, ks, cu, 3, 0.f, nullptr, 0.0, 0, 1, nullptr) == LA_OK);
  CHECK(g_stub.pre.acc_mode == 1 && g_stub.pre.q_off == 128 && g_stub.pre.k_off == 0);
  CHECK(gqa_prefill_ring_step(fake(), fake(), fake(), (float*)fake(), (float*)fake(), LA_BF16, B, 64, 128, 64,
                              64, Hq, Hkv, D, qs, ks, ks, cu, 3, 0.f, nullptr, 0.0, 0, 0, nullptr) == LA_OK);
  CHECK(g_stub.pre.acc_mode == 2 && g_stub.pre.k_off == 64);
  // a merging step whose keys all lie after the block's queries launches nothing
  {
    const int before = g_stub.prefill;
    CHECK(gqa_prefill_ring_step(fake(), fake(), fake(), (float*)fake(), (float*)fake(), LA_BF16, B, 64, 128, 64,
                                192, Hq, Hkv, D, qs, ks, ks, cu, 3, 0.f, nullptr, 0.0, 0, 0, nullptr) == LA_OK);
    CHECK(g_stub.prefill == before);
    // (the same shard as the first step still writes the accumulators)
    CHECK(gqa_prefill_ring_step(fake(), fake(), fake(), (float*)fake(), (float*)fake(), LA_BF16, B, 64, 128, 64,
                                192, Hq, Hkv, D, qs, ks, ks, cu, 3, 0.f, nullptr, 0.0, 0, 1, nullptr) == LA_OK);
    CHECK(g_stub.prefill == before + 1 && g_stub.pre.acc_mode == 1);
    // keys starting inside the block are launched
    CHECK(gqa_prefill_ring_step(fake(), fake(), fake(), (float*)fake(), (float*)fake(), LA_BF16, B, 64, 128, 64,
                                191, Hq, Hkv, D, qs, ks, ks, cu, 3, 0.f, nullptr, 0.0, 0, 0, nullptr) == LA_OK);
    CHECK(g_stub.prefill == before + 2);
  }
  CHECK(gqa_prefill_ring_finalize((float*)fake(), (float*)fake(), fake(), qs, nullptr, LA_BF16, B, 64, Hq, D,
                                  nullptr) == LA_OK);
  // the ring's last step: merges and writes o (acc_mode 3), or, also the first,
  // is the shard's plain prefill without accumulators; keys after the block's
  // queries make it the finalize alone
  {
    CHECK(gqa_prefill_ring_step_final(fake(), fake(), fake(), (float*)fake(), (float*)fake(), fake(), qs, nullptr,
                                      LA_BF16, B, 64, 128, 64, 64, Hq, Hkv, D, qs, ks, ks, cu, 3, 0.f, nullptr,
                                      0.0, 0, 0, nullptr) == LA_OK);
    CHECK(g_stub.pre.acc_mode == 3 && g_stub.pre.ring_out == 1 && g_stub.pre.o != nullptr &&
          g_stub.pre.os_s == qs[1]);
    CHECK(gqa_prefill_ring_step_final(fake(), fake(), fake(), nullptr, nullptr, fake(), qs, nullptr, LA_BF16, B,
                                      64, 128, 64, 128, Hq, Hkv, D, qs, ks, ks, cu, 3, 0.f, nullptr, 0.0, 0, 1,
                                      nullptr) == LA_OK);
    CHECK(g_stub.pre.acc_mode == 0 && g_stub.pre.ring_out == 1);
    CHECK(gqa_prefill_ring_step_final(fake(), fake(), fake(), nullptr, nullptr, fake(), qs, nullptr, LA_BF16, B,
                                      64, 128, 64, 64, Hq, Hkv, D, qs, ks, ks, cu, 3, 0.f, nullptr, 0.0, 0, 0,
                                      nullptr) == LA_ERR_INVALID_ARG);
    const int before = g_stub.prefill, merges = g_stub.merge;
    CHECK(gqa_prefill_ring_step_final(fake(), fake(), fake(), (float*)fake(), (float*)fake(), fake(), qs, nullptr,
                                      LA_BF16, B, 64, 128, 64, 192, Hq, Hkv, D, qs, ks, ks, cu, 3, 0.f, nullptr,
                                      0.0, 0, 0, nullptr) == LA_OK);
    CHECK(g_stub.prefill == before && g_stub.merge == merges + 1 && g_stub.pre_merge.max_splits == 1);
  }

  // decode, paged decode, combine
  const int64_t q2[2] = {Hq * D, D};
  const int64_t cs[3] = {(int64_t)Hkv * 4096 * D, 4096 * D, D};
  const int32_t* sl = reinterpret_cast<const int32_t*>(fake(0x200));
  CHECK(gqa_decode(fake(), q2, fake(), fake(), cs, sl, B, Hq, Hkv, D, 4096, 256, 16, 0.f, (float*)fake(),
                   (float*)fake(), nullptr) == LA_OK);
  CHECK(g_stub.dec.grid > 0 && g_stub.dec.max_splits == 16 && g_stub.G == 4);
  const int64_t ps[3] = {(int64_t)Hkv * 64 * D, 64 * D, D};
  CHECK(gqa_decode_paged(fake(), q2, fake(), fake(), ps, 64, sl, 64, sl, B, Hq, Hkv, D, 4096, 256, 16, 0.f,
                         (float*)fake(), (float*)fake(), nullptr) == LA_OK);
  CHECK(g_stub.dec.page_shift == 6 && g_stub.dec.bt_stride == 64);
  CHECK(gqa_decode_combine((float*)fake(), (float*)fake(), sl, B, Hq, D, 256, 16, fake(), q2, nullptr, LA_BF16,
                           nullptr) == LA_OK);
  CHECK(gqa_decode_combine((float*)fake(4), (float*)fake(), sl, B, Hq, D, 256, 16, fake(), q2, nullptr, LA_BF16,
                           nullptr) == LA_ERR_INVALID_ARG);
  CHECK(gqa_decode_combine((float*)fake(), (float*)fake(2), sl, B, Hq, D, 256, 16, fake(), q2, nullptr, LA_BF16,
                           nullptr) == LA_ERR_INVALID_ARG);

  // allocation-free decode: argument checks, then (no device here) the
  // scratch lookup fails before anything is launched
  const int dec_before = g_stub.decode;
  CHECK(gqa_decode_noalloc(fake(), q2, fake(), fake(), cs, sl, B, Hq, Hkv, D, 4096, 100, 0.f, fake(), q2, nullptr,
                           LA_BF16, nullptr) == LA_ERR_INVALID_ARG);
  CHECK(gqa_decode_noalloc(fake(), q2, fake(), fake(), cs, sl, B, Hq, Hkv, 96, 4096, 256, 0.f, fake(), q2, nullptr,
                           LA_BF16, nullptr) == LA_ERR_UNSUPPORTED);
  CHECK(gqa_decode_noalloc(fake(), q2, fake(), fake(), cs, sl, B, Hq, Hkv, D, 4096, 256, 0.f, nullptr, q2, nullptr,
                           LA_BF16, nullptr) == LA_ERR_INVALID_ARG);
  CHECK(gqa_decode_noalloc(fake(), q2, fake(), fake(), cs, sl, B, Hq, Hkv, D, 4096, 256, 0.f, fake(), q2, nullptr,
                           LA_BF16, nullptr) == LA_ERR_LAUNCH);
  CHECK(g_stub.decode == dec_before);
  CHECK(std::string(la_status_str(LA_ERR_SCRATCH)).find("scratch") != std::string::npos);

  // backward
  CHECK(gqa_attention_backward(fake(), fake(), fake(), fake(), fake(), (float*)fake(), (float*)fake(), fake(),
                               fake(), fake(), LA_BF16, B, S, Hq, Hkv, D, qs, ks, ks, qs, qs, qs, ks, ks, cu, 3,
                               0.f, nullptr, nullptr) == LA_OK);
  CHECK(g_stub.backward == 1 && g_stub.bwd.dkv_part == nullptr);
  CHECK(gqa_attention_backward(fake(), fake(), fake(), fake(), fake(), (float*)fake(), (float*)fake(), fake(),
                               fake(), fake(), LA_FP32, B, S, Hq, Hkv, D, qs, ks, ks, qs, qs, qs, ks, ks, cu, 3,
                               0.f, nullptr, nullptr) == LA_ERR_UNSUPPORTED);

  // LLAMA_ATTN_DEBUG=1 with no device to read the offsets from: the call is
  // refused before any launch
  setenv("LLAMA_ATTN_DEBUG", "1", 1);
  const int before = g_stub.prefill;
  CHECK(gqa_prefill(fake(), fake(), fake(), fake(), nullptr, LA_BF16, B, S, Hq, Hkv, D, qs, ks, ks, qs, cu, 3,
                    0.f, nullptr) == LA_ERR_INVALID_ARG);
  CHECK(g_stub.prefill == before);
  // without device contents to check (no offsets) the call proceeds
  CHECK(gqa_prefill(fake(), fake(), fake(), fake(), nullptr, LA_BF16, B, S, Hq, Hkv, D, qs, ks, ks, qs,
                    nullptr, 1, 0.f, nullptr) == LA_OK);
  unsetenv("LLAMA_ATTN_DEBUG");

  if (g_fail) std::fprintf(stderr, "%d checks failed\n", g_fail);
  else std::printf("all host checks passed\n");
  return g_fail ? 1 : 0;
}
