// Host side of the C ABI declared in include/llama_attn.h: argument checks
// (all made before anything is enqueued), variant selection, and launches on
// the caller's stream. The library allocates no device memory; its only
// state is a per-device compute-unit count read once.
#include "llama_attn.h"

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <mutex>
#include <vector>

#include "kernels.hpp"

namespace {

constexpr int kVersion = 100;  // 0.1.0

bool supported_d(int D) { return D == 64 || D == 128; }
bool supported_g(int G) { return G == 1 || G == 2 || G == 4 || G == 8 || G == 16; }
int elem_size(la_dtype dt) { return dt == LA_BF16 ? 2 : 4; }
bool known_dtype(la_dtype dt) { return dt == LA_BF16 || dt == LA_FP32; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Strides must be non-negative multiples of 16 bytes' worth of elements.
bool strides_ok(const int64_t* s, int n, int esize) {
  if (s == nullptr) return false;
  const int64_t q = 16 / esize;
  for (int i = 0; i < n; ++i)
    if (s[i] < 0 || s[i] % q != 0) return false;
  return true;
}

la_status launched(hipError_t e) { return e == hipSuccess ? LA_OK : LA_ERR_LAUNCH; }

// ---- compute units per device, read once per process --------------------
constexpr int kMaxDevices = 64;
int g_cu_count[kMaxDevices];
std::once_flag g_cu_once;

// The current device's compute-unit count (the persistent decode grid);
// 256 if the runtime cannot tell. The table is filled once, under
// std::call_once, so concurrent first calls from several threads are safe.
int current_cu_count() {
  std::call_once(g_cu_once, [] {
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess) n = 0;
    for (int d = 0; d < kMaxDevices; ++d) {
      int c = 0;
      if (d >= n || hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, d) != hipSuccess) c = 0;
      g_cu_count[d] = c > 0 ? c : 256;
    }
  });
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  return g_cu_count[dev];
}

// ---- LLAMA_ATTN_DEBUG=1: contents of the device index arrays -------------
// The environment variable is read at every call. When it is "1", a call
// first copies the device-resident index arrays it was given (document
// offsets, sequence lengths, positions, block tables) to the host on the
// caller's stream, waits for that stream, and returns LA_ERR_INVALID_ARG
// without launching anything if a value breaks the call's contract. This
// synchronises the stream, so it is a debugging aid, not for graph capture.
bool debug_mode() {
  const char* e = std::getenv("LLAMA_ATTN_DEBUG");
  return e != nullptr && e[0] == '1' && e[1] == '\0';
}

// The persistent prefill grid for n_items work items: one workgroup per
// compute unit where the items number at least kPersistentItemsPerCu per
// compute unit (a persistent workgroup draws its next item when the current
// one starts, which costs balance where each workgroup runs only a few
// items), else 0 (one workgroup per item). LLAMA_ATTN_PERSISTENT, when it
// holds a number, overrides this: 0 turns the persistent grid off, n > 0 sets
// it to n workgroups wherever the items outnumber them (so that small
// problems run many items per workgroup).
constexpr long long kPersistentItemsPerCu = 16;
int persistent_grid(long long n_items) {
  const char* e = std::getenv("LLAMA_ATTN_PERSISTENT");
  if (e != nullptr && e[0] != '\0') {
    char* end = nullptr;
    const long n = std::strtol(e, &end, 10);
    if (end != e && *end == '\0' && n >= 0 && n <= 65535) return n_items > n ? (int)n : 0;
  }
  const int ncu = current_cu_count();
  return n_items >= kPersistentItemsPerCu * ncu ? ncu : 0;
}

bool fetch_i32(const int32_t* d, int64_t n, hipStream_t st, std::vector<int32_t>& h) {
  h.assign((size_t)std::max<int64_t>(n, 0), 0);
  if (n <= 0) return true;
  if (hipMemcpyAsync(h.data(), d, (size_t)n * sizeof(int32_t), hipMemcpyDeviceToHost, st) != hipSuccess)
    return false;
  return hipStreamSynchronize(st) == hipSuccess;
}

// Document offsets [B, n_docs + 1]: each row starts at 0, never decreases and
// ends at `end` (at or past `end` when exact is false).
bool docs_ok(const int32_t* cu, int B, int n_docs, int64_t end, bool exact, hipStream_t st) {
  if (!cu) return true;
  std::vector<int32_t> h;
  if (!fetch_i32(cu, (int64_t)B * (n_docs + 1), st, h)) return false;
  for (int b = 0; b < B; ++b) {
    const int32_t* r = h.data() + (size_t)b * (n_docs + 1);
    if (r[0] != 0) return false;
    for (int d = 0; d < n_docs; ++d)
      if (r[d + 1] < r[d]) return false;
    if (exact ? r[n_docs] != end : r[n_docs] < end) return false;
  }
  return true;
}

// Positions [n]: non-negative token positions.
bool positions_ok(const int32_t* pos, int64_t n, hipStream_t st) {
  if (!pos) return true;
  std::vector<int32_t> h;
  if (!fetch_i32(pos, n, st, h)) return false;
  for (int32_t x : h)
    if (x < 0) return false;
  return true;
}

// Sequence lengths [B]: lo <= L <= hi.
bool lens_ok(const int32_t* lens, int B, int64_t lo, int64_t hi, hipStream_t st) {
  std::vector<int32_t> h;
  if (!fetch_i32(lens, B, st, h)) return false;
  for (int32_t x : h)
    if (x < lo || x > hi) return false;
  return true;
}

// Block table rows [B] of bt_stride entries: the pages that hold slots
// 0 .. seq_lens[b] - 1 are named by non-negative ids.
bool block_table_ok(const int32_t* table, int bt_stride, const int32_t* lens, int B, int page_size,
                    hipStream_t st) {
  std::vector<int32_t> t, l;
  if (!fetch_i32(lens, B, st, l) || !fetch_i32(table, (int64_t)B * bt_stride, st, t)) return false;
  for (int b = 0; b < B; ++b) {
    const int64_t pages = ((int64_t)l[b] + page_size - 1) / page_size;
    if (pages > bt_stride) return false;
    for (int64_t j = 0; j < pages; ++j)
      if (t[(size_t)b * bt_stride + j] < 0) return false;
  }
  return true;
}

// theta_k = base^(-2k/D) (the RoPE frequencies), divided by 2 pi: the kernels
// form the angles in revolutions
void theta_revolutions(double base, int D, double* out) {
  for (int kk = 0; kk < D / 2; ++kk)
    out[kk] = std::exp2(-(2.0 * kk / D) * std::log2(base)) / 6.283185307179586476925286766559;
}

}  // namespace

extern "C" {

const char* la_status_str(la_status s) {
  switch (s) {
    case LA_OK: return "ok";
    case LA_ERR_INVALID_ARG: return "invalid argument";
    case LA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case LA_ERR_LAUNCH: return "kernel launch failed";
    case LA_ERR_SCRATCH: return "working set exceeds the allocation-free scratch buffer";
  }
  return "unknown status";
}

int la_version(void) { return kVersion; }

}  // extern "C"

namespace {

// rope_qk and rope_qk_backward: direction +1 rotates by the position's angles,
// -1 by their negatives (the transpose of the rotation)
la_status rope_impl(const void* q_in, void* q_out, const int64_t q_in_strides[3],
                    const int64_t q_out_strides[3], const void* k_in, void* k_out,
                    const int64_t k_in_strides[3], const int64_t k_out_strides[3], la_dtype dt,
                    int B, int S, int Hq, int Hkv, int D, const int32_t* positions,
                    double rope_base, int rope_pairing, int direction, hipStream_t stream) {
  if (!known_dtype(dt)) return LA_ERR_UNSUPPORTED;
  const bool has_q = q_in != nullptr || q_out != nullptr;
  const bool has_k = k_in != nullptr || k_out != nullptr;
  if (!has_q && !has_k) return LA_ERR_INVALID_ARG;
  if (has_q && (q_in == nullptr || q_out == nullptr)) return LA_ERR_INVALID_ARG;
  if (has_k && (k_in == nullptr || k_out == nullptr)) return LA_ERR_INVALID_ARG;
  if (B < 1 || S < 1 || (has_q && Hq < 1) || (has_k && Hkv < 1)) return LA_ERR_INVALID_ARG;
  if (!(rope_base > 0.0) || !std::isfinite(rope_base)) return LA_ERR_INVALID_ARG;
  if (rope_pairing != 0 && rope_pairing != 1) return LA_ERR_INVALID_ARG;
  if ((long long)B * S > 0x7fffffffLL) return LA_ERR_INVALID_ARG;
  if (!supported_d(D)) return LA_ERR_UNSUPPORTED;
  const int es = elem_size(dt);
  if (has_q && (!aligned16(q_in) || !aligned16(q_out) || !strides_ok(q_in_strides, 3, es) ||
                !strides_ok(q_out_strides, 3, es)))
    return LA_ERR_INVALID_ARG;
  if (has_k && (!aligned16(k_in) || !aligned16(k_out) || !strides_ok(k_in_strides, 3, es) ||
                !strides_ok(k_out_strides, 3, es)))
    return LA_ERR_INVALID_ARG;

  if (debug_mode() && !positions_ok(positions, (int64_t)B * S, stream)) return LA_ERR_INVALID_ARG;

  la::RopeArgs qa{}, ka{};
  if (has_q) {
    qa = la::RopeArgs{q_in, q_out, q_in_strides[0], q_in_strides[1], q_in_strides[2],
                      q_out_strides[0], q_out_strides[1], q_out_strides[2], Hq, positions, B, S};
  }
  if (has_k) {
    ka = la::RopeArgs{k_in, k_out, k_in_strides[0], k_in_strides[1], k_in_strides[2],
                      k_out_strides[0], k_out_strides[1], k_out_strides[2], Hkv, positions, B, S};
  }
  la::RopeAngles ang{};
  theta_revolutions(rope_base, D, ang.theta_rev);
  if (direction < 0)
    for (int kk = 0; kk < D / 2; ++kk) ang.theta_rev[kk] = -ang.theta_rev[kk];
  ang.half = rope_pairing;
  return launched(la::launch_rope_pair(qa, ka, ang, D, dt == LA_BF16 ? 0 : 1, stream));
}

}  // namespace

extern "C" {

la_status rope_qk(const void* q_in, void* q_out, const int64_t q_in_strides[3],
                  const int64_t q_out_strides[3], const void* k_in, void* k_out,
                  const int64_t k_in_strides[3], const int64_t k_out_strides[3], la_dtype dt,
                  int B, int S, int Hq, int Hkv, int D, const int32_t* positions,
                  double rope_base, int rope_pairing, hipStream_t stream) {
  return rope_impl(q_in, q_out, q_in_strides, q_out_strides, k_in, k_out, k_in_strides,
                   k_out_strides, dt, B, S, Hq, Hkv, D, positions, rope_base, rope_pairing, 1,
                   stream);
}

la_status rope_qk_backward(const void* dq_in, void* dq_out, const int64_t dq_in_strides[3],
                           const int64_t dq_out_strides[3], const void* dk_in, void* dk_out,
                           const int64_t dk_in_strides[3], const int64_t dk_out_strides[3],
                           la_dtype dt, int B, int S, int Hq, int Hkv, int D,
                           const int32_t* positions, double rope_base, int rope_pairing,
                           hipStream_t stream) {
  return rope_impl(dq_in, dq_out, dq_in_strides, dq_out_strides, dk_in, dk_out, dk_in_strides,
                   dk_out_strides, dt, B, S, Hq, Hkv, D, positions, rope_base, rope_pairing, -1,
                   stream);
}

}  // extern "C"

namespace {

// gqa_prefill, gqa_prefill_rope and gqa_prefill_chunk: the Sq queries of each
// sequence are its last Sq tokens of S; rope_base > 0 asks the kernel to
// rotate the queries itself (positions as in rope_qk)
la_status prefill_impl(const void* q, const void* k, const void* v, void* o, float* lse,
                       la_dtype dt, int B, int Sq, int S, int Hq, int Hkv, int D,
                       const int64_t q_strides[3], const int64_t k_strides[3],
                       const int64_t v_strides[3], const int64_t o_strides[3],
                       const int32_t* cu_docs, int n_docs, float softmax_scale,
                       const int32_t* positions, double rope_base, int rope_pairing,
                       hipStream_t stream, int split_tiles = 0, int max_splits = 0, float* o_part = nullptr,
                       float* lse_part = nullptr, bool ring = false, int q_off = 0, int k_off = 0,
                       int acc_mode = 0, float* o_acc = nullptr, float* lse_acc = nullptr,
                       bool ring_out = false) {
  if (!known_dtype(dt)) return LA_ERR_UNSUPPORTED;
  // (a ring step writes o only as the ring's last step)
  const bool has_o = !ring || ring_out;
  if (!q || !k || !v || (!o && has_o)) return LA_ERR_INVALID_ARG;
  if (rope_pairing != 0 && rope_pairing != 1) return LA_ERR_INVALID_ARG;
  if (B < 1 || S < 1 || Hq < 1 || Hkv < 1) return LA_ERR_INVALID_ARG;
  if (Sq < 1 || (!ring && Sq > S)) return LA_ERR_INVALID_ARG;
  if (ring) {
    if (q_off < 0 || k_off < 0 || (long long)q_off + Sq > 0x7fffffffLL ||
        (long long)k_off + S > 0x7fffffffLL)
      return LA_ERR_INVALID_ARG;
    if (acc_mode != 0 && (!o_acc || !lse_acc || !aligned16(o_acc))) return LA_ERR_INVALID_ARG;
  }
  if (cu_docs && n_docs < 1) return LA_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return LA_ERR_INVALID_ARG;
  if (!supported_d(D) || !supported_g(Hq / Hkv)) return LA_ERR_UNSUPPORTED;
  const int es = elem_size(dt);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || (has_o && !aligned16(o))) return LA_ERR_INVALID_ARG;
  if (!strides_ok(q_strides, 3, es) || !strides_ok(k_strides, 3, es) ||
      !strides_ok(v_strides, 3, es) || (has_o && !strides_ok(o_strides, 3, es)))
    return LA_ERR_INVALID_ARG;
  // key/value rows of consecutive tokens may not overlap (tiles are fetched
  // with a byte range that ends at the last token's row)
  if (k_strides[1] < D || v_strides[1] < D) return LA_ERR_INVALID_ARG;
  // a 64-key tile is fetched through one buffer descriptor whose per-lane byte
  // offsets are 32-bit: its rows must span less than 2 GiB
  if (64 * k_strides[1] * es > 0x7fffffffLL || 64 * v_strides[1] * es > 0x7fffffffLL)
    return LA_ERR_INVALID_ARG;
  if (!std::isfinite(softmax_scale)) return LA_ERR_INVALID_ARG;
  const int G = Hq / Hkv;
  const int tq = la::prefill_tokens_per_block(G);
  const long long n_qtiles = (Sq + tq - 1) / tq;
  if ((long long)B * Hkv * n_qtiles > 0x7fffffffLL) return LA_ERR_INVALID_ARG;
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)D);
  if (split_tiles != 0) {
    if (split_tiles < 1 || !o_part || !lse_part || !aligned16(o_part)) return LA_ERR_INVALID_ARG;
    // a query tile's key range holds at most ceil(S / 64) tiles of 64 keys
    const long long need = ((S + 63) / 64 + split_tiles - 1) / split_tiles;
    if (max_splits < need || max_splits > 65535) return LA_ERR_INVALID_ARG;
    if ((long long)max_splits * B * Sq * Hq * D > (1LL << 46)) return LA_ERR_INVALID_ARG;
  }

  if (debug_mode()) {
    // key positions end at S (or, for a ring step, the offsets cover both shards)
    const int64_t end = ring ? std::max<int64_t>((int64_t)q_off + Sq, (int64_t)k_off + S) : S;
    if (!docs_ok(cu_docs, B, n_docs, end, !ring, stream)) return LA_ERR_INVALID_ARG;
    if (rope_base > 0.0 && !positions_ok(positions, (int64_t)B * Sq, stream)) return LA_ERR_INVALID_ARG;
  }

  // a ring step that merges (acc_mode 2) keys that all lie after the block's
  // queries: the causal mask hides every key from every row, and the
  // accumulators stay as they are, so nothing is launched
  if (ring && acc_mode == 2 && (long long)k_off >= (long long)q_off + Sq) return LA_OK;
  // the same as the ring's last step: the accumulators are the result
  if (ring && acc_mode == 3 && (long long)k_off >= (long long)q_off + Sq) {
    la::PrefillArgs f{};
    f.o = o; f.lse = lse;
    f.os_b = o_strides[0]; f.os_s = o_strides[1]; f.os_h = o_strides[2];
    f.B = B; f.Sq = Sq; f.Hq = Hq;
    f.max_splits = 1;
    f.o_part = o_acc;
    f.lse_part = lse_acc;
    return launched(la::launch_ring_finalize(f, D, dt == LA_BF16 ? 0 : 1, stream));
  }

  la::PrefillArgs a{};
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.qs_b = q_strides[0]; a.qs_s = q_strides[1]; a.qs_h = q_strides[2];
  a.ks_b = k_strides[0]; a.ks_s = k_strides[1]; a.ks_h = k_strides[2];
  a.vs_b = v_strides[0]; a.vs_s = v_strides[1]; a.vs_h = v_strides[2];
  if (has_o) {
    a.os_b = o_strides[0]; a.os_s = o_strides[1]; a.os_h = o_strides[2];
  }
  a.cu_docs = cu_docs; a.n_docs = cu_docs ? n_docs : 1;
  a.B = B; a.S = S; a.Hq = Hq; a.Hkv = Hkv;
  a.Sq = Sq; a.q_off = ring ? q_off : S - Sq;
  a.k_off = ring ? k_off : 0;
  a.acc_mode = ring ? acc_mode : 0;
  a.ring_out = ring && ring_out;
  a.o_acc = o_acc;
  a.lse_acc = lse_acc;
  a.n_qtiles = (int)n_qtiles;
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  if (rope_base > 0.0) {
    a.rope_q = 1;
    a.rope_half = rope_pairing;
    a.positions = positions;
    theta_revolutions(rope_base, D, a.theta_rev);
  }
  a.split_tiles = split_tiles;
  a.max_splits = split_tiles ? max_splits : 1;
  a.o_part = o_part;
  a.lse_part = lse_part;
  // bf16 without split key ranges or a ring step, with at most 63 documents
  // per sequence, and many items per compute unit: a persistent grid that
  // balances the items over the XCDs as they finish (the XCDs of one part
  // run at different clocks) and loads each item's first tiles while the
  // previous one ends
  if (dt == LA_BF16 && split_tiles == 0 && !ring && (!cu_docs || n_docs < 64)) {
    const int pg = persistent_grid((long long)B * Hkv * n_qtiles);
    if (pg > 0) {
      unsigned* sched = nullptr;
      if (la::prefill_sched(stream, &sched) != hipSuccess) return LA_ERR_LAUNCH;
      a.sched = sched;
      a.pgrid = pg;
    }
  }
  const int dti = dt == LA_BF16 ? 0 : 1;
  const la_status st = launched(la::launch_prefill(a, D, G, dti, stream));
  if (st != LA_OK || split_tiles == 0) return st;
  return launched(la::launch_prefill_merge(a, D, dti, stream));
}

}  // namespace

extern "C" {

la_status gqa_prefill(const void* q, const void* k, const void* v, void* o, float* lse,
                      la_dtype dt, int B, int S, int Hq, int Hkv, int D,
                      const int64_t q_strides[3], const int64_t k_strides[3],
                      const int64_t v_strides[3], const int64_t o_strides[3],
                      const int32_t* cu_docs, int n_docs, float softmax_scale,
                      hipStream_t stream) {
  return prefill_impl(q, k, v, o, lse, dt, B, S, S, Hq, Hkv, D, q_strides, k_strides, v_strides,
                      o_strides, cu_docs, n_docs, softmax_scale, nullptr, 0.0, 0, stream);
}

la_status gqa_prefill_rope(const void* q, const void* k, const void* v, void* o, float* lse,
                           la_dtype dt, int B, int S, int Hq, int Hkv, int D,
                           const int64_t q_strides[3], const int64_t k_strides[3],
                           const int64_t v_strides[3], const int64_t o_strides[3],
                           const int32_t* cu_docs, int n_docs, float softmax_scale,
                           const int32_t* positions, double rope_base, int rope_pairing,
                           hipStream_t stream) {
  if (!(rope_base > 0.0) || !std::isfinite(rope_base)) return LA_ERR_INVALID_ARG;
  return prefill_impl(q, k, v, o, lse, dt, B, S, S, Hq, Hkv, D, q_strides, k_strides, v_strides,
                      o_strides, cu_docs, n_docs, softmax_scale, positions, rope_base, rope_pairing,
                      stream);
}

la_status gqa_prefill_chunk(const void* q, const void* k, const void* v, void* o, float* lse,
                            la_dtype dt, int B, int Sq, int S, int Hq, int Hkv, int D,
                            const int64_t q_strides[3], const int64_t k_strides[3],
                            const int64_t v_strides[3], const int64_t o_strides[3],
                            const int32_t* cu_docs, int n_docs, float softmax_scale,
                            const int32_t* positions, double rope_base, int rope_pairing,
                            hipStream_t stream) {
  if (!(rope_base >= 0.0) || !std::isfinite(rope_base)) return LA_ERR_INVALID_ARG;
  return prefill_impl(q, k, v, o, lse, dt, B, Sq, S, Hq, Hkv, D, q_strides, k_strides, v_strides,
                      o_strides, cu_docs, n_docs, softmax_scale, positions, rope_base, rope_pairing,
                      stream);
}

la_status gqa_prefill_split(const void* q, const void* k, const void* v, void* o, float* lse,
                            la_dtype dt, int B, int Sq, int S, int Hq, int Hkv, int D,
                            const int64_t q_strides[3], const int64_t k_strides[3],
                            const int64_t v_strides[3], const int64_t o_strides[3],
                            const int32_t* cu_docs, int n_docs, float softmax_scale,
                            const int32_t* positions, double rope_base, int rope_pairing,
                            int split_tiles, int max_splits, float* o_part, float* lse_part,
                            hipStream_t stream) {
  if (!(rope_base >= 0.0) || !std::isfinite(rope_base)) return LA_ERR_INVALID_ARG;
  if (split_tiles < 1) return LA_ERR_INVALID_ARG;
  return prefill_impl(q, k, v, o, lse, dt, B, Sq, S, Hq, Hkv, D, q_strides, k_strides, v_strides,
                      o_strides, cu_docs, n_docs, softmax_scale, positions, rope_base, rope_pairing,
                      stream, split_tiles, max_splits, o_part, lse_part);
}

la_status gqa_prefill_ring_step(const void* q, const void* k, const void* v, float* o_acc,
                                float* lse_acc, la_dtype dt, int B, int Sq, int q_off, int Skv,
                                int k_off, int Hq, int Hkv, int D, const int64_t q_strides[3],
                                const int64_t k_strides[3], const int64_t v_strides[3],
                                const int32_t* cu_docs, int n_docs, float softmax_scale,
                                const int32_t* positions, double rope_base, int rope_pairing,
                                int first, hipStream_t stream) {
  if (!(rope_base >= 0.0) || !std::isfinite(rope_base)) return LA_ERR_INVALID_ARG;
  return prefill_impl(q, k, v, nullptr, nullptr, dt, B, Sq, Skv, Hq, Hkv, D, q_strides, k_strides,
                      v_strides, nullptr, cu_docs, n_docs, softmax_scale, positions, rope_base,
                      rope_pairing, stream, 0, 0, nullptr, nullptr, true, q_off, k_off,
                      first ? 1 : 2, o_acc, lse_acc);
}

la_status gqa_prefill_ring_step_final(const void* q, const void* k, const void* v, float* o_acc,
                                      float* lse_acc, void* o, const int64_t o_strides[3], float* lse,
                                      la_dtype dt, int B, int Sq, int q_off, int Skv, int k_off, int Hq,
                                      int Hkv, int D, const int64_t q_strides[3],
                                      const int64_t k_strides[3], const int64_t v_strides[3],
                                      const int32_t* cu_docs, int n_docs, float softmax_scale,
                                      const int32_t* positions, double rope_base, int rope_pairing,
                                      int first, hipStream_t stream) {
  if (!(rope_base >= 0.0) || !std::isfinite(rope_base)) return LA_ERR_INVALID_ARG;
  return prefill_impl(q, k, v, o, lse, dt, B, Sq, Skv, Hq, Hkv, D, q_strides, k_strides,
                      v_strides, o_strides, cu_docs, n_docs, softmax_scale, positions, rope_base,
                      rope_pairing, stream, 0, 0, nullptr, nullptr, true, q_off, k_off,
                      first ? 0 : 3, o_acc, lse_acc, true);
}

la_status gqa_prefill_ring_finalize(const float* o_acc, const float* lse_acc, void* o,
                                    const int64_t o_strides[3], float* lse, la_dtype dt, int B,
                                    int Sq, int Hq, int D, hipStream_t stream) {
  if (!known_dtype(dt)) return LA_ERR_UNSUPPORTED;
  if (!o_acc || !lse_acc || !o) return LA_ERR_INVALID_ARG;
  if (B < 1 || Sq < 1 || Hq < 1) return LA_ERR_INVALID_ARG;
  if (!supported_d(D)) return LA_ERR_UNSUPPORTED;
  if (!aligned16(o_acc) || !aligned16(o) || !strides_ok(o_strides, 3, elem_size(dt)))
    return LA_ERR_INVALID_ARG;
  la::PrefillArgs a{};
  a.o = o; a.lse = lse;
  a.os_b = o_strides[0]; a.os_s = o_strides[1]; a.os_h = o_strides[2];
  a.B = B; a.Sq = Sq; a.Hq = Hq;
  // the accumulators are a merge's single slot
  a.max_splits = 1;
  a.o_part = const_cast<float*>(o_acc);
  a.lse_part = const_cast<float*>(lse_acc);
  return launched(la::launch_ring_finalize(a, D, dt == LA_BF16 ? 0 : 1, stream));
}

}  // extern "C"

namespace {

la_status decode_check(const void* q, const int64_t q_strides[2], const void* k_cache,
                       const void* v_cache, const int64_t cache_strides[3],
                       const int32_t* seq_lens, int B, int Hq, int Hkv, int D, int Lmax,
                       int kv_chunk, int max_splits, float softmax_scale, float* o_part,
                       float* lse_part) {
  if (!q || !k_cache || !v_cache || !seq_lens || !o_part || !lse_part) return LA_ERR_INVALID_ARG;
  if (B < 1 || Hq < 1 || Hkv < 1 || Lmax < 1 || max_splits < 1) return LA_ERR_INVALID_ARG;
  if (kv_chunk < 64 || kv_chunk % 64 != 0) return LA_ERR_INVALID_ARG;
  if ((long long)max_splits * kv_chunk < Lmax) return LA_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return LA_ERR_INVALID_ARG;
  if (!supported_d(D) || !supported_g(Hq / Hkv)) return LA_ERR_UNSUPPORTED;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o_part))
    return LA_ERR_INVALID_ARG;
  if (!strides_ok(q_strides, 2, 2) || !strides_ok(cache_strides, 3, 2)) return LA_ERR_INVALID_ARG;
  if (!std::isfinite(softmax_scale)) return LA_ERR_INVALID_ARG;
  if ((long long)B * Hkv * max_splits > 0x7fffffffLL) return LA_ERR_INVALID_ARG;
  if ((long long)B * Hkv * ((Lmax + 15) / 16) > 0x7fffffffLL) return LA_ERR_INVALID_ARG;
  if ((long long)B * Hq * max_splits * D > 0x7fffffffffffLL) return LA_ERR_INVALID_ARG;
  if (B > la::kDecodeMaxBatch) return LA_ERR_UNSUPPORTED;
  // cache rows may not overlap, and a 16-key tile must span less than 2 GiB
  // (32-bit buffer range)
  if (cache_strides[2] < D) return LA_ERR_INVALID_ARG;
  if (cache_strides[2] > (1LL << 24)) return LA_ERR_UNSUPPORTED;
  return LA_OK;
}

la::DecodeArgs decode_args(const void* q, const int64_t q_strides[2], const void* k_cache,
                           const void* v_cache, const int64_t cache_strides[3],
                           const int32_t* seq_lens, int B, int Hq, int Hkv, int D, int Lmax,
                           int kv_chunk, int max_splits, float softmax_scale, float* o_part,
                           float* lse_part) {
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)D);
  la::DecodeArgs a{};
  a.q = q; a.qs_b = q_strides[0]; a.qs_h = q_strides[1];
  a.k = k_cache; a.v = v_cache;
  a.cs_b = cache_strides[0]; a.cs_h = cache_strides[1]; a.cs_l = cache_strides[2];
  a.seq_lens = seq_lens;
  a.B = B; a.Hq = Hq; a.Hkv = Hkv; a.Lmax = Lmax; a.kv_chunk = kv_chunk; a.max_splits = max_splits;
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.o_part = o_part; a.lse_part = lse_part;
  a.grid = current_cu_count();
  return a;
}

}  // namespace

extern "C" {

la_status gqa_decode(const void* q, const int64_t q_strides[2], const void* k_cache,
                     const void* v_cache, const int64_t cache_strides[3],
                     const int32_t* seq_lens, int B, int Hq, int Hkv, int D, int Lmax,
                     int kv_chunk, int max_splits, float softmax_scale, float* o_part,
                     float* lse_part, hipStream_t stream) {
  const la_status st = decode_check(q, q_strides, k_cache, v_cache, cache_strides, seq_lens, B, Hq,
                                    Hkv, D, Lmax, kv_chunk, max_splits, softmax_scale, o_part,
                                    lse_part);
  if (st != LA_OK) return st;
  if (debug_mode() && !lens_ok(seq_lens, B, 1, Lmax, stream)) return LA_ERR_INVALID_ARG;
  const la::DecodeArgs a = decode_args(q, q_strides, k_cache, v_cache, cache_strides, seq_lens, B,
                                       Hq, Hkv, D, Lmax, kv_chunk, max_splits, softmax_scale,
                                       o_part, lse_part);
  return launched(la::launch_decode(a, D, Hq / Hkv, stream));
}

la_status gqa_decode_paged(const void* q, const int64_t q_strides[2], const void* k_pages,
                           const void* v_pages, const int64_t page_strides[3], int page_size,
                           const int32_t* block_table, int bt_stride, const int32_t* seq_lens,
                           int B, int Hq, int Hkv, int D, int Lmax, int kv_chunk, int max_splits,
                           float softmax_scale, float* o_part, float* lse_part,
                           hipStream_t stream) {
  if (!block_table || !k_pages || !v_pages) return LA_ERR_INVALID_ARG;
  if (page_size < 16 || page_size > (1 << 20) || (page_size & (page_size - 1)) != 0)
    return LA_ERR_INVALID_ARG;
  if (Lmax < 1 || bt_stride < (Lmax + page_size - 1) / page_size) return LA_ERR_INVALID_ARG;
  if (!strides_ok(page_strides, 3, 2)) return LA_ERR_INVALID_ARG;
  // the checks and arguments of the contiguous call, with the page stride in
  // place of the sequence stride
  const int64_t cache_strides[3] = {page_strides[0], page_strides[1], page_strides[2]};
  la_status st = decode_check(q, q_strides, k_pages, v_pages, cache_strides, seq_lens, B, Hq, Hkv,
                              D, Lmax, kv_chunk, max_splits, softmax_scale, o_part, lse_part);
  if (st != LA_OK) return st;
  if (debug_mode() && (!lens_ok(seq_lens, B, 1, Lmax, stream) ||
                       !block_table_ok(block_table, bt_stride, seq_lens, B, page_size, stream)))
    return LA_ERR_INVALID_ARG;
  la::DecodeArgs a = decode_args(q, q_strides, k_pages, v_pages, cache_strides, seq_lens, B, Hq,
                                 Hkv, D, Lmax, kv_chunk, max_splits, softmax_scale, o_part,
                                 lse_part);
  a.block_table = block_table;
  a.bt_stride = bt_stride;
  int shift = 0;
  while ((1 << shift) < page_size) ++shift;
  a.page_shift = shift;
  return launched(la::launch_decode(a, D, Hq / Hkv, stream));
}

la_status gqa_decode_combine(const float* o_part, const float* lse_part, const int32_t* seq_lens,
                             int B, int Hq, int D, int kv_chunk, int max_splits, void* o,
                             const int64_t o_strides[2], float* lse, la_dtype dt,
                             hipStream_t stream) {
  if (!known_dtype(dt)) return LA_ERR_UNSUPPORTED;
  if (!o_part || !lse_part || !seq_lens || !o) return LA_ERR_INVALID_ARG;
  if (B < 1 || Hq < 1 || max_splits < 1) return LA_ERR_INVALID_ARG;
  if (kv_chunk < 64 || kv_chunk % 64 != 0) return LA_ERR_INVALID_ARG;
  if (!supported_d(D)) return LA_ERR_UNSUPPORTED;
  if (!o_strides || o_strides[0] < 0 || o_strides[1] < 0) return LA_ERR_INVALID_ARG;
  if ((long long)B * Hq > 0x7fffffffLL - 3) return LA_ERR_INVALID_ARG;
  // the workspace gqa_decode writes (16-byte aligned rows)
  if (!aligned16(o_part) || (reinterpret_cast<uintptr_t>(lse_part) & 3u) != 0) return LA_ERR_INVALID_ARG;
  if (debug_mode() && !lens_ok(seq_lens, B, 1, (int64_t)max_splits * kv_chunk, stream))
    return LA_ERR_INVALID_ARG;

  la::CombineArgs a{};
  a.o_part = o_part; a.lse_part = lse_part; a.seq_lens = seq_lens;
  a.B = B; a.Hq = Hq; a.kv_chunk = kv_chunk; a.max_splits = max_splits;
  a.o = o; a.os_b = o_strides[0]; a.os_h = o_strides[1];
  a.lse = lse;
  return launched(la::launch_combine(a, D, dt == LA_BF16 ? 0 : 1, stream));
}

la_status gqa_decode_noalloc(const void* q, const int64_t q_strides[2], const void* k_cache,
                             const void* v_cache, const int64_t cache_strides[3],
                             const int32_t* seq_lens, int B, int Hq, int Hkv, int D, int Lmax,
                             int kv_chunk, float softmax_scale, void* o, const int64_t o_strides[2],
                             float* lse, la_dtype dt, hipStream_t stream) {
  // every check that does not need the scratch comes first (placeholder,
  // aligned workspace pointers for the decode's own checks)
  if (!known_dtype(dt)) return LA_ERR_UNSUPPORTED;
  if (!o || !o_strides || o_strides[0] < 0 || o_strides[1] < 0) return LA_ERR_INVALID_ARG;
  if (kv_chunk < 64 || kv_chunk % 64 != 0 || Lmax < 1) return LA_ERR_INVALID_ARG;
  const int max_splits = (int)(((long long)Lmax + kv_chunk - 1) / kv_chunk);
  float* placeholder = reinterpret_cast<float*>(uintptr_t(256));
  la_status st = decode_check(q, q_strides, k_cache, v_cache, cache_strides, seq_lens, B, Hq, Hkv, D,
                              Lmax, kv_chunk, max_splits, softmax_scale, placeholder, placeholder);
  if (st != LA_OK) return st;
  if (debug_mode() && !lens_ok(seq_lens, B, 1, Lmax, stream)) return LA_ERR_INVALID_ARG;

  void* base = nullptr;
  size_t cap = 0;
  if (la::decode_scratch(&base, &cap) != hipSuccess) return LA_ERR_LAUNCH;
  // scratch: wave headers, then the run slots' o and lse (one run per wave
  // and (sequence, KV head) pair it touches: at most waves + B * Hkv slots)
  const int grid = current_cu_count();
  const long long W = (long long)grid * la::kDecodeWaves;
  const long long G = Hq / Hkv;
  const long long slots = W + (long long)B * Hkv;
  auto up256 = [](long long x) { return (x + 255) / 256 * 256; };
  const long long hdr_bytes = up256(8 * W);
  const long long o_bytes = up256(slots * G * D * 4);
  const long long need = hdr_bytes + o_bytes + slots * G * 4;
  if (need > (long long)cap) return LA_ERR_SCRATCH;
  char* sp = static_cast<char*>(base);
  int* hdr = reinterpret_cast<int*>(sp);
  float* o_c = reinterpret_cast<float*>(sp + hdr_bytes);
  float* l_c = reinterpret_cast<float*>(sp + hdr_bytes + o_bytes);

  la::DecodeArgs a = decode_args(q, q_strides, k_cache, v_cache, cache_strides, seq_lens, B, Hq, Hkv,
                                 D, Lmax, kv_chunk, max_splits, softmax_scale, o_c, l_c);
  a.grid = grid;
  a.hdr = hdr;
  st = launched(la::launch_decode(a, D, Hq / Hkv, stream));
  if (st != LA_OK) return st;
  la::CombineArgs c{};
  c.o_part = o_c; c.lse_part = l_c; c.seq_lens = seq_lens;
  c.B = B; c.Hq = Hq; c.kv_chunk = kv_chunk; c.max_splits = max_splits;
  c.o = o; c.os_b = o_strides[0]; c.os_h = o_strides[1];
  c.lse = lse;
  c.hdr = hdr; c.Hkv = Hkv; c.W = (int)W;
  return launched(la::launch_combine(c, D, dt == LA_BF16 ? 0 : 1, stream));
}

}  // extern "C"

namespace {

// the rows of q and dout are fetched as blocks of whole token rows: each
// token's heads lie within its token stride, and block offsets fit in 32 bits
bool bwd_rows_ok(const int64_t* st, int H, int D) {
  return st[2] >= D && st[1] >= (int64_t)H * st[2] && 64 * st[1] + 16 * st[2] < (1LL << 29);
}

}  // namespace

extern "C" {

la_status gqa_attention_backward(const void* q, const void* k, const void* v, const void* o,
                                 const void* dout, const float* lse, float* delta, void* dq,
                                 void* dk, void* dv, la_dtype dt, int B, int S, int Hq, int Hkv,
                                 int D, const int64_t q_strides[3], const int64_t k_strides[3],
                                 const int64_t v_strides[3], const int64_t o_strides[3],
                                 const int64_t dout_strides[3], const int64_t dq_strides[3],
                                 const int64_t dk_strides[3], const int64_t dv_strides[3],
                                 const int32_t* cu_docs, int n_docs, float softmax_scale,
                                 float* dkv_workspace, hipStream_t stream) {
  if (dt != LA_BF16) return LA_ERR_UNSUPPORTED;
  if (dkv_workspace && !aligned16(dkv_workspace)) return LA_ERR_INVALID_ARG;
  if (!q || !k || !v || !o || !dout || !lse || !delta || !dq || !dk || !dv) return LA_ERR_INVALID_ARG;
  if (B < 1 || S < 1 || Hq < 1 || Hkv < 1) return LA_ERR_INVALID_ARG;
  if (cu_docs && n_docs < 1) return LA_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return LA_ERR_INVALID_ARG;
  if (!supported_d(D) || !supported_g(Hq / Hkv)) return LA_ERR_UNSUPPORTED;
  if (!std::isfinite(softmax_scale)) return LA_ERR_INVALID_ARG;
  for (const void* p : {q, k, v, o, dout, (const void*)dq, (const void*)dk, (const void*)dv})
    if (!aligned16(p)) return LA_ERR_INVALID_ARG;
  for (const int64_t* st : {q_strides, k_strides, v_strides, o_strides, dout_strides, dq_strides,
                            dk_strides, dv_strides})
    if (!strides_ok(st, 3, 2)) return LA_ERR_INVALID_ARG;
  if (!bwd_rows_ok(q_strides, Hq, D) || !bwd_rows_ok(dout_strides, Hq, D)) return LA_ERR_INVALID_ARG;
  if (k_strides[1] < D || v_strides[1] < D) return LA_ERR_INVALID_ARG;
  if (64 * k_strides[1] >= (1LL << 30) || 64 * v_strides[1] >= (1LL << 30)) return LA_ERR_INVALID_ARG;
  const int G = Hq / Hkv;
  if ((long long)G * S >= (1LL << 28)) return LA_ERR_INVALID_ARG;
  const long long nkb = (S + la::kBwdKeysPerBlock - 1) / la::kBwdKeysPerBlock;
  const long long tq = la::bwd_dq_tokens_per_block(G);
  if ((long long)B * Hkv * std::max(nkb, (S + tq - 1) / tq) > 0x7fffffffLL) return LA_ERR_INVALID_ARG;
  if ((long long)B * S * Hq > (1LL << 40)) return LA_ERR_INVALID_ARG;
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / std::sqrt((float)D);
  if (debug_mode() && !docs_ok(cu_docs, B, n_docs, S, true, stream)) return LA_ERR_INVALID_ARG;

  la::BwdArgs a{};
  a.q = q; a.k = k; a.v = v; a.o = o; a.dout = dout; a.lse = lse; a.delta = delta;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.qs_b = q_strides[0]; a.qs_s = q_strides[1]; a.qs_h = q_strides[2];
  a.ks_b = k_strides[0]; a.ks_s = k_strides[1]; a.ks_h = k_strides[2];
  a.vs_b = v_strides[0]; a.vs_s = v_strides[1]; a.vs_h = v_strides[2];
  a.os_b = o_strides[0]; a.os_s = o_strides[1]; a.os_h = o_strides[2];
  a.gs_b = dout_strides[0]; a.gs_s = dout_strides[1]; a.gs_h = dout_strides[2];
  a.dqs_b = dq_strides[0]; a.dqs_s = dq_strides[1]; a.dqs_h = dq_strides[2];
  a.dks_b = dk_strides[0]; a.dks_s = dk_strides[1]; a.dks_h = dk_strides[2];
  a.dvs_b = dv_strides[0]; a.dvs_s = dv_strides[1]; a.dvs_h = dv_strides[2];
  a.cu_docs = cu_docs; a.n_docs = cu_docs ? n_docs : 1;
  a.B = B; a.S = S; a.Hq = Hq; a.Hkv = Hkv;
  a.scale = scale;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.dkv_part = dkv_workspace;
  return launched(la::launch_backward(a, D, G, stream));
}

}  // extern "C"
