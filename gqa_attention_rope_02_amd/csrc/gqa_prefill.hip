// Grouped-query causal attention with the cross-document mask, prefill.
//
// What is computed: for query head h of token i, o_i = sum_j p_ij v_j over the
// keys j of KV head h / g that are visible (j <= i, same document), with
// p_ij = softmax_j(q_i . k_j * scale) ("The Llama 3 Herd of Models", "A
// Deliberately Standard Dense Transformer": GQA with 8 KV heads and a
// cross-document mask; "How Meta's Llama 3.1 405B Architecture Actually
// Works", GQA paragraph: query heads grouped onto a shared KV head). Queries
// and keys arrive already rotated.
//
// How (gfx950):
// * One workgroup = one (sequence, KV head, tile of 256/g tokens): its 256
//   "columns" are the (token, query head) pairs of the g heads sharing the KV
//   head, so each K/V byte staged in LDS feeds 256 query rows. Eight waves own
//   32 columns each, two waves per SIMD.
// * The contractions run transposed on the 32x32x16 bf16 MFMA: S^T = K Q^T
//   (keys on M, columns on N) and O^T = V^T P^T (head_dim on M). In both
//   results a lane owns one column, so the softmax statistics and the output
//   rescale stay in the lane; only the row max needs one cross-lane step
//   (v_permlane32_swap between lanes l and l^32), and the S^T accumulator
//   already has the layout of the P^T operand.
// * Q stays in registers for the whole key loop. K and V tiles of 64 keys go
//   from HBM straight into LDS (buffer_load_dwordx4 ... lds, no register
//   staging), row-major with XOR swizzles, through two rings of four stages
//   (K in the first 64 KB of LDS, V in the second). The buffer descriptor
//   moves with the tile and its size ends at the sequence end, so rows past
//   the end read as zero. K operands are read with ds_read_b128; the V^T
//   operand with the transposing ds_read_b64_tr_b16 from the row-major V tile.
// * The query operand carries scale * log2(e) (multiplied in fp32 before its
//   one rounding to bf16, after the rotation when the kernel rotates), and
//   the score MFMA starts its accumulation from -Mref instead of 0, so it
//   yields the exponent t = s * scale * log2(e) - Mref directly: no VALU
//   operation per score before the exponential (the VALU time of a tile adds
//   to its MFMA time on this part, so each operation removed counts).
// * Software pipeline, one workgroup barrier per tile: between two barriers
//   every wave runs the PV product of the previous tile, then the QK product
//   of the next tile with the exponentials, bf16 rounding and row sums of the
//   current one interleaved. Each piece (one MFMA, its operand read a few
//   MFMAs ahead, two transcendental and two VALU operations) is emitted in
//   program order and fenced, so a wave keeps its matrix core and its VALU
//   busy at the same time; the two waves of a SIMD fill each other's waits.
//   The exponents of consecutive tiles alternate between two register
//   buffers. The loop is unrolled over the four stage indices, so every LDS
//   operand address is a per-lane register plus a constant offset.
// * Online softmax in the base-2 domain with fp32 statistics; probabilities
//   are rounded to bf16 once and the row sums accumulate those rounded values
//   (v_dot2_f32_bf16), so numerator and denominator use the same weights. The
//   reference the exponents are taken against is moved lazily (exact: softmax
//   does not depend on the reference): a tile's weights are first taken
//   against the current reference, and only if some lane's sum of them
//   exceeds 2^8 (so possibly one weight does) is the tile max formed, the
//   reference moved up to it, the accumulator rescaled and the weights redone.
//   Weights therefore stay at most 256, and most tiles need neither a max nor
//   a rescale. Masks are evaluated only on tiles that cross a causal or
//   document edge of the wave's columns.
// * Start of a workgroup: with at most 63 documents the row of document
//   offsets is read with one load per lane and searched with wave ballots, the
//   Q loads are issued right after it, and the first K/V tiles as soon as the
//   key range is known, so these latencies overlap.
// * The output goes through LDS (free once the last tile is read): each lane
//   leaves its 4-value pieces of its column's row there and reads back 16
//   contiguous bytes, so a wave stores whole rows with 16-byte writes
//   instead of 8-byte pieces 256 bytes apart.
// * Workgroups are issued longest-first (last token tiles first), and the KV
//   head is the fastest-varying index so the workgroups of one KV head land on
//   one XCD (blockIdx % 8) and share its L2.
// * Long prefills run on a persistent grid instead (one workgroup per compute
//   unit, the same items drawn from one queue per XCD, other XCDs' queues
//   once its own is empty): the eight XCDs of one part run at different
//   clocks under the power limit, a few percent apart, and a fixed split of
//   the items leaves the faster ones idle at the end. While an item runs its
//   last key tiles, the next item's first tiles load into the rings, its
//   queries into registers.
#include <algorithm>
#include <mutex>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace la {
namespace {

constexpr int kCols = 256;    // columns per workgroup
constexpr int kNW = 8;        // waves per workgroup
constexpr int kCB = kCols / kNW / 32;   // 32-column blocks per wave
static_assert(kCB == 1, "one 32-column block per wave");
constexpr int kKT = 64;       // keys per tile
constexpr float kLazyW = 256.f;   // bound on a weight under the lazily moved softmax reference
// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8; a field at its maximum does not wait)
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int kLgkm0 = 15 | (3 << 14) | (7 << 4);

__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// QS: the query operand carries scale * log2(e) (queries rotated in the
// kernel, or fp32 queries: either way rounded once to bf16 from fp32). For
// queries that arrive rotated in bf16 (QS false) the operand is the query
// itself, since scaling it would round it a second time, and the exponents
// are formed from the scores by one FMA each.
//
// PERS: a persistent grid (one workgroup per compute unit) that takes its
// items, one (sequence, KV head, query tile) each, from the work queues in
// a.sched; while an item runs its last key tiles, the first tiles of the next
// item already load into the rings (bf16 only).
template <typename T, int D, int G, bool QS, bool PERS>
__global__ __launch_bounds__(64 * kNW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_kernel(PrefillArgs a) {
  constexpr int TQ = kCols / G;          // tokens per workgroup
  constexpr int KS = D / 16;             // k-steps of S^T = K Q^T
  constexpr int DB = D / 32;             // 32-row blocks of O^T
  constexpr int CH = D / 8;              // 16-byte chunks per row
  constexpr int ROW = D * 2;             // bytes per LDS row
  constexpr int TILE = kKT * ROW;        // bytes per K or V tile
  constexpr int NL = kKT * CH / 64 / kNW;  // 1 KB loads per wave per K or V tile

  // four stages: K of stage s at s TILE, V of stage s at (4 + s) TILE, so
  // every operand address is one per-lane register plus an offset below 64 KB
  // (persistent: a ninth tile at 8 TILE for the output, and the next item's
  // index after it)
  static_assert(!PERS || std::is_same<T, __bf16>::value, "persistent grid: bf16 only");
  __shared__ __attribute__((aligned(1024))) char lds[PERS ? 9 * TILE + 512 : 8 * TILE];
  int* const sh_next = reinterpret_cast<int*>(lds + 9 * TILE);
  // (persistent) per wave, the next item's K and V bases, first key and tile
  // count: kept in LDS rather than in scalar registers through the key loop,
  // and read back by the iterations that load the next item's tiles
  struct NextItem {
    const T* kb;
    const T* vb;
    int kvlo, nt;
  };
  auto uniform_ptr = [](const T* p) __attribute__((always_inline)) {
    const uint64_t x = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(x >> 32));
    return reinterpret_cast<const T*>(((uint64_t)hi << 32) | lo);
  };

  // Work items: item = (qtiles from the last, sequence, KV head), KV head
  // fastest, so that longer items come first. Without PERS workgroup i runs
  // item i. With PERS workgroup i runs item i first; the items congruent to x
  // mod 8 form queue x, and a workgroup draws further items from queue
  // blockIdx % 8 (the workgroups of one XCD, sharing one L2), then from the
  // other queues once its own is empty. Counter x of a.sched counts the draws
  // on queue x past the items the grid started with; counter 8 counts the
  // workgroups that found every queue empty, and the last of them sets all
  // nine back to zero for the next launch on the stream.
  const int n_items = a.B * a.Hkv * a.n_qtiles;
  int item = blockIdx.x;
  int ph_c = 0;              // ring stage of the item's tile 0 (PERS)
  int kpf_c = 3, vpf_c = 2;  // the item's own start loads K tiles j < kpf_c and V tiles j < vpf_c
  // the item's offsets row (one entry per lane) and raw queries, loaded
  // before the item starts (PERS)
  int cu_n = 0;
  bf16x8 qn[D / 16];
  // offsets row of sequence bb, one entry per lane
  auto load_cu = [&](int bb) __attribute__((always_inline)) {
    return a.cu_docs[(int64_t)bb * (a.n_docs + 1) + min((int)threadIdx.x & 63, a.n_docs)];
  };
  // raw queries of this lane's column of item (bb, hh, qt)
  auto load_q = [&](int bb, int hh, int qt) __attribute__((always_inline)) {
    const int lc = threadIdx.x & 31, hi = (threadIdx.x >> 5) & 1;
    const int col = (int)(threadIdx.x >> 6) * 32 + lc;
    const int t = min(qt * TQ + col / G, a.Sq - 1);
    const T* qp = static_cast<const T*>(a.q) + bb * a.qs_b + t * a.qs_s + (hh * G + col % G) * a.qs_h + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qn[ks] = load8(qp + 16 * ks);
  };
  if constexpr (PERS) {
    const int h0 = item % a.Hkv, r0 = item / a.Hkv;
    if (a.cu_docs && a.n_docs < 64) cu_n = load_cu(r0 % a.B);
    load_q(r0 % a.B, h0, a.n_qtiles - 1 - r0 / a.B);
  }

  for (;;) {
  // (persistent) the thread index passes through an empty asm at the top of
  // every item, so that what is derived from it is formed inside the item
  // instead of hoisted out of the loop and held, or spilled, across it
  int zz = 0;
  if constexpr (PERS) asm volatile("" : "+v"(zz));
  const int tid = (int)threadIdx.x + zz;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lc = lane & 31, hi = lane >> 5;
  const int bid = item;
  const int kvh = bid % a.Hkv;
  const int r = bid / a.Hkv;
  const int b = r % a.B;
  const int qtile = a.n_qtiles - 1 - r / a.B;
  // Query rows 0 .. Sq-1 sit at key positions qo .. qo+Sq-1 of the S keys
  // (qo = S - Sq: a block of new tokens after a cached prefix; 0 otherwise).
  // Token indices below are query rows; positions (masks, documents, the key
  // range) add qo.
  const int S = a.S, Sq = a.Sq, qo = a.q_off;
  // keys: positions k_off .. kend-1 in rows 0 .. S-1 of k and v (k_off = 0
  // except for a key shard of a context-parallel ring step)
  const int k_off = a.k_off, kend = a.k_off + a.S;
  const int t0 = qtile * TQ;
  const int t_end = min(t0 + TQ, Sq);
  const int32_t* cu = a.cu_docs ? a.cu_docs + (int64_t)b * (a.n_docs + 1) : nullptr;
  const int n_docs = a.n_docs;

  const T* qbase = static_cast<const T*>(a.q) + b * a.qs_b;
  const T* kbase = static_cast<const T*>(a.k) + b * a.ks_b + kvh * a.ks_h;
  const T* vbase = static_cast<const T*>(a.v) + b * a.vs_b + kvh * a.vs_h;

  // ---- this lane's columns (one per 32-column block) -------------------------
  int tok[kCB], head[kCB], st[kCB];
  bool valid[kCB];
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) {
    const int col = wave * 32 * kCB + cb * 32 + lc;
    tok[cb] = t0 + col / G;
    head[cb] = kvh * G + col % G;
    valid[cb] = tok[cb] < Sq;
  }
  const int w_tmin = min(t0 + (wave * 32 * kCB) / G, Sq - 1);
  const int w_tmax_raw = t0 + (wave * 32 * kCB + 32 * kCB - 1) / G;
  const bool wave_all_valid = w_tmax_raw < Sq;
  const int w_tmax = min(w_tmax_raw, Sq - 1);

  // ---- document starts ---------------------------------------------------------
  // With at most 63 documents the offsets row is read once, one entry per
  // lane, and every search is a ballot over the lanes. Longer rows are
  // binary-searched in memory, before any other load is issued, so that the
  // waits of one path do not land on the loads of the other.
  const bool docs_in_lanes = cu && n_docs < 64;
  int kv_start = 0, w_smax = 0;
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) st[cb] = 0;
  if (cu && !docs_in_lanes) {
    kv_start = doc_start(cu, n_docs, t0 + qo);
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) st[cb] = valid[cb] ? doc_start(cu, n_docs, tok[cb] + qo) : 0;
    w_smax = doc_start(cu, n_docs, w_tmax + qo);
  }
  int cu_l = 0;
  if constexpr (PERS) cu_l = cu_n;
  else if (docs_in_lanes) cu_l = cu[min(lane, n_docs)];

  // ---- Q operand (B of S^T = K Q^T): Q[col][16ks + 8hi + i] ----------------
  // Columns past the sequence end load the last token's row (no branch, so
  // the wait for the offsets row does not also wait for Q); every key is
  // masked for them and their outputs are not stored.
  // With QS the operand holds q * scale * log2(e), rounded once to bf16
  // (after the rotation when the kernel rotates), so the score MFMA yields
  // the exponent in log2 units directly.
  bf16x8 qreg[kCB][KS];
  float qraw[kCB][KS][8];   // the loaded queries in fp32 (QS)
  const bool rope_q = a.rope_q != 0;
  const float qscale = QS ? a.scale_log2 : 1.f;
  auto load_queries = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
      const T* qp = qbase + min(tok[cb], Sq - 1) * a.qs_s + head[cb] * a.qs_h + 8 * hi;
      if constexpr (QS) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) load8_f32(qp + 16 * ks, qraw[cb][ks]);
        if (!rope_q) {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int i = 0; i < 8; ++i) qreg[cb][ks][i] = to_bf16(qraw[cb][ks][i] * qscale);
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qreg[cb][ks] = load8(qp + 16 * ks);
      }
    }
  };
  // The pieces after the first of a split key range load their queries only
  // once they know they have keys: most of them have none (short documents)
  // and exit right after the document search.
  const bool q_after_split = !PERS && a.split_tiles > 0 && blockIdx.y > 0;
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) {
    if constexpr (PERS) {
      // loaded before the item started
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if constexpr (QS) {
#pragma unroll
          for (int i = 0; i < 8; ++i) qraw[cb][ks][i] = (float)qn[ks][i];
          if (!rope_q) {
#pragma unroll
            for (int i = 0; i < 8; ++i) qreg[cb][ks][i] = to_bf16(qraw[cb][ks][i] * qscale);
          }
        } else {
          qreg[cb][ks] = qn[ks];
        }
      }
    }
  }
  if (!PERS && !q_after_split) load_queries();

  if (docs_in_lanes) {
    // index of the document holding position t (the same t in every lane):
    // the last of the first n_docs offsets that is <= t, else 0
    auto doc_of = [&](int t) __attribute__((always_inline)) -> int {
      const unsigned long long mk = __ballot(lane < n_docs && cu_l <= t);
      return mk ? 63 - __clzll(mk) : 0;
    };
    const int d0 = doc_of(t0 + qo);
    kv_start = __builtin_amdgcn_readlane(cu_l, d0);
    // the documents that start inside this workgroup's tokens follow d0
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) st[cb] = kv_start;
    for (int d = d0 + 1; d < n_docs; ++d) {
      const int c = __builtin_amdgcn_readlane(cu_l, d);
      if (c >= t_end + qo) break;
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb) st[cb] = tok[cb] + qo >= c ? c : st[cb];
    }
    w_smax = __builtin_amdgcn_readlane(cu_l, doc_of(w_tmax + qo));
  }
  // clamp: out-of-contract offsets must not move the key range out of
  // [0, t0 + qo]
  int kv_lo = max(k_off, max(0, min(kv_start, t0 + qo)));
  const int kv_hi = min(kend - 1, t_end - 1 + qo);
  if (!PERS && kv_lo > kv_hi) {
    // no key of this shard is visible to any of the tile's rows (ring step):
    // the first step of an accumulation still starts the rows at o = 0,
    // lse = -inf; a last step writes the rows' final o and lse from the
    // accumulators (or, also the first, o = 0 and lse = -inf)
    if (a.ring_out) {
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb) {
        if (!valid[cb]) continue;
        const float* ap = a.o_acc + (((int64_t)b * Sq + tok[cb]) * a.Hq + head[cb]) * D;
        T* op = static_cast<T*>(a.o) + b * a.os_b + tok[cb] * a.os_s + head[cb] * a.os_h;
        const int64_t li = ((int64_t)b * a.Hq + head[cb]) * Sq + tok[cb];
        const float ls = a.acc_mode == 3 ? a.lse_acc[li] : -INFINITY;
        const float keep = ls > -INFINITY ? 1.f : 0.f;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int jq = 0; jq < 4; ++jq) {
            const int d = db * 32 + 8 * jq + 4 * hi;
            const f32x4 x = a.acc_mode == 3 ? *reinterpret_cast<const f32x4*>(ap + d) : f32x4{0.f, 0.f, 0.f, 0.f};
            store4(op + d, x[0] * keep, x[1] * keep, x[2] * keep, x[3] * keep);
          }
        if (hi == 0 && a.lse) a.lse[li] = ls;
      }
    } else if (a.acc_mode == 1) {
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb) {
        if (!valid[cb]) continue;
        float* op = a.o_acc + (((int64_t)b * Sq + tok[cb]) * a.Hq + head[cb]) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int jq = 0; jq < 4; ++jq)
            *reinterpret_cast<f32x4*>(op + db * 32 + 8 * jq + 4 * hi) = f32x4{0.f, 0.f, 0.f, 0.f};
        if (hi == 0) a.lse_acc[((int64_t)b * a.Hq + head[cb]) * Sq + tok[cb]] = -INFINITY;
      }
    }
    __builtin_amdgcn_s_waitcnt(0);   // the Q loads already issued
    return;
  }
  int n_tiles = (kv_hi - kv_lo) / kKT + 1;

  // Split key ranges (split_tiles > 0): workgroup (tile, split sp) takes the
  // key tiles [sp * split_tiles, (sp + 1) * split_tiles) of its query tile's
  // range. A query tile that needs one split writes its final output (and
  // marks its rows with lse_part = +inf in slot 0); one that needs more
  // writes partial results to slot sp for the merge, and the workgroups of
  // its unused slots mark them lse_part = -inf. Nothing has touched LDS yet.
  const int sp = blockIdx.y;
  int n_split = 1;
  if (!PERS && a.split_tiles > 0) {
    n_split = (n_tiles + a.split_tiles - 1) / a.split_tiles;
    if (sp >= n_split) {
      if (n_split > 1 && hi == 0)
#pragma unroll
        for (int cb = 0; cb < kCB; ++cb)
          if (valid[cb])
            a.lse_part[(((int64_t)sp * a.B + b) * a.Hq + head[cb]) * Sq + tok[cb]] = -INFINITY;
      __builtin_amdgcn_s_waitcnt(0);   // the Q loads already issued (first piece)
      return;
    }
    kv_lo += sp * a.split_tiles * kKT;
    n_tiles = min(a.split_tiles, n_tiles - sp * a.split_tiles);
  }
  if (q_after_split) load_queries();

  // ---- online-softmax state of this lane's column ------------------------------
  // Mref: the reference the exponents are taken against, in log2 units
  // (scale * log2(e) * score); -inf until the column has seen a visible key.
  // negM: what the score MFMA starts its accumulation from (-Mref, or 0 while
  // Mref is -inf), splat in negMv.
  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[db][j] = 0.f;
  float Mref = -INFINITY, negM = 0.f, l = 0.f;
  f32x16 negMv;
#pragma unroll
  for (int j = 0; j < 16; ++j) negMv[j] = 0.f;

  // ---- tile staging: per-lane byte offsets of this wave's 1 KB loads --------
  int koff[NL], voff[NL];
#pragma unroll
  for (int n = 0; n < NL; ++n) {
    const int p = (n * kNW + wave) * 64 + lane;   // LDS chunk written by this lane
    const int row = p / CH, ph = p % CH;
    koff[n] = (int)(row * a.ks_s * (int64_t)sizeof(T) + 8 * k_chunk<CH>(ph, row) * (int)sizeof(T));
    voff[n] = (int)(row * a.vs_s * (int64_t)sizeof(T) + 8 * v_chunk<CH>(ph, row) * (int)sizeof(T));
  }
  // The K (V) rows of the tile at key position kt into the stage at dst: rows
  // at or past kend read as zero. bf16: this wave's NL direct-to-LDS loads,
  // tracked by vmcnt; fp32: converted to bf16 through registers and written
  // with ds_write (complete once lgkmcnt drains).
  auto stage_kv_b = [&](const T* base, int kt, char* dst, bool is_v) __attribute__((always_inline)) {
    const int64_t ss = is_v ? a.vs_s : a.ks_s;
    if constexpr (std::is_same<T, __bf16>::value) {
      const int64_t rows = max(kend - kt, 0);
      const int nb = (int)min(rows * ss * 2, (int64_t)0x7fffffff);
      const void* p = base + (int64_t)(kt - k_off) * ss;
#pragma unroll
      for (int n = 0; n < NL; ++n)
        load_lds16(p, nb, is_v ? voff[n] : koff[n], dst + (n * kNW + wave) * 1024);
    } else {
      for (int p = tid; p < kKT * CH; p += 64 * kNW) {
        const int row = p / CH, ph = p % CH;
        const int j = kt + row;
        bf16x8 x = zero_bf16x8();
        if (j < kend) x = load8(base + (int64_t)(j - k_off) * ss + 8 * (is_v ? v_chunk<CH>(ph, row) : k_chunk<CH>(ph, row)));
        *reinterpret_cast<bf16x8*>(dst + p * 16) = x;
      }
    }
  };
  auto stage_kv = [&](int kt, char* dst, bool is_v) __attribute__((always_inline)) {
    stage_kv_b(is_v ? vbase : kbase, kt, dst, is_v);
  };
  // tile k's key position; tiles past the last one load nothing (zero rows),
  // so every wave has the same loads in flight at every wait
  auto tile_kt = [&](int k) __attribute__((always_inline)) { return k < n_tiles ? kv_lo + k * kKT : kend; };
  // The next item (PERS): its index nx (-1: none), and once nx_ok its key
  // range (nkvlo, nnt tiles) and K/V bases. Tile k >= n_tiles of this item's
  // stream is then the next item's tile k - n_tiles: the loads past this
  // item's last tile fetch the next item's first tiles, into the ring stages
  // that item will read them from.
  // (nt = 0 until the next item is known)
  NextItem* const nxi = reinterpret_cast<NextItem*>(lds + 9 * TILE + 64) + wave;
  if (PERS && lane == 0) nxi->nt = 0;

  // ---- the next item (PERS) ------------------------------------------------------
  // A workgroup draws its next item when the current one starts, settles the
  // draw at the item's first barrier (once its start loads have landed),
  // loads the next item's offsets row before iteration 0 issues its tiles,
  // and forms the next item's key range after B(0): from tile 1 on, the loads
  // past this item's last tile fetch the next item's first tiles. (Drawing
  // at the start holds one item ahead; the host takes the persistent grid
  // only where the items are many per workgroup, so that this costs little
  // balance.) These steps read the kernel arguments through a pointer the
  // compiler cannot follow, so that it loads them where they are used
  // instead of holding them in scalar registers through the key loop.
  unsigned tk = 0;
  auto kargs = []() __attribute__((always_inline)) {
    auto p = (const __attribute__((address_space(4))) PrefillArgs*)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(p));
    return p;
  };
  auto draw = [&]() __attribute__((always_inline)) {
    if (wave == 0 && lane == 0)
      tk = __hip_atomic_fetch_add((__attribute__((address_space(1))) unsigned*)(kargs()->sched + (blockIdx.x & 7)), 1u,
                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  // (wave 0) the draw's item, or one taken from another queue once this
  // queue is empty, or -1, into sh_next; a barrier must follow
  auto resolve = [&]() __attribute__((always_inline)) {
    if (wave == 0) {
      if (lane == 0) {
        const auto A = kargs();
        unsigned* const sched = A->sched;
        auto ctr = [&](int y) __attribute__((always_inline)) {
          return (__attribute__((address_space(1))) unsigned*)(sched + y);
        };
        const int n_it = A->B * A->Hkv * A->n_qtiles;
        const int grid = min(n_it, A->pgrid), home = (int)(blockIdx.x & 7);
        auto started = [&](int y) __attribute__((always_inline)) { return (unsigned)((grid - y + 7) >> 3); };
        auto queued = [&](int y) __attribute__((always_inline)) { return (unsigned)((n_it - y + 7) >> 3); };
        int nxt = -1;
        const unsigned v = tk + started(home);
        if (v < queued(home)) {
          nxt = (int)(v * 8 + home);
        } else {
          for (int s2 = 1; s2 < 8 && nxt < 0; ++s2) {
            const int y = (home + s2) & 7;
            const unsigned w = __hip_atomic_fetch_add(ctr(y), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + started(y);
            if (w < queued(y)) nxt = (int)(w * 8 + y);
          }
          if (nxt < 0 &&
              __hip_atomic_fetch_add(ctr(8), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (unsigned)grid - 1) {
            for (int y = 0; y < 9; ++y) __hip_atomic_store(ctr(y), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
        *sh_next = nxt;
      }
      __builtin_amdgcn_s_waitcnt(kLgkm0);
    }
  };
  // (after that barrier) the next item's offsets row
  auto fetch_next = [&]() __attribute__((always_inline)) {
    const auto A = kargs();
    const int nx = __builtin_amdgcn_readfirstlane(*sh_next);
    if (A->cu_docs && A->n_docs < 64)
      cu_n = A->cu_docs[(int64_t)(max(nx, 0) / A->Hkv % A->B) * (A->n_docs + 1) + min(lane, A->n_docs)];
  };
  // (once the row has landed) the next item's key range and K/V bases, into
  // this wave's slot: the loads past this item's last tile fetch its first
  // tiles from here on
  auto publish_next = [&]() __attribute__((always_inline)) {
    const auto A = kargs();
    const int nx = __builtin_amdgcn_readfirstlane(*sh_next);
    if (nx >= 0) {
      const int nkv = nx % A->Hkv, nr = nx / A->Hkv, nbb = nr % A->B;
      const int q0 = A->q_off, nd = A->n_docs;
      const int nt0 = (A->n_qtiles - 1 - nr / A->B) * TQ;
      int nst = 0;
      if (A->cu_docs && nd < 64) {
        const unsigned long long mk = __ballot(lane < nd && cu_n <= nt0 + q0);
        nst = __builtin_amdgcn_readlane(cu_n, mk ? 63 - __clzll(mk) : 0);
      } else if (A->cu_docs) {
        nst = doc_start(A->cu_docs + (int64_t)nbb * (nd + 1), nd, nt0 + q0);
      }
      const int nkvlo = max(0, min(nst, nt0 + q0));
      if (lane == 0) {
        nxi->kb = static_cast<const T*>(A->k) + nbb * A->ks_b + nkv * A->ks_h;
        nxi->vb = static_cast<const T*>(A->v) + nbb * A->vs_b + nkv * A->vs_h;
        nxi->kvlo = nkvlo;
        nxi->nt = (min(A->k_off + A->S - 1, min(nt0 + TQ, A->Sq) - 1 + q0) - nkvlo) / kKT + 1;
      }
    }
  };
  if (PERS) draw();
  auto stage_c = [&](int k, char* dst, bool is_v) __attribute__((always_inline)) {
    if constexpr (PERS) {
      if (k >= n_tiles) {
        const int nnt = __builtin_amdgcn_readfirstlane(nxi->nt);
        const int j = k - n_tiles;
        if (j < nnt)
          stage_kv_b(uniform_ptr(is_v ? nxi->vb : nxi->kb), __builtin_amdgcn_readfirstlane(nxi->kvlo) + j * kKT, dst,
                     is_v);
        else
          stage_kv(kend, dst, is_v);
      } else {
        stage_kv(tile_kt(k), dst, is_v);
      }
    } else {
      stage_kv(tile_kt(k), dst, is_v);
    }
  };

  // ---- per-lane LDS operand offsets ------------------------------------------
  // K operand: row 32kb + lc, logical chunk 2ks + hi.
  const int k_lane = lc * ROW;
  const int k_x = hi ^ (lc & (CH - 1));              // physical chunk = (2ks) ^ k_x
  const int k_row_x = k_lane + 16 * k_x;
  // V^T operand (transposing read): the 16-lane group g = lane/16 covers
  // d = 32db + 16(g&1) + (lane&15) and keys 16ks + 4hi (+8) + 0..3; its input
  // lane L = lane&15 addresses row 16ks + 4hi + L/4 at d0 = 32db + 16(g&1) + 4(L%4).
  const int L16 = lane & 15;
  const int vrow = 4 * hi + (L16 >> 2);
  int v_lane[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
    v_lane[db] = vrow * ROW + 16 * v_chunk<CH>(4 * db + 2 * ((lane >> 4) & 1) + ((L16 >> 1) & 1), vrow) + 8 * (L16 & 1);
  // the V region's start (64 KB) goes into the per-lane offsets, kept opaque
  // so that it is not folded back into the reads' immediate offsets, which
  // hold 16 bits: V reads take lds + stage * TILE as their base
  int v_region = 4 * TILE;
  asm volatile("" : "+v"(v_region));
#pragma unroll
  for (int db = 0; db < DB; ++db) v_lane[db] += v_region;

  // ---- the tile pipeline -----------------------------------------------------
  // K and V tiles go through separate four-stage rings: K of tile j in
  // K stage j % 4 (lds + (j % 4) TILE), V of tile j in V stage j % 4 (V region,
  // lds + (4 + j % 4) TILE). Barrier B(k) ends iteration k. Between B(k-1) and
  // B(k) every wave runs, for its 32 columns:
  //   PV(k-1): 4 DB MFMAs O^T += V^T P^T of tile k-1;
  //   the causal/document mask of tile k (edge tiles only);
  //   QK(k+1): 2 KS MFMAs t^T = K Q^T - Mref of tile k+1 (the queries carry
  //            scale * log2(e) and the accumulation starts from -Mref, so t
  //            is the exponent in log2 units), with the exponentials, bf16
  //            rounding and row sums of tile k interleaved;
  //   the lazy reference check of tile k.
  // The exponents of consecutive tiles are in two register buffers (tile
  // parity): QK(k+1) writes one while the exponentials read the other.
  // Operand reads run PF MFMAs ahead of their use, across the phase boundary
  // and across the barrier. Each piece of work is emitted in program order and
  // fenced (sched_barrier), so every wave keeps its own matrix core and VALU
  // busy at once; the two waves of a SIMD fill each other's waits.
  // Loads: in iteration k a wave issues K of tile k+3 (into the stage of
  // K(k-1), last read before B(k-2)) and V of tile k+2 (the stage of V(k-2),
  // last read before B(k-1)); before B(k) it waits until only the loads it
  // issued in iteration k may be pending, so K(k+2) and V(k+1), the first
  // tiles read after B(k), have landed for every wave once B(k) passes.
  constexpr int NQ = 2 * KS;      // QK MFMAs per tile
  constexpr int NP = 4 * DB;      // PV MFMAs per tile
  constexpr int PF = 3;           // operand reads ahead
  constexpr int EQ = 32 / NQ;     // scores per lane exponentiated per QK MFMA
  static_assert(PF <= NQ && PF <= NP && EQ % 2 == 0, "pipeline shape");
  char* const kst[4] = {lds, lds + TILE, lds + 2 * TILE, lds + 3 * TILE};
  char* const vst[4] = {lds + 4 * TILE, lds + 5 * TILE, lds + 6 * TILE, lds + 7 * TILE};
  // stages of the item's tile j (the ring position of tile 0 rotates from
  // item to item in a persistent workgroup)
  const int ph = PERS ? ph_c : 0;
  auto kst_at = [&](int j) __attribute__((always_inline)) { return lds + ((ph + j) & 3) * TILE; };
  auto vst_at = [&](int j) __attribute__((always_inline)) { return lds + (4 + ((ph + j) & 3)) * TILE; };

  // exponents t of tile j in tA (j even) or tB (j odd): element e = 16 kb + i
  // is element i of key block kb's t^T accumulator
  f32x16 tA[2], tB[2];
  uint32_t pw[16];                // weights e, e+1 as a bf16 pair in pw[e / 2]
  bf16x8 kbuf[NQ], vbuf[NP];      // operands read ahead
  float rs = 0.f;                 // this lane's sum of the tile's rounded weights

  // operand of QK MFMA i (key block i / KS, k-step i % KS) from the K stage
  // lk: row 32 kb + lc, physical chunk (2 ks) ^ k_x; k_lane is a multiple of
  // the row size, so the in-row byte offset 16 ((2 ks) ^ k_x) is the XOR of
  // k_row_x = k_lane + 16 k_x with 32 ks (one VALU op per k-step instead of a
  // register per k-step)
  auto rd_k = [&](const char* lk, int i) __attribute__((always_inline)) {
    return *reinterpret_cast<const bf16x8*>(lk + (i / KS) * 32 * ROW + (k_row_x ^ (32 * (i % KS))));
  };
  // operand of PV MFMA i (16-key step i / DB, 32-row block i % DB); lv is the
  // stage's offset from the V region (v_lane holds the region start)
  auto rd_v = [&](const char* lv, int i) __attribute__((always_inline)) {
    const char* vp = lv + 16 * (i / DB) * ROW + v_lane[i % DB];
    const i16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vp));
    const i16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vp + 8 * ROW));
    return __builtin_shufflevector(__builtin_bit_cast(bf16x4, r0), __builtin_bit_cast(bf16x4, r1),
                                   0, 1, 2, 3, 4, 5, 6, 7);
  };
  const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
  // weights of exponents e, e+1 of tt into P^T and the row sum
  auto exp_pair = [&](const f32x16 (&tt)[2], int e) __attribute__((always_inline)) {
    bf16x2 pr;
    pr[0] = to_bf16(fast_exp2(tt[e >> 4][e & 15]));
    pr[1] = to_bf16(fast_exp2(tt[(e + 1) >> 4][(e + 1) & 15]));
    pw[e >> 1] = __builtin_bit_cast(uint32_t, pr);
    rs = __builtin_amdgcn_fdot2_f32_bf16(pr, one2, rs, false);
  };
  // P^T operand of 16-key step ks (key block ks / 2, half ks % 2): weights
  // 8 ks .. 8 ks + 7
  auto p_op = [&](int ks) __attribute__((always_inline)) {
    const u32x4 w = {pw[4 * ks], pw[4 * ks + 1], pw[4 * ks + 2], pw[4 * ks + 3]};
    return __builtin_bit_cast(bf16x8, w);
  };
  // QK of the next tile (K stage lk) into tn with the weights of the current
  // one (exponents tc); the reads past the QK operands fetch the first PF V
  // operands of the current tile (V stage lv)
  auto phase_qk = [&](const char* __restrict__ lk, const char* __restrict__ lv, f32x16 (&tn)[2],
                      const f32x16 (&tc)[2]) __attribute__((always_inline)) {
    rs = 0.f;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const int kb = i / KS, ks = i % KS;
      tn[kb] = mfma32(kbuf[i], qreg[0][ks], ks == 0 ? negMv : tn[kb]);
      const int j = i + PF;
      if (j < NQ) kbuf[j] = rd_k(lk, j);
      else vbuf[j - NQ] = rd_v(lv, j - NQ);
#pragma unroll
      for (int e = EQ * i; e < EQ * (i + 1); e += 2) exp_pair(tc, e);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // tile k crosses a causal or document edge of the wave's columns, or the end
  // of the keys held
  // (bitwise, so that no branch is formed: a branch right after an MFMA can
  // leave the MFMA result read in its target without enough wait states)
  auto needs_mask = [&](int k) __attribute__((always_inline)) {
    const int kt = kv_lo + k * kKT;
    return (!wave_all_valid) | (kt + kKT - 1 > w_tmin + qo) | (kt < w_smax) | (kt + kKT > kend);
  };
  // PV of the previous tile (V stage lv); the reads past the PV operands
  // fetch the first PF K operands of tile k+1 (K stage lk2). Without QS the
  // scale FMA of tile k's scores (tc) is interleaved, each result pinned
  // where it is formed (an empty asm that takes it in a register), or the
  // compiler would move the FMAs out of the MFMA stream.
  constexpr int EP = 32 / NP;     // scores per lane scaled per PV MFMA (without QS)
  auto phase_pv = [&](const char* __restrict__ lv, const char* __restrict__ lk2, f32x16 (&tc)[2])
      __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int ks = i / DB, db = i % DB;
      acc[db] = mfma32(vbuf[i], p_op(ks), acc[db]);
      const int j = i + PF;
      if (j < NP) vbuf[j] = rd_v(lv, j);
      else kbuf[j - NP] = rd_k(lk2, j - NP);
      if constexpr (!QS) {
#pragma unroll
        for (int e = EP * i; e < EP * (i + 1); ++e) {
          tc[e >> 4][e & 15] = fmaf(tc[e >> 4][e & 15], a.scale_log2, negM);
          asm volatile("" : "+v"(tc[e >> 4][e & 15]));
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // the causal/document mask of tile k's scores (applied to tiles that cross
  // an edge of the wave's columns): key rows of this lane's scores are
  // 32 kb + 8 (j / 4) + 4 hi + j % 4, visible when in [st, min(tok + qo,
  // kend - 1)]; keys at or past kend (a ring step's key shard can end before
  // the rows' positions) are masked too
  auto mask_tile = [&](int k, f32x16 (&tt)[2]) __attribute__((always_inline)) {
    const int kt = kv_lo + k * kKT;
    const int lo4 = (valid[0] ? st[0] - kt : kKT) - 4 * hi;
    const int hi4 = (valid[0] ? min(tok[0] + qo, kend - 1) - kt : -1) - 4 * hi;
#pragma unroll
    for (int e = 0; e < 32; ++e) {
      const int r = 32 * (e >> 4) + 8 * ((e & 15) >> 2) + (e & 3);
      tt[e >> 4][e & 15] = (r >= lo4 && r <= hi4) ? tt[e >> 4][e & 15] : -INFINITY;
    }
  };
  // the last PV (tile n_tiles - 1, V stage lv): its first PF operands were
  // read by the last QK phase
  auto phase_pv_last = [&](const char* lv) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int ks = i / DB, db = i % DB;
      if (i + PF < NP) vbuf[i + PF] = rd_v(lv, i + PF);
      acc[db] = mfma32(vbuf[i], p_op(ks), acc[db]);
    }
  };
  // After the weights of a tile (exponents tc): the reference must move only
  // if a weight may exceed kLazyW (some lane's sum of them does) or the column
  // has no reference yet. It then moves up to the tile's column max (d = how
  // far, in log2 units), the accumulator and row sum are scaled by 2^-d and
  // the weights are formed again; the next tile's exponents (tn, formed from
  // the old reference) move by d too. A column still without a visible key
  // keeps Mref = -inf. Softmax does not depend on the reference, so this is
  // exact.
  auto settle = [&](f32x16 (&tc)[2], f32x16 (&tn)[2]) __attribute__((always_inline)) {
    if (__any(Mref == -INFINITY || !(rs <= kLazyW))) {
      float mx = tc[0][0];
#pragma unroll
      for (int e = 1; e < 32; ++e) mx = fmaxf(mx, tc[e >> 4][e & 15]);
      mx = max_xor32(mx);
      const bool none = Mref == -INFINITY;
      const float d = none ? (mx > -INFINITY ? mx : 0.f) : fmaxf(mx, 0.f);
      const float al = none ? 1.f : fast_exp2(-d);
      Mref = none ? (mx > -INFINITY ? mx : -INFINITY) : Mref + d;
      negM = Mref == -INFINITY ? 0.f : -Mref;
      if constexpr (QS) {
#pragma unroll
        for (int j = 0; j < 16; ++j) negMv[j] = negM;
      }
      l *= al;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db] *= al;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        tc[kb] -= d;
        if constexpr (QS) tn[kb] -= d;   // (without QS tn holds raw scores)
      }
      rs = 0.f;
#pragma unroll
      for (int e = 0; e < 32; e += 2) exp_pair(tc, e);
    }
    l += rs;
  };
  // only the loads issued after the previous barrier (2 NL per wave) may be
  // pending, then the barrier (the fp32 path writes its stages with ds_write:
  // drain those first)
  auto sync_tiles = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * NL));
    if constexpr (!std::is_same<T, __bf16>::value) __builtin_amdgcn_s_waitcnt(kLgkm0);
    __builtin_amdgcn_s_barrier();
  };
  // Iteration k (1 <= k < n_tiles) of the loop below, stage indices as
  // constants: PV(k-1) with the scale FMA (and mask) of tile k, the loads of
  // K(k+3) and V(k+2), then QK(k+1) with the weights of tile k. Its LDS
  // pointers are restrict parameters of one call, so the compiler does not
  // take the direct-to-LDS loads it issues as writers of what its reads fetch;
  // the waits and barriers order the stages.
  auto iter = [&](char* __restrict__ kdst, char* __restrict__ vdst, const char* __restrict__ vprev,
                  const char* __restrict__ knext, const char* __restrict__ vcur, int k, f32x16 (&tc)[2],
                  f32x16 (&tn)[2]) __attribute__((always_inline)) {
    const bool masked = needs_mask(k);
    phase_pv(vprev - 4 * TILE, knext, tc);
    if (masked) mask_tile(k, tc);
    // (issued here rather than before the PV: the register allocator then
    // keeps every operand in registers; issued earlier they measured no faster)
    stage_c(k + 3, kdst, false);
    stage_c(k + 2, vdst, true);
    phase_qk(knext, vcur - 4 * TILE, tn, tc);
  };
  // Iteration 0: the loads of K3 and V2, QK of tile 0 (its operands read
  // here), the scale FMA and mask of tile 0, the first K1 operands, then QK(1)
  // with the weights of tile 0.
  // (P: tile 0's exponents go to tB instead of tA, for a ring position of odd
  // parity)
  auto iter0 = [&](auto P, char* __restrict__ kdst, char* __restrict__ vdst, const char* __restrict__ k0,
                   const char* __restrict__ k1, const char* __restrict__ v0) __attribute__((always_inline)) {
    f32x16(&t0)[2] = decltype(P)::value ? tB : tA;
    f32x16(&t1)[2] = decltype(P)::value ? tA : tB;
    const bool masked = needs_mask(0);
    stage_c(3, kdst, false);
    stage_c(2, vdst, true);
#pragma unroll
    for (int i = 0; i < NQ; ++i) kbuf[i] = rd_k(k0, i);
#pragma unroll
    for (int i = 0; i < NQ; ++i) t0[i / KS] = mfma32(kbuf[i], qreg[0][i % KS], i % KS == 0 ? negMv : t0[i / KS]);
    // (no PV precedes tile 0: its scale FMA (without QS) and mask run on
    // their own)
    if constexpr (!QS) {
#pragma unroll
      for (int e = 0; e < 32; ++e) t0[e >> 4][e & 15] = fmaf(t0[e >> 4][e & 15], a.scale_log2, negM);
    }
    if (masked) mask_tile(0, t0);
#pragma unroll
    for (int i = 0; i < PF; ++i) kbuf[i] = rd_k(k1, i);
    phase_qk(k1, v0 - 4 * TILE, t1, t0);
  };

  // ---- prologue loads: K0, K1, V0, K2, V1 (K and V stage 3 hold the RoPE table) --
  // (those the previous item of a persistent workgroup has not loaded)
  const int kpf = PERS ? kpf_c : 3, vpf = PERS ? vpf_c : 2;
  if (kpf > 0) stage_c(0, kst_at(0), false);
  if (kpf > 1) stage_c(1, kst_at(1), false);
  if (vpf > 0) stage_c(0, vst_at(0), true);
  if (kpf > 2) stage_c(2, kst_at(2), false);
  if (vpf > 1) stage_c(1, vst_at(1), true);
  if (QS && rope_q) {
    // RoPE of this lane's query channels 16ks + 8hi + 0..7, i.e. the pairs
    // k = 8ks + 4hi + p (adjacent pairs (2k, 2k+1)) or, for half-split pairs
    // (k, k + D/2), k = 16ks + 8hi + i for ks < KS/2 with the same channels of
    // ks + KS/2 as partners: the angle position * theta_k is formed and reduced
    // in fp64 in revolutions (theta_k / 2pi from the host), its sine and
    // cosine taken in fp32 (v_sin/v_cos take revolutions), the pair rotated
    // in fp32 and rounded to bf16. Runs while the first K/V tiles load.
    auto rotate = [&](const float* x, const f32x4& cv, const f32x4& sv) __attribute__((always_inline)) {
      bf16x8 r;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        r[2 * p] = to_bf16(fmaf(x[2 * p], cv[p], -x[2 * p + 1] * sv[p]) * qscale);
        r[2 * p + 1] = to_bf16(fmaf(x[2 * p], sv[p], x[2 * p + 1] * cv[p]) * qscale);
      }
      return r;
    };
    // half-split pairs: elements e0 + 0..3 of x (first half) and y (second
    // half, same positions), rotated into r and t
    auto rotate_half = [&](const float* x, const float* y, int e0, const f32x4& cv, const f32x4& sv,
                           bf16x8& r, bf16x8& t) __attribute__((always_inline)) {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        r[e0 + p] = to_bf16(fmaf(x[e0 + p], cv[p], -y[e0 + p] * sv[p]) * qscale);
        t[e0 + p] = to_bf16(fmaf(x[e0 + p], sv[p], y[e0 + p] * cv[p]) * qscale);
      }
    };
    if constexpr (TQ * (D / 2) * 4 <= TILE) {
      // The g lanes of a token share its angles: the workgroup forms the
      // cosine and sine of each (token, pair) once, into the fourth K and V
      // stages (free until tile 3 is issued), token rows of D/2 values with
      // 16-byte chunk c at c ^ (row & (CH - 1)).
      for (int e = tid; e < TQ * CH; e += 64 * kNW) {
        const int tt = e % TQ, c = e / TQ;
        const int t = min(t0 + tt, Sq - 1);
        const double pos = a.positions ? (double)a.positions[(int64_t)b * Sq + t] : (double)(t + qo);
        f32x4 cv, sv;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const double rev = pos * a.theta_rev[4 * c + p];
          const float fr = (float)(rev - rint(rev));   // in [-1/2, 1/2]
          cv[p] = __builtin_amdgcn_cosf(fr);
          sv[p] = __builtin_amdgcn_sinf(fr);
        }
        const int off = tt * ROW + 16 * (c ^ (tt & (CH - 1)));
        *reinterpret_cast<f32x4*>(kst_at(3) + off) = cv;
        *reinterpret_cast<f32x4*>(vst_at(3) + off) = sv;
      }
      // the table's writes are LDS only: the barrier waits for them, not for
      // the tile loads in flight (__syncthreads would wait for those too)
      __builtin_amdgcn_s_waitcnt(kLgkm0);
      __builtin_amdgcn_s_barrier();
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb) {
        const int tt = (wave * 32 * kCB + cb * 32 + lc) / G;
        auto tab = [&](int c, int which) __attribute__((always_inline)) {   // 4 pairs from chunk c
          return *reinterpret_cast<const f32x4*>((which ? vst_at(3) : kst_at(3)) + tt * ROW +
                                                  16 * (c ^ (tt & (CH - 1))));
        };
        if (a.rope_half) {
          // channel 16ks + 8hi + i of the first half pairs with the same
          // channel of the second half (ks + KS/2): pairs 16ks + 8hi + i
#pragma unroll
          for (int ks = 0; ks < KS / 2; ++ks)
#pragma unroll
            for (int h = 0; h < 2; ++h)
              rotate_half(qraw[cb][ks], qraw[cb][ks + KS / 2], 4 * h, tab(4 * ks + 2 * hi + h, 0),
                          tab(4 * ks + 2 * hi + h, 1), qreg[cb][ks], qreg[cb][ks + KS / 2]);
        } else {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            qreg[cb][ks] = rotate(qraw[cb][ks], tab(2 * ks + hi, 0), tab(2 * ks + hi, 1));
        }
      }
    } else {
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb) {
        const int t = min(tok[cb], Sq - 1);
        const double pos = a.positions ? (double)a.positions[(int64_t)b * Sq + t] : (double)(t + qo);
        // cos and sin of pairs k0 + hi_step * hi + 0..3
        auto angles = [&](int k0, int hi_step, f32x4& cv, f32x4& sv) __attribute__((always_inline)) {
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const double th = hi ? a.theta_rev[k0 + hi_step + p] : a.theta_rev[k0 + p];
            const double rev = pos * th;
            const float fr = (float)(rev - rint(rev));   // in [-1/2, 1/2]
            cv[p] = __builtin_amdgcn_cosf(fr);
            sv[p] = __builtin_amdgcn_sinf(fr);
          }
        };
        if (a.rope_half) {
#pragma unroll
          for (int ks = 0; ks < KS / 2; ++ks)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              f32x4 cv, sv;
              angles(16 * ks + 4 * h, 8, cv, sv);
              rotate_half(qraw[cb][ks], qraw[cb][ks + KS / 2], 4 * h, cv, sv, qreg[cb][ks],
                          qreg[cb][ks + KS / 2]);
            }
        } else {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            f32x4 cv, sv;
            angles(8 * ks, 4, cv, sv);
            qreg[cb][ks] = rotate(qraw[cb][ks], cv, sv);
          }
        }
      }
    }
  }
  if constexpr (PERS) {
    // every load of the item's start has landed (and the previous item's
    // stores, and the draw); the next item's offsets row is loaded before
    // iteration 0 issues its tiles, so that B(0) covers it
    __builtin_amdgcn_s_waitcnt(0);
    resolve();
    __builtin_amdgcn_s_barrier();
    fetch_next();
  } else {
    sync_tiles();   // K0, K1, V0 landed; every wave is done with the RoPE table
  }
  if (!PERS || (ph & 1) == 0) {
    iter0(std::integral_constant<int, 0>{}, kst_at(3), vst_at(2), kst_at(0), kst_at(1), vst_at(0));
    settle(tA, tB);
  } else {
    iter0(std::integral_constant<int, 1>{}, kst_at(3), vst_at(2), kst_at(0), kst_at(1), vst_at(0));
    settle(tB, tA);
  }
  sync_tiles();   // B(0)
  if (PERS) publish_next();
  // Unrolled over the four stage indices so every stage offset is a constant.
  // The loop has one exit: steps at or past the last tile are skipped by a
  // uniform branch that rejoins (an exit after every unrolled step keeps the
  // register allocator from merging the accumulators' copies).
  auto step = [&](auto U, int k) __attribute__((always_inline)) {
    constexpr int u = decltype(U)::value;   // ring stage of tile k: (ph + k) % 4
    if (k < n_tiles && (!PERS || k >= 1)) {
      // exponents of tile k in tA (k even) or tB; tile k+1's go to the other
      f32x16(&tc)[2] = (u & 1) ? tB : tA;
      f32x16(&tn)[2] = (u & 1) ? tA : tB;
      iter(kst[(u + 3) & 3], vst[(u + 2) & 3], vst[(u + 3) & 3], kst[(u + 1) & 3], vst[u], k, tc, tn);
      settle(tc, tn);
      sync_tiles();   // B(k)
    }
  };
  for (int k = 1 - ph; k < n_tiles; k += 4) {
    step(std::integral_constant<int, 1>{}, k);
    step(std::integral_constant<int, 2>{}, k + 1);
    step(std::integral_constant<int, 3>{}, k + 2);
    step(std::integral_constant<int, 0>{}, k + 3);
  }
  // PV of the last tile, from V stage (ph + n_tiles - 1) % 4
  switch ((ph + n_tiles - 1) & 3) {
    case 0: phase_pv_last(vst[0] - 4 * TILE); break;
    case 1: phase_pv_last(vst[1] - 4 * TILE); break;
    case 2: phase_pv_last(vst[2] - 4 * TILE); break;
    default: phase_pv_last(vst[3] - 4 * TILE); break;
  }
  if constexpr (PERS) {
    // the next item's queries, while this one's output is written (the
    // loads past the last tile, the next item's first tiles, stay in flight)
    // (unconditional, so that the registers are not live across the item:
    // with no next item this item's queries are fetched again, unused)
    const int nx = __builtin_amdgcn_readfirstlane(*sh_next);
    const int nr = nx / a.Hkv;
    load_q(nx >= 0 ? nr % a.B : b, nx >= 0 ? nx % a.Hkv : kvh, nx >= 0 ? a.n_qtiles - 1 - nr / a.B : qtile);
  } else {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));          // loads past the last tile
  }

  // ---- epilogue --------------------------------------------------------------
  // o = acc / lt as the reciprocal's product plus one residual step
  // (q + (acc - q lt) / lt, residual by FMA): a quotient that fp32 can hold
  // comes out exactly, so a row whose weights are all exact gets an exactly
  // rounded mean
  // (a row with no visible key in its range, possible with split key
  // ranges, gets o = 0 and lse = -inf)
  float lt[kCB], rl[kCB];
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) {
    lt[cb] = l + __shfl_xor(l, 32);
    rl[cb] = lt[cb] > 0.f ? __builtin_amdgcn_rcpf(lt[cb]) : 0.f;
  }
  auto quot = [&](float x, int cb) __attribute__((always_inline)) {
    const float q = x * rl[cb];
    return fmaf(fmaf(-q, lt[cb], x), rl[cb], q);
  };
  auto row_lse = [&](int cb) __attribute__((always_inline)) {
    return lt[cb] > 0.f ? (Mref + fast_log2(lt[cb])) * kLn2 : -INFINITY;
  };
  if (!PERS && a.acc_mode) {
    // ring step: this shard's (o, lse) of every row, written (first step) or
    // merged by log-sum-exp weight into the fp32 accumulators (o_acc, lse_acc);
    // a workgroup owns its rows, so the read-merge-write needs no atomics.
    // A last merging step (acc_mode 3) writes the merged rows as the final o
    // and lse instead, the values the finalize would take from the
    // accumulators (o = 0 where lse = -inf)
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
      if (!valid[cb]) continue;
      float* op = a.o_acc + (((int64_t)b * Sq + tok[cb]) * a.Hq + head[cb]) * D;
      float* lp = a.lse_acc + ((int64_t)b * a.Hq + head[cb]) * Sq + tok[cb];
      const float ln = row_lse(cb);
      float wo = 0.f, wn = 1.f, rw = 1.f, lout = ln;
      if (a.acc_mode >= 2) {
        const float lo_ = *lp;
        const float mx = fmaxf(lo_, ln);
        if (mx > -INFINITY) {
          wo = __expf(lo_ - mx);
          wn = __expf(ln - mx);
          rw = 1.f / (wo + wn);
          lout = mx + __logf(wo + wn);
        } else {
          wo = 1.f;   // nothing seen yet on either side: o stays 0
          wn = 0.f;
          lout = -INFINITY;
        }
      }
      // the accumulated row x merged with this shard's v, in one fixed order of
      // operations for both forms of the merging step
      auto merge4 = [&](const f32x4& x, const f32x4& v) __attribute__((always_inline)) {
        f32x4 r;
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = fmaf(wo, x[e], wn * v[e]) * rw;
        return r;
      };
      if (a.acc_mode == 3) {
        T* fo = static_cast<T*>(a.o) + b * a.os_b + tok[cb] * a.os_s + head[cb] * a.os_h;
        const float keep = lout > -INFINITY ? 1.f : 0.f;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int jq = 0; jq < 4; ++jq) {
            const int d = db * 32 + 8 * jq + 4 * hi;
            f32x4 v = {quot(acc[db][4 * jq], cb), quot(acc[db][4 * jq + 1], cb),
                       quot(acc[db][4 * jq + 2], cb), quot(acc[db][4 * jq + 3], cb)};
            v = merge4(*reinterpret_cast<const f32x4*>(op + d), v);
            store4(fo + d, v[0] * keep, v[1] * keep, v[2] * keep, v[3] * keep);
          }
        if (hi == 0 && a.lse) a.lse[((int64_t)b * a.Hq + head[cb]) * Sq + tok[cb]] = lout;
        continue;
      }
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int jq = 0; jq < 4; ++jq) {
          f32x4* dst = reinterpret_cast<f32x4*>(op + db * 32 + 8 * jq + 4 * hi);
          f32x4 v = {quot(acc[db][4 * jq], cb), quot(acc[db][4 * jq + 1], cb),
                     quot(acc[db][4 * jq + 2], cb), quot(acc[db][4 * jq + 3], cb)};
          if (a.acc_mode == 2) v = merge4(*dst, v);
          *dst = v;
        }
      __builtin_amdgcn_s_waitcnt(0);   // both halves of the row have read lse before it changes
      __builtin_amdgcn_wave_barrier();
      if (hi == 0) *lp = lout;
    }
    return;
  }
  if (!PERS && n_split > 1) {
    // partial result of this split: fp32 o (normalised by its own row sum)
    // and lse, slot sp
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
      if (!valid[cb]) continue;
      float* op = a.o_part + ((((int64_t)sp * a.B + b) * Sq + tok[cb]) * a.Hq + head[cb]) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int jq = 0; jq < 4; ++jq) {
          const f32x4 v = {quot(acc[db][4 * jq], cb), quot(acc[db][4 * jq + 1], cb),
                           quot(acc[db][4 * jq + 2], cb), quot(acc[db][4 * jq + 3], cb)};
          *reinterpret_cast<f32x4*>(op + db * 32 + 8 * jq + 4 * hi) = v;
        }
      if (hi == 0) a.lse_part[(((int64_t)sp * a.B + b) * a.Hq + head[cb]) * Sq + tok[cb]] = row_lse(cb);
    }
    return;
  }
  if constexpr (std::is_same<T, __bf16>::value) {
    // Through LDS, so that the stores are whole rows: a lane holds 4-value
    // pieces of its column's row; each wave writes its 32 rows into its own
    // 32 x ROW bytes of LDS (16-byte chunk c of row r at c ^ (r & (CH - 1)),
    // so the 32 rows of one write do not all land in one bank) and reads them
    // back 16 contiguous bytes per lane, D/8 lanes per row. The barrier
    // orders every wave's last operand reads and LDS-direct loads before the
    // stage memory is reused; each wave then only touches its own rows.
    char* ow = lds + wave * 32 * ROW;
    if constexpr (PERS) {
      // Only the stages the next item's first tiles do not use: K stage of
      // its tile 3, V stages of its tiles 2 and 3, and the ninth tile, two
      // waves to a tile. The barrier orders every wave's last operand reads.
      const int nph = (ph + n_tiles) & 3;
      const int rg = wave >> 1;
      char* const base = rg == 0 ? lds + ((nph + 3) & 3) * TILE
                         : rg == 1 ? lds + (4 + ((nph + 2) & 3)) * TILE
                         : rg == 2 ? lds + (4 + ((nph + 3) & 3)) * TILE
                                   : lds + 8 * TILE;
      ow = base + (wave & 1) * 32 * ROW;
      __builtin_amdgcn_s_waitcnt(kLgkm0);
      __builtin_amdgcn_s_barrier();
    } else {
      __syncthreads();
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = to_bf16(quot(acc[db][4 * jq + e], 0));
        *reinterpret_cast<bf16x4*>(ow + lc * ROW + 16 * ((4 * db + jq) ^ (lc & (CH - 1))) + 8 * hi) = v;
      }
    constexpr int RPI = 64 / CH;   // rows per wave-wide 16-byte access
    const int ch = lane % CH;
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int row = i * RPI + lane / CH;
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(ow + row * ROW + 16 * (ch ^ (row & (CH - 1))));
      const int col = wave * 32 + row;
      const int t = t0 + col / G;
      if (t < Sq)
        *reinterpret_cast<bf16x8*>(static_cast<T*>(a.o) + b * a.os_b + t * a.os_s + (kvh * G + col % G) * a.os_h +
                                   8 * ch) = v;
    }
  } else {
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
      if (!valid[cb]) continue;
      T* op = static_cast<T*>(a.o) + b * a.os_b + tok[cb] * a.os_s + head[cb] * a.os_h;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int jq = 0; jq < 4; ++jq) {
          const int d = db * 32 + 8 * jq + 4 * hi;
          store4(op + d, quot(acc[db][4 * jq], cb), quot(acc[db][4 * jq + 1], cb),
                 quot(acc[db][4 * jq + 2], cb), quot(acc[db][4 * jq + 3], cb));
        }
    }
  }
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) {
    if (hi != 0 || !valid[cb]) continue;
    if (a.lse) a.lse[((int64_t)b * a.Hq + head[cb]) * Sq + tok[cb]] = row_lse(cb);
    if (a.split_tiles > 0) a.lse_part[((int64_t)b * a.Hq + head[cb]) * Sq + tok[cb]] = INFINITY;
  }
  if constexpr (PERS) {
    const int nx = __builtin_amdgcn_readfirstlane(*sh_next);
    if (nx < 0) {
      __builtin_amdgcn_s_waitcnt(0);   // the loads past the last tile
      return;
    }
    // every wave's output reads are done before the next item's RoPE table
    // reuses those stages
    __builtin_amdgcn_s_waitcnt(kLgkm0);
    __builtin_amdgcn_s_barrier();
    // The next item starts at ring stage ph + n_tiles. The loads of
    // iterations 1 .. n_tiles - 1 fetched its K tiles j >= 4 - n_tiles and V
    // tiles j >= 3 - n_tiles; its start loads the others.
    item = nx;
    ph_c = (ph + n_tiles) & 3;
    kpf_c = n_tiles >= 2 ? max(0, 4 - n_tiles) : 3;
    vpf_c = n_tiles >= 2 ? max(0, 3 - n_tiles) : 2;
  } else {
    return;
  }
  }   // items
}

template <typename T, int D, int G>
hipError_t launch_t(const PrefillArgs& a, hipStream_t st) {
  const unsigned grid = (unsigned)a.B * a.Hkv * a.n_qtiles;
  const unsigned splits = a.split_tiles > 0 ? (unsigned)a.max_splits : 1u;
  // bf16 queries that arrive rotated keep their exact values (no QS); fp32
  // queries and queries the kernel rotates are scaled before their rounding
  if constexpr (std::is_same<T, __bf16>::value) {
    if (a.sched) {
      // persistent grid: one workgroup per compute unit (the LDS use allows
      // no more), items drawn from the queues in a.sched
      const unsigned pg = std::min(grid, (unsigned)a.pgrid);
      if (!a.rope_q)
        hipLaunchKernelGGL((prefill_kernel<T, D, G, false, true>), dim3(pg), dim3(64 * kNW), 0, st, a);
      else
        hipLaunchKernelGGL((prefill_kernel<T, D, G, true, true>), dim3(pg), dim3(64 * kNW), 0, st, a);
      return hipGetLastError();
    }
    if (!a.rope_q) {
      hipLaunchKernelGGL((prefill_kernel<T, D, G, false, false>), dim3(grid, splits), dim3(64 * kNW), 0, st, a);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((prefill_kernel<T, D, G, true, false>), dim3(grid, splits), dim3(64 * kNW), 0, st, a);
  return hipGetLastError();
}

// Merge of split partials: one group of D/4 lanes per (sequence, query row,
// head), 4 values per lane. Rows marked +inf in slot 0 were written whole by
// the prefill kernel; the others take M = max_s lse_s, w_s = exp(lse_s - M),
// o = sum_s w_s o_s / sum_s w_s, lse = M + ln(sum_s w_s) over the slots with
// lse_s > -inf.
constexpr int kMergeSlots = 8;   // slots merged with all loads issued at once

template <typename T, int D>
__global__ __launch_bounds__(256) void merge_kernel(PrefillArgs a) {
  constexpr int LPR = D / 4;             // lanes per row
  constexpr int RPB = 256 / LPR;         // rows per block
  const int64_t r = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;   // (b, tok, head), head fastest
  const int lane = threadIdx.x % LPR;
  const int64_t rows = (int64_t)a.B * a.Sq * a.Hq;
  if (r >= rows) return;
  const int h = (int)(r % a.Hq);
  const int64_t bt = r / a.Hq;
  const int tok = (int)(bt % a.Sq), b = (int)(bt / a.Sq);
  const int64_t slot_stride = (int64_t)a.B * a.Hq * a.Sq;
  const float* lp = a.lse_part + ((int64_t)b * a.Hq + h) * a.Sq + tok;
  if (lp[0] == INFINITY) return;
  float M = -INFINITY;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float W = 0.f;
  auto o_of = [&](int s) __attribute__((always_inline)) {
    return *reinterpret_cast<const f32x4*>(a.o_part + ((((int64_t)s * a.B + b) * a.Sq + tok) * a.Hq + h) * D +
                                           4 * lane);
  };
  if (a.max_splits <= kMergeSlots) {
    // every slot's lse and o loaded at once (an unused slot's o is whatever
    // the workspace holds: it is selected away, never multiplied)
    float ls[kMergeSlots];
    f32x4 o[kMergeSlots];
#pragma unroll
    for (int s = 0; s < kMergeSlots; ++s) {
      ls[s] = s < a.max_splits ? lp[s * slot_stride] : -INFINITY;
      if (s < a.max_splits) o[s] = o_of(s);
      M = fmaxf(M, ls[s]);
    }
    if (M > -INFINITY) {
#pragma unroll
      for (int s = 0; s < kMergeSlots; ++s) {
        const bool live = ls[s] > -INFINITY;
        const float w = live ? __expf(ls[s] - M) : 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = live ? acc[i] + w * o[s][i] : acc[i];
        W += w;
      }
    }
  } else {
    for (int s = 0; s < a.max_splits; ++s) M = fmaxf(M, lp[s * slot_stride]);
    if (M > -INFINITY) {
      for (int s = 0; s < a.max_splits; ++s) {
        const float ls = lp[s * slot_stride];
        if (!(ls > -INFINITY)) continue;
        const float w = __expf(ls - M);
        acc += w * o_of(s);
        W += w;
      }
    }
  }
  const float rw = W > 0.f ? 1.f / W : 0.f;
  T* op = static_cast<T*>(a.o) + b * a.os_b + tok * a.os_s + h * a.os_h + 4 * lane;
  store4(op, acc[0] * rw, acc[1] * rw, acc[2] * rw, acc[3] * rw);
  if (a.lse && lane == 0) a.lse[((int64_t)b * a.Hq + h) * a.Sq + tok] = W > 0.f ? M + __logf(W) : -INFINITY;
}

// The ring's finalize: one fp32 accumulator slot, already normalised, so the
// merge above reduces to o = o_acc where lse_acc > -inf (else 0) and lse =
// lse_acc (its weight is exp(0) = 1, the same values bit for bit). D/8 lanes
// per (sequence, query row, head), 8 values per lane; the row's lse and its o
// are loaded together, not one after the other.
template <typename T, int D>
__global__ __launch_bounds__(256) void finalize_kernel(PrefillArgs a) {
  constexpr int LPR = D / 8;             // lanes per row
  constexpr int RPB = 256 / LPR;         // rows per block
  const int64_t r = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;   // (b, tok, head), head fastest
  const int lane = threadIdx.x % LPR;
  const int64_t rows = (int64_t)a.B * a.Sq * a.Hq;
  if (r >= rows) return;
  const int h = (int)(r % a.Hq);
  const int64_t bt = r / a.Hq;
  const int tok = (int)(bt % a.Sq), b = (int)(bt / a.Sq);
  const int64_t li = ((int64_t)b * a.Hq + h) * a.Sq + tok;
  const float* src = a.o_part + r * D + 8 * lane;
  const float ls = a.lse_part[li];
  const f32x4 o0 = *reinterpret_cast<const f32x4*>(src);
  const f32x4 o1 = *reinterpret_cast<const f32x4*>(src + 4);
  const float keep = ls > -INFINITY ? 1.f : 0.f;
  T* op = static_cast<T*>(a.o) + b * a.os_b + tok * a.os_s + h * a.os_h + 8 * lane;
  store4(op, o0[0] * keep, o0[1] * keep, o0[2] * keep, o0[3] * keep);
  store4(op + 4, o1[0] * keep, o1[1] * keep, o1[2] * keep, o1[3] * keep);
  if (a.lse && lane == 0) a.lse[li] = ls > -INFINITY ? ls : -INFINITY;
}

template <typename T, int D>
hipError_t launch_finalize_t(const PrefillArgs& a, hipStream_t st) {
  constexpr int RPB = 256 / (D / 8);
  const int64_t rows = (int64_t)a.B * a.Sq * a.Hq;
  hipLaunchKernelGGL((finalize_kernel<T, D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_merge_t(const PrefillArgs& a, hipStream_t st) {
  constexpr int RPB = 256 / (D / 4);
  const int64_t rows = (int64_t)a.B * a.Sq * a.Hq;
  hipLaunchKernelGGL((merge_kernel<T, D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_g(const PrefillArgs& a, int G, hipStream_t st) {
  switch (G) {
    case 1: return launch_t<T, D, 1>(a, st);
    case 2: return launch_t<T, D, 2>(a, st);
    case 4: return launch_t<T, D, 4>(a, st);
    case 8: return launch_t<T, D, 8>(a, st);
    case 16: return launch_t<T, D, 16>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// ---- work-queue counters of the persistent grid --------------------------------
// A file-scope device array: each device holds its own copy, zero from module
// load. A stream gets one 128-byte slot of it on first use and keeps it:
// launches on one stream run one after another, and each launch leaves its
// counters at zero, so the slot needs no clearing. A stream under graph
// capture gets none (the launch then takes one workgroup per item), so a
// captured graph never shares a slot with calls made outside it.
constexpr int kSchedSlots = 64;
constexpr int kSchedWords = 32;
static __device__ __align__(256) unsigned prefill_queues[kSchedSlots * kSchedWords];

namespace {
constexpr int kMaxSchedDevices = 64;
std::mutex g_sched_mu;
unsigned* g_sched_base[kMaxSchedDevices];
hipStream_t g_sched_stream[kMaxSchedDevices][kSchedSlots];
int g_sched_used[kMaxSchedDevices];
}  // namespace

hipError_t prefill_sched(hipStream_t st, unsigned** out) {
  *out = nullptr;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cs) != hipSuccess) {
    (void)hipGetLastError();
    return hipSuccess;
  }
  if (cs != hipStreamCaptureStatusNone) return hipSuccess;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxSchedDevices) return hipSuccess;
  std::lock_guard<std::mutex> lock(g_sched_mu);
  if (g_sched_base[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(prefill_queues));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_sched_base[dev] = static_cast<unsigned*>(p);
  }
  int slot = -1;
  for (int i = 0; i < g_sched_used[dev]; ++i)
    if (g_sched_stream[dev][i] == st) slot = i;
  if (slot < 0) {
    if (g_sched_used[dev] == kSchedSlots) return hipSuccess;   // out of slots: no persistent grid
    slot = g_sched_used[dev]++;
    g_sched_stream[dev][slot] = st;
  }
  *out = g_sched_base[dev] + slot * kSchedWords;
  return hipSuccess;
}

hipError_t launch_prefill(const PrefillArgs& a, int D, int G, int dt, hipStream_t st) {
  if (dt == 0) return D == 64 ? launch_g<__bf16, 64>(a, G, st) : launch_g<__bf16, 128>(a, G, st);
  return D == 64 ? launch_g<float, 64>(a, G, st) : launch_g<float, 128>(a, G, st);
}

hipError_t launch_ring_finalize(const PrefillArgs& a, int D, int dt, hipStream_t st) {
  if (dt == 0) return D == 64 ? launch_finalize_t<__bf16, 64>(a, st) : launch_finalize_t<__bf16, 128>(a, st);
  return D == 64 ? launch_finalize_t<float, 64>(a, st) : launch_finalize_t<float, 128>(a, st);
}

hipError_t launch_prefill_merge(const PrefillArgs& a, int D, int dt, hipStream_t st) {
  if (dt == 0) return D == 64 ? launch_merge_t<__bf16, 64>(a, st) : launch_merge_t<__bf16, 128>(a, st);
  return D == 64 ? launch_merge_t<float, 64>(a, st) : launch_merge_t<float, 128>(a, st);
}

}  // namespace la
