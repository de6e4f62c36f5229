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
//   staging), row-major with XOR swizzles, through four stages: a tile is
//   issued three tiles before it is read. The buffer descriptor moves with the
//   tile and its size ends at the sequence end, so rows past the end read as
//   zero. K operands are read with ds_read_b128; the V^T operand with the
//   transposing ds_read_b64_tr_b16 from the row-major V tile. The four K
//   stages fill the first 64 KB of LDS and the four V stages the second; the
//   tile loop is unrolled over the stages, so every operand read is one
//   per-lane address register plus a constant offset (no address arithmetic
//   in the loop).
// * The two waves of a SIMD run one phase apart ("ping-pong"): each wave
//   alternates an MFMA phase (PV of tile k and QK of tile k+1: 32 MFMAs and
//   their 48 operand reads, kept eight reads ahead) with a softmax phase
//   (mask, max, exp, bf16 rounding, row sums of tile k+1), every phase ends at
//   a workgroup barrier, and the other wave of the SIMD is then in the other
//   kind of phase. On gfx950 the VALU work of one wave and the MFMAs of the
//   other do not run concurrently; what the offset buys is that each wave's
//   waits (MFMA results, LDS reads, exp latency) are filled by the other.
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
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace la {
namespace {

constexpr int kCols = 256;    // columns per workgroup
constexpr int kNW = 8;        // waves per workgroup
constexpr int kCB = kCols / kNW / 32;   // 32-column blocks per wave
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

template <typename T, int D, int G>
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
  __shared__ __attribute__((aligned(1024))) char lds[8 * TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lc = lane & 31, hi = lane >> 5;

  const int bid = blockIdx.x;
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
  if (docs_in_lanes) cu_l = cu[min(lane, n_docs)];

  // ---- Q operand (B of S^T = K Q^T): Q[col][16ks + 8hi + i] ----------------
  // Columns past the sequence end load the last token's row (no branch, so
  // the wait for the offsets row does not also wait for Q); every key is
  // masked for them and their outputs are not stored.
  bf16x8 qreg[kCB][KS];
  float qraw[kCB][KS][8];   // unrotated queries (RoPE in the kernel), else unused
  const bool rope_q = a.rope_q != 0;
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) {
    const T* qp = qbase + min(tok[cb], Sq - 1) * a.qs_s + head[cb] * a.qs_h + 8 * hi;
    if (rope_q) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) load8_f32(qp + 16 * ks, qraw[cb][ks]);
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qreg[cb][ks] = load8(qp + 16 * ks);
    }
  }

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
  if (kv_lo > kv_hi) {
    // no key of this shard is visible to any of the tile's rows (ring step):
    // the first step of an accumulation still starts the rows at o = 0,
    // lse = -inf
    if (a.acc_mode == 1) {
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
  if (a.split_tiles > 0) {
    n_split = (n_tiles + a.split_tiles - 1) / a.split_tiles;
    if (sp >= n_split) {
      if (n_split > 1 && hi == 0)
#pragma unroll
        for (int cb = 0; cb < kCB; ++cb)
          if (valid[cb])
            a.lse_part[(((int64_t)sp * a.B + b) * a.Hq + head[cb]) * Sq + tok[cb]] = -INFINITY;
      __builtin_amdgcn_s_waitcnt(0);   // the Q loads already issued
      return;
    }
    kv_lo += sp * a.split_tiles * kKT;
    n_tiles = min(a.split_tiles, n_tiles - sp * a.split_tiles);
  }

  f32x16 acc[DB][kCB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[db][cb][j] = 0.f;
  float m[kCB], l[kCB];
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) {
    m[cb] = -INFINITY;
    l[cb] = 0.f;
  }

  // ---- tile staging: per-lane byte offsets of this wave's 1 KB loads --------
  int koff[NL], voff[NL];
#pragma unroll
  for (int n = 0; n < NL; ++n) {
    const int p = (n * kNW + wave) * 64 + lane;   // LDS chunk written by this lane
    const int row = p / CH, ph = p % CH;
    koff[n] = (int)(row * a.ks_s * (int64_t)sizeof(T) + 8 * k_chunk<CH>(ph, row) * (int)sizeof(T));
    voff[n] = (int)(row * a.vs_s * (int64_t)sizeof(T) + 8 * v_chunk<CH>(ph, row) * (int)sizeof(T));
  }
  auto stage = [&](int kt, char* dst) __attribute__((always_inline)) {
    if constexpr (std::is_same<T, __bf16>::value) {
      const int64_t rows = max(kend - kt, 0);   // rows past the last key read as zero
      const int kb_ = (int)min(rows * a.ks_s * 2, (int64_t)0x7fffffff);
      const int vb_ = (int)min(rows * a.vs_s * 2, (int64_t)0x7fffffff);
      const void* kp = kbase + (int64_t)(kt - k_off) * a.ks_s;
      const void* vp = vbase + (int64_t)(kt - k_off) * a.vs_s;
#pragma unroll
      for (int n = 0; n < NL; ++n) {
        load_lds16(kp, kb_, koff[n], dst + (n * kNW + wave) * 1024);
        load_lds16(vp, vb_, voff[n], dst + 4 * TILE + (n * kNW + wave) * 1024);
      }
    } else {   // fp32 inputs: convert to bf16 on the way into LDS
      for (int p = tid; p < kKT * CH; p += 64 * kNW) {
        const int row = p / CH, ph = p % CH;
        const int j = kt + row;
        bf16x8 kv = zero_bf16x8(), vv = zero_bf16x8();
        if (j < kend) {
          kv = load8(kbase + (int64_t)(j - k_off) * a.ks_s + 8 * k_chunk<CH>(ph, row));
          vv = load8(vbase + (int64_t)(j - k_off) * a.vs_s + 8 * v_chunk<CH>(ph, row));
        }
        *reinterpret_cast<bf16x8*>(dst + p * 16) = kv;
        *reinterpret_cast<bf16x8*>(dst + 4 * TILE + p * 16) = vv;
      }
    }
  };

  // ---- per-lane LDS operand offsets ------------------------------------------
  // K operand: row 32kb + lc, logical chunk 2ks + hi.
  const int k_lane = lc * ROW;
  const int k_x = hi ^ (lc & (CH - 1));              // physical chunk = (2ks) ^ k_x
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

  // ---- ping-pong schedule ------------------------------------------------------
  // Waves w and w + 4 share a SIMD; they form groups A (waves 0-3) and B (4-7).
  // Work of a wave per tile k: QK(k) (MFMA), SM(k) (mask + softmax, VALU),
  // PV(k) (MFMA). Every wave runs QK(0) | SM(0) | X(0) | SM(1) | X(1) | ... |
  // X(n-1), X(k) = PV(k) + QK(k+1); group B runs it one phase behind group A
  // and every phase ends with a workgroup barrier, so in every phase one wave
  // of each SIMD feeds the matrix core while the other runs its softmax on the
  // VALU. K/V: four LDS stages; tile k+3 is issued at the start of iteration k
  // (phase 2k+2, when the stage of tile k-1 is free in both groups) and must
  // have landed at the end of phase 2k+5, before its first read in phase 2k+6.
  const int group = wave >> 2;
  auto stage_ptr = [&](int k) __attribute__((always_inline)) -> char* { return lds + (k & 3) * TILE; };
  // tiles past the last one are issued as loads that read nothing, so every
  // wave has the same number of loads in flight at every wait
  auto issue = [&](int k) __attribute__((always_inline)) { stage(k < n_tiles ? kv_lo + k * kKT : kend, stage_ptr(k)); };
  auto barrier = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(kLgkm0);   // this wave's LDS reads are done
    __builtin_amdgcn_s_barrier();
  };

  f32x16 sc[2];           // S^T of one tile: [32-key block]
  bf16x8 pc[2][2];        // P^T of one tile: [32-key block][16-key half]

  auto qk_tile = [&](const char* lk) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int j = 0; j < 16; ++j) sc[kb][j] = 0.f;
#pragma unroll
      for (int k4 = 0; k4 < KS; k4 += 4) {
        bf16x8 ka[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
          ka[u] = *reinterpret_cast<const bf16x8*>(lk + kb * 32 * ROW + k_lane + 16 * ((2 * (k4 + u)) ^ k_x));
#pragma unroll
        for (int u = 0; u < 4; ++u) sc[kb] = mfma32(ka[u], qreg[0][k4 + u], sc[kb]);
      }
    }
  };
  auto pv_tile = [&](const char* lv) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 va[DB];
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const char* vp = lv + 16 * ks * ROW + v_lane[db];
        const i16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vp));
        const i16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vp + 8 * ROW));
        va[db] = __builtin_shufflevector(__builtin_bit_cast(bf16x4, r0), __builtin_bit_cast(bf16x4, r1),
                                         0, 1, 2, 3, 4, 5, 6, 7);
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db][0] = mfma32(va[db], pc[ks >> 1][ks & 1], acc[db][0]);
    }
  };
  auto sm_tile = [&](int k) __attribute__((always_inline)) {
    const int kt = kv_lo + k * kKT;
    // (keys at or past kend, the end of the keys held, are masked too: a
    // ring step's key shard can end before the rows' positions)
    if (!wave_all_valid || kt + kKT - 1 > w_tmin + qo || kt < w_smax || kt + kKT > kend) {
      const int lo = valid[0] ? st[0] - kt : kKT;
      const int hi_ = valid[0] ? min(tok[0] + qo, kend - 1) - kt : -1;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int kr = kb * 32 + 8 * (j >> 2) + 4 * hi + (j & 3);
          sc[kb][j] = (kr >= lo && kr <= hi_) ? sc[kb][j] : -INFINITY;
        }
    }
    // P^T of the tile against the reference mc (log2 units); returns this
    // lane's sum of the rounded weights
    auto weights = [&](float mc) __attribute__((always_inline)) -> float {
      float rs = 0.f;
      const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int i = 0; i < 8; i += 2) {
            bf16x2 pr;
            pr[0] = to_bf16(fast_exp2(fmaf(sc[kb][8 * h2 + i], a.scale_log2, -mc)));
            pr[1] = to_bf16(fast_exp2(fmaf(sc[kb][8 * h2 + i + 1], a.scale_log2, -mc)));
            pc[kb][h2][i] = pr[0];
            pc[kb][h2][i + 1] = pr[1];
            rs = __builtin_amdgcn_fdot2_f32_bf16(pr, one, rs, false);
          }
      return rs;
    };
    // The reference must move only when a weight would exceed kLazyW. The
    // weights are non-negative, so a lane whose sum is at most kLazyW holds
    // none larger, and the tile max is needed only when some lane's sum is
    // larger (or a column has no reference yet); the reference then moves to
    // the tile max whenever that is higher.
    bool slow = __any(m[0] == -INFINITY);
    float rs = 0.f;
    if (!slow) {
      rs = weights(m[0] * a.scale_log2);
      slow = __any(!(rs <= kLazyW));
    }
    if (slow) {
      float mx = sc[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = fmaxf(mx, sc[kb][j]);
      mx = max_xor32(mx);
      const bool mv = mx > m[0];
      const float al = mv ? fast_exp2((m[0] - mx) * a.scale_log2) : 1.f;   // 0 when m = -inf
      m[0] = mv ? mx : m[0];
      l[0] *= al;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[db][0] *= al;
      rs = weights(m[0] == -INFINITY ? 0.f : m[0] * a.scale_log2);
    }
    l[0] += rs;
  };
  // the MFMA phase runs at raised priority, so the SIMD's arbiter keeps the
  // matrix core fed from it first
  // The refill of tile k+3 and the operand reads of the MFMA phase go through
  // one call whose stage pointers are restrict, so the compiler does not take
  // the refill's LDS-direct loads as writers of what the phase reads (it would
  // otherwise wait for every load in flight before the first read); the
  // vmcnt waits before the barriers order each stage's loads before its reads.
  auto x_phase = [&](char* __restrict__ dst, int kd, const char* __restrict__ lv,
                     const char* __restrict__ lk, int k) __attribute__((always_inline)) {
    if (dst) stage(kd < n_tiles ? kv_lo + kd * kKT : kend, dst);
    __builtin_amdgcn_s_setprio(1);
    // one block of 32 MFMAs and their 48 operand reads (after the last tile
    // the QK of the stage beyond it is computed and dropped): keep eight reads
    // ahead of the MFMAs instead of the one or two the default schedule keeps
    pv_tile(lv);
    qk_tile(lk);
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);   // DS reads
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    __builtin_amdgcn_s_setprio(0);
  };
  // tile k+2 landed: only the loads issued after it (tile k+3) may be pending
  auto landed = [&]() __attribute__((always_inline)) { __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * NL)); };

  issue(0);
  issue(1);
  issue(2);
  if (rope_q) {
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
        r[2 * p] = to_bf16(fmaf(x[2 * p], cv[p], -x[2 * p + 1] * sv[p]));
        r[2 * p + 1] = to_bf16(fmaf(x[2 * p], sv[p], x[2 * p + 1] * cv[p]));
      }
      return r;
    };
    // half-split pairs: elements e0 + 0..3 of x (first half) and y (second
    // half, same positions), rotated into r and t
    auto rotate_half = [&](const float* x, const float* y, int e0, const f32x4& cv, const f32x4& sv,
                           bf16x8& r, bf16x8& t) __attribute__((always_inline)) {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        r[e0 + p] = to_bf16(fmaf(x[e0 + p], cv[p], -y[e0 + p] * sv[p]));
        t[e0 + p] = to_bf16(fmaf(x[e0 + p], sv[p], y[e0 + p] * cv[p]));
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
        *reinterpret_cast<f32x4*>(lds + 3 * TILE + off) = cv;
        *reinterpret_cast<f32x4*>(lds + 7 * TILE + off) = sv;
      }
      __syncthreads();
#pragma unroll
      for (int cb = 0; cb < kCB; ++cb) {
        const int tt = (wave * 32 * kCB + cb * 32 + lc) / G;
        auto tab = [&](int c, int which) __attribute__((always_inline)) {   // 4 pairs from chunk c
          return *reinterpret_cast<const f32x4*>(lds + (which ? 7 : 3) * TILE + tt * ROW +
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
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(4 * NL));   // tile 0 landed
  __builtin_amdgcn_s_barrier();
  if (group == 0) {
    __builtin_amdgcn_s_setprio(1);
    qk_tile(stage_ptr(0));
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * NL));   // tile 1 landed
    barrier();                                       // end of phase 0
    sm_tile(0);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));        // tile 2 landed
    barrier();                                       // end of phase 1
    // unrolled over the four stages so every stage offset is a constant
    auto step = [&](auto U, int k) __attribute__((always_inline)) {
      constexpr int u = decltype(U)::value;
      x_phase(lds + ((u + 3) & 3) * TILE, k + 3, lds + u * TILE, lds + ((u + 1) & 3) * TILE, k);
      barrier();                                     // end of phase 2k+2
      if (k + 1 < n_tiles) sm_tile(k + 1);
      landed();
      barrier();                                     // end of phase 2k+3
    };
    for (int k = 0; k < n_tiles; k += 4) {
      step(std::integral_constant<int, 0>{}, k);
      if (k + 1 >= n_tiles) break;
      step(std::integral_constant<int, 1>{}, k + 1);
      if (k + 2 >= n_tiles) break;
      step(std::integral_constant<int, 2>{}, k + 2);
      if (k + 3 >= n_tiles) break;
      step(std::integral_constant<int, 3>{}, k + 3);
    }
  } else {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * NL));
    barrier();                                       // end of phase 0
    __builtin_amdgcn_s_setprio(1);
    qk_tile(stage_ptr(0));
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    barrier();                                       // end of phase 1
    auto step = [&](auto U, int k) __attribute__((always_inline)) {
      constexpr int u = decltype(U)::value;
      stage(k + 3 < n_tiles ? kv_lo + (k + 3) * kKT : kend, lds + ((u + 3) & 3) * TILE);
      sm_tile(k);
      barrier();                                     // end of phase 2k+2
      x_phase(nullptr, 0, lds + u * TILE, lds + ((u + 1) & 3) * TILE, k);
      landed();
      barrier();                                     // end of phase 2k+3
    };
    for (int k = 0; k < n_tiles; k += 4) {
      step(std::integral_constant<int, 0>{}, k);
      if (k + 1 >= n_tiles) break;
      step(std::integral_constant<int, 1>{}, k + 1);
      if (k + 2 >= n_tiles) break;
      step(std::integral_constant<int, 2>{}, k + 2);
      if (k + 3 >= n_tiles) break;
      step(std::integral_constant<int, 3>{}, k + 3);
    }
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));          // loads past the last tile

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
    lt[cb] = l[cb] + __shfl_xor(l[cb], 32);
    rl[cb] = lt[cb] > 0.f ? __builtin_amdgcn_rcpf(lt[cb]) : 0.f;
  }
  auto quot = [&](float x, int cb) __attribute__((always_inline)) {
    const float q = x * rl[cb];
    return fmaf(fmaf(-q, lt[cb], x), rl[cb], q);
  };
  auto row_lse = [&](int cb) __attribute__((always_inline)) {
    return lt[cb] > 0.f ? m[cb] * a.scale + fast_log2(lt[cb]) * kLn2 : -INFINITY;
  };
  if (a.acc_mode) {
    // ring step: this shard's (o, lse) of every row, written (first step) or
    // merged by log-sum-exp weight into the fp32 accumulators (o_acc, lse_acc);
    // a workgroup owns its rows, so the read-merge-write needs no atomics
#pragma unroll
    for (int cb = 0; cb < kCB; ++cb) {
      if (!valid[cb]) continue;
      float* op = a.o_acc + (((int64_t)b * Sq + tok[cb]) * a.Hq + head[cb]) * D;
      float* lp = a.lse_acc + ((int64_t)b * a.Hq + head[cb]) * Sq + tok[cb];
      const float ln = row_lse(cb);
      float wo = 0.f, wn = 1.f, rw = 1.f, lout = ln;
      if (a.acc_mode == 2) {
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
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int jq = 0; jq < 4; ++jq) {
          f32x4* dst = reinterpret_cast<f32x4*>(op + db * 32 + 8 * jq + 4 * hi);
          f32x4 v = {quot(acc[db][cb][4 * jq], cb), quot(acc[db][cb][4 * jq + 1], cb),
                     quot(acc[db][cb][4 * jq + 2], cb), quot(acc[db][cb][4 * jq + 3], cb)};
          if (a.acc_mode == 2) v = (wo * (*dst) + wn * v) * rw;
          *dst = v;
        }
      __builtin_amdgcn_s_waitcnt(0);   // both halves of the row have read lse before it changes
      __builtin_amdgcn_wave_barrier();
      if (hi == 0) *lp = lout;
    }
    return;
  }
  if (n_split > 1) {
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
          const f32x4 v = {quot(acc[db][cb][4 * jq], cb), quot(acc[db][cb][4 * jq + 1], cb),
                           quot(acc[db][cb][4 * jq + 2], cb), quot(acc[db][cb][4 * jq + 3], cb)};
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
    static_assert(kCB == 1, "one 32-column block per wave");
    __syncthreads();
    char* ow = lds + wave * 32 * ROW;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = to_bf16(quot(acc[db][0][4 * jq + e], 0));
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
          store4(op + d, quot(acc[db][cb][4 * jq], cb), quot(acc[db][cb][4 * jq + 1], cb),
                 quot(acc[db][cb][4 * jq + 2], cb), quot(acc[db][cb][4 * jq + 3], cb));
        }
    }
  }
#pragma unroll
  for (int cb = 0; cb < kCB; ++cb) {
    if (hi != 0 || !valid[cb]) continue;
    if (a.lse) a.lse[((int64_t)b * a.Hq + head[cb]) * Sq + tok[cb]] = row_lse(cb);
    if (a.split_tiles > 0) a.lse_part[((int64_t)b * a.Hq + head[cb]) * Sq + tok[cb]] = INFINITY;
  }
}

template <typename T, int D, int G>
hipError_t launch_t(const PrefillArgs& a, hipStream_t st) {
  const unsigned grid = (unsigned)a.B * a.Hkv * a.n_qtiles;
  const unsigned splits = a.split_tiles > 0 ? (unsigned)a.max_splits : 1u;
  hipLaunchKernelGGL((prefill_kernel<T, D, G>), dim3(grid, splits), dim3(64 * kNW), 0, st, a);
  return hipGetLastError();
}

// Merge of split partials: one group of D/4 lanes per (sequence, query row,
// head), 4 values per lane. Rows marked +inf in slot 0 were written whole by
// the prefill kernel; the others take M = max_s lse_s, w_s = exp(lse_s - M),
// o = sum_s w_s o_s / sum_s w_s, lse = M + ln(sum_s w_s) over the slots with
// lse_s > -inf.
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
  for (int s = 0; s < a.max_splits; ++s) M = fmaxf(M, lp[s * slot_stride]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float W = 0.f;
  if (M > -INFINITY) {
    for (int s = 0; s < a.max_splits; ++s) {
      const float ls = lp[s * slot_stride];
      if (!(ls > -INFINITY)) continue;
      const float w = __expf(ls - M);
      const f32x4 o = *reinterpret_cast<const f32x4*>(
          a.o_part + ((((int64_t)s * a.B + b) * a.Sq + tok) * a.Hq + h) * D + 4 * lane);
      acc += w * o;
      W += w;
    }
  }
  const float rw = W > 0.f ? 1.f / W : 0.f;
  T* op = static_cast<T*>(a.o) + b * a.os_b + tok * a.os_s + h * a.os_h + 4 * lane;
  store4(op, acc[0] * rw, acc[1] * rw, acc[2] * rw, acc[3] * rw);
  if (a.lse && lane == 0) a.lse[((int64_t)b * a.Hq + h) * a.Sq + tok] = W > 0.f ? M + __logf(W) : -INFINITY;
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

hipError_t launch_prefill(const PrefillArgs& a, int D, int G, int dt, hipStream_t st) {
  if (dt == 0) return D == 64 ? launch_g<__bf16, 64>(a, G, st) : launch_g<__bf16, 128>(a, G, st);
  return D == 64 ? launch_g<float, 64>(a, G, st) : launch_g<float, 128>(a, G, st);
}

hipError_t launch_prefill_merge(const PrefillArgs& a, int D, int dt, hipStream_t st) {
  if (dt == 0) return D == 64 ? launch_merge_t<__bf16, 64>(a, st) : launch_merge_t<__bf16, 128>(a, st);
  return D == 64 ? launch_merge_t<float, 64>(a, st) : launch_merge_t<float, 128>(a, st);
}

}  // namespace la
