// Gradient pass of grouped-query causal attention with the cross-document
// mask: given the output gradient dO, the gradients of the loss with respect
// to the rotated queries and keys and to the values.
//
// What is computed (the forward is "The Llama 3 Herd of Models", "A
// Deliberately Standard Dense Transformer": GQA, causal and cross-document
// mask; the gradients are its plain derivatives). With P_ij the softmax
// weights of the forward (recomputed here from the saved log-sum-exp: P_ij =
// exp(s_ij * scale - lse_i) on visible pairs, 0 elsewhere) and
// delta_i = dO_i . O_i:
//   dv_j = sum_i P_ij dO_i
//   dS_ij = P_ij (dO_i . v_j - delta_i)
//   dq_i = scale sum_j dS_ij k_j,   dk_j = scale sum_i dS_ij q_i
// where the sums over i for a key also run over the g query heads that share
// its KV head.
//
// How (gfx950), on the caller's stream: the dq kernel (which also writes
// delta), then the dk/dv kernel, then, with a workspace, the merge of cut
// query ranges:
// * dk/dv, key-stationary: one workgroup = (sequence, KV head, 128 keys),
//   eight waves, two per SIMD sharing a group of 32 keys. The (token, query
//   head) columns that can see the keys go by in blocks of 64 staged in LDS
//   (Q, dO, lse, delta; two stages, loaded straight from HBM with
//   buffer_load ... lds). Per block, with the key on the lane: one wave of the
//   pair forms S = Q K^T, P, and dV^T += dO^T P; the other forms dP = dO V^T
//   and, with the first wave's P passed through LDS, dS = P (dP - delta) and
//   dK^T += Q^T dS (32x32x16 bf16 MFMA; dO^T and Q^T read from the same LDS
//   rows with the transposing ds_read_b64_tr_b16). Each wave thus holds one
//   operand row (K or V) and one accumulator (dV or dK), which fits two waves
//   per SIMD, so one wave's waits are filled by the other's work. With a
//   workspace, a long query range is cut into pieces (one workgroup each)
//   whose fp32 partials a merge launch sums in a fixed order.
// * dq (first), query-stationary (the forward's shape): one workgroup = (sequence,
//   KV head, 256 / g tokens x g heads), eight waves of 32 columns; Q and dO
//   rows in registers, key tiles of 64 K and V rows staged in LDS (two
//   stages); S^T = K Q^T and dP^T = V dO^T (lane = column), then
//   dQ^T += K^T dS^T with K^T read transposed from the K tile. Each column's
//   delta = dO . O is formed here from the dO rows in registers and written
//   for the dk/dv kernel.
// dq is therefore formed without atomics and every gradient is written once;
// the cost is recomputing S and dP in the dq kernel (7 products per visible
// pair instead of 5).
// P and dS are rounded to bf16 for the products that use them, fp32
// accumulation throughout; masks are evaluated only where a block straddles
// a causal or document edge.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace la {
namespace {

constexpr int kNC = 64;                  // columns per block (dk/dv kernel)
constexpr int kKvGroups = 4;             // 32-key groups per workgroup (dk/dv kernel)
constexpr int kKvWaves = 2 * kKvGroups;  // two waves per group
constexpr int kKvKeys = 32 * kKvGroups;  // keys per workgroup (dk/dv kernel)
constexpr int kQWaves = 8;
constexpr int kQCols = 32 * kQWaves;     // columns per workgroup (dq kernel)
constexpr int kKT = 64;                  // keys per tile (dq kernel)
// key blocks with more query blocks than this are split (when a workspace
// is given): below it the split's extra traffic and merge outweigh the
// balance it buys (the 8B backward measured 128-256 alike, 1.5-2% faster
// than 48, 8% faster than no split)
constexpr int kSplitMin = 128;
static_assert(kKvKeys == kBwdKeysPerBlock, "host and kernel disagree on the key block");

__device__ __forceinline__ void wait_all() { __builtin_amdgcn_s_waitcnt(0); }

// bf16 rows of 8 values from 8 fp32 (round to nearest even)
__device__ __forceinline__ bf16x8 pack8(const f32x16& x, int off) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = to_bf16(x[off + i]);
  return r;
}

// Physical 16-byte chunk of logical chunk c in row r of a tile read both as
// rows (ds_read_b128: 16 consecutive rows of one chunk per 16 lanes) and
// transposed (ds_read_b64_tr_b16: 4 consecutive rows x 4 consecutive chunks
// per 32 lanes). For D = 128 the row term is the 4-bit transpose of r & 15:
// any 16 consecutive rows get 16 distinct chunks and the 4 rows of an aligned
// group land 64 bytes apart, so neither read conflicts (the transposing
// reads' swizzle 4 (r & 3) alone gives the row reads a 4-way conflict). An
// XOR with a row-only term is its own inverse, which the loaders rely on.
template <int CH>
__device__ __forceinline__ int t_chunk(int c, int r) {
  return CH == 16 ? c ^ ((4 * (r & 3)) | ((r >> 2) & 3)) : v_chunk<CH>(c, r);
}

// A operand of a product whose M is head_dim and K 16 rows of a row-major
// tile: rows 4hi + 0..3 (first read) and 8 + 4hi + 0..3 (second) of the 16
// rows at p, for lane half hi; o1, o2 are the lane's offsets (tr_lane_off).
__device__ __forceinline__ bf16x8 read_tr_rows(const char* p, int o1, int o2) {
  const i16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + o1));
  const i16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + o2));
  return __builtin_shufflevector(__builtin_bit_cast(bf16x4, r0), __builtin_bit_cast(bf16x4, r1),
                                 0, 1, 2, 3, 4, 5, 6, 7);
}

// Per-lane byte offset of a transposing read within a 16-row group of a
// row-major tile stored with t_chunk: the 16-lane group g = lane / 16 covers
// d = 32db + 16(g & 1) + (lane & 15); its input lane L = lane & 15 addresses
// row r8 + 4hi + L/4 (r8 = 0 or 8) at d0 = 32db + 16(g & 1) + 4(L % 4).
template <int D>
__device__ __forceinline__ int tr_lane_off(int lane, int db, int r8) {
  constexpr int CH = D / 8, ROW = 2 * D;
  const int L16 = lane & 15, hi = lane >> 5;
  const int row = r8 + 4 * hi + (L16 >> 2);
  return row * ROW + 16 * t_chunk<CH>(4 * db + 2 * ((lane >> 4) & 1) + ((L16 >> 1) & 1), row) + 8 * (L16 & 1);
}

// ---------------------------------------------------------------- dk, dv

template <int D, int G>
__global__ __launch_bounds__(64 * kKvWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
void dkdv_kernel(BwdArgs a) {
  constexpr int KS = D / 16, DB = D / 32, CH = D / 8, ROW = 2 * D;
  constexpr int TB = kNC / G;                 // tokens per column block
  constexpr int QT = kNC * ROW;               // bytes of a Q or dO block
  constexpr int STAGE = 2 * QT + 2 * kNC * 4;
  constexpr int RPI = 64 / CH;                // rows per 1 KB load
  constexpr int NLW = kNC / RPI / kKvWaves;   // 1 KB loads per wave per Q or dO block
  constexpr int NCB = kNC / 32;               // 32-column blocks per block
  constexpr int PB = NCB * 16 * 64 * 4;       // P of one key group: [cb][i/4][lane] f32x4
  static_assert(NLW >= 1 && NLW * RPI * kKvWaves == kNC, "block loads must cover the rows");
  __shared__ __attribute__((aligned(1024))) char lds[2 * STAGE + kKvGroups * PB];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lc = lane & 31, hi = lane >> 5;
  // waves w and w + 4 (one SIMD) share a group of 32 keys: role 0 forms S and
  // P and accumulates dV, role 1 forms dP and, from role 0's P, dS, and
  // accumulates dK
  const int grp = wave & (kKvGroups - 1);
  const int role = wave / kKvGroups;

  const int bid = blockIdx.x;
  const int kvh = bid % a.Hkv;
  const int r = bid / a.Hkv;
  const int b = r % a.B;
  const int k0 = (r / a.B) * kKvKeys;          // key blocks in order: the first sees the most queries
  const int S = a.S;
  const int kw0 = k0 + grp * 32;
  const int j = kw0 + lc;                     // this lane's key
  const int32_t* cu = a.cu_docs ? a.cu_docs + (int64_t)b * (a.n_docs + 1) : nullptr;

  // document ends: of this lane's key, of the group's first and last keys, of
  // the block's last key (queries at or past it see none of the block's keys)
  int dend = S, w_dend_first = S, w_dend_last = S, q_end = S;
  if (cu) {
    dend = doc_end(cu, a.n_docs, min(j, S - 1));
    w_dend_first = doc_end(cu, a.n_docs, min(kw0, S - 1));
    w_dend_last = doc_end(cu, a.n_docs, min(kw0 + 31, S - 1));
    q_end = doc_end(cu, a.n_docs, min(k0 + kKvKeys, S) - 1);
  }
  w_dend_first = __builtin_amdgcn_readfirstlane(w_dend_first);
  w_dend_last = __builtin_amdgcn_readfirstlane(w_dend_last);
  q_end = __builtin_amdgcn_readfirstlane(q_end);
  // the lane's key is visible to the tokens t with 0 <= t - j < lim
  const unsigned lim = j < S ? (unsigned)(dend - j) : 0u;

  // the key's K row (role 0) or V row (role 1) as B operand: [j][16ks + 8hi + i]
  bf16x8 kv[KS];
  {
    const int jc = min(j, S - 1);
    const __bf16* p = role == 0
        ? static_cast<const __bf16*>(a.k) + b * a.ks_b + jc * a.ks_s + kvh * a.ks_h + 8 * hi
        : static_cast<const __bf16*>(a.v) + b * a.vs_b + jc * a.vs_s + kvh * a.vs_h + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kv[ks] = load8(p + 16 * ks);
  }

  // query columns: tokens k0 .. q_end - 1, column c of a block = (token
  // tb0 + c / G, head kvh G + c % G); a long range is cut into pieces
  // (blockIdx.y), each summing over its share of the blocks
  const int n_all = (q_end - k0 + TB - 1) / TB;
  const bool split = a.dkv_part != nullptr && n_all > kSplitMin;
  const int piece = blockIdx.y;
  if (!split && piece > 0) return;
  const int per = split ? (n_all + kBwdPieces - 1) / kBwdPieces : n_all;
  const int blk0 = piece * per;
  const int n_blk = max(min(n_all - blk0, per), 0);
  const __bf16* qb = static_cast<const __bf16*>(a.q) + b * a.qs_b + (int64_t)kvh * G * a.qs_h;
  const __bf16* gb = static_cast<const __bf16*>(a.dout) + b * a.gs_b + (int64_t)kvh * G * a.gs_h;
  const float* lb = a.lse + ((int64_t)b * a.Hq + kvh * G) * S;
  const float* eb = a.delta + ((int64_t)b * a.Hq + kvh * G) * S;
  int qoff[NLW], goff[NLW];
#pragma unroll
  for (int p = 0; p < NLW; ++p) {
    const int row = (wave * NLW + p) * RPI + lane / CH;
    const int lch = t_chunk<CH>(lane % CH, row);
    qoff[p] = (int)(((row / G) * a.qs_s + (row % G) * a.qs_h) * 2 + 16 * lch);
    goff[p] = (int)(((row / G) * a.gs_s + (row % G) * a.gs_h) * 2 + 16 * lch);
  }
  const int loff = ((lane % G) * S + lane / G) * 4;
  // block m (of the key block's range) into stage (m - blk0) & 1
  // block m of the key block's range into the stage at dst
  auto issue = [&](int m, char* dst) __attribute__((always_inline)) {
    const int tb0 = k0 + m * TB;
    const int rows = min(S - tb0, TB);        // >= 1: tb0 < q_end <= S
    // byte ranges end at the last valid token's last head row: rows past the
    // sequence end read as zero
    const int qbytes = (int)(((rows - 1) * a.qs_s + (G - 1) * a.qs_h + D) * 2);
    const int gbytes = (int)(((rows - 1) * a.gs_s + (G - 1) * a.gs_h + D) * 2);
#pragma unroll
    for (int p = 0; p < NLW; ++p) {
      load_lds16(qb + tb0 * a.qs_s, qbytes, qoff[p], dst + (wave * NLW + p) * 1024);
      load_lds16(gb + tb0 * a.gs_s, gbytes, goff[p], dst + QT + (wave * NLW + p) * 1024);
    }
    const int lbytes = ((G - 1) * S + (S - tb0)) * 4;
    if (wave == 0) load_lds4(lb + tb0, lbytes, loff, dst + 2 * QT);
    if (wave == 1) load_lds4(eb + tb0, lbytes, loff, dst + 2 * QT + kNC * 4);
  };

  int tr1[DB], tr2[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    tr1[db] = tr_lane_off<D>(lane, db, 0);
    tr2[db] = tr_lane_off<D>(lane, db, 8);
  }
  char* pbuf = lds + 2 * STAGE + grp * PB;    // the group's P, role 0 -> role 1

  f32x16 acc[DB];                             // dV^T (role 0) or dK^T (role 1)
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;

  // Block n of the piece from stage stg = n % 2; the loop below is unrolled
  // over the two stages so that every LDS offset is a constant.
  auto block = [&](int n, auto STG) __attribute__((always_inline)) {
    constexpr int stg = decltype(STG)::value;
    wait_all();
    __syncthreads();
    if (n + 1 < n_blk) issue(blk0 + n + 1, lds + (1 - stg) * STAGE);
    const char* st = lds + stg * STAGE;
    const int tb0 = k0 + (blk0 + n) * TB;
    // nothing of this block visible to the group's keys: both roles skip the
    // work (never the barriers)
    const bool skip = kw0 > tb0 + TB - 1 || tb0 >= w_dend_last;
    // every pair visible: all keys at or before every token, all tokens
    // before the first key's document end (no mask needed)
    const bool full = kw0 + 31 <= tb0 && tb0 + TB <= w_dend_first;
    // S = Q K^T (role 0) or dP = dO V^T (role 1), lane = key j; element i of
    // column block cb is column 32cb + 8(i/4) + 4hi + i%4
    f32x16 sd[NCB];
    if (!skip) {
      const char* src = st + role * QT;
      // role 1 starts dP from the columns' staged -delta, so its MFMAs yield
      // dP - delta directly; role 0 starts S from 0
      auto products = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int ch = 16 * t_chunk<CH>(2 * ks + hi, lc);
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb)
            sd[cb] = mfma32(*reinterpret_cast<const bf16x8*>(src + (32 * cb + lc) * ROW + ch), kv[ks], sd[cb]);
        }
      };
      if (role == 0) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
          for (int i = 0; i < 16; ++i) sd[cb][i] = 0.f;
        products();
      } else {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int c0 = 32 * cb + 8 * q4 + 4 * hi;
            const f32x4 e4 = *reinterpret_cast<const f32x4*>(st + 2 * QT + kNC * 4 + 4 * c0);
#pragma unroll
            for (int u = 0; u < 4; ++u) sd[cb][4 * q4 + u] = e4[u];
          }
        products();
      }
      if (role == 0) {
        // P = exp(s scale - lse) on visible pairs, to LDS for role 1
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int c0 = 32 * cb + 8 * q4 + 4 * hi;
            const f32x4 l4 = *reinterpret_cast<const f32x4*>(st + 2 * QT + 4 * c0);
#pragma unroll
            for (int u = 0; u < 4; ++u)
              sd[cb][4 * q4 + u] = fast_exp2(fmaf(sd[cb][4 * q4 + u], a.scale_log2, -l4[u] * kLog2e));
          }
        if (!full) {   // only blocks on a causal or document edge
#pragma unroll
          for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int t = tb0 + (32 * cb + 8 * (i >> 2) + 4 * hi + (i & 3)) / G;
              sd[cb][i] = (unsigned)(t - j) < lim ? sd[cb][i] : 0.f;
            }
        }
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const f32x4 pv = {sd[cb][4 * q4], sd[cb][4 * q4 + 1], sd[cb][4 * q4 + 2], sd[cb][4 * q4 + 3]};
            *reinterpret_cast<f32x4*>(pbuf + ((cb * 4 + q4) * 64 + lane) * 16) = pv;
          }
      }
    }
    __syncthreads();   // role 0's P is in LDS
    if (!skip) {
      if (role == 1) {
        // dS = P (dP - delta), sd holding dP - delta
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const f32x4 pv = *reinterpret_cast<const f32x4*>(pbuf + ((cb * 4 + q4) * 64 + lane) * 16);
#pragma unroll
            for (int u = 0; u < 4; ++u) sd[cb][4 * q4 + u] = pv[u] * sd[cb][4 * q4 + u];
          }
      }
      // dV^T += dO^T P (role 0) or dK^T += Q^T dS (role 1), the A operand read
      // transposed from the other tile
      const char* tsrc = st + (1 - role) * QT;
#pragma unroll
      for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const bf16x8 x = pack8(sd[cb], 8 * h2);
          const int roff = 16 * (2 * cb + h2) * ROW;
#pragma unroll
          for (int db = 0; db < DB; ++db) acc[db] = mfma32(read_tr_rows(tsrc + roff, tr1[db], tr2[db]), x, acc[db]);
        }
    }
  };
  if (n_blk > 0) issue(blk0, lds);
  for (int n = 0; n < n_blk; n += 2) {
    block(n, std::integral_constant<int, 0>{});
    if (n + 1 < n_blk) block(n + 1, std::integral_constant<int, 1>{});
  }

  // lane = key j, element i of block db is d = 32db + 8(i/4) + 4hi + i%4;
  // role 0 holds dv, role 1 dk (times the scale)
  const float f = role == 0 ? 1.f : a.scale;
  if (split && j < S) {
    float* part = a.dkv_part + ((((int64_t)piece * a.B + b) * S + j) * a.Hkv + kvh) * 2 * D + (role == 0 ? D : 0);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        store4(part + 32 * db + 8 * q4 + 4 * hi, f * acc[db][4 * q4], f * acc[db][4 * q4 + 1],
               f * acc[db][4 * q4 + 2], f * acc[db][4 * q4 + 3]);
  } else if (j < S) {
    __bf16* out = role == 0 ? static_cast<__bf16*>(a.dv) + b * a.dvs_b + j * a.dvs_s + kvh * a.dvs_h
                            : static_cast<__bf16*>(a.dk) + b * a.dks_b + j * a.dks_s + kvh * a.dks_h;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        store4(out + 32 * db + 8 * q4 + 4 * hi, f * acc[db][4 * q4], f * acc[db][4 * q4 + 1],
               f * acc[db][4 * q4 + 2], f * acc[db][4 * q4 + 3]);
  }
}

// ---------------------------------------------------------------- dq

template <int D, int G>
__global__ __launch_bounds__(64 * kQWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
void dq_kernel(BwdArgs a, int n_qtiles) {
  constexpr int KS = D / 16, DB = D / 32, CH = D / 8, ROW = 2 * D;
  constexpr int TQ = kQCols / G;
  constexpr int TILE = kKT * ROW;
  constexpr int RPI = 64 / CH;
  constexpr int NLW = kKT / RPI / kQWaves;    // 1 KB loads per wave per K or V tile
  static_assert(NLW >= 1 && NLW * RPI * kQWaves == kKT, "tile loads must cover the rows");
  // stage s: K at 2s TILE, V at (2s + 1) TILE
  __shared__ __attribute__((aligned(1024))) char lds[4 * TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lc = lane & 31, hi = lane >> 5;

  const int bid = blockIdx.x;
  const int kvh = bid % a.Hkv;
  const int r = bid / a.Hkv;
  const int b = r % a.B;
  const int t0 = (n_qtiles - 1 - r / a.B) * TQ;   // longest key ranges first
  const int S = a.S;
  const int32_t* cu = a.cu_docs ? a.cu_docs + (int64_t)b * (a.n_docs + 1) : nullptr;

  // this lane's column
  const int col = wave * 32 + lc;
  const int t = t0 + col / G;
  const int head = kvh * G + col % G;
  const bool valid = t < S;
  const int tc = valid ? t : S - 1;
  bf16x8 qreg[KS], greg[KS];
  {
    const __bf16* qp = static_cast<const __bf16*>(a.q) + b * a.qs_b + tc * a.qs_s + head * a.qs_h + 8 * hi;
    const __bf16* gp = static_cast<const __bf16*>(a.dout) + b * a.gs_b + tc * a.gs_s + head * a.gs_h + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qreg[ks] = load8(qp + 16 * ks);
      greg[ks] = load8(gp + 16 * ks);
    }
  }
  const int64_t li = ((int64_t)b * a.Hq + head) * S + tc;
  const float lse2 = a.lse[li] * kLog2e;
  // delta of the column, dO . O: this lane's half of the row (the d of its
  // operand registers) plus the other half from lane l ^ 32; written negated
  // for the dk/dv kernel, which runs after this one and starts its dP
  // accumulation from it
  float dlt = 0.f;
  {
    const __bf16* op = static_cast<const __bf16*>(a.o) + b * a.os_b + tc * a.os_s + head * a.os_h + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      float x[8];
      load8_f32(op + 16 * ks, x);
#pragma unroll
      for (int i = 0; i < 8; ++i) dlt = fmaf(x[i], (float)greg[ks][i], dlt);
    }
    const auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(dlt), __float_as_uint(dlt), false, false);
    dlt = __uint_as_float(pr[0]) + __uint_as_float(pr[1]);
    if (valid && hi == 0) a.delta[li] = -dlt;
  }
  const int dstart = cu ? doc_start(cu, a.n_docs, tc) : 0;
  // keys dstart .. t are visible: 0 <= key - dstart < lim
  const unsigned lim = valid ? (unsigned)(t - dstart + 1) : 0u;

  // the workgroup's keys and the wave's bounds
  const int t_last = min(t0 + TQ, S) - 1;
  int kv_lo = 0, w_smin = 0, w_smax = 0;
  const int w_tmin = min(t0 + (wave * 32) / G, S - 1);
  const int w_tmax_raw = t0 + (wave * 32 + 31) / G;
  const int w_tmax = min(w_tmax_raw, S - 1);
  if (cu) {
    kv_lo = doc_start(cu, a.n_docs, t0);
    w_smin = doc_start(cu, a.n_docs, w_tmin);
    w_smax = doc_start(cu, a.n_docs, w_tmax);
  }
  kv_lo = __builtin_amdgcn_readfirstlane(kv_lo);
  w_smin = __builtin_amdgcn_readfirstlane(w_smin);
  w_smax = __builtin_amdgcn_readfirstlane(w_smax);
  const bool wave_all_valid = w_tmax_raw < S;
  const int n_tiles = (t_last - kv_lo + kKT) / kKT;

  const __bf16* kb_ = static_cast<const __bf16*>(a.k) + b * a.ks_b + kvh * a.ks_h;
  const __bf16* vb_ = static_cast<const __bf16*>(a.v) + b * a.vs_b + kvh * a.vs_h;
  int koff[NLW], voff[NLW];
#pragma unroll
  for (int p = 0; p < NLW; ++p) {
    const int row = (wave * NLW + p) * RPI + lane / CH;
    koff[p] = (int)(row * a.ks_s * 2 + 16 * t_chunk<CH>(lane % CH, row));
    voff[p] = (int)(row * a.vs_s * 2 + 16 * k_chunk<CH>(lane % CH, row));
  }
  // tile n's K and V into the stage at dst
  auto issue = [&](int n, char* dst) __attribute__((always_inline)) {
    const int kt = kv_lo + n * kKT;
    const int rows = min(S - kt, kKT);         // >= 1: kt <= t_last < S
    const int kbytes = (int)(((rows - 1) * a.ks_s + D) * 2);
    const int vbytes = (int)(((rows - 1) * a.vs_s + D) * 2);
#pragma unroll
    for (int p = 0; p < NLW; ++p) {
      load_lds16(kb_ + (int64_t)kt * a.ks_s, kbytes, koff[p], dst + (wave * NLW + p) * 1024);
      load_lds16(vb_ + (int64_t)kt * a.vs_s, vbytes, voff[p], dst + TILE + (wave * NLW + p) * 1024);
    }
  };

  int tr1[DB], tr2[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    tr1[db] = tr_lane_off<D>(lane, db, 0);
    tr2[db] = tr_lane_off<D>(lane, db, 8);
  }

  f32x16 dq[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dq[db][i] = 0.f;

  // Tile n from stage stg = n % 2; the loop below is unrolled over the two
  // stages so that every LDS operand offset is a constant (with a run-time
  // stage each read's address took VALU adds).
  auto tile = [&](int n, auto STG) __attribute__((always_inline)) {
    constexpr int stg = decltype(STG)::value;
    wait_all();
    __syncthreads();
    if (n + 1 < n_tiles) issue(n + 1, lds + (1 - stg) * 2 * TILE);
    const char* lk = lds + stg * 2 * TILE;
    const char* lv = lk + TILE;
    const int kt = kv_lo + n * kKT;
    if (kt > w_tmax || kt + kKT - 1 < w_smin) return;   // no key of the tile visible to the wave
    const bool full = wave_all_valid && kt + kKT - 1 <= w_tmin && kt >= w_smax;

    f32x16 s[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        s[kb][i] = 0.f;
        dp[kb][i] = 0.f;
      }
      const int arow = (32 * kb + lc) * ROW;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(lk + arow + 16 * t_chunk<CH>(2 * ks + hi, lc));
        const bf16x8 va = *reinterpret_cast<const bf16x8*>(lv + arow + 16 * k_chunk<CH>(2 * ks + hi, lc));
        s[kb] = mfma32(ka, qreg[ks], s[kb]);
        dp[kb] = mfma32(va, greg[ks], dp[kb]);
      }
    }
    // lane = column; element i of block kb is key kt + 32kb + 8(i/4) + 4hi + i%4
    bf16x8 sb[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = fast_exp2(fmaf(s[kb][i], a.scale_log2, -lse2));
    }
    if (!full) {   // only tiles on a causal or document edge
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kt + 32 * kb + 8 * (i >> 2) + 4 * hi + (i & 3);
          s[kb][i] = (unsigned)(key - dstart) < lim ? s[kb][i] : 0.f;
        }
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 ds;
#pragma unroll
      for (int i = 0; i < 16; ++i) ds[i] = s[kb][i] * (dp[kb][i] - dlt);
      sb[kb][0] = pack8(ds, 0);
      sb[kb][1] = pack8(ds, 8);
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int db = 0; db < DB; ++db)
        dq[db] = mfma32(read_tr_rows(lk + 16 * ks * ROW, tr1[db], tr2[db]), sb[ks >> 1][ks & 1], dq[db]);
  };
  issue(0, lds);
  for (int n = 0; n < n_tiles; n += 2) {
    tile(n, std::integral_constant<int, 0>{});
    if (n + 1 < n_tiles) tile(n + 1, std::integral_constant<int, 1>{});
  }

  // lane = column, element i of block db is d = 32db + 8(i/4) + 4hi + i%4
  if (valid) {
    __bf16* qd = static_cast<__bf16*>(a.dq) + b * a.dqs_b + t * a.dqs_s + head * a.dqs_h;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        store4(qd + 32 * db + 8 * q4 + 4 * hi, a.scale * dq[db][4 * q4], a.scale * dq[db][4 * q4 + 1],
               a.scale * dq[db][4 * q4 + 2], a.scale * dq[db][4 * q4 + 3]);
  }
}

// Sum of the pieces' partial dk, dv (in piece order) for the key blocks the
// dk/dv kernel split, as bf16; one thread per 8 values of a key's row.
template <int D, int G>
__global__ __launch_bounds__(256) void dkdv_merge_kernel(BwdArgs a) {
  constexpr int CH = D / 8;
  constexpr int TB = kNC / G;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;   // over (b, j, kvh, chunk of 2D)
  const int c = (int)(idx % (2 * CH));
  const int64_t r = idx / (2 * CH);
  const int kvh = (int)(r % a.Hkv);
  const int64_t bj = r / a.Hkv;
  const int j = (int)(bj % a.S);
  const int b = (int)(bj / a.S);
  if (b >= a.B) return;
  const int S = a.S;
  const int k0 = j / kKvKeys * kKvKeys;
  int q_end = S;
  if (a.cu_docs) q_end = doc_end(a.cu_docs + (int64_t)b * (a.n_docs + 1), a.n_docs, min(k0 + kKvKeys, S) - 1);
  if ((q_end - k0 + TB - 1) / TB <= kSplitMin) return;     // written directly by the dk/dv kernel
  float x[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const int64_t slot = (int64_t)a.B * S * a.Hkv * 2 * D;
  const float* p = a.dkv_part + (((int64_t)b * S + j) * a.Hkv + kvh) * 2 * D + 8 * c;
#pragma unroll
  for (int pc = 0; pc < kBwdPieces; ++pc) {
    float y[8];
    load8_f32(p + pc * slot, y);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] += y[i];
  }
  __bf16* dst = c < CH ? static_cast<__bf16*>(a.dk) + b * a.dks_b + (int64_t)j * a.dks_s + kvh * a.dks_h + 8 * c
                       : static_cast<__bf16*>(a.dv) + b * a.dvs_b + (int64_t)j * a.dvs_s + kvh * a.dvs_h + 8 * (c - CH);
  store4(dst, x[0], x[1], x[2], x[3]);
  store4(dst + 4, x[4], x[5], x[6], x[7]);
}

template <int D, int G>
hipError_t launch_dg(const BwdArgs& a, hipStream_t st) {
  // dq first: it also writes delta, which the dk/dv kernel reads
  {
    const int tq = kQCols / G;
    const int nqt = (a.S + tq - 1) / tq;
    hipLaunchKernelGGL((dq_kernel<D, G>), dim3(a.B * a.Hkv * nqt), dim3(64 * kQWaves), 0, st, a, nqt);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    const int nkb = (a.S + kKvKeys - 1) / kKvKeys;
    const int pieces = a.dkv_part ? kBwdPieces : 1;
    hipLaunchKernelGGL((dkdv_kernel<D, G>), dim3(a.B * a.Hkv * nkb, pieces), dim3(64 * kKvWaves), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.dkv_part) {
      const int64_t threads = (int64_t)a.B * a.S * a.Hkv * 2 * (D / 8);
      hipLaunchKernelGGL((dkdv_merge_kernel<D, G>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st, a);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

template <int D>
hipError_t launch_d(const BwdArgs& a, int G, hipStream_t st) {
  switch (G) {
    case 1: return launch_dg<D, 1>(a, st);
    case 2: return launch_dg<D, 2>(a, st);
    case 4: return launch_dg<D, 4>(a, st);
    case 8: return launch_dg<D, 8>(a, st);
    case 16: return launch_dg<D, 16>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_backward(const BwdArgs& a, int D, int G, hipStream_t st) {
  if (D == 128) return launch_d<128>(a, G, st);
  if (D == 64) return launch_d<64>(a, G, st);
  return hipErrorInvalidValue;
}

}  // namespace la
