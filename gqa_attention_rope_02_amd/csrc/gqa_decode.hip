// Split-KV decode over a KV cache and the log-sum-exp merge of its partials.
//
// What is computed: one new token per sequence attends, with each of its Hq
// query heads, to every cached token of the KV head its group shares ("How
// Meta's Llama 3.1 405B Architecture Actually Works", GQA paragraph: grouping
// query heads onto one key/value head shrinks the cache read while decoding).
// Partial results over runs of consecutive cache slots are merged afterwards
// by O = sum_s w_s o_s / sum_s w_s, w_s = exp(lse_s - max lse).
//
// How (gfx950): the step is bound by the HBM read of the cache (16 FLOP per
// byte at 16 query heads per KV head), so the kernel exists to keep enough
// cache bytes in flight, to read each byte once and to keep every wave busy to
// the end:
// * the cache of all (sequence, KV head) pairs forms one stream of 16-key
//   tiles, cut into splits of kv_chunk slots; every wave of a persistent grid
//   (one workgroup of four waves per CU) takes the splits that start in its
//   equal slice of the tile stream, so waves end within a split of each other;
// * consecutive splits of one (sequence, KV head) taken by one wave form a run
//   with one online-softmax state; the run's partial goes to the slot of its
//   first split and the other slots of the run get lse = -inf;
// * each wave streams its tiles HBM -> LDS directly (buffer_load_dwordx4 ...
//   lds) through its own four-stage ring, three tiles of K and V in flight, so
//   waves never wait on each other; a buffer descriptor ends at the split's
//   last valid row, so rows past it read as zero, and the stream continues
//   across splits and runs, so it never drains between them;
// * a paged cache (a pool of pages of 2^k slots and a block table per
//   sequence) only changes a tile's address: its page comes from the table,
//   read one tile ahead of the tile's issue;
// * the g query heads of the group are the 16 columns of the MFMA tiles:
//   S^T = K Q^T on the 16x16x32 MFMA, O^T += V^T P^T on the 16x16x16 MFMA with
//   V^T read by the transposing ds_read_b64_tr_b16; every K/V byte loaded
//   serves all g heads. Online softmax with a lazily moved reference (moved
//   only when a score exceeds it by 2^8), row sums from the bf16-rounded P.
// * Every load of the stream is an LDS-direct buffer load and they complete in
//   issue order, so "tile p has landed" is "at most the loads of the tiles
//   issued after it are pending", whatever other memory operations (query
//   loads, partial stores) are outstanding.
#include <mutex>

#include "common.hpp"
#include "kernels.hpp"

namespace la {
namespace {

constexpr int kKT = 16;       // keys per wave tile
constexpr int kNS = 4;        // LDS ring stages per wave
constexpr int kWaves = kDecodeWaves;   // waves per workgroup
constexpr float kLazy = 8.f;  // log2 headroom of the lazily moved softmax reference
constexpr int kMaxB = kDecodeMaxBatch;   // sequences per call (tables in LDS)

// Physical 16-byte chunk of logical chunk c in row r of a V tile. The
// transposing reads of the 16x16x16 products take, per 32 lanes, 8
// consecutive rows x 32 bytes: the row term spreads those 8 rows over the
// 256-byte bank row (D = 128: 32-byte steps over 8 rows; D = 64, two rows per
// bank row: 32-byte steps over row pairs), so no two lanes share a bank.
template <int CH>
__device__ __forceinline__ int dv_chunk(int c, int r) { return c ^ (CH == 16 ? 2 * (r & 7) : 2 * ((r >> 1) & 3)); }

__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Lane exchanges on the VALU (v_permlane16/32_swap), not through the LDS
// crossbar that __shfl_xor (ds_bpermute) uses: the tile loop runs them while
// its LDS-direct loads are in flight.
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float add_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float add_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// One work item: split s of KV head kvh of sequence b, keys [k0, k1).
struct Item {
  int b, kvh, s, ns, L, k0, k1, nt;   // ns: splits of sequence b; nt: tiles of the item
};

template <int D, int G, bool PAGED>
__global__ __launch_bounds__(64 * kWaves) void decode_kernel(DecodeArgs a) {
  constexpr int CH = D / 8;            // 16-byte chunks per row
  constexpr int ROW = D * 2;           // bytes per row
  constexpr int TB = kKT * ROW;        // bytes of one K or V tile
  constexpr int NLD = kKT * CH / 64;   // 1 KB loads per tile per tensor
  constexpr int KS = D / 32;           // k-steps of S^T (16x16x32)
  constexpr int DB = D / 16;           // 16-row blocks of O^T

  __shared__ __attribute__((aligned(1024))) char ring[kWaves][kNS][2][TB];
  __shared__ int s_len[kMaxB];         // clamped sequence lengths
  __shared__ int s_items[kMaxB + 1];   // items before sequence b
  __shared__ int s_tiles[kMaxB + 1];   // tiles before sequence b

  const int lane = threadIdx.x & 63, wave = uni(threadIdx.x >> 6);
  const int lc = lane & 15, lg = lane >> 4;
  const int C = a.kv_chunk;
  const int TPS = C / kKT;             // tiles of a full split

  // ---- item and tile tables (the stream order is b, kvh, split) --------------
  for (int b = threadIdx.x; b < a.B; b += blockDim.x) s_len[b] = max(1, min(a.seq_lens[b], a.Lmax));
  __syncthreads();
  if (wave == 0) {
    int ci = 0, ct = 0;
    for (int b0 = 0; b0 < a.B; b0 += 64) {
      const int b = b0 + lane;
      int ni = 0, nt = 0;
      if (b < a.B) {
        const int L = s_len[b];
        ni = ((L + C - 1) / C) * a.Hkv;
        nt = ((L + kKT - 1) / kKT) * a.Hkv;
      }
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int x = __shfl_up(ni, o), y = __shfl_up(nt, o);
        if (lane >= o) {
          ni += x;
          nt += y;
        }
      }
      if (b < a.B) {
        s_items[b + 1] = ci + ni;
        s_tiles[b + 1] = ct + nt;
      }
      ci += __shfl(ni, 63);
      ct += __shfl(nt, 63);
    }
    if (lane == 0) {
      s_items[0] = 0;
      s_tiles[0] = 0;
    }
  }
  __syncthreads();

  const int NI = uni(s_items[a.B]);
  const int T = uni(s_tiles[a.B]);
  auto item_at = [&](int i) -> Item {
    int lo = 0, hi = a.B;   // s_items[lo] <= i < s_items[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (uni(s_items[mid]) <= i) lo = mid; else hi = mid;
    }
    Item it;
    it.b = lo;
    it.L = uni(s_len[lo]);
    it.ns = (it.L + C - 1) / C;
    const int r = i - uni(s_items[lo]);
    it.kvh = r / it.ns;
    it.s = r - it.kvh * it.ns;
    it.k0 = it.s * C;
    it.k1 = min(it.k0 + C, it.L);
    it.nt = (it.k1 - it.k0 + kKT - 1) / kKT;
    return it;
  };
  auto next_item = [&](Item& it) {   // the item after it in stream order (b, kvh, split)
    if (++it.s == it.ns) {
      it.s = 0;
      if (++it.kvh == a.Hkv) {
        it.kvh = 0;
        ++it.b;
        it.L = uni(s_len[it.b]);
        it.ns = (it.L + C - 1) / C;
      }
    }
    it.k0 = it.s * C;
    it.k1 = min(it.k0 + C, it.L);
    it.nt = (it.k1 - it.k0 + kKT - 1) / kKT;
  };
  auto start_tile = [&](int i) -> int {
    if (i >= NI) return T;
    const Item it = item_at(i);
    return uni(s_tiles[it.b]) + it.kvh * ((it.L + kKT - 1) / kKT) + it.s * TPS;
  };
  auto first_item_from = [&](int64_t t) -> int {   // smallest i with start_tile(i) >= t
    int lo = 0, hi = NI;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (start_tile(mid) >= t) hi = mid; else lo = mid + 1;
    }
    return lo;
  };
  // this wave's share: the items starting in its equal slice of the tile stream
  const int W = gridDim.x * kWaves;
  const int gw = blockIdx.x * kWaves + wave;
  const int i0 = first_item_from((int64_t)gw * T / W);
  const int i1 = first_item_from((int64_t)(gw + 1) * T / W);
  if (a.hdr) {   // compact partials: which (sequence, KV head) pairs this wave holds runs of
    int first = 0x7fffffff, last = -1;
    if (i0 < i1) {
      const Item f = item_at(i0), t = item_at(i1 - 1);
      first = f.b * a.Hkv + f.kvh;
      last = t.b * a.Hkv + t.kvh;
    }
    if (lane == 0) {
      a.hdr[2 * gw] = first;
      a.hdr[2 * gw + 1] = last;
    }
  }
  if (i0 >= i1) return;

  // ---- per-lane constant offsets ---------------------------------------------
  int koffv[NLD], voffv[NLD];
#pragma unroll
  for (int n = 0; n < NLD; ++n) {
    const int p = n * 64 + lane;   // LDS chunk written by this lane
    const int row = p / CH, ph = p % CH;
    koffv[n] = (int)(row * a.cs_l * 2 + 16 * k_chunk<CH>(ph, row));
    voffv[n] = (int)(row * a.cs_l * 2 + 16 * dv_chunk<CH>(ph, row));
  }
  // K operand (A of S^T = K Q^T): row lc, logical chunk 4ks + lg
  const int k_lane = lc * ROW;
  // V^T operand (A of O^T += V^T P^T, 16x16x16): group lg covers keys 4lg + 0..3;
  // input lane L = lc addresses row 4lg + L/4 at d0 = 16db + 4(L%4)
  const int vrow = 4 * lg + (lc >> 2);
  int v_lane[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
    v_lane[db] = vrow * ROW + 16 * dv_chunk<CH>(2 * db + ((lc >> 1) & 1), vrow) + 8 * (lc & 1);

  char* my = &ring[wave][0][0][0];

  // ---- load cursor over the wave's tile stream --------------------------------
  int li = i0, lt = 0;
  Item lit = item_at(i0);
  // paged cache: the page of the cursor's tile, loaded one issue ahead so its
  // latency overlaps a tile's work (a 16-key tile never crosses a page). The
  // loaded id stays in a VGPR until that issue takes it to a scalar register:
  // vector loads complete in issue order, so the wait there covers only the
  // loads issued before it, not the tiles in flight after it.
  const int page_mask = (1 << a.page_shift) - 1;
  int pgv = 0;
  auto page_of = [&](const Item& it, int t) -> int {
    return a.block_table[(int64_t)it.b * a.bt_stride + ((it.k0 + t * kKT) >> a.page_shift)];
  };
  if constexpr (PAGED) pgv = page_of(lit, 0);
  auto issue = [&](int st) {
    const __bf16* kb = static_cast<const __bf16*>(a.k);
    const __bf16* vb = static_cast<const __bf16*>(a.v);
    int bytes = 0;   // past the stream end: loads that read nothing keep the count uniform
    if (li < i1) {
      const int key = lit.k0 + lt * kKT;
      int pg = 0;
      if constexpr (PAGED) {
        // the id's VGPR is read here only; the empty asm keeps the compiler
        // from moving the read (and its wait) up to the load
        asm volatile("" : "+v"(pgv));
        pg = __builtin_amdgcn_readfirstlane(pgv);
      }
      const int64_t base = PAGED ? (int64_t)pg * a.cs_b + lit.kvh * a.cs_h + (int64_t)(key & page_mask) * a.cs_l
                                 : lit.b * a.cs_b + lit.kvh * a.cs_h + (int64_t)key * a.cs_l;
      kb += base;
      vb += base;
      const int rows = min(kKT, lit.k1 - key);
      bytes = (int)(((int64_t)(rows - 1) * a.cs_l + D) * 2);
      if (++lt == lit.nt) {
        ++li;
        lt = 0;
        if (li < i1) next_item(lit);
      }
      if constexpr (PAGED)
        if (li < i1) pgv = page_of(lit, lt);
    }
    char* dst = my + st * 2 * TB;
#pragma unroll
    for (int n = 0; n < NLD; ++n) {
      load_lds16(kb, bytes, koffv[n], dst + n * 1024);
      load_lds16(vb, bytes, voffv[n], dst + TB + n * 1024);
    }
  };

#pragma unroll
  for (int s = 0; s < kNS - 1; ++s) issue(s);

  // ---- compute cursor -------------------------------------------------------------
  bf16x8 qreg[KS];
  f32x4 acc[DB];
  float m = -INFINITY, l = 0.f;
  int ci = i0, ct = 0, run_s0 = 0;
  Item cit = item_at(i0);
  // the loop is unrolled over the kNS stages, so every stage's LDS offset is a
  // constant: the compiler can then tell a stage being filled from the one
  // being read and waits only for the loads of the tile it reads (with a
  // run-time stage index it waits for every load in flight before each read)
  while (ci < i1) {
#pragma unroll
    for (int u = 0; u < kNS; ++u) {
      if (ci < i1) {   // uniform: once the stream ends, the remaining steps are skipped
        if (ct == 0 && (ci == i0 || cit.s == 0)) {   // a run of this (b, kvh) starts
          const bool ok = lc < G;
          const __bf16* qp = static_cast<const __bf16*>(a.q) + cit.b * a.qs_b +
                             (cit.kvh * G + (ok ? lc : 0)) * a.qs_h + 8 * lg;
    #pragma unroll
          for (int ks = 0; ks < KS; ++ks) qreg[ks] = ok ? load8(qp + 32 * ks) : zero_bf16x8();
    #pragma unroll
          for (int db = 0; db < DB; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
          m = -INFINITY;
          l = 0.f;
          run_s0 = cit.s;
        }
        // tile p has landed once no more than the loads of tiles p+1 .. p+kNS-2 are pending
        asm volatile("s_waitcnt vmcnt(%0)" :: "n"(2 * NLD * (kNS - 2)) : "memory");
        issue((u + kNS - 1) % kNS);

        const char* lk = my + u * 2 * TB;
        const char* lv = lk + TB;
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
    #pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 ka = *reinterpret_cast<const bf16x8*>(lk + k_lane + 16 * k_chunk<CH>(4 * ks + lg, lc));
          s = mfma16k32(ka, qreg[ks], s);
        }
        // lane holds S^T[key = key0 + 4lg + j][col = lc]. Keys past the item's
        // end (only in its last tile) are masked without a branch: the scores are
        // read here right after their MFMA, and the compiler pads that read with
        // the wait the matrix core needs only on a single path.
        const int kbase = cit.k0 + ct * kKT + 4 * lg;
    #pragma unroll
        for (int j = 0; j < 4; ++j) s[j] = kbase + j < cit.k1 ? s[j] : -INFINITY;
        float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
        mx = max_xor32(max_xor16(mx));
        const bool mv = mx * a.scale_log2 > m * a.scale_log2 + kLazy;
        if (__any(mv)) {   // rare after a run's first tile
          const float al = mv ? fast_exp2((m - mx) * a.scale_log2) : 1.f;   // 0 when m = -inf
          m = mv ? mx : m;
          l *= al;
    #pragma unroll
          for (int db = 0; db < DB; ++db) acc[db] *= al;
        }
        const float mc = m * a.scale_log2;   // finite: the tile holds at least one key
        bf16x2 p01, p23;
        p01[0] = to_bf16(fast_exp2(fmaf(s[0], a.scale_log2, -mc)));
        p01[1] = to_bf16(fast_exp2(fmaf(s[1], a.scale_log2, -mc)));
        p23[0] = to_bf16(fast_exp2(fmaf(s[2], a.scale_log2, -mc)));
        p23[1] = to_bf16(fast_exp2(fmaf(s[3], a.scale_log2, -mc)));
        const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
        l = __builtin_amdgcn_fdot2_f32_bf16(p01, one, l, false);
        l = __builtin_amdgcn_fdot2_f32_bf16(p23, one, l, false);
        const bf16x4 pv = {p01[0], p01[1], p23[0], p23[1]};
    #pragma unroll
        for (int db = 0; db < DB; ++db) {
          const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lv + v_lane[db]));
          acc[db] = mfma16k16(__builtin_bit_cast(bf16x4, r), pv, acc[db]);
        }

        if (++ct == cit.nt) {   // item done
          if (ci + 1 == i1 || cit.s + 1 == cit.ns) {   // run done: its partial goes to slot run_s0
            const float lt2 = add_xor32(add_xor16(l));
            if (lc < G && a.hdr) {   // compact: slot gw + bh, head lc of the group
              const int64_t slot = ((int64_t)gw + cit.b * a.Hkv + cit.kvh) * G + lc;
              float* op = a.o_part + slot * D;
    #pragma unroll
              for (int db = 0; db < DB; ++db)
                *reinterpret_cast<f32x4*>(op + 16 * db + 4 * lg) = acc[db] / lt2;
              if (lg == 0) a.lse_part[slot] = m * a.scale + fast_log2(lt2) * kLn2;
            } else if (lc < G) {
              const int64_t row = ((int64_t)cit.b * a.Hq + cit.kvh * G + lc) * a.max_splits;
              float* op = a.o_part + (row + run_s0) * D;
    #pragma unroll
              for (int db = 0; db < DB; ++db)
                *reinterpret_cast<f32x4*>(op + 16 * db + 4 * lg) = acc[db] / lt2;
              if (lg == 0) a.lse_part[row + run_s0] = m * a.scale + fast_log2(lt2) * kLn2;
              for (int s2 = run_s0 + 1 + lg; s2 <= cit.s; s2 += 4) a.lse_part[row + s2] = -INFINITY;
            }
          }
          ++ci;
          ct = 0;
          if (ci < i1) next_item(cit);
        }
      }
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // loads past the stream end
}

template <int D>
__global__ __launch_bounds__(256) void combine_kernel_f(CombineArgs a, int dt) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int pair = blockIdx.x * 4 + wave;
  if (pair >= a.B * a.Hq) return;
  const int b = pair / a.Hq, h = pair % a.Hq;
  float W = 0.f;
  float o[D / 64];
#pragma unroll
  for (int i = 0; i < D / 64; ++i) o[i] = 0.f;
  float M = -INFINITY;
  if (a.hdr) {
    // compact partials: the runs of pair bh are held by the waves whose
    // header range contains bh, in slot w + bh; merged in wave order, which is
    // the split order of the slot layout below
    const int G = a.Hq / a.Hkv;
    const int bh = b * a.Hkv + h / G, gh = h % G;
    auto run_lse = [&](int w) -> float {
      const bool in = w < a.W && a.hdr[2 * w] <= bh && bh <= a.hdr[2 * w + 1];
      return in ? a.lse_part[((int64_t)w + bh) * G + gh] : -INFINITY;
    };
    for (int w = lane; w < a.W; w += 64) M = fmaxf(M, run_lse(w));
#pragma unroll
    for (int x = 32; x > 0; x >>= 1) M = fmaxf(M, __shfl_xor(M, x));
    for (int w0 = 0; w0 < a.W; w0 += 64) {
      const float ls = run_lse(w0 + lane);
      uint64_t live = __ballot(ls != -INFINITY);
      while (live) {
        const int j = __builtin_ctzll(live);
        live &= live - 1;
        const float w = expf(__shfl(ls, j) - M);
        W += w;
        const float* op = a.o_part + (((int64_t)w0 + j + bh) * G + gh) * D;
#pragma unroll
        for (int i = 0; i < D / 64; ++i) o[i] += w * op[lane + 64 * i];
      }
    }
  } else {
    const int L = max(1, a.seq_lens[b]);
    const int n = min((L + a.kv_chunk - 1) / a.kv_chunk, a.max_splits);
    const float* lp = a.lse_part + (int64_t)pair * a.max_splits;
    const float* op = a.o_part + (int64_t)pair * a.max_splits * D;
    for (int s = lane; s < n; s += 64) M = fmaxf(M, lp[s]);
#pragma unroll
    for (int x = 32; x > 0; x >>= 1) M = fmaxf(M, __shfl_xor(M, x));
    for (int s0 = 0; s0 < n; s0 += 64) {   // slots with lse = -inf carry nothing and are skipped
      const float ls = s0 + lane < n ? lp[s0 + lane] : -INFINITY;
      uint64_t live = __ballot(ls != -INFINITY);
      while (live) {
        const int j = __builtin_ctzll(live);
        live &= live - 1;
        const float w = expf(__shfl(ls, j) - M);
        W += w;
#pragma unroll
        for (int i = 0; i < D / 64; ++i) o[i] += w * op[(int64_t)(s0 + j) * D + lane + 64 * i];
      }
    }
  }
  if (dt == 0) {
    __bf16* out = static_cast<__bf16*>(a.o) + b * a.os_b + h * a.os_h;
#pragma unroll
    for (int i = 0; i < D / 64; ++i) out[lane + 64 * i] = to_bf16(o[i] / W);
  } else {
    float* out = static_cast<float*>(a.o) + b * a.os_b + h * a.os_h;
#pragma unroll
    for (int i = 0; i < D / 64; ++i) out[lane + 64 * i] = o[i] / W;
  }
  if (a.lse && lane == 0) a.lse[pair] = M + logf(W);
}

template <int D, int G>
hipError_t launch_dt(const DecodeArgs& a, hipStream_t st) {
  // persistent grid: one workgroup per CU (the LDS ring takes most of a CU's
  // LDS); the grid size only shapes the work split, never the result
  const unsigned grid = (unsigned)(a.grid > 0 ? a.grid : 256);
  if (a.block_table)
    hipLaunchKernelGGL((decode_kernel<D, G, true>), dim3(grid), dim3(64 * kWaves), 0, st, a);
  else
    hipLaunchKernelGGL((decode_kernel<D, G, false>), dim3(grid), dim3(64 * kWaves), 0, st, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DecodeArgs& a, int G, hipStream_t st) {
  switch (G) {
    case 1: return launch_dt<D, 1>(a, st);
    case 2: return launch_dt<D, 2>(a, st);
    case 4: return launch_dt<D, 4>(a, st);
    case 8: return launch_dt<D, 8>(a, st);
    case 16: return launch_dt<D, 16>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int D, int G, hipStream_t st) {
  return D == 64 ? launch_d<64>(a, G, st) : launch_d<128>(a, G, st);
}

// ---- scratch of the allocation-free decode ----------------------------------
// A file-scope device array: each device the library runs on holds its own
// copy from module load until the process ends. Host code takes its device
// address from hipGetSymbolAddress, once per device with that device current;
// the array's name itself is only a host-side stand-in.
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices];
}  // namespace

hipError_t decode_scratch(void** ptr, size_t* bytes) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  *bytes = kScratchBytes;
  return hipSuccess;
}

hipError_t launch_combine(const CombineArgs& a, int D, int dt, hipStream_t st) {
  const unsigned grid = (unsigned)((a.B * a.Hq + 3) / 4);
  if (D == 64)
    hipLaunchKernelGGL((combine_kernel_f<64>), dim3(grid), dim3(256), 0, st, a, dt);
  else
    hipLaunchKernelGGL((combine_kernel_f<128>), dim3(grid), dim3(256), 0, st, a, dt);
  return hipGetLastError();
}

}  // namespace la
