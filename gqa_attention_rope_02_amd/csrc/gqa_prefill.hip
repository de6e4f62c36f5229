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
//   head, so each K/V byte staged in LDS feeds 256 query rows. Four waves own
//   64 columns each.
// * The contractions run transposed on the 32x32x16 bf16 MFMA: S^T = K Q^T
//   (keys on M, columns on N) and O^T = V^T P^T (head_dim on M). In both
//   results a lane owns one column, so the softmax statistics and the output
//   rescale stay in the lane; only the row max needs one cross-lane step
//   (lanes l and l^32), and the S^T accumulator already has the layout of the
//   P^T operand (no shuffle between the two products).
// * Q stays in registers for the whole key loop. K (row-major) and V
//   (transposed to [d][key]) are staged per 64-key tile in LDS, double
//   buffered, with XOR swizzles against bank conflicts; the next tile's global
//   loads are issued before the current tile's MFMAs.
// * Online softmax in the base-2 domain with fp32 statistics; the accumulator
//   is rescaled only when some lane's running max moved. Masks are evaluated
//   only on tiles that cross a causal or document edge of the wave's columns;
//   tiles entirely outside them are skipped.
// * Workgroups are issued longest-first (last token tiles first), and the KV
//   head is the fastest-varying index so the workgroups of one KV head land on
//   one XCD (blockIdx % 8) and share its L2.
#include "common.hpp"
#include "kernels.hpp"

namespace la {
namespace {

constexpr int kWaves = 4;
constexpr int kCols = 256;   // columns per workgroup
constexpr int kKT = 64;      // keys per tile

template <typename T, int D, int G>
__global__ __launch_bounds__(256) void prefill_kernel(PrefillArgs a) {
  constexpr int TQ = kCols / G;          // tokens per workgroup
  constexpr int KS = D / 16;             // k-steps of S^T = K Q^T
  constexpr int DB = D / 32;             // 32-row blocks of O^T
  constexpr int CH = D / 8;              // 16-byte chunks per K row
  constexpr int KLOADS = kKT * CH / 256; // K chunks loaded per thread
  constexpr int VTHREADS = (kKT / 4) * CH;

  __shared__ __attribute__((aligned(16))) __bf16 lds_k[2][kKT * D];
  __shared__ __attribute__((aligned(16))) __bf16 lds_v[2][D * kKT];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lc = lane & 31, hi = lane >> 5;

  const int bid = blockIdx.x;
  const int kvh = bid % a.Hkv;
  const int r = bid / a.Hkv;
  const int b = r % a.B;
  const int qtile = a.n_qtiles - 1 - r / a.B;
  const int S = a.S;
  const int t0 = qtile * TQ;
  const int t_end = min(t0 + TQ, S);
  const int32_t* cu = a.cu_docs ? a.cu_docs + (int64_t)b * (a.n_docs + 1) : nullptr;
  const int n_docs = a.n_docs;
  auto start_of = [&](int t) -> int { return cu ? doc_start(cu, n_docs, t) : 0; };
  // clamp: out-of-contract offsets must not move the key range out of [0, t0]
  const int kv_lo = max(0, min(start_of(t0), t0));
  const int kv_hi = t_end - 1;

  const T* qbase = static_cast<const T*>(a.q) + b * a.qs_b;
  const T* kbase = static_cast<const T*>(a.k) + b * a.ks_b + kvh * a.ks_h;
  const T* vbase = static_cast<const T*>(a.v) + b * a.vs_b + kvh * a.vs_h;

  // ---- this lane's two columns (one per 32-column block) -------------------
  int tok[2], head[2], st[2];
  bool valid[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int col = wave * 64 + cb * 32 + lc;
    tok[cb] = t0 + col / G;
    head[cb] = kvh * G + col % G;
    valid[cb] = tok[cb] < S;
    st[cb] = valid[cb] ? start_of(tok[cb]) : 0;
  }
  const int w_tmin = t0 + (wave * 64) / G;
  const int w_tmax_raw = t0 + (wave * 64 + 63) / G;
  const bool wave_active = w_tmin < S;
  const bool wave_all_valid = w_tmax_raw < S;
  const int w_tmax = min(w_tmax_raw, S - 1);
  const int w_smin = wave_active ? start_of(w_tmin) : 0;
  const int w_smax = wave_active ? start_of(w_tmax) : 0;

  // ---- Q operand (B of S^T = K Q^T): Q[col][16ks + 8hi + i] ----------------
  bf16x8 qreg[2][KS];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const T* qp = qbase + tok[cb] * a.qs_s + head[cb] * a.qs_h + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qreg[cb][ks] = valid[cb] ? load8(qp + 16 * ks) : zero_bf16x8();
  }

  f32x16 acc[DB][2];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[db][cb][j] = 0.f;
  float m[2] = {-INFINITY, -INFINITY};
  float l[2] = {0.f, 0.f};

  // ---- K/V tile staging ----------------------------------------------------
  bf16x8 kr[KLOADS];
  bf16x8 vr[4];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int n = 0; n < KLOADS; ++n) {
      const int id = tid + 256 * n;
      const int key = id / CH, c = id % CH;
      const int j = kt + key;
      kr[n] = j < S ? load8(kbase + j * a.ks_s + 8 * c) : zero_bf16x8();
    }
    if (tid < VTHREADS) {
      const int kg = tid / CH, c = tid % CH;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = kt + 4 * kg + i;
        vr[i] = j < S ? load8(vbase + j * a.vs_s + 8 * c) : zero_bf16x8();
      }
    }
  };
  auto store_tile = [&](int stage) {
    __bf16* lk = lds_k[stage];
#pragma unroll
    for (int n = 0; n < KLOADS; ++n) {
      const int id = tid + 256 * n;
      const int key = id / CH, c = id % CH;
      *reinterpret_cast<bf16x8*>(lk + key * D + 8 * (c ^ (key & (CH - 1)))) = kr[n];
    }
    if (tid < VTHREADS) {
      __bf16* lv = lds_v[stage];
      const int kg = tid / CH, c = tid % CH;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int d = 8 * c + e;
        bf16x4 w;
        w[0] = vr[0][e];
        w[1] = vr[1][e];
        w[2] = vr[2][e];
        w[3] = vr[3][e];
        *reinterpret_cast<bf16x4*>(lv + d * kKT + 4 * (kg ^ (d & 15))) = w;
      }
    }
  };

  const int n_tiles = (kv_hi - kv_lo) / kKT + 1;
  load_tile(kv_lo);
  store_tile(0);
  __syncthreads();

  for (int n = 0; n < n_tiles; ++n) {
    const int kt = kv_lo + n * kKT;
    const int stage = n & 1;
    if (n + 1 < n_tiles) load_tile(kt + kKT);

    const bool skip = !wave_active || kt > w_tmax || kt + kKT - 1 < w_smin;
    if (!skip) {
      const bool need_mask = !wave_all_valid || kt + kKT - 1 > w_tmin || kt < w_smax;
      const __bf16* lk = lds_k[stage];
      const __bf16* lv = lds_v[stage];

      // The tile is consumed in two 32-key halves kb, each with its own
      // online-softmax step, which keeps the score block at 32 registers.
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        // S^T[key][col] for keys kt + 32kb .. kt + 32kb + 31
        f32x16 s[2];
#pragma unroll
        for (int cb = 0; cb < 2; ++cb)
#pragma unroll
          for (int j = 0; j < 16; ++j) s[cb][j] = 0.f;
        const int key = kb * 32 + lc;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int c = 2 * ks + hi;
          const bf16x8 ka = *reinterpret_cast<const bf16x8*>(lk + key * D + 8 * (c ^ (key & (CH - 1))));
          s[0] = mfma32(ka, qreg[0][ks], s[0]);
          s[1] = mfma32(ka, qreg[1][ks], s[1]);
        }

        if (need_mask) {
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int kj = kt + kb * 32 + 8 * (j >> 2) + 4 * hi + (j & 3);
#pragma unroll
            for (int cb = 0; cb < 2; ++cb) {
              const bool vis = valid[cb] && kj >= st[cb] && kj <= tok[cb];
              if (!vis) s[cb][j] = -INFINITY;
            }
          }
        }

        // online softmax, base 2
        float alpha[2];
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
          float mx = -INFINITY;
#pragma unroll
          for (int j = 0; j < 16; ++j) mx = fmaxf(mx, s[cb][j]);
          mx = fmaxf(mx, __shfl_xor(mx, 32));
          const float mnew = fmaxf(m[cb], mx);
          const float mc = mnew == -INFINITY ? 0.f : mnew * a.scale_log2;
          alpha[cb] = fast_exp2(m[cb] * a.scale_log2 - mc);
          m[cb] = mnew;
          float rs = 0.f;
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const float p = fast_exp2(fmaf(s[cb][j], a.scale_log2, -mc));
            s[cb][j] = p;
            rs += p;
          }
          l[cb] = l[cb] * alpha[cb] + rs;
        }
        if (__any(alpha[0] != 1.f || alpha[1] != 1.f)) {
#pragma unroll
          for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int cb = 0; cb < 2; ++cb)
#pragma unroll
              for (int j = 0; j < 16; ++j) acc[db][cb][j] *= alpha[cb];
        }

        // O^T += V^T P^T, 16 keys per step
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int ks = 2 * kb + h2;
          bf16x8 p[2];
#pragma unroll
          for (int cb = 0; cb < 2; ++cb)
#pragma unroll
            for (int i = 0; i < 8; ++i) p[cb][i] = to_bf16(s[cb][8 * h2 + i]);
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const int d = db * 32 + lc;
            const __bf16* row = lv + d * kKT;
            const bf16x4 v0 = *reinterpret_cast<const bf16x4*>(row + 4 * ((4 * ks + hi) ^ (d & 15)));
            const bf16x4 v1 = *reinterpret_cast<const bf16x4*>(row + 4 * ((4 * ks + 2 + hi) ^ (d & 15)));
            const bf16x8 va = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
            acc[db][0] = mfma32(va, p[0], acc[db][0]);
            acc[db][1] = mfma32(va, p[1], acc[db][1]);
          }
        }
      }
    }

    if (n + 1 < n_tiles) store_tile(stage ^ 1);
    __syncthreads();
  }

  // ---- epilogue --------------------------------------------------------------
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const float lt = l[cb] + __shfl_xor(l[cb], 32);
    if (!valid[cb]) continue;
    // true division (once per output): a row whose weights are all exact gets
    // an exactly rounded mean
    T* op = static_cast<T*>(a.o) + b * a.os_b + tok[cb] * a.os_s + head[cb] * a.os_h;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int jq = 0; jq < 4; ++jq) {
        const int d = db * 32 + 8 * jq + 4 * hi;
        store4(op + d, acc[db][cb][4 * jq] / lt, acc[db][cb][4 * jq + 1] / lt,
               acc[db][cb][4 * jq + 2] / lt, acc[db][cb][4 * jq + 3] / lt);
      }
    if (a.lse && hi == 0)
      a.lse[((int64_t)b * a.Hq + head[cb]) * S + tok[cb]] = m[cb] * a.scale + fast_log2(lt) * kLn2;
  }
}

template <typename T, int D, int G>
hipError_t launch_t(const PrefillArgs& a, hipStream_t st) {
  const unsigned grid = (unsigned)a.B * a.Hkv * a.n_qtiles;
  hipLaunchKernelGGL((prefill_kernel<T, D, G>), dim3(grid), dim3(256), 0, st, a);
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

}  // namespace la
