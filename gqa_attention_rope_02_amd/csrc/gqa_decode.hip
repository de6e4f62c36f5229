// Split-KV decode over a KV cache and the log-sum-exp merge of its splits.
//
// What is computed: one new token per sequence attends, with each of its Hq
// query heads, to every cached token of the KV head its group shares ("How
// Meta's Llama 3.1 405B Architecture Actually Works", GQA paragraph: grouping
// query heads onto one key/value head shrinks the cache read while decoding).
// The cache window is cut into splits of kv_chunk slots; each split's
// softmax-normalised output and log-sum-exp are merged afterwards by
// O = sum_s w_s o_s / sum_s w_s, w_s = exp(lse_s - max lse).
//
// How (gfx950): the path is bound by the HBM read of the cache (16 FLOP per
// byte at 16 query heads per KV head), so the kernel is built to keep cache
// bytes in flight and to read each byte exactly once:
// * one workgroup = one (sequence, KV head, split); the g query heads of the
//   group are the 16 columns of a 16x16 MFMA tile, so every K/V byte loaded
//   serves all g heads;
// * 64-key tiles are fetched with coalesced 16-byte loads (each 256-byte row
//   by 16 consecutive lanes), the next tile's loads issued before the current
//   tile is consumed, and staged through LDS (V transposed to [d][key]) with
//   XOR swizzles; each of the four waves takes 16 keys of the tile, runs
//   S^T = K Q^T on the 16x16x32 MFMA and O^T += V^T P^T on the 16x16x16 MFMA,
//   and keeps its own online-softmax state, merged across waves through LDS
//   at the end of the split.
#include "common.hpp"
#include "kernels.hpp"

namespace la {
namespace {

constexpr int kKT = 64;

template <int D, int G>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
  constexpr int CH = D / 8;
  constexpr int KLOADS = kKT * CH / 256;
  constexpr int VTHREADS = (kKT / 4) * CH;
  constexpr int KS = D / 32;      // k-steps of S^T (16x16x32)
  constexpr int DB = D / 16;      // 16-row blocks of O^T

  __shared__ __attribute__((aligned(16))) __bf16 lds_k[2][kKT * D];
  __shared__ __attribute__((aligned(16))) __bf16 lds_v[2][D * kKT];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lc = lane & 15, lg = lane >> 4;

  // blockIdx.x = (b * Hkv + kvh) * max_splits + split
  const int split = blockIdx.x % a.max_splits;
  const int bh = blockIdx.x / a.max_splits;
  const int kvh = bh % a.Hkv, b = bh / a.Hkv;
  const int L = min(a.seq_lens[b], a.Lmax);   // never read past the cache window
  const int k_begin = split * a.kv_chunk;
  const int k_end = min(k_begin + a.kv_chunk, L);

  float* o_part = a.o_part;
  float* lse_part = a.lse_part;
  if (k_begin >= k_end) {  // empty split: o = 0, lse = -inf
    for (int x = tid; x < G * D; x += 256) {
      const int col = x / D, d = x % D;
      const int64_t row = ((int64_t)b * a.Hq + kvh * G + col) * a.max_splits + split;
      o_part[row * D + d] = 0.f;
      if (d == 0) lse_part[row] = -INFINITY;
    }
    return;
  }

  const __bf16* kbase = static_cast<const __bf16*>(a.k) + b * a.cs_b + kvh * a.cs_h;
  const __bf16* vbase = static_cast<const __bf16*>(a.v) + b * a.cs_b + kvh * a.cs_h;

  // Q operand (B of S^T = K Q^T): Q[col][32ks + 8lg + i]; columns >= G are 0.
  bf16x8 qreg[KS];
  {
    const bool ok = lc < G;
    const __bf16* qp = static_cast<const __bf16*>(a.q) + b * a.qs_b + (kvh * G + (ok ? lc : 0)) * a.qs_h + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qreg[ks] = ok ? load8(qp + 32 * ks) : zero_bf16x8();
  }

  f32x4 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;

  bf16x8 kr[KLOADS];
  bf16x8 vr[4];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int n = 0; n < KLOADS; ++n) {
      const int id = tid + 256 * n;
      const int key = id / CH, c = id % CH;
      const int j = kt + key;
      kr[n] = j < k_end ? load8(kbase + j * a.cs_l + 8 * c) : zero_bf16x8();
    }
    if (tid < VTHREADS) {
      const int kg = tid / CH, c = tid % CH;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = kt + 4 * kg + i;
        vr[i] = j < k_end ? load8(vbase + j * a.cs_l + 8 * c) : zero_bf16x8();
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

  const int n_tiles = (k_end - k_begin + kKT - 1) / kKT;
  load_tile(k_begin);
  store_tile(0);
  __syncthreads();

  for (int n = 0; n < n_tiles; ++n) {
    const int kt = k_begin + n * kKT;
    const int stage = n & 1;
    if (n + 1 < n_tiles) load_tile(kt + kKT);

    const int wk0 = kt + 16 * wave;   // first key of this wave's slice
    if (wk0 < k_end) {
      const __bf16* lk = lds_k[stage];
      const __bf16* lv = lds_v[stage];
      f32x4 s = {0.f, 0.f, 0.f, 0.f};
      const int key = 16 * wave + lc;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int c = 4 * ks + lg;
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(lk + key * D + 8 * (c ^ (key & (CH - 1))));
        s = mfma16k32(ka, qreg[ks], s);
      }
      // lane holds S^T[key = wk0 + 4lg + j][col = lc]
      if (wk0 + 16 > k_end) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (wk0 + 4 * lg + j >= k_end) s[j] = -INFINITY;
      }
      float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(m, mx);
      const float mc = mnew * a.scale_log2;   // finite: the slice holds >= 1 key
      const float alpha = fast_exp2(m * a.scale_log2 - mc);
      m = mnew;
      bf16x4 p;
      float rs = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float e = fast_exp2(fmaf(s[j], a.scale_log2, -mc));
        rs += e;
        p[j] = to_bf16(e);
      }
      l = l * alpha + rs;
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db] *= alpha;
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int d = 16 * db + lc;
        const bf16x4 va = *reinterpret_cast<const bf16x4*>(lv + d * kKT + 4 * ((4 * wave + lg) ^ (d & 15)));
        acc[db] = mfma16k16(va, p, acc[db]);
      }
    }

    if (n + 1 < n_tiles) store_tile(stage ^ 1);
    __syncthreads();
  }

  // ---- merge the four waves' partial softmax states --------------------------
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  float* red = reinterpret_cast<float*>(&lds_k[0][0]);   // [4][16][D] accumulators
  float* red_m = reinterpret_cast<float*>(&lds_v[0][0]); // [4][16]
  float* red_l = red_m + 64;                              // [4][16]
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 4; ++j) red[(wave * 16 + lc) * D + 16 * db + 4 * lg + j] = acc[db][j];
  if (lg == 0) {
    red_m[wave * 16 + lc] = m;
    red_l[wave * 16 + lc] = l;
  }
  __syncthreads();
  for (int x = tid; x < G * (D / 4); x += 256) {
    const int col = x / (D / 4), d0 = 4 * (x % (D / 4));
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, red_m[w * 16 + col]);
    const float Mc = M * a.scale_log2;
    float Ltot = 0.f;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float e = fast_exp2(red_m[w * 16 + col] * a.scale_log2 - Mc);   // 0 for an idle wave
      Ltot += e * red_l[w * 16 + col];
      const f32x4 v = *reinterpret_cast<const f32x4*>(&red[(w * 16 + col) * D + d0]);
      o += e * v;
    }
    const int64_t row = ((int64_t)b * a.Hq + kvh * G + col) * a.max_splits + split;
    *reinterpret_cast<f32x4*>(&o_part[row * D + d0]) = o / Ltot;
    if (d0 == 0) lse_part[row] = M * a.scale + fast_log2(Ltot) * kLn2;
  }
}

template <int D>
__global__ __launch_bounds__(256) void combine_kernel_f(CombineArgs a, int dt) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int pair = blockIdx.x * 4 + wave;
  if (pair >= a.B * a.Hq) return;
  const int b = pair / a.Hq, h = pair % a.Hq;
  const int L = max(1, a.seq_lens[b]);
  const int n = min((L + a.kv_chunk - 1) / a.kv_chunk, a.max_splits);
  const float* lp = a.lse_part + (int64_t)pair * a.max_splits;
  const float* op = a.o_part + (int64_t)pair * a.max_splits * D;
  float M = -INFINITY;
  for (int s = 0; s < n; ++s) M = fmaxf(M, lp[s]);
  float W = 0.f;
  float o[D / 64];
#pragma unroll
  for (int i = 0; i < D / 64; ++i) o[i] = 0.f;
  for (int s = 0; s < n; ++s) {
    const float w = expf(lp[s] - M);
    W += w;
#pragma unroll
    for (int i = 0; i < D / 64; ++i) o[i] += w * op[(int64_t)s * D + lane + 64 * i];
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
  const unsigned grid = (unsigned)a.B * a.Hkv * a.max_splits;
  hipLaunchKernelGGL((decode_kernel<D, G>), dim3(grid), dim3(256), 0, st, a);
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

hipError_t launch_combine(const CombineArgs& a, int D, int dt, hipStream_t st) {
  const unsigned grid = (unsigned)((a.B * a.Hq + 3) / 4);
  if (D == 64)
    hipLaunchKernelGGL((combine_kernel_f<64>), dim3(grid), dim3(256), 0, st, a, dt);
  else
    hipLaunchKernelGGL((combine_kernel_f<128>), dim3(grid), dim3(256), 0, st, a, dt);
  return hipGetLastError();
}

}  // namespace la
