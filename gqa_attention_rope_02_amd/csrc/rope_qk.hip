// Rotary position embedding of queries and keys ("Llama 3.1 Architecture:
// Dense Scaling to 405B and 128K Context", "1. High Base Frequency":
// theta_k = base^(-2k/d), k in [0, d/2-1]; base 500,000 per "The Llama 3 Herd
// of Models", "A Deliberately Standard Dense Transformer").
//
// A thread owns the pairs 4c..4c+3 of a head row (channels 8c..8c+7, one
// 16-byte chunk, for adjacent pairs (2k, 2k+1); channels 4c..4c+3 and
// D/2 + 4c..D/2 + 4c+3 for half-split pairs (k, k + D/2)) in every HG-th head of Q and K (Q's heads then K's, as
// one list) of one token; the D/8 threads of a chunk row cover a head row
// contiguously. A workgroup forms the angles position * theta_k of its tokens
// once, in revolutions (theta_k / 2pi comes from the host in fp64), reduces
// them to [-1/2, 1/2], takes sine and cosine in fp64 (sincospi) and shares
// them through LDS. Each thread's first kBatch rows are loaded before that,
// and each further batch of rows before any of it is rotated, so the memory
// latencies overlap the fp64 work and each other. The rotation runs in fp32
// on the fp64 sine and cosine split into high and low fp32 parts, with the
// first product's rounding error recovered by an FMA: the fp32 result is
// within 2^-23 relative of the exact rotation of the (exact) input, and a
// bf16 output, rounded from it to nearest even, within 0.5 ulp + 2^-23
// relative. At 128K positions an fp32 angle would already be off by ~1e-2 rad,
// hence the fp64 angle; it is formed once per (token, pair).
#include "common.hpp"
#include "kernels.hpp"

namespace la {
namespace {

constexpr int kThreads = 256;
constexpr int kBatch = 8;   // head rows in flight per thread

template <typename T>
struct Row8 {
  T v[8];
};

template <typename T>
__device__ __forceinline__ Row8<T> load_row(const T* p) {
  Row8<T> r;
  if constexpr (sizeof(T) == 2) {
    *reinterpret_cast<bf16x8*>(r.v) = *reinterpret_cast<const bf16x8*>(p);
  } else {
    *reinterpret_cast<f32x4*>(r.v) = *reinterpret_cast<const f32x4*>(p);
    *reinterpret_cast<f32x4*>(r.v + 4) = *reinterpret_cast<const f32x4*>(p + 4);
  }
  return r;
}

template <typename T>
__device__ __forceinline__ void store_row(T* p, const float* y) {
  if constexpr (sizeof(T) == 2) {
    bf16x8 v;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = to_bf16(y[i]);
    *reinterpret_cast<bf16x8*>(p) = v;
  } else {
    *reinterpret_cast<f32x4*>(p) = f32x4{y[0], y[1], y[2], y[3]};
    *reinterpret_cast<f32x4*>(p + 4) = f32x4{y[4], y[5], y[6], y[7]};
  }
}

// Half-split layout: the thread's four pairs are channels 4c..4c+3 and
// D/2 + 4c..D/2 + 4c+3; a Row8 holds the first four then the second four.
template <typename T>
__device__ __forceinline__ Row8<T> load_row_half(const T* p, int half_d) {
  Row8<T> r;
  if constexpr (sizeof(T) == 2) {
    typedef __bf16 b4 __attribute__((ext_vector_type(4)));
    *reinterpret_cast<b4*>(r.v) = *reinterpret_cast<const b4*>(p);
    *reinterpret_cast<b4*>(r.v + 4) = *reinterpret_cast<const b4*>(p + half_d);
  } else {
    *reinterpret_cast<f32x4*>(r.v) = *reinterpret_cast<const f32x4*>(p);
    *reinterpret_cast<f32x4*>(r.v + 4) = *reinterpret_cast<const f32x4*>(p + half_d);
  }
  return r;
}

template <typename T>
__device__ __forceinline__ void store_row_half(T* p, int half_d, const float* y) {
  if constexpr (sizeof(T) == 2) {
    typedef __bf16 b4 __attribute__((ext_vector_type(4)));
    b4 a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = to_bf16(y[i]);
      b[i] = to_bf16(y[4 + i]);
    }
    *reinterpret_cast<b4*>(p) = a;
    *reinterpret_cast<b4*>(p + half_d) = b;
  } else {
    *reinterpret_cast<f32x4*>(p) = f32x4{y[0], y[1], y[2], y[3]};
    *reinterpret_cast<f32x4*>(p + half_d) = f32x4{y[4], y[5], y[6], y[7]};
  }
}

// (y0, y1) = (x0 c - x1 s, x0 s + x1 c) in fp32, with c = ch + cl and
// s = sh + sl split into fp32 high and low parts of the fp64 values: the
// rounding error of the first product is recovered exactly by an FMA and the
// low parts enter as a correction, so y is the exact rotation up to the two
// fp32 roundings of the final sums (and terms 2^-48 smaller).
template <typename T>
__device__ __forceinline__ void rotate_pair(T a, T b, float ch, float cl, float sh, float sl, float* y) {
  const float x0 = (float)a, x1 = (float)b;
  {
    const float p = x1 * sh;
    const float ep = fmaf(x1, sh, -p);
    const float hi = fmaf(x0, ch, -p);
    const float lo = fmaf(x0, cl, -(x1 * sl)) - ep;
    y[0] = hi + lo;
  }
  {
    const float p = x1 * ch;
    const float ep = fmaf(x1, ch, -p);
    const float hi = fmaf(x0, sh, p);
    const float lo = fmaf(x0, sl, x1 * cl) + ep;
    y[1] = hi + lo;
  }
}

// A row of one head of Q (v < Hq) or K (v - Hq), as one list of heads.
template <typename T>
struct Rows {
  const T* qin;
  T* qout;
  const T* kin;
  T* kout;
  int64_t qis, qos, kis, kos;   // head strides
  int Hq, H;                    // Q heads, Q + K heads
  __device__ const T* in(int v) const { return v < Hq ? qin + v * qis : kin + (v - Hq) * kis; }
  __device__ T* out(int v) const { return v < Hq ? qout + v * qos : kout + (v - Hq) * kos; }
};

template <typename T, int D, int HG, bool HALF>
__global__ __launch_bounds__(kThreads) void rope_kernel(RopeArgs qa, RopeArgs ka, RopeAngles ang) {
  constexpr int CH = D / 8;              // 16-byte chunks (4 pairs) per head row
  constexpr int TT = kThreads / CH / HG; // tokens per workgroup
  __shared__ double lds_cs[TT][D / 2], lds_sn[TT][D / 2];
  const RopeArgs& any = qa.in ? qa : ka;
  const int64_t ntok = (int64_t)any.B * any.S;
  const int64_t tok0 = (int64_t)blockIdx.x * TT;
  const int c = threadIdx.x % CH;
  const int slot = threadIdx.x / CH;
  const int tt = slot / HG, g = slot % HG;
  const int64_t tok = tok0 + tt;
  const bool live = tok < ntok;
  const int b = live ? (int)(tok / any.S) : 0;
  const int s = live ? (int)(tok - (int64_t)b * any.S) : 0;

  Rows<T> rw;
  rw.Hq = qa.in ? qa.H : 0;
  rw.H = rw.Hq + (ka.in ? ka.H : 0);
  // this thread's channels start at 8c (adjacent pairs 4c..4c+3) or at 4c
  // and D/2 + 4c (half-split pairs 4c..4c+3)
  const int ch0 = HALF ? 4 * c : 8 * c;
  rw.qin = qa.in ? static_cast<const T*>(qa.in) + b * qa.is_b + s * qa.is_s + ch0 : nullptr;
  rw.qout = qa.in ? static_cast<T*>(qa.out) + b * qa.os_b + s * qa.os_s + ch0 : nullptr;
  rw.kin = ka.in ? static_cast<const T*>(ka.in) + b * ka.is_b + s * ka.is_s + ch0 : nullptr;
  rw.kout = ka.in ? static_cast<T*>(ka.out) + b * ka.os_b + s * ka.os_s + ch0 : nullptr;
  rw.qis = qa.is_h; rw.qos = qa.os_h; rw.kis = ka.is_h; rw.kos = ka.os_h;
  const int H = live ? rw.H : 0;

  // this thread's heads g, g + HG, ...: the first kBatch rows go out before
  // the angles are formed, so their latency overlaps the fp64 work
  Row8<T> r[kBatch];
#pragma unroll
  for (int i = 0; i < kBatch; ++i)
    if (g + i * HG < H) r[i] = HALF ? load_row_half<T>(rw.in(g + i * HG), D / 2) : load_row<T>(rw.in(g + i * HG));

  // sine and cosine of every (token, pair) of the workgroup, once, into LDS
  for (int e = threadIdx.x; e < TT * (D / 2); e += kThreads) {
    const int et = e / (D / 2), k = e % (D / 2);
    const int64_t t = tok0 + et;
    double sv = 0.0, cv = 1.0;
    if (t < ntok) {
      const int st_ = (int)(t % any.S);
      const double pos = any.positions ? (double)any.positions[t] : (double)st_;
      const double rev = pos * ang.theta_rev[k];
      sincospi(2.0 * (rev - rint(rev)), &sv, &cv);
    }
    lds_cs[et][k] = cv;
    lds_sn[et][k] = sv;
  }
  __syncthreads();
  float ch[4], cl[4], sh[4], sl[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const double cv = lds_cs[tt][4 * c + p], sv = lds_sn[tt][4 * c + p];
    ch[p] = (float)cv;
    cl[p] = (float)(cv - (double)ch[p]);
    sh[p] = (float)sv;
    sl[p] = (float)(sv - (double)sh[p]);
  }

  for (int v0 = g;; v0 += kBatch * HG) {
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int v = v0 + i * HG;
      if (v >= H) break;
      float y[8];
      if constexpr (HALF) {
        float yp[2];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          rotate_pair(r[i].v[p], r[i].v[4 + p], ch[p], cl[p], sh[p], sl[p], yp);
          y[p] = yp[0];
          y[4 + p] = yp[1];
        }
        store_row_half<T>(rw.out(v), D / 2, y);
      } else {
#pragma unroll
        for (int p = 0; p < 4; ++p) rotate_pair(r[i].v[2 * p], r[i].v[2 * p + 1], ch[p], cl[p], sh[p], sl[p], y + 2 * p);
        store_row<T>(rw.out(v), y);
      }
    }
    const int v1 = v0 + kBatch * HG;
    if (v1 >= H) break;
#pragma unroll
    for (int i = 0; i < kBatch; ++i)
      if (v1 + i * HG < H)
        r[i] = HALF ? load_row_half<T>(rw.in(v1 + i * HG), D / 2) : load_row<T>(rw.in(v1 + i * HG));
  }
}

template <typename T, int D, int HG>
hipError_t launch_hg(const RopeArgs& q, const RopeArgs& k, const RopeAngles& ang, hipStream_t st) {
  const RopeArgs& any = q.in ? q : k;
  constexpr int tpb = kThreads / (D / 8) / HG;
  const long long ntok = (long long)any.B * any.S;
  const dim3 grid((unsigned)((ntok + tpb - 1) / tpb));
  if (ang.half)
    hipLaunchKernelGGL((rope_kernel<T, D, HG, true>), grid, dim3(kThreads), 0, st, q, k, ang);
  else
    hipLaunchKernelGGL((rope_kernel<T, D, HG, false>), grid, dim3(kThreads), 0, st, q, k, ang);
  return hipGetLastError();
}

// head groups per token: few heads (keys alone) are spread over 4 threads per
// chunk and 4 tokens per workgroup; many heads over 16 threads per chunk, one
// token per workgroup for D = 128
template <typename T, int D>
hipError_t launch_t(const RopeArgs& q, const RopeArgs& k, const RopeAngles& ang, hipStream_t st) {
  const int heads = (q.in ? q.H : 0) + (k.in ? k.H : 0);
  return heads <= 16 ? launch_hg<T, D, 4>(q, k, ang, st) : launch_hg<T, D, 16>(q, k, ang, st);
}

}  // namespace

hipError_t launch_rope_pair(const RopeArgs& q, const RopeArgs& k, const RopeAngles& ang, int D, int dt,
                            hipStream_t st) {
  if (dt == 0) return D == 64 ? launch_t<__bf16, 64>(q, k, ang, st) : launch_t<__bf16, 128>(q, k, ang, st);
  return D == 64 ? launch_t<float, 64>(q, k, ang, st) : launch_t<float, 128>(q, k, ang, st);
}

}  // namespace la
