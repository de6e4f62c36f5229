// Rotary position embedding of queries and keys ("Llama 3.1 Architecture:
// Dense Scaling to 405B and 128K Context", "1. High Base Frequency":
// theta_k = base^(-2k/d), k in [0, d/2-1]; base 500,000 per "The Llama 3 Herd
// of Models", "A Deliberately Standard Dense Transformer").
//
// One workgroup per token. Its first D/2 threads form the angles
// position * theta_k in fp64, reduce them modulo 2*pi and take their sine and
// cosine in fp64 into LDS; then thread t rotates the 8 channels 8c..8c+7
// (pairs 4c..4c+3, c = t % (D/8)) of every (D/8)-th head with 16-byte loads
// and stores, the threads of one head row covering it contiguously. The
// rotation is done in fp64 and rounded to the storage type through fp32, so
// every bf16 output lies within 0.5 ulp + 2^-25 relative of the exact
// rotation of its (exact) input. At 128K positions an fp32 angle would
// already be off by ~1e-2 rad; the fp64 work (D/2 sincos per token and 4 FMAs
// per pair per head) hides under the HBM traffic.
#include "common.hpp"
#include "kernels.hpp"

namespace la {
namespace {

template <typename T>
__device__ __forceinline__ void load8f(const T* p, float* x);
template <>
__device__ __forceinline__ void load8f<__bf16>(const __bf16* p, float* x) {
  const bf16x8 v = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = (float)v[i];
}
template <>
__device__ __forceinline__ void load8f<float>(const float* p, float* x) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = a[i];
    x[i + 4] = b[i];
  }
}

template <typename T>
__device__ __forceinline__ void store8f(T* p, const float* x);
template <>
__device__ __forceinline__ void store8f<__bf16>(__bf16* p, const float* x) {
  bf16x8 v;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = to_bf16(x[i]);
  *reinterpret_cast<bf16x8*>(p) = v;
}
template <>
__device__ __forceinline__ void store8f<float>(float* p, const float* x) {
  f32x4 a = {x[0], x[1], x[2], x[3]};
  f32x4 b = {x[4], x[5], x[6], x[7]};
  *reinterpret_cast<f32x4*>(p) = a;
  *reinterpret_cast<f32x4*>(p + 4) = b;
}

template <typename T, int D>
__device__ __forceinline__ void rotate_heads(const RopeArgs& a, int b, int s, int c, int h0,
                                             int hstep, const double* cs, const double* sn) {
  if (a.in == nullptr) return;
  const T* in = static_cast<const T*>(a.in) + b * a.is_b + s * a.is_s + 8 * c;
  T* out = static_cast<T*>(a.out) + b * a.os_b + s * a.os_s + 8 * c;
  for (int h = h0; h < a.H; h += hstep) {
    float x[8], y[8];
    load8f<T>(in + h * a.is_h, x);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const double x0 = x[2 * p], x1 = x[2 * p + 1];
      y[2 * p] = (float)fma(x0, cs[p], -x1 * sn[p]);
      y[2 * p + 1] = (float)fma(x0, sn[p], x1 * cs[p]);
    }
    store8f<T>(out + h * a.os_h, y);
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void rope_kernel(RopeArgs qa, RopeArgs ka) {
  constexpr int CH = D / 8;            // 16-byte chunks (4 pairs) per head row
  constexpr int HSTEP = 256 / CH;      // heads covered per pass of the workgroup
  __shared__ double lds_cos[D / 2], lds_sin[D / 2];
  const int tok = blockIdx.x;
  const int B = qa.in ? qa.B : ka.B;
  const int S = qa.in ? qa.S : ka.S;
  const int b = tok / S, s = tok - b * S;
  if (b >= B) return;
  if (threadIdx.x < D / 2) {
    const int32_t* positions = qa.in ? qa.positions : ka.positions;
    const double base = qa.in ? qa.base : ka.base;
    const double pos = positions ? (double)positions[b * S + s] : (double)s;
    const int k = threadIdx.x;
    const double theta = exp2(-(2.0 * k / D) * log2(base));
    const double ang = pos * theta;
    const double two_pi = 6.283185307179586476925286766559;
    const double r = ang - rint(ang / two_pi) * two_pi;   // in [-pi, pi]
    double sv, cv;
    sincos(r, &sv, &cv);
    lds_cos[k] = cv;
    lds_sin[k] = sv;
  }
  __syncthreads();
  const int c = threadIdx.x % CH;
  const int h0 = threadIdx.x / CH;
  double cs[4], sn[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    cs[p] = lds_cos[4 * c + p];
    sn[p] = lds_sin[4 * c + p];
  }
  rotate_heads<T, D>(qa, b, s, c, h0, HSTEP, cs, sn);
  rotate_heads<T, D>(ka, b, s, c, h0, HSTEP, cs, sn);
}

template <typename T, int D>
hipError_t launch_t(const RopeArgs& q, const RopeArgs& k, hipStream_t st) {
  const RopeArgs& any = q.in ? q : k;
  const long long ntok = (long long)any.B * any.S;
  hipLaunchKernelGGL((rope_kernel<T, D>), dim3((unsigned)ntok), dim3(256), 0, st, q, k);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rope_pair(const RopeArgs& q, const RopeArgs& k, int D, int dt, hipStream_t st) {
  if (dt == 0) return D == 64 ? launch_t<__bf16, 64>(q, k, st) : launch_t<__bf16, 128>(q, k, st);
  return D == 64 ? launch_t<float, 64>(q, k, st) : launch_t<float, 128>(q, k, st);
}

}  // namespace la
