// GroupNorm statistics (tensortonic "Spatial Self-Attention": GN with
// num_groups groups, eps 1e-5, affine norm_weight / norm_bias).
//
// Group g of sample b is channels g*C/G .. (g+1)*C/G-1 over all pixels, which
// in NCHW is ONE contiguous run of (C/G)*T elements.  The pass is HBM-bound:
//
//   gn_partial_kernel   grid B*G*splits: each work-group streams one chunk
//                       of a segment with 16-byte loads and produces
//                       (count, mean, M2) of that chunk.  Per vector the mean
//                       and M2 are formed two-pass in registers, then merged
//                       with Chan's pairwise update (thread -> wave -> block).
//   gn_finalize_kernel  grid (B*G): one wave merges the chunks of a segment,
//                       forms mean and rstd = 1/sqrt(M2/count + eps) (biased
//                       variance), and emits per-channel coefficients
//                       a = gamma*rstd, s = beta - mean*a, so that the
//                       projection prologue normalises with one FMA.
#include "ssa_internal.h"

namespace ssa {
namespace {

struct Moments {
  float n, mean, m2;
};

__device__ __forceinline__ Moments merge(Moments a, Moments b) {
  const float n = a.n + b.n;
  if (n == 0.f) return a;
  const float delta = b.mean - a.mean;
  const float fb = b.n / n;
  Moments r;
  r.n = n;
  r.mean = a.mean + delta * fb;
  r.m2 = a.m2 + b.m2 + delta * delta * a.n * fb;
  return r;
}

__device__ __forceinline__ Moments shfl_xor(Moments m, int mask) {
  Moments r;
  r.n = __shfl_xor(m.n, mask, 64);
  r.mean = __shfl_xor(m.mean, mask, 64);
  r.m2 = __shfl_xor(m.m2, mask, 64);
  return r;
}

__device__ __forceinline__ Moments wave_merge(Moments m) {
#pragma unroll
  for (int mask = 32; mask >= 1; mask >>= 1) m = merge(m, shfl_xor(m, mask));
  return m;
}

template <typename T, int VEC>
struct VecOf;
template <>
struct VecOf<float, 4> { typedef f32x4 type; };
template <>
struct VecOf<bf16, 8> { typedef bf16x8 type; };

template <typename T, int VEC>
__global__ __launch_bounds__(256) void gn_partial_kernel(const T* __restrict__ x,
                                                         float4* __restrict__ partial,
                                                         int64_t seg_len, int64_t chunk,
                                                         int splits) {
  const int s = int(blockIdx.x % unsigned(splits));
  const int64_t seg = blockIdx.x / unsigned(splits);
  const int64_t begin = int64_t(s) * chunk;
  const int64_t end = min(begin + chunk, seg_len);
  const T* base = x + seg * seg_len;
  Moments acc{0.f, 0.f, 0.f};
  if constexpr (VEC > 1) {
    typedef typename VecOf<T, VEC>::type V;
    const V* vb = reinterpret_cast<const V*>(base);
    for (int64_t i = begin / VEC + threadIdx.x; i < end / VEC; i += 256) {
      V v = vb[i];
      float f[VEC];
      float sum = 0.f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        f[e] = to_f32(v[e]);
        sum += f[e];
      }
      Moments m;
      m.n = float(VEC);
      m.mean = sum * (1.f / VEC);
      m.m2 = 0.f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) m.m2 += (f[e] - m.mean) * (f[e] - m.mean);
      acc = merge(acc, m);
    }
  } else {
    for (int64_t i = begin + threadIdx.x; i < end; i += 256) {
      Moments m{1.f, to_f32(base[i]), 0.f};
      acc = merge(acc, m);
    }
  }
  acc = wave_merge(acc);
  __shared__ Moments waves[4];
  const int wave = threadIdx.x / 64;
  if ((threadIdx.x & 63) == 0) waves[wave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    Moments r = waves[0];
    r = merge(r, waves[1]);
    r = merge(r, waves[2]);
    r = merge(r, waves[3]);
    partial[seg * splits + s] = make_float4(r.n, r.mean, r.m2, 0.f);
  }
}

template <typename T>
__global__ __launch_bounds__(64) void gn_finalize_kernel(const float4* __restrict__ partial,
                                                         int splits, const T* __restrict__ gamma,
                                                         const T* __restrict__ beta,
                                                         float2* __restrict__ stats,
                                                         float2* __restrict__ coef, int G,
                                                         int Cg, int C) {
  const int seg = blockIdx.x;  // b*G + g
  const int lane = threadIdx.x;
  Moments acc{0.f, 0.f, 0.f};
  for (int s = lane; s < splits; s += 64) {
    float4 q = partial[int64_t(seg) * splits + s];
    acc = merge(acc, Moments{q.x, q.y, q.z});
  }
  acc = wave_merge(acc);
  const float var = acc.m2 / acc.n;
  const float rstd = 1.0f / sqrtf(var + kGnEps);
  if (lane == 0) stats[seg] = make_float2(acc.mean, rstd);
  const int b = seg / G, g = seg % G;
  for (int c = lane; c < Cg; c += 64) {
    const int ch = g * Cg + c;
    const float a = to_f32(gamma[ch]) * rstd;
    coef[int64_t(b) * C + ch] = make_float2(a, to_f32(beta[ch]) - acc.mean * a);
  }
}

template <typename T>
hipError_t launch_typed(const Plan& p, const Args& a) {
  const T* x = static_cast<const T*>(a.x);
  float4* partial = reinterpret_cast<float4*>(a.ws + p.ws.gn_partial);
  float2* stats = reinterpret_cast<float2*>(a.ws + p.ws.gn_stats);
  float2* coef = reinterpret_cast<float2*>(a.ws + p.ws.gn_coef);
  dim3 grid(unsigned(p.splits * p.B * p.G));
  constexpr int kVec = 16 / sizeof(T);
  if (p.gn_vec == kVec)
    gn_partial_kernel<T, kVec><<<grid, 256, 0, a.stream>>>(x, partial, p.seg_len, p.chunk,
                                                           int(p.splits));
  else
    gn_partial_kernel<T, 1><<<grid, 256, 0, a.stream>>>(x, partial, p.seg_len, p.chunk,
                                                        int(p.splits));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  gn_finalize_kernel<T><<<dim3(unsigned(p.B * p.G)), 64, 0, a.stream>>>(
      partial, int(p.splits), static_cast<const T*>(a.norm_weight),
      static_cast<const T*>(a.norm_bias), stats, coef, int(p.G), int(p.C / p.G), int(p.C));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gn_stats(const Plan& p, const Args& a) {
  return p.dtype == SSA_F32 ? launch_typed<float>(p, a) : launch_typed<bf16>(p, a);
}

}  // namespace ssa
