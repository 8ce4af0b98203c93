// GroupNorm statistics (tensortonic "Spatial Self-Attention": GN with
// num_groups groups, eps 1e-5, affine norm_weight / norm_bias).
//
// Group g of sample b is channels g*C/G .. (g+1)*C/G-1 over all pixels, which
// in NCHW is ONE contiguous run of (C/G)*T elements.  The pass is HBM-bound.
//
//   gn_stats_kernel<FINAL>  grid B*G*splits: each work-group streams one chunk
//       of a segment with 16-byte loads (four in flight per thread).  A thread
//       accumulates shifted sums, d = x - x0 with x0 the chunk's first element
//       (sum d and sum d^2: no division in the loop, and little cancellation
//       because x0 is a sample of the same data); the (count, mean, M2) of the
//       threads are then merged with Chan's pairwise update (wave -> block).
//       FINAL (one chunk per segment): the same work-group forms mean and
//       rstd = 1/sqrt(M2/count + eps) (biased variance) and the per-channel
//       coefficients a = gamma*rstd, s = beta - mean*a, so that the projection
//       prologue normalises with one FMA.  Otherwise it writes its chunk's
//       (count, mean, M2) and
//   gn_finalize_kernel      grid B*G: one wave merges the chunks of a segment
//       and emits the same statistics and coefficients.
//   gn_stats_wave_kernel    many short segments: one wave per segment.
//   gn_seg_kernel           long segments, at least a quarter as many as CUs:
//       one 512-thread work-group per segment with eight 16-byte loads in
//       flight per thread, finalising in place (one kernel instead of the split
//       pass and its merge).
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

// mean / rstd of one segment and its per-channel coefficients (all threads
// of the work-group call it; threads 0.. write).
template <typename T>
__device__ __forceinline__ void finalize(Moments m, int seg, const T* __restrict__ gamma,
                                         const T* __restrict__ beta, float2* __restrict__ stats,
                                         float2* __restrict__ coef, int G, int Cg, int C,
                                         int tid, int nthreads) {
  const float var = m.m2 / m.n;
  const float rstd = 1.0f / sqrtf(var + kGnEps);
  if (tid == 0) stats[seg] = make_float2(m.mean, rstd);
  const int b = seg / G, g = seg % G;
  for (int c = tid; c < Cg; c += nthreads) {
    const int ch = g * Cg + c;
    const float a = to_f32(gamma[ch]) * rstd;
    coef[int64_t(b) * C + ch] = make_float2(a, to_f32(beta[ch]) - m.mean * a);
  }
}

template <typename T, int VEC, bool FINAL>
__global__ __launch_bounds__(256) void gn_stats_kernel(const T* __restrict__ x,
                                                       float4* __restrict__ partial,
                                                       int64_t seg_len, int64_t chunk, int splits,
                                                       const T* __restrict__ gamma,
                                                       const T* __restrict__ beta,
                                                       float2* __restrict__ stats,
                                                       float2* __restrict__ coef, int G, int Cg,
                                                       int C) {
  const int tid = threadIdx.x;
  const int s = int(blockIdx.x % unsigned(splits));
  const int64_t seg = blockIdx.x / unsigned(splits);
  const int64_t begin = int64_t(s) * chunk;
  const int64_t end = min(begin + chunk, seg_len);
  const T* base = x + seg * seg_len;
  const float x0 = to_f32(base[begin]);
  float sd = 0.f, sq = 0.f;
  int64_t cnt = 0;
  if constexpr (VEC > 1) {
    typedef typename VecOf<T, VEC>::type V;
    const V* vb = reinterpret_cast<const V*>(base);
    const int64_t v0 = begin / VEC, v1 = end / VEC;
    int64_t i = v0 + tid;
    for (; i + 3 * 256 < v1; i += 4 * 256) {  // four independent 16-byte loads in flight
      V v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = vb[i + u * 256];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const float d = to_f32(v[u][e]) - x0;
          sd += d;
          sq = fmaf(d, d, sq);
        }
      cnt += 4 * VEC;
    }
    for (; i < v1; i += 256) {
      const V v = vb[i];
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float d = to_f32(v[e]) - x0;
        sd += d;
        sq = fmaf(d, d, sq);
      }
      cnt += VEC;
    }
  } else {
    for (int64_t i = begin + tid; i < end; i += 256) {
      const float d = to_f32(base[i]) - x0;
      sd += d;
      sq = fmaf(d, d, sq);
      ++cnt;
    }
  }
  Moments acc{0.f, 0.f, 0.f};
  if (cnt > 0) {
    const float n = float(cnt);
    const float md = sd / n;
    acc = Moments{n, x0 + md, fmaxf(sq - sd * md, 0.f)};
  }
  acc = wave_merge(acc);
  __shared__ Moments waves[4];
  const int wave = tid / 64;
  if ((tid & 63) == 0) waves[wave] = acc;
  __syncthreads();
  Moments r = merge(merge(waves[0], waves[1]), merge(waves[2], waves[3]));
  if constexpr (FINAL) {
    finalize<T>(r, int(seg), gamma, beta, stats, coef, G, Cg, C, tid, 256);
  } else {
    if (tid == 0) partial[seg * splits + s] = make_float4(r.n, r.mean, r.m2, 0.f);
  }
}

// Many short segments (at most kWaveSeg elements, at least four per CU): one
// wave per segment, four per work-group, every load of a lane issued before
// the sums; the merge is the wave's alone (no LDS, no barrier).  A quarter of
// the work-groups of one-per-segment, which matters when the segments are
// small and the launch is mostly latency.
constexpr int kWaveSeg = 4096;

template <typename T, int VEC>
__global__ __launch_bounds__(256) void gn_stats_wave_kernel(const T* __restrict__ x, int64_t segs,
                                                            int seg_len,
                                                            const T* __restrict__ gamma,
                                                            const T* __restrict__ beta,
                                                            float2* __restrict__ stats,
                                                            float2* __restrict__ coef, int G,
                                                            int Cg, int C) {
  typedef typename VecOf<T, VEC>::type V;
  constexpr int NV = kWaveSeg / VEC / 64;  // vectors per lane at most
  const int lane = threadIdx.x & 63;
  const int64_t seg = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (seg >= segs) return;  // whole waves
  const V* vb = reinterpret_cast<const V*>(x + seg * seg_len);
  const int nv = seg_len / VEC;
  const float x0 = to_f32(x[seg * seg_len]);
  V v[NV];
#pragma unroll
  for (int u = 0; u < NV; ++u)
    if (lane + 64 * u < nv) v[u] = vb[lane + 64 * u];
  float sd = 0.f, sq = 0.f;
  int cnt = 0;
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    if (lane + 64 * u < nv) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float d = to_f32(v[u][e]) - x0;
        sd += d;
        sq = fmaf(d, d, sq);
      }
      cnt += VEC;
    }
  }
  Moments acc{0.f, 0.f, 0.f};
  if (cnt > 0) {
    const float n = float(cnt);
    const float md = sd / n;
    acc = Moments{n, x0 + md, fmaxf(sq - sd * md, 0.f)};
  }
  acc = wave_merge(acc);
  finalize<T>(acc, int(seg), gamma, beta, stats, coef, G, Cg, C, lane, 64);
}

// One work-group of NT threads per segment, UNR 16-byte loads in flight per
// thread; the waves' (count, mean, M2) merged through LDS, then finalised.
template <typename T, int VEC, int NT, int UNR>
__global__ __launch_bounds__(NT) void gn_seg_kernel(const T* __restrict__ x, int64_t seg_len,
                                                    const T* __restrict__ gamma,
                                                    const T* __restrict__ beta,
                                                    float2* __restrict__ stats,
                                                    float2* __restrict__ coef, int G, int Cg, int C) {
  typedef typename VecOf<T, VEC>::type V;
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x;
  const int64_t seg = blockIdx.x;
  const T* base = x + seg * seg_len;
  const float x0 = to_f32(base[0]);
  const V* vb = reinterpret_cast<const V*>(base);
  const int64_t nv = seg_len / VEC;
  float sd = 0.f, sq = 0.f;
  int cnt = 0;
  int64_t i = tid;
  for (; i + (UNR - 1) * NT < nv; i += UNR * NT) {
    V v[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u) v[u] = vb[i + u * NT];
#pragma unroll
    for (int u = 0; u < UNR; ++u)
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float d = to_f32(v[u][e]) - x0;
        sd += d;
        sq = fmaf(d, d, sq);
      }
    cnt += UNR * VEC;
  }
  for (; i < nv; i += NT) {
    const V v = vb[i];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const float d = to_f32(v[e]) - x0;
      sd += d;
      sq = fmaf(d, d, sq);
    }
    cnt += VEC;
  }
  Moments acc{0.f, 0.f, 0.f};
  if (cnt > 0) {
    const float n = float(cnt);
    const float md = sd / n;
    acc = Moments{n, x0 + md, fmaxf(sq - sd * md, 0.f)};
  }
  acc = wave_merge(acc);
  __shared__ Moments waves[NW];
  const int wave = tid / 64;
  if ((tid & 63) == 0) waves[wave] = acc;
  __syncthreads();
  Moments r = waves[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) r = merge(r, waves[w]);
  finalize<T>(r, int(seg), gamma, beta, stats, coef, G, Cg, C, tid, NT);
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
  finalize<T>(acc, seg, gamma, beta, stats, coef, G, Cg, C, lane, 64);
}

template <typename T, int VEC>
hipError_t launch_vec(const Plan& p, const Args& a) {
  const T* x = static_cast<const T*>(a.x);
  float4* partial = reinterpret_cast<float4*>(a.ws + p.ws.gn_partial);
  float2* stats = reinterpret_cast<float2*>(a.ws + p.ws.gn_stats);
  float2* coef = reinterpret_cast<float2*>(a.ws + p.ws.gn_coef);
  const T* gamma = static_cast<const T*>(a.norm_weight);
  const T* beta = static_cast<const T*>(a.norm_bias);
  const int G = int(p.G), Cg = int(p.C / p.G), C = int(p.C);
  dim3 grid(unsigned(p.splits * p.B * p.G));
  if constexpr (VEC > 1) {
    if (p.gn_seg) {
      gn_seg_kernel<T, VEC, 512, 8><<<dim3(unsigned(p.B * p.G)), 512, 0, a.stream>>>(
          x, p.seg_len, gamma, beta, stats, coef, G, Cg, C);
      return hipGetLastError();
    }
    if (p.splits == 1 && p.seg_len <= kWaveSeg && p.B * p.G >= 4 * int64_t(p.cus)) {
      const int64_t segs = p.B * p.G;
      gn_stats_wave_kernel<T, VEC><<<dim3(unsigned((segs + 3) / 4)), 256, 0, a.stream>>>(
          x, segs, int(p.seg_len), gamma, beta, stats, coef, G, Cg, C);
      return hipGetLastError();
    }
  }
  if (p.splits == 1) {
    gn_stats_kernel<T, VEC, true><<<grid, 256, 0, a.stream>>>(x, partial, p.seg_len, p.chunk, 1,
                                                              gamma, beta, stats, coef, G, Cg, C);
    return hipGetLastError();
  }
  gn_stats_kernel<T, VEC, false><<<grid, 256, 0, a.stream>>>(x, partial, p.seg_len, p.chunk,
                                                             int(p.splits), gamma, beta, stats,
                                                             coef, G, Cg, C);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  gn_finalize_kernel<T><<<dim3(unsigned(p.B * p.G)), 64, 0, a.stream>>>(
      partial, int(p.splits), gamma, beta, stats, coef, G, Cg, C);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_typed(const Plan& p, const Args& a) {
  constexpr int kVec = 16 / sizeof(T);
  return p.gn_vec == kVec ? launch_vec<T, kVec>(p, a) : launch_vec<T, 1>(p, a);
}

}  // namespace

hipError_t launch_gn_stats(const Plan& p, const Args& a) {
  return p.dtype == SSA_F32 ? launch_typed<float>(p, a) : launch_typed<bf16>(p, a);
}

}  // namespace ssa
