// Optional per-head steps between the projections and the scores, in place on
// the workspace Q and K (B, n, T, d):
//  * query/key normalisation (vit-pytorch simple_vit_with_qk_norm.py, class
//    RMSNorm): x / max(||x||_2, 1e-12) * sqrt(d) * gamma[head];
//  * rotary embedding over the token index t (HNDL attention operator,
//    "Rotary embeddings"): rotate-half over the full head, element i paired
//    with i + d/2, angle t * theta_i with theta_i = 10000^(-2i/d); theta is a
//    table rounded to float32 on the host and the angle one float32 product,
//    the float32 construction the page describes.
// Normalisation comes first, then the rotation (which keeps norms).
//
// General kernel: one group of P lanes (P a power of two >= ceil(d/2)) owns
// one (token, head) row; lane i holds elements i and i + ceil(d/2).  The
// squared norm is summed over the group with lane shuffles.
// bf16 kernel for d % 8 == 0: one group of P lanes owns one (sample, token)
// and walks the 2n rows of Q and K that share it (every head), lane j holding
// elements 4j..4j+3 and d/2 + 4j..4j+3 as 8-byte vectors; the rotation's
// sines and cosines depend only on (token, element), so a lane forms its four
// once for all 2n rows.  The bf16 queries arrive multiplied by
// log2(e)/sqrt(d) (the attention kernel's score scale): normalisation removes
// that factor, so normalised bf16 queries are multiplied by log2(e) (scores in
// the log2 domain, no 1/sqrt(d)); the rotation is linear and keeps it.
#include <math.h>

#include "ssa_internal.h"

namespace ssa {
namespace {

constexpr int kMaxHalf = 64;  // d <= 128

struct QkPostParams {
  void* q;             // (B, n, T, d)
  void* k;
  const void* gq;      // (n, d) or NULL
  const void* gk;
  int T, n, d, hd;     // hd = ceil(d / 2)
  int rows;            // B * n * T rows in each of Q and K
  int rope;
  float qmul;          // extra factor on normalised queries (log2(e) for bf16, 1 for fp32)
  float theta[kMaxHalf];
};

template <typename T, int P>
__global__ __launch_bounds__(256) void qk_post_kernel(QkPostParams pp) {
  const int tid = threadIdx.x;
  const int i = tid % P;
  const int grow = blockIdx.x * (256 / P) + tid / P;  // Q rows, then K rows
  const bool live = grow < 2 * pp.rows;               // uniform over the P-lane group
  const bool isq = grow < pp.rows;
  const int row = live ? (isq ? grow : grow - pp.rows) : 0;
  T* base = static_cast<T*>(isq ? pp.q : pp.k) + int64_t(row) * pp.d;
  const int t = row % pp.T;
  const int head = (row / pp.T) % pp.n;
  const int hd = pp.hd, d = pp.d;
  const bool ha = live && i < hd, hb = live && i < hd && i + hd < d;
  float a = ha ? to_f32(base[i]) : 0.f;
  float b = hb ? to_f32(base[i + hd]) : 0.f;
  const T* g = static_cast<const T*>(isq ? pp.gq : pp.gk);
  if (g != nullptr) {
    float ss = a * a + b * b;
#pragma unroll
    for (int m = P / 2; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, P);
    const float f = sqrtf(float(d)) / fmaxf(sqrtf(ss), 1e-12f) * (isq ? pp.qmul : 1.f);
    if (ha) a *= f * to_f32(g[head * d + i]);
    if (hb) b *= f * to_f32(g[head * d + i + hd]);
  }
  if (pp.rope && ha) {
    const float ang = float(t) * pp.theta[i];
    float sn, cs;
    sincosf(ang, &sn, &cs);
    const float na = a * cs - b * sn, nb = b * cs + a * sn;
    a = na;
    b = nb;
  }
  if (ha) base[i] = from_f32<T>(a);
  if (hb) base[i + hd] = from_f32<T>(b);
}

template <int P>
__global__ __launch_bounds__(256) void qk_post_bf16_kernel(QkPostParams pp) {
  const int tid = threadIdx.x;
  const int j = tid % P;                          // this lane's element chunk
  const int item = blockIdx.x * (256 / P) + tid / P;  // (b, t)
  const int hd = pp.hd, d = pp.d, n = pp.n, T = pp.T;
  const int nitems = pp.rows / n;                 // B * T
  if (item >= nitems) return;                     // whole groups leave together
  const bool act = 4 * j < hd;
  const int b = item / T, t = item - b * T;
  const int i = act ? 4 * j : 0;
  float cs[4] = {1.f, 1.f, 1.f, 1.f}, sn[4] = {0.f, 0.f, 0.f, 0.f};
  if (pp.rope) {
#pragma unroll
    for (int e = 0; e < 4; ++e) sincosf(float(t) * pp.theta[i + e], &sn[e], &cs[e]);
  }
  const bf16* gq = static_cast<const bf16*>(pp.gq);
  const bf16* gk = static_cast<const bf16*>(pp.gk);
  for (int r = 0; r < 2 * n; ++r) {
    const bool isq = r < n;
    const int head = isq ? r : r - n;
    bf16* base = static_cast<bf16*>(isq ? pp.q : pp.k) + ((int64_t(b) * n + head) * T + t) * d;
    bf16x4 va = {}, vb = {};
    if (act) {
      va = *reinterpret_cast<const bf16x4*>(base + i);
      vb = *reinterpret_cast<const bf16x4*>(base + hd + i);
    }
    float a[4], c[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a[e] = static_cast<float>(va[e]);
      c[e] = static_cast<float>(vb[e]);
    }
    if (gq != nullptr) {
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) ss += a[e] * a[e] + c[e] * c[e];
#pragma unroll
      for (int m = P / 2; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, P);
      const float f = sqrtf(float(d)) / fmaxf(sqrtf(ss), 1e-12f) * (isq ? pp.qmul : 1.f);
      if (act) {
        const bf16* g = (isq ? gq : gk) + head * d;
        const bf16x4 ga = *reinterpret_cast<const bf16x4*>(g + i);
        const bf16x4 gb = *reinterpret_cast<const bf16x4*>(g + hd + i);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[e] *= f * static_cast<float>(ga[e]);
          c[e] *= f * static_cast<float>(gb[e]);
        }
      }
    }
    if (pp.rope) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float na = a[e] * cs[e] - c[e] * sn[e], nc = c[e] * cs[e] + a[e] * sn[e];
        a[e] = na;
        c[e] = nc;
      }
    }
    if (act) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        va[e] = static_cast<bf16>(a[e]);
        vb[e] = static_cast<bf16>(c[e]);
      }
      *reinterpret_cast<bf16x4*>(base + i) = va;
      *reinterpret_cast<bf16x4*>(base + hd + i) = vb;
    }
  }
}

template <typename T>
hipError_t launch_typed(const QkPostParams& pp, hipStream_t stream) {
  const int hd = pp.hd;
  const int P = hd <= 2 ? 2 : hd <= 4 ? 4 : hd <= 8 ? 8 : hd <= 16 ? 16 : hd <= 32 ? 32 : 64;
  const int64_t rows2 = 2 * int64_t(pp.rows);
  const unsigned grid = unsigned((rows2 * P + 255) / 256);
  switch (P) {
    case 2: qk_post_kernel<T, 2><<<grid, 256, 0, stream>>>(pp); break;
    case 4: qk_post_kernel<T, 4><<<grid, 256, 0, stream>>>(pp); break;
    case 8: qk_post_kernel<T, 8><<<grid, 256, 0, stream>>>(pp); break;
    case 16: qk_post_kernel<T, 16><<<grid, 256, 0, stream>>>(pp); break;
    case 32: qk_post_kernel<T, 32><<<grid, 256, 0, stream>>>(pp); break;
    default: qk_post_kernel<T, 64><<<grid, 256, 0, stream>>>(pp); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qk_post(const Plan& p, const Args& a) {
  QkPostParams pp{};
  pp.q = a.ws + p.ws.q;
  pp.k = a.ws + p.ws.k;
  pp.gq = a.q_norm_gamma;
  pp.gk = a.k_norm_gamma;
  pp.T = int(p.T);
  pp.n = int(p.n);
  pp.d = int(p.d);
  pp.hd = int((p.d + 1) / 2);
  pp.rows = int(p.B * p.n * p.T);
  pp.rope = a.rope ? 1 : 0;
  pp.qmul = p.dtype == SSA_BF16 ? 1.4426950408889634f : 1.f;
  for (int i = 0; i < pp.hd && i < kMaxHalf; ++i)
    pp.theta[i] = float(pow(10000.0, -2.0 * double(i) / double(p.d)));
  if (p.dtype == SSA_BF16 && p.d % 8 == 0) {
    const int chunks = pp.hd / 4;  // 4, 8, 12 or 16
    const int P = chunks <= 4 ? 4 : chunks <= 8 ? 8 : 16;
    const int64_t items = p.B * p.T;
    const unsigned grid = unsigned((items * P + 255) / 256);
    switch (P) {
      case 4: qk_post_bf16_kernel<4><<<grid, 256, 0, a.stream>>>(pp); break;
      case 8: qk_post_bf16_kernel<8><<<grid, 256, 0, a.stream>>>(pp); break;
      default: qk_post_bf16_kernel<16><<<grid, 256, 0, a.stream>>>(pp); break;
    }
    return hipGetLastError();
  }
  return p.dtype == SSA_F32 ? launch_typed<float>(pp, a.stream) : launch_typed<bf16>(pp, a.stream);
}

}  // namespace ssa
