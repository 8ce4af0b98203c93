// Optional per-head steps between the projections and the scores:
//  * query/key normalisation (vit-pytorch simple_vit_with_qk_norm.py, class
//    RMSNorm): x / max(||x||_2, 1e-12) * sqrt(d) * gamma[head];
//  * rotary embedding over the token index t (HNDL attention operator,
//    "Rotary embeddings"): rotate-half over the full head, element i paired
//    with i + d/2, angle t * theta_i with theta_i = 10000^(-2i/d); theta is a
//    table rounded to float32 on the host and the angle one float32 product,
//    the float32 construction the page describes.
// Normalisation comes first, then the rotation (which keeps norms).
//
// Where the QKV projection's epilogue applies both steps itself (bf16, head
// sizes 16, 32, 64, 128 on its main path), this file only provides the
// rotation's (cos, sin) table for it.  Otherwise the projection leaves Q and
// K unrounded -- fp32 in the qk32 region (bf16 problems) or in the fp32 q / k
// layouts themselves -- and qk_post_kernel applies the steps and writes the q
// and k layouts, so that bf16 Q and K are rounded once.
//
// Also here: zeroing the padding columns d .. dp-1 of bf16 q and k (heads
// narrower than the attention kernels' operand width), which keeps every
// score unchanged.
#include <math.h>

#include "ssa_internal.h"

namespace ssa {
namespace {

constexpr int kMaxHalf = 64;  // d <= 128
constexpr float kLog2e = 1.4426950408889634f;

// theta_i = 10000^(-2i/d) rounded to float32 (double on the host, as the
// angles of the page are built), i < ceil(d/2).
void fill_theta(float* theta, int64_t d) {
  const int64_t hd = (d + 1) / 2;
  for (int64_t i = 0; i < hd && i < kMaxHalf; ++i)
    theta[i] = float(pow(10000.0, -2.0 * double(i) / double(d)));
}

struct RopeTabParams {
  float2* tab;  // (T, d/2): (cos, sin) of t * theta_i
  int T, hd;
  float theta[kMaxHalf];
};

// One thread per table entry (t, i), i fastest, so that the stores are
// consecutive; theta is staged in LDS for the per-lane index.
__global__ __launch_bounds__(256) void rope_table_kernel(RopeTabParams rp) {
  __shared__ float th[kMaxHalf];
  if (int(threadIdx.x) < rp.hd) th[threadIdx.x] = rp.theta[threadIdx.x];
  __syncthreads();
  const int64_t total = int64_t(rp.T) * rp.hd;
  for (int64_t e = int64_t(blockIdx.x) * 256 + threadIdx.x; e < total; e += int64_t(gridDim.x) * 256) {
    const int t = int(e / rp.hd), i = int(e - int64_t(t) * rp.hd);
    const float ang = float(t) * th[i];  // one float32 product
    float s, c;
    sincosf(ang, &s, &c);
    rp.tab[e] = make_float2(c, s);
  }
}

struct ZeroPadParams {
  bf16* q;
  bf16* k;
  int64_t rows;  // B * n * T rows in each of q and k
  int d, dp;
};

// One thread per (row, padding element) of q, then of k.
__global__ __launch_bounds__(256) void zero_pad_kernel(ZeroPadParams zp) {
  const int w = zp.dp - zp.d;
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= 2 * zp.rows * w) return;
  const int64_t r = i / w;
  const int c = zp.d + int(i - r * w);
  bf16* base = r < zp.rows ? zp.q + r * zp.dp : zp.k + (r - zp.rows) * zp.dp;
  base[c] = static_cast<bf16>(0.f);
}

struct QkPostParams {
  const float* sq;     // (B, n, T, d) fp32 Q and K as projected (bias added, unscaled)
  const float* sk;
  void* q;             // destination layouts (B, n, T, dp)
  void* k;
  const void* gq;      // (n, d) or NULL
  const void* gk;
  int T, n, d, dp, hd; // hd = ceil(d / 2)
  int rows;            // B * n * T rows in each of Q and K
  int rope;
  float qmul;          // factor on the stored queries (bf16: the score scale in log2 units)
  float theta[kMaxHalf];
};

// One group of P lanes (P a power of two >= ceil(d/2)) per (token, head) row;
// lane i holds elements i and i + ceil(d/2); the squared norm is summed over
// the group with lane shuffles.  Reads fp32, writes DT once.
template <typename DT, int P>
__global__ __launch_bounds__(256) void qk_post_kernel(QkPostParams pp) {
  const int tid = threadIdx.x;
  const int i = tid % P;
  const int grow = blockIdx.x * (256 / P) + tid / P;  // Q rows, then K rows
  const bool live = grow < 2 * pp.rows;               // uniform over the P-lane group
  const bool isq = grow < pp.rows;
  const int row = live ? (isq ? grow : grow - pp.rows) : 0;
  const float* src = (isq ? pp.sq : pp.sk) + int64_t(row) * pp.d;
  DT* dst = static_cast<DT*>(isq ? pp.q : pp.k) + int64_t(row) * pp.dp;
  const int t = row % pp.T;
  const int head = (row / pp.T) % pp.n;
  const int hd = pp.hd, d = pp.d;
  const bool ha = live && i < hd, hb = live && i < hd && i + hd < d;
  float a = ha ? src[i] : 0.f;
  float b = hb ? src[i + hd] : 0.f;
  const DT* g = static_cast<const DT*>(isq ? pp.gq : pp.gk);
  if (g != nullptr) {
    float ss = a * a + b * b;
#pragma unroll
    for (int m = P / 2; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, P);
    const float f = sqrtf(float(d)) / fmaxf(sqrtf(ss), 1e-12f);
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
  const float sc = isq ? pp.qmul : 1.f;
  if (ha) dst[i] = from_f32<DT>(a * sc);
  if (hb) dst[i + hd] = from_f32<DT>(b * sc);
}

template <typename DT>
hipError_t launch_typed(const QkPostParams& pp, hipStream_t stream) {
  const int hd = pp.hd;
  const int P = hd <= 2 ? 2 : hd <= 4 ? 4 : hd <= 8 ? 8 : hd <= 16 ? 16 : hd <= 32 ? 32 : 64;
  const int64_t rows2 = 2 * int64_t(pp.rows);
  const unsigned grid = unsigned((rows2 * P + 255) / 256);
  switch (P) {
    case 2: qk_post_kernel<DT, 2><<<grid, 256, 0, stream>>>(pp); break;
    case 4: qk_post_kernel<DT, 4><<<grid, 256, 0, stream>>>(pp); break;
    case 8: qk_post_kernel<DT, 8><<<grid, 256, 0, stream>>>(pp); break;
    case 16: qk_post_kernel<DT, 16><<<grid, 256, 0, stream>>>(pp); break;
    case 32: qk_post_kernel<DT, 32><<<grid, 256, 0, stream>>>(pp); break;
    default: qk_post_kernel<DT, 64><<<grid, 256, 0, stream>>>(pp); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qk_post(const Plan& p, const Args& a) {
  QkPostParams pp{};
  const int64_t rows = p.B * p.n * p.T;
  if (p.dtype == SSA_BF16) {
    const float* s = reinterpret_cast<const float*>(a.ws + p.ws.qk32);
    pp.sq = s;
    pp.sk = s + rows * p.d;
  } else {  // fp32: in place on the q / k layouts (dp = d)
    pp.sq = reinterpret_cast<const float*>(a.ws + p.ws.q);
    pp.sk = reinterpret_cast<const float*>(a.ws + p.ws.k);
  }
  pp.q = a.ws + p.ws.q;
  pp.k = a.ws + p.ws.k;
  pp.gq = a.q_norm_gamma;
  pp.gk = a.k_norm_gamma;
  pp.T = int(p.T);
  pp.n = int(p.n);
  pp.d = int(p.d);
  pp.dp = int(p.dp);
  pp.hd = int((p.d + 1) / 2);
  pp.rows = int(rows);
  pp.rope = a.rope ? 1 : 0;
  // bf16 queries carry the score scale (log2 units; no 1/sqrt(d) after the
  // normalisation); the fp32 attention kernel applies it itself
  pp.qmul = p.dtype == SSA_BF16
                ? (a.q_norm_gamma != nullptr ? kLog2e : kLog2e / sqrtf(float(p.d)))
                : 1.f;
  fill_theta(pp.theta, p.d);
  return p.dtype == SSA_F32 ? launch_typed<float>(pp, a.stream) : launch_typed<bf16>(pp, a.stream);
}

hipError_t launch_rope_table(const Plan& p, const Args& a) {
  RopeTabParams rp{};
  rp.tab = reinterpret_cast<float2*>(a.ws + p.ws.rope);
  rp.T = int(p.T);
  rp.hd = int(p.d / 2);
  fill_theta(rp.theta, p.d);
  const int64_t total = p.T * int64_t(rp.hd);
  const int64_t blocks = (total + 255) / 256;
  rope_table_kernel<<<dim3(unsigned(blocks < 4096 ? blocks : 4096)), 256, 0, a.stream>>>(rp);
  return hipGetLastError();
}

hipError_t launch_zero_pad(const Plan& p, const Args& a) {
  ZeroPadParams zp{};
  zp.q = reinterpret_cast<bf16*>(a.ws + p.ws.q);
  zp.k = reinterpret_cast<bf16*>(a.ws + p.ws.k);
  zp.rows = p.B * p.n * p.T;
  zp.d = int(p.d);
  zp.dp = int(p.dp);
  const int64_t total = 2 * zp.rows * (zp.dp - zp.d);
  zero_pad_kernel<<<dim3(unsigned((total + 255) / 256)), 256, 0, a.stream>>>(zp);
  return hipGetLastError();
}

}  // namespace ssa
