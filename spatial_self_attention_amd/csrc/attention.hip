// Per-head attention O_j = softmax(Q_j K_j^T / sqrt(d)) V_j over all pixels
// (tensortonic "Spatial Self-Attention": formula; softmax over the key axis;
// scores divided by sqrt(d) as its first worked example states), computed
// flash-style: the T x T score matrix is never stored.  Each work-group owns
// one (sample, head, query tile), walks the key tiles once and keeps a running
// row max m and row sum l (online softmax):
//
//     m' = max(m, max_k s_k),  O <- O * 2^(m - m'),  l <- l * 2^(m - m') + sum 2^(s_k - m'),
//     O <- O + P V,            finally O / l,
//
// with the scores in the log2 domain (s = q.k * log2(e) / sqrt(d)).
//
// bf16 kernel (gfx950 MFMA): 4 waves x 32 queries, key tiles of 64.  The
// score block is formed TRANSPOSED, S^T = K Q^T with v_mfma_f32_32x32x16_bf16,
// so each lane holds one query (its column) and 16 keys per 32-key block:
//  * the row max / row sum need no shuffles except one exchange with lane^32
//    (the other half of the keys of the same query);
//  * the rescale by 2^(m - m') is per lane;
//  * the probabilities, rounded to bf16, are already in the register layout of
//    MFMA's B operand for O^T += V^T P^T, up to a permutation of the key
//    index that the V^T operand loads apply identically (a dot product does
//    not depend on the order of its terms).
// V is read from the transposed (d, Tp) layout, so each V^T operand is two
// 8-byte LDS reads.  O is written token-major (B, T, C), heads concatenated.
//
// fp32 kernel: 64 queries x 4 lanes per query (each lane owns d/4 dims),
// FMA only, key tiles of 32 in LDS.
#include <math.h>

#include "ssa_internal.h"

namespace ssa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

struct AttnParams {
  const void* q;   // (B, n, T, d)
  const void* k;   // (B, n, T, d)
  const void* vt;  // (B, n, d, Tp)
  void* o;         // (B, T, C)
  int T, Tp, n, d, C;
  int qtiles;      // query tiles per (b, head)
  float scale;     // log2(e) / sqrt(d)
};

// ---------------------------------------------------------------------------
// bf16 MFMA kernel
// ---------------------------------------------------------------------------
constexpr int QT = 128;  // queries per work-group
constexpr int KT = 64;   // keys per tile

template <int D>
__global__ __launch_bounds__(256) void attn_bf16_kernel(AttnParams ap) {
  constexpr int KP = D + 8;   // Ks row pitch (bf16)
  constexpr int VP = KT + 8;  // Vs row pitch (bf16)
  __shared__ __attribute__((aligned(16))) bf16 Ks[KT * KP];
  __shared__ __attribute__((aligned(16))) bf16 Vs[D * VP];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int qtile = blockIdx.x % ap.qtiles;
  const int bh = blockIdx.x / ap.qtiles;  // b * n + head
  const int head = bh % ap.n, b = bh / ap.n;
  const int T = ap.T;

  const bf16* Q = static_cast<const bf16*>(ap.q) + int64_t(bh) * T * D;
  const bf16* K = static_cast<const bf16*>(ap.k) + int64_t(bh) * T * D;
  const bf16* Vt = static_cast<const bf16*>(ap.vt) + int64_t(bh) * D * ap.Tp;

  const int qi = qtile * QT + wave * 32 + col;
  const bf16x8 zero8 = {};
  bf16x8 qf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
    qf[ks] = qi < T ? *reinterpret_cast<const bf16x8*>(Q + int64_t(qi) * D + ks * 16 + half * 8)
                    : zero8;

  f32x16 o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float sc = ap.scale;

  for (int k0 = 0; k0 < T; k0 += KT) {
    __syncthreads();  // previous tile fully consumed
    for (int v = tid; v < KT * D / 8; v += 256) {
      const int r = v / (D / 8), c8 = v % (D / 8);
      const int key = k0 + r;
      bf16x8 val = zero8;
      if (key < T) val = *reinterpret_cast<const bf16x8*>(K + int64_t(key) * D + c8 * 8);
      *reinterpret_cast<bf16x8*>(&Ks[r * KP + c8 * 8]) = val;
    }
    for (int v = tid; v < D * KT / 8; v += 256) {
      const int r = v / (KT / 8), c8 = v % (KT / 8);
      const int key = k0 + c8 * 8;
      const bf16* src = Vt + int64_t(r) * ap.Tp + key;
      bf16x8 val;
      if (key + 8 <= T) {
        val = *reinterpret_cast<const bf16x8*>(src);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) val[e] = key + e < T ? src[e] : static_cast<bf16>(0.f);
      }
      *reinterpret_cast<bf16x8*>(&Vs[r * VP + c8 * 8]) = val;
    }
    __syncthreads();

    // S^T block: lane (half, col) holds query col, keys kb*32 + 8*(r/4) + 4*half + r%4.
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const bf16x8 a =
            *reinterpret_cast<const bf16x8*>(&Ks[(kb * 32 + col) * KP + ks * 16 + half * 8]);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[kb], 0, 0, 0);
      }
    }
    float mx = -INFINITY;
    const bool tail = k0 + KT > T;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v = s[kb][r] * sc;
        if (tail) {
          const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          if (key >= T) v = -INFINITY;
        }
        s[kb][r] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] *= alpha;

#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(s[kb][r] - m_new);
        l_run += p;
        s[kb][r] = p;
      }
#pragma unroll
      for (int gp = 0; gp < 2; ++gp) {
        bf16x8 pb;
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[e] = static_cast<bf16>(s[kb][8 * gp + e]);
        const int kofs = kb * 32 + 16 * gp + 4 * half;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const bf16* vrow = &Vs[(db * 32 + col) * VP + kofs];
          const bf16x4 lo = *reinterpret_cast<const bf16x4*>(vrow);
          const bf16x4 hi = *reinterpret_cast<const bf16x4*>(vrow + 8);
          const bf16x8 va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, o[db], 0, 0, 0);
        }
      }
    }
  }

  const float l = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.0f / l;
  if (qi < T) {
    bf16* O = static_cast<bf16*>(ap.o) + (int64_t(b) * T + qi) * ap.C + head * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 pk;
#pragma unroll
        for (int e = 0; e < 4; ++e) pk[e] = static_cast<bf16>(o[db][4 * g + e] * inv);
        *reinterpret_cast<bf16x4*>(O + db * 32 + 8 * g + 4 * half) = pk;
      }
  }
}

// ---------------------------------------------------------------------------
// fp32 kernel
// ---------------------------------------------------------------------------
constexpr int FQT = 64, FKT = 32;

template <int DP>  // d rounded up to a supported width; each lane owns DP/4 dims
__global__ __launch_bounds__(256) void attn_f32_kernel(AttnParams ap) {
  constexpr int NPT = DP / 4;
  __shared__ float Ks[FKT * (DP + 1)];
  __shared__ float Vs[FKT * (DP + 1)];
  const int tid = threadIdx.x;
  const int sub = tid & 3, ql = tid >> 2;
  const int qtile = blockIdx.x % ap.qtiles;
  const int bh = blockIdx.x / ap.qtiles;
  const int head = bh % ap.n, b = bh / ap.n;
  const int T = ap.T, d = ap.d;
  const float* Q = static_cast<const float*>(ap.q) + int64_t(bh) * T * d;
  const float* K = static_cast<const float*>(ap.k) + int64_t(bh) * T * d;
  const float* Vt = static_cast<const float*>(ap.vt) + int64_t(bh) * d * ap.Tp;
  const int qi = qtile * FQT + ql;

  float qv[NPT], ov[NPT];
#pragma unroll
  for (int i = 0; i < NPT; ++i) {
    const int dd = i * 4 + sub;
    qv[i] = (qi < T && dd < d) ? Q[int64_t(qi) * d + dd] : 0.f;
    ov[i] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;
  const float sc = ap.scale;

  for (int k0 = 0; k0 < T; k0 += FKT) {
    __syncthreads();
    for (int v = tid; v < FKT * DP; v += 256) {
      const int r = v / DP, c = v % DP;
      const int key = k0 + r;
      Ks[r * (DP + 1) + c] = (key < T && c < d) ? K[int64_t(key) * d + c] : 0.f;
    }
    for (int v = tid; v < FKT * DP; v += 256) {
      const int c = v / FKT, r = v % FKT;
      const int key = k0 + r;
      Vs[r * (DP + 1) + c] = (key < T && c < d) ? Vt[int64_t(c) * ap.Tp + key] : 0.f;
    }
    __syncthreads();
    float s[FKT];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < FKT; ++j) {
      float part = 0.f;
#pragma unroll
      for (int i = 0; i < NPT; ++i) part += qv[i] * Ks[j * (DP + 1) + i * 4 + sub];
      part += __shfl_xor(part, 1, 64);
      part += __shfl_xor(part, 2, 64);
      s[j] = (k0 + j < T) ? part * sc : -INFINITY;
      mx = fmaxf(mx, s[j]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int i = 0; i < NPT; ++i) ov[i] *= alpha;
#pragma unroll
    for (int j = 0; j < FKT; ++j) {
      const float p = exp2f(s[j] - m_new);
      l_run += p;
#pragma unroll
      for (int i = 0; i < NPT; ++i) ov[i] += p * Vs[j * (DP + 1) + i * 4 + sub];
    }
  }
  if (qi < T) {
    float* O = static_cast<float*>(ap.o) + (int64_t(b) * T + qi) * ap.C + head * d;
    const float inv = 1.0f / l_run;
#pragma unroll
    for (int i = 0; i < NPT; ++i) {
      const int dd = i * 4 + sub;
      if (dd < d) O[dd] = ov[i] * inv;
    }
  }
}

}  // namespace

hipError_t launch_attention(const Plan& p, const Args& a) {
  AttnParams ap{};
  ap.q = a.ws + p.ws.q;
  ap.k = a.ws + p.ws.k;
  ap.vt = a.ws + p.ws.vt;
  ap.o = a.ws + p.ws.o;
  ap.T = int(p.T);
  ap.Tp = int(p.Tp);
  ap.n = int(p.n);
  ap.d = int(p.d);
  ap.C = int(p.C);
  ap.scale = kLog2e / sqrtf(float(p.d));
  const int64_t bh = p.B * p.n;
  if (p.dtype == SSA_BF16) {
    ap.qtiles = int((p.T + QT - 1) / QT);
    dim3 grid(unsigned(bh * ap.qtiles));
    switch (p.d) {
      case 32: attn_bf16_kernel<32><<<grid, 256, 0, a.stream>>>(ap); break;
      case 64: attn_bf16_kernel<64><<<grid, 256, 0, a.stream>>>(ap); break;
      case 96: attn_bf16_kernel<96><<<grid, 256, 0, a.stream>>>(ap); break;
      default: attn_bf16_kernel<128><<<grid, 256, 0, a.stream>>>(ap); break;
    }
  } else {
    ap.qtiles = int((p.T + FQT - 1) / FQT);
    dim3 grid(unsigned(bh * ap.qtiles));
    if (p.d <= 32)
      attn_f32_kernel<32><<<grid, 256, 0, a.stream>>>(ap);
    else if (p.d <= 64)
      attn_f32_kernel<64><<<grid, 256, 0, a.stream>>>(ap);
    else
      attn_f32_kernel<128><<<grid, 256, 0, a.stream>>>(ap);
  }
  return hipGetLastError();
}

}  // namespace ssa
