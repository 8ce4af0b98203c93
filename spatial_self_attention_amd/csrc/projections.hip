// The block's two linear layers (tensortonic "Spatial Self-Attention":
// Q = Z Wq^T + bq, K = Z Wk^T + bk, V = Z Wv^T + bv with Z = tokens(GN(x));
// out = x + image(O Wo^T + bo)).
//
// Both are computed in the transposed orientation D = W * Z^T (M = output
// channels, N = tokens, K = input channels).  With the MFMA output layout a
// lane then owns one token column and runs of 4 consecutive channels, which
//  * for Q and K gives 8-byte stores into the token-major (B, n, T, d) layout
//    (bf16 Q is stored times log2(e) / sqrt(d), the attention kernel's score
//    scale, folded in before the one rounding),
//  * for V gives token-contiguous stores into the transposed (B, n, d, Tp)
//    layout the attention kernel's P*V product reads (bf16: tokens in the
//    vt_slot order of that kernel's MFMA operand),
//  * for the output projection gives token-contiguous stores straight into
//    NCHW, so bias + residual + the token-to-image transpose are one epilogue.
//
// QKV prologue: the B tile is read from x in NCHW (token-contiguous rows of
// one channel, 8-byte loads), normalised with one FMA per element using the
// per-(b, c) coefficients of the statistics pass, rounded to bf16 and written
// to LDS channel-contiguous -- the layout MFMA's B operand wants.  GN(x) is
// never stored.
//
// bf16: 128x128x64 work-group tiles, 4 waves each owning a 64x64 quadrant as
// 2x2 v_mfma_f32_32x32x16_bf16 blocks, fp32 accumulation.
// fp32: 64x64x16 LDS-tiled FMA kernels (no reduced-precision shortcuts).
#include <math.h>

#include "ssa_internal.h"

namespace ssa {
namespace {

enum Mode { kQkv = 0, kOut = 1 };

struct ProjParams {
  const void* x;       // (B, C, T)
  const void* w[3];    // row sources: q,k,v weights (kQkv) or out weight (kOut)
  const void* bias[3];
  const float2* coef;  // (B, C) GN coefficients (kQkv)
  const void* o;       // (B*T, C) attention output (kOut)
  void* q;             // (B, n, T, d)
  void* k;
  void* vt;            // (B, n, d, Tp)
  void* out;           // (B, C, T) (kOut)
  int C, T, n, d, Tp;
  int M;               // 3C (kQkv) or C (kOut)
  float q_scale;       // bf16 Q is stored times log2(e) / sqrt(d) (kQkv)
  int64_t NT;          // B*T tokens
};

// ---------------------------------------------------------------------------
// bf16 MFMA kernels
// ---------------------------------------------------------------------------
constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDP = BK + 8;  // LDS row pitch (bf16): 144 B rows spread the banks

// Quad-token loads need T % 4 == 0 (a quad never straddles two samples).
template <int MODE, bool QUAD>
__global__ __launch_bounds__(256) void proj_bf16_kernel(ProjParams pp) {
  __shared__ __attribute__((aligned(16))) bf16 As[BM * LDP];
  __shared__ __attribute__((aligned(16))) bf16 Bs[BN * LDP];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * BM;
  const int64_t n0 = int64_t(blockIdx.x) * BN;
  const int C = pp.C, T = pp.T;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const bf16x8 zero8 = {};
  for (int k0 = 0; k0 < C; k0 += BK) {
    // ---- A: weight rows m0.., 64 input channels, 16-byte loads ----
    bf16x8 ra[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (tid >> 3) + 32 * i;
      const int m = m0 + r;
      const int k = k0 + (tid & 7) * 8;
      ra[i] = zero8;
      if (m < pp.M && k < C) {
        const int which = MODE == kQkv ? m / C : 0;
        const int row = MODE == kQkv ? m - which * C : m;
        const bf16* w = static_cast<const bf16*>(pp.w[which]);
        ra[i] = *reinterpret_cast<const bf16x8*>(w + int64_t(row) * C + k);
      }
    }
    // ---- B: 128 tokens x 64 channels ----
    bf16x8 rb[4];
    if constexpr (MODE == kOut) {
      const bf16* o = static_cast<const bf16*>(pp.o);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = (tid >> 3) + 32 * i;
        const int64_t nn = n0 + r;
        const int k = k0 + (tid & 7) * 8;
        rb[i] = zero8;
        if (nn < pp.NT && k < C) rb[i] = *reinterpret_cast<const bf16x8*>(o + nn * C + k);
      }
    } else {
      // thread = (token quad tq, channel octet co); rb[tok] = 8 channels of token tok
      const bf16* x = static_cast<const bf16*>(pp.x);
      const int tq = tid & 31, co = tid >> 5;
      const int kb = k0 + co * 8;
      float z[4][8];
      if (QUAD) {
        const int64_t nn = n0 + tq * 4;
        if (nn < pp.NT && kb < C) {
          const int64_t b = nn / T;
          const int t = int(nn - b * T);
          const bf16* xp = x + (b * C + kb) * T + t;
          const float2* cf = pp.coef + b * C + kb;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const bf16x4 v = *reinterpret_cast<const bf16x4*>(xp + int64_t(j) * T);
            const float2 ab = cf[j];
#pragma unroll
            for (int e = 0; e < 4; ++e) z[e][j] = ab.x * static_cast<float>(v[e]) + ab.y;
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int j = 0; j < 8; ++j) z[e][j] = 0.f;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t nn = n0 + tq * 4 + e;
          if (nn < pp.NT && kb < C) {
            const int64_t b = nn / T;
            const int t = int(nn - b * T);
            const bf16* xp = x + (b * C + kb) * T + t;
            const float2* cf = pp.coef + b * C + kb;
#pragma unroll
            for (int j = 0; j < 8; ++j)
              z[e][j] = cf[j].x * static_cast<float>(xp[int64_t(j) * T]) + cf[j].y;
          } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) z[e][j] = 0.f;
          }
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int j = 0; j < 8; ++j) rb[e][j] = static_cast<bf16>(z[e][j]);
    }

    __syncthreads();  // previous tile's MFMA reads are done
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (tid >> 3) + 32 * i;
      *reinterpret_cast<bf16x8*>(&As[r * LDP + (tid & 7) * 8]) = ra[i];
    }
    if constexpr (MODE == kOut) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = (tid >> 3) + 32 * i;
        *reinterpret_cast<bf16x8*>(&Bs[r * LDP + (tid & 7) * 8]) = rb[i];
      }
    } else {
      const int tq = tid & 31, co = tid >> 5;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        *reinterpret_cast<bf16x8*>(&Bs[(tq * 4 + e) * LDP + co * 8]) = rb[e];
    }
    __syncthreads();

#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int kofs = ks * 16 + (lane >> 5) * 8;
      bf16x8 fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        fa[i] = *reinterpret_cast<const bf16x8*>(&As[(wm * 64 + i * 32 + (lane & 31)) * LDP + kofs]);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        fb[j] = *reinterpret_cast<const bf16x8*>(&Bs[(wn * 64 + j * 32 + (lane & 31)) * LDP + kofs]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
  }

  // ---- epilogue: lane owns token column (lane & 31) of each 32x32 block and
  // rows 8*g + 4*(lane >> 5) + e, e = 0..3, of each group g = 0..3 ----
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t nn = n0 + wn * 64 + j * 32 + (lane & 31);
    if (nn >= pp.NT) continue;
    const int64_t b = nn / T;
    const int t = int(nn - b * T);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int m = m0 + wm * 64 + i * 32 + 8 * g + 4 * (lane >> 5);
        if (m >= pp.M) continue;
        const int which = MODE == kQkv ? m / C : 0;
        const int c = m - which * C;
        const bf16* bias = static_cast<const bf16*>(pp.bias[which]);
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * g + e] + static_cast<float>(bias[c + e]);
        if constexpr (MODE == kQkv) {
          const int head = c / pp.d, dd = c - head * pp.d;
          const int64_t bh = b * pp.n + head;
          if (which < 2) {
            const float sc = which == 0 ? pp.q_scale : 1.f;
            bf16x4 pk;
#pragma unroll
            for (int e = 0; e < 4; ++e) pk[e] = static_cast<bf16>(v[e] * sc);
            bf16* dst = static_cast<bf16*>(which == 0 ? pp.q : pp.k);
            *reinterpret_cast<bf16x4*>(dst + (bh * T + t) * pp.d + dd) = pk;
          } else {
            bf16* dst = static_cast<bf16*>(pp.vt);
            const int slot = vt_slot(t);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              dst[(bh * pp.d + dd + e) * pp.Tp + slot] = static_cast<bf16>(v[e]);
          }
        } else {
          const bf16* x = static_cast<const bf16*>(pp.x);
          bf16* out = static_cast<bf16*>(pp.out);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int64_t idx = (b * C + c + e) * T + t;
            out[idx] = static_cast<bf16>(static_cast<float>(x[idx]) + v[e]);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 FMA kernels
// ---------------------------------------------------------------------------
constexpr int FM = 64, FN = 64, FK = 16, FP = 64 + 4;

template <int MODE>
__global__ __launch_bounds__(256) void proj_f32_kernel(ProjParams pp) {
  __shared__ float As[FK * FP];  // As[k][m]
  __shared__ float Bs[FK * FP];  // Bs[k][n]
  const int tid = threadIdx.x;
  const int m0 = blockIdx.y * FM;
  const int64_t n0 = int64_t(blockIdx.x) * FN;
  const int C = pp.C, T = pp.T;
  const int ty = tid >> 4, tx = tid & 15;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < C; k0 += FK) {
    {  // A: row tid/4, 4 consecutive k
      const int r = tid >> 2, kk = (tid & 3) * 4;
      const int m = m0 + r;
      const int which = MODE == kQkv ? (m < pp.M ? m / C : 0) : 0;
      const int row = m - which * C;
      const float* w = static_cast<const float*>(pp.w[which]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int k = k0 + kk + e;
        As[(kk + e) * FP + r] = (m < pp.M && k < C) ? w[int64_t(row) * C + k] : 0.f;
      }
    }
    if constexpr (MODE == kQkv) {  // B: channel tid/16, 4 tokens
      const float* x = static_cast<const float*>(pp.x);
      const int kk = tid >> 4, nq = (tid & 15) * 4;
      const int k = k0 + kk;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t nn = n0 + nq + e;
        float z = 0.f;
        if (nn < pp.NT && k < C) {
          const int64_t b = nn / T;
          const int t = int(nn - b * T);
          const float2 ab = pp.coef[b * C + k];
          z = ab.x * x[(b * C + k) * T + t] + ab.y;
        }
        Bs[kk * FP + nq + e] = z;
      }
    } else {  // B: token tid/4, 4 consecutive k
      const float* o = static_cast<const float*>(pp.o);
      const int r = tid >> 2, kk = (tid & 3) * 4;
      const int64_t nn = n0 + r;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int k = k0 + kk + e;
        Bs[(kk + e) * FP + r] = (nn < pp.NT && k < C) ? o[nn * C + k] : 0.f;
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < FK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk * FP + ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk * FP + tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] += a[i] * b[j];
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= pp.M) continue;
    const int which = MODE == kQkv ? m / C : 0;
    const int c = m - which * C;
    const float bias = static_cast<const float*>(pp.bias[which])[c];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t nn = n0 + tx * 4 + j;
      if (nn >= pp.NT) continue;
      const int64_t b = nn / T;
      const int t = int(nn - b * T);
      const float v = acc[i][j] + bias;
      if constexpr (MODE == kQkv) {
        const int head = c / pp.d, dd = c - head * pp.d;
        const int64_t bh = b * pp.n + head;
        if (which == 0)
          static_cast<float*>(pp.q)[(bh * T + t) * pp.d + dd] = v;
        else if (which == 1)
          static_cast<float*>(pp.k)[(bh * T + t) * pp.d + dd] = v;
        else
          static_cast<float*>(pp.vt)[(bh * pp.d + dd) * pp.Tp + t] = v;
      } else {
        const int64_t idx = (b * C + c) * T + t;
        static_cast<float*>(pp.out)[idx] = static_cast<const float*>(pp.x)[idx] + v;
      }
    }
  }
}

ProjParams make_params(const Plan& p, const Args& a, int mode) {
  ProjParams pp{};
  pp.x = a.x;
  if (mode == kQkv) {
    for (int i = 0; i < 3; ++i) {
      pp.w[i] = a.w[i];
      pp.bias[i] = a.b[i];
    }
  } else {
    for (int i = 0; i < 3; ++i) {
      pp.w[i] = a.w[3];
      pp.bias[i] = a.b[3];
    }
  }
  pp.coef = reinterpret_cast<const float2*>(a.ws + p.ws.gn_coef);
  pp.o = a.ws + p.ws.o;
  pp.q = a.ws + p.ws.q;
  pp.k = a.ws + p.ws.k;
  pp.vt = a.ws + p.ws.vt;
  pp.out = a.out;
  pp.C = int(p.C);
  pp.T = int(p.T);
  pp.n = int(p.n);
  pp.d = int(p.d);
  pp.Tp = int(p.Tp);
  pp.M = mode == kQkv ? int(3 * p.C) : int(p.C);
  pp.q_scale = 1.4426950408889634f / sqrtf(float(p.d));
  pp.NT = p.B * p.T;
  return pp;
}

template <int MODE>
hipError_t launch_mode(const Plan& p, const Args& a) {
  const ProjParams pp = make_params(p, a, MODE);
  if (p.dtype == SSA_BF16) {
    dim3 grid(unsigned((pp.NT + BN - 1) / BN), unsigned((pp.M + BM - 1) / BM));
    if (MODE == kOut || p.T % 4 != 0)
      proj_bf16_kernel<MODE, false><<<grid, 256, 0, a.stream>>>(pp);
    else
      proj_bf16_kernel<MODE, true><<<grid, 256, 0, a.stream>>>(pp);
  } else {
    dim3 grid(unsigned((pp.NT + FN - 1) / FN), unsigned((pp.M + FM - 1) / FM));
    proj_f32_kernel<MODE><<<grid, 256, 0, a.stream>>>(pp);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qkv_proj(const Plan& p, const Args& a) { return launch_mode<kQkv>(p, a); }
hipError_t launch_out_proj(const Plan& p, const Args& a) { return launch_mode<kOut>(p, a); }

}  // namespace ssa
