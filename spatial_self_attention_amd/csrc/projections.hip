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
  int dp;              // head width of the q / k / vt layouts (bf16: d rounded up to 32)
  int M;               // 3C (kQkv) or C (kOut)
  float q_scale;       // bf16 Q is stored times log2(e) / sqrt(d) (kQkv)
  int64_t NT;          // B*T tokens
  // optional query/key steps (kQkv, bf16)
  const void* gq;      // (n, d) query / key normalisation gammas, or NULL
  const void* gk;
  int rope;            // rotary embedding on
  const float2* rope_tab;  // (T, d/2) (cos, sin) of the rotary angles
  float* qk32;         // (2, B, n, T, d) fp32 Q and K for the separate option pass, or NULL
  int nt_out;          // kOut: T % 64 == 0, so a wave's 64-token run of an output channel row
                       // is whole 128-byte lines (stored non-temporally); otherwise the runs
                       // straddle lines, whose pieces L2 joins (cached stores)
};

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// bf16 MFMA kernels
// ---------------------------------------------------------------------------
constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDP = BK + 8;  // LDS row pitch (bf16): 144 B rows spread the banks

// Quad-token loads need T % 4 == 0 (a quad never straddles two samples);
// V8: C % 8 == 0, so every 8-channel vector that starts inside a row ends
// inside it (otherwise the loads go element by element).
template <int MODE, bool QUAD, bool V8>
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
        const bf16* w = static_cast<const bf16*>(pp.w[which]) + int64_t(row) * C + k;
        if (V8) {
          ra[i] = *reinterpret_cast<const bf16x8*>(w);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (k + e < C) ra[i][e] = w[e];
        }
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
        if (nn < pp.NT && k < C) {
          if (V8) {
            rb[i] = *reinterpret_cast<const bf16x8*>(o + nn * C + k);
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (k + e < C) rb[i][e] = o[nn * C + k + e];
          }
        }
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
            if (!V8 && kb + j >= C) {  // channels past C: zero operand columns
#pragma unroll
              for (int e = 0; e < 4; ++e) z[e][j] = 0.f;
              continue;
            }
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
              z[e][j] = (V8 || kb + j < C) ? cf[j].x * static_cast<float>(xp[int64_t(j) * T]) + cf[j].y
                                           : 0.f;
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
        float v[4];
        if constexpr (MODE == kQkv) {
          // element by element: any C, so the 4 rows may straddle Q / K / V and
          // heads of any size
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int me = m + e;
            if (me >= pp.M) break;
            const int which = me / C;
            const int c = me - which * C;
            const bf16* bias = static_cast<const bf16*>(pp.bias[which]);  // NULL: no bias
            const float val = acc[i][j][4 * g + e] + (bias ? static_cast<float>(bias[c]) : 0.f);
            const int head = c / pp.d, dd = c - head * pp.d;
            const int64_t bh = b * pp.n + head;
            if (which < 2 && pp.qk32 != nullptr) {  // fp32 for the separate option pass
              pp.qk32[(int64_t(which) * pp.NT * pp.n + bh * T + t) * pp.d + dd] = val;
            } else if (which < 2) {
              bf16* dst = static_cast<bf16*>(which == 0 ? pp.q : pp.k);
              dst[(bh * T + t) * pp.dp + dd] = static_cast<bf16>(val * (which == 0 ? pp.q_scale : 1.f));
            } else {
              static_cast<bf16*>(pp.vt)[(bh * pp.dp + dd) * pp.Tp + vt_slot(t)] = static_cast<bf16>(val);
            }
          }
        } else {
          const bf16* bias = static_cast<const bf16*>(pp.bias[0]);  // NULL: no bias
#pragma unroll
          for (int e = 0; e < 4; ++e)
            v[e] = acc[i][j][4 * g + e] + (bias && m + e < C ? static_cast<float>(bias[m + e]) : 0.f);
          const int c = m;
          const bf16* x = static_cast<const bf16*>(pp.x);
          bf16* out = static_cast<bf16*>(pp.out);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (c + e >= C) break;
            const int64_t idx = (b * C + c + e) * T + t;
            out[idx] = static_cast<bf16>(static_cast<float>(x[idx]) + v[e]);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 MFMA kernels, main path (C % 64 == 0 and T % 4 == 0)
//
// 128 x 128 x 64 work-group tiles, two LDS buffers and two register stages:
// the loads of a k-step go out two steps ahead, and a step is written to LDS
// (for Q/K/V normalised) part by part between the MFMAs of the step before;
// one barrier per k-step.  The epilogue's loads (bias, residual) go out before
// the last two steps.  Each wave owns a 64 x 64 quadrant as 2 x 2
// v_mfma_f32_32x32x16_bf16 blocks.
// The orientation of a wave's product follows its store layout:
//  * Q and K (token-major): D = W Z^T, a lane holds 4 consecutive channels of
//    one token -> 8-byte stores into (B, n, T, d);
//  * V (V^T rows) and the output projection (NCHW rows): D = Z W^T (operands
//    swapped), a lane holds 4 consecutive tokens of one channel -> 8-byte
//    stores of 4 V^T slots (vt_slot keeps aligned runs of 4 together) or of 4
//    pixels of one output channel, with the residual read the same way.
// Work-group ids are remapped so the m-tiles of one token tile (which share
// the x / O rows they read) run on the same XCD and share its L2.
// ---------------------------------------------------------------------------
constexpr int GM = 128, GN = 128, GK = 64;
constexpr int GP = GK + 8;  // LDS row pitch (bf16): 144-byte rows, conflict-free 16-byte reads

// Word 3 of a raw buffer resource on the gfx9 family (32-bit data format).
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), kRsrcWord3);
}

__device__ __forceinline__ bf16x8 ld16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// Work-group id -> logical id: work-groups go to the 8 XCDs round-robin, so
// XCD x receives ids x, x+8, ...; consecutive logical ids land on one XCD.
__device__ __forceinline__ int xcd_remap_gemm(int w, int nwg) {
  const int q = nwg >> 3, r = nwg & 7, x = w & 7;
  return x * q + min(x, r) + (w >> 3);
}

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// One k-step of A (weight rows) and B in registers, as loaded: for the QKV
// projection B is raw x (8 channel rows x 4 tokens) and the (a, s) GN
// coefficients of those 8 channels, normalised only when written to LDS, so
// that the loads stay in flight behind the MFMAs of the step before.
struct Stage {
  bf16x8 a[4];
  bf16x8 b[4];     // kOut: 4 token rows of O
  u32x2 xr[8];     // kQkv: x rows, 4 bf16 tokens each
  f32x4 cf[4];     // kQkv: (a, s) of the 8 channels
};

// Loop-invariant addressing of one thread's loads: buffer resources and
// per-thread byte offsets are fixed; each k-step only moves a scalar offset.
//  A: vector i = tid + 256 i is row (tid >> 3) + 32 i, channels (tid & 7) * 8;
//     the 32 rows of one i lie in one 64-row block, so they belong to one of
//     Wq / Wk / Wv (C % 64 == 0) and the resource is uniform.
//  B (Q/K/V): thread = (token quad tq, channel octet co), 8 channel rows of 4
//     tokens each.  Lanes are laid out so that each group of 16 lanes stores
//     its 16-byte LDS vectors to 16 distinct bank groups, while 16 lanes of
//     one channel row still read 128 contiguous bytes of x.
//  B (out projection): vector i is token row (tid >> 3) + 32 i of O.
// Rows past M and tokens past B*T are clamped onto valid ones: they only feed
// accumulator rows / columns that the epilogue never stores.
struct LoadCtx {
  __amdgpu_buffer_rsrc_t ra[4];
  int sa[4];       // scalar byte offset of row block i in its weight
  int va;          // per-thread byte offset inside a row block
  __amdgpu_buffer_rsrc_t rb, rc;
  int vb[4];       // kOut: byte offset of token row i in O
  int vx, vc;      // kQkv: byte offsets of x[b][co*8][t] and coef[b][co*8]
  int xrow;        // kQkv: bytes between consecutive channel rows of x (2T)
};

__device__ __forceinline__ int qkv_tq(int tid) {
  return (tid & 3) | (((tid >> 4) & 7) << 2);
}
__device__ __forceinline__ int qkv_co(int tid) { return ((tid >> 2) & 3) | ((tid >> 7) << 2); }

template <int MODE>
__device__ __forceinline__ void gemm_setup(LoadCtx& lc, const ProjParams& pp, int m0, int n0,
                                           int tid) {
  // Byte offsets are formed in 32-bit unsigned arithmetic: a tensor holds at
  // most 2^31 - 1 elements, so a bf16 offset stays below 2^32 but may pass 2^31.
  const unsigned C = unsigned(pp.C);
  const uint32_t wbytes = C * C * 2u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rb = m0 + 32 * i < pp.M ? m0 + 32 * i : 0;
    const int which = MODE == kQkv ? rb / int(C) : 0;
    lc.ra[i] = make_rsrc(pp.w[which], wbytes);
    lc.sa[i] = int((unsigned(rb) - unsigned(which) * C) * C * 2u);
  }
  lc.va = int((unsigned(tid >> 3) * C + unsigned(tid & 7) * 8u) * 2u);
  if constexpr (MODE == kOut) {
    lc.rb = make_rsrc(pp.o, uint32_t(pp.NT) * C * 2u);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int nn = min(n0 + (tid >> 3) + 32 * i, int(pp.NT) - 1);
      lc.vb[i] = int((unsigned(nn) * C + unsigned(tid & 7) * 8u) * 2u);
    }
  } else {
    const unsigned T = unsigned(pp.T);
    const int tq = qkv_tq(tid), co = qkv_co(tid);
    const int nn = min(n0 + tq * 4, int(pp.NT) - 4);
    const unsigned b = unsigned(nn) / T;
    const unsigned t = unsigned(nn) - b * T;
    lc.rb = make_rsrc(pp.x, uint32_t(pp.NT) * C * 2u);
    lc.rc = make_rsrc(pp.coef, uint32_t(pp.NT / pp.T) * C * 8u);
    lc.vx = int(((b * C + unsigned(co) * 8u) * T + t) * 2u);
    lc.vc = int((b * C + unsigned(co) * 8u) * 8u);
    lc.xrow = int(T * 2u);
  }
}

template <int MODE>
__device__ __forceinline__ void gemm_load(Stage& sg, const LoadCtx& lc, int k0) {
#pragma unroll
  for (int i = 0; i < 4; ++i) sg.a[i] = ld16(lc.ra[i], lc.va, lc.sa[i] + k0 * 2);
  if constexpr (MODE == kOut) {
#pragma unroll
    for (int i = 0; i < 4; ++i) sg.b[i] = ld16(lc.rb, lc.vb[i], k0 * 2);
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      sg.cf[q] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(lc.rc, lc.vc, k0 * 8 + 16 * q, 0));
    // channel row k0 + j: the row step goes into the scalar offset, so one
    // per-thread offset serves all eight loads
#pragma unroll
    for (int j = 0; j < 8; ++j)
      sg.xr[j] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(lc.rb, lc.vx, int(unsigned(k0 + j) * unsigned(lc.xrow)), 0));
  }
}

// LDS row of token t in the QKV projection's B tile.  A thread writes rows
// tq*4 + u of four token quads per 8-lane group, which with 144-byte rows puts
// two lanes on the same banks; flipping bit 1 of the row when bit 3 is set
// spreads those writes over 8 bank groups and keeps the fragment reads (8
// consecutive tokens) on 8 distinct groups as well.
__device__ __forceinline__ int brow(int t) { return t ^ ((t >> 2) & 2); }

// Part u (0..3) of writing a register stage to LDS: A vector u (row
// (tid >> 3) + 32u) and, for the output projection, B vector u (token row
// (tid >> 3) + 32u of O); for Q/K/V token tq*4 + u of the thread's quad,
// normalised: GN(x) = a x + s in fp32, rounded once to bf16, 8 channels.
template <int MODE>
__device__ __forceinline__ void store_part(bf16* As, bf16* Bs, const Stage& sg, int tid, int u) {
  const int v = tid + 256 * u;
  *reinterpret_cast<bf16x8*>(&As[(v >> 3) * GP + (v & 7) * 8]) = sg.a[u];
  if constexpr (MODE == kOut) {
    *reinterpret_cast<bf16x8*>(&Bs[(v >> 3) * GP + (v & 7) * 8]) = sg.b[u];
  } else {
    bf16x8 z;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float a = sg.cf[j >> 1][(j & 1) * 2], sh = sg.cf[j >> 1][(j & 1) * 2 + 1];
      const unsigned w = sg.xr[j][u >> 1];  // tokens 2(u>>1), 2(u>>1)+1 of the quad
      const float xv = __uint_as_float((u & 1) ? (w & 0xffff0000u) : (w << 16));
      z[j] = static_cast<bf16>(fmaf(a, xv, sh));
    }
    const int tq = qkv_tq(tid), co = qkv_co(tid);
    *reinterpret_cast<bf16x8*>(&Bs[brow(tq * 4 + u) * GP + co * 8]) = z;
  }
}

template <int MODE>
__device__ __forceinline__ void gemm_store(bf16* As, bf16* Bs, const Stage& sg, int tid) {
#pragma unroll
  for (int u = 0; u < 4; ++u) store_part<MODE>(As, Bs, sg, tid, u);
}

// Operand fragments of sub-step s (16 channels) of one k-step, read from LDS.
struct Frags {
  bf16x8 a[2], b[2];
};

template <int MODE>
__device__ __forceinline__ void read_frags(Frags& f, const bf16* As, const bf16* Bs, int wm,
                                           int wn, int half, int col, int s) {
  const int kofs = s * 16 + half * 8;
  const int bcol = MODE == kQkv ? brow(col) : col;  // rows wn*64 + j*32 keep bits 1 and 3 clear
#pragma unroll
  for (int i = 0; i < 2; ++i)
    f.a[i] = *reinterpret_cast<const bf16x8*>(&As[(wm * 64 + i * 32 + col) * GP + kofs]);
#pragma unroll
  for (int j = 0; j < 2; ++j)
    f.b[j] = *reinterpret_cast<const bf16x8*>(&Bs[(wn * 64 + j * 32 + bcol) * GP + kofs]);
}

// The 2 x 2 MFMAs of one sub-step.
template <bool TR>
__device__ __forceinline__ void mfma_sub(f32x16 (&acc)[2][2], const Frags& f) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
      acc[i][j] = TR ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[j], f.a[i], acc[i][j], 0, 0, 0)
                     : __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
}

// Epilogue geometry: each wave stages its 64 x 64 quadrant in its own LDS
// region in the destination's layout (bias added; Q scaled), then stores it
// with coalesced vectors.
//  * Q / K: E[token][channel] bf16; a lane stores 16-byte runs of 8 channels
//    of one token, 8 lanes covering one token's 64 channels.
//  * V: E[channel][token] bf16; a lane owns one run of 4 tokens and stores it
//    (4 consecutive V^T slots) for 16 channels, 16 lanes per channel row.
//  * output: E[channel][token] fp32 (so x + Y is rounded once), same lanes,
//    with the residual read in the same 8-byte runs.
// Staging pitches (elements): 144-byte bf16 rows and 272-byte fp32 rows keep
// the 8- and 16-byte staging writes of 16 lanes on distinct banks.
constexpr int EPB = 72, EPF = 68;
static_assert(2 * 64 * EPF * 4 <= (GM + GN) * GP * 2, "two fp32 staging regions fit one buffer");

struct EpiCtx {
  int mw, nw;            // first row / token of the wave's quadrant (wave-uniform)
  int lane, half, col;
};

// What the epilogue reads from global memory, fetched before the last k-steps'
// MFMAs so that its latency is hidden behind them rather than paid once per
// store: the bias values of the lane's channels and, for the output
// projection, the residual x of the lane's 16 store runs.
struct EpiPre {
  bf16x4 qk_bias[2][4];  // Q / K: channels i*32 + 8g + 4*half + 0..3
  float col_bias[2];     // V / output: channel i*32 + col
  u32x2 res[16];         // output: x at the 16 runs epi_store writes
};

// The bias of the wave's rows (NULL: no bias), selected with a uniform branch
// so the pointer comes from the kernel arguments, not from a dynamic index.
__device__ __forceinline__ const bf16* row_bias(const ProjParams& pp, int which) {
  return static_cast<const bf16*>(which == 0 ? pp.bias[0] : which == 1 ? pp.bias[1] : pp.bias[2]);
}

// The sample b and token t of this lane's run of 4 tokens in the V^T and
// output epilogues (lane & 15 picks the run); false past the last token.
__device__ __forceinline__ bool res_run(const ProjParams& pp, const EpiCtx& ec, int& b, int& t) {
  const int nn = ec.nw + 4 * (ec.lane & 15);
  if (nn >= pp.NT) return false;  // NT % 4 == 0: a run is all in or all out
  b = int(unsigned(nn) / unsigned(pp.T));
  t = nn - b * pp.T;
  return true;
}

template <int MODE, bool TR>
__device__ __forceinline__ void epi_prefetch(EpiPre& ep, const ProjParams& pp, const EpiCtx& ec) {
  const int C = pp.C;
  if (ec.mw >= pp.M) return;  // the upper half of a 64-row last tile stores nothing
  if constexpr (MODE == kOut) {
    const bf16* bp = row_bias(pp, 0);
#pragma unroll
    for (int i = 0; i < 2; ++i) ep.col_bias[i] = bp ? static_cast<float>(bp[ec.mw + i * 32 + ec.col]) : 0.f;
    int b = 0, t = 0;
    const bool ok = res_run(pp, ec, b, t);
    // out-of-range runs read offset 0x80000000, past the resource: zeros
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(pp.x, unsigned(pp.NT) * unsigned(C) * 2u);
    const unsigned v0 = ok ? ((unsigned(b) * unsigned(C) + unsigned(ec.mw + (ec.lane >> 4))) *
                                  unsigned(pp.T) + unsigned(t)) * 2u
                           : 0x80000000u;
    const unsigned row4 = unsigned(pp.T) * 8u;  // four channel rows
#pragma unroll
    for (int u = 0; u < 16; ++u)
      ep.res[u] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rx, int(v0), int(u * row4), 0));
  } else if constexpr (TR) {  // V
    const bf16* bp = row_bias(pp, 2);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      ep.col_bias[i] = bp ? static_cast<float>(bp[ec.mw - 2 * C + i * 32 + ec.col]) : 0.f;
  } else {  // Q or K
    const int which = ec.mw / C;
    const bf16* bp = row_bias(pp, which);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        ep.qk_bias[i][g] = bp ? *reinterpret_cast<const bf16x4*>(bp + (ec.mw - which * C) + i * 32 +
                                                                 8 * g + 4 * ec.half)
                              : bf16x4{};
  }
}

// acc[i][j]: channel block i x token block j of the wave's quadrant.
// TR = false: rows are channels; TR = true: rows are tokens.
// Two LDS buffers (distinct arrays, so the compiler may interleave their
// accesses) and two register stages.  Step s: after the barrier the loads of
// step s+2 go out into one register stage; step s+1, loaded during step s-1,
// is written (for Q/K/V normalised) from the other into the buffer step s-1
// read, while the MFMAs of step s read the other buffer.  The epilogue's own
// loads go out before the last two steps.
// BUSY = false: the wave's rows all lie past M (the upper half of a 64-row
// last tile); it still loads and stores its share of the tiles and meets
// every barrier, but reads no fragments and issues no MFMAs.
template <int MODE, bool TR, bool BUSY = true>
__device__ __forceinline__ void gemm_main(f32x16 (&acc)[2][2], EpiPre& ep, const ProjParams& pp,
                                          bf16* lds0, bf16* lds1, int m0, int n0, int tid,
                                          int wave, const EpiCtx& ec) {
  const int wm = wave >> 1, wn = wave & 1;
  const int half = ec.half, col = ec.col;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  LoadCtx lc;
  gemm_setup<MODE>(lc, pp, m0, n0, tid);
  const int nk = pp.C / GK;  // >= 1
  Stage s0, s1;
  gemm_load<MODE>(s0, lc, 0);
  gemm_store<MODE>(lds0, lds0 + GM * GP, s0, tid);
  if (nk > 1) gemm_load<MODE>(s1, lc, GK);
  // rd: step ks's buffer; wr: the other one, which receives step ks+1 from
  // `nxt` (when `more`); `fre` receives the loads of step ks+2 (when `load`).
  auto step = [&](int ks, const bf16* rd, bf16* wr, const Stage& nxt, Stage& fre, bool more,
                  bool load) {
    __syncthreads();  // rd is complete; wr is no longer read
    if (load) gemm_load<MODE>(fre, lc, (ks + 2) * GK);
    __builtin_amdgcn_sched_barrier(0);  // the loads stay at the top of the step
    // sub-step u's MFMAs, then part u of the next stage, so that the in-order
    // issue of a wave puts the normalisation between its own MFMAs.  The
    // output projection (fewer work-groups per CU to hide LDS latency, and
    // registers to spare) reads the fragments of sub-step u+1 before sub-step
    // u's MFMAs.
    constexpr bool kAhead = MODE == kOut;
    Frags f[2];
    if (BUSY && kAhead) read_frags<MODE>(f[0], rd, rd + GM * GP, wm, wn, half, col, 0);
#pragma unroll
    for (int u = 0; u < GK / 16; ++u) {
      if constexpr (BUSY) {
        if (kAhead) {
          if (u + 1 < GK / 16) read_frags<MODE>(f[(u + 1) & 1], rd, rd + GM * GP, wm, wn, half, col, u + 1);
        } else {
          read_frags<MODE>(f[u & 1], rd, rd + GM * GP, wm, wn, half, col, u);
        }
        mfma_sub<TR>(acc, f[u & 1]);
      }
      if (more) store_part<MODE>(wr, wr + GM * GP, nxt, tid, u);
    }
  };
  // Which register stage and buffer a step uses is fixed at compile time in
  // each branch (chosen at run time, both stages would stay live in the tail).
  const int body = nk > 2 ? nk - 2 : 0;  // steps that still load
  if (nk == 1) {
    epi_prefetch<MODE, TR>(ep, pp, ec);
    step(0, lds0, lds1, s1, s0, false, false);
  } else if (body & 1) {
    step(0, lds0, lds1, s1, s0, true, true);
    for (int ks = 1; ks < body; ks += 2) {
      step(ks, lds1, lds0, s0, s1, true, true);
      step(ks + 1, lds0, lds1, s1, s0, true, true);
    }
    epi_prefetch<MODE, TR>(ep, pp, ec);
    step(body, lds1, lds0, s0, s1, true, false);
    step(body + 1, lds0, lds1, s1, s0, false, false);
  } else {
    for (int ks = 0; ks < body; ks += 2) {
      step(ks, lds0, lds1, s1, s0, true, true);
      step(ks + 1, lds1, lds0, s0, s1, true, true);
    }
    epi_prefetch<MODE, TR>(ep, pp, ec);
    step(body, lds0, lds1, s1, s0, true, false);
    step(body + 1, lds1, lds0, s0, s1, false, false);
  }
}

template <int MODE, bool TR, int QKO>
__device__ __forceinline__ void epi_stage(const f32x16 (&acc)[2][2], const EpiPre& ep,
                                          const ProjParams& pp, bf16* stg, const EpiCtx& ec) {
  const int C = pp.C, half = ec.half, col = ec.col;
  if constexpr (MODE == kQkv && !TR && QKO != 0) {
    // Q or K with an optional step: acc + bias in fp32, token-major, so that
    // the steps run on unrounded values and Q and K are rounded once
    float* E = reinterpret_cast<float*>(stg);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int cl = i * 32 + 8 * g + 4 * half;
        const bf16x4 bv = ep.qk_bias[i][g];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          f32x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * g + e] + static_cast<float>(bv[e]);
          *reinterpret_cast<f32x4*>(&E[(j * 32 + col) * EPF + cl]) = v;
        }
      }
  } else if constexpr (MODE == kOut) {
    float* E = reinterpret_cast<float*>(stg);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int cl = i * 32 + col;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * g + e] + ep.col_bias[i];
          *reinterpret_cast<f32x4*>(&E[cl * EPF + j * 32 + 8 * g + 4 * half]) = v;
        }
    }
  } else if constexpr (TR) {  // V
    bf16* E = stg;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int cl = i * 32 + col;
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          bf16x4 pk;
#pragma unroll
          for (int e = 0; e < 4; ++e) pk[e] = static_cast<bf16>(acc[i][j][4 * g + e] + ep.col_bias[i]);
          *reinterpret_cast<bf16x4*>(&E[cl * EPB + j * 32 + 8 * g + 4 * half]) = pk;
        }
    }
  } else {  // Q or K
    bf16* E = stg;
    const float sc = ec.mw < C ? pp.q_scale : 1.f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int cl = i * 32 + 8 * g + 4 * half;
        const bf16x4 bv = ep.qk_bias[i][g];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          bf16x4 pk;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            pk[e] = static_cast<bf16>((acc[i][j][4 * g + e] + static_cast<float>(bv[e])) * sc);
          *reinterpret_cast<bf16x4*>(&E[(j * 32 + col) * EPB + cl]) = pk;
        }
      }
  }
}

// The staging region of wave w (its 64 x 64 quadrant, fp32 or bf16).
__device__ __forceinline__ bf16* stage_region(bf16* lds0, bf16* lds1, int w) {
  return (w < 2 ? lds0 : lds1) + (w & 1) * 64 * EPF * 2;
}

// Query/key normalisation and rotary embedding in the Q / K epilogue
// (d in {16, 32, 64, 128}; vit-pytorch simple_vit_with_qk_norm.py, RMSNorm:
// x / max(||x||, 1e-12) * sqrt(d) * gamma; HNDL attention operator, "Rotary
// embeddings": rotate-half, element i paired with i + d/2), from acc + bias
// staged in fp32 by every wave.  A lane takes 4 items (token, head, chunk ic
// of 8 element pairs) of its wave's 64 x 64 quadrant; with d = 128 a head's
// two halves lie in the quadrants of waves (0, wn) and (1, wn), which then
// take 32 tokens each.  The d/16 lanes of one (token, head) are consecutive,
// so the squared norm is summed with lane shuffles.  The rotation's (cos,
// sin) come from the per-call table (float32 angle t * theta_i).  Q and K are
// rounded to bf16 once; Q is stored times log2(e) (normalised: its scores are
// not divided by sqrt(d)) or times log2(e)/sqrt(d).
__device__ __forceinline__ void epi_store_qkopt(const ProjParams& pp, bf16* lds0, bf16* lds1,
                                                const EpiCtx& ec, int wave) {
  const int d = pp.d, C = pp.C, T = pp.T, lane = ec.lane;
  const int wm = wave >> 1, wn = wave & 1;
  const int which = ec.mw / C;                  // 0: Q, 1: K (V waves never come here)
  const int lg = d == 16 ? 0 : d == 32 ? 1 : d == 64 ? 2 : 3;  // log2(d / 16)
  const int nic = 1 << lg;                      // chunks of 8 pairs per head
  const bool wide = d == 128;
  const int lh = wide ? 0 : 2 - lg;             // log2(heads per quadrant)
  const int head0 = ((wide ? ec.mw - 64 * wm : ec.mw) - which * C) / d;
  const float* Ra = reinterpret_cast<const float*>(stage_region(lds0, lds1, (wide ? 0 : wm) * 2 + wn));
  const float* Rb = reinterpret_cast<const float*>(stage_region(lds0, lds1, (wide ? 1 : wm) * 2 + wn));
  const int ic = lane & (nic - 1);
  const bf16* gam = static_cast<const bf16*>(which == 0 ? pp.gq : pp.gk);
  const float sc = which == 0 ? (gam != nullptr ? kLog2e : pp.q_scale) : 1.f;
  bf16* dst = static_cast<bf16*>(which == 0 ? pp.q : pp.k);
  const float sqd = sqrtf(float(d));
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int rest = (lane + 64 * u) >> lg;
    const int hs = rest & ((1 << lh) - 1);
    const int tl = (wide ? 32 * wm : 0) + (rest >> lh);
    const int ca = hs * d + ic * 8;             // a-run in Ra (first half of the head)
    const int cb = wide ? ic * 8 : ca + d / 2;  // b-run in Rb (second half)
    float a[8], b[8];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const f32x4 va = *reinterpret_cast<const f32x4*>(&Ra[tl * EPF + ca + 4 * h]);
      const f32x4 vb = *reinterpret_cast<const f32x4*>(&Rb[tl * EPF + cb + 4 * h]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a[4 * h + e] = va[e];
        b[4 * h + e] = vb[e];
      }
    }
    const int head = head0 + hs;
    const int nn = ec.nw + tl;
    const int nc = min(nn, int(pp.NT) - 1);   // rows past the last token: any valid one
    const int bs = int(unsigned(nc) / unsigned(T)), t = nc - bs * T;
    if (gam != nullptr) {
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += a[e] * a[e] + b[e] * b[e];
      for (int m = 1; m < nic; m <<= 1) ss += __shfl_xor(ss, m, 64);
      const float f = sqd / fmaxf(sqrtf(ss), 1e-12f);
      const bf16x8 ga = *reinterpret_cast<const bf16x8*>(gam + head * d + ic * 8);
      const bf16x8 gb = *reinterpret_cast<const bf16x8*>(gam + head * d + d / 2 + ic * 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        a[e] *= f * static_cast<float>(ga[e]);
        b[e] *= f * static_cast<float>(gb[e]);
      }
    }
    if (pp.rope) {
      const f32x4* rt = reinterpret_cast<const f32x4*>(pp.rope_tab + int64_t(t) * (d / 2) + ic * 8);
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const f32x4 cs = rt[h];  // (cos, sin) of pairs 2h and 2h + 1 of the chunk
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const float c = cs[2 * e], sn = cs[2 * e + 1];
          const float na = a[2 * h + e] * c - b[2 * h + e] * sn;
          const float nb = b[2 * h + e] * c + a[2 * h + e] * sn;
          a[2 * h + e] = na;
          b[2 * h + e] = nb;
        }
      }
    }
    if (nn < pp.NT) {
      bf16x8 pa, pb;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pa[e] = static_cast<bf16>(a[e] * sc);
        pb[e] = static_cast<bf16>(b[e] * sc);
      }
      bf16* row = dst + (int64_t(bs * pp.n + head) * T + t) * pp.dp;
      store_nt(row + ic * 8, pa);
      store_nt(row + d / 2 + ic * 8, pb);
    }
  }
}

// Q or K in fp32 (acc + bias, unscaled) into the qk32 region, for the separate
// pass of the optional steps (head sizes the fused epilogue does not take):
// lane (8-channel run q8, tokens r0 + 8u), d % 8 == 0 keeps a run in one head.
__device__ __forceinline__ void epi_store_qk32(const ProjParams& pp, const bf16* stg,
                                               const EpiCtx& ec) {
  const int C = pp.C, T = pp.T, lane = ec.lane;
  const float* E = reinterpret_cast<const float*>(stg);
  const int which = ec.mw / C;
  float* dst = pp.qk32 + int64_t(which) * pp.NT * C;
  const int q8 = lane & 7;
  const int c = ec.mw - which * C + q8 * 8;
  const int head = int(unsigned(c) / unsigned(pp.d)), dd = c - head * pp.d;
  const int r0 = lane >> 3;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int nn = ec.nw + r0 + 8 * u;
    if (nn >= pp.NT) break;
    const int b = int(unsigned(nn) / unsigned(T)), t = nn - b * T;
    float* row = dst + (int64_t(b * pp.n + head) * T + t) * pp.d + dd;
#pragma unroll
    for (int h = 0; h < 2; ++h)
      *reinterpret_cast<f32x4*>(row + 4 * h) =
          *reinterpret_cast<const f32x4*>(&E[(r0 + 8 * u) * EPF + q8 * 8 + 4 * h]);
  }
}

template <int MODE, bool TR>
__device__ __forceinline__ void epi_store(const EpiPre& ep, const ProjParams& pp, const bf16* stg,
                                          const EpiCtx& ec) {
  const int C = pp.C, T = pp.T, lane = ec.lane;
  if constexpr (MODE == kOut || TR) {
    const int tq = lane & 15;  // this lane's run of 4 tokens
    int b = 0, t = 0;
    if (!res_run(pp, ec, b, t)) return;
    if constexpr (MODE == kOut) {
      const float* E = reinterpret_cast<const float*>(stg);
      bf16* out = static_cast<bf16*>(pp.out);
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int cl = 4 * u + (lane >> 4);
        const int64_t idx = (int64_t(b) * C + ec.mw + cl) * T + t;
        const u32x2 xr = ep.res[u];
        const float xv[4] = {__uint_as_float(xr[0] << 16), __uint_as_float(xr[0] & 0xffff0000u),
                             __uint_as_float(xr[1] << 16), __uint_as_float(xr[1] & 0xffff0000u)};
        const f32x4 y = *reinterpret_cast<const f32x4*>(&E[cl * EPF + 4 * tq]);
        bf16x4 pk;
#pragma unroll
        for (int e = 0; e < 4; ++e) pk[e] = static_cast<bf16>(xv[e] + y[e]);
        if (pp.nt_out)
          store_nt(out + idx, pk);
        else
          *reinterpret_cast<bf16x4*>(out + idx) = pk;
      }
    } else {
      const bf16* E = stg;
      bf16* vt = static_cast<bf16*>(pp.vt);
      const int slot = vt_slot(t);  // aligned runs of 4 tokens keep their order
      const int cw = ec.mw - 2 * C;
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int cl = 4 * u + (lane >> 4);
        const int c = cw + cl;
        const int head = int(unsigned(c) / unsigned(pp.d)), dd = c - head * pp.d;
        store_nt(vt + (int64_t(b * pp.n + head) * pp.dp + dd) * pp.Tp + slot,
                 *reinterpret_cast<const bf16x4*>(&E[cl * EPB + 4 * tq]));
      }
    }
  } else {
    const bf16* E = stg;
    const int which = ec.mw / C;
    bf16* dst = static_cast<bf16*>(which == 0 ? pp.q : pp.k);
    const int q8 = lane & 7;  // this lane's 8-channel run
    const int c = ec.mw - which * C + q8 * 8;
    const int head = int(unsigned(c) / unsigned(pp.d)), dd = c - head * pp.d;
    const int r0 = lane >> 3;
    int nn = ec.nw + r0;
    int b = int(unsigned(min(nn, pp.NT - 1)) / unsigned(T));
    int t = nn - b * T;
#pragma unroll
    for (int u = 0; u < 8; ++u) {  // token r0 + 8u
      if (u > 0) {
        nn += 8;
        t += 8;
        while (t >= T) { t -= T; ++b; }
      }
      if (nn < pp.NT)
        store_nt(dst + (int64_t(b * pp.n + head) * T + t) * pp.dp + dd,
                 *reinterpret_cast<const bf16x8*>(&E[(r0 + 8 * u) * EPB + q8 * 8]));
    }
  }
}

// QKO (Q / K epilogue): 0 the plain bf16 store, 1 the optional query/key
// steps applied in the epilogue, 2 fp32 Q and K into the qk32 region.
template <int MODE, int QKO>
__global__ __launch_bounds__(256, 2) void gemm_bf16_kernel(ProjParams pp, int mtiles) {
  __shared__ __attribute__((aligned(16))) bf16 lds0[(GM + GN) * GP];
  __shared__ __attribute__((aligned(16))) bf16 lds1[(GM + GN) * GP];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lid = xcd_remap_gemm(int(blockIdx.x), int(gridDim.x));
  const int m0 = (lid % mtiles) * GM;
  const int n0 = (lid / mtiles) * GN;
  EpiCtx ec;
  ec.mw = m0 + (wave >> 1) * 64;
  ec.nw = n0 + (wave & 1) * 64;
  ec.lane = lane;
  ec.half = lane >> 5;
  ec.col = lane & 31;
  // V rows and the output projection take the swapped orientation
  const bool tr = MODE == kOut || ec.mw >= 2 * pp.C;
  const bool valid = ec.mw < pp.M;  // false for the upper half of a 64-row last tile
  f32x16 acc[2][2];
  EpiPre ep;
  // the wave's staging region: two per buffer (two fp32 regions fit one buffer)
  bf16* stg = (wave < 2 ? lds0 : lds1) + (wave & 1) * 64 * EPF * 2;
  // The epilogue works on copies that the compiler cannot see through, so that
  // its index arithmetic (divisions by T and d, lane offsets) is not hoisted
  // above the main loop, where it would hold registers the loop needs.
  auto epilogue_inputs = [&](ProjParams& pe, EpiCtx& ee) {
    pe = pp;
    ee = ec;
    asm volatile("" : "+s"(pe.T), "+s"(pe.d), "+s"(pe.n), "+s"(pe.Tp));
    asm volatile("" : "+v"(ee.lane), "+v"(ee.half), "+v"(ee.col));
  };
  ProjParams pe;
  EpiCtx ee;
  if (tr) {
    if (valid)
      gemm_main<MODE, true>(acc, ep, pp, lds0, lds1, m0, n0, tid, wave, ec);
    else
      gemm_main<MODE, true, false>(acc, ep, pp, lds0, lds1, m0, n0, tid, wave, ec);
    epilogue_inputs(pe, ee);
    __syncthreads();  // every wave is done reading the operand tiles
    if (valid) epi_stage<MODE, true, QKO>(acc, ep, pe, stg, ee);
    __syncthreads();
    if (valid) epi_store<MODE, true>(ep, pe, stg, ee);
  } else {
    if (valid)
      gemm_main<MODE, false>(acc, ep, pp, lds0, lds1, m0, n0, tid, wave, ec);
    else
      gemm_main<MODE, false, false>(acc, ep, pp, lds0, lds1, m0, n0, tid, wave, ec);
    epilogue_inputs(pe, ee);
    __syncthreads();
    if (valid) epi_stage<MODE, false, QKO>(acc, ep, pe, stg, ee);
    __syncthreads();  // (QKO 1, d = 128: a wave also reads its column partner's region)
    if constexpr (MODE == kQkv && QKO == 1) {
      if (valid) epi_store_qkopt(pe, lds0, lds1, ee, wave);
    } else if constexpr (MODE == kQkv && QKO == 2) {
      if (valid) epi_store_qk32(pe, stg, ee);
    } else {
      if (valid) epi_store<MODE, false>(ep, pe, stg, ee);
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
    const float* bp = static_cast<const float*>(pp.bias[which]);  // NULL: no bias
    const float bias = bp ? bp[c] : 0.f;
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
  pp.nt_out = p.T % 64 == 0;
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
  pp.dp = int(p.dp);
  pp.M = mode == kQkv ? int(3 * p.C) : int(p.C);
  pp.q_scale = kLog2e / sqrtf(float(p.d));
  pp.NT = p.B * p.T;
  if (mode == kQkv && p.dtype == SSA_BF16) {
    pp.gq = a.q_norm_gamma;
    pp.gk = a.k_norm_gamma;
    pp.rope = a.rope ? 1 : 0;
    pp.rope_tab = reinterpret_cast<const float2*>(a.ws + p.ws.rope);
    if (!p.qk_fuse && (a.rope || a.q_norm_gamma != nullptr))
      pp.qk32 = reinterpret_cast<float*>(a.ws + p.ws.qk32);
  }
  return pp;
}

template <int MODE>
hipError_t launch_mode(const Plan& p, const Args& a) {
  const ProjParams pp = make_params(p, a, MODE);
  const bool main = MODE == kQkv ? p.qkv_main
                                 : p.dtype == SSA_BF16 && p.C % 64 == 0 && p.T % 4 == 0;
  if (main) {
    const int mtiles = int((pp.M + GM - 1) / GM);
    const int64_t ntiles = (pp.NT + GN - 1) / GN;
    const dim3 grid(unsigned(mtiles * ntiles));
    const bool opt = pp.rope != 0 || pp.gq != nullptr;
    if (MODE == kQkv && opt && p.qk_fuse)
      gemm_bf16_kernel<MODE, 1><<<grid, 256, 0, a.stream>>>(pp, mtiles);
    else if (MODE == kQkv && opt)
      gemm_bf16_kernel<MODE, 2><<<grid, 256, 0, a.stream>>>(pp, mtiles);
    else
      gemm_bf16_kernel<MODE, 0><<<grid, 256, 0, a.stream>>>(pp, mtiles);
  } else if (p.dtype == SSA_BF16) {
    dim3 grid(unsigned((pp.NT + BN - 1) / BN), unsigned((pp.M + BM - 1) / BM));
    const bool quad = MODE == kQkv && p.T % 4 == 0;
    const bool v8 = p.C % 8 == 0;
    if (quad && v8) proj_bf16_kernel<MODE, true, true><<<grid, 256, 0, a.stream>>>(pp);
    else if (quad) proj_bf16_kernel<MODE, true, false><<<grid, 256, 0, a.stream>>>(pp);
    else if (v8) proj_bf16_kernel<MODE, false, true><<<grid, 256, 0, a.stream>>>(pp);
    else proj_bf16_kernel<MODE, false, false><<<grid, 256, 0, a.stream>>>(pp);
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
