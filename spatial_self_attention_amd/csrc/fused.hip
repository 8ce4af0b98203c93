// Projections and attention of one (sample, head) in one work-group, for
// short sequences (tensortonic "Spatial Self-Attention": Q = Z Wq^T + bq,
// K = Z Wk^T + bk, V = Z Wv^T + bv with Z = tokens(GN(x)), then per head
// O = softmax(Q K^T / sqrt(d)) V).
//
// When the T x d matrices of a head fit in LDS, the projection kernel's
// Q / K / V round trip through HBM (written once, read back by the attention
// kernel) and its rounds of 128 x 128 tiles are the larger part of the
// block's time.  Here one work-group of 8 waves owns one (b, head):
//
//  1. Q pass: Q = GN(x_b) Wq_h^T for the head's d channels and all T tokens,
//     written to LDS (bf16, times log2(e) / sqrt(d) as the scores want);
//  2. K/V pass: K and V the same way, kept in the MFMA accumulators; each
//     wave then takes its 32 queries' Q fragments from LDS into registers and
//     the accumulators go to LDS as K (token-major) and V^T (tokens in
//     vt_slot order), the layouts the attention steps read;
//  3. attention: wave w owns queries 32w .. 32w+31 and walks the keys from
//     LDS with the online softmax of the attention kernel, in its tiles of 64
//     keys and its order of score, softmax and P V steps, no global loads;
//  4. O = O^T / l, staged per wave in LDS and stored token-major into
//     (B, T, C) at the head's columns, as the attention kernel does.
//
// The projection passes are LDS-tiled GEMMs over the input channels in steps
// of 32: the weight rows (16-byte loads) and the x rows of the sample (8-byte
// loads of 4 tokens, normalised with the per-(b, c) GroupNorm coefficients
// and rounded to bf16 when written to LDS, as in the projection kernel) go
// through two LDS buffers, with two register stages so that each step's
// loads are issued two steps before their LDS writes.  Q and K come from
// D = W Z^T (a lane holds 4 consecutive channels of one token), V from
// D = Z W^T (4 consecutive tokens of one channel).  The bf16 values of Q, K
// and V are those the projection kernel stores (the same products in the
// same k order, the same bias add, scale and rounding), and the attention
// runs the same operations on them, so O is that of the two kernels, bit for
// bit.
//
// Work-group ids are remapped so that the heads of one sample (which read the
// same x) run on one XCD.
#include <type_traits>

#include "attn_core.h"

namespace ssa {
namespace {

struct FusedParams {
  const bf16* x;        // (B, C, T)
  const float2* coef;   // (B, C): GN(x) = a x + s
  const bf16* w[3];     // Wq, Wk, Wv (C, C), rows = output channels
  const bf16* bias[3];  // bq, bk, bv, or NULL
  bf16* o;              // (B, T, C)
  int B, C, T, n;
  float q_scale;        // log2(e) / sqrt(d)
};

constexpr int FNW = 8;         // waves per work-group
constexpr int FNT = 64 * FNW;  // threads

// Staging geometry of a pass that takes GK input channels per step.
template <int GK>
struct FGeom {
  static constexpr int GP = GK + 8;      // row pitch (bf16): 16-byte reads of 8 rows hit distinct banks
  static constexpr int CH = GK / 8;      // 16-byte chunks per weight row
  static constexpr int RPV = FNT / CH;   // weight rows per round of one vector per thread
  static constexpr int CQ = GK / 32;     // channel quads of x per thread
  static constexpr int SUB = GK / 16;    // MFMA sub-steps per step
};

template <int D, int NB>
struct FLayout {
  static constexpr int TOK = NB * 32;   // tokens, padded to whole 32-key blocks
  static constexpr int QP = D + 8;      // Q / K row pitch
  static constexpr int VP = TOK + 8;    // V^T row pitch
  // pass 1 (Q): two staging buffers from 0; Q is written
  // over them after the pass
  static constexpr int QGK = 32, KVGK = 32;
  static constexpr int QSZ = (D + TOK) * FGeom<QGK>::GP;
  static constexpr int QR = 0;          // Q (TOK x QP), passes 1-2
  // pass 2 (K/V, 32 channels per step): two staging buffers after Q
  static constexpr int ST = TOK * QP;
  static constexpr int STSZ = (2 * D + TOK) * FGeom<KVGK>::GP;
  static constexpr int KR = 0;          // K (TOK x QP), step 3
  static constexpr int VR = TOK * QP;   // V^T (D x VP), step 3
  static constexpr int A = ST + 2 * STSZ, A1 = 2 * QSZ, B = VR + D * VP, C = FNW * 32 * QP;
  static constexpr int AA = A > A1 ? A : A1;
  static constexpr int ELEMS = AA > B ? (AA > C ? AA : C) : (B > C ? B : C);
  static_assert(ELEMS * 2 <= 160 * 1024, "the work-group's LDS fits one CU");
};

// Input channels whose GroupNorm coefficients (8 bytes each) fit beside the
// work-group's tiles in the 160 KB of LDS.
template <int D, int NB>
constexpr int fused_max_c() { return (160 * 1024 - FLayout<D, NB>::ELEMS * 2) / 8; }
constexpr int kFusedMaxC = 1536;  // fused_max_c<128, 8>() rounded down to whole 128-channel heads

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// One step's loads in registers.  Thread (wave w, lane l): weight vectors
// v = tid + FNT*i, row ((v>>3) / CH)*8 + (v&7), chunk (v>>3) % CH, so that 8
// consecutive lanes write one 16-byte column of 8 rows (distinct banks);
// x: channels 4*(l&7) + 32q .. +3 (q < CQ) of the step, tokens
// 4*((l>>3) + 8w) .. +3.  (The GroupNorm coefficients of the sample sit in an
// LDS table.)
template <int GK, int R>
struct FStage {
  static constexpr int NWV = R / FGeom<GK>::RPV;
  bf16x8 w[NWV];
  u32x2 x[4 * FGeom<GK>::CQ];
};

// Per-thread load addressing of one pass (R weight rows: rows 0..D-1 from
// w[first], D..2D-1 from w[first+1]) through buffer resources: the
// per-thread byte offsets are fixed, each step only moves a scalar offset.
// (A tensor holds fewer than 2^31 elements, so bf16 byte offsets fit 32 bits.)
template <int GK, int R>
struct FLoad {
  static constexpr int NWV = R / FGeom<GK>::RPV;
  __amdgpu_buffer_rsrc_t rw[NWV];  // the weight matrix of vector i
  int vw[NWV];                     // byte offset of vector i's row and chunk at channel 0
  __amdgpu_buffer_rsrc_t rx;
  int vx;                          // byte offset of x[b][4*(l&7)][4*tq]
  int xrow;                        // bytes between channel rows of x (2T)
};

template <int D, int GK, int R>
__device__ __forceinline__ void f_setup(FLoad<GK, R>& ld, const FusedParams& fp, int first,
                                        int b, int head, int tid, int wave, int lane) {
  typedef FGeom<GK> G;
  static_assert(D % G::RPV == 0, "a round of weight rows lies in one matrix");
  const unsigned C = unsigned(fp.C), T = unsigned(fp.T);
#pragma unroll
  for (int i = 0; i < FLoad<GK, R>::NWV; ++i) {
    const int v = tid + FNT * i;
    const int r = ((v >> 3) / G::CH) * 8 + (v & 7);
    const int which = first + (G::RPV * i) / D;
    const bf16* w = which == 0 ? fp.w[0] : which == 1 ? fp.w[1] : fp.w[2];
    ld.rw[i] = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(w), 0, int(C * C * 2u),
                                                  kRsrcWord3);
    ld.vw[i] = int((unsigned(head * D + r % D) * C + unsigned((v >> 3) % G::CH) * 8u) * 2u);
  }
  const unsigned tq = unsigned(min((lane >> 3) + 8 * wave, int(T) / 4 - 1));  // padding tokens repeat the last quad
  const unsigned c4 = 4u * unsigned(lane & 7);
  ld.rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16*>(fp.x), 0,
                                            int(unsigned(fp.B) * C * T * 2u), kRsrcWord3);
  ld.vx = int(((unsigned(b) * C + c4) * T + 4u * tq) * 2u);
  ld.xrow = int(T * 2u);
}

// Every wave issues the same loads (a wave past the last token block reads
// the clamped quad and writes nothing), so the number of loads in flight is
// the same on every path and each step waits only for the loads it stores.
template <int GK, int R>
__device__ __forceinline__ void f_load(FStage<GK, R>& sg, const FLoad<GK, R>& ld, int k0) {
#pragma unroll
  for (int i = 0; i < FLoad<GK, R>::NWV; ++i)
    sg.w[i] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(ld.rw[i], ld.vw[i],
                                                                                k0 * 2, 0));
#pragma unroll
  for (int q = 0; q < FGeom<GK>::CQ; ++q)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      sg.x[4 * q + j] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
          ld.rx, ld.vx, int(unsigned(k0 + 32 * q + j) * unsigned(ld.xrow)), 0));
}

// Part p (one per MFMA sub-step) of writing a register stage (channels
// k0 ..) to a staging buffer: the weight vectors i with i % SUB == p, and two
// of the thread's (channel quad, token) items, normalised (GN(x) = a x + s in
// fp32, one bf16 rounding; (a, s) from the sample's coefficient table cft).
template <int GK, int R>
__device__ __forceinline__ void f_store(bf16* buf, const FStage<GK, R>& sg, const float2* cft,
                                        int k0, int tid, int wave, int lane, bool zact, int p) {
  typedef FGeom<GK> G;
#pragma unroll
  for (int i = 0; i < FStage<GK, R>::NWV; ++i) {
    if (i % G::SUB != p) continue;
    const int v = tid + FNT * i;
    const int r = ((v >> 3) / G::CH) * 8 + (v & 7);
    *reinterpret_cast<bf16x8*>(&buf[r * G::GP + ((v >> 3) % G::CH) * 8]) = sg.w[i];
  }
  if (zact) {
    bf16* Zs = buf + R * G::GP;
    const int tq = (lane >> 3) + 8 * wave;
    const int q = p / 2;  // items 2p, 2p+1: channel quad (2p)/4, tokens (2p)%4 ..
    const int c4 = 4 * (lane & 7) + 32 * q;
    const f32x4 cf[2] = {*reinterpret_cast<const f32x4*>(&cft[k0 + c4]),
                         *reinterpret_cast<const f32x4*>(&cft[k0 + c4 + 2])};
#pragma unroll
    for (int uu = 0; uu < 2; ++uu) {
      const int u = (2 * p + uu) % 4;
      bf16x4 z;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float a = cf[j >> 1][(j & 1) * 2], sh = cf[j >> 1][(j & 1) * 2 + 1];
        const unsigned w2 = sg.x[4 * q + j][u >> 1];
        const float xv = __uint_as_float((u & 1) ? (w2 & 0xffff0000u) : (w2 << 16));
        z[j] = static_cast<bf16>(fmaf(a, xv, sh));
      }
      *reinterpret_cast<bf16x4*>(&Zs[(4 * tq + u) * G::GP + c4]) = z;
    }
  }
}

// Sub-step s (16 channels) of one step for one wave: weight rows wrow ..
// wrow+63 (2 blocks) against token blocks tb0 .. tb0+NV-1.
template <int GK, int R, int NV, bool TR>
__device__ __forceinline__ void f_mfma(f32x16 (&acc)[2][NV], const bf16* buf, int wrow, int tb0,
                                       int half, int col, int s) {
  constexpr int GP = FGeom<GK>::GP;
  const bf16* Zs = buf + R * GP;
  const int ko = s * 16 + half * 8;
  bf16x8 fa[2], fb[NV];
#pragma unroll
  for (int i = 0; i < 2; ++i)
    fa[i] = *reinterpret_cast<const bf16x8*>(&buf[(wrow + i * 32 + col) * GP + ko]);
#pragma unroll
  for (int j = 0; j < NV; ++j)
    fb[j] = *reinterpret_cast<const bf16x8*>(&Zs[((tb0 + j) * 32 + col) * GP + ko]);
#pragma unroll
  for (int j = 0; j < NV; ++j)
#pragma unroll
    for (int i = 0; i < 2; ++i)
      acc[i][j] = TR ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0)
                     : __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
}

// One projection pass over all input channels: R weight rows (rows from
// w[first] then w[first+1]) x all tokens.  Wave w takes rows 64*(w % (R/64))
// .. +63 and token blocks TB*(w / (R/64)) .. +NV-1 (NV = TB except in the last
// wave group, which takes the blocks left below NB); TR: the wave's rows are
// V rows (swapped orientation).  st0/st1: the staging buffers.
template <int D, int NB, int GK, int R, int TB, int NV, bool TR, typename Epi>
__device__ __forceinline__ void f_pass(const FusedParams& fp, int first, bf16* st0, bf16* st1,
                                       const float2* cft, int b, int head, int tid, int wave,
                                       int lane, Epi& epi) {
  constexpr int WR = R / 64;
  const int half = lane >> 5, col = lane & 31;
  const int wrow = (wave % WR) * 64;
  const int tb0 = (wave / WR) * TB;
  const bool zact = wave < NB;  // the waves whose token quads lie below TOK
  f32x16 acc[2][NV];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < NV; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  FLoad<GK, R> ld;
  f_setup<D, GK, R>(ld, fp, first, b, head, tid, wave, lane);
  const int nk = fp.C / GK;  // even (C is a multiple of 128), >= 2
  FStage<GK, R> s0, s1;
  f_load(s0, ld, 0);
#pragma unroll
  for (int p = 0; p < FGeom<GK>::SUB; ++p) f_store<GK, R>(st0, s0, cft, 0, tid, wave, lane, zact, p);
  f_load(s1, ld, GK);
  // step ks reads rd; nxt (step ks+1) is written to wr when `more`; fre takes
  // the loads of step ks+2 when `load`
  auto step = [&](const bf16* rd, bf16* wr, const FStage<GK, R>& nxt, FStage<GK, R>& fre,
                  int ks, bool more, bool load) {
    __syncthreads();  // rd is complete; wr is no longer read
    if (load) f_load(fre, ld, (ks + 2) * GK);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < FGeom<GK>::SUB; ++s) {
      f_mfma<GK, R, NV, TR>(acc, rd, wrow, tb0, half, col, s);
      if (more) f_store<GK, R>(wr, nxt, cft, (ks + 1) * GK, tid, wave, lane, zact, s);
    }
  };
  // the register stages alternate at compile time (nk is even); steps
  // 0 .. nk-3 load, the last two do not
  for (int ks = 0; ks < nk - 2; ks += 2) {
    step(st0, st1, s1, s0, ks, true, true);
    step(st1, st0, s0, s1, ks + 1, true, true);
  }
  step(st0, st1, s1, s0, nk - 2, true, false);
  step(st1, st0, s0, s1, nk - 1, false, false);
  epi(acc, std::integral_constant<int, NV>(), std::integral_constant<bool, TR>());
}

// f_pass for this wave's group: WT = 8 / (R/64) groups of TB token blocks,
// the last one holding NB - (WT-1) TB of them.  epi(acc, NV, TR) runs after
// the pass with the accumulators of the wave's NV blocks.
template <int D, int NB, int GK, int R, int TB, bool TR, typename Epi>
__device__ __forceinline__ void f_pass_wave(const FusedParams& fp, int first, bf16* st0,
                                            bf16* st1, const float2* cft, int b, int head,
                                            int tid, int wave, int lane, Epi& epi) {
  constexpr int WT = FNW / (R / 64);
  constexpr int NVL = NB - (WT - 1) * TB;
  static_assert(NVL >= 1 && NVL <= TB, "every wave group has token blocks");
  if constexpr (NVL == TB) {
    f_pass<D, NB, GK, R, TB, TB, TR>(fp, first, st0, st1, cft, b, head, tid, wave, lane, epi);
  } else {
    if (wave / (R / 64) == WT - 1)
      f_pass<D, NB, GK, R, TB, NVL, TR>(fp, first, st0, st1, cft, b, head, tid, wave, lane, epi);
    else
      f_pass<D, NB, GK, R, TB, TB, TR>(fp, first, st0, st1, cft, b, head, tid, wave, lane, epi);
  }
}

template <int D, int NB>
__global__ __launch_bounds__(FNT, 1) void fused_bf16_kernel(FusedParams fp) {
  typedef FLayout<D, NB> L;
  __shared__ __attribute__((aligned(16))) bf16 lds[L::ELEMS];
  __shared__ __attribute__((aligned(16))) float2 cft[kFusedMaxC];  // GN (a, s) of sample b
  static_assert(kFusedMaxC <= fused_max_c<D, NB>(), "the coefficient table fits");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, col = lane & 31;
  const int lid = xcd_remap(int(blockIdx.x), int(gridDim.x));
  const int b = lid / fp.n, head = lid - b * fp.n;
  const int T = fp.T, C = fp.C;
  bf16* st0 = lds + L::ST;  // K/V pass staging
  bf16* st1 = lds + L::ST + L::STSZ;
  for (int c = tid; c < C; c += FNT) cft[c] = fp.coef[int64_t(b) * C + c];
  __syncthreads();  // the table is read from the first staging writes on

  // ---- 1. Q pass: rows = the head's d query channels ----
  {
    constexpr int TB = (NB + 3) / 4;
    const int wrow = (wave % (D / 64)) * 64, tb0 = (wave / (D / 64)) * TB;
    auto epi = [&](auto& acc, auto nv, auto) {
      constexpr int NV = decltype(nv)::value;
      int half = lane >> 5, col = lane & 31;
      asm volatile("" : "+v"(half), "+v"(col));  // keep the epilogue's addressing below the loop
      __syncthreads();  // every wave is done with the staging buffers Q is written over
      const bf16* bq = fp.bias[0];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int dd = wrow + i * 32 + 8 * g + 4 * half;
          const bf16x4 bv = bq ? *reinterpret_cast<const bf16x4*>(bq + head * D + dd) : bf16x4{};
#pragma unroll
          for (int j = 0; j < NV; ++j) {
            bf16x4 pk;
#pragma unroll
            for (int e = 0; e < 4; ++e)
              pk[e] = static_cast<bf16>((acc[i][j][4 * g + e] + static_cast<float>(bv[e])) *
                                        fp.q_scale);
            *reinterpret_cast<bf16x4*>(&lds[L::QR + ((tb0 + j) * 32 + col) * L::QP + dd]) = pk;
          }
        }
    };
    f_pass_wave<D, NB, L::QGK, D, TB, false>(fp, 0, lds, lds + L::QSZ, cft, b, head, tid, wave,
                                              lane, epi);
  }

  // ---- 2. K/V pass: rows 0..D-1 = K channels, D..2D-1 = V channels ----
  AttnState<D, 1> st;
  {
    constexpr int TB = (NB + 1) / 2;
    constexpr int WR = 2 * D / 64;
    const int wrow = (wave % WR) * 64, tb0 = (wave / WR) * TB;
    auto epi = [&](auto& acc, auto nv, auto tr) {
      constexpr int NV = decltype(nv)::value;
      int half = lane >> 5, col = lane & 31;
      asm volatile("" : "+v"(half), "+v"(col));  // keep the epilogue's addressing below the loop
      __syncthreads();  // the staging buffers and Q are complete
      // this wave's queries 32*wave + col: Q fragments (B operand of S^T = K Q^T)
      const bf16x8 zero8 = {};
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks)
        st.qf[0][ks] = wave < NB ? *reinterpret_cast<const bf16x8*>(
                                       &lds[L::QR + (wave * 32 + col) * L::QP + ks * 16 + half * 8])
                                 : zero8;
      __syncthreads();  // every wave has its Q: the region becomes K and V^T
      if constexpr (decltype(tr)::value) {  // V rows: V^T[channel][vt_slot(token)]
        const bf16* bvp = fp.bias[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int dd = wrow - D + i * 32 + col;
          const float bv = bvp ? static_cast<float>(bvp[head * D + dd]) : 0.f;
#pragma unroll
          for (int j = 0; j < NV; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              bf16x4 pk;
#pragma unroll
              for (int e = 0; e < 4; ++e) pk[e] = static_cast<bf16>(acc[i][j][4 * g + e] + bv);
              const int slot = vt_slot((tb0 + j) * 32 + 8 * g + 4 * half);
              *reinterpret_cast<bf16x4*>(&lds[L::VR + dd * L::VP + slot]) = pk;
            }
        }
      } else {  // K rows: K[token][channel]
        const bf16* bkp = fp.bias[1];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int dd = wrow + i * 32 + 8 * g + 4 * half;
            const bf16x4 bv =
                bkp ? *reinterpret_cast<const bf16x4*>(bkp + head * D + dd) : bf16x4{};
#pragma unroll
            for (int j = 0; j < NV; ++j) {
              bf16x4 pk;
#pragma unroll
              for (int e = 0; e < 4; ++e)
                pk[e] = static_cast<bf16>(acc[i][j][4 * g + e] + static_cast<float>(bv[e]));
              *reinterpret_cast<bf16x4*>(&lds[L::KR + ((tb0 + j) * 32 + col) * L::QP + dd]) = pk;
            }
          }
      }
    };
    if (wrow >= D)  // wave-uniform: V rows take the swapped orientation
      f_pass_wave<D, NB, L::KVGK, 2 * D, TB, true>(fp, 1, st0, st1, cft, b, head, tid, wave, lane,
                                                  epi);
    else
      f_pass_wave<D, NB, L::KVGK, 2 * D, TB, false>(fp, 1, st0, st1, cft, b, head, tid, wave, lane,
                                                   epi);
  }
  __syncthreads();  // K and V^T are complete

  // ---- 3. attention of the wave's 32 queries over all keys ----
  const bool qact = wave < NB && wave * 32 < T;  // wave-uniform
  if (qact) {
#pragma unroll
    for (int r = 0; r < 16; ++r) st.nm[0][r] = 0.f;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.o[0][db][r] = 0.f;
    st.m[0] = 0.f;
    st.l[0] = 0.f;
    const bf16* Ks = lds + L::KR;
    const bf16* Vs = lds + L::VR;
    auto read_k = [&](KFrag<D>& f, int kb) {
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks)
        f.a[ks] = *reinterpret_cast<const bf16x8*>(&Ks[(kb * 32 + col) * L::QP + ks * 16 + half * 8]);
    };
    auto read_v = [&](VFrag<D>& f, int kb) {
#pragma unroll
      for (int gp = 0; gp < 2; ++gp)
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
          f.a[gp][db] = *reinterpret_cast<const bf16x8*>(
              &Vs[(db * 32 + col) * L::VP + kb * 32 + 16 * gp + 8 * half]);
    };
    RelPos<1> rp{};
    f32x16 sc[2][1];
    bf16x8 pb[2][1][2];
    float delta[1];
    // Keys in tiles of 64 (two 32-key blocks), each tile pipelined as in the
    // attention kernel (QK^T of block 1 issued before the softmax of block 0,
    // P V of block 0 after it), and a partial last tile one block at a time:
    // the same operations in the same order as that kernel, so O is the same.
    const int nfull = T / 64, ntiles = (T + 63) / 64;
    for (int j = 0; j < nfull; ++j) {
      KFrag<D> kf[2];
      VFrag<D> vf[2];
      read_k(kf[0], 2 * j);
      qk_mfma<D, 1>(sc[0], st, kf[0]);
      read_k(kf[1], 2 * j + 1);
      qk_mfma<D, 1>(sc[1], st, kf[1]);
      const bool raised = softmax_block<D, 1, 64, false, 0>(st, sc[0], pb[0], delta, 0, 64 * j, T,
                                                            half, j == 0, rp);
      if (raised) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[1][0][r] -= delta[0];
      }
      read_v(vf[0], 2 * j);
      pv_mfma<D, 1>(st, pb[0], vf[0]);
      softmax_block<D, 1, 64, false, 0>(st, sc[1], pb[1], delta, 1, 64 * j, T, half, false, rp);
      read_v(vf[1], 2 * j + 1);
      pv_mfma<D, 1>(st, pb[1], vf[1]);
    }
    if (nfull < ntiles) {
      const int nv = min(2, (T - 64 * nfull + 31) / 32);
      for (int kb = 0; kb < nv; ++kb) {
        KFrag<D> kf;
        VFrag<D> vf;
        read_k(kf, 2 * nfull + kb);
        qk_mfma<D, 1>(sc[0], st, kf);
        softmax_block<D, 1, 64, true, 0>(st, sc[0], pb[0], delta, kb, 64 * nfull, T, half,
                                         nfull == 0 && kb == 0, rp);
        read_v(vf, 2 * nfull + kb);
        pv_mfma<D, 1>(st, pb[0], vf);
      }
    }
  }
  __syncthreads();  // every wave is done with K and V^T: LDS becomes output staging

  // ---- 4. O = O^T / l, staged per wave, 16-byte stores of whole rows ----
  if (qact) {
    constexpr int EP = L::QP;
    bf16* stg = lds + wave * 32 * EP;
    const float inv = 1.0f / halves_sum(st.l[0]);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 pk;
#pragma unroll
        for (int e = 0; e < 4; ++e) pk[e] = static_cast<bf16>(st.o[0][db][4 * g + e] * inv);
        *reinterpret_cast<bf16x4*>(&stg[col * EP + db * 32 + 8 * g + 4 * half]) = pk;
      }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    constexpr int CPR = D / 8;  // 16-byte chunks per query row
    bf16* O = fp.o + int64_t(b) * T * C + head * D;
#pragma unroll
    for (int i = 0; i < D / 16; ++i) {
      const int c = lane + 64 * i;
      const int q = c / CPR, dc = c % CPR;
      const int qi = wave * 32 + q;
      if (qi < T)
        store_nt(O + int64_t(qi) * C + dc * 8, *reinterpret_cast<const bf16x8*>(&stg[q * EP + dc * 8]));
    }
  }
}

}  // namespace

bool fused_available(const Plan& p) {
  return p.dtype == SSA_BF16 && p.d == 128 && p.T % 4 == 0 && p.T > 192 && p.T <= 256 &&
         p.C % 64 == 0 && p.C <= kFusedMaxC && p.B * p.n >= p.cus;
}

hipError_t launch_fused(const Plan& p, const Args& a) {
  FusedParams fp{};
  fp.x = static_cast<const bf16*>(a.x);
  fp.coef = reinterpret_cast<const float2*>(a.ws + p.ws.gn_coef);
  for (int i = 0; i < 3; ++i) {
    fp.w[i] = static_cast<const bf16*>(a.w[i]);
    fp.bias[i] = static_cast<const bf16*>(a.b[i]);
  }
  fp.o = reinterpret_cast<bf16*>(a.ws + p.ws.o);
  fp.B = int(p.B);
  fp.C = int(p.C);
  fp.T = int(p.T);
  fp.n = int(p.n);
  fp.q_scale = kLog2e / sqrtf(float(p.d));
  const unsigned grid = unsigned(p.B * p.n);
  if (p.T <= 224)
    fused_bf16_kernel<128, 7><<<grid, FNT, 0, a.stream>>>(fp);
  else
    fused_bf16_kernel<128, 8><<<grid, FNT, 0, a.stream>>>(fp);
  return hipGetLastError();
}

}  // namespace ssa
