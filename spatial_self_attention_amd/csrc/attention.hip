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
// with the scores in the log2 domain (s = q.k * log2(e) / sqrt(d); the bf16
// path gets Q already multiplied by log2(e) / sqrt(d) from the projection).
//
// bf16 kernel (gfx950 MFMA): 4 waves x 32 queries per work-group, key tiles of
// 64 double-buffered in LDS (the next tile is fetched into registers while the
// current one is used).  The score block is formed TRANSPOSED, S^T = K Q^T with
// v_mfma_f32_32x32x16_bf16, so each lane holds one query (its column) and 16
// keys per 32-key sub-block:
//  * the row max / row sum need no shuffles except one exchange with lane^32
//    (the other half of the keys of the same query);
//  * the rescale by 2^(m - m') is per lane;
//  * the probabilities, rounded to bf16, are already in the register layout of
//    MFMA's B operand for O^T += V^T P^T, up to a permutation of the key
//    index that the V^T operand loads apply identically (a dot product does
//    not depend on the order of its terms).
// V is read from the transposed (d, Tp) layout whose tokens sit in vt_slot
// order, so each V^T operand is one conflict-free 16-byte LDS read.  O is
// written token-major (B, T, C), heads concatenated.
// The softmax runs per 32-key sub-block; the QK^T MFMAs of the next sub-block
// are issued before it so matrix-core and VALU work overlap.  The running max
// m is subtracted by the matrix core (the score MFMAs accumulate onto a C
// operand holding -m), so a probability costs one v_exp, half a v_cvt_pk and
// one v_add (the row sum).  m is raised lazily, only when a lane's 16 probabilities of a
// sub-block sum past 2^8; then O and l are rescaled and that sub-block redone.
//
// Long sequences at d = 64 take kernels with two 32-query blocks per wave
// (each K and V^T fragment read feeds two MFMAs): attn2_bf16_kernel (512- or
// 256-query work-groups) and attnpp_bf16_kernel (one 8-wave work-group per
// 256-query tile, two 4-wave groups walking the two halves of the keys in
// alternating half steps -- one wave of each SIMD issues MFMAs while the other
// runs its softmax -- merged in LDS at the end).  When the tiles of a last,
// partial round fill at most half the CUs, each of them is cut into key ranges
// run as separate work-groups, whose partial (O, m, l) attn_merge_kernel
// combines.  The relative-position bias (REL) is staged per key tile as a
// slice of the head's table column in LDS.
//
// fp32 kernel: 64 queries x 4 lanes per query (each lane owns d/4 dims),
// FMA only, key tiles of 32 in LDS.
#include <math.h>

#include "attn_core.h"

namespace ssa {
namespace {

struct AttnParams {
  const void* q;   // (B, n, T, dp)
  const void* k;   // (B, n, T, dp)
  const void* vt;  // (B, n, dp, Tp)
  void* o;         // (B, T, C)
  int T, Tp, n, d, C;  // d: the head's width (bf16 kernels run at D = dp >= d)
  int qtiles;      // query tiles per (b, head)
  float scale;     // log2(e) / sqrt(d) (fp32 path; log2(e) with query/key normalisation)
  const void* rel; // ((2H-1)(2W-1), n) relative-position table, or NULL
  int H, W;
  // key-splitting kernel: tiles [0, full) run whole, each later tile as
  // `split` key ranges whose (O, m, l) go to `part` for attn_merge_kernel
  int full, split;
  float* part;
};

// ---------------------------------------------------------------------------
// bf16 MFMA kernel
// ---------------------------------------------------------------------------
template <int D, int QB, int KT, int NW = 4>
struct Tile {
  static constexpr int QPW = 32 * QB;      // queries per wave
  static constexpr int QT = NW * QPW;      // queries per work-group (NW waves)
  static constexpr int NTHR = 64 * NW;     // threads per work-group
  static constexpr int NKB = KT / 32;      // 32-key sub-blocks per tile
  static constexpr int KP = D + 8;         // K tile row pitch (bf16)
  static constexpr int VP = KT + 8;        // V^T tile row pitch (bf16)
  static constexpr int KSZ = KT * KP;      // K tile (bf16 elements)
  static constexpr int VSZ = D * VP;       // V^T tile
  static constexpr int BUF = KSZ + VSZ;
  static constexpr int VPT = KT * D / 8 / NTHR;  // 16-byte vectors per thread per operand
  static_assert(VPT * NTHR == KT * D / 8, "tile vectors must split evenly over the threads");
};


// Registers holding the next K and V^T tiles while the current one is used.
template <int D, int QB, int KT, int NW>
struct Prefetch {
  u32x4 k[Tile<D, QB, KT, NW>::VPT];
  u32x4 v[Tile<D, QB, KT, NW>::VPT];
};

// Global -> registers for one K tile and one V^T tile (keys k0 .. k0+KT-1),
// through buffer resources based at the tile, so the per-thread offsets are
// loop-invariant.  K rows >= T lie past num_records and read as zero; MASK
// zeroes the V^T slots of tokens >= T (their columns are never written).
template <int D, int QB, int KT, int NW, bool MASK>
__device__ __forceinline__ void load_tile(Prefetch<D, QB, KT, NW>& pf, const bf16* K, const bf16* Vt,
                                          int Tp, int k0, int T, int tid) {
  typedef Tile<D, QB, KT, NW> TL;
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(K + int64_t(k0) * D, int64_t(T - k0) * D * 2);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(Vt + k0, (int64_t(D) * Tp - k0) * 2);
#pragma unroll
  for (int i = 0; i < TL::VPT; ++i)
    pf.k[i] = __builtin_amdgcn_raw_buffer_load_b128(kr, (tid + TL::NTHR * i) * 16, 0, 0);
#pragma unroll
  for (int i = 0; i < TL::VPT; ++i) {
    const int v = tid + TL::NTHR * i;
    const int r = v / (KT / 8), c8 = v % (KT / 8);
    u32x4 val = __builtin_amdgcn_raw_buffer_load_b128(vr, (r * Tp + c8 * 8) * 2, 0, 0);
    if (MASK) {  // slot k0+c8*8+e holds token vt_slot(k0+c8*8+e)
      const int key = k0 + c8 * 8;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const unsigned lo = vt_slot(key + 2 * w) < T ? 0xffffu : 0u;
        const unsigned hi = vt_slot(key + 2 * w + 1) < T ? 0xffff0000u : 0u;
        val[w] &= lo | hi;
      }
    }
    pf.v[i] = val;
  }
}

template <int D, int QB, int KT, int NW>
__device__ __forceinline__ void store_tile(bf16* buf, const Prefetch<D, QB, KT, NW>& pf, int tid) {
  typedef Tile<D, QB, KT, NW> TL;
#pragma unroll
  for (int i = 0; i < TL::VPT; ++i) {
    const int v = tid + TL::NTHR * i;
    const int r = v / (D / 8), c8 = v % (D / 8);
    *reinterpret_cast<u32x4*>(&buf[r * TL::KP + c8 * 8]) = pf.k[i];
  }
#pragma unroll
  for (int i = 0; i < TL::VPT; ++i) {
    const int v = tid + TL::NTHR * i;
    const int r = v / (KT / 8), c8 = v % (KT / 8);
    *reinterpret_cast<u32x4*>(&buf[TL::KSZ + r * TL::VP + c8 * 8]) = pf.v[i];
  }
}

// Global -> LDS for one full K and V^T tile without VGPRs: buffer loads that
// write LDS directly, 16 bytes per lane, each wave instruction filling 64
// consecutive 16-byte chunks of the tile buffer (a K row is D/8 chunks and one
// chunk of padding, a V^T row KT/8 and one: the padding chunks load the row's
// first chunk again and are never read).  The rows' padding keeps the operand
// fragment reads free of bank conflicts, as with the register path.
template <int D, int QB, int KT, int NW>
__device__ __forceinline__ void dma_tile(bf16* buf, const bf16* K, const bf16* Vt, int Tp, int k0,
                                         int T, int wave, int lane) {
  typedef Tile<D, QB, KT, NW> TL;
  constexpr int KC = TL::KP / 8, VC = TL::VP / 8;  // 16-byte chunks per row
  constexpr int NK = KT * KC, NV = D * VC;         // chunks per region
  static_assert(NK % 64 == 0 && NV % 64 == 0, "every wave instruction stays in one region");
  constexpr int NI = (NK + NV) / 64;               // wave instructions per tile
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(K + int64_t(k0) * D, int64_t(T - k0) * D * 2);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(Vt + k0, (int64_t(D) * Tp - k0) * 2);
#pragma unroll
  for (int i0 = 0; i0 < NI; i0 += NW) {
    const int i = i0 + wave;  // wave-uniform
    if (i < NI) {
      bf16* dst = buf + i * 64 * 8;  // this instruction's chunks (the LDS base goes to M0)
      const int c = i * 64 + lane;
      if (i * 64 < NK) {
        const int r = c / KC, ch = c % KC;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, dst, 16, (r * D + (ch < D / 8 ? ch : 0) * 8) * 2,
                                                 0, 0, 0);
      } else {
        const int r = (c - NK) / VC, ch = (c - NK) % VC;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, dst, 16,
                                                 (r * Tp + (ch < KT / 8 ? ch : 0) * 8) * 2, 0, 0, 0);
      }
    }
  }
}

template <int D, int QB, int KT>
__device__ __forceinline__ void read_k(KFrag<D>& f, const bf16* Ks, int kb, int half, int col) {
  typedef Tile<D, QB, KT> TL;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
    f.a[ks] = *reinterpret_cast<const bf16x8*>(&Ks[(kb * 32 + col) * TL::KP + ks * 16 + half * 8]);
}

// The B operand element e of MFMA step gp is key kb*32 + 16*gp + 8*(e/4) +
// 4*half + e%4; V^T rows hold token t in slot vt_slot(t), which puts those 8
// keys at slots kb*32 + 16*gp + 8*half + e: one 16-byte read.
template <int D, int QB, int KT>
__device__ __forceinline__ void read_v(VFrag<D>& f, const bf16* Vs, int kb, int half, int col) {
  typedef Tile<D, QB, KT> TL;
#pragma unroll
  for (int gp = 0; gp < 2; ++gp)
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
      f.a[gp][db] = *reinterpret_cast<const bf16x8*>(
          &Vs[(db * 32 + col) * TL::VP + kb * 32 + 16 * gp + 8 * half]);
}

// One key tile for one wave, software-pipelined over its 32-key sub-blocks.
// Step kb runs the softmax of sub-block kb on the VALU while the matrix core
// works on QK^T of sub-block kb+1 and P V of sub-block kb-1; the LDS operand
// fragments those MFMAs need were read during step kb-1, and step kb reads
// the fragments of step kb+1 (K of kb+2, V of kb).  When the softmax raises
// m, the scores of kb+1 (formed against the old m) are shifted by the raise.
template <int D, int QB, int KT, bool MASK, int REL>
__device__ __forceinline__ void attend_tile(AttnState<D, QB>& st, const bf16* buf, int k0,
                                            int T, int half, int col, bool first,
                                            const RelPos<QB>& rp) {
  typedef Tile<D, QB, KT> TL;
  constexpr int NKB = TL::NKB;
  const bf16* Ks = buf;
  const bf16* Vs = buf + TL::KSZ;
  f32x16 s[2][QB];
  bf16x8 pb[2][QB][2];
  float delta[QB];
  if constexpr (MASK) {
    // The partial last tile: only its sub-blocks that hold keys < T, one at a
    // time (the tile is visited once per work-group).
    const int nv = min(NKB, (T - k0 + 31) / 32);
    for (int kb = 0; kb < nv; ++kb) {
      KFrag<D> kf;
      VFrag<D> vf;
      read_k<D, QB, KT>(kf, Ks, kb, half, col);
      qk_mfma<D, QB>(s[0], st, kf);
      softmax_block<D, QB, KT, true, REL>(st, s[0], pb[0], delta, kb, k0, T, half,
                                          first && kb == 0, rp);
      read_v<D, QB, KT>(vf, Vs, kb, half, col);
      pv_mfma<D, QB>(st, pb[0], vf);
    }
    return;
  }
  // Wide heads (d > 64) read their fragments in the step that uses them:
  // their MFMA work per step is twice as long, and two fragment sets would
  // not fit beside the accumulators.
  constexpr bool kAhead = D <= 64;
  KFrag<D> kf[2];
  VFrag<D> vf[2];
  read_k<D, QB, KT>(kf[0], Ks, 0, half, col);
  if (kAhead && NKB > 1) read_k<D, QB, KT>(kf[1], Ks, 1, half, col);
  qk_mfma<D, QB>(s[0], st, kf[0]);
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    if (kAhead) {
      // fragments for the next step: K of kb+2, V of kb
      if (kb + 2 < NKB) read_k<D, QB, KT>(kf[kb & 1], Ks, kb + 2, half, col);
      read_v<D, QB, KT>(vf[kb & 1], Vs, kb, half, col);
    } else {
      if (kb + 1 < NKB) read_k<D, QB, KT>(kf[(kb + 1) & 1], Ks, kb + 1, half, col);
      if (kb > 0) read_v<D, QB, KT>(vf[(kb - 1) & 1], Vs, kb - 1, half, col);
    }
    if (kb + 1 < NKB) qk_mfma<D, QB>(s[(kb + 1) & 1], st, kf[(kb + 1) & 1]);
    if (kb > 0) pv_mfma<D, QB>(st, pb[(kb - 1) & 1], vf[(kb - 1) & 1]);
    const bool raised = softmax_block<D, QB, KT, MASK, REL>(st, s[kb & 1], pb[kb & 1], delta, kb,
                                                            k0, T, half, first && kb == 0, rp);
    if (kb + 1 < NKB && raised) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[(kb + 1) & 1][qb][r] -= delta[qb];
    }
  }
  if (!kAhead) read_v<D, QB, KT>(vf[(NKB - 1) & 1], Vs, NKB - 1, half, col);
  pv_mfma<D, QB>(st, pb[(NKB - 1) & 1], vf[(NKB - 1) & 1]);
}

// Per-wave state for queries qbase + 32 qb + col: Q fragments, zero O, m, l.
template <int D, int QB>
__device__ __forceinline__ void init_state(AttnState<D, QB>& st, const bf16* Q, int qbase, int T,
                                           int half, int col) {
  const bf16x8 zero8 = {};
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qi = qbase + qb * 32 + col;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
      st.qf[qb][ks] = qi < T ? *reinterpret_cast<const bf16x8*>(Q + int64_t(qi) * D + ks * 16 +
                                                                 half * 8)
                             : zero8;
#pragma unroll
    for (int r = 0; r < 16; ++r) st.nm[qb][r] = 0.f;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.o[qb][db][r] = 0.f;
    st.m[qb] = 0.f;
    st.l[qb] = 0.f;
  }
}

// O = O^T accumulators / l, token-major (B, T, C) with heads concatenated.
// A lane holds runs of 4 dims of one query, so the wave first stages its
// 32*QB queries x D in LDS (rows of D + 8 bf16, its own region `stg`), then
// stores 16 bytes per lane with each query's D dims contiguous: whole rows of
// the output instead of 8-byte pieces of 32 rows per instruction.
template <int D, int QB>
__device__ __forceinline__ void write_o(const AttnState<D, QB>& st, const AttnParams& ap, int b,
                                        int head, int qbase, int half, int col, int lane,
                                        bf16* stg) {
  constexpr int EP = D + 8;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float inv = 1.0f / halves_sum(st.l[qb]);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 pk;
#pragma unroll
        for (int e = 0; e < 4; ++e) pk[e] = static_cast<bf16>(st.o[qb][db][4 * g + e] * inv);
        *reinterpret_cast<bf16x4*>(&stg[(qb * 32 + col) * EP + db * 32 + 8 * g + 4 * half]) = pk;
      }
  }
  // the wave reads what its own lanes wrote: LDS operations of one wave stay in order
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  constexpr int CPR = D / 8;  // 16-byte chunks per query row
  // a head of d < D channels (zero-padded operands): its first d columns
  const int d = ap.d;
  bf16* O = static_cast<bf16*>(ap.o) + (int64_t(b) * ap.T) * ap.C + head * d;
  if (d == D) {
#pragma unroll
    for (int i = 0; i < QB * D / 16; ++i) {
      const int c = lane + 64 * i;
      const int q = c / CPR, dc = c % CPR;
      const int qi = qbase + q;
      if (qi < ap.T)
        store_nt(O + int64_t(qi) * ap.C + dc * 8, *reinterpret_cast<const bf16x8*>(&stg[q * EP + dc * 8]));
    }
  } else {
    for (int i = 0; i < QB * D / 16; ++i) {
      const int c = lane + 64 * i;
      const int q = c / CPR, dc = c % CPR;
      const int qi = qbase + q;
      if (qi < ap.T && dc * 8 < d)
        for (int e = 0; e < 8 && dc * 8 + e < d; ++e)
          O[int64_t(qi) * ap.C + dc * 8 + e] = stg[q * EP + dc * 8 + e];
    }
  }
}

// Three work-groups per CU (12 waves) for the narrow heads; the wide heads
// need more registers and run two.
template <int D>
constexpr int attn_min_blocks() { return D <= 64 ? 3 : 2; }

// NW = 4: 128 queries per work-group, several work-groups per CU.  NW = 8:
// 256 queries per work-group, used for short sequences (T <= 256, one
// work-group per (sample, head)) so that K and V are read once per head.
// (The relative-position variant needs a few more registers: two work-groups per CU.)
template <int D, int QB, int KT, int NW, int REL>
__global__ __launch_bounds__(64 * NW, NW == 4 ? (REL != 0 ? 2 : attn_min_blocks<D>()) : 1) void attn_bf16_kernel(AttnParams ap) {
  typedef Tile<D, QB, KT, NW> TL;
  __shared__ __attribute__((aligned(16))) bf16 lds[2 * TL::BUF];
  __shared__ float rel_lds[REL == 2 ? 2 * kRelSlice : 1];  // table slices of two key tiles
  __shared__ __attribute__((aligned(16))) int kterm_lds[REL == 2 ? 2 * KT : 1];  // their key terms

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int lid = xcd_remap(int(blockIdx.x), int(gridDim.x));
  const int qtile = lid % ap.qtiles;
  const int bh = lid / ap.qtiles;  // b * n + head
  const int head = bh % ap.n, b = bh / ap.n;
  const int T = ap.T;

  const bf16* Q = static_cast<const bf16*>(ap.q) + int64_t(bh) * T * D;
  const bf16* K = static_cast<const bf16*>(ap.k) + int64_t(bh) * T * D;
  const bf16* Vt = static_cast<const bf16*>(ap.vt) + int64_t(bh) * D * ap.Tp;

  AttnState<D, QB> st;
  init_state<D, QB>(st, Q, qtile * TL::QT + wave * TL::QPW, T, half, col);
  RelPos<QB> rp;
  if constexpr (REL != 0) {
    rp.tab = static_cast<const bf16*>(ap.rel) + head;
    rp.H = ap.H;
    rp.W = ap.W;
    rp.w4 = ap.W % 4 == 0;
    rp.n = ap.n;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {  // rows past T take the last query's place
      const int qi = min(qtile * TL::QT + wave * TL::QPW + qb * 32 + col, T - 1);
      rp.qr[qb] = qi / ap.W;
      rp.qc[qb] = qi - rp.qr[qb] * ap.W;
    }
  }

  const int ntiles = (T + KT - 1) / KT;
  const int nfull = T / KT;
  // REL = 2: the table slice of key tile j travels with the tile (loaded with
  // the tile's prefetch, written to rel_lds slot j&1 with it).
  constexpr int RPT = REL == 2 ? kRelSlice / TL::NTHR : 1;  // slice entries per thread
  float rel_pf[RPT];
  int kterm_pf = 0;  // key term of key k0 + tid (tid < KT); keys past T take key T-1's
  auto q_range = [&](int& q0, int& q1) {
    q0 = qtile * TL::QT;
    q1 = min(q0 + TL::QT, T) - 1;
  };
  auto rel_load = [&](int k0) {
    if constexpr (REL == 2) {
      int q0, q1, lo, len;
      q_range(q0, q1);
      rel_rows(q0, q1, k0, min(k0 + KT, T) - 1, ap.H, ap.W, lo, len);
#pragma unroll
      for (int u = 0; u < RPT; ++u) {
        const int i = tid + TL::NTHR * u;
        rel_pf[u] = i < len ? kLog2e * static_cast<float>(rp.tab[int64_t(lo + i) * ap.n]) : 0.f;
      }
      const int key = min(k0 + tid, T - 1);
      const int kr = key / ap.W;
      kterm_pf = kr * (2 * ap.W - 1) + (key - kr * ap.W);
    }
  };
  auto rel_store = [&](int slot) {
    if constexpr (REL == 2) {
#pragma unroll
      for (int u = 0; u < RPT; ++u) rel_lds[slot * kRelSlice + tid + TL::NTHR * u] = rel_pf[u];
      if (tid < KT) kterm_lds[slot * KT + tid] = kterm_pf;
    }
  };
  auto rel_use = [&](int j) {  // the slice of tile j (its LDS slot and first row)
    if constexpr (REL == 2) {
      int q0, q1, len;
      q_range(q0, q1);
      rel_rows(q0, q1, j * KT, min(j * KT + KT, T) - 1, ap.H, ap.W, rp.lo, len);
      rp.slice = rel_lds + (j & 1) * kRelSlice;
      rp.kterm = kterm_lds + (j & 1) * KT;
      rp.k0 = j * KT;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        rp.qrow[qb] = (rp.qr[qb] + ap.H - 1) * (2 * ap.W - 1) + rp.qc[qb] + ap.W - 1 - rp.lo;
    }
  };
  Prefetch<D, QB, KT, NW> pf;
  if (nfull > 0)
    load_tile<D, QB, KT, NW, false>(pf, K, Vt, ap.Tp, 0, T, tid);
  else
    load_tile<D, QB, KT, NW, true>(pf, K, Vt, ap.Tp, 0, T, tid);
  rel_load(0);
  store_tile<D, QB, KT, NW>(lds, pf, tid);
  rel_store(0);

  for (int j = 0; j < nfull; ++j) {
    __syncthreads();  // tile j is in buffer j&1; buffer (j+1)&1 is free
    const int kn = (j + 1) * KT;
    if (j + 1 < nfull)
      load_tile<D, QB, KT, NW, false>(pf, K, Vt, ap.Tp, kn, T, tid);
    else if (j + 1 < ntiles)
      load_tile<D, QB, KT, NW, true>(pf, K, Vt, ap.Tp, kn, T, tid);
    if (j + 1 < ntiles) rel_load(kn);
    rel_use(j);
    attend_tile<D, QB, KT, false, REL>(st, lds + (j & 1) * TL::BUF, j * KT, T, half, col, j == 0,
                                       rp);
    if (j + 1 < ntiles) {
      store_tile<D, QB, KT, NW>(lds + ((j + 1) & 1) * TL::BUF, pf, tid);
      rel_store((j + 1) & 1);
    }
  }
  if (nfull < ntiles) {  // the partial last tile
    __syncthreads();
    rel_use(nfull);
    attend_tile<D, QB, KT, true, REL>(st, lds + (nfull & 1) * TL::BUF, nfull * KT, T, half, col,
                                      nfull == 0, rp);
  }

  __syncthreads();  // every wave is done with the key tiles: LDS becomes staging
  static_assert(NW * 32 * QB * (D + 8) <= 2 * TL::BUF, "output staging fits the tile buffers");
  write_o<D, QB>(st, ap, b, head, qtile * TL::QT + wave * TL::QPW, half, col, lane,
                 lds + wave * 32 * QB * (D + 8));
}

// ---------------------------------------------------------------------------
// bf16 MFMA kernel with two 32-query blocks per wave
// ---------------------------------------------------------------------------
// Every K and V^T operand fragment a wave reads from LDS feeds two MFMAs, one
// per query block, so the LDS reads per MFMA are half those of the one-block
// kernel (at the price of 256 VGPRs: two waves per SIMD).  Full key tiles come
// from global memory straight into LDS (dma_tile) and are walked by pipe_tile,
// which issues each block's softmax beside eight MFMAs that do not wait for
// it; the partial last tile goes through registers and attend_tile2 (both
// blocks' scores, then block by block the softmax and O^T += V^T P^T).

// Online softmax of one query block's 32-key sub-block (scores relative to
// its running max): the bf16 probabilities in MFMA B-operand order and the
// row-sum update; m is raised (and O, l rescaled) as in softmax_block.
template <int D, int QB, bool MASK, bool PIN = false>
__device__ __forceinline__ void softmax_qb(AttnState<D, QB>& st, int qb, f32x16& s,
                                           bf16x8 (&pb)[2], int kfirst, int T, int half,
                                           bool first) {
  if constexpr (MASK) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (kfirst + 8 * (r >> 2) + 4 * half + (r & 3) >= T) s[r] = -INFINITY;
  }
  float part = probs(pb, s, 0.f);
  // PIN: the bf16 probabilities are formed before the branch (beside the
  // MFMAs already issued) rather than sunk into the common path after it
  if (PIN) asm volatile("" : : "v"(pb[0]), "v"(pb[1]));
  if (first || __builtin_amdgcn_ballot_w64(!(part <= kLazySum))) {
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = halves_max(mx);
    const float m_new = first ? mx : fmaxf(st.m[qb], st.m[qb] + mx);
    const float delta = m_new - st.m[qb];
    if (!first) {
      const float alpha = __builtin_amdgcn_exp2f(-delta);
      st.l[qb] *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) st.o[qb][db][r] *= alpha;
    }
    st.m[qb] = m_new;
    // in place, so that the common path (no raise) needs no copy of nm
#pragma unroll
    for (int r = 0; r < 16; ++r) st.nm[qb][r] = first ? -m_new : st.nm[qb][r] - delta;
    part = probs(pb, s, delta);
  }
  st.l[qb] += part;
}

// 2^(s - delta) of one lane's 16 scores as bf16 (MFMA B-operand order) and
// their fp32 sum, added as a tree (depth 4: the adds wait less on each other
// than in two running chains).
__device__ __forceinline__ float probs_tree(bf16x8 (&pb)[2], const f32x16& s, float delta) {
  float p[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(s[r] - delta);
  float t[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) t[i] = p[2 * i] + p[2 * i + 1];
#pragma unroll
  for (int i = 0; i < 4; ++i) t[i] = t[2 * i] + t[2 * i + 1];
  t[0] = t[0] + t[1];
  t[2] = t[2] + t[3];
#pragma unroll
  for (int gp = 0; gp < 2; ++gp)
#pragma unroll
    for (int e = 0; e < 8; ++e) pb[gp][e] = static_cast<bf16>(p[8 * gp + e]);
  return t[0] + t[2];
}

// Online softmax of both query blocks' 32-key sub-block at once: their 32
// exponentials and two sum trees are independent work the VALU can overlap,
// and one lazy check covers the pair (a raise then updates both blocks: with
// a block's max below its m the raise leaves that block unchanged).
template <int D>
__device__ __forceinline__ void softmax_pair(AttnState<D, 2>& st, f32x16 (&s)[2],
                                             bf16x8 (&pb)[2][2], bool first) {
  float part[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) part[qb] = probs_tree(pb[qb], s[qb], 0.f);
  if (first || __builtin_amdgcn_ballot_w64(!(fmaxf(part[0], part[1]) <= kLazySum))) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float mx = s[qb][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[qb][r]);
      mx = halves_max(mx);
      const float m_new = first ? mx : fmaxf(st.m[qb], st.m[qb] + mx);
      const float delta = m_new - st.m[qb];
      if (!first) {
        const float alpha = __builtin_amdgcn_exp2f(-delta);
        st.l[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) st.o[qb][db][r] *= alpha;
      }
      st.m[qb] = m_new;
#pragma unroll
      for (int r = 0; r < 16; ++r) st.nm[qb][r] = first ? -m_new : st.nm[qb][r] - delta;
      part[qb] = probs_tree(pb[qb], s[qb], delta);
    }
  }
  st.l[0] += part[0];
  st.l[1] += part[1];
}

// O^T += V^T P^T of one query block.
template <int D, int QB>
__device__ __forceinline__ void pv_qb(AttnState<D, QB>& st, int qb, const bf16x8 (&pb)[2],
                                      const VFrag<D>& f) {
#pragma unroll
  for (int gp = 0; gp < 2; ++gp)
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
      st.o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[gp][db], pb[gp], st.o[qb][db], 0, 0, 0);
}

// One key tile for one wave holding two query blocks.  kf holds the K
// fragments of the tile's first sub-block on entry (each sub-block reads the
// next one's while its scores are formed).  PRIO: the wave raises its issue
// priority from its scores until the first block's P V products are issued,
// so that of two waves sharing a SIMD (work-groups of 8 waves run their tiles
// in step) the one entering its softmax keeps the VALU and reaches its next
// MFMAs sooner (measured: 5% faster with 8-wave work-groups, slower with two
// 4-wave work-groups per CU).
template <int D, int KT, bool MASK, bool PRIO>
__device__ __forceinline__ void attend_tile2(AttnState<D, 2>& st, KFrag<D>& kf, const bf16* buf,
                                             int k0, int T, int half, int col, bool first) {
  typedef Tile<D, 2, KT> TL;
  constexpr int NKB = TL::NKB;
  const bf16* Vs = buf + TL::KSZ;
  const int nv = MASK ? min(NKB, (T - k0 + 31) / 32) : NKB;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    if (MASK && kb >= nv) break;
    f32x16 s[2];
    qk_mfma<D, 2>(s, st, kf);
    if (PRIO) __builtin_amdgcn_s_setprio(1);
    VFrag<D> vf;
    read_v<D, 2, KT>(vf, Vs, kb, half, col);
    if (kb + 1 < nv) read_k<D, 2, KT>(kf, buf, kb + 1, half, col);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      bf16x8 pb[2];
      softmax_qb<D, 2, MASK>(st, qb, s[qb], pb, k0 + kb * 32, T, half, first && kb == 0);
      pv_qb<D, 2>(st, qb, pb, vf);
      if (PRIO && qb == 0) __builtin_amdgcn_s_setprio(0);
    }
  }
}

// Scores of one query block against one sub-block's keys, relative to the
// block's running max (the C operand nm).
template <int D>
__device__ __forceinline__ void qk_qb(f32x16& s, const AttnState<D, 2>& st, int qb,
                                      const KFrag<D>& f) {
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[ks], st.qf[qb][ks], ks == 0 ? st.nm[qb] : s,
                                                0, 0, 0);
}

// State carried from one sub-block to the next by the pipelined tile walk:
// the first block's scores of the sub-block about to run (issued), its K
// fragments, and the previous sub-block's second-block probabilities and V^T
// fragments, whose P V product is still to be issued.
template <int D>
struct Pipe {
  f32x16 s0;
  KFrag<D> kf;
  bf16x8 pb1[2];
  VFrag<D> vf;
};

// One full key tile, software-pipelined across sub-blocks.  Sub-block kb
// runs as two groups of eight MFMAs, each beside one block's softmax:
//   A: second block's scores, previous sub-block's second-block P V
//      | first block's softmax;
//   B: first block's P V, next sub-block's first-block scores
//      | second block's softmax,
// so no MFMA of a group waits for the softmax beside it.  The previous
// second-block P V is always issued (zero probabilities before the first
// sub-block).  For the tile's last sub-block the next scores need the next
// tile, so the caller issues them after the barrier.
template <int D, int KT>
__device__ __forceinline__ void pipe_tile(AttnState<D, 2>& st, Pipe<D>& pp, const bf16* buf,
                                          int k0, int T, int half, int col, bool first_tile) {
  typedef Tile<D, 2, KT> TL;
  constexpr int NKB = TL::NKB;
  const bf16* Vs = buf + TL::KSZ;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    const bool first = first_tile && kb == 0;
    f32x16 s1;
    qk_qb<D>(s1, st, 1, pp.kf);
    pv_qb<D, 2>(st, 1, pp.pb1, pp.vf);
    read_v<D, 2, KT>(pp.vf, Vs, kb, half, col);
    if (kb + 1 < NKB) read_k<D, 2, KT>(pp.kf, buf, kb + 1, half, col);
    bf16x8 pb0[2];
    softmax_qb<D, 2, false, true>(st, 0, pp.s0, pb0, k0 + kb * 32, T, half, first);
    pv_qb<D, 2>(st, 0, pb0, pp.vf);
    if (kb + 1 < NKB) qk_qb<D>(pp.s0, st, 0, pp.kf);
    softmax_qb<D, 2, false, true>(st, 1, s1, pp.pb1, k0 + kb * 32, T, half, first);
  }
}

// NW waves x 64 queries per work-group.
template <int D, int KT, int NW, int MINB>
__global__ __launch_bounds__(64 * NW, MINB) void attn2_bf16_kernel(AttnParams ap) {
  typedef Tile<D, 2, KT, NW> TL;
  constexpr int kStage = NW * 64 * (D + 8);  // output staging, after the key tiles
  __shared__ __attribute__((aligned(16))) bf16 lds[2 * TL::BUF > kStage ? 2 * TL::BUF : kStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int lid = xcd_remap(int(blockIdx.x), int(gridDim.x));
  const int qtile = lid % ap.qtiles;
  const int bh = lid / ap.qtiles;  // b * n + head
  const int head = bh % ap.n, b = bh / ap.n;
  const int T = ap.T;

  const bf16* Q = static_cast<const bf16*>(ap.q) + int64_t(bh) * T * D;
  const bf16* K = static_cast<const bf16*>(ap.k) + int64_t(bh) * T * D;
  const bf16* Vt = static_cast<const bf16*>(ap.vt) + int64_t(bh) * D * ap.Tp;

  AttnState<D, 2> st;
  init_state<D, 2>(st, Q, qtile * TL::QT + wave * TL::QPW, T, half, col);

  const int ntiles = (T + KT - 1) / KT;
  const int nfull = T / KT;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  // Full tiles go global -> LDS directly (no prefetch registers): tile j+1's
  // loads are issued into the free buffer before tile j is used, and the
  // barrier that ends tile j waits for them.  The partial last tile (keys past
  // T zeroed) goes through registers once, after the full tiles.
  if (nfull > 0) dma_tile<D, 2, KT, NW>(lds, K, Vt, ap.Tp, 0, T, wv, lane);

  Pipe<D> pp;
  {
    const bf16x8 z = {};
    pp.pb1[0] = pp.pb1[1] = z;
#pragma unroll
    for (int gp = 0; gp < 2; ++gp)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) pp.vf.a[gp][db] = z;
  }
  __syncthreads();
  if (nfull > 0) {
    read_k<D, 2, KT>(pp.kf, lds, 0, half, col);
    qk_qb<D>(pp.s0, st, 0, pp.kf);
  }
  for (int j = 0; j < nfull; ++j) {
    bf16* cur = lds + (j & 1) * TL::BUF;
    bf16* nxt = lds + ((j + 1) & 1) * TL::BUF;
    // the other buffer held tile j-1, which every wave finished before the
    // barrier that ended the previous iteration
    if (j + 1 < nfull) dma_tile<D, 2, KT, NW>(nxt, K, Vt, ap.Tp, (j + 1) * KT, T, wv, lane);
    pipe_tile<D, KT>(st, pp, cur, j * KT, T, half, col, j == 0);
    __syncthreads();  // tile j+1 is in place; tile j is free
    if (j + 1 < nfull) {
      read_k<D, 2, KT>(pp.kf, nxt, 0, half, col);
      qk_qb<D>(pp.s0, st, 0, pp.kf);
    }
  }
  pv_qb<D, 2>(st, 1, pp.pb1, pp.vf);
  if (nfull < ntiles) {  // the partial last tile
    bf16* buf = lds + (nfull & 1) * TL::BUF;
    Prefetch<D, 2, KT, NW> pf;
    load_tile<D, 2, KT, NW, true>(pf, K, Vt, ap.Tp, nfull * KT, T, tid);
    store_tile<D, 2, KT, NW>(buf, pf, tid);
    __syncthreads();
    read_k<D, 2, KT>(pp.kf, buf, 0, half, col);
    attend_tile2<D, KT, true, NW == 8>(st, pp.kf, buf, nfull * KT, T, half, col, nfull == 0);
  }

  __syncthreads();  // every wave is done with the key tiles: LDS becomes staging
  write_o<D, 2>(st, ap, b, head, qtile * TL::QT + wave * TL::QPW, half, col, lane,
                lds + wave * 64 * (D + 8));
}

// ---------------------------------------------------------------------------
// bf16 MFMA kernel: two wave groups in alternation (d = 64, long sequences)
// ---------------------------------------------------------------------------
// One 256-query tile per work-group of 8 waves; waves 0-3 (group 0) and 4-7
// (group 1) take the same 256 queries (64 per wave, two 32-query blocks)
// against the two halves of the keys, so a CU finishes one tile at a time and
// a partial last round of tiles is a round of whole CUs.  Group 1 leaves its
// (O, m, l) in LDS at the end and group 0 merges:
//   O = O_0 2^(m_0 - M) + O_1 2^(m_1 - M),  l likewise,  M = max(m_0, m_1).
// A SIMD holds one wave of each group (waves s and s + 4).  Each wave
// alternates two kinds of half step over its 32-key sub-blocks j:
//   M_j  the MFMAs: scores S_j = K_j Q^T - m of both query blocks (8), then
//        O^T += V_{j-1}^T P_{j-1}^T of both (8);
//   V_j  the softmax of S_j on the VALU (bf16 probabilities P_j, row sums,
//        the lazy raise of m; without the bias both query blocks at once, at
//        raised issue priority) and the LDS reads of V_j's fragments (M_{j+1}
//        reads K_{j+1}'s before its P V products).
// The groups run half a step apart and every half step ends at a barrier of
// all 8 waves, so on each SIMD one wave's MFMAs run while the other wave's
// softmax runs: the matrix core and the VALU work side by side instead of
// both waves of a SIMD wanting the same unit at the same time (which is what
// a tile barrier shared by two waves in step produces).  The barriers carry no
// memory fence: each wave waits for its own tile loads explicitly.
// Key tiles (64 keys: two sub-blocks) go from global memory straight into LDS,
// three buffers per group: tile u+2 is requested in M_{2u+1} (its buffer held
// tile u-1, last read in V_{2u-1}) and waited for at the end of V_{2u+2}, the
// half step before its first read (V_{2u+3} reads K_{2u+4}) -- at that point
// no later load of the wave is outstanding, so every wait is vmcnt(0).
// Needs T % 128 == 0 (whole tiles, an even number of them).
// REL = 2: the 2-D relative-position logit bias, with table slices per key
// tile in LDS as in attn_bf16_kernel (the slice a key tile needs for the
// work-group's 256 queries, fp32 times log2(e), and each key's grid term):
// loaded into registers in the half step that requests the tile, stored to
// LDS in the next M half step (three slots per group, like the tiles), and
// added to the scores at the start of each V half step (gathered there: an
// MFMA half step that waits on LDS holds both waves of its SIMD at the next
// barrier).
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

template <int D, int KT, int REL>
__global__ __launch_bounds__(512, 1) void attnpp_bf16_kernel(AttnParams ap) {
  typedef Tile<D, 2, KT, 4> TL;  // one group's geometry
  constexpr int NBUF = 3;
  static_assert(TL::NKB == 2, "the tile loads are scheduled by sub-block parity");
  static_assert(REL == 0 || REL == 2, "table slices in LDS only");
  constexpr int kState = 4 * 64 * (2 * (D / 32) * 16 + 4);  // floats: group 1's O, m, l
  constexpr int kMerge = kState * 2 + 4 * 64 * (D + 8);     // + group 0's output staging (bf16)
  constexpr int kTiles = 2 * NBUF * TL::BUF;
  __shared__ __attribute__((aligned(16))) bf16 lds[kTiles > kMerge ? kTiles : kMerge];
  __shared__ float rel_lds[REL ? 2 * NBUF * kRelSlice : 1];                       // slices
  __shared__ __attribute__((aligned(16))) int kterm_lds[REL ? 2 * NBUF * KT : 1];  // key terms

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, col = lane & 31;
  const int grp = __builtin_amdgcn_readfirstlane(wave >> 2);  // key half
  const int gw = __builtin_amdgcn_readfirstlane(wave & 3);    // wave within the group
  // Work-groups [0, full) take whole tiles and are dispatched first (one
  // round or more of whole CUs); the rest take key ranges of the last tiles.
  // Each part is remapped on its own so that consecutive ids share an XCD.
  const int w = int(blockIdx.x);
  int lid, piece = -1;
  if (w < ap.full) {
    lid = xcd_remap(w, ap.full);
  } else {
    piece = xcd_remap(w - ap.full, int(gridDim.x) - ap.full);
    lid = ap.full + piece / ap.split;
  }
  const int qtile = lid % ap.qtiles;
  const int bh = lid / ap.qtiles;
  const int head = bh % ap.n, b = bh / ap.n;
  const int T = ap.T;
  const bf16* Q = static_cast<const bf16*>(ap.q) + int64_t(bh) * T * D;
  const bf16* K = static_cast<const bf16*>(ap.k) + int64_t(bh) * T * D;
  const bf16* Vt = static_cast<const bf16*>(ap.vt) + int64_t(bh) * D * ap.Tp;
  const int qbase = qtile * TL::QT + gw * TL::QPW;

  AttnState<D, 2> st;
  init_state<D, 2>(st, Q, qbase, T, half, col);
  // The keys come in pairs of tiles, one tile of each pair per group; a key
  // range is a run of pairs (ranges of one tile differ by at most one pair).
  const int pairs = T / KT / 2;
  int p0 = 0, p1 = pairs;
  if (piece >= 0) {
    const int i = piece % ap.split;
    p0 = i * pairs / ap.split;
    p1 = (i + 1) * pairs / ap.split;
  }
  const int nh = p1 - p0;  // key tiles per group (>= 1)
  const int k0 = (2 * p0 + grp * nh) * KT;
  bf16* mine = lds + grp * NBUF * TL::BUF;

  // relative-position bias (REL = 2): the table column of the head, the
  // work-group's query range, this lane's query terms
  f32x16 s[2];  // scores of the current sub-block, both query blocks
  RelPos<2> rp;
  float rel_pf[REL ? kRelSlice / 256 : 1];  // slice entries of one tile (4 per thread)
  int kterm_pf = 0;
  int qrow0[2] = {0, 0};
  const int gtid = gw * 64 + lane;  // thread within the group
  const int rq0 = qtile * TL::QT, rq1 = min(rq0 + TL::QT, T) - 1;
  if constexpr (REL != 0) {
    rp.tab = static_cast<const bf16*>(ap.rel) + head;
    rp.H = ap.H;
    rp.W = ap.W;
    rp.w4 = ap.W % 4 == 0;
    rp.n = ap.n;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {  // rows past T take the last query's place
      const int qi = min(qbase + qb * 32 + col, T - 1);
      const int r = qi / ap.W;
      qrow0[qb] = (r + ap.H - 1) * (2 * ap.W - 1) + (qi - r * ap.W) + ap.W - 1;
    }
  }
  auto rel_load = [&](int u) {  // slice and key terms of tile u into registers
    if constexpr (REL != 0) {
      const int kt = k0 + u * KT;
      int lo, len;
      rel_rows(rq0, rq1, kt, kt + KT - 1, ap.H, ap.W, lo, len);
#pragma unroll
      for (int e = 0; e < kRelSlice / 256; ++e) {
        const int i = gtid + 256 * e;
        rel_pf[e] = i < len ? kLog2e * static_cast<float>(rp.tab[int64_t(lo + i) * ap.n]) : 0.f;
      }
      const int key = kt + (gtid & (KT - 1));
      const int kr = key / ap.W;
      kterm_pf = kr * (2 * ap.W - 1) + (key - kr * ap.W);
    }
  };
  auto rel_store = [&](int u) {  // into slot u % 3 of the group
    if constexpr (REL != 0) {
      const int slot = u % NBUF;
      float* sl = rel_lds + (grp * NBUF + slot) * kRelSlice;
#pragma unroll
      for (int e = 0; e < kRelSlice / 256; ++e) sl[gtid + 256 * e] = rel_pf[e];
      if (gtid < KT) kterm_lds[(grp * NBUF + slot) * KT + gtid] = kterm_pf;
    }
  };
  auto rel_add = [&](int u, int kb) {  // bias of tile u, sub-block kb, onto the scores
    if constexpr (REL != 0) {
      const int kt = k0 + u * KT;
      int len;
      rel_rows(rq0, rq1, kt, kt + KT - 1, ap.H, ap.W, rp.lo, len);
      const int slot = u % NBUF;
      rp.slice = rel_lds + (grp * NBUF + slot) * kRelSlice;
      rp.kterm = kterm_lds + (grp * NBUF + slot) * KT;
      rp.k0 = kt;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) rp.qrow[qb] = qrow0[qb] - rp.lo;
      add_rel<2, 2>(s, rp, kt + kb * 32, T, half);
    }
  };

  dma_tile<D, 2, KT, 4>(mine, K, Vt, ap.Tp, k0, T, gw, lane);
  if (nh > 1) dma_tile<D, 2, KT, 4>(mine + TL::BUF, K, Vt, ap.Tp, k0 + KT, T, gw, lane);
  rel_load(0);
  rel_store(0);
  if (nh > 1) {
    rel_load(1);
    rel_store(1);
  }
  __syncthreads();  // tiles 0 and 1 of both groups (and their slices) are in place

  KFrag<D> kf;
  VFrag<D> vf;
  bf16x8 pb[2][2];
  // M half step on sub-block kb of the tile in `cur`: K_j's fragment reads,
  // O^T += V_{j-1}^T P_{j-1}^T, then S_j = K_j Q^T - m.  (The compiler issues
  // the reads after the P V products, into the registers their V operands
  // free, so the score MFMAs wait on the LDS latency; issuing them first, in
  // registers of their own, measured slower: MFMAs issued earlier take issue
  // slots from the other wave's softmax.)
  auto m_step = [&](const bf16* cur, int kb, bool pv, bool qk) {
    if (qk) read_k<D, 2, KT>(kf, cur, kb, half, col);
    if (pv) {
      pv_qb<D, 2>(st, 0, pb[0], vf);
      pv_qb<D, 2>(st, 1, pb[1], vf);
    }
    if (qk) {
      qk_qb<D>(s[0], st, 0, kf);
      qk_qb<D>(s[1], st, 1, kf);
    }
  };
  // V half step: softmax of S_j; V_j's fragments are needed first by the next
  // M's P V products.  Without the bias: both blocks at once, the fragments
  // requested before it, at raised issue priority (the exponentials bound the
  // step, and the MFMA wave beside it on the SIMD needs few issue slots;
  // measured: 2-3% faster than block by block at the default priority).
  auto v_step = [&](const bf16* cur, int u, int kb, bool first) {
    rel_add(u, kb);
    if constexpr (REL == 0) {
      __builtin_amdgcn_s_setprio(1);
      read_v<D, 2, KT>(vf, cur + TL::KSZ, kb, half, col);
      __builtin_amdgcn_sched_barrier(0);
      softmax_pair<D>(st, s, pb, first);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
    } else {
      // with the bias the step is longer and the V^T reads are better placed
      // between the blocks, block by block at default priority (measured: the
      // paired form 3-4% slower here)
      softmax_qb<D, 2, false>(st, 0, s[0], pb[0], 0, T, half, first);
      __builtin_amdgcn_sched_barrier(0);
      read_v<D, 2, KT>(vf, cur + TL::KSZ, kb, half, col);
      __builtin_amdgcn_sched_barrier(0);
      softmax_qb<D, 2, false>(st, 1, s[1], pb[1], 0, T, half, first);
    }
  };
  auto request = [&](int u) {  // tile u of the group into buffer u % 3 (slice first)
    rel_load(u);
    dma_tile<D, 2, KT, 4>(mine + (u % NBUF) * TL::BUF, K, Vt, ap.Tp, k0 + u * KT, T, gw, lane);
  };

  if (grp == 1) phase_barrier();  // group 1 runs half a step behind
  // tile 0: its first sub-block starts the running max
  m_step(mine, 0, false, true);
  phase_barrier();
  v_step(mine, 0, 0, true);
  phase_barrier();  // (tile 1 arrived before the first barrier)
  m_step(mine, 1, true, true);
  if (2 < nh) request(2);
  phase_barrier();
  v_step(mine, 0, 1, false);
  phase_barrier();
  int bu = 1;  // buffer of tile u
  for (int u = 1; u < nh; ++u) {
    const bf16* cur = mine + bu * TL::BUF;
    m_step(cur, 0, true, true);
    if (u + 1 < nh) rel_store(u + 1);  // requested in the M half step before
    phase_barrier();
    v_step(cur, u, 0, false);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): tile u + 1 is in
    phase_barrier();
    m_step(cur, 1, true, true);
    if (u + 2 < nh) request(u + 2);    // into the buffer of tile u - 1
    phase_barrier();
    v_step(cur, u, 1, false);
    phase_barrier();
    bu = bu + 1 == NBUF ? 0 : bu + 1;
  }
  m_step(mine, 0, true, false);  // the last sub-block's P V
  phase_barrier();
  if (grp == 0) phase_barrier();  // both groups pass the same number of barriers

  // group 1's accumulators, running max and row sums through LDS (register
  // order: every store and load one row of 64 lanes), merged by group 0
  __syncthreads();  // every wave is done with the key tiles
  float* stt = reinterpret_cast<float*>(lds);
  constexpr int kO = 2 * (D / 32) * 16;
  float* my = stt + gw * 64 * (kO + 4);
  if (grp == 1) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) my[((qb * (D / 32) + db) * 16 + r) * 64 + lane] = st.o[qb][db][r];
      my[(kO + qb) * 64 + lane] = st.m[qb];
      my[(kO + 2 + qb) * 64 + lane] = st.l[qb];
    }
  }
  __syncthreads();
  if (grp == 0) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float m1 = my[(kO + qb) * 64 + lane], l1 = my[(kO + 2 + qb) * 64 + lane];
      const float mx = fmaxf(st.m[qb], m1);
      const float w0 = __builtin_amdgcn_exp2f(st.m[qb] - mx), w1 = __builtin_amdgcn_exp2f(m1 - mx);
      st.l[qb] = st.l[qb] * w0 + l1 * w1;
      st.m[qb] = mx;  // O and l are now relative to the common maximum
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          st.o[qb][db][r] =
              st.o[qb][db][r] * w0 + my[((qb * (D / 32) + db) * 16 + r) * 64 + lane] * w1;
    }
    if (piece < 0) {
      write_o<D, 2>(st, ap, b, head, qbase, half, col, lane,
                    reinterpret_cast<bf16*>(stt + kState) + gw * 64 * (D + 8));
    } else {
      // this key range's (O, m, l): per wave, accumulator block c = (qb, db)
      // as 64 lanes x 16 floats, then (m0, m1, l0, l1) per lane; 16-byte
      // stores, cached (the merge kernel reads them next)
      float* pt = ap.part + (int64_t(piece) * 4 + gw) * (kO + 4) * 64;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4 v = {st.o[qb][db][4 * g], st.o[qb][db][4 * g + 1], st.o[qb][db][4 * g + 2],
                             st.o[qb][db][4 * g + 3]};
            *reinterpret_cast<f32x4*>(pt + ((qb * (D / 32) + db) * 64 + lane) * 16 + 4 * g) = v;
          }
      const f32x4 ml = {st.m[0], st.m[1], st.l[0], st.l[1]};
      *reinterpret_cast<f32x4*>(pt + kO * 64 + lane * 4) = ml;
    }
  }
}

// Tiles cut into key ranges: the ranges' partial results are combined
// (rescaled to their common maximum: the exact combination of softmax partial
// sums) and O written.  A work-group per 64 queries of a tile (one wave of
// the ranges' group 0); thread (c, lane) takes that lane's accumulator block
// c = (qb, db), 16 registers stored contiguously: a thread's loads are
// independent 16-byte loads, all in flight at once (S, the number of ranges,
// is a template parameter so that none of them waits behind a branch).  O
// goes out in 8-byte pieces, a row's 128 bytes from two waves and four
// instructions each, through the caches, where L2 joins them (non-temporal
// stores wrote 3.3 times O's bytes to HBM and took 18% longer).
template <int D, int S>
__global__ __launch_bounds__(64 * 2 * (D / 32)) void attn_merge_kernel(AttnParams ap) {
  constexpr int kO = 2 * (D / 32) * 16;
  const int lane = threadIdx.x & 63, c = threadIdx.x >> 6;
  const int qb = c / (D / 32), db = c % (D / 32);
  const int half = lane >> 5, col = lane & 31;
  const int j = int(blockIdx.x) >> 2, gw = int(blockIdx.x) & 3;  // tail tile, wave
  const int lid = ap.full + j;
  const int qtile = lid % ap.qtiles;
  const int bh = lid / ap.qtiles;
  const int head = bh % ap.n, b = bh / ap.n;
  const int64_t stride = int64_t(4) * (kO + 4) * 64;  // floats per key range
  const float* pt = ap.part + (int64_t(j) * S * 4 + gw) * (kO + 4) * 64;
  const float* po = pt + (c * 64 + lane) * 16;  // this thread's 16 accumulators
  const float* pm = pt + kO * 64 + lane * 4;     // (m0, m1, l0, l1)
  f32x4 ml[S], ov[S][4];
#pragma unroll
  for (int i = 0; i < S; ++i) {
    ml[i] = *reinterpret_cast<const f32x4*>(pm + i * stride);
#pragma unroll
    for (int g = 0; g < 4; ++g) ov[i][g] = *reinterpret_cast<const f32x4*>(po + i * stride + 4 * g);
  }
  float mx = ml[0][qb];
#pragma unroll
  for (int i = 1; i < S; ++i) mx = fmaxf(mx, ml[i][qb]);
  float acc[16], l = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
  for (int i = 0; i < S; ++i) {
    const float wgt = __builtin_amdgcn_exp2f(ml[i][qb] - mx);
    l += ml[i][2 + qb] * wgt;
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[4 * g + e] += ov[i][g][e] * wgt;
  }
  const float inv = 1.0f / halves_sum(l);
  // register 4g + e of block (qb, db) is query qb*32 + col, dim db*32 + 8g + 4*half + e
  const int qi = qtile * 256 + gw * 64 + qb * 32 + col;
  if (qi >= ap.T) return;
  const int d = ap.d;
  bf16* O = static_cast<bf16*>(ap.o) + (int64_t(b) * ap.T + qi) * ap.C + head * d;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int d0 = db * 32 + 8 * g + 4 * half;
    if (d == D) {
      bf16x4 pk;
#pragma unroll
      for (int e = 0; e < 4; ++e) pk[e] = static_cast<bf16>(acc[4 * g + e] * inv);
      *reinterpret_cast<bf16x4*>(O + d0) = pk;  // cached: L2 joins the 16-byte pieces of a row
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (d0 + e < d) O[d0 + e] = static_cast<bf16>(acc[4 * g + e] * inv);
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 kernel
// ---------------------------------------------------------------------------
constexpr int FQT = 64, FKT = 32;

template <int DP, bool REL>  // d rounded up to a supported width; each lane owns DP/4 dims
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
  // relative-position bias: this lane's query row / column (rows past T
  // take the last query's place)
  const float* rtab = REL ? static_cast<const float*>(ap.rel) + head : nullptr;
  const int qc_ = min(qi, T - 1);
  const int qrow = REL ? qc_ / ap.W : 0, qcol = REL ? qc_ - qrow * ap.W : 0;

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
      float rel = 0.f;
      if (REL && k0 + j < T) {
        const int kr = (k0 + j) / ap.W, kc = (k0 + j) - kr * ap.W;
        rel = kLog2e * rtab[int64_t((qrow - kr + ap.H - 1) * (2 * ap.W - 1) + (qcol - kc + ap.W - 1)) * ap.n];
      }
      s[j] = (k0 + j < T) ? part * sc + rel : -INFINITY;
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

template <int D, int QB, int KT, int NW, int REL>
void launch_bf16_v(AttnParams ap, int64_t bh, hipStream_t stream) {
  typedef Tile<D, QB, KT, NW> TL;
  ap.qtiles = int((ap.T + TL::QT - 1) / TL::QT);
  attn_bf16_kernel<D, QB, KT, NW, REL><<<dim3(unsigned(bh * ap.qtiles)), TL::NTHR, 0, stream>>>(ap);
}

template <int D, int KT, int NW, int MINB>
void launch_bf16_2(AttnParams ap, int64_t bh, hipStream_t stream) {
  typedef Tile<D, 2, KT, NW> TL;
  ap.qtiles = int((ap.T + TL::QT - 1) / TL::QT);
  attn2_bf16_kernel<D, KT, NW, MINB><<<dim3(unsigned(bh * ap.qtiles)), TL::NTHR, 0, stream>>>(ap);
}


// The relative-position variant of this kernel comes in the 4-wave shape
// only; its table slices go through LDS when they fit (rel_slice_fits), else
// each entry is gathered from the table in global memory.
bool rel_slice_fits(int QT, int KT, int W);

template <int D, int QB, int KT, int NW>
void launch_bf16(AttnParams ap, int64_t bh, hipStream_t stream) {
  if (ap.rel != nullptr) {
    typedef Tile<D, QB, KT, 4> TL;
    if (rel_slice_fits(TL::QT, KT, ap.W))
      launch_bf16_v<D, QB, KT, 4, 2>(ap, bh, stream);
    else
      launch_bf16_v<D, QB, KT, 4, 1>(ap, bh, stream);
  } else {
    launch_bf16_v<D, QB, KT, NW, 0>(ap, bh, stream);
  }
}

// d = 64 without the relative-position bias, long sequences: the two-block
// kernel reads half the LDS operand bytes per MFMA but holds twice the
// queries per wave, so it needs whole rounds of work-groups to pay.  512-query
// work-groups (8 waves, key tiles of 128, one per CU) when the query tiles
// fill whole rounds of the CUs or many of them; 256-query tiles (key tiles of
// 64: one 8-wave key-splitting work-group or two 4-wave work-groups per CU)
// when they fill at least one round of two per CU;
// otherwise (shorter or fewer sequences) the one-block kernel, whose
// 128-query work-groups spread the work more evenly.
// True when every (query tile, key tile) pair's slice of the relative-position
// table fits kRelSlice entries: a query tile of QT spans at most
// ceil((QT-1)/W) + 1 grid rows and a key tile ceil((KT-1)/W) + 1, and a slice
// covers (the two spans - 1) blocks of 2W - 1 rows.
bool rel_slice_fits(int QT, int KT, int W) {
  const int64_t spans = (QT - 1 + W - 1) / W + (KT - 1 + W - 1) / W + 1;
  return spans * (2 * int64_t(W) - 1) <= kRelSlice;
}

// The key-splitting kernel over 256-query tiles, with the tiles of a partial
// last round cut into key ranges when the plan says so (then the merge
// kernel follows on the same stream).
void launch_pp(const Plan& p, AttnParams ap, int64_t t256, hipStream_t stream) {
  typedef Tile<64, 2, 64, 4> TL;
  ap.qtiles = int((ap.T + TL::QT - 1) / TL::QT);
  const int split = p.attn_split;
  const int64_t full = split > 1 ? p.attn_full : t256;
  const int64_t grid = full + (t256 - full) * split;
  ap.full = int(full);
  ap.split = split;
  if (ap.rel != nullptr)
    attnpp_bf16_kernel<64, 64, 2><<<dim3(unsigned(grid)), 512, 0, stream>>>(ap);
  else
    attnpp_bf16_kernel<64, 64, 0><<<dim3(unsigned(grid)), 512, 0, stream>>>(ap);
  if (split > 1) {
    const dim3 mg(unsigned((t256 - full) * 4));
    switch (split) {  // 2 .. 8
      case 2: attn_merge_kernel<64, 2><<<mg, 256, 0, stream>>>(ap); break;
      case 3: attn_merge_kernel<64, 3><<<mg, 256, 0, stream>>>(ap); break;
      case 4: attn_merge_kernel<64, 4><<<mg, 256, 0, stream>>>(ap); break;
      case 5: attn_merge_kernel<64, 5><<<mg, 256, 0, stream>>>(ap); break;
      case 6: attn_merge_kernel<64, 6><<<mg, 256, 0, stream>>>(ap); break;
      case 7: attn_merge_kernel<64, 7><<<mg, 256, 0, stream>>>(ap); break;
      default: attn_merge_kernel<64, 8><<<mg, 256, 0, stream>>>(ap); break;
    }
  }
}

void launch_bf16_64(const Plan& p, AttnParams ap, int64_t bh, hipStream_t stream) {
  if (p.T >= 1024) {
    const int64_t t512 = bh * ((p.T + 511) / 512), t256 = bh * ((p.T + 255) / 256);
    if (ap.rel == nullptr && (t512 % p.cus == 0 || t512 >= 4 * int64_t(p.cus))) {
      launch_bf16_2<64, 128, 8, 1>(ap, bh, stream);
      return;
    }
    // (the one-block kernel's relative-position variant runs two work-groups
    // per CU, so a single round of 256-query tiles already pays for it; with
    // the last round's tiles cut into key ranges, so does the plain kernel)
    if (t256 >= (ap.rel != nullptr || p.attn_split > 1 ? 1 : 2) * int64_t(p.cus)) {
      // 256-query tiles.  With an even number of full key tiles each tile runs
      // as one 8-wave work-group whose halves split the keys (attnpp): faster
      // per tile than two 4-wave work-groups sharing a CU, and a partial last
      // round is then a round of whole CUs; otherwise two 4-wave work-groups
      // per CU.  The relative-position bias takes the same kernel where its
      // table slices fit.
      if (p.T % 128 == 0 && (ap.rel == nullptr || rel_slice_fits(256, 64, ap.W))) {
        launch_pp(p, ap, t256, stream);
        return;
      }
      if (ap.rel == nullptr) {
        launch_bf16_2<64, 64, 4, 2>(ap, bh, stream);
        return;
      }
    }
  }
  launch_bf16<64, 1, 64, 4>(ap, bh, stream);
}

}  // namespace

// The key-splitting kernel's partial last round (bf16, dp = 64, T >= 1024,
// T % 128 == 0, at least one round of 256-query tiles): when its r tiles
// fill at most half the CUs, each is cut into S = min(cus / r, 8, T / 128)
// key ranges, so that the last round takes about 1/S of a tile's time.
void plan_attention_tail(Plan& p) {
  p.attn_split = 1;
  p.attn_full = 0;
  if (p.dtype != SSA_BF16 || p.dp != 64 || p.T < 1024 || p.T % 128 != 0) return;
  const int64_t cus = p.cus;
  const int64_t t256 = p.B * p.n * ((p.T + 255) / 256);
  const int64_t r = t256 % cus;
  if (t256 < cus || r == 0 || 2 * r > cus) return;
  int64_t s = cus / r;
  if (s > 8) s = 8;
  if (s > p.T / 128) s = p.T / 128;
  p.attn_split = int(s);
  p.attn_full = t256 - r;
}

size_t attn_part_bytes() { return size_t(4) * 64 * (2 * (64 / 32) * 16 + 4) * sizeof(float); }

hipError_t launch_attention(const Plan& p, const Args& a) {
  AttnParams ap{};
  ap.q = a.ws + p.ws.q;
  ap.k = a.ws + p.ws.k;
  ap.vt = a.ws + p.ws.vt;
  ap.o = a.ws + p.ws.o;
  ap.T = int(p.T);
  // bf16 kernels run at the padded width dp (q, k zero past d); d is the
  // head's own width (score scale, output columns)
  ap.Tp = int(p.Tp);
  ap.n = int(p.n);
  ap.d = int(p.d);
  ap.C = int(p.C);
  // normalised queries and keys are not divided by sqrt(d) (bf16 folds the
  // scale into the stored queries instead)
  ap.scale = a.q_norm_gamma != nullptr ? kLog2e : kLog2e / sqrtf(float(p.d));
  ap.rel = a.rel_pos_table;
  ap.H = int(p.H);
  ap.W = int(p.W);
  ap.full = 0;
  ap.split = 1;
  ap.part = reinterpret_cast<float*>(a.ws + p.ws.attn_part);
  const int64_t bh = p.B * p.n;
  if (p.dtype == SSA_BF16) {
    // one 256-query work-group per head when the heads alone fill the chip
    const bool wide = p.T <= 256 && bh >= p.cus;
    switch (p.dp) {
      case 32: launch_bf16<32, 1, 64, 4>(ap, bh, a.stream); break;
      case 64:
        if (wide) launch_bf16<64, 1, 64, 8>(ap, bh, a.stream);
        else launch_bf16_64(p, ap, bh, a.stream);
        break;
      case 96: launch_bf16<96, 1, 64, 4>(ap, bh, a.stream); break;
      default:
        if (wide) launch_bf16<128, 1, 64, 8>(ap, bh, a.stream);
        else launch_bf16<128, 1, 64, 4>(ap, bh, a.stream);
        break;
    }
  } else {
    ap.qtiles = int((p.T + FQT - 1) / FQT);
    dim3 grid(unsigned(bh * ap.qtiles));
    const bool rel = ap.rel != nullptr;
    if (p.d <= 32)
      rel ? attn_f32_kernel<32, true><<<grid, 256, 0, a.stream>>>(ap)
          : attn_f32_kernel<32, false><<<grid, 256, 0, a.stream>>>(ap);
    else if (p.d <= 64)
      rel ? attn_f32_kernel<64, true><<<grid, 256, 0, a.stream>>>(ap)
          : attn_f32_kernel<64, false><<<grid, 256, 0, a.stream>>>(ap);
    else
      rel ? attn_f32_kernel<128, true><<<grid, 256, 0, a.stream>>>(ap)
          : attn_f32_kernel<128, false><<<grid, 256, 0, a.stream>>>(ap);
  }
  return hipGetLastError();
}

}  // namespace ssa
