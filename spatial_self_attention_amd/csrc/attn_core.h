// Pieces of the bf16 attention shared by the attention kernel and the fused
// projection + attention kernel: the per-wave online-softmax state, the
// score and P V MFMA steps, the softmax of one 32-key sub-block and the
// relative-position bias terms.  The scores are in the log2 domain
// (s = q.k * log2(e) / sqrt(d)); see attention.hip for the algorithm.
#pragma once

#include "ssa_internal.h"

namespace ssa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// A sub-block's probabilities 2^(s - m) are accepted against the running max
// m while this lane's 16 of them sum to at most 2^8 (so none exceeds 2^8 and
// the fp32 accumulators stay far from overflow); otherwise m is raised first.
constexpr float kLazySum = 256.f;

// Word 3 of a raw buffer resource on the gfx9 family: 32-bit data format, no
// swizzle.  Loads at or past num_records bytes return zero.
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), kRsrcWord3);
}

// Work-group id -> logical id so that consecutive logical ids (query tiles of
// one head, which share K and V) run on the same XCD: work-groups are handed
// to the 8 XCDs round-robin, so XCD x receives ids x, x+8, x+16, ...
__device__ __forceinline__ int xcd_remap(int w, int nwg) {
  const int q = nwg >> 3, r = nwg & 7, x = w & 7;
  return x * q + min(x, r) + (w >> 3);
}

// max / sum of v over lanes l and l^32 (one v_permlane32_swap, no LDS)
__device__ __forceinline__ float halves_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D, int QB>
struct AttnState {
  bf16x8 qf[QB][D / 16];   // B operand of S^T = K Q^T, one query per lane column
  f32x16 nm[QB];           // -m in every entry: the C operand the score MFMAs start from
  f32x16 o[QB][D / 32];    // O^T accumulators (d x 32 queries per block)
  float m[QB];             // running max, log2 units
  float l[QB];             // running row sum (this lane's half of the keys)
};

// Operand fragments of one 32-key sub-block, read from LDS one pipeline
// step before the MFMAs that use them (the LDS latency is then hidden behind
// a step of MFMA and softmax work instead of stalling each MFMA).
template <int D>
struct KFrag {  // A operand of S^T = K Q^T: keys kb*32 + col, dims ks*16 + half*8 ..
  bf16x8 a[D / 16];
};
template <int D>
struct VFrag {  // A operand of O^T += V^T P^T: dims db*32 + col, keys per step gp
  bf16x8 a[2][D / 32];
};

// S^T - m for one 32-key sub-block: lane (half, col) gets, for each 32-query
// block, query col against keys kb*32 + 8*(r/4) + 4*half + r%4, r = 0..15.
// All 16 entries of a lane belong to one query, so the accumulation starts
// from the C operand nm = (-m, .., -m) and the matrix core subtracts the max.
template <int D, int QB>
__device__ __forceinline__ void qk_mfma(f32x16 (&s)[QB], const AttnState<D, QB>& st,
                                        const KFrag<D>& f) {
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
      s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[ks], st.qf[qb][ks],
                                                      ks == 0 ? st.nm[qb] : s[qb], 0, 0, 0);
}

// O^T += V^T P^T for one sub-block.
template <int D, int QB>
__device__ __forceinline__ void pv_mfma(AttnState<D, QB>& st, const bf16x8 (&pb)[QB][2],
                                        const VFrag<D>& f) {
#pragma unroll
  for (int gp = 0; gp < 2; ++gp)
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        st.o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[gp][db], pb[qb][gp], st.o[qb][db], 0, 0, 0);
}

// 2^(s - delta) of one lane's 16 scores, rounded to bf16 in MFMA B-operand
// order, and their fp32 sum.  The sum uses plain adds (two chains): v_add
// issues in the shadow of the matrix core, while v_dot2 stalls it.
__device__ __forceinline__ float probs(bf16x8 (&pb)[2], const f32x16& s, float delta) {
  float p[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(s[r] - delta);
  float part[2] = {p[0], p[1]};
#pragma unroll
  for (int r = 2; r < 16; ++r) part[r & 1] += p[r];
#pragma unroll
  for (int gp = 0; gp < 2; ++gp)
#pragma unroll
    for (int e = 0; e < 8; ++e) pb[gp][e] = static_cast<bf16>(p[8 * gp + e]);
  return part[0] + part[1];
}

// Online softmax of one 32-key sub-block (scores already relative to m):
// the bf16 probabilities in MFMA B-operand order and the row-sum update.
// FIRST: the first sub-block, which sets m.  Returns whether m was raised
// (wave-uniform), with the raise per query block in delta; O is rescaled
// after the P V products already issued for earlier sub-blocks.
// Relative-position bias of one wave's queries (HNDL attention operator,
// "Relative position bias"): column `head` of the table (stride n), and the
// grid row / column of each of the wave's query blocks' lane query.  REL = 1
// gathers every entry from the table in global memory; REL = 2 reads it from
// `slice`, the part of the head's column the current key tile needs (table
// rows lo .., staged in LDS with the tile).
template <int QB>
struct RelPos {
  const bf16* tab;   // table + head
  int H, W, n;
  int qr[QB], qc[QB];
  const float* slice;  // REL = 2: table rows lo .. of this head times log2(e), fp32 (LDS)
  int lo;
  int qrow[QB];        // REL = 2: (row(q) + H - 1)(2W - 1) + col(q) + W - 1 - lo
  const int* kterm;    // REL = 2: row(k)(2W - 1) + col(k) of the tile's keys (LDS)
  int k0;              // REL = 2: the tile's first key
  bool w4;             // REL = 2: W % 4 == 0 (4-aligned runs of keys stay in one grid row)
};

// Entries of the table slice one work-group stages per key tile (REL = 2),
// kept in LDS as fp32 already multiplied by log2(e): a score then takes one
// LDS read and one add.
constexpr int kRelSlice = 1024;

// Table rows (first, count) that queries q0..q1 meet against keys k0..k1.
// A row is (dr + H - 1)(2W - 1) + (dc + W - 1) with dr = row(q) - row(k) and
// dc = col(q) - col(k), 0 <= dc + W - 1 < 2W - 1: the rows are ordered by
// (dr, dc), so the extreme (dr, dc) pairs bound them.
__device__ __forceinline__ void rel_rows(int q0, int q1, int k0, int k1, int H, int W, int& lo,
                                         int& len) {
  const int qr0 = q0 / W, qr1 = q1 / W, kr0 = k0 / W, kr1 = k1 / W;
  const int qc0 = qr0 == qr1 ? q0 - qr0 * W : 0, qc1 = qr0 == qr1 ? q1 - qr0 * W : W - 1;
  const int kc0 = kr0 == kr1 ? k0 - kr0 * W : 0, kc1 = kr0 == kr1 ? k1 - kr0 * W : W - 1;
  lo = (qr0 - kr1 + H - 1) * (2 * W - 1) + (qc0 - kc1 + W - 1);
  len = (qr1 - kr0 + H - 1) * (2 * W - 1) + (qc1 - kc0 + W - 1) - lo + 1;
}

// Adds log2(e) * table[(row(q)-row(k)+H-1)(2W-1) + col(q)-col(k)+W-1, head]
// to the scores of one 32-key sub-block (keys >= T are left alone: masked).
template <int QB, int REL>
__device__ __forceinline__ void add_rel(f32x16 (&s)[QB], const RelPos<QB>& rp, int kfirst, int T,
                                        int half) {
  if constexpr (REL == 2) {
    // table row of (q, k) = qrow(q) + lo - kterm(k).  With W % 4 == 0 a run
    // of four keys (4-aligned) lies in one grid row, so their terms are
    // kterm(k0) + 0..3 and the entries are four consecutive slice entries
    // below one base: one address and two paired LDS reads per run and query
    // block.  Otherwise a run's four key terms come in one 16-byte LDS read,
    // each score's entry in one more.
    if (rp.w4) {
#pragma unroll
      for (int run = 0; run < 4; ++run) {
        const int kk = kfirst - rp.k0 + 8 * run + 4 * half;
        const int kt0 = rp.kterm[kk];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const float* b = rp.slice + (rp.qrow[qb] - kt0 - 3);  // entries of keys 3, 2, 1, 0
#pragma unroll
          for (int e = 0; e < 4; ++e) s[qb][4 * run + e] += b[3 - e];
        }
      }
    } else {
#pragma unroll
      for (int run = 0; run < 4; ++run) {  // keys kfirst + 8 run + 4 half + e, e = 0..3
        const int kk = kfirst - rp.k0 + 8 * run + 4 * half;
        const int4 kt = *reinterpret_cast<const int4*>(rp.kterm + kk);
        const int kte[4] = {kt.x, kt.y, kt.z, kt.w};
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int e = 0; e < 4; ++e) s[qb][4 * run + e] += rp.slice[rp.qrow[qb] - kte[e]];
      }
    }
  } else {
#pragma unroll
    for (int run = 0; run < 4; ++run) {  // keys kfirst + 8 run + 4 half + e, e = 0..3
      const int k0 = kfirst + 8 * run + 4 * half;
      int kr = k0 / rp.W, kc = k0 - kr * rp.W;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (k0 + e < T) {
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            const int idx = (rp.qr[qb] - kr + rp.H - 1) * (2 * rp.W - 1) + (rp.qc[qb] - kc + rp.W - 1);
            s[qb][4 * run + e] += kLog2e * static_cast<float>(rp.tab[int64_t(idx) * rp.n]);
          }
        }
        if (++kc == rp.W) {
          kc = 0;
          ++kr;
        }
      }
    }
  }
}

template <int D, int QB, int KT, bool MASK, int REL>
__device__ __forceinline__ bool softmax_block(AttnState<D, QB>& st, f32x16 (&s)[QB],
                                              bf16x8 (&pb)[QB][2], float (&delta)[QB], int kb,
                                              int kbase, int T, int half, bool first,
                                              const RelPos<QB>& rp) {
  if constexpr (REL != 0) add_rel<QB, REL>(s, rp, kbase + kb * 32, T, half);
  if constexpr (MASK) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kbase + kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
      if (key >= T)
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[qb][r] = -INFINITY;
    }
  }
  float part[QB];
  bool big = false;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    part[qb] = probs(pb[qb], s[qb], 0.f);
    big = big || !(part[qb] <= kLazySum);
  }
  const bool raise = first || __builtin_amdgcn_ballot_w64(big);
  if (raise) {
    // Raise m to this sub-block's row max, rescale O and l, and redo the
    // probabilities.
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = s[qb][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[qb][r]);
      mx = halves_max(mx);
      const float m_new = first ? mx : fmaxf(st.m[qb], st.m[qb] + mx);
      delta[qb] = m_new - st.m[qb];
      if (!first) {
        const float alpha = __builtin_amdgcn_exp2f(-delta[qb]);
        st.l[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) st.o[qb][db][r] *= alpha;
      }
      st.m[qb] = m_new;
#pragma unroll
      for (int r = 0; r < 16; ++r) st.nm[qb][r] = -m_new;
      part[qb] = probs(pb[qb], s[qb], delta[qb]);
    }
  }
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) st.l[qb] += part[qb];
  return raise;
}

}  // namespace
}  // namespace ssa
