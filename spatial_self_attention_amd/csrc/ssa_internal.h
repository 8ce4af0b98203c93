// Internal declarations shared by the HIP sources of libssa (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "ssa.h"

namespace ssa {

typedef __bf16 bf16;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kGnEps = 1e-5f;
constexpr int kTokPad = 64;  // vt row pitch is T rounded up to this

// Slot of token t in a bf16 V^T row: bits 2 and 3 of t are swapped, so in
// every run of 16 tokens the groups 4..7 and 8..11 trade places.  That puts
// the 8 keys one lane of v_mfma_f32_32x32x16_bf16 multiplies in one B-operand
// step (4*half + {0..3} and 8 + 4*half + {0..3}) next to each other, so the
// attention kernel reads its V^T operand with one 16-byte LDS load.  The map
// is its own inverse and stays inside each run of 16 (and inside Tp).
__host__ __device__ __forceinline__ int vt_slot(int t) {
  return (t & ~12) | ((t & 4) << 1) | ((t & 8) >> 1);
}

// Everything a launch needs, derived once from the sizes by make_plan().
struct Plan {
  int64_t B, C, H, W, G, n;
  int64_t T, d, Tp;
  int64_t dp;      // head width of the q, k, vt layouts: d, or for bf16 d rounded up
                   // to a multiple of 32 (the attention kernels' operand width)
  int dtype;       // ssa_dtype
  int esize;       // bytes per element of x / params / q,k,vt,o
  // GroupNorm statistics split: each (b, g) segment of Cg*T contiguous
  // elements is cut into `splits` chunks of `chunk` elements.
  int64_t seg_len, chunk, splits;
  int gn_vec;      // elements per vector load in the stats pass (1 = scalar)
  bool gn_seg;     // one 512-thread work-group per segment (splits == 1)
  int cus;         // compute units of the current device (launch shaping)
  // bf16 Q/K/V projection on the 128 x 128 MFMA kernel (C % 64 == 0,
  // T % 4 == 0, d % 8 == 0); otherwise the general tile kernel
  bool qkv_main;
  // query/key normalisation and rotary embedding inside that kernel's
  // epilogue (qkv_main and d in {16, 32, 64, 128}); otherwise the projection
  // writes fp32 Q and K to the qk32 region and one pass applies them
  bool qk_fuse;
  // attention on 256-query tiles that split their keys between the two
  // halves of a work-group: the first attn_full tiles run whole; each of the
  // rest (a partial last round of at most half the compute units) is cut into
  // attn_split key ranges whose partial results are merged afterwards
  // (attn_split == 1: every tile whole)
  int attn_split;
  int64_t attn_full;
  ssa_workspace_layout ws;
};

// Pointers of one call, already validated.
struct Args {
  const void* x;
  void* out;
  const void* norm_weight;
  const void* norm_bias;
  const void* w[4];  // q, k, v, out weights
  const void* b[4];  // q, k, v, out biases (NULL: no bias)
  char* ws;
  hipStream_t stream;
  // optional steps (ssa_options); NULL / false when off
  const void* rel_pos_table;
  const void* q_norm_gamma;
  const void* k_norm_gamma;
  bool rope;
};

// Query/key normalisation and rotary embedding from the fp32 Q and K that
// the projection left in the qk32 region, into the bf16 / fp32 q and k
// layouts (the QKV stage when an option is on and qk_fuse is false).
hipError_t launch_qk_post(const Plan& p, const Args& a);
// (cos, sin) of the rotary angles of every (token, pair) into the rope region
// (the QKV stage when rotary embeddings are on and qk_fuse is true).
hipError_t launch_rope_table(const Plan& p, const Args& a);
// Zeros in the padding columns d .. dp-1 of the q and k layouts (bf16, dp > d).
hipError_t launch_zero_pad(const Plan& p, const Args& a);

// Fills p.attn_split and p.attn_full from the sizes and p.cus.
void plan_attention_tail(Plan& p);
// Bytes of the attn_part region per split key range.
size_t attn_part_bytes();

// Launchers (one per stage); each returns hipSuccess or the launch error.
hipError_t launch_gn_stats(const Plan& p, const Args& a);
hipError_t launch_qkv_proj(const Plan& p, const Args& a);
hipError_t launch_attention(const Plan& p, const Args& a);
hipError_t launch_out_proj(const Plan& p, const Args& a);

// Q/K/V projections and attention in one kernel (SSA_STAGE_QKV_ATTENTION),
// for the sizes fused_available() accepts: its O equals that of the QKV and
// attention stages bit for bit.
bool fused_available(const Plan& p);
hipError_t launch_fused(const Plan& p, const Args& a);

// Stores of write-once streams (Q, K, V^T, O, the block's output):
// non-temporal, so that they do not evict from L2 the operands that other
// work-groups of the same launch still re-read (weight panels, key tiles, x).
// Not for data the next kernel reads at once (the attention partials): those
// are read back faster when written through the caches.  8- or 16-byte values.
typedef unsigned nt_u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned nt_u32x4 __attribute__((ext_vector_type(4)));
template <typename V>
__device__ __forceinline__ void store_nt(void* p, const V& v) {
  static_assert(sizeof(V) == 8 || sizeof(V) == 16, "8- or 16-byte stores");
  if constexpr (sizeof(V) == 16)
    __builtin_nontemporal_store(__builtin_bit_cast(nt_u32x4, v), static_cast<nt_u32x4*>(p));
  else
    __builtin_nontemporal_store(__builtin_bit_cast(nt_u32x2, v), static_cast<nt_u32x2*>(p));
}

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return static_cast<float>(v); }

template <typename T>
__device__ __forceinline__ T from_f32(float v);
template <>
__device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float v) { return static_cast<bf16>(v); }

}  // namespace ssa
