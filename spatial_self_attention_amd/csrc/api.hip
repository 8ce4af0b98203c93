// Host side of the C ABI declared in include/ssa.h: argument validation,
// launch planning, workspace layout and stage dispatch.  Nothing here touches
// device memory; every check runs before the first launch.
#include <string.h>

#include <atomic>

#include "ssa_internal.h"

namespace ssa {
namespace {

// The workspace of ssa_forward_noalloc: a static device array, one per GPU the
// library runs on, held until the process ends.  128 MiB covers every
// workload measured here (the high-resolution one needs 97 MB).  In host code
// `scratch` is only a stand-in symbol: its device address (per device) comes
// from hipGetSymbolAddress, in scratch_base().
constexpr size_t kScratchBytes = size_t(128) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr size_t kAlign = 256;
constexpr int64_t kMaxElems = (int64_t(1) << 31) - 1;  // per tensor, for 32-bit row math

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Compute units of the current device, cached per device (256 when no device
// can be queried, e.g. for workspace sizing on a host without a GPU).
int device_cus() {
  static int cache[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      cus = 256;
    cache[dev] = cus;
  }
  return cache[dev];
}

// Every head size up to 128, in both dtypes (bf16 heads are zero-padded to a
// multiple of 32, the widths of the attention kernels' MFMA operands).
bool supported_head(int64_t d) { return d >= 1 && d <= 128; }

// Size checks shared by every entry point.  On success fills *p (when the
// input is non-empty) and sets *empty.
ssa_status make_plan(int64_t B, int64_t C, int64_t H, int64_t W, int64_t G,
                     int64_t n, int dtype, Plan* p, bool* empty) {
  if (dtype != SSA_F32 && dtype != SSA_BF16) return SSA_E_DTYPE;
  if (B < 0 || H < 0 || W < 0 || C < 1) return SSA_E_SHAPE;
  if (G < 1 || n < 1 || C % G != 0 || C % n != 0) return SSA_E_CONSTRAINT;
  const int64_t d = C / n;
  if (!supported_head(d)) return SSA_E_UNSUPPORTED;
  *empty = (B == 0 || H == 0 || W == 0);
  if (*empty) return SSA_OK;
  const int64_t T = H * W;
  if (T > kMaxElems || B > kMaxElems / T || B * T > kMaxElems / (3 * C))
    return SSA_E_UNSUPPORTED;
  memset(p, 0, sizeof(*p));
  p->B = B; p->C = C; p->H = H; p->W = W; p->G = G; p->n = n;
  p->T = T; p->d = d;
  p->Tp = (T + kTokPad - 1) / kTokPad * kTokPad;
  p->dtype = dtype;
  p->esize = dtype == SSA_F32 ? 4 : 2;
  p->dp = dtype == SSA_F32 ? d : (d + 31) / 32 * 32;
  p->cus = device_cus();
  p->qkv_main = dtype == SSA_BF16 && C % 64 == 0 && T % 4 == 0 && d % 8 == 0;
  p->qk_fuse = p->qkv_main && (d == 16 || d == 32 || d == 64 || d == 128);

  // Statistics split.  With enough (b, g) segments to fill the chip and
  // segments a work-group streams quickly, one work-group per segment also
  // finalises the statistics (one kernel); likewise, with a wider work-group,
  // for longer or fewer segments down to a quarter as many as CUs (vector
  // loads only).  Otherwise each segment is cut into chunks of at least 8192
  // elements, about 2048 work-groups in all, and a second kernel merges them.
  const int64_t L = (C / G) * T;
  const int vec = 16 / p->esize;
  p->gn_vec = (L % vec == 0) ? vec : 1;
  p->seg_len = L;
  int64_t segs = B * G;
  int64_t splits = 1;
  p->gn_seg = (segs < 256 || L > 65536) && p->gn_vec == vec && 4 * segs >= p->cus &&
              L <= (int64_t(1) << 20);
  if ((segs < 256 || L > 65536) && !p->gn_seg) {
    const int64_t want = (2048 + segs - 1) / segs;
    const int64_t cap = (L + 8191) / 8192;
    splits = want < cap ? want : cap;
    if (splits < 1) splits = 1;
  }
  int64_t chunk = (L + splits - 1) / splits;
  chunk = (chunk + p->gn_vec - 1) / p->gn_vec * p->gn_vec;
  p->chunk = chunk;
  p->splits = (L + chunk - 1) / chunk;

  ssa_workspace_layout& ws = p->ws;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = round_up(off + bytes, kAlign); return o; };
  ws.gn_partial = take(size_t(segs * p->splits) * 16);
  ws.gn_stats = take(size_t(segs) * 8);
  ws.gn_coef = take(size_t(B * C) * 8);
  const size_t e = p->esize;
  const int64_t dp = p->dp;
  ws.q = take(size_t(B * n * T * dp) * e);
  ws.k = take(size_t(B * n * T * dp) * e);
  ws.vt = take(size_t(B * n * dp * p->Tp) * e);
  ws.o = take(size_t(B * T * C) * e);
  // The optional query/key steps' buffers are sized from the problem alone
  // (ssa_workspace_size does not see the options): the rotary table where the
  // projection epilogue applies the steps, else fp32 Q and K for the pass
  // that does (bf16 only: fp32 Q and K are written unrounded anyway).
  ws.rope = take(p->qk_fuse ? size_t(T * (d / 2)) * 8 : 0);
  ws.qk32 = take(dtype == SSA_BF16 && !p->qk_fuse ? size_t(2 * B * T * C) * 4 : 0);
  plan_attention_tail(*p);
  const int64_t tail = p->attn_split > 1 ? B * n * ((T + 255) / 256) - p->attn_full : 0;
  ws.attn_part = take(size_t(tail * p->attn_split) * attn_part_bytes());
  ws.total = off;
  ws.gn_splits = p->splits;
  ws.t_pad = p->Tp;
  ws.d_pad = dp;
  return SSA_OK;
}

struct Range {
  uintptr_t lo, hi;
};

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

// NULL and alignment checks of the caller's tensors (not the workspace).
ssa_status check_tensor_pointers(const Args& a) {
  const void* required[] = {a.x, a.out, a.norm_weight, a.norm_bias, a.w[0], a.w[1], a.w[2],
                            a.w[3]};
  for (const void* q : required)
    if (q == nullptr) return SSA_E_NULL;
  const void* all[] = {a.x, a.out, a.norm_weight, a.norm_bias, a.w[0], a.w[1], a.w[2], a.w[3],
                       a.b[0], a.b[1], a.b[2], a.b[3],
                       a.rel_pos_table, a.q_norm_gamma, a.k_norm_gamma};
  for (const void* q : all)  // NULL (an absent optional tensor) is aligned
    if (reinterpret_cast<uintptr_t>(q) % 16 != 0) return SSA_E_ALIGN;
  return SSA_OK;
}

ssa_status check_pointers(const Plan& p, const Args& a, size_t ws_bytes) {
  ssa_status st = check_tensor_pointers(a);
  if (st != SSA_OK) return st;
  if (a.ws == nullptr) return SSA_E_NULL;
  if (reinterpret_cast<uintptr_t>(a.ws) % 16 != 0) return SSA_E_ALIGN;
  if (ws_bytes < p.ws.total) return SSA_E_WORKSPACE;
  const size_t e = p.esize;
  const size_t img = size_t(p.B * p.C * p.T) * e;
  auto rng = [](const void* q, size_t bytes) {
    uintptr_t lo = reinterpret_cast<uintptr_t>(q);
    return Range{lo, q == nullptr ? lo : lo + bytes};  // absent: empty range
  };
  Range out = rng(a.out, img);
  Range ws = rng(a.ws, p.ws.total);
  const size_t table = size_t((2 * p.H - 1) * (2 * p.W - 1) * p.n) * e;
  Range inputs[] = {rng(a.x, img),
                    rng(a.norm_weight, p.C * e), rng(a.norm_bias, p.C * e),
                    rng(a.w[0], p.C * p.C * e), rng(a.w[1], p.C * p.C * e),
                    rng(a.w[2], p.C * p.C * e), rng(a.w[3], p.C * p.C * e),
                    rng(a.b[0], p.C * e), rng(a.b[1], p.C * e),
                    rng(a.b[2], p.C * e), rng(a.b[3], p.C * e),
                    rng(a.rel_pos_table, table),
                    rng(a.q_norm_gamma, p.C * e), rng(a.k_norm_gamma, p.C * e)};
  if (overlap(out, ws)) return SSA_E_ALIAS;
  for (const Range& r : inputs)
    if (overlap(out, r) || overlap(ws, r)) return SSA_E_ALIAS;
  return SSA_OK;
}

// Rules of the optional steps that depend on the sizes.
ssa_status check_options(const Plan& p, const Args& a) {
  if ((a.q_norm_gamma == nullptr) != (a.k_norm_gamma == nullptr)) return SSA_E_CONSTRAINT;
  if (a.rope && p.d % 2 != 0) return SSA_E_UNSUPPORTED;
  return SSA_OK;
}

void* scratch_base();

// stages: the stage codes to enqueue, in order; stage < 0: the whole block
// (stages 0, 1, 2, 3, or 0, 4, 3 where the fused kernel is available and no
// optional step is on).  workspace NULL with noalloc: the static scratch, once
// every other argument has been checked.
ssa_status run(int stage, const void* x, void* out, const void* nw, const void* nb,
               const void* qw, const void* kw, const void* vw, const void* ow,
               const void* qb, const void* kb, const void* vb, const void* ob,
               int64_t B, int64_t C, int64_t H, int64_t W, int64_t G, int64_t n, int dtype,
               const ssa_options* opt, void* workspace, size_t workspace_bytes, void* stream,
               bool noalloc = false) {
  Plan p;
  bool empty = false;
  ssa_status st = make_plan(B, C, H, W, G, n, dtype, &p, &empty);
  if (st != SSA_OK || empty) return st;
  if (noalloc && p.ws.total > kScratchBytes) return SSA_E_SCRATCH;
  Args a;
  a.x = x; a.out = out; a.norm_weight = nw; a.norm_bias = nb;
  a.w[0] = qw; a.w[1] = kw; a.w[2] = vw; a.w[3] = ow;
  a.b[0] = qb; a.b[1] = kb; a.b[2] = vb; a.b[3] = ob;
  a.ws = static_cast<char*>(workspace);
  a.stream = static_cast<hipStream_t>(stream);
  a.rel_pos_table = opt ? opt->rel_pos_table : nullptr;
  a.q_norm_gamma = opt ? opt->q_norm_gamma : nullptr;
  a.k_norm_gamma = opt ? opt->k_norm_gamma : nullptr;
  a.rope = opt != nullptr && opt->rope != 0;
  st = check_options(p, a);
  if (st != SSA_OK) return st;
  if (noalloc) {
    st = check_tensor_pointers(a);
    if (st != SSA_OK) return st;
    a.ws = static_cast<char*>(scratch_base());
    if (a.ws == nullptr) return SSA_E_HIP;
    workspace_bytes = kScratchBytes;
  }
  st = check_pointers(p, a, workspace_bytes);
  if (st != SSA_OK) return st;
  const bool plain = a.rel_pos_table == nullptr && a.q_norm_gamma == nullptr && !a.rope;
  int stages[4] = {SSA_STAGE_GN_STATS, SSA_STAGE_QKV, SSA_STAGE_ATTENTION, SSA_STAGE_OUT_PROJ};
  int count = 4;
  if (stage >= 0) {
    if (stage == SSA_STAGE_QKV_ATTENTION && (!fused_available(p) || !plain))
      return SSA_E_UNSUPPORTED;
    stages[0] = stage;
    count = 1;
  } else if (plain && fused_available(p)) {
    stages[1] = SSA_STAGE_QKV_ATTENTION;
    stages[2] = SSA_STAGE_OUT_PROJ;
    count = 3;
  }
  for (int i = 0; i < count; ++i) {
    hipError_t e = hipSuccess;
    switch (stages[i]) {
      case SSA_STAGE_GN_STATS: e = launch_gn_stats(p, a); break;
      case SSA_STAGE_QKV: {
        const bool qk_opt = a.rope || a.q_norm_gamma != nullptr;
        if (p.dp > p.d) e = launch_zero_pad(p, a);
        if (e == hipSuccess && qk_opt && a.rope && p.qk_fuse) e = launch_rope_table(p, a);
        if (e == hipSuccess) e = launch_qkv_proj(p, a);
        if (e == hipSuccess && qk_opt && !p.qk_fuse) e = launch_qk_post(p, a);
        break;
      }
      case SSA_STAGE_ATTENTION: e = launch_attention(p, a); break;
      case SSA_STAGE_OUT_PROJ: e = launch_out_proj(p, a); break;
      case SSA_STAGE_QKV_ATTENTION: e = launch_fused(p, a); break;
    }
    if (e != hipSuccess) return SSA_E_HIP;
  }
  return SSA_OK;
}

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept; NULL on a HIP error.
void* scratch_base() {
  static std::atomic<void*> base[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  void* p = base[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    base[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace
}  // namespace ssa

extern "C" {

size_t ssa_workspace_size(int64_t B, int64_t C, int64_t H, int64_t W, int64_t num_groups,
                          int64_t num_heads, int dtype) {
  ssa::Plan p;
  bool empty = false;
  if (ssa::make_plan(B, C, H, W, num_groups, num_heads, dtype, &p, &empty) != SSA_OK || empty)
    return 0;
  return p.ws.total;
}

ssa_status ssa_get_workspace_layout(int64_t B, int64_t C, int64_t H, int64_t W,
                                    int64_t num_groups, int64_t num_heads, int dtype,
                                    ssa_workspace_layout* layout) {
  if (layout == nullptr) return SSA_E_NULL;
  ssa::Plan p;
  bool empty = false;
  ssa_status st = ssa::make_plan(B, C, H, W, num_groups, num_heads, dtype, &p, &empty);
  memset(layout, 0, sizeof(*layout));
  if (st == SSA_OK && !empty) *layout = p.ws;
  return st;
}

ssa_status ssa_forward(const void* x, void* out, const void* norm_weight, const void* norm_bias,
                       const void* q_weight, const void* k_weight, const void* v_weight,
                       const void* out_weight, const void* q_bias, const void* k_bias,
                       const void* v_bias, const void* out_bias, int64_t B, int64_t C, int64_t H,
                       int64_t W, int64_t num_groups, int64_t num_heads, int dtype,
                       void* workspace, size_t workspace_bytes, void* stream) {
  return ssa::run(-1, x, out, norm_weight, norm_bias, q_weight, k_weight, v_weight, out_weight,
                  q_bias, k_bias, v_bias, out_bias, B, C, H, W, num_groups, num_heads, dtype,
                  nullptr, workspace, workspace_bytes, stream);
}

ssa_status ssa_forward_ex(const void* x, void* out, const void* norm_weight,
                          const void* norm_bias, const void* q_weight, const void* k_weight,
                          const void* v_weight, const void* out_weight, const void* q_bias,
                          const void* k_bias, const void* v_bias, const void* out_bias,
                          int64_t B, int64_t C, int64_t H, int64_t W, int64_t num_groups,
                          int64_t num_heads, int dtype, const ssa_options* options,
                          void* workspace, size_t workspace_bytes, void* stream) {
  return ssa::run(-1, x, out, norm_weight, norm_bias, q_weight, k_weight, v_weight, out_weight,
                  q_bias, k_bias, v_bias, out_bias, B, C, H, W, num_groups, num_heads, dtype,
                  options, workspace, workspace_bytes, stream);
}

ssa_status ssa_forward_stage(int stage, const void* x, void* out, const void* norm_weight,
                             const void* norm_bias, const void* q_weight, const void* k_weight,
                             const void* v_weight, const void* out_weight, const void* q_bias,
                             const void* k_bias, const void* v_bias, const void* out_bias,
                             int64_t B, int64_t C, int64_t H, int64_t W, int64_t num_groups,
                             int64_t num_heads, int dtype, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (stage < SSA_STAGE_GN_STATS || stage > SSA_STAGE_QKV_ATTENTION) return SSA_E_STAGE;
  return ssa::run(stage, x, out, norm_weight, norm_bias, q_weight, k_weight, v_weight,
                  out_weight, q_bias, k_bias, v_bias, out_bias, B, C, H, W, num_groups,
                  num_heads, dtype, nullptr, workspace, workspace_bytes, stream);
}

ssa_status ssa_forward_stage_ex(int stage, const void* x, void* out, const void* norm_weight,
                                const void* norm_bias, const void* q_weight, const void* k_weight,
                                const void* v_weight, const void* out_weight, const void* q_bias,
                                const void* k_bias, const void* v_bias, const void* out_bias,
                                int64_t B, int64_t C, int64_t H, int64_t W, int64_t num_groups,
                                int64_t num_heads, int dtype, const ssa_options* options,
                                void* workspace, size_t workspace_bytes, void* stream) {
  if (stage < SSA_STAGE_GN_STATS || stage > SSA_STAGE_QKV_ATTENTION) return SSA_E_STAGE;
  return ssa::run(stage, x, out, norm_weight, norm_bias, q_weight, k_weight, v_weight,
                  out_weight, q_bias, k_bias, v_bias, out_bias, B, C, H, W, num_groups,
                  num_heads, dtype, options, workspace, workspace_bytes, stream);
}

ssa_status ssa_forward_noalloc(const void* x, void* out, const void* norm_weight,
                               const void* norm_bias, const void* q_weight, const void* k_weight,
                               const void* v_weight, const void* out_weight, const void* q_bias,
                               const void* k_bias, const void* v_bias, const void* out_bias,
                               int64_t B, int64_t C, int64_t H, int64_t W, int64_t num_groups,
                               int64_t num_heads, int dtype, void* stream) {
  return ssa::run(-1, x, out, norm_weight, norm_bias, q_weight, k_weight, v_weight, out_weight,
                  q_bias, k_bias, v_bias, out_bias, B, C, H, W, num_groups, num_heads, dtype,
                  nullptr, nullptr, 0, stream, /*noalloc=*/true);
}

size_t ssa_noalloc_max_workspace(void) { return ssa::kScratchBytes; }

int ssa_uses_fused_stage(int64_t B, int64_t C, int64_t H, int64_t W, int64_t num_groups,
                         int64_t num_heads, int dtype) {
  ssa::Plan p;
  bool empty = false;
  if (ssa::make_plan(B, C, H, W, num_groups, num_heads, dtype, &p, &empty) != SSA_OK || empty)
    return 0;
  return ssa::fused_available(p) ? 1 : 0;
}

const char* ssa_status_string(int status) {
  switch (status) {
    case SSA_OK: return "ok";
    case SSA_E_NULL: return "a required pointer is NULL (only the biases may be NULL)";
    case SSA_E_SHAPE: return "invalid shape: sizes must be >= 0 and C >= 1";
    case SSA_E_CONSTRAINT:
      return "num_groups and num_heads must be >= 1 and divide C; query and key norm gammas "
             "come together";
    case SSA_E_DTYPE: return "unknown dtype";
    case SSA_E_UNSUPPORTED:
      return "unsupported size: head size must be 1..128, even with rotary embeddings, and "
             "3*B*H*W*C below 2^31; the fused stage only where ssa_uses_fused_stage() is 1";
    case SSA_E_WORKSPACE: return "workspace smaller than ssa_workspace_size()";
    case SSA_E_ALIAS: return "out or workspace overlaps another buffer";
    case SSA_E_ALIGN: return "a pointer is not 16-byte aligned";
    case SSA_E_HIP: return "a HIP kernel launch failed";
    case SSA_E_STAGE: return "unknown stage";
    case SSA_E_SCRATCH:
      return "ssa_forward_noalloc: the problem's workspace exceeds the library's static scratch "
             "(ssa_noalloc_max_workspace() bytes); use ssa_forward with a caller workspace";
    default: return "unknown status";
  }
}

}  // extern "C"
