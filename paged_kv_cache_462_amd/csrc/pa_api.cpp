// C-ABI entry points: host-side validation, planning and dispatch.
//
// Every check below runs before any HIP call, so an invalid request returns
// an error code without touching the device (and can be tested on a machine
// without a GPU).
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <string>

#include "../../include/pa.h"
#include "pa_internal.h"
#include "pa_prefill.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int elem_size(int dt) {
  switch (dt) {
    case PA_F32: return 4;
    case PA_F16: return 2;
    case PA_BF16: return 2;
    case PA_FP8_E4M3: return 1;
    case PA_I32: return 4;
    case PA_I64: return 8;
    default: return 0;
  }
}

int kind_of(int dt) {
  switch (dt) {
    case PA_F32: return pa::K_F32;
    case PA_F16: return pa::K_F16;
    case PA_BF16: return pa::K_BF16;
    case PA_FP8_E4M3: return pa::K_FP8;
    default: return -1;
  }
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_tensor(const pa_tensor* t, const char* name, int ndim) {
  if (!t) return fail(PA_ERR_INVALID_ARG, "%s: null descriptor", name);
  if (t->ndim != ndim) return fail(PA_ERR_INVALID_ARG, "%s: expected %d dims, got %d", name, ndim, t->ndim);
  if (elem_size(t->dtype) == 0) return fail(PA_ERR_INVALID_ARG, "%s: unknown dtype %d", name, t->dtype);
  int64_t numel = 1;
  for (int i = 0; i < ndim; ++i) {
    if (t->shape[i] < 0) return fail(PA_ERR_INVALID_ARG, "%s: negative extent", name);
    numel *= t->shape[i];
  }
  if (numel > 0 && !t->data) return fail(PA_ERR_INVALID_ARG, "%s: null data", name);
  return PA_OK;
}

bool contiguous(const pa_tensor* t) {
  int64_t s = 1;
  for (int i = t->ndim - 1; i >= 0; --i) {
    if (t->shape[i] != 1 && t->stride[i] != s) return false;
    s *= t->shape[i];
  }
  return true;
}

int check_cache_pair(const pa_tensor* k, const pa_tensor* v) {
  int rc;
  if ((rc = check_tensor(k, "key_cache", 4)) || (rc = check_tensor(v, "value_cache", 4))) return rc;
  for (int i = 0; i < 4; ++i)
    if (k->shape[i] != v->shape[i]) return fail(PA_ERR_INVALID_ARG, "key_cache and value_cache shapes differ");
  if (k->dtype != v->dtype) return fail(PA_ERR_INVALID_ARG, "key_cache and value_cache dtypes differ");
  if (!contiguous(k) || !contiguous(v))
    return fail(PA_ERR_INVALID_ARG, "caches must be contiguous [num_blocks, block_size, num_kv_heads, head_dim]");
  if (kind_of(k->dtype) < 0) return fail(PA_ERR_INVALID_ARG, "cache dtype must be f32, f16, bf16 or fp8");
  if (!aligned16(k->data) || !aligned16(v->data)) return fail(PA_ERR_INVALID_ARG, "caches must be 16-byte aligned");
  if (k->dtype == PA_FP8_E4M3) {
    if (!(k->scale > 0.f) || !isfinite(k->scale) || !(v->scale > 0.f) || !isfinite(v->scale))
      return fail(PA_ERR_INVALID_ARG, "fp8 caches need a positive finite scale");
  }
  return PA_OK;
}

struct Plan {
  int sched = pa::kSchedFixed;
  int split = 0;
  int part_tokens = 0;
  int num_parts = 1;
  int64_t slots = 0;     // triple slots in the workspace
  int64_t ws_bytes = 0;
};

// Shared by pa_decode and the plan / workspace queries.  The host never
// reads seq_lens (they live on the device): the balanced schedule finds the
// lengths on the device, and a fixed split covers the table width (its
// partitions past a sequence's end exit at once).
// Query-tile ranks of the prefill grid (Hq * ranks * B workgroups; past
// 2^24 workgroups the kernel loops over the remaining ranks instead).
int64_t prefill_ranks(int64_t B, int64_t Hq, int64_t T, int64_t max_query_len) {
  const int64_t bm = pa::prefill_rows_per_workgroup();
  const int64_t mq = max_query_len > 0 && max_query_len < T ? max_query_len : T;
  int64_t ranks = (mq + bm - 1) / bm;
  const int64_t per_rank = Hq * B;
  if (per_rank > 0 && ranks * per_rank > (1LL << 24))
    ranks = (1LL << 24) / per_rank > 0 ? (1LL << 24) / per_rank : 1;
  return ranks;
}

// The caller's error flags (launch->error_flags): null, or 4-byte aligned.
int flags_of(const pa_launch* launch, int32_t** out) {
  *out = launch ? launch->error_flags : nullptr;
  if (*out && reinterpret_cast<uintptr_t>(*out) % 4)
    return fail(PA_ERR_INVALID_ARG, "error_flags must be 4-byte aligned");
  return PA_OK;
}

// Contexts this short (every sequence within 256 tokens, 16 tiles) run in
// one pass under the automatic plan: a workgroup per (sequence, unit
// chunk) walks them in about the time a second (merge) launch would take.
constexpr int kSinglePassMaxTokens = 256;

// Tiles' worth of time charged for each sequence a balanced share starts,
// in the decode of the rest after a shared prefix.  A piece's start costs a
// wave about three tiles' time (3 to 4 us against 0.8 to 1.2 us a tile,
// measured on the shared-prompt batches), and the rest of each sequence is
// short, so shares hold several pieces; the charge gives the shares that
// start more sequences fewer tiles.  Plain decode deals equal shares of
// tiles: with equal lengths they fall on sequence boundaries, which the
// charge would shift (the 70B-shaped batch measured 0.6 % slower with it).
constexpr int kPieceCost = 3;

// balanced_only: the automatic plan is always the balanced schedule (the
// shared-prefix decode needs it), whatever the context length.
int make_plan(int B, int Hq, int Hkv, int D, int bs, int max_blocks, int req, Plan* out,
              bool balanced_only = false) {
  if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || bs <= 0 || max_blocks < 0)
    return fail(PA_ERR_INVALID_ARG, "sizes must be positive");
  if (Hq % Hkv) return fail(PA_ERR_INVALID_ARG, "num_q_heads (%d) is not a multiple of num_kv_heads (%d)", Hq, Hkv);
  if (bs % 16) return fail(PA_ERR_UNSUPPORTED, "block_size must be a multiple of 16 (got %d)", bs);
  if (D != 64 && D != 128) return fail(PA_ERR_UNSUPPORTED, "head_dim must be 64 or 128 (got %d)", D);
  const int64_t max_ctx64 = (int64_t)max_blocks * bs;
  if (max_ctx64 > (1 << 30)) return fail(PA_ERR_INVALID_ARG, "block table addresses too many tokens");
  const int max_ctx = (int)max_ctx64;
  if (req > 0 && req % 16) return fail(PA_ERR_INVALID_ARG, "partition_tokens must be a multiple of 16");
  if (req < -1) return fail(PA_ERR_INVALID_ARG, "partition_tokens must be -1, 0 or positive");
  Plan p;
  const int64_t max_tiles = (int64_t)B * ((max_ctx + 15) / 16);
  if (req == 0 && !balanced_only && max_ctx <= kSinglePassMaxTokens) {
    p.part_tokens = max_ctx > 0 ? ((max_ctx + 15) / 16) * 16 : 16;
  } else if (req == 0 && B <= pa::kBalancedMaxBatch && max_tiles < (int64_t)1 << 30) {
    // automatic: equal shares of the batch's tiles per workgroup
    p.sched = pa::kSchedBalanced;
    p.split = 1;
    p.slots = (int64_t)pa::kBalancedSlots + B;
  } else {
    const int pt = req == 0 ? 512 : req;  // automatic fallback: 512-token partitions
    if (pt == -1 || pt >= max_ctx) {
      p.part_tokens = max_ctx > 0 ? ((max_ctx + 15) / 16) * 16 : 16;
    } else {
      p.split = 1;
      p.part_tokens = pt;
      p.num_parts = (max_ctx + pt - 1) / pt;
      if (p.num_parts > 65535) return fail(PA_ERR_UNSUPPORTED, "too many partitions (%d)", p.num_parts);
      p.slots = (int64_t)B * p.num_parts;
    }
  }
  // workspace: acc [slots, Hq, D] f32, then (max, sum) [slots, Hq, 2] f32,
  // then per-sequence (first slot, pieces) [B, 2] i32 (balanced only)
  p.ws_bytes = p.slots * Hq * (D + 2) * (int64_t)sizeof(float) +
               (p.sched == pa::kSchedBalanced ? (int64_t)B * 2 * (int64_t)sizeof(int32_t) : 0);
  *out = p;
  return PA_OK;
}

// Validation, plan and kernel parameters of a decode call (everything but
// the launch); *empty is set when there is nothing to launch.
int decode_setup(pa_tensor* out, const pa_tensor* query, const pa_tensor* key_cache,
                 const pa_tensor* value_cache, const pa_tensor* block_tables,
                 const pa_tensor* seq_lens, float scale, int32_t block_size,
                 int32_t num_kv_heads, const pa_launch* launch, int64_t extra_ws_bytes,
                 pa::DecodeParams* out_p, pa::DecodeVariant* out_v, Plan* out_plan, bool* empty,
                 bool balanced_only = false, int64_t scratch_cap = -1,
                 int64_t* out_slots = nullptr) {
  // scratch_cap >= 0: the triples go to the library's own scratch of that
  // many bytes instead of the caller's workspace (the launch must carry
  // none); the layout is the one below with slots = the shares the launch
  // deals plus B, and the pointers are left for the caller to set
  *empty = false;
  int rc;
  if ((rc = check_tensor(query, "query", 3)) || (rc = check_tensor(out, "out", 3)) ||
      (rc = check_cache_pair(key_cache, value_cache)) ||
      (rc = check_tensor(block_tables, "block_tables", 2)) ||
      (rc = check_tensor(seq_lens, "seq_lens", 1)))
    return rc;
  const int qdt = query->dtype;
  if (qdt != PA_F32 && qdt != PA_F16 && qdt != PA_BF16)
    return fail(PA_ERR_INVALID_ARG, "query dtype must be f32, f16 or bf16");
  if (out->dtype != qdt) return fail(PA_ERR_INVALID_ARG, "out dtype must equal the query dtype");
  const int64_t B = query->shape[0], Hq = query->shape[1], D = query->shape[2];
  for (int i = 0; i < 3; ++i)
    if (out->shape[i] != query->shape[i]) return fail(PA_ERR_INVALID_ARG, "out shape must equal the query shape");
  if (query->stride[2] != 1 || out->stride[2] != 1)
    return fail(PA_ERR_INVALID_ARG, "query/out head_dim stride must be 1");
  const int64_t N = key_cache->shape[0], bs = key_cache->shape[1], Hkv = key_cache->shape[2];
  if (key_cache->shape[3] != D) return fail(PA_ERR_INVALID_ARG, "cache head_dim %lld != query head_dim %lld",
                                            (long long)key_cache->shape[3], (long long)D);
  if (bs != block_size) return fail(PA_ERR_INVALID_ARG, "block_size %d != cache block dimension %lld",
                                    block_size, (long long)bs);
  if (Hkv != num_kv_heads) return fail(PA_ERR_INVALID_ARG, "num_kv_heads %d != cache head dimension %lld",
                                       num_kv_heads, (long long)Hkv);
  const int kvdt = key_cache->dtype;
  if (!(kvdt == qdt || (kvdt == PA_FP8_E4M3 && (qdt == PA_F16 || qdt == PA_BF16))))
    return fail(PA_ERR_INVALID_ARG, "cache dtype must equal the query dtype, or be fp8 with an f16/bf16 query");
  if (block_tables->dtype != PA_I32 || seq_lens->dtype != PA_I32)
    return fail(PA_ERR_INVALID_ARG, "block_tables and seq_lens must be int32");
  if (block_tables->shape[0] != B || seq_lens->shape[0] != B)
    return fail(PA_ERR_INVALID_ARG, "block_tables / seq_lens batch must equal the query batch");
  if (block_tables->stride[1] != 1 || (seq_lens->stride[0] != 1 && B > 1))
    return fail(PA_ERR_INVALID_ARG, "block_tables column stride and seq_lens stride must be 1");
  const int64_t max_blocks = block_tables->shape[1];
  if (B > 65535) return fail(PA_ERR_UNSUPPORTED, "batch above 65535");
  if (N > 0x7FFFFFFFLL || max_blocks > 0x7FFFFFFFLL) return fail(PA_ERR_UNSUPPORTED, "pool or table too large");
  if (!isfinite(scale)) return fail(PA_ERR_INVALID_ARG, "scale must be finite");
  const int qes = elem_size(qdt);
  const int64_t vec = 16 / qes;
  if (!aligned16(query->data) || query->stride[0] % vec || query->stride[1] % vec)
    return fail(PA_ERR_INVALID_ARG, "query rows must be 16-byte aligned");
  if (!aligned16(out->data) || out->stride[0] % vec || out->stride[1] % vec)
    return fail(PA_ERR_INVALID_ARG, "out rows must be 16-byte aligned");
  Plan plan;
  if ((rc = make_plan((int)B, (int)Hq, (int)Hkv, (int)D, (int)bs, (int)max_blocks,
                      launch ? launch->partition_tokens : 0, &plan, balanced_only)))
    return rc;
  const int G = (int)(Hq / Hkv);
  const int req_path = launch ? launch->path : PA_PATH_AUTO;
  pa::DecodeVariant v;
  v.qkind = kind_of(qdt);
  v.kvkind = kind_of(kvdt);
  v.D = (int)D;
  if (req_path == PA_PATH_MFMA) {
    if (qdt == PA_F32) return fail(PA_ERR_UNSUPPORTED, "the MFMA path needs an f16/bf16 query");
    v.path = 2;
  } else if (req_path == PA_PATH_VALU) {
    v.path = 1;
  } else if (req_path == PA_PATH_AUTO) {
    v.path = (qdt != PA_F32 && G >= 4) ? 2 : 1;
  } else {
    return fail(PA_ERR_INVALID_ARG, "unknown path %d", req_path);
  }
  v.gt = v.path == 2 ? 16 : (G == 1 ? 1 : (G == 2 ? 2 : 4));
  if (!pa::decode_variant_built(v)) return fail(PA_ERR_UNSUPPORTED, "no decode variant for this dtype / head_dim");
  if (plan.split && scratch_cap < 0) {
    const int64_t need = plan.ws_bytes + extra_ws_bytes;
    if (!launch || !launch->workspace || launch->workspace_bytes < (size_t)need)
      return fail(PA_ERR_WORKSPACE, "split decode needs %lld workspace bytes", (long long)need);
    if (!aligned16(launch->workspace)) return fail(PA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  }
  if (B == 0 || Hq == 0) {
    *empty = true;
    return PA_OK;
  }

  pa::DecodeParams p;
  memset(&p, 0, sizeof p);
  if ((rc = flags_of(launch, &p.flags))) return rc;
  p.out = out->data;
  p.q = query->data;
  p.kc = key_cache->data;
  p.vc = value_cache->data;
  p.tables = static_cast<const int32_t*>(block_tables->data);
  p.lens = static_cast<const int32_t*>(seq_lens->data);
  p.q_sb = query->stride[0];
  p.q_sh = query->stride[1];
  p.o_sb = out->stride[0];
  p.o_sh = out->stride[1];
  p.tab_stride = block_tables->stride[0];
  p.B = (int)B;
  p.Hq = (int)Hq;
  p.Hkv = (int)Hkv;
  p.G = G;
  p.D = (int)D;
  p.bs = (int)bs;
  p.max_blocks = (int)max_blocks;
  p.num_blocks = (int)N;
  p.head_tiles = (G + v.gt - 1) / v.gt;
  const int64_t units = Hkv * (int64_t)p.head_tiles;
  if (units > 0x7FFFFFFFLL) return fail(PA_ERR_UNSUPPORTED, "grid too large");
  p.units = (int)units;
  {
    int max_waves, workgroups;
    pa::decode_launch_shape(v, &max_waves, &workgroups);
    p.waves = (int)(units < max_waves ? units : max_waves);
    const int chunks = (p.units + p.waves - 1) / p.waves;
    const int nwc = workgroups / chunks;
    p.nwc = nwc < 1 ? 1 : nwc;
  }
  p.sched = plan.sched;
  p.part_tokens = plan.part_tokens;
  p.num_parts = plan.num_parts;
  p.split = plan.split;
  const double ks = kvdt == PA_FP8_E4M3 ? (double)key_cache->scale : 1.0;
  p.qk_scale_log2 = (float)((double)scale * ks * 1.4426950408889634);
  p.v_scale = kvdt == PA_FP8_E4M3 ? value_cache->scale : 1.0f;
  // a balanced piece of sequence b sits at slot (its share) + b
  const int64_t slots = scratch_cap >= 0 && plan.sched == pa::kSchedBalanced
                            ? (int64_t)p.nwc + B : plan.slots;
  if (plan.split && scratch_cap >= 0) {
    const int64_t need = slots * Hq * (D + 2) * (int64_t)sizeof(float) +
                         (plan.sched == pa::kSchedBalanced ? B * 2 * (int64_t)sizeof(int32_t) : 0);
    if (need > scratch_cap)
      return fail(PA_ERR_WORKSPACE,
                  "this plan needs %lld bytes of scratch; the library holds %lld (use pa_decode "
                  "with a workspace)", (long long)need, (long long)scratch_cap);
  }
  if (out_slots) *out_slots = slots;
  if (plan.split && scratch_cap < 0) {
    p.ws_acc = static_cast<float*>(launch->workspace);
    p.ws_ml = p.ws_acc + plan.slots * Hq * D;
    p.ws_meta = reinterpret_cast<int32_t*>(p.ws_ml + plan.slots * Hq * 2);
  }
  *out_p = p;
  *out_v = v;
  *out_plan = plan;
  return PA_OK;
}

// How the shared-prefix decode takes its prefix part.  Each kv head's
// prefix keys serve rows = B * G (sequence, query head) rows.
// - Grouped (rows < kPassRows): inside the matrix-core decode launch, the
//   rows in groups of 16 (one wave each, the kernel's query columns) over
//   pieces of about kGroupTokens keys (24 tiles), about what a decode
//   share holds, so that neither kind of wave is left to finish alone;
//   every group reads the prefix tiles it needs again (from the caches).
// - Pass (rows >= kPassRows): a launch of the prefill kernel before the
//   decode, 256-row tiles of the rows against pieces of a multiple of 64
//   keys, enough pieces for about 256 workgroups; each tile of the prefix
//   is read once per 256 rows, which pays for the extra launch when the
//   rows are many.
constexpr int kGroupTokens = 384;
constexpr int64_t kPassRows = 1024;
struct PrefixPlan {
  bool pass = false;
  int pieces = 0;
  int tokens = 0;              // keys per piece
  int64_t row_groups = 0;      // grouped: groups of 16 rows per kv head
  int row_tiles = 0;           // pass: 256-row tiles per kv head
  int64_t extra_ws_bytes = 0;  // triples of the prefix pieces
};

PrefixPlan prefix_plan(int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int prefix_tokens) {
  PrefixPlan pp;
  const int64_t rows = B * (Hq / Hkv);
  pp.pass = rows >= kPassRows;
  if (pp.pass) {
    const int64_t bm = pa::prefill_rows_per_workgroup();
    pp.row_tiles = (int)((rows + bm - 1) / bm);
    const int64_t target = std::max<int64_t>(1, 256 / std::max<int64_t>(1, Hkv * pp.row_tiles));
    const int64_t most = std::max<int64_t>(1, (prefix_tokens + 63) / 64);
    const int64_t want = std::min(target, most);
    pp.tokens = (int)(((prefix_tokens + want - 1) / want + 63) / 64 * 64);
  } else {
    pp.row_groups = (rows + 15) / 16;
    const int want = std::max(1, (prefix_tokens + kGroupTokens - 1) / kGroupTokens);
    pp.tokens = ((prefix_tokens + want - 1) / want + 15) / 16 * 16;
  }
  pp.pieces = (prefix_tokens + pp.tokens - 1) / pp.tokens;
  pp.extra_ws_bytes = B * pp.pieces * Hq * (D + 2) * (int64_t)sizeof(float);
  return pp;
}

}  // namespace

extern "C" {

const char* pa_last_error(void) { return g_err.c_str(); }

const char* pa_build_info(void) {
  return "target gfx950 (CDNA4); decode VALU {f32,f16,bf16,fp8-kv} x head_dim {64,128} x "
         "heads/tile {1,2,4}; decode MFMA {f16,bf16,fp8-kv} x head_dim {64,128} x 16 heads/tile; "
         "split-partition merge; prefill MFMA {f16,bf16} x {same,fp8} kv x head_dim {64,128}; "
         "cache write {copy, fp8 e4m3 quantise}; block copy";
}

int64_t pa_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t block_size, int32_t max_blocks,
                                  int32_t partition_tokens) {
  Plan p;
  int rc = make_plan(batch, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks,
                     partition_tokens, &p);
  return rc ? rc : p.ws_bytes;
}

int pa_decode_plan(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                   int32_t block_size, int32_t max_blocks, int32_t partition_tokens,
                   pa_decode_plan_info* info) {
  if (!info) return fail(PA_ERR_INVALID_ARG, "null plan descriptor");
  Plan p;
  int rc = make_plan(batch, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks,
                     partition_tokens, &p);
  if (rc) return rc;
  info->schedule = p.sched == pa::kSchedBalanced ? PA_SCHEDULE_BALANCED
                   : p.split                     ? PA_SCHEDULE_PARTITIONS
                                                 : PA_SCHEDULE_SINGLE;
  info->partition_tokens = p.sched == pa::kSchedBalanced || !p.split ? 0 : p.part_tokens;
  info->workspace_bytes = p.ws_bytes;
  return PA_OK;
}

int pa_decode(pa_tensor* out, const pa_tensor* query, const pa_tensor* key_cache,
              const pa_tensor* value_cache, const pa_tensor* block_tables,
              const pa_tensor* seq_lens, float scale, int32_t block_size,
              int32_t num_kv_heads, const pa_launch* launch) {
  pa::DecodeParams p;
  pa::DecodeVariant v;
  Plan plan;
  bool empty;
  int rc = decode_setup(out, query, key_cache, value_cache, block_tables, seq_lens, scale,
                        block_size, num_kv_heads, launch, 0, &p, &v, &plan, &empty);
  if (rc || empty) return rc;
  hipStream_t stream = launch ? static_cast<hipStream_t>(launch->stream) : nullptr;
  hipError_t e = pa::launch_decode(p, v, stream);
  if (e != hipSuccess) return fail(PA_ERR_HIP, "decode launch failed: %s", hipGetErrorString(e));
  return PA_OK;
}

int pa_decode_noalloc(pa_tensor* out, const pa_tensor* query, const pa_tensor* key_cache,
                      const pa_tensor* value_cache, const pa_tensor* block_tables,
                      const pa_tensor* seq_lens, float scale, int32_t block_size,
                      int32_t num_kv_heads, const pa_launch* launch) {
  if (launch && (launch->workspace || launch->workspace_bytes))
    return fail(PA_ERR_INVALID_ARG, "pa_decode_noalloc takes no workspace (it uses the library's own)");
  pa::DecodeParams p;
  pa::DecodeVariant v;
  Plan plan;
  bool empty;
  int64_t slots = 0;
  int rc = decode_setup(out, query, key_cache, value_cache, block_tables, seq_lens, scale,
                        block_size, num_kv_heads, launch, 0, &p, &v, &plan, &empty, false,
                        pa::kDecodeScratchBytes, &slots);
  if (rc || empty) return rc;
  hipStream_t stream = launch ? static_cast<hipStream_t>(launch->stream) : nullptr;
  if (plan.split) {
    void* base = nullptr;
    hipError_t e = pa::decode_scratch(stream, &base);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "scratch lookup failed: %s", hipGetErrorString(e));
    const int64_t Hq = p.Hq, D = p.D;
    p.ws_acc = static_cast<float*>(base);
    p.ws_ml = p.ws_acc + slots * Hq * D;
    p.ws_meta = reinterpret_cast<int32_t*>(p.ws_ml + slots * Hq * 2);
  }
  hipError_t e = pa::launch_decode(p, v, stream);
  if (e != hipSuccess) return fail(PA_ERR_HIP, "decode launch failed: %s", hipGetErrorString(e));
  return PA_OK;
}

int64_t pa_decode_shared_prefix_workspace_bytes(int32_t batch, int32_t num_q_heads,
                                                int32_t num_kv_heads, int32_t head_dim,
                                                int32_t block_size, int32_t max_blocks,
                                                int32_t prefix_tokens) {
  Plan p;
  int rc = make_plan(batch, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks, 0, &p,
                     true);
  if (rc) return rc;
  if (p.sched != pa::kSchedBalanced)
    return fail(PA_ERR_UNSUPPORTED, "the shared-prefix decode takes batches of at most %d",
                pa::kBalancedMaxBatch);
  if (prefix_tokens <= 0 || prefix_tokens % block_size)
    return fail(PA_ERR_INVALID_ARG, "prefix_tokens must be a positive multiple of block_size");
  return p.ws_bytes + prefix_plan(batch, num_q_heads, num_kv_heads, head_dim, prefix_tokens).extra_ws_bytes;
}

int pa_decode_shared_prefix(pa_tensor* out, const pa_tensor* query, const pa_tensor* key_cache,
                            const pa_tensor* value_cache, const pa_tensor* block_tables,
                            const pa_tensor* seq_lens, const pa_tensor* prefix_blocks,
                            int32_t prefix_tokens, float scale, int32_t block_size,
                            int32_t num_kv_heads, const pa_launch* launch) {
  int rc;
  if ((rc = check_tensor(query, "query", 3)) || (rc = check_tensor(prefix_blocks, "prefix_blocks", 1)))
    return rc;
  if (query->dtype != PA_F16 && query->dtype != PA_BF16)
    return fail(PA_ERR_INVALID_ARG, "the shared-prefix decode needs an f16 or bf16 query");
  if (!(scale > 0.f) || !isfinite(scale)) return fail(PA_ERR_INVALID_ARG, "scale must be positive and finite");
  if (block_size <= 0 || prefix_tokens <= 0 || prefix_tokens % block_size)
    return fail(PA_ERR_INVALID_ARG, "prefix_tokens must be a positive multiple of block_size");
  if (prefix_blocks->dtype != PA_I32 || prefix_blocks->shape[0] < prefix_tokens / block_size ||
      (prefix_blocks->shape[0] > 1 && prefix_blocks->stride[0] != 1))
    return fail(PA_ERR_INVALID_ARG, "prefix_blocks must be int32 [>= prefix_tokens / block_size], contiguous");
  // the plan is always the balanced schedule (automatic partitioning)
  pa_launch ln = launch ? *launch : pa_launch{nullptr, nullptr, 0, 0, 0};
  if (ln.partition_tokens != 0)
    return fail(PA_ERR_INVALID_ARG, "the shared-prefix decode plans its own pieces (partition_tokens 0)");
  const int64_t B = query->shape[0], Hq = query->shape[1], D = query->shape[2];
  if (num_kv_heads <= 0) return fail(PA_ERR_INVALID_ARG, "num_kv_heads must be positive");
  const PrefixPlan pp = prefix_plan(B, Hq, num_kv_heads, D, prefix_tokens);
  // the grouped prefix work lives in the matrix-core decode kernel, which
  // then runs the rest of every sequence too, whatever the group size
  if (!pp.pass) {
    if (ln.path == PA_PATH_AUTO) ln.path = PA_PATH_MFMA;
    if (ln.path != PA_PATH_MFMA)
      return fail(PA_ERR_UNSUPPORTED,
                  "with fewer than %lld (sequence, query head) rows per kv head the shared-prefix "
                  "decode runs on the matrix-core path", (long long)kPassRows);
  }
  pa::DecodeParams p;
  pa::DecodeVariant v;
  Plan plan;
  bool empty;
  if ((rc = decode_setup(out, query, key_cache, value_cache, block_tables, seq_lens, scale, block_size,
                         num_kv_heads, &ln, pp.extra_ws_bytes, &p, &v, &plan, &empty,
                         true)))
    return rc;
  if (plan.sched != pa::kSchedBalanced)
    return fail(PA_ERR_UNSUPPORTED, "the shared-prefix decode takes batches of at most %d",
                pa::kBalancedMaxBatch);
  if (pp.pass && !pa::prefill_variant_built(v.qkind, v.kvkind, (int)D))
    return fail(PA_ERR_UNSUPPORTED, "no shared-prefix pass for this dtype / head_dim");
  if ((int64_t)prefix_tokens > (int64_t)p.max_blocks * p.bs)
    return fail(PA_ERR_INVALID_ARG, "prefix_tokens exceeds what the block table addresses");
  if (empty) return PA_OK;
  // workspace: acc [slots, Hq, D], (max, sum) [slots, Hq, 2], meta [B, 2],
  // with the prefix pieces' slots after the decode's own
  const int64_t slots = plan.slots + B * pp.pieces;
  p.ws_acc = static_cast<float*>(ln.workspace);
  p.ws_ml = p.ws_acc + slots * Hq * D;
  p.ws_meta = reinterpret_cast<int32_t*>(p.ws_ml + slots * Hq * 2);
  p.skip = prefix_tokens;
  p.prefix_pieces = pp.pieces;
  p.prefix_slot0 = (int32_t)plan.slots;
  p.piece_cost = kPieceCost;
  hipStream_t stream = static_cast<hipStream_t>(ln.stream);
  hipError_t e;
  if (pp.pass) {
    pa::PrefillParams f;
    memset(&f, 0, sizeof f);
    f.flags = p.flags;
    f.q = query->data;
    f.kc = key_cache->data;
    f.vc = value_cache->data;
    f.tables = static_cast<const int32_t*>(prefix_blocks->data);
    f.tab_stride = 0;
    f.lens = p.lens;
    f.q_st = query->stride[0];
    f.q_sh = query->stride[1];
    f.B = p.B;
    f.Hq = p.Hq;
    f.Hkv = p.Hkv;
    f.G = p.G;
    f.D = p.D;
    f.bs = p.bs;
    f.T = p.B;
    f.max_blocks = p.max_blocks;
    f.num_blocks = p.num_blocks;
    f.spb_shift = -1;
    for (int sh = 0; sh < 24; ++sh)
      if ((16 << sh) == p.bs) f.spb_shift = sh;
    f.qk_scale_log2 = p.qk_scale_log2;
    f.v_scale = p.v_scale;
    f.ws_acc = p.ws_acc;
    f.ws_ml = p.ws_ml;
    f.pfx_slot0 = p.prefix_slot0;
    f.pfx_pieces = pp.pieces;
    f.pfx_tokens = prefix_tokens;
    f.pfx_chunk = pp.tokens;
    f.pfx_row_tiles = pp.row_tiles;
    e = pa::launch_prefix_pass(f, v.qkind, v.kvkind, stream);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "prefix pass launch failed: %s", hipGetErrorString(e));
  } else {
    p.prefix_blocks = static_cast<const int32_t*>(prefix_blocks->data);
    p.grp_tokens = pp.tokens;
    // the grouped work's rows of workgroups come out of the decode shares'
    // budget, so that the whole grid is resident at once
    const int64_t grp_units = (int64_t)p.Hkv * pp.row_groups;
    const int64_t chunks = (p.units + p.waves - 1) / p.waves;
    const int64_t grp_y = ((grp_units * pp.pieces + p.waves - 1) / p.waves + chunks - 1) / chunks;
    int max_waves, workgroups;
    pa::decode_launch_shape(v, &max_waves, &workgroups);
    const int64_t per = std::max<int64_t>(1, workgroups / chunks);
    const int64_t nwc = std::max(per - grp_y, std::max<int64_t>(per / 4, 1));
    if (grp_units > 0x7FFFFFFF / pp.pieces || nwc + grp_y > 65535)
      return fail(PA_ERR_UNSUPPORTED, "batch too large for the shared-prefix decode");
    p.grp_units = (int32_t)grp_units;
    p.grp_y = (int32_t)grp_y;
    p.nwc = (int32_t)nwc;
  }
  e = pa::launch_decode(p, v, stream);
  if (e != hipSuccess) return fail(PA_ERR_HIP, "decode launch failed: %s", hipGetErrorString(e));
  return PA_OK;
}

int pa_reshape_and_cache(const pa_tensor* key, const pa_tensor* value, const pa_tensor* slot_mapping,
                         pa_tensor* key_cache, pa_tensor* value_cache, const pa_launch* launch) {
  int rc;
  if ((rc = check_tensor(key, "key", 3)) || (rc = check_tensor(value, "value", 3)) ||
      (rc = check_tensor(slot_mapping, "slot_mapping", 1)) ||
      (rc = check_cache_pair(key_cache, value_cache)))
    return rc;
  const int sdt = key->dtype;
  if (value->dtype != sdt) return fail(PA_ERR_INVALID_ARG, "key and value dtypes differ");
  if (sdt != PA_F32 && sdt != PA_F16 && sdt != PA_BF16)
    return fail(PA_ERR_INVALID_ARG, "key/value dtype must be f32, f16 or bf16");
  const int cdt = key_cache->dtype;
  if (cdt != sdt && cdt != PA_FP8_E4M3)
    return fail(PA_ERR_INVALID_ARG, "cache dtype must equal the key dtype or be fp8");
  const int64_t T = key->shape[0], Hkv = key->shape[1], D = key->shape[2];
  for (int i = 0; i < 3; ++i)
    if (value->shape[i] != key->shape[i]) return fail(PA_ERR_INVALID_ARG, "key and value shapes differ");
  if (slot_mapping->dtype != PA_I64 || slot_mapping->shape[0] != T)
    return fail(PA_ERR_INVALID_ARG, "slot_mapping must be int64 [num_tokens]");
  if (T > 1 && slot_mapping->stride[0] != 1) return fail(PA_ERR_INVALID_ARG, "slot_mapping must be contiguous");
  if (key_cache->shape[2] != Hkv || key_cache->shape[3] != D)
    return fail(PA_ERR_INVALID_ARG, "cache [.., .., Hkv, D] must match key [T, Hkv, D]");
  if (key->stride[2] != 1 || value->stride[2] != 1 || key->stride[1] != D || value->stride[1] != D)
    return fail(PA_ERR_INVALID_ARG, "key/value rows [Hkv, D] must be contiguous");
  if ((Hkv * D) % 8) return fail(PA_ERR_UNSUPPORTED, "num_kv_heads * head_dim must be a multiple of 8");
  const int64_t vec = 16 / elem_size(sdt);
  if (!aligned16(key->data) || !aligned16(value->data) || (T > 1 && (key->stride[0] % vec || value->stride[0] % vec)))
    return fail(PA_ERR_INVALID_ARG, "key/value token rows must be 16-byte aligned");
  if (T == 0) return PA_OK;
  pa::CacheWriteParams p;
  memset(&p, 0, sizeof p);
  int frc = flags_of(launch, &p.flags);
  if (frc) return frc;
  p.key = key->data;
  p.value = value->data;
  p.slots = static_cast<const int64_t*>(slot_mapping->data);
  p.kc = key_cache->data;
  p.vc = value_cache->data;
  p.k_stride_tok = key->stride[0];
  p.v_stride_tok = value->stride[0];
  p.T = T;
  p.Hkv = (int)Hkv;
  p.D = (int)D;
  p.bs = (int)key_cache->shape[1];
  p.num_slots = key_cache->shape[0] * key_cache->shape[1];
  p.k_scale = key_cache->scale;
  p.v_scale = value_cache->scale;
  hipStream_t stream = launch ? static_cast<hipStream_t>(launch->stream) : nullptr;
  hipError_t e = pa::launch_cache_write(p, kind_of(sdt), kind_of(cdt), stream);
  if (e != hipSuccess) return fail(PA_ERR_HIP, "cache write launch failed: %s", hipGetErrorString(e));
  return PA_OK;
}

int pa_prefill(pa_tensor* out, const pa_tensor* query, const pa_tensor* key_cache,
               const pa_tensor* value_cache, const pa_tensor* block_tables,
               const pa_tensor* seq_lens, const pa_tensor* query_start_loc,
               int32_t max_query_len, float scale, int32_t block_size, int32_t num_kv_heads,
               const pa_launch* launch) {
  int rc;
  if ((rc = check_tensor(query, "query", 3)) || (rc = check_tensor(out, "out", 3)) ||
      (rc = check_cache_pair(key_cache, value_cache)) ||
      (rc = check_tensor(block_tables, "block_tables", 2)) ||
      (rc = check_tensor(seq_lens, "seq_lens", 1)) ||
      (rc = check_tensor(query_start_loc, "query_start_loc", 1)))
    return rc;
  const int qdt = query->dtype;
  if (qdt != PA_F16 && qdt != PA_BF16) return fail(PA_ERR_INVALID_ARG, "query dtype must be f16 or bf16");
  if (out->dtype != qdt) return fail(PA_ERR_INVALID_ARG, "out dtype must equal the query dtype");
  const int64_t T = query->shape[0], Hq = query->shape[1], D = query->shape[2];
  for (int i = 0; i < 3; ++i)
    if (out->shape[i] != query->shape[i]) return fail(PA_ERR_INVALID_ARG, "out shape must equal the query shape");
  if (query->stride[2] != 1 || out->stride[2] != 1)
    return fail(PA_ERR_INVALID_ARG, "query/out head_dim stride must be 1");
  const int64_t N = key_cache->shape[0], bs = key_cache->shape[1], Hkv = key_cache->shape[2];
  if (key_cache->shape[3] != D) return fail(PA_ERR_INVALID_ARG, "cache head_dim %lld != query head_dim %lld",
                                            (long long)key_cache->shape[3], (long long)D);
  if (bs != block_size) return fail(PA_ERR_INVALID_ARG, "block_size %d != cache block dimension %lld",
                                    block_size, (long long)bs);
  if (Hkv != num_kv_heads) return fail(PA_ERR_INVALID_ARG, "num_kv_heads %d != cache head dimension %lld",
                                       num_kv_heads, (long long)Hkv);
  if (Hkv <= 0 || Hq % Hkv) return fail(PA_ERR_INVALID_ARG, "num_q_heads must be a multiple of num_kv_heads");
  if (bs % 16) return fail(PA_ERR_UNSUPPORTED, "block_size must be a multiple of 16 (got %lld)", (long long)bs);
  const int kvdt = key_cache->dtype;
  if (kvdt != qdt && kvdt != PA_FP8_E4M3)
    return fail(PA_ERR_INVALID_ARG, "cache dtype must equal the query dtype, or be fp8");
  if (block_tables->dtype != PA_I32 || seq_lens->dtype != PA_I32 || query_start_loc->dtype != PA_I32)
    return fail(PA_ERR_INVALID_ARG, "block_tables, seq_lens and query_start_loc must be int32");
  const int64_t B = seq_lens->shape[0];
  if (block_tables->shape[0] != B || query_start_loc->shape[0] != B + 1)
    return fail(PA_ERR_INVALID_ARG, "block_tables [B, .] and query_start_loc [B + 1] must match seq_lens [B]");
  if (block_tables->stride[1] != 1 || (seq_lens->stride[0] != 1 && B > 1) || query_start_loc->stride[0] != 1)
    return fail(PA_ERR_INVALID_ARG, "block_tables column stride, seq_lens and query_start_loc strides must be 1");
  if (B > 65535) return fail(PA_ERR_UNSUPPORTED, "batch above 65535");
  if (Hq > 65535) return fail(PA_ERR_UNSUPPORTED, "more than 65535 query heads");
  if (Hq * B > (1LL << 24)) return fail(PA_ERR_UNSUPPORTED, "num_q_heads * batch above 2^24");
  if (T > 0x7FFFFFFFLL || N > 0x7FFFFFFFLL || block_tables->shape[1] > 0x7FFFFFFFLL)
    return fail(PA_ERR_UNSUPPORTED, "rows, pool or table too large");
  if ((int64_t)block_tables->shape[1] * bs > (1LL << 30))
    return fail(PA_ERR_INVALID_ARG, "block table addresses too many tokens");
  if (!isfinite(scale) || !(scale > 0.f)) return fail(PA_ERR_INVALID_ARG, "scale must be positive and finite");
  const int64_t vec = 8;  // 16-bit elements per 16 bytes
  if (!aligned16(query->data) || query->stride[0] % vec || query->stride[1] % vec)
    return fail(PA_ERR_INVALID_ARG, "query rows must be 16-byte aligned");
  if (!aligned16(out->data) || out->stride[0] % vec || out->stride[1] % vec)
    return fail(PA_ERR_INVALID_ARG, "out rows must be 16-byte aligned");
  if (!pa::prefill_variant_built(kind_of(qdt), kind_of(kvdt), (int)D))
    return fail(PA_ERR_UNSUPPORTED, "no prefill variant for this dtype / head_dim (64 and 128 are built)");
  if (B == 0 || T == 0 || Hq == 0) return PA_OK;

  const int64_t ranks = prefill_ranks(B, Hq, T, max_query_len);
  pa::PrefillParams p;
  memset(&p, 0, sizeof p);
  int frc = flags_of(launch, &p.flags);
  if (frc) return frc;
  p.out = out->data;
  p.q = query->data;
  p.kc = key_cache->data;
  p.vc = value_cache->data;
  p.tables = static_cast<const int32_t*>(block_tables->data);
  p.lens = static_cast<const int32_t*>(seq_lens->data);
  p.qsl = static_cast<const int32_t*>(query_start_loc->data);
  p.q_st = query->stride[0];
  p.q_sh = query->stride[1];
  p.o_st = out->stride[0];
  p.o_sh = out->stride[1];
  p.tab_stride = block_tables->stride[0];
  p.B = (int)B;
  p.Hq = (int)Hq;
  p.Hkv = (int)Hkv;
  p.G = (int)(Hq / Hkv);
  p.D = (int)D;
  p.bs = (int)bs;
  p.tile_ranks = (int)ranks;
  p.T = (int)T;
  p.max_blocks = (int)block_tables->shape[1];
  p.num_blocks = (int)N;
  p.xcd_groups = (B * Hkv) % 8 == 0 ? (int)(B * Hkv / 8) : 0;
  p.spb_shift = -1;
  for (int sh = 0; sh < 24; ++sh)
    if ((int64_t)16 << sh == bs) p.spb_shift = sh;
  const double ks = kvdt == PA_FP8_E4M3 ? (double)key_cache->scale : 1.0;
  p.qk_scale_log2 = (float)((double)scale * ks * 1.4426950408889634);
  p.v_scale = kvdt == PA_FP8_E4M3 ? value_cache->scale : 1.0f;
  // bf16 query and K/V: with a workspace for the per-workgroup flags, P x V
  // runs in f16 (and a second launch redoes the flagged workgroups in bf16)
  if (qdt == PA_BF16 && kvdt == PA_BF16 && launch && launch->workspace) {
    const int64_t need = pa::prefill_grid_size(B, Hq, ranks) * (int64_t)sizeof(int32_t);
    if (reinterpret_cast<uintptr_t>(launch->workspace) % 4)
      return fail(PA_ERR_INVALID_ARG, "workspace must be 4-byte aligned");
    if (launch->workspace_bytes >= (size_t)need) p.wide_flags = static_cast<int32_t*>(launch->workspace);
  }
  hipStream_t stream = launch ? static_cast<hipStream_t>(launch->stream) : nullptr;
  hipError_t e = pa::launch_prefill(p, kind_of(qdt), kind_of(kvdt), stream);
  if (e != hipSuccess) return fail(PA_ERR_HIP, "prefill launch failed: %s", hipGetErrorString(e));
  return PA_OK;
}

int64_t pa_prefill_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_rows,
                                   int32_t max_query_len) {
  if (batch < 0 || num_q_heads < 0 || num_rows < 0)
    return fail(PA_ERR_INVALID_ARG, "sizes must not be negative");
  const int64_t ranks = prefill_ranks(batch, num_q_heads, num_rows, max_query_len);
  return pa::prefill_grid_size(batch, num_q_heads, ranks) * (int64_t)sizeof(int32_t);
}

namespace {

// shared checks of pa_copy_blocks / pa_swap_blocks; fills the byte size
int check_block_copy(const pa_tensor* dk, const pa_tensor* dv, const pa_tensor* sk,
                     const pa_tensor* sv, const pa_tensor* pairs, int64_t* block_bytes) {
  int rc;
  if ((rc = check_cache_pair(dk, dv)) || (rc = check_cache_pair(sk, sv)) ||
      (rc = check_tensor(pairs, "block_pairs", 2)))
    return rc;
  if (sk->dtype != dk->dtype) return fail(PA_ERR_INVALID_ARG, "source and destination pools differ in dtype");
  for (int i = 1; i < 4; ++i)
    if (sk->shape[i] != dk->shape[i])
      return fail(PA_ERR_INVALID_ARG, "source and destination blocks differ in shape");
  if (pairs->dtype != PA_I32 || pairs->shape[1] != 2 || !contiguous(pairs))
    return fail(PA_ERR_INVALID_ARG, "block_pairs must be contiguous int32 [n, 2]");
  const int64_t bytes = dk->shape[1] * dk->shape[2] * dk->shape[3] * elem_size(dk->dtype);
  if (bytes % 16) return fail(PA_ERR_UNSUPPORTED, "block bytes must be a multiple of 16");
  *block_bytes = bytes;
  return PA_OK;
}

int launch_block_copy(const pa_tensor* dk, const pa_tensor* dv, const pa_tensor* sk,
                      const pa_tensor* sv, const pa_tensor* pairs, int64_t bytes,
                      const pa_launch* launch, const char* what) {
  pa::CopyBlocksParams p;
  int frc = flags_of(launch, &p.flags);
  if (frc) return frc;
  p.src_k = sk->data;
  p.src_v = sv->data;
  p.dst_k = dk->data;
  p.dst_v = dv->data;
  p.pairs = static_cast<const int32_t*>(pairs->data);
  p.n = pairs->shape[0];
  p.block_bytes = bytes;
  p.src_blocks = sk->shape[0];
  p.dst_blocks = dk->shape[0];
  if (p.n == 0) return PA_OK;
  hipStream_t stream = launch ? static_cast<hipStream_t>(launch->stream) : nullptr;
  hipError_t e = pa::launch_copy_blocks(p, stream);
  if (e != hipSuccess) return fail(PA_ERR_HIP, "%s launch failed: %s", what, hipGetErrorString(e));
  return PA_OK;
}

}  // namespace

int pa_copy_blocks(pa_tensor* key_cache, pa_tensor* value_cache, const pa_tensor* block_pairs,
                   const pa_launch* launch) {
  int64_t bytes;
  int rc = check_block_copy(key_cache, value_cache, key_cache, value_cache, block_pairs, &bytes);
  if (rc) return rc;
  return launch_block_copy(key_cache, value_cache, key_cache, value_cache, block_pairs, bytes, launch,
                           "block copy");
}

int pa_swap_blocks(pa_tensor* dst_key_cache, pa_tensor* dst_value_cache,
                   const pa_tensor* src_key_cache, const pa_tensor* src_value_cache,
                   const pa_tensor* block_pairs, const pa_launch* launch) {
  int64_t bytes;
  int rc = check_block_copy(dst_key_cache, dst_value_cache, src_key_cache, src_value_cache,
                            block_pairs, &bytes);
  if (rc) return rc;
  return launch_block_copy(dst_key_cache, dst_value_cache, src_key_cache, src_value_cache,
                           block_pairs, bytes, launch, "block swap");
}

}  // extern "C"

// shared with the allocator translation unit
namespace pa {
int set_error(int code, const char* msg) { return fail(code, "%s", msg); }
}  // namespace pa
