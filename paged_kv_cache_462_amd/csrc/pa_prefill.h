// Internal interface of the paged prefill kernel (pa_prefill.hip) for the
// C-ABI layer.  Host code only; no torch types.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// Everything the prefill kernel reads, resolved on the host.
struct PrefillParams {
  void* out;              // [T, Hq, D] query dtype
  const void* q;          // [T, Hq, D]
  const void* kc;         // [N, bs, Hkv, D]
  const void* vc;
  const int32_t* tables;  // [B, tab_stride]
  const int32_t* lens;    // [B] tokens in the cache, new ones included
  const int32_t* qsl;     // [B + 1] first packed row of each sequence
  int64_t q_st, q_sh;     // query strides (elements): token, head
  int64_t o_st, o_sh;     // output strides
  int64_t tab_stride;     // block-table row stride
  int32_t B, Hq, Hkv, G, D, bs;
  int32_t T;              // query / output rows
  int32_t max_blocks;     // block-table width (lengths are clamped to it)
  int32_t num_blocks;     // pool size (ids outside it read block 0)
  int32_t tile_ranks;     // query-tile ranks in the grid (grid.x / (Hq * B))
  int32_t spb_shift;      // log2(bs / 16) when bs / 16 is a power of two, else -1
  int32_t xcd_groups;     // (sequence, kv head) groups per XCD when B * Hkv is a
                          // multiple of 8, else 0 (plain order)
  float qk_scale_log2;    // scale * k_scale * log2(e)
  float v_scale;          // fp8 V scale (1 otherwise)
  // Shared-prefix pass of a decode batch (prefix_pass_* launch): the rows
  // are every (sequence, query head) of one kv head, the keys the first
  // pfx_tokens tokens (blocks listed in `tables`, tab_stride 0), row b's
  // limited to min(lens[b], pfx_tokens); q_st is the query's sequence
  // stride.  Workgroup (kv head, row tile, key piece) leaves one (max, sum,
  // unnormalised output) triple per row at slot pfx_slot0 + b * pfx_pieces
  // + piece of ws_acc [slots, Hq, D] / ws_ml [slots, Hq, 2].
  float* ws_acc;
  float* ws_ml;
  int32_t pfx_slot0, pfx_pieces, pfx_tokens, pfx_chunk, pfx_row_tiles;
  int32_t* flags;         // caller's error flags [kNumFlags], or null
  // bf16 query and bf16 K/V (causal prefill): one int per workgroup of the
  // grid, or null.  With it the prefill runs P x V in f16 (V converted while
  // staged, exact below 2^16) and each workgroup stores whether it met a V
  // value outside f16's range; a second launch recomputes exactly those
  // workgroups with the bf16 product (the others exit at once).
  int32_t* wide_flags;
};

// Query rows one workgroup takes.
int prefill_rows_per_workgroup();

// hipErrorNotSupported when no built variant matches (qkind, kvkind, D).
// A bf16 query with fp8 K/V runs P x V in f16 (fp8 values always fit); with
// bf16 K/V it does when p.wide_flags is set (two launches), else in bf16.
hipError_t launch_prefill(const PrefillParams& p, int qkind, int kvkind, hipStream_t stream);

// Workgroups of the causal prefill grid (the wide_flags entries it needs).
int64_t prefill_grid_size(int64_t B, int64_t Hq, int64_t tile_ranks);

bool prefill_variant_built(int qkind, int kvkind, int D);

// The shared-prefix pass (same variants as prefill); grid Hkv * pfx_row_tiles
// * pfx_pieces workgroups.
hipError_t launch_prefix_pass(const PrefillParams& p, int qkind, int kvkind, hipStream_t stream);

}  // namespace pa
