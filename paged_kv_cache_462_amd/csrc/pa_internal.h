// Internal interface between the C-ABI layer (pa_api.cpp) and the HIP
// launchers.  Host code only; no torch types.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

enum Kind : int { K_F32 = 0, K_F16 = 1, K_BF16 = 2, K_FP8 = 3 };

// Decode schedules.  Fixed: grid (unit chunks, partitions, sequences), one
// workgroup per fixed-size token partition of one sequence.  Balanced: grid
// (unit chunks, nwc), the batch's 16-token tiles (all sequences back to
// back) dealt out in equal contiguous shares, one per workgroup; a share
// may cover the end of one sequence and the start of the next.
enum Sched : int { kSchedFixed = 0, kSchedBalanced = 1 };

// Caller's error flags (the launch's error_flags): index of the flag a
// kernel sets to 1 when it takes device-resident contents outside their
// contract the documented way (same order as the C ABI's PA_FLAG_*).
enum Flag : int { kFlagBlockId = 0, kFlagLength = 1, kFlagSlot = 2, kFlagQueryStart = 3, kNumFlags = 4 };

// Balanced schedule limits: workgroups per unit chunk (the workspace is
// sized for this many) and the largest batch it takes (the per-sequence
// tile offsets live in LDS).
constexpr int kBalancedWorkgroups = 256;
// The fp8 matrix-core kernel's registers and LDS leave room for three waves
// per SIMD: it runs 4-wave workgroups, three per CU (768 in all), which
// hides its per-tile latency better than two 8-wave waves per SIMD do.
constexpr int kFp8Waves = 4;
constexpr int kBalancedWorkgroupsFp8 = 768;
// Shares per unit chunk the workspace holds slots for (the larger grid).
constexpr int kBalancedSlots = kBalancedWorkgroupsFp8;
constexpr int kBalancedMaxBatch = 2048;

// Everything the decode kernels read, resolved on the host.
struct DecodeParams {
  void* out;              // [B, Hq, D] query dtype
  const void* q;          // [B, Hq, D]
  const void* kc;         // [N, bs, Hkv, D]
  const void* vc;
  const int32_t* tables;  // [B, tab_stride]
  const int32_t* lens;    // [B]
  float* ws_acc;          // [slots, Hq, D] partial outputs (split only)
  float* ws_ml;           // [slots, Hq, 2] (max, sum) (split only)
  int32_t* ws_meta;       // [B, 2] (first slot, pieces) (balanced schedule)
  int64_t q_sb, q_sh;     // query strides (elements)
  int64_t o_sb, o_sh;     // output strides
  int64_t tab_stride;     // block-table row stride
  int32_t B, Hq, Hkv, G, D, bs, max_blocks;
  int32_t num_blocks;     // physical pool size
  int32_t head_tiles;     // ceil(G / tile heads)
  int32_t units;          // Hkv * head_tiles: one wave each per partition
  int32_t waves;          // waves per workgroup (consecutive units)
  int32_t sched;          // kSchedFixed or kSchedBalanced
  int32_t part_tokens;    // fixed: tokens per partition (multiple of 16)
  int32_t num_parts;      // fixed: partitions per sequence in the grid (>= 1)
  int32_t nwc;            // balanced: workgroups per unit chunk
  int32_t split;          // 1: pieces may leave triples, merged afterwards
  float qk_scale_log2;    // scale * k_scale * log2(e)
  float v_scale;          // fp8 V scale (1 otherwise)
  // Shared-prefix split (balanced schedule only): the first `skip` tokens
  // of every sequence are attended by a separate pass that leaves
  // `prefix_pieces` triples per (sequence, query head) at slots
  // prefix_slot0 + b * prefix_pieces + k; this pass covers the rest and
  // every one of its pieces leaves a triple.  All 0 for plain decode.
  int32_t skip;
  int32_t prefix_pieces;
  int32_t prefix_slot0;
  int32_t* flags;         // caller's error flags [kNumFlags], or null
  // Balanced schedule: the cost, in tiles, charged for the start of every
  // non-empty sequence when the shares are dealt (0: shares of equal tiles;
  // the shared-prefix decode charges 3)
  int32_t piece_cost;
  // Grouped prefix work of a shared-prefix decode (matrix-core kernel,
  // balanced schedule): grp_y more rows of workgroups after the nwc decode
  // shares.  A unit is (row group, kv head): the kv head's (sequence, query
  // head) rows, sequence-major, in groups of 16 that share each K/V tile of
  // the prefix (blocks prefix_blocks[0 ..]); a wave takes one unit over one
  // piece of grp_tokens tokens of the first skip tokens, each row limited
  // to its own sequence's length, and leaves one triple per row at the
  // prefix slots.  grp_units 0: none.
  const int32_t* prefix_blocks;
  int32_t grp_units;      // Hkv * ceil(B * G / 16)
  int32_t grp_tokens;     // tokens per piece (multiple of 16)
  int32_t grp_y;
};

struct DecodeVariant {
  int qkind;   // K_F32 / K_F16 / K_BF16
  int kvkind;  // K_F32 / K_F16 / K_BF16 / K_FP8
  int D;
  int path;    // 1 VALU, 2 MFMA
  int gt;      // query heads per workgroup tile (MFMA: 16; VALU: 1, 2 or 4)
};

// Device scratch the library keeps for pa_decode_noalloc: one fixed array
// per device (a file-scope __device__ array in pa_decode.hip), found once per
// device.  decode_scratch gives its address on the device of `stream` (the
// current device for the null stream); no allocation is made.
constexpr int64_t kDecodeScratchBytes = 16ll << 20;
hipError_t decode_scratch(hipStream_t stream, void** ptr);

// Launch the decode (and the merge when p.split).  Returns hipSuccess or the
// launch error; hipErrorNotSupported when no variant matches.
hipError_t launch_decode(const DecodeParams& p, const DecodeVariant& v,
                         hipStream_t stream);

struct CacheWriteParams {
  const void* key;        // [T, Hkv, D]
  const void* value;
  const int64_t* slots;   // [T]
  void* kc;               // [N, bs, Hkv, D]
  void* vc;
  int64_t k_stride_tok, v_stride_tok;  // elements between tokens of key/value
  int64_t T;
  int32_t Hkv, D, bs;
  int64_t num_slots;      // N * bs (slots beyond are ignored)
  float k_scale, v_scale; // fp8 caches
  int32_t* flags;         // caller's error flags [kNumFlags], or null
};

hipError_t launch_cache_write(const CacheWriteParams& p, int src_kind,
                              int cache_kind, hipStream_t stream);

// Whole-block copies from one pair of pools to another (the same pools for
// copy-on-write; a device pool and a pool in pinned host memory for swap).
struct CopyBlocksParams {
  const void* src_k;
  const void* src_v;
  void* dst_k;
  void* dst_v;
  const int32_t* pairs;   // [n, 2] (source block, destination block)
  int64_t n;
  int64_t block_bytes;    // bytes of one physical block (bs * Hkv * D * esize)
  int64_t src_blocks;     // pool sizes; pairs outside them are skipped
  int64_t dst_blocks;
  int32_t* flags;         // caller's error flags [kNumFlags], or null
};

hipError_t launch_copy_blocks(const CopyBlocksParams& p, hipStream_t stream);

// Variants built into this library (for pa_build_info / validation).
bool decode_variant_built(const DecodeVariant& v);

// Launch shape of a decode variant: waves per workgroup at most, and the
// balanced schedule's workgroups in all.
void decode_launch_shape(const DecodeVariant& v, int* max_waves, int* workgroups);

}  // namespace pa
