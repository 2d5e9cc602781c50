// Paged decode attention kernels for gfx950 (CDNA4).
//
// The method: for one query token per sequence, walk the sequence's logical
// blocks, look each one up in the block table, read that physical block's K
// and V rows (the last block only partly filled), and fold the scores into a
// running (max, sum, output) state that is rescaled whenever the maximum
// grows; the result is output / sum ("paged-attention-and-vllm-inference",
// code block `paged_attention`; "5.KV Cache 管理 & PagedAttention",
// question 19, block-wise fusion of the block table with the online
// softmax).  Query heads share kv heads in groups of G = Hq / Hkv
// (same page, question 7).
//
// Work decomposition.  A work unit is one (kv head, tile of query heads of
// its group).  A workgroup is up to eight consecutive units (a unit chunk),
// one wave each; the waves walk the same token range of the same sequences,
// so each physical block's K (and V) rows of neighbouring heads, which are
// adjacent in memory, are fetched together.  On MI355X that keeps the DRAM
// access stream close to a sequential one (6.9 TB/s for the bare gather,
// against 5.7 TB/s when each workgroup walks one head on its own).  A wave
// keeps its own softmax state per sequence piece and never merges it with
// another wave's.
//
// Which token ranges a workgroup takes (the schedule):
//  * balanced: the 16-token tiles of all sequences, back to back, are dealt
//    out in equal contiguous shares, one per workgroup of a unit chunk, so
//    every workgroup moves the same number of bytes whatever the length mix.
//    Each workgroup works the per-sequence tile offsets out itself from
//    seq_lens (a prefix sum in LDS), so the host never needs the lengths.
//  * fixed: one workgroup per fixed-size token partition of one sequence
//    (or per sequence when unsplit).
// A sequence that ends up in several pieces leaves one (max, sum,
// unnormalised output) triple per piece and query head in the workspace;
// merge_kernel combines them in piece order (no atomics, so results are
// bit-reproducible).

// Every K/V load reads whole token rows (16 lanes x 16 bytes for a 256-byte
// row), so a load instruction covers complete 128-byte lines.
//
// Two inner loops:
//  * VALU (small groups): lanes of a row of LPT lanes cover one token's
//    head_dim; q.k partial dot products (v_dot2 for 16-bit data) are summed
//    across the row with DPP; every row keeps its own online-softmax state
//    and the rows are merged with lane shuffles at the end.
//  * MFMA (groups >= 4): scores = K-tile[16 x D] x Q-group^T[D x 16] on
//    v_mfma_f32_16x16x32, then out^T += V^T[D x 16] x P^T[16 x 16] on
//    v_mfma_f32_16x16x16.  The K operand wants one token per lane column,
//    which row loads do not give, so K rows go straight from HBM into a
//    per-wave LDS tile (global_load_lds_dwordx4, no registers held while in
//    flight), stored with an XOR swizzle of the 16-byte chunks so that the
//    transposing ds_read_b128 of 16 different rows hits 16 different bank
//    groups.  The score tile comes out with lane l holding tokens 4*(l/16)+i
//    of head l%16, which is exactly the layout of the P operand; V rows are
//    row loads already in the layout of the V^T operand (MFMA j, row m
//    computes dim m * (D/16) + j).
//
// Block ids are prefetched 64 tiles at a time into one VGPR per wave and
// read with v_readlane, so every K/V address is a scalar 64-bit block base
// plus a 32-bit per-lane offset; the next tile's loads are issued before the
// current tile is computed.
#include <mutex>
#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

// The library's own decode scratch (pa_decode_noalloc): triples and the
// merge plan of one call, for callers that cannot allocate.  Every GPU the
// library runs on holds one copy until the process ends.  In host code
// this name stands for the array, not for its device address: the address
// is looked up per device below and only that is handed to kernels.
static __device__ __align__(256) unsigned char scratch[pa::kDecodeScratchBytes];

namespace pa {

namespace {

constexpr int kTile = 16;
// Lazy-rescale threshold of the matrix-core loop (log2 units).
constexpr float kLazyLog2 = 8.0f;
constexpr int kMaxWaves = 8;
constexpr int kMaxThreads = kMaxWaves * 64;

template <int KIND>
struct Esz {
  static constexpr int v = KIND == K_F32 ? 4 : (KIND == K_FP8 ? 1 : 2);
};

template <int QK>
__device__ __forceinline__ void store_out(void* out, int64_t off, float x) {
  if constexpr (QK == K_F32)
    static_cast<float*>(out)[off] = x;
  else if constexpr (QK == K_F16)
    static_cast<_Float16*>(out)[off] = (_Float16)x;
  else
    static_cast<__bf16*>(out)[off] = (__bf16)x;
}

// N consecutive output elements from fp32 (N a multiple of 4), one store.
template <int QK, int N>
__device__ __forceinline__ void store_out_vec(void* out, int64_t off, const float* x) {
  if constexpr (QK == K_F32) {
#pragma unroll
    for (int k = 0; k < N; k += 4)
      *reinterpret_cast<f32x4*>(static_cast<float*>(out) + off + k) =
          f32x4{x[k], x[k + 1], x[k + 2], x[k + 3]};
  } else {
    uint32_t w[N / 2];
#pragma unroll
    for (int k = 0; k < N / 2; ++k)
      w[k] = QK == K_F16 ? pack_f16(x[2 * k], x[2 * k + 1]) : pack_bf16(x[2 * k], x[2 * k + 1]);
    if constexpr (N == 4) {
      *reinterpret_cast<i32x2*>(static_cast<uint16_t*>(out) + off) = i32x2{(int)w[0], (int)w[1]};
    } else {
#pragma unroll
      for (int k = 0; k < N / 2; k += 4)
        *reinterpret_cast<i32x4*>(static_cast<uint16_t*>(out) + off + 2 * k) =
            i32x4{(int)w[k], (int)w[k + 1], (int)w[k + 2], (int)w[k + 3]};
    }
  }
}

template <int N>
__device__ __forceinline__ void store_f32_vec(float* dst, const float* x) {
#pragma unroll
  for (int k = 0; k < N; k += 4)
    *reinterpret_cast<f32x4*>(dst + k) = f32x4{x[k], x[k + 1], x[k + 2], x[k + 3]};
}

// Sequence length clamped to what the block table can address (a longer
// length is a caller error; clamping keeps every read inside the table).
__device__ __forceinline__ int clamp_len(const DecodeParams& p, int b) {
  const int L = p.lens[b];
  const int cap = p.max_blocks * p.bs;
  if (L < 0 || L > cap) raise_flag(p.flags, kFlagLength);
  return L < 0 ? 0 : (L > cap ? cap : L);
}

// One piece of work of a wave: tokens [t_lo, t_hi) of sequence b, whose
// block-table row is `row`.  The tiles are walked from tile `rot` on,
// wrapping around (the grouped prefix work staggers the waves that read
// the same tiles; 0 elsewhere).
struct Work {
  const int32_t* row;
  int b, L, t_lo, t_hi, n_tiles, rot;
};

// Tile of a piece at walk position i.
__device__ __forceinline__ int walk_tile(const Work& wk, int i) {
  const int j = i + wk.rot;
  return j >= wk.n_tiles ? j - wk.n_tiles : j;
}

// Owner (workgroup index within a unit chunk) of tile t when T tiles are
// dealt to NW workgroups as [floor(w T / NW), floor((w + 1) T / NW)).
__device__ __forceinline__ int tile_owner(int t, int T, int NW) {
  return (int)(((int64_t)(t + 1) * NW - 1) / T);
}

// Tiles of sequence b (tokens from p.skip on) when its length is L.
__device__ __forceinline__ int tiles_of(const DecodeParams& p, int L) {
  return (max(L - p.skip, 0) + kTile - 1) / kTile;
}

// Balanced schedule: s_pref[b] = cost of sequences 0..b-1 (b = 0..B), by a
// workgroup-wide prefix sum; every thread of the workgroup must call it.
// A non-empty sequence costs its tiles plus p.piece_cost: the start of a
// piece (its query and block ids, then its first tile, with nothing in
// flight) takes about as long as that many tiles, so a share that starts
// several sequences gets fewer tiles.  Returns the total cost.
__device__ __forceinline__ int tile_prefix(const DecodeParams& p, int* s_pref, int* s_wtot) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  if (threadIdx.x == 0) s_pref[0] = 0;
  int carry = 0;
  for (int base = 0; base < p.B; base += blockDim.x) {
    const int b = base + threadIdx.x;
    int x = b < p.B ? tiles_of(p, clamp_len(p, b)) : 0;
    if (x > 0) x += p.piece_cost;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (lane == 63) s_wtot[w] = x;
    __syncthreads();
    int before = carry, total = 0;
    for (int k = 0; k < nw; ++k) {
      const int t = s_wtot[k];
      if (k < w) before += t;
      total += t;
    }
    if (b < p.B) s_pref[b + 1] = before + x;
    carry += total;
    __syncthreads();
  }
  __syncthreads();
  return carry;
}

// Calls f(work, slot) for every piece this wave owns, in order: slot < 0
// means the piece is the whole sequence (write the output), else the
// triple slot of the piece.  Every thread of the workgroup must call it
// (the balanced schedule synchronises the workgroup once at the start);
// has_unit is false for waves past the last unit.
template <class F>
__device__ __forceinline__ void for_each_piece(const DecodeParams& p, int* s_pref, int* s_wtot,
                                               bool has_unit, F&& f) {
  if (p.sched == kSchedBalanced) {
    const int T = tile_prefix(p, s_pref, s_wtot);
    // Cost positions: sequence b's first piece_cost positions from s_pref[b]
    // are its start, its tiles follow.  Shares at least piece_cost + 1
    // wide: every one then holds a tile, and the owners of one sequence's
    // tiles are consecutive workgroups (piece k of a sequence is processed
    // by workgroup first + k).
    const int K = p.piece_cost;
    const int NW = min(p.nwc, T > 0 ? max(T / (K + 1), 1) : 0);
    const int wi = blockIdx.y;
    if (blockIdx.x == 0 && wi == 0) {
      // the merge kernel's plan: (first slot, pieces) of every sequence,
      // 0 pieces for an empty one
      for (int b = threadIdx.x; b < p.B; b += blockDim.x) {
        const int sb = s_pref[b], se = s_pref[b + 1];
        int first = 0, pieces = 0;
        if (se > sb) {
          first = tile_owner(sb + K, T, NW);
          pieces = tile_owner(se - 1, T, NW) - first + 1;
        }
        p.ws_meta[2 * b] = first + b;
        p.ws_meta[2 * b + 1] = pieces;
      }
    }
    if (!has_unit || wi >= NW) return;
    const int tb = (int)((int64_t)wi * T / NW);
    const int te = (int)((int64_t)(wi + 1) * T / NW);
    // first sequence whose tiles reach past tb
    int lo = 0, hi = p.B;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (s_pref[mid + 1] > tb) hi = mid;
      else lo = mid + 1;
    }
    for (int b = lo; b < p.B; ++b) {
      const int sb = s_pref[b], se = s_pref[b + 1];
      if (sb >= te) break;
      if (se == sb) continue;  // empty: the merge kernel writes its zeros
      const int r0 = sb + K;  // position of the sequence's first tile
      const int a = max(tb, r0) - r0;
      const int e = min(te, se) - r0;
      if (e <= a) continue;  // the share ends inside the sequence's start
      const int first = tile_owner(r0, T, NW);
      const int pieces = tile_owner(se - 1, T, NW) - first + 1;
      Work wk;
      wk.row = p.tables + (int64_t)b * p.tab_stride;
      wk.rot = 0;
      wk.b = b;
      wk.L = clamp_len(p, b);
      wk.t_lo = p.skip + a * kTile;
      wk.t_hi = min(p.skip + e * kTile, wk.L);
      wk.n_tiles = e - a;
      // slots first + b .. first + b + pieces - 1 belong to sequence b:
      // first_wg(b) + b grows by at least pieces(b) from b to b + 1
      f(wk, pieces > 1 || p.prefix_pieces > 0 ? first + b + (wi - first) : -1);
    }
  } else {
    if (!has_unit) return;
    Work wk;
    wk.b = blockIdx.z;
    wk.row = p.tables + (int64_t)wk.b * p.tab_stride;
    wk.rot = 0;
    const int part = blockIdx.y;
    wk.L = clamp_len(p, wk.b);
    wk.t_lo = part * p.part_tokens;
    if (part > 0 && wk.t_lo >= wk.L) return;  // its triple is never read
    wk.t_hi = min(wk.L, wk.t_lo + p.part_tokens);
    wk.n_tiles = wk.t_hi > wk.t_lo ? (wk.t_hi - wk.t_lo + kTile - 1) / kTile : 0;
    f(wk, p.split && wk.L > p.part_tokens ? wk.b * p.num_parts + part : -1);
  }
}

// Physical block ids of tiles chunk*64 .. chunk*64+63 of the wave's range:
// lane j holds the id of tile chunk*64 + j.
__device__ __forceinline__ int load_block_ids(const DecodeParams& p, const Work& wk, int chunk) {
  const int lane = threadIdx.x & 63;
  const int i = chunk * 64 + lane;
  int id = 0;
  if (i < wk.n_tiles) {
    const int t = wk.t_lo + kTile * walk_tile(wk, i);
    id = wk.row[t / p.bs];
    // an id outside the pool is a caller error; read block 0 instead of
    // faulting
    if ((unsigned)id >= (unsigned)p.num_blocks) {
      raise_flag(p.flags, kFlagBlockId);
      id = 0;
    }
  }
  return id;
}

// Byte offset of tile i inside the pool (block base + row offset in block);
// `ids` holds the block ids of tiles (i & ~63) .. (i | 63).
__device__ __forceinline__ int64_t tile_base(const DecodeParams& p, const Work& wk, int i,
                                             int ids, int64_t blk_bytes, int64_t rs) {
  const int blk = __builtin_amdgcn_readlane(ids, i & 63);
  const int t0 = wk.t_lo + kTile * walk_tile(wk, i);
  return (int64_t)blk * blk_bytes + (int64_t)(t0 % p.bs) * rs;
}

// Two-stage software pipeline over tiles 0..n-1 with buffers A (even tiles)
// and B (odd tiles): tile i + 2's loads are issued right after tile i is
// computed.  In the steady state both next loads are unconditional, so at
// every compute the loads still in flight are exactly the other buffer's,
// and the compiler's wait before it is a count, not a full drain; the last
// one to three tiles are peeled.
template <class LA, class LB, class CA, class CB>
__device__ __forceinline__ void run_pipeline(int base, int n, LA load_a, LB load_b, CA compute_a,
                                             CB compute_b) {
  if (n <= 0) return;
  if (n == 1) {
    load_a(base);
    compute_a(base);
    return;
  }
  load_a(base);
  load_b(base + 1);
  int i = base;
  const int end = base + n;
  // sched_barrier keeps the compiler from sinking a stage's loads below the
  // next compute (which would leave nothing in flight during it)
  for (; i + 3 < end; i += 2) {
    compute_a(i);
    __builtin_amdgcn_sched_barrier(0);
    load_a(i + 2);
    __builtin_amdgcn_sched_barrier(0);
    compute_b(i + 1);
    __builtin_amdgcn_sched_barrier(0);
    load_b(i + 3);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (i + 2 < end) {  // three left
    compute_a(i);
    __builtin_amdgcn_sched_barrier(0);
    load_a(i + 2);
    __builtin_amdgcn_sched_barrier(0);
    compute_b(i + 1);
    compute_a(i + 2);
  } else {            // two left
    compute_a(i);
    compute_b(i + 1);
  }
}

// Wait until every memory operation this wave has issued has completed
// (s_waitcnt with all counters at zero).  The compiler does not reliably
// order an LDS read after a load-to-LDS that fills the same bytes, so the
// LDS tile reads below wait explicitly.
__device__ __forceinline__ void wait_all_memory() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_sched_barrier(0);
}

// One-deep pipeline for kernels whose tiles pass through LDS by
// load-to-LDS.  Tile i is read out of LDS into registers (fetch) after an
// explicit full wait and before tile i + 1's loads are issued, so the wait
// covers exactly tile i and tile i + 1's loads are in flight while tile i is
// computed.
template <class LA, class LB, class FA, class FB, class CA, class CB>
__device__ __forceinline__ void run_pipeline_lds(int base, int n, LA load_a, LB load_b,
                                                 FA fetch_a, FB fetch_b, CA compute_a,
                                                 CB compute_b) {
  if (n <= 0) return;
  const int end = base + n;
  load_a(base);
  for (int i = base; i < end; i += 2) {
    wait_all_memory();
    fetch_a();
    __builtin_amdgcn_sched_barrier(0);
    if (i + 1 < end) load_b(i + 1);
    __builtin_amdgcn_sched_barrier(0);
    compute_a(i);
    __builtin_amdgcn_sched_barrier(0);
    if (i + 1 >= end) break;
    wait_all_memory();
    fetch_b();
    __builtin_amdgcn_sched_barrier(0);
    if (i + 2 < end) load_a(i + 2);
    __builtin_amdgcn_sched_barrier(0);
    compute_b(i + 1);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// All tiles of a wave's range: block ids are fetched 64 tiles at a time
// (one lane each) and the pipeline runs over each 64-tile chunk.
template <class LA, class LB, class CA, class CB>
__device__ __forceinline__ void run_tiles(const DecodeParams& p, const Work& wk, int& ids,
                                          LA load_a, LB load_b, CA compute_a, CB compute_b) {
  for (int c0 = 0; c0 < wk.n_tiles; c0 += 64) {
    ids = load_block_ids(p, wk, c0 >> 6);
    run_pipeline(c0, min(64, wk.n_tiles - c0), load_a, load_b, compute_a, compute_b);
  }
}

template <class LA, class LB, class FA, class FB, class CA, class CB>
__device__ __forceinline__ void run_tiles_lds(const DecodeParams& p, const Work& wk, int& ids,
                                              LA load_a, LB load_b, FA fetch_a, FB fetch_b,
                                              CA compute_a, CB compute_b) {
  for (int c0 = 0; c0 < wk.n_tiles; c0 += 64) {
    ids = load_block_ids(p, wk, c0 >> 6);
    run_pipeline_lds(c0, min(64, wk.n_tiles - c0), load_a, load_b, fetch_a, fetch_b, compute_a,
                     compute_b);
  }
}

// Workspace index of the triple of (slot, query head).
__device__ __forceinline__ int64_t triple_index(const DecodeParams& p, int slot, int h) {
  return (int64_t)slot * p.Hq + h;
}

// ============================================================================
// MFMA inner loop: 16-bit query, 16-bit or fp8 KV, head_dim 64 or 128, a tile
// of up to 16 query heads of one kv group.
// ============================================================================
template <int QK, int KVK, int D>
// The fp8 kernel is sized for three waves per SIMD (at most 168 registers
// a lane, matrix-core accumulators included); the hint keeps the grouped
// copy of the loop from taking more.
__global__ __launch_bounds__(64 * (KVK == K_FP8 ? kFp8Waves : kMaxWaves))
__attribute__((amdgpu_waves_per_eu(KVK == K_FP8 ? 3 : 1))) void decode_mfma_kernel(
    const DecodeParams p) {
  constexpr bool kBF16 = QK == K_BF16;
  constexpr bool kFP8 = KVK == K_FP8;
  // P x V runs in bf16 (P as hi + lo parts) only for bf16 V; fp8 V decodes
  // to f16 exactly (every E4M3 value is an f16 value), so with an fp8 cache
  // it runs in f16 with f16 P, one product, whatever the query type
  constexpr bool kPVBF16 = kBF16 && !kFP8;
  constexpr int ESZ = kFP8 ? 1 : 2;
  constexpr int RB = D * ESZ;          // bytes of one token's head row
  constexpr int LR = RB / 16;          // 16-byte chunks per row
  constexpr int TPI = 64 / LR;         // rows per 1 KiB load-to-LDS instruction
  constexpr int NK = kTile / TPI;      // load-to-LDS instructions per tile
  constexpr int SWZ = 256 / RB;        // consecutive rows sharing one swizzle
  constexpr int NR = LR / 4;           // 16-byte LDS reads per lane per tile
  constexpr int NJQ = D / 32;          // score MFMAs per tile (K = 32 dims each)
  constexpr int NJV = D / 16;          // P x V MFMAs per tile; V elements per lane per token
  constexpr int VBYTES = NJV * ESZ;    // V bytes per lane per token
  constexpr int SLOTS = kTile * LR;    // 16-byte LDS slots per tile
  static_assert(NK >= 1 && NR >= 1 && (kFP8 ? 2 * NR == NJQ : NR == NJQ), "shape");
  static_assert(VBYTES == 16 || VBYTES == 8 || VBYTES == 4, "shape");

  // waves per workgroup at most (the fp8 kernel runs 4-wave workgroups,
  // three per CU)
  constexpr int WMAX = kFP8 ? kFp8Waves : kMaxWaves;
  // two K tiles per wave, in two arrays so the compiler can tell the
  // in-flight tile's LDS writes from the current tile's reads
  __shared__ i32x4 kt0[WMAX][SLOTS];
  __shared__ i32x4 kt1[WMAX][SLOTS];
  // fp8 V goes through LDS as well: its per-lane register loads would be 8
  // bytes (8 dims of a token), half a 16-byte load, so V would cost as many
  // load instructions as K for half the bytes; load-to-LDS moves 1 KiB per
  // instruction and the lanes read their 8 bytes back after the tile's wait
  constexpr bool kVLds = kFP8;
  __shared__ i32x4 vt0[kVLds ? WMAX : 1][kVLds ? SLOTS : 1];
  __shared__ i32x4 vt1[kVLds ? WMAX : 1][kVLds ? SLOTS : 1];
  __shared__ int s_pref[kBalancedMaxBatch + 1];
  __shared__ int s_wtot[kMaxWaves];

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int n = lane & 15;
  const int g = lane >> 4;
  // Workgroups past the decode shares (blockIdx.y >= nwc) take the
  // grouped prefix work of a shared-prefix decode: wave gw is unit
  // gw % grp_units of piece gw / grp_units, a unit being (row group, kv
  // head) with the kv head fastest, so the waves of a workgroup read
  // neighbouring heads of the same tokens.
  const bool grp = p.grp_units > 0 && (int)blockIdx.y >= p.nwc;
  int unit, grp_piece = 0;
  bool has_unit;
  if (grp) {
    const int gw = (((int)blockIdx.y - p.nwc) * (int)gridDim.x + (int)blockIdx.x) * p.waves + w;
    grp_piece = gw / p.grp_units;
    unit = gw - grp_piece * p.grp_units;
    has_unit = grp_piece < p.prefix_pieces;
  } else {
    unit = blockIdx.x * p.waves + w;
    has_unit = unit < p.units;
  }
  const int kvh = grp ? unit % p.Hkv : unit / p.head_tiles;
  const int gh0 = grp ? 0 : (unit - kvh * p.head_tiles) * 16;
  const int nh = grp ? 16 : min(16, p.G - gh0);
  const int head0 = kvh * p.G + gh0;
  // grouped work: this lane's column n is row r of the kv head's
  // (sequence, query head) rows, sequence-major: sequence gb, query head
  // gh, keys [0, glim) of the prefix; the wave's smallest and largest
  // limits decide which tiles need the per-column mask and where its work
  // ends
  // (gb and gh are found again where they are used, which keeps them out
  // of the registers the tile loop holds)
  auto grp_row = [&](int& gb, int& gh) {
    const int r = (unit / p.Hkv) * 16 + n;
    gb = r / p.G;
    gh = kvh * p.G + (r - gb * p.G);
  };
  bool gvalid = false;
  int glim = 0, glmin = 0, glmax = 0;
  if (grp) {
    gvalid = has_unit && (unit / p.Hkv) * 16 + n < p.B * p.G;
    if (gvalid) {
      int gb, gh;
      grp_row(gb, gh);
      glim = min(clamp_len(p, gb), p.skip);
    }
    glmin = gvalid ? glim : 0x7FFFFFFF;
    glmax = gvalid ? glim : 0;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      glmin = min(glmin, __shfl_xor(glmin, off));
      glmax = max(glmax, __shfl_xor(glmax, off));
    }
    glmin = __builtin_amdgcn_readfirstlane(glmin);
    glmax = __builtin_amdgcn_readfirstlane(glmax);
  }

  const int64_t rs = (int64_t)p.Hkv * RB;  // bytes between tokens
  const int64_t blk_bytes = rs * p.bs;
  const char* kbase = static_cast<const char*>(p.kc) + (int64_t)kvh * RB;
  const char* vbase = static_cast<const char*>(p.vc) + (int64_t)kvh * RB;
  // K to LDS: instruction j, lane l loads row tt = j*TPI + l/LR, chunk
  // (l % LR) ^ swz(tt), landing in slot tt*LR + l%LR; so slot tt*LR + s
  // holds chunk s ^ swz(tt) of row tt.
  uint32_t kdma[NK];
#pragma unroll
  for (int j = 0; j < NK; ++j) {
    const int tt = j * TPI + lane / LR;
    const int ch = (lane % LR) ^ ((tt / SWZ) % LR);
    kdma[j] = (uint32_t)(tt * rs + ch * 16);
  }
  // K operand reads: lane (n, g), read r wants chunk 4r + g of row n
  int kslot[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) kslot[r] = n * LR + ((4 * r + g) ^ ((n / SWZ) % LR));
  // V: lane (dim chunk n, group g) reads VBYTES at n*VBYTES of tokens 4g+i.
  uint32_t voff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) voff[i] = (uint32_t)((4 * g + i) * rs + n * VBYTES);
  // fp8 V to LDS: instruction j, lane l loads chunk l % LR of row
  // j*TPI + l/LR into slot j*64 + l (rows unswizzled: slot tt*LR + c holds
  // chunk c of row tt); lane (n, g) reads its VBYTES of token 4g+i back
  uint32_t vdma[NK];
#pragma unroll
  for (int j = 0; j < NK; ++j) vdma[j] = (uint32_t)((j * TPI + lane / LR) * rs + (lane % LR) * 16);
  int vrd[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) vrd[i] = (4 * g + i) * RB + n * VBYTES;

  struct Regs {
    Bytes<VBYTES> v[4];
  };

  // kG: the grouped prefix work's copy of the loop (a compile-time flag, so
  // the decode's copy keeps no register for it)
  auto piece = [&](const Work& wk, int slot, auto grp_tag) {
    constexpr bool kG = decltype(grp_tag)::value;
    // Query group as the B operand of the score MFMAs: lane (n, g) holds
    // column n (head n, or row n of the grouped work), 8 dims per MFMA:
    // those of 16-byte K chunk 4r + g (16-bit K: MFMA r; fp8 K: the low /
    // high half of that chunk for MFMAs 2r, 2r + 1).
    i32x4 qop[NJQ];
    {
      int gb = 0, gh = 0;
      if constexpr (kG) grp_row(gb, gh);
      const uint16_t* qrow =
          static_cast<const uint16_t*>(p.q) +
          (kG ? (int64_t)gb * p.q_sb + (int64_t)gh * p.q_sh
              : (int64_t)wk.b * p.q_sb + (int64_t)(head0 + min(n, nh - 1)) * p.q_sh);
      const bool live = kG ? gvalid : n < nh;
#pragma unroll
      for (int j = 0; j < NJQ; ++j) {
        const int d0 = kFP8 ? ((j >> 1) * 64 + g * 16 + (j & 1) * 8) : (j * 32 + g * 8);
        const i32x4 v = *reinterpret_cast<const i32x4*>(qrow + d0);
        qop[j] = live ? v : i32x4{0, 0, 0, 0};
      }
    }

    int ids = 0;
    auto load_tile = [&](int i, i32x4* kt, i32x4* vt, Regs& r) {
      const int64_t tb = tile_base(p, wk, i, ids, blk_bytes, rs);
      const char* kb = kbase + tb;
      const char* vb = vbase + tb;
#pragma unroll
      for (int j = 0; j < NK; ++j) load_lds16(kb + kdma[j], kt + j * 64);
      if constexpr (kVLds) {
#pragma unroll
        for (int j = 0; j < NK; ++j) load_lds16(vb + vdma[j], vt + j * 64);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) r.v[q] = load_bytes<VBYTES>(vb, voff[q]);
      }
    };

    float m = kMaxFloor;
    float l = 0.f;
    f32x4 acc[NJV];
#pragma unroll
    for (int j = 0; j < NJV; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // K operand chunks of the tile in LDS (and fp8 V's bytes)
    i32x4 kreg[NR];
    Bytes<VBYTES> vreg[4];
    auto fetch_tile = [&](const i32x4* kt, const i32x4* vt) {
#pragma unroll
      for (int rr = 0; rr < NR; ++rr) kreg[rr] = kt[kslot[rr]];
      if constexpr (kVLds) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          vreg[q] = *reinterpret_cast<const Bytes<VBYTES>*>(reinterpret_cast<const char*>(vt) + vrd[q]);
      }
    };

    auto compute_tile = [&](int i, Regs& r) {
      const int t0 = wk.t_lo + kTile * walk_tile(wk, i);
      // only a piece's last tile can reach past its end (wave-uniform)
      const bool partial = t0 + kTile > wk.t_hi;
      // scores: D[token 4g+q][head n]
      f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int rr = 0; rr < NR; ++rr) {
        const i32x4 kc = kreg[rr];
        if constexpr (kFP8) {
          const i32x2 c0 = kBF16 ? fp8x4_to_bf16x4((uint32_t)kc[0]) : fp8x4_to_f16x4((uint32_t)kc[0]);
          const i32x2 c1 = kBF16 ? fp8x4_to_bf16x4((uint32_t)kc[1]) : fp8x4_to_f16x4((uint32_t)kc[1]);
          const i32x2 c2 = kBF16 ? fp8x4_to_bf16x4((uint32_t)kc[2]) : fp8x4_to_f16x4((uint32_t)kc[2]);
          const i32x2 c3 = kBF16 ? fp8x4_to_bf16x4((uint32_t)kc[3]) : fp8x4_to_f16x4((uint32_t)kc[3]);
          s = mfma_k32<kBF16>(i32x4{c0[0], c0[1], c1[0], c1[1]}, qop[2 * rr], s);
          s = mfma_k32<kBF16>(i32x4{c2[0], c2[1], c3[0], c3[1]}, qop[2 * rr + 1], s);
        } else {
          s = mfma_k32<kBF16>(kc, qop[rr], s);
        }
      }
      float sv[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) sv[q] = s[q] * p.qk_scale_log2;
      if (partial) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (t0 + 4 * g + q >= wk.t_hi) sv[q] = -INFINITY;
      }
      // grouped work: each column's own length (wave-uniform test: only
      // the tiles that reach past the shortest row of the wave)
      if (kG && t0 + kTile > glmin) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (t0 + 4 * g + q >= glim) sv[q] = -INFINITY;
      }
      float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      // Lazy rescale: the weights are taken against a reference m that
      // moves (rescaling the sum and the output by 2^(m - m_new)) only when
      // some head's maximum passes it by more than 2^kLazyLog2, so the
      // weights stay below 2^kLazyLog2 and most tiles skip the rescale.
      // The result acc / l, and any merge of (m, l, acc) triples, is the
      // same for every choice of reference.
      const float m_new = fmaxf(m, mx);
      if (__builtin_amdgcn_ballot_w64(m_new > m + kLazyLog2) != 0) {
        const float alpha = fast_exp2(m - m_new);
#pragma unroll
        for (int j = 0; j < NJV; ++j) acc[j] = acc[j] * alpha;
        l *= alpha;
        m = m_new;
      }
      const float p0 = fast_exp2(sv[0] - m), p1 = fast_exp2(sv[1] - m);
      const float p2 = fast_exp2(sv[2] - m), p3 = fast_exp2(sv[3] - m);
      // P as the B operand of the P x V MFMAs.  fp16 (11-bit significand)
      // is precise enough on its own; bf16 (8 bits) would put errors of
      // 2^-9 |v| on outputs whose terms nearly cancel, so there P goes in
      // as hi + lo, two bf16 values whose sum carries 16 bits, and the
      // product runs twice.  The denominator sums the same rounded weights
      // the product uses.
      const uint32_t pw0 = kPVBF16 ? pack_bf16(p0, p1) : pack_f16(p0, p1);
      const uint32_t pw1 = kPVBF16 ? pack_bf16(p2, p3) : pack_f16(p2, p3);
      float ps;
      i32x2 pop_lo = {0, 0};
      if constexpr (kPVBF16) {
        const float h0 = bf16_lo(pw0), h1 = bf16_hi(pw0), h2 = bf16_lo(pw1), h3 = bf16_hi(pw1);
        const uint32_t lw0 = pack_bf16(p0 - h0, p1 - h1);
        const uint32_t lw1 = pack_bf16(p2 - h2, p3 - h3);
        ps = ((h0 + bf16_lo(lw0)) + (h1 + bf16_hi(lw0))) + ((h2 + bf16_lo(lw1)) + (h3 + bf16_hi(lw1)));
        pop_lo = i32x2{(int)lw0, (int)lw1};
      } else {
        ps = (f16_lo(pw0) + f16_hi(pw0)) + (f16_lo(pw1) + f16_hi(pw1));
      }
      l += ps;
      const i32x2 pop = {(int)pw0, (int)pw1};

      // V^T operand words of MFMA j: a0[j] = element j of tokens 4g, 4g+1,
      // a1[j] = of tokens 4g+2, 4g+3.  Tokens past the end of the sequence
      // may hold anything (NaN poison): on a partial tile their rows are
      // replaced by zeros before P x V.
      uint32_t rw[4][VBYTES / 4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int k = 0; k < VBYTES / 4; ++k) rw[q][k] = kVLds ? vreg[q].w(k) : r.v[q].w(k);
      if (partial) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const bool ok = t0 + 4 * g + q < wk.t_hi;
#pragma unroll
          for (int k = 0; k < VBYTES / 4; ++k) rw[q][k] = ok ? rw[q][k] : 0u;
        }
      }
      uint32_t a0[NJV], a1[NJV];
      if constexpr (kFP8) {
        // interleave the two tokens' fp8 bytes, then convert pairs: one
        // byte select and two conversions give four operand words
#pragma unroll
        for (int k = 0; k < VBYTES / 4; ++k) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const uint32_t sel = h ? 0x07030602u : 0x05010400u;
            const uint32_t x0 = __builtin_amdgcn_perm(rw[1][k], rw[0][k], sel);
            const uint32_t x1 = __builtin_amdgcn_perm(rw[3][k], rw[2][k], sel);
            const i32x2 c0 = fp8x4_to_f16x4(x0);
            const i32x2 c1 = fp8x4_to_f16x4(x1);
            a0[4 * k + 2 * h] = (uint32_t)c0[0];
            a0[4 * k + 2 * h + 1] = (uint32_t)c0[1];
            a1[4 * k + 2 * h] = (uint32_t)c1[0];
            a1[4 * k + 2 * h + 1] = (uint32_t)c1[1];
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < NJV; ++j) {
          const int k = j >> 1;
          a0[j] = (j & 1) ? pack_hi_halves(rw[0][k], rw[1][k]) : pack_lo_halves(rw[0][k], rw[1][k]);
          a1[j] = (j & 1) ? pack_hi_halves(rw[2][k], rw[3][k]) : pack_lo_halves(rw[2][k], rw[3][k]);
        }
      }
#pragma unroll
      for (int j = 0; j < NJV; ++j) {
        acc[j] = mfma_k16<kPVBF16>(i32x2{(int)a0[j], (int)a1[j]}, pop, acc[j]);
        if constexpr (kPVBF16) acc[j] = mfma_k16<kPVBF16>(i32x2{(int)a0[j], (int)a1[j]}, pop_lo, acc[j]);
      }
    };

    // two K tiles in LDS and two V register sets in ping-pong: the next
    // tile's loads are in flight while the current tile is computed
    {
      Regs r0, r1;
      run_tiles_lds(
          p, wk, ids, [&](int i) { load_tile(i, kt0[w], vt0[kVLds ? w : 0], r0); },
          [&](int i) { load_tile(i, kt1[w], vt1[kVLds ? w : 0], r1); },
          [&]() { fetch_tile(kt0[w], vt0[kVLds ? w : 0]); },
          [&]() { fetch_tile(kt1[w], vt1[kVLds ? w : 0]); }, [&](int i) { compute_tile(i, r0); },
          [&](int i) { compute_tile(i, r1); });
    }

    // lane groups hold partial sums over different tokens
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    int gb = 0, gh = 0;
    if constexpr (kG) {
      if (!gvalid) return;
      grp_row(gb, gh);
      slot = p.prefix_slot0 + gb * p.prefix_pieces + grp_piece;
    } else {
      if (n >= nh) return;
    }
    const int h = kG ? gh : head0 + n;
    // lane (n, g) holds out[h][(4g+i)*NJV + j] in acc[j][i]
    if (slot >= 0) {
      const int64_t ti = triple_index(p, slot, h);
      if (g == 0) {
        p.ws_ml[2 * ti] = m;
        p.ws_ml[2 * ti + 1] = l;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x[NJV];
#pragma unroll
        for (int j = 0; j < NJV; ++j) x[j] = acc[j][i];
        store_f32_vec<NJV>(p.ws_acc + ti * D + (4 * g + i) * NJV, x);
      }
    } else {
      const float sc = l > 0.f ? p.v_scale / l : 0.f;
      const int64_t ob = (int64_t)wk.b * p.o_sb + (int64_t)h * p.o_sh;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x[NJV];
#pragma unroll
        for (int j = 0; j < NJV; ++j) x[j] = acc[j][i] * sc;
        store_out_vec<QK, NJV>(p.out, ob + (4 * g + i) * NJV, x);
      }
    }
  };
  if (grp) {
    // piece grp_piece of grp_tokens tokens of the prefix (its blocks are
    // the one table row), up to the longest row of the wave
    if (!has_unit) return;
    Work wk;
    wk.row = p.prefix_blocks;
    wk.b = 0;
    wk.L = p.skip;
    wk.t_lo = grp_piece * p.grp_tokens;
    const int hi = min(min(p.skip, wk.t_lo + p.grp_tokens), glmax);
    wk.n_tiles = hi > wk.t_lo ? (hi - wk.t_lo + kTile - 1) / kTile : 0;
    wk.t_hi = wk.t_lo + wk.n_tiles * kTile;  // whole tiles: no token mask
    // the row groups of one kv head read the same tiles: each starts at
    // its own tile (the result does not depend on the order)
    wk.rot = wk.n_tiles > 0 ? (unit / p.Hkv) % wk.n_tiles : 0;
    piece(wk, 0, std::true_type{});
  } else {
    for_each_piece(p, s_pref, s_wtot, has_unit,
                   [&](const Work& wk, int slot) { piece(wk, slot, std::false_type{}); });
  }
}

// ============================================================================
// VALU inner loop: any supported dtype pair, GT query heads per wave.
// ============================================================================
template <int QK, int KVK, int D, int GT>
__global__ __launch_bounds__(kMaxThreads) void decode_valu_kernel(const DecodeParams p) {
  constexpr int ESZ = Esz<KVK>::v;
  constexpr int VEC = 16 / ESZ;      // KV elements per 16-byte load
  constexpr int LPT = D / VEC;       // lanes per token row
  constexpr int TPL = 64 / LPT;      // tokens per load instruction
  constexpr int NL = kTile / TPL;    // loads per tile (K and V each)
  constexpr bool kDot2 = KVK == K_F16 || KVK == K_BF16;
  constexpr int QE = VEC;            // query elements per lane
  static_assert(LPT >= 1 && LPT <= 64 && 64 % LPT == 0 && kTile % TPL == 0, "shape");
  static_assert(!kDot2 || QK == KVK, "16-bit KV needs a query of the same type");
  static_assert(VEC % 4 == 0, "shape");

  __shared__ int s_pref[kBalancedMaxBatch + 1];
  __shared__ int s_wtot[kMaxWaves];

  const int lane = threadIdx.x & 63;
  const int r = lane / LPT;          // token slot of this lane in a load
  const int c = lane - r * LPT;      // 16-byte chunk of the row
  const int unit = blockIdx.x * p.waves + (threadIdx.x >> 6);
  const bool has_unit = unit < p.units;
  const int kvh = unit / p.head_tiles;
  const int gh0 = (unit - kvh * p.head_tiles) * GT;
  const int nh = min(GT, p.G - gh0);
  const int head0 = kvh * p.G + gh0;

  const int64_t rs = (int64_t)p.Hkv * D * ESZ;
  const int64_t blk_bytes = rs * p.bs;
  const char* kbase = static_cast<const char*>(p.kc) + (int64_t)kvh * D * ESZ;
  const char* vbase = static_cast<const char*>(p.vc) + (int64_t)kvh * D * ESZ;
  uint32_t off[NL];
#pragma unroll
  for (int li = 0; li < NL; ++li) off[li] = (uint32_t)((li * TPL + r) * rs + c * 16);

  struct Regs {
    Bytes<16> k[NL];
    Bytes<16> v[NL];
  };

  for_each_piece(p, s_pref, s_wtot, has_unit, [&](const Work& wk, int slot) {
    // query chunk of each head: packed 16-bit words for v_dot2, else fp32
    // pre-multiplied by the score scale
    uint32_t qw[GT][kDot2 ? QE / 2 : 1];
    float qf[GT][kDot2 ? 1 : QE];
#pragma unroll
    for (int gh = 0; gh < GT; ++gh) {
      const int hq = head0 + min(gh, nh - 1);
      const int64_t qo = (int64_t)wk.b * p.q_sb + (int64_t)hq * p.q_sh + c * QE;
      if constexpr (kDot2) {
        const i32x4 v = *reinterpret_cast<const i32x4*>(static_cast<const uint16_t*>(p.q) + qo);
#pragma unroll
        for (int k = 0; k < 4; ++k) qw[gh][k] = (uint32_t)v[k];
      } else if constexpr (QK == K_F32) {
#pragma unroll
        for (int k = 0; k < QE; k += 4) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(static_cast<const float*>(p.q) + qo + k);
          qf[gh][k] = v[0] * p.qk_scale_log2;
          qf[gh][k + 1] = v[1] * p.qk_scale_log2;
          qf[gh][k + 2] = v[2] * p.qk_scale_log2;
          qf[gh][k + 3] = v[3] * p.qk_scale_log2;
        }
      } else {
#pragma unroll
        for (int k = 0; k < QE; k += 8) {
          const i32x4 v = *reinterpret_cast<const i32x4*>(static_cast<const uint16_t*>(p.q) + qo + k);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t wd = (uint32_t)v[e];
            const float lo = QK == K_BF16 ? bf16_lo(wd) : f16_lo(wd);
            const float hi = QK == K_BF16 ? bf16_hi(wd) : f16_hi(wd);
            qf[gh][k + 2 * e] = lo * p.qk_scale_log2;
            qf[gh][k + 2 * e + 1] = hi * p.qk_scale_log2;
          }
        }
      }
    }

    int ids = 0;
    auto load_tile = [&](int i, Regs& rg) {
      const int64_t tb = tile_base(p, wk, i, ids, blk_bytes, rs);
#pragma unroll
      for (int li = 0; li < NL; ++li) rg.k[li] = load_bytes<16>(kbase + tb, off[li]);
#pragma unroll
      for (int li = 0; li < NL; ++li) rg.v[li] = load_bytes<16>(vbase + tb, off[li]);
    };

    float m[GT], lsum[GT], acc[GT][VEC];
#pragma unroll
    for (int gh = 0; gh < GT; ++gh) {
      m[gh] = kMaxFloor;
      lsum[gh] = 0.f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) acc[gh][e] = 0.f;
    }

    auto compute_tile = [&](int i, Regs& rg) {
      const int t0 = wk.t_lo + kTile * i;
      // tokens past the end of the sequence may hold anything (NaN poison):
      // their scores become -inf and their V rows zeros, by selects (not
      // branches, so the loads still in flight are not waited for)
      bool valid[NL];
#pragma unroll
      for (int li = 0; li < NL; ++li) valid[li] = t0 + li * TPL + r < wk.t_hi;
      // scores (log2 units) of the NL tokens this row holds
      float sc[GT][NL];
#pragma unroll
      for (int li = 0; li < NL; ++li) {
#pragma unroll
        for (int gh = 0; gh < GT; ++gh) {
          float d = 0.f;
          if constexpr (KVK == K_F16) {
#pragma unroll
            for (int k = 0; k < 4; ++k)
              d = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, rg.k[li].w(k)),
                                         __builtin_bit_cast(f16x2, qw[gh][k]), d, false);
          } else if constexpr (KVK == K_BF16) {
#pragma unroll
            for (int k = 0; k < 4; ++k)
              d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, rg.k[li].w(k)),
                                                  __builtin_bit_cast(bf16x2, qw[gh][k]), d, false);
          } else if constexpr (KVK == K_F32) {
#pragma unroll
            for (int k = 0; k < 4; ++k) d += __builtin_bit_cast(float, rg.k[li].w(k)) * qf[gh][k];
          } else {  // fp8: 16 elements
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const f32x4 kv = fp8x4_to_f32x4(rg.k[li].w(k));
              d += kv[0] * qf[gh][4 * k] + kv[1] * qf[gh][4 * k + 1] +
                   kv[2] * qf[gh][4 * k + 2] + kv[3] * qf[gh][4 * k + 3];
            }
          }
          d = group_sum<LPT>(d);
          if constexpr (kDot2) d *= p.qk_scale_log2;
          sc[gh][li] = valid[li] ? d : -INFINITY;
        }
      }
      // V rows to fp32
      float vf[NL][VEC];
#pragma unroll
      for (int li = 0; li < NL; ++li) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t wd = valid[li] ? rg.v[li].w(k) : 0u;
          if constexpr (KVK == K_F32) {
            vf[li][k] = __builtin_bit_cast(float, wd);
          } else if constexpr (KVK == K_F16) {
            vf[li][2 * k] = f16_lo(wd);
            vf[li][2 * k + 1] = f16_hi(wd);
          } else if constexpr (KVK == K_BF16) {
            vf[li][2 * k] = bf16_lo(wd);
            vf[li][2 * k + 1] = bf16_hi(wd);
          } else {
            const f32x4 x = fp8x4_to_f32x4(wd);
            vf[li][4 * k] = x[0];
            vf[li][4 * k + 1] = x[1];
            vf[li][4 * k + 2] = x[2];
            vf[li][4 * k + 3] = x[3];
          }
        }
      }
#pragma unroll
      for (int gh = 0; gh < GT; ++gh) {
        float mx = sc[gh][0];
#pragma unroll
        for (int li = 1; li < NL; ++li) mx = fmaxf(mx, sc[gh][li]);
        const float m_new = fmaxf(m[gh], mx);
        const float alpha = fast_exp2(m[gh] - m_new);
        float pr[NL];
        float ps = 0.f;
#pragma unroll
        for (int li = 0; li < NL; ++li) {
          pr[li] = fast_exp2(sc[gh][li] - m_new);
          ps += pr[li];
        }
        lsum[gh] = lsum[gh] * alpha + ps;
        m[gh] = m_new;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          float a = acc[gh][e] * alpha;
#pragma unroll
          for (int li = 0; li < NL; ++li) a += pr[li] * vf[li][e];
          acc[gh][e] = a;
        }
      }
    };

    // two register sets in ping-pong: the next tile's loads are in flight
    // while the current tile is computed
    {
      Regs r0, r1;
      run_tiles(
          p, wk, ids, [&](int i) { load_tile(i, r0); }, [&](int i) { load_tile(i, r1); },
          [&](int i) { compute_tile(i, r0); }, [&](int i) { compute_tile(i, r1); });
    }

    // rows of the wave hold disjoint tokens: merge their states (lanes with
    // the same chunk c sit LPT, 2*LPT, ... lanes apart)
#pragma unroll
    for (int step = LPT; step < 64; step <<= 1) {
#pragma unroll
      for (int gh = 0; gh < GT; ++gh) {
        const float mo = __shfl_xor(m[gh], step);
        const float lo = __shfl_xor(lsum[gh], step);
        const float mm = fmaxf(m[gh], mo);
        const float s1 = fast_exp2(m[gh] - mm);
        const float s2 = fast_exp2(mo - mm);
        lsum[gh] = lsum[gh] * s1 + lo * s2;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const float ao = __shfl_xor(acc[gh][e], step);
          acc[gh][e] = acc[gh][e] * s1 + ao * s2;
        }
        m[gh] = mm;
      }
    }
    if (r != 0) return;
#pragma unroll
    for (int gh = 0; gh < GT; ++gh) {
      if (gh >= nh) break;
      const int h = head0 + gh;
      if (slot >= 0) {
        const int64_t ti = triple_index(p, slot, h);
        if (c == 0) {
          p.ws_ml[2 * ti] = m[gh];
          p.ws_ml[2 * ti + 1] = lsum[gh];
        }
        store_f32_vec<VEC>(p.ws_acc + ti * D + c * VEC, acc[gh]);
      } else {
        const float sc = lsum[gh] > 0.f ? p.v_scale / lsum[gh] : 0.f;
        float x[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) x[e] = acc[gh][e] * sc;
        store_out_vec<QK, VEC>(p.out, (int64_t)wk.b * p.o_sb + (int64_t)h * p.o_sh + c * VEC, x);
      }
    }
  });
}

// ============================================================================
// Piece merge: out = sum_p acc_p 2^(m_p - M) / sum_p l_p 2^(m_p - M) with
// M = max_p m_p.  A 256-thread workgroup takes R (query head, sequence)
// rows, consecutive heads of one sequence; each row gets GROUPS groups of
// D/4 threads (4 dims each, 16-byte loads) that fold every GROUPS-th piece
// into a running (max, sum, output), loads of up to four pieces in flight at
// once; then a row's group states are combined in group order (a fixed
// order: the result does not depend on timing).  Plans with many pieces per
// row take R = 1 (eight groups folding side by side), plans with few take
// more rows per workgroup, so that the launch is not thousands of
// workgroups that each wait on one dependent load.  The piece plan comes
// from the decode kernel (balanced schedule: per-sequence first slot and
// piece count, 0 pieces for an empty sequence, whose zero row is written
// here) or from the partition size (fixed schedule).
// ============================================================================
constexpr int kMergeThreads = 256;

template <int QK, int D, int R>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(const DecodeParams p) {
  constexpr int TPR = D / 4;                        // threads per piece row
  constexpr int GROUPS = kMergeThreads / (TPR * R);  // pieces folded side by side per row
  constexpr int U = 4;                              // pieces in flight per group
  static_assert(GROUPS >= 1, "rows per workgroup");
  __shared__ f32x4 s_num[R][GROUPS][TPR];
  __shared__ float s_m[R][GROUPS], s_den[R][GROUPS];

  const int tid = threadIdx.x;
  const int rr = tid / (GROUPS * TPR);  // row of the workgroup
  const int t2 = tid - rr * GROUPS * TPR;
  const int grp = t2 / TPR;
  const int c = t2 - grp * TPR;
  const int row = blockIdx.x * R + rr;
  const bool live = row < p.B * p.Hq;
  const int b = live ? row / p.Hq : 0;
  const int h = live ? row - b * p.Hq : 0;
  const int64_t ob = (int64_t)b * p.o_sb + (int64_t)h * p.o_sh;
  int slot0 = 0, PS = 0, P = 0;  // PS pieces of this pass at slots slot0 .., P in all
  bool direct = !live;           // nothing to merge for this row
  if (live) {
    if (p.sched == kSchedBalanced) {
      slot0 = p.ws_meta[2 * b];
      PS = p.ws_meta[2 * b + 1];
      P = PS + p.prefix_pieces;
      if (P == 0) {
        if (grp == 0) {
          const float z[4] = {0.f, 0.f, 0.f, 0.f};
          store_out_vec<QK, 4>(p.out, ob + 4 * c, z);
        }
        direct = true;
      }
      if (P == 1 && p.prefix_pieces == 0) direct = true;  // single piece: written directly
    } else {
      const int L = clamp_len(p, b);
      if (L <= p.part_tokens) {
        direct = true;  // single partition: written directly
      } else {
        slot0 = b * p.num_parts;
        P = PS = (L + p.part_tokens - 1) / p.part_tokens;
      }
    }
  }
  if (direct) P = 0;
  // triple index of piece q: this pass's pieces, then the prefix pass's
  auto piece_index = [&](int q) -> int64_t {
    const int slot = q < PS ? slot0 + q : p.prefix_slot0 + b * p.prefix_pieces + (q - PS);
    return triple_index(p, slot, h);
  };

  float M = kMaxFloor, den = 0.f;
  f32x4 num = {0.f, 0.f, 0.f, 0.f};
  for (int q0 = grp; q0 < P; q0 += U * GROUPS) {
    float mq[U], lq[U];
    f32x4 aq[U];
    // unconditional loads (a piece past the end reloads the last one and is
    // masked afterwards), so all of them are in flight together
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int q = min(q0 + u * GROUPS, P - 1);
      const int64_t ti = piece_index(q);
      mq[u] = p.ws_ml[2 * ti];
      lq[u] = p.ws_ml[2 * ti + 1];
      aq[u] = *reinterpret_cast<const f32x4*>(p.ws_acc + ti * D + 4 * c);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (q0 + u * GROUPS >= P) {
        mq[u] = kMaxFloor;
        lq[u] = 0.f;
        aq[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float mn = fmaxf(M, mq[u]);
      const float s_old = fast_exp2(M - mn), s_new = fast_exp2(mq[u] - mn);
      den = den * s_old + lq[u] * s_new;
      num = num * s_old + aq[u] * s_new;
      M = mn;
    }
  }
  if constexpr (GROUPS == 1) {
    if (direct) return;
    const float sc = den > 0.f ? p.v_scale / den : 0.f;
    const float x[4] = {num[0] * sc, num[1] * sc, num[2] * sc, num[3] * sc};
    store_out_vec<QK, 4>(p.out, ob + 4 * c, x);
  } else {
    s_num[rr][grp][c] = num;
    if (c == 0) {
      s_m[rr][grp] = M;
      s_den[rr][grp] = den;
    }
    __syncthreads();
    if (direct || grp != 0) return;
    float Mt = s_m[rr][0];
#pragma unroll
    for (int k = 1; k < GROUPS; ++k) Mt = fmaxf(Mt, s_m[rr][k]);
    f32x4 tot = {0.f, 0.f, 0.f, 0.f};
    float dtot = 0.f;
#pragma unroll
    for (int k = 0; k < GROUPS; ++k) {
      const float sc = fast_exp2(s_m[rr][k] - Mt);
      tot += s_num[rr][k][c] * sc;
      dtot += s_den[rr][k] * sc;
    }
    const float sc = dtot > 0.f ? p.v_scale / dtot : 0.f;
    const float x[4] = {tot[0] * sc, tot[1] * sc, tot[2] * sc, tot[3] * sc};
    store_out_vec<QK, 4>(p.out, ob + 4 * c, x);
  }
}

// Rows per merge workgroup from the expected pieces per row: the balanced
// plan deals nwc shares of each unit chunk over the batch (about nwc / B + 1
// pieces per sequence, plus the prefix pass's), the fixed plan splits long
// sequences into num_parts.
template <int QK, int D>
hipError_t launch_merge(const DecodeParams& p, hipStream_t stream) {
  const int pieces = p.sched == kSchedBalanced
                         ? p.nwc / max(p.B, 1) + 1 + p.prefix_pieces
                         : p.num_parts;
  const int rows = p.B * p.Hq;
  auto go = [&](auto rtag) {
    constexpr int R = decltype(rtag)::value;
    hipLaunchKernelGGL((merge_kernel<QK, D, R>), dim3((rows + R - 1) / R), dim3(kMergeThreads), 0, stream, p);
    return hipGetLastError();
  };
  if (pieces > 16) return go(std::integral_constant<int, 1>{});
  if (pieces > 8) return go(std::integral_constant<int, 2>{});
  if (pieces > 4) return go(std::integral_constant<int, 4>{});
  return go(std::integral_constant<int, 8>{});
}

template <int QK, int KVK, int D>
hipError_t launch_valu(const DecodeParams& p, int gt, dim3 grid, dim3 block, hipStream_t stream) {
  switch (gt) {
    case 1: hipLaunchKernelGGL((decode_valu_kernel<QK, KVK, D, 1>), grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL((decode_valu_kernel<QK, KVK, D, 2>), grid, block, 0, stream, p); break;
    case 4: hipLaunchKernelGGL((decode_valu_kernel<QK, KVK, D, 4>), grid, block, 0, stream, p); break;
    default: return hipErrorNotSupported;
  }
  return hipGetLastError();
}

template <int QK, int KVK, int D>
hipError_t launch_all(const DecodeParams& p, const DecodeVariant& v, hipStream_t stream) {
  int max_waves, workgroups;
  decode_launch_shape(v, &max_waves, &workgroups);
  if (p.waves < 1 || p.waves > max_waves) return hipErrorInvalidValue;
  if (p.sched == kSchedBalanced && (p.B > kBalancedMaxBatch || p.nwc < 1 || p.nwc > kBalancedSlots))
    return hipErrorInvalidValue;
  if (p.grp_units > 0) {
    // grouped prefix work: matrix-core kernel, balanced schedule, and
    // enough workgroups for every (unit, piece)
    const int64_t grp_waves = (int64_t)p.grp_units * p.prefix_pieces;
    const int64_t chunks = (p.units + p.waves - 1) / p.waves;
    if (v.path != 2 || p.sched != kSchedBalanced || !p.prefix_blocks || p.grp_tokens < 16 ||
        p.grp_tokens % 16 || p.prefix_pieces < 1 || p.grp_y < 1 ||
        (int64_t)p.grp_y * chunks * p.waves < grp_waves || p.nwc + p.grp_y > 65535)
      return hipErrorInvalidValue;
  }
  const int chunks = (p.units + p.waves - 1) / p.waves;
  const dim3 grid = p.sched == kSchedBalanced ? dim3(chunks, p.nwc + p.grp_y, 1)
                                              : dim3(chunks, p.num_parts, p.B);
  const dim3 block(p.waves * 64);
  hipError_t e;
  if (v.path == 2) {
    if constexpr (QK == K_F32 || KVK == K_F32) {
      return hipErrorNotSupported;
    } else {
      hipLaunchKernelGGL((decode_mfma_kernel<QK, KVK, D>), grid, block, 0, stream, p);
      e = hipGetLastError();
    }
  } else {
    e = launch_valu<QK, KVK, D>(p, v.gt, grid, block, stream);
  }
  if (e != hipSuccess) return e;
  if (p.split) return launch_merge<QK, D>(p, stream);
  return hipSuccess;
}

template <int QK, int KVK>
hipError_t launch_d(const DecodeParams& p, const DecodeVariant& v, hipStream_t stream) {
  switch (v.D) {
    case 64: return launch_all<QK, KVK, 64>(p, v, stream);
    case 128: return launch_all<QK, KVK, 128>(p, v, stream);
    default: return hipErrorNotSupported;
  }
}

}  // namespace

bool decode_variant_built(const DecodeVariant& v) {
  if (v.D != 64 && v.D != 128) return false;
  const bool pair_ok = (v.qkind == v.kvkind && v.qkind >= K_F32 && v.qkind <= K_BF16) ||
                       (v.kvkind == K_FP8 && (v.qkind == K_F16 || v.qkind == K_BF16));
  if (!pair_ok) return false;
  if (v.path == 2) return v.qkind != K_F32 && v.gt == 16;
  if (v.path == 1) return v.gt == 1 || v.gt == 2 || v.gt == 4;
  return false;
}

void decode_launch_shape(const DecodeVariant& v, int* max_waves, int* workgroups) {
  const bool fp8_mfma = v.path == 2 && v.kvkind == K_FP8;
  *max_waves = fp8_mfma ? kFp8Waves : kMaxWaves;
  *workgroups = fp8_mfma ? kBalancedWorkgroupsFp8 : kBalancedWorkgroups;
}

namespace {
constexpr int kScratchMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchMaxDevices] = {};
}  // namespace

hipError_t decode_scratch(hipStream_t stream, void** ptr) {
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    // first use on this device: its address, with that device current
    int cur = -1;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_decode(const DecodeParams& p, const DecodeVariant& v, hipStream_t stream) {
  if (!decode_variant_built(v)) return hipErrorNotSupported;
  if (v.qkind == K_F32 && v.kvkind == K_F32) return launch_d<K_F32, K_F32>(p, v, stream);
  if (v.qkind == K_F16 && v.kvkind == K_F16) return launch_d<K_F16, K_F16>(p, v, stream);
  if (v.qkind == K_BF16 && v.kvkind == K_BF16) return launch_d<K_BF16, K_BF16>(p, v, stream);
  if (v.qkind == K_F16 && v.kvkind == K_FP8) return launch_d<K_F16, K_FP8>(p, v, stream);
  if (v.qkind == K_BF16 && v.kvkind == K_FP8) return launch_d<K_BF16, K_FP8>(p, v, stream);
  return hipErrorNotSupported;
}

}  // namespace pa
