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
// its group); one wave owns one unit over one partition of one sequence and
// walks every 16-token tile of that partition itself, so its softmax state
// never has to be merged with another wave's.  A workgroup is up to eight
// consecutive units of the same (sequence, partition): its waves read the
// same physical blocks at the same time, so each block's K (and V) rows of
// neighbouring heads, which are adjacent in memory, are fetched together.
// On MI355X that keeps the DRAM access stream close to a sequential one
// (6.9 TB/s for the bare gather, against 5.7 TB/s when each workgroup walks
// one head on its own).  With a split, each partition leaves a
// (max, sum, unnormalised output) triple in the workspace and merge_kernel
// combines them in a fixed order (no atomics, so results are
// bit-reproducible).
//
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
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kTile = 16;
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
  return L < 0 ? 0 : (L > cap ? cap : L);
}

// What one wave works on: its unit, sequence, partition and token range.
struct Work {
  int kvh, htile, b, part, L, t_lo, t_hi, n_tiles;
};

// false when the wave has nothing to do (unit past the end, or a partition
// that starts beyond the sequence: its triple is never read).
__device__ __forceinline__ bool wave_work(const DecodeParams& p, Work& wk) {
  const int unit = blockIdx.x * p.waves + (threadIdx.x >> 6);
  if (unit >= p.units) return false;
  wk.kvh = unit / p.head_tiles;
  wk.htile = unit - wk.kvh * p.head_tiles;
  wk.b = blockIdx.z;
  wk.part = blockIdx.y;
  wk.L = clamp_len(p, wk.b);
  wk.t_lo = wk.part * p.part_tokens;
  if (wk.part > 0 && wk.t_lo >= wk.L) return false;
  wk.t_hi = min(wk.L, wk.t_lo + p.part_tokens);
  wk.n_tiles = wk.t_hi > wk.t_lo ? (wk.t_hi - wk.t_lo + kTile - 1) / kTile : 0;
  return true;
}

// Physical block ids of tiles chunk*64 .. chunk*64+63 of the wave's range:
// lane j holds the id of tile chunk*64 + j.
__device__ __forceinline__ int load_block_ids(const DecodeParams& p, const Work& wk, int chunk) {
  const int lane = threadIdx.x & 63;
  const int i = chunk * 64 + lane;
  int id = 0;
  if (i < wk.n_tiles) {
    const int t = wk.t_lo + kTile * i;
    id = p.tables[(int64_t)wk.b * p.tab_stride + t / p.bs];
    // an id outside the pool is a caller error; read block 0 instead of
    // faulting
    if ((unsigned)id >= (unsigned)p.num_blocks) id = 0;
  }
  return id;
}

// Byte offset of tile i inside the pool (block base + row offset in block);
// `ids` holds the block ids of tiles (i & ~63) .. (i | 63).
__device__ __forceinline__ int64_t tile_base(const DecodeParams& p, const Work& wk, int i,
                                             int ids, int64_t blk_bytes, int64_t rs) {
  const int blk = __builtin_amdgcn_readlane(ids, i & 63);
  const int t0 = wk.t_lo + kTile * i;
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

// Triple slot of (sequence, query head, partition).
__device__ __forceinline__ int64_t triple_index(const DecodeParams& p, int b, int h, int part) {
  return ((int64_t)b * p.Hq + h) * p.num_parts + part;
}

// ============================================================================
// MFMA inner loop: 16-bit query, 16-bit or fp8 KV, head_dim 64 or 128, a tile
// of up to 16 query heads of one kv group.
// ============================================================================
template <int QK, int KVK, int D>
__global__ __launch_bounds__(kMaxThreads) void decode_mfma_kernel(const DecodeParams p) {
  constexpr bool kBF16 = QK == K_BF16;
  constexpr bool kFP8 = KVK == K_FP8;
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
  constexpr int VW = NJV / 2;          // V words per token after conversion to 16-bit
  constexpr int SLOTS = kTile * LR;    // 16-byte LDS slots per tile
  static_assert(NK >= 1 && NR >= 1 && (kFP8 ? 2 * NR == NJQ : NR == NJQ), "shape");
  static_assert(VBYTES == 16 || VBYTES == 8 || VBYTES == 4, "shape");

  // two K tiles per wave, in two arrays so the compiler can tell the
  // in-flight tile's LDS writes from the current tile's reads
  __shared__ i32x4 kt0[kMaxWaves][SLOTS];
  __shared__ i32x4 kt1[kMaxWaves][SLOTS];

  Work wk;
  if (!wave_work(p, wk)) return;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int n = lane & 15;
  const int g = lane >> 4;
  const int gh0 = wk.htile * 16;
  const int nh = min(16, p.G - gh0);
  const int head0 = wk.kvh * p.G + gh0;

  // Query group as the B operand of the score MFMAs: lane (n, g) holds head
  // n, 8 dims per MFMA: those of 16-byte K chunk 4r + g (16-bit K: MFMA r;
  // fp8 K: the low / high half of that chunk for MFMAs 2r, 2r + 1).
  i32x4 qop[NJQ];
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(p.q) + (int64_t)wk.b * p.q_sb +
                           (int64_t)(head0 + min(n, nh - 1)) * p.q_sh;
#pragma unroll
    for (int j = 0; j < NJQ; ++j) {
      const int d0 = kFP8 ? ((j >> 1) * 64 + g * 16 + (j & 1) * 8) : (j * 32 + g * 8);
      const i32x4 v = *reinterpret_cast<const i32x4*>(qrow + d0);
      qop[j] = n < nh ? v : i32x4{0, 0, 0, 0};
    }
  }

  const int64_t rs = (int64_t)p.Hkv * RB;  // bytes between tokens
  const int64_t blk_bytes = rs * p.bs;
  const char* kbase = static_cast<const char*>(p.kc) + (int64_t)wk.kvh * RB;
  const char* vbase = static_cast<const char*>(p.vc) + (int64_t)wk.kvh * RB;
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

  struct Regs {
    Bytes<VBYTES> v[4];
  };

  int ids = 0;
  auto load_tile = [&](int i, i32x4* kt, Regs& r) {
    const int64_t tb = tile_base(p, wk, i, ids, blk_bytes, rs);
    const char* kb = kbase + tb;
    const char* vb = vbase + tb;
#pragma unroll
    for (int j = 0; j < NK; ++j)
      load_lds16(kb + kdma[j], kt + j * 64);
#pragma unroll
    for (int q = 0; q < 4; ++q) r.v[q] = load_bytes<VBYTES>(vb, voff[q]);
  };

  float m = kMaxFloor;
  float l = 0.f;
  f32x4 acc[NJV];
#pragma unroll
  for (int j = 0; j < NJV; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // K operand chunks of the tile in LDS
  i32x4 kreg[NR];
  auto fetch_tile = [&](const i32x4* kt) {
#pragma unroll
    for (int rr = 0; rr < NR; ++rr) kreg[rr] = kt[kslot[rr]];
  };

  auto compute_tile = [&](int i, Regs& r) {
    const int t0 = wk.t_lo + kTile * i;
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
    for (int q = 0; q < 4; ++q)
      sv[q] = (t0 + 4 * g + q < wk.t_hi) ? s[q] * p.qk_scale_log2 : -INFINITY;
    float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m, mx);
    const float alpha = fast_exp2(m - m_new);
    const float p0 = fast_exp2(sv[0] - m_new), p1 = fast_exp2(sv[1] - m_new);
    const float p2 = fast_exp2(sv[2] - m_new), p3 = fast_exp2(sv[3] - m_new);
    const uint32_t pw0 = kBF16 ? pack_bf16(p0, p1) : pack_f16(p0, p1);
    const uint32_t pw1 = kBF16 ? pack_bf16(p2, p3) : pack_f16(p2, p3);
    // the denominator sums the same rounded weights the product uses
    const float ps = kBF16 ? (bf16_lo(pw0) + bf16_hi(pw0)) + (bf16_lo(pw1) + bf16_hi(pw1))
                           : (f16_lo(pw0) + f16_hi(pw0)) + (f16_lo(pw1) + f16_hi(pw1));
    l = l * alpha + ps;
    m = m_new;
    const i32x2 pop = {(int)pw0, (int)pw1};

    // V rows as 16-bit words: vw[q][k] holds elements 2k, 2k+1 of token 4g+q.
    // Tokens past the end of the sequence may hold anything (NaN poison):
    // their rows are replaced by zeros (a select, not a branch, so the loads
    // still in flight are not waited for) before the P x V product.
    uint32_t vw[4][VW];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const bool ok = t0 + 4 * g + q < wk.t_hi;
      if constexpr (kFP8) {
#pragma unroll
        for (int k = 0; k < VW / 2; ++k) {
          const i32x2 c2 = kBF16 ? fp8x4_to_bf16x4(r.v[q].w(k)) : fp8x4_to_f16x4(r.v[q].w(k));
          vw[q][2 * k] = ok ? (uint32_t)c2[0] : 0u;
          vw[q][2 * k + 1] = ok ? (uint32_t)c2[1] : 0u;
        }
      } else {
#pragma unroll
        for (int k = 0; k < VW; ++k) vw[q][k] = ok ? r.v[q].w(k) : 0u;
      }
    }
#pragma unroll
    for (int j = 0; j < NJV; ++j) {
      const int k = j >> 1;
      uint32_t a0, a1;
      if (j & 1) {
        a0 = pack_hi_halves(vw[0][k], vw[1][k]);
        a1 = pack_hi_halves(vw[2][k], vw[3][k]);
      } else {
        a0 = pack_lo_halves(vw[0][k], vw[1][k]);
        a1 = pack_lo_halves(vw[2][k], vw[3][k]);
      }
      acc[j] = acc[j] * alpha;
      acc[j] = mfma_k16<kBF16>(i32x2{(int)a0, (int)a1}, pop, acc[j]);
    }
  };

  // two K tiles in LDS and two V register sets in ping-pong: the next
  // tile's loads are in flight while the current tile is computed
  {
    Regs r0, r1;
    run_tiles_lds(
        p, wk, ids, [&](int i) { load_tile(i, kt0[w], r0); },
        [&](int i) { load_tile(i, kt1[w], r1); }, [&]() { fetch_tile(kt0[w]); },
        [&]() { fetch_tile(kt1[w]); }, [&](int i) { compute_tile(i, r0); },
        [&](int i) { compute_tile(i, r1); });
  }

  // lane groups hold partial sums over different tokens
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (n >= nh) return;
  const int h = head0 + n;
  // lane (n, g) holds out[h][(4g+i)*NJV + j] in acc[j][i]
  const bool triple = p.split && wk.L > p.part_tokens;
  if (triple) {
    const int64_t ti = triple_index(p, wk.b, h, wk.part);
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

  Work wk;
  if (!wave_work(p, wk)) return;
  const int lane = threadIdx.x & 63;
  const int r = lane / LPT;          // token slot of this lane in a load
  const int c = lane - r * LPT;      // 16-byte chunk of the row
  const int gh0 = wk.htile * GT;
  const int nh = min(GT, p.G - gh0);
  const int head0 = wk.kvh * p.G + gh0;

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

  const int64_t rs = (int64_t)p.Hkv * D * ESZ;
  const int64_t blk_bytes = rs * p.bs;
  const char* kbase = static_cast<const char*>(p.kc) + (int64_t)wk.kvh * D * ESZ;
  const char* vbase = static_cast<const char*>(p.vc) + (int64_t)wk.kvh * D * ESZ;
  uint32_t off[NL];
#pragma unroll
  for (int li = 0; li < NL; ++li) off[li] = (uint32_t)((li * TPL + r) * rs + c * 16);

  struct Regs {
    Bytes<16> k[NL];
    Bytes<16> v[NL];
  };
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

  // rows of the wave hold disjoint tokens: merge their states (lanes with the
  // same chunk c sit LPT, 2*LPT, ... lanes apart)
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
  const bool triple = p.split && wk.L > p.part_tokens;
#pragma unroll
  for (int gh = 0; gh < GT; ++gh) {
    if (gh >= nh) break;
    const int h = head0 + gh;
    if (triple) {
      const int64_t ti = triple_index(p, wk.b, h, wk.part);
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
}

// ============================================================================
// Partition merge: out = sum_p acc_p 2^(m_p - M) / sum_p l_p 2^(m_p - M),
// partitions in increasing order.
// ============================================================================
template <int QK, int D>
__global__ __launch_bounds__(D) void merge_kernel(const DecodeParams p) {
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int d = threadIdx.x;
  const int L = clamp_len(p, b);
  if (L <= p.part_tokens) return;  // single partition: written directly
  const int P = (L + p.part_tokens - 1) / p.part_tokens;
  const int64_t base = triple_index(p, b, h, 0);
  const float* ml = p.ws_ml + 2 * base;
  const float* acc = p.ws_acc + base * D + d;
  float M = kMaxFloor;
  for (int q = 0; q < P; ++q) M = fmaxf(M, ml[2 * q]);
  float num = 0.f, den = 0.f;
  for (int q = 0; q < P; ++q) {
    const float sc = fast_exp2(ml[2 * q] - M);
    den += ml[2 * q + 1] * sc;
    num += acc[(int64_t)q * D] * sc;
  }
  const float o = den > 0.f ? num / den * p.v_scale : 0.f;
  store_out<QK>(p.out, (int64_t)b * p.o_sb + (int64_t)h * p.o_sh + d, o);
}

template <int QK, int D>
hipError_t launch_merge(const DecodeParams& p, hipStream_t stream) {
  hipLaunchKernelGGL((merge_kernel<QK, D>), dim3(p.Hq, p.B), dim3(D), 0, stream, p);
  return hipGetLastError();
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
  if (p.waves < 1 || p.waves > kMaxWaves) return hipErrorInvalidValue;
  const dim3 grid((p.units + p.waves - 1) / p.waves, p.num_parts, p.B);
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

int decode_max_waves() { return kMaxWaves; }

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
