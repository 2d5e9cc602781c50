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
// Work decomposition: one workgroup (4 waves) per (sequence, kv head, head
// tile, partition).  A partition is `part_tokens` consecutive tokens; the
// waves of a workgroup take its 16-token tiles round-robin, each keeping its
// own softmax state, and the states are merged through LDS.  With a split,
// each partition leaves a (max, sum, unnormalised output) triple in the
// workspace and merge_kernel combines them in a fixed order (no atomics, so
// results are bit-reproducible).
//
// Two inner loops:
//  * VALU (small groups): lanes of a row of LPT lanes cover one token's
//    head_dim with 16-byte loads; q.k partial dot products (v_dot2 for 16-bit
//    data) are summed across the row with DPP; every row keeps its own
//    online-softmax state.
//  * MFMA (groups >= 4): scores = K-tile[16 x D] x Q-group^T[D x 16] on
//    v_mfma_f32_16x16x32, then out^T += V^T[D x 16] x P^T[16 x 16] on
//    v_mfma_f32_16x16x16.  The score tile comes out with lane l holding
//    tokens 4*(l/16)+i of head l%16, which is exactly the layout of the P
//    operand; V is loaded with one 16-byte (or 8-byte) row chunk per lane and
//    per token, and the output dims are permuted instead of transposing V
//    (MFMA j, row m computes dim m * (D/16) + j).  No LDS on the hot loop.
//
// Block ids are prefetched 64 tiles at a time into one VGPR per wave and
// read with v_readlane, so every K/V load is a scalar 64-bit block base plus
// a 32-bit per-lane offset; the next tile's loads are issued before the
// current tile is computed.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kTile = 16;
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kPad = 4;  // LDS row padding (floats)

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

// Sequence length clamped to what the block table can address (a longer
// length is a caller error; clamping keeps every read inside the table).
__device__ __forceinline__ int clamp_len(const DecodeParams& p, int b) {
  const int L = p.lens[b];
  const int cap = p.max_blocks * p.bs;
  return L < 0 ? 0 : (L > cap ? cap : L);
}

// Physical block id of this wave's i-th tile (tiles w, w+4, w+8, ... of the
// partition), 64 tiles per chunk.  Lane j of the chunk holds tile c*64+j.
__device__ __forceinline__ int load_block_ids(const DecodeParams& p, int b, int t_lo,
                                              int w, int chunk, int n_my) {
  const int lane = threadIdx.x & 63;
  const int i = chunk * 64 + lane;
  int id = 0;
  if (i < n_my) {
    const int t = t_lo + kTile * (w + kWaves * i);
    id = p.tables[(int64_t)b * p.tab_stride + t / p.bs];
    // an id outside the pool is a caller error; read block 0 instead of
    // faulting
    if ((unsigned)id >= (unsigned)p.num_blocks) id = 0;
  }
  return id;
}

// Merge S softmax states per head from LDS and write the output row (or the
// partition triple when the sequence spans several partitions).
template <int QK, int D, int GT, int S>
__device__ __forceinline__ void combine_and_store(const DecodeParams& p,
                                                  const float (*ml)[GT][2],
                                                  const float (*acc)[GT][D + kPad],
                                                  int b, int part, int head0, int nh,
                                                  int L) {
  const bool triple = p.split && L > p.part_tokens;
  for (int idx = threadIdx.x; idx < GT * D; idx += kThreads) {
    const int hh = idx / D;
    const int d = idx - hh * D;
    if (hh >= nh) continue;
    float M = kMaxFloor;
#pragma unroll
    for (int s = 0; s < S; ++s) M = fmaxf(M, ml[s][hh][0]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const float sc = fast_exp2(ml[s][hh][0] - M);
      den += ml[s][hh][1] * sc;
      num += acc[s][hh][d] * sc;
    }
    const int h = head0 + hh;
    if (triple) {
      const int64_t base = ((int64_t)b * p.Hq + h) * p.num_parts + part;
      p.ws_acc[base * D + d] = num;
      if (d == 0) {
        p.ws_ml[2 * base] = M;
        p.ws_ml[2 * base + 1] = den;
      }
    } else {
      const float o = den > 0.f ? num / den * p.v_scale : 0.f;
      store_out<QK>(p.out, (int64_t)b * p.o_sb + (int64_t)h * p.o_sh + d, o);
    }
  }
}

// ============================================================================
// MFMA inner loop: 16-bit query, 16-bit or fp8 KV, head_dim 64 or 128, a tile
// of up to 16 query heads of one kv group.
// ============================================================================
template <int QK, int KVK, int D>
__global__ __launch_bounds__(kThreads) void decode_mfma_kernel(const DecodeParams p) {
  constexpr bool kBF16 = QK == K_BF16;
  constexpr bool kFP8 = KVK == K_FP8;
  constexpr int ESZ = kFP8 ? 1 : 2;
  constexpr int NJQ = D / 32;             // score MFMAs per tile (K = 32 dims each)
  constexpr int NJV = D / 16;             // P x V MFMAs per tile; V elements per lane per token
  constexpr int KLOADS = D * ESZ / 64;    // 16-byte K loads per lane per tile
  constexpr int VBYTES = NJV * ESZ;       // V bytes per lane per token
  constexpr int VW = NJV / 2;             // V words per token after conversion to 16-bit
  static_assert(KLOADS >= 1 && (VBYTES == 16 || VBYTES == 8 || VBYTES == 4), "shape");

  __shared__ float sm_ml[kWaves][16][2];
  __shared__ float sm_acc[kWaves][16][D + kPad];

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int n = lane & 15;
  const int g = lane >> 4;
  const int b = blockIdx.z;
  const int part = blockIdx.y;
  const int kvh = blockIdx.x / p.head_tiles;
  const int htile = blockIdx.x - kvh * p.head_tiles;
  const int L = clamp_len(p, b);
  const int t_lo = part * p.part_tokens;
  if (part > 0 && t_lo >= L) return;  // whole workgroup: nothing in this partition
  const int t_hi = min(L, t_lo + p.part_tokens);
  const int n_tiles = t_hi > t_lo ? (t_hi - t_lo + kTile - 1) / kTile : 0;
  const int n_my = n_tiles > w ? (n_tiles - w + kWaves - 1) / kWaves : 0;
  const int gh0 = htile * 16;
  const int nh = min(16, p.G - gh0);
  const int head0 = kvh * p.G + gh0;

  // Query group as the B operand of the score MFMAs: lane (n, g) holds head n,
  // 8 dims per MFMA.  The dims a lane contributes must match the K operand.
  i32x4 qop[NJQ];
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(p.q) + (int64_t)b * p.q_sb +
                           (int64_t)(head0 + min(n, nh - 1)) * p.q_sh;
#pragma unroll
    for (int j = 0; j < NJQ; ++j) {
      const int d0 = kFP8 ? ((j >> 1) * 64 + g * 16 + (j & 1) * 8) : (j * 32 + g * 8);
      const i32x4 v = *reinterpret_cast<const i32x4*>(qrow + d0);
      qop[j] = n < nh ? v : i32x4{0, 0, 0, 0};
    }
  }

  const int64_t rs = (int64_t)p.Hkv * D * ESZ;  // bytes between tokens
  const int64_t blk_bytes = rs * p.bs;
  const char* kbase = static_cast<const char*>(p.kc) + (int64_t)kvh * D * ESZ;
  const char* vbase = static_cast<const char*>(p.vc) + (int64_t)kvh * D * ESZ;
  // K: lane (token n, group g) reads 16 bytes at jl*64 + g*16 of its token row.
  // V: lane (dim chunk n, group g) reads VBYTES at n*VBYTES of tokens 4g+i.
  uint32_t koff[KLOADS];
#pragma unroll
  for (int jl = 0; jl < KLOADS; ++jl) koff[jl] = (uint32_t)(n * rs + jl * 64 + g * 16);
  uint32_t voff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) voff[i] = (uint32_t)((4 * g + i) * rs + n * VBYTES);

  struct Regs {
    Bytes<16> k[KLOADS];
    Bytes<VBYTES> v[4];
  };

  int ids = 0, ids_chunk = -1;
  auto load_tile = [&](int i, Regs& r) {
    const int c = i >> 6;
    if (c != ids_chunk) {
      ids = load_block_ids(p, b, t_lo, w, c, n_my);
      ids_chunk = c;
    }
    const int blk = __builtin_amdgcn_readlane(ids, i & 63);
    const int t0 = t_lo + kTile * (w + kWaves * i);
    const int64_t tb = (int64_t)blk * blk_bytes + (int64_t)(t0 % p.bs) * rs;
    const char* kb = kbase + tb;
    const char* vb = vbase + tb;
#pragma unroll
    for (int jl = 0; jl < KLOADS; ++jl) r.k[jl] = load_bytes<16>(kb, koff[jl]);
#pragma unroll
    for (int q = 0; q < 4; ++q) r.v[q] = load_bytes<VBYTES>(vb, voff[q]);
  };

  float m = kMaxFloor;
  float l = 0.f;
  f32x4 acc[NJV];
#pragma unroll
  for (int j = 0; j < NJV; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute_tile = [&](int i, Regs& r) {
    const int t0 = t_lo + kTile * (w + kWaves * i);
    if (t0 + kTile > t_hi) {
      // tokens past the end of the sequence may hold anything (NaN poison):
      // their V rows must not reach the P x V product
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (t0 + 4 * g + q >= t_hi) r.v[q].zero();
    }
    // scores: D[token 4g+q][head n]
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NJQ; ++j) {
      i32x4 a;
      if constexpr (kFP8) {
        const uint32_t w0 = r.k[j >> 1].w((j & 1) * 2);
        const uint32_t w1 = r.k[j >> 1].w((j & 1) * 2 + 1);
        const i32x2 lo = kBF16 ? fp8x4_to_bf16x4(w0) : fp8x4_to_f16x4(w0);
        const i32x2 hi = kBF16 ? fp8x4_to_bf16x4(w1) : fp8x4_to_f16x4(w1);
        a = i32x4{lo[0], lo[1], hi[0], hi[1]};
      } else {
        a = r.k[j].v;
      }
      s = mfma_k32<kBF16>(a, qop[j], s);
    }
    float sv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      sv[q] = (t0 + 4 * g + q < t_hi) ? s[q] * p.qk_scale_log2 : -INFINITY;
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

    // V rows as 16-bit words: vw[q][k] holds elements 2k, 2k+1 of token 4g+q
    uint32_t vw[4][VW];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if constexpr (kFP8) {
#pragma unroll
        for (int k = 0; k < VW / 2; ++k) {
          const i32x2 c2 = kBF16 ? fp8x4_to_bf16x4(r.v[q].w(k)) : fp8x4_to_f16x4(r.v[q].w(k));
          vw[q][2 * k] = (uint32_t)c2[0];
          vw[q][2 * k + 1] = (uint32_t)c2[1];
        }
      } else {
#pragma unroll
        for (int k = 0; k < VW; ++k) vw[q][k] = r.v[q].w(k);
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

  // two register sets in ping-pong: the next tile's loads are in flight
  // while the current tile is computed
  if (n_my > 0) {
    Regs r0, r1;
    load_tile(0, r0);
    int i = 0;
    for (; i + 1 < n_my; i += 2) {
      load_tile(i + 1, r1);
      compute_tile(i, r0);
      if (i + 2 < n_my) load_tile(i + 2, r0);
      compute_tile(i + 1, r1);
    }
    if (i < n_my) compute_tile(i, r0);
  }

  // lane groups hold partial sums over different tokens
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (g == 0) {
    sm_ml[w][n][0] = m;
    sm_ml[w][n][1] = l;
  }
#pragma unroll
  for (int j = 0; j < NJV; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) sm_acc[w][n][(4 * g + q) * NJV + j] = acc[j][q];
  __syncthreads();
  combine_and_store<QK, D, 16, kWaves>(p, sm_ml, sm_acc, b, part, head0, nh, L);
}

// ============================================================================
// VALU inner loop: any supported dtype pair, GT query heads per workgroup.
// ============================================================================
template <int QK, int KVK, int D, int GT>
__global__ __launch_bounds__(kThreads) void decode_valu_kernel(const DecodeParams p) {
  constexpr int ESZ = Esz<KVK>::v;
  constexpr int VEC = 16 / ESZ;      // KV elements per 16-byte load
  constexpr int LPT = D / VEC;       // lanes per token row
  constexpr int TPL = 64 / LPT;      // tokens per load instruction
  constexpr int NL = kTile / TPL;    // loads per tile (K and V each)
  constexpr bool kDot2 = KVK == K_F16 || KVK == K_BF16;
  constexpr int QE = VEC;            // query elements per lane
  static_assert(LPT >= 1 && LPT <= 64 && 64 % LPT == 0 && kTile % TPL == 0, "shape");
  static_assert(!kDot2 || QK == KVK, "16-bit KV needs a query of the same type");

  __shared__ float sm_ml[kWaves][GT][2];
  __shared__ float sm_acc[kWaves][GT][D + kPad];

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int r = lane / LPT;          // token slot of this lane in a load
  const int c = lane - r * LPT;      // 16-byte chunk of the row
  const int b = blockIdx.z;
  const int part = blockIdx.y;
  const int kvh = blockIdx.x / p.head_tiles;
  const int htile = blockIdx.x - kvh * p.head_tiles;
  const int L = clamp_len(p, b);
  const int t_lo = part * p.part_tokens;
  if (part > 0 && t_lo >= L) return;
  const int t_hi = min(L, t_lo + p.part_tokens);
  const int n_tiles = t_hi > t_lo ? (t_hi - t_lo + kTile - 1) / kTile : 0;
  const int n_my = n_tiles > w ? (n_tiles - w + kWaves - 1) / kWaves : 0;
  const int gh0 = htile * GT;
  const int nh = min(GT, p.G - gh0);
  const int head0 = kvh * p.G + gh0;

  // query chunk of each head: packed 16-bit words for v_dot2, else fp32
  // pre-multiplied by the score scale
  uint32_t qw[GT][kDot2 ? QE / 2 : 1];
  float qf[GT][kDot2 ? 1 : QE];
#pragma unroll
  for (int gh = 0; gh < GT; ++gh) {
    const int hq = head0 + min(gh, nh - 1);
    const int64_t qo = (int64_t)b * p.q_sb + (int64_t)hq * p.q_sh + c * QE;
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
  const char* kbase = static_cast<const char*>(p.kc) + (int64_t)kvh * D * ESZ;
  const char* vbase = static_cast<const char*>(p.vc) + (int64_t)kvh * D * ESZ;
  uint32_t off[NL];
#pragma unroll
  for (int li = 0; li < NL; ++li) off[li] = (uint32_t)((li * TPL + r) * rs + c * 16);

  struct Regs {
    Bytes<16> k[NL];
    Bytes<16> v[NL];
  };
  int ids = 0, ids_chunk = -1;
  auto load_tile = [&](int i, Regs& rg) {
    const int ch = i >> 6;
    if (ch != ids_chunk) {
      ids = load_block_ids(p, b, t_lo, w, ch, n_my);
      ids_chunk = ch;
    }
    const int blk = __builtin_amdgcn_readlane(ids, i & 63);
    const int t0 = t_lo + kTile * (w + kWaves * i);
    const int64_t tb = (int64_t)blk * blk_bytes + (int64_t)(t0 % p.bs) * rs;
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
    const int t0 = t_lo + kTile * (w + kWaves * i);
    bool valid[NL];
#pragma unroll
    for (int li = 0; li < NL; ++li) valid[li] = t0 + li * TPL + r < t_hi;
    if (t0 + kTile > t_hi) {
#pragma unroll
      for (int li = 0; li < NL; ++li)
        if (!valid[li]) {
          rg.k[li].zero();
          rg.v[li].zero();
        }
    }
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
        const uint32_t wd = rg.v[li].w(k);
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
  if (n_my > 0) {
    Regs r0, r1;
    load_tile(0, r0);
    int i = 0;
    for (; i + 1 < n_my; i += 2) {
      load_tile(i + 1, r1);
      compute_tile(i, r0);
      if (i + 2 < n_my) load_tile(i + 2, r0);
      compute_tile(i + 1, r1);
    }
    if (i < n_my) compute_tile(i, r0);
  }

  // rows of one wave hold disjoint tokens: merge their states (lanes with the
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
  if (r == 0) {
#pragma unroll
    for (int gh = 0; gh < GT; ++gh) {
      if (c == 0) {
        sm_ml[w][gh][0] = m[gh];
        sm_ml[w][gh][1] = lsum[gh];
      }
#pragma unroll
      for (int e = 0; e < VEC; ++e) sm_acc[w][gh][c * VEC + e] = acc[gh][e];
    }
  }
  __syncthreads();
  combine_and_store<QK, D, GT, kWaves>(p, sm_ml, sm_acc, b, part, head0, nh, L);
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
  const int64_t base = ((int64_t)b * p.Hq + h) * p.num_parts;
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
hipError_t launch_valu(const DecodeParams& p, int gt, dim3 grid, hipStream_t stream) {
  switch (gt) {
    case 1: hipLaunchKernelGGL((decode_valu_kernel<QK, KVK, D, 1>), grid, dim3(kThreads), 0, stream, p); break;
    case 2: hipLaunchKernelGGL((decode_valu_kernel<QK, KVK, D, 2>), grid, dim3(kThreads), 0, stream, p); break;
    case 4: hipLaunchKernelGGL((decode_valu_kernel<QK, KVK, D, 4>), grid, dim3(kThreads), 0, stream, p); break;
    default: return hipErrorNotSupported;
  }
  return hipGetLastError();
}

template <int QK, int KVK, int D>
hipError_t launch_mfma(const DecodeParams& p, dim3 grid, hipStream_t stream) {
  hipLaunchKernelGGL((decode_mfma_kernel<QK, KVK, D>), grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <int QK, int KVK, int D>
hipError_t launch_all(const DecodeParams& p, const DecodeVariant& v, hipStream_t stream) {
  const dim3 grid(p.Hkv * p.head_tiles, p.num_parts, p.B);
  hipError_t e;
  if (v.path == 2) {
    if constexpr (QK == K_F32 || KVK == K_F32) return hipErrorNotSupported;
    else e = launch_mfma<QK, KVK, D>(p, grid, stream);
  } else {
    e = launch_valu<QK, KVK, D>(p, v.gt, grid, stream);
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
