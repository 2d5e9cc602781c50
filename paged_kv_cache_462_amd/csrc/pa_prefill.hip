// Paged prefill attention for gfx950 (CDNA4).
//
// The method: a batch of new tokens per sequence, whose K/V are already in
// the paged cache, attends causally over the sequence's cached tokens.  The
// rows of a sequence are its last n tokens; the row at position p sees the
// tokens at positions 0..p ("5.KV Cache 管理 & PagedAttention", question 6,
// `MHAWithCache` prefill branch: lower-triangular mask; question 19: outer
// loop over query tiles, inner loop over the logical KV blocks looked up in
// the block table, online softmax, normalise at the end; question 3,
// section 3.3: the prefill pass keeps its K/V in the cache).  With a few
// hundred query rows per tile this is a dense contraction, so both products
// run on the matrix cores.
//
// Work decomposition.  A workgroup is kWaves (8) waves and takes one query
// head and one tile of kBM (256) consecutive rows of one sequence; each
// wave owns kQSub (2) 16-row subtiles and two waves share a SIMD.  The grid
// is (query head, tile rank x sequence): rank 0 is the last (heaviest, it
// sees the most keys) tile of every sequence, so the long tiles are
// dispatched first and the short ones fill in at the end; a grid with fewer
// ranks than tiles loops.  A workgroup walks the keys its tile needs, 64 at
// a time:
//  * the four 16-token subtiles of a 64-key tile each lie inside one
//    physical block (the block size is a multiple of 16); the block ids of
//    64 subtiles are prefetched into one VGPR, one chunk ahead, and read
//    with v_readlane, so every K/V address is a scalar block base plus a
//    per-lane offset and no table load sits between the K/V loads;
//  * every thread loads 16-byte chunks of K and V rows (16 lanes per
//    256-byte row) into registers one tile ahead and stores them to a
//    double-buffered LDS tile at the top of the next iteration (slots past
//    the keys the tile needs are zeroed there, so a stale NaN never meets a
//    zero weight).  LDS rows are padded (K 272, V 288 bytes at head_dim
//    128) so that the operand reads hit distinct banks.
// Per wave and KV tile:
//  * scores^T[16 keys x 16 rows] = K[16 x D] . Q^T[D x 16] on
//    v_mfma_f32_16x16x32; Q stays in registers.  Lane l gets keys
//    4*(l/16)+i of query row l%16;
//  * online softmax per row in the exp2 domain (the score scale carries
//    log2 e).  The reference max is shared by the four lanes of a row and
//    only moves (with a cross-lane max and a rescale of the output) when a
//    score exceeds it by more than 2^8; otherwise the tile needs no
//    cross-lane step at all.  The mask is applied only on the KV tiles that
//    cross the wave's diagonal;
//  * out^T[D x 16] += V^T[D x 32 keys] . P^T[32 keys x 16] on
//    v_mfma_f32_16x16x32: the k index of that product runs over keys in
//    the order the score tile left them in the lanes, so P^T needs no data
//    movement, and the V^T operand comes straight out of LDS transpose
//    reads (ds_read_b64_tr_b16); a row of ones as V^T gives the weight sums
//    on the matrix cores as well;
//  * P needs more than bf16's 8 significant bits (a single bf16 P uses most
//    of the error budget of a 16-bit result).  A bf16 query therefore runs
//    P x V in f16 with f16 P (11 bits, like the f16 query): V is converted
//    to f16 while staged (fp8 V decodes to f16 directly), exactly for bf16
//    magnitudes from 2^-14 up to (not including) 2^16; smaller ones land on
//    f16's subnormal grid (spacing 2^-24), an absolute error of at most
//    2^-25 per value and so at most 2^-25 on an output, which is a weighted
//    mean of the values.  A workgroup that staged a value of 2^16 or more
//    is flagged
//    and recomputed by a second launch in bf16, P split into a high and a
//    low bf16 part with a product each (~16 significant bits).  Without
//    the flag array the bf16 product runs throughout.
#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"
#include "pa_prefill.h"

namespace pa {

namespace {

#ifndef PA_PREFILL_WAVES
#define PA_PREFILL_WAVES 8
#endif
constexpr int kWaves = PA_PREFILL_WAVES;
constexpr int kThreads = kWaves * 64;
constexpr int kBN = 64;                      // keys per KV tile
#ifndef PA_PREFILL_QSUB
#define PA_PREFILL_QSUB 2
#endif
#ifndef PA_PREFILL_WAVES_PER_EU
#define PA_PREFILL_WAVES_PER_EU 2
#endif
constexpr int kQSub = PA_PREFILL_QSUB;       // 16-row query subtiles per wave
constexpr int kBM = kWaves * kQSub * 16;     // query rows per workgroup
// largest growth of a row max (log2 units) absorbed without rescaling the
// accumulated output: weights stay below 2^8, far inside f16 / bf16 range
constexpr float kLazyRescale = 8.0f;
// bf16 magnitude bits (sign cleared) from which a value no longer fits f16:
// 0x4780 is 2^16, and everything above it up to inf and NaN.  Below it a
// bf16 value converts to f16 exactly down to 2^-14; smaller ones round to
// f16's subnormal spacing (2^-24), an absolute error below 2^-25.
constexpr uint32_t kBf16F16Limit = 0x4780u;

template <int KIND>
struct Esz {
  static constexpr int v = KIND == K_FP8 ? 1 : 2;
};

// 16 bytes of one K/V row chunk (8 elements) as 16-bit MFMA input.
template <int KVK, bool BF>
__device__ __forceinline__ i32x4 load_chunk(const char* p) {
  if constexpr (KVK == K_FP8) {
    const i32x2 raw = *reinterpret_cast<const i32x2*>(p);
    const i32x2 lo = BF ? fp8x4_to_bf16x4((uint32_t)raw[0]) : fp8x4_to_f16x4((uint32_t)raw[0]);
    const i32x2 hi = BF ? fp8x4_to_bf16x4((uint32_t)raw[1]) : fp8x4_to_f16x4((uint32_t)raw[1]);
    return i32x4{lo[0], lo[1], hi[0], hi[1]};
  } else {
    return *reinterpret_cast<const i32x4*>(p);
  }
}

// LDS transpose read (ds_read_b64_tr_b16), 4 16-bit values
__device__ __forceinline__ i32x2 lds_tr16(const char* p) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(__attribute__((address_space(3))) const char*)p);
  return __builtin_bit_cast(i32x2, r);
}

// PFX = false: causal prefill.  PFX = true: the shared-prefix pass of a
// decode batch (see PrefillParams): the same tile machinery with rows taken
// from every sequence, a per-row key limit instead of the causal one, one
// key piece per workgroup, and triples instead of normalised rows.
template <int QK, int KVK, int D, bool PFX, bool F16PV>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(PA_PREFILL_WAVES_PER_EU)))
void prefill_mfma_kernel(PrefillParams p) {
  static_assert(D == 64 || D == 128, "head_dim 64 or 128");
  constexpr bool BF = QK == K_BF16;
  constexpr int CH = D / 8;                      // 16-byte chunks (8 values) per row
  constexpr int DB = D / 16;                     // 16-dim output blocks
  // LDS row pitches (D 16-bit values + pad), chosen for the 64 four-byte
  // banks: a K row starts 4 banks after the previous one, so the 16 rows a
  // 16-lane group reads at one chunk (ds_read_b128) cover all 64 banks; a V
  // row starts 8 banks after the previous one (D = 128; 40 for D = 64), so
  // the 8 rows x 32 bytes that 32 lanes' transpose reads (ds_read_b64_tr_b16)
  // cover do not overlap
  constexpr int kRowK = D * 2 + 16;
  constexpr int kRowV = D * 2 + 32;
  constexpr int kStageRows = kThreads / CH;      // KV-tile rows one staging pass covers
  constexpr int kStagePasses = kBN / kStageRows;
  constexpr int KS = D / 32;    // k-steps of the score product
  constexpr int ESZ = Esz<KVK>::v;
  // F16PV (bf16 query only): V is staged as f16 (fp8 V decodes to f16;
  // bf16 V converts exactly below 2^16) and P x V runs in f16 with f16 P,
  // one product.  Otherwise P x V runs in the query's type, bf16 P as a hi
  // and a lo part with a product each.
  constexpr bool BFPV = BF && !F16PV;
  constexpr bool kCheckWide = F16PV && KVK == K_BF16;
  static_assert(!F16PV || (BF && (!PFX || KVK == K_FP8)),
                "f16 P x V: bf16 query; in the prefix pass only with fp8 K/V (no flags)");
  constexpr int kOne2 = BFPV ? 0x3F803F80 : 0x3C003C00;  // two 16-bit ones
  const i32x4 kOnes = i32x4{kOne2, kOne2, kOne2, kOne2};
  // K and V tiles, double-buffered, with the padded pitches above: the
  // operand reads below are conflict-free with plain (immediate-offset)
  // addressing
  __shared__ __attribute__((aligned(16))) char k_lds[2][kBN * kRowK];
  __shared__ __attribute__((aligned(16))) char v_lds[2][kBN * kRowV];

  if constexpr (!PFX && BFPV && KVK == K_BF16) {
    // second launch after the f16 pass: only the workgroups it flagged
    if (p.wide_flags && p.wide_flags[blockIdx.x] == 0) return;
  }
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int n16 = lane & 15;
  const int g = lane >> 4;
  // Workgroup id -> (query head, sequence, tile rank).  Workgroups are
  // dealt to the eight XCDs round-robin (id % 8), each with its own L2.
  // When the (sequence, kv head) groups split evenly over the XCDs, XCD x
  // takes whole groups (every query head of the group, every tile), so a
  // group's K/V is fetched into one L2 and reused there by all its query
  // heads and tiles; inside an XCD the order is heaviest tile rank first.
  int h, b, rank, kvh, piece = 0;
  if constexpr (PFX) {
    // (kv head, key piece, row tile), row tiles fastest
    const int id = blockIdx.x;
    rank = id % p.pfx_row_tiles;
    const int t2 = id / p.pfx_row_tiles;
    piece = t2 % p.pfx_pieces;
    kvh = t2 / p.pfx_pieces;
    h = kvh * p.G;
    b = 0;
  } else {
    const int id = blockIdx.x;
    if (p.xcd_groups) {
      const int x = id & 7, slot = id >> 3;
      const int per_rank = p.xcd_groups * p.G;  // items of one rank on an XCD
      rank = slot / per_rank;
      const int r2 = slot - rank * per_rank;
      const int gi = (r2 / p.G) * 8 + x;        // (sequence, kv head) group
      b = gi / p.Hkv;
      h = (gi - b * p.Hkv) * p.G + r2 % p.G;
    } else {
      h = id % p.Hq;
      const int y = id / p.Hq;
      b = y % p.B;
      rank = y / p.B;
    }
    kvh = h / p.G;
  }
  // causal: rows of sequence b; prefix pass: all B * G (sequence, head) rows
  // device-resident sizes are clamped to what the buffers hold (a value
  // outside them is a caller error; clamping keeps every access in bounds)
  if constexpr (!PFX) {
    const int s0 = p.qsl[b], s1 = p.qsl[b + 1], len = p.lens[b];
    if (s0 < 0 || s1 > p.T || s1 < s0) raise_flag(p.flags, kFlagQueryStart);
    if (len < 0 || len > p.max_blocks * p.bs) raise_flag(p.flags, kFlagLength);
  }
  const int q0 = PFX ? 0 : min(max(p.qsl[b], 0), p.T);
  const int n = PFX ? p.B * p.G : min(p.qsl[b + 1], p.T) - q0;
  const int L = PFX ? p.pfx_tokens : min(p.lens[b], p.max_blocks * p.bs);
  const int ntiles = (n + kBM - 1) / kBM;
  const int ctx = L - n;  // position of row 0 (negative when n > L)
  const int32_t* tab = p.tables + (int64_t)b * p.tab_stride;
  const int64_t tok_bytes = (int64_t)p.Hkv * D * ESZ;
  const char* kbase = static_cast<const char*>(p.kc) + (int64_t)kvh * D * ESZ;
  const char* vbase = static_cast<const char*>(p.vc) + (int64_t)kvh * D * ESZ;
  // staging: thread -> row srow + kStageRows i of the KV tile, chunk sch;
  // a wave covers 64 / CH consecutive rows of one 16-token subtile, so the
  // subtile (srow >> 4) + (kStageRows / 16) i is wave-uniform
  const int srow = threadIdx.x / CH;
  const int sch = threadIdx.x % CH;
  // the wave's first staging subtile (srow >> 4 is the same for all its
  // lanes), as a scalar, so the block lookups and K/V addresses below are
  // scalar arithmetic with scalar branches
  const int sub_w = __builtin_amdgcn_readfirstlane(srow >> 4);
  // a 16-token subtile lies in one block: uniform base + this per-lane part
  const uint32_t lane_off = (uint32_t)((srow & 15) * tok_bytes + sch * 8 * ESZ);
  const int64_t blk_bytes = (int64_t)p.bs * tok_bytes;
  // LDS byte offsets this lane reads from: the K operand (row n16 of a key
  // subtile, chunk g of a k-step) and the V^T transpose source (row 4g +
  // n16/4 of a 4-key group, dims 4 (n16 % 4) .. +3 of a 16-dim block)
  const int k_rd = n16 * kRowK + g * 16;
  const int v_rd = (4 * g + (n16 >> 2)) * kRowV + (n16 & 3) * 8;

  // causal: heaviest tile first, looping when the grid has fewer ranks than
  // tiles; prefix pass: exactly row tile `rank`
  bool wide = false;  // f16 pass: a staged V value outside f16's range
  for (int tile = PFX ? rank : ntiles - 1 - rank; tile >= 0; tile = PFX ? -1 : tile - p.tile_ranks) {
    const int row0 = tile * kBM;
    const int rows = min(kBM, n - row0);
    // keys [k_begin, kv_end) of this workgroup
    const int k_begin = PFX ? piece * p.pfx_chunk : 0;
    const int kv_end = PFX ? min(L, k_begin + p.pfx_chunk) : min(L, ctx + row0 + rows);
    const int kt0 = k_begin / kBN;
    const int ntk = kv_end > 0 ? (kv_end + kBN - 1) / kBN : 0;
    const int wrow0 = row0 + w * kQSub * 16;
    const int wrows = max(0, min(kQSub * 16, n - wrow0));

    i32x4 qf[kQSub][KS];
    int pos[kQSub];  // the row sees keys 0 .. pos
#pragma unroll
    for (int qs = 0; qs < kQSub; ++qs) {
      const int row = wrow0 + qs * 16 + n16;
      const int rc = min(row, n - 1);
      int64_t qoff;
      if constexpr (PFX) {
        // row = b * G + j: sequence b, query head kvh * G + j
        const int rb = rc / p.G;
        pos[qs] = row < n ? min(max(p.lens[rb], 0), L) - 1 : -1;  // L <= the table's reach
        qoff = (int64_t)rb * p.q_st + (int64_t)(h + rc - rb * p.G) * p.q_sh;
      } else {
        pos[qs] = ctx + row;
        qoff = (int64_t)(q0 + rc) * p.q_st + (int64_t)h * p.q_sh;
      }
      const char* qp = static_cast<const char*>(p.q) + qoff * 2;
#pragma unroll
      for (int st = 0; st < KS; ++st) qf[qs][st] = *reinterpret_cast<const i32x4*>(qp + (4 * st + g) * 16);
    }
    // keys this wave needs: [.., w_end); the mask is needed from w_first on
    int w_end, w_first;
    if constexpr (PFX) {
      int hi = -1, lo = 1 << 30;
#pragma unroll
      for (int qs = 0; qs < kQSub; ++qs) {
        hi = max(hi, pos[qs]);
        lo = min(lo, pos[qs]);
      }
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        hi = max(hi, __shfl_xor(hi, off));
        lo = min(lo, __shfl_xor(lo, off));
      }
      w_end = min(kv_end, hi + 1);
      w_first = lo;
    } else {
      w_end = wrows > 0 ? min(L, ctx + wrow0 + wrows) : 0;
      w_first = ctx + wrow0;
    }
    // running max (log2 units), output and weight sum (every element of
    // ls[qs] holds the sum of its lane's row)
    float m[kQSub];
    f32x4 o[kQSub][DB], ls[kQSub];
#pragma unroll
    for (int qs = 0; qs < kQSub; ++qs) {
      m[qs] = kMaxFloor;
      ls[qs] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < DB; ++j) o[qs][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // Block ids, 64 subtiles (16 KV tiles) per VGPR: lane i of chunk c
    // holds the id of subtile 64c + i; the next chunk is fetched one chunk
    // ahead, so reading an id (v_readlane) never waits on the table
    auto fetch_ids = [&](int chunk) {
      const int tok0 = (chunk * 64 + lane) * 16;
      const int id = tok0 < kv_end ? tab[tok0 / p.bs] : 0;
      if ((unsigned)id < (unsigned)p.num_blocks) return id;
      raise_flag(p.flags, kFlagBlockId);
      return 0;
    };
    int ids_cur = fetch_ids(kt0 >> 4), ids_nxt = fetch_ids((kt0 >> 4) + 1), ids_chunk = kt0 >> 4;

    i32x4 kr[kStagePasses], vr[kStagePasses];
    // raw chunks of the four 16-token subtiles of KV tile kt (nothing is
    // done with them until they are stored, so no wait lands in the compute)
    auto load_tile = [&](int kt) {
      if ((kt >> 4) != ids_chunk) {  // workgroup-uniform
        ids_cur = ids_nxt;
        ids_chunk = kt >> 4;
        ids_nxt = fetch_ids(ids_chunk + 1);
      }
#pragma unroll
      for (int i = 0; i < kStagePasses; ++i) {
        const int sub = kt * 4 + sub_w + (kStageRows / 16) * i;
        const int sub0 = sub * 16;
        if (sub0 < kv_end) {
          const int blk = __builtin_amdgcn_readlane(ids_cur, sub & 63);
          const int in_blk = p.spb_shift >= 0 ? (sub & ((1 << p.spb_shift) - 1)) * 16 : sub0 % p.bs;
          const int64_t ub = (int64_t)blk * blk_bytes + (int64_t)in_blk * tok_bytes;
          kr[i] = load_chunk<KVK, BF>(kbase + ub + lane_off);
          vr[i] = load_chunk<KVK, BFPV>(vbase + ub + lane_off);
        } else {
          kr[i] = i32x4{0, 0, 0, 0};
          vr[i] = i32x4{0, 0, 0, 0};
        }
      }
    };

    __syncthreads();  // the previous tile's last KV tile is no longer read
    if (ntk > kt0) load_tile(kt0);
    for (int kt = kt0; kt < ntk; ++kt) {
      const int buf = kt & 1;
      const int key0 = kt * kBN;
      // bf16 V on the f16 path: converted here; `wide` notes a value
      // outside f16's range
      auto v_stage = [&](const i32x4& raw) {
        if constexpr (kCheckWide) {
          i32x4 o2;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const uint32_t w2 = (uint32_t)raw[e];
            wide |= (w2 & 0x7FFFu) >= kBf16F16Limit || (w2 >> 16 & 0x7FFFu) >= kBf16F16Limit;
            o2[e] = (int)pack_f16(bf16_lo(w2), bf16_hi(w2));
          }
          return o2;
        } else {
          return raw;
        }
      };
      if (key0 + kBN <= kv_end) {
#pragma unroll
        for (int i = 0; i < kStagePasses; ++i) {
          const int r = srow + kStageRows * i;
          *reinterpret_cast<i32x4*>(&k_lds[buf][r * kRowK + sch * 16]) = kr[i];
          *reinterpret_cast<i32x4*>(&v_lds[buf][r * kRowV + sch * 16]) = v_stage(vr[i]);
        }
      } else {
        // the keys end inside this tile: slots past the sequence's end hold
        // stale data, and keys past the tile's last row are never weighted
        // (zero them so that 0 * stale never reaches the output)
#pragma unroll
        for (int i = 0; i < kStagePasses; ++i) {
          const int r = srow + kStageRows * i;
          const bool live = key0 + r < kv_end;
          *reinterpret_cast<i32x4*>(&k_lds[buf][r * kRowK + sch * 16]) = live ? kr[i] : i32x4{0, 0, 0, 0};
          *reinterpret_cast<i32x4*>(&v_lds[buf][r * kRowV + sch * 16]) =
              v_stage(live ? vr[i] : i32x4{0, 0, 0, 0});
        }
      }
      __syncthreads();
      if (kt + 1 < ntk) load_tile(kt + 1);

      if (key0 >= w_end) continue;  // every row of this wave is done

      // scores^T for the 4 key subtiles x kQSub row subtiles
      f32x4 s[kQSub][4];
#pragma unroll
      for (int qs = 0; qs < kQSub; ++qs)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) s[qs][ks] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < KS; ++st) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const i32x4 kf = *reinterpret_cast<const i32x4*>(&k_lds[buf][k_rd + ks * 16 * kRowK + st * 64]);
#pragma unroll
          for (int qs = 0; qs < kQSub; ++qs) s[qs][ks] = mfma_k32<BF>(kf, qf[qs][st], s[qs][ks]);
        }
      }

      // online softmax; P^T operands (keys 4g+e of subtiles 2s2 and 2s2+1).
      // Only the KV tiles that cross the wave's diagonal take the mask.
      i32x4 ph[kQSub][2], pl[kQSub][2];
      auto softmax = [&](auto masked) {
#pragma unroll
        for (int qs = 0; qs < kQSub; ++qs) {
          float x[4][4];
          float tmax = -INFINITY;
          const int lim = pos[qs] - key0 - 4 * g;  // keys ks*16+e <= lim are seen
#pragma unroll
          for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float v = s[qs][ks][e];
              if constexpr (decltype(masked)::value) v = ks * 16 + e <= lim ? v : -INFINITY;
              x[ks][e] = v;
              tmax = fmaxf(tmax, v);
            }
          // The reference max m[qs] is shared by the four lanes of a row
          // and only moves when some row of the wave has a score more than
          // kLazyRescale (log2 units) above it; the per-tile check needs no
          // cross-lane step (the scale is positive, so the scaled max is the
          // max scaled).  Between moves the weights stay below
          // 2^kLazyRescale, and output and sum share the reference, so the
          // result is the same.
          if (__any(tmax * p.qk_scale_log2 > m[qs] + kLazyRescale)) {
            asm volatile("" ::);  // keep this a branch (rarely taken)
            tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
            const float mn = fmaxf(m[qs], tmax * p.qk_scale_log2);
            const float alpha = fast_exp2(m[qs] - mn);
            m[qs] = mn;
            ls[qs] *= alpha;
#pragma unroll
            for (int j = 0; j < DB; ++j) o[qs][j] *= alpha;
          }
          const float mref = m[qs];
#pragma unroll
          for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int e = 0; e < 4; ++e) x[ks][e] = fast_exp2(__builtin_fmaf(x[ks][e], p.qk_scale_log2, -mref));
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            const float* a = x[2 * s2];
            const float* c = x[2 * s2 + 1];
            if constexpr (BFPV) {
              const uint32_t h0 = pack_bf16(a[0], a[1]), h1 = pack_bf16(a[2], a[3]);
              const uint32_t h2 = pack_bf16(c[0], c[1]), h3 = pack_bf16(c[2], c[3]);
              ph[qs][s2] = i32x4{(int)h0, (int)h1, (int)h2, (int)h3};
              pl[qs][s2] = i32x4{(int)pack_bf16(a[0] - bf16_lo(h0), a[1] - bf16_hi(h0)),
                                 (int)pack_bf16(a[2] - bf16_lo(h1), a[3] - bf16_hi(h1)),
                                 (int)pack_bf16(c[0] - bf16_lo(h2), c[1] - bf16_hi(h2)),
                                 (int)pack_bf16(c[2] - bf16_lo(h3), c[3] - bf16_hi(h3))};
            } else {
              ph[qs][s2] = i32x4{(int)pack_f16(a[0], a[1]), (int)pack_f16(a[2], a[3]),
                                 (int)pack_f16(c[0], c[1]), (int)pack_f16(c[2], c[3])};
            }
          }
        }
      };
      if (key0 + kBN - 1 > w_first)
        softmax(std::true_type{});
      else
        softmax(std::false_type{});

      // out^T += V^T . P^T, 32 keys per step.  The V^T operand of dims
      // 16 jb .. 16 jb + 15 comes straight out of two LDS transpose reads
      // (ds_read_b64_tr_b16): within each 16-lane group, lane j receives
      // element j % 4 of the 8 bytes lane 4e + j / 4 points at, so with
      // lane (g, j) pointing at row 4g + j/4 of a 4-key group, dims
      // 16 jb + 4 (j % 4) .. +3, lane (g, j) gets dim 16 jb + j of keys
      // 4g .. 4g+3 -- the k slots the score tile gave lane group g.
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
        for (int jb = 0; jb < DB; ++jb) {
          const char* vp = &v_lds[buf][v_rd + s2 * 32 * kRowV + jb * 32];
          const i32x2 lo = lds_tr16(vp);
          const i32x2 hi = lds_tr16(vp + 16 * kRowV);
          const i32x4 a = i32x4{lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
          for (int qs = 0; qs < kQSub; ++qs) {
            o[qs][jb] = mfma_k32<BFPV>(a, ph[qs][s2], o[qs][jb]);
            if constexpr (BFPV) o[qs][jb] = mfma_k32<BFPV>(a, pl[qs][s2], o[qs][jb]);
          }
        }
        // the weight sums on the matrix cores too: a row of ones as V^T
        // gives every lane its row's sum of exactly the weights the output
        // took (cheaper than 32 adds and two cross-lane steps per tile)
#pragma unroll
        for (int qs = 0; qs < kQSub; ++qs) {
          ls[qs] = mfma_k32<BFPV>(kOnes, ph[qs][s2], ls[qs]);
          if constexpr (BFPV) ls[qs] = mfma_k32<BFPV>(kOnes, pl[qs][s2], ls[qs]);
        }
      }
    }

    if constexpr (PFX) {
      // this piece's triple of every row: (max, sum) and the unnormalised
      // output, lane holding dims 16 jb + 4g .. +3
#pragma unroll
      for (int qs = 0; qs < kQSub; ++qs) {
        const int row = wrow0 + qs * 16 + n16;
        if (row < n) {
          const int rb = row / p.G;
          const int64_t ti = (int64_t)(p.pfx_slot0 + rb * p.pfx_pieces + piece) * p.Hq + h + (row - rb * p.G);
          float* acc = p.ws_acc + ti * D + 4 * g;
#pragma unroll
          for (int jb = 0; jb < DB; ++jb) *reinterpret_cast<f32x4*>(acc + jb * 16) = o[qs][jb];
          if (g == 0) {
            p.ws_ml[2 * ti] = m[qs];
            p.ws_ml[2 * ti + 1] = ls[qs][0];
          }
        }
      }
      continue;
    }
    // normalise and store: lane holds dims 16 jb + 4g .. 16 jb + 4g + 3
#pragma unroll
    for (int qs = 0; qs < kQSub; ++qs) {
      const float lt = ls[qs][0];
      const float inv = lt > 0.f ? p.v_scale / lt : 0.f;
      const int row = wrow0 + qs * 16 + n16;
      if (row < n) {
        char* op = static_cast<char*>(p.out) + ((int64_t)(q0 + row) * p.o_st + (int64_t)h * p.o_sh + 4 * g) * 2;
#pragma unroll
        for (int jb = 0; jb < DB; ++jb) {
          const f32x4 v = o[qs][jb] * inv;
          const i32x2 w2 = BF ? i32x2{(int)pack_bf16(v[0], v[1]), (int)pack_bf16(v[2], v[3])}
                              : i32x2{(int)pack_f16(v[0], v[1]), (int)pack_f16(v[2], v[3])};
          *reinterpret_cast<i32x2*>(op + jb * 32) = w2;
        }
      }
    }
  }
  if constexpr (kCheckWide) {
    // every thread of the workgroup gets here: one flag per workgroup, 1
    // when any of its tiles staged a V value outside f16's range
    if (p.wide_flags) {
      const int any = __syncthreads_or(wide ? 1 : 0);
      if (threadIdx.x == 0) p.wide_flags[blockIdx.x] = any != 0;
    }
  }
}

template <int QK, int KVK, int D, bool PFX, bool F16PV = false>
hipError_t launch_one(const PrefillParams& p, hipStream_t stream) {
  const dim3 grid(PFX ? (unsigned)(p.Hkv * p.pfx_row_tiles * p.pfx_pieces)
                      : (unsigned)(p.Hq * p.tile_ranks * p.B));
  hipLaunchKernelGGL((prefill_mfma_kernel<QK, KVK, D, PFX, F16PV>), grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

template <bool PFX>
hipError_t launch_mode(const PrefillParams& p, int qkind, int kvkind, hipStream_t stream) {
  if (!prefill_variant_built(qkind, kvkind, p.D)) return hipErrorNotSupported;
  const bool fp8 = kvkind == K_FP8;
  if (p.D == 64) {
    if (qkind == K_F16)
      return fp8 ? launch_one<K_F16, K_FP8, 64, PFX>(p, stream) : launch_one<K_F16, K_F16, 64, PFX>(p, stream);
    return fp8 ? launch_one<K_BF16, K_FP8, 64, PFX>(p, stream) : launch_one<K_BF16, K_BF16, 64, PFX>(p, stream);
  }
  if (qkind == K_F16)
    return fp8 ? launch_one<K_F16, K_FP8, 128, PFX>(p, stream) : launch_one<K_F16, K_F16, 128, PFX>(p, stream);
  return fp8 ? launch_one<K_BF16, K_FP8, 128, PFX>(p, stream) : launch_one<K_BF16, K_BF16, 128, PFX>(p, stream);
}

// bf16 query, P x V in f16: fp8 K/V in one launch; bf16 K/V in the f16
// launch and the launch that redoes the flagged workgroups in bf16
template <int D>
hipError_t launch_bf16_f16pv(const PrefillParams& p, int kvkind, hipStream_t stream) {
  if (kvkind == K_FP8) return launch_one<K_BF16, K_FP8, D, false, true>(p, stream);
  const hipError_t e = launch_one<K_BF16, K_BF16, D, false, true>(p, stream);
  if (e != hipSuccess) return e;
  return launch_one<K_BF16, K_BF16, D, false, false>(p, stream);
}

}  // namespace

int prefill_rows_per_workgroup() { return kBM; }

bool prefill_variant_built(int qkind, int kvkind, int D) {
  if (D != 64 && D != 128) return false;
  if (qkind != K_F16 && qkind != K_BF16) return false;
  return kvkind == qkind || kvkind == K_FP8;
}

hipError_t launch_prefill(const PrefillParams& p, int qkind, int kvkind, hipStream_t stream) {
  if (prefill_variant_built(qkind, kvkind, p.D) && qkind == K_BF16 &&
      (kvkind == K_FP8 || p.wide_flags))
    return p.D == 64 ? launch_bf16_f16pv<64>(p, kvkind, stream) : launch_bf16_f16pv<128>(p, kvkind, stream);
  PrefillParams q = p;
  q.wide_flags = nullptr;  // the plain bf16 launch redoes nothing
  return launch_mode<false>(q, qkind, kvkind, stream);
}

int64_t prefill_grid_size(int64_t B, int64_t Hq, int64_t tile_ranks) { return Hq * tile_ranks * B; }

hipError_t launch_prefix_pass(const PrefillParams& p, int qkind, int kvkind, hipStream_t stream) {
  // fp8 values always fit f16: a bf16 query takes the f16 product there
  if (prefill_variant_built(qkind, kvkind, p.D) && qkind == K_BF16 && kvkind == K_FP8)
    return p.D == 64 ? launch_one<K_BF16, K_FP8, 64, true, true>(p, stream)
                     : launch_one<K_BF16, K_FP8, 128, true, true>(p, stream);
  return launch_mode<true>(p, qkind, kvkind, stream);
}

}  // namespace pa
