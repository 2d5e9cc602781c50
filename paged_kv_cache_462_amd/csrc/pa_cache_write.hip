// Cache write (reshape_and_cache) and whole-block copy kernels for gfx950.
//
// Writing a token: slot s -> block s / bs, offset s % bs; the token's
// [Hkv, D] row lands at cache[block, offset, :, :] ("5.KV Cache 管理 &
// PagedAttention", question 12, append_token).  Because the cache layout is
// [N, bs, Hkv, D], one token's Hkv*D elements are contiguous in both the
// source and the cache, so the write is a plain streaming copy (or fp8
// quantisation) of 16-byte chunks; each thread owns 8 elements.
//
// Block copy: the device half of copy-on-write (same page, question 18,
// copy_block), and block swap between a device pool and a pool in pinned
// host memory ("KV Cache 优化与内存管理深度解析：PagedAttention 原理与实践",
// `CPUSwap`): whole blocks with 16-byte loads and stores, thousands in
// flight, so a swap runs at the host link's rate without a copy call per
// block.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kElemsPerThread = 8;
constexpr int kThreads = 256;

// fp32 -> E4M3FN code: one correctly rounded fp32 division by the scale, then
// the hardware round-to-nearest-even conversion of a value clamped to the
// finite range (so saturation never depends on the converter); NaN keeps its
// sign and maps to S.1111.111.
__device__ __forceinline__ uint32_t quant_pair(float a, float b, float scale) {
  // scale is positive and finite (checked on the host), so y is NaN exactly
  // when x is, and carries x's sign.
  float ya = a / scale;
  float yb = b / scale;
  const bool na = a != a, nb = b != b;
  ya = fminf(fmaxf(ya, -448.0f), 448.0f);
  yb = fminf(fmaxf(yb, -448.0f), 448.0f);
  uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(ya, yb, 0, false) & 0xFFFFu;
  if (na) w = (w & 0xFF00u) | 0x7Fu | ((__builtin_bit_cast(uint32_t, a) >> 24) & 0x80u);
  if (nb) w = (w & 0x00FFu) | 0x7F00u | ((__builtin_bit_cast(uint32_t, b) >> 16) & 0x8000u);
  return w;
}

template <int SRC>
__device__ __forceinline__ void load8(const void* src, int64_t off, float (&x)[8]) {
  if constexpr (SRC == K_F32) {
    const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(src) + off);
    f32x4 a = p[0], b = p[1];
    x[0] = a[0]; x[1] = a[1]; x[2] = a[2]; x[3] = a[3];
    x[4] = b[0]; x[5] = b[1]; x[6] = b[2]; x[7] = b[3];
  } else {
    i32x4 v = *reinterpret_cast<const i32x4*>(static_cast<const uint16_t*>(src) + off);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w = (uint32_t)v[i];
      if constexpr (SRC == K_BF16) {
        x[2 * i] = bf16_lo(w);
        x[2 * i + 1] = bf16_hi(w);
      } else {
        x[2 * i] = f16_lo(w);
        x[2 * i + 1] = f16_hi(w);
      }
    }
  }
}

// SRC: element kind of key/value; QUANT: the cache is fp8.
template <int SRC, bool QUANT>
__global__ __launch_bounds__(kThreads) void cache_write_kernel(const CacheWriteParams p) {
  const int64_t row = (int64_t)p.Hkv * p.D;            // elements per token
  const int64_t chunks = row / kElemsPerThread;
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= p.T * chunks) return;
  const int64_t t = i / chunks;
  const int64_t c = i - t * chunks;
  const int64_t slot = p.slots[t];
  if (slot < 0) return;
  if (slot >= p.num_slots) {
    raise_flag(p.flags, kFlagSlot);
    return;
  }
  const int64_t dst = slot * row + c * kElemsPerThread;
  const int64_t ks = t * p.k_stride_tok + c * kElemsPerThread;
  const int64_t vs = t * p.v_stride_tok + c * kElemsPerThread;
  if constexpr (!QUANT) {
    constexpr int esz = SRC == K_F32 ? 4 : 2;
    if constexpr (esz == 4) {
      const f32x4* ksrc = reinterpret_cast<const f32x4*>(static_cast<const float*>(p.key) + ks);
      const f32x4* vsrc = reinterpret_cast<const f32x4*>(static_cast<const float*>(p.value) + vs);
      f32x4* kd = reinterpret_cast<f32x4*>(static_cast<float*>(p.kc) + dst);
      f32x4* vd = reinterpret_cast<f32x4*>(static_cast<float*>(p.vc) + dst);
      f32x4 k0 = ksrc[0], k1 = ksrc[1], v0 = vsrc[0], v1 = vsrc[1];
      kd[0] = k0; kd[1] = k1; vd[0] = v0; vd[1] = v1;
    } else {
      const i32x4 k = *reinterpret_cast<const i32x4*>(static_cast<const uint16_t*>(p.key) + ks);
      const i32x4 v = *reinterpret_cast<const i32x4*>(static_cast<const uint16_t*>(p.value) + vs);
      *reinterpret_cast<i32x4*>(static_cast<uint16_t*>(p.kc) + dst) = k;
      *reinterpret_cast<i32x4*>(static_cast<uint16_t*>(p.vc) + dst) = v;
    }
  } else {
    float k[8], v[8];
    load8<SRC>(p.key, ks, k);
    load8<SRC>(p.value, vs, v);
    i32x2 kq, vq;
    kq[0] = (int)(quant_pair(k[0], k[1], p.k_scale) | (quant_pair(k[2], k[3], p.k_scale) << 16));
    kq[1] = (int)(quant_pair(k[4], k[5], p.k_scale) | (quant_pair(k[6], k[7], p.k_scale) << 16));
    vq[0] = (int)(quant_pair(v[0], v[1], p.v_scale) | (quant_pair(v[2], v[3], p.v_scale) << 16));
    vq[1] = (int)(quant_pair(v[4], v[5], p.v_scale) | (quant_pair(v[6], v[7], p.v_scale) << 16));
    *reinterpret_cast<i32x2*>(static_cast<uint8_t*>(p.kc) + dst) = kq;
    *reinterpret_cast<i32x2*>(static_cast<uint8_t*>(p.vc) + dst) = vq;
  }
}

__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(const CopyBlocksParams p) {
  // one 16-byte chunk of one block of K and of V per thread
  const int64_t chunks = p.block_bytes / 16;
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= p.n * chunks) return;
  const int64_t pair = i / chunks;
  const int64_t c = i - pair * chunks;
  const int64_t src = p.pairs[2 * pair];
  const int64_t dst = p.pairs[2 * pair + 1];
  if (src < 0 || dst < 0 || src >= p.src_blocks || dst >= p.dst_blocks) {
    raise_flag(p.flags, kFlagBlockId);
    return;
  }
  const int64_t so = src * p.block_bytes + c * 16;
  const int64_t d_o = dst * p.block_bytes + c * 16;
  const i32x4 k = *reinterpret_cast<const i32x4*>(static_cast<const char*>(p.src_k) + so);
  const i32x4 v = *reinterpret_cast<const i32x4*>(static_cast<const char*>(p.src_v) + so);
  *reinterpret_cast<i32x4*>(static_cast<char*>(p.dst_k) + d_o) = k;
  *reinterpret_cast<i32x4*>(static_cast<char*>(p.dst_v) + d_o) = v;
}

}  // namespace

hipError_t launch_cache_write(const CacheWriteParams& p, int src_kind, int cache_kind,
                              hipStream_t stream) {
  if (p.T == 0) return hipSuccess;
  const int64_t chunks = (int64_t)p.Hkv * p.D / kElemsPerThread;
  const int64_t total = p.T * chunks;
  const int64_t grid = (total + kThreads - 1) / kThreads;
  if (grid > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  const bool quant = cache_kind == K_FP8;
  if (!quant && cache_kind != src_kind) return hipErrorNotSupported;
#define PA_CW(SRC, Q)                                                        \
  hipLaunchKernelGGL((cache_write_kernel<SRC, Q>), dim3((unsigned)grid),     \
                     dim3(kThreads), 0, stream, p)
  switch (src_kind) {
    case K_F32: if (quant) PA_CW(K_F32, true); else PA_CW(K_F32, false); break;
    case K_F16: if (quant) PA_CW(K_F16, true); else PA_CW(K_F16, false); break;
    case K_BF16: if (quant) PA_CW(K_BF16, true); else PA_CW(K_BF16, false); break;
    default: return hipErrorNotSupported;
  }
#undef PA_CW
  return hipGetLastError();
}

hipError_t launch_copy_blocks(const CopyBlocksParams& p, hipStream_t stream) {
  if (p.n == 0) return hipSuccess;
  const int64_t total = p.n * (p.block_bytes / 16);
  const int64_t grid = (total + kThreads - 1) / kThreads;
  if (grid > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pa
