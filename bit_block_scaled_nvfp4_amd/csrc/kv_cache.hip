// FP8 E4M3 KV cache for gfx950: new tokens' keys and values are encoded under one static
// (calibrated) scale per tensor and scattered into cache rows; the reverse gathers and decodes.
//
// Source: "Why Gated DeltaNet Survives 4-Bit Quantization" (arXiv 2609.04098), ai.info summary,
// "Key Contributions" (an FP8 KV cache with calibrated per-layer scales) and "Main Findings" (static
// per-tensor FP8 scales, one for each K and V tensor of the attention layers).  The encoding rules
// the pages leave open are stated in include/nvfp4.h: decode-direction scale, y = fl(x * fl(1/s)),
// E4M3 nearest-even saturating at 448, sign copied.
//
// The encode uses the CDNA4 conversion v_cvt_pk_fp8_f32 (OCP E4M3, round to nearest even,
// subnormals kept) on y clamped to [-448, 448] first, so nothing can overflow to NaN; the decode
// uses v_cvt_pk_f32_fp8, which is exact.
//
// Work split of the store: a thread owns 16 consecutive elements of one token's row (32 bytes of
// bf16/f16 or 64 bytes of f32 in, 16 code bytes out).  A row of width/16 chunks is served by the L
// lanes of a wave (L the power of two >= width/16, at most 64), so a wave covers 64/L whole tokens
// when rows are short and a 64-chunk stretch of one token when they are long; loads and stores of
// a wave are contiguous per token.  The load (decode direction) splits rows the same way into
// pieces of 8 (bf16 out) or 4 (f32 out) codes, so each lane writes one 16-byte piece.  The kernels
// are bound by HBM bandwidth (3 bytes moved per bf16 element).
#include "codec.h"
#include "nvfp4_internal.h"

namespace nvfp4 {
namespace {

using namespace codec;

constexpr int kThreads = 256;

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct KvStoreArgs {
  const uint8_t* src[2];  // key, value rows (bytes)
  int64_t ld_src[2];      // row pitch in bytes
  const float* scale[2];
  uint8_t* cache[2];
  const int64_t* slots;   // nullptr: token t -> slot t
  int64_t cache_ld;       // bytes
  int64_t num_slots;
  int32_t tokens;
  int32_t chunks;         // width / 16
  int32_t lane_bits;      // log2 of lanes per token
};

// Slot of token t, or -1 when the token is not stored (outside [0, num_slots)).
__device__ __forceinline__ int64_t slot_of(const int64_t* slots, int64_t num_slots, int32_t t) {
  const int64_t s = slots ? slots[t] : (int64_t)t;
  return (s >= 0 && s < num_slots) ? s : -1;
}

// grid: x over groups of 256 >> lane_bits tokens, y over stretches of (1 << lane_bits) chunks,
// z over the tensors (1: key only, 2: key and value).
template <nvfp4_dtype DT>
__global__ void __launch_bounds__(kThreads) kv_store_kernel(KvStoreArgs a) {
  const int z = blockIdx.z;
  const int lb = a.lane_bits;
  const int32_t t = (int32_t)(blockIdx.x * (kThreads >> lb)) + (int32_t)(threadIdx.x >> lb);
  const int32_t c = (int32_t)(blockIdx.y << lb) + (int32_t)(threadIdx.x & ((1u << lb) - 1));
  if (t >= a.tokens || c >= a.chunks) return;
  // the row is loaded before the slot is known, so both loads are in flight together
  constexpr int kEb = DT == NVFP4_F32 ? 4 : 2;
  float v[16];
  load_block<DT>(a.src[z] + (int64_t)t * a.ld_src[z] + (int64_t)c * 16 * kEb, v);
  const int64_t slot = slot_of(a.slots, a.num_slots, t);
  const float inv = 1.0f / *a.scale[z];  // correctly rounded (built with IEEE division)
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float y[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) y[j] = __builtin_fminf(__builtin_fmaxf(v[4 * i + j] * inv, -448.0f), 448.0f);
    int p = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
    p = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], p, true);
    w[i] = (uint32_t)p;
  }
  if (slot < 0) return;
  u32x4 o;
  o.x = w[0];
  o.y = w[1];
  o.z = w[2];
  o.w = w[3];
  __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(a.cache[z] + slot * a.cache_ld + (int64_t)c * 16));
}

struct KvLoadArgs {
  const uint8_t* cache;
  int64_t cache_ld;  // bytes
  int64_t num_slots;
  const float* scale;
  const int64_t* slots;
  uint8_t* out;
  int64_t ld_out;    // bytes
  int32_t tokens;
  int32_t pieces;     // width / kLoadElems
  int32_t lane_bits;  // log2 of lanes per token
};

__device__ __forceinline__ uint32_t bf16_pair_rne(float lo, float hi) {
  // nearest-even rounding of finite binary32 values to bfloat16, two per word
  const uint32_t a = __float_as_uint(lo), b = __float_as_uint(hi);
  const uint32_t ra = (a + 0x7FFFu + ((a >> 16) & 1u)) >> 16;
  const uint32_t rb = (b + 0x7FFFu + ((b >> 16) & 1u)) & 0xFFFF0000u;
  return ra | rb;
}

// Decode direction.  A lane owns kLoadElems<BF16_OUT> codes of one row: 8 for bfloat16 output and
// 4 for float32, so that it writes exactly 16 bytes.  A wavefront's loads (8 or 4 bytes per lane)
// and stores (16 bytes per lane) are then contiguous per token.  With 16 codes per lane, each lane
// wrote 32 or 64 bytes in several 16-byte stores, and a wavefront store instruction covered only
// every second or fourth 16-byte piece of the row.
template <bool BF16_OUT>
constexpr int kLoadElems = BF16_OUT ? 8 : 4;

// The kLoadElems codes of one piece, as one or two 32-bit words.
template <bool BF16_OUT>
struct KvPiece {
  uint32_t w[kLoadElems<BF16_OUT> / 4];
};

template <bool BF16_OUT>
__device__ __forceinline__ KvPiece<BF16_OUT> kv_load_piece(const uint8_t* src) {
  KvPiece<BF16_OUT> p;
  if constexpr (BF16_OUT) {
    const u32x2 q = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(src));
    p.w[0] = q.x;
    p.w[1] = q.y;
  } else {
    p.w[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(src));
  }
  return p;
}

// Decoded piece (zeros when `valid` is false), packed as the 16 output bytes.
template <bool BF16_OUT>
__device__ __forceinline__ u32x4 kv_decode_piece(const KvPiece<BF16_OUT>& p, float s, bool valid) {
  constexpr int E = kLoadElems<BF16_OUT>;
  float v[E];
#pragma unroll
  for (int i = 0; i < E / 4; ++i) {
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)p.w[i], false);
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)p.w[i], true);
    v[4 * i + 0] = valid ? lo[0] * s : 0.0f;
    v[4 * i + 1] = valid ? lo[1] * s : 0.0f;
    v[4 * i + 2] = valid ? hi[0] * s : 0.0f;
    v[4 * i + 3] = valid ? hi[1] * s : 0.0f;
  }
  u32x4 o;
  if constexpr (BF16_OUT) {
    o.x = bf16_pair_rne(v[0], v[1]);
    o.y = bf16_pair_rne(v[2], v[3]);
    o.z = bf16_pair_rne(v[4], v[5]);
    o.w = bf16_pair_rne(v[6], v[7]);
  } else {
    o.x = __float_as_uint(v[0]);
    o.y = __float_as_uint(v[1]);
    o.z = __float_as_uint(v[2]);
    o.w = __float_as_uint(v[3]);
  }
  return o;
}

// grid: x over groups of 2 * (256 >> lane_bits) tokens (each thread takes two tokens, the second
// 256 >> lane_bits tokens after the first), y over stretches of (1 << lane_bits) pieces.  Both
// tokens' slots, then both rows, are loaded before anything is decoded, so the two dependent load
// chains overlap.  A token whose slot is outside the cache reads row 0 (present whenever the cache
// has rows) and writes zeros.
template <bool BF16_OUT>
__global__ void __launch_bounds__(kThreads) kv_load_kernel(KvLoadArgs a) {
  constexpr int E = kLoadElems<BF16_OUT>;
  const int lb = a.lane_bits;
  const int32_t per = kThreads >> lb;
  const int32_t t0 = (int32_t)(blockIdx.x * 2 * per) + (int32_t)(threadIdx.x >> lb);
  const int32_t t1 = t0 + per;
  const int32_t c = (int32_t)(blockIdx.y << lb) + (int32_t)(threadIdx.x & ((1u << lb) - 1));
  if (t0 >= a.tokens || c >= a.pieces) return;
  const bool has1 = t1 < a.tokens;
  const int64_t s0 = slot_of(a.slots, a.num_slots, t0);
  const int64_t s1 = has1 ? slot_of(a.slots, a.num_slots, t1) : -1;
  KvPiece<BF16_OUT> p0{}, p1{};
  if (a.num_slots > 0) {
    p0 = kv_load_piece<BF16_OUT>(a.cache + (s0 >= 0 ? s0 : 0) * a.cache_ld + (int64_t)c * E);
    p1 = kv_load_piece<BF16_OUT>(a.cache + (s1 >= 0 ? s1 : 0) * a.cache_ld + (int64_t)c * E);
  }
  const float s = *a.scale;
  const u32x4 o0 = kv_decode_piece<BF16_OUT>(p0, s, s0 >= 0);
  __builtin_nontemporal_store(o0, reinterpret_cast<u32x4*>(a.out + (int64_t)t0 * a.ld_out + (int64_t)c * 16));
  if (has1) {
    const u32x4 o1 = kv_decode_piece<BF16_OUT>(p1, s, s1 >= 0);
    __builtin_nontemporal_store(o1, reinterpret_cast<u32x4*>(a.out + (int64_t)t1 * a.ld_out + (int64_t)c * 16));
  }
}

// Lanes per token: the power of two >= the pieces of a row, at most 64 (a wavefront).
int lane_bits_for(int64_t pieces) {
  int lb = 0;
  while (lb < 6 && (int64_t(1) << lb) < pieces) ++lb;
  return lb;
}

}  // namespace

hipError_t launch_kv_store(const void* key, const void* value, nvfp4_dtype dt, int64_t tokens,
                           int64_t width, int64_t ld_key, int64_t ld_value, const float* key_scale,
                           const float* value_scale, const int64_t* slots, uint8_t* key_cache,
                           uint8_t* value_cache, int64_t num_slots, int64_t cache_ld,
                           hipStream_t stream) {
  const int64_t eb = dt == NVFP4_F32 ? 4 : 2;
  KvStoreArgs a{};
  a.src[0] = static_cast<const uint8_t*>(key);
  a.src[1] = static_cast<const uint8_t*>(value);
  a.ld_src[0] = ld_key * eb;
  a.ld_src[1] = ld_value * eb;
  a.scale[0] = key_scale;
  a.scale[1] = value_scale;
  a.cache[0] = key_cache;
  a.cache[1] = value_cache;
  a.slots = slots;
  a.cache_ld = cache_ld;
  a.num_slots = num_slots;
  a.tokens = (int32_t)tokens;
  a.chunks = (int32_t)(width / 16);
  a.lane_bits = lane_bits_for(a.chunks);
  const int64_t tok_per_block = kThreads >> a.lane_bits;
  const dim3 grid((uint32_t)((tokens + tok_per_block - 1) / tok_per_block),
                  (uint32_t)((a.chunks + (1 << a.lane_bits) - 1) >> a.lane_bits),
                  value_scale ? 2u : 1u);
  switch (dt) {
    case NVFP4_F32:
      hipLaunchKernelGGL(kv_store_kernel<NVFP4_F32>, grid, dim3(kThreads), 0, stream, a);
      break;
    case NVFP4_BF16:
      hipLaunchKernelGGL(kv_store_kernel<NVFP4_BF16>, grid, dim3(kThreads), 0, stream, a);
      break;
    default:
      hipLaunchKernelGGL(kv_store_kernel<NVFP4_F16>, grid, dim3(kThreads), 0, stream, a);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_kv_load(const uint8_t* cache, int64_t num_slots, int64_t cache_ld,
                          int64_t width, const float* scale, const int64_t* slots, int64_t tokens,
                          void* out, nvfp4_dtype out_dt, int64_t ld_out, hipStream_t stream) {
  KvLoadArgs a{};
  a.cache = cache;
  a.cache_ld = cache_ld;
  a.num_slots = num_slots;
  a.scale = scale;
  a.slots = slots;
  a.out = static_cast<uint8_t*>(out);
  a.ld_out = ld_out * (out_dt == NVFP4_F32 ? 4 : 2);
  a.tokens = (int32_t)tokens;
  a.pieces = (int32_t)(width / (out_dt == NVFP4_BF16 ? kLoadElems<true> : kLoadElems<false>));
  a.lane_bits = lane_bits_for(a.pieces);
  const int64_t tok_per_block = 2 * (kThreads >> a.lane_bits);
  const dim3 grid((uint32_t)((tokens + tok_per_block - 1) / tok_per_block),
                  (uint32_t)((a.pieces + (1 << a.lane_bits) - 1) >> a.lane_bits), 1u);
  if (out_dt == NVFP4_BF16)
    hipLaunchKernelGGL(kv_load_kernel<true>, grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(kv_load_kernel<false>, grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace nvfp4
