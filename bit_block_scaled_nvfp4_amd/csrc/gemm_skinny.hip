// W4A4 NVFP4 product for decode-shaped problems (M <= 16 activation rows), gfx950.
//
// Source: "Why Gated DeltaNet Survives 4-Bit Quantization" (arXiv 2609.04098), ai.info summary,
// "Main Findings": decode is weight-bandwidth-bound, so the work here is streaming the NVFP4
// weights once at HBM rate while the few activation rows ride along.
//
// Work split.  One workgroup per compute unit: workgroup b owns the `ncols` output columns
// [b * ncols, (b + 1) * ncols) -- ncols = ceil(N / compute units), so every compute unit streams the
// same number of weight bytes -- as T = 1 or 2 MFMA tiles of 16 columns (the second tile may be
// partly empty), plus all M <= 16 activation rows.  K is cut into phases of 1024 and each phase
// into 8 chunks of 128 (64 code bytes of a row); each wavefront owns one chunk of every phase.
// Phases go in pairs, and in a pair wavefront w owns chunks 2w and 2w + 1 of the pair's 16, so its
// loads of one row in the two phases fill the two halves of one 128-byte line (an unpaired last
// phase keeps chunk q * 8 + w): half as many cache lines touched per wavefront as with one chunk
// per wavefront in each phase's 512 bytes.
//
// Every lane loads exactly the bytes it feeds to the MFMA: in a 16x16x32 MFMA, lane l supplies
// row/column r = l % 16 and 8 of the 32 k-slots (group g = l / 16); within a chunk of 128, lane
// group g uses the 16 bytes holding elements [32g, 32g + 32) of its row, 32-bit word j of them in
// MFMA step j (j = 0..3), inside 16-blocks 2g and 2g + 1 (two scale bytes).  Both operands use this
// map.  So a wavefront's weight load of one tile and phase reads 16 rows x 64 contiguous bytes,
// straight into registers: no LDS staging and no workgroup barrier while the weights stream.  The
// weight scales are loaded 8 bytes per lane (a wavefront's chunk of one row holds the scale bytes
// of all four k groups): lane (r, g) loads those of phases g and 4 + g, and each lane then fetches
// phase q's word from lane (q % 4) * 16 + r with a cross-lane permute, so a tile's scales take one
// or two load instructions instead of one per phase.  Up to 8 phases, all loads of the launch are
// issued up front, the activation's first (small, and the same for every workgroup, so served from
// L2), then the weight scales, then the weight codes phase by phase; the activation fragments of
// all phases are decoded to f16 while the weights are in flight, so once phase q's weights land
// only their decode and the MFMAs remain.  Longer K streams through registers a fixed number of
// phases ahead (gemm_skinny_long_kernel).  Rows of the activation at or past M are zero.
//
// Activation input.  Either its NVFP4 codes and scales (the product alone), or the raw activation
// (f32, bf16 or f16) with its static global scale: then every wavefront first encodes exactly the
// blocks its own fragments need (its chunk of every phase, all M rows) with the encoder's block
// routine (bit-identical codes and scales) into its own LDS area, and the lanes read their
// fragments back -- no workgroup barrier; the wavefronts of workgroup 0 write their blocks out for
// the caller after their MFMAs.  That makes a decode step's activation encode and product one
// launch.  The raw blocks of a wavefront (M * NPH * 8 of them, at most 256) are loaded in one batch
// before the weights: a load issued after the weight loads could only be waited for together with
// all of them (the load counter drains in issue order), which would hold every decode and MFMA
// back until the wavefront's last weight byte had landed.
//
// Reduction: the 8 wavefronts' partial 16x16 tiles of each tile are summed through LDS in a fixed
// order (deterministic), scaled per column by 1 / (gA * gW[seg(n)]) and stored.  Every output
// element is accumulated the same way whichever workgroup and tile slot its column falls in.
#include <utility>

#include "codec.h"
#include "gemm_common.h"

namespace nvfp4 {
namespace {

constexpr int kSkinnyWaves = 8;
constexpr int kSkinnyThreads = kSkinnyWaves * 64;
constexpr int kPhaseK = 1024;  // K elements per phase (8 chunks of 128, one per wavefront)

typedef float floatx4_t __attribute__((ext_vector_type(4)));

// Raw activation input of the encoding form (null `x`: the activation comes encoded in GemmArgs).
struct DecodeEncode {
  const void* x;
  int64_t ldx;      // elements per row of x
  uint8_t* codes;   // the activation's codes and scales, written by workgroup 0 (row pitch K/2, K/16)
  uint8_t* scales;
};

// 16-byte and 8-byte loads of one lane's fragment bytes.
__device__ __forceinline__ uint4 load16(const uint8_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ uint2 load8(const uint8_t* p) { return *reinterpret_cast<const uint2*>(p); }

// Chunk of K (128 elements, 64 code bytes of a row) that wavefront w owns in phase q.  Phases go
// in pairs, and in a pair wavefront w owns chunks 2w and 2w + 1 of the pair's 16, so its loads of
// one row in the two phases fill the two halves of one 128-byte line; an unpaired last phase keeps
// chunk q * 8 + w.  Activation and weights use the same map, so every k is contracted once.
template <int NPH>
__device__ __forceinline__ int chunk_of(int q, int w) {
  constexpr int kPaired = NPH - NPH % 2;
  return q < kPaired ? (q / 2) * 16 + 2 * w + (q % 2) : q * 8 + w;
}

// An empty asm that takes and returns the value in registers: arithmetic on a loaded value stays
// behind the point where this is called.
__device__ __forceinline__ void pin(uint32_t& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void pin(uint2& v) {
  pin(v.x);
  pin(v.y);
}
__device__ __forceinline__ void pin(uint4& v) {
  pin(v.x);
  pin(v.y);
  pin(v.z);
  pin(v.w);
}

// Phase q's two scale bytes of lane (r, g) (low half of the result), from the 8-byte scale words
// that lanes (r, g') loaded for phases g' and 4 + g': lane (q % 4) * 16 + r holds them.
__device__ __forceinline__ uint32_t pick_scales(uint2 v, int q, int r, int g) {
  const int src = ((q & 3) * 16 + r) * 4;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)v.x);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)v.y);
  return ((g & 2) ? hi : lo) >> ((g & 1) * 16);
}

// The encoding form's activation loads: kEncodeBatch blocks per lane (so at most 256 blocks per
// wavefront: M * NPH <= 32), 32-bit words per block.
constexpr int kEncodeBatch = 4;
template <nvfp4_dtype XDT>
constexpr int encode_words() {
  return 4 * codec::elem_bytes<XDT>();
}

// The blocks a wavefront encodes are exactly those its fragments need: block b of its M * NPH * 8
// is row b / (8 NPH), phase (b / 8) % NPH, block b % 8 of the wavefront's chunk of that phase.
template <int NPH>
__device__ __forceinline__ void wave_block(int b, int wave, int& row, int& col) {
  row = b / (NPH * 8);
  const int rem = b - row * (NPH * 8);
  col = chunk_of<NPH>(rem >> 3, wave) * 128 + (rem & 7) * 16;  // element offset within the row
}

// Load this wavefront's blocks j * 64 + lane, j < kEncodeBatch (clamped to its last block), of the
// raw activation into registers.
template <nvfp4_dtype XDT, int NPH>
__device__ __forceinline__ void encode_load(const GemmArgs& p, const DecodeEncode& e, int wave,
                                            int lane,
                                            uint32_t (&raw)[kEncodeBatch][encode_words<XDT>()]) {
  constexpr int W = encode_words<XDT>();
  const int nblk = p.M * NPH * 8;
  const uint8_t* const xb = reinterpret_cast<const uint8_t*>(e.x);
#pragma unroll
  for (int j = 0; j < kEncodeBatch; ++j) {
    int row, col;
    wave_block<NPH>(min(j * 64 + lane, nblk - 1), wave, row, col);
    const uint8_t* src = xb + ((int64_t)row * e.ldx + col) * codec::elem_bytes<XDT>();
#pragma unroll
    for (int i = 0; i < W / 4; ++i) {
      const uint4 v = *reinterpret_cast<const uint4*>(src + 16 * i);
      raw[j][4 * i] = v.x;
      raw[j][4 * i + 1] = v.y;
      raw[j][4 * i + 2] = v.z;
      raw[j][4 * i + 3] = v.w;
    }
  }
}

// Encode this wavefront's blocks of the activation (`raw`, all of them) with the static scale g and
// the encoder's block routine into its own LDS area (codes [row][phase][64 bytes of its chunk],
// scales [row][phase][8]), spread over its 64 lanes.  No other wavefront reads the area, so no
// barrier is needed: the wavefront's LDS accesses complete in order.
template <nvfp4_dtype XDT, int NPH>
__device__ __forceinline__ void encode_activation(const GemmArgs& p, float g, int lane,
                                                  const uint32_t (&raw)[kEncodeBatch][encode_words<XDT>()],
                                                  uint8_t* lcodes, uint8_t* lscales) {
  const float gs6 = g / 6.0f;
  const int nblk = p.M * NPH * 8;
#pragma unroll
  for (int j = 0; j < kEncodeBatch; ++j) {
    const int b = j * 64 + lane;
    if (b >= nblk) continue;
    float v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if constexpr (XDT == NVFP4_F32) {
        v[i] = __uint_as_float(raw[j][i]);
      } else if constexpr (XDT == NVFP4_BF16) {
        const uint32_t w2 = raw[j][i / 2];
        v[i] = __uint_as_float((i & 1) ? (w2 & 0xFFFF0000u) : (w2 << 16));
      } else {
        const uint32_t w2 = raw[j][i / 2];
        v[i] = (float)__builtin_bit_cast(_Float16, (uint16_t)((i & 1) ? (w2 >> 16) : (w2 & 0xFFFFu)));
      }
    }
    uint32_t word[2];
    const uint32_t sc = codec::encode_codes(v, g, gs6, word);
    *reinterpret_cast<uint2*>(lcodes + b * 8) = uint2{word[0], word[1]};
    lscales[b] = (uint8_t)sc;
  }
}

// The wavefront's encoded blocks (its LDS area), written out to `e`: the wavefronts of workgroup 0
// together write the whole encoded activation.
template <int NPH>
__device__ __forceinline__ void write_encoded(const GemmArgs& p, const DecodeEncode& e, int wave,
                                              int lane, const uint8_t* lcodes,
                                              const uint8_t* lscales) {
  const int nblk = p.M * NPH * 8;
  for (int b = lane; b < nblk; b += 64) {
    int row, col;
    wave_block<NPH>(b, wave, row, col);
    *reinterpret_cast<uint2*>(e.codes + (int64_t)row * (p.K / 2) + col / 2) =
        *reinterpret_cast<const uint2*>(lcodes + b * 8);
    e.scales[(int64_t)row * (p.K / 16) + col / 16] = lscales[b];
  }
}

// K = NPH * 1024, T tiles of 16 columns, XDT = the raw activation's type in the encoding form
// (NVFP4_F32 / BF16 / F16) or -1 when the activation comes encoded; ASPREAD: the encoded
// activation has more than 4 rows (how its scales are loaded, below).
template <int NPH, int T, int XDT, bool ASPREAD>
__global__ void __launch_bounds__(kSkinnyThreads)
gemm_skinny_kernel(GemmArgs p, DecodeEncode e, int ncols) {
  constexpr bool kEncode = XDT >= 0;
  __shared__ floatx4_t partial[T][kSkinnyWaves][64];
  // the encoded activation (encoding form only): codes [M][K/2], scales [M][K/16]
  // the encoded activation, each wavefront's own blocks (encoding form only): codes
  // [row][phase][64], then scales [row][phase][8], for up to 16 rows
  __shared__ __attribute__((aligned(16))) uint8_t act[kSkinnyWaves][kEncode ? 16 * NPH * 72 : 16];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15;  // weight row (output column) and activation row of this lane
  const int g = lane >> 4;  // k group
  const int c0 = blockIdx.x * ncols;
  const int cend = min(c0 + ncols, p.N);
  const int clast = cend - 1;
  const bool arow_valid = r < p.M;
  const int64_t kb = p.k_pitch / 2, ks = p.k_pitch / 16;
  // byte offsets of this lane's 16 code bytes and 2 scale bytes within a row, for phase q:
  // chunk c = q * 8 + wave, codes at c * 64 + g * 16, scales at c * 8 + g * 2

  // activation fragments (encoded form: straight from global memory, L2-resident after the first
  // workgroup); rows >= M load the last row and are zeroed at decode
  const int arow = min(r, p.M - 1);
  uint4 aq[NPH];
  uint32_t as2[NPH];
  constexpr int kSq = (NPH + 3) / 4;  // 8-byte scale loads per row (phases g and 4 + g, see below)
  uint2 asq[kSq];
  // the activation's scales: with at most 4 rows most lanes share a row and one 2-byte load per
  // phase is cheapest; with more rows, 8-byte loads and the cross-lane pick used for the weights
  if constexpr (!kEncode) {
#pragma unroll
    for (int q = 0; q < NPH; ++q) aq[q] = load16(p.a_codes + arow * kb + chunk_of<NPH>(q, wave) * 64 + g * 16);
    if constexpr (ASPREAD) {
#pragma unroll
      for (int i = 0; i < kSq; ++i)
        asq[i] = load8(p.a_scales + arow * ks + chunk_of<NPH>(min(4 * i + g, NPH - 1), wave) * 8);
    } else {
#pragma unroll
      for (int q = 0; q < NPH; ++q)
        as2[q] = *reinterpret_cast<const uint16_t*>(p.a_scales + arow * ks + chunk_of<NPH>(q, wave) * 8 + g * 2);
    }
  }
  // encoding form: the activation's global scale and raw blocks, loaded before any weight load so
  // that the encode waits only for them
  constexpr nvfp4_dtype kXdt = kEncode ? (nvfp4_dtype)XDT : NVFP4_BF16;
  float enc_g = 0.0f;
  uint32_t enc_raw[kEncodeBatch][encode_words<kXdt>()];
  if constexpr (kEncode) {
    enc_g = __builtin_nontemporal_load(p.a_g);
    encode_load<kXdt, NPH>(p, e, wave, lane, enc_raw);
  }
  __builtin_amdgcn_sched_barrier(0);
  // weight scales of every phase, then the weight codes phase by phase (rows past the workgroup's
  // columns load its last column, never stored)
  int wrow[T];
#pragma unroll
  for (int t = 0; t < T; ++t) wrow[t] = min(c0 + t * 16 + r, clast);
  // weight scales: lane (r, g) loads the 8 scale bytes of this wavefront's chunk of row r (those of
  // all four k groups) for phases g and 4 + g, so one load per tile covers four phases; each lane
  // later fetches phase q's bytes from lane (q % 4) * 16 + r and keeps its own two
  uint2 sq[kSq][T];
#pragma unroll
  for (int i = 0; i < kSq; ++i)
#pragma unroll
    for (int t = 0; t < T; ++t)
      sq[i][t] = load8(p.w_scales + wrow[t] * ks + chunk_of<NPH>(min(4 * i + g, NPH - 1), wave) * 8);
  __builtin_amdgcn_sched_barrier(0);
  uint4 wq[NPH][T];
#pragma unroll
  for (int q = 0; q < NPH; ++q) {
#pragma unroll
    for (int t = 0; t < T; ++t) wq[q][t] = load16(p.w_codes + wrow[t] * kb + chunk_of<NPH>(q, wave) * 64 + g * 16);
    __builtin_amdgcn_sched_barrier(0);  // keep the phases' loads in phase order
  }
  // global scales for the epilogue factors 1 / (gA * gW[seg(n)]), used only at the end
  const float ga = p.a_g[0];
  float gw[T];
#pragma unroll
  for (int t = 0; t < T; ++t) gw[t] = p.seg_g[column_segment(p.seg, wrow[t])];
  __builtin_amdgcn_sched_barrier(0);

  if constexpr (kEncode) {
    uint8_t* const lcodes = act[wave];
    uint8_t* const lscales = act[wave] + 16 * NPH * 64;
    encode_activation<kXdt, NPH>(p, enc_g, lane, enc_raw, lcodes, lscales);
#pragma unroll
    for (int q = 0; q < NPH; ++q) {
      aq[q] = *reinterpret_cast<const uint4*>(lcodes + (arow * NPH + q) * 64 + g * 16);
      as2[q] = *reinterpret_cast<const uint16_t*>(lscales + (arow * NPH + q) * 8 + g * 2);
    }
  }

  if constexpr (!kEncode) {
    if constexpr (ASPREAD) {
#pragma unroll
      for (int q = 0; q < NPH; ++q) as2[q] = pick_scales(asq[q >> 2], q, r, g);
    }
  }

  // decode every phase's activation fragment (the weights are still streaming in)
  const uint32_t keep = arow_valid ? 0xFFFFFFFFu : 0u;  // padded rows contribute zeros
  half8_t av[NPH][4];
#pragma unroll
  for (int q = 0; q < NPH; ++q) {
    const half2_t sa = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(as2[q] & keep, 1.0f, false);
    const uint32_t w4[4] = {aq[q].x & keep, aq[q].y & keep, aq[q].z & keep, aq[q].w & keep};
#pragma unroll
    for (int j = 0; j < 4; ++j) av[q][j] = decode8(w4[j], j < 2 ? sa[0] : sa[1]);
  }

  // this lane's two weight scale bytes of every phase and tile (low half of ws2)
  uint32_t ws2[NPH][T];
#pragma unroll
  for (int q = 0; q < NPH; ++q)
#pragma unroll
    for (int t = 0; t < T; ++t) ws2[q][t] = pick_scales(sq[q >> 2][t], q, r, g);

  floatx4_t acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int q = 0; q < NPH; ++q) {
    // phase q's weights: decode and contract (the compiler waits for exactly these loads)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const half2_t sw = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(ws2[q][t], 1.0f, false);
      const uint32_t w4[4] = {wq[q][t].x, wq[q][t].y, wq[q][t].z, wq[q][t].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const half8_t bv = decode8(w4[j], j < 2 ? sw[0] : sw[1]);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[q][j], bv, acc[t], 0, 0, 0);
      }
    }
  }

  // the encoded activation out for the caller, after every weight load has been waited for
  if constexpr (kEncode) {
    if (blockIdx.x == 0 && e.codes != nullptr)
      write_encoded<NPH>(p, e, wave, lane, act[wave], act[wave] + 16 * NPH * 64);
  }

  // deterministic reduction of the 8 partial tiles of each tile: wavefront `tile` adds the 8 in
  // order
#pragma unroll
  for (int t = 0; t < T; ++t) partial[t][wave][lane] = acc[t];
  __syncthreads();
  if (wave >= T) return;
  floatx4_t sum = partial[wave][0][lane];
#pragma unroll
  for (int w = 1; w < kSkinnyWaves; ++w) sum += partial[wave][w][lane];

  // output tile `wave`: lane holds column c0 + 16 * wave + (l % 16), rows 4 * (l / 16) + e
  const int n = c0 + wave * 16 + r;
  if (n >= cend) return;
  const float al = 1.0f / (ga * (wave == 0 ? gw[0] : gw[T - 1]));
#pragma unroll
  for (int e4 = 0; e4 < 4; ++e4) {
    const int m = 4 * g + e4;
    if (m < p.M) store_c(p.c, p.c_bf16, p.ldc, m, n, sum[e4] * al);
  }
}

// Long-K form of the product (K = NPH * 1024 above the one-pass kernel's 8 phases): the same work
// split, fragments and scale loads, but the loads stream through registers D phases ahead instead of
// all being issued at once, each phase's activation fragment is decoded when its phase comes, and
// the weight codes arrive as whole cache lines that the wavefront rearranges into fragments through
// its own LDS area (below).
// Phase q's loads (activation codes and scales, then the weights' scale group when q % 4 == 0, then
// the weight codes) are issued right after phase q - D has been contracted, so D phases' bytes are
// always in flight and the register footprint is that of D phases.  Every index is a compile-time
// constant (the phase loop is unrolled), so each wait is for exactly the phase it needs.
template <int NPH, int T, bool ASPREAD, int D>
__global__ void __launch_bounds__(kSkinnyThreads)
gemm_skinny_long_kernel(GemmArgs p, int ncols) {
  __shared__ floatx4_t partial[T][kSkinnyWaves][64];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15;
  const int g = lane >> 4;
  const int c0 = blockIdx.x * ncols;
  const int cend = min(c0 + ncols, p.N);
  const int clast = cend - 1;
  const int64_t kb = p.k_pitch / 2, ks = p.k_pitch / 16;
  const int arow = min(r, p.M - 1);
  const uint32_t keep = r < p.M ? 0xFFFFFFFFu : 0u;  // padded activation rows contribute zeros
  int wrow[T];
#pragma unroll
  for (int t = 0; t < T; ++t) wrow[t] = min(c0 + t * 16 + r, clast);
  const uint8_t* const ac = p.a_codes + arow * kb + g * 16;
  const uint8_t* const asb = p.a_scales + arow * ks;

  // Weight codes of a phase pair come as whole 128-byte lines: the load of the pair's first phase
  // brings rows 0..7 of the tile and that of its second rows 8..15, lane L holding piece L % 8 of
  // row L / 8; at the pair's first phase each lane writes its piece to the wavefront's LDS area
  // (piece h of row r at slot h ^ (r % 8) ^ (r / 8): conflict-free writes and reads) and reads back
  // its fragments of both phases.  An unpaired last phase loads its fragments directly.
  constexpr int kPaired = NPH - NPH % 2;
  __shared__ __attribute__((aligned(16))) uint8_t xpose[kSkinnyWaves][T * 2048];
  int lrow[T][2];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int i = 0; i < 2; ++i) lrow[t][i] = min(c0 + t * 16 + 8 * i + (lane >> 3), clast);
  const int wslot0 = (lane >> 3) * 128 + (((lane & 7) ^ (lane >> 3)) * 16);
  const int wslot1 = 1024 + (lane >> 3) * 128 + (((lane & 7) ^ (lane >> 3) ^ 1) * 16);
  const int r8 = r & 7, ri = r >> 3;
  const int rslot0 = ri * 1024 + r8 * 128 + ((g ^ r8 ^ ri) * 16);
  const int rslot1 = ri * 1024 + r8 * 128 + (((4 + g) ^ r8 ^ ri) * 16);
  uint8_t* const xw = xpose[wave];

  constexpr int kSq = (NPH + 3) / 4;
  uint4 aq[NPH];
  uint32_t as2[NPH];
  uint2 asq[kSq];
  uint2 sq[kSq][T];
  uint4 wq[NPH][T];
  uint4 wodd[T];  // the fragments of a pair's second phase, read with the first's
  auto issue = [&](int q) {
    aq[q] = load16(ac + chunk_of<NPH>(q, wave) * 64);
    if constexpr (ASPREAD) {
      if (q % 4 == 0) asq[q / 4] = load8(asb + chunk_of<NPH>(min(q + g, NPH - 1), wave) * 8);
    } else {
      // the aligned word holding this lane's two scale bytes (shifted out at use)
      as2[q] = *reinterpret_cast<const uint32_t*>(asb + chunk_of<NPH>(q, wave) * 8 + (g >> 1) * 4);
    }
    if (q % 4 == 0) {
#pragma unroll
      for (int t = 0; t < T; ++t)
        sq[q / 4][t] = load8(p.w_scales + wrow[t] * ks + chunk_of<NPH>(min(q + g, NPH - 1), wave) * 8);
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
      if (q < kPaired) {
        // whole lines: rows 8 (q % 2) .. + 7 of the tile, the wavefront's 128 bytes of the pair
        wq[q][t] = load16(p.w_codes + lrow[t][q % 2] * kb + (q / 2) * 1024 + wave * 128 + (lane & 7) * 16);
      } else {
        wq[q][t] = load16(p.w_codes + wrow[t] * kb + chunk_of<NPH>(q, wave) * 64 + g * 16);
      }
    }
  };

#pragma unroll
  for (int q = 0; q < D; ++q) {
    issue(q);
    __builtin_amdgcn_sched_barrier(0);  // keep the phases' loads in phase order
  }
  const float ga = p.a_g[0];
  float gw[T];
#pragma unroll
  for (int t = 0; t < T; ++t) gw[t] = p.seg_g[column_segment(p.seg, wrow[t])];
  __builtin_amdgcn_sched_barrier(0);

  floatx4_t acc[T];
#pragma unroll
  for (int t = 0; t < T; ++t) acc[t] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int q = 0; q < NPH; ++q) {
    // phase q: the activation fragment, then the weights (the compiler waits for exactly these).
    // Its loaded words pass through an empty asm first, so no arithmetic on them is hoisted into
    // the prologue, where it would wait for phases still streaming in.
    if constexpr (ASPREAD) {
      if (q % 4 == 0) pin(asq[q / 4]);
    } else {
      pin(as2[q]);
    }
    pin(aq[q]);
    if (q % 4 == 0) {
#pragma unroll
      for (int t = 0; t < T; ++t) pin(sq[q / 4][t]);
    }
    uint4 wf[T];
    if (q < kPaired && q % 2 == 0) {
      // the pair's lines through the LDS area into fragments of both phases
#pragma unroll
      for (int t = 0; t < T; ++t) {
        pin(wq[q][t]);
        pin(wq[q + 1][t]);
        *reinterpret_cast<uint4*>(xw + t * 2048 + wslot0) = wq[q][t];
        *reinterpret_cast<uint4*>(xw + t * 2048 + wslot1) = wq[q + 1][t];
        wf[t] = *reinterpret_cast<const uint4*>(xw + t * 2048 + rslot0);
        wodd[t] = *reinterpret_cast<const uint4*>(xw + t * 2048 + rslot1);
      }
    } else if (q < kPaired) {
#pragma unroll
      for (int t = 0; t < T; ++t) wf[t] = wodd[t];
    } else {
#pragma unroll
      for (int t = 0; t < T; ++t) {
        pin(wq[q][t]);
        wf[t] = wq[q][t];
      }
    }
    const uint32_t sa_bits = ASPREAD ? pick_scales(asq[q / 4], q, r, g) : as2[q] >> ((g & 1) * 16);
    const half2_t sa = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sa_bits & keep, 1.0f, false);
    const uint32_t a4[4] = {aq[q].x & keep, aq[q].y & keep, aq[q].z & keep, aq[q].w & keep};
    half8_t av[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) av[j] = decode8(a4[j], j < 2 ? sa[0] : sa[1]);
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const half2_t sw =
          __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(pick_scales(sq[q / 4][t], q, r, g), 1.0f, false);
      const uint32_t w4[4] = {wf[t].x, wf[t].y, wf[t].z, wf[t].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const half8_t bv = decode8(w4[j], j < 2 ? sw[0] : sw[1]);
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[j], bv, acc[t], 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (q + D < NPH) issue(q + D);
    __builtin_amdgcn_sched_barrier(0);
  }

  // deterministic reduction of the 8 partial tiles of each tile, as in the one-pass kernel
#pragma unroll
  for (int t = 0; t < T; ++t) partial[t][wave][lane] = acc[t];
  __syncthreads();
  if (wave >= T) return;
  floatx4_t sum = partial[wave][0][lane];
#pragma unroll
  for (int w = 1; w < kSkinnyWaves; ++w) sum += partial[wave][w][lane];
  const int n = c0 + wave * 16 + r;
  if (n >= cend) return;
  const float al = 1.0f / (ga * (wave == 0 ? gw[0] : gw[T - 1]));
#pragma unroll
  for (int e4 = 0; e4 < 4; ++e4) {
    const int m = 4 * g + e4;
    if (m < p.M) store_c(p.c, p.c_bf16, p.ldc, m, n, sum[e4] * al);
  }
}

// Many-column form (more than 32 columns per compute unit, K up to kWideMaxPhases phases): the
// one-pass kernel's fragments, phase pairing, whole-line weight loads and scale loads, walking the
// workgroup's ncols columns as up to kWideMaxTiles tiles of 16.  The activation's fragments of all
// phases are decoded once and reused by every tile.  Tiles stream through registers kWideRing tiles
// ahead: tile t + kWideRing's loads are issued once tile t has been contracted, into the register
// set tile t used (the tile loop is unrolled over the ring, so every set is statically named and
// each wait is for exactly the tile it needs; the loads of tiles past the last repeat the last
// tile and are never used).  Each tile's 8 partial sums wait in LDS; after the last tile every
// wavefront reduces its share of the tiles in the one-pass kernel's fixed order, so every element
// is accumulated exactly as there.
constexpr int kWideMaxTiles = 16;
constexpr int kWideMaxPhases = 5;
constexpr int kWideRing = 2;

template <int NPH>
struct WideTile {
  uint4 w[NPH];              // weight codes (whole lines for paired phases)
  uint2 s[(NPH + 3) / 4];    // weight scale words (phases g and 4 + g)
};

template <int NPH, bool ASPREAD>
__global__ void __launch_bounds__(kSkinnyThreads)
gemm_skinny_wide_kernel(GemmArgs p, int ncols) {
  constexpr int kPaired = NPH - NPH % 2;
  constexpr int kSq = (NPH + 3) / 4;
  __shared__ floatx4_t partial[kWideMaxTiles][kSkinnyWaves][64];
  __shared__ __attribute__((aligned(16))) uint8_t xpose[kSkinnyWaves][2048];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15;
  const int g = lane >> 4;
  const int c0 = blockIdx.x * ncols;
  const int cend = min(c0 + ncols, p.N);
  const int clast = cend - 1;
  const int ntiles = (cend - c0 + 15) / 16;
  const int64_t kb = p.k_pitch / 2, ks = p.k_pitch / 16;
  const int arow = min(r, p.M - 1);
  const uint32_t keep = r < p.M ? 0xFFFFFFFFu : 0u;

  // the activation, loaded first (the same for every workgroup, so served from L2)
  uint4 aq[NPH];
  uint32_t as2[NPH];
  uint2 asq[kSq];
#pragma unroll
  for (int q = 0; q < NPH; ++q) aq[q] = load16(p.a_codes + arow * kb + chunk_of<NPH>(q, wave) * 64 + g * 16);
  if constexpr (ASPREAD) {
#pragma unroll
    for (int i = 0; i < kSq; ++i)
      asq[i] = load8(p.a_scales + arow * ks + chunk_of<NPH>(min(4 * i + g, NPH - 1), wave) * 8);
  } else {
#pragma unroll
    for (int q = 0; q < NPH; ++q)
      as2[q] = *reinterpret_cast<const uint16_t*>(p.a_scales + arow * ks + chunk_of<NPH>(q, wave) * 8 + g * 2);
  }
  __builtin_amdgcn_sched_barrier(0);

  auto issue_tile = [&](int t, WideTile<NPH>& L) {
    const int base = c0 + min(t, ntiles - 1) * 16;
    const int wrow = min(base + r, clast);
#pragma unroll
    for (int i = 0; i < kSq; ++i)
      L.s[i] = load8(p.w_scales + wrow * ks + chunk_of<NPH>(min(4 * i + g, NPH - 1), wave) * 8);
#pragma unroll
    for (int q = 0; q < NPH; ++q) {
      if (q < kPaired) {
        const int lrow = min(base + 8 * (q % 2) + (lane >> 3), clast);
        L.w[q] = load16(p.w_codes + lrow * kb + (q / 2) * 1024 + wave * 128 + (lane & 7) * 16);
      } else {
        L.w[q] = load16(p.w_codes + wrow * kb + chunk_of<NPH>(q, wave) * 64 + g * 16);
      }
    }
  };

  WideTile<NPH> ring[kWideRing];
#pragma unroll
  for (int k = 0; k < kWideRing; ++k) {
    issue_tile(k, ring[k]);
    __builtin_amdgcn_sched_barrier(0);
  }

  // the activation's fragments of every phase, decoded once (the weights are streaming in)
  if constexpr (ASPREAD) {
#pragma unroll
    for (int q = 0; q < NPH; ++q) as2[q] = pick_scales(asq[q >> 2], q, r, g);
  }
  half8_t av[NPH][4];
#pragma unroll
  for (int q = 0; q < NPH; ++q) {
    const half2_t sa = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(as2[q] & keep, 1.0f, false);
    const uint32_t a4[4] = {aq[q].x & keep, aq[q].y & keep, aq[q].z & keep, aq[q].w & keep};
#pragma unroll
    for (int j = 0; j < 4; ++j) av[q][j] = decode8(a4[j], j < 2 ? sa[0] : sa[1]);
  }

  const int wslot0 = (lane >> 3) * 128 + (((lane & 7) ^ (lane >> 3)) * 16);
  const int wslot1 = 1024 + (lane >> 3) * 128 + (((lane & 7) ^ (lane >> 3) ^ 1) * 16);
  const int r8 = r & 7, ri = r >> 3;
  const int rslot0 = ri * 1024 + r8 * 128 + ((g ^ r8 ^ ri) * 16);
  const int rslot1 = ri * 1024 + r8 * 128 + (((4 + g) ^ r8 ^ ri) * 16);
  uint8_t* const xw = xpose[wave];

  // contract tile t from register set L (when t is a real tile), leave its partial sums in LDS,
  // and load tile t + ring into L
  auto tile_step = [&](int t, WideTile<NPH>& L) {
    if (t < ntiles) {
#pragma unroll
      for (int i = 0; i < kSq; ++i) pin(L.s[i]);
      floatx4_t acc = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int q = 0; q < NPH; q += 2) {
        uint4 wf0, wf1;
        if (q < kPaired) {
          pin(L.w[q]);
          pin(L.w[q + 1]);
          *reinterpret_cast<uint4*>(xw + wslot0) = L.w[q];
          *reinterpret_cast<uint4*>(xw + wslot1) = L.w[q + 1];
          wf0 = *reinterpret_cast<const uint4*>(xw + rslot0);
          wf1 = *reinterpret_cast<const uint4*>(xw + rslot1);
        } else {
          pin(L.w[q]);
          wf0 = L.w[q];
          wf1 = wf0;
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int qq = q + h;
          if (qq < NPH) {
            const uint4 wf = h ? wf1 : wf0;
            const half2_t sw = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(
                pick_scales(L.s[qq / 4], qq, r, g), 1.0f, false);
            const uint32_t w4[4] = {wf.x, wf.y, wf.z, wf.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const half8_t bv = decode8(w4[j], j < 2 ? sw[0] : sw[1]);
              acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[qq][j], bv, acc, 0, 0, 0);
            }
          }
        }
      }
      partial[t][wave][lane] = acc;
    }
    __builtin_amdgcn_sched_barrier(0);
    issue_tile(t + kWideRing, L);
    __builtin_amdgcn_sched_barrier(0);
  };

  // whole rounds of the ring (steps past the last tile only refill, with the last tile's bytes)
  for (int t0 = 0; t0 < ntiles; t0 += kWideRing) {
#pragma unroll
    for (int k = 0; k < kWideRing; ++k) tile_step(t0 + k, ring[k]);
  }

  // every wavefront's loads have landed (the last refills repeat the last tile); reduce the tiles
  // in the fixed order of the one-pass kernel: wavefront w takes tiles w, w + 8, ...
  __syncthreads();
  const float ga = p.a_g[0];
  for (int t = wave; t < ntiles; t += kSkinnyWaves) {
    floatx4_t sum = partial[t][0][lane];
#pragma unroll
    for (int w = 1; w < kSkinnyWaves; ++w) sum += partial[t][w][lane];
    const int n = c0 + t * 16 + r;
    if (n < cend) {
      const float al = 1.0f / (ga * p.seg_g[column_segment(p.seg, n)]);
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int m = 4 * g + e4;
        if (m < p.M) store_c(p.c, p.c_bf16, p.ldc, m, n, sum[e4] * al);
      }
    }
  }
}

}  // namespace

namespace {

// One workgroup per compute unit: ncols = ceil(N / compute units) columns each (two tiles when
// that is more than 16), so every compute unit streams the same number of weight bytes.
template <int NPH, int XDT>
hipError_t launch_skinny_nph(const GemmArgs& a, const DecodeEncode& e, int cus, hipStream_t stream) {
  const dim3 block(kSkinnyThreads);
  const int per_cu = (a.N + cus - 1) / cus;
  // more than 4 encoded activation rows: the spread scale loads (the encoding form has none)
  constexpr bool kSpreadForm = XDT < 0;
  const bool spread = kSpreadForm && a.M > 4;
  const int ncols = per_cu > 16 ? (per_cu <= 32 ? per_cu : 32) : 16;
  const dim3 grid((a.N + ncols - 1) / ncols);
  if (per_cu > 16) {
    if (spread)
      hipLaunchKernelGGL((gemm_skinny_kernel<NPH, 2, XDT, kSpreadForm>), grid, block, 0, stream, a, e, ncols);
    else
      hipLaunchKernelGGL((gemm_skinny_kernel<NPH, 2, XDT, false>), grid, block, 0, stream, a, e, ncols);
  } else {
    if (spread)
      hipLaunchKernelGGL((gemm_skinny_kernel<NPH, 1, XDT, kSpreadForm>), grid, block, 0, stream, a, e, ncols);
    else
      hipLaunchKernelGGL((gemm_skinny_kernel<NPH, 1, XDT, false>), grid, block, 0, stream, a, e, ncols);
  }
  return hipGetLastError();
}

// Phases of K the one-launch encoding form takes for an f32 activation (its encode batches hold
// twice the registers of a 16-bit one's): at most 5.
constexpr int kEncodeF32MaxPhases = 5;

template <int XDT>
hipError_t launch_skinny_piece(const GemmArgs& a, const DecodeEncode& e, int cus, hipStream_t stream) {
  constexpr bool f32enc = XDT == NVFP4_F32;
  switch (a.K / kPhaseK) {
    case 1: return launch_skinny_nph<1, XDT>(a, e, cus, stream);
    case 2: return launch_skinny_nph<2, XDT>(a, e, cus, stream);
    case 3: return launch_skinny_nph<3, XDT>(a, e, cus, stream);
    case 4: return launch_skinny_nph<4, XDT>(a, e, cus, stream);
    case 5: return launch_skinny_nph<5, XDT>(a, e, cus, stream);
    case 6: return f32enc ? hipErrorInvalidValue : launch_skinny_nph<(f32enc ? 1 : 6), XDT>(a, e, cus, stream);
    case 7: return f32enc ? hipErrorInvalidValue : launch_skinny_nph<(f32enc ? 1 : 7), XDT>(a, e, cus, stream);
    case 8: return f32enc ? hipErrorInvalidValue : launch_skinny_nph<(f32enc ? 1 : 8), XDT>(a, e, cus, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int NPH>
hipError_t launch_skinny_wide_nph(const GemmArgs& a, int ncols, hipStream_t stream) {
  const dim3 grid((a.N + ncols - 1) / ncols), block(kSkinnyThreads);
  if (a.M > 4)
    hipLaunchKernelGGL((gemm_skinny_wide_kernel<NPH, true>), grid, block, 0, stream, a, ncols);
  else
    hipLaunchKernelGGL((gemm_skinny_wide_kernel<NPH, false>), grid, block, 0, stream, a, ncols);
  return hipGetLastError();
}

// More than 32 and at most 16 * kWideMaxTiles columns per compute unit, K up to kWideMaxPhases
// phases.
bool skinny_wide(const GemmArgs& a, int cus) {
  const int per_cu = (a.N + cus - 1) / cus;
  return per_cu > 32 && (per_cu + 15) / 16 <= kWideMaxTiles && a.K % kPhaseK == 0 &&
         a.K / kPhaseK <= kWideMaxPhases;
}

hipError_t launch_skinny_wide(const GemmArgs& a, int cus, hipStream_t stream) {
  const int ncols = (a.N + cus - 1) / cus;
  switch (a.K / kPhaseK) {
    case 1: return launch_skinny_wide_nph<1>(a, ncols, stream);
    case 2: return launch_skinny_wide_nph<2>(a, ncols, stream);
    case 3: return launch_skinny_wide_nph<3>(a, ncols, stream);
    case 4: return launch_skinny_wide_nph<4>(a, ncols, stream);
    case 5: return launch_skinny_wide_nph<5>(a, ncols, stream);
    default: return hipErrorInvalidValue;
  }
}

// Phases in flight in the long-K form.
constexpr int kLongDepth = 8;

template <int NPH>
hipError_t launch_skinny_long_nph(const GemmArgs& a, int cus, hipStream_t stream) {
  const dim3 block(kSkinnyThreads);
  const int per_cu = (a.N + cus - 1) / cus;
  const int ncols = per_cu > 16 ? per_cu : 16;
  const dim3 grid((a.N + ncols - 1) / ncols);
  constexpr int D = kLongDepth;
  if (per_cu > 16) {
    if (a.M > 4)
      hipLaunchKernelGGL((gemm_skinny_long_kernel<NPH, 2, true, D>), grid, block, 0, stream, a, ncols);
    else
      hipLaunchKernelGGL((gemm_skinny_long_kernel<NPH, 2, false, D>), grid, block, 0, stream, a, ncols);
  } else {
    if (a.M > 4)
      hipLaunchKernelGGL((gemm_skinny_long_kernel<NPH, 1, true, D>), grid, block, 0, stream, a, ncols);
    else
      hipLaunchKernelGGL((gemm_skinny_long_kernel<NPH, 1, false, D>), grid, block, 0, stream, a, ncols);
  }
  return hipGetLastError();
}

template <int... Q>
hipError_t launch_skinny_long_switch(const GemmArgs& a, int cus, hipStream_t stream,
                                     std::integer_sequence<int, Q...>) {
  hipError_t e = hipErrorInvalidValue;
  const int nph = (int)(a.K / kPhaseK);
  ((nph == Q + kSkinnyMaxK / kPhaseK + 1 ? (e = launch_skinny_long_nph<Q + kSkinnyMaxK / kPhaseK + 1>(a, cus, stream), 0) : 0), ...);
  return e;
}

// K above kSkinnyMaxK up to kStreamMaxK, at most 32 columns per compute unit.
hipError_t launch_skinny_long(const GemmArgs& a, int cus, hipStream_t stream) {
  return launch_skinny_long_switch(
      a, cus, stream, std::make_integer_sequence<int, (int)((kStreamMaxK - kSkinnyMaxK) / kPhaseK)>{});
}

hipError_t compute_units(int& cus) {
  int dev = 0;
  cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  cus = cus > 0 ? cus : 1;
  return e;
}

}  // namespace

// Rows up to which the encoding form runs: every workgroup encodes all M activation rows itself,
// so its encode work grows with M while a separate encode launch spreads it over the device.  On
// the 5120 x 5120 decode product one launch took 7.8 / 8.8 / 9.2 us at M = 1 / 4 / 6 against
// 9.0 / 9.5 / 9.7 us for encode + product as two launches (graph replays); an earlier form that
// could take more rows took 11.1 / 14.4 us at M = 8 / 16 against 9.9 / 10.0 us.
constexpr int64_t kEncodeMaxRows = 6;

// A wavefront's raw activation blocks (M * K / 128 of them) fit the one batch it loads before the
// weights.
static bool encode_fits_one_batch(int64_t M, int64_t K) {
  return M * (K / kPhaseK) * 8 <= kEncodeBatch * 64;
}

bool skinny_one_pass(int64_t M, int64_t N, int64_t K, int x_dtype) {
  int cus = 0;
  if (compute_units(cus) != hipSuccess) return false;
  if (x_dtype == NVFP4_F32 && K > kEncodeF32MaxPhases * kPhaseK) return false;
  return M >= 1 && M <= kEncodeMaxRows && K % kPhaseK == 0 && K <= kSkinnyMaxK &&
         encode_fits_one_batch(M, K) && (N + cus - 1) / cus <= 32;
}

hipError_t launch_gemm_skinny_encode(const GemmArgs& a, const void* x, nvfp4_dtype x_dtype,
                                     int64_t ldx, uint8_t* codes, uint8_t* scales,
                                     hipStream_t stream) {
  if (!encode_fits_one_batch(a.M, a.K)) return hipErrorInvalidValue;
  int cus = 0;
  hipError_t e = compute_units(cus);
  if (e != hipSuccess) return e;
  const DecodeEncode de{x, ldx, codes, scales};
  switch (x_dtype) {
    case NVFP4_F32: return launch_skinny_piece<NVFP4_F32>(a, de, cus, stream);
    case NVFP4_BF16: return launch_skinny_piece<NVFP4_BF16>(a, de, cus, stream);
    case NVFP4_F16: return launch_skinny_piece<NVFP4_F16>(a, de, cus, stream);
  }
  return hipErrorInvalidValue;
}

// Decode-shaped products.  Up to 32 columns per compute unit and K up to kSkinnyMaxK: the one-pass
// kernel; K up to kStreamMaxK: its long-K form.  More columns, up to 16 * kWideMaxTiles per compute
// unit with K up to kWideMaxPhases phases: the many-column form.  Other shapes with more columns:
// the streaming kernels (gemm_stream.hip), which stream weight copies through LDS.  K beyond
// kStreamMaxK (f32 output only): the streaming kernel on the fewest pieces of K of at most 8
// phases, as equal as possible; the first piece writes C and each later one, launched after it on
// the same stream, adds its scaled partial product: C = fl(...fl(acc_0 a) + acc_1 a ...).  The
// one-pass, long-K and many-column forms accumulate every element the same way as each other, the
// streaming kernels in another order (one chunk per wavefront in each phase), within the same
// tolerance.
hipError_t launch_gemm_skinny(const GemmArgs& a, hipStream_t stream) {
  int cus = 0;
  hipError_t e = compute_units(cus);
  if (e != hipSuccess) return e;
  const int per_cu = (a.N + cus - 1) / cus;
  if (a.K <= kSkinnyMaxK && per_cu <= 32)
    return launch_skinny_piece<-1>(a, DecodeEncode{nullptr, 0, nullptr, nullptr}, cus, stream);
  if (a.K <= kStreamMaxK && per_cu <= 32) return launch_skinny_long(a, cus, stream);
  if (skinny_wide(a, cus)) return launch_skinny_wide(a, cus, stream);
  if (a.K <= kStreamMaxK) return launch_gemm_stream(a, stream);
  const int phases = a.K / kPhaseK;
  const int pieces = (phases + 7) / 8;
  int k0 = 0;
  for (int i = 0; i < pieces; ++i) {
    const int nph = phases / pieces + (i < phases % pieces ? 1 : 0);
    GemmArgs b = a;
    b.a_codes = a.a_codes + k0 / 2;
    b.a_scales = a.a_scales + k0 / 16;
    b.w_codes = a.w_codes + k0 / 2;
    b.w_scales = a.w_scales + k0 / 16;
    b.K = nph * kPhaseK;
    b.k_pitch = a.K;
    b.c_accumulate = i > 0 ? 1 : 0;
    e = launch_gemm_stream(b, stream);
    if (e != hipSuccess) return e;
    k0 += b.K;
  }
  return hipSuccess;
}

}  // namespace nvfp4
