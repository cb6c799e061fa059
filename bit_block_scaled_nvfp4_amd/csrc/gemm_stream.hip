// W4A4 NVFP4 product for decode-shaped problems (M <= 16 activation rows) whose weight is too
// large for one pass of the skinny kernel: many output columns per compute unit or a long K.
// gfx950.
//
// Source: "Why Gated DeltaNet Survives 4-Bit Quantization" (arXiv 2609.04098), ai.info summary,
// "Main Findings": decode is weight-bandwidth-bound, so the weights stream once at HBM rate.
//
// Work split.  One persistent workgroup (8 wavefronts) per compute unit walks its tiles of 16
// output columns, b, b + G, b + 2G, ...  A tile's weight rows are consumed in units of one
// 1024-element K phase: 16 rows x 512 code bytes and 16 rows x 64 scale bytes.  Units stream
// through LDS slots while earlier units are computed, so the weight stream never waits for a tile
// boundary.  Three forms:
//  * K <= 8192 (gemm_stream_cached_kernel): every wavefront decodes its activation fragments of all
//    phases once and keeps them in registers; slots hold two tiles, unit (t + 1, q) is copied
//    while unit (t, q) is computed, two copies per unit.
//  * longer K, more than 16 columns per compute unit (gemm_stream_pair_kernel): equal column
//    ranges instead of tiles dealt round robin, two tiles per unit; described at the kernel.
// (Longer K with fewer columns per compute unit runs the skinny kernel's long-K form.)
// Every wavefront issues the same vector memory instructions per unit, so each wait is a
// compile-time vmcnt.
//
// Per unit each wavefront takes one eighth of the phase (128 elements) with the K-slot permutation
// and code-slot swizzle of the skinny kernel: lane (r, g) = (l % 16, l / 16) holds weight row r and
// activation row r, elements [32g, 32g + 32) of its 128, word j in MFMA step j of
// v_mfma_f32_16x16x32_f16.  At a tile's last unit the 8 partial 16x16 tiles are summed through
// LDS in a fixed order, scaled by 1 / (gA * gW[seg(n)]) from a table kept in LDS, and stored by
// wavefront 0: results are deterministic.
#include "gemm_common.h"

namespace nvfp4 {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kUnitK = 1024;         // K elements per unit
constexpr int kPieces = kUnitK / 32;               // 16-byte code pieces per row per unit (32)
constexpr int kCodeBytes = 16 * kPieces * 16;      // 8 KiB
constexpr int kScaleBytes = 16 * (kUnitK / 16);    // 16 rows x 64 bytes
constexpr int kSlotBytes = kCodeBytes + kScaleBytes;

typedef float floatx4_t __attribute__((ext_vector_type(4)));

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | (((N >> 4) & 3) << 14));
}

// wait_vmcnt with a count that loop unrolling makes constant: the switch folds to one wait (any
// other count waits for everything, which is always safe)
__device__ __forceinline__ void wait_vmcnt_folded(int n) {
  switch (n) {
    case 2: wait_vmcnt<2>(); break;
    case 4: wait_vmcnt<4>(); break;
    case 6: wait_vmcnt<6>(); break;
    case 8: wait_vmcnt<8>(); break;
    case 10: wait_vmcnt<10>(); break;
    case 12: wait_vmcnt<12>(); break;
    case 14: wait_vmcnt<14>(); break;
    default: wait_vmcnt<0>(); break;
  }
}

struct StreamArgs {
  GemmArgs p;
  int ntiles;  // ceil(N / 16)
  int nph;     // K / 1024
};

// The epilogue's global scales gW[0 .. nseg - 1] and gA into the LDS table, called once the first
// weight copies are in flight.  They are scalar loads, whose waits count scalar memory operations
// only (not the copies); the barrier before the first epilogue publishes the table.
__device__ __forceinline__ void stage_global_scales(const GemmArgs& p, float* gtab) {
  // read through the constant address space: the values were written by earlier launches and do not
  // change during this one, and such uniform loads are scalar loads wherever they sit (after the
  // copies a plain global load could not be proven unclobbered and would be a vector load)
  typedef const __attribute__((address_space(4))) float* const_f32_ptr;
  const const_f32_ptr sg = (const_f32_ptr)p.seg_g;
  const const_f32_ptr ag = (const_f32_ptr)p.a_g;
  float v[NVFP4_MAX_SEGMENTS + 1];
#pragma unroll
  for (int t = 0; t < NVFP4_MAX_SEGMENTS; ++t) v[t] = sg[min(t, p.seg.nseg - 1)];
  v[NVFP4_MAX_SEGMENTS] = ag[0];
  if (threadIdx.x == 0) {
#pragma unroll
    for (int t = 0; t <= NVFP4_MAX_SEGMENTS; ++t) gtab[t] = v[t];
  }
}

// K <= 8192 (NPH phases): the same stream with the activations decoded once.  Every tile reuses
// the activation fragments of the NPH phases, so each wavefront decodes its fragment of every
// phase before the stream starts and keeps it in registers (NPH x 16 VGPRs); a unit is then two
// copies and no activation work.  Slots hold two tiles (2 NPH, statically named): unit (t + 1, q)
// is copied into the slot of unit (t - 1, q) while unit (t, q) is computed, so NPH units are in
// flight, and with the tile loop unrolled by two every slot and phase index is a compile-time
// constant.
constexpr int kVmemPerUnitCached = 2;

__device__ __forceinline__ void issue_weights(const GemmArgs& p, int tile, int q, uint8_t* slot,
                                              int wave, int lane) {
  const int kb = p.k_pitch / 2, ks = p.k_pitch / 16;  // row pitches (a piece of K may be narrower)
  const int t = wave * 64 + lane;
  const int row = t / kPieces;
  const int jl = t - row * kPieces;
  const int j = (jl & ~15) | ((jl ^ row) & 15);
  const int grow = min(tile * 16 + row, p.N - 1);
  __builtin_amdgcn_global_load_lds(p.w_codes + (int64_t)grow * kb + q * (kUnitK / 2) + j * 16,
                                   slot + wave * 64 * 16, 16, 0, 0);
  const int ts = t & 255;
  const int srow = ts >> 4, dw = ts & 15;
  const int gsrow = min(tile * 16 + srow, p.N - 1);
  __builtin_amdgcn_global_load_lds(p.w_scales + (int64_t)gsrow * ks + q * (kUnitK / 16) + dw * 4,
                                   slot + kCodeBytes + (wave & 3) * 64 * 4, 4, 0, 0);
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ void compute_weights(const uint8_t* slot, const half8_t (&av)[4],
                                                int wave, int r, int g, floatx4_t& acc) {
  const int j = wave * 4 + g;
  const uint4 ww =
      *reinterpret_cast<const uint4*>(slot + (r * kPieces + ((j & ~15) | ((j ^ r) & 15))) * 16);
  const uint32_t ws2 = *reinterpret_cast<const uint16_t*>(slot + kCodeBytes + r * 64 + j * 2);
  const half2_t sw = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(ws2, 1.0f, false);
  const uint32_t wq[4] = {ww.x, ww.y, ww.z, ww.w};
#pragma unroll
  for (int s2 = 0; s2 < 4; ++s2) {
    const half8_t bv = decode8(wq[s2], s2 < 2 ? sw[0] : sw[1]);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[s2], bv, acc, 0, 0, 0);
  }
}

// End of tile t: fixed-order sum of the 8 wavefronts' partial tiles, scaled, stored by wavefront 0.
__device__ __forceinline__ void tile_epilogue(const GemmArgs& p, floatx4_t (&partial)[kWaves][64],
                                              const float* gtab, int tile, int wave, int lane,
                                              int r, int g, floatx4_t& acc) {
  partial[wave][lane] = acc;
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0) only: copies in flight are not waited for
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  if (wave == 0) {
    floatx4_t sum = partial[0][lane];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) sum += partial[w][lane];
    const int n = tile * 16 + r;
    if (n < p.N) {
      const float al = 1.0f / (gtab[NVFP4_MAX_SEGMENTS] * gtab[column_segment(p.seg, n)]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = 4 * g + e;
        if (m >= p.M) continue;
        if (p.c_accumulate)  // a later piece of a split K: f32 C, stream-ordered after the first
          reinterpret_cast<float*>(p.c)[(int64_t)m * p.ldc + n] += sum[e] * al;
        else
          store_c(p.c, p.c_bf16, p.ldc, m, n, sum[e] * al);
      }
    }
  }
  acc = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
}

// The last tile of gemm_stream_cached_kernel, held in slots PAR * NPH ...: no copies are issued, and
// the wait at step q leaves its NPH - 1 - q later units outstanding.
template <int NPH, int PAR>
__device__ __forceinline__ void cached_last_tile(const GemmArgs& p, uint8_t* const (&slot)[16],
                                                 const half8_t (&act)[NPH][4],
                                                 floatx4_t (&partial)[kWaves][64],
                                                 const float* gtab, int tile, int wave, int lane,
                                                 int r, int g, floatx4_t& acc) {
#pragma unroll
  for (int q = 0; q < NPH; ++q) {
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt_folded((NPH - 1 - q) * kVmemPerUnitCached);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    compute_weights(slot[PAR * NPH + q], act[q], wave, r, g, acc);
    if (q == NPH - 1) tile_epilogue(p, partial, gtab, tile, wave, lane, r, g, acc);
  }
}

template <int NPH>
__global__ void __launch_bounds__(kThreads) gemm_stream_cached_kernel(StreamArgs s) {
  static_assert(NPH >= 1 && NPH <= 8, "K up to 8192");
  constexpr int S = 2 * NPH;
#define NVFP4_SLOT(i) \
  __shared__ __attribute__((aligned(16))) uint8_t sl##i[(i) < S ? kSlotBytes : 16];
  NVFP4_SLOT(0) NVFP4_SLOT(1) NVFP4_SLOT(2) NVFP4_SLOT(3) NVFP4_SLOT(4) NVFP4_SLOT(5)
  NVFP4_SLOT(6) NVFP4_SLOT(7) NVFP4_SLOT(8) NVFP4_SLOT(9) NVFP4_SLOT(10) NVFP4_SLOT(11)
  NVFP4_SLOT(12) NVFP4_SLOT(13) NVFP4_SLOT(14) NVFP4_SLOT(15)
#undef NVFP4_SLOT
  uint8_t* const slot[16] = {sl0, sl1, sl2, sl3, sl4, sl5, sl6, sl7,
                             sl8, sl9, sl10, sl11, sl12, sl13, sl14, sl15};
  __shared__ floatx4_t partial[kWaves][64];
  __shared__ float gtab[NVFP4_MAX_SEGMENTS + 1];

  const GemmArgs& p = s.p;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const bool arow_valid = r < p.M;
  const int ksa = p.K / 16;
  const int my_tiles = (s.ntiles - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
  const int tile0 = (int)blockIdx.x, tstep = (int)gridDim.x;


  // (here the table is read first: issuing tile 0's copies before the activation work measured
  // slower in this form)
  if (threadIdx.x < p.seg.nseg) gtab[threadIdx.x] = p.seg_g[threadIdx.x];
  if (threadIdx.x == 0) gtab[NVFP4_MAX_SEGMENTS] = *p.a_g;

  // activation scales of all K staged in slot 0 (K / 16 <= 512 bytes per row, 16 rows), and this
  // lane's activation codes of every phase
  uint8_t* const asc = sl0;
  {
    const int per_row = ksa / 16;
    for (int i = threadIdx.x; i < p.M * per_row; i += kThreads) {
      const int row = i / per_row;
      __builtin_amdgcn_global_load_lds(
          p.a_scales + (int64_t)row * (p.k_pitch / 16) + (i - row * per_row) * 16,
          asc + (i & ~63) * 16, 16, 0, 0);
    }
  }
  uint4 aw[NPH];
  const int arow = min(r, p.M - 1);
#pragma unroll
  for (int q = 0; q < NPH; ++q)
    aw[q] = *reinterpret_cast<const uint4*>(p.a_codes + (int64_t)arow * (p.k_pitch / 2) +
                                            q * (kUnitK / 2) + wave * 64 + g * 16);
  wait_vmcnt<0>();
  __syncthreads();
  half8_t act[NPH][4];
  const uint32_t keep = arow_valid ? 0xFFFFFFFFu : 0u;
#pragma unroll
  for (int q = 0; q < NPH; ++q) {
    const int c = q * (kUnitK / 128) + wave;
    const uint32_t as2 = *reinterpret_cast<const uint16_t*>(asc + r * ksa + c * 8 + g * 2) & keep;
    const half2_t sa = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(as2, 1.0f, false);
    const uint32_t aq[4] = {aw[q].x & keep, aw[q].y & keep, aw[q].z & keep, aw[q].w & keep};
#pragma unroll
    for (int s2 = 0; s2 < 4; ++s2) act[q][s2] = decode8(aq[s2], s2 < 2 ? sa[0] : sa[1]);
  }
  __syncthreads();  // every wavefront has read the staged scales before slot 0 is reused

  // tile 0's units
#pragma unroll
  for (int q = 0; q < NPH; ++q) issue_weights(p, tile0, q, slot[q], wave, lane);

  floatx4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
  // every tile but the last: the next tile's units are copied during this one
  for (int i = 0; i < my_tiles - 1; i += 2) {
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      const int ti = i + par;
      if (ti >= my_tiles - 1) break;  // uniform over the workgroup
      const int tile = tile0 + ti * tstep;
#pragma unroll
      for (int q = 0; q < NPH; ++q) {
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<(NPH - 1) * kVmemPerUnitCached>();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        issue_weights(p, tile + tstep, q, slot[(1 - par) * NPH + q], wave, lane);
        compute_weights(slot[par * NPH + q], act[q], wave, r, g, acc);
        if (q == NPH - 1) tile_epilogue(p, partial, gtab, tile, wave, lane, r, g, acc);
      }
    }
  }
  // the last tile copies nothing: at its step q only its own later units are outstanding
  const int tl = my_tiles - 1;
  if (tl & 1)
    cached_last_tile<NPH, 1>(p, slot, act, partial, gtab, tile0 + tl * tstep, wave, lane, r, g, acc);
  else
    cached_last_tile<NPH, 0>(p, slot, act, partial, gtab, tile0 + tl * tstep, wave, lane, r, g, acc);
}

// Column-pair form (K beyond the cached form, more than 16 columns per compute unit when the
// columns are shared evenly).  Workgroup b owns the `ncols` columns [b ncols, (b + 1) ncols), ncols =
// ceil(N / compute units), so every compute unit streams the same number of weight bytes (tiles of
// 16 dealt round robin leave some compute units two tiles and others one when N / 16 is not a
// multiple of their count).  It walks them in groups of 32 columns (two tiles; rows past the last
// column repeat it and are never stored), and a unit is one K phase of a group: both tiles' codes
// and scales (18 KiB) and the activation fragment, which is decoded once for the two tiles.  Units
// stream through a ring of kPairRing statically named slots with kPairRing - 1 in flight (fewer
// slots measured faster here: 3 against 4 to 6).
constexpr int kPairRing = 3;
constexpr int kPairAhead = kPairRing - 1;
constexpr int kPairBytes = 2 * kCodeBytes + 2 * kScaleBytes;
constexpr int kVmemPerPair = 4;

struct PairArgs {
  GemmArgs p;
  int ncols;  // columns per workgroup
  int nph;    // K / 1024
};

__device__ __forceinline__ void issue_pair(const PairArgs& s, int cb, int clast, int q,
                                           uint8_t* slot, int wave, int lane, uint4& aw) {
  const GemmArgs& p = s.p;
  const int kb = p.k_pitch / 2, ks = p.k_pitch / 16;
  const int t = wave * 64 + lane;
  const int row = t / kPieces;
  const int jl = t - row * kPieces;
  const int j = (jl & ~15) | ((jl ^ row) & 15);
#pragma unroll
  for (int tile = 0; tile < 2; ++tile) {
    const int grow = min(cb + tile * 16 + row, clast);
    __builtin_amdgcn_global_load_lds(p.w_codes + (int64_t)grow * kb + q * (kUnitK / 2) + j * 16,
                                     slot + tile * kCodeBytes + wave * 64 * 16, 16, 0, 0);
  }
  // scale bytes of the 32 rows, 64 each: thread t copies dword t % 16 of row t / 16
  const int gsrow = min(cb + (t >> 4), clast);
  __builtin_amdgcn_global_load_lds(p.w_scales + (int64_t)gsrow * ks + q * (kUnitK / 16) + (t & 15) * 4,
                                   slot + 2 * kCodeBytes + wave * 64 * 4, 4, 0, 0);
  const int r = lane & 15, g = lane >> 4;
  const int arow = min(r, p.M - 1);
  aw = *reinterpret_cast<const uint4*>(p.a_codes + (int64_t)arow * kb + q * (kUnitK / 2) +
                                       wave * 64 + g * 16);
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ void compute_pair(const uint8_t* slot, const uint8_t* asc, int ksa,
                                             int q, int wave, int r, int g, bool arow_valid,
                                             const uint4& aw_in, floatx4_t (&acc)[2]) {
  const uint32_t keep = arow_valid ? 0xFFFFFFFFu : 0u;
  const uint32_t aq[4] = {aw_in.x & keep, aw_in.y & keep, aw_in.z & keep, aw_in.w & keep};
  const int c = q * (kUnitK / 128) + wave;
  const uint32_t as2 = *reinterpret_cast<const uint16_t*>(asc + r * ksa + c * 8 + g * 2) & keep;
  const half2_t sa = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(as2, 1.0f, false);
  const int j = wave * 4 + g;
  const int piece = (r * kPieces + ((j & ~15) | ((j ^ r) & 15))) * 16;
  uint4 ww[2];
  half2_t sw[2];
#pragma unroll
  for (int tile = 0; tile < 2; ++tile) {
    ww[tile] = *reinterpret_cast<const uint4*>(slot + tile * kCodeBytes + piece);
    const uint32_t ws2 =
        *reinterpret_cast<const uint16_t*>(slot + 2 * kCodeBytes + (tile * 16 + r) * 64 + j * 2);
    sw[tile] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(ws2, 1.0f, false);
  }
#pragma unroll
  for (int s2 = 0; s2 < 4; ++s2) {
    const half8_t av = decode8(aq[s2], s2 < 2 ? sa[0] : sa[1]);
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
      const uint32_t wq = s2 == 0 ? ww[tile].x : s2 == 1 ? ww[tile].y : s2 == 2 ? ww[tile].z
                                                                                   : ww[tile].w;
      const half8_t bv = decode8(wq, s2 < 2 ? sw[tile][0] : sw[tile][1]);
      acc[tile] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, acc[tile], 0, 0, 0);
    }
  }
}

// End of a group (columns cb ..): fixed-order sums of the 8 wavefronts' partial tiles; wavefront
// `tile` scales and stores tile `tile`.
__device__ __forceinline__ void pair_epilogue(const GemmArgs& p,
                                              floatx4_t (&partial)[2][kWaves][64],
                                              const float* gtab, int cb, int cend, int wave,
                                              int lane, int r, int g, floatx4_t (&acc)[2]) {
  partial[0][wave][lane] = acc[0];
  partial[1][wave][lane] = acc[1];
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0) only
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  if (wave < 2) {
    floatx4_t sum = partial[wave][0][lane];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) sum += partial[wave][w][lane];
    const int n = cb + 16 * wave + r;
    if (n < cend) {
      const float al = 1.0f / (gtab[NVFP4_MAX_SEGMENTS] * gtab[column_segment(p.seg, n)]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = 4 * g + e;
        if (m >= p.M) continue;
        if (p.c_accumulate)
          reinterpret_cast<float*>(p.c)[(int64_t)m * p.ldc + n] += sum[e] * al;
        else
          store_c(p.c, p.c_bf16, p.ldc, m, n, sum[e] * al);
      }
    }
  }
  acc[0] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
  acc[1] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
}

// The last REM units of gemm_stream_pair_kernel (kPairAhead <= REM < kPairAhead + kPairRing),
// starting at unit u0 in slot 0: step j copies unit u0 + j + kPairAhead only while that unit
// exists, and waits for unit u0 + j with the one later unit still outstanding, or none at the last.
template <int REM>
__device__ __forceinline__ void pair_tail(const PairArgs& s, uint8_t* const (&ring)[kPairRing],
                                          uint4 (&aw)[kPairRing], const uint8_t* asc,
                                          floatx4_t (&partial)[2][kWaves][64], const float* gtab,
                                          int u0, int c0, int clast, int cend, int wave, int lane,
                                          floatx4_t (&acc)[2]) {
  static_assert(kPairAhead == 2 && REM >= kPairAhead && REM < kPairAhead + kPairRing,
                "tail length");
  const GemmArgs& p = s.p;
  const int r = lane & 15, g = lane >> 4;
#pragma unroll
  for (int j = 0; j < REM; ++j) {
    __builtin_amdgcn_sched_barrier(0);
    if (j + 1 < REM)
      wait_vmcnt<(kPairAhead - 1) * kVmemPerPair>();
    else
      wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (j + kPairAhead < REM) {
      const int un = u0 + j + kPairAhead;
      const int i = un / s.nph;
      issue_pair(s, c0 + 32 * i, clast, un - i * s.nph, ring[(j + kPairAhead) % kPairRing], wave,
                 lane, aw[(j + kPairAhead) % kPairRing]);
    }
    const int u = u0 + j;
    const int i = u / s.nph;
    const int q = u - i * s.nph;
    compute_pair(ring[j % kPairRing], asc, p.K / 16, q, wave, r, g, r < p.M, aw[j % kPairRing],
                 acc);
    if (q == s.nph - 1) pair_epilogue(p, partial, gtab, c0 + 32 * i, cend, wave, lane, r, g, acc);
  }
}

__global__ void __launch_bounds__(kThreads) gemm_stream_pair_kernel(PairArgs s) {
  __shared__ __attribute__((aligned(16))) uint8_t q0[kPairBytes];
  __shared__ __attribute__((aligned(16))) uint8_t q1[kPairBytes];
  __shared__ __attribute__((aligned(16))) uint8_t q2[kPairBytes];
  uint8_t* const ring[kPairRing] = {q0, q1, q2};
  __shared__ __attribute__((aligned(16))) uint8_t asc[16 * (kStreamMaxK / 16)];
  __shared__ floatx4_t partial[2][kWaves][64];
  __shared__ float gtab[NVFP4_MAX_SEGMENTS + 1];

  const GemmArgs& p = s.p;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const bool arow_valid = r < p.M;
  const int ksa = p.K / 16;
  const int c0 = (int)blockIdx.x * s.ncols;
  const int cend = min(c0 + s.ncols, p.N);
  const int clast = cend - 1;
  const int units = ((cend - c0 + 31) / 32) * s.nph;

  // activation block scales of all K, copied once to LDS: they are older than every unit's copies,
  // so the unit waits cover them
  {
    const int per_row = ksa / 16;
    for (int i = threadIdx.x; i < p.M * per_row; i += kThreads) {
      const int row = i / per_row;
      __builtin_amdgcn_global_load_lds(
          p.a_scales + (int64_t)row * (p.k_pitch / 16) + (i - row * per_row) * 16,
          asc + (i & ~63) * 16, 16, 0, 0);
    }
  }

  // unit u: group u / nph (columns c0 + 32 (u / nph) ...), phase u % nph, in slot u % kPairRing
  // (units >= nph > 8 > kPairAhead)
  uint4 aw[kPairRing];
#pragma unroll
  for (int k = 0; k < kPairAhead; ++k) {
    const int i = k / s.nph;
    issue_pair(s, c0 + 32 * i, clast, k - i * s.nph, ring[k], wave, lane, aw[k]);
  }
  stage_global_scales(p, gtab);

  floatx4_t acc[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
  // whole rounds of kPairRing units while every unit they copy exists
  int u0 = 0;
  for (; u0 + kPairRing + kPairAhead <= units; u0 += kPairRing) {
#pragma unroll
    for (int k = 0; k < kPairRing; ++k) {
      const int u = u0 + k;
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<(kPairAhead - 1) * kVmemPerPair>();
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      {
        const int un = u + kPairAhead;
        const int i = un / s.nph;
        issue_pair(s, c0 + 32 * i, clast, un - i * s.nph, ring[(k + kPairAhead) % kPairRing],
                   wave, lane, aw[(k + kPairAhead) % kPairRing]);
      }
      const int i = u / s.nph;
      const int q = u - i * s.nph;
      compute_pair(ring[k], asc, ksa, q, wave, r, g, arow_valid, aw[k], acc);
      if (q == s.nph - 1)
        pair_epilogue(p, partial, gtab, c0 + 32 * i, cend, wave, lane, r, g, acc);
    }
  }
  // the remaining kPairAhead .. kPairAhead + kPairRing - 1 units, from slot 0
  switch (units - u0) {
    case 2: pair_tail<2>(s, ring, aw, asc, partial, gtab, u0, c0, clast, cend, wave, lane, acc); break;
    case 3: pair_tail<3>(s, ring, aw, asc, partial, gtab, u0, c0, clast, cend, wave, lane, acc); break;
    default: pair_tail<4>(s, ring, aw, asc, partial, gtab, u0, c0, clast, cend, wave, lane, acc); break;
  }
}

}  // namespace

hipError_t launch_gemm_stream(const GemmArgs& a, hipStream_t stream) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  StreamArgs s{};
  s.p = a;
  s.ntiles = (a.N + 15) / 16;
  s.nph = a.K / kUnitK;
  cus = cus > 0 ? cus : 1;
  const int per_cu = (a.N + cus - 1) / cus;
  if (s.nph > 8 && per_cu > 16) {
    PairArgs pa{};
    pa.p = a;
    pa.ncols = per_cu;
    pa.nph = s.nph;
    hipLaunchKernelGGL(gemm_stream_pair_kernel, dim3((a.N + per_cu - 1) / per_cu), dim3(kThreads),
                       0, stream, pa);
    return hipGetLastError();
  }
  const int grid = s.ntiles < cus ? s.ntiles : cus;
  switch (s.nph) {
    case 1: hipLaunchKernelGGL(gemm_stream_cached_kernel<1>, dim3(grid), dim3(kThreads), 0, stream, s); break;
    case 2: hipLaunchKernelGGL(gemm_stream_cached_kernel<2>, dim3(grid), dim3(kThreads), 0, stream, s); break;
    case 3: hipLaunchKernelGGL(gemm_stream_cached_kernel<3>, dim3(grid), dim3(kThreads), 0, stream, s); break;
    case 4: hipLaunchKernelGGL(gemm_stream_cached_kernel<4>, dim3(grid), dim3(kThreads), 0, stream, s); break;
    case 5: hipLaunchKernelGGL(gemm_stream_cached_kernel<5>, dim3(grid), dim3(kThreads), 0, stream, s); break;
    case 6: hipLaunchKernelGGL(gemm_stream_cached_kernel<6>, dim3(grid), dim3(kThreads), 0, stream, s); break;
    case 7: hipLaunchKernelGGL(gemm_stream_cached_kernel<7>, dim3(grid), dim3(kThreads), 0, stream, s); break;
    case 8: hipLaunchKernelGGL(gemm_stream_cached_kernel<8>, dim3(grid), dim3(kThreads), 0, stream, s); break;
    default: return hipErrorInvalidValue;  // longer K with at most 16 columns per compute unit: not here
  }
  return hipGetLastError();
}

}  // namespace nvfp4
