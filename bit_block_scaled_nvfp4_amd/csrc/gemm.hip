// W4A4 NVFP4 product kernels for gfx950 with the per-segment global-scale epilogue.
//
// Source: "Why Gated DeltaNet Survives 4-Bit Quantization" (arXiv 2609.04098), ai.info summary,
// "Main Findings": both operands NVFP4 (W4A4), one FP32 global scale per calibrated module, and
// fused serving GEMMs whose output segments need their own module's global scale.
//
// C[m, n] = (sum_k a[m,k] * w[n,k]) * alpha[seg(n)],  alpha[j] = 1 / (gA * gW[j]),
// the sum over exactly decoded elements accumulated in FP32 by v_mfma_f32_32x32x16_f16.
//
// Two kernels:
//  * gemm_general_kernel: any K that is a multiple of 16.  One wavefront per 32x32 output tile,
//    operands read straight from global memory 4 bytes (8 codes) per lane per K step.
//  * gemm_tiled_kernel: K a multiple of 64.  A workgroup owns a BM x BN output tile (256 x 256 or
//    256 x 192 chosen per problem, 64 x 64 for the last N % 256 columns when a problem is split
//    into two launches); each K chunk of 256 is staged in LDS as raw 4-bit codes plus
//    E4M3 bytes (9/16 byte per element instead of 2 for f16, so staging costs a quarter of the LDS
//    space and bandwidth of an f16 GEMM), then every wavefront decodes its own fragments in
//    registers right before the MFMAs, one sub-chunk of 64 at a time.
//
// K-slot permutation.  In a 32x32x16 MFMA, lane l supplies row (l % 32) and 8 of the 16 k-slots
// (half h = l / 32).  Within a sub-chunk of 64, lane half h reads the 16 contiguous bytes holding
// elements [32h, 32h + 32) of its row and uses 32-bit word j of them in MFMA step j (j = 0..3).
// A and W use the same map, so after 4 steps every k of the sub-chunk has been contracted once.
// Word j covers elements 32h + 8j .. +7, which lie in 16-block 2h + j/2 of the sub-chunk.
#include <type_traits>

#include "gemm_common.h"

namespace nvfp4 {
namespace {

// ------------------------------------------------------------------------------------------------
// general kernel
// ------------------------------------------------------------------------------------------------

__global__ void __launch_bounds__(256) gemm_general_kernel(GemmArgs p, uint32_t tiles_n) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const uint32_t tile = blockIdx.x;
  const int tm = (int)(tile / tiles_n) * 64 + (wave >> 1) * 32;
  const int tn = (int)(tile % tiles_n) * 64 + (wave & 1) * 32;
  if (tm >= p.M || tn >= p.N) return;
  const int r = lane & 31;
  const int h = lane >> 5;
  const int am = min(tm + r, p.M - 1);
  const int wn = min(tn + r, p.N - 1);
  const int64_t kb = p.K / 2, ks = p.K / 16;
  const uint8_t* ac = p.a_codes + am * kb + h * 4;
  const uint8_t* wc = p.w_codes + wn * kb + h * 4;
  const uint8_t* as = p.a_scales + am * ks;
  const uint8_t* ws = p.w_scales + wn * ks;

  floatx16 acc = {};
  for (int k0 = 0; k0 < p.K; k0 += 16) {
    const uint32_t qa = *reinterpret_cast<const uint32_t*>(ac + k0 / 2);
    const uint32_t qw = *reinterpret_cast<const uint32_t*>(wc + k0 / 2);
    const _Float16 sa = e4m3_to_half(as[k0 / 16]);
    const _Float16 sw = e4m3_to_half(ws[k0 / 16]);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(decode8(qa, sa), decode8(qw, sw), acc, 0, 0, 0);
  }

  const int n = tn + r;
  if (n >= p.N) return;
  const float alpha = column_alpha(p.seg, p.seg_g, *p.a_g, n);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int m = tm + 8 * (i / 4) + 4 * h + (i % 4);
    if (m < p.M) store_c(p.c, p.c_bf16, p.ldc, m, n, acc[i] * alpha);
  }
}

// ------------------------------------------------------------------------------------------------
// tiled kernel
// ------------------------------------------------------------------------------------------------

template <int WAVES_M, int WAVES_N, int FM, int FN>
struct TileCfg {
  static constexpr int kThreads = WAVES_M * WAVES_N * 64;
  static constexpr int BM = WAVES_M * FM * 32;
  static constexpr int BN = WAVES_N * FN * 32;
  // one LDS stage holds a K chunk of 256: the codes of BM + BN rows (128 bytes each), then the
  // scales of each operand (16 bytes each)
  static constexpr int kCodesA = BM * 128;
  static constexpr int kCodesB = BN * 128;
  static constexpr int kScalesA = BM * 16;
  static constexpr int kScalesB = BN * 16;
  static constexpr int kStage = kCodesA + kCodesB + kScalesA + kScalesB;
  // 16-byte copies per thread per chunk, of codes and of scales (the last may be partial)
  static constexpr int kPiecesA = (BM * 8 + kThreads - 1) / kThreads;
  static constexpr int kPiecesB = (BN * 8 + kThreads - 1) / kThreads;
  static constexpr int kWordsA = (BM + kThreads - 1) / kThreads;
  static constexpr int kWordsB = (BN + kThreads - 1) / kThreads;
  static_assert(FM >= 1 && FM <= 8 && FN >= 1 && FN <= 8, "fragments per wavefront");
  static_assert(BM % 64 == 0 && BN % 64 == 0, "whole wavefronts of copies");
};

// Per-thread byte offsets of the global rows this thread copies (rows beyond the matrix are
// clamped to the last row: they are loaded but never stored).
template <class Cfg>
struct RowOffsets {
  uint32_t a[Cfg::kPiecesA];
  uint32_t b[Cfg::kPiecesB];
  uint32_t sa[Cfg::kWordsA];
  uint32_t sb[Cfg::kWordsB];
};

// LDS layout of one stage and the copy that fills it.  Copies are direct memory->LDS: copy index
// d = i * threads + tid lands at LDS slot d (16 bytes), because the 64 lanes of a wavefront write
// consecutive slots.  The layout is chosen by which global bytes each copy index fetches, so that
// one wavefront copy reads whole 128-byte rows and every code fragment read is conflict-free:
//  * codes: slot d holds row (d / 256) * 32 + (d / 8) % 32, 16-byte piece (d % 8) ^ swz((d / 8) %
//    32) of the row's 128 bytes in the chunk.  A wavefront copy covers 8 rows x 128 bytes; each
//    32-row group is 4 KiB.  Lane (r, h) of a fragment reads piece 2u + h of its row for sub-chunk
//    u; the XOR swizzle puts any 8 consecutive rows on distinct bank groups for every piece.
//  * scales: slot d holds row d's 16 scale bytes in the chunk (a wavefront copy covers 64 rows);
//    a lane reads its rows' 4-byte word u for sub-chunk u.
__host__ __device__ constexpr int piece_swizzle(int r) { return ((r >> 1) ^ (r << 2)) & 7; }

template <class Cfg, int FM, int FN>
__device__ __forceinline__ void row_offsets(const GemmArgs& p, int m0, int n0, int tid,
                                            RowOffsets<Cfg>& o) {
  const uint32_t kb = (uint32_t)p.K / 2, ks = (uint32_t)p.K / 16;
  auto code_row = [](int d) { return (d >> 8) * 32 + ((d >> 3) & 31); };
  auto code_piece = [](int d) { return (d & 7) ^ piece_swizzle((d >> 3) & 31); };
#pragma unroll
  for (int i = 0; i < Cfg::kPiecesA; ++i) {
    const int d = tid + i * Cfg::kThreads;
    o.a[i] = (uint32_t)min(m0 + code_row(d), p.M - 1) * kb + code_piece(d) * 16;
  }
#pragma unroll
  for (int i = 0; i < Cfg::kPiecesB; ++i) {
    const int d = tid + i * Cfg::kThreads;
    o.b[i] = (uint32_t)min(n0 + code_row(d), p.N - 1) * kb + code_piece(d) * 16;
  }
#pragma unroll
  for (int i = 0; i < Cfg::kWordsA; ++i)
    o.sa[i] = (uint32_t)min(m0 + tid + i * Cfg::kThreads, p.M - 1) * ks;
#pragma unroll
  for (int i = 0; i < Cfg::kWordsB; ++i)
    o.sb[i] = (uint32_t)min(n0 + tid + i * Cfg::kThreads, p.N - 1) * ks;
}

// Copies go through buffer loads, whose range check returns zeros instead of touching memory
// past an operand: a chunk of 256 that extends past K (K not a multiple of 256) reads the next
// row's first bytes, or zeros past the last row, into LDS slots that are never used.  Each chunk's
// resource starts at the chunk (base + chunk offset, size reduced by as much), so the whole
// per-lane offset is range-checked.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t chunk_rsrc(const uint8_t* base, int64_t bytes,
                                                           int offset) {
  // raw buffer (stride 0), 32-bit data format word of the gfx9 resource descriptor
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base) + offset, (short)0,
                                           (int)(bytes - offset), 0x00020000);
}

template <int BYTES>  // 16 or 4
__device__ __forceinline__ void copy_to_lds(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint8_t* lds) {
  auto* const dst = (__attribute__((address_space(3))) void*)lds;
  if constexpr (BYTES == 16)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, (int)voff, 0, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 4, (int)voff, 0, 0, 0);
}

// Issue copies FROM .. TO-1 of K chunk `kc` (of 256) into `stage`, counting A's code pieces, W's
// code pieces, A's scale rows, then W's scale rows (kCopies per thread in all).  A wavefront whose
// copy slots of the last, partial round lie past the area skips that copy (the test is uniform
// across the wavefront).  The wavefront's first copy slot and the resources are uniform (scalar
// registers); each copy is a resource plus this lane's 32-bit row offset.
template <class Cfg, int FROM, int TO>
__device__ __forceinline__ void issue_part(const GemmArgs& p, const RowOffsets<Cfg>& o, int kc,
                                           uint8_t* stage) {
  const int wave_slot = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) * 64;
  const int64_t kb = p.K / 2, ks = p.K / 16;
  constexpr int PA = Cfg::kPiecesA, PB = Cfg::kPiecesB, WA = Cfg::kWordsA;
#pragma unroll
  for (int x = FROM; x < TO; ++x) {
    if (x < PA) {
      const int i = x;
      if ((i + 1) * Cfg::kThreads <= Cfg::BM * 8 || i * Cfg::kThreads + wave_slot < Cfg::BM * 8)
        copy_to_lds<16>(chunk_rsrc(p.a_codes, p.M * kb, kc * 128), o.a[i],
                        stage + (i * Cfg::kThreads + wave_slot) * 16);
    } else if (x < PA + PB) {
      const int i = x - PA;
      if ((i + 1) * Cfg::kThreads <= Cfg::BN * 8 || i * Cfg::kThreads + wave_slot < Cfg::BN * 8)
        copy_to_lds<16>(chunk_rsrc(p.w_codes, p.N * kb, kc * 128), o.b[i],
                        stage + Cfg::kCodesA + (i * Cfg::kThreads + wave_slot) * 16);
    } else if (x < PA + PB + WA) {
      const int i = x - PA - PB;
      if ((i + 1) * Cfg::kThreads <= Cfg::BM || i * Cfg::kThreads + wave_slot < Cfg::BM)
        copy_to_lds<16>(chunk_rsrc(p.a_scales, p.M * ks, kc * 16), o.sa[i],
                        stage + Cfg::kCodesA + Cfg::kCodesB + (i * Cfg::kThreads + wave_slot) * 16);
    } else {
      const int i = x - PA - PB - WA;
      if ((i + 1) * Cfg::kThreads <= Cfg::BN || i * Cfg::kThreads + wave_slot < Cfg::BN)
        copy_to_lds<16>(chunk_rsrc(p.w_scales, p.N * ks, kc * 16), o.sb[i],
                        stage + Cfg::kCodesA + Cfg::kCodesB + Cfg::kScalesA +
                            (i * Cfg::kThreads + wave_slot) * 16);
    }
  }
}

// The copies of a chunk go out in three parts: part 0 right after the barrier that frees the
// stage, parts 1 and 2 during the first two sub-chunks of the chunk before it.  Spreading them
// keeps each hand-over's burst of copies short (issuing all of them at once was 2-4 % slower).
template <class Cfg>
struct CopyParts {
  static constexpr int kCopies = Cfg::kPiecesA + Cfg::kPiecesB + Cfg::kWordsA + Cfg::kWordsB;
  static constexpr int k1 = kCopies / 3, k2 = 2 * kCopies / 3;
};

// Tile order: hardware hands workgroup ids to the 8 XCDs round-robin, so id b runs on XCD b % 8.
// Remap ids so each XCD walks a contiguous range of the logical order, and walk the logical order
// in groups of kGroupM tile-rows (column-major inside a group): the tiles an XCD runs at the same
// time then share a few A row-blocks and a few W row-blocks in that XCD's L2.
constexpr int kGroupM = 8;

__device__ __forceinline__ void tile_coords(uint32_t bid, uint32_t tiles_m, uint32_t tiles_n,
                                            uint32_t& tm, uint32_t& tn) {
  const uint32_t ntiles = tiles_m * tiles_n;
  uint32_t t = bid;
  if (ntiles % 8u == 0u) t = (bid % 8u) * (ntiles / 8u) + bid / 8u;
  const uint32_t per_group = kGroupM * tiles_n;
  const uint32_t group = t / per_group;
  const uint32_t first_m = group * kGroupM;
  const uint32_t gsize = min(tiles_m - first_m, (uint32_t)kGroupM);
  const uint32_t in_group = t - group * per_group;
  tm = first_m + in_group % gsize;
  tn = in_group / gsize;
}

// One sub-chunk (K = 64) of a wavefront's fragments, read from LDS: FM + FN code words of 16
// bytes (32 codes) and one 4-byte scale word (four E4M3 bytes) per fragment row.
template <int FM, int FN>
struct Frags {
  uint4 qa[FM];
  uint4 qb[FN];
  uint32_t sa[FM];
  uint32_t sb[FN];
};

// Byte offsets of this lane's reads within a stage: fragment 0 of each operand for sub-chunk 0
// (sub-chunk u is the same XOR 32 u for codes, plus 4 u for scales); fragment i adds i * 4096
// (codes) or i * 512 (scales).
struct FragOffsets {
  int a_frag, b_frag, a_scl, b_scl;
};

template <class Cfg, int FM, int FN>
__device__ __forceinline__ FragOffsets frag_offsets(int wm, int wn, int lane) {
  const int r = lane & 31, h = lane >> 5;
  const int in_group = r * 128 + ((h ^ piece_swizzle(r)) * 16);
  return FragOffsets{wm * FM * 4096 + in_group, Cfg::kCodesA + wn * FN * 4096 + in_group,
                     Cfg::kCodesA + Cfg::kCodesB + (wm * FM * 32 + r) * 16,
                     Cfg::kCodesA + Cfg::kCodesB + Cfg::kScalesA + (wn * FN * 32 + r) * 16};
}

__device__ __forceinline__ FragOffsets sub_chunk(const FragOffsets& o, int u) {
  return FragOffsets{o.a_frag ^ (32 * u), o.b_frag ^ (32 * u), o.a_scl + 4 * u, o.b_scl + 4 * u};
}

template <int FM, int FN>
__device__ __forceinline__ void read_frags(const uint8_t* stage, const FragOffsets& o,
                                           Frags<FM, FN>& f) {
#pragma unroll
  for (int i = 0; i < FM; ++i)
    f.qa[i] = *reinterpret_cast<const uint4*>(stage + o.a_frag + i * 4096);
#pragma unroll
  for (int j = 0; j < FN; ++j)
    f.qb[j] = *reinterpret_cast<const uint4*>(stage + o.b_frag + j * 4096);
#pragma unroll
  for (int i = 0; i < FM; ++i)
    f.sa[i] = *reinterpret_cast<const uint32_t*>(stage + o.a_scl + i * 512);
#pragma unroll
  for (int j = 0; j < FN; ++j)
    f.sb[j] = *reinterpret_cast<const uint32_t*>(stage + o.b_scl + j * 512);
}

template <int STEP>
__device__ __forceinline__ uint32_t word(const uint4& q) {
  return STEP == 0 ? q.x : STEP == 1 ? q.y : STEP == 2 ? q.z : q.w;
}

template <int STEP, int FM, int FN>
__device__ __forceinline__ void decode_step(const Frags<FM, FN>& f, const half2_t (&sa)[FM],
                                            const half2_t (&sb)[FN], half8_t (&av)[FM],
                                            half8_t (&bv)[FN]) {
#pragma unroll
  for (int i = 0; i < FM; ++i) av[i] = decode8(word<STEP>(f.qa[i]), STEP < 2 ? sa[i][0] : sa[i][1]);
#pragma unroll
  for (int j = 0; j < FN; ++j) bv[j] = decode8(word<STEP>(f.qb[j]), STEP < 2 ? sb[j][0] : sb[j][1]);
}

// The weight fragment is the MFMA's first operand, so acc[i][j] holds the transposed 32x32 block:
// lane (r, h) owns row m = r of A fragment i and columns n = 8 q + 4 h + (0..3) of W fragment j
// in registers 4 q .. 4 q + 3 -- four consecutive columns of one row of C, stored as one vector.
template <int FM, int FN>
__device__ __forceinline__ void mfma_step(const half8_t (&av)[FM], const half8_t (&bv)[FN],
                                          floatx16 (&acc)[FM][FN]) {
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bv[j], av[i], acc[i][j], 0, 0, 0);
}

// Interleave the FM*FN MFMAs of one step with the VALU work of decoding the next step: one MFMA,
// then a few VALU instructions, so the matrix core stays busy while the decode runs beside it.
template <int FM, int FN>
__device__ __forceinline__ void interleave_mfma_valu() {
  constexpr int kValuPerMfma = (8 * (FM + FN)) / (FM * FN) + 1;
#pragma unroll
  for (int k = 0; k < FM * FN; ++k) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, kValuPerMfma, 0);
  }
}

template <int FM, int FN>
__device__ __forceinline__ void decode_scales(const Frags<FM, FN>& f, uint32_t sh,
                                              half2_t (&sa)[FM], half2_t (&sb)[FN]) {
#pragma unroll
  for (int i = 0; i < FM; ++i)
    sa[i] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(f.sa[i] >> sh, 1.0f, false);
#pragma unroll
  for (int j = 0; j < FN; ++j)
    sb[j] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(f.sb[j] >> sh, 1.0f, false);
}

// Wait until this wavefront's copies of the chunk in `stage` have landed, meet the other
// wavefronts (after which the chunk is complete in LDS and every wavefront has read its fragments
// of the chunk before it), and read this lane's fragments of its first sub-chunk.  The scheduling
// fences keep the work issued before this point ahead of the wait.
template <int FM, int FN>
__device__ __forceinline__ void sync_and_read(const uint8_t* stage, const FragOffsets& o,
                                              Frags<FM, FN>& f) {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0x3F70);  // vmcnt(0)
  __builtin_amdgcn_s_barrier();
  read_frags(stage, o, f);
}

// MFMAs k = FROM .. TO-1 of one step, k = i * FN + j.
template <int FROM, int TO, int FM, int FN>
__device__ __forceinline__ void mfma_range(const half8_t (&av)[FM], const half8_t (&bv)[FN],
                                           floatx16 (&acc)[FM][FN]) {
#pragma unroll
  for (int k = FROM; k < TO; ++k)
    acc[k / FN][k % FN] =
        __builtin_amdgcn_mfma_f32_32x32x16_f16(bv[k % FN], av[k / FN], acc[k / FN][k % FN], 0, 0, 0);
}

// MFMAs of step 2 issued before the mid-sub-chunk hand-over: they keep the matrix core busy while
// the wavefronts meet (4 of the 12 or 16 of the wide tiles, half of a small tile's).
template <int FM, int FN>
constexpr int pre_barrier_mfma() {
  return FM * FN >= 8 ? 4 : FM * FN / 2;
}

// Schedule of the MFMAs after the hand-over: the next sub-chunk's LDS reads (two per MFMA) and the
// copies of the chunk after the next go out between MFMAs, with the decode VALU spread over all
// of them, rather than as one block in front of the MFMAs.
template <int FM, int FN, int NDS, int NVM>
__device__ __forceinline__ void interleave_after_barrier() {
  constexpr int kM = FM * FN - pre_barrier_mfma<FM, FN>();
  constexpr int kDsMfma = (NDS + 1) / 2;          // MFMAs carrying two LDS reads
  constexpr int kVmPerMfma = (NVM + kM - 1) / kM;  // copies per MFMA (the last group may be short)
  constexpr int kValu = (8 * (FM + FN) + kM - 1) / kM + 1;
#pragma unroll
  for (int k = 0; k < kM; ++k) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    if (k < kDsMfma) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS read
    if constexpr (NVM > 0) {  // VMEM
      if ((k + 1) * kVmPerMfma <= NVM) __builtin_amdgcn_sched_group_barrier(0x010, kVmPerMfma, 0);
      else if (k * kVmPerMfma < NVM)
        __builtin_amdgcn_sched_group_barrier(0x010, NVM % kVmPerMfma, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x002, kValu, 0);  // VALU
  }
}

// One sub-chunk (K = 64), software-pipelined with the next.  The MFMAs of steps 0-1 run under the
// decode of steps 1-2.  The first MFMAs of step 2 are issued; then comes the hand-over to the next
// sub-chunk.  For the second sub-chunk of a chunk (SYNC), every wavefront first waits for its own
// copies of the next chunk and meets the others at a barrier (the next chunk is complete in LDS,
// and every wavefront has read the current chunk, whose stage is free); for the first sub-chunk,
// the next one is already in the same stage.  The remaining MFMAs of step 2 run under the LDS reads
// of the next sub-chunk's fragments (from `nstage` at offsets `no`), NVM copies into the stage
// that is free (`issue`), and the decode of step 3; the MFMAs of
// step 3 run under the decode of the next sub-chunk's step 0.  On entry `cur` holds this
// sub-chunk's fragments and a0/b0 its decoded step 0; on exit (HAS_NEXT) `nxt` holds the next
// sub-chunk's fragments and a0/b0 its decoded step 0.
template <bool HAS_NEXT, bool SYNC, int NVM, int FM, int FN, class Issue>
__device__ __forceinline__ void pipelined_chunk(const Frags<FM, FN>& cur, Frags<FM, FN>& nxt,
                                                const uint8_t* nstage, const FragOffsets& no,
                                                half2_t (&sa)[FM], half2_t (&sb)[FN],
                                                half8_t (&a0)[FM], half8_t (&b0)[FN],
                                                half8_t (&a1)[FM], half8_t (&b1)[FN], uint32_t sh,
                                                floatx16 (&acc)[FM][FN], Issue&& issue) {
  mfma_step(a0, b0, acc);
  decode_step<1>(cur, sa, sb, a1, b1);
  interleave_mfma_valu<FM, FN>();
  mfma_step(a1, b1, acc);
  decode_step<2>(cur, sa, sb, a0, b0);
  interleave_mfma_valu<FM, FN>();
  __builtin_amdgcn_sched_barrier(0);
  mfma_range<0, pre_barrier_mfma<FM, FN>()>(a0, b0, acc);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (HAS_NEXT) {
    if constexpr (SYNC) {
      __builtin_amdgcn_s_waitcnt(0x3F70);  // vmcnt(0): this lane's copies of the next chunk landed
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
    }
    read_frags(nstage, no, nxt);
    if constexpr (NVM > 0) issue();
  }
  mfma_range<pre_barrier_mfma<FM, FN>(), FM * FN>(a0, b0, acc);
  decode_step<3>(cur, sa, sb, a1, b1);
  interleave_after_barrier<FM, FN, HAS_NEXT ? 2 * (FM + FN) : 0, HAS_NEXT ? NVM : 0>();
  __builtin_amdgcn_sched_barrier(0);
  mfma_step(a1, b1, acc);
  if constexpr (HAS_NEXT) {
    decode_scales(nxt, sh, sa, sb);
    decode_step<0>(nxt, sa, sb, a0, b0);
  }
  interleave_mfma_valu<FM, FN>();
}

// The thread index behind a compiler barrier: values derived from it inside a loop are not hoisted
// out of the loop, so they do not occupy registers across the main loop.
__device__ __forceinline__ int opaque_tid() {
  int t = threadIdx.x;
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass parses device code but cannot take AMDGPU constraints
  asm volatile("" : "+v"(t));
#endif
  return t;
}

// Epilogue of one tile: C = acc * alpha[column], through LDS one fragment row (32 rows of the
// wavefront's sub-tile) and up to four fragment columns (128 columns) at a time.  Each lane writes
// its four-column pieces into the wavefront's own staging rows, then reads back four consecutive
// columns of one row, so that a wavefront store covers whole rows of up to 512 contiguous bytes
// instead of 32 rows x 32 bytes.  The staging area belongs to one wavefront and LDS instructions
// of a wavefront execute in order, so no barrier is needed.  Rows and columns past the matrix are
// masked at the store; a lane stores its four columns as one vector when they are all inside and
// rows of C start 16-byte aligned (`vec`).
// Floats per staged row: the widest column group (4, 2 or 1 fragments of 32 columns) plus a pad
// that spreads rows over banks.
template <int FN>
__host__ __device__ constexpr int epi_stride() {
  return (FN >= 4 ? 4 : FN >= 2 ? 2 : 1) * 32 + 4;
}

template <bool BF16, int G, int J0, int FM, int FN>
__device__ __forceinline__ void store_group(const GemmArgs& p, const floatx16 (&acc)[FM][FN],
                                            const float* alpha, float* epi, int m0, int n0, int wm,
                                            int wn, int lane, bool vec, bool interior, int i) {
  using OutT = typename std::conditional<BF16, uint16_t, float>::type;
  OutT* const c = reinterpret_cast<OutT*>(p.c);
  constexpr int S = epi_stride<FN>();
  constexpr int LPR = G * 8;    // lanes per staged row (four columns each)
  constexpr int RPI = 64 / LPR;  // rows per read-back instruction
  constexpr int NT = 32 / RPI;   // read-backs per fragment row
  const int r = lane & 31, h = lane >> 5;
  const int rr = lane / LPR;
  const int cc = (lane % LPR) * 4;  // read-back columns of this lane within the group
  const int col = wn * FN * 32 + J0 * 32 + cc;
  const int n = n0 + col;
  const floatx4 al = *reinterpret_cast<const floatx4*>(alpha + col);
#pragma unroll
  for (int j = 0; j < G; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<floatx4*>(epi + r * S + j * 32 + 8 * q + 4 * h) =
          floatx4{acc[i][J0 + j][4 * q], acc[i][J0 + j][4 * q + 1], acc[i][J0 + j][4 * q + 2],
                  acc[i][J0 + j][4 * q + 3]};
  floatx4 x[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) x[t] = *reinterpret_cast<const floatx4*>(epi + (RPI * t + rr) * S + cc);
  const int mb = m0 + wm * FM * 32 + i * 32 + rr;
  const bool full = vec && n + 3 < p.N;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const floatx4 v = {x[t][0] * al[0], x[t][1] * al[1], x[t][2] * al[2], x[t][3] * al[3]};
    const int m = mb + RPI * t;
    if (!interior && m >= p.M) continue;
    OutT* const dst = c + (int64_t)m * p.ldc + n;
    if (interior || full) {
      if constexpr (BF16) {
        const uint32_t lo = f32_to_bf16_rne(v[0]) | ((uint32_t)f32_to_bf16_rne(v[1]) << 16);
        const uint32_t hi = f32_to_bf16_rne(v[2]) | ((uint32_t)f32_to_bf16_rne(v[3]) << 16);
        *reinterpret_cast<uint2*>(dst) = uint2{lo, hi};
      } else {
        *reinterpret_cast<floatx4*>(dst) = v;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (n + e < p.N) {
          if constexpr (BF16)
            dst[e] = f32_to_bf16_rne(v[e]);
          else
            dst[e] = v[e];
        }
      }
    }
  }
  // one staged block at a time: its accumulators are read into registers only here
  __builtin_amdgcn_sched_barrier(0);
}

// Column groups of 4, 2 and 1 fragments (a group's rows must fill whole wavefront reads).
template <bool BF16, int J0, int FM, int FN>
__device__ __forceinline__ void store_groups(const GemmArgs& p, const floatx16 (&acc)[FM][FN],
                                             const float* alpha, float* epi, int m0, int n0,
                                             int wm, int wn, int lane, bool vec, bool interior,
                                             int i) {
  if constexpr (J0 < FN) {
    constexpr int G = FN - J0 >= 4 ? 4 : FN - J0 >= 2 ? 2 : 1;
    store_group<BF16, G, J0>(p, acc, alpha, epi, m0, n0, wm, wn, lane, vec, interior, i);
    store_groups<BF16, J0 + G>(p, acc, alpha, epi, m0, n0, wm, wn, lane, vec, interior, i);
  }
}

template <bool BF16, int FM, int FN>
__device__ __forceinline__ void store_tile(const GemmArgs& p, const floatx16 (&acc)[FM][FN],
                                           const float* alpha, float* epi, int m0, int n0, int wm,
                                           int wn, int lane, bool vec, bool interior) {
#pragma unroll
  for (int i = 0; i < FM; ++i)
    store_groups<BF16, 0>(p, acc, alpha, epi, m0, n0, wm, wn, lane, vec, interior, i);
}

// Main kernel, persistent: workgroup b runs tiles b, b + G, b + 2G, ... (G = grid size, at most
// one workgroup per compute unit).  Two LDS stages of one K chunk (256) each, filled by direct
// memory->LDS copies; two register sets of fragments, alternating over the chunk's four
// sub-chunks (64).  In the middle of the last sub-chunk of chunk kc every wavefront waits for its
// own copies of chunk kc+1, meets the others at a barrier (chunk kc+1 is then complete in LDS and
// every wavefront has read chunk kc, whose stage is free), reads its fragments of chunk kc+1's
// first sub-chunk, and issues the first third of chunk kc+2's copies into chunk kc's stage (the
// other two thirds go out during chunk kc+1's first two sub-chunks); in the middle of the other
// sub-chunks it reads the next sub-chunk's fragments from the same stage.  The remaining
// MFMA steps of each sub-chunk cover those LDS reads and the decode of the next sub-chunk's first
// step, so the matrix core does not idle across sub-chunks.  The loop runs two whole chunks per
// pass; the 0-7 sub-chunks left after it run once every copy has landed, with no further barrier.
// Past the last chunk, reads and copies are clamped to it (redundant, never used).
// Between tiles, the copies of the next tile's first chunk are issued before the stores of the
// finished tile, so the store traffic and the next tile's first loads are in flight together; the
// stores stage the accumulators through the second stage, whose first copies follow the stores.
// Each lane waits for its own copies and a barrier precedes every reuse of a stage, so stages never
// see two tiles' copies or the staging race.
template <int WAVES_M, int WAVES_N, int FM, int FN>
__global__ void __launch_bounds__(WAVES_M * WAVES_N * 64, 1)
gemm_tiled_kernel(GemmArgs p, uint32_t tiles_m, uint32_t tiles_n) {
  using Cfg = TileCfg<WAVES_M, WAVES_N, FM, FN>;
  __shared__ __attribute__((aligned(16))) uint8_t s0[Cfg::kStage];
  __shared__ __attribute__((aligned(16))) uint8_t s1[Cfg::kStage];
  // per-column epilogue factors of the current tile, double-buffered by tile parity
  __shared__ __attribute__((aligned(16))) float alpha_s[2][Cfg::BN];
  // the epilogue stages accumulators in s1: one area of 32 rows per wavefront
  constexpr int kEpiArea = 32 * epi_stride<FN>();
  static_assert(WAVES_M * WAVES_N * kEpiArea * 4 <= Cfg::kStage, "epilogue staging fits a stage");

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave / WAVES_N;
  const int wn = wave % WAVES_N;
  const int h = lane >> 5;
  const int r = lane & 31;
  const uint32_t sh = 16u * (uint32_t)h;  // lane half h uses scale bytes 2h, 2h+1
  const uint32_t ntiles = tiles_m * tiles_n;
  const int nsub = p.K / 64;            // sub-chunks of 64
  const int last = (nsub + 1) / 2 - 1;  // last chunk of 128 (it may hold one sub-chunk)
  const float ga = *p.a_g;
  const bool vec = (p.ldc & 3) == 0;  // rows of C start 16-byte aligned (C itself is)

  // LDS read offsets of this lane's fragments (within a stage), for each sub-chunk
  const FragOffsets fo = frag_offsets<Cfg, FM, FN>(wm, wn, lane);

  uint32_t v = blockIdx.x;
  uint32_t tmi, tni;
  tile_coords(v, tiles_m, tiles_n, tmi, tni);
  int m0 = (int)tmi * Cfg::BM;
  int n0 = (int)tni * Cfg::BN;
  {
    const int tid_t = threadIdx.x;
    RowOffsets<Cfg> ro;
    row_offsets<Cfg, FM, FN>(p, m0, n0, tid_t, ro);
    issue_part<Cfg, 0, CopyParts<Cfg>::kCopies>(p, ro, 0, s0);
    issue_part<Cfg, 0, CopyParts<Cfg>::k1>(p, ro, min(1, last), s1);
  }

  for (int par = 0;; par ^= 1) {
    // The copy offsets are recomputed here rather than carried over from the early issue of this
    // tile's first chunks: carried over, they would stay live across the previous tile's stores
    // (the empty asm keeps the two computations apart).
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("" : "+s"(m0), "+s"(n0));
#endif
    const int tid_t = opaque_tid();
    RowOffsets<Cfg> ro;
    row_offsets<Cfg, FM, FN>(p, m0, n0, tid_t, ro);
    for (int c = tid_t; c < Cfg::BN; c += Cfg::kThreads)
      alpha_s[par][c] = column_alpha(p.seg, p.seg_g, ga, min(n0 + c, p.N - 1));

    floatx16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = floatx16{};

    Frags<FM, FN> f0, f1;
    half2_t sa[FM], sb[FN];
    half8_t a0[FM], b0[FN], a1[FM], b1[FN];

    // chunk 0's first sub-chunk into registers (chunk 1 is already in flight into s1)
    sync_and_read(s0, fo, f0);
    decode_scales(f0, sh, sa, sb);
    decode_step<0>(f0, sa, sb, a0, b0);

    using CP = CopyParts<Cfg>;
    // One chunk: sub-chunks 0-2 each read the next one from the same stage, and sub-chunks 0 and
    // 1 copy parts 1 and 2 of chunk kc+1 into the other stage; sub-chunk 3 reads the next chunk's
    // first sub-chunk after the barrier and copies part 0 of chunk kc+2 into this chunk's stage.
    // The register sets alternate f0, f1, f0, f1, so a chunk starts and ends with f0.  The stages
    // are named statically (the loop runs two chunks per pass), so the compiler sees that reads of
    // one stage do not alias the copies in flight into the other.
    auto run_chunk = [&](uint8_t* stage, uint8_t* next_stage, int kc) {
      const int k1 = min(kc + 1, last), k2 = min(kc + 2, last);
      pipelined_chunk<true, false, CP::k2 - CP::k1>(
          f0, f1, stage, sub_chunk(fo, 1), sa, sb, a0, b0, a1, b1, sh, acc,
          [&] { issue_part<Cfg, CP::k1, CP::k2>(p, ro, k1, next_stage); });
      pipelined_chunk<true, false, CP::kCopies - CP::k2>(
          f1, f0, stage, sub_chunk(fo, 2), sa, sb, a0, b0, a1, b1, sh, acc,
          [&] { issue_part<Cfg, CP::k2, CP::kCopies>(p, ro, k1, next_stage); });
      pipelined_chunk<true, false, 0>(f0, f1, stage, sub_chunk(fo, 3), sa, sb, a0, b0, a1, b1, sh,
                                      acc, [] {});
      pipelined_chunk<true, true, CP::k1>(f1, f0, next_stage, fo, sa, sb, a0, b0, a1, b1, sh, acc,
                                          [&] { issue_part<Cfg, 0, CP::k1>(p, ro, k2, stage); });
    };
    int kc = 0;
    for (; 4 * kc + 7 < nsub; kc += 2) {
      run_chunk(s0, s1, kc);
      run_chunk(s1, s0, kc + 1);
    }
    // 0 to 7 sub-chunks remain: chunk kc in s0 (its first sub-chunk already in f0), then chunk
    // kc+1 in s1, whose parts 1 and 2 are copied now.  Once every copy of both has landed they run
    // with no further barrier, two sub-chunks (f0 then f1) per pass; the last read of a pass is
    // clamped to the last sub-chunk.
    int sc = 4 * kc;
    if (sc < nsub) {
      issue_part<Cfg, CP::k1, CP::kCopies>(p, ro, min(kc + 1, last), s1);
      __builtin_amdgcn_s_waitcnt(0x3F70);  // vmcnt(0)
      __builtin_amdgcn_s_barrier();
      auto stage_of = [&](int c) -> const uint8_t* { return (c >> 2) > kc ? s1 : s0; };
      for (; sc + 1 < nsub; sc += 2) {
        pipelined_chunk<true, false, 0>(f0, f1, stage_of(sc + 1), sub_chunk(fo, (sc + 1) & 3), sa,
                                        sb, a0, b0, a1, b1, sh, acc, [] {});
        const int nx = min(sc + 2, nsub - 1);
        pipelined_chunk<true, false, 0>(f1, f0, stage_of(nx), sub_chunk(fo, nx & 3), sa, sb, a0, b0,
                                        a1, b1, sh, acc, [] {});
      }
      if (sc < nsub)
        pipelined_chunk<false, false, 0>(f0, f1, s0, fo, sa, sb, a0, b0, a1, b1, sh, acc, [] {});
    }
    // this lane's redundant copies past the last chunk have landed before its stages are reused
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0x3F70);
    __builtin_amdgcn_sched_barrier(0);

    // lane values of the epilogue and of the next tile's copies, derived afresh (not hoisted)
    const int tid_e = opaque_tid();
    const int lane_e = tid_e & 63, wave_e = tid_e >> 6;
    const int tm0 = m0, tn0 = n0;
    v += gridDim.x;
    const bool more = v < ntiles;
    // every wavefront is past its last reads of both stages, and every copy into them has landed
    __builtin_amdgcn_s_barrier();
    if (more) {
      tile_coords(v, tiles_m, tiles_n, tmi, tni);
      m0 = (int)tmi * Cfg::BM;
      n0 = (int)tni * Cfg::BN;
      RowOffsets<Cfg> ron;
      row_offsets<Cfg, FM, FN>(p, m0, n0, tid_e, ron);
      issue_part<Cfg, 0, CopyParts<Cfg>::kCopies>(p, ron, 0, s0);
    }
    const bool interior = vec && tm0 + Cfg::BM <= p.M && tn0 + Cfg::BN <= p.N;
    float* const epi = reinterpret_cast<float*>(s1) + wave_e * kEpiArea;
    if (p.c_bf16)
      store_tile<true>(p, acc, alpha_s[par], epi, tm0, tn0, wave_e / WAVES_N, wave_e % WAVES_N,
                       lane_e, vec, interior);
    else
      store_tile<false>(p, acc, alpha_s[par], epi, tm0, tn0, wave_e / WAVES_N, wave_e % WAVES_N,
                        lane_e, vec, interior);
    if (more) {
      // every wavefront has read back its staged accumulators before copies land in s1
      __builtin_amdgcn_s_barrier();
      const int tid_c = opaque_tid();
      RowOffsets<Cfg> ron;
      row_offsets<Cfg, FM, FN>(p, m0, n0, tid_c, ron);
      issue_part<Cfg, 0, CopyParts<Cfg>::k1>(p, ron, min(1, last), s1);
    }
    if (!more) break;
  }
}

template <int WAVES_M, int WAVES_N, int FM, int FN>
hipError_t launch_tiled_cfg(const GemmArgs& a, int cus, hipStream_t stream) {
  using Cfg = TileCfg<WAVES_M, WAVES_N, FM, FN>;
  const uint32_t tiles_m = (a.M + Cfg::BM - 1) / Cfg::BM;
  const uint32_t tiles_n = (a.N + Cfg::BN - 1) / Cfg::BN;
  // one workgroup per compute unit (the kernel's registers allow one per compute unit), each
  // walking its share of the tiles
  const uint32_t ntiles = tiles_m * tiles_n;
  const uint32_t grid = min(ntiles, (uint32_t)max(cus, 1));
  hipLaunchKernelGGL((gemm_tiled_kernel<WAVES_M, WAVES_N, FM, FN>), dim3(grid),
                     dim3(Cfg::kThreads), 0, stream, a, tiles_m, tiles_n);
  return hipGetLastError();
}

// Tile shapes of the persistent kernel: 256 x 256 (4 x 4 fragments per wavefront), 256 x 192
// (4 x 3) and, for the last columns only, 64 x 64 (1 x 1).  The narrower wide tile decodes more per
// MFMA (7 fragment words per 12 MFMAs instead of 8 per 16) and measured about 0.89 of the wider
// one's rate per tile FLOP, but it can save a whole round of tiles: the GDN in_proj (4096 x 8288)
// is 528 tiles of 256 x 256 on 256 compute units, three rounds of which the last is 1/16 full, and
// 704 of 256 x 192, three rounds of 3/4 the work.  The third way runs the whole 256-column tile
// columns (8192 there, two full rounds) as one launch and the remaining N % 256 columns as a second
// launch of 64 x 64 tiles, 128 of them at the GDN in_proj.  A small tile gives each wavefront a
// single 32 x 32 accumulator, one dependent chain of MFMAs with little work per K chunk to cover the
// copies of the next: one round of them took 0.2-0.4 of a 256 x 256 round at the same K, and the
// estimate takes 0.4 (GDN in_proj: 0.267 ms split against 0.281 ms in 256 x 192 tiles and 0.333 ms
// in 256 x 256, on one machine).  The way is chosen by the estimated time, in rounds of
// 256 x 256 tiles.  Every output element is accumulated the same way in every shape (same K
// chunks, steps and MFMA), so the choice never changes a result.
constexpr float kNarrowTileRate = 0.89f;
constexpr float kStripRoundCost = 0.4f;

// The tile columns of 256 as one launch, the last a.N % 256 columns as a launch of 64 x 64 tiles
// on the same stream: the second sees the columns [nfull, N) of W and C as its whole problem, with
// the segment table cut and rebased to them (the same alpha values, so the same bits).
hipError_t launch_tiled_split(const GemmArgs& a, int nfull, int cus, hipStream_t stream) {
  GemmArgs body = a;
  body.N = nfull;
  const hipError_t e = launch_tiled_cfg<2, 2, 4, 4>(body, cus, stream);
  if (e != hipSuccess) return e;
  GemmArgs strip = a;
  strip.w_codes = a.w_codes + (int64_t)nfull * (a.K / 2);
  strip.w_scales = a.w_scales + (int64_t)nfull * (a.K / 16);
  strip.c = a.c_bf16 ? (void*)(reinterpret_cast<uint16_t*>(a.c) + nfull)
                     : (void*)(reinterpret_cast<float*>(a.c) + nfull);
  strip.N = a.N - nfull;
  int first = 0;  // the segment that holds column nfull
  while (first + 1 < a.seg.nseg && a.seg.off[first + 1] <= nfull) ++first;
  strip.seg_g = a.seg_g + first;
  strip.seg.nseg = a.seg.nseg - first;
  for (int t = 0; t <= NVFP4_MAX_SEGMENTS; ++t)
    strip.seg.off[t] = t <= strip.seg.nseg ? max(a.seg.off[first + t] - nfull, 0) : strip.N;
  return launch_tiled_cfg<2, 2, 1, 1>(strip, cus, stream);
}

}  // namespace

hipError_t launch_gemm_tiled(const GemmArgs& a, hipStream_t stream) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  cus = max(cus, 1);
  auto rounds = [&](int64_t m, int64_t n, int bm, int bn) {
    const int64_t t = ((m + bm - 1) / bm) * ((n + bn - 1) / bn);
    return (float)((t + cus - 1) / cus);
  };
  const float wide = rounds(a.M, a.N, 256, 256);
  const float narrow = rounds(a.M, a.N, 256, 192) * (192.0f / 256.0f) / kNarrowTileRate;
  const int nfull = a.N / 256 * 256;
  const float split = nfull > 0 && nfull < a.N
                          ? rounds(a.M, nfull, 256, 256) +
                                rounds(a.M, a.N - nfull, 64, 64) * kStripRoundCost
                          : wide + 1.0f;
  if (split < wide && split < narrow) return launch_tiled_split(a, nfull, cus, stream);
  if (narrow < wide) return launch_tiled_cfg<2, 2, 4, 3>(a, cus, stream);
  return launch_tiled_cfg<2, 2, 4, 4>(a, cus, stream);
}

hipError_t launch_gemm_general(const GemmArgs& a, hipStream_t stream) {
  const uint32_t tiles_m = (a.M + 63) / 64;
  const uint32_t tiles_n = (a.N + 63) / 64;
  hipLaunchKernelGGL(gemm_general_kernel, dim3(tiles_m * tiles_n), dim3(256), 0, stream, a,
                     tiles_n);
  return hipGetLastError();
}

GemmPath choose_gemm_path(int64_t M, int64_t K, bool c_bf16) {
  // decode shapes (at most 16 activation rows) stream the weights with the skinny or the streaming
  // kernel, a K above kStreamMaxK in pieces that add into an f32 C (a bf16 C would round every
  // partial sum); the tiled kernel needs whole K chunks of 64 (the host layer keeps every operand
  // below 2 GiB, so 32-bit row offsets suffice)
  if (M <= 16 && K % 1024 == 0 && (K <= kStreamMaxK || !c_bf16)) return GemmPath::Skinny;
  return K % 64 == 0 ? GemmPath::Tiled : GemmPath::General;
}

}  // namespace nvfp4
