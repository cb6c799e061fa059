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
//  * gemm_tiled_kernel: K a multiple of 64.  A workgroup owns a BM x BN output tile; each K chunk of
//    64 is staged in LDS as raw 4-bit codes plus E4M3 bytes (9/16 byte per element instead of 2 for
//    f16, so staging costs a quarter of the LDS space and bandwidth of an f16 GEMM), then every
//    wavefront decodes its own fragments in registers right before the MFMAs.
//
// K-slot permutation.  In a 32x32x16 MFMA, lane l supplies row (l % 32) and 8 of the 16 k-slots
// (half h = l / 32).  Within a K chunk of 64, lane half h reads the 16 contiguous bytes holding
// elements [32h, 32h + 32) of its row and uses 32-bit word j of them in MFMA step j (j = 0..3).
// A and W use the same map, so after 4 steps every k of the chunk has been contracted once.  Word
// j covers elements 32h + 8j .. +7, which lie in 16-block 2h + j/2 of the chunk.
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
  // one LDS stage: the codes of BM + BN rows (32 bytes each per K chunk of 64), then their 4 scale
  // bytes per row
  static constexpr int kCodesA = BM * 32;
  static constexpr int kCodesB = BN * 32;
  static constexpr int kScalesA = BM * 4;
  static constexpr int kScalesB = BN * 4;
  static constexpr int kStage = kCodesA + kCodesB + kScalesA + kScalesB;
  static constexpr int kPiecesA = BM * 2 / kThreads;  // 16-byte copies per thread per chunk
  static constexpr int kPiecesB = BN * 2 / kThreads;
  static constexpr int kWordsA = BM / kThreads;  // 4-byte scale copies per thread per chunk
  static constexpr int kWordsB = BN / kThreads;
  static_assert(BM * 2 % kThreads == 0 && BN * 2 % kThreads == 0, "piece split");
  static_assert(BM % kThreads == 0 && BN % kThreads == 0, "scale split");
  static_assert(FM == 4 && FN == 4, "one 16-byte scale read per operand assumes 4 fragments");
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

// LDS layout of one stage and the copy that fills it.  Copies are direct global->LDS: copy index
// d = i * threads + tid lands at LDS slot d (16 bytes for codes, 4 bytes for scales), because the
// 64 lanes of a wavefront write consecutive slots.  The layout is chosen by which global row each
// copy index fetches:
//  * codes: slot d holds row (d / 64) * 32 + (d % 32), bytes [16 * ((d % 64) / 32), +16) of the
//    chunk.  Each 32-row group is 1 KiB laid out [half][row][16 B] -- exactly the order in which
//    the 64 lanes of a fragment read it (lane l at 16 l): reads are contiguous, conflict-free.
//  * scales: slot d holds the 4 scale bytes of row (d / (32F)) * 32F + (d % F) * 32 + (d / F) % 32
//    (F fragments per wavefront): the F scale words one lane needs sit in one 16-byte slot group.
template <int F>
__device__ __forceinline__ int scale_slot_row(int d) {
  return (d / (32 * F)) * (32 * F) + (d % F) * 32 + (d / F) % 32;
}

template <class Cfg, int FM, int FN>
__device__ __forceinline__ void row_offsets(const GemmArgs& p, int m0, int n0, int tid,
                                            RowOffsets<Cfg>& o) {
  const uint32_t kb = (uint32_t)p.K / 2, ks = (uint32_t)p.K / 16;
#pragma unroll
  for (int i = 0; i < Cfg::kPiecesA; ++i) {
    const int d = tid + i * Cfg::kThreads;
    const int row = (d >> 6) * 32 + (d & 31);
    o.a[i] = (uint32_t)min(m0 + row, p.M - 1) * kb + ((d >> 5) & 1) * 16;
  }
#pragma unroll
  for (int i = 0; i < Cfg::kPiecesB; ++i) {
    const int d = tid + i * Cfg::kThreads;
    const int row = (d >> 6) * 32 + (d & 31);
    o.b[i] = (uint32_t)min(n0 + row, p.N - 1) * kb + ((d >> 5) & 1) * 16;
  }
#pragma unroll
  for (int i = 0; i < Cfg::kWordsA; ++i)
    o.sa[i] = (uint32_t)min(m0 + scale_slot_row<FM>(tid + i * Cfg::kThreads), p.M - 1) * ks;
#pragma unroll
  for (int i = 0; i < Cfg::kWordsB; ++i)
    o.sb[i] = (uint32_t)min(n0 + scale_slot_row<FN>(tid + i * Cfg::kThreads), p.N - 1) * ks;
}

// Issue the direct global->LDS copies of K chunk `kc` into `stage`.
template <class Cfg>
__device__ __forceinline__ void issue_chunk(const GemmArgs& p, const RowOffsets<Cfg>& o, int kc,
                                            uint8_t* stage) {
  const int wave_slot = (threadIdx.x >> 6) * 64;
#pragma unroll
  for (int i = 0; i < Cfg::kPiecesA; ++i)
    __builtin_amdgcn_global_load_lds(p.a_codes + o.a[i] + kc * 32,
                                     stage + (i * Cfg::kThreads + wave_slot) * 16, 16, 0, 0);
#pragma unroll
  for (int i = 0; i < Cfg::kPiecesB; ++i)
    __builtin_amdgcn_global_load_lds(p.w_codes + o.b[i] + kc * 32,
                                     stage + Cfg::kCodesA + (i * Cfg::kThreads + wave_slot) * 16,
                                     16, 0, 0);
#pragma unroll
  for (int i = 0; i < Cfg::kWordsA; ++i)
    __builtin_amdgcn_global_load_lds(p.a_scales + o.sa[i] + kc * 4,
                                     stage + Cfg::kCodesA + Cfg::kCodesB +
                                         (i * Cfg::kThreads + wave_slot) * 4,
                                     4, 0, 0);
#pragma unroll
  for (int i = 0; i < Cfg::kWordsB; ++i)
    __builtin_amdgcn_global_load_lds(p.w_scales + o.sb[i] + kc * 4,
                                     stage + Cfg::kCodesA + Cfg::kCodesB + Cfg::kScalesA +
                                         (i * Cfg::kThreads + wave_slot) * 4,
                                     4, 0, 0);
}

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

// One K chunk of a wavefront's fragments, read from LDS: FM + FN code words of 16 bytes (32
// codes) and one 16-byte scale group per operand.
template <int FM, int FN>
struct Frags {
  uint4 qa[FM];
  uint4 qb[FN];
  uint4 sa;
  uint4 sb;
};

template <int FM, int FN>
__device__ __forceinline__ void read_frags(const uint8_t* stage, int a_frag, int b_frag, int a_scl,
                                           int b_scl, Frags<FM, FN>& f) {
#pragma unroll
  for (int i = 0; i < FM; ++i) f.qa[i] = *reinterpret_cast<const uint4*>(stage + a_frag + i * 1024);
#pragma unroll
  for (int j = 0; j < FN; ++j) f.qb[j] = *reinterpret_cast<const uint4*>(stage + b_frag + j * 1024);
  f.sa = *reinterpret_cast<const uint4*>(stage + a_scl);
  f.sb = *reinterpret_cast<const uint4*>(stage + b_scl);
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
  const uint32_t swa[4] = {f.sa.x, f.sa.y, f.sa.z, f.sa.w};
  const uint32_t swb[4] = {f.sb.x, f.sb.y, f.sb.z, f.sb.w};
#pragma unroll
  for (int i = 0; i < FM; ++i)
    sa[i] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(swa[i] >> sh, 1.0f, false);
#pragma unroll
  for (int j = 0; j < FN; ++j)
    sb[j] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(swb[j] >> sh, 1.0f, false);
}

// Wait until this wavefront's copies of the chunk in `stage` have landed, meet the other
// wavefronts (after which the chunk is complete in LDS and every wavefront has read its fragments
// of the chunk before it), and read this lane's fragments.  The scheduling fences keep the work
// issued before this point ahead of the wait.
template <int FM, int FN>
__device__ __forceinline__ void sync_and_read(const uint8_t* stage, int a_frag, int b_frag,
                                              int a_scl, int b_scl, Frags<FM, FN>& f) {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0x3F70);  // vmcnt(0)
  __builtin_amdgcn_s_barrier();
  read_frags(stage, a_frag, b_frag, a_scl, b_scl, f);
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

// MFMAs of step 2 issued before the mid-chunk barrier: they keep the matrix core busy while the
// wavefronts meet.
constexpr int kPreBarrierMfma = 4;

// Schedule of the MFMAs after the mid-chunk barrier: the next chunk's LDS reads (two per MFMA) and
// the copies of the chunk after it go out between MFMAs, with the decode VALU spread over all of
// them, rather than as one block in front of the MFMAs.
template <int FM, int FN, int NDS, int NVM>
__device__ __forceinline__ void interleave_after_barrier() {
  constexpr int kM = FM * FN - kPreBarrierMfma;
  constexpr int kDsMfma = (NDS + 1) / 2;  // MFMAs carrying two LDS reads
  constexpr int kValu = (8 * (FM + FN) + NVM + kM - 1) / kM + 1;
#pragma unroll
  for (int k = 0; k < kM; ++k) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    if (k < kDsMfma) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS read
    else if (k - kDsMfma < NVM) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);  // VMEM
    __builtin_amdgcn_sched_group_barrier(0x002, kValu, 0);  // VALU
  }
}

// One K chunk, software-pipelined with the next.  The MFMAs of steps 0-1 of chunk kc run under
// the decode of steps 1-2.  The first MFMAs of step 2 are issued; then every wavefront waits for
// its own copies of chunk kc+1 and meets the others at a barrier (chunk kc+1 is complete in LDS,
// and every wavefront has read chunk kc, whose stage is free).  The remaining MFMAs of step 2 run
// under the LDS reads of chunk kc+1's fragments, the copies of chunk kc+2 (`issue`, into chunk
// kc's stage) and the decode of step 3; the MFMAs of step 3 run under the decode of the next
// chunk's step 0.  On entry `cur` holds chunk kc's fragments and a0/b0 its decoded step 0; on exit
// (HAS_NEXT) `nxt` holds chunk kc+1's fragments and a0/b0 its decoded step 0.
template <bool HAS_NEXT, int NVM, int FM, int FN, class Issue>
__device__ __forceinline__ void pipelined_chunk(const Frags<FM, FN>& cur, Frags<FM, FN>& nxt,
                                                const uint8_t* nstage, int a_frag, int b_frag,
                                                int a_scl, int b_scl, half2_t (&sa)[FM],
                                                half2_t (&sb)[FN], half8_t (&a0)[FM],
                                                half8_t (&b0)[FN], half8_t (&a1)[FM],
                                                half8_t (&b1)[FN], uint32_t sh,
                                                floatx16 (&acc)[FM][FN], Issue&& issue) {
  mfma_step(a0, b0, acc);
  decode_step<1>(cur, sa, sb, a1, b1);
  interleave_mfma_valu<FM, FN>();
  mfma_step(a1, b1, acc);
  decode_step<2>(cur, sa, sb, a0, b0);
  interleave_mfma_valu<FM, FN>();
  __builtin_amdgcn_sched_barrier(0);
  mfma_range<0, kPreBarrierMfma>(a0, b0, acc);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (HAS_NEXT) {
    __builtin_amdgcn_s_waitcnt(0x3F70);  // vmcnt(0): this lane's copies of chunk kc+1 landed
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    read_frags(nstage, a_frag, b_frag, a_scl, b_scl, nxt);
    issue();
  }
  mfma_range<kPreBarrierMfma, FM * FN>(a0, b0, acc);
  decode_step<3>(cur, sa, sb, a1, b1);
  interleave_after_barrier<FM, FN, HAS_NEXT ? FM + FN + 2 : 0, HAS_NEXT ? NVM : 0>();
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
// wavefront's sub-tile) at a time.  Each lane writes its four-column pieces into the wavefront's
// own staging rows, then reads back four consecutive columns of one row, so that a wavefront store
// covers two rows x 512 bytes -- whole cache lines, not 32 rows x 32 bytes.  The staging area
// belongs to one wavefront and LDS instructions of a wavefront execute in order, so no barrier is
// needed.  Rows and columns past the matrix are masked at the store; a lane stores its four
// columns as one vector when they are all inside and rows of C start 16-byte aligned (`vec`).
template <int FN>
constexpr int kEpiStride = FN * 32 + 4;  // floats per staged row; the pad spreads rows over banks

template <bool BF16, int FM, int FN>
__device__ __forceinline__ void store_tile(const GemmArgs& p, const floatx16 (&acc)[FM][FN],
                                           const float* alpha, float* epi, int m0, int n0, int wm,
                                           int wn, int lane, bool vec, bool interior) {
  using OutT = typename std::conditional<BF16, uint16_t, float>::type;
  OutT* const c = reinterpret_cast<OutT*>(p.c);
  constexpr int S = kEpiStride<FN>;
  const int r = lane & 31, h = lane >> 5;
  const int cc = (lane & 31) * 4;  // read-back columns of this lane within the wavefront's 128
  const int n = n0 + wn * FN * 32 + cc;
  const floatx4 al = *reinterpret_cast<const floatx4*>(alpha + wn * FN * 32 + cc);
  if (interior) {
    // the tile lies inside C and rows are 16-byte aligned: no masks, and the 16 read-backs of a
    // fragment row are all issued before the first store, so their LDS latency overlaps
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          *reinterpret_cast<floatx4*>(epi + r * S + j * 32 + 8 * q + 4 * h) =
              floatx4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                      acc[i][j][4 * q + 3]};
      floatx4 x[16];
#pragma unroll
      for (int t = 0; t < 16; ++t) x[t] = *reinterpret_cast<const floatx4*>(epi + (2 * t + h) * S + cc);
      OutT* const dst = c + (int64_t)(m0 + wm * FM * 32 + i * 32 + h) * p.ldc + n;
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const floatx4 v = {x[t][0] * al[0], x[t][1] * al[1], x[t][2] * al[2], x[t][3] * al[3]};
        if constexpr (BF16) {
          const uint32_t lo = f32_to_bf16_rne(v[0]) | ((uint32_t)f32_to_bf16_rne(v[1]) << 16);
          const uint32_t hi = f32_to_bf16_rne(v[2]) | ((uint32_t)f32_to_bf16_rne(v[3]) << 16);
          *reinterpret_cast<uint2*>(dst + (int64_t)(2 * t) * p.ldc) = uint2{lo, hi};
        } else {
          *reinterpret_cast<floatx4*>(dst + (int64_t)(2 * t) * p.ldc) = v;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    return;
  }
  const bool full = vec && n + 3 < p.N;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<floatx4*>(epi + r * S + j * 32 + 8 * q + 4 * h) =
            floatx4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                    acc[i][j][4 * q + 3]};
    const int mb = m0 + wm * FM * 32 + i * 32 + h;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const floatx4 x = *reinterpret_cast<const floatx4*>(epi + (2 * t + h) * S + cc);
      const floatx4 v = {x[0] * al[0], x[1] * al[1], x[2] * al[2], x[3] * al[3]};
      const int m = mb + 2 * t;
      if (m >= p.M) continue;
      OutT* const dst = c + (int64_t)m * p.ldc + n;
      if (full) {
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
    // one fragment row at a time: its accumulators are read into registers only here
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Main kernel, persistent: workgroup b runs tiles b, b + G, b + 2G, ... (G = grid size, at most
// one workgroup per compute unit).  Two LDS stages filled by direct global->LDS copies, two
// register sets of fragments.  In the middle of K chunk kc (after its second MFMA step) every
// wavefront waits for its own copies of chunk kc+1, meets the others at a barrier (chunk kc+1 is
// then complete in LDS and every wavefront has read chunk kc, whose stage is free), reads its
// fragments of chunk kc+1, and issues the copies of chunk kc+2 into chunk kc's stage.  The
// remaining MFMA steps of chunk kc then cover the LDS reads and the decode of chunk kc+1's first
// step, so the matrix core does not idle across chunks.
// The K loop is unrolled by 2 so each stage and register set is named statically; past the last
// chunk, reads and copies are clamped to it (redundant, never used), keeping the loop branch-free.
// Between tiles, the copies of the next tile's first two chunks are issued before the stores of
// the finished tile, so the store traffic and the next tile's first loads are in flight together.
// Each lane copies into LDS slots of its own wavefront only, and waits for its own copies before
// issuing the next tile's, so stages never see two tiles' copies race.
template <int WAVES_M, int WAVES_N, int FM, int FN>
__global__ void __launch_bounds__(WAVES_M * WAVES_N * 64, 1)
gemm_tiled_kernel(GemmArgs p, uint32_t tiles_m, uint32_t tiles_n) {
  using Cfg = TileCfg<WAVES_M, WAVES_N, FM, FN>;
  __shared__ __attribute__((aligned(16))) uint8_t s0[Cfg::kStage];
  __shared__ __attribute__((aligned(16))) uint8_t s1[Cfg::kStage];
  // per-column epilogue factors of the current tile, double-buffered by tile parity
  __shared__ __attribute__((aligned(16))) float alpha_s[2][Cfg::BN];
  // epilogue staging, one area of 32 rows per wavefront
  __shared__ __attribute__((aligned(16))) float epi_s[WAVES_M * WAVES_N][32 * kEpiStride<FN>];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave / WAVES_N;
  const int wn = wave % WAVES_N;
  const int h = lane >> 5;
  const int r = lane & 31;
  const uint32_t sh = 16u * (uint32_t)h;  // lane half h uses scale bytes 2h, 2h+1
  const uint32_t ntiles = tiles_m * tiles_n;
  const int nchunks = p.K / 64;
  const int last = nchunks - 1;
  const float ga = *p.a_g;
  const bool vec = (p.ldc & 3) == 0;  // rows of C start 16-byte aligned (C itself is)

  // LDS read offsets of this lane's fragments and scale groups (within a stage)
  const int a_frag = (wm * FM) * 1024 + lane * 16;
  const int b_frag = Cfg::kCodesA + (wn * FN) * 1024 + lane * 16;
  const int a_scl = Cfg::kCodesA + Cfg::kCodesB + (wm * 32 + r) * FM * 4;
  const int b_scl = Cfg::kCodesA + Cfg::kCodesB + Cfg::kScalesA + (wn * 32 + r) * FN * 4;

  uint32_t v = blockIdx.x;
  uint32_t tmi, tni;
  tile_coords(v, tiles_m, tiles_n, tmi, tni);
  int m0 = (int)tmi * Cfg::BM;
  int n0 = (int)tni * Cfg::BN;
  {
    const int tid_t = threadIdx.x;
    RowOffsets<Cfg> ro;
    row_offsets<Cfg, FM, FN>(p, m0, n0, tid_t, ro);
    issue_chunk<Cfg>(p, ro, 0, s0);
    issue_chunk<Cfg>(p, ro, min(1, last), s1);
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

    // chunk 0 into registers (chunk 1 is already in flight into s1)
    sync_and_read(s0, a_frag, b_frag, a_scl, b_scl, f0);
    decode_scales(f0, sh, sa, sb);
    decode_step<0>(f0, sa, sb, a0, b0);

    constexpr int kCopies = Cfg::kPiecesA + Cfg::kPiecesB + Cfg::kWordsA + Cfg::kWordsB;
    int kc = 0;
    for (; kc + 1 < nchunks; kc += 2) {
      // chunk kc (in f0; stage s0), chunk kc+1 in flight into s1
      pipelined_chunk<true, kCopies>(f0, f1, s1, a_frag, b_frag, a_scl, b_scl, sa, sb, a0, b0,
                                     a1, b1, sh, acc,
                                     [&] { issue_chunk<Cfg>(p, ro, min(kc + 2, last), s0); });
      // chunk kc+1 (in f1; stage s1), chunk kc+2 in flight into s0
      pipelined_chunk<true, kCopies>(f1, f0, s0, a_frag, b_frag, a_scl, b_scl, sa, sb, a0, b0,
                                     a1, b1, sh, acc,
                                     [&] { issue_chunk<Cfg>(p, ro, min(kc + 3, last), s1); });
    }
    if (kc < nchunks)  // odd number of chunks: the last one is in f0
      pipelined_chunk<false, kCopies>(f0, f1, s1, a_frag, b_frag, a_scl, b_scl, sa, sb, a0, b0,
                                      a1, b1, sh, acc, [] {});
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
    if (more) {
      tile_coords(v, tiles_m, tiles_n, tmi, tni);
      m0 = (int)tmi * Cfg::BM;
      n0 = (int)tni * Cfg::BN;
      RowOffsets<Cfg> ron;
      row_offsets<Cfg, FM, FN>(p, m0, n0, tid_e, ron);
      issue_chunk<Cfg>(p, ron, 0, s0);
      issue_chunk<Cfg>(p, ron, min(1, last), s1);
    }
    const bool interior = vec && tm0 + Cfg::BM <= p.M && tn0 + Cfg::BN <= p.N;
    if (p.c_bf16)
      store_tile<true>(p, acc, alpha_s[par], epi_s[wave_e], tm0, tn0, wave_e / WAVES_N,
                       wave_e % WAVES_N, lane_e, vec, interior);
    else
      store_tile<false>(p, acc, alpha_s[par], epi_s[wave_e], tm0, tn0, wave_e / WAVES_N,
                        wave_e % WAVES_N, lane_e, vec, interior);
    if (!more) break;
  }
}

#ifndef NVFP4_TILED_CFG
#define NVFP4_TILED_CFG 2, 2, 4, 4
#endif

template <int WAVES_M, int WAVES_N, int FM, int FN>
hipError_t launch_tiled_cfg(const GemmArgs& a, hipStream_t stream) {
  using Cfg = TileCfg<WAVES_M, WAVES_N, FM, FN>;
  const uint32_t tiles_m = (a.M + Cfg::BM - 1) / Cfg::BM;
  const uint32_t tiles_n = (a.N + Cfg::BN - 1) / Cfg::BN;
  // one workgroup per compute unit (the kernel's registers allow one per compute unit), each
  // walking its share of the tiles
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const uint32_t ntiles = tiles_m * tiles_n;
  const uint32_t grid = min(ntiles, (uint32_t)max(cus, 1));
  hipLaunchKernelGGL((gemm_tiled_kernel<WAVES_M, WAVES_N, FM, FN>), dim3(grid),
                     dim3(Cfg::kThreads), 0, stream, a, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_general(const GemmArgs& a, hipStream_t stream) {
  const uint32_t tiles_m = (a.M + 63) / 64;
  const uint32_t tiles_n = (a.N + 63) / 64;
  hipLaunchKernelGGL(gemm_general_kernel, dim3(tiles_m * tiles_n), dim3(256), 0, stream, a,
                     tiles_n);
  return hipGetLastError();
}

hipError_t launch_gemm_tiled(const GemmArgs& a, hipStream_t stream) {
  return launch_tiled_cfg<NVFP4_TILED_CFG>(a, stream);
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
