// Block-tile bf16 GEMM core for gfx950 (CDNA4), shared by every contraction of
// the fused linear cross-entropy head.
//
// A block of 512 threads (8 wave64s, two per SIMD) owns a 256 x 256 output
// tile C[m][n] = sum_k A[m][k] * B[n][k], fp32 accumulators. Wave w computes
// rows [128*(w&1), +128) x cols [64*(w>>1), +64) with
// v_mfma_f32_32x32x16_bf16 (4 x 2 blocks of 32 x 32, 128 accumulators per
// lane). Two K-loop schedules share the stages and loaders below: a ping-pong
// one (the two waves of a SIMD alternate between MFMAs and memory work, so
// the matrix unit is fed while the other wave waits) for contractions whose
// operands are both blocked, and an interleaved one for the logit tiles, whose
// transposing LDS reads are too slow to fit in a ping-pong half period.
//
// Operand layout ("blocked"). Every GEMM operand is first arranged in HBM as
// strips of 256 rows; a strip is a sequence of K blocks of 32 values, and a
// block is 16 KiB holding exactly the bytes one LDS stage of that operand
// needs, in LDS order: row r (0..255) takes 64 bytes, its four 16-byte chunks
// of 8 K values stored at positions c ^ ((r >> 2) & 3). Rows and K values past
// the operand's extent are zero. The arrangement pays off twice:
//   * global -> LDS is a straight copy: each DMA instruction
//     (buffer_load_dwordx4 ... lds) moves 1 KiB of contiguous memory, and a
//     strip is streamed front to back, so HBM sees long sequential runs rather
//     than one 64-byte piece per row;
//   * every fragment is read with ds_read_b128 (full LDS rate on gfx950; the
//     transposing ds_read_b64_tr_b16 runs at well under half of it).
// The producers of blocked operands (pack kernels, the logit-gradient
// epilogue) live in flce_kernels.hpp.
//
// The A operand may instead come straight from a row-contiguous tensor
// (element (r, k) at ptr[k * ld + r], e.g. the [H,V] weight as the
// vocabulary x H operand): one DMA instruction then moves two K rows of 512
// contiguous bytes, and fragments are read with the gfx950 transposing read
// ds_read_b64_tr_b16. This spares a transposed copy of the weight; the slower
// LDS reads only touch one of the two operands.
//
// Four LDS stages (16 KiB per operand each, 128 KiB in all) keep two to three
// K blocks in flight while one is consumed; every stage is a separate
// __shared__ array.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "flce_layout.hpp"

namespace flce {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

constexpr int kStages = 4;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kDmaBlocks = kBlockBytes / 1024 / kWaves;  // 1 KiB DMA pieces per wave per block

// Byte offset of element (r, k) inside a block (r < 256, k < 32).
__host__ __device__ __forceinline__ int blk_byte(int r, int k) {
  return r * 64 + ((((k >> 3) ^ ((r >> 2) & 3))) << 4) + (k & 7) * 2;
}

// One strip of a blocked operand.
struct Strip {
  const uint16_t* ptr;  // block 0 of the strip
  int nkb;              // K blocks the strip holds (bounds every load)
};

// ---- block numbering ------------------------------------------------------------

// Hardware dispatches workgroup p to XCD p % 8. Renumber so that logical ids
// [x*q + min(x,rem), ...) run on XCD x: consecutive logical ids share an XCD
// and its L2.
__device__ __forceinline__ int xcd_remap(int p, int G) {
  const int q = G >> 3, rem = G & 7;
  const int x = p & 7;
  return x * q + (x < rem ? x : rem) + (p >> 3);
}

// Maps logical block id L onto a rows x cols grid of output tiles, walking
// `g` tile-rows at a time so that a run of consecutive ids (the blocks that
// share an XCD) covers a compact g x (run/g) patch: both operands of that patch
// are reused from the XCD's L2.
__device__ __forceinline__ void group_map(int L, int rows, int cols, int g, int& r, int& c) {
  const int group = L / (g * cols);
  const int first = group * g;
  const int gr = rows - first < g ? rows - first : g;
  const int w = L - first * cols;
  r = first + w % gr;
  c = w / gr;
}

// ---- buffer resources, waits, barriers -------------------------------------------

constexpr uint32_t kOOB = 0x80000000u;  // an offset past every resource's size

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const uint32_t n = bytes <= 0 ? 0u : (bytes >= 0x7FFFFFFFll ? 0x7FFFFFFFu : (uint32_t)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, 0x00020000);
}
__device__ __forceinline__ float buf_load_f32(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0));
}
__device__ __forceinline__ void buf_store_f32(float v, __amdgpu_buffer_rsrc_t r, uint32_t voff) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, voff, 0, 0);
}
__device__ __forceinline__ void buf_store_u16(uint32_t v, __amdgpu_buffer_rsrc_t r, uint32_t voff) {
  __builtin_amdgcn_raw_buffer_store_b16((unsigned short)v, r, voff, 0, 0);
}
__device__ __forceinline__ void buf_store_u32x2(u32x2_t v, __amdgpu_buffer_rsrc_t r, uint32_t voff) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, voff, 0, 0);
}
__device__ __forceinline__ u32x2_t buf_load_u32x2(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, voff, 0, 0);
}
typedef float f32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4_t buf_load_f32x4(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}
__device__ __forceinline__ void buf_store_f32x4(f32x4_t v, __amdgpu_buffer_rsrc_t r, uint32_t voff) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, voff, 0, 0);
}
__device__ __forceinline__ void buf_store_u32x4(u32x4_t v, __amdgpu_buffer_rsrc_t r, uint32_t voff) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, 0, 0);
}

// Keeps the compiler from hoisting work that depends on `x` out of a loop.
template <class T>
__device__ __forceinline__ void opaque(T& x) {
  __asm__ volatile("" : "+v"(x));
}

// s_waitcnt on vmcnt only (expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (0x0 << 8) | (0x3 << 14));
}
// A block barrier that does not drain outstanding global loads (unlike
// __syncthreads, which waits for every one of them): the stages still in
// flight stay in flight.
__device__ __forceinline__ void block_barrier() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

// ---- global -> LDS DMA of one block -------------------------------------------------

// Wave-uniform index of the calling wave (an SGPR value, so LDS addresses
// derived from it need no VGPR).
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

// One 1 KiB global -> LDS DMA instruction (buffer_load_dwordx4 ... lds): lane
// l moves the 16 bytes at voff + soff (+16 l is in voff) of resource rs to
// LDS byte lds + 16 l. It is issued from inline assembly so that the
// compiler, which cannot tell the LDS stages apart through M0, does not make
// fragment reads of one stage wait for the DMA of another: every wait on these
// loads is an explicit s_waitcnt vmcnt in the main loop below. The
// instruction writes no register, so nothing the compiler allocates is left
// pending.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rs, const char* lds, uint32_t voff,
                                          uint32_t soff) {
  asm volatile(
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen lds"
      :
      : "{m0}"((uint32_t)(uintptr_t)(const lds_void_t*)lds), "v"(voff), "s"(rs), "s"(soff)
      : "memory");
}

// Wave w copies pieces [w * kDmaBlocks, +kDmaBlocks) of 1 KiB; lane l moves
// bytes [16 l, +16) of each piece. The resource is rebased to the block and
// has size 0 for block indices at or past the strip's end (no memory access;
// zeros land in LDS), so every step issues the same number of loads; the
// piece index rides in the scalar offset, so one VGPR serves every piece.
struct Dma {
  const uint16_t* ptr;
  uint32_t off;
  int wofs;
  int nkb;
  __device__ __forceinline__ void init(const Strip& s) {
    const int lane = threadIdx.x & 63;
    ptr = s.ptr;
    wofs = wave_id() * kDmaBlocks * 1024;
    off = (uint32_t)(wofs + lane * 16);
    nkb = s.nkb;
  }
  __device__ __forceinline__ void issue(char* dst, int kb) const {
    const bool ok = kb < nkb;
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(ptr + (int64_t)(ok ? kb : 0) * kBlockElems, ok ? kBlockBytes : 0);
#pragma unroll
    for (int q = 0; q < kDmaBlocks; ++q) lds_dma16(rs, dst + wofs + q * 1024, off, q * 1024);
  }
};

// A operand taken from a blocked strip, K blocks [kb0, kb0 + nk).
struct BlockedA {
  Dma d;
  int kb0;
  __device__ __forceinline__ void init(const Strip& s, int kb0_) {
    d.init(s);
    kb0 = kb0_;
  }
  __device__ __forceinline__ void issue(char* dst, int kt, int nk) const {
    d.issue(dst, kt < nk ? kb0 + kt : d.nkb);
  }
};

// LDS layout of a row-contiguous stage: K row k is 512 bytes (all 256 tile
// rows); the 64-byte segment of tile rows [32s, 32s+32) sits at position
// s ^ (k & 3), so the four K rows a transposing read touches land in four
// distinct bank groups.
__device__ __forceinline__ int rmaj_byte(int k, int m) {
  return k * 512 + ((((m >> 5) ^ (k & 3))) << 6) + (m & 31) * 2;
}

// A operand taken from a row-contiguous tensor: element (r, k) at
// ptr[k * ld + r], tile rows [r0, r0 + 256) of `rows` valid ones, K values
// [kbeg, kend). A 1 KiB DMA piece is 2 K rows x 512 bytes; lane l fetches the
// 16-byte piece whose swizzled slot is l % 32 of K row l / 32. The resource is
// rebased to each stage's first K row and ends at kend, so K tails and blocks
// past the range read as zero. `rows`, r0 and ld must be multiples of 8.
struct RowA {
  const uint16_t* ptr;
  int64_t ld, kbeg, kend;
  uint32_t off[kDmaBlocks];
  __device__ __forceinline__ void init(const uint16_t* p, int64_t ld_, int64_t rows, int64_t r0,
                                       int64_t kb, int64_t ke) {
    const int lane = threadIdx.x & 63, w = wave_id();
    ptr = p;
    ld = ld_;
    kbeg = kb;
    kend = ke;
#pragma unroll
    for (int q = 0; q < kDmaBlocks; ++q) {
      const int k = (w * kDmaBlocks + q) * 2 + (lane >> 5);
      const int slot = lane & 31;
      const int m = (((slot >> 2) ^ (k & 3)) << 5) + (slot & 3) * 8;
      off[q] = r0 + m < rows ? (uint32_t)((k * ld_ + r0 + m) * 2) : kOOB;
    }
  }
  __device__ __forceinline__ void issue(char* dst, int kt, int nk) const {
    const int w = wave_id();
    const int64_t k0 = kbeg + (int64_t)kt * kBK;
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(ptr + k0 * ld, kt < nk ? (kend - k0) * ld * 2 : 0);
#pragma unroll
    for (int q = 0; q < kDmaBlocks; ++q) lds_dma16(rs, dst + (w * kDmaBlocks + q) * 1024, off[q], 0);
  }
};

// ---- LDS -> register operand fragments ---------------------------------------------

// NB blocks of 32 tile rows from row0 (a multiple of 32); 16-wide K step kk
// of a stage. 32x32x16 MFMA lane layout: lane l supplies tile row l % 32 and
// K values 8*(l/32) .. +7 of the step, i.e. chunk 2kk + l/32 of its row.
// Eight consecutive rows reading one logical chunk hit eight distinct 16-byte
// bank groups thanks to the chunk swizzle.
template <int NB>
struct FragSrc {
  static constexpr int kReadsPerStep = NB;
  int base[NB];
  __device__ __forceinline__ void init(int row0) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < NB; ++i) base[i] = blk_byte(row0 + i * 32 + (lane & 31), 8 * (lane >> 5));
  }
  // Chunk 2kk + l/32: step kk = 1 flips bit 5 of the byte offset.
  __device__ __forceinline__ void read(const char* st, int kk, bf16x8_t (&f)[NB]) const {
#pragma unroll
    for (int i = 0; i < NB; ++i)
      f[i] = *reinterpret_cast<const bf16x8_t*>(st + (base[i] ^ (kk << 5)));
  }
};

// Fragments of a row-contiguous stage. ds_read_b64_tr_b16: within each
// 16-lane group, lane i receives element i % 4 of the 8 bytes that lane
// 4j + i/4 addressed, for j = 0..3. Lane a of group g addresses K row
// 8(g/2) + 4h + a/4 at tile rows 16(g%2) + 4(a%4) .. +3, so lane i ends up with
// 4 consecutive K values of tile row 16(g%2) + i; the two reads h = 0, 1 give
// the 8 K values of a 16-wide step.
template <int NB>
struct FragRow {
  static constexpr int kReadsPerStep = 2 * NB;
  int base;
  __device__ __forceinline__ void init(int row0) {
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4, a = lane & 15;
    base = rmaj_byte(8 * (g >> 1) + (a >> 2), row0 + 16 * (g & 1) + 4 * (a & 3));
  }
  // Block i adds 32i to the row: with row0 / 32 a multiple of NB that is an XOR
  // of the segment bits; step kk adds 16 K rows.
  __device__ __forceinline__ void read(const char* st, int kk, bf16x8_t (&f)[NB]) const {
    int b = base;
    opaque(b);
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int o = (b ^ (i << 6)) + kk * 16 * 512;
      const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(st + o));
      const i16x4_t hi =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(st + o + 4 * 512));
      const i16x8_t v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      f[i] = __builtin_bit_cast(bf16x8_t, v);
    }
  }
};

// Accumulator element r of block (i, j) of wave (wm, wn), lane l, sits at
// tile row  wm*128 + i*32 + 8*(r/4) + 4*(l/32) + r%4  and
// tile col  wn*64 + j*32 + l%32.
__device__ __forceinline__ int acc_row(int wm, int i, int r, int lane) {
  return wm * 128 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}
__device__ __forceinline__ int acc_col(int wn, int j, int lane) {
  return wn * 64 + j * 32 + (lane & 31);
}

typedef f32x16_t Acc[4][2];

// LDS for one block: four stages per operand, each a separate array.
#define FLCE_DECLARE_STAGES(sa, sb)                                                   \
  __shared__ __attribute__((aligned(1024))) char sa##_0[flce::kBlockBytes],            \
      sa##_1[flce::kBlockBytes], sa##_2[flce::kBlockBytes], sa##_3[flce::kBlockBytes]; \
  __shared__ __attribute__((aligned(1024))) char sb##_0[flce::kBlockBytes],            \
      sb##_1[flce::kBlockBytes], sb##_2[flce::kBlockBytes], sb##_3[flce::kBlockBytes]; \
  char* const sa[flce::kStages] = {sa##_0, sa##_1, sa##_2, sa##_3};                    \
  char* const sb[flce::kStages] = {sb##_0, sb##_1, sb##_2, sb##_3}

// ---- the pipelined K loop ------------------------------------------------------


// Instruction-class masks of __builtin_amdgcn_sched_group_barrier.
enum : int { SG_MFMA = 0x8, SG_VMEM_RD = 0x20, SG_DS_RD = 0x100 };

// Scheduling groups: 8 MFMAs, each followed by its share of NR LDS reads.
template <int NR, int Q>
__device__ __forceinline__ void sg_mfma_then_reads() {
  __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
  if constexpr ((NR + 7 - Q) / 8 > 0)
    __builtin_amdgcn_sched_group_barrier(SG_DS_RD, (NR + 7 - Q) / 8, 0);
}
template <int NR>
__device__ __forceinline__ void interleave_reads() {
  sg_mfma_then_reads<NR, 0>();
  sg_mfma_then_reads<NR, 1>();
  sg_mfma_then_reads<NR, 2>();
  sg_mfma_then_reads<NR, 3>();
  sg_mfma_then_reads<NR, 4>();
  sg_mfma_then_reads<NR, 5>();
  sg_mfma_then_reads<NR, 6>();
  sg_mfma_then_reads<NR, 7>();
}

// Interleaved schedule: both waves of a SIMD run the same phase of every K
// block, with the fragment reads of the next 16-wide substep spread over the
// MFMAs of the current one and one block barrier per K block. Used where the
// A operand is row-contiguous: its transposing LDS reads take longer than the
// MFMAs of a half period, so the ping-pong schedule below would leave the
// matrix units waiting on them. ASrc: BlockedA or RowA (already initialised by
// the caller); AFrag: the matching fragment reader, FragSrc<4> or FragRow<4>.
// A per-stage callback of the interleaved loop that does nothing.
struct NoStageHook {
  __device__ __forceinline__ void operator()(const char*, int) const {}
};

template <class ASrc, class AFrag>
struct MainloopIL {
  struct Frags {
    bf16x8_t a[4], b[2];
  };
  AFrag fa;
  FragSrc<2> fb;
  ASrc da;
  Dma db;
  int b_kb0;

  __device__ __forceinline__ void frags(const char* a, const char* b, int kk, Frags& f) const {
    fa.read(a, kk, f.a);
    fb.read(b, kk, f.b);
  }
  __device__ __forceinline__ static void mma(const Frags& f, Acc& acc) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
  }
  // Block kt of the K range; past the range both operands get out-of-range
  // offsets.
  __device__ __forceinline__ void issue(char* a, char* b, int kt, int nk) const {
    da.issue(a, kt, nk);
    db.issue(b, kt < nk ? b_kb0 + kt : db.nkb);
  }

  // LDS fragment-read instructions per 16-wide K step.
  static constexpr int kReads = AFrag::kReadsPerStep + FragSrc<2>::kReadsPerStep;

  // One K block, reading stage S: first the DMA of the block three ahead is
  // issued into the stage consumed last step; sub-step 1's fragments are read
  // while sub-step 0's MFMAs run; then this wave's DMA of the next block is
  // awaited and the block synchronises (the next stage is now complete in
  // LDS); the next block's sub-step 0 fragments are read while this block's
  // sub-step 1 MFMAs run (they only need registers).
  // `hook(stage, k)` sees the complete A stage of K block k (kiss - 3) once;
  // its LDS reads finish before the block barrier below, so before any wave
  // refills that stage.
  template <int S, class Hook>
  __device__ __forceinline__ void step(char* const (&sa)[kStages], char* const (&sb)[kStages],
                                       Frags (&f)[2], Acc& acc, int kiss, int nk,
                                       const Hook& hook) {
    constexpr int SI = (S + kStages - 1) % kStages;
    constexpr int SN = (S + 1) % kStages;
    issue(sa[SI], sb[SI], kiss, nk);
    frags(sa[S], sb[S], 1, f[1]);
    hook(sa[S], kiss - (kStages - 1));
    mma(f[0], acc);
    // DMA issue first, then the fragment reads spread over the MFMAs, so the
    // LDS sees a steady stream rather than a burst per wave.
    __builtin_amdgcn_sched_group_barrier(SG_VMEM_RD, 2 * kDmaBlocks, 0);
    interleave_reads<kReads>();
    // The hook's stores, if any, count here too: the wait may then also cover
    // part of the next stage's DMA, never less than this one.
    wait_vmcnt<2 * kDmaBlocks * (kStages - 2)>();
    wait_lgkmcnt0();
    block_barrier();
    frags(sa[SN], sb[SN], 0, f[0]);
    mma(f[1], acc);
    interleave_reads<kReads>();
  }

  // C tile = A x strip B over nk K blocks (B's from bkb0). Leaves every DMA
  // drained and the block synchronised, so callers may reuse the stage arrays
  // afterwards.
  __device__ __forceinline__ void run(char* const (&sa)[kStages], char* const (&sb)[kStages],
                                      const ASrc& A, const Strip& B, int bkb0, int nk, Acc& acc) {
    run(sa, sb, A, B, bkb0, nk, acc, NoStageHook{});
  }
  template <class Hook>
  __device__ __forceinline__ void run(char* const (&sa)[kStages], char* const (&sb)[kStages],
                                      const ASrc& A, const Strip& B, int bkb0, int nk, Acc& acc,
                                      const Hook& hook) {
    const int wave = threadIdx.x >> 6;
    const int wm = wave & 1, wn = wave >> 1;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    if (nk <= 0) return;
    da = A;
    db.init(B);
    b_kb0 = bkb0;
    fa.init(wm * 128);
    fb.init(wn * 64);
#pragma unroll
    for (int s = 0; s + 1 < kStages; ++s) issue(sa[s], sb[s], s, nk);
    wait_vmcnt<2 * kDmaBlocks * (kStages - 2)>();
    block_barrier();
    Frags f[2];
    frags(sa[0], sb[0], 0, f[0]);
    for (int kt = 0; kt < nk; kt += kStages) {
      const int k3 = kt + kStages - 1;
      step<0>(sa, sb, f, acc, k3, nk, hook);
      if (kt + 1 < nk) step<1>(sa, sb, f, acc, k3 + 1, nk, hook);
      if (kt + 2 < nk) step<2>(sa, sb, f, acc, k3 + 2, nk, hook);
      if (kt + 3 < nk) step<3>(sa, sb, f, acc, k3 + 3, nk, hook);
    }
    wait_vmcnt<0>();
    block_barrier();
  }
};


// Ping-pong schedule. The hardware puts wave w of a block on SIMD w % 4, so
// waves 0-3 (the leader group) and 4-7 (the follower group) share each SIMD
// one to one. The two groups run half a K block apart: in every half period
// one group issues the 16 MFMAs of a whole 32-deep K block back to back from
// registers, at raised priority, while the other reads the next block's
// fragments from LDS and issues its part of the global -> LDS DMA; a block
// barrier ends each half period. The matrix unit of each SIMD is thus fed by
// one wave while the other waits on LDS, DMA and the barrier, instead of both
// waves draining it at a common barrier.
//   half period 2k:    leader M(k)          follower DMA(k+3), R(k)
//   half period 2k+1:  leader DMA(k+3), R(k+1)   follower M(k)
// M = MFMAs, R = fragment reads; block b lives in stage b % 4. The DMA of
// block k+3 overwrites the stage of block k-1, which both groups finished
// reading (waited on before their barriers) by the end of half period 2k-1.
// Before the barrier that ends half period 2k every wave has its own pieces of
// block k+1 in LDS: the leader has issued blocks up to k+2 (one may stay in
// flight), the follower up to k+3 (two may).
template <class ASrc, class AFrag>
struct MainloopPP {
  struct Frags {
    bf16x8_t a[2][4], b[2][2];  // both 16-wide substeps of one K block
  };
  AFrag fa;
  FragSrc<2> fb;
  ASrc da;
  Dma db;
  int b_kb0;

  // DMA instructions per block and wave.
  static constexpr int kDma = 2 * kDmaBlocks;

  template <int S>
  __device__ __forceinline__ void issue(char* const (&sa)[kStages], char* const (&sb)[kStages], int kt,
                                        int nk) const {
    da.issue(sa[S], kt, nk);
    db.issue(sb[S], kt < nk ? b_kb0 + kt : db.nkb);
  }
  template <int S>
  __device__ __forceinline__ void read(char* const (&sa)[kStages], char* const (&sb)[kStages],
                                       Frags& f) const {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      fa.read(sa[S], kk, f.a[kk]);
      fb.read(sb[S], kk, f.b[kk]);
    }
  }
  __device__ __forceinline__ static void math(const Frags& f, Acc& acc) {
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[kk][i], f.b[kk][j], acc[i][j], 0, 0, 0);
    __builtin_amdgcn_s_setprio(0);
  }
  // Keeps the scheduler from moving instructions across a phase boundary.
  __device__ __forceinline__ static void fence() { __builtin_amdgcn_sched_barrier(0); }

  // Leader, block k in stage S.
  template <int S>
  __device__ __forceinline__ void lead(char* const (&sa)[kStages], char* const (&sb)[kStages], Frags& f,
                                       Acc& acc, int k, int nk) const {
    math(f, acc);
    fence();
    wait_vmcnt<kDma * (kStages - 3)>();
    block_barrier();
    fence();
    issue<(S + kStages - 1) % kStages>(sa, sb, k + kStages - 1, nk);
    if (k + 1 < nk) read<(S + 1) % kStages>(sa, sb, f);
    wait_lgkmcnt0();
    block_barrier();
    fence();
  }
  // Follower, block k in stage S.
  template <int S>
  __device__ __forceinline__ void follow(char* const (&sa)[kStages], char* const (&sb)[kStages],
                                         Frags& f, Acc& acc, int k, int nk) const {
    issue<(S + kStages - 1) % kStages>(sa, sb, k + kStages - 1, nk);
    read<S>(sa, sb, f);
    wait_lgkmcnt0();
    wait_vmcnt<kDma * (kStages - 2)>();
    block_barrier();
    fence();
    math(f, acc);
    fence();
    block_barrier();
    fence();
  }

  // C tile = A x strip B over nk K blocks (B's from bkb0). Leaves every DMA
  // drained and the block synchronised, so callers may reuse the stage arrays
  // afterwards. Every wave passes the same number of barriers.
  __device__ __forceinline__ void run(char* const (&sa)[kStages], char* const (&sb)[kStages],
                                      const ASrc& A, const Strip& B, int bkb0, int nk, Acc& acc) {
    static_assert(kStages == 4, "the schedule above assumes four stages");
    const int wave = wave_id();
    const int wm = wave & 1, wn = wave >> 1;
    const bool leader = wave < 4;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    if (nk <= 0) return;
    da = A;
    db.init(B);
    b_kb0 = bkb0;
    fa.init(wm * 128);
    fb.init(wn * 64);
    issue<0>(sa, sb, 0, nk);
    issue<1>(sa, sb, 1, nk);
    issue<2>(sa, sb, 2, nk);
    wait_vmcnt<kDma * (kStages - 2)>();
    block_barrier();
    Frags f;
    if (leader) {
      read<0>(sa, sb, f);
      wait_lgkmcnt0();
    }
    block_barrier();
    fence();
    if (leader)
      leader_loop(sa, sb, f, acc, nk);
    else
      follower_loop(sa, sb, f, acc, nk);
    wait_vmcnt<0>();
    block_barrier();
  }

  __device__ __forceinline__ void leader_loop(char* const (&sa)[kStages],
                                              char* const (&sb)[kStages], Frags& f, Acc& acc,
                                              int nk) {
    for (int kt = 0; kt < nk; kt += kStages) {
      lead<0>(sa, sb, f, acc, kt, nk);
      if (kt + 1 < nk) lead<1>(sa, sb, f, acc, kt + 1, nk);
      if (kt + 2 < nk) lead<2>(sa, sb, f, acc, kt + 2, nk);
      if (kt + 3 < nk) lead<3>(sa, sb, f, acc, kt + 3, nk);
    }
  }
  __device__ __forceinline__ void follower_loop(char* const (&sa)[kStages],
                                                char* const (&sb)[kStages], Frags& f, Acc& acc,
                                                int nk) {
    for (int kt = 0; kt < nk; kt += kStages) {
      follow<0>(sa, sb, f, acc, kt, nk);
      if (kt + 1 < nk) follow<1>(sa, sb, f, acc, kt + 1, nk);
      if (kt + 2 < nk) follow<2>(sa, sb, f, acc, kt + 2, nk);
      if (kt + 3 < nk) follow<3>(sa, sb, f, acc, kt + 3, nk);
    }
  }
};

typedef MainloopPP<BlockedA, FragSrc<4>> Mainloop;     // both operands blocked
typedef MainloopIL<RowA, FragRow<4>> MainloopRowA;     // A row-contiguous, B blocked

// Blocked A operand descriptor for Mainloop::run.
__device__ __forceinline__ BlockedA blocked_a(const Strip& s, int kb0) {
  BlockedA a;
  a.init(s, kb0);
  return a;
}

// ---- small numeric helpers ---------------------------------------------------

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegBig = -1e30f;  // finite "minus infinity" for masked logits

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// c * tanh(z / c) = c - 2c / (exp(2z/c) + 1); saturates cleanly to +-c.
// two_l2e_over_c = 2 * log2(e) / c.
__device__ __forceinline__ float softcap_apply(float z, float c, float two_l2e_over_c) {
  const float t = fast_exp2(z * two_l2e_over_c);
  return c - 2.f * c * fast_rcp(t + 1.f);
}

// float -> bf16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
// Two floats -> packed bf16 pair (lo in the low half), round to nearest even,
// with the gfx950 conversion instruction.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{lo, hi}), bf16x2_t));
}

// 4 x 4 transpose of bf16 values across the lanes of a quad (lanes 4q..4q+3).
// On entry lane 4q+a holds X[a][0..3] packed as p0 = (X[a][0], X[a][1]),
// p1 = (X[a][2], X[a][3]); on return it holds (X[0][a], X[1][a]) and
// (X[2][a], X[3][a]). Two DPP stages: swap 2 x 2 blocks between lanes a and
// a ^ 2, then 16-bit halves between lanes a and a ^ 1.
__device__ __forceinline__ u32x2_t quad_transpose_bf16(uint32_t p0, uint32_t p1) {
  const int a = threadIdx.x & 3;
  const bool lo = a < 2;
  const uint32_t sel = lo ? p1 : p0;
  const uint32_t recv = (uint32_t)__builtin_amdgcn_mov_dpp((int)sel, 0x4E, 0xF, 0xF, false);  // [2,3,0,1]
  const uint32_t q0 = lo ? p0 : recv, q1 = lo ? recv : p1;
  const uint32_t o0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)q0, 0xB1, 0xF, 0xF, false);    // [1,0,3,2]
  const uint32_t o1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)q1, 0xB1, 0xF, 0xF, false);
  // Odd lanes keep their high half and take the partner's high half below it,
  // even lanes keep their low half and take the partner's low half above it:
  // one byte permute of {o, q} each (bytes 0-3 of q, 4-7 of o), no branch.
  const uint32_t bsel = (a & 1) ? 0x03020706u : 0x05040100u;
  u32x2_t r;
  r[0] = __builtin_amdgcn_perm(o0, q0, bsel);
  r[1] = __builtin_amdgcn_perm(o1, q1, bsel);
  return r;
}

// The same transpose for fp32 values: lane 4q+a holds X[a][0..3] on entry and
// returns (X[0][a], X[1][a], X[2][a], X[3][a]).
__device__ __forceinline__ float dpp_f32(float x, int ctrl_is_swap2) {
  const int v = __builtin_bit_cast(int, x);
  return __builtin_bit_cast(float, ctrl_is_swap2 ? __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false)
                                                 : __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ f32x4_t quad_transpose_f32(float x0, float x1, float x2, float x3) {
  const int a = threadIdx.x & 3;
  const bool lo = a < 2;
  const float r0 = dpp_f32(lo ? x2 : x0, 1), r1 = dpp_f32(lo ? x3 : x1, 1);
  const float y0 = lo ? x0 : r0, y1 = lo ? x1 : r1, y2 = lo ? r0 : x2, y3 = lo ? r1 : x3;
  const bool ev = (a & 1) == 0;
  const float u0 = dpp_f32(ev ? y1 : y0, 0), u1 = dpp_f32(ev ? y3 : y2, 0);
  return ev ? f32x4_t{y0, u0, y2, u1} : f32x4_t{u0, y1, u1, y3};
}

}  // namespace flce
