// Block-tile bf16 GEMM core for gfx950 (CDNA4), used by every kernel of the
// fused linear cross-entropy head.
//
// A block of 256 threads (4 wave64s, one per SIMD) owns a 256 x 256 output
// tile C[m][n] = sum_k A[m][k] * B[n][k]. Both operands are staged through LDS
// in the same K-contiguous layout, 64 K-elements per stage, two stages
// (128 KiB of LDS). Each wave computes a 128 x 128 sub-tile with
// v_mfma_f32_32x32x16_bf16 (4 x 4 blocks of 32 x 32, fp32 accumulators).
//
// Operands in global memory come in two layouts:
//   KMAJOR  element (r, k) at ptr[r * ld + k]   (K contiguous)
//   RMAJOR  element (r, k) at ptr[k * ld + r]   (rows contiguous)
// KMAJOR tiles are copied to LDS as 16-byte chunks. RMAJOR tiles are loaded as
// 8 x 8 element blocks (eight 16-byte row segments) and transposed in
// registers before the LDS store, so the MFMA operand reads are always one
// 16-byte LDS read per lane.
//
// LDS tile layout: row r (0..255) holds 64 bf16 = eight 16-byte chunks; chunk
// c is stored at position c ^ (r & 7). Eight consecutive rows reading the same
// logical chunk therefore touch eight distinct 16-byte bank groups.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flce {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kTile = 256;                    // M and N extent of a block tile
constexpr int kBK = 64;                       // K extent of one LDS stage
constexpr int kThreads = 256;                 // 4 waves of 64
constexpr int kStageElems = kTile * kBK;      // elements per operand per stage
constexpr int kLdsElems = 4 * kStageElems;    // 2 stages x 2 operands (128 KiB)

enum { KMAJOR = 0, RMAJOR = 1 };

struct Operand {
  const uint16_t* ptr;  // bf16 bits
  int64_t ld;           // leading dimension, elements
  int64_t rows;         // valid rows; rows >= this read as zero
};

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

// ---- global -> registers ---------------------------------------------------
//
// Loads go through raw buffer resources: a 32-bit byte offset per lane, and the
// hardware returns zeros for any offset at or past the resource's size. Tails
// (rows past `rows`, K past `kend`) are handled that way, with no branches.

constexpr uint32_t kOOB = 0x80000000u;  // an offset past every resource's size

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const uint32_t n = bytes <= 0 ? 0u : (bytes >= 0x7FFFFFFFll ? 0x7FFFFFFFu : (uint32_t)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, 0x00020000);
}

__device__ __forceinline__ u32x4_t buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
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

// KMAJOR: 2048 chunks of 8 elements per tile; thread t takes row t/8 + 32q,
// chunk t%8, for q = 0..7. The resource starts at row r0 and ends at `rows`.
__device__ __forceinline__ void load_kmajor(const Operand& op, int64_t r0, int64_t k0,
                                            int64_t kend, u32x4_t (&buf)[8]) {
  const int t = threadIdx.x;
  const int rowb = t >> 3, kc = t & 7;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(op.ptr + r0 * op.ld, (op.rows - r0) * op.ld * 2);
  const bool kok = k0 + kc * 8 < kend;
  const uint32_t base = (uint32_t)((rowb * op.ld + k0 + kc * 8) * 2);
  const uint32_t step = (uint32_t)(32 * op.ld * 2);
#pragma unroll
  for (int q = 0; q < 8; ++q) buf[q] = buf_load16(rs, kok ? base + q * step : kOOB);
}

// RMAJOR: thread t owns the 8 x 8 block (rows 8*(t>>3).., k 8*(t&7)..). The
// resource starts at K row k0 and ends at kend. rows must be a multiple of 8
// so a block is either fully valid or not.
__device__ __forceinline__ void load_rmajor(const Operand& op, int64_t r0, int64_t k0,
                                            int64_t kend, u32x4_t (&buf)[8]) {
  const int t = threadIdx.x;
  const int rb = t >> 3, kb = t & 7;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(op.ptr + k0 * op.ld, (kend - k0) * op.ld * 2);
  const bool rok = r0 + rb * 8 < op.rows;
  const uint32_t base = (uint32_t)(((int64_t)kb * 8 * op.ld + r0 + rb * 8) * 2);
  const uint32_t step = (uint32_t)(op.ld * 2);
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) buf[kk] = buf_load16(rs, rok ? base + kk * step : kOOB);
}

template <int L>
__device__ __forceinline__ void load_tile(const Operand& op, int64_t r0, int64_t k0, int64_t kend,
                                          u32x4_t (&buf)[8]) {
  if constexpr (L == KMAJOR) load_kmajor(op, r0, k0, kend, buf);
  else load_rmajor(op, r0, k0, kend, buf);
}

// ---- registers -> LDS --------------------------------------------------------

__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * kBK + ((chunk ^ (row & 7)) << 3);
}

__device__ __forceinline__ void store_kmajor(uint16_t* lds, const u32x4_t (&buf)[8]) {
  const int t = threadIdx.x;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int c = t + q * kThreads;
    const int row = c >> 3, kc = c & 7;
    *reinterpret_cast<u32x4_t*>(lds + lds_off(row, kc)) = buf[q];
  }
}

// buf[kk] holds rows 8*rb .. 8*rb+7 (two per dword) at k = 8*kb + kk. Row j of
// the block gets dword q = (k 2q, k 2q+1) = (buf[2q] elem j, buf[2q+1] elem j).
__device__ __forceinline__ void store_rmajor(uint16_t* lds, const u32x4_t (&buf)[8]) {
  const int t = threadIdx.x;
  const int rb = t >> 3, kb = t & 7;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    u32x4_t o;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t lo = buf[2 * q][j >> 1];
      const uint32_t hi = buf[2 * q + 1][j >> 1];
      o[q] = (j & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
    }
    const int row = rb * 8 + j;
    *reinterpret_cast<u32x4_t*>(lds + lds_off(row, kb)) = o;
  }
}

template <int L>
__device__ __forceinline__ void store_tile(uint16_t* lds, const u32x4_t (&buf)[8]) {
  if constexpr (L == KMAJOR) store_kmajor(lds, buf);
  else store_rmajor(lds, buf);
}

// ---- MFMA on one LDS stage ---------------------------------------------------

// Wave (wm, wn) multiplies rows [wm*128, +128) of A by rows [wn*128, +128) of
// B over the stage's 64 K values. Operand lane layout of the 32x32x16 MFMA:
// lane l supplies row l%32 and K elements 8*(l/32) .. +7 of the 16-wide step.
__device__ __forceinline__ void mma_stage(const uint16_t* sA, const uint16_t* sB, int wm, int wn,
                                          f32x16_t (&acc)[4][4]) {
  const int lane = threadIdx.x & 63;
  const int lr = lane & 31, lh = lane >> 5;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    bf16x8_t a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      a[i] = *reinterpret_cast<const bf16x8_t*>(sA + lds_off(wm * 128 + i * 32 + lr, kk * 2 + lh));
#pragma unroll
    for (int j = 0; j < 4; ++j)
      b[j] = *reinterpret_cast<const bf16x8_t*>(sB + lds_off(wn * 128 + j * 32 + lr, kk * 2 + lh));
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
}

// Accumulator element r of block (i, j) of wave (wm, wn), lane l, sits at
// tile row  wm*128 + i*32 + 8*(r/4) + 4*(l/32) + r%4  and
// tile col  wn*128 + j*32 + l%32.
__device__ __forceinline__ int acc_row(int wm, int i, int r, int lane) {
  return wm * 128 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
}
__device__ __forceinline__ int acc_col(int wn, int j, int lane) {
  return wn * 128 + j * 32 + (lane & 31);
}

// ---- the pipelined tile loop -------------------------------------------------

// Runs `ntiles` output tiles back to back, each over K in [kbeg, kend). The
// last K step of a tile already loads and stages the next tile's first K
// slice, so the pipeline does not drain between tiles. coord(tile, a_row0,
// b_row0) names the tile; epi(tile, acc, wm, wn) consumes the accumulators
// after the tile's last block barrier (it must not touch LDS).
template <int LA, int LB, class Coord, class Epi>
__device__ __forceinline__ void gemm_tiles(const Operand& A, const Operand& B, int ntiles,
                                           Coord coord, int64_t kbeg, int64_t kend, Epi epi,
                                           uint16_t* lds) {
  const int nk = (int)((kend - kbeg + kBK - 1) / kBK);
  if (ntiles <= 0 || nk <= 0) return;
  const int wave = threadIdx.x >> 6;
  const int wm = wave & 1, wn = wave >> 1;

  u32x4_t ra[8], rb[8];
  int64_t ar, br;
  coord(0, ar, br);
  load_tile<LA>(A, ar, kbeg, kend, ra);
  load_tile<LB>(B, br, kbeg, kend, rb);
  store_tile<LA>(lds, ra);
  store_tile<LB>(lds + kStageElems, rb);
  __syncthreads();

  int stage = 0;
  for (int tile = 0; tile < ntiles; ++tile) {
    f32x16_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    for (int kt = 0; kt < nk; ++kt) {
      const bool last = kt + 1 == nk;
      const bool more = !last || tile + 1 < ntiles;
      if (more) {
        int64_t k0 = kbeg + (int64_t)(kt + 1) * kBK;
        if (last) {
          coord(tile + 1, ar, br);
          k0 = kbeg;
        }
        load_tile<LA>(A, ar, k0, kend, ra);
        load_tile<LB>(B, br, k0, kend, rb);
      }
      uint16_t* cur = lds + stage * (2 * kStageElems);
      uint16_t* nxt = lds + (stage ^ 1) * (2 * kStageElems);
      mma_stage(cur, cur + kStageElems, wm, wn, acc);
      if (more) {
        store_tile<LA>(nxt, ra);
        store_tile<LB>(nxt + kStageElems, rb);
      }
      __syncthreads();
      stage ^= 1;
    }
    epi(tile, acc, wm, wn);
  }
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
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return bf16_bits(lo) | (bf16_bits(hi) << 16);
}

}  // namespace flce
