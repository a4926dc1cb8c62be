// Kernels of the fused linear cross-entropy + entropy head (gfx950).
//
// Forward:  fwd_prep (label checks, compaction of the valid tokens),
//           pack (hidden) -> fwd_tile -> fwd_combine (-> fwd_reduce)
// Backward: bwd_prep (compaction, per-token gradient constants),
//           zero_ignored_rows, pack (hidden, hidden^T) -> per vocabulary chunk
//           { bwd_dlogits (also writing the weight chunk's image for dH) ->
//             bwd_dx (-> dx_finalize after the last chunk when dH is
//             K-split) -> bwd_dw (-> dw_reduce) }
// Fused (gradient in the forward, when the upstream gradients are known
// before the forward runs): fwd_prep, pack (hidden, hidden^T) ->
//           per chunk of tokens { fwd_tile storing z' - m (bf16; the first
//             chunk also writes the weight's image for dH) ->
//             fwd_combine (+ gradient constants) -> fused_dlogits ->
//             bwd_dx (-> dx_finalize) -> bwd_dw (accumulating over chunks) }
//           (-> fwd_reduce)
// Only the valid tokens, compacted in token order, enter the contractions;
// results are scattered back to the original token rows.
//
// GEMM operands are read in the blocked layout of flce_gemm.hpp (the pack
// kernels below build it from the caller's row-major hidden tensor, the
// logit tiles copy the weight's image out of their own LDS stages, and the
// logit-gradient epilogue writes its output directly in it), except the
// weight as the vocabulary x H operand of the logit tiles, which is read
// row-contiguous from the caller's [H,V] tensor.
//
// The quantities follow the definition in verl pull request #462 ("Equivalent
// compute logic"): per token the logsumexp of the logits, the entropy
// logsumexp - sum(softmax * logits), and the label log-probability (minus the
// cross-entropy). The tanh cap is the Gemma2 one of Liger-Kernel issue #127.
// The per-token state kept while streaming over the vocabulary is
//   m = running max,  s = sum exp(z' - m),  u = sum exp(z' - m) (z' - m),
// so that lse = m + ln s and entropy = ln s - u / s (no cancellation between
// two large numbers).
#pragma once

#include "flce_gemm.hpp"
#include <type_traits>

namespace flce {

// ---- block reductions (deterministic fixed trees) ---------------------------

template <class T, int NT>
__device__ __forceinline__ T block_sum(T v, T* sh) {
  const int t = threadIdx.x;
  sh[t] = v;
  __syncthreads();
#pragma unroll
  for (int w = NT / 2; w > 0; w >>= 1) {
    if (t < w) sh[t] = sh[t] + sh[t + w];
    __syncthreads();
  }
  const T r = sh[0];
  __syncthreads();
  return r;
}

// ---- forward: labels -> int32, counts ---------------------------------------

// Order-preserving compaction step inside one block of 1024 threads (16
// waves): every thread passes its flag for the current chunk of 1024 items;
// returns the rank of the thread's item among the flagged items of the chunk
// (meaningful when flagged) and sets `total` to the chunk's flagged count.
// Wave ballots and a fixed-order sum of the 16 wave counts: deterministic.
__device__ __forceinline__ int chunk_rank(bool flag, int* sh, int& total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint64_t b = __builtin_amdgcn_ballot_w64(flag);
  const int pre = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32),
                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
  if (lane == 0) sh[w] = __popcll(b);
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int c = sh[k];
    off += k < w ? c : 0;
    tot += c;
  }
  __syncthreads();  // sh is reused by the next chunk
  total = tot;
  return off + pre;
}

// Label code of one token: -1 when ignored or outside [0, V_total) (an
// invalid label), y - v_begin when inside the slice [v_begin, v_begin + Vs),
// kLabelElsewhere when valid but outside the slice.
constexpr int32_t kLabelElsewhere = -2;
__device__ __forceinline__ int32_t label_code(int64_t y, int64_t ignore_index, int64_t V_total,
                                              int64_t v_begin, int64_t Vs, bool& invalid) {
  invalid = false;
  if (y == ignore_index) return -1;
  if (y < 0 || y >= V_total) {
    invalid = true;
    return -1;
  }
  return (y >= v_begin && y < v_begin + Vs) ? (int32_t)(y - v_begin) : kLabelElsewhere;
}

struct FwdPrepArgs {
  const int64_t* labels;
  int64_t N, V_total, v_begin, Vs, ignore_index;  // the slice of this call (whole vocabulary unsharded)
  int32_t* idx;            // [N] compacted: original index of the r-th valid token
  int32_t* labc;           // [N] compacted label codes; -1 past the valid tokens
  float* zlab;             // [N] compacted label logits, zeroed here
  float *lse, *logprob, *entropy, *uniform_ce, *z_loss;  // zeroed at ignored tokens (may be null)
  float4* state_out;       // slice mode: the empty state at ignored tokens
  float* label_logit;      // slice mode: zeroed for every token
  int32_t* header;         // [0] invalid labels, [1] valid tokens n
  const float* cw;         // optional class weights [V_total]: their sum over valid
                           // tokens goes to header_wsum(header)
};

// The float64 sum of the class weights of the valid tokens, kept in the
// header after the two counts (bytes 16..23).
__host__ __device__ __forceinline__ double* header_wsum(int32_t* h) {
  return reinterpret_cast<double*>(h + 4);
}
__host__ __device__ __forceinline__ const double* header_wsum(const int32_t* h) {
  return reinterpret_cast<const double*>(h + 4);
}

// One block of 1024 threads: compacts the valid tokens (in token order) and
// writes the per-token outputs of ignored tokens, which no later kernel
// touches.
__global__ void __launch_bounds__(1024) fwd_prep_kernel(FwdPrepArgs a) {
  __shared__ int sh[1024];
  __shared__ double shd[1024];
  int inv = 0, base = 0;
  double ws = 0.0;
  for (int64_t c0 = 0; c0 < a.N; c0 += 1024) {
    const int64_t t = c0 + threadIdx.x;
    bool bad = false;
    const int32_t code = t < a.N ? label_code(a.labels[t], a.ignore_index, a.V_total, a.v_begin,
                                              a.Vs, bad)
                                 : -1;
    inv += bad ? 1 : 0;
    const bool valid = code != -1;
    int total;
    const int r = base + chunk_rank(valid, sh, total);
    if (valid) {
      a.idx[r] = (int32_t)t;
      a.labc[r] = code;
      if (a.cw != nullptr) ws += (double)a.cw[a.labels[t]];
    } else if (t < a.N) {
      if (a.lse) a.lse[t] = 0.f;
      if (a.logprob) a.logprob[t] = 0.f;
      if (a.entropy) a.entropy[t] = 0.f;
      if (a.uniform_ce) a.uniform_ce[t] = 0.f;
      if (a.z_loss) a.z_loss[t] = 0.f;
      if (a.state_out) a.state_out[t] = make_float4(kNegBig, 0.f, 0.f, 0.f);
    }
    if (t < a.N) {
      a.zlab[t] = 0.f;
      if (a.label_logit) a.label_logit[t] = 0.f;
    }
    base += total;
  }
  for (int64_t r = base + threadIdx.x; r < a.N; r += 1024) a.labc[r] = -1;
  inv = block_sum<int, 1024>(inv, sh);
  if (a.cw != nullptr) ws = block_sum<double, 1024>(ws, shd);
  if (threadIdx.x == 0) {
    a.header[0] = inv;
    a.header[1] = base;
    if (a.cw != nullptr) *header_wsum(a.header) = ws;
  }
}

// ---- blocked operand images ----------------------------------------------------

// Operand (R rows, K values per row) whose source is K-contiguous:
// element (r, k) at src[r * ld + k]. Writes the blocked image `dst` of
// ceil(R/256) strips x nkb K blocks; rows >= R and K values >= K are zero.
// With `gather`, operand row r is source row gather[r] for r < *count and
// zero beyond (the compacted valid tokens). A workgroup fills 8 consecutive K
// blocks of one strip; consecutive threads read consecutive 16-byte pieces of
// one source row (512 bytes per row). K must be a multiple of 8 and ld a
// multiple of 8.
__global__ void __launch_bounds__(256) pack_rows_kernel(const uint16_t* __restrict__ src,
                                                        int64_t R, int64_t K, int64_t ld, int nkb,
                                                        const int32_t* __restrict__ gather,
                                                        const int32_t* __restrict__ count,
                                                        uint16_t* __restrict__ dst) {
  const int64_t strip = blockIdx.y;
  const int kb0 = blockIdx.x * 8;
  const int t = threadIdx.x;
  const int64_t rows = gather != nullptr ? *count : R;
#pragma unroll 4
  for (int p = 0; p < 32; ++p) {
    const int i = p * 256 + t;
    const int r = i >> 5, kbl = (i >> 2) & 7, c = i & 3;
    const int kb = kb0 + kbl;
    if (kb >= nkb) continue;
    const int64_t row = strip * kTile + r;
    const int64_t k = (int64_t)kb * kBK + c * 8;
    u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
    if (row < rows && k < K) {
      const int64_t srow = gather != nullptr ? gather[row] : row;
      v = *reinterpret_cast<const u32x4_t*>(src + srow * ld + k);
    }
    char* blk = reinterpret_cast<char*>(dst) + (strip * nkb + kb) * (int64_t)kBlockBytes;
    *reinterpret_cast<u32x4_t*>(blk + blk_byte(r, c * 8)) = v;
  }
}

// Operand (R rows, K values per row) whose source is row-contiguous:
// element (r, k) at src[k * ld + r] (a transposing pack). Writes the blocked
// image `dst` of ceil(R/256) strips x nkb K blocks, zero past R and K. With
// `gather`, K index k reads source row gather[k] for k < *count and zero
// beyond (the compacted valid tokens). A workgroup fills K blocks
// (2 bx, 2 bx + 1) of one strip: thread (g, q) reads rows r = 8g .. 8g+7 of
// the 8 source rows k = 8q .. 8q+7 (16 bytes each; 32 consecutive threads
// read 512 contiguous bytes), transposes the 8 x 8 piece in registers and
// writes eight 16-byte chunks. R must be a multiple of 8 and ld a multiple of
// 8.
__global__ void __launch_bounds__(256) pack_cols_kernel(const uint16_t* __restrict__ src,
                                                        int64_t R, int64_t K, int64_t ld, int nkb,
                                                        const int32_t* __restrict__ gather,
                                                        const int32_t* __restrict__ count,
                                                        uint16_t* __restrict__ dst) {
  const int64_t strip = blockIdx.y;
  const int64_t kval = gather != nullptr ? *count : K;
  const int t = threadIdx.x;
  const int g = t & 31, q = t >> 5;                 // row group, K chunk (0..7)
  const int kb = blockIdx.x * 2 + (q >> 2);
  if (kb >= nkb) return;
  const int c = q & 3;                              // chunk within the block
  const int64_t r0 = strip * kTile + 8 * g;
  const int64_t k0 = (int64_t)kb * kBK + c * 8;
  u32x4_t in[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    in[e] = u32x4_t{0u, 0u, 0u, 0u};
    if (r0 < R && k0 + e < kval) {
      const int64_t srow = gather != nullptr ? gather[k0 + e] : k0 + e;
      in[e] = *reinterpret_cast<const u32x4_t*>(src + srow * ld + r0);
    }
  }
  char* blk = reinterpret_cast<char*>(dst) + (strip * nkb + kb) * (int64_t)kBlockBytes;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    // Output row 8g + j holds K values k0 .. k0+7: element j of each in[e].
    u32x4_t o;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t x = in[2 * w][j >> 1], y = in[2 * w + 1][j >> 1];
      o[w] = (j & 1) ? ((x >> 16) | (y & 0xFFFF0000u)) : ((x & 0xFFFFu) | (y << 16));
    }
    *reinterpret_cast<u32x4_t*>(blk + blk_byte(8 * g + j, c * 8)) = o;
  }
}

// ---- forward: fused logit tiles + online row statistics ---------------------

struct FwdTileArgs {
  const uint16_t* weight;  // [H,V], rows ldw apart
  int64_t ldw;             // row stride of weight (V, or V rounded up to 8 for a padded copy
                           // whose extra columns are zero)
  const uint16_t* xb;      // blocked hidden: strips of 256 tokens, K = H
  const int32_t* lab;      // [N] compacted label codes (label logit captured when >= 0)
  const int32_t* nvalid;   // device: number n of compacted tokens
  int64_t N, H, V;
  int hkb;                 // K blocks per strip, ceil(H / 32)
  int VT, TB;              // vocabulary tiles, token blocks of this launch
  int tb0;                 // first token block of this launch
  int group;               // token blocks per XCD patch (see group_map)
  float cap, cap_k;        // softcap c and 2*log2(e)/c
  float4* part;            // [VT][N] {m, s, u, sum z'} per vocabulary tile (compacted tokens)
  float* zlab;             // [N] capped logit of the label (compacted tokens)
  // STORE only: z' - mref as bf16 in a blocked image of the launch's tokens
  // (strips of 256 tokens, K = vocabulary, kbv blocks per strip), and mref,
  // the maximum of z' over each wave's 128 vocabulary rows, at
  // mref[(2 vt + half) * mld + local token].
  uint16_t* dz;
  int kbv;
  float* mref;
  int64_t mld;
  // STORE only, or null: the blocked weight as the dH operand (strips of 256
  // hidden rows, K = vocabulary, kbv blocks each), written by this launch.
  uint16_t* wimg;
};

// Copies a tile's eight 16 KiB blocks from the stage arrays (block b in sa[b]
// for b < 4, sb[b - 4] otherwise) to 128 KiB of contiguous memory: each wave
// instruction stores 1 KiB. Iteration it covers half of block it / 2. The
// caller synchronises the block before.
__device__ __forceinline__ void copy_out_tile(char* const (&sa)[kStages],
                                              char* const (&sb)[kStages],
                                              __amdgpu_buffer_rsrc_t dst) {
#pragma unroll
  for (int it = 0; it < 16; ++it) {
    const int b = it >> 1;
    const int off = ((it & 1) * kThreads + (int)threadIdx.x) * 16;
    const char* src = (b < 4 ? sa[b & 3] : sb[b & 3]) + off;
    __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const u32x4_t*>(src), dst,
                                           (uint32_t)(b * kBlockBytes + off), 0, 0);
  }
}

// Merge state (m2, s2, u2) into (m, s, u); u in base-2 units (times log2 e).
__device__ __forceinline__ void merge_state2(float& m, float& s, float& u, float m2, float s2,
                                             float u2) {
  const float mn = fmaxf(m, m2);
  const float d1 = (m - mn) * kLog2e, d2 = (m2 - mn) * kLog2e;
  const float a1 = fast_exp2(d1), a2 = fast_exp2(d2);
  u = a1 * fmaf(d1, s, u) + a2 * fmaf(d2, s2, u2);
  s = a1 * s + a2 * s2;
  m = mn;
}

// Online-softmax state of one token column j of a wave's 128 x 32 block
// (64 accumulators per lane): m = max z', s = sum exp(z' - m),
// u = sum exp(z' - m)(z' - m) in base-2 units, and zs = sum z' (for the
// uniform cross-entropy). The capped logits are left in z[] for the label
// capture. MASK drops rows at offset >= lim (the last vocabulary tile only).
template <bool CAP, bool MASK>
__device__ __forceinline__ void column_stats(const Acc& acc, int j, float cap, float cap_k, int lim,
                                             float (&z)[64], float& m, float& s, float& u,
                                             float& zs) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float x = acc[i][j][r];
      if constexpr (CAP) x = softcap_apply(x, cap, cap_k);
      if constexpr (MASK) x = (i * 32 + 8 * (r >> 2) + (r & 3)) < lim ? x : kNegBig;
      z[i * 16 + r] = x;
    }
  float mx[4], sz[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float x = z[i * 16];
    float t = MASK ? (z[i * 16] == kNegBig ? 0.f : z[i * 16]) : z[i * 16];
#pragma unroll
    for (int r = 1; r < 16; ++r) {
      x = fmaxf(x, z[i * 16 + r]);
      if constexpr (MASK)
        t += z[i * 16 + r] == kNegBig ? 0.f : z[i * 16 + r];
      else
        t += z[i * 16 + r];
    }
    mx[i] = x;
    sz[i] = t;
  }
  const float mb = fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3]));
  zs = (sz[0] + sz[1]) + (sz[2] + sz[3]);
  const float nm = -mb * kLog2e;
  float sp[4], up[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sp[i] = 0.f;
    up[i] = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      // A masked entry sits at kNegBig: if some entry of the lane is valid,
      // mb is finite, d is hugely negative and e = 0; if none is, mb is
      // kNegBig itself and the select drops the entry.
      const float d = fmaf(z[i * 16 + r], kLog2e, nm);
      float e = fast_exp2(d);
      if constexpr (MASK) e = z[i * 16 + r] == kNegBig ? 0.f : e;
      sp[i] += e;
      up[i] = fmaf(e, d, up[i]);
    }
  }
  m = mb;
  s = (sp[0] + sp[1]) + (sp[2] + sp[3]);
  u = (up[0] + up[1]) + (up[2] + up[3]);
}

// The dH contraction reads the weight as its B operand in the blocked layout
// (strips of 256 hidden rows, K = vocabulary). A logit-tile block streams the
// same bytes through its A stages: the stage of K block k holds hidden rows
// 32k .. 32k+31 of the tile's 256 vocabulary columns, i.e. rows
// 32 (k % 8) .. +31 of strip k / 8 in the tile's 8 vocabulary blocks
// kb0 .. kb0+7. One block per vocabulary tile (image_writer) copies every
// stage into that image, so the image costs no pass over the weight of its
// own. Rows past H in the last strip are left as they are: they only reach dH
// columns past H, which are never stored.
struct WeightImageHook {
  uint16_t* img;  // block 0 of strip 0
  int kbv;        // K blocks per strip
  int kb0;        // the tile's first vocabulary block
  __device__ __forceinline__ void operator()(const char* st, int k) const {
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(img + (int64_t)(k >> 3) * kbv * kBlockElems, (int64_t)kbv * kBlockBytes);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int p = (int)threadIdx.x + kThreads * i;  // 16-byte piece of the stage
      const int kr = p >> 5, j = (p >> 2) & 7, c = p & 3;
      // RowA stage layout: K row kr takes 512 bytes; its 16-byte slot s holds
      // columns 32 ((s >> 2) ^ (kr & 3)) + 8 (s & 3) .. +7.
      const u32x4_t v =
          *reinterpret_cast<const u32x4_t*>(st + kr * 512 + ((((j ^ (kr & 3)) << 2) + c) << 4));
      const int r = 32 * (k & 7) + kr;
      buf_store_u32x4(v, rs, (uint32_t)((kb0 + j) * kBlockBytes + r * 64 + ((c ^ ((r >> 2) & 3)) << 4)));
    }
  }
};

// Whether tile (tb, vt) writes the weight image: the tile of token block
// vt % tbv, so that the writers spread over token blocks and thus over XCDs.
__device__ __forceinline__ bool image_writer(int tb, int vt, int tbv) {
  return tb == vt % tbv;
}

// Block (tb, vt): tokens [256 tb, +256) against vocabulary [256 vt, +256).
// The MFMA tile is z^T: rows = vocabulary (A = the [H,V] weight read
// row-contiguous), cols = tokens (B = hidden strip), so each lane's 64
// accumulators of one 32-column block
// belong to one token and the row statistics need no cross-lane work until the
// end. The block reduces its tile to (m, s, u) per token and stores it as the
// tile's partial state. STORE also keeps the capped logits for the fused
// path, as z' - mref in bf16 (mref: the maximum over the wave's 128
// vocabulary rows), so that the logit gradient can be formed later without
// recomputing the tile.
template <bool CAP, bool STORE>
__device__ __forceinline__ void fwd_tile_body(const FwdTileArgs& a) {
  FLCE_DECLARE_STAGES(sa, sb);
  // Only the token tiles of this launch that hold compacted tokens take part;
  // the tile numbering runs over them alone, so every XCD gets its share.
  const int left = (*a.nvalid + kTile - 1) / kTile - a.tb0;
  const int tbv = left < a.TB ? (left > 0 ? left : 0) : a.TB;
  if ((int)blockIdx.x >= tbv * a.VT) return;
  int tbl, vt;
  group_map(xcd_remap(blockIdx.x, tbv * a.VT), tbv, a.VT, a.group, tbl, vt);
  const int tb = a.tb0 + tbl;
  const int lane = threadIdx.x & 63, lh = lane >> 5;
  const int wave = wave_id(), wm = wave & 1, wn = wave >> 1;
  const int64_t n0 = (int64_t)tb * kTile;

  Acc acc;
  {
    MainloopRowA ml;
    RowA A;
    A.init(a.weight, a.ldw, a.ldw, (int64_t)vt * kTile, 0, a.H);
    const Strip B{a.xb + (int64_t)tb * a.hkb * kBlockElems, a.hkb};
    bool wrote = false;
    if constexpr (STORE) {
      // As in bwd_dlogits_kernel: one tile per vocabulary tile writes the
      // weight image for dH.
      if (a.wimg != nullptr && image_writer(tbl, vt, tbv)) {
        ml.run(sa, sb, A, B, 0, a.hkb, acc, WeightImageHook{a.wimg, a.kbv, 8 * vt});
        wrote = true;
      }
    }
    if (!wrote) ml.run(sa, sb, A, B, 0, a.hkb, acc);
  }

  const int vb = vt * kTile + wm * 128;  // first vocabulary row of this wave
  const bool full = (int64_t)vb + 128 <= a.V;
  // Rows at offset o (0..127, without the lane-half term) are valid iff o < lim.
  const int lim = (int)(a.V - vb) - 4 * lh;
  // STORE: the tile's eight dz blocks are assembled in the stage arrays,
  // block 4 wm + i (vocabulary rows [32 (4 wm + i), +32)) in lds[i].
  char* lds[4];
  if constexpr (STORE) {
#pragma unroll
    for (int i = 0; i < 4; ++i) lds[i] = wm ? sb[i] : sa[i];
  }
  float m[2], s[2], u[2], zs[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    float z[64];
    if (full) {
      column_stats<CAP, false>(acc, j, a.cap, a.cap_k, lim, z, m[j], s[j], u[j], zs[j]);
    } else {
      // lim passes through an empty asm here so that the row tests, needed
      // by the last vocabulary tile only, are not hoisted into every tile.
      int l = lim;
      opaque(l);
      column_stats<CAP, true>(acc, j, a.cap, a.cap_k, l, z, m[j], s[j], u[j], zs[j]);
    }

    if constexpr (STORE) {
      // Rows m0 .. m0+3 (vocabulary) of token column n: one 8-byte piece.
      // Masked rows hold kNegBig - mw (or 0 when the wave has no valid row);
      // the gradient pass zeroes them.
      const float mw = fmaxf(m[j], __shfl_xor(m[j], 32));
      const int n = acc_col(wn, j, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int q = i * 16 + rq * 4;
          const int m0 = acc_row(wm, i, rq * 4, lane);
          *reinterpret_cast<u32x2_t*>(lds[i] + blk_byte(n, m0 & 31)) =
              u32x2_t{pack_bf16x2(z[q] - mw, z[q + 1] - mw), pack_bf16x2(z[q + 2] - mw, z[q + 3] - mw)};
        }
      if (lh == 0) a.mref[(int64_t)(2 * vt + wm) * a.mld + tbl * kTile + n] = mw;
    }

    // The label's logit: exactly one lane of one block in the grid owns it,
    // and most waves own none (skipped by a wave-uniform test).
    const int64_t t = n0 + acc_col(wn, j, lane);
    const int y = t < a.N ? a.lab[t] : -1;
    const int off = y - vb;
    const bool hit = (unsigned)off < 128u && (((off & 31) >> 2) & 1) == lh;
    if (__builtin_amdgcn_ballot_w64(hit) != 0 && hit) {
      const int sel = (off >> 5) * 16 + ((((off & 31) >> 3) << 2) | (off & 3));
      float zl = 0.f;
#pragma unroll
      for (int q = 0; q < 64; ++q) zl = q == sel ? z[q] : zl;
      a.zlab[t] = zl;
    }
    __builtin_amdgcn_sched_barrier(0);  // one token column at a time
  }

  // Merge the two lane halves (same tokens, other vocabulary rows), then the
  // two waves that share a token range, and store the tile's partial state.
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const float m2 = __shfl_xor(m[j], 32), s2 = __shfl_xor(s[j], 32), u2 = __shfl_xor(u[j], 32);
    merge_state2(m[j], s[j], u[j], m2, s2, u2);
    zs[j] += __shfl_xor(zs[j], 32);
  }
  // (The stage arrays hold the dz blocks under STORE.)
  __shared__ float4 red_store[STORE ? kTile : 1];
  float4* red = STORE ? red_store : reinterpret_cast<float4*>(sa[0]);
  if (wm == 1 && lane < 32) {
#pragma unroll
    for (int j = 0; j < 2; ++j) red[acc_col(wn, j, lane)] = make_float4(m[j], s[j], u[j], zs[j]);
  }
  __syncthreads();
  if (wm == 0 && lane < 32) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = acc_col(wn, j, lane);
      const float4 q = red[c];
      merge_state2(m[j], s[j], u[j], q.x, q.y, q.z);
      const int64_t t = n0 + c;
      if (t < a.N) a.part[(int64_t)vt * a.N + t] = make_float4(m[j], s[j], u[j] * kLn2, zs[j] + q.w);
    }
  }
  if constexpr (STORE)
    copy_out_tile(sa, sb, make_rsrc(a.dz + ((int64_t)tbl * a.kbv + 8 * vt) * kBlockElems,
                                    8 * (int64_t)kBlockBytes));
}

template <bool CAP>
__global__ void __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                               amdgpu_waves_per_eu(2, 2)))
fwd_tile_kernel(FwdTileArgs a) {
  fwd_tile_body<CAP, false>(a);
}

// The fused path's logit tiles: fwd_tile_kernel plus the kept logits.
template <bool CAP>
__global__ void __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                               amdgpu_waves_per_eu(2, 2)))
fused_tile_kernel(FwdTileArgs a) {
  fwd_tile_body<CAP, true>(a);
}

// ---- forward: merge the vocabulary splits -------------------------------------

// Merge state (m2, s2, u2) into (m, s, u), natural-log units. An empty state
// is (kNegBig, 0, 0).
__device__ __forceinline__ void merge_state(float& m, float& s, float& u, float m2, float s2,
                                            float u2) {
  const float mn = fmaxf(m, m2);
  const float a1 = expf(m - mn), a2 = expf(m2 - mn);
  u = a1 * fmaf(m - mn, s, u) + a2 * fmaf(m2 - mn, s2, u2);
  s = a1 * s + a2 * s2;
  m = mn;
}

// 1 / (the mean's divisor): the valid count n, or the class-weight sum with
// class weights; 0 when that divisor is 0 (every mean and gradient then 0).
__device__ __forceinline__ float mean_divisor_inv(const int32_t* header, bool weighted) {
  const double d = weighted ? *header_wsum(header) : (double)header[1];
  return d != 0.0 ? (float)(1.0 / d) : 0.f;
}

// DzToken (the per-token constants of the logit gradient) and kCombineTokens:
// flce_layout.hpp.
constexpr int kCombineWaves = 16;    // vocabulary-tile groups per combine block

// Block of 1024 threads for 64 tokens: wave w merges the partial states of
// vocabulary tiles w, w + 16, ... of token t0 + lane (consecutive lanes read
// consecutive 16-byte states), then wave 0 merges the 16 states in wave order
// and writes lse, logprob, entropy and, when requested, the uniform
// cross-entropy lse - (1/V) sum z' and the z-loss lam * lse^2. With
// bsum != nullptr it also writes the block's float64 sums of the four outputs
// over valid tokens. Fixed merge and summation orders: the result does not
// depend on timing.
struct CombineArgs {
  const float4* part;      // [S][N] partial states
  int S;                   // vocabulary tiles (or slices)
  const float* zlab;       // [nz][N] label logits, summed (one of them holds each label)
  int nz;
  // Compacted (idx set): entry r < *nvalid belongs to token idx[r]. Direct
  // (idx null): entry t is token t, valid when labels[t] is.
  const int32_t* idx;
  const int32_t* nvalid;
  const int64_t* labels;   // direct mode
  int64_t ignore_index;
  int64_t N, V;            // V: the whole vocabulary
  float zl_scale;          // lam
  float *lse, *logprob, *entropy;
  float *uniform_ce, *z_loss;  // optional
  double4* bsum;               // optional: {logprob, entropy, uniform_ce, z_loss} per block
  float4* state_out;           // if set: write the merged state {m, s, u, sum z'} instead
  float* label_logit;          // with state_out: the label logit per token
  int64_t r0;                  // first entry of this launch (a multiple of 64)
  // If coef is set (fused path, compacted mode): also the logit-gradient
  // constants of each entry (see DzToken), from the upstream gradients
  // glp, gent, guce, gzl ([N] under reduction none, [1] otherwise, null =
  // zero); under mean the scalars are divided by the valid count header[1].
  DzToken* coef;
  const float *glp, *gent, *guce, *gzl;
  int reduction;
  int ent_tok;             // 1: gent is per token [N] under mean / sum too
  const int32_t* header;
  // Optional class weights [V]: token t's block sums and (fused path) its
  // scalar gradients carry cw[labels[t]]; the mean divides by the weight sum
  // header_wsum(header). labels must then be set in compacted mode too.
  const float* cw;
};

// Class weight of valid token t (1 without class weights).
__device__ __forceinline__ float token_weight(const float* cw, const int64_t* labels, int64_t t) {
  return cw == nullptr ? 1.f : cw[labels[t]];
}

// Gradient constants of valid token t with lse l and entropy e (fused path;
// the same arithmetic as bwd_prep_kernel, every label inside the vocabulary).
__device__ __forceinline__ DzToken token_coef(const CombineArgs& a, int64_t t, float l, float e) {
  const bool scalar = a.reduction != 0;
  const float div = a.reduction == 1 ? mean_divisor_inv(a.header, a.cw != nullptr) : 1.f;
  const float om = scalar ? token_weight(a.cw, a.labels, t) * div : 1.f;
  auto grad = [&](const float* g, bool sc) {
    return g == nullptr ? 0.f : (sc ? g[0] * om : g[t]);
  };
  const float g = grad(a.glp, scalar), ge = grad(a.gent, scalar && a.ent_tok == 0),
              gu = grad(a.guce, scalar), gz = grad(a.gzl, scalar);
  const float S = l - e;
  DzToken c;
  c.lse = l;
  c.ebar = ge;
  c.cs = g - ge * S - gu - 2.f * a.zl_scale * gz * l;
  c.gbar = g;
  c.k0 = -gu * (1.f / (float)a.V);
  c.pad0 = c.pad1 = c.pad2 = 0.f;
  return c;
}

__global__ void __launch_bounds__(1024) fwd_combine_kernel(CombineArgs a) {
  __shared__ float4 st[kCombineWaves][kCombineTokens];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t r = a.r0 + (int64_t)blockIdx.x * kCombineTokens + lane;  // entry
  bool valid;
  int64_t t;  // token
  if (a.idx != nullptr) {
    valid = r < *a.nvalid;
    t = valid ? a.idx[r] : -1;
  } else {
    bool bad;
    valid = r < a.N && label_code(a.labels[r], a.ignore_index, a.V, 0, a.V, bad) != -1;
    t = r;
  }
  float m = kNegBig, s = 0.f, u = 0.f, zs = 0.f;
  if (valid)
    for (int k = w; k < a.S; k += kCombineWaves) {
      const float4 q = a.part[(int64_t)k * a.N + r];
      merge_state(m, s, u, q.x, q.y, q.z);
      zs += q.w;
    }
  st[w][lane] = make_float4(m, s, u, zs);
  __syncthreads();
  if (w != 0) return;
#pragma unroll 1
  for (int k = 1; k < kCombineWaves; ++k) {
    const float4 q = st[k][lane];
    merge_state(m, s, u, q.x, q.y, q.z);
    zs += q.w;
  }
  if (a.state_out != nullptr) {
    // Ignored tokens got the empty state from the prep kernel.
    if (valid) {
      a.state_out[t] = make_float4(m, s, u, zs);
      a.label_logit[t] = a.zlab[r];
    }
    return;
  }
  double r0 = 0.0, r1 = 0.0, r2 = 0.0, r3 = 0.0;
  if (valid) {
    const float ls = logf(s);
    const float l = m + ls;
    const float e = ls - u / s;
    float zy = 0.f;
    for (int k = 0; k < a.nz; ++k) zy += a.zlab[(int64_t)k * a.N + r];
    const float lp = zy - l;
    const float uc = l - zs / (float)a.V;
    const float zl = a.zl_scale * l * l;
    a.lse[t] = l;
    a.entropy[t] = e;
    a.logprob[t] = lp;
    if (a.uniform_ce) a.uniform_ce[t] = uc;
    if (a.z_loss) a.z_loss[t] = zl;
    const double om = a.bsum != nullptr ? (double)token_weight(a.cw, a.labels, t) : 1.0;
    r0 = om * lp;
    r1 = om * e;
    r2 = om * uc;
    r3 = om * zl;
    if (a.coef != nullptr) a.coef[r] = token_coef(a, t, l, e);
  } else if (a.coef != nullptr) {
    a.coef[r] = DzToken{1e30f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  } else if (a.idx == nullptr && r < a.N) {
    a.lse[r] = 0.f;
    a.entropy[r] = 0.f;
    a.logprob[r] = 0.f;
    if (a.uniform_ce) a.uniform_ce[r] = 0.f;
    if (a.z_loss) a.z_loss[r] = 0.f;
  }
  if (a.bsum != nullptr) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      r0 += __shfl_xor(r0, o);
      r1 += __shfl_xor(r1, o);
      r2 += __shfl_xor(r2, o);
      r3 += __shfl_xor(r3, o);
    }
    if (lane == 0) a.bsum[a.r0 / kCombineTokens + blockIdx.x] = make_double4(r0, r1, r2, r3);
  }
}

// One block: sums the per-block partial sums in a fixed order; under "mean"
// divides by the number of valid tokens, or with class weights by their sum
// (0 when that divisor is 0). Writes each of the four reduced outputs whose
// pointer is not null.
__global__ void __launch_bounds__(256) fwd_reduce_kernel(const double4* __restrict__ bsum, int nb,
                                                         const int32_t* __restrict__ header,
                                                         int mean, int weighted, float* out_lp,
                                                         float* out_ent, float* out_uce,
                                                         float* out_zl) {
  __shared__ double sh[256];
  double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
  for (int i = threadIdx.x; i < nb; i += 256) {
    const double4 b = bsum[i];
    a0 += b.x;
    a1 += b.y;
    a2 += b.z;
    a3 += b.w;
  }
  a0 = block_sum<double, 256>(a0, sh);
  a1 = block_sum<double, 256>(a1, sh);
  a2 = block_sum<double, 256>(a2, sh);
  a3 = block_sum<double, 256>(a3, sh);
  if (threadIdx.x == 0) {
    const double d = mean ? (weighted ? *header_wsum(header) : (double)header[1]) : 1.0;
    const double f = d != 0.0 ? 1.0 / d : 0.0;
    if (out_lp) out_lp[0] = (float)(a0 * f);
    if (out_ent) out_ent[0] = (float)(a1 * f);
    if (out_uce) out_uce[0] = (float)(a2 * f);
    if (out_zl) out_zl[0] = (float)(a3 * f);
  }
}

// ---- backward: per-token coefficients ------------------------------------------


struct PrepArgs {
  const int64_t* labels;
  int64_t N, V, ignore_index;  // V: the whole vocabulary
  int64_t v_begin, Vs;         // vocabulary slice of this call
  int32_t* idx;                // [N] compacted: original index of the r-th valid token
  int reduction;               // 0 none, 1 mean, 2 sum
  float zl_scale;              // lam
  const float *lse, *entropy;
  const float *glp, *gent, *guce, *gzl;  // [N] (none), [1] (mean, sum) or null
  DzToken* coef;
  int32_t* lab32;
  int32_t* header;
  const float* cw;             // optional class weights [V] (mean, sum)
  int ent_tok;                 // 1: gent is per token [N] under mean / sum too
};

// One block of 1024: compacts the valid tokens (in token order) and writes
// their coefficients and label offsets in compacted order; entries past the
// valid tokens get the ignored-token values. Label offsets are relative to
// the slice; -1 when the label lies outside it, which drops the label term
// but keeps the token's other terms.
__global__ void __launch_bounds__(1024) bwd_prep_kernel(PrepArgs a) {
  __shared__ int sh[1024];
  __shared__ double shd[1024];
  int inv = 0, nv = 0;
  double ws = 0.0;
  for (int64_t t = threadIdx.x; t < a.N; t += 1024) {
    bool bad;
    if (label_code(a.labels[t], a.ignore_index, a.V, a.v_begin, a.Vs, bad) != -1) {
      ++nv;
      if (a.cw != nullptr) ws += (double)a.cw[a.labels[t]];
    }
    inv += bad ? 1 : 0;
  }
  inv = block_sum<int, 1024>(inv, sh);
  nv = block_sum<int, 1024>(nv, sh);
  if (a.cw != nullptr) ws = block_sum<double, 1024>(ws, shd);
  // Scalar gradients of a mean are spread over the n valid tokens (with class
  // weights: token t takes the share cw[y_t] / sum of the weights); those of
  // a sum apply as they are (times cw[y_t]).
  const bool scalar = a.reduction != 0;
  const bool escalar = scalar && a.ent_tok == 0;  // the entropy gradient is a scalar too
  const double dv = a.cw != nullptr ? ws : (double)nv;
  const float div = a.reduction == 1 ? (dv != 0.0 ? (float)(1.0 / dv) : 0.f) : 1.f;
  auto scal = [&](const float* g) { return (scalar && g != nullptr) ? g[0] * div : 0.f; };
  const float g0 = scal(a.glp), u0 = scal(a.guce), z0 = scal(a.gzl);
  const float e0 = (escalar && a.gent != nullptr) ? a.gent[0] * div : 0.f;
  const float invV = 1.f / (float)a.V;
  int base = 0;
  for (int64_t c0 = 0; c0 < a.N; c0 += 1024) {
    const int64_t t = c0 + threadIdx.x;
    bool bad;
    const int32_t code =
        t < a.N ? label_code(a.labels[t], a.ignore_index, a.V, a.v_begin, a.Vs, bad) : -1;
    const bool valid = code != -1;
    int total;
    const int r = base + chunk_rank(valid, sh, total);
    if (valid) {
      const float om = (scalar && a.cw != nullptr) ? a.cw[a.labels[t]] : 1.f;
      auto per = [&](const float* g, float s0, bool sc) {
        return sc ? s0 * om : (g != nullptr ? g[t] : 0.f);
      };
      const float g = per(a.glp, g0, scalar), e = per(a.gent, e0, escalar),
                  u = per(a.guce, u0, scalar), z = per(a.gzl, z0, scalar);
      const float l = a.lse[t];
      const float S = l - a.entropy[t];
      DzToken c;
      c.lse = l;
      c.ebar = e;
      c.cs = g - e * S - u - 2.f * a.zl_scale * z * l;
      c.gbar = code >= 0 ? g : 0.f;
      c.k0 = -u * invV;
      c.pad0 = c.pad1 = c.pad2 = 0.f;
      a.coef[r] = c;
      a.lab32[r] = code >= 0 ? code : -1;
      a.idx[r] = (int32_t)t;
    }
    base += total;
  }
  for (int64_t r = base + threadIdx.x; r < a.N; r += 1024) {
    a.coef[r] = DzToken{1e30f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    a.lab32[r] = -1;
  }
  if (threadIdx.x == 0) {
    a.header[0] = inv;
    a.header[1] = nv;
  }
}

// Zeroes the rows of `out` ([N, row_bytes]) whose token is ignored or has an
// invalid label: the compacted contractions never write them. One block per
// token (grid-stride), 16-byte stores; row_bytes is a multiple of 16.
__global__ void __launch_bounds__(256) zero_ignored_rows_kernel(const int64_t* __restrict__ labels,
                                                                int64_t N, int64_t V,
                                                                int64_t ignore_index,
                                                                char* __restrict__ out,
                                                                int64_t row_bytes) {
  for (int64_t t = blockIdx.x; t < N; t += gridDim.x) {
    bool bad;
    if (label_code(labels[t], ignore_index, V, 0, V, bad) != -1) continue;
    char* row = out + t * row_bytes;
    for (int64_t o = (int64_t)threadIdx.x * 16; o < row_bytes; o += 256 * 16)
      *reinterpret_cast<u32x4_t*>(row + o) = u32x4_t{0u, 0u, 0u, 0u};
  }
}

// ---- backward: recompute logits, form the logit gradient ----------------------

struct DlogitsArgs {
  const uint16_t* weight;  // [H,V], rows ldw apart (see FwdTileArgs)
  int64_t ldw;
  const uint16_t* xb;      // blocked hidden
  const DzToken* coef;     // [N] compacted tokens
  const int32_t* lab;      // [N] compacted label offsets in the slice (-1: none)
  const int32_t* nvalid;   // device: number of compacted tokens
  int64_t N, H, V;
  int hkb;                 // K blocks of the hidden strips
  int64_t v0;              // first vocabulary column of this chunk (multiple of 256)
  int VTc, TB;             // vocabulary tiles in the chunk, token blocks
  int group;
  int kbv;                 // K blocks per strip of dtv (chunk capacity / 32)
  int kbn;                 // K blocks per strip of dvt (token blocks * 8)
  float cap, cap_k, inv_cap;
  uint16_t* dtv;           // blocked D, strips of 256 tokens, K = chunk vocabulary
  uint16_t* dvt;           // blocked D^T, strips of 256 chunk vocabulary rows, K = tokens
  uint16_t* wimg;          // blocked weight chunk as the dH operand (strips of 256 hidden
                           // rows, K = chunk vocabulary, kbv blocks each), written here; or null
};

// Per-token constants of the logit gradient.
struct DzCoef {
  float nl;       // -lse * log2(e)
  float ebar;     // upstream entropy gradient
  float cS;       // gbar - ebar S - gu - 2 lam gz lse
  float gbar;     // upstream logprob gradient (the label term)
  float k0;       // -gu / V (the uniform cross-entropy term)
  float cap, cap_k, inv_cap;
  // Capped tile from raw logits (see dz_column): a1 = -2 c log2(e),
  // b1 = c log2(e) + nl, a2 = -8 c ebar, b2 = 4 (c ebar + cS), k4 = 4 k0,
  // gk4 = 4 (gbar + k0).
  float a1, b1, a2, b2, k4, gk4;
};

// The per-token constants of token coefficients c for the cap constants of kc.
__device__ __forceinline__ DzCoef dz_coef(const DzToken& c, const DzCoef& kc) {
  const float nl = -c.lse * kLog2e;
  const float cl = kc.cap * kLog2e;
  return DzCoef{nl,        c.ebar,
                c.cs,      c.gbar,
                c.k0,      kc.cap,
                kc.cap_k,  kc.inv_cap,
                -2.f * cl, cl + nl,
                -8.f * kc.cap * c.ebar, 4.f * fmaf(kc.cap, c.ebar, c.cs),
                4.f * c.k0, 4.f * (c.gbar + c.k0)};
}

// The logit gradient of token column j of a wave's 128 x 32 block, rounded to
// bf16, for both blocked images (see bwd_dlogits_kernel). The accumulators
// hold raw logits (RAW: the cap is applied here) or capped ones. LABEL adds
// gbar at the label's row offset yl; MASK zeroes rows at offset >= lim.
// The token-major piece of rows m0 .. m0+3 goes to out(i, n, m0, piece)
// (block 4 wm + i of the tile's 8 dtv blocks); the vocabulary-major image is
// stored directly.
template <bool CAP, bool RAW, bool MASK, bool LABEL, class Out>
__device__ __forceinline__ void dz_column(const Acc& acc, int j, const DzCoef& k, int yl, int lim,
                                          int n, int wm, int wn, int lane, const Out& out,
                                          __amdgpu_buffer_rsrc_t rvt) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int rq = 0; rq < 4; ++rq) {
      float d[4];
#pragma unroll
      for (int r3 = 0; r3 < 4; ++r3) {
        const int o = i * 32 + 8 * rq + r3;
        float z = acc[i][j][rq * 4 + r3];
        float v;
        if constexpr (CAP && RAW) {
          // In terms of r = 1 / (1 + e^(2z/c)): z' = c (1 - 2r) and
          // 1 - (z'/c)^2 = 4 r (1 - r), so with the per-token constants of
          // DzCoef (the factor 4 folded in) the capped gradient is
          // (K4 - p (b2 + a2 r)) (r - r^2), p = 2^(a1 r + b1).
          const float r = fast_rcp(fast_exp2(z * k.cap_k) + 1.f);
          const float p = fast_exp2(fmaf(k.a1, r, k.b1));
          if constexpr (LABEL)
            v = fmaf(-p, fmaf(k.a2, r, k.b2), o == yl ? k.gk4 : k.k4);
          else
            v = fmaf(-p, fmaf(k.a2, r, k.b2), k.k4);
          v *= fmaf(-r, r, r);
        } else {
          const float p = fast_exp2(fmaf(z, kLog2e, k.nl));
          if constexpr (LABEL)
            v = fmaf(-p, fmaf(k.ebar, z, k.cS), o == yl ? k.gbar + k.k0 : k.k0);
          else
            v = fmaf(-p, fmaf(k.ebar, z, k.cS), k.k0);
          if constexpr (CAP) {
            const float qz = z * k.inv_cap;
            v *= fmaf(-qz, qz, 1.f);
          }
        }
        if constexpr (MASK) v = o < lim ? v : 0.f;
        d[r3] = v;
      }
      // Rows m0 .. m0+3 (vocabulary) of token column n.
      const int m0 = acc_row(wm, i, rq * 4, lane);
      const uint32_t p0 = pack_bf16x2(d[0], d[1]), p1 = pack_bf16x2(d[2], d[3]);
      // dtv: row n (token), K = vocabulary m0 .. m0+3: one 8-byte piece.
      out(i, n, m0, u32x2_t{p0, p1});
      // dvt: after the quad transpose, lane 4q+a holds row m0 + a for the
      // four token columns of its quad: one 8-byte piece at K = n & ~3.
      const u32x2_t tv = quad_transpose_bf16(p0, p1);
      buf_store_u32x2(tv, rvt, (uint32_t)((wn * 2 + j) * kBlockBytes +
                                          blk_byte(m0 + (lane & 3), (lane & 31) & ~3)));
    }
  }
}

// The logit gradient of a tile held in the accumulators (raw logits when RAW,
// capped ones otherwise), for both images: token-major pieces to out(), see
// dz_column, and the vocabulary-major image through rvt. coef and lab are
// indexed by compacted row; rows at or past `rows` get zero gradient. vg0 is
// the tile's first vocabulary column within [0, V); kc carries the cap
// constants.
template <bool CAP, bool RAW, class Out>
__device__ __forceinline__ void dlogits_epilogue(const Acc& acc, const DzToken* coef,
                                                 const int32_t* lab, int64_t rows, int64_t n0,
                                                 int64_t vg0, int64_t V, const DzCoef& kc, int wm,
                                                 int wn, int lane, const Out& out,
                                                 __amdgpu_buffer_rsrc_t rvt) {
  const int lh = lane >> 5;
  // Rows at offset o (i*32 + 8*(r/4) + r%4) of this lane are inside the
  // vocabulary iff o < lim.
  const int lim = (int)(V - vg0) - wm * 128 - 4 * lh;
  const bool full = vg0 + kTile <= V;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = acc_col(wn, j, lane);
    const int64_t t = n0 + n;
    DzToken c{1e30f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int y = -1;
    if (t < rows) {
      c = coef[t];
      y = lab[t];
    }
    // The label's row offset within this lane's rows, or -1.
    const int64_t yo = (int64_t)y - vg0 - wm * 128 - 4 * lh;
    const int yl = (y >= 0 && yo >= 0 && yo < 128) ? (int)yo : -1;
    const DzCoef k = dz_coef(c, kc);
    // Wave-uniform choice of the variant: the label term is needed by few
    // waves, the row mask only in the last vocabulary tile.
    const bool any_label = __builtin_amdgcn_ballot_w64(yl >= 0) != 0;
    if (full) {
      if (any_label)
        dz_column<CAP, RAW, false, true>(acc, j, k, yl, lim, n, wm, wn, lane, out, rvt);
      else
        dz_column<CAP, RAW, false, false>(acc, j, k, yl, lim, n, wm, wn, lane, out, rvt);
    } else {
      // As in fwd_tile_body: the row tests stay in the last vocabulary tile.
      int l = lim;
      opaque(l);
      if (any_label)
        dz_column<CAP, RAW, true, true>(acc, j, k, yl, l, n, wm, wn, lane, out, rvt);
      else
        dz_column<CAP, RAW, true, false>(acc, j, k, yl, l, n, wm, wn, lane, out, rvt);
    }
    __builtin_amdgcn_sched_barrier(0);  // one token column at a time
  }
}

// dz' = gbar ([v == y] - p) - ebar p (z' - S) + gu (p - 1/V) + 2 lam gz lse p
// (the gradient of the four per-token outputs), dz = dz' (1 - (z'/c)^2) if
// capped, rounded to bf16 and written into both blocked images of the chunk:
// dtv (the A operand of dH = D W^T) and dvt (the B operand of dW = hidden^T D).
// Tokens past N have coefficients that make dz = 0, vocabulary rows past V
// are set to 0, so the padded parts of both images hold zeros.
template <bool CAP>
__global__ void __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                               amdgpu_waves_per_eu(2, 2)))
bwd_dlogits_kernel(DlogitsArgs a) {
  FLCE_DECLARE_STAGES(sa, sb);
  // Tiles numbered over the token tiles that hold compacted tokens only.
  const int tbv = (*a.nvalid + kTile - 1) / kTile;
  if ((int)blockIdx.x >= tbv * a.VTc) return;
  int tb, vt;
  group_map(xcd_remap(blockIdx.x, tbv * a.VTc), tbv, a.VTc, a.group, tb, vt);
  const int lane = threadIdx.x & 63;
  const int wave = wave_id(), wm = wave & 1, wn = wave >> 1;
  const int64_t n0 = (int64_t)tb * kTile;
  const int64_t vg0 = a.v0 + (int64_t)vt * kTile;  // first vocabulary column of the tile

  Acc acc;
  {
    MainloopRowA ml;
    RowA A;
    A.init(a.weight, a.ldw, a.ldw, vg0, 0, a.H);
    const Strip B{a.xb + (int64_t)tb * a.hkb * kBlockElems, a.hkb};
    // One tile per vocabulary tile also writes its weight columns into the
    // dH operand image.
    if (a.wimg != nullptr && image_writer(tb, vt, tbv))
      ml.run(sa, sb, A, B, 0, a.hkb, acc, WeightImageHook{a.wimg, a.kbv, 8 * vt});
    else
      ml.run(sa, sb, A, B, 0, a.hkb, acc);
  }

  // Each tile owns 8 consecutive K blocks in each image: dtv strip tb, blocks
  // [8 vt, +8) (K = vocabulary); dvt strip vt, blocks [8 tb, +8) (K = tokens).
  const __amdgpu_buffer_rsrc_t rtv = make_rsrc(
      a.dtv + ((int64_t)tb * a.kbv + 8 * vt) * kBlockElems, 8 * (int64_t)kBlockBytes);
  const __amdgpu_buffer_rsrc_t rvt = make_rsrc(
      a.dvt + ((int64_t)vt * a.kbn + 8 * tb) * kBlockElems, 8 * (int64_t)kBlockBytes);
  // The stage arrays are free after the main loop: the tile's 8 dtv blocks
  // (128 KiB) are assembled there, block b in sa[b] (b < 4) or sb[b - 4].
  char* lds[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) lds[i] = wm ? sb[i] : sa[i];
  dlogits_epilogue<CAP, true>(
      acc, a.coef, a.lab, a.N, n0, vg0, a.V, DzCoef{0.f, 0.f, 0.f, 0.f, 0.f, a.cap, a.cap_k, a.inv_cap, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f},
      wm, wn, lane,
      [&](int i, int n, int m0, u32x2_t v) {
        *reinterpret_cast<u32x2_t*>(lds[i] + blk_byte(n, m0 & 31)) = v;
      },
      rvt);
  __syncthreads();
  copy_out_tile(sa, sb, rtv);
}

// ---- fused path: the logit gradient from the stored logits ----------------------

struct FusedDzArgs {
  uint16_t* dtv;           // chunk image (strips of 256 tokens, K = vocabulary): z' - mref in
                           // bf16 on entry (fwd_tile STORE), the logit gradient on exit
  uint16_t* dvt;           // chunk image of its transpose (strips of 256 vocabulary rows,
                           // K = the chunk's tokens)
  const float* mref;       // [2 VT][mld] reference maxima (fwd_tile STORE)
  int64_t mld;
  const DzToken* coef;     // the chunk's rows (compacted)
  const int32_t* lab;      // the chunk's label codes
  const int32_t* nvalid;   // device: number of compacted tokens
  int r0;                  // first compacted row of the chunk
  int64_t rows;            // chunk rows that have coefficients and label codes (rows past
                           // them get zero gradient)
  int64_t V;
  int VT, TB;              // vocabulary tiles, token blocks of the chunk
  int group;
  int kbv, kbn;            // K blocks per strip of dtv (VT * 8) and dvt (TB * 8)
  float cap, inv_cap;
};

// Half wm of tile (tb, vt) of a token chunk: vocabulary rows [128 wm, +128)
// of the tile, all 256 tokens, by four waves wn = 0..3 laid out as in the
// GEMM tile. The half tile's four dtv blocks (64 KiB, contiguous) come into
// LDS by direct DMA (1 KiB per wave instruction); each lane reads its pieces
// of the stored z' - mref in the lane layout of the MFMA accumulators, adds
// mref back and forms the logit gradient exactly as bwd_dlogits_kernel does
// from its recomputed tile, writing the dtv pieces back in place in LDS and
// the dvt pieces directly; the four blocks then go back to dtv with 16-byte
// stores (1 KiB per wave instruction). Memory-bound: 2 bytes read and 4
// written per logit. 64 KiB of LDS per block leaves room for two blocks per
// CU, so one block's transfers overlap the other's arithmetic.
constexpr int kDzThreads = 256;

template <bool CAP>
__global__ void __launch_bounds__(kDzThreads) fused_dlogits_kernel(FusedDzArgs a) {
  __shared__ __attribute__((aligned(1024))) char lds[4 * kBlockBytes];
  const int left = (*a.nvalid - a.r0 + kTile - 1) / kTile;
  const int tbv = left < a.TB ? (left > 0 ? left : 0) : a.TB;
  const int tile = (int)(blockIdx.x >> 1);
  if (tile >= tbv * a.VT) return;
  int tb, vt;
  group_map(xcd_remap(tile, tbv * a.VT), tbv, a.VT, a.group, tb, vt);
  const int lane = threadIdx.x & 63;
  const int wm = (int)(blockIdx.x & 1), wn = threadIdx.x >> 6;
  const int64_t n0 = (int64_t)tb * kTile;
  const int64_t vg0 = (int64_t)vt * kTile;
  constexpr int kHalf = 4 * kBlockBytes;
  const __amdgpu_buffer_rsrc_t rtv = make_rsrc(
      a.dtv + ((int64_t)tb * a.kbv + 8 * vt + 4 * wm) * kBlockElems, kHalf);
  const __amdgpu_buffer_rsrc_t rvt = make_rsrc(
      a.dvt + ((int64_t)vt * a.kbn + 8 * tb) * kBlockElems, 8 * (int64_t)kBlockBytes);
#pragma unroll
  for (int q = 0; q < kHalf / 1024 / 4; ++q) {
    const int c = wn * (kHalf / 1024 / 4) + q;  // 1 KiB piece of this wave instruction
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rtv, (lds_void_t*)(lds + c * 1024), 16,
                                             (uint32_t)(c * 1024 + lane * 16), 0, 0, 0);
  }
  wait_vmcnt<0>();
  __syncthreads();
  // Byte offset in LDS of rows m0 .. m0+3 (block i of the half) of token column n.
  auto piece = [&](int i, int n, int m0) { return i * kBlockBytes + blk_byte(n, m0 & 31); };
  Acc acc;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = acc_col(wn, j, lane);
    const float mw = a.mref[(int64_t)(2 * vt + wm) * a.mld + n0 + n];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const u32x2_t v =
            *reinterpret_cast<const u32x2_t*>(lds + piece(i, n, acc_row(wm, i, rq * 4, lane)));
        acc[i][j][rq * 4 + 0] = __uint_as_float(v[0] << 16) + mw;
        acc[i][j][rq * 4 + 1] = __uint_as_float(v[0] & 0xFFFF0000u) + mw;
        acc[i][j][rq * 4 + 2] = __uint_as_float(v[1] << 16) + mw;
        acc[i][j][rq * 4 + 3] = __uint_as_float(v[1] & 0xFFFF0000u) + mw;
      }
  }
  // Each lane rewrites only the pieces it read: no barrier between.
  dlogits_epilogue<CAP, false>(
      acc, a.coef, a.lab, a.rows, n0, vg0, a.V, DzCoef{0.f, 0.f, 0.f, 0.f, 0.f, a.cap, 0.f, a.inv_cap, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f},
      wm, wn, lane,
      [&](int i, int n, int m0, u32x2_t v) { *reinterpret_cast<u32x2_t*>(lds + piece(i, n, m0)) = v; },
      rvt);
  __syncthreads();
#pragma unroll
  for (int q = 0; q < kHalf / (kDzThreads * 16); ++q) {
    const int off = (q * kDzThreads + (int)threadIdx.x) * 16;
    __builtin_amdgcn_raw_buffer_store_b128(*reinterpret_cast<const u32x4_t*>(lds + off), rtv,
                                           (uint32_t)off, 0, 0);
  }
}

// ---- backward: dH (+)= D W_chunk^T ---------------------------------------------

enum { DX_ONLY = 0, DX_FIRST = 1, DX_MID = 2, DX_LAST = 3 };

struct DxArgs {
  const uint16_t* dtv;     // blocked D of the chunk (strips of tokens, K = vocabulary)
  const uint16_t* wb;      // blocked weight of the chunk (strips of 256 hidden rows, K = vocabulary)
  int64_t N, H, V;
  int kbv;                 // K blocks per strip of both images (chunk capacity / 32)
  int nk;                  // K blocks of the chunk
  int TB, HT;              // token blocks, hidden tiles
  int group;
  int splits;              // K splits of the chunk; split s accumulates into acc + s*N*H
  float* acc;              // [splits][N,H] fp32 accumulators over chunks (compacted rows)
  void* gh;                // [N,H] output, bf16 or fp32 (F32OUT); row idx[r] of compacted row r
  const int32_t* idx;      // [N] compacted -> original token (of this launch's rows)
  const int32_t* nvalid;   // device: number of compacted tokens
  int r0;                  // compacted row of this launch's row 0 (a token chunk; else 0);
                           // N, TB, acc, idx and dtv cover the launch's rows
};

// C[t][h] = sum_v D[t][v] W[h][v0 + v] over the chunk. MODE: DX_ONLY (single chunk: write
// the output), DX_FIRST (store fp32), DX_MID (add into fp32), DX_LAST (add and
// write the output). F32OUT: the output is fp32, else bf16. Out-of-range rows
// and columns fall outside the buffer resources.
// Token tiles of a dH launch that hold compacted tokens; the tiles are
// numbered over them only (dx_tiles() of them in all).
__device__ __forceinline__ int dx_token_tiles(const DxArgs& a) {
  const int left = (*a.nvalid - a.r0 + kTile - 1) / kTile;
  return left < a.TB ? (left > 0 ? left : 0) : a.TB;
}
__device__ __forceinline__ int dx_tiles(const DxArgs& a) {
  return dx_token_tiles(a) * a.HT * a.splits;
}

// Tile L (logical, < dx_tiles(a)) of the dH contraction.
template <int MODE, bool F32OUT>
__device__ __forceinline__ void dx_tile(const DxArgs& a, int L, char* const (&sa)[kStages],
                                        char* const (&sb)[kStages]) {
  const int nval = *a.nvalid - a.r0;  // valid rows from this launch's row 0
  const int tbv = dx_token_tiles(a);
  const int per_split = tbv * a.HT;
  const int sp = L / per_split;
  int tb, ht;
  group_map(L - sp * per_split, tbv, a.HT, a.group, tb, ht);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6, wm = wave & 1, wn = wave >> 1;
  const int64_t m0 = (int64_t)tb * kTile, h0 = (int64_t)ht * kTile;
  // K blocks [kb0, kb1) of the chunk belong to split sp.
  const int kper = (a.nk + a.splits - 1) / a.splits;
  const int kb0 = sp * kper;
  const int kb1 = kb0 + kper < a.nk ? kb0 + kper : a.nk;
  Acc acc;
  {
    Mainloop ml;
    ml.run(sa, sb, blocked_a(Strip{a.dtv + (int64_t)tb * a.kbv * kBlockElems, a.kbv}, kb0),
           Strip{a.wb + (int64_t)ht * a.kbv * kBlockElems, a.kbv}, kb0, kb1 - kb0, acc);
  }
  const int64_t base = (int64_t)sp * a.N * a.H + m0 * a.H + h0;
  const int64_t span = (a.N - m0) * a.H - h0;  // elements from the tile origin to the split's end
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.acc + base, span * 4);
  constexpr int kOut = F32OUT ? 4 : 2;  // bytes per output element
  char* const gh = static_cast<char*>(a.gh);
  // Per 4 accumulator rows of a 32 x 32 block, a quad transpose hands lane
  // 4q+a row (first + a) at the quad's four columns: 16-byte fp32 and 8-byte
  // bf16 accesses. H is a multiple of 4, so a quad's columns are all inside or
  // all outside. Output rows go to their original token (idx); compacted rows
  // past the valid tokens are not written.
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int hq = acc_col(wn, j, lane) & ~3;
    const bool hok = h0 + hq < a.H;
    // The accumulator values this column pair adds to (DX_MID, DX_LAST), all
    // requested before the first is used.
    f32x4_t old[16];
    if constexpr (MODE == DX_MID || MODE == DX_LAST) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int row = acc_row(wm, i, rq * 4, lane) + (lane & 3);
          old[i * 4 + rq] = buf_load_f32x4(ra, hok ? (uint32_t)(row * a.H + hq) * 4 : kOOB);
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int row = acc_row(wm, i, rq * 4, lane) + (lane & 3);
        const uint32_t e = (uint32_t)(row * a.H + hq);
        const bool out_ok = hok && m0 + row < nval;
        char* dst = out_ok ? gh + ((int64_t)a.idx[m0 + row] * a.H + h0 + hq) * kOut : nullptr;
        const float x[4] = {acc[i][j][rq * 4], acc[i][j][rq * 4 + 1], acc[i][j][rq * 4 + 2],
                            acc[i][j][rq * 4 + 3]};
        if constexpr (MODE == DX_ONLY && !F32OUT) {
          const u32x2_t v = quad_transpose_bf16(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]));
          if (out_ok) *reinterpret_cast<u32x2_t*>(dst) = v;
        } else if constexpr (MODE == DX_ONLY) {
          const f32x4_t v = quad_transpose_f32(x[0], x[1], x[2], x[3]);
          if (out_ok) *reinterpret_cast<f32x4_t*>(dst) = v;
        } else {
          f32x4_t v = quad_transpose_f32(x[0], x[1], x[2], x[3]);
          const uint32_t o = hok ? e * 4 : kOOB;
          if constexpr (MODE != DX_FIRST) v += old[i * 4 + rq];
          if constexpr (MODE == DX_LAST && F32OUT) {
            if (out_ok) *reinterpret_cast<f32x4_t*>(dst) = v;
          } else if constexpr (MODE == DX_LAST) {
            const u32x2_t b = u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
            if (out_ok) *reinterpret_cast<u32x2_t*>(dst) = b;
          } else {
            buf_store_f32x4(v, ra, o);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);  // one 32 x 32 block at a time
    }
  }
}

template <int MODE, bool F32OUT>
__global__ void __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                               amdgpu_waves_per_eu(2, 2)))
bwd_dx_kernel(DxArgs a) {
  FLCE_DECLARE_STAGES(sa, sb);
  const int total = dx_tiles(a);
  if ((int)blockIdx.x >= total) return;
  dx_tile<MODE, F32OUT>(a, xcd_remap(blockIdx.x, total), sa, sb);
}

// With K-split dH: grad_hidden row idx[r] = sum over splits of acc[s][r],
// for the rows r < min(n - r0, N) (n valid tokens, r0 the compacted row of
// row 0), in split order; bf16 (RNE) or fp32.
template <bool F32OUT>
__global__ void __launch_bounds__(256) dx_finalize_kernel(const float* __restrict__ acc, int splits,
                                                          int64_t N, int64_t H,
                                                          const int32_t* __restrict__ idx,
                                                          const int32_t* __restrict__ nvalid,
                                                          int64_t r0, void* __restrict__ gh) {
  const int64_t nl = (int64_t)*nvalid - r0;
  const int64_t n = nl < N ? (nl > 0 ? nl : 0) : N;
  const int64_t q = H / 4;  // 4-element groups per row
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n * q; e += (int64_t)gridDim.x * 256) {
    const int64_t r = e / q, c = (e % q) * 4;
    f32x4_t v = *reinterpret_cast<const f32x4_t*>(acc + r * H + c);
    for (int s = 1; s < splits; ++s)
      v += *reinterpret_cast<const f32x4_t*>(acc + (int64_t)s * N * H + r * H + c);
    const int64_t o = (int64_t)idx[r] * H + c;
    if constexpr (F32OUT)
      *reinterpret_cast<f32x4_t*>(static_cast<float*>(gh) + o) = v;
    else
      *reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(gh) + o) =
          u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  }
}

// ---- backward: dW_chunk = hidden^T D ------------------------------------------

// How bwd_dw_kernel stores its tile: DW_DIRECT writes dW (bf16 or fp32);
// DW_SPLIT writes an fp32 partial of its token split. DW_CHUNK is the fused
// path's token chunk, whose store is chosen on the device from the number n
// of valid tokens: a chunk holding none exits (chunk 0 excepted, which writes
// zeros when n = 0); chunk 0 stores the fp32 accumulator, or writes dW when
// it also holds the last valid token; later chunks add into the accumulator,
// and the one holding the last valid token adds and writes dW. Empty chunks
// thus cost no pass over the accumulator.
enum { DW_DIRECT = 0, DW_SPLIT = 1, DW_CHUNK = 2 };
enum { DWS_DIRECT = 0, DWS_SPLIT = 1, DWS_FIRST = 2, DWS_MID = 3, DWS_LAST = 4 };

struct DwArgs {
  const uint16_t* xtb;     // blocked hidden^T (strips of 256 hidden rows, K = tokens)
  const uint16_t* dvt;     // blocked D^T of the chunk (strips of 256 vocabulary rows, K = tokens)
  int64_t N, H, V, v0, vc;
  int kbn;                 // K blocks per strip of dvt (token blocks * 8)
  int kbn_a;               // K blocks per strip of xtb
  int ka0;                 // xtb's K block at dvt's K block 0 (a token chunk's first block)
  const int32_t* nvalid;   // device: number of compacted tokens (the K extent)
  int r0;                  // compacted row at dvt's K index 0
  int64_t rows;            // DW_CHUNK: rows of this chunk
  int first;               // DW_CHUNK: 1 for the first chunk
  int HT, VTc, splits;
  int group;
  int kper;                // K blocks per split
  int64_t ldp;             // row stride of the split partials
  void* gw;                // [H,V] output, bf16 or fp32 (F32OUT), rows ldo apart
  int64_t ldo;             // row stride of gw and accw (V, or V rounded up to 8 when the
                           // output goes to a padded buffer)
  float* part;             // [splits][H][ldp] fp32 (DW_SPLIT)
  float* accw;             // [H,V] fp32 accumulator over chunks (DW_CHUNK; grad_weight
                           // itself when F32OUT)
};

// Stores tile (h0, vl0) of split sp as STORE (a DWS_ value) says.
template <int STORE, bool F32OUT>
__device__ __forceinline__ void dw_store_tile(const Acc& acc, const DwArgs& a, int64_t h0,
                                              int64_t vl0, int sp, int wm, int wn, int lane) {
  constexpr bool kSplit = STORE == DWS_SPLIT;
  constexpr bool kRead = STORE == DWS_MID || STORE == DWS_LAST;
  int64_t ld, base, span;
  if constexpr (kSplit) {
    ld = a.ldp;
    base = ((int64_t)sp * a.H + h0) * ld + vl0;
    span = (a.H - h0) * ld - vl0;
  } else {
    ld = a.ldo;
    base = h0 * ld + a.v0 + vl0;
    span = (a.H - h0) * ld - (a.v0 + vl0);
  }
  // Bytes per stored element: fp32 for partials, the accumulator and fp32 dW.
  constexpr int kOut = (STORE == DWS_DIRECT || STORE == DWS_LAST) && !F32OUT ? 2 : 4;
  float* const fdst =
      kSplit ? a.part : ((STORE == DWS_FIRST || STORE == DWS_MID) ? a.accw : nullptr);
  const __amdgpu_buffer_rsrc_t rs =
      fdst != nullptr ? make_rsrc(fdst + base, span * 4)
                      : make_rsrc(static_cast<char*>(a.gw) + base * kOut, span * kOut);
  const __amdgpu_buffer_rsrc_t racc = kRead ? make_rsrc(a.accw + base, span * 4) : rs;
  // Quad transposes as in bwd_dx_kernel. A quad at vq < vc may reach past vc
  // (vc not a multiple of 4) only into a padded output, whose row stride ldo
  // is vc rounded up to 8 and whose extra columns are never read back.
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int vq = acc_col(wn, j, lane) & ~3;
    const bool vok = vl0 + vq < a.vc;
    // The accumulator values this column pair adds to, all requested before
    // the first is used: one memory latency per 16 loads rather than per load.
    f32x4_t old[16];
    if constexpr (kRead) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int row = acc_row(wm, i, rq * 4, lane) + (lane & 3);
          old[i * 4 + rq] = buf_load_f32x4(racc, vok ? (uint32_t)(row * ld + vq) * 4 : kOOB);
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int row = acc_row(wm, i, rq * 4, lane) + (lane & 3);
        const uint32_t e = (uint32_t)(row * ld + vq);
        const float x[4] = {acc[i][j][rq * 4], acc[i][j][rq * 4 + 1], acc[i][j][rq * 4 + 2],
                            acc[i][j][rq * 4 + 3]};
        if constexpr (kOut == 4) {
          f32x4_t v = quad_transpose_f32(x[0], x[1], x[2], x[3]);
          if constexpr (kRead) v += old[i * 4 + rq];
          buf_store_f32x4(v, rs, vok ? e * 4 : kOOB);
        } else if constexpr (kRead) {
          const f32x4_t v = quad_transpose_f32(x[0], x[1], x[2], x[3]) + old[i * 4 + rq];
          buf_store_u32x2(u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])}, rs,
                          vok ? e * 2 : kOOB);
        } else {
          buf_store_u32x2(quad_transpose_bf16(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])), rs,
                          vok ? e * 2 : kOOB);
        }
      }
    }
  }
}

// Tile L (logical, < HT * VTc * splits) of the dW contraction:
// C[h][v] = sum_t hidden[t][h] D[t][v] over the split's (or chunk's) tokens.
// `last` (DW_CHUNK): the chunk holds the last valid token.
template <int MODE, bool F32OUT>
__device__ __forceinline__ void dw_tile(const DwArgs& a, int L, bool last,
                                        char* const (&sa)[kStages], char* const (&sb)[kStages]) {
  const int n = *a.nvalid;
  const int per = a.HT * a.VTc;
  const int sp = L / per;
  int ht, vt;
  group_map(L - sp * per, a.HT, a.VTc, a.group, ht, vt);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6, wm = wave & 1, wn = wave >> 1;
  const int64_t h0 = (int64_t)ht * kTile, vl0 = (int64_t)vt * kTile;
  const int kbeg = sp * a.kper;
  // K blocks holding compacted tokens, from the launch's first row.
  const int kval = (n - a.r0 + kBK - 1) / kBK;
  const int klim = kval < a.kbn ? (kval > 0 ? kval : 0) : a.kbn;
  const int kend = kbeg + a.kper < klim ? kbeg + a.kper : klim;
  Acc acc;
  {
    Mainloop ml;
    ml.run(sa, sb,
           blocked_a(Strip{a.xtb + (int64_t)ht * a.kbn_a * kBlockElems, a.kbn_a}, a.ka0 + kbeg),
           Strip{a.dvt + (int64_t)vt * a.kbn * kBlockElems, a.kbn}, kbeg, kend - kbeg, acc);
  }
  if constexpr (MODE == DW_SPLIT) {
    dw_store_tile<DWS_SPLIT, F32OUT>(acc, a, h0, vl0, sp, wm, wn, lane);
  } else if constexpr (MODE == DW_DIRECT) {
    dw_store_tile<DWS_DIRECT, F32OUT>(acc, a, h0, vl0, sp, wm, wn, lane);
  } else {
    if (a.first && last)
      dw_store_tile<DWS_DIRECT, F32OUT>(acc, a, h0, vl0, sp, wm, wn, lane);
    else if (a.first)
      dw_store_tile<DWS_FIRST, F32OUT>(acc, a, h0, vl0, sp, wm, wn, lane);
    else if (last)
      dw_store_tile<DWS_LAST, F32OUT>(acc, a, h0, vl0, sp, wm, wn, lane);
    else
      dw_store_tile<DWS_MID, F32OUT>(acc, a, h0, vl0, sp, wm, wn, lane);
  }
}

template <int MODE, bool F32OUT>
__global__ void __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                               amdgpu_waves_per_eu(2, 2)))
bwd_dw_kernel(DwArgs a) {
  FLCE_DECLARE_STAGES(sa, sb);
  bool last = true;
  if constexpr (MODE == DW_CHUNK) {
    const int n = *a.nvalid;
    if (!a.first && n <= a.r0) return;  // no valid token in this chunk
    last = n <= a.r0 + a.rows;          // the chunk holds the last valid token
  }
  dw_tile<MODE, F32OUT>(a, xcd_remap(blockIdx.x, gridDim.x), last, sa, sb);
}

// dH and dW of one vocabulary chunk in a single launch (dW stored directly):
// the dH tiles take logical ids [0, dx_tiles), the dW tiles the rest, so
// with equal K lengths the two tile sets fill the GPU as one grid (e.g. two
// grids of 4.5 rounds of CUs each become one of 9 rounds). The XCD-aware
// numbering gives each XCD a contiguous range of the combined ids.
template <int DXMODE, bool F32OUT>
__global__ void __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                               amdgpu_waves_per_eu(2, 2)))
bwd_dxdw_kernel(DxArgs x, DwArgs w) {
  FLCE_DECLARE_STAGES(sa, sb);
  const int ndx = dx_tiles(x);
  const int total = ndx + w.HT * w.VTc * w.splits;
  if ((int)blockIdx.x >= total) return;
  const int L = xcd_remap(blockIdx.x, total);
  if (L < ndx)
    dx_tile<DXMODE, F32OUT>(x, L, sa, sb);
  else
    dw_tile<DW_DIRECT, F32OUT>(w, L - ndx, true, sa, sb);
}

// Sums the split partials in split order and writes dW for the chunk (bf16,
// or fp32 with F32OUT).
template <bool F32OUT>
__global__ void __launch_bounds__(256) dw_reduce_kernel(const float* __restrict__ part, int splits,
                                                        int64_t H, int64_t vc, int64_t ldd,
                                                        int64_t ldo, int64_t v0, void* gw) {
  const int64_t n = H * vc;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) {
    const int64_t h = e / vc, v = e % vc;
    float s = 0.f;
    for (int k = 0; k < splits; ++k) s += part[((int64_t)k * H + h) * ldd + v];
    if constexpr (F32OUT)
      static_cast<float*>(gw)[h * ldo + v0 + v] = s;
    else
      static_cast<uint16_t*>(gw)[h * ldo + v0 + v] = (uint16_t)(pack_bf16x2(s, 0.f) & 0xFFFFu);
  }
}

// ---- measurement: the sustained MFMA rate ------------------------------------------

// lowbias32, an integer mixer published with C. Wellons' hash-prospector:
// a counter-based source of operand bits for the probe below.
__device__ __forceinline__ uint32_t probe_hash(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// Eight bf16 values uniform in [-2, 2) from counter c (or zeros).
__device__ __forceinline__ bf16x8_t probe_frag(uint32_t c, bool zero) {
  u32x4_t w;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float v[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t x = probe_hash(c * 8u + (uint32_t)(2 * e + h));
      v[h] = zero ? 0.f : (float)(x >> 8) * (4.f / 16777216.f) - 2.f;
    }
    w[e] = pack_bf16x2(v[0], v[1]);
  }
  return __builtin_bit_cast(bf16x8_t, w);
}

// Throughput of the GEMM kernels' wave tile (`steps` 16-wide K steps of
// 4 x 2 v_mfma_f32_32x32x16_bf16 per wave, two waves per SIMD, one block per
// CU) with the GEMM kernels' data movement added piece by piece (the
// template argument is the mode; mode 1 runs the mode-0 code with `zero`):
//   mode 0  operands in registers, pseudo-random, four sets cycled;
//   mode 1  the same with zero operands (a run-time flag, so the compiler
//           cannot fold the products);
//   mode 2  mode 0 with every step's six operand fragments read from LDS
//           (ds_read_b128, as the blocked operands are), 32 KiB of random data;
//   mode 3  mode 2 plus the global -> LDS DMA of a 256 x 256 block tile,
//           32 KiB per block per 32-deep K block (1 KiB pieces), from a 2 MiB
//           window of `src` that all blocks share, so it stays in L2.
// No result depends on the loaded data; the accumulators are summed into
// out (one float per thread) so that nothing is elided.
template <int MODE>
__global__ void __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                               amdgpu_waves_per_eu(2, 2)))
mfma_probe_kernel(int steps, int zero, float* __restrict__ out, const uint16_t* __restrict__ src) {
  constexpr bool kLds = MODE >= 2;
  __shared__ __attribute__((aligned(1024))) char fr[kLds ? kBlockBytes * 2 : 16];
  __shared__ __attribute__((aligned(1024))) char dm[MODE == 3 ? kBlockBytes * 2 : 16];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint32_t id = blockIdx.x * kThreads + threadIdx.x;
  bf16x8_t a[4][4], b[4][2];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
#pragma unroll
    for (int i = 0; i < 4; ++i) a[s][i] = probe_frag(id * 24u + (uint32_t)(s * 6 + i), zero != 0);
#pragma unroll
    for (int j = 0; j < 2; ++j) b[s][j] = probe_frag(id * 24u + (uint32_t)(s * 6 + 4 + j), zero != 0);
  }
  if constexpr (kLds) {
    // 64 bytes of random fragments per thread.
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<bf16x8_t*>(fr + threadIdx.x * 64 + q * 16) = probe_frag(id * 4u + q + 7u, false);
    __syncthreads();
  }
  Acc acc;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  for (int t = 0; t < steps; t += 4) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if constexpr (MODE == 3) {
        if ((s & 1) == 0) {
          // One 32-deep K block every two steps: 4 KiB per wave in 1 KiB pieces.
          const uint32_t kb = (uint32_t)((t + s) >> 1) & 63u;  // 64 x 32 KiB = 2 MiB window
          const __amdgpu_buffer_rsrc_t rs =
              make_rsrc(src + (size_t)kb * (2 * kBlockElems), 2 * kBlockBytes);
#pragma unroll
          for (int q = 0; q < 4; ++q)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rs, (lds_void_t*)(dm + (w * 4 + q) * 1024), 16,
                (uint32_t)((w * 4 + q) * 1024 + lane * 16), 0, 0, 0);
          wait_vmcnt<8>();
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s][i], b[s][j], acc[i][j], 0, 0, 0);
      if constexpr (kLds) {
        // Next use of this operand set: six fragments from LDS (distinct
        // 1 KiB rows per instruction, 16 consecutive bytes per lane).
        const int o = (((t + s) * 6) & 31) * 1024 + lane * 16;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          a[s][i] = *reinterpret_cast<const bf16x8_t*>(fr + ((o + i * 1024) & (2 * kBlockBytes - 1)));
#pragma unroll
        for (int j = 0; j < 2; ++j)
          b[s][j] =
              *reinterpret_cast<const bf16x8_t*>(fr + ((o + (4 + j) * 1024) & (2 * kBlockBytes - 1)));
      }
    }
  }
  if constexpr (MODE == 3) wait_vmcnt<0>();
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) sum += acc[i][j][r];
  out[id] = sum;
}

// Fills n 16-bit values with pseudo-random bf16 bit patterns in [-2, 2).
__global__ void __launch_bounds__(256) probe_fill_kernel(uint16_t* __restrict__ p, int64_t n) {
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) {
    const uint32_t x = probe_hash((uint32_t)e * 2654435761u + 12345u);
    p[e] = (uint16_t)(bf16_bits((float)(x >> 8) * (4.f / 16777216.f) - 2.f));
  }
}

// dst [rows, ldd] = src [rows, cols] (16-bit elements) with columns cols..ldd-1
// zero: a weight whose row length is not a multiple of 8, re-laid out so that
// every row starts 16-byte aligned. One element per thread, grid-stride.
__global__ void __launch_bounds__(256) pad_cols_kernel(const uint16_t* __restrict__ src,
                                                       int64_t rows, int64_t cols, int64_t ldd,
                                                       uint16_t* __restrict__ dst) {
  const int64_t n = rows * ldd;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) {
    const int64_t r = e / ldd, c = e - r * ldd;
    dst[e] = c < cols ? src[r * cols + c] : (uint16_t)0;
  }
}

// dst [rows, cols] = the first cols columns of src [rows, lds]; elements of
// ELEM bytes (2: bf16, 4: fp32).
template <int ELEM>
__global__ void __launch_bounds__(256) unpad_cols_kernel(const void* __restrict__ src, int64_t rows,
                                                         int64_t lds, int64_t cols,
                                                         void* __restrict__ dst) {
  typedef typename std::conditional<ELEM == 4, uint32_t, uint16_t>::type T;
  const T* s = static_cast<const T*>(src);
  T* d = static_cast<T*>(dst);
  const int64_t n = rows * cols;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) {
    const int64_t r = e / cols, c = e - r * cols;
    d[e] = s[r * lds + c];
  }
}

// Writes zeros (used for empty inputs; a kernel rather than a memset so the
// enqueued work is plain kernels only).
__global__ void __launch_bounds__(256) fill_zero_kernel(uint32_t* __restrict__ p, int64_t n32) {
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n32; e += (int64_t)gridDim.x * 256)
    p[e] = 0u;
}

}  // namespace flce
