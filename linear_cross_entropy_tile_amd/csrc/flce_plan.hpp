// The host planner of the fused linear cross-entropy head: argument checks,
// the launch plan (tile counts, vocabulary and token chunks, K splits) and the
// byte layout of every workspace. Host-only C++ without HIP, so that it also
// builds on its own for sanitizer checks of the layout arithmetic.
#pragma once

#include <cmath>
#include <cstddef>
#include <cstdint>
#include <cstdlib>

#include "flce.h"
#include "flce_layout.hpp"

namespace flce {

constexpr size_t kAlign = 256;
constexpr size_t kHeaderBytes = 256;
// Limits keep every 32-bit buffer offset below 2^31: a blocked strip of K
// values takes K * 512 bytes (K padded to 256 for the vocabulary).
constexpr int64_t kMaxN = (int64_t)1 << 21;
constexpr int64_t kMaxH = (int64_t)1 << 20;
constexpr int64_t kMaxV = ((int64_t)1 << 22) - 256;
constexpr int64_t kMaxVc = (int64_t)1 << 18;
constexpr int kNumCUs = 256;                              // MI355X
// Bytes of both bf16 logit-gradient images: enough for 16384 columns per
// chunk (fewer passes over the fp32 dH accumulator, full tile rounds), within
// [1 GiB, 4 GiB].
constexpr size_t kMinDBudget = (size_t)1 << 30;
constexpr size_t kMaxDBudget = (size_t)4 << 30;
constexpr int64_t kTargetVc = 16384;

inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---- the plan: every size the kernels and the workspace depend on ----------
struct Plan {
  int64_t N, H, V;
  int TB, VT, HT;      // token blocks, vocabulary tiles, hidden tiles (256 each)
  int hkb;             // K blocks of a strip with K = H
  int nkb;             // K blocks of a strip with K = tokens (TB * 8)
  int64_t Vc;          // vocabulary chunk capacity (multiple of 256)
  int kbv;             // Vc / 32
  int nchunks;
  int VTc;             // vocabulary tiles per chunk
  int dx_splits;       // K splits of the dH contraction within a chunk
  int dw_splits;       // split over tokens of the dW contraction
  int dw_kper;         // K blocks per dW split
  int group;           // tile rows per XCD patch of the block -> tile map
  // A vocabulary that is not a multiple of 8: the weight is copied with rows
  // of V8 = V rounded up to 8 (zero columns past V), and dW is formed in a
  // buffer of the same row stride and copied out.
  bool padw;
  int64_t V8;
  // forward workspace
  size_t f_idx, f_labc, f_part, f_zlab, f_bsum, f_xb, f_wp, f_total;
  // backward workspace
  size_t b_lab, b_idx, b_coef, b_wb, b_xb, b_xtb, b_dtv, b_dvt, b_acc, b_part, b_wp, b_gwp,
      b_total;
};

inline size_t env_size(const char* name, size_t dflt) {
  const char* s = std::getenv(name);
  if (s == nullptr || *s == 0) return dflt;
  char* end = nullptr;
  const unsigned long long v = std::strtoull(s, &end, 10);
  return (end != s && v > 0) ? (size_t)v : dflt;
}

inline Plan make_plan(int64_t N, int64_t H, int64_t V, int reduction) {
  Plan p{};
  p.N = N;
  p.H = H;
  p.V = V;
  p.TB = (int)ceil_div(N, kTile);
  p.VT = (int)ceil_div(V, kTile);
  p.HT = (int)ceil_div(H, kTile);
  p.hkb = (int)ceil_div(H, kBK);
  p.V8 = ceil_div(V, 8) * 8;
  p.padw = p.V8 != V;
  p.nkb = p.TB * (kTile / kBK);
  // The vocabulary is processed in chunks of Vc columns: the weight images
  // are built per chunk, and the backward's two bf16 images of the logit
  // gradient (2 x 2 bytes x 256 TB x Vc) stay within budget. FLCE_D_BUDGET (bytes)
  // overrides the budget, for tests and tuning only; the 2048-column floor
  // applies to the default budget.
  const size_t budget = env_size("FLCE_D_BUDGET", 0);
  const int64_t vfull = (int64_t)p.VT * kTile;
  const int64_t npad = (int64_t)(p.TB > 0 ? p.TB : 1) * kTile;
  size_t bud = budget;
  if (bud == 0) {
    bud = 4 * (size_t)npad * (size_t)kTargetVc;
    bud = bud < kMinDBudget ? kMinDBudget : (bud > kMaxDBudget ? kMaxDBudget : bud);
  }
  int64_t vc = (int64_t)(bud / (4 * (size_t)npad)) / kTile * kTile;
  if (vc < (budget > 0 ? kTile : 2048)) vc = budget > 0 ? kTile : 2048;
  if (vc > kMaxVc) vc = kMaxVc;
  if (vc > vfull) vc = vfull;
  p.Vc = vc;
  p.kbv = (int)(vc / kBK);
  p.nchunks = (int)ceil_div(V, vc);
  p.VTc = (int)(vc / kTile);
  // dH: split each chunk's K range when the N x H tiles alone fill the GPU
  // poorly; S minimises ceil(tiles * S / CUs) / S (rounds per unit of work).
  {
    const int64_t t = (int64_t)p.TB * p.HT;
    int best = 1;
    double bcost = 1e30;
    for (int sk = 1; sk <= 4; ++sk) {
      const double cost = (double)ceil_div(t * sk, kNumCUs) / sk;
      if (cost < bcost - 1e-9) {
        bcost = cost;
        best = sk;
      }
    }
    p.dx_splits = best;
  }
  // dW: split the token reduction when there are too few output tiles.
  const int64_t tiles = (int64_t)p.HT * p.VTc;
  int sp = 1;
  if (tiles < kNumCUs) {
    sp = (int)(kNumCUs / tiles);
    const int64_t maxsp = p.nkb / 32;  // keep >= 1024 tokens per split
    if (sp > maxsp) sp = (int)(maxsp > 1 ? maxsp : 1);
  }
  p.dw_kper = p.nkb > 0 ? (int)ceil_div(p.nkb, sp) : 1;
  p.dw_splits = p.nkb > 0 ? (int)ceil_div(p.nkb, p.dw_kper) : 1;
  // FLCE_GROUP overrides the patch height, for tuning only.
  p.group = (int)env_size("FLCE_GROUP", 4);

  const size_t blk = (size_t)kBlockBytes;
  size_t off = kHeaderBytes;
  p.f_idx = off;
  off = align_up(off + 4 * (size_t)N);
  p.f_labc = off;
  off = align_up(off + 4 * (size_t)N);
  p.f_part = off;
  off = align_up(off + 16 * (size_t)p.VT * (size_t)N);
  p.f_zlab = off;
  off = align_up(off + 4 * (size_t)N);
  p.f_bsum = off;
  off = align_up(off + (reduction != FLCE_REDUCTION_NONE ? 32 * (size_t)ceil_div(N, kCombineTokens) : 0));
  p.f_xb = off;
  off = align_up(off + blk * (size_t)p.TB * (size_t)p.hkb);
  p.f_wp = off;
  off = align_up(off + (p.padw ? 2 * (size_t)H * (size_t)p.V8 : 0));
  p.f_total = off;

  off = kHeaderBytes;
  p.b_lab = off;
  off = align_up(off + 4 * (size_t)N);
  p.b_idx = off;
  off = align_up(off + 4 * (size_t)N);
  p.b_coef = off;
  off = align_up(off + sizeof(DzToken) * (size_t)N);
  p.b_wb = off;
  off = align_up(off + blk * (size_t)p.HT * (size_t)p.kbv);
  p.b_xb = off;
  off = align_up(off + blk * (size_t)p.TB * (size_t)p.hkb);
  p.b_xtb = off;
  off = align_up(off + blk * (size_t)p.HT * (size_t)p.nkb);
  p.b_dtv = off;
  off = align_up(off + blk * (size_t)p.TB * (size_t)p.kbv);
  p.b_dvt = off;
  off = align_up(off + blk * (size_t)p.VTc * (size_t)p.nkb);
  p.b_acc = off;
  off = align_up(off + (p.nchunks > 1 || p.dx_splits > 1
                            ? 4 * (size_t)p.dx_splits * (size_t)N * (size_t)H : 0));
  p.b_part = off;
  off = align_up(off + (p.dw_splits > 1 ? 4 * (size_t)p.dw_splits * (size_t)H * (size_t)p.Vc : 0));
  // Padded weight copy and padded dW (room for fp32 gradients).
  p.b_wp = off;
  off = align_up(off + (p.padw ? 2 * (size_t)H * (size_t)p.V8 : 0));
  p.b_gwp = off;
  off = align_up(off + (p.padw ? 4 * (size_t)H * (size_t)p.V8 : 0));
  p.b_total = off;
  return p;
}

// Workspace of flce_merge_shards: header, compaction index and codes (the prep
// kernel's scratch), label logits, block sums.
inline size_t merge_idx_off(int64_t N) { return align_up(kHeaderBytes); }
inline size_t merge_labc_off(int64_t N) { return align_up(merge_idx_off(N) + 4 * (size_t)N); }
inline size_t merge_zlab_off(int64_t N) { return align_up(merge_labc_off(N) + 4 * (size_t)N); }
inline size_t merge_bsum_off(int64_t N) { return align_up(merge_zlab_off(N) + 4 * (size_t)N); }
inline size_t merge_bytes(int64_t N) {
  return align_up(merge_bsum_off(N) + 32 * (size_t)ceil_div(N > 0 ? N : 1, kCombineTokens));
}

// ---- the fused path's plan --------------------------------------------------
// The tokens are processed in chunks of TBc token blocks. Per chunk the
// forward keeps the capped logits of all V columns (bf16, two bytes each) and
// the logit gradient is formed from them in both blocked layouts, so the
// chunk images take 4 * 256 TBc * 256 VT bytes; with several chunks dW is
// accumulated over them in fp32 (H * V * 4 bytes, or in grad_weight itself
// when it is fp32). By default a chunk is the largest number of token blocks
// whose images fit in kFusedImageBudget (the recompute path's budget for its
// logit-gradient images), at least one block.
constexpr size_t kFusedImageBudget = (size_t)1 << 30;

struct FusedPlan {
  Plan b;              // TB, VT, HT, hkb, nkb, group of the shape
  int TBc;             // token blocks per chunk
  int nchunks;
  int dx_splits;       // K splits of dH per chunk
  int kbv;             // VT * 8: K blocks of a vocabulary-long strip
  bool dw_acc;         // a separate fp32 dW accumulator
  size_t idx, labc, zlab, part, bsum, coef, xb, xtb, wb, dtv, dvt, mref, dxacc, dwacc, wp, gwp,
      total;
};

inline FusedPlan make_fused_plan(int64_t N, int64_t H, int64_t V, const flce_options_t& o,
                          int64_t chunk_tokens) {
  FusedPlan f{};
  f.b = make_plan(N, H, V, o.reduction);
  const Plan& p = f.b;
  const int TB = p.TB;
  int tbc;
  if (chunk_tokens > 0) {
    tbc = (int)ceil_div(chunk_tokens, kTile);
  } else {
    const size_t per_block = 4 * (size_t)kTile * (size_t)kTile * (size_t)(p.VT > 0 ? p.VT : 1);
    const size_t fit = kFusedImageBudget / per_block;
    tbc = fit > (size_t)TB ? TB : (int)fit;
  }
  if (tbc > TB) tbc = TB;
  if (tbc < 1) tbc = 1;
  f.TBc = tbc;
  f.nchunks = TB > 0 ? (int)ceil_div(TB, tbc) : 0;
  f.kbv = p.VT * (kTile / kBK);
  {
    const int64_t t = (int64_t)tbc * p.HT;
    int best = 1;
    double bcost = 1e30;
    for (int sk = 1; sk <= 4; ++sk) {
      const double cost = (double)ceil_div(t * sk, kNumCUs) / sk;
      if (cost < bcost - 1e-9) {
        bcost = cost;
        best = sk;
      }
    }
    f.dx_splits = best;
  }
  f.dw_acc = f.nchunks > 1 && o.grad_dtype != FLCE_GRAD_F32;
  const size_t blk = (size_t)kBlockBytes;
  const size_t rows = (size_t)TB * kTile;    // compacted rows, padded
  const size_t crow = (size_t)tbc * kTile;   // rows of one chunk
  size_t off = kHeaderBytes;
  auto take = [&](size_t& field, size_t bytes) {
    field = off;
    off = align_up(off + bytes);
  };
  take(f.idx, 4 * (size_t)N);
  take(f.labc, 4 * (size_t)N);
  take(f.zlab, 4 * (size_t)N);
  take(f.part, 16 * (size_t)p.VT * (size_t)N);
  take(f.bsum, o.reduction != FLCE_REDUCTION_NONE ? 32 * rows / kCombineTokens : 0);
  take(f.coef, sizeof(DzToken) * rows);
  take(f.xb, blk * (size_t)TB * (size_t)p.hkb);
  take(f.xtb, blk * (size_t)p.HT * (size_t)p.nkb);
  take(f.wb, blk * (size_t)p.HT * (size_t)f.kbv);
  take(f.dtv, blk * (size_t)tbc * (size_t)f.kbv);
  take(f.dvt, blk * (size_t)p.VT * (size_t)tbc * (kTile / kBK));
  take(f.mref, 4 * 2 * (size_t)p.VT * crow);
  take(f.dxacc, f.dx_splits > 1 ? 4 * (size_t)f.dx_splits * crow * (size_t)H : 0);
  take(f.dwacc, f.dw_acc ? 4 * (size_t)H * (size_t)p.V8 : 0);
  // A vocabulary that is not a multiple of 8: padded weight copy and padded
  // dW (fp32 room), as on the recompute path.
  take(f.wp, p.padw ? 2 * (size_t)H * (size_t)p.V8 : 0);
  take(f.gwp, p.padw ? 4 * (size_t)H * (size_t)p.V8 : 0);
  f.total = off;
  return f;
}

// H must be a multiple of 8; V may take any value (see Plan::padw).
inline flce_status_t check_shape(int64_t N, int64_t H, int64_t V) {
  if (N < 0 || H < 1 || V < 1) return FLCE_ERR_BAD_SHAPE;
  if (N > kMaxN || H > kMaxH || V > kMaxV) return FLCE_ERR_BAD_SHAPE;
  if (H % 8 != 0) return FLCE_ERR_MISALIGNED;
  return FLCE_OK;
}

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

inline bool valid_reduction(int r) {
  return r == FLCE_REDUCTION_NONE || r == FLCE_REDUCTION_MEAN || r == FLCE_REDUCTION_SUM;
}

// fp32 gradient outputs: a dW tile's byte offsets (up to ~1024 * V) must stay
// below 2^31.
constexpr int64_t kMaxVF32 = (int64_t)1 << 21;


inline flce_status_t check_options(const flce_options_t* o) {
  if (o == nullptr) return FLCE_ERR_NULL_POINTER;
  if (!valid_reduction(o->reduction)) return FLCE_ERR_BAD_REDUCTION;
  if (!std::isfinite(o->softcap)) return FLCE_ERR_BAD_SOFTCAP;
  if (!std::isfinite(o->z_loss_scale) || o->z_loss_scale < 0.f) return FLCE_ERR_BAD_OPTION;
  if (o->grad_dtype != FLCE_GRAD_BF16 && o->grad_dtype != FLCE_GRAD_F32) return FLCE_ERR_BAD_OPTION;
  // Class weights only enter the mean and sum reductions.
  if (o->class_weight != nullptr && o->reduction == FLCE_REDUCTION_NONE) return FLCE_ERR_BAD_OPTION;
  if (((uintptr_t)o->class_weight & 3u) != 0) return FLCE_ERR_MISALIGNED;
  if (o->entropy_per_token != 0 && o->entropy_per_token != 1) return FLCE_ERR_BAD_OPTION;
  return FLCE_OK;
}

}  // namespace flce
