// Host side of libflce: argument checks, the launch plan, the workspace
// layout, kernel launches and the optional per-kernel event timing.
// Declarations and their documentation: include/flce.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <mutex>
#include <new>
#include <vector>

#include "flce.h"
#include "flce_kernels.hpp"
#include "flce_plan.hpp"

namespace {

using namespace flce;

// ---- kernel timing hooks --------------------------------------------------------
// flce_profile_read reports per kind in this order. K_PACK_WEIGHT no longer
// launches (the weight's dH image is written by the logit tiles themselves);
// its slot stays so that the indices of the later kinds do not move.
enum Kind {
  K_FWD_PREP, K_FWD_TILE, K_FWD_COMBINE, K_FWD_REDUCE, K_BWD_PREP, K_BWD_DLOGITS, K_BWD_DX,
  K_BWD_DW, K_DW_REDUCE, K_FILL, K_PACK_WEIGHT, K_PACK_HIDDEN, K_DX_FINALIZE, K_FUSED_TILE,
  K_FUSED_DLOGITS, K_BWD_DXDW, K_NUM
};
const char* kKindNames[K_NUM] = {"fwd_prep", "fwd_tile", "fwd_combine", "fwd_reduce", "bwd_prep",
                                 "bwd_dlogits", "bwd_dx", "bwd_dw", "dw_reduce", "fill_zero",
                                 "pack_weight", "pack_hidden", "dx_finalize", "fused_tile",
                                 "fused_dlogits", "bwd_dxdw"};

struct Pending {
  int kind;
  hipEvent_t a, b;
};
struct Profiler {
  std::mutex mu;
  bool on = false;
  std::vector<Pending> pending;
  std::vector<hipEvent_t> pool;
  int64_t launches[K_NUM] = {};
  double ms[K_NUM] = {};
  hipEvent_t get() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
  void drain() {
    for (auto& p : pending) {
      float t = 0.f;
      if (hipEventSynchronize(p.b) == hipSuccess && hipEventElapsedTime(&t, p.a, p.b) == hipSuccess) {
        launches[p.kind] += 1;
        ms[p.kind] += t;
      }
      pool.push_back(p.a);
      pool.push_back(p.b);
    }
    pending.clear();
  }
};
Profiler& prof() {
  static Profiler* p = new Profiler();
  return *p;
}

// Launches through `fn` on `st`, bracketed by events when timing is on.
template <class F>
flce_status_t launch(int kind, hipStream_t st, F fn) {
  Profiler& P = prof();
  hipEvent_t a = nullptr, b = nullptr;
  const bool timed = P.on;
  if (timed) {
    std::lock_guard<std::mutex> g(P.mu);
    a = P.get();
    b = P.get();
    if (a != nullptr) (void)hipEventRecord(a, st);
  }
  fn();
  if (hipGetLastError() != hipSuccess) return FLCE_ERR_HIP;
  if (timed && a != nullptr && b != nullptr) {
    (void)hipEventRecord(b, st);
    std::lock_guard<std::mutex> g(P.mu);
    P.pending.push_back({kind, a, b});
  }
  return FLCE_OK;
}

#define FLCE_TRY(x)                    \
  do {                                 \
    const flce_status_t _s = (x);      \
    if (_s != FLCE_OK) return _s;      \
  } while (0)

char* wsp(void* ws, size_t off) { return static_cast<char*>(ws) + off; }

flce_status_t zero_fill(void* p, size_t bytes, hipStream_t st) {
  const int64_t n32 = (int64_t)(bytes / 4);
  if (n32 == 0) return FLCE_OK;
  const int blocks = (int)(n32 / 256 + 1 < 4096 ? n32 / 256 + 1 : 4096);
  return launch(K_FILL, st, [&] {
    fill_zero_kernel<<<blocks, 256, 0, st>>>(static_cast<uint32_t*>(p), n32);
  });
}

// Blocked image of a K-contiguous source (element (r, k) at src[r * ld + k]);
// with `gather`, row r is source row gather[r] for r < *count.
flce_status_t pack_rows(int kind, const void* src, int64_t R, int64_t K, int64_t ld, int nkb,
                        const int32_t* gather, const int32_t* count, uint16_t* dst,
                        hipStream_t st) {
  const dim3 grid((unsigned)ceil_div(nkb, 8), (unsigned)ceil_div(R, kTile));
  return launch(kind, st, [&] {
    pack_rows_kernel<<<grid, 256, 0, st>>>(static_cast<const uint16_t*>(src), R, K, ld, nkb,
                                           gather, count, dst);
  });
}

// Blocked image of a row-contiguous source (element (r, k) at src[k * ld + r]);
// with `gather`, K index k reads source row gather[k] for k < *count.
flce_status_t pack_cols(int kind, const void* src, int64_t R, int64_t K, int64_t ld, int nkb,
                        const int32_t* gather, const int32_t* count, uint16_t* dst,
                        hipStream_t st) {
  const dim3 grid((unsigned)ceil_div(nkb, 2), (unsigned)ceil_div(R, kTile));
  return launch(kind, st, [&] {
    pack_cols_kernel<<<grid, 256, 0, st>>>(static_cast<const uint16_t*>(src), R, K, ld, nkb,
                                           gather, count, dst);
  });
}

// dst [rows, ldd] = src [rows, cols] with zero columns past cols.
flce_status_t pad_cols(const void* src, int64_t rows, int64_t cols, int64_t ldd, void* dst,
                       hipStream_t st) {
  const int64_t n = rows * ldd;
  const int blocks = (int)(ceil_div(n, 256) < 16384 ? ceil_div(n, 256) : 16384);
  return launch(K_FILL, st, [&] {
    pad_cols_kernel<<<blocks, 256, 0, st>>>(static_cast<const uint16_t*>(src), rows, cols, ldd,
                                            static_cast<uint16_t*>(dst));
  });
}

// dst [rows, cols] = the first cols columns of src [rows, lds] (2- or 4-byte elements).
flce_status_t unpad_cols(const void* src, int64_t rows, int64_t lds, int64_t cols, void* dst,
                         bool f32, hipStream_t st) {
  const int64_t n = rows * cols;
  const int blocks = (int)(ceil_div(n, 256) < 16384 ? ceil_div(n, 256) : 16384);
  return launch(K_FILL, st, [&] {
    if (f32)
      unpad_cols_kernel<4><<<blocks, 256, 0, st>>>(src, rows, lds, cols, dst);
    else
      unpad_cols_kernel<2><<<blocks, 256, 0, st>>>(src, rows, lds, cols, dst);
  });
}

// dH tiles in `mode` (DX_ONLY / FIRST / MID / LAST), bf16 or fp32 output.
flce_status_t launch_dx(const DxArgs& x, int mode, bool f32, int grid, hipStream_t st) {
  return launch(K_BWD_DX, st, [&] {
    switch (mode * 2 + (f32 ? 1 : 0)) {
      case DX_ONLY * 2: bwd_dx_kernel<DX_ONLY, false><<<grid, kThreads, 0, st>>>(x); break;
      case DX_ONLY * 2 + 1: bwd_dx_kernel<DX_ONLY, true><<<grid, kThreads, 0, st>>>(x); break;
      case DX_FIRST * 2: bwd_dx_kernel<DX_FIRST, false><<<grid, kThreads, 0, st>>>(x); break;
      case DX_FIRST * 2 + 1: bwd_dx_kernel<DX_FIRST, true><<<grid, kThreads, 0, st>>>(x); break;
      case DX_MID * 2: bwd_dx_kernel<DX_MID, false><<<grid, kThreads, 0, st>>>(x); break;
      case DX_MID * 2 + 1: bwd_dx_kernel<DX_MID, true><<<grid, kThreads, 0, st>>>(x); break;
      case DX_LAST * 2: bwd_dx_kernel<DX_LAST, false><<<grid, kThreads, 0, st>>>(x); break;
      default: bwd_dx_kernel<DX_LAST, true><<<grid, kThreads, 0, st>>>(x); break;
    }
  });
}

// dH tiles in `mode` and direct dW tiles of one chunk in one launch.
flce_status_t launch_dxdw(const DxArgs& x, const DwArgs& w, int mode, bool f32, int grid,
                          hipStream_t st) {
  return launch(K_BWD_DXDW, st, [&] {
    switch (mode * 2 + (f32 ? 1 : 0)) {
      case DX_ONLY * 2: bwd_dxdw_kernel<DX_ONLY, false><<<grid, kThreads, 0, st>>>(x, w); break;
      case DX_ONLY * 2 + 1: bwd_dxdw_kernel<DX_ONLY, true><<<grid, kThreads, 0, st>>>(x, w); break;
      case DX_FIRST * 2: bwd_dxdw_kernel<DX_FIRST, false><<<grid, kThreads, 0, st>>>(x, w); break;
      case DX_FIRST * 2 + 1: bwd_dxdw_kernel<DX_FIRST, true><<<grid, kThreads, 0, st>>>(x, w); break;
      case DX_MID * 2: bwd_dxdw_kernel<DX_MID, false><<<grid, kThreads, 0, st>>>(x, w); break;
      case DX_MID * 2 + 1: bwd_dxdw_kernel<DX_MID, true><<<grid, kThreads, 0, st>>>(x, w); break;
      case DX_LAST * 2: bwd_dxdw_kernel<DX_LAST, false><<<grid, kThreads, 0, st>>>(x, w); break;
      default: bwd_dxdw_kernel<DX_LAST, true><<<grid, kThreads, 0, st>>>(x, w); break;
    }
  });
}

// Whether a chunk's dH and dW tiles go into one launch (bwd_dxdw_kernel):
// only with direct dW stores, when the dH tiles' K length (per split) equals
// dW's (the token blocks) so that the combined grid stays balanced, and when
// one grid needs fewer rounds of CUs than the two. FLCE_DXDW=0 never
// combines, FLCE_DXDW=1 always does with direct dW stores (tests and tuning
// only).
bool combine_dxdw(const Plan& p, int nk, int64_t ndx, int64_t ndw) {
  if (p.dw_splits != 1) return false;
  const char* e = std::getenv("FLCE_DXDW");
  if (e != nullptr && e[0] == '0') return false;
  if (e != nullptr && e[0] == '1') return true;
  const int kper = (int)ceil_div(nk, p.dx_splits);
  if (kper != p.nkb) return false;
  return ceil_div(ndx, kNumCUs) + ceil_div(ndw, kNumCUs) > ceil_div(ndx + ndw, kNumCUs);
}

// grad_hidden rows of compacted rows [r0, r0 + rows) from the K-split dH
// accumulators (`splits` of rows x H each).
flce_status_t launch_dx_finalize(const float* acc, int splits, int64_t rows, int64_t H,
                                 const int32_t* idx, const int32_t* nvalid, int64_t r0, void* gh,
                                 bool f32, hipStream_t st) {
  const int64_t work = rows * (H / 4);
  const int fb = (int)(ceil_div(work, 256) < 16384 ? ceil_div(work, 256) : 16384);
  return launch(K_DX_FINALIZE, st, [&] {
    if (f32)
      dx_finalize_kernel<true><<<fb, 256, 0, st>>>(acc, splits, rows, H, idx, nvalid, r0, gh);
    else
      dx_finalize_kernel<false><<<fb, 256, 0, st>>>(acc, splits, rows, H, idx, nvalid, r0, gh);
  });
}

// The reduced outputs (reduced[k] may be null) from the nb combine blocks'
// sums; the mean divides by the valid count header[1], or with class weights
// by their sum in the header.
flce_status_t launch_fwd_reduce(const double4* bsum, int nb, const int32_t* header, bool mean,
                                bool weighted, float* const (&reduced)[4], hipStream_t st) {
  return launch(K_FWD_REDUCE, st, [&] {
    fwd_reduce_kernel<<<1, 256, 0, st>>>(bsum, nb, header, mean ? 1 : 0, weighted ? 1 : 0,
                                         reduced[0], reduced[1], reduced[2], reduced[3]);
  });
}

// Zero rows (row_bytes each) of `out` for ignored or invalid tokens.
flce_status_t launch_zero_ignored(const int64_t* labels, int64_t N, int64_t V_total,
                                  int64_t ignore_index, void* out, int64_t row_bytes,
                                  hipStream_t st) {
  const int zb = (int)(N < 16384 ? N : 16384);
  return launch(K_FILL, st, [&] {
    zero_ignored_rows_kernel<<<zb, 256, 0, st>>>(labels, N, V_total, ignore_index,
                                                 static_cast<char*>(out), row_bytes);
  });
}

}  // namespace

extern "C" {

flce_status_t flce_workspace_size(int64_t N, int64_t H, int64_t V, int reduction,
                                  size_t* fwd_bytes, size_t* bwd_bytes) {
  FLCE_TRY(check_shape(N, H, V));
  if (!valid_reduction(reduction)) return FLCE_ERR_BAD_REDUCTION;
  const Plan p = make_plan(N, H, V, reduction);
  if (fwd_bytes) *fwd_bytes = p.f_total;
  if (bwd_bytes) *bwd_bytes = p.b_total;
  return FLCE_OK;
}

}  // extern "C"

namespace {


// reduced[k] receives the reduction of output k (logprob, entropy,
// uniform_ce, z_loss); each may be null.
// V is the vocabulary of `weight` ([H,V]), the slice [v_begin, v_begin + V)
// of a vocabulary of V_total classes (V_total = V, v_begin = 0 unless
// sharded). With state_out set (a slice), the per-token merged state and the
// label logit (label_logit, 0 when the label lies elsewhere) are the outputs
// instead of the statistics.
flce_status_t forward_impl(const void* hidden, const void* weight, const int64_t* labels,
                           int64_t N, int64_t H, int64_t V, int64_t v_begin, int64_t V_total,
                           const flce_options_t& o, float* lse, float* logprob, float* entropy,
                           float* uniform_ce, float* z_loss, float* const (&reduced)[4],
                           float4* state_out, float* label_logit, void* workspace,
                           size_t workspace_bytes, void* stream) {
  const bool shard = state_out != nullptr;
  const int reduction = shard ? FLCE_REDUCTION_NONE : o.reduction;
  const bool reduce = reduction != FLCE_REDUCTION_NONE;
  if (workspace == nullptr) return FLCE_ERR_NULL_POINTER;
  if (N > 0 && (hidden == nullptr || weight == nullptr || labels == nullptr))
    return FLCE_ERR_NULL_POINTER;
  if (N > 0 && !shard && (lse == nullptr || logprob == nullptr || entropy == nullptr))
    return FLCE_ERR_NULL_POINTER;
  if (N > 0 && shard && label_logit == nullptr) return FLCE_ERR_NULL_POINTER;
  if (!aligned16(hidden) || !aligned16(weight) || !aligned16(workspace)) return FLCE_ERR_MISALIGNED;
  const Plan p = make_plan(N, H, V, reduction);
  if (workspace_bytes < p.f_total) return FLCE_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const float softcap = o.softcap;

  int32_t* header = reinterpret_cast<int32_t*>(workspace);
  const int32_t* nvalid = header + 1;
  int32_t* idx = reinterpret_cast<int32_t*>(wsp(workspace, p.f_idx));
  int32_t* labc = reinterpret_cast<int32_t*>(wsp(workspace, p.f_labc));
  float4* part = reinterpret_cast<float4*>(wsp(workspace, p.f_part));
  float* zlab = reinterpret_cast<float*>(wsp(workspace, p.f_zlab));
  double4* bsum = reduce ? reinterpret_cast<double4*>(wsp(workspace, p.f_bsum)) : nullptr;

  FwdPrepArgs pr{};
  pr.labels = labels;
  pr.N = N;
  pr.V_total = V_total;
  pr.v_begin = v_begin;
  pr.Vs = V;
  pr.ignore_index = o.ignore_index;
  pr.idx = idx;
  pr.labc = labc;
  pr.zlab = zlab;
  pr.lse = lse;
  pr.logprob = logprob;
  pr.entropy = entropy;
  pr.uniform_ce = uniform_ce;
  pr.z_loss = z_loss;
  pr.state_out = state_out;
  pr.label_logit = shard ? label_logit : nullptr;
  pr.header = header;
  const float* cw = reduce ? o.class_weight : nullptr;
  pr.cw = cw;
  FLCE_TRY(launch(K_FWD_PREP, st, [&] { fwd_prep_kernel<<<1, 1024, 0, st>>>(pr); }));
  const int nb = (int)ceil_div(N, kCombineTokens);
  if (N > 0) {
    uint16_t* xb = reinterpret_cast<uint16_t*>(wsp(workspace, p.f_xb));
    // Only the valid tokens, compacted in token order, enter the contractions.
    FLCE_TRY(pack_rows(K_PACK_HIDDEN, hidden, N, H, H, p.hkb, idx, nvalid, xb, st));
    // A vocabulary that is not a multiple of 8 is read from a copy whose rows
    // are 16-byte aligned (zero columns past V, masked like any tile tail).
    const void* wrd = weight;
    if (p.padw) {
      void* wp = wsp(workspace, p.f_wp);
      FLCE_TRY(pad_cols(weight, H, V, p.V8, wp, st));
      wrd = wp;
    }
    FwdTileArgs a{};
    a.weight = static_cast<const uint16_t*>(wrd);
    a.ldw = p.V8;
    a.xb = xb;
    a.lab = labc;
    a.nvalid = nvalid;
    a.N = N;
    a.H = H;
    a.V = V;
    a.hkb = p.hkb;
    a.VT = p.VT;
    a.TB = p.TB;
    a.tb0 = 0;
    a.group = p.group;
    a.cap = softcap > 0.f ? softcap : 0.f;
    a.cap_k = softcap > 0.f ? 2.f * kLog2e / softcap : 0.f;
    a.part = part;
    a.zlab = zlab;
    const int grid = p.TB * p.VT;
    FLCE_TRY(launch(K_FWD_TILE, st, [&] {
      if (softcap > 0.f)
        fwd_tile_kernel<true><<<grid, kThreads, 0, st>>>(a);
      else
        fwd_tile_kernel<false><<<grid, kThreads, 0, st>>>(a);
    }));
    CombineArgs c{};
    c.part = part;
    c.S = p.VT;
    c.zlab = zlab;
    c.nz = 1;
    c.idx = idx;
    c.nvalid = nvalid;
    c.N = N;
    c.V = V_total;
    c.state_out = state_out;
    c.label_logit = label_logit;
    c.zl_scale = o.z_loss_scale;
    c.lse = lse;
    c.logprob = logprob;
    c.entropy = entropy;
    c.uniform_ce = uniform_ce;
    c.z_loss = z_loss;
    c.bsum = bsum;
    c.labels = labels;
    c.cw = cw;
    FLCE_TRY(launch(K_FWD_COMBINE, st, [&] {
      fwd_combine_kernel<<<nb, 64 * kCombineWaves, 0, st>>>(c);
    }));
  }
  if (reduce)
    FLCE_TRY(launch_fwd_reduce(bsum, N > 0 ? nb : 0, header, reduction == FLCE_REDUCTION_MEAN,
                               cw != nullptr, reduced, st));
  return FLCE_OK;
}

// V, v_begin, V_total as for forward_impl.
flce_status_t backward_impl(const void* hidden, const void* weight, const int64_t* labels,
                            int64_t N, int64_t H, int64_t V, int64_t v_begin, int64_t V_total,
                            const flce_options_t& o,
                            const float* lse, const float* entropy, const float* grad_logprob,
                            const float* grad_entropy, const float* grad_uniform_ce,
                            const float* grad_z_loss, void* grad_hidden, void* grad_weight,
                            void* workspace, size_t workspace_bytes, void* stream) {
  const int reduction = o.reduction;
  const bool f32 = o.grad_dtype == FLCE_GRAD_F32;
  if (f32 && V > kMaxVF32) return FLCE_ERR_BAD_SHAPE;
  if (workspace == nullptr || weight == nullptr || grad_weight == nullptr)
    return FLCE_ERR_NULL_POINTER;
  if (N > 0 && (hidden == nullptr || labels == nullptr || lse == nullptr || entropy == nullptr ||
                grad_hidden == nullptr))
    return FLCE_ERR_NULL_POINTER;
  if (!aligned16(hidden) || !aligned16(weight) || !aligned16(grad_hidden) ||
      !aligned16(grad_weight) || !aligned16(workspace))
    return FLCE_ERR_MISALIGNED;
  const Plan p = make_plan(N, H, V, reduction);
  if (workspace_bytes < p.b_total) return FLCE_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const size_t out_elem = f32 ? 4 : 2;

  if (N == 0) return zero_fill(grad_weight, out_elem * (size_t)H * (size_t)V, st);

  int32_t* header = reinterpret_cast<int32_t*>(workspace);
  const int32_t* nvalid = header + 1;
  int32_t* lab32 = reinterpret_cast<int32_t*>(wsp(workspace, p.b_lab));
  int32_t* idx = reinterpret_cast<int32_t*>(wsp(workspace, p.b_idx));
  DzToken* coef = reinterpret_cast<DzToken*>(wsp(workspace, p.b_coef));
  uint16_t* wb = reinterpret_cast<uint16_t*>(wsp(workspace, p.b_wb));
  uint16_t* xb = reinterpret_cast<uint16_t*>(wsp(workspace, p.b_xb));
  uint16_t* xtb = reinterpret_cast<uint16_t*>(wsp(workspace, p.b_xtb));
  uint16_t* dtv = reinterpret_cast<uint16_t*>(wsp(workspace, p.b_dtv));
  uint16_t* dvt = reinterpret_cast<uint16_t*>(wsp(workspace, p.b_dvt));
  float* acc = reinterpret_cast<float*>(wsp(workspace, p.b_acc));
  float* part = reinterpret_cast<float*>(wsp(workspace, p.b_part));

  PrepArgs pa{};
  pa.labels = labels;
  pa.N = N;
  pa.V = V_total;
  pa.ignore_index = o.ignore_index;
  pa.v_begin = v_begin;
  pa.Vs = V;
  pa.reduction = reduction;
  pa.zl_scale = o.z_loss_scale;
  pa.lse = lse;
  pa.entropy = entropy;
  pa.glp = grad_logprob;
  pa.gent = grad_entropy;
  pa.guce = grad_uniform_ce;
  pa.gzl = grad_z_loss;
  pa.coef = coef;
  pa.lab32 = lab32;
  pa.idx = idx;
  pa.header = header;
  pa.cw = reduction != FLCE_REDUCTION_NONE ? o.class_weight : nullptr;
  pa.ent_tok = o.entropy_per_token;
  FLCE_TRY(launch(K_BWD_PREP, st, [&] { bwd_prep_kernel<<<1, 1024, 0, st>>>(pa); }));
  // Rows of ignored tokens are never written by the compacted contractions.
  FLCE_TRY(launch_zero_ignored(labels, N, V_total, o.ignore_index, grad_hidden,
                               (int64_t)out_elem * H, st));

  // Blocked operands, over the valid tokens compacted in token order: hidden
  // (tokens x H) for the recompute, hidden^T (H x tokens) for dW, and per
  // chunk the weight (H x vocabulary) for dH. The recompute reads the weight
  // (vocabulary x H) row-contiguous.
  FLCE_TRY(pack_rows(K_PACK_HIDDEN, hidden, N, H, H, p.hkb, idx, nvalid, xb, st));
  FLCE_TRY(pack_cols(K_PACK_HIDDEN, hidden, H, N, H, p.nkb, idx, nvalid, xtb, st));
  const float softcap = o.softcap;
  const bool capped = softcap > 0.f;
  // A vocabulary that is not a multiple of 8: the weight is read from a copy
  // with 16-byte aligned rows of V8 columns (zero past V) and dW is formed in
  // a buffer of the same row stride, copied out at the end.
  const uint16_t* wrd = static_cast<const uint16_t*>(weight);
  void* gw_out = grad_weight;
  if (p.padw) {
    uint16_t* wp = reinterpret_cast<uint16_t*>(wsp(workspace, p.b_wp));
    FLCE_TRY(pad_cols(weight, H, V, p.V8, wp, st));
    wrd = wp;
    gw_out = wsp(workspace, p.b_gwp);
  }
  for (int c = 0; c < p.nchunks; ++c) {
    const int64_t v0 = (int64_t)c * p.Vc;
    const int64_t vc = V - v0 < p.Vc ? V - v0 : p.Vc;
    const int vtc = (int)ceil_div(vc, kTile);

    // bwd_dlogits also writes the chunk's weight image for dH (wimg).
    DlogitsArgs d{};
    d.weight = wrd;
    d.ldw = p.V8;
    d.xb = xb;
    d.coef = coef;
    d.lab = lab32;
    d.nvalid = nvalid;
    d.N = N;
    d.H = H;
    d.V = V;
    d.hkb = p.hkb;
    d.v0 = v0;
    d.VTc = vtc;
    d.TB = p.TB;
    d.group = p.group;
    d.kbv = p.kbv;
    d.kbn = p.nkb;
    d.cap = capped ? softcap : 0.f;
    d.cap_k = capped ? 2.f * kLog2e / softcap : 0.f;
    d.inv_cap = capped ? 1.f / softcap : 0.f;
    d.dtv = dtv;
    d.dvt = dvt;
    d.wimg = wb;
    FLCE_TRY(launch(K_BWD_DLOGITS, st, [&] {
      if (capped)
        bwd_dlogits_kernel<true><<<vtc * p.TB, kThreads, 0, st>>>(d);
      else
        bwd_dlogits_kernel<false><<<vtc * p.TB, kThreads, 0, st>>>(d);
    }));

    DxArgs x{};
    x.dtv = dtv;
    x.wb = wb;
    x.N = N;
    x.H = H;
    x.V = V;
    x.kbv = p.kbv;
    x.nk = vtc * (kTile / kBK);
    x.TB = p.TB;
    x.HT = p.HT;
    x.group = p.group;
    x.acc = acc;
    x.gh = grad_hidden;
    x.idx = idx;
    x.nvalid = nvalid;
    x.splits = p.dx_splits;
    x.r0 = 0;
    // With K splits every split accumulates (first chunk stores, later ones
    // add) and dx_finalize writes the output after the last chunk.
    const bool split = p.dx_splits > 1;
    const int mode = split ? (c == 0 ? DX_FIRST : DX_MID)
                           : (p.nchunks == 1 ? DX_ONLY
                                             : (c == 0 ? DX_FIRST
                                                       : (c == p.nchunks - 1 ? DX_LAST : DX_MID)));
    const int gx = p.TB * p.HT * p.dx_splits;

    DwArgs w{};
    w.xtb = xtb;
    w.dvt = dvt;
    w.N = N;
    w.H = H;
    w.V = V;
    w.v0 = v0;
    w.vc = vc;
    w.kbn = p.nkb;
    w.kbn_a = p.nkb;
    w.ka0 = 0;
    w.r0 = 0;
    w.nvalid = nvalid;
    w.ldp = p.Vc;
    w.HT = p.HT;
    w.VTc = vtc;
    w.splits = p.dw_splits;
    w.group = p.group;
    w.kper = p.dw_kper;
    w.gw = gw_out;
    w.ldo = p.V8;
    w.part = part;
    const int gw = p.HT * vtc * p.dw_splits;
    if (combine_dxdw(p, x.nk, gx, gw)) {
      FLCE_TRY(launch_dxdw(x, w, mode, f32, gx + gw, st));
    } else {
      FLCE_TRY(launch_dx(x, mode, f32, gx, st));
      FLCE_TRY(launch(K_BWD_DW, st, [&] {
        if (p.dw_splits > 1)
          bwd_dw_kernel<DW_SPLIT, false><<<gw, kThreads, 0, st>>>(w);
        else if (f32)
          bwd_dw_kernel<DW_DIRECT, true><<<gw, kThreads, 0, st>>>(w);
        else
          bwd_dw_kernel<DW_DIRECT, false><<<gw, kThreads, 0, st>>>(w);
      }));
    }
    if (split && c == p.nchunks - 1)
      FLCE_TRY(launch_dx_finalize(acc, p.dx_splits, N, H, idx, nvalid, 0, grad_hidden, f32, st));
    if (p.dw_splits > 1) {
      const int64_t n = H * vc;
      const int blocks = (int)(ceil_div(n, 256) < 8192 ? ceil_div(n, 256) : 8192);
      FLCE_TRY(launch(K_DW_REDUCE, st, [&] {
        if (f32)
          dw_reduce_kernel<true><<<blocks, 256, 0, st>>>(part, p.dw_splits, H, vc, p.Vc, p.V8,
                                                         v0, gw_out);
        else
          dw_reduce_kernel<false><<<blocks, 256, 0, st>>>(part, p.dw_splits, H, vc, p.Vc, p.V8,
                                                          v0, gw_out);
      }));
    }
  }
  if (p.padw) FLCE_TRY(unpad_cols(gw_out, H, p.V8, V, grad_weight, f32, st));
  return FLCE_OK;
}

// The fused forward + backward (gradient in the forward): the outputs of
// forward_impl and the gradients of backward_impl in one pass over the
// logits per chunk of tokens, without the backward's recompute.
flce_status_t fused_impl(const void* hidden, const void* weight, const int64_t* labels, int64_t N,
                         int64_t H, int64_t V, const flce_options_t& o, int64_t chunk_tokens,
                         const float* grad_logprob, const float* grad_entropy,
                         const float* grad_uniform_ce, const float* grad_z_loss, float* lse,
                         float* logprob, float* entropy, float* uniform_ce, float* z_loss,
                         float* reduced, void* grad_hidden, void* grad_weight, void* workspace,
                         size_t workspace_bytes, void* stream) {
  const int reduction = o.reduction;
  const bool reduce = reduction != FLCE_REDUCTION_NONE;
  const bool f32 = o.grad_dtype == FLCE_GRAD_F32;
  if (V > kMaxVF32) return FLCE_ERR_BAD_SHAPE;
  if (chunk_tokens < 0) return FLCE_ERR_BAD_SHAPE;
  if (workspace == nullptr || weight == nullptr || grad_weight == nullptr)
    return FLCE_ERR_NULL_POINTER;
  if (reduce && reduced == nullptr) return FLCE_ERR_NULL_POINTER;
  if (N > 0 && (hidden == nullptr || labels == nullptr || lse == nullptr || logprob == nullptr ||
                entropy == nullptr || grad_hidden == nullptr))
    return FLCE_ERR_NULL_POINTER;
  if (!aligned16(hidden) || !aligned16(weight) || !aligned16(grad_hidden) ||
      !aligned16(grad_weight) || !aligned16(workspace))
    return FLCE_ERR_MISALIGNED;
  const FusedPlan f = make_fused_plan(N, H, V, o, chunk_tokens);
  const Plan& p = f.b;
  if (workspace_bytes < f.total) return FLCE_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const size_t out_elem = f32 ? 4 : 2;
  const float softcap = o.softcap;
  const bool capped = softcap > 0.f;

  int32_t* header = reinterpret_cast<int32_t*>(workspace);
  const int32_t* nvalid = header + 1;
  int32_t* idx = reinterpret_cast<int32_t*>(wsp(workspace, f.idx));
  int32_t* labc = reinterpret_cast<int32_t*>(wsp(workspace, f.labc));
  float* zlab = reinterpret_cast<float*>(wsp(workspace, f.zlab));
  float4* part = reinterpret_cast<float4*>(wsp(workspace, f.part));
  double4* bsum = reduce ? reinterpret_cast<double4*>(wsp(workspace, f.bsum)) : nullptr;
  DzToken* coef = reinterpret_cast<DzToken*>(wsp(workspace, f.coef));
  uint16_t* xb = reinterpret_cast<uint16_t*>(wsp(workspace, f.xb));
  uint16_t* xtb = reinterpret_cast<uint16_t*>(wsp(workspace, f.xtb));
  uint16_t* wb = reinterpret_cast<uint16_t*>(wsp(workspace, f.wb));
  uint16_t* dtv = reinterpret_cast<uint16_t*>(wsp(workspace, f.dtv));
  uint16_t* dvt = reinterpret_cast<uint16_t*>(wsp(workspace, f.dvt));
  float* mref = reinterpret_cast<float*>(wsp(workspace, f.mref));
  float* dxacc = reinterpret_cast<float*>(wsp(workspace, f.dxacc));
  // dW goes to grad_weight, or with a vocabulary that is not a multiple of 8
  // to a padded buffer copied out at the end (the weight is then read from a
  // padded copy).
  void* gw_out = p.padw ? static_cast<void*>(wsp(workspace, f.gwp)) : grad_weight;
  float* dwacc = f32 ? static_cast<float*>(gw_out)
                     : reinterpret_cast<float*>(wsp(workspace, f.dwacc));

  FwdPrepArgs pr{};
  pr.labels = labels;
  pr.N = N;
  pr.V_total = V;
  pr.v_begin = 0;
  pr.Vs = V;
  pr.ignore_index = o.ignore_index;
  pr.idx = idx;
  pr.labc = labc;
  pr.zlab = zlab;
  pr.lse = lse;
  pr.logprob = logprob;
  pr.entropy = entropy;
  pr.uniform_ce = uniform_ce;
  pr.z_loss = z_loss;
  pr.header = header;
  const float* cw = reduce ? o.class_weight : nullptr;
  pr.cw = cw;
  FLCE_TRY(launch(K_FWD_PREP, st, [&] { fwd_prep_kernel<<<1, 1024, 0, st>>>(pr); }));
  const int nb = p.TB * (kTile / kCombineTokens);
  if (N == 0) {
    FLCE_TRY(zero_fill(grad_weight, out_elem * (size_t)H * (size_t)V, st));
  } else {
    FLCE_TRY(launch_zero_ignored(labels, N, V, o.ignore_index, grad_hidden,
                                 (int64_t)out_elem * H, st));
    // Blocked operands over the valid tokens compacted in token order: hidden
    // (K = H) for the logit tiles, hidden^T (K = tokens) for dW, and the
    // weight (H rows, K = vocabulary) for dH.
    FLCE_TRY(pack_rows(K_PACK_HIDDEN, hidden, N, H, H, p.hkb, idx, nvalid, xb, st));
    FLCE_TRY(pack_cols(K_PACK_HIDDEN, hidden, H, N, H, p.nkb, idx, nvalid, xtb, st));
    const uint16_t* wrd = static_cast<const uint16_t*>(weight);
    if (p.padw) {
      uint16_t* wp = reinterpret_cast<uint16_t*>(wsp(workspace, f.wp));
      FLCE_TRY(pad_cols(weight, H, V, p.V8, wp, st));
      wrd = wp;
    }
    // The weight image for dH (wb) is written by the first chunk's logit tiles.
    const int64_t mld = (int64_t)f.TBc * kTile;
    for (int c = 0; c < f.nchunks; ++c) {
      const int tb0 = c * f.TBc;
      const int tbc = p.TB - tb0 < f.TBc ? p.TB - tb0 : f.TBc;
      const int r0 = tb0 * kTile;
      const int64_t rows = (int64_t)tbc * kTile;

      FwdTileArgs a{};
      a.weight = wrd;
      a.ldw = p.V8;
      a.xb = xb;
      a.lab = labc;
      a.nvalid = nvalid;
      a.N = N;
      a.H = H;
      a.V = V;
      a.hkb = p.hkb;
      a.VT = p.VT;
      a.TB = tbc;
      a.tb0 = tb0;
      a.group = p.group;
      a.cap = capped ? softcap : 0.f;
      a.cap_k = capped ? 2.f * kLog2e / softcap : 0.f;
      a.part = part;
      a.zlab = zlab;
      a.dz = dtv;
      a.kbv = f.kbv;
      a.mref = mref;
      a.mld = mld;
      a.wimg = c == 0 ? wb : nullptr;
      FLCE_TRY(launch(K_FUSED_TILE, st, [&] {
        if (capped)
          fused_tile_kernel<true><<<tbc * p.VT, kThreads, 0, st>>>(a);
        else
          fused_tile_kernel<false><<<tbc * p.VT, kThreads, 0, st>>>(a);
      }));

      CombineArgs cb{};
      cb.part = part;
      cb.S = p.VT;
      cb.zlab = zlab;
      cb.nz = 1;
      cb.idx = idx;
      cb.nvalid = nvalid;
      cb.N = N;
      cb.V = V;
      cb.zl_scale = o.z_loss_scale;
      cb.lse = lse;
      cb.logprob = logprob;
      cb.entropy = entropy;
      cb.uniform_ce = uniform_ce;
      cb.z_loss = z_loss;
      cb.bsum = bsum;
      cb.r0 = r0;
      cb.coef = coef;
      cb.glp = grad_logprob;
      cb.gent = grad_entropy;
      cb.guce = grad_uniform_ce;
      cb.gzl = grad_z_loss;
      cb.reduction = reduction;
      cb.ent_tok = o.entropy_per_token;
      cb.header = header;
      cb.labels = labels;
      cb.cw = cw;
      FLCE_TRY(launch(K_FWD_COMBINE, st, [&] {
        fwd_combine_kernel<<<(int)(rows / kCombineTokens), 64 * kCombineWaves, 0, st>>>(cb);
      }));

      FusedDzArgs d{};
      d.dtv = dtv;
      d.dvt = dvt;
      d.mref = mref;
      d.mld = mld;
      d.coef = coef + r0;
      d.lab = labc + r0;
      d.nvalid = nvalid;
      d.r0 = r0;
      d.rows = N - r0 < rows ? N - r0 : rows;  // rows with coefficients and label codes
      d.V = V;
      d.VT = p.VT;
      d.TB = tbc;
      d.group = p.group;
      d.kbv = f.kbv;
      d.kbn = tbc * (kTile / kBK);
      d.cap = capped ? softcap : 0.f;
      d.inv_cap = capped ? 1.f / softcap : 0.f;
      FLCE_TRY(launch(K_FUSED_DLOGITS, st, [&] {
        if (capped)
          fused_dlogits_kernel<true><<<2 * tbc * p.VT, kDzThreads, 0, st>>>(d);
        else
          fused_dlogits_kernel<false><<<2 * tbc * p.VT, kDzThreads, 0, st>>>(d);
      }));

      DxArgs x{};
      x.dtv = dtv;
      x.wb = wb;
      x.N = rows;
      x.H = H;
      x.V = V;
      x.kbv = f.kbv;
      x.nk = f.kbv;
      x.TB = tbc;
      x.HT = p.HT;
      x.group = p.group;
      x.acc = dxacc;
      x.gh = grad_hidden;
      x.idx = idx + r0;
      x.nvalid = nvalid;
      x.splits = f.dx_splits;
      x.r0 = r0;
      // One vocabulary range per chunk: the output directly, or K-split
      // accumulators and their sum.
      const bool split = f.dx_splits > 1;
      FLCE_TRY(launch_dx(x, split ? DX_FIRST : DX_ONLY, f32, tbc * p.HT * f.dx_splits, st));
      if (split)
        FLCE_TRY(launch_dx_finalize(dxacc, f.dx_splits, rows, H, idx + r0, nvalid, r0,
                                    grad_hidden, f32, st));

      DwArgs w{};
      w.xtb = xtb;
      w.dvt = dvt;
      w.N = N;
      w.H = H;
      w.V = V;
      w.v0 = 0;
      w.vc = V;
      w.kbn = tbc * (kTile / kBK);
      w.kbn_a = p.nkb;
      w.ka0 = tb0 * (kTile / kBK);
      w.nvalid = nvalid;
      w.r0 = r0;
      w.HT = p.HT;
      w.VTc = p.VT;
      w.splits = 1;
      w.group = p.group;
      w.kper = w.kbn;
      w.ldp = 0;
      w.gw = gw_out;
      w.ldo = p.V8;
      w.part = nullptr;
      w.accw = dwacc;
      w.rows = rows;
      w.first = c == 0;
      // The chunk holding the last valid token writes dW; earlier chunks
      // accumulate it in fp32 (in grad_weight itself when that is fp32);
      // later, empty chunks exit. Decided on the device from the valid count.
      const int gw = p.HT * p.VT;
      FLCE_TRY(launch(K_BWD_DW, st, [&] {
        if (f32)
          bwd_dw_kernel<DW_CHUNK, true><<<gw, kThreads, 0, st>>>(w);
        else
          bwd_dw_kernel<DW_CHUNK, false><<<gw, kThreads, 0, st>>>(w);
      }));
    }
    if (p.padw) FLCE_TRY(unpad_cols(gw_out, H, p.V8, V, grad_weight, f32, st));
  }
  if (reduce) {
    float* const red[4] = {reduced, reduced + 1, reduced + 2, reduced + 3};
    FLCE_TRY(launch_fwd_reduce(bsum, N > 0 ? nb : 0, header, reduction == FLCE_REDUCTION_MEAN,
                               cw != nullptr, red, st));
  }
  return FLCE_OK;
}

}  // namespace

extern "C" {

flce_status_t flce_forward(const void* hidden, const void* weight, const int64_t* labels,
                           int64_t N, int64_t H, int64_t V, int64_t ignore_index,
                           float softcap, int reduction, float* lse, float* logprob,
                           float* entropy, float* logprob_mean, float* entropy_mean,
                           void* workspace, size_t workspace_bytes, void* stream) {
  FLCE_TRY(check_shape(N, H, V));
  const flce_options_t o{ignore_index, softcap, reduction, 0.f, FLCE_GRAD_BF16, nullptr};
  FLCE_TRY(check_options(&o));
  if (reduction != FLCE_REDUCTION_NONE && (logprob_mean == nullptr || entropy_mean == nullptr))
    return FLCE_ERR_NULL_POINTER;
  float* const red[4] = {logprob_mean, entropy_mean, nullptr, nullptr};
  return forward_impl(hidden, weight, labels, N, H, V, 0, V, o, lse, logprob, entropy, nullptr,
                      nullptr, red, nullptr, nullptr, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

// The no-allocation forward's scratch: one array per device that the library
// runs on, held until the process ends. In host code `noalloc_scratch` names
// a host-side stand-in, not device memory: only the per-device address that
// hipGetSymbolAddress returns is ever handed to kernels.
constexpr size_t kNoallocScratchBytes = (size_t)FLCE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char noalloc_scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex noalloc_mu;
void* noalloc_ptr[kMaxDevices] = {};

// The current device's copy of the scratch array (looked up once per device,
// with that device current).
flce_status_t noalloc_scratch_ptr(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FLCE_ERR_HIP;
  std::lock_guard<std::mutex> lock(noalloc_mu);
  if (noalloc_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(noalloc_scratch)) != hipSuccess || p == nullptr)
      return FLCE_ERR_HIP;
    noalloc_ptr[dev] = p;
  }
  *out = noalloc_ptr[dev];
  return FLCE_OK;
}

}  // namespace

extern "C" {

flce_status_t flce_forward_noalloc(const void* hidden, const void* weight, const int64_t* labels,
                                   int64_t N, int64_t H, int64_t V, int64_t ignore_index,
                                   float softcap, int reduction, float* lse, float* logprob,
                                   float* entropy, float* logprob_mean, float* entropy_mean,
                                   void* stream) {
  FLCE_TRY(check_shape(N, H, V));
  const flce_options_t o{ignore_index, softcap, reduction, 0.f, FLCE_GRAD_BF16, nullptr};
  FLCE_TRY(check_options(&o));
  if (make_plan(N, H, V, reduction).f_total > kNoallocScratchBytes) return FLCE_ERR_TOO_LARGE;
  void* scratch = nullptr;
  FLCE_TRY(noalloc_scratch_ptr(&scratch));
  return flce_forward(hidden, weight, labels, N, H, V, ignore_index, softcap, reduction, lse,
                      logprob, entropy, logprob_mean, entropy_mean, scratch,
                      kNoallocScratchBytes, stream);
}

flce_status_t flce_forward_ex(const void* hidden, const void* weight, const int64_t* labels,
                              int64_t N, int64_t H, int64_t V, const flce_options_t* opt,
                              float* lse, float* logprob, float* entropy, float* uniform_ce,
                              float* z_loss, float* reduced, void* workspace,
                              size_t workspace_bytes, void* stream) {
  FLCE_TRY(check_shape(N, H, V));
  FLCE_TRY(check_options(opt));
  if (opt->reduction != FLCE_REDUCTION_NONE && reduced == nullptr) return FLCE_ERR_NULL_POINTER;
  float* const red[4] = {reduced, reduced ? reduced + 1 : nullptr, reduced ? reduced + 2 : nullptr,
                         reduced ? reduced + 3 : nullptr};
  return forward_impl(hidden, weight, labels, N, H, V, 0, V, *opt, lse, logprob, entropy,
                      uniform_ce, z_loss, red, nullptr, nullptr, workspace, workspace_bytes,
                      stream);
}

flce_status_t flce_backward(const void* hidden, const void* weight, const int64_t* labels,
                            int64_t N, int64_t H, int64_t V, int64_t ignore_index,
                            float softcap, int reduction, const float* lse,
                            const float* entropy, const float* grad_logprob,
                            const float* grad_entropy, void* grad_hidden, void* grad_weight,
                            void* workspace, size_t workspace_bytes, void* stream) {
  FLCE_TRY(check_shape(N, H, V));
  const flce_options_t o{ignore_index, softcap, reduction, 0.f, FLCE_GRAD_BF16, nullptr};
  FLCE_TRY(check_options(&o));
  return backward_impl(hidden, weight, labels, N, H, V, 0, V, o, lse, entropy, grad_logprob,
                       grad_entropy, nullptr, nullptr, grad_hidden, grad_weight, workspace,
                       workspace_bytes, stream);
}

flce_status_t flce_backward_ex(const void* hidden, const void* weight, const int64_t* labels,
                               int64_t N, int64_t H, int64_t V, const flce_options_t* opt,
                               const float* lse, const float* entropy,
                               const float* grad_logprob, const float* grad_entropy,
                               const float* grad_uniform_ce, const float* grad_z_loss,
                               void* grad_hidden, void* grad_weight, void* workspace,
                               size_t workspace_bytes, void* stream) {
  FLCE_TRY(check_shape(N, H, V));
  FLCE_TRY(check_options(opt));
  return backward_impl(hidden, weight, labels, N, H, V, 0, V, *opt, lse, entropy, grad_logprob,
                       grad_entropy, grad_uniform_ce, grad_z_loss, grad_hidden, grad_weight,
                       workspace, workspace_bytes, stream);
}

// ---- fused forward + backward ------------------------------------------------------

flce_status_t flce_fused_workspace_size(int64_t N, int64_t H, int64_t V, const flce_options_t* opt,
                                        int64_t chunk_tokens, size_t* bytes) {
  FLCE_TRY(check_shape(N, H, V));
  FLCE_TRY(check_options(opt));
  if (V > kMaxVF32 || chunk_tokens < 0) return FLCE_ERR_BAD_SHAPE;
  if (bytes) *bytes = make_fused_plan(N, H, V, *opt, chunk_tokens).total;
  return FLCE_OK;
}

flce_status_t flce_forward_backward(const void* hidden, const void* weight, const int64_t* labels,
                                    int64_t N, int64_t H, int64_t V, const flce_options_t* opt,
                                    int64_t chunk_tokens, const float* grad_logprob,
                                    const float* grad_entropy, const float* grad_uniform_ce,
                                    const float* grad_z_loss, float* lse, float* logprob,
                                    float* entropy, float* uniform_ce, float* z_loss,
                                    float* reduced, void* grad_hidden, void* grad_weight,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  FLCE_TRY(check_shape(N, H, V));
  FLCE_TRY(check_options(opt));
  return fused_impl(hidden, weight, labels, N, H, V, *opt, chunk_tokens, grad_logprob,
                    grad_entropy, grad_uniform_ce, grad_z_loss, lse, logprob, entropy, uniform_ce,
                    z_loss, reduced, grad_hidden, grad_weight, workspace, workspace_bytes, stream);
}

// ---- vocabulary-sharded head ---------------------------------------------------

static flce_status_t check_slice(int64_t Vs, int64_t v_begin, int64_t V_total) {
  if (v_begin < 0 || V_total < 1 || V_total > kMaxV || v_begin + Vs > V_total)
    return FLCE_ERR_BAD_SHAPE;
  return FLCE_OK;
}

flce_status_t flce_forward_shard(const void* hidden, const void* weight_shard,
                                 const int64_t* labels, int64_t N, int64_t H, int64_t Vs,
                                 int64_t v_begin, int64_t V_total, const flce_options_t* opt,
                                 float* state, float* label_logit, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  FLCE_TRY(check_shape(N, H, Vs));
  FLCE_TRY(check_slice(Vs, v_begin, V_total));
  FLCE_TRY(check_options(opt));
  if (N > 0 && state == nullptr) return FLCE_ERR_NULL_POINTER;
  if (state != nullptr && !aligned16(state)) return FLCE_ERR_MISALIGNED;
  float* const red[4] = {nullptr, nullptr, nullptr, nullptr};
  flce_options_t o = *opt;
  o.reduction = FLCE_REDUCTION_NONE;
  // A non-null state pointer selects the slice outputs, also for N = 0.
  float4* st4 = reinterpret_cast<float4*>(state != nullptr ? state : workspace);
  return forward_impl(hidden, weight_shard, labels, N, H, Vs, v_begin, V_total, o, nullptr,
                      nullptr, nullptr, nullptr, nullptr, red, st4, label_logit, workspace,
                      workspace_bytes, stream);
}

flce_status_t flce_merge_workspace_size(int64_t N, size_t* bytes) {
  if (N < 0 || N > kMaxN) return FLCE_ERR_BAD_SHAPE;
  if (bytes) *bytes = merge_bytes(N);
  return FLCE_OK;
}

flce_status_t flce_merge_shards(const float* states, const float* label_logits, int64_t S,
                                const int64_t* labels, int64_t N, int64_t V_total,
                                const flce_options_t* opt, float* lse, float* logprob,
                                float* entropy, float* uniform_ce, float* z_loss, float* reduced,
                                void* workspace, size_t workspace_bytes, void* stream) {
  if (N < 0 || N > kMaxN || S < 1 || S > (int64_t)1 << 16 || V_total < 1 || V_total > kMaxV)
    return FLCE_ERR_BAD_SHAPE;
  FLCE_TRY(check_options(opt));
  const bool reduce = opt->reduction != FLCE_REDUCTION_NONE;
  if (workspace == nullptr) return FLCE_ERR_NULL_POINTER;
  if (reduce && reduced == nullptr) return FLCE_ERR_NULL_POINTER;
  if (N > 0 && (states == nullptr || label_logits == nullptr || labels == nullptr ||
                lse == nullptr || logprob == nullptr || entropy == nullptr))
    return FLCE_ERR_NULL_POINTER;
  if (!aligned16(states) || !aligned16(workspace)) return FLCE_ERR_MISALIGNED;
  if (workspace_bytes < merge_bytes(N)) return FLCE_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  int32_t* header = reinterpret_cast<int32_t*>(workspace);
  double4* bsum = reduce ? reinterpret_cast<double4*>(wsp(workspace, merge_bsum_off(N))) : nullptr;
  // The prep kernel counts the valid tokens for the mean (its compaction is
  // unused here: the slice states are indexed by token).
  FwdPrepArgs pr{};
  pr.labels = labels;
  pr.N = N;
  pr.V_total = V_total;
  pr.v_begin = 0;
  pr.Vs = V_total;
  pr.ignore_index = opt->ignore_index;
  pr.idx = reinterpret_cast<int32_t*>(wsp(workspace, merge_idx_off(N)));
  pr.labc = reinterpret_cast<int32_t*>(wsp(workspace, merge_labc_off(N)));
  pr.zlab = reinterpret_cast<float*>(wsp(workspace, merge_zlab_off(N)));
  pr.header = header;
  const float* cw = reduce ? opt->class_weight : nullptr;
  pr.cw = cw;
  FLCE_TRY(launch(K_FWD_PREP, st, [&] { fwd_prep_kernel<<<1, 1024, 0, st>>>(pr); }));
  const int nb = (int)ceil_div(N, kCombineTokens);
  if (N > 0) {
    CombineArgs c{};
    c.part = reinterpret_cast<const float4*>(states);
    c.S = (int)S;
    c.zlab = label_logits;
    c.nz = (int)S;
    c.idx = nullptr;
    c.labels = labels;
    c.ignore_index = opt->ignore_index;
    c.N = N;
    c.V = V_total;
    c.zl_scale = opt->z_loss_scale;
    c.lse = lse;
    c.logprob = logprob;
    c.entropy = entropy;
    c.uniform_ce = uniform_ce;
    c.z_loss = z_loss;
    c.bsum = bsum;
    c.cw = cw;
    FLCE_TRY(launch(K_FWD_COMBINE, st, [&] {
      fwd_combine_kernel<<<nb, 64 * kCombineWaves, 0, st>>>(c);
    }));
  }
  if (reduce) {
    float* const red[4] = {reduced, reduced ? reduced + 1 : nullptr,
                           reduced ? reduced + 2 : nullptr, reduced ? reduced + 3 : nullptr};
    FLCE_TRY(launch_fwd_reduce(bsum, N > 0 ? nb : 0, header,
                               opt->reduction == FLCE_REDUCTION_MEAN, cw != nullptr, red, st));
  }
  return FLCE_OK;
}

flce_status_t flce_backward_shard(const void* hidden, const void* weight_shard,
                                  const int64_t* labels, int64_t N, int64_t H, int64_t Vs,
                                  int64_t v_begin, int64_t V_total, const flce_options_t* opt,
                                  const float* lse, const float* entropy,
                                  const float* grad_logprob, const float* grad_entropy,
                                  const float* grad_uniform_ce, const float* grad_z_loss,
                                  void* grad_hidden_partial, void* grad_weight_shard,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  FLCE_TRY(check_shape(N, H, Vs));
  FLCE_TRY(check_slice(Vs, v_begin, V_total));
  FLCE_TRY(check_options(opt));
  return backward_impl(hidden, weight_shard, labels, N, H, Vs, v_begin, V_total, *opt, lse,
                       entropy, grad_logprob, grad_entropy, grad_uniform_ce, grad_z_loss,
                       grad_hidden_partial, grad_weight_shard, workspace, workspace_bytes,
                       stream);
}

flce_status_t flce_get_status(const void* workspace, int64_t* invalid_labels, void* stream) {
  if (workspace == nullptr) return FLCE_ERR_NULL_POINTER;
  hipStream_t st = static_cast<hipStream_t>(stream);
  int32_t h[2] = {0, 0};
  if (hipMemcpyAsync(h, workspace, sizeof(h), hipMemcpyDeviceToHost, st) != hipSuccess)
    return FLCE_ERR_HIP;
  if (hipStreamSynchronize(st) != hipSuccess) return FLCE_ERR_HIP;
  if (invalid_labels) *invalid_labels = h[0];
  return h[0] != 0 ? FLCE_ERR_INVALID_LABEL : FLCE_OK;
}

const char* flce_status_string(flce_status_t s) {
  switch (s) {
    case FLCE_OK: return "ok";
    case FLCE_ERR_NULL_POINTER: return "a required pointer is NULL";
    case FLCE_ERR_BAD_SHAPE: return "bad shape (need N >= 0, H >= 1, V >= 1 within limits)";
    case FLCE_ERR_BAD_REDUCTION: return "reduction must be NONE (0), MEAN (1) or SUM (2)";
    case FLCE_ERR_MISALIGNED:
      return "pointers must be 16-byte aligned and H a multiple of 8";
    case FLCE_ERR_WORKSPACE_TOO_SMALL: return "workspace smaller than flce_workspace_size";
    case FLCE_ERR_BAD_SOFTCAP: return "softcap must be finite";
    case FLCE_ERR_HIP: return "HIP runtime error or failed kernel launch";
    case FLCE_ERR_INVALID_LABEL: return "labels outside [0, V) that are not ignore_index";
    case FLCE_ERR_BAD_OPTION:
      return "z_loss_scale must be finite and >= 0; grad_dtype BF16 or F32; class_weight needs "
             "MEAN or SUM; entropy_per_token 0 or 1";
    case FLCE_ERR_TOO_LARGE:
      return "the call needs more scratch than flce_forward_noalloc's static buffer "
             "(FLCE_NOALLOC_SCRATCH_BYTES) holds; use flce_forward with a workspace";
  }
  return "unknown status";
}

int flce_version(void) { return 212; }

flce_status_t flce_probe_mfma_rate(int mode, int64_t steps, double* tflops, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  if (tflops == nullptr || workspace == nullptr) return FLCE_ERR_NULL_POINTER;
  if (mode < 0 || mode > 3) return FLCE_ERR_BAD_OPTION;
  if (steps < 4 || steps > ((int64_t)1 << 24)) return FLCE_ERR_BAD_SHAPE;
  const int blocks = kNumCUs;
  const size_t out_bytes = (size_t)blocks * kThreads * 4;
  const size_t win_bytes = (size_t)2 << 20;  // the DMA source window of mode 3
  if (workspace_bytes < out_bytes + (mode == 3 ? win_bytes : 0)) return FLCE_ERR_WORKSPACE_TOO_SMALL;
  if (!aligned16(workspace)) return FLCE_ERR_MISALIGNED;
  hipStream_t st = static_cast<hipStream_t>(stream);
  float* out = static_cast<float*>(workspace);
  uint16_t* win = reinterpret_cast<uint16_t*>(wsp(workspace, out_bytes));
  if (mode == 3) {
    probe_fill_kernel<<<1024, 256, 0, st>>>(win, (int64_t)(win_bytes / 2));
    if (hipGetLastError() != hipSuccess) return FLCE_ERR_HIP;
  }
  const int n = (int)(steps / 4 * 4);
  hipEvent_t a = nullptr, b = nullptr;
  if (hipEventCreate(&a) != hipSuccess) return FLCE_ERR_HIP;
  if (hipEventCreate(&b) != hipSuccess) {
    (void)hipEventDestroy(a);
    return FLCE_ERR_HIP;
  }
  float ms = 0.f;
  bool ok = hipEventRecord(a, st) == hipSuccess;
  if (ok) {
    switch (mode) {
      case 0: mfma_probe_kernel<0><<<blocks, kThreads, 0, st>>>(n, 0, out, win); break;
      case 1: mfma_probe_kernel<0><<<blocks, kThreads, 0, st>>>(n, 1, out, win); break;
      case 2: mfma_probe_kernel<2><<<blocks, kThreads, 0, st>>>(n, 0, out, win); break;
      default: mfma_probe_kernel<3><<<blocks, kThreads, 0, st>>>(n, 0, out, win); break;
    }
    ok = hipGetLastError() == hipSuccess && hipEventRecord(b, st) == hipSuccess &&
         hipEventSynchronize(b) == hipSuccess && hipEventElapsedTime(&ms, a, b) == hipSuccess;
  }
  (void)hipEventDestroy(a);
  (void)hipEventDestroy(b);
  if (!ok || ms <= 0.f) return FLCE_ERR_HIP;
  // Per wave and step: 4 x 2 MFMAs of 32 x 32 x 16 multiply-adds.
  const double flops = (double)blocks * kWaves * (double)n * 8.0 * 2.0 * 32 * 32 * 16;
  *tflops = flops / ((double)ms * 1e-3) / 1e12;
  return FLCE_OK;
}

flce_status_t flce_profile_enable(int enable) {
  Profiler& P = prof();
  std::lock_guard<std::mutex> g(P.mu);
  P.on = enable != 0;
  return FLCE_OK;
}

flce_status_t flce_profile_reset(void) {
  Profiler& P = prof();
  std::lock_guard<std::mutex> g(P.mu);
  P.drain();
  for (int k = 0; k < K_NUM; ++k) {
    P.launches[k] = 0;
    P.ms[k] = 0.0;
  }
  return FLCE_OK;
}

int flce_profile_kinds(void) { return K_NUM; }

flce_status_t flce_profile_read(int kind, const char** name, int64_t* launches, double* total_ms) {
  if (kind < 0 || kind >= K_NUM) return FLCE_ERR_BAD_SHAPE;
  Profiler& P = prof();
  std::lock_guard<std::mutex> g(P.mu);
  P.drain();
  if (name) *name = kKindNames[kind];
  if (launches) *launches = P.launches[kind];
  if (total_ms) *total_ms = P.ms[kind];
  return FLCE_OK;
}

}  // extern "C"
