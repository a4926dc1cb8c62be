// Host-only check of the planner (flce_plan.hpp): for a sweep of shapes up to
// the library's limits, every workspace layout that make_plan and
// make_fused_plan produce is 256-byte aligned, its regions follow one another
// without overlap inside the total, and the chunk and split counts cover the
// vocabulary and the tokens. Built with AddressSanitizer and
// UndefinedBehaviorSanitizer (integer overflow, shifts, bounds) by
// tests/test_plan_sanitizers.py; exits 1 on the first violation.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "flce_plan.hpp"

using namespace flce;

static int failures = 0;

#define CHECK(cond, ...)                                  \
  do {                                                    \
    if (!(cond)) {                                        \
      std::fprintf(stderr, "FAIL %s: ", #cond);           \
      std::fprintf(stderr, __VA_ARGS__);                  \
      std::fprintf(stderr, "\n");                         \
      if (++failures > 20) std::exit(1);                  \
    }                                                     \
  } while (0)

struct Region {
  const char* name;
  size_t off, bytes;
};

// Regions in layout order: aligned, inside [first, total), not overlapping.
static void check_layout(const char* what, int64_t N, int64_t H, int64_t V,
                         const std::vector<Region>& r, size_t first, size_t total) {
  size_t end = first;
  for (const Region& g : r) {
    CHECK(g.off % kAlign == 0, "%s %s offset %zu not aligned (N=%lld H=%lld V=%lld)", what, g.name,
          g.off, (long long)N, (long long)H, (long long)V);
    CHECK(g.off >= end, "%s %s starts at %zu inside the previous region ending %zu", what, g.name,
          g.off, end);
    end = g.off + g.bytes;
    CHECK(end >= g.off, "%s %s size wraps", what, g.name);
  }
  CHECK(end <= total, "%s regions end at %zu past the total %zu (N=%lld H=%lld V=%lld)", what, end,
        total, (long long)N, (long long)H, (long long)V);
}

static void check_plan(int64_t N, int64_t H, int64_t V, int red) {
  const Plan p = make_plan(N, H, V, red);
  const size_t blk = kBlockBytes;
  CHECK(p.TB == ceil_div(N, kTile) && p.VT == ceil_div(V, kTile) && p.HT == ceil_div(H, kTile),
        "tile counts");
  CHECK(p.Vc % kTile == 0 && p.Vc >= kTile && p.Vc <= kMaxVc, "Vc %lld", (long long)p.Vc);
  CHECK(p.nchunks == ceil_div(V, p.Vc), "chunks %d", p.nchunks);
  CHECK((int64_t)p.nchunks * p.Vc >= V && (int64_t)(p.nchunks - 1) * p.Vc < V, "chunk cover");
  CHECK(p.kbv == p.Vc / kBK && p.VTc == p.Vc / kTile, "chunk blocks");
  CHECK(p.dx_splits >= 1 && p.dx_splits <= 4, "dx splits %d", p.dx_splits);
  CHECK(p.dw_splits >= 1 && p.dw_kper >= 1, "dw splits");
  if (p.nkb > 0)
    CHECK((int64_t)p.dw_splits * p.dw_kper >= p.nkb && (int64_t)(p.dw_splits - 1) * p.dw_kper < p.nkb,
          "dw split cover %d x %d for %d", p.dw_splits, p.dw_kper, p.nkb);
  // The two bf16 logit-gradient images of a chunk stay within the largest
  // budget (4 GiB) unless the 2048-column floor needs more.
  const size_t images = 4 * (size_t)(p.TB > 0 ? p.TB : 1) * kTile * (size_t)p.Vc;
  CHECK(images <= kMaxDBudget || p.Vc <= 2048 || p.Vc == (int64_t)p.VT * kTile, "images %zu Vc %lld",
        images, (long long)p.Vc);
  // Byte offsets inside one strip of a blocked image stay below 2^31 (the
  // kernels address strips with 32-bit offsets).
  CHECK((size_t)p.kbv * blk < ((size_t)1 << 31), "dtv strip");
  CHECK((size_t)p.nkb * blk < ((size_t)1 << 31), "dvt strip");
  CHECK((size_t)p.hkb * blk < ((size_t)1 << 31), "hidden strip");
  const bool reduce = red != FLCE_REDUCTION_NONE;
  check_layout("forward", N, H, V,
               {{"idx", p.f_idx, 4 * (size_t)N},
                {"labc", p.f_labc, 4 * (size_t)N},
                {"part", p.f_part, 16 * (size_t)p.VT * (size_t)N},
                {"zlab", p.f_zlab, 4 * (size_t)N},
                {"bsum", p.f_bsum, reduce ? 32 * (size_t)ceil_div(N, kCombineTokens) : 0},
                {"xb", p.f_xb, blk * (size_t)p.TB * (size_t)p.hkb},
                {"wp", p.f_wp, p.padw ? 2 * (size_t)H * (size_t)p.V8 : 0}},
               kHeaderBytes, p.f_total);
  check_layout("backward", N, H, V,
               {{"lab", p.b_lab, 4 * (size_t)N},
                {"idx", p.b_idx, 4 * (size_t)N},
                {"coef", p.b_coef, sizeof(DzToken) * (size_t)N},
                {"wb", p.b_wb, blk * (size_t)p.HT * (size_t)p.kbv},
                {"xb", p.b_xb, blk * (size_t)p.TB * (size_t)p.hkb},
                {"xtb", p.b_xtb, blk * (size_t)p.HT * (size_t)p.nkb},
                {"dtv", p.b_dtv, blk * (size_t)p.TB * (size_t)p.kbv},
                {"dvt", p.b_dvt, blk * (size_t)p.VTc * (size_t)p.nkb},
                {"acc", p.b_acc,
                 (p.nchunks > 1 || p.dx_splits > 1) ? 4 * (size_t)p.dx_splits * (size_t)N * (size_t)H : 0},
                {"part", p.b_part, p.dw_splits > 1 ? 4 * (size_t)p.dw_splits * (size_t)H * (size_t)p.Vc : 0},
                {"wp", p.b_wp, p.padw ? 2 * (size_t)H * (size_t)p.V8 : 0},
                {"gwp", p.b_gwp, p.padw ? 4 * (size_t)H * (size_t)p.V8 : 0}},
               kHeaderBytes, p.b_total);
}

static void check_fused(int64_t N, int64_t H, int64_t V, int red, int64_t chunk, int gdt) {
  flce_options_t o{-100, 0.f, red, 0.f, gdt, nullptr, 0};
  if (check_options(&o) != FLCE_OK) return;
  const FusedPlan f = make_fused_plan(N, H, V, o, chunk);
  const Plan& p = f.b;
  const size_t blk = kBlockBytes;
  CHECK(f.TBc >= 1, "TBc %d", f.TBc);
  CHECK((int64_t)f.nchunks * f.TBc >= p.TB && (f.nchunks == 0 || (int64_t)(f.nchunks - 1) * f.TBc < p.TB),
        "token chunk cover %d x %d for %d", f.nchunks, f.TBc, p.TB);
  if (chunk == 0 && f.TBc > 1)
    CHECK(4 * (size_t)f.TBc * kTile * (size_t)p.VT * kTile <= kFusedImageBudget,
          "default chunk images over budget: TBc %d VT %d", f.TBc, p.VT);
  const size_t rows = (size_t)p.TB * kTile, crow = (size_t)f.TBc * kTile;
  check_layout("fused", N, H, V,
               {{"idx", f.idx, 4 * (size_t)N},
                {"labc", f.labc, 4 * (size_t)N},
                {"zlab", f.zlab, 4 * (size_t)N},
                {"part", f.part, 16 * (size_t)p.VT * (size_t)N},
                {"bsum", f.bsum, red != FLCE_REDUCTION_NONE ? 32 * rows / kCombineTokens : 0},
                {"coef", f.coef, sizeof(DzToken) * rows},
                {"xb", f.xb, blk * (size_t)p.TB * (size_t)p.hkb},
                {"xtb", f.xtb, blk * (size_t)p.HT * (size_t)p.nkb},
                {"wb", f.wb, blk * (size_t)p.HT * (size_t)f.kbv},
                {"dtv", f.dtv, blk * (size_t)f.TBc * (size_t)f.kbv},
                {"dvt", f.dvt, blk * (size_t)p.VT * (size_t)f.TBc * (kTile / kBK)},
                {"mref", f.mref, 4 * 2 * (size_t)p.VT * crow},
                {"dxacc", f.dxacc, f.dx_splits > 1 ? 4 * (size_t)f.dx_splits * crow * (size_t)H : 0},
                {"dwacc", f.dwacc, f.dw_acc ? 4 * (size_t)H * (size_t)p.V8 : 0},
                {"wp", f.wp, p.padw ? 2 * (size_t)H * (size_t)p.V8 : 0},
                {"gwp", f.gwp, p.padw ? 4 * (size_t)H * (size_t)p.V8 : 0}},
               kHeaderBytes, f.total);
}

int main() {
  const int64_t Ns[] = {0, 1, 77, 255, 256, 257, 4096, 8192, 32768, 300000, kMaxN};
  const int64_t Hs[] = {8, 64, 96, 2304, 4096, 5120, 65536, kMaxH};
  const int64_t Vs[] = {1, 7, 8, 1000, 1001, 2048, 32000, 128256, 152064, 256000, 1 << 21,
                        kMaxV};
  int plans = 0;
  for (int64_t N : Ns)
    for (int64_t H : Hs)
      for (int64_t V : Vs) {
        if (check_shape(N, H, V) != FLCE_OK) continue;
        for (int red = 0; red < 3; ++red) {
          check_plan(N, H, V, red);
          ++plans;
          if (V <= ((int64_t)1 << 21))
            for (int64_t chunk : {(int64_t)0, (int64_t)256, (int64_t)2048, N})
              for (int gdt = 0; gdt < 2; ++gdt) check_fused(N, H, V, red, chunk, gdt);
        }
      }
  // Limits are refused.
  CHECK(check_shape(-1, 8, 8) == FLCE_ERR_BAD_SHAPE, "N < 0");
  CHECK(check_shape(kMaxN + 1, 8, 8) == FLCE_ERR_BAD_SHAPE, "N > max");
  CHECK(check_shape(8, kMaxH + 8, 8) == FLCE_ERR_BAD_SHAPE, "H > max");
  CHECK(check_shape(8, 8, kMaxV + 1) == FLCE_ERR_BAD_SHAPE, "V > max");
  CHECK(check_shape(8, 12, 8) == FLCE_ERR_MISALIGNED, "H not a multiple of 8");
  std::printf("plans checked: %d, failures: %d\n", plans, failures);
  return failures == 0 ? 0 : 1;
}
