// Sizes shared by the kernels and the host planner of the fused linear
// cross-entropy head: the GEMM tile, the K block of the blocked operand
// images, the combine's token group, and the per-token gradient constants.
// Plain C++ (no HIP), so the planner compiles on its own for host-only checks.
#pragma once

#include <stdint.h>

namespace flce {

constexpr int kTile = 256;                          // M and N extent of a block tile; strip height
constexpr int kBK = 32;                             // K values per block / LDS stage
constexpr int kBlockBytes = kTile * kBK * 2;        // 16 KiB: one K block of one strip
constexpr int kBlockElems = kBlockBytes / 2;
constexpr int kCombineTokens = 64;                  // tokens per combine block (one per lane)

// Per-token constants of the logit gradient (see bwd_dlogits_kernel):
//   dz'_v = gbar [v == y] + k0 - p_v (ebar z'_v + cs),
//   cs = gbar - ebar S - gu - 2 lam gz lse,  k0 = -gu / V,
// from the upstream gradients gbar (logprob), ebar (entropy), gu
// (uniform_ce) and gz (z_loss). Ignored tokens: lse = 1e30 (every p
// underflows to 0) and zeros.
struct DzToken {
  float lse, ebar, cs, gbar;
  float k0, pad0, pad1, pad2;
};

}  // namespace flce
