// Kernels of the fused linear cross-entropy + entropy head (gfx950).
//
// Forward:  fwd_prep, transpose -> fwd_tile -> fwd_combine (-> fwd_mean)
// Backward: bwd_prep, transpose -> per vocabulary chunk { bwd_dlogits -> bwd_dx
//           -> bwd_dw (-> dw_reduce) }
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

// One block of 1024 threads. lab32[t] = label if it is a valid class id, else
// -1 (ignored or out of range). header[0] = #labels neither ignore_index nor in
// [0, V); header[1] = #valid tokens.
__global__ void __launch_bounds__(1024) fwd_prep_kernel(const int64_t* __restrict__ labels,
                                                        int64_t N, int64_t V, int64_t ignore_index,
                                                        int32_t* __restrict__ lab32,
                                                        int32_t* __restrict__ header) {
  __shared__ int sh[1024];
  int inv = 0, nv = 0;
  for (int64_t t = threadIdx.x; t < N; t += 1024) {
    const int64_t y = labels[t];
    int32_t o = -1;
    if (y != ignore_index) {
      if (y >= 0 && y < V) {
        o = (int32_t)y;
        ++nv;
      } else {
        ++inv;
      }
    }
    lab32[t] = o;
  }
  inv = block_sum<int, 1024>(inv, sh);
  nv = block_sum<int, 1024>(nv, sh);
  if (threadIdx.x == 0) {
    header[0] = inv;
    header[1] = nv;
  }
}

// ---- hidden^T, the token-contiguous copy the logit GEMMs read ------------------

// XT[h][t] = hidden[t][h] for t < N; columns t in [N, ldt) are zero. 64 x 64
// tiles through LDS, 16-byte loads and stores.
__global__ void __launch_bounds__(256) transpose_kernel(const uint16_t* __restrict__ X, int64_t N,
                                                        int64_t H, int64_t ldt,
                                                        uint16_t* __restrict__ XT) {
  __shared__ uint16_t tile[64][72];
  const int64_t h0 = (int64_t)blockIdx.x * 64, t0 = (int64_t)blockIdx.y * 64;
  const int tid = threadIdx.x;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int r = tid / 8 + 32 * p, c = (tid % 8) * 8;
    u32x4_t v = u32x4_t{0u, 0u, 0u, 0u};
    if (t0 + r < N && h0 + c < H) v = *reinterpret_cast<const u32x4_t*>(X + (t0 + r) * H + h0 + c);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      tile[r][c + 2 * e] = (uint16_t)(v[e] & 0xFFFFu);
      tile[r][c + 2 * e + 1] = (uint16_t)(v[e] >> 16);
    }
  }
  __syncthreads();
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int hr = tid / 8 + 32 * p, tc = (tid % 8) * 8;
    if (h0 + hr < H && t0 + tc < ldt) {
      u32x4_t v;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        v[e] = (uint32_t)tile[tc + 2 * e][hr] | ((uint32_t)tile[tc + 2 * e + 1][hr] << 16);
      *reinterpret_cast<u32x4_t*>(XT + (h0 + hr) * ldt + t0 + tc) = v;
    }
  }
}

// ---- forward: fused logit tiles + online row statistics ---------------------

struct FwdTileArgs {
  const uint16_t* weight;  // [H,V]
  const uint16_t* xt;      // [H, ldt] hidden^T
  const int32_t* lab;      // [N], -1 = no label
  int64_t N, H, V, ldt;
  int VT, TB;              // vocabulary tiles, token blocks (256 each)
  int group;               // token blocks per XCD patch (see group_map)
  float cap, cap_k;        // softcap c and 2*log2(e)/c
  float4* part;            // [VT][N] {m, s, u, 0} per vocabulary tile
  float* zlab;             // [N] capped logit of the label
};

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

// Block (tb, vt): tokens [256 tb, +256) against vocabulary [256 vt, +256).
// The MFMA tile is z^T: rows = vocabulary (A = weight, row-major [H,V]), cols =
// tokens (B = hidden^T), so each lane's 64 accumulators of one 32-column block
// belong to one token and the row statistics need no cross-lane work until the
// end. The block reduces its tile to (m, s, u) per token and stores it as the
// tile's partial state.
template <bool CAP>
__global__ void __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                               amdgpu_waves_per_eu(2, 2)))
fwd_tile_kernel(FwdTileArgs a) {
  FLCE_DECLARE_STAGES(sa, sb);
  int tb, vt;
  group_map(xcd_remap(blockIdx.x, gridDim.x), a.TB, a.VT, a.group, tb, vt);
  const int lane = threadIdx.x & 63, lh = lane >> 5;
  const int wave = threadIdx.x >> 6, wm = wave & 1, wn = wave >> 1;
  const int64_t n0 = (int64_t)tb * kTile;

  Acc acc;
  {
    Mainloop<RMAJOR, RMAJOR> ml;
    ml.run(sa, sb, Operand{a.weight, a.V, a.V}, Operand{a.xt, a.ldt, a.N}, (int64_t)vt * kTile,
           n0, 0, a.H, acc);
  }

  const int vb = vt * kTile + wm * 128;  // first vocabulary row of this wave
  const bool full = (int64_t)vb + 128 <= a.V;
  // Rows at offset o (0..127, without the lane-half term) are valid iff o < lim.
  const int lim = (int)(a.V - vb) - 4 * lh;
  float m[2], s[2], u[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    float z[64];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = acc[i][j][r];
        if constexpr (CAP) x = softcap_apply(x, a.cap, a.cap_k);
        if (!full) x = (i * 32 + 8 * (r >> 2) + (r & 3)) < lim ? x : kNegBig;
        z[i * 16 + r] = x;
      }
    float mx[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float x = z[i * 16];
#pragma unroll
      for (int r = 1; r < 16; ++r) x = fmaxf(x, z[i * 16 + r]);
      mx[i] = x;
    }
    const float mb = fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3]));
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
        if (!full) e = z[i * 16 + r] == kNegBig ? 0.f : e;
        sp[i] += e;
        up[i] = fmaf(e, d, up[i]);
      }
    }
    m[j] = mb;
    s[j] = (sp[0] + sp[1]) + (sp[2] + sp[3]);
    u[j] = (up[0] + up[1]) + (up[2] + up[3]);

    // The label's logit: exactly one lane of one block in the grid owns it.
    const int64_t t = n0 + acc_col(wn, j, lane);
    const int y = t < a.N ? a.lab[t] : -1;
    const int off = y - vb;
    if ((unsigned)off < 128u && (((off & 31) >> 2) & 1) == lh) {
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
  }
  float* red = reinterpret_cast<float*>(sa[0]);
  if (wm == 1 && lane < 32) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = acc_col(wn, j, lane);
      red[c * 3 + 0] = m[j];
      red[c * 3 + 1] = s[j];
      red[c * 3 + 2] = u[j];
    }
  }
  __syncthreads();
  if (wm == 0 && lane < 32) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = acc_col(wn, j, lane);
      merge_state2(m[j], s[j], u[j], red[c * 3 + 0], red[c * 3 + 1], red[c * 3 + 2]);
      const int64_t t = n0 + c;
      if (t < a.N) a.part[(int64_t)vt * a.N + t] = make_float4(m[j], s[j], u[j] * kLn2, 0.f);
    }
  }
}

// ---- forward: merge the vocabulary splits -------------------------------------

// One thread per token. Writes lse, logprob, entropy; with bsum != nullptr also
// the block's sums of logprob and entropy over valid tokens (float64).
__global__ void __launch_bounds__(256) fwd_combine_kernel(const float4* __restrict__ part, int S,
                                                          const float* __restrict__ zlab,
                                                          const int32_t* __restrict__ lab32,
                                                          int64_t N, float* __restrict__ lse,
                                                          float* __restrict__ logprob,
                                                          float* __restrict__ entropy,
                                                          double2* __restrict__ bsum) {
  __shared__ double sh[256];
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  double slp = 0.0, sent = 0.0;
  if (t < N) {
    if (lab32[t] >= 0) {
      float4 p = part[t];
      float m = p.x, s = p.y, u = p.z;
      for (int k = 1; k < S; ++k) {
        const float4 q = part[(int64_t)k * N + t];
        const float mn = fmaxf(m, q.x);
        const float a1 = expf(m - mn), a2 = expf(q.x - mn);
        u = a1 * fmaf(m - mn, s, u) + a2 * fmaf(q.x - mn, q.y, q.z);
        s = a1 * s + a2 * q.y;
        m = mn;
      }
      const float ls = logf(s);
      const float l = m + ls;
      const float e = ls - u / s;
      const float lp = zlab[t] - l;
      lse[t] = l;
      entropy[t] = e;
      logprob[t] = lp;
      slp = lp;
      sent = e;
    } else {
      lse[t] = 0.f;
      entropy[t] = 0.f;
      logprob[t] = 0.f;
    }
  }
  if (bsum != nullptr) {
    slp = block_sum<double, 256>(slp, sh);
    sent = block_sum<double, 256>(sent, sh);
    if (threadIdx.x == 0) bsum[blockIdx.x] = make_double2(slp, sent);
  }
}

// One block: sums the per-block partial sums in a fixed order and divides by
// the number of valid tokens (0 when there are none).
__global__ void __launch_bounds__(256) fwd_mean_kernel(const double2* __restrict__ bsum, int nb,
                                                       const int32_t* __restrict__ header,
                                                       float* __restrict__ lp_mean,
                                                       float* __restrict__ ent_mean) {
  __shared__ double sh[256];
  double a = 0.0, b = 0.0;
  for (int i = threadIdx.x; i < nb; i += 256) {
    a += bsum[i].x;
    b += bsum[i].y;
  }
  a = block_sum<double, 256>(a, sh);
  b = block_sum<double, 256>(b, sh);
  if (threadIdx.x == 0) {
    const int n = header[1];
    lp_mean[0] = n > 0 ? (float)(a / n) : 0.f;
    ent_mean[0] = n > 0 ? (float)(b / n) : 0.f;
  }
}

// ---- backward: per-token coefficients ------------------------------------------

// One block of 1024. coef[t] = {lse, S = lse - entropy, gbar, ebar} for valid
// tokens; for others lse = 1e30 (so every p underflows to 0) and zeros.
__global__ void __launch_bounds__(1024) bwd_prep_kernel(
    const int64_t* __restrict__ labels, int64_t N, int64_t V, int64_t ignore_index, int mean,
    const float* __restrict__ lse, const float* __restrict__ entropy,
    const float* __restrict__ glp, const float* __restrict__ gent, float4* __restrict__ coef,
    int32_t* __restrict__ lab32, int32_t* __restrict__ header) {
  __shared__ int sh[1024];
  int inv = 0, nv = 0;
  for (int64_t t = threadIdx.x; t < N; t += 1024) {
    const int64_t y = labels[t];
    if (y != ignore_index) {
      if (y >= 0 && y < V) ++nv;
      else ++inv;
    }
  }
  inv = block_sum<int, 1024>(inv, sh);
  nv = block_sum<int, 1024>(nv, sh);
  const float g0 = (mean && glp != nullptr && nv > 0) ? glp[0] / (float)nv : 0.f;
  const float e0 = (mean && gent != nullptr && nv > 0) ? gent[0] / (float)nv : 0.f;
  for (int64_t t = threadIdx.x; t < N; t += 1024) {
    const int64_t y = labels[t];
    if (y != ignore_index && y >= 0 && y < V) {
      const float g = mean ? g0 : (glp != nullptr ? glp[t] : 0.f);
      const float e = mean ? e0 : (gent != nullptr ? gent[t] : 0.f);
      const float l = lse[t];
      coef[t] = make_float4(l, l - entropy[t], g, e);
      lab32[t] = (int32_t)y;
    } else {
      coef[t] = make_float4(1e30f, 0.f, 0.f, 0.f);
      lab32[t] = -1;
    }
  }
  if (threadIdx.x == 0) {
    header[0] = inv;
    header[1] = nv;
  }
}

// ---- backward: recompute logits, form the logit gradient ----------------------

struct DlogitsArgs {
  const uint16_t* weight;  // [H,V]
  const uint16_t* xt;      // [H, ldt] hidden^T
  const float4* coef;      // [N]
  const int32_t* lab;      // [N]
  int64_t N, H, V, ldt;
  int64_t v0;              // first vocabulary column of this chunk
  int64_t vc;              // valid columns in this chunk
  int VTc, TB;             // vocabulary tiles in the chunk, token blocks
  int group;
  float cap, cap_k, inv_cap;
  uint16_t* dt;            // [vc, ldt] bf16 logit gradient of the chunk, vocabulary-major
};

// dz' = gbar ([v == y] - p) - ebar p (z' - S), dz = dz' (1 - (z'/c)^2) if
// capped; written as bf16 dt[v - v0][t]. Token columns in [N, ldt) get 0.
template <bool CAP>
__global__ void __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                               amdgpu_waves_per_eu(2, 2)))
bwd_dlogits_kernel(DlogitsArgs a) {
  FLCE_DECLARE_STAGES(sa, sb);
  int tb, vt;
  group_map(xcd_remap(blockIdx.x, gridDim.x), a.TB, a.VTc, a.group, tb, vt);
  const int lane = threadIdx.x & 63, lh = lane >> 5;
  const int wave = threadIdx.x >> 6, wm = wave & 1, wn = wave >> 1;
  const int64_t n0 = (int64_t)tb * kTile;
  const int64_t vl0 = (int64_t)vt * kTile;  // chunk-local first column of the tile

  Acc acc;
  {
    Mainloop<RMAJOR, RMAJOR> ml;
    ml.run(sa, sb, Operand{a.weight + a.v0, a.V, a.vc}, Operand{a.xt, a.ldt, a.N}, vl0, n0, 0,
           a.H, acc);
  }

  // Rows (vocabulary) past vc fall outside the resource; columns (tokens) past
  // ldt are masked explicitly.
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(a.dt, a.vc * a.ldt * 2);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int64_t t = n0 + acc_col(wn, j, lane);
    float4 c = make_float4(1e30f, 0.f, 0.f, 0.f);
    int y = -1;
    if (t < a.N) {
      c = a.coef[t];
      y = a.lab[t];
    }
    const bool tok = t < a.ldt;
    const float nl = -c.x * kLog2e;
    const float cS = c.z - c.w * c.y;  // gbar - ebar * S
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float z = acc[i][j][r];
        if constexpr (CAP) z = softcap_apply(z, a.cap, a.cap_k);
        const float p = fast_exp2(fmaf(z, kLog2e, nl));
        float d = -p * fmaf(c.w, z, cS);
        if constexpr (CAP) {
          const float q = z * a.inv_cap;
          d *= fmaf(-q, q, 1.f);
        }
        const int64_t vl = vl0 + acc_row(wm, i, r, lane);
        buf_store_u16(bf16_bits(d), rd, tok ? (uint32_t)((vl * a.ldt + t) * 2) : kOOB);
      }
    // The label entry gets + gbar (times the cap factor): rewrite that element
    // after the stores above (same lane and address, so it lands last).
    const int64_t off = (int64_t)y - a.v0 - vl0 - wm * 128;
    if (y >= 0 && off >= 0 && off < 128 && (((off & 31) >> 2) & 1) == lh) {
      const int isel = (int)(off >> 5);
      const int rsel = (int)((((off & 31) >> 3) << 2) | (off & 3));
      float z = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) z = (i == isel && r == rsel) ? acc[i][j][r] : z;
      if constexpr (CAP) z = softcap_apply(z, a.cap, a.cap_k);
      const float p = fast_exp2(fmaf(z, kLog2e, nl));
      float d = c.z - p * fmaf(c.w, z, cS);
      if constexpr (CAP) {
        const float q = z * a.inv_cap;
        d *= fmaf(-q, q, 1.f);
      }
      buf_store_u16(bf16_bits(d), rd, (uint32_t)(((y - a.v0) * a.ldt + t) * 2));
    }
    __builtin_amdgcn_sched_barrier(0);  // one token column at a time
  }
}

// ---- backward: dH (+)= D W_chunk^T ---------------------------------------------

enum { DX_ONLY = 0, DX_FIRST = 1, DX_MID = 2, DX_LAST = 3 };

struct DxArgs {
  const uint16_t* dt;      // [vc, ldt] logit gradient, vocabulary-major
  const uint16_t* weight;  // [H,V]
  int64_t N, H, V, v0, vc, ldt;
  int TB, HT;              // token blocks, hidden tiles
  int group;
  float* acc;              // [N,H] fp32 accumulator over chunks
  uint16_t* gh;            // [N,H] bf16 output
};

// C[t][h] = sum_v dt[v][t] W[h][v0 + v]. MODE: DX_ONLY (single chunk: write
// bf16), DX_FIRST (store fp32), DX_MID (add into fp32), DX_LAST (add and write
// bf16). Out-of-range rows and columns fall outside the buffer resources.
template <int MODE>
__global__ void __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                               amdgpu_waves_per_eu(2, 2)))
bwd_dx_kernel(DxArgs a) {
  FLCE_DECLARE_STAGES(sa, sb);
  int tb, ht;
  group_map(xcd_remap(blockIdx.x, gridDim.x), a.TB, a.HT, a.group, tb, ht);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6, wm = wave & 1, wn = wave >> 1;
  const int64_t m0 = (int64_t)tb * kTile, h0 = (int64_t)ht * kTile;
  Acc acc;
  {
    Mainloop<RMAJOR, KMAJOR> ml;
    ml.run(sa, sb, Operand{a.dt, a.ldt, a.N}, Operand{a.weight + a.v0, a.V, a.H}, m0, h0, 0,
           a.vc, acc);
  }
  const int64_t base = m0 * a.H + h0;
  const int64_t span = (a.N - m0) * a.H - h0;  // elements from the tile origin to the end
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(a.gh + base, span * 2);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(a.acc + base, span * 4);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int hl = acc_col(wn, j, lane);
    const bool hok = h0 + hl < a.H;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint32_t e = (uint32_t)(acc_row(wm, i, r, lane) * a.H + hl);
        const float v = acc[i][j][r];
        if constexpr (MODE == DX_ONLY) {
          buf_store_u16(bf16_bits(v), rg, hok ? e * 2 : kOOB);
        } else if constexpr (MODE == DX_FIRST) {
          buf_store_f32(v, ra, hok ? e * 4 : kOOB);
        } else if constexpr (MODE == DX_MID) {
          const uint32_t o = hok ? e * 4 : kOOB;
          buf_store_f32(buf_load_f32(ra, o) + v, ra, o);
        } else {
          const uint32_t o = hok ? e * 4 : kOOB;
          buf_store_u16(bf16_bits(buf_load_f32(ra, o) + v), rg, hok ? e * 2 : kOOB);
        }
      }
      __builtin_amdgcn_sched_barrier(0);  // one 32 x 32 block at a time
    }
  }
}

// ---- backward: dW_chunk = hidden^T D ------------------------------------------

struct DwArgs {
  const uint16_t* hidden;  // [N,H]
  const uint16_t* dt;      // [vc, ldt] logit gradient, vocabulary-major
  int64_t N, H, V, v0, vc, ldt;
  int HT, VTc, splits;
  int group;
  int64_t kper;            // tokens per split (multiple of 32)
  int64_t ldp;             // row stride of the split partials
  uint16_t* gw;            // [H,V] bf16 output
  float* part;             // [splits][H][ldp] fp32 (SPLIT only)
};

// C[h][v] = sum_t hidden[t][h] dt[v][t] over the split's tokens.
template <bool SPLIT>
__global__ void __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                               amdgpu_waves_per_eu(2, 2)))
bwd_dw_kernel(DwArgs a) {
  FLCE_DECLARE_STAGES(sa, sb);
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int per = a.HT * a.VTc;
  const int sp = L / per;
  int ht, vt;
  group_map(L - sp * per, a.HT, a.VTc, a.group, ht, vt);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6, wm = wave & 1, wn = wave >> 1;
  const int64_t h0 = (int64_t)ht * kTile, vl0 = (int64_t)vt * kTile;
  const int64_t kbeg = (int64_t)sp * a.kper;
  const int64_t kend = kbeg + a.kper < a.N ? kbeg + a.kper : a.N;
  Acc acc;
  {
    Mainloop<RMAJOR, KMAJOR> ml;
    ml.run(sa, sb, Operand{a.hidden, a.H, a.H}, Operand{a.dt, a.ldt, a.vc}, h0, vl0, kbeg, kend,
           acc);
  }
  int64_t ld, base, span;
  if constexpr (SPLIT) {
    ld = a.ldp;
    base = ((int64_t)sp * a.H + h0) * ld + vl0;
    span = (a.H - h0) * ld - vl0;
  } else {
    ld = a.V;
    base = h0 * ld + a.v0 + vl0;
    span = (a.H - h0) * ld - (a.v0 + vl0);
  }
  const __amdgpu_buffer_rsrc_t rs =
      SPLIT ? make_rsrc(a.part + base, span * 4) : make_rsrc(a.gw + base, span * 2);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int vl = acc_col(wn, j, lane);
    const bool vok = vl0 + vl < a.vc;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint32_t e = (uint32_t)(acc_row(wm, i, r, lane) * ld + vl);
        if constexpr (SPLIT)
          buf_store_f32(acc[i][j][r], rs, vok ? e * 4 : kOOB);
        else
          buf_store_u16(bf16_bits(acc[i][j][r]), rs, vok ? e * 2 : kOOB);
      }
  }
}

// Sums the split partials in split order and writes bf16 dW for the chunk.
__global__ void __launch_bounds__(256) dw_reduce_kernel(const float* __restrict__ part, int splits,
                                                        int64_t H, int64_t vc, int64_t ldd,
                                                        int64_t V, int64_t v0,
                                                        uint16_t* __restrict__ gw) {
  const int64_t n = H * vc;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) {
    const int64_t h = e / vc, v = e % vc;
    float s = 0.f;
    for (int k = 0; k < splits; ++k) s += part[((int64_t)k * H + h) * ldd + v];
    gw[h * V + v0 + v] = (uint16_t)bf16_bits(s);
  }
}

// Writes zeros (used for empty inputs; a kernel rather than a memset so the
// enqueued work is plain kernels only).
__global__ void __launch_bounds__(256) fill_zero_kernel(uint32_t* __restrict__ p, int64_t n32) {
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n32; e += (int64_t)gridDim.x * 256)
    p[e] = 0u;
}

}  // namespace flce
