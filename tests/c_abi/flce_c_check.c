/*
 * The C ABI of libflce.so used from plain C99 (no Python, no torch): device
 * buffers from the HIP runtime, one stream, forward then backward, checked
 * against what the definition fixes without any reference implementation:
 *
 *   - zero weight: every logit is 0, so lse = entropy = ln V and
 *     logprob = -ln V on valid tokens (0 on ignored ones); dHidden = 0 and
 *     dWeight[k][j] = sum_i h_ik g_i ([j = y_i] - 1/V) (the entropy term
 *     vanishes because every z' - S is 0);
 *   - random weight: 0 <= entropy <= ln V, logprob <= 0,
 *     ln V + mean_j z_j <= lse <= ln V + max_j z_j (Jensen; the largest term),
 *     and logprob = z_y - lse with the logits z recomputed here in double
 *     from the same bf16 inputs;
 *   - the invalid-label count of flce_get_status, and host-side argument
 *     errors (misaligned pointer, bad reduction, too small a workspace);
 *   - class weights through flce_forward_ex (the options struct built in C):
 *     with 0/1 weights the weighted mean of logprob equals the plain mean over
 *     the tokens of weight 1, computed here from the per-token outputs of the
 *     same call; class weights under reduction NONE are refused.
 *
 * Prints "flce_c_check ok" and returns 0 on success, 1 on the first failure.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "flce.h"

#define N 300
#define H 64
#define V 1000

static int fails = 0;
#define CHECK(cond, ...)                 \
  do {                                   \
    if (!(cond)) {                       \
      printf("FAIL: " __VA_ARGS__);      \
      printf("\n");                      \
      fails++;                           \
      return 1;                          \
    }                                    \
  } while (0)
#define HIPCK(x) CHECK((x) == hipSuccess, "HIP call %s", #x)
#define FLCK(x) CHECK((x) == FLCE_OK, "%s -> %s", #x, flce_status_string(x))

static uint32_t lcg = 12345u;
static float urand(void) { /* uniform in [-1, 1) */
  lcg = lcg * 1664525u + 1013904223u;
  return (float)(lcg >> 8) * (2.0f / 16777216.0f) - 1.0f;
}
static uint16_t bf16(float f) { /* round to nearest even */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}
static float from_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static int run(int zero_weight) {
  static uint16_t hh[N * H], hw[H * V], hgh[N * H], hgw[H * V];
  static int64_t hy[N];
  static float hg[N], he[N], hlse[N], hlp[N], hent[N];
  for (int i = 0; i < N * H; ++i) hh[i] = bf16(urand());
  for (int i = 0; i < H * V; ++i) hw[i] = zero_weight ? 0 : bf16(0.25f * urand());
  for (int i = 0; i < N; ++i) {
    lcg = lcg * 1664525u + 1013904223u;
    hy[i] = (int64_t)((lcg >> 8) % V);
    hg[i] = urand();
    he[i] = urand();
  }
  hy[7] = -100;    /* ignored */
  hy[8] = V + 5;   /* invalid: counted, treated as ignored */

  void *dh, *dw, *dgh, *dgw, *ws;
  int64_t* dy;
  float *dlse, *dlp, *dent, *dg, *de;
  size_t fb = 0, bb = 0;
  FLCK(flce_workspace_size(N, H, V, FLCE_REDUCTION_NONE, &fb, &bb));
  const size_t wsb = fb > bb ? fb : bb;
  HIPCK(hipMalloc(&dh, sizeof hh));
  HIPCK(hipMalloc(&dw, sizeof hw));
  HIPCK(hipMalloc(&dgh, sizeof hgh));
  HIPCK(hipMalloc(&dgw, sizeof hgw));
  HIPCK(hipMalloc((void**)&dy, sizeof hy));
  HIPCK(hipMalloc((void**)&dlse, sizeof hlse));
  HIPCK(hipMalloc((void**)&dlp, sizeof hlp));
  HIPCK(hipMalloc((void**)&dent, sizeof hent));
  HIPCK(hipMalloc((void**)&dg, sizeof hg));
  HIPCK(hipMalloc((void**)&de, sizeof he));
  HIPCK(hipMalloc(&ws, wsb));
  HIPCK(hipMemcpy(dh, hh, sizeof hh, hipMemcpyHostToDevice));
  HIPCK(hipMemcpy(dw, hw, sizeof hw, hipMemcpyHostToDevice));
  HIPCK(hipMemcpy(dy, hy, sizeof hy, hipMemcpyHostToDevice));
  HIPCK(hipMemcpy(dg, hg, sizeof hg, hipMemcpyHostToDevice));
  HIPCK(hipMemcpy(de, he, sizeof he, hipMemcpyHostToDevice));
  hipStream_t st;
  HIPCK(hipStreamCreate(&st));

  /* Host-side argument errors: nothing is launched. */
  CHECK(flce_forward((char*)dh + 2, dw, dy, N, H, V, -100, 0.f, FLCE_REDUCTION_NONE, dlse, dlp,
                     dent, NULL, NULL, ws, wsb, st) == FLCE_ERR_MISALIGNED, "misaligned hidden");
  CHECK(flce_forward(dh, dw, dy, N, H, V, -100, 0.f, 7, dlse, dlp, dent, NULL, NULL, ws, wsb,
                     st) == FLCE_ERR_BAD_REDUCTION, "bad reduction");
  CHECK(flce_backward(dh, dw, dy, N, H, V, -100, 0.f, FLCE_REDUCTION_NONE, dlse, dent, dg, de,
                      dgh, dgw, ws, 64, st) == FLCE_ERR_WORKSPACE_TOO_SMALL, "small workspace");

  FLCK(flce_forward(dh, dw, dy, N, H, V, -100, 0.f, FLCE_REDUCTION_NONE, dlse, dlp, dent, NULL,
                    NULL, ws, wsb, st));
  int64_t invalid = -1;
  CHECK(flce_get_status(ws, &invalid, st) == FLCE_ERR_INVALID_LABEL && invalid == 1,
        "invalid-label count %lld", (long long)invalid);
  FLCK(flce_backward(dh, dw, dy, N, H, V, -100, 0.f, FLCE_REDUCTION_NONE, dlse, dent, dg, de,
                     dgh, dgw, ws, wsb, st));
  HIPCK(hipStreamSynchronize(st));
  HIPCK(hipMemcpy(hlse, dlse, sizeof hlse, hipMemcpyDeviceToHost));
  HIPCK(hipMemcpy(hlp, dlp, sizeof hlp, hipMemcpyDeviceToHost));
  HIPCK(hipMemcpy(hent, dent, sizeof hent, hipMemcpyDeviceToHost));
  HIPCK(hipMemcpy(hgh, dgh, sizeof hgh, hipMemcpyDeviceToHost));
  HIPCK(hipMemcpy(hgw, dgw, sizeof hgw, hipMemcpyDeviceToHost));

  const double lnV = log((double)V);
  for (int i = 0; i < N; ++i) {
    const int valid = hy[i] >= 0 && hy[i] < V;
    if (!valid) {
      CHECK(hlse[i] == 0.f && hlp[i] == 0.f && hent[i] == 0.f, "ignored token %d not zero", i);
      for (int k = 0; k < H; ++k) CHECK(hgh[i * H + k] == 0, "ignored token %d has a gradient", i);
      continue;
    }
    if (zero_weight) {
      CHECK(fabs(hlse[i] - lnV) < 1e-4 && fabs(hent[i] - lnV) < 1e-4 && fabs(hlp[i] + lnV) < 1e-4,
            "token %d: lse %g entropy %g logprob %g, want ln V = %g", i, hlse[i], hent[i],
            hlp[i], lnV);
    } else {
      double zmax = -1e300, zsum = 0.0, zy = 0.0;
      for (int j = 0; j < V; ++j) {
        double z = 0.0;
        for (int k = 0; k < H; ++k) z += (double)from_bf16(hh[i * H + k]) * from_bf16(hw[k * V + j]);
        zmax = z > zmax ? z : zmax;
        zsum += z;
        if (j == hy[i]) zy = z;
      }
      CHECK(hent[i] >= -1e-4 && hent[i] <= lnV + 1e-4, "token %d entropy %g", i, hent[i]);
      CHECK(hlp[i] <= 1e-6, "token %d logprob %g", i, hlp[i]);
      CHECK(hlse[i] >= lnV + zsum / V - 2e-3 && hlse[i] <= lnV + zmax + 2e-3,
            "token %d lse %g outside [%g, %g]", i, hlse[i], lnV + zsum / V, lnV + zmax);
      CHECK(fabs(hlp[i] - (zy - hlse[i])) < 2e-3, "token %d logprob %g, z_y - lse = %g", i,
            hlp[i], zy - hlse[i]);
    }
  }
  if (zero_weight) {
    double num = 0.0, den = 0.0;
    for (int i = 0; i < N * H; ++i) CHECK(hgh[i] == 0 || hgh[i] == 0x8000, "dHidden not 0");
    for (int k = 0; k < H; ++k)
      for (int j = 0; j < V; ++j) {
        double ref = 0.0;
        for (int i = 0; i < N; ++i) {
          if (hy[i] < 0 || hy[i] >= V) continue;
          ref += (double)from_bf16(hh[i * H + k]) * hg[i] * ((j == hy[i] ? 1.0 : 0.0) - 1.0 / V);
        }
        const double got = from_bf16(hgw[k * V + j]);
        num += (got - ref) * (got - ref);
        den += ref * ref;
      }
    CHECK(sqrt(num / den) < 1e-2, "dWeight closed form: rel L2 %g", sqrt(num / den));
  }
  hipFree(dh); hipFree(dw); hipFree(dgh); hipFree(dgw); hipFree(dy); hipFree(dlse);
  hipFree(dlp); hipFree(dent); hipFree(dg); hipFree(de); hipFree(ws);
  hipStreamDestroy(st);
  return 0;
}

static int run_class_weights(void) {
  static uint16_t hh[N * H], hw[H * V];
  static int64_t hy[N];
  static float hcw[V], hlp[N], hred[4];
  for (int i = 0; i < N * H; ++i) hh[i] = bf16(urand());
  for (int i = 0; i < H * V; ++i) hw[i] = bf16(0.25f * urand());
  for (int j = 0; j < V; ++j) hcw[j] = (j % 3 == 0) ? 0.f : 1.f;
  for (int i = 0; i < N; ++i) {
    lcg = lcg * 1664525u + 1013904223u;
    hy[i] = (int64_t)((lcg >> 8) % V);
  }
  hy[11] = -100;
  void *dh, *dw, *ws;
  int64_t* dy;
  float *dcw, *dlse, *dlp, *dent, *dred;
  size_t fb = 0;
  FLCK(flce_workspace_size(N, H, V, FLCE_REDUCTION_MEAN, &fb, NULL));
  HIPCK(hipMalloc(&dh, sizeof hh));
  HIPCK(hipMalloc(&dw, sizeof hw));
  HIPCK(hipMalloc((void**)&dy, sizeof hy));
  HIPCK(hipMalloc((void**)&dcw, sizeof hcw));
  HIPCK(hipMalloc((void**)&dlse, sizeof hlp));
  HIPCK(hipMalloc((void**)&dlp, sizeof hlp));
  HIPCK(hipMalloc((void**)&dent, sizeof hlp));
  HIPCK(hipMalloc((void**)&dred, sizeof hred));
  HIPCK(hipMalloc(&ws, fb));
  HIPCK(hipMemcpy(dh, hh, sizeof hh, hipMemcpyHostToDevice));
  HIPCK(hipMemcpy(dw, hw, sizeof hw, hipMemcpyHostToDevice));
  HIPCK(hipMemcpy(dy, hy, sizeof hy, hipMemcpyHostToDevice));
  HIPCK(hipMemcpy(dcw, hcw, sizeof hcw, hipMemcpyHostToDevice));
  hipStream_t st;
  HIPCK(hipStreamCreate(&st));
  flce_options_t opt = {.ignore_index = -100, .softcap = 0.f, .reduction = FLCE_REDUCTION_NONE,
                        .z_loss_scale = 0.f, .grad_dtype = FLCE_GRAD_BF16, .class_weight = dcw};
  CHECK(flce_forward_ex(dh, dw, dy, N, H, V, &opt, dlse, dlp, dent, NULL, NULL, NULL, ws, fb, st) ==
            FLCE_ERR_BAD_OPTION, "class weights under reduction none");
  opt.reduction = FLCE_REDUCTION_MEAN;
  FLCK(flce_forward_ex(dh, dw, dy, N, H, V, &opt, dlse, dlp, dent, NULL, NULL, dred, ws, fb, st));
  HIPCK(hipStreamSynchronize(st));
  HIPCK(hipMemcpy(hlp, dlp, sizeof hlp, hipMemcpyDeviceToHost));
  HIPCK(hipMemcpy(hred, dred, sizeof hred, hipMemcpyDeviceToHost));
  double sum = 0.0;
  int count = 0;
  for (int i = 0; i < N; ++i)
    if (hy[i] >= 0 && hcw[hy[i]] != 0.f) {
      sum += hlp[i];
      ++count;
    }
  const double want = count ? sum / count : 0.0;
  CHECK(count > 0 && fabs(hred[0] - want) <= 1e-5 * (1.0 + fabs(want)),
        "weighted logprob mean %g, mean over weight-1 tokens %g", hred[0], want);
  hipFree(dh); hipFree(dw); hipFree(dy); hipFree(dcw); hipFree(dlse); hipFree(dlp);
  hipFree(dent); hipFree(dred); hipFree(ws);
  hipStreamDestroy(st);
  return 0;
}

int main(void) {
  printf("libflce version %d\n", flce_version());
  if (run(1)) return 1;
  if (run(0)) return 1;
  if (run_class_weights()) return 1;
  printf("flce_c_check ok\n");
  return 0;
}
