"""Plain float64 CPU oracle for the fused linear cross-entropy + entropy head.

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this module. It shares no code, table or helper
with the GPU library, and the GPU library never imports it.

Everything here is the plain definition written out: the full logits row is
materialised (in blocks of rows, for memory only), in float64, from the exact
bf16 input values. No blocking over the vocabulary, no online softmax, no
fusion.

Sources (web pages on fusing the LM head with cross-entropy and entropy):

  [verl-462]  verl pull request #462 (memory-efficient entropy,
              ``linear_cross_entropy``): sections "Equivalent compute logic"
              and "API".
  [liger-551] Liger-Kernel pull request #551, "[Verl] Add entropy loss to
              cross_entropy_loss and fused_linear_cross_entropy_loss":
              Summary and the review thread.
  [liger-435] Liger-Kernel pull request #435, "Fix LigerCrossEntropyLoss
              Reduction Behavior for 'None' Mode": Summary and "Why we pass
              gradient to output.backward()".
  [liger-127] Liger-Kernel issue #127, "[feat] FusedLinearCrossEntropy support
              for Gemma2": the proposal and the maintainer's discussion
              (points 2 to 4 and the closing suggestion).

Readings taken where the pages are silent or ambiguous:

  R1  The first output is the label log-probability logprob = z'_y - lse,
      i.e. minus the cross-entropy, as the compute logic of [verl-462] negates
      the cross-entropy; the API example there calls it "loss".
  R2  Tokens whose label equals ``ignore_index`` produce lse = logprob =
      entropy = 0, get no gradient, and are excluded from the count n used by
      the mean ([liger-551] review: the mean divides by the number of
      non-ignored tokens).
  R3  reduction="mean" reduces both outputs over the n valid tokens; the
      per-token vectors are returned as well. With n = 0 both means are 0.
  R4  Softcap: z' = c * tanh(z / c) with c > 0; c <= 0 means no cap
      ([liger-127]: scaling plus a tanh that caps the range).
  R5  Labels outside [0, V) that are not ``ignore_index`` are an error here.
  R6  Upstream gradients: under "none" one value per token for each output
      ([liger-435]: a non-scalar output needs an explicit per-element
      gradient); under "mean" one scalar per output, applied to the mean.
  R7  reduction="sum" sums each output over the valid tokens (the
      reduction modes the [liger-435] Summary refers to); its scalar upstream
      gradients apply undivided. With n = 0 the sums are 0.
  R8  Z-loss. The [liger-551] review names a fused "Z loss" without a
      formula; it is taken as the usual auxiliary term z_loss = lam * lse^2 per
      valid token (lam >= 0 a scale), computed on the capped logits.
  R9  Label smoothing. The [liger-551] review lists label smoothing among the
      fused options, again without a formula. The head exposes the building
      block uniform_ce = lse - (1/V) sum_j z'_j, the cross-entropy against the
      uniform distribution; the smoothed cross-entropy with weight eps is
      (1 - eps) * (-logprob) + eps * uniform_ce, which is how
      torch.nn.functional.cross_entropy defines label_smoothing.
  R10 Target (class) weights. The [liger-551] review lists target weights
      among the fused options and, for the weighted case, normalises by the
      sum of the weights of the non-ignored tokens instead of their count.
      Taken here as: an optional weight per class; a valid token i carries
      omega_i = class_weight[y_i]; under "mean" every output's mean is
      sum_i omega_i x_i / sum_i omega_i (0 when that sum is 0), under "sum"
      it is sum_i omega_i x_i, and the scalar upstream gradients reach token i
      multiplied by omega_i (and divided by the weight sum under "mean"). This
      is torch.nn.functional.cross_entropy's ``weight`` for the cross-entropy
      term, and the same per-token weight for the entropy and the auxiliary
      outputs. Per-token vectors stay unweighted; under "none" no weights are
      taken (a caller folds them into its per-token gradients).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "softcap",
    "softcap_grad",
    "logits",
    "row_stats",
    "forward",
    "dlogits",
    "backward",
    "dhidden_rows",
    "dweight_columns",
]

_ROW_BLOCK = 128


def _as_f64(a):
    return np.asarray(a, dtype=np.float64)


def softcap(z, c):
    """Gemma2 final-logit capping, z' = c * tanh(z / c).

    [liger-127] proposal: apply the capping steps right after the head matmul;
    discussion point 2: the cap is a scaling plus tanh, bounding z' to (-c, c).
    ``c <= 0`` disables the cap (reading R4).
    """
    if c is None or c <= 0:
        return z
    return c * np.tanh(z / c)


def softcap_grad(zc, c):
    """dz'/dz written through the capped value: 1 - (z'/c)^2.

    [liger-127] discussion point 3 and the closing suggestion: the gradient of
    the tanh cap enters the hidden and weight gradients by the chain rule;
    d/dx tanh(x) = 1 - tanh(x)^2 and tanh(z/c) = z'/c.
    """
    if c is None or c <= 0:
        return np.ones_like(zc)
    return 1.0 - (zc / c) ** 2


def logits(hidden_rows, weight, c=0.0):
    """Capped logits z' = cap(hidden @ weight) for a block of rows.

    [verl-462] "Equivalent compute logic": logits = hidden @ weight with both
    operands up-cast before the product (float32 there, float64 here); "API":
    hidden is [num_tokens, hidden_size], weight is [hidden_size, vocab_size].
    """
    z = _as_f64(hidden_rows) @ _as_f64(weight)
    return softcap(z, c)


def row_stats(zc):
    """Per-row logsumexp, S = sum_j p_j z'_j, entropy = lse - S, and p.

    [verl-462] "Equivalent compute logic": pd = softmax(logits),
    entropy = logsumexp(logits) - sum(pd * logits). The max shift inside the
    logsumexp is the usual exact rewrite that keeps exp finite.
    """
    m = zc.max(axis=1)
    lse = m + np.log(np.exp(zc - m[:, None]).sum(axis=1))
    p = np.exp(zc - lse[:, None])
    s = (p * zc).sum(axis=1)
    return lse, s, lse - s, p


def _valid_mask(labels, V, ignore_index):
    labels = np.asarray(labels, dtype=np.int64)
    valid = labels != ignore_index
    bad = valid & ((labels < 0) | (labels >= V))
    if bad.any():
        raise ValueError("label outside [0, V) that is not ignore_index (reading R5)")
    return labels, valid


_REDUCTIONS = ("none", "mean", "sum")
_OUTPUTS = ("logprob", "entropy", "uniform_ce", "z_loss")


def _token_weights(labels, valid, reduction, class_weight):
    """omega_i = class_weight[y_i] on valid tokens, 1 without class weights,
    0 on ignored tokens (reading R10)."""
    if class_weight is None:
        return valid.astype(np.float64)
    if reduction == "none":
        raise ValueError("class weights apply to the 'mean' and 'sum' reductions (reading R10)")
    cw = _as_f64(class_weight).reshape(-1)
    om = np.zeros(labels.shape[0])
    om[valid] = cw[labels[valid]]
    return om


def forward(hidden, weight, labels, ignore_index=-100, softcap_c=0.0,
            reduction="none", z_loss_scale=0.0, row_block=_ROW_BLOCK, class_weight=None):
    """Per-token lse, logprob, entropy, uniform_ce and z_loss, plus their
    reductions under "mean" (keys ``<output>_mean``) and "sum" (``<output>_sum``).

    [verl-462] "Equivalent compute logic" (lse and entropy per token;
    logprobs = -cross_entropy) with the cap of [liger-127], the ignore rule and
    the mean of [liger-551] (readings R1 to R4), per-token outputs under
    "none" as in [liger-435] Summary, the sum of R7, the two auxiliary
    outputs of R8 and R9 and the class weights of R10 (``weight_sum`` is
    the weight of the valid tokens, n without class weights).
    """
    if reduction not in _REDUCTIONS:
        raise ValueError("reduction must be 'none', 'mean' or 'sum'")
    N = hidden.shape[0]
    V = weight.shape[1]
    labels, valid = _valid_mask(labels, V, ignore_index)
    if class_weight is not None and _as_f64(class_weight).size != V:
        raise ValueError("class_weight needs one weight per class")
    omega = _token_weights(labels, valid, reduction, class_weight)
    w = _as_f64(weight)
    lse = np.zeros(N)
    lp = np.zeros(N)
    ent = np.zeros(N)
    uce = np.zeros(N)
    for r0 in range(0, N, row_block):
        rows = np.arange(r0, min(N, r0 + row_block))
        rows = rows[valid[rows]]
        if rows.size == 0:
            continue
        zc = logits(hidden[rows], w, softcap_c)
        l_, _, e_, _ = row_stats(zc)
        lse[rows] = l_
        ent[rows] = e_
        lp[rows] = zc[np.arange(rows.size), labels[rows]] - l_
        uce[rows] = l_ - zc.mean(axis=1)
    zl = z_loss_scale * lse * lse
    n = int(valid.sum())
    wsum = float(omega[valid].sum())
    out = {"lse": lse, "logprob": lp, "entropy": ent, "uniform_ce": uce, "z_loss": zl,
           "n_valid": n, "weight_sum": wsum}
    for name in _OUTPUTS:
        tot = float((omega[valid] * out[name][valid]).sum())
        if reduction == "mean":
            out[name + "_mean"] = tot / wsum if wsum != 0.0 else 0.0
        elif reduction == "sum":
            out[name + "_sum"] = tot
    return out


def _token_grads(labels, valid, reduction, class_weight, *grads):
    """Per-token upstream gradients of the outputs, in the order given.

    "none": one value per token ([liger-435], "Why we pass gradient to
    output.backward()"); None means zero. "mean": the scalar gradient of each
    mean, times omega_i / sum omega on valid tokens (omega_i = 1 without class
    weights, so 1/n: readings R3, R10). "sum": the scalar gradient of each
    sum, times omega_i (readings R7, R10). Ignored tokens get 0.
    """
    N = labels.shape[0]
    omega = _token_weights(labels, valid, reduction, class_weight)
    wsum = float(omega[valid].sum())

    def expand(g):
        if g is None:
            return np.zeros(N)
        g = _as_f64(g).reshape(-1)
        if reduction == "none":
            if g.size != N:
                raise ValueError("reduction='none' needs one gradient per token")
            return g.copy()
        if g.size != 1:
            raise ValueError("reduction='%s' needs one scalar gradient" % reduction)
        if reduction == "sum":
            return g[0] * omega
        return g[0] * omega / wsum if wsum != 0.0 else np.zeros(N)

    out = []
    for g in grads:
        e = expand(g)
        e[~valid] = 0.0
        out.append(e)
    return tuple(out)


def dlogits(zc, labels_rows, lse, s, gbar, ebar, c, gunif=None, gzl=None, z_loss_scale=0.0):
    """Gradient of g_bar * logprob + e_bar * entropy + g_u * uniform_ce +
    g_z * z_loss w.r.t. the raw logits z.

    Derivation from the definitions of [verl-462] (chain rule, float64):
      d logprob / d z'_j    = [j == y] - p_j
      d entropy / d z'_j    = -p_j (z'_j - S),  S = sum_k p_k z'_k
      d uniform_ce / d z'_j = p_j - 1/V                      (reading R9)
      d z_loss / d z'_j     = 2 lam lse p_j                  (reading R8)
    then the cap's chain rule factor 1 - (z'/c)^2 ([liger-127]).
    """
    V = zc.shape[1]
    p = np.exp(zc - lse[:, None])
    onehot = np.zeros_like(zc)
    hit = gbar != 0.0
    onehot[np.arange(zc.shape[0])[hit], labels_rows[hit]] = 1.0
    dzc = gbar[:, None] * (onehot - p) - ebar[:, None] * p * (zc - s[:, None])
    if gunif is not None:
        dzc = dzc + gunif[:, None] * (p - 1.0 / V)
    if gzl is not None:
        dzc = dzc + (2.0 * z_loss_scale * gzl * lse)[:, None] * p
    return dzc * softcap_grad(zc, c)


def _block_dz(hidden, w, labels, rows, grads, softcap_c, z_loss_scale):
    gb, eb, gu, gz = grads
    zc = logits(hidden[rows], w, softcap_c)
    l_, s_, _, _ = row_stats(zc)
    return dlogits(zc, labels[rows], l_, s_, gb[rows], eb[rows], softcap_c,
                   gu[rows], gz[rows], z_loss_scale)


def backward(hidden, weight, labels, ignore_index=-100, softcap_c=0.0,
             reduction="none", grad_logprob=None, grad_entropy=None,
             grad_uniform_ce=None, grad_z_loss=None, z_loss_scale=0.0,
             row_block=_ROW_BLOCK, class_weight=None):
    """dHidden [N,H] and dWeight [H,V] in float64.

    Recomputes the logits of each row block, forms dlogits (see ``dlogits``)
    and contracts it: dH = dZ @ weight^T and dW = hidden^T @ dZ, the grad_input
    and grad_weights of [liger-127] discussion point 3.
    """
    N, H = hidden.shape
    V = weight.shape[1]
    labels, valid = _valid_mask(labels, V, ignore_index)
    grads = _token_grads(labels, valid, reduction, class_weight, grad_logprob, grad_entropy,
                         grad_uniform_ce, grad_z_loss)
    w = _as_f64(weight)
    dh = np.zeros((N, H))
    dw = np.zeros((H, V))
    for r0 in range(0, N, row_block):
        rows = np.arange(r0, min(N, r0 + row_block))
        rows = rows[valid[rows]]
        if rows.size == 0:
            continue
        dz = _block_dz(hidden, w, labels, rows, grads, softcap_c, z_loss_scale)
        dh[rows] = dz @ w.T
        dw += _as_f64(hidden[rows]).T @ dz
    return dh, dw


def dhidden_rows(hidden, weight, labels, rows, ignore_index=-100, softcap_c=0.0,
                 reduction="none", grad_logprob=None, grad_entropy=None,
                 grad_uniform_ce=None, grad_z_loss=None, z_loss_scale=0.0, class_weight=None):
    """Rows ``rows`` of dHidden. A row of dH depends only on its own token
    (and on n under "mean", so all labels are passed)."""
    V = weight.shape[1]
    labels, valid = _valid_mask(labels, V, ignore_index)
    grads = _token_grads(labels, valid, reduction, class_weight, grad_logprob, grad_entropy,
                         grad_uniform_ce, grad_z_loss)
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros((rows.size, hidden.shape[1]))
    keep = valid[rows]
    if keep.any():
        w = _as_f64(weight)
        dz = _block_dz(hidden, w, labels, rows[keep], grads, softcap_c, z_loss_scale)
        out[keep] = dz @ w.T
    return out


def dweight_columns(hidden, weight, labels, cols, ignore_index=-100, softcap_c=0.0,
                    reduction="none", grad_logprob=None, grad_entropy=None,
                    grad_uniform_ce=None, grad_z_loss=None, z_loss_scale=0.0,
                    row_block=_ROW_BLOCK, class_weight=None):
    """Columns ``cols`` of dWeight, i.e. dW[:, cols] = hidden^T @ dZ[:, cols].

    Each column sums over every token, and each token's dZ needs its full
    softmax row, so this costs a full forward pass."""
    N, H = hidden.shape
    V = weight.shape[1]
    labels, valid = _valid_mask(labels, V, ignore_index)
    grads = _token_grads(labels, valid, reduction, class_weight, grad_logprob, grad_entropy,
                         grad_uniform_ce, grad_z_loss)
    cols = np.asarray(cols, dtype=np.int64)
    w = _as_f64(weight)
    out = np.zeros((H, cols.size))
    for r0 in range(0, N, row_block):
        rows = np.arange(r0, min(N, r0 + row_block))
        rows = rows[valid[rows]]
        if rows.size == 0:
            continue
        dz = _block_dz(hidden, w, labels, rows, grads, softcap_c, z_loss_scale)
        out += _as_f64(hidden[rows]).T @ dz[:, cols]
    return out
