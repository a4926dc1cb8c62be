"""Pins for the float64 oracle: checks against facts fixed outside the oracle.

Each pin returns the largest error it saw (0 is perfect) and a tolerance, so
the same pins serve the plain tests and the planted-mistake tests, which
mutate the oracle and require that some pin fails.

Sources of truth used here, none of which is the oracle's own code path:
  * closed forms of the definitions (zero weight, one dominant logit, k tied
    logits, zero-weight gradient);
  * invariants of softmax, entropy and the tanh cap;
  * torch float64 library routines on the CPU (logsumexp, cross_entropy with
    ignore_index, reductions, label_smoothing and class weights,
    Categorical.entropy, autograd);
  * central finite differences of the oracle's forward.
"""
from __future__ import annotations

import math

import numpy as np
import torch
import torch.nn.functional as F

import oracle.flce_oracle as O

TOL_CLOSED = 1e-10
TOL_LIB = 1e-9
TOL_FD = 1e-6


def _rand_case(seed, N=5, H=6, V=9, wstd=0.7, ignore_rows=(), c=0.0):
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((N, H))
    w = rng.standard_normal((H, V)) * wstd
    y = rng.integers(0, V, size=N).astype(np.int64)
    for r in ignore_rows:
        y[r] = -100
    return h, w, y, c


# ---------------------------------------------------------------- closed forms

def pin_zero_weight_forward():
    """W = 0: every logit is 0, so lse = entropy = ln V and logprob = -ln V."""
    err = 0.0
    for V in (7, 4096, 32000):
        h = np.random.default_rng(V).standard_normal((3, 2))
        w = np.zeros((2, V))
        y = np.array([0, V - 1, V // 2])
        out = O.forward(h, w, y)
        lnV = math.log(V)
        err = max(err, np.abs(out["lse"] - lnV).max(), np.abs(out["entropy"] - lnV).max(),
                  np.abs(out["logprob"] + lnV).max())
    return err, TOL_CLOSED


def pin_dominant_logit():
    """One logit L, the other V-1 at 0: lse = ln(e^L + V - 1),
    entropy = lse - L e^L / (e^L + V - 1), logprob = L - lse at the label,
    -lse elsewhere."""
    err = 0.0
    for V, L, j in ((11, 3.0, 4), (1000, 9.5, 0), (50, 40.0, 49)):
        w = np.zeros((1, V))
        w[0, j] = L
        h = np.ones((2, 1))
        y = np.array([j, (j + 1) % V])
        out = O.forward(h, w, y)
        den = math.exp(L) + V - 1
        lse = math.log(den)
        ent = lse - L * math.exp(L) / den
        err = max(err, abs(out["lse"][0] - lse) / max(1, lse), abs(out["entropy"][0] - ent),
                  abs(out["logprob"][0] - (L - lse)), abs(out["logprob"][1] + lse))
    return err, TOL_CLOSED


def pin_k_tied():
    """k logits at L, the rest 0: lse = ln(k e^L + V - k); entropy tends to
    ln k as L grows (the exact form is checked)."""
    err = 0.0
    for V, k, L in ((20, 3, 2.0), (4096, 17, 60.0), (300, 300, 1.5)):
        w = np.zeros((1, V))
        w[0, :k] = L
        h = np.ones((1, 1))
        out = O.forward(h, w, np.array([0]))
        den = k * math.exp(L) + (V - k)
        lse = math.log(den)
        ent = lse - k * L * math.exp(L) / den
        err = max(err, abs(out["lse"][0] - lse) / max(1, lse), abs(out["entropy"][0] - ent))
        if L >= 60:
            err = max(err, abs(out["entropy"][0] - math.log(k)))
    return err, TOL_CLOSED


def pin_zero_weight_grads():
    """W = 0: p = 1/V and z' = S = 0, so the entropy term vanishes,
    dH = 0 and dW[k, j] = sum_i h_ik g_i ([j == y_i] - 1/V)."""
    rng = np.random.default_rng(5)
    N, H, V = 6, 4, 10
    h = rng.standard_normal((N, H))
    w = np.zeros((H, V))
    y = rng.integers(0, V, size=N)
    y[2] = -100
    g = rng.standard_normal(N)
    e = rng.standard_normal(N)
    dh, dw = O.backward(h, w, y, grad_logprob=g, grad_entropy=e)
    ref = np.zeros((H, V))
    for i in range(N):
        if y[i] == -100:
            continue
        t = -np.full(V, 1.0 / V)
        t[y[i]] += 1.0
        ref += np.outer(h[i], g[i] * t)
    return max(np.abs(dh).max(), np.abs(dw - ref).max()), TOL_CLOSED


# ---------------------------------------------------------------- invariants

def pin_invariants():
    """0 <= entropy <= ln V, logprob <= 0, lse >= max z', ignored rows 0."""
    worst = 0.0
    for seed, c in ((1, 0.0), (2, 3.0)):
        h, w, y, _ = _rand_case(seed, N=40, H=16, V=33, wstd=1.5, ignore_rows=(3, 7), c=c)
        out = O.forward(h, w, y, softcap_c=c)
        zc = O.softcap(h @ w, c)
        valid = y != -100
        lnV = math.log(33)
        ent = out["entropy"][valid]
        worst = max(worst, max(0.0, -ent.min()), max(0.0, ent.max() - lnV),
                    max(0.0, out["logprob"].max()),
                    max(0.0, (zc.max(axis=1) - out["lse"])[valid].max()),
                    np.abs(out["lse"][~valid]).max(), np.abs(out["entropy"][~valid]).max(),
                    np.abs(out["logprob"][~valid]).max())
    return worst, 1e-12


def pin_softcap_bounds():
    """|z'| < c; the cap is odd; z' ~ z - z^3/(3c^2) for small z; a huge c
    leaves logits unchanged; large logits saturate lse below c + ln V."""
    z = np.linspace(-200, 200, 4001)
    c = 30.0
    zc = O.softcap(z, c)
    err = max(0.0, np.abs(zc).max() - c)
    err = max(err, np.abs(zc + O.softcap(-z, c)).max())
    zs = np.linspace(-0.3, 0.3, 61)
    err = max(err, np.abs(O.softcap(zs, c) - (zs - zs ** 3 / (3 * c * c))).max())
    h, w, y, _ = _rand_case(9, N=4, H=6, V=9, wstd=1.0)
    a = O.forward(h, w, y, softcap_c=1e6)
    b = O.forward(h, w, y, softcap_c=0.0)
    err = max(err, np.abs(a["lse"] - b["lse"]).max(), np.abs(a["entropy"] - b["entropy"]).max())
    h, w, y, _ = _rand_case(10, N=4, H=6, V=9, wstd=100.0)
    o = O.forward(h, w, y, softcap_c=2.0)
    err = max(err, max(0.0, (o["lse"] - (2.0 + math.log(9))).max()))
    return err, 1e-9


def pin_softcap_derivative():
    """softcap_grad(softcap(z)) equals the central difference of softcap."""
    z = np.linspace(-90, 90, 721)
    c, step = 30.0, 1e-5
    fd = (O.softcap(z + step, c) - O.softcap(z - step, c)) / (2 * step)
    return np.abs(O.softcap_grad(O.softcap(z, c), c) - fd).max(), 1e-8


def pin_mean_empty():
    """reduction='mean' with every token ignored: means and gradients are 0."""
    h, w, y, _ = _rand_case(11, N=4)
    y[:] = -100
    out = O.forward(h, w, y, reduction="mean")
    dh, dw = O.backward(h, w, y, reduction="mean", grad_logprob=[1.0], grad_entropy=[1.0])
    return max(abs(out["logprob_mean"]), abs(out["entropy_mean"]), np.abs(dh).max(),
               np.abs(dw).max()), 0.0


def pin_dz_row_sums():
    """Without a cap each row of dlogits sums to 0, so each row of dW sums to
    0 over the vocabulary."""
    h, w, y, _ = _rand_case(12, N=7, H=5, V=11, ignore_rows=(1,))
    g = np.random.default_rng(1).standard_normal(7)
    e = np.random.default_rng(2).standard_normal(7)
    _, dw = O.backward(h, w, y, grad_logprob=g, grad_entropy=e)
    return np.abs(dw.sum(axis=1)).max(), 1e-12


# ---------------------------------------------------------------- library

def _torch_forward(h, w, y, c, ii=-100):
    z = torch.as_tensor(h, dtype=torch.float64) @ torch.as_tensor(w, dtype=torch.float64)
    if c > 0:
        z = c * torch.tanh(z / c)
    yt = torch.as_tensor(y)
    lse = torch.logsumexp(z, dim=-1)
    lp = -F.cross_entropy(z, yt, ignore_index=ii, reduction="none")
    ent = torch.distributions.Categorical(logits=z).entropy()
    return z, lse, lp, ent


def pin_library_forward():
    """lse vs torch.logsumexp, logprob vs -F.cross_entropy (ignore_index,
    'none' and 'mean'), entropy vs Categorical(logits).entropy()."""
    err = 0.0
    for seed, c in ((20, 0.0), (21, 2.5)):
        h, w, y, _ = _rand_case(seed, N=12, H=8, V=15, wstd=1.2, ignore_rows=(0, 5), c=c)
        out = O.forward(h, w, y, softcap_c=c, reduction="mean")
        _, lse, lp, ent = _torch_forward(h, w, y, c)
        valid = y != -100
        err = max(err, np.abs(out["lse"][valid] - lse.numpy()[valid]).max(),
                  np.abs(out["logprob"] - lp.numpy()).max(),
                  np.abs(out["entropy"][valid] - ent.numpy()[valid]).max())
        zt = torch.as_tensor(O.softcap(h @ w, c))
        mean_ce = F.cross_entropy(zt, torch.as_tensor(y), ignore_index=-100, reduction="mean")
        err = max(err, abs(out["logprob_mean"] + mean_ce.item()),
                  abs(out["entropy_mean"] - ent.numpy()[valid].mean()))
    return err, TOL_LIB


def pin_library_grads():
    """Oracle gradients vs torch autograd (float64) of the same objective."""
    err = 0.0
    for seed, c, red in ((30, 0.0, "none"), (31, 2.0, "none"), (32, 0.0, "mean"), (33, 3.0, "mean")):
        h, w, y, _ = _rand_case(seed, N=6, H=5, V=8, wstd=1.0, ignore_rows=(2,), c=c)
        rng = np.random.default_rng(seed + 100)
        if red == "none":
            g = rng.standard_normal(6)
            e = rng.standard_normal(6)
        else:
            g = np.array([0.7])
            e = np.array([-1.3])
        ht = torch.tensor(h, requires_grad=True)
        wt = torch.tensor(w, requires_grad=True)
        z = ht @ wt
        if c > 0:
            z = c * torch.tanh(z / c)
        yt = torch.as_tensor(y)
        valid = yt != -100
        lp = -F.cross_entropy(z, yt, ignore_index=-100, reduction="none")
        ent = torch.distributions.Categorical(logits=z).entropy() * valid
        if red == "none":
            loss = (torch.as_tensor(g) * lp).sum() + (torch.as_tensor(e) * ent).sum()
        else:
            n = valid.sum()
            loss = g[0] * lp.sum() / n + e[0] * ent.sum() / n
        loss.backward()
        dh, dw = O.backward(h, w, y, softcap_c=c, reduction=red, grad_logprob=g, grad_entropy=e)
        scale = max(np.abs(ht.grad.numpy()).max(), np.abs(wt.grad.numpy()).max())
        err = max(err, np.abs(dh - ht.grad.numpy()).max() / scale,
                  np.abs(dw - wt.grad.numpy()).max() / scale)
    return err, TOL_LIB


# ---------------------------------------------------------------- finite differences

def _objective(h, w, y, c, red, g, e):
    out = O.forward(h, w, y, softcap_c=c, reduction=red)
    if red == "none":
        return float((g * out["logprob"]).sum() + (e * out["entropy"]).sum())
    return g[0] * out["logprob_mean"] + e[0] * out["entropy_mean"]


def pin_finite_differences():
    """Central differences (float64, step 1e-6) of the forward objective
    g.logprob + e.entropy vs the oracle's backward, for none/mean, cap off/on,
    with an ignored token."""
    worst = 0.0
    step = 1e-6
    for seed, c, red in ((40, 0.0, "none"), (41, 2.0, "none"), (42, 0.0, "mean"), (43, 1.5, "mean")):
        h, w, y, _ = _rand_case(seed, N=4, H=3, V=6, wstd=1.0, ignore_rows=(1,), c=c)
        rng = np.random.default_rng(seed + 7)
        if red == "none":
            g = rng.standard_normal(4)
            e = rng.standard_normal(4)
        else:
            g = np.array([1.1])
            e = np.array([-0.8])
        dh, dw = O.backward(h, w, y, softcap_c=c, reduction=red, grad_logprob=g, grad_entropy=e)
        fdh = np.zeros_like(h)
        fdw = np.zeros_like(w)
        for arr, out in ((h, fdh), (w, fdw)):
            for idx in np.ndindex(arr.shape):
                old = arr[idx]
                arr[idx] = old + step
                fp = _objective(h, w, y, c, red, g, e)
                arr[idx] = old - step
                fm = _objective(h, w, y, c, red, g, e)
                arr[idx] = old
                out[idx] = (fp - fm) / (2 * step)
        scale = max(np.abs(fdh).max(), np.abs(fdw).max())
        worst = max(worst, np.abs(dh - fdh).max() / scale, np.abs(dw - fdw).max() / scale)
    return worst, TOL_FD


def pin_sampled_helpers():
    """dhidden_rows / dweight_columns agree with the full backward (they are
    the same definition restricted to rows / columns)."""
    h, w, y, _ = _rand_case(50, N=9, H=4, V=13, ignore_rows=(4,), c=2.0)
    g = np.array([0.9])
    e = np.array([0.4])
    dh, dw = O.backward(h, w, y, softcap_c=2.0, reduction="mean", grad_logprob=g, grad_entropy=e)
    rows = np.array([0, 4, 8])
    cols = np.array([1, 12])
    a = O.dhidden_rows(h, w, y, rows, softcap_c=2.0, reduction="mean", grad_logprob=g, grad_entropy=e)
    b = O.dweight_columns(h, w, y, cols, softcap_c=2.0, reduction="mean", grad_logprob=g,
                          grad_entropy=e, row_block=4)
    return max(np.abs(a - dh[rows]).max(), np.abs(b - dw[:, cols]).max()), 1e-12


# ---------------------------------------------------------------- auxiliary outputs

def pin_aux_closed_forms():
    """W = 0: every logit is 0, so uniform_ce = ln V and z_loss = lam (ln V)^2;
    on random logits 0 <= lse - max z' <= uniform_ce <= lse - min z'."""
    err = 0.0
    for V in (7, 4096):
        h = np.random.default_rng(V + 1).standard_normal((3, 2))
        out = O.forward(h, np.zeros((2, V)), np.array([0, V - 1, 1]), z_loss_scale=0.25)
        lnV = math.log(V)
        err = max(err, np.abs(out["uniform_ce"] - lnV).max(),
                  np.abs(out["z_loss"] - 0.25 * lnV * lnV).max())
    h, w, y, c = _rand_case(60, N=10, H=6, V=11, wstd=1.5, ignore_rows=(3,), c=2.0)
    out = O.forward(h, w, y, softcap_c=c)
    zc = O.softcap(h @ w, c)
    valid = y != -100
    u = out["uniform_ce"][valid]
    lo = out["lse"][valid] - zc[valid].max(axis=1)
    hi = out["lse"][valid] - zc[valid].min(axis=1)
    viol = max(0.0, (lo - u).max(), (u - hi).max(), -lo.min())
    return max(err, viol, np.abs(out["uniform_ce"][~valid]).max()), TOL_CLOSED


def pin_library_label_smoothing():
    """(1 - eps) logprob - eps uniform_ce equals -F.cross_entropy(...,
    label_smoothing=eps) per token ('none') and for 'sum' and 'mean', with an
    ignored token, cap off and on."""
    err = 0.0
    for seed, c, eps in ((61, 0.0, 0.1), (62, 2.5, 0.3)):
        h, w, y, _ = _rand_case(seed, N=12, H=8, V=15, wstd=1.2, ignore_rows=(0, 5), c=c)
        zt = torch.as_tensor(O.softcap(h @ w, c))
        yt = torch.as_tensor(y)
        for red in ("none", "sum", "mean"):
            out = O.forward(h, w, y, softcap_c=c, reduction=red)
            ref = -F.cross_entropy(zt, yt, ignore_index=-100, label_smoothing=eps, reduction=red)
            if red == "none":
                mine = (1 - eps) * out["logprob"] - eps * out["uniform_ce"]
                err = max(err, np.abs(mine - ref.numpy()).max())
            else:
                mine = (1 - eps) * out["logprob_" + red] - eps * out["uniform_ce_" + red]
                err = max(err, abs(mine - ref.item()))
    return err, TOL_LIB


def pin_library_sum():
    """'sum': logprob_sum = -F.cross_entropy(..., reduction='sum'),
    entropy_sum = sum of Categorical(logits).entropy() over valid tokens,
    z_loss_sum = lam * sum of torch.logsumexp^2 over valid tokens."""
    err = 0.0
    for seed, c in ((63, 0.0), (64, 1.7)):
        h, w, y, _ = _rand_case(seed, N=10, H=7, V=13, wstd=1.1, ignore_rows=(2, 9), c=c)
        out = O.forward(h, w, y, softcap_c=c, reduction="sum", z_loss_scale=0.3)
        z, lse, lp, ent = _torch_forward(h, w, y, c)
        valid = y != -100
        ce_sum = F.cross_entropy(z, torch.as_tensor(y), ignore_index=-100, reduction="sum").item()
        err = max(err, abs(out["logprob_sum"] + ce_sum),
                  abs(out["entropy_sum"] - ent.numpy()[valid].sum()),
                  abs(out["z_loss_sum"] - 0.3 * (lse.numpy()[valid] ** 2).sum()))
    return err, TOL_LIB


def pin_library_aux_grads():
    """Gradients vs torch autograd (float64): of
    F.cross_entropy(..., label_smoothing=eps, reduction='sum') (= the oracle's
    backward with grad_logprob = -(1 - eps), grad_uniform_ce = eps under
    'sum') and of lam * sum torch.logsumexp(z')^2 (grad_z_loss = 1), cap off
    and on, with an ignored token."""
    err = 0.0
    for seed, c, eps, lam in ((65, 0.0, 0.2, 0.1), (66, 2.0, 0.05, 0.7)):
        h, w, y, _ = _rand_case(seed, N=6, H=5, V=8, wstd=1.0, ignore_rows=(3,), c=c)
        ht = torch.tensor(h, requires_grad=True)
        wt = torch.tensor(w, requires_grad=True)
        z = ht @ wt
        if c > 0:
            z = c * torch.tanh(z / c)
        yt = torch.as_tensor(y)
        valid = (yt != -100).to(torch.float64)
        loss = F.cross_entropy(z, yt, ignore_index=-100, label_smoothing=eps, reduction="sum")
        loss = loss + lam * (torch.logsumexp(z, dim=-1) ** 2 * valid).sum()
        loss.backward()
        dh, dw = O.backward(h, w, y, softcap_c=c, reduction="sum", grad_logprob=np.array([-(1 - eps)]),
                            grad_uniform_ce=np.array([eps]), grad_z_loss=np.array([1.0]),
                            z_loss_scale=lam)
        scale = max(np.abs(ht.grad.numpy()).max(), np.abs(wt.grad.numpy()).max())
        err = max(err, np.abs(dh - ht.grad.numpy()).max() / scale,
                  np.abs(dw - wt.grad.numpy()).max() / scale)
    return err, TOL_LIB


def _aux_objective(h, w, y, c, red, gs, lam):
    out = O.forward(h, w, y, softcap_c=c, reduction=red, z_loss_scale=lam)
    names = ("logprob", "entropy", "uniform_ce", "z_loss")
    if red == "none":
        return float(sum((g * out[k]).sum() for g, k in zip(gs, names)))
    return float(sum(g[0] * out[k + "_" + red] for g, k in zip(gs, names)))


def pin_aux_finite_differences():
    """Central differences of g.logprob + e.entropy + u.uniform_ce + q.z_loss
    (none / sum / mean, cap off and on, an ignored token) vs the backward."""
    worst = 0.0
    step = 1e-6
    for seed, c, red, lam in ((67, 0.0, "none", 0.2), (68, 2.0, "sum", 0.5), (69, 1.5, "mean", 0.3)):
        h, w, y, _ = _rand_case(seed, N=4, H=3, V=6, wstd=1.0, ignore_rows=(2,), c=c)
        rng = np.random.default_rng(seed + 11)
        gs = [rng.standard_normal(4) if red == "none" else rng.standard_normal(1) for _ in range(4)]
        dh, dw = O.backward(h, w, y, softcap_c=c, reduction=red, grad_logprob=gs[0],
                            grad_entropy=gs[1], grad_uniform_ce=gs[2], grad_z_loss=gs[3],
                            z_loss_scale=lam)
        fdh = np.zeros_like(h)
        fdw = np.zeros_like(w)
        for arr, out in ((h, fdh), (w, fdw)):
            for idx in np.ndindex(arr.shape):
                old = arr[idx]
                arr[idx] = old + step
                fp = _aux_objective(h, w, y, c, red, gs, lam)
                arr[idx] = old - step
                fm = _aux_objective(h, w, y, c, red, gs, lam)
                arr[idx] = old
                out[idx] = (fp - fm) / (2 * step)
        scale = max(np.abs(fdh).max(), np.abs(fdw).max())
        worst = max(worst, np.abs(dh - fdh).max() / scale, np.abs(dw - fdw).max() / scale)
    return worst, TOL_FD


# ---------------------------------------------------------------- class weights (reading R10)

def _class_weights(seed, V, zero=()):
    cw = np.random.default_rng(seed).uniform(0.2, 3.0, size=V)
    for j in zero:
        cw[j] = 0.0
    return cw


def pin_library_class_weights():
    """Class weights: logprob_mean = -F.cross_entropy(weight=cw, 'mean') and
    logprob_sum = -F.cross_entropy(weight=cw, 'sum') (float64), cap off and
    on, with ignored tokens; the weight sum is sum_i cw[y_i] over valid
    tokens."""
    err = 0.0
    for seed, c in ((70, 0.0), (71, 2.2)):
        h, w, y, _ = _rand_case(seed, N=11, H=6, V=10, wstd=1.1, ignore_rows=(1, 7), c=c)
        cw = _class_weights(seed, 10)
        z, _, _, _ = _torch_forward(h, w, y, c)
        yt = torch.as_tensor(y)
        cwt = torch.as_tensor(cw)
        for red in ("mean", "sum"):
            out = O.forward(h, w, y, softcap_c=c, reduction=red, class_weight=cw)
            ref = F.cross_entropy(z, yt, weight=cwt, ignore_index=-100, reduction=red).item()
            err = max(err, abs(out["logprob_" + red] + ref))
        valid = y != -100
        err = max(err, abs(out["weight_sum"] - cw[y[valid]].sum()))
    return err, TOL_LIB


def _masked_labels(y, cw):
    """Labels whose class weight is 0 turned into ignore_index."""
    ym = y.copy()
    v = ym != -100
    ym[v & (cw[np.where(v, ym, 0)] == 0.0)] = -100
    return ym


def pin_class_weights_as_mask():
    """0/1 class weights give exactly the unweighted results with the
    weight-0 classes' tokens ignored (all four reduced outputs and both
    gradients, mean and sum); a constant weight k leaves every mean unchanged
    and multiplies every sum by k."""
    err = 0.0
    for seed, c in ((72, 0.0), (73, 1.8)):
        h, w, y, _ = _rand_case(seed, N=12, H=5, V=6, wstd=1.0, ignore_rows=(9,), c=c)
        y[:6] = np.arange(6)          # every class occurs
        mask = np.array([1.0, 0.0, 1.0, 1.0, 0.0, 1.0])
        ym = _masked_labels(y, mask)
        names = ("logprob", "entropy", "uniform_ce", "z_loss")
        g = [np.array([0.8]), np.array([-1.1]), np.array([0.3]), np.array([0.5])]
        for red in ("mean", "sum"):
            a = O.forward(h, w, y, softcap_c=c, reduction=red, z_loss_scale=0.2, class_weight=mask)
            b = O.forward(h, w, ym, softcap_c=c, reduction=red, z_loss_scale=0.2)
            err = max(err, max(abs(a[k + "_" + red] - b[k + "_" + red]) for k in names))
            kw = dict(softcap_c=c, reduction=red, grad_logprob=g[0], grad_entropy=g[1],
                      grad_uniform_ce=g[2], grad_z_loss=g[3], z_loss_scale=0.2)
            dha, dwa = O.backward(h, w, y, class_weight=mask, **kw)
            dhb, dwb = O.backward(h, w, ym, **kw)
            err = max(err, np.abs(dha - dhb).max(), np.abs(dwa - dwb).max())
            k = 2.5
            cst = np.full(6, k)
            a = O.forward(h, w, y, softcap_c=c, reduction=red, z_loss_scale=0.2, class_weight=cst)
            b = O.forward(h, w, y, softcap_c=c, reduction=red, z_loss_scale=0.2)
            f = 1.0 if red == "mean" else k
            err = max(err, max(abs(a[n + "_" + red] - f * b[n + "_" + red]) for n in names))
    return err, TOL_CLOSED


def pin_library_class_weight_grads():
    """Gradients vs torch autograd (float64) of
    g * -F.cross_entropy(weight=cw, ignore_index) + e * (class-weighted
    entropy), mean and sum, cap off and on."""
    err = 0.0
    for seed, c, red in ((74, 0.0, "mean"), (75, 2.0, "mean"), (76, 1.5, "sum")):
        h, w, y, _ = _rand_case(seed, N=7, H=4, V=8, wstd=1.0, ignore_rows=(3,), c=c)
        cw = _class_weights(seed, 8, zero=(int(y[0]),))
        ht = torch.tensor(h, requires_grad=True)
        wt = torch.tensor(w, requires_grad=True)
        z = ht @ wt
        if c > 0:
            z = c * torch.tanh(z / c)
        yt = torch.as_tensor(y)
        valid = yt != -100
        om = torch.where(valid, torch.as_tensor(cw)[torch.where(valid, yt, 0)], 0.0)
        ce = F.cross_entropy(z, yt, weight=torch.as_tensor(cw), ignore_index=-100, reduction=red)
        ent = (torch.distributions.Categorical(logits=z).entropy() * om).sum()
        if red == "mean":
            ent = ent / om.sum()
        g, e = 0.9, -1.4
        (-g * ce + e * ent).backward()
        dh, dw = O.backward(h, w, y, softcap_c=c, reduction=red, grad_logprob=np.array([g]),
                            grad_entropy=np.array([e]), class_weight=cw)
        scale = max(np.abs(ht.grad.numpy()).max(), np.abs(wt.grad.numpy()).max())
        err = max(err, np.abs(dh - ht.grad.numpy()).max() / scale,
                  np.abs(dw - wt.grad.numpy()).max() / scale)
    return err, TOL_LIB


def pin_class_weight_finite_differences():
    """Central differences of the class-weighted objective (mean and sum, cap
    off and on, an ignored token, z-loss) vs the backward."""
    worst = 0.0
    step = 1e-6
    names = ("logprob", "entropy", "uniform_ce", "z_loss")
    for seed, c, red in ((77, 0.0, "mean"), (78, 2.0, "sum")):
        h, w, y, _ = _rand_case(seed, N=4, H=3, V=5, wstd=1.0, ignore_rows=(1,), c=c)
        cw = _class_weights(seed, 5)
        rng = np.random.default_rng(seed + 3)
        gs = [rng.standard_normal(1) for _ in range(4)]

        def obj():
            out = O.forward(h, w, y, softcap_c=c, reduction=red, z_loss_scale=0.4, class_weight=cw)
            return float(sum(g[0] * out[k + "_" + red] for g, k in zip(gs, names)))

        dh, dw = O.backward(h, w, y, softcap_c=c, reduction=red, grad_logprob=gs[0],
                            grad_entropy=gs[1], grad_uniform_ce=gs[2], grad_z_loss=gs[3],
                            z_loss_scale=0.4, class_weight=cw)
        fdh = np.zeros_like(h)
        fdw = np.zeros_like(w)
        for arr, out in ((h, fdh), (w, fdw)):
            for idx in np.ndindex(arr.shape):
                old = arr[idx]
                arr[idx] = old + step
                fp = obj()
                arr[idx] = old - step
                fm = obj()
                arr[idx] = old
                out[idx] = (fp - fm) / (2 * step)
        scale = max(np.abs(fdh).max(), np.abs(fdw).max())
        worst = max(worst, np.abs(dh - fdh).max() / scale, np.abs(dw - fdw).max() / scale)
    return worst, TOL_FD


def pin_class_weights_zero_sum():
    """Every valid token's class weight 0: the means are 0 and the gradients 0
    (as for a mean over no tokens)."""
    h, w, y, _ = _rand_case(79, N=5, H=3, V=4, ignore_rows=(2,))
    cw = np.zeros(4)
    out = O.forward(h, w, y, reduction="mean", class_weight=cw)
    dh, dw = O.backward(h, w, y, reduction="mean", grad_logprob=np.array([1.0]),
                        grad_entropy=np.array([1.0]), class_weight=cw)
    err = max(abs(out["logprob_mean"]), abs(out["entropy_mean"]), np.abs(dh).max(), np.abs(dw).max())
    return err, 0.0


ALL_PINS = [
    pin_library_class_weights,
    pin_class_weights_as_mask,
    pin_library_class_weight_grads,
    pin_class_weight_finite_differences,
    pin_class_weights_zero_sum,
    pin_aux_closed_forms,
    pin_library_label_smoothing,
    pin_library_sum,
    pin_library_aux_grads,
    pin_aux_finite_differences,
    pin_zero_weight_forward,
    pin_dominant_logit,
    pin_k_tied,
    pin_zero_weight_grads,
    pin_invariants,
    pin_softcap_bounds,
    pin_softcap_derivative,
    pin_mean_empty,
    pin_dz_row_sums,
    pin_library_forward,
    pin_library_grads,
    pin_finite_differences,
    pin_sampled_helpers,
]


def failing_pins():
    """Names of the pins whose error exceeds their tolerance (or that raise)."""
    bad = []
    for pin in ALL_PINS:
        try:
            err, tol = pin()
            if not (err <= tol):
                bad.append(pin.__name__)
        except Exception:  # a mutated oracle may also break shapes
            bad.append(pin.__name__)
    return bad
