"""Planted mistakes in the oracle must be caught by at least one pin.

Each case swaps one piece of the oracle (on the CPU, through monkeypatch) for
a plausible wrong version: a dropped term, a flipped sign, an index off by
one, a wrong normaliser, a transposed operand. The pins of
tests/oracle_pins.py are then rerun and at least one must fail.
"""
import numpy as np
import pytest

import oracle.flce_oracle as O
import oracle_pins as P


def _entropy_sign(mp):
    orig = O.dlogits

    def bad(zc, y, lse, s, g, e, c, *rest):
        return orig(zc, y, lse, s, g, -e, c, *rest)
    mp.setattr(O, "dlogits", bad)


def _drop_cap_factor(mp):
    mp.setattr(O, "softcap_grad", lambda zc, c: np.ones_like(zc))


def _cap_factor_not_squared(mp):
    mp.setattr(O, "softcap_grad", lambda zc, c: np.ones_like(zc) if c <= 0 else 1.0 - np.abs(zc / c))


def _label_off_by_one(mp):
    orig = O.forward

    def bad(h, w, y, *a, **k):
        y = np.asarray(y).copy()
        v = y != -100
        y[v] = (y[v] + 1) % w.shape[1]
        return orig(h, w, y, *a, **k)
    mp.setattr(O, "forward", bad)


def _entropy_plus(mp):
    orig = O.row_stats

    def bad(zc):
        lse, s, ent, p = orig(zc)
        return lse, s, lse + s, p
    mp.setattr(O, "row_stats", bad)


def _mean_over_all_tokens(mp):
    orig = O.forward

    def bad(h, w, y, *a, **k):
        out = orig(h, w, y, *a, **k)
        if "logprob_mean" in out:
            n = len(y)
            out["logprob_mean"] = float(out["logprob"].sum() / n)
            out["entropy_mean"] = float(out["entropy"].sum() / n)
        return out
    mp.setattr(O, "forward", bad)


def _no_cap_in_logits(mp):
    mp.setattr(O, "softcap", lambda z, c: z)


def _entropy_grad_uses_lse(mp):
    orig = O.dlogits

    def bad(zc, y, lse, s, g, e, c, *rest):
        return orig(zc, y, lse, lse, g, e, c, *rest)
    mp.setattr(O, "dlogits", bad)


def _onehot_dropped(mp):
    orig = O.dlogits

    def bad(zc, y, lse, s, g, e, c, *rest):
        p = np.exp(zc - lse[:, None])
        d = -g[:, None] * p - e[:, None] * p * (zc - s[:, None])
        return d * O.softcap_grad(zc, c)
    mp.setattr(O, "dlogits", bad)


def _transposed_weight_in_dh(mp):
    orig = O._block_dz

    def bad(*args):
        # reverses the vocabulary order of dZ: as if W^T were indexed backwards
        return orig(*args)[:, ::-1]
    mp.setattr(O, "_block_dz", bad)


def _uniform_grad_drops_inv_v(mp):
    orig = O.dlogits

    def bad(zc, y, lse, s, g, e, c, gu=None, gz=None, lam=0.0):
        d = orig(zc, y, lse, s, g, e, c, None, gz, lam)
        if gu is not None:
            d = d + (gu[:, None] * np.exp(zc - lse[:, None])) * O.softcap_grad(zc, c)
        return d
    mp.setattr(O, "dlogits", bad)


def _zloss_grad_no_factor2(mp):
    orig = O.dlogits

    def bad(zc, y, lse, s, g, e, c, gu=None, gz=None, lam=0.0):
        return orig(zc, y, lse, s, g, e, c, gu, gz, lam / 2)
    mp.setattr(O, "dlogits", bad)


def _sum_divides_by_n(mp):
    orig = O.forward

    def bad(h, w, y, *a, **k):
        out = orig(h, w, y, *a, **k)
        n = out["n_valid"]
        for key in list(out):
            if key.endswith("_sum") and n:
                out[key] = out[key] / n
        return out
    mp.setattr(O, "forward", bad)


def _uniform_ce_sums_logits(mp):
    orig = O.forward

    def bad(h, w, y, *a, **k):
        out = orig(h, w, y, *a, **k)
        V = w.shape[1]
        valid = np.asarray(y) != -100
        out["uniform_ce"] = np.where(valid, out["lse"] - V * (out["lse"] - out["uniform_ce"]), 0.0)
        return out
    mp.setattr(O, "forward", bad)


def _weighted_mean_divides_by_n(mp):
    orig = O.forward

    def bad(h, w, y, *a, **k):
        out = orig(h, w, y, *a, **k)
        n, ws = out["n_valid"], out["weight_sum"]
        for key in list(out):
            if key.endswith("_mean") and n and ws:
                out[key] = out[key] * ws / n
        return out
    mp.setattr(O, "forward", bad)


def _grads_ignore_class_weights(mp):
    orig = O._token_grads

    def bad(labels, valid, reduction, class_weight, *grads):
        if class_weight is None or reduction != "mean":
            return orig(labels, valid, reduction, class_weight, *grads)
        n = int(valid.sum())
        out = orig(labels, valid, reduction, None, *grads)
        ws = float(np.asarray(class_weight)[labels[valid]].sum())
        return tuple(g * n / ws if ws else g for g in out)
    mp.setattr(O, "_token_grads", bad)


def _class_weight_of_next_class(mp):
    orig = O._token_weights

    def bad(labels, valid, reduction, class_weight):
        if class_weight is None:
            return orig(labels, valid, reduction, class_weight)
        return orig(labels, valid, reduction, np.roll(np.asarray(class_weight), -1))
    mp.setattr(O, "_token_weights", bad)


MUTATIONS = [_weighted_mean_divides_by_n, _grads_ignore_class_weights,
             _class_weight_of_next_class, _entropy_sign, _drop_cap_factor, _cap_factor_not_squared, _label_off_by_one,
             _entropy_plus, _mean_over_all_tokens, _no_cap_in_logits, _entropy_grad_uses_lse,
             _onehot_dropped, _transposed_weight_in_dh, _uniform_grad_drops_inv_v,
             _zloss_grad_no_factor2, _sum_divides_by_n, _uniform_ce_sums_logits]


def test_pins_pass_unmutated():
    assert P.failing_pins() == []


@pytest.mark.parametrize("mutate", MUTATIONS, ids=lambda f: f.__name__.strip("_"))
def test_mutation_caught(mutate, monkeypatch):
    mutate(monkeypatch)
    bad = P.failing_pins()
    assert bad, f"planted mistake {mutate.__name__} passed every pin"
