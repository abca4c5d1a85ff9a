"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each mutant is a copy of oracle/attention.py with one plausible slip (a
dropped term, a wrong sign or index, a transposed operand).  The pins of
test_oracle_forward.py / test_oracle_backward.py are re-run against the
mutant; at least one of them must fail.  This shows the pins constrain every
part of the definition, not only the parts a correct oracle happens to pass.
"""

import importlib.util
import os
import types

import pytest

import tests.test_oracle_backward as TB
import tests.test_oracle_forward as TF

SRC = os.path.join(os.path.dirname(os.path.dirname(__file__)), "oracle", "attention.py")

MUTANTS = {
    "scale dropped (fwd)": ("s = scale * (q[r] @ k.T)\n        p, lse[", "s = (q[r] @ k.T)\n        p, lse["),
    "causal excludes diagonal": ("cols[None, :] <= rows[:, None]", "cols[None, :] < rows[:, None]"),
    "causal reversed": ("cols[None, :] <= rows[:, None]", "cols[None, :] >= rows[:, None]"),
    "block mask transposed": ("bm[rows[:, None] // mask_block, cols[None, :] // mask_block]",
                              "bm[cols[None, :] // mask_block, rows[:, None] // mask_block]"),
    "max not subtracted in lse": ("m_safe + np.log(ell_safe)", "np.log(ell_safe)"),
    "no normalisation": ("p = e / ell_safe[:, None]", "p = e"),
    "mask not applied": ("s = np.where(ok, s, -np.inf)", "s = s"),
    "dS sign flipped": ("ds = p * (dp - d_row[:, None])", "ds = p * (d_row[:, None] - dp)"),
    "D term dropped": ("ds = p * (dp - d_row[:, None])", "ds = p * dp"),
    "dV transposed": ("dv += p.T @ do[r]", "dv += p @ do[r]"),
    "dK scale dropped": ("dk += scale * (ds.T @ q[r])", "dk += (ds.T @ q[r])"),
    "dQ uses V": ("dq[r] = scale * (ds @ k)", "dq[r] = scale * (ds @ v)"),
    "dP transposed operand": ("dp = do[r] @ v.T", "dp = v[r] @ do.T"),
}

PINS = [
    lambda: TF.test_brute_force_tiny(8, 8, True),
    lambda: TF.test_brute_force_tiny(5, 3, False),
    lambda: TF.test_brute_force_tiny_block_mask(),
    lambda: TF.test_identical_keys_give_mean_of_allowed_values(),
    lambda: TF.test_matches_torch_attention_fp64(True, True),
    lambda: TB.test_gradients_match_finite_differences(13, 8, True, True),
    lambda: TB.test_gradients_match_finite_differences(16, 8, False, False),
    lambda: TB.test_gradient_invariants(),
]


def load_mutant(old, new):
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation anchor not unique or missing: {old!r}"
    spec = importlib.util.spec_from_loader("oracle_mutant", loader=None)
    mod = importlib.util.module_from_spec(spec)
    exec(compile(text.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    mut = load_mutant(*MUTANTS[name])
    fake_pkg = types.SimpleNamespace(allowed=mut.allowed, rowsum_do_o=mut.rowsum_do_o,
                                     forward=mut.forward, backward=mut.backward)
    for mod in (TF, TB):
        monkeypatch.setattr(mod, "oracle", fake_pkg)
        if hasattr(mod, "forward_head"):
            monkeypatch.setattr(mod, "forward_head", mut.forward_head)
        if hasattr(mod, "backward_head"):
            monkeypatch.setattr(mod, "backward_head", mut.backward_head)
    caught = []
    for i, pin in enumerate(PINS):
        try:
            pin()
        except (AssertionError, ValueError, FloatingPointError, IndexError):
            caught.append(i)
    assert caught, f"no pin detects the mutant '{name}'"


def test_unmutated_copy_passes_all_pins(monkeypatch):
    mut = load_mutant("def allowed(", "def allowed(")
    fake_pkg = types.SimpleNamespace(allowed=mut.allowed, rowsum_do_o=mut.rowsum_do_o,
                                     forward=mut.forward, backward=mut.backward)
    for mod in (TF, TB):
        monkeypatch.setattr(mod, "oracle", fake_pkg)
        if hasattr(mod, "forward_head"):
            monkeypatch.setattr(mod, "forward_head", mut.forward_head)
        if hasattr(mod, "backward_head"):
            monkeypatch.setattr(mod, "backward_head", mut.backward_head)
    for pin in PINS:
        pin()
