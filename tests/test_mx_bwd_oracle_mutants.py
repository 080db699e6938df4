"""Plant plausible mistakes in the MXFP8 backward oracle (on the CPU) and
check that its pins catch each one.  A mutant is one textual change of a
function of oracle/mx_oracle.py, compiled into that module's namespace for
the duration of the test."""
import inspect
import textwrap

import pytest

from oracle import mx_oracle as mo
from tests import test_mx_bwd_oracle_pins as pins


def _mutate(fn, old, new):
    src = textwrap.dedent(inspect.getsource(fn))
    assert src.count(old) == 1, (fn.__name__, old)
    ns = dict(vars(mo))
    exec(compile(src.replace(old, new), mo.__file__, "exec"), ns)
    return ns[fn.__name__]


MUTANTS = {
    # which encoding each product reads
    "dv_from_rowwise_do": ("sequence_backward", "dv = pq.T @ doc", "dv = pq.T @ dor"),
    "dk_from_rowwise_q": ("sequence_backward", "dk = scale * (dsq.T @ qc)", "dk = scale * (dsq.T @ qr)"),
    "dq_from_rowwise_k": ("sequence_backward", "dq = scale * (dsk @ kc)", "dq = scale * (dsk @ kr)"),
    "delta_from_query_blocked_do": ("sequence_backward", "delta = (dor * o).sum(axis=1)",
                                    "delta = (doc * o).sum(axis=1)"),
    # arithmetic
    "ds_sign": ("sequence_backward", "ds = p * (dp - delta[:, None])", "ds = p * (delta[:, None] - dp)"),
    "dk_without_scale": ("sequence_backward", "dk = scale * (dsq.T @ qc)", "dk = (dsq.T @ qc)"),
    "p_without_lse": ("sequence_backward", "s - np.where(np.isfinite(lse), lse, 0.0)[:, None]", "s"),
    "dv_from_unquantized_p": ("sequence_backward", "dv = pq.T @ doc", "dv = p.T @ doc"),
    # where the blocks fall
    "p_blocks_along_keys": ("sequence_backward", "pq, dev_p = quantize_along(p, qpos, 0, eps_p)",
                            "pq, dev_p = quantize_along(p, kpos, 1, eps_p)"),
    "ds_for_dq_blocked_along_queries": ("sequence_backward", "dsk, dev_k = quantize_along(ds, kpos, 1, eps_ds)",
                                        "dsk, dev_k = quantize_along(ds, qpos, 0, eps_ds)"),
    "ds_for_dk_blocked_along_keys": ("sequence_backward", "dsq, dev_q = quantize_along(ds, qpos, 0, eps_ds)",
                                     "dsq, dev_q = quantize_along(ds, kpos, 1, eps_ds)"),
    "blocks_relative_to_the_first_position": ("quantize_along", "blk = pos // BLOCK - first",
                                              "blk = (pos - pos[0]) // BLOCK"),
    "self_query_blocks_per_sequence": ("backward_item", "out[s0:s1, h], lse[s0:s1, h], kpos, kpos, scale",
                                       "out[s0:s1, h], lse[s0:s1, h], kpos - s0, kpos, scale"),
    "broadcast_query_blocks_from_s0": ("backward_item", "np.arange(Lq), kpos, scale, causal)",
                                       "np.arange(Lq) + s0, kpos, scale, causal)"),
    # the block rule and its allowance
    "scale_exponent_minus_7": ("quantize_along", "- E4M3_EMAX, 0.0)", "- E4M3_EMAX + 1, 0.0)"),
    "allowance_ignores_the_scale_flip": ("quantize_along", "for a_alt in (amax - E, amax, amax + E):",
                                         "for a_alt in (amax,):"),
    "allowance_ignores_input_error": ("quantize_along", "xa = xb + s * eb * sgn", "xa = xb"),
    # the batch entry point
    "gqa_heads_not_summed": ("jagged_backward", "dk[s0:s1, h // G] += g[1]", "dk[s0:s1, h // G] = g[1]"),
    "broadcast_dq_not_summed": ("jagged_backward", "dq[h] += g[0]", "dq[h] = g[0]"),
}


def _call(fn, arg=None):
    """A runner of pin fn (with its parameter value, if it takes one) under
    a monkeypatch context."""
    params = inspect.signature(fn).parameters
    has_arg = "causal" in params or "bq" in params

    def run(mp):
        args = [arg] if has_arg else []
        if "monkeypatch" in params:
            args.append(mp)
        fn(*args)
    return run


def _pin_suite():
    out = []
    for name in dir(pins):
        if not name.startswith("test_"):
            continue
        fn = getattr(pins, name)
        params = inspect.signature(fn).parameters
        if "causal" in params:
            out += [(f"{name}[{c}]", _call(fn, c)) for c in (False, True)]
        elif "bq" in params:
            out += [(f"{name}[{b}]", _call(fn, b)) for b in (True, False)]
        else:
            out.append((name, _call(fn)))
    return out


def _fails(run, monkeypatch):
    with monkeypatch.context() as mp:
        try:
            run(mp)
        except AssertionError:
            return True
    return False


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    fn_name, old, new = MUTANTS[name]
    monkeypatch.setattr(mo, fn_name, _mutate(getattr(mo, fn_name), old, new))
    caught = [pin for pin, run in _pin_suite() if _fails(run, monkeypatch)]
    assert caught, f"no pin caught the planted mistake {name}"


def test_unmutated_oracle_passes_every_pin(monkeypatch):
    assert not [pin for pin, run in _pin_suite() if _fails(run, monkeypatch)]
