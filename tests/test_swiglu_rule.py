"""CPU checks of the tests' SwiGLU validity rule (tests/swiglu_rule.py): it
admits exactly the neighbour across a nearby bf16 midpoint, and the block
check accepts an MX operand built from an admitted choice of H while
rejecting one built from any other change."""
import numpy as np

import oracle
from tests.swiglu_rule import allowed_range, check_h, check_quantized_h


def case(seed=3, R=8, F=256):
    rng = np.random.default_rng(seed)
    g = rng.normal(0, 4, (R, F)).astype(np.float32)
    u = rng.normal(0, 1, (R, F)).astype(np.float32)
    gb = (g.view(np.uint32) >> 16).astype(np.uint16)
    ub = (u.view(np.uint32) >> 16).astype(np.uint16)
    c = np.concatenate([gb, ub], axis=1)
    h, hv = oracle.swiglu_bf16(c, F, F, with_f64=True)
    uf = (ub.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return h, hv, uf


def near_midpoint_value():
    # g = 96, u = 1 + 2^-7: the binary64 value is the midpoint 96.75 itself
    c = np.array([[0x42C0, 0x3F81]], dtype=np.uint16)
    h, hv = oracle.swiglu_bf16(c, 1, 1, with_f64=True)
    return h, hv, np.array([[1.0078125]])


def test_rule_admits_the_neighbour_across_a_midpoint_only():
    h, hv, u = near_midpoint_value()
    lo, hi = allowed_range(h, hv, u)
    assert (lo[0, 0], hi[0, 0]) == (0x42C1, 0x42C2)
    assert check_h(np.array([[0x42C1]], dtype=np.uint16), h, hv, u) == (1, 1)
    try:
        check_h(np.array([[0x42C3]], dtype=np.uint16), h, hv, u)
    except AssertionError:
        pass
    else:
        raise AssertionError("a value two steps away was admitted")


def test_block_check_accepts_admitted_choice_rejects_others():
    h, hv, u = case()
    # plant the near-midpoint element in a block, with its admitted neighbour
    hn, hvn, un = near_midpoint_value()
    h[2, 40], hv[2, 40], u[2, 40] = hn[0, 0], hvn[0, 0], un[0, 0]
    c0, s0 = oracle.quantize_mx(h)
    assert check_quantized_h(c0, s0, h, hv, u, oracle.quantize_mx)[0] == 0
    alt = h.copy()
    alt[2, 40] = 0x42C1
    c1, s1 = oracle.quantize_mx(alt)
    nb, na = check_quantized_h(c1, s1, h, hv, u, oracle.quantize_mx)
    assert nb == (0 if np.array_equal(c1, c0) and np.array_equal(s1, s0) else 1) and na >= 1
    # an element far from any midpoint changed: rejected
    bad = h.copy()
    bad[5, 100] ^= 0x0040
    c2, s2 = oracle.quantize_mx(bad)
    if np.array_equal(c2, c0) and np.array_equal(s2, s0):
        return  # the change did not reach the codes
    try:
        check_quantized_h(c2, s2, h, hv, u, oracle.quantize_mx)
    except AssertionError:
        pass
    else:
        raise AssertionError("a change outside the rule was accepted")
