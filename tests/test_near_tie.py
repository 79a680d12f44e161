"""The near-tie validity checks (tests/near_tie.py) on the CPU: they accept
the quantization of a group with a flagged element rounded the other way and
reject a group with a wrong code or scale (a mistake planted on the CPU)."""
import numpy as np
import pytest

import oracle
import synthetic
from near_tie import bf16_candidates, check_bf16_near_ties, check_group, check_rowq_near_ties

G = 128


def test_candidates():
    assert sorted(bf16_candidates(0x3F80)) == [0x3F7F, 0x3F80, 0x3F81]
    assert sorted(bf16_candidates(0xBF80)) == [0xBF7F, 0xBF80, 0xBF81]
    assert sorted(bf16_candidates(0x0000)) == [0x0000, 0x0001]


def test_group_other_rounding_accepted_wrong_rejected():
    h = synthetic.gaussian_bf16((1, G), 1.0, 3, 1)[0]
    near = np.zeros(G, bool)
    near[17] = True
    alt = h.copy()
    alt[17] = (int(h[17]) & 0x8000) | ((int(h[17]) & 0x7FFF) + 1)
    q, s = oracle.quant_act(alt.reshape(1, G))
    check_group(h, near, q[0], s[0, 0], "other rounding")           # accepted
    bad = q[0].copy()
    bad[5] ^= 1
    with pytest.raises(AssertionError):
        check_group(h, near, bad, s[0, 0], "wrong code")
    with pytest.raises(AssertionError):
        check_group(h, near, q[0], np.nextafter(s[0, 0], np.float32(1)), "wrong scale")


def test_rowq_checks_unflagged_groups_exactly():
    h = synthetic.gaussian_bf16((3, 2 * G), 1.0, 4, 1)
    near = np.zeros_like(h, dtype=bool)
    q, s = oracle.quant_act(h)
    assert check_rowq_near_ties(h, near, q, s, "exact") == 0
    q2 = q.copy()
    q2[1, 200] ^= 0x80
    with pytest.raises(AssertionError):
        check_rowq_near_ties(h, near, q2, s, "planted")


def test_bf16_near_ties():
    ref = np.array([[0x3F80, 0x4000]], np.uint16)
    near = np.array([[True, False]])
    check_bf16_near_ties(np.array([[0x3F81, 0x4000]], np.uint16), ref, near, "neighbour")
    with pytest.raises(AssertionError):
        check_bf16_near_ties(np.array([[0x3F82, 0x4000]], np.uint16), ref, near, "two steps")
    with pytest.raises(AssertionError):
        check_bf16_near_ties(np.array([[0x3F80, 0x4001]], np.uint16), ref, near, "off the flag")
