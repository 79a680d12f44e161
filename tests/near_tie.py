"""Validity checks for results where several are correct.

An element whose exact value (evaluated in fp64 by the oracle) lies next to a
BF16 rounding midpoint may round to either neighbour: the oracle flags such
elements (near_tie).  For them the GPU must have picked one of the BF16
values next to the oracle's (bits b - 1, b or b + 1 in sign-magnitude order),
and a 1x128 group that holds flagged elements must be the quantization of the
group with each flagged element replaced by one of those candidates: every
combination is enumerated and the GPU's codes and scale must equal one of
them bit for bit."""
import itertools

import numpy as np

import oracle

G = 128


def bf16_candidates(b):
    """The BF16 bit patterns next to b (and b itself), same sign."""
    mag, sign = int(b) & 0x7FFF, int(b) & 0x8000
    out = [int(b)]
    if mag > 0:
        out.append(sign | (mag - 1))
    if mag < 0x7F7F:
        out.append(sign | (mag + 1))
    return out


def check_bf16_near_ties(got, ref, near, what):
    """BF16 outputs: equal to the oracle off the flags, one of the candidates
    on them."""
    got = np.asarray(got, np.uint16)
    ref = np.asarray(ref, np.uint16)
    off = ~near
    assert np.array_equal(got[off], ref[off]), "%s: mismatch off the near-tie elements" % what
    for idx in zip(*np.nonzero(near)):
        assert int(got[idx]) in bf16_candidates(ref[idx]), "%s: %s gpu %#06x ref %#06x" % (
            what, idx, got[idx], ref[idx])


def check_group(values_bf16, flagged, got_codes, got_scale, what, max_flags=6):
    """One 1x128 group: the GPU's codes and scale equal the oracle's
    quantization of the group for some choice of candidate per flagged
    element."""
    pos = np.nonzero(flagged)[0]
    assert len(pos) <= max_flags, "%s: %d flagged elements in one group" % (what, len(pos))
    want_s = np.float32(got_scale).view(np.uint32)
    got_codes = np.asarray(got_codes, np.uint8)
    options = [bf16_candidates(values_bf16[p]) for p in pos]
    for combo in itertools.product(*options):
        v = np.array(values_bf16, np.uint16).copy()
        v[pos] = combo
        q, s = oracle.quant_act(v.reshape(1, G))
        if np.array_equal(q[0], got_codes) and s[0, 0].view(np.uint32) == want_s:
            return
    raise AssertionError("%s: no choice of the %d flagged element(s) gives the GPU's codes and scale" % (
        what, len(pos)))


def check_rowq_near_ties(h, near, gq, gs, what):
    """Row (1x128) quantization of h [M, C]: groups without flags bit-exact,
    groups with flags by enumeration.  Returns the number of flagged groups."""
    M, C = h.shape
    oq, os_ = oracle.quant_act(h)
    flag_g = near.reshape(M, C // G, G).any(axis=2)
    keep = ~flag_g
    assert np.array_equal(np.asarray(gs).view(np.uint32)[keep], os_.view(np.uint32)[keep]), what + " scales"
    assert np.array_equal(np.asarray(gq).reshape(M, -1, G)[keep], oq.reshape(M, -1, G)[keep]), what + " codes"
    for m, g in zip(*np.nonzero(flag_g)):
        sl = slice(g * G, (g + 1) * G)
        check_group(h[m, sl], near[m, sl], gq[m, sl], gs[m, g], "%s row %d group %d" % (what, m, g))
    return int(flag_g.sum())


def check_colq_near_ties(h, near, gqT, gsT, what):
    """Transposed (128 along rows) quantization of h [T, C] into [C, T]: the
    same check per column group.  Returns the number of flagged groups."""
    T, C = h.shape
    oqT, osT = oracle.quant_transpose_bf16(h)
    flag_g = near.T.reshape(C, T // G, G).any(axis=2)
    keep = ~flag_g
    assert np.array_equal(np.asarray(gsT).view(np.uint32)[keep], osT.view(np.uint32)[keep]), what + " scalesT"
    assert np.array_equal(np.asarray(gqT).reshape(C, -1, G)[keep], oqT.reshape(C, -1, G)[keep]), what + " codesT"
    for c, t in zip(*np.nonzero(flag_g)):
        sl = slice(t * G, (t + 1) * G)
        check_group(np.ascontiguousarray(h[sl, c]), near[sl, c], gqT[c, sl], gsT[c, t],
                    "%s column %d group %d" % (what, c, t))
    return int(flag_g.sum())
