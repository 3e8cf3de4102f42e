"""Planted mistakes in copies of the oracle must be caught by the pins.

Each mutant is the oracle's decode attention with one plausible mistake (a
dropped term, a wrong sign or index, a transposed operand, an off-by-one in
the valid length). The pins in ``oracle_pins`` are run against every mutant
and at least one must fail. The mutants live only here, on the CPU; the
oracle itself is untouched.
"""

import numpy as np
import pytest

import oracle_pins as pins
from oracle.codec import widen


def make_decode(flaw):
    def fn(q, k_cache, v_cache, valid_lens, sm_scale):
        q = widen(q)
        B, H, D = q.shape
        H_kv = k_cache.shape[1]
        G = H // H_kv
        out = np.zeros((B, H, D))
        for b in range(B):
            n = int(valid_lens[b])
            if flaw == "n_minus_one":
                n = max(n - 1, 1) if n > 0 else 0
            if flaw == "n_plus_one":
                n = min(n + 1, k_cache.shape[2])
            if n == 0:
                if flaw == "empty_is_mean":
                    out[b] = widen(v_cache[b]).mean(axis=1).repeat(G, axis=0)
                continue
            for h in range(H):
                g = h % H_kv if flaw == "interleaved_groups" else h // G
                kk = widen(k_cache[b, g, :n])
                vv = widen(v_cache[b, g, :n])
                if flaw == "kv_swapped":
                    kk, vv = vv, kk
                scale = 1.0 if flaw == "no_scale" else sm_scale
                if flaw == "sqrt_scale":
                    scale = np.sqrt(sm_scale)
                s = scale * (kk @ q[b, h])
                if flaw == "sign":
                    s = -s
                p = np.exp(s - s.max())
                if flaw == "no_normalise":
                    out[b, h] = p @ vv
                elif flaw == "first_row_dropped":
                    out[b, h] = (p[1:] @ vv[1:]) / p[1:].sum() if n > 1 else vv[0]
                elif flaw == "max_not_subtracted_twice":
                    out[b, h] = (p @ vv) / np.sum(np.exp(s))
                else:
                    out[b, h] = (p @ vv) / p.sum()
        return out
    return fn


FLAWS = ["n_minus_one", "n_plus_one", "empty_is_mean", "interleaved_groups", "kv_swapped",
         "no_scale", "sqrt_scale", "sign", "no_normalise", "first_row_dropped",
         "max_not_subtracted_twice"]


def _caught(fn):
    for check in pins.ALL_CHECKS:
        try:
            check(fn)
        except AssertionError:
            return check.__name__
        except (ValueError, IndexError, FloatingPointError):
            return check.__name__
    return None


def test_unmutated_copy_passes():
    assert _caught(make_decode(None)) is None


@pytest.mark.parametrize("flaw", FLAWS)
def test_mutant_is_caught(flaw):
    with np.errstate(all="ignore"):
        assert _caught(make_decode(flaw)) is not None, f"no pin catches '{flaw}'"
