"""The benchmark's accounting against the oracle's own storage and budget
figures: the algorithmic bytes and flops that every roofline fraction of the
bench line divides by, and the sign / scale bits per weight it reports
(the aibk.xyz article "三星把权重压到 0.1 比特，追平 1 比特基线", in its points
on judging such schemes, asks that the bits-per-weight accounting be stated).
bench.py computes these from the shapes and ranks itself; the oracle's
functions are pinned in test_oracle.py."""
from fractions import Fraction

import pytest

import bench
import oracle
import synth
import binary_rank_gemm_amd as lb

WL = ["llama2-7b-0.1bpw", "llama2-13b-0.55bpw", "llama3-8b-0.3bpw", "llama2-70b-0.1bpw"]


@pytest.mark.parametrize("name", WL)
@pytest.mark.parametrize("T", [1, 16, 2048])
def test_algorithmic_bytes_and_flops_match_the_oracle(name, T):
    wl = synth.WORKLOADS[name]
    ranks_of = [bench.ranks_for(wl, s, lb) for s in wl.mats]
    byts, flops = bench.algorithmic(wl, ranks_of, T)
    want_b = Fraction(0)
    want_f = 0
    for _, j, s in wl.entries():
        want_b += oracle.linear_storage_bytes(s.m, s.n, ranks_of[j]) + T * (s.m + s.n) * 2
        want_f += sum(2 * T * (s.m + s.n) * r for r in ranks_of[j])
    assert byts == want_b
    assert flops == want_f


@pytest.mark.parametrize("name", WL)
def test_bit_budget_matches_the_oracle(name):
    wl = synth.WORKLOADS[name]
    ranks_of = [bench.ranks_for(wl, s, lb) for s in wl.mats]
    bb = bench.bit_budget(wl, ranks_of)
    weights = sum(s.m * s.n for s in wl.mats)
    scale = sum(oracle.scale_bits_per_weight(s.m, s.n, ranks_of[j]) * s.m * s.n for j, s in enumerate(wl.mats))
    sign = sum(Fraction(sum(r * (s.m + s.n) for r in ranks_of[j])) for j, s in enumerate(wl.mats))
    assert bb["scale_bpw"] == round(float(scale / weights), 5)
    assert bb["sign_bpw"] == round(float(sign / weights), 5)
    assert bb["total_bpw"] == round(float((scale + sign) / weights), 5)
    # the rank rule spends the sign-bit budget: within one rank step of it
    assert abs(Fraction(bb["sign_bpw"]).limit_denominator(10 ** 6) - wl.bpw) < Fraction(1, 50)


def test_headline_algorithmic_bytes():
    """The figure the headline roofline divides by (Llama-2-70B stack, one token)."""
    wl = synth.WORKLOADS["llama2-70b-0.1bpw"]
    ranks_of = [bench.ranks_for(wl, s, lb) for s in wl.mats]
    byts, _ = bench.algorithmic(wl, ranks_of, 1)
    assert int(byts) == 935010240
