"""The stored digests of the full-size workloads (tests/golden/
full_size_sha256.json, written by the oracle): every workload has one per
mode, and the oracle on this host reproduces those of the cheaper workloads
("Exact mode", section "Checking it": exact-mode hash lines are the same on
every machine).  The GPU parity tests recompute all of them with the oracle
and compare the GPU's outputs with it element by element."""
import re

import pytest

import full_size
import oracle

CHEAP = ["gemm_256", "gemm_ragged_specials", "gemm_ragged_clean", "gemm_skinny",
         "grouped_dilated", "resnet50_b1"]


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def test_every_workload_has_both_digests():
    stored = full_size.stored()
    for name in list(full_size.GEMMS) + list(full_size.CONVS):
        assert set(stored[name]) == set(full_size.MODES), name
        for mname in full_size.MODES:
            assert re.fullmatch(r"[0-9a-f]{64}", stored[name][mname]), (name, mname)
    # no two workloads or modes share a digest (a digest of the wrong outputs would)
    flat = [d for name, e in stored.items() if not name.startswith("_") for d in e.values()]
    assert len(flat) == len(set(flat))


@pytest.mark.parametrize("name", CHEAP)
def test_oracle_reproduces_the_stored_digest(orc, name):
    stored = full_size.stored()[name]
    for mname, mode in full_size.MODES.items():
        assert full_size.oracle_digest(orc, name, mode) == stored[mname], (name, mname)
