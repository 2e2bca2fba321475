"""The memory ledger against the figures the pages print (tests/golden)."""
import json
import os

import pytest

from oracle import ledger

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ledger_examples.json")
_DATA = json.load(open(GOLDEN))


@pytest.mark.parametrize("ex", _DATA["examples"], ids=lambda e: f"{e['psi']:.3g}-{e['n_d']}-{e['stage']}")
def test_printed_model_state_figures(ex):
    got_gb = ledger.model_state_bytes(ex["psi"], ex["n_d"], ex["stage"]) / 1e9
    assert got_gb == pytest.approx(ex["printed_gb"], rel=max(ex["rel_tol"], 1e-12)), ex["cite"]


@pytest.mark.parametrize("ex", _DATA["examples_m"], ids=lambda e: e["stage"])
def test_printed_generalised_ledger(ex):
    got_gb = ledger.model_state_bytes_m(ex["n"], ex["m"], ex["k"], ex["stage"]) / 1e9
    assert got_gb == pytest.approx(ex["printed_gb"], rel=1e-12), ex["cite"]


def test_sixteen_psi_and_limits():
    psi = 123_456_789
    assert ledger.model_state_bytes(psi, 1, "dp") == 16 * psi
    # with N_d = 1 every stage is the plain 16 psi ledger
    for st in ledger.STAGES:
        assert ledger.model_state_bytes(psi, 1, st) == pytest.approx(16 * psi)
    # large-N_d limits: 4x, 8x and N_d-fold reductions
    big = 10 ** 9
    assert ledger.model_state_bytes(psi, big, "os") == pytest.approx(4 * psi, rel=1e-8)
    assert ledger.model_state_bytes(psi, big, "os_g") == pytest.approx(2 * psi, rel=1e-8)
    assert ledger.model_state_bytes(psi, 64, "os_g_p") == pytest.approx(16 * psi / 64)


def test_generalised_ledger_reduces_to_k12():
    # M = 12 bytes of optimizer state reproduces the paper's K = 12 forms
    for st_m, st in (("ddp", "dp"), ("zero1", "os"), ("zero2", "os_g"), ("zero3", "os_g_p")):
        assert ledger.model_state_bytes_m(7.5e9, 12, 64, st_m) == pytest.approx(
            ledger.model_state_bytes(7.5e9, 64, st))


def test_comm_volume():
    assert ledger.comm_volume_elems(10, "dp") == 20
    assert ledger.comm_volume_elems(10, "os_g") == 20
    assert ledger.comm_volume_elems(10, "os_g_p") == 30
