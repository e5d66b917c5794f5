"""Pins of the oracle's model-state accounting against the worked figures of the upskillscore
summary of "ZeRO: Memory Optimizations Toward Training Trillion Parameter Models" (stored in
tests/golden/zero_paper_model_states.txt), the briefia.fr 7B memory example ("Problème de
mémoire dans DDP") and the TorchDistPackage "Intro.md" optimizer-state example (section 3)."""
import os

import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "zero_paper_model_states.txt")


def _rows():
    for line in open(GOLDEN):
        line = line.split("#")[0].split()
        if line:
            kind, psi, nd, stage, val, tol = line
            yield kind, float(psi), float(nd), int(stage), float(val), float(tol)


@pytest.mark.parametrize("row", list(_rows()))
def test_paper_figures(row):
    kind, psi, nd, stage, val, tol = row
    if kind == "state":
        got = oracle.model_state_bytes(psi, nd, stage)
    else:  # largest psi with model states <= the device memory (bytes are linear in psi)
        got = psi / oracle.model_state_bytes(1.0, nd, stage)
    assert abs(got - val) <= tol * val


def test_exact_stage_values_at_nd64():
    """The closed forms behind the page's rounded 120 / 31.4 / 16.6 / 1.9 GB."""
    psi = 7.5e9
    assert oracle.model_state_bytes(psi, 64, 0) == 120e9
    assert oracle.model_state_bytes(psi, 64, 1) == 31.40625e9
    assert oracle.model_state_bytes(psi, 64, 2) == 16.640625e9
    assert oracle.model_state_bytes(psi, 64, 3) == 1.875e9


def test_component_figures():
    psi = 1.5e9
    assert oracle.model_state_bytes(psi, 1, 3) == 24e9           # 16 bytes per parameter
    assert oracle.model_state_bytes(psi, 1e30, 1) == pytest.approx(4 * psi)  # Nd -> inf: 4 psi
    assert oracle.model_state_bytes(psi, 1e30, 2) == pytest.approx(2 * psi)  # Nd -> inf: 2 psi
    # 16-bit weights of the 1.5B model: 3 GB; the fp32 copy alone: 6 GB (the fused buffer)
    stage0 = oracle.model_state_bytes(psi, 1, 0)
    assert stage0 / 16 * 2 == 3e9 and stage0 / 16 * 4 == 6e9


def test_seven_billion_ddp_total():
    """briefia.fr: 7B parameters under plain data parallel hold 112 GB of model state per GPU
    (they count fp32 parameters, gradients and two Adam moments; 16 bytes per parameter,
    the same total as mixed precision's 2 + 2 + 12)."""
    assert oracle.model_state_bytes(7e9, 8, 0) == 112e9


def test_optimizer_state_split():
    """TorchDistPackage Intro: 40 GB of optimizer state is 5 GB per card on 8 cards and a
    little over 1 GB on 32.  Stage 1 minus the unpartitioned 4 psi is the 12 psi / Nd part."""
    psi = 40e9 / 12
    for nd, want in ((8, 5e9), (32, 1.25e9)):
        got = oracle.model_state_bytes(psi, nd, 1) - 4 * psi
        assert got == pytest.approx(want, rel=1e-12)


def test_invalid_stage():
    assert oracle.model_state_bytes(1.0, 1.0, 4) < 0
