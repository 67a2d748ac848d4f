"""Pins for the oracle's per-stage accounting (CPU only): model-state bytes a
rank holds and elements it sends per step under ZeRO stages 0-3, checked
against what the pages print and state ("ZeRO Stages: Sharding Optimizer
State, Gradients, and Parameters", stage sections and "Communication volume
compared"; "ZeRO Stage 3: Parameter Partitioning", equation M_Stage3 and its
7B / 64-GPU example)."""
import pytest

import oracle
from golden_io import read as read_golden

PSI = 7_000_000_000


def test_stage3_worked_example():
    """M_Stage3: 16 * 7e9 / 64 = 1.75 GB per GPU, every term sharded."""
    g = read_golden("accounting_7b_n64.txt")
    s = g["psi"] // g["n_d"]
    assert oracle.stage_state_bytes(3, g["psi"], s, grad_bytes=2) == g["per_gpu_bytes"]
    assert oracle.stage_state_bytes(0, g["psi"], s, grad_bytes=2) == g["total_bytes"]


def test_eighteen_byte_budget_and_stage1_two_thirds():
    """[ZST]: the budget is 18 bytes per parameter (4-byte gradients); the
    optimizer term stage 1 shards is 12 of them, so with many ranks stage 1
    removes two thirds of the state."""
    assert oracle.stage_state_bytes(0, PSI, PSI // 8, grad_bytes=4) == 18 * PSI
    for nd in (2, 8, 64, 1000):
        s = PSI // nd
        s0 = oracle.stage_state_bytes(0, PSI, s, 4)
        s1 = oracle.stage_state_bytes(1, PSI, s, 4)
        assert s0 - s1 == 12 * (PSI - s)          # only the optimizer term shrinks
    s = PSI // 7_000_000                          # 7e6 ranks: S = 1000
    s0, s1 = oracle.stage_state_bytes(0, PSI, s, 4), oracle.stage_state_bytes(1, PSI, s, 4)
    assert abs((s0 - s1) / s0 - 2 / 3) < 1e-6


def test_stage2_saves_the_gradient_term():
    """[ZST]: stage 2 saves the gradient term, 4 bytes per parameter, on top
    of stage 1."""
    for nd in (2, 8, 64):
        s = PSI // nd
        s1 = oracle.stage_state_bytes(1, PSI, s, 4)
        s2 = oracle.stage_state_bytes(2, PSI, s, 4)
        assert s1 - s2 == 4 * (PSI - s)


def test_parameter_replica_floor_and_linear_stage3():
    """[ZS3]: stages 1 and 2 keep a full 16-bit parameter replica, 2 bytes per
    parameter that no rank count removes; stage 3 halves when the rank count
    doubles."""
    for nd in (8, 64, 7_000_000):
        s = PSI // nd
        assert oracle.stage_state_bytes(2, PSI, s, 2) > 2 * PSI
        assert oracle.stage_state_bytes(1, PSI, s, 2) > 4 * PSI   # gradients replicated too
    big = PSI // 7_000_000
    assert abs(oracle.stage_state_bytes(2, PSI, big, 2) / (2 * PSI) - 1) < 1e-5
    for nd in (1, 2, 4, 8, 16, 32):
        assert oracle.stage_state_bytes(3, PSI, PSI // nd, 2) == \
            2 * oracle.stage_state_bytes(3, PSI, PSI // (2 * nd), 2)


def test_one_rank_shards_nothing():
    for stage in range(4):
        assert oracle.stage_state_bytes(stage, 12345, 12345, 2) == 16 * 12345
        assert oracle.stage_comm_elems(stage, 12345, 1) == 0.0
    assert oracle.stage_state_bytes(4, 1, 1, 2) == -1
    assert oracle.stage_comm_elems(-1, 1, 2) == -1.0


@pytest.mark.parametrize("n,p", [(7_000_000_000, 64), (1000, 8), (202_383_360, 8), (10, 3)])
def test_communication_table(n, p):
    """The per-rank volumes the table prints, and its prose: stage 2 moves
    exactly what the baseline all-reduce moved; stage 1 adds one gather on
    top; stage 3 moves about three gathers' worth."""
    unit = n * (p - 1) / p
    want = {0: 2 * unit, 1: 2 * unit + unit, 2: unit + unit, 3: 3 * unit}
    for stage, w in want.items():
        assert oracle.stage_comm_elems(stage, n, p) == pytest.approx(w, rel=1e-12)
    assert oracle.stage_comm_elems(2, n, p) == pytest.approx(oracle.stage_comm_elems(0, n, p))
    assert oracle.stage_comm_elems(1, n, p) - oracle.stage_comm_elems(2, n, p) == \
        pytest.approx(unit)
