"""GPU parity of the row kernel's ticket order (rows of at least 192 KB)
at its boundaries, against the oracle, every dlogits element: batches just
below, at and above the 256 completions where the row plan moves from the
first wavefront's registers to k_plan's prefix; a batch without an active
row (every workgroup takes a zero row); a batch in which every row is active
(no zero rows); and a few active rows among many zero rows.  Inputs are
seeded (numpy's generator); expected values come from the oracle only."""
import numpy as np
import pytest
import torch

from test_gpu_edges import _check, _run_case

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
V = 98304  # 192 KB bfloat16 rows: the smallest that takes the ticket order


def _batch(N, C, seed, eos_frac=0.6, p=0.3):
    rng = np.random.default_rng(seed)
    x = rng.normal(0, 2, (N, C, V))
    tokens = rng.integers(1, V, (N, C)).astype(np.int64)
    rows = rng.permutation(N)[: int(eos_frac * N)]
    tokens[rows, rng.integers(0, C, rows.size)] = 0
    rewards = (rng.random(N) < p).astype(np.float32)
    return x, tokens, rewards


@pytest.mark.parametrize("N", [248, 256, 264])
def test_ticket_order_around_256_completions(N):
    print(f"case N={N}", flush=True)
    x, tokens, rewards = _batch(N, 2, 100 + N)
    loss, got, res, aux, cfg = _run_case(x, tokens, 0, rewards, 8, "bf16", seed=N)
    act = int(aux["counts"][1])
    assert 0 < act < N * 2
    _check(loss, got, res, aux, cfg)


def test_ticket_order_no_active_row():
    x, tokens, _ = _batch(16, 4, 7)
    rewards = np.repeat(np.array([0, 1], np.float32), 8)
    loss, got, res, aux, cfg = _run_case(x, tokens, 0, rewards, 8, "bf16")
    assert int(aux["counts"][1]) == 0
    assert loss == 0.0 and (got == 0).all()


def test_ticket_order_every_row_active():
    """beta > 0 and no EOS id: every token row is counted and active."""
    x, tokens, rewards = _batch(16, 4, 8)
    loss, got, res, aux, cfg = _run_case(x, tokens, -1, rewards, 8, "bf16", beta=0.04)
    assert int(aux["counts"][1]) == 16 * 4
    _check(loss, got, res, aux, cfg)


def test_ticket_order_few_active_rows():
    """One group with reward contrast whose completions are short: 9 active
    rows among 72, every other row a zero row."""
    x, tokens, _ = _batch(24, 3, 9, eos_frac=0.0)
    tokens[8:16, 0] = 0  # group 1's completions end at their first token ...
    tokens[13, 0], tokens[13, 1] = 5, 0  # ... but completion 13, at its second
    rewards = np.zeros(24, np.float32)
    rewards[13] = 1.0
    loss, got, res, aux, cfg = _run_case(x, tokens, 0, rewards, 8, "bf16")
    assert int(aux["counts"][1]) == 9
    _check(loss, got, res, aux, cfg)
