"""GPU parity of the offloaded linear (W split by output rows between mapped
host memory and HBM) against the fp64 oracle y = x W^T.

Products of bf16 values are exact in fp32 and accumulate in fp32, so the bar
is relative to the scale of the sum: |y - y_ref| <= 1e-5 * sqrt(K) * max|x||w|
rows, with the 2e-3 absolute bar of the path as a ceiling.
"""
import numpy as np
import pytest

import oracle as O
from synth import normal_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dk():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    import decode_attention_host_amd as dk
    dk.reset_tuning()
    return dk


def _run(dk, w, x, ratio):
    import torch
    lin = dk.OffloadedLinear(w, ratio)
    y = lin(torch.from_numpy(x.view(np.int16)).cuda())
    torch.cuda.synchronize()
    out = y.cpu().numpy().astype(np.float64)
    lin.free()
    return out


def _check(y, ref, K, what):
    err = np.abs(y - ref).max()
    tol = min(2e-3, 1e-5 * np.sqrt(K) * max(1.0, np.abs(ref).max() / np.sqrt(K)))
    print(f"{what}: max|dy|={err:.3g} (tol {tol:.3g})", flush=True)
    assert err <= tol, what


CASES = [
    # (m, N, K, ratio, w_std)
    (1, 64, 64, 1.0, 1.0),
    (1, 100, 264, 0.5, 1.0),        # ragged rows, K tail not a multiple of 32
    (7, 1000, 1024, 0.3, 0.05),
    (16, 4096, 4096, 0.0, 0.02),    # K split into partials
    (17, 777, 2056, 0.9, 0.02),     # two token tiles
    (64, 256, 512, 0.75, 1.0),      # four token tiles
    (100, 300, 4096, 0.5, 0.02),    # two launches of tokens
    (5, 200, 3000, 0.0, 0.5),       # K split into ranges of 1504 and 1496: both end inside a chunk
    (9, 8192, 4096, 0.01, 0.02),    # host tier split over K (2 blocks x 4 ranges), HBM tier whole
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_linear_parity(dk, case):
    m, N, K, r, std = CASES[case]
    w = normal_bf16(90 + case, 5, (N, K), std=std)
    x = normal_bf16(90 + case, 4, (m, K))
    y = _run(dk, w, x, r)
    _check(y, O.linear(x, w), K, f"case {case}")


def test_linear_identity_weight_returns_x(dk):
    from synth import bf16_bits_from_f32
    K = 128
    w = bf16_bits_from_f32(np.eye(K, dtype=np.float32))
    x = normal_bf16(95, 4, (5, K))
    y = _run(dk, w, x, 0.5)
    assert np.array_equal(y, O.bf16_to_f64(x))


def test_linear_ratios_agree_and_llama_mlp_full_size(dk):
    # LLaMA-3-8B MLP up-projection shape, 16 tokens: every ratio gives the
    # same result as r = 0 to fp32 summation-order noise; sampled rows vs oracle
    N, K, m = 14336, 4096, 16
    w = normal_bf16(96, 5, (N, K), std=0.02)
    x = normal_bf16(96, 4, (m, K))
    ys = {r: _run(dk, w, x, r) for r in (0.0, 0.5, 1.0)}
    for r in (0.5, 1.0):
        assert np.abs(ys[r] - ys[0.0]).max() < 1e-4
    rows = np.random.default_rng(0).choice(N, 64, replace=False)
    ref = O.linear(x, w[rows])
    _check(ys[1.0][:, rows], ref, K, "llama mlp sampled rows r=1")


def test_linear_smallest_shapes(dk):
    # one output row, K = 8 (a single 16-byte group, not a multiple of 32)
    for N, K, m, r in [(1, 8, 1, 1.0), (1, 8, 3, 0.0), (2, 8, 1, 0.5), (65, 40, 2, 0.5)]:
        w = normal_bf16(97, 5, (N, K))
        x = normal_bf16(97, 4, (m, K))
        y = _run(dk, w, x, r)
        _check(y, O.linear(x, w), K, f"N={N} K={K} m={m} r={r}")


def test_linear_workspace_reused_and_left_zeroed(dk):
    """K split over both tiers (tuned ranges), partials summed in the launch:
    calls of 100 tokens (two launches), 3 and 64 tokens on one workspace must
    each match the oracle and leave the workspace counters at zero."""
    import torch
    N, K = 300, 2056
    w = normal_bf16(98, 5, (N, K), std=0.05)
    try:
        dk.set_tuning(host_chunk=256, dev_chunk=512)
        lin = dk.OffloadedLinear(w, 0.4)
        info = lin.plan(100)
        assert info["num_splits"] == info["host_items"] + info["dev_items"] > 0
        ws = lin.workspace(100)
        for m in (100, 3, 64):
            x = normal_bf16(98 + m, 4, (m, K))
            y = lin(torch.from_numpy(x.view(np.int16)).cuda(), workspace=ws)
            torch.cuda.synchronize()
            _check(y.cpu().numpy().astype(np.float64), O.linear(x, w), K, f"reused workspace m={m}")
            assert int(torch.count_nonzero(ws[:256])) == 0, "counters not left at zero"
        lin.free()
    finally:
        dk.reset_tuning()


@pytest.mark.parametrize("tune", [{}, {"dev_chunk": 512, "host_chunk": 1024}])
def test_linear_graph_replays_match_eager(dk, tune):
    """A linear call captured in a HIP graph (no host plan: nothing is
    uploaded per call) replays to the eager result bit for bit, with eager
    calls on the same workspace between replays."""
    import torch
    N, K, m = 1000, 4096, 5
    w = normal_bf16(99, 5, (N, K), std=0.02)
    try:
        if tune:
            dk.set_tuning(**tune)
        lin = dk.OffloadedLinear(w, 0.25)
        ws = lin.workspace(m)
        x = torch.from_numpy(normal_bf16(99, 4, (m, K)).view(np.int16)).cuda()
        y = torch.empty((m, N), dtype=torch.float32, device="cuda")
        lin(x, y, ws)
        torch.cuda.synchronize()
        eager = y.clone()
        g = dk.StepGraph(lambda: lin(x, y, ws))
        for i in range(4):
            y.zero_()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(y, eager), f"replay {i}"
            lin(x, workspace=ws)
            torch.cuda.synchronize()
        _check(eager.cpu().numpy().astype(np.float64), O.linear(normal_bf16(99, 4, (m, K)), w), K, "graph case")
        lin.free()
    finally:
        dk.reset_tuning()
