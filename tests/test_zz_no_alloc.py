"""GPU: ssm_scan_prefill_static, the prefill for callers that cannot
allocate, against ssm_scan_prefill_ws with a caller's workspace.

Both run the same plan and kernels, so y and the final states must agree bit
for bit; both are also held to the oracle's bar (max |gpu - ref| / (1 + |ref|)
<= 1e-4).  The static scratch keeps the previous call's contents, so the cases
run back to back, larger first: the headline 1 x 4096 prefill (16 segments,
33 MB of scratch), then a smaller batch on the matrix-core split, then the
mixed batch on the register-path split (which also uses the running decays).
A call that would need more than the scratch holds is refused before anything
is enqueued.  The entry point also runs under HIP graph capture: four replays,
bit for bit against eager calls.
"""
import numpy as np
import pytest

import oracle
import ssm_inputs
from gpu_helpers import assert_parity, say

pytestmark = pytest.mark.gpu


def _run(ssm, case, entry, max_seqlen, segments):
    import torch
    dev = "cuda:0"
    d = ssm.to_device(case, dev)
    y = torch.full((case.n_tokens, case.H, case.P), float("nan"), device=dev)
    if entry == "static":
        ssm.prefill_static(d["x"], d["dt"], d["A"], d["B"], d["C"], d["state"], d["cu_seqlens"],
                           d["slot"], d["fresh"], max_seqlen, segments=segments, y=y)
    else:
        need = ssm.workspace_size(case.H, case.P, case.N, case.G, case.n_seqs, case.n_tokens,
                                  max_seqlen, segments)
        ws = torch.full((max(need, 1),), 0xFF, dtype=torch.uint8, device=dev)
        ssm.prefill_ws(d["x"], d["dt"], d["A"], d["B"], d["C"], d["state"], d["cu_seqlens"],
                       d["slot"], d["fresh"], max_seqlen, segments=segments, workspace=ws, y=y)
    torch.cuda.synchronize()
    return y.cpu().numpy(), d["state"].cpu().numpy()


def test_static_scratch_matches_workspace_entry():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import mamba2_selective_scan_amd as ssm
    orc = oracle.default()
    small = ssm_inputs.make_case(4, 64, 128, 2, [700, 300, 0], [1, 0, 1], seed=77,
                                 slots=[2, 0, 1], n_slots=4, poison_fresh=True,
                                 sentinel_unused=True, name="static_small")
    cases = [(ssm_inputs.workload("prefill4096"), 4096, 0),
             (small, 700, 3),
             (ssm_inputs.workload("mixed"), 150, 3)]
    for case, max_seqlen, segments in cases:
        plan = ssm.prefill_plan(case.H, case.P, case.N, case.G, case.n_seqs, max_seqlen, segments)
        need = ssm.workspace_size(case.H, case.P, case.N, case.G, case.n_seqs, case.n_tokens,
                                  max_seqlen, segments)
        say(f"static scratch: {case.name} max_seqlen={max_seqlen} segments={segments}: "
            f"{plan['segments']} segments, {need} bytes of scratch")
        assert plan["segments"] > 1 and 0 < need <= ssm.STATIC_SCRATCH_BYTES
        y_s, st_s = _run(ssm, case, "static", max_seqlen, segments)
        y_w, st_w = _run(ssm, case, "ws", max_seqlen, segments)
        assert np.array_equal(y_s, y_w), case.name
        assert np.array_equal(st_s, st_w, equal_nan=True), case.name
        y32, st32 = orc.scan_case(case, precision="f32")
        assert_parity(case, y_s, st_s, y32, st32, label=f"{case.name} static vs fp32 oracle")


def test_static_scratch_random_sweep():
    """Twelve seeded random batches back to back, in no size order (so each
    call finds the previous one's leftovers in the scratch): heads, head dim,
    state size, lengths, fresh flags, scattered slots, forced or automatic
    segments.  Bit for bit against the workspace entry, and to the oracle's
    bar."""
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import mamba2_selective_scan_amd as ssm
    orc = oracle.default()
    for seed in range(12):
        rng = np.random.Generator(np.random.PCG64(99700 + seed))
        H = int(rng.choice([1, 2, 4, 8, 16]))
        G = int(rng.choice([g for g in (1, 2, 4) if H % g == 0]))
        if seed % 2 == 0:
            P, N = int(rng.choice([16, 32, 64, 96])), 4 * int(rng.integers(1, 33))
        else:
            P, N = int(rng.integers(1, 100)), int(rng.integers(1, 260))
        n = int(rng.integers(1, 6))
        lengths = [int(v) for v in rng.integers(0, 1500, size=n)]
        case = ssm_inputs.make_case(H, P, N, G, lengths, [int(v) for v in rng.integers(0, 2, size=n)],
                                    seed=99800 + seed, slots=[int(v) for v in rng.permutation(n + 2)[:n]],
                                    n_slots=n + 2, poison_fresh=True, sentinel_unused=True,
                                    name=f"static_sweep{seed}_H{H}_G{G}_P{P}_N{N}_{lengths}")
        segments = int(rng.choice([0, 2, 3, 5]))
        max_seqlen = max(lengths)
        need = ssm.workspace_size(H, P, N, G, n, case.n_tokens, max_seqlen, segments)
        say(f"{case.name} segments={segments}: {need} bytes of scratch")
        if need > ssm.STATIC_SCRATCH_BYTES:
            continue
        y_s, st_s = _run(ssm, case, "static", max_seqlen, segments)
        y_w, st_w = _run(ssm, case, "ws", max_seqlen, segments)
        assert np.array_equal(y_s, y_w), case.name
        assert np.array_equal(st_s, st_w, equal_nan=True), case.name
        y32, st32 = orc.scan_case(case, precision="f32")
        assert_parity(case, y_s, st_s, y32, st32, label=f"{case.name} static vs fp32 oracle")


def test_static_scratch_under_graph_capture():
    """The entry point's purpose: a split prefill captured in a HIP graph
    (after one eager call, which looks the scratch up).  Every replay, with
    eager calls and synchronisations between them, gives the same bits as the
    same call made eagerly on a copy of the inputs; resumed sequences carry
    their state forward replay by replay, as the eager copy does."""
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import mamba2_selective_scan_amd as ssm
    case = ssm_inputs.make_case(8, 64, 128, 2, [1200, 700, 0, 333], [1, 0, 1, 0], seed=79,
                                slots=[3, 0, 1, 4], n_slots=6, name="static_graph")
    max_seqlen, segments = 1200, 4
    assert ssm.prefill_plan(8, 64, 128, 2, 4, max_seqlen, segments)["segments"] == 4
    g_in = ssm.to_device(case, "cuda:0")
    e_in = ssm.to_device(case, "cuda:0")
    yg = torch.empty((case.n_tokens, case.H, case.P), device="cuda:0")
    ye = torch.empty_like(yg)

    def call(d, y):
        ssm.prefill_static(d["x"], d["dt"], d["A"], d["B"], d["C"], d["state"], d["cu_seqlens"],
                           d["slot"], d["fresh"], max_seqlen, segments=segments, y=y)

    call(g_in, yg)                     # eager on both copies: the scratch is looked up here
    call(e_in, ye)
    torch.cuda.synchronize()
    assert torch.equal(yg, ye)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(g_in, yg)
    torch.cuda.synchronize()
    for rep in range(4):
        graph.replay()
        torch.cuda.synchronize()
        call(e_in, ye)
        torch.cuda.synchronize()
        assert torch.equal(yg, ye), rep
        assert torch.equal(g_in["state"], e_in["state"]), rep
    say(f"static split prefill under graph capture: 4 replays bit for bit")


def test_static_scratch_refuses_oversized_split():
    import torch
    import mamba2_selective_scan_amd as ssm
    case = ssm_inputs.make_case(64, 64, 128, 8, [2048, 2048], [1, 1], seed=78)
    need = ssm.workspace_size(64, 64, 128, 8, 2, 4096, 2048, 16)
    assert need > ssm.STATIC_SCRATCH_BYTES
    dev = "cuda:0"
    d = ssm.to_device(case, dev)
    y = torch.full((case.n_tokens, 64, 64), 7.0, device=dev)
    before = d["state"].clone()
    with pytest.raises(ssm.ScanError) as e:
        ssm.prefill_static(d["x"], d["dt"], d["A"], d["B"], d["C"], d["state"], d["cu_seqlens"],
                           d["slot"], d["fresh"], 2048, segments=16, y=y)
    assert e.value.code == ssm.SSM_ERR_SCRATCH
    torch.cuda.synchronize()
    assert torch.all(y == 7.0) and torch.equal(d["state"], before)
