"""Host-side logic of bench.py: the pick accounting behind its byte and flop
figures (touched experts and kept slots per call) agrees with the oracle's
router on the same logits, for the plain router, expert top-p and the
variant routers."""
import numpy as np
import pytest

import bench
import oracle


@pytest.mark.parametrize("router", ["softmax", "sigmoid", "softmax-bias", "sigmoid-bias"])
def test_routing_counts_match_oracle(router):
    rng = np.random.default_rng(11)
    E, k = 128, 8
    L = (rng.standard_normal((64, E)) * 1.5).astype(np.float32)
    bias = bench.router_bias(router, E)
    assert (bias is None) == (not router.endswith("-bias"))
    gate = "sigmoid" if router.startswith("sigmoid") else "softmax"
    idx, _, _ = oracle.router_topk(L, k, gate=gate, bias=bias)
    touched, slots = bench.routing_counts(L, k, router=router, bias=bias)
    assert touched == len(np.unique(idx)) and slots == idx.size


@pytest.mark.parametrize("p", [0.3, 0.7, 0.95])
def test_routing_counts_top_p_match_oracle(p):
    rng = np.random.default_rng(12)
    L = (rng.standard_normal((64, 256)) * 4.0).astype(np.float32)  # peaked rows
    idx, _, _ = oracle.router_topk(L, 8, top_p=p)
    kept = idx[idx >= 0]
    touched, slots = bench.routing_counts(L, 8, top_p=p)
    assert touched == len(np.unique(kept)) and slots == kept.size
    assert slots < idx.size  # top-p dropped some picks


def test_stage_work_counts_touched_experts_only():
    import moe_synth as S
    wl = S.WORKLOADS["decode"]
    w = bench.stage_work(wl, 1, 8, gemm=False)
    # 8 experts x 2 planes x (nibbles + fp16 scales), the bf16 row, the fp16 hidden rows
    per_plane = wl.I * wl.H // 2 + wl.I * (wl.H // 32) * 2
    assert w["gate_up"]["bytes"] == 8 * 2 * per_plane + wl.H * 2 + 8 * wl.I * 2
    assert w["gate_up"]["flops"] == 4.0 * 8 * wl.H * wl.I
    assert w["down"]["flops"] == 2.0 * 8 * wl.H * wl.I
