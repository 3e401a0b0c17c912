"""GPU parity of the joint-code path over a seeded random sweep of small
configurations: loop count, head dim, page size, heads, batch and ragged
lengths (0, 1, 63, 64 and 65 mixed in) are drawn per case; every stored
index of every sequence is checked against the oracle's nearest codewords
and every loop's decode against the oracle (bar of tests/test_gpu_vq.py)."""
import numpy as np
import pytest

from loop_aware_quantized_amd import inputs as wl
from loop_aware_quantized_amd import runner
from parity_util import say
from test_gpu_vq import check_indices, compare

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu
DEV = "cuda"
EDGE_LENS = [0, 1, 63, 64, 65]


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.empty_cache()


def draw_case(case: int):
    rng = np.random.default_rng([11, case])
    R = int(rng.integers(2, 5))
    D = int(rng.choice([64, 128]))
    P = int(rng.choice([16, 32, 64]))
    H = int(rng.integers(1, 5))
    B = int(rng.integers(1, 6))
    lens = [int(x) for x in rng.integers(0, 4001, size=B)]
    for i in range(B):
        if rng.random() < 0.3:
            lens[i] = int(rng.choice(EDGE_LENS))
    return R, D, P, H, B, lens


@pytest.mark.parametrize("case", range(16))
def test_vq_random_configuration(case):
    R, D, P, H, B, lens = draw_case(case)
    say(f"vq sweep case {case}: R={R} D={D} P={P} H={H} B={B} lens={lens}")
    w = wl.VqWorkload(f"vq-sweep-{case}", 400 + case, batch=B, loops=R, layers=1, heads=H, head_dim=D, page=P,
                      ctx=max(max(lens), 1))
    st = runner.VqState(w, DEV, lengths=lens)
    kept = st.prefill_layer(0, keep=set(range(B)))
    torch.cuda.synchronize()
    host = {b: kept.get(b, (np.zeros((R, 0, H, D), np.uint16),) * 2) for b in range(B)}
    for b in range(B):
        if lens[b]:
            ki, vi = st.pool_indices(0, b, lens[b])
            check_indices(ki, host[b][0], st.codebooks[0][0])
            check_indices(vi, host[b][1], st.codebooks[0][1])
    for loop in range(R):
        q = wl.vq_query(w, 0, loop, DEV)
        out = torch.empty(B, H, D, dtype=torch.float32, device=DEV)
        st.decode(0, loop, q, out)
        torch.cuda.synchronize()
        nonempty = [b for b in range(B) if lens[b]]
        for b in range(B):
            if not lens[b]:
                assert torch.count_nonzero(out[b]) == 0, "an empty sequence decodes to zeros"
        if nonempty:
            rel = compare(st, 0, loop, q, out, host, nonempty, lens)
            say(f"  loop {loop}: rel err {rel:.2e}")
