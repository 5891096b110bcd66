"""The decode entry points under HIP graph capture: nothing in a call allocates,
synchronises or clears memory with a memset, so a captured step replays to the
eager result.  Each replay is followed by eager work and a synchronisation, and
every replay is compared with the eager output bit for bit."""
import os
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import mla_latent_kv_16_amd as mla  # noqa: E402
from mla_latent_kv_16_amd.workloads import make_workload  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(mla.LIB_PATH):
        pytest.fail("libmla.so is not built")
    torch.cuda.init()


@pytest.mark.parametrize("parts", [1, 9, 40], ids=["whole", "pieces-per-wave", "pieces-per-group"])
def test_captured_decode_replays_to_the_eager_result(parts):
    w = make_workload("tiny", seed=1301, B=2, Sq=4, H=16, lens=("uniform", 900, 2600))
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
    qn, qr, pool = t(w.q_nope), t(w.q_rope), t(w.kv_pool)
    bt, sl = torch.from_numpy(w.block_table).cuda(), torch.from_numpy(w.seq_lens).cuda()
    print(f"[gpu-graph] parts={parts}", flush=True)
    sys.stdout.flush()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        bd = mla.BoundDecode(qn, qr, pool, bt, sl, float(w.scale), True, parts, stream=s)
        bd()
    torch.cuda.synchronize()
    O_eager, l_eager = bd.out.clone(), bd.lse.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        bd()
    for rep in range(4):
        bd.out.fill_(float("nan"))          # eager work between replays
        bd.lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bd.out, O_eager) and torch.equal(bd.lse, l_eager), rep
    assert mla.read_error_flags(bd.workspace) == 0
