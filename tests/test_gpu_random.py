"""GPU parity on randomized small workloads (synthetic.workloads.random_mix):
random head shapes, stream counts, free-list orders, split strategies,
causal or not, sliding windows, and batches mixing prompt runs, decode
tokens, slots shared by several sequences and positions drawn at random;
half of the seeds place their sequence ids across [0, 256), so that cell
sets span several 64-bit words.  Cells and dense masks bit for bit, cache bytes bit for bit, every output of
every slot within tolerance of the fp64 oracle."""

import numpy as np
import pytest

from synthetic import workloads as W
from tests.helpers import assert_parity, gpu_run, oracle_run

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


@pytest.mark.parametrize("seed", range(96))
def test_random_mix_parity(seed):
    wl = W.random_mix(seed)
    layers = [0]
    print(f"[gpu] {wl.note}", flush=True)
    eng, ref, masks, meta = oracle_run(wl, layers, keep_masks=True)
    ub_index = {b: 0 for b in range(len(wl.batches))}
    checked = {"mask": 0}

    def check(ctx, b, ub):
        u = ub_index[b]
        r = meta[(b, u)]
        assert ub.cells.tolist() == r.cells
        m = ctx.mask(ub).cpu().numpy().view(np.uint16)
        assert np.array_equal(m, masks[(b, u)].view(np.uint16)), f"mask differs (batch {b}, ubatch {u})"
        checked["mask"] += 1
        ub_index[b] += 1

    ctx, got = gpu_run(wl, layers, on_ubatch=check)
    assert checked["mask"] == len(meta)
    worst = 0.0
    for key in ref:
        ma, _ = assert_parity(got[key], ref[key], tag=f"seed {seed} batch {key[0]}", **ref.model(key))
        worst = max(worst, ma)
    gk = ctx.K[0].cpu().numpy().view(np.uint16)
    gv = ctx.V[0].cpu().numpy().view(np.uint16)
    occ = eng.cells.pos >= 0
    assert np.array_equal(gk[occ], eng.K[0][occ].view(np.uint16))
    assert np.array_equal(gv[occ], eng.V[0][occ].view(np.uint16))
    ctx.close()
