"""The ceiling probes the benchmark reports (kvattn_probe_gather,
kvattn_probe_mfma) compute what their declarations say, so their rates are
rates of real work: the gather reads every listed row (its sums match the
rows it was pointed at, clamped indices included) and the matrix-core probe
performs every product (its outputs equal the closed form)."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
K = pytest.importorskip("ubatch_attention_paged_amd")


def test_probe_gather_reads_the_listed_rows():
    dev = torch.device("cuda:0")
    g = torch.Generator(device="cpu")
    g.manual_seed(11)
    n_rows, n_index, n_wg = 1000, 5003, 37
    rows = torch.randn((n_rows, 1024), generator=g).to(torch.float16)
    index = torch.randint(-5, n_rows + 5, (n_index,), generator=g, dtype=torch.int32)   # some clamped
    print(f"[gpu] probe gather: {n_index} rows of {n_rows}, {n_wg} workgroups", flush=True)
    out = torch.full((n_wg * 256,), float("nan"), device=dev)
    rd, idd = rows.to(dev), index.to(dev)
    K.kvattn_probe_gather(rd.data_ptr(), n_rows, idd.data_ptr(), n_index, out.data_ptr(), n_wg,
                          torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    got = out.double().sum().item()
    ref = rows.double()[index.clamp(0, n_rows - 1).long()].sum().item()
    scale = rows.double()[index.clamp(0, n_rows - 1).long()].abs().sum().item()
    assert np.isfinite(out.cpu().numpy()).all()
    assert abs(got - ref) <= 1e-6 * scale, (got, ref)


def test_probe_mfma_performs_every_product():
    dev = torch.device("cuda:0")
    ab = torch.tensor([1, 2, 3, 4, 1, 2, 3, 4, 2, 1, 2, 1, 1, 1, 1, 1], dtype=torch.float16)
    dot = float((ab[:8].double() * ab[8:].double()).sum())
    n_wg, iters = 9, 100
    print(f"[gpu] probe mfma: {n_wg} workgroups x {iters} rounds", flush=True)
    out = torch.full((n_wg * 256,), float("nan"), device=dev)
    K.kvattn_probe_mfma(ab.to(dev).data_ptr(), out.data_ptr(), n_wg, iters, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert torch.all(out.cpu() == 128.0 * iters * dot), out[:4]
