"""Sequence-state save / restore on the GPU (kvattn_seq_state_*).

* saved blobs are byte-identical to the oracle's (oracle/seqstate.py, pinned
  to the .bin dump's sizes and offsets): the page's own case (7 cells, 28
  layers, 803,596 bytes), a shared prefix, four streams;
* restoring into another context (other free-cell order) gives the oracle's
  cell table bit for bit, and attention over the restored sequences matches
  the oracle's within the parity tolerance;
* a restore that does not fit or a blob that does not match the context
  changes nothing;
* at full size (28 layers, a 2048-position sequence) every saved row equals
  the cache row it came from, and save -> restore elsewhere -> save
  reproduces the blob exactly.
"""

import numpy as np
import pytest
import torch

import ubatch_attention_paged_amd as K
from oracle import OracleEngine
from oracle import seqstate as S
from synthetic import workloads as W

from helpers import ATOL, RTOL, assert_parity, gpu_run, make_ctx, model_for, oracle_run

pytestmark = pytest.mark.gpu


def blob_bytes(t):
    return bytes(t.cpu().numpy().tobytes())


def saved_pair(wl, seqs):
    layers = list(range(wl.n_layer))
    print(f"seqstate: {wl.name} {wl.note}", flush=True)
    ctx, _ = gpu_run(wl, layers)
    eng, _, _, _ = oracle_run(wl, layers, measured_only=False, sigma=False)
    out = {}
    for q in seqs:
        g = blob_bytes(ctx.state_save(q))
        r = S.save(eng, q)
        assert len(g) == len(r) == ctx.state_size(q)
        assert g == r, f"sequence {q}: first differing byte {next(i for i in range(len(g)) if g[i] != r[i])}"
        out[q] = r
    torch.cuda.synchronize()
    return ctx, eng, out


def test_page_case_seven_cells_28_layers():
    wl = W.qwen_prefill(n_prompt=7, n_layer=28, kv_size=256, n_batch=64, n_ubatch=64)
    _, _, out = saved_pair(wl, [0])
    assert len(out[0]) == 803596
    assert S.record_offset(28, 8, 128, 7, 0, 0) == 108


def test_shared_prefix_and_streams():
    saved_pair(W.prefix_decode(n_seq=4, prefix=40, private=9, n_layer=2, kv_size=256), [0, 1, 2, 3])
    saved_pair(W.mixed(n_prompt_seq=2, n_decoders=6, prompt_range=(20, 70), ctx_range=(10, 60), n_layer=2,
                       n_stream=4, kv_size=128, n_batch=128, n_ubatch=32), list(range(8)))


def test_restore_then_attend_matches_oracle():
    wl = W.prefix_decode(n_seq=4, prefix=40, private=9, n_layer=2, kv_size=256)
    _, _, blobs = saved_pair(wl, [0, 1])
    order = np.random.default_rng(77).permutation(wl.kv_size).astype(np.int32)[None, :]
    dst = K.Context(wl.n_layer, wl.n_head, wl.n_head_kv, wl.head_dim, wl.kv_size, 1, wl.n_seq_max, 64, 64,
                    cell_order=order, device="cuda:0", attend_layers=2)
    eng = OracleEngine(wl.n_layer, wl.n_head, wl.n_head_kv, wl.head_dim, wl.kv_size, 1, wl.n_seq_max, 64, 64,
                       cell_order=order)
    for seq, src in ((2, 0), (3, 1)):
        dev = torch.frombuffer(bytearray(blobs[src]), dtype=torch.uint8).to("cuda:0")
        assert dst.state_load(seq, dev) == 0
        S.load(eng, seq, blobs[src])
    pos, mask = dst.cells(0)
    assert np.array_equal(pos, eng.cells.pos[0])
    assert np.array_equal(K.seqset_members(mask, K.MAX_SEQ)[:, :wl.n_seq_max], eng.cells.member[0])
    assert not K.seqset_members(mask, K.MAX_SEQ)[:, wl.n_seq_max:].any()
    assert blob_bytes(dst.state_save(2)) == blobs[0] and blob_bytes(dst.state_save(3)) == blobs[1]
    # one decode token for each restored sequence, attention over the copies
    n, p = 2, 40 + 9 + 1
    rng = np.random.default_rng(5)
    kv = [(rng.standard_normal((n, wl.E), dtype=np.float32), rng.standard_normal((n, wl.E), dtype=np.float32))
          for _ in range(2)]
    q = [rng.standard_normal((n, wl.n_head * wl.head_dim), dtype=np.float32) for _ in range(2)]
    st, ubs, _ = dst.split(n, [p, p], [(2,), (3,)], [1, 1])
    rst, rubs, _ = eng.split(n, [p, p], [(2,), (3,)], [1, 1])
    assert st == rst == 0 and len(ubs) == len(rubs) == 1
    u, ru = ubs[0], rubs[0]
    assert u.cells.tolist() == list(ru.cells)
    d = lambda x: torch.from_numpy(x[u.src]).to("cuda:0")
    dst.store(u, 0, [d(kv[l][0]) for l in range(2)], [d(kv[l][1]) for l in range(2)])
    outs = [torch.empty((n, wl.n_head * wl.head_dim), device="cuda:0") for _ in range(2)]
    dst.attend(u, 0, [d(q[l]) for l in range(2)], outs)
    eng.commit(ru, build_mask=True)
    for l in range(2):
        eng.store(ru, l, kv[l][0][ru.src], kv[l][1][ru.src])
        alt, sig = model_for(eng, ru, l, q[l][ru.src])
        assert_parity(outs[l].double().cpu().numpy(), eng.attend(ru, l, q[l][ru.src]), tag=f"layer {l}",
                      alt=alt, sigma=sig)


def test_restore_refusals_change_nothing():
    wl = W.prefix_decode(n_seq=4, prefix=40, private=9, n_layer=2, kv_size=256)
    _, _, blobs = saved_pair(wl, [0])
    dev = torch.frombuffer(bytearray(blobs[0]), dtype=torch.uint8).to("cuda:0")
    small = K.Context(2, wl.n_head, wl.n_head_kv, wl.head_dim, 64, 1, 4, 64, 64, device="cuda:0")
    st, ubs, _ = small.split(20, list(range(20)), [(1,)] * 20, None)
    for u in ubs:
        small.store(u, 0, [torch.zeros((u.n_tokens, wl.E), device="cuda:0")] * 2,
                    [torch.zeros((u.n_tokens, wl.E), device="cuda:0")] * 2)
    before = small.cells(0)
    assert small.state_load(0, dev) == K.KVATTN_NO_SLOT          # 50 cells > 44 free
    after = small.cells(0)
    assert np.array_equal(before[0], after[0]) and np.array_equal(before[1], after[1])
    other = K.Context(2, wl.n_head, wl.n_head_kv, 64, 256, 1, 4, 64, 64, device="cuda:0")
    with pytest.raises(K.KvattnError) as e:
        other.state_load(0, dev)                                  # head_dim differs
    assert e.value.code == K.KVATTN_EINVAL
    bad = bytearray(blobs[0])
    bad[S.record_offset(2, 8, 128, 50, 1, 1)] = 7               # last V record's type
    roomy = K.Context(2, wl.n_head, wl.n_head_kv, wl.head_dim, 256, 1, 4, 64, 64, device="cuda:0")
    with pytest.raises(K.KvattnError) as e:
        roomy.state_load(0, torch.frombuffer(bad, dtype=torch.uint8).to("cuda:0"))
    assert e.value.code == K.KVATTN_EINVAL
    with pytest.raises(K.KvattnError):
        roomy.state_load(0, dev[:-4])                             # truncated
    assert (roomy.cells(0)[0] == -1).all()
    assert roomy.state_load(0, dev) == 0
    assert blob_bytes(roomy.state_save(0)) == blobs[0]
    empty = roomy.state_save(3)
    assert empty.numel() == S.state_bytes(2, 8, 128, 0) and blob_bytes(empty) == S.save(
        OracleEngine(2, wl.n_head, wl.n_head_kv, wl.head_dim, 256, 1, 4, 64, 64), 3)


def test_full_size_rows_and_round_trip():
    L, E, n = 28, 1024, 2048
    dev = torch.device("cuda:0")
    print("seqstate: full size, 28 layers, 2048 positions", flush=True)
    src = K.Context(L, 16, 8, 128, 4096, 1, 2, 2048, 512, device="cuda:0", attend_layers=L,
                    cell_order=np.random.default_rng(3).permutation(4096).astype(np.int32)[None, :])
    g = torch.Generator(device=dev)
    g.manual_seed(11)
    st, ubs, _ = src.split(n, list(range(n)), [(0,)] * n, None)
    assert st == 0
    for u in ubs:
        k = [torch.randn((u.n_tokens, E), generator=g, device=dev) for _ in range(L)]
        v = [torch.randn((u.n_tokens, E), generator=g, device=dev) for _ in range(L)]
        src.store(u, 0, k, v)
    blob = src.state_save(0)
    torch.cuda.synchronize()
    assert blob.numel() == S.state_bytes(L, 8, 128, n)
    head = blob[:80 + 4 * n].cpu().numpy().tobytes()
    assert head[:4] == b"KVSS" and np.array_equal(np.frombuffer(head, "<i4", n, 80), np.arange(n))
    pos, _ = src.cells(0)
    cells = torch.as_tensor(np.argsort(np.where(pos >= 0, pos, 1 << 30))[:n], device=dev)
    rec = 12 + n * E * 2
    for kind, T in enumerate((src.K, src.V)):
        for l in range(L):
            off = 80 + 4 * n + (kind * L + l) * rec + 12
            rows = blob[off:off + n * E * 2].view(n, E * 2)
            want = T[l][0].index_select(0, cells).contiguous().view(torch.uint8).view(n, E * 2)
            assert torch.equal(rows, want), (kind, l)
    dst = K.Context(L, 16, 8, 128, 4096, 1, 8, 2048, 512, device="cuda:0", attend_layers=L)
    assert dst.state_load(5, blob) == 0
    again = dst.state_save(5)
    torch.cuda.synchronize()
    assert torch.equal(again, blob)
