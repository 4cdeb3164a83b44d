"""The allocation-free backward (recis_pool_bwd_update_noalloc) against the
backward it is a variant of (recis_pool_bwd_update), through the C ABI: two
tables fed the same lookups, one updated by each entry point, must hold the
same keys, counts and rows, and parameters and optimizer state within the
parity bar -- over two calls in a row, the second smaller than the first,
so the shared fixed scratch still holds the first call's partials when the
second runs.  The no-allocation call makes no allocator call, and a call too
large for the fixed scratch is refused before any work."""
import numpy as np
import pytest

import workloads as W
from harness import canon_export, check_export, device_features, forward_out, make_table

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from dynamic_embedding_tables_amd import recis
    recis.load_library()


def _step(table, spec, b, noalloc):
    import torch
    from dynamic_embedding_tables_amd import recis
    res = recis.LookupResult(b.n, b.num_feats * b.batch)
    flags = recis.RECIS_GROUP_BY_OCCURRENCE if spec.pool == "none" else 0
    table.insert_find(device_features(b), b.batch, res, flags=flags)
    out = forward_out(spec, b, res)
    table.forward(res, spec.pool, out)
    g = torch.from_numpy(np.ascontiguousarray(b.grad, dtype=np.float32)).cuda()
    if spec.grad_dtype == "bf16":
        g = g.to(torch.bfloat16)
    before = recis.allocator_calls()
    table.backward_update(res, spec.pool, g, spec.grad_dtype, lr=spec.lr, beta1=spec.beta1, beta2=spec.beta2,
                          eps=spec.eps, noalloc=noalloc)
    if noalloc:
        assert recis.allocator_calls() == before, "the allocation-free backward called the allocator"
    return res


@pytest.mark.parametrize("case", ["ctr_adam_mean", "seq_bf16_gather"])
def test_noalloc_backward_matches_the_backward(case):
    import torch
    if case == "ctr_adam_mean":
        spec = W.spec_ctr()
        batches = [W.ctr_batch(0, batch=2048, num_feats=8), W.ctr_batch(1, batch=300, num_feats=3)]
    else:
        spec = W.spec_seq()
        batches = [W.seq_batch(0, batch=24, seq_len=1000), W.seq_batch(1, batch=5, seq_len=1000)]
    # the reference takes the bag-major pass for its hot keys wherever it can
    # (pooled, dim 64 or 128); the allocation-free call always sums key by key
    ref, mine = make_table(spec, hot_grad_bytes=1), make_table(spec)
    for k, b in enumerate(batches):
        print(f"[noalloc] {case} call {k} N={b.n}", flush=True)
        r1 = _step(ref, spec, b, noalloc=False)
        r2 = _step(mine, spec, b, noalloc=True)
        torch.cuda.synchronize()
        assert ref.get_error() == 0 and mine.get_error() == 0
        assert r1.U() == r2.U()
        long_keys = int(r1.plan[0].item())
        assert k > 0 or long_keys > 0, "the first call must have long keys (chunk partials in the scratch)"
        # keys, counts and row presence exact; parameters and state to the
        # parity bar (the two lookups may group a key's occurrences in another
        # order, and double sums in another order can round differently)
        check_export(canon_export(mine), canon_export(ref), spec)
        assert ref.stats().adam_step == mine.stats().adam_step
    ref.close()
    mine.close()


def test_noalloc_backward_refuses_a_call_beyond_its_scratch():
    import torch
    from dynamic_embedding_tables_amd import recis
    spec = W.TableSpec(dim=256, dtype="f32", optim="adam", pool="sum", lr=1e-3, eps=1e-8)
    lim = recis.recis_noalloc_scratch_bytes()
    assert lim == 64 << 20
    # n occurrences may need n/32 + 2 chunk partials of 256 doubles (2 KiB each)
    n = (lim // (256 * 8)) * 32 + 4096
    table = make_table(spec)
    vals = np.arange(n, dtype=np.int64) % 1000
    b = W.Batch([W.FeatureInput(values=vals, bag_offsets=np.array([0, n], np.int32), slot=0)], 1,
                np.ones((1, 256), np.float32))
    res = recis.LookupResult(n, 1)
    table.insert_find(device_features(b), 1, res)
    g = torch.ones(1, 256, device="cuda")
    with pytest.raises(recis.RecisError) as e:
        table.backward_update(res, "sum", g, "f32", lr=spec.lr, eps=spec.eps, noalloc=True)
    assert e.value.status == recis.RECIS_ERR_INVALID_ARG
    assert table.stats().adam_step == 0       # refused before any work
    table.backward_update(res, "sum", g, "f32", lr=spec.lr, eps=spec.eps)  # the allocating one takes it
    torch.cuda.synchronize()
    assert table.get_error() == 0 and table.stats().adam_step == 1
    table.close()
