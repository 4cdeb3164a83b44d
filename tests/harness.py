"""Shared helpers of the GPU parity tests and the benchmark's checks: move
workload arrays to the GPU, run the HIP path through the C ABI, and bring
both sides into the canonical form (distinct keys sorted; rows compared by
key, never by offset).  Holds no arithmetic of the method."""
from __future__ import annotations

import numpy as np

import oracle
from dynamic_embedding_tables_amd import recis


def device_features(batch):
    import torch
    out = []
    for f in batch.features:
        v = torch.from_numpy(np.ascontiguousarray(f.values, dtype=np.int64)).cuda()
        o = torch.from_numpy(np.ascontiguousarray(f.bag_offsets, dtype=np.int32)).cuda()
        out.append(recis.DeviceFeature(v, o, f.slot, f.ops, f.mod, f.boundaries))
    return out


def device_grad(batch, spec):
    import torch
    g = batch.grad
    if spec.grad_dtype == "bf16":
        from workloads import to_bf16_bits
        bits = to_bf16_bits(g)
        return torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16), bits
    return torch.from_numpy(np.ascontiguousarray(g, dtype=np.float32)).cuda(), g


def make_table(spec, **kw):
    return recis.Table(spec.dim, spec.dtype, spec.optim, seed=spec.seed, init_bound=spec.init_bound,
                       admit_threshold=spec.admit_threshold, **kw)


def lookup_flags(spec, find_only=False):
    f = recis.RECIS_GROUP_BY_OCCURRENCE if spec.pool == "none" else 0
    return f | (recis.RECIS_FIND_ONLY if find_only else 0)


def forward_out(spec, batch, res):
    import torch
    if spec.pool == "none":
        dt = torch.bfloat16 if spec.dtype == "bf16" else torch.float32
        return torch.empty(res.n, spec.dim, dtype=dt, device="cuda")
    return torch.empty(batch.batch, batch.num_feats * spec.dim, dtype=torch.float32, device="cuda")


def canon_lookup(res):
    """numpy view of a GPU lookup: sorted keys, per-occurrence key, counts and
    row presence by key, merged offsets."""
    U = res.U()
    n = res.n
    keys = res.unique_keys[:U].cpu().numpy()
    rows = res.unique_rows[:U].cpu().numpy()
    counts = res.counts[:U].cpu().numpy()
    inv = res.inverse[:n].cpu().numpy()
    order = np.argsort(keys, kind="stable")
    return {
        "keys": keys[order], "rows": rows[order], "counts": counts[order],
        "occ_keys": keys[inv] if n else np.zeros(0, np.int64),
        "offsets": res.bag_offsets.cpu().numpy(),
        "raw_keys": keys, "raw_inv": inv,
    }


def check_lookup(g, r):
    """Bit-exact lookup parity (distinct keys, inverse, counts, offsets, rows present)."""
    U = r.U
    np.testing.assert_array_equal(g["keys"], r.unique_keys[:U])
    np.testing.assert_array_equal(g["occ_keys"], r.unique_keys[r.inverse[:r.n]] if r.n else np.zeros(0, np.int64))
    np.testing.assert_array_equal(g["counts"], r.counts[:U])
    np.testing.assert_array_equal(g["offsets"], r.merged_offsets)
    np.testing.assert_array_equal(g["rows"] >= 0, r.unique_rows[:U] >= 0)


def canon_export(table):
    import torch
    ex = table.export()
    keys = ex["keys"].cpu().numpy()
    order = np.argsort(keys, kind="stable")
    params = ex["params"].float().cpu().numpy() if ex["params"].dtype == torch.bfloat16 else ex["params"].cpu().numpy()
    return {
        "keys": keys[order], "rows": ex["rows"].cpu().numpy()[order],
        "counts": ex["counts"].cpu().numpy().astype(np.uint32)[order],
        "params": params[order], "state": ex["state"].cpu().numpy()[order],
    }


def check_export(g, o, spec, rtol_state=1e-5):
    """Keys, counts and row presence exact; params within the tolerance of the
    storage dtype (1e-5 fp32, 1e-2 bf16, relative to max(|w|, lr)); optimizer
    state within 1e-5 of its scale.  Adagrad's accumulator and Adam's v add
    non-negative terms, so their scale is their value.  Adam's m = b1*m +
    (1-b1)*G can cancel; its terms are bounded through v (each past
    (1-b1)|G_t| <= (1-b1) sqrt(v / ((1-b2) b2^k))), so its scale is
    |m| + sqrt(v / (1 - b2))."""
    np.testing.assert_array_equal(g["keys"], o["keys"])
    np.testing.assert_array_equal(g["counts"], o["counts"])
    np.testing.assert_array_equal(g["rows"] >= 0, o["rows"] >= 0)
    has = o["rows"] >= 0
    tol = 1e-2 if spec.dtype == "bf16" else 1e-5
    scale = np.maximum(np.abs(o["params"][has]), spec.lr if spec.optim != "none" else 0.0)
    err = np.abs(g["params"][has] - o["params"][has])
    bad = err > tol * scale + 1e-30
    assert not bad.any(), f"{bad.sum()} param elements off; worst {np.max(err / np.maximum(scale, 1e-30))}"
    if o["state"].size:
        s_ref = o["state"][has].astype(np.float64)
        sc = np.abs(s_ref)
        if spec.optim == "adam":
            D = spec.dim
            v = s_ref[:, D:]
            sc[:, :D] = np.abs(s_ref[:, :D]) + np.sqrt(v / (1.0 - spec.beta2))
        se = np.abs(g["state"][has] - s_ref)
        sb = se > rtol_state * sc + 1e-12
        assert not sb.any(), f"{sb.sum()} state elements off; worst {np.max(se / np.maximum(sc, 1e-30))}"


def check_forward(out_gpu, spec, oracle_out, oracle_abs, merged_offsets=None, num_feats=1, exact=None):
    """gather: a copy of the stored rows -- bit-exact while every row still holds
    its initial values (exact=True, the first step), afterwards within the
    parameter tolerance (rows updated on both sides may differ by an ulp).
    pooled: |y - y_ref| <= tol * (sum |terms| + terms * lr), the summation-order
    bound of fp32 plus the parameter tolerance that earlier updates may already
    have used (terms = bag length for sum, 1 for mean); tol = 1e-5, or 1e-2 for
    bf16 storage once rows have been updated (the stored rows themselves may
    then differ by a bf16 rounding step, within the 1e-2 relative bar for bf16
    storage on pooled outputs and updated rows)."""
    if spec.pool == "none":
        import torch
        if spec.dtype == "bf16":
            g = out_gpu.view(torch.int16).cpu().numpy().view(np.uint16)
        else:
            g = out_gpu.cpu().numpy()
        if exact or spec.optim == "none":
            np.testing.assert_array_equal(g, oracle_out)
            return
        to_f = (lambda b: (b.astype(np.uint32) << 16).view(np.float32)) if spec.dtype == "bf16" else (lambda x: x)
        gv, ov = to_f(g).astype(np.float64), to_f(oracle_out).astype(np.float64)
        tol = 1e-2 if spec.dtype == "bf16" else 1e-5
        bad = np.abs(gv - ov) > tol * np.maximum(np.abs(ov), spec.lr)
        assert not bad.any(), f"{bad.sum()} gathered elements off"
        return
    g = out_gpu.cpu().numpy()
    err = np.abs(g.astype(np.float64) - oracle_out.astype(np.float64))
    tol = 1e-2 if spec.dtype == "bf16" and not exact and spec.optim != "none" else 1e-5
    bound = tol * oracle_abs
    if merged_offsets is not None and spec.optim != "none":
        B = g.shape[0]
        lens = np.diff(merged_offsets.astype(np.int64)).reshape(num_feats, B).T   # [B, F]
        terms = lens if spec.pool == "sum" else (lens > 0).astype(np.int64)
        bound = bound + tol * spec.lr * np.repeat(terms, spec.dim, axis=1)
    bad = err > bound + 1e-30
    assert not bad.any(), f"{bad.sum()} pooled elements off; worst {np.max(err - bound)}"


def check_gather_is_copy(out_gpu, table, res, spec):
    """POOL_NONE: every output row is bit for bit the row the table itself
    holds for that occurrence's key (its export, read between the forward and
    the backward), zeros for a key without a row."""
    import torch
    ex = table.export()
    ekeys = ex["keys"].cpu().numpy()
    order = np.argsort(ekeys, kind="stable")
    ekeys = ekeys[order]
    erows = ex["rows"].cpu().numpy()[order]
    p = ex["params"]
    eparams = (p.view(torch.int16).cpu().numpy().view(np.uint16) if p.dtype == torch.bfloat16
               else p.cpu().numpy().view(np.uint32))[order]
    g = out_gpu[:res.n]
    g = g.view(torch.int16).cpu().numpy().view(np.uint16) if g.dtype == torch.bfloat16 else g.cpu().numpy().view(np.uint32)
    U = res.U()
    occ_keys = res.unique_keys[:U].cpu().numpy()[res.inverse[:res.n].cpu().numpy()]
    pos = np.searchsorted(ekeys, occ_keys)
    pos_c = np.minimum(pos, max(ekeys.size - 1, 0))
    found = (pos < ekeys.size) & (ekeys[pos_c] == occ_keys) if ekeys.size else np.zeros(occ_keys.size, bool)
    has = np.zeros(occ_keys.size, bool)
    has[found] = erows[pos_c[found]] >= 0
    want = np.zeros_like(g)
    want[has] = eparams[pos_c[has]]
    np.testing.assert_array_equal(g, want)


def gpu_step(table, spec, batch, res, find_only=False, with_backward=True, after_forward=None):
    """insert_find -> forward -> backward+update on the current stream;
    after_forward(out) runs between the forward and the backward."""
    feats = device_features(batch)
    table.insert_find(feats, batch.batch, res, flags=lookup_flags(spec, find_only))
    out = forward_out(spec, batch, res)
    table.forward(res, spec.pool, out)
    if after_forward is not None:
        after_forward(out)
    if with_backward and spec.optim != "none":
        g, _ = device_grad(batch, spec)
        table.backward_update(res, spec.pool, g, spec.grad_dtype, lr=spec.lr, beta1=spec.beta1,
                              beta2=spec.beta2, eps=spec.eps)
    return out, feats


def oracle_step(otab, spec, batch, find_only=False, with_backward=True):
    r = otab.insert_find(batch.features, batch.batch, flags=oracle.FIND_ONLY if find_only else 0)
    assert r.status == 0, r.status
    if spec.pool == "none":
        out, ab = otab.forward(r, "none"), None
    else:
        out, ab = otab.forward(r, spec.pool, with_abs=True)
    if with_backward and spec.optim != "none":
        g = batch.grad
        if spec.grad_dtype == "bf16":
            from workloads import to_bf16_bits
            g = to_bf16_bits(g)
        assert otab.backward_update(r, spec.pool, g, spec.grad_dtype) == 0
    return r, out, ab
