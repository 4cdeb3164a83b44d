"""The SafeTensors file layer of the saver, on the host: what is written is
read back bit for bit, with its metadata, and other files are refused."""
import numpy as np
import pytest


def test_roundtrip_all_tensor_kinds(tmp_path):
    import torch
    from dynamic_embedding_tables_amd import saver
    rng = np.random.default_rng(5)
    t = {
        "keys": torch.from_numpy(rng.integers(0, 1 << 62, 100, dtype=np.int64)),
        "has_row": torch.from_numpy((rng.random(100) < 0.7).astype(np.uint8)),
        "counts": torch.from_numpy(rng.integers(1, 1000, 100, dtype=np.int64)),
        "params": torch.from_numpy(rng.standard_normal((100, 16), dtype=np.float32)).to(torch.bfloat16),
        "state": torch.from_numpy(rng.standard_normal((100, 32), dtype=np.float32)),
    }
    p = str(tmp_path / "t.safetensors")
    saver.write(p, t, {"dim": 16, "dtype": "bf16", "adam_step": 7})
    back, meta = saver.read(p)
    assert meta == {"format": saver.FORMAT, "dim": "16", "dtype": "bf16", "adam_step": "7"}
    assert set(back) == set(t)
    for k in t:
        assert back[k].dtype == t[k].dtype and torch.equal(back[k], t[k]), k


def test_other_files_are_refused(tmp_path):
    import torch
    from safetensors.torch import save_file
    from dynamic_embedding_tables_amd import saver
    p = str(tmp_path / "other.safetensors")
    save_file({"x": torch.zeros(3)}, p, metadata={"format": "pt"})
    with pytest.raises(ValueError):
        saver.read(p)
