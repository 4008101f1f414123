"""Helpers shared by the GPU parity tests (no attention arithmetic here)."""
import sys

import numpy as np

# tolerances (max-abs): bf16 inputs with fp32 accumulation, and the fp32 path
O_ATOL = {"bf16": 2e-2, "f32": 1e-5}
LSE_ATOL = {"bf16": 1e-3, "f32": 1e-5}


def say(msg: str) -> None:
    """Name the case before a GPU step, flushed, so a crash log shows it."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(x: np.ndarray, dtype: str, device):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x)).to(device)
    return t.to(torch.bfloat16) if dtype == "bf16" else t.to(torch.float32)


def to_host(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def sample_rows(N: int, rng, extra: int = 40) -> np.ndarray:
    """Rows at wave and block edges (32, 64, 128, 256), the middle, the end,
    plus random ones."""
    fixed = [0, 1, 2, 31, 32, 63, 64, 65, 127, 128, 129, 255, 256, 257,
             N // 2 - 1, N // 2, N - 2, N - 1]
    rows = np.concatenate([np.array(fixed), rng.choice(N, size=min(extra, N), replace=False)])
    return np.unique(np.clip(rows, 0, N - 1))


def assert_close(name, got, want, atol):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (name, got.shape, want.shape)
    if np.isinf(want).any():
        # -inf entries (empty softmax) must match exactly
        inf = np.isinf(want)
        assert np.array_equal(got[inf], want[inf]), f"{name}: infinite entries differ"
        got, want = got[~inf], want[~inf]
    assert not np.isnan(got).any(), f"{name}: NaN in GPU result"
    err = float(np.max(np.abs(got - want))) if got.size else 0.0
    assert err <= atol, f"{name}: max-abs error {err:.3e} > {atol:.1e}"
    return err
