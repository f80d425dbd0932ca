"""Helpers for the GPU parity tests: moving rank buffers to and from the GPU
and comparing them bit for bit."""
import numpy as np


def dev():
    import torch
    return torch.device("cuda", 0)


def upload(x: list, dtype: str):
    """Stack p host rank buffers into one [p, n] GPU tensor."""
    import torch
    arr = np.stack(x) if len(x) else np.zeros((0, 0), np.float32)
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(arr.astype(np.float32))).to(dev())
    t = torch.from_numpy(np.ascontiguousarray(arr.astype(np.uint16)).view(np.int16)).to(dev())
    return t.view(torch.bfloat16)


def upload_list(x: list, dtype: str):
    return [upload([v], dtype)[0] for v in x]


def download(t, dtype: str) -> np.ndarray:
    import torch
    if dtype == "f32":
        return t.detach().cpu().numpy().view(np.uint32)
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def bits(x: np.ndarray, dtype: str) -> np.ndarray:
    return np.asarray(x).view(np.uint32 if dtype == "f32" else np.uint16)


def assert_bits_equal(got: np.ndarray, want: np.ndarray, what: str) -> None:
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, f"{what}: shape {got.shape} != {want.shape}"
    bad = np.flatnonzero(got.ravel() != want.ravel())
    assert bad.size == 0, (f"{what}: {bad.size} of {got.size} elements differ; first at {bad[:5].tolist()}: "
                           f"got {got.ravel()[bad[:5]].tolist()} want {want.ravel()[bad[:5]].tolist()}")


def say(msg: str) -> None:
    print(msg, flush=True)
