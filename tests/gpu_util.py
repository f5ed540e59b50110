"""Helpers for the GPU tests: moving seeded numpy inputs to the device and
back. No arithmetic of the method lives here."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def dev_bf16(bits: np.ndarray) -> "torch.Tensor":
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def host_bits(t: "torch.Tensor") -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def dev_u8(a: np.ndarray) -> "torch.Tensor":
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def dev_f32(a: np.ndarray) -> "torch.Tensor":
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def same_bits_f32(a: np.ndarray, b: np.ndarray) -> bool:
    return np.array_equal(np.asarray(a, np.float32).view(np.uint32), np.asarray(b, np.float32).view(np.uint32))


def announce(*parts):
    print("[gpu-case]", *parts, flush=True)
