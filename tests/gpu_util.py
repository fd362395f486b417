"""Helpers for the GPU tests: move bf16 bit patterns between numpy and the device."""
import numpy as np
import torch

from packed_full_attention_amd import workloads as wl


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns (numpy) -> torch.bfloat16 on cuda:0, same shape."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda")


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def host_f64(t: torch.Tensor) -> np.ndarray:
    return wl.bf16_bits_to_f32(host_bits(t)).astype(np.float64)


def dev_inputs(inp: wl.Inputs):
    """Device copies of one workload's inputs (q, k, v, gamma_q, gamma_k, pos)."""
    return (dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v),
            torch.from_numpy(inp.gamma_q).to("cuda"), torch.from_numpy(inp.gamma_k).to("cuda"),
            torch.from_numpy(inp.pos).to("cuda"))


def head_f64(bits: np.ndarray):
    """Accessor h -> float64 [L, 128] slice of a bf16 [L, H, 128] array."""
    return lambda h: wl.bf16_bits_to_f32(np.ascontiguousarray(bits[:, h, :])).astype(np.float64)


def sample_rows(w: wl.Workload, n: int, seed: int) -> np.ndarray:
    """Rows checked one by one on the long workloads: modality boundaries, the
    last two 64-key tiles, and n random rows."""
    L = w.seq_len
    special = [0, 1, w.n_text - 1, w.n_text, w.n_text + w.n_video - 1, w.n_text + w.n_video,
               L - 129, L - 128, L - 65, L - 64, L - 2, L - 1]
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([special, rng.choice(L, n, replace=False)])).astype(np.int64)


def sample_heads(w: wl.Workload) -> np.ndarray:
    return np.unique([0, w.heads // 3, (2 * w.heads) // 3, w.heads - 1]).astype(np.int64)
