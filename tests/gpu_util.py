"""Helpers shared by the GPU tests: host<->device moves and the parity bars."""

import sys

import numpy as np
import torch

from learned_token_pruning_tg_amd import inputs

# Parity bars (attention outputs bf16 in, fp32 accumulate vs the float64 oracle).
ATTN_MAX_ABS = 1e-2
ATTN_REL_L2 = 5e-3
SCORE_REL = 1e-3


def say(msg: str) -> None:
    """Name the case before a GPU step (flushed, so it survives a crash)."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def dev_bf16(x: np.ndarray) -> torch.Tensor:
    """Upload bf16-exact float32 values as a bf16 tensor (bit copy)."""
    bits = inputs.bf16_bits(inputs.round_bf16(x))
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()


def dev_f32(x) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(np.asarray(x, dtype=np.float32))).cuda()


def host_bf16(t: torch.Tensor) -> np.ndarray:
    bits = t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return inputs.bf16_to_f32(bits)


def check_attn(got: np.ndarray, ref: np.ndarray, what: str) -> None:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), what
    err = np.abs(got - ref)
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    print(f"[attn] {what}: max-abs {err.max():.3e} rel-L2 {rel:.3e}", flush=True)
    assert err.max() <= ATTN_MAX_ABS, f"{what}: max-abs {err.max():.3e}"
    assert rel <= ATTN_REL_L2, f"{what}: rel-L2 {rel:.3e}"


def check_scores(got: np.ndarray, ref: np.ndarray, what: str) -> None:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    floor = SCORE_REL * np.maximum(np.abs(ref), np.sqrt(np.mean(ref ** 2)))
    assert rel <= SCORE_REL, f"{what}: rel-L2 {rel:.3e}"
    bad = np.abs(got - ref) > floor
    assert not bad.any(), f"{what}: {bad.sum()} scores off, worst {np.abs(got - ref).max():.3e}"
