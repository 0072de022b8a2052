"""Helpers shared by the GPU tests: host <-> device bf16 transfers, ulp distance, cached
seeded inputs.  Expected values always come from the oracle or from closed forms."""
import functools
import sys

import numpy as np

from global_attention_image_amd.inputs import CONFIGS, CONFIG_SEEDS, make_qkv_bits


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(bits: np.ndarray):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def from_dev(t) -> np.ndarray:
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_bf16_rne(x: np.ndarray) -> np.ndarray:
    """fp64 -> bf16 bits, round to nearest even, without double-rounding error.

    Step 1 rounds to fp32 by round-to-odd (truncate toward zero, then set the last bit if
    anything was dropped); step 2 rounds that fp32 value to bf16 with ties to even.
    Round-to-odd at 23 bits followed by any rounding at 7 bits equals direct rounding.
    """
    x = np.asarray(x, dtype=np.float64)
    f = x.astype(np.float32)
    over = np.abs(f.astype(np.float64)) > np.abs(x)
    f = np.where(over, np.nextafter(f, np.float32(0)), f).astype(np.float32)
    u = f.view(np.uint32).copy()
    u[f.astype(np.float64) != x] |= np.uint32(1)
    lsb = (u >> 16) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> 16).astype(np.uint16)


def bf16_order(bits: np.ndarray) -> np.ndarray:
    """Map bf16 bits to integers whose order is the numeric order (for ulp distances)."""
    b = bits.astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def ulp_distance(a_bits, b_bits) -> np.ndarray:
    return np.abs(bf16_order(a_bits) - bf16_order(b_bits))


@functools.lru_cache(maxsize=2)
def config_inputs(name: str):
    """(geom, q_bits, k_bits, v_bits) for a named workload (cached per process)."""
    geom = CONFIGS[name]
    return (geom,) + make_qkv_bits(geom, CONFIG_SEEDS[name])
