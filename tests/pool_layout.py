"""The paged pool's in-block layout, restated from the public header for the tests
(independently of both the oracle and the library).

A (page, kv head) block holds 16 tokens x D channels:
  K: token t, channel d at (d // 32) * 512 + ((d % 32) // 8) * 128 + t * 8 + d % 8
  V: token t, channel d at (d // 16) * 256 + (t // 4) * 64 + (d % 16) * 4 + t % 4
"""
import numpy as np


def k_offsets(D):
    t = np.arange(16)[:, None]
    d = np.arange(D)[None, :]
    return (d // 32) * 512 + ((d % 32) // 8) * 128 + t * 8 + d % 8


def v_offsets(D):
    t = np.arange(16)[:, None]
    d = np.arange(D)[None, :]
    return (d // 16) * 256 + (t // 4) * 64 + (d % 16) * 4 + t % 4


def pack(logical, offsets):
    """[..., 16, D] token-major blocks -> [..., 16 * D] in the pool layout."""
    lead = logical.shape[:-2]
    D = logical.shape[-1]
    out = np.empty(lead + (16 * D,), logical.dtype)
    out[..., offsets.reshape(-1)] = logical.reshape(lead + (16 * D,))
    return out


def unpack(packed, offsets):
    """[..., 16 * D] pool blocks -> [..., 16, D] token-major."""
    D = offsets.shape[1]
    return packed[..., offsets.reshape(-1)].reshape(packed.shape[:-1] + (16, D))
