"""Helpers shared by the tests: torch tensors -> the oracle's NumPy storage forms."""
import json
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def np_store(t: torch.Tensor) -> np.ndarray:
    """Stored form: bf16 -> uint16 bit patterns, fp32 -> float32, ints as is."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bf16_bits(x) -> np.ndarray:
    """float values exactly representable in bf16 -> uint16 bits."""
    f = np.asarray(x, dtype=np.float32)
    b = f.view(np.uint32)
    assert not np.any(b & 0xFFFF), "not a bf16 value"
    return (b >> 16).astype(np.uint16)


def case_np(case):
    """The arrays of a workloads.PagedCase in oracle form."""
    d = dict(
        q=np_store(case.q), k_pool=np_store(case.k_pool), v_pool=np_store(case.v_pool),
        page_indptr=np_store(case.page_indptr), page_indices=np_store(case.page_indices),
        seq_lens=np_store(case.seq_lens), dtype=case.dtype, Hkv=case.Hkv,
    )
    if case.prefix_pages is not None:
        d["prefix_pages"] = np_store(case.prefix_pages)
    return d
