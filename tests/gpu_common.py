"""Shared set-up for the GPU tests (not collected by pytest)."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import kv_cache_calibration_amd as nsnq  # noqa: E402
from tests.golden import load_codebook  # noqa: E402

requires_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a HIP GPU")

DEV = "cuda:0"


def table_for(m, G=128, scale_adjust=True, codebook=None):
    """(Params, device table, float32 numpy codebook) for the golden codebook."""
    C = load_codebook(m) if codebook is None else np.asarray(codebook, np.float32)
    p = nsnq.Params(sub_dim=m, group_size=G, scale_adjust=scale_adjust)
    cb = torch.from_numpy(C).to(DEV)
    table = torch.empty(nsnq.nsn_table_size(p), dtype=torch.uint8, device=DEV)
    nsnq.nsn_prepare_codebook(p, cb, table)
    return p, table, C


def alloc_outputs(n_seq, cap, m, G):
    codes = torch.zeros((n_seq, cap, 128 // m), dtype=torch.uint8, device=DEV)
    meta = torch.zeros((n_seq, cap, 2), dtype=torch.float16, device=DEV)
    shift = torch.zeros((n_seq, cap // G, 128), dtype=torch.float16, device=DEV)
    return codes, meta, shift


def quantize_gpu(x_np, m, G, scale_adjust=True, p_table=None):
    """Quantize host array x (n_seq, T, 128) on the GPU; returns numpy outputs
    plus the device tensors."""
    p, table, C = p_table or table_for(m, G, scale_adjust)
    x = torch.from_numpy(np.ascontiguousarray(x_np)).to(DEV)
    n_seq, T, _ = x.shape
    codes, meta, shift = alloc_outputs(n_seq, T, m, G)
    nsnq.nsn_quantize(p, x, table, codes, meta, shift)
    torch.cuda.synchronize()
    return (codes.cpu().numpy(), meta.cpu().numpy(), shift.cpu().numpy(), (codes, meta, shift),
            (p, table, C))
