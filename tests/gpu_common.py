"""Shared helpers of the GPU parity tests (imported by the gpu test modules)."""
import numpy as np
import torch

from bit_sparse_attention_amd.workloads import bf16_bits

ATOL = 2e-3     # max abs error of the output against the oracle's declared numerics
REL_L2 = 1e-3   # relative L2 error bound, same reference


def bits(t, BH=None):
    """bf16 tensor [B,H,N,D] -> numpy uint16 [B*H,N,D]."""
    a = bf16_bits(t.detach().cpu())
    return a.reshape(-1, a.shape[-2], a.shape[-1])


def flat(t):
    a = t.detach().cpu().numpy()
    return a.reshape((-1,) + a.shape[2:])


def say(msg):
    print(msg, flush=True)


def check_attn(got32, got16, ref, what):
    """got32/got16: [R, D] GPU rows (fp32, bf16 as float); ref: oracle dict."""
    decl, amb = ref["decl"], ref["amb"]
    err = np.abs(got32 - decl)
    bound = ATOL + amb[:, None]
    bad = err > bound
    assert not bad.any(), f"{what}: {bad.sum()} elements over 2e-3 (+flip bound); max {err.max():.3e}"
    rel = np.linalg.norm(got32 - decl) / max(np.linalg.norm(decl), 1e-30)
    assert rel <= REL_L2, f"{what}: rel-L2 {rel:.3e} > 1e-3"
    # bf16 output = round-to-nearest-even of the fp32 result
    want16 = torch.from_numpy(got32.astype(np.float32)).to(torch.bfloat16).float().numpy()
    assert np.array_equal(got16, want16), f"{what}: bf16 output is not RNE of the fp32 output"
    rel_exact = np.linalg.norm(got32 - ref["exact"]) / max(np.linalg.norm(ref["exact"]), 1e-30)
    return rel, float(err.max()), rel_exact
