"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI and bring results
back to the host as numpy arrays."""
import sys

import numpy as np
import torch

from weight_only_int4_act_amd import inputs as I


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def awq():
    from weight_only_int4_act_amd import awq as mod   # fails loudly when libawq.so is missing
    return mod


def gpu_layer(X_bf16, W_bf16, group_size, zero_point, n_grid=21):
    """stats -> search -> pack on cuda:0; returns host copies of every output."""
    A = awq()
    dev = torch.device("cuda:0")
    X = X_bf16.to(dev)
    W = W_bf16.to(dev)
    cfg = A.qconfig(group_size, zero_point, n_grid)
    r = A.run_layer(X, W, cfg)
    torch.cuda.synchronize()
    q = r["q"]
    return {
        "X": X, "W": W, "cfg": cfg, "q": q,
        "sum_abs": r["sum_abs"].cpu().numpy(),
        "mean_abs": r["mean_abs"].cpu().numpy(),
        "losses": r["losses"].cpu().numpy(),
        "best": int(r["best"].cpu().item()),
        "s_best": q.s.cpu().numpy(),
        "codes": q.codes.cpu().numpy().view(np.uint32),
        "scales": q.scales.cpu().numpy(),
        "zeros": q.zeros.cpu().numpy(),
    }


def gpu_gemm(X_rows_bf16, q):
    A = awq()
    Y = A.gemm(X_rows_bf16.to("cuda:0"), q)
    torch.cuda.synchronize()
    return I.bf16_to_f64(Y)


def rel_fro(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))
