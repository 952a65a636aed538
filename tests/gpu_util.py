"""Helpers for the GPU parity tests (HIP path vs the CPU oracle)."""
import os
import sys

import numpy as np
import pytest

import oracle
import quantized_weight_gemv_q8_amd as q8
from quantized_weight_gemv_q8_amd import synth

torch = pytest.importorskip("torch")


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    rc = q8.device_check(torch.cuda.current_device())
    assert rc == 0, f"device is not gfx950: {q8.status_str(rc)}"


def note(msg: str):
    """Name the case before a GPU step (survives a crash of the step)."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def threads() -> int:
    return min(16, oracle.default_threads())


def upload(q, d):
    return q8.pack(synth.to_gguf_blocks(q, d))


def upload_bank(qb, db):
    E = qb.shape[0]
    blocks = np.stack([synth.to_gguf_blocks(qb[e], db[e]) for e in range(E)])
    return q8.pack_bank(blocks)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def assert_parity(y_gpu, y, A, out_dtype="f32", what=""):
    ok, rel, nbad = oracle.check_close(np.asarray(y_gpu, np.float64), y, A, out_dtype)
    assert ok, f"{what}: {nbad} outputs outside 1e-3*sum|dqx| (max rel {rel:.3e})"
    return rel
