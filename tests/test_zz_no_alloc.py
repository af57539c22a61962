"""zebra_linear_attn_noalloc (linear stage with the library's static device
scratch, for callers that cannot allocate) against zebra_linear_attn (the
same stage with a caller-provided workspace), through the C ABI: two calls
in a row on one device, the second with a smaller layout, each within the
stage tolerance of the allocating entry point's output (max-abs 2e-2,
mean-abs 2e-3)."""
import numpy as np
import pytest
import torch

import linear_global_attention_amd as zb
import zebra_synth as zs
from gpu_helpers import Stage, bf16_host, close, dev_f32, log

pytestmark = pytest.mark.gpu


def _both(L, seed):
    q, k, v = zs.stage_inputs(L, seed=seed)
    W, b = zs.affine_params(L, seed=seed)
    g = np.random.default_rng(seed)
    mu = (0.01 * g.standard_normal((L.heads, 64))).astype(np.float32)
    gq = (0.5 + g.random((L.heads, 64))).astype(np.float32)
    st = Stage(L, q, k, v, 0.0, sparse=False)
    kw = dict(W=dev_f32(W), b=dev_f32(b), mu=dev_f32(mu), gq=dev_f32(gq))
    zb.linear_attn(st.args(**kw))
    torch.cuda.synchronize()
    want = bf16_host(st.out)
    st.out.fill_(0x7F7F)  # stale values must not survive
    a = st.args(**kw)
    a.workspace, a.workspace_bytes = None, 0
    zb.linear_attn_noalloc(a)
    torch.cuda.synchronize()
    got = bf16_host(st.out)
    same = bool(np.array_equal(got, want))
    log(f"noalloc {L}: bit-identical to zebra_linear_attn: {same}")
    close(got, want, f"noalloc vs zebra_linear_attn {L.frames} frames")


def test_noalloc_linear_two_calls_second_smaller():
    _both(zs.Layout(8, 5, 37, 37, heads=4), seed=31)
    _both(zs.Layout(3, 2, 11, 13, heads=2), seed=32)
