"""moe_forward_noalloc: the layer with the library's own per-GPU workspace, for callers that cannot
allocate. Its output must equal moe_forward's (same kernels) bit for bit, on consecutive calls that reuse
the same library-owned array, the second with a smaller input; a call whose workspace would exceed the
array is refused before anything is enqueued."""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import dev_tensor, dims_of, packed_of, shared_of, upload

pytestmark = pytest.mark.gpu


def _both(cfg, d, M, with_shared):
    import mxfp4_routed_expert_moe_amd as m
    dims = dims_of(cfg)
    sh = shared_of(d) if with_shared else None
    res = []
    for noalloc in (False, True):
        out = torch.full((M, cfg.H), 0x7FC0, dtype=torch.int16, device="cuda")
        ids = torch.full((M, cfg.k), -7, dtype=torch.int32, device="cuda")
        rw = torch.full((M, cfg.k), float("nan"), dtype=torch.float32, device="cuda")
        sh_out = torch.full((M, cfg.H), 0x7FC0, dtype=torch.int16, device="cuda") if sh is not None else None
        if noalloc:
            m.moe_forward_noalloc(dims, d["x"][:M], d["gate_w"], d["gate_b"], packed_of(d), None, sh, out, ids, rw,
                                  sh_out)
        else:
            m.moe_forward(dims, d["x"][:M], d["gate_w"], d["gate_b"], packed_of(d), None, sh, out, ids, rw, sh_out,
                          m.workspace(dims, M))
        torch.cuda.synchronize()
        res.append((out.cpu().numpy(), ids.cpu().numpy(), rw.cpu().numpy().view(np.int32),
                    None if sh_out is None else sh_out.cpu().numpy()))
    for a, b in zip(res[0], res[1]):
        if a is not None:
            assert np.array_equal(a, b)
    return res[1]


def test_noalloc_equals_forward_full_size_two_calls():
    """The full-size layer (hidden 5120, 128 experts, intermediate 2304, top-6): 64 tokens, then 8."""
    cfg = synth.get_config(2)
    d = upload(synth.make_inputs(cfg))
    first = _both(cfg, d, 64, False)
    second = _both(cfg, d, 8, False)
    # the smaller call's outputs are those of its own tokens, not leftovers of the first call
    assert np.array_equal(second[1], first[1][:8])
    assert np.array_equal(second[0], first[0][:8])


def test_noalloc_equals_forward_with_shared_expert_two_calls():
    """A layer with the FP8 shared expert: 37 tokens, then 5."""
    cfg = synth.get_config(0, M=37, H=512, I=256, E=8, k=2, shared=True)
    d = upload(synth.make_inputs(cfg))
    _both(cfg, d, 37, True)
    _both(cfg, d, 5, True)


def test_noalloc_refuses_beyond_its_workspace():
    import mxfp4_routed_expert_moe_amd as m
    cfg = synth.get_config(2)
    dims = dims_of(cfg)
    M = 256
    assert m.moe_workspace_bytes(dims, M) > m.NOALLOC_SCRATCH_BYTES
    x = dev_tensor(np.zeros((M, cfg.H), dtype=np.uint16))
    gw = torch.zeros((cfg.E, cfg.H), dtype=torch.float32, device="cuda")
    gb = torch.zeros(cfg.E, dtype=torch.float32, device="cuda")
    w = torch.zeros(16, dtype=torch.uint8, device="cuda")
    pk = m.MXFP4Experts(w, w, w, w, w, w)
    out = torch.empty((M, cfg.H), dtype=torch.int16, device="cuda")
    with pytest.raises(m.MoeError, match="MOE_ERR_WORKSPACE"):
        m.moe_forward_noalloc(dims, x, gw, gb, pk, None, None, out)
