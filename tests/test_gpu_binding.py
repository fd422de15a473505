"""The binding refuses mis-sized outputs before any kernel is launched."""
import pytest
import torch

import long_context_attention_dca_amd as dca
from long_context_attention_dca_amd import inputs

pytestmark = pytest.mark.gpu


def test_entry_points_refuse_missized_outputs():
    dev = torch.device("cuda:0")
    q, k, v = (x.to(dev) for x in inputs.prefill_inputs(1, 200, 4, 2, 128, "bf16", seed=1))
    with pytest.raises(ValueError):
        dca.rope_remap(k, dca.DCA_MAP_KEY, 128, 32, out=torch.empty(1, 199, 2, 128, dtype=k.dtype, device=dev))
    with pytest.raises(ValueError):
        dca.coarse_fine_key_remap(k, 64, 128, 256, out=torch.empty(1, 200, 2, 64, dtype=k.dtype, device=dev))
    ws = dca.prefill_prepare(k, v, 128, 32)
    with pytest.raises(ValueError):
        dca.prefill_attend(q, ws, 2, 128, 32, out=torch.empty(1, 200, 3, 128, dtype=q.dtype, device=dev))
    with pytest.raises(ValueError):
        dca.prefill_attend(q, ws, 2, 128, 32, lse=torch.empty(1, 4, 199, dtype=torch.float32, device=dev))
    with pytest.raises(TypeError):
        dca.prefill_attend(q, ws, 2, 128, 32, lse=torch.empty(1, 4, 200, dtype=torch.bfloat16, device=dev))
    with pytest.raises(ValueError):
        dca.prefill_attend(q, ws[:1024], 2, 128, 32)
    kc = dca.rope_remap(k, dca.DCA_MAP_KEY, 128, 32)
    with pytest.raises(ValueError):
        dca.prefill_chunk(q[:, 100:].contiguous(), kc, v, 100, 128, 32,
                          out=torch.empty(1, 99, 4, 128, dtype=q.dtype, device=dev))
    # the matching outputs are accepted and give the same result as fresh ones
    o = torch.empty_like(q)
    lse = torch.empty(1, 4, 200, dtype=torch.float32, device=dev)
    dca.prefill_attend(q, ws, 2, 128, 32, out=o, lse=lse)
    assert torch.equal(o, dca.prefill(q, k, v, 128, 32))
