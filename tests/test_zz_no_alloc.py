"""fa_decode_noalloc (split partials in the library's scratch array, no
workspace) against fa_decode with a caller workspace: the same kernels, so the
same bits; and both against the oracle, to the parity bar.  Two calls in a
row, the second smaller, share the array."""
import numpy as np
import pytest

import oracle
from tests.gpu_util import BF16_LSE_REL_TOL, BF16_O_TOL, bf16_to_device, compare, say, to_f64
from transformer_attention_fa_amd import api, inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu(require_gpu):
    api.load()


def _case(spec, lens, splits):
    import torch
    data = inputs.decode_inputs(spec, seq_lens=np.array(lens, np.int32))
    q = bf16_to_device(data.q)
    kc, vc = bf16_to_device(data.k_cache), bf16_to_device(data.v_cache)
    dl = torch.from_numpy(data.seq_lens).cuda()
    return data, (q, kc, vc, dl, splits)


def test_noalloc_matches_workspace_entry_twice_shrinking():
    import torch
    big = inputs.Decode("noalloc_big", 32, 32, 8, 128, 1, 9000, 9000, 16, 91)      # 8.45 MB of partials
    small = inputs.Decode("noalloc_small", 3, 12, 4, 64, 1, 700, 700, 5, 93)
    cases = [_case(big, np.random.default_rng(5).integers(1, 9001, 32), 16),
             _case(small, [1, 300, 700], 5)]
    for data, (q, kc, vc, dl, S) in cases:
        spec = data.spec
        say(f"fa_decode_noalloc {spec.name} S={S}")
        o_n, l_n = api.decode_noalloc(q, kc, vc, dl, num_splits=S, scale=spec.scale)
        torch.cuda.synchronize()
        o_w, l_w = api.decode(q, kc, vc, dl, num_splits=S, scale=spec.scale)
        torch.cuda.synchronize()
        assert torch.equal(o_n.view(torch.int16), o_w.view(torch.int16))
        assert torch.equal(l_n.view(torch.int32), l_w.view(torch.int32))
        o_ref, lse_ref = oracle.decode(data.q, data.k_cache, data.v_cache, data.seq_lens, spec.scale)
        compare(to_f64(o_n), to_f64(l_n), o_ref, lse_ref, BF16_O_TOL, BF16_LSE_REL_TOL, label=f"noalloc {spec.name}")


def test_noalloc_rejects_oversized_partials():
    import torch
    spec = inputs.Decode("noalloc_over", 2, 4, 1, 128, 1, 64, 64, 16, 95)
    data, (q, kc, vc, dl, _) = _case(spec, [64, 64], 16)
    with pytest.raises(api.FAError, match="num_splits"):
        api.decode_noalloc(q, kc, vc, dl, num_splits=4096)      # num_splits > 256 is invalid first
    # 16 MiB holds B*H*S*(d+1)*4 bytes up to 2032 rows of 16 splits at d = 128: 8000 rows exceed it
    q_big = torch.zeros((8000, 1, 128), dtype=torch.bfloat16, device="cuda")
    kc_big = torch.zeros((8000, 1, 16, 128), dtype=torch.bfloat16, device="cuda")
    dl_big = torch.full((8000,), 16, dtype=torch.int32, device="cuda")
    with pytest.raises(api.FAError, match="scratch"):
        api.decode_noalloc(q_big, kc_big, kc_big, dl_big, num_splits=16)
