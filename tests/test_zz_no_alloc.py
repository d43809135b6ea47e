"""The allocation-free attention step (for callers that cannot allocate device memory)
against the attention step it varies, through the C ABI: two calls in a row, the
second with a smaller input, each bit for bit equal to ube_step_attention on the
same buffers; a request beyond the fixed buffer is refused before any launch."""
import numpy as np
import pytest

from multimodal_embeddings_amd import synth
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


def _case(lengths, heads, seed):
    import torch
    rng = np.random.default_rng(seed)
    T = int(sum(lengths))
    W = heads * 64
    Tp = (T + 255) // 256 * 256 + 256

    def bf16(shape):
        bits = synth.to_bf16_bits(rng.standard_normal(shape).astype(np.float32))
        return torch.from_numpy(bits.view(np.int16)).to("cuda:0").view(torch.bfloat16)

    q, k = bf16((Tp, W)), bf16((Tp, W))
    vt = torch.zeros((W, Tp), dtype=torch.bfloat16, device="cuda:0")
    vt[:, :T] = bf16((W, T))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.uint32)
    return q, k, vt, cu, T, W, Tp


def test_static_attention_matches_the_allocating_step_on_two_calls():
    import torch
    import multimodal_embeddings_amd as ube
    for lengths, heads, seed in (([300, 1, 1024, 0, 77, 513], 4, 1), ([5, 64, 3], 2, 2)):
        say(f"static attention lengths={lengths} heads={heads}")
        q, k, vt, cu, T, W, Tp = _case(lengths, heads, seed)
        want = torch.full((T, W), float("nan"), dtype=torch.bfloat16, device="cuda:0")
        got = torch.full((T, W), float("nan"), dtype=torch.bfloat16, device="cuda:0")
        ube.step_attention(q, k, W, vt, Tp, want, W, cu, heads)
        ube.step_attention_static(q, k, W, vt, Tp, got, W, cu, heads)
        torch.cuda.synchronize()
        a, b = want.view(torch.int16).cpu().numpy(), got.view(torch.int16).cpu().numpy()
        assert not torch.isnan(want.float()).any()
        np.testing.assert_array_equal(b, a)


def test_static_attention_refuses_requests_beyond_its_buffer():
    import torch
    import multimodal_embeddings_amd as ube
    q = torch.zeros((512, 64), dtype=torch.bfloat16, device="cuda:0")
    o = torch.zeros((256, 64), dtype=torch.bfloat16, device="cuda:0")
    # 300,000 empty items: their bounds alone exceed the 262,144-entry buffer
    cu = np.zeros(300001, np.uint32)
    with pytest.raises(ube.UbeError) as e:
        ube.step_attention_static(q, q, 64, q, 512, o, 64, cu, 1)
    assert e.value.status == "invalid_argument"
