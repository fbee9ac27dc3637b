"""The seeded input generator: determinism, encodings and the workloads' shapes."""
import numpy as np
import pytest
import torch

import gdn_inputs as gi


def test_bf16_encoding_matches_torch_rne():
    x = np.random.default_rng(0).standard_normal(200000).astype(np.float32) * np.float32(7.0)
    x[:4] = [0.0, -0.0, 1e-30, -3.0e38]
    ours = gi.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = gi.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_generator_is_deterministic_and_streams_differ():
    a = gi.tiny_fp32()
    b = gi.tiny_fp32()
    assert a.digest() == b.digest()
    assert not torch.equal(a.q, a.k)
    c = gi.make_inputs(0, [256], 2, 2, 16, 16, io="f32", sub=1)
    assert c.digest() != a.digest()


def test_tiny_shapes_and_distributions():
    x = gi.tiny_fp32()
    assert x.q.shape == (256, 2, 16) and x.v.shape == (256, 2, 16) and x.a.shape == (256, 2)
    assert x.q.dtype == torch.float32 and x.a.dtype == torch.float32
    assert bool((x.a > 0).all() and (x.a < 1).all() and (x.b > 0).all() and (x.b < 1).all())
    nrm = np.linalg.norm(x.widen("k"), axis=-1)
    assert np.allclose(nrm, 1.0, atol=1e-6)
    assert list(x.cu_seqlens) == [0, 256]
    assert abs(float(x.a.double().mean()) - 0.5) < 0.05      # E[sigmoid(-x)] = 1/2


def test_bf16_batch_is_rounded_fp32_sample():
    x = gi.make_inputs(5, [3, 70, 1], h_k=2, h_v=4, dk=16, dv=16, io="bf16")
    y = gi.make_inputs(5, [3, 70, 1], h_k=2, h_v=4, dk=16, dv=16, io="f32")
    assert x.q.dtype == torch.bfloat16 and x.total_tokens == 74
    assert torch.equal(x.q, y.q.to(torch.bfloat16)) and torch.equal(x.v, y.v.to(torch.bfloat16))
    assert torch.equal(x.a, y.a)
    assert np.allclose(np.linalg.norm(x.widen("k"), axis=-1), 1.0, atol=2 ** -7)


def test_select_and_concat():
    x = gi.make_inputs(5, [3, 70, 1], h_k=2, h_v=4, dk=16, dv=16, io="bf16")
    y = gi.GdnInputs.concat([x.select([2]), x.select([0, 1])])
    assert list(y.lengths) == [1, 3, 70]
    assert torch.equal(y.v[0], x.v[73]) and torch.equal(y.v[1:], x.v[:73])
    z = x.token_slice(3, 73)
    assert torch.equal(z.q, x.q[3:73]) and list(z.cu_seqlens) == [0, 70]


def test_trainer_lengths():
    L = gi.trainer_lengths()
    assert sum(L) == 10240 and all(64 <= l <= 4096 for l in L)


def test_decode_prompt_lengths():
    L = gi.decode_prompt_lengths()
    assert len(L) == 256 and L.min() >= 1 and L.max() <= 2048


@pytest.mark.parametrize("batch", [1, 2, 5])
def test_long_in_batch_keeps_x(batch):
    x = gi.make_inputs(4, [300], h_k=1, h_v=2, dk=16, dv=16, io="bf16")
    y, pos = gi.long_in_batch(x, batch, sub=batch, max_len=50)
    assert y.num_seqs == batch
    t0 = int(y.cu_seqlens[pos])
    assert y.lengths[pos] == 300
    assert torch.equal(y.q[t0:t0 + 300], x.q) and torch.equal(y.a[t0:t0 + 300], x.a)
