"""The seeded input generator: determinism, shapes, structure and bf16 rounding."""
import numpy as np
import torch

from gen import WORKLOADS, bf16_round, bf16_to_f32, make_inputs, workload
from gen.inputs import latent_field


def test_determinism_and_head_subsets():
    a = make_inputs(1)
    b = make_inputs(1)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.v, b.v)
    c = make_inputs(1, heads=[1])
    assert np.array_equal(c.k[:, 0], a.k[:, 1])


def test_shapes_match_workloads():
    for cid, w in WORKLOADS.items():
        assert w.N == w.T * w.Hh * w.Ww
        assert w.N % w.block_q == 0 and w.N % w.block_k == 0
    assert WORKLOADS[4].N == 65536 and WORKLOADS[5].N == 202752
    assert WORKLOADS[5].T == 22 and (WORKLOADS[5].T - 5) % 17 == 0   # a 17n+5 frame count


def test_latent_is_standardised_and_smooth():
    w = workload(1)
    z = latent_field(w)
    assert np.allclose(z.mean(0), 0, atol=1e-4) and np.allclose(z.std(0), 1, atol=1e-3)
    # neighbouring tokens along x are strongly correlated after the blur
    zz = z.reshape(w.T, w.Hh, w.Ww, w.d)
    r = np.mean(zz[:, :, 1:] * zz[:, :, :-1])
    assert r > 0.8


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 10
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0]      # exact ties
    ours = bf16_round(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(bf16_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_bf16_workload_values_are_exact_bits():
    w = workload(2, H=1, T=1)
    x = make_inputs(w)
    assert np.array_equal(bf16_to_f32(x.q_bits), x.q)
