"""The seeded input generator: determinism, addressability, distributions."""
import torch

import synthetic as syn


def test_rows_match_full_tensor():
    full = syn.make((3, 50, 8), 5, syn.TID["k"], dtype=torch.bfloat16, scale=0.125)
    rows = syn.rows((3, 50, 8), [0, 7, 149, 60], 5, syn.TID["k"], dtype=torch.bfloat16,
                    scale=0.125)
    flat = full.view(-1, 8)
    assert torch.equal(rows, flat[[0, 7, 149, 60]])


def test_repeatable_and_seed_dependent():
    a = syn.make((1000,), 1, 3)
    assert torch.equal(a, syn.make((1000,), 1, 3))
    assert not torch.equal(a, syn.make((1000,), 2, 3))
    assert not torch.equal(a, syn.make((1000,), 1, 4))
    assert not torch.equal(a, syn.make((1000,), 1, 3, layer=1))


def test_normal_moments_and_chunking():
    a = syn.make((1 << 20,), 7, 1)
    assert abs(a.mean().item()) < 0.01 and abs(a.std().item() - 1) < 0.01
    b = torch.empty(1 << 20)
    syn.fill_(b, 7, 1, chunk=12345)
    assert torch.equal(a, b)


def test_grid_and_uniform_are_exact():
    g = syn.make((4096,), 3, 2, kind="grid", grid=8, scale=2.0 ** -4)
    assert torch.equal(g * 16, torch.round(g * 16)) and g.abs().max() <= 0.5
    u = syn.make((4096,), 3, 2, kind="uniform")
    assert u.min() >= 0 and u.max() < 1


def test_sample_indices_sorted_unique_padded():
    idx = syn.sample_indices(1, 22, 4, 8, torch.tensor([100, 5, 8, 0]))
    for r, nv in enumerate([100, 5, 8, 0]):
        v = idx[r][idx[r] >= 0]
        assert v.numel() == min(8, nv)
        assert torch.equal(v, torch.sort(torch.unique(v)).values)
        assert (v < max(nv, 1)).all()
