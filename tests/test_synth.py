"""The seeded input generators: every seed field changes the stream, and the
same seed gives the same bits (CPU)."""
import pytest
import torch

import moe_synth as S


def test_each_seed_field_changes_the_draw():
    base = S.draw(18, S.T_X, 0, (64,), 1.0, torch.float32)
    assert torch.equal(base, S.draw(18, S.T_X, 0, (64,), 1.0, torch.float32))
    for other in [S.draw(19, S.T_X, 0, (64,), 1.0, torch.float32),      # seed_base
                  S.draw(18 + 101, S.T_X, 0, (64,), 1.0, torch.float32),
                  S.draw(18, S.T_DY, 0, (64,), 1.0, torch.float32),    # tensor id
                  S.draw(18, S.T_X, 1, (64,), 1.0, torch.float32)]:    # expert id
        assert not torch.equal(base, other)


def test_configs_draw_distinct_inputs():
    xs = [S.x(S.mini(c, T=8, d=128, f=128)) for c in S.CONFIGS]
    for i in range(len(xs)):
        for j in range(i + 1, len(xs)):
            assert not torch.equal(xs[i].float(), xs[j].float()), (i, j)


def test_seed_fields_are_range_checked():
    with pytest.raises(ValueError):
        S.draw(1 << 16, S.T_X, 0, (4,), 1.0, torch.float32)
    with pytest.raises(ValueError):
        S.draw(1, S.T_X, 1 << 11, (4,), 1.0, torch.float32)
