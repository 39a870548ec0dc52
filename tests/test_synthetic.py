"""The seeded input generators: determinism and the seed-0 routing statistics."""
import hashlib

import numpy as np
import pytest

import synthetic

# seed-0 statistics of `sizes`: (zero-row experts, max rows, min non-zero, experts with 1..8 rows)
SEED0 = {
    "tiny": (0, 20, 10, 0),
    "olmoe_gate_up_t1": (56, 1, 1, 8),
    "olmoe_gate_up_t2048": (0, 287, 215, 0),
    "qwen3_gate_up_t1": (120, 1, 1, 8),
    "qwen3_gate_up_t64": (79, 63, 1, 33),
    "qwen3_gate_up_t4096": (4, 3973, 1, 45),
    "gptoss_gate_up_t1": (28, 1, 1, 4),
    "gptoss_gate_up_t2048": (0, 299, 224, 0),
    "mixtral_w13_t4096": (0, 1039, 999, 0),
}
FIRST8 = {
    "tiny": [20, 19, 10, 19, 16, 15, 12, 17],
    "qwen3_gate_up_t4096": [6, 248, 75, 2, 2, 146, 2, 12],
    "mixtral_w13_t4096": [1022, 1029, 999, 1037, 1028, 1039, 1004, 1034],
}


@pytest.mark.parametrize("name", sorted(SEED0))
def test_seed0_routing_statistics(name):
    c = synthetic.case(name)
    sizes, token = synthetic.routing(c, 0)
    nz = sizes[sizes > 0]
    got = ((sizes == 0).sum(), sizes.max(), nz.min(), ((sizes >= 1) & (sizes <= 8)).sum())
    assert tuple(int(v) for v in got) == SEED0[name]
    assert sizes.sum() == c.M and len(token) == c.M
    if name in FIRST8:
        assert sizes[:8].tolist() == FIRST8[name]


def test_rows_grouped_by_expert_in_token_order():
    c = synthetic.case("tiny")
    sizes, token = synthetic.routing(c, 0)
    ids = synthetic.topk_ids(c, 0)
    off = np.concatenate([[0], np.cumsum(sizes)])
    for e in range(c.E):
        toks = token[off[e]:off[e + 1]]
        assert np.all(np.diff(toks) > 0)                 # top-k ids are distinct per token
        assert all(e in ids[t] for t in toks)


def test_generators_are_deterministic():
    c = synthetic.case("tiny")
    h = lambda x: hashlib.sha256(np.ascontiguousarray(x).tobytes()).hexdigest()
    assert h(synthetic.rows_bf16(c, 3)[0]) == h(synthetic.rows_bf16(c, 3)[0])
    assert h(synthetic.nf4_weight_f32(c, 3, 5)) == h(synthetic.nf4_weight_f32(c, 3, 5))
    assert h(synthetic.nf4_weight_f32(c, 3, 5)) != h(synthetic.nf4_weight_f32(c, 3, 6))
    g = synthetic.case("gptoss_down_t1")
    codes, scales = synthetic.mxfp4_bytes(g, 0, 1)
    assert codes.shape == (2880, 1440) and scales.shape == (2880, 90)
    assert scales.min() == 119 and scales.max() == 129
    nib = np.concatenate([codes & 15, codes >> 4]).ravel()
    counts = np.bincount(nib, minlength=16)
    assert counts.min() > 0.98 * counts.mean()           # uniform over all 16 nibbles


def test_first_rows_draw_is_a_prefix_of_the_whole_expert():
    c = synthetic.case("qwen3_down_t1")
    whole = synthetic.nf4_weight_f32(c, 0, 5)
    for n in (1, 7, 300):
        assert np.array_equal(synthetic.nf4_weight_f32(c, 0, 5, first_rows=n), whole[:n])
