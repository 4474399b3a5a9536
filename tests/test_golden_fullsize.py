"""The stored full-size outputs (tests/golden/fullsize_*.npz, written by
tests/golden/make_fullsize.py with the oracle) belong to the current workloads
(fingerprint) and equal the oracle recomputed here on one (agent, q head) of
each file, up to their float32 storage."""
import numpy as np
import pytest

from oracle import attention
from tests.golden import make_fullsize as golden
from workload import spec


@pytest.mark.parametrize("name,agent,head,layer", [("inms", 5, 17, 0), ("tokendance", 37, 22, 0), ("q4", 9, 30, 0),
                                                   ("scale", 139, 33, 47)])
def test_stored_outputs_are_the_oracle(name, agent, head, layer):
    wl = spec.make(name)
    out, agents, layers = golden.load(name, wl)
    sel_agents, sel_layers = golden.selection(name)
    assert agents == sel_agents and layers == sel_layers
    assert out.shape == (len(layers), len(agents), wl.shape.n_q_heads, wl.shape.head_dim)
    assert np.isfinite(out).all() and (np.abs(out).max(axis=(2, 3)) > 0).all()
    ref = attention.decode(wl, layer, agents=[agent], heads=[head])[0, head]
    got = out[layers.index(layer), agents.index(agent), head]
    # float32 storage: round to nearest, 2^-24 relative
    assert np.all(np.abs(got - ref) <= 2.0 ** -24 * np.abs(ref) + 1e-30)


def test_scale_selection_spans_every_consumer_group():
    """Both ends of the round, and at least three agents of each of the ten
    groups of 25 consecutive agents whose shared-segment rows are split into
    separate work items (5 q heads per kv head: 125 rows per group)."""
    agents, layers = golden.selection("scale")
    assert len(agents) >= 32 and 0 in agents and 249 in agents and layers == [0, 47]
    for k in range(10):
        assert sum(25 * k <= j < 25 * (k + 1) for j in agents) >= 3
