"""The workload table and optimiser defaults agree with the values the NNTile
README prints for its GPT2 example (tests/golden/readme_gpt2_example.txt)."""
import os

import synth

HERE = os.path.dirname(os.path.abspath(__file__))


def _golden():
    out = {}
    with open(os.path.join(HERE, "golden", "readme_gpt2_example.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, v = line.split()
                out[k] = v
    return out


def test_gpt2_small_tiles_and_hparams_match_readme():
    g = _golden()
    w = synth.WORKLOADS["gpt2_small"]
    assert w.tiles.batch == int(g["minibatch-tile"])
    assert w.tiles.seq == int(g["seq-tile"])
    assert w.tiles.embd == int(g["embd-tile"])
    assert w.tiles.inner == int(g["inner-tile"])
    assert w.tiles.head == int(g["head-tile"])
    assert w.eps == float(g["optimizer-eps"])
    assert w.weight_decay == float(g["weight-decay"])
    assert w.lr == float(g["lr"])
    assert g["loss-reduction"] == "mean" and g["optimizer"] == "fusedadamw"
    # divisibility rules of the README flags: seq, head and batch tiles divide their axis
    for w in synth.WORKLOADS.values():
        s, t = w.shape, w.tiles
        assert s.seq % t.seq == 0 and s.n_head % t.head == 0 and s.batch % t.batch == 0
