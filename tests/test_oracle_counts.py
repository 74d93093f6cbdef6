"""The counts the pages print, checked against the site structure the oracle assumes.

Fixture: golden/paper_counts.json (each entry cites its page and section).
LLaMA-3 8B: hidden size 4096, 32 layers, head size 128; r = 32.
"""
import json
import os

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "paper_counts.json")
D, LAYERS, HEAD, R = 4096, 32, 128, 32


def _printed_millions(s):
    return float(s.rstrip("M"))


def _load():
    with open(GOLDEN) as f:
        return json.load(f)


def test_online_parameters_are_one_basis_per_junction_two_junctions_per_layer():
    # Two correction sites per layer (the MHSA and FFN blocks each get rotations,
    # zh §2.2), each holding one D x r basis: 64 * D * r.
    printed = _printed_millions(_load()["online_parameters"]["printed"])
    sites = 2 * LAYERS
    assert round(sites * D * R / 1e6, 1) == printed
    # one site per layer, or a D x D matrix per site, would not print as 8.4M
    assert round(LAYERS * D * R / 1e6, 1) != printed
    assert round(sites * D * D / 1e6, 1) != printed
    # and it is about 0.1% of an 8B model
    assert abs(sites * D * R / 8.0e9 - 0.001) < 0.0005


def test_training_parameters_count_full_rotations():
    g = _load()
    full = _printed_millions(g["training_parameters"]["printed"])
    glob = _printed_millions(g["global_rotation_training_parameters"]["printed"])
    per_head = LAYERS * HEAD * HEAD
    # 65 full D x D rotations (two per layer plus one) and one head rotation per layer
    assert round((65 * D * D + per_head) / 1e6, 1) == full
    # a single global D x D rotation plus the same head rotations
    assert round((D * D + per_head) / 1e6, 1) == glob
    assert round(full / glob) == int(g["global_rotation_training_parameters"]["ratio_printed"])


def test_full_rank_of_ablation_is_the_hidden_size():
    g = _load()["rank_ablation"]
    assert g["r"][1] == D
    assert g["ppl"][1] < g["ppl"][0]  # more rank, lower perplexity
