"""The benchmark configurations carry the model shapes the pages print."""
import json
import os

import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden", "page_shapes.json")


def test_pangu_shape_matches_pages():
    g = json.load(open(GOLD))
    p, grp = g["pangu_ultra_moe"], g["pangu_expert_groups"]
    c = synth.get_config("pangu")
    assert (c.H, c.I, c.E) == (p["hidden"], p["expert_hidden"], p["routed_experts"])
    assert c.shared == (p["shared_experts"] == 1)
    # one device holds one expert group of whole experts
    assert c.groups == p["routed_experts"] // grp["expert_groups"] == grp["experts_per_group"]


def test_deepseek_shape_matches_pages():
    g = json.load(open(GOLD))
    assert synth.get_config("deepseek").E == g["deepseek_v3"]["routed_experts"]


def test_tp_extend_ep_keeps_experts_whole():
    f = json.load(open(GOLD))["tp_extend_ep_figure"]
    # splitting the expert count over TP*EP ranks leaves whole experts per rank
    assert f["experts"] % (f["tp"] * f["ep"]) == 0


def test_generator_is_deterministic_and_bf16_exact():
    c = synth.get_config("tiny")
    a, b = synth.make_inputs(c), synth.make_inputs(c)
    assert (a.x == b.x).all() and (a.w13 == b.w13).all()
    s = synth.get_config("small", T=64, H=128, I=64, E=8, k=2)
    i = synth.make_inputs(s)
    for arr in (i.x, i.w13, i.w2, i.dy):
        assert (synth.bf16_round(arr) == arr).all()
