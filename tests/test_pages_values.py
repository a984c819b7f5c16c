"""The workload definitions use the numbers the pages print."""
import json
import os

from kv_cache_compression_encode_amd import synth

P = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_values.json")))


def test_step_presets():
    for name in ("high", "balanced", "fast"):
        assert list(synth.PRESET_STEPS[name]) == P["step_presets"][name]


def test_layerwise_steps_grow_with_depth():
    for cfg in synth.CONFIGS.values():
        for lv in cfg.levels:
            steps = [lv.steps[g] for g in lv.layer_group]
            assert steps == sorted(steps)
    bal = synth.PRESET_STEPS["balanced"]
    assert bal[0] == P["layer_steps_example"]["shallow"] and bal[-1] == P["layer_steps_example"]["deep"]


def test_chunking_and_levels():
    for name in ("7b", "34b", "long", "stream"):
        assert synth.CONFIGS[name].chunk_tokens == P["chunk_tokens"]["value"]
    assert len(synth.CONFIGS["long"].levels) == P["levels_per_chunk"]["count"]
