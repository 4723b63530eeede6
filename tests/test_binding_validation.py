"""The Python binding checks every layer's tensors, the caller's outputs and the index
cache before anything reaches the library: a later F layer in the wrong dtype, a short
k_I, a wrong-shaped output or index cache is a ValueError / TypeError, never a launch
that reads or writes out of bounds.  Shapes are checked before the device, so these run
on CPU tensors; a call whose shapes are all right then stops at the device check."""
import pytest
import torch

import dsa_lightning_indexer_scores_amd as ic

B, L, H_I, d_I, H, d, K = 1, 64, 4, 32, 4, 64, 16


def _layer(full=True, dtype=torch.bfloat16, L_=L, Lk=L, H_I_=H_I):
    lay = {"q": torch.zeros((B, L_, H, d), dtype=torch.bfloat16), "kv": torch.zeros((B, Lk, 2, d), dtype=torch.bfloat16)}
    if full:
        lay["q_I"] = torch.zeros((B, L_, H_I_, d_I), dtype=dtype)
        lay["w"] = torch.zeros((B, L_, H_I_), dtype=torch.float32)
        lay["k_I"] = torch.zeros((B, Lk, d_I), dtype=dtype)
    return lay


def _stack():
    return [_layer(True), _layer(False), _layer(True), _layer(False)]


def test_consistent_cpu_stack_reaches_the_device_check():
    with pytest.raises(ValueError, match="GPU tensor"):
        ic.run_stack("FSFS", _stack(), K)


def test_later_f_layer_dtype_is_checked():
    layers = _stack()
    layers[2]["q_I"] = layers[2]["q_I"].to(torch.uint8)
    layers[2]["k_I"] = layers[2]["k_I"].to(torch.uint8)
    with pytest.raises(TypeError, match=r"layers\[2\]\.q_I"):
        ic.run_stack("FSFS", layers, K)


def test_later_f_layer_short_k_I_is_checked():
    layers = _stack()
    layers[2]["k_I"] = torch.zeros((B, L // 2, d_I), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match=r"layers\[2\]\.k_I"):
        ic.run_stack("FSFS", layers, K)


def test_later_f_layer_head_count_is_checked():
    layers = _stack()
    layers[2] = _layer(True, H_I_=H_I + 1)
    with pytest.raises(ValueError, match=r"layers\[2\]\.q_I"):
        ic.run_stack("FSFS", layers, K)


def test_f_layer_without_indexer_inputs():
    layers = _stack()
    del layers[2]["w"]
    with pytest.raises(ValueError, match="F layer 2"):
        ic.run_stack("FSFS", layers, K)


def test_layer_q_and_kv_shapes_are_checked():
    layers = _stack()
    layers[3]["kv"] = torch.zeros((B, L - 1, 2, d), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match=r"layers\[3\]\.kv"):
        ic.run_stack("FSFS", layers, K)
    layers = _stack()
    layers[1]["q"] = torch.zeros((B, L, H, d), dtype=torch.float16)
    with pytest.raises(TypeError, match=r"layers\[1\]\.q"):
        ic.run_stack("FSFS", layers, K)


def test_pattern_length_is_checked():
    with pytest.raises(ValueError, match="pattern length"):
        ic.run_stack("FSF", _stack(), K)


@pytest.mark.parametrize("bad", ["short_k", "wrong_dtype", "wrong_rows"])
def test_idx_cache_is_checked(bad):
    idx = {"short_k": torch.zeros((B, L, K - 1), dtype=torch.int32),
           "wrong_dtype": torch.zeros((B, L, K), dtype=torch.int64),
           "wrong_rows": torch.zeros((B, L - 1, K), dtype=torch.int32)}[bad]
    with pytest.raises((ValueError, TypeError), match="idx_cache"):
        ic.run_stack("FSFS", _stack(), K, idx_cache=idx)


def test_outs_are_checked():
    outs = [torch.zeros((B, L, H, d), dtype=torch.bfloat16) for _ in range(4)]
    outs[2] = torch.zeros((B, L, H, d // 2), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match=r"outs\[2\]"):
        ic.run_stack("FSFS", _stack(), K, outs=outs)
    with pytest.raises(ValueError, match="outs must list"):
        ic.run_stack("FSFS", _stack(), K, outs=outs[:3])
    outs[2] = torch.zeros((B, L, H, d), dtype=torch.bfloat16).transpose(2, 3).contiguous().transpose(2, 3)
    with pytest.raises(ValueError, match="contiguous"):
        ic.run_stack("FSFS", _stack(), K, outs=outs)


def test_dynamic_s_layer_indexer_inputs_are_checked():
    layers = [_layer(True), _layer(True), _layer(False), _layer(True)]
    layers[3]["w"] = torch.zeros((B, L, H_I + 2), dtype=torch.float32)
    with pytest.raises(ValueError, match=r"layers\[3\]\.w"):
        ic.run_stack_dynamic("FSSS", layers, K, probe_stride=4, tau=0.5)
    layers = [_layer(True), _layer(True), _layer(False), _layer(True)]
    del layers[1]["k_I"]
    with pytest.raises(ValueError, match="all present or all absent"):
        ic.run_stack_dynamic("FSSS", layers, K, probe_stride=4, tau=0.5)


def test_decode_idx_cache_and_seq_len_are_checked():
    layers = [_layer(True, L_=1, Lk=100), _layer(False, L_=1, Lk=100)]
    sl = torch.full((B,), 50, dtype=torch.int32)
    with pytest.raises(ValueError, match="idx_cache"):
        ic.decode_step("FS", layers, sl, K, idx_cache=torch.zeros((B, 2, K), dtype=torch.int32))
    with pytest.raises(ValueError, match="seq_len"):
        ic.decode_step("FS", layers, torch.full((B + 1,), 50, dtype=torch.int32), K)
    with pytest.raises(TypeError, match="seq_len"):
        ic.decode_step("FS", layers, sl.long(), K)
    with pytest.raises(ValueError, match="GPU tensor"):
        ic.decode_step("FS", layers, sl, K)


def test_varlen_later_layers_are_checked():
    T = 40
    base = {"q": torch.zeros((T, H, d), dtype=torch.bfloat16), "kv": torch.zeros((2, L, 2, d), dtype=torch.bfloat16)}
    f = dict(base, q_I=torch.zeros((T, H_I, d_I), dtype=torch.bfloat16), w=torch.zeros((T, H_I)),
             k_I=torch.zeros((2, L, d_I), dtype=torch.bfloat16))
    bad = dict(f, k_I=torch.zeros((2, L - 8, d_I), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match=r"layers\[2\]\.k_I"):
        ic.run_stack_varlen("FSF", [f, dict(base), bad], K, [30, 10], [0, 5])
    with pytest.raises(ValueError, match="idx_cache"):
        ic.run_stack_varlen("FSF", [f, dict(base), f], K, [30, 10], [0, 5],
                            idx_cache=torch.zeros((T + 1, K), dtype=torch.int32))
    with pytest.raises(ValueError, match="GPU tensor"):
        ic.run_stack_varlen("FSF", [f, dict(base), f], K, [30, 10], [0, 5])


def test_pattern_rules_come_before_tensor_checks():
    layers = _stack()
    del layers[2]["w"]                                           # would fail a tensor check
    with pytest.raises(ic.NoCachedIndices):
        ic.run_stack("SFFS", layers, K)
    with pytest.raises(ic.ICError, match="not one of"):
        ic.run_stack("FSXS", _stack(), K)
    with pytest.raises(ic.NoCachedIndices):
        ic.decode_step("SF", [_layer(False, L_=1), _layer(True, L_=1)], torch.ones(B, dtype=torch.int32), K)
