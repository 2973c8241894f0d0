"""The seeded input generator: reproducible bytes and the documented structure."""
import numpy as np

from synth import bf16_to_f32, make_step, make_weights, workload


def test_generator_is_deterministic_and_shaped():
    w = workload("rejection-b1", V=4096, d=256)
    W1, W2 = make_weights(w), make_weights(w)
    assert W1.dtype == np.uint16 and W1.shape == (4096, 256) and np.array_equal(W1, W2)
    s1, s2 = make_step(w, W1, 3), make_step(w, W1, 3)
    for f in ["draft_tokens", "hidden", "draft_logits", "u_accept", "u_resample"]:
        assert np.array_equal(getattr(s1, f), getattr(s2, f))
    assert s1.hidden.shape == (1, 17, 256) and s1.draft_logits.shape == (1, 16, 4096)
    assert not np.array_equal(make_step(w, W1, 4).hidden, s1.hidden)
    Wf = bf16_to_f32(W1)
    assert abs(Wf.std() * np.sqrt(256) - 1.0) < 0.02
    # The drafted token carries the +6 boost in the draft logits.
    dl = bf16_to_f32(s1.draft_logits[0])
    assert np.all(np.argmax(dl, axis=1) == s1.draft_tokens[0])


def test_confidences_decrease_and_truncate_near_expected_length():
    w = workload("ragged-b32", V=1024, d=64)
    W = make_weights(w)
    Ls = []
    for step in range(20):
        c = make_step(w, W, step).conf
        assert np.all(np.diff(c, axis=1) <= 0) and np.all(c[:, 0] >= 0.6)
        Ls += list(np.argmax(np.concatenate([c < 0.3, np.ones((w.B, 1), bool)], 1), axis=1))
    assert 5.5 < np.mean(Ls) < 7.5
