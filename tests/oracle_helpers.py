"""Small test-only helpers around the oracle and the synthetic inputs."""
import numpy as np

import synth


def mini_model(**over):
    """A very small model dict in the S2 layout, for oracle pins."""
    m = dict(
        n_layer=2, dim=32, n_head=4, n_kv_head=2, head_dim=8, ffn_dim=48, vocab_size=300,
        n_fast_layer=2, fast_dim=32, fast_n_head=4, fast_n_kv_head=2, fast_head_dim=8,
        fast_ffn_dim=48, slow_qk_norm=1, fast_qk_norm=1, num_codebooks=4, codebook_size=16,
        semantic_begin_id=200, semantic_end_id=215, end_id=150, scale_codebook_embeddings=1,
        rope_base=1.0e6, norm_eps=1.0e-6, weight_dtype="f32", text_vocab=150, acoustic_size=16,
    )
    m.update(over)
    return m


def f32_weights(m, seed=0):
    return synth.weights_as_f32(m, synth.make_weights(m, seed=seed, threads=2))
