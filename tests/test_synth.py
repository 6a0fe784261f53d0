"""The seeded input generators: reproducible, and bf16 rounding is RNE."""

import numpy as np
import torch

import synth


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100_000).astype(np.float32),
                        np.array([1.0 + 2**-8, 1.0 + 3 * 2**-8, -1.0 - 2**-8, 0.0, -0.0], np.float32)])
    ours = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = synth.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_generators_are_reproducible_and_independent():
    a = synth.decode_batch(n_seqs=4, len_lo=5, len_hi=40, num_pages=64, page_size=4)
    b = synth.decode_batch(n_seqs=4, len_lo=5, len_hi=40, num_pages=64, page_size=4)
    assert np.array_equal(a.k, b.k) and np.array_equal(a.free_order, b.free_order)
    c = synth.decode_batch(n_seqs=4, len_lo=5, len_hi=40, num_pages=64, page_size=4, instance=1)
    assert not np.array_equal(a.q, c.q)
    assert sorted(a.free_order.tolist()) == list(range(64))


def test_workload_shapes():
    t = synth.tiny_batch()
    assert t.lengths.tolist() == [7, 6] and t.k.shape == (13, 1, 64) and t.q.shape == (13, 2, 64)
    p = synth.prefix_traces(n_rows=10, n_traces=4, trace_len=2000, len_hi=2000)
    assert p.row_len[:3].tolist() == [1000, 1400, 1900] and (p.row_trace[:3] == 0).all()
    assert (p.row_trace[3:] >= 1).all() and (p.row_trace[3:] <= 3).all()
    r = synth.rewind_docs(n_docs=3, num_pages=64)
    assert r.doc_k.shape == (3, 300, 8, 128) and r.q2_q.shape == (3, 50, 32, 128)
    s = synth.spec_decode(n_seqs=2, len_lo=100, len_hi=200, steps=3)
    assert s.keep.shape == (3, 2) and s.keep.min() >= 0 and s.keep.max() <= 5
