"""The seeded input generators: determinism, the stated structure, and the
bf16 rounding of inputs (checked against torch's own conversion)."""

import hashlib

import numpy as np
import torch

import workloads


def _digest(w):
    h = hashlib.sha256()
    for a in [w.q, w.page_table, w.seq_lens] + [x for b in w.appends for x in (b.k, b.v, b.cu_new, b.start_pos)]:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def test_deterministic_per_seed():
    a = workloads.gqa_decode(512, seed=1)
    b = workloads.gqa_decode(512, seed=1)
    c = workloads.gqa_decode(512, seed=2)
    assert _digest(a) == _digest(b) != _digest(c)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * 10.0 ** rng.uniform(-5, 5, 100000)).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(workloads.f32_to_bf16_bits(x), want)


def test_structure_of_named_workloads():
    w = workloads.gqa_decode_4k()
    assert (w.num_q_heads, w.num_kv_heads, w.head_dim, w.dtype) == (32, 8, 128, "bf16")
    assert w.seq_lens.tolist() == [4096] and w.n_draft == 0
    assert int(np.sum(w.sigma_v == 8)) == 10 and int(np.sum(w.sigma_k == 8)) == 10
    assert sorted(w.page_table[0].tolist()) == list(range(256))
    assert w.page_table[0].tolist() != list(range(256))
    t = workloads.tiny_decode()
    assert (t.num_q_heads, t.num_kv_heads, t.head_dim, t.dtype, t.seq_lens.tolist()) == (2, 1, 64, "f32", [256])


def test_multi_session_shares_prefix_pages():
    w = workloads.multi_session(sessions=5, prefix=64, max_suffix=50)
    pre = 4
    assert all(np.array_equal(w.page_table[0, :pre], w.page_table[s, :pre]) for s in range(5))
    used = [w.page_table[s, pre:(int(w.seq_lens[s]) + 15) // 16] for s in range(5)]
    flat = np.concatenate(used + [w.page_table[0, :pre]])
    assert len(set(flat.tolist())) == len(flat)          # suffix pages private
    assert w.unique_tokens() == 64 + int(np.sum(w.seq_lens - 64))


def test_verify_appends_drafts_last():
    w = workloads.build("v", seed=1, num_q_heads=4, num_kv_heads=1, head_dim=64, dtype="bf16",
                        seq_lens=[40, 20], n_draft=3)
    last = w.appends[-1]
    assert last.start_pos.tolist() == [37, 17] and last.cu_new.tolist() == [0, 3, 6]
    assert w.q.shape == (2, 3, 4, 64)
