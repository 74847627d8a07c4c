"""Writes the oracle outputs of the tuner's reference terms.

Terms (the order of q8k4v_tune_request.ref): decode and verify at 4096 and
65536 cached tokens, 32 query / 8 kv heads, D 128, 8 drafts, on the seeded
inputs of ``workloads.tune_reference`` (seed 11 at 4096, 12 at 65536).  The
decode term attends the first ``context`` tokens with draft 0's query; the
verify term attends all ``context + 8`` tokens with every draft.  Then the
two multi-session terms, 32 query / 4 kv heads, D 128: 16 sessions over a
``context / 2`` shared prefix with ragged private suffixes, on the inputs of
``workloads.tune_sessions_reference`` (seed 13 at 4096, 14 at 65536).  Every
value comes from ``oracle/`` (the fp32 quantizer, then fp64 softmax
attention); ``bench.py --tune`` hands them to tune_select as its oracle gate.

    python tests/golden/make_tune_refs.py   # writes tune_refs_32q8kv_d128_w8.npz
                                            # and tune_refs_32q4kv_d128_s16.npz
"""

import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402
from oracle import attention, codec  # noqa: E402

OUT = os.path.join(HERE, "tune_refs_32q8kv_d128_w8.npz")
SESSIONS_OUT = os.path.join(HERE, "tune_refs_32q4kv_d128_s16.npz")
CONTEXTS = {"small": (4096, 11), "large": (65536, 12)}
SESSION_CONTEXTS = {"small": (4096, 13), "large": (65536, 14)}
N_DRAFT = 8
N_SESSIONS = 16


def reference_terms(size: str):
    """(decode [Hq][D], verify [W][Hq][D], sigma [Hq][D]) from the oracle."""
    ctx, seed = CONTEXTS[size]
    w = workloads.tune_reference(ctx, N_DRAFT, seed)
    cache = codec.PagedCache(w.num_pages, w.num_kv_heads, w.head_dim)
    for a in w.appends:
        codec.append(cache, a.k, a.v, w.dtype, a.cu_new, a.start_pos, a.page_table)
    ver = attention.verify(cache, w.q, w.dtype, w.page_table, w.seq_lens, w.softmax_scale)[0]
    dec = attention.decode(cache, np.ascontiguousarray(w.q[:, 0]), w.dtype, w.page_table,
                           np.array([ctx], np.int32), w.softmax_scale)[0]
    sigma = np.repeat(w.sigma_v.astype(np.float64), w.num_q_heads // w.num_kv_heads, axis=0)
    return dec, ver, sigma


def session_terms(size: str):
    """(output [sessions][Hq][D], sigma [Hq][D]) of the multi-session term."""
    ctx, seed = SESSION_CONTEXTS[size]
    w = workloads.tune_sessions_reference(ctx, N_SESSIONS, seed)
    cache = codec.PagedCache(w.num_pages, w.num_kv_heads, w.head_dim)
    for a in w.appends:
        codec.append(cache, a.k, a.v, w.dtype, a.cu_new, a.start_pos, a.page_table)
    out = attention.decode(cache, w.q, w.dtype, w.page_table, w.seq_lens, w.softmax_scale)
    sigma = np.repeat(w.sigma_v.astype(np.float64), w.num_q_heads // w.num_kv_heads, axis=0)
    return out, sigma


def main():
    arrays = {}
    for size in CONTEXTS:
        dec, ver, sigma = reference_terms(size)
        arrays[f"decode_{size}"] = dec.astype(np.float32)
        arrays[f"verify_{size}"] = ver.astype(np.float32)
        arrays[f"sigma_{size}"] = sigma.astype(np.float32)
    np.savez_compressed(OUT, **arrays)
    print(f"wrote {OUT}")
    arrays = {}
    for size in SESSION_CONTEXTS:
        out, sigma = session_terms(size)
        arrays[f"multi_session_{size}"] = out.astype(np.float32)
        arrays[f"sigma_{size}"] = sigma.astype(np.float32)
    np.savez_compressed(SESSIONS_OUT, **arrays)
    print(f"wrote {SESSIONS_OUT}")


if __name__ == "__main__":
    main()
