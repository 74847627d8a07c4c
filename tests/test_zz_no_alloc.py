"""GPU test of attn_decode_q8k4v_noalloc, the decode entry point that
allocates nothing (its split records and merge counters live in the
library's static per-GPU array).  Through the C ABI, two calls in a row --
the second on a smaller input -- must give exactly what attn_decode_q8k4v
gives with a caller workspace (same plan, same kernels), and both must be
within the oracle's tolerance; the in-launch merge (whose counters live in
the static array's header) and the separate combine are both covered, and a
launch too large for the array is refused."""

import ctypes as C

import numpy as np
import pytest

import workloads
from tests.util import ATOL_SIGMA, normalized_err, oracle_out

pytestmark = pytest.mark.gpu


def _noalloc(lib, cache, q, lens, msl, pt, scale, out, cfg):
    import torch
    import decode_attention_quantized_kv_amd as q8
    B, Hq, _ = q.shape
    rc = lib.attn_decode_q8k4v_noalloc(C.byref(cache.desc), q.data_ptr(), q8.BF16 if q.dtype == torch.bfloat16 else q8.F32,
                                       out.data_ptr(), B, Hq, lens.data_ptr(), msl, pt.data_ptr(), pt.shape[1],
                                       C.c_float(scale), C.byref(cfg) if cfg is not None else None,
                                       torch.cuda.current_stream().cuda_stream)
    return rc


@pytest.mark.parametrize("cfg", [None, dict(fused_combine=1), dict(fused_combine=1, variant=5)], ids=str)
def test_noalloc_matches_workspace_entry_point(cfg):
    import torch
    import decode_attention_quantized_kv_amd as q8
    from tests.gpu_util import to_dev, upload_cache
    lib = q8.load_library()
    c = None if cfg is None else q8.make_config(**cfg)
    big = workloads.build("noalloc_big", seed=501, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16",
                          seq_lens=[9000, 3000], outliers=True)
    small = workloads.build("noalloc_small", seed=502, num_q_heads=32, num_kv_heads=8, head_dim=128, dtype="bf16",
                            seq_lens=[700], outliers=True)
    for w in (big, small):                      # two calls in a row, the second smaller
        cache = upload_cache(w)
        q, lens, pt = to_dev(w.q, "bf16"), to_dev(w.seq_lens), to_dev(w.page_table)
        msl = int(w.seq_lens.max())
        out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
        rc = _noalloc(lib, cache, q, lens, msl, pt, w.softmax_scale, out, c)
        assert rc == 0, lib.q8k4v_last_error()
        ref = q8.attn_decode_q8k4v(cache, q, lens, msl, pt, w.softmax_scale, cfg=c)
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        assert np.array_equal(got, ref.cpu().numpy().astype(np.float64)), w.name
        err = normalized_err(w, got, oracle_out(w))
        print(f"[noalloc] {w.name} cfg {cfg}: bit-identical to attn_decode_q8k4v, max |err|/sigma = {err:.3e}",
              flush=True)
        assert err <= ATOL_SIGMA, (w.name, err)


def test_noalloc_refuses_a_launch_beyond_the_static_array():
    import torch
    import decode_attention_quantized_kv_amd as q8
    lib = q8.load_library()
    # 64 sequences x 8 kv heads x 8 rows x 64 splits of 528-byte records: more
    # than 16 MiB; refused on the host before any launch
    d = q8.CacheDesc(65536, 8, 128, 16, 1, 1, 1, 1)
    cfg = q8.make_config(split_pages=8)
    rc = lib.attn_decode_q8k4v_noalloc(C.byref(d), 1, q8.BF16, 1, 64, 64, 1, 8192, 1, 512, C.c_float(0.1),
                                       C.byref(cfg), None)
    assert rc == -3 and b"static" in lib.q8k4v_last_error()
