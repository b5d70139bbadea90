"""Host logic of bench.py: the one-GPU refusal, and the byte accounting its roofline figure divides by the kernel
time, checked against the records the oracle packs and against the lengths the oracle's cache reaches."""
import numpy as np
import pytest

import bench
from oracle import cache as oc
from tests import helpers


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def _filled(bits=2, sparse=False, sink=False, tokens=160):
    rng = np.random.default_rng(5)
    k = rng.standard_normal((1, tokens, 128)).astype(np.float16)
    v = rng.standard_normal((1, tokens, 128)).astype(np.float16)
    c = oc.SliceCache(1, bits=bits, sparse=sparse, sink=sink)
    c.append(k, v)
    return c


@pytest.mark.parametrize("bits,sparse", [(2, False), (2, True), (4, False), (4, True)])
def test_quantized_bytes_per_token_are_the_packed_record_size(bits, sparse):
    """Per quantized token and KV head the call reads one 32-token tile record: the oracle's packed record bytes
    over 32 (2-bit 3072 B, 4-bit 5120 B; with the outlier section 3840 B and 5888 B)."""
    c = _filled(bits, sparse)
    rec = helpers.oracle_records(c) if bits == 2 else helpers.oracle_records4(c)
    assert rec.shape[:2] == (1, c.n_quant // 32)
    per_token = rec.shape[-1] / 32
    got = bench.algorithmic_bytes(1, 1, 1, c.n_quant, 0, bits=bits, sparse=sparse)
    # query (fp16) read and output (fp32) written once per query head
    assert got == c.n_quant * per_token + 128 * 2 + 128 * 4


def test_window_bytes_are_its_fp16_rows():
    c = _filled()
    got = bench.algorithmic_bytes(1, 1, 1, 0, c.n_resid)
    assert got == c.k_res.nbytes + c.v_res.nbytes + 128 * 6


def test_kv_slices_count_once_however_many_query_heads_read_them():
    a = bench.algorithmic_bytes(2, 8, 8, 1024, 64)
    b = bench.algorithmic_bytes(2, 8, 32, 1024, 64)
    assert b - a == 2 * (32 - 8) * 128 * 6


def test_the_32k_workload_figure():
    """B64, 32 query / 8 KV heads, 32640 quantized + 128 window tokens: the per-call figure stated for the
    dominant kernel."""
    assert bench.algorithmic_bytes(64, 8, 32, 32640, 128) == 1_639_448_576


@pytest.mark.parametrize("n_quant,n_resid,appended", [(0, 0, 1), (0, 0, 300), (3968, 128, 1), (3968, 128, 129),
                                                       (4096, 5, 123), (4096, 5, 124)])
def test_lengths_after_appends_follow_the_oracle_cache(n_quant, n_resid, appended):
    """The bench's length bookkeeping (used to count the bytes of each timed call) equals the oracle's closed form
    for the lazy flush."""
    want_q = n_quant + oc.flushed_tokens(n_resid, appended, 128)
    assert bench.lengths_after(n_quant, n_resid, appended, 128) == (want_q, n_resid + appended - (want_q - n_quant))
