"""Pins of the oracle's tile-record packing and of its grouped + residual cache state machine.

Packing is a layout of this library (not of the pages): it is pinned by being a bijection of every code onto
256 words x 16 two-bit slots, by exact round trips, and exhaustively over every byte value.

State machine (KIVI page, paragraph on the recent-token window): the newest tokens, up to R = 128, stay in full
precision and are quantized in blocks when the window fills. Pinned by: a token-by-token simulation against the
closed form; prefill equal to token-by-token appends (bit for bit); the residual reproducing its input bytes; and
the lengths the workloads expect (1024 tokens -> 896 quantized + 128 residual; 4096 + 256 steps -> flushes at
steps 1 and 129, final 4224 + 128).
"""
import json
import os

import numpy as np
import pytest

from oracle import cache as oc
from oracle import layout, quant

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ packing
def test_code_placement_is_a_bijection():
    for pos in (layout.key_code_position, layout.value_code_position):
        seen = set()
        for t in range(32):
            for c in range(128):
                w, b = pos(t, c)
                assert 0 <= w < 256 and b % 2 == 0 and 0 <= b < 32
                seen.add((w, b))
        assert len(seen) == 32 * 128


def test_each_lane_reads_its_own_16_bytes():
    """Word w belongs to lane w // 4: the key codes a lane holds are the two tokens n and 16 + n of its row and
    the 32 channels of its column group; the value codes are the 8 channels n + 16 j and the 8 tokens of its
    column group."""
    for t in range(32):
        for c in range(128):
            w, _ = layout.key_code_position(t, c)
            lane = w // 4
            assert lane % 16 == t % 16 and lane // 16 == (c % 32) // 8
            w, _ = layout.value_code_position(t, c)
            lane = w // 4
            assert lane % 16 == c % 16
            assert lane // 16 == ((t % 16) // 4)


def test_pack_round_trip_random():
    rng = np.random.default_rng(1)
    n = 7
    parts = (rng.integers(0, 4, (n, 32, 128)).astype(np.uint8), rng.standard_normal((n, 128)).astype(np.float16),
             rng.standard_normal((n, 128)).astype(np.float16), rng.integers(0, 4, (n, 32, 128)).astype(np.uint8),
             rng.standard_normal((n, 32, 4)).astype(np.float16), rng.standard_normal((n, 32, 4)).astype(np.float16))
    rec = layout.pack_tiles(*parts)
    assert rec.shape == (n, 3072)
    for a, b in zip(layout.unpack_tiles(rec), parts):
        assert np.array_equal(a, b)
    # record -> fields -> record is the identity for any bytes (every bit of a record is used exactly once)
    raw = rng.integers(0, 256, (n, 3072)).astype(np.uint8)
    again = layout.pack_tiles(*layout.unpack_tiles(raw))
    assert np.array_equal(again, raw)


def test_pack_exhaustive_bytes():
    """Every byte value at every byte position of both code regions survives unpack -> pack."""
    for region in (0, 1024):
        for byte_pos in range(0, 1024, 61):
            rec = np.zeros((256, 3072), np.uint8)
            rec[np.arange(256), region + byte_pos] = np.arange(256)
            assert np.array_equal(layout.pack_tiles(*layout.unpack_tiles(rec)), rec)


def test_record_field_offsets():
    rng = np.random.default_rng(2)
    ks = rng.standard_normal(128).astype(np.float16)
    vs = rng.standard_normal((32, 4)).astype(np.float16)
    z8 = np.zeros((32, 128), np.uint8)
    rec = layout.pack_tiles(z8, ks, np.zeros(128, np.float16), z8, vs, np.zeros((32, 4), np.float16))
    assert np.array_equal(rec[2048:2304].view(np.float16), ks)
    assert rec[2304:2560].view(np.float16).tolist() == [0.0] * 128
    # value scales are stored group-major: s_V[g][t] at index 32 g + t
    assert np.array_equal(rec[2560:2816].view(np.float16).reshape(4, 32), vs.T)


# ------------------------------------------------------------------ state machine
@pytest.mark.parametrize("R", [32, 128])
def test_flushed_tokens_closed_form_matches_simulation(R):
    for n0 in range(0, R + 1):
        for T in list(range(0, 2 * R + 3)) + [5 * R, 5 * R + 1]:
            if n0 == 0 and T == 0:
                continue
            # simulate the per-token rule on lengths only
            nr, flushed = n0, 0
            for _ in range(T):
                if nr == R:
                    flushed += R
                    nr = 0
                nr += 1
            assert oc.flushed_tokens(n0, T, R) == flushed, (n0, T)


def _tokens(rng, s, t, d=128):
    return rng.standard_normal((s, t, d)).astype(np.float16)


@pytest.mark.parametrize("T", [1, 31, 32, 127, 128, 129, 300, 513])
def test_prefill_equals_token_by_token(T):
    rng = np.random.default_rng(T)
    k, v = _tokens(rng, 3, T), _tokens(rng, 3, T)
    a = oc.SliceCache(3)
    a.append(k, v)
    b = oc.SliceCache(3)
    oc.append_block(b, k, v)
    assert (a.n_quant, a.n_resid) == (b.n_quant, b.n_resid)
    for x, y in zip(a.quantized(), b.quantized()):
        assert np.array_equal(x, y)
    assert np.array_equal(a.k_res, b.k_res) and np.array_equal(a.v_res, b.v_res)
    # the residual holds the newest tokens, byte for byte
    assert np.array_equal(a.k_res.view(np.uint16), k[:, T - a.n_resid:].view(np.uint16))
    assert np.array_equal(a.v_res.view(np.uint16), v[:, T - a.n_resid:].view(np.uint16))
    # the quantized part is the per-channel / per-token quantization of the oldest tokens
    kq, ks, kz = quant.quantize_keys_per_channel(k[:, :a.n_quant])
    assert np.array_equal(a.quantized()[0], kq) and np.array_equal(a.quantized()[1], ks)


def test_mixed_appends_match_one_prefill():
    rng = np.random.default_rng(4)
    k, v = _tokens(rng, 2, 700), _tokens(rng, 2, 700)
    a = oc.SliceCache(2)
    for lo, hi in [(0, 5), (5, 133), (133, 134), (134, 400), (400, 401), (401, 700)]:
        oc.append_block(a, k[:, lo:hi], v[:, lo:hi])
    b = oc.SliceCache(2)
    oc.append_block(b, k, v)
    for x, y in zip(a.quantized(), b.quantized()):
        assert np.array_equal(x, y)
    assert np.array_equal(a.k_res, b.k_res)


def test_workload_lengths():
    with open(os.path.join(GOLDEN, "cache_lengths.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        R = case["residual_cap"]
        sink = case.get("sink", 0)        # the first `sink` tokens are held apart before the window logic
        nr, nq = 0, 0
        flush_steps = []
        for i in range(case["prefill"] - sink):
            if nr == R:
                nq, nr = nq + R, 0
            nr += 1
        assert [nq, nr] == case["after_prefill"], case["name"]
        for step in range(1, case["steps"] + 1):
            if nr == R:
                nq, nr = nq + R, 0
                flush_steps.append(step)
            nr += 1
        assert [nq, nr] == case["final"], case["name"]
        assert flush_steps == case["flush_steps"], case["name"]
        f = oc.flushed_tokens(0, case["prefill"] + case["steps"] - sink, R)
        assert f == case["final"][0]
