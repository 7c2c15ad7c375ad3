"""Streaming hand-off (hta_stream_*, host only): incremental un-delay in chunks equals the
oracle's one-shot un-delay, and the repeated-code stop guard fires where the oracle's
restatement of the rule does.  The oracle's guard is pinned here by hand-built cases."""
import numpy as np
import pytest

from autoregressive_codebook_tts_amd import hta
from oracle.delay import delay_frames, find_eoc, repeat_guard, undelay

C = 8


def _frames(rng, n):
    return rng.integers(0, 1024, size=(n, C))


# ----------------------------------------------------------------------------- oracle pins
def test_oracle_guard_hand_cases():
    rng = np.random.default_rng(1)
    distinct = _frames(rng, 30)
    assert repeat_guard(distinct, 10, 4) is None
    const = np.vstack([distinct[:12], np.tile(distinct[12], (15, 1))])
    # the constant run starts at frame 12; its 10th frame is frame 21
    assert repeat_guard(const, 10, 4) == 21
    assert repeat_guard(const, 10, 0) is None
    per3 = np.vstack([distinct[:5], np.tile(distinct[5:8], (6, 1))])  # frames 5.. repeat with period 3
    assert repeat_guard(per3, 9, 4) == 13
    assert repeat_guard(per3, 9, 2) is None
    per5 = np.vstack([distinct[:2], np.tile(distinct[2:7], (5, 1))])
    assert repeat_guard(per5, 12, 4) is None
    assert repeat_guard(per5, 12, 5) == 13
    # a window shorter than the period it would need never fires
    assert repeat_guard(per5, 5, 5) is None


# ----------------------------------------------------------------------------- library vs oracle
def _stream(steps, chunk, window, max_period, push_sizes, max_frames=1 << 16):
    out, sizes = [], []
    with hta.Streamer(C, 1024, 1025, chunk, window, max_period) as s:
        i = 0
        j = 0
        while i < len(steps) and s.status == hta.STREAM_RUNNING:
            n = push_sizes[j % len(push_sizes)]
            got = s.push(steps[i: i + n], max_frames)
            out.append(got)
            sizes.append(len(got))
            i += n
            j += 1
        if s.status == hta.STREAM_RUNNING:
            got = s.finish(max_frames)
            out.append(got)
            sizes.append(len(got))
        while True:  # drain what max_frames held back
            got = s.push(np.zeros((0, C), np.int32), max_frames)
            if len(got) == 0:
                break
            out.append(got)
            sizes.append(len(got))
        status = s.status
    return np.concatenate(out) if out else np.zeros((0, C)), sizes, status


@pytest.mark.parametrize("chunk", [1, 3, 25])
@pytest.mark.parametrize("n", [0, 1, 7, 60])
def test_stream_with_eoc_equals_one_shot_undelay(chunk, n):
    rng = np.random.default_rng(100 + n)
    steps = delay_frames(_frames(rng, n))  # EOC at step n, done after step n + 7
    got, sizes, status = _stream(steps, chunk, 0, 0, [1, 5, 2, 11])
    assert np.array_equal(got, undelay(steps, find_eoc(steps)))
    assert status == hta.STREAM_DONE
    assert all(k % chunk == 0 for k in sizes[:-1] if k)  # whole chunks until the end


@pytest.mark.parametrize("T", [3, 8, 40])
def test_stream_capped_without_eoc_equals_one_shot_undelay(T):
    rng = np.random.default_rng(T)
    steps = rng.integers(0, 1024, size=(T, C))
    got, _, status = _stream(steps, 4, 0, 0, [3])
    assert np.array_equal(got, undelay(steps, None))
    assert status == hta.STREAM_CAPPED


@pytest.mark.parametrize("window,max_period", [(10, 1), (12, 4), (20, 3)])
def test_stream_guard_matches_oracle(window, max_period):
    rng = np.random.default_rng(window)
    frames = np.vstack([_frames(rng, 17), np.tile(_frames(rng, max_period), (12, 1)), _frames(rng, 10)])
    steps = delay_frames(frames)
    f = repeat_guard(undelay(steps, find_eoc(steps)), window, max_period)
    assert f is not None
    got, _, status = _stream(steps, 5, window, max_period, [4, 1])
    assert status == hta.STREAM_STOPPED
    assert np.array_equal(got, frames[: f + 1])


def test_stream_guard_quiet_on_distinct_frames_and_small_output_buffers():
    rng = np.random.default_rng(9)
    steps = delay_frames(_frames(rng, 80))
    got, sizes, status = _stream(steps, 8, 50, 4, [13], max_frames=16)
    assert status == hta.STREAM_DONE
    assert np.array_equal(got, undelay(steps, find_eoc(steps)))
    assert max(sizes) <= 16


def test_stream_argument_errors():
    L = hta.lib()
    import ctypes
    s = ctypes.c_void_p()
    assert L.hta_stream_create(0, 1024, 1025, 4, 0, 0, ctypes.byref(s)) == hta.HTA_E_ARG
    assert L.hta_stream_create(8, 1024, 1025, 0, 0, 0, ctypes.byref(s)) == hta.HTA_E_ARG
    assert L.hta_stream_create(8, 1024, 1025, 4, -1, 0, ctypes.byref(s)) == hta.HTA_E_ARG
    with hta.Streamer(C, 1024, 1025, 4, 0, 0) as st:
        n = ctypes.c_int(0)
        assert L.hta_stream_push(st.s, None, 2, None, 0, ctypes.byref(n), None) == hta.HTA_E_ARG
