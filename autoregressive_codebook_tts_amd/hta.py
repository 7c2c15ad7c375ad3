"""ctypes binding of libhta.so (the gfx950 codebook-TTS decode library).

Argument marshalling only: every step of the decode path runs in the HIP
kernels behind the C ABI declared in include/hta.h.  torch provides device
memory (the workspace and weight tensors) and the stream.  When the library is
missing the import fails loudly; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import sys
import weakref

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libhta.so")

HTA_OK, HTA_DONE = 0, 1
HTA_E_ARG, HTA_E_STATE, HTA_E_CAPACITY, HTA_E_RANGE, HTA_E_UNSUPPORTED, HTA_E_HIP, HTA_E_TIMEOUT = range(-1, -8, -1)
ERRORS = {-1: "HTA_E_ARG", -2: "HTA_E_STATE", -3: "HTA_E_CAPACITY", -4: "HTA_E_RANGE", -5: "HTA_E_UNSUPPORTED",
          -6: "HTA_E_HIP", -7: "HTA_E_TIMEOUT"}
HTA_BF16, HTA_FP8_E4M3 = 0, 1
HTA_SRC_F32, HTA_SRC_BF16 = 0, 1
(TAP_HIDDEN, TAP_LOGITS, TAP_STATE, TAP_KV, TAP_AMAX, TAP_PREFILL_HIDDEN, TAP_W_QKV, TAP_S_QKV, TAP_W_GU, TAP_S_GU,
 TAP_LAYER_H, TAP_PREFILL_LAYER, TAP_TRACE, TAP_ACT, TAP_Q) = range(15)
ACTS_WIDTH = 10240  # row width of TAP_ACT
OPT_USE_GRAPH = 0
OPT_TAPS = 2
OPT_PREFILL_TAP_LAYER = 3
OPT_TRACE = 4
OPT_FORCE_TIMEOUT = 5
OPT_FP8_MFMA = 6
SITES_PER_LAYER = 4

LAYER_TENSORS = ("g_attn", "wq", "wk", "wv", "g_q", "g_k", "wo", "g_mlp", "wg", "wu", "wd")


class HtaConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in ("n_layers", "hidden", "n_q_heads", "n_kv_heads", "head_dim", "ffn",
                                             "text_vocab", "n_codebooks", "codebook_size", "bos_id", "eos_id")] + [
        ("rope_theta", ctypes.c_float), ("rms_eps", ctypes.c_float),
        ("max_seq", ctypes.c_int), ("max_prefill", ctypes.c_int), ("precision", ctypes.c_int),
        ("n_streams", ctypes.c_int)]


class HtaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{ERRORS.get(code, code)}: {msg}")
        self.code = code


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        P, I, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        sig = {
            "hta_create": (I, [ctypes.POINTER(HtaConfig), P, ctypes.POINTER(P)]),
            "hta_workspace_bytes": (S, [ctypes.POINTER(HtaConfig)]),
            "hta_bind_workspace": (I, [P, P, S]),
            "hta_load_weights": (I, [P, ctypes.POINTER(P), I, I, P]),
            "hta_prefill": (I, [P, P, I]),
            "hta_decode_frame": (I, [P, P]),
            "hta_decode_frames": (I, [P, I, P, P]),
            "hta_decode_frames_noalloc": (I, [P, I, P, P]),
            "hta_reset": (I, [P, I]),
            "hta_select_stream": (I, [P, I]),
            "hta_force_codes": (I, [P, P]),
            "hta_set_sampling": (I, [P, ctypes.c_float, ctypes.c_uint64]),
            "hta_read_tap": (I, [P, I, I, P, S]),
            "hta_calibrate": (I, [P, P, I, I, P, P]),
            "hta_layer_step": (I, [P, I, I, P, P, P]),
            "hta_gemm": (I, [P, P, P, P, ctypes.c_float, I, I, I, P]),
            "hta_undelay": (I, [P, I, I, I, P, P]),
            "hta_stream_create": (I, [I, I, I, I, I, I, ctypes.POINTER(P)]),
            "hta_stream_push": (I, [P, P, I, P, I, P, P]),
            "hta_stream_finish": (I, [P, P, I, P]),
            "hta_stream_destroy": (None, [P]),
            "hta_set_option": (I, [P, I, I]),
            "hta_time_kernels": (I, [P, I, P, I]),
            "hta_destroy": (None, [P]),
            "hta_last_error": (ctypes.c_char_p, [P]),
            "hta_version": (ctypes.c_char_p, []),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> ctypes.c_void_p:
    return ctypes.c_void_p(a.ctypes.data)


def make_config(shape, precision: int, max_seq: int, max_prefill: int, n_streams: int = 1) -> HtaConfig:
    return HtaConfig(shape.n_layers, shape.hidden, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.ffn,
                     shape.text_vocab, shape.n_codebooks, shape.codebook_size, shape.bos_id, shape.eos_id,
                     float(shape.rope_theta), float(shape.rms_eps), max_seq, max_prefill, precision, n_streams)


def workspace_bytes(cfg: HtaConfig) -> int:
    return int(lib().hta_workspace_bytes(ctypes.byref(cfg)))


def abi_tensor_names(n_layers: int):
    """Weight tensor order hta_load_weights expects."""
    names = ["e_text", "e_aud"]
    for layer in range(n_layers):
        names += [f"layers.{layer}.{n}" for n in LAYER_TENSORS]
    return names + ["g_final", "w_head"]


def undelay(step_codes: np.ndarray, eos: int = 1025) -> np.ndarray:
    """Host-only un-delay through the library's hta_undelay."""
    steps = np.ascontiguousarray(step_codes, dtype=np.int32)
    T, C = steps.shape
    out = np.zeros((max(T, 1), C), dtype=np.int32)
    n = ctypes.c_int(0)
    rc = lib().hta_undelay(_ptr(steps), T, C, eos, _ptr(out), ctypes.byref(n))
    if rc != HTA_OK:
        raise HtaError(rc, "hta_undelay")
    return out[: n.value].copy()


_open = weakref.WeakSet()  # live contexts, closed by close_all()


STREAM_RUNNING, STREAM_DONE, STREAM_STOPPED, STREAM_CAPPED = 0, 1, 2, 3


class Streamer:
    """hta_stream_*: incremental un-delay, chunked hand-off and the repeated-code stop guard."""

    def __init__(self, n_codebooks: int = 8, bos: int = 1024, eos: int = 1025, chunk_frames: int = 25,
                 guard_window: int = 50, guard_max_period: int = 4):
        self.C = n_codebooks
        self.s = ctypes.c_void_p()
        rc = lib().hta_stream_create(n_codebooks, bos, eos, chunk_frames, guard_window, guard_max_period,
                                     ctypes.byref(self.s))
        if rc != HTA_OK:
            raise HtaError(rc, "hta_stream_create")
        self.status = STREAM_RUNNING

    def push(self, step_codes, max_frames: int = 1 << 16) -> np.ndarray:
        steps = np.ascontiguousarray(step_codes, dtype=np.int32).reshape(-1, self.C)
        out = np.zeros((max_frames, self.C), dtype=np.int32)
        n, st = ctypes.c_int(0), ctypes.c_int(0)
        rc = lib().hta_stream_push(self.s, _ptr(steps), steps.shape[0], _ptr(out), max_frames, ctypes.byref(n),
                                   ctypes.byref(st))
        if rc != HTA_OK:
            raise HtaError(rc, "hta_stream_push")
        self.status = st.value
        return out[: n.value].copy()

    def finish(self, max_frames: int = 1 << 16) -> np.ndarray:
        out = np.zeros((max_frames, self.C), dtype=np.int32)
        n = ctypes.c_int(0)
        rc = lib().hta_stream_finish(self.s, _ptr(out), max_frames, ctypes.byref(n))
        if rc != HTA_OK:
            raise HtaError(rc, "hta_stream_finish")
        if self.status == STREAM_RUNNING:
            self.status = STREAM_CAPPED
        return out[: n.value].copy()

    def close(self) -> None:
        if self.s:
            lib().hta_stream_destroy(self.s)
            self.s = ctypes.c_void_p()

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()
        return False


def close_all() -> None:
    """Destroy every open context (tests and the benchmark call this before exiting, so
    that no graph or stream is destroyed during interpreter teardown)."""
    for ctx in list(_open):
        ctx.close()


class Hta:
    """One decode context on the current GPU with a torch-allocated workspace.

    Close it explicitly (close(), or use it as a context manager): hta_destroy waits for
    the stream and destroys the captured frame graph, which must happen while the HIP
    runtime is still up and before torch frees the workspace the graph references."""

    def __init__(self, shape, precision: str = "bf16", max_seq: int = 2048, max_prefill: int = 512, stream=None,
                 fill_byte: int | None = None, n_streams: int = 1):
        import torch

        self.torch = torch
        self.shape = shape
        self.precision = precision
        self.cfg = make_config(shape, HTA_FP8_E4M3 if precision == "fp8" else HTA_BF16, max_seq, max_prefill, n_streams)
        self.M = max(1, n_streams)
        self.stream = stream if stream is not None else torch.cuda.Stream()
        self.ctx = ctypes.c_void_p()
        rc = lib().hta_create(ctypes.byref(self.cfg), ctypes.c_void_p(self.stream.cuda_stream), ctypes.byref(self.ctx))
        if rc != HTA_OK:
            raise HtaError(rc, "hta_create")
        nbytes = workspace_bytes(self.cfg)
        self.ws = torch.empty(nbytes + 256, dtype=torch.uint8, device="cuda")
        if fill_byte is not None:  # sentinel fill, so tests can see which bytes the kernels wrote
            self.ws.fill_(fill_byte)
        base = self.ws.data_ptr()
        aligned = (base + 255) // 256 * 256
        torch.cuda.synchronize()
        self._check(lib().hta_bind_workspace(self.ctx, ctypes.c_void_p(aligned), nbytes), "hta_bind_workspace")
        self.C = shape.n_codebooks
        self.V = shape.codebook_size
        _open.add(self)

    # ------------------------------------------------------------------ plumbing
    def _check(self, rc: int, what: str) -> int:
        if rc < 0:
            raise HtaError(rc, f"{what}: {lib().hta_last_error(self.ctx).decode()}")
        return rc

    def close(self) -> None:
        if self.ctx:
            lib().hta_destroy(self.ctx)
            self.ctx = ctypes.c_void_p()
        self.ws = None
        _open.discard(self)

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()
        return False

    def __del__(self, _finalizing=sys.is_finalizing):
        # During interpreter teardown the HIP runtime (and a profiler's tool library)
        # may already be gone: a context still open then is left to process exit
        # rather than destroyed through a runtime that no longer exists.  (The check is
        # bound at definition: module globals such as sys may already be None then.)
        if _finalizing():
            return
        try:
            self.close()
        except Exception:
            pass

    # ------------------------------------------------------------------ API
    def load_weights(self, tensors, src_dtype: int, act_scales=None) -> None:
        """``tensors``: device tensors in ``abi_tensor_names`` order."""
        self.torch.cuda.synchronize()
        arr = (ctypes.c_void_p * len(tensors))(*[t.data_ptr() for t in tensors])
        sc = None
        if act_scales is not None:
            self._scales = np.ascontiguousarray(act_scales, dtype=np.float32)
            sc = _ptr(self._scales)
        self._check(lib().hta_load_weights(self.ctx, arr, len(tensors), src_dtype, sc), "hta_load_weights")

    def prefill(self, tokens) -> None:
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        self._check(lib().hta_prefill(self.ctx, _ptr(t), t.shape[0]), "hta_prefill")

    def decode_frame(self):
        """One step: codes [C] (single stream) or [M][C] (batched)."""
        out = np.zeros((self.M, self.C) if self.M > 1 else self.C, dtype=np.int32)
        rc = self._check(lib().hta_decode_frame(self.ctx, _ptr(out)), "hta_decode_frame")
        return out, rc == HTA_DONE

    def decode_frames(self, n: int):
        """n steps: codes [n][C] (single stream) or [n][M][C] (batched)."""
        out = np.zeros((n, self.M, self.C) if self.M > 1 else (n, self.C), dtype=np.int32)
        nd = ctypes.c_int(0)
        rc = self._check(lib().hta_decode_frames(self.ctx, n, _ptr(out), ctypes.byref(nd)), "hta_decode_frames")
        return out, rc == HTA_DONE

    def select_stream(self, m: int) -> None:
        """hta_select_stream: the stream that prefill, reset, force_codes and the taps act on."""
        self._check(lib().hta_select_stream(self.ctx, m), "hta_select_stream")

    def decode_frames_noalloc(self, n: int, out=None):
        """hta_decode_frames_noalloc: the exchange words in the library's static per-GPU array.
        `out` (int32 [n][C], C-contiguous) is filled in place when given."""
        if out is None:
            out = np.zeros((n, self.C), dtype=np.int32)
        if out.dtype != np.int32 or out.shape != (n, self.C) or not out.flags.c_contiguous:
            raise ValueError("out must be a C-contiguous int32 array of shape (n, C)")
        nd = ctypes.c_int(0)
        rc = self._check(lib().hta_decode_frames_noalloc(self.ctx, n, _ptr(out), ctypes.byref(nd)),
                         "hta_decode_frames_noalloc")
        return out, rc == HTA_DONE

    def reset(self, keep_len: int = 0) -> None:
        self._check(lib().hta_reset(self.ctx, keep_len), "hta_reset")

    def set_sampling(self, temperature: float, seed: int = 0) -> None:
        """hta_set_sampling: 0 = greedy argmax; > 0 = categorical draw keyed by (seed, step, codebook)."""
        self._check(lib().hta_set_sampling(self.ctx, float(temperature), int(seed) & 0xFFFFFFFFFFFFFFFF),
                    "hta_set_sampling")

    def force_codes(self, codes) -> None:
        c = np.ascontiguousarray(codes, dtype=np.int32)
        self._check(lib().hta_force_codes(self.ctx, _ptr(c)), "hta_force_codes")

    KERNEL_CLASSES = ("embed", "qkv", "attn", "o_proj", "gate_up", "down", "head", "frame")

    def time_kernels(self, n_frames: int) -> dict:
        """Average device microseconds per launch of each decode kernel class over n_frames
        eagerly launched frames (events on the context stream)."""
        out = np.zeros(len(self.KERNEL_CLASSES), np.float32)
        self._check(lib().hta_time_kernels(self.ctx, n_frames, _ptr(out), out.shape[0]), "hta_time_kernels")
        return dict(zip(self.KERNEL_CLASSES, out.tolist()))

    def set_option(self, option: int, value: int) -> None:
        self._check(lib().hta_set_option(self.ctx, option, value), "hta_set_option")

    def _tap(self, tap: int, layer: int, out: np.ndarray) -> np.ndarray:
        self._check(lib().hta_read_tap(self.ctx, tap, layer, _ptr(out), out.nbytes), "hta_read_tap")
        return out

    def tap_hidden(self) -> np.ndarray:
        return self._tap(TAP_HIDDEN, 0, np.zeros(self.shape.hidden, np.float32))

    def tap_logits(self) -> np.ndarray:
        return self._tap(TAP_LOGITS, 0, np.zeros((self.C, self.V), np.float32))

    def tap_state(self) -> dict:
        s = self._tap(TAP_STATE, 0, np.zeros(4 + 2 * self.C, np.int32))
        return {"len": int(s[0]), "t": int(s[1]), "eoc": int(s[2]), "done": int(s[3]),
                "prev": s[4:4 + self.C].copy(), "codes": s[4 + self.C:].copy()}

    def tap_kv(self, layer: int, length: int) -> tuple:
        """K and V (bf16 bits, [Hkv][length][hd]) of positions [0, length)."""
        sh = self.shape
        buf = np.zeros((2, sh.n_kv_heads, length, sh.head_dim), np.uint16)
        self._tap(TAP_KV, layer, buf)
        return buf[0], buf[1]

    def tap_amax(self) -> np.ndarray:
        return self._tap(TAP_AMAX, 0, np.zeros(SITES_PER_LAYER * self.shape.n_layers + 1, np.float32))

    def tap_packed(self, layer: int, which: str) -> np.ndarray:
        """Packed weight rows ('qkv' or 'gu') as uint16 bf16 bits or uint8 e4m3 codes, or their
        FP8 scales ('s_qkv', 's_gu')."""
        sh = self.shape
        rows = (sh.n_q_heads + 2 * sh.n_kv_heads) * sh.head_dim if which in ("qkv", "s_qkv") else 2 * sh.ffn
        tap = {"qkv": TAP_W_QKV, "s_qkv": TAP_S_QKV, "gu": TAP_W_GU, "s_gu": TAP_S_GU}[which]
        if which.startswith("s_"):
            buf = np.zeros(rows, np.float32)
        else:
            buf = np.zeros((rows, sh.hidden), np.uint8 if self.precision == "fp8" else np.uint16)
        return self._tap(tap, layer, buf)

    def tap_layers(self) -> np.ndarray:
        """[n_layers + 1][d]: the residual entering each layer of the last frame, then the final one
        (needs OPT_TAPS on)."""
        return self._tap(TAP_LAYER_H, 0, np.zeros((self.shape.n_layers + 1, self.shape.hidden), np.float32))

    def tap_prefill_layer(self, P: int) -> np.ndarray:
        """[2][P][d]: the rows entering and leaving the selected layer in the last prefill (OPT_TAPS on)."""
        return self._tap(TAP_PREFILL_LAYER, 0, np.zeros((2, P, self.shape.hidden), np.float32))

    def tap_trace(self, blocks: int) -> np.ndarray:
        """[blocks][5 * n_layers + 1][8] uint32 phase timestamps (100 MHz clock) and stream
        counters of the last persistent frame (needs OPT_TRACE on)."""
        return self._tap(TAP_TRACE, 0, np.zeros((blocks, 5 * self.shape.n_layers + 1, 8), np.uint32))

    def tap_acts(self) -> np.ndarray:
        """[5 * n_layers + 1][ACTS_WIDTH] uint16: the GEMV input of every phase of the last
        frame as bf16 bits (needs OPT_TAPS on)."""
        return self._tap(TAP_ACT, 0, np.zeros((5 * self.shape.n_layers + 1, ACTS_WIDTH), np.uint16))

    def tap_q(self) -> np.ndarray:
        """[n_layers][Hq][hd] uint16: bf16 bits of the rotated queries of the last frame (OPT_TAPS on)."""
        sh = self.shape
        return self._tap(TAP_Q, 0, np.zeros((sh.n_layers, sh.n_q_heads, sh.head_dim), np.uint16))

    def tap_prefill_hidden(self, P: int) -> np.ndarray:
        return self._tap(TAP_PREFILL_HIDDEN, 0, np.zeros((P, self.shape.hidden), np.float32))

    def calibrate(self, tokens, n_frames: int, forced_codes=None) -> np.ndarray:
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        out = np.zeros(SITES_PER_LAYER * self.shape.n_layers + 1, np.float32)
        fc = None
        if forced_codes is not None:
            self._forced = np.ascontiguousarray(forced_codes, dtype=np.int32)
            fc = _ptr(self._forced)
        self._check(lib().hta_calibrate(self.ctx, _ptr(t), t.shape[0], n_frames, fc, _ptr(out)), "hta_calibrate")
        return out

    def layer_step(self, layer: int, kv_len: int, k_init, v_init, h) -> None:
        """One-layer context: run the frame kernel's layer 0 on device tensor ``h`` (float32 [d],
        in place) at position kv_len - 1, after filling KV positions [0, kv_len - 1)."""
        self.torch.cuda.synchronize()
        kp = ctypes.c_void_p(k_init.data_ptr()) if k_init is not None else None
        vp = ctypes.c_void_p(v_init.data_ptr()) if v_init is not None else None
        self._check(lib().hta_layer_step(self.ctx, layer, kv_len, kp, vp, ctypes.c_void_p(h.data_ptr())),
                    "hta_layer_step")


    def gemm(self, A, W, w_scale, a_scale: float, C) -> None:
        """C = A . W^T with the prefill's GEMM kernels: device tensors A [M][K] and W [N][K]
        (uint8 e4m3 codes with float32 w_scale [N] on an FP8 context; bf16 on a BF16 one,
        w_scale None), C float32 [M][N]."""
        M, K = A.shape
        N = W.shape[0]
        if W.shape[1] != K or tuple(C.shape) != (M, N) or not (A.is_contiguous() and W.is_contiguous()
                                                               and C.is_contiguous()):
            raise ValueError("gemm: A [M][K], W [N][K] and C [M][N] must be contiguous and agree")
        self.torch.cuda.synchronize()
        ws = ctypes.c_void_p(w_scale.data_ptr()) if w_scale is not None else None
        self._check(lib().hta_gemm(self.ctx, ctypes.c_void_p(A.data_ptr()), ctypes.c_void_p(W.data_ptr()), ws,
                                   float(a_scale), M, N, K, ctypes.c_void_p(C.data_ptr())), "hta_gemm")


def weights_to_device(named: dict, n_layers: int):
    """Upload numpy weights (float32 arrays, or uint16 bfloat16 bit patterns) as torch
    device tensors in ABI order; returns (tensors, src_dtype)."""
    import torch

    names = abi_tensor_names(n_layers)
    first = named[names[0]]
    src = HTA_SRC_BF16 if first.dtype == np.uint16 else HTA_SRC_F32
    out = []
    for n in names:
        a = np.ascontiguousarray(named[n])
        if src == HTA_SRC_BF16:
            t = torch.from_numpy(a.view(np.int16)).to("cuda")
        else:
            t = torch.from_numpy(a.astype(np.float32, copy=False)).to("cuda")
        out.append(t)
    return out, src
