"""One step of wide, trie-constrained beam search on AMD MI355X (gfx950).

Python face of the C ABI in include/gr.h.  Every step of the beam search runs
in the library's HIP kernels; this module only marshals arguments, and uses
PyTorch for device memory and streams.

    import torch, trie_constrained_beam_step_amd as gr
    trie = gr.Trie(offsets, tokens, children, vocab=V)        # per-level CSR
    beam = gr.Beam(batch=B, beam_width=K, vocab=V, max_steps=D, trie=trie,
                   dtype="bf16")
    for t in range(D):
        beam.step(logits_t)          # torch cuda tensor [B, K, V]
    st = beam.state()                # scores, nodes, sequences, parents, ...
"""
from __future__ import annotations

import ctypes as C
from typing import Optional, Sequence

import numpy as np

from . import _lib
from ._lib import BeamConfig, BeamView, StepIO, StepStats

__all__ = ["GrError", "Trie", "Beam", "beam_step_static", "trie_validate", "probe_read", "probe_copy",
           "probe_draw_error", "draw_error_bound", "version", "lib"]


def lib():
    return _lib.load()


class GrError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        name = lib().gr_status_string(status).decode()
        super().__init__(f"{name}: {message}")


def _check(status: int):
    if status != _lib.GR_OK:
        raise GrError(status, lib().gr_last_error().decode())


def _stream_ptr(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def version() -> str:
    return lib().gr_version().decode()


def _csr_arrays(offsets, tokens, children):
    offs = [np.ascontiguousarray(o, np.int64) for o in offsets]
    toks = [np.ascontiguousarray(t, np.int32) for t in tokens]
    chs = [np.ascontiguousarray(c, np.int32) for c in children]
    if not (len(offs) == len(toks) == len(chs)):
        raise ValueError("offsets, tokens and children need one array per level")
    return offs, toks, chs


def _csr_pointers(offs, toks, chs, num_nodes):
    D = len(offs)
    if num_nodes is None:
        num_nodes = [len(o) - 1 for o in offs] + [int(chs[-1].max()) + 1 if len(chs[-1]) else 0]
    nn = np.ascontiguousarray(num_nodes, np.int64)
    P = C.c_void_p * D
    po = P(*[o.ctypes.data for o in offs])
    pt = P(*[t.ctypes.data for t in toks])
    pc = P(*[c.ctypes.data for c in chs])
    return nn, po, pt, pc


def trie_validate(offsets, tokens, children, vocab: int, num_nodes: Optional[Sequence[int]] = None):
    """Host-only CSR check (gr_trie_validate); raises GrError on a violation."""
    offs, toks, chs = _csr_arrays(offsets, tokens, children)
    nn, po, pt, pc = _csr_pointers(offs, toks, chs, num_nodes)
    _check(lib().gr_trie_validate(len(offs), int(vocab), nn.ctypes.data, po, pt, pc))


class Trie:
    """A per-level CSR trie copied to device memory (gr_trie_build)."""

    def __init__(self, offsets, tokens, children, vocab: int,
                 num_nodes: Optional[Sequence[int]] = None, stream=None):
        offs, toks, chs = _csr_arrays(offsets, tokens, children)
        nn, po, pt, pc = _csr_pointers(offs, toks, chs, num_nodes)
        h = C.c_void_p()
        _check(lib().gr_trie_build(len(offs), int(vocab), nn.ctypes.data, po, pt, pc,
                                   _stream_ptr(stream), C.byref(h)))
        self._h = h
        self.depth = len(offs)
        self.vocab = int(vocab)

    @classmethod
    def from_csr(cls, obj, stream=None) -> "Trie":
        """From any object with .offsets, .tokens, .children lists and .vocab."""
        return cls(obj.offsets, obj.tokens, obj.children, obj.vocab,
                   getattr(obj, "num_nodes", None), stream)

    @property
    def handle(self):
        if self._h is None:
            raise ValueError("trie is closed")
        return self._h

    def info(self):
        d, v = C.c_int32(), C.c_int32()
        nn = np.zeros(self.depth + 1, np.int64)
        mf = np.zeros(self.depth, np.int32)
        _check(lib().gr_trie_info(self.handle, C.byref(d), C.byref(v), nn.ctypes.data, mf.ctypes.data))
        return dict(depth=d.value, vocab=v.value, num_nodes=nn.tolist(), max_fanout=mf.tolist())

    def densify(self, level: int, max_bytes: int = -1, stream=None) -> int:
        """Give `level` its dense child table (gr_trie_densify); returns the
        table's size in bytes.  Raises GrError (status GR_ERR_UNSUPPORTED)
        when the table would exceed max_bytes (>= 0)."""
        nb = C.c_int64()
        _check(lib().gr_trie_densify(self.handle, int(level), int(max_bytes), _stream_ptr(stream),
                                     C.byref(nb)))
        return nb.value

    def close(self):
        if getattr(self, "_h", None) is not None:
            lib().gr_trie_free(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Beam:
    """Beam state of B requests on the GPU, advanced by ``step``."""

    def __init__(self, batch: int, beam_width: int, vocab: int, max_steps: int, *,
                 eos: int = -1, dtype: str = "f32", trie: Optional[Trie] = None,
                 row_stride: int = 0, stream=None):
        if dtype not in ("f32", "bf16"):
            raise ValueError("dtype must be 'f32' or 'bf16'")
        self.cfg = BeamConfig(batch=batch, beam_width=beam_width, vocab=vocab,
                              max_steps=max_steps, eos_token=eos,
                              logits_dtype=_lib.GR_BF16 if dtype == "bf16" else _lib.GR_F32,
                              logits_row_stride=row_stride)
        self.dtype = dtype
        self.trie = trie  # keeps the trie alive as long as the beam
        h = C.c_void_p()
        _check(lib().gr_beam_init(C.byref(self.cfg), trie.handle if trie is not None else None,
                                  _stream_ptr(stream), C.byref(h)))
        self._h = h
        self.row_stride = row_stride or vocab

    @property
    def handle(self):
        if self._h is None:
            raise ValueError("beam is closed")
        return self._h

    def _check_logits(self, logits):
        import torch
        if not isinstance(logits, torch.Tensor) or not logits.is_cuda:
            raise TypeError("logits must be a torch tensor on the GPU")
        ok = {"f32": (torch.float32,), "bf16": (torch.bfloat16, torch.int16, torch.uint16)}
        if logits.dtype not in ok[self.dtype]:
            raise TypeError(f"logits dtype {logits.dtype} does not match the beam's {self.dtype}")
        c = self.cfg
        need = (c.batch * c.beam_width - 1) * self.row_stride + c.vocab
        if not logits.is_contiguous() or logits.numel() < need:
            raise ValueError(f"logits must be contiguous with >= {need} elements "
                             f"(B*K rows of stride {self.row_stride})")

    def step(self, logits, stream=None):
        """Enqueue one beam step on the stream (default: torch's current)."""
        self._check_logits(logits)
        _check(lib().gr_beam_step(self.handle, logits.data_ptr(), _stream_ptr(stream)))

    def step_ptr(self, ptr: int, stream=None):
        """Enqueue one step on a raw device pointer (no checks beyond the C ABI's)."""
        _check(lib().gr_beam_step(self.handle, int(ptr), _stream_ptr(stream)))

    def reset(self, stream=None):
        _check(lib().gr_beam_reset(self.handle, _stream_ptr(stream)))

    def search(self, logits, stream=None):
        """Enqueue len(logits) steps as one graph launch (see gr_beam_search);
        logits: contiguous device tensors [B, K, V] of the configured dtype."""
        for x in logits:
            self._check_logits(x)
        ptrs = (C.c_void_p * len(logits))(*[x.data_ptr() for x in logits])
        _check(lib().gr_beam_search(self.handle, ptrs, len(logits), _stream_ptr(stream)))

    def backward(self, grad_final, stream=None) -> dict:
        """Path gradients of the search so far (gr_beam_backward).

        grad_final: cuda float32 [B, K], the upstream gradient of each final
        slot's ranked score.  Returns cuda tensors path_slot, path_token
        [steps, B, K] (int32) and weight [B, K] (float32)."""
        import torch
        c = self.cfg
        B, K = c.batch, c.beam_width
        if not (isinstance(grad_final, torch.Tensor) and grad_final.is_cuda and
                grad_final.dtype == torch.float32 and grad_final.is_contiguous() and
                grad_final.numel() == B * K):
            raise TypeError("grad_final must be a contiguous cuda float32 tensor of B*K elements")
        steps = self.step_index
        dev = grad_final.device
        out = dict(path_slot=torch.empty((steps, B, K), dtype=torch.int32, device=dev),
                   path_token=torch.empty((steps, B, K), dtype=torch.int32, device=dev),
                   weight=torch.empty((B, K), dtype=torch.float32, device=dev))
        _check(lib().gr_beam_backward(self.handle, grad_final.data_ptr(), out["path_slot"].data_ptr(),
                                      out["path_token"].data_ptr(), out["weight"].data_ptr(),
                                      _stream_ptr(stream)))
        return out

    def backward_scatter(self, step: int, paths: dict, grad, stream=None):
        """Add step `step`'s log-probability gradient to grad, a contiguous
        cuda float32 [B, K, V] tensor (gr_beam_backward_scatter)."""
        import torch
        c = self.cfg
        if not (isinstance(grad, torch.Tensor) and grad.is_cuda and grad.dtype == torch.float32 and
                grad.is_contiguous() and grad.numel() == c.batch * c.beam_width * c.vocab):
            raise TypeError("grad must be a contiguous cuda float32 tensor [B, K, V]")
        _check(lib().gr_beam_backward_scatter(self.handle, int(step), paths["path_slot"].data_ptr(),
                                              paths["path_token"].data_ptr(), paths["weight"].data_ptr(),
                                              grad.data_ptr(), c.vocab, _stream_ptr(stream)))
        return grad

    def rewind(self):
        """Undo the last step (no copy, nothing enqueued); once per step."""
        _check(lib().gr_beam_rewind(self.handle))

    def view(self) -> BeamView:
        v = BeamView()
        _check(lib().gr_beam_view_get(self.handle, C.byref(v)))
        return v

    @property
    def step_index(self) -> int:
        return self.view().step

    def state(self, stream=None) -> dict:
        """Copies of the device state as torch cuda tensors."""
        import torch
        v = self.view()
        B, K, T = v.batch, v.beam_width, v.max_steps
        dev = torch.device("cuda", torch.cuda.current_device())
        out = dict(
            scores=torch.empty((B, K), dtype=torch.float32, device=dev),
            nodes=torch.empty((B, K), dtype=torch.int32, device=dev),
            finished=torch.empty((B, K), dtype=torch.uint8, device=dev),
            sequences=torch.empty((B, K, T), dtype=torch.int32, device=dev),
            parents=torch.empty((T, B, K), dtype=torch.int32, device=dev),
            tokens=torch.empty((T, B, K), dtype=torch.int32, device=dev),
            lse=torch.empty((B, K), dtype=torch.float32, device=dev),
        )
        s = _stream_ptr(stream)
        for name, ptr in (("scores", v.scores), ("nodes", v.nodes), ("finished", v.finished),
                          ("sequences", v.sequences), ("parents", v.parents),
                          ("tokens", v.tokens), ("lse", v.lse)):
            t = out[name]
            _check(lib().gr_memcpy(t.data_ptr(), ptr, t.numel() * t.element_size(), s))
        out["step"] = v.step
        return out

    def set_state(self, step: int, scores, nodes, finished, sequences, stream=None):
        import torch
        for t, dt in ((scores, torch.float32), (nodes, torch.int32), (finished, torch.uint8),
                      (sequences, torch.int32)):
            if not (isinstance(t, torch.Tensor) and t.is_cuda and t.dtype == dt and t.is_contiguous()):
                raise TypeError(f"state tensors must be contiguous cuda {dt}")
        _check(lib().gr_beam_set_state(self.handle, int(step), scores.data_ptr(), nodes.data_ptr(),
                                       finished.data_ptr(), sequences.data_ptr(),
                                       _stream_ptr(stream)))

    def set_sampling(self, temperature: float, seed: int = 0):
        """Gumbel top-K sampling at temperature > 0 from the next step on
        (0 restores the deterministic top-K); see gr_beam_set_sampling."""
        _check(lib().gr_beam_set_sampling(self.handle, float(temperature), int(seed) & (2**64 - 1)))

    def set_penalties(self, alpha: float = 0.0, min_length: int = 0, banned=None, stream=None):
        """GNMT length penalty exponent, minimum hypothesis length for EOS and
        tokens never emitted, from the next step on (gr_beam_set_penalties)."""
        ban = np.ascontiguousarray(banned if banned is not None else [], np.int32)
        _check(lib().gr_beam_set_penalties(self.handle, float(alpha), int(min_length),
                                           ban.ctypes.data if len(ban) else None, len(ban),
                                           _stream_ptr(stream)))

    def set_normalization(self, mode: str = "full", lo: int = 0, hi: int = 0):
        """Normaliser of later steps: "full" (the row), "range" (tokens
        [lo, hi) only), "slice" (a trie row's children only) or "none" (the
        values are log-probabilities already: lse = 0)."""
        m = {"full": 0, "range": 1, "slice": 2, "none": 3}[mode]
        _check(lib().gr_beam_set_normalization(self.handle, m, int(lo), int(hi)))

    def set_fused(self, mode=True):
        """gr_beam_set_fused: True / 1 (default) fuses the launch-bound
        short-row trie steps, False / 0 runs every step as the row and request
        kernels, 2 also fuses requests split over several workgroups."""
        _check(lib().gr_beam_set_fused(self.handle, int(mode)))

    def timing_enable(self, on: bool = True):
        _check(lib().gr_beam_timing_enable(self.handle, 1 if on else 0))

    def timing(self):
        r, s, n = C.c_double(), C.c_double(), C.c_int64()
        _check(lib().gr_beam_timing_get(self.handle, C.byref(r), C.byref(s), C.byref(n)))
        return dict(row_ms=r.value, select_ms=s.value, steps=n.value)

    def timing_reset(self):
        _check(lib().gr_beam_timing_reset(self.handle))

    def last_stats(self) -> dict:
        st = StepStats()
        _check(lib().gr_beam_last_stats(self.handle, C.byref(st)))
        return dict(rows_read=st.rows_read, candidates=st.candidates, survivors=st.survivors,
                    slow_path_requests=st.slow_path_requests, rescanned_rows=st.rescanned_rows,
                    fused_requests=st.fused_requests)

    def close(self):
        if getattr(self, "_h", None) is not None:
            lib().gr_beam_free(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def beam_step_static(batch: int, beam_width: int, vocab: int, max_steps: int, step: int, logits,
                     state: dict, out: dict, *, eos: int = -1, dtype: str = "f32",
                     trie: Optional[Trie] = None, live_bound: int = 0, row_stride: int = 0,
                     temperature: float = 0.0, seed: int = 0, stream=None):
    """One beam step without a handle and without allocating
    (gr_beam_step_static): the step's workspace is the library's static
    buffer of GR_STATIC_SCRATCH_BYTES per GPU, shared by every call on that
    GPU (calls that overlap on one GPU race).

    state: cuda tensors scores [B, K] f32, nodes [B, K] i32, finished
    [B, K] u8, sequences [B, K, T] i32 -- the state before the step.
    out: the same four plus parents, tokens [B, K] i32 and lse [B, K] f32,
    written by the step (they must not overlap state)."""
    import torch
    if dtype not in ("f32", "bf16"):
        raise ValueError("dtype must be 'f32' or 'bf16'")
    want = dict(scores=torch.float32, nodes=torch.int32, finished=torch.uint8, sequences=torch.int32,
                parents=torch.int32, tokens=torch.int32, lse=torch.float32)
    for d, names in ((state, ("scores", "nodes", "finished", "sequences")), (out, tuple(want))):
        for k in names:
            t = d[k]
            if not (isinstance(t, torch.Tensor) and t.is_cuda and t.dtype == want[k] and t.is_contiguous()):
                raise TypeError(f"{k} must be a contiguous cuda {want[k]} tensor")
    if not (isinstance(logits, torch.Tensor) and logits.is_cuda and logits.is_contiguous()):
        raise TypeError("logits must be a contiguous cuda tensor")
    io = StepIO()
    io.config = BeamConfig(batch=batch, beam_width=beam_width, vocab=vocab, max_steps=max_steps,
                           eos_token=eos, logits_dtype=_lib.GR_BF16 if dtype == "bf16" else _lib.GR_F32,
                           logits_row_stride=row_stride)
    io.trie = trie.handle if trie is not None else None
    io.step, io.live_bound = int(step), int(live_bound)
    io.temperature, io.seed = float(temperature), int(seed) & (2**64 - 1)
    io.logits = logits.data_ptr()
    io.scores, io.nodes = state["scores"].data_ptr(), state["nodes"].data_ptr()
    io.finished, io.sequences = state["finished"].data_ptr(), state["sequences"].data_ptr()
    io.scores_out, io.nodes_out = out["scores"].data_ptr(), out["nodes"].data_ptr()
    io.finished_out, io.sequences_out = out["finished"].data_ptr(), out["sequences"].data_ptr()
    io.parents_out, io.tokens_out, io.lse_out = (out["parents"].data_ptr(), out["tokens"].data_ptr(),
                                                 out["lse"].data_ptr())
    _check(lib().gr_beam_step_static(C.byref(io), _stream_ptr(stream)))


def probe_read(src, sink, stream=None):
    """Streaming-read probe over a cuda tensor (gr_probe_read)."""
    nbytes = src.numel() * src.element_size()
    _check(lib().gr_probe_read(src.data_ptr(), nbytes - nbytes % 16, sink.data_ptr(),
                               _stream_ptr(stream)))


def probe_draw_error(out, r0: int = 0, count: int = 1 << 32, stream=None):
    """Largest |fast - exact| Gumbel variate over Philox words r0 .. r0+count-1
    into the cuda float64 tensor `out` (one element; gr_probe_draw_error)."""
    assert out.dtype.itemsize == 8 and out.numel() >= 1
    _check(lib().gr_probe_draw_error(r0, count, out.data_ptr(), _stream_ptr(stream)))


def draw_error_bound() -> float:
    """The bound on that difference the sampled-row pruning assumes."""
    return float(lib().gr_draw_error_bound())


def probe_copy(dst, src, stream=None):
    """Plain copy kernel of known traffic (gr_probe_copy)."""
    nbytes = min(src.numel() * src.element_size(), dst.numel() * dst.element_size())
    _check(lib().gr_probe_copy(dst.data_ptr(), src.data_ptr(), nbytes - nbytes % 16,
                               _stream_ptr(stream)))
