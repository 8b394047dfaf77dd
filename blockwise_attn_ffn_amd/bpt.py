"""Thin ctypes binding of libbpt.so (declared in include/bpt.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels. torch is used for device memory and streams; the binding passes
``tensor.data_ptr()`` and the stream handle through unchanged.
"""
from __future__ import annotations

import ctypes
import os

from .build import LIB_PATH

F32, BF16 = 0, 1
STATUS = {0: "BPT_OK", 1: "BPT_ERR_NULL", 2: "BPT_ERR_SHAPE", 3: "BPT_ERR_UNSUPPORTED",
          4: "BPT_ERR_ALIGN", 5: "BPT_ERR_WORKSPACE", 6: "BPT_ERR_ALIAS", 7: "BPT_ERR_HIP"}
WEIGHT_FIELDS = ("ln1_g", "ln1_b", "w_q", "w_k", "w_v", "w_o", "ln2_g", "ln2_b", "w_1", "w_2")
EXPORTED = ("bpt_layer_workspace_bytes", "bpt_stack_workspace_bytes", "bpt_layer_fwd",
            "bpt_layer_fwd_profiled", "bpt_layer_fwd_lse", "bpt_stack_fwd",
            "bpt_attention_bwd_workspace_bytes", "bpt_attention_bwd",
            "bpt_attention_bwd_profiled", "bpt_attention_fwd_workspace_bytes", "bpt_attention_fwd",
            "bpt_attention_merge", "bpt_layer_host_workspace_bytes", "bpt_layer_fwd_host",
            "bpt_layer_fwd_noalloc", "bpt_layer_bwd_workspace_bytes", "bpt_layer_bwd",
            "bpt_ring_kv_bytes", "bpt_ring_pack_kv", "bpt_ring_share_workspace_bytes",
            "bpt_ring_share_fwd", "bpt_status_str",
            "bpt_last_error", "bpt_version")


class LayerDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seq_len", ctypes.c_int32),
                ("d_model", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("d_ff", ctypes.c_int32), ("block_q", ctypes.c_int32),
                ("block_kv", ctypes.c_int32), ("causal", ctypes.c_int32),
                ("ln_eps", ctypes.c_float), ("dtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32), ("act", ctypes.c_int32),
                ("precision", ctypes.c_int32), ("window", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32)]


class AttnDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seq_len", ctypes.c_int32),
                ("d_model", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("causal", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("window", ctypes.c_int32), ("chunk", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32)]


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in WEIGHT_FIELDS]


class LayerGrads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in WEIGHT_FIELDS]


class BptError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status
        self.detail = detail


_lib = None


def lib() -> ctypes.CDLL:
    """Load the in-tree library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m blockwise_attn_ffn_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        L.bpt_layer_workspace_bytes.argtypes = [P(LayerDesc)]
        L.bpt_layer_workspace_bytes.restype = ctypes.c_size_t
        L.bpt_stack_workspace_bytes.argtypes = [P(LayerDesc), ctypes.c_int32]
        L.bpt_stack_workspace_bytes.restype = ctypes.c_size_t
        L.bpt_layer_fwd.argtypes = [P(LayerDesc), ctypes.c_void_p, P(LayerWeights),
                                    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                    ctypes.c_void_p]
        L.bpt_layer_fwd.restype = ctypes.c_int
        L.bpt_layer_fwd_profiled.argtypes = L.bpt_layer_fwd.argtypes + [P(ctypes.c_void_p)]
        L.bpt_layer_fwd_profiled.restype = ctypes.c_int
        L.bpt_layer_fwd_lse.argtypes = [P(LayerDesc), ctypes.c_void_p, P(LayerWeights),
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_size_t, ctypes.c_void_p]
        L.bpt_layer_fwd_lse.restype = ctypes.c_int
        L.bpt_stack_fwd.argtypes = [P(LayerDesc), ctypes.c_int32, ctypes.c_void_p,
                                    P(LayerWeights), ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_size_t, ctypes.c_void_p]
        L.bpt_stack_fwd.restype = ctypes.c_int
        L.bpt_attention_bwd_workspace_bytes.argtypes = [P(AttnDesc)]
        L.bpt_attention_bwd_workspace_bytes.restype = ctypes.c_size_t
        L.bpt_attention_bwd.argtypes = [P(AttnDesc)] + [ctypes.c_void_p] * 10 + [
            ctypes.c_size_t, ctypes.c_void_p]
        L.bpt_attention_bwd.restype = ctypes.c_int
        L.bpt_attention_bwd_profiled.argtypes = L.bpt_attention_bwd.argtypes + [P(ctypes.c_void_p)]
        L.bpt_attention_bwd_profiled.restype = ctypes.c_int
        L.bpt_attention_fwd_workspace_bytes.argtypes = [P(AttnDesc)]
        L.bpt_attention_fwd_workspace_bytes.restype = ctypes.c_size_t
        L.bpt_attention_fwd.argtypes = [P(AttnDesc)] + [ctypes.c_void_p] * 6 + [ctypes.c_size_t,
                                                                               ctypes.c_void_p]
        L.bpt_attention_fwd.restype = ctypes.c_int
        L.bpt_attention_merge.argtypes = [P(AttnDesc)] + [ctypes.c_void_p] * 5
        L.bpt_attention_merge.restype = ctypes.c_int
        L.bpt_layer_host_workspace_bytes.argtypes = [P(LayerDesc), ctypes.c_int32]
        L.bpt_layer_host_workspace_bytes.restype = ctypes.c_size_t
        L.bpt_layer_fwd_host.argtypes = [P(LayerDesc), ctypes.c_void_p, P(LayerWeights),
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                         ctypes.c_int32]
        L.bpt_layer_fwd_host.restype = ctypes.c_int
        L.bpt_layer_fwd_noalloc.argtypes = [P(LayerDesc), ctypes.c_void_p, P(LayerWeights),
                                            ctypes.c_void_p, ctypes.c_void_p]
        L.bpt_layer_fwd_noalloc.restype = ctypes.c_int
        L.bpt_layer_bwd_workspace_bytes.argtypes = [P(LayerDesc)]
        L.bpt_layer_bwd_workspace_bytes.restype = ctypes.c_size_t
        L.bpt_layer_bwd.argtypes = [P(LayerDesc), ctypes.c_void_p, P(LayerWeights), ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_void_p, P(LayerGrads), ctypes.c_void_p,
                                    ctypes.c_size_t, ctypes.c_void_p]
        L.bpt_layer_bwd.restype = ctypes.c_int
        L.bpt_ring_kv_bytes.argtypes = [P(AttnDesc)]
        L.bpt_ring_kv_bytes.restype = ctypes.c_size_t
        L.bpt_ring_pack_kv.argtypes = [P(AttnDesc)] + [ctypes.c_void_p] * 3 + [ctypes.c_size_t, ctypes.c_void_p]
        L.bpt_ring_pack_kv.restype = ctypes.c_int
        L.bpt_ring_share_workspace_bytes.argtypes = [P(AttnDesc)]
        L.bpt_ring_share_workspace_bytes.restype = ctypes.c_size_t
        L.bpt_ring_share_fwd.argtypes = [P(AttnDesc), ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                         P(ctypes.c_void_p), ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        L.bpt_ring_share_fwd.restype = ctypes.c_int
        L.bpt_status_str.argtypes = [ctypes.c_int]
        L.bpt_status_str.restype = ctypes.c_char_p
        L.bpt_last_error.argtypes = []
        L.bpt_last_error.restype = ctypes.c_char_p
        L.bpt_version.argtypes = []
        L.bpt_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


def make_desc(*, batch, seq_len, d_model, n_heads, d_ff, block_q, block_kv, causal,
              dtype, out_dtype=F32, ln_eps=1e-5, act=0, precision=0, window=0,
              chunk=0, n_kv_heads=0) -> LayerDesc:
    as_code = lambda t: t if isinstance(t, int) else {"f32": F32, "bf16": BF16}[t]  # noqa: E731
    return LayerDesc(batch, seq_len, d_model, n_heads, d_ff, block_q, block_kv, int(causal),
                     ln_eps, as_code(dtype), as_code(out_dtype), act, precision, window, chunk,
                     n_kv_heads)


def desc_for(w, out_dtype=F32) -> LayerDesc:
    """Descriptor of a synth.Workload."""
    return make_desc(batch=w.batch, seq_len=w.seq_len, d_model=w.d_model, n_heads=w.n_heads,
                     d_ff=w.d_ff, block_q=w.block_q, block_kv=w.block_kv, causal=w.causal,
                     dtype=w.dtype, out_dtype=out_dtype, ln_eps=w.ln_eps,
                     precision=getattr(w, "precision", 0), window=getattr(w, "window", 0),
                     chunk=getattr(w, "chunk", 0), n_kv_heads=getattr(w, "n_kv_heads", 0))


def layer_workspace_bytes(desc: LayerDesc) -> int:
    return int(lib().bpt_layer_workspace_bytes(ctypes.byref(desc)))


def stack_workspace_bytes(desc: LayerDesc, n_layers: int) -> int:
    return int(lib().bpt_stack_workspace_bytes(ctypes.byref(desc), n_layers))


def last_error() -> str:
    return lib().bpt_last_error().decode()


def _ptr(t) -> int:
    if t is None:
        return 0
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("device tensors are required")
    if not t.is_contiguous():
        raise ValueError("contiguous tensors are required")
    return t.data_ptr()


def _weights(layer: dict) -> LayerWeights:
    return LayerWeights(*[_ptr(layer[n]) for n in WEIGHT_FIELDS])


def _stream(stream) -> int:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def _check(status: int) -> None:
    if status != 0:
        raise BptError(status, last_error())


def layer_fwd(desc: LayerDesc, x, layer: dict, z, workspace, stream=None) -> None:
    """Enqueue Z = layer(X) on the stream (torch's current stream by default)."""
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().bpt_layer_fwd(ctypes.byref(desc), _ptr(x), ctypes.byref(_weights(layer)),
                               _ptr(z), _ptr(workspace), nbytes, _stream(stream)))


NOALLOC_SCRATCH_BYTES = 64 << 20   # BPT_NOALLOC_SCRATCH_BYTES


def layer_fwd_noalloc(desc: LayerDesc, x, layer: dict, z, stream=None) -> None:
    """bpt_layer_fwd_noalloc: the workspace is the library's fixed device scratch."""
    _check(lib().bpt_layer_fwd_noalloc(ctypes.byref(desc), _ptr(x), ctypes.byref(_weights(layer)),
                                       _ptr(z), _stream(stream)))


def layer_fwd_profiled(desc: LayerDesc, x, layer: dict, z, workspace, events, stream=None) -> None:
    """layer_fwd, recording the five hipEvent_t handles in `events` around its kernels."""
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    arr = (ctypes.c_void_p * 5)(*events)
    _check(lib().bpt_layer_fwd_profiled(ctypes.byref(desc), _ptr(x), ctypes.byref(_weights(layer)),
                                        _ptr(z), _ptr(workspace), nbytes, _stream(stream), arr))


def layer_fwd_lse(desc: LayerDesc, x, layer: dict, z, lse, workspace, stream=None) -> None:
    """layer_fwd that also writes the attention statistic lse [batch, n_heads, seq_len]
    (fp32, natural log of each row's softmax normaliser)."""
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().bpt_layer_fwd_lse(ctypes.byref(desc), _ptr(x), ctypes.byref(_weights(layer)),
                                   _ptr(z), _ptr(lse), _ptr(workspace), nbytes, _stream(stream)))


def layer_bwd_workspace_bytes(desc: LayerDesc) -> int:
    return lib().bpt_layer_bwd_workspace_bytes(ctypes.byref(desc))


def layer_bwd(desc: LayerDesc, x, layer: dict, lse, dz, dx, grads: dict, workspace,
              stream=None) -> None:
    """Enqueue the layer backward: dX and every parameter's gradient (``grads``: fp32
    tensors keyed like the weights, written) from X, the weights, the forward's lse
    and dZ."""
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    g = LayerGrads(*[_ptr(grads[n]) for n in WEIGHT_FIELDS])
    _check(lib().bpt_layer_bwd(ctypes.byref(desc), _ptr(x), ctypes.byref(_weights(layer)), _ptr(lse),
                               _ptr(dz), _ptr(dx), ctypes.byref(g), _ptr(workspace), nbytes,
                               _stream(stream)))


def make_attn_desc(*, batch, seq_len, d_model, n_heads, causal, dtype="bf16", window=0, chunk=0,
                   n_kv_heads=0) -> AttnDesc:
    code = dtype if isinstance(dtype, int) else {"f32": F32, "bf16": BF16}[dtype]
    return AttnDesc(batch, seq_len, d_model, n_heads, int(causal), code, window, chunk, n_kv_heads)


def attention_bwd_workspace_bytes(desc: AttnDesc) -> int:
    return int(lib().bpt_attention_bwd_workspace_bytes(ctypes.byref(desc)))


def attention_bwd(desc: AttnDesc, q, k, v, o, do, lse, dq, dk, dv, workspace, stream=None) -> None:
    """dQ, dK, dV (fp32 [batch * seq_len, d_model]) of the attention given the
    forward's output o, the gradient do and the saved statistic lse."""
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().bpt_attention_bwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                   _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                                   _ptr(workspace), nbytes, _stream(stream)))


def attention_bwd_profiled(desc: AttnDesc, q, k, v, o, do, lse, dq, dk, dv, workspace, events,
                           stream=None) -> None:
    """attention_bwd recording 5 hipEvent_t handles between its kernels."""
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    arr = (ctypes.c_void_p * 5)(*events)
    _check(lib().bpt_attention_bwd_profiled(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                            _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                                            _ptr(workspace), nbytes, _stream(stream), arr))


def attention_fwd_workspace_bytes(desc: AttnDesc) -> int:
    return int(lib().bpt_attention_fwd_workspace_bytes(ctypes.byref(desc)))


def attention_fwd(desc: AttnDesc, q, k, v, o, lse, workspace, stream=None) -> None:
    """One ring step: attention of the query shard q against the key/value shard (k, v)."""
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().bpt_attention_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                   _ptr(workspace), nbytes, _stream(stream)))


def attention_merge(desc: AttnDesc, o_acc, lse_acc, o_part, lse_part, stream=None) -> None:
    """Fold one ring step's (o_part, lse_part) into the running (o_acc, lse_acc)."""
    _check(lib().bpt_attention_merge(ctypes.byref(desc), _ptr(o_acc), _ptr(lse_acc), _ptr(o_part),
                                     _ptr(lse_part), _stream(stream)))


def ring_kv_bytes(desc: AttnDesc) -> int:
    return lib().bpt_ring_kv_bytes(ctypes.byref(desc))


def ring_pack_kv(desc: AttnDesc, k, v, kv, stream=None) -> None:
    """Pack one key/value shard into the attention kernels' layout (kv: a device
    buffer of ring_kv_bytes)."""
    nbytes = kv.numel() * kv.element_size()
    _check(lib().bpt_ring_pack_kv(ctypes.byref(desc), _ptr(k), _ptr(v), _ptr(kv), nbytes, _stream(stream)))


def ring_share_workspace_bytes(desc: AttnDesc) -> int:
    return lib().bpt_ring_share_workspace_bytes(ctypes.byref(desc))


def ring_share_fwd(desc: AttnDesc, own: int, q, kv_shards: list, o, lse, workspace, stream=None) -> None:
    """One device's share of Ring Attention: q against the packed shards (a list of
    device buffers or None for shards the causal mask never reaches)."""
    n = len(kv_shards)
    arr = (ctypes.c_void_p * n)(*[_ptr(t) if t is not None else 0 for t in kv_shards])
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib().bpt_ring_share_fwd(ctypes.byref(desc), n, own, _ptr(q), arr, _ptr(o), _ptr(lse),
                                    _ptr(workspace), nbytes, _stream(stream)))


def layer_host_workspace_bytes(desc: LayerDesc, n_threads: int) -> int:
    return int(lib().bpt_layer_host_workspace_bytes(ctypes.byref(desc), n_threads))


def _hptr(t) -> int:
    if t is None:
        return 0
    if t.is_cuda:
        raise ValueError("host tensors are required")
    if not t.is_contiguous():
        raise ValueError("contiguous tensors are required")
    return t.data_ptr()


def layer_fwd_host(desc: LayerDesc, x, layer: dict, z, workspace, n_threads: int) -> None:
    """The host (CPU) fused layer on CPU tensors (synchronous)."""
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    w = LayerWeights(*[_hptr(layer[n]) for n in WEIGHT_FIELDS])
    _check(lib().bpt_layer_fwd_host(ctypes.byref(desc), _hptr(x), ctypes.byref(w), _hptr(z),
                                    _hptr(workspace), nbytes, n_threads))


def stack_fwd(desc: LayerDesc, x, layers: list, z, workspace, stream=None) -> None:
    """Enqueue Z = layer_{L-1}(... layer_0(X)) on the stream."""
    arr = (LayerWeights * len(layers))(*[_weights(l) for l in layers])
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().bpt_stack_fwd(ctypes.byref(desc), len(layers), _ptr(x), arr, _ptr(z),
                               _ptr(workspace), nbytes, _stream(stream)))


def alloc_workspace(nbytes: int, device="cuda"):
    """A uint8 device tensor of nbytes (at least 1 byte), for the workspace argument."""
    import torch
    return torch.empty(max(1, nbytes), dtype=torch.uint8, device=device)
