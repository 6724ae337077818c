"""ctypes binding of libpeagle.so (argument marshalling only).

Every step of the parallel-draft round runs in the HIP library; this module
only turns torch tensors into device pointers and sizes, allocates outputs
with torch (device memory plumbing), and maps status codes to exceptions.
There is no fallback: if the library is missing, loading fails loudly.
"""

from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpeagle.so")

PE_OK, PE_EINVAL, PE_EUNSUPPORTED, PE_EWORKSPACE, PE_EHIP = 0, -1, -2, -3, -4
PE_F32, PE_BF16 = 0, 1
PE_KERNEL_LM_HEAD, PE_KERNEL_PREPARE, PE_KERNEL_ATTENTION = 0, 1, 2

EXPORTED = ("pe_model_create", "pe_model_destroy", "pe_workspace_bytes", "pe_prepare_draft_batch",
            "pe_draft_forward", "pe_accept", "pe_status_string", "pe_timing_enable", "pe_timing_read",
            "pe_autoregressive_workspace_bytes", "pe_draft_autoregressive", "pe_next_verified_batch",
            "pe_prepare_draft_batch_compact", "pe_packed_weights_bytes", "pe_model_pack_weights",
            "pe_check_verified_batch", "pe_draft_forward_noalloc")

STATIC_SCRATCH_BYTES = 32 << 20  # PE_STATIC_SCRATCH_BYTES


class PeError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)} (status {status})")
        self.status = status


class ModelDesc(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("vocab", ctypes.c_int32), ("n_layers", ctypes.c_int32),
                ("n_q", ctypes.c_int32), ("n_kv", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("inter", ctypes.c_int32), ("block_size", ctypes.c_int32), ("rms_eps", ctypes.c_float),
                ("rope_theta", ctypes.c_float), ("mask_token_id", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("ln1", "wq", "wk", "wv", "wo", "ln2", "w_gate", "w_up", "w_down")]


class Weights(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("w_fc", ctypes.c_void_p), ("ln_f", ctypes.c_void_p),
                ("w_lm", ctypes.c_void_p), ("h_shared", ctypes.c_void_p),
                ("layers", ctypes.POINTER(LayerWeights))]


_lib: Optional[ctypes.CDLL] = None


def load() -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m drafting_draft_expand_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.pe_model_create.argtypes = [ctypes.POINTER(ModelDesc), ctypes.POINTER(Weights), ctypes.POINTER(P)]
    lib.pe_model_create.restype = I32
    lib.pe_check_verified_batch.argtypes = [P, I32, I32, I32] + [P] * 6 + [I32, P, P]
    lib.pe_check_verified_batch.restype = I32
    lib.pe_packed_weights_bytes.argtypes = [P]
    lib.pe_packed_weights_bytes.restype = SZ
    lib.pe_model_pack_weights.argtypes = [P, P, SZ, P]
    lib.pe_model_pack_weights.restype = I32
    lib.pe_model_destroy.argtypes = [P]
    lib.pe_model_destroy.restype = None
    lib.pe_workspace_bytes.argtypes = [P, I32, I32, I32]
    lib.pe_workspace_bytes.restype = SZ
    lib.pe_prepare_draft_batch.argtypes = [P, I32, I32, I32] + [P] * 7 + [I32] + [P] * 10 + [P]
    lib.pe_prepare_draft_batch.restype = I32
    lib.pe_prepare_draft_batch_compact.argtypes = lib.pe_prepare_draft_batch.argtypes
    lib.pe_prepare_draft_batch_compact.restype = I32
    lib.pe_draft_forward.argtypes = [P, I32, I32, I32] + [P] * 9 + [I32] + [P, P, P, SZ] + [P, P, P] + [P]
    lib.pe_draft_forward.restype = I32
    lib.pe_draft_forward_noalloc.argtypes = [P, I32, I32, I32] + [P] * 9 + [I32] + [P, P] + [P, P, P] + [P]
    lib.pe_draft_forward_noalloc.restype = I32
    lib.pe_accept.argtypes = [I32, I32, P, P, P, P, P]
    lib.pe_accept.restype = I32
    lib.pe_status_string.argtypes = [I32]
    lib.pe_status_string.restype = ctypes.c_char_p
    lib.pe_timing_enable.argtypes = [I32, I32]
    lib.pe_timing_enable.restype = I32
    lib.pe_timing_read.argtypes = [I32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(I64), P, I64]
    lib.pe_timing_read.restype = I32
    lib.pe_autoregressive_workspace_bytes.argtypes = [P, I32, I32, I32]
    lib.pe_autoregressive_workspace_bytes.restype = SZ
    lib.pe_draft_autoregressive.argtypes = [P, I32, I32, I32] + [P] * 7 + [I32] + [P, P, P, SZ, P, P, P, P]
    lib.pe_draft_autoregressive.restype = I32
    lib.pe_next_verified_batch.argtypes = [I32, I32] + [P] * 10 + [P]
    lib.pe_next_verified_batch.restype = I32
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().pe_status_string(status).decode()


def _check(status: int, where: str) -> None:
    if status != PE_OK:
        raise PeError(status, where)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dtype_code(dtype: str) -> int:
    return {"fp32": PE_F32, "bf16": PE_BF16}[dtype]


class DraftModel:
    """A drafter handle: shape description + borrowed device weights, plus (for
    bf16 drafters, unless ``pack=False``) the packed copy of the projection
    weights that pe_model_pack_weights fills."""

    def __init__(self, hidden: int, vocab: int, n_layers: int, n_q: int, n_kv: int, head_dim: int,
                 inter: int, dtype: str, weights: Dict, block_size: int = 16, rms_eps: float = 1e-6,
                 rope_theta: float = 10000.0, mask_token_id: Optional[int] = None, pack: bool = True):
        lib = load()
        self.dtype = dtype
        self.torch_dtype = torch.float32 if dtype == "fp32" else torch.bfloat16
        self.desc = ModelDesc(hidden, vocab, n_layers, n_q, n_kv, head_dim, inter, block_size, rms_eps,
                              rope_theta, vocab - 1 if mask_token_id is None else mask_token_id,
                              _dtype_code(dtype))
        self._keep = weights  # keep device tensors alive for the handle's lifetime
        layers = weights.get("layers", [])
        self._layers = (LayerWeights * max(1, len(layers)))()
        for i, lw in enumerate(layers):
            self._layers[i] = LayerWeights(*[_ptr(lw[n]) for n, _ in LayerWeights._fields_])
        g = lambda n: _ptr(weights[n]) if n in weights else None  # noqa: E731
        self._w = Weights(g("embed"), g("w_fc"), g("ln_f"), g("w_lm"), g("h_shared"),
                          ctypes.cast(self._layers, ctypes.POINTER(LayerWeights)) if layers else None)
        h = ctypes.c_void_p()
        _check(lib.pe_model_create(ctypes.byref(self.desc), ctypes.byref(self._w), ctypes.byref(h)),
               "pe_model_create")
        self.handle = h
        self.packed = None
        nbytes = int(lib.pe_packed_weights_bytes(h))
        if pack and nbytes > 0:
            dev = next(t.device for t in weights.values() if isinstance(t, torch.Tensor))
            self.packed = torch.empty(nbytes, dtype=torch.uint8, device=dev)
            _check(lib.pe_model_pack_weights(h, _ptr(self.packed), nbytes, _stream(None)), "pe_model_pack_weights")

    @classmethod
    def from_spec(cls, spec, weights: Dict, pack: bool = True) -> "DraftModel":
        return cls(spec.hidden, spec.vocab, spec.n_layers, spec.n_q, spec.n_kv, spec.head_dim, spec.inter,
                   spec.dtype, weights, spec.block_size, spec.rms_eps, spec.rope_theta, spec.mask_token_id, pack)

    def workspace_bytes(self, num_seqs: int, K: int, num_rows: int) -> int:
        return int(load().pe_workspace_bytes(self.handle, num_seqs, K, num_rows))

    def autoregressive_workspace_bytes(self, num_seqs: int, K: int, total_target_rows: int) -> int:
        return int(load().pe_autoregressive_workspace_bytes(self.handle, num_seqs, K, total_target_rows))

    def close(self) -> None:
        if getattr(self, "handle", None):
            load().pe_model_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def timing_enable(kernel: int, enable: bool = True) -> None:
    """Start (or stop) recording launch times of a kernel class (see pe_timing_enable)."""
    _check(load().pe_timing_enable(kernel, int(enable)), "pe_timing_enable")


def timing_read(kernel: int):
    """(total ms, launches, per-launch ms list) recorded since timing_enable (see pe_timing_read)."""
    lib = load()
    ms, n = ctypes.c_double(), ctypes.c_int64()
    _check(lib.pe_timing_read(kernel, ctypes.byref(ms), ctypes.byref(n), None, 0), "pe_timing_read")
    per = (ctypes.c_float * max(1, n.value))()
    _check(lib.pe_timing_read(kernel, ctypes.byref(ms), ctypes.byref(n), ctypes.cast(per, ctypes.c_void_p),
                              n.value), "pe_timing_read")
    return ms.value, n.value, list(per[:n.value])


def prepare_draft_batch(model: DraftModel, K: int, query_lens: torch.Tensor, target_ids: torch.Tensor,
                        target_pos: torch.Tensor, num_accepted: torch.Tensor, bonus_ids: torch.Tensor,
                        target_hidden: torch.Tensor, block_table: torch.Tensor,
                        out: Optional[Dict[str, torch.Tensor]] = None, stream=None,
                        compact: bool = False) -> Dict[str, torch.Tensor]:
    """Expand the verified batch (see pe_prepare_draft_batch; compact=True:
    pe_prepare_draft_batch_compact).  Returns the draft batch tensors."""
    c = int(query_lens.numel())
    T = int(target_ids.numel())
    N = T + c * (K - 1)
    dev = target_ids.device
    if out is None:
        i32 = dict(dtype=torch.int32, device=dev)
        out = dict(draft_ids=torch.empty(N, **i32), draft_pos=torch.empty(N, **i32),
                   slot_mapping=torch.empty(N, dtype=torch.int64, device=dev),
                   is_rejected=torch.empty(N, dtype=torch.uint8, device=dev),
                   is_masked=torch.empty(N, dtype=torch.uint8, device=dev),
                   hidden_map=torch.empty(T, **i32), cu_draft=torch.empty(c + 1, **i32),
                   kv_lens=torch.empty(c, **i32), sample_idx=torch.empty(c * K, **i32),
                   draft_hidden=torch.empty((N, target_hidden.shape[1]), dtype=target_hidden.dtype, device=dev))
    fn = load().pe_prepare_draft_batch_compact if compact else load().pe_prepare_draft_batch
    st = fn(
        model.handle, c, K, T, _ptr(query_lens), _ptr(target_ids), _ptr(target_pos), _ptr(num_accepted),
        _ptr(bonus_ids), _ptr(target_hidden), _ptr(block_table), int(block_table.shape[1]),
        _ptr(out["draft_ids"]), _ptr(out["draft_pos"]), _ptr(out["slot_mapping"]), _ptr(out["is_rejected"]),
        _ptr(out["is_masked"]), _ptr(out["hidden_map"]), _ptr(out["cu_draft"]), _ptr(out["kv_lens"]),
        _ptr(out["sample_idx"]), _ptr(out["draft_hidden"]), _stream(stream))
    _check(st, "pe_prepare_draft_batch_compact" if compact else "pe_prepare_draft_batch")
    out["num_seqs"], out["K"], out["num_rows"] = c, K, N
    return out


def draft_forward(model: DraftModel, batch: Dict[str, torch.Tensor], block_table: torch.Tensor,
                  k_cache: Sequence[torch.Tensor], v_cache: Sequence[torch.Tensor],
                  workspace: Optional[torch.Tensor] = None, tokens: Optional[torch.Tensor] = None,
                  logits: Optional[torch.Tensor] = None, top2_gap: Optional[torch.Tensor] = None,
                  stream=None) -> torch.Tensor:
    """One drafter pass (see pe_draft_forward).  Returns draft tokens [c, K] (int32)."""
    c, K, N = batch["num_seqs"], batch["K"], batch["num_rows"]
    dev = batch["draft_ids"].device
    if workspace is None:
        workspace = torch.empty(model.workspace_bytes(c, K, N), dtype=torch.uint8, device=dev)
    if tokens is None:
        tokens = torch.empty((c, K), dtype=torch.int32, device=dev)
    kp = (ctypes.c_void_p * len(k_cache))(*[_ptr(t) for t in k_cache])
    vp = (ctypes.c_void_p * len(v_cache))(*[_ptr(t) for t in v_cache])
    st = load().pe_draft_forward(
        model.handle, c, K, N, _ptr(batch["draft_ids"]), _ptr(batch["draft_pos"]), _ptr(batch["slot_mapping"]),
        _ptr(batch["is_rejected"]), _ptr(batch["cu_draft"]), _ptr(batch["kv_lens"]), _ptr(batch["sample_idx"]),
        _ptr(batch["draft_hidden"]), _ptr(block_table), int(block_table.shape[1]),
        ctypes.cast(kp, ctypes.c_void_p), ctypes.cast(vp, ctypes.c_void_p), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(tokens), _ptr(logits), _ptr(top2_gap), _stream(stream))
    _check(st, "pe_draft_forward")
    return tokens


def draft_forward_noalloc(model: DraftModel, batch: Dict[str, torch.Tensor], block_table: torch.Tensor,
                          k_cache: Sequence[torch.Tensor], v_cache: Sequence[torch.Tensor],
                          tokens: torch.Tensor, logits: Optional[torch.Tensor] = None,
                          top2_gap: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """One drafter pass on the library's static scratch (see pe_draft_forward_noalloc): no workspace,
    nothing allocated here or in the library; the caller passes every output.  Returns ``tokens``."""
    c, K, N = batch["num_seqs"], batch["K"], batch["num_rows"]
    kp = (ctypes.c_void_p * len(k_cache))(*[_ptr(t) for t in k_cache])
    vp = (ctypes.c_void_p * len(v_cache))(*[_ptr(t) for t in v_cache])
    st = load().pe_draft_forward_noalloc(
        model.handle, c, K, N, _ptr(batch["draft_ids"]), _ptr(batch["draft_pos"]), _ptr(batch["slot_mapping"]),
        _ptr(batch["is_rejected"]), _ptr(batch["cu_draft"]), _ptr(batch["kv_lens"]), _ptr(batch["sample_idx"]),
        _ptr(batch["draft_hidden"]), _ptr(block_table), int(block_table.shape[1]),
        ctypes.cast(kp, ctypes.c_void_p), ctypes.cast(vp, ctypes.c_void_p), _ptr(tokens), _ptr(logits),
        _ptr(top2_gap), _stream(stream))
    _check(st, "pe_draft_forward_noalloc")
    return tokens


def accept(draft_tokens: torch.Tensor, target_tokens: torch.Tensor, num_accepted: Optional[torch.Tensor] = None,
           bonus_ids: Optional[torch.Tensor] = None, stream=None):
    """Greedy acceptance (see pe_accept).  Returns (num_accepted [c], bonus_ids [c]) int32."""
    c, K = draft_tokens.shape
    dev = draft_tokens.device
    if num_accepted is None:
        num_accepted = torch.empty(c, dtype=torch.int32, device=dev)
    if bonus_ids is None:
        bonus_ids = torch.empty(c, dtype=torch.int32, device=dev)
    st = load().pe_accept(c, K, _ptr(draft_tokens), _ptr(target_tokens), _ptr(num_accepted), _ptr(bonus_ids),
                          _stream(stream))
    _check(st, "pe_accept")
    return num_accepted, bonus_ids


def draft_autoregressive(model: DraftModel, K: int, query_lens: torch.Tensor, target_ids: torch.Tensor,
                         target_pos: torch.Tensor, num_accepted: torch.Tensor, bonus_ids: torch.Tensor,
                         target_hidden: torch.Tensor, block_table: torch.Tensor, k_cache: Sequence[torch.Tensor],
                         v_cache: Sequence[torch.Tensor], workspace: Optional[torch.Tensor] = None,
                         tokens: Optional[torch.Tensor] = None, logits: Optional[torch.Tensor] = None,
                         fed_hidden: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """K sequential one-token drafter passes (see pe_draft_autoregressive).  Returns tokens [c, K] (int32);
    ``logits`` (optional float32 [K, c, V]) receives each pass's logits, ``fed_hidden`` (optional
    [K-1, c, H], model dtype) the hidden input of passes 1..K-1."""
    c = int(query_lens.numel())
    T = int(target_ids.numel())
    dev = target_ids.device
    if workspace is None:
        workspace = torch.empty(model.autoregressive_workspace_bytes(c, K, T), dtype=torch.uint8, device=dev)
    if tokens is None:
        tokens = torch.empty((c, K), dtype=torch.int32, device=dev)
    kp = (ctypes.c_void_p * len(k_cache))(*[_ptr(t) for t in k_cache])
    vp = (ctypes.c_void_p * len(v_cache))(*[_ptr(t) for t in v_cache])
    st = load().pe_draft_autoregressive(
        model.handle, c, K, T, _ptr(query_lens), _ptr(target_ids), _ptr(target_pos), _ptr(num_accepted),
        _ptr(bonus_ids), _ptr(target_hidden), _ptr(block_table), int(block_table.shape[1]),
        ctypes.cast(kp, ctypes.c_void_p), ctypes.cast(vp, ctypes.c_void_p), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(tokens), _ptr(logits), _ptr(fed_hidden),
        _stream(stream))
    _check(st, "pe_draft_autoregressive")
    return tokens


PE_CHECK_QUERY_LEN, PE_CHECK_ACCEPTED, PE_CHECK_TOKEN_ID, PE_CHECK_POSITION, PE_CHECK_BLOCK_TABLE = 1, 2, 4, 8, 16


def check_verified_batch(model: DraftModel, K: int, query_lens: torch.Tensor, target_ids: torch.Tensor,
                         target_pos: torch.Tensor, num_accepted: torch.Tensor, bonus_ids: torch.Tensor,
                         block_table: torch.Tensor, error_bits: Optional[torch.Tensor] = None,
                         stream=None) -> torch.Tensor:
    """Device check of the verified batch (see pe_check_verified_batch).
    Returns the int32 [1] device word of PE_CHECK_* bits (zeroed here when not
    given, accumulated into when given)."""
    c = int(query_lens.numel())
    if error_bits is None:
        error_bits = torch.zeros(1, dtype=torch.int32, device=query_lens.device)
    st = load().pe_check_verified_batch(
        model.handle, c, K, int(target_ids.numel()), _ptr(query_lens), _ptr(target_ids), _ptr(target_pos),
        _ptr(num_accepted), _ptr(bonus_ids), _ptr(block_table), int(block_table.shape[1]), _ptr(error_bits),
        _stream(stream))
    _check(st, "pe_check_verified_batch")
    return error_bits


def next_verified_batch(K: int, kv_lens: torch.Tensor, bonus_ids: torch.Tensor, draft_tokens: torch.Tensor,
                        num_accepted_next: torch.Tensor, bonus_next: torch.Tensor,
                        out: Optional[Dict[str, torch.Tensor]] = None, stream=None) -> Dict[str, torch.Tensor]:
    """Next round's verified batch metadata (see pe_next_verified_batch)."""
    c = int(kv_lens.numel())
    dev = kv_lens.device
    if out is None:
        i32 = dict(dtype=torch.int32, device=dev)
        out = dict(query_lens=torch.empty(c, **i32), target_ids=torch.empty(c * (K + 1), **i32),
                   target_pos=torch.empty(c * (K + 1), **i32), num_accepted=torch.empty(c, **i32),
                   bonus_ids=torch.empty(c, **i32))
    st = load().pe_next_verified_batch(
        c, K, _ptr(kv_lens), _ptr(bonus_ids), _ptr(draft_tokens), _ptr(num_accepted_next), _ptr(bonus_next),
        _ptr(out["query_lens"]), _ptr(out["target_ids"]), _ptr(out["target_pos"]), _ptr(out["num_accepted"]),
        _ptr(out["bonus_ids"]), _stream(stream))
    _check(st, "pe_next_verified_batch")
    return out
