"""Thin Python binding of the decoder library: torch allocates device memory
and supplies the stream; every computation runs in libsdm.so's kernels.

Method names follow the C ABI (include/sdm.h): ``prefill``, ``diffuse_step``,
``draft_block``, ``verify_block``, ``commit_kv``, ``decode_ar``.
"""
from __future__ import annotations

import ctypes
from ctypes import POINTER, c_int32, c_void_p
from typing import Dict, Optional, Sequence

import numpy as np
import torch

from . import _lib as L


def _dev_tensor(a: np.ndarray, device) -> torch.Tensor:
    """numpy (float32, or uint16 bf16 bits) -> device tensor of the same bytes."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a.astype(np.float32, copy=False)).to(device)


def make_config(shape, max_seqs=1, max_block=32, max_context=4096, max_rows=32,
                weight_format=L.SDM_WEIGHTS_BF16) -> L.SdmConfig:
    return L.SdmConfig(shape.n_layers, shape.d_model, shape.n_q_heads, shape.n_kv_heads, shape.head_dim,
                       shape.ffn_dim, shape.vocab, shape.mask_id, shape.rope_base, shape.rms_eps,
                       L.SDM_BF16 if shape.dtype == "bf16" else L.SDM_F32, 64, max_seqs, max_block, max_context,
                       max_rows, weight_format)


class Model:
    """A decoder on one GPU.  ``weights`` is a dict as produced by
    ``workloads.make_weights`` or ``workloads.make_w4_weights`` (host numpy
    arrays; 4-bit decoder matrices are recognised by their ``.codes``
    entries); they are uploaded and packed into the library's layout once."""

    def __init__(self, shape, weights: Dict[str, np.ndarray], *, max_seqs: int = 1, max_block: int = 32,
                 max_context: int = 4096, max_rows: int = 32, n_pages: Optional[int] = None,
                 device: str = "cuda", free_host: bool = False):
        self.lib = L.lib()
        self.shape = shape
        self.device = torch.device(device)
        self.w4 = "layers.0.w_qkv.codes" in weights
        self.cfg = make_config(shape, max_seqs, max_block, max_context, max_rows,
                               L.SDM_WEIGHTS_INT4 if self.w4 else L.SDM_WEIGHTS_BF16)
        self.stream = torch.cuda.current_stream(self.device)
        st = c_void_p(self.stream.cuda_stream)
        cfgp = ctypes.byref(self.cfg)
        self._keep = []

        def packed(kind, rows, cols, src, src2=None):
            nbytes = self.lib.sdm_packed_bytes(cfgp, rows * (2 if kind == L.SDM_PACK_GATE_UP else 1), cols)
            dst = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
            L.check(self.lib.sdm_pack_matrix(cfgp, kind, L.ptr(src), L.ptr(src2), L.ptr(dst), rows, cols, st))
            self._keep.append(dst)
            return dst

        def packed_int4(kind, rows, cols, name, name2=None):
            """Upload <name>.codes / .scales (and name2's for gate/up), pack them."""
            srcs = []
            for n in (name, name2):
                if n is None:
                    srcs += [None, None]
                    continue
                c = torch.from_numpy(np.ascontiguousarray(weights[n + ".codes"])).to(self.device)
                sc = torch.from_numpy(np.ascontiguousarray(weights[n + ".scales"]).view(np.int16)).to(self.device)
                srcs += [c, sc]
                if free_host:
                    weights.pop(n + ".codes")
                    weights.pop(n + ".scales")
            nbytes = self.lib.sdm_packed_bytes_int4(cfgp, rows * (2 if kind == L.SDM_PACK_GATE_UP else 1), cols)
            if nbytes == 0:
                raise L.SdmError(L.SDM_ERR_UNSUPPORTED, f"4-bit matrix {name} [{rows}, {cols}]")
            dst = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
            L.check(self.lib.sdm_pack_matrix_int4(cfgp, kind, *[L.ptr(x) for x in srcs], L.ptr(dst), rows, cols, st))
            self._keep.append(dst)
            return dst

        def plain(name):
            t = _dev_tensor(weights[name], self.device)
            self._keep.append(t)
            if free_host:
                weights.pop(name)
            return t

        def upload(name):
            t = _dev_tensor(weights[name], self.device)
            if free_host:
                weights.pop(name)
            return t

        s = shape
        embed = plain("embed")
        final_norm = plain("final_norm")
        lm = upload("lm_head")
        lm_p = packed(L.SDM_PACK_PLAIN, s.vocab, s.d_model, lm)
        del lm
        per = {k: [] for k in ("attn_norm", "w_qkv", "w_o", "ffn_norm", "w_gate_up", "w_down")}
        for l in range(s.n_layers):
            p = f"layers.{l}."
            per["attn_norm"].append(plain(p + "attn_norm"))
            per["ffn_norm"].append(plain(p + "ffn_norm"))
            if self.w4:
                per["w_qkv"].append(packed_int4(L.SDM_PACK_QKV, s.qkv_dim, s.d_model, p + "w_qkv"))
                per["w_o"].append(packed_int4(L.SDM_PACK_PLAIN, s.d_model, s.q_dim, p + "w_o"))
                per["w_gate_up"].append(packed_int4(L.SDM_PACK_GATE_UP, s.ffn_dim, s.d_model, p + "w_gate",
                                                    p + "w_up"))
                per["w_down"].append(packed_int4(L.SDM_PACK_PLAIN, s.d_model, s.ffn_dim, p + "w_down"))
                continue
            t = upload(p + "w_qkv")
            per["w_qkv"].append(packed(L.SDM_PACK_QKV, s.qkv_dim, s.d_model, t))
            t = upload(p + "w_o")
            per["w_o"].append(packed(L.SDM_PACK_PLAIN, s.d_model, s.q_dim, t))
            g, u = upload(p + "w_gate"), upload(p + "w_up")
            per["w_gate_up"].append(packed(L.SDM_PACK_GATE_UP, s.ffn_dim, s.d_model, g, u))
            t = upload(p + "w_down")
            per["w_down"].append(packed(L.SDM_PACK_PLAIN, s.d_model, s.ffn_dim, t))
            del t, g, u
        arr = lambda lst: (c_void_p * len(lst))(*[L.ptr(x) for x in lst])
        self._arrays = {k: arr(v) for k, v in per.items()}
        self.weights_c = L.SdmWeights(L.ptr(embed), L.ptr(final_norm), L.ptr(lm_p),
                                      *[ctypes.cast(self._arrays[k], POINTER(c_void_p)) for k in
                                        ("attn_norm", "w_qkv", "w_o", "ffn_norm", "w_gate_up", "w_down")])
        if n_pages is None:
            n_pages = max_seqs * ((max_context + 63) // 64)
        self.n_pages = n_pages
        self.page_bytes = self.lib.sdm_kv_page_bytes(cfgp)
        self.kv_pool = torch.empty(n_pages * self.page_bytes, dtype=torch.uint8, device=self.device)
        self.ws_bytes = self.lib.sdm_workspace_bytes(cfgp)
        if self.ws_bytes == 0:
            raise L.SdmError(L.SDM_ERR_ARG, self.lib.sdm_last_error().decode())
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)
        h = c_void_p()
        L.check(self.lib.sdm_init_model(cfgp, ctypes.byref(self.weights_c), L.ptr(self.kv_pool), n_pages,
                                        L.ptr(self.workspace), self.ws_bytes, st, ctypes.byref(h)))
        self.handle = h
        self.weight_bytes = sum(t.numel() * t.element_size() for t in self._keep)

    # -- the C-ABI calls -----------------------------------------------------
    def prefill(self, seq: int, tokens: torch.Tensor, next_token: torch.Tensor, logits: torch.Tensor = None):
        L.check(self.lib.sdm_prefill(self.handle, seq, L.ptr(tokens), tokens.numel(), L.ptr(next_token),
                                     L.ptr(logits)))

    def diffuse_step(self, seq_ids: Sequence[int], block: torch.Tensor, B: int, tau: float, force_all: bool,
                     n_masked: torch.Tensor, conf: torch.Tensor = None, logits: torch.Tensor = None):
        ids = (c_int32 * len(seq_ids))(*seq_ids)
        L.check(self.lib.sdm_diffuse_step(self.handle, len(seq_ids), ids, L.ptr(block), B, float(tau),
                                          int(bool(force_all)), L.ptr(n_masked), L.ptr(conf), L.ptr(logits)))

    def diffuse_step_revise(self, seq_ids: Sequence[int], block: torch.Tensor, B: int, tau: float, tau_revise: float,
                            force_all: bool, n_masked: torch.Tensor, n_revised: torch.Tensor = None,
                            conf: torch.Tensor = None, logits: torch.Tensor = None):
        ids = (c_int32 * len(seq_ids))(*seq_ids)
        L.check(self.lib.sdm_diffuse_step_revise(self.handle, len(seq_ids), ids, L.ptr(block), B, float(tau),
                                                 float(tau_revise), int(bool(force_all)), L.ptr(n_masked),
                                                 L.ptr(n_revised), L.ptr(conf), L.ptr(logits)))

    def draft_block(self, seq: int, anchor: int | torch.Tensor, B: int, block_out: torch.Tensor,
                    logits: torch.Tensor = None):
        L.check(self.lib.sdm_draft_block(self.handle, seq, self._addr(anchor), B, L.ptr(block_out), L.ptr(logits)))

    def verify_block(self, seq_ids: Sequence[int], block: torch.Tensor, B: int, ar_argmax: torch.Tensor,
                     accept_len: torch.Tensor, logits: torch.Tensor = None):
        ids = (c_int32 * len(seq_ids))(*seq_ids)
        L.check(self.lib.sdm_verify_block(self.handle, len(seq_ids), ids, self._addr(block), B, L.ptr(ar_argmax),
                                          L.ptr(accept_len), L.ptr(logits)))

    def verify_block_quadratic(self, seq: int, block: int | torch.Tensor, B: int, ar_argmax: torch.Tensor,
                               accept_len: torch.Tensor, next_blocks: torch.Tensor, logits: torch.Tensor = None):
        L.check(self.lib.sdm_verify_block_quadratic(self.handle, seq, self._addr(block), B, L.ptr(ar_argmax),
                                                    L.ptr(accept_len), L.ptr(next_blocks), L.ptr(logits)))

    def commit_kv(self, seq: int, n_accept: int):
        L.check(self.lib.sdm_commit_kv(self.handle, seq, int(n_accept)))

    def decode_ar(self, seq: int, token: int | torch.Tensor, next_token: int | torch.Tensor,
                  logits: torch.Tensor = None):
        L.check(self.lib.sdm_decode_ar(self.handle, seq, self._addr(token), self._addr(next_token), L.ptr(logits)))

    # -- sampling at temperature > 0 ----------------------------------------------
    def prefill_sample(self, seq: int, tokens: torch.Tensor, T: float, seed: int, next_token: torch.Tensor,
                       logits: torch.Tensor = None):
        L.check(self.lib.sdm_prefill_sample(self.handle, seq, L.ptr(tokens), tokens.numel(), float(T), int(seed),
                                            L.ptr(next_token), L.ptr(logits)))

    def decode_ar_sample(self, seq: int, token: int | torch.Tensor, T: float, seed: int,
                         next_token: int | torch.Tensor, logits: torch.Tensor = None):
        L.check(self.lib.sdm_decode_ar_sample(self.handle, seq, self._addr(token), float(T), int(seed),
                                              self._addr(next_token), L.ptr(logits)))

    def draft_block_sample(self, seq: int, anchor: int | torch.Tensor, B: int, T: float, seed: int,
                           block_out: torch.Tensor, draft_logits: torch.Tensor, draft_stats: torch.Tensor):
        L.check(self.lib.sdm_draft_block_sample(self.handle, seq, self._addr(anchor), B, float(T), int(seed),
                                                L.ptr(block_out), L.ptr(draft_logits), L.ptr(draft_stats)))

    def verify_block_sample(self, seq: int, block: torch.Tensor, B: int, T: float, seed: int,
                            draft_logits: torch.Tensor, draft_stats: torch.Tensor, accept_len: torch.Tensor,
                            next_token: int | torch.Tensor, logits: torch.Tensor = None):
        L.check(self.lib.sdm_verify_block_sample(self.handle, seq, L.ptr(block), B, float(T), int(seed),
                                                 L.ptr(draft_logits), L.ptr(draft_stats), L.ptr(accept_len),
                                                 self._addr(next_token), L.ptr(logits)))

    def row_stats(self, tok=None, conf=None, margin=None):
        L.check(self.lib.sdm_row_stats(self.handle, L.ptr(tok), L.ptr(conf), L.ptr(margin)))

    def seq_reset(self, seq: int):
        L.check(self.lib.sdm_seq_reset(self.handle, seq))

    def seq_length(self, seq: int) -> int:
        out = c_int32()
        L.check(self.lib.sdm_seq_length(self.handle, seq, ctypes.byref(out)))
        return out.value

    def free_pages(self) -> int:
        return self.lib.sdm_free_pages(self.handle)

    def shuffle_free_pages(self, seed: int):
        L.check(self.lib.sdm_shuffle_free_pages(self.handle, seed))

    def timing_start(self, kernel_class: str, capacity: int = 1 << 16):
        L.check(self.lib.sdm_timing_start(self.handle, L.KERNEL_CLASSES[kernel_class], capacity))

    def timing_stop(self):
        """-> (launches, total_ms, min_ms, max_ms) of the timed kernel class."""
        n, tot, mn, mx = ctypes.c_int64(), ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
        L.check(self.lib.sdm_timing_stop(self.handle, ctypes.byref(n), ctypes.byref(tot), ctypes.byref(mn),
                                         ctypes.byref(mx)))
        return n.value, tot.value, mn.value, mx.value

    def close(self):
        if getattr(self, "handle", None):
            self.lib.sdm_free_model(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @staticmethod
    def _addr(x) -> int:
        """A device tensor, or a raw device address (an element inside a tensor)."""
        return x if isinstance(x, int) else x.data_ptr()
