"""Device buffers for one block-diffusion step, and the calls that run it.

``DeviceStep`` uploads a host-side step (numpy arrays in the layouts of
include/bd.h) to HBM once, sizes and zero-fills the workspaces, and exposes
the library calls on those buffers.  torch supplies device memory and the
stream; the arithmetic runs in libbd.so.

With ``guard_bytes > 0`` every buffer the library writes (outputs, block
state, caches, prefix lengths, workspaces) sits between two bands of canary
bytes, and outputs start filled with a poison pattern; ``check_guards()``
then names every buffer whose bands were overwritten.
"""

import ctypes

import numpy as np
import torch

from . import bd

CANARY = 0xA7   # guard-band byte
POISON = 0x5A   # initial bytes of outputs (finite as fp32 / bf16, never a valid result here)


class GuardedBuffers:
    """Device tensors carved out of larger byte buffers with canary bands on both sides."""

    def __init__(self, device, guard_bytes):
        assert guard_bytes % 256 == 0
        self.device = device
        self.guard = guard_bytes
        self.bufs = []  # (name, raw uint8 tensor, interior bytes)

    def make(self, name, shape, dtype, init=None, fill=None):
        """A tensor of ``shape``/``dtype``: a copy of ``init`` (a device tensor), or
        filled with the byte ``fill``, or uninitialised."""
        elem = torch.empty((), dtype=dtype).element_size()
        n = int(np.prod(shape)) * elem
        if self.guard == 0:
            t = torch.empty(shape, dtype=dtype, device=self.device)
        else:
            raw = torch.full((n + 2 * self.guard,), CANARY, dtype=torch.uint8, device=self.device)
            t = raw[self.guard:self.guard + n].view(dtype).view(shape)
            self.bufs.append((name, raw, n))
        if init is not None:
            t.copy_(init.reshape(shape))
        elif fill is not None:
            t.view(torch.uint8).fill_(fill)
        return t

    def damaged(self):
        """Names of the buffers whose guard bands no longer hold the canary."""
        bad = []
        for name, raw, n in self.bufs:
            g = self.guard
            if bool((raw[:g] != CANARY).any()) or bool((raw[g + n:] != CANARY).any()):
                bad.append(name)
        return bad


def to_device(a: np.ndarray, device="cuda") -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


def _dt(a: np.ndarray):
    """torch dtype of the device copy of a host array (bf16 bits travel as int16)."""
    return {np.dtype(np.float32): torch.float32, np.dtype(np.uint16): torch.int16, np.dtype(np.uint8): torch.uint8,
            np.dtype(np.int32): torch.int32}[a.dtype]


def to_host(t: torch.Tensor, like=None) -> np.ndarray:
    a = t.detach().cpu().numpy()
    if like is not None and like == np.uint16:
        a = a.view(np.uint16)
    return a


class DeviceStep:
    """One step's inputs resident in HBM, with outputs and workspaces."""

    def __init__(self, step: dict, device="cuda", max_prefix=None, guard_bytes=0, balanced=False):
        """``max_prefix`` (default: the longest prefix of ``step``) is the host-side
        bound the attention plan is sized for; it must not exceed the cache capacity.
        ``guard_bytes`` > 0 puts canary bands of that size around every buffer the
        library writes (see check_guards).  ``balanced`` marks the batch as ragged
        (BD_PLAN_BALANCED in the attention descriptor's mode)."""
        p = step["params"]
        self.gb = GuardedBuffers(device, guard_bytes)
        mk = self.gb.make
        self.p = p
        self.dtype = p["dtype"]
        self.device = device
        n, D, Hq, Hkv, d = p["n_items"], p["D"], p["Hq"], p["Hkv"], p["d"]
        self.cap = int(step["cap"])
        self.max_prefix = int(step["prefix"].max()) if max_prefix is None else int(max_prefix)
        self.q = to_device(step["q"], device)
        self.k_blk = to_device(step["k_blk"], device)
        self.v_blk = to_device(step["v_blk"], device)
        self.k_cache = mk("k_cache", step["k_cache"].shape, _dt(step["k_cache"]), init=to_device(step["k_cache"], device))
        self.v_cache = mk("v_cache", step["v_cache"].shape, _dt(step["v_cache"]), init=to_device(step["v_cache"], device))
        self.prefix = mk("prefix", step["prefix"].shape, torch.int32, init=to_device(step["prefix"], device))
        # E4M3 K/V carry one fp32 scale per (item, KV head) for keys and for values.
        self.fp8kv = self.dtype == bd.BD_FP8KV
        self.k_scale = to_device(step["k_scale"], device) if self.fp8kv else None
        self.v_scale = to_device(step["v_scale"], device) if self.fp8kv else None
        self.logits = to_device(step["logits"], device)
        self.masked0 = to_device(step["masked"], device)
        self.tokens0 = to_device(step["tokens"], device)
        self.masked = mk("masked", self.masked0.shape, torch.uint8, init=self.masked0)
        self.tokens = mk("tokens", self.tokens0.shape, torch.int32, init=self.tokens0)
        self.draft = to_device(step["draft"], device) if "draft" in step else None
        self.out = mk("out", self.q.shape, self.q.dtype, fill=POISON)
        # The quadratic mode's descriptor takes the draft block size B; its tensors hold D = B (B + 3) / 2 slots.
        d_desc = p["B"] if p["mode"] == bd.BD_BLOCK_QUAD else D
        self.plan_flag = bd.BD_PLAN_BALANCED if balanced else 0
        self.adesc = bd.attn_desc(n, d_desc, Hq, Hkv, d, self.cap, self.dtype, p["mode"] | self.plan_flag,
                                  self.max_prefix)
        self.cdesc = bd.commit_desc(p["n_req"], D, p["V"], p["S"], p["tau"])
        ab = bd.bd_attn_workspace_bytes(self.adesc)
        cb = bd.bd_commit_workspace_bytes(self.cdesc)
        vb = bd.bd_verify_workspace_bytes(p["n_req"], D, p["V"])
        # A block shape the commit / verify calls do not take (the quadratic mode's
        # slot count) leaves their workspaces minimal; those calls then report it.
        cb = 16 if cb == bd.SIZE_MAX else cb
        vb = 16 if vb == bd.SIZE_MAX else vb
        self.attn_ws = mk("attn_ws", (max(ab, 16),), torch.uint8, fill=0)
        self.commit_ws = mk("commit_ws", (max(cb, 16),), torch.uint8, fill=0)
        self.verify_ws = mk("verify_ws", (max(vb, 16),), torch.uint8, fill=0)
        nr = p["n_req"]
        self.conf = mk("conf", (nr, D), torch.float32, fill=POISON)
        self.argmax = mk("argmax", (nr, D), torch.int32, fill=POISON)
        self.committed = mk("committed", (nr, D), torch.uint8, fill=POISON)
        self.n_committed = mk("n_committed", (nr,), torch.int32, fill=POISON)
        self.accepted = mk("accepted", (nr,), torch.int32, fill=POISON)
        self.dev_err = mk("dev_err", (1,), torch.int32, fill=0)

    def check_guards(self):
        """Names of the buffers whose canary bands were overwritten (empty if none,
        or if the step was built without guards)."""
        if torch.device(self.device).type == "cuda":
            torch.cuda.synchronize(self.device)
        return self.gb.damaged()

    def reset_block_state(self):
        self.masked.copy_(self.masked0)
        self.tokens.copy_(self.tokens0)

    def attn(self, mode=None, stream=None):
        desc = self.adesc
        if mode is not None and (mode | self.plan_flag) != desc.mode:
            desc = bd.attn_desc(desc.n_items, desc.D, desc.Hq, desc.Hkv, desc.d, desc.cap, desc.dtype,
                                mode | self.plan_flag, desc.max_prefix, desc.scale)
        if self.fp8kv:
            bd.bd_attn_step_fp8kv(desc, self.q, self.k_blk, self.v_blk, self.k_cache, self.v_cache, self.k_scale,
                                  self.v_scale, self.prefix, self.out, self.attn_ws, stream=stream)
        else:
            bd.bd_attn_step(desc, self.q, self.k_blk, self.v_blk, self.k_cache, self.v_cache, self.prefix,
                            self.out, self.attn_ws, stream=stream)
        return self.out

    def confidence_commit(self, logits=None, stream=None):
        bd.bd_confidence_commit(self.cdesc, self.logits if logits is None else logits, self.masked,
                                self.tokens, self.conf, self.argmax, self.committed, self.n_committed,
                                self.commit_ws, stream=stream)

    def step(self, stream=None):
        """One denoise step: block attention, then confidence + commit."""
        self.attn(stream=stream)
        self.confidence_commit(stream=stream)

    def layer_attn_args(self, it, stream=None):
        """bd_attn_step arguments for item ``it`` alone (one layer of a model), as a
        tuple for the raw C call: the descriptor has n_items = 1 and every pointer
        is offset to the item's slice."""
        a = self.adesc
        if not hasattr(self, "_layer_desc"):
            self._layer_desc = bd.attn_desc(1, a.D, a.Hq, a.Hkv, a.d, a.cap, a.dtype, a.mode, a.max_prefix,
                                            a.scale)
        eb = self.q.element_size()
        S = self.q.shape[1]  # block slots per item
        qo = it * S * a.Hq * a.d * eb
        bo = it * S * a.Hkv * a.d * eb
        co = it * a.Hkv * a.cap * a.d * eb
        return (ctypes.byref(self._layer_desc), self.q.data_ptr() + qo, self.k_blk.data_ptr() + bo,
                self.v_blk.data_ptr() + bo, self.k_cache.data_ptr() + co, self.v_cache.data_ptr() + co,
                self.prefix.data_ptr() + 4 * it, self.out.data_ptr() + qo, self.attn_ws.data_ptr(),
                self.attn_ws.numel(), bd._stream(stream))

    def layer_serial_step(self, stream=None):
        """The step as a model runs it: one bd_attn_step per item (layer), one after
        another on the stream, then confidence + commit."""
        for it in range(self.adesc.n_items):
            bd._check("bd_attn_step", bd.lib.bd_attn_step(*self.layer_attn_args(it, stream)))
        self.confidence_commit(stream=stream)

    def capture_layer_serial(self, restore_state=True):
        """A HIP graph of layer_serial_step (captured through torch): 36 dependent
        attention launches plus the commit become one replayable unit.  With
        ``restore_state`` the graph first copies the block's initial masked /
        tokens state back, so every replay does the same work."""
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.layer_serial_step(stream=side)  # warm-up outside the capture
            if restore_state:
                self.reset_block_state()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            if restore_state:
                self.reset_block_state()
            self.layer_serial_step(stream=side)
        return g

    def verify(self, logits=None, draft=None, stream=None):
        p = self.p
        bd.bd_spec_verify(p["n_req"], p["D"], p["V"], self.logits if logits is None else logits,
                          self.draft if draft is None else draft, self.accepted, self.argmax,
                          self.verify_ws, stream=stream)
        return self.accepted

    def append(self, n_accept=None, stream=None):
        bd.bd_kv_append(self.adesc, self.k_cache, self.v_cache, self.prefix, self.k_blk, self.v_blk,
                        n_accept, self.dev_err, stream=stream)
