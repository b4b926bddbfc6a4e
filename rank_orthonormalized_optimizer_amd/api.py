"""torch-facing wrappers of dion_step_batched (marshalling only, no arithmetic)."""
from __future__ import annotations

from collections import OrderedDict

import torch

from . import _lib

_DT = {torch.float32: _lib.F32, torch.bfloat16: _lib.BF16}


def _check(t: torch.Tensor, name: str, shape, dtypes) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live on a GPU, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")


def workspace_for(m: int, n: int, batch: int, rank: int, device) -> torch.Tensor:
    """Device scratch for one call (allocated by torch; 256-byte aligned)."""
    nbytes = _lib.workspace_size(m, n, batch, rank)
    ws = torch.empty(max(nbytes, 256) + 256, dtype=torch.uint8, device=device)
    off = (-ws.data_ptr()) % 256
    return ws[off:off + max(nbytes, 256)]


def step_(X: torch.Tensor, G: torch.Tensor, M: torch.Tensor, Q: torch.Tensor | None, rank: int,
          mu: float, lr: float, eps: float = 1e-8, *, workspace: torch.Tensor | None = None,
          flags: torch.Tensor | None = None, options: int = 0, stream=None, events=None,
          rmmc: torch.Tensor | None = None) -> None:
    """One Dion step on a stack, in place on X, M and Q.

    X, G: [b, m, n] float32 or bfloat16; M: [b, m, n] float32; Q: [b, n, rank] float32.
    ``flags`` (int32 [b], optional) receives the per-matrix FLAG_* bits.
    Enqueued on ``stream`` (default: torch's current stream) with no host sync.
    ``events``: optional NUM_PHASES + 1 recorded torch.cuda.Event objects, re-recorded at the
    phase boundaries of the step (profiling).
    ``rmmc`` (float32 [b], optional) receives each matrix's relative maximum momentum change
    max |M' - M| / max |M| over the step.
    """
    if X.dim() != 3:
        raise ValueError("X must be a stack [batch, m, n]; route 1-D parameters to AdamW or Lion")
    b, m, n = X.shape
    _check(X, "X", (b, m, n), tuple(_DT))
    _check(G, "G", (b, m, n), tuple(_DT))
    _check(M, "M", (b, m, n), (torch.float32,))
    if rank > 0:
        _check(Q, "Q", (b, n, rank), (torch.float32,))
    if flags is not None:
        _check(flags, "flags", (b,), (torch.int32,))
    if rmmc is not None:
        _check(rmmc, "rmmc", (b,), (torch.float32,))
    if workspace is None:
        workspace = workspace_for(m, n, b, rank, X.device)
    if stream is None:
        stream = torch.cuda.current_stream(X.device)
    st = _lib.step_batched_raw(X.data_ptr(), G.data_ptr(), M.data_ptr(), Q.data_ptr() if rank > 0 else 0,
                               m, n, b, rank, float(mu), float(lr), float(eps), _DT[X.dtype], _DT[G.dtype],
                               workspace.data_ptr(), workspace.numel(),
                               flags.data_ptr() if flags is not None else 0, int(options),
                               int(stream.cuda_stream),
                               None if events is None else [e.cuda_event for e in events],
                               rmmc.data_ptr() if rmmc is not None else 0)
    if st != _lib.OK:
        raise _lib.DionError(st)


class StickyF64Hint:
    """Host-side knowledge, gathered without a host sync, that a whole stack is on the fp64 chain.

    Under OPT_STICKY_F64 a matrix whose FLAG_F64 is set skips the fp32 attempt and keeps the
    flag, so once every flag is set the fp32 chain has no matrix left and OPT_FORCE_F64 gives
    the same kernels' work and bitwise the same results while not launching the (empty) fp32
    chain at all.  After each step the flags are copied to pinned host memory; the copy is
    looked at on a later step, once its event has completed.  Call ``reset()`` after changing
    the flags tensor by hand.
    """

    def __init__(self, flags: torch.Tensor):
        self.flags = flags
        self.host = torch.zeros(tuple(flags.shape), dtype=torch.int32, pin_memory=True)
        self.event = None
        self.all_f64 = False

    def reset(self) -> None:
        self.event = None
        self.all_f64 = False

    def options(self, base: int) -> int:
        if self.all_f64 and (base & _lib.OPT_STICKY_F64) and not (base & _lib.OPT_FORCE_F32):
            return base | _lib.OPT_FORCE_F64
        return base

    def after_step(self, stream) -> None:
        if self.all_f64:
            return
        if self.event is not None:
            if not self.event.query():
                return                       # the last copy is still in flight: look next step
            self.all_f64 = bool(((self.host & _lib.FLAG_F64) != 0).all())
            if self.all_f64:
                return
        with torch.cuda.stream(stream):
            self.host.copy_(self.flags, non_blocking=True)
            self.event = torch.cuda.Event()
            self.event.record(stream)


class DionStack:
    """Optimizer state (M, Q, flags, workspace) of one stack of same-shape matrices.

    ``rank_fraction`` picks r = floor(fraction * min(m, n)) (the rank-fraction
    knob of the rivista.ai Dion page) unless ``rank`` is given.  The fp64
    fallback is sticky by default: a matrix that needed it keeps it.
    """

    def __init__(self, batch: int, m: int, n: int, *, rank: int | None = None, rank_fraction: float = 0.25,
                 mu: float = 0.95, lr: float = 0.01, eps: float = 1e-8, device="cuda", sticky: bool = True,
                 seed: int = 0):
        self.batch, self.m, self.n = batch, m, n
        self.rank = int(rank if rank is not None else int(rank_fraction * min(m, n)))
        self.mu, self.lr, self.eps = mu, lr, eps
        self.options = _lib.OPT_STICKY_F64 if sticky else 0
        dev = torch.device(device)
        self.M = torch.zeros(batch, m, n, dtype=torch.float32, device=dev)
        gen = torch.Generator(device="cpu").manual_seed(seed)
        q = torch.randn(batch, n, self.rank, generator=gen, dtype=torch.float64)
        if self.rank:
            q /= q.norm(dim=1, keepdim=True)
        self.Q = q.to(torch.float32).to(dev).contiguous()
        self.flags = torch.zeros(batch, dtype=torch.int32, device=dev)
        self.workspace = workspace_for(m, n, batch, self.rank, dev)
        self.hint = StickyF64Hint(self.flags) if sticky else None

    def step(self, X: torch.Tensor, G: torch.Tensor) -> None:
        opts = self.hint.options(self.options) if self.hint is not None else self.options
        stream = torch.cuda.current_stream(self.flags.device)
        step_(X, G, self.M, self.Q, self.rank, self.mu, self.lr, self.eps, workspace=self.workspace,
              flags=self.flags, options=opts, stream=stream)
        if self.hint is not None:
            self.hint.after_step(stream)

    def state_dict(self) -> dict:
        """The state a checkpoint needs, as CPU tensors: the momentum M, the right factor Q and
        the per-matrix flags (their fp64 mark keeps a matrix on the fp64 chain), with the
        sizes and hyper-parameters.  The workspace carries nothing from one step to the next, so
        a stack restored with load_state_dict continues bitwise as if it had not stopped."""
        return {"M": self.M.cpu(), "Q": self.Q.cpu(), "flags": self.flags.cpu(),
                "shape": [self.batch, self.m, self.n], "rank": self.rank, "mu": self.mu, "lr": self.lr,
                "eps": self.eps, "options": self.options}

    def load_state_dict(self, sd: dict) -> None:
        """Restore a state_dict() of a stack with the same sizes (copied into this stack's
        device tensors; the host's fp64 hint starts over, which selects the same work)."""
        if list(sd["shape"]) != [self.batch, self.m, self.n] or int(sd["rank"]) != self.rank:
            raise ValueError(f"state of a {sd['shape']} r={sd['rank']} stack, this one is "
                             f"{[self.batch, self.m, self.n]} r={self.rank}")
        self.M.copy_(sd["M"])
        self.Q.copy_(sd["Q"])
        self.flags.copy_(sd["flags"])
        self.mu, self.lr, self.eps, self.options = float(sd["mu"]), float(sd["lr"]), float(sd["eps"]), int(sd["options"])
        self.hint = StickyF64Hint(self.flags) if self.options & _lib.OPT_STICKY_F64 else None

    @property
    def P(self) -> torch.Tensor:
        """This step's orthonormal factor P [b, m, r] (fp32), read from the workspace."""
        n = self.batch * self.m * self.rank
        return self.workspace[:4 * n].view(torch.float32).view(self.batch, self.m, self.rank)


class GraphedStep:
    """One DionStack step captured in a HIP graph for fixed tensors, replayed by ``replay()``.

    The step's kernels and arguments are those of ``stack.step(X, G)`` at capture time
    (including the options the host hint has settled on), so a replay gives bitwise the result
    of an eager step on the same inputs, without the host launching each kernel.  ``G`` is read
    at replay time: refill it in place between replays.  Capture after at least one eager step
    (the sticky flags and the hint settle there); recapture if the options should change.
    """

    def __init__(self, stack: "DionStack", X: torch.Tensor, G: torch.Tensor):
        self.stack, self.X, self.G = stack, X, G
        dev = stack.flags.device
        opts = stack.hint.options(stack.options) if stack.hint is not None else stack.options
        cur = torch.cuda.current_stream(dev)
        cap = torch.cuda.Stream(device=dev)
        cap.wait_stream(cur)
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(cap):
            self.graph.capture_begin()
            step_(X, G, stack.M, stack.Q, stack.rank, stack.mu, stack.lr, stack.eps, workspace=stack.workspace,
                  flags=stack.flags, options=opts, stream=cap)
            self.graph.capture_end()
        cur.wait_stream(cap)

    def replay(self) -> None:
        """Enqueue the captured step on torch's current stream."""
        self.graph.replay()


def group_matrices(params) -> "OrderedDict[tuple, list]":
    """Group 2-D tensors by (shape, dtype) into stackable lists; reject anything else.

    Dion updates 2-D weight matrices only; biases and other 1-D tensors go to
    AdamW or Lion, so they raise here instead of being silently skipped.
    """
    groups: "OrderedDict[tuple, list]" = OrderedDict()
    for i, p in enumerate(params):
        if p.dim() != 2:
            raise ValueError(f"parameter {i} has shape {tuple(p.shape)}: only 2-D matrices go to Dion")
        groups.setdefault((tuple(p.shape), p.dtype), []).append(p)
    return groups


def _flat_check(t: torch.Tensor, name: str, n: int, dtypes) -> None:
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous GPU tensor")
    if t.numel() != n or t.dtype not in dtypes:
        raise ValueError(f"{name}: {t.numel()} elements of {t.dtype}, expected {n} of {dtypes}")


def adamw_step_(param: torch.Tensor, grad: torch.Tensor, exp_avg: torch.Tensor, exp_avg_sq: torch.Tensor, t: int,
                lr: float, beta1: float = 0.9, beta2: float = 0.999, eps: float = 1e-8, weight_decay: float = 0.0,
                *, stream=None) -> None:
    """One AdamW step (dion_adamw_step) on a contiguous tensor of any shape, in place; t counts from 1."""
    n = param.numel()
    _flat_check(param, "param", n, tuple(_DT))
    _flat_check(grad, "grad", n, tuple(_DT))
    _flat_check(exp_avg, "exp_avg", n, (torch.float32,))
    _flat_check(exp_avg_sq, "exp_avg_sq", n, (torch.float32,))
    if stream is None:
        stream = torch.cuda.current_stream(param.device)
    st = _lib.adamw_step_raw(param.data_ptr(), grad.data_ptr(), exp_avg.data_ptr(), exp_avg_sq.data_ptr(), n, int(t),
                             float(lr), float(beta1), float(beta2), float(eps), float(weight_decay),
                             _DT[param.dtype], _DT[grad.dtype], int(stream.cuda_stream))
    if st != _lib.OK:
        raise _lib.DionError(st, "dion_adamw_step")


def lambda_max_(W: torch.Tensor, k: int = 32, iters: int = 10, V0: torch.Tensor | None = None,
                out: torch.Tensor | None = None, *, stream=None) -> torch.Tensor:
    """Multi-power-iteration estimate of lambda_max for each symmetric PSD matrix of the fp64
    stack W [b, r, r] (dion_lambda_max_batched; only the lower triangle is read).  V0 [b, r, k]
    fp64 or None for the library's start vectors.  Returns (or fills) fp64 [b] on W's device."""
    if not isinstance(W, torch.Tensor) or W.device.type != "cuda" or W.dtype != torch.float64 or W.dim() != 3 \
            or W.shape[1] != W.shape[2] or not W.is_contiguous():
        raise ValueError("W must be a contiguous fp64 GPU tensor [b, r, r]")
    b, r = int(W.shape[0]), int(W.shape[1])
    if V0 is not None:
        if V0.dtype != torch.float64 or tuple(V0.shape) != (b, r, k) or not V0.is_contiguous() or V0.device != W.device:
            raise ValueError(f"V0 must be a contiguous fp64 tensor [{b}, {r}, {k}] on W's device")
    if out is None:
        out = torch.empty(b, dtype=torch.float64, device=W.device)
    elif out.dtype != torch.float64 or out.numel() != b or not out.is_contiguous() or out.device != W.device:
        raise ValueError("out must be a contiguous fp64 tensor of b elements on W's device")
    nbytes = _lib.lambda_max_workspace_size(r, b, k)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=W.device)
    if stream is None:
        stream = torch.cuda.current_stream(W.device)
    st = _lib.lambda_max_raw(W.data_ptr(), r, b, 0 if V0 is None else V0.data_ptr(), int(k), int(iters),
                             out.data_ptr(), ws.data_ptr(), nbytes, int(stream.cuda_stream))
    if st != _lib.OK:
        raise _lib.DionError(st, "dion_lambda_max_batched")
    return out


def lion_step_(param: torch.Tensor, grad: torch.Tensor, exp_avg: torch.Tensor, lr: float, beta1: float = 0.9,
               beta2: float = 0.99, weight_decay: float = 0.0, *, stream=None) -> None:
    """One Lion step (dion_lion_step) on a contiguous tensor of any shape, in place."""
    n = param.numel()
    _flat_check(param, "param", n, tuple(_DT))
    _flat_check(grad, "grad", n, tuple(_DT))
    _flat_check(exp_avg, "exp_avg", n, (torch.float32,))
    if stream is None:
        stream = torch.cuda.current_stream(param.device)
    st = _lib.lion_step_raw(param.data_ptr(), grad.data_ptr(), exp_avg.data_ptr(), n, float(lr), float(beta1),
                            float(beta2), float(weight_decay), _DT[param.dtype], _DT[grad.dtype],
                            int(stream.cuda_stream))
    if st != _lib.OK:
        raise _lib.DionError(st, "dion_lion_step")


class MixedDion:
    """Dion for the 2-D parameters, AdamW or Lion for the rest (rivista.ai, "Tecnicamente").

    ``params``: a list of GPU tensors.  2-D ones are grouped by (shape, dtype) into stacks
    (each step copies the group's weights and gradients into [b, m, n] stacks and back, since
    torch parameters are separate tensors); every other tensor gets element-wise state.
    ``step(grads)`` takes the gradients in the same order.
    """

    def __init__(self, params, *, lr: float = 0.01, mu: float = 0.95, rank_fraction: float = 0.25,
                 other: str = "adamw", other_lr: float = 1e-3, betas=(0.9, 0.999), eps: float = 1e-8,
                 weight_decay: float = 0.0):
        if other not in ("adamw", "lion"):
            raise ValueError("other must be 'adamw' or 'lion'")
        self.params = list(params)
        self.other, self.other_lr, self.betas, self.eps, self.wd = other, other_lr, betas, eps, weight_decay
        self.t = 0
        self.groups = []   # (indices, DionStack)
        mats = OrderedDict()
        for i, p in enumerate(self.params):
            if p.dim() == 2:
                mats.setdefault((tuple(p.shape), p.dtype), []).append(i)
        for (shape, _), idx in mats.items():
            st = DionStack(len(idx), shape[0], shape[1], rank_fraction=rank_fraction, mu=mu, lr=lr,
                           device=self.params[idx[0]].device)
            self.groups.append((idx, st))
        self.rest = [i for i, p in enumerate(self.params) if p.dim() != 2]
        self.state = {i: (torch.zeros(self.params[i].numel(), dtype=torch.float32, device=self.params[i].device),
                          torch.zeros(self.params[i].numel(), dtype=torch.float32, device=self.params[i].device)
                          if other == "adamw" else None) for i in self.rest}

    @torch.no_grad()
    def step(self, grads) -> None:
        grads = list(grads)
        self.t += 1
        for idx, st in self.groups:
            X = torch.stack([self.params[i] for i in idx]).contiguous()
            G = torch.stack([grads[i] for i in idx]).contiguous()
            st.step(X, G)
            for k, i in enumerate(idx):
                self.params[i].copy_(X[k])
        for i in self.rest:
            p, g = self.params[i], grads[i].contiguous()
            m, v = self.state[i]
            if self.other == "adamw":
                adamw_step_(p, g, m, v, self.t, self.other_lr, self.betas[0], self.betas[1], self.eps, self.wd)
            else:
                lion_step_(p, g, m, self.other_lr, self.betas[0], self.betas[1], self.wd)
