"""Drop-in torch.optim optimizers over split weights and 8-bit states.

FlashOptim's optimizers are drop-in replacements for torch.optim that compute
the same updates with less memory ([BLOG] "FlashOptim: Breaking the Memory
Wall ...", Conclusion & Perspective; Davis Blalock's FlashOptim thread, the
launch post).  Here the model parameter itself becomes the 16-bit theta' (the
thread's post on avoiding the redundant f32 + low-precision copies); the
optimizer keeps the ECC and the 8-bit states.  Gradients therefore arrive in
16 bits (the post on keeping gradients in backward precision).  Optional
gradient release steps parameters while backward runs, as their gradients
are accumulated, and frees those gradients (the post on gradient release);
parameters are stepped in buckets of at least `release_bucket` elements so
that many small tensors share one fused call.

All arithmetic runs in the HIP library (fo_fused_adamw_step /
fo_fused_sgdm_step); this module only groups tensors and keeps step counts.
FlashAdamW, FlashAdam and FlashSGD follow torch.optim.AdamW, Adam and SGD.
codec="companded4" keeps 4-bit state codes instead (two per byte; the
blog's Conclusion & Perspective names lower-bit states as the next step), and
codec="companded_bf16scale" keeps the 8-bit codes with bfloat16 block scales.

Between steps the optimizers keep the device addresses of each parameter's
state tensors (ECC, codes, scales); only theta' and gradient addresses are
read at every step.  State changes through load_state_dict(),
import_torch_state(), import_torch_optimizer() and load_master_weights() are
safe (they write in place or drop the kept addresses).  Code that replaces a
state tensor in `optimizer.state` by other means must call
invalidate_launch_cache() before the next step.
"""

from __future__ import annotations

import importlib.util
import itertools
import operator
import os
from typing import Iterable

import torch

from . import binding as B

_W16 = {"bf16": torch.bfloat16, "fp16": torch.float16}
_ECC = {8: torch.int8, 16: torch.int16}


def _nb(n: int) -> int:
    return (n + 31) // 32


def _load_fill_rows():
    """fill_rows of the host marshalling extension (lib/fo_marshal.so, built
    with the library), or None when it has not been built: the optimizers then
    marshal their launch rows in Python (the same rows, more host time)."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "fo_marshal.so")
    if not os.path.exists(path):
        return None
    spec = importlib.util.spec_from_file_location("fo_marshal", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod.fill_rows


_fill_rows = _load_fill_rows()
_STEP = operator.itemgetter("step")


class _Plan:
    """What a parameter list needs at every step, built once per list: the
    parameters (held, so their ids stay theirs), their state dicts and the
    address-independent part of each launch row.  `gen` is unique per plan
    and keys the marshalled lists built from it.  With the marshalling
    extension the plan also holds those parts as an int64 matrix (`fixed`)
    and one launch list (`tl`) whose rows the extension rewrites at every
    step (the library reads a list only during the call)."""

    __slots__ = ("params", "states", "static", "gen", "fixed", "tl", "rows_addr")
    _gens = itertools.count()

    def __init__(self, params, states, static, list_from_rows=None):
        self.params, self.states, self.static = params, states, static
        self.gen = next(_Plan._gens)
        self.fixed = self.tl = self.rows_addr = None
        if list_from_rows is not None and static:
            import ctypes
            self.fixed = torch.tensor(static, dtype=torch.int64)
            self.tl = list_from_rows([(0,) * (len(static[0]) + 2)] * len(static))
            self.rows_addr = ctypes.addressof(self.tl.array)


class _FlashBase(torch.optim.Optimizer):
    _state_keys: tuple = ()

    def __init__(self, params, defaults, wfmt, ecc_bits, codec, grad_release, release_bucket=1 << 26):
        if (wfmt, ecc_bits) not in (("bf16", 8), ("bf16", 16), ("fp16", 8)):
            raise ValueError(f"unsupported weight format {wfmt}+ECC{ecc_bits}")
        if codec not in ("companded", "linear", "companded4", "companded_bf16scale"):
            raise ValueError(f"unknown codec {codec}")
        self.wfmt, self.ecc_bits, self.codec = wfmt, ecc_bits, codec
        self.grad_release = grad_release
        # gradient release steps parameters in buckets of at least this many
        # elements (one fused call each); the rest is stepped when backward ends
        self.release_bucket = int(release_bucket)
        self._pending = []
        self._pending_elems = 0
        self._flush_queued = False
        self._hooks = []
        # per parameter list: a _Plan, and the marshalled launch lists keyed by
        # (plan, theta' addresses, gradient addresses) -- ints only, so nothing
        # here keeps a gradient alive
        self._plans = {}
        self._lists = {}
        self._group_of = {}
        super().__init__(params, defaults)
        for group in self.param_groups:
            for p in group["params"]:
                self._adopt(p)
                if grad_release:
                    self._hooks.append(p.register_post_accumulate_grad_hook(self._release_hook))

    # -- conversion of a parameter into theta' + ECC ------------------------
    def _adopt(self, p: torch.nn.Parameter) -> None:
        if not p.is_cuda:
            raise ValueError("parameters must live on the GPU")
        st = self.state[p]
        if "ecc" in st:
            return
        n = p.numel()
        w16 = torch.empty(p.shape, dtype=_W16[self.wfmt], device=p.device)
        ecc = torch.empty(p.shape, dtype=_ECC[self.ecc_bits], device=p.device)
        master = p.detach().to(torch.float32).contiguous()
        B.fo_split_weights(master.view(-1), w16.view(-1), ecc.view(-1), self.wfmt, self.ecc_bits)
        p.data = w16
        st["step"] = 0
        st["ecc"] = ecc
        for key, dt, per_block in self._state_keys:
            if per_block or self.codec != "companded4":
                st[key] = torch.zeros(_nb(n) if per_block else n, dtype=dt, device=p.device)
            else:                                        # two 4-bit codes per byte
                st[key] = torch.zeros((n + 1) // 2, dtype=torch.uint8, device=p.device)

    # -- master weights -------------------------------------------------------
    @torch.no_grad()
    def master_weights(self, p: torch.nn.Parameter) -> torch.Tensor:
        """The reconstructed f32 master weight of `p` (theta' + ECC)."""
        out = torch.empty(p.shape, dtype=torch.float32, device=p.device)
        B.fo_reconstruct_weights(p.detach().view(-1), self.state[p]["ecc"].view(-1), out.view(-1),
                                 self.wfmt, self.ecc_bits)
        return out

    @torch.no_grad()
    def load_master_weights(self, p: torch.nn.Parameter, w32: torch.Tensor) -> None:
        """Re-split an f32 master weight into `p` (theta') and its ECC."""
        w32 = w32.to(device=p.device, dtype=torch.float32).contiguous().view(-1)
        B.fo_split_weights(w32, p.data.view(-1), self.state[p]["ecc"].view(-1), self.wfmt, self.ecc_bits)

    # -- stepping ---------------------------------------------------------------
    def _static(self, p):
        """(ecc address, state addresses..., numel): the part of p's launch row
        that does not change between steps."""
        raise NotImplementedError

    def _launch(self, entries, group, step):
        raise NotImplementedError

    def _plan(self, params):
        ids = tuple(map(id, params))
        plan = self._plans.get(ids)
        if plan is None or not all(map(operator.is_, plan.params, params)):
            if len(self._plans) >= 4096:
                self._plans.clear()
                self._lists.clear()
            plan = self._plans[ids] = _Plan(list(params), [self.state[p] for p in params],
                                            [self._static(p) for p in params],
                                            self._list_from_rows if _fill_rows is not None else None)
        return plan

    def _list_for(self, plan, params, static, grads=None):
        # rows of raw addresses (w16, ecc, grad, states..., n); the ctypes array
        # is rebuilt only when a theta' or gradient address changes
        w = tuple([p.data_ptr() for p in params])
        g = tuple([x.data_ptr() for x in grads]) if grads is not None else tuple([p.grad.data_ptr() for p in params])
        key = (plan.gen, w, g)
        tl = self._lists.get(key)
        if tl is None:
            if len(self._lists) >= 4096:
                self._lists.clear()
            rows = tuple((wp, st[0], gp) + st[1:] for wp, gp, st in zip(w, g, static))
            tl = self._lists[key] = self._list_from_rows(rows)
        return tl

    def _step_params(self, group, params, grads=None, plan=None, tl=None):
        plan = plan or self._plan(params)
        if tl is None and plan.tl is not None and \
                _fill_rows(params, plan.fixed, plan.rows_addr, _W16[self.wfmt]) == 0:
            tl = plan.tl
        for st in plan.states:
            st["step"] += 1
        steps = list(map(_STEP, plan.states))
        if steps.count(steps[0]) == len(steps):
            self._launch(tl or self._list_for(plan, params, plan.static, grads), group, steps[0])
            return
        # parameters with different step counts (imported or reloaded states):
        # one launch per count
        by_step = {}
        for i, s in enumerate(steps):
            by_step.setdefault(s, []).append(i)
        for s, idx in by_step.items():
            sub = self._plan([params[i] for i in idx])
            self._launch(self._list_for(sub, sub.params, sub.static), group, s)

    @torch.no_grad()
    def step(self, closure=None):
        loss = None
        if closure is not None:
            with torch.enable_grad():
                loss = closure()
        wdt = _W16[self.wfmt]
        for group in self.param_groups:
            ps = group["params"]
            if not ps:
                continue
            if _fill_rows is not None:
                # every gradient present, in theta's format and contiguous: the
                # extension writes the plan's launch rows in one call
                plan = self._plan(ps)
                if _fill_rows(ps, plan.fixed, plan.rows_addr, wdt) == 0:
                    self._step_params(group, ps, plan=plan, tl=plan.tl)
                    continue
            # otherwise: drop parameters without gradients, convert the others
            # where needed (the rows of the remaining list are then filled as above,
            # or in Python without the extension)
            gs = [p.grad for p in ps]
            if any(map(operator.is_, gs, itertools.repeat(None))):
                keep = [i for i, g in enumerate(gs) if g is not None]
                ps, gs = [ps[i] for i in keep], [gs[i] for i in keep]
            if not ps:
                continue
            # gradients in the 16-bit format of theta' and contiguous (what autograd
            # produces for these parameters); anything else is converted here
            for i in [i for i, g in enumerate(gs) if g.dtype is not wdt or not g.is_contiguous()]:
                ps[i].grad = gs[i] = gs[i].to(wdt).contiguous()
            self._step_params(group, ps, gs)
        return loss

    def _group(self, p):
        # id -> (group, parameter); the stored parameter guards against a
        # reused id, and a miss (e.g. after add_param_group) rebuilds the map
        e = self._group_of.get(id(p))
        if e is None or e[1] is not p:
            self._group_of = {id(q): (grp, q) for grp in self.param_groups for q in grp["params"]}
            e = self._group_of[id(p)]
        return e[0]

    def _release_hook(self, p):
        """Runs when p's gradient is complete during backward.  Parameters are
        queued; a bucket of at least `release_bucket` elements is stepped in one
        fused call and its gradients freed at once, and whatever is still queued
        when backward finishes is stepped then (the end-of-backward callback).
        It runs once per parameter, so it enters no grad-mode context unless it
        converts a gradient (the bucket step enters its own)."""
        g = p.grad
        if g.dtype is not p.dtype or not g.is_contiguous():
            with torch.no_grad():
                p.grad = g.to(p.dtype).contiguous()
        self._pending.append(p)
        self._pending_elems += p.numel()
        if not self._flush_queued:
            try:
                torch.autograd.Variable._execution_engine.queue_callback(self.flush_released)
            except RuntimeError:        # not inside a backward pass: the caller flushes
                pass
            self._flush_queued = True   # either way, until the next flush
        if self._pending_elems >= self.release_bucket:
            self._step_pending()

    @torch.no_grad()
    def _step_pending(self):
        if len(self.param_groups) == 1:
            self._step_params(self.param_groups[0], self._pending)
        else:
            by_group = {}
            for q in self._pending:
                g = self._group(q)
                by_group.setdefault(id(g), (g, []))[1].append(q)
            for g, ps in by_group.values():
                self._step_params(g, ps)
        for q in self._pending:
            q.grad = None       # freed in stream order by torch's caching allocator
        self._pending = []
        self._pending_elems = 0

    @torch.no_grad()
    def flush_released(self):
        """Step every parameter still queued by gradient release.  Called by
        autograd at the end of each backward pass; call it directly when the
        hooks were driven outside a backward pass."""
        self._flush_queued = False
        if self._pending:
            self._step_pending()

    def load_state_dict(self, state_dict):
        """torch's loader casts every tensor of a floating-point parameter's
        state to the parameter dtype; the ECC, codes and scale patterns are raw
        integers, so they are re-installed unchanged after the base loader."""
        saved_ids = [i for g in state_dict["param_groups"] for i in g["params"]]
        raw = {k: {kk: vv for kk, vv in v.items() if torch.is_tensor(vv)}
               for k, v in state_dict["state"].items()}
        super().load_state_dict(state_dict)
        self.invalidate_launch_cache()
        self._group_of = {}
        params = [p for g in self.param_groups for p in g["params"]]
        for pid, p in zip(saved_ids, params):
            for key, val in raw.get(pid, {}).items():
                self.state[p][key] = val.to(device=p.device).clone()
            if "step" in self.state[p]:
                self.state[p]["step"] = int(self.state[p]["step"])

    def invalidate_launch_cache(self):
        """Forget the kept state addresses and marshalled launch lists (after
        state tensors were replaced outside this class's methods)."""
        self._plans.clear()
        self._lists.clear()

    def remove_hooks(self):
        for h in self._hooks:
            h.remove()
        self._hooks = []


class FlashAdamW(_FlashBase):
    """AdamW (decoupled weight decay, bias correction) with bf16/fp16 theta' +
    8/16-bit ECC master weights and companded 8-bit m, v."""

    # scales are kept as int16 bit patterns of fp16 values: torch's
    # load_state_dict would cast floating-point state to the parameter dtype
    _state_keys = (("m_q", torch.int8, False), ("m_s", torch.int16, True),
                   ("v_q", torch.uint8, False), ("v_s", torch.int16, True))

    def __init__(self, params: Iterable, lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=1e-2, *,
                 wfmt="bf16", ecc_bits=8, codec="companded", grad_release=False, release_bucket=1 << 26):
        defaults = dict(lr=lr, betas=betas, eps=eps, weight_decay=weight_decay)
        super().__init__(params, defaults, wfmt, ecc_bits, codec, grad_release, release_bucket)

    def _static(self, p):
        st = self.state[p]
        return (st["ecc"].data_ptr(), st["m_q"].data_ptr(), st["m_s"].data_ptr(), st["v_q"].data_ptr(),
                st["v_s"].data_ptr(), p.numel())

    @staticmethod
    def _list_from_rows(rows):
        return B.AdamWList.from_rows(rows)

    _l2_decay = False

    def _launch(self, tl, group, step):
        b1, b2 = group["betas"]
        B.fo_fused_adamw_step(tl, B.adamw_hparams(group["lr"], b1, b2, group["eps"], group["weight_decay"], step,
                                                  self.wfmt, self.ecc_bits, self.codec, self._l2_decay))

    @torch.no_grad()
    def export_torch_state(self, p):
        """f32 (exp_avg, exp_avg_sq) of `p`, decoded from the 8-bit states."""
        st = self.state[p]
        m = torch.empty(p.numel(), dtype=torch.float32, device=p.device)
        v = torch.empty_like(m)
        B.fo_dequantize(st["m_q"], st["m_s"], m, "m", self.codec)
        B.fo_dequantize(st["v_q"], st["v_s"], v, "v", self.codec)   # scale patterns in the codec's format
        return m.view(p.shape), v.view(p.shape)

    @torch.no_grad()
    def import_torch_state(self, p, exp_avg, exp_avg_sq, step):
        """Quantise an f32 (exp_avg, exp_avg_sq) pair, e.g. from torch.optim.AdamW,
        into the 8-bit states of `p` and set its step count."""
        st = self.state[p]
        for key, x, kind in (("m", exp_avg, "m"), ("v", exp_avg_sq, "v")):
            x = x.detach().to(device=p.device, dtype=torch.float32).contiguous().view(-1)
            if x.numel() != p.numel():
                raise ValueError(f"state of {x.numel()} elements for a parameter of {p.numel()}")
            B.fo_companded_quantize(x, st[key + "_q"], st[key + "_s"], kind, self.codec)
        st["step"] = int(step)

    def import_torch_optimizer(self, torch_opt):
        """Take over the moments and step counts of a torch.optim.Adam/AdamW that
        was stepping the same parameters (its state is keyed by them)."""
        for group in self.param_groups:
            for p in group["params"]:
                s = torch_opt.state.get(p)
                if s and "exp_avg" in s:
                    self.import_torch_state(p, s["exp_avg"], s["exp_avg_sq"], int(s["step"]))


class FlashAdam(FlashAdamW):
    """Adam as torch.optim.Adam: the weight decay is added to the gradient
    (L2 regularisation) instead of being applied to the weights."""

    _l2_decay = True

    def __init__(self, params: Iterable, lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.0, **kw):
        super().__init__(params, lr=lr, betas=betas, eps=eps, weight_decay=weight_decay, **kw)


class FlashSGD(_FlashBase):
    """SGD with momentum as torch.optim.SGD (coupled weight decay, optional
    dampening and Nesterov momentum) with split master weights and a companded
    8-bit momentum buffer."""

    _state_keys = (("b_q", torch.int8, False), ("b_s", torch.int16, True))

    def __init__(self, params: Iterable, lr=1e-2, momentum=0.9, dampening=0.0, weight_decay=0.0, nesterov=False, *,
                 wfmt="bf16", ecc_bits=8, codec="companded", grad_release=False, release_bucket=1 << 26):
        if nesterov and (momentum <= 0.0 or dampening != 0.0):
            raise ValueError("Nesterov momentum requires a momentum and zero dampening")
        defaults = dict(lr=lr, momentum=momentum, dampening=dampening, weight_decay=weight_decay, nesterov=nesterov)
        super().__init__(params, defaults, wfmt, ecc_bits, codec, grad_release, release_bucket)

    def _static(self, p):
        st = self.state[p]
        return (st["ecc"].data_ptr(), st["b_q"].data_ptr(), st["b_s"].data_ptr(), p.numel())

    @staticmethod
    def _list_from_rows(rows):
        return B.SGDMList.from_rows(rows)

    @torch.no_grad()
    def export_torch_state(self, p):
        """f32 momentum_buffer of `p`, decoded from the 8-bit state."""
        st = self.state[p]
        b = torch.empty(p.numel(), dtype=torch.float32, device=p.device)
        B.fo_dequantize(st["b_q"], st["b_s"], b, "m", self.codec)
        return b.view(p.shape)

    @torch.no_grad()
    def import_torch_state(self, p, momentum_buffer, step):
        """Quantise an f32 momentum buffer (torch.optim.SGD) into `p`'s state."""
        st = self.state[p]
        x = momentum_buffer.detach().to(device=p.device, dtype=torch.float32).contiguous().view(-1)
        if x.numel() != p.numel():
            raise ValueError(f"state of {x.numel()} elements for a parameter of {p.numel()}")
        B.fo_companded_quantize(x, st["b_q"], st["b_s"], "m", self.codec)
        st["step"] = int(step)

    def _launch(self, tl, group, step):
        B.fo_fused_sgdm_step(tl, B.sgdm_hparams(group["lr"], group["momentum"], group["weight_decay"], step,
                                                self.wfmt, self.ecc_bits, self.codec,
                                                group["dampening"], group["nesterov"]))
