"""The drop-in optimizers (FlashAdamW, FlashAdam, FlashSGD) on a small model: every step
matches the oracle bit for bit in lock-step (the oracle steps a host copy of
the optimizer's state before each step), gradient release matches the plain
step, state_dict save/load resumes bit for bit, and training tracks
torch.optim.AdamW in float32."""

import copy

import numpy as np
import pytest
import torch

import oracle as O
from precision_optimizer_state_amd import FlashAdam, FlashAdamW, FlashSGD
from tests.gpu_helpers import check_state, check_weights, to_host

pytestmark = pytest.mark.gpu


def _model(seed=0):
    torch.manual_seed(seed)
    m = torch.nn.Sequential(torch.nn.Linear(64, 96), torch.nn.GELU(), torch.nn.Linear(96, 33))
    return m.cuda()


def _batch(i, dtype=torch.bfloat16):
    g = torch.Generator(device="cuda")
    g.manual_seed(1000 + i)
    x = torch.randn(128, 64, generator=g, device="cuda").to(dtype)
    y = torch.randn(128, 33, generator=g, device="cuda").to(dtype)
    return x, y


def _loss(model, i):
    x, y = _batch(i)
    return torch.nn.functional.mse_loss(model(x).float(), y.float())


HP = dict(lr=3e-3, betas=(0.9, 0.95), eps=1e-8, weight_decay=0.1)


def _host_state(opt, p, adam=True):
    st = opt.state[p]
    out = {"w16": to_host(p.data.view(-1)), "ecc": to_host(st["ecc"].view(-1))}
    for k in (("m_q", "m_s", "v_q", "v_s") if adam else ("b_q", "b_s")):
        out[k] = to_host(st[k].view(-1))
    return out


def _check_initial_split(opt, params, x0):
    torch.cuda.synchronize()
    for i, p in enumerate(params):
        w_ref, e_ref = O.split_weights(x0[i])
        check_weights(f"initial split param {i}", to_host(p.data.view(-1)), to_host(opt.state[p]["ecc"].view(-1)),
                      w_ref, e_ref, "bf16", 8)


def _lockstep(model, opt, steps, hp_of, adam=True, tag="", codec="companded"):
    """Run `steps` optimizer steps; before each one the oracle takes a host
    copy of every parameter's state, and after it the states must match."""
    params = list(model.parameters())
    for step in range(1, steps + 1):
        opt.zero_grad(set_to_none=True)
        _loss(model, step).backward()
        grads = [to_host(p.grad.view(-1)) for p in params]
        before = [_host_state(opt, p, adam) for p in params]
        opt.step()
        torch.cuda.synchronize()
        for i, p in enumerate(params):
            hp = dict(hp_of(p), step=step)
            want = (O.adamw_step(before[i], grads[i], hp, codec=codec) if adam
                    else O.sgdm_step(before[i], grads[i], hp, codec=codec))
            check_state(f"{tag} step {step} param {i}", _host_state(opt, p, adam), want)


@pytest.mark.parametrize("cls", [FlashAdamW, FlashAdam])
def test_flash_adamw_matches_oracle_every_step(cls):
    model = _model()
    x0 = [p.detach().float().cpu().numpy().ravel().copy() for p in model.parameters()]
    opt = cls(model.parameters(), **HP)
    _check_initial_split(opt, list(model.parameters()), x0)
    hp = dict(lr=HP["lr"], beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, l2_decay=cls is FlashAdam)
    _lockstep(model, opt, 5, lambda p: hp, tag=cls.__name__)
    # master weights are the oracle's reconstruction of the stored split
    for p in model.parameters():
        mw = opt.master_weights(p).view(-1).cpu().numpy()
        want = O.reconstruct_weights(to_host(p.data.view(-1)), to_host(opt.state[p]["ecc"].view(-1)))
        assert np.array_equal(mw.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("extra", [{}, {"nesterov": True}, {"dampening": 0.3}, {"momentum": 0.0, "dampening": 0.5}])
def test_flash_sgd_matches_oracle_every_step(extra):
    model = _model(1)
    x0 = [p.detach().float().cpu().numpy().ravel().copy() for p in model.parameters()]
    kw = dict(dict(lr=0.05, momentum=0.9, weight_decay=1e-4), **extra)
    opt = FlashSGD(model.parameters(), **kw)
    _check_initial_split(opt, list(model.parameters()), x0)
    _lockstep(model, opt, 5, lambda p: kw, adam=False, tag=f"FlashSGD {extra}")


def test_flash_optimizers_with_bf16_block_scales():
    """The drop-in classes with codec="companded_bf16scale" (bfloat16 block
    scales) step like the oracle, AdamW and SGD."""
    model = _model(3)
    opt = FlashAdamW(model.parameters(), **HP, codec="companded_bf16scale")
    hp = dict(lr=HP["lr"], beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
    _lockstep(model, opt, 4, lambda p: hp, tag="FlashAdamW bf16 scales", codec="companded_bf16scale")
    model = _model(4)
    kw = dict(lr=0.05, momentum=0.9, weight_decay=1e-4)
    opt = FlashSGD(model.parameters(), **kw, codec="companded_bf16scale")
    _lockstep(model, opt, 4, lambda p: kw, adam=False, tag="FlashSGD bf16 scales", codec="companded_bf16scale")


def _train(model, opt, steps, start=1):
    for step in range(start, start + steps):
        opt.zero_grad(set_to_none=True)
        _loss(model, step).backward()
        opt.step()


def _snapshot(model, opt):
    out = [p.detach().clone() for p in model.parameters()]
    for p in model.parameters():
        out += [v.clone() for k, v in opt.state[p].items() if torch.is_tensor(v)]
    return out


@pytest.mark.parametrize("bucket", [1, 5000, 1 << 30])
def test_gradient_release_equals_plain_step(bucket):
    """Release in buckets (every parameter alone, flushes in the middle of
    backward, everything at the end-of-backward flush) is bitwise the plain
    step, and no gradient survives the backward pass."""
    a, b = _model(2), _model(2)
    oa = FlashAdamW(a.parameters(), **HP)
    ob = FlashAdamW(b.parameters(), **HP, grad_release=True, release_bucket=bucket)
    _train(a, oa, 4)
    _train(b, ob, 4)
    for p in b.parameters():
        assert p.grad is None                 # released
    for x, y in zip(_snapshot(a, oa), _snapshot(b, ob)):
        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8))


def test_state_dict_resume_is_bitwise():
    a = _model(3)
    oa = FlashAdamW(a.parameters(), **HP)
    _train(a, oa, 4)
    ref = _snapshot(a, oa)

    b = _model(3)
    ob = FlashAdamW(b.parameters(), **HP)
    _train(b, ob, 2)
    msd, osd = copy.deepcopy(b.state_dict()), copy.deepcopy(ob.state_dict())
    c = _model(99)                            # different init, then restored
    oc = FlashAdamW(c.parameters(), **HP)
    c.load_state_dict(msd)
    oc.load_state_dict(osd)
    _train(c, oc, 2, start=3)
    for x, y in zip(ref, _snapshot(c, oc)):
        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8))


def test_replaced_state_tensors_after_invalidate_launch_cache():
    """State tensors swapped by hand (clones at new addresses, the old ones
    freed) are picked up after invalidate_launch_cache(): the run stays bitwise
    equal to an untouched twin."""
    a, b = _model(5), _model(5)
    oa, ob = FlashAdamW(a.parameters(), **HP), FlashAdamW(b.parameters(), **HP)
    _train(a, oa, 2)
    _train(b, ob, 2)
    for p in b.parameters():
        st = ob.state[p]
        for k in ("ecc", "m_q", "m_s", "v_q", "v_s"):
            st[k] = st[k].clone()
    ob.invalidate_launch_cache()
    torch.cuda.synchronize()
    _train(a, oa, 2, start=3)
    _train(b, ob, 2, start=3)
    for x, y in zip(_snapshot(a, oa), _snapshot(b, ob)):
        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8))


def test_checkpoint_through_torch_save_and_safe_load_resumes_bitwise():
    """state_dict() written with torch.save and read back with
    torch.load(weights_only=True) (no unpickling of code) resumes bit for bit."""
    import io
    a = _model(7)
    oa = FlashAdamW(a.parameters(), **HP)
    _train(a, oa, 4)
    ref = _snapshot(a, oa)

    b = _model(7)
    ob = FlashAdamW(b.parameters(), **HP)
    _train(b, ob, 2)
    buf = io.BytesIO()
    torch.save({"model": b.state_dict(), "opt": ob.state_dict()}, buf)
    buf.seek(0)
    ck = torch.load(buf, weights_only=True, map_location="cuda")
    c = _model(98)
    oc = FlashAdamW(c.parameters(), **HP)
    c.load_state_dict(ck["model"])
    oc.load_state_dict(ck["opt"])
    _train(c, oc, 2, start=3)
    for x, y in zip(ref, _snapshot(c, oc)):
        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8))


def test_training_tracks_fp32_adamw():
    torch.manual_seed(5)
    w_true = torch.randn(64, 33, device="cuda") / 8
    ref = torch.nn.Linear(64, 33, bias=False).cuda()
    fl = copy.deepcopy(ref)
    o_ref = torch.optim.AdamW(ref.parameters(), lr=1e-2, weight_decay=0.0)
    o_fl = FlashAdamW(fl.parameters(), lr=1e-2, weight_decay=0.0)
    for i in range(200):
        x, _ = _batch(i, torch.float32)
        y = x @ w_true
        for m, o, dt in ((ref, o_ref, torch.float32), (fl, o_fl, torch.bfloat16)):
            o.zero_grad(set_to_none=True)
            loss = torch.nn.functional.mse_loss(m(x.to(dt)).float(), y)
            loss.backward()
            o.step()
    # compare the optimizers, not the bf16 forward pass: evaluate both in f32,
    # FlashAdamW through its reconstructed master weights
    w_fl = o_fl.master_weights(fl.weight)
    err_ref = (ref.weight.detach().T - w_true).norm() / w_true.norm()
    err_fl = (w_fl.T - w_true).norm() / w_true.norm()
    print(f"relative weight error after 200 steps: fp32 AdamW {err_ref:.3e}, FlashAdamW {err_fl:.3e}", flush=True)
    assert err_fl < 2e-2 and err_ref < 2e-2


def test_torch_state_import_export_round_trip():
    """Moments of a torch.optim.AdamW run, imported into FlashAdamW, come back
    out as the oracle's quantise -> dequantise of the same f32 values; the
    next step then matches the oracle started from those codes."""
    model = _model(4)
    tor = torch.optim.AdamW(model.parameters(), lr=1e-3, weight_decay=0.1)
    for step in range(1, 4):
        tor.zero_grad(set_to_none=True)
        x, y = _batch(step, torch.float32)
        torch.nn.functional.mse_loss(model(x), y).backward()
        tor.step()
    mom = {p: (tor.state[p]["exp_avg"].clone(), tor.state[p]["exp_avg_sq"].clone()) for p in model.parameters()}
    model.to(torch.bfloat16)                      # the parameters stay the same objects
    fl = FlashAdamW(model.parameters(), lr=1e-3, weight_decay=0.1)
    fl.import_torch_optimizer(tor)
    for p in model.parameters():
        assert fl.state[p]["step"] == 3
        m, v = fl.export_torch_state(p)
        for got, x, kind in ((m, mom[p][0], "m"), (v, mom[p][1], "v")):
            q, sc = O.quantize_state(x.float().cpu().numpy().ravel(), kind, "companded")
            want = O.dequantize_state(q, sc, kind, "companded")
            assert np.array_equal(got.cpu().numpy().ravel().view(np.uint32), want.view(np.uint32))
    sgd = FlashSGD(_model(5).parameters(), lr=0.1, momentum=0.9)
    p = next(iter(sgd.param_groups[0]["params"]))
    buf = torch.randn(p.shape, device="cuda") * 1e-2
    sgd.import_torch_state(p, buf, 7)
    q, sc = O.quantize_state(buf.cpu().numpy().ravel(), "m", "companded")
    assert np.array_equal(sgd.export_torch_state(p).cpu().numpy().ravel().view(np.uint32),
                          O.dequantize_state(q, sc, "m", "companded").view(np.uint32))


def test_param_groups_use_their_own_hyperparameters():
    """Weights and biases in separate groups (different lr, decay only on
    weights), as training scripts set them up: each group matches the oracle
    with its own hyperparameters at every step."""
    model = _model(6)
    params = list(model.parameters())
    groups = [{"params": [p for p in params if p.dim() > 1], "lr": 2e-3, "weight_decay": 0.1},
              {"params": [p for p in params if p.dim() == 1], "lr": 5e-3, "weight_decay": 0.0}]
    opt = FlashAdamW(groups, betas=(0.9, 0.95), eps=1e-8)
    group_of = {id(p): g for g in opt.param_groups for p in g["params"]}

    def hp_of(p):
        g = group_of[id(p)]
        return dict(lr=g["lr"], beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=g["weight_decay"])

    _lockstep(model, opt, 3, hp_of, tag="groups")


@pytest.mark.parametrize("release", [False, True], ids=["step", "grad_release"])
def test_native_row_marshalling_equals_python_marshalling(release):
    """The launch rows written by the host extension (lib/fo_marshal.so) and
    by the Python fallback drive the same steps: two copies of a model, one
    stepped with each, end bitwise equal.  In step() mode the last layer's
    bias is frozen (no gradient), so the extension first refuses the full
    list and then fills the rows of the list without it; gradient release
    steps buckets through the same rows."""
    import precision_optimizer_state_amd.optim as optim_mod
    if optim_mod._fill_rows is None:
        pytest.skip("the marshalling extension is not built")
    models, opts = [], []
    for native in (True, False):
        m = _model(5)
        if not release:
            m[2].bias.requires_grad_(False)
        models.append(m)
        opts.append(FlashAdamW(list(m.parameters()), **HP, grad_release=release, release_bucket=3000))
    saved = optim_mod._fill_rows
    try:
        for i in range(4):
            for native, (m, opt) in enumerate(zip(models, opts)):
                optim_mod._fill_rows = saved if native == 0 else None
                loss = _loss(m, i)
                loss.backward()
                if not release:
                    opt.step()
                opt.zero_grad(set_to_none=True)
    finally:
        optim_mod._fill_rows = saved
    torch.cuda.synchronize()
    for (na, pa), (nb, pb) in zip(models[0].named_parameters(), models[1].named_parameters()):
        assert torch.equal(pa.data.view(torch.int16), pb.data.view(torch.int16)), f"{na}: theta' differs"
        sa, sb = opts[0].state[pa], opts[1].state[pb]
        for k in ("ecc", "m_q", "m_s", "v_q", "v_s"):
            assert torch.equal(sa[k], sb[k]), f"{na}: {k} differs"
        assert sa["step"] == sb["step"]
    print(f"native and Python launch rows: 4 steps bitwise equal ({'gradient release' if release else 'step()'})",
          flush=True)
