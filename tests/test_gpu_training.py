"""GPU: the collection optimizers inside an autograd training loop.

A small MLP is trained on a fixed synthetic regression task. The gradients
come from backward() into the .grad buffers that the optimizer captured
when it was built. AdamW32 follows torch.optim.AdamW: both compute the
textbook AdamW, and the placements of eps and of the bias corrections are
algebraically equal, so the parameters agree to rounding level after 30
steps. That is a check of the training-loop wiring (Parameters, captured
gradients, step counting, graph replay), not of the arithmetic, which the
parity tests pin bitwise to the oracle. AdamW8bit must reduce the loss.
"""
import pytest
import torch

pytestmark = pytest.mark.gpu

STEPS = 30


def _model(seed):
    torch.manual_seed(seed)
    return torch.nn.Sequential(torch.nn.Linear(64, 256), torch.nn.GELU(), torch.nn.Linear(256, 256),
                               torch.nn.GELU(), torch.nn.Linear(256, 8)).cuda()


def _data():
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    x = torch.randn(512, 64, device="cuda", generator=gen)
    w = torch.randn(64, 8, device="cuda", generator=gen) / 8
    return x, torch.tanh(x @ w)


def _train(model, step, steps=STEPS):
    x, y = _data()
    losses = []
    for _ in range(steps):
        model.zero_grad(set_to_none=False)   # the optimizer holds these buffers
        loss = torch.nn.functional.mse_loss(model(x), y)
        loss.backward()
        step()
        losses.append(loss.item())
    return losses


@pytest.mark.parametrize("graph", [False, True])
def test_adamw32_follows_torch_adamw(graph):
    """The same model, data and hyperparameters: AdamW32 (plan launch or graph
    replay) and torch.optim.AdamW end within 2e-5 of each other, relative to
    each parameter tensor's scale, and the loss falls."""
    import optimizer_update_amd as ou
    a, b = _model(0), _model(0)
    opt_a = ou.AdamW32(list(a.parameters()), lr=3e-3, weight_decay=0.01)
    opt_b = torch.optim.AdamW(b.parameters(), lr=3e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01,
                              foreach=False)
    la = _train(a, lambda: opt_a.step(graph=graph))
    lb = _train(b, opt_b.step)
    torch.cuda.synchronize()
    assert opt_a.step_count == STEPS
    assert la[-1] < 0.5 * la[0], la
    for (name, pa), pb in zip(a.named_parameters(), b.parameters()):
        scale = pb.detach().abs().max().item()
        err = (pa.detach() - pb.detach()).abs().max().item()
        assert err <= 2e-5 * scale, (name, err, scale)
    assert abs(la[-1] - lb[-1]) <= 1e-3 * lb[-1], (la[-1], lb[-1])
    opt_a.close()


def test_adamw8bit_trains():
    """AdamW8bit over the same MLP (the 256x256 weight and the first layer's
    weight keep 8-bit states, the rest fp32 states): the loss falls about as
    fast as with 32-bit states."""
    import optimizer_update_amd as ou
    a, b = _model(1), _model(1)
    opt8 = ou.AdamW8bit(list(a.parameters()), lr=3e-3, weight_decay=0.01, min_8bit_size=4096)
    opt32 = ou.AdamW32(list(b.parameters()), lr=3e-3, weight_decay=0.01)
    l8 = _train(a, opt8.step)
    l32 = _train(b, opt32.step)
    torch.cuda.synchronize()
    assert l8[-1] < 0.5 * l8[0], l8
    assert l8[-1] < 1.5 * l32[-1], (l8[-1], l32[-1])
    opt8.close()
    opt32.close()


@pytest.mark.parametrize("which", ["adamw32", "adamw8bit"])
def test_set_to_none_gradients_are_followed(which):
    """torch's default zero_grad(set_to_none=True) makes every backward
    allocate new .grad tensors.  The optimizer notices at the next step
    (the captured tensor is no longer the Parameter's .grad), rebuilds its
    plan on the new buffers and trains as with in-place zeroing: the
    parameters agree within 1e-4 of each tensor's scale after the same
    steps (the backward's GEMMs need not be bitwise repeatable; a step on
    stale or freed gradient buffers would be off by orders more)."""
    import optimizer_update_amd as ou
    make = {"adamw32": lambda ps: ou.AdamW32(ps, lr=3e-3, weight_decay=0.01),
            "adamw8bit": lambda ps: ou.AdamW8bit(ps, lr=3e-3, weight_decay=0.01, min_8bit_size=4096)}[which]
    a, b = _model(2), _model(2)
    opt_a, opt_b = make(list(a.parameters())), make(list(b.parameters()))
    x, y = _data()
    for _ in range(6):
        a.zero_grad(set_to_none=True)          # new .grad tensors at the next backward
        torch.nn.functional.mse_loss(a(x), y).backward()
        opt_a.step()
        opt_b.zero_grad()                      # the optimizer's own, in place
        torch.nn.functional.mse_loss(b(x), y).backward()
        opt_b.step()
    torch.cuda.synchronize()
    for pa, pb in zip(a.parameters(), b.parameters()):
        scale = pb.detach().abs().max().item()
        assert (pa.detach() - pb.detach()).abs().max().item() <= 1e-4 * scale
    a.zero_grad(set_to_none=True)
    with pytest.raises(RuntimeError, match="no .grad"):
        opt_a.step()
    opt_a.close()
    opt_b.close()
