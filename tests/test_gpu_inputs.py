"""GPU parity for every kind of input the C ABI accepts beyond the fixed and fuzz
shapes: num_blocks up to the maximum of 16 (in bf16 the forward merges the
diagonal blocks in groups of 8, so 9..16 run a second, partly filled group),
k/v tensors passed through batch and block strides (a [B, nb, T, H, D] cache
with no copy), the autograd wrapper in its list and stacked forms, score rows
with a wide range (the forward's lazily moved running max must rescale in the
middle of the key walk) and rows dominated by their diagonal blocks. Each case
is compared with the CPU oracle on the same inputs at the parity tolerances."""
import numpy as np
import pytest
import torch

import eagle_draft_amd as e3
import synth
from tests.parity import assert_within, compare, run_hip, run_oracle, say

pytestmark = pytest.mark.gpu

W = synth.small_workload


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("nb", [9, 10, 12, 16])
def test_many_blocks(dtype, nb):
    D = 128 if dtype == "bf16" else 64
    w = W(dtype=dtype, S=300, H=2, D=D, num_blocks=nb, seed=nb)
    say(f"[inputs] num_blocks={nb} {dtype}: {w}")
    inp = synth.make_inputs(w)
    m = compare(w, run_hip(w, inp), run_oracle(w, inp))
    say(f"[inputs] num_blocks={nb} {dtype}: {m}")
    assert_within(w, m)


def _stacked(inp):
    """[B, nb, T, H, D] caches holding block 0 then the diagonal blocks."""
    ck = torch.cat([inp["k0"].unsqueeze(1), inp["kd"]], 1).contiguous()
    cv = torch.cat([inp["v0"].unsqueeze(1), inp["vd"]], 1).contiguous()
    return ck, cv


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_strided_cache_through_the_abi(dtype):
    """k0 = cache[:, 0], kd = cache[:, 1:] passed with k0_batch_stride =
    kd_batch_stride = nb*T*H*D and kd_block_stride = T*H*D; the gradients are
    written through the same strides into one cache-shaped buffer."""
    D = 128 if dtype == "bf16" else 64
    w = W(dtype=dtype, B=2, S=260, H=3, D=D, num_blocks=5, seed=7)
    say(f"[inputs] strided cache {dtype}: {w}")
    inp = synth.make_inputs(w)
    ck, cv = _stacked(inp)
    B, nb, T, H, _ = ck.shape
    blk = nb * T * H * D
    prob = e3.Problem(B, T, T, H, D, nb, w.scale, dtype=w.torch_dtype, device="cuda",
                      k0_batch_stride=blk, kd_batch_stride=blk, kd_block_stride=T * H * D)
    ck, cv = ck.cuda(), cv.cuda()
    q, dout = inp["q"].cuda(), inp["dout"].cuda()
    out, lse = e3.fwd(prob, q, ck[:, 0], cv[:, 0], ck[:, 1:], cv[:, 1:])
    dck = torch.full_like(ck, float("nan"))
    dcv = torch.full_like(cv, float("nan"))
    grads = (torch.empty_like(q), dck[:, 0], dcv[:, 0], dck[:, 1:], dcv[:, 1:])
    dq, _, _, _, _ = e3.bwd(prob, dout, q, ck[:, 0], cv[:, 0], ck[:, 1:], cv[:, 1:], out, lse,
                            grads=grads)
    torch.cuda.synchronize()
    assert torch.isfinite(dck).all() and torch.isfinite(dcv).all()   # every element written
    hip = (out.cpu(), lse.cpu(), [dq.cpu(), dck[:, 0].cpu(), dcv[:, 0].cpu(),
                                  dck[:, 1:].cpu(), dcv[:, 1:].cpu()])
    m = compare(w, hip, run_oracle(w, inp))
    say(f"[inputs] strided cache {dtype}: {m}")
    assert_within(w, m)


@pytest.mark.parametrize("form", ["list", "stacked"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_cached_attention_autograd(form, dtype):
    """One forward and backward through torch.autograd, compared with the
    oracle's gradients of sum(out * dout)."""
    D = 128 if dtype == "bf16" else 64
    w = W(dtype=dtype, B=2, S=200, H=2, D=D, num_blocks=4, seed=11)
    say(f"[inputs] cached_attention {form} {dtype}: {w}")
    inp = synth.make_inputs(w)
    q = inp["q"].cuda().requires_grad_()
    if form == "list":
        ks = [inp["k0"]] + [inp["kd"][:, i] for i in range(w.N)]
        vs = [inp["v0"]] + [inp["vd"][:, i] for i in range(w.N)]
        ks = [k.cuda().contiguous().requires_grad_() for k in ks]
        vs = [v.cuda().contiguous().requires_grad_() for v in vs]
        out = e3.cached_attention(q, ks, vs, w.scale)
        out.backward(inp["dout"].cuda())
        dk = torch.stack([k.grad for k in ks], 1)
        dv = torch.stack([v.grad for v in vs], 1)
    else:
        ck, cv = _stacked(inp)
        ck = ck.cuda().requires_grad_()
        cv = cv.cuda().requires_grad_()
        out = e3.cached_attention(q, ck, cv, w.scale)
        out.backward(inp["dout"].cuda())
        dk, dv = ck.grad, cv.grad
    torch.cuda.synchronize()
    ref = run_oracle(w, inp)
    lse_ref = torch.from_numpy(ref[1]).float()     # autograd returns out only
    hip = (out.detach().cpu(), lse_ref, [q.grad.cpu(), dk[:, 0].cpu(), dv[:, 0].cpu(),
                                         dk[:, 1:].cpu(), dv[:, 1:].cpu()])
    m = compare(w, hip, ref)
    say(f"[inputs] cached_attention {form} {dtype}: {m}")
    assert_within(w, m)


def test_cached_attention_zigzag_share_with_stacked_cache():
    """A ring share through the stacked form: block 0 comes in separately (the
    full sequence), the cache holds the local diagonal blocks."""
    w = W(S=1024, H=2, D=128, num_blocks=3, layout="zigzag", cp=4, rank=1, seed=3)
    inp = synth.make_inputs(w)
    ck, cv = _stacked({"k0": torch.zeros_like(inp["q"]), "v0": torch.zeros_like(inp["q"]),
                       "kd": inp["kd"], "vd": inp["vd"]})
    q = inp["q"].cuda().requires_grad_()
    k0 = inp["k0"].cuda().requires_grad_()
    v0 = inp["v0"].cuda().requires_grad_()
    ck = ck.cuda().requires_grad_()
    cv = cv.cuda().requires_grad_()
    out = e3.cached_attention(q, ck, cv, w.scale, layout="zigzag", cp=4, rank=1, k0=k0, v0=v0)
    out.backward(inp["dout"].cuda())
    torch.cuda.synchronize()
    assert torch.count_nonzero(ck.grad[:, 0]) == 0 and torch.count_nonzero(cv.grad[:, 0]) == 0
    ref = run_oracle(w, inp)
    hip = (out.detach().cpu(), torch.from_numpy(ref[1]).float(),
           [q.grad.cpu(), k0.grad.cpu(), v0.grad.cpu(), ck.grad[:, 1:].cpu(), cv.grad[:, 1:].cpu()])
    m = compare(w, hip, ref)
    say(f"[inputs] cached_attention zigzag: {m}")
    assert_within(w, m)


def _scaled(t, f):
    return (t.float() * f).to(t.dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("layout", ["full", "zigzag"])
def test_wide_score_range(dtype, layout):
    """q scaled by 6 (bf16) or 2 (float32) and every 97th block-0 key by 4: scores
    span tens of log2 units and the largest ones lie late in the key walk, so the
    forward's running max (moved only when a row max grows by more than 2^8) is
    moved in the middle of the loop, and the backward's probabilities are nearly
    one-hot. float32 uses the smaller factor because its tolerance is an absolute
    1e-5 on out and lse: with q x 6 the scores reach about 150, where one float32
    ulp is already 1.5e-5, so the bar would measure the rounding of the scores
    themselves rather than the kernels (x 2 still gives scores of about 25)."""
    D = 128 if dtype == "bf16" else 64
    if layout == "full":
        w = W(dtype=dtype, S=700, H=2, D=D, num_blocks=4, seed=21, doc_lens=[250, 450])
    else:
        w = W(dtype=dtype, S=768, H=2, D=D, num_blocks=3, seed=21, layout="zigzag", cp=3, rank=1)
    inp = synth.make_inputs(w)
    inp["q"] = _scaled(inp["q"], 6.0 if dtype == "bf16" else 2.0)
    k0 = inp["k0"].float()
    k0[:, 96::97] *= 4.0
    inp["k0"] = k0.to(inp["k0"].dtype)
    m = compare(w, run_hip(w, inp), run_oracle(w, inp))
    say(f"[inputs] wide scores {dtype} {layout}: {m}")
    assert_within(w, m)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_diagonal_dominant_rows(dtype):
    """kd_i = q for every block: the diagonal scores scale*|q|^2 (about 11 for
    D = 128) dominate every row, so the epilogue's merge moves the running max
    and block 0 carries probabilities of order e^-11."""
    D = 128 if dtype == "bf16" else 64
    w = W(dtype=dtype, S=333, H=2, D=D, num_blocks=5, seed=31)
    inp = synth.make_inputs(w)
    inp["kd"] = inp["q"].unsqueeze(1).expand(-1, w.N, -1, -1, -1).contiguous()
    m = compare(w, run_hip(w, inp), run_oracle(w, inp))
    say(f"[inputs] diagonal-dominant {dtype}: {m}")
    assert_within(w, m)
