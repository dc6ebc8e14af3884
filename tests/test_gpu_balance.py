"""Parity of the routing bias update (moe_expert_load, moe_bias_update) with
the CPU oracle, through the C ABI.  Both are integer decisions and one fp32
addition, so the GPU results must equal the oracle's bit for bit: at the
Kimi K2 prefill shape (8,192 tokens x 8 choices over 384 experts, the batch
the benchmark times), at the largest expert count the library takes (1,024,
top-32) and at the smallest."""
import numpy as np
import pytest
import torch

import synth
from oracle import balance_ref as B

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_moe_transformer_sigmoid_amd import _lib
    _lib.load()          # raises if libk2moe.so is missing: no fallback path
    yield
    torch.cuda.synchronize()


def _layer_cfg(E, k):
    """A config with E routed experts and top-k (the entry points read only those)."""
    from sparse_moe_transformer_sigmoid_amd import _lib as L
    from sparse_moe_transformer_sigmoid_amd.layer import config_from_shape
    if E == 384 and k == 8:
        shape = synth.K2_PREFILL
    else:
        shape = synth.small_fp8(tokens=16, d_model=256, n_experts=E, n_shared=1, top_k=k, d_ff=128)
    return L, config_from_shape(shape)


def _expert_load(E, k, ids, counts):
    import ctypes as C
    L, cfg = _layer_cfg(E, k)
    L.call("moe_expert_load", C.byref(cfg), ids.shape[0], ids.data_ptr(), counts.data_ptr(),
           C.c_void_p(torch.cuda.current_stream().cuda_stream))


def _bias_update(E, k, counts, speed, bias):
    import ctypes as C
    L, cfg = _layer_cfg(E, k)
    L.call("moe_bias_update", C.byref(cfg), counts.data_ptr(), C.c_float(speed), bias.data_ptr(),
           C.c_void_p(torch.cuda.current_stream().cuda_stream))


@pytest.mark.parametrize("T,k,E,skew", [
    (8192, 8, 384, 0.5),       # K2 prefill batch
    (8192, 8, 384, 1.5),       # one expert picked by most tokens
    (64, 8, 384, 0.0),         # K2 decode batch, most experts unpicked
    (4096, 32, 1024, 1.0),     # largest expert count and top-k
    (1, 1, 16, 0.0),
    (3000, 4, 16, 0.3),        # few experts: heavy LDS-atomic contention
])
def test_expert_load_exact(T, k, E, skew):
    ids = synth.topk_choices(T, k, E, seed=T + E, skew=skew)
    ids2 = synth.topk_choices(T, k, E, seed=T + E + 1, skew=skew)
    want = B.expert_load(ids.numpy(), E)
    counts = torch.zeros(E, dtype=torch.int32, device="cuda")
    _expert_load(E, k, ids.cuda(), counts)
    torch.cuda.synchronize()
    assert np.array_equal(counts.cpu().numpy(), want)
    # a second micro-batch accumulates into the same counts
    _expert_load(E, k, ids2.cuda(), counts)
    torch.cuda.synchronize()
    assert np.array_equal(counts.cpu().numpy(), want + B.expert_load(ids2.numpy(), E))


def test_expert_load_skips_ids_outside_the_layer_and_zero_tokens():
    T, k, E = 2048, 8, 384
    ids = synth.topk_choices(T, k, E, seed=7, skew=0.5).clone()
    ids[::5, 0] = -1              # not a routed expert of this layer
    ids[::7, 3] = E
    ids[::11, 7] = 1 << 30
    counts = torch.zeros(E, dtype=torch.int32, device="cuda")
    _expert_load(E, k, ids.cuda(), counts)
    torch.cuda.synchronize()
    assert np.array_equal(counts.cpu().numpy(), B.expert_load(ids.numpy(), E))
    before = counts.clone()
    _expert_load(E, k, ids[:0].cuda(), counts)
    torch.cuda.synchronize()
    assert torch.equal(counts, before)


@pytest.mark.parametrize("E,k,mean,spread", [(384, 8, 170, 150), (1024, 32, 5000, 4000),
                                              (16, 1, 3, 2)])
@pytest.mark.parametrize("speed", [1e-3, 2.0 ** -10, 2.0 ** -30, 0.0])
def test_bias_update_exact(E, k, mean, spread, speed):
    counts = synth.expert_loads(E, mean, spread, seed=E)
    bias = synth.bias_values(E, seed=E)
    want = B.bias_update(bias.numpy(), counts.numpy(), speed)
    b = bias.cuda()
    _bias_update(E, k, counts.cuda(), speed, b)
    torch.cuda.synchronize()
    got = b.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    if speed > 0:      # all three directions occurred
        assert set(B.load_direction(counts.numpy()).tolist()) == {-1, 0, 1}


def test_bias_update_near_fp32_limits():
    """Loads beyond fp32's integer range and biases where the update rounds."""
    E, k = 16, 2
    base = 1 << 26
    counts = torch.tensor([base + 1, base - 1] + [base] * 14, dtype=torch.int32)
    bias = torch.tensor([1.0, 1.0 + 2.0 ** -23, -0.0, 2.0 ** -126] + [0.5] * 12,
                        dtype=torch.float32)
    for speed in (2.0 ** -24, 2.0 ** -25, 3.0):
        want = B.bias_update(bias.numpy(), counts.numpy(), speed)
        b = bias.cuda()
        _bias_update(E, k, counts.cuda(), speed, b)
        torch.cuda.synchronize()
        assert np.array_equal(b.cpu().numpy().view(np.uint32), want.view(np.uint32)), speed


def test_one_training_step_in_the_k2_prefill_shape():
    """Two micro-batches of K2 prefill choices, then the update, against the
    oracle's composition of the same steps."""
    E, k = 384, 8
    bias = synth.bias_values(E, seed=3)
    batches = [synth.topk_choices(8192, k, E, seed=s, skew=0.7) for s in (11, 12)]
    counts = torch.zeros(E, dtype=torch.int32, device="cuda")
    for ids in batches:
        _expert_load(E, k, ids.cuda(), counts)
    b = bias.cuda()
    _bias_update(E, k, counts, 1e-3, b)
    torch.cuda.synchronize()
    c = sum(B.expert_load(ids.numpy(), E) for ids in batches)
    want = B.bias_update(bias.numpy(), c, 1e-3)
    assert np.array_equal(b.cpu().numpy().view(np.uint32), want.view(np.uint32))
