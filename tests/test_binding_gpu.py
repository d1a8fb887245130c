"""The binding rejects caller-supplied buffers that do not match what the
kernels write (out, final_state, workspace) and tensors on another device,
with a ValueError raised before anything is enqueued."""
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_80_amd as K
    K.lib()


def prefill_inputs(B=1, T=70, H=2, d=128):
    gen = torch.Generator(device="cuda").manual_seed(5)
    q = torch.randn(B, T, H, d, generator=gen, device="cuda").to(torch.bfloat16)
    k = torch.nn.functional.normalize(torch.randn(B, T, H, d, generator=gen, device="cuda"),
                                      dim=-1).to(torch.bfloat16)
    v = torch.randn(B, T, H, d, generator=gen, device="cuda").to(torch.bfloat16)
    g = -0.1 * torch.rand(B, T, H, d, generator=gen, device="cuda")
    beta = torch.rand(B, T, H, generator=gen, device="cuda")
    return q, k, v, g, beta


BF, F32, U8 = torch.bfloat16, torch.float32, torch.uint8
# keyword -> a buffer the kernels cannot write (made on the device unless named "host")
BAD_PREFILL = {
    "out shape": lambda: dict(out=torch.empty(1, 70, 2, 64, dtype=BF, device="cuda")),
    "out dtype": lambda: dict(out=torch.empty(1, 70, 2, 128, dtype=F32, device="cuda")),
    "out on host": lambda: dict(out=torch.empty(1, 70, 2, 128, dtype=BF)),
    "out strided": lambda: dict(out=torch.empty(1, 70, 2, 256, dtype=BF, device="cuda")[..., :128]),
    "final_state dtype": lambda: dict(final_state=torch.empty(1, 2, 128, 128, dtype=BF,
                                                              device="cuda")),
    "final_state shape": lambda: dict(final_state=torch.empty(2, 2, 128, 128, device="cuda")),
    "workspace dtype": lambda: dict(workspace=torch.empty(1 << 20, dtype=F32, device="cuda")),
    "workspace on host": lambda: dict(workspace=torch.empty(1 << 20, dtype=U8)),
}


@pytest.mark.parametrize("case", sorted(BAD_PREFILL))
def test_prefill_rejects_mismatched_buffers(case):
    import gated_delta_rule_80_amd as K
    q, k, v, g, beta = prefill_inputs()
    with pytest.raises(ValueError):
        K.chunk_fwd(q, k, v, g, beta, **BAD_PREFILL[case]())


def test_prefill_rejects_an_input_on_the_host():
    import gated_delta_rule_80_amd as K
    q, k, v, g, beta = prefill_inputs()
    with pytest.raises(ValueError):
        K.chunk_fwd(q, k, v, g, beta.cpu())
    with pytest.raises(ValueError):
        K.chunk_fwd(q, k, v, g, beta, initial_state=torch.zeros(1, 2, 128, 128))


def test_decode_and_output_stage_reject_mismatched_out():
    import gated_delta_rule_80_amd as K
    N, H, d = 4, 2, 128
    q = torch.randn(N, H, d, device="cuda").to(torch.bfloat16)
    g = torch.zeros(N, H, d, device="cuda")
    beta = torch.rand(N, H, device="cuda")
    st = torch.zeros(N, H, d, d, device="cuda")
    with pytest.raises(ValueError):
        K.decode_step(q, q, q, g, beta, st, out=torch.empty(N, H, d, device="cuda"))
    with pytest.raises(ValueError):
        K.decode_step(q, q, q, g, beta, st, out=torch.empty(N, H, d, dtype=torch.bfloat16))
    o = torch.randn(10, d, device="cuda")
    w = torch.ones(d, device="cuda")
    with pytest.raises(ValueError):
        K.output_rmsnorm_gate(o, o, w, out=torch.empty(10, d))
    with pytest.raises(ValueError):
        K.output_rmsnorm_gate(o, o, w.cpu())


def test_backward_rejects_a_host_workspace():
    import gated_delta_rule_80_amd as K
    B, T, H, d = 1, 40, 2, 32
    x = [torch.randn(B, T, H, d, device="cuda") for _ in range(4)]
    g = -0.1 * torch.rand(B, T, H, d, device="cuda")
    beta = torch.rand(B, T, H, device="cuda")
    with pytest.raises(ValueError):
        K.chunk_bwd(x[0], x[1], x[2], g, beta, x[3], chunk_size=32,
                    workspace=torch.empty(1 << 20, dtype=torch.uint8))
