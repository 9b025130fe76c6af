"""Layer-level forward + backward: the projections of a multi-scale deformable
attention layer around the library's softmax-method kernels, against the same
layer with the operator composed from torch.softmax and F.grid_sample, run on
the CPU in fp64 with the same parameters and inputs.  Outputs and every
gradient (parameters, queries, value features) are compared."""
import copy

import numpy as np
import pytest
import torch

import bench
import workloads
from parity import check, say
from scale_deformable_attention_msda_amd.layer import MultiScaleDeformAttn

pytestmark = pytest.mark.gpu

PYR = ((20, 30), (10, 15), (5, 8))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("B,M,K,scatter", [(2, 4, 4, "binned"), (1, 8, 2, "binned"),
                                           (2, 4, 4, "atomic")])
def test_layer_matches_grid_sample_composition(B, M, K, scatter):
    D, L = 32, len(PYR)
    C = M * D
    S = sum(h * w for h, w in PYR)
    say(f"[layer] B={B} Q=S={S} dim={C} heads={M} levels={L} points={K} scatter={scatter}")
    torch.manual_seed(B * 100 + M * 10 + K)
    gpu = MultiScaleDeformAttn(C, M, L, K, scatter=scatter).cuda()
    with torch.no_grad():  # offsets of a few pixels, so points spread over cells and edges
        gpu.sampling_offsets.weight.mul_(4.0)
    cpu = copy.deepcopy(gpu).cpu().double()
    cpu.sampler = bench.grid_sample_msda_softmax  # the same parameters, composed from torch ops
    gen = torch.Generator().manual_seed(7)
    query = torch.randn(B, S, C, generator=gen)
    value = torch.randn(B, S, C, generator=gen)
    gout = torch.randn(B, S, C, generator=gen)
    ref = torch.from_numpy(workloads.pixel_centre_refs(PYR)).float()[None, :, None, :]
    ref = ref.expand(B, S, L, 2).contiguous()
    host = np.asarray(PYR, dtype=np.int64)
    starts = workloads.level_start_index(PYR)

    def run(layer, dev, dt):
        q = query.to(dev, dt).requires_grad_()
        v = value.to(dev, dt).requires_grad_()
        out = layer(q, ref.to(dev, dt), v, torch.from_numpy(host).to(dev),
                    torch.from_numpy(starts).to(dev), host)
        out.backward(gout.to(dev, dt))
        grads = {n: p.grad.double().cpu().numpy() for n, p in layer.named_parameters()}
        grads["query"] = q.grad.double().cpu().numpy()
        grads["value"] = v.grad.double().cpu().numpy()
        return out.detach().double().cpu().numpy(), grads

    out_g, grads_g = run(gpu, "cuda", torch.float32)
    torch.cuda.synchronize()
    out_c, grads_c = run(cpu, "cpu", torch.float64)
    check("out", out_g, out_c, 1e-4, 1e-5)
    for name in grads_c:
        # parameter gradients sum over every query: scale atol by the reference's size
        scale = max(1.0, float(np.abs(grads_c[name]).max()))
        check(f"grad {name}", grads_g[name], grads_c[name], 1e-4, 1e-5 * scale)
