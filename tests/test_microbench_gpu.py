"""GPU: the memory-path microbenchmarks of libmsda.so run and report plausible rates
for one MI355X (wide bounds: they catch a broken kernel or a wrong unit count, not a
slow GPU)."""
import pytest
import torch

import scale_deformable_attention_msda_amd as msda

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def buf():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    msda.load_library()
    b = torch.empty(2 ** 28, dtype=torch.uint8, device="cuda")
    yield b
    del b


@pytest.mark.parametrize("kind,span,lo,hi", [
    ("read", 0, 500e9, 9e12),                  # bytes/s
    ("copy", 0, 500e9, 9e12),
    ("atomic_f32", 2 ** 26, 10e9, 5e12),       # element adds/s
    ("atomic_f32", 2 ** 16, 1e9, 5e12),
    ("atomic_pk_bf16", 2 ** 26, 10e9, 5e12),   # pair adds/s
    ("gather_global", 2 ** 14, 1e12, 200e12),  # bytes/s
    ("gather_global", 2 ** 26, 1e12, 200e12),
    ("gather_lds", 0, 1e12, 400e12),
    ("lds_atomic_f32", 0, 1e10, 1e15),         # lane adds/s
])
def test_microbench_rates(buf, kind, span, lo, hi):
    ms, units = msda.msda_microbench_run(kind, buf, span=span, reps=3)
    rate = units / (ms * 1e-3)
    print(f"[microbench] {kind} span={span}: {ms:.4f} ms per launch, {rate:.4g} per s", flush=True)
    assert ms > 0 and units > 0
    assert lo < rate < hi, (kind, rate)
