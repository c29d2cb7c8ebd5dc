"""The C-ABI library loads without a GPU, exports every function the header
declares, and validates arguments on the host before any HIP call."""
import ctypes
import os
import re

import pytest

from gated_delta_rule_85_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdr.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(binding.LIB_PATH):
        pytest.skip("libgdr.so not built (run __graft_entry__.build())")
    return binding.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdr_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("gdr_forward_chunked", "gdr_decode_step", "gdr_forward_workspace_size",
              "gdr_check_args", "gdr_status_string", "gdr_last_error_detail",
              "gdr_backward_chunked", "gdr_backward_workspace_size", "gdr_forward_chunked_noalloc",
              "gdr_forward_chunked_save", "gdr_backward_chunked_saved"):
        assert n in names


def test_every_declared_symbol_is_exported(L):
    for n in declared_functions():
        assert hasattr(L, n), n


def test_struct_layout_matches_header():
    # int32 x2, int64 x5, int32 x2, pointers x7, float x2, pointers x5
    assert ctypes.sizeof(binding.GdrArgs) == 8 + 40 + 8 + 7 * 8 + 8 + 5 * 8
    assert binding.GdrArgs.v_route.offset == 144 and binding.GdrArgs.delta_out.offset == 152
    assert binding.GdrArgs.q.offset == 56
    assert binding.GdrArgs.eps.offset == 112


def _args(name="gated_deltanet", B=2, T=100, H=3, dk=128, dv=64, dtype=binding.GDR_BF16,
          **over):
    variant = name
    v = binding.VARIANTS[variant]
    a = binding.GdrArgs(v, dtype, B, T, H, dk, dv, 0, 0, 0x1000, 0x2000, 0x3000,
                        0x4000 if variant != "deltanet" else None,
                        0x5000 if variant != "gdn2" else None,
                        0x6000 if variant == "gdn2" else None,
                        0x7000 if variant == "gdn2" else None,
                        1e-6 if variant == "kla" else 0.0, 0.0, None, 0x8000, 0x9000, None, None)
    for key, val in over.items():
        setattr(a, key, val)
    return a


@pytest.mark.parametrize("variant", list(binding.VARIANTS))
def test_valid_arguments_pass(L, variant):
    assert binding.gdr_check_args(_args(variant), 0) == 0


@pytest.mark.parametrize("over,status", [
    (dict(variant=7), 1), (dict(dtype=5), 1), (dict(B=0), 1), (dict(T=0), 1),
    (dict(H=-1), 1), (dict(dk=96), 2), (dict(dv=32), 2), (dict(chunk=32), 2),
    (dict(B=65536), 2), (dict(B=4097, H=4096), 2), (dict(T=(1 << 31) + 1), 2),
    (dict(q=None), 1), (dict(o=None), 1), (dict(alpha=None), 1), (dict(beta=None), 1),
    (dict(erase_b=0xa000), 1), (dict(q=0x1004), 1), (dict(state_in=0x100c), 1),
    (dict(o=0x1000), 1), (dict(flags=4), 1), (dict(flags=-1), 1), (dict(decay_scale=1.0), 1),
    (dict(flags=2, decay_scale=0.0), 1), (dict(flags=2, decay_scale=-1.0), 1),
    (dict(flags=2, decay_scale=float("inf")), 1), (dict(flags=2, decay_scale=float("nan")), 1),
])
def test_invalid_arguments_rejected(L, over, status):
    a = _args(**over)
    assert binding.gdr_check_args(a, 0) == status
    assert binding.gdr_last_error_detail() != ""
    # The entry points reject the same call before touching the GPU.
    assert binding.gdr_forward_chunked(a, 0x10000, 1 << 30, 0) == status
    assert binding.gdr_forward_chunked_noalloc(a, 0) == status


def test_noalloc_workspace_limit_matches_header():
    m = re.search(r"#define GDR_NOALLOC_WORKSPACE_MAX \(\(size_t\)(\d+) << (\d+)\)",
                  open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == binding.NOALLOC_WORKSPACE_MAX


@pytest.mark.parametrize("variant", list(binding.VARIANTS))
def test_input_transform_flags(L, variant):
    """q/k normalisation needs nothing else; activated gates need a positive,
    finite decay scale exactly when the variant decays."""
    assert binding.gdr_check_args(_args(variant, flags=binding.GDR_FLAG_QK_L2NORM), 0) == 0
    raw = binding.GDR_FLAG_RAW_GATES | binding.GDR_FLAG_QK_L2NORM
    if variant == "deltanet":
        assert binding.gdr_check_args(_args(variant, flags=raw), 0) == 0
        assert binding.gdr_check_args(_args(variant, flags=raw, decay_scale=0.5), 0) == 1
    else:
        assert binding.gdr_check_args(_args(variant, flags=raw, decay_scale=0.5), 0) == 0
        assert binding.gdr_check_args(_args(variant, flags=raw), 0) == 1
    a = _args(variant, flags=raw, decay_scale=0.0 if variant == "deltanet" else 0.5, T=1,
              state_in=0xa000)
    assert binding.gdr_check_args(a, 1) == 0


def test_variant_specific_pointers(L):
    assert binding.gdr_check_args(_args("deltanet", alpha=0x4000), 0) == 1
    assert binding.gdr_check_args(_args("gdn2", beta=0x5000), 0) == 1
    assert binding.gdr_check_args(_args("gdn2", write_w=None), 0) == 1
    assert binding.gdr_check_args(_args("kla", eps=-1.0), 0) == 1


def test_decode_validation(L):
    a = _args(T=1, state_in=0x8000)
    assert binding.gdr_check_args(a, 1) == 0
    assert binding.gdr_check_args(_args(T=2, state_in=0x8000), 1) == 1
    assert binding.gdr_check_args(_args(T=1, state_in=None), 1) == 1
    assert binding.gdr_check_args(_args(T=1, state_in=0x8000, state_out=None), 1) == 1
    assert binding.gdr_decode_step(_args(T=2, state_in=0x8000), 0) == 1


def test_workspace_size_and_errors(L):
    a = _args(B=2, T=100, H=3, dk=128, dv=64)
    n = binding.gdr_forward_workspace_size(a)
    nch = 2 * 3 * 2  # two chunks of 64 per head
    per_chunk = 2 * (64 * 128 * 3 + 64 * 64 + 64 * 64) + 4 * 128  # bf16 factors + gammas
    assert nch * per_chunk <= n <= nch * per_chunk + 6 * 256
    assert binding.gdr_forward_workspace_size(_args(dk=96)) == 0
    assert binding.gdr_forward_chunked(a, None, n, 0) == 3
    assert binding.gdr_forward_chunked(a, 0x10080, n, 0) == 3     # misaligned
    assert binding.gdr_forward_chunked(a, 0x10000, n - 1, 0) == 3  # too small
    f32 = _args(B=2, T=100, H=3, dk=128, dv=64, dtype=binding.GDR_F32)
    assert binding.gdr_forward_workspace_size(f32) >= 2 * nch * per_chunk - 4 * 128 * nch


def test_status_strings(L):
    for code, name in binding.STATUS.items():
        assert binding.gdr_status_string(code) == name
    assert "unknown" in binding.gdr_status_string(99)


def _grads(variant="gated_deltanet", **over):
    g = binding.GdrGrads(0x11000, 0x12000, 0x13000, 0x14000, 0x15000,
                         0x16000 if variant != "deltanet" else None,
                         0x17000 if variant != "gdn2" else None,
                         0x18000 if variant == "gdn2" else None,
                         0x19000 if variant == "gdn2" else None, 0x1a000)
    for key, val in over.items():
        setattr(g, key, val)
    return g


def test_grads_struct_layout():
    assert ctypes.sizeof(binding.GdrGrads) == 10 * 8
    assert binding.GdrGrads.d_q.offset == 16
    assert binding.GdrGrads.d_state_in.offset == 72


@pytest.mark.parametrize("variant", list(binding.VARIANTS))
def test_backward_validation(L, variant):
    """The gradient takes the forward's arguments without o; its outputs are
    required exactly for the inputs the variant has; every rejection happens
    on the host."""
    a = _args(variant, o=None, state_out=None)
    n = binding.gdr_backward_workspace_size(a)
    assert n > binding.gdr_forward_workspace_size(_args(variant))
    bad_args = [dict(flags=binding.GDR_FLAG_QK_L2NORM), dict(q=None), dict(dk=96)]
    for over in bad_args:
        b = _args(variant, o=None, **over)
        assert binding.gdr_backward_workspace_size(b) == 0
        assert binding.gdr_backward_chunked(b, _grads(variant), 0x100000, n, 0) in (1, 2)
    assert binding.gdr_backward_chunked(_args(variant, o=None, flags=1), _grads(variant),
                                        0x100000, n, 0) == 2
    missing = "d_alpha" if variant != "deltanet" else "d_k"
    assert binding.gdr_backward_chunked(a, _grads(variant, **{missing: None}), 0x100000, n, 0) == 1
    extra = "d_erase_b" if variant != "gdn2" else "d_beta"
    assert binding.gdr_backward_chunked(a, _grads(variant, **{extra: 0x1b000}), 0x100000, n, 0) == 1
    assert binding.gdr_backward_chunked(a, _grads(variant, d_q=0x1000), 0x100000, n, 0) == 1  # = q
    assert binding.gdr_backward_chunked(a, _grads(variant, d_k=0x13000), 0x100000, n, 0) == 1
    assert binding.gdr_backward_chunked(a, _grads(variant, d_v=0x15004), 0x100000, n, 0) == 1
    assert binding.gdr_backward_chunked(a, _grads(variant), None, n, 0) == 3
    assert binding.gdr_backward_chunked(a, _grads(variant), 0x100080, n, 0) == 3
    assert binding.gdr_backward_chunked(a, _grads(variant), 0x100000, n - 1, 0) == 3


@pytest.mark.parametrize("variant", list(binding.VARIANTS))
def test_forward_save_and_saved_backward_validation(L, variant):
    """The forward that keeps its records takes the forward's arguments (o
    required) and the gradient's (flags 0, no routed value), no residual
    output, and the gradient's workspace; the saved gradient validates like
    gdr_backward_chunked.  Every rejection happens on the host."""
    a = _args(variant)
    n = binding.gdr_backward_workspace_size(a)
    assert n > 0
    # the forward's own checks
    assert binding.gdr_forward_chunked_save(_args(variant, o=None), 0x100000, n, 0) == 1
    assert binding.gdr_forward_chunked_save(_args(variant, o=0x1000), 0x100000, n, 0) == 1  # = q
    # the gradient's
    assert binding.gdr_forward_chunked_save(_args(variant, flags=1), 0x100000, n, 0) == 2
    assert binding.gdr_forward_chunked_save(_args(variant, v_route=0x1c000), 0x100000, n, 0) == 2
    assert binding.gdr_forward_chunked_save(_args(variant, delta_out=0x1d000), 0x100000, n, 0) == 2
    # its workspace
    assert binding.gdr_forward_chunked_save(a, None, n, 0) == 3
    assert binding.gdr_forward_chunked_save(a, 0x100080, n, 0) == 3
    assert binding.gdr_forward_chunked_save(a, 0x100000, n - 1, 0) == 3
    g = _args(variant, o=None, state_out=None)
    missing = "d_alpha" if variant != "deltanet" else "d_k"
    assert binding.gdr_backward_chunked_saved(g, _grads(variant, **{missing: None}), 0x100000,
                                              n, 0) == 1
    assert binding.gdr_backward_chunked_saved(_args(variant, o=None, flags=1), _grads(variant),
                                              0x100000, n, 0) == 2
    assert binding.gdr_backward_chunked_saved(g, _grads(variant), None, n, 0) == 3
    assert binding.gdr_backward_chunked_saved(g, _grads(variant), 0x100000, n - 1, 0) == 3


def test_backward_workspace_grows_with_length(L):
    a1 = _args("kda", o=None, T=64 * 10)
    a2 = _args("kda", o=None, T=64 * 20)
    n1, n2 = binding.gdr_backward_workspace_size(a1), binding.gdr_backward_workspace_size(a2)
    # per chunk-head, in bf16: the forward factors (+ e^{g_C} in fp32); the
    # state, its gradient and Qt^T dO [dk, dv]; Delta, its gradient and P^T dO
    # [C, dv]; Kbar and W^T [C, dk]
    per = (2 * (64 * 128 * 3 + 64 * 64 + 64 * 64) + 4 * 128 + 3 * 2 * 128 * 64 + 3 * 2 * 64 * 64
           + 2 * 2 * 64 * 128)
    assert abs((n2 - n1) - 2 * 3 * 10 * per) <= 8 * 256


def test_routing_arguments(L):
    """The routed value and the residual output are optional, aligned, and the
    output aliases nothing; the gradient takes no routed value."""
    assert binding.gdr_check_args(_args(v_route=0xa000, delta_out=0xb000), 0) == 0
    assert binding.gdr_check_args(_args(T=1, state_in=0x8000, v_route=0xa000,
                                        delta_out=0xb000), 1) == 0
    assert binding.gdr_check_args(_args(v_route=0xa008), 0) == 1
    assert binding.gdr_check_args(_args(delta_out=0xb004), 0) == 1
    for alias in (0x1000, 0x3000, 0x9000, 0xa000):
        assert binding.gdr_check_args(_args(v_route=0xa000, delta_out=alias), 0) == 1
    assert binding.gdr_check_args(_args(o=0xa000, v_route=0xa000), 0) == 1
    b = _args(o=None, state_out=None, v_route=0xa000)
    assert binding.gdr_backward_chunked(b, _grads(), 0x100000, 1 << 40, 0) == 2
    assert binding.gdr_backward_workspace_size(b) == 0
