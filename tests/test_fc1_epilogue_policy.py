"""Host logic: which forwards run the activation in FC1's GEMM epilogue (ExpertMLP's fuse_fc1_act)."""

import pytest

from moe_grouped_scaled_amd.expert_mlp import EPILOGUE_ACTS, GATED, use_fc1_epilogue

KINDS = ("srelu", "tanh_srelu", "gelu", "sigmoid", "swiglu", "clamped_swiglu", "glu")


@pytest.mark.parametrize("kind", KINDS)
def test_policy(kind):
    unary = kind not in GATED
    # forced on: every unary kind on MXFP8 without a columnwise copy
    assert use_fc1_epilogue(True, kind, "mxfp8", False) == unary
    # never for NVFP4, gated kinds, or a forward that writes the columnwise copy
    for fuse in (True, False, "auto"):
        assert not use_fc1_epilogue(fuse, kind, "nvfp4", False)
        assert not use_fc1_epilogue(fuse, kind, "mxfp8", True)
    assert not use_fc1_epilogue(False, kind, "mxfp8", False)
    # auto: only where the epilogue measured faster than the separate pass
    assert use_fc1_epilogue("auto", kind, "mxfp8", False) == (unary and kind in EPILOGUE_ACTS)


def test_auto_keeps_srelu_and_sigmoid_only():
    assert set(EPILOGUE_ACTS) == {"srelu", "sigmoid"}


def test_bad_value_raises():
    with pytest.raises(ValueError):
        use_fc1_epilogue("yes", "srelu", "mxfp8", False)
