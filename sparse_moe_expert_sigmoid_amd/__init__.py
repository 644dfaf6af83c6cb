"""MI355X-native routed mixture-of-experts layer (gfx950 HIP kernels behind a C ABI).

The C ABI is include/moe.h; libmoe_mi355x.so implements it; `binding` is the
ctypes layer over it, `layer.MoELayer` chains its five calls and
`stack.MoEStack` runs layers one after another with the residual between them;
`restrict` picks per-layer expert subsets from recorded routing counts.
"""
from .binding import (Context, DeviceExperts, MoeError, load_library, LIB_PATH,  # noqa: F401
                      MOE_ACT_GELU_TANH, MOE_ACT_SILU, MOE_ROUTER_SIGMOID_BIAS,
                      MOE_ROUTER_SOFTMAX, MOE_W_FP32, MOE_W_INT4_B128, MOE_W_INT4_B32,
                      MOE_W_INT8_ROW)
from .layer import MoELayer  # noqa: F401
from .stack import MoEStack  # noqa: F401
from .restrict import coverage_set, expert_mask  # noqa: F401
