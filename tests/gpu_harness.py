"""GPU-side test plumbing: the device workloads of ``workloads.device``."""
from workloads.device import (DeviceWorkload, TORCH_DTYPE, INT_VIEW, i32, poison_pool,  # noqa: F401
                              prefill, to_f64, varlen)
