"""MI355X-native forward pass of a DeepSeek-V3-style mixture-of-experts feed-forward layer.

The layer runs in hand-written HIP kernels behind the C ABI of include/moe.h (libmoe.so); this package
holds those sources (csrc/), their build script, a ctypes binding with the same entry-point names and the
seeded synthetic workloads.
"""
from .binding import (MOE_BF16, MOE_F32, MOE_FP8_E4M3, MoeError, forward_inputs, make_shape, moe_expert_utilization,
                      moe_forward, moe_forward_shard, moe_route, moe_route_limited, moe_status_string,
                      moe_workspace_size, shard_inputs, shard_weights)
