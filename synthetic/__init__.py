"""Seeded synthetic KV-cache workloads.

This package holds only input generators and workload shapes: none of the codec's
arithmetic. Both the oracle-side tests and the HIP path draw their inputs from here.

The shapes follow the model families the TurboAngle abstract (arXiv 2603.27467)
evaluates (1B-7B decoder models, Mistral-7B among them) plus a long-context and a
large-batch 70B-class case. Real activations are not available, so keys carry the
traits the PatternKV abstract (ICML 2026) describes for real KV caches: a few
high-magnitude channels that widen the range, a per-token scale, and (long-context
case) a slow structure that evolves along the sequence.
"""

from .configs import CONFIGS, Workload, get  # noqa: F401
from .gen import layer_kv, query, tiny_inputs  # noqa: F401
