"""MI355X-native product-VQ KV-cache hot path (encode, decode, attention from codes).

The compute runs in libvq.so (hand-written HIP kernels for gfx950) behind the
C ABI declared in include/vq.h; this package only marshals torch tensors to it.
"""
from .api import (VQError, attend_workspace, vq_attend, vq_attend_noalloc, vq_attend_path,  # noqa: F401
                  vq_attend_workspace_bytes, vq_decode, vq_decode_step, vq_encode, vq_encode_decode,
                  vq_encode_kv, vq_kmeans, vq_kmeans_workspace_bytes, vq_supports_shape,
                  vq_transform)
from .cache import CacheLayout, VQKVCache  # noqa: F401
