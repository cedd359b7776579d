"""Host paths of the C ABI, run in a child process against the build of the
library with AddressSanitizer on its host code (libflint_moe_asan.so, the
sanitizer runtime preloaded).  Started by test_abi_asan.py; not a test module.

``python tests/asan_paths.py`` runs the argument validation of every entry
point, and create calls that fail after their handle is allocated (no device,
or the first device allocation failing), which release that handle.

Only paths that allocate no device memory run here: the compiler's sanitizer
runtime also intercepts the HSA device-memory allocator, and that interceptor
needs XNACK, which these GPUs run without.  The partial-release paths of a
create that fails at each of its device allocations are checked on the GPU
with the plain library (device memory returns to its baseline).
"""
import ctypes
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path[:0] = [ROOT, HERE]

import numpy as np  # noqa: E402

import int4_expert_ffn_amd as F  # noqa: E402

def say(msg):
    print(msg, flush=True)


def host_layer(bufs):
    """A layer descriptor whose 14 tensors are small host buffers: valid
    pointers for validation, never read because create fails first."""
    return F.flint_moe_layer(bufs[0].ctypes.data, bufs[1].ctypes.data,
                             *[F.flint_q4(bufs[2 + 2 * i].ctypes.data, bufs[3 + 2 * i].ctypes.data) for i in range(6)])


def cpu_paths():
    import test_abi
    for name in ("test_header_declares_the_binding_names", "test_library_exports_every_declared_symbol",
                 "test_attention_rejects_bad_arguments_before_any_hip_call",
                 "test_create_rejects_bad_arguments_before_any_hip_call", "test_null_handle_calls",
                 "test_dense_and_head_reject_bad_arguments_before_any_hip_call"):
        getattr(test_abi, name)()
        say(f"ok {name}")
    lib = F.lib()
    bufs = [np.zeros(64, np.uint8) for _ in range(14)]
    layers = (F.flint_moe_layer * 3)(*[host_layer(bufs)] * 3)
    os.environ["FLINT_MOE_FAIL_ALLOC"] = "1"
    try:
        for _ in range(3):
            h = ctypes.c_void_p(1234)
            rc = lib.flint_moe_create(layers, 3, ctypes.byref(h))
            # no device: the device query fails; with one, the first allocation does
            assert rc in (F.FLINT_ERR_HIP, F.FLINT_ERR_OUT_OF_MEMORY), rc
            assert h.value is None
            assert F.flint_moe_last_error()
    finally:
        del os.environ["FLINT_MOE_FAIL_ALLOC"]
    say("ok create failure after the handle is allocated")


if __name__ == "__main__":
    cpu_paths()
    say("asan paths done")
