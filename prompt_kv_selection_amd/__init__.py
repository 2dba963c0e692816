"""MI355X-native observation-window KV-cache selection (SnapKV scoring).

The compute path lives in the HIP library ``libkvsel.so`` (sources under
``csrc/``, C ABI in ``include/kvsel.h``).  ``binding`` marshals PyTorch device
tensors into that ABI; importing it loads the library and fails loudly when it
has not been built.  ``workloads`` draws the seeded synthetic inputs.
"""

__all__ = ["binding", "workloads", "build"]
