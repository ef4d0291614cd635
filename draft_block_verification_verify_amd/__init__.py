"""MI355X-native verify step for parallel draft blocks (chains and proposal trees).

The compute path is the HIP library libspecverify.so (C ABI in
include/spec_verify.h); `binding` marshals arguments to it.  Importing this
package does not load the library; the first call through `binding` does, and
raises if it is not built.
"""
__all__ = ["binding", "workloads", "accounting"]
