"""MI355X-native (gfx950) routed-expert MoE FFN with block-quantized low-bit experts.

Modules:
    qmoe       ctypes binding of libqmoe (C ABI in include/qmoe.h); raises on import if the
               compiled library is missing
    synth      seeded synthetic inputs (host and device fills of the packed weights)
    workloads  synthetic layers and inputs in device memory
    build      hipcc build of the two shared libraries
"""
