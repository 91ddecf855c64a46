"""MI355X-native gradient all-reduce schedules (ring, hierarchical, Rabenseifner).

The compute path is the HIP library libar.so (csrc/), reached through the
C ABI declared in include/ar.h; this package only marshals arguments.
"""
