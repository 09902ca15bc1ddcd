"""MI355X-native sparse global attention (Speed3R dual-branch forward pass).

The compute path lives in ``libspeed3r.so`` (HIP kernels for gfx950 behind a C ABI); this
package only holds the Python binding and the workload definitions.
"""
