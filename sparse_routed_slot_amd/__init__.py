"""MI355X-native (gfx950) Routing State Model mixer of Raven: sigmoid + top-k router,
chunked forward and fused decode step, behind the C ABI of ``librsm.so``.

The HIP library is loaded lazily by :mod:`sparse_routed_slot_amd.rsm`; importing the
package does not touch the GPU.
"""
__all__ = ["inputs", "rsm"]
