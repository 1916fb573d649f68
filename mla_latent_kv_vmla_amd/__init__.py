"""MI355X-native latent-KV chunk attention (VideoMLA hot path).

The compute lives in the HIP library ``libvmla.so`` (C ABI declared in
``include/vmla.h``); :mod:`mla_latent_kv_vmla_amd.vmla` is the thin ctypes
binding over it.  :mod:`mla_latent_kv_vmla_amd.workloads` holds geometries and
seeded synthetic inputs.  Importing the package loads nothing native.
"""
