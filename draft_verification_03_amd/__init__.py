"""MI355X-native speculative-sampling verification step.

The compute path is the C-ABI library ``libspecv.so`` (hand-written HIP for gfx950) behind
``include/spec_verify.h``; :mod:`draft_verification_03_amd.binding` is its thin ctypes
binding (argument marshalling only). :mod:`draft_verification_03_amd.workloads` draws the
seeded synthetic inputs. Importing the package loads nothing; the binding loads the library
on first use and raises if it is missing.
"""
