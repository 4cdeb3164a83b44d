"""MI355X-native dynamic-embedding hot path (HIP library librecis.so + ctypes binding).

The C ABI is declared in ``include/recis.h``; ``recis`` binds it by name.
"""
from .recis import (DeviceFeature, LookupResult, RecisError, Table, load_library,  # noqa: F401
                    make_descs)
