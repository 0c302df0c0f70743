// Host-only stand-in for <hip/hip_runtime.h> in the sanitizer build of the library's host sources
// (tests/test_sanitize.py): the host files use nothing from it but the stream handle type.
#pragma once
typedef struct ihipStream_t *hipStream_t;
