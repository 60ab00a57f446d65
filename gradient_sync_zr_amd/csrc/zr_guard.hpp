// Host-side wrapper for the C entry points: a C++ exception raised inside
// one (a host allocation that fails) becomes a status and an error message
// instead of unwinding through a C caller.
#pragma once

#include <new>

#include "zr.h"

namespace zr {

zr_status set_error(zr_status st, const char* msg);

template <class F>
zr_status guarded(F&& body) noexcept {
    try {
        return body();
    } catch (const std::bad_alloc&) {
        return set_error(ZR_ERR_NOMEM, "out of host memory");
    } catch (...) {
        return set_error(ZR_ERR_INVALID, "unexpected C++ exception");
    }
}

}  // namespace zr
