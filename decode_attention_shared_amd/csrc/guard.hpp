// No C++ exception may leave an extern "C" entry point: each entry point runs
// its body through guarded(), which turns any exception (in practice
// std::bad_alloc from a host-side container) into HP_ERR_HOST.
#pragma once

#include "hp_attn.h"

namespace hp {

template <class F>
hp_status guarded(F &&body) noexcept {
    try {
        return body();
    } catch (...) {
        return HP_ERR_HOST;
    }
}

}  // namespace hp
