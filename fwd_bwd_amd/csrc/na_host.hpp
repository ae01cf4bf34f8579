// na_host.hpp -- host-side launch helpers shared by the sources of libna.
#pragma once

#include <hip/hip_runtime.h>

#include <mutex>
#include <set>
#include <utility>

namespace na_host {

// Largest dynamic LDS a workgroup may use on gfx950.
constexpr int kLdsLimit = 160 * 1024;

// Raises a kernel's dynamic-LDS limit to the hardware maximum, once per
// (kernel, device). The limit is per-function state of the runtime: setting it
// per call to that call's own size would let two host threads launching
// different problem sizes shrink it under each other. A launch still passes
// its own dynamic LDS size, which alone sets the kernel's occupancy.
inline bool lds_limit_once(const void *kern) {
    static std::mutex mu;
    static std::set<std::pair<const void *, int>> done;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return false;
    std::lock_guard<std::mutex> lock(mu);
    if (done.count({kern, dev})) return true;
    if (hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsLimit) !=
        hipSuccess)
        return false;
    done.insert({kern, dev});
    return true;
}

}  // namespace na_host
