// staging.hpp -- bookkeeping of the per-device staging buffers of the two-stage
// path (the per-rank staging region of ROCm/aiter PR #6699 "gfx1250 fused
// all-reduce + RMSNorm", section Changes).
//
// A two-stage launch bakes the staging address into its kernel arguments, and
// so into any HIP graph captured around it. Growing the buffer therefore never
// frees the one it replaces: the superseded buffer is retired and stays
// allocated until release(), so that launches in flight and graphs captured
// earlier keep valid memory. release() frees the current and every retired
// buffer of a device; graphs captured on the two-stage path must be destroyed
// before it.
//
// The allocator is a parameter (device memory in the library, a host fake in
// the CPU test of this bookkeeping). Not thread-safe: the caller holds a lock.
#pragma once

#include <stddef.h>

#include <vector>

namespace arrms {

struct StagingOps {
    int (*alloc)(void **p, size_t bytes);  // 0 on success
    int (*release_all)(void);             // before frees: wait for work in flight; 0 on success
    int (*free)(void *p);                  // 0 on success
};

template <int MaxDevices> class StagingPool {
public:
    explicit StagingPool(const StagingOps &ops) : ops_(ops) {}

    // Current buffer of a device (nullptr if none) and its size.
    void *ptr(int dev) const { return d_[dev].ptr; }
    size_t bytes(int dev) const { return d_[dev].ptr ? d_[dev].bytes : 0; }
    size_t retired_count(int dev) const { return d_[dev].retired.size(); }

    // At least `bytes` on device dev. A larger current buffer is kept; a
    // smaller one is retired (kept allocated) and replaced. 0 on success, -1
    // if the allocation failed (nothing changed then).
    int reserve(int dev, size_t bytes)
    {
        Dev &d = d_[dev];
        if (d.ptr && d.bytes >= bytes)
            return 0;
        if (d.ptr) {
            // room for the retired entry first, so that nothing below can throw
            // (no exception may cross the C ABI)
            try {
                d.retired.reserve(d.retired.size() + 1);
            } catch (...) {
                return -1;
            }
        }
        void *p = nullptr;
        if (ops_.alloc(&p, bytes) != 0 || !p)
            return -1;
        if (d.ptr)
            d.retired.push_back(d.ptr);
        d.ptr = p;
        d.bytes = bytes;
        return 0;
    }

    // Frees the current and the retired buffers of device dev. 0 on success;
    // -1 if waiting or a free failed (buffers not yet freed stay listed).
    int release(int dev)
    {
        Dev &d = d_[dev];
        if (!d.ptr && d.retired.empty())
            return 0;
        if (ops_.release_all() != 0)
            return -1;
        while (!d.retired.empty()) {
            if (ops_.free(d.retired.back()) != 0)
                return -1;
            d.retired.pop_back();
        }
        if (d.ptr) {
            if (ops_.free(d.ptr) != 0)
                return -1;
            d.ptr = nullptr;
            d.bytes = 0;
        }
        return 0;
    }

private:
    struct Dev {
        void *ptr = nullptr;
        size_t bytes = 0;
        std::vector<void *> retired;
    };
    StagingOps ops_;
    Dev d_[MaxDevices];
};

}  // namespace arrms
