// Bookkeeping of the two-stage staging buffers (csrc/staging.hpp) with a host
// allocator standing in for device memory: growth retires the old buffer
// without freeing it, release frees every buffer once, a failed allocation
// changes nothing. Built with AddressSanitizer, so a double free or a leak of a
// retired buffer fails the run. Prints "staging ok" on success.
#include <stdio.h>
#include <stdlib.h>

#include <set>

#include "staging.hpp"

static std::set<void *> live;
static int fail_next_alloc = 0;
static int waits = 0;

static int fake_alloc(void **p, size_t bytes)
{
    if (fail_next_alloc) {
        fail_next_alloc = 0;
        return -1;
    }
    *p = malloc(bytes);
    live.insert(*p);
    return 0;
}
static int fake_wait(void)
{
    ++waits;
    return 0;
}
static int fake_free(void *p)
{
    if (!live.count(p)) {
        fprintf(stderr, "free of a buffer that is not live\n");
        abort();
    }
    live.erase(p);
    free(p);
    return 0;
}

#define CHECK(c)                                                    \
    do {                                                            \
        if (!(c)) {                                                 \
            fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
            return 1;                                               \
        }                                                           \
    } while (0)

int main()
{
    arrms::StagingPool<4> pool({fake_alloc, fake_wait, fake_free});
    CHECK(pool.ptr(0) == nullptr && pool.bytes(0) == 0);
    CHECK(pool.release(0) == 0 && waits == 0);  // nothing to free: no wait

    CHECK(pool.reserve(0, 100) == 0);
    void *a = pool.ptr(0);
    CHECK(a && pool.bytes(0) == 100 && live.size() == 1);
    CHECK(pool.reserve(0, 50) == 0 && pool.ptr(0) == a && pool.bytes(0) == 100);  // kept

    // growth: a new buffer, the old one retired and still allocated
    CHECK(pool.reserve(0, 300) == 0);
    void *b = pool.ptr(0);
    CHECK(b != a && pool.bytes(0) == 300 && pool.retired_count(0) == 1 && live.count(a) == 1);
    CHECK(pool.reserve(0, 1000) == 0);
    CHECK(pool.retired_count(0) == 2 && live.size() == 3 && live.count(a) && live.count(b));

    // a failed allocation changes nothing
    void *c = pool.ptr(0);
    fail_next_alloc = 1;
    CHECK(pool.reserve(0, 5000) == -1);
    CHECK(pool.ptr(0) == c && pool.bytes(0) == 1000 && pool.retired_count(0) == 2);

    // devices are independent
    CHECK(pool.reserve(1, 64) == 0 && live.size() == 4 && pool.bytes(0) == 1000);

    // release frees the current and the retired buffers of that device only
    CHECK(pool.release(0) == 0 && waits == 1);
    CHECK(pool.ptr(0) == nullptr && pool.bytes(0) == 0 && pool.retired_count(0) == 0);
    CHECK(live.size() == 1 && pool.bytes(1) == 64);
    CHECK(pool.release(0) == 0 && waits == 1);
    CHECK(pool.reserve(0, 10) == 0 && pool.bytes(0) == 10 && pool.retired_count(0) == 0);
    CHECK(pool.release(0) == 0 && pool.release(1) == 0 && live.empty());
    printf("staging ok\n");
    return 0;
}
