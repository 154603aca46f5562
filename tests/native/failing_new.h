// Host allocations that fail on request, for tests of the library's
// out-of-memory handling. The test executables are linked with
// -Wl,--wrap=<symbol> for the four plain operator new forms, so calls from
// the library's and the test's own objects come here, and the sanitizer's
// allocator (the __real_ symbols) does the work otherwise. Allocations made
// inside the C++ runtime library itself are not counted.
//
// g_new_budget < 0: allocations succeed; otherwise the next g_new_budget
// allocations succeed and the one after that fails.
#pragma once

#include <cstddef>
#include <new>

static long g_new_budget = -1;

static bool allocation_fails()
{
    if (g_new_budget == 0) return true;
    if (g_new_budget > 0) --g_new_budget;
    return false;
}

extern "C" {
void *__real__Znwm(std::size_t);
void *__real__Znam(std::size_t);
void *__real__ZnwmRKSt9nothrow_t(std::size_t, const std::nothrow_t &) noexcept;
void *__real__ZnamRKSt9nothrow_t(std::size_t, const std::nothrow_t &) noexcept;

void *__wrap__Znwm(std::size_t n)
{
    if (allocation_fails()) throw std::bad_alloc();
    return __real__Znwm(n);
}

void *__wrap__Znam(std::size_t n)
{
    if (allocation_fails()) throw std::bad_alloc();
    return __real__Znam(n);
}

void *__wrap__ZnwmRKSt9nothrow_t(std::size_t n, const std::nothrow_t &t) noexcept
{
    return allocation_fails() ? nullptr : __real__ZnwmRKSt9nothrow_t(n, t);
}

void *__wrap__ZnamRKSt9nothrow_t(std::size_t n, const std::nothrow_t &t) noexcept
{
    return allocation_fails() ? nullptr : __real__ZnamRKSt9nothrow_t(n, t);
}
}
