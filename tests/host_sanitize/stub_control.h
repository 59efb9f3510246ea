// Controls of the host-only stand-ins in stub_kernels.cpp.
#pragma once
#include <stddef.h>

void stub_set_workspace(const void* ws, size_t bytes);  // bounds for the extent checks
long stub_launches();                                   // launch wrappers called so far
void stub_events_work(int on);                          // fake HIP events succeed
