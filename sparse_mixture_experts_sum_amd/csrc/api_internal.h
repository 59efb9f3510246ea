// Host-side helpers shared between the entry points of the C ABI (internal).
#pragma once

#include <stddef.h>

#include "moe.h"

// Every host check of moe_forward except those of the workspace (shape, routing mode,
// training noise, null and misaligned pointers); on success *ws_need is the workspace size
// the shape needs. Makes no HIP call.
moe_status forward_host_checks(const moe_shape* shape, const void* x, const void* W_g,
                               const moe_noise* noise, const void* W_gate, const void* W_up,
                               const void* W_down, const float* y, const float* f,
                               const float* p, const float* loss, size_t* ws_need);
