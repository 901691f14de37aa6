// Host-side validation of a routing a caller hands to moe_dispatch
// (compiled into debug builds' checks, and on its own into the CPU tests).
#pragma once

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

// idx [T, k] on the host. Returns 0 when every entry lies in [0, N) and no
// token names an expert twice; otherwise 1 (an index out of range) or 2 (a
// repeated expert), with a message naming the first such (t, j) in msg.
int moe_check_routing_host(const int32_t* idx, int64_t T, int32_t k, int32_t N, char* msg, size_t msg_len);

#ifdef __cplusplus
}
#endif
