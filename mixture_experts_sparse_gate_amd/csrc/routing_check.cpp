// Host-side validation of a caller's routing (see routing_check.h).
#include "routing_check.h"

#include <stdio.h>

extern "C" int moe_check_routing_host(const int32_t* idx, int64_t T, int32_t k, int32_t N, char* msg,
                                      size_t msg_len) {
  for (int64_t t = 0; t < T; ++t) {
    const int32_t* row = idx + t * k;
    for (int32_t j = 0; j < k; ++j) {
      if (row[j] < 0 || row[j] >= N) {
        if (msg && msg_len) snprintf(msg, msg_len, "entry (%lld, %d) = %d is outside [0, %d)", (long long)t, j, row[j], N);
        return 1;
      }
      for (int32_t jj = 0; jj < j; ++jj)
        if (row[jj] == row[j]) {
          if (msg && msg_len)
            snprintf(msg, msg_len, "token %lld names expert %d twice (choices %d and %d)", (long long)t, row[j], jj, j);
          return 2;
        }
    }
  }
  if (msg && msg_len) msg[0] = '\0';
  return 0;
}
