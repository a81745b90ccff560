/* Plans a group through the C ABI from plain C99 (no HIP headers, no C++):
 * reads "n V" and then n lines "rows cols kind p0 p1" on stdin, prints
 * "S", the starts and the order kind, or "error <status> <message>". Used by
 * tests/test_abi_c.py. */
#include <stdio.h>
#include <stdlib.h>

#include "rs.h"

int main(void) {
  long long n, V;
  if (scanf("%lld %lld", &n, &V) != 2 || n < 1) return 2;
  rs_tensor_spec* specs = calloc((size_t)n, sizeof *specs);
  int64_t* starts = calloc((size_t)n, sizeof *starts);
  int64_t* order = calloc((size_t)n, sizeof *order);
  if (!specs || !starts || !order) return 2;
  for (long long i = 0; i < n; ++i) {
    long long r, c, k, p0, p1;
    if (scanf("%lld %lld %lld %lld %lld", &r, &c, &k, &p0, &p1) != 5) return 2;
    specs[i].rows = r;
    specs[i].cols = c;
    specs[i].kind = (int32_t)k;
    specs[i].reserved = 0;
    specs[i].p0 = p0;
    specs[i].p1 = p1;
  }
  int64_t S = 0;
  int32_t kind = -1;
  const int st = rs_plan_build(specs, n, V, 16, RS_ORDER_BEST, &S, starts, order, &kind);
  if (st != RS_OK) {
    printf("error %d %s\n", st, rs_last_error());
  } else {
    printf("%lld\n", (long long)S);
    for (long long i = 0; i < n; ++i) printf("%lld%c", (long long)starts[i], i + 1 < n ? ' ' : '\n');
    printf("%d\n", kind);
  }
  free(specs);
  free(starts);
  free(order);
  return 0;
}
