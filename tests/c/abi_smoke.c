/* Plain C99 user of include/fa.h: takes the address of every entry point and
 * calls the ones that need no device (argument rejection, workspace size,
 * status strings). Built and run by tests/test_c_header.py. */
#include <stdio.h>

#include "fa.h"

int main(void) {
  void* fns[] = {(void*)fa_forward, (void*)fa_backward, (void*)fa_forward_ex,
                 (void*)fa_backward_ex, (void*)fa_forward_fp8,
                 (void*)fa_backward_workspace_size, (void*)fa_status_string,
                 (void*)fa_last_error_message};
  for (unsigned i = 0; i < sizeof fns / sizeof fns[0]; ++i)
    if (fns[i] == NULL) return 2;
  fa_status_t s = fa_forward(NULL, NULL, NULL, NULL, NULL, NULL, 1, 1, 16, 64, 0.125f, 0, -1, -1,
                             FA_DTYPE_BF16, NULL);
  printf("status=%d name=%s detail=%s\n", (int)s, fa_status_string(s), fa_last_error_message());
  s = fa_forward_fp8(NULL, NULL, NULL, NULL, NULL, NULL, 1, 1, 16, 64, 0.125f, 1.f, 1.f, 0.f, 0,
                     -1, -1, NULL);
  printf("status=%d detail=%s\n", (int)s, fa_last_error_message());
  printf("workspace=%zu\n", fa_backward_workspace_size(1, 1, 16, 64, FA_DTYPE_BF16));
  return 0;
}
