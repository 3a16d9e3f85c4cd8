/* Out-of-range enum arguments, as a C caller (or a foreign-function binding)
 * may pass them: in C an enum argument is just an int, so the library must
 * treat unknown values as errors without undefined behaviour on its side.
 * Called by abi_driver.cpp; returns 0 when every call answers as documented. */
#include <stddef.h>
#include <string.h>

#include "msa.h"

int abi_enum_range_checks(void) {
  msa_dims d = {1, 1024, 8, 2, 128, 64, 4, 0.f};
  const int ops[] = {-1, 6, 99, 0x7fffffff};
  for (size_t i = 0; i < sizeof ops / sizeof ops[0]; ++i)
    if (msa_workspace_bytes(&d, (msa_op)ops[i]) != 0 || msa_workspace_min_bytes(&d, (msa_op)ops[i]) != 0) return 1;
  const int codes[] = {-1, 99, 0x7fffffff};
  for (size_t i = 0; i < sizeof codes / sizeof codes[0]; ++i)
    if (strcmp(msa_status_str((msa_status)codes[i]), "unknown status") != 0) return 2;
  return 0;
}
