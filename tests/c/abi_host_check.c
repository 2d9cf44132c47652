/* Compiled as C99 against include/moe_shuffle.h and linked to the library:
 * checks that the header is plain C and that the host-only entry points
 * (no device work) behave as declared.  Prints one line per check and
 * exits non-zero on the first failure. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "moe_shuffle.h"

static int fail(const char* what)
{
    printf("FAIL %s\n", what);
    return 1;
}

int main(void)
{
    moe_shuffle_dims d = {8192, 7168, 256, 8, 32};
    size_t bytes = 0;
    if (moe_shuffle_workspace_size(&d, &bytes) != MOE_SHUFFLE_OK || bytes == 0) return fail("workspace size");
    printf("workspace %zu\n", bytes);

    moe_shuffle_dims odd = {4, 12, 8, 2, 4}; /* H not a multiple of 8 */
    if (moe_shuffle_workspace_size(&odd, &bytes) != MOE_SHUFFLE_E_ALIGN) return fail("alignment code");
    moe_shuffle_dims uneven = {4, 8, 8, 2, 3}; /* E % R != 0 */
    if (moe_shuffle_workspace_size(&uneven, &bytes) != MOE_SHUFFLE_E_INVALID_ARG) return fail("invalid code");
    moe_shuffle_dims wide = {4, 8, 128, 65, 4}; /* k > 64 */
    if (moe_shuffle_workspace_size(&wide, &bytes) != MOE_SHUFFLE_E_OVERFLOW) return fail("overflow code");
    if (moe_shuffle_workspace_size(NULL, &bytes) != MOE_SHUFFLE_E_INVALID_ARG) return fail("null dims");

    /* every call on a null plan fails with INVALID_ARG before touching a device */
    if (moe_shuffle_dispatch(NULL, NULL, NULL, 0, NULL, NULL) != MOE_SHUFFLE_E_INVALID_ARG) return fail("dispatch");
    if (moe_shuffle_combine(NULL, NULL, NULL, NULL, NULL) != MOE_SHUFFLE_E_INVALID_ARG) return fail("combine");
    moe_shuffle_plan_info info;
    if (moe_shuffle_plan_query(NULL, NULL, &info) != MOE_SHUFFLE_E_INVALID_ARG) return fail("query");
    moe_shuffle_plan_arrays arrays;
    if (moe_shuffle_plan_arrays_get(NULL, &arrays) != MOE_SHUFFLE_E_INVALID_ARG) return fail("arrays");
    moe_shuffle_plan_destroy(NULL);

    /* the reference copy rejects bad arguments on the host, before any launch */
    char* const fake = (char*)(uintptr_t)4096; /* never dereferenced */
    if (moe_shuffle_copy_reference(NULL, fake, 16, NULL) != MOE_SHUFFLE_E_INVALID_ARG) return fail("copy null");
    if (moe_shuffle_copy_reference(fake, fake + 4096, 24, NULL) != MOE_SHUFFLE_E_ALIGN) return fail("copy size");
    if (moe_shuffle_copy_reference(fake + 8, fake + 4096, 16, NULL) != MOE_SHUFFLE_E_ALIGN) return fail("copy align");
    if (moe_shuffle_copy_reference(fake, fake + 16, 64, NULL) != MOE_SHUFFLE_E_INVALID_ARG) return fail("copy overlap");
    if (moe_shuffle_copy_reference(fake, fake + 16, 0, NULL) != MOE_SHUFFLE_OK) return fail("copy empty");

    const int codes[] = {MOE_SHUFFLE_OK, MOE_SHUFFLE_E_INVALID_ARG, MOE_SHUFFLE_E_ALIGN, MOE_SHUFFLE_E_WORKSPACE,
                         MOE_SHUFFLE_E_BAD_INDEX, MOE_SHUFFLE_E_HIP, MOE_SHUFFLE_E_OVERFLOW};
    for (size_t i = 0; i < sizeof codes / sizeof codes[0]; ++i) {
        const char* s = moe_shuffle_strerror(codes[i]);
        if (!s || !strlen(s)) return fail("strerror");
        printf("%d %s\n", codes[i], s);
    }
    printf("ok\n");
    return 0;
}
