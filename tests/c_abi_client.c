/* A plain C99 client of include/mhc.h: it builds against the header alone, links
 * libmhc.so and calls only the entry points that answer on the host (version, status
 * strings, sizes, validation), so it runs without a GPU. Exit code 0 and "ok" when every
 * answer is the documented one. */
#include <stdio.h>
#include <string.h>

#include "mhc.h"

static int failures = 0;
#define EXPECT(cond)                                                   \
    do {                                                               \
        if (!(cond)) {                                                 \
            fprintf(stderr, "failed: %s (line %d)\n", #cond, __LINE__); \
            ++failures;                                                \
        }                                                              \
    } while (0)

int main(void)
{
    mhc_pre_params p;
    mhc_pre_bwd_params bp;
    mhc_pre_tensors t;
    size_t bytes = 0, packed = 0;
    int32_t path = -1;

    EXPECT(mhc_version() > 0);
    EXPECT(mhc_status_string(MHC_OK) != NULL);
    EXPECT(strcmp(mhc_status_string(MHC_ERR_NULLPTR), mhc_status_string(MHC_ERR_PARAM_INVALID)) != 0);

    /* the large prefill shape: T = 16384, n = 4, D = 7168, alpha[3], 20 iterations */
    memset(&p, 0, sizeof p);
    p.T = 16384;
    p.n = 4;
    p.D = 7168;
    p.n_alpha = 3;
    p.num_iters = 20;
    p.norm_eps = 1e-6;
    p.hc_eps = 1e-6;
    p.need_backward = 1;
    p.x_dtype = MHC_DTYPE_BF16;
    EXPECT(mhc_pre_workspace_size(&p, &bytes) == MHC_OK && bytes > 0);
    EXPECT(mhc_pre_packed_size(&p, &packed) == MHC_OK && packed >= (size_t)3 * 24 * 4 * 7168 * 2);
    EXPECT(mhc_pre_workspace_size(NULL, &bytes) == MHC_ERR_NULLPTR);
    EXPECT(mhc_pre_workspace_size(&p, NULL) == MHC_ERR_NULLPTR);

    /* invalid problem descriptions, refused before any HIP call */
    p.n = 5;
    EXPECT(mhc_pre_workspace_size(&p, &bytes) == MHC_ERR_PARAM_INVALID);
    p.n = 4;
    p.D = 12;
    EXPECT(mhc_pre_workspace_size(&p, &bytes) == MHC_ERR_PARAM_INVALID);
    p.D = 7168;
    p.x_dtype = 2;
    EXPECT(mhc_pre_workspace_size(&p, &bytes) == MHC_ERR_PARAM_INVALID);
    p.x_dtype = MHC_DTYPE_F16;
    EXPECT(mhc_pre_workspace_size(&p, &bytes) == MHC_OK);

    /* a forward with its required pointers missing returns before launching anything */
    memset(&t, 0, sizeof t);
    EXPECT(mhc_pre_forward(&p, &t, NULL, 0, NULL) == MHC_ERR_NULLPTR);
    EXPECT(mhc_pre_forward(NULL, &t, NULL, 0, NULL) == MHC_ERR_NULLPTR);
    EXPECT(mhc_pre_forward_path(NULL, 0, &path) == MHC_ERR_NULLPTR);

    /* the backward's sizes for every n it takes, both 16-bit formats */
    memset(&bp, 0, sizeof bp);
    bp.T = 1024;
    bp.D = 512;
    bp.hc_eps = 1e-6;
    for (int n = 4; n <= 8; n += 2) {
        for (int f16 = 0; f16 <= 1; ++f16) {
            bp.n = n;
            bp.x_f16 = f16;
            bytes = 0;
            EXPECT(mhc_pre_backward_workspace_size(&bp, &bytes) == MHC_OK && bytes > 0);
        }
    }
    bp.n = 5;
    EXPECT(mhc_pre_backward_workspace_size(&bp, &bytes) == MHC_ERR_PARAM_INVALID);
    bp.n = 4;
    bp.x_f16 = 3;
    EXPECT(mhc_pre_backward_workspace_size(&bp, &bytes) == MHC_ERR_PARAM_INVALID);

    if (failures == 0) printf("ok\n");
    return failures == 0 ? 0 : 1;
}
