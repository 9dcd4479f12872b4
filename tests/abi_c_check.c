/* Calls the library's pure host entry points from plain C (C99), through
 * include/gemm_f16_nt.h only, and prints what they return, one "key value..."
 * line each, for tests/test_abi_c.py to compare with the Python binding. */
#include <stdio.h>
#include "gemm_f16_nt.h"

int main(void)
{
    const int64_t shapes[][3] = {{8192, 8192, 8192}, {4999, 7001, 4160}, {128, 16384, 16384},
                                 {1024, 1024, 65536}, {256, 256, 256}};
    int i;
    printf("configs %d\n", gemm_f16_nt_num_configs());
    printf("status %s|%s\n", gemm_f16_nt_status_string(0), gemm_f16_nt_status_string(2));
    printf("validate %d %d\n", gemm_f16_nt_validate(64, 64, 64, (void *)0x10000,
                                                    (void *)0x20000000, (void *)0x40000000),
           gemm_f16_nt_validate(-1, 64, 64, (void *)0x10000, (void *)0x20000000,
                                (void *)0x40000000));
    for (i = 0; i < (int)(sizeof shapes / sizeof shapes[0]); ++i) {
        gemm_f16_nt_plan_t p;
        int32_t splits = 0, tm = 0, tn = 0, n = 0;
        int64_t ws = 0, need = 0;
        const int64_t M = shapes[i][0], N = shapes[i][1], K = shapes[i][2];
        if (gemm_f16_nt_plan(M, N, K, 256, &p) != GEMM_F16_OK) return 1;
        if (gemm_f16_nt_tile_of_slot(&p, p.tiles - 1, &tm, &tn) != GEMM_F16_OK) return 2;
        printf("plan %lld %d %d %d %lld %d %d\n", (long long)M, p.config_id, p.block_m,
               p.block_n, (long long)p.tiles, tm, tn);
        if (gemm_f16_nt_splitk_plan(M, N, K, 256, 0, &p, &splits, &ws) != GEMM_F16_OK) return 3;
        printf("split %lld %d %d %lld\n", (long long)M, p.config_id, splits, (long long)ws);
        if (gemm_f16_tt_plan(M, N, K, 256, &p) != GEMM_F16_OK) return 4;
        printf("tt %lld %d\n", (long long)M, p.config_id);
        if (gemm_f16_autotune_candidates(0, M, N, K, 256, 1, (int64_t)1 << 40, NULL, 0, &n,
                                         &need) != GEMM_F16_OK)
            return 5;
        printf("tune %lld %d %lld\n", (long long)M, n, (long long)need);
        if (gemm_f16_splitk_workspace_bytes(M, N, 8, &ws) != GEMM_F16_OK) return 6;
        printf("bound %lld %lld\n", (long long)M, (long long)ws);
    }
    return 0;
}
