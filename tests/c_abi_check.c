/* A plain C99 user of kvstream.h: the header compiles as C and the library
 * links and answers its host-only calls from C (no device needed).  Prints
 * one "name value" line per check for tests/test_c_abi.py. */
#include "kvstream.h"

#include <stdio.h>

int main(void)
{
    kv_layout lay;
    int32_t count[8] = {1000, 1000, 1000, 1000, 1000, 1000, 1000, 1000};
    printf("layout_init %d\n", kv_layout_init(&lay, 48, 8, 25, 64, 1024, KV_F16));
    printf("k_bytes %lld\n", (long long)lay.k_bytes);
    printf("pack_bytes %lld\n", (long long)kv_pack_bytes(&lay, 48, count, 0));
    printf("pack_bytes_uniform %lld\n", (long long)kv_pack_bytes(&lay, 48, NULL, 1000));
    printf("bad_layout %d\n", kv_layout_init(&lay, 0, 8, 25, 64, 1024, KV_F16));
    printf("error_message_set %d\n", kv_last_error() != NULL && kv_last_error()[0] != 0);

    kv_paged pg;
    printf("paged_init %d\n", kv_paged_init(&pg, 48, 552, 25, 64, 16, KV_F16));
    printf("paged_pack_bytes %lld\n", (long long)kv_paged_pack_bytes(&pg, 48, 8, count));

    kv_layout src_lay;
    kv_layout_init(&src_lay, 16, 8, 72, 128, 2048, KV_F16);
    kv_part src = {0, 16, 0, 72, 0, 8}, dst = {8, 8, 36, 36, 0, 8};
    int32_t lens[8] = {300, 301, 302, 303, 304, 305, 306, 307};
    printf("stream_bytes %lld\n", (long long)kv_stream_bytes(&src_lay, &src, &dst, lens));

    double lhs = 0, rhs = 0;
    printf("swap_pays %d\n", kv_swap_pays(2, 2.5, 1, 1, 1.0, 1.0, &lhs, &rhs));
    printf("swap_pays_sides %.1f %.1f\n", lhs, rhs);

    kv_acklog *a = NULL;
    int32_t j = -1;
    int64_t t = -1;
    kv_acklog_create(&a, 2, 2);
    kv_ack(a, 0, 0, 3);
    kv_ack(a, 1, 0, 3);
    kv_ack(a, 0, 1, 3);
    kv_ack_restart_point(a, &j, &t);
    printf("restart_point %d %lld\n", j, (long long)t);
    kv_acklog_destroy(a);
    kv_profile_window win;
    win.span_ms = -1.0;
    win.hbm_launches = -1;
    const int win_st = kv_profile_last_window(&win);
    const int win_null = kv_profile_last_window(NULL);
    printf("profile_window %d %.1f %lld %d\n", win_st, win.span_ms, (long long)win.hbm_launches,
           win_null);
    printf("version %d\n", kv_version());
    return 0;
}
