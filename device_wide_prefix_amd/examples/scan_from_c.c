/*
 * Calling the scan library from C through its C ABI (include/dws_scan.h):
 * device buffers from hipMalloc, a stream, an exclusive scan in place, a
 * compaction with its count in device memory, the same scan split into two
 * shards (each shard's total, the scan of the totals, each shard scanned seeded
 * with its offset), and a check of every result on the host with exact
 * integer arithmetic. Exit status 0 on success.
 *
 * Build: hipcc -I include scan_from_c.c -L device_wide_prefix_amd -ldws_scan
 *        -Wl,-rpath,<that directory> -o scan_from_c
 * Usage: scan_from_c [n]   (default 10000019)
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "dws_scan.h"

#define CHECK_HIP(call)                                                                      \
    do {                                                                                     \
        hipError_t e_ = (call);                                                              \
        if (e_ != hipSuccess) {                                                              \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));                \
            return 2;                                                                        \
        }                                                                                    \
    } while (0)

#define CHECK_DWS(call)                                                                      \
    do {                                                                                     \
        dws_status s_ = (call);                                                              \
        if (s_ != DWS_OK) {                                                                  \
            fprintf(stderr, "%s failed: %s\n", #call, dws_status_string(s_));                \
            return 3;                                                                        \
        }                                                                                    \
    } while (0)

int main(int argc, char** argv)
{
    const size_t n = argc > 1 ? (size_t)strtoull(argv[1], NULL, 10) : (size_t)10000019;
    uint32_t* h_x = (uint32_t*)malloc(n * sizeof(uint32_t));
    int32_t* h_f = (int32_t*)malloc(n * sizeof(int32_t));
    uint32_t* h_y = (uint32_t*)malloc(n * sizeof(uint32_t));
    if (!h_x || !h_f || !h_y) return 4;
    uint64_t state = 88172645463325252ull;   /* xorshift64 inputs */
    for (size_t i = 0; i < n; ++i) {
        state ^= state << 13;
        state ^= state >> 7;
        state ^= state << 17;
        h_x[i] = (uint32_t)state;
        h_f[i] = (int32_t)((state >> 40) & 1u);
    }

    hipStream_t stream;
    CHECK_HIP(hipStreamCreate(&stream));
    uint32_t *d_x, *d_out;
    int32_t* d_f;
    unsigned long long* d_count;
    CHECK_HIP(hipMalloc((void**)&d_x, n * sizeof(uint32_t)));
    CHECK_HIP(hipMalloc((void**)&d_out, n * sizeof(uint32_t)));
    CHECK_HIP(hipMalloc((void**)&d_f, n * sizeof(int32_t)));
    CHECK_HIP(hipMalloc((void**)&d_count, sizeof(unsigned long long)));
    CHECK_HIP(hipMemcpyAsync(d_x, h_x, n * sizeof(uint32_t), hipMemcpyHostToDevice, stream));
    CHECK_HIP(hipMemcpyAsync(d_f, h_f, n * sizeof(int32_t), hipMemcpyHostToDevice, stream));

    /* exclusive scan in place, modulo 2^32 */
    CHECK_DWS(scan_exclusive(d_x, d_x, n, DWS_UINT32, stream));
    CHECK_HIP(hipMemcpyAsync(h_y, d_x, n * sizeof(uint32_t), hipMemcpyDeviceToHost, stream));
    CHECK_HIP(hipStreamSynchronize(stream));
    uint32_t running = 0u;
    for (size_t i = 0; i < n; ++i) {
        if (h_y[i] != running) {
            fprintf(stderr, "scan mismatch at %zu: %u != %u\n", i, h_y[i], running);
            return 1;
        }
        running += h_x[i];
    }

    /* compaction of the original values by the flags */
    CHECK_HIP(hipMemcpyAsync(d_x, h_x, n * sizeof(uint32_t), hipMemcpyHostToDevice, stream));
    CHECK_DWS(dws_select_flagged(d_x, d_f, d_out, n, DWS_UINT32, d_count, stream));
    unsigned long long count = 0;
    CHECK_HIP(hipMemcpyAsync(&count, d_count, sizeof(count), hipMemcpyDeviceToHost, stream));
    CHECK_HIP(hipMemcpyAsync(h_y, d_out, n * sizeof(uint32_t), hipMemcpyDeviceToHost, stream));
    CHECK_HIP(hipStreamSynchronize(stream));
    size_t k = 0;
    for (size_t i = 0; i < n; ++i) {
        if (h_f[i] == 0) continue;
        if (k >= count || h_y[k] != h_x[i]) {
            fprintf(stderr, "select mismatch at output %zu\n", k);
            return 1;
        }
        ++k;
    }
    if (k != count) {
        fprintf(stderr, "select count %llu, expected %zu\n", count, k);
        return 1;
    }

    /* the exclusive scan again, as two shards of n / 2 and n - n / 2 elements:
     * totals (dws_reduce), their exclusive scan, then each shard scanned
     * seeded with its offset (dws_scan_seeded), all enqueued on the stream */
    uint32_t *d_tot, *d_off;
    CHECK_HIP(hipMalloc((void**)&d_tot, 2 * sizeof(uint32_t)));
    CHECK_HIP(hipMalloc((void**)&d_off, 2 * sizeof(uint32_t)));
    const size_t half = n / 2;
    CHECK_DWS(dws_reduce(d_x, half, DWS_UINT32, d_tot, stream));
    CHECK_DWS(dws_reduce(d_x + half, n - half, DWS_UINT32, d_tot + 1, stream));
    CHECK_DWS(scan_exclusive(d_tot, d_off, 2, DWS_UINT32, stream));
    CHECK_DWS(dws_scan_seeded(d_x, d_out, half, DWS_UINT32, 1, d_off, stream));
    CHECK_DWS(dws_scan_seeded(d_x + half, d_out + half, n - half, DWS_UINT32, 1, d_off + 1, stream));
    CHECK_HIP(hipMemcpyAsync(h_y, d_out, n * sizeof(uint32_t), hipMemcpyDeviceToHost, stream));
    CHECK_HIP(hipStreamSynchronize(stream));
    running = 0u;
    for (size_t i = 0; i < n; ++i) {
        if (h_y[i] != running) {
            fprintf(stderr, "two-shard scan mismatch at %zu: %u != %u\n", i, h_y[i], running);
            return 1;
        }
        running += h_x[i];
    }
    CHECK_HIP(hipFree(d_tot));
    CHECK_HIP(hipFree(d_off));

    /* errors come back as status codes, before any work is enqueued: with
     * n >= 2, d_x + 1 .. d_x + n overlaps d_x .. d_x + n - 1 without equalling it */
    if (n >= 2 && scan_exclusive(d_x, d_x + 1, n, DWS_UINT32, stream) != DWS_ERR_OVERLAP) {
        fprintf(stderr, "a partially overlapping output was not rejected\n");
        return 1;
    }

    CHECK_HIP(hipFree(d_x));
    CHECK_HIP(hipFree(d_out));
    CHECK_HIP(hipFree(d_f));
    CHECK_HIP(hipFree(d_count));
    CHECK_DWS(dws_release_workspaces());
    CHECK_HIP(hipStreamDestroy(stream));
    printf("scan_from_c: n=%zu exclusive scan, compaction (%llu selected) and two-shard scan correct\n", n, count);
    free(h_x);
    free(h_f);
    free(h_y);
    return 0;
}
