/*
 * mgs_c_consumer.c — a plain C program that uses libmgs.so through
 * include/mgs.h alone: HIP runtime calls for device memory and a stream, the
 * library's entry points for the work, no Python and no torch.
 *
 * Usage: mgs_c_consumer DIR
 * DIR/cases.txt holds one case per line: "<kind> <M> <K> <G> <arg>" with
 * kind dim0 (the library's own workspace), dim0_ws (a workspace of the size
 * mgs_dim0_workspace_bytes reports, allocated and zeroed here), dim1 or mx;
 * arg is the flags (dim0, dim0_ws, dim1) or the MX mode. Case i reads
 * DIR/i.x (M*K bf16 values) and, except for mx, DIR/i.off (G int32 end
 * offsets), and writes DIR/i.q (M*K E4M3 bytes) and DIR/i.s (the scales:
 * G*K or M*G float32, or M*K/32 E8M0 bytes). Exit status 0 when every call
 * returned MGS_OK and every file was written.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "mgs.h"

#define HIP_CHECK(call)                                                                   \
    do {                                                                                  \
        hipError_t e_ = (call);                                                           \
        if (e_ != hipSuccess) {                                                           \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));             \
            exit(2);                                                                      \
        }                                                                                 \
    } while (0)

#define MGS_CHECK(call)                                                                   \
    do {                                                                                  \
        int s_ = (call);                                                                  \
        if (s_ != MGS_OK) {                                                               \
            fprintf(stderr, "%s returned %s (hip error %d)\n", #call, mgs_status_string(s_), \
                    mgs_last_hip_error());                                                \
            exit(3);                                                                      \
        }                                                                                 \
    } while (0)

static void *read_file(const char *dir, int i, const char *ext, size_t n) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%d.%s", dir, i, ext);
    FILE *f = fopen(path, "rb");
    if (!f) { perror(path); exit(4); }
    void *p = malloc(n ? n : 1);
    if (!p || fread(p, 1, n, f) != n) { fprintf(stderr, "short read: %s\n", path); exit(4); }
    fclose(f);
    return p;
}

static void write_file(const char *dir, int i, const char *ext, const void *p, size_t n) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%d.%s", dir, i, ext);
    FILE *f = fopen(path, "wb");
    if (!f || fwrite(p, 1, n, f) != n) { fprintf(stderr, "cannot write %s\n", path); exit(5); }
    fclose(f);
}

int main(int argc, char **argv) {
    if (argc != 2) { fprintf(stderr, "usage: %s DIR\n", argv[0]); return 1; }
    const char *dir = argv[1];
    char path[4096];
    snprintf(path, sizeof path, "%s/cases.txt", dir);
    FILE *cases = fopen(path, "r");
    if (!cases) { perror(path); return 4; }
    hipStream_t stream;
    HIP_CHECK(hipStreamCreate(&stream));
    char kind[16];
    long long M, K, G, arg;
    int i = 0;
    while (fscanf(cases, "%15s %lld %lld %lld %lld", kind, &M, &K, &G, &arg) == 5) {
        const int mx = strcmp(kind, "mx") == 0, dim1 = strcmp(kind, "dim1") == 0;
        const size_t xb = (size_t)(M * K) * 2, qb = (size_t)(M * K);
        const size_t sb = mx ? (size_t)(M * (K / 32)) : (size_t)(dim1 ? M * G : G * K) * sizeof(float);
        void *hx = read_file(dir, i, "x", xb);
        void *hoff = mx ? NULL : read_file(dir, i, "off", (size_t)G * sizeof(int32_t));
        void *dx, *dq, *ds, *doff = NULL, *dws = NULL;
        HIP_CHECK(hipMalloc(&dx, xb));
        HIP_CHECK(hipMalloc(&dq, qb));
        HIP_CHECK(hipMalloc(&ds, sb));
        HIP_CHECK(hipMemcpyAsync(dx, hx, xb, hipMemcpyHostToDevice, stream));
        if (!mx) {
            HIP_CHECK(hipMalloc(&doff, (size_t)G * sizeof(int32_t)));
            HIP_CHECK(hipMemcpyAsync(doff, hoff, (size_t)G * sizeof(int32_t), hipMemcpyHostToDevice, stream));
        }
        if (strcmp(kind, "dim0") == 0) {
            MGS_CHECK(mgs_quant_groups_dim0(dx, M, K, doff, (int32_t)G, (uint32_t)arg, dq, ds, stream));
        } else if (strcmp(kind, "dim0_ws") == 0) {
            int64_t wsb = 0;
            MGS_CHECK(mgs_dim0_workspace_bytes(M, K, &wsb));
            if (wsb > 0) {
                HIP_CHECK(hipMalloc(&dws, (size_t)wsb));
                HIP_CHECK(hipMemsetAsync(dws, 0, (size_t)wsb, stream));
            }
            /* twice on the same workspace: every call leaves it zero again */
            MGS_CHECK(mgs_quant_groups_dim0_ws(dx, M, K, doff, (int32_t)G, (uint32_t)arg, dq, ds, dws,
                                               wsb, stream));
            MGS_CHECK(mgs_quant_groups_dim0_ws(dx, M, K, doff, (int32_t)G, (uint32_t)arg, dq, ds, dws,
                                               wsb, stream));
        } else if (dim1) {
            MGS_CHECK(mgs_quant_groups_dim1(dx, M, K, doff, (int32_t)G, (uint32_t)arg, dq, ds, stream));
        } else if (mx) {
            MGS_CHECK(mgs_mx_quant_dim0(dx, M, K, NULL, 0, (int)arg, dq, (uint8_t *)ds, stream));
        } else {
            fprintf(stderr, "unknown case kind %s\n", kind);
            return 1;
        }
        void *hq = malloc(qb ? qb : 1), *hs = malloc(sb ? sb : 1);
        HIP_CHECK(hipMemcpyAsync(hq, dq, qb, hipMemcpyDeviceToHost, stream));
        HIP_CHECK(hipMemcpyAsync(hs, ds, sb, hipMemcpyDeviceToHost, stream));
        HIP_CHECK(hipStreamSynchronize(stream));
        write_file(dir, i, "q", hq, qb);
        write_file(dir, i, "s", hs, sb);
        HIP_CHECK(hipFree(dx));
        HIP_CHECK(hipFree(dq));
        HIP_CHECK(hipFree(ds));
        if (doff) HIP_CHECK(hipFree(doff));
        if (dws) HIP_CHECK(hipFree(dws));
        free(hx);
        free(hoff);
        free(hq);
        free(hs);
        printf("case %d (%s %lld x %lld) ok\n", i, kind, M, K);
        fflush(stdout);
        ++i;
    }
    fclose(cases);
    HIP_CHECK(hipStreamDestroy(stream));
    return i > 0 ? 0 : 1;
}
