/*
 * vrc_c_check.c -- the C ABI of include/vrc.h used from plain C, with no
 * Python and no PyTorch: rank buffers come from hipMalloc and the HIP
 * runtime is /opt/rocm's.  Every collective runs in every mode on int32 and
 * on fp32 holding small integers, whose sums are exact in any order, and is
 * checked against the sum computed here; so is the bucketed all-reduce, with
 * and without its per-bucket events.  Prints "ok" and exits 0, or
 * prints the first mismatch and exits 1.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "vrc.h"

#define N 8
#define CHECK_HIP(x)                                                                  \
    do {                                                                              \
        hipError_t e_ = (x);                                                          \
        if (e_ != hipSuccess) {                                                       \
            fprintf(stderr, "HIP error %d at %s:%d\n", (int)e_, __FILE__, __LINE__); \
            return 2;                                                                 \
        }                                                                             \
    } while (0)

static int32_t value(int r, size_t i) { return (int32_t)((i * 2654435761u + (unsigned)r * 40503u) % 61u) - 30; }

/* Every rank's all-reduce output against the exact sums. */
static int check_sums(vrc_dtype_t dt, void* const* y, size_t count, const int64_t* want, unsigned char* got,
                      const char* what, int mode)
{
    const size_t esz = 4;
    for (int r = 0; r < N; r++) {
        CHECK_HIP(hipMemcpy(got, y[r], count * esz, hipMemcpyDeviceToHost));
        for (size_t i = 0; i < count; i++) {
            int64_t v;
            if (dt == VRC_INT32) {
                int32_t t;
                memcpy(&t, got + i * esz, 4);
                v = t;
            } else {
                float f;
                memcpy(&f, got + i * esz, 4);
                v = (int64_t)f;
                if ((float)v != f) v = INT64_MIN;
            }
            if (v != want[i]) {
                fprintf(stderr, "%s dtype %d mode %d rank %d element %zu: %lld != %lld\n", what, (int)dt, mode, r, i,
                        (long long)v, (long long)want[i]);
                return 1;
            }
        }
    }
    return 0;
}

static int run_dtype(vrc_dtype_t dt, size_t count)
{
    const size_t esz = 4;
    void* x[N];
    void* y[N];
    void* rs[N];
    void* ag[N];
    unsigned char* host = (unsigned char*)malloc(count * esz * N);
    int64_t* want = (int64_t*)calloc(count, sizeof(int64_t));
    unsigned char* got = (unsigned char*)malloc(count * esz * N);
    if (!host || !want || !got) return 2;
    for (int r = 0; r < N; r++) {
        for (size_t i = 0; i < count; i++) {
            int32_t v = value(r, i);
            want[i] += v;
            if (dt == VRC_INT32) memcpy(host + i * esz, &v, 4);
            else {
                float f = (float)v;
                memcpy(host + i * esz, &f, 4);
            }
        }
        CHECK_HIP(hipMalloc(&x[r], count * esz));
        CHECK_HIP(hipMalloc(&y[r], count * esz));
        CHECK_HIP(hipMalloc(&rs[r], count * esz));       /* room for any chunk */
        CHECK_HIP(hipMalloc(&ag[r], count * esz * N));
        CHECK_HIP(hipMemcpy(x[r], host, count * esz, hipMemcpyHostToDevice));
    }
    const vrc_mode_t modes[] = {VRC_RING, VRC_FUSED, VRC_RING_CHAINED, VRC_RING_ORDER, VRC_HD, VRC_HD_ORDER, VRC_SELECT,
                                VRC_TREE};
    for (size_t m = 0; m < sizeof(modes) / sizeof(modes[0]); m++) {
        /* The tree is an all-gather algorithm: the reduce collectives refuse it
         * (and run fused here, so the checks below still apply to them). */
        vrc_mode_t reduce_mode = modes[m];
        if (modes[m] == VRC_TREE) {
            if (vrc_allreduce((const void* const*)x, y, N, count, dt, VRC_SUM, VRC_TREE, NULL) != VRC_ERR_UNSUPPORTED ||
                vrc_reduce_scatter((const void* const*)x, rs, N, count, 1, dt, VRC_SUM, VRC_TREE, NULL) !=
                    VRC_ERR_UNSUPPORTED) {
                fprintf(stderr, "VRC_TREE accepted by a reduce collective\n");
                return 1;
            }
            reduce_mode = VRC_FUSED;
        }
        vrc_status_t st = vrc_allreduce((const void* const*)x, y, N, count, dt, VRC_SUM, reduce_mode, NULL);
        if (st != VRC_OK) {
            fprintf(stderr, "vrc_allreduce mode %d: %s\n", (int)modes[m], vrc_status_string(st));
            return 1;
        }
        st = vrc_reduce_scatter((const void* const*)x, rs, N, count, 1, dt, VRC_SUM, reduce_mode, NULL);
        if (st != VRC_OK) {
            fprintf(stderr, "vrc_reduce_scatter mode %d: %s\n", (int)modes[m], vrc_status_string(st));
            return 1;
        }
        st = vrc_all_gather((const void* const*)x, ag, N, count, 1, dt, modes[m], NULL);
        if (st != VRC_OK) {
            fprintf(stderr, "vrc_all_gather mode %d: %s\n", (int)modes[m], vrc_status_string(st));
            return 1;
        }
        CHECK_HIP(hipDeviceSynchronize());
        for (int r = 0; r < N; r++) {
            CHECK_HIP(hipMemcpy(got, y[r], count * esz, hipMemcpyDeviceToHost));
            for (size_t i = 0; i < count; i++) {
                int64_t v;
                if (dt == VRC_INT32) {
                    int32_t t;
                    memcpy(&t, got + i * esz, 4);
                    v = t;
                } else {
                    float f;
                    memcpy(&f, got + i * esz, 4);
                    v = (int64_t)f;
                    if ((float)v != f) v = INT64_MIN;
                }
                if (v != want[i]) {
                    fprintf(stderr, "all-reduce dtype %d mode %d rank %d element %zu: %lld != %lld\n", (int)dt,
                            (int)modes[m], r, i, (long long)v, (long long)want[i]);
                    return 1;
                }
            }
            size_t off, len;
            if (vrc_chunk_range(count, N, r, &off, &len) != VRC_OK) return 1;
            CHECK_HIP(hipMemcpy(got, rs[r], len * esz, hipMemcpyDeviceToHost));
            for (size_t k = 0; k < len; k++) {
                int64_t v;
                if (dt == VRC_INT32) {
                    int32_t t;
                    memcpy(&t, got + k * esz, 4);
                    v = t;
                } else {
                    float f;
                    memcpy(&f, got + k * esz, 4);
                    v = (int64_t)f;
                }
                if (v != want[off + k]) {
                    fprintf(stderr, "reduce-scatter dtype %d mode %d chunk %d element %zu\n", (int)dt,
                            (int)modes[m], r, k);
                    return 1;
                }
            }
            /* all-gather: slab q of every output is input q */
            for (int q = 0; q < N; q++) {
                CHECK_HIP(hipMemcpy(got, (unsigned char*)ag[r] + (size_t)q * count * esz, count * esz,
                                    hipMemcpyDeviceToHost));
                for (size_t i = 0; i < count; i++) {
                    int32_t t;
                    memcpy(&t, got + i * esz, 4);
                    int32_t v = value(q, i);
                    int32_t w;
                    if (dt == VRC_INT32) w = v;
                    else {
                        float f = (float)v;
                        memcpy(&w, &f, 4);
                    }
                    if (t != w) {
                        fprintf(stderr, "all-gather dtype %d mode %d rank %d slab %d element %zu\n", (int)dt,
                                (int)modes[m], r, q, i);
                        return 1;
                    }
                }
            }
        }
    }
    /* The bucketed all-reduce on its own stream: buckets of 100,003 elements
     * (the last one shorter), each gated by an event recorded on that stream,
     * and the same call with no events. */
    {
        const size_t bucket = 100003;
        const int nb = (int)((count + bucket - 1) / bucket);
        hipStream_t s;
        CHECK_HIP(hipStreamCreate(&s));
        vrc_event_t* ev = (vrc_event_t*)malloc((size_t)nb * sizeof *ev);
        if (!ev) return 2;
        for (int k = 0; k < nb; k++) {
            hipEvent_t e;
            CHECK_HIP(hipEventCreateWithFlags(&e, hipEventDisableTiming));
            CHECK_HIP(hipEventRecord(e, s));
            ev[k] = (vrc_event_t)e;
        }
        const vrc_mode_t bmodes[] = {VRC_FUSED, VRC_RING, VRC_SELECT};
        for (size_t m = 0; m < sizeof(bmodes) / sizeof(bmodes[0]); m++) {
            for (int with_events = 0; with_events < 2; with_events++) {
                for (int r = 0; r < N; r++) CHECK_HIP(hipMemsetAsync(y[r], 0, count * esz, s));
                vrc_status_t st = vrc_allreduce_bucketed((const void* const*)x, y, N, count, dt, VRC_SUM, bmodes[m],
                                                         bucket, with_events ? ev : NULL, with_events ? nb : 0,
                                                         (vrc_stream_t)s);
                if (st != VRC_OK) {
                    fprintf(stderr, "vrc_allreduce_bucketed mode %d: %s\n", (int)bmodes[m], vrc_status_string(st));
                    return 1;
                }
                CHECK_HIP(hipStreamSynchronize(s));
                if (check_sums(dt, y, count, want, got, "bucketed all-reduce", (int)bmodes[m])) return 1;
            }
        }
        for (int k = 0; k < nb; k++) CHECK_HIP(hipEventDestroy((hipEvent_t)ev[k]));
        free(ev);
        CHECK_HIP(hipStreamDestroy(s));
    }
    for (int r = 0; r < N; r++) {
        CHECK_HIP(hipFree(x[r]));
        CHECK_HIP(hipFree(y[r]));
        CHECK_HIP(hipFree(rs[r]));
        CHECK_HIP(hipFree(ag[r]));
    }
    free(host);
    free(want);
    free(got);
    return 0;
}

int main(void)
{
    if (vrc_version() != VRC_VERSION) {
        fprintf(stderr, "library version %d, header %d\n", vrc_version(), VRC_VERSION);
        return 1;
    }
    int rc = run_dtype(VRC_INT32, 1000003);
    if (!rc) rc = run_dtype(VRC_FP32, 1000003);
    if (!rc) rc = run_dtype(VRC_INT32, 13); /* fewer than two elements per rank */
    if (rc) return rc;
    printf("ok\n");
    return 0;
}
