// vrc_api.hip -- the C ABI of include/vrc.h: argument checks, chunk
// partition, ring schedule, launch sizing and dtype/N dispatch.
//
// The schedule follows the pages cited in vrc.h: reduce-scatter step s has
// rank r add the partial of chunk (r-1-s) held by rank r-1 into its own
// copy (ai6s.net/6a102b5410ee7a33f2746c06.html, "hcomm 与 HCCL 的关系",
// ReduceScatter listing; hwcomputing.csdn.net/6a0dc11a10ee7a33f273f7fd.html,
// "Ring 通信为什么常见"), and all-gather step s has rank r copy chunk (r-s)
// from rank r-1.  A "send" is the receiving rank's kernel reading the
// neighbour's buffer in place (the zero-copy path of the first page's
// "hcomm 的数据传输路径" section): every virtual rank lives in this GPU's HBM.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>

// The C ABI keeps default visibility; everything else in the library is hidden.
#pragma GCC visibility push(default)
#include "vrc.h"
#pragma GCC visibility pop

#include "vrc_host.hpp"

namespace vrc {
namespace host {
thread_local int g_last_hip_error = 0;
thread_local Plan* g_plan = nullptr;
}  // namespace host
}  // namespace vrc

namespace {

using namespace vrc::host;
using vrc::kMaxRanks;

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

hipError_t cu_count(int* out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev >= 0 && dev < kMaxDevices) {
        int c = g_cu_count[dev].load(std::memory_order_relaxed);
        if (c > 0) {
            *out = c;
            return hipSuccess;
        }
    }
    int c = 0;
    e = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    if (c < 1) c = 1;
    if (dev >= 0 && dev < kMaxDevices) g_cu_count[dev].store(c, std::memory_order_relaxed);
    *out = c;
    return hipSuccess;
}

bool overlap(uintptr_t a, uint64_t na, uintptr_t b, uint64_t nb)
{
    if (na == 0 || nb == 0) return false;
    return a < b + nb && b < a + na;
}

// Validation shared by the three calls.  recv_bytes[r] is rank r's output
// size.  allow_in_place: recv[r] == send[r] is accepted (all-reduce only).
vrc_status_t check_buffers(const void* const* send, void* const* recv, int n, uint64_t send_bytes,
                           const uint64_t* recv_bytes, bool allow_in_place)
{
    for (int r = 0; r < n; r++) {
        if (send_bytes && !send[r]) return VRC_ERR_INVALID_ARG;
        if (recv_bytes[r] && !recv[r]) return VRC_ERR_INVALID_ARG;
    }
    for (int r = 0; r < n; r++) {
        const uintptr_t d = (uintptr_t)recv[r];
        for (int q = 0; q < n; q++) {
            const uintptr_t s = (uintptr_t)send[q];
            if (q == r && allow_in_place && s == d) continue;
            if (overlap(d, recv_bytes[r], s, send_bytes)) return VRC_ERR_ALIAS;
            if (q != r && overlap(d, recv_bytes[r], (uintptr_t)recv[q], recv_bytes[q])) return VRC_ERR_ALIAS;
        }
    }
    return VRC_OK;
}

// Counts above 2^56 elements are rejected: every byte size computed from
// them (at most count * 16 ranks * 4 bytes) then fits in 64 bits.
constexpr uint64_t kMaxCount = 1ull << 56;

// The enum arguments of the C ABI hold whatever int a C caller passes.  In
// C++ an enum object whose value lies outside its enumerators' range may not
// be read as that enum, so every entry point reads them as plain ints (from
// the object's bytes) and the implementations check the ints before turning
// them back into enums.
template <class E>
int raw(const E& e)
{
    static_assert(sizeof(E) == sizeof(int), "the C enums of vrc.h are int-sized");
    int v;
    std::memcpy(&v, &e, sizeof v);
    return v;
}

bool dtype_valid(int d) { return d >= VRC_INT32 && d <= VRC_BF16; }
bool mode_valid(int m) { return m >= VRC_RING && m <= VRC_TREE; }

vrc_status_t check_common(const void* const* send, void* const* recv, int n, uint64_t count, int dtype)
{
    if (!send || !recv) return VRC_ERR_INVALID_ARG;
    if (n < 1 || n > kMaxRanks) return VRC_ERR_INVALID_ARG;
    if (count > kMaxCount) return VRC_ERR_INVALID_ARG;
    if (!dtype_valid(dtype)) return VRC_ERR_UNSUPPORTED;
    return VRC_OK;
}


vrc_status_t run(Coll coll, vrc_mode_t mode, vrc_dtype_t dt, const void* const* send, void* const* recv, int n,
                 uint64_t count, uint64_t outer, hipStream_t st)
{
    int cus = 256;  // a plan launches nothing and needs no device
    if (!g_plan) {
        hipError_t e = cu_count(&cus);
        if (e != hipSuccess) return hip_fail(e);
        (void)hipGetLastError();  // start from a clean per-thread error state
    }
    const char* x[kMaxRanks];
    char* y[kMaxRanks];
    for (int r = 0; r < n; r++) {
        x[r] = static_cast<const char*>(send[r]);
        y[r] = static_cast<char*>(recv[r]);
    }
    switch (dt) {
    case VRC_INT32: return run_typed<vrc::I32>(coll, mode, x, y, n, count, outer, cus, st);
    case VRC_FP32: return run_typed<vrc::F32>(coll, mode, x, y, n, count, outer, cus, st);
    case VRC_FP16: return run_typed<vrc::F16>(coll, mode, x, y, n, count, outer, cus, st);
    case VRC_BF16: return run_typed<vrc::BF16>(coll, mode, x, y, n, count, outer, cus, st);
    }
    return VRC_ERR_UNSUPPORTED;
}

// VRC_SELECT: halving-doubling for power-of-two rank counts and inputs of at
// most VRC_SELECT_HD_MAX_BYTES per rank (log2 N steps win while launches
// dominate).  For the all-gather at other rank counts, the binomial tree
// while it saves launches ((N-1) - 2 ceil(log2 N) of them) and each rank's
// input is at most VRC_SELECT_TREE_BYTES_PER_SAVED_LAUNCH per launch saved
// (it copies more slabs than the ring).  Else the ring.
vrc_mode_t resolve_mode(vrc_mode_t m, int n, uint64_t bytes_per_rank, Coll coll)
{
    if (m != VRC_SELECT) return m;
    const bool pow2 = (n & (n - 1)) == 0;
    if (pow2 && bytes_per_rank <= VRC_SELECT_HD_MAX_BYTES) return VRC_HD;
    if (coll == Coll::AG && !pow2) {
        int lg = 0;
        while ((1 << lg) < n) lg++;
        const int saved = (n - 1) - 2 * lg;
        if (saved > 0 && bytes_per_rank <= (uint64_t)saved * VRC_SELECT_TREE_BYTES_PER_SAVED_LAUNCH) return VRC_TREE;
    }
    return VRC_RING;
}

// Halving-doubling pairs rank r with r XOR d, so it needs a power of two.
bool ranks_ok_for(vrc_mode_t m, int n)
{
    if (m != VRC_HD && m != VRC_HD_ORDER) return true;
    return (n & (n - 1)) == 0;
}

// The collectives, on validated int arguments (see raw()).
vrc_status_t allreduce_impl(const void* const* send, void* const* recv, int nranks, size_t count, int dtype, int op,
                            int mode_raw, hipStream_t stream)
{
    vrc_status_t rc = check_common(send, recv, nranks, count, dtype);
    if (rc) return rc;
    if (op != VRC_SUM || !mode_valid(mode_raw) || mode_raw == VRC_TREE) return VRC_ERR_UNSUPPORTED;
    const vrc_dtype_t dt = static_cast<vrc_dtype_t>(dtype);
    const uint64_t bytes = (uint64_t)count * (uint64_t)esize(dt);
    const vrc_mode_t mode = resolve_mode(static_cast<vrc_mode_t>(mode_raw), nranks, bytes, Coll::AR);
    if (!ranks_ok_for(mode, nranks)) return VRC_ERR_INVALID_ARG;
    uint64_t rb[kMaxRanks];
    for (int r = 0; r < nranks; r++) rb[r] = bytes;
    rc = check_buffers(send, recv, nranks, bytes, rb, true);
    if (rc) return rc;
    if (count == 0) return VRC_OK;
    return run(Coll::AR, mode, dt, send, recv, nranks, count, 1, stream);
}

vrc_status_t bucketed_impl(const void* const* send, void* const* recv, int nranks, size_t count, int dtype, int op,
                           int mode_raw, size_t bucket, const vrc_event_t* ready, int nready, hipStream_t stream)
{
    vrc_status_t rc = check_common(send, recv, nranks, count, dtype);
    if (rc) return rc;
    if (op != VRC_SUM || !mode_valid(mode_raw) || mode_raw == VRC_TREE) return VRC_ERR_UNSUPPORTED;
    const vrc_dtype_t dt = static_cast<vrc_dtype_t>(dtype);
    const vrc_mode_t mode = static_cast<vrc_mode_t>(mode_raw);
    if (!ranks_ok_for(mode, nranks)) return VRC_ERR_INVALID_ARG;
    if (bucket == 0) return VRC_ERR_INVALID_ARG;
    const uint64_t nb = count == 0 ? 0 : (count - 1) / bucket + 1;
    if (ready ? (nready < 0 || (uint64_t)nready != nb) : nready != 0) return VRC_ERR_INVALID_ARG;
    if (ready)
        for (uint64_t k = 0; k < nb; k++)
            if (!ready[k]) return VRC_ERR_INVALID_ARG;
    const int E = esize(dt);
    uint64_t rb[kMaxRanks];
    for (int r = 0; r < nranks; r++) rb[r] = (uint64_t)count * E;
    rc = check_buffers(send, recv, nranks, (uint64_t)count * E, rb, true);
    if (rc) return rc;
    const void* xs[kMaxRanks];
    void* ys[kMaxRanks];
    for (uint64_t k = 0; k < nb; k++) {
        const uint64_t off = k * bucket, len = count - off < bucket ? count - off : bucket;
        if (ready && !g_plan) {
            const hipError_t e = hipStreamWaitEvent(stream, (hipEvent_t)ready[k], 0);
            if (e != hipSuccess) return hip_fail(e);
        }
        for (int r = 0; r < nranks; r++) {
            xs[r] = static_cast<const char*>(send[r]) + off * E;
            ys[r] = static_cast<char*>(recv[r]) + off * E;
        }
        rc = run(Coll::AR, resolve_mode(mode, nranks, len * E, Coll::AR), dt, xs, ys, nranks, len, 1, stream);
        if (rc) return rc;
    }
    return VRC_OK;
}

vrc_status_t reduce_scatter_impl(const void* const* send, void* const* recv, int nranks, size_t count, size_t outer,
                                 int dtype, int op, int mode_raw, hipStream_t stream)
{
    vrc_status_t rc = check_common(send, recv, nranks, count, dtype);
    if (rc) return rc;
    if (op != VRC_SUM || !mode_valid(mode_raw) || mode_raw == VRC_TREE) return VRC_ERR_UNSUPPORTED;
    const vrc_dtype_t dt = static_cast<vrc_dtype_t>(dtype);
    const int E = esize(dt);
    const vrc_mode_t mode = resolve_mode(static_cast<vrc_mode_t>(mode_raw), nranks, (uint64_t)count * E, Coll::RS);
    if (!ranks_ok_for(mode, nranks)) return VRC_ERR_INVALID_ARG;
    if (outer == 0 || count % outer != 0) return VRC_ERR_INVALID_ARG;
    if (outer > 1 && (count / outer) % (uint64_t)nranks != 0) return VRC_ERR_INVALID_ARG;
    uint64_t rb[kMaxRanks];
    for (int c = 0; c < nranks; c++) {
        if (outer == 1) {
            uint64_t off, len;
            chunk_range(count, nranks, c, &off, &len);
            rb[c] = len * E;
        } else {
            rb[c] = (uint64_t)count / (uint64_t)nranks * E;
        }
    }
    rc = check_buffers(send, recv, nranks, (uint64_t)count * E, rb, false);
    if (rc) return rc;
    if (count == 0) return VRC_OK;
    return run(Coll::RS, mode, dt, send, recv, nranks, count, outer, stream);
}

vrc_status_t all_gather_impl(const void* const* send, void* const* recv, int nranks, size_t count, size_t outer,
                             int dtype, int mode_raw, hipStream_t stream)
{
    vrc_status_t rc = check_common(send, recv, nranks, count, dtype);
    if (rc) return rc;
    if (!mode_valid(mode_raw)) return VRC_ERR_UNSUPPORTED;
    const vrc_dtype_t dt = static_cast<vrc_dtype_t>(dtype);
    const int E = esize(dt);
    const vrc_mode_t mode = resolve_mode(static_cast<vrc_mode_t>(mode_raw), nranks, (uint64_t)count * E, Coll::AG);
    if (!ranks_ok_for(mode, nranks)) return VRC_ERR_INVALID_ARG;
    if (outer == 0 || count % outer != 0) return VRC_ERR_INVALID_ARG;
    uint64_t rb[kMaxRanks];
    for (int r = 0; r < nranks; r++) rb[r] = (uint64_t)count * (uint64_t)nranks * E;
    rc = check_buffers(send, recv, nranks, (uint64_t)count * E, rb, false);
    if (rc) return rc;
    if (count == 0) return VRC_OK;
    return run(Coll::AG, mode, dt, send, recv, nranks, count, outer, stream);
}

}  // namespace

// ============================================================================
// C ABI
// ============================================================================
extern "C" {

vrc_status_t vrc_plan(vrc_coll_t coll, const void* const* send, void* const* recv, int nranks, size_t count,
                      size_t outer, vrc_dtype_t dtype, vrc_mode_t mode, vrc_op_desc* ops, int cap, int* n_ops,
                      int* n_launches)
{
    if (!n_ops || !n_launches || cap < 0 || (cap > 0 && !ops)) return VRC_ERR_INVALID_ARG;
    Plan plan = {ops, cap, 0, 0};
    g_plan = &plan;
    vrc_status_t rc = VRC_ERR_UNSUPPORTED;
    const int dt = raw(dtype), md = raw(mode);
    switch (raw(coll)) {
    case VRC_COLL_ALLREDUCE: rc = allreduce_impl(send, recv, nranks, count, dt, VRC_SUM, md, nullptr); break;
    case VRC_COLL_REDUCE_SCATTER: rc = reduce_scatter_impl(send, recv, nranks, count, outer, dt, VRC_SUM, md, nullptr); break;
    case VRC_COLL_ALL_GATHER: rc = all_gather_impl(send, recv, nranks, count, outer, dt, md, nullptr); break;
    case VRC_COLL_ALLREDUCE_BUCKETED:
        rc = bucketed_impl(send, recv, nranks, count, dt, VRC_SUM, md, outer, nullptr, 0, nullptr);
        break;
    default: break;
    }
    g_plan = nullptr;
    *n_ops = plan.n;
    *n_launches = plan.launches;
    if (rc == VRC_OK && plan.n > cap) return VRC_ERR_INVALID_ARG;
    return rc;
}

vrc_status_t vrc_allreduce(const void* const* send, void* const* recv, int nranks, size_t count,
                           vrc_dtype_t dtype, vrc_op_t op, vrc_mode_t mode, vrc_stream_t stream)
{
    return allreduce_impl(send, recv, nranks, count, raw(dtype), raw(op), raw(mode), (hipStream_t)stream);
}

vrc_status_t vrc_allreduce_bucketed(const void* const* send, void* const* recv, int nranks, size_t count,
                                    vrc_dtype_t dtype, vrc_op_t op, vrc_mode_t mode, size_t bucket,
                                    const vrc_event_t* ready, int nready, vrc_stream_t stream)
{
    return bucketed_impl(send, recv, nranks, count, raw(dtype), raw(op), raw(mode), bucket, ready, nready,
                         (hipStream_t)stream);
}

vrc_status_t vrc_reduce_scatter(const void* const* send, void* const* recv, int nranks, size_t count,
                                size_t outer, vrc_dtype_t dtype, vrc_op_t op, vrc_mode_t mode,
                                vrc_stream_t stream)
{
    return reduce_scatter_impl(send, recv, nranks, count, outer, raw(dtype), raw(op), raw(mode), (hipStream_t)stream);
}

vrc_status_t vrc_all_gather(const void* const* send, void* const* recv, int nranks, size_t count,
                            size_t outer, vrc_dtype_t dtype, vrc_mode_t mode, vrc_stream_t stream)
{
    return all_gather_impl(send, recv, nranks, count, outer, raw(dtype), raw(mode), (hipStream_t)stream);
}

vrc_status_t vrc_chunk_range(size_t count, int nranks, int chunk, size_t* offset, size_t* length)
{
    if (nranks < 1 || chunk < 0 || chunk >= nranks || !offset || !length) return VRC_ERR_INVALID_ARG;
    uint64_t off, len;
    chunk_range(count, nranks, chunk, &off, &len);
    *offset = (size_t)off;
    *length = (size_t)len;
    return VRC_OK;
}

const char* vrc_status_string(vrc_status_t status)
{
    switch (raw(status)) {
    case VRC_OK: return "VRC_OK: success";
    case VRC_ERR_INVALID_ARG: return "VRC_ERR_INVALID_ARG: invalid argument (null pointer, nranks or shape)";
    case VRC_ERR_UNSUPPORTED: return "VRC_ERR_UNSUPPORTED: unknown dtype, op or mode";
    case VRC_ERR_ALIAS: return "VRC_ERR_ALIAS: buffers overlap in a way the call does not allow";
    case VRC_ERR_HIP: return "VRC_ERR_HIP: a HIP runtime call or kernel launch failed";
    }
    return "unknown vrc status";
}

int vrc_last_hip_error(void) { return g_last_hip_error; }

int vrc_version(void) { return VRC_VERSION; }

}  // extern "C"
