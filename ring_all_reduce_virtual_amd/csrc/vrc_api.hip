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
#include <cstdlib>
#include <type_traits>

#include "vrc.h"
#include "vrc_kernels.hpp"

namespace {

using vrc::kBlock;
using vrc::kMaxRanks;
using vrc::RowSplit;

thread_local int g_last_hip_error = 0;

// When set (by vrc_plan on this thread), launches are recorded here instead
// of being enqueued.
struct Plan {
    vrc_op_desc* ops;
    int cap;
    int n;
    int launches;
};
thread_local Plan* g_plan = nullptr;

void plan_op(const vrc_op_desc& op)
{
    if (g_plan->n < g_plan->cap) g_plan->ops[g_plan->n] = op;
    g_plan->n++;
}

// A single-launch kernel: one entry with its kind, size and launch geometry.
vrc_status_t plan_single(vrc_op_kind_t kind, uint64_t count, dim3 grid, int block, int vectors)
{
    vrc_op_desc op = {};
    op.launch = g_plan->launches++;
    op.kind = kind;
    op.rows = 1;
    op.width = count;
    op.grid_x = grid.x;
    op.grid_y = grid.y;
    op.block = (unsigned)block;
    op.vectors = (unsigned)vectors;
    plan_op(op);
    return VRC_OK;
}

// ----------------------------------------------------------------------------
// Device facts and launch tuning
// ----------------------------------------------------------------------------
constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

int env_int(const char* name, int dflt, int lo, int hi)
{
    const char* s = std::getenv(name);
    if (!s || !*s) return dflt;
    char* end = nullptr;
    long v = std::strtol(s, &end, 10);
    if (end == s || v < lo || v > hi) return dflt;
    return (int)v;
}

// Launch shape, from measurements on MI355X (HIP events):
//  - fused all-reduce: one-wave workgroups sized to the rank count
//    (fused_ar_shape); single-launch ring all-reduce: one-wave workgroups
//    (chain_ar_shape);
//  - fused and ring-order reduce-scatter: over flat chunks from 64 MiB moved,
//    one-wave workgroups (fused_rs_flat_blocks_per_cu); otherwise 256-lane
//    workgroups, one per CU (two at 2 ranks) once the whole operation moves
//    >= 4 GiB, 2 per CU from 1 GiB, 8 per CU below that, where the Infinity
//    Cache holds much of the data and latency hiding matters more than open
//    DRAM rows; fused all-gather: 16 per CU (ag_blocks_per_cu);
//  - ring and halving-doubling steps: by the bytes a step moves and its number
//    of per-rank operations (step_shape), workgroups counted over all of them.
// Loads and stores carry the non-temporal hint (measured faster for this
// never-reused stream), except small relay copies (step_nontemporal) and the
// partials the single-launch ring reads back.  The environment variables
// override the policy, for measurement.
struct Tuning {
    int fused_blocks_per_cu;  // 0: size policy
    int step_blocks_per_cu;   // 0: size policy
    int chain_blocks_per_cu;  // 0: size policy
    int unroll;               // 0: size policy; else vectors per rank per lane per fused all-reduce iteration
    int step_nt;              // -1: size policy; 1: non-temporal steps; 0: regular loads/stores;
                              // 2: non-temporal adds and regular copies
    int step_unroll;          // 0: size policy; else vectors per lane per step iteration (1 or 2)
    int fused_block;          // 0: size policy; else lanes per fused all-reduce workgroup (64 or 256)
    int chain_block;          // 0: policy; else lanes per single-launch ring all-reduce workgroup (64 or 256)
    int step_block;           // 0: size policy; else lanes per step workgroup (64, with one vector per lane, or 256)
};

const Tuning& tuning()
{
    static const Tuning t = {env_int("VRC_FUSED_BLOCKS_PER_CU", 0, 1, 64),
                             env_int("VRC_STEP_BLOCKS_PER_CU", 0, 1, 64),
                             env_int("VRC_CHAIN_BLOCKS_PER_CU", 0, 1, 64), env_int("VRC_UNROLL", 0, 1, 2),
                             env_int("VRC_STEP_NT", -1, 0, 2), env_int("VRC_STEP_UNROLL", 0, 1, 2),
                             env_int("VRC_FUSED_BLOCK", 0, 64, 256), env_int("VRC_CHAIN_BLOCK", 0, 64, 256),
                             env_int("VRC_STEP_BLOCK", 0, 64, 256)};
    return t;
}

constexpr uint64_t kMiB = 1ull << 20;
constexpr uint64_t kGiB = 1ull << 30;

// Two ranks keep only a quarter of the eight-rank loads in flight per lane,
// so at 2 ranks the large-size grid doubles (8 GiB moved: 1.64-1.70 ms
// against 1.78-1.80 ms at one workgroup per CU; 4 and 16 ranks are best at one).
int fused_blocks_per_cu(uint64_t bytes_moved, int n)
{
    if (tuning().fused_blocks_per_cu) return tuning().fused_blocks_per_cu;
    if (bytes_moved >= 4 * kGiB) return n <= 2 ? 2 : 1;
    if (bytes_moved >= kGiB) return 2;
    return 8;
}

// Launch shape of the fused all-reduce (rank-order and butterfly folds):
// lanes per workgroup, workgroups per CU and vectors per rank that a lane
// keeps in flight.
//
// From 64 MiB moved the kernel runs one-wave workgroups.  Workgroups are
// handed to the 8 XCDs in turn, so consecutive 1 KiB tiles of every buffer
// are served by different XCDs; with 256-lane workgroups each XCD owned 4 KiB
// runs.  The grid keeps about 32 KiB of loads in flight per CU (workgroups per
// CU x ranks x vectors per rank <= 32, at most 8 workgroups): more
// outstanding requests made the mixed read/write stream slower, not faster.
// Two vectors per rank at 3 and 4 ranks, one otherwise.  Measured on MI355X,
// all shapes compared in one process on the same buffers (GB/s, old shape:
// 256 lanes, two vectors, 1-2 per CU at these sizes -> this policy):
//   8 x 512 MiB bf16 5,454 -> 5,648;  8 x 64 MiB 5,460 -> 5,902;
//   16 x 256 MiB 5,025 -> 5,522;      4 x 128 MiB 5,428 -> 5,978;
//   2 x 2 GiB 5,180 -> 5,576;         8 x 16 MiB (cache flushed) 4,505 -> 5,314.
// Below 64 MiB moved a call is launch-bound and keeps 256-lane workgroups,
// 8 per CU, two vectors per rank.
struct FusedShape {
    int block;
    int blocks_per_cu;
    int unroll;
};

FusedShape fused_ar_shape(uint64_t bytes_moved, int n)
{
    FusedShape s = {kBlock, 8, 2};
    if (bytes_moved >= 64 * kMiB) {
        s.block = 64;
        s.unroll = (n == 3 || n == 4) ? 2 : 1;
        s.blocks_per_cu = 8;
        while (s.blocks_per_cu > 1 && s.blocks_per_cu * n * s.unroll > 32) s.blocks_per_cu /= 2;
    }
    if (tuning().fused_blocks_per_cu) s.blocks_per_cu = tuning().fused_blocks_per_cu;
    if (tuning().fused_block) s.block = tuning().fused_block == 64 ? 64 : kBlock;
    if (tuning().unroll) s.unroll = tuning().unroll;
    return s;
}

// Launch shape of a ring or halving-doubling step of `nops` per-rank
// operations moving `bytes_moved` in all.  Launch-bound steps (< 64 MiB) use
// one vector per lane at 8 workgroups per CU.  Larger steps of up to 7
// operations that each move >= 48 MiB use one vector at 4 per CU.  Other
// steps keep two vectors per lane in flight (four loads for an add): at 8 per
// CU when there are fewer than 12 operations and each moves >= 128 MiB, else
// at 16 per CU.
// Measured on MI355X, bf16 all-reduce, ms per call for (vectors per lane,
// workgroups per CU) on one box; ring unless marked hd:
//   2 ranks x 2 GiB:     (1, 4) 2.012; (2, 8) 2.310; (2, 16) 2.237
//   4 ranks x 1 GiB:     (1, 4) 2.886 (hd 2.930); (2, 8) 3.031 (hd 3.211)
//   5 ranks x 819 MiB:   (1, 4) 3.376; (2, 8) 3.649; (2, 16) 3.769
//   6 ranks x 682 MiB:   (1, 4) 3.542; (2, 8) 3.763
//   7 ranks x 73 MiB:    (2, 16) 0.423; (1, 4) 0.438 (31 MiB per reduce operation)
//   8 ranks x 512 MiB:   (2, 8) 3.310 (hd 3.385); (1, 4) 3.271 (hd 3.480); (2, 16) 3.302 (hd 3.483)
//   8 ranks x 64 MiB:    (2, 16) 0.384; (2, 8) 0.403; (1, 4) 0.409
//   12 ranks x 341 MiB:  (2, 16) 3.876; (1, 4) 3.848; (2, 8) 3.985
//   16 ranks x 256 MiB:  (2, 16) 3.423 (hd 3.578); (2, 8) 3.584 (hd 3.705); (1, 4) 3.958
//   8 ranks x 16 MiB:    (1, 8) 0.115; (2, 16) 0.122 (48 MiB steps)
// Adds of up to 7 operations of >= 48 MiB whose operations all vectorize
// run one-wave workgroups, 8 per CU, one vector per lane.  One process, same
// buffers, one reduce-scatter add step (GB/s; 256 lanes at 4 per CU -> one
// wave at 8 per CU): 2 x 2 GiB 5,473 -> 5,804; 4 x 1 GiB 5,456 -> 5,779.
// The copy steps lost with one wave (2 x 2 GiB 5,477 -> 5,051; 4 x 1 GiB
// 5,740 -> 4,431) and keep 256 lanes; at 8 and 16 ranks neither kind gained
// reliably.  A step with a scalar operation (operands on different 16-byte
// offsets) keeps 256 lanes: its scalar elements need the lanes in flight
// (5 x 819 MiB ring reduce-scatter: 3.05 ms with 256 lanes, 7.97 ms with one
// wave).
struct StepShape {
    int blocks_per_cu;
    int unroll;
    int block;  // lanes per workgroup; 64 implies unroll 1
};

StepShape step_shape(uint64_t bytes_moved, int nops, bool vector_add)
{
    StepShape s = {8, 1, kBlock};
    const uint64_t per_op = bytes_moved / (uint64_t)(nops > 0 ? nops : 1);
    if (bytes_moved >= kGiB / 16) {
        if (nops <= 7 && per_op >= 48 * kMiB) s = vector_add ? StepShape{8, 1, 64} : StepShape{4, 1, kBlock};
        else if (nops < 12 && per_op >= kGiB / 8) s = {8, 2, kBlock};
        else s = {16, 2, kBlock};
    }
    if (tuning().step_blocks_per_cu) s.blocks_per_cu = tuning().step_blocks_per_cu;
    if (tuning().step_unroll) s.unroll = tuning().step_unroll;
    if (tuning().step_block) s.block = tuning().step_block == 64 ? 64 : kBlock;
    if (s.block == 64) s.unroll = 1;
    return s;
}

// Cache hint of a ring or halving-doubling step.  Adds stream with the
// non-temporal hint.  A copy step relays data that the next step reads back,
// so copies that write at most 64 MiB (well inside the 256 MB Infinity
// Cache) use regular loads and stores, and larger ones stream.  Measured on
// MI355X: regular copies cut the 8 x 16 MiB ring all-reduce by 4 % and the
// 8 x 5 MiB ring all-gather (40 MiB per step) by 9 %, and cost 2 % at
// 8 x 512 MiB.
bool step_nontemporal(bool add, uint64_t bytes_moved)
{
    switch (tuning().step_nt) {
    case 0: return false;
    case 1: return true;
    case 2: return add;
    }
    return add || bytes_moved / 2 > 64 * kMiB;
}

// The fused reduce-scatter over flat chunks, from 64 MiB moved: one-wave
// workgroups walking all chunks in address order, 8 per CU up to 4 ranks and
// 4 above.  Measured on MI355X in one process on the same buffers (GB/s of
// (N+1)·S; one grid row per chunk with 256-lane workgroups, as below 64 MiB
// -> this shape, rank-order fold): 8 x 512 MiB 5,402 -> 5,885;
// 8 x 128 MiB 5,109 -> 6,156; 16 x 256 MiB 5,350 -> 5,615; 4 x 1 GiB
// 5,457 -> 5,916.  The butterfly fold of the halving-doubling reduce-scatter
// does N-1 rounded adds per element over fewer bytes per fold than an
// all-reduce, and turns ALU-bound with too few waves: at 16 ranks it took
// 1,480 us at 2 per CU against 847-853 us at 4 (the rank fold: 863-871 us
// at either), so 4 per CU is the floor from 5 ranks up.
int fused_rs_flat_blocks_per_cu(int n)
{
    if (tuning().fused_blocks_per_cu) return tuning().fused_blocks_per_cu;
    return n <= 4 ? 8 : 4;
}

// The memory-faithful reduce-scatter chain over flat chunks (one-wave
// workgroups): its lanes wait on their own stores at every step, so like the
// all-reduce chain it keeps more waves resident.
int chain_rs_flat_blocks_per_cu()
{
    if (tuning().chain_blocks_per_cu) return tuning().chain_blocks_per_cu;
    return 16;
}

// The fused all-gather reads each input once and stores it N times: 16
// workgroups per CU at every size.  Measured on MI355X in one process on the
// same buffers (us, 8 / 16 per CU): 8 x 5 MiB fp16 heads 77.2 / 75.2 and
// 81.4 / 77.0 (cache flushed); 8 x 64 MiB 953 / 943; 16 x 5 MiB 292 / 289;
// 4 x 5 MiB 24.6 / 24.8.  One-wave workgroups were slower (79-89 us on the
// heads).
int ag_blocks_per_cu()
{
    if (tuning().fused_blocks_per_cu) return tuning().fused_blocks_per_cu;
    return 16;
}

// Memory-faithful chains wait on their own stores between steps, so they
// need more resident waves than the fused loop to hide latency.  This shape
// serves the single-launch reduce-scatter and all-gather relays (256-lane
// workgroups).
int chain_blocks_per_cu(uint64_t bytes_moved)
{
    if (tuning().chain_blocks_per_cu) return tuning().chain_blocks_per_cu;
    return bytes_moved >= 4 * kGiB ? 4 : 8;
}

// Launch shape of the single-launch ring all-reduce.  Like the fused kernel
// it runs one-wave workgroups, so consecutive wave tiles go to different
// XCDs.  The ring-order kernel (partials in registers, N loads in flight per
// lane) uses 4 per CU (8 at 2 ranks); the memory-faithful chain, whose lanes
// wait on their own stores at every step, uses 16.  Measured on MI355X in one
// process on the same buffers (GB/s of 2·N·S; 256-lane shape -> this one):
//   ring order:  8 x 512 MiB 5,498 -> 5,565; 8 x 128 MiB 5,304 -> 5,663;
//                8 x 16 MiB (cache flushed) 5,077 -> 5,187; 16 x 256 MiB 5,262 -> 5,259;
//                2 x 2 GiB 5,485 -> 5,493; 4 x 1 GiB 5,420 -> 5,297;
//   chained:     8 x 512 MiB 4,521 -> 4,835; 8 x 16 MiB 3,779 -> 4,012;
//                4 x 1 GiB 4,790 -> 4,846; 2 x 2 GiB 4,857 -> 4,999.
struct ChainShape {
    int block;
    int blocks_per_cu;
};

ChainShape chain_ar_shape(bool mem, int n)
{
    ChainShape s = {64, mem ? 16 : (n <= 2 ? 8 : 4)};
    if (mem && tuning().chain_blocks_per_cu) s.blocks_per_cu = tuning().chain_blocks_per_cu;
    if (!mem && tuning().fused_blocks_per_cu) s.blocks_per_cu = tuning().fused_blocks_per_cu;
    if (tuning().chain_block) s.block = tuning().chain_block == 256 ? kBlock : 64;
    return s;
}

#define VRC_FOR_N(X) X(2) X(3) X(4) X(5) X(6) X(7) X(8) X(9) X(10) X(11) X(12) X(13) X(14) X(15) X(16)

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

// Grid x for `ops` operations of at most `work` lane-items each, capped at
// blocks_per_cu workgroups per CU over the whole grid.
unsigned grid_x(int cus, uint64_t work, int ops, int blocks_per_cu, int block = kBlock)
{
    const uint64_t want = (work + block - 1) / block;
    uint64_t cap = (uint64_t)cus * (uint64_t)blocks_per_cu / (uint64_t)(ops > 0 ? ops : 1);
    if (cap < 1) cap = 1;
    uint64_t g = want < cap ? want : cap;
    if (g < 1) g = 1;
    if (g > 0x7fffffffull) g = 0x7fffffffull;
    return (unsigned)g;
}

vrc_status_t check_launch()
{
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        g_last_hip_error = (int)e;
        return VRC_ERR_HIP;
    }
    return VRC_OK;
}

vrc_status_t hip_fail(hipError_t e)
{
    g_last_hip_error = (int)e;
    return VRC_ERR_HIP;
}

// ----------------------------------------------------------------------------
// Element sizes, chunking, alignment split
// ----------------------------------------------------------------------------
int esize(vrc_dtype_t dt)
{
    switch (dt) {
    case VRC_INT32: return 4;
    case VRC_FP32: return 4;
    case VRC_FP16: return 2;
    case VRC_BF16: return 2;
    }
    return 0;
}

int mod(int a, int n) { return ((a % n) + n) % n; }

// Flat chunk c of `count` elements over n ranks: equal chunks of count/n,
// the last one takes the remainder.
void chunk_range(uint64_t count, int n, int c, uint64_t* off, uint64_t* len)
{
    const uint64_t base = count / (uint64_t)n;
    *off = (uint64_t)c * base;
    *len = (c == n - 1) ? count - base * (uint64_t)(n - 1) : base;
}

// Split rows of `width` elements whose operands start at `addr[0..np)` into
// a scalar head, 16-byte vectors and a scalar tail.  Vectors are only used
// when every operand has the same address offset modulo 16 and (for more
// than one row) every row stride is a multiple of 16 bytes.
RowSplit split_rows(const uintptr_t* addr, int np, uint64_t rows, const uint64_t* stride_bytes, int ns,
                    uint64_t width, int esz)
{
    RowSplit g = {width, 0, 0};
    const uintptr_t res = addr[0] & 15u;
    if (res % (uintptr_t)esz) return g;
    for (int i = 1; i < np; i++)
        if ((addr[i] & 15u) != res) return g;
    if (rows > 1)
        for (int i = 0; i < ns; i++)
            if (stride_bytes[i] & 15u) return g;
    uint64_t head = ((16u - res) & 15u) / (uint64_t)esz;
    if (head > width) head = width;
    const uint64_t vec = 16u / (uint64_t)esz;
    g.head = head;
    g.nvb = (width - head) / vec;
    g.tail = width - head - g.nvb * vec;
    return g;
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

vrc_status_t check_common(const void* const* send, void* const* recv, int n, uint64_t count, vrc_dtype_t dtype)
{
    if (!send || !recv) return VRC_ERR_INVALID_ARG;
    if (n < 1 || n > kMaxRanks) return VRC_ERR_INVALID_ARG;
    if (count > kMaxCount) return VRC_ERR_INVALID_ARG;
    if (esize(dtype) == 0) return VRC_ERR_UNSUPPORTED;
    return VRC_OK;
}

// ----------------------------------------------------------------------------
// Typed launchers
// ----------------------------------------------------------------------------
template <class T>
struct Launch {
    static constexpr int E = T::ESZ;

    // Bytes one step moves: per operation, width*rows elements read from each
    // operand and written once.
    template <bool ADD>
    static uint64_t step_bytes(const vrc::StepArgs& args, int nops)
    {
        uint64_t b = 0;
        for (int i = 0; i < nops; i++) b += args.op[i].rows * args.op[i].width * (uint64_t)E * (ADD ? 3 : 2);
        return b;
    }

    template <bool ADD>
    static vrc_status_t step(const vrc::StepArgs& args, int nops, uint64_t work, int cus, hipStream_t st)
    {
        const uint64_t bytes = step_bytes<ADD>(args, nops);
        bool vector = true;  // every operation's body runs 16-byte vectors
        for (int i = 0; i < nops; i++)
            if (args.op[i].g.head + args.op[i].g.tail >= 2 * (uint64_t)(16 / E)) vector = false;
        const StepShape shape = step_shape(bytes, nops, ADD && vector);
        const dim3 grid(grid_x(cus, work, nops, shape.blocks_per_cu, shape.block), (unsigned)nops);
        if (g_plan) {
            for (int i = 0; i < nops; i++) {
                const vrc::StepOp& o = args.op[i];
                vrc_op_desc op = {};
                op.launch = g_plan->launches;
                op.kind = ADD ? VRC_OP_ADD : VRC_OP_COPY;
                op.a = o.a;
                op.b = ADD ? o.b : nullptr;
                op.d = o.d;
                op.rows = o.rows;
                op.width = o.width;
                op.stride_a = o.sa;
                op.stride_b = ADD ? o.sb : 0;
                op.stride_d = o.sd;
                op.grid_x = grid.x;
                op.grid_y = grid.y;
                op.block = (unsigned)shape.block;
                op.vectors = (unsigned)shape.unroll;
                plan_op(op);
            }
            g_plan->launches++;
            return VRC_OK;
        }
        const bool nt = step_nontemporal(ADD, bytes);
        const bool u2 = shape.unroll == 2, wave = shape.block == 64;
        if (nops <= 4) launch_step<ADD, 4>(args, nops, nt, u2, wave, grid, st);
        else if (nops <= 8) launch_step<ADD, 8>(args, nops, nt, u2, wave, grid, st);
        else if (nops <= 16) launch_step<ADD, 16>(args, nops, nt, u2, wave, grid, st);
        else launch_step<ADD, vrc::kMaxStepOps>(args, nops, nt, u2, wave, grid, st);
        return check_launch();
    }

    // Launch a step with an argument block of K operation slots (the first
    // nops filled; blockIdx.y < nops never reads the others).  `wave`: one-wave
    // workgroups, one vector per lane.
    template <bool ADD, int K>
    static void launch_step(const vrc::StepArgs& args, int nops, bool nt, bool u2, bool wave, dim3 grid,
                            hipStream_t st)
    {
        vrc::StepArgsK<K> a = {};
        for (int i = 0; i < nops && i < K; i++) a.op[i] = args.op[i];
        if (wave) {
            if (nt) hipLaunchKernelGGL((vrc::k_ring_step<T, ADD, true, K, 1, 64>), grid, dim3(64), 0, st, a);
            else hipLaunchKernelGGL((vrc::k_ring_step<T, ADD, false, K, 1, 64>), grid, dim3(64), 0, st, a);
        } else if (u2) {
            if (nt) hipLaunchKernelGGL((vrc::k_ring_step<T, ADD, true, K, 2>), grid, dim3(kBlock), 0, st, a);
            else hipLaunchKernelGGL((vrc::k_ring_step<T, ADD, false, K, 2>), grid, dim3(kBlock), 0, st, a);
        } else {
            if (nt) hipLaunchKernelGGL((vrc::k_ring_step<T, ADD, true, K>), grid, dim3(kBlock), 0, st, a);
            else hipLaunchKernelGGL((vrc::k_ring_step<T, ADD, false, K>), grid, dim3(kBlock), 0, st, a);
        }
    }

    // Work items of one operation: vectors plus scalar slots.
    static uint64_t op_work(const vrc::StepOp& op) { return op.rows * (op.g.nvb + op.g.head + op.g.tail); }

    static vrc::StepOp make_op(const char* a, const char* b, char* d, uint64_t rows, uint64_t width,
                               uint64_t sa, uint64_t sb, uint64_t sd)
    {
        vrc::StepOp op;
        op.a = a;
        op.b = b ? b : a;
        op.d = d;
        op.rows = rows;
        op.width = width;
        op.sa = sa;
        op.sb = b ? sb : sa;
        op.sd = sd;
        const uintptr_t addr[3] = {(uintptr_t)a, (uintptr_t)op.b, (uintptr_t)d};
        const uint64_t strides[3] = {sa * E, op.sb * E, sd * E};
        op.g = split_rows(addr, 3, rows, strides, 3, width, E);
        return op;
    }

    static vrc_status_t copy(const char* a, char* d, uint64_t rows, uint64_t width, uint64_t sa, uint64_t sd,
                             int cus, hipStream_t st)
    {
        vrc::StepArgs args;
        args.op[0] = make_op(a, nullptr, d, rows, width, sa, 0, sd);
        return step<false>(args, 1, op_work(args.op[0]), cus, st);
    }

    // Ring all-reduce: N-1 reduce-scatter launches, then N-1 all-gather launches.
    static vrc_status_t ring_allreduce(const char* const* x, char* const* y, int n, uint64_t count, int cus,
                                       hipStream_t st)
    {
        if (n == 1) return x[0] == y[0] ? VRC_OK : copy(x[0], y[0], 1, count, 0, 0, cus, st);
        vrc::StepArgs args;
        for (int s = 0; s < n - 1; s++) {
            uint64_t work = 0;
            for (int r = 0; r < n; r++) {
                const int c = mod(r - 1 - s, n);
                const int p = mod(r - 1, n);
                uint64_t off, len;
                chunk_range(count, n, c, &off, &len);
                const char* partial = (s == 0 ? x[p] : y[p]) + off * E;
                args.op[r] = make_op(partial, x[r] + off * E, y[r] + off * E, 1, len, 0, 0, 0);
                const uint64_t w = op_work(args.op[r]);
                if (w > work) work = w;
            }
            vrc_status_t rc = step<true>(args, n, work, cus, st);
            if (rc) return rc;
        }
        for (int s = 0; s < n - 1; s++) {
            uint64_t work = 0;
            for (int r = 0; r < n; r++) {
                const int c = mod(r - s, n);
                uint64_t off, len;
                chunk_range(count, n, c, &off, &len);
                args.op[r] = make_op(y[mod(r - 1, n)] + off * E, nullptr, y[r] + off * E, 1, len, 0, 0, 0);
                const uint64_t w = op_work(args.op[r]);
                if (w > work) work = w;
            }
            vrc_status_t rc = step<false>(args, n, work, cus, st);
            if (rc) return rc;
        }
        return VRC_OK;
    }

    // Chunk c of an input viewed as [outer, row]: element offset of its
    // (0,0), rows, width and the input row stride.
    struct Chunk {
        uint64_t off, rows, width, stride;
    };
    static Chunk rs_chunk(uint64_t count, uint64_t outer, int n, int c)
    {
        Chunk k;
        if (outer == 1) {
            chunk_range(count, n, c, &k.off, &k.width);
            k.rows = 1;
            k.stride = 0;
        } else {
            const uint64_t row = count / outer, w = row / (uint64_t)n;
            k.off = (uint64_t)c * w;
            k.rows = outer;
            k.width = w;
            k.stride = row;
        }
        return k;
    }

    // Ring reduce-scatter: step s adds rank (c+1+s)'s chunk c into the
    // running partial of chunk c, which lives in output c.
    static vrc_status_t ring_reduce_scatter(const char* const* x, char* const* y, int n, uint64_t count,
                                            uint64_t outer, int cus, hipStream_t st)
    {
        if (n == 1) return copy(x[0], y[0], 1, count, 0, 0, cus, st);
        vrc::StepArgs args;
        for (int s = 0; s < n - 1; s++) {
            uint64_t work = 0;
            for (int c = 0; c < n; c++) {
                const Chunk k = rs_chunk(count, outer, n, c);
                const int r = mod(c + 1 + s, n);
                const char* partial = (s == 0) ? x[c] + k.off * E : y[c];
                const uint64_t sp = (s == 0) ? k.stride : k.width;
                args.op[c] = make_op(partial, x[r] + k.off * E, y[c], k.rows, k.width, sp, k.stride, k.width);
                const uint64_t w = op_work(args.op[c]);
                if (w > work) work = w;
            }
            vrc_status_t rc = step<true>(args, n, work, cus, st);
            if (rc) return rc;
        }
        return VRC_OK;
    }

    // Ring all-gather: step 0 places every rank's own slab and the slab of
    // its predecessor; step s >= 1 relays slab (r-1-s) from rank r-1.
    static vrc_status_t ring_all_gather(const char* const* x, char* const* y, int n, uint64_t count,
                                        uint64_t outer, int cus, hipStream_t st)
    {
        const uint64_t row = count / outer, sy = (uint64_t)n * row;
        if (n == 1) return copy(x[0], y[0], 1, count, 0, 0, cus, st);
        vrc::StepArgs args;
        uint64_t work = 0;
        for (int r = 0; r < n; r++) {
            const int p = mod(r - 1, n);
            args.op[2 * r] = make_op(x[r], nullptr, y[r] + (uint64_t)r * row * E, outer, row, row, 0, sy);
            args.op[2 * r + 1] = make_op(x[p], nullptr, y[r] + (uint64_t)p * row * E, outer, row, row, 0, sy);
            const uint64_t w = op_work(args.op[2 * r]) > op_work(args.op[2 * r + 1]) ? op_work(args.op[2 * r])
                                                                                      : op_work(args.op[2 * r + 1]);
            if (w > work) work = w;
        }
        vrc_status_t rc = step<false>(args, 2 * n, work, cus, st);
        if (rc) return rc;
        for (int s = 1; s < n - 1; s++) {
            work = 0;
            for (int r = 0; r < n; r++) {
                const int slab = mod(r - 1 - s, n);
                const uint64_t off = (uint64_t)slab * row * E;
                args.op[r] = make_op(y[mod(r - 1, n)] + off, nullptr, y[r] + off, outer, row, sy, 0, sy);
                const uint64_t w = op_work(args.op[r]);
                if (w > work) work = w;
            }
            rc = step<false>(args, n, work, cus, st);
            if (rc) return rc;
        }
        return VRC_OK;
    }

    // ---- fused family ----------------------------------------------------
    template <int N, class Fold>
    static void launch_fused_ar_n(const vrc::FusedArArgs& a, dim3 grid, FusedShape sh, hipStream_t st)
    {
        if (sh.block == 64) {
            if (sh.unroll == 2)
                hipLaunchKernelGGL((vrc::k_fused_allreduce<T, N, 2, true, Fold, 64>), grid, dim3(64), 0, st, a);
            else
                hipLaunchKernelGGL((vrc::k_fused_allreduce<T, N, 1, true, Fold, 64>), grid, dim3(64), 0, st, a);
        } else {
            if (sh.unroll == 2)
                hipLaunchKernelGGL((vrc::k_fused_allreduce<T, N, 2, true, Fold>), grid, dim3(kBlock), 0, st, a);
            else
                hipLaunchKernelGGL((vrc::k_fused_allreduce<T, N, 1, true, Fold>), grid, dim3(kBlock), 0, st, a);
        }
    }

    template <class Fold = vrc::RankFold>
    static vrc_status_t fused_allreduce(const char* const* x, char* const* y, int n, uint64_t count, int cus,
                                        hipStream_t st)
    {
        if (n == 1) return x[0] == y[0] ? VRC_OK : copy(x[0], y[0], 1, count, 0, 0, cus, st);
        vrc::FusedArArgs a;
        uintptr_t addr[2 * kMaxRanks];
        for (int r = 0; r < n; r++) {
            a.src[r] = x[r];
            a.dst[r] = y[r];
            addr[2 * r] = (uintptr_t)x[r];
            addr[2 * r + 1] = (uintptr_t)y[r];
        }
        for (int r = n; r < kMaxRanks; r++) {
            a.src[r] = nullptr;
            a.dst[r] = nullptr;
        }
        a.count = count;
        a.g = split_rows(addr, 2 * n, 1, nullptr, 0, count, E);
        const uint64_t work = a.g.nvb > a.g.head + a.g.tail ? a.g.nvb : a.g.head + a.g.tail;
        const FusedShape sh = fused_ar_shape(2 * (uint64_t)n * count * E, n);
        const dim3 grid(grid_x(cus, work, 1, sh.blocks_per_cu, sh.block));
        if (g_plan)
            return plan_single(std::is_same<Fold, vrc::Butterfly>::value ? VRC_OP_BUTTERFLY_ALLREDUCE
                                                                          : VRC_OP_FUSED_ALLREDUCE,
                               count, grid, sh.block, sh.unroll);
        if constexpr (std::is_same<Fold, vrc::Butterfly>::value) {
            switch (n) {
            case 2: launch_fused_ar_n<2, Fold>(a, grid, sh, st); break;
            case 4: launch_fused_ar_n<4, Fold>(a, grid, sh, st); break;
            case 8: launch_fused_ar_n<8, Fold>(a, grid, sh, st); break;
            case 16: launch_fused_ar_n<16, Fold>(a, grid, sh, st); break;
            default: return VRC_ERR_INVALID_ARG;
            }
        } else {
            switch (n) {
#define VRC_CASE(K) \
    case K: launch_fused_ar_n<K, Fold>(a, grid, sh, st); break;
                VRC_FOR_N(VRC_CASE)
#undef VRC_CASE
            default: return VRC_ERR_INVALID_ARG;
            }
        }
        return check_launch();
    }

    template <int N, class Fold>
    static void launch_fused_rs_n(const vrc::FusedRsArgs& a, dim3 grid, hipStream_t st)
    {
        hipLaunchKernelGGL((vrc::k_fused_reduce_scatter<T, N, true, Fold>), grid, dim3(kBlock), 0, st, a);
    }

    template <int N, class Fold>
    static void launch_fused_rs_flat_n(const vrc::ChainArgs& a, dim3 grid, hipStream_t st)
    {
        hipLaunchKernelGGL((vrc::k_fused_reduce_scatter_flat<T, N, true, Fold>), grid, dim3(64), 0, st, a);
    }

    // Flat chunks (outer == 1) from 64 MiB moved: one-wave tiles over all
    // chunks in address order (fused_rs_flat_blocks_per_cu), for the fused
    // and ring-order reduce-scatters.  The flat kernels' scalar pass runs one
    // wave per chunk, so they are used only when every chunk's operands share
    // their offset modulo 16 bytes (at most a head and a tail run scalar);
    // otherwise the caller takes the per-chunk grid, which spreads scalar
    // elements over all lanes.  Fills the chunk table and grid and returns
    // false in that case.
    static bool rs_flat_layout(const char* const* x, char* const* y, int n, uint64_t count, int cus,
                               vrc::ChainArgs* pa, dim3* grid)
    {
        vrc::ChainArgs& a = *pa;
        a = {};
        for (int r = 0; r < kMaxRanks; r++) {
            a.src[r] = r < n ? x[r] : nullptr;
            a.dst[r] = r < n ? y[r] : nullptr;
        }
        a.tile0[0] = 0;
        for (int c = 0; c < n; c++) {
            uint64_t off, len;
            chunk_range(count, n, c, &off, &len);
            uintptr_t addr[kMaxRanks + 1];
            for (int r = 0; r < n; r++) addr[r] = (uintptr_t)(x[r] + off * E);
            addr[n] = (uintptr_t)y[c];
            a.ch[c] = {off, 1, len, 0, split_rows(addr, n + 1, 1, nullptr, 0, len, E)};
            if (a.ch[c].g.head + a.ch[c].g.tail >= 2 * (uint64_t)T::VEC) return false;
            a.tile0[c + 1] = a.tile0[c] + (a.ch[c].g.nvb + 63) / 64;
        }
        // At least one wave per chunk for the scalar head/tail pass.
        const uint64_t lanes = a.tile0[n] * 64, scalar_lanes = (uint64_t)n * 64;
        const uint64_t work = lanes > scalar_lanes ? lanes : scalar_lanes;
        *grid = dim3(grid_x(cus, work, 1, fused_rs_flat_blocks_per_cu(n), 64));
        return true;
    }

    template <class Fold>
    static bool fused_reduce_scatter_flat(const char* const* x, char* const* y, int n, uint64_t count, int cus,
                                          hipStream_t st, vrc_status_t* rc)
    {
        vrc::ChainArgs a;
        dim3 grid;
        if (!rs_flat_layout(x, y, n, count, cus, &a, &grid)) return false;
        if (g_plan) {
            *rc = plan_single(std::is_same<Fold, vrc::Butterfly>::value ? VRC_OP_BUTTERFLY_REDUCE_SCATTER
                                                                         : VRC_OP_FUSED_REDUCE_SCATTER,
                              count, grid, 64, 1);
            return true;
        }
        *rc = VRC_OK;
        if constexpr (std::is_same<Fold, vrc::Butterfly>::value) {
            switch (n) {
            case 2: launch_fused_rs_flat_n<2, Fold>(a, grid, st); break;
            case 4: launch_fused_rs_flat_n<4, Fold>(a, grid, st); break;
            case 8: launch_fused_rs_flat_n<8, Fold>(a, grid, st); break;
            case 16: launch_fused_rs_flat_n<16, Fold>(a, grid, st); break;
            default: *rc = VRC_ERR_INVALID_ARG; return true;
            }
        } else {
            switch (n) {
#define VRC_CASE(K) \
    case K: launch_fused_rs_flat_n<K, Fold>(a, grid, st); break;
                VRC_FOR_N(VRC_CASE)
#undef VRC_CASE
            default: *rc = VRC_ERR_INVALID_ARG; return true;
            }
        }
        *rc = check_launch();
        return true;
    }

    template <class Fold = vrc::RankFold>
    static vrc_status_t fused_reduce_scatter(const char* const* x, char* const* y, int n, uint64_t count,
                                             uint64_t outer, int cus, hipStream_t st)
    {
        if (n == 1) return copy(x[0], y[0], 1, count, 0, 0, cus, st);
        vrc_status_t rc = VRC_OK;
        if (outer == 1 && (uint64_t)(n + 1) * count * E >= 64 * kMiB &&
            fused_reduce_scatter_flat<Fold>(x, y, n, count, cus, st, &rc))
            return rc;
        vrc::FusedRsArgs a;
        uint64_t work = 0;
        for (int r = 0; r < kMaxRanks; r++) a.src[r] = r < n ? x[r] : nullptr;
        for (int c = 0; c < n; c++) {
            const Chunk k = rs_chunk(count, outer, n, c);
            vrc::RsChunk& ch = a.ch[c];
            ch.src_off = k.off;
            ch.d = y[c];
            ch.rows = k.rows;
            ch.width = k.width;
            ch.s_src = k.stride;
            ch.s_dst = k.width;
            uintptr_t addr[kMaxRanks + 1];
            for (int r = 0; r < n; r++) addr[r] = (uintptr_t)(x[r] + k.off * E);
            addr[n] = (uintptr_t)y[c];
            const uint64_t strides[2] = {k.stride * E, k.width * E};
            ch.g = split_rows(addr, n + 1, k.rows, strides, 2, k.width, E);
            const uint64_t w = k.rows * (ch.g.nvb + ch.g.head + ch.g.tail);
            if (w > work) work = w;
        }
        const dim3 grid(grid_x(cus, work, n, fused_blocks_per_cu((uint64_t)(n + 1) * count * E, n)), (unsigned)n);
        if (g_plan)
            return plan_single(std::is_same<Fold, vrc::Butterfly>::value ? VRC_OP_BUTTERFLY_REDUCE_SCATTER
                                                                          : VRC_OP_FUSED_REDUCE_SCATTER,
                               count, grid, kBlock, 1);
        if constexpr (std::is_same<Fold, vrc::Butterfly>::value) {
            switch (n) {
            case 2: launch_fused_rs_n<2, Fold>(a, grid, st); break;
            case 4: launch_fused_rs_n<4, Fold>(a, grid, st); break;
            case 8: launch_fused_rs_n<8, Fold>(a, grid, st); break;
            case 16: launch_fused_rs_n<16, Fold>(a, grid, st); break;
            default: return VRC_ERR_INVALID_ARG;
            }
        } else {
            switch (n) {
#define VRC_CASE(K) \
    case K: launch_fused_rs_n<K, Fold>(a, grid, st); break;
                VRC_FOR_N(VRC_CASE)
#undef VRC_CASE
            default: return VRC_ERR_INVALID_ARG;
            }
        }
        return check_launch();
    }

    static vrc_status_t fused_all_gather(const char* const* x, char* const* y, int n, uint64_t count,
                                         uint64_t outer, int cus, hipStream_t st)
    {
        vrc::FusedAgArgs a;
        const uint64_t row = count / outer;
        a.rows = outer;
        a.width = row;
        a.n = n;
        uint64_t work = 0;
        for (int r = 0; r < kMaxRanks; r++) {
            a.src[r] = r < n ? x[r] : nullptr;
            a.dst[r] = r < n ? y[r] : nullptr;
        }
        for (int q = 0; q < n; q++) {
            uintptr_t addr[kMaxRanks + 1];
            addr[0] = (uintptr_t)x[q];
            for (int r = 0; r < n; r++) addr[r + 1] = (uintptr_t)(y[r] + (uint64_t)q * row * E);
            const uint64_t strides[2] = {row * E, (uint64_t)n * row * E};
            a.g[q] = split_rows(addr, n + 1, outer, strides, 2, row, E);
            const uint64_t w = outer * (a.g[q].nvb + a.g[q].head + a.g[q].tail);
            if (w > work) work = w;
        }
        const dim3 grid(grid_x(cus, work, n, ag_blocks_per_cu()), (unsigned)n);
        if (g_plan) return plan_single(VRC_OP_FUSED_ALL_GATHER, count, grid, kBlock, 1);
        hipLaunchKernelGGL((vrc::k_fused_all_gather<T, true>), grid, dim3(kBlock), 0, st, a);
        return check_launch();
    }

    // ---- halving-doubling, one launch per step ---------------------------
    // Block range [lo, hi) of a flat buffer as an element range.
    static void block_span(uint64_t count, int n, int lo, int hi, uint64_t* off, uint64_t* len)
    {
        const uint64_t base = count / (uint64_t)n;
        const uint64_t end = (hi == n) ? count : (uint64_t)hi * base;
        *off = (uint64_t)lo * base;
        *len = end - *off;
    }

    // Recursive halving (distances N/2 .. 1): rank r keeps the half of its
    // block range that holds block r and adds the partner's (r XOR d) copy
    // of that half.  Then recursive doubling (distances 1 .. N/2): rank r
    // copies the partner's range.  2 log2 N launches.
    static vrc_status_t hd_allreduce(const char* const* x, char* const* y, int n, uint64_t count, int cus,
                                     hipStream_t st)
    {
        if (n == 1) return x[0] == y[0] ? VRC_OK : copy(x[0], y[0], 1, count, 0, 0, cus, st);
        int lo[kMaxRanks], hi[kMaxRanks], nlo[kMaxRanks], nhi[kMaxRanks];
        for (int r = 0; r < n; r++) {
            lo[r] = 0;
            hi[r] = n;
        }
        vrc::StepArgs args;
        bool first = true;
        for (int d = n / 2; d >= 1; d /= 2) {
            uint64_t work = 0;
            for (int r = 0; r < n; r++) {
                const int p = r ^ d, mid = (lo[r] + hi[r]) / 2;
                const bool upper = (r & d) != 0;
                nlo[r] = upper ? mid : lo[r];
                nhi[r] = upper ? hi[r] : mid;
                uint64_t off, len;
                block_span(count, n, nlo[r], nhi[r], &off, &len);
                const char* own = (first ? x[r] : y[r]) + off * E;
                const char* other = (first ? x[p] : y[p]) + off * E;
                args.op[r] = make_op(own, other, y[r] + off * E, 1, len, 0, 0, 0);
                const uint64_t w = op_work(args.op[r]);
                if (w > work) work = w;
            }
            vrc_status_t rc = step<true>(args, n, work, cus, st);
            if (rc) return rc;
            for (int r = 0; r < n; r++) {
                lo[r] = nlo[r];
                hi[r] = nhi[r];
            }
            first = false;
        }
        for (int d = 1; d < n; d *= 2) {
            uint64_t work = 0;
            for (int r = 0; r < n; r++) {
                const int p = r ^ d;
                uint64_t off, len;
                block_span(count, n, lo[p], hi[p], &off, &len);
                args.op[r] = make_op(y[p] + off * E, nullptr, y[r] + off * E, 1, len, 0, 0, 0);
                const uint64_t w = op_work(args.op[r]);
                if (w > work) work = w;
            }
            vrc_status_t rc = step<false>(args, n, work, cus, st);
            if (rc) return rc;
            for (int r = 0; r < n; r++) {
                nlo[r] = lo[r] < lo[r ^ d] ? lo[r] : lo[r ^ d];
                nhi[r] = hi[r] > hi[r ^ d] ? hi[r] : hi[r ^ d];
            }
            for (int r = 0; r < n; r++) {
                lo[r] = nlo[r];
                hi[r] = nhi[r];
            }
        }
        return VRC_OK;
    }

    // Recursive-doubling all-gather over the slabs of [outer, N*row]
    // outputs.  Step 0 copies each rank's own slab and its distance-1
    // partner's slab from the inputs; step d copies the partner's slab range
    // from the partner's output.  log2 N launches.
    static vrc_status_t hd_all_gather(const char* const* x, char* const* y, int n, uint64_t count, uint64_t outer,
                                      int cus, hipStream_t st)
    {
        const uint64_t row = count / outer, sy = (uint64_t)n * row;
        if (n == 1) return copy(x[0], y[0], 1, count, 0, 0, cus, st);
        int lo[kMaxRanks], hi[kMaxRanks], nlo[kMaxRanks], nhi[kMaxRanks];
        vrc::StepArgs args;
        uint64_t work = 0;
        for (int r = 0; r < n; r++) {
            const int p = r ^ 1;
            args.op[2 * r] = make_op(x[r], nullptr, y[r] + (uint64_t)r * row * E, outer, row, row, 0, sy);
            args.op[2 * r + 1] = make_op(x[p], nullptr, y[r] + (uint64_t)p * row * E, outer, row, row, 0, sy);
            const uint64_t w0 = op_work(args.op[2 * r]), w1 = op_work(args.op[2 * r + 1]);
            if (w0 > work) work = w0;
            if (w1 > work) work = w1;
            lo[r] = r < p ? r : p;
            hi[r] = (r < p ? p : r) + 1;
        }
        vrc_status_t rc = step<false>(args, 2 * n, work, cus, st);
        if (rc) return rc;
        for (int d = 2; d < n; d *= 2) {
            work = 0;
            for (int r = 0; r < n; r++) {
                const int p = r ^ d;
                const uint64_t off = (uint64_t)lo[p] * row * E;
                const uint64_t width = (uint64_t)(hi[p] - lo[p]) * row;
                args.op[r] = make_op(y[p] + off, nullptr, y[r] + off, outer, width, sy, 0, sy);
                const uint64_t w = op_work(args.op[r]);
                if (w > work) work = w;
            }
            rc = step<false>(args, n, work, cus, st);
            if (rc) return rc;
            for (int r = 0; r < n; r++) {
                nlo[r] = lo[r] < lo[r ^ d] ? lo[r] : lo[r ^ d];
                nhi[r] = hi[r] > hi[r ^ d] ? hi[r] : hi[r ^ d];
            }
            for (int r = 0; r < n; r++) {
                lo[r] = nlo[r];
                hi[r] = nhi[r];
            }
        }
        return VRC_OK;
    }

    // ---- single-launch ring (chained per element) ------------------------
    template <bool MEM>
    static vrc_status_t chain_allreduce(const char* const* x, char* const* y, int n, uint64_t count, int cus,
                                        hipStream_t st)
    {
        if (n == 1) return x[0] == y[0] ? VRC_OK : copy(x[0], y[0], 1, count, 0, 0, cus, st);
        vrc::ChainArgs a = {};
        for (int r = 0; r < kMaxRanks; r++) {
            a.src[r] = r < n ? x[r] : nullptr;
            a.dst[r] = r < n ? y[r] : nullptr;
        }
        // Tiles of one 16-byte vector per lane of a 64-lane wave, per chunk.
        a.tile0[0] = 0;
        for (int c = 0; c < n; c++) {
            uint64_t off, len;
            chunk_range(count, n, c, &off, &len);
            uintptr_t addr[2 * kMaxRanks];
            for (int r = 0; r < n; r++) {
                addr[2 * r] = (uintptr_t)(x[r] + off * E);
                addr[2 * r + 1] = (uintptr_t)(y[r] + off * E);
            }
            a.ch[c] = {off, 1, len, 0, split_rows(addr, 2 * n, 1, nullptr, 0, len, E)};
            a.tile0[c + 1] = a.tile0[c] + (a.ch[c].g.nvb + 63) / 64;
        }
        // At least one wave per chunk for the scalar head/tail pass.
        const uint64_t lanes = a.tile0[n] * 64, scalar_lanes = (uint64_t)n * 64;
        const uint64_t work = lanes > scalar_lanes ? lanes : scalar_lanes;
        const ChainShape sh = chain_ar_shape(MEM, n);
        const dim3 grid(grid_x(cus, work, 1, sh.blocks_per_cu, sh.block));
        if (g_plan)
            return plan_single(MEM ? VRC_OP_CHAIN_ALLREDUCE : VRC_OP_RING_ORDER_ALLREDUCE, count, grid, sh.block, 1);
        switch (n) {
#define VRC_CASE(K)                                                                                      \
    case K:                                                                                              \
        if (sh.block == 64)                                                                              \
            hipLaunchKernelGGL((vrc::k_ring_chain_allreduce<T, K, MEM, true, 64>), grid, dim3(64), 0, st, a); \
        else                                                                                             \
            hipLaunchKernelGGL((vrc::k_ring_chain_allreduce<T, K, MEM, true>), grid, dim3(kBlock), 0, st, a); \
        break;
            VRC_FOR_N(VRC_CASE)
#undef VRC_CASE
        default: return VRC_ERR_INVALID_ARG;
        }
        return check_launch();
    }

    template <bool MEM>
    static vrc_status_t chain_reduce_scatter(const char* const* x, char* const* y, int n, uint64_t count,
                                             uint64_t outer, int cus, hipStream_t st)
    {
        if (n == 1) return copy(x[0], y[0], 1, count, 0, 0, cus, st);
        if (outer == 1 && (uint64_t)(n + 1) * count * E >= 64 * kMiB) {
            // Flat chunks: the flat walk of the fused reduce-scatter.
            vrc::ChainArgs fa;
            dim3 fgrid;
            if (rs_flat_layout(x, y, n, count, cus, &fa, &fgrid)) {
                if (MEM) {
                    const uint64_t lanes = fa.tile0[n] * 64, scalar_lanes = (uint64_t)n * 64;
                    fgrid.x = grid_x(cus, lanes > scalar_lanes ? lanes : scalar_lanes, 1, chain_rs_flat_blocks_per_cu(), 64);
                }
                if (g_plan)
                    return plan_single(MEM ? VRC_OP_CHAIN_REDUCE_SCATTER : VRC_OP_RING_ORDER_REDUCE_SCATTER, count,
                                       fgrid, 64, 1);
                switch (n) {
#define VRC_CASE(K)                                                                                              \
    case K:                                                                                                      \
        hipLaunchKernelGGL((vrc::k_ring_chain_reduce_scatter_flat<T, K, MEM, true>), fgrid, dim3(64), 0, st, fa); \
        break;
                    VRC_FOR_N(VRC_CASE)
#undef VRC_CASE
                default: return VRC_ERR_INVALID_ARG;
                }
                return check_launch();
            }
        }
        vrc::ChainArgs a = {};
        uint64_t work = 0;
        for (int r = 0; r < kMaxRanks; r++) {
            a.src[r] = r < n ? x[r] : nullptr;
            a.dst[r] = r < n ? y[r] : nullptr;
        }
        for (int c = 0; c < n; c++) {
            const Chunk k = rs_chunk(count, outer, n, c);
            uintptr_t addr[kMaxRanks + 1];
            for (int r = 0; r < n; r++) addr[r] = (uintptr_t)(x[r] + k.off * E);
            addr[n] = (uintptr_t)y[c];
            const uint64_t strides[2] = {k.stride * E, k.width * E};
            a.ch[c] = {k.off, k.rows, k.width, k.stride, split_rows(addr, n + 1, k.rows, strides, 2, k.width, E)};
            const uint64_t w = k.rows * (a.ch[c].g.nvb + a.ch[c].g.head + a.ch[c].g.tail);
            if (w > work) work = w;
        }
        const uint64_t bytes = MEM ? 3 * (uint64_t)(n - 1) * count * E : (uint64_t)(n + 1) * count * E;
        const int bpc = MEM ? chain_blocks_per_cu(bytes) : fused_blocks_per_cu(bytes, n);
        const dim3 grid(grid_x(cus, work, n, bpc), (unsigned)n);
        if (g_plan)
            return plan_single(MEM ? VRC_OP_CHAIN_REDUCE_SCATTER : VRC_OP_RING_ORDER_REDUCE_SCATTER, count, grid,
                               kBlock, 1);
        switch (n) {
#define VRC_CASE(K) \
    case K:         \
        hipLaunchKernelGGL((vrc::k_ring_chain_reduce_scatter<T, K, MEM, true>), grid, dim3(kBlock), 0, st, a); break;
            VRC_FOR_N(VRC_CASE)
#undef VRC_CASE
        default: return VRC_ERR_INVALID_ARG;
        }
        return check_launch();
    }

    static vrc_status_t chain_all_gather(const char* const* x, char* const* y, int n, uint64_t count,
                                         uint64_t outer, int cus, hipStream_t st)
    {
        if (n == 1) return copy(x[0], y[0], 1, count, 0, 0, cus, st);
        vrc::FusedAgArgs a;
        const uint64_t row = count / outer;
        a.rows = outer;
        a.width = row;
        a.n = n;
        uint64_t work = 0;
        for (int r = 0; r < kMaxRanks; r++) {
            a.src[r] = r < n ? x[r] : nullptr;
            a.dst[r] = r < n ? y[r] : nullptr;
        }
        for (int q = 0; q < n; q++) {
            uintptr_t addr[kMaxRanks + 1];
            addr[0] = (uintptr_t)x[q];
            for (int r = 0; r < n; r++) addr[r + 1] = (uintptr_t)(y[r] + (uint64_t)q * row * E);
            const uint64_t strides[2] = {row * E, (uint64_t)n * row * E};
            a.g[q] = split_rows(addr, n + 1, outer, strides, 2, row, E);
            const uint64_t w = outer * (a.g[q].nvb + a.g[q].head + a.g[q].tail);
            if (w > work) work = w;
        }
        const dim3 grid(grid_x(cus, work, n, chain_blocks_per_cu(2 * (uint64_t)n * n * count * E)), (unsigned)n);
        if (g_plan) return plan_single(VRC_OP_CHAIN_ALL_GATHER, count, grid, kBlock, 1);
        switch (n) {
#define VRC_CASE(K) \
    case K: hipLaunchKernelGGL((vrc::k_ring_chain_all_gather<T, K, true>), grid, dim3(kBlock), 0, st, a); break;
            VRC_FOR_N(VRC_CASE)
#undef VRC_CASE
        default: return VRC_ERR_INVALID_ARG;
        }
        return check_launch();
    }
};

enum class Coll { AR, RS, AG };

template <class T>
vrc_status_t run_typed(Coll coll, vrc_mode_t mode, const char* const* x, char* const* y, int n, uint64_t count,
                       uint64_t outer, int cus, hipStream_t st)
{
    using L = Launch<T>;
    switch (coll) {
    case Coll::AR:
        switch (mode) {
        case VRC_RING: return L::ring_allreduce(x, y, n, count, cus, st);
        case VRC_FUSED: return L::fused_allreduce(x, y, n, count, cus, st);
        case VRC_RING_CHAINED: return L::template chain_allreduce<true>(x, y, n, count, cus, st);
        case VRC_RING_ORDER: return L::template chain_allreduce<false>(x, y, n, count, cus, st);
        case VRC_HD: return L::hd_allreduce(x, y, n, count, cus, st);
        // At 2 ranks the butterfly is one add rounded once, the rank fold bit for bit; the rank-fold
        // kernel runs it as fast as the fused mode (2 x 2 GiB bf16: 1.65 ms against 1.96 ms).
        case VRC_HD_ORDER:
            return n == 2 ? L::fused_allreduce(x, y, n, count, cus, st)
                          : L::template fused_allreduce<vrc::Butterfly>(x, y, n, count, cus, st);
        case VRC_SELECT: break;  // resolved to VRC_HD or VRC_RING by the entry point
        }
        break;
    case Coll::RS:
        switch (mode) {
        case VRC_RING: return L::ring_reduce_scatter(x, y, n, count, outer, cus, st);
        case VRC_FUSED: return L::fused_reduce_scatter(x, y, n, count, outer, cus, st);
        case VRC_RING_CHAINED: return L::template chain_reduce_scatter<true>(x, y, n, count, outer, cus, st);
        case VRC_RING_ORDER: return L::template chain_reduce_scatter<false>(x, y, n, count, outer, cus, st);
        case VRC_HD:
        case VRC_HD_ORDER:
            return n == 2 ? L::fused_reduce_scatter(x, y, n, count, outer, cus, st)
                          : L::template fused_reduce_scatter<vrc::Butterfly>(x, y, n, count, outer, cus, st);
        case VRC_SELECT: break;
        }
        break;
    case Coll::AG:
        switch (mode) {
        case VRC_RING: return L::ring_all_gather(x, y, n, count, outer, cus, st);
        case VRC_FUSED:
        case VRC_RING_ORDER:
        case VRC_HD_ORDER: return L::fused_all_gather(x, y, n, count, outer, cus, st);
        case VRC_RING_CHAINED: return L::chain_all_gather(x, y, n, count, outer, cus, st);
        case VRC_HD: return L::hd_all_gather(x, y, n, count, outer, cus, st);
        case VRC_SELECT: break;
        }
        break;
    }
    return VRC_ERR_UNSUPPORTED;
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

bool mode_ok(vrc_mode_t m)
{
    return m == VRC_RING || m == VRC_FUSED || m == VRC_RING_CHAINED || m == VRC_RING_ORDER || m == VRC_HD ||
           m == VRC_HD_ORDER || m == VRC_SELECT;
}

// VRC_SELECT: halving-doubling for power-of-two rank counts and inputs of at
// most VRC_SELECT_HD_MAX_BYTES per rank (log2 N steps win while launches
// dominate), else the ring.
vrc_mode_t resolve_mode(vrc_mode_t m, int n, uint64_t bytes_per_rank)
{
    if (m != VRC_SELECT) return m;
    const bool pow2 = (n & (n - 1)) == 0;
    return pow2 && bytes_per_rank <= VRC_SELECT_HD_MAX_BYTES ? VRC_HD : VRC_RING;
}

// Halving-doubling pairs rank r with r XOR d, so it needs a power of two.
bool ranks_ok_for(vrc_mode_t m, int n)
{
    if (m != VRC_HD && m != VRC_HD_ORDER) return true;
    return (n & (n - 1)) == 0;
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
    switch (coll) {
    case VRC_COLL_ALLREDUCE: rc = vrc_allreduce(send, recv, nranks, count, dtype, VRC_SUM, mode, nullptr); break;
    case VRC_COLL_REDUCE_SCATTER:
        rc = vrc_reduce_scatter(send, recv, nranks, count, outer, dtype, VRC_SUM, mode, nullptr);
        break;
    case VRC_COLL_ALL_GATHER: rc = vrc_all_gather(send, recv, nranks, count, outer, dtype, mode, nullptr); break;
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
    vrc_status_t rc = check_common(send, recv, nranks, count, dtype);
    if (rc) return rc;
    if (op != VRC_SUM || !mode_ok(mode)) return VRC_ERR_UNSUPPORTED;
    const uint64_t bytes = (uint64_t)count * (uint64_t)esize(dtype);
    mode = resolve_mode(mode, nranks, bytes);
    if (!ranks_ok_for(mode, nranks)) return VRC_ERR_INVALID_ARG;
    uint64_t rb[kMaxRanks];
    for (int r = 0; r < nranks; r++) rb[r] = bytes;
    rc = check_buffers(send, recv, nranks, bytes, rb, true);
    if (rc) return rc;
    if (count == 0) return VRC_OK;
    return run(Coll::AR, mode, dtype, send, recv, nranks, count, 1, (hipStream_t)stream);
}

vrc_status_t vrc_reduce_scatter(const void* const* send, void* const* recv, int nranks, size_t count,
                                size_t outer, vrc_dtype_t dtype, vrc_op_t op, vrc_mode_t mode,
                                vrc_stream_t stream)
{
    vrc_status_t rc = check_common(send, recv, nranks, count, dtype);
    if (rc) return rc;
    if (op != VRC_SUM || !mode_ok(mode)) return VRC_ERR_UNSUPPORTED;
    const int E = esize(dtype);
    mode = resolve_mode(mode, nranks, (uint64_t)count * E);
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
    return run(Coll::RS, mode, dtype, send, recv, nranks, count, outer, (hipStream_t)stream);
}

vrc_status_t vrc_all_gather(const void* const* send, void* const* recv, int nranks, size_t count,
                            size_t outer, vrc_dtype_t dtype, vrc_mode_t mode, vrc_stream_t stream)
{
    vrc_status_t rc = check_common(send, recv, nranks, count, dtype);
    if (rc) return rc;
    if (!mode_ok(mode)) return VRC_ERR_UNSUPPORTED;
    const int E = esize(dtype);
    mode = resolve_mode(mode, nranks, (uint64_t)count * E);
    if (!ranks_ok_for(mode, nranks)) return VRC_ERR_INVALID_ARG;
    if (outer == 0 || count % outer != 0) return VRC_ERR_INVALID_ARG;
    uint64_t rb[kMaxRanks];
    for (int r = 0; r < nranks; r++) rb[r] = (uint64_t)count * (uint64_t)nranks * E;
    rc = check_buffers(send, recv, nranks, (uint64_t)count * E, rb, false);
    if (rc) return rc;
    if (count == 0) return VRC_OK;
    return run(Coll::AG, mode, dtype, send, recv, nranks, count, outer, (hipStream_t)stream);
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
    switch (status) {
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
