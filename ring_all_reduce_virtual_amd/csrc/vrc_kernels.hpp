// vrc_kernels.hpp -- HIP kernels (gfx950) for the virtual-rank collectives.
//
// All kernels are bandwidth-bound streaming loops: a grid sized to the CU
// count, grid-stride iteration over 16-byte vectors, and a scalar pass for
// the elements before the first 16-byte boundary and after the last one.
// Workgroups have 256 lanes (four wave64s), except in the all-reduce kernels
// that read every rank at once (fused and single-launch ring) and the ring
// step, which the host may launch with workgroups of one wave (template
// argument B = 64).  No MFMA:
// the work is a sum, not a contraction.
//
// Geometry.  An operand region is `rows` rows of `width` elements with a row
// stride in elements.  The host splits each row into `head` scalar elements
// (up to the destination's first 128-byte boundary), `nvb` 16-byte vectors
// and `tail` scalar elements (less than one vector).  Operands on other
// offsets than the destination still move in 16-byte vectors (unaligned
// access), so only heads and tails run scalar: at most 127 + 15 bytes per
// row.
#pragma once

#include "vrc_elem.hpp"

namespace vrc {

constexpr int kBlock = 256;
constexpr int kMaxRanks = 16;
constexpr int kMaxStepOps = 2 * kMaxRanks;

struct RowSplit {
    uint64_t head, nvb, tail;
};

// Map a scalar slot k (0 <= k < rows*(head+tail)) to (row, column).
__device__ __forceinline__ void scalar_slot(uint64_t k, const RowSplit& g, uint64_t vec, uint64_t& row,
                                            uint64_t& col)
{
    const uint64_t per_row = g.head + g.tail;
    row = k / per_row;
    const uint64_t j = k - row * per_row;
    col = (j < g.head) ? j : g.head + g.nvb * vec + (j - g.head);
}

// ---------------------------------------------------------------------------
// Ring step: one launch runs one reduce-scatter step (d = a + b) or one
// all-gather step (d = a) for every rank at once; blockIdx.y is the rank's
// operation.  Both operands of an add are loaded before the add, and with
// U = 2 a lane keeps two vectors (four loads of an add) in flight.  B lanes
// per workgroup (256, or one wave for the large adds of a few ranks).
// ---------------------------------------------------------------------------
struct StepOp {
    const char* a;  // element (0,0) of the first operand region
    const char* b;  // second operand (add only)
    char* d;        // destination
    uint64_t rows, width;
    uint64_t sa, sb, sd;  // row strides, elements
    RowSplit g;
};

// The operations of one step.  A kernel's arguments are copied at every
// launch, so each launch passes only as many slots as its step uses: K = 4,
// 8, 16 or 32 (352 B to 2,816 B; six back-to-back launches of an empty
// kernel take 16.6 us with 352 B of arguments and 25.2 us with 2,816 B).
template <int K>
struct StepArgsK {
    StepOp op[K];
};
using StepArgs = StepArgsK<kMaxStepOps>;

template <class T, bool ADD, bool NT, int K, int U = 1, int B = kBlock>
__global__ __launch_bounds__(B) void k_ring_step(StepArgsK<K> args)
{
    const StepOp& op = args.op[blockIdx.y];
    const uint64_t tid = (uint64_t)blockIdx.x * B + threadIdx.x;
    const uint64_t nthreads = (uint64_t)gridDim.x * B;
    constexpr uint64_t E = T::ESZ;

    const uint64_t nv = op.rows * op.g.nvb;
    const uint64_t body = op.g.head * E;
    if (op.rows == 1) {
        uint64_t v = tid;
        if constexpr (U > 1) {
            for (; v + (U - 1) * nthreads < nv; v += U * nthreads) {
                u32x4 x[U], y[U];
#pragma unroll
                for (int u = 0; u < U; u++) {
                    x[u] = ld16<NT>(op.a + body + (v + u * nthreads) * 16);
                    if constexpr (ADD) y[u] = ld16<NT>(op.b + body + (v + u * nthreads) * 16);
                }
                issue_loads_first();
#pragma unroll
                for (int u = 0; u < U; u++) {
                    if constexpr (ADD) x[u] = add_v<T>(x[u], y[u]);
                    st16<NT>(op.d + body + (v + u * nthreads) * 16, x[u]);
                }
            }
        }
        for (; v < nv; v += nthreads) {
            const uint64_t off = body + v * 16;
            u32x4 x = ld16<NT>(op.a + off), y;
            if constexpr (ADD) y = ld16<NT>(op.b + off);
            issue_loads_first();
            if constexpr (ADD) x = add_v<T>(x, y);
            st16<NT>(op.d + off, x);
        }
    } else {
        for (uint64_t v = tid; v < nv; v += nthreads) {
            const uint64_t row = v / op.g.nvb;
            const uint64_t col = (v - row * op.g.nvb) * 16 + body;
            u32x4 x = ld16<NT>(op.a + row * op.sa * E + col), y;
            if constexpr (ADD) y = ld16<NT>(op.b + row * op.sb * E + col);
            issue_loads_first();
            if constexpr (ADD) x = add_v<T>(x, y);
            st16<NT>(op.d + row * op.sd * E + col, x);
        }
    }

    // Scalar elements: heads and tails, which make up whole regions of many
    // narrow rows.  A lane takes SU elements per iteration and issues all
    // their loads before the adds and stores.
    constexpr int SU = 8;
    const uint64_t ns = op.rows * (op.g.head + op.g.tail);
    uint64_t k = tid;
    for (; k + (SU - 1) * nthreads < ns; k += SU * nthreads) {
        typename T::S x[SU], y[SU];
        uint64_t od[SU];
#pragma unroll
        for (int u = 0; u < SU; u++) {
            uint64_t row, col;
            scalar_slot(k + u * nthreads, op.g, T::VEC, row, col);
            x[u] = load_s<T>(op.a + (row * op.sa + col) * E);
            if constexpr (ADD) y[u] = load_s<T>(op.b + (row * op.sb + col) * E);
            od[u] = (row * op.sd + col) * E;
        }
        issue_loads_first();
#pragma unroll
        for (int u = 0; u < SU; u++) {
            if constexpr (ADD) x[u] = add_s<T>(x[u], y[u]);
            store_s<T>(op.d + od[u], x[u]);
        }
    }
    for (; k < ns; k += nthreads) {
        uint64_t row, col;
        scalar_slot(k, op.g, T::VEC, row, col);
        typename T::S x = load_s<T>(op.a + (row * op.sa + col) * E);
        if constexpr (ADD) x = add_s<T>(x, load_s<T>(op.b + (row * op.sb + col) * E));
        store_s<T>(op.d + (row * op.sd + col) * E, x);
    }
}

// ---------------------------------------------------------------------------
// Fused all-reduce: every lane reads element block i of all N inputs, folds
// them in rank order in the accumulator, rounds once and writes the result
// to all N outputs.  Reads precede writes within a lane, so in-place calls
// are safe.  U vectors per lane per iteration keep U*N 16-byte loads in
// flight.
//  B = 64 (one-wave workgroups): a wave takes U consecutive 1 KiB tiles per
//  iteration and stores them back to back, so a 64-byte write block that an
//  output off the vector grid splits between two of its tiles is filled by
//  one wave at once, and the cache merges it; workgroups go to the XCDs in
//  turn, U KiB each.  (Outputs on different 128-byte offsets with none in
//  place take k_fused_allreduce_realigned below instead.)
//  B = 256: the U vectors of a lane are one grid stride apart.
// ---------------------------------------------------------------------------
struct FusedArArgs {
    const char* src[kMaxRanks];
    char* dst[kMaxRanks];
    uint64_t count;  // elements per rank
    RowSplit g;      // one row of `count` elements
};

template <class T, int N>
__device__ __forceinline__ u32x4 fold_v(const u32x4* in)
{
    typename T::A acc[T::VEC], x[T::VEC];
    T::unpack(in[0], acc);
#pragma unroll
    for (int r = 1; r < N; r++) {
        T::unpack(in[r], x);
#pragma unroll
        for (int i = 0; i < T::VEC; i++) acc[i] = T::add(acc[i], x[i]);
    }
    return T::pack(acc);
}

// How the fused kernels combine the N values of one element.
//  RankFold:  x_0 + x_1 + ... + x_{N-1} folded left in the accumulator type,
//             rounded once (the collector all-reduce).
//  Butterfly: halving-doubling order, N a power of two: pairs at distance
//             N/2 first, then N/4, ..., each partial rounded to the storage
//             type: v[r] = v[r] (+) v[r + d] for r < d, d = N/2 .. 1.
struct RankFold {
    template <class T, int N>
    __device__ static u32x4 vec(u32x4* in) { return fold_v<T, N>(in); }
    template <class T, int N>
    __device__ static typename T::S scalar(typename T::S* in)
    {
        typename T::A acc = T::widen(in[0]);
#pragma unroll
        for (int r = 1; r < N; r++) acc = T::add(acc, T::widen(in[r]));
        return T::narrow(acc);
    }
};

struct Butterfly {
    template <class T, int N>
    __device__ static u32x4 vec(u32x4* in)
    {
        static_assert((N & (N - 1)) == 0, "butterfly needs a power of two");
#pragma unroll
        for (int d = N / 2; d >= 1; d /= 2)
#pragma unroll
            for (int r = 0; r < d; r++) in[r] = add_v<T>(in[r], in[r + d]);
        return in[0];
    }
    template <class T, int N>
    __device__ static typename T::S scalar(typename T::S* in)
    {
#pragma unroll
        for (int d = N / 2; d >= 1; d /= 2)
#pragma unroll
            for (int r = 0; r < d; r++) in[r] = add_s<T>(in[r], in[r + d]);
        return in[0];
    }
};

// The fused all-reduce's vectors, U per lane one grid stride apart.
template <class T, int N, int U, bool NT, class Fold>
__device__ __forceinline__ void fused_strided(const FusedArArgs& a, uint64_t tid, uint64_t nthreads, uint64_t body,
                                              uint64_t nv)
{
    uint64_t v = tid;
    if constexpr (U > 1) {
        for (; v + (U - 1) * nthreads < nv; v += U * nthreads) {
            u32x4 in[U][N];
#pragma unroll
            for (int u = 0; u < U; u++)
#pragma unroll
                for (int r = 0; r < N; r++) in[u][r] = ld16<NT>(a.src[r] + body + (v + u * nthreads) * 16);
            issue_loads_first();
#pragma unroll
            for (int u = 0; u < U; u++) {
                const u32x4 s = Fold::template vec<T, N>(in[u]);
#pragma unroll
                for (int r = 0; r < N; r++) st16<NT>(a.dst[r] + body + (v + u * nthreads) * 16, s);
            }
        }
    }
    for (; v < nv; v += nthreads) {
        u32x4 in[N];
#pragma unroll
        for (int r = 0; r < N; r++) in[r] = ld16<NT>(a.src[r] + body + v * 16);
        issue_loads_first();
        const u32x4 s = Fold::template vec<T, N>(in);
#pragma unroll
        for (int r = 0; r < N; r++) st16<NT>(a.dst[r] + body + v * 16, s);
    }
}

template <class T, int N, int U, bool NT, class Fold = RankFold, int B = kBlock>
__global__ __launch_bounds__(B) void k_fused_allreduce(FusedArArgs a)
{
    const uint64_t tid = (uint64_t)blockIdx.x * B + threadIdx.x;
    const uint64_t nthreads = (uint64_t)gridDim.x * B;
    constexpr uint64_t E = T::ESZ;
    const uint64_t body = a.g.head * E;
    const uint64_t nv = a.g.nvb;

    if constexpr (B == 64) {
        // Groups of U whole wave tiles, with no bounds test inside: across a
        // branch the compiler cannot count the outstanding accesses, and it
        // waits for every one of them (a tile's stores included) before the
        // next tile's fold.  The tiles after the last whole group, the last one
        // partial, go one per wave.
        constexpr uint64_t W = 64;
        const uint64_t lane = threadIdx.x;
        const uint64_t groups = nv / W / U;
        for (uint64_t g = blockIdx.x; g < groups; g += gridDim.x) {
            const uint64_t v0 = g * U * W + lane;
            u32x4 in[U][N];
#pragma unroll
            for (int u = 0; u < U; u++)
#pragma unroll
                for (int r = 0; r < N; r++) in[u][r] = ld16<NT>(a.src[r] + body + (v0 + u * W) * 16);
            issue_loads_first();
#pragma unroll
            for (int u = 0; u < U; u++) {
                const u32x4 s = Fold::template vec<T, N>(in[u]);
#pragma unroll
                for (int r = 0; r < N; r++) st16<NT>(a.dst[r] + body + (v0 + u * W) * 16, s);
            }
        }
        for (uint64_t v = (groups * U + blockIdx.x) * W + lane; v < nv; v += (uint64_t)gridDim.x * W) {
            u32x4 in[N];
#pragma unroll
            for (int r = 0; r < N; r++) in[r] = ld16<NT>(a.src[r] + body + v * 16);
            issue_loads_first();
            const u32x4 s = Fold::template vec<T, N>(in);
#pragma unroll
            for (int r = 0; r < N; r++) st16<NT>(a.dst[r] + body + v * 16, s);
        }
    } else {
        fused_strided<T, N, U, NT, Fold>(a, tid, nthreads, body, nv);
    }

    const uint64_t ns = a.g.head + a.g.tail;
    for (uint64_t k = tid; k < ns; k += nthreads) {
        const uint64_t i = (k < a.g.head) ? k : a.g.head + a.g.nvb * T::VEC + (k - a.g.head);
        typename T::S in[N];
#pragma unroll
        for (int r = 0; r < N; r++) in[r] = load_s<T>(a.src[r] + i * E);
        const typename T::S s = Fold::template scalar<T, N>(in);
#pragma unroll
        for (int r = 0; r < N; r++) store_s<T>(a.dst[r] + i * E, s);
    }
}

// ---------------------------------------------------------------------------
// Phased fused all-reduce: one 256-lane workgroup per CU, one wave per SIMD.
// Half reads and half writes make the DRAM turn its bus around between read
// and write bursts, and writes held in the Infinity Cache behind L2 drain
// among later reads unless a run of writes is much longer than that cache.
// So every lane folds K = KR + KL vectors of every input (KR sums held in
// registers, KL in LDS; N * K * 16 bytes of reads per lane, 0.5-1 GiB per
// phase over the grid), the grid meets, and every lane then writes its K
// sums to all N outputs.
//
// The meeting only shapes the timing: a lane reads and writes its own
// vectors only, so a late or skipped meeting cannot change any result.  A
// workgroup waits at most as long as its own read phase took (at least
// kPhaseWaitFloor ticks); one that gives up once stops waiting for the rest
// of the launch, so a grid that is not all resident (a busy GPU, another
// such launch at the same time) costs bounded time and finishes.
// ---------------------------------------------------------------------------

// Arrivals at the phased kernels' meetings on this device since the library
// was loaded (64 bits: never wraps).  Every launch has one workgroup per CU,
// G of them, and each adds G per meeting, so between launches the count is a
// multiple of G and count / G numbers the meetings.  Each translation unit
// (one per element type) has its own count.
static __device__ unsigned long long g_phase_arrivals;

// 20 us of the 100 MHz wall clock gfx950 reports.
constexpr uint64_t kPhaseWaitFloor = 2000;

__device__ __forceinline__ void phase_meet(uint64_t G, uint64_t limit, bool& waiting)
{
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned long long seen =
            __hip_atomic_fetch_add(&g_phase_arrivals, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (waiting) {
            const unsigned long long all = (seen / G + 1) * G;
            const uint64_t t0 = wall_clock64();
            while (__hip_atomic_load(&g_phase_arrivals, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < all) {
                if (wall_clock64() - t0 > limit) {
                    waiting = false;
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
            }
        }
    }
    __syncthreads();
}

// Slot k of lane ((w * G + b) * 64 + l), for wave w of workgroup b and lane
// l, is vector k * L + that lane of its phase (L lanes in the grid), so
// consecutive 1 KiB tiles go to consecutive workgroups (consecutive XCDs),
// as in the one-wave kernel above.  With `skew` > 0 (G a multiple of 8) the
// workgroups of odd index hold `skew` fewer LDS sums than the others: every
// workgroup holds the first K - skew slots in that layout, and the even
// workgroups' last `skew` slots follow them, L / 2 lanes wide (lane
// ((w * G/2 + b/2) * 64 + l)).  On MI355X the workgroups on odd XCDs issue
// their stores more slowly than those on even ones, and the lighter share
// evens out the time each spends on a phase.  The vectors after the last
// whole phase and the scalar head and tail follow with the grid-stride
// loops.  `wait` = 0 skips every meeting.
template <class T, int N, int KR, int KL, bool NT, class Fold = RankFold>
__global__ __launch_bounds__(kBlock, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_fused_allreduce_phased(FusedArArgs a, uint64_t phases, uint32_t wait, uint32_t skew)
{
    constexpr int K = KR + KL;
    __shared__ u32x4 held[KL * kBlock];
    const uint64_t G = gridDim.x;
    const uint64_t L = G * kBlock;
    const uint64_t w = threadIdx.x >> 6, l = threadIdx.x & 63;
    const uint64_t lane = (w * G + blockIdx.x) * 64 + l;
    const uint64_t lane_even = (w * (G / 2) + (blockIdx.x >> 1)) * 64 + l;
    const uint64_t shared_slots = (uint64_t)K - skew;
    const int held_here = (blockIdx.x & 1) ? KL - (int)skew : KL;
    const uint64_t per_phase = shared_slots * L + (uint64_t)skew * (L / 2);
    constexpr uint64_t E = T::ESZ;
    const uint64_t body = a.g.head * E;
    bool waiting = wait != 0;

    for (uint64_t p = 0; p < phases; p++) {
        const uint64_t start = p * per_phase;
        // vector of LDS slot k (register slots k < KR <= K - skew are at start + k * L + lane)
        auto held_at = [&](int k) -> uint64_t {
            const uint64_t slot = (uint64_t)(KR + k);
            return slot < shared_slots ? start + slot * L + lane
                                       : start + shared_slots * L + (slot - shared_slots) * (L / 2) + lane_even;
        };
        const uint64_t t_read = wall_clock64();
        u32x4 s[KR];
#pragma unroll
        for (int k = 0; k < KR; k++) {
            u32x4 in[N];
            const uint64_t v = start + k * L + lane;
#pragma unroll
            for (int r = 0; r < N; r++) in[r] = ld16<NT>(a.src[r] + body + v * 16);
            issue_loads_first();
            s[k] = Fold::template vec<T, N>(in);
            __asm__ __volatile__("" : "+v"(s[k]));  // keep the sum in a register until the write phase
        }
#pragma unroll
        for (int k = 0; k < KL; k++) {
            if (k < held_here) {
                u32x4 in[N];
                const uint64_t v = held_at(k);
#pragma unroll
                for (int r = 0; r < N; r++) in[r] = ld16<NT>(a.src[r] + body + v * 16);
                issue_loads_first();
                held[k * kBlock + threadIdx.x] = Fold::template vec<T, N>(in);
            }
        }
        const uint64_t took = wall_clock64() - t_read;
        phase_meet(G, took > kPhaseWaitFloor ? took : kPhaseWaitFloor, waiting);
#pragma unroll
        for (int k = 0; k < KR; k++) {
            const uint64_t v = start + k * L + lane;
#pragma unroll
            for (int r = 0; r < N; r++) st16<NT>(a.dst[r] + body + v * 16, s[k]);
        }
#pragma unroll
        for (int k = 0; k < KL; k++) {
            if (k < held_here) {
                const u32x4 f = held[k * kBlock + threadIdx.x];
                const uint64_t v = held_at(k);
#pragma unroll
                for (int r = 0; r < N; r++) st16<NT>(a.dst[r] + body + v * 16, f);
            }
        }
    }

    for (uint64_t v = phases * per_phase + lane; v < a.g.nvb; v += L) {
        u32x4 in[N];
#pragma unroll
        for (int r = 0; r < N; r++) in[r] = ld16<NT>(a.src[r] + body + v * 16);
        issue_loads_first();
        const u32x4 f = Fold::template vec<T, N>(in);
#pragma unroll
        for (int r = 0; r < N; r++) st16<NT>(a.dst[r] + body + v * 16, f);
    }

    const uint64_t ns = a.g.head + a.g.tail;
    for (uint64_t k = (uint64_t)blockIdx.x * kBlock + threadIdx.x; k < ns; k += L) {
        const uint64_t i = (k < a.g.head) ? k : a.g.head + a.g.nvb * T::VEC + (k - a.g.head);
        typename T::S in[N];
#pragma unroll
        for (int r = 0; r < N; r++) in[r] = load_s<T>(a.src[r] + i * E);
        const typename T::S s = Fold::template scalar<T, N>(in);
#pragma unroll
        for (int r = 0; r < N; r++) store_s<T>(a.dst[r] + i * E, s);
    }
}

// ---------------------------------------------------------------------------
// Fused all-reduce for outputs on different 128-byte offsets (one-wave
// workgroups, no output overlapping an input).  The loads follow one
// reference grid; output r is stored `shift[r]` bytes later, on its own
// 128-byte grid, so every store of the main loop fills whole write blocks
// whatever the output offsets.  A wave folds U tiles of the reference grid
// plus the 128 bytes after them into LDS, then reads each output's 16 bytes
// per lane back at that output's shift.  The 128 bytes are read again by the
// next group's wave (1/(8U) more input reads).
//
// Stores outside the groups (the 128 bytes before every output's first
// boundary, the vectors after the last group, the scalar head and tail) go
// to every output at the reference offsets.  Where they overlap a group's
// stores both write the same sum, and no input is overwritten: inputs and
// outputs are disjoint.
// ---------------------------------------------------------------------------
struct FusedRealignArgs {
    const char* src[kMaxRanks];
    char* dst[kMaxRanks];
    uint32_t shift[kMaxRanks];  // bytes from the body start to output r's next 128-byte boundary, < 128
    uint64_t groups;            // groups of U tiles whose next 128 bytes lie in the body
    RowSplit g;
};

// Lane `lane`'s 16 bytes of U tiles of one output, d bytes past the sums
// staged in LDS (d < 128, (d / 4) % 4 == Q).
template <int Q, int U>
__device__ __forceinline__ void shifted(u32x4* out, const u32x4* sum, uint64_t lane, uint32_t d)
{
    const uint64_t k0 = lane + d / 16;  // + u * 64 + 1 <= U * 64 + 7
    const uint32_t s = d % 4;
#pragma unroll
    for (int u = 0; u < U; u++) {
        const u32x4 lo = sum[u * 64 + k0], hi = sum[u * 64 + k0 + 1];
        const unsigned w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        out[u] = funnel<Q>(w, s);
    }
}

template <class T, int N, int U, bool NT, class Fold>
__global__ __launch_bounds__(64) void k_fused_allreduce_realigned(FusedRealignArgs a)
{
    constexpr uint64_t W = 64;
    constexpr uint64_t E = T::ESZ;
    constexpr uint64_t X = 8;  // 16-byte vectors past a group: 128 bytes
    __shared__ u32x4 sum[U * W + X];
    const uint64_t lane = threadIdx.x;
    const uint64_t body = a.g.head * E;

    for (uint64_t g = blockIdx.x; g < a.groups; g += gridDim.x) {
        const uint64_t v0 = g * U * W;
        u32x4 in[U + 1][N];
#pragma unroll
        for (int u = 0; u < U; u++)
#pragma unroll
            for (int r = 0; r < N; r++) in[u][r] = ld16<NT>(a.src[r] + body + (v0 + u * W + lane) * 16);
#pragma unroll
        for (int r = 0; r < N; r++) in[U][r] = ld16<NT>(a.src[r] + body + (v0 + U * W + (lane % X)) * 16);
        issue_loads_first();
#pragma unroll
        for (int u = 0; u < U; u++) sum[u * W + lane] = Fold::template vec<T, N>(in[u]);
        const u32x4 next = Fold::template vec<T, N>(in[U]);
        if (lane < X) sum[U * W + lane] = next;
        __syncthreads();
        // Every output's vectors first, then all U * N stores back to back: a
        // register that still feeds a store in flight is not overwritten
        // before that store completes, so the stores must not share registers.
        u32x4 out[N][U];
#pragma unroll
        for (int r = 0; r < N; r++) {
            const uint32_t d = a.shift[r];
            switch ((d / 4) % 4) {  // the same for every lane: one scalar branch per output
            case 0: shifted<0, U>(out[r], sum, lane, d); break;
            case 1: shifted<1, U>(out[r], sum, lane, d); break;
            case 2: shifted<2, U>(out[r], sum, lane, d); break;
            default: shifted<3, U>(out[r], sum, lane, d); break;
            }
        }
        issue_loads_first();
#pragma unroll
        for (int r = 0; r < N; r++)
#pragma unroll
            for (int u = 0; u < U; u++)
                st16<NT>(a.dst[r] + body + (v0 + u * W + lane) * 16 + a.shift[r], out[r][u]);
        __syncthreads();
    }

    // The first X vectors and those after the last group, at the reference
    // offsets (groups >= 1, so the two ranges are disjoint).
    const uint64_t rest0 = a.groups * U * W;
    const uint64_t nrest = X + (a.g.nvb - rest0);
    for (uint64_t k = (uint64_t)blockIdx.x * W + lane; k < nrest; k += (uint64_t)gridDim.x * W) {
        const uint64_t v = k < X ? k : rest0 + (k - X);
        u32x4 in[N];
#pragma unroll
        for (int r = 0; r < N; r++) in[r] = ld16<NT>(a.src[r] + body + v * 16);
        const u32x4 s = Fold::template vec<T, N>(in);
#pragma unroll
        for (int r = 0; r < N; r++) st16<NT>(a.dst[r] + body + v * 16, s);
    }

    const uint64_t ns = a.g.head + a.g.tail;
    for (uint64_t k = (uint64_t)blockIdx.x * W + lane; k < ns; k += (uint64_t)gridDim.x * W) {
        const uint64_t i = (k < a.g.head) ? k : a.g.head + a.g.nvb * T::VEC + (k - a.g.head);
        typename T::S in[N];
#pragma unroll
        for (int r = 0; r < N; r++) in[r] = load_s<T>(a.src[r] + i * E);
        const typename T::S s = Fold::template scalar<T, N>(in);
#pragma unroll
        for (int r = 0; r < N; r++) store_s<T>(a.dst[r] + i * E, s);
    }
}

// ---------------------------------------------------------------------------
// Fused reduce-scatter: blockIdx.y = chunk c.  Output c is the rank-order
// fold of chunk c over all N inputs, rounded once.
// ---------------------------------------------------------------------------
struct RsChunk {
    uint64_t src_off;  // element offset of chunk c's (0,0) in every input
    char* d;           // output c
    uint64_t rows, width;
    uint64_t s_src, s_dst;  // row strides, elements
    RowSplit g;
};

struct FusedRsArgs {
    const char* src[kMaxRanks];
    RsChunk ch[kMaxRanks];
};

template <class T, int N, bool NT, class Fold = RankFold>
__global__ __launch_bounds__(kBlock) void k_fused_reduce_scatter(FusedRsArgs a)
{
    const RsChunk& c = a.ch[blockIdx.y];
    const uint64_t tid = (uint64_t)blockIdx.x * kBlock + threadIdx.x;
    const uint64_t nthreads = (uint64_t)gridDim.x * kBlock;
    constexpr uint64_t E = T::ESZ;
    const uint64_t nv = c.rows * c.g.nvb;
    for (uint64_t v = tid; v < nv; v += nthreads) {
        const uint64_t row = (c.rows == 1) ? 0 : v / c.g.nvb;
        const uint64_t col = (v - row * c.g.nvb) * 16 + c.g.head * E;
        const uint64_t so = (c.src_off + row * c.s_src) * E + col;
        u32x4 in[N];
#pragma unroll
        for (int r = 0; r < N; r++) in[r] = ld16<NT>(a.src[r] + so);
        issue_loads_first();
        st16<NT>(c.d + row * c.s_dst * E + col, Fold::template vec<T, N>(in));
    }
    // Scalar elements (heads, tails; whole chunks of many narrow rows): a
    // lane takes SU elements per iteration (about 16 loads) and issues their
    // loads first.
    constexpr int SU = N >= 16 ? 1 : 16 / N;
    const uint64_t ns = c.rows * (c.g.head + c.g.tail);
    uint64_t k = tid;
    if constexpr (SU > 1) {
        for (; k + (SU - 1) * nthreads < ns; k += SU * nthreads) {
            typename T::S in[SU][N];
            uint64_t od[SU];
#pragma unroll
            for (int u = 0; u < SU; u++) {
                uint64_t row, col;
                scalar_slot(k + u * nthreads, c.g, T::VEC, row, col);
                const uint64_t so = (c.src_off + row * c.s_src + col) * E;
#pragma unroll
                for (int r = 0; r < N; r++) in[u][r] = load_s<T>(a.src[r] + so);
                od[u] = (row * c.s_dst + col) * E;
            }
            issue_loads_first();
#pragma unroll
            for (int u = 0; u < SU; u++) store_s<T>(c.d + od[u], Fold::template scalar<T, N>(in[u]));
        }
    }
    for (; k < ns; k += nthreads) {
        uint64_t row, col;
        scalar_slot(k, c.g, T::VEC, row, col);
        const uint64_t so = (c.src_off + row * c.s_src + col) * E;
        typename T::S in[N];
#pragma unroll
        for (int r = 0; r < N; r++) in[r] = load_s<T>(a.src[r] + so);
        store_s<T>(c.d + (row * c.s_dst + col) * E, Fold::template scalar<T, N>(in));
    }
}

// ---------------------------------------------------------------------------
// Fused all-gather: blockIdx.y = source rank q.  Input q ([rows, width]) is
// read once and written into column slab q of every output ([rows,
// n*width]).
// ---------------------------------------------------------------------------
struct FusedAgArgs {
    const char* src[kMaxRanks];
    char* dst[kMaxRanks];
    uint64_t rows, width;  // input geometry; output row stride is n * width
    int n;
    RowSplit g[kMaxRanks];  // per source rank (its slab offset sets the alignment)
};

// THROTTLE: each store waits for the wave's previous one, so a wave keeps
// one store in flight and the grid's many waves carry the stream.
template <class T, bool NT, bool THROTTLE = false>
__global__ __launch_bounds__(kBlock) void k_fused_all_gather(FusedAgArgs a)
{
    const int q = blockIdx.y;
    const RowSplit& g = a.g[q];
    const uint64_t tid = (uint64_t)blockIdx.x * kBlock + threadIdx.x;
    const uint64_t nthreads = (uint64_t)gridDim.x * kBlock;
    constexpr uint64_t E = T::ESZ;
    const uint64_t s_dst = (uint64_t)a.n * a.width;
    const uint64_t slab = (uint64_t)q * a.width;
    const uint64_t nv = a.rows * g.nvb;
    for (uint64_t v = tid; v < nv; v += nthreads) {
        const uint64_t row = (a.rows == 1) ? 0 : v / g.nvb;
        const uint64_t col = (v - row * g.nvb) * 16 + g.head * E;
        const u32x4 x = ld16<NT>(a.src[q] + row * a.width * E + col);
        const uint64_t dof = (row * s_dst + slab) * E + col;
        for (int r = 0; r < a.n; r++) {
            st16<NT>(a.dst[r] + dof, x);
            if constexpr (THROTTLE) wait_vmem_below<0>();
        }
    }
    const uint64_t ns = a.rows * (g.head + g.tail);
    for (uint64_t k = tid; k < ns; k += nthreads) {
        uint64_t row, col;
        scalar_slot(k, g, T::VEC, row, col);
        const typename T::S x = load_s<T>(a.src[q] + (row * a.width + col) * E);
        const uint64_t dof = (row * s_dst + slab + col) * E;
        for (int r = 0; r < a.n; r++) store_s<T>(a.dst[r] + dof, x);
    }
}

// ---------------------------------------------------------------------------
// Single-launch ring.  In the ring schedule element i of chunk c depends only
// on element i of chunk c at the previous step: the reduce-scatter carries
// the partial of chunk c from rank c+1 to c+2 ... to c+N-1 (= c-1), and the
// all-gather relays the finished chunk from rank c-1 to c, c+1, ..., c+N-2.
// Each element is therefore an independent chain of 2(N-1) operations, and
// one launch can run every chain to the end with no grid-wide barrier.
// The all-reduce chain walks wave tiles that never cross a chunk; the
// reduce-scatter chain takes blockIdx.y = chunk c.  Either way the rank
// rotation is uniform per wave.
//
// MEM = true ("chained"): every step writes its partial into the next
// rank's buffer and the following step reads it back from there, so the
// reads and writes per step are those of the per-step ring launches.
// MEM = false ("ring order"): the partial stays in registers; every input is
// read once and every output written once (the fused kernel's traffic), with
// the ring's summation order and per-step rounding.  Both give the per-step
// ring's bits.
// ---------------------------------------------------------------------------
struct ChainChunk {
    uint64_t off;          // element offset of chunk (0,0) in every rank buffer
    uint64_t rows, width;  // chunk geometry
    uint64_t stride;       // row stride of the rank buffers, elements
    RowSplit g;
};

struct ChainArgs {
    const char* src[kMaxRanks];
    char* dst[kMaxRanks];
    ChainChunk ch[kMaxRanks];
    // Flat all-reduce layout: chunk c's 16-byte vectors form tiles of one
    // vector per lane of a wave; tile0[c] is its first tile and tile0[N]
    // the total.
    uint64_t tile0[kMaxRanks + 1];
};

// Index of the range holding `i` in a table of N+1 non-decreasing starts
// (empty ranges are skipped).
template <int N>
__device__ __forceinline__ int range_of(uint64_t i, const uint64_t* start)
{
    int c = 0;
#pragma unroll
    for (int q = 1; q < N; q++) c += (i >= start[q]) ? 1 : 0;
    return c;
}

// Element access for the chain kernels: 16-byte vectors or scalars.  Inputs
// and once-written outputs are streamed with the non-temporal hint.  The
// partials a memory-faithful chain stores and reads back a step later use
// regular loads and stores, so the re-read is served by L2 (measured on
// 8 x 512 MiB bf16: 1.91 ms, against 3.55 ms with non-temporal partials
// that go to HBM and back).
template <class T, bool NT>
struct VecIO {
    using V = u32x4;
    __device__ static V ld_in(const char* p) { return ld16<NT>(p); }
    __device__ static V ld_part(const char* p) { return ld16<false>(p); }
    __device__ static void st_part(char* p, const V& x) { st16<false>(p, x); }
    __device__ static void st_out(char* p, const V& x) { st16<NT>(p, x); }
    __device__ static V add(const V& x, const V& y) { return add_v<T>(x, y); }
};

template <class T>
struct ScalarIO {
    using V = typename T::S;
    __device__ static V ld_in(const char* p) { return load_s<T>(p); }
    __device__ static V ld_part(const char* p) { return load_s<T>(p); }
    __device__ static void st_part(char* p, const V& x) { store_s<T>(p, x); }
    __device__ static void st_out(char* p, const V& x) { store_s<T>(p, x); }
    __device__ static V add(const V& x, const V& y) { return add_s<T>(x, y); }
};

// One element block of the all-reduce chain of chunk c at byte offset o;
// in[t] and out[t] are the input and output of rank c+t (mod N).  Every
// rank's input is read once, up front (each rank holds its own data from
// the start).
//  MEM:  the ring step by step through memory.  Reduce-scatter step t adds
//        rank (c+t)'s input to the partial read back from rank (c+t-1)'s
//        output and stores the sum in rank (c+t)'s output; all-gather step s
//        reads the complete chunk back from output (c+s-1) and stores it in
//        output (c+s).  Per element: N input reads, N-2 partial reads, N-1
//        relay reads and 2(N-1) stores, the step ring's 5(N-1).
//  !MEM: the same order of additions with the partial in registers, and the
//        result stored once to every output.
template <int N, bool MEM, class IO>
__device__ __forceinline__ void chain_block(const char* const* in, char* const* out, uint64_t o)
{
    using V = typename IO::V;
    V x[N];
#pragma unroll
    for (int t = 0; t < N; t++) x[t] = IO::ld_in(in[t] + o);
    issue_loads_first();
    V p = x[0];
    if constexpr (MEM) {
#pragma unroll
        for (int t = 1; t < N; t++) {
            if (t > 1) {
                reload_fence();
                p = IO::ld_part(out[t - 1] + o);
            }
            p = IO::add(p, x[t]);
            IO::st_part(out[t] + o, p);
        }
#pragma unroll
        for (int s = 0; s < N - 1; s++) {
            reload_fence();
            IO::st_part(out[s] + o, IO::ld_part(out[(s + N - 1) % N] + o));
        }
    } else {
#pragma unroll
        for (int t = 1; t < N; t++) p = IO::add(p, x[t]);
#pragma unroll
        for (int t = 0; t < N; t++) IO::st_out(out[t] + o, p);
    }
}

// The rank buffers in ring order from chunk c's first contributor.
template <int N>
__device__ __forceinline__ void rotate_ranks(const ChainArgs& a, int c, const char** in, char** out)
{
#pragma unroll
    for (int t = 0; t < N; t++) {
        in[t] = a.src[(c + t) % N];
        out[t] = a.dst[(c + t) % N];
    }
}

// All-reduce chain over flat chunks (rows == 1).  Waves walk the tiles of
// all chunks in address order, like the fused kernel, so the whole grid
// streams through the buffers together.  A tile never crosses a chunk, so
// the chunk (and with it the ring order) is uniform across the wave; a wave
// reloads the chunk's geometry and rotated rank pointers only when its next
// tile lies in another chunk.
template <class T, int N, bool MEM, bool NT, int B = kBlock>
__global__ __launch_bounds__(B) void k_ring_chain_allreduce(ChainArgs a)
{
    constexpr uint64_t W = 64;
    constexpr uint64_t E = T::ESZ;
    const uint64_t lane = threadIdx.x % W;
    const uint64_t wave = (uint64_t)blockIdx.x * (B / W) + threadIdx.x / W;
    const uint64_t nwaves = (uint64_t)gridDim.x * (B / W);
    const uint64_t ntiles = a.tile0[N];
    const char* in[N];
    char* out[N];
    int cur = -1;
    uint64_t body = 0, nvb = 0, first = 0;
    for (uint64_t t = wave; t < ntiles; t += nwaves) {
        const int c = __builtin_amdgcn_readfirstlane(range_of<N>(t, a.tile0));
        if (c != cur) {
            cur = c;
            rotate_ranks<N>(a, c, in, out);
            body = (a.ch[c].off + a.ch[c].g.head) * E;
            nvb = a.ch[c].g.nvb;
            first = a.tile0[c];
        }
        const uint64_t v = (t - first) * W + lane;
        if (v < nvb) chain_block<N, MEM, VecIO<T, NT>>(in, out, body + v * 16);
    }

    // Scalar head and tail elements (at most 127 + 15 bytes per chunk): one
    // wave per chunk, so the chunk stays uniform here too.
    for (uint64_t cw = wave; cw < (uint64_t)N; cw += nwaves) {
        const int c = __builtin_amdgcn_readfirstlane((int)cw);
        const ChainChunk& k = a.ch[c];
        const uint64_t ns = k.g.head + k.g.tail;
        if (lane >= ns) continue;
        rotate_ranks<N>(a, c, in, out);
        for (uint64_t j = lane; j < ns; j += W) {
            const uint64_t col = (j < k.g.head) ? j : k.g.head + k.g.nvb * T::VEC + (j - k.g.head);
            chain_block<N, MEM, ScalarIO<T>>(in, out, (k.off + col) * E);
        }
    }
}

// Phased ring-order all-reduce: the phased fused kernel's schedule (one
// 256-lane workgroup per CU; read K slots, meet, write them, the odd
// workgroups `skew` slots fewer) over the tiles of the kernel above.  Slot k
// of a phase is tile k W + w of it for wave w of the W in the grid (the even
// workgroups' last `skew` slots: W / 2 tiles per slot, after the others), so
// the chunk, and with it the rank rotation that fixes the ring's fold order,
// is uniform over a wave's slot.  Lanes past a
// chunk's last vector (its last tile may be partial) load and fold that last
// vector and store its sum there again: the bits the owning lane of the same
// wave stores, which keeps every slot free of branches.  The tiles after the
// last whole phase take the loop above; so do the scalar heads and tails.
template <class T, int N, int KR, int KL, bool NT>
__global__ __launch_bounds__(kBlock, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
void k_ring_order_allreduce_phased(ChainArgs a, uint64_t phases, uint32_t wait, uint32_t skew)
{
    constexpr int K = KR + KL;
    constexpr uint64_t W = 64;
    constexpr uint64_t E = T::ESZ;
    __shared__ u32x4 held[KL * kBlock];
    const uint64_t G = gridDim.x;
    const uint64_t WV = G * (kBlock / W);
    const uint64_t lane = threadIdx.x % W;
    const uint64_t wave = ((uint64_t)(threadIdx.x / W)) * G + blockIdx.x;
    const uint64_t wave_even = ((uint64_t)(threadIdx.x / W)) * (G / 2) + (blockIdx.x >> 1);
    const uint64_t shared_slots = (uint64_t)K - skew;
    const int held_here = (blockIdx.x & 1) ? KL - (int)skew : KL;
    const uint64_t per_phase = shared_slots * WV + (uint64_t)skew * (WV / 2);
    bool waiting = wait != 0;

    // Byte offset of a slot's vector in every rank buffer, and its chunk.
    auto slot = [&](uint64_t t, int& c) {
        c = __builtin_amdgcn_readfirstlane(range_of<N>(t, a.tile0));
        const uint64_t nvb = a.ch[c].g.nvb;
        uint64_t v = (t - a.tile0[c]) * W + lane;
        v = v < nvb ? v : nvb - 1;
        return (a.ch[c].off + a.ch[c].g.head) * E + v * 16;
    };
    auto fold = [&](int c, uint64_t o) {
        u32x4 x[N];
#pragma unroll
        for (int i = 0; i < N; i++) x[i] = ld16<NT>(a.src[(c + i) % N] + o);
        issue_loads_first();
        u32x4 f = x[0];
#pragma unroll
        for (int i = 1; i < N; i++) f = add_v<T>(f, x[i]);
        return f;
    };

    for (uint64_t p = 0; p < phases; p++) {
        const uint64_t t0 = p * per_phase;
        // tile of LDS slot k (register slots k < KR <= K - skew are tile t0 + k * WV + wave)
        auto held_tile = [&](int k) -> uint64_t {
            const uint64_t j = (uint64_t)(KR + k);
            return j < shared_slots ? t0 + j * WV + wave : t0 + shared_slots * WV + (j - shared_slots) * (WV / 2) + wave_even;
        };
        const uint64_t t_read = wall_clock64();
        u32x4 s[KR > 0 ? KR : 1];
#pragma unroll
        for (int k = 0; k < KR; k++) {
            int c;
            const uint64_t o = slot(t0 + k * WV + wave, c);
            s[k] = fold(c, o);
            __asm__ __volatile__("" : "+v"(s[k]));  // keep the sum in a register until the write phase
        }
#pragma unroll
        for (int k = 0; k < KL; k++) {
            if (k < held_here) {
                int c;
                const uint64_t o = slot(held_tile(k), c);
                held[k * kBlock + threadIdx.x] = fold(c, o);
            }
        }
        const uint64_t took = wall_clock64() - t_read;
        phase_meet(G, took > kPhaseWaitFloor ? took : kPhaseWaitFloor, waiting);
#pragma unroll
        for (int k = 0; k < KR; k++) {
            int c;
            const uint64_t o = slot(t0 + k * WV + wave, c);
#pragma unroll
            for (int r = 0; r < N; r++) st16<NT>(a.dst[r] + o, s[k]);
        }
#pragma unroll
        for (int k = 0; k < KL; k++) {
            if (k < held_here) {
                int c;
                const uint64_t o = slot(held_tile(k), c);
                const u32x4 f = held[k * kBlock + threadIdx.x];
#pragma unroll
                for (int r = 0; r < N; r++) st16<NT>(a.dst[r] + o, f);
            }
        }
    }

    const char* in[N];
    char* out[N];
    for (uint64_t t = phases * per_phase + wave; t < a.tile0[N]; t += WV) {
        const int c = __builtin_amdgcn_readfirstlane(range_of<N>(t, a.tile0));
        rotate_ranks<N>(a, c, in, out);
        const uint64_t v = (t - a.tile0[c]) * W + lane;
        if (v < a.ch[c].g.nvb) chain_block<N, false, VecIO<T, NT>>(in, out, (a.ch[c].off + a.ch[c].g.head) * E + v * 16);
    }
    for (uint64_t cw = wave; cw < (uint64_t)N; cw += WV) {
        const int c = __builtin_amdgcn_readfirstlane((int)cw);
        const ChainChunk& k = a.ch[c];
        const uint64_t ns = k.g.head + k.g.tail;
        if (lane >= ns) continue;
        rotate_ranks<N>(a, c, in, out);
        for (uint64_t j = lane; j < ns; j += W) {
            const uint64_t col = (j < k.g.head) ? j : k.g.head + k.g.nvb * T::VEC + (j - k.g.head);
            chain_block<N, false, ScalarIO<T>>(in, out, (k.off + col) * E);
        }
    }
}

// Ring-order all-reduce for outputs on different 128-byte offsets (one-wave
// workgroups, no output in place): the realigned stores of the fused
// kernel, chunk by chunk.  A group of U tiles lies inside one chunk, whose
// rank rotation it takes, with the 128 bytes after it; chunk c's groups are
// [group0[c], group0[c+1]).  The vectors of a chunk outside its groups (the
// first X and those after its last group, or all of them in a chunk too
// small for a group) form rest tiles [rest0[c], rest0[c+1]), stored at the
// reference offsets like the tile kernel's.
struct RingOrderRealignArgs {
    const char* src[kMaxRanks];
    char* dst[kMaxRanks];
    ChainChunk ch[kMaxRanks];
    uint64_t group0[kMaxRanks + 1];
    uint64_t rest0[kMaxRanks + 1];       // in tiles of 64 vectors
    uint8_t shift[kMaxRanks][kMaxRanks];  // [c][r]: bytes from chunk c's body to output r's next 128-byte boundary
};

template <class T, int N, int U, bool NT>
__global__ __launch_bounds__(64) void k_ring_order_allreduce_realigned(RingOrderRealignArgs a)
{
    constexpr uint64_t W = 64;
    constexpr uint64_t E = T::ESZ;
    constexpr uint64_t X = 8;
    __shared__ u32x4 sum[U * W + X];
    const uint64_t lane = threadIdx.x;
    const char* in[N];
    char* out[N];
    uint32_t sh[N];

    // The chunk's rank rotation, offsets and shifts are reloaded only when a
    // wave's next group lies in another chunk.
    int cur = -1;
    uint64_t body = 0, first = 0;
    for (uint64_t g = blockIdx.x; g < a.group0[N]; g += gridDim.x) {
        const int c = __builtin_amdgcn_readfirstlane(range_of<N>(g, a.group0));
        if (c != cur) {
            cur = c;
            body = (a.ch[c].off + a.ch[c].g.head) * E;
            first = a.group0[c];
#pragma unroll
            for (int t = 0; t < N; t++) {
                in[t] = a.src[(c + t) % N];
                sh[t] = a.shift[c][t];
            }
        }
        const uint64_t v0 = (g - first) * U * W;
        u32x4 x[U + 1][N];
#pragma unroll
        for (int u = 0; u < U; u++)
#pragma unroll
            for (int t = 0; t < N; t++) x[u][t] = ld16<NT>(in[t] + body + (v0 + u * W + lane) * 16);
#pragma unroll
        for (int t = 0; t < N; t++) x[U][t] = ld16<NT>(in[t] + body + (v0 + U * W + (lane % X)) * 16);
        issue_loads_first();
        // The ring's order: rank c's value, then ranks c+1, ..., c+N-1, each
        // partial rounded to the storage type.
#pragma unroll
        for (int u = 0; u <= U; u++) {
            u32x4 p = x[u][0];
#pragma unroll
            for (int t = 1; t < N; t++) p = add_v<T>(p, x[u][t]);
            if (u < U) sum[u * W + lane] = p;
            else if (lane < X) sum[U * W + lane] = p;
        }
        __syncthreads();
        u32x4 o[N][U];
#pragma unroll
        for (int r = 0; r < N; r++) {
            const uint32_t d = sh[r];
            switch ((d / 4) % 4) {
            case 0: shifted<0, U>(o[r], sum, lane, d); break;
            case 1: shifted<1, U>(o[r], sum, lane, d); break;
            case 2: shifted<2, U>(o[r], sum, lane, d); break;
            default: shifted<3, U>(o[r], sum, lane, d); break;
            }
        }
        issue_loads_first();
#pragma unroll
        for (int r = 0; r < N; r++)
#pragma unroll
            for (int u = 0; u < U; u++)
                st16<NT>(a.dst[r] + body + (v0 + u * W + lane) * 16 + sh[r], o[r][u]);
        __syncthreads();
    }

    for (uint64_t t = blockIdx.x; t < a.rest0[N]; t += gridDim.x) {
        const int c = __builtin_amdgcn_readfirstlane(range_of<N>(t, a.rest0));
        const ChainChunk& k = a.ch[c];
        const uint64_t groups = a.group0[c + 1] - a.group0[c];
        const uint64_t nrest = groups ? X + (k.g.nvb - groups * U * W) : k.g.nvb;
        const uint64_t kk = (t - a.rest0[c]) * W + lane;
        if (kk >= nrest) continue;
        const uint64_t v = (groups == 0 || kk < X) ? kk : groups * U * W + (kk - X);
#pragma unroll
        for (int q = 0; q < N; q++) {
            in[q] = a.src[(c + q) % N];
            out[q] = a.dst[(c + q) % N];
        }
        chain_block<N, false, VecIO<T, NT>>(in, out, (k.off + k.g.head) * E + v * 16);
    }

    // Scalar head and tail elements: one wave per chunk.
    for (uint64_t cw = blockIdx.x; cw < (uint64_t)N; cw += gridDim.x) {
        const int c = __builtin_amdgcn_readfirstlane((int)cw);
        const ChainChunk& k = a.ch[c];
        const uint64_t ns = k.g.head + k.g.tail;
        if (lane >= ns) continue;
#pragma unroll
        for (int q = 0; q < N; q++) {
            in[q] = a.src[(c + q) % N];
            out[q] = a.dst[(c + q) % N];
        }
        for (uint64_t j = lane; j < ns; j += W) {
            const uint64_t col = (j < k.g.head) ? j : k.g.head + k.g.nvb * T::VEC + (j - k.g.head);
            chain_block<N, false, ScalarIO<T>>(in, out, (k.off + col) * E);
        }
    }
}

// Fused reduce-scatter over flat chunks (outer == 1), walked like the
// all-reduce chain: wave-sized tiles of all chunks in address order, so the
// whole grid streams through the inputs together instead of one grid row
// per chunk.  Output c (its own buffer, a.dst[c]) is the fold of chunk c of
// every input.  Scalar head and tail elements of each chunk: one wave per
// chunk.
template <class T, int N, bool NT, class Fold = RankFold, int B = 64>
__global__ __launch_bounds__(B) void k_fused_reduce_scatter_flat(ChainArgs a)
{
    constexpr uint64_t W = 64;
    constexpr uint64_t E = T::ESZ;
    const uint64_t lane = threadIdx.x % W;
    const uint64_t wave = (uint64_t)blockIdx.x * (B / W) + threadIdx.x / W;
    const uint64_t nwaves = (uint64_t)gridDim.x * (B / W);
    const uint64_t ntiles = a.tile0[N];
    int cur = -1;
    uint64_t in_body = 0, out_body = 0, nvb = 0, first = 0;
    char* out = nullptr;
    for (uint64_t t = wave; t < ntiles; t += nwaves) {
        const int c = __builtin_amdgcn_readfirstlane(range_of<N>(t, a.tile0));
        if (c != cur) {
            cur = c;
            in_body = (a.ch[c].off + a.ch[c].g.head) * E;
            out_body = a.ch[c].g.head * E;
            nvb = a.ch[c].g.nvb;
            first = a.tile0[c];
            out = a.dst[c];
        }
        const uint64_t v = (t - first) * W + lane;
        if (v < nvb) {
            u32x4 in[N];
#pragma unroll
            for (int r = 0; r < N; r++) in[r] = ld16<NT>(a.src[r] + in_body + v * 16);
            issue_loads_first();
            st16<NT>(out + out_body + v * 16, Fold::template vec<T, N>(in));
        }
    }
    for (uint64_t cw = wave; cw < (uint64_t)N; cw += nwaves) {
        const int c = __builtin_amdgcn_readfirstlane((int)cw);
        const ChainChunk& k = a.ch[c];
        const uint64_t ns = k.g.head + k.g.tail;
        for (uint64_t j = lane; j < ns; j += W) {
            const uint64_t col = (j < k.g.head) ? j : k.g.head + k.g.nvb * T::VEC + (j - k.g.head);
            typename T::S in[N];
#pragma unroll
            for (int r = 0; r < N; r++) in[r] = load_s<T>(a.src[r] + (k.off + col) * E);
            store_s<T>(a.dst[c] + col * E, Fold::template scalar<T, N>(in));
        }
    }
}

// Reduce-scatter chain: chunk c of every rank ([rows, width] with row stride
// `stride`) is summed in ring order into output c ([rows, width], dense).
// MEM keeps the running partial in output c and reads it back before each
// step's add (the step ring's 3(N-1) accesses per element); !MEM keeps it in
// registers and stores the sum once.
template <int N, bool MEM, class IO>
__device__ __forceinline__ void chain_rs_block(const char* const* in, uint64_t so, char* out)
{
    using V = typename IO::V;
    V x[N];
#pragma unroll
    for (int t = 0; t < N; t++) x[t] = IO::ld_in(in[t] + so);
    issue_loads_first();
    V p = x[0];
#pragma unroll
    for (int t = 1; t < N; t++) {
        if (MEM && t > 1) {
            reload_fence();
            p = IO::ld_part(out);
        }
        p = IO::add(p, x[t]);
        if (MEM && t < N - 1) IO::st_part(out, p);
    }
    IO::st_out(out, p);
}

// Ring reduce-scatter chain over flat chunks: the per-chunk grid of
// k_ring_chain_reduce_scatter replaced by the flat walk of
// k_fused_reduce_scatter_flat.  Chunk c folds the ranks in ring order from
// rank c, as in the per-chunk kernel, so the bits are the same; MEM keeps the
// running partial in output c and reads it back before each step's add.
template <class T, int N, bool MEM, bool NT, int B = 64>
__global__ __launch_bounds__(B) void k_ring_chain_reduce_scatter_flat(ChainArgs a)
{
    constexpr uint64_t W = 64;
    constexpr uint64_t E = T::ESZ;
    const uint64_t lane = threadIdx.x % W;
    const uint64_t wave = (uint64_t)blockIdx.x * (B / W) + threadIdx.x / W;
    const uint64_t nwaves = (uint64_t)gridDim.x * (B / W);
    const uint64_t ntiles = a.tile0[N];
    const char* in[N];
    int cur = -1;
    uint64_t in_body = 0, out_body = 0, nvb = 0, first = 0;
    char* out = nullptr;
    for (uint64_t t = wave; t < ntiles; t += nwaves) {
        const int c = __builtin_amdgcn_readfirstlane(range_of<N>(t, a.tile0));
        if (c != cur) {
            cur = c;
#pragma unroll
            for (int k = 0; k < N; k++) in[k] = a.src[(c + k) % N];
            in_body = (a.ch[c].off + a.ch[c].g.head) * E;
            out_body = a.ch[c].g.head * E;
            nvb = a.ch[c].g.nvb;
            first = a.tile0[c];
            out = a.dst[c];
        }
        const uint64_t v = (t - first) * W + lane;
        if (v < nvb) chain_rs_block<N, MEM, VecIO<T, NT>>(in, in_body + v * 16, out + out_body + v * 16);
    }
    for (uint64_t cw = wave; cw < (uint64_t)N; cw += nwaves) {
        const int c = __builtin_amdgcn_readfirstlane((int)cw);
        const ChainChunk& k = a.ch[c];
        const uint64_t ns = k.g.head + k.g.tail;
        if (lane >= ns) continue;
#pragma unroll
        for (int q = 0; q < N; q++) in[q] = a.src[(c + q) % N];
        for (uint64_t j = lane; j < ns; j += W) {
            const uint64_t col = (j < k.g.head) ? j : k.g.head + k.g.nvb * T::VEC + (j - k.g.head);
            chain_rs_block<N, MEM, ScalarIO<T>>(in, (k.off + col) * E, a.dst[c] + col * E);
        }
    }
}

template <class T, int N, bool MEM, bool NT>
__global__ __launch_bounds__(kBlock) void k_ring_chain_reduce_scatter(ChainArgs a)
{
    const int c = blockIdx.y;
    const ChainChunk& k = a.ch[c];
    const uint64_t tid = (uint64_t)blockIdx.x * kBlock + threadIdx.x;
    const uint64_t nthreads = (uint64_t)gridDim.x * kBlock;
    constexpr uint64_t E = T::ESZ;
    const char* in[N];
#pragma unroll
    for (int t = 0; t < N; t++) in[t] = a.src[(c + t) % N];
    char* out = a.dst[c];
    const uint64_t nv = k.rows * k.g.nvb;
    for (uint64_t v = tid; v < nv; v += nthreads) {
        const uint64_t row = (k.rows == 1) ? 0 : v / k.g.nvb;
        const uint64_t col = (v - row * k.g.nvb) * 16 + k.g.head * E;
        chain_rs_block<N, MEM, VecIO<T, NT>>(in, (k.off + row * k.stride) * E + col, out + row * k.width * E + col);
    }
    const uint64_t ns = k.rows * (k.g.head + k.g.tail);
    uint64_t j = tid;
    if constexpr (!MEM) {
        // Heads, tails and chunks of many narrow rows: a lane takes SU
        // elements per iteration (about 16 loads) and issues their loads
        // before the ring-order folds.
        using IO = ScalarIO<T>;
        constexpr int SU = N >= 16 ? 1 : 16 / N;
        if constexpr (SU > 1) {
            for (; j + (SU - 1) * nthreads < ns; j += SU * nthreads) {
                typename T::S x[SU][N];
                uint64_t od[SU];
#pragma unroll
                for (int u = 0; u < SU; u++) {
                    uint64_t row, col;
                    scalar_slot(j + u * nthreads, k.g, T::VEC, row, col);
                    const uint64_t so = (k.off + row * k.stride + col) * E;
#pragma unroll
                    for (int t = 0; t < N; t++) x[u][t] = IO::ld_in(in[t] + so);
                    od[u] = (row * k.width + col) * E;
                }
                issue_loads_first();
#pragma unroll
                for (int u = 0; u < SU; u++) {
                    typename T::S p = x[u][0];
#pragma unroll
                    for (int t = 1; t < N; t++) p = IO::add(p, x[u][t]);
                    IO::st_out(out + od[u], p);
                }
            }
        }
    }
    for (; j < ns; j += nthreads) {
        uint64_t row, col;
        scalar_slot(j, k.g, T::VEC, row, col);
        chain_rs_block<N, MEM, ScalarIO<T>>(in, (k.off + row * k.stride + col) * E, out + (row * k.width + col) * E);
    }
}

// All-gather chain (memory-faithful relay): slab q (blockIdx.y) is copied
// from input q into output q and output q+1, then read back from output
// q+t-1 and stored in output q+t for t = 2..N-1.  Inputs are [rows, width];
// outputs are [rows, N*width] with slab q at column q*width.
template <int N, class IO>
__device__ __forceinline__ void chain_ag_block(const char* in, char* const* out, uint64_t dof)
{
    const typename IO::V x = IO::ld_in(in);
    IO::st_part(out[0] + dof, x);
    IO::st_part(out[1] + dof, x);
#pragma unroll
    for (int t = 2; t < N; t++) {
        reload_fence();
        IO::st_part(out[t] + dof, IO::ld_part(out[t - 1] + dof));
    }
}

template <class T, int N, bool NT>
__global__ __launch_bounds__(kBlock) void k_ring_chain_all_gather(FusedAgArgs a)
{
    const int q = blockIdx.y;
    const RowSplit& g = a.g[q];
    const uint64_t tid = (uint64_t)blockIdx.x * kBlock + threadIdx.x;
    const uint64_t nthreads = (uint64_t)gridDim.x * kBlock;
    constexpr uint64_t E = T::ESZ;
    const uint64_t s_dst = (uint64_t)N * a.width;
    const uint64_t slab = (uint64_t)q * a.width;
    char* out[N];
#pragma unroll
    for (int t = 0; t < N; t++) out[t] = a.dst[(q + t) % N];
    const uint64_t nv = a.rows * g.nvb;
    for (uint64_t v = tid; v < nv; v += nthreads) {
        const uint64_t row = (a.rows == 1) ? 0 : v / g.nvb;
        const uint64_t col = (v - row * g.nvb) * 16 + g.head * E;
        chain_ag_block<N, VecIO<T, NT>>(a.src[q] + row * a.width * E + col, out, (row * s_dst + slab) * E + col);
    }
    const uint64_t ns = a.rows * (g.head + g.tail);
    for (uint64_t j = tid; j < ns; j += nthreads) {
        uint64_t row, col;
        scalar_slot(j, g, T::VEC, row, col);
        chain_ag_block<N, ScalarIO<T>>(a.src[q] + (row * a.width + col) * E, out, (row * s_dst + slab + col) * E);
    }
}

}  // namespace vrc
