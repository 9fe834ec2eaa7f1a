// vrc_host.hpp -- host-side pieces shared by the library's translation units:
// the launch-plan recorder, the launch-shape policy, the chunk partition and
// the alignment split.  Internal to libvrc.so; the C ABI is include/vrc.h.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>
#include <type_traits>

#include "vrc.h"
#include "vrc_kernels.hpp"

namespace vrc {
namespace host {


using vrc::kBlock;
using vrc::kMaxRanks;
using vrc::RowSplit;

extern thread_local int g_last_hip_error;

// When set (by vrc_plan on this thread), launches are recorded here instead
// of being enqueued.
struct Plan {
    vrc_op_desc* ops;
    int cap;
    int n;
    int launches;
};
extern thread_local Plan* g_plan;

inline void plan_op(const vrc_op_desc& op)
{
    if (g_plan->n < g_plan->cap) g_plan->ops[g_plan->n] = op;
    g_plan->n++;
}

// A single-launch kernel: one entry with its kind, size and launch geometry.
inline vrc_status_t plan_single(vrc_op_kind_t kind, uint64_t count, dim3 grid, int block, int vectors)
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
inline int env_int(const char* name, int dflt, int lo, int hi)
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
//    DRAM rows; fused all-gather: 32 per CU with one store in flight per
//    wave up to 2 GiB written, 16 per CU above (ag_shape);
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
    int realign;              // 1: outputs on different 128-byte offsets take the realigned fused kernel; 0: never
    int phased;               // 1: large fused all-reduces take the phased kernel (phased_phases); 0: never
    int phase_wait;           // 1: the phased kernel's workgroups meet between phases; 0: they never wait
    int phase_skew;           // 1: odd workgroups of the phased kernel hold fewer sums (phased_skew); 0: all hold K
    int ag_throttle;          // -1: size policy (ag_shape); 1: the fused all-gather keeps one store in flight per wave; 0: never
};

inline const Tuning& tuning()
{
    static const Tuning t = {env_int("VRC_FUSED_BLOCKS_PER_CU", 0, 1, 64),
                             env_int("VRC_STEP_BLOCKS_PER_CU", 0, 1, 64),
                             env_int("VRC_CHAIN_BLOCKS_PER_CU", 0, 1, 64), env_int("VRC_UNROLL", 0, 1, 8),
                             env_int("VRC_STEP_NT", -1, 0, 2), env_int("VRC_STEP_UNROLL", 0, 1, 2),
                             env_int("VRC_FUSED_BLOCK", 0, 64, 256), env_int("VRC_CHAIN_BLOCK", 0, 64, 256),
                             env_int("VRC_STEP_BLOCK", 0, 64, 256), env_int("VRC_REALIGN", 1, 0, 1),
                             env_int("VRC_PHASED", 1, 0, 1), env_int("VRC_PHASE_WAIT", 1, 0, 1),
                             env_int("VRC_PHASE_SKEW", 1, 0, 1), env_int("VRC_AG_THROTTLE", -1, 0, 1)};
    return t;
}

constexpr uint64_t kMiB = 1ull << 20;
constexpr uint64_t kGiB = 1ull << 30;

// Two ranks keep only a quarter of the eight-rank loads in flight per lane,
// so at 2 ranks the large-size grid doubles (8 GiB moved: 1.64-1.70 ms
// against 1.78-1.80 ms at one workgroup per CU; 4 and 16 ranks are best at one).
inline int fused_blocks_per_cu(uint64_t bytes_moved, int n)
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
// handed to the 8 XCDs in turn, so consecutive wave tiles of every buffer go
// to different XCDs.  A wave takes U consecutive 1 KiB tiles per iteration
// (all U * N loads in flight, then the U folds and U * N stores back to
// back).  The grid keeps 16-48 KiB of loads in flight per CU (workgroups per
// CU x ranks x U): more outstanding requests made the mixed read/write stream
// slower, not faster.  Shapes measured on MI355X, bf16, 8 GiB moved, all
// shapes in one process on the same buffers, interleaved over four rounds,
// three runs (time relative to the previous policy, U vectors one grid stride
// apart at 3-4 ranks and U = 1 otherwise, at the largest power of two <= 8
// per CU with workgroups x N x U <= 32):
//   2 ranks: U 8, 2 per CU 0.91-0.92 (U 4 or 2 at 4 per CU 0.92-0.93);
//   3 ranks: U 4, 2 per CU 0.97-0.98;   4 ranks: U 8, 1 per CU 0.92;
//   5 ranks: U 2, 2 per CU 0.97-0.98;   8 ranks: U 1 at 2 or 4 per CU within
//   2 % (4 kept), every U > 1 2-4 % slower;  12 and 16 ranks: U 1, 2 per CU
//   (U 2 or 4 per CU 1-7 % slower at 16).
// Outputs that do not all share the vector grid (write_ref) split a 64-byte
// write block at each tile edge; with consecutive tiles a wave fills those
// blocks itself, back to back, and the cache merges them.  Those calls take
// the largest U <= 8 with U x N <= 32 at 64 / (U x N) per CU.  8 ranks with
// inputs and outputs on offsets 2r bytes (ms; aligned U 1 at 4 per CU:
// 1.532): rank fold U 4 at 2 per CU 1.781, U 2 at 2 per CU 1.798, U 4 at 1
// per CU 1.814, U 1 at 4 per CU 2.017; the butterfly fold 1.770, 1.819, 2.743
// and 2.021 (with one wave per CU it turns ALU-bound).  Calls with no
// output in place take the realigned kernels instead (realign_unroll, the
// same U and workgroups per CU; 8 ranks, every operand on its own offset,
// against the aligned call: rank fold 1.05-1.09x at 2 per CU, 1.12x at 4,
// 1.14x at 3; butterfly 1.05-1.09x; ring order 1.10x); this shape remains
// for in-place calls.
// Below 64 MiB moved a call is launch-bound and keeps 256-lane workgroups,
// 8 per CU, two vectors per rank one grid stride apart.
struct FusedShape {
    int block;
    int blocks_per_cu;
    int unroll;
};

inline FusedShape fused_ar_shape(uint64_t bytes_moved, int n, bool outputs_share_grid)
{
    FusedShape s = {kBlock, 8, 2};
    if (bytes_moved >= 64 * kMiB) {
        s.block = 64;
        if (!outputs_share_grid) {
            s.unroll = 8;
            while (s.unroll > 1 && s.unroll * n > 32) s.unroll /= 2;
            s.blocks_per_cu = 1;
            while (2 * s.blocks_per_cu * s.unroll * n <= 64) s.blocks_per_cu *= 2;
        } else if (n == 2) {
            s = {64, 2, 8};
        } else if (n == 3) {
            s = {64, 2, 4};
        } else if (n == 4) {
            s = {64, 1, 8};
        } else if (n <= 7) {
            s = {64, 2, 2};
        } else if (n == 8) {
            s = {64, 4, 1};
        } else {
            s = {64, 2, 1};
        }
    }
    if (tuning().fused_blocks_per_cu) s.blocks_per_cu = tuning().fused_blocks_per_cu;
    if (tuning().fused_block) s.block = tuning().fused_block == 64 ? 64 : kBlock;
    if (tuning().unroll) s.unroll = tuning().unroll;
    // One-wave kernels exist for U = 1, 2, 4 and 8 with U x N <= 32 (a lane's
    // loads stay in registers); 256-lane ones for U = 1 and 2.
    const int umax = s.block == 64 ? 8 : 2;
    int u = 1;
    while (2 * u <= s.unroll && 2 * u <= umax && (s.block != 64 || 2 * u * n <= 32)) u *= 2;
    s.unroll = u;
    return s;
}

// Vectors per rank per lane of the realigned fused all-reduce, one kernel
// per rank count: the largest U <= 8 with U x N <= 32, at least 2 (a group
// of U tiles re-reads 128 bytes of the next group, 1/(8U) of its reads).
constexpr int realign_unroll(int n) { return 8 * n <= 32 ? 8 : (4 * n <= 32 ? 4 : 2); }

// The phased fused all-reduce (k_fused_allreduce_phased): sums held per lane
// between a phase's reads and its writes, in registers (64 up to 8 ranks;
// 32 above, where the N loads in flight need the room) and in LDS (32:
// 128 KiB per workgroup).  The butterfly of 16-bit types rounds every
// partial and keeps more values live: 32 and 16.  More would spill to
// memory (the compiler then stops using the AGPRs).
constexpr int phased_regs(int n, bool narrow_butterfly = false)
{
    return narrow_butterfly ? (n <= 8 ? 32 : 16) : (n <= 8 ? 64 : 32);
}
constexpr int kPhasedLds = 32;

// The phased ring-order all-reduce rounds every partial like the butterfly;
// its per-slot chunk lookup and rank rotation add code to every slot, and
// past a size the compiler stops unrolling the slot loop, which leaves the
// register sums in scratch memory.  Sums in registers: per element type and
// rank count, a count that compiles without scratch (from a sweep over
// 16-64, less where the 160 KiB of LDS sums below pushed a kernel past 512
// registers); 40 more per lane (160 KiB per workgroup) in LDS.
template <class T>
constexpr int ring_order_phased_regs(int n)
{
    if constexpr (std::is_same<T, BF16>::value) return n <= 7 ? 32 : n <= 9 ? 24 : n <= 14 ? 16 : 0;
    if constexpr (std::is_same<T, F16>::value) return n <= 8 ? 40 : n <= 11 ? 32 : n <= 15 ? 24 : 16;
    return 40;
}
constexpr int kRingOrderPhasedLds = 40;

// LDS sums fewer per lane for the odd workgroups of the phased ring-order
// kernel, as phased_skew for the fused one.
inline int ring_order_phased_skew(int cus) { return tuning().phase_skew && cus % 8 == 0 ? 8 : 0; }

// LDS sums fewer per lane for the odd workgroups of the phased kernel (0:
// every workgroup holds K).  On MI355X the workgroups of odd index (odd XCDs)
// issued a phase's stores in 125-151 us where the even ones took 97-109 us
// (8 x 512 MiB bf16, per-workgroup wall-clock timelines), and every phase
// waited for the slowest.  Measured against no skew in one process on the
// same buffers, bf16, over six runs: at 8 ranks (96 sums per lane) 16 fewer
// gave +2.0-2.5 % (8 fewer +0.8 %, 24 fewer was slower); at 6, 12 and 16 ranks
// 8 fewer gave +1.4-2 %; the even workgroups lighter instead was 3-4 % slower.
// It needs a grid of whole XCD rounds (a multiple of 8 workgroups).
inline int phased_skew(int n, int cus, bool narrow_butterfly = false)
{
    if (!tuning().phase_skew || cus % 8 != 0) return 0;
    return n == 8 && !narrow_butterfly ? 16 : 8;
}

// Vectors per rank that one phase of the phased kernel covers.
inline uint64_t phased_vectors(int n, int cus, bool narrow_butterfly = false)
{
    const uint64_t lanes = (uint64_t)cus * kBlock;
    const uint64_t k = (uint64_t)(phased_regs(n, narrow_butterfly) + kPhasedLds);
    const uint64_t skew = (uint64_t)phased_skew(n, cus, narrow_butterfly);
    return (k - skew) * lanes + skew * (lanes / 2);
}

// Whole phases of the phased kernel for `nvb` vectors per rank, or 0 where
// the one-wave kernel stays.  A phase reads N x 256 lanes per CU x K
// vectors (less the skew above): 576 MiB at 6 ranks, 768 MiB at 8, 1 GiB at
// 16 on 256 CUs (the 16-bit butterfly: 512 MiB at 8, 768 MiB at 16).  It
// runs from 6 ranks and at least 3 whole phases.  Measured on MI355X against
// the one-wave kernel, bf16, bit-identical outputs (time ratio, one process,
// four interleaved rounds, before the skew): 8 x 512 MiB 0.946-0.963,
// 8 x 1 GiB 0.935, 12 x 341 MiB 0.860, 6 x 682 MiB 0.954, 16 x 256 MiB 0.973;
// and where it is not taken, 8 x 256 MiB 0.969 (2 phases), 8 x 128 MiB 1.003
// (1), 16 x 128 MiB 1.008 (2), 4 x 512 MiB 1.030 (384 MiB phases).
inline uint64_t phased_phases(int n, uint64_t nvb, int cus, bool narrow_butterfly = false)
{
    if (!tuning().phased || n < 6) return 0;
    const uint64_t p = nvb / phased_vectors(n, cus, narrow_butterfly);
    return p >= 3 ? p : 0;
}

// Workgroups per CU of the realigned fused all-reduce: 64 / (U x N) rounded
// down to a power of two, at least 1.
inline int realign_blocks_per_cu(int n)
{
    if (tuning().fused_blocks_per_cu) return tuning().fused_blocks_per_cu;
    int b = 1;
    while (2 * b * realign_unroll(n) * n <= 64) b *= 2;
    return b;
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
// Adds of up to 7 operations of >= 48 MiB run one-wave workgroups, 8 per CU,
// one vector per lane.  One process, same buffers, one reduce-scatter add
// step (GB/s; 256 lanes at 4 per CU -> one wave at 8 per CU): 2 x 2 GiB
// 5,473 -> 5,804; 4 x 1 GiB 5,456 -> 5,779.  The copy steps lost with one
// wave (2 x 2 GiB 5,477 -> 5,051; 4 x 1 GiB 5,740 -> 4,431) and keep 256
// lanes; at 8 and 16 ranks neither kind gained reliably.
struct StepShape {
    int blocks_per_cu;
    int unroll;
    int block;  // lanes per workgroup; 64 implies unroll 1
};

inline StepShape step_shape(uint64_t bytes_moved, int nops, bool add)
{
    StepShape s = {8, 1, kBlock};
    const uint64_t per_op = bytes_moved / (uint64_t)(nops > 0 ? nops : 1);
    if (bytes_moved >= kGiB / 16) {
        if (nops <= 7 && per_op >= 48 * kMiB) s = add ? StepShape{8, 1, 64} : StepShape{4, 1, kBlock};
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
inline bool step_nontemporal(bool add, uint64_t bytes_moved)
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
inline int fused_rs_flat_blocks_per_cu(int n)
{
    if (tuning().fused_blocks_per_cu) return tuning().fused_blocks_per_cu;
    return n <= 4 ? 8 : 4;
}

// The memory-faithful reduce-scatter chain over flat chunks (one-wave
// workgroups): its lanes wait on their own stores at every step, so like the
// all-reduce chain it keeps more waves resident.
inline int chain_rs_flat_blocks_per_cu()
{
    if (tuning().chain_blocks_per_cu) return tuning().chain_blocks_per_cu;
    return 16;
}

// The fused all-gather reads each input once and stores it N times.  Up to
// 2 GiB written, each wave keeps one store in flight (it waits for the
// previous store before the next) and the grid has 32 workgroups per CU;
// above that, stores go back to back at 16 per CU.  Measured on MI355X,
// fp16, each call after a cache-evicting write (us; back to back at 16 per
// CU / one store in flight at 32 per CU, three processes each): 8 x 5 MiB
// heads 74.4-75.0 / 71.1-71.7 (in one process on the same buffers
// 75.8-76.0 / 69.6-71.0), 8 x 1 MiB 17.0-17.2 / 15.3-15.7, 4 x 5 MiB
// 23.1-23.8 / 21.9-22.2, 16 x 5 MiB (1.25 GiB written) 300-302 / 288-289,
// 4 x 64 MiB 265-282 / 254-265, 2 x 256 MiB 310-312 / 307-310, 8 x 16 MiB
// 235-237 / 235-236; and at 4 GiB written and more 8 x 64 MiB 953-957 /
// 954-958, 16 x 16 MiB 924-928 / 936-940, 8 x 128 MiB 1,890-1,892 /
// 1,915-1,918.  Back to back, more workgroups were slower (the heads at 32
// per CU: 77.6-84.5 us).
struct AgShape {
    int blocks_per_cu;
    bool one_store_in_flight;
};

inline AgShape ag_shape(uint64_t bytes_written)
{
    const bool throttle = tuning().ag_throttle >= 0 ? tuning().ag_throttle != 0 : bytes_written <= 2 * kGiB;
    const int bpc = tuning().fused_blocks_per_cu ? tuning().fused_blocks_per_cu : (throttle ? 32 : 16);
    return {bpc, throttle};
}

// Memory-faithful chains wait on their own stores between steps, so they
// need more resident waves than the fused loop to hide latency.  This shape
// serves the single-launch reduce-scatter and all-gather relays (256-lane
// workgroups).
inline int chain_blocks_per_cu(uint64_t bytes_moved)
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

inline ChainShape chain_ar_shape(bool mem, int n)
{
    ChainShape s = {64, mem ? 16 : (n <= 2 ? 8 : 4)};
    if (mem && tuning().chain_blocks_per_cu) s.blocks_per_cu = tuning().chain_blocks_per_cu;
    if (!mem && tuning().fused_blocks_per_cu) s.blocks_per_cu = tuning().fused_blocks_per_cu;
    if (tuning().chain_block) s.block = tuning().chain_block == 256 ? kBlock : 64;
    return s;
}

#define VRC_FOR_N(X) X(2) X(3) X(4) X(5) X(6) X(7) X(8) X(9) X(10) X(11) X(12) X(13) X(14) X(15) X(16)

// Grid x for `ops` operations of at most `work` lane-items each, capped at
// blocks_per_cu workgroups per CU over the whole grid.
inline unsigned grid_x(int cus, uint64_t work, int ops, int blocks_per_cu, int block = kBlock)
{
    const uint64_t want = (work + block - 1) / block;
    uint64_t cap = (uint64_t)cus * (uint64_t)blocks_per_cu / (uint64_t)(ops > 0 ? ops : 1);
    if (cap < 1) cap = 1;
    uint64_t g = want < cap ? want : cap;
    if (g < 1) g = 1;
    if (g > 0x7fffffffull) g = 0x7fffffffull;
    return (unsigned)g;
}

inline vrc_status_t check_launch()
{
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        g_last_hip_error = (int)e;
        return VRC_ERR_HIP;
    }
    return VRC_OK;
}

inline vrc_status_t hip_fail(hipError_t e)
{
    g_last_hip_error = (int)e;
    return VRC_ERR_HIP;
}

// ----------------------------------------------------------------------------
// Element sizes, chunking, alignment split
// ----------------------------------------------------------------------------
inline int esize(vrc_dtype_t dt)
{
    switch (dt) {
    case VRC_INT32: return 4;
    case VRC_FP32: return 4;
    case VRC_FP16: return 2;
    case VRC_BF16: return 2;
    }
    return 0;
}

inline int mod(int a, int n) { return ((a % n) + n) % n; }

// Flat chunk c of `count` elements over n ranks: equal chunks of count/n,
// the last one takes the remainder.
inline void chunk_range(uint64_t count, int n, int c, uint64_t* off, uint64_t* len)
{
    const uint64_t base = count / (uint64_t)n;
    *off = (uint64_t)c * base;
    *len = (c == n - 1) ? count - base * (uint64_t)(n - 1) : base;
}

// Alignment of a region's 16-byte vector grid.  Reads leave L2 as 128-byte
// requests and writes as 64-byte ones; a wave whose 1 KiB run of stores is off
// that grid splits a write block with the neighbouring wave (usually on
// another XCD), and the block reaches memory as two partial writes.  Measured
// on MI355X (8 x 512 MiB fused bf16 all-reduce, one process): outputs 16
// bytes off a 64-byte boundary 1.91 ms against 1.53 ms; the L2-to-memory
// counters show one extra 32-byte write per 1 KiB run and output.  Inputs off
// the grid cost one extra 128-byte read per run (+8 %).
constexpr uintptr_t kGridAlign = 128;

// Split rows of `width` elements into a scalar head, 16-byte vectors and a
// scalar tail.  Every operand's vectors are read and written with 16-byte
// accesses whatever its offset (unaligned access mode).  The head puts the
// reference operand `ref` -- the region's destination -- on a 128-byte
// boundary, so its vector stores fill whole write blocks; it holds at most
// 127 bytes, and the tail less than one vector.  A `ref` that is not a
// multiple of the element size gets no head.  With more than one row the head
// is the first row's: rows whose stride is not a multiple of 128 bytes run
// their vectors off the grid, which costs bandwidth but not correctness.
inline RowSplit split_rows(uintptr_t ref, uint64_t width, int esz)
{
    uint64_t head = 0;
    if (ref % (uintptr_t)esz == 0) head = ((kGridAlign - ref % kGridAlign) % kGridAlign) / (uint64_t)esz;
    if (head > width) head = width;
    const uint64_t vec = 16u / (uint64_t)esz;
    RowSplit g;
    g.head = head;
    g.nvb = (width - head) / vec;
    g.tail = width - head - g.nvb * vec;
    return g;
}

// The reference for a region with several destinations: the address whose
// offset modulo 128 bytes the most of them share (the first such address on
// a tie).  Destinations on that grid store whole blocks; the others pay the
// split blocks.
inline uintptr_t write_ref(const uintptr_t* addr, int n)
{
    int best = 0, best_count = 0;
    for (int i = 0; i < n; i++) {
        int c = 0;
        for (int j = 0; j < n; j++) c += (addr[j] % kGridAlign) == (addr[i] % kGridAlign);
        if (c > best_count) {
            best = i;
            best_count = c;
        }
    }
    return addr[best];
}

enum class Coll { AR, RS, AG };

// One collective for one element type; defined in vrc_launch.hpp and
// instantiated once per type (vrc_type_*.hip).
template <class T>
vrc_status_t run_typed(Coll coll, vrc_mode_t mode, const char* const* x, char* const* y, int n, uint64_t count,
                       uint64_t outer, int cus, hipStream_t st);

}  // namespace host
}  // namespace vrc
