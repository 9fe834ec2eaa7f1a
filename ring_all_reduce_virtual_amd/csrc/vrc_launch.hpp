// vrc_launch.hpp -- typed launchers: the ring schedule, the fused,
// single-launch and halving-doubling families, and the launch sizing of each
// kernel, for one element type T.  Included by one translation unit per type.
#pragma once

#include <type_traits>

#include "vrc_host.hpp"

namespace vrc {
namespace host {

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
        const StepShape shape = step_shape(bytes, nops, ADD);
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
        op.g = split_rows((uintptr_t)d, width, E);
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
        // One-wave workgroups take U consecutive tiles; U * N <= 32 (fused_ar_shape clamps it) keeps a
        // lane's loads in registers, and no other U is instantiated.
        constexpr int U8 = 8 * N <= 32 ? 8 : 1, U4 = 4 * N <= 32 ? 4 : 1;
        if (sh.block == 64) {
            if (sh.unroll == 8)
                hipLaunchKernelGGL((vrc::k_fused_allreduce<T, N, U8, true, Fold, 64>), grid, dim3(64), 0, st, a);
            else if (sh.unroll == 4)
                hipLaunchKernelGGL((vrc::k_fused_allreduce<T, N, U4, true, Fold, 64>), grid, dim3(64), 0, st, a);
            else if (sh.unroll == 2)
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

    // The fused all-reduce with each output stored on its own 128-byte grid
    // (groups >= 1 groups of realign_unroll(n) tiles, no output in place).
    template <class Fold>
    static vrc_status_t fused_allreduce_realigned(const vrc::FusedArArgs& f, int n, uint64_t count, uint64_t groups,
                                                  int cus, hipStream_t st)
    {
        constexpr bool butterfly = std::is_same<Fold, vrc::Butterfly>::value;
        vrc::FusedRealignArgs a = {};
        for (int r = 0; r < kMaxRanks; r++) {
            a.src[r] = f.src[r];
            a.dst[r] = f.dst[r];
        }
        a.g = f.g;
        a.groups = groups;
        const uintptr_t body = f.g.head * E;
        for (int r = 0; r < n; r++)
            a.shift[r] = (uint32_t)((kGridAlign - ((uintptr_t)f.dst[r] + body) % kGridAlign) % kGridAlign);
        const int U = realign_unroll(n);
        const dim3 grid(grid_x(cus, groups * 64, 1, realign_blocks_per_cu(n), 64));
        if (g_plan)
            return plan_single(butterfly ? VRC_OP_BUTTERFLY_ALLREDUCE_REALIGNED : VRC_OP_FUSED_ALLREDUCE_REALIGNED,
                               count, grid, 64, U);
#define VRC_REALIGNED(K)                                                                                           \
    hipLaunchKernelGGL((vrc::k_fused_allreduce_realigned<T, K, realign_unroll(K), true, Fold>), grid, dim3(64), 0, \
                       st, a)
        if constexpr (butterfly) {
            switch (n) {
            case 2: VRC_REALIGNED(2); break;
            case 4: VRC_REALIGNED(4); break;
            case 8: VRC_REALIGNED(8); break;
            case 16: VRC_REALIGNED(16); break;
            default: return VRC_ERR_INVALID_ARG;
            }
        } else {
            switch (n) {
#define VRC_CASE(K) \
    case K: VRC_REALIGNED(K); break;
                VRC_FOR_N(VRC_CASE)
#undef VRC_CASE
            default: return VRC_ERR_INVALID_ARG;
            }
        }
#undef VRC_REALIGNED
        return check_launch();
    }

    // The phased fused all-reduce: one 256-lane workgroup per CU, `phases`
    // whole phases (phased_phases), then the rest of the vectors and the
    // scalar head and tail.
    template <class Fold>
    static vrc_status_t fused_allreduce_phased(const vrc::FusedArArgs& a, int n, uint64_t count, uint64_t phases,
                                               int cus, hipStream_t st)
    {
        constexpr bool butterfly = std::is_same<Fold, vrc::Butterfly>::value;
        constexpr bool nb = butterfly && T::ESZ == 2;
        const dim3 grid((unsigned)cus);
        if (g_plan)
            return plan_single(butterfly ? VRC_OP_BUTTERFLY_ALLREDUCE_PHASED : VRC_OP_FUSED_ALLREDUCE_PHASED, count,
                               grid, kBlock, phased_regs(n, nb) + kPhasedLds);
        const uint32_t wait = (uint32_t)tuning().phase_wait;
        const uint32_t skew = (uint32_t)phased_skew(n, cus, nb);
#define VRC_PHASED(K)                                                                                                 \
    hipLaunchKernelGGL((vrc::k_fused_allreduce_phased<T, K, phased_regs(K, nb), kPhasedLds, true, Fold>), grid,    \
                       dim3(kBlock), 0, st, a, phases, wait, skew)
        if constexpr (butterfly) {
            switch (n) {
            case 8: VRC_PHASED(8); break;
            case 16: VRC_PHASED(16); break;
            default: return VRC_ERR_INVALID_ARG;
            }
        } else {
            switch (n) {
#define VRC_CASE(K) \
    case K: VRC_PHASED(K); break;
                VRC_CASE(6) VRC_CASE(7) VRC_CASE(8) VRC_CASE(9) VRC_CASE(10) VRC_CASE(11) VRC_CASE(12) VRC_CASE(13)
                VRC_CASE(14) VRC_CASE(15) VRC_CASE(16)
#undef VRC_CASE
            default: return VRC_ERR_INVALID_ARG;
            }
        }
#undef VRC_PHASED
        return check_launch();
    }

    template <class Fold = vrc::RankFold>
    static vrc_status_t fused_allreduce(const char* const* x, char* const* y, int n, uint64_t count, int cus,
                                        hipStream_t st)
    {
        if (n == 1) return x[0] == y[0] ? VRC_OK : copy(x[0], y[0], 1, count, 0, 0, cus, st);
        vrc::FusedArArgs a;
        uintptr_t out[kMaxRanks];
        for (int r = 0; r < n; r++) {
            a.src[r] = x[r];
            a.dst[r] = y[r];
            out[r] = (uintptr_t)y[r];
        }
        for (int r = n; r < kMaxRanks; r++) {
            a.src[r] = nullptr;
            a.dst[r] = nullptr;
        }
        a.count = count;
        const uintptr_t ref = write_ref(out, n);
        a.g = split_rows(ref, count, E);
        bool share = true;  // every output on the vector grid
        for (int r = 0; r < n; r++)
            if (out[r] % kGridAlign != ref % kGridAlign) share = false;
        if (share) {
            // Every output on one 128-byte grid: large calls read and write in
            // phases (the butterfly needs a power of two: 8 or 16 ranks here).
            constexpr bool butterfly = std::is_same<Fold, vrc::Butterfly>::value;
            const bool fold_ok = !butterfly || n == 8 || n == 16;
            const uint64_t phases = fold_ok ? phased_phases(n, a.g.nvb, cus, butterfly && T::ESZ == 2) : 0;
            if (phases) return fused_allreduce_phased<Fold>(a, n, count, phases, cus, st);
        }
        const uint64_t work = a.g.nvb > a.g.head + a.g.tail ? a.g.nvb : a.g.head + a.g.tail;
        const FusedShape sh = fused_ar_shape(2 * (uint64_t)n * count * E, n, share);
        if (!share && sh.block == 64 && tuning().realign) {
            // Outputs on different 128-byte offsets: store each on its own
            // grid, unless an output is its input (the realigned stores run
            // up to 127 bytes ahead of the reads).
            bool in_place = false;
            for (int r = 0; r < n; r++) in_place = in_place || x[r] == y[r];
            const uint64_t gv = (uint64_t)realign_unroll(n) * 64;
            const uint64_t groups = a.g.nvb >= gv + 8 ? (a.g.nvb - 8) / gv : 0;
            if (!in_place && groups > 0) return fused_allreduce_realigned<Fold>(a, n, count, groups, cus, st);
        }
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
    // and ring-order reduce-scatters.  Chunk c's vectors sit on output c's
    // 128-byte grid, so only its head (at most 127 bytes) and tail (less than
    // one vector) run scalar, one wave per chunk.  Fills the chunk table and
    // grid.
    static void rs_flat_layout(const char* const* x, char* const* y, int n, uint64_t count, int cus,
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
            a.ch[c] = {off, 1, len, 0, split_rows((uintptr_t)y[c], len, E)};
            a.tile0[c + 1] = a.tile0[c] + (a.ch[c].g.nvb + 63) / 64;
        }
        // At least one wave per chunk for the scalar head/tail pass.
        const uint64_t lanes = a.tile0[n] * 64, scalar_lanes = (uint64_t)n * 64;
        const uint64_t work = lanes > scalar_lanes ? lanes : scalar_lanes;
        *grid = dim3(grid_x(cus, work, 1, fused_rs_flat_blocks_per_cu(n), 64));
    }

    template <class Fold>
    static vrc_status_t fused_reduce_scatter_flat(const char* const* x, char* const* y, int n, uint64_t count,
                                                  int cus, hipStream_t st)
    {
        vrc::ChainArgs a;
        dim3 grid;
        rs_flat_layout(x, y, n, count, cus, &a, &grid);
        if (g_plan)
            return plan_single(std::is_same<Fold, vrc::Butterfly>::value ? VRC_OP_BUTTERFLY_REDUCE_SCATTER
                                                                          : VRC_OP_FUSED_REDUCE_SCATTER,
                               count, grid, 64, 1);
        if constexpr (std::is_same<Fold, vrc::Butterfly>::value) {
            switch (n) {
            case 2: launch_fused_rs_flat_n<2, Fold>(a, grid, st); break;
            case 4: launch_fused_rs_flat_n<4, Fold>(a, grid, st); break;
            case 8: launch_fused_rs_flat_n<8, Fold>(a, grid, st); break;
            case 16: launch_fused_rs_flat_n<16, Fold>(a, grid, st); break;
            default: return VRC_ERR_INVALID_ARG;
            }
        } else {
            switch (n) {
#define VRC_CASE(K) \
    case K: launch_fused_rs_flat_n<K, Fold>(a, grid, st); break;
                VRC_FOR_N(VRC_CASE)
#undef VRC_CASE
            default: return VRC_ERR_INVALID_ARG;
            }
        }
        return check_launch();
    }

    template <class Fold = vrc::RankFold>
    static vrc_status_t fused_reduce_scatter(const char* const* x, char* const* y, int n, uint64_t count,
                                             uint64_t outer, int cus, hipStream_t st)
    {
        if (n == 1) return copy(x[0], y[0], 1, count, 0, 0, cus, st);
        if (outer == 1 && (uint64_t)(n + 1) * count * E >= 64 * kMiB)
            return fused_reduce_scatter_flat<Fold>(x, y, n, count, cus, st);
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
            ch.g = split_rows((uintptr_t)y[c], k.width, E);
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
            uintptr_t out[kMaxRanks];
            for (int r = 0; r < n; r++) out[r] = (uintptr_t)(y[r] + (uint64_t)q * row * E);
            a.g[q] = split_rows(write_ref(out, n), row, E);
            const uint64_t w = outer * (a.g[q].nvb + a.g[q].head + a.g[q].tail);
            if (w > work) work = w;
        }
        const AgShape sh = ag_shape((uint64_t)n * n * count * E);
        const dim3 grid(grid_x(cus, work, n, sh.blocks_per_cu), (unsigned)n);
        if (g_plan) return plan_single(VRC_OP_FUSED_ALL_GATHER, count, grid, kBlock, 1);
        if (sh.one_store_in_flight)
            hipLaunchKernelGGL((vrc::k_fused_all_gather<T, true, true>), grid, dim3(kBlock), 0, st, a);
        else
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

    // ---- binomial-tree all-gather -----------------------------------------
    // Gather to rank 0, then broadcast from it (the textbook binomial tree;
    // Thakur, Rabenseifner and Gropp 2005).  Gather distance d = 1, 2, 4, ...
    // (< N): rank r with r mod 2d == 0 copies the slabs rank r + d holds,
    // [r + d, hi[r + d]), into the same columns of its output.  The d = 1
    // launch also places every receiving rank's own slab and reads the
    // sending ranks' slabs straight from their inputs.  Broadcast distances run
    // in reverse: rank r with r mod 2d == 0 copies its whole output to rank
    // r + d.  2 ceil(log2 N) launches; a launch writes only ranks that none of
    // its operations reads.
    static vrc_status_t tree_all_gather(const char* const* x, char* const* y, int n, uint64_t count,
                                        uint64_t outer, int cus, hipStream_t st)
    {
        const uint64_t row = count / outer, sy = (uint64_t)n * row;
        if (n == 1) return copy(x[0], y[0], 1, count, 0, 0, cus, st);
        int hi[kMaxRanks];
        for (int r = 0; r < n; r++) hi[r] = r + 1;
        vrc::StepArgs args;
        for (int d = 1; d < n; d *= 2) {
            int nops = 0;
            uint64_t work = 0;
            for (int r = 0; r < n; r += 2 * d) {
                if (d == 1) args.op[nops++] = make_op(x[r], nullptr, y[r] + (uint64_t)r * row * E, outer, row, row, 0, sy);
                if (r + d < n) {
                    const int p = r + d;
                    const uint64_t off = (uint64_t)p * row * E, width = (uint64_t)(hi[p] - p) * row;
                    args.op[nops++] = d == 1 ? make_op(x[p], nullptr, y[r] + off, outer, row, row, 0, sy)
                                             : make_op(y[p] + off, nullptr, y[r] + off, outer, width, sy, 0, sy);
                    hi[r] = hi[p];
                }
            }
            for (int i = 0; i < nops; i++)
                if (op_work(args.op[i]) > work) work = op_work(args.op[i]);
            vrc_status_t rc = step<false>(args, nops, work, cus, st);
            if (rc) return rc;
        }
        int top = 1;
        while (2 * top < n) top *= 2;
        for (int d = top; d >= 1; d /= 2) {
            int nops = 0;
            for (int r = 0; r + d < n; r += 2 * d)
                args.op[nops++] = make_op(y[r], nullptr, y[r + d], 1, (uint64_t)n * count, 0, 0, 0);
            vrc_status_t rc = step<false>(args, nops, op_work(args.op[0]), cus, st);
            if (rc) return rc;
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
            uintptr_t out[kMaxRanks];
            for (int r = 0; r < n; r++) out[r] = (uintptr_t)(y[r] + off * E);
            a.ch[c] = {off, 1, len, 0, split_rows(write_ref(out, n), len, E)};
            a.tile0[c + 1] = a.tile0[c] + (a.ch[c].g.nvb + 63) / 64;
        }
        bool share = true;  // every output on one 128-byte grid (the chunks start at the same element of every buffer)
        for (int r = 0; r < n; r++) share = share && (uintptr_t)y[r] % kGridAlign == (uintptr_t)y[0] % kGridAlign;
        if (!MEM && share) {
            // Large calls read and write in phases, like the fused kernel.
            const uint64_t waves = (uint64_t)cus * (kBlock / 64), skew = (uint64_t)ring_order_phased_skew(cus);
            const uint64_t per_phase =
                waves * ((uint64_t)(ring_order_phased_regs<T>(n) + kRingOrderPhasedLds) - skew) + waves / 2 * skew;
            const uint64_t phases = tuning().phased && n >= 6 ? a.tile0[n] / per_phase : 0;
            if (phases >= 3) return ring_order_phased(a, n, count, phases, cus, st);
        }
        if (!MEM && tuning().realign && chain_ar_shape(MEM, n).block == 64) {
            // Outputs on different 128-byte offsets, none in place: every
            // output stored on its own grid (the chunks start at the same
            // element of every buffer, so one test covers all chunks).
            bool in_place = false;
            for (int r = 0; r < n; r++) in_place = in_place || x[r] == y[r];
            if (!share && !in_place && 2 * (uint64_t)n * count * E >= 64 * kMiB)
                return ring_order_realigned(a, n, count, cus, st);
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

    // The phased ring-order all-reduce: one 256-lane workgroup per CU,
    // `phases` whole phases of tiles, then the rest of the tiles and the
    // scalar heads and tails; ring_order_phased_regs<T>(n) sums per lane in
    // registers and kRingOrderPhasedLds in LDS.
    static vrc_status_t ring_order_phased(const vrc::ChainArgs& a, int n, uint64_t count, uint64_t phases, int cus,
                                          hipStream_t st)
    {
        const dim3 grid((unsigned)cus);
        if (g_plan)
            return plan_single(VRC_OP_RING_ORDER_ALLREDUCE_PHASED, count, grid, kBlock,
                               ring_order_phased_regs<T>(n) + kRingOrderPhasedLds);
        const uint32_t wait = (uint32_t)tuning().phase_wait, skew = (uint32_t)ring_order_phased_skew(cus);
        switch (n) {
#define VRC_CASE(K)                                                                                              \
    case K:                                                                                                      \
        hipLaunchKernelGGL((vrc::k_ring_order_allreduce_phased<T, K, ring_order_phased_regs<T>(K),                \
                                                               kRingOrderPhasedLds, true>),                      \
                           grid, dim3(kBlock), 0, st, a, phases, wait, skew);                                    \
        break;
            VRC_CASE(6) VRC_CASE(7) VRC_CASE(8) VRC_CASE(9) VRC_CASE(10) VRC_CASE(11) VRC_CASE(12) VRC_CASE(13)
            VRC_CASE(14) VRC_CASE(15) VRC_CASE(16)
#undef VRC_CASE
        default: return VRC_ERR_INVALID_ARG;
        }
        return check_launch();
    }

    // The ring-order all-reduce with every output stored on its own 128-byte
    // grid; `c` holds the chunk geometry of the tile kernel.
    static vrc_status_t ring_order_realigned(const vrc::ChainArgs& c, int n, uint64_t count, int cus, hipStream_t st)
    {
        const int U = realign_unroll(n);
        const uint64_t gv = (uint64_t)U * 64;
        vrc::RingOrderRealignArgs a = {};
        for (int r = 0; r < kMaxRanks; r++) {
            a.src[r] = c.src[r];
            a.dst[r] = c.dst[r];
            a.ch[r] = c.ch[r];
        }
        a.group0[0] = 0;
        a.rest0[0] = 0;
        for (int k = 0; k < n; k++) {
            const uint64_t nvb = c.ch[k].g.nvb;
            const uint64_t groups = nvb >= gv + 8 ? (nvb - 8) / gv : 0;
            const uint64_t rest = groups ? 8 + (nvb - groups * gv) : nvb;
            a.group0[k + 1] = a.group0[k] + groups;
            a.rest0[k + 1] = a.rest0[k] + (rest + 63) / 64;
            const uintptr_t body = (c.ch[k].off + c.ch[k].g.head) * E;
            for (int r = 0; r < n; r++)
                a.shift[k][r] = (uint8_t)((kGridAlign - ((uintptr_t)c.dst[r] + body) % kGridAlign) % kGridAlign);
        }
        for (int k = n; k < kMaxRanks; k++) {
            a.group0[k + 1] = a.group0[n];
            a.rest0[k + 1] = a.rest0[n];
        }
        uint64_t work = a.group0[n] > a.rest0[n] ? a.group0[n] : a.rest0[n];
        if (work < (uint64_t)n) work = n;  // one wave per chunk for the scalar pass
        const dim3 grid(grid_x(cus, work * 64, 1, realign_blocks_per_cu(n), 64));
        if (g_plan) return plan_single(VRC_OP_RING_ORDER_ALLREDUCE_REALIGNED, count, grid, 64, U);
        switch (n) {
#define VRC_CASE(K)                                                                                              \
    case K:                                                                                                      \
        hipLaunchKernelGGL((vrc::k_ring_order_allreduce_realigned<T, K, realign_unroll(K), true>), grid, dim3(64), \
                           0, st, a);                                                                            \
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
            rs_flat_layout(x, y, n, count, cus, &fa, &fgrid);
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
        vrc::ChainArgs a = {};
        uint64_t work = 0;
        for (int r = 0; r < kMaxRanks; r++) {
            a.src[r] = r < n ? x[r] : nullptr;
            a.dst[r] = r < n ? y[r] : nullptr;
        }
        for (int c = 0; c < n; c++) {
            const Chunk k = rs_chunk(count, outer, n, c);
            a.ch[c] = {k.off, k.rows, k.width, k.stride, split_rows((uintptr_t)y[c], k.width, E)};
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
            uintptr_t out[kMaxRanks];
            for (int r = 0; r < n; r++) out[r] = (uintptr_t)(y[r] + (uint64_t)q * row * E);
            a.g[q] = split_rows(write_ref(out, n), row, E);
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
        case VRC_TREE: break;    // all-gather only
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
        case VRC_SELECT:
        case VRC_TREE: break;
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
        case VRC_TREE: return L::tree_all_gather(x, y, n, count, outer, cus, st);
        case VRC_SELECT: break;
        }
        break;
    }
    return VRC_ERR_UNSUPPORTED;
}

}  // namespace host
}  // namespace vrc
