// mmvq_id.hip -- expert-routed TQ1_0 x Q8_1 mat-vec (mixture of experts) on gfx950.
//
// y[t][s][:] = W[ids[t][s]] x a[t]: each token's one activation column meets
// the matrices of the experts it is routed to ("CUDA: TQ1_0 mat-vec is
// load-bound by the per-32-element chunk contract", "Acceptance criteria":
// expert mat-vec at one activation per token, fewer experts used than
// available). Tokens routed to the same expert are grouped so that the
// expert's weights stream once per group of up to kIdCols tokens, the compacted
// per-expert grid that "tools: add mmq-tune, an MMQ tile-width autotuning
// harness" (Summary) describes for the production MoE path.
//
// Work item: one expert and up to kIdCols of its (token, slot) pairs. Two ways
// to find them, both exact and both free of host round trips:
//   - up to 64 pairs: inside every wave, from ids alone. Each lane holds one
//     pair; ballots over the bits of the expert id give each lane the set of
//     lanes routed to the same expert, hence its rank among them. A pair whose
//     rank is a multiple of kIdCols opens an item; items are numbered in
//     pair-index order of their first pair.
//   - more pairs: a one-workgroup pre-pass (mmvq_id_route_kernel) counts,
//     scans and scatters the pairs by expert into the caller's workspace, and
//     the product kernel reads its item from there.
// The multiply is the staged multi-column body (byte-major decode, activations
// in LDS) with the columns gathered by token and the outputs scattered by pair.
// A workgroup stages its item's columns once and then walks several groups of
// rows, so the staging is amortised over more weight bytes as the number of
// items grows. Each column's arithmetic does not depend on which other columns
// share the item, nor on the rows a workgroup walks, so results are bitwise
// those of a plain one-column call on the expert.
#include <atomic>

#include "launch.hpp"
#include "mmvq_staged.hpp"

namespace bqm {

// Pairs per work item of the staged expert kernel. It finishes an item's
// columns one after another, so under skewed routing the few items of the
// most used experts set the kernel's length; four splits them at the cost of
// a second read of those experts' weights (moe 128 x 1536 x 4096, T = 8:
// 24.9 us at eight, 23.3 at four, 25.1 at two).
constexpr int kIdCols = 4;
constexpr int kIdWaveRouteMax = 64;    // pairs routed inside the wave
constexpr int kIdMaxExperts = 4096;    // experts the routing pre-pass handles
constexpr int kRouteThreads = 1024;

// Upper bound of the number of work items: sum over experts of
// ceil(count / kIdCols) with at most min(E, P) experts in use.
static int64_t id_max_items(int64_t E, int64_t P)
{
    const int64_t active = E < P ? E : P;
    return (P + (kIdCols - 1) * active + kIdCols - 1) / kIdCols;
}

// ---------------------------------------------------------------------------
// Routing pre-pass. An expert with at least wide_min pairs gets wide items of
// up to kWideCols pairs (the matrix-core kernel's 16 columns), any other
// expert narrow items of up to narrow_cap pairs (the staged kernel). Workspace
// layout (int32, M = max_items):
//   ws[0], ws[1]                        number of narrow, wide items
//   ws[2 + 3k .. 4 + 3k]                narrow item k: expert, first run slot, pairs
//   ws[2 + 3(M + k) .. 4 + 3(M + k)]    wide item k, the same fields
//   ws[2 + 6M + slot]                   pair index held by run slot `slot`
// An expert's pairs occupy consecutive run slots; the order inside the run
// follows atomic timing, which is harmless because the columns of an item are
// computed independently. Pairs whose id is outside [0, E) are dropped.
// ---------------------------------------------------------------------------
constexpr int kWideCols = 16;
// Pairs from which an expert takes the matrix cores (wide items) once the
// pre-pass has sorted the pairs. From three pairs, one decode per 16-row tile
// shared by all of an item's columns beats the staged kernel's one floor-pair
// pass per column (moe 128 x 1536 x 4096, 512 pairs: 92.5 us at five pairs,
// 87.3 us at three, 96.7 us at two).
constexpr int kIdWideMin = 3;

// Inclusive sum over lanes 0..L of the wave, for every lane L: within each
// 16-lane row by shifts of 1, 2, 4, 8 (lanes without a source add 0), then
// row 1 and 3 add lane 15 of the row before, rows 2 and 3 lane 31 (DPP row
// broadcasts).
__device__ __forceinline__ int wave_inclusive_sum(int v)
{
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
    return v;
}

// Exclusive scan of three per-thread values over a kRouteThreads workgroup
// (in place in v0..v2, which hold one value per thread); the totals go to
// tot[0..2]. One wave scans, 16 values per lane.
__device__ __forceinline__ void route_scan3(int *v0, int *v1, int *v2, int *tot)
{
    const int tid = threadIdx.x;
    if (tid < 64) {
        int *v[3] = {v0, v1, v2};
        int x[3][16], r[3];
#pragma unroll
        for (int k = 0; k < 3; k++) {
            r[k] = 0;
#pragma unroll
            for (int i = 0; i < 16; i++) {
                x[k][i] = v[k][tid * 16 + i];
                r[k] += x[k][i];
            }
        }
#pragma unroll
        for (int k = 0; k < 3; k++) {
            const int inc = wave_inclusive_sum(r[k]);
            int o = inc - r[k];
#pragma unroll
            for (int i = 0; i < 16; i++) {
                v[k][tid * 16 + i] = o;
                o += x[k][i];
            }
            if (tid == 63)
                tot[k] = inc;
        }
    }
}

__global__ __launch_bounds__(kRouteThreads) void mmvq_id_route_kernel(
    const int32_t *__restrict__ ids, int32_t *__restrict__ ws, int E, int P, int max_items,
    int narrow_cap, int wide_min)
{
    __shared__ int cnt[kIdMaxExperts];   // pair counts, then first run slots
    __shared__ int fill[kIdMaxExperts];  // run slots taken so far
    __shared__ int pp[kRouteThreads];    // per-thread pairs, narrow and wide items,
    __shared__ int np[kRouteThreads];    // then their exclusive scans
    __shared__ int wp[kRouteThreads];
    __shared__ int tot[3];
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += kRouteThreads) {
        cnt[e] = 0;
        fill[e] = 0;
    }
    __syncthreads();
    // the first kRouteHeld ids of each thread stay in registers for the
    // scatter below (P <= kRouteHeld * kRouteThreads reads ids once)
    constexpr int kRouteHeld = 4;
    int held[kRouteHeld];
#pragma unroll
    for (int h = 0; h < kRouteHeld; h++) {
        const int p = tid + h * kRouteThreads;
        held[h] = p < P ? ids[p] : -1;
        if ((unsigned)held[h] < (unsigned)E)
            atomicAdd(&cnt[held[h]], 1);
    }
    for (int p = tid + kRouteHeld * kRouteThreads; p < P; p += kRouteThreads) {
        const int e = ids[p];
        if ((unsigned)e < (unsigned)E)
            atomicAdd(&cnt[e], 1);
    }
    __syncthreads();
    // thread t owns experts [t*per, (t+1)*per)
    const int per = (E + kRouteThreads - 1) / kRouteThreads;
    auto narrow_items = [&](int c) { return c >= wide_min ? 0 : (c + narrow_cap - 1) / narrow_cap; };
    auto wide_items = [&](int c) { return c >= wide_min ? (c + kWideCols - 1) / kWideCols : 0; };
    int sp = 0, sn = 0, sw = 0;
    for (int k = 0; k < per; k++) {
        const int e = tid * per + k;
        if (e < E) {
            sp += cnt[e];
            sn += narrow_items(cnt[e]);
            sw += wide_items(cnt[e]);
        }
    }
    pp[tid] = sp;
    np[tid] = sn;
    wp[tid] = sw;
    __syncthreads();
    route_scan3(pp, np, wp, tot);
    __syncthreads();
    if (tid == 0) {
        ws[0] = tot[1];
        ws[1] = tot[2];
    }
    int32_t *runs = ws + 2 + 6 * max_items;
    int off = pp[tid], noff = np[tid], woff = wp[tid];
    for (int k = 0; k < per; k++) {
        const int e = tid * per + k;
        if (e < E) {
            const int c = cnt[e];
            const bool wide = c >= wide_min;
            const int cap = wide ? kWideCols : narrow_cap;
            int32_t *list = ws + 2 + 3 * (wide ? max_items + woff : noff);
            const int n = (c + cap - 1) / cap;
            for (int i = 0; i < n; i++) {
                list[3 * i] = e;
                list[3 * i + 1] = off + i * cap;
                list[3 * i + 2] = min(cap, c - i * cap);
            }
            if (wide)
                woff += n;
            else
                noff += n;
            cnt[e] = off;
            off += c;
        }
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < kRouteHeld; h++) {
        const int p = tid + h * kRouteThreads;
        if ((unsigned)held[h] < (unsigned)E)
            runs[cnt[held[h]] + atomicAdd(&fill[held[h]], 1)] = p;
    }
    for (int p = tid + kRouteHeld * kRouteThreads; p < P; p += kRouteThreads) {
        const int e = ids[p];
        if ((unsigned)e < (unsigned)E)
            runs[cnt[e] + atomicAdd(&fill[e], 1)] = p;
    }
}

// ---------------------------------------------------------------------------
// The work item of this workgroup (values uniform across the workgroup).
// ---------------------------------------------------------------------------
struct IdItem {
    int e;               // expert
    int Tc;              // pairs, 1..kIdCols
    int sel[kIdCols];    // pair indices (t >= Tc: a copy of sel[0])
};

// Wave-local routing of P <= 64 pairs: each lane's pair, its rank among the
// pairs of the same expert, and the lanes that open an item.
struct WaveRoute {
    int e;              // this lane's expert (-1 past P)
    bool valid;         // e in [0, E)
    int rank;           // pairs of the same expert in lanes below
    uint64_t openers;   // lanes whose rank is a multiple of kIdCols
};

__device__ __forceinline__ WaveRoute wave_route(const int32_t *__restrict__ ids, int E, int P)
{
    const int lane = threadIdx.x & 63;
    WaveRoute r;
    r.e = lane < P ? ids[lane] : -1;
    r.valid = (unsigned)r.e < (unsigned)E;
    // lanes routed to my expert: valid lanes that agree on every id bit
    uint64_t same = __ballot(r.valid);
    const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
    for (int k = 0; k < nbits; k++) {
        const bool bit = (r.e >> k) & 1;
        const uint64_t b = __ballot(bit);
        same &= bit ? b : ~b;
    }
    r.rank = __popcll(same & ((1ull << lane) - 1ull));
    r.openers = __ballot(r.valid && r.rank % kIdCols == 0);
    return r;
}

// Item `item` (< popcount(openers)) of a wave-local routing.
__device__ __forceinline__ void wave_route_item(const WaveRoute &r, int item, IdItem &it)
{
    const int lane = threadIdx.x & 63;
    const bool opens = (r.openers >> lane) & 1;
    const uint64_t mine =
        __ballot(opens && __popcll(r.openers & ((1ull << lane) - 1ull)) == item);
    const int lead = __builtin_amdgcn_readfirstlane(__builtin_ctzll(mine));
    const int e_it = __builtin_amdgcn_readlane(r.e, lead);
    const int r0 = __builtin_amdgcn_readlane(r.rank, lead);
    uint64_t m = __ballot(r.valid && r.e == e_it && r.rank >= r0 && r.rank < r0 + kIdCols);
    it.e = e_it;
    it.Tc = __popcll(m);
    const int first = __builtin_ctzll(m);
#pragma unroll
    for (int t = 0; t < kIdCols; t++) {
        it.sel[t] = m ? (int)__builtin_ctzll(m) : first;
        m &= m - 1;
    }
}

// Narrow item `item` (< routed[0]) written by the routing pre-pass.
__device__ __forceinline__ void workspace_item(const int32_t *__restrict__ routed, int max_items,
                                               int item, IdItem &it)
{
    const int32_t *p = routed + 2 + 3 * item;
    const int32_t *runs = routed + 2 + 6 * max_items + p[1];
    it.e = p[0];
    it.Tc = p[2];
#pragma unroll
    for (int t = 0; t < kIdCols; t++)
        it.sel[t] = runs[t < it.Tc ? t : 0];
}

// Stage Tc whole activation columns (nb blocks each) in the staged layout,
// column t at act + t * nb * kActStride, with several loads in flight per lane.
__device__ __forceinline__ void stage_item_columns(uint32_t *__restrict__ act,
                                                   __amdgpu_buffer_rsrc_t ra,
                                                   const uint32_t (&col_off)[kIdCols], int Tc,
                                                   int nb)
{
    constexpr int kAhead = 4;
    const int tid = threadIdx.x;
    const int per_col = nb * 8;
    const int tasks = Tc * per_col;
    for (int base = 0; base < tasks; base += kAhead * 256) {
        u32x4 v0[kAhead], v1[kAhead];
        uint32_t ds[kAhead];
#pragma unroll
        for (int k = 0; k < kAhead; k++) {
            const int i = base + k * 256 + tid;
            if (i < tasks) {
                const int t = i / per_col, j = i - t * per_col;
                uint32_t coff = col_off[0];
#pragma unroll
                for (int u = 1; u < kIdCols; u++)
                    coff = t == u ? col_off[u] : coff;
                const uint32_t off = coff + (uint32_t)j * kQ81BlockBytes;
                v0[k] = ld_b128(ra, off);
                v1[k] = ld_b128(ra, off + 16);
                ds[k] = ld_b32(ra, off + 32);
            }
        }
#pragma unroll
        for (int k = 0; k < kAhead; k++) {
            const int i = base + k * 256 + tid;
            if (i < tasks) {
                const int t = i / per_col, j = i - t * per_col;
                const int bi = j >> 3, c = j & 7;
                uint32_t *dst = act + (t * nb + bi) * kActStride;
                const uint32_t q[8] = {v0[k].x, v0[k].y, v0[k].z, v0[k].w,
                                       v1[k].x, v1[k].y, v1[k].z, v1[k].w};
                int sq = 0;
#pragma unroll
                for (int jj = 0; jj < 8; jj++) {
                    dst[8 * jj + c] = q[jj];
                    sq = sdot4(0x01010101u, q[jj], sq);
                }
                dst[64 + c] = __float_as_uint(f16_bits_to_f32(ds[k] & 0xffffu));
                dst[72 + c] = (uint32_t)(-sq);
            }
        }
    }
}

// One group of rows (the 4 waves x 64/Lr rows of one workgroup step) against
// the item's staged columns. The kernel takes rows of at most 64 blocks, so
// Lr >= nb and lane `sub` of a row owns block sub alone (none if sub >= nb): a
// column's result is that one block's fmaf(dw, s, 0), summed over the row's
// lanes by the xor butterfly -- the library's fp32 order for a row of
// nb <= Lr blocks. Columns are finished one after the other, each through the
// one-column floor-pair sums, so no per-column state stays live across
// columns.
struct RowWalk {
    __amdgpu_buffer_rsrc_t rw;
    int64_t N;
    int nb, lr_log2, wave, sub;

    __device__ int64_t row(int g) const
    {
        const int lane = threadIdx.x & 63;
        return ((int64_t)g * 4 + wave) * (64 >> lr_log2) + (lane >> lr_log2);
    }
    // this lane's block of its row in group g, if there is one
    __device__ void load(int g, RawBlock &b) const
    {
        const int64_t r = row(g);
        if (r < N && sub < nb)
            b = load_raw_block(rw, (uint32_t)((r * nb + sub) * kTq1BlockBytes));
    }
};

__device__ __forceinline__ void group_rows(const RowWalk &wk, int g, const RawBlock &cur,
                                           const uint32_t *act, float *__restrict__ y,
                                           const int *pair, int Tc)
{
    // blocks past the row's end read block nb - 1's staged columns, and
    // contribute +0 like the lanes of the other kernels that own no block
    const uint32_t *ab0 = act + (wk.sub < wk.nb ? wk.sub : wk.nb - 1) * kActStride;
    const int64_t row = wk.row(g);
    const bool own = row < wk.N && wk.sub < wk.nb;
    const float dw = f16_bits_to_f32(raw_scale_bits(cur));
    for (int t = 0; t < Tc; t++) {
        const uint32_t *ab = ab0 + t * wk.nb * kActStride;
        int isum[8];
        block_sums_staged(cur, ab, isum);
        float da[8];
#pragma unroll
        for (int b = 0; b < 8; b++)
            da[b] = __uint_as_float(ab[64 + b]);
        float v = own ? fmaf(dw, block_dot_f32(isum, da), 0.0f) : 0.0f;
        v = row_sum(v, wk.lr_log2);
        if (row < wk.N && wk.sub == 0)
            y[(int64_t)pair[t] * wk.N + row] = v;
    }
}

// Product kernel. grid.y: work items (an upper bound; workgroups past the
// last item return at once); grid.x: slices of the item's row groups, the
// workgroup taking groups blockIdx.x, blockIdx.x + gridDim.x, ... The many
// small workgroups of unequal cost (an item's pairs set its cost) are balanced
// by the hardware's dispatch. The item's columns are staged once; the lane's
// block in the next group is loaded before the current one is used.
__global__ __launch_bounds__(256) void mmvq_id_kernel(const uint8_t *__restrict__ w,
                                                      const uint8_t *__restrict__ a,
                                                      const int32_t *__restrict__ ids,
                                                      const int32_t *__restrict__ routed,
                                                      float *__restrict__ y, int E, int64_t N,
                                                      int nb, int T, int n_used, int lr_log2,
                                                      int max_items, int ngroups, int pairs_per_col)
{
    extern __shared__ uint4 lds4[];
    uint32_t *act = reinterpret_cast<uint32_t *>(lds4);
    __shared__ int pair[kIdCols];
    const int item = blockIdx.y;
    IdItem it;
    if (routed) {
        if (item >= routed[0])
            return;  // uniform
        workspace_item(routed, max_items, item, it);
    } else {
        const WaveRoute wr = wave_route(ids, E, T * n_used);
        if (item >= __popcll(wr.openers))
            return;  // uniform
        wave_route_item(wr, item, it);
    }
    const uint64_t expert_bytes = (uint64_t)N * nb * kTq1BlockBytes;
    const uint64_t col_bytes = (uint64_t)nb * 8 * kQ81BlockBytes;
    RowWalk wk;
    wk.rw = make_rsrc(w + (uint64_t)it.e * expert_bytes, expert_bytes);
    wk.N = N;
    wk.nb = nb;
    wk.lr_log2 = lr_log2;
    wk.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    wk.sub = (threadIdx.x & 63) & ((1 << lr_log2) - 1);
    // the first weight block is in flight while the columns are staged
    RawBlock cur;
    wk.load(blockIdx.x, cur);
    uint32_t col_off[kIdCols];
#pragma unroll
    for (int t = 0; t < kIdCols; t++)
        col_off[t] = (uint32_t)((it.sel[t] / pairs_per_col) * col_bytes);
#pragma unroll
    for (int t = 0; t < kIdCols; t++)
        if ((int)threadIdx.x == t)
            pair[t] = it.sel[t];
    stage_item_columns(act, make_rsrc(a, (uint64_t)(T * n_used / pairs_per_col) * col_bytes),
                       col_off, it.Tc, nb);
    __syncthreads();
    for (int g = blockIdx.x; g < ngroups; g += gridDim.x) {
        RawBlock nxt;
        if (g + (int)gridDim.x < ngroups)
            wk.load(g + gridDim.x, nxt);
        group_rows(wk, g, cur, act, y, pair, it.Tc);
        cur = nxt;
    }
}

static bool id_uses_prepass(int64_t E, int64_t P)
{
    return P > kIdWaveRouteMax && E <= kIdMaxExperts;
}

size_t mmvq_id_workspace_bytes(int64_t E, int64_t T, int32_t n_used)
{
    const int64_t P = T * n_used;
    if (!id_uses_prepass(E, P))
        return 0;
    const size_t words = 2 + 6 * (size_t)id_max_items(E, P) + (size_t)P;
    return (words * 4 + 255) & ~(size_t)255;
}

int launch_mmvq_id(const void *w, const void *a, const int32_t *ids, float *y, int64_t E,
                   int64_t N, int64_t K, int64_t T, int32_t n_used, bool per_slot,
                   void *workspace, hipStream_t stream)
{
    // consecutive pairs that read one activation column: a token's slots, or
    // each pair alone
    const int pairs_per_col = per_slot ? 1 : n_used;
    const int nb = (int)(K / kTq1BlockElems);
    const int lr = lanes_per_row_log2(nb);
    const int64_t P = T * n_used;
    const bool prepass = id_uses_prepass(E, P);
    // experts with at least kIdWideMin pairs go to the matrix cores when the
    // pre-pass sorts the pairs; then every other expert holds at most
    // kIdWideMin - 1 pairs, one narrow item
    const bool wide = prepass && mfma_resident_id_supported(K);
    const int narrow_cap = wide ? kIdWideMin - 1 : kIdCols;
    // the item's columns must fit LDS whole (on 160 KiB: K <= 15360), and a
    // row must have at most 64 blocks (one per lane)
    const size_t lds = (size_t)narrow_cap * nb * kActStride * 4;
    if (nb > 64 || lds > lds_budget() || (P > kIdWaveRouteMax && !prepass))
        return launch_mmvq_id_pairs(w, a, ids, y, E, N, K, T, n_used, pairs_per_col, stream);
    const int64_t max_items = id_max_items(E, P);
    int32_t *routed = nullptr;
    if (prepass) {
        routed = static_cast<int32_t *>(workspace);
        hipLaunchKernelGGL(mmvq_id_route_kernel, dim3(1), dim3(kRouteThreads), 0, stream, ids,
                           routed, (int)E, (int)P, (int)max_items, narrow_cap,
                           wide ? kIdWideMin : INT32_MAX);
        if (int rc = check_launch())
            return rc;
    }
    const int64_t active = E < P ? E : P;
    const int64_t max_narrow = wide ? active : max_items;
    const int64_t rows_per_wg = 4 * (64 >> lr);
    const int64_t ngroups = (N + rows_per_wg - 1) / rows_per_wg;
    allow_dynamic_lds(reinterpret_cast<const void *>(&mmvq_id_kernel), lds);
    // about kIdTargetWorkgroups workgroups when every item is in use, but at
    // most kIdGroupsPerSlice row groups per workgroup: restaging the columns
    // costs less than the lost balance of longer workgroups
    constexpr int64_t kIdTargetWorkgroups = 2048, kIdGroupsPerSlice = 3;
    int64_t slices = (kIdTargetWorkgroups + max_narrow - 1) / max_narrow;
    const int64_t fewest = (ngroups + kIdGroupsPerSlice - 1) / kIdGroupsPerSlice;
    slices = slices > fewest ? slices : fewest;
    slices = slices < ngroups ? slices : ngroups;
    hipLaunchKernelGGL(mmvq_id_kernel, dim3((unsigned)slices, (unsigned)max_narrow), dim3(256),
                       lds, stream, static_cast<const uint8_t *>(w),
                       static_cast<const uint8_t *>(a), ids, routed, y, (int)E, N, nb, (int)T,
                       (int)n_used, lr, (int)max_items, (int)ngroups, pairs_per_col);
    if (int rc = check_launch())
        return rc;
    if (!wide)
        return BQM_OK;
    // wide items: at most one per expert with kIdWideMin or more pairs, plus
    // one per further kWideCols pairs
    const int64_t wide_experts = P / kIdWideMin < E ? P / kIdWideMin : E;
    const int64_t max_wide = wide_experts + P / kWideCols;
    return launch_mmvq_mfma_resident_id(w, a, y, N, K, P / pairs_per_col, routed, (int)max_items,
                                        (int)max_wide, pairs_per_col, stream);
}

// ---------------------------------------------------------------------------
// Device scratch of the allocation-free expert-routed entry point: the
// routing pre-pass's workspace, held in a file-scope device array that each
// GPU the library runs on keeps until the process ends. Host code never
// passes the array's name to a kernel (on the host it names a stand-in, not
// device memory): the entry point looks up the array's device address once
// per device, with that device current, and passes that address.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

int noalloc_scratch(void **ptr)
{
    static std::atomic<void *> addr[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return BQM_ERR_DEVICE;
    void *p = addr[dev].load(std::memory_order_acquire);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return BQM_ERR_LAUNCH;
        addr[dev].store(p, std::memory_order_release);
    }
    *ptr = p;
    return BQM_OK;
}

}  // namespace bqm
