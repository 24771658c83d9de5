// mmvq_id.hip -- expert-routed TQ1_0 x Q8_1 mat-vec (mixture of experts) on gfx950.
//
// y[t][s][:] = W[ids[t][s]] x a[t]: each token's one activation column meets
// the matrices of the experts it is routed to ("CUDA: TQ1_0 mat-vec is
// load-bound by the per-32-element chunk contract", "Acceptance criteria":
// expert mat-vec at one activation per token, fewer experts used than
// available). Tokens routed to the same expert are grouped so that the
// expert's weights stream once per group of up to eight tokens, the compacted
// per-expert grid that "tools: add mmq-tune, an MMQ tile-width autotuning
// harness" (Summary) describes for the production MoE path.
//
// Routing runs inside every workgroup, from ids alone, with no second launch
// and no host round trip:
//   1. count the (token, slot) pairs of each expert (LDS atomics; exact);
//   2. exclusive scan of ceil(count / 8) over experts gives each expert's
//      first work item; work item blockIdx.y belongs to the expert whose range
//      holds it, and is that expert's k-th group of eight pairs;
//   3. the workgroup's pairs are the k-th eight of its expert in pair-index
//      order (one wave, ballots and prefix popcounts), so every workgroup of
//      an item agrees on its columns.
// The multiply itself is the staged multi-column body of mmvq_staged.hip with
// the columns gathered by token and the outputs scattered by pair. Each
// column's arithmetic does not depend on which other columns share the item,
// so results are bitwise those of a plain one-column call on the expert.
#include "launch.hpp"
#include "mmvq_staged.hpp"

namespace bqm {

constexpr int kIdCols = 8;       // pairs per work item
constexpr int kIdMaxExperts = 4096;

__global__ __launch_bounds__(256) void mmvq_id_kernel(const uint8_t *__restrict__ w,
                                                      const uint8_t *__restrict__ a,
                                                      const int32_t *__restrict__ ids,
                                                      float *__restrict__ y, int E, int64_t N,
                                                      int nb, int T, int n_used, int lr_log2,
                                                      int chunk, int route_dwords)
{
    extern __shared__ uint4 lds4[];
    int *cnt = reinterpret_cast<int *>(lds4);        // [E]
    int *start = cnt + E;                             // [E + 1]
    int *sel = start + E + 1;                         // [kIdCols + 1]
    uint32_t *act = reinterpret_cast<uint32_t *>(lds4) + route_dwords;
    const int tid = threadIdx.x;
    const int P = T * n_used;

    // 1. pairs per expert
    for (int e = tid; e < E; e += 256)
        cnt[e] = 0;
    __syncthreads();
    for (int p = tid; p < P; p += 256) {
        const int e = ids[p];
        if ((unsigned)e < (unsigned)E)
            atomicAdd(&cnt[e], 1);
    }
    __syncthreads();
    // 2. first work item of each expert
    if (tid < 64) {
        int run = 0;
        for (int base = 0; base < E; base += 64) {
            const int e = base + tid;
            const int v = e < E ? (cnt[e] + kIdCols - 1) / kIdCols : 0;
            int x = v;
            for (int m = 1; m < 64; m <<= 1) {
                const int u = __shfl_up(x, m, 64);
                if (tid >= m)
                    x += u;
            }
            if (e < E)
                start[e] = run + x - v;
            run += __shfl(x, 63, 64);
        }
        if (tid == 0)
            start[E] = run;
    }
    __syncthreads();
    const int item = blockIdx.y;
    if (item >= start[E])
        return;  // uniform: every thread read the same LDS value
    int lo = 0, hi = E;  // largest expert whose first item is <= item
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (start[mid] <= item)
            lo = mid;
        else
            hi = mid;
    }
    const int e = lo;
    const int want0 = (item - start[e]) * kIdCols;
    // 3. this item's pairs, in pair-index order
    if (tid < 64) {
        int run = 0;
        for (int base = 0; base < P && run < want0 + kIdCols; base += 64) {
            const int p = base + tid;
            const bool m = p < P && ids[p] == e;
            const unsigned long long mask = __ballot(m);
            const int rank = run + __popcll(mask & ((1ull << tid) - 1ull));
            if (m && rank >= want0 && rank < want0 + kIdCols)
                sel[rank - want0] = p;
            run += __popcll(mask);
        }
        if (tid == 0)
            sel[kIdCols] = min(run - want0, kIdCols);
    }
    __syncthreads();
    const int Tc = sel[kIdCols];
    const int nblk = nb * 8;
    const uint64_t expert_bytes = (uint64_t)N * nb * kTq1BlockBytes;
    const uint64_t col_bytes = (uint64_t)nblk * kQ81BlockBytes;
    uint32_t col_off[kIdCols];
    float *out[kIdCols];
#pragma unroll
    for (int t = 0; t < kIdCols; t++) {
        const int p = t < Tc ? sel[t] : sel[0];
        col_off[t] = (uint32_t)((p / n_used) * col_bytes);
        out[t] = y + (int64_t)p * N;
    }
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(w + (uint64_t)e * expert_bytes, expert_bytes);
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(a, (uint64_t)T * col_bytes);
    const int wave = tid >> 6, lane = tid & 63;
    const int64_t row = ((int64_t)blockIdx.x * 4 + wave) * (64 >> lr_log2) + (lane >> lr_log2);
    staged_rows<kIdCols, false>(rw, ra, col_off, out, nullptr, act, row, row < N, N, nb, Tc,
                                lr_log2, chunk);
}

// LDS words of the routing tables (counts, first items, the item's pairs),
// rounded to 16 bytes so the staged activations that follow stay aligned.
static int route_dwords(int64_t E) { return (int)((2 * E + 1 + kIdCols + 1 + 3) & ~3ll); }

static int id_chunk(int64_t E, int nb, int lr)
{
    if (E > kIdMaxExperts)
        return 0;
    return staged_chunk(nb, lr, kIdCols, lds_budget() - (size_t)route_dwords(E) * 4);
}

size_t mmvq_id_workspace_bytes(int64_t E, int64_t T, int32_t n_used)
{
    (void)E;
    (void)T;
    (void)n_used;
    return 0;  // routing happens in LDS inside the kernel
}

int launch_mmvq_id(const void *w, const void *a, const int32_t *ids, float *y, int64_t E,
                   int64_t N, int64_t K, int64_t T, int32_t n_used, void *workspace,
                   hipStream_t stream)
{
    (void)workspace;
    const int nb = (int)(K / kTq1BlockElems);
    const int lr = lanes_per_row_log2(nb);
    const int chunk = id_chunk(E, nb, lr);
    if (chunk == 0)
        return launch_mmvq_id_pairs(w, a, ids, y, E, N, K, T, n_used, stream);
    const int64_t P = T * n_used;
    const int64_t active = E < P ? E : P;
    const int64_t max_items = (P + (kIdCols - 1) * active + kIdCols - 1) / kIdCols;
    const int64_t rows_per_wg = 4 * (64 >> lr);
    const dim3 grid((unsigned)((N + rows_per_wg - 1) / rows_per_wg), (unsigned)max_items);
    const int rd = route_dwords(E);
    const size_t lds = (size_t)rd * 4 + (size_t)kIdCols * chunk * kActStride * 4;
    allow_dynamic_lds(reinterpret_cast<const void *>(&mmvq_id_kernel), lds);
    hipLaunchKernelGGL(mmvq_id_kernel, grid, dim3(256), lds, stream,
                       static_cast<const uint8_t *>(w), static_cast<const uint8_t *>(a), ids, y,
                       (int)E, N, nb, (int)T, (int)n_used, lr, chunk, rd);
    return check_launch();
}

}  // namespace bqm
